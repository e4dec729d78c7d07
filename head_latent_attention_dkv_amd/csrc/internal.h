// Internal parameter blocks and launchers of the MLA library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kMaxRopePairs = 64;   // rotary width <= 128 (half-split head) or <= 64 (decoupled)

// Inverse RoPE frequencies theta_j = base^(-2j/d), split into an fp32 head and an
// fp32 tail so the device can rebuild them to ~double precision.
struct RopeTable {
  float hi[kMaxRopePairs];
  float lo[kMaxRopePairs];
};
void make_rope_table(RopeTable* t, int dim, float base);

// ---------------------------------------------------------------------------
// Projection GEMM: out[m, n] = sum_k A[m, k] * W[n, k]   (W [N][K], "NT")
//            or    out[m, n] = sum_k A[m, k] * W[k, n]   (W [K][N], w_kmajor)
// Rows of A and of the output may live in a cache ([batch][max_seq][.]) and the
// output columns of a segment may be scattered head by head.
// ---------------------------------------------------------------------------
enum RopeKind { ROPE_OFF = 0, ROPE_INTERLEAVED = 1, ROPE_HALFSPLIT = 2 };

struct GemmSeg {
  const void* w;        // this segment's first weight row (NT) / column (k-major)
  long long w_ld;       // elements between consecutive W rows
  int n;                // output columns of this segment
  void* out;            // output base
  long long out_ld;     // elements between output rows
  int out_f32;          // 1: float output, 0: element type of the GEMM
  int out_hw, out_hs;   // column map oc = (c / hw) * hs + c % hw   (hw = 0: oc = c)
  int out_cache;        // 1: output row of (b, t) is b * out_bstride + pos0[b] + t
  int rope;             // RopeKind applied to this segment's columns before the store
  int rope_d;           // rotary width: pairs live inside [h*rope_d, (h+1)*rope_d)
  // Output layout (row m = (b, t) with t = m % rows_per_batch; column c = head * out_hw + j):
  //   OUT_ROWS        out[row * out_ld + column map above]
  //   OUT_HEAD_MAJOR  out[((b * out_nh + head) * rows_per_batch + t) * out_hw + j]
  //   OUT_HEAD_T16    out[((b * out_nh + head) * out_hw + j) * out_ld + perm16(t)], perm16
  //                   swapping positions 4..7 and 8..11 inside every group of 16
  int layout;
  int out_nh;
};

enum OutLayout { OUT_ROWS = 0, OUT_HEAD_MAJOR = 1, OUT_HEAD_T16 = 2 };

// Position of token t inside a group of 16 in the OUT_HEAD_T16 layout (an involution):
// 0..3 -> 0..3, 4..7 -> 8..11, 8..11 -> 4..7, 12..15 -> 12..15.
__host__ __device__ inline int perm16(int t) {
  const int q = (t >> 2) & 3;
  return (t & ~15) | (((q == 1) ? 2 : (q == 2) ? 1 : q) << 2) | (t & 3);
}

constexpr int kMaxSeg = 3;   // output segments of one product (three only on the few-row path)

struct GemmParams {
  const void* a;            // A base
  long long a_ld;           // elements between A rows
  int a_cache;              // 1: A row of (b, t) is b * a_bstride + t
  long long a_bstride;      // rows per batch entry in A's storage (cache max_seq)
  long long out_bstride;    // rows per batch entry in a cache output
  int M, K;
  int rows_per_batch;       // t = m % rows_per_batch, b = m / rows_per_batch
  const int* pos0;          // per-batch first position (NULL = 0); RoPE angle uses pos0[b] + t
  int nseg;
  GemmSeg seg[kMaxSeg];
  // grouped launch (blockIdx.z = group): offsets in elements, g = (z / zdiv, z % zdiv)
  int zdiv;
  long long a_goff[2];      // added to A's column start
  long long w_goff[2];      // added to every segment's W pointer
  long long o_goff[2];      // added to every segment's output column start
  int w_kmajor;
  RopeTable rope;
  // split-K partial sums for few-row products: workspace supplied by the caller (may be
  // NULL: then the product runs unsplit); splits / kchunk are set by the launcher
  float* part;
  size_t part_bytes;
  int splits, kchunk;
  int fast_epilogue;        // set by the launcher: 0 generic, 1 vectorised, 2 flash layouts direct
};

// Output columns of all segments, and the segment holding output column n (*nn: its column
// inside that segment); segments are laid side by side in order.
__host__ __device__ inline int seg_total(const GemmParams& p) {
  return p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0) + (p.nseg > 2 ? p.seg[2].n : 0);
}
__host__ __device__ inline int seg_of(const GemmParams& p, int n, int* nn) {
  const int e0 = p.seg[0].n, e1 = e0 + (p.nseg > 1 ? p.seg[1].n : 0);
  const int s = n < e0 ? 0 : (n < e1 || p.nseg < 3) ? 1 : 2;
  *nn = n - (s == 0 ? 0 : s == 1 ? e0 : e1);
  return s;
}

// Output fields of segment s when s differs between the lanes of a wave.  Every field is
// read at a constant index (a scalar load of the kernel arguments) and picked per lane:
// indexing p.seg with a lane-dependent s makes the compiler read the argument block with
// vector loads, one memory round trip per field, one behind the other (a projection's
// output stage waited several microseconds on such chains).
struct SegOut {
  void* out;
  long long out_ld;
  int out_f32, out_hw, out_hs, out_cache, rope, rope_d, layout, out_nh;
};

__device__ __forceinline__ SegOut seg_out(const GemmParams& p, int s) {
  SegOut r;
#define MLA_SEG_PICK(f) (s == 0 ? p.seg[0].f : s == 1 ? p.seg[1].f : p.seg[2].f)
  r.out = MLA_SEG_PICK(out);
  r.out_ld = MLA_SEG_PICK(out_ld);
  r.out_f32 = MLA_SEG_PICK(out_f32);
  r.out_hw = MLA_SEG_PICK(out_hw);
  r.out_hs = MLA_SEG_PICK(out_hs);
  r.out_cache = MLA_SEG_PICK(out_cache);
  r.rope = MLA_SEG_PICK(rope);
  r.rope_d = MLA_SEG_PICK(rope_d);
  r.layout = MLA_SEG_PICK(layout);
  r.out_nh = MLA_SEG_PICK(out_nh);
#undef MLA_SEG_PICK
  return r;
}

// The inverse-frequency table in LDS (hi[0..kMaxRopePairs), then lo[...]) for output stages
// that look entries up per lane: on the kernel arguments each lookup would be a vector load.
constexpr int kRopeTabFloats = 2 * kMaxRopePairs;

__device__ __forceinline__ bool gemm_has_rope(const GemmParams& p) {
  return p.seg[0].rope != ROPE_OFF || (p.nseg > 1 && p.seg[1].rope != ROPE_OFF) ||
         (p.nseg > 2 && p.seg[2].rope != ROPE_OFF);
}

// Threads tid, tid + nthreads, ... copy the table (one round of loads, in parallel); the
// caller synchronises before the first lookup.
__device__ __forceinline__ void stage_rope_table(const GemmParams& p, float* tab, int tid, int nthreads) {
  for (int j = tid; j < kMaxRopePairs; j += nthreads) {
    tab[j] = p.rope.hi[j];
    tab[kMaxRopePairs + j] = p.rope.lo[j];
  }
}

hipError_t launch_gemm(const GemmParams& p, int groups, bool use_bf16, hipStream_t s);

// Few-row (M <= 128) weight-streaming path used by launch_gemm when its layout allows.
bool skinny_supported(const GemmParams& p, int groups);
hipError_t launch_skinny(GemmParams p, int groups, hipStream_t s);
// workspace bytes launch_skinny uses for split-K partials of an M x N x K product
size_t skinny_ws_bytes(int M, int N, int K, int groups);
// Few-row (M <= 256) grouped product with a k-major weight (absorbed queries).
bool kmajor_small_supported(const GemmParams& p, int groups);
hipError_t launch_kmajor_small(const GemmParams& p, int groups, hipStream_t s);
// Many-row (M >= 256) bf16 path: 256 x 256 tiles streamed through LDS.
bool gemm_big_supported(const GemmParams& p, int groups);
// Vectorised epilogue preconditions: 8-element runs never straddle a segment or a head,
// stores are 16-byte aligned, transposed segments see whole 4-token runs of one sequence.
bool gemm_fast_epilogue_ok(const GemmParams& p, int groups);
hipError_t launch_gemm_big(const GemmParams& p, int groups, hipStream_t s);

// ---------------------------------------------------------------------------
// Split-context decode over the latent cache + log-sum-exp combine
// ---------------------------------------------------------------------------
struct DecodeParams {
  const void* q_lat;        // q_lat[(b*H + h)*q_lat_hs + d], d < rb
  const void* q_rope;       // q_rope[(b*H + h)*q_rope_hs + d], d < d_rope (NULL if none)
  int q_lat_hs, q_rope_hs;
  const void* ckv;          // cache latent [max_batch][max_seq][r_kv]
  const void* kr;           // cache rotary key [max_batch][max_seq][d_rope] or NULL
  long long cache_bstride;  // max_seq
  const int* ctx_len;       // [B]: the query attends rows 0..ctx_len[b]
  int B, H, L, hpb;         // hpb = H / L heads per latent block
  int r_kv, rb, d_rope;     // total latent, block width, rotary width
  int chunk;                // tokens per split (multiple of 32)
  int nsplit;               // partial rows per (b, head): splits x sub
  int sub;                  // partial rows per split (4: one per wave of the token-split kernel)
  int head_tiles;           // head tiles per latent block
  float scale_log2;         // softmax scale * log2(e)
  float* part_z;            // [B][H][nsplit][DLP]: fp32 z, or bf16 z / l when part_bf16
  float* part_ml;           // [B][H][nsplit][2]  (running max in log2 units, sum)
  int part_bf16;            // set by the launcher for the split kernel that stores bf16 z / l
  void* z;                  // [B][H][rb] output
};

// Keys of sequence b: ctx_len[b] + 1, clamped to what the cache rows and the splits hold
// (callers keep ctx_len[b] <= max_ctx; the clamp only keeps a bad value from reading past
// the cache or the split partials).
__device__ inline int decode_tokens(const DecodeParams& p, int b) {
  const long long n = (long long)p.ctx_len[b] + 1;
  const long long cap = min((long long)p.cache_bstride, (long long)(p.nsplit / p.sub) * p.chunk);
  return (int)(n < 1 ? 1 : (n > cap ? cap : n));
}

hipError_t launch_decode(const DecodeParams& p, bool use_bf16, int dl_pad, int dr_pad, int nw,
                         hipStream_t s);
bool decode_supported(bool use_bf16, int rb, int d_rope, int hpb, int* dl_pad, int* dr_pad, int* nw);
hipError_t launch_combine(const DecodeParams& p, bool use_bf16, int dl_pad, hipStream_t s);
// Decode step: combine of bf16 partials (part_bf16) fused with o[b][h] = W_UV,h z[b][h]
// (latent 512, d_v 128; o bf16 [B][H][d_v]).
bool combine_uv_supported(const DecodeParams& p, int d_v, const void* w_uv);
hipError_t launch_combine_uv(const DecodeParams& p, int d_v, const void* w_uv, void* o, hipStream_t s);

// bf16 fast path (direct-to-LDS staging, LDS transpose loads): shapes it serves, the
// heads one workgroup covers, and the launch (split kernel only; combine separately).
bool decode_fast_supported(const DecodeParams& p, int* variant);
int decode_fast_head_tile(int variant);
// whether the variant's split kernel stores its partial results as bf16 z / l
bool decode_fast_bf16_partials(int variant);
hipError_t launch_decode_fast(const DecodeParams& p, int variant, hipStream_t s);

// ---------------------------------------------------------------------------
// Flash-style causal prefill
// ---------------------------------------------------------------------------
struct PrefillParams {
  const void* q;            // [B][T][H][dq]: T queries per sequence at positions q_off .. q_off+T-1
  const void* k;            // decompressed keys [B*S][H*dn] (head h at columns h*dn)
  const void* kr;           // rotated shared key rows: kr + (b*kr_bstride + t)*d_rope, or NULL
  long long kr_bstride;
  const void* v;            // values [B*S][H*dv]
  void* o;                  // [B][T][H][dv]
  int B, S, H, dn, d_rope, dv;   // S keys per sequence (positions 0 .. S-1)
  int T, q_off;             // queries per sequence and the position of the first (T = S, 0: prefill)
  float scale_log2;
  int kv_group;             // query heads per key / value head (0 or 1: one each); keys and values
                            // then hold H / kv_group heads and head h reads head h / kv_group
  // training: dropout of the attention weights (keep_thr = 0: none) and the per-row log2
  // normaliser lse[(b H + h) T + i] = log2 sum_j exp2(scale_log2 s_ij) (lse NULL: not written)
  uint32_t keep_thr;        // floor(p 2^32)
  float keep_scale;         // 1 / (1 - p)
  unsigned long long seed;
  float* lse;
};

hipError_t launch_prefill(const PrefillParams& p, bool use_bf16, int dq_pad, int dv_pad, hipStream_t s);

// bf16 flash prefill over head-major keys and transposed values (see prefill_fast.hip).
struct FlashParams {
  const void* q;            // [B][T][H][dn + d_rope]: T queries at positions q_off .. q_off+T-1
  const void* k;            // decompressed keys, head-major [B][H][S][dn]
  const void* kr;           // rotated shared key rows: kr + (b*kr_bstride + t)*d_rope, or NULL
  long long kr_bstride;
  const void* vt;           // values, per head transposed [B][H][dv][S] (perm16 token order)
  void* o;                  // [B][T][H][dv]
  int B, S, H, dn, d_rope;  // S keys per sequence (positions 0 .. S-1)
  int T, q_off;             // queries per sequence and the position of the first (T = S, 0: prefill)
  float scale_log2;
  int ntq;                  // query tiles per (sequence, head); set by the launcher
  int kv_group;             // query heads per key / value head (0 or 1: one each); k and vt
                            // then hold H / kv_group heads
  int dv_out;               // value features stored per head in o (0: all dn; else a multiple of
                            // 32 -- the rest are zero-padding of narrower heads)
  // training forward (dropout on the attention weights, per-row log-sum-exp); zero otherwise
  uint32_t keep_thr;        // keep when a draw's 16-bit field is >= keep_thr (0: no dropout)
  float keep_scale;         // 1 / (1 - p)
  unsigned long long seed;
  float* lse;               // [B][H][T] log2 of each row's softmax normaliser (scaled scores), or NULL
};
bool prefill_fast_supported(int dn, int d_rope, int dv, int S);
hipError_t launch_prefill_fast(const FlashParams& p, hipStream_t s);
bool prefill_supported(bool use_bf16, int dq, int dv, int* dq_pad, int* dv_pad);

// ---------------------------------------------------------------------------
// Compressed convolutional attention (CCA / CCGQA): the step between the packed down-
// projection and attention (causal convolutions, q-k-mean, value shift, QK L2-norm with the
// key temperature, half-split RoPE in the latent)
// ---------------------------------------------------------------------------
struct CcaPrepParams {
  const float* P;           // [B*S][(Hq + Hkv) dh] packed q | k projections (fp32)
  const float* V;           // [B*S][Hkv dh] value projections, unshifted (fp32)
  const void* conv_seq;     // [(Hq + Hkv) dh][kseq]      (element type of the layer)
  const void* conv_ch;      // [(Hq + Hkv) dh][dh][kch]
  void* q;                  // [B*S][Hq][dh]
  void* k;                  // [B*S][Hkv][dh]
  void* v;                  // [B*S][Hkv][dh]
  int B, S, Hq, Hkv, dh;
  int layers, kseq, kch;    // convolutions (0, 1 or 2) and their kernels
  int qk_mean, value_shift;
  float sqrt_dh, key_gain;  // sqrt(d_h) and exp(beta)
  RopeTable rope;           // half-split frequencies of width d_h
  // 0: q / k / v rows [B*S][heads][d_h].  1: the flash prefill layouts with heads padded with
  // zeros to dqp features: q [B*S][Hq][dqp], k head-major [B][Hkv][S][dqp], values transposed
  // per head [B][Hkv][dqp][S] with the tokens of each 16-group in the order 0-3, 8-11, 4-7, 12-15
  int flash, dqp;
};
constexpr int kCcaMaxKernel = 8;
constexpr int kCcaMaxHeadDim = 128;
hipError_t launch_cca_prep(const CcaPrepParams& p, bool use_bf16, hipStream_t s);

// ---------------------------------------------------------------------------
// Flash-style attention backward of the training step (bf16, decoupled-RoPE heads of
// 128 + 64 query / key features and 128 value features, S a multiple of 64)
// ---------------------------------------------------------------------------
struct TrainBwdParams {
  const bf16* q;            // [B*S][H][192] queries (rotary part rotated)
  const bf16* kf;           // [B][H][S][128] decompressed keys, head-major
  const bf16* kr;           // [B*S][64] rotated rotary keys (shared by the heads)
  const bf16* vt;           // [B][H][128][S] values transposed per head (16-token groups 0-3, 8-11, 4-7, 12-15)
  const bf16* dO;           // [B*S][H][128] output gradient (bf16)
  const float* lse;         // [B][H][S] log2 of each row's softmax normaliser (scaled scores)
  const float* D;           // [B][H][S] rowsum(dO o)
  float* dkc;               // [B*S][H][128] key gradient, decompressed part
  float* dkr;               // [B*S][H][64] key gradient, rotary part, per head
  float* dv;                // [B*S][H][128]
  float* dqc;               // [B*S][H][128]
  float* dqr;               // [B*S][H][64]
  int B, S, H;
  float scale_log2, tau;    // tau log2(e), tau (the softmax scale)
  uint32_t keep_thr;        // dropout (0: none)
  float keep_scale;
  unsigned long long seed;
};
bool train_flash_supported(int dn, int d_rope, int dv, int S);
hipError_t launch_train_bwd(const TrainBwdParams& p, hipStream_t s);
hipError_t launch_train_do_prep(const float* dO, const void* o, void* dO16, float* D, int B, int S, int H,
                                hipStream_t s);

// ---------------------------------------------------------------------------
// Training backward
// ---------------------------------------------------------------------------
// C[z] = alpha A[z] B[z] + beta C[z] for Z batches (z = z0 zdiv + z1), element (m, k) of A at
// A + z0 sAz0 + z1 sAz1 + m sAm + k sAk (likewise B (k, n), C (m, n)); A and B fp32 (x_f32 = 1)
// or bf16; products on the MFMA of the launch's element type, fp32 accumulation, fp32 C.
struct SgemmParams {
  const void* A;
  const void* B;
  float* C;
  int M, N, K, Z, zdiv;
  long long sAm, sAk, sBk, sBn, sCm, sCn;
  long long sAz0, sAz1, sBz0, sBz1, sCz0, sCz1;
  int a_f32, b_f32;
  float alpha, beta;
};
hipError_t launch_sgemm(const SgemmParams& p, bool use_bf16, hipStream_t s);

// One query block of the attention backward (queries i0 .. i0+Tq-1 against keys 0 .. Kn-1,
// for the Z = B H (sequence, head) pairs): [z][Tq][Kn] buffers.
struct AttnBwdParams {
  const float* S_;          // scores (bwd_p) or dPd (bwd_ds), fp32
  void* P;                  // softmax weights (element type)
  void* Pd;                 // dropped-out weights (element type)
  void* dS;                 // score gradients times the softmax scale (element type)
  const float* lse;         // [z][S] log2 normalisers from the forward
  const float* D;           // [z][S] rowsum(dO o)
  int Z, S, i0, Tq, Kn;
  float scale_log2, scale;  // softmax scale times log2(e), and the softmax scale
  uint32_t keep_thr;
  float keep_scale;
  unsigned long long seed;
};
hipError_t launch_bwd_p(const AttnBwdParams& p, bool use_bf16, hipStream_t s);
hipError_t launch_bwd_ds(const AttnBwdParams& p, bool use_bf16, hipStream_t s);
hipError_t launch_rowdot(const float* dO, const void* o, float* D, int B, int S, int H, int dv, bool use_bf16,
                         hipStream_t s);
hipError_t launch_rope_bwd(const float* dqr, const float* dkr, float* dqr0, float* dkr0, int B, int S, int H, int dr,
                           const RopeTable& rope, hipStream_t s);
hipError_t launch_fill_f32(float* p, long long n, float v, hipStream_t s);

int device_cu_count();

}  // namespace mla
