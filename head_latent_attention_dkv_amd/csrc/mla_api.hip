// Host side of the C ABI: argument checks, workspace layout and the launch sequence of
// each entry point.  No allocation, no host synchronisation; everything is enqueued on
// the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/mla.h"
#include "common.h"
#include "internal.h"

namespace mla {

void make_rope_table(RopeTable* t, int dim, float base) {
  memset(t, 0, sizeof(*t));
  if (dim <= 0) return;
  for (int j = 0; j < dim / 2 && j < kMaxRopePairs; ++j) {
    double th = pow((double)base, -2.0 * j / (double)dim);
    float hi = (float)th;
    t->hi[j] = hi;
    t->lo[j] = (float)(th - (double)hi);
  }
}

// Compute units of the current device, queried once per device.  The split plans (and so
// the workspace sizes) follow it; mla_workspace_bytes and the launch that uses the workspace
// must therefore run with the same device current.  Without a usable device (a host that
// only sizes buffers) the plans take the 256 compute units of one MI355X.
int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace mla

using namespace mla;

namespace {

constexpr size_t kAlign = 256;
constexpr float kLog2e = 1.4426950408889634f;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_bf16(const mla_dims* d) { return d->dtype == MLA_DTYPE_BF16; }
size_t esize(const mla_dims* d) { return is_bf16(d) ? 2 : 4; }
int rblock(const mla_dims* d) { return d->r_kv / d->n_latent_heads; }
int dq_of(const mla_dims* d) { return d->d_nope + d->d_rope; }

float softmax_scale(const mla_dims* d) {
  if (d->softmax_scale > 0.f) return d->softmax_scale;
  if (d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED) return (float)(1.0 / sqrt((double)(d->d_nope + d->d_rope)));
  return (float)(1.0 / sqrt((double)d->d_nope));
}

// Decode split plan: tokens per split (multiple of 32) and splits per (sequence, head).
// The bf16 fast path covers MLA with a 512-wide latent (+ rotary 64), one workgroup per
// (sequence, split, 64 heads), and MLRA with four latent blocks of 128; either runs one
// workgroup per CU (its LDS pipeline takes most of the CU's 160 KB), so the plan aims at
// whole waves of 256 workgroups.
struct SplitPlan {
  int chunk, nsplit, head_tiles, dl, dr, nw;
  int sub = 1;        // partial rows per split (nsplit counts rows)
  int fast_variant;   // -1: generic kernel
  int fast_head_tiles;
  bool ok;
};

int fast_variant_for(const mla_dims* d) {
  if (!is_bf16(d)) return -1;
  const int L = d->n_latent_heads, hpb = d->n_heads / L;
  if (L == 1 && d->r_kv == 512 && (d->d_rope == 64 || d->d_rope == 0)) return d->d_rope ? 3 : 4;
  if (L == 4 && d->r_kv == 512 && d->d_rope == 0 && hpb <= 16) return 2;
  if (L == 1 && d->r_kv == 128 && d->d_rope == 0) return 5;   // one rank-128 latent block
  return -1;
}

SplitPlan plan_decode(const mla_dims* d, int B, int max_ctx) {
  SplitPlan sp{};
  const int L = d->n_latent_heads, hpb = d->n_heads / L;
  sp.ok = decode_supported(is_bf16(d), rblock(d), d->d_rope, hpb, &sp.dl, &sp.dr, &sp.nw);
  if (!sp.ok) return sp;
  sp.head_tiles = cdiv(hpb, 32 * sp.nw);
  sp.fast_variant = fast_variant_for(d);
  const int kCUs = device_cu_count();
  const int ntok = max_ctx + 1;
  int chunk;
  if (sp.fast_variant >= 0) {
    sp.fast_head_tiles = sp.fast_variant == 2 ? 1 : sp.fast_variant == 5 ? cdiv(hpb, 16) : cdiv(hpb, 128);
    const long long wgs = (long long)B * sp.fast_head_tiles;
    int ns = (int)((kCUs + wgs - 1) / wgs);
    chunk = round_up(cdiv(ntok, ns < 1 ? 1 : ns), 32);
    // MLRA (latent blocks): splits of at most 1536 tokens keep ragged batches balanced over
    // the CUs while each workgroup streams long enough to amortise its start.  Contexts
    // U[512, 16384] at B = 128 (≈800 splits, just over three per CU): 1024 / 1280 / 1536 /
    // 1792 / 2048 tokens took 219 / 215 / 190 / 204 / 242 us per call.
    if (sp.fast_variant == 2 && chunk > 1536) chunk = 1536;
    // token split (four waves on four 32-token slices of 128-token tiles): at most 4096 tokens
    // of 256-byte rows (the MLRA latent-head contexts: caps of 1536 / 2048 / 3072 / 5120 / 6144
    // took 62.6 / 74.1 / 66.7 / 69.5 / 73.8 us per call against 60.5 us)
    if (sp.fast_variant == 5) chunk = min(round_up(chunk, 128), 4096);
  } else {
    const long long wgs = (long long)B * L * sp.head_tiles;
    const int wg_per_cu = sp.nw == 4 ? 1 : 8;
    int ns = (int)((kCUs * wg_per_cu + wgs - 1) / wgs);
    chunk = round_up(cdiv(ntok, ns < 1 ? 1 : ns), 32);
    if (sp.nw == 1 && chunk > 1024) chunk = 1024;
  }
  if (chunk < 32) chunk = 32;
  sp.chunk = chunk;
  sp.nsplit = cdiv(ntok, chunk);
  if (sp.fast_variant == 5) {
    sp.sub = 4;
    sp.nsplit *= 4;
  }
  return sp;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Split kernel (fast path when shapes and alignment allow) followed by the combine.  Given
// w_uv and o (the decode step), the combine also applies the value up-projection when a
// fused kernel serves the shape; *fused_uv says whether it did (z is then not written).
hipError_t run_decode_attention(const mla_dims* d, DecodeParams p, const SplitPlan& sp, hipStream_t st,
                                const void* w_uv = nullptr, void* o = nullptr, bool* fused_uv = nullptr) {
  int variant = -1;
  const bool fast = sp.fast_variant >= 0 && decode_fast_supported(p, &variant) &&
                    aligned16(p.q_lat) && (p.q_lat_hs % 8 == 0) && aligned16(p.ckv) &&
                    (p.d_rope == 0 || (aligned16(p.q_rope) && p.q_rope_hs % 8 == 0 && aligned16(p.kr)));
  hipError_t e;
  p.part_bf16 = 0;
  p.sub = 1;                     // the generic kernel writes one row per split
  if (fast) {
    p.head_tiles = sp.fast_head_tiles;
    p.sub = variant == 5 ? sp.sub : 1;
    p.part_bf16 = decode_fast_bf16_partials(variant) ? 1 : 0;
    e = launch_decode_fast(p, variant, st);
  } else {
    p.head_tiles = sp.head_tiles;
    e = launch_decode(p, is_bf16(d), sp.dl, sp.dr, sp.nw, st);
  }
  if (e != hipSuccess) return e;
  if (fused_uv && w_uv && o && combine_uv_supported(p, d->d_v, w_uv)) {
    *fused_uv = true;
    return launch_combine_uv(p, d->d_v, w_uv, o, st);
  }
  return launch_combine(p, is_bf16(d), sp.dl, st);
}

struct DecodeWs {
  size_t cq, q, qlat, z, o, gsplit, gsplit_bytes, part_z, part_ml, total;
};

// Split-K partial sums of the few-row projections of one decode step (largest of them).
size_t decode_gemm_split_bytes(const mla_dims* d, int B) {
  const bool dec = d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED;
  const int H = d->n_heads;
  const int src_w = (dec && d->r_q > 0) ? d->r_q : d->d_model;
  size_t m = 0;
  auto take = [&](size_t v) { m = v > m ? v : m; };
  if (dec && d->r_q > 0) take(skinny_ws_bytes(B, d->r_q, d->d_model, 1));
  if (dec && d->r_q > 0) take(skinny_ws_bytes(B, d->r_q + d->r_kv + d->d_rope, d->d_model, 1));
  if (d->r_q == 0 && d->d_rope == 0) take(skinny_ws_bytes(B, H * d->d_nope + d->r_kv, d->d_model, 1));
  take(skinny_ws_bytes(B, H * d->d_nope + (dec ? H * d->d_rope : 0), src_w, 1));
  take(skinny_ws_bytes(B, d->r_kv + d->d_rope, d->d_model, 1));
  take(skinny_ws_bytes(B, d->d_v, rblock(d), H));
  take(skinny_ws_bytes(B, d->d_model, H * d->d_v, 1));
  return m;
}

DecodeWs decode_layout(const mla_dims* d, int B, int max_ctx, bool attention_only) {
  DecodeWs w{};
  SplitPlan sp = plan_decode(d, B, max_ctx);
  const size_t es = esize(d);
  const int H = d->n_heads, rb = rblock(d);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  if (!attention_only) {
    w.cq = take(d->r_q > 0 ? (size_t)B * d->r_q * es : 0);
    w.q = take((size_t)B * H * dq_of(d) * es);
    w.qlat = take((size_t)B * H * rb * es);
    w.z = take((size_t)B * H * rb * es);
    w.o = take((size_t)B * H * d->d_v * es);
    w.gsplit_bytes = decode_gemm_split_bytes(d, B);
    w.gsplit = take(w.gsplit_bytes);
  }
  w.part_z = take((size_t)B * H * sp.nsplit * sp.dl * sizeof(float));
  w.part_ml = take((size_t)B * H * sp.nsplit * 2 * sizeof(float));
  w.total = off;
  return w;
}

struct PrefillWs {
  size_t cq, q, lat, latr, k, v, o, total;
};

PrefillWs prefill_layout(const mla_dims* d, int B, int S, bool attention_only) {
  PrefillWs w{};
  const size_t es = esize(d);
  const size_t rows = (size_t)B * S;
  const int H = d->n_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  if (!attention_only) {
    w.cq = take(d->r_q > 0 && d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED ? rows * d->r_q * es : 0);
    w.q = take(rows * H * dq_of(d) * es);
    w.lat = take(rows * d->r_kv * es);
    w.latr = take(rows * d->d_rope * es);
    w.o = take(rows * H * d->d_v * es);
  }
  w.k = take(rows * H * d->d_nope * es);
  w.v = take(rows * H * d->d_v * es);
  w.total = off;
  return w;
}

mla_status check_weights(const mla_dims* d, const mla_weights* w, bool need_q, bool need_kv_up,
                         bool need_out) {
  if (!w) return MLA_ERR_INVALID_ARG;
  if (!w->w_dkv) return MLA_ERR_INVALID_ARG;
  const bool dec = d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED;
  if (dec && !w->w_kr) return MLA_ERR_INVALID_ARG;
  if (need_q) {
    if (dec && d->r_q > 0) {
      if (!w->w_dq || !w->w_uq || !w->w_qr) return MLA_ERR_INVALID_ARG;
    } else {
      if (!w->w_q) return MLA_ERR_INVALID_ARG;
      if (dec && !w->w_qr) return MLA_ERR_INVALID_ARG;
    }
  }
  if (need_kv_up && (!w->w_uk || !w->w_uv)) return MLA_ERR_INVALID_ARG;
  if (need_out && !w->w_o) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status check_cache(const mla_dims* d, const mla_cache* c) {
  if (!c || !c->ckv || c->max_batch <= 0 || c->max_seq <= 0) return MLA_ERR_INVALID_ARG;
  if (d->d_rope > 0 && !c->kr) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

GemmParams gemm_base(const mla_dims* d) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.zdiv = 1;
  p.rows_per_batch = 1;
  p.nseg = 1;
  (void)d;
  return p;
}

GemmSeg plain_seg(const void* w, long long w_ld, int n, void* out, long long out_ld, bool f32) {
  GemmSeg s;
  memset(&s, 0, sizeof(s));
  s.w = w;
  s.w_ld = w_ld;
  s.n = n;
  s.out = out;
  s.out_ld = out_ld;
  s.out_f32 = f32 ? 1 : 0;
  return s;
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

// Scratch for split-K partial sums of few-row projections (none: products run unsplit).
struct SplitWs {
  float* part = nullptr;
  size_t bytes = 0;
};
void use_split(GemmParams& p, const SplitWs& sw) {
  p.part = sw.part;
  p.part_bytes = sw.bytes;
}
const char* atc(const void* base, size_t off) { return static_cast<const char*>(base) + off; }

// c = W_DKV x and k_R = RoPE(W_KR x) for `rows` rows, written to cache rows (b, pos0[b]+t)
// or, without a cache, to plain row-major buffers.
hipError_t run_latent(const mla_dims* d, const mla_weights* w, const void* x, int B, int T,
                      const int32_t* pos0, const mla_cache* cache, void* lat, void* latr,
                      hipStream_t st, const SplitWs& sw = SplitWs()) {
  GemmParams p = gemm_base(d);
  use_split(p, sw);
  p.a = x;
  p.a_ld = d->d_model;
  p.M = B * T;
  p.K = d->d_model;
  p.rows_per_batch = T;
  p.pos0 = pos0;
  const bool bf = is_bf16(d);
  p.seg[0] = plain_seg(w->w_dkv, d->d_model, d->r_kv, cache ? cache->ckv : lat, d->r_kv, false);
  if (cache) {
    p.seg[0].out_cache = 1;
    p.out_bstride = cache->max_seq;
  }
  if (d->d_rope > 0) {
    p.nseg = 2;
    p.seg[1] = plain_seg(w->w_kr, d->d_model, d->d_rope, cache ? cache->kr : latr, d->d_rope, false);
    p.seg[1].out_cache = cache ? 1 : 0;
    p.seg[1].rope = ROPE_INTERLEAVED;
    p.seg[1].rope_d = d->d_rope;
    make_rope_table(&p.rope, d->d_rope, d->rope_base);
  }
  return launch_gemm(p, 1, bf, st);
}

// Queries q[rows][H][d_nope + d_rope] from x (and the query latent when r_q > 0).
hipError_t run_queries(const mla_dims* d, const mla_weights* w, const void* x, int rows,
                       int rows_per_batch, const int32_t* pos0, void* cq, void* q, hipStream_t st,
                       const SplitWs& sw = SplitWs(), bool cq_ready = false) {
  const bool bf = is_bf16(d);
  const int H = d->n_heads, dq = dq_of(d);
  const size_t es = esize(d);
  const bool dec = d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED;
  const void* src = x;
  int src_w = d->d_model;
  hipError_t e;
  if (dec && d->r_q > 0) {
    if (!cq_ready) {
      GemmParams p = gemm_base(d);
      use_split(p, sw);
      p.a = x;
      p.a_ld = d->d_model;
      p.M = rows;
      p.K = d->d_model;
      p.seg[0] = plain_seg(w->w_dq, d->d_model, d->r_q, cq, d->r_q, false);
      e = launch_gemm(p, 1, bf, st);
      if (e != hipSuccess) return e;
    }
    src = cq;
    src_w = d->r_q;
  }
  GemmParams p = gemm_base(d);
  use_split(p, sw);
  p.a = src;
  p.a_ld = src_w;
  p.M = rows;
  p.K = src_w;
  p.rows_per_batch = rows_per_batch;
  p.pos0 = pos0;
  const void* wq = (dec && d->r_q > 0) ? w->w_uq : w->w_q;
  p.seg[0] = plain_seg(wq, src_w, H * d->d_nope, q, (long long)H * dq, false);
  p.seg[0].out_hw = d->d_nope;
  p.seg[0].out_hs = dq;
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) {
    p.seg[0].rope = ROPE_HALFSPLIT;
    p.seg[0].rope_d = d->d_nope;
    make_rope_table(&p.rope, d->d_nope, d->rope_base);
  }
  if (dec) {
    p.nseg = 2;
    p.seg[1] = plain_seg(w->w_qr, src_w, H * d->d_rope, at(q, d->d_nope * es), (long long)H * dq, false);
    p.seg[1].out_hw = d->d_rope;
    p.seg[1].out_hs = dq;
    p.seg[1].rope = ROPE_INTERLEAVED;
    p.seg[1].rope_d = d->d_rope;
    make_rope_table(&p.rope, d->d_rope, d->rope_base);
  }
  return launch_gemm(p, 1, bf, st);
}

// Decode step: the products of the new tokens x in one few-row product with several output
// segments (one launch, one split-K reduce; latent rows go to cache rows (b, pos0[b])):
//   DOWN_CQ  query latent present: c_Q = W_DQ x, c = W_DKV x, k_R = RoPE(W_KR x);
//   DOWN_Q   no query latent and no rotary part (MLRA): q = W_Q x, c = W_DKV x.
// Returns DOWN_NONE, launching nothing, when the shape does not take that path.
enum DownMerge { DOWN_NONE = 0, DOWN_CQ = 1, DOWN_Q = 2 };
DownMerge run_down_proj(const mla_dims* d, const mla_weights* w, const void* x, int B, const int32_t* pos0,
                        const mla_cache* cache, void* cq, void* q, hipStream_t st, const SplitWs& sw,
                        hipError_t* err) {
  if (!is_bf16(d) || B > 128) return DOWN_NONE;
  GemmParams p = gemm_base(d);
  use_split(p, sw);
  p.a = x;
  p.a_ld = d->d_model;
  p.M = B;
  p.K = d->d_model;
  p.rows_per_batch = 1;
  p.pos0 = pos0;
  p.out_bstride = cache->max_seq;
  DownMerge kind;
  if (d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED && d->r_q > 0 && d->d_rope > 0) {
    kind = DOWN_CQ;
    p.nseg = 3;
    p.seg[0] = plain_seg(w->w_dq, d->d_model, d->r_q, cq, d->r_q, false);
    p.seg[1] = plain_seg(w->w_dkv, d->d_model, d->r_kv, cache->ckv, d->r_kv, false);
    p.seg[1].out_cache = 1;
    p.seg[2] = plain_seg(w->w_kr, d->d_model, d->d_rope, cache->kr, d->d_rope, false);
    p.seg[2].out_cache = 1;
    p.seg[2].rope = ROPE_INTERLEAVED;
    p.seg[2].rope_d = d->d_rope;
    make_rope_table(&p.rope, d->d_rope, d->rope_base);
  } else if (d->rope_mode == MLA_ROPE_NONE && d->r_q == 0 && d->d_rope == 0) {
    kind = DOWN_Q;                     // q rows [H][d_nope] are plain rows of H * d_nope
    p.nseg = 2;
    p.seg[0] = plain_seg(w->w_q, d->d_model, d->n_heads * d->d_nope, q, (long long)d->n_heads * d->d_nope, false);
    p.seg[1] = plain_seg(w->w_dkv, d->d_model, d->r_kv, cache->ckv, d->r_kv, false);
    p.seg[1].out_cache = 1;
  } else {
    return DOWN_NONE;
  }
  if (!skinny_supported(p, 1)) return DOWN_NONE;
  *err = launch_gemm(p, 1, true, st);
  return kind;
}

// Explicit keys / values from the latent rows 0..S-1 of each sequence.
// Flash-prefill layouts: keys head-major [B][H][S][dn], values per head transposed
// [B][H][dv][S] (perm16 token order).  Otherwise both [B*S][H][d].
bool use_flash(const mla_dims* d, int S) {
  return is_bf16(d) && prefill_fast_supported(d->d_nope, d->d_rope, d->d_v, S);
}

hipError_t run_kv_up(const mla_dims* d, const mla_weights* w, const void* lat, bool lat_cache,
                     long long lat_bstride, int B, int S, void* k, void* v, hipStream_t st,
                     bool flash_layout) {
  const bool bf = is_bf16(d);
  const int H = d->n_heads, L = d->n_latent_heads, rb = rblock(d);
  const int sub_out = H * d->d_nope / L;
  GemmParams p = gemm_base(d);
  p.a = lat;
  p.a_ld = d->r_kv;
  p.a_cache = lat_cache ? 1 : 0;
  p.a_bstride = lat_bstride;
  p.M = B * S;
  p.K = rb;
  p.rows_per_batch = S;
  p.nseg = 2;
  p.seg[0] = plain_seg(w->w_uk, rb, sub_out, k, (long long)H * d->d_nope, false);
  p.seg[1] = plain_seg(w->w_uv, rb, sub_out, v, (long long)H * d->d_v, false);
  if (flash_layout) {
    p.seg[0].layout = OUT_HEAD_MAJOR;
    p.seg[0].out_hw = d->d_nope;
    p.seg[0].out_nh = H;
    p.seg[1].layout = OUT_HEAD_T16;
    p.seg[1].out_hw = d->d_v;
    p.seg[1].out_nh = H;
    p.seg[1].out_ld = S;
  }
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) {
    p.seg[0].rope = ROPE_HALFSPLIT;
    p.seg[0].rope_d = d->d_nope;
    make_rope_table(&p.rope, d->d_nope, d->rope_base);
  }
  // latent block g feeds output columns [g*sub_out, (g+1)*sub_out)
  p.zdiv = 1;
  p.a_goff[0] = rb;
  p.w_goff[0] = (long long)sub_out * rb;
  p.o_goff[0] = sub_out;
  return launch_gemm(p, L, bf, st);
}

// Per head h (block g, index hi in the block): out[:, h*out_w ...] = A_h . W_h, with W_h
// the head's rows of a (block) up-projection, read k-major (absorb) or [out][in] (W_UV).
hipError_t run_per_head(const mla_dims* d, const void* a, long long a_ld, long long a_head,
                        int K, const void* wmat, bool kmajor, int n, void* out, long long out_ld,
                        long long out_head, int B, hipStream_t st, const SplitWs& sw = SplitWs()) {
  const int H = d->n_heads, L = d->n_latent_heads, hpb = H / L, rb = rblock(d);
  const int sub_out = H * d->d_nope / L;
  GemmParams p = gemm_base(d);
  use_split(p, sw);
  p.a = a;
  p.a_ld = a_ld;
  p.M = B;
  p.K = K;
  p.w_kmajor = kmajor ? 1 : 0;
  p.seg[0] = plain_seg(wmat, rb, n, out, out_ld, false);
  p.zdiv = hpb;
  p.a_goff[0] = a_head * hpb;
  p.a_goff[1] = a_head;
  p.w_goff[0] = (long long)sub_out * rb;
  p.w_goff[1] = (long long)d->d_nope * rb;
  p.o_goff[0] = out_head * hpb;
  p.o_goff[1] = out_head;
  return launch_gemm(p, H, is_bf16(d), st);
}

hipError_t run_out_proj(const mla_dims* d, const mla_weights* w, const void* o, int rows, float* y,
                        hipStream_t st, const SplitWs& sw = SplitWs()) {
  GemmParams p = gemm_base(d);
  use_split(p, sw);
  const int hv = d->n_heads * d->d_v;
  p.a = o;
  p.a_ld = hv;
  p.M = rows;
  p.K = hv;
  p.seg[0] = plain_seg(w->w_o, hv, d->d_model, y, d->d_model, true);
  return launch_gemm(p, 1, is_bf16(d), st);
}

hipError_t run_flash(const mla_dims* d, const void* q, const void* k, const void* kr, long long kr_bstride,
                     const void* vt, void* o, int B, int S, int T, int q_off, hipStream_t st) {
  FlashParams fp;
  memset(&fp, 0, sizeof(fp));
  fp.q = q;
  fp.k = k;
  fp.kr = d->d_rope > 0 ? kr : nullptr;
  fp.kr_bstride = kr_bstride;
  fp.vt = vt;
  fp.o = o;
  fp.B = B;
  fp.S = S;
  fp.T = T;
  fp.q_off = q_off;
  fp.H = d->n_heads;
  fp.dn = d->d_nope;
  fp.d_rope = d->d_rope;
  fp.scale_log2 = softmax_scale(d) * kLog2e;
  return launch_prefill_fast(fp, st);
}

DecodeParams decode_params(const mla_dims* d, const mla_cache* cache, const int32_t* ctx_len,
                           int B, int max_ctx, void* ws, const DecodeWs& lay) {
  SplitPlan sp = plan_decode(d, B, max_ctx);
  DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.ckv = cache->ckv;
  p.kr = cache->kr;
  p.cache_bstride = cache->max_seq;
  p.ctx_len = ctx_len;
  p.B = B;
  p.H = d->n_heads;
  p.L = d->n_latent_heads;
  p.hpb = d->n_heads / d->n_latent_heads;
  p.r_kv = d->r_kv;
  p.rb = rblock(d);
  p.d_rope = d->d_rope;
  p.chunk = sp.chunk;
  p.nsplit = sp.nsplit;
  p.sub = 1;
  p.head_tiles = sp.head_tiles;
  p.scale_log2 = softmax_scale(d) * kLog2e;
  p.part_z = reinterpret_cast<float*>(at(ws, lay.part_z));
  p.part_ml = reinterpret_cast<float*>(at(ws, lay.part_ml));
  return p;
}

// ---------------------------------------------------------------------------
// Scratch of mla_decode_attention_noalloc: a file-scope device array of fixed size, one copy
// per GPU, held until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is a stand-in, not a device address): its address on each device comes
// from hipGetSymbolAddress, taken once per device on the entry point's first call there.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (nullptr and *err set on failure).
void* scratch_for_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !ptr) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// v[i] = value for i < n (a device array of per-sequence start positions)
__global__ void fill_i32_kernel(int32_t* v, int n, int32_t value) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) v[i] = value;
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_CAPACITY: return "MLA_ERR_CAPACITY";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

mla_status mla_validate(const mla_dims* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->d_model <= 0 || d->n_heads <= 0 || d->d_nope <= 0 || d->d_v <= 0 || d->r_kv <= 0 ||
      d->r_q < 0 || d->d_rope < 0 || d->n_latent_heads <= 0)
    return MLA_ERR_INVALID_ARG;
  if (d->dtype != MLA_DTYPE_F32 && d->dtype != MLA_DTYPE_BF16) return MLA_ERR_INVALID_ARG;
  if (d->rope_mode < MLA_ROPE_NONE || d->rope_mode > MLA_ROPE_FULL_HALFSPLIT) return MLA_ERR_INVALID_ARG;
  if (!(d->softmax_scale == d->softmax_scale)) return MLA_ERR_INVALID_ARG;
  // Family rules of the pages.
  if (d->rope_mode == MLA_ROPE_DECOUPLED_INTERLEAVED) {
    if (d->d_rope <= 0 || (d->d_rope & 1)) return MLA_ERR_SHAPE;    // even rotary dim
  } else if (d->d_rope != 0) {
    return MLA_ERR_SHAPE;
  }
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT && (d->d_nope & 1)) return MLA_ERR_SHAPE;
  if (d->rope_mode != MLA_ROPE_NONE && !(d->rope_base > 0.f)) return MLA_ERR_INVALID_ARG;
  if (d->n_latent_heads > 1) {
    if (d->r_kv % d->n_latent_heads) return MLA_ERR_SHAPE;          // L | latent rank
    if (d->n_heads % d->n_latent_heads) return MLA_ERR_SHAPE;       // L | heads
    if (d->rope_mode != MLA_ROPE_NONE) return MLA_ERR_UNSUPPORTED;  // partitioned latent has no RoPE
  }
  // Kernel limits.
  if (d->d_v != d->d_nope) return MLA_ERR_UNSUPPORTED;
  if (d->d_nope % 8) return MLA_ERR_UNSUPPORTED;
  if (d->d_rope > 64) return MLA_ERR_UNSUPPORTED;
  if (d->d_rope > 0 && (d->r_kv & 1)) return MLA_ERR_UNSUPPORTED;
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT && (128 % d->d_nope)) return MLA_ERR_UNSUPPORTED;
  int a, b;
  if (!prefill_supported(is_bf16(d), dq_of(d), d->d_v, &a, &b)) return MLA_ERR_UNSUPPORTED;
  if (d->rope_mode != MLA_ROPE_FULL_HALFSPLIT) {
    int x, y, z;
    if (!decode_supported(is_bf16(d), rblock(d), d->d_rope, d->n_heads / d->n_latent_heads, &x, &y, &z))
      return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

size_t mla_workspace_bytes(const mla_dims* d, int op, int32_t batch, int32_t seq) {
  if (mla_validate(d) != MLA_OK || batch <= 0 || seq < 0) return 0;
  switch (op) {
    case MLA_OP_CACHE_APPEND: return 0;
    case MLA_OP_PREFILL: return seq > 0 ? prefill_layout(d, batch, seq, false).total : 0;
    case MLA_OP_PREFILL_ATTENTION: return seq > 0 ? prefill_layout(d, batch, seq, true).total : 0;
    case MLA_OP_PREFILL_CHUNK: return seq > 0 ? prefill_layout(d, batch, seq, false).total + align_up((size_t)batch * 4) : 0;
    case MLA_OP_DECODE:
      if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) return 0;
      return decode_layout(d, batch, seq, false).total;
    case MLA_OP_DECODE_ATTENTION:
      if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) return 0;
      return decode_layout(d, batch, seq, true).total;
    default: return 0;
  }
}

mla_status mla_cache_append(const mla_dims* d, const mla_weights* w, const void* x, int32_t B,
                            int32_t T, const int32_t* start_pos_dev, int32_t max_start,
                            const mla_cache* cache, void* stream) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (!x || !start_pos_dev || B <= 0 || T <= 0 || max_start < 0) return MLA_ERR_INVALID_ARG;
  if ((s = check_weights(d, w, false, false, false)) != MLA_OK) return s;
  if ((s = check_cache(d, cache)) != MLA_OK) return s;
  if (B > cache->max_batch || (long long)max_start + T > cache->max_seq) return MLA_ERR_CAPACITY;
  return hip_status(run_latent(d, w, x, B, T, start_pos_dev, cache, nullptr, nullptr,
                               static_cast<hipStream_t>(stream)));
}

mla_status mla_prefill_attention(const mla_dims* d, const mla_weights* w, const void* q,
                                 int32_t B, int32_t S, const mla_cache* cache, void* o,
                                 void* ws, size_t ws_bytes, void* stream) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (!q || !o || B <= 0 || S <= 0 || !w || !w->w_uk || !w->w_uv) return MLA_ERR_INVALID_ARG;
  if ((s = check_cache(d, cache)) != MLA_OK) return s;
  if (B > cache->max_batch || S > cache->max_seq) return MLA_ERR_CAPACITY;
  PrefillWs lay = prefill_layout(d, B, S, true);
  if (!ws || ws_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* k = at(ws, lay.k);
  void* v = at(ws, lay.v);
  const bool flash = use_flash(d, S);
  hipError_t e = run_kv_up(d, w, cache->ckv, true, cache->max_seq, B, S, k, v, st, flash);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (flash) return hip_status(run_flash(d, q, k, cache->kr, cache->max_seq, v, o, B, S, S, 0, st));
  int dqp, dvp;
  prefill_supported(is_bf16(d), dq_of(d), d->d_v, &dqp, &dvp);
  PrefillParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = q;
  pp.k = k;
  pp.kr = cache->kr;
  pp.kr_bstride = cache->max_seq;
  pp.v = v;
  pp.o = o;
  pp.B = B;
  pp.S = S;
  pp.T = S;
  pp.q_off = 0;
  pp.H = d->n_heads;
  pp.dn = d->d_nope;
  pp.d_rope = d->d_rope;
  pp.dv = d->d_v;
  pp.scale_log2 = softmax_scale(d) * kLog2e;
  return hip_status(launch_prefill(pp, is_bf16(d), dqp, dvp, st));
}

mla_status mla_prefill(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, int32_t S,
                       const mla_cache* cache, float* y, void* ws, size_t ws_bytes, void* stream) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (!x || !y || B <= 0 || S <= 0) return MLA_ERR_INVALID_ARG;
  if ((s = check_weights(d, w, true, true, true)) != MLA_OK) return s;
  if (cache) {
    if ((s = check_cache(d, cache)) != MLA_OK) return s;
    if (B > cache->max_batch || S > cache->max_seq) return MLA_ERR_CAPACITY;
  }
  PrefillWs lay = prefill_layout(d, B, S, false);
  if (!ws || ws_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  void* q = at(ws, lay.q);
  e = run_queries(d, w, x, B * S, S, nullptr, at(ws, lay.cq), q, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  void* lat = at(ws, lay.lat);
  void* latr = at(ws, lay.latr);
  e = run_latent(d, w, x, B, S, nullptr, cache, lat, latr, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  void* k = at(ws, lay.k);
  void* v = at(ws, lay.v);
  const bool flash = use_flash(d, S);
  if (cache)
    e = run_kv_up(d, w, cache->ckv, true, cache->max_seq, B, S, k, v, st, flash);
  else
    e = run_kv_up(d, w, lat, false, 0, B, S, k, v, st, flash);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (flash) {
    void* o = at(ws, lay.o);
    e = run_flash(d, q, k, cache ? cache->kr : latr, cache ? cache->max_seq : S, v, o, B, S, S, 0, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    return hip_status(run_out_proj(d, w, o, B * S, y, st));
  }
  int dqp, dvp;
  prefill_supported(is_bf16(d), dq_of(d), d->d_v, &dqp, &dvp);
  PrefillParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = q;
  pp.k = k;
  pp.kr = cache ? cache->kr : latr;
  pp.kr_bstride = cache ? cache->max_seq : S;
  pp.v = v;
  pp.o = at(ws, lay.o);
  pp.B = B;
  pp.S = S;
  pp.T = S;
  pp.q_off = 0;
  pp.H = d->n_heads;
  pp.dn = d->d_nope;
  pp.d_rope = d->d_rope;
  pp.dv = d->d_v;
  pp.scale_log2 = softmax_scale(d) * kLog2e;
  e = launch_prefill(pp, is_bf16(d), dqp, dvp, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return hip_status(run_out_proj(d, w, pp.o, B * S, y, st));
}

mla_status mla_prefill_chunk(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, int32_t T,
                             int32_t start_pos, const mla_cache* cache, float* y, void* ws, size_t ws_bytes,
                             void* stream) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (!x || !y || B <= 0 || T <= 0 || start_pos < 0) return MLA_ERR_INVALID_ARG;
  if ((s = check_weights(d, w, true, true, true)) != MLA_OK) return s;
  if ((s = check_cache(d, cache)) != MLA_OK) return s;
  if (B > cache->max_batch || (long long)start_pos + T > cache->max_seq) return MLA_ERR_CAPACITY;
  const int S = start_pos + T;                      // keys per sequence: cached + new
  PrefillWs lay = prefill_layout(d, B, S, false);
  const size_t pos_off = lay.total;
  if (!ws || ws_bytes < pos_off + align_up((size_t)B * 4)) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  // per-sequence start rows for the append and the query rotation
  int32_t* pos = reinterpret_cast<int32_t*>(at(ws, pos_off));
  hipLaunchKernelGGL(fill_i32_kernel, dim3(cdiv(B, 256)), dim3(256), 0, st, pos, B, start_pos);
  if ((e = hipGetLastError()) != hipSuccess) return MLA_ERR_HIP;
  void* q = at(ws, lay.q);
  if ((e = run_queries(d, w, x, B * T, T, pos, at(ws, lay.cq), q, st)) != hipSuccess) return MLA_ERR_HIP;
  if ((e = run_latent(d, w, x, B, T, pos, cache, nullptr, nullptr, st)) != hipSuccess) return MLA_ERR_HIP;
  // keys and values of every cached row 0..S-1, then the new queries over them
  void* k = at(ws, lay.k);
  void* v = at(ws, lay.v);
  void* o = at(ws, lay.o);
  const bool flash = use_flash(d, S) && start_pos % 64 == 0;
  if ((e = run_kv_up(d, w, cache->ckv, true, cache->max_seq, B, S, k, v, st, flash)) != hipSuccess)
    return MLA_ERR_HIP;
  if (flash) {
    e = run_flash(d, q, k, cache->kr, cache->max_seq, v, o, B, S, T, start_pos, st);
  } else {
    int dqp, dvp;
    prefill_supported(is_bf16(d), dq_of(d), d->d_v, &dqp, &dvp);
    PrefillParams pp;
    memset(&pp, 0, sizeof(pp));
    pp.q = q;
    pp.k = k;
    pp.kr = cache->kr;
    pp.kr_bstride = cache->max_seq;
    pp.v = v;
    pp.o = o;
    pp.B = B;
    pp.S = S;
    pp.T = T;
    pp.q_off = start_pos;
    pp.H = d->n_heads;
    pp.dn = d->d_nope;
    pp.d_rope = d->d_rope;
    pp.dv = d->d_v;
    pp.scale_log2 = softmax_scale(d) * kLog2e;
    e = launch_prefill(pp, is_bf16(d), dqp, dvp, st);
  }
  if (e != hipSuccess) return MLA_ERR_HIP;
  return hip_status(run_out_proj(d, w, o, B * T, y, st));
}

mla_status mla_decode_attention_noalloc(const mla_dims* d, const void* q_lat, const void* q_rope, int32_t B,
                                        const int32_t* ctx_len_dev, int32_t max_ctx, const mla_cache* cache,
                                        void* z, void* stream) {
  // the same checks as mla_decode_attention, then the scratch size, all before any HIP call
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) return MLA_ERR_UNSUPPORTED;
  if (!q_lat || !z || !ctx_len_dev || B <= 0 || max_ctx < 0) return MLA_ERR_INVALID_ARG;
  if (d->d_rope > 0 && !q_rope) return MLA_ERR_INVALID_ARG;
  if ((s = check_cache(d, cache)) != MLA_OK) return s;
  if (B > cache->max_batch || (long long)max_ctx + 1 > cache->max_seq) return MLA_ERR_CAPACITY;
  const size_t need = decode_layout(d, B, max_ctx, true).total;
  if (need > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
  hipError_t e;
  void* ws = scratch_for_current_device(&e);
  if (!ws) return MLA_ERR_HIP;
  return mla_decode_attention(d, q_lat, q_rope, B, ctx_len_dev, max_ctx, cache, z, ws, need, stream);
}

size_t mla_decode_attention_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

mla_status mla_decode_attention(const mla_dims* d, const void* q_lat, const void* q_rope, int32_t B,
                                const int32_t* ctx_len_dev, int32_t max_ctx, const mla_cache* cache,
                                void* z, void* ws, size_t ws_bytes, void* stream) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) return MLA_ERR_UNSUPPORTED;
  if (!q_lat || !z || !ctx_len_dev || B <= 0 || max_ctx < 0) return MLA_ERR_INVALID_ARG;
  if (d->d_rope > 0 && !q_rope) return MLA_ERR_INVALID_ARG;
  if ((s = check_cache(d, cache)) != MLA_OK) return s;
  if (B > cache->max_batch || (long long)max_ctx + 1 > cache->max_seq) return MLA_ERR_CAPACITY;
  DecodeWs lay = decode_layout(d, B, max_ctx, true);
  if (!ws || ws_bytes < lay.total) return MLA_ERR_WORKSPACE;
  DecodeParams p = decode_params(d, cache, ctx_len_dev, B, max_ctx, ws, lay);
  p.q_lat = q_lat;
  p.q_lat_hs = rblock(d);
  p.q_rope = q_rope;
  p.q_rope_hs = d->d_rope;
  p.z = z;
  SplitPlan sp = plan_decode(d, B, max_ctx);
  return hip_status(run_decode_attention(d, p, sp, static_cast<hipStream_t>(stream)));
}

mla_status mla_decode(const mla_dims* d, const mla_weights* w, const void* x, int32_t B,
                      const int32_t* ctx_len_dev, int32_t max_ctx, const mla_cache* cache, float* y,
                      void* ws, size_t ws_bytes, void* stream) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (d->rope_mode == MLA_ROPE_FULL_HALFSPLIT) return MLA_ERR_UNSUPPORTED;
  if (!x || !y || !ctx_len_dev || B <= 0 || max_ctx < 0) return MLA_ERR_INVALID_ARG;
  if ((s = check_weights(d, w, true, true, true)) != MLA_OK) return s;
  if ((s = check_cache(d, cache)) != MLA_OK) return s;
  if (B > cache->max_batch || (long long)max_ctx + 1 > cache->max_seq) return MLA_ERR_CAPACITY;
  DecodeWs lay = decode_layout(d, B, max_ctx, false);
  if (!ws || ws_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = d->n_heads, dq = dq_of(d), rb = rblock(d);
  const size_t es = esize(d);
  hipError_t e;
  SplitWs sw;
  sw.part = reinterpret_cast<float*>(at(ws, lay.gsplit));
  sw.bytes = lay.gsplit_bytes;
  void* q = at(ws, lay.q);
  // 1. the query latent and the new latent / rotary key (appended at row ctx_len[b]) in one
  //    product where the shape allows, then the queries rotated at position ctx_len[b]
  const DownMerge merged = run_down_proj(d, w, x, B, ctx_len_dev, cache, at(ws, lay.cq), q, st, sw, &e);
  if (merged != DOWN_NONE && e != hipSuccess) return MLA_ERR_HIP;
  if (merged != DOWN_Q) {
    e = run_queries(d, w, x, B, 1, ctx_len_dev, at(ws, lay.cq), q, st, sw, merged == DOWN_CQ);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  // 2. otherwise append the new latent / rotary key at row ctx_len[b] here
  if (merged == DOWN_NONE) {
    e = run_latent(d, w, x, B, 1, ctx_len_dev, cache, nullptr, nullptr, st, sw);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  // 3. absorbed query q_lat[b][h] = W_UK,h^T q_C[b][h]
  void* qlat = at(ws, lay.qlat);
  e = run_per_head(d, q, (long long)H * dq, dq, d->d_nope, w->w_uk, true, rb, qlat,
                   (long long)H * rb, rb, B, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // 4. split-context attention over the latent cache + combine
  DecodeParams p = decode_params(d, cache, ctx_len_dev, B, max_ctx, ws, lay);
  p.q_lat = qlat;
  p.q_lat_hs = rb;
  p.q_rope = d->d_rope > 0 ? atc(q, d->d_nope * es) : nullptr;
  p.q_rope_hs = dq;
  void* z = at(ws, lay.z);
  p.z = z;
  SplitPlan sp = plan_decode(d, B, max_ctx);
  void* o = at(ws, lay.o);
  bool fused_uv = false;
  e = run_decode_attention(d, p, sp, st, w->w_uv, o, &fused_uv);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // 5. o[b][h] = W_UV,h z[b][h] (unless fused into the combine), then y = W_O o
  if (!fused_uv) {
    e = run_per_head(d, z, (long long)H * rb, rb, rb, w->w_uv, false, d->d_v, o,
                     (long long)H * d->d_v, d->d_v, B, st, sw);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  return hip_status(run_out_proj(d, w, o, B, y, st, sw));
}

}  // extern "C"

// ===========================================================================================
// Training: forward with dropout on the attention weights, and its backward ([DSV2 page]
// MultiHeadLatentAttention, [MLA page] MLAAttention: trainable modules with dropout after the
// softmax).  Decoupled-RoPE family with a query latent.
// ===========================================================================================
namespace {

struct TrainSaved {
  size_t cq, q, c, kr, kc, v, o, lse, total;
};

TrainSaved train_saved_layout(const mla_dims* d, int B, int S) {
  TrainSaved t{};
  const size_t rows = (size_t)B * S, es = esize(d);
  const int H = d->n_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  t.cq = take(rows * d->r_q * es);
  t.q = take(rows * H * dq_of(d) * es);
  t.c = take(rows * d->r_kv * es);
  t.kr = take(rows * d->d_rope * es);
  t.kc = take(rows * H * d->d_nope * es);
  t.v = take(rows * H * d->d_v * es);
  t.o = take(rows * H * d->d_v * es);
  t.lse = take((size_t)B * H * S * 4);
  t.total = off;
  return t;
}

// Queries per block of the attention backward: at most 256, and the [B H][Tq][S] fp32 score
// block within ~2 GiB.
int train_query_block(const mla_dims* d, int B, int S) {
  const long long z = (long long)B * d->n_heads;
  long long tq = (2ll << 30) / (4ll * z * S);
  tq = tq >= 64 ? tq / 64 * 64 : (tq < 1 ? 1 : tq);
  if (tq > 256) tq = 256;
  return (int)(tq < S ? tq : S);
}

// The bf16 decoupled-RoPE heads of 128 + 64 features over whole 64-token tiles train on the
// flash kernels: the forward on the flash prefill kernel with dropout (keys and values saved
// in its head-major / transposed layouts), the attention backward on train_bwd_kv_kernel and
// train_bwd_q_kernel.  Other shapes use the generic prefill kernel and the blockwise
// backward below.
bool train_flash(const mla_dims* d, int S) {
  return is_bf16(d) && train_flash_supported(d->d_nope, d->d_rope, d->d_v, S) &&
         prefill_fast_supported(d->d_nope, d->d_rope, d->d_v, S);
}

struct TrainWs {
  size_t dO, D, dqc, dqr, dkc, dkr, dv, dqr0, dkr0, dcq, dc, sbuf, pbuf, pdbuf, dsbuf, dO16, total;
  int tq;
};

TrainWs train_ws_layout(const mla_dims* d, int B, int S) {
  TrainWs w{};
  const size_t rows = (size_t)B * S, es = esize(d);
  const int H = d->n_heads, dn = d->d_nope, dr = d->d_rope, dv = d->d_v;
  const bool flash = train_flash(d, S);
  w.tq = train_query_block(d, B, S);
  const size_t blk = flash ? 0 : (size_t)B * H * w.tq * S;   // score blocks of the blockwise backward
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  w.dO = take(rows * H * dv * 4);
  w.D = take((size_t)B * H * S * 4);
  w.dqc = take(rows * H * dn * 4);
  w.dqr = take(rows * H * dr * 4);
  w.dkc = take(rows * H * dn * 4);
  w.dkr = take(rows * H * dr * 4);
  w.dv = take(rows * H * dv * 4);
  w.dqr0 = take(rows * H * dr * 4);
  w.dkr0 = take(rows * dr * 4);
  w.dcq = take(rows * d->r_q * 4);
  w.dc = take(rows * d->r_kv * 4);
  w.sbuf = take(blk * 4);
  w.pbuf = take(blk * es);
  w.pdbuf = take(blk * es);
  w.dsbuf = take(blk * es);
  w.dO16 = take(flash ? rows * H * dv * 2 : 0);
  w.total = off;
  return w;
}

mla_status train_check(const mla_dims* d, float p, int B, int S) {
  mla_status s = mla_validate(d);
  if (s != MLA_OK) return s;
  if (d->rope_mode != MLA_ROPE_DECOUPLED_INTERLEAVED || d->r_q <= 0 || d->n_latent_heads != 1) return MLA_ERR_UNSUPPORTED;
  if (!(p >= 0.f && p < 1.f)) return MLA_ERR_INVALID_ARG;
  // the dropout counter packs (b H + h, query, key / 4) into 26, 20 and 18 bits
  if ((long long)B * d->n_heads > (1ll << 24) || S > (1 << 20)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// keep when the 16-bit field of the draw is >= floor(p 2^16)
uint32_t keep_threshold(float p) {
  const double t = floor((double)p * 65536.0);
  return t >= 65535.0 ? 65535u : (uint32_t)t;
}

// one strided product (batch 1) of the backward
SgemmParams sg(const void* A, bool a_f32, long long sAm, long long sAk, const void* Bm, bool b_f32, long long sBk,
               long long sBn, float* C, long long sCm, int M, int N, int K, float beta) {
  SgemmParams g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.B = Bm;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.Z = 1;
  g.zdiv = 1;
  g.sAm = sAm;
  g.sAk = sAk;
  g.sBk = sBk;
  g.sBn = sBn;
  g.sCm = sCm;
  g.sCn = 1;
  g.a_f32 = a_f32 ? 1 : 0;
  g.b_f32 = b_f32 ? 1 : 0;
  g.alpha = 1.f;
  g.beta = beta;
  return g;
}

}  // namespace

extern "C" {

size_t mla_train_saved_bytes(const mla_dims* d, int32_t B, int32_t S) {
  if (B <= 0 || S <= 0 || train_check(d, 0.f, B, S) != MLA_OK) return 0;
  return train_saved_layout(d, B, S).total;
}

size_t mla_train_workspace_bytes(const mla_dims* d, int32_t B, int32_t S) {
  if (B <= 0 || S <= 0 || train_check(d, 0.f, B, S) != MLA_OK) return 0;
  return train_ws_layout(d, B, S).total;
}

mla_status mla_train_forward(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, int32_t S,
                             float dropout_p, uint64_t seed, float* y, void* saved, size_t saved_bytes, void* stream) {
  mla_status s = train_check(d, dropout_p, B, S);
  if (s != MLA_OK) return s;
  if (!x || !y || B <= 0 || S <= 0) return MLA_ERR_INVALID_ARG;
  if ((s = check_weights(d, w, true, true, true)) != MLA_OK) return s;
  const TrainSaved sv = train_saved_layout(d, B, S);
  if (!saved || saved_bytes < sv.total) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int M = B * S;
  if (run_queries(d, w, x, M, S, nullptr, at(saved, sv.cq), at(saved, sv.q), st) != hipSuccess) return MLA_ERR_HIP;
  if (run_latent(d, w, x, B, S, nullptr, nullptr, at(saved, sv.c), at(saved, sv.kr), st) != hipSuccess) return MLA_ERR_HIP;
  const bool flash = train_flash(d, S);
  if (run_kv_up(d, w, at(saved, sv.c), false, 0, B, S, at(saved, sv.kc), at(saved, sv.v), st, flash) != hipSuccess)
    return MLA_ERR_HIP;
  if (flash) {
    FlashParams fp;
    memset(&fp, 0, sizeof(fp));
    fp.q = at(saved, sv.q);
    fp.k = at(saved, sv.kc);
    fp.kr = at(saved, sv.kr);
    fp.kr_bstride = S;
    fp.vt = at(saved, sv.v);
    fp.o = at(saved, sv.o);
    fp.B = B;
    fp.S = S;
    fp.T = S;
    fp.q_off = 0;
    fp.H = d->n_heads;
    fp.dn = d->d_nope;
    fp.d_rope = d->d_rope;
    fp.scale_log2 = softmax_scale(d) * kLog2e;
    fp.keep_thr = keep_threshold(dropout_p);
    fp.keep_scale = (float)(1.0 / (1.0 - (double)dropout_p));
    fp.seed = seed;
    fp.lse = reinterpret_cast<float*>(at(saved, sv.lse));
    if (launch_prefill_fast(fp, st) != hipSuccess) return MLA_ERR_HIP;
    return hip_status(run_out_proj(d, w, at(saved, sv.o), M, y, st));
  }
  int dqp, dvp;
  if (!prefill_supported(is_bf16(d), dq_of(d), d->d_v, &dqp, &dvp)) return MLA_ERR_UNSUPPORTED;
  PrefillParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = at(saved, sv.q);
  pp.k = at(saved, sv.kc);
  pp.kr = at(saved, sv.kr);
  pp.kr_bstride = S;
  pp.v = at(saved, sv.v);
  pp.o = at(saved, sv.o);
  pp.B = B;
  pp.S = S;
  pp.T = S;
  pp.H = d->n_heads;
  pp.dn = d->d_nope;
  pp.d_rope = d->d_rope;
  pp.dv = d->d_v;
  pp.scale_log2 = softmax_scale(d) * kLog2e;
  pp.keep_thr = keep_threshold(dropout_p);
  pp.keep_scale = (float)(1.0 / (1.0 - (double)dropout_p));
  pp.seed = seed;
  pp.lse = reinterpret_cast<float*>(at(saved, sv.lse));
  if (launch_prefill(pp, is_bf16(d), dqp, dvp, st) != hipSuccess) return MLA_ERR_HIP;
  return hip_status(run_out_proj(d, w, at(saved, sv.o), M, y, st));
}

mla_status mla_train_backward(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, int32_t S,
                              float dropout_p, uint64_t seed, const float* dy, const void* saved, size_t saved_bytes,
                              const mla_grads* g, void* ws, size_t ws_bytes, void* stream) {
  mla_status s = train_check(d, dropout_p, B, S);
  if (s != MLA_OK) return s;
  if (!x || !dy || !g || B <= 0 || S <= 0) return MLA_ERR_INVALID_ARG;
  if (!g->dx || !g->dw_dq || !g->dw_uq || !g->dw_qr || !g->dw_dkv || !g->dw_kr || !g->dw_uk || !g->dw_uv || !g->dw_o)
    return MLA_ERR_INVALID_ARG;
  if ((s = check_weights(d, w, true, true, true)) != MLA_OK) return s;
  const TrainSaved sv = train_saved_layout(d, B, S);
  if (!saved || saved_bytes < sv.total) return MLA_ERR_WORKSPACE;
  const TrainWs lw = train_ws_layout(d, B, S);
  if (!ws || ws_bytes < lw.total) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = is_bf16(d);
  const size_t es = esize(d);
  const int H = d->n_heads, dn = d->d_nope, dr = d->d_rope, dv = d->d_v, dq = dq_of(d);
  const int E = d->d_model, rq = d->r_q, rkv = d->r_kv;
  const int M = B * S;
  const long long HD = (long long)H * dn, HR = (long long)H * dr, HV = (long long)H * dv, HQ = (long long)H * dq;
  auto F = [&](size_t off) { return reinterpret_cast<float*>(at(ws, off)); };
  const char* sd = static_cast<const char*>(saved);
  const void *cq = sd + sv.cq, *q = sd + sv.q, *c = sd + sv.c, *kr = sd + sv.kr, *kc = sd + sv.kc;
  const void *v = sd + sv.v, *o = sd + sv.o;
  const float* lse = reinterpret_cast<const float*>(sd + sv.lse);
  float *dO = F(lw.dO), *D = F(lw.D), *dqc = F(lw.dqc), *dqr = F(lw.dqr), *dkc = F(lw.dkc), *dkr = F(lw.dkr);
  float *dV = F(lw.dv), *dqr0 = F(lw.dqr0), *dkr0 = F(lw.dkr0), *dcq = F(lw.dcq), *dc = F(lw.dc);
#define MLA_TRY(expr) \
  do {                \
    if ((expr) != hipSuccess) return MLA_ERR_HIP; \
  } while (0)
  auto GEMM = [&](const SgemmParams& p) { return launch_sgemm(p, bf, st); };
  const bool tf = !bf;   // storage flag of weights and saved tensors: fp32 when the layer is fp32

  // output projection y = o W_o^T:  dW_o = dy^T o,  dO = dy W_o
  MLA_TRY(GEMM(sg(dy, true, 1, E, o, tf, HV, 1, g->dw_o, HV, E, (int)HV, M, 0.f)));
  MLA_TRY(GEMM(sg(dy, true, E, 1, w->w_o, tf, HV, 1, dO, HV, M, (int)HV, E, 0.f)));
  const float tau = softmax_scale(d);
  if (train_flash(d, S)) {
    // flash backward: keys / values as saved in the flash layouts (head-major keys, values
    // transposed per head)
    void* dO16 = at(ws, lw.dO16);
    MLA_TRY(launch_train_do_prep(dO, o, dO16, D, B, S, H, st));
    TrainBwdParams tb;
    memset(&tb, 0, sizeof(tb));
    tb.q = static_cast<const bf16*>(q);
    tb.kf = static_cast<const bf16*>(kc);
    tb.kr = static_cast<const bf16*>(kr);
    tb.vt = static_cast<const bf16*>(v);
    tb.dO = static_cast<const bf16*>(dO16);
    tb.lse = lse;
    tb.D = D;
    tb.dkc = dkc;
    tb.dkr = dkr;
    tb.dv = dV;
    tb.dqc = dqc;
    tb.dqr = dqr;
    tb.B = B;
    tb.S = S;
    tb.H = H;
    tb.scale_log2 = tau * kLog2e;
    tb.tau = tau;
    tb.keep_thr = keep_threshold(dropout_p);
    tb.keep_scale = (float)(1.0 / (1.0 - (double)dropout_p));
    tb.seed = seed;
    MLA_TRY(launch_train_bwd(tb, st));
  } else {
    MLA_TRY(launch_rowdot(dO, o, D, B, S, H, dv, bf, st));
    MLA_TRY(launch_fill_f32(dkc, (long long)M * HD, 0.f, st));
    MLA_TRY(launch_fill_f32(dkr, (long long)M * HR, 0.f, st));
    MLA_TRY(launch_fill_f32(dV, (long long)M * HV, 0.f, st));

    // attention, one block of queries at a time for every (sequence, head) pair z = b H + h
    const int tq = lw.tq;
    AttnBwdParams ab;
    memset(&ab, 0, sizeof(ab));
    ab.S_ = F(lw.sbuf);
    ab.P = at(ws, lw.pbuf);
    ab.Pd = at(ws, lw.pdbuf);
    ab.dS = at(ws, lw.dsbuf);
    ab.lse = lse;
    ab.D = D;
    ab.Z = B * H;
    ab.S = S;
    ab.scale_log2 = tau * kLog2e;
    ab.scale = tau;
    ab.keep_thr = keep_threshold(dropout_p);
    ab.keep_scale = (float)(1.0 / (1.0 - (double)dropout_p));
    ab.seed = seed;
    // batched operand views: a [rows][H][width] tensor has batch strides (S H width, width)
    auto batched = [&](SgemmParams p, long long az0, long long az1, long long bz0, long long bz1, long long cz0,
                       long long cz1) {
      p.Z = B * H;
      p.zdiv = H;
      p.sAz0 = az0;
      p.sAz1 = az1;
      p.sBz0 = bz0;
      p.sBz1 = bz1;
      p.sCz0 = cz0;
      p.sCz1 = cz1;
      return p;
    };
    for (int i0 = 0; i0 < S; i0 += tq) {
      const int T = S - i0 < tq ? S - i0 : tq;          // queries of this block
      const int Kn = i0 + T;                            // keys they can see
      const long long blk = (long long)tq * Kn;         // [Tq][Kn] block of one (sequence, head)
      const char* qb = static_cast<const char*>(q) + (size_t)i0 * HQ * es;
      ab.i0 = i0;
      ab.Tq = tq;
      ab.Kn = Kn;
      // scores S = q_C k_C^T + q_R k_R^T (unscaled)
      MLA_TRY(GEMM(batched(sg(qb, tf, HQ, 1, kc, tf, 1, HD, F(lw.sbuf), Kn, T, Kn, dn, 0.f),
                           (long long)S * HQ, dq, (long long)S * HD, dn, (long long)H * blk, blk)));
      MLA_TRY(GEMM(batched(sg(static_cast<const char*>(qb) + (size_t)dn * es, tf, HQ, 1, kr, tf, 1, dr, F(lw.sbuf), Kn,
                              T, Kn, dr, 1.f),
                           (long long)S * HQ, dq, (long long)S * dr, 0, (long long)H * blk, blk)));
      MLA_TRY(launch_bwd_p(ab, bf, st));
      // dV[0:Kn] += Pd^T dO_blk
      const float* dOb = dO + (size_t)i0 * HV;
      MLA_TRY(GEMM(batched(sg(ab.Pd, tf, 1, Kn, dOb, true, HV, 1, dV, HV, Kn, dv, T, 1.f), (long long)H * blk, blk,
                           (long long)S * HV, dv, (long long)S * HV, dv)));
      // dPd = dO_blk V^T  (into the score buffer)
      MLA_TRY(GEMM(batched(sg(dOb, true, HV, 1, v, tf, 1, HV, F(lw.sbuf), Kn, T, Kn, dv, 0.f), (long long)S * HV, dv,
                           (long long)S * HV, dv, (long long)H * blk, blk)));
      MLA_TRY(launch_bwd_ds(ab, bf, st));
      // dq_blk = dS k:  decompressed part and rotary part (k_R shared by the heads)
      MLA_TRY(GEMM(batched(sg(ab.dS, tf, Kn, 1, kc, tf, HD, 1, dqc + (size_t)i0 * HD, HD, T, dn, Kn, 0.f),
                           (long long)H * blk, blk, (long long)S * HD, dn, (long long)S * HD, dn)));
      MLA_TRY(GEMM(batched(sg(ab.dS, tf, Kn, 1, kr, tf, dr, 1, dqr + (size_t)i0 * HR, HR, T, dr, Kn, 0.f),
                           (long long)H * blk, blk, (long long)S * dr, 0, (long long)S * HR, dr)));
      // dk[0:Kn] += dS^T q_blk (per head; the rotary parts are summed over heads below)
      MLA_TRY(GEMM(batched(sg(ab.dS, tf, 1, Kn, qb, tf, HQ, 1, dkc, HD, Kn, dn, T, 1.f), (long long)H * blk, blk,
                           (long long)S * HQ, dq, (long long)S * HD, dn)));
      MLA_TRY(GEMM(batched(sg(ab.dS, tf, 1, Kn, static_cast<const char*>(qb) + (size_t)dn * es, tf, HQ, 1, dkr, HR,
                              Kn, dr, T, 1.f),
                           (long long)H * blk, blk, (long long)S * HQ, dq, (long long)S * HR, dr)));
    }
  }

  // rotary parts back through the rotations (negative angle); k_R summed over heads
  RopeTable rope;
  make_rope_table(&rope, dr, d->rope_base);
  MLA_TRY(launch_rope_bwd(dqr, dkr, dqr0, dkr0, B, S, H, dr, rope, st));
  // query path: q_C = c_Q W_UQ^T, q_R0 = c_Q W_QR^T, c_Q = x W_DQ^T
  MLA_TRY(GEMM(sg(dqc, true, 1, HD, cq, tf, rq, 1, g->dw_uq, rq, (int)HD, rq, M, 0.f)));
  MLA_TRY(GEMM(sg(dqr0, true, 1, HR, cq, tf, rq, 1, g->dw_qr, rq, (int)HR, rq, M, 0.f)));
  MLA_TRY(GEMM(sg(dqc, true, HD, 1, w->w_uq, tf, rq, 1, dcq, rq, M, rq, (int)HD, 0.f)));
  MLA_TRY(GEMM(sg(dqr0, true, HR, 1, w->w_qr, tf, rq, 1, dcq, rq, M, rq, (int)HR, 1.f)));
  MLA_TRY(GEMM(sg(dcq, true, 1, rq, x, tf, E, 1, g->dw_dq, E, rq, E, M, 0.f)));
  // key / value path: k_C = c W_UK^T, v = c W_UV^T, c = x W_DKV^T, k_R0 = x W_KR^T
  MLA_TRY(GEMM(sg(dkc, true, 1, HD, c, tf, rkv, 1, g->dw_uk, rkv, (int)HD, rkv, M, 0.f)));
  MLA_TRY(GEMM(sg(dV, true, 1, HV, c, tf, rkv, 1, g->dw_uv, rkv, (int)HV, rkv, M, 0.f)));
  MLA_TRY(GEMM(sg(dkc, true, HD, 1, w->w_uk, tf, rkv, 1, dc, rkv, M, rkv, (int)HD, 0.f)));
  MLA_TRY(GEMM(sg(dV, true, HV, 1, w->w_uv, tf, rkv, 1, dc, rkv, M, rkv, (int)HV, 1.f)));
  MLA_TRY(GEMM(sg(dc, true, 1, rkv, x, tf, E, 1, g->dw_dkv, E, rkv, E, M, 0.f)));
  MLA_TRY(GEMM(sg(dkr0, true, 1, dr, x, tf, E, 1, g->dw_kr, E, dr, E, M, 0.f)));
  // dx = dc_Q W_DQ + dc W_DKV + dk_R0 W_KR
  MLA_TRY(GEMM(sg(dcq, true, rq, 1, w->w_dq, tf, E, 1, g->dx, E, M, E, rq, 0.f)));
  MLA_TRY(GEMM(sg(dc, true, rkv, 1, w->w_dkv, tf, E, 1, g->dx, E, M, E, rkv, 1.f)));
  MLA_TRY(GEMM(sg(dkr0, true, dr, 1, w->w_kr, tf, E, 1, g->dx, E, M, E, dr, 1.f)));
#undef MLA_TRY
  return MLA_OK;
}

}  // extern "C"
