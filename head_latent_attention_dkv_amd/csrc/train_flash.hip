// Flash-style attention backward of the training step for the decoupled-RoPE heads of the
// DSV2 page's MultiHeadLatentAttention (bf16; queries and keys of 128 decompressed + 64 rotary
// features, the rotary key shared by the heads; values of 128), causal, with the dropout mask
// redrawn from the forward's generator counters.  With P = 2^(scale_log2 s - lse) the
// softmax weights recomputed from the forward's per-row log-sum-exp, keep the mask and
// 1 / (1 - p) its scale:
//   dV = (P keep)^T dO / (1 - p),   dP = dO V^T,   dS = P (dP keep / (1 - p) - D),
//   dK = tau dS^T Q,   dQ = tau dS K,   D = rowsum(dO o).
// Two kernels, so that no output is accumulated by more than one workgroup:
//   * train_bwd_kv_kernel: one workgroup per (sequence, head, 128 keys), 4 waves of 32 keys;
//     the wave keeps its keys' K and V as MFMA operands in registers and its dK, dV
//     accumulators, and walks the 32-query tiles from the diagonal to the end (Q, dO, lse and
//     D tiles staged in LDS, double-buffered through registers);
//   * train_bwd_q_kernel: one workgroup per (sequence, head, 128 queries), 4 waves of 32
//     queries; the wave keeps its queries' Q and dO in registers and its dQ accumulators, and
//     walks the 64-key tiles up to the diagonal (K and V tiles staged in LDS).
// Operand orientation: kernel A computes S and dP with a lane per key (the accumulator
// column), which is the A operand of dV += P^T dO and dK += dS^T Q once converted to bf16;
// kernel B computes S^T and dP^T with a lane per query, the B operand of dQ^T += K^T dS^T.
// In both, an accumulator's k slots (rows 4h..4h+3 and 8+4h..8+4h+3 of each 16-row step,
// h = lane / 32) are matched on the other operand by LDS transpose reads
// (ds_read_b64_tr_b16) at rows 4h and 4h + 8.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int TDN = 128, TDR = 64, TDQ = TDN + TDR, TDV = 128;
constexpr int QLD = TDQ + 8;      // LDS row strides (elements): rows 400 B / 272 B apart keep
constexpr int OLD = TDV + 8;      // the 16-row operand reads and the transpose reads on
constexpr int KLD = TDQ + 8;      // distinct banks
constexpr int VLD = TDV + 8;
constexpr int AQT = 32;           // queries per tile (kernel A)
constexpr int AKB = 128;          // keys per workgroup (kernel A)
constexpr int BKT = 64;           // keys per tile (kernel B)
constexpr int BQB = 128;          // queries per workgroup (kernel B)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Operand from a row-major [k rows][n cols] bf16 LDS tile by two transpose reads: the lane gets
// column col0 + lane % 32 at k rows row0 + {4h .. 4h+3, 8+4h .. 8+4h+3} (h = lane / 32), the
// order of an accumulator's rows.
__device__ __forceinline__ Frag<bf16> tr_frag(const bf16* tile, int ld, int row0, int col0, int lane) {
  const int k16 = lane & 15, g16 = lane >> 4, half = lane >> 5;
  const int r = row0 + 4 * half + (k16 >> 2);
  const int c = col0 + 16 * (g16 & 1) + 4 * (k16 & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + r * ld + c));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + (r + 8) * ld + c));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, v);
  return f;
}

// the 64-bit value of lane SRC of this lane's quad (DPP quad permutation)
template <int SRC>
__device__ __forceinline__ uint64_t quad_bcast(uint64_t v) {
  constexpr int ctrl = SRC * 0x55;   // quad_perm(SRC, SRC, SRC, SRC)
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, ctrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), ctrl, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// value slot of token t in the values' transposed layout (16-groups in the order 0-3, 8-11,
// 4-7, 12-15: slots 4-7 and 8-11 swapped; the map is its own inverse)
__device__ __forceinline__ int perm16(int t) {
  const int u = t & 15;
  return (t & ~15) | ((u >= 4 && u < 8) ? u + 4 : (u >= 8 && u < 12) ? u - 4 : u);
}

// ---------------------------------------------------------------------------------------
// Kernel A: dK, dV
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256, 1) train_bwd_kv_kernel(TrainBwdParams p) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][AQT * QLD];
  __shared__ __attribute__((aligned(16))) bf16 Os[2][AQT * OLD];
  __shared__ __attribute__((aligned(16))) float Ls[2][AQT];
  __shared__ __attribute__((aligned(16))) float Dm[2][AQT];
  __shared__ __attribute__((aligned(16))) bf16 Vk[AKB * VLD];   // the block's values, [key][dv]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S, H = p.H;
  const int nkb = cdiv(S, AKB);
  // block -> (sequence, head, key block): each (sequence, head) group on one XCD (blocks go
  // to the XCDs in turn), its key blocks in ascending order (the first ones see the most
  // queries: longest first)
  const int L = blockIdx.x, ngroups = p.B * H;
  int g, kb;
  if (ngroups % 8 == 0) {
    const int x = L & 7, slot = L >> 3;
    g = (slot / nkb) * 8 + x;
    kb = slot % nkb;
  } else {
    g = L / nkb;
    kb = L % nkb;
  }
  const int h = g % H, b = g / H;
  const long long bh = (long long)b * H + h;
  const int k0 = kb * AKB;
  const int kw = k0 + 32 * wave;            // this wave's first key
  const int key = kw + col;                 // this lane's key (accumulator column)
  const int keyc = min(key, S - 1);

  // K (decompressed | rotary) of the lane's key as B operands in registers: k slots =
  // features 16 ks + 8 half .. + 7
  Frag<bf16> kf[TDQ / 16];
#pragma unroll
  for (int ks = 0; ks < TDN / 16; ++ks) kf[ks] = frag_load(p.kf + (bh * S + keyc) * TDN + 16 * ks + 8 * half);
#pragma unroll
  for (int ks = 0; ks < TDR / 16; ++ks)
    kf[TDN / 16 + ks] = frag_load(p.kr + ((long long)b * S + keyc) * TDR + 16 * ks + 8 * half);
  // the block's values, de-permuted into LDS as [key][dv] (their B operands are read from
  // there: registers are short); rows past S are clamped copies, never used
  {
    constexpr int NVC = TDV * (AKB / 8) / 256;   // 16-byte chunks per thread
#pragma unroll
    for (int i = 0; i < NVC; ++i) {
      const int c = tid + 256 * i, d = c / (AKB / 8), u = c - d * (AKB / 8);
      const int s0 = min(k0 + 8 * u, S - 8);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(p.vt + (bh * TDV + d) * S + s0);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vk[perm16(8 * u + j) * VLD + d] = v[j];
    }
  }

  f32x16 dk[TDQ / 32], dv[TDV / 32];
#pragma unroll
  for (int i = 0; i < TDQ / 32; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < TDV / 32; ++i) dv[i] = f32x16{};

  // tile staging: 32 query rows of Q (24 chunks of 16 B) and dO (16 chunks), plus lse and D
  constexpr int QCH = TDQ / 8, OCH = TDV / 8, RCH = QCH + OCH, NCH = AQT * RCH / 256;   // 5 per thread
  static_assert(AQT * RCH % 256 == 0, "staging chunks split evenly");
  // (the staged registers are plain locals of the loop body below: an array captured by a
  // lambda stays in scratch memory)
  // Chunk i of a thread is a Q chunk for i < NQC and a dO chunk after (the split is a
  // compile-time fact: 768 Q chunks and 512 dO chunks per tile); its offset inside the tile's
  // rows is fixed, so a tile costs one add per chunk.  Rows of query q: (b S + q) H + h.
  constexpr int NQC = AQT * QCH / 256, NOC_ = AQT * OCH / 256;
  static_assert(NQC * 256 == AQT * QCH && NOC_ * 256 == AQT * OCH && NQC + NOC_ == NCH, "typed chunks");
  int goff[NCH], loff[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (i < NQC) {
      const int c = tid + 256 * i, r = c / QCH, u = c - r * QCH;
      goff[i] = r * H * TDQ + 8 * u;
      loff[i] = r * QLD + 8 * u;
    } else {
      const int c = tid + 256 * (i - NQC), r = c / OCH, u = c - r * OCH;
      goff[i] = r * H * TDV + 8 * u;
      loff[i] = r * OLD + 8 * u;
    }
  }
  const bf16* qbase = p.q + ((long long)b * S * H + h) * TDQ;     // query 0 of (b, h)
  const bf16* obase = p.dO + ((long long)b * S * H + h) * TDV;
#define MLA_A_GLOAD(qt_, pre, pre_s)                                                          \
  {                                                                                           \
    const int q0_ = (qt_) * AQT;                                                              \
    const bf16* qt_base = qbase + (long long)q0_ * H * TDQ;                                   \
    const bf16* ot_base = obase + (long long)q0_ * H * TDV;                                   \
    _Pragma("unroll") for (int i = 0; i < NCH; ++i)                                           \
      pre[i] = *reinterpret_cast<const bf16x8*>((i < NQC ? qt_base : ot_base) + goff[i]);     \
    if (tid < AQT) pre_s = p.lse[bh * S + q0_ + tid];                                         \
    else if (tid < 2 * AQT) pre_s = p.D[bh * S + q0_ + tid - AQT];                            \
  }
#define MLA_A_LSTORE(buf_, pre, pre_s)                                                        \
  {                                                                                           \
    _Pragma("unroll") for (int i = 0; i < NCH; ++i)                                           \
      *reinterpret_cast<bf16x8*>(i < NQC ? &Qs[buf_][loff[i]] : &Os[buf_][loff[i]]) = pre[i]; \
    if (tid < AQT) Ls[buf_][tid] = pre_s;                                                     \
    else if (tid < 2 * AQT) Dm[buf_][tid - AQT] = pre_s;                                      \
  }
  // the accumulators live in accumulation registers across tiles (without this the compiler
  // keeps them in VGPRs for the products and parks them in AGPRs between tiles: 320 copies
  // per tile)
#define MLA_A_PIN()                                                         \
  {                                                                         \
    _Pragma("unroll") for (int i = 0; i < TDQ / 32; ++i) asm volatile("" : "+a"(dk[i])); \
    _Pragma("unroll") for (int i = 0; i < TDV / 32; ++i) asm volatile("" : "+a"(dv[i])); \
  }
  // Tile loop: the global loads of tile qt + 1 are in flight while tile qt is computed.
#define MLA_A_TILE(buf, qt) \
    if (qt * AQT + AQT - 1 >= kw) { /* else every query of the tile is before the wave's keys */ \
      const int q0 = qt * AQT; \
      const bf16* Q = Qs[buf]; \
      const bf16* O = Os[buf]; \
      /* S[q][key] = Q K^T and dP[q][key] = dO V^T (A operands: query row col of the tile) */ \
      f32x16 sa = f32x16{}, dpa = f32x16{}; \
_Pragma("unroll") \
      for (int ks = 0; ks < TDQ / 16; ++ks) sa = mma32(frag_load(Q + col * QLD + 16 * ks + 8 * half), kf[ks], sa); \
_Pragma("unroll") \
      for (int ks = 0; ks < TDV / 16; ++ks) \
        dpa = mma32(frag_load(O + col * OLD + 16 * ks + 8 * half), frag_load(Vk + (32 * wave + col) * VLD + 16 * ks + 8 * half), \
                    dpa); \
      /* element e: query q0 + qr(e), qr(e) = 8 (e / 4) + 4 half + e % 4; key: the lane's */ \
      /* keep bits: the four lanes of a quad hold four consecutive keys (one draw per query); */ \
      /* lane r of the quad draws for the queries of e = r, r + 4, r + 8, r + 12 and the quad */ \
      /* shares them */ \
      unsigned keep = 0xFFFFu; \
      if (p.keep_thr) { \
        /* the draws' states step by additions: + 8 queries per group (dstate: this tile's */ \
        /* first, for query q0 + 4 half + col % 4 and key / 4) */ \
        uint64_t dr[4]; \
_Pragma("unroll") \
        for (int g4 = 0; g4 < 4; ++g4) \
          dr[g4] = splitmix_mix(dstate + (uint64_t)(8 * g4) * ((1ull << 18) * kSplitmixGamma)); \
        const int sh = 16 * (col & 3); \
        keep = 0; \
_Pragma("unroll") \
        for (int g4 = 0; g4 < 4; ++g4) { \
          const uint64_t d0 = quad_bcast<0>(dr[g4]), d1 = quad_bcast<1>(dr[g4]); \
          const uint64_t d2 = quad_bcast<2>(dr[g4]), d3 = quad_bcast<3>(dr[g4]); \
          keep |= (((uint32_t)(d0 >> sh) & 0xFFFFu) >= p.keep_thr ? 1u : 0u) << (4 * g4 + 0); \
          keep |= (((uint32_t)(d1 >> sh) & 0xFFFFu) >= p.keep_thr ? 1u : 0u) << (4 * g4 + 1); \
          keep |= (((uint32_t)(d2 >> sh) & 0xFFFFu) >= p.keep_thr ? 1u : 0u) << (4 * g4 + 2); \
          keep |= (((uint32_t)(d3 >> sh) & 0xFFFFu) >= p.keep_thr ? 1u : 0u) << (4 * g4 + 3); \
        } \
      } \
      __builtin_amdgcn_sched_barrier(0); \
      const float kscale = p.keep_thr ? p.keep_scale : 1.f; \
      float pd[16], ds[16]; \
_Pragma("unroll") \
      for (int g4 = 0; g4 < 4; ++g4) { \
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][8 * g4 + 4 * half]); \
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dm[buf][8 * g4 + 4 * half]); \
_Pragma("unroll") \
        for (int j = 0; j < 4; ++j) { \
          const int e = 4 * g4 + j, qi = q0 + 8 * g4 + 4 * half + j; \
          const float pv = key <= qi ? __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], p.scale_log2, -l4[j])) : 0.f; \
          const bool kp = (keep >> e) & 1u; \
          pd[e] = kp ? pv : 0.f; \
          ds[e] = pv * ((kp ? dpa[e] * kscale : 0.f) - d4[j]); \
        } \
      } \
      /* dV[key][dv] += Pd^T dO and dK[key][f] += dS^T Q over the tile's two 16-query steps */ \
      /* (sched_barrier: each product's operand read stays next to it, which bounds the live */ \
      /* registers) */ \
      const Frag<bf16> pf0 = frag_from_f32<bf16>(pd), pf1 = frag_from_f32<bf16>(pd + 8); \
      const Frag<bf16> sf0 = frag_from_f32<bf16>(ds), sf1 = frag_from_f32<bf16>(ds + 8); \
      __builtin_amdgcn_sched_barrier(0); \
_Pragma("unroll") \
      for (int db = 0; db < TDV / 32; ++db) { \
        dv[db] = mma32(pf0, tr_frag(O, OLD, 0, 32 * db, lane), dv[db]); \
        dv[db] = mma32(pf1, tr_frag(O, OLD, 16, 32 * db, lane), dv[db]); \
        __builtin_amdgcn_sched_barrier(0); \
      } \
_Pragma("unroll") \
      for (int fb = 0; fb < TDQ / 32; ++fb) { \
        dk[fb] = mma32(sf0, tr_frag(Q, QLD, 0, 32 * fb, lane), dk[fb]); \
        dk[fb] = mma32(sf1, tr_frag(Q, QLD, 16, 32 * fb, lane), dk[fb]); \
        __builtin_amdgcn_sched_barrier(0); \
      } \
    }
  bf16x8 pa[NCH];
  float pa_s = 0.f;

  const int qt0 = k0 / AQT, nqt = S / AQT;
  // dropout draw state of tile qt0 for query qt0 AQT + 4 half + col % 4 and the lane's key
  // group (stepped by AQT queries per tile)
  uint64_t dstate = splitmix_state(p.seed, dropout_counter4((int)bh, qt0 * AQT + 4 * half + (col & 3), key >> 2));
  MLA_A_GLOAD(qt0, pa, pa_s);
  MLA_A_LSTORE(0, pa, pa_s);
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) MLA_A_GLOAD(qt + 1, pa, pa_s);
    MLA_A_TILE(buf, qt);
    dstate += (uint64_t)AQT * ((1ull << 18) * kSplitmixGamma);
    if (qt + 1 < nqt) MLA_A_LSTORE(buf ^ 1, pa, pa_s);
    MLA_A_PIN();
    __syncthreads();
  }
#undef MLA_A_TILE
#undef MLA_A_PIN
#undef MLA_A_GLOAD
#undef MLA_A_LSTORE

  // accumulator element e of lane l: key kw + 8 (e / 4) + 4 half + e % 4, feature / value
  // column 32 block + col
  const float vscale = p.keep_thr ? p.keep_scale : 1.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int kr_ = kw + 8 * (e >> 2) + 4 * half + (e & 3);
    if (kr_ >= S) continue;
    const long long row = ((long long)b * S + kr_) * H + h;
#pragma unroll
    for (int db = 0; db < TDV / 32; ++db) p.dv[row * TDV + 32 * db + col] = dv[db][e] * vscale;
#pragma unroll
    for (int fb = 0; fb < TDN / 32; ++fb) p.dkc[row * TDN + 32 * fb + col] = dk[fb][e] * p.tau;
#pragma unroll
    for (int fb = TDN / 32; fb < TDQ / 32; ++fb) p.dkr[row * TDR + 32 * fb - TDN + col] = dk[fb][e] * p.tau;
  }
}

// ---------------------------------------------------------------------------------------
// Kernel B: dQ
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256, 1) train_bwd_q_kernel(TrainBwdParams p) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BKT * KLD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BKT * VLD];
  __shared__ __attribute__((aligned(16))) bf16 Ob[BQB * OLD];    // the block's dO rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S, H = p.H;
  const int nqb = cdiv(S, BQB);
  // block -> (sequence, head, query block): groups on one XCD, the last query blocks (the most
  // keys) first
  const int L = blockIdx.x, ngroups = p.B * H;
  int g, qrev;
  if (ngroups % 8 == 0) {
    const int x = L & 7, slot = L >> 3;
    g = (slot / nqb) * 8 + x;
    qrev = slot % nqb;
  } else {
    g = L / nqb;
    qrev = L % nqb;
  }
  const int qblk = nqb - 1 - qrev;
  const int h = g % H, b = g / H;
  const long long bh = (long long)b * H + h;
  const int q0 = qblk * BQB;
  const int qw = q0 + 32 * wave;            // this wave's first query
  const int qi = qw + col;                  // this lane's query (accumulator column)
  const int qic = min(qi, S - 1);

  // Q of the lane's query as B operands in registers (k slots: features 16 ks + 8 half ..
  // + 7); the block's dO rows in LDS (their B operands are read from there)
  Frag<bf16> qf[TDQ / 16];
  const long long qrow = ((long long)b * S + qic) * H + h;
#pragma unroll
  for (int ks = 0; ks < TDQ / 16; ++ks) qf[ks] = frag_load(p.q + qrow * TDQ + 16 * ks + 8 * half);
  {
    constexpr int NOC = BQB * (TDV / 8) / 256;   // 16-byte chunks per thread
#pragma unroll
    for (int i = 0; i < NOC; ++i) {
      const int c = tid + 256 * i, r = c / (TDV / 8), u = c - r * (TDV / 8);
      const long long orow = ((long long)b * S + min(q0 + r, S - 1)) * H + h;
      *reinterpret_cast<bf16x8*>(&Ob[r * OLD + 8 * u]) = *reinterpret_cast<const bf16x8*>(p.dO + orow * TDV + 8 * u);
    }
  }
  const float lse_q = p.lse[bh * S + qic], d_q = p.D[bh * S + qic];

  f32x16 dq[TDQ / 32];
#pragma unroll
  for (int i = 0; i < TDQ / 32; ++i) dq[i] = f32x16{};

  // tile staging: 64 key rows of K (16 decompressed + 8 rotary chunks of 16 B each) and the
  // values of 64 keys from the transposed layout (128 value rows x 8 chunks of 8 tokens)
  constexpr int KCH = TDQ / 8, NKC = BKT * KCH, NVC = TDV * (BKT / 8);
  constexpr int NCH = (NKC + NVC) / 256;   // 10 per thread
  static_assert((NKC + NVC) % 256 == 0 && NKC % 256 == 0, "staging chunks split evenly");
  // Chunk i of a thread: decompressed-key chunks for i < 4, rotary-key chunks for i < 6,
  // value chunks after (1024 + 512 + 1024 per tile); offsets fixed, one add per chunk a tile.
  constexpr int NKN = BKT * (TDN / 8) / 256, NKR = BKT * (TDR / 8) / 256, NVV = TDV * (BKT / 8) / 256;
  static_assert(NKN * 256 == BKT * (TDN / 8) && NKR * 256 == BKT * (TDR / 8) && NVV * 256 == TDV * (BKT / 8) &&
                NKN + NKR + NVV == NCH, "typed chunks");
  int goff[NCH], loff[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (i < NKN) {
      const int c = tid + 256 * i, r = c / (TDN / 8), u = c - r * (TDN / 8);
      goff[i] = r * TDN + 8 * u;
      loff[i] = r * KLD + 8 * u;
    } else if (i < NKN + NKR) {
      const int c = tid + 256 * (i - NKN), r = c / (TDR / 8), u = c - r * (TDR / 8);
      goff[i] = r * TDR + 8 * u;
      loff[i] = r * KLD + TDN + 8 * u;
    } else {
      const int c = tid + 256 * (i - NKN - NKR), d = c >> 3, u = c & 7;
      goff[i] = d * S + 8 * u;
      loff[i] = (d << 3) | u;          // value row d, slot group u (stored element by element)
    }
  }
  const bf16* kfb = p.kf + bh * S * TDN;                 // key 0 of (b, h)
  const bf16* krb = p.kr + (long long)b * S * TDR;
  const bf16* vtb = p.vt + bh * TDV * S;
#define MLA_B_GLOAD(kt_)                                                                          \
  {                                                                                               \
    const int kt0_ = (kt_) * BKT;                                                                 \
    _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                                             \
      const bf16* src = i < NKN ? kfb + (long long)kt0_ * TDN : i < NKN + NKR ? krb + (long long)kt0_ * TDR \
                                                                                : vtb + kt0_;     \
      pre[i] = *reinterpret_cast<const bf16x8*>(src + goff[i]);                                   \
    }                                                                                             \
  }
#define MLA_B_LSTORE(buf_)                                                                        \
  {                                                                                               \
    _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                                             \
      if (i < NKN + NKR) {                                                                        \
        *reinterpret_cast<bf16x8*>(&Ks[buf_][loff[i]]) = pre[i];                                  \
      } else {                                                                                    \
        /* value row d, slots 8 u .. 8 u + 7 of the tile -> keys perm16(slot), column d */        \
        const int d = loff[i] >> 3, u = loff[i] & 7;                                              \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) Vs[buf_][perm16(8 * u + j) * VLD + d] = pre[i][j]; \
      }                                                                                           \
    }                                                                                             \
  }
  bf16x8 pre[NCH];

  // dropout draw state of the current key tile for the lane's query and keys kt0 + 4 half ..
  // (stepped by BKT / 4 draws per tile)
  uint64_t dstate = splitmix_state(p.seed, dropout_counter4((int)bh, qi, half));
  auto compute = [&](int buf, int kt) {
    const int kt0 = kt * BKT;
    const bf16* K = Ks[buf];
    const bf16* V = Vs[buf];
#pragma unroll
    for (int kh = 0; kh < BKT / 32; ++kh) {
      const int kb0 = kt0 + 32 * kh;
      if (kb0 > qw + 31) break;             // every key of the half is after the wave's queries
      // S^T[key][q] = K Q^T and dP^T[key][q] = V dO^T (A operands: key row col of the half)
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int ks = 0; ks < TDQ / 16; ++ks)
        st = mma32(frag_load(K + (32 * kh + col) * KLD + 16 * ks + 8 * half), qf[ks], st);
#pragma unroll
      for (int ks = 0; ks < TDV / 16; ++ks)
        dpt = mma32(frag_load(V + (32 * kh + col) * VLD + 16 * ks + 8 * half),
                    frag_load(Ob + (32 * wave + col) * OLD + 16 * ks + 8 * half), dpt);
      // element e: key kb0 + 8 (e / 4) + 4 half + e % 4, query: the lane's; one draw per
      // four consecutive keys
      float ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int kg = kb0 + 8 * g4 + 4 * half;
        // draw for keys kg .. kg + 3: the tile's state stepped by (kb0 - kt0 + 8 g4) / 4
        const uint64_t dr =
            p.keep_thr ? splitmix_mix(dstate + (uint64_t)(8 * kh + 2 * g4) * kSplitmixGamma) : 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * g4 + j;
          const float pv =
              kg + j <= qi ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], p.scale_log2, -lse_q)) : 0.f;
          const bool kp = !p.keep_thr || (((uint32_t)(dr >> (16 * j)) & 0xFFFFu) >= p.keep_thr);
          ds[e] = pv * ((kp ? dpt[e] * (p.keep_thr ? p.keep_scale : 1.f) : 0.f) - d_q);
        }
      }
      // dQ^T[f][q] += K^T dS^T over the half's two 16-key steps
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const Frag<bf16> sf = frag_from_f32<bf16>(ds + 8 * t);
#pragma unroll
        for (int fb = 0; fb < TDQ / 32; ++fb) dq[fb] = mma32(tr_frag(K, KLD, 32 * kh + 16 * t, 32 * fb, lane), sf, dq[fb]);
      }
    }
  };

  const int kend = min(S, q0 + BQB);        // keys 0 .. kend - 1 (a multiple of 64)
  const int nkt = kend / BKT;
  MLA_B_GLOAD(0);
  MLA_B_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) MLA_B_GLOAD(kt + 1);
    if (kt * BKT <= qw + 31) compute(buf, kt);
    dstate += (uint64_t)(BKT / 4) * kSplitmixGamma;
    if (kt + 1 < nkt) MLA_B_LSTORE(buf ^ 1);
#pragma unroll
    for (int i = 0; i < TDQ / 32; ++i) asm volatile("" : "+a"(dq[i]));   // (as in the key kernel)
    __syncthreads();
  }
#undef MLA_B_GLOAD
#undef MLA_B_LSTORE

  // accumulator element e of lane l: feature 32 fb + 8 (e / 4) + 4 half + e % 4, query qi;
  // four consecutive features per 16-byte store
  if (qi >= S) return;
  const long long row = ((long long)b * S + qi) * H + h;
#pragma unroll
  for (int fb = 0; fb < TDQ / 32; ++fb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int f = 32 * fb + 8 * g4 + 4 * half;
      const f32x4 v = {dq[fb][4 * g4] * p.tau, dq[fb][4 * g4 + 1] * p.tau, dq[fb][4 * g4 + 2] * p.tau,
                       dq[fb][4 * g4 + 3] * p.tau};
      if (f < TDN) *reinterpret_cast<f32x4*>(p.dqc + row * TDN + f) = v;
      else *reinterpret_cast<f32x4*>(p.dqr + row * TDR + f - TDN) = v;
    }
}

// dO (fp32, [rows][H][128]) -> bf16 copy and D = rowsum(dO o) per (row, head): one wave per
// (row, head), two values per lane
__global__ void __launch_bounds__(256) train_do_prep_kernel(const float* dO, const bf16* o, bf16* dO16, float* D,
                                                            int B, int S, int H) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long long)B * S * H) return;
  const float2 g = *reinterpret_cast<const float2*>(dO + w * TDV + 2 * lane);
  const bf16 o0 = o[w * TDV + 2 * lane], o1 = o[w * TDV + 2 * lane + 1];
  dO16[w * TDV + 2 * lane] = (bf16)g.x;
  dO16[w * TDV + 2 * lane + 1] = (bf16)g.y;
  float s = g.x * (float)o0 + g.y * (float)o1;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (lane == 0) {
    const long long row = w / H;           // b S + s
    const int h = (int)(w - row * H);
    const long long b = row / S, t = row - b * S;
    D[(b * H + h) * S + t] = s;
  }
}

}  // namespace

bool train_flash_supported(int dn, int d_rope, int dv, int S) {
  return dn == TDN && d_rope == TDR && dv == TDV && S > 0 && S % 64 == 0;
}

hipError_t launch_train_bwd(const TrainBwdParams& p, hipStream_t s) {
  if (!train_flash_supported(TDN, TDR, TDV, p.S) || p.B <= 0 || p.H <= 0) return hipErrorInvalidValue;
  const int ngroups = p.B * p.H;
  hipLaunchKernelGGL(train_bwd_kv_kernel, dim3(ngroups * cdiv(p.S, AKB)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(train_bwd_q_kernel, dim3(ngroups * cdiv(p.S, BQB)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_train_do_prep(const float* dO, const void* o, void* dO16, float* D, int B, int S, int H,
                                hipStream_t s) {
  const long long waves = (long long)B * S * H;
  const long long blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(train_do_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dO, static_cast<const bf16*>(o),
                     static_cast<bf16*>(dO16), D, B, S, H);
  return hipGetLastError();
}

}  // namespace mla
