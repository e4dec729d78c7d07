// Flash-style causal prefill for gfx950, bf16, over explicitly up-projected keys/values.
//
// Per head: o_i = sum_{j<=i} softmax_j(scale * q_i . k_j) v_j with k_j = [k^C_j ; k_R,j]
// (the DSV2 page's concatenation of the decompressed key with the rotary key shared by
// all heads; DR = 0 for the MLA and MLRA pages' keys, which carry no separate rotary part).
//
// Workgroup: 256 queries of one (sequence, head); 8 waves x 32 queries (one 32-query column
// block per wave, two waves per SIMD), Q^T held in VGPRs as the B operand.  Keys stream in tiles of 64 through
// LDS, NST stages deep, moved with 16-byte direct-to-LDS copies:
//   K tile  [64 keys][DN] (decompressed part) and [64 keys][DR] (rotary part, shared rows),
//   V tile  [DV][64 keys] -- values stored transposed per head by the up-projection, with
//           the keys of every group of 16 in the order 0-3, 8-11, 4-7, 12-15.
// Per tile and wave:
//   S^T[64 keys x 32 queries]  = K . Q^T       (32x32x16 MFMA, K index = feature)
//   O^T[DV x 32 queries]      += V^T . P^T     (32x32x16 MFMA, K index = key)
// In the S^T accumulator lane l holds, for its query column, keys 4h..4h+3 and 8+4h..8+4h+3
// (h = l / 32) of every 16-key group: exactly the order in which the transposed value rows
// are stored, so P^T feeds the second product straight from registers and the V^T operand
// is a plain 16-byte LDS read.  Softmax per query column (lane-local, one exchange between
// the two lane halves) against a fixed reference maximum (see the pass below).  16-byte
// chunks are XOR-swizzled per row so that operand reads of 8 rows hit distinct LDS banks.
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int FQ = 256;          // queries per workgroup
constexpr int FK = 64;           // keys per tile
constexpr int FNST = 3;          // LDS stages
constexpr int kFlashQB = 1;      // 32-query blocks per wave (waves per workgroup = 8 / QB)
constexpr float kFlashGap = 64.0f;    // log2 units: p <= 2^64 stays far from bf16 / fp32 overflow
constexpr float kFlashLimit = 0x1p64f;  // 2^kFlashGap

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#define kOnes2 ((bf16x2){(__bf16)1.0f, (__bf16)1.0f})

__device__ __forceinline__ int opaque_i(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int DN, int DR, int QB>
struct FlashCfg {
  static constexpr int NWV = 8 / QB;                  // waves per workgroup (256 queries)
  static constexpr int DV = DN;
  static constexpr int KSN = DN / 16, KSR = DR / 16, KS = KSN + KSR;
  static constexpr int CN = DN / 8;                   // 16-byte chunks per key row (decompressed)
  static constexpr int KN_BYTES = FK * DN * 2;
  static constexpr int KR_BYTES = FK * DR * 2;
  static constexpr int V_BYTES = DV * FK * 2;
  static constexpr int STAGE = KN_BYTES + KR_BYTES + V_BYTES;
  static constexpr int KN_COPIES = KN_BYTES / 1024;   // 1 KB per copy instruction
  static constexpr int KR_COPIES = KR_BYTES / 1024;
  static constexpr int V_COPIES = V_BYTES / 1024;
  static constexpr int COPIES = KN_COPIES + KR_COPIES + V_COPIES;
  static constexpr int CPW = COPIES / NWV;            // per wave per stage
  static constexpr int KN_RPC = 1024 / (DN * 2);      // key rows per copy
  static constexpr int DB = DV / 32;                  // 32-row blocks of O^T
  static constexpr size_t LDS = (size_t)FNST * STAGE;
  static_assert(KN_COPIES % NWV == 0 && KR_COPIES % NWV == 0 && V_COPIES % NWV == 0, "copies split evenly over the waves");
  static_assert(DN == 64 || DN == 128, "decompressed width");
  static_assert(DR == 0 || DR == 64, "rotary width");
};

// One work item: the 256 queries of query tile L's (sequence, head), in the block order
// below.  TRAIN: the training forward -- dropout on the attention weights (keep bits drawn
// per group of four keys, see dropout_keep4) and the per-row log-sum-exp written for the
// backward.
template <int DN, int DR, int QB, bool TRAIN>
__device__ __forceinline__ void flash_item(const FlashParams& p, const int L, unsigned char* smem) {
  using C = FlashCfg<DN, DR, QB>;
  constexpr int QW = 32 * QB;                          // queries per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Block -> (sequence, head, query tile).  Workgroups are handed to the 8 XCDs in turn
  // (block L to XCD L % 8), so the map keeps each (sequence, head) group on one XCD: XCD x
  // runs groups x, x + 8, ..., each as ntq consecutive blocks, longest query tile first.
  // Every XCD then gets the same work, and a group's keys / values are reused from its
  // XCD's L2.  (Group counts not divisible by 8 use the plain order.)
  const int ntq = p.ntq;
  const int ngroups = p.B * p.H;
  int g, qrev;
  if (ngroups % 8 == 0) {
    const int x = L & 7, slot = L >> 3;
    g = (slot / ntq) * 8 + x;
    qrev = slot % ntq;
  } else {
    g = L / ntq;
    qrev = L % ntq;
  }
  const int qt = ntq - 1 - qrev;
  const int h = g % p.H, b = g / p.H;
  const int S = p.S;                                    // keys per sequence
  const int q0 = qt * FQ;
  const int qw = q0 + QW * wave;                        // this wave's first query (index among the T)
  const int qwa = p.q_off + qw;                         // its position
  const int kend = min(S, p.q_off + q0 + FQ);           // keys 0 .. kend-1 (multiple of 64)
  const int ntiles = kend / FK;
  const long long bh_q = (long long)b * p.H + h;         // query head stream (dropout counter)
  // key / value head of this query head (grouped heads share one)
  const int kvg = p.kv_group > 1 ? p.kv_group : 1;
  const long long bh = (long long)b * (p.H / kvg) + h / kvg;

  // ---- Q^T fragments: query 32 qb + col of the wave, features 16 ks + 8 half .. +7 ----
  Frag<bf16> qf[QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = min(qw + 32 * qb + col, p.T - 1);
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + (((long long)b * p.T + qi) * p.H + h) * (DN + DR) + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[qb][ks] = frag_load<bf16>(qp + 16 * ks);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(qf[qb][ks].v));
  copies_begin();   // lds_dma.h, rule 1

  // ---- copy sources (byte offsets relative to the tile's first key) ----
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bh * S * DN * 2;
  const unsigned char* rbase = DR ? reinterpret_cast<const unsigned char*>(p.kr) + (long long)b * p.kr_bstride * DR * 2
                                  : nullptr;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.vt) + bh * C::DV * (long long)S * 2;
  // Every wave issues the same mix per stage: KNW decompressed-key copies, KRW rotary-key
  // copies, VW value copies (its quarter of each region).  Rotary and value rows have 8
  // chunks and 8 rows per copy, so their swizzle depends on the lane only.
  constexpr int KNW = C::KN_COPIES / C::NWV, KRW = C::KR_COPIES / C::NWV, VW = C::V_COPIES / C::NWV;
  int kn_src[KNW];           // lane byte offset of decompressed-key copy j of this wave
#pragma unroll
  for (int j = 0; j < KNW; ++j) {
    const int row = (wave * KNW + j) * C::KN_RPC + lane / C::CN;
    kn_src[j] = row * DN * 2 + (((lane % C::CN) ^ (row % C::CN)) << 4);
  }
  // 128-byte rows (rotary keys, transposed values): chunk c of row r sits at
  // c ^ ((r >> 1) & 7), so the 16 rows of one 16-lane read phase (two rows per 256-byte
  // bank line) land on distinct bank windows.  Copies cover 8 rows starting at a multiple
  // of 8, so the key of lane row r8 = lane / 8 is (r8 >> 1) + 4 ((copy row0 / 8) & 1).
  const int r8 = lane / 8;
  auto c8 = [&](int row0) { return ((lane % 8) ^ (((row0 + r8) >> 1) & 7)) << 4; };
  const uint32_t lds0 = lds_addr_of(smem);
  auto issue = [&](int tile) {
    const uint32_t sbase = lds0 + (tile % FNST) * C::STAGE;
    const int key0 = tile * FK;
#pragma unroll
    for (int j = 0; j < KNW; ++j)
      dma16(kbase + (long long)key0 * DN * 2 + kn_src[j],
            __builtin_amdgcn_readfirstlane(sbase + (wave * KNW + j) * 1024));
#pragma unroll
    for (int j = 0; j < KRW; ++j) {
      const int row0 = (wave * KRW + j) * 8;
      dma16(rbase + (long long)key0 * DR * 2 + (row0 + r8) * DR * 2 + c8(row0),
            __builtin_amdgcn_readfirstlane(sbase + C::KN_BYTES + (wave * KRW + j) * 1024));
    }
#pragma unroll
    for (int j = 0; j < VW; ++j) {
      const int row0 = (wave * VW + j) * 8;
      dma16(vbase + (long long)key0 * 2 + (long long)(row0 + r8) * S * 2 + c8(row0),
            __builtin_amdgcn_readfirstlane(sbase + C::KN_BYTES + C::KR_BYTES + (wave * VW + j) * 1024));
    }
  };

  // ---- operand LDS addresses: row base | (swizzled chunk << 4); the logical chunk of
  // k-step ks is 2 ks + half, and (2 ks + half) ^ key = 2 ks ^ (half ^ key), so one base per
  // region and an XOR with ks << 5 give every address ----
  const int kn_base = col * DN * 2 | (((col % C::CN) ^ half) << 4);
  const int kr_base = C::KN_BYTES + (col * DR * 2 | ((((col >> 1) & 7) ^ half) << 4));
  const int v_base = C::KN_BYTES + C::KR_BYTES + (col * FK * 2 | ((((col >> 1) & 7) ^ half) << 4));

  f32x16 oacc[C::DB][QB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x16{};
  // Softmax reference per query column: the maximum of its first key tile (key 0 is visible
  // to every query, so the reference never exceeds the exact maximum and the denominator is
  // at least 1).  p = 2^(s - m_ref) is exact in bf16 / fp32 while s - m_ref < kFlashGap.
  // Every p is non-negative and so bounded by its lane's running sum: one test of the sums
  // after the pass tells whether a score rose further.  The workgroup then finds the exact
  // maximum (scores only) and runs the pass again with it as the reference.  No accumulator
  // rescale and no per-tile maximum sit in the loop.
  float m_ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  bool redo = false;

  // One key tile of one wave.  MODE 0: accumulate against the first tile's maximum (first:
  // this is that tile); MODE 1: exact maximum only; MODE 2: accumulate against the exact
  // maximum.  diag: the tile holds keys after some of the wave's queries (causal mask).
  // first / diag are wave-uniform run-time flags: one instruction stream serves all tiles.
  auto tile = [&](const unsigned char* T, int key0, auto mode_c, bool first, bool diag) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool STREAM = MODE != 1;
    // per-lane address bases, kept opaque so the compiler rebuilds (not hoists) addresses
    const int kn_b = opaque_i(kn_base), kr_b = opaque_i(kr_base), v_b = opaque_i(v_base);
    auto kfrag = [&](int kb, int ks) {
      const int off = ks < C::KSN ? (kn_b ^ (ks << 5)) + kb * 32 * DN * 2
                                  : (kr_b ^ ((ks - C::KSN) << 5)) + kb * 32 * DR * 2;
      return frag_load<bf16>(reinterpret_cast<const bf16*>(T + off));
    };
    // scores S^T[32 keys x QW queries] of tile half kb (K index = feature)
    auto scores = [&](int kb, f32x16 (&sc)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const Frag<bf16> fa = kfrag(kb, ks);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb] = mma32(fa, qf[qb][ks], sc[qb]);
      }
    };
    auto mask = [&](int kb, f32x16 (&sc)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qwa + 32 * qb + col;             // query position
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3) > qi) sc[qb][i] = -INFINITY;
      }
    };
    // scaled maximum over both halves of the tile, both lane halves (log2 units)
    auto tile_max = [&](const f32x16 (&a)[QB], const f32x16 (&c)[QB], int qb) {
      float mx = fmaxf(a[qb][0], c[qb][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(a[qb][i], c[qb][i]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      return mx * p.scale_log2;
    };
    f32x16 s0[QB], s1[QB];
    Frag<bf16> pf0[QB][2], pf1[QB][2];
    if constexpr (STREAM) {
      // Accumulating tile, one explicit instruction stream: operand n (K fragments of both
      // halves, then V^T fragments of both halves) is read 4 steps before its products (one
      // per 32-query block); the exponentials of half 0 ride between the products of half
      // 1's scores, those of half 1 between the first half's value products.  sched_barrier
      // keeps every step in place.  The first tile takes the reference maximum from its
      // first half (keys 0..31, key 0 visible to every query: still at most the exact
      // maximum); diagonal tiles mask each half before its exponentials.
      constexpr int KS = C::KS, NV = 2 * C::DB, NOP = 2 * KS + 2 * NV, PF = 4, NE = 16 * QB;
      auto operand = [&](int n) {
        if (n < 2 * KS) return kfrag(n / KS, n % KS);
        const int r = n - 2 * KS, kb = r / NV, t = (r % NV) / C::DB, db = r % C::DB;
        return frag_load<bf16>(reinterpret_cast<const bf16*>(T + (v_b ^ ((2 * kb + t) << 5)) + db * 32 * FK * 2));
      };
      float nm[QB], ps[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) ps[qb] = l_run[qb];
      float pv0[QB][16], pv1[QB][16];
      // probability x = 16 qb + e of a half: exponential, and on every odd e the bf16 pair
      // and its contribution to the denominator.  TRAIN: the pair then loses its dropped
      // weights (the denominator keeps them; 1 / (1 - p) is applied with the normalisation).
      // Element e of half kb is key key0 + 32 kb + 8 (e / 4) + 4 half + e % 4: one draw per
      // group of four e serves four consecutive keys.
      uint64_t draw[QB], dbase[QB];
      if constexpr (TRAIN) {
        // draw state of this tile's first key group of the lane (keys key0 + 4 half ..); the
        // group of element e of half kb is 8 kb + 2 (e / 4) groups further (state steps by
        // additions)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          dbase[qb] = p.keep_thr ? splitmix_state(p.seed, dropout_counter4((int)bh_q, qwa + 32 * qb + col,
                                                                          (key0 >> 2) + half))
                                 : 0ull;
      }
      auto prob = [&](const f32x16 (&sc)[QB], float (&pv)[QB][16], Frag<bf16> (&pf)[QB][2], int x, int kb) {
        const int qb = x >> 4, e = x & 15;
        pv[qb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][e], p.scale_log2, nm[qb]));
        if constexpr (TRAIN) {
          if ((e & 3) == 0 && p.keep_thr)
            draw[qb] = splitmix_mix(dbase[qb] + (uint64_t)(8 * kb + 2 * (e >> 2)) * kSplitmixGamma);
        }
        if (e & 1) {
          pf[qb][e >> 3].v[(e & 7) - 1] = (bf16)pv[qb][e - 1];
          pf[qb][e >> 3].v[e & 7] = (bf16)pv[qb][e];
          ps[qb] = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[qb][e >> 3].v[(e & 7) - 1], pf[qb][e >> 3].v[e & 7]},
                                                   kOnes2, ps[qb], false);
          if constexpr (TRAIN) {
            if (p.keep_thr) {
              const uint32_t f0 = (uint32_t)(draw[qb] >> (16 * ((e - 1) & 3))) & 0xFFFFu;
              const uint32_t f1 = (uint32_t)(draw[qb] >> (16 * (e & 3))) & 0xFFFFu;
              if (f0 < p.keep_thr) pf[qb][e >> 3].v[(e & 7) - 1] = (bf16)0.f;
              if (f1 < p.keep_thr) pf[qb][e >> 3].v[e & 7] = (bf16)0.f;
            }
          }
        }
      };
      Frag<bf16> ring[PF + 1];
#pragma unroll
      for (int n = 0; n < PF; ++n) ring[n] = operand(n);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s0[qb] = f32x16{};
        s1[qb] = f32x16{};
      }
      // step n: its products, the read of operand n + PF, and its share of exponentials
      auto step = [&](auto n_c) {
        constexpr int n = decltype(n_c)::value;
        const Frag<bf16>& op = ring[n % (PF + 1)];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if constexpr (n < KS) {
            s0[qb] = mma32(op, qf[qb][n], s0[qb]);
          } else if constexpr (n < 2 * KS) {
            s1[qb] = mma32(op, qf[qb][n - KS], s1[qb]);
          } else {
            constexpr int r = n - 2 * KS, kb = r / NV, t = (r % NV) / C::DB, db = r % C::DB;
            oacc[db][qb] = mma32(op, kb ? pf1[qb][t] : pf0[qb][t], oacc[db][qb]);
          }
        }
        if constexpr (n + PF < NOP) ring[(n + PF) % (PF + 1)] = operand(n + PF);
        if constexpr (n >= KS && n < 2 * KS) {
          constexpr int k = n - KS;
#pragma unroll
          for (int x = (NE * k) / KS; x < (NE * (k + 1)) / KS; ++x) prob(s0, pv0, pf0, x, 0);
        } else if constexpr (n >= 2 * KS && n < 2 * KS + NV) {
          constexpr int k = n - 2 * KS;
#pragma unroll
          for (int x = (NE * k) / NV; x < (NE * (k + 1)) / NV; ++x) prob(s1, pv1, pf1, x, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      auto steps = [&](auto lo_c, auto hi_c) {
        constexpr int lo = decltype(lo_c)::value, hi = decltype(hi_c)::value;
        unroll_from<lo>(step, std::make_integer_sequence<int, hi - lo>{});
      };
      using I0 = std::integral_constant<int, 0>;
      using IK = std::integral_constant<int, KS>;
      using I2K = std::integral_constant<int, 2 * KS>;
      using IN = std::integral_constant<int, NOP>;
      __builtin_amdgcn_sched_barrier(0);
      steps(I0{}, IK{});                       // half 0 scores
      if (diag) {
        asm volatile("; diagonal tile");        // keeps these branches
        mask(0, s0);
      }
      if (MODE == 0 && first) {
        asm volatile("; first tile");
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx = s0[qb][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[qb][i]);
          m_ref[qb] = fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2;
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) nm[qb] = -m_ref[qb];
      __builtin_amdgcn_sched_barrier(0);
      steps(IK{}, I2K{});                      // half 1 scores | half 0 exponentials
      if (diag) {
        asm volatile("; diagonal tile");
        mask(1, s1);
      }
      __builtin_amdgcn_sched_barrier(0);
      steps(I2K{}, IN{});                      // value products | half 1 exponentials
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] = ps[qb];
      return;
    }
    // exact-maximum pass: scores only
    scores(0, s0);
    if (diag) mask(0, s0);
    scores(1, s1);
    if (diag) mask(1, s1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = fmaxf(m_ref[qb], tile_max(s0, s1, qb));
  };

  auto pass = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    using M0 = std::integral_constant<int, MODE>;
#pragma unroll
    for (int s = 0; s < FNST - 1; ++s)
      if (s < ntiles) issue(s);
    for (int it = 0; it < ntiles; ++it) {
      if (it + 1 < ntiles) wait_vmcnt<C::CPW>();
      else wait_vmcnt<0>();
      barrier_only();
      if (it + FNST - 1 < ntiles) issue(it + FNST - 1);
      const int key0 = it * FK;
      if (key0 > qwa + QW - 1) continue;                    // every key of the tile is after this wave's queries
      if (MODE != 0 && !redo) continue;
      const unsigned char* T = smem + (it % FNST) * C::STAGE;
      const bool diag = key0 + 63 > qwa;                    // some keys after some of this wave's queries
      tile(T, key0, M0{}, it == 0, diag);
    }
  };

  pass(std::integral_constant<int, 0>{});
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    if (__builtin_amdgcn_readfirstlane(__any(!(l_run[qb] <= kFlashLimit)))) redo = true;
  // workgroup-wide vote: does any wave need the exact-maximum passes?
  __shared__ int redo_flag;
  copies_end();   // lds_dma.h, rule 3 (also before the output stores below)
  if (threadIdx.x == 0) redo_flag = 0;
  __syncthreads();
  if (redo) redo_flag = 1;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(redo_flag)) {
    if (redo) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x16{};
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = -INFINITY;
        l_run[qb] = 0.f;
      }
    }
    pass(std::integral_constant<int, 1>{});
    wait_vmcnt<0>();
    __syncthreads();
    pass(std::integral_constant<int, 2>{});
    copies_end();
    __syncthreads();   // every wave is done with the stages before the output staging below
  }

  // ---- normalise and store o[b][q][h][:].  The wave's rows (one query each) go through LDS
  // (row stride DV * 2 + 16 bytes) so that every store instruction writes whole 16-byte
  // pieces of four query rows; written from the accumulators, a store instruction touched
  // 32 query rows 16 bytes each.  Every wave is past the vote barriers: the stages are free.
  constexpr int ORS = C::DV * 2 + 16;                  // staging row stride (bytes)
  static_assert(C::NWV * QW * ORS <= C::LDS, "output staging fits the stages");
  unsigned char* orow = smem + wave * QW * ORS;
  const int dvo = p.dv_out > 0 ? p.dv_out : C::DV;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = (TRAIN && p.keep_thr ? p.keep_scale : 1.f) / lt;
    const int qi = qw + 32 * qb + col;
    if (TRAIN && p.lse && half == 0 && qi < p.T) p.lse[bh_q * p.T + qi] = m_ref[qb] + __log2f(lt);
    // accumulator element 4 g + e of lane l in block db: feature 32 db + 8 g + 4 (l/32) + e
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][qb][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + (32 * qb + col) * ORS + (32 * db + 8 * g + 4 * half) * 2) = v;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = C::DV / 8;                       // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;                        // rows per store instruction
#pragma unroll
  for (int r0 = 0; r0 < QW; r0 += RPI) {
    const int r = r0 + lane / CPR, c = lane % CPR;
    const int qi = qw + r;
    if (qi >= p.T || 8 * c >= dvo) continue;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(orow + r * ORS + 16 * c);
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(p.o) + (((long long)b * p.T + qi) * p.H + h) * dvo + 8 * c) = v;
  }
}

// One workgroup per work item.
template <int DN, int DR, int QB, bool TRAIN>
__global__ void __launch_bounds__(64 * (8 / QB), 1) prefill_flash_kernel(FlashParams p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  flash_item<DN, DR, QB, TRAIN>(p, blockIdx.x, smem);
}

// Persistent form: one workgroup per CU walks the items of its XCD (block w runs on XCD
// w % 8, so workgroup w takes the items L with L % 8 = w % 8).  Launching one workgroup per
// item left a CU idle between items for ~14 % of the kernel (per-workgroup stamps: 220 of
// 256 workgroups active on average).  XCD x's items are its slots: groups x, x + 8, ...,
// ntq query tiles each, slot ntq j + r holding query tile ntq - 1 - r of the XCD's group j.
// With ntq even, a round gives each of ntq / 2 workgroups a pair of one group's tiles, the
// long tile ntq - 1 - t and then the short tile t: every pair costs the same, so the CPX
// workgroups of an XCD stay in step and work on CPX / (ntq / 2) groups at a time, whose keys
// and values their L2 holds; the long tiles, most of the work, start together and read the
// keys in the same order.  (A rotation of single tiles over the workgroups, equal over ntq
// rounds but not per round, let the workgroups drift apart over ~10 groups: 9.2 GB fetched
// per launch against 5.9 GB with pairs, and 1.2 % slower; short tile first, 1.3 % slower
// than long first.)  With ntq odd,
// workgroup c takes query tile (c + k) % ntq of group c / ntq of round k.
template <int DN, int DR, int QB, bool TRAIN>
__global__ void __launch_bounds__(64 * (8 / QB), 1) prefill_flash_persist_kernel(FlashParams p, int n_items) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int ntq = p.ntq;
  const int cpx = gridDim.x >> 3;                      // workgroups per XCD
  const int x = blockIdx.x & 7, c = blockIdx.x >> 3;
  const int n_slots = n_items >> 3;
  if (ntq % 2 == 0) {                                  // cpx is a multiple of ntq / 2
    const int hq = ntq >> 1, n_groups = n_slots / ntq;
    const int gpr = cpx / hq, t = c % hq;
    for (int g = c / hq; g < n_groups; g += gpr) {
      flash_item<DN, DR, QB, TRAIN>(p, (g * ntq + t) * 8 + x, smem);            // tile ntq - 1 - t
      __syncthreads();   // every wave is done with the item's LDS before the next one's copies
      flash_item<DN, DR, QB, TRAIN>(p, (g * ntq + ntq - 1 - t) * 8 + x, smem);   // query tile t
      __syncthreads();
    }
    return;
  }
  const int jbase = (c / ntq) * ntq, jq = c % ntq;     // cpx is a multiple of ntq
  for (int k = 0;; ++k) {
    const int slot = cpx * k + jbase + (jq + k) % ntq;
    if (slot >= n_slots) break;
    flash_item<DN, DR, QB, TRAIN>(p, slot * 8 + x, smem);
    __syncthreads();
  }
}

}  // namespace

bool prefill_fast_supported(int dn, int d_rope, int dv, int S) {
  return dv == dn && (dn == 64 || dn == 128) && (d_rope == 0 || d_rope == 64) && S % FK == 0 && S > 0;
}

namespace {
template <int DN, int DR, int QB, bool TRAIN = false>
hipError_t launch_flash(const FlashParams& pin, hipStream_t s) {
  FlashParams p = pin;
  p.ntq = cdiv(p.T, FQ);
  const int n_items = p.ntq * p.H * p.B;
  constexpr size_t lds = FlashCfg<DN, DR, QB>::LDS;
  // persistent form when the items split evenly over the XCDs and a round of whole groups
  // (pairs of tiles for even ntq) fits the XCD's CUs
  const int per = p.ntq % 2 == 0 ? p.ntq / 2 : p.ntq;    // workgroups per group and round
  const int cpx = (device_cu_count() / 8) / per * per;
  if ((p.B * p.H) % 8 == 0 && cpx > 0 && n_items > 8 * cpx) {
    hipLaunchKernelGGL((prefill_flash_persist_kernel<DN, DR, QB, TRAIN>), dim3(8 * cpx), dim3(64 * (8 / QB)), lds, s,
                       p, n_items);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_flash_kernel<DN, DR, QB, TRAIN>), dim3(n_items), dim3(64 * (8 / QB)), lds, s, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_fast(const FlashParams& p, hipStream_t s) {
  const int kvg = p.kv_group > 1 ? p.kv_group : 1;
  if (p.H % kvg) return hipErrorInvalidValue;
  if (p.dv_out < 0 || p.dv_out > p.dn || p.dv_out % 32) return hipErrorInvalidValue;
  if (p.keep_thr || p.lse) {
    // training forward: the decoupled-RoPE shape only
    if (p.dn == 128 && p.d_rope == 64 && p.kv_group <= 1 && p.dv_out == 0)
      return launch_flash<128, 64, kFlashQB, true>(p, s);
    return hipErrorInvalidValue;
  }
  if (p.dn == 128 && p.d_rope == 64) return launch_flash<128, 64, kFlashQB>(p, s);
  if (p.dn == 128 && p.d_rope == 0) return launch_flash<128, 0, kFlashQB>(p, s);
  if (p.dn == 64 && p.d_rope == 0) return launch_flash<64, 0, kFlashQB>(p, s);
  if (p.dn == 64 && p.d_rope == 64) return launch_flash<64, 64, kFlashQB>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
