// Flash-style causal prefill for gfx950, bf16, over explicitly up-projected keys/values.
//
// Per head: o_i = sum_{j<=i} softmax_j(scale * q_i . k_j) v_j with k_j = [k^C_j ; k_R,j]
// (the DSV2 page's concatenation of the decompressed key with the rotary key shared by
// all heads; DR = 0 for the MLA and MLRA pages' keys, which carry no separate rotary part).
//
// Workgroup: 256 queries of one (sequence, head); 4 waves x 64 queries (two 32-query
// column blocks), Q^T held in VGPRs as the B operand.  Keys stream in tiles of 64 through
// LDS, NST stages deep, moved with 16-byte direct-to-LDS copies:
//   K tile  [64 keys][DN] (decompressed part) and [64 keys][DR] (rotary part, shared rows),
//   V tile  [DV][64 keys] -- values stored transposed per head by the up-projection, with
//           the keys of every group of 16 in the order 0-3, 8-11, 4-7, 12-15.
// Per tile and wave:
//   S^T[64 keys x 64 queries]  = K . Q^T       (32x32x16 MFMA, K index = feature)
//   O^T[DV x 64 queries]      += V^T . P^T     (32x32x16 MFMA, K index = key)
// In the S^T accumulator lane l holds, for its query column, keys 4h..4h+3 and 8+4h..8+4h+3
// (h = l / 32) of every 16-key group: exactly the order in which the transposed value rows
// are stored, so P^T feeds the second product straight from registers and the V^T operand
// is a plain 16-byte LDS read.  Softmax per query column (lane-local, one exchange between
// the two lane halves) against a fixed reference maximum (see the pass below).  16-byte
// chunks are XOR-swizzled per row so that operand reads of 8 rows hit distinct LDS banks.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int FQ = 256;          // queries per workgroup
constexpr int FK = 64;           // keys per tile
constexpr int FNST = 3;          // LDS stages
#ifndef MLA_FLASH_QB
#define MLA_FLASH_QB 1
#endif
constexpr int kFlashQB = MLA_FLASH_QB;   // 32-query blocks per wave (waves per workgroup = 8 / QB)
constexpr float kFlashGap = 64.0f;    // log2 units: p <= 2^64 stays far from bf16 / fp32 overflow

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

template <int DN, int DR, int QB>
__global__ void __launch_bounds__(64 * (8 / QB), 1) prefill_flash_kernel(FlashParams p) {
  using C = FlashCfg<DN, DR, QB>;
  constexpr int QW = 32 * QB;                          // queries per wave
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Block -> (sequence, head, query tile).  Workgroups are handed to the 8 XCDs in turn
  // (block L to XCD L % 8), so the map keeps each (sequence, head) group on one XCD: XCD x
  // runs groups x, x + 8, ..., each as ntq consecutive blocks, longest query tile first.
  // Every XCD then gets the same work, and a group's keys / values are reused from its
  // XCD's L2.  (Group counts not divisible by 8 use the plain order.)
  const int ntq = p.ntq;
  const int L = blockIdx.x;
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
  const int S = p.S;
  const int q0 = qt * FQ;
  const int qw = q0 + QW * wave;                        // this wave's first query
  const int kend = min(S, q0 + FQ);                     // keys 0 .. kend-1 (multiple of 64)
  const int ntiles = kend / FK;
  const long long bh = (long long)b * p.H + h;

  // ---- Q^T fragments: query 32 qb + col of the wave, features 16 ks + 8 half .. +7 ----
  Frag<bf16> qf[QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = min(qw + 32 * qb + col, S - 1);
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + (((long long)b * S + qi) * p.H + h) * (DN + DR) + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[qb][ks] = frag_load<bf16>(qp + 16 * ks);
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(qf[qb][ks].v));

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
  // Softmax reference per query column: the maximum of its first key tile.  p = 2^(s - m_ref)
  // stays exact in bf16 / fp32 while s - m_ref < kFlashGap; a wave whose scores rise
  // further stops accumulating but keeps tracking its exact maximum (m_seen), and the
  // workgroup then re-streams the keys once with that maximum as the reference.  No
  // accumulator rescale sits in the loop.
  float m_ref[QB], m_seen[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    m_seen[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  bool redo = false;

  auto pass = [&](auto second_pass) {
    constexpr bool SECOND = decltype(second_pass)::value;
#pragma unroll
    for (int s = 0; s < FNST - 1; ++s)
      if (s < ntiles) issue(s);
    for (int it = 0; it < ntiles; ++it) {
      if (it + 1 < ntiles) wait_vmcnt<C::CPW>();
      else wait_vmcnt<0>();
      barrier_only();
      if (it + FNST - 1 < ntiles) issue(it + FNST - 1);
      const int key0 = it * FK;
      if (key0 > qw + QW - 1) continue;                     // every key of the tile is after this wave's queries
      if (SECOND && !redo) continue;

      const unsigned char* T = smem + (it % FNST) * C::STAGE;
      // per-lane address bases, kept opaque so the compiler rebuilds (not hoists) addresses
      const int kn_b = opaque_i(kn_base), kr_b = opaque_i(kr_base), v_b = opaque_i(v_base);

      const bool diag = key0 + 63 > qw;                 // some keys after some of this wave's queries
      // Half kb of the tile: scores S^T[32 keys x 64 queries], causal mask, maxima (log2 units)
      auto kfrag = [&](int kb, int ks) {
        const int off = ks < C::KSN ? (kn_b ^ (ks << 5)) + kb * 32 * DN * 2
                                    : (kr_b ^ ((ks - C::KSN) << 5)) + kb * 32 * DR * 2;
        return frag_load<bf16>(reinterpret_cast<const bf16*>(T + off));
      };
      // operand reads run two k-steps ahead of the MFMAs that consume them
      auto scores = [&](int kb, f32x16 (&sc)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb] = f32x16{};
        Frag<bf16> fa[3];
        fa[0] = kfrag(kb, 0);
        fa[1] = kfrag(kb, 1);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          if (ks + 2 < C::KS) fa[(ks + 2) % 3] = kfrag(kb, ks + 2);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sc[qb] = mma32(fa[ks % 3], qf[qb][ks], sc[qb]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int ks = 0; ks < C::KS - 2; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      };
      auto mask_max = [&](int kb, f32x16 (&sc)[QB], float (&mt)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qi = qw + 32 * qb + col;
          if (diag) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3) > qi) sc[qb][i] = -INFINITY;
          }
          float mx = sc[qb][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[qb][i]);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          mt[qb] = mx * p.scale_log2;
        }
      };
      auto track = [&](const float (&mt)[QB], bool first) {
        if constexpr (!SECOND) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            m_seen[qb] = fmaxf(m_seen[qb], mt[qb]);
            if (first) m_ref[qb] = mt[qb];                // key 0 is visible to every query
            if (__builtin_amdgcn_readfirstlane(__any(mt[qb] > m_ref[qb] + kFlashGap))) redo = true;
          }
        }
      };
      // p = 2^(scale s - m_ref) (raw v_exp_f32: the argument stays below kFlashGap unless the
      // wave is re-streaming anyway, and -inf gives 0)
      auto probs = [&](const f32x16 (&sc)[QB], Frag<bf16> (&pf)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float nm = -m_ref[qb];
          float ps = l_run[qb];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][8 * t + j], p.scale_log2, nm));
            pf[qb][t] = frag_from_f32<bf16>(pv);
            // the denominator sums the same bf16 probabilities the products use
#pragma unroll
            for (int j = 0; j < 4; ++j)
              ps = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[qb][t].v[2 * j], pf[qb][t].v[2 * j + 1]}, kOnes2, ps, false);
          }
          l_run[qb] = ps;
        }
      };
      auto pv_products = [&](int kb, const Frag<bf16> (&pf)[QB][2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const int off = (v_b ^ ((2 * kb + t) << 5)) + db * 32 * FK * 2;
            const Frag<bf16> fv = frag_load<bf16>(reinterpret_cast<const bf16*>(T + off));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mma32(fv, pf[qb][t], oacc[db][qb]);
          }
      };

      // Order: S0, mask/max 0, [S1 MFMAs | exponentials of half 0], mask/max 1,
      // [P0 V products | exponentials of half 1], P1 V products.  A wave that must re-stream
      // keeps computing scores and maxima (exact maximum) but adds nothing to O.
      f32x16 s0[QB], s1[QB];
      float mt0[QB], mt1[QB];
      Frag<bf16> pf0[QB][2], pf1[QB][2];
      scores(0, s0);
      mask_max(0, s0, mt0);
      track(mt0, it == 0);
      probs(s0, pf0);
      scores(1, s1);
      mask_max(1, s1, mt1);
      track(mt1, false);
      if (SECOND || !redo) {
        pv_products(0, pf0);
        probs(s1, pf1);
        pv_products(1, pf1);
      }
    }
  };

  pass(std::false_type{});
  // workgroup-wide vote: does any wave need the exact-maximum pass?
  __shared__ int redo_flag;
  wait_vmcnt<0>();
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
        m_ref[qb] = m_seen[qb];
        l_run[qb] = 0.f;
      }
    }
    pass(std::true_type{});
    wait_vmcnt<0>();
  }

  // ---- normalise and store o[b][q][h][:] (4 consecutive features per 8-byte store) ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.f / lt;
    const int qi = qw + 32 * qb + col;
    if (qi >= S) continue;
    bf16* op = reinterpret_cast<bf16*>(p.o) + (((long long)b * S + qi) * p.H + h) * C::DV + 4 * half;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][qb][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g) = v;
      }
  }
}

}  // namespace

bool prefill_fast_supported(int dn, int d_rope, int dv, int S) {
  return dv == dn && (dn == 64 || dn == 128) && (d_rope == 0 || d_rope == 64) && S % FK == 0 && S > 0;
}

namespace {
template <int DN, int DR, int QB>
hipError_t launch_flash(const FlashParams& pin, hipStream_t s) {
  FlashParams p = pin;
  p.ntq = cdiv(p.S, FQ);
  dim3 grid(p.ntq * p.H * p.B);
  constexpr size_t lds = FlashCfg<DN, DR, QB>::LDS;
  hipLaunchKernelGGL((prefill_flash_kernel<DN, DR, QB>), grid, dim3(64 * (8 / QB)), lds, s, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_fast(const FlashParams& p, hipStream_t s) {
  if (p.dn == 128 && p.d_rope == 64) return launch_flash<128, 64, kFlashQB>(p, s);
  if (p.dn == 128 && p.d_rope == 0) return launch_flash<128, 0, kFlashQB>(p, s);
  if (p.dn == 64 && p.d_rope == 0) return launch_flash<64, 0, kFlashQB>(p, s);
  if (p.dn == 64 && p.d_rope == 64) return launch_flash<64, 64, kFlashQB>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
