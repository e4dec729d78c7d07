// Split-context absorbed decode, bf16 fast path for full-width latent rows.
//
// Same mathematics as decode.hip (scores q_lat . c_j + q_R . k_R,j over the cached rows
// 0..ctx_len[b], online softmax, z = sum_j p_j c_j), organised for gfx950:
//   * the cache tile (32 tokens x the whole row: latent + rotary key) moves global -> LDS
//     with 16-byte direct-to-LDS loads (no registers), NSTAGE tiles deep, so each CU keeps
//     ~100 KB of the latent stream in flight while it computes;
//   * the row-major tile serves both products: C . Q^T reads it with 16-byte LDS loads, and
//     C^T . P^T reads it with the gfx950 LDS transpose load (ds_read_b64_tr_b16), which
//     hands each lane four consecutive tokens of one latent column -- the A operand of a
//     32x32x16 MFMA whose k index is the token;
//   * 16-byte chunks are XOR-swizzled inside groups of 8 per token row so that both read
//     patterns hit distinct LDS banks.
// Workgroup = 4 waves.  MLA (one latent block): wave w owns heads 32w..32w+31 of a
// 128-head tile and reads the whole row.  MLRA (4 latent blocks): wave w owns latent
// block w (its heads padded to 32) and reads its own quarter of the row; the tile is
// still streamed once for all blocks.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int TT = 32;
constexpr float kLazyRescale = 8.0f;
constexpr float kRestartGap = 64.0f;       // log2 units: p <= 2^64 keeps bf16 / fp32 far from overflow
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Stage layout (per 32-token tile):
//   latent region: 32 rows x 1024 B (64 chunks of 16 B).  Logical chunk c of token row t
//     sits at physical chunk c ^ bitrev4(t & 15) (XOR inside aligned groups of 16), so
//     the 16 rows of a score-operand read and the 4 rows x 32 B of a transpose read fall
//     on distinct LDS banks.
//   rotary region: 32 rows x 128 B (8 chunks), chunk c of row t at c ^ ((t >> 1) & 7).
template <int VL, int VR, int NW, int NSTAGE>
struct FastCfg {
  static constexpr int LAT_BYTES = TT * 1024;
  static constexpr int ROPE_BYTES = VR ? TT * 128 : 0;
  static constexpr int STAGE_BYTES = LAT_BYTES + ROPE_BYTES;
  static constexpr int RPW = TT / NW;                // latent rows per wave per tile
  static constexpr int DMA_PER_WAVE = RPW + (VR ? 1 : 0);
  static constexpr int KSL = VL / 32, KSR = VR / 32, KS = KSL + KSR;   // 32-wide k-steps
  static constexpr int MB = VL / 16;                 // 16-column blocks of z
  static constexpr size_t LDS = (size_t)NSTAGE * STAGE_BYTES;
  static_assert(VR == 0 || VR == 64, "rotary width");
  static_assert(NW == 4 || NW == 8, "waves");
};

// 32x32x16 bf16 MFMA accumulate (the compiler tracks its hazards and register classes).
__device__ __forceinline__ void mma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// Opaque copy: keeps lane-dependent address arithmetic inside the loop instead of
// letting the compiler hoist dozens of precomputed addresses into registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// One workgroup = NW waves x 16 heads (16x16x32 MFMA): per tile of 32 tokens
//   S^T[32 tokens x 16 heads] = C_tile[32 x (VL+VR)] . Q^T   (2 row blocks, K = VL+VR)
//   Z^T[VL x 16 heads]       += C_tile^T[VL x 32] . P^T    (VL/16 row blocks, K = 32 tokens)
// Lane l owns head l%16; its 8 scores of a tile sit at tokens 4(l/16)+i and 16+4(l/16)+i,
// which is exactly its slice of P^T as the B operand, so P never leaves registers.
template <int VL, int VR, int NW, int NSTAGE>
__global__ void __launch_bounds__(NW * 64) decode_fast_kernel(DecodeParams p) {
  using C = FastCfg<VL, VR, NW, NSTAGE>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;        // k-group of the MFMA operands / row group of results
  const int hl = lane & 15;         // head within the wave
  const int split = blockIdx.x;
  const int ht = blockIdx.y;
  const int b = blockIdx.z;

  const int n_tok = p.ctx_len[b] + 1;
  const int tok_begin = split * p.chunk;
  if (tok_begin >= n_tok) return;
  const int tok_end = min(n_tok, tok_begin + p.chunk);
  const int ntiles = (tok_end - tok_begin + TT - 1) / TT;

  // wave -> (latent block, heads, latent view)
  int g, hloc;
  if (p.L == 1) {
    g = 0;
    hloc = ht * (16 * NW) + wave * 16 + hl;
  } else {
    g = wave;
    hloc = hl;
  }
  const bool head_ok = hloc < p.hpb;
  const int head = g * p.hpb + hloc;
  const int vc0 = (p.L == 1) ? 0 : g * (VL / 8);       // first latent chunk of the view

  // ---- Q^T slice (B operand), loaded branch-free (padded heads read a valid row, then zero) ----
  const bf16* ql = reinterpret_cast<const bf16*>(p.q_lat);
  const bf16* qr = reinterpret_cast<const bf16*>(p.q_rope);
  const int head_ld = head_ok ? head : g * p.hpb;
  const bf16* qlp = ql + ((long long)b * p.H + head_ld) * p.q_lat_hs + 8 * grp;
  const bf16* qrp = qr + ((long long)b * p.H + head_ld) * p.q_rope_hs + 8 * grp;
  Frag<bf16> qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = frag_load<bf16>(ks < C::KSL ? qlp + ks * 32 : qrp + (ks - C::KSL) * 32);
    if (!head_ok) qf[ks] = frag_zero<bf16>();
  }
  // Materialise Q before the first copies are issued, so that no wait for these loads
  // lands behind (and drains) the copy pipeline.
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(qf[ks].v));

  const bf16* ckv = reinterpret_cast<const bf16*>(p.ckv);
  const bf16* kr = reinterpret_cast<const bf16*>(p.kr);
  const long long row0 = (long long)b * p.cache_bstride;
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)smem_raw);

  // DMA: latent row t of the tile is one wave-wide 1 KB load (lane = physical chunk);
  // each wave also loads TT/NW rotary rows (lanes 0..8*(TT/NW)-1: 8 chunks per row).
  auto issue_tile = [&](int tile, int stage) {
    const int t0 = tok_begin + tile * TT;
    const uint32_t sbase = lds_base + stage * C::STAGE_BYTES;
    const int ln = opaque(lane);
#pragma unroll
    for (int i = 0; i < C::RPW; ++i) {
      const int t = wave * C::RPW + i;
      const int tok = min(t0 + t, tok_end - 1);
      const int c = ln ^ bitrev4(t & 15);
      const bf16* src = ckv + (row0 + tok) * p.r_kv + c * 8;
      dma16(src, __builtin_amdgcn_readfirstlane(sbase + t * 1024));
    }
    if constexpr (VR > 0) {
      constexpr int RROWS = TT / NW;                  // rotary rows per wave (4 or 8)
      if (ln < RROWS * 8) {
        const int t = wave * RROWS + (ln >> 3);
        const int tok = min(t0 + t, tok_end - 1);
        const int c = (ln & 7) ^ ((t >> 1) & 7);
        const bf16* src = kr + (row0 + tok) * p.d_rope + c * 8;
        dma16(src, __builtin_amdgcn_readfirstlane(sbase + C::LAT_BYTES + wave * RROWS * 128));
      }
    }
  };

  f32x4 acc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS byte offsets inside a stage (see the swizzle above).
  int qk_off[4];
  {
    const int f = bitrev4(hl);
#pragma unroll
    for (int q = 0; q < 4; ++q) qk_off[q] = hl * 1024 + (((vc0 + 4 * q + grp) ^ f) << 4);
  }
  int rope_off[2][VR ? C::KSR : 1];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int t = 16 * rb + hl;
#pragma unroll
    for (int ks = 0; ks < (VR ? C::KSR : 1); ++ks) rope_off[rb][ks] = t * 128 + (((4 * ks + grp) ^ ((t >> 1) & 7)) << 4);
  }
  int pv_off[8];
  {
    const int k16 = lane & 15;
    const int r0 = 4 * grp + (k16 >> 2);                     // rows r0 and r0 + 16 share the swizzle
    const int f0 = bitrev4(r0);
    const int x = (k16 & 3) >> 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) pv_off[q] = r0 * 1024 + 8 * (k16 & 1) + (((vc0 + 2 * q + x) ^ f0) << 4);
  }

#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < ntiles) issue_tile(s, s);

  for (int it = 0; it < ntiles; ++it) {
    const int left = ntiles - 1 - it;
    if (NSTAGE >= 4 && left >= 2) wait_vmcnt<2 * C::DMA_PER_WAVE>();
    else if (NSTAGE >= 3 && left >= 1) wait_vmcnt<C::DMA_PER_WAVE>();
    else wait_vmcnt<0>();
    barrier_only();
    if (it + NSTAGE - 1 < ntiles) issue_tile(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);

    const unsigned char* T = smem_raw + (it % NSTAGE) * C::STAGE_BYTES;
    const int t0 = tok_begin + it * TT;

    // S^T: row block rb covers tokens 16 rb .. 16 rb + 15; lane reads token 16 rb + hl at
    // logical chunk vc0 + 4 ks + grp.  With f = bitrev4(hl) only the low 4 bits of the
    // chunk are permuted, so the byte offset is qk_off[ks % 4] + 256 (ks / 4) + 16 KB rb.
    f32x4 s[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < C::KSL; ++ks) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        Frag<bf16> a = frag_load<bf16>(reinterpret_cast<const bf16*>(
            T + qk_off[ks & 3] + 256 * (ks >> 2) + 16 * 1024 * rb));
        s[rb] = mma16(a, qf[ks], s[rb]);
      }
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (VR > 0) {
#pragma unroll
      for (int ks = 0; ks < C::KSR; ++ks)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          Frag<bf16> a = frag_load<bf16>(reinterpret_cast<const bf16*>(T + C::LAT_BYTES + rope_off[rb][ks]));
          s[rb] = mma16(a, qf[C::KSL + ks], s[rb]);
        }
    }
    float pv[8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[4 * rb + i] = s[rb][i] * p.scale_log2;
    if (t0 + TT > tok_end) {                                // ragged last tile only
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * rb + 4 * grp + i >= tok_end) pv[4 * rb + i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(fmaxf(pv[0], pv[1]), fmaxf(pv[2], pv[3])),
                     fmaxf(fmaxf(pv[4], pv[5]), fmaxf(pv[6], pv[7])));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // The running maximum is raised only when a tile exceeds it by more than 2^8
    // (always on the first tile); the branch is wave-uniform and rarely taken.
    if (__builtin_amdgcn_readfirstlane(__any(mt > m_run + kLazyRescale))) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) acc[mb] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = exp2f(pv[i] - m_run);
      ps += pv[i];
    }
    l_run += ps;
    const Frag<bf16> pf = frag_from_f32<bf16>(pv);
    __builtin_amdgcn_sched_barrier(0);

    // Z^T += C^T . P^T with the A operand from the LDS transpose load: lane k of 16-lane
    // group grp addresses row 4 grp + k/4 (and + 16), columns 16 mb + 4 (k % 4), and
    // receives column 16 mb + k at four consecutive rows.  Offsets: pv_off[mb % 8] +
    // 256 (mb / 8) (+ 16 KB for the second read).
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const unsigned char* a0 = T + pv_off[mb & 7] + 256 * (mb >> 3);
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a0);
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0 + 16 * 1024));
      s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      Frag<bf16> a;
      a.v = __builtin_bit_cast(bf16x8, v);
      acc[mb] = mma16(a, pf, acc[mb]);
      if ((mb & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!head_ok) return;
  const long long pidx = ((long long)b * p.H + head) * p.nsplit + split;
  if (grp == 0) {
    p.part_ml[pidx * 2 + 0] = m_run;
    p.part_ml[pidx * 2 + 1] = l_tot;
  }
  float* pz = p.part_z + pidx * VL + 4 * grp;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) *reinterpret_cast<f32x4*>(pz + 16 * mb) = acc[mb];
}

// Wide variant: NW = 4 waves x 32 heads (32x32x16 MFMA) for the 128-head latent-512 case.
// Half the LDS traffic of the 16-head variant (each 32-head group reads the tile once for
// the scores and once for the values); z accumulators (32 heads x 512 fp32) take the
// 256 accumulation registers, Q (32 heads x 576 bf16) 144 vector registers.
//   S^T[32 tokens x 32 heads] = C_tile . Q^T      (K = 512 + 64, 36 k-steps of 16)
//   Z^T[512 x 32 heads]      += C_tile^T . P^T   (16 row blocks of 32 columns, K = 32 tokens)
// Lane l owns head l%32; S^T rows (tokens) 8(i/4) + 4(l/32) + i%4, which, grouped by
// 16 tokens, is the lane's P^T slice in the k order {4h..4h+3, 8+4h..8+4h+3}.
template <int VR, int NSTAGE>
__global__ void __launch_bounds__(256, 1) decode_wide_kernel(DecodeParams p) {
  constexpr int VL = 512, NW = 4;
  using C = FastCfg<VL, VR, 8, NSTAGE>;              // stage layout: latent rows + rotary rows
  constexpr int KSL = VL / 16, KSR = VR / 16, KS = KSL + KSR;
  constexpr int MB = VL / 32;
  constexpr int RPW = TT / NW;                        // latent rows per wave per tile
  constexpr int DMA_PER_WAVE = RPW + (VR ? 1 : 0);
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  __shared__ int restart_flag;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int split = blockIdx.x;
  const int ht = blockIdx.y;
  const int b = blockIdx.z;

  const int n_tok = p.ctx_len[b] + 1;
  const int tok_begin = split * p.chunk;
  if (tok_begin >= n_tok) return;
  const int tok_end = min(n_tok, tok_begin + p.chunk);
  const int ntiles = (tok_end - tok_begin + TT - 1) / TT;

  const int hloc = ht * 128 + wave * 32 + col;
  const bool head_ok = hloc < p.hpb;
  const int head = hloc;

  // ---- Q^T (B operand): lane holds head `col`, k = 16 ks + 8 half + [0..7] ----
  const bf16* ql = reinterpret_cast<const bf16*>(p.q_lat);
  const bf16* qr = reinterpret_cast<const bf16*>(p.q_rope);
  const int head_ld = head_ok ? head : 0;
  const bf16* qlp = ql + ((long long)b * p.H + head_ld) * p.q_lat_hs + 8 * half;
  const bf16* qrp = qr + ((long long)b * p.H + head_ld) * p.q_rope_hs + 8 * half;
  Frag<bf16> qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = frag_load<bf16>(ks < KSL ? qlp + ks * 16 : qrp + (ks - KSL) * 16);
    if (!head_ok) qf[ks] = frag_zero<bf16>();
  }
  if (threadIdx.x == 0) restart_flag = 0;
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks].v));

  const bf16* ckv = reinterpret_cast<const bf16*>(p.ckv);
  const bf16* kr = reinterpret_cast<const bf16*>(p.kr);
  const long long row0 = (long long)b * p.cache_bstride;
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)smem_raw);

  auto issue_tile = [&](int tile, int stage) {
    const int t0 = tok_begin + tile * TT;
    const uint32_t sbase = lds_base + stage * C::STAGE_BYTES;
    const int ln = opaque(lane);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int t = wave * RPW + i;
      const int tok = min(t0 + t, tok_end - 1);
      const int c = ln ^ bitrev4(t & 15);
      dma16(ckv + (row0 + tok) * p.r_kv + c * 8, __builtin_amdgcn_readfirstlane(sbase + t * 1024));
    }
    if constexpr (VR > 0) {
      // 8 rotary rows per wave: lane -> (row wave*8 + lane/8, physical chunk lane%8)
      const int t = wave * 8 + (ln >> 3);
      const int tok = min(t0 + t, tok_end - 1);
      const int c = (ln & 7) ^ ((t >> 1) & 7);
      dma16(kr + (row0 + tok) * p.d_rope + c * 8, __builtin_amdgcn_readfirstlane(sbase + C::LAT_BYTES + wave * 1024));
    }
  };

  // per-lane byte offsets inside a stage
  int qk_off[8];
  {
    const int f = bitrev4(col & 15);
#pragma unroll
    for (int q = 0; q < 8; ++q) qk_off[q] = col * 1024 + (((2 * q + half) ^ f) << 4);
  }
  int rope_off[VR ? KSR : 1];
#pragma unroll
  for (int ks = 0; ks < (VR ? KSR : 1); ++ks) rope_off[ks] = col * 128 + (((2 * ks + half) ^ ((col >> 1) & 7)) << 4);
  int pv_off[2][4];                                   // [lo/hi read][mb % 4]
  {
    const int k16 = lane & 15, g16 = lane >> 4;
    const int r0 = 4 * half + (k16 >> 2);             // + 16 ks; hi read + 8
    const int x = 2 * (g16 & 1) + ((k16 & 3) >> 1);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = r0 + 8 * hi;
      const int f = bitrev4(r & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) pv_off[hi][q] = r * 1024 + 8 * (k16 & 1) + (((4 * q + x) ^ f) << 4);
    }
  }

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_ref = -INFINITY;   // reference maximum (log2 units)
  float m_seen = -INFINITY;  // largest tile maximum seen
  float l_run = 0.f;
  bool redo = false;         // this wave stopped accumulating in pass 1

  // Pass 1 uses the first tile's maximum as a fixed reference: p = 2^(s - m_ref) is exact
  // in bf16 / fp32 while s - m_ref < kRestartGap.  A wave whose tile would exceed that
  // (never for ordinary attention scores) stops accumulating but keeps computing scores,
  // so that m_seen ends as its exact maximum; pass 2 then re-streams the split with that
  // reference for the waves that stopped.  No per-register rescale sits in either loop.
  auto pass = [&](auto second_pass) {
    constexpr bool SECOND = decltype(second_pass)::value;
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < ntiles) issue_tile(s, s);
    for (int it = 0; it < ntiles; ++it) {
      const int left = ntiles - 1 - it;
      if (NSTAGE >= 4 && left >= 2) wait_vmcnt<2 * DMA_PER_WAVE>();
      else if (NSTAGE >= 3 && left >= 1) wait_vmcnt<DMA_PER_WAVE>();
      else wait_vmcnt<0>();
      barrier_only();
      if (it + NSTAGE - 1 < ntiles) issue_tile(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
      if (SECOND && !redo) continue;

      const unsigned char* T = smem_raw + (it % NSTAGE) * C::STAGE_BYTES;
      const int t0 = tok_begin + it * TT;

      // scores: one 16-byte LDS read per k-step feeds one MFMA; the schedule below keeps
      // two reads in flight ahead of the MFMA that consumes them.
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const unsigned char* src = (ks < KSL) ? T + qk_off[ks & 7] + 256 * (ks >> 3)
                                              : T + C::LAT_BYTES + rope_off[(ks - KSL) & (KSR ? KSR - 1 : 0)];
        Frag<bf16> a = frag_load<bf16>(reinterpret_cast<const bf16*>(src));
        s = mma32(a, qf[ks], s);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < KS - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = s[i] * p.scale_log2;
      if (t0 + TT > tok_end) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (t0 + 8 * (i >> 2) + 4 * half + (i & 3) >= tok_end) pv[i] = -INFINITY;
      }
      if constexpr (!SECOND) {
        float mt = pv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, pv[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        m_seen = fmaxf(m_seen, mt);
        if (it == 0) m_ref = mt;
        if (__builtin_amdgcn_readfirstlane(__any(mt > m_ref + kRestartGap))) redo = true;
        if (redo) continue;
      }
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = exp2f(pv[i] - m_ref);
        ps += pv[i];
      }
      l_run += ps;
      Frag<bf16> pf[2];
      pf[0] = frag_from_f32<bf16>(pv);
      pf[1] = frag_from_f32<bf16>(pv + 8);
      __builtin_amdgcn_sched_barrier(0);

      // values: two transpose reads per MFMA; the schedule keeps one block (4 reads) ahead.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const unsigned char* a0 = T + pv_off[0][mb & 3] + 256 * (mb >> 2) + 16 * 1024 * ks;
          const unsigned char* a1 = T + pv_off[1][mb & 3] + 256 * (mb >> 2) + 16 * 1024 * ks;
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a0);
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a1);
          s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          mma32_acc(acc[mb], __builtin_bit_cast(bf16x8, v), pf[ks].v);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int i = 0; i < MB - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  pass(std::false_type{});
  // workgroup-wide vote: does any wave need the exact-maximum pass?
  wait_vmcnt<0>();
  barrier_only();
  if (redo) restart_flag = 1;
  barrier_only();
  if (__builtin_amdgcn_readfirstlane(restart_flag)) {
    if (redo) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
      m_ref = m_seen;
      l_run = 0.f;
    }
    pass(std::true_type{});
    wait_vmcnt<0>();
  }

  const float l_tot = wave_sum32(l_run);
  if (!head_ok) return;
  const long long pidx = ((long long)b * p.H + head) * p.nsplit + split;
  if (half == 0) {
    p.part_ml[pidx * 2 + 0] = m_ref;
    p.part_ml[pidx * 2 + 1] = l_tot;
  }
  float* pz = p.part_z + pidx * VL;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(pz + mb * 32 + 8 * q + 4 * half) =
          (f32x4){acc[mb][4 * q + 0], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]};
}

}  // namespace

// Shapes served by the fast path: bf16; MLA with latent 512 (+ rotary 64 or none) and a
// multiple of 128 heads... or fewer; MLRA with 4 blocks of 128 and <= 32 heads per block.
bool decode_fast_supported(const DecodeParams& p, int* variant) {
  const bool rope_ok = p.d_rope == 64 || p.d_rope == 0;
  if (p.L == 1 && p.r_kv == 512 && p.rb == 512 && rope_ok) {
    *variant = p.d_rope ? 3 : 4;
    return true;
  }
  if (p.L == 4 && p.r_kv == 512 && p.rb == 128 && p.d_rope == 0 && p.hpb <= 16) {
    *variant = 2;
    return true;
  }
  return false;
}

int decode_fast_head_tile(int variant) { return variant == 2 ? 16 : 128; }

hipError_t launch_decode_fast(const DecodeParams& p, int variant, hipStream_t s) {
  dim3 grid(p.nsplit, p.head_tiles, p.B);
  switch (variant) {
    case 3: {
      using C = FastCfg<512, 64, 8, 4>;
      hipLaunchKernelGGL((decode_wide_kernel<64, 4>), grid, dim3(256), C::LDS, s, p);
      break;
    }
    case 4: {
      using C = FastCfg<512, 0, 8, 4>;
      hipLaunchKernelGGL((decode_wide_kernel<0, 4>), grid, dim3(256), C::LDS, s, p);
      break;
    }
    case 2: {
      using C = FastCfg<128, 0, 4, 4>;
      hipLaunchKernelGGL((decode_fast_kernel<128, 0, 4, 4>), grid, dim3(256), C::LDS, s, p);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
