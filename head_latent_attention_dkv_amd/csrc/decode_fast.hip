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
// Workgroup = 4 waves, one per SIMD, and the tile is streamed once for all heads.  MLA
// (one latent block of 512): wave w owns heads 32w..32w+31 and reads the whole row
// (decode_h128_kernel).  MLRA (4 latent blocks of 128): wave w owns latent block w and
// reads its own quarter of the row (decode_fast_kernel).
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int TT = 32;
constexpr float kRestartGap = 64.0f;       // log2 units: p <= 2^64 keeps bf16 / fp32 far from overflow
constexpr float kRestartLimit = 0x1p64f;   // 2^kRestartGap
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#define kOnes2 ((bf16x2){(__bf16)1.0f, (__bf16)1.0f})

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
// Softmax against a fixed reference per head (the maximum of its first tile), with the
// overflow test on the row sums and the rare exact-maximum re-stream of decode_h128_kernel.
//
// TSPLIT (one latent block of rank 128 per token, e.g. one latent head of MLRA on its own):
// the four waves take different tokens instead of different latent blocks.  A tile is 128
// tokens of 256 B; LDS row t of a stage holds tokens t, 32 + t, 64 + t, 96 + t in its four
// 256-byte quarters, so wave w's quarter-row reads (the same code as above) are its own 32
// tokens.  Each wave keeps its own softmax state and writes its own partial row (sub-split
// w of the split); the combine merges the 4 x splits rows like any others.
template <int VL, int VR, int NW, int NSTAGE, bool TSPLIT = false>
__global__ void __launch_bounds__(NW * 64) decode_fast_kernel(DecodeParams p) {
  using C = FastCfg<VL, VR, NW, NSTAGE>;
  static_assert(VR == 0, "latent blocks without a rotary key (the copies below move latent rows only)");
  static_assert(!TSPLIT || (VL == 128 && NW == 4), "token split: rank-128 rows, four waves");
  constexpr int TOK = TSPLIT ? 4 * TT : TT;            // tokens per tile
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  int* const vote = reinterpret_cast<int*>(smem_raw + C::LDS);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4;        // k-group of the MFMA operands / row group of results
  const int hl = lane & 15;         // head within the wave
  const int split = blockIdx.x;
  const int ht = blockIdx.y;
  const int b = blockIdx.z;

  const int n_tok = decode_tokens(p, b);
  const int tok_begin = split * p.chunk;
  if (tok_begin >= n_tok) return;
  const int tok_end = min(n_tok, tok_begin + p.chunk);
  const int ntiles = (tok_end - tok_begin + TOK - 1) / TOK;

  // wave -> (latent block, heads, latent view)
  int g, hloc;
  if (TSPLIT) {
    g = 0;
    hloc = ht * 16 + hl;
  } else if (p.L == 1) {
    g = 0;
    hloc = ht * (16 * NW) + wave * 16 + hl;
  } else {
    g = wave;
    hloc = hl;
  }
  const bool head_ok = hloc < p.hpb;
  const int head = g * p.hpb + hloc;
  // first latent chunk of the view (TSPLIT: the quarter of each LDS row holding the wave's tokens)
  const int vc0 = TSPLIT ? wave * 16 : (p.L == 1) ? 0 : g * (VL / 8);

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
  // Materialise Q, then open the copy phase (lds_dma.h, rule 1).
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(qf[ks].v));
  copies_begin();

  // DMA: latent row t of the tile is one wave-wide 1 KB load (scalar row base, 32-bit lane
  // offset: physical chunk ln holds logical chunk ln ^ bitrev4(t))
  const unsigned char* ckv_seq = reinterpret_cast<const unsigned char*>(p.ckv) + (long long)b * p.cache_bstride * p.r_kv * 2;
  const uint32_t lds_base = lds_addr_of(smem_raw);
  auto issue_tile = [&](int tile, int stage) {
    const int t0 = tok_begin + tile * TOK;
    const uint32_t sbase = lds_base + stage * C::STAGE_BYTES;
    const int ln = opaque(lane);
    const uint32_t ln16 = (uint32_t)ln << 4;
#pragma unroll
    for (int i = 0; i < C::RPW; ++i) {
      const int t = wave * C::RPW + i;
      if constexpr (TSPLIT) {
        // lane ln fills physical chunk ln of LDS row t: quarter ln / 16 = token 32 (ln / 16) + t
        // of the tile, its chunk (ln ^ key) % 16 (key < 16 leaves the quarter unchanged)
        const int tok = min(t0 + 32 * (ln >> 4) + t, tok_end - 1);
        const uint32_t c = (uint32_t)((ln ^ bitrev4(t & 15)) & 15);
        dma16_s_nt(ckv_seq, (uint32_t)tok * (VL * 2) + (c << 4), __builtin_amdgcn_readfirstlane(sbase + t * 1024));
      } else {
        const int tok = min(t0 + t, tok_end - 1);
        dma16_s_nt(ckv_seq + (long long)tok * p.r_kv * 2, ln16 ^ ((uint32_t)bitrev4(t & 15) << 4),
                __builtin_amdgcn_readfirstlane(sbase + t * 1024));
      }
    }
  };

  // Per-lane LDS byte offsets inside a stage (see the swizzle above).
  int qk_off[4];
  {
    const int f = bitrev4(hl);
#pragma unroll
    for (int q = 0; q < 4; ++q) qk_off[q] = hl * 1024 + (((vc0 + 4 * q + grp) ^ f) << 4);
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

  f32x4 acc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;   // reference maximum of this lane's head (log2 units)
  float l_run = 0.f;         // this lane's share of the head's sum of p
  bool redo = false;

  // max / sum over the four lanes hl + 16 g' holding the same head
  auto head_max = [](float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
  };
  auto head_sum = [](float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
  };

  // One tile.  MODE 0: accumulate against the first tile's maximum; MODE 1: exact maximum
  // only; MODE 2: accumulate against the exact maximum.
  auto tile = [&](const unsigned char* T, int t0, bool first, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
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
    }
    const int tw = TSPLIT ? t0 + 32 * wave : t0;           // this wave's first token
    if (tw + TT > tok_end) {                                // ragged last tile only
      asm volatile("; ragged tile");                        // keeps this a branch
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tw + 16 * rb + 4 * grp + i >= tok_end) s[rb][i] = -INFINITY;
    }
    if (MODE == 1 || first) {
      const float mt = head_max(fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                      fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])))) * p.scale_log2;
      m_ref = MODE == 1 ? fmaxf(m_ref, mt) : mt;
    }
    if constexpr (MODE == 1) return;
    // a token-split wave can hold no token of its split at all (m_ref = -inf): its p are 0
    const float nm = (TSPLIT && m_ref == -INFINITY) ? 0.f : -m_ref;
    float pv[8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[4 * rb + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][i], p.scale_log2, nm));
    const Frag<bf16> pf = frag_from_f32<bf16>(pv);
    // the denominator sums the same bf16 probabilities the products use
#pragma unroll
    for (int j = 0; j < 4; ++j) l_run = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf.v[2 * j], pf.v[2 * j + 1]}, kOnes2, l_run, false);
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
    }
  };

  auto pass = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
      if (st < ntiles) issue_tile(st, st);
    for (int it = 0; it < ntiles; ++it) {
      const int left = ntiles - 1 - it;
      if (NSTAGE >= 4 && left >= 2) wait_vmcnt<2 * C::DMA_PER_WAVE>();
      else if (NSTAGE >= 3 && left >= 1) wait_vmcnt<C::DMA_PER_WAVE>();
      else wait_vmcnt<0>();
      barrier_only();
      if (it + NSTAGE - 1 < ntiles) issue_tile(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
      if (MODE != 0 && !redo) continue;
      tile(smem_raw + (it % NSTAGE) * C::STAGE_BYTES, tok_begin + it * TOK, MODE == 0 && it == 0, mode_c);
    }
  };

  pass(std::integral_constant<int, 0>{});
  // p >= 0, so a p above 2^kRestartGap shows in its lane's sum
  if (__builtin_amdgcn_readfirstlane(__any(!(l_run <= kRestartLimit)))) redo = true;
  copies_end();
  __syncthreads();
  if (threadIdx.x == 0) *vote = 0;
  __syncthreads();
  if (redo && lane == 0) *vote = 1;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(*vote)) {
    if (redo) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) acc[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      m_ref = -INFINITY;
      l_run = 0.f;
    }
    pass(std::integral_constant<int, 1>{});
    wait_vmcnt<0>();
    __syncthreads();
    pass(std::integral_constant<int, 2>{});
    copies_end();   // lds_dma.h, rule 3: before the partial-result stores
  }

  const float l_tot = head_sum(l_run);
  if (!head_ok) return;
  const long long pidx = ((long long)b * p.H + head) * p.nsplit + split * p.sub + (TSPLIT ? wave : 0);
  if (grp == 0) {
    p.part_ml[pidx * 2 + 0] = m_ref;
    p.part_ml[pidx * 2 + 1] = l_tot;
  }
  float* pz = p.part_z + pidx * VL + 4 * grp;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) *reinterpret_cast<f32x4*>(pz + 16 * mb) = acc[mb];
}

// 128-head variant for the latent-512 case (MLA with one latent block): one workgroup per
// (sequence, split) streams each cache tile once for all heads.  4 waves, one per SIMD;
// wave w owns heads 32w..32w+31 for both products, so a head's softmax never leaves its wave:
//   scores  S^T[32 tokens x 32 heads] = C_tile[32 x (512+VR)] . Q^T   (32x32x16 MFMA, K =
//           feature; the k-steps alternate between two accumulators so that a single wave
//           does not wait on one dependent chain);
//   values  Z^T[512 x 32 heads] += C_tile^T[512 x 32 tokens] . P^T   (16 column blocks x 2
//           k-steps of 16 tokens; C^T comes from the LDS transpose load).
// Score lane l holds head l%32 at tokens 8(e/4) + 4(l/32) + e%4; read as a k-step of 16
// tokens, those are tokens {4h..4h+3, 8+4h..8+4h+3} (h = l/32), which the transpose load
// hands the value MFMA in the same order, so P^T is the B operand straight from registers.
// Each tile runs as one explicit instruction stream: score operands read 4 steps ahead of
// their products, the value operands of the first column blocks in flight during the
// exponentials, then the value products with their operands read ahead.
// Registers: Q (32 heads x 576 bf16) 144, z accumulators (512 x 32 fp32) 256 per wave.
template <int VR, int NSTAGE>
__global__ void __launch_bounds__(256, 1) decode_h128_kernel(DecodeParams p) {
  constexpr int VL = 512, NWV = 4;
  using C = FastCfg<VL, VR, NWV, NSTAGE>;
  constexpr int KSL = VL / 16, KSR = VR / 16, KS = KSL + KSR;   // 16-wide k-steps (36 or 32)
  constexpr int RPW = TT / NWV;                       // latent rows per wave per tile (8)
  constexpr int DMA_PER_WAVE = RPW + (VR ? 1 : 0);    // + one 8-row rotary copy
  constexpr int MBS = VL / 32;                        // 32-column blocks of z (16)
  constexpr int SPF = 4, VPF = 4;                     // score / value operands read ahead
  static_assert(NSTAGE == 4, "three tiles in flight");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  int* const vote = reinterpret_cast<int*>(smem_raw + C::LDS);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int i16 = lane & 15, g16 = lane >> 4;

  // Workgroups are dealt to the 8 XCDs round robin (XCD = index % 8).  When the grid is a
  // multiple of 8 whose per-XCD share holds whole sequences, XCD x takes the x-th contiguous
  // range of (sequence, split) work items, so the splits of a sequence share one L2 for
  // their query block.
  int wi = blockIdx.x;
  {
    const int G = gridDim.x, per = G >> 3;
    if ((G & 7) == 0 && per % (p.nsplit * p.head_tiles) == 0) wi = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  const int hg = wi % p.head_tiles;
  const int pair = wi / p.head_tiles;
  const int b = pair / p.nsplit;
  const int split = pair - b * p.nsplit;
  const int n_tok = decode_tokens(p, b);
  const int tok_begin = split * p.chunk;
  if (tok_begin >= n_tok) return;
  const int tok_end = min(n_tok, tok_begin + p.chunk);
  const int ntiles = (tok_end - tok_begin + TT - 1) / TT;

  const int head = hg * 128 + 32 * wave + col;
  const bool head_ok = head < p.hpb;

  // ---- copies: latent row t of a tile is one wave-wide 1 KB load at chunk ln ^ bitrev4(t);
  // the wave's 8 rotary rows are one 1 KB load (lane -> row 8 wave + ln/8, chunk ln%8) ----
  const unsigned char* ckv_seq = reinterpret_cast<const unsigned char*>(p.ckv) + (long long)b * p.cache_bstride * (VL * 2);
  const unsigned char* kr_seq = reinterpret_cast<const unsigned char*>(p.kr) + (long long)b * p.cache_bstride * (VR * 2);
  const uint32_t lds_base = lds_addr_of(smem_raw);
  auto issue_tile = [&](int tile, int stage) {
    const int t0 = tok_begin + tile * TT;
    const uint32_t sbase = lds_base + stage * C::STAGE_BYTES;
    const int ln = opaque(lane);
    const uint32_t ln16 = (uint32_t)ln << 4;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int t = wave * RPW + i;                    // wave-uniform
      const int tok = min(t0 + t, tok_end - 1);
      const uint32_t key16 = (uint32_t)bitrev4(t & 15) << 4;
      dma16_s_nt(ckv_seq + (long long)tok * (VL * 2), ln16 ^ key16, __builtin_amdgcn_readfirstlane(sbase + t * 1024));
    }
    if constexpr (VR > 0) {
      const int t = wave * RPW + (ln >> 3);
      const int tok = min(t0 + t, tok_end - 1);
      const uint32_t c = (uint32_t)(((ln & 7) ^ ((t >> 1) & 7)) << 4);
      dma16_s_nt(kr_seq, (uint32_t)tok * (VR * 2) + c, __builtin_amdgcn_readfirstlane(sbase + C::LAT_BYTES + wave * RPW * 128));
    }
  };

  // ---- the first tiles' copies, then Q^T (B operand: lane holds head col, k = 16 ks +
  // 8 half + [0..7]) behind them, so that the query block and the pipeline's first tiles
  // arrive together; one full drain before anything is used (lds_dma.h, rule 4) ----
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st)
    if (st < ntiles) issue_tile(st, st);
  const int head_ld = head_ok ? head : 0;
  const bf16* qlp = reinterpret_cast<const bf16*>(p.q_lat) + ((long long)b * p.H + head_ld) * p.q_lat_hs + 8 * half;
  const bf16* qrp = reinterpret_cast<const bf16*>(p.q_rope) + ((long long)b * p.H + head_ld) * p.q_rope_hs + 8 * half;
  Frag<bf16> qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = frag_load<bf16>(ks < KSL ? qlp + 16 * ks : qrp + 16 * (ks - KSL));
  drain_all();   // lds_dma.h, rule 4
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (!head_ok) qf[ks] = frag_zero<bf16>();
    asm volatile("" ::"v"(qf[ks].v));
  }

  // ---- per-lane LDS byte offsets inside a stage.  The XOR swizzle only touches the low 4
  // bits of a chunk index, so for a step index n = 8 j + r (scores) or 4 j + r (values) the
  // address is base[r] + 256 j: a few base registers plus instruction offsets ----
  // score operand (row = token col, logical chunk 2 ks + half of its latent row; rotary
  // k-step ks' = ks - KSL at chunk 2 ks' + half of its 128-byte row)
  int s_base[8], r_base[KSR ? KSR : 1];
  {
    const int f = bitrev4(col & 15), fr = (col >> 1) & 7;
#pragma unroll
    for (int r = 0; r < 8; ++r) s_base[r] = col * 1024 + (((2 * r + half) ^ f) << 4);
#pragma unroll
    for (int r = 0; r < (KSR ? KSR : 1); ++r) r_base[r] = C::LAT_BYTES + col * 128 + (((2 * r + half) ^ fr) << 4);
  }
  // value operand (transpose load): lane i16 of group g16 reads token row
  // 16 kt + 8 hi + 4 half + i16/4, 8 bytes at latent column 32 mb + 16 (g16 % 2) + 4 (i16 % 4),
  // i.e. logical chunk 4 mb + x: for mb = 4 j + r, v_base[hi][r] + 256 j + 16 KB kt
  int v_base[2][4];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int rr = 8 * hi + 4 * half + (i16 >> 2);
    const int x = 2 * (g16 & 1) + ((i16 & 3) >> 1), f = bitrev4(rr);
#pragma unroll
    for (int r = 0; r < 4; ++r) v_base[hi][r] = rr * 1024 + 8 * (i16 & 1) + (((4 * r + x) ^ f) << 4);
  }

  f32x16 acc[MBS];
#pragma unroll
  for (int mb = 0; mb < MBS; ++mb) acc[mb] = f32x16{};
  float m_ref = -INFINITY;   // reference maximum of this lane's head (log2 units)
  float l_run = 0.f;         // this lane's share of the head's sum of p
  bool redo = false;

  // One tile.  MODE 0: accumulate against the first tile's maximum; MODE 1: exact maximum
  // only; MODE 2: accumulate against the exact maximum.
  auto tile = [&](int stage_off, int t0, bool first, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    // this stage's bases (one add each); every read is base + an instruction offset
    int sb[8], rbs[KSR ? KSR : 1], vb[2][4];
#pragma unroll
    for (int r = 0; r < 8; ++r) sb[r] = s_base[r] + stage_off;
#pragma unroll
    for (int r = 0; r < (KSR ? KSR : 1); ++r) rbs[r] = r_base[r] + stage_off;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int r = 0; r < 4; ++r) vb[hi][r] = v_base[hi][r] + stage_off;
    auto sread = [&](int n) {
      const unsigned char* src = n < KSL ? smem_raw + sb[n % 8] + 256 * (n / 8) : smem_raw + rbs[n - KSL];
      return *reinterpret_cast<const bf16x8*>(src);
    };
    auto vread = [&](int n) {              // value operand n = 16 kt + mb
      const int kt = n / MBS, mb = n % MBS;
      const unsigned char* a0 = smem_raw + vb[0][mb % 4] + 256 * (mb / 4) + 16384 * kt;
      const unsigned char* a1 = smem_raw + vb[1][mb % 4] + 256 * (mb / 4) + 16384 * kt;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a1);
      const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, v);
    };
    // scores: two accumulator chains over alternating k-steps
    f32x16 sa = f32x16{}, sc = f32x16{};
    bf16x8 sring[SPF + 1];
#pragma unroll
    for (int n = 0; n < SPF; ++n) sring[n] = sread(n);
    __builtin_amdgcn_sched_barrier(0);
    // (an empty asm reading one element of every fourth product of a chain keeps the pure
    // MFMAs in their steps: without it the products sink to their first use and every
    // operand read stays live at once.  It names the element as an accumulation register,
    // where the product leaves it: a VGPR operand cost a copy and a hazard wait each time.)
    auto sstep = [&](auto n_c) {
      constexpr int n = decltype(n_c)::value;
      if constexpr (n % 2 == 0) {
        mma32_acc(sa, sring[n % (SPF + 1)], qf[n].v);
        if constexpr (n % 8 == 6) asm volatile("" ::"a"(sa[0]));
      } else {
        mma32_acc(sc, sring[n % (SPF + 1)], qf[n].v);
        if constexpr (n % 8 == 7) asm volatile("" ::"a"(sc[0]));
      }
      if constexpr (n + SPF < KS) sring[(n + SPF) % (SPF + 1)] = sread(n + SPF);
      __builtin_amdgcn_sched_barrier(0);
    };
    unroll_from<0>(sstep, std::make_integer_sequence<int, KS>{});
    // value operands of the first steps go out before the exponentials
    bf16x8 vring[VPF + 1];
    if constexpr (MODE != 1) {
#pragma unroll
      for (int n = 0; n < VPF; ++n) vring[n] = vread(n);
    }
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = sa[e] + sc[e];
    if (t0 + TT > tok_end) {                          // the ragged last tile only
      asm volatile("; ragged tile");                  // keeps this a branch
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (t0 + 8 * (e >> 2) + 4 * half + (e & 3) >= tok_end) s[e] = -INFINITY;
    }
    if (MODE == 1 || first) {
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
      auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1])) * p.scale_log2;
      m_ref = MODE == 1 ? fmaxf(m_ref, mx) : mx;
    }
    if constexpr (MODE == 1) return;
    bf16x8 pf[2];
    {
      const float nm = -m_ref;
      float ps = l_run;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kt + j], p.scale_log2, nm));
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[kt][j] = (bf16)pv[j];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ps = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pf[kt][2 * j], pf[kt][2 * j + 1]}, kOnes2, ps, false);
      }
      l_run = ps;
    }
    __builtin_amdgcn_sched_barrier(0);
    auto vstep = [&](auto n_c) {
      constexpr int n = decltype(n_c)::value;
      constexpr int kt = n / MBS, mb = n % MBS;
      mma32_acc(acc[mb], vring[n % (VPF + 1)], pf[kt]);
      if constexpr (n + VPF < 2 * MBS) vring[(n + VPF) % (VPF + 1)] = vread(n + VPF);
      __builtin_amdgcn_sched_barrier(0);
    };
    unroll_from<0>(vstep, std::make_integer_sequence<int, 2 * MBS>{});
  };

  auto pass = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    if constexpr (MODE != 0) {   // (the main pass's first tiles went out with the query loads)
#pragma unroll
      for (int st = 0; st < NSTAGE - 1; ++st)
        if (st < ntiles) issue_tile(st, st);
    }
    for (int it = 0; it < ntiles; ++it) {
      // wait until only the newest tile is outstanding: two tiles in flight per CU while a
      // tile computes (a third in flight measured slower: more concurrent DRAM streams)
      if (ntiles - 1 - it >= 1) wait_vmcnt<DMA_PER_WAVE>();
      else wait_vmcnt<0>();
      barrier_only();
      if (it + NSTAGE - 1 < ntiles) issue_tile(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
      if (MODE != 0 && !redo) continue;
      tile((it % NSTAGE) * C::STAGE_BYTES, tok_begin + it * TT, MODE == 0 && it == 0, mode_c);
    }
  };

  pass(std::integral_constant<int, 0>{});
  // p >= 0, so a p above 2^kRestartGap shows in its lane's sum
  if (__builtin_amdgcn_readfirstlane(__any(!(l_run <= kRestartLimit)))) redo = true;
  copies_end();
  __syncthreads();
  if (threadIdx.x == 0) *vote = 0;
  __syncthreads();
  if (redo && lane == 0) *vote = 1;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(*vote)) {
    if (redo) {
#pragma unroll
      for (int mb = 0; mb < MBS; ++mb) acc[mb] = f32x16{};
      m_ref = -INFINITY;
      l_run = 0.f;
    }
    pass(std::integral_constant<int, 1>{});
    wait_vmcnt<0>();
    __syncthreads();
    pass(std::integral_constant<int, 2>{});
    copies_end();   // lds_dma.h, rule 3: before the partial-result stores
  }

  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(c[0]) + __uint_as_float(c[1]);
  const long long pidx = ((long long)b * p.H + head) * p.nsplit + split;
  if (head_ok && half == 0) {
    p.part_ml[pidx * 2 + 0] = m_ref;
    p.part_ml[pidx * 2 + 1] = l_tot;
  }
  // The split's result is stored normalised (z / l, bf16, like the output z itself); the
  // combine weights it by l 2^(m - M) in fp32.  l >= 1: the reference maximum is a score of
  // this split, whose p is 1.
  // Accumulator element e of lane l in block mb is latent column 32 mb + 8 (e/4) + 4 (l/32)
  // + e%4 of head col: each wave first writes its 32 rows to LDS (row stride 1040 B), then
  // stores one whole 1 KB row per instruction (written straight from the accumulators, a
  // store instruction touched 32 rows 16 bytes each).
  __syncthreads();   // every wave is done with the stages
  unsigned char* rows = smem_raw + wave * 32 * 1040;
  const float inv_l = 1.f / l_tot;
#pragma unroll
  for (int mb = 0; mb < MBS; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<bf16x4*>(rows + col * 1040 + (32 * mb + 8 * q + 4 * half) * 2) =
          (bf16x4){(bf16)(acc[mb][4 * q + 0] * inv_l), (bf16)(acc[mb][4 * q + 1] * inv_l),
                   (bf16)(acc[mb][4 * q + 2] * inv_l), (bf16)(acc[mb][4 * q + 3] * inv_l)};
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const int head0 = hg * 128 + 32 * wave;   // the wave's first head
  bf16* pz0 = reinterpret_cast<bf16*>(p.part_z) + (((long long)b * p.H + head0) * p.nsplit + split) * VL + 8 * lane;
  const long long hstride = (long long)p.nsplit * VL;
#pragma unroll
  for (int h = 0; h < 32; ++h) {
    if (head0 + h >= p.hpb) break;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(rows + h * 1040 + 16 * lane);
    *reinterpret_cast<bf16x8*>(pz0 + h * hstride) = v;
  }
}

}  // namespace

// Shapes served by the fast path: bf16; MLA with latent 512 (+ rotary 64 or none) and a
// multiple of 128 heads... or fewer; MLRA with 4 blocks of 128 and <= 32 heads per block.
bool decode_fast_supported(const DecodeParams& p, int* variant) {
  // (the rotary rows are addressed inside their sequence with a 32-bit byte offset)
  const bool rope_ok = p.d_rope == 0 || (p.d_rope == 64 && p.cache_bstride < (1LL << 25));
  if (p.L == 1 && p.r_kv == 512 && p.rb == 512 && rope_ok) {
    *variant = p.d_rope ? 3 : 4;
    return true;
  }
  if (p.L == 4 && p.r_kv == 512 && p.rb == 128 && p.d_rope == 0 && p.hpb <= 16) {
    *variant = 2;
    return true;
  }
  // (the token-split copies address a row inside its sequence with a 32-bit byte offset)
  if (p.L == 1 && p.r_kv == 128 && p.rb == 128 && p.d_rope == 0 && p.cache_bstride < (1LL << 23)) {
    *variant = 5;
    return true;
  }
  return false;
}

int decode_fast_head_tile(int variant) { return (variant == 2 || variant == 5) ? 16 : 128; }

bool decode_fast_bf16_partials(int variant) { return variant == 3 || variant == 4; }

hipError_t launch_decode_fast(const DecodeParams& p, int variant, hipStream_t s) {
  dim3 grid(p.nsplit, p.head_tiles, p.B);
  switch (variant) {
    case 3:
    case 4: {
      // 1-D grid over (sequence, split, 128-head group)
      const dim3 g1((unsigned)(p.B * p.nsplit * p.head_tiles));
      if (variant == 3) {
        constexpr size_t lds = FastCfg<512, 64, 4, 4>::LDS + 16;
        hipLaunchKernelGGL((decode_h128_kernel<64, 4>), g1, dim3(256), lds, s, p);
      } else {
        constexpr size_t lds = FastCfg<512, 0, 4, 4>::LDS + 16;
        hipLaunchKernelGGL((decode_h128_kernel<0, 4>), g1, dim3(256), lds, s, p);
      }
      break;
    }
    case 2: {
      // two stages (64 KB): two workgroups share a CU, so one's start and tail overlap the
      // other's stream
      using C = FastCfg<128, 0, 4, 2>;
      hipLaunchKernelGGL((decode_fast_kernel<128, 0, 4, 2>), grid, dim3(256), C::LDS + 16, s, p);
      break;
    }
    case 5: {
      using C = FastCfg<128, 0, 4, 2>;
      if (p.sub != 4) return hipErrorInvalidValue;
      dim3 g5(p.nsplit / p.sub, p.head_tiles, p.B);
      hipLaunchKernelGGL((decode_fast_kernel<128, 0, 4, 2, true>), g5, dim3(256), C::LDS + 16, s, p);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
