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
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int TT = 32;
constexpr float kLazyRescale = 8.0f;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// 16-byte global -> LDS copy per lane (lane l writes lds_addr + 16 l).  Issued as inline
// assembly so the compiler does not drain all outstanding copies (vmcnt(0)) before every
// LDS read it cannot disambiguate; completion is tracked explicitly with wait_vmcnt<>.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}

// Stage layout (per 32-token tile):
//   latent region: 32 rows x 1024 B (64 chunks of 16 B).  Logical chunk c of token row t
//     sits at physical chunk c ^ bitrev4(t & 15) (XOR inside aligned groups of 16), so
//     the 16 rows of a score-operand read and the 4 rows x 32 B of a transpose read fall
//     on distinct LDS banks.
//   rotary region: 32 rows x 128 B (8 chunks), chunk c of row t at c ^ ((t >> 1) & 7).
__device__ __forceinline__ int bitrev4(int x) {
  return ((x & 1) << 3) | ((x & 2) << 1) | ((x & 4) >> 1) | ((x & 8) >> 3);
}

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
    const int h16 = opaque(hl);
    const int gg = opaque(grp);

    // S^T: row block rb covers tokens 16 rb .. 16 rb + 15; lane reads token 16 rb + h16,
    // logical chunk 4 ks + gg (eight k values per chunk)
    f32x4 s[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int t = 16 * rb + h16;
      const unsigned char* rowp = T + t * 1024;
      const int f = bitrev4(h16);
#pragma unroll
      for (int ks = 0; ks < C::KSL; ++ks) {
        const int c = vc0 + 4 * ks + gg;
        Frag<bf16> a = frag_load<bf16>(reinterpret_cast<const bf16*>(rowp + ((c ^ f) << 4)));
        s[rb] = mma16(a, qf[ks], s[rb]);
        if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (VR > 0) {
        const unsigned char* rrow = T + C::LAT_BYTES + t * 128;
        const int fr = (t >> 1) & 7;
#pragma unroll
        for (int ks = 0; ks < C::KSR; ++ks) {
          const int c = 4 * ks + gg;
          Frag<bf16> a = frag_load<bf16>(reinterpret_cast<const bf16*>(rrow + ((c ^ fr) << 4)));
          s[rb] = mma16(a, qf[C::KSL + ks], s[rb]);
        }
      }
    }
    float pv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * rb + 4 * grp + i;
        const float x = (tok < tok_end) ? s[rb][i] * p.scale_log2 : -INFINITY;
        pv[4 * rb + i] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // The running maximum is raised only when a tile exceeds it by more than 2^8; the
    // z accumulators are rescaled block by block inside the product loop below.
    const bool raise = __any(mt > m_run + kLazyRescale);
    float alpha = 1.f;
    if (raise) {
      const float m_new = fmaxf(m_run, mt);
      alpha = exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
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
    // group gg addresses row 4 gg + k/4 (and + 16), columns 16 mb + 4 (k % 4), and receives
    // column 16 mb + k at four consecutive rows.
    {
      const int ln = opaque(lane);
      const int k16 = ln & 15, g16 = ln >> 4;
      const int r0 = 4 * g16 + (k16 >> 2);
      const int f0 = bitrev4(r0);                            // rows r0 and r0 + 16 share it
      const int x = (k16 & 3) >> 1;
      const unsigned char* base = T + r0 * 1024 + 8 * (k16 & 1);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int c = vc0 + 2 * mb + x;
        const unsigned char* a0 = base + ((c ^ f0) << 4);
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a0);
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0 + 16 * 1024));
        s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        Frag<bf16> a;
        a.v = __builtin_bit_cast(bf16x8, v);
        if (raise) acc[mb] *= alpha;
        acc[mb] = mma16(a, pf, acc[mb]);
        if ((mb & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
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

}  // namespace

// Shapes served by the fast path: bf16; MLA with latent 512 (+ rotary 64 or none) and a
// multiple of 128 heads... or fewer; MLRA with 4 blocks of 128 and <= 32 heads per block.
bool decode_fast_supported(const DecodeParams& p, int* variant) {
  const bool rope_ok = p.d_rope == 64 || p.d_rope == 0;
  if (p.L == 1 && p.r_kv == 512 && p.rb == 512 && rope_ok) {
    *variant = p.d_rope ? 0 : 1;
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
    case 0: {
      using C = FastCfg<512, 64, 8, 4>;
      hipLaunchKernelGGL((decode_fast_kernel<512, 64, 8, 4>), grid, dim3(512), C::LDS, s, p);
      break;
    }
    case 1: {
      using C = FastCfg<512, 0, 8, 4>;
      hipLaunchKernelGGL((decode_fast_kernel<512, 0, 8, 4>), grid, dim3(512), C::LDS, s, p);
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
