// Large projection GEMM for gfx950 (bf16, many rows): out[m, n] = sum_k A[m, k] W[n, k].
//
// Workgroup tile 256 x 256, 8 waves (two per SIMD) in a 4 x 2 grid, or 256 x 128 with 4 waves
// in a 4 x 1 grid and two workgroups per CU (one's output stage overlaps the other's main
// loop); each wave a 64 x 128 block of 32x32x16 MFMA accumulators (8 x 16 fp32 per lane, in
// the accumulation registers).  K advances 32 at a time through NST LDS stages filled by
// 16-byte direct-to-LDS copies: each copy instruction moves 16 rows x 64 bytes of A or of W.  Rows are 64 bytes (four
// 16-byte chunks); chunk c of row r sits at c ^ ((r >> 2) & 3), which puts the 8 rows of
// one LDS read phase (row stride 64 B) on 8 distinct 16-byte bank windows.
//
// Output stages:
//   * the keys / values of flash prefill (every wave's 128 columns inside one head of one
//     segment, bf16, no rotation) are written straight from the accumulators (values,
//     transposed) or through a small bf16 transpose in LDS (keys, head-major);
//   * everything else goes through LDS per wave, 32 rows at a time, into the shared output
//     stage (rotary pairs, head scatter, cache rows, head-major / transposed layouts).
#include <type_traits>

#include "common.h"
#include "gemm_epilogue.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int GBM = 256, GBK = 32;
constexpr int G_AB = GBM * GBK * 2;                 // A bytes per stage (16 KB)
constexpr int G_LDC = 128 + 4;                      // epilogue LDS row stride (floats)
constexpr int KV_CS = 72;                           // bf16 column stride (bytes) of the key transpose
constexpr int KV_BUF = 128 * KV_CS;                 // one 32-row x 128-column chunk

template <int NW>
struct BigCfg {
  static constexpr int BN = 32 * NW;                // workgroup columns (256 or 128)
  static constexpr int NST = NW == 8 ? 4 : 3;       // LDS stages
  static constexpr int WB = BN * GBK * 2;           // W bytes per stage
  static constexpr int STAGE = G_AB + WB;
  static constexpr int A_CPW = (G_AB / 1024) / NW;  // copies per wave per stage: A, W
  static constexpr int W_CPW = (WB / 1024) / NW;
  static constexpr int DPW = A_CPW + W_CPW;
  static constexpr size_t EPI = (size_t)NW * 32 * G_LDC * 4;   // per-wave 32-row epilogue chunks
  static constexpr size_t LDS = (size_t)NST * STAGE > EPI ? (size_t)NST * STAGE : EPI;
  static constexpr int MINB = NW == 8 ? 1 : 2;      // workgroups per CU
  static_assert((size_t)NW * KV_BUF <= LDS, "key transpose buffers fit in the stages");
  static_assert(MINB * LDS <= 160 * 1024, "workgroups per CU fit the LDS");
};
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ long long big_a_row(const GemmParams& p, int m) {
  if (!p.a_cache) return m;
  const int b = m / p.rows_per_batch;
  return (long long)b * p.a_bstride + (m - b * p.rows_per_batch);
}

__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// DIRECT: the flash-layout output stage (own instantiation: sharing one register allocation
// with the generic stage costs spills)
template <bool DIRECT, int NW>
__global__ void __launch_bounds__(64 * NW, BigCfg<NW>::MINB) gemm_big_kernel(GemmParams p) {
  using C = BigCfg<NW>;
  constexpr int GNST = C::NST;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 4), wn = wave % (NW / 4);   // 64-row block wm, 128-column block wn
  const int col = lane & 31, half = lane >> 5;
  int bx = blockIdx.x, by = blockIdx.y;
  if (DIRECT && gridDim.z == 1 && gridDim.x % 8 == 0) {
    // Workgroups go to the 8 XCDs in turn (linear block L to XCD L % 8).  XCD k takes the
    // column tiles k NT/8 .. (k+1) NT/8 - 1, in phases of up to 16 tiles, each phase over all
    // row tiles: a phase's weight rows (16 x 128 x K bf16, 2 MB at K = 512) stay in the
    // XCD's L2 while its row tiles stream past, instead of every row tile re-reading the
    // whole weight from beyond L2.
    const int NT = gridDim.x, MT = gridDim.y, per = NT / 8;
    const int pw = per % 16 == 0 ? 16 : per;
    const int L = by * NT + bx, xcd = L & 7, slot = L >> 3;
    const int ph = slot / (MT * pw), rem = slot - ph * (MT * pw);
    by = rem / pw;
    bx = xcd * per + ph * pw + (rem - by * pw);
  }
  const int n0 = bx * C::BN;
  const int m0 = by * GBM;
  const int z = blockIdx.z;
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  const long long a_goff = zo * p.a_goff[0] + zi * p.a_goff[1];
  const long long w_goff = zo * p.w_goff[0] + zi * p.w_goff[1];
  const long long o_goff = zo * p.o_goff[0] + zi * p.o_goff[1];
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const int nst = p.K / GBK;

  // copy sources: copy j of wave w covers rows 16 (CPW w + j) + lane / 4 of its operand,
  // physical chunk lane % 4, which holds logical chunk (lane % 4) ^ ((row >> 2) & 3)
  const bf16* asrc[C::A_CPW];
  const bf16* wsrc[C::W_CPW];
#pragma unroll
  for (int j = 0; j < C::A_CPW; ++j) {
    const int t = 16 * (C::A_CPW * wave + j) + lane / 4;
    const int c = (lane & 3) ^ ((t >> 2) & 3);
    const int m = min(m0 + t, p.M - 1);
    asrc[j] = reinterpret_cast<const bf16*>(p.a) + big_a_row(p, m) * p.a_ld + a_goff + 8 * c;
  }
#pragma unroll
  for (int j = 0; j < C::W_CPW; ++j) {
    const int t = 16 * (C::W_CPW * wave + j) + lane / 4;
    const int c = (lane & 3) ^ ((t >> 2) & 3);
    const int n = min(n0 + t, N - 1);
    const int s = (n < p.seg[0].n) ? 0 : 1;
    const int nn = n - (s ? p.seg[0].n : 0);
    wsrc[j] = reinterpret_cast<const bf16*>(p.seg[s].w) + w_goff + (long long)nn * p.seg[s].w_ld + 8 * c;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto issue = [&](int st) {
    const uint32_t base = lds0 + (st % GNST) * C::STAGE;
    const int k0 = st * GBK;
#pragma unroll
    for (int j = 0; j < C::A_CPW; ++j)
      dma16(asrc[j] + k0, __builtin_amdgcn_readfirstlane(base + (C::A_CPW * wave + j) * 1024));
#pragma unroll
    for (int j = 0; j < C::W_CPW; ++j)
      dma16(wsrc[j] + k0, __builtin_amdgcn_readfirstlane(base + G_AB + (C::W_CPW * wave + j) * 1024));
  };

  // operand read: row r (= 32 blk + col within the wave's block), logical chunk 2 ks + half;
  // r mod 32 = col, so the swizzle key (r >> 2) & 3 = (col >> 2) & 3 for every block
  const int rd_base = col * 64 | ((((col >> 2) & 3) ^ half) << 4);   // XOR (2 ks) << 4 below

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  copies_begin();   // lds_dma.h, rule 1
#pragma unroll
  for (int st = 0; st < GNST - 1; ++st)
    if (st < nst) issue(st);
  for (int it = 0; it < nst; ++it) {
    const int left = nst - 1 - it;
    if (GNST >= 4 && left >= 2) wait_vmcnt<2 * C::DPW>();
    else if (left >= 1) wait_vmcnt<C::DPW>();
    else wait_vmcnt<0>();
    barrier_only();
    if (it + GNST - 1 < nst) issue(it + GNST - 1);
    const unsigned char* T = smem + (it % GNST) * C::STAGE;
    const int rb0 = opaque_int(rd_base);
    Frag<bf16> fa[2][2], fb[2][4];
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      const int off = rb0 ^ (ks << 5);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[ks][i] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + off + (64 * wm + 32 * i) * 64));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[ks][j] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + G_AB + off + (128 * wn + 32 * j) * 64));
    }
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma32(fa[ks][i], fb[ks][j], acc[i][j]);
    // issue order: the first step's 6 operand reads, then its 8 products with the second
    // step's 6 reads slotted in after the first 6, then the second step's products
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
  }
  copies_end();   // lds_dma.h, rule 3
  __syncthreads();

  if constexpr (DIRECT) {
    // Flash layouts.  The wave's columns N0 .. N0 + 127 are columns j0 .. j0 + 127 of one head.
    const int N0 = n0 + 128 * wn;
    if (N0 >= N) return;
    const int s = N0 < p.seg[0].n ? 0 : 1;
    const GemmSeg& sg = p.seg[s];
    const int cc = N0 - (s ? p.seg[0].n : 0) + (int)o_goff;
    const int head = cc / sg.out_hw, j0 = cc - head * sg.out_hw;
    bf16* out = reinterpret_cast<bf16*>(sg.out);
    if (sg.layout == OUT_HEAD_T16) {
      // Row j of a head holds the tokens in perm16 order: positions 8 u .. 8 u + 7 of a
      // 16-token group are tokens 4 u .. 4 u + 3 and 8 + 4 u .. 8 + 4 u + 3, i.e. the
      // accumulator elements 8 g .. 8 g + 7 of the lanes with l / 32 = u (rows
      // 16 g + 4 u + e % 4 and 16 g + 8 + 4 u + e % 4).  One 16-byte store per lane,
      // 32-column block and 16-token group.
      const long long jstride = 32LL * sg.out_ld;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + 64 * wm + 32 * i;
        if (m >= p.M) break;
        const int b = m / p.rows_per_batch, t = m - b * p.rows_per_batch;
        bf16* base = out + ((long long)(b * sg.out_nh + head) * sg.out_hw + j0 + col) * sg.out_ld + t + 8 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[i][j][8 * g + e];
            *reinterpret_cast<bf16x8*>(base + j * jstride + 16 * g) = o;
          }
      }
    } else {
      // Head-major rows: chunk i (32 rows) goes to LDS column-major as bf16 (column stride
      // 72 B: the 16 columns of one write phase fall on distinct bank pairs); the LDS
      // transpose load then hands lane x of a 16-lane group 4 consecutive columns of row
      // r0 + x, and two loads make one 16-byte store.
      // (one buffer per wave: a wave's LDS accesses complete in issue order)
      unsigned char* buf = smem + wave * KV_BUF;
      const int g16 = lane >> 4, x16 = lane & 15;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + 64 * wm + 32 * i;
        if (m >= p.M) break;
        const int b = m / p.rows_per_batch, t = m - b * p.rows_per_batch;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[i][j][4 * q + e];
            *reinterpret_cast<bf16x4*>(buf + (32 * j + col) * KV_CS + (8 * q + 4 * half) * 2) = o;
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        bf16* base = out + ((long long)(b * sg.out_nh + head) * p.rows_per_batch + t) * sg.out_hw + j0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r0 = 16 * (u & 1), c0 = 32 * (u >> 1) + 8 * g16;
          const unsigned char* rd = buf + (c0 + (x16 >> 2)) * KV_CS + (r0 + 4 * (x16 & 3)) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(rd));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(rd + 4 * KV_CS));
          const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          *reinterpret_cast<s16x8*>(base + (r0 + x16) * sg.out_hw + c0) = v;
        }
      }
    }
  } else {
  // Epilogue per wave: its 64 x 128 block in two chunks of 32 rows.  Accumulator element
  // e of lane l in block (i, j) is out[64 wm + 32 i + 8 (e/4) + 4 (l/32) + e%4][128 wn + 32 j + l%32].
  float* Cs = reinterpret_cast<float*>(smem) + wave * 32 * G_LDC;
  auto stage = [&](auto I) {                    // chunk I with compile-time accumulator indices
    constexpr int i = decltype(I)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) Cs[(8 * (e >> 2) + 4 * half + (e & 3)) * G_LDC + 32 * j + col] = acc[i][j][e];
  };
#pragma nounroll
  for (int i = 0; i < 2; ++i) {
    if (i == 0) stage(std::integral_constant<int, 0>{});
    else stage(std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    if (p.fast_epilogue)
      epilogue_block_fast<bf16>(p, Cs, G_LDC, m0 + 64 * wm + 32 * i, 32, n0 + 128 * wn, 128, o_goff, lane);
    else
      epilogue_block<bf16>(p, Cs, G_LDC, m0 + 64 * wm + 32 * i, 32, n0 + 128 * wn, 128, o_goff, lane, 64);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
  }
}

}  // namespace

bool gemm_big_supported(const GemmParams& p, int groups) {
  (void)groups;
  if (p.w_kmajor || p.M < GBM || p.K % GBK != 0 || p.a_ld % 8 != 0) return false;
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  if (N < 128) return false;
  for (int i = 0; i < 2; ++i)
    if (p.a_goff[i] % 8 != 0 || p.w_goff[i] % 8 != 0) return false;
  if ((reinterpret_cast<uintptr_t>(p.a) & 15) != 0) return false;
  int start = 0;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (sg.w_ld % 8 != 0 || (reinterpret_cast<uintptr_t>(sg.w) & 15) != 0) return false;
    if (sg.rope == ROPE_INTERLEAVED && (start % 2 != 0 || sg.rope_d % 2 != 0)) return false;
    if (sg.rope == ROPE_HALFSPLIT && (start % 128 != 0 || sg.rope_d > 128 || 128 % sg.rope_d != 0)) return false;
    start += sg.n;
  }
  return true;
}

bool gemm_fast_epilogue_ok(const GemmParams& p, int groups) {
  auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
  if (p.seg[0].n % 8 != 0) return false;
  for (int i = 0; i < 2; ++i)
    if (p.o_goff[i] % 8 != 0) return false;
  (void)groups;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (!al16(sg.out)) return false;
    if (sg.rope != ROPE_OFF && sg.rope_d % 8 != 0) return false;
    if (sg.rope == ROPE_HALFSPLIT && (sg.rope_d / 2) % 8 != 0) return false;
    if (sg.layout == OUT_ROWS) {
      if (sg.out_hw % 8 != 0 || sg.out_hs % 8 != 0 || sg.out_ld % 8 != 0) return false;
    } else if (sg.layout == OUT_HEAD_MAJOR) {
      if (sg.out_hw % 8 != 0) return false;
    } else {
      if (sg.out_f32 || sg.out_ld % 16 != 0 || p.rows_per_batch % 32 != 0) return false;
    }
  }
  return true;
}

// Flash-layout output stage: bf16 head-major / transposed segments without rotation, every
// 128-column block inside one head of one segment, 32-row chunks inside one sequence.
static bool kv_direct_ok(const GemmParams& p) {
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  if (N % 128 != 0 || p.rows_per_batch % 32 != 0 || p.M % 32 != 0) return false;
  for (int i = 0; i < 2; ++i)
    if (p.o_goff[i] % 128 != 0) return false;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (sg.layout == OUT_ROWS || sg.out_f32 || sg.rope != ROPE_OFF) return false;
    if (sg.n % 128 != 0 || sg.out_hw % 128 != 0) return false;
  }
  return true;
}

hipError_t launch_gemm_big(const GemmParams& pin, int groups, hipStream_t s) {
  GemmParams p = pin;
  p.fast_epilogue = gemm_fast_epilogue_ok(p, groups) ? (kv_direct_ok(p) ? 2 : 1) : 0;
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  // The flash-layout stage (the prefill K/V up-projection) takes 256 x 128 tiles, two
  // workgroups per CU (820 -> 780 us at B=4, S=4096); the other projections measured the
  // same or slower that way and keep 256 x 256.
  if (p.fast_epilogue == 2) {
    using C = BigCfg<4>;
    dim3 grid(cdiv(N, C::BN), cdiv(p.M, GBM), groups);
    hipLaunchKernelGGL((gemm_big_kernel<true, 4>), grid, dim3(64 * 4), C::LDS, s, p);
  } else {
    using C = BigCfg<8>;
    dim3 grid(cdiv(N, C::BN), cdiv(p.M, GBM), groups);
    hipLaunchKernelGGL((gemm_big_kernel<false, 8>), grid, dim3(64 * 8), C::LDS, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
