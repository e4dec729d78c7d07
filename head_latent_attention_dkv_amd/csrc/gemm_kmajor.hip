// Few-row grouped GEMM with a k-major weight (bf16): out[m, n] = sum_k A[m, k] W[k, n],
// W stored [K][N] (rows along k).  This is the absorbed-query product of the DSV2 page's
// absorbed decode, q~_h = W_UK,h^T q_C,h, run for every head at once (groups = heads).
//
// Workgroup = one group x 64 rows x 128 columns (256 in the wide form below), 4 waves (one 32-column block each, both
// 32-row blocks), 32x32x16 MFMA.  K advances 128 at a time through LDS:
//   A chunk [64 rows][128 k] at a row stride of 272 B (16 rows of one read phase fall on
//     16 distinct 16-byte bank windows);
//   W chunk [128 k][128 n] at a row stride of 288 B, read with the LDS transpose load:
//     lane (column n, half g) of the B operand receives W[16 ks + 8 g + 0..7][n] from two
//     reads of four k-rows each, so the 4 rows x 32 bytes of a 16-lane read land on
//     disjoint bank windows.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int KM_BM = 64, KM_BN = 128, KM_KC = 128;
constexpr int KM_ALD = KM_KC + 8;      // A row stride in LDS (elements): 272 B
constexpr int KM_WLD = KM_BN + 16;     // W row stride in LDS (elements): 288 B
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(256) kmajor_small_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16 As[KM_BM * KM_ALD];
  __shared__ __attribute__((aligned(16))) bf16 Ws[KM_KC * KM_WLD];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int k16 = lane & 15, g16 = lane >> 4;
  const int n0 = blockIdx.x * KM_BN;
  const int m0 = blockIdx.y * KM_BM;
  const int z = blockIdx.z;
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  const long long a_goff = zo * p.a_goff[0] + zi * p.a_goff[1];
  const long long w_goff = zo * p.w_goff[0] + zi * p.w_goff[1];
  const long long o_goff = zo * p.o_goff[0] + zi * p.o_goff[1];
  const GemmSeg& sg = p.seg[0];
  const bf16* A = reinterpret_cast<const bf16*>(p.a) + a_goff;
  const bf16* W = reinterpret_cast<const bf16*>(sg.w) + w_goff;

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int k0 = 0; k0 < p.K; k0 += KM_KC) {
    const int kc = min(KM_KC, p.K - k0);           // a multiple of 16
    // A chunk (64 rows x kc; rows beyond M repeat row M-1) and W chunk (kc rows x 128
    // columns) in 16-byte pieces: all of a thread's 12 loads are issued before the first
    // LDS store, so they are in flight together
    constexpr int NA = KM_BM * (KM_KC / 8) / 256, NW = KM_KC * (KM_BN / 8) / 256;
    bf16x8 va[NA], vw[NW];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KM_KC / 8), c = (i % (KM_KC / 8)) * 8;
      const int m = min(m0 + r, p.M - 1);
      if (c < kc) va[j] = *reinterpret_cast<const bf16x8*>(A + (long long)m * p.a_ld + k0 + c);
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KM_BN / 8), c = (i % (KM_BN / 8)) * 8;
      if (r < kc) vw[j] = *reinterpret_cast<const bf16x8*>(W + (long long)(k0 + r) * sg.w_ld + n0 + c);
    }
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KM_KC / 8), c = (i % (KM_KC / 8)) * 8;
      if (c < kc) *reinterpret_cast<bf16x8*>(&As[r * KM_ALD + c]) = va[j];
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KM_BN / 8), c = (i % (KM_BN / 8)) * 8;
      if (r < kc) *reinterpret_cast<bf16x8*>(&Ws[r * KM_WLD + c]) = vw[j];
    }
    __syncthreads();
    for (int ks = 0; ks < kc / 16; ++ks) {
      // B operand: rows 16 ks + 8 half + 4 hi + k16 / 4, columns 32 wave + 16 (g16 % 2) + 4 (k16 % 4)
      const int wr = 16 * ks + 8 * half + (k16 >> 2);
      const int wc = 32 * wave + 16 * (g16 & 1) + 4 * (k16 & 3);
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(&Ws[wr * KM_WLD + wc]));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(&Ws[(wr + 4) * KM_WLD + wc]));
      s16x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 b = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[(32 * rb + col) * KM_ALD + 16 * ks + 8 * half]);
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[rb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // accumulator element e of lane l: row 32 rb + 8 (e/4) + 4 (l/32) + e%4, column 32 wave + l%32
  const int n = n0 + 32 * wave + col;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + 32 * rb + 8 * (e >> 2) + 4 * half + (e & 3);
      if (m >= p.M) continue;
      const long long idx = (long long)m * sg.out_ld + o_goff + n;
      if (sg.out_f32) reinterpret_cast<float*>(sg.out)[idx] = acc[rb][e];
      else reinterpret_cast<bf16*>(sg.out)[idx] = (bf16)acc[rb][e];
    }
}

// Wide form for up to 64 rows and 256-column blocks: the 64 x 128 A block of a group is
// read by half as many blocks, W rows move 512 contiguous bytes at a time, and the results
// leave through LDS as whole 16-byte pieces of output rows (the 128-column form stores
// two-byte elements straight from the accumulators).  Wave w owns columns 64 w .. 64 w + 63
// (two 32-column blocks) of both 32-row blocks.
constexpr int KW_BN = 256;
constexpr int KW_WLD = KW_BN + 16;     // W row stride in LDS (elements): 544 B
constexpr int KW_OLD = KW_BN + 8;      // output staging row stride (elements): 528 B
constexpr size_t KW_LDS = (size_t)KM_BM * KM_ALD * 2 + (size_t)KM_KC * KW_WLD * 2;
static_assert((size_t)KM_BM * KW_OLD * 2 <= (size_t)KM_KC * KW_WLD * 2, "output staging fits W's space");

__global__ void __launch_bounds__(256) kmajor_wide_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char kw_smem[];
  bf16* As = reinterpret_cast<bf16*>(kw_smem);
  bf16* Ws = reinterpret_cast<bf16*>(kw_smem + (size_t)KM_BM * KM_ALD * 2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int k16 = lane & 15, g16 = lane >> 4;
  const int n0 = blockIdx.x * KW_BN;
  const int m0 = blockIdx.y * KM_BM;
  const int z = blockIdx.z;
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  const long long a_goff = zo * p.a_goff[0] + zi * p.a_goff[1];
  const long long w_goff = zo * p.w_goff[0] + zi * p.w_goff[1];
  const long long o_goff = zo * p.o_goff[0] + zi * p.o_goff[1];
  const GemmSeg& sg = p.seg[0];
  const bf16* A = reinterpret_cast<const bf16*>(p.a) + a_goff;
  const bf16* W = reinterpret_cast<const bf16*>(sg.w) + w_goff;

  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
  for (int k0 = 0; k0 < p.K; k0 += KM_KC) {
    const int kc = min(KM_KC, p.K - k0);           // a multiple of 16
    constexpr int NA = KM_BM * (KM_KC / 8) / 256, NW = KM_KC * (KW_BN / 8) / 256;
    bf16x8 va[NA], vw[NW];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KM_KC / 8), c = (i % (KM_KC / 8)) * 8;
      const int m = min(m0 + r, p.M - 1);
      if (c < kc) va[j] = *reinterpret_cast<const bf16x8*>(A + (long long)m * p.a_ld + k0 + c);
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KW_BN / 8), c = (i % (KW_BN / 8)) * 8;
      if (r < kc) vw[j] = *reinterpret_cast<const bf16x8*>(W + (long long)(k0 + r) * sg.w_ld + n0 + c);
    }
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KM_KC / 8), c = (i % (KM_KC / 8)) * 8;
      if (c < kc) *reinterpret_cast<bf16x8*>(&As[r * KM_ALD + c]) = va[j];
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int i = tid + 256 * j;
      const int r = i / (KW_BN / 8), c = (i % (KW_BN / 8)) * 8;
      if (r < kc) *reinterpret_cast<bf16x8*>(&Ws[r * KW_WLD + c]) = vw[j];
    }
    __syncthreads();
    for (int ks = 0; ks < kc / 16; ++ks) {
      // B operands: rows 16 ks + 8 half + 4 hi + k16 / 4, columns 64 wave + 32 cb + 16 (g16 % 2) + 4 (k16 % 4)
      const int wr = 16 * ks + 8 * half + (k16 >> 2);
      bf16x8 bcol[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int wc = 64 * wave + 32 * cb + 16 * (g16 & 1) + 4 * (k16 & 3);
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(&Ws[wr * KW_WLD + wc]));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(&Ws[(wr + 4) * KW_WLD + wc]));
        s16x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bcol[cb] = __builtin_bit_cast(bf16x8, bv);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[(32 * rb + col) * KM_ALD + 16 * ks + 8 * half]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bcol[cb], acc[rb][cb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // accumulator element e of lane l in (rb, cb): row 32 rb + 8 (e/4) + 4 (l/32) + e%4,
  // column 64 wave + 32 cb + l%32; staged as bf16 rows in W's space, then stored 16 bytes a lane
  bf16* Os = Ws;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        Os[(32 * rb + 8 * (e >> 2) + 4 * half + (e & 3)) * KW_OLD + 64 * wave + 32 * cb + col] = (bf16)acc[rb][cb][e];
  __syncthreads();
  bf16* out = reinterpret_cast<bf16*>(sg.out);
#pragma unroll
  for (int j = 0; j < KM_BM * (KW_BN / 8) / 256; ++j) {
    const int i = tid + 256 * j;
    const int r = i / (KW_BN / 8), c = (i % (KW_BN / 8)) * 8;
    if (m0 + r >= p.M) continue;
    *reinterpret_cast<bf16x8*>(out + (long long)(m0 + r) * sg.out_ld + o_goff + n0 + c) =
        *reinterpret_cast<const bf16x8*>(&Os[r * KW_OLD + c]);
  }
}

bool kmajor_wide_ok(const GemmParams& p) {
  const GemmSeg& sg = p.seg[0];
  if (p.M > KM_BM || sg.n % KW_BN != 0 || sg.out_f32 || sg.out_ld % 8 != 0) return false;
  for (int i = 0; i < 2; ++i)
    if (p.o_goff[i] % 8 != 0) return false;
  return (reinterpret_cast<uintptr_t>(sg.out) & 15) == 0;
}

}  // namespace

bool kmajor_small_supported(const GemmParams& p, int groups) {
  (void)groups;
  const GemmSeg& sg = p.seg[0];
  if (!p.w_kmajor || p.nseg != 1 || p.a_cache || p.M <= 0 || p.M > 256) return false;
  if (p.K % 16 != 0 || sg.n % KM_BN != 0 || p.a_ld % 8 != 0 || sg.w_ld % 8 != 0) return false;
  if (sg.layout != OUT_ROWS || sg.rope != ROPE_OFF || sg.out_cache || sg.out_hw != 0) return false;
  for (int i = 0; i < 2; ++i)
    if (p.a_goff[i] % 8 != 0 || p.w_goff[i] % 8 != 0) return false;
  return (reinterpret_cast<uintptr_t>(p.a) & 15) == 0 && (reinterpret_cast<uintptr_t>(sg.w) & 15) == 0;
}

hipError_t launch_kmajor_small(const GemmParams& p, int groups, hipStream_t s) {
  if (kmajor_wide_ok(p)) {
    dim3 grid(p.seg[0].n / KW_BN, 1, groups);
    hipLaunchKernelGGL(kmajor_wide_kernel, grid, dim3(256), KW_LDS, s, p);
    return hipGetLastError();
  }
  dim3 grid(p.seg[0].n / KM_BN, cdiv(p.M, KM_BM), groups);
  hipLaunchKernelGGL(kmajor_small_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
