// Weight-streaming projection GEMM for few rows (M <= 128: one new token per sequence in
// decode, or a short append).  out[m, n] = sum_k A[m, k] W[n, k] with W in [out][in] layout.
//
// With M this small the product reads each weight once and does 2M flops per weight
// element, far below the matrix-core ridge, so the kernel is built to stream W at HBM
// rate: a block owns 64 output columns (two 32-row blocks of W) and a slab of K; its four
// waves take interleaved 16-wide k-steps, loading W and A fragments straight from global
// memory in the 32x32x16 MFMA operand layout (a wave's four neighbours read the other
// quarters of the same 128-byte lines at the same time), with U k-steps of loads in flight
// per wave.  The waves' accumulators are summed through LDS in a fixed order.  A single
// slab applies the shared epilogue directly; several slabs (split K, so that enough blocks
// cover the 256 compute units when N is small) write fp32 partial blocks to the caller's
// workspace and a second kernel sums them in slab order and applies the epilogue.
#include "common.h"
#include "gemm_epilogue.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int kCols = 64;           // output columns per block
constexpr int kLdc = kCols + 4;     // LDS row stride (floats)
constexpr int kTargetBlocks = 256;  // one block per compute unit

struct Goff {
  long long a, w, o;
};

__device__ __forceinline__ Goff group_offsets(const GemmParams& p, int z) {
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  return {zo * p.a_goff[0] + zi * p.a_goff[1], zo * p.w_goff[0] + zi * p.w_goff[1],
          zo * p.o_goff[0] + zi * p.o_goff[1]};
}

__device__ __forceinline__ long long a_row(const GemmParams& p, int m) {
  if (!p.a_cache) return m;
  const int b = m / p.rows_per_batch;
  return (long long)b * p.a_bstride + (m - b * p.rows_per_batch);
}

// CB = 32-row blocks of A (M <= 32 CB); U = k-steps per wave per loop trip.
template <int CB, int U>
__global__ void __launch_bounds__(256) skinny_kernel(GemmParams p) {
  __shared__ float Cs[32 * CB * kLdc];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int n0 = blockIdx.x * kCols;
  const int split = blockIdx.y;
  const int z = blockIdx.z;
  const Goff g = group_offsets(p, z);
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const int k_begin = split * p.kchunk;
  const int k_end = min(p.K, k_begin + p.kchunk);

  // lane -> W row n0 + 32 rb + col (clamped into range; such columns are never stored)
  const bf16* wrow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int n = min(n0 + 32 * rb + col, N - 1);
    const int s = (n < p.seg[0].n) ? 0 : 1;
    const int nn = n - (s ? p.seg[0].n : 0);
    wrow[rb] = reinterpret_cast<const bf16*>(p.seg[s].w) + g.w + (long long)nn * p.seg[s].w_ld + 8 * half;
  }
  // lane -> A row 32 cb + col (clamped likewise)
  const bf16* xrow[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int m = min(32 * cb + col, p.M - 1);
    xrow[cb] = reinterpret_cast<const bf16*>(p.a) + a_row(p, m) * p.a_ld + g.a + 8 * half;
  }

  f32x16 acc[2][CB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16{};

  for (int kb = k_begin + 16 * wave; kb < k_end; kb += 64 * U) {
    Frag<bf16> fw[U][2], fx[U][CB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + 64 * u;
      const bool ok = k < k_end;   // k_end - k is a multiple of 16
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) fw[u][rb] = ok ? frag_load<bf16>(wrow[rb] + k) : frag_zero<bf16>();
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) fx[u][cb] = ok ? frag_load<bf16>(xrow[cb] + k) : frag_zero<bf16>();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mma32(fw[u][rb], fx[u][cb], acc[rb][cb]);
  }

  // Sum the four waves' partial products in wave order.  Accumulator element e of lane l
  // is out[32 cb + l%32][32 rb + 8 (e/4) + 4 (l/32) + e%4].
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float* dst = &Cs[(32 * cb + col) * kLdc + 32 * rb + 8 * (e >> 2) + 4 * half + (e & 3)];
            *dst = (w == 0) ? acc[rb][cb][e] : *dst + acc[rb][cb][e];
          }
    }
    __syncthreads();
  }

  if (p.splits == 1) {
    epilogue_block<bf16>(p, Cs, kLdc, 0, 32 * CB, n0, kCols, g.o, tid, 256);
    return;
  }
  float* part = p.part + ((long long)z * p.splits + split) * p.M * N;
  for (int e = tid; e < 32 * CB * kCols; e += 256) {
    const int r = e / kCols, c = e - r * kCols;
    if (r < p.M && n0 + c < N) part[(long long)r * N + n0 + c] = Cs[r * kLdc + c];
  }
}

// Sum of the slabs' partial blocks (slab order) followed by the shared epilogue.
__global__ void __launch_bounds__(256) split_reduce_kernel(GemmParams p) {
  __shared__ float Cs[128 * kLdc];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kCols;
  const int z = blockIdx.z;
  const Goff g = group_offsets(p, z);
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const long long plane = (long long)p.M * N;
  const float* part = p.part + (long long)z * p.splits * plane;
  for (int e = tid; e < p.M * kCols; e += 256) {
    const int r = e / kCols, c = e - r * kCols;
    float v = 0.f;
    if (n0 + c < N) {
      const float* src = part + (long long)r * N + n0 + c;
      for (int s = 0; s < p.splits; ++s) v += src[s * plane];
    }
    Cs[r * kLdc + c] = v;
  }
  __syncthreads();
  epilogue_block<bf16>(p, Cs, kLdc, 0, p.M, n0, kCols, g.o, tid, 256);
}

bool aligned16(const void* ptr, long long elem_off) {
  return ((reinterpret_cast<uintptr_t>(ptr) + 2 * elem_off) & 15) == 0;
}

void plan(int M, int N, int K, int groups, int* splits, int* kchunk) {
  const int tiles = cdiv(N, kCols) * groups;
  int s = kTargetBlocks / tiles;
  s = s < 1 ? 1 : s;
  const int max_s = K / 64 > 0 ? K / 64 : 1;
  s = s > max_s ? max_s : s;
  int kc = round_up(cdiv(K, s), 64);
  s = cdiv(K, kc);
  if (s <= 1) kc = K;
  *splits = s;
  *kchunk = kc;
  (void)M;
}

}  // namespace

size_t skinny_ws_bytes(int M, int N, int K, int groups) {
  if (M <= 0 || M > 128 || N <= 0 || K <= 0 || groups <= 0) return 0;
  int s, kc;
  plan(M, N, K, groups, &s, &kc);
  return s > 1 ? (size_t)s * groups * M * N * sizeof(float) : 0;
}

bool skinny_supported(const GemmParams& p, int groups) {
  if (p.w_kmajor || p.M <= 0 || p.M > 128 || p.K % 16 != 0 || p.a_ld % 8 != 0) return false;
  (void)groups;
  for (int i = 0; i < 2; ++i)
    if (p.a_goff[i] % 8 != 0 || p.w_goff[i] % 8 != 0) return false;
  if (!aligned16(p.a, 0)) return false;
  int start = 0;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (sg.w_ld % 8 != 0 || !aligned16(sg.w, 0)) return false;
    if (sg.rope == ROPE_INTERLEAVED && (start % 2 != 0 || sg.rope_d % 2 != 0)) return false;
    if (sg.rope == ROPE_HALFSPLIT && (start % kCols != 0 || sg.rope_d > kCols || kCols % sg.rope_d != 0))
      return false;
    start += sg.n;
  }
  return true;
}

hipError_t launch_skinny(GemmParams p, int groups, hipStream_t s) {
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  int splits, kc;
  plan(p.M, N, p.K, groups, &splits, &kc);
  const size_t need = splits > 1 ? (size_t)splits * groups * p.M * N * sizeof(float) : 0;
  if (splits > 1 && (p.part == nullptr || p.part_bytes < need)) {
    splits = 1;
    kc = p.K;
  }
  p.splits = splits;
  p.kchunk = kc;
  dim3 grid(cdiv(N, kCols), splits, groups);
  if (p.M <= 32)
    hipLaunchKernelGGL((skinny_kernel<1, 8>), grid, dim3(256), 0, s, p);
  else if (p.M <= 64)
    hipLaunchKernelGGL((skinny_kernel<2, 8>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((skinny_kernel<4, 4>), grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(split_reduce_kernel, dim3(cdiv(N, kCols), 1, groups), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
