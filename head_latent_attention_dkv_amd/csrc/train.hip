// Kernels of the training backward (the DSV2 page's MultiHeadLatentAttention and the MLA
// page's MLAAttention are trainable modules with dropout on the attention weights):
//   * sgemm_kernel: C = alpha A B + beta C for batches of strided operands (either operand
//     transposed or not, fp32 or bf16, fp32 accumulate on the MFMA of the layer's element
//     type), used for every contraction of the backward: the attention products of a query
//     block for all (sequence, head) pairs at once, and the weight and input gradients;
//   * bwd_p_kernel / bwd_ds_kernel: the softmax and dropout steps of the attention backward
//     between those products (P from the saved log-sum-exp, the dropout mask redrawn from
//     the same generator counters as the forward);
//   * rowdot_kernel (rowsum(dO o)), rope_bwd_kernel (rotations by the negative angle, the
//     rotary key's gradient summed over heads), fill_f32_kernel.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int BM = 64, BN = 64, BK = 32;   // block tile; four waves of 32 x 32
constexpr int LDT = BK + 8;                // LDS row stride (elements): spreads the 8-element reads

template <typename T>
__device__ __forceinline__ float load_any(const void* p, long long i, int is_f32) {
  return is_f32 ? reinterpret_cast<const float*>(p)[i] : to_f32(reinterpret_cast<const bf16*>(p)[i]);
}

// One workgroup per 64 x 64 block of C and batch z (blockIdx.z = z0 * zdiv + z1).  Each
// operand tile (64 rows x 32 k) is loaded element by element with its strides, the index
// that has stride 1 running fastest across the threads, converted to T and stored k-contiguous
// in LDS, so that both MFMA operands are 16-byte reads (A: row m, B: column n).
template <typename T>
__global__ void __launch_bounds__(256) sgemm_kernel(SgemmParams p) {
  __shared__ __attribute__((aligned(16))) T As[BM * LDT];
  __shared__ __attribute__((aligned(16))) T Bs[BN * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int z = blockIdx.z, z0 = z / p.zdiv, z1 = z - z0 * p.zdiv;
  const long long offA = z0 * p.sAz0 + z1 * p.sAz1, offB = z0 * p.sBz0 + z1 * p.sBz1;
  const long long offC = z0 * p.sCz0 + z1 * p.sCz1;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  f32x16 acc = f32x16{};
  for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
    for (int r = 0; r < BM * BK / 256; ++r) {
      const int e = tid + 256 * r;
      // A element (m, k): k fastest when A is k-contiguous, else m fastest
      int m, k;
      if (p.sAk == 1) { m = e / BK; k = e - m * BK; } else { k = e / BM; m = e - k * BM; }
      const int gm = m0 + m, gk = k0 + k;
      const float va = (gm < p.M && gk < p.K) ? load_any<T>(p.A, offA + gm * p.sAm + gk * p.sAk, p.a_f32) : 0.f;
      As[m * LDT + k] = from_f32<T>(va);
      int n, kb;
      if (p.sBk == 1) { n = e / BK; kb = e - n * BK; } else { kb = e / BN; n = e - kb * BN; }
      const int gn = n0 + n, gkb = k0 + kb;
      const float vb = (gn < p.N && gkb < p.K) ? load_any<T>(p.B, offB + gkb * p.sBk + gn * p.sBn, p.b_f32) : 0.f;
      Bs[n * LDT + kb] = from_f32<T>(vb);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const Frag<T> fa = frag_load<T>(As + (wm + col) * LDT + 16 * ks + 8 * half);
      const Frag<T> fb = frag_load<T>(Bs + (wn + col) * LDT + 16 * ks + 8 * half);
      acc = mma32(fa, fb, acc);
    }
    __syncthreads();
  }
  // accumulator element e of lane l: column wn + l % 32, row wm + 8 (e / 4) + 4 (l / 32) + e % 4
  const int gn = n0 + wn + col;
  if (gn >= p.N) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int gm = m0 + wm + 8 * (e >> 2) + 4 * half + (e & 3);
    if (gm >= p.M) continue;
    float* c = p.C + offC + gm * p.sCm + gn * p.sCn;
    const float v = p.alpha * acc[e];
    *c = p.beta != 0.f ? v + p.beta * *c : v;
  }
}

// P and the dropped-out P of one query block: S holds the scores of queries i0 + i (i < Tq)
// against keys j < Kn for batch z = b H + h, [z][Tq][Kn] fp32 (natural units, unscaled).
template <typename T>
__global__ void __launch_bounds__(256) bwd_p_kernel(AttnBwdParams p) {
  const long long n = (long long)p.Z * p.Tq * p.Kn;
  for (long long e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int j = (int)(e % p.Kn);
    const long long zi = e / p.Kn;
    const int i = (int)(zi % p.Tq), z = (int)(zi / p.Tq);
    const int qi = p.i0 + i;
    float pv = 0.f, pd = 0.f;
    if (j <= qi && qi < p.S) {
      pv = exp2f(p.S_[e] * p.scale_log2 - p.lse[(long long)z * p.S + qi]);
      pd = pv;
      if (p.keep_thr) {
        const unsigned bits = dropout_keep4(p.seed, p.keep_thr, j >> 2, qi, z);
        pd = ((bits >> (j & 3)) & 1u) ? pv * p.keep_scale : 0.f;
      }
    }
    reinterpret_cast<T*>(p.P)[e] = from_f32<T>(pv);
    reinterpret_cast<T*>(p.Pd)[e] = from_f32<T>(pd);
  }
}

// dS = scale (P (dPd keep / (1 - p) - D_i)) of one query block, written over dPd's type T
// buffer; D_i = rowsum(dO_i o_i).
template <typename T>
__global__ void __launch_bounds__(256) bwd_ds_kernel(AttnBwdParams p) {
  const long long n = (long long)p.Z * p.Tq * p.Kn;
  for (long long e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int j = (int)(e % p.Kn);
    const long long zi = e / p.Kn;
    const int i = (int)(zi % p.Tq), z = (int)(zi / p.Tq);
    const int qi = p.i0 + i;
    float ds = 0.f;
    if (j <= qi && qi < p.S) {
      float dp = p.S_[e];
      if (p.keep_thr) {
        const unsigned bits = dropout_keep4(p.seed, p.keep_thr, j >> 2, qi, z);
        dp = ((bits >> (j & 3)) & 1u) ? dp * p.keep_scale : 0.f;
      }
      const float pv = to_f32(reinterpret_cast<const T*>(p.P)[e]);
      ds = p.scale * pv * (dp - p.D[(long long)z * p.S + qi]);
    }
    reinterpret_cast<T*>(p.dS)[e] = from_f32<T>(ds);
  }
}

// D[(b H + h) S + i] = sum_d dO[b S + i][h][d] o[b S + i][h][d]   (dO fp32, o in T)
template <typename T>
__global__ void __launch_bounds__(256) rowdot_kernel(const float* __restrict__ dO, const T* __restrict__ o,
                                                     float* __restrict__ D, int B, int S, int H, int dv) {
  const long long r = blockIdx.x * 4ll + (threadIdx.x >> 6);     // one wave per (token, head) row
  const int lane = threadIdx.x & 63;
  if (r >= (long long)B * S * H) return;
  float acc = 0.f;
  for (int d = lane; d < dv; d += 64) acc += dO[r * dv + d] * to_f32(o[r * dv + d]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) {
    const long long bs = r / H;
    const int h = (int)(r - bs * H);
    const long long b = bs / S, i = bs - b * S;
    D[(b * H + h) * S + i] = acc;
  }
}

// Backward of the interleaved rotations: dqr0[bs][h] = R(-t) dqr[bs][h], and
// dkr0[bs] = R(-t) sum_h dkr[bs][h] (the rotary key is shared by the heads); t = bs % S.
__global__ void __launch_bounds__(256) rope_bwd_kernel(const float* __restrict__ dqr, const float* __restrict__ dkr,
                                                       float* __restrict__ dqr0, float* __restrict__ dkr0, int B,
                                                       int S, int H, int dr, RopeTable rope) {
  const long long n = (long long)B * S * (dr / 2);
  for (long long e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int j = (int)(e % (dr / 2));
    const long long bs = e / (dr / 2);
    const int t = (int)(bs % S);
    float sn, cs;
    rope_sincos(t, rope.hi[j], rope.lo[j], &sn, &cs);
    float k0 = 0.f, k1 = 0.f;
    for (int h = 0; h < H; ++h) {
      const long long o = (bs * H + h) * dr + 2 * j;
      const float a = dqr[o], b = dqr[o + 1];
      dqr0[o] = a * cs + b * sn;
      dqr0[o + 1] = -a * sn + b * cs;
      k0 += dkr[o];
      k1 += dkr[o + 1];
    }
    dkr0[bs * dr + 2 * j] = k0 * cs + k1 * sn;
    dkr0[bs * dr + 2 * j + 1] = -k0 * sn + k1 * cs;
  }
}

__global__ void fill_f32_kernel(float* p, long long n, float v) {
  for (long long e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (long long)gridDim.x * 256) p[e] = v;
}

int grid_for(long long n) {
  const long long g = (n + 255) / 256;
  return (int)(g < 65535 ? (g < 1 ? 1 : g) : 65535);
}

}  // namespace

hipError_t launch_sgemm(const SgemmParams& p, bool use_bf16, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || p.Z <= 0) return hipSuccess;
  const dim3 grid(cdiv(p.N, BN), cdiv(p.M, BM), p.Z);
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (use_bf16)
    hipLaunchKernelGGL(sgemm_kernel<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(sgemm_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_p(const AttnBwdParams& p, bool use_bf16, hipStream_t s) {
  const int g = grid_for((long long)p.Z * p.Tq * p.Kn);
  if (use_bf16) hipLaunchKernelGGL(bwd_p_kernel<bf16>, dim3(g), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(bwd_p_kernel<float>, dim3(g), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_ds(const AttnBwdParams& p, bool use_bf16, hipStream_t s) {
  const int g = grid_for((long long)p.Z * p.Tq * p.Kn);
  if (use_bf16) hipLaunchKernelGGL(bwd_ds_kernel<bf16>, dim3(g), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(bwd_ds_kernel<float>, dim3(g), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rowdot(const float* dO, const void* o, float* D, int B, int S, int H, int dv, bool use_bf16,
                         hipStream_t s) {
  const long long rows = (long long)B * S * H;
  const int g = (int)((rows + 3) / 4);
  if (use_bf16)
    hipLaunchKernelGGL(rowdot_kernel<bf16>, dim3(g), dim3(256), 0, s, dO, reinterpret_cast<const bf16*>(o), D, B, S, H, dv);
  else
    hipLaunchKernelGGL(rowdot_kernel<float>, dim3(g), dim3(256), 0, s, dO, reinterpret_cast<const float*>(o), D, B, S, H,
                       dv);
  return hipGetLastError();
}

hipError_t launch_rope_bwd(const float* dqr, const float* dkr, float* dqr0, float* dkr0, int B, int S, int H, int dr,
                           const RopeTable& rope, hipStream_t s) {
  hipLaunchKernelGGL(rope_bwd_kernel, dim3(grid_for((long long)B * S * (dr / 2))), dim3(256), 0, s, dqr, dkr, dqr0,
                     dkr0, B, S, H, dr, rope);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, long long n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace mla
