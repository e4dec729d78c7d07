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
#include <initializer_list>

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

// ---------------------------------------------------------------------------------------
// Tiled MFMA GEMM for the bf16 layers' training products: C = alpha A B + beta C with A
// [M][K] and B [K][N] of any strides whose contiguous dimension is K or M (A) / K or N (B),
// stored bf16 or fp32 (rounded to bf16 when staged), batches as in sgemm_kernel.
// 128 x 128 block tile, 32-deep k steps, 4 waves of 64 x 64 (2 x 2 accumulators of 32 x 32);
// 16-byte (bf16) or 2 x 16-byte (fp32) loads along the contiguous dimension, two LDS
// buffers filled through registers while the other is consumed.  An operand stored
// k-contiguous is staged [row][k] and read with plain 16-byte reads; one stored row-
// contiguous is staged [k][row] and read with LDS transpose reads.
// ---------------------------------------------------------------------------------------
constexpr int TM = 128, TN = 128, TK = 32;
constexpr int LDKC = TK + 8;    // [row][k] tiles: rows 80 B apart (16-row reads on distinct banks)
constexpr int LDMC = TM + 8;    // [k][row] tiles: rows 272 B apart

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// 8 consecutive elements along the operand's contiguous dimension (the first `avail` of them;
// zeros for the rest)
template <bool F32>
__device__ __forceinline__ bf16x8 load8(const void* base, long long off, int avail) {
  bf16x8 v;
  if (avail >= 8) {
    if constexpr (F32) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
      const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off + 4);
      v = (bf16x8){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
    } else {
      v = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(base) + off);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = 0.f;
      if (j < avail) x = F32 ? static_cast<const float*>(base)[off + j] : (float)static_cast<const bf16*>(base)[off + j];
      v[j] = (bf16)x;
    }
  }
  return v;
}

// Operand from a [k][row] tile by two transpose reads: the lane gets column c0 + lane % 32 at
// k rows r0 + 8 half .. r0 + 8 half + 7 (the natural k order of a 16-deep MFMA step)
__device__ __forceinline__ Frag<bf16> tr_natural(const bf16* tile, int ld, int r0, int c0, int lane) {
  const int k16 = lane & 15, g16 = lane >> 4, half = lane >> 5;
  const int r = r0 + 8 * half + (k16 >> 2);
  const int c = c0 + 16 * (g16 & 1) + 4 * (k16 & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + r * ld + c));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + (r + 4) * ld + c));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, v);
  return f;
}

// AKC: A stored k-contiguous (sAk == 1), else m-contiguous (sAm == 1); BKC likewise for B
// (sBk == 1, else sBn == 1); AF / BF: fp32 storage.
template <bool AKC, bool BKC, bool AF, bool BF>
__global__ void __launch_bounds__(256, 2) gemm_mfma_kernel(SgemmParams p) {
  constexpr int A_TILE = AKC ? TM * LDKC : TK * LDMC;
  constexpr int B_TILE = BKC ? TN * LDKC : TK * LDMC;
  __shared__ __attribute__((aligned(16))) bf16 As[2][A_TILE];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][B_TILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int z = blockIdx.z, z0 = z / p.zdiv, z1 = z - z0 * p.zdiv;
  const long long offA = z0 * p.sAz0 + z1 * p.sAz1, offB = z0 * p.sBz0 + z1 * p.sBz1;
  const long long offC = z0 * p.sCz0 + z1 * p.sCz1;

  // staging: each operand tile is 128 x 32 = 512 vectors of 8; two per thread
  bf16x8 pa[2], pb[2];
  auto gload = [&](int k0, bf16x8 (&va)[2], bf16x8 (&vb)[2]) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = tid + 256 * v;
      if constexpr (AKC) {
        const int r = idx >> 2, kc = (idx & 3) * 8, m = m0 + r, k = k0 + kc;
        va[v] = load8<AF>(p.A, offA + (long long)min(m, p.M - 1) * p.sAm + k, m < p.M ? p.K - k : 0);
      } else {
        const int kr = idx >> 4, mc = (idx & 15) * 8, k = k0 + kr, m = m0 + mc;
        va[v] = load8<AF>(p.A, offA + (long long)min(k, p.K - 1) * p.sAk + m, k < p.K ? p.M - m : 0);
      }
      if constexpr (BKC) {
        const int r = idx >> 2, kc = (idx & 3) * 8, n = n0 + r, k = k0 + kc;
        vb[v] = load8<BF>(p.B, offB + (long long)min(n, p.N - 1) * p.sBn + k, n < p.N ? p.K - k : 0);
      } else {
        const int kr = idx >> 4, nc = (idx & 15) * 8, k = k0 + kr, n = n0 + nc;
        vb[v] = load8<BF>(p.B, offB + (long long)min(k, p.K - 1) * p.sBk + n, k < p.K ? p.N - n : 0);
      }
    }
  };
  auto lstore = [&](int buf, const bf16x8 (&va)[2], const bf16x8 (&vb)[2]) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = tid + 256 * v;
      if constexpr (AKC) *reinterpret_cast<bf16x8*>(&As[buf][(idx >> 2) * LDKC + (idx & 3) * 8]) = va[v];
      else *reinterpret_cast<bf16x8*>(&As[buf][(idx >> 4) * LDMC + (idx & 15) * 8]) = va[v];
      if constexpr (BKC) *reinterpret_cast<bf16x8*>(&Bs[buf][(idx >> 2) * LDKC + (idx & 3) * 8]) = vb[v];
      else *reinterpret_cast<bf16x8*>(&Bs[buf][(idx >> 4) * LDMC + (idx & 15) * 8]) = vb[v];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = cdiv(p.K, TK);
  gload(0, pa, pb);
  lstore(0, pa, pb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * TK, pa, pb);
    const bf16* A = As[buf];
    const bf16* B = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      Frag<bf16> fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm + 32 * i;
        fa[i] = AKC ? frag_load(A + (r + col) * LDKC + 16 * ks + 8 * half) : tr_natural(A, LDMC, 16 * ks, r, lane);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn + 32 * j;
        fb[j] = BKC ? frag_load(B + (c + col) * LDKC + 16 * ks + 8 * half) : tr_natural(B, LDMC, 16 * ks, c, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma32(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1, pa, pb);
    __syncthreads();
  }
  // accumulator element e of lane l: row wm + 32 i + 8 (e / 4) + 4 half + e % 4, column
  // wn + 32 j + l % 32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn + 32 * j + col;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m >= p.M) continue;
        float* c = p.C + offC + m * p.sCm + n * p.sCn;
        const float v = p.alpha * acc[i][j][e];
        *c = p.beta != 0.f ? v + p.beta * *c : v;
      }
  }
}

template <bool AKC, bool BKC>
hipError_t launch_mfma4(const SgemmParams& p, dim3 grid, hipStream_t s) {
  if (p.a_f32 && p.b_f32) hipLaunchKernelGGL((gemm_mfma_kernel<AKC, BKC, true, true>), grid, dim3(256), 0, s, p);
  else if (p.a_f32) hipLaunchKernelGGL((gemm_mfma_kernel<AKC, BKC, true, false>), grid, dim3(256), 0, s, p);
  else if (p.b_f32) hipLaunchKernelGGL((gemm_mfma_kernel<AKC, BKC, false, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((gemm_mfma_kernel<AKC, BKC, false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
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
  // bf16 layers: the tiled MFMA kernel when each operand has a contiguous dimension whose
  // 8-element vectors are 16-byte (bf16) / 32-byte (fp32) aligned
  if (use_bf16) {
    auto aligned = [](const void* base, bool f32, std::initializer_list<long long> strides) {
      const long long es = f32 ? 4 : 2;
      if (reinterpret_cast<uintptr_t>(base) % 16 != 0) return false;
      for (long long st : strides)
        if ((st * es) % 16 != 0) return false;
      return true;
    };
    const bool akc = p.sAk == 1, amc = p.sAm == 1, bkc = p.sBk == 1, bnc = p.sBn == 1;
    const bool a_ok = (akc && aligned(p.A, p.a_f32, {p.sAm, p.sAz0, p.sAz1})) ||
                      (amc && aligned(p.A, p.a_f32, {p.sAk, p.sAz0, p.sAz1}));
    const bool b_ok = (bkc && aligned(p.B, p.b_f32, {p.sBn, p.sBz0, p.sBz1})) ||
                      (bnc && aligned(p.B, p.b_f32, {p.sBk, p.sBz0, p.sBz1}));
    if (a_ok && b_ok) {
      const dim3 grid(cdiv(p.N, TN), cdiv(p.M, TM), p.Z);
      if (grid.y > 65535 || grid.z > 65535) return hipErrorInvalidValue;
      const bool a_k = akc && aligned(p.A, p.a_f32, {p.sAm, p.sAz0, p.sAz1});
      const bool b_k = bkc && aligned(p.B, p.b_f32, {p.sBn, p.sBz0, p.sBz1});
      if (a_k && b_k) return launch_mfma4<true, true>(p, grid, s);
      if (a_k) return launch_mfma4<true, false>(p, grid, s);
      if (b_k) return launch_mfma4<false, true>(p, grid, s);
      return launch_mfma4<false, false>(p, grid, s);
    }
  }
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
