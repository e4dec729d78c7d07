// Projection GEMM for the MLA layer on gfx950 matrix cores.
//
// out[m, n] = sum_k A[m, k] W[n, k] (weights in [out][in] layout), or with a k-major W
// for the absorbed query W_UK,h^T q_C,h.  The epilogue applies the rotary embedding
// (interleaved pairs of the DSV2 page's ``apply_rotary_emb`` or half-split pairs of the
// MLA page's ``_apply_rope``) at each row's absolute position, scatters columns head by
// head and writes either plain rows or cache rows (the DSV2 page's cache update at rows
// start_pos .. start_pos+T-1), so the down-projection, RoPE and cache write of a new
// token are one launch.
//
// Tiling: BM x BN output tile, BK = 64 per stage, 4 waves in a 2 x 2 grid, each wave
// owning a (BM/2) x (BN/2) block of 16x16 MFMA accumulators.  A and W tiles are staged
// global -> registers -> LDS with k contiguous (row stride BK + 8 elements, which puts
// the 16 rows of one fragment read on distinct LDS banks); the next stage's global loads
// are issued before the current stage's MFMAs.
#include "common.h"
#include "gemm_epilogue.h"
#include "internal.h"

namespace mla {

namespace {

template <int BM, int BN>
struct Tile {
  static constexpr int BK = 64;
  static constexpr int LDK = BK + 8;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_PER_T = BM * BK / 8 / 256;
  static constexpr int B_PER_T = BN * BK / 8 / 256;
  static constexpr int LDC = BN + 4;
};

__device__ __forceinline__ long long a_row_index(const GemmParams& p, int m) {
  if (!p.a_cache) return m;
  int b = m / p.rows_per_batch;
  int t = m - b * p.rows_per_batch;
  return (long long)b * p.a_bstride + t;
}

template <typename T>
__device__ __forceinline__ void load_vec_or_partial(Chunk<T>& c, const T* ptr, int nvalid) {
  if (nvalid >= 8 && ((reinterpret_cast<uintptr_t>(ptr) & 15) == 0)) {
    chunk_load<T>(c, ptr);
  } else if (nvalid > 0) {
    chunk_load_partial<T>(c, ptr, nvalid < 8 ? nvalid : 8);
  } else {
    chunk_zero<T>(c);
  }
}

template <typename T, int BM, int BN>
__global__ void __launch_bounds__(256) gemm_kernel(GemmParams p) {
  using TL = Tile<BM, BN>;
  constexpr int BK = TL::BK, LDK = TL::LDK;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* As = reinterpret_cast<T*>(smem_raw);
  T* Bs = As + BM * LDK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int z = blockIdx.z;
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  const long long a_goff = zo * p.a_goff[0] + zi * p.a_goff[1];
  const long long w_goff = zo * p.w_goff[0] + zi * p.w_goff[1];
  const long long o_goff = zo * p.o_goff[0] + zi * p.o_goff[1];
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const int K = p.K;
  const T* A = reinterpret_cast<const T*>(p.a);

  Chunk<T> ra[TL::A_PER_T];
  Chunk<T> rb[TL::B_PER_T];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < TL::A_PER_T; ++i) {
      int ci = tid + i * 256;
      int r = ci / (BK / 8), c = ci % (BK / 8);
      int m = m0 + r, k = k0 + c * 8;
      if (m < p.M) {
        const T* ptr = A + a_row_index(p, m) * p.a_ld + a_goff + k;
        load_vec_or_partial<T>(ra[i], ptr, K - k);
      } else {
        chunk_zero<T>(ra[i]);
      }
    }
    if (!p.w_kmajor) {
#pragma unroll
      for (int i = 0; i < TL::B_PER_T; ++i) {
        int ci = tid + i * 256;
        int r = ci / (BK / 8), c = ci % (BK / 8);
        int n = n0 + r, k = k0 + c * 8;
        if (n < N) {
          int s = (n < p.seg[0].n) ? 0 : 1;
          int nn = n - (s ? p.seg[0].n : 0);
          const T* ptr = reinterpret_cast<const T*>(p.seg[s].w) + w_goff + (long long)nn * p.seg[s].w_ld + k;
          load_vec_or_partial<T>(rb[i], ptr, K - k);
        } else {
          chunk_zero<T>(rb[i]);
        }
      }
    } else {
      // W[k][n]: chunks run along n; a wave covers 8 k-rows x 8 n-chunks.
#pragma unroll
      for (int i = 0; i < TL::B_PER_T; ++i) {
        int ci = tid + i * 256;
        int blk = ci >> 6, l = ci & 63;
        int kk = 8 * (blk % (BK / 8)) + (l & 7);
        int c = 8 * (blk / (BK / 8)) + (l >> 3);
        int k = k0 + kk, n = n0 + c * 8;
        if (k < K && n < N) {
          const T* ptr = reinterpret_cast<const T*>(p.seg[0].w) + w_goff + (long long)k * p.seg[0].w_ld + n;
          load_vec_or_partial<T>(rb[i], ptr, N - n);
        } else {
          chunk_zero<T>(rb[i]);
        }
      }
    }
  };

  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < TL::A_PER_T; ++i) {
      int ci = tid + i * 256;
      int r = ci / (BK / 8), c = ci % (BK / 8);
      chunk_store<T>(As + r * LDK + c * 8, ra[i]);
    }
    if (!p.w_kmajor) {
#pragma unroll
      for (int i = 0; i < TL::B_PER_T; ++i) {
        int ci = tid + i * 256;
        int r = ci / (BK / 8), c = ci % (BK / 8);
        chunk_store<T>(Bs + r * LDK + c * 8, rb[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TL::B_PER_T; ++i) {
        int ci = tid + i * 256;
        int blk = ci >> 6, l = ci & 63;
        int kk = 8 * (blk % (BK / 8)) + (l & 7);
        int c = 8 * (blk / (BK / 8)) + (l >> 3);
        chunk_store_column<T>(Bs + (c * 8) * LDK + kk, LDK, rb[i]);
      }
    }
  };

  f32x4 acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nk = cdiv(K, BK);
  load_stage(0);
  for (int kt = 0; kt < nk; ++kt) {
    store_stage();
    __syncthreads();
    if (kt + 1 < nk) load_stage((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      Frag<T> fb[TL::FN];
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
        fb[j] = frag_load<T>(Bs + (wn * TL::WN + j * 16 + (lane & 15)) * LDK + ks * 32 + 8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        Frag<T> fa = frag_load<T>(As + (wm * TL::WM + i * 16 + (lane & 15)) * LDK + ks * 32 + 8 * (lane >> 4));
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = mma16(fa, fb[j], acc[i][j]);
      }
    }
    __syncthreads();
  }

  // ---- epilogue through LDS: rotary pairs may sit in other lanes / waves ----
  __shared__ float rtab[kRopeTabFloats];
  if (gemm_has_rope(p)) stage_rope_table(p, rtab, tid, 256);
  float* Cs = reinterpret_cast<float*>(smem_raw);
  constexpr int LDC = TL::LDC;
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int r = wm * TL::WM + i * 16 + 4 * (lane >> 4) + e;
        int c = wn * TL::WN + j * 16 + (lane & 15);
        Cs[r * LDC + c] = acc[i][j][e];
      }
  __syncthreads();

  epilogue_block<T>(p, Cs, LDC, m0, BM, n0, BN, o_goff, tid, 256, rtab);
}

template <typename T, int BM, int BN>
hipError_t launch_tile(const GemmParams& p, int groups, hipStream_t s) {
  using TL = Tile<BM, BN>;
  int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  size_t stage = (size_t)(BM + BN) * TL::LDK * sizeof(T);
  size_t epi = (size_t)BM * TL::LDC * sizeof(float);
  size_t lds = stage > epi ? stage : epi;
  dim3 grid(cdiv(N, BN), cdiv(p.M, BM), groups);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, int groups, bool use_bf16, hipStream_t s) {
  int N = seg_total(p);
  if (p.M <= 0 || N <= 0 || groups <= 0) return hipSuccess;
  // three output segments: the few-row path only (the other kernels index two)
  if (p.nseg > 2) {
    if (use_bf16 && !kmajor_small_supported(p, groups) && skinny_supported(p, groups)) return launch_skinny(p, groups, s);
    return hipErrorInvalidValue;
  }
  int max_rope_d = 0;
  for (int i = 0; i < p.nseg; ++i)
    if (p.seg[i].rope == ROPE_HALFSPLIT && p.seg[i].rope_d > max_rope_d) max_rope_d = p.seg[i].rope_d;
  if (!use_bf16) return launch_tile<float, 64, 64>(p, groups, s);
  if (kmajor_small_supported(p, groups)) return launch_kmajor_small(p, groups, s);
  if (skinny_supported(p, groups)) return launch_skinny(p, groups, s);
  if (gemm_big_supported(p, groups)) return launch_gemm_big(p, groups, s);
  bool big = (long long)cdiv(p.M, 128) * cdiv(N, 128) * groups >= 512;
  if (big || max_rope_d > 64) return launch_tile<bf16, 128, 128>(p, groups, s);
  return launch_tile<bf16, 64, 64>(p, groups, s);
}

}  // namespace mla
