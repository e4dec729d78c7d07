// Output stage shared by the projection GEMM kernels: a block of fp32 results sits in LDS
// (rows = GEMM rows m, columns = output columns n) and is rotated, scattered and stored.
//
// The rotary embedding acts on column pairs at each row's absolute position: interleaved
// pairs (2j, 2j+1) of the DSV2 page's ``apply_rotary_emb`` or half-split pairs (j, j+d/2)
// of the MLA page's ``_apply_rope``.  A pair always lies inside the block, so the partner
// value is read from LDS.  Columns of a segment may be scattered head by head, and rows may
// be cache rows (the DSV2 page's cache update at rows start_pos .. start_pos+T-1).
#pragma once

#include "common.h"
#include "internal.h"

namespace mla {

// The rotation of rope_sincos for outputs stored in bf16: the angle in revolutions, reduced to
// [-1/2, 1/2] in double, then the hardware sine and cosine (V_SIN_F32 / V_COS_F32 take
// revolutions).  Their error, about 1e-6, is far below the bf16 rounding of the rotated
// values, and they cost a few instructions against a few dozen for sincosf.
__device__ __forceinline__ void rope_sincos_rev(int pos, float inv_freq_hi, float inv_freq_lo,
                                                float* s, float* c) {
  double r = (double)pos * (((double)inv_freq_hi + (double)inv_freq_lo) * 0.15915494309189533577);
  r -= rint(r);
  const float rf = (float)r;
  *s = __builtin_amdgcn_sinf(rf);
  *c = __builtin_amdgcn_cosf(rf);
}

// Sine and cosine of a rotary angle: fp32 outputs keep sincosf, bf16 outputs take the
// hardware functions (rope_sincos_rev).
template <typename T>
__device__ __forceinline__ void rope_angle(int pos, float hi, float lo, float* s, float* c) {
  if constexpr (sizeof(T) == 2) {
    rope_sincos_rev(pos, hi, lo, s, c);
  } else {
    rope_sincos(pos, hi, lo, s, c);
  }
}

// Segment s of p for a lane-dependent s: picked from the kernel arguments (seg_out), or
// read straight from p when p is a copy in LDS (fewer registers live: the fields are loaded
// where they are used).
template <bool PLDS>
__device__ __forceinline__ decltype(auto) seg_view(const GemmParams& p, int s) {
  if constexpr (PLDS) {
    return (p.seg[s]);   // a reference into the LDS copy
  } else {
    return seg_out(p, s);
  }
}

// Cs[r * ldc + c] holds out[m0 + r][n0 + c] for r < rows, c < cols.  All threads of the
// block take part (stride `nthreads`); the caller synchronises before and after.  rtab: the
// inverse-frequency table staged in LDS by stage_rope_table (read only for rotated segments).
//
// PLDS: p is a copy of the parameters in LDS, whose segments are indexed per lane directly;
// otherwise p is the kernel argument block and seg_out picks the fields.
template <typename T, bool PLDS = false>
__device__ __forceinline__ void epilogue_block(const GemmParams& p, const float* Cs, int ldc, int m0,
                                               int rows, int n0, int cols, long long o_goff,
                                               int tid, int nthreads, const float* rtab) {
  const int N = seg_total(p);
  bool any_t = false;
  for (int i = 0; i < p.nseg; ++i) any_t = any_t || p.seg[i].layout == OUT_HEAD_T16;
  // pass 0: row-major sweep (stores contiguous along columns); pass 1: column-major sweep
  // for transposed segments (stores contiguous along tokens)
  for (int pass = 0; pass < (any_t ? 2 : 1); ++pass) {
    for (int e = tid; e < rows * cols; e += nthreads) {
      int r, c;
      if (pass == 0) {
        r = e / cols;
        c = e - r * cols;
      } else {
        c = e / rows;
        r = e - c * rows;
      }
      const int m = m0 + r, n = n0 + c;
      if (m >= p.M || n >= N) continue;
      int nn;
      const int s = seg_of(p, n, &nn);
      const auto& sg = seg_view<PLDS>(p, s);
      if ((sg.layout == OUT_HEAD_T16) != (pass == 1)) continue;
      float v = Cs[r * ldc + c];
      const int b = m / p.rows_per_batch;
      const int t = m - b * p.rows_per_batch;
      if (sg.rope != ROPE_OFF) {
        const int pos = (p.pos0 ? p.pos0[b] : 0) + t;
        const int hh = nn % sg.rope_d;
        float sn, cs;
        if (sg.rope == ROPE_INTERLEAVED) {
          const int j = hh >> 1;
          rope_angle<T>(pos, rtab[j], rtab[kMaxRopePairs + j], &sn, &cs);
          if ((hh & 1) == 0) {
            const float o = Cs[r * ldc + c + 1];
            v = v * cs - o * sn;
          } else {
            const float o = Cs[r * ldc + c - 1];
            v = o * sn + v * cs;
          }
        } else {
          const int half = sg.rope_d >> 1;
          const int j = hh % half;
          rope_angle<T>(pos, rtab[j], rtab[kMaxRopePairs + j], &sn, &cs);
          if (hh < half) {
            const float o = Cs[r * ldc + c + half];
            v = v * cs - o * sn;
          } else {
            const float o = Cs[r * ldc + c - half];
            v = o * sn + v * cs;
          }
        }
      }
      long long idx;
      if (sg.layout == OUT_ROWS) {
        long long oc = sg.out_hw ? (long long)(nn / sg.out_hw) * sg.out_hs + (nn % sg.out_hw) : nn;
        oc += o_goff;
        long long orow = m;
        if (sg.out_cache) {
          // a cache row outside the sequence's rows (a start position beyond the host bound)
          // is dropped rather than written into a neighbouring sequence
          const long long crow = (long long)(p.pos0 ? p.pos0[b] : 0) + t;
          if (crow < 0 || crow >= p.out_bstride) continue;
          orow = (long long)b * p.out_bstride + crow;
        }
        idx = orow * sg.out_ld + oc;
      } else {
        const long long cc = nn + o_goff;
        const long long head = cc / sg.out_hw, j = cc - head * sg.out_hw;
        const long long bh = (long long)b * sg.out_nh + head;
        idx = sg.layout == OUT_HEAD_MAJOR ? (bh * p.rows_per_batch + t) * sg.out_hw + j
                                          : (bh * sg.out_hw + j) * sg.out_ld + perm16(t);
      }
      if (sg.out_f32)
        reinterpret_cast<float*>(sg.out)[idx] = v;
      else
        reinterpret_cast<T*>(sg.out)[idx] = from_f32<T>(v);
    }
  }
}

}  // namespace mla

namespace mla {

// Vectorised form of epilogue_block for one wave and a block of ROWS (a multiple of 4; a
// multiple of 32 starting at a multiple of 32 inside one batch entry when a segment is
// transposed) x `cols` (a multiple of 8) values: lane l takes the 8-column runs l % 16
// (+16 ...) and rows l / 16 + 4 i, and stores 8 outputs at once; transposed segments are
// written 16 bytes per lane along the token axis.  The value at (r, c) is the sum of NPART
// blocks part_stride floats apart, added in block order.
//
// The rows of a lane are independent, so each phase (operand reads, rotation, stores) runs
// over all of them at once: with one wave per SIMD nothing else hides a row's dependent
// chain (reads, 64-bit index arithmetic, conversion), and row after row the stage had cost
// about a thousand cycles per row.
// Requires gemm_fast_epilogue_ok() on the host.  rtab as in epilogue_block.
template <typename T, int ROWS, int NPART = 1, int RGMAX = 4, bool PLDS = false>
__device__ __forceinline__ void epilogue_block_fast(const GemmParams& p, const float* Cs, int ldc, int part_stride,
                                                    int m0, int n0, int cols, long long o_goff, int lane,
                                                    const float* rtab) {
  static_assert(ROWS % 4 == 0, "rows per lane");
  constexpr int RL = ROWS / 4;                         // rows per lane
  constexpr int RG = RL < RGMAX ? RL : RGMAX;          // rows per lane taken together
  const int N = seg_total(p);
  auto cs_sum8 = [&](const float* src, float* v) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[e];
#pragma unroll
    for (int w = 1; w < NPART; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += src[w * part_stride + e];
  };
  for (int cr = lane & 15; cr < cols / 8; cr += 16) {
    const int n = n0 + 8 * cr;
    if (n >= N) continue;
    int nn;
    const int s = seg_of(p, n, &nn);
    const auto& sg = seg_view<PLDS>(p, s);
    if (sg.layout == OUT_HEAD_T16) continue;
    const long long cc = nn + o_goff;
    const int hw = sg.out_hw;
    long long head = 0, j0 = cc;
    if (hw) {
      // 32-bit division whenever the column fits (it always does for the library's shapes)
      if ((cc >> 31) == 0) {
        head = (long long)((unsigned)cc / (unsigned)hw);
      } else {
        head = cc / hw;
      }
      j0 = cc - head * hw;
    }
    const int hh = sg.rope != ROPE_OFF ? nn % sg.rope_d : 0;
    const int half = sg.rope_d >> 1;
    const bool lo = hh < half;
    // rows in groups of RG (the registers of more rows at once spilled in the larger blocks)
#pragma nounroll
    for (int g0 = 0; g0 < RL; g0 += RG) {
    float v[RG][8];
    int mrow[RG], brow[RG], trow[RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = (lane >> 4) + 4 * (g0 + i);
      mrow[i] = m0 + r;
      brow[i] = mrow[i] / p.rows_per_batch;
      trow[i] = mrow[i] - brow[i] * p.rows_per_batch;
      cs_sum8(Cs + r * ldc + 8 * cr, v[i]);
    }
    if (sg.rope == ROPE_INTERLEAVED) {
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        if (mrow[i] >= p.M) continue;
        const int pos = (p.pos0 ? p.pos0[brow[i]] : 0) + trow[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float sn, cs;
          const int jj = (hh >> 1) + q;
          rope_angle<T>(pos, rtab[jj], rtab[kMaxRopePairs + jj], &sn, &cs);
          const float x0 = v[i][2 * q], x1 = v[i][2 * q + 1];
          v[i][2 * q] = x0 * cs - x1 * sn;
          v[i][2 * q + 1] = x0 * sn + x1 * cs;
        }
      }
    } else if (sg.rope == ROPE_HALFSPLIT) {
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        if (mrow[i] >= p.M) continue;
        const int r = (lane >> 4) + 4 * (g0 + i);
        const int pos = (p.pos0 ? p.pos0[brow[i]] : 0) + trow[i];
        float o[8];
        cs_sum8(Cs + r * ldc + 8 * cr + (lo ? half : -half), o);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float sn, cs;
          const int jj = (hh + e) % half;
          rope_angle<T>(pos, rtab[jj], rtab[kMaxRopePairs + jj], &sn, &cs);
          v[i][e] = lo ? v[i][e] * cs - o[e] * sn : o[e] * sn + v[i][e] * cs;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int m = mrow[i], b = brow[i], t = trow[i];
      if (m >= p.M) continue;
      long long idx;
      if (sg.layout == OUT_ROWS) {
        const long long oc = hw ? head * sg.out_hs + j0 : cc;
        long long orow = m;
        if (sg.out_cache) {
          const long long crow = (long long)(p.pos0 ? p.pos0[b] : 0) + t;
          if (crow < 0 || crow >= p.out_bstride) continue;
          orow = (long long)b * p.out_bstride + crow;
        }
        idx = orow * sg.out_ld + oc;
      } else {
        idx = (((long long)b * sg.out_nh + head) * p.rows_per_batch + t) * hw + j0;
      }
      if (sg.out_f32) {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(sg.out) + idx);
        dst[0] = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
        dst[1] = make_float4(v[i][4], v[i][5], v[i][6], v[i][7]);
      } else {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)v[i][e];
        *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(sg.out) + idx) = o;
      }
    }
    }
  }
  // transposed segments: 8 consecutive output positions (16 bytes) per lane, 4 lanes per
  // 32-position row segment, so one store instruction fills 16 whole 64-byte segments.
  // Positions 8 u .. 8 u + 7 of a 16-group hold tokens 4 u' .. 4 u' + 3 and 8 + 4 u' ..
  // 8 + 4 u' + 3 (u' = u % 2) of the same group (perm16).
  auto cs_at = [&](int r, int c) {
    float x = Cs[r * ldc + c];
#pragma unroll
    for (int w = 1; w < NPART; ++w) x += Cs[w * part_stride + r * ldc + c];
    return x;
  };
  for (int base = 0; base < ROWS; base += 32) {
    const int m = m0 + base;
    if (m >= p.M) break;
    const int b = m / p.rows_per_batch;
    const int t0 = m - b * p.rows_per_batch;           // a multiple of 32
    const int seg = lane & 3;                          // positions 8 seg .. 8 seg + 7
    const int grp = seg >> 1, u = seg & 1;
    const int ra = base + 16 * grp + 4 * u;            // local rows of the first 4 tokens
    for (int c = lane >> 2; c < cols; c += 16) {
      const int n = n0 + c;
      if (n >= N) continue;
      int nn;
      const int s = seg_of(p, n, &nn);
      const auto& sg = seg_view<PLDS>(p, s);
      if (sg.layout != OUT_HEAD_T16) continue;
      const long long cc = nn + o_goff;
      const long long head = cc / sg.out_hw, j = cc - head * sg.out_hw;
      const long long idx = (((long long)b * sg.out_nh + head) * sg.out_hw + j) * sg.out_ld + t0 + 8 * seg;
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (bf16)cs_at(ra + e, c);
        o[4 + e] = (bf16)cs_at(ra + 8 + e, c);
      }
      *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(sg.out) + idx) = o;
    }
  }
}

}  // namespace mla
