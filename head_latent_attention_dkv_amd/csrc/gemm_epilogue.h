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

// Cs[r * ldc + c] holds out[m0 + r][n0 + c] for r < rows, c < cols.  All threads of the
// block take part (stride `nthreads`); the caller synchronises before and after.
template <typename T>
__device__ __forceinline__ void epilogue_block(const GemmParams& p, const float* Cs, int ldc, int m0,
                                               int rows, int n0, int cols, long long o_goff,
                                               int tid, int nthreads) {
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const bool any_t = p.seg[0].layout == OUT_HEAD_T16 || (p.nseg > 1 && p.seg[1].layout == OUT_HEAD_T16);
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
      const int s = (n < p.seg[0].n) ? 0 : 1;
      const GemmSeg& sg = p.seg[s];
      if ((sg.layout == OUT_HEAD_T16) != (pass == 1)) continue;
      const int nn = n - (s ? p.seg[0].n : 0);
      float v = Cs[r * ldc + c];
      const int b = m / p.rows_per_batch;
      const int t = m - b * p.rows_per_batch;
      if (sg.rope != ROPE_OFF) {
        const int pos = (p.pos0 ? p.pos0[b] : 0) + t;
        const int hh = nn % sg.rope_d;
        float sn, cs;
        if (sg.rope == ROPE_INTERLEAVED) {
          const int j = hh >> 1;
          rope_sincos(pos, p.rope.hi[j], p.rope.lo[j], &sn, &cs);
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
          rope_sincos(pos, p.rope.hi[j], p.rope.lo[j], &sn, &cs);
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
        const long long orow = sg.out_cache ? (long long)b * p.out_bstride + (p.pos0 ? p.pos0[b] : 0) + t : m;
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
