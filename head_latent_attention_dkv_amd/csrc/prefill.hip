// Flash-style causal prefill over explicitly up-projected keys and values.
//
// Computes, per head, o_i = sum_{j<=i} softmax_j(scale * q_i . k_j) v_j with the keys
// k_j = [W_UK c_j ; k_R,j] (the DSV2 page's concatenation of the decompressed key and the
// rotary key shared by all heads), or the rotated decompressed key of the MLA page, or
// the block up-projected key of the MLRA page.  The query tile never materialises the
// full score matrix: keys stream through LDS in tiles of 64 with an online softmax.
//
// Workgroup: 128 queries of one (sequence, head), 4 waves x 32 queries.  Per key tile
//   S^T[64 keys x 32 queries] = K_tile[64 x DQ] . Q^T          (32x32x16 MFMA, K = DQ)
//   O^T[DV x 32 queries]     += V_tile^T[DV x 64] . P^T[64 x 32] (32x32x16 MFMA, K = keys)
// so each lane owns one query's column: the row maximum / sum and the rescale of O are
// per-lane scalars.  K is staged row-major, V transposed (keys contiguous per value
// column), both from registers that were loaded while the previous tile computed.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int BQ = 128;    // queries per workgroup
constexpr int BKEY = 64;   // keys per tile
constexpr float kLazyRescale = 8.0f;

template <typename T, int DQP, int DVP>
struct PrefillCfg {
  static constexpr int KS = DQP / 16;
  static constexpr int RPAD = 16 / (int)sizeof(T);
  static constexpr int KRS = DQP + RPAD;             // K tile row stride
  static constexpr int VTS = BKEY + 4;               // V^T row stride
  static constexpr int CK = DQP / 8, CV = DVP / 8;   // chunks per key row
  static constexpr int KCB = (CK + 7) / 8, VCB = (CV + 7) / 8;
  static constexpr int KBLK = (BKEY / 8) * KCB, VBLK = (BKEY / 8) * VCB;
  static constexpr int NBLK = KBLK + VBLK;
  static constexpr int BPW = (NBLK + 3) / 4;
  static constexpr size_t LDS = (size_t)BKEY * KRS * sizeof(T) + (size_t)DVP * VTS * sizeof(T);
  static_assert(DQP % 16 == 0 && DVP % 32 == 0, "padded widths");
};

template <typename T, int DQP, int DVP>
__global__ void __launch_bounds__(256) prefill_kernel(PrefillParams p) {
  using C = PrefillCfg<T, DQP, DVP>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* Ks = reinterpret_cast<T*>(smem_raw);      // [BKEY][KRS]
  T* Vt = Ks + BKEY * C::KRS;                  // [DVP][VTS]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int n_qt = (p.T + BQ - 1) / BQ;
  const int qt = n_qt - 1 - blockIdx.x;          // heaviest (latest) query tiles first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int q0 = qt * BQ;
  const int qw0 = q0 + wave * 32;                 // this wave's first query (index among the T)
  const int query = qw0 + col;
  const int qa0 = p.q_off + qw0, qabs = p.q_off + query;   // their positions
  const int dq = p.dn + p.d_rope;

  const T* Q = reinterpret_cast<const T*>(p.q);
  const T* Kg = reinterpret_cast<const T*>(p.k);
  const T* KRg = reinterpret_cast<const T*>(p.kr);
  const T* Vg = reinterpret_cast<const T*>(p.v);

  Frag<T> qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int d = ks * 16 + 8 * half + j;
      v[j] = (query < p.T && d < dq) ? to_f32(Q[(((long long)b * p.T + query) * p.H + h) * dq + d]) : 0.f;
    }
    qf[ks] = frag_from_f32<T>(v);
  }

  f32x16 acc[DVP / 32];
#pragma unroll
  for (int mb = 0; mb < DVP / 32; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // key / value head of this query head (grouped-query attention when kv_group > 1)
  const int kvg = p.kv_group > 1 ? p.kv_group : 1;
  const int hk = h / kvg;
  const long long hdn = (long long)(p.H / kvg) * p.dn, hdv = (long long)(p.H / kvg) * p.dv;
  Chunk<T> st[C::BPW];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
      int blk = wave + i * 4;
      chunk_zero<T>(st[i]);
      if (blk >= C::NBLK) continue;
      bool isv = blk >= C::KBLK;
      int bb = isv ? blk - C::KBLK : blk;
      int cb = isv ? C::VCB : C::KCB;
      int rblk = bb / cb, cblk = bb - rblk * cb;
      int r = rblk * 8 + (lane & 7);
      int c = cblk * 8 + (lane >> 3);
      int key = k0 + r;
      if (key >= p.S) continue;
      int d = c * 8;
      const T* src = nullptr;
      int nv = 0;
      if (!isv) {
        if (c >= C::CK) continue;
        if (d < p.dn) {
          src = Kg + ((long long)b * p.S + key) * hdn + (long long)hk * p.dn + d;
          nv = p.dn - d;
        } else if (d - p.dn < p.d_rope) {
          src = KRg + ((long long)b * p.kr_bstride + key) * p.d_rope + (d - p.dn);
          nv = p.d_rope - (d - p.dn);
        }
      } else {
        if (c >= C::CV) continue;
        if (d < p.dv) {
          src = Vg + ((long long)b * p.S + key) * hdv + (long long)hk * p.dv + d;
          nv = p.dv - d;
        }
      }
      if (nv <= 0) continue;
      if (nv >= 8 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) chunk_load<T>(st[i], src);
      else chunk_load_partial<T>(st[i], src, nv < 8 ? nv : 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
      int blk = wave + i * 4;
      if (blk >= C::NBLK) continue;
      bool isv = blk >= C::KBLK;
      int bb = isv ? blk - C::KBLK : blk;
      int cb = isv ? C::VCB : C::KCB;
      int rblk = bb / cb, cblk = bb - rblk * cb;
      int r = rblk * 8 + (lane & 7);
      int c = cblk * 8 + (lane >> 3);
      if (!isv) {
        if (c < C::CK) chunk_store<T>(Ks + r * C::KRS + c * 8, st[i]);
      } else {
        if (c < C::CV) chunk_store_column<T>(Vt + (c * 8) * C::VTS + r, C::VTS, st[i]);
      }
    }
  };

  const int kend = min(p.S, p.q_off + q0 + BQ);  // keys beyond the tile's last query are masked
  load_tile(0);
  for (int k0 = 0; k0 < kend; k0 += BKEY) {
    store_tile();
    __syncthreads();
    if (k0 + BKEY < kend) load_tile(k0 + BKEY);

    if (k0 <= qa0 + 31) {                         // some key of the tile is visible to this wave
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          Frag<T> a = frag_load<T>(Ks + (mb * 32 + col) * C::KRS + ks * 16 + 8 * half);
          s[mb] = mma32(a, qf[ks], s[mb]);
        }
      }
      float pv[32];
      float mt = -INFINITY;
      const bool diag = (k0 + BKEY - 1 > qa0) || (k0 + BKEY > p.S);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          int key = k0 + mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          float x = s[mb][i] * p.scale_log2;
          if (diag && (key > qabs || key >= p.S)) x = -INFINITY;
          pv[mb * 16 + i] = x;
          mt = fmaxf(mt, x);
        }
      mt = wave_max32(mt);
      if (__any(mt > m_run + kLazyRescale)) {
        float m_new = fmaxf(m_run, mt);
        float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < DVP / 32; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
        m_run = m_new;
      }
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        pv[i] = (m_run == -INFINITY) ? 0.f : exp2f(pv[i] - m_run);
        ps += pv[i];
      }
      l_run += ps;
      if (p.keep_thr) {
        // dropout after the softmax: the normaliser keeps every weight, the value product
        // only the kept ones, scaled by 1 / (1 - p).  A lane's keys come in aligned runs of
        // four (keys 8 (i/4) + 4 half + i%4 of each 32-key block): one draw per run.
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int key4 = k0 + (r >> 2) * 32 + 8 * (r & 3) + 4 * half;
          const unsigned bits = dropout_keep4(p.seed, p.keep_thr, key4 >> 2, qabs, b * p.H + h);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[4 * r + e] = ((bits >> e) & 1u) ? pv[4 * r + e] * p.keep_scale : 0.f;
        }
      }
      Frag<T> pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pf[ks] = frag_from_f32<T>(pv + 8 * ks);
#pragma unroll
      for (int mb = 0; mb < DVP / 32; ++mb) {
        const T* base = Vt + (mb * 32 + col) * C::VTS + 4 * half;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          Frag<T> a = frag_load_2x4<T>(base + 16 * ks, base + 16 * ks + 8);
          acc[mb] = mma32(a, pf[ks], acc[mb]);
        }
      }
    }
    __syncthreads();
  }

  const float l_tot = wave_sum32(l_run);
  if (query >= p.T) return;
  const float inv = 1.f / l_tot;
  if (p.lse && half == 0) p.lse[((long long)b * p.H + h) * p.T + query] = m_run + log2f(l_tot);
  T* O = reinterpret_cast<T*>(p.o) + (((long long)b * p.T + query) * p.H + h) * p.dv;
#pragma unroll
  for (int mb = 0; mb < DVP / 32; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int d = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (d < p.dv) O[d] = from_f32<T>(acc[mb][i] * inv);
    }
}

template <typename T, int DQP, int DVP>
hipError_t launch_impl(const PrefillParams& p, hipStream_t s) {
  using C = PrefillCfg<T, DQP, DVP>;
  dim3 grid((p.T + BQ - 1) / BQ, p.H, p.B);
  hipLaunchKernelGGL((prefill_kernel<T, DQP, DVP>), grid, dim3(256), C::LDS, s, p);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(bool use_bf16, int dq, int dv, int* dq_pad, int* dv_pad) {
  if (dq <= 0 || dv <= 0) return false;
  if (use_bf16) {
    if (dq <= 64 && dv <= 64) { *dq_pad = 64; *dv_pad = 64; return true; }
    if (dq <= 128 && dv <= 128) { *dq_pad = 128; *dv_pad = 128; return true; }
    if (dq <= 192 && dv <= 128) { *dq_pad = 192; *dv_pad = 128; return true; }
    return false;
  }
  if (dq <= 16 && dv <= 32) { *dq_pad = 16; *dv_pad = 32; return true; }
  if (dq <= 64 && dv <= 64) { *dq_pad = 64; *dv_pad = 64; return true; }
  return false;
}

hipError_t launch_prefill(const PrefillParams& p, bool use_bf16, int dqp, int dvp, hipStream_t s) {
#define MLA_PRE(T, A, B_) \
  if (dqp == A && dvp == B_) return launch_impl<T, A, B_>(p, s);
  if (use_bf16) {
    MLA_PRE(bf16, 64, 64)
    MLA_PRE(bf16, 128, 128)
    MLA_PRE(bf16, 192, 128)
  } else {
    MLA_PRE(float, 16, 32)
    MLA_PRE(float, 64, 64)
  }
#undef MLA_PRE
  return hipErrorInvalidValue;
}

}  // namespace mla
