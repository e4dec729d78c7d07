// Split-context absorbed decode over the latent cache, plus the log-sum-exp combine.
//
// One decode step attends from one new token per sequence over rows 0..ctx_len[b] of the
// latent cache (the DSV2 page's cached path: the query at position p sees the cached
// rows < p + 1).  With W_UK folded into the query (q_lat = W_UK,h^T q_C,h) the score of
// head h against cached token j is  q_lat_h . c_j + q_R,h . k_R,j  and the head's
// output before W_UV is  z_h = sum_j softmax_j c_j  -- so the cache is read as stored,
// never up-projected.
//
// Work split: a workgroup owns (sequence b, latent block g, head tile, split of the
// context).  Its NW waves hold 32 heads each; every 32-token tile of the latent (plus
// rotary key) is staged once into LDS and consumed by all heads of the workgroup:
//   S^T[32 tokens x 32 heads] = C_tile[32 x (DL+DR)] . Q^T      (32x32x16 MFMA, K = DL+DR)
//   Z^T[DL x 32 heads]       += C_tile^T[DL x 32] . P^T[32 x 32] (32x32x16 MFMA, K = tokens)
// Each lane owns one head's column of S^T and Z^T, so the softmax row statistics and
// the rescale of Z are per-lane scalars (one exchange with the lane 32 apart).  The
// running maximum is only raised when a tile's maximum exceeds it by more than 2^8,
// which keeps the result exact while making the rescale of Z rare.
// The second product reads the latent token-contiguous, so staging writes a transposed
// copy of the latent part next to the row-major copy the first product reads.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int TT = 32;                 // tokens per tile
constexpr float kLazyRescale = 8.0f;   // log2 headroom before the running max is raised

template <typename T, int DL, int DR, int NW>
struct DecodeCfg {
  static constexpr int DQ = DL + DR;
  static constexpr int KS = DQ / 16;                 // k-steps of the score product
  static constexpr int RPAD = 16 / (int)sizeof(T);
  static constexpr int RS = DQ + RPAD;               // row-major tile stride (elements)
  static constexpr int CTS = TT + 4;                 // transposed tile stride (elements)
  static constexpr int CC = DQ / 8;                  // 8-element chunks per token row
  static constexpr int CBLK = (CC + 7) / 8;          // chunk-column blocks
  static constexpr int NBLK = (TT / 8) * CBLK;       // 8x8-chunk blocks per tile
  static constexpr int BPW = (NBLK + NW - 1) / NW;   // blocks per wave
  static constexpr size_t LDS = (size_t)TT * RS * sizeof(T) + (size_t)DL * CTS * sizeof(T);
  static_assert(DL % 32 == 0 && DR % 16 == 0, "padded widths");
};

template <typename T, int DL, int DR, int NW>
__global__ void __launch_bounds__(NW * 64) decode_kernel(DecodeParams p) {
  using C = DecodeCfg<T, DL, DR, NW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* R = reinterpret_cast<T*>(smem_raw);              // [TT][RS]   token-major
  T* CT = R + TT * C::RS;                             // [DL][CTS]  latent-column-major

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int split = blockIdx.x;
  const int g = blockIdx.y / p.head_tiles;
  const int ht = blockIdx.y - g * p.head_tiles;
  const int b = blockIdx.z;

  const int n_tok = decode_tokens(p, b);
  const int tok_begin = split * p.chunk;
  if (tok_begin >= n_tok) return;
  const int tok_end = min(n_tok, tok_begin + p.chunk);

  const int hloc = ht * (32 * NW) + wave * 32 + col;         // head within block g
  const bool head_ok = hloc < p.hpb;
  const int head = g * p.hpb + hloc;

  // ---- this lane's slice of Q^T (B operand), padded with zeros ----
  const T* ql = reinterpret_cast<const T*>(p.q_lat);
  const T* qr = reinterpret_cast<const T*>(p.q_rope);
  Frag<T> qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int d0 = ks * 16 + 8 * half;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int d = d0 + j;
      float x = 0.f;
      if (head_ok) {
        if (d < DL) {
          if (d < p.rb) x = to_f32(ql[((long long)b * p.H + head) * p.q_lat_hs + d]);
        } else if (d - DL < p.d_rope) {
          x = to_f32(qr[((long long)b * p.H + head) * p.q_rope_hs + (d - DL)]);
        }
      }
      v[j] = x;
    }
    qf[ks] = frag_from_f32<T>(v);
  }

  f32x16 acc[DL / 32];
#pragma unroll
  for (int mb = 0; mb < DL / 32; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const T* ckv = reinterpret_cast<const T*>(p.ckv);
  const T* kr = reinterpret_cast<const T*>(p.kr);
  const long long row0 = (long long)b * p.cache_bstride;

  Chunk<T> st[C::BPW];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
      int blk = wave + i * NW;
      int rblk = blk / C::CBLK, cblk = blk - rblk * C::CBLK;
      int r = rblk * 8 + (lane & 7);
      int c = cblk * 8 + (lane >> 3);
      int tok = t0 + r;
      chunk_zero<T>(st[i]);
      if (blk < C::NBLK && c < C::CC && tok < tok_end) {
        int d = c * 8;
        if (d < DL) {
          int nv = p.rb - d;
          if (nv > 0) {
            const T* src = ckv + (row0 + tok) * p.r_kv + (long long)g * p.rb + d;
            if (nv >= 8 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) chunk_load<T>(st[i], src);
            else chunk_load_partial<T>(st[i], src, nv < 8 ? nv : 8);
          }
        } else {
          int dr = d - DL;
          int nv = p.d_rope - dr;
          if (nv > 0) {
            const T* src = kr + (row0 + tok) * p.d_rope + dr;
            if (nv >= 8 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) chunk_load<T>(st[i], src);
            else chunk_load_partial<T>(st[i], src, nv < 8 ? nv : 8);
          }
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
      int blk = wave + i * NW;
      int rblk = blk / C::CBLK, cblk = blk - rblk * C::CBLK;
      int r = rblk * 8 + (lane & 7);
      int c = cblk * 8 + (lane >> 3);
      if (blk < C::NBLK && c < C::CC) {
        chunk_store<T>(R + r * C::RS + c * 8, st[i]);
        if (c * 8 < DL) chunk_store_column<T>(CT + (c * 8) * C::CTS + r, C::CTS, st[i]);
      }
    }
  };

  load_tile(tok_begin);
  for (int t0 = tok_begin; t0 < tok_end; t0 += TT) {
    store_tile();
    __syncthreads();
    if (t0 + TT < tok_end) load_tile(t0 + TT);

    // scores of 32 tokens x this wave's 32 heads
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      Frag<T> a = frag_load<T>(R + col * C::RS + ks * 16 + 8 * half);
      s = mma32(a, qf[ks], s);
    }
    float pv[16];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int tok = t0 + 8 * (i >> 2) + 4 * half + (i & 3);
      float x = (tok < tok_end) ? s[i] * p.scale_log2 : -INFINITY;
      pv[i] = x;
      mt = fmaxf(mt, x);
    }
    mt = wave_max32(mt);
    if (__any(mt > m_run + kLazyRescale)) {
      float m_new = fmaxf(m_run, mt);
      float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < DL / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
      m_run = m_new;
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pv[i] = exp2f(pv[i] - m_run);
      ps += pv[i];
    }
    l_run += ps;
    Frag<T> pf0 = frag_from_f32<T>(pv);
    Frag<T> pf1 = frag_from_f32<T>(pv + 8);
#pragma unroll
    for (int mb = 0; mb < DL / 32; ++mb) {
      const T* base = CT + (mb * 32 + col) * C::CTS + 4 * half;
      Frag<T> a0 = frag_load_2x4<T>(base, base + 8);
      acc[mb] = mma32(a0, pf0, acc[mb]);
      Frag<T> a1 = frag_load_2x4<T>(base + 16, base + 24);
      acc[mb] = mma32(a1, pf1, acc[mb]);
    }
    __syncthreads();
  }

  const float l_tot = wave_sum32(l_run);
  if (!head_ok) return;
  const long long pidx = ((long long)b * p.H + head) * p.nsplit + split;
  if (half == 0) {
    p.part_ml[pidx * 2 + 0] = m_run;
    p.part_ml[pidx * 2 + 1] = l_tot;
  }
  float* pz = p.part_z + pidx * DL;
#pragma unroll
  for (int mb = 0; mb < DL / 32; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c0 = mb * 32 + 8 * q + 4 * half;
      *reinterpret_cast<f32x4*>(pz + c0) =
          (f32x4){acc[mb][4 * q + 0], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]};
    }
}

// z[b][h] = sum_s 2^(m_s - M) z_s / sum_s 2^(m_s - M) l_s over the splits of sequence b
// (fp32 split results; the bf16 ones of the 128-head kernel go to combine_uv_kernel).  One 64-lane workgroup per (head, sequence); lane c owns CPT consecutive columns (vector
// loads), the split weights are formed once per split, and the split loop is unrolled so
// that several partial rows are in flight at once.
template <typename T, int DL>
__global__ void __launch_bounds__(64) combine_kernel(DecodeParams p) {
  constexpr int CPT = DL >= 64 ? DL / 64 : 1;
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int n_tok = decode_tokens(p, b);
  const int ns = p.sub * ((n_tok + p.chunk - 1) / p.chunk);   // partial rows written for b
  const long long base = ((long long)b * p.H + head) * p.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, p.part_ml[(base + s) * 2]);
  float Lsum = 0.f;
  for (int s = 0; s < ns; ++s) Lsum += exp2f(p.part_ml[(base + s) * 2] - M) * p.part_ml[(base + s) * 2 + 1];
  const float inv = 1.f / Lsum;
  const int c0 = threadIdx.x * CPT;
  if (c0 >= p.rb) return;
  float a[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) a[j] = 0.f;
  const float* zs = p.part_z + base * DL + c0;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float w = exp2f(p.part_ml[(base + s) * 2] - M);
    float v[CPT];
    if constexpr (CPT % 4 == 0) {
#pragma unroll
      for (int j = 0; j < CPT; j += 4) *reinterpret_cast<f32x4*>(v + j) = *reinterpret_cast<const f32x4*>(zs + (long long)s * DL + j);
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) v[j] = zs[(long long)s * DL + j];
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) a[j] += w * v[j];
  }
  T* z = reinterpret_cast<T*>(p.z) + ((long long)b * p.H + head) * p.rb + c0;
#pragma unroll
  for (int j = 0; j < CPT; ++j)
    if (c0 + j < p.rb) z[j] = from_f32<T>(a[j] * inv);
}

template <typename T, int DL>
hipError_t launch_combine_impl(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, DL>), dim3(p.H, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <typename T, int DL, int DR, int NW>
hipError_t launch_impl(const DecodeParams& p, hipStream_t s) {
  using C = DecodeCfg<T, DL, DR, NW>;
  dim3 grid(p.nsplit, p.L * p.head_tiles, p.B);
  hipLaunchKernelGGL((decode_kernel<T, DL, DR, NW>), grid, dim3(NW * 64), C::LDS, s, p);
  return hipGetLastError();
}

// Decode step only: the combine of the 128-head split kernel's bf16 partials fused with the
// per-head value up-projection o[b][h] = W_UV,h z[b][h] (W_UV,h = rows h*DV .. h*DV+DV-1 of
// w_uv, [DV][512]), so z never leaves the workgroup.  One workgroup per (head, 32 sequences):
//   1. wave w combines sequences 8w .. 8w+7 (lane: 8 consecutive latent columns; split
//      weights l_s 2^(m_s - M) / sum; the loads of all splits of four sequences are in
//      flight together) and leaves z in LDS as bf16 (the precision the separate combine
//      hands the product); the wave's weight rows for step 2 are loaded before all this;
//   2. O^T[DV x 32 sequences] = W_UV,h[DV x 512] . Z^T: wave w takes rows 32w .. 32w+31 with
//      32x32x16 MFMAs, A straight from global memory, B from LDS.  The contraction index is
//      relabelled (k-step ks, lane half hk <-> latent columns 256 hk + 8 ks ..) identically on
//      both operands, so every lane reads one contiguous 512-byte run of its weight row.
// UV = false: the combine alone (mla_decode_attention), z[b][h] written to p.z; the same
// workgroup shape, so that a wave has the partial rows of four sequences in flight at once.
template <int DV, bool UV = true>
__global__ void __launch_bounds__(64 * (DV / 32)) combine_uv_kernel(DecodeParams p, const bf16* __restrict__ w_uv,
                                                                    bf16* __restrict__ o) {
  constexpr int DL = 512, SEQ = 32, NWV = DV / 32, SPW = SEQ / NWV, LDZ = DL + 8, MAXS = 4;
  __shared__ __attribute__((aligned(16))) bf16 zs[UV ? SEQ * LDZ : 8];
  const int h = blockIdx.x, b0 = blockIdx.y * SEQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bf16* part = reinterpret_cast<const bf16*>(p.part_z);
  // this wave's W_UV,h rows go out first; their latency overlaps the combine
  const int col = lane & 31, hk = lane >> 5;
  bf16x8 af[UV ? 32 : 1];
  if constexpr (UV) {
    const bf16* wrow = w_uv + ((long long)h * DV + 32 * wave + col) * DL + 256 * hk;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) af[ks] = *reinterpret_cast<const bf16x8*>(wrow + 8 * ks);
  }

  // 1. combine.  Split weights first: thread (sequence t/8, lane t%8) scans splits t%8,
  // t%8 + 8, ..; the eight lanes of a sequence meet through lane shuffles.
  __shared__ float wts[SEQ][MAXS], smx[SEQ], sinv[SEQ];
  __shared__ int sns[SEQ];
  __shared__ long long sbase[SEQ];
  {
    const int sl = threadIdx.x >> 3, j = threadIdx.x & 7;
    const int b = b0 + sl;
    const int ns = b < p.B ? p.sub * ((decode_tokens(p, b) + p.chunk - 1) / p.chunk) : 0;
    const long long base = ((long long)min(b, p.B - 1) * p.H + h) * p.nsplit;
    float mx = -INFINITY;
    for (int s = j; s < ns; s += 8) mx = fmaxf(mx, p.part_ml[(base + s) * 2]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    float L = 0.f;
    for (int s = j; s < ns; s += 8) L += exp2f(p.part_ml[(base + s) * 2] - mx) * p.part_ml[(base + s) * 2 + 1];
    L += __shfl_xor(L, 1);
    L += __shfl_xor(L, 2);
    L += __shfl_xor(L, 4);
    const float inv = ns > 0 ? 1.f / L : 0.f;
    if (j < MAXS) wts[sl][j] = j < ns ? exp2f(p.part_ml[(base + j) * 2] - mx) * p.part_ml[(base + j) * 2 + 1] * inv : 0.f;
    if (j == 0) {
      smx[sl] = mx;
      sinv[sl] = inv;
      sns[sl] = ns;
      sbase[sl] = base;
    }
  }
  __syncthreads();
  long long rowb[SPW];
  int nsb[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    rowb[i] = sbase[wave * SPW + i];
    nsb[i] = sns[wave * SPW + i];
  }
  constexpr int SH = SPW / 2;                             // sequences per half
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float a[SH][8];
#pragma unroll
    for (int i = 0; i < SH; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[i][e] = 0.f;
    for (int s0 = 0; s0 < p.nsplit; s0 += MAXS) {
      bf16x8 y[SH][MAXS];
#pragma unroll
      for (int i = 0; i < SH; ++i)
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
          const int ii = hh * SH + i;
          const int sc = min(s0 + s, max(nsb[ii] - 1, 0));  // past the last split: a valid row, weight 0
          y[i][s] = *reinterpret_cast<const bf16x8*>(part + (rowb[ii] + sc) * DL + 8 * lane);
        }
#pragma unroll
      for (int i = 0; i < SH; ++i)
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
          const int ii = hh * SH + i, sl = wave * SPW + ii;
          float w = wts[sl][s];
          if (s0 > 0) {                                   // splits beyond the first MAXS
            const int sg = s0 + s;
            w = sg < nsb[ii] ? exp2f(p.part_ml[(rowb[ii] + sg) * 2] - smx[sl]) * p.part_ml[(rowb[ii] + sg) * 2 + 1] * sinv[sl] : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) a[i][e] += w * (float)y[i][s][e];
        }
    }
#pragma unroll
    for (int i = 0; i < SH; ++i) {
      bf16x8 zz;
#pragma unroll
      for (int e = 0; e < 8; ++e) zz[e] = (bf16)a[i][e];
      if constexpr (UV) {
        *reinterpret_cast<bf16x8*>(zs + (wave * SPW + hh * SH + i) * LDZ + 8 * lane) = zz;
      } else {
        const int b = b0 + wave * SPW + hh * SH + i;
        if (b < p.B) *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(p.z) + ((long long)b * p.H + h) * DL + 8 * lane) = zz;
      }
    }
  }
  if constexpr (!UV) return;
  __syncthreads();

  // 2. O^T = W_UV,h . Z^T
  const bf16* zrow = zs + col * LDZ + 256 * hk;
  f32x16 c0 = f32x16{}, c1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 32; ks += 2) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], *reinterpret_cast<const bf16x8*>(zrow + 8 * ks), c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks + 1], *reinterpret_cast<const bf16x8*>(zrow + 8 * ks + 8), c1, 0, 0, 0);
  }
  // lane: sequence b0 + col, rows 32 wave + 8 q + 4 hk + 0..3
  const int b = b0 + col;
  if (b >= p.B) return;
  bf16* orow = o + ((long long)b * p.H + h) * DV + 32 * wave + 4 * hk;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<bf16x4*>(orow + 8 * q) =
        (bf16x4){(bf16)(c0[4 * q] + c1[4 * q]), (bf16)(c0[4 * q + 1] + c1[4 * q + 1]),
                 (bf16)(c0[4 * q + 2] + c1[4 * q + 2]), (bf16)(c0[4 * q + 3] + c1[4 * q + 3])};
}

}  // namespace

bool decode_supported(bool use_bf16, int rb, int d_rope, int hpb, int* dl_pad, int* dr_pad, int* nw) {
  if (use_bf16) {
    if (rb <= 0 || rb > 512 || d_rope < 0 || d_rope > 64) return false;
    *dl_pad = rb <= 128 ? 128 : 512;
    *dr_pad = d_rope == 0 ? 0 : 64;
    *nw = hpb <= 32 ? 1 : 4;
    return true;
  }
  if (rb <= 0 || rb > 128 || d_rope < 0 || d_rope > 64) return false;
  *dl_pad = rb <= 32 ? 32 : 128;
  *dr_pad = d_rope == 0 ? 0 : (d_rope <= 16 ? 16 : 64);
  *nw = 1;
  return true;
}

hipError_t launch_combine(const DecodeParams& p, bool use_bf16, int dl, hipStream_t s) {
  if (use_bf16) {
    if (p.part_bf16) {                     // bf16 split results: latent 512 only
      if (dl != 512 || p.rb != 512) return hipErrorInvalidValue;
      hipLaunchKernelGGL((combine_uv_kernel<128, false>), dim3(p.H, (p.B + 31) / 32), dim3(256), 0, s, p,
                         nullptr, nullptr);
      return hipGetLastError();
    }
    if (dl == 512) return launch_combine_impl<bf16, 512>(p, s);
    if (dl == 128) return launch_combine_impl<bf16, 128>(p, s);
  } else {
    if (dl == 32) return launch_combine_impl<float, 32>(p, s);
    if (dl == 128) return launch_combine_impl<float, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

bool combine_uv_supported(const DecodeParams& p, int d_v, const void* w_uv) {
  return p.part_bf16 && p.rb == 512 && p.r_kv == 512 && d_v == 128 &&
         (reinterpret_cast<uintptr_t>(w_uv) & 15) == 0;
}

hipError_t launch_combine_uv(const DecodeParams& p, int d_v, const void* w_uv, void* o, hipStream_t s) {
  if (!combine_uv_supported(p, d_v, w_uv)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_uv_kernel<128>, dim3(p.H, (p.B + 31) / 32), dim3(256), 0, s, p,
                     reinterpret_cast<const bf16*>(w_uv), reinterpret_cast<bf16*>(o));
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, bool use_bf16, int dl, int dr, int nw, hipStream_t s) {
#define MLA_DEC(T, DL_, DR_, NW_) \
  if (dl == DL_ && dr == DR_ && nw == NW_) return launch_impl<T, DL_, DR_, NW_>(p, s);
  if (use_bf16) {
    MLA_DEC(bf16, 512, 64, 4)
    MLA_DEC(bf16, 512, 0, 4)
    MLA_DEC(bf16, 128, 0, 1)
    MLA_DEC(bf16, 128, 64, 1)
    MLA_DEC(bf16, 512, 0, 1)
    MLA_DEC(bf16, 512, 64, 1)
    MLA_DEC(bf16, 128, 0, 4)
    MLA_DEC(bf16, 128, 64, 4)
  } else {
    MLA_DEC(float, 32, 0, 1)
    MLA_DEC(float, 32, 16, 1)
    MLA_DEC(float, 32, 64, 1)
    MLA_DEC(float, 128, 0, 1)
    MLA_DEC(float, 128, 16, 1)
    MLA_DEC(float, 128, 64, 1)
  }
#undef MLA_DEC
  return hipErrorInvalidValue;
}

}  // namespace mla
