// Compressed convolutional attention (CCA / CCGQA): the steps between the packed q / k
// down-projection and attention, [CCA page] ``CCAAttention.forward`` and
// ``CCGQAAttention.forward`` (decoder mode):
//   * the causal convolutions of ``_apply_causal_convs``: a depth-wise one along the sequence
//     (kernel kseq), then one grouped by head (kernel kch, mixing the d_h channels of a head);
//     both left-padded with zeros, no bias;
//   * q-k-mean: the mean of the pre-convolution query and key added after the convolutions
//     (CCGQA: a query head pairs with its group's key head, a key head takes the group mean);
//   * the QK L2-norm (each head vector scaled to length sqrt(d_h), norm clamped at 1e-6) and
//     the key temperature exp(beta) on the keys;
//   * half-split RoPE in the latent at positions 0..S-1;
//   * value shift: value channels of the first half come from the current token's projection,
//     those of the second half from the previous token's (zero at t = 0).
//
// One workgroup per (sequence, 64-token block, head of the packed tensor), 256 threads:
//   * the head's packed columns for the block and its convolution halo are staged in LDS
//     (fp32), then the depth-wise sequence convolution runs there;
//   * the grouped channel convolution is a small contraction over (input channel, tap): its
//     weights go through LDS in chunks, transposed so that the lanes of a wave (consecutive
//     output channels) read consecutive words, and each thread keeps the accumulators of
//     several tokens of one output channel in registers, so one weight read serves them all;
//   * q-k-mean, the L2 norm, the key temperature and the rotation follow; queries, keys and
//     values leave in the layer's element type in [B*S][heads][d_h] rows for attention.
// The work is a few hundred flops per output, a small part of the layer: the kernel is bound
// by its reads of the fp32 projections and its writes of q, k and v.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int TB = 64;                 // tokens per workgroup
constexpr int kMaxTpt = 32;            // tokens per thread in the channel convolution (d_h <= 128)
constexpr int kWChunk = 3584;          // channel-convolution weights per LDS round (floats)
constexpr int kUnroll = 8;             // global loads in flight per thread in the staging loops

struct PrepLds {
  int R, R1, cc, wfl;                  // staged rows, sequence-conv rows, channels per weight chunk
  int wsl;                             // sequence-convolution weights (floats)
  int a0rows;                          // rows of the sequence-convolution output region
  int a0fl;                            // floats of that region
  size_t bytes;
};

PrepLds prep_lds(const CcaPrepParams& p) {
  PrepLds l;
  const int h0 = p.layers >= 1 ? p.kseq - 1 : 0, h1 = p.layers >= 2 ? p.kch - 1 : 0;
  l.R = TB + h0 + h1;
  l.R1 = TB + h1;
  l.cc = 0;
  l.wfl = 0;
  if (p.layers >= 2) {
    l.cc = kWChunk / (p.kch * p.dh);
    if (l.cc < 1) l.cc = 1;
    if (l.cc > p.dh) l.cc = p.dh;
    // + room for the unguarded tap-weight reads past the chunk (taps kch .. kCcaMaxKernel - 1
    // of its last channel, never used)
    l.wfl = l.cc * p.kch * p.dh + (kCcaMaxKernel - 1) * p.dh;
  }
  l.wsl = p.layers >= 1 ? p.dh * p.kseq : 0;
  // u, a0, the two weight regions, the row scales and the staged values ([TB][dh + 1])
  l.a0rows = TB + kCcaMaxKernel - 1;   // room for the unguarded window reads (rows >= R1 unused)
  // the a0 region also holds the staged value rows ([TB][dh + 1]) once the convolutions are done
  l.a0fl = l.a0rows * p.dh > TB * (p.dh + 1) ? l.a0rows * p.dh : TB * (p.dh + 1);
  l.bytes = ((size_t)l.R * p.dh + (size_t)l.a0fl + l.wfl + l.wsl + TB) * sizeof(float);
  return l;
}

// The steps after the convolutions and the q-k-mean, shared by both kernels: the key head's
// value rows staged in vs ([TB][dh + 1], shifted by one token in the second half of the value
// channels), the per-row L2 norm of o ([TB][dh]) with the key temperature, the half-split
// rotation, and the stores of q / k / v.  Every thread of the workgroup calls it; o is complete
// and vs free when it is called.
template <typename T>
__device__ __forceinline__ void cca_finish(const CcaPrepParams& p, float* o, float* vs, float* rscale, int dh,
                                           int t0, int g, int b, int tid) {
  const bool is_q = g < p.Hq;
  const int Lkv = p.Hkv * dh;
  // the key head's value rows of the block, shifted by one token in the second half of the
  // value channels (read along the channels; stored below)
  if (!is_q) {
    const int j = g - p.Hq;
    for (int e0 = tid; e0 < TB * dh; e0 += kUnroll * 256) {
      float v[kUnroll];
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int e = e0 + 256 * k;
        const int r = e / dh, c = e - r * dh;
        const int t = t0 + r, ch = j * dh + c;
        const int ts = (p.value_shift && ch >= Lkv / 2) ? t - 1 : t;
        v[k] = (e < TB * dh && t < p.S && ts >= 0) ? p.V[((long long)b * p.S + ts) * Lkv + ch] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int e = e0 + 256 * k;
        const int r = e / dh, c = e - r * dh;
        if (e < TB * dh) vs[r * (dh + 1) + c] = v[k];
      }
    }
  }
  __syncthreads();

  // per-row L2 norm over the head's d_h channels (4 threads per row)
  {
    const int r = tid >> 2, l = tid & 3;
    float ss = 0.f;
    for (int c = l; c < dh; c += 4) ss = __builtin_fmaf(o[r * dh + c], o[r * dh + c], ss);
    ss += __shfl_xor(ss, 2, 4);
    ss += __shfl_xor(ss, 1, 4);
    if (l == 0) rscale[r] = p.sqrt_dh / fmaxf(sqrtf(ss), 1e-6f) * (is_q ? 1.f : p.key_gain);
  }
  __syncthreads();

  // half-split rotation at the token's position, then the store
  const int half = dh >> 1;
  T* dst = is_q ? reinterpret_cast<T*>(p.q) : reinterpret_cast<T*>(p.k);
  const int nh = is_q ? p.Hq : p.Hkv, hh = is_q ? g : g - p.Hq;
  const int dw = p.flash ? p.dqp : dh;                  // stored features per head row
  auto qk_row = [&](int t) -> T* {
    if (p.flash && !is_q) return dst + (((long long)b * p.Hkv + hh) * p.S + t) * dw;   // head-major keys
    return dst + (((long long)b * p.S + t) * nh + hh) * dw;
  };
  for (int e = tid; e < TB * half; e += 256) {
    const int r = e / half, jj = e - r * half;
    const int t = t0 + r;
    if (t >= p.S) continue;
    const float x1 = o[r * dh + jj] * rscale[r], x2 = o[r * dh + jj + half] * rscale[r];
    float sn, cs;
    rope_sincos(t, p.rope.hi[jj], p.rope.lo[jj], &sn, &cs);
    T* row = qk_row(t);
    row[jj] = from_f32<T>(x1 * cs - x2 * sn);
    row[jj + half] = from_f32<T>(x1 * sn + x2 * cs);
  }
  if (dw > dh) {                                        // zero padding of the feature rows
    const int pad = dw - dh;
    for (int e = tid; e < TB * pad; e += 256) {
      const int r = e / pad, c = dh + e - r * pad;
      if (t0 + r < p.S) qk_row(t0 + r)[c] = from_f32<T>(0.f);
    }
  }

  // the key head's values (staged above)
  if (!is_q) {
    const int j = g - p.Hq;
    T* vdst = reinterpret_cast<T*>(p.v);
    if (p.flash) {
      // transposed per head: feature row c holds the tokens, each 16-group stored in the
      // order 0-3, 8-11, 4-7, 12-15 (token slots 4-7 and 8-11 swapped); consecutive threads
      // take consecutive tokens of one row (the staged rows' padded stride keeps the column
      // reads on distinct banks)
      for (int e = tid; e < TB * dw; e += 256) {
        const int c = e / TB, r = e - c * TB;
        const int t = t0 + r;
        if (t >= p.S) continue;
        const float val = c < dh ? vs[r * (dh + 1) + c] : 0.f;
        const int t16 = t & 15;
        const int slot = (t & ~15) + ((t16 >= 4 && t16 < 8) ? t16 + 4 : (t16 >= 8 && t16 < 12) ? t16 - 4 : t16);
        vdst[(((long long)b * p.Hkv + j) * dw + c) * p.S + slot] = from_f32<T>(val);
      }
    } else {
      for (int e = tid; e < TB * dh; e += 256) {
        const int r = e / dh, c = e - r * dh;
        const int t = t0 + r;
        if (t >= p.S) continue;
        vdst[(((long long)b * p.S + t) * p.Hkv + j) * dh + c] = from_f32<T>(vs[r * (dh + 1) + c]);
      }
    }
  }
}

// DH: the head width as a compile-time constant (32, 64, 128), or 0 for any other width.
template <typename T, int DH>
__global__ void __launch_bounds__(256) cca_prep_kernel(CcaPrepParams p, PrepLds lay) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int dh = DH ? DH : p.dh, t0 = blockIdx.x * TB, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const bool is_q = g < p.Hq;
  const int Lq = p.Hq * dh, Lkv = p.Hkv * dh, Cp = Lq + Lkv;
  const int gs = p.Hq / p.Hkv;
  const int c0 = is_q ? g * dh : Lq + (g - p.Hq) * dh;   // first packed channel of this head
  const int h0 = p.layers >= 1 ? p.kseq - 1 : 0;          // halo of the sequence convolution
  const int h1 = p.layers >= 2 ? p.kch - 1 : 0;           // halo of the channel convolution
  const float* P = p.P + (long long)b * p.S * Cp;
  const T* wseq = reinterpret_cast<const T*>(p.conv_seq);
  const T* wch = reinterpret_cast<const T*>(p.conv_ch);
  const int R = lay.R, R1 = lay.R1;
  float* u = sm;                        // [R][dh]   packed rows t0 - h0 - h1 ..
  float* a0 = u + R * dh;               // [R1][dh]  after the sequence convolution, from t0 - h1
  float* wl = a0 + lay.a0fl;            // [cc][kch][dh] channel-convolution weight chunk
  float* wsq = wl + lay.wfl;            // [dh][kseq] sequence-convolution weights of the head
  float* rscale = wsq + lay.wsl;        // [TB]
  float* vs = a0;                       // [TB][dh + 1] value rows, once a0 is no longer read
  float* o = u;                         // [TB][dh]  reuses u once the convolutions are done

  // packed rows t0 - h0 - h1 .. t0 + TB - 1 (zero before the sequence and past its end), and
  // the head's sequence-convolution weights (one contiguous run); kUnroll loads in flight
  for (int e0 = tid; e0 < R * dh; e0 += kUnroll * 256) {
    float v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int e = e0 + 256 * k;
      const int i = e / dh, c = e - i * dh;
      const int t = t0 - h0 - h1 + i;
      v[k] = (e < R * dh && t >= 0 && t < p.S) ? P[(long long)t * Cp + c0 + c] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      if (e0 + 256 * k < R * dh) u[e0 + 256 * k] = v[k];
  }
  for (int e = tid; e < lay.wsl; e += 256) wsq[e] = to_f32(wseq[(long long)c0 * p.kseq + e]);
  __syncthreads();

  // depth-wise sequence convolution: a0 row i is token t0 - h1 + i; a row before the
  // sequence stays zero (the channel convolution pads the sequence convolution's output)
  for (int e = tid; e < R1 * dh; e += 256) {
    const int i = e / dh, c = e - i * dh;
    float acc = 0.f;
    if (t0 - h1 + i >= 0) {
      if (p.layers >= 1) {
        for (int j = 0; j < p.kseq; ++j) acc = __builtin_fmaf(wsq[c * p.kseq + j], u[(i + j) * dh + c], acc);
      } else {
        acc = u[i * dh + c];
      }
    }
    a0[i * dh + c] = acc;
  }

  // channel convolution grouped by head: thread (output channel oc, token group tg) keeps
  // the tokens rbeg .. rbeg + tpt - 1 of its channel.  With a compile-time width the token
  // count is exact (TB d_h / 256) and, per input channel, the thread loads the window of
  // tpt + kch - 1 rows once and reuses it for every tap.
  constexpr int TPT = DH ? TB * DH / 256 : kMaxTpt;
  const int ntg = 256 / dh, oc = tid % dh, tg = tid / dh;
  const bool act = tg < ntg;
  const int tpt = DH ? TPT : (TB + ntg - 1) / ntg;
  const int rbeg = tg * tpt;
  float acc[TPT];
#pragma unroll
  for (int r = 0; r < TPT; ++r) acc[r] = 0.f;
  if (p.layers >= 2) {
    const int kch = p.kch;
    for (int cb = 0; cb < dh; cb += lay.cc) {
      const int cn = min(lay.cc, dh - cb);
      __syncthreads();                  // a0 complete / the previous chunk consumed
      // wl[(ci kch + j) dh + oc'] = conv_ch[c0 + oc'][cb + ci][j]: each output channel's
      // weights of the chunk are one contiguous run in memory
      const int nw = cn * kch * dh;
      for (int e0 = tid; e0 < nw; e0 += kUnroll * 256) {
        float v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
          const int e = e0 + 256 * k;
          const int ocp = e / (cn * kch), rem = e - ocp * (cn * kch);
          v[k] = e < nw ? to_f32(wch[((long long)(c0 + ocp) * dh + cb) * kch + rem]) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
          const int e = e0 + 256 * k;
          const int ocp = e / (cn * kch), rem = e - ocp * (cn * kch);
          if (e < nw) wl[rem * dh + ocp] = v[k];
        }
      }
      __syncthreads();
      if (act) {
        if constexpr (DH != 0) {
          for (int ci = 0; ci < cn; ++ci) {
            const float* col = a0 + rbeg * dh + cb + ci;
            // rows rbeg .. rbeg + TPT + kCcaMaxKernel - 2 < a0rows: read without a guard (a
            // guarded read becomes a branch and a wait per row); rows past R1 are never used
            float win[TPT + kCcaMaxKernel - 1];
#pragma unroll
            for (int i = 0; i < TPT + kCcaMaxKernel - 1; ++i) win[i] = col[i * DH];
            // the taps' weights, also unguarded: words past the chunk (taps >= kch of its last
            // channel) fall in the slack at the end of the wl region
            float wv[kCcaMaxKernel];
#pragma unroll
            for (int j = 0; j < kCcaMaxKernel; ++j) wv[j] = wl[(ci * kch + j) * DH + oc];
            // (keeps the reads here, ahead of the taps' branches, instead of one read and
            // one wait inside each)
#pragma unroll
            for (int j = 0; j < kCcaMaxKernel; ++j) asm volatile("" ::"v"(wv[j]));
#pragma unroll
            for (int j = 0; j < kCcaMaxKernel; ++j) {
              if (j < kch) {
#pragma unroll
                for (int r = 0; r < TPT; ++r) acc[r] = __builtin_fmaf(wv[j], win[r + j], acc[r]);
              }
            }
          }
        } else {
          for (int ci = 0; ci < cn; ++ci) {
            for (int j = 0; j < kch; ++j) {
              const float w = wl[(ci * kch + j) * dh + oc];
              const float* col = a0 + (rbeg + j) * dh + cb + ci;
#pragma unroll
              for (int r = 0; r < TPT; ++r)
                if (r < tpt && rbeg + r < TB) acc[r] = __builtin_fmaf(w, col[r * dh], acc[r]);
            }
          }
        }
      }
    }
  } else {
    __syncthreads();
    if (act) {
#pragma unroll
      for (int r = 0; r < TPT; ++r)
        if (r < tpt && rbeg + r < TB) acc[r] = a0[(rbeg + r) * dh + oc];
    }
  }

  // q-k-mean of the pre-convolution values (the head's own are in u; its partner heads'
  // come from the packed projections)
  if (act && p.qk_mean) {
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int t = t0 + rbeg + r;
      if (r < tpt && rbeg + r < TB && t < p.S) {
        const float own = u[(rbeg + r + h0 + h1) * dh + oc];
        const float* row = P + (long long)t * Cp;
        if (is_q) {
          acc[r] += 0.5f * (own + row[Lq + (g / gs) * dh + oc]);
        } else {
          const int j = g - p.Hq;
          float m = 0.f;
          for (int hq = j * gs; hq < (j + 1) * gs; ++hq) m += row[hq * dh + oc];
          acc[r] += 0.5f * (m / (float)gs + own);
        }
      }
    }
  }
  __syncthreads();                      // every read of u and a0 is done: o and vs take their place
  if (act) {
#pragma unroll
    for (int r = 0; r < TPT; ++r)
      if (r < tpt && rbeg + r < TB) o[(rbeg + r) * dh + oc] = acc[r];
  }
  cca_finish<T>(p, o, vs, rscale, dh, t0, g, b, tid);
}

// MFMA form of the grouped channel convolution for bf16 layers with both convolutions and a
// head width of 32, 64 or 128: for each tap j the contraction over input channels is a
// [64 tokens x d_h] x [d_h x d_h] product, A_j[t][c] = a0[t + j][c] (the sequence
// convolution's output, shifted by j rows) and B_j[c][oc] = w[oc][c][j]; a0 is kept in LDS
// in bf16 and the tap's weights are staged [oc][c], both read with plain 16-byte operand
// reads (32x32x16 MFMA, fp32 accumulation).  The other steps are those of cca_prep_kernel.
struct PrepLdsM {
  int R, R1, ald, wld;                 // staged rows, conv rows, LDS strides of a0 and a tap (bf16)
  size_t u_fl, a0_bytes, w_bytes, o_fl;
  size_t bytes;
};

PrepLdsM prep_lds_mfma(const CcaPrepParams& p) {
  PrepLdsM l;
  const int h0 = p.kseq - 1, h1 = p.kch - 1;
  l.R = TB + h0 + h1;
  l.R1 = TB + h1;
  l.ald = p.dh + 8;
  l.wld = p.dh + 8;
  // u holds the staged rows, later the value rows ([TB][dh + 1])
  l.u_fl = (size_t)l.R * p.dh > (size_t)TB * (p.dh + 1) ? (size_t)l.R * p.dh : (size_t)TB * (p.dh + 1);
  l.a0_bytes = ((size_t)(TB + kCcaMaxKernel - 1) * l.ald * 2 + 15) / 16 * 16;
  l.w_bytes = ((size_t)p.dh * l.wld * 2 + 15) / 16 * 16;
  l.o_fl = (size_t)TB * p.dh;
  l.bytes = l.u_fl * 4 + l.a0_bytes + l.w_bytes + l.o_fl * 4 + (size_t)p.dh * p.kseq * 4 + TB * 4;
  return l;
}

template <int DH>
__global__ void __launch_bounds__(256) cca_prep_mfma_kernel(CcaPrepParams p, PrepLdsM lay) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int dh = DH;
  const int t0 = blockIdx.x * TB, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const bool is_q = g < p.Hq;
  const int Lq = p.Hq * dh, Lkv = p.Hkv * dh, Cp = Lq + Lkv;
  const int gs = p.Hq / p.Hkv;
  const int c0 = is_q ? g * dh : Lq + (g - p.Hq) * dh;
  const int kseq = p.kseq, kch = p.kch, h0 = kseq - 1, h1 = kch - 1;
  const float* P = p.P + (long long)b * p.S * Cp;
  const bf16* wseq = reinterpret_cast<const bf16*>(p.conv_seq);
  const bf16* wch = reinterpret_cast<const bf16*>(p.conv_ch);
  const int R = lay.R, R1 = lay.R1, ALD = lay.ald, WLD = lay.wld;
  float* u = sm;                                                           // [R][dh], later vs
  bf16* a0b = reinterpret_cast<bf16*>(u + lay.u_fl);                       // [TB + 7][ALD]
  bf16* wt = reinterpret_cast<bf16*>(reinterpret_cast<char*>(a0b) + lay.a0_bytes);   // [dh][WLD]
  float* o = reinterpret_cast<float*>(reinterpret_cast<char*>(wt) + lay.w_bytes);    // [TB][dh]
  float* wsq = o + lay.o_fl;                                               // [dh][kseq]
  float* rscale = wsq + dh * kseq;                                         // [TB]

  // packed rows t0 - h0 - h1 .. t0 + TB - 1 and the head's sequence-convolution weights
  for (int e0 = tid; e0 < R * dh; e0 += kUnroll * 256) {
    float v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int e = e0 + 256 * k;
      const int i = e / dh, c = e - i * dh;
      const int t = t0 - h0 - h1 + i;
      v[k] = (e < R * dh && t >= 0 && t < p.S) ? P[(long long)t * Cp + c0 + c] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      if (e0 + 256 * k < R * dh) u[e0 + 256 * k] = v[k];
  }
  for (int e = tid; e < dh * kseq; e += 256) wsq[e] = (float)wseq[(long long)c0 * kseq + e];
  __syncthreads();

  // depth-wise sequence convolution into a0b (bf16): row i is token t0 - h1 + i, zero before
  // the sequence
  for (int e = tid; e < R1 * dh; e += 256) {
    const int i = e / dh, c = e - i * dh;
    float acc = 0.f;
    if (t0 - h1 + i >= 0)
      for (int j = 0; j < kseq; ++j) acc = __builtin_fmaf(wsq[c * kseq + j], u[(i + j) * dh + c], acc);
    a0b[i * ALD + c] = (bf16)acc;
  }

  // grouped channel convolution: wave w takes output blocks w and w + 4 of the 2 x dh / 32
  // blocks of 32 tokens x 32 channels
  constexpr int NB = 2 * (dh / 32), BPW = (NB + 3) / 4;
  f32x16 acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) acc[i] = f32x16{};
  for (int j = 0; j < kch; ++j) {
    __syncthreads();                  // a0b complete / the previous tap's weights consumed
    // tap j's weights: wt[oc][c] = w[c0 + oc][c][j] (dh^2 / 256 loads per thread, all in flight)
    {
      constexpr int NWE = dh * dh / 256;
      bf16 wv[NWE];
#pragma unroll
      for (int k = 0; k < NWE; ++k) {
        const int e = tid + 256 * k, oc = e / dh, c = e - oc * dh;
        wv[k] = wch[((long long)(c0 + oc) * dh + c) * kch + j];
      }
#pragma unroll
      for (int k = 0; k < NWE; ++k) {
        const int e = tid + 256 * k, oc = e / dh, c = e - oc * dh;
        wt[oc * WLD + c] = wv[k];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + 4 * i;
      if (blk < NB) {
        const int mb = blk & 1, nb = blk >> 1;
#pragma unroll
        for (int ks = 0; ks < dh / 16; ++ks) {
          const Frag<bf16> fa = frag_load(a0b + (32 * mb + col + j) * ALD + 16 * ks + 8 * half);
          const Frag<bf16> fb = frag_load(wt + (32 * nb + col) * WLD + 16 * ks + 8 * half);
          acc[i] = mma32(fa, fb, acc[i]);
        }
      }
    }
  }
  // o[t][oc]: lane column oc = 32 nb + col, rows t = 32 mb + 8 (e / 4) + 4 half + e % 4
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + 4 * i;
    if (blk < NB) {
      const int mb = blk & 1, nb = blk >> 1;
#pragma unroll
      for (int e = 0; e < 16; ++e) o[(32 * mb + 8 * (e >> 2) + 4 * half + (e & 3)) * dh + 32 * nb + col] = acc[i][e];
    }
  }
  __syncthreads();

  // q-k-mean of the pre-convolution values (the head's own are in u; its partner heads'
  // come from the packed projections)
  if (p.qk_mean) {
    // partner values loaded kUnroll elements at a time (all in flight), then added
    const int jh = g - p.Hq;
    for (int e0 = tid; e0 < TB * dh; e0 += kUnroll * 256) {
      float m[kUnroll];
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int e = e0 + 256 * k, r = e / dh, c = e - r * dh, t = t0 + r;
        m[k] = 0.f;
        if (e < TB * dh && t < p.S) {
          const float* row = P + (long long)t * Cp;
          if (is_q) {
            m[k] = row[Lq + (g / gs) * dh + c];
          } else {
            for (int hq = jh * gs; hq < (jh + 1) * gs; ++hq) m[k] += row[hq * dh + c];
            m[k] /= (float)gs;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int e = e0 + 256 * k, r = e / dh, c = e - r * dh;
        if (e < TB * dh && t0 + r < p.S) o[e] += 0.5f * (m[k] + u[(r + h0 + h1) * dh + c]);
      }
    }
  }
  __syncthreads();                    // u is free: the value rows take its place
  cca_finish<bf16>(p, o, u, rscale, dh, t0, g, b, tid);
}

}  // namespace

hipError_t launch_cca_prep(const CcaPrepParams& p, bool use_bf16, hipStream_t s) {
  if (p.dh <= 0 || p.dh > kCcaMaxHeadDim || (p.dh & 1) || p.kseq > kCcaMaxKernel || p.kch > kCcaMaxKernel)
    return hipErrorInvalidValue;
  if ((TB + 256 / p.dh - 1) / (256 / p.dh) > kMaxTpt) return hipErrorInvalidValue;
  if (p.flash && (p.dqp < p.dh || p.S % 16 != 0)) return hipErrorInvalidValue;
  const PrepLds lay = prep_lds(p);
  const dim3 grid(cdiv(p.S, TB), p.Hq + p.Hkv, p.B);
  if (use_bf16 && p.layers == 2 && (p.dh == 32 || p.dh == 64 || p.dh == 128)) {
    const PrepLdsM lm = prep_lds_mfma(p);
    if (p.dh == 32) hipLaunchKernelGGL(cca_prep_mfma_kernel<32>, grid, dim3(256), lm.bytes, s, p, lm);
    else if (p.dh == 64) hipLaunchKernelGGL(cca_prep_mfma_kernel<64>, grid, dim3(256), lm.bytes, s, p, lm);
    else hipLaunchKernelGGL(cca_prep_mfma_kernel<128>, grid, dim3(256), lm.bytes, s, p, lm);
    return hipGetLastError();
  }
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), lay.bytes, s, p, lay); };
  if (use_bf16) {
    if (p.dh == 32) go(cca_prep_kernel<bf16, 32>);
    else if (p.dh == 64) go(cca_prep_kernel<bf16, 64>);
    else if (p.dh == 128) go(cca_prep_kernel<bf16, 128>);
    else go(cca_prep_kernel<bf16, 0>);
  } else {
    if (p.dh == 32) go(cca_prep_kernel<float, 32>);
    else if (p.dh == 64) go(cca_prep_kernel<float, 64>);
    else go(cca_prep_kernel<float, 0>);
  }
  return hipGetLastError();
}

}  // namespace mla
