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

}  // namespace

hipError_t launch_cca_prep(const CcaPrepParams& p, bool use_bf16, hipStream_t s) {
  if (p.dh <= 0 || p.dh > kCcaMaxHeadDim || (p.dh & 1) || p.kseq > kCcaMaxKernel || p.kch > kCcaMaxKernel)
    return hipErrorInvalidValue;
  if ((TB + 256 / p.dh - 1) / (256 / p.dh) > kMaxTpt) return hipErrorInvalidValue;
  if (p.flash && (p.dqp < p.dh || p.S % 16 != 0)) return hipErrorInvalidValue;
  const PrepLds lay = prep_lds(p);
  const dim3 grid(cdiv(p.S, TB), p.Hq + p.Hkv, p.B);
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
