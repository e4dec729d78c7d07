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
// One workgroup per (sequence, 16-token block, head of the packed tensor): the packed
// columns of that head for the block and its convolution halo are staged in LDS (fp32); the
// two convolutions, the mean, the norm and the rotation run there; queries, keys and values
// leave in the layer's element type in [B*S][heads][d_h] rows for the attention kernel.
// The work is a few hundred flops per output: a small fraction of the layer.
#include "common.h"
#include "internal.h"

namespace mla {

namespace {

constexpr int TB = 16;                                    // tokens per workgroup
constexpr int MAXR = TB + 2 * (kCcaMaxKernel - 1);        // staged rows (block + both halos)

template <typename T>
__global__ void __launch_bounds__(256) cca_prep_kernel(CcaPrepParams p) {
  __shared__ float u[MAXR * kCcaMaxHeadDim];              // packed rows of this head
  __shared__ float a0[(TB + kCcaMaxKernel - 1) * kCcaMaxHeadDim];   // after the sequence conv
  __shared__ float o[TB * kCcaMaxHeadDim];                // after the channel conv and the mean
  __shared__ float rscale[TB];

  const int dh = p.dh, t0 = blockIdx.x * TB, g = blockIdx.y, b = blockIdx.z;
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

  // packed rows t0 - h0 - h1 .. t0 + TB - 1 (zero before the sequence and past its end)
  const int R = TB + h0 + h1;
  for (int e = tid; e < R * dh; e += 256) {
    const int i = e / dh, c = e - i * dh;
    const int t = t0 - h0 - h1 + i;
    u[i * dh + c] = (t >= 0 && t < p.S) ? P[(long long)t * Cp + c0 + c] : 0.f;
  }
  __syncthreads();

  // depth-wise sequence convolution: a0 row i is token t0 - h1 + i; a row before the
  // sequence stays zero (the channel convolution pads the sequence convolution's output)
  const int R1 = TB + h1;
  for (int e = tid; e < R1 * dh; e += 256) {
    const int i = e / dh, c = e - i * dh;
    float acc = 0.f;
    if (t0 - h1 + i >= 0) {
      if (p.layers >= 1) {
        const T* w = wseq + (long long)(c0 + c) * p.kseq;
        for (int j = 0; j < p.kseq; ++j) acc = __builtin_fmaf(to_f32(w[j]), u[(i + j) * dh + c], acc);
      } else {
        acc = u[i * dh + c];
      }
    }
    a0[i * dh + c] = acc;
  }
  __syncthreads();

  // channel convolution grouped by head, then the q-k-mean of the pre-convolution values
  for (int e = tid; e < TB * dh; e += 256) {
    const int r = e / dh, oc = e - r * dh;
    const int t = t0 + r;
    float acc = 0.f;
    if (p.layers >= 2) {
      const T* w = wch + (long long)(c0 + oc) * dh * p.kch;
      for (int c = 0; c < dh; ++c)
        for (int j = 0; j < p.kch; ++j) acc = __builtin_fmaf(to_f32(w[c * p.kch + j]), a0[(r + j) * dh + c], acc);
    } else {
      acc = a0[r * dh + oc];
    }
    if (p.qk_mean && t < p.S) {
      const float* row = P + (long long)t * Cp;
      if (is_q) {
        acc += 0.5f * (row[c0 + oc] + row[Lq + (g / gs) * dh + oc]);
      } else {
        const int j = g - p.Hq;
        float m = 0.f;
        for (int hq = j * gs; hq < (j + 1) * gs; ++hq) m += row[hq * dh + oc];
        acc += 0.5f * (m / (float)gs + row[c0 + oc]);
      }
    }
    o[r * dh + oc] = acc;
  }
  __syncthreads();

  // per-row L2 norm over the head's d_h channels (16 threads per row)
  {
    const int r = tid >> 4, l = tid & 15;
    float ss = 0.f;
    for (int c = l; c < dh; c += 16) ss = __builtin_fmaf(o[r * dh + c], o[r * dh + c], ss);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 16);
    if (l == 0) rscale[r] = p.sqrt_dh / fmaxf(sqrtf(ss), 1e-6f) * (is_q ? 1.f : p.key_gain);
  }
  __syncthreads();

  // half-split rotation at the token's position, then the store
  const int half = dh >> 1;
  T* dst = is_q ? reinterpret_cast<T*>(p.q) : reinterpret_cast<T*>(p.k);
  const int nh = is_q ? p.Hq : p.Hkv, hh = is_q ? g : g - p.Hq;
  for (int e = tid; e < TB * half; e += 256) {
    const int r = e / half, jj = e - r * half;
    const int t = t0 + r;
    if (t >= p.S) continue;
    const float x1 = o[r * dh + jj] * rscale[r], x2 = o[r * dh + jj + half] * rscale[r];
    float sn, cs;
    rope_sincos(t, p.rope.hi[jj], p.rope.lo[jj], &sn, &cs);
    T* row = dst + (((long long)b * p.S + t) * nh + hh) * dh;
    row[jj] = from_f32<T>(x1 * cs - x2 * sn);
    row[jj + half] = from_f32<T>(x1 * sn + x2 * cs);
  }

  // the key head's values, shifted by one token in the second half of the channels
  if (!is_q) {
    const int j = g - p.Hq;
    T* vdst = reinterpret_cast<T*>(p.v);
    for (int e = tid; e < TB * dh; e += 256) {
      const int r = e / dh, c = e - r * dh;
      const int t = t0 + r;
      if (t >= p.S) continue;
      const int ch = j * dh + c;
      const int ts = (p.value_shift && ch >= Lkv / 2) ? t - 1 : t;
      const float val = ts >= 0 ? p.V[((long long)b * p.S + ts) * Lkv + ch] : 0.f;
      vdst[(((long long)b * p.S + t) * p.Hkv + j) * dh + c] = from_f32<T>(val);
    }
  }
}

}  // namespace

hipError_t launch_cca_prep(const CcaPrepParams& p, bool use_bf16, hipStream_t s) {
  if (p.dh > kCcaMaxHeadDim || p.kseq > kCcaMaxKernel || p.kch > kCcaMaxKernel) return hipErrorInvalidValue;
  const dim3 grid(cdiv(p.S, TB), p.Hq + p.Hkv, p.B);
  if (use_bf16)
    hipLaunchKernelGGL(cca_prep_kernel<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(cca_prep_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
