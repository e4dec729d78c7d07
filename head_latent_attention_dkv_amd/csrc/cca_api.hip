// Host side of the CCA / CCGQA entry points: argument checks, workspace layout and the
// launch sequence (no allocation, no host synchronisation; everything on the caller's stream).
//   1. packed q | k projections and value projections of x in one GEMM (fp32 outputs);
//   2. cca_prep_kernel: convolutions, q-k-mean, value shift, L2-norm, key temperature, RoPE;
//   3. causal attention, key / value heads grouped: the flash prefill kernel for bf16 heads of
//      32, 64 or 128 features over whole 64-token tiles, the generic prefill kernel otherwise;
//   4. output up-projection.
#include <math.h>
#include <string.h>

#include "../../include/mla.h"
#include "common.h"
#include "internal.h"

using namespace mla;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct CcaWs {
  size_t P, V, q, k, v, o, total;
  int dqp;      // > 0: attention on the flash prefill kernel, heads padded to dqp features
};

// The flash prefill kernel takes bf16 heads of 64 or 128 features and whole 64-token tiles;
// heads of 32 features are zero-padded to 64 (the padding adds nothing to the scores, and
// the padded value features are not stored).  Other shapes use the generic kernel.
int flash_width(const mla_cca_dims* d, int S) {
  if (d->dtype != MLA_DTYPE_BF16 || S <= 0) return 0;
  const int dqp = d->head_dim == 32 ? 64 : d->head_dim;
  return prefill_fast_supported(dqp, 0, dqp, S) ? dqp : 0;
}

CcaWs cca_layout(const mla_cca_dims* d, int B, int S) {
  CcaWs w{};
  const size_t rows = (size_t)B * S;
  const size_t es = d->dtype == MLA_DTYPE_BF16 ? 2 : 4;
  const size_t Lq = (size_t)d->n_heads * d->head_dim, Lkv = (size_t)d->n_kv_heads * d->head_dim;
  w.dqp = flash_width(d, S);
  const size_t wq = (size_t)d->n_heads * (w.dqp ? w.dqp : d->head_dim);
  const size_t wkv = (size_t)d->n_kv_heads * (w.dqp ? w.dqp : d->head_dim);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  w.P = take(rows * (Lq + Lkv) * 4);
  w.V = take(rows * Lkv * 4);
  w.q = take(rows * wq * es);
  w.k = take(rows * wkv * es);
  w.v = take(rows * wkv * es);
  w.o = take(rows * Lq * es);
  w.total = off;
  return w;
}

GemmSeg seg(const void* wt, long long w_ld, int n, void* out, long long out_ld, bool f32) {
  GemmSeg s;
  memset(&s, 0, sizeof(s));
  s.w = wt;
  s.w_ld = w_ld;
  s.n = n;
  s.out = out;
  s.out_ld = out_ld;
  s.out_f32 = f32 ? 1 : 0;
  return s;
}

GemmParams gemm_rows(const void* a, long long a_ld, int M, int K) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = a;
  p.a_ld = a_ld;
  p.M = M;
  p.K = K;
  p.zdiv = 1;
  p.rows_per_batch = 1;
  p.nseg = 1;
  return p;
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

}  // namespace

extern "C" {

mla_status mla_cca_validate(const mla_cca_dims* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->d_model <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0) return MLA_ERR_INVALID_ARG;
  if (d->dtype != MLA_DTYPE_F32 && d->dtype != MLA_DTYPE_BF16) return MLA_ERR_INVALID_ARG;
  if (d->num_conv_layers < 0 || d->num_conv_layers > 2) return MLA_ERR_SHAPE;
  if (d->num_conv_layers >= 1 && d->conv_kernel_seq <= 0) return MLA_ERR_INVALID_ARG;
  if (d->num_conv_layers >= 2 && d->conv_kernel_ch <= 0) return MLA_ERR_INVALID_ARG;
  if (!(d->rope_base > 0.f)) return MLA_ERR_INVALID_ARG;
  // the page's constructor checks
  if (d->d_model % d->n_heads) return MLA_ERR_SHAPE;                  // E divisible by the heads
  if (d->n_heads % d->n_kv_heads) return MLA_ERR_SHAPE;               // Hkv divides Hq
  if (d->head_dim % 2) return MLA_ERR_SHAPE;                          // RoPE in the latent
  if (d->value_shift && (d->n_kv_heads % 2)) return MLA_ERR_SHAPE;    // halves of the value heads
  // kernel limits
  const int max_dh = d->dtype == MLA_DTYPE_BF16 ? 128 : 64;
  if (d->head_dim > max_dh || d->head_dim > kCcaMaxHeadDim) return MLA_ERR_UNSUPPORTED;
  if (d->num_conv_layers >= 1 && d->conv_kernel_seq > kCcaMaxKernel) return MLA_ERR_UNSUPPORTED;
  if (d->num_conv_layers >= 2 && d->conv_kernel_ch > kCcaMaxKernel) return MLA_ERR_UNSUPPORTED;
  int a, b;
  if (!prefill_supported(d->dtype == MLA_DTYPE_BF16, d->head_dim, d->head_dim, &a, &b)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t mla_cca_workspace_bytes(const mla_cca_dims* d, int32_t B, int32_t S) {
  if (mla_cca_validate(d) != MLA_OK || B <= 0 || S <= 0) return 0;
  return cca_layout(d, B, S).total;
}

mla_status mla_cca_prefill(const mla_cca_dims* d, const mla_cca_weights* w, const void* x, int32_t B, int32_t S,
                           float* y, void* ws, size_t ws_bytes, void* stream) {
  mla_status s = mla_cca_validate(d);
  if (s != MLA_OK) return s;
  if (!w || !x || !y || B <= 0 || S <= 0) return MLA_ERR_INVALID_ARG;
  if (!w->w_qk || !w->w_v || !w->w_o) return MLA_ERR_INVALID_ARG;
  if (d->num_conv_layers >= 1 && !w->conv_seq) return MLA_ERR_INVALID_ARG;
  if (d->num_conv_layers >= 2 && !w->conv_ch) return MLA_ERR_INVALID_ARG;
  if (!(w->key_temperature == w->key_temperature)) return MLA_ERR_INVALID_ARG;
  const CcaWs lay = cca_layout(d, B, S);
  if (!ws || ws_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = d->dtype == MLA_DTYPE_BF16;
  const int E = d->d_model, Hq = d->n_heads, Hkv = d->n_kv_heads, dh = d->head_dim;
  const int Lq = Hq * dh, Lkv = Hkv * dh, M = B * S;
  float* P = reinterpret_cast<float*>(at(ws, lay.P));
  float* V = reinterpret_cast<float*>(at(ws, lay.V));

  // 1. [q | k] = x W_qk^T and the value projections (current- and previous-token rows of w_v
  //    applied to every token; the shift happens in step 2)
  GemmParams g = gemm_rows(x, E, M, E);
  g.nseg = 2;
  g.seg[0] = seg(w->w_qk, E, Lq + Lkv, P, Lq + Lkv, true);
  g.seg[1] = seg(w->w_v, E, Lkv, V, Lkv, true);
  if (launch_gemm(g, 1, bf, st) != hipSuccess) return MLA_ERR_HIP;

  // 2. convolutions, q-k-mean, value shift, normalisation, temperature, RoPE
  CcaPrepParams cp;
  memset(&cp, 0, sizeof(cp));
  cp.P = P;
  cp.V = V;
  cp.conv_seq = w->conv_seq;
  cp.conv_ch = w->conv_ch;
  cp.q = at(ws, lay.q);
  cp.k = at(ws, lay.k);
  cp.v = at(ws, lay.v);
  cp.B = B;
  cp.S = S;
  cp.Hq = Hq;
  cp.Hkv = Hkv;
  cp.dh = dh;
  cp.layers = d->num_conv_layers;
  cp.kseq = d->num_conv_layers >= 1 ? d->conv_kernel_seq : 1;
  cp.kch = d->num_conv_layers >= 2 ? d->conv_kernel_ch : 1;
  cp.qk_mean = d->qk_mean ? 1 : 0;
  cp.value_shift = d->value_shift ? 1 : 0;
  cp.sqrt_dh = (float)sqrt((double)dh);
  cp.key_gain = (float)exp((double)w->key_temperature);
  make_rope_table(&cp.rope, dh, d->rope_base);
  cp.flash = lay.dqp > 0 ? 1 : 0;
  cp.dqp = lay.dqp;
  if (launch_cca_prep(cp, bf, st) != hipSuccess) return MLA_ERR_HIP;

  // 3. causal softmax attention inside the latent, scale d_h^-1/2
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));
  if (lay.dqp) {
    FlashParams fp;
    memset(&fp, 0, sizeof(fp));
    fp.q = cp.q;
    fp.k = cp.k;
    fp.kr = nullptr;
    fp.vt = cp.v;
    fp.o = at(ws, lay.o);
    fp.B = B;
    fp.S = S;
    fp.T = S;
    fp.q_off = 0;
    fp.H = Hq;
    fp.dn = lay.dqp;
    fp.d_rope = 0;
    fp.scale_log2 = scale_log2;
    fp.kv_group = Hq / Hkv;
    fp.dv_out = dh;
    if (launch_prefill_fast(fp, st) != hipSuccess) return MLA_ERR_HIP;
    GemmParams go = gemm_rows(fp.o, Lq, M, Lq);
    go.seg[0] = seg(w->w_o, Lq, E, y, E, true);
    return launch_gemm(go, 1, bf, st) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  int dqp, dvp;
  prefill_supported(bf, dh, dh, &dqp, &dvp);
  PrefillParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = cp.q;
  pp.k = cp.k;
  pp.kr = nullptr;
  pp.v = cp.v;
  pp.o = at(ws, lay.o);
  pp.B = B;
  pp.S = S;
  pp.T = S;
  pp.q_off = 0;
  pp.H = Hq;
  pp.dn = dh;
  pp.d_rope = 0;
  pp.dv = dh;
  pp.kv_group = Hq / Hkv;
  pp.scale_log2 = scale_log2;
  if (launch_prefill(pp, bf, dqp, dvp, st) != hipSuccess) return MLA_ERR_HIP;

  // 4. y = o W_o^T
  GemmParams go = gemm_rows(pp.o, Lq, M, Lq);
  go.seg[0] = seg(w->w_o, Lq, E, y, E, true);
  return launch_gemm(go, 1, bf, st) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
