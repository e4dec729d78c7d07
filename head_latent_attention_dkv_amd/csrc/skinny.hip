// Weight-streaming projection GEMM for few rows (M <= 128: one new token per sequence in
// decode, or a short append).  out[m, n] = sum_k A[m, k] W[n, k] with W in [out][in] layout.
//
// With M this small the product reads each weight once and does 2M flops per weight
// element, far below the matrix-core ridge, so the kernel is built to stream W at HBM
// rate: a block owns 64 output columns (two 32-row blocks of W) and a slab of K; its four
// waves take interleaved 16-wide k-steps, loading W and A fragments straight from global
// memory in the 32x32x16 MFMA operand layout (a wave's four neighbours read the other
// quarters of the same 128-byte lines at the same time), with U k-steps of loads in flight
// per wave.  The waves' accumulators are summed through LDS in a fixed order.  A single
// slab applies the shared epilogue directly; several slabs (split K, so that enough blocks
// cover the 256 compute units when N is small) write fp32 partial blocks to the caller's
// workspace and a second kernel sums them in slab order and applies the epilogue.
#include "common.h"
#include "gemm_epilogue.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int kCols = 64;           // output columns per block
constexpr int kLdc = kCols + 4;     // LDS row stride (floats)
constexpr int kTargetBlocks = 512;  // two blocks per compute unit

struct Goff {
  long long a, w, o;
};

__device__ __forceinline__ Goff group_offsets(const GemmParams& p, int z) {
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  return {zo * p.a_goff[0] + zi * p.a_goff[1], zo * p.w_goff[0] + zi * p.w_goff[1],
          zo * p.o_goff[0] + zi * p.o_goff[1]};
}

__device__ __forceinline__ long long a_row(const GemmParams& p, int m) {
  if (!p.a_cache) return m;
  const int b = m / p.rows_per_batch;
  return (long long)b * p.a_bstride + (m - b * p.rows_per_batch);
}

// CB = 32-row blocks of A (M <= 32 CB); U = k-steps per wave per loop trip.
template <int CB, int U>
__global__ void __launch_bounds__(256) skinny_kernel(GemmParams p) {
  __shared__ float Cs[32 * CB * kLdc];
  __shared__ float rtab[kRopeTabFloats];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform k schedule
  const int col = lane & 31, half = lane >> 5;
  const int n0 = blockIdx.x * kCols;
  const int split = blockIdx.y;
  const int z = blockIdx.z;
  const Goff g = group_offsets(p, z);
  const int N = seg_total(p);
  const int k_begin = split * p.kchunk;
  const int k_end = min(p.K, k_begin + p.kchunk);

  // lane -> W row n0 + 32 rb + col (clamped into range; such columns are never stored)
  const bf16* wrow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int n = min(n0 + 32 * rb + col, N - 1);
    int nn;
    const int s = seg_of(p, n, &nn);
    wrow[rb] = reinterpret_cast<const bf16*>(p.seg[s].w) + g.w + (long long)nn * p.seg[s].w_ld + 8 * half;
  }
  // lane -> A row 32 cb + col (clamped likewise)
  const bf16* xrow[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int m = min(32 * cb + col, p.M - 1);
    xrow[cb] = reinterpret_cast<const bf16*>(p.a) + a_row(p, m) * p.a_ld + g.a + 8 * half;
  }

  f32x16 acc[2][CB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16{};

  // Two register buffers of U k-steps per wave (a trip covers 64 U elements of K for the
  // block): the loads of the next trip are in flight while the MFMAs of the current one
  // run.  Whole pairs of trips run unpredicated; a remainder (K not a multiple of the
  // pair) runs trip by trip with predicated loads.
  Frag<bf16> fw[2][U][2], fx[2][U][CB];
  auto load = [&](int buf, int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + 16 * wave + 64 * u;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) fw[buf][u][rb] = frag_load<bf16>(wrow[rb] + k);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) fx[buf][u][cb] = frag_load<bf16>(xrow[cb] + k);
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mma32(fw[buf][u][rb], fx[buf][u][cb], acc[rb][cb]);
  };
  constexpr int TRIP = 64 * U;
  int kb = k_begin;
  const int pairs = (k_end - k_begin) / (2 * TRIP);
  if (pairs > 0) {
    load(0, kb);
    for (int i = 1; i < pairs; ++i) {
      load(1, kb + TRIP);
      mma(0);
      load(0, kb + 2 * TRIP);
      mma(1);
      kb += 2 * TRIP;
    }
    load(1, kb + TRIP);
    mma(0);
    mma(1);
    kb += 2 * TRIP;
  }
  for (; kb < k_end; kb += TRIP) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + 16 * wave + 64 * u;
      const bool ok = k < k_end;   // k_end - k is a multiple of 16
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) fw[0][u][rb] = ok ? frag_load<bf16>(wrow[rb] + k) : frag_zero<bf16>();
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) fx[0][u][cb] = ok ? frag_load<bf16>(xrow[cb] + k) : frag_zero<bf16>();
    }
    mma(0);
  }

  if (p.splits == 1 && gemm_has_rope(p)) stage_rope_table(p, rtab, tid, 256);
  // Sum the four waves' partial products in wave order.  Accumulator element e of lane l
  // is out[32 cb + l%32][32 rb + 8 (e/4) + 4 (l/32) + e%4].
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float* dst = &Cs[(32 * cb + col) * kLdc + 32 * rb + 8 * (e >> 2) + 4 * half + (e & 3)];
            *dst = (w == 0) ? acc[rb][cb][e] : *dst + acc[rb][cb][e];
          }
    }
    __syncthreads();
  }

  if (p.splits == 1) {
    epilogue_block<bf16>(p, Cs, kLdc, 0, 32 * CB, n0, kCols, g.o, tid, 256, rtab);
    return;
  }
  float* part = p.part + ((long long)z * p.splits + split) * p.M * N;
  for (int e = tid; e < 32 * CB * kCols; e += 256) {
    const int r = e / kCols, c = e - r * kCols;
    if (r < p.M && n0 + c < N) part[(long long)r * N + n0 + c] = Cs[r * kLdc + c];
  }
}

// Streaming variant.  Per stage of KT k-elements, the block's 128 weight rows and its
// 32 CB activation rows move global -> LDS with 16-byte direct-to-LDS copies; each copy
// instruction reads ROWS_PER_COPY whole row segments (coalesced, unlike the 32-row operand
// pattern of the direct kernel), and NST stages are in flight.  Both operands are read
// back in the 32x32x16 layout (lane -> row l%32, k-group l/32) through an XOR swizzle:
// 16-byte chunk c of row r sits at c ^ (r mod CHUNKS), so the 8 rows of one LDS read
// phase hit distinct banks.  Wave w takes k-steps KSW w .. KSW w + KSW - 1 of every
// stage; the waves' partial sums meet in LDS as in the direct kernel.
template <int CB, int ROWS_, int KT, int NST>
struct StreamCfg {
  static constexpr int ROWS = ROWS_;               // weight rows per block (32, 64, 96 or 128)
  static constexpr int RB = ROWS / 32;
  static constexpr int XROWS = 32 * CB;            // activation rows per block
  static constexpr int CHUNKS = KT / 8;            // 16-byte chunks per row segment
  static constexpr int RPC = 64 / CHUNKS;          // rows per copy instruction
  static constexpr int WPW = ROWS / RPC / 4;       // weight copies per wave per stage
  static constexpr int XPW = XROWS / RPC / 4;      // activation copies per wave per stage
  static constexpr int DPW = WPW + XPW;
  static constexpr int KSW = KT / 64;              // k-steps per wave per stage
  static constexpr int WBYTES = ROWS * KT * 2;
  static constexpr int STAGE = (ROWS + XROWS) * KT * 2;
  static constexpr int LDC = ROWS + 4;
  static constexpr size_t PART = (size_t)XROWS * LDC;   // floats of one wave's partial block
  static constexpr size_t LDS = (size_t)NST * STAGE > 4 * PART * 4 ? (size_t)NST * STAGE : 4 * PART * 4;
  static_assert(KT == 64 || KT == 128, "stage width");
  static_assert(XPW >= 1 && WPW >= 1 && NST >= 2 && NST <= 4, "pipeline shape");
};

template <int CB, int ROWS, int KT, int NST>
__global__ void __launch_bounds__(256, CB * ROWS <= 256 ? 2 : 1) skinny_stream_kernel(GemmParams p) {
  using C = StreamCfg<CB, ROWS, KT, NST>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int n0 = blockIdx.x * C::ROWS;
  const int split = blockIdx.y;
  const int z = blockIdx.z;
  const Goff g = group_offsets(p, z);
  const int N = seg_total(p);
  const int k_begin = split * p.kchunk;
  const int nst = (min(p.K, k_begin + p.kchunk) - k_begin) / KT;   // stages of this slab
  const uint32_t lds0 = lds_addr_of(smem);
  const int pc = lane % C::CHUNKS;                 // physical chunk this lane's copies fill

  // copy sources (row t of a copy = copy index * RPC + lane / CHUNKS; the lane fetches the
  // logical chunk that belongs at physical chunk pc)
  const bf16* wsrc[C::WPW];
#pragma unroll
  for (int i = 0; i < C::WPW; ++i) {
    const int t = (wave * C::WPW + i) * C::RPC + lane / C::CHUNKS;
    const int n = min(n0 + t, N - 1);
    int nn;
    const int s = seg_of(p, n, &nn);
    wsrc[i] = reinterpret_cast<const bf16*>(p.seg[s].w) + g.w + (long long)nn * p.seg[s].w_ld + k_begin +
              8 * (pc ^ (t % C::CHUNKS));
  }
  const bf16* xsrc[C::XPW];
#pragma unroll
  for (int i = 0; i < C::XPW; ++i) {
    const int t = (wave * C::XPW + i) * C::RPC + lane / C::CHUNKS;
    const int m = min(t, p.M - 1);
    xsrc[i] = reinterpret_cast<const bf16*>(p.a) + a_row(p, m) * p.a_ld + g.a + k_begin + 8 * (pc ^ (t % C::CHUNKS));
  }
  // operand LDS offsets: row col (+ 32 per row block), logical chunk 2 (KSW w + j) + half
  int off[C::KSW];
#pragma unroll
  for (int j = 0; j < C::KSW; ++j) {
    const int c = 2 * (C::KSW * wave + j) + half;
    off[j] = col * (KT * 2) + ((c ^ (col % C::CHUNKS)) << 4);
  }

  auto issue = [&](int st) {
    const uint32_t base = lds0 + (st % NST) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::WPW; ++i)
      dma16_nt(wsrc[i] + st * KT, __builtin_amdgcn_readfirstlane(base + (wave * C::WPW + i) * 1024));   // read once
#pragma unroll
    for (int i = 0; i < C::XPW; ++i)
      dma16(xsrc[i] + st * KT, __builtin_amdgcn_readfirstlane(base + C::WBYTES + (wave * C::XPW + i) * 1024));
  };

  f32x16 acc[C::RB][CB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16{};

  copies_begin();   // lds_dma.h, rule 1
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nst) issue(st);
  for (int it = 0; it < nst; ++it) {
    const int left = nst - 1 - it;                 // stages after this one
    if (NST >= 4 && left >= 2) wait_vmcnt<2 * C::DPW>();
    else if (NST >= 3 && left >= 1) wait_vmcnt<C::DPW>();
    else wait_vmcnt<0>();
    barrier_only();
    if (it + NST - 1 < nst) issue(it + NST - 1);

    const unsigned char* T = smem + (it % NST) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::KSW; ++j) {
      Frag<bf16> fx[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        fx[cb] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + C::WBYTES + off[j] + cb * 32 * KT * 2));
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        const Frag<bf16> fa = frag_load<bf16>(reinterpret_cast<const bf16*>(T + off[j] + rb * 32 * KT * 2));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mma32(fa, fx[cb], acc[rb][cb]);
      }
    }
  }
  copies_end();   // lds_dma.h, rule 3
  // the inverse-frequency table sits behind the stages and partial buffers
  float* rtab = reinterpret_cast<float*>(smem + C::LDS);
  if (p.splits == 1 && gemm_has_rope(p)) stage_rope_table(p, rtab, tid, 256);
  __syncthreads();

  // The four waves' partial products are summed in wave order.  Each wave stores its block
  // to a buffer of its own (accumulator elements 4q..4q+3 of a lane are four consecutive
  // columns: one 16-byte store); the readers then add buffers 0, 1, 2, 3 in that order.
  // (Adding them wave after wave into one buffer -- a load, an add and a store per element,
  // a barrier per wave -- had cost more than the whole K loop of a block.)
  float* Cs = reinterpret_cast<float*>(smem);
  {
    float* Pw = Cs + wave * C::PART;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(&Pw[(32 * cb + col) * C::LDC + 32 * rb + 8 * q + 4 * half]) =
              (f32x4){acc[rb][cb][4 * q], acc[rb][cb][4 * q + 1], acc[rb][cb][4 * q + 2], acc[rb][cb][4 * q + 3]};
  }
  __syncthreads();
  auto sum4 = [&](int r, int c) {
    f32x4 v = *reinterpret_cast<const f32x4*>(&Cs[r * C::LDC + c]);
#pragma unroll
    for (int w = 1; w < 4; ++w) v = v + *reinterpret_cast<const f32x4*>(&Cs[w * C::PART + r * C::LDC + c]);
    return v;
  };
  if (p.splits == 1 && p.fast_epilogue) {
    // vectorised stage straight from the four buffers: each wave a quarter of the rows,
    // 8 columns per lane
    constexpr int RW = C::XROWS / 4;
    epilogue_block_fast<bf16, RW, 4>(p, Cs + wave * RW * C::LDC, C::LDC, (int)C::PART, wave * RW, n0, C::ROWS,
                                     g.o, lane, rtab);
    return;
  }
  if (p.splits > 1) {
    // split K: the block's sums go to the workspace in fp32, 16 bytes per store where the
    // row allows it
    float* part = p.part + ((long long)z * p.splits + split) * p.M * N;
    for (int i = tid; i < C::XROWS * (C::ROWS / 4); i += 256) {
      const int r = i / (C::ROWS / 4), c = 4 * (i - r * (C::ROWS / 4));
      if (r >= p.M || n0 + c >= N) continue;
      const f32x4 v = sum4(r, c);
      float* dst = part + (long long)r * N + n0 + c;
      if ((N & 3) == 0 && n0 + c + 4 <= N) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
        for (int e = 0; e < 4 && n0 + c + e < N; ++e) dst[e] = v[e];
      }
    }
    return;
  }
  // generic stage: the sums into buffer 0 first
  for (int i = tid; i < C::XROWS * (C::ROWS / 4); i += 256) {
    const int r = i / (C::ROWS / 4), c = 4 * (i - r * (C::ROWS / 4));
    const f32x4 v = sum4(r, c);
    *reinterpret_cast<f32x4*>(&Cs[r * C::LDC + c]) = v;
  }
  __syncthreads();
  epilogue_block<bf16>(p, Cs, C::LDC, 0, C::XROWS, n0, C::ROWS, g.o, tid, 256, rtab);
}

// Sum of the slabs' partial blocks (slab order) followed by the shared epilogue; a
// block covers kRedRows rows x 64 columns, one element per thread.
constexpr int kRedRows = 4;

__global__ void __launch_bounds__(256) split_reduce_kernel(GemmParams p) {
  __shared__ float Cs[kRedRows * kLdc];
  __shared__ float rtab[kRopeTabFloats];
  const int tid = threadIdx.x;
  if (gemm_has_rope(p)) stage_rope_table(p, rtab, tid, 256);
  const int n0 = blockIdx.x * kCols;
  const int m0 = blockIdx.y * kRedRows;
  const int z = blockIdx.z;
  const Goff g = group_offsets(p, z);
  const int N = seg_total(p);
  const long long plane = (long long)p.M * N;
  const int r = tid / kCols, c = tid - r * kCols;
  float v = 0.f;
  if (m0 + r < p.M && n0 + c < N) {
    const float* src = p.part + (long long)z * p.splits * plane + (long long)(m0 + r) * N + n0 + c;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 4 <= p.splits; s += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = src[(s + j) * plane];
#pragma unroll
      for (int j = 0; j < 4; ++j) v += a[j];
    }
    for (; s < p.splits; ++s) v += src[s * plane];
  }
  Cs[r * kLdc + c] = v;
  __syncthreads();
  epilogue_block<bf16>(p, Cs, kLdc, m0, kRedRows, n0, kCols, g.o, tid, 256, rtab);
}

bool aligned16(const void* ptr, long long elem_off) {
  return ((reinterpret_cast<uintptr_t>(ptr) + 2 * elem_off) & 15) == 0;
}

// Per-wave k-steps of one loop trip of the direct kernel for an M-row product.
int trip_steps(int M) { return M <= 64 ? 4 : 2; }

// Split-K plan: enough blocks for `slots` resident blocks, K slabs a multiple of `unit`,
// and a bounded volume of fp32 partials (2 S M / K of the weight bytes).
void plan_splits(int M, int N, int K, int groups, int cols, int slots, int unit, int* splits,
                 int* kchunk) {
  const int tiles = cdiv(N, cols) * groups;
  int s = slots / tiles;
  // partials up to half the weight bytes, or up to all of them when the tiles are few
  const int by_bytes = tiles >= 64 ? K / (4 * M) : K / (2 * M);
  const int by_unit = K / unit;
  s = s > by_bytes ? by_bytes : s;
  s = s > by_unit ? by_unit : s;
  s = s < 1 ? 1 : s;
  int kc = round_up(cdiv(K, s), unit);
  s = cdiv(K, kc);
  if (s <= 1) kc = K;
  *splits = s;
  *kchunk = kc;
}

constexpr int kStreamKT = 64;
constexpr int kMinStagesPerSlab = 4;

bool use_stream(int K) { return K % kStreamKT == 0; }

struct SkinnyPlan {
  int rows, splits, kchunk;
  bool deep = false;   // one block per CU: 128-row tiles take four stages instead of three
};

constexpr int kLongSlab = 2048;           // K per block from which one block per CU pays

// Streaming plan: the weight-row tile (32, 64 or 128 rows) and the number of K slabs that
// reach kMinBlocks blocks (or as many as the shape allows) with the least extra traffic:
// fp32 partials written and read back (8 S M N bytes when S > 1) plus the activations
// re-read from L2 by every row tile (weighted 1/2: they do not come from HBM).
//
// min_rows: the smallest tile that keeps every half-split rotary pair (j, j + d/2) of a head
// inside one tile, whose epilogue reads the partner column from LDS (64 when a segment is
// rotated half-split, 32 otherwise).
SkinnyPlan plan_stream(int M, int N, int K, int groups, int min_rows = 32) {
  const int kCUs = device_cu_count();
  const int kMinBlocks = kCUs * 3 / 2;    // enough resident blocks to keep HBM busy
  SkinnyPlan best{M > 64 ? 64 : 128, 1, K};
  double best_cost = 1e300;
  int best_blocks = 0;
  const int max_s = K / (kStreamKT * kMinStagesPerSlab) > 0 ? K / (kStreamKT * kMinStagesPerSlab) : 1;
  // Wide outputs (512 or more 32-row tiles) take 32-row tiles without split: three blocks fit
  // on a CU, so the blocks land evenly on the compute units (64-row tiles leave half of
  // them with one block and half with two).
  const bool wide = (long long)cdiv(N, 32) * groups >= 512;
  // Wide outputs whose 96-row tiles number between half a CU and one CU each take them, one
  // block per CU: every CU then reads the activation rows once (with 32-row tiles, three
  // blocks per CU read them three times).  The decode step's query up-projection (24576 x
  // 1536) is 256 such tiles.
  if (wide && min_rows <= 32 && M <= 64) {
    const long long t96 = (long long)cdiv(N, 96) * groups;
    if (t96 <= kCUs && 2 * t96 > kCUs) return SkinnyPlan{96, 1, K, false};
  }
  for (int rows : {128, 64, 32}) {
    if (M > 64 && rows == 128) continue;                 // accumulator budget
    if (rows < min_rows) continue;
    if (wide && rows != (min_rows > 32 ? min_rows : 32)) continue;
    const long long tiles = (long long)cdiv(N, rows) * groups;
    int s = (int)((kMinBlocks + tiles - 1) / tiles);
    s = s < 1 ? 1 : (s > max_s ? max_s : s);
    int kc = round_up(cdiv(K, s), kStreamKT);
    s = cdiv(K, kc);
    if (s <= 1) kc = K;
    const long long blocks = tiles * s;
    const double cost = (s > 1 ? 8.0 * s * M * N * groups : 0.0) + 0.5 * (double)tiles * M * K * 2;
    const bool enough = blocks >= kMinBlocks;
    const bool best_enough = best_blocks >= kMinBlocks;
    if ((enough && !best_enough) || (enough == best_enough && (enough ? cost < best_cost : blocks > best_blocks))) {
      best = {rows, s, kc};
      best_cost = cost;
      best_blocks = (int)blocks;
    }
  }
  // Between one and two blocks per CU, the CUs holding two set the time.  When every block's
  // K slab stays long, fewer slabs that give one block per CU are faster (the decode step's
  // output projection, 5120 x 16384 at 64 rows: 128 rows x 10 slabs 46 us, x 6 slabs 40 us).
  if (best_blocks > kCUs && best_blocks < 2 * kCUs) {
    const long long tiles = (long long)cdiv(N, best.rows) * groups;
    const int s = (int)(kCUs / tiles);
    if (s >= 1) {
      int kc = round_up(cdiv(K, s), kStreamKT);
      if (kc >= kLongSlab) {
        const int s2 = cdiv(K, kc);
        best = {best.rows, s2, s2 <= 1 ? K : kc, true};
      }
    }
  }
  return best;
}

SkinnyPlan plan_direct(int M, int N, int K, int groups) {
  int s, kc;
  plan_splits(M, N, K, groups, kCols, kTargetBlocks, 2 * 64 * trip_steps(M), &s, &kc);
  return {kCols, s, kc};
}

SkinnyPlan plan(int M, int N, int K, int groups, int min_rows = 32) {
  return use_stream(K) ? plan_stream(M, N, K, groups, min_rows) : plan_direct(M, N, K, groups);
}

// Smallest streaming tile (output columns) whose blocks hold whole half-split rotary heads.
int min_stream_rows(const GemmParams& p) {
  for (int i = 0; i < p.nseg; ++i)
    if (p.seg[i].rope == ROPE_HALFSPLIT) return 64;
  return 32;
}

template <int CB, int ROWS, int NST = ROWS == 128 ? 3 : 4>
hipError_t launch_stream(const GemmParams& p, int groups, hipStream_t s) {
  using C = StreamCfg<CB, ROWS, kStreamKT, NST>;
  const int N = seg_total(p);
  dim3 grid(cdiv(N, ROWS), p.splits, groups);
  hipLaunchKernelGGL((skinny_stream_kernel<CB, ROWS, kStreamKT, NST>), grid, dim3(256), C::LDS + kRopeTabFloats * 4, s, p);
  return hipGetLastError();
}

template <int CB>
hipError_t launch_stream_rows(const GemmParams& p, const SkinnyPlan& pl, int groups, hipStream_t s) {
  if (pl.rows == 32) return launch_stream<CB, 32>(p, groups, s);
  if (pl.rows == 64) return launch_stream<CB, 64>(p, groups, s);
  if constexpr (CB <= 2) {
    if (pl.rows == 96) return launch_stream<CB, 96, 4>(p, groups, s);
    if (pl.deep) return launch_stream<CB, 128, 4>(p, groups, s);
    return launch_stream<CB, 128>(p, groups, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t skinny_ws_bytes(int M, int N, int K, int groups) {
  if (M <= 0 || M > 128 || N <= 0 || K <= 0 || groups <= 0) return 0;
  const SkinnyPlan pl = plan(M, N, K, groups);
  return pl.splits > 1 ? (size_t)pl.splits * groups * M * N * sizeof(float) : 0;
}

bool skinny_supported(const GemmParams& p, int groups) {
  if (p.w_kmajor || p.M <= 0 || p.M > 128 || p.K % 16 != 0 || p.a_ld % 8 != 0) return false;
  (void)groups;
  for (int i = 0; i < 2; ++i)
    if (p.a_goff[i] % 8 != 0 || p.w_goff[i] % 8 != 0) return false;
  if (!aligned16(p.a, 0)) return false;
  int start = 0;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (sg.w_ld % 8 != 0 || !aligned16(sg.w, 0)) return false;
    if (sg.rope == ROPE_INTERLEAVED && (start % 2 != 0 || sg.rope_d % 2 != 0)) return false;
    if (sg.rope == ROPE_HALFSPLIT && (start % kCols != 0 || sg.rope_d > kCols || kCols % sg.rope_d != 0))
      return false;
    start += sg.n;
  }
  return true;
}

// The vectorised output stage (8 columns per lane, one sine / cosine per rotary pair) when the
// segments allow it; transposed segments keep the generic stage (they need 32-row chunks).
bool skinny_fast_epilogue(const GemmParams& p, int groups) {
  for (int i = 0; i < p.nseg; ++i)
    if (p.seg[i].layout == OUT_HEAD_T16) return false;
  return gemm_fast_epilogue_ok(p, groups);
}

hipError_t launch_skinny(GemmParams p, int groups, hipStream_t s) {
  const int N = seg_total(p);
  p.fast_epilogue = skinny_fast_epilogue(p, groups) ? 1 : 0;
  SkinnyPlan pl = plan(p.M, N, p.K, groups, min_stream_rows(p));
  const size_t need = pl.splits > 1 ? (size_t)pl.splits * groups * p.M * N * sizeof(float) : 0;
  if (pl.splits > 1 && (p.part == nullptr || p.part_bytes < need)) {
    pl.splits = 1;
    pl.kchunk = p.K;
    pl.deep = false;
  }
  p.splits = pl.splits;
  p.kchunk = pl.kchunk;
  hipError_t e;
  if (use_stream(p.K)) {
    if (p.M <= 32) e = launch_stream_rows<1>(p, pl, groups, s);
    else if (p.M <= 64) e = launch_stream_rows<2>(p, pl, groups, s);
    else e = launch_stream_rows<4>(p, pl, groups, s);
  } else {
    dim3 grid(cdiv(N, kCols), p.splits, groups);
    if (p.M <= 32)
      hipLaunchKernelGGL((skinny_kernel<1, 4>), grid, dim3(256), 0, s, p);
    else if (p.M <= 64)
      hipLaunchKernelGGL((skinny_kernel<2, 4>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((skinny_kernel<4, 2>), grid, dim3(256), 0, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(split_reduce_kernel, dim3(cdiv(N, kCols), cdiv(p.M, kRedRows), groups), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
