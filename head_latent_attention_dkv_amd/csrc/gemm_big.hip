// Large projection GEMM for gfx950 (bf16, many rows): out[m, n] = sum_k A[m, k] W[n, k].
//
// Workgroup tile 256 x 256, 8 waves (two per SIMD) in a 4 x 2 grid, or 256 x 128 with 4 waves
// in a 4 x 1 grid and two workgroups per CU (one's output stage overlaps the other's main
// loop); each wave a 64 x 128 block of 32x32x16 MFMA accumulators (8 x 16 fp32 per lane, in
// the accumulation registers).  K advances 32 at a time through NST LDS stages filled by
// 16-byte direct-to-LDS copies: each copy instruction moves 16 rows x 64 bytes of A or of W.  Rows are 64 bytes (four
// 16-byte chunks); chunk c of row r sits at c ^ ((r >> 2) & 3), which puts the 8 rows of
// one LDS read phase (row stride 64 B) on 8 distinct 16-byte bank windows.
//
// Output stages:
//   * the keys / values of flash prefill (every wave's 128 columns inside one head of one
//     segment, bf16, no rotation) are written straight from the accumulators (values,
//     transposed) or through a small bf16 transpose in LDS (keys, head-major);
//   * everything else goes through LDS per wave, 32 rows at a time, into the shared output
//     stage (rotary pairs, head scatter, cache rows, head-major / transposed layouts).
#include <type_traits>

#include "common.h"
#include "gemm_epilogue.h"
#include "internal.h"
#include "lds_dma.h"

namespace mla {

namespace {

constexpr int GBM = 256, GBK = 32;
constexpr int G_AB = GBM * GBK * 2;                 // A bytes per stage (16 KB)
constexpr int G_LDC = 128 + 4;                      // epilogue LDS row stride (floats)
constexpr int KV_CS = 72;                           // bf16 column stride (bytes) of the key transpose
constexpr int KV_BUF = 128 * KV_CS;                 // one 32-row x 128-column chunk

template <int NW>
struct BigCfg {
  static constexpr int BN = 32 * NW;                // workgroup columns (256 or 128)
  static constexpr int NST = NW == 8 ? 4 : 3;       // LDS stages
  static constexpr int WB = BN * GBK * 2;           // W bytes per stage
  static constexpr int STAGE = G_AB + WB;
  static constexpr int A_CPW = (G_AB / 1024) / NW;  // copies per wave per stage: A, W
  static constexpr int W_CPW = (WB / 1024) / NW;
  static constexpr int DPW = A_CPW + W_CPW;
  static constexpr size_t EPI = (size_t)NW * 32 * G_LDC * 4;   // per-wave 32-row epilogue chunks
  static constexpr size_t LDS = (size_t)NST * STAGE > EPI ? (size_t)NST * STAGE : EPI;
  static constexpr int MINB = NW == 8 ? 1 : 2;      // workgroups per CU
  static_assert((size_t)NW * KV_BUF <= LDS, "key transpose buffers fit in the stages");
  static_assert(MINB * LDS <= 160 * 1024, "workgroups per CU fit the LDS");
};
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ long long big_a_row(const GemmParams& p, int m) {
  if (!p.a_cache) return m;
  const int b = m / p.rows_per_batch;
  return (long long)b * p.a_bstride + (m - b * p.rows_per_batch);
}

__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// DIRECT: the flash-layout output stage (own instantiation: sharing one register allocation
// with the generic stage costs spills)
template <bool DIRECT, int NW>
__global__ void __launch_bounds__(64 * NW, BigCfg<NW>::MINB) gemm_big_kernel(GemmParams p) {
  using C = BigCfg<NW>;
  constexpr int GNST = C::NST;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 4), wn = wave % (NW / 4);   // 64-row block wm, 128-column block wn
  const int col = lane & 31, half = lane >> 5;
  int bx = blockIdx.x, by = blockIdx.y;
  if (DIRECT && gridDim.z == 1 && gridDim.x % 8 == 0) {
    // Workgroups go to the 8 XCDs in turn (linear block L to XCD L % 8).  XCD k takes the
    // column tiles k NT/8 .. (k+1) NT/8 - 1, in phases of up to 16 tiles, each phase over all
    // row tiles: a phase's weight rows (16 x 128 x K bf16, 2 MB at K = 512) stay in the
    // XCD's L2 while its row tiles stream past, instead of every row tile re-reading the
    // whole weight from beyond L2.
    const int NT = gridDim.x, MT = gridDim.y, per = NT / 8;
    const int pw = per % 16 == 0 ? 16 : per;
    const int L = by * NT + bx, xcd = L & 7, slot = L >> 3;
    const int ph = slot / (MT * pw), rem = slot - ph * (MT * pw);
    by = rem / pw;
    bx = xcd * per + ph * pw + (rem - by * pw);
  }
  const int n0 = bx * C::BN;
  const int m0 = by * GBM;
  const int z = blockIdx.z;
  const int zo = z / p.zdiv, zi = z - zo * p.zdiv;
  const long long a_goff = zo * p.a_goff[0] + zi * p.a_goff[1];
  const long long w_goff = zo * p.w_goff[0] + zi * p.w_goff[1];
  const long long o_goff = zo * p.o_goff[0] + zi * p.o_goff[1];
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const int nst = p.K / GBK;

  // copy sources: copy j of wave w covers rows 16 (CPW w + j) + lane / 4 of its operand,
  // physical chunk lane % 4, which holds logical chunk (lane % 4) ^ ((row >> 2) & 3)
  const bf16* asrc[C::A_CPW];
  const bf16* wsrc[C::W_CPW];
#pragma unroll
  for (int j = 0; j < C::A_CPW; ++j) {
    const int t = 16 * (C::A_CPW * wave + j) + lane / 4;
    const int c = (lane & 3) ^ ((t >> 2) & 3);
    const int m = min(m0 + t, p.M - 1);
    asrc[j] = reinterpret_cast<const bf16*>(p.a) + big_a_row(p, m) * p.a_ld + a_goff + 8 * c;
  }
#pragma unroll
  for (int j = 0; j < C::W_CPW; ++j) {
    const int t = 16 * (C::W_CPW * wave + j) + lane / 4;
    const int c = (lane & 3) ^ ((t >> 2) & 3);
    const int n = min(n0 + t, N - 1);
    const int s = (n < p.seg[0].n) ? 0 : 1;
    const int nn = n - (s ? p.seg[0].n : 0);
    wsrc[j] = reinterpret_cast<const bf16*>(p.seg[s].w) + w_goff + (long long)nn * p.seg[s].w_ld + 8 * c;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto issue = [&](int st) {
    const uint32_t base = lds0 + (st % GNST) * C::STAGE;
    const int k0 = st * GBK;
#pragma unroll
    for (int j = 0; j < C::A_CPW; ++j)
      dma16(asrc[j] + k0, __builtin_amdgcn_readfirstlane(base + (C::A_CPW * wave + j) * 1024));
#pragma unroll
    for (int j = 0; j < C::W_CPW; ++j)
      dma16(wsrc[j] + k0, __builtin_amdgcn_readfirstlane(base + G_AB + (C::W_CPW * wave + j) * 1024));
  };

  // operand read: row r (= 32 blk + col within the wave's block), logical chunk 2 ks + half;
  // r mod 32 = col, so the swizzle key (r >> 2) & 3 = (col >> 2) & 3 for every block
  const int rd_base = col * 64 | ((((col >> 2) & 3) ^ half) << 4);   // XOR (2 ks) << 4 below

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  copies_begin();   // lds_dma.h, rule 1
#pragma unroll
  for (int st = 0; st < GNST - 1; ++st)
    if (st < nst) issue(st);
  for (int it = 0; it < nst; ++it) {
    const int left = nst - 1 - it;
    if (GNST >= 4 && left >= 2) wait_vmcnt<2 * C::DPW>();
    else if (left >= 1) wait_vmcnt<C::DPW>();
    else wait_vmcnt<0>();
    barrier_only();
    if (it + GNST - 1 < nst) issue(it + GNST - 1);
    const unsigned char* T = smem + (it % GNST) * C::STAGE;
    const int rb0 = opaque_int(rd_base);
    Frag<bf16> fa[2][2], fb[2][4];
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      const int off = rb0 ^ (ks << 5);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[ks][i] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + off + (64 * wm + 32 * i) * 64));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[ks][j] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + G_AB + off + (128 * wn + 32 * j) * 64));
    }
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma32(fa[ks][i], fb[ks][j], acc[i][j]);
    // issue order: the first step's 6 operand reads, then its 8 products with the second
    // step's 6 reads slotted in after the first 6, then the second step's products
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
  }
  copies_end();   // lds_dma.h, rule 3
  // The output stage reads the parameters from a copy in LDS: it indexes the segments and the
  // inverse-frequency table per lane, which on the kernel arguments would be vector loads,
  // one memory round trip each (and picking the fields by selects keeps too many registers).
  __shared__ GemmParams sp;
  if constexpr (!DIRECT) {
    static_assert(sizeof(GemmParams) % 4 == 0, "parameter copy in 4-byte words");
    const int* src = reinterpret_cast<const int*>(&p);
    int* dst = reinterpret_cast<int*>(&sp);
    for (int i = threadIdx.x; i < (int)(sizeof(GemmParams) / 4); i += 64 * NW) dst[i] = src[i];
  }
  const float* rtab = sp.rope.hi;   // hi[], then lo[] (RopeTable)
  __syncthreads();

  if constexpr (DIRECT) {
    // Flash layouts.  The wave's columns N0 .. N0 + 127 are columns j0 .. j0 + 127 of one head.
    const int N0 = n0 + 128 * wn;
    if (N0 >= N) return;
    const int s = N0 < p.seg[0].n ? 0 : 1;
    const GemmSeg& sg = p.seg[s];
    const int cc = N0 - (s ? p.seg[0].n : 0) + (int)o_goff;
    const int head = cc / sg.out_hw, j0 = cc - head * sg.out_hw;
    bf16* out = reinterpret_cast<bf16*>(sg.out);
    if (sg.layout == OUT_HEAD_T16) {
      // Row j of a head holds the tokens in perm16 order: positions 8 u .. 8 u + 7 of a
      // 16-token group are tokens 4 u .. 4 u + 3 and 8 + 4 u .. 8 + 4 u + 3, i.e. the
      // accumulator elements 8 g .. 8 g + 7 of the lanes with l / 32 = u (rows
      // 16 g + 4 u + e % 4 and 16 g + 8 + 4 u + e % 4).  One 16-byte store per lane,
      // 32-column block and 16-token group.
      const long long jstride = 32LL * sg.out_ld;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + 64 * wm + 32 * i;
        if (m >= p.M) break;
        const int b = m / p.rows_per_batch, t = m - b * p.rows_per_batch;
        bf16* base = out + ((long long)(b * sg.out_nh + head) * sg.out_hw + j0 + col) * sg.out_ld + t + 8 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[i][j][8 * g + e];
            *reinterpret_cast<bf16x8*>(base + j * jstride + 16 * g) = o;
          }
      }
    } else {
      // Head-major rows: chunk i (32 rows) goes to LDS column-major as bf16 (column stride
      // 72 B: the 16 columns of one write phase fall on distinct bank pairs); the LDS
      // transpose load then hands lane x of a 16-lane group 4 consecutive columns of row
      // r0 + x, and two loads make one 16-byte store.
      // (one buffer per wave: a wave's LDS accesses complete in issue order)
      unsigned char* buf = smem + wave * KV_BUF;
      const int g16 = lane >> 4, x16 = lane & 15;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + 64 * wm + 32 * i;
        if (m >= p.M) break;
        const int b = m / p.rows_per_batch, t = m - b * p.rows_per_batch;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[i][j][4 * q + e];
            *reinterpret_cast<bf16x4*>(buf + (32 * j + col) * KV_CS + (8 * q + 4 * half) * 2) = o;
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        bf16* base = out + ((long long)(b * sg.out_nh + head) * p.rows_per_batch + t) * sg.out_hw + j0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r0 = 16 * (u & 1), c0 = 32 * (u >> 1) + 8 * g16;
          const unsigned char* rd = buf + (c0 + (x16 >> 2)) * KV_CS + (r0 + 4 * (x16 & 3)) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(rd));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(rd + 4 * KV_CS));
          const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          *reinterpret_cast<s16x8*>(base + (r0 + x16) * sg.out_hw + c0) = v;
        }
      }
    }
  } else {
  // Epilogue per wave: its 64 x 128 block in two chunks of 32 rows.  Accumulator element
  // e of lane l in block (i, j) is out[64 wm + 32 i + 8 (e/4) + 4 (l/32) + e%4][128 wn + 32 j + l%32].
  float* Cs = reinterpret_cast<float*>(smem) + wave * 32 * G_LDC;
  auto stage = [&](auto I) {                    // chunk I with compile-time accumulator indices
    constexpr int i = decltype(I)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) Cs[(8 * (e >> 2) + 4 * half + (e & 3)) * G_LDC + 32 * j + col] = acc[i][j][e];
  };
#pragma nounroll
  for (int i = 0; i < 2; ++i) {
    if (i == 0) stage(std::integral_constant<int, 0>{});
    else stage(std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    if (p.fast_epilogue)
      epilogue_block_fast<bf16, 32, 1, 1, true>(sp, Cs, G_LDC, 0, m0 + 64 * wm + 32 * i, n0 + 128 * wn, 128, o_goff,
                                                lane, rtab);
    else
      epilogue_block<bf16, true>(sp, Cs, G_LDC, m0 + 64 * wm + 32 * i, 32, n0 + 128 * wn, 128, o_goff, lane, 64, rtab);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
  }
}


// ---- Flash-layout K/V up-projection, persistent form ----
//
// The prefill keys / values (the output stage of DIRECT above) from 256 x 256 tiles held by
// four waves of 128 x 128 (4 x 4 accumulator blocks each, in the accumulation registers):
// per 16-wide k-step a wave reads 8 operand fragments for 16 products, two thirds of the LDS
// operand bytes per product of the 64 x 128 wave tile, whose two waves per SIMD left the
// main loop bound by LDS traffic.  One workgroup per CU walks its tiles with the copy
// pipeline running across tile boundaries: while a tile's results are stored, the next
// tile's first two stages are already in flight, so no workgroup start, operand prologue or
// drain sits between tiles.  The key transposes use a per-wave LDS buffer of their own.
//
// The stores of a tile are in flight together with the next tile's copies (the exception for
// stores in lds_dma.h: a wait for "all but the newest N copies" stays exact for the copies).
// They are non-temporal: the 1 GB of keys and values streams past the L2, which keeps the
// operand tiles instead (804 -> 379 MB fetched per launch at B=4, S=4096, same time).
constexpr int KVP_T = 256;                         // tile rows and columns
constexpr int KVP_NST = 3;                         // LDS stages
constexpr int KVP_AB = KVP_T * GBK * 2;            // bytes per operand per stage (16 KB)
constexpr int KVP_STAGE = 2 * KVP_AB;
constexpr int KVP_CPW = KVP_AB / 1024 / 4;         // copies per wave per operand per stage
constexpr int KVP_DPW = 2 * KVP_CPW;
constexpr size_t KVP_TR = (size_t)KVP_NST * KVP_STAGE;   // key transpose buffers follow the stages
constexpr size_t KVP_LDS = KVP_TR + 4 * KV_BUF;
static_assert(KVP_LDS <= 160 * 1024, "LDS budget");
static_assert(128 * 64 <= KV_BUF, "the value transpose (128 rows of 64 bytes) fits a key transpose buffer");

// Tile i of workgroup w (tiles: mt row tiles x nt column tiles).  With whole XCD groups,
// XCD x (workgroups w = x mod 8) takes the column tiles x nt/8 .. (x+1) nt/8 - 1 in phases
// of up to 8, each phase over all row tiles, and its workgroups deal the XCD's list out
// round-robin: the XCD's 32 workgroups then hold a few row tiles and one phase's weight
// rows (8 x 256 x K bf16, 2 MB at K = 512) in its L2.
struct KvpOrder {
  int mt, nt, G, xcd, j, gx, per, pw, count;
  __device__ KvpOrder(int mt_, int nt_, int G_, int w) : mt(mt_), nt(nt_), G(G_) {
    if (G % 8 == 0 && nt % 8 == 0) {
      xcd = w & 7;
      j = w >> 3;
      gx = G >> 3;
      per = nt >> 3;
      pw = per % 8 == 0 ? 8 : per;
      const int len = per * mt;
      count = j < len ? (len - 1 - j) / gx + 1 : 0;
    } else {
      xcd = -1;
      j = w;
      count = j < mt * nt ? (mt * nt - 1 - j) / G + 1 : 0;
    }
  }
  __device__ void tile(int i, int& by, int& bx) const {
    if (xcd >= 0) {
      const int e = j + gx * i;
      const int ph = e / (mt * pw), rem = e - ph * (mt * pw);
      by = rem / pw;
      bx = xcd * per + ph * pw + (rem - by * pw);
    } else {
      const int t = j + G * i;
      by = t / nt;
      bx = t - by * nt;
    }
  }
};

__global__ void __launch_bounds__(256, 1) gemm_kv_kernel(GemmParams p, int mt, int nt) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;           // 128-row block wm, 128-column block wn
  const int col = lane & 31, half = lane >> 5;
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  const int nst = p.K / GBK;
  const KvpOrder ord(mt, nt, gridDim.x, blockIdx.x);
  const int total = ord.count * nst;                 // stages this workgroup consumes
  if (total == 0) return;

  // copy j of wave w covers rows 16 (KVP_CPW w + j) + lane / 4 of each operand, physical
  // chunk lane % 4 (logical chunk (lane % 4) ^ ((row >> 2) & 3))
  const bf16* asrc[KVP_CPW];
  const bf16* wsrc[KVP_CPW];
  auto set_src = [&](int i) {
    int by, bx;
    ord.tile(i, by, bx);
#pragma unroll
    for (int j = 0; j < KVP_CPW; ++j) {
      const int t = 16 * (KVP_CPW * wave + j) + lane / 4;
      const int c = (lane & 3) ^ ((t >> 2) & 3);
      const int m = min(by * KVP_T + t, p.M - 1);
      asrc[j] = reinterpret_cast<const bf16*>(p.a) + big_a_row(p, m) * p.a_ld + 8 * c;
      const int n = min(bx * KVP_T + t, N - 1);
      const int s = (n < p.seg[0].n) ? 0 : 1;
      const int nn = n - (s ? p.seg[0].n : 0);
      wsrc[j] = reinterpret_cast<const bf16*>(p.seg[s].w) + (long long)nn * p.seg[s].w_ld + 8 * c;
    }
  };
  const uint32_t lds0 = lds_addr_of(smem);
  // issue position: stage gi of the flattened (tile, k-step) sequence, tile ii, k-step ik
  int gi = 0, ii = 0, ik = 0;
  auto issue_next = [&]() {
    const uint32_t base = lds0 + (gi % KVP_NST) * KVP_STAGE;
    const int k0 = ik * GBK;
#pragma unroll
    for (int j = 0; j < KVP_CPW; ++j)
      dma16(asrc[j] + k0, __builtin_amdgcn_readfirstlane(base + (KVP_CPW * wave + j) * 1024));
#pragma unroll
    for (int j = 0; j < KVP_CPW; ++j)
      dma16(wsrc[j] + k0, __builtin_amdgcn_readfirstlane(base + KVP_AB + (KVP_CPW * wave + j) * 1024));
    ++gi;
    if (++ik == nst) {
      ik = 0;
      if (++ii < ord.count) set_src(ii);
    }
  };

  const int rd_base = col * 64 | ((((col >> 2) & 3) ^ half) << 4);   // as in gemm_big_kernel
  f32x16 acc[4][4];

  copies_begin();   // lds_dma.h, rule 1 (nothing compiler-visible is in flight)
  set_src(0);
  issue_next();
  if (total > 1) issue_next();
  // one k-step of stage gs; FIRST: the tile's first, whose products start from zero (the
  // accumulators are not live across tiles, which keeps the allocator from moving them)
  auto step = [&](int gs, auto first_c) {
    constexpr bool FIRST = decltype(first_c)::value;
    if (gs + 1 < total) wait_vmcnt<KVP_DPW>();
    else wait_vmcnt<0>();
    barrier_only();
    if (gi < total) issue_next();
    const unsigned char* T = smem + (gs % KVP_NST) * KVP_STAGE;
    const int rb0 = opaque_int(rd_base);
    Frag<bf16> fa[2][4], fb[2][4];
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      const int off = rb0 ^ (ks << 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[ks][i] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + off + (128 * wm + 32 * i) * 64));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[ks][j] = frag_load<bf16>(reinterpret_cast<const bf16*>(T + KVP_AB + off + (128 * wn + 32 * j) * 64));
    }
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma32(fa[ks][i], fb[ks][j], (FIRST && ks == 0) ? f32x16{} : acc[i][j]);
    // the first k-step's 8 reads, then its 16 products with the second k-step's 8 reads
    // slotted in after the first 8, then the second k-step's products
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
  };
  int gs = 0;
  for (int ti = 0; ti < ord.count; ++ti) {
    step(gs++, std::true_type{});
    for (int it = 1; it < nst; ++it) step(gs++, std::false_type{});

    // ---- output stage of tile ti (flash layouts; see gemm_big_kernel's DIRECT stage) ----
    // Each accumulator block moves to VGPRs at an explicit point (the empty asm with the memory
    // clobber keeps the move after the previous block's stores): left to itself the compiler
    // copies all 256 accumulators out at once and spills.
    int by, bx;
    ord.tile(ti, by, bx);
    const int N0 = bx * KVP_T + 128 * wn;
    if (N0 < N) {
      const int s = N0 < p.seg[0].n ? 0 : 1;
      const GemmSeg& sg = p.seg[s];
      const int cc = N0 - (s ? p.seg[0].n : 0);
      const int head = cc / sg.out_hw, j0 = cc - head * sg.out_hw;
      bf16* out = reinterpret_cast<bf16*>(sg.out);
      const bool vt = sg.layout == OUT_HEAD_T16;
      unsigned char* buf = smem + KVP_TR + wave * KV_BUF;
      const int g16 = lane >> 4, x16 = lane & 15;
      auto chunk = [&](auto I, int m) {
        constexpr int i = decltype(I)::value;
        const int b = m / p.rows_per_batch, t = m - b * p.rows_per_batch;
        if (vt) {
          // Values: the chunk's [128 features][32 tokens] block goes through the wave's LDS
          // buffer (rows of 64 bytes, 16-byte pieces XOR-swizzled by (row >> 1) & 3: both the
          // writes and the reads below are free of bank conflicts), so that 4 lanes store one
          // feature row's 64 bytes together; 16-byte pieces scattered over 32 rows straight
          // from the accumulators cost the kernel a quarter of its time.  Piece 2 g + half of a
          // row is perm16 positions 8 half .. 8 half + 7 of token group g, i.e. accumulator
          // elements 8 g .. 8 g + 7.
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            asm volatile("" : "+v"(acc[i][j])::"memory");
            const int row = 32 * j + col;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              bf16x8 o;
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[i][j][8 * g + e];
              *reinterpret_cast<bf16x8*>(buf + row * 64 + (((2 * g + half) ^ ((row >> 1) & 3)) << 4)) = o;
            }
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
          __builtin_amdgcn_wave_barrier();
          bf16* base = out + ((long long)(b * sg.out_nh + head) * sg.out_hw + j0) * sg.out_ld + t + 8 * (lane & 3);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int row = 16 * k + (lane >> 2);
            const s16x8 v = *reinterpret_cast<const s16x8*>(buf + row * 64 + (((lane & 3) ^ ((row >> 1) & 3)) << 4));
            __builtin_nontemporal_store(v, reinterpret_cast<s16x8*>(base + (long long)row * sg.out_ld));
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);   // the reads are done before the next chunk's writes
          __builtin_amdgcn_wave_barrier();
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            asm volatile("" : "+v"(acc[i][j])::"memory");
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              bf16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[i][j][4 * q + e];
              *reinterpret_cast<bf16x4*>(buf + (32 * j + col) * KV_CS + (8 * q + 4 * half) * 2) = o;
            }
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
          __builtin_amdgcn_wave_barrier();
          bf16* base = out + ((long long)(b * sg.out_nh + head) * p.rows_per_batch + t) * sg.out_hw + j0;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r0 = 16 * (u & 1), c0 = 32 * (u >> 1) + 8 * g16;
            const unsigned char* rd = buf + (c0 + (x16 >> 2)) * KV_CS + (r0 + 4 * (x16 & 3)) * 2;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(rd));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(rd + 4 * KV_CS));
            const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<s16x8*>(base + (r0 + x16) * sg.out_hw + c0));
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);   // the reads are done before the next chunk's writes
          __builtin_amdgcn_wave_barrier();
        }
      };
      const int mw = by * KVP_T + 128 * wm;
      if (mw < p.M) chunk(std::integral_constant<int, 0>{}, mw);
      if (mw + 32 < p.M) chunk(std::integral_constant<int, 1>{}, mw + 32);
      if (mw + 64 < p.M) chunk(std::integral_constant<int, 2>{}, mw + 64);
      if (mw + 96 < p.M) chunk(std::integral_constant<int, 3>{}, mw + 96);
    }
  }
  copies_end();   // lds_dma.h, rule 3
}

}  // namespace

bool gemm_big_supported(const GemmParams& p, int groups) {
  (void)groups;
  if (p.w_kmajor || p.M < GBM || p.K % GBK != 0 || p.a_ld % 8 != 0) return false;
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  if (N < 128) return false;
  for (int i = 0; i < 2; ++i)
    if (p.a_goff[i] % 8 != 0 || p.w_goff[i] % 8 != 0) return false;
  if ((reinterpret_cast<uintptr_t>(p.a) & 15) != 0) return false;
  int start = 0;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (sg.w_ld % 8 != 0 || (reinterpret_cast<uintptr_t>(sg.w) & 15) != 0) return false;
    if (sg.rope == ROPE_INTERLEAVED && (start % 2 != 0 || sg.rope_d % 2 != 0)) return false;
    if (sg.rope == ROPE_HALFSPLIT && (start % 128 != 0 || sg.rope_d > 128 || 128 % sg.rope_d != 0)) return false;
    start += sg.n;
  }
  return true;
}

bool gemm_fast_epilogue_ok(const GemmParams& p, int groups) {
  auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
  if (p.seg[0].n % 8 != 0) return false;
  for (int i = 0; i < 2; ++i)
    if (p.o_goff[i] % 8 != 0) return false;
  (void)groups;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (!al16(sg.out)) return false;
    if (sg.rope != ROPE_OFF && sg.rope_d % 8 != 0) return false;
    if (sg.rope == ROPE_HALFSPLIT && (sg.rope_d / 2) % 8 != 0) return false;
    if (sg.layout == OUT_ROWS) {
      if (sg.out_hw % 8 != 0 || sg.out_hs % 8 != 0 || sg.out_ld % 8 != 0) return false;
    } else if (sg.layout == OUT_HEAD_MAJOR) {
      if (sg.out_hw % 8 != 0) return false;
    } else {
      if (sg.out_f32 || sg.out_ld % 16 != 0 || p.rows_per_batch % 32 != 0) return false;
    }
  }
  return true;
}

// Flash-layout output stage: bf16 head-major / transposed segments without rotation, every
// 128-column block inside one head of one segment, 32-row chunks inside one sequence.
static bool kv_direct_ok(const GemmParams& p) {
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  if (N % 128 != 0 || p.rows_per_batch % 32 != 0 || p.M % 32 != 0) return false;
  for (int i = 0; i < 2; ++i)
    if (p.o_goff[i] % 128 != 0) return false;
  for (int i = 0; i < p.nseg; ++i) {
    const GemmSeg& sg = p.seg[i];
    if (sg.layout == OUT_ROWS || sg.out_f32 || sg.rope != ROPE_OFF) return false;
    if (sg.n % 128 != 0 || sg.out_hw % 128 != 0) return false;
  }
  return true;
}

hipError_t launch_gemm_big(const GemmParams& pin, int groups, hipStream_t s) {
  GemmParams p = pin;
  p.fast_epilogue = gemm_fast_epilogue_ok(p, groups) ? (kv_direct_ok(p) ? 2 : 1) : 0;
  const int N = p.seg[0].n + (p.nseg > 1 ? p.seg[1].n : 0);
  // The flash-layout stage (the prefill K/V up-projection) takes 256 x 128 tiles, two
  // workgroups per CU (820 -> 780 us at B=4, S=4096); the other projections measured the
  // same or slower that way and keep 256 x 256.
  if (p.fast_epilogue == 2 && groups == 1 && N % KVP_T == 0) {
    // persistent form: one workgroup per CU (or per tile when there are fewer tiles)
    const int mt = cdiv(p.M, KVP_T), nt = N / KVP_T;
    const int G = min(mt * nt, device_cu_count());
    hipLaunchKernelGGL(gemm_kv_kernel, dim3(G), dim3(256), KVP_LDS, s, p, mt, nt);
    return hipGetLastError();
  }
  if (p.fast_epilogue == 2) {
    using C = BigCfg<4>;
    dim3 grid(cdiv(N, C::BN), cdiv(p.M, GBM), groups);
    hipLaunchKernelGGL((gemm_big_kernel<true, 4>), grid, dim3(64 * 4), C::LDS, s, p);
  } else {
    using C = BigCfg<8>;
    dim3 grid(cdiv(N, C::BN), cdiv(p.M, GBM), groups);
    hipLaunchKernelGGL((gemm_big_kernel<false, 8>), grid, dim3(64 * 8), C::LDS, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
