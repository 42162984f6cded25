// MFMA GEMM core of libdp: y[m, n] = sum_k A[m, k] * Wt[n, k] (+ bias[n]).
//
// Two operand sources share one kernel body:
//  - dense rows (the Q/K/V/output projections of the rank's own tokens);
//  - the implicit im2col of a 3x3 stride-1 convolution over the rank's row
//    band, where the row above the band comes from the stale `halo_top`
//    buffer, the row below from `halo_bot`, and out-of-image columns are zero
//    ("OTIL for SDXL on 4x L40S", "What is implemented where": the displaced
//    conv; "Benchmarking DistVAE", "Glossary": halo rows).
// Reduction index of the conv: k = tap * Cin + c with tap = (dy+1)*3 + (dx+1),
// matching the [Cout, 3, 3, Cin] weight layout, so weight rows are K-contiguous.
//
// bf16 path (gfx950): a block of NW waves (4 in every shape used) computes one
// output tile of a shape chosen per problem so the tiles spread evenly over the
// CUs (128x128, 64x128, 64x64, 160x128, 96x128 or 128x160); tiles sharing A
// rows are dealt to one XCD.  K moves through an LDS ring by direct global->LDS loads issued ahead, 64
// of K per stage (128-byte rows, one L2 line each) or 32 when K or Cin is not a
// multiple of 64.  LDS rows are XOR-swizzled.  Each wave owns a quarter of the tile as
// v_mfma_f32_32x32x16_bf16 blocks computed as (W rows) x (A rows)^T, so an
// accumulator lane holds 4 consecutive output channels of one output row and
// the epilogue writes 8-byte runs.
// f32 path: a plain LDS-tiled FMA kernel (correctness path for fp32 shares).
#include <algorithm>
#include <cmath>

#include "dp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;            // narrowest reduction slice (64 bytes of bf16 per row)
constexpr int kStages = 3;         // LDS ring depth of the narrow-slice fallback
constexpr int kXcds = 8;

// Zero page read by padding rows of the implicit im2col (columns outside the
// image, rows beyond a NULL halo, rows past M).  Such rows are re-pointed at
// the page at every tap and advance at most Cin*2 <= 4096 bytes within it.
__device__ __attribute__((aligned(256))) unsigned char g_zero_page[4096 + 256];

struct ConvGeom {
  const bf16_t* x;
  const bf16_t* halo_top;
  const bf16_t* halo_bot;
  int h, W, Cin;
};

// Output columns come in segments of seg_n (n_seg of them, N = n_seg * seg_n).
// Column n of segment s = n / seg_n takes its weight row from wts[s] (row
// n - s*seg_n) and its result goes to outs[s], column n - s*seg_n (leading
// dimension seg_n), output row (m / rpg) * grp_rows[s] + row_off[s] + m % rpg.
// A plain GEMM is one segment with rpg = grp_rows = M and row_off = 0; the
// fused Q/K/V projection is three, K and V landing at rows t0 + i of every
// batch item's full-image buffer.
struct OutMap {
  const void* wts[3];
  void* outs[3];
  int n_seg, seg_n, rpg;
  int grp_rows[3], row_off[3];
};

__device__ __forceinline__ int64_t out_row(const OutMap& o, int s, int m) {
  const int g = m / o.rpg;
  return static_cast<int64_t>(g) * o.grp_rows[s] + o.row_off[s] + (m - g * o.rpg);
}

struct GemmArgs {
  const bf16_t* a;     // dense rows [M, K] (projections)
  ConvGeom geo;        // implicit im2col (conv)
  OutMap map;          // weights [N, K] by segment, outputs
  const float* bias;   // [N] or null
  int M, N, K;
  int tiles_m, tiles_n, units, units_per_xcd;
  // conv with GroupNorm sums only:
  float2* gpart;       // per (tile row, batch segment, tile column, group slot) partials
  float* gsums;        // [B][G][2] output
  int gT;              // output tokens per batch item
  int G, Cg, slots;
};

// Sum of v over `lanes` adjacent lanes (a power of two <= 64) by a fixed xor
// butterfly: every lane ends with the same, order-fixed total.
__device__ __forceinline__ float2 lane_sum(float2 v, int lanes) {
  for (int off = 1; off < lanes; off <<= 1) {
    v.x += __shfl_xor(v.x, off, 64);
    v.y += __shfl_xor(v.y, off, 64);
  }
  return v;
}
// Largest power of two <= min(n, 64), at least 1.
__device__ __forceinline__ int pow2_lanes(int n) {
  n = n < 1 ? 1 : (n > 64 ? 64 : n);
  return 1 << (31 - __clz(n));
}

// Tile rows [lo, hi] holding the output rows of batch item b.
__device__ __forceinline__ int2 batch_tile_rows(int b, int gT, int BM) {
  return make_int2(static_cast<int>((static_cast<int64_t>(b) * gT) / BM),
                   static_cast<int>(((static_cast<int64_t>(b) + 1) * gT - 1) / BM));
}

// LDS rows of 64 bytes (BK = 32) or 128 bytes (BK = 64): 16-byte chunk c of
// row r lives in slot c ^ swz(r), chosen so the 16 rows one operand read
// touches per LDS cycle (same chunk) hit 16 distinct 4-bank groups of the 64
// banks, and the DMA writes (1 KB contiguous) are conflict-free.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  return BK == 64 ? (row >> 1) & 7 : (row >> 2) & 3;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is written on purpose; nothing else here uses it
// 16 bytes per lane straight into LDS at M0 + 16*lane (global_load_lds_dwordx4),
// issued as inline assembly so completion is tracked only by the explicit
// vmcnt waits of the k loop (compiler-inserted waits can only over-wait).
__device__ __forceinline__ void gdma16(const void* gsrc, unsigned int m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(gsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int S>
struct Stage {
  static constexpr int value = S;
};

// One block computes a BM x BN output tile with NW waves arranged WGM x WGN
// (WGM * WGN = NW); each wave owns (BM/WGM) x (BN/WGN) as 32 x 32 MFMA blocks
// computed as (W rows) x (A rows)^T, so an accumulator lane holds 4
// consecutive output channels of one output row.  K advances BK (32 or 64) per
// stage through an ST-stage LDS ring.
//
// DMA: a stage is BM A rows followed by BN W rows of BK bf16 (RB = 2*BK bytes,
// one L2 line when BK = 64), cut into 1 KB slabs; slab s is loaded by wave
// s % NW with one instruction in which RB/16 consecutive lanes fetch one row.
// When the slab count is not a multiple of NW the first waves own one slab
// more, and each wave waits on its own outstanding count.
template <int BM, int BN, int WGM, int NW, int BK, int ST, int OCC, bool CONV, bool GNS = false>
__global__ void __launch_bounds__(64 * NW, OCC) gemm_bf16(GemmArgs g) {
  constexpr int WGN = NW / WGM;
  constexpr int RB = BK * 2, LPR = RB / 16, RPS = 64 / LPR;  // row bytes, lanes per row, rows per slab
  constexpr int kABytes = BM * RB;
  constexpr int kStageBytes = (BM + BN) * RB;
  constexpr int kASl = BM / RPS, kSl = (BM + BN) / RPS;    // slabs: A first, then W
  constexpr int kJ = (kSl + NW - 1) / NW;                  // slab slots per wave
  constexpr int kRem = kSl % NW;                           // waves < kRem own kJ slabs, the rest kJ - 1
  constexpr int kDmaHi = kJ, kDmaLo = kRem ? kJ - 1 : kJ;  // DMAs per stage per wave
  constexpr int kQ = BK / 16;                              // 16-wide MFMA k steps per stage
  constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32;
  static_assert(BK == 32 || BK == 64, "slice width");
  static_assert(ST >= 2 && ST <= 4, "the k loop below unrolls at most four ring stages");
  static_assert(WGM * WGN == NW && WM % 32 == 0 && WN % 32 == 0 && BM % RPS == 0 && BN % RPS == 0, "tile");
  __shared__ __attribute__((aligned(1024))) char lds[ST * kStageBytes];

  const int u = (blockIdx.x % kXcds) * g.units_per_xcd + blockIdx.x / kXcds;
  if (u >= g.units) return;
  const int tn = u % g.tiles_n, tm = u / g.tiles_n;  // tiles sharing A rows stay on one XCD
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, gq = lane >> 5;
  const bool dma_hi = kRem == 0 || wave < kRem;

  const unsigned int lds0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned int>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds)) +
      wave * 1024);
  const char* src[kJ];
  int a_b[kJ], a_i[kJ], a_c[kJ], a_chunk[kJ];
  bool has[kJ], is_a[kJ], a_ok[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int sl = NW * j + wave;
    has[j] = sl < kSl;
    is_a[j] = sl < kASl;
    const int row = RPS * (is_a[j] ? sl : sl - kASl) + lane / LPR;
    const int chunk = (lane % LPR) ^ swz<BK>(row);
    a_chunk[j] = chunk;
    a_b[j] = a_i[j] = a_c[j] = 0;
    a_ok[j] = false;
    if (!is_a[j]) {
      const int n = min(n0 + row, g.N - 1);  // rows past N repeat the last one; never stored
      const int seg = n / g.map.seg_n;
      src[j] = reinterpret_cast<const char*>(static_cast<const bf16_t*>(g.map.wts[seg]) +
                                             static_cast<int64_t>(n - seg * g.map.seg_n) * g.K) +
               chunk * 16;
    } else {
      const int m = m0 + row;
      a_ok[j] = m < g.M;
      if constexpr (CONV) {
        const int hw = g.geo.h * g.geo.W;
        const int mm = a_ok[j] ? m : 0;
        a_b[j] = mm / hw;
        const int rem = mm - a_b[j] * hw;
        a_i[j] = rem / g.geo.W;
        a_c[j] = rem - a_i[j] * g.geo.W;
        src[j] = nullptr;
      } else {
        // rows past M repeat the last one; never stored
        src[j] = reinterpret_cast<const char*>(g.a + static_cast<int64_t>(min(m, g.M - 1)) * g.K) + chunk * 16;
      }
    }
  }
  // conv: point the A rows at the source pixel of tap `tap` (channel 0), or the zero page
  auto conv_rows = [&](int tap) {
    const int dy = tap / 3 - 1, dx = tap % 3 - 1;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (!is_a[j]) continue;
      const int row = a_i[j] + dy, col = a_c[j] + dx;
      const bf16_t* p = nullptr;
      if (a_ok[j] && col >= 0 && col < g.geo.W) {
        if (row < 0) {
          if (g.geo.halo_top) p = g.geo.halo_top + (static_cast<int64_t>(a_b[j]) * g.geo.W + col) * g.geo.Cin;
        } else if (row >= g.geo.h) {
          if (g.geo.halo_bot) p = g.geo.halo_bot + (static_cast<int64_t>(a_b[j]) * g.geo.W + col) * g.geo.Cin;
        } else {
          p = g.geo.x + ((static_cast<int64_t>(a_b[j]) * g.geo.h + row) * g.geo.W + col) * g.geo.Cin;
        }
      }
      src[j] = (p ? reinterpret_cast<const char*>(p) : reinterpret_cast<const char*>(g_zero_page)) +
               a_chunk[j] * 16;
    }
  };

  const int n_kt = g.K / BK;
  const int kpt = CONV ? g.geo.Cin / BK : n_kt;  // stages per conv tap
  // Issues the next slice into stage st; pointers advance one slice (RB bytes)
  // per issue, and conv rows are re-pointed at each tap.
  int tap_next = 0, in_tap = 0;
  auto issue = [&](int st) {
    if constexpr (CONV) {
      if (in_tap == 0) conv_rows(tap_next);
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (!has[j]) continue;
      gdma16(src[j], lds0 + st * kStageBytes + j * (NW * 1024));
      src[j] += RB;
    }
    if constexpr (CONV) {
      if (++in_tap == kpt) {
        in_tap = 0;
        ++tap_next;
      }
    }
  };

  // ---- operand offsets: A rows of this wave, W rows of this wave
  int aoff[MB][kQ], boff[NB][kQ];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int s = 0; s < kQ; ++s) {
      const int row = wm * WM + 32 * i + l32;
      aoff[i][s] = row * RB + (((2 * s + gq) ^ swz<BK>(row)) << 4);
    }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int s = 0; s < kQ; ++s) {
      const int row = wn * WN + 32 * i + l32;
      boff[i][s] = kABytes + row * RB + (((2 * s + gq) ^ swz<BK>(row)) << 4);
    }

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto step = [&](auto stage_c, int kt) {
    constexpr int S = decltype(stage_c)::value;
    if (kt + ST - 2 < n_kt) {  // stage kt done, later ones may be in flight
      if (dma_hi) wait_vm<(ST - 2) * kDmaHi>();
      else wait_vm<(ST - 2) * kDmaLo>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();  // stage kt visible; the stage of kt-1 is free
    if (kt + ST - 1 < n_kt) issue((S + ST - 1) % ST);
    // operands of k step q+1 are read from LDS before the MFMAs of step q, so
    // LDS latency hides behind the MFMAs
    bf16x8 wa[2][NB], xb[2][MB];
    auto frag = [&](int q, int b) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        wa[b][i] = *reinterpret_cast<const bf16x8*>(lds + S * kStageBytes + boff[i][q]);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        xb[b][j] = *reinterpret_cast<const bf16x8*>(lds + S * kStageBytes + aoff[j][q]);
    };
    frag(0, 0);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (q + 1 < kQ) frag(q + 1, (q + 1) & 1);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[q & 1][i], xb[q & 1][j], acc[i][j], 0, 0, 0);
    }
    // Keep that order through instruction scheduling (which would otherwise
    // sink each read next to its MFMA): the reads of step 0, then per step one
    // read of the next step after each MFMA.
    constexpr int kR = NB + MB, kP = NB * MB;
    __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);  // DS reads
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (q + 1 < kQ) {
#pragma unroll
        for (int t = 0; t < kP; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (t < kR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (kR > kP) __builtin_amdgcn_sched_group_barrier(0x100, kR > kP ? kR - kP : 1, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, kP, 0);
      }
    }
  };

#pragma unroll
  for (int p = 0; p < ST - 1; ++p)
    if (p < n_kt) issue(p);
  for (int kt = 0; kt < n_kt; kt += ST) {
    step(Stage<0>{}, kt);
    if (kt + 1 < n_kt) step(Stage<1>{}, kt + 1);
    if constexpr (ST > 2) {
      if (kt + 2 < n_kt) step(Stage<2 % ST>{}, kt + 2);
    }
    if constexpr (ST > 3) {
      if (kt + 3 < n_kt) step(Stage<3 % ST>{}, kt + 3);
    }
  }

  // Bias of the lane's 16 channels of column block i, loaded into registers
  // once: read inside the store loop, the compiler reloads it (and waits for
  // it) after every store, one memory round trip per row block.
  auto bias_of = [&](int i, float (&bq)[4][4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bq[q][e] = g.bias ? g.bias[min(n0 + wn * WN + 32 * i + 8 * q + 4 * gq + e, g.N - 1)] : 0.f;
  };

  // Epilogue through LDS.  Each wave's accumulators hold 4 consecutive
  // channels of one output row per lane, so stores straight from registers
  // write 16 bytes to each of 32 rows per instruction: partial cache lines,
  // which cost a third of a short-K projection.  Instead the tile (bias
  // added, rounded to bf16) goes to LDS (the ring is free once every wave is
  // past its last operand read), rows padded by 16 bytes, and leaves in
  // 16-byte chunks, consecutive threads on consecutive chunks of a row, by
  // nontemporal stores (outputs of 18 MB and more do not stay in a 4 MB L2;
  // the next op reads them from the last-level cache either way).
  constexpr int kTileStride = BN * 2 + 16;  // bytes per tile row
  // GroupNorm column sums: one thread per channel pair and row part
  constexpr int kPairs = BN / 2, kParts = (64 * NW) / kPairs > 0 ? (64 * NW) / kPairs : 1;
  static_assert(BM * kTileStride + (GNS ? (2 + 2 * kParts) * BN * 8 : 0) <= ST * kStageBytes,
                "output tile in LDS");
  __syncthreads();

  // lane holds rows n = 8*(e/4) + 4*gq + e%4 of column m = l32
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float bq[4][4];
    bias_of(i, bq);
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int ml = wm * WM + 32 * j + l32;
      const int nl = wn * WN + 32 * i;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] + bq[q][e];
        const u32x2 packed = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(lds + ml * kTileStride + (nl + 8 * q + 4 * gq) * 2) = packed;
      }
    }
  }
  __syncthreads();
  {
    constexpr int kChunks = BN / 8;  // 16-byte chunks per tile row
    const int rows = min(BM, g.M - m0), cols = min(BN, g.N - n0);
    for (int e = tid; e < rows * kChunks; e += 64 * NW) {
      const int r = e / kChunks, c = (e - r * kChunks) * 8;
      if (c >= cols) continue;
      const int m = m0 + r, n = n0 + c;
      const int seg = n / g.map.seg_n;  // 8 channels never straddle a segment (seg_n % 32 == 0)
      bf16_t* yrow = static_cast<bf16_t*>(g.map.outs[seg]) + out_row(g.map, seg, m) * g.map.seg_n -
                     seg * g.map.seg_n;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(lds + r * kTileStride + c * 2),
                                  reinterpret_cast<u32x4*>(yrow + n));
    }
  }

  if constexpr (GNS) {
    // GroupNorm sums of the stored (bf16-rounded) outputs, from the tile copy
    // in LDS.  A tile spans at most two batch items (segments 0 and 1, since
    // gT >= BM).  Per channel pair and row part, one thread sums its rows of
    // each segment in row order; the parts are then added in part order, the
    // block sums the channels of each group its columns touch, in a fixed
    // order, and stores one partial per (batch segment, group slot); the
    // fold launch that follows adds them into gsums.
    float2* chan = reinterpret_cast<float2*>(lds + BM * kTileStride);  // [2][BN]
    float2* parts = chan + 2 * BN;                                     // [kParts][2][BN]
    const int b0 = m0 / g.gT;
    const int rows = min(BM, g.M - m0);
    const int nseg = (m0 + rows - 1) / g.gT - b0 + 1;
    const int split = min(rows, (b0 + 1) * g.gT - m0);  // rows [0, split) belong to batch item b0
    {
      const int cp = tid % kPairs, pi = tid / kPairs;
      if (pi < kParts) {
        const char* col = lds + cp * 4;
        for (int sg = 0; sg < nseg; ++sg) {
          const int ra = sg ? split : 0, rb = sg ? rows : split;
          const int len = (rb - ra + kParts - 1) / kParts;
          const int r0 = ra + pi * len, r1 = min(rb, r0 + len);
          float a1 = 0.f, a2 = 0.f, b1 = 0.f, b2 = 0.f;  // channels 2cp and 2cp + 1
#pragma unroll 4
          for (int r = r0; r < r1; ++r) {
            const unsigned int w2 = *reinterpret_cast<const unsigned int*>(col + r * kTileStride);
            const float y0 = bf16_lo(w2), y1 = bf16_hi(w2);
            a1 += y0;
            a2 = fmaf(y0, y0, a2);
            b1 += y1;
            b2 = fmaf(y1, y1, b2);
          }
          parts[(pi * 2 + sg) * BN + 2 * cp] = make_float2(a1, a2);
          parts[(pi * 2 + sg) * BN + 2 * cp + 1] = make_float2(b1, b2);
        }
      }
    }
    __syncthreads();
    for (int e = tid; e < nseg * BN; e += 64 * NW) {
      const int sg = e / BN, c = e - sg * BN;
      float2 acc2 = make_float2(0.f, 0.f);
#pragma unroll
      for (int p = 0; p < kParts; ++p) {
        const float2 v = parts[(p * 2 + sg) * BN + c];
        acc2.x += v.x;
        acc2.y += v.y;
      }
      chan[sg * BN + c] = acc2;
    }
    __syncthreads();
    const int n1 = min(n0 + BN, g.N);
    const int g_lo = n0 / g.Cg, nslots = (n1 - 1) / g.Cg - g_lo + 1;
    {
      // `sl` adjacent lanes per (segment, slot): lane l takes the slot's
      // channels l, l + sl, ... (all WGM wave rows each), then a lane tree
      const int sl = pow2_lanes((64 * NW) / (nseg * nslots));
      for (int t = tid; t < ((nseg * nslots * sl + 63) / 64) * 64; t += 64 * NW) {
        const int st = t / sl, l = t % sl;
        float2 acc2 = make_float2(0.f, 0.f);
        if (st < nseg * nslots) {
          const int sg = st / nslots, jj = st - sg * nslots, gi = g_lo + jj;
          const int c0 = max(gi * g.Cg, n0), c1 = min((gi + 1) * g.Cg, n1);
          for (int c = c0 + l; c < c1; c += sl) {
            const float2 v = chan[sg * BN + c - n0];
            acc2.x += v.x;
            acc2.y += v.y;
          }
        }
        acc2 = lane_sum(acc2, sl);
        if (st < nseg * nslots && l == 0) {
          const int sg = st / nslots, jj = st - sg * nslots;
          g.gpart[((static_cast<int64_t>(tm) * 2 + sg) * g.tiles_n + tn) * g.slots + jj] = acc2;
        }
      }
    }
  }
}

// The fold of the conv's tile partials into gsums, a launch of its own after
// the conv: one block per (group, batch item).  The group's partials are the
// slot it owns in each (tile row, tile column) of the item's tile rows and the
// group's tile columns; lane q takes entries q, q + 256, ... in (tile row,
// tile column) order (eight loads in flight per pass when there are more
// entries than lanes), then each wave adds its lanes by DPP steps within
// 16-lane rows and its four row totals in order, and thread 0 the four waves
// in order: one fixed order for a given shape.
constexpr int kFoldThreads = 256;

// The partial of entry e (tile row r0 + e / ntn, tile column tn_lo + e % ntn)
// of group gi for batch item b; slot0 is gi's slot index in column tn_lo.
template <int BM, int BN>
__device__ __forceinline__ float2 fold_entry(const GemmArgs& g, int e, int r0, int tn_lo, int ntn, int gi,
                                             int slot0, int64_t first_row) {
  const int rr = ntn == 1 ? e : e / ntn, c = e - rr * ntn;
  const int tr = r0 + rr, tc = tn_lo + c;
  // a tile row that starts in batch item b - 1 holds b in its segment 1
  const int sgt = static_cast<int64_t>(tr) * BM < first_row ? 1 : 0;
  const int slot = c == 0 ? slot0 : gi - (tc * BN) / g.Cg;
  return g.gpart[((static_cast<int64_t>(tr) * 2 + sgt) * g.tiles_n + tc) * g.slots + slot];
}

// Sum over the 64 lanes of a wave (lane 0 returns it): DPP steps inside each
// 16-lane row (every lane then holds its row's total), then rows 0..3 in order.
__device__ __forceinline__ float wave_sum(float v) {
  const int x0 = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x0, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  const int xi = __float_as_int(v);
  return ((__int_as_float(__builtin_amdgcn_readlane(xi, 0)) + __int_as_float(__builtin_amdgcn_readlane(xi, 16))) +
          __int_as_float(__builtin_amdgcn_readlane(xi, 32))) +
         __int_as_float(__builtin_amdgcn_readlane(xi, 48));
}

template <int BM, int BN>
__global__ void __launch_bounds__(kFoldThreads) gn_conv_fold(GemmArgs g) {
  __shared__ float2 red[kFoldThreads / 64];
  const int gi = blockIdx.x, b = blockIdx.y, q = threadIdx.x;
  const int2 r = batch_tile_rows(b, g.gT, BM);
  const int tn_lo = (gi * g.Cg) / BN, ntn = ((gi + 1) * g.Cg - 1) / BN - tn_lo + 1;
  const int total = (r.y - r.x + 1) * ntn;
  const int slot0 = gi - (tn_lo * BN) / g.Cg;
  const int64_t first_row = static_cast<int64_t>(b) * g.gT;  // b's first output row
  float2 s = make_float2(0.f, 0.f);
  if (total <= kFoldThreads) {  // one entry per lane at most
    if (q < total) s = fold_entry<BM, BN>(g, q, r.x, tn_lo, ntn, gi, slot0, first_row);
  } else {
    constexpr int U = 8;
    for (int e0 = q; e0 < total; e0 += U * kFoldThreads) {
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = fold_entry<BM, BN>(g, min(e0 + u * kFoldThreads, total - 1), r.x, tn_lo, ntn, gi, slot0, first_row);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (e0 + u * kFoldThreads < total) {
          s.x += v[u].x;
          s.y += v[u].y;
        }
      }
    }
  }
  const float sx = wave_sum(s.x), sy = wave_sum(s.y);
  if ((q & 63) == 0) red[q >> 6] = make_float2(sx, sy);
  __syncthreads();
  if (q == 0) {
    float2 sum = red[0];
#pragma unroll
    for (int w = 1; w < kFoldThreads / 64; ++w) {
      sum.x += red[w].x;
      sum.y += red[w].y;
    }
    g.gsums[(static_cast<int64_t>(b) * g.G + gi) * 2] = sum.x;
    g.gsums[(static_cast<int64_t>(b) * g.G + gi) * 2 + 1] = sum.y;
  }
}

int gemm_cus() {
  static thread_local int cached_dev = -1, cached = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      cached = cus;
    else
      (void)hipGetLastError();
    cached_dev = dev;
  }
  return cached;
}

// Tile configurations: shape, wave layout, slice width and ring depth when
// K % 64 == 0 (else 32-wide slices in a 3-stage ring), blocks per CU for the
// launch bounds, relative time per output element (fitted to MI355X timings).
struct TileCfg {
  int bm, bn, wgm, nw, bk, st, occ;
  double cost_per_elem;
};
constexpr TileCfg kTiles[] = {
    {128, 128, 2, 4, 64, 2, 2, 1.0},   {64, 128, 2, 4, 64, 3, 2, 1.19},  {64, 64, 2, 4, 64, 3, 2, 1.23},
    {160, 128, 1, 4, 64, 2, 2, 0.875}, {96, 128, 1, 4, 32, 3, 3, 1.07},  {128, 160, 4, 4, 64, 2, 2, 0.94},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int C, bool CONV>
void launch_bf16(const GemmArgs& base, hipStream_t st) {
  constexpr TileCfg t = kTiles[C];
  GemmArgs g = base;
  g.tiles_m = (g.M + t.bm - 1) / t.bm;
  g.tiles_n = (g.N + t.bn - 1) / t.bn;
  g.units = g.tiles_m * g.tiles_n;
  g.units_per_xcd = (g.units + kXcds - 1) / kXcds;
  const dim3 grid(static_cast<unsigned>(g.units_per_xcd * kXcds));
  if (g.K % t.bk == 0)
    hipLaunchKernelGGL((gemm_bf16<t.bm, t.bn, t.wgm, t.nw, t.bk, t.st, t.occ, CONV>), grid, dim3(64 * t.nw), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16<t.bm, t.bn, t.wgm, t.nw, kBK, kStages, t.occ, CONV>), grid, dim3(64 * t.nw), 0, st, g);
}

// Conv with GroupNorm sums: same tile choice, GNS epilogue, then the fold
// launch.
template <int C>
void launch_bf16_gns(const GemmArgs& base, hipStream_t st) {
  constexpr TileCfg t = kTiles[C];
  GemmArgs g = base;
  g.tiles_m = (g.M + t.bm - 1) / t.bm;
  g.tiles_n = (g.N + t.bn - 1) / t.bn;
  g.units = g.tiles_m * g.tiles_n;
  g.units_per_xcd = (g.units + kXcds - 1) / kXcds;
  g.slots = (t.bn + g.Cg - 1) / g.Cg + 1;
  const int64_t B = g.M / g.gT;
  const dim3 grid(static_cast<unsigned>(g.units_per_xcd * kXcds));
  if (g.K % t.bk == 0)
    hipLaunchKernelGGL((gemm_bf16<t.bm, t.bn, t.wgm, t.nw, t.bk, t.st, t.occ, true, true>), grid, dim3(64 * t.nw), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16<t.bm, t.bn, t.wgm, t.nw, kBK, kStages, t.occ, true, true>), grid, dim3(64 * t.nw), 0, st, g);
  hipLaunchKernelGGL((gn_conv_fold<t.bm, t.bn>), dim3(static_cast<unsigned>(g.G), static_cast<unsigned>(B)),
                     dim3(kFoldThreads), 0, st, g);
}

// Tile shape: fewest tiles per CU times tile area times the shape's cost per
// output element.  The costs were fitted to MI355X timings of the SDXL conv,
// projection and fused Q/K/V shapes; L2 request traffic per MFMA falls as the
// tile grows, which is what the larger shapes buy.
int pick_tile(const GemmArgs& g) {
  const int cus = gemm_cus();
  int best = 0;
  double best_cost = 1e300;
  for (int c = 0; c < kNumTiles; ++c) {
    const TileCfg& t = kTiles[c];
    const int64_t tiles = static_cast<int64_t>((g.M + t.bm - 1) / t.bm) * ((g.N + t.bn - 1) / t.bn);
    const double per_cu = std::ceil(static_cast<double>(tiles) / cus);
    const double cost = per_cu * t.bm * t.bn * t.cost_per_elem;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

template <bool CONV>
void launch_bf16_auto(const GemmArgs& g, hipStream_t st) {
  switch (pick_tile(g)) {
    case 0: launch_bf16<0, CONV>(g, st); break;
    case 1: launch_bf16<1, CONV>(g, st); break;
    case 2: launch_bf16<2, CONV>(g, st); break;
    case 3: launch_bf16<3, CONV>(g, st); break;
    case 4: launch_bf16<4, CONV>(g, st); break;
    default: launch_bf16<5, CONV>(g, st); break;
  }
}

// ------------------------------------------------------------------ f32 path
constexpr int kFT = 64, kFK = 16;

template <bool CONV>
__device__ __forceinline__ float a_elem_f32(const float* a, const float* x, const float* ht,
                                            const float* hb, int h, int W, int Cin, int m, int k,
                                            int M, int K) {
  if (m >= M || k >= K) return 0.f;
  if constexpr (!CONV) {
    return a[static_cast<int64_t>(m) * K + k];
  } else {
    const int tap = k / Cin, c = k - tap * Cin;
    const int dy = tap / 3 - 1, dx = tap % 3 - 1;
    const int hw = h * W;
    const int b = m / hw, rem = m - b * hw;
    const int row = rem / W + dy, col = rem % W + dx;
    if (col < 0 || col >= W) return 0.f;
    if (row < 0) return ht ? ht[(static_cast<int64_t>(b) * W + col) * Cin + c] : 0.f;
    if (row >= h) return hb ? hb[(static_cast<int64_t>(b) * W + col) * Cin + c] : 0.f;
    return x[((static_cast<int64_t>(b) * h + row) * W + col) * Cin + c];
  }
}

template <bool CONV>
__global__ void __launch_bounds__(kThreads)
gemm_f32(const float* __restrict__ a, const float* __restrict__ x, const float* __restrict__ ht,
         const float* __restrict__ hb, int h, int W, int Cin, OutMap map,
         const float* __restrict__ bias, int M, int N, int K) {
  __shared__ float As[kFK][kFT + 1];
  __shared__ float Bs[kFK][kFT + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * kFT, m0 = blockIdx.y * kFT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kFK) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kThreads * u;
      const int r = e / kFK, kk = e % kFK;
      As[kk][r] = a_elem_f32<CONV>(a, x, ht, hb, h, W, Cin, m0 + r, k0 + kk, M, K);
      const int n = n0 + r, k = k0 + kk;
      float bv = 0.f;
      if (n < N && k < K) {
        const int seg = n / map.seg_n;
        bv = static_cast<const float*>(map.wts[seg])[static_cast<int64_t>(n - seg * map.seg_n) * K + k];
      }
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) {
        const int seg = n / map.seg_n;
        static_cast<float*>(map.outs[seg])[out_row(map, seg, m) * map.seg_n + n - seg * map.seg_n] =
            acc[i][j] + (bias ? bias[n] : 0.f);
      }
    }
}

// A plain GEMM's output map: one segment, rows as computed.
OutMap plain_map(const void* wt, void* y, int64_t M, int64_t N) {
  OutMap m{};
  m.wts[0] = wt;
  m.outs[0] = y;
  m.n_seg = 1;
  m.seg_n = static_cast<int>(N);
  m.rpg = static_cast<int>(M);
  m.grp_rows[0] = static_cast<int>(M);
  m.row_off[0] = 0;
  return m;
}

dp_status run_gemm(bool conv, const void* a, const void* x, const void* ht, const void* hb, int h,
                   int W, int Cin, const OutMap& map, const float* bias, int64_t M, int64_t N,
                   int64_t K, dp_dtype dt, hipStream_t st, const char* name) {
  if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF)
    return dp::fail(DP_ERR_UNSUPPORTED, "%s: dimension exceeds 2^31", name);
  if (dt == DP_BF16) {
    bool al = dp::aligned16(conv ? x : a) && (!ht || dp::aligned16(ht)) && (!hb || dp::aligned16(hb));
    for (int s = 0; s < map.n_seg; ++s) al = al && dp::aligned16(map.wts[s]) && dp::aligned16(map.outs[s]);
    if (!al) return dp::fail(DP_ERR_INVALID_ARG, "%s: bf16 tensors must be 16-byte aligned", name);
  }
  dp::clear_error();
  if (dt == DP_BF16) {
    if (K % kBK != 0 || map.seg_n % 32 != 0 || (conv && (Cin % kBK != 0 || Cin > 2048)))
      return dp::fail(DP_ERR_UNSUPPORTED, "%s: bf16 path needs Cin %% 32 == 0 (conv: Cin <= 2048) and Cout %% 32 == 0", name);
    if ((M + 63) / 64 * ((N + 63) / 64) > 0x3FFFFFFF)
      return dp::fail(DP_ERR_UNSUPPORTED, "%s: too many tiles", name);
    GemmArgs g{};
    g.a = static_cast<const bf16_t*>(a);
    g.geo = ConvGeom{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(ht),
                     static_cast<const bf16_t*>(hb), h, W, Cin};
    g.map = map;
    g.bias = bias;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    if (conv) launch_bf16_auto<true>(g, st);
    else launch_bf16_auto<false>(g, st);
  } else {
    const int64_t gy = (M + kFT - 1) / kFT;
    if (gy > 65535) return dp::fail(DP_ERR_UNSUPPORTED, "%s: M too large", name);
    const dim3 grid(static_cast<unsigned>((N + kFT - 1) / kFT), static_cast<unsigned>(gy));
    if (conv)
      hipLaunchKernelGGL(gemm_f32<true>, grid, dim3(kThreads), 0, st, nullptr,
                         static_cast<const float*>(x), static_cast<const float*>(ht),
                         static_cast<const float*>(hb), h, W, Cin, map, bias, (int)M, (int)N, (int)K);
    else
      hipLaunchKernelGGL(gemm_f32<false>, grid, dim3(kThreads), 0, st,
                         static_cast<const float*>(a), nullptr, nullptr, nullptr, 0, 0, 0, map, bias,
                         (int)M, (int)N, (int)K);
  }
  return dp::check_launch(name);
}

}  // namespace

DP_API dp_status dp_linear(const void* x, const void* w, const float* bias, void* y, int64_t M,
                           int64_t Cin, int64_t Cout, dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  if (!x || !w || !y) return fail(DP_ERR_INVALID_ARG, "dp_linear: NULL pointer");
  if (M <= 0 || Cin <= 0 || Cout <= 0) return fail(DP_ERR_INVALID_ARG, "dp_linear: sizes must be positive");
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "dp_linear: bad dtype");
  const size_t es = dp::dtype_size(dt);
  if (dp::overlaps(x, M * Cin * es, y, M * Cout * es) || dp::overlaps(w, Cout * Cin * es, y, M * Cout * es))
    return fail(DP_ERR_INVALID_ARG, "dp_linear: output overlaps an input");
  return run_gemm(false, x, nullptr, nullptr, nullptr, 0, 0, 0, plain_map(w, y, M, Cout), bias, M, Cout,
                  Cin, dt, stream, "dp_linear");
}

DP_API dp_status dp_conv3x3_stale_halo(const void* x, const void* halo_top, const void* halo_bot,
                                       const void* w, const float* bias, void* y, int64_t B,
                                       int64_t h, int64_t W, int64_t Cin, int64_t Cout,
                                       dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  if (!x || !w || !y) return fail(DP_ERR_INVALID_ARG, "dp_conv3x3_stale_halo: NULL pointer");
  if (B <= 0 || h <= 0 || W <= 0 || Cin <= 0 || Cout <= 0)
    return fail(DP_ERR_INVALID_ARG, "dp_conv3x3_stale_halo: sizes must be positive");
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "dp_conv3x3_stale_halo: bad dtype");
  const size_t es = dp::dtype_size(dt);
  const size_t yb = static_cast<size_t>(B * h * W * Cout) * es;
  const size_t hb = static_cast<size_t>(B * W * Cin) * es;
  if (dp::overlaps(x, B * h * W * Cin * es, y, yb) || dp::overlaps(w, Cout * 9 * Cin * es, y, yb) ||
      (halo_top && dp::overlaps(halo_top, hb, y, yb)) || (halo_bot && dp::overlaps(halo_bot, hb, y, yb)))
    return fail(DP_ERR_INVALID_ARG, "dp_conv3x3_stale_halo: output overlaps an input");
  if (h > 0x7FFFFFFF || W > 0x7FFFFFFF || Cin > 0x7FFFFFFF)
    return fail(DP_ERR_UNSUPPORTED, "dp_conv3x3_stale_halo: dimension exceeds 2^31");
  return run_gemm(true, nullptr, x, halo_top, halo_bot, (int)h, (int)W, (int)Cin,
                  plain_map(w, y, B * h * W, Cout), bias, B * h * W, Cout, 9 * Cin, dt, stream,
                  "dp_conv3x3_stale_halo");
}

DP_API dp_status dp_qkv_projection_into_buffers(const void* x, const void* wq, const void* wk,
                                                const void* wv, void* q, void* k_buf, void* v_buf,
                                                int64_t B, int64_t T_loc, int64_t T_kv, int64_t t0,
                                                int64_t C, dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_qkv_projection_into_buffers";
  if (!x || !wq || !wk || !wv || !q || !k_buf || !v_buf) return fail(DP_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if (B <= 0 || T_loc <= 0 || T_kv <= 0 || C <= 0) return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (t0 < 0 || t0 + T_loc > T_kv) return fail(DP_ERR_INVALID_ARG, "%s: rows [t0, t0+T_loc) outside [0, T_kv)", name);
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  if (B * T_kv > 0x7FFFFFFF || 3 * C > 0x7FFFFFFF) return fail(DP_ERR_UNSUPPORTED, "%s: dimension exceeds 2^31", name);
  const size_t es = dp::dtype_size(dt);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * es, bb = static_cast<size_t>(B * T_kv * C) * es;
  const size_t wb = static_cast<size_t>(C * C) * es;
  const void* ins[4] = {x, wq, wk, wv};
  const size_t insz[4] = {xb, wb, wb, wb};
  void* outs[3] = {q, k_buf, v_buf};
  const size_t outsz[3] = {xb, bb, bb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (dp::overlaps(ins[i], insz[i], outs[o], outsz[o])) return fail(DP_ERR_INVALID_ARG, "%s: an output overlaps an input", name);
    for (int p = o + 1; p < 3; ++p)
      if (dp::overlaps(outs[p], outsz[p], outs[o], outsz[o])) return fail(DP_ERR_INVALID_ARG, "%s: outputs overlap", name);
  }
  OutMap m{};
  m.wts[0] = wq;
  m.wts[1] = wk;
  m.wts[2] = wv;
  m.outs[0] = q;
  m.outs[1] = k_buf;
  m.outs[2] = v_buf;
  m.n_seg = 3;
  m.seg_n = static_cast<int>(C);
  m.rpg = static_cast<int>(T_loc);
  m.grp_rows[0] = static_cast<int>(T_loc);
  m.row_off[0] = 0;
  m.grp_rows[1] = m.grp_rows[2] = static_cast<int>(T_kv);
  m.row_off[1] = m.row_off[2] = static_cast<int>(t0);
  return run_gemm(false, x, nullptr, nullptr, nullptr, 0, 0, 0, m, nullptr, B * T_loc, 3 * C, C, dt, stream,
                  name);
}

namespace {
// Workspace of the conv with GroupNorm sums: the (tile row, batch segment,
// tile column, group slot) partials, sized for every tile shape the planner
// may pick and for one channel per group.  Every slot the fold reads is
// written by the same call, so the workspace needs no initial contents.
struct ConvGnWs {
  size_t partial_off, total;
};
ConvGnWs conv_gn_ws(int64_t B, int64_t h, int64_t W, int64_t Cout) {
  const int64_t M = B * h * W;
  int64_t part = 0;
  for (const TileCfg& t : kTiles) {
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (Cout + t.bn - 1) / t.bn;
    part = std::max(part, tm * 2 * tn * (t.bn + 1));
  }
  ConvGnWs w{};
  w.partial_off = 0;
  w.total = w.partial_off + static_cast<size_t>(part) * sizeof(float2);
  return w;
}
}  // namespace

DP_API size_t dp_conv3x3_gn_sums_workspace(int64_t B, int64_t h, int64_t W, int64_t Cout) {
  if (B <= 0 || h <= 0 || W <= 0 || Cout <= 0) return 0;
  if (B * h * W > 0x7FFFFFFF || Cout > 0x7FFFFFFF) return 0;
  return conv_gn_ws(B, h, W, Cout).total;
}

DP_API dp_status dp_conv3x3_stale_halo_gn_sums(const void* x, const void* halo_top, const void* halo_bot,
                                               const void* w, const float* bias, void* y, float* gn_sums,
                                               int64_t G, void* ws, size_t ws_bytes, int64_t B, int64_t h,
                                               int64_t W, int64_t Cin, int64_t Cout, dp_dtype dt,
                                               hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_conv3x3_stale_halo_gn_sums";
  if (!x || !w || !y || !gn_sums) return fail(DP_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if (B <= 0 || h <= 0 || W <= 0 || Cin <= 0 || Cout <= 0 || G <= 0)
    return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (Cout % G != 0) return fail(DP_ERR_INVALID_ARG, "%s: Cout %% G != 0", name);
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  const size_t need = dp_conv3x3_gn_sums_workspace(B, h, W, Cout);
  if (!ws || ws_bytes < need) return fail(DP_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  const size_t es = dp::dtype_size(dt);
  const size_t yb = static_cast<size_t>(B * h * W * Cout) * es, hbb = static_cast<size_t>(B * W * Cin) * es;
  const size_t sb = static_cast<size_t>(B * G) * 8;
  if (dp::overlaps(x, B * h * W * Cin * es, y, yb) || dp::overlaps(w, Cout * 9 * Cin * es, y, yb) ||
      (halo_top && dp::overlaps(halo_top, hbb, y, yb)) || (halo_bot && dp::overlaps(halo_bot, hbb, y, yb)) ||
      dp::overlaps(gn_sums, sb, y, yb) || dp::overlaps(gn_sums, sb, ws, need) || dp::overlaps(ws, need, y, yb) ||
      dp::overlaps(gn_sums, sb, x, B * h * W * Cin * es) || dp::overlaps(gn_sums, sb, w, Cout * 9 * Cin * es) ||
      dp::overlaps(ws, need, x, B * h * W * Cin * es) || dp::overlaps(ws, need, w, Cout * 9 * Cin * es))
    return fail(DP_ERR_INVALID_ARG, "%s: an output overlaps an input or the workspace", name);
  if (dt != DP_BF16 || Cin % kBK != 0 || Cin > 2048 || Cout % 32 != 0 || Cout > 2048)
    return fail(DP_ERR_UNSUPPORTED, "%s: needs bf16 with Cin %% 32 == 0, Cin <= 2048, Cout %% 32 == 0, Cout <= 2048",
                name);
  if (h * W < 160) return fail(DP_ERR_UNSUPPORTED, "%s: needs at least 160 tokens per batch item", name);
  if (!dp::aligned16(x) || !dp::aligned16(w) || !dp::aligned16(y) || (halo_top && !dp::aligned16(halo_top)) ||
      (halo_bot && !dp::aligned16(halo_bot)))
    return fail(DP_ERR_INVALID_ARG, "%s: bf16 tensors must be 16-byte aligned", name);
  if (B * h * W > 0x7FFFFFFF || 9 * Cin > 0x7FFFFFFF) return fail(DP_ERR_UNSUPPORTED, "%s: dimension exceeds 2^31", name);
  dp::clear_error();
  GemmArgs g{};
  g.geo = ConvGeom{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(halo_top),
                   static_cast<const bf16_t*>(halo_bot), (int)h, (int)W, (int)Cin};
  g.map = plain_map(w, y, B * h * W, Cout);
  g.bias = bias;
  g.M = (int)(B * h * W);
  g.N = (int)Cout;
  g.K = (int)(9 * Cin);
  const ConvGnWs lay = conv_gn_ws(B, h, W, Cout);
  g.gpart = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.partial_off);
  g.gsums = gn_sums;
  g.gT = (int)(h * W);
  g.G = (int)G;
  g.Cg = (int)(Cout / G);
  switch (pick_tile(g)) {
    case 0: launch_bf16_gns<0>(g, stream); break;
    case 1: launch_bf16_gns<1>(g, stream); break;
    case 2: launch_bf16_gns<2>(g, stream); break;
    case 3: launch_bf16_gns<3>(g, stream); break;
    case 4: launch_bf16_gns<4>(g, stream); break;
    default: launch_bf16_gns<5>(g, stream); break;
  }
  return dp::check_launch(name);
}
