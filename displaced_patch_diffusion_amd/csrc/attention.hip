// Attention of the rank's query rows over the whole spliced K/V buffer.
//
// Method source: "OTIL for SDXL on 4x L40S", "What is implemented where" (the
// displaced self-attention layer) and "Read this before interpreting the
// numbers", item 3 (its stale state is the attention K/V buffer); the xDiT
// issue thread "Tensor Parallelism with Stale Activations ..." (the buffer has
// the full spatial shape; local rows fresh, remote rows stale).  Every local
// query attends to all T_kv keys, no mask: o = softmax(scale * q K^T) V.
//
// bf16, d = 64 (gfx950 MFMA path)
// -------------------------------
// A block of 4 waves owns 128 consecutive queries of one (batch, head); each
// wave owns 32 of them.  Key/value tiles of 64 tokens are staged in LDS
// (K as [key][d], V as [key][d] read transposed) by LDS DMA in a 3-stage
// ring, the next tile's load in flight during the current one, one barrier
// per tile; 48 KB per block lets three blocks share a CU.  Per 32-key
// block a wave computes the transposed scores
//     S^T[key][query] = K . Q^T      (v_mfma_f32_32x32x16_bf16, 4 k-steps over d)
// so that accumulator lane l holds 16 scores of the single query l % 32: the
// softmax is in-lane, plus one exchange with lane l ^ 32.  K rows are loaded
// with row index bits 2 and 3 swapped; with that permutation the 8
// probabilities a lane holds for each 16-key step are 8 consecutive keys, which
// is exactly the B operand layout of the transposed output product
//     O^T[d][query] += V^T . P^T      (2 d-blocks x 2 k-steps per 32 keys).
// Softmax in base 2: a probability is exp2(c * s - m_ref) with c = scale *
// log2(e) applied to the float32 score s by one FMA (Q enters the product as
// stored, so no rounding of q * c to bf16 perturbs the scores).  The reference
// m_ref is the first block's max and only moves when a block's probabilities
// would grow huge (see the key loop).  P is rounded to bf16 for the second
// product; row sums and O accumulate in float32; output rows are normalised
// once at the end.
//
// Schedules.  A unit is (batch, head, 128-query block) against all keys.  The
// split schedule gives each block one unit, or one of S equal key chunks of
// it (partials merged by attn_combine), with the blocks of one key chunk
// resident together on one XCD; when the units fill whole rounds of resident
// blocks and leave a remainder, the full rounds may run whole and only the
// remainder split.  When the units do not fill whole rounds, the balanced
// schedule gives each resident block an equal contiguous range of the
// (unit, key tile) sequence; attn_combine_sk merges the pieces of the units
// that neighbouring blocks share.
//
// f32 (d = 32 or 64)
// ------------------
// One thread per query, K/V tiles of 32 keys in LDS, the same online softmax
// in float32 with expf: the correctness path for fp32 shares.
#include <math.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "dp_internal.h"

namespace {

constexpr int kD = 64;
constexpr int kBMq = 128;              // queries per block (4 waves x 32)
constexpr int kBNk = 64;               // keys per tile
constexpr int kStages = 3;             // LDS ring depth (the next tile loads during the current one)
constexpr int kTileBytes = kBNk * kD * 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kBig = 1.8446744e19f;  // 2^64: a lane's block sum above this recentres
constexpr int kXcds = 8;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Row swizzle of a 128-byte LDS row: 16-byte chunk c of row r lives in slot
// c ^ swz(r).  With this swizzle the K operand reads (16 rows, one chunk) and
// the V transpose reads (4 rows x 32 bytes per 16-lane group) are free of bank
// conflicts.
__device__ __forceinline__ int swz(int row) { return ((row & 2) << 1) | ((row >> 2) & 3); }

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* out;
  float* part_o;    // [S][B][Tq][C] unnormalised partial outputs (split only)
  float* part_ml;   // [S][B][H][Tq][2] running max (base 2) and row sum (split only)
  int B, H, Tq, Tkv;
  float c;          // scale * log2(e)
  int n_qblk, n_split, chunk_tiles, n_tiles, units, units_per_xcd;
  int n_whole;      // split schedule: units 0..n_whole-1 run whole in the first blocks
  int sk;           // 1: balanced contiguous work ranges per block (see attn_bf16_d64)
  int sk_grid;      // blocks of the balanced schedule (a multiple of kXcds)
  long long work;   // units * n_tiles (balanced schedule)
};

// Balanced schedule: block position p owns the work items
// [sk_start(p), sk_start(p+1)) of the (unit, tile) sequence.
__device__ __host__ __forceinline__ long long sk_start(long long p, long long work, long long grid) {
  return p * work / grid;
}
// Position owning work item w: the largest p with sk_start(p) <= w.
__device__ __host__ __forceinline__ long long sk_owner(long long w, long long work, long long grid) {
  return ((w + 1) * grid - 1) / work;
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  u32x4 u;
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(s[base + 2 * j], s[base + 2 * j + 1]);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_dst + 16*l (global_load_lds_dwordx4; the LDS base goes through M0).
// Issued as inline assembly so that the compiler does not treat it as a
// pending LDS write: completion is tracked only by the explicit vmcnt waits in
// the key loop, and the compiler's own waits can only over-wait.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is written on purpose; nothing else here uses it
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// M0 + 16*l (buffer_load_dwordx4 ... lds).  Reads at offsets at or beyond the
// descriptor's num_records return zeros.  Issued as inline assembly so that
// the compiler does not treat it as a pending LDS write: completion is
// tracked only by the explicit vmcnt waits in the key loop, and the compiler's
// own waits can only over-wait.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, unsigned int m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int S>
struct Stage {
  static constexpr int value = S;
};

// One segment: the queries of block qb of (b, h) against key tiles
// [t_begin, t_end).  Split schedule (SK false): `piece` is the key chunk;
// with one chunk the normalised bf16 rows go to out, otherwise unnormalised
// float32 rows and (m_ref, row sum) go to the chunk's partial arrays.
// Balanced schedule (SK true): `piece` < 0 writes out; otherwise it is the
// partial slot of the rows.
template <bool SK>
__device__ __forceinline__ void attn_segment(const AttnArgs& a, char* lds, int b, int h, int qb, int t_begin,
                                             int t_end, long long piece) {
  constexpr int kVring = kStages * kTileBytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int C = a.H * kD;
  const int qi = qb * kBMq + wave * 32 + l32;
  const bool q_ok = qi < a.Tq;

  // Q as stored (the scale is applied to the float32 scores).
  bf16x8 qop[4];
  {
    const bf16_t* qp = a.q + (static_cast<int64_t>(b) * a.Tq + (q_ok ? qi : 0)) * C + h * kD + 8 * g;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 w = q_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * st) : u32x4{0u, 0u, 0u, 0u};
      qop[st] = __builtin_bit_cast(bf16x8, w);
    }
    // Consume Q here so its loads are complete before the key loop; otherwise
    // the compiler would keep a vmcnt(0) wait for them in every iteration,
    // which would also drain the K/V prefetch.
    asm volatile("" ::"v"(qop[0]), "v"(qop[1]), "v"(qop[2]), "v"(qop[3]));
  }

  // K operand: lane row l32 holds key 32*blk + pi(l32), pi = swap of row bits 2
  // and 3; then the probabilities a lane holds per 16-key step are 8
  // consecutive keys, the B operand layout of the P.V product.
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  int koff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) koff[st] = krow * 128 + (((2 * st + g) ^ swz(krow)) << 4);
  // V^T operand via ds_read_b64_tr_b16: in each 16-lane group, lane j = 4a+b
  // receives element b of the 8-byte pieces addressed by lanes a, a+4, a+8,
  // a+12.  Lane i of group (g, half) addresses key row 8g + 4h + i/4 and
  // channel 32*db + 16*half + 4*(i%4), so lane l ends up with channel l%32 of
  // four consecutive keys.
  int voff[2][2];
  {
    const int i = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 8 * g + 4 * hh + (i >> 2);
        const int chunk = 4 * db + 2 * half + ((i & 3) >> 1);
        voff[db][hh] = kVring + row * 128 + ((chunk ^ swz(row)) << 4) + (i & 1) * 8;
      }
  }
  // DMA: wave w fills rows 16w .. 16w+15 of each tile, one 1 KB (8-row) slab
  // per instruction; lane l writes slot l%8 of row l/8, i.e. chunk
  // (l%8) ^ swz(row) of that row.
  int gbyte[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * wave + j) * 8 + (lane >> 3);
    gbyte[j] = (row * C + (((lane & 7) ^ swz(row)) << 3)) * 2;
  }
  const unsigned int lds0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned int>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds)) +
      wave * 2048);
  const bf16_t* kbh = a.k + static_cast<int64_t>(b) * a.Tkv * C + h * kD;
  const bf16_t* vbh = a.v + static_cast<int64_t>(b) * a.Tkv * C + h * kD;
  // Bytes from a (batch, head) base to the end of that batch item's buffer.
  const int64_t span = (static_cast<int64_t>(a.Tkv) * C - h * kD) * 2;

  auto issue = [&](int t, int stage) {
    const int64_t off = static_cast<int64_t>(t) * kBNk * C;  // elements
    const int nrec = static_cast<int>(span - off * 2);       // rows past T_kv read as 0
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbh + off), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbh + off), 0, nrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16(rk, gbyte[j], lds0 + stage * kTileBytes + j * 1024);
      dma16(rv, gbyte[j], lds0 + kVring + stage * kTileBytes + j * 1024);
    }
  };

  // Software pipeline over 32-key blocks j (two per 64-key tile).  Slot j
  // issues the scores of block j+1 and the P.V product of block j-1 (8 MFMAs)
  // and, independent of both, the exponentials, bf16 probabilities and row
  // sums of block j, so the MFMA and VALU pipes can run side by side.
  //
  // Reference: a block's probabilities are exp2(c * s - m_ref), c = scale *
  // log2(e), s the raw float32 scores.  m_ref is set once from the first
  // block's max; later blocks only need a new reference when their
  // probabilities grow huge, which the lane's block row sum reveals (it also
  // catches inf).  That rare case is handled at the slot boundary: move the
  // reference to the block max, rescale o and l, and recompute the block's
  // probabilities.
  const float cs = a.c;
  float m_ref = 0.f, l_part = 0.f;
  f32x16 o[2], sc_cur, sc_nxt;
  bf16x8 p_prv[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[0][e] = o[1][e] = 0.f;

  auto qk = [&](auto ks_c, auto kb_c) {
    constexpr int KS = decltype(ks_c)::value, KB = decltype(kb_c)::value;
    bf16x8 ka[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      ka[st] = *reinterpret_cast<const bf16x8*>(lds + KS * kTileBytes + KB * 4096 + koff[st]);
    f32x16 r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qop[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int st = 1; st < 4; ++st) r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qop[st], r, 0, 0, 0);
    return r;
  };
  auto pv = [&](auto vs_c, auto vb_c) {
    constexpr int VS = decltype(vs_c)::value, VB = decltype(vb_c)::value;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const char* vb = lds + VS * kTileBytes + VB * 4096 + s2 * 2048;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[db][0]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[db][1]));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p_prv[s2], o[db], 0, 0, 0);
      }
  };
  // keys of block (t, blk) at or beyond T_kv get -inf (only the last tile)
  auto mask = [&](f32x16& x, int t, int blk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * g + (e & 3);
      const int pr = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
      if (t * kBNk + 32 * blk + pr >= a.Tkv) x[e] = -INFINITY;
    }
  };
  // Exponentials, bf16 probabilities and the lane's row sum of one block.  The
  // sum is taken over the bf16-rounded P that enters the product, as eight
  // v_dot2_f32_bf16 against (1, 1) in four independent chains, in one asm
  // block: the compiler cannot see DOT hazards through inline assembly (and
  // its own v_dot2c form read wrong values on gfx950 right after the pack), so
  // the block carries its own wait states -- five before the first DOT, three
  // instructions between dependent DOTs, five before plain VALU reads of DOT
  // results.
  auto probs = [&](const f32x16& x, bf16x8* p) {
    f32x16 ex;
#pragma unroll
    for (int e = 0; e < 16; ++e) ex[e] = __builtin_amdgcn_exp2f(fmaf(x[e], cs, -m_ref));
    p[0] = pack8(ex, 0);
    p[1] = pack8(ex, 8);
    const u32x4 w0 = __builtin_bit_cast(u32x4, p[0]), w1 = __builtin_bit_cast(u32x4, p[1]);
    const unsigned int ones = 0x3F803F80u;
    float r0, r1, r2, r3;
    asm("s_nop 4\n\t"
        "v_dot2_f32_bf16 %0, %4, %12, 0\n\t"
        "v_dot2_f32_bf16 %1, %5, %12, 0\n\t"
        "v_dot2_f32_bf16 %2, %6, %12, 0\n\t"
        "v_dot2_f32_bf16 %3, %7, %12, 0\n\t"
        "v_dot2_f32_bf16 %0, %8, %12, %0\n\t"
        "v_dot2_f32_bf16 %1, %9, %12, %1\n\t"
        "v_dot2_f32_bf16 %2, %10, %12, %2\n\t"
        "v_dot2_f32_bf16 %3, %11, %12, %3\n\t"
        "s_nop 4\n\t"
        "v_add_f32 %0, %0, %1\n\t"
        "v_add_f32 %2, %2, %3\n\t"
        "v_add_f32 %0, %0, %2"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(w0[0]), "v"(w0[1]), "v"(w0[2]), "v"(w0[3]), "v"(w1[0]), "v"(w1[1]), "v"(w1[2]), "v"(w1[3]),
          "v"(ones));
    return r0;
  };
  // Move the reference to the block max (when above it): rescale o and l.
  auto recentre = [&](const f32x16& x) {
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
    const float delta = fmaxf(fmaf(swap_max(mx), cs, -m_ref), 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-delta);
    l_part *= alpha;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      o[0][e] *= alpha;
      o[1][e] *= alpha;
    }
    m_ref += delta;
  };

  // One slot: block (t, blk) is current; K of the next block at (KS, KB), V of
  // the previous one at (VS, VB).  Straight-line from the MFMAs to the row
  // sums so that the scheduler can interleave them; the ragged-key mask and
  // the rare recentring sit at the slot boundaries.
  auto slot = [&](auto ks_c, auto kb_c, auto vs_c, auto vb_c, bool ragged, int t, int blk) {
    if (ragged) mask(sc_cur, t, blk);
    sc_nxt = qk(ks_c, kb_c);
    pv(vs_c, vb_c);
    bf16x8 p_new[2];
    float ls = probs(sc_cur, p_new);
    if (__builtin_amdgcn_ballot_w64(!(ls < kBig))) {  // rare
      recentre(sc_cur);
      ls = probs(sc_cur, p_new);
    }
    l_part += ls;
    p_prv[0] = p_new[0];
    p_prv[1] = p_new[1];
    sc_cur = sc_nxt;
  };
  // Tile t in LDS stage S: slot (t, 0), then wait for tile t+1 and refill the
  // stage of tile t-1 with tile t+3, then slot (t, 1).  The first tile's slot
  // (t, 0) multiplies a zero P by a zeroed V stage; the last tile's slot (t, 1)
  // computes scores of a block that does not exist and never uses them.
  auto tile = [&](auto stage_c, int t) {
    constexpr int S = decltype(stage_c)::value;
    const bool ragged = (t + 1) * kBNk > a.Tkv;
    slot(Stage<S>{}, Stage<1>{}, Stage<(S + 2) % 3>{}, Stage<1>{}, ragged, t, 0);
    if (t + 1 < t_end) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t+1 done
      __syncthreads();  // tile t+1 visible; stage of tile t-1 no longer read
      if (t + 2 < t_end) issue(t + 2, (S + 2) % 3);
    }
    slot(Stage<(S + 1) % 3>{}, Stage<0>{}, Stage<S>{}, Stage<0>{}, ragged, t, 1);
  };

  // zero V of stage 3, read (times a zero P) by the first tile's first slot
  {
    u32x4* z = reinterpret_cast<u32x4*>(lds + kVring + 2 * kTileBytes);
    z[tid] = u32x4{0u, 0u, 0u, 0u};
    z[tid + 256] = u32x4{0u, 0u, 0u, 0u};
  }
  p_prv[0] = p_prv[1] = bf16x8{};
  issue(t_begin, 0);
  if (t_begin + 1 < t_end) issue(t_begin + 1, 1);
  if (t_begin + 1 < t_end) {
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  // first block: its max is the reference
  sc_cur = qk(Stage<0>{}, Stage<0>{});
  if ((t_begin + 1) * kBNk > a.Tkv) mask(sc_cur, t_begin, 0);
  {
    float mx = sc_cur[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc_cur[e]);
    m_ref = swap_max(mx) * cs;
  }
  tile(Stage<0>{}, t_begin);
  for (int t = t_begin + 1; t < t_end; t += 3) {
    tile(Stage<1>{}, t);
    if (t + 1 < t_end) tile(Stage<2>{}, t + 1);
    if (t + 2 < t_end) tile(Stage<0>{}, t + 2);
  }
  // P.V of the last block
  switch ((t_end - 1 - t_begin) % 3) {
    case 0: pv(Stage<0>{}, Stage<1>{}); break;
    case 1: pv(Stage<1>{}, Stage<1>{}); break;
    default: pv(Stage<2>{}, Stage<1>{}); break;
  }

  const float l_tot = swap_sum(l_part);
  if (!q_ok) return;
  if (piece < 0) {
    const float inv = 1.0f / l_tot;
    bf16_t* op = a.out + (static_cast<int64_t>(b) * a.Tq + qi) * C + h * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * g;
        u32x2 pk = {pack_bf16x2(o[db][4 * qq] * inv, o[db][4 * qq + 1] * inv),
                    pack_bf16x2(o[db][4 * qq + 2] * inv, o[db][4 * qq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
  } else {
    float* op;
    float* ml;
    if constexpr (SK) {
      const int64_t row = piece * kBMq + (qi - qb * kBMq);
      op = a.part_o + row * kD;
      ml = a.part_ml + row * 2;
    } else {
      op = a.part_o + ((piece * a.B + b) * a.Tq + qi) * C + h * kD;
      ml = a.part_ml + (((piece * a.B + b) * a.H + h) * a.Tq + qi) * 2;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * g;
        *reinterpret_cast<f32x4*>(op + d) =
            f32x4{o[db][4 * qq], o[db][4 * qq + 1], o[db][4 * qq + 2], o[db][4 * qq + 3]};
      }
    if (g == 0) {
      ml[0] = m_ref;
      ml[1] = l_tot;
    }
  }
}

// Split schedule (SK == false): one segment per block.  Blocks are dealt to
// the XCDs round-robin, so XCD x receives blocks x, x+8, ...; each XCD gets a
// contiguous run of units, ordered (batch, head, key chunk, query block), so
// the blocks resident on one XCD share a key chunk and read it from that
// XCD's L2.  The first n_whole blocks (whole rounds, a multiple of 8) run
// units 0..n_whole-1 whole; the key chunks of the other units follow.
//
// Balanced schedule (SK == true): position p (XCD-contiguous) owns a
// contiguous range of the (unit, tile) sequence, units ordered (batch, head,
// query block).  A unit wholly inside the range is written directly; the
// first and the last segment of the range may be pieces of units shared with
// the neighbouring positions, written to partial slots 0 and 1 of p.
template <bool SK>
__global__ void __launch_bounds__(256, 3) attn_bf16_d64(AttnArgs a) {
  // K tiles at stage*8 KB, V tiles at 24 KB + stage*8 KB.
  __shared__ __attribute__((aligned(1024))) char lds[kStages * 2 * kTileBytes];
  if constexpr (!SK) {
    if (static_cast<int>(blockIdx.x) < a.n_whole) {
      // first round: whole units, n_whole / 8 consecutive ones per XCD
      const int u = (blockIdx.x % kXcds) * (a.n_whole / kXcds) + blockIdx.x / kXcds;
      attn_segment<false>(a, lds, u / a.n_qblk / a.H, (u / a.n_qblk) % a.H, u % a.n_qblk, 0, a.n_tiles, -1);
      return;
    }
    // the key chunks of the remaining units, ordered (batch, head, chunk,
    // query block); the first (batch, head) may start part-way through its
    // query blocks
    const int i = blockIdx.x - a.n_whole;
    const int k = (i % kXcds) * a.units_per_xcd + i / kXcds;
    if (k >= a.units) return;
    const int nq = a.n_qblk, S = a.n_split;
    const int g0 = a.n_whole / nq, off0 = a.n_whole - g0 * nq, n0 = nq - off0;
    int g, split, qb;
    if (k < n0 * S) {
      g = g0;
      split = k / n0;
      qb = off0 + k % n0;
    } else {
      const int r = k - n0 * S;
      g = g0 + 1 + r / (nq * S);
      split = (r % (nq * S)) / nq;
      qb = r % nq;
    }
    const int t_begin = split * a.chunk_tiles;
    const int t_end = min(a.n_tiles, t_begin + a.chunk_tiles);
    attn_segment<false>(a, lds, g / a.H, g % a.H, qb, t_begin, t_end, S == 1 ? -1 : split);
  } else {
    const long long p = static_cast<long long>(blockIdx.x % kXcds) * (a.sk_grid / kXcds) + blockIdx.x / kXcds;
    const long long w0 = sk_start(p, a.work, a.sk_grid), w1 = sk_start(p + 1, a.work, a.sk_grid);
    for (long long w = w0; w < w1;) {
      const int u = static_cast<int>(w / a.n_tiles);
      const int t_begin = static_cast<int>(w - static_cast<long long>(u) * a.n_tiles);
      const int t_end = static_cast<int>(min(static_cast<long long>(a.n_tiles), t_begin + (w1 - w)));
      const int qb = u % a.n_qblk;
      const int h = (u / a.n_qblk) % a.H;
      const int b = u / a.n_qblk / a.H;
      const bool whole = t_begin == 0 && t_end == a.n_tiles;
      if (w != w0) {
        // the previous segment's LDS reads and stores are complete before
        // this segment's loads refill the ring
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
      attn_segment<true>(a, lds, b, h, qb, t_begin, t_end, whole ? -1 : p * 2 + (w == w0 ? 0 : 1));
      w += t_end - t_begin;
    }
  }
}

// Merges the key-chunk partials: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Only the split units (n_whole on) are launched: four 256-thread blocks per
// unit, one thread per (query row, 8-channel group), so the unit's (batch,
// head, query block) is the same for the whole block.  SS > 0 compiles the
// merge for exactly SS chunks with every load issued before the first is
// used; SS = 0 loops over S chunks.  Both add in chunk order.
constexpr int kCombineBlocksPerUnit = kBMq * 8 / 256;
template <int SS>
__global__ void __launch_bounds__(256)
attn_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
             bf16_t* __restrict__ out, int B, int H, int Tq, int S_arg, int n_whole, int n_qblk) {
  const int u = n_whole + static_cast<int>(blockIdx.x) / kCombineBlocksPerUnit;
  const int row = (static_cast<int>(blockIdx.x) % kCombineBlocksPerUnit) * (256 / 8) + static_cast<int>(threadIdx.x) / 8;
  const int ch = static_cast<int>(threadIdx.x) & 7;
  const int qb = u % n_qblk, bh = u / n_qblk, h = bh % H, b = bh / H;
  const int q = qb * kBMq + row;
  if (q >= Tq) return;
  const int C = H * kD;
  const int S = SS > 0 ? SS : S_arg;
  auto ml_of = [&](int s) { return part_ml + (((static_cast<int64_t>(s) * B + b) * H + h) * Tq + q) * 2; };
  auto o_of = [&](int s) { return part_o + ((static_cast<int64_t>(s) * B + b) * Tq + q) * C + h * kD + ch * 8; };
  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (SS > 0) {
    float2 ml[SS];
    f32x4 x0[SS], x1[SS];
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      ml[s] = *reinterpret_cast<const float2*>(ml_of(s));
      x0[s] = *reinterpret_cast<const f32x4*>(o_of(s));
      x1[s] = *reinterpret_cast<const f32x4*>(o_of(s) + 4);
    }
#pragma unroll
    for (int s = 0; s < SS; ++s) M = fmaxf(M, ml[s].x);
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      const float w = __builtin_amdgcn_exp2f(ml[s].x - M);
      L = fmaf(w, ml[s].y, L);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = fmaf(w, x0[s][j], acc[j]);
        acc[4 + j] = fmaf(w, x1[s][j], acc[4 + j]);
      }
    }
  } else {
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml_of(s)[0]);
    for (int s = 0; s < S; ++s) {
      const float* ml = ml_of(s);
      const float w = __builtin_amdgcn_exp2f(ml[0] - M);
      L = fmaf(w, ml[1], L);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(o_of(s));
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(o_of(s) + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = fmaf(w, x0[j], acc[j]);
        acc[4 + j] = fmaf(w, x1[j], acc[4 + j]);
      }
    }
  }
  const float inv = 1.0f / L;
  u32x4 pk;
#pragma unroll
  for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(b) * Tq + q) * C + h * kD + ch * 8) = pk;
}

struct AttnPlan {
  int n_qblk, n_tiles, n_split, chunk_tiles, units, units_per_xcd, grid;
  int n_whole;
  int sk;
  long long work;
  size_t ws_bytes;
};

// Merges the pieces of the units that the balanced schedule split between
// positions.  One thread per (batch, query, head, 8-channel group); a unit
// owned wholly by one position was written directly and is skipped.  Pieces
// are added in position order.
__global__ void __launch_bounds__(256)
attn_combine_sk(const float* __restrict__ part_o, const float* __restrict__ part_ml, bf16_t* __restrict__ out,
                int B, int H, int Tq, int n_qblk, int n_tiles, long long work, int grid) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(B) * Tq * H * 8;
  if (idx >= total) return;
  const int ch = static_cast<int>(idx & 7);
  int64_t r = idx >> 3;
  const int h = static_cast<int>(r % H);
  r /= H;
  const int q = static_cast<int>(r % Tq);
  const int b = static_cast<int>(r / Tq);
  const int qb = q / kBMq, row = q - qb * kBMq;
  const long long u = (static_cast<long long>(b) * H + h) * n_qblk + qb;
  const long long wf = u * n_tiles, wl = wf + n_tiles - 1;
  const long long p0 = sk_owner(wf, work, grid), p1 = sk_owner(wl, work, grid);
  if (p0 == p1) return;
  constexpr int kPieces = 4;
  if (p1 - p0 < kPieces) {
    // Up to kPieces positions: each range start computed once, every load
    // issued before the first is used (unused entries re-read piece 0, which
    // always exists: position p0 holds the unit's first work item).
    long long slot[kPieces];
    bool use[kPieces];
    long long s_lo = sk_start(p0, work, grid);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const long long p = p0 + i, s_hi = sk_start(p + 1, work, grid);
      use[i] = p <= p1 && s_hi != s_lo;  // an empty range holds no piece
      slot[i] = p * 2 + (i == 0 && s_lo < wf ? 1 : 0);
      s_lo = s_hi;
    }
    float2 ml[kPieces];
    f32x4 x0[kPieces], x1[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const long long sl = use[i] ? slot[i] : slot[0];
      ml[i] = *reinterpret_cast<const float2*>(part_ml + (sl * kBMq + row) * 2);
      const float* po = part_o + (sl * kBMq + row) * kD + ch * 8;
      x0[i] = *reinterpret_cast<const f32x4*>(po);
      x1[i] = *reinterpret_cast<const f32x4*>(po + 4);
    }
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (use[i]) M = fmaxf(M, ml[i].x);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      if (!use[i]) continue;
      const float w = __builtin_amdgcn_exp2f(ml[i].x - M);
      L = fmaf(w, ml[i].y, L);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = fmaf(w, x0[i][j], acc[j]);
        acc[4 + j] = fmaf(w, x1[i][j], acc[4 + j]);
      }
    }
    const float inv = 1.0f / L;
    u32x4 pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
    *reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(b) * Tq + q) * H * kD + h * kD + ch * 8) = pk;
    return;
  }
  float M = -INFINITY;
  for (long long p = p0; p <= p1; ++p) {
    if (sk_start(p + 1, work, grid) == sk_start(p, work, grid)) continue;  // empty range
    const long long slot = p * 2 + (p == p0 && sk_start(p, work, grid) < wf ? 1 : 0);
    M = fmaxf(M, part_ml[(slot * kBMq + row) * 2]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (long long p = p0; p <= p1; ++p) {
    if (sk_start(p + 1, work, grid) == sk_start(p, work, grid)) continue;
    const long long slot = p * 2 + (p == p0 && sk_start(p, work, grid) < wf ? 1 : 0);
    const float* ml = part_ml + (slot * kBMq + row) * 2;
    const float w = __builtin_amdgcn_exp2f(ml[0] - M);
    L = fmaf(w, ml[1], L);
    const float* po = part_o + (slot * kBMq + row) * kD + ch * 8;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(po);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(po + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = fmaf(w, x0[j], acc[j]);
      acc[4 + j] = fmaf(w, x1[j], acc[4 + j]);
    }
  }
  const float inv = 1.0f / L;
  u32x4 pk;
#pragma unroll
  for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(b) * Tq + q) * H * kD + h * kD + ch * 8) = pk;
}

int device_cus() {
  static thread_local int cached_dev = -1, cached_cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      cached_cus = cus;
    else
      (void)hipGetLastError();
    cached_dev = dev;
  }
  return cached_cus;
}

// Resident attention blocks per CU (registers and LDS), asked of the runtime
// once per device and thread.
template <bool SK>
int blocks_per_cu() {
  constexpr int kMaxDev = 64;
  static thread_local int cached[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = -1;
  }
  if (dev >= 0 && dev < kMaxDev && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_d64<SK>, 256, 0) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 2;
  }
  if (dev >= 0 && dev < kMaxDev) cached[dev] = n;
  return n;
}

// Schedule override from DP_ATTN_SCHEDULE (tests and tuning): 0 none,
// 1 split, 2 balanced.
enum { kSchedAuto = 0, kSchedSplit = 1, kSchedBalanced = 2 };
int schedule_override() {
  const char* env = getenv("DP_ATTN_SCHEDULE");
  if (!env) return kSchedAuto;
  if (strcmp(env, "split") == 0) return kSchedSplit;
  if (strcmp(env, "balanced") == 0) return kSchedBalanced;
  return kSchedAuto;
}

// Picks the schedule.  Split schedule: the number of key chunks; each block
// runs one (batch, head, chunk, query block) unit and the XCDs receive equal
// contiguous runs of units; the estimated time is (rounds of resident blocks
// per XCD) x (tiles per unit), plus the cost of the extra partial-output
// traffic when the keys are split.  The balanced schedule is priced the same
// way: tiles per resident block plus its partial traffic.
AttnPlan plan_attention(int64_t B, int64_t H, int64_t Tq, int64_t Tkv, int sched) {
  AttnPlan p{};
  p.n_qblk = static_cast<int>((Tq + kBMq - 1) / kBMq);
  p.n_tiles = static_cast<int>((Tkv + kBNk - 1) / kBNk);
  const int slots_per_xcd = std::max(1, device_cus() / kXcds) * blocks_per_cu<false>();
  const double base_units = static_cast<double>(B) * H * p.n_qblk;
  // cost unit: one 64-key tile of one block (~1 us); the split's partial
  // outputs cost their bytes at ~5 TB/s, i.e. ~5 MB per unit
  const double tile_cost = 1.0;
  const double bytes_per_tile_cost = 5.0e6;
  // The split schedule may run the units of its full rounds whole (n_whole
  // of them, the first blocks) and split only the rest: the same rounds, but
  // partial outputs for the last round's units alone.
  const int slots = slots_per_xcd * kXcds;
  const int whole_max = static_cast<int>(base_units) / slots * slots;
  double best = 1e300;
  for (int S = 1; S <= 16 && S <= p.n_tiles; ++S) {
    const int chunk = (p.n_tiles + S - 1) / S;
    const int s_eff = (p.n_tiles + chunk - 1) / chunk;
    if (s_eff != S && S > 1) continue;
    for (int whole : {0, whole_max}) {
      if (whole > 0 && (s_eff == 1 || whole == static_cast<int>(base_units))) continue;
      const double rest = base_units - whole;
      const double per_xcd = std::ceil(rest * s_eff / kXcds);
      const double rounds = static_cast<double>(whole) / slots + std::ceil(per_xcd / slots_per_xcd) * chunk /
                                                                      static_cast<double>(p.n_tiles);
      double cost = rounds * p.n_tiles * tile_cost;
      if (s_eff > 1)
        cost += (static_cast<double>(s_eff) * 8.0 + 2.0) * (rest / base_units) * B * Tq * H * kD / bytes_per_tile_cost;
      if (cost < best * 0.999) {
        best = cost;
        p.n_split = s_eff;
        p.chunk_tiles = chunk;
        p.n_whole = whole;
      }
    }
  }
  // Balanced schedule: one block per resident slot, each owning an equal
  // contiguous share of the (unit, tile) sequence; at most two partial pieces
  // per block go through the combine.  Blocks then read their keys at
  // staggered offsets instead of in step with the other query blocks of their
  // (batch, head), so their L2 reuse is lower: taken only where the K/V
  // buffers fit well inside the last-level cache (half of its 256 MB) and the
  // estimate beats the split schedule by 3%.  `sched` forces either
  // schedule (DP_ATTN_SCHEDULE=split or =balanced, for tests and tuning).
  {
    const int sk_slots = std::max(1, device_cus() / kXcds) * blocks_per_cu<true>() * kXcds;
    const long long work = static_cast<long long>(base_units) * p.n_tiles;
    const double per_slot = std::ceil(static_cast<double>(work) / sk_slots);
    const double sk_cost = per_slot + 2.0 * tile_cost +
                           (2.0 * sk_slots * kBMq * kD * 8.0 + 2.0 * B * Tq * H * kD) / bytes_per_tile_cost;
    const double kv_bytes = 2.0 * B * Tkv * H * kD * 2;
    const bool force_sk = sched == kSchedBalanced;
    const bool force_split = sched == kSchedSplit;
    if (!force_split && (force_sk || (sk_cost < best * 0.97 && kv_bytes <= 128.0e6))) {
      p.sk = 1;
      p.work = work;
      p.n_split = 1;
      p.chunk_tiles = p.n_tiles;
      p.n_whole = 0;
      p.units = static_cast<int>(base_units);
      p.units_per_xcd = 0;
      p.grid = sk_slots;
      p.ws_bytes = static_cast<size_t>(sk_slots) * 2 * (kBMq * kD + kBMq * 2) * sizeof(float);
      return p;
    }
  }
  p.units = (static_cast<int>(base_units) - p.n_whole) * p.n_split;
  p.units_per_xcd = (p.units + kXcds - 1) / kXcds;
  p.grid = p.n_whole + p.units_per_xcd * kXcds;
  p.ws_bytes = p.n_split > 1 ? static_cast<size_t>(p.n_split) * B * Tq * H * kD * sizeof(float) +
                                   static_cast<size_t>(p.n_split) * B * H * Tq * 2 * sizeof(float)
                             : 0;
  return p;
}

// ------------------------------------------------------------------ f32 path
constexpr int kFQ = 128, kFK = 32;

template <int D>
__global__ void __launch_bounds__(kFQ)
attn_f32(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
         float* __restrict__ out, int Tq, int Tkv, int H, float scale) {
  __shared__ float Ks[kFK][D];
  __shared__ float Vs[kFK][D];
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t C = static_cast<int64_t>(H) * D;
  const int qi = blockIdx.x * kFQ + threadIdx.x;
  const bool q_ok = qi < Tq;
  float qr[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = q_ok ? q[(static_cast<int64_t>(b) * Tq + qi) * C + h * D + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* kb = k + static_cast<int64_t>(b) * Tkv * C + h * D;
  const float* vb = v + static_cast<int64_t>(b) * Tkv * C + h * D;
  for (int key0 = 0; key0 < Tkv; key0 += kFK) {
    for (int e = threadIdx.x; e < kFK * D; e += kFQ) {
      const int j = e / D, dd = e % D;
      const bool ok = key0 + j < Tkv;
      Ks[j][dd] = ok ? kb[static_cast<int64_t>(key0 + j) * C + dd] : 0.f;
      Vs[j][dd] = ok ? vb[static_cast<int64_t>(key0 + j) * C + dd] : 0.f;
    }
    __syncthreads();
    const int nk = min(kFK, Tkv - key0);
    float s[kFK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kFK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qr[e], Ks[j][e], dot);
      s[j] = j < nk ? dot * scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kFK; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, Vs[j][e], o[e]);
    }
    m = m_new;
    __syncthreads();
  }
  if (q_ok) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) out[(static_cast<int64_t>(b) * Tq + qi) * C + h * D + e] = o[e] * inv;
  }
}

}  // namespace

DP_API size_t dp_attn_stale_kv_workspace(int64_t B, int64_t H, int64_t Tq, int64_t T_kv, int64_t d,
                                         dp_dtype dt) {
  if (dt != DP_BF16 || d != kD || B <= 0 || H <= 0 || Tq <= 0 || T_kv <= 0) return 0;
  // Enough for either schedule, so the size does not depend on which one a
  // later call picks (or is forced to).
  return std::max(plan_attention(B, H, Tq, T_kv, kSchedSplit).ws_bytes,
                  plan_attention(B, H, Tq, T_kv, kSchedBalanced).ws_bytes);
}

DP_API dp_status dp_attn_stale_kv(const void* q, const void* k_buf, const void* v_buf, void* out,
                                  int64_t B, int64_t H, int64_t Tq, int64_t T_kv, int64_t d,
                                  float scale, dp_dtype dt, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  using dp::fail;
  if (!q || !k_buf || !v_buf || !out) return fail(DP_ERR_INVALID_ARG, "dp_attn_stale_kv: NULL pointer");
  if (B <= 0 || H <= 0 || Tq <= 0 || T_kv <= 0 || d <= 0)
    return fail(DP_ERR_INVALID_ARG, "dp_attn_stale_kv: sizes must be positive");
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "dp_attn_stale_kv: bad dtype");
  const size_t es = dp::dtype_size(dt);
  const size_t qb = static_cast<size_t>(B * Tq * H * d) * es, kb = static_cast<size_t>(B * T_kv * H * d) * es;
  if (dp::overlaps(out, qb, q, qb) || dp::overlaps(out, qb, k_buf, kb) || dp::overlaps(out, qb, v_buf, kb))
    return fail(DP_ERR_INVALID_ARG, "dp_attn_stale_kv: output overlaps an input");
  if (!(dt == DP_BF16 && d == 64) && !(dt == DP_F32 && (d == 32 || d == 64)))
    return fail(DP_ERR_UNSUPPORTED, "dp_attn_stale_kv: head dim %lld not supported for this dtype",
                (long long)d);
  if (Tq > 0x7FFFFFFF || T_kv > 0x7FFFFFFF || H > 65535 || B > 65535)
    return fail(DP_ERR_UNSUPPORTED, "dp_attn_stale_kv: size exceeds grid limits");
  if (dt == DP_BF16 && (!dp::aligned16(q) || !dp::aligned16(k_buf) || !dp::aligned16(v_buf) || !dp::aligned16(out)))
    return fail(DP_ERR_INVALID_ARG, "dp_attn_stale_kv: q, k_buf, v_buf and out must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
  dp::clear_error();
  if (dt == DP_BF16) {
    if (T_kv * H * d > 0x7FFFFFFF || Tq * H * d > 0x7FFFFFFF)
      return fail(DP_ERR_UNSUPPORTED, "dp_attn_stale_kv: one batch item exceeds 2^31 elements");
    const AttnPlan p = plan_attention(B, H, Tq, T_kv, schedule_override());
    if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes))
      return fail(DP_ERR_INVALID_ARG, "dp_attn_stale_kv: workspace %zu < %zu bytes", ws_bytes, p.ws_bytes);
    AttnArgs args;
    args.q = static_cast<const bf16_t*>(q);
    args.k = static_cast<const bf16_t*>(k_buf);
    args.v = static_cast<const bf16_t*>(v_buf);
    args.out = static_cast<bf16_t*>(out);
    args.part_o = static_cast<float*>(ws);
    args.part_ml = p.ws_bytes ? args.part_o + static_cast<size_t>(p.n_split) * B * Tq * H * kD : nullptr;
    args.B = (int)B;
    args.H = (int)H;
    args.Tq = (int)Tq;
    args.Tkv = (int)T_kv;
    args.c = sc * kLog2e;
    args.n_qblk = p.n_qblk;
    args.n_split = p.n_split;
    args.chunk_tiles = p.chunk_tiles;
    args.n_tiles = p.n_tiles;
    args.units = p.units;
    args.units_per_xcd = p.units_per_xcd;
    args.n_whole = p.n_whole;
    args.sk = p.sk;
    args.sk_grid = p.grid;
    args.work = p.work;
    if (p.sk) {
      args.part_ml = args.part_o + static_cast<size_t>(p.grid) * 2 * kBMq * kD;
    }
    if (p.sk)
      hipLaunchKernelGGL(attn_bf16_d64<true>, dim3(static_cast<unsigned>(p.grid)), dim3(256), 0, stream, args);
    else
      hipLaunchKernelGGL(attn_bf16_d64<false>, dim3(static_cast<unsigned>(p.grid)), dim3(256), 0, stream, args);
    if (p.sk) {
      const int64_t threads = B * Tq * H * 8;
      hipLaunchKernelGGL(attn_combine_sk, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                         stream, args.part_o, args.part_ml, args.out, (int)B, (int)H, (int)Tq, p.n_qblk,
                         p.n_tiles, p.work, p.grid);
    } else if (p.n_split > 1) {
      const int64_t split_units = B * H * p.n_qblk - p.n_whole;
      const dim3 grid(static_cast<unsigned>(split_units * kCombineBlocksPerUnit));
      switch (p.n_split) {
        case 2:
          hipLaunchKernelGGL(attn_combine<2>, grid, dim3(256), 0, stream, args.part_o, args.part_ml, args.out, (int)B,
                             (int)H, (int)Tq, p.n_split, p.n_whole, p.n_qblk);
          break;
        case 3:
          hipLaunchKernelGGL(attn_combine<3>, grid, dim3(256), 0, stream, args.part_o, args.part_ml, args.out, (int)B,
                             (int)H, (int)Tq, p.n_split, p.n_whole, p.n_qblk);
          break;
        case 4:
          hipLaunchKernelGGL(attn_combine<4>, grid, dim3(256), 0, stream, args.part_o, args.part_ml, args.out, (int)B,
                             (int)H, (int)Tq, p.n_split, p.n_whole, p.n_qblk);
          break;
        default:
          hipLaunchKernelGGL(attn_combine<0>, grid, dim3(256), 0, stream, args.part_o, args.part_ml, args.out, (int)B,
                             (int)H, (int)Tq, p.n_split, p.n_whole, p.n_qblk);
          break;
      }
    }
  } else {
    const dim3 grid(static_cast<unsigned>((Tq + kFQ - 1) / kFQ), static_cast<unsigned>(H),
                    static_cast<unsigned>(B));
    if (d == 32)
      hipLaunchKernelGGL(attn_f32<32>, grid, dim3(kFQ), 0, stream, static_cast<const float*>(q),
                         static_cast<const float*>(k_buf), static_cast<const float*>(v_buf),
                         static_cast<float*>(out), (int)Tq, (int)T_kv, (int)H, sc);
    else
      hipLaunchKernelGGL(attn_f32<64>, grid, dim3(kFQ), 0, stream, static_cast<const float*>(q),
                         static_cast<const float*>(k_buf), static_cast<const float*>(v_buf),
                         static_cast<float*>(out), (int)Tq, (int)T_kv, (int)H, sc);
  }
  return dp::check_launch("dp_attn_stale_kv");
}
