// GroupNorm of the rank's tokens with whole-image statistics: fresh sums over
// the local tokens plus stale sums from the other patches.
//
// Method source: "OTIL for SDXL on 4x L40S", "What is implemented where" (two
// scalars per group, combined across slices, decide slice brightness and
// contrast) and the xDiT issue thread "Tensor Parallelism with Stale
// Activations ..." (a feature may combine fresh partial values with stale ones).
//
// Two launches, deterministic (fixed reduction order, no float atomics, no
// block ever waits for another):
//   1. gn_partial over (token tile, batch item): per tile and group (sum x,
//      sum x^2) into the workspace; each block then takes a ticket, and the
//      block that arrives last for its batch item folds that item's tile
//      partials, in one fixed order, into the local sums [B, G, 2] (also the
//      fresh sums the caller may ask for).  Tickets are two-level (16 blocks
//      per first-level counter): on MI355X a single counter taken by ~500
//      blocks costs ~5 us of contention, two levels ~1 us.
//   2. gn_apply over its own, finer (token tile, batch item) grid: every block
//      reads the local sums, adds the other patches' stale sums, derives
//      a_c = rstd*gamma_c and b_c = beta_c - mean*a_c and writes
//      y = x * a_c + b_c (optional SiLU) for its tile: a plain streaming pass.
// The tile partials and the tickets cross XCDs inside one launch, so they are
// written and read with device-coherent accesses (agent-scope atomic loads
// and stores, which bypass the non-coherent per-XCD L2), ordered by a wait for
// the stores' completion before the ticket.  The last arrivals put the
// counters back to zero, so a workspace that starts zero-filled stays ready.
//
// Every thread owns one 16-byte channel vector of a token, so loads and stores
// are 16 B wide and consecutive threads touch consecutive bytes.
#include <algorithm>
#include <mutex>

#include "dp_internal.h"

namespace {

constexpr int kThreads = 512;
constexpr int kTargetBlocks = 512;  // sums pass: about two blocks per CU
constexpr int kUnroll = 8;          // 16-byte loads in flight per thread (the sums pass's remainder switch assumes 8)
constexpr int kApplyPasses = 8;     // apply pass: token passes per thread
constexpr int kTicketGroup = 16;    // blocks per first-level ticket counter
constexpr int kCounterStride = 32;  // uints between counters (one 128-byte line each)
// Ticket counters live in a fixed region at the start of the workspace, the
// same for every shape, and nothing else is ever written there: a workspace
// zero-filled once stays valid for any sequence of calls.  A sums-pass launch
// covers at most kMaxChunk batch items, so its counters always fit.
constexpr int kCounterBytes = 32768;
constexpr int kMaxChunk = 128;

struct GnArgs {
  const void* x;
  void* y;
  float2* partial;     // [B][tiles][G] (sums pass)
  unsigned* counters;  // [B][1 + ticket groups] ticket counters, kCounterStride apart
  float* sums;         // [B][G][2] the folded local sums (sums pass output)
  const float* stale;  // [n_patches][B][G][2]
  const float* gamma;
  const float* beta;
  float* fresh;        // [B][G][2] second copy of the local sums, or NULL
  const float* given;  // [B][G][2] local sums the apply pass normalises with
  int T, C, G, tiles, tile_tokens, n_patches, rank, B, silu, counter_stride;
  int b0;  // first batch item of the launch (blockIdx.y counts from it); B is the total
  float inv_count, eps;
};

// Upper bound of tiles per batch item of the sums pass, independent of C,
// dtype and device (it sizes the workspace).
int64_t max_tiles(int64_t B, int64_t T) {
  const int64_t want = (kTargetBlocks + B - 1) / B;
  return want < T ? want : T;
}

// ------------------------------------------------------------ device helpers
template <bool BF16>
__device__ __forceinline__ void unpack_vec(const u32x4& u, float* v) {
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(u[j]);
      v[2 * j + 1] = bf16_hi(u[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(u[j]);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack_vec(const float* v) {
  u32x4 u;
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = __float_as_uint(v[j]);
  }
  return u;
}

// Byte offset of the 16-byte vector vi of token t of batch item b.
template <bool BF16>
__device__ __forceinline__ int64_t vec_byte(int b, int t, int vi, const GnArgs& a) {
  return ((static_cast<int64_t>(b) * a.T + t) * a.C) * (BF16 ? 2 : 4) + static_cast<int64_t>(vi) * 16;
}

template <bool BF16>
__device__ __forceinline__ void acc_vec(const u32x4& u, float* s1, float* s2) {
  constexpr int VEC = BF16 ? 8 : 4;
  float v[VEC];
  unpack_vec<BF16>(u, v);
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    s1[j] += v[j];
    s2[j] = fmaf(v[j], v[j], s2[j]);
  }
}

// Adds R block passes of the thread's channel vector vi, tokens t0, t0 + tpp,
// ..., to s1/s2 (zeros when `on` is false).  The loads are unconditional (a
// token at or past t_end re-reads token t_end - 1 and adds zeros), so they
// all go out before the first add and each add waits only for its own load.
template <bool BF16, int R>
__device__ __forceinline__ void acc_passes(const GnArgs& a, int b, int t0, int tpp, int t_end, int vi, bool on,
                                           float* s1, float* s2) {
  u32x4 raw[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int t = min(t0 + u * tpp, t_end - 1);
    raw[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + vec_byte<BF16>(b, t, vi, a));
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const bool ok = on && t0 + u * tpp < t_end;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = ok ? raw[u][e] : 0u;
    acc_vec<BF16>(w, s1, s2);
  }
}

// gamma/beta of the thread's VEC channels (1 and 0 when NULL); vector loads
// when the arrays are 16-byte aligned.
__device__ __forceinline__ void load_param(const float* p, int c0, int n, float dflt, float* out) {
  if (!p) {
    for (int j = 0; j < n; ++j) out[j] = dflt;
  } else if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    for (int j = 0; j < n; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + c0 + j);
      out[j] = v[0];
      out[j + 1] = v[1];
      out[j + 2] = v[2];
      out[j + 3] = v[3];
    }
  } else {
    for (int j = 0; j < n; ++j) out[j] = p[c0 + j];
  }
}

template <int VEC>
__device__ __forceinline__ void load_affine(const GnArgs& a, int vi, float* gm, float* bt) {
  load_param(a.gamma, vi * VEC, VEC, 1.f, gm);
  load_param(a.beta, vi * VEC, VEC, 0.f, bt);
}

// Lanes per group for the block reductions below: a group's partial sums
// are spread over `lanes` adjacent threads (so, when lanes <= 64, over lanes
// of one wave, combined by a fixed shuffle tree).
__device__ __forceinline__ int group_lanes(int G) {
  int l = kThreads / G;
  if (l > 64) l = 64;
  if (l < 1) l = 1;
  return 1 << (31 - __clz(l));  // a power of two
}

// Sum of v over `lanes` adjacent lanes (a power of two <= 64), the same
// order-fixed total in every lane.  Up to 16 lanes by DPP within a row: swap
// neighbours, then pairs, then mirror the half-rows and the row (each step
// adds two equal-sized partial totals, so all lanes of a group agree); beyond
// that by an xor butterfly through LDS permutes.  Every lane of the wave must
// be active.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int o = 0;
  const int x = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: o = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: o = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: o = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: o = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return v + __int_as_float(o);
}
__device__ __forceinline__ float2 lane_sum(float2 v, int lanes) {
  if (lanes <= 16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if ((2 << k) > lanes) break;
      v.x = dpp_add(v.x, k);
      v.y = dpp_add(v.y, k);
    }
    return v;
  }
  for (int off = 1; off < lanes; off <<= 1) {
    v.x += __shfl_xor(v.x, off, 64);
    v.y += __shfl_xor(v.y, off, 64);
  }
  return v;
}

// Block-wide per-group sums of the per-thread channel sums s1/s2 (thread =
// token lane tl x channel vector vi), in a fixed order and in two steps: the
// threads' sums go to lds_r as [2][tpp][C]; thread c adds channel c over the
// token lanes, in lane order, into chan[c]; then one thread per group adds
// the group's channel sums in order (groups of more than 32 channels: 16
// lanes take channels j, j + 16, ... and are combined by lane_sum).  Every LDS
// access of the first two steps is unit-stride across threads.  The result
// lands in gsum[G].  Starts and ends with a barrier.
template <int VEC>
__device__ void block_group_sums(const float* s1, const float* s2, bool active, int tl, int vi,
                                 int tpp, int C, int G, float* lds_r, float2* chan, float2* gsum) {
  __syncthreads();
  if (active) {
    f32x4* r1 = reinterpret_cast<f32x4*>(lds_r + tl * C + vi * VEC);
    f32x4* r2 = reinterpret_cast<f32x4*>(lds_r + (tpp + tl) * C + vi * VEC);
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      r1[j] = f32x4{s1[4 * j], s1[4 * j + 1], s1[4 * j + 2], s1[4 * j + 3]};
      r2[j] = f32x4{s2[4 * j], s2[4 * j + 1], s2[4 * j + 2], s2[4 * j + 3]};
    }
  }
  __syncthreads();
  constexpr int U = 8;
  for (int c = threadIdx.x; c < C; c += kThreads) {
    float2 acc = make_float2(0.f, 0.f);
    for (int t0 = 0; t0 < tpp; t0 += U) {
      float v1[U], v2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(t0 + u, tpp - 1);
        v1[u] = lds_r[t * C + c];
        v2[u] = lds_r[(tpp + t) * C + c];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t0 + u < tpp) {
          acc.x += v1[u];
          acc.y += v2[u];
        }
      }
    }
    chan[c] = acc;
  }
  __syncthreads();
  const int Cg = C / G;
  if (Cg <= 32) {  // one thread per group, its channels in order
    for (int g = threadIdx.x; g < G; g += kThreads) {
      float2 acc = make_float2(0.f, 0.f);
      for (int e0 = 0; e0 < Cg; e0 += U) {
        float2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = chan[g * Cg + min(e0 + u, Cg - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (e0 + u < Cg) {
            acc.x += v[u].x;
            acc.y += v[u].y;
          }
        }
      }
      gsum[g] = acc;
    }
  } else {  // 16 lanes per group: channels j, j + 16, ..., then lane_sum
    for (int f = threadIdx.x; f < ((G * 16 + 63) / 64) * 64; f += kThreads) {
      const int g = f >> 4, j = f & 15;
      float2 acc = make_float2(0.f, 0.f);
      if (g < G) {
        for (int e = j; e < Cg; e += 16) {
          const float2 v = chan[g * Cg + e];
          acc.x += v.x;
          acc.y += v.y;
        }
      }
      acc = lane_sum(acc, 16);
      if (g < G && j == 0) gsum[g] = acc;
    }
  }
  __syncthreads();
}

// Device-coherent 8-byte store and load (agent scope: they bypass the per-XCD
// L2, so blocks on other XCDs see them within the same launch).
__device__ __forceinline__ void store_coherent(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __builtin_bit_cast(unsigned long long, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent(const float2* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Folds the tile partials of batch item b into red[g] (float2 per group).
// The loads are coalesced: thread f = q * G + g takes group g of tiles q,
// q + lanes, ..., U loads in flight per pass (indexes past the last tile
// re-read that tile and are not added); its sum goes to red[f], and after a
// barrier the group's `lanes` sums are combined by lane_sum over adjacent
// threads.  One fixed order, whichever block runs it.  red holds
// lanes * G float2.  Starts and ends with a barrier.
__device__ void fold_partials(const GnArgs& a, int b, float2* red) {
  const int G = a.G, lanes = group_lanes(G);
  const float2* pb = a.partial + static_cast<int64_t>(b) * a.tiles * G;
  constexpr int U = 16;
  __syncthreads();
  for (int f = threadIdx.x; f < lanes * G; f += kThreads) {
    const int g = f % G, q = f / G;
    float2 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = make_float2(0.f, 0.f);
    for (int t0 = q; t0 < a.tiles; t0 += U * lanes) {
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = load_coherent(pb + static_cast<int64_t>(min(t0 + u * lanes, a.tiles - 1)) * G + g);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t0 + u * lanes < a.tiles) {
          acc[u].x += v[u].x;
          acc[u].y += v[u].y;
        }
      }
    }
    float2 s = acc[0];
#pragma unroll
    for (int u = 1; u < U; ++u) {
      s.x += acc[u].x;
      s.y += acc[u].y;
    }
    red[f] = s;
  }
  __syncthreads();
  float2 mine[(2048 + kThreads - 1) / kThreads];
  int k = 0;
  for (int f = threadIdx.x; f < ((G * lanes + 63) / 64) * 64; f += kThreads, ++k) {
    const int g = f / lanes, q = f % lanes;
    const float2 v = lane_sum(g < G ? red[q * G + g] : make_float2(0.f, 0.f), lanes);
    mine[k] = v;
  }
  __syncthreads();
  k = 0;
  for (int f = threadIdx.x; f < ((G * lanes + 63) / 64) * 64; f += kThreads, ++k) {
    const int g = f / lanes, q = f % lanes;
    if (g < G && q == 0) red[g] = mine[k];
  }
  __syncthreads();
}

// (mean, rstd) of one group from its sums over the image (biased variance,
// clamped at zero since stale remote sums can make it negative), and a
// channel's (scale, shift) from them.  Explicit fused operations, so every
// kernel that calls these rounds identically.
__device__ __forceinline__ float2 group_stats(float f1, float f2, float inv_count, float eps) {
  const float mean = f1 * inv_count;
  const float var = fmaxf(fmaf(-mean, mean, f2 * inv_count), 0.f);
  return make_float2(mean, 1.0f / sqrtf(var + eps));
}
__device__ __forceinline__ float2 channel_affine(float2 ms, float gamma, float beta) {
  const float sc = ms.y * gamma;
  return make_float2(sc, fmaf(-ms.x, sc, beta));
}

// Patches from p_start on are taken eight at a time, all eight loads in
// flight before any is added.
__device__ __forceinline__ float2 add_stale(const GnArgs& a, float2 loc, int gb, int g, int p_start) {
  constexpr int U = 8;
  for (int p0 = p_start; p0 < a.n_patches; p0 += U) {
    float2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* st = a.stale + ((static_cast<int64_t>(min(p0 + u, a.n_patches - 1)) * a.B + gb) * a.G + g) * 2;
      v[u] = make_float2(st[0], st[1]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p0 + u < a.n_patches && p0 + u != a.rank) {
        loc.x += v[u].x;
        loc.y += v[u].y;
      }
    }
  }
  return loc;
}
// ------------------------------------------------------------ tickets
// Counts block `tile` of batch item b in; true for exactly one block, the last
// of the item's `tiles` to arrive.  First-level counters take kTicketGroup
// blocks each, the item's top counter one arrival per group.  Every counter is
// back at zero once all blocks of the launch have arrived.
__device__ bool take_ticket(const GnArgs& a, int b, int tile) {
  unsigned* base = a.counters + static_cast<int64_t>(b) * a.counter_stride;
  const int grp = tile / kTicketGroup;
  const unsigned in_grp = static_cast<unsigned>(min(kTicketGroup, a.tiles - grp * kTicketGroup));
  const unsigned n_grp = static_cast<unsigned>((a.tiles + kTicketGroup - 1) / kTicketGroup);
  unsigned* gc = base + (1 + grp) * kCounterStride;
  if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != in_grp - 1) return false;
  __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__hip_atomic_fetch_add(base, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != n_grp - 1) return false;
  __hip_atomic_store(base, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ------------------------------------------------------------ kernels
// Sums pass: tile partials, then the last block of each batch item folds them
// into a.sums (and a.fresh when given).
template <bool BF16>
__global__ void __launch_bounds__(kThreads) gn_partial(GnArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;
  __shared__ __attribute__((aligned(16))) float lds_r[2 * kThreads * VEC];
  __shared__ __attribute__((aligned(16))) float lds_c[2 * 2048];
  __shared__ float2 gsum[2048];
  __shared__ int last;
  const int vpt = a.C / VEC, tpp = kThreads / vpt;
  const int tid = threadIdx.x, tl = tid / vpt, vi = tid % vpt;
  const bool active = tl < tpp;
  const int b = blockIdx.y, tile = blockIdx.x;
  const int t_begin = tile * a.tile_tokens;
  const int t_end = min(a.T, t_begin + a.tile_tokens);
  const int npass = a.tile_tokens / tpp;

  float s1[VEC], s2[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) s1[j] = s2[j] = 0.f;
  // idle threads (tl >= tpp) read the last token lane's vectors, which that
  // lane's wave reads anyway, and add zeros
  const int tlr = min(tl, tpp - 1);
  int k0 = 0;
  for (; k0 + kUnroll <= npass; k0 += kUnroll)
    acc_passes<BF16, kUnroll>(a, b, t_begin + tlr + k0 * tpp, tpp, t_end, vi, active, s1, s2);
  const int t0 = t_begin + tlr + k0 * tpp;
  static_assert(kUnroll == 8, "one case per remainder below");
  switch (npass - k0) {  // the remaining passes, fewer than kUnroll
    case 1: acc_passes<BF16, 1>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    case 2: acc_passes<BF16, 2>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    case 3: acc_passes<BF16, 3>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    case 4: acc_passes<BF16, 4>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    case 5: acc_passes<BF16, 5>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    case 6: acc_passes<BF16, 6>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    case 7: acc_passes<BF16, 7>(a, b, t0, tpp, t_end, vi, active, s1, s2); break;
    default: break;
  }
  block_group_sums<VEC>(s1, s2, active, tl, vi, tpp, a.C, a.G, lds_r, reinterpret_cast<float2*>(lds_c), gsum);
  for (int g = tid; g < a.G; g += kThreads)
    store_coherent(a.partial + (static_cast<int64_t>(b) * a.tiles + tile) * a.G + g, gsum[g]);
  // the block's partials are complete at the coherence point before its ticket
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) last = take_ticket(a, b, tile);
  __syncthreads();
  if (!last) return;
  fold_partials(a, b, gsum);
  for (int g = tid; g < a.G; g += kThreads) {
    const float2 f = gsum[g];
    const int64_t o = (static_cast<int64_t>(b) * a.G + g) * 2;
    a.sums[o] = f.x;
    a.sums[o + 1] = f.y;
    if (a.fresh) {
      a.fresh[o] = f.x;
      a.fresh[o + 1] = f.y;
    }
  }
}

// Apply passes: y = x * scale_c + shift_c (SiLU optional) over a tile of
// tokens.  A thread owns one 16-byte channel vector of kApplyPasses tokens
// (tokens tl, tl + tpp, ...), issues all its loads at once and stores with
// nontemporal 16-byte writes.
// SILU is a template parameter: a runtime branch would have the compiler
// evaluate the SiLU's two transcendentals for every element and then select.
template <bool BF16, bool SILU>
__device__ __forceinline__ void apply_store(const GnArgs& a, const u32x4* raw, int64_t base, int stride_vec,
                                            int n, const float* sc, const float* sh) {
  constexpr int VEC = BF16 ? 8 : 4;
#pragma unroll
  for (int u = 0; u < kApplyPasses; ++u) {
    if (u >= n) break;
    float v[VEC];
    unpack_vec<BF16>(raw[u], v);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      float z = fmaf(v[j], sc[j], sh[j]);
      if constexpr (SILU) z *= __builtin_amdgcn_rcpf(1.0f + __expf(-z));  // v_rcp_f32, 1 ulp
      v[j] = z;
    }
    __builtin_nontemporal_store(pack_vec<BF16>(v), static_cast<u32x4*>(a.y) + base + static_cast<int64_t>(u) * stride_vec);
  }
}

// The thread's tokens: n of them, starting at vector index `base` of x/y
// (16-byte units), stride_vec apart.  Idle threads (false) get the last token
// lane's slot with n = 0.
template <bool BF16, int NT>
__device__ __forceinline__ bool apply_slot(const GnArgs& a, int& vi, int64_t& base, int& stride_vec, int& n) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int vpt = a.C / VEC, tpp = NT / vpt;
  const int tl = threadIdx.x / vpt;
  vi = threadIdx.x - tl * vpt;
  const int t = blockIdx.x * a.tile_tokens + min(tl, tpp - 1);
  n = t < a.T && tl < tpp ? min(kApplyPasses, (a.T - t + tpp - 1) / tpp) : 0;
  base = (static_cast<int64_t>(blockIdx.y) * a.T + min(t, a.T - 1)) * vpt + vi;
  stride_vec = tpp * vpt;
  return tl < tpp;
}

// The thread's kApplyPasses x vectors, loaded unconditionally so that every
// load is in flight before the first is used and each use waits only for its
// own: passes from n on re-read pass n - 1 (pass 0 when n = 0, whose base
// apply_slot clamps to the last token), and their stores are skipped.
__device__ __forceinline__ void apply_loads(const GnArgs& a, int64_t base, int stride_vec, int n, u32x4* raw) {
  const u32x4* x = static_cast<const u32x4*>(a.x);
#pragma unroll
  for (int u = 0; u < kApplyPasses; ++u) raw[u] = x[base + static_cast<int64_t>(min(u, max(n - 1, 0))) * stride_vec];
}

// Apply pass, from local sums (the workspace's, after the sums pass, or the
// caller's): the block stages its batch item's local sums and the other
// patches' stale sums in LDS.  With REG (G and n_patches * G at most NT) each
// thread loads one entry of each into registers before its x loads and
// writes them to LDS after issuing those, so no wait for the small loads
// holds up the x loads; otherwise a loop stages them first.  Thread g then
// derives group g's (mean, rstd) from the local sums plus the patches' stale
// sums in patch order, and after a second barrier every thread takes its
// channels' (scale, shift).  Stale sums beyond kStaleLds entries are read
// from memory by thread g instead.
constexpr int kStaleLds = 1024;  // float2 entries: patches * G
template <bool BF16, int NT, bool SILU, bool REG>
__global__ void __launch_bounds__(NT) gn_apply_sums(GnArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;
  __shared__ float2 st_lds[kStaleLds];  // [n_patches][G] stale sums
  __shared__ float2 g_lds[2048];        // [G] local sums, then (mean, rstd)
  int vi = 0, stride_vec = 0, n = 0;
  int64_t base = 0;
  const bool on = apply_slot<BF16, NT>(a, vi, base, stride_vec, n);
  const int G = a.G, Cg = a.C / G, gb = a.b0 + blockIdx.y;
  const bool staged = a.n_patches * G <= kStaleLds;
  const float* loc = a.given + static_cast<int64_t>(blockIdx.y) * G * 2;
  float gm[VEC], bt[VEC];
  u32x4 raw[kApplyPasses];
  if constexpr (REG) {
    // every thread loads (clamped indexes; the stale pointer falls back to
    // the local sums when there are no other patches) and writes only its own
    const int tid = threadIdx.x, fl = min(tid, G - 1);
    const float2 lv = make_float2(loc[fl * 2], loc[fl * 2 + 1]);
    const int fs = min(tid, a.n_patches * G - 1), sp = fs / G, sg = fs - sp * G;
    const float* st = a.n_patches > 1 ? a.stale + ((static_cast<int64_t>(sp) * a.B + gb) * G + sg) * 2 : loc;
    const float2 sv = make_float2(st[0], st[1]);
    load_affine<VEC>(a, vi, gm, bt);
    apply_loads(a, base, stride_vec, n, raw);
    if (tid < G) g_lds[tid] = lv;
    if (a.n_patches > 1 && tid < a.n_patches * G) st_lds[tid] = sv;
  } else {
    for (int f = threadIdx.x; f < G; f += NT) g_lds[f] = make_float2(loc[f * 2], loc[f * 2 + 1]);
    if (staged && a.n_patches > 1) {
      for (int f = threadIdx.x; f < a.n_patches * G; f += NT) {
        const int p = f / G, g = f - p * G;
        const float* st = a.stale + ((static_cast<int64_t>(p) * a.B + gb) * G + g) * 2;
        st_lds[f] = make_float2(st[0], st[1]);
      }
    }
    if (on) load_affine<VEC>(a, vi, gm, bt);
    apply_loads(a, base, stride_vec, n, raw);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += NT) {
    float2 f = g_lds[g];
    if (staged) {
      constexpr int U = 8;
      for (int p0 = 0; p0 < a.n_patches; p0 += U) {
        float2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = st_lds[min(p0 + u, a.n_patches - 1) * G + g];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (p0 + u < a.n_patches && p0 + u != a.rank) {
            f.x += v[u].x;
            f.y += v[u].y;
          }
        }
      }
    } else {
      f = add_stale(a, f, gb, g, 0);
    }
    g_lds[g] = group_stats(f.x, f.y, a.inv_count, a.eps);
  }
  __syncthreads();
  if (!on) return;
  float sc[VEC], sh[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const float2 af = channel_affine(g_lds[(vi * VEC + j) / Cg], gm[j], bt[j]);
    sc[j] = af.x;
    sh[j] = af.y;
  }
  apply_store<BF16, SILU>(a, raw, base, stride_vec, n, sc, sh);
}

// ------------------------------------------------------------ planning
struct GnPlan {
  int tile_tokens, tiles;
};

// Sums pass: tokens per tile a whole number of block passes (tpp tokens each),
// at most max_tiles(B, T) tiles per batch item.
int tokens_per_pass(int64_t C, dp_dtype dt) { return kThreads / static_cast<int>(C / (dt == DP_BF16 ? 8 : 4)); }

GnPlan sums_plan(int64_t B, int64_t T, int64_t C, dp_dtype dt) {
  const int tpp = tokens_per_pass(C, dt);
  const int64_t per_b = max_tiles(B, T);
  int64_t tt = (T + per_b - 1) / per_b;
  tt = (tt + tpp - 1) / tpp * tpp;
  return GnPlan{static_cast<int>(tt), static_cast<int>((T + tt - 1) / tt)};
}

// Apply pass: blocks of 256 threads (512 when a token has more than 256
// channel vectors), kApplyPasses block passes per tile.
int apply_threads(int64_t C, dp_dtype dt) { return C / (dt == DP_BF16 ? 8 : 4) <= 256 ? 256 : 512; }
GnPlan apply_plan(int64_t T, int64_t C, dp_dtype dt) {
  const int64_t tpp = apply_threads(C, dt) / (C / (dt == DP_BF16 ? 8 : 4));
  const int64_t tt = tpp * kApplyPasses;
  return GnPlan{static_cast<int>(tt), static_cast<int>((T + tt - 1) / tt)};
}

// Workspace: the fixed counter region, then for one launch of up to
// kMaxChunk batch items the folded sums and the tile partials.
struct GnWs {
  size_t sums_off, partial_off, total;
  int counter_stride;  // uints per batch item
};
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
GnWs ws_layout(int64_t B, int64_t T, int64_t C, int64_t G) {
  (void)C;
  const int64_t Bc = std::min<int64_t>(B, kMaxChunk);
  GnWs w{};
  const int64_t groups = (max_tiles(Bc, T) + kTicketGroup - 1) / kTicketGroup;
  w.counter_stride = static_cast<int>((1 + groups) * kCounterStride);
  w.sums_off = kCounterBytes;
  w.partial_off = w.sums_off + round256(static_cast<size_t>(Bc) * G * 2 * sizeof(float));
  w.total = w.partial_off + static_cast<size_t>(Bc) * max_tiles(Bc, T) * G * sizeof(float2);
  return w;
}
// Bytes for a call over B batch items: the largest chunk layout it uses.
size_t ws_bytes(int64_t B, int64_t T, int64_t C, int64_t G) {
  size_t n = ws_layout(std::min<int64_t>(B, kMaxChunk), T, C, G).total;
  if (B > kMaxChunk && B % kMaxChunk) n = std::max(n, ws_layout(B % kMaxChunk, T, C, G).total);
  return n;
}
// With at most kMaxChunk batch items per launch, Bc * (1 + ceil(tiles / 16))
// counter lines never exceed the region: checked for every chunk size.
static_assert(kMaxChunk * (1 + ((kTargetBlocks + kMaxChunk - 1) / kMaxChunk + kTicketGroup - 1) / kTicketGroup) *
                      kCounterStride * 4 <= kCounterBytes,
              "counter region");

// Checks shared by the GroupNorm calls; fills the shape fields of `ga`.
dp_status check_common(const char* name, const void* x, int64_t B, int64_t T_loc, int64_t C, int64_t G,
                       dp_dtype dt, GnArgs& ga) {
  using dp::fail;
  if (!x) return fail(DP_ERR_INVALID_ARG, "%s: NULL x", name);
  if (B <= 0 || T_loc <= 0 || C <= 0 || G <= 0) return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (C % G != 0) return fail(DP_ERR_INVALID_ARG, "%s: C %% G != 0", name);
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  const int vec = dt == DP_BF16 ? 8 : 4;
  if (C % vec != 0 || C > 2048 || C / vec > kThreads || T_loc > 0x7FFFFFFF || B > 65535 || B * G > 0x7FFFFFFF)
    return fail(DP_ERR_UNSUPPORTED, "%s: C=%lld G=%lld not supported", name, (long long)C, (long long)G);
  if (!dp::aligned16(x)) return fail(DP_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", name);
  ga.x = x;
  ga.T = static_cast<int>(T_loc);
  ga.C = static_cast<int>(C);
  ga.G = static_cast<int>(G);
  ga.B = static_cast<int>(B);
  return DP_OK;
}

dp_status check_stats_args(const char* name, const float* stale_sums, int64_t n_patches, int64_t rank,
                           int64_t T_total, int64_t T_loc, float eps) {
  using dp::fail;
  if (n_patches <= 0) return fail(DP_ERR_INVALID_ARG, "%s: n_patches must be positive", name);
  if (!stale_sums && n_patches > 1)
    return fail(DP_ERR_INVALID_ARG, "%s: NULL stale_sums with %lld patches", name, (long long)n_patches);
  if (rank < 0 || rank >= n_patches)
    return fail(DP_ERR_INVALID_ARG, "%s: rank %lld outside [0, %lld)", name, (long long)rank, (long long)n_patches);
  if (T_total < T_loc) return fail(DP_ERR_INVALID_ARG, "%s: T_total < T_loc", name);
  if (!(eps >= 0.f)) return fail(DP_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
  return DP_OK;
}

void set_stats(GnArgs& ga, const float* stale_sums, int64_t n_patches, int64_t rank, int64_t T_total,
               const float* gamma, const float* beta, float eps, int fuse_silu) {
  ga.stale = stale_sums;
  ga.gamma = gamma;
  ga.beta = beta;
  ga.n_patches = static_cast<int>(n_patches);
  ga.rank = static_cast<int>(rank);
  ga.silu = fuse_silu;
  ga.inv_count = static_cast<float>(1.0 / (static_cast<double>(T_total) * (ga.C / ga.G)));
  ga.eps = eps;
}

// Sums pass over batch items [b0, b0 + Bc) of the call (Bc <= kMaxChunk):
// local sums into the workspace (and `fresh`, already offset to b0).
void launch_sums(GnArgs ga, int b0, int Bc, void* ws, float* fresh, dp_dtype dt, hipStream_t st) {
  const GnWs w = ws_layout(Bc, ga.T, ga.C, ga.G);
  const GnPlan p = sums_plan(Bc, ga.T, ga.C, dt);
  char* base = static_cast<char*>(ws);
  ga.x = static_cast<const char*>(ga.x) + static_cast<size_t>(b0) * ga.T * ga.C * dp::dtype_size(dt);
  ga.b0 = b0;
  ga.counters = reinterpret_cast<unsigned*>(base);
  ga.counter_stride = w.counter_stride;
  ga.sums = reinterpret_cast<float*>(base + w.sums_off);
  ga.partial = reinterpret_cast<float2*>(base + w.partial_off);
  ga.fresh = fresh;
  ga.tiles = p.tiles;
  ga.tile_tokens = p.tile_tokens;
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(Bc));
  if (dt == DP_BF16) hipLaunchKernelGGL(gn_partial<true>, grid, dim3(kThreads), 0, st, ga);
  else hipLaunchKernelGGL(gn_partial<false>, grid, dim3(kThreads), 0, st, ga);
}

// Apply pass over batch items [b0, b0 + Bc) from their local sums
// `local_sums` ([Bc][G][2]) and the stale sums.
void launch_apply(GnArgs ga, int b0, int Bc, const float* local_sums, void* y, dp_dtype dt, hipStream_t st) {
  const GnPlan p = apply_plan(ga.T, ga.C, dt);
  const size_t off = static_cast<size_t>(b0) * ga.T * ga.C * dp::dtype_size(dt);
  ga.x = static_cast<const char*>(ga.x) + off;
  ga.y = static_cast<char*>(y) + off;
  ga.b0 = b0;
  ga.given = local_sums;
  ga.tiles = p.tiles;
  ga.tile_tokens = p.tile_tokens;
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(Bc));
  const bool wide = apply_threads(ga.C, dt) == 512;
  const int nt = wide ? 512 : 256;
  const bool reg = ga.G <= nt && static_cast<int64_t>(ga.n_patches) * ga.G <= nt;
  const int k = (dt == DP_BF16 ? 8 : 0) + (wide ? 4 : 0) + (ga.silu ? 2 : 0) + (reg ? 1 : 0);
  switch (k) {
#define DP_GN_SUMS(K, BF, NT, SI) \
  case 2 * K: hipLaunchKernelGGL((gn_apply_sums<BF, NT, SI, false>), grid, dim3(NT), 0, st, ga); break; \
  case 2 * K + 1: hipLaunchKernelGGL((gn_apply_sums<BF, NT, SI, true>), grid, dim3(NT), 0, st, ga); break;
    DP_GN_SUMS(0, false, 256, false)
    DP_GN_SUMS(1, false, 256, true)
    DP_GN_SUMS(2, false, 512, false)
    DP_GN_SUMS(3, false, 512, true)
    DP_GN_SUMS(4, true, 256, false)
    DP_GN_SUMS(5, true, 256, true)
    DP_GN_SUMS(6, true, 512, false)
    DP_GN_SUMS(7, true, 512, true)
#undef DP_GN_SUMS
  }
}

}  // namespace

DP_API size_t dp_groupnorm_stale_stats_workspace(int64_t B, int64_t T_loc, int64_t C, int64_t G) {
  if (B <= 0 || T_loc <= 0 || C <= 0 || G <= 0) return 0;
  return ws_bytes(B, T_loc, C, G);
}

DP_API dp_status dp_groupnorm_stale_stats(const void* x, const float* stale_sums, int64_t n_patches,
                                          int64_t rank, int64_t T_total, const float* gamma,
                                          const float* beta, float eps, int fuse_silu, void* y,
                                          float* fresh_sums_out, int64_t B, int64_t T_loc,
                                          int64_t C, int64_t G, dp_dtype dt, void* ws,
                                          size_t ws_size, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_groupnorm_stale_stats";
  if (!x || !y) return fail(DP_ERR_INVALID_ARG, "%s: NULL x or y", name);
  GnArgs ga{};
  dp_status st = check_common(name, x, B, T_loc, C, G, dt, ga);
  if (st != DP_OK) return st;
  if ((st = check_stats_args(name, stale_sums, n_patches, rank, T_total, T_loc, eps)) != DP_OK) return st;
  const size_t need = ws_bytes(B, T_loc, C, G);
  if (!ws || ws_size < need) return fail(DP_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", name, ws_size, need);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * dp::dtype_size(dt);
  if (dp::overlaps(x, xb, y, xb)) return fail(DP_ERR_INVALID_ARG, "%s: x and y overlap", name);
  if (!dp::aligned16(y)) return fail(DP_ERR_INVALID_ARG, "%s: y must be 16-byte aligned", name);
  set_stats(ga, stale_sums, n_patches, rank, T_total, gamma, beta, eps, fuse_silu);
  dp::clear_error();
  for (int64_t b0 = 0; b0 < B; b0 += kMaxChunk) {
    const int Bc = static_cast<int>(std::min<int64_t>(kMaxChunk, B - b0));
    launch_sums(ga, static_cast<int>(b0), Bc, ws, fresh_sums_out ? fresh_sums_out + b0 * G * 2 : nullptr, dt, stream);
    launch_apply(ga, static_cast<int>(b0), Bc,
                 reinterpret_cast<const float*>(static_cast<char*>(ws) + ws_layout(Bc, T_loc, C, G).sums_off), y, dt,
                 stream);
  }
  return dp::check_launch(name);
}

// ---------------------------------------------- no-allocation entry point
// dp_groupnorm_stale_stats_noalloc runs the kernels above with this file-scope
// device array as their workspace: every device holds its own copy, at its
// own address, until the process ends.  On the host the array's name denotes
// a host-side shadow, never the device memory, so host code only ever uses
// the address hipGetSymbolAddress returns, looked up once per device.  The
// ticket counters at its start are zeroed by a fill kernel on the first call
// for a device and are put back to zero by every call's last arrivals; the
// rest is rewritten before it is read by every call.
namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words(unsigned* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's copy of `scratch`; the first call for a device looks
// it up and enqueues the counter region's zero fill on `stream`.
dp_status device_scratch(const char* name, hipStream_t stream, void** out) {
  using dp::fail;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DP_ERR_HIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DP_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices supported", name, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DP_ERR_HIP, "%s: hipGetSymbolAddress: %s", name, hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words, dim3(8), dim3(256), 0, stream, static_cast<unsigned*>(p), kCounterBytes / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(DP_ERR_HIP, "%s: scratch zero fill: %s", name, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DP_OK;
}

}  // namespace

DP_API dp_status dp_groupnorm_stale_stats_noalloc(const void* x, const float* stale_sums, int64_t n_patches,
                                                  int64_t rank, int64_t T_total, const float* gamma,
                                                  const float* beta, float eps, int fuse_silu, void* y,
                                                  float* fresh_sums_out, int64_t B, int64_t T_loc, int64_t C,
                                                  int64_t G, dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_groupnorm_stale_stats_noalloc";
  if (!x || !y) return fail(DP_ERR_INVALID_ARG, "%s: NULL x or y", name);
  GnArgs ga{};
  dp_status st = check_common(name, x, B, T_loc, C, G, dt, ga);
  if (st != DP_OK) return st;
  if ((st = check_stats_args(name, stale_sums, n_patches, rank, T_total, T_loc, eps)) != DP_OK) return st;
  const size_t need = ws_bytes(B, T_loc, C, G);
  if (need > kScratchBytes)
    return fail(DP_ERR_UNSUPPORTED, "%s: the shape needs %zu bytes of scratch, the static scratch holds %zu", name,
                need, kScratchBytes);
  // every check of the workspace entry point is done here too, before the
  // first call's zero fill may be enqueued: a non-OK return enqueues nothing
  const size_t xb = static_cast<size_t>(B * T_loc * C) * dp::dtype_size(dt);
  if (dp::overlaps(x, xb, y, xb)) return fail(DP_ERR_INVALID_ARG, "%s: x and y overlap", name);
  if (!dp::aligned16(y)) return fail(DP_ERR_INVALID_ARG, "%s: y must be 16-byte aligned", name);
  void* ws = nullptr;
  if ((st = device_scratch(name, stream, &ws)) != DP_OK) return st;
  return dp_groupnorm_stale_stats(x, stale_sums, n_patches, rank, T_total, gamma, beta, eps, fuse_silu, y,
                                  fresh_sums_out, B, T_loc, C, G, dt, ws, kScratchBytes, stream);
}

DP_API dp_status dp_groupnorm_sums(const void* x, float* sums_out, int64_t B, int64_t T_loc, int64_t C, int64_t G,
                                   dp_dtype dt, void* ws, size_t ws_size, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_groupnorm_sums";
  if (!x || !sums_out) return fail(DP_ERR_INVALID_ARG, "%s: NULL x or sums_out", name);
  GnArgs ga{};
  dp_status st = check_common(name, x, B, T_loc, C, G, dt, ga);
  if (st != DP_OK) return st;
  const size_t need = ws_bytes(B, T_loc, C, G);
  if (!ws || ws_size < need) return fail(DP_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", name, ws_size, need);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * dp::dtype_size(dt);
  if (dp::overlaps(x, xb, sums_out, static_cast<size_t>(B * G) * 8) || dp::overlaps(ws, need, sums_out, static_cast<size_t>(B * G) * 8))
    return fail(DP_ERR_INVALID_ARG, "%s: sums_out overlaps x or the workspace", name);
  dp::clear_error();
  for (int64_t b0 = 0; b0 < B; b0 += kMaxChunk)
    launch_sums(ga, static_cast<int>(b0), static_cast<int>(std::min<int64_t>(kMaxChunk, B - b0)), ws,
                sums_out + b0 * G * 2, dt, stream);
  return dp::check_launch(name);
}

DP_API dp_status dp_groupnorm_apply(const void* x, const float* local_sums, const float* stale_sums,
                                    int64_t n_patches, int64_t rank, int64_t T_total, const float* gamma,
                                    const float* beta, float eps, int fuse_silu, void* y, int64_t B, int64_t T_loc,
                                    int64_t C, int64_t G, dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_groupnorm_apply";
  if (!x || !y || !local_sums) return fail(DP_ERR_INVALID_ARG, "%s: NULL x, y or local_sums", name);
  GnArgs ga{};
  dp_status st = check_common(name, x, B, T_loc, C, G, dt, ga);
  if (st != DP_OK) return st;
  if ((st = check_stats_args(name, stale_sums, n_patches, rank, T_total, T_loc, eps)) != DP_OK) return st;
  const size_t xb = static_cast<size_t>(B * T_loc * C) * dp::dtype_size(dt);
  if (dp::overlaps(x, xb, y, xb)) return fail(DP_ERR_INVALID_ARG, "%s: x and y overlap", name);
  if (!dp::aligned16(y)) return fail(DP_ERR_INVALID_ARG, "%s: y must be 16-byte aligned", name);
  set_stats(ga, stale_sums, n_patches, rank, T_total, gamma, beta, eps, fuse_silu);
  dp::clear_error();
  launch_apply(ga, 0, static_cast<int>(B), local_sums, y, dt, stream);
  return dp::check_launch(name);
}
