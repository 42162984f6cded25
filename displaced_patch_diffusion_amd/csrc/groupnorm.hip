// GroupNorm of the rank's tokens with whole-image statistics: fresh sums over
// the local tokens plus stale sums from the other patches.
//
// Method source: "OTIL for SDXL on 4x L40S", "What is implemented where" (two
// scalars per group, combined across slices, decide slice brightness and
// contrast) and the xDiT issue thread "Tensor Parallelism with Stale
// Activations ..." (a feature may combine fresh partial values with stale ones).
//
// Two launches over the same (token tile, batch item) grid, deterministic
// (fixed reduction order, no float atomics, no inter-block waiting):
//   1. gn_partial: per tile, per group (sum x, sum x^2) -> workspace
//   2. gn_apply:   every block folds the partials of its batch item in one
//                  fixed order (so all blocks derive bit-identical statistics),
//                  adds the other patches' stale sums and writes
//                  y = x * a_c + b_c (a_c = rstd*gamma_c, b_c = beta_c - mean*a_c,
//                  optional SiLU) for its tile; the block of tile 0 also writes
//                  the fresh local sums.
// Both launches use the same block -> tile mapping, so the tile block i
// re-reads in pass 2 was read by block i, on the same XCD, in pass 1.
//
// A single pass that keeps each tile in registers while the blocks exchange
// partials through device-scope atomics was measured slower on MI355X than
// these two launches: the cross-XCD exchange (coherent stores, arrival
// counter, uncached reads of every partial by every block) costs more than
// re-reading x from the cache hierarchy.
//
// Every thread owns one 16-byte channel vector of a token, so loads and stores
// are 16 B wide and consecutive threads touch consecutive bytes.
#include <algorithm>

#include "dp_internal.h"

namespace {

constexpr int kThreads = 512;
constexpr int kTargetBlocks = 512;  // about two blocks per CU
constexpr int kUnroll = 8;          // 16-byte loads in flight per thread

struct GnArgs {
  const void* x;
  void* y;
  float2* partial;     // [B][tiles][G]
  const float* stale;  // [n_patches][B][G][2]
  const float* gamma;
  const float* beta;
  float* fresh;        // [B][G][2] or NULL
  const float* given;  // [B][G][2] local sums computed elsewhere, or NULL (fold the partials)
  int T, C, G, tiles, tile_tokens, n_patches, rank, B, silu;
  float inv_count, eps;
};

// Upper bound of tiles per batch item, independent of C, dtype and device (it
// sizes the workspace).
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

// The 16-byte vector vi of token t, or zeros when `on` is false or t >= t_end.
template <bool BF16>
__device__ __forceinline__ u32x4 load_or_zero(const GnArgs& a, int b, int t, int t_end, int vi, bool on) {
  u32x4 u = u32x4{0u, 0u, 0u, 0u};
  if (on && t < t_end)
    u = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + vec_byte<BF16>(b, t, vi, a));
  return u;
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

// Block-wide per-group sums of the per-thread channel sums s1/s2, in a fixed
// order: token lanes in order per channel, then channels in order per group.
// lds_r holds [2][tpp*C] floats, lds_c [2][C]; the result lands in gsum[G].
// Starts and ends with a barrier, so it may be called back to back.
template <int VEC>
__device__ void block_group_sums(const float* s1, const float* s2, bool active, int tl, int vi,
                                 int tpp, int C, int G, float* lds_r, float* lds_c, float2* gsum) {
  __syncthreads();
  if (active) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      lds_r[tl * C + vi * VEC + j] = s1[j];
      lds_r[tpp * C + tl * C + vi * VEC + j] = s2[j];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += kThreads) {
    float p1 = 0.f, p2 = 0.f;
    for (int k = 0; k < tpp; ++k) {
      p1 += lds_r[k * C + c];
      p2 += lds_r[tpp * C + k * C + c];
    }
    lds_c[c] = p1;
    lds_c[C + c] = p2;
  }
  __syncthreads();
  const int Cg = C / G;
  for (int g = threadIdx.x; g < G; g += kThreads) {
    float p1 = 0.f, p2 = 0.f;
    for (int c = g * Cg; c < (g + 1) * Cg; ++c) {
      p1 += lds_c[c];
      p2 += lds_c[C + c];
    }
    gsum[g] = make_float2(p1, p2);
  }
  __syncthreads();
}

// Folds the tile partials of batch item b into lane sums red[q*G + g] (lane q
// takes tiles q, q + lanes, ..., U per pass in U accumulators); returns the
// lane count.  A pass issues all U loads before it adds any of them (indexes
// past the last tile re-read that tile and are not added), so one memory
// round trip covers up to U * lanes tiles.  One fixed order, so every block
// (and dp_groupnorm_sums) derives bit-identical sums.
__device__ int fold_partials(const GnArgs& a, int b, float2* red) {
  const int G = a.G;
  const int lanes = G >= kThreads ? 1 : kThreads / G;
  const float2* pb = a.partial + static_cast<int64_t>(b) * a.tiles * G;
  constexpr int U = 16;
  for (int f = threadIdx.x; f < lanes * G; f += kThreads) {
    const int g = f % G, q = f / G;
    float2 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = make_float2(0.f, 0.f);
    for (int t0 = q; t0 < a.tiles; t0 += U * lanes) {
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = pb[static_cast<int64_t>(min(t0 + u * lanes, a.tiles - 1)) * G + g];
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
  return lanes;
}

// The first kStalePre patches' stale sums of group g of batch item b, loaded
// ahead of the fold so that their latency overlaps it (the thread of group g
// finalises that group).
constexpr int kStalePre = 8;
struct StalePre {
  float2 v[kStalePre];
};

__device__ __forceinline__ StalePre prefetch_stale(const GnArgs& a, int b, int g) {
  StalePre sp;
#pragma unroll
  for (int j = 0; j < kStalePre; ++j) sp.v[j] = make_float2(0.f, 0.f);
  if (g < a.G && a.n_patches > 1) {
#pragma unroll
    for (int j = 0; j < kStalePre; ++j) {
      const float* st = a.stale + ((static_cast<int64_t>(min(j, a.n_patches - 1)) * a.B + b) * a.G + g) * 2;
      sp.v[j] = make_float2(st[0], st[1]);
    }
  }
  return sp;
}

// Statistics of batch item b from the lane sums red[q*G + g] (lanes in
// order): fresh local sums out (tile 0 only), stale sums of the other
// patches added in patch order (the first kStalePre from `pre`, prefetched by
// the thread of group g = threadIdx.x), (mean, rstd) per group into gstat.
__device__ void finalize_stats(const GnArgs& a, int b, int tile, int lanes, const float2* red,
                               const StalePre& pre, float2* gstat) {
  const int G = a.G;
  for (int g = threadIdx.x; g < G; g += kThreads) {
    float f1 = 0.f, f2 = 0.f;
    for (int q = 0; q < lanes; ++q) {
      f1 += red[q * G + g].x;
      f2 += red[q * G + g].y;
    }
    if (tile == 0 && a.fresh) {
      a.fresh[(static_cast<int64_t>(b) * G + g) * 2 + 0] = f1;
      a.fresh[(static_cast<int64_t>(b) * G + g) * 2 + 1] = f2;
    }
    if (g == static_cast<int>(threadIdx.x)) {
#pragma unroll
      for (int j = 0; j < kStalePre; ++j) {
        if (j < a.n_patches && j != a.rank) {
          f1 += pre.v[j].x;
          f2 += pre.v[j].y;
        }
      }
    }
    for (int p = g == static_cast<int>(threadIdx.x) ? kStalePre : 0; p < a.n_patches; ++p) {
      if (p == a.rank) continue;
      const float* st = a.stale + ((static_cast<int64_t>(p) * a.B + b) * G + g) * 2;
      f1 += st[0];
      f2 += st[1];
    }
    const float mean = f1 * a.inv_count;
    const float var = fmaxf(f2 * a.inv_count - mean * mean, 0.f);
    gstat[g] = make_float2(mean, 1.0f / sqrtf(var + a.eps));
  }
}

template <int VEC>
__device__ __forceinline__ void channel_coeffs(const float2* gstat, int vi, int Cg, const float* gm,
                                               const float* bt, float* ca, float* cb) {
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const float2 ms = gstat[(vi * VEC + j) / Cg];
    ca[j] = ms.y * gm[j];
    cb[j] = bt[j] - ms.x * ca[j];
  }
}

template <bool BF16>
__device__ __forceinline__ void normalize_store(const GnArgs& a, int b, int t, int vi, const u32x4& u,
                                                const float* ca, const float* cb) {
  constexpr int VEC = BF16 ? 8 : 4;
  float v[VEC];
  unpack_vec<BF16>(u, v);
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    float z = fmaf(v[j], ca[j], cb[j]);
    if (a.silu) z *= __builtin_amdgcn_rcpf(1.0f + __expf(-z));  // v_rcp_f32, 1 ulp
    v[j] = z;
  }
  __builtin_nontemporal_store(
      pack_vec<BF16>(v), reinterpret_cast<u32x4*>(static_cast<char*>(a.y) + vec_byte<BF16>(b, t, vi, a)));
}

// ------------------------------------------------------------ kernels
template <bool BF16>
__global__ void __launch_bounds__(kThreads) gn_partial(GnArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;
  __shared__ float lds_r[2 * kThreads * VEC];
  __shared__ float lds_c[2 * 2048];
  __shared__ float2 gsum[2048];
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
  for (int k0 = 0; k0 < npass; k0 += kUnroll) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      raw[u] = load_or_zero<BF16>(a, b, t_begin + tl + (k0 + u) * tpp, t_end, vi,
                                  active && k0 + u < npass);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (k0 + u < npass) acc_vec<BF16>(raw[u], s1, s2);
  }
  block_group_sums<VEC>(s1, s2, active, tl, vi, tpp, a.C, a.G, lds_r, lds_c, gsum);
  for (int g = tid; g < a.G; g += kThreads)
    a.partial[(static_cast<int64_t>(b) * a.tiles + tile) * a.G + g] = gsum[g];
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) gn_apply(GnArgs a) {
  constexpr int VEC = BF16 ? 8 : 4;
  __shared__ float2 red[2048];    // [lanes][G], lanes * G <= max(G, kThreads)
  __shared__ float2 gstat[2048];  // (mean, rstd) per group
  const int G = a.G;
  const int vpt = a.C / VEC, tpp = kThreads / vpt;
  const int tid = threadIdx.x, tl = tid / vpt, vi = tid % vpt;
  const bool active = tl < tpp;
  const int b = blockIdx.y, tile = blockIdx.x;
  const int t_begin = tile * a.tile_tokens;
  const int t_end = min(a.T, t_begin + a.tile_tokens);
  const int npass = a.tile_tokens / tpp;

  // gamma/beta and the first loads of the tile go out before the fold, which
  // then runs under their latency
  float gm[VEC], bt[VEC];
  if (active) load_affine<VEC>(a, vi, gm, bt);
  u32x4 first[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    first[u] = load_or_zero<BF16>(a, b, t_begin + tl + u * tpp, t_end, vi, active && u < npass);

  const StalePre pre = prefetch_stale(a, b, tid);
  int lanes = 1;
  if (a.given) {  // the local sums come from the caller: one lane holding them
    for (int g = tid; g < G; g += kThreads)
      red[g] = make_float2(a.given[(static_cast<int64_t>(b) * G + g) * 2], a.given[(static_cast<int64_t>(b) * G + g) * 2 + 1]);
  } else {
    lanes = fold_partials(a, b, red);
  }
  __syncthreads();
  finalize_stats(a, b, tile, lanes, red, pre, gstat);
  __syncthreads();

  if (!active) return;
  float ca[VEC], cb[VEC];
  channel_coeffs<VEC>(gstat, vi, a.C / G, gm, bt, ca, cb);
  if (npass <= kUnroll) {  // one group of passes: its loads went out before the fold
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t_begin + tl + u * tpp;
      if (u < npass && t < t_end) normalize_store<BF16>(a, b, t, vi, first[u], ca, cb);
    }
    return;
  }
  // double-buffered: the loads of the next kUnroll passes go out before this
  // group's normalise-and-store, so reads and writes stay in flight together
  u32x4 cur[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) cur[u] = first[u];
  for (int k0 = 0; k0 < npass; k0 += kUnroll) {
    u32x4 nxt[kUnroll];
    const bool more = k0 + kUnroll < npass;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      nxt[u] = load_or_zero<BF16>(a, b, t_begin + tl + (k0 + kUnroll + u) * tpp, t_end, vi,
                                  more && k0 + kUnroll + u < npass);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t_begin + tl + (k0 + u) * tpp;
      if (k0 + u < npass && t < t_end) normalize_store<BF16>(a, b, t, vi, cur[u], ca, cb);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
  }
}

// Local sums only: one block per batch item folds the partials (in the order
// gn_apply uses) and writes (sum x, sum x^2) per group.
__global__ void __launch_bounds__(kThreads) gn_sums(GnArgs a) {
  __shared__ float2 red[2048];
  const int b = blockIdx.y, G = a.G;
  const int lanes = fold_partials(a, b, red);
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kThreads) {
    float f1 = 0.f, f2 = 0.f;
    for (int q = 0; q < lanes; ++q) {
      f1 += red[q * G + g].x;
      f2 += red[q * G + g].y;
    }
    a.fresh[(static_cast<int64_t>(b) * G + g) * 2 + 0] = f1;
    a.fresh[(static_cast<int64_t>(b) * G + g) * 2 + 1] = f2;
  }
}

// ------------------------------------------------------------ planning
struct GnPlan {
  int tile_tokens, tiles;
};

// Tokens per tile: a whole number of block passes (tpp tokens each); at most
// max_tiles(B, T) tiles per batch item.
GnPlan make_plan(int64_t B, int64_t T, int64_t C, dp_dtype dt) {
  const int vec = dt == DP_BF16 ? 8 : 4;
  const int tpp = kThreads / static_cast<int>(C / vec);
  const int64_t per_b = max_tiles(B, T);
  int64_t tt = (T + per_b - 1) / per_b;
  tt = (tt + tpp - 1) / tpp * tpp;
  return GnPlan{static_cast<int>(tt), static_cast<int>((T + tt - 1) / tt)};
}

// Workspace: the per-tile partials [B][max_tiles][G] of float2.
size_t workspace_bytes(int64_t B, int64_t T, int64_t G) {
  return static_cast<size_t>(B) * static_cast<size_t>(max_tiles(B, T)) * static_cast<size_t>(G) *
         sizeof(float2);
}

}  // namespace

DP_API size_t dp_groupnorm_stale_stats_workspace(int64_t B, int64_t T_loc, int64_t C, int64_t G) {
  (void)C;
  if (B <= 0 || T_loc <= 0 || G <= 0) return 0;
  return workspace_bytes(B, T_loc, G);
}

DP_API dp_status dp_groupnorm_stale_stats(const void* x, const float* stale_sums, int64_t n_patches,
                                          int64_t rank, int64_t T_total, const float* gamma,
                                          const float* beta, float eps, int fuse_silu, void* y,
                                          float* fresh_sums_out, int64_t B, int64_t T_loc,
                                          int64_t C, int64_t G, dp_dtype dt, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  using dp::fail;
  if (!x || !y) return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: NULL x or y");
  if (B <= 0 || T_loc <= 0 || C <= 0 || G <= 0 || n_patches <= 0)
    return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: sizes must be positive");
  if (!stale_sums && n_patches > 1)
    return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: NULL stale_sums with %lld patches",
                (long long)n_patches);
  if (rank < 0 || rank >= n_patches)
    return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: rank %lld outside [0, %lld)",
                (long long)rank, (long long)n_patches);
  if (T_total < T_loc)
    return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: T_total < T_loc");
  if (!(eps >= 0.f)) return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: eps must be >= 0");
  if (C % G != 0) return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: C %% G != 0");
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: bad dtype");
  const size_t need = workspace_bytes(B, T_loc, G);
  if (!ws || ws_bytes < need)
    return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: workspace %zu < %zu bytes",
                ws_bytes, need);
  const int vec = dt == DP_BF16 ? 8 : 4;
  if (C % vec != 0 || C > 2048 || C / vec > kThreads || T_loc > 0x7FFFFFFF || B > 65535 ||
      B * G > 0x7FFFFFFF)
    return fail(DP_ERR_UNSUPPORTED, "dp_groupnorm_stale_stats: C=%lld G=%lld not supported",
                (long long)C, (long long)G);
  const size_t es = dp::dtype_size(dt);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * es;
  if (dp::overlaps(x, xb, y, xb)) return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: x and y overlap");

  const GnPlan p = make_plan(B, T_loc, C, dt);
  GnArgs ga{};
  ga.x = x;
  ga.y = y;
  ga.partial = static_cast<float2*>(ws);
  ga.stale = stale_sums;
  ga.gamma = gamma;
  ga.beta = beta;
  ga.fresh = fresh_sums_out;
  ga.T = static_cast<int>(T_loc);
  ga.C = static_cast<int>(C);
  ga.G = static_cast<int>(G);
  ga.tiles = p.tiles;
  ga.tile_tokens = p.tile_tokens;
  ga.n_patches = static_cast<int>(n_patches);
  ga.rank = static_cast<int>(rank);
  ga.B = static_cast<int>(B);
  ga.silu = fuse_silu;
  ga.inv_count = static_cast<float>(1.0 / (static_cast<double>(T_total) * (C / G)));
  ga.eps = eps;
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(B));
  dp::clear_error();
  if (dt == DP_BF16) {
    hipLaunchKernelGGL(gn_partial<true>, grid, dim3(kThreads), 0, stream, ga);
    hipLaunchKernelGGL(gn_apply<true>, grid, dim3(kThreads), 0, stream, ga);
  } else {
    hipLaunchKernelGGL(gn_partial<false>, grid, dim3(kThreads), 0, stream, ga);
    hipLaunchKernelGGL(gn_apply<false>, grid, dim3(kThreads), 0, stream, ga);
  }
  return dp::check_launch("dp_groupnorm_stale_stats");
}

DP_API dp_status dp_groupnorm_sums(const void* x, float* sums_out, int64_t B, int64_t T_loc, int64_t C, int64_t G,
                                   dp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_groupnorm_sums";
  if (!x || !sums_out) return fail(DP_ERR_INVALID_ARG, "%s: NULL x or sums_out", name);
  if (B <= 0 || T_loc <= 0 || C <= 0 || G <= 0) return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (C % G != 0) return fail(DP_ERR_INVALID_ARG, "%s: C %% G != 0", name);
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  const size_t need = workspace_bytes(B, T_loc, G);
  if (!ws || ws_bytes < need) return fail(DP_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  const int vec = dt == DP_BF16 ? 8 : 4;
  if (C % vec != 0 || C > 2048 || C / vec > kThreads || T_loc > 0x7FFFFFFF || B > 65535 || B * G > 0x7FFFFFFF)
    return fail(DP_ERR_UNSUPPORTED, "%s: C=%lld G=%lld not supported", name, (long long)C, (long long)G);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * dp::dtype_size(dt);
  if (dp::overlaps(x, xb, sums_out, static_cast<size_t>(B * G) * 8) || dp::overlaps(ws, need, sums_out, static_cast<size_t>(B * G) * 8))
    return fail(DP_ERR_INVALID_ARG, "%s: sums_out overlaps x or the workspace", name);
  const GnPlan p = make_plan(B, T_loc, C, dt);
  GnArgs ga{};
  ga.x = x;
  ga.partial = static_cast<float2*>(ws);
  ga.fresh = sums_out;
  ga.T = static_cast<int>(T_loc);
  ga.C = static_cast<int>(C);
  ga.G = static_cast<int>(G);
  ga.tiles = p.tiles;
  ga.tile_tokens = p.tile_tokens;
  ga.n_patches = 1;
  ga.B = static_cast<int>(B);
  dp::clear_error();
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(B));
  if (dt == DP_BF16) hipLaunchKernelGGL(gn_partial<true>, grid, dim3(kThreads), 0, stream, ga);
  else hipLaunchKernelGGL(gn_partial<false>, grid, dim3(kThreads), 0, stream, ga);
  hipLaunchKernelGGL(gn_sums, dim3(1, static_cast<unsigned>(B)), dim3(kThreads), 0, stream, ga);
  return dp::check_launch(name);
}

DP_API dp_status dp_groupnorm_apply(const void* x, const float* local_sums, const float* stale_sums,
                                    int64_t n_patches, int64_t rank, int64_t T_total, const float* gamma,
                                    const float* beta, float eps, int fuse_silu, void* y, int64_t B, int64_t T_loc,
                                    int64_t C, int64_t G, dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_groupnorm_apply";
  if (!x || !y || !local_sums) return fail(DP_ERR_INVALID_ARG, "%s: NULL x, y or local_sums", name);
  if (B <= 0 || T_loc <= 0 || C <= 0 || G <= 0 || n_patches <= 0) return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (!stale_sums && n_patches > 1) return fail(DP_ERR_INVALID_ARG, "%s: NULL stale_sums with %lld patches", name, (long long)n_patches);
  if (rank < 0 || rank >= n_patches) return fail(DP_ERR_INVALID_ARG, "%s: rank outside [0, n_patches)", name);
  if (T_total < T_loc) return fail(DP_ERR_INVALID_ARG, "%s: T_total < T_loc", name);
  if (!(eps >= 0.f)) return fail(DP_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
  if (C % G != 0) return fail(DP_ERR_INVALID_ARG, "%s: C %% G != 0", name);
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  const int vec = dt == DP_BF16 ? 8 : 4;
  if (C % vec != 0 || C > 2048 || C / vec > kThreads || T_loc > 0x7FFFFFFF || B > 65535 || B * G > 0x7FFFFFFF)
    return fail(DP_ERR_UNSUPPORTED, "%s: C=%lld G=%lld not supported", name, (long long)C, (long long)G);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * dp::dtype_size(dt);
  if (dp::overlaps(x, xb, y, xb)) return fail(DP_ERR_INVALID_ARG, "%s: x and y overlap", name);
  const GnPlan p = make_plan(B, T_loc, C, dt);
  GnArgs ga{};
  ga.x = x;
  ga.y = y;
  ga.given = local_sums;
  ga.stale = stale_sums;
  ga.gamma = gamma;
  ga.beta = beta;
  ga.T = static_cast<int>(T_loc);
  ga.C = static_cast<int>(C);
  ga.G = static_cast<int>(G);
  ga.tiles = p.tiles;
  ga.tile_tokens = p.tile_tokens;
  ga.n_patches = static_cast<int>(n_patches);
  ga.rank = static_cast<int>(rank);
  ga.B = static_cast<int>(B);
  ga.silu = fuse_silu;
  ga.inv_count = static_cast<float>(1.0 / (static_cast<double>(T_total) * (C / G)));
  ga.eps = eps;
  dp::clear_error();
  const dim3 grid(static_cast<unsigned>(p.tiles), static_cast<unsigned>(B));
  if (dt == DP_BF16) hipLaunchKernelGGL(gn_apply<true>, grid, dim3(kThreads), 0, stream, ga);
  else hipLaunchKernelGGL(gn_apply<false>, grid, dim3(kThreads), 0, stream, ga);
  return dp::check_launch(name);
}
