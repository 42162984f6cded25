// GroupNorm of the rank's tokens with whole-image statistics: fresh sums over
// the local tokens plus stale sums from the other patches.
//
// Method source: "OTIL for SDXL on 4x L40S", "What is implemented where" (two
// scalars per group, combined across slices, decide slice brightness and
// contrast) and the xDiT issue thread "Tensor Parallelism with Stale
// Activations ..." (a feature may combine fresh partial values with stale ones).
//
// Three HBM-streaming passes, all deterministic (fixed reduction order, no
// float atomics):
//   1. gn_partial:  per (batch, token tile) per-group (sum x, sum x^2)
//   2. gn_finalize: per batch, fold the tiles in order, write the fresh local
//                   sums, add the other patches' stale sums, derive mean/rstd
//   3. gn_apply:    y = x * a_c + b_c (a_c = rstd*gamma, b_c = beta - mean*a_c),
//                   optional SiLU, written in the storage type
// Every thread owns one 16-byte channel vector of a token, so loads and stores
// are 16 B wide and consecutive threads touch consecutive bytes.
#include "dp_internal.h"

namespace {

constexpr int kMaxThreads = 256;

struct GnPlan {
  int vec;          // channels per 16-byte vector
  int vpt;          // vectors per token
  int tpp;          // tokens per pass of one block
  int threads;      // tpp * vpt
  int tile_tokens;  // tokens per block
  int tiles;        // blocks per batch item
};

// Tiling depends on (B, T, C) only, so the workspace size does not depend on
// the dtype.
void tiles_for(int64_t B, int64_t T, int& tile_tokens, int& tiles) {
  int64_t tt = (T * B + 1023) / 1024;
  if (tt < 16) tt = 16;
  if (tt > T) tt = T;
  tile_tokens = static_cast<int>(tt);
  tiles = static_cast<int>((T + tt - 1) / tt);
}

GnPlan make_plan(int64_t B, int64_t T, int64_t C, dp_dtype dt) {
  GnPlan p;
  p.vec = dt == DP_BF16 ? 8 : 4;
  p.vpt = static_cast<int>(C / p.vec);
  p.tpp = kMaxThreads / p.vpt;
  p.threads = p.tpp * p.vpt;
  tiles_for(B, T, p.tile_tokens, p.tiles);
  return p;
}

template <bool BF16>
__device__ __forceinline__ void load_vec(const void* base, int64_t elem, float* v) {
  if constexpr (BF16) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(u[j]);
      v[2 * j + 1] = bf16_hi(u[j]);
    }
  } else {
    const f32x4 u = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = u[j];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_vec(void* base, int64_t elem, const float* v) {
  if constexpr (BF16) {
    u32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(base) + elem) = u;
  } else {
    f32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = v[j];
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + elem) = u;
  }
}

// partial[(b*tiles + tile)*G + g][2] = (sum x, sum x^2) over the tile's tokens.
template <bool BF16>
__global__ void __launch_bounds__(kMaxThreads)
gn_partial(const void* __restrict__ x, float* __restrict__ partial, int T, int C, int G,
           int tile_tokens, int tiles) {
  constexpr int VEC = BF16 ? 8 : 4;
  extern __shared__ float lds[];  // [2][tpp][C], then [2][C]
  const int vpt = C / VEC;
  const int tpp = blockDim.x / vpt;
  const int tl = threadIdx.x / vpt, vi = threadIdx.x % vpt;
  const int b = blockIdx.y, tile = blockIdx.x;
  const int t_begin = tile * tile_tokens;
  const int t_end = min(T, t_begin + tile_tokens);

  float s1[VEC], s2[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) s1[j] = s2[j] = 0.f;
  const int64_t row0 = static_cast<int64_t>(b) * T;
  for (int t = t_begin + tl; t < t_end; t += tpp) {
    float v[VEC];
    load_vec<BF16>(x, (row0 + t) * C + vi * VEC, v);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      s1[j] += v[j];
      s2[j] = fmaf(v[j], v[j], s2[j]);
    }
  }
  float* r1 = lds;
  float* r2 = lds + tpp * C;
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    r1[tl * C + vi * VEC + j] = s1[j];
    r2[tl * C + vi * VEC + j] = s2[j];
  }
  __syncthreads();
  float* c1 = lds + 2 * tpp * C;
  float* c2 = c1 + C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float a = 0.f, q = 0.f;
    for (int k = 0; k < tpp; ++k) {
      a += r1[k * C + c];
      q += r2[k * C + c];
    }
    c1[c] = a;
    c2[c] = q;
  }
  __syncthreads();
  const int Cg = C / G;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    float a = 0.f, q = 0.f;
    for (int c = g * Cg; c < (g + 1) * Cg; ++c) {
      a += c1[c];
      q += c2[c];
    }
    float* out = partial + ((static_cast<int64_t>(b) * tiles + tile) * G + g) * 2;
    out[0] = a;
    out[1] = q;
  }
}

// One block per batch item.  stats[b][g] = (mean, rstd); fresh[b][g] = local sums.
__global__ void __launch_bounds__(kMaxThreads)
gn_finalize(const float* __restrict__ partial, const float* __restrict__ stale, int n_patches,
            int rank, int B, int G, int tiles, float inv_count, float eps,
            float* __restrict__ stats, float* __restrict__ fresh) {
  __shared__ float red[2][kMaxThreads];
  const int b = blockIdx.x;
  // Threads sharing g = tid % G each fold a strided subset of the tiles.
  const int lanes_per_g = G <= kMaxThreads ? kMaxThreads / G : 1;
  for (int g0 = 0; g0 < G; g0 += kMaxThreads) {
    const int span = min(G - g0, kMaxThreads);
    const int per = G <= kMaxThreads ? lanes_per_g : 1;
    const int gi = threadIdx.x % span;
    const int part = threadIdx.x / span;
    float a = 0.f, q = 0.f;
    if (part < per) {
      for (int t = part; t < tiles; t += per) {
        const float* p = partial + ((static_cast<int64_t>(b) * tiles + t) * G + g0 + gi) * 2;
        a += p[0];
        q += p[1];
      }
    }
    red[0][threadIdx.x] = a;
    red[1][threadIdx.x] = q;
    __syncthreads();
    if (threadIdx.x < span) {
      float s1 = 0.f, s2 = 0.f;
      for (int k = 0; k < per; ++k) {
        s1 += red[0][k * span + threadIdx.x];
        s2 += red[1][k * span + threadIdx.x];
      }
      const int g = g0 + threadIdx.x;
      if (fresh) {
        fresh[(b * G + g) * 2 + 0] = s1;
        fresh[(b * G + g) * 2 + 1] = s2;
      }
      for (int p = 0; p < n_patches; ++p) {
        if (p == rank) continue;
        s1 += stale[((static_cast<int64_t>(p) * B + b) * G + g) * 2 + 0];
        s2 += stale[((static_cast<int64_t>(p) * B + b) * G + g) * 2 + 1];
      }
      const float mean = s1 * inv_count;
      const float var = fmaxf(s2 * inv_count - mean * mean, 0.f);
      stats[(b * G + g) * 2 + 0] = mean;
      stats[(b * G + g) * 2 + 1] = 1.0f / sqrtf(var + eps);
    }
    __syncthreads();
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kMaxThreads)
gn_apply(const void* __restrict__ x, void* __restrict__ y, const float* __restrict__ stats,
         const float* __restrict__ gamma, const float* __restrict__ beta, int T, int C, int G,
         int tile_tokens, int silu) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int vpt = C / VEC;
  const int tpp = blockDim.x / vpt;
  const int tl = threadIdx.x / vpt, vi = threadIdx.x % vpt;
  const int b = blockIdx.y;
  const int t_begin = blockIdx.x * tile_tokens;
  const int t_end = min(T, t_begin + tile_tokens);
  const int Cg = C / G;
  float a[VEC], sh[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int c = vi * VEC + j;
    const int g = c / Cg;
    const float mean = stats[(b * G + g) * 2 + 0];
    const float rstd = stats[(b * G + g) * 2 + 1];
    const float gm = gamma ? gamma[c] : 1.f;
    const float bt = beta ? beta[c] : 0.f;
    a[j] = rstd * gm;
    sh[j] = bt - mean * a[j];
  }
  const int64_t row0 = static_cast<int64_t>(b) * T;
  for (int t = t_begin + tl; t < t_end; t += tpp) {
    const int64_t e = (row0 + t) * C + vi * VEC;
    float v[VEC];
    load_vec<BF16>(x, e, v);
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      float o = fmaf(v[j], a[j], sh[j]);
      if (silu) o = o / (1.0f + __expf(-o));
      v[j] = o;
    }
    store_vec<BF16>(y, e, v);
  }
}

size_t workspace_bytes(int64_t B, int64_t T, int64_t G) {
  int tt, tiles;
  tiles_for(B, T, tt, tiles);
  return static_cast<size_t>(B) * (static_cast<size_t>(tiles) + 1) * static_cast<size_t>(G) * 2 *
         sizeof(float);
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
  if (C % vec != 0 || C / vec > kMaxThreads || T_loc > 0x7FFFFFFF || B > 65535 || G > 65535 ||
      B * G > 0x7FFFFFFF)
    return fail(DP_ERR_UNSUPPORTED, "dp_groupnorm_stale_stats: C=%lld G=%lld not supported",
                (long long)C, (long long)G);
  const size_t es = dp::dtype_size(dt);
  const size_t xb = static_cast<size_t>(B * T_loc * C) * es;
  if (dp::overlaps(x, xb, y, xb)) return fail(DP_ERR_INVALID_ARG, "dp_groupnorm_stale_stats: x and y overlap");

  const GnPlan p = make_plan(B, T_loc, C, dt);
  float* partial = static_cast<float*>(ws);
  float* stats = partial + static_cast<size_t>(B) * p.tiles * G * 2;
  const float inv_count = static_cast<float>(1.0 / (static_cast<double>(T_total) * (C / G)));
  const size_t lds1 = (2 * static_cast<size_t>(p.tpp) * C + 2 * C) * sizeof(float);
  dp::clear_error();
  const dim3 grid(p.tiles, static_cast<unsigned>(B));
  if (dt == DP_BF16)
    hipLaunchKernelGGL(gn_partial<true>, grid, dim3(p.threads), lds1, stream, x, partial,
                       (int)T_loc, (int)C, (int)G, p.tile_tokens, p.tiles);
  else
    hipLaunchKernelGGL(gn_partial<false>, grid, dim3(p.threads), lds1, stream, x, partial,
                       (int)T_loc, (int)C, (int)G, p.tile_tokens, p.tiles);
  hipLaunchKernelGGL(gn_finalize, dim3(static_cast<unsigned>(B)), dim3(kMaxThreads), 0, stream,
                     partial, stale_sums, (int)n_patches, (int)rank, (int)B, (int)G, p.tiles,
                     inv_count, eps, stats, fresh_sums_out);
  if (dt == DP_BF16)
    hipLaunchKernelGGL(gn_apply<true>, grid, dim3(p.threads), 0, stream, x, y, stats, gamma, beta,
                       (int)T_loc, (int)C, (int)G, p.tile_tokens, fuse_silu);
  else
    hipLaunchKernelGGL(gn_apply<false>, grid, dim3(p.threads), 0, stream, x, y, stats, gamma, beta,
                       (int)T_loc, (int)C, (int)G, p.tile_tokens, fuse_silu);
  return dp::check_launch("dp_groupnorm_stale_stats");
}
