// OTIL selective block transmit ("OTIL for SDXL on 4x L40S", "What is
// implemented where": one topk over the dissimilarity plus ten times an
// unvisited flag, packing by index select, reconstruction by one index copy per
// remote device, zero host synchronisations per step; "Self-tests": never a
// blend, exactly k blocks per peer).
//
// A rank's band of the latent is token-major [B, h, W, C]; sub-block j is the
// bh x bw spatial block (row-major over the block grid) with all batch items
// and channels.  Sender side, on one stream and with no host sync; bands of at
// most 128K elements (and 4096 blocks) run the three phases in one workgroup
// (otil_fused), larger ones as three kernels:
//   otil_score   one wave per block: 1 - cos(x_j, last_sent_j) (+ bonus if
//                unvisited), fp32 dot products and norms;
//   otil_select  one 1024-thread block ranks every score against all others
//                (descending, ties to the lower id) from LDS; rank < k lands
//                in idx[rank];
//   otil_pack    one block per selected block: copies it into the send buffer
//                and into last_sent, and marks it visited.
// Receiver side, otil_unpack copies each received block into the peer's band.
#include <cmath>
#include <initializer_list>

#include "dp_internal.h"

namespace {

constexpr int kScoreThreads = 256;  // 4 waves, one block each
constexpr int kSelectThreads = 1024;
constexpr int kMaxBlocks = 16384;   // scores staged in 64 KB of LDS
constexpr int kCopyThreads = 256;

template <int DT>
__device__ __forceinline__ float load_as_float(const void* p, int64_t i) {
  if constexpr (DT == DP_F32) {
    return static_cast<const float*>(p)[i];
  } else if constexpr (DT == DP_BF16) {
    return __uint_as_float(static_cast<unsigned int>(static_cast<const unsigned short*>(p)[i]) << 16);
  } else {
    return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  }
}

struct BandGeom {
  int B, h, W, C, bh, bw, nbx, K;
};

// Element offset of element e (in [0, B*bh*bw*C)) of block j; the elements of
// a block are ordered [b][row][col][channel], the order of the packed layout.
__device__ __forceinline__ int64_t block_elem(const BandGeom& g, int j, int e) {
  const int run = g.bw * g.C;
  const int b = e / (g.bh * run);
  const int rem = e - b * g.bh * run;
  const int r = rem / run, c = rem - r * run;
  const int by = j / g.nbx, bx = j - by * g.nbx;
  return ((static_cast<int64_t>(b) * g.h + by * g.bh + r) * g.W + bx * g.bw) * g.C + c;
}

template <int DT>
__global__ void __launch_bounds__(kScoreThreads)
otil_score(const void* __restrict__ x, const void* __restrict__ ref, const unsigned char* __restrict__ visited,
           float* __restrict__ scores, BandGeom g, int K, float bonus) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kScoreThreads / 64) + (threadIdx.x >> 6);
  if (j >= K) return;
  const int n = g.B * g.bh * g.bw * g.C;
  float dot = 0.f, na = 0.f, nb = 0.f;
  for (int e = lane; e < n; e += 64) {
    const int64_t o = block_elem(g, j, e);
    const float a = load_as_float<DT>(x, o), b = load_as_float<DT>(ref, o);
    dot = fmaf(a, b, dot);
    na = fmaf(a, a, na);
    nb = fmaf(b, b, nb);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    dot += __shfl_xor(dot, off, 64);
    na += __shfl_xor(na, off, 64);
    nb += __shfl_xor(nb, off, 64);
  }
  if (lane == 0) {
    const float cosv = dot / fmaxf(sqrtf(na) * sqrtf(nb), 1e-8f);
    scores[j] = (1.f - cosv) + (visited[j] ? 0.f : bonus);
  }
}

// idx[rank(i)] = i for the k highest-ranked blocks; rank = number of blocks
// ordered before i (higher score, or equal score and lower id).
__global__ void __launch_bounds__(kSelectThreads)
otil_select(const float* __restrict__ scores, int K, int k, int* __restrict__ idx) {
  __shared__ float s[kMaxBlocks];
  for (int i = threadIdx.x; i < K; i += kSelectThreads) {
    const float v = scores[i];
    s[i] = v != v ? -INFINITY : v;  // a NaN ranks last, so the ranks stay a permutation
  }
  __syncthreads();
  for (int i = threadIdx.x; i < K; i += kSelectThreads) {
    const float si = s[i];
    int rank = 0;  // ranks are a permutation of [0, K): every idx[0..k) is written once
    for (int jj = 0; jj < K; ++jj) {
      const float sj = s[jj];
      rank += (sj > si) || (sj == si && jj < i);
    }
    if (rank < k) idx[rank] = i;
  }
}

// Small bands: the three sender phases in one workgroup and one launch (the
// scores and the selection stay in LDS; barriers order the phases, and every
// read of last_sent in phase 1 precedes its update in phase 3).
constexpr int kFusedThreads = 1024;
constexpr int kFusedMaxBlocks = 4096;
constexpr int64_t kFusedMaxElems = 131072;  // band elements one CU moves in a few microseconds

// Chunk c of block j (chunks of CH bytes, row-major over the block's B*bh
// rows of bw*C elements): byte offset in a tensor of `rows` rows per batch
// item whose band starts at row r0.
__device__ __forceinline__ int64_t chunk_off(const BandGeom& g, int j, int c, int cpr, int es, int CH,
                                             int rows = -1, int r0 = 0) {
  const int rr = c / cpr, cc = c - rr * cpr;
  const int b = rr / g.bh, r = rr - b * g.bh;
  const int by = j / g.nbx, bx = j - by * g.nbx;
  const int R = rows < 0 ? g.h : rows;
  return ((static_cast<int64_t>(b) * R + r0 + by * g.bh + r) * g.W + bx * g.bw) * g.C * es + cc * CH;
}

template <int CH>
struct Chunk;
template <>
struct Chunk<16> { typedef u32x4 T; };
template <>
struct Chunk<4> { typedef unsigned int T; };
template <>
struct Chunk<2> { typedef unsigned short T; };

// Accumulates <a, b>, |a|^2, |b|^2 over the elements of one chunk.
template <int DT, int CH>
__device__ __forceinline__ void chunk_dot(const typename Chunk<CH>::T& ua, const typename Chunk<CH>::T& ub,
                                          float& dot, float& na, float& nb) {
  constexpr int ES = DT == DP_F32 ? 4 : 2;
  constexpr int NE = CH / ES;
  float a[NE], b[NE];
  if constexpr (DT == DP_F32) {
    if constexpr (CH == 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = __uint_as_float(ua[i]);
        b[i] = __uint_as_float(ub[i]);
      }
    } else {
      a[0] = __uint_as_float(ua);
      b[0] = __uint_as_float(ub);
    }
  } else {
    unsigned short ha[NE], hb[NE];
    __builtin_memcpy(ha, &ua, CH);
    __builtin_memcpy(hb, &ub, CH);
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      if constexpr (DT == DP_BF16) {
        a[i] = __uint_as_float(static_cast<unsigned int>(ha[i]) << 16);
        b[i] = __uint_as_float(static_cast<unsigned int>(hb[i]) << 16);
      } else {
        a[i] = static_cast<float>(__builtin_bit_cast(_Float16, ha[i]));
        b[i] = static_cast<float>(__builtin_bit_cast(_Float16, hb[i]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    dot = fmaf(a[i], b[i], dot);
    na = fmaf(a[i], a[i], na);
    nb = fmaf(b[i], b[i], nb);
  }
}

template <int DT, int CH>
__global__ void __launch_bounds__(kFusedThreads)
otil_fused(const char* __restrict__ x, char* __restrict__ last_sent, unsigned char* __restrict__ visited,
           float* __restrict__ scores, int* __restrict__ idx, char* __restrict__ packed, BandGeom g, int k,
           float bonus) {
  typedef typename Chunk<CH>::T VT;
  constexpr int ES = DT == DP_F32 ? 4 : 2;
  constexpr int U = 4;  // blocks per wave in flight
  __shared__ float s[kFusedMaxBlocks];
  __shared__ int sel[kFusedMaxBlocks];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kFusedThreads / 64;
  const int cpr = g.bw * g.C * ES / CH;  // chunks per block row
  const int nch = g.B * g.bh * cpr;      // chunks per block
  // phase 1: scores, one wave per block, U blocks per wave at a time
  for (int j0 = wave; j0 < g.K; j0 += nw * U) {
    float dot[U], na[U], nb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) dot[u] = na[u] = nb[u] = 0.f;
    for (int c = lane; c < nch; c += 64) {
      VT ua[U], ub[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + nw * u;
        if (j < g.K) {
          const int64_t o = chunk_off(g, j, c, cpr, ES, CH);
          ua[u] = *reinterpret_cast<const VT*>(x + o);
          ub[u] = *reinterpret_cast<const VT*>(last_sent + o);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (j0 + nw * u < g.K) chunk_dot<DT, CH>(ua[u], ub[u], dot[u], na[u], nb[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        dot[u] += __shfl_xor(dot[u], off, 64);
        na[u] += __shfl_xor(na[u], off, 64);
        nb[u] += __shfl_xor(nb[u], off, 64);
      }
      const int j = j0 + nw * u;
      if (lane == 0 && j < g.K) {
        const float cosv = dot[u] / fmaxf(sqrtf(na[u]) * sqrtf(nb[u]), 1e-8f);
        const float v = (1.f - cosv) + (visited[j] ? 0.f : bonus);
        scores[j] = v;
        s[j] = v != v ? -INFINITY : v;
      }
    }
  }
  __syncthreads();
  // phase 2: rank every block (descending score, ties to the lower id)
  for (int i = threadIdx.x; i < g.K; i += kFusedThreads) {
    const float si = s[i];
    int rank = 0;
    for (int jj = 0; jj < g.K; ++jj) {
      const float sj = s[jj];
      rank += (sj > si) || (sj == si && jj < i);
    }
    if (rank < k) {
      idx[rank] = i;
      sel[rank] = i;
    }
  }
  __syncthreads();
  // phase 3: pack and update, (selected block, chunk) pairs over all threads
  const int total = k * nch;
  for (int t0 = threadIdx.x; t0 < total; t0 += kFusedThreads * U) {
    VT v[U];
    int64_t so[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + kFusedThreads * u;
      if (t < total) {
        const int p = t / nch, c = t - p * nch;
        so[u] = chunk_off(g, sel[p], c, cpr, ES, CH);
        v[u] = *reinterpret_cast<const VT*>(x + so[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + kFusedThreads * u;
      if (t < total) {
        *reinterpret_cast<VT*>(packed + static_cast<int64_t>(t) * CH) = v[u];
        *reinterpret_cast<VT*>(last_sent + so[u]) = v[u];
      }
    }
  }
  for (int p = threadIdx.x; p < k; p += kFusedThreads) visited[sel[p]] = 1;
}

// Pack (multi-kernel path): one CH-byte chunk per thread over all selected
// blocks; block idx[p] of x -> packed[p] and -> last_sent; visited[idx[p]] = 1.
template <int CH>
__global__ void __launch_bounds__(kCopyThreads)
otil_pack(const char* __restrict__ x, char* __restrict__ last_sent, unsigned char* __restrict__ visited,
          const int* __restrict__ idx, char* __restrict__ packed, BandGeom g, int es, int cpr, int nch,
          int total) {
  typedef typename Chunk<CH>::T VT;
  const int t = blockIdx.x * kCopyThreads + threadIdx.x;
  if (t >= total) return;
  const int p = t / nch, c = t - p * nch;
  const int j = idx[p];
  if (j < 0 || j >= g.K) return;
  const int64_t o = chunk_off(g, j, c, cpr, es, CH);
  const VT v = *reinterpret_cast<const VT*>(x + o);
  *reinterpret_cast<VT*>(packed + static_cast<int64_t>(t) * CH) = v;
  *reinterpret_cast<VT*>(last_sent + o) = v;
  if (c == 0) visited[j] = 1;
}

// Unpack: one CH-byte chunk per thread; packed[p] -> block idx[p] of the
// peer's band, rows [r0, r0 + h) of dst [B, H, W, C].  Ids outside the block
// grid are skipped.
template <int CH>
__global__ void __launch_bounds__(kCopyThreads)
otil_unpack(char* __restrict__ dst, const char* __restrict__ packed, const int* __restrict__ idx, BandGeom g,
            int H, int r0, int es, int cpr, int nch, int total) {
  typedef typename Chunk<CH>::T VT;
  const int t = blockIdx.x * kCopyThreads + threadIdx.x;
  if (t >= total) return;
  const int p = t / nch, c = t - p * nch;
  const int j = idx[p];
  if (j < 0 || j >= g.K) return;
  *reinterpret_cast<VT*>(dst + chunk_off(g, j, c, cpr, es, CH, H, r0)) =
      *reinterpret_cast<const VT*>(packed + static_cast<int64_t>(t) * CH);
}

// Chunk width for runs of `run` bytes (bw * C * es) starting at multiples of
// `run` from bases that are all aligned as checked.
int chunk_width(int64_t run, std::initializer_list<const void*> ptrs) {
  auto all = [&](size_t a) {
    for (const void* p : ptrs)
      if (reinterpret_cast<uintptr_t>(p) % a) return false;
    return true;
  };
  if (run % 16 == 0 && all(16)) return 16;
  if (run % 4 == 0 && all(4)) return 4;
  return 2;
}

size_t otil_elem_size(dp_dtype dt) { return dt == DP_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
bool otil_dtype_ok(dp_dtype dt) { return dt == DP_F32 || dt == DP_BF16 || dt == DP_F16; }

}  // namespace

DP_API dp_status dp_otil_select_pack(const void* x, void* last_sent, uint8_t* visited, float* scores,
                                     int32_t* idx, void* packed, int64_t B, int64_t h, int64_t W, int64_t C,
                                     int64_t bh, int64_t bw, int64_t k, float bonus, dp_dtype dt,
                                     hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_otil_select_pack";
  if (!x || !last_sent || !visited || !scores || !idx || !packed) return fail(DP_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if (B <= 0 || h <= 0 || W <= 0 || C <= 0 || bh <= 0 || bw <= 0 || k <= 0)
    return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (!otil_dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  if (h % bh != 0 || W % bw != 0) return fail(DP_ERR_INVALID_ARG, "%s: h, W must be multiples of bh, bw", name);
  if (!std::isfinite(bonus)) return fail(DP_ERR_INVALID_ARG, "%s: bonus must be finite", name);
  const int64_t K = (h / bh) * (W / bw);
  if (k > K) return fail(DP_ERR_INVALID_ARG, "%s: k = %lld exceeds the %lld blocks", name, (long long)k, (long long)K);
  if (K > kMaxBlocks) return fail(DP_ERR_UNSUPPORTED, "%s: more than %d blocks", name, kMaxBlocks);
  const int64_t n_band = B * h * W * C;
  if (n_band > 0x7FFFFFFF || B * bh * bw * C > 0x7FFFFFFF) return fail(DP_ERR_UNSUPPORTED, "%s: band exceeds 2^31 elements", name);
  const size_t es = otil_elem_size(dt);
  const size_t nb = static_cast<size_t>(n_band) * es, pb = static_cast<size_t>(k * B * bh * bw * C) * es;
  const void* p[6] = {x, last_sent, visited, scores, idx, packed};
  const size_t sz[6] = {nb, nb, static_cast<size_t>(K), static_cast<size_t>(K) * 4, static_cast<size_t>(k) * 4, pb};
  for (int a = 0; a < 6; ++a)
    for (int b = a + 1; b < 6; ++b)
      if (dp::overlaps(p[a], sz[a], p[b], sz[b])) return fail(DP_ERR_INVALID_ARG, "%s: buffers overlap", name);
  if (!aligned(x, es) || !aligned(last_sent, es) || !aligned(packed, es) || !aligned(scores, 4) || !aligned(idx, 4))
    return fail(DP_ERR_INVALID_ARG, "%s: pointers must be aligned to their element size", name);
  if (nb > 0x7FFFFFFFu) return fail(DP_ERR_UNSUPPORTED, "%s: band exceeds 2 GiB", name);
  dp::clear_error();
  const BandGeom g{(int)B, (int)h, (int)W, (int)C, (int)bh, (int)bw, (int)(W / bw), (int)K};
  const char* xc = static_cast<const char*>(x);
  char* lc = static_cast<char*>(last_sent);
  char* pc = static_cast<char*>(packed);
  // block rows start at multiples of bw * C * es from the band's base
  const int CH = chunk_width(bw * C * static_cast<int64_t>(es), {x, last_sent, packed});
  if (K <= kFusedMaxBlocks && n_band <= kFusedMaxElems) {
#define DP_OTIL_FUSED(DT, CW) \
  hipLaunchKernelGGL((otil_fused<DT, CW>), dim3(1), dim3(kFusedThreads), 0, stream, xc, lc, visited, scores, idx, pc, g, (int)k, bonus)
    if (dt == DP_F32) {
      if (CH == 16) DP_OTIL_FUSED(DP_F32, 16);
      else DP_OTIL_FUSED(DP_F32, 4);
    } else if (dt == DP_BF16) {
      if (CH == 16) DP_OTIL_FUSED(DP_BF16, 16);
      else if (CH == 4) DP_OTIL_FUSED(DP_BF16, 4);
      else DP_OTIL_FUSED(DP_BF16, 2);
    } else {
      if (CH == 16) DP_OTIL_FUSED(DP_F16, 16);
      else if (CH == 4) DP_OTIL_FUSED(DP_F16, 4);
      else DP_OTIL_FUSED(DP_F16, 2);
    }
#undef DP_OTIL_FUSED
    return dp::check_launch(name);
  }
  const dim3 sgrid(static_cast<unsigned>((K + 3) / 4));
  if (dt == DP_F32)
    hipLaunchKernelGGL(otil_score<DP_F32>, sgrid, dim3(kScoreThreads), 0, stream, x, last_sent, visited, scores, g, (int)K, bonus);
  else if (dt == DP_BF16)
    hipLaunchKernelGGL(otil_score<DP_BF16>, sgrid, dim3(kScoreThreads), 0, stream, x, last_sent, visited, scores, g, (int)K, bonus);
  else
    hipLaunchKernelGGL(otil_score<DP_F16>, sgrid, dim3(kScoreThreads), 0, stream, x, last_sent, visited, scores, g, (int)K, bonus);
  hipLaunchKernelGGL(otil_select, dim3(1), dim3(kSelectThreads), 0, stream, scores, (int)K, (int)k, idx);
  const int cpr = static_cast<int>(bw * C * es / CH), nch = static_cast<int>(B * bh) * cpr;
  const int total = static_cast<int>(k) * nch;
  const dim3 pgrid(static_cast<unsigned>((total + kCopyThreads - 1) / kCopyThreads));
  if (CH == 16)
    hipLaunchKernelGGL(otil_pack<16>, pgrid, dim3(kCopyThreads), 0, stream, xc, lc, visited, idx, pc, g, (int)es, cpr, nch, total);
  else if (CH == 4)
    hipLaunchKernelGGL(otil_pack<4>, pgrid, dim3(kCopyThreads), 0, stream, xc, lc, visited, idx, pc, g, (int)es, cpr, nch, total);
  else
    hipLaunchKernelGGL(otil_pack<2>, pgrid, dim3(kCopyThreads), 0, stream, xc, lc, visited, idx, pc, g, (int)es, cpr, nch, total);
  return dp::check_launch(name);
}

DP_API dp_status dp_otil_unpack(void* dst, const void* packed, const int32_t* idx, int64_t B, int64_t H, int64_t W,
                                int64_t C, int64_t r0, int64_t h, int64_t bh, int64_t bw, int64_t k, dp_dtype dt,
                                hipStream_t stream) {
  using dp::fail;
  const char* name = "dp_otil_unpack";
  if (!dst || !packed || !idx) return fail(DP_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if (B <= 0 || H <= 0 || W <= 0 || C <= 0 || h <= 0 || bh <= 0 || bw <= 0 || k <= 0)
    return fail(DP_ERR_INVALID_ARG, "%s: sizes must be positive", name);
  if (!otil_dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "%s: bad dtype", name);
  if (r0 < 0 || r0 + h > H) return fail(DP_ERR_INVALID_ARG, "%s: rows [r0, r0+h) outside [0, H)", name);
  if (h % bh != 0 || W % bw != 0) return fail(DP_ERR_INVALID_ARG, "%s: h, W must be multiples of bh, bw", name);
  const int64_t K = (h / bh) * (W / bw);
  if (k > K) return fail(DP_ERR_INVALID_ARG, "%s: k exceeds the number of blocks", name);
  if (B * H * W * C > 0x7FFFFFFF) return fail(DP_ERR_UNSUPPORTED, "%s: latent exceeds 2^31 elements", name);
  const size_t es = otil_elem_size(dt);
  const size_t db = static_cast<size_t>(B * H * W * C) * es, pb = static_cast<size_t>(k * B * bh * bw * C) * es;
  if (dp::overlaps(dst, db, packed, pb) || dp::overlaps(dst, db, idx, static_cast<size_t>(k) * 4))
    return fail(DP_ERR_INVALID_ARG, "%s: buffers overlap", name);
  if (!aligned(dst, es) || !aligned(packed, es) || !aligned(idx, 4))
    return fail(DP_ERR_INVALID_ARG, "%s: pointers must be aligned to their element size", name);
  if (db > 0x7FFFFFFFu) return fail(DP_ERR_UNSUPPORTED, "%s: latent exceeds 2 GiB", name);
  dp::clear_error();
  const BandGeom g{(int)B, (int)h, (int)W, (int)C, (int)bh, (int)bw, (int)(W / bw), (int)K};
  const int CH = chunk_width(bw * C * static_cast<int64_t>(es), {dst, packed});
  const int cpr = static_cast<int>(bw * C * es / CH), nch = static_cast<int>(B * bh) * cpr;
  const int total = static_cast<int>(k) * nch;
  const dim3 grid(static_cast<unsigned>((total + kCopyThreads - 1) / kCopyThreads));
  char* dc = static_cast<char*>(dst);
  const char* pc = static_cast<const char*>(packed);
  if (CH == 16)
    hipLaunchKernelGGL(otil_unpack<16>, grid, dim3(kCopyThreads), 0, stream, dc, pc, idx, g, (int)H, (int)r0, (int)es, cpr, nch, total);
  else if (CH == 4)
    hipLaunchKernelGGL(otil_unpack<4>, grid, dim3(kCopyThreads), 0, stream, dc, pc, idx, g, (int)H, (int)r0, (int)es, cpr, nch, total);
  else
    hipLaunchKernelGGL(otil_unpack<2>, grid, dim3(kCopyThreads), 0, stream, dc, pc, idx, g, (int)H, (int)r0, (int)es, cpr, nch, total);
  return dp::check_launch(name);
}
