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
// bf16 path (gfx950): 128x128 output tile per 256-thread block, K staged
// through LDS in 64-wide slices (double-buffered, one barrier per slice).
// Each wave owns a 64x64 sub-tile computed with v_mfma_f32_32x32x16_bf16 as
// (W rows) x (A rows)^T, so an accumulator lane holds 4 consecutive output
// channels of one output row and the epilogue writes 8-byte runs.
// f32 path: a plain LDS-tiled FMA kernel (correctness path for fp32 shares).
#include "dp_internal.h"

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64, kPad = 8, kLd = kBK + kPad;
constexpr int kThreads = 256;

struct ConvGeom {
  const bf16_t* x;
  const bf16_t* halo_top;
  const bf16_t* halo_bot;
  int h, W, Cin;
};

template <bool CONV>
__global__ void __launch_bounds__(kThreads, 2)
gemm_bf16_mfma(const bf16_t* __restrict__ a, ConvGeom geo, const bf16_t* __restrict__ wt,
               const float* __restrict__ bias, bf16_t* __restrict__ y, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kBM * kLd];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kBN * kLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;

  // Global->LDS assignment: 16-byte chunk kc of rows r_u = (tid>>3) + 32u.
  const int kc = tid & 7;
  const int rbase = tid >> 3;
  int am_b[4], am_i[4], am_c[4];
  bool am_ok[4], wn_ok[4];
  int64_t a_row_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + rbase + 32 * u;
    am_ok[u] = m < M;
    wn_ok[u] = (n0 + rbase + 32 * u) < N;
    if constexpr (CONV) {
      const int hw = geo.h * geo.W;
      const int mm = am_ok[u] ? m : 0;
      am_b[u] = mm / hw;
      const int rem = mm - am_b[u] * hw;
      am_i[u] = rem / geo.W;
      am_c[u] = rem - am_i[u] * geo.W;
      a_row_off[u] = 0;
    } else {
      a_row_off[u] = static_cast<int64_t>(m) * K;
      am_b[u] = am_i[u] = am_c[u] = 0;
    }
  }

  const int n_kt = K / kBK;
  const int kpt = CONV ? geo.Cin / kBK : 1;  // k-slices per conv tap
  u32x4 ra[4], rw[4];

  auto load_tile = [&](int kt) {
    const int kofs = kt * kBK + kc * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // activations
      const bf16_t* src = nullptr;
      if (am_ok[u]) {
        if constexpr (CONV) {
          const int tap = kt / kpt;
          const int c0 = (kt - tap * kpt) * kBK + kc * 8;
          const int dy = tap / 3 - 1, dx = tap % 3 - 1;
          const int row = am_i[u] + dy, col = am_c[u] + dx;
          if (col >= 0 && col < geo.W) {
            if (row < 0) {
              if (geo.halo_top)
                src = geo.halo_top + (static_cast<int64_t>(am_b[u]) * geo.W + col) * geo.Cin + c0;
            } else if (row >= geo.h) {
              if (geo.halo_bot)
                src = geo.halo_bot + (static_cast<int64_t>(am_b[u]) * geo.W + col) * geo.Cin + c0;
            } else {
              src = geo.x + ((static_cast<int64_t>(am_b[u]) * geo.h + row) * geo.W + col) * geo.Cin + c0;
            }
          }
        } else {
          src = a + a_row_off[u] + kofs;
        }
      }
      ra[u] = src ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
      // weights
      const int n = n0 + rbase + 32 * u;
      rw[u] = wn_ok[u] ? *reinterpret_cast<const u32x4*>(wt + static_cast<int64_t>(n) * K + kofs)
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = rbase + 32 * u;
      *reinterpret_cast<u32x4*>(&As[buf][r * kLd + kc * 8]) = ra[u];
      *reinterpret_cast<u32x4*>(&Bs[buf][r * kLd + kc * 8]) = rw[u];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      bf16x8 wa[2], xb[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        wa[nb] = *reinterpret_cast<const bf16x8*>(
            &Bs[cur][(wn * 64 + nb * 32 + l32) * kLd + s * 16 + g * 8]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        xb[mb] = *reinterpret_cast<const bf16x8*>(
            &As[cur][(wm * 64 + mb * 32 + l32) * kLd + s * 16 + g * 8]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[nb], xb[mb], acc[nb][mb], 0, 0, 0);
    }
    if (kt + 1 < n_kt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds rows n = 8*(e/4) + 4*g + e%4 of column m = l32.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = m0 + wm * 64 + mb * 32 + l32;
      const int nblk = n0 + wn * 64 + nb * 32;
      if (m >= M || nblk >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nblk + 8 * q + 4 * g;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[nb][mb][4 * q + e] + (bias ? bias[n + e] : 0.f);
        u32x2 packed = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(y + static_cast<int64_t>(m) * N + n) = packed;
      }
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
         const float* __restrict__ hb, int h, int W, int Cin, const float* __restrict__ wt,
         const float* __restrict__ bias, float* __restrict__ y, int M, int N, int K) {
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
      Bs[kk][r] = (n < N && k < K) ? wt[static_cast<int64_t>(n) * K + k] : 0.f;
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
      if (m < M && n < N) y[static_cast<int64_t>(m) * N + n] = acc[i][j] + (bias ? bias[n] : 0.f);
    }
}

dp_status run_gemm(bool conv, const void* a, const void* x, const void* ht, const void* hb, int h,
                   int W, int Cin, const void* wt, const float* bias, void* y, int64_t M,
                   int64_t N, int64_t K, dp_dtype dt, hipStream_t st, const char* name) {
  if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF)
    return dp::fail(DP_ERR_UNSUPPORTED, "%s: dimension exceeds 2^31", name);
  dp::clear_error();
  if (dt == DP_BF16) {
    if (K % kBK != 0 || N % 32 != 0 || (conv && Cin % kBK != 0))
      return dp::fail(DP_ERR_UNSUPPORTED, "%s: bf16 path needs Cin %% 64 == 0 and Cout %% 32 == 0", name);
    const int64_t gy = (M + kBM - 1) / kBM;
    if (gy > 65535) return dp::fail(DP_ERR_UNSUPPORTED, "%s: M too large", name);
    const dim3 grid(static_cast<unsigned>((N + kBN - 1) / kBN), static_cast<unsigned>(gy));
    ConvGeom geo{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(ht),
                 static_cast<const bf16_t*>(hb), h, W, Cin};
    if (conv)
      hipLaunchKernelGGL(gemm_bf16_mfma<true>, grid, dim3(kThreads), 0, st, nullptr, geo,
                         static_cast<const bf16_t*>(wt), bias, static_cast<bf16_t*>(y), (int)M,
                         (int)N, (int)K);
    else
      hipLaunchKernelGGL(gemm_bf16_mfma<false>, grid, dim3(kThreads), 0, st,
                         static_cast<const bf16_t*>(a), geo, static_cast<const bf16_t*>(wt), bias,
                         static_cast<bf16_t*>(y), (int)M, (int)N, (int)K);
  } else {
    const int64_t gy = (M + kFT - 1) / kFT;
    if (gy > 65535) return dp::fail(DP_ERR_UNSUPPORTED, "%s: M too large", name);
    const dim3 grid(static_cast<unsigned>((N + kFT - 1) / kFT), static_cast<unsigned>(gy));
    if (conv)
      hipLaunchKernelGGL(gemm_f32<true>, grid, dim3(kThreads), 0, st, nullptr,
                         static_cast<const float*>(x), static_cast<const float*>(ht),
                         static_cast<const float*>(hb), h, W, Cin, static_cast<const float*>(wt),
                         bias, static_cast<float*>(y), (int)M, (int)N, (int)K);
    else
      hipLaunchKernelGGL(gemm_f32<false>, grid, dim3(kThreads), 0, st,
                         static_cast<const float*>(a), nullptr, nullptr, nullptr, 0, 0, 0,
                         static_cast<const float*>(wt), bias, static_cast<float*>(y), (int)M,
                         (int)N, (int)K);
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
  return run_gemm(false, x, nullptr, nullptr, nullptr, 0, 0, 0, w, bias, y, M, Cout, Cin, dt, stream,
                  "dp_linear");
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
  return run_gemm(true, nullptr, x, halo_top, halo_bot, (int)h, (int)W, (int)Cin, w, bias, y,
                  B * h * W, Cout, 9 * Cin, dt, stream, "dp_conv3x3_stale_halo");
}
