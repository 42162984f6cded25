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
// (K as [key][d], V transposed as [d][key]), double-buffered with one barrier
// per tile.  Per 32-key block a wave computes the transposed scores
//     S^T[key][query] = K . Q^T      (v_mfma_f32_32x32x16_bf16, 4 k-steps over d)
// so that accumulator lane l holds 16 scores of the single query l % 32: the
// softmax max/sum are in-lane, plus one exchange with lane l ^ 32.  K rows are
// loaded with row index bits 2 and 3 swapped; with that permutation the 8
// probabilities a lane holds for each 16-key step are 8 consecutive keys, which
// is exactly the B operand layout of the transposed output product
//     O^T[d][query] += V^T . P^T      (2 d-blocks x 2 k-steps per 32 keys).
// Online softmax in base 2 (scale * log2 e folded into one FMA per score),
// float32 running max and per-lane partial row sums, P rounded to bf16 for
// the second product.  Output rows are normalised once at the end.
//
// f32 (d = 32 or 64)
// ------------------
// One thread per query, K/V tiles of 32 keys in LDS, the same online softmax
// in float32 with expf: the correctness path for fp32 shares.
#include <math.h>

#include "dp_internal.h"

namespace {

constexpr int kD = 64;
constexpr int kBMq = 128;  // queries per block
constexpr int kBNk = 64;   // keys per tile
constexpr int kKLd = kD + 8;
constexpr int kVLd = kBNk + 8;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  u32x4 u;
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(s[base + 2 * j], s[base + 2 * j + 1]);
  return __builtin_bit_cast(bf16x8, u);
}

__global__ void __launch_bounds__(256, 2)
attn_bf16_d64(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
              const bf16_t* __restrict__ v, bf16_t* __restrict__ out, int Tq, int Tkv, int H,
              float c) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][kBNk * kKLd];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][kD * kVLd];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t C = static_cast<int64_t>(H) * kD;
  const int qi = blockIdx.x * kBMq + wave * 32 + l32;
  const bool q_ok = qi < Tq;

  bf16x8 qop[4];
  {
    const bf16_t* qp = q + (static_cast<int64_t>(b) * Tq + (q_ok ? qi : 0)) * C + h * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 u = q_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qop[s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  // K row permutation: swap bits 2 and 3 of the row index.
  const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);

  const bf16_t* kbase = k + static_cast<int64_t>(b) * Tkv * C + h * kD;
  const bf16_t* vbase = v + static_cast<int64_t>(b) * Tkv * C + h * kD;
  const int ld_key = tid >> 3, ld_ch = (tid & 7) * 8;
  u32x4 rk[2], rv[2];
  auto load = [&](int kt) {
    const int key0 = kt * kBNk;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = key0 + ld_key + 32 * u;
      rk[u] = kk < Tkv ? *reinterpret_cast<const u32x4*>(kbase + kk * C + ld_ch) : u32x4{0u, 0u, 0u, 0u};
      const int vk = key0 + 2 * ld_key + u;
      rv[u] = vk < Tkv ? *reinterpret_cast<const u32x4*>(vbase + vk * C + ld_ch) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<u32x4*>(&Ks[buf][(ld_key + 32 * u) * kKLd + ld_ch]) = rk[u];
    // rv[0] = V[2p][d0..d0+7], rv[1] = V[2p+1][d0..d0+7]: write (V[2p][d], V[2p+1][d]) pairs.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned int lo = (rv[0][j] & 0xFFFFu) | (rv[1][j] << 16);
      const unsigned int hi = (rv[0][j] >> 16) | (rv[1][j] & 0xFFFF0000u);
      *reinterpret_cast<unsigned int*>(&Vt[buf][(ld_ch + 2 * j) * kVLd + 2 * ld_key]) = lo;
      *reinterpret_cast<unsigned int*>(&Vt[buf][(ld_ch + 2 * j + 1) * kVLd + 2 * ld_key]) = hi;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[0][i] = o[1][i] = 0.f;

  const int nt = (Tkv + kBNk - 1) / kBNk;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nt) load(kt + 1);

    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[blk][i] = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&Ks[cur][(32 * blk + krow) * kKLd + 16 * st + 8 * g]);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[st], s[blk], 0, 0, 0);
      }
    }
    if ((kt + 1) * kBNk > Tkv) {  // ragged last tile: mask keys beyond T_kv
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * g + (i & 3);
          const int pr = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
          if (kt * kBNk + 32 * blk + pr >= Tkv) s[blk][i] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[blk][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[blk][i], c, -m_new));
        s[blk][i] = p;
        rs += p;
      }
    l_run = fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[0][i] *= alpha;
      o[1][i] *= alpha;
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pack8(s[blk], 8 * s2);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(
              &Vt[cur][(32 * db + l32) * kVLd + 32 * blk + 16 * s2 + 8 * g]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
        }
      }
    if (kt + 1 < nt) store(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (q_ok) {
    bf16_t* op = out + (static_cast<int64_t>(b) * Tq + qi) * C + h * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * g;
        u32x2 pk = {pack_bf16x2(o[db][4 * qq] * inv, o[db][4 * qq + 1] * inv),
                    pack_bf16x2(o[db][4 * qq + 2] * inv, o[db][4 * qq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
  }
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
  (void)B, (void)H, (void)Tq, (void)T_kv, (void)d, (void)dt;
  return 0;
}

DP_API dp_status dp_attn_stale_kv(const void* q, const void* k_buf, const void* v_buf, void* out,
                                  int64_t B, int64_t H, int64_t Tq, int64_t T_kv, int64_t d,
                                  float scale, dp_dtype dt, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  using dp::fail;
  (void)ws, (void)ws_bytes;
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
  const float sc = scale > 0.f ? scale : static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
  dp::clear_error();
  if (dt == DP_BF16) {
    const dim3 grid(static_cast<unsigned>((Tq + kBMq - 1) / kBMq), static_cast<unsigned>(H),
                    static_cast<unsigned>(B));
    hipLaunchKernelGGL(attn_bf16_d64, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k_buf), static_cast<const bf16_t*>(v_buf),
                       static_cast<bf16_t*>(out), (int)Tq, (int)T_kv, (int)H, sc * kLog2e);
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
