// K/V buffer splice: the rank's fresh K/V rows overwrite their own token range
// of the full-image stale buffers; every other token keeps its bits.
//
// Method source: "OTIL for SDXL on 4x L40S", "Self-tests" (the local slice is
// exactly fresh, a remote position is stale memory, never a blend) and the xDiT
// issue thread "Tensor Parallelism with Stale Activations ..." (full spatial
// shape K/V buffers per layer).
//
// The copy is HBM-bound: 2 * (read fresh + write buffer) bytes.  The band of
// each batch item is one contiguous byte range of both the fresh tensor and
// the buffer, so the kernel streams 2*B contiguous segments with the widest
// access (16 B when every address and the segment length allow it).
#include "dp_internal.h"

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 2;

template <typename V>
__global__ void __launch_bounds__(kThreads)
splice_kernel(char* __restrict__ k_buf, char* __restrict__ v_buf, const char* __restrict__ k_fresh,
              const char* __restrict__ v_fresh, int64_t n_vec, int64_t buf_batch_bytes,
              int64_t dst_offset_bytes, int64_t fresh_batch_bytes) {
  const int seg = blockIdx.y;  // (batch, K or V)
  const int64_t b = seg >> 1;
  char* dst = ((seg & 1) ? v_buf : k_buf) + b * buf_batch_bytes + dst_offset_bytes;
  const char* src = ((seg & 1) ? v_fresh : k_fresh) + b * fresh_batch_bytes;
  V* __restrict__ d = reinterpret_cast<V*>(dst);
  const V* __restrict__ s = reinterpret_cast<const V*>(src);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  V tmp[kUnroll];
  if (base + (kUnroll - 1) * kThreads < n_vec) {
    // a whole block's worth: no per-load conditions, so both loads are in
    // flight before the first store waits for its own
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) tmp[u] = __builtin_nontemporal_load(s + base + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(tmp[u], d + base + u * kThreads);
    return;
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + u * kThreads;
    if (i < n_vec) tmp[u] = __builtin_nontemporal_load(s + i);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + u * kThreads;
    if (i < n_vec) __builtin_nontemporal_store(tmp[u], d + i);
  }
}

template <typename V>
dp_status launch(char* kb, char* vb, const char* kf, const char* vf, int64_t B, int64_t seg_bytes,
                 int64_t buf_batch, int64_t off, int64_t fresh_batch, hipStream_t st) {
  const int64_t n_vec = seg_bytes / static_cast<int64_t>(sizeof(V));
  const int64_t per_block = kThreads * kUnroll;
  const int64_t gx = (n_vec + per_block - 1) / per_block;
  if (gx > 0x7FFFFFFF || 2 * B > 65535)
    return dp::fail(DP_ERR_UNSUPPORTED, "dp_kv_buffer_splice: grid too large");
  hipLaunchKernelGGL(splice_kernel<V>, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(2 * B)),
                     dim3(kThreads), 0, st, kb, vb, kf, vf, n_vec, buf_batch, off, fresh_batch);
  return dp::check_launch("dp_kv_buffer_splice");
}

}  // namespace

DP_API dp_status dp_kv_buffer_splice(void* k_buf, void* v_buf, const void* k_fresh,
                                     const void* v_fresh, int64_t B, int64_t T_kv, int64_t C,
                                     int64_t t0, int64_t T_loc, dp_dtype dt, hipStream_t stream) {
  using dp::fail;
  if (!k_buf || !v_buf || !k_fresh || !v_fresh)
    return fail(DP_ERR_INVALID_ARG, "dp_kv_buffer_splice: NULL pointer");
  if (B <= 0 || T_kv <= 0 || C <= 0 || T_loc <= 0)
    return fail(DP_ERR_INVALID_ARG, "dp_kv_buffer_splice: sizes must be positive");
  if (t0 < 0 || t0 + T_loc > T_kv)
    return fail(DP_ERR_INVALID_ARG, "dp_kv_buffer_splice: rows [%lld, %lld) outside [0, %lld)",
                (long long)t0, (long long)(t0 + T_loc), (long long)T_kv);
  if (!dp::dtype_ok(dt)) return fail(DP_ERR_INVALID_ARG, "dp_kv_buffer_splice: bad dtype");
  const int64_t es = static_cast<int64_t>(dp::dtype_size(dt));
  const size_t buf_bytes = static_cast<size_t>(B * T_kv * C * es);
  const size_t fresh_bytes = static_cast<size_t>(B * T_loc * C * es);
  if (dp::overlaps(k_buf, buf_bytes, v_buf, buf_bytes) ||
      dp::overlaps(k_fresh, fresh_bytes, k_buf, buf_bytes) ||
      dp::overlaps(k_fresh, fresh_bytes, v_buf, buf_bytes) ||
      dp::overlaps(v_fresh, fresh_bytes, k_buf, buf_bytes) ||
      dp::overlaps(v_fresh, fresh_bytes, v_buf, buf_bytes))
    return fail(DP_ERR_INVALID_ARG, "dp_kv_buffer_splice: buffers overlap");

  const int64_t seg = T_loc * C * es, buf_batch = T_kv * C * es, off = t0 * C * es;
  // Widest access that every segment start and length allow.
  uintptr_t bits = reinterpret_cast<uintptr_t>(k_buf) | reinterpret_cast<uintptr_t>(v_buf) |
                   reinterpret_cast<uintptr_t>(k_fresh) | reinterpret_cast<uintptr_t>(v_fresh) |
                   static_cast<uintptr_t>(seg) | static_cast<uintptr_t>(buf_batch) |
                   static_cast<uintptr_t>(off);
  char* kb = static_cast<char*>(k_buf);
  char* vb = static_cast<char*>(v_buf);
  const char* kf = static_cast<const char*>(k_fresh);
  const char* vf = static_cast<const char*>(v_fresh);
  dp::clear_error();
  if ((bits & 15) == 0) return launch<u32x4>(kb, vb, kf, vf, B, seg, buf_batch, off, seg, stream);
  if ((bits & 7) == 0) return launch<u32x2>(kb, vb, kf, vf, B, seg, buf_batch, off, seg, stream);
  if ((bits & 3) == 0) return launch<unsigned int>(kb, vb, kf, vf, B, seg, buf_batch, off, seg, stream);
  if ((bits & 1) == 0) return launch<unsigned short>(kb, vb, kf, vf, B, seg, buf_batch, off, seg, stream);
  return launch<unsigned char>(kb, vb, kf, vf, B, seg, buf_batch, off, seg, stream);
}
