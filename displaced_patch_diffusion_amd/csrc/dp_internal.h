// Internal helpers shared by the libdp translation units (host validation,
// error reporting, vector types for gfx950 kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "dp.h"

#define DP_API extern "C" __attribute__((visibility("default")))

namespace dp {

// Records `msg` as the calling thread's last error and returns `st`.
dp_status fail(dp_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread's last error.
void clear_error();
// Converts the HIP launch status into a dp_status (recording the detail).
dp_status check_launch(const char* what);

inline bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + bn && pb < pa + an;
}

inline size_t dtype_size(dp_dtype dt) { return dt == DP_BF16 ? 2 : 4; }

// The vector kernels move activations, weights and outputs in 16-byte pieces.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool dtype_ok(dp_dtype dt) { return dt == DP_BF16 || dt == DP_F32; }

}  // namespace dp

// ---------------------------------------------------------------- device side
typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(unsigned int u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int u) { return __uint_as_float(u & 0xFFFF0000u); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned int, v);
}
