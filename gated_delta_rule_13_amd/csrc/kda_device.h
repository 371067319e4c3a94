// Small device helpers shared by the kernels: element loads/stores for the two
// supported element types and the chain -> token-range mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Token range of sequence n: tokens [t0, t0 + len) of batch row b on the T axis.
// Without cu_seqlens sequence n is batch row n. Offsets are clamped to [0, T] so that a
// malformed cu_seqlens can never move an access outside the buffers.
struct TokenRange {
  int b;
  int t0;
  int len;
};

__device__ __forceinline__ TokenRange token_range(const int32_t* cu, int n, int T) {
  TokenRange r;
  if (cu) {
    int a = min(max(cu[n], 0), T);
    int e = min(max(cu[n + 1], a), T);
    r.b = 0;
    r.t0 = a;
    r.len = e - a;
  } else {
    r.b = n;
    r.t0 = 0;
    r.len = T;
  }
  return r;
}

}  // namespace kda
