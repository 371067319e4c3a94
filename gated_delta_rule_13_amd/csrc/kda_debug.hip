// Precondition checks of the KDA_DEBUG build (libkda_debug.so): before an operator call
// launches its work, one kernel scans the value arrays for the ranges that kda.h states and
// the kernels rely on -- the log-decay g in [-5, 0] (the lower bound g_min = -5 of KDA's
// decay, page "【轻量化复刻大模型】线性注意力（Linear Attention）", section 3.1; the block
// operands of the matrix-core kernels stay within e^+-80 only above it), beta and the Gated
// Delta Rule-2 erase / write gates in [0, 1], and cu_seqlens non-decreasing from 0 to T --
// and sets one bit per violated condition in a flag word. The host waits for it on the
// caller's stream and reports a violation as KDA_ERR_PRECONDITION without launching the work.
// NaN fails every range test. The release build compiles none of this.
#if KDA_DEBUG
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kda_internal.h"

namespace kda {
namespace {

// Violations found by the last check on this device (bits of DebugCheck::Bit).
__device__ unsigned g_debug_flags;

__global__ void debug_clear_kernel() {
  if (threadIdx.x == 0) atomicAnd(&g_debug_flags, 0u);
}

// One array checked against [lo, hi]; n elements.
struct Range {
  const float* p;
  long long n;
  float lo, hi;
  unsigned bit;
};

__global__ __launch_bounds__(256) void debug_range_kernel(Range r0, Range r1, Range r2, Range r3) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned bad = 0;
  const Range rs[4] = {r0, r1, r2, r3};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const Range& r = rs[a];
    if (!r.p) continue;
    bool ok = true;
    for (long long i = i0; i < r.n; i += stride) {
      const float x = r.p[i];
      ok = ok && (x >= r.lo && x <= r.hi);  // false for NaN
    }
    if (!ok) bad |= r.bit;
  }
  if (bad) atomicOr(&g_debug_flags, bad);
}

__global__ void debug_cu_kernel(const int32_t* cu, int N, int T, unsigned bit) {
  bool ok = true;
  for (int i = threadIdx.x; i <= N; i += blockDim.x) {
    const int c = cu[i];
    if (i == 0 && c != 0) ok = false;
    if (i == N && c != T) ok = false;
    if (i > 0 && c < cu[i - 1]) ok = false;
  }
  if (!ok) atomicOr(&g_debug_flags, bit);
}

}  // namespace

hipError_t debug_check(const DebugCheck& c, hipStream_t stream, unsigned& flags) {
  flags = 0;
  debug_clear_kernel<<<1, 64, 0, stream>>>();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Range r[4];
  for (int i = 0; i < 4; ++i) r[i] = Range{c.arr[i], c.n[i], c.lo[i], c.hi[i], c.bit[i]};
  long long most = 1;
  for (int i = 0; i < 4; ++i)
    if (c.arr[i] && c.n[i] > most) most = c.n[i];
  const long long blocks = std::min<long long>(4096, (most + 255) / 256);
  debug_range_kernel<<<(unsigned)blocks, 256, 0, stream>>>(r[0], r[1], r[2], r[3]);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (c.cu) {
    debug_cu_kernel<<<1, 256, 0, stream>>>(c.cu, c.N, c.T, DebugCheck::kCu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  return hipMemcpyFromSymbol(&flags, HIP_SYMBOL(g_debug_flags), sizeof(flags), 0,
                             hipMemcpyDeviceToHost);
}

}  // namespace kda
#endif  // KDA_DEBUG
