// Test probe (test infrastructure, not part of the library): the XCD (accelerator complex
// die) that runs each workgroup of a launch, read from the XCC_ID hardware register.
// The chunk kernels' schedules put the two workgroups that read the same chain's inputs (the
// two value-column halves of a chain, or a later segment's zero-state and transition items)
// a multiple of 8 workgroup indices apart, on the reading that workgroups are dispatched
// round-robin over the device's 8 XCDs: the second then finds the inputs in the first's L2.
// This probe lets a test check that reading on the device at hand.
#include <hip/hip_runtime.h>

namespace {

__global__ void xcd_probe_kernel(int* out, int n) {
  if (threadIdx.x == 0 && (int)blockIdx.x < n) {
    unsigned v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    out[blockIdx.x] = (int)(v & 0xfu);
  }
}

}  // namespace

// out: host array of n ints, filled with the XCD of workgroup i of one launch of n
// workgroups of `threads` threads (1 .. 1024). Returns 0, or a negative code on a bad
// argument or a HIP error.
extern "C" int xcd_of_workgroups(int* out, int n, int threads) {
  if (!out || n <= 0 || threads <= 0 || threads > 1024) return -1;
  int* d = nullptr;
  if (hipMalloc(&d, sizeof(int) * (size_t)n) != hipSuccess) return -2;
  xcd_probe_kernel<<<dim3((unsigned)n), dim3((unsigned)threads)>>>(d, n);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpy(out, d, sizeof(int) * (size_t)n, hipMemcpyDeviceToHost);
  (void)hipFree(d);
  return e == hipSuccess ? 0 : -3;
}
