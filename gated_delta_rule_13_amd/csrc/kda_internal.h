// Internal interface between the C-ABI host code (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Arguments of one kda_chunk_fwd call, already validated on the host.
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* s0;     // [N, H, dk, dv] or nullptr
  float* sT;           // [N, H, dk, dv] or nullptr
  void* o;
  const int32_t* cu;   // [N + 1] or nullptr
  int N;               // sequences
  int H;
  int T;               // length of the T axis of every [B, H, T, .] tensor
  int dk;
  int dv;
};

// Arguments of one kda_recurrent_step call.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* state;
  void* o;
  int N;
  int H;
};

// Each launcher returns the launch's hipError_t; `bf16` selects the element type of
// q, k, v, o, `per_channel` the gate layout. Unsupported (dk, dv) return
// hipErrorInvalidValue (the host validates before calling).
hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_channel,
                         hipStream_t stream);
hipError_t launch_chunk_f32(const ChunkArgs& a, bool bf16, bool per_channel, hipStream_t stream);
hipError_t launch_chunk_mfma(const ChunkArgs& a, bool per_channel, hipStream_t stream);
bool chunk_mfma_supports(int dk, int dv, int T);

}  // namespace kda
