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
  const float* beta;   // [B, H, T]; unused with the Gated Delta Rule-2 gates below
  const float* erase;  // Gated Delta Rule-2 erase gate [B, H, T, dk], or nullptr (KDA)
  const float* write;  // Gated Delta Rule-2 write gate [B, H, T, dv] (with erase)
  const float* s0;     // [N, H, dk, dv] or nullptr
  float* sT;           // [N, H, dk, dv] or nullptr
  void* o;
  const int32_t* cu;   // [N + 1] or nullptr
  int N;               // sequences
  int H;
  int T;               // length of the T axis of every [B, H, T, .] tensor
  int dk;
  int dv;
  // Work list built on the device by the scheduler (see chunk_plan_bytes), or nullptr for
  // one workgroup per chain in chain order. Entry 0 is the item count; item i is
  // ((n * H + h) << 2) | part with part 0 = all value columns, 1 / 2 = first / second half.
  uint32_t* plan;
  int cus;             // compute units of the device (sizes the schedule)
  // Without a work list: split every chain's value columns over two workgroups (the two
  // halves of a chain 8 items apart). Chosen on the host for equal-length batches.
  int split_all;
  // Backward pass only: the state history (see hist_chain_offset), or nullptr.
  void* hist;
  // Segments (chunk_seg_config): items are segments of seg_len tokens, nseg per chain at
  // most; seg_len = 0 for whole chains.
  int seg_len;
  int nseg;
  // Segment plans (launch_chunk_mfma_segplan): capacity in segments, the start states,
  // transitions and zero-start end states of the segments (fp32, seg_slots x H matrices
  // each), and the carried-back queries (bf16 rows of dk values: per head, one row per token
  // past the first segment of its sequence).
  int seg_slots;
  float* seg_mats;
  void* qt;
};

// Arguments of one kda_chunk_bwd call (shapes and validation as kda_chunk_fwd).
struct BwdArgs {
  ChunkArgs f;             // the forward's inputs (o, sT, plan unused)
  const void* dout;        // [B, H, T, dv] gradient of the loss with respect to o
  const float* dsT;        // [N, H, dk, dv] gradient with respect to the final states, or nullptr
  void* dq;                // [B, H, T, dk]
  void* dk;                // [B, H, T, dk]
  void* dv;                // [B, H, T, dv]
  float* dg;               // like g
  float* dbeta;            // [B, H, T] (KDA / Gated DeltaNet)
  float* derase;           // [B, H, T, dk] (Gated Delta Rule-2: f.erase set)
  float* dwrite;           // [B, H, T, dv]
  float* ds0;              // [N, H, dk, dv] or nullptr
  void* hist_s;            // workspace: states at every 16-token block start
  void* hist_ds;           // workspace: state gradients at every 16-token block end
  uint32_t* plan;          // workspace: the work list of the two sequential launches, or nullptr
};

// Arguments of one kda_recurrent_step call.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;   // [N, H]; unused with the Gated Delta Rule-2 gates below
  const float* erase;  // [N, H, dk] or nullptr (KDA)
  const float* write;  // [N, H, dv] (with erase)
  float* state;
  void* o;
  int N;
  int H;
};

// Arguments of one kda_prologue call (every pointer a device array, head-major).
struct PrologueArgs {
  const void* q_in;       // [B, H, T, dk]
  const void* k_in;
  const float* u;         // [B, H, T, dk] decay pre-activation
  const float* A_log;     // [H]
  const float* dt_bias;   // [H, dk]
  const float* beta_in;   // [B, H, T] or nullptr
  void* q_out;
  void* k_out;
  float* g_out;           // [B, H, T, dk]
  float* beta_out;        // [B, H, T] (with beta_in)
  int B, H, T;
};

// Arguments of one kda_epilogue call.
struct EpilogueArgs {
  const void* o_in;       // [B, H, T, dv]
  const void* z;          // [B, H, T, dv] output-gate pre-activation
  const float* weight;    // [dv] or nullptr (= 1)
  float eps;
  void* o_out;
  int B, H, T;
};

// Each launcher returns the launch's hipError_t; `bf16` selects the element type of
// q, k, v, o, `per_channel` the gate layout. Unsupported (dk, dv) return
// hipErrorInvalidValue (the host validates before calling).
hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_channel,
                         hipStream_t stream);
hipError_t launch_chunk_f32(const ChunkArgs& a, bool bf16, bool per_channel, hipStream_t stream);
hipError_t launch_chunk_mfma(const ChunkArgs& a, bool per_channel, hipStream_t stream);
// Head sizes of the matrix-core path, and whether it runs whole chains of T tokens (longer
// chains run only as segment plans, below).
bool chunk_mfma_dims(int dk, int dv);
bool chunk_mfma_supports(int dk, int dv, int T);
hipError_t launch_prologue(const PrologueArgs& a, int dk, bool bf16, hipStream_t stream);
hipError_t launch_epilogue(const EpilogueArgs& a, int dv, bool bf16, hipStream_t stream);
// Bytes of workspace the matrix-core path uses for its schedule (0: no schedule).
size_t chunk_plan_bytes(int N, int H, int dv);

// Chains cut into segments (few chains, long sequences): seg_len tokens each, nseg per
// chain at most; seg_len = 0 when whole chains fill the device. chunk_seg_bytes is the
// workspace of launch_chunk_mfma_segmented (0 when not segmented).
void chunk_seg_config(int N, int H, int T, int dv, int cus, int& seg_len, int& nseg);
size_t chunk_seg_bytes(int N, int H, int T, int dv, int cus);
hipError_t launch_chunk_mfma_segmented(const ChunkArgs& a, bool per_channel, void* ws,
                                       hipStream_t stream);
// Segment plan of the forward (dv = dk = 128, any gates): the launches (planner, items,
// segment chain, corrections). chunk_segplan_bytes is the recommended workspace,
// chunk_segplan_min_bytes the smallest one the plan runs in (0 when not available; for chains
// that whole-chain items can hold, it is the work list the plan may fall back to);
// launch_chunk_mfma_segplan plans within ws_bytes. Chains too long for whole-chain items
// (chunk_mfma_supports false) are always cut into items of at most 2^21 tokens.
size_t chunk_segplan_bytes(int N, int H, int T, int dv, bool packed, int cus);
size_t chunk_segplan_min_bytes(int N, int H, int T, int dv, bool packed);
hipError_t launch_chunk_mfma_segplan(const ChunkArgs& a, bool per_channel, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

// Backward pass (bf16, dk = 128, dv in {64, 128}, one decay per channel or per head).
bool chunk_bwd_supports(int dk, int dv, int T);
// Bytes of one of the two state histories of the backward pass.
size_t chunk_bwd_hist_bytes(int N, int H, int T, int dv, bool packed);
// Forward state pass that records the history (kda_chunk_mfma.hip).
hipError_t launch_chunk_mfma_hist(const ChunkArgs& a, bool per_channel, hipStream_t stream,
                                  bool build_plan = true);
// The work list of packed sequences for the backward's chain passes (whole chains, longest
// first; a.plan, a.cu set).
hipError_t launch_chunk_plan(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd(const BwdArgs& a, bool per_channel, hipStream_t stream);
// Row copies with a zero tail (kda_chunk_bwd.hip): dst[r][c] = src[r][c] for c < min(w_src,
// w_dst), 0 for the rest of the w_dst elements; elem_bytes 2 or 4.
hipError_t launch_pad_rows(const void* src, void* dst, long long rows, int w_src, int w_dst,
                           int elem_bytes, hipStream_t stream);

// KDA_DEBUG builds: the value preconditions of one call (up to four float arrays, each with
// its range and flag bit, and cu_seqlens), checked on the device before the work;
// debug_check waits for the check on `stream` and returns the violated bits in `flags`.
struct DebugCheck {
  static constexpr unsigned kG = 1, kBeta = 2, kErase = 4, kWrite = 8, kCu = 16;
  const float* arr[4] = {nullptr, nullptr, nullptr, nullptr};
  long long n[4] = {0, 0, 0, 0};
  float lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0};
  unsigned bit[4] = {0, 0, 0, 0};
  const int32_t* cu = nullptr;
  int N = 0, T = 0;
  void add(const float* p, long long count, float l, float h, unsigned b) {
    for (int i = 0; i < 4; ++i)
      if (!arr[i]) {
        arr[i] = p; n[i] = count; lo[i] = l; hi[i] = h; bit[i] = b;
        return;
      }
  }
};
hipError_t debug_check(const DebugCheck& c, hipStream_t stream, unsigned& flags);

}  // namespace kda
