/*
 * kda.h — C ABI of the MI355X (gfx950) gated delta rule forward library, libkda.so.
 *
 * The operator is the gated delta rule with per-key-channel decay (Kimi Delta
 * Attention, "KDA"), for every independent chain (one sequence of one head):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = S_t^T q_t,          S_t in R^{dk x dv},  alpha_t = exp(g_t),
 *
 * as boxed in "Token Mixer I", section "Kimi Delta Attention: Improving Delta Rule
 * with Fine-grained Gating". Gated DeltaNet is the case of one decay per head
 * (KDA_GATE_PER_HEAD: g_t is a scalar broadcast over the key channels; "Token
 * Mixer I", section "Linear Attention and the Gated Delta Rule"). There is no query
 * scale. The state is stored row-major with rows = key channels.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HBM of the current HIP device), the
 *    tensors are contiguous and head-major: [B, H, T, d] for per-token data.
 *  - The caller owns every buffer. The library allocates no device memory and never
 *    synchronises the host; work is enqueued on `stream` (NULL = the null stream), and
 *    calls are asynchronous: a KDA_OK return means "enqueued". Its only global state is a
 *    per-device cache of the compute-unit count and, from the first kda_chunk_bwd /
 *    kda_gdr2_chunk_bwd call on a device, one more stream of that device (default
 *    priority, non-blocking, created under a lock and kept until the process ends). The
 *    backward's state-history pass and its reverse carry are independent, and running them
 *    side by side shortens the call; the library keeps that stream rather than take a
 *    second stream argument in every backward entry point for this one use. Each call forks
 *    onto it with an event recorded on `stream` and joins back with a second event before
 *    its last launch (both events belong to the call and are destroyed on every return
 *    path), so all of a call's work still completes in `stream` order.
 *  - Argument errors are detected on the host before anything is launched and are
 *    returned as a status; no exception crosses the ABI. A failed launch returns
 *    KDA_ERR_HIP.
 *  - Preconditions that the host cannot see without reading device memory: g in [-5, 0]
 *    (the lower bound g_min = -5 of KDA's log-decay, page "【轻量化复刻大模型】线性注意力
 *    （Linear Attention）", section 3.1; the kernels rely on it for the exponent ranges of
 *    their scaled operands), beta and the Gated Delta Rule-2 erase / write gates in [0, 1],
 *    cu_seqlens non-decreasing from 0 to T (cu_seqlens[0] = 0, cu_seqlens[num_seqs] = T).
 *    Release builds (libkda.so) do not check them and the results are undefined if they are
 *    violated; out-of-range cu_seqlens entries are clamped to [0, T] so that no access leaves
 *    the buffers. KDA_DEBUG builds (libkda_debug.so, `build.py --debug`) check them in every
 *    forward, decode and backward entry point: a kernel on `stream` scans g, beta or the
 *    gates (every element of the arrays as passed) and cu_seqlens, the host waits for it
 *    (the call synchronises `stream`, so it cannot be captured in a HIP graph), and a
 *    violation returns KDA_ERR_PRECONDITION without launching the work.
 *  - Buffers may not alias each other, except initial_state with final_state.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1,  /* NULL required pointer, non-positive size, inconsistent shape */
  KDA_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement (e.g. dk = 96) */
  KDA_ERR_HIP = 3,          /* a HIP runtime error while launching */
  KDA_ERR_PRECONDITION = 4  /* KDA_DEBUG builds only: an input value outside its stated range */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;   /* element type of q, k, v and o */

typedef enum {
  KDA_GATE_PER_CHANNEL = 0,  /* KDA: g is [.., dk], one log-decay per key channel */
  KDA_GATE_PER_HEAD = 1      /* Gated DeltaNet: g is [..], one log-decay per head and token */
} kda_gate_mode;

/*
 * Bytes of device workspace that kda_chunk_fwd recommends for this problem on the current
 * device (bf16 matrix-core path, dk = 128; every other case returns 0). num_seqs > 0 describes
 * a packed call (cu_seqlens set, B = 1; any other B returns 0), num_seqs = 0 a batch of B
 * sequences of T tokens. kda_chunk_fwd plans within whatever workspace it is given: any size
 * from the work list's (below) up is accepted; the recommended size lets it cut long
 * sequences as it sees fit, a smaller one may make it cut fewer or none. Three uses:
 *
 *  - dv = dk = 128 with packed sequences (num_seqs in 1 .. 1024), or equal-length batches
 *    with fewer chains (B * H) than compute units: the segment plan. A planning kernel
 *    reads the sequence lengths on the device and picks a segment length X (a multiple of
 *    64 tokens, at least max(512, 64 * ceil(T / 4096)) tokens) when cutting the longest
 *    sequences lowers the launch's critical path and the segments fit the workspace;
 *    otherwise it builds the work list described below. The first segment of a cut sequence
 *    runs from the initial state; every later segment runs twice at the same time, from the
 *    zero state (outputs O0, end state B) and from the identity (the dk x dk transition A of
 *    the segment, the product of its token maps, and the queries carried back to the segment
 *    start, Qt). The recurrence is linear in the state, so with S the segment's start state
 *    its outputs are O0 + Qt S and its end state A S + B: a chain over the segments gives
 *    every S and a correction pass adds Qt S. Results equal the whole-chain computation up
 *    to rounding. The workspace holds the plan words, three fp32 dk x dk matrices per segment
 *    slot and head, and one bf16 row of dk carried-back queries per head and token past the
 *    first segment of its sequence. With C = ceil(T / 64), Xmin = min(2^15, max(8,
 *    ceil(C / 64))), M = min(1024, N + floor(N / 8) + ceil(C / Xmin) + 1) and cus the compute
 *    units, the recommendation is S = max(N, min(M, N + ceil(cus / H) + 1)) slots and Q rows
 *    per head, Q = T for packed sequences and B T otherwise when N H < cus, else
 *    Q = ceil(T / 4) (for T >= 2^22, S at least and Q exactly as kda_chunk_fwd's minimum):
 *    R(4 (N + 2 S + 11 + 4 H S)) + 3 S H dk^2 * 4 + Q H dk * 2 bytes, R rounding up to a
 *    multiple of 256 (230 MiB for 8 packed sequences, H = 32, T = 65536). Given another
 *    size, the plan takes as many of the S slots as fit with their matrices, and the rest for
 *    carried-back queries. kda_gdr2_chunk_fwd takes the same plan (its recurrence is linear
 *    in the state too).
 *  - Otherwise, few chains for the device (N * H chains, two workgroups each at dv = 128,
 *    fewer than the compute units) and sequences of at least 1024 tokens: every sequence
 *    is cut into P segments of L tokens (P = CUs / (2 N H) or CUs / (N H) at dv = 64,
 *    L >= 512 a multiple of 64); each segment but the last gets B and A as above,
 *    S_{s+1} = A_s S_s + B_s gives every start state, then all segments compute their
 *    outputs in parallel. Workspace: N H P (2 dk dv + dk^2) * 4 bytes (a smaller workspace
 *    runs without these segments). kda_gdr2_chunk_fwd takes it at dv = 64.
 *  - Otherwise, packed sequences (num_seqs > 0, at most 1024): a work list of
 *    4 * (1 + 2 * num_seqs * H) bytes rounded up to 256, filled on the device by a small
 *    scheduling kernel: it splits the value columns of the longest sequences' chains over
 *    two workgroups and orders the work longest first, so that packed sequences of unequal
 *    length keep every compute unit busy. Work lists do not change results bit for bit:
 *    each value column is computed the same way. This is the smallest workspace a packed
 *    call accepts. (Equal-length batches with enough chains need no workspace: their split
 *    is decided on the host.)
 */
size_t kda_chunk_fwd_workspace_size(int B, int H, int T, int dk, int dv, int num_seqs,
                                    kda_dtype dt);

/*
 * Chunked prefill / training forward over whole sequences.
 *
 * Computes, for every chain, all outputs o_t and optionally the state after the last
 * token. Internally the sequence is cut into chunks and processed with the chunkwise
 * form of "Token Mixer I", section "Kimi Delta Attention" (WY representation, UT
 * transform, inter-chunk state update, chunk output), re-derived with exponent
 * differences so that no factor is divided by a small decay; the result equals the
 * token recurrence up to rounding and does not depend on the (internal) chunk size.
 *
 *   q, k          [B, H, T, dk], dtype dt
 *   v             [B, H, T, dv], dtype dt
 *   g             float32 log-decay per token (NOT cumulative), in [-5, 0]:
 *                 [B, H, T, dk] (KDA_GATE_PER_CHANNEL) or [B, H, T] (KDA_GATE_PER_HEAD)
 *   beta          float32 [B, H, T], in [0, 1]
 *   initial_state float32 [N, H, dk, dv] or NULL (= zero state)
 *   final_state   float32 [N, H, dk, dv] or NULL (= not written); may equal initial_state
 *   o             [B, H, T, dv], dtype dt; written for every token of every sequence
 *                 q, k, v, g and o (and the Gated Delta Rule-2 gates below) must be 16-byte
 *                 aligned, as every PyTorch allocation is (else KDA_ERR_INVALID_ARG).
 *   cu_seqlens    NULL: N = B sequences of length T (batch row b is sequence b).
 *                 Otherwise a DEVICE int32 array of num_seqs + 1 offsets into the T
 *                 axis (packed variable-length sequences); B must be 1 and N = num_seqs.
 *                 Tokens of o outside every sequence are left untouched.
 *   dk, dv        each 64 or 128 (anything else: KDA_ERR_UNSUPPORTED)
 *   workspace     device buffer of workspace_bytes bytes, owned by the caller and not read
 *                 before this call writes it (kda_chunk_fwd_workspace_size gives the
 *                 recommended size; the call plans within any size it is given); or
 *                 workspace_bytes = 0 (workspace ignored) to run one workgroup per chain
 *                 in chain order. With cu_seqlens, 0 < workspace_bytes < the work list's
 *                 4 * (1 + 2 * num_seqs * H) bytes rounded up to 256 (num_seqs <= 1024), or
 *                 a NULL workspace with workspace_bytes > 0: KDA_ERR_INVALID_ARG. Without
 *                 cu_seqlens the batch rows are the sequences (num_seqs must be 0 or B).
 *                 Calls that overlap on one workspace race.
 *
 * Arithmetic: state and accumulation in float32. With dt = KDA_BF16 the dense
 * contractions take bf16 operands on the matrix cores (float32 accumulate); with
 * dt = KDA_F32 every operation is float32. The matrix-core kernel serves dt = KDA_BF16
 * with dk = 128. It runs a chain as one item while the chain's per-channel decay, T * dk
 * float32 values, stays under 2^31 bytes (T < 2^22). Longer T axes run on the matrix cores
 * with dv = 128 and a workspace of at least the minimum below: the call then cuts every
 * sequence into segments of at most 2^21 tokens. The minimum is the plan words and three
 * fp32 dk x dk matrices per head for each of S slots, plus dk bf16 values per head for
 * every token of the T axis (N * T tokens without cu_seqlens), where, with
 * m = ceil(T / 2^21), S = 2 N + 2 m + 1 with cu_seqlens and 2 m N + 1 without (S <= 1024;
 * kda_chunk_fwd_workspace_size returns at least this). A smaller workspace, dv = 64,
 * dk = 64 and dt = KDA_F32 run on the fp32 matrix-core kernel (16x16x4 fp32 products, 64-bit
 * addressing, no length limit).
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, float* final_state,
                         void* o, const int32_t* cu_seqlens, int num_seqs, int B, int H,
                         int T, int dk, int dv, kda_dtype dt, kda_gate_mode gm,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Every other argument, layout, error and result is kda_chunk_fwd's. In place of the
 * workspace the call uses a file-scope device array of the library, 64 MiB on every device
 * the library runs on (held until the process ends), as the workspace kda_chunk_fwd would
 * recommend, capped at that size: problems whose segment plan needs more simply cut fewer
 * sequences. Packed calls whose work list (4 * (1 + 2 * num_seqs * H) bytes) exceeds the array
 * return KDA_ERR_UNSUPPORTED. Nothing in the array needs clearing between calls (every call
 * writes what it reads), but every call on one device shares that device's array: calls that
 * overlap on one device (other streams or host threads) race.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state,
                                 float* final_state, void* o, const int32_t* cu_seqlens,
                                 int num_seqs, int B, int H, int T, int dk, int dv,
                                 kda_dtype dt, kda_gate_mode gm, hipStream_t stream);

/*
 * One single-token decode step for N sequences x H heads on a resident state.
 * Per chain: S~ = Diag(exp g) S; p = S~^T k; S = S~ + beta k (v - p)^T; o = S^T q —
 * the decay-then-delta form of the page "KDA 与 Gated DeltaNet：线性注意力怎样读写有限状态",
 * section 2, and the fused recurrent path of its section 4.
 *
 *   q, k   [N, H, dk], dtype dt        v, o  [N, H, dv], dtype dt
 *   g      float32 [N, H, dk] (per channel) or [N, H] (per head), in [-5, 0]
 *   beta   float32 [N, H]
 *   state  float32 [N, H, dk, dv], read and overwritten IN PLACE with S_t
 *   dk, dv each 64 or 128
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, float* state, void* o, int N, int H, int dk,
                              int dv, kda_dtype dt, kda_gate_mode gm, hipStream_t stream);

/*
 * Gated Delta Rule-2 ("Token Mixer I", section "Gated DeltaNet-2: Decoupling Erase and
 * Write"): the scalar gate beta is replaced by a per-key-channel erase gate b_t and a
 * per-value-channel write gate w_t. Per chain, decay first, then
 *   S_t = S~ + k_t (w_t * v_t - S~^T (b_t * k_t))^T,  S~ = Diag(exp g_t) S_{t-1},
 *   o_t = S_t^T q_t            (* elementwise)
 * which is the residual z_t - S~^T e_t of the section's fast-weight view with
 * e_t = b_t * k_t and z_t = w_t * v_t. b = beta 1 and w = beta 1 give kda_chunk_fwd.
 *
 * kda_gdr2_chunk_fwd takes every argument of kda_chunk_fwd (same layouts, workspace,
 * errors and arithmetic), with beta replaced by
 *   erase  float32 [B, H, T, dk], in [0, 1]  (read side: which key channels are erased)
 *   write  float32 [B, H, T, dv], in [0, 1]  (write side: which value channels are written)
 * NULL erase or write: KDA_ERR_INVALID_ARG. The chunkwise form is the one of
 * kda_chunk_fwd with the erase-gated keys b * k on the read side (the prediction and the
 * strictly lower matrix of the UT transform) and w * v in place of beta v.
 */
kda_status kda_gdr2_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                              const float* erase, const float* write,
                              const float* initial_state, float* final_state, void* o,
                              const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                              int dk, int dv, kda_dtype dt, kda_gate_mode gm, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Gated Delta Rule-2 decode step: kda_recurrent_step with beta replaced by
 *   erase  float32 [N, H, dk], write  float32 [N, H, dv]
 * per chain: S~ = Diag(exp g) S; p = S~^T (b * k); S = S~ + k (w * v - p)^T; o = S^T q.
 * NULL erase or write: KDA_ERR_INVALID_ARG; everything else as kda_recurrent_step.
 */
kda_status kda_gdr2_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                                   const float* erase, const float* write, float* state,
                                   void* o, int N, int H, int dk, int dv, kda_dtype dt,
                                   kda_gate_mode gm, hipStream_t stream);

/*
 * Prologue: the steps that turn per-token pre-activations into the operator's inputs,
 * fused into one pass ("Token Mixer I", section "The Kimi Linear Model Architecture",
 * neural parameterization; the decay function of the page "阅读笔记: Kimi Delta
 * Attention", section 6). Per head h and token:
 *   q_out = q_in / sqrt(sum q_in^2 + 1e-6), k_out likewise      (L2Norm over dk)
 *   g_out = max(-exp(A_log[h]) * softplus(u + dt_bias[h, :]), -5)  (fp32 log-decay, the
 *           g of kda_chunk_fwd; -5 is KDA's lower bound g_min, page "【轻量化复刻大模型】
 *           线性注意力（Linear Attention）", section 3.1)
 *   beta_out = Sigmoid(beta_in)                                 (optional)
 *
 *   q_in, k_in, q_out, k_out  [B, H, T, dk], dtype dt; q_out / k_out may equal q_in / k_in
 *   u, g_out   float32 [B, H, T, dk] (may be the same buffer)
 *   A_log      float32 [H]        dt_bias  float32 [H, dk]
 *   beta_in, beta_out  float32 [B, H, T], both NULL or both set (may be the same buffer)
 *   dk         64 or 128 (else KDA_ERR_UNSUPPORTED)
 * Any other NULL array, or any [.., dk] array or dt_bias not 16-byte aligned:
 * KDA_ERR_INVALID_ARG. With cu_seqlens packing, pass B = 1 and the packed T. fp32
 * arithmetic throughout; bf16 outputs are rounded once.
 */
kda_status kda_prologue(const void* q_in, const void* k_in, const float* u, const float* A_log,
                        const float* dt_bias, const float* beta_in, void* q_out, void* k_out,
                        float* g_out, float* beta_out, int B, int H, int T, int dk,
                        kda_dtype dt, hipStream_t stream);

/*
 * Epilogue: the per-head RMSNorm and output gate applied to the operator's output before
 * the output projection (same section), fused into one pass. Per head and token:
 *   o_out = Sigmoid(z) * o_in / sqrt(mean(o_in^2) + eps) * weight     (over dv)
 *
 *   o_in, z, o_out  [B, H, T, dv], dtype dt; o_out may equal o_in
 *   weight          float32 [dv] (shared by the heads), or NULL for 1
 *   eps             finite, > 0 (else KDA_ERR_INVALID_ARG): an all-zero row of o_in
 *                   (a zero value or a token outside every packed sequence) maps to 0
 *   dv              64 or 128 (else KDA_ERR_UNSUPPORTED)
 * A NULL o_in, z or o_out, or any array not 16-byte aligned: KDA_ERR_INVALID_ARG.
 */
kda_status kda_epilogue(const void* o_in, const void* z, const float* weight, float eps,
                        void* o_out, int B, int H, int T, int dv, kda_dtype dt,
                        hipStream_t stream);

/*
 * Bytes of device workspace that kda_chunk_bwd needs for these shapes (0 when the call
 * would be rejected as unsupported): two bf16 state histories of dk * dv / 16 bytes per
 * token (one dk x dv matrix per pair of 16-token blocks: the states entering the pairs and
 * the state gradients at their ends), sequences padded to whole 64-token steps (each
 * rounded up to 256 bytes), at dk = 64 preceded by copies of the key-side arrays and states
 * padded to 128 channels (q, k, dq, dk bf16 and g, erase, dg, d erase float32 of
 * B * H * T rows; initial state, final-state gradient and initial-state gradient of N * H
 * chains), and for
 * packed sequences (num_seqs at most 1024) the work list of kda_chunk_fwd_workspace_size's
 * last case.
 */
size_t kda_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int num_seqs,
                                    kda_dtype dt);

/*
 * Backward pass of kda_chunk_fwd: the gradients of a scalar loss L with respect to every
 * input, given dL/do and dL/dS_T. The pages describe the forward only; these are its
 * derivatives (the chain rule through the chunkwise form of "Token Mixer I", section
 * "Kimi Delta Attention", recomputing the forward states; exact up to rounding).
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv, gm:
 *                    the forward's inputs, as in kda_chunk_fwd
 *   grad_o           [B, H, T, dv], dtype dt: dL/do
 *   grad_final_state float32 [N, H, dk, dv] or NULL (= 0): dL/dS_T
 *   grad_q, grad_k   [B, H, T, dk], dtype dt        grad_v  [B, H, T, dv], dtype dt
 *   grad_g           float32, shaped like g          grad_beta  float32 [B, H, T]
 *   grad_initial_state float32 [N, H, dk, dv], or NULL (not written)
 *   workspace        device buffer of at least kda_chunk_bwd_workspace_size(...) bytes,
 *                    owned by the caller (contents on entry ignored; calls that overlap
 *                    on one workspace race)
 * Gradients are written for every token of every sequence; tokens outside every
 * sequence are left untouched. Supported: dt = KDA_BF16, dk = 64 or 128, dv = 64 or 128,
 * either gate mode, and T with (T + 64) * 8 * dv < 2^31, so that one chain's history fits
 * a buffer descriptor (T <= 2,097,087 at dv = 128; anything else: KDA_ERR_UNSUPPORTED).
 * dk = 64 runs the dk = 128 kernels on copies padded with zero key channels (a zero key
 * channel never enters the state, so the other gradients are those of the dk = 64 problem).
 * A NULL required array, a workspace
 * smaller than the size above, or the forward's argument errors: KDA_ERR_INVALID_ARG.
 * Arithmetic: bf16 operands on the matrix cores with float32 accumulation and float32
 * state gradients; the stored forward states are bf16.
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, const void* grad_o,
                         const float* grad_final_state, void* grad_q, void* grad_k,
                         void* grad_v, float* grad_g, float* grad_beta,
                         float* grad_initial_state, const int32_t* cu_seqlens, int num_seqs,
                         int B, int H, int T, int dk, int dv, kda_dtype dt, kda_gate_mode gm,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of kda_gdr2_chunk_fwd: kda_chunk_bwd with beta replaced by the Gated Delta
 * Rule-2 gates erase float32 [B, H, T, dk] and write float32 [B, H, T, dv], whose gradients
 * grad_erase [B, H, T, dk] and grad_write [B, H, T, dv] (float32) replace grad_beta.
 * Workspace: kda_chunk_bwd_workspace_size. A NULL erase, write, grad_erase or grad_write:
 * KDA_ERR_INVALID_ARG; everything else as kda_chunk_bwd.
 */
kda_status kda_gdr2_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                              const float* erase, const float* write,
                              const float* initial_state, const void* grad_o,
                              const float* grad_final_state, void* grad_q, void* grad_k,
                              void* grad_v, float* grad_g, float* grad_erase,
                              float* grad_write, float* grad_initial_state,
                              const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                              int dk, int dv, kda_dtype dt, kda_gate_mode gm, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_string(kda_status s);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
