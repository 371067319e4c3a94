// C ABI of libkda.so (declared in include/kda.h): argument validation on the host,
// then dispatch to the kernels on the caller's stream. Nothing here allocates,
// synchronises or keeps state between calls.
#include <cstdint>
#include <cstring>

#include <algorithm>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool supported_dim(int d) { return d == 64 || d == 128; }

// Enum arguments arrive from C, where any int is a valid value; a C++ enum without a fixed
// underlying type holds only the values of its enumerators' bit width, so every entry point
// reads its enum arguments as plain ints (a byte copy from the argument's address: no
// enum-typed load or copy) and the code below compares ints.
template <typename E>
int enum_value(const E* e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, e, sizeof v);
  return v;
}

// The row-streaming kernels access eight channels at a time (16 bytes in bf16).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (enum_value(&s)) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported shape or mode";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error";
  }
  return "KDA_ERR_UNKNOWN: unknown status code";
}

// Compute units of the current device, cached per device (sizes the chunk schedule).
static int device_compute_units() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

static size_t chunk_fwd_workspace(int B, int H, int T, int dk, int dv, int num_seqs, int dt) {
  // only the matrix-core path uses a workspace: its work list (every intermediate of the
  // method stays on chip)
  if (B <= 0 || H <= 0 || T <= 0 || num_seqs < 0) return 0;
  if (dt != KDA_BF16 || !kda::chunk_mfma_supports(dk, dv, T)) return 0;
  const long long N = num_seqs > 0 ? num_seqs : B;
  if (N * H > (1ll << 24)) return 0;
  const int cus = device_compute_units();
  // dv = dk: the segment plan (packed sequences, or fewer equal-length chains than compute
  // units); it also holds the work list that the Gated Delta Rule-2 gates use
  if (dv == dk && (num_seqs > 0 || N * H < cus)) {
    const size_t sp = kda::chunk_segplan_bytes((int)N, H, T, dv, num_seqs > 0);
    if (sp > 0) return std::max(sp, num_seqs > 0 ? kda::chunk_plan_bytes(num_seqs, H, dv) : 0);
  }
  // few chains for the device: segments and their states (this also covers the work list)
  const size_t seg = kda::chunk_seg_bytes((int)N, H, T, dv, cus);
  if (seg > 0) return seg;
  // equal-length batches are scheduled on the host: only packed sequences need a work list
  if (num_seqs == 0) return 0;
  return kda::chunk_plan_bytes(num_seqs, H, dv);
}

size_t kda_chunk_fwd_workspace_size(int B, int H, int T, int dk, int dv, int num_seqs,
                                    kda_dtype dt) {
  return chunk_fwd_workspace(B, H, T, dk, dv, num_seqs, enum_value(&dt));
}

// The two forward paths differ only in their gates: beta (KDA, Gated DeltaNet) or the
// erase / write vectors of Gated Delta Rule-2 (erase != nullptr).
static kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* erase, const float* write,
                                 const float* initial_state, float* final_state, void* o,
                                 const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                                 int dk, int dv, int dt, int gm, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !g || !o) return KDA_ERR_INVALID_ARG;
  if (erase ? !write : !beta) return KDA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (gm != KDA_GATE_PER_CHANNEL && gm != KDA_GATE_PER_HEAD) return KDA_ERR_INVALID_ARG;
  if (cu_seqlens && (B != 1 || num_seqs <= 0)) return KDA_ERR_INVALID_ARG;
  if (!cu_seqlens && num_seqs != 0 && num_seqs != B) return KDA_ERR_INVALID_ARG;
  const size_t need = chunk_fwd_workspace(B, H, T, dk, dv, num_seqs, dt);
  // workspace_bytes == 0: run without the schedule; otherwise it must hold the schedule
  if (workspace_bytes > 0 && (workspace_bytes < need || !workspace)) return KDA_ERR_INVALID_ARG;
  const bool scheduled = need > 0 && workspace_bytes > 0;
  if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
  const long long N = cu_seqlens ? num_seqs : B;
  if (N * H > (1ll << 24) || (long long)B * H * T > (1ll << 40)) return KDA_ERR_UNSUPPORTED;

  kda::ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.erase = erase; a.write = write;
  a.s0 = initial_state; a.sT = final_state; a.o = o; a.cu = cu_seqlens;
  a.N = (int)N; a.H = H; a.T = T; a.dk = dk; a.dv = dv;
  a.plan = scheduled ? static_cast<uint32_t*>(workspace) : nullptr;
  a.cus = device_compute_units();
  a.split_all = 0;
  a.hist = nullptr;
  a.seg_len = 0;
  a.nseg = 1;
  a.seg_slots = 0;
  a.seg_mats = nullptr;
  a.qt = nullptr;
  const bool per_channel = gm == KDA_GATE_PER_CHANNEL;
  hipError_t err;
  if (dt == KDA_BF16 && kda::chunk_mfma_supports(dk, dv, T)) {
    const size_t sp = kda::chunk_segplan_bytes(a.N, H, T, dv, cu_seqlens != nullptr);
    if (scheduled && sp > 0 && workspace_bytes >= sp)
      err = kda::launch_chunk_mfma_segplan(a, per_channel, workspace, stream);
    else if (scheduled && !erase && kda::chunk_seg_bytes(a.N, H, T, dv, a.cus) > 0)
      err = kda::launch_chunk_mfma_segmented(a, per_channel, workspace, stream);
    else
      err = kda::launch_chunk_mfma(a, per_channel, stream);
  } else
    err = kda::launch_chunk_f32(a, dt == KDA_BF16, per_channel, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static kda_status recurrent_step_impl(const void* q, const void* k, const void* v,
                                      const float* g, const float* beta, const float* erase,
                                      const float* write, float* state, void* o, int N, int H,
                                      int dk, int dv, int dt, int gm, hipStream_t stream) {
  if (!q || !k || !v || !g || !state || !o) return KDA_ERR_INVALID_ARG;
  if (erase ? !write : !beta) return KDA_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (gm != KDA_GATE_PER_CHANNEL && gm != KDA_GATE_PER_HEAD) return KDA_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
  if ((long long)N * H > 0x7fffffffll) return KDA_ERR_UNSUPPORTED;
  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.erase = erase; a.write = write;
  a.state = state; a.o = o;
  a.N = N; a.H = H;
  const hipError_t err =
      kda::launch_decode(a, dk, dv, dt == KDA_BF16, gm == KDA_GATE_PER_CHANNEL, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, float* final_state,
                         void* o, const int32_t* cu_seqlens, int num_seqs, int B, int H,
                         int T, int dk, int dv, kda_dtype dt, kda_gate_mode gm,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!beta) return KDA_ERR_INVALID_ARG;
  return chunk_fwd_impl(q, k, v, g, beta, nullptr, nullptr, initial_state, final_state, o,
                        cu_seqlens, num_seqs, B, H, T, dk, dv, enum_value(&dt), enum_value(&gm),
                        workspace, workspace_bytes, stream);
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, float* state, void* o, int N, int H, int dk,
                              int dv, kda_dtype dt, kda_gate_mode gm, hipStream_t stream) {
  if (!beta) return KDA_ERR_INVALID_ARG;
  return recurrent_step_impl(q, k, v, g, beta, nullptr, nullptr, state, o, N, H, dk, dv,
                             enum_value(&dt), enum_value(&gm), stream);
}

kda_status kda_gdr2_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                              const float* erase, const float* write,
                              const float* initial_state, float* final_state, void* o,
                              const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                              int dk, int dv, kda_dtype dt, kda_gate_mode gm, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (!erase || !write) return KDA_ERR_INVALID_ARG;
  return chunk_fwd_impl(q, k, v, g, nullptr, erase, write, initial_state, final_state, o,
                        cu_seqlens, num_seqs, B, H, T, dk, dv, enum_value(&dt), enum_value(&gm),
                        workspace, workspace_bytes, stream);
}

kda_status kda_gdr2_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                                   const float* erase, const float* write, float* state,
                                   void* o, int N, int H, int dk, int dv, kda_dtype dt,
                                   kda_gate_mode gm, hipStream_t stream) {
  if (!erase || !write) return KDA_ERR_INVALID_ARG;
  return recurrent_step_impl(q, k, v, g, nullptr, erase, write, state, o, N, H, dk, dv,
                             enum_value(&dt), enum_value(&gm), stream);
}

static size_t chunk_bwd_workspace(int B, int H, int T, int dk, int dv, int num_seqs, int dt) {
  if (B <= 0 || H <= 0 || T <= 0 || num_seqs < 0 || dt != KDA_BF16) return 0;
  if (!kda::chunk_bwd_supports(dk, dv, T)) return 0;
  const int N = num_seqs > 0 ? num_seqs : B;
  const size_t one = kda::chunk_bwd_hist_bytes(N, H, T, dv, num_seqs > 0);
  // the two histories, then the work list of packed sequences
  const size_t plan = num_seqs > 0 ? kda::chunk_plan_bytes(num_seqs, H, dv) : 0;
  return 2 * ((one + 255) / 256 * 256) + plan;
}

size_t kda_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int num_seqs,
                                    kda_dtype dt) {
  return chunk_bwd_workspace(B, H, T, dk, dv, num_seqs, enum_value(&dt));
}

// The two backward paths differ only in their gates: beta (KDA, Gated DeltaNet) or the
// erase / write vectors of Gated Delta Rule-2 (erase != nullptr).
static kda_status chunk_bwd_impl(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* erase, const float* write,
                                 const float* initial_state, const void* grad_o,
                                 const float* grad_final_state, void* grad_q, void* grad_k,
                                 void* grad_v, float* grad_g, float* grad_beta,
                                 float* grad_erase, float* grad_write,
                                 float* grad_initial_state, const int32_t* cu_seqlens,
                                 int num_seqs, int B, int H, int T, int dk, int dv, int dt,
                                 int gm, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (!q || !k || !v || !g || !grad_o) return KDA_ERR_INVALID_ARG;
  if (erase ? (!write || !grad_erase || !grad_write) : (!beta || !grad_beta))
    return KDA_ERR_INVALID_ARG;
  if (!grad_q || !grad_k || !grad_v || !grad_g) return KDA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (gm != KDA_GATE_PER_CHANNEL && gm != KDA_GATE_PER_HEAD) return KDA_ERR_INVALID_ARG;
  if (cu_seqlens && (B != 1 || num_seqs <= 0)) return KDA_ERR_INVALID_ARG;
  if (!cu_seqlens && num_seqs != 0 && num_seqs != B) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_BF16 || !kda::chunk_bwd_supports(dk, dv, T)) return KDA_ERR_UNSUPPORTED;
  const long long N = cu_seqlens ? num_seqs : B;
  if (N * H > (1ll << 24) || (long long)B * H * T > (1ll << 40)) return KDA_ERR_UNSUPPORTED;
  const size_t need =
      chunk_bwd_workspace(B, H, T, dk, dv, cu_seqlens ? num_seqs : 0, dt);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID_ARG;

  kda::BwdArgs b;
  kda::ChunkArgs& a = b.f;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.erase = erase; a.write = write;
  a.s0 = initial_state; a.sT = nullptr; a.o = nullptr; a.cu = cu_seqlens;
  a.N = (int)N; a.H = H; a.T = T; a.dk = dk; a.dv = dv;
  a.plan = nullptr; a.cus = device_compute_units(); a.split_all = 0; a.hist = nullptr;
  a.seg_len = 0; a.nseg = 1;
  a.seg_slots = 0; a.seg_mats = nullptr; a.qt = nullptr;
  b.dout = grad_o; b.dsT = grad_final_state;
  b.dq = grad_q; b.dk = grad_k; b.dv = grad_v; b.dg = grad_g; b.dbeta = grad_beta;
  b.derase = grad_erase; b.dwrite = grad_write;
  b.ds0 = grad_initial_state;
  const size_t one = (kda::chunk_bwd_hist_bytes((int)N, H, T, dv, cu_seqlens != nullptr) + 255) /
                    256 * 256;
  b.hist_s = workspace;
  b.hist_ds = static_cast<char*>(workspace) + one;
  b.plan = need > 2 * one ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + 2 * one)
                          : nullptr;
  const hipError_t err = kda::launch_chunk_bwd(b, gm == KDA_GATE_PER_CHANNEL, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, const void* grad_o,
                         const float* grad_final_state, void* grad_q, void* grad_k,
                         void* grad_v, float* grad_g, float* grad_beta,
                         float* grad_initial_state, const int32_t* cu_seqlens, int num_seqs,
                         int B, int H, int T, int dk, int dv, kda_dtype dt, kda_gate_mode gm,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!beta) return KDA_ERR_INVALID_ARG;
  return chunk_bwd_impl(q, k, v, g, beta, nullptr, nullptr, initial_state, grad_o,
                        grad_final_state, grad_q, grad_k, grad_v, grad_g, grad_beta, nullptr,
                        nullptr, grad_initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv,
                        enum_value(&dt), enum_value(&gm), workspace, workspace_bytes, stream);
}

kda_status kda_gdr2_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                              const float* erase, const float* write,
                              const float* initial_state, const void* grad_o,
                              const float* grad_final_state, void* grad_q, void* grad_k,
                              void* grad_v, float* grad_g, float* grad_erase,
                              float* grad_write, float* grad_initial_state,
                              const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                              int dk, int dv, kda_dtype dt, kda_gate_mode gm, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (!erase || !write) return KDA_ERR_INVALID_ARG;
  return chunk_bwd_impl(q, k, v, g, nullptr, erase, write, initial_state, grad_o,
                        grad_final_state, grad_q, grad_k, grad_v, grad_g, nullptr, grad_erase,
                        grad_write, grad_initial_state, cu_seqlens, num_seqs, B, H, T, dk, dv,
                        enum_value(&dt), enum_value(&gm), workspace, workspace_bytes, stream);
}

kda_status kda_prologue(const void* q_in, const void* k_in, const float* u, const float* A_log,
                        const float* dt_bias, const float* beta_in, void* q_out, void* k_out,
                        float* g_out, float* beta_out, int B, int H, int T, int dk,
                        kda_dtype dt, hipStream_t stream) {
  if (!q_in || !k_in || !u || !A_log || !dt_bias || !q_out || !k_out || !g_out)
    return KDA_ERR_INVALID_ARG;
  if (!beta_in != !beta_out) return KDA_ERR_INVALID_ARG;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(u) || !aligned16(dt_bias) ||
      !aligned16(q_out) || !aligned16(k_out) || !aligned16(g_out))
    return KDA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0) return KDA_ERR_INVALID_ARG;
  const int dtype = enum_value(&dt);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (!supported_dim(dk)) return KDA_ERR_UNSUPPORTED;
  if ((long long)B * H * T > (1ll << 40)) return KDA_ERR_UNSUPPORTED;
  kda::PrologueArgs a;
  a.q_in = q_in; a.k_in = k_in; a.u = u; a.A_log = A_log; a.dt_bias = dt_bias;
  a.beta_in = beta_in; a.q_out = q_out; a.k_out = k_out; a.g_out = g_out; a.beta_out = beta_out;
  a.B = B; a.H = H; a.T = T;
  const hipError_t err = kda::launch_prologue(a, dk, dtype == KDA_BF16, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_epilogue(const void* o_in, const void* z, const float* weight, float eps,
                        void* o_out, int B, int H, int T, int dv, kda_dtype dt,
                        hipStream_t stream) {
  if (!o_in || !z || !o_out) return KDA_ERR_INVALID_ARG;
  if (!aligned16(o_in) || !aligned16(z) || !aligned16(o_out) || !aligned16(weight))
    return KDA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !(eps < 1e30f)) return KDA_ERR_INVALID_ARG;  // also rejects NaN
  if (B <= 0 || H <= 0 || T <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
  const int dtype = enum_value(&dt);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (!supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
  if ((long long)B * H * T > (1ll << 40)) return KDA_ERR_UNSUPPORTED;
  kda::EpilogueArgs a;
  a.o_in = o_in; a.z = z; a.weight = weight; a.eps = eps; a.o_out = o_out;
  a.B = B; a.H = H; a.T = T;
  const hipError_t err = kda::launch_epilogue(a, dv, dtype == KDA_BF16, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
