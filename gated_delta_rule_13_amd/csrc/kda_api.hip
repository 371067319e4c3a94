// C ABI of libkda.so (declared in include/kda.h): argument validation on the host,
// then dispatch to the kernels on the caller's stream. Nothing here allocates device memory
// or synchronises the host (except the KDA_DEBUG build's precondition checks, which wait for
// their result); the state kept between calls is the per-device compute-unit count below,
// the no-allocation entry point's static scratch array and the backward's per-device second
// stream (kda_chunk_bwd.hip).
#include <cstdint>
#include <cstring>

#include <algorithm>
#include <atomic>
#include <mutex>

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
    case KDA_ERR_PRECONDITION:
      return "KDA_ERR_PRECONDITION: an input value is outside the documented range";
  }
  return "KDA_ERR_UNKNOWN: unknown status code";
}

// Compute units of the current device, cached per device (sizes the chunk schedule). The
// cache entries are atomics: concurrent first calls may both query the device, and both
// store the same value.
static int device_compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// KDA_DEBUG builds: the value preconditions of an operator call, checked on the device
// before its work (the work is not launched when one fails).
#if KDA_DEBUG
static int debug_preconditions(const float* g, bool per_channel, const float* beta,
                               const float* erase, const float* write,
                               const int32_t* cu_seqlens, int num_seqs, long long rows, int T,
                               int dk, int dv, hipStream_t stream) {
  kda::DebugCheck c;
  c.add(g, per_channel ? rows * dk : rows, -5.f, 0.f, kda::DebugCheck::kG);
  if (erase) {
    c.add(erase, rows * dk, 0.f, 1.f, kda::DebugCheck::kErase);
    c.add(write, rows * dv, 0.f, 1.f, kda::DebugCheck::kWrite);
  } else {
    c.add(beta, rows, 0.f, 1.f, kda::DebugCheck::kBeta);
  }
  if (cu_seqlens) {
    c.cu = cu_seqlens;
    c.N = num_seqs;
    c.T = T;
  }
  unsigned flags = 0;
  if (kda::debug_check(c, stream, flags) != hipSuccess) return KDA_ERR_HIP;
  return flags ? KDA_ERR_PRECONDITION : KDA_OK;
}
#endif

// The workspace the forward recommends. A call is packed when it passes cu_seqlens (then B = 1
// and num_seqs sequences); the size query takes num_seqs > 0 for such a call.
static size_t chunk_fwd_workspace(int B, int H, int T, int dk, int dv, int num_seqs, int dt) {
  // only the matrix-core path uses a workspace: its schedule (every intermediate of the
  // method stays on chip) and, for the segment plan, the segments' states
  if (B <= 0 || H <= 0 || T <= 0 || num_seqs < 0) return 0;
  if (dt != KDA_BF16 || !kda::chunk_mfma_dims(dk, dv)) return 0;
  const bool packed = num_seqs > 0;
  if (packed && B != 1) return 0;  // no such call is accepted
  const long long N = packed ? num_seqs : B;
  if (N * H > (1ll << 24)) return 0;
  const int cus = device_compute_units();
  // chains too long for whole-chain items: only the segment plan (dv = dk) runs them on the
  // matrix cores; without it the call takes the fp32 path, which needs no workspace
  if (!kda::chunk_mfma_supports(dk, dv, T))
    return dv == dk ? kda::chunk_segplan_bytes((int)N, H, T, dv, packed, cus) : 0;
  // dv = dk: the segment plan (packed sequences, or fewer equal-length chains than compute
  // units); its plan words also hold the work list that it falls back to
  if (dv == dk && (packed || N * H < cus)) {
    const size_t sp = kda::chunk_segplan_bytes((int)N, H, T, dv, packed, cus);
    if (sp > 0) return sp;
  }
  // few chains for the device: segments and their states (this also covers the work list)
  const size_t seg = kda::chunk_seg_bytes((int)N, H, T, dv, cus);
  if (seg > 0) return seg;
  // equal-length batches are scheduled on the host: only packed sequences need a work list
  if (!packed) return 0;
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
  // the kernels move token rows as 16-byte vectors
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
      (erase && (!aligned16(erase) || !aligned16(write))))
    return KDA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (gm != KDA_GATE_PER_CHANNEL && gm != KDA_GATE_PER_HEAD) return KDA_ERR_INVALID_ARG;
  if (cu_seqlens && (B != 1 || num_seqs <= 0)) return KDA_ERR_INVALID_ARG;
  if (!cu_seqlens && num_seqs != 0 && num_seqs != B) return KDA_ERR_INVALID_ARG;
  // packed exactly when cu_seqlens is given (num_seqs = B without it is B sequences of T)
  const bool packed = cu_seqlens != nullptr;
  const long long N = packed ? num_seqs : B;
  const bool dims = dt == KDA_BF16 && kda::chunk_mfma_dims(dk, dv);
  const bool whole = dims && kda::chunk_mfma_supports(dk, dv, T);
  // chains too long for whole-chain items run on the matrix cores only as a segment plan,
  // which needs its matrices and carried-back queries in the workspace; else the fp32 path
  const size_t long_min = dims && !whole && N <= (1ll << 24)
                              ? kda::chunk_segplan_min_bytes((int)N, H, T, dv, packed)
                              : 0;
  const bool seg_long = long_min > 0 && workspace && workspace_bytes >= long_min;
  const bool mfma = whole || seg_long;
  // workspace_bytes == 0: run without a schedule. Otherwise packed sequences need at least
  // their work list; every larger buffer is planned within (each path below checks that its
  // own layout fits).
  const size_t work_list = mfma && packed ? kda::chunk_plan_bytes((int)N, H, dv) : 0;
  if (workspace_bytes > 0 && (!workspace || workspace_bytes < work_list))
    return KDA_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
  if (N * H > (1ll << 24) || (long long)B * H * T > (1ll << 40)) return KDA_ERR_UNSUPPORTED;

#if KDA_DEBUG
  if (const int pre = debug_preconditions(g, gm == KDA_GATE_PER_CHANNEL, beta, erase, write,
                                          cu_seqlens, num_seqs, (long long)B * H * T, T, dk,
                                          dv, stream))
    return static_cast<kda_status>(pre);
#endif
  kda::ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.erase = erase; a.write = write;
  a.s0 = initial_state; a.sT = final_state; a.o = o; a.cu = cu_seqlens;
  a.N = (int)N; a.H = H; a.T = T; a.dk = dk; a.dv = dv;
  a.plan = nullptr;
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
  if (mfma) {
    const size_t sp_min = kda::chunk_segplan_min_bytes(a.N, H, T, dv, packed);
    const size_t seg = kda::chunk_seg_bytes(a.N, H, T, dv, a.cus);
    if (seg_long || (workspace_bytes > 0 && (packed || N * H < a.cus) && sp_min > 0 &&
                     workspace_bytes >= sp_min)) {
      err = kda::launch_chunk_mfma_segplan(a, per_channel, workspace, workspace_bytes, stream);
    } else if (workspace_bytes > 0 && (!erase || dv != dk) && seg > 0 && workspace_bytes >= seg) {
      err = kda::launch_chunk_mfma_segmented(a, per_channel, workspace, stream);
    } else {
      // the work list of packed sequences when it fits (chunk_plan_bytes is 0 past the
      // sequences one planning workgroup sorts), else one workgroup per chain
      if (packed && work_list > 0 && workspace_bytes >= work_list)
        a.plan = static_cast<uint32_t*>(workspace);
      err = kda::launch_chunk_mfma(a, per_channel, stream);
    }
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
#if KDA_DEBUG
  if (const int pre = debug_preconditions(g, gm == KDA_GATE_PER_CHANNEL, beta, erase, write,
                                          nullptr, 0, (long long)N * H, 1, dk, dv, stream))
    return static_cast<kda_status>(pre);
#endif
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

// Scratch memory of kda_chunk_fwd_noalloc: a file-scope device array, so that the call never
// allocates. In host code the array's name is only a host-side stand-in; its device address
// is looked up once per device (hipGetSymbolAddress, with that device current) and only that
// address is handed to kernels. Every call on a device shares its array.
static constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state,
                                 float* final_state, void* o, const int32_t* cu_seqlens,
                                 int num_seqs, int B, int H, int T, int dk, int dv,
                                 kda_dtype dt, kda_gate_mode gm, hipStream_t stream) {
  if (!beta) return KDA_ERR_INVALID_ARG;
  const int dtype = enum_value(&dt);
  if (B <= 0 || H <= 0 || T <= 0 || num_seqs < 0) return KDA_ERR_INVALID_ARG;
  if (cu_seqlens && (B != 1 || num_seqs <= 0)) return KDA_ERR_INVALID_ARG;
  // the workspace kda_chunk_fwd would recommend, within the scratch array; packed sequences
  // need at least their work list, which must fit
  const long long N = cu_seqlens ? num_seqs : B;
  const bool mfma = dtype == KDA_BF16 && kda::chunk_mfma_supports(dk, dv, T);
  const size_t work_list = mfma && cu_seqlens ? kda::chunk_plan_bytes((int)N, H, dv) : 0;
  if (work_list > kNoAllocScratchBytes) return KDA_ERR_UNSUPPORTED;
  size_t bytes = chunk_fwd_workspace(B, H, T, dk, dv, cu_seqlens ? num_seqs : 0, dtype);
  bytes = std::min(bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (bytes > 0 && noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
  return chunk_fwd_impl(q, k, v, g, beta, nullptr, nullptr, initial_state, final_state, o,
                        cu_seqlens, num_seqs, B, H, T, dk, dv, dtype, enum_value(&gm),
                        bytes > 0 ? ws : nullptr, bytes, stream);
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

// dk = 64 runs the dk = 128 kernels on copies of the key-side arrays padded with zero
// channels (q, k; g with g = 0, the identity decay, per channel; the erase gates), the states
// padded with zero rows: a zero key channel never enters the state and a zero query channel
// reads nothing, so every other gradient is that of the dk = 64 problem, and the padded
// channels' gradients are dropped. The copies sit at the front of the workspace.
struct Pad64 {
  size_t q, k, g, e, s0, dsT, dq, dk, dg, de, ds0, inner;
};
static Pad64 pad64_layout(int B, int H, int T, int dv, int N) {
  const size_t rows = (size_t)B * H * T, nh = (size_t)N * H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  Pad64 L;
  L.q = take(rows * 128 * 2);
  L.k = take(rows * 128 * 2);
  L.g = take(rows * 128 * 4);
  L.e = take(rows * 128 * 4);
  L.s0 = take(nh * 128 * dv * 4);
  L.dsT = take(nh * 128 * dv * 4);
  L.dq = take(rows * 128 * 2);
  L.dk = take(rows * 128 * 2);
  L.dg = take(rows * 128 * 4);
  L.de = take(rows * 128 * 4);
  L.ds0 = take(nh * 128 * dv * 4);
  L.inner = off;
  return L;
}

static size_t chunk_bwd_workspace(int B, int H, int T, int dk, int dv, int num_seqs, int dt) {
  if (B <= 0 || H <= 0 || T <= 0 || num_seqs < 0 || dt != KDA_BF16) return 0;
  if (dk == 64) {
    const size_t inner = chunk_bwd_workspace(B, H, T, 128, dv, num_seqs, dt);
    return inner ? pad64_layout(B, H, T, dv, num_seqs > 0 ? num_seqs : B).inner + inner : 0;
  }
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
  if (dt != KDA_BF16 || !kda::chunk_bwd_supports(dk == 64 ? 128 : dk, dv, T))
    return KDA_ERR_UNSUPPORTED;
  const long long N = cu_seqlens ? num_seqs : B;
  if (N * H > (1ll << 24) || (long long)B * H * T > (1ll << 40)) return KDA_ERR_UNSUPPORTED;
  const size_t need =
      chunk_bwd_workspace(B, H, T, dk, dv, cu_seqlens ? num_seqs : 0, dt);
  if (!workspace || workspace_bytes < need) return KDA_ERR_INVALID_ARG;
  if (dk == 64) {
    const Pad64 L = pad64_layout(B, H, T, dv, (int)N);
    char* w = static_cast<char*>(workspace);
    const long long rows = (long long)B * H * T, nh = N * H;
    const bool per_channel = gm == KDA_GATE_PER_CHANNEL;
    hipError_t e = hipSuccess;
    auto pad = [&](const void* src, size_t off, long long n, int ws, int wd, int eb) {
      if (e == hipSuccess) e = kda::launch_pad_rows(src, w + off, n, ws, wd, eb, stream);
    };
    auto unpad = [&](size_t off, void* dst, long long n, int ws, int wd, int eb) {
      if (e == hipSuccess) e = kda::launch_pad_rows(w + off, dst, n, ws, wd, eb, stream);
    };
    pad(q, L.q, rows, 64, 128, 2);
    pad(k, L.k, rows, 64, 128, 2);
    if (per_channel) pad(g, L.g, rows, 64, 128, 4);
    if (erase) pad(erase, L.e, rows, 64, 128, 4);
    if (initial_state) pad(initial_state, L.s0, nh, 64 * dv, 128 * dv, 4);
    if (grad_final_state) pad(grad_final_state, L.dsT, nh, 64 * dv, 128 * dv, 4);
    // the outputs start as the caller's arrays, so that tokens outside every sequence keep
    // their values through the copies back
    pad(grad_q, L.dq, rows, 64, 128, 2);
    pad(grad_k, L.dk, rows, 64, 128, 2);
    if (per_channel) pad(grad_g, L.dg, rows, 64, 128, 4);
    if (erase) pad(grad_erase, L.de, rows, 64, 128, 4);
    if (e != hipSuccess) return KDA_ERR_HIP;
    auto at = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
    const kda_status st = chunk_bwd_impl(
        w + L.q, w + L.k, v, per_channel ? at(L.g) : g, beta, erase ? at(L.e) : nullptr, write,
        initial_state ? at(L.s0) : nullptr, grad_o, grad_final_state ? at(L.dsT) : nullptr,
        w + L.dq, w + L.dk, grad_v, per_channel ? at(L.dg) : grad_g, grad_beta,
        erase ? at(L.de) : nullptr, grad_write, grad_initial_state ? at(L.ds0) : nullptr,
        cu_seqlens, num_seqs, B, H, T, 128, dv, dt, gm, w + L.inner, workspace_bytes - L.inner,
        stream);
    if (st != KDA_OK) return st;
    unpad(L.dq, grad_q, rows, 128, 64, 2);
    unpad(L.dk, grad_k, rows, 128, 64, 2);
    if (per_channel) unpad(L.dg, grad_g, rows, 128, 64, 4);
    if (erase) unpad(L.de, grad_erase, rows, 128, 64, 4);
    if (grad_initial_state) unpad(L.ds0, grad_initial_state, nh, 128 * dv, 64 * dv, 4);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }

#if KDA_DEBUG
  if (const int pre = debug_preconditions(g, gm == KDA_GATE_PER_CHANNEL, beta, erase, write,
                                          cu_seqlens, num_seqs, (long long)B * H * T, T, dk,
                                          dv, stream))
    return static_cast<kda_status>(pre);
#endif
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
  // eps > 0 keeps an all-zero row finite (0 / sqrt(eps) = 0); also rejects NaN and inf
  if (!(eps > 0.f) || !(eps < 1e30f)) return KDA_ERR_INVALID_ARG;
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
