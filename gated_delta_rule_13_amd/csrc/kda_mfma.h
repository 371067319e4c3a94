// Device helpers shared by the matrix-core kernels (the chunked forward and the backward
// pass): operand types, matrix-core products, bf16 packing, bounded buffer accesses,
// the LDS fences and barriers, and the per-lane loads of one 16-token block.
//
// Matrix-core operand layouts (lane l, r = l % 16, p = l / 16):
//   16x16x32 bf16: A[r][8p + i], B[8p + i][r] (i < 8); D[4p + e][r] (e < 4)
//   16x16x16 bf16: A[r][4p + i], B[4p + i][r] (i < 4); D[4p + e][r]
//   16x16x4  fp32: A[r][p], B[p][r]; D[4p + e][r]
// The D layout of one product is the B layout of a 16x16x16 product.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kDK = 128;  // key head size of the matrix-core kernels

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes are done
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits for this wavefront's LDS operations, not for its global
// loads (prefetches stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Round to bf16 pairwise (one v_cvt_pk_bf16_f32 per pair; converting the 4-vector
// directly is split into single-element conversions by the compiler).
__device__ __forceinline__ unsigned pack2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ bf16x4 pack4(f32x4 v) {
  return __builtin_bit_cast(bf16x4, (u32x2){pack2(v[0], v[1]), pack2(v[2], v[3])});
}
__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  return pack4(f32x4{a, b, c, d});
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = a[i];
    r[4 + i] = b[i];
  }
  return r;
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

// Raw buffer descriptor over `bytes` bytes from p (stride 0: offsets are byte offsets and
// an access at or past `bytes` reads zero / writes nothing).
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x4 ld_b64(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 ld_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float ld_b32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ bf16 ld_b16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
__device__ __forceinline__ void st_b128(rsrc_t r, uint32_t off, bf16x8 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, x), r, off, 0, 0);
}
__device__ __forceinline__ void st_b64(rsrc_t r, uint32_t off, bf16x4 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, x), r, off, 0, 0);
}

// x from lane 4 (lane / 4) + E of this lane's quad (DPP quad permutation, no LDS access).
template <int E>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), E * 0x55, 0xf, 0xf, true));
}

// Raw inputs of one 16-token block held by one prep lane: 8 tokens (half hf = lane / 32)
// x 4 channels (4 * (lane % 32) + j); beta of token lane for lanes < 16.
struct BlockRegs {
  bf16x4 q[8];
  bf16x4 k[8];
  f32x4 g[8];
  f32x4 b[8];  // erase gate (Gated Delta Rule-2 only)
  float beta;
};

// Bounded views of one chain's inputs, and this prep lane's byte offsets within a chunk.
struct PrepSrc {
  rsrc_t q, k, g, beta, erase;
  uint32_t qk_off, g_off, b_off, e_off;
};

template <bool PER_CHANNEL, bool GDR2>
__device__ __forceinline__ PrepSrc prep_src(const ChunkArgs& a, size_t row0, int len, int I,
                                            int lane) {
  const int cq = lane & 31, hf = lane >> 5;
  PrepSrc s;
  s.q = make_rsrc(static_cast<const bf16*>(a.q) + row0 * kDK, (uint32_t)len * kDK * 2);
  s.k = make_rsrc(static_cast<const bf16*>(a.k) + row0 * kDK, (uint32_t)len * kDK * 2);
  s.g = PER_CHANNEL ? make_rsrc(a.g + row0 * kDK, (uint32_t)len * kDK * 4)
                    : make_rsrc(a.g + row0, (uint32_t)len * 4);
  s.beta = make_rsrc(a.beta + row0, (uint32_t)len * 4);
  s.qk_off = ((16 * I + 8 * hf) * kDK + 4 * cq) * 2;
  s.g_off = PER_CHANNEL ? ((16 * I + 8 * hf) * kDK + 4 * cq) * 4 : (16 * I + 8 * hf) * 4;
  s.b_off = (16 * I + (lane & 15)) * 4;
  if (GDR2) {
    s.erase = make_rsrc(a.erase + row0 * kDK, (uint32_t)len * kDK * 4);
    s.e_off = ((16 * I + 8 * hf) * kDK + 4 * cq) * 4;
  }
  return s;
}

// Loads block I of the 64 tokens starting at c0 (rows past the chain read as zero); the
// queries only when NEEDQ (a pass that writes no outputs does not read them).
template <bool PER_CHANNEL, bool GDR2, bool NEEDQ = true>
__device__ __forceinline__ void load_block(BlockRegs& r, const PrepSrc& s, int c0) {
  const uint32_t qk = s.qk_off + (uint32_t)c0 * kDK * 2;
  const uint32_t go = s.g_off + (uint32_t)c0 * (PER_CHANNEL ? kDK * 4 : 4);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (NEEDQ) r.q[u] = ld_b64(s.q, qk + u * kDK * 2);
    r.k[u] = ld_b64(s.k, qk + u * kDK * 2);
    if (PER_CHANNEL) {
      r.g[u] = ld_b128(s.g, go + u * kDK * 4);
    } else {
      const float gg = ld_b32(s.g, go + u * 4);
      r.g[u] = f32x4{gg, gg, gg, gg};
    }
    if (GDR2) r.b[u] = ld_b128(s.erase, s.e_off + (uint32_t)c0 * kDK * 4 + u * kDK * 4);
  }
  // Gated Delta Rule-2 has no scalar gate: its erase gate sits in the key operand
  r.beta = GDR2 ? 1.f : ld_b32(s.beta, s.b_off + (uint32_t)c0 * 4);
}

// 16 x 16 fp32 products on the matrix cores with X in row layout (lane 16p + r holds
// X[r][4p + e]) and Y in column layout (holds Y[4p + e][r], the accumulator layout); the
// contraction index of step s is 4p + s, which both layouts hold as element s.
// mm_col returns X Y in column layout; mm_row returns X Y in row layout, computed as the
// column layout of Y^T X^T.
__device__ __forceinline__ f32x4 mm_col(const f32x4& xr, const f32x4& yc) {
  f32x4 acc = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f32(xr[s], yc[s], acc);
  return acc;
}
__device__ __forceinline__ f32x4 mm_row(const f32x4& xr, const f32x4& yc) {
  f32x4 acc = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f32(yc[s], xr[s], acc);
  return acc;
}

// Inverse of (I + N) for N strictly lower triangular (16 x 16), given N in column layout
// (nc: lane holds N[4p + e][r]) and row layout (nr: lane holds N[r][4p + e]). N is
// nilpotent (N^16 = 0), so (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) exactly; the
// factors are polynomials in N and commute, which lets every product take its left factor
// in row layout and its right factor in column layout. Returns the inverse in column
// layout (lane holds Inv[4p + e][r]).
__device__ __forceinline__ f32x4 unit_lower_inverse(const f32x4& nc, const f32x4& nr, int rr,
                                                    int p) {
  const f32x4 n2c = mm_col(nr, nc), n2r = mm_row(nr, nc);
  const f32x4 n4c = mm_col(n2r, n2c), n4r = mm_row(n2r, n2c);
  const f32x4 n8r = mm_row(n4r, n4c);
  const f32x4 nn2c = mm_col(nr, n2c);
  f32x4 y1;
#pragma unroll
  for (int e = 0; e < 4; ++e) y1[e] = (4 * p + e == rr ? 1.f : 0.f) - nc[e] + n2c[e] - nn2c[e];
  const f32x4 t1 = mm_col(n4r, y1);
  f32x4 y2;
#pragma unroll
  for (int e = 0; e < 4; ++e) y2[e] = y1[e] + t1[e];
  const f32x4 t2 = mm_col(n8r, y2);
  f32x4 inv;
#pragma unroll
  for (int e = 0; e < 4; ++e) inv[e] = y2[e] + t2[e];
  return inv;
}

// Position `local` among the 2 n items of n split chains: groups of (up to) 8 chains list
// their first halves, then their second halves, so the two halves of a chain are 8 items
// apart. Workgroups are dispatched round-robin over the 8 XCDs, so both halves run on one
// XCD and the second reads the chain's q, k, g through that XCD's L2.
__host__ __device__ inline void split_item(uint32_t local, uint32_t n, uint32_t& chain,
                                           uint32_t& part) {
  const uint32_t group = local / 16, within = local % 16;
  const uint32_t gsize = n - 8 * group < 8 ? n - 8 * group : 8;
  chain = 8 * group + within % gsize;
  part = 1 + within / gsize;
}

// State history of the backward pass. For every chain (sequence n, head h) the kernels
// keep one dk x dv bf16 matrix per pair of 16-token blocks of the chain (its 64-token
// steps padded with identity tokens): the history of states holds the state entering the
// pair's first (even) block, the history of state gradients the gradient reaching the end
// of its second (odd) block; the state between the two blocks and the gradient between
// them follow from these within the pair. A matrix is stored as the 16x16x32 B operands of
// the state tiles: for value tile ct and channel slab ks, lane l = 16 p + r holds the 8
// channels 32 ks + 8 p + i (i < 8) of column 16 ct + r, 16 bytes at
// ((ct * 4 + ks) * 64 + l) * 16. One matrix is dk * dv * 2 bytes, i.e. dk * dv / 16 bytes
// per token, and the chains of head h are laid out along the padded token axis: sequence n
// starts at padded token cu[n] + 64 n with packed sequences (B = 1), at n * ceil64(T)
// otherwise; no two sequences' padded ranges overlap.
__device__ __forceinline__ size_t hist_tokens(const ChunkArgs& a) {
  return a.cu ? (size_t)a.T + 64 * (size_t)a.N : (size_t)a.N * (((size_t)a.T + 63) / 64 * 64);
}
__device__ __forceinline__ size_t hist_chain_offset(const ChunkArgs& a, int n, int h,
                                                    const TokenRange& tr) {
  const size_t start = a.cu ? (size_t)tr.t0 + 64 * (size_t)n : (size_t)n * (((size_t)a.T + 63) / 64 * 64);
  return ((size_t)h * hist_tokens(a) + start) * (kDK / 16) * (size_t)a.dv;
}

}  // namespace kda
