// Device-side helpers shared by the verify-round kernels (gfx950 / CDNA4).
//
// Numerics used throughout:
//  * Activations stay fp32.  Before a matrix-core product each fp32 value x
//    is split into two fp16 parts, hi = fp16(x) and lo = fp16((x - hi) * 2^11),
//    which together carry 22 significant bits; the low part is scaled so it
//    stays a normal fp16 number for |x| down to about 1e-4.  Products of the
//    two parts go to separate fp32 accumulators, combined as hi + 2^-11 lo.
//  * Weights enter the matrix cores as exact small integers in fp16 (a
//    4-bit code times a 6-bit scale is at most 945; a 6-bit code times an
//    8-bit scale is split into an exact fp16 high part and a one-ulp
//    remainder), so every product is exact and every sum is fp32.
//  * v_mfma_f32_16x16x32_f16 operand layout (checked on gfx950): lane l of
//    the A operand holds row l%16, k = 8*(l/16) + s in slot s (s = 0..7);
//    the B operand holds column l%16 with the same k mapping; the result
//    holds row 4*(l/16) + i, column l%16 in slot i (i = 0..3).  A row's
//    result bits do not depend on the other rows of the tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SV_WAVE 64
#ifndef SV_KV_CHUNK
#define SV_KV_CHUNK 128   // KV capacity granularity (positions)
#endif

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ half2v fma_h2(half2v a, half2v b, half2v c) {
  return __builtin_elementwise_fma(a, b, c);
}

#define SV_LO_SCALE 2048.0f
#define SV_LO_INV (1.0f / 2048.0f)

// fp32 -> fp16 rounding toward zero through one explicit conversion
// instruction.  The low part below must be computed from exactly the high
// part that is stored; a plain (f16) cast may be lowered to two different
// conversion instructions for the two uses, and they can round an exact tie
// differently.
__device__ __forceinline__ f16 to_f16_rtz(float x) {
  auto p = __builtin_amdgcn_cvt_pkrtz(x, 0.0f);
  return __builtin_bit_cast(half2v, p)[0];
}

__device__ __forceinline__ void split_hl(float x, f16 &hi, f16 &lo) {
  hi = to_f16_rtz(x);
  lo = (f16)((x - (float)hi) * SV_LO_SCALE);
}

__device__ __forceinline__ half8 make_half8(u32x4 u) { return __builtin_bit_cast(half8, u); }

// ---- packed activation operand ("apack") -----------------------------------
// For an activation matrix X[M][K] (K a multiple of 32): M-tile mt, k-step
// ks (32 values of k), part hl (0 = hi, 1 = lo) is a 1024-byte block at
// ((mt*KS + ks)*2 + hl)*1024 of 64 pieces of 16 bytes, each holding row
// 16*mt + r, k = 32*ks + 8*g + s for s = 0..7 (the operand of MFMA lane
// r + 16 g).  Up to SV_APACK_ROWMAJOR_MAX rows (the small-row kernel) the
// piece is 4 r + g: a 128-byte line holds two whole rows, so a tile with few
// real rows touches few lines.  Beyond (the wide kernel, whose tiles are
// full) it is r + 16 g: each lane's 16 bytes follow the previous lane's.
#define SV_APACK_ROWMAJOR_MAX 32
__device__ __forceinline__ int apack_piece(int r, int g, int M) {
  return M <= SV_APACK_ROWMAJOR_MAX ? 4 * r + g : r + 16 * g;
}
__device__ __forceinline__ size_t apack_off(int mt, int KS, int ks, int hl, int piece) {
  return ((size_t)(mt * KS + ks) * 2 + hl) * 1024 + (size_t)piece * 16;
}
// Rounds of at most 4 rows (SV_APACK4_ROWS) use a compact arrangement
// instead, which holds only real rows and puts two k-steps in one 64-lane
// load: k-step pair p = ks / 2 occupies 1024 bytes at p * 1024, lane l of it
// = k-octet l / 16, part (l / 8) % 2, k-step parity (l / 4) % 2, row l % 4.
#define SV_APACK4_ROWS 4
__device__ __forceinline__ size_t apack4_off(int ks, int hl, int g, int r) {
  return (size_t)(ks >> 1) * 1024 + (size_t)(16 * g + 8 * hl + 4 * (ks & 1) + r) * 16;
}
// Byte offset of element (m, k) inside the packed operand (part hl) of a
// round of M rows.
__device__ __forceinline__ size_t apack_elem(int m, int k, int KS, int hl, int M) {
  int mt = m >> 4, ks = k >> 5, g = (k >> 3) & 3, s = k & 7;
  if (M <= SV_APACK4_ROWS) return apack4_off(ks, hl, g, m) + 2 * s;
  return apack_off(mt, KS, ks, hl, apack_piece(m & 15, g, M)) + 2 * s;
}

// ---- packed sub-block sums ("sxpack") for the 4-bit super-block format ----
// Sx[m][j] = sum of the 32 activations of sub-block j.  For M-tile mt,
// super-block sb (8 sub-blocks), part hl: 16 lanes x 16 bytes at
// ((mt*NSB + sb)*2 + hl)*256 + (m%16)*16, slot s = sub-block 8*sb + s.
__device__ __forceinline__ size_t sxpack_off(int mt, int NSB, int sb, int hl, int row16) {
  return ((size_t)(mt * NSB + sb) * 2 + hl) * 256 + (size_t)row16 * 16;
}

// Lane l ^ 1 and l ^ 2's value within a quad (DPP quad permutations), and
// lane l ^ 16 and l ^ 32's (the cross-row lane swaps): register moves, no LDS
// round trip.  Every lane of the quad, or of the pair of rows (l ^ 16) or
// wave (l ^ 32), must be active; workgroups are one-dimensional with whole
// waves, so threadIdx.x's low six bits are the lane.
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor16(float v) {
  const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);   // rows {0 0 2 2}, {1 1 3 3}
  return __uint_as_float((threadIdx.x & 16) ? h[0] : h[1]);
}
__device__ __forceinline__ float lane_xor32(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);   // rows {0 1 0 1}, {2 3 2 3}
  return __uint_as_float((threadIdx.x & 32) ? h[0] : h[1]);
}

// Lane l ^ 8's value (rotation by 8 within a row of 16), and, where lanes l
// and l ^ 8 already hold the same value, lane l ^ 4's (rotation by 4 then
// lands on a lane equal to it).
__device__ __forceinline__ float lane_xor8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor4_sym8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
}

// 4-lane fixed-order sum: lanes 4q..4q+3 -> (v0 + v1) + (v2 + v3) in all four.
__device__ __forceinline__ float sum4_fixed(float v) {
  float a = v + lane_xor1(v);
  return a + lane_xor2(a);
}

__device__ __forceinline__ float max_f(float a, float b) { return a > b ? a : b; }

// ---- device-scope stores and the arrival counter ---------------------------
// Results that another workgroup of the same launch reads (the decision
// kernels' per-row argmax) are written with agent-scope accesses (sc1):
// they are coherent across the per-XCD L2 caches by themselves, so
// publishing them needs only the wait for this wave's own stores before the
// arrival counter is bumped -- no cache-wide writeback or invalidate.  (Such
// an arrival costs microseconds; results that a later kernel reads, like
// the attention chunk slots, go through the kernel boundary instead.)
typedef __amdgpu_buffer_rsrc_t sv_rsrc;
#define SV_CPOL_AGENT 16  // sc1: agent-scope coherence

__device__ __forceinline__ sv_rsrc sv_make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent4(sv_rsrc r, uint32_t off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, SV_CPOL_AGENT);
}
// Stores of data that other workgroups of the same launch read (the fused
// layer kernel's activations): agent-scope (sc1) stores, written through the
// XCD's L2 to the device's point of coherence.  COH = false: plain stores.
template <bool COH>
__device__ __forceinline__ void st_h8(void *p, half8 v) {
  if constexpr (COH) {
    const u32x4 u = __builtin_bit_cast(u32x4, v);
    uint64_t *q = (uint64_t *)p;
    __hip_atomic_store(q, (uint64_t)u[0] | ((uint64_t)u[1] << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)u[2] | ((uint64_t)u[3] << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *(half8 *)p = v;
  }
}
template <bool COH>
__device__ __forceinline__ void st_h4(void *p, half4 v) {
  if constexpr (COH)
    __hip_atomic_store((uint64_t *)p, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *(half4 *)p = v;
}
template <bool COH>
__device__ __forceinline__ void st_f16(void *p, f16 v) {
  if constexpr (COH)
    __hip_atomic_store((uint16_t *)p, __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *(f16 *)p = v;
}
template <bool COH>
__device__ __forceinline__ void st_f32(float *p, float v) {
  if constexpr (COH)
    __hip_atomic_store((uint32_t *)p, __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Wait until this wave's stores are performed; also a compiler barrier.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_barrier() { asm volatile("" ::: "memory"); }

// Arrival on a launch-local counter: returns true in exactly one caller, the
// n-th to arrive, which also resets the counter to zero for the next launch.
// Call after wait_stores(); lane 0 of the wave performs the atomic.
__device__ __forceinline__ bool arrive_last(int32_t *cnt, int n, int lane) {
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  const bool last = (prev == n - 1);
  if (last && lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  compiler_barrier();
  return last;
}

// Deterministic row scale of the deferred RMSNorm: 1/sqrt(sum(ssq)/H + eps),
// the partial sums of squares summed in increasing order.
__device__ __forceinline__ float inv_rms_from(const float *ssq_row, int nparts, int H,
                                              float eps) {
  float s = 0.f;
  for (int j = 0; j < nparts; ++j) s += ssq_row[j];
  return 1.0f / sqrtf(s / (float)H + eps);
}
