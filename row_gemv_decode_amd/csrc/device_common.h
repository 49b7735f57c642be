// device_common.h -- small device-side helpers shared by the library's kernels
// (gfx950 only).  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace skinny {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Reinterpret a dword as two f16 / two bf16.  Always pass a plain scalar:
// applying __builtin_bit_cast directly to an ext-vector element expression
// (v.y, v.z, ...) reads element 0 with this compiler, so every cast of a
// vector lane goes through these by-value helpers.
__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ b2_t as_b2(uint32_t u) { return __builtin_bit_cast(b2_t, u); }
__device__ __forceinline__ uint32_t h2_bits(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ _Float16 half_from_bits(uint16_t b) {
  return __builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float f32_from_bits(uint32_t b) { return __builtin_bit_cast(float, b); }

// Eight fp32 values (two 16-byte words, in memory order) -> eight bf16 packed
// in four dwords, each rounded to nearest even by the compiler's
// float -> __bf16 conversion (the one the window-row cast uses), so a row
// converted here equals the same row cast beforehand, bit for bit.
__device__ __forceinline__ uint32_t bf16x2_rne(uint32_t lo_bits, uint32_t hi_bits) {
  const b2_t v = {(__bf16)f32_from_bits(lo_bits), (__bf16)f32_from_bits(hi_bits)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 bf16x8_rne(u32x4 lo, u32x4 hi) {
  u32x4 out;
  out[0] = bf16x2_rne(lo[0], lo[1]);
  out[1] = bf16x2_rne(lo[2], lo[3]);
  out[2] = bf16x2_rne(hi[0], hi[1]);
  out[3] = bf16x2_rne(hi[2], hi[3]);
  return out;
}

// ---------------------------------------------------------------------------
// Q8_0-style dequant of eight consecutive codes of one 32-block (opus r35
// track A, section 1: block-quantised weights become f16 through `dq_f16`).
// Each weight is RNE_f16(d * q): the code is converted to f16 exactly
// (|q| <= 128) and one IEEE f16 multiply rounds the exact product once, to
// nearest even, with the product's sign (so d < 0, q = 0 gives -0).  Every
// path of the library -- the standalone dequant kernel, the fused GEMV and the
// fused GEMM B-loader -- calls this one function, so their weights are equal
// bit for bit.
// ---------------------------------------------------------------------------
// The code reaches f16 without a conversion instruction: with u = q + 128
// (the byte q ^ 0x80), the f16 whose bits are 0x6400 | u is 1024 + u exactly,
// and subtracting 1152 leaves q exactly (every step is exact in f16).  Two
// byte permutes build four such f16 from four codes, so eight codes cost one
// xor per four, two permutes, two packed subtracts and two packed multiplies
// per four.
__device__ __forceinline__ void q8_quad(uint32_t four_codes, h2_t d2, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = four_codes ^ 0x80808080u;
  const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  // bytes (low first): lo = u0, 0x64, u1, 0x64; hi = u2, 0x64, u3, 0x64
  const uint32_t plo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t phi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  lo = h2_bits(d2 * (as_h2(plo) - bias));
  hi = h2_bits(d2 * (as_h2(phi) - bias));
}

// eight codes (two dwords, little-endian bytes) -> eight f16 packed in 4 dwords
__device__ __forceinline__ u32x4 q8_dequant8(u32x2 codes, _Float16 d) {
  const uint32_t c0 = codes[0];
  const uint32_t c1 = codes[1];
  const h2_t d2 = {d, d};
  u32x4 out;
  uint32_t a, b;
  q8_quad(c0, d2, a, b);
  out[0] = a;
  out[1] = b;
  q8_quad(c1, d2, a, b);
  out[2] = a;
  out[3] = b;
  return out;
}

// ---------------------------------------------------------------------------
// Q4_0-style dequant of eight consecutive 4-bit codes of one 32-block.  The
// pages name 4-bit block formats (the Strata PR #109 page, "Measured")
// without defining one; the format here: unsigned codes q in 0..15, two per
// byte (element 2i in the low nibble of byte i, 2i + 1 in the high nibble),
// one f16 scale d per 32-block, weight RNE_f16(d * (q - 8)).  As for Q8_0,
// the code reaches f16 exactly (bits 0x6400 | q are 1024 + q; subtracting
// 1032 leaves q - 8 exactly) and one IEEE f16 multiply rounds the exact
// product once.  Every path (standalone, fused GEMV, fused GEMM) calls this.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 q4_dequant8(uint32_t codes, _Float16 d) {
  const uint32_t lo = codes & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6 (one per byte)
  const uint32_t hi = (codes >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
  const h2_t d2 = {d, d};
  const h2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  // pair i = (element 2i, element 2i + 1): byte i of lo in the low half, byte
  // i of hi in the high half (selector 0x0c gives a zero byte)
  const uint32_t p0 = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
  const uint32_t p1 = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
  const uint32_t p2 = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
  const uint32_t p3 = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
  u32x4 out;
  out[0] = h2_bits(d2 * (as_h2(p0) - bias));
  out[1] = h2_bits(d2 * (as_h2(p1) - bias));
  out[2] = h2_bits(d2 * (as_h2(p2) - bias));
  out[3] = h2_bits(d2 * (as_h2(p3) - bias));
  return out;
}

// ---------------------------------------------------------------------------
// Q2_0-style dequant of eight consecutive 2-bit codes of one 32-block, given
// as the low 16 bits of `codes` (code i at bits 2i and 2i + 1).  The pages
// name a 2-bit block format (the Strata PR #109 page, "Measured": Q2_0 runs)
// without defining one; the format here: unsigned codes q in 0..3, four per
// byte (element 4b + i at bits 2i of byte b), one f16 scale d per 32-block,
// weight RNE_f16(d * (q - 2)).  As for Q4_0, a code reaches f16 exactly in
// the low bits of 0x6400 (1024 + q), subtracting 1026 leaves q - 2 exactly,
// and one IEEE f16 multiply rounds the exact product once.  With
// s = codes | codes << 14, bits 4p .. 4p + 1 of s hold code 2p and bits
// 4p + 16 .. 4p + 17 hold code 2p + 1, so one shift and one and-or place
// each pair of codes in the two halves of a dword.  Every path (standalone,
// fused GEMV, fused GEMM) calls this.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 q2_dequant8(uint32_t codes, _Float16 d) {
  const uint32_t c = codes & 0xFFFFu;
  const uint32_t s = c | (c << 14);
  const h2_t d2 = {d, d};
  const h2_t bias = {(_Float16)1026.0f, (_Float16)1026.0f};
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t pair = ((s >> (4 * p)) & 0x00030003u) | 0x64006400u;
    out[p] = h2_bits(d2 * (as_h2(pair) - bias));
  }
  return out;
}

// Device-coherent accesses for data handed from one workgroup to another in
// the same launch.  Relaxed agent-scope atomic stores/loads compile to plain
// global stores/loads with the sc1 (device scope) bit: they are coherent
// across the XCDs' L2 caches without the whole-L2 write-back and invalidate
// that an agent-scope fence costs.  A writer waits for its stores to complete
// (s_waitcnt) before it counts itself in with an atomic; the reader issues its
// loads only after its atomic returned the final count.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // every outstanding load and store of this wave completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// fp32 -> stored output element, round to nearest even
template <int CK>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float v) {
  if constexpr (CK == CK_F32) {
    ((float*)base)[idx] = v;
  } else if constexpr (CK == CK_F16) {
    ((_Float16*)base)[idx] = (_Float16)v;
  } else {
    ((__bf16*)base)[idx] = (__bf16)v;
  }
}

}  // namespace skinny
