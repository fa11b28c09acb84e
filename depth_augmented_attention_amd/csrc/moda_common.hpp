// Shared device-side helpers for the MoDA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Per element type: VE = elements per 16-byte vector; Frag = the 8 k-values a
// lane contributes to one 16-wide k-chunk of a 32x32 matrix-core product.
template <typename E> struct Traits;
template <> struct Traits<bf16> {
  static constexpr int VE = 8;
  using Frag = bf16x8;
};
template <> struct Traits<float> {
  static constexpr int VE = 4;
  using Frag = f32x8;
};

// 16-byte vector load / store of raw bits.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One k-chunk fragment (8 consecutive elements) from memory.
__device__ __forceinline__ bf16x8 load_frag(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f32x8 load_frag(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <typename Frag> __device__ __forceinline__ Frag zero_frag() { return Frag{}; }

// C[32x32] += A[32x16] * B[16x32] on the matrix cores.  Lane l supplies
// A[l%32][8*(l/32)+j] and B[8*(l/32)+j][l%32], j = 0..7.
__device__ __forceinline__ f32x16 mma16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// float32: eight 32x32x2 products; product j sums over the k-pair {j, 8+j}
// (lane half 0 holds k = j, lane half 1 holds k = 8+j), so the eight together
// cover the same 16 k-values with the same lane ownership as the bf16 case.
__device__ __forceinline__ f32x16 mma16(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// Eight float32 probabilities as a B-operand fragment.
__device__ __forceinline__ void to_frag(const float* p, bf16x8& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)p[j];
}
__device__ __forceinline__ void to_frag(const float* p, f32x8& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = p[j];
}

// Output element stores (round to nearest even for bf16).
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Eight int8 codes (8 bytes at p) times a float32 scale, as a fragment of the
// element type (8-bit depth KV: one scale per packed key or value row).
__device__ __forceinline__ void dequant8(const int8_t* p, float scale, float (&v)[8]) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int code = (int)(int8_t)(w[j >> 2] >> (8 * (j & 3)));
    v[j] = scale * (float)code;
  }
}
__device__ __forceinline__ bf16x8 dequant_frag_bf16(const int8_t* p, float scale) {
  float v[8];
  dequant8(p, scale, v);
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)v[j];
  return f;
}
__device__ __forceinline__ f32x8 dequant_frag_f32(const int8_t* p, float scale) {
  float v[8];
  dequant8(p, scale, v);
  return f32x8{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
}
template <typename E> struct Dequant;
template <> struct Dequant<bf16> {
  static __device__ __forceinline__ bf16x8 frag(const int8_t* p, float s) { return dequant_frag_bf16(p, s); }
  static __device__ __forceinline__ bf16 one(int8_t c, float s) { return (bf16)(s * (float)c); }
};
template <> struct Dequant<float> {
  static __device__ __forceinline__ f32x8 frag(const int8_t* p, float s) { return dequant_frag_f32(p, s); }
  static __device__ __forceinline__ float one(int8_t c, float s) { return s * (float)c; }
};

// Quotient by a divisor fixed for the launch (the GQA group size, the depth
// count) through one 32x32->64-bit multiply (the round-up reciprocal of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): exact for 0 <= x < 2^31 with
// magic = ceil(2^(31+s) / G), s = ceil(log2 G), shift = 31 + s.
__device__ __forceinline__ int div_g(int x, uint32_t magic, int shift) {
  return (int)(((uint64_t)(uint32_t)x * magic) >> shift);
}

// Row order of the 32-key operand tiles.  A 32x32 accumulator gives lane half
// h the rows {8q + 4h + i : q = 0..3, i = 0..3}; loading key pi(m) into operand
// row m (pi swaps bits 2 and 3 of m) makes the 16 values a lane holds be the
// keys {16c + 8h + j : c = 0,1; j = 0..7} -- exactly the 8-key runs that the
// following P.V product takes from lane half h.  So probabilities feed the
// second product without any exchange between lanes.
__device__ __forceinline__ int key_row_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// Key (0..31 within the tile) of accumulator register r in lane half h.
__device__ __forceinline__ int reg_key(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

}  // namespace moda
