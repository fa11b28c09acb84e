// Depth-KV repack for gfx950.
//
// The depth KV of one token position is the set of K/V that the L_d earlier
// layers wrote for it.  The logical layout [B, T, L_d, Hkv, d] interleaves kv
// heads and puts the slots of one position next to those of other heads.  The
// pages flatten depth KV along a single T x L axis per head so that a query
// chunk reads one contiguous range (gist.science (de) "Mixture-of-Depths
// Attention", Technische Zusammenfassung section 2, Flash-Compatible Layout and
// Chunk-Aware Layout; mhpn.cn article section 2.1, chunked contiguous
// storage).  This kernel writes, per (b, kv head), key n = t * L_d + j:
//   k_packed [B][Hkv][NKp][D]   rows of d elements
//   v_packed [B][Hkv][NKp][D]   the same for the values
// with zero rows for n >= T * L_d (NKp = T * L_d rounded up to 32).  One
// thread per 16-byte chunk of a packed row; reads and writes are contiguous
// 16-byte accesses.
#pragma once

#include "moda_common.hpp"

namespace moda {

struct PackParams {
  const void* kd;
  const void* vd;
  void* kp;
  void* vp;
  int B, T, Hkv, L_d;
  long long NKp;
};

template <typename E, int D>
__global__ __launch_bounds__(256) void moda_pack_depth_kernel(PackParams p) {
  constexpr int VE = Traits<E>::VE;
  constexpr int CPR = D / VE;                   // 16-byte chunks per row
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rows = (long long)p.B * p.Hkv * p.NKp;
  if (idx >= rows * CPR) return;
  const long long row = idx / CPR;              // (bh, n) in packed order
  const int c = (int)(idx % CPR);
  const long long bh = row / p.NKp;
  const int n = (int)(row % p.NKp);             // T * L_d < 2^31 (checked at the boundary)
  const int b = (int)(bh / p.Hkv), kvh = (int)(bh % p.Hkv);
  u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
  if (n < p.T * p.L_d) {
    const int t = n / p.L_d, j = n - t * p.L_d;
    const long long src = ((((long long)b * p.T + t) * p.L_d + j) * p.Hkv + kvh) * D + c * VE;
    kv = ld16(reinterpret_cast<const E*>(p.kd) + src);
    vv = ld16(reinterpret_cast<const E*>(p.vd) + src);
  }
  st16(reinterpret_cast<E*>(p.kp) + row * D + c * VE, kv);
  st16(reinterpret_cast<E*>(p.vp) + row * D + c * VE, vv);
}

}  // namespace moda

namespace moda {

// Write step: one layer's K/V of every position into one slot of the packed
// depth buffers (the layer appends its KV to the depth stream that later
// layers read -- gist.science (de) "Mixture-of-Depths Attention", Technische
// Zusammenfassung section 2, Write-Step).  Same packed layout as
// moda_pack_depth_kernel with L_cap slots per position:
//   k_packed[b][kvh][t * L_cap + slot][:]   = k_new[b][t][kvh][:]
//   v_packed[b][kvh][t * L_cap + slot][:]   = v_new[b][t][kvh][:]
// One thread per 16-byte chunk of one (b, t, kvh) row: one 16-byte load and
// one 16-byte store per tensor.
struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* kp;
  void* vp;
  int B, T, Hkv, L_cap, slot;
  long long NKp;
};

template <typename E, int D>
__global__ __launch_bounds__(256) void moda_append_depth_kernel(AppendParams p) {
  constexpr int VE = Traits<E>::VE;
  constexpr int CPR = D / VE;     // 16-byte chunks per row
  const long long rows = (long long)p.B * p.T * p.Hkv;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * CPR) return;
  const long long row = idx / CPR;              // (b, t, kvh) in input order
  const int c = (int)(idx % CPR);
  const int kvh = (int)(row % p.Hkv);
  const long long bt = row / p.Hkv;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);
  const long long bh = (long long)b * p.Hkv + kvh;
  const long long n = (long long)t * p.L_cap + p.slot;
  const E* ks = reinterpret_cast<const E*>(p.k_new) + row * D + c * VE;
  const E* vs = reinterpret_cast<const E*>(p.v_new) + row * D + c * VE;
  E* kd = reinterpret_cast<E*>(p.kp) + (bh * p.NKp + n) * D + c * VE;
  E* vd = reinterpret_cast<E*>(p.vp) + (bh * p.NKp + n) * D + c * VE;
  st16(kd, ld16(ks));
  st16(vd, ld16(vs));
}

}  // namespace moda

namespace moda {

// 8-bit depth KV (a memory tip of the mhpn.cn article, section 4.2): the same
// packed rows as moda_pack_depth_kernel, each stored as d int8 codes plus one
// float32 scale, scale = max|x| / 127 and code = rint(x / scale) clamped to
// +-127 (0 for an all-zero row), every step in float32.  LPR lanes per packed
// row, 8 elements each; the row maximum is reduced across those lanes.
struct PackQ8Params {
  const void* kd;
  const void* vd;
  int8_t* kq;
  int8_t* vq;
  float* ks;
  float* vs;
  int B, T, Hkv, L_d;
  long long NKp;
};

template <typename E>
__device__ __forceinline__ void load8(const E* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&v)[8]) {
  const bf16x8 f = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (float)f[j];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
}

__device__ __forceinline__ u32x2 quantize8(const float (&x)[8], float scale) {
  u32x2 w = {0u, 0u};
  if (scale > 0.f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float c = rintf(x[j] / scale);
      c = fminf(fmaxf(c, -127.f), 127.f);
      w[j >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (j & 3));
    }
  }
  return w;
}

// Quantise one row of K and one row of V (D elements each) with LPR = D / 8
// lanes per row, 8 elements per lane: the row maximum is reduced across the
// row's lanes (every lane of the wave takes part in the exchange), then codes
// and scales are written when `valid`.  Rows with valid == false but
// store == true are padding: scale 0, codes 0.
template <typename E, int D>
__device__ __forceinline__ void quant_rows(const E* srck, const E* srcv, bool load, bool store, int l,
                                           int8_t* dk, int8_t* dv, float* sk_out, float* sv_out) {
  constexpr int LPR = D / 8;
  float xk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (load) {
    load8(srck + l * 8, xk);
    load8(srcv + l * 8, xv);
  }
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) { mk = fmaxf(mk, fabsf(xk[j])); mv = fmaxf(mv, fabsf(xv[j])); }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, off));
    mv = fmaxf(mv, __shfl_xor(mv, off));
  }
  const float sk = mk / 127.f, sv = mv / 127.f;
  if (store) {
    *reinterpret_cast<u32x2*>(dk + l * 8) = quantize8(xk, sk);
    *reinterpret_cast<u32x2*>(dv + l * 8) = quantize8(xv, sv);
    if (l == 0) {
      *sk_out = sk;
      *sv_out = sv;
    }
  }
}

template <typename E, int D>
__global__ __launch_bounds__(256) void moda_pack_depth_q8_kernel(PackQ8Params p) {
  constexpr int LPR = D / 8;                    // lanes per packed row
  constexpr int RPB = 256 / LPR;                // rows per workgroup
  const long long rows = (long long)p.B * p.Hkv * p.NKp;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int l = threadIdx.x % LPR;
  bool load = false;
  long long src = 0;
  if (row < rows) {
    const long long bh = row / p.NKp;
    const int n = (int)(row % p.NKp);
    if (n < p.T * p.L_d) {
      const int b = (int)(bh / p.Hkv), kvh = (int)(bh % p.Hkv);
      const int t = n / p.L_d, j = n - t * p.L_d;
      src = ((((long long)b * p.T + t) * p.L_d + j) * p.Hkv + kvh) * D;
      load = true;
    }
  }
  const long long r = row < rows ? row : 0;
  quant_rows<E, D>(reinterpret_cast<const E*>(p.kd) + src, reinterpret_cast<const E*>(p.vd) + src, load,
                   row < rows, l, p.kq + r * D, p.vq + r * D, p.ks + r, p.vs + r);
}

// Write step with 8-bit depth KV: one layer's K/V rows quantised into slot
// `slot` of int8 packed buffers with L_cap slots per position (same codes as
// moda_pack_depth_q8_kernel would give those rows).
struct AppendQ8Params {
  const void* k_new;
  const void* v_new;
  int8_t* kq;
  int8_t* vq;
  float* ks;
  float* vs;
  int B, T, Hkv, L_cap, slot;
  long long NKp;
};

template <typename E, int D>
__global__ __launch_bounds__(256) void moda_append_depth_q8_kernel(AppendQ8Params p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const long long rows = (long long)p.B * p.T * p.Hkv;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;   // (b, t, kvh) in input order
  const int l = threadIdx.x % LPR;
  const bool ok = row < rows;
  const long long r = ok ? row : 0;
  const int kvh = (int)(r % p.Hkv);
  const long long bt = r / p.Hkv;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);
  const long long dst = ((long long)b * p.Hkv + kvh) * p.NKp + (long long)t * p.L_cap + p.slot;
  quant_rows<E, D>(reinterpret_cast<const E*>(p.k_new) + r * D, reinterpret_cast<const E*>(p.v_new) + r * D,
                   ok, ok, l, p.kq + dst * D, p.vq + dst * D, p.ks + dst, p.vs + dst);
}

}  // namespace moda
