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
// thread per 16-byte chunk, taken in the source order, so that consecutive
// threads read consecutive bytes of both kv heads' rows; each (b, kv head)
// destination then receives whole 256-byte rows (d = 128, bf16).  The threads
// past the source chunks write the zero rows.
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
  const long long TL = (long long)p.T * p.L_d;
  const long long nsrc = (long long)p.B * TL * p.Hkv * CPR;
  if (idx < nsrc) {
    // source order: consecutive threads read consecutive bytes of [B,T,L_d,Hkv,d]
    const long long rs = idx / CPR;
    const int c = (int)(idx % CPR);
    const long long r1 = rs / p.Hkv;
    const int kvh = (int)(rs % p.Hkv);
    const long long b = r1 / TL, n = r1 % TL;
    const long long dst = ((b * p.Hkv + kvh) * p.NKp + n) * D + c * VE;
    const u32x4 kv = ld16(reinterpret_cast<const E*>(p.kd) + rs * D + c * VE);
    const u32x4 vv = ld16(reinterpret_cast<const E*>(p.vd) + rs * D + c * VE);
    st16(reinterpret_cast<E*>(p.kp) + dst, kv);
    st16(reinterpret_cast<E*>(p.vp) + dst, vv);
    return;
  }
  // zero rows n in [T L_d, NKp) of every (b, kv head)
  const int npad = (int)(p.NKp - TL);
  if (npad == 0) return;
  const long long k = idx - nsrc;
  const long long pr = k / CPR;
  const int c = (int)(k % CPR);
  const long long bh = pr / npad;
  if (bh >= (long long)p.B * p.Hkv) return;
  const long long dst = (bh * p.NKp + TL + pr % npad) * D + c * VE;
  const u32x4 z = {0, 0, 0, 0};
  st16(reinterpret_cast<E*>(p.kp) + dst, z);
  st16(reinterpret_cast<E*>(p.vp) + dst, z);
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
// +-127 (0 for an all-zero row), every step in float32.  D / 16 lanes per
// packed row, 16 elements each; the row maximum is reduced across those
// lanes.  A two-dimensional grid ((b, kv head) planes by row blocks) and a
// multiply-shift quotient by L_d keep 64-bit divisions out of the index math.
struct PackQ8Params {
  const void* kd;
  const void* vd;
  int8_t* kq;
  int8_t* vq;
  float* ks;
  float* vs;
  int B, T, Hkv, L_d;
  long long NKp;
  uint32_t ld_magic;  // n / L_d == (n * ld_magic) >> ld_shift for 0 <= n < 2^31
  int ld_shift;
  long long rb0;      // first block of rows of this launch
};

constexpr int kQ8Elems = 16;   // elements per lane

template <typename E>
__device__ __forceinline__ void load16(const E* p, float (&v)[kQ8Elems]);
template <>
__device__ __forceinline__ void load16<bf16>(const bf16* p, float (&v)[kQ8Elems]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x8 f = *reinterpret_cast<const bf16x8*>(p + 8 * h);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[8 * h + j] = (float)f[j];
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&v)[kQ8Elems]) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * h + j] = a[j];
  }
}

// Codes rint(x / scale), clamped to +-127, of 16 elements; the quotient is
// the correctly rounded float32 one.  It is formed as x * r first, with r the
// hardware reciprocal of scale (within 1 ulp, 2^-23 relative): that product
// is within 2^-22 relative (at most 3.1e-5 for |x / scale| <= 127) of the
// exact quotient, and the correctly rounded quotient within 2^-24 relative
// of it, so both round to the same integer unless one of them lies within
// about 4e-5 of a half-integer.  An element whose product lies within 1e-4
// of a half-integer (rare) is divided exactly instead, on its own: the other
// elements of the lane keep their codes.  Same codes either way, at a
// fraction of the cost of IEEE divisions.
__device__ __forceinline__ u32x4 quantize16(const float (&x)[kQ8Elems], float scale) {
  u32x4 w = {0u, 0u, 0u, 0u};
  if (scale > 0.f) {
    const float r = __builtin_amdgcn_rcpf(scale);
    float c[kQ8Elems], y[kQ8Elems];
    float dev = 0.f;   // the lane's largest distance from an integer
#pragma unroll
    for (int j = 0; j < kQ8Elems; ++j) {
      y[j] = x[j] * r;
      c[j] = rintf(y[j]);
      dev = fmaxf(dev, fabsf(y[j] - c[j]));
    }
    if (__builtin_expect(dev > 0.4999f, 0)) {
      // only the elements near a half-integer divide exactly; an element
      // that no lane of the wave needs is skipped
#pragma unroll
      for (int j = 0; j < kQ8Elems; ++j)
        if (fabsf(y[j] - c[j]) > 0.4999f) c[j] = rintf(x[j] / scale);
    }
    // |x| <= max|x| and scale = max|x| / 127 rounded, so |x / scale| <=
    // 127 (1 + 2^-24) and every code is already within +-127: the clamp is
    // a no-op here.  Four codes go into one word by byte permutes (the low
    // byte of each 32-bit integer).
#pragma unroll
    for (int q = 0; q < kQ8Elems / 4; ++q) {
      const uint32_t i0 = (uint32_t)(int)c[4 * q], i1 = (uint32_t)(int)c[4 * q + 1];
      const uint32_t i2 = (uint32_t)(int)c[4 * q + 2], i3 = (uint32_t)(int)c[4 * q + 3];
      const uint32_t lo = __builtin_amdgcn_perm(i1, i0, 0x0c0c0400u);   // bytes: i0.b0, i1.b0, 0, 0
      const uint32_t hi = __builtin_amdgcn_perm(i3, i2, 0x04000c0cu);   // bytes: 0, 0, i2.b0, i3.b0
      w[q] = lo | hi;
    }
  }
  return w;
}

// Quantise one row of K and one row of V (D elements each) with D / 16
// lanes per row, 16 elements per lane: the row maximum is reduced across the
// row's lanes (every lane of the wave takes part in the exchange), then codes
// and scales are written when `store`.  Rows with load == false but
// store == true are padding: scale 0, codes 0.
template <typename E, int D>
__device__ __forceinline__ void quant_rows(const E* srck, const E* srcv, bool load, bool store, int l,
                                           int8_t* dk, int8_t* dv, float* sk_out, float* sv_out) {
  constexpr int LPR = D / kQ8Elems;
  float xk[kQ8Elems], xv[kQ8Elems];
#pragma unroll
  for (int j = 0; j < kQ8Elems; ++j) { xk[j] = 0.f; xv[j] = 0.f; }
  if (load) {
    load16(srck + l * kQ8Elems, xk);
    load16(srcv + l * kQ8Elems, xv);
  }
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int j = 0; j < kQ8Elems; ++j) { mk = fmaxf(mk, fabsf(xk[j])); mv = fmaxf(mv, fabsf(xv[j])); }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, off));
    mv = fmaxf(mv, __shfl_xor(mv, off));
  }
  const float sk = mk / 127.f, sv = mv / 127.f;
  if (store) {
    *reinterpret_cast<u32x4*>(dk + l * kQ8Elems) = quantize16(xk, sk);
    *reinterpret_cast<u32x4*>(dv + l * kQ8Elems) = quantize16(xv, sv);
    if (l == 0) {
      *sk_out = sk;
      *sv_out = sv;
    }
  }
}

// Two packed rows per lane group, their loads issued together (more loads in
// flight per thread).
template <typename E, int D>
__global__ __launch_bounds__(256) void moda_pack_depth_q8_kernel(PackQ8Params p) {
  constexpr int LPR = D / kQ8Elems;             // lanes per packed row
  constexpr int RPB = 256 / LPR;                // rows per workgroup and pass
  // consecutive workgroups: the same rows of consecutive (b, kv head) planes,
  // so that together they read consecutive bytes of [B, T, L_d, Hkv, d]
  const int planes = p.B * p.Hkv;
  const int bh = (int)(blockIdx.x % planes);    // (b, kv head) plane
  const long long rblk = p.rb0 + blockIdx.x / planes;   // block of 2 * RPB packed rows
  const int l = threadIdx.x % LPR;
  const int b = bh / p.Hkv, kvh = bh - b * p.Hkv;
  float xk[2][kQ8Elems], xv[2][kQ8Elems];
  bool in_plane[2];
  long long dst[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const long long nl = (rblk * 2 + u) * RPB + (int)threadIdx.x / LPR;   // packed row in the plane
    in_plane[u] = nl < p.NKp;
    const int n = in_plane[u] ? (int)nl : 0;
    dst[u] = (long long)bh * p.NKp + (in_plane[u] ? n : 0);
#pragma unroll
    for (int j = 0; j < kQ8Elems; ++j) { xk[u][j] = 0.f; xv[u][j] = 0.f; }
    if (in_plane[u] && n < p.T * p.L_d) {
      const int t = div_g(n, p.ld_magic, p.ld_shift), jj = n - t * p.L_d;
      const long long src = ((((long long)b * p.T + t) * p.L_d + jj) * p.Hkv + kvh) * D + l * kQ8Elems;
      load16(reinterpret_cast<const E*>(p.kd) + src, xk[u]);
      load16(reinterpret_cast<const E*>(p.vd) + src, xv[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float mk = 0.f, mv = 0.f;
#pragma unroll
    for (int j = 0; j < kQ8Elems; ++j) { mk = fmaxf(mk, fabsf(xk[u][j])); mv = fmaxf(mv, fabsf(xv[u][j])); }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) {
      mk = fmaxf(mk, __shfl_xor(mk, off));
      mv = fmaxf(mv, __shfl_xor(mv, off));
    }
    const float sk = mk / 127.f, sv = mv / 127.f;
    if (in_plane[u]) {
      *reinterpret_cast<u32x4*>(p.kq + dst[u] * D + l * kQ8Elems) = quantize16(xk[u], sk);
      *reinterpret_cast<u32x4*>(p.vq + dst[u] * D + l * kQ8Elems) = quantize16(xv[u], sv);
      if (l == 0) {
        p.ks[dst[u]] = sk;
        p.vs[dst[u]] = sv;
      }
    }
  }
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
  constexpr int LPR = D / kQ8Elems;
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
