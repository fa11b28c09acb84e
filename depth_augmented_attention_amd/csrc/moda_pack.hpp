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
//   k_packed [B][Hkv][NKp][D]          rows of d elements
//   v_packed [B][Hkv][NKp/32][D][32]   32-key chunks stored d-major
// with zero rows for n >= T * L_d.  One workgroup handles one 32-key chunk:
// it reads 32 rows coalesced, copies the keys through, and transposes the
// values through LDS so that both writes are contiguous 8 KB (bf16, d = 128)
// blocks.
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
  constexpr int LD = D + VE;
  __shared__ __attribute__((aligned(16))) E tile[32 * LD];

  const long long nchunks = p.NKp / 32;
  const long long chunk = blockIdx.x % nchunks;
  const int bh = (int)(blockIdx.x / nchunks);
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const long long n0 = chunk * 32;
  const long long nvalid = (long long)p.T * p.L_d;

  const E* kd = reinterpret_cast<const E*>(p.kd);
  const E* vd = reinterpret_cast<const E*>(p.vd);
  E* kp = reinterpret_cast<E*>(p.kp) + ((long long)bh * p.NKp + n0) * D;
  E* vp = reinterpret_cast<E*>(p.vp) + ((long long)bh * p.NKp + n0) * D;

  for (int c = threadIdx.x; c < 32 * D / VE; c += 256) {
    const int row = c / (D / VE), col = c % (D / VE);
    const long long key = n0 + row;
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (key < nvalid) {
      const long long t = key / p.L_d, j = key % p.L_d;
      const long long src = (((long long)b * p.T + t) * p.L_d + j) * p.Hkv * D + (long long)kvh * D + col * VE;
      kv = ld16(kd + src);
      vv = ld16(vd + src);
    }
    st16(kp + row * D + col * VE, kv);
    st16(tile + row * LD + col * VE, vv);
  }
  __syncthreads();
  // values: [D][32] -- each thread writes VE consecutive keys of one dim
  for (int c = threadIdx.x; c < D * 32 / VE; c += 256) {
    const int dim = c / (32 / VE), k0 = (c % (32 / VE)) * VE;
    E vals[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) vals[e] = tile[(k0 + e) * LD + dim];
    st16(vp + dim * 32 + k0, *reinterpret_cast<const u32x4*>(vals));
  }
}

}  // namespace moda

namespace moda {

// Write step: one layer's K/V of every position into one slot of the packed
// depth buffers (the layer appends its KV to the depth stream that later
// layers read -- gist.science (de) "Mixture-of-Depths Attention", Technische
// Zusammenfassung section 2, Write-Step).  Same packed layout as
// moda_pack_depth_kernel with L_cap slots per position:
//   k_packed[b][kvh][t * L_cap + slot][:]   = k_new[b][t][kvh][:]
//   v_packed[b][kvh][n / 32][e][n % 32]      = v_new[b][t][kvh][e],  n = t * L_cap + slot
// One thread per 16-byte chunk of one (b, t, kvh) row: the key chunk is one
// 16-byte store, the value chunk VE strided element stores.
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
  st16(kd, ld16(ks));
  E vals[VE];
  *reinterpret_cast<u32x4*>(vals) = ld16(vs);
  E* vd = reinterpret_cast<E*>(p.vp) + bh * p.NKp * D + (n / 32) * D * 32 + (n % 32);
#pragma unroll
  for (int e = 0; e < VE; ++e) vd[(c * VE + e) * 32] = vals[e];
}

}  // namespace moda
