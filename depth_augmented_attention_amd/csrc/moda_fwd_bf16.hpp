// Fused MoDA forward, bf16 inputs, for gfx950 (CDNA4).
//
// Same computation and row folding as the generic kernel in moda_fwd.hpp (see
// the description there); this variant is laid out for the gfx950 memory
// path:
//   * K and V blocks are double-buffered in LDS: block j+1 is fetched into
//     registers while block j is computed, then written to the other LDS
//     stage; one workgroup barrier per block.
//   * V stays key-major in LDS; the P.V product reads it with the LDS
//     transpose load (ds_read_b64_tr_b16), which hands each lane four
//     consecutive keys of one head dimension -- the operand order the matrix
//     cores want -- without any shuffles.
//   * LDS rows are 256 bytes with no padding; bank conflicts are avoided by an
//     XOR swizzle of the 16-byte chunk index (K: chunk ^ (row & 15);
//     V: chunk ^ 4 * (row & 3)), chosen so that every 16-lane K read and every
//     32-lane transposed V read touches 64 distinct banks.
//   * At most 256 registers per wave, so two workgroups share a compute unit
//     and one wave's softmax overlaps the other's matrix-core work.
//   * The running max is only moved (and O rescaled) when a new score exceeds
//     it by more than 2^8; until then probabilities are taken against the
//     stale max, which changes nothing in exact arithmetic (out = O / l and
//     lse = m + log2 l use the same m) and keeps them <= 256.
#pragma once

#include "moda_common.hpp"
#include "moda_fwd.hpp"

namespace moda {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// Online-softmax step with a lazily moved max (threshold 8 in log2 units).
template <int NV, int NDT>
__device__ __forceinline__ void online_update_lazy(float (&sv)[NV], float& m_run, float& l_run,
                                                   f32x16 (&o)[NDT]) {
  float mx = sv[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) mx = fmaxf(mx, sv[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__any(mx > m_run + 8.f)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    m_run = m_new;
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    sv[i] = __builtin_amdgcn_exp2f(sv[i] - m_run);
    sum += sv[i];
  }
  l_run += sum;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moda_fwd_bf16_kernel(FwdParams p) {
  constexpr int NW = 4;
  constexpr int BN = 64;                  // keys per sequence block
  constexpr int NKC = D / 16;             // 16-wide k-chunks over d
  constexpr int NDT = D / 32;             // 32-row tiles of O^T over d
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int TILE = BN * D;            // elements of one K (or V) block
  constexpr int LOADS = TILE / 8 / (NW * 64);   // 16-byte loads per thread per block
  static_assert(CPR == 16 || CPR == 8, "head size 64 or 128");
  static_assert(LOADS * NW * 64 * 8 == TILE, "tile / thread mismatch");

  // [stage][K | V][BN][D]
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH;
  const int tile = p.ntiles - 1 - (int)(blockIdx.x / BH);
  const int b = bh / p.Hkv;
  const int kvh = bh % p.Hkv;
  const int G = p.G;
  const int T = p.T;
  const long long TG = (long long)T * G;

  const long long R0 = (long long)tile * (NW * 32);
  const long long Rw = R0 + wave * 32;
  const long long R = Rw + n;
  const bool row_ok = R < TG;
  const bool wave_active = Rw < TG;
  const int t_row = row_ok ? (int)(R / G) : T - 1;
  const int hq = kvh * G + (row_ok ? (int)(R % G) : 0);
  const int tw_min = wave_active ? (int)(Rw / G) : T - 1;
  const int tw_max = wave_active ? (int)((Rw + 31 < TG ? Rw + 31 : TG - 1) / G) : T - 1;
  const long long Rlast = (R0 + NW * 32 < TG ? R0 + NW * 32 : TG) - 1;
  const int t_last = (int)(Rlast / G);
  const int nblocks = t_last / BN + 1;

  bf16x8 qf[NKC];
  {
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + (((long long)b * T + t_row) * p.Hq + hq) * D + hh * 8;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qf[kc] = row_ok ? load_frag(qp + kc * 16) : bf16x8{};
  }

  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x16{};
  float m_run = -1e30f;
  float l_run = 0.f;

  const long long kstride = (long long)p.Hkv * D;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long long)b * T * p.Hkv + kvh) * D;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long long)b * T * p.Hkv + kvh) * D;

  // Block kb is read from HBM into registers (issued one block ahead) and
  // written to LDS stage st after the current block's compute.  Wave w, load i
  // covers the 1 KB LDS span (i*NW + w); lane l fills 16-byte position l of
  // it, i.e. row r = span * (64 / CPR) + l / CPR, physical chunk l % CPR,
  // which holds the logical chunk physical ^ swizzle(r).
  u32x4 kreg[LOADS], vreg[LOADS];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int span = i * NW + wave;
      const int r = span * (64 / CPR) + lane / CPR;
      const int pc = lane % CPR;
      int s = kb * BN + r;
      s = s < T ? s : T - 1;     // rows past the end: real (finite) data, masked later
      const int ck = pc ^ (r & (CPR - 1));
      const int cv = pc ^ ((4 * (r & 3)) & (CPR - 1));
      kreg[i] = ld16(kbase + (long long)s * kstride + ck * 8);
      vreg[i] = ld16(vbase + (long long)s * kstride + cv * 8);
    }
  };
  auto store_block = [&](int st) {
    bf16* sK = smem + st * 2 * TILE;
    bf16* sV = sK + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int span = i * NW + wave;
      st16(sK + span * 512 + lane * 8, kreg[i]);
      st16(sV + span * 512 + lane * 8, vreg[i]);
    }
  };

  const int key_row = key_row_perm(n);
  const float sl2 = p.scale_log2;
  const int q16 = lane >> 4;        // 16-lane group
  const int j16 = lane & 15;

  load_block(0);
  store_block(0);
  __syncthreads();
  for (int kb = 0; kb < nblocks; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nblocks) load_block(kb + 1);
    const bf16* sK = smem + st * 2 * TILE;
    const bf16* sV = sK + TILE;

    if (wave_active && kb * BN <= tw_max) {
      float sv[32];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x16 acc = f32x16{};
        const int r = sub * 32 + key_row;
        const bf16* krow = sK + r * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const int c = (2 * kc + hh) ^ (r & (CPR - 1));
          acc = mma16(load_frag(krow + c * 8), qf[kc], acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[sub * 16 + i] = acc[i] * sl2;
      }
      if (kb * BN + BN - 1 > tw_min) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * BN + sub * 32 + reg_key(i, hh) > t_row) sv[sub * 16 + i] = -INFINITY;
      }
      online_update_lazy(sv, m_run, l_run, o);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bf16x8 pf;
          to_frag(sv + sub * 16 + c * 8, pf);
          // rows (keys) of the two transposed reads of this lane's 16-lane group
          const int r0 = sub * 32 + c * 16 + 8 * (q16 >> 1) + (j16 >> 2);
          const int r1 = r0 + 4;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int chunk = (dt * 4 + 2 * (q16 & 1) + ((j16 & 3) >> 1)) & (CPR - 1);
            const int half = (j16 & 1) * 4;
            // r0 & 3 == r1 & 3 == (j16 >> 2)
            const int pcv = chunk ^ ((4 * (r0 & 3)) & (CPR - 1));
            const s16x4 lo = lds_read_tr(sV + r0 * D + pcv * 8 + half);
            const s16x4 hi = lds_read_tr(sV + r1 * D + pcv * 8 + half);
            const s16x4 a8[2] = {lo, hi};
            bf16x8 af = *reinterpret_cast<const bf16x8*>(a8);
            o[dt] = mma16(af, pf, o[dt]);
          }
        }
      }
    }
    if (kb + 1 < nblocks) store_block(st ^ 1);
    __syncthreads();
  }

  // ---- depth fold: this wave's positions only (see moda_fwd.hpp) ----
  if (wave_active && p.L_d > 0) {
    const int L_d = p.L_d;
    const long long nlo = (long long)tw_min * L_d;
    const long long nhi = (long long)(tw_max + 1) * L_d;
    const bf16* kdb = reinterpret_cast<const bf16*>(p.kd) + (long long)bh * p.NKp * D;
    const bf16* vdb = reinterpret_cast<const bf16*>(p.vd) + (long long)bh * p.NKp * D;
    for (long long n0 = nlo & ~31LL; n0 < nhi; n0 += 32) {
      f32x16 acc = f32x16{};
      const bf16* krow = kdb + (n0 + key_row) * D + hh * 8;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) acc = mma16(load_frag(krow + kc * 16), qf[kc], acc);
      float sv[16];
      const long long own_lo = (long long)t_row * L_d - n0;
      const long long own_hi = own_lo + L_d;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = reg_key(i, hh);
        sv[i] = (key >= own_lo && key < own_hi) ? acc[i] * sl2 : -INFINITY;
      }
      online_update_lazy(sv, m_run, l_run, o);
      const bf16* vchunk = vdb + n0 * D;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pf;
        to_frag(sv + c * 8, pf);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          o[dt] = mma16(load_frag(vchunk + (dt * 32 + n) * 32 + c * 16 + hh * 8), pf, o[dt]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    bf16* op = reinterpret_cast<bf16*>(p.out) + (((long long)b * T + t_row) * p.Hq + hq) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        store4(op + dt * 32 + g4 * 8 + hh * 4, o[dt][g4 * 4 + 0] * inv, o[dt][g4 * 4 + 1] * inv,
               o[dt][g4 * 4 + 2] * inv, o[dt][g4 * 4 + 3] * inv);
    if (hh == 0 && p.lse)
      p.lse[((long long)b * p.Hq + hq) * T + t_row] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

}  // namespace moda
