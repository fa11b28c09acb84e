// Fused MoDA forward kernel for gfx950.
//
// One workgroup owns BM = 32 * NW query rows of one (batch, kv head).  Rows
// fold GQA: row R of a (b, kvh) pair is position t = R / G, head kvh*G + R % G,
// so the G query heads that share a KV head sit next to each other and share
// one base position (gist.science (de) "Mixture-of-Depths Attention",
// Technische Zusammenfassung section 2, Group-Aware Indexing).  Each wave owns
// 32 consecutive rows.
//
// Per workgroup:
//   1. Q fragments of the wave's 32 rows are loaded once into registers.
//   2. Causal sweep over key blocks of BN = 64 positions: the block's K rows
//      and its V (transposed, d-major) are staged in LDS; each wave computes
//      S^T = K Q^T on the matrix cores (keys down, its 32 queries across, so a
//      lane owns one query and softmax needs one cross-half exchange), applies
//      the causal mask s <= t on the diagonal blocks, updates the running max
//      m, running sum l and accumulator O^T (the online softmax with the three
//      states of the pages' Algorithm 1, mhpn.cn article section 2.2), and
//      accumulates O^T += V^T P^T.
//   3. Depth fold: each wave reads only the depth keys of its own positions
//      (chunk-aware access, gist.science (de) section 2) straight from the
//      packed depth buffers into registers, scores them at the same scale,
//      masks every slot that belongs to another position (depth mask, mhpn.cn
//      article section 2.2), and updates the same m / l / O^T.
//   4. out = O / l, lse = (m + log2 l) * ln 2.
#pragma once

#include "moda_common.hpp"

namespace moda {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* kd;   // packed depth keys   [B][Hkv][NKp][D] (dtype, or int8 codes when q8)
  const void* vd;   // packed depth values [B][Hkv][NKp][D]
  const float* ksc; // q8: float32 scale per packed key row   [B][Hkv][NKp]
  const float* vsc; // q8: float32 scale per packed value row [B][Hkv][NKp]
  int q8;           // depth KV stored as int8 codes + row scales
  void* out;
  float* lse;
  int B, T, Hq, Hkv, G;
  int L_d;          // depth slots read per position (slot_lo .. slot_lo+L_d-1)
  int L_cap;        // slots per position in the packed buffers (key n = t*L_cap + slot)
  int slot_lo;      // first slot read
  int ntiles;       // query tiles per (b, kvh)
  int paired;       // tile order for grids of at most two rounds (query_tile)
  long long NKp;    // padded depth keys per (b, kvh)
  float scale_log2; // log2(e) / sqrt(d)
  // split key ranges (bf16 fast path on small grids only; see
  // moda_fwd_bf16.hpp): the nsplit longest query tiles of each (b, kvh) are
  // swept by two workgroups, each over part of the key blocks, whose partial
  // states meet in `ws`; `cnt` counts the arrivals per (split tile, wave) and
  // is zero before and after every launch.
  int nsplit;       // split tiles per (b, kvh); 0: every tile is whole
  float* ws;        // [BH * nsplit][2 parts][NW waves][66][64] float32 partial states
  uint32_t* cnt;    // [BH * nsplit][NW] arrival counters
  // eight-wave grids of several rounds: this launch's counter slot,
  // [work items taken, waves done], zero before and after the launch; null:
  // work items in blockIdx order
  uint32_t* tick;
};

// Whether the 32 packed depth keys [n0, n0 + 32) hold any slot of the window
// [slot_lo, slot_lo + L_d) of some position (a tile inside one position that
// misses the window is skipped; tiles spanning several positions are kept).
__device__ __forceinline__ bool depth_tile_used(long long n0, int L_cap, int slot_lo, int L_d) {
  const long long t0 = n0 / L_cap, t1 = (n0 + 31) / L_cap;
  if (t0 != t1) return true;
  const long long w0 = t0 * L_cap + slot_lo;
  return w0 < n0 + 32 && w0 + L_d > n0;
}

// Rows of the 32-key depth tile at packed key n0 that hold a slot of the
// window [slot_lo, slot_lo + L_d) of a position t < T: bit r for key n0 + r
// (a wave-wide vote; n0 + 31 < 2^31, checked at the boundary).  Every row
// outside the window gets probability 0, but 0 * x is NaN for a non-finite x,
// so the values (and, in the backward, the keys) of unread slots and of the
// padding rows past T * L_cap are zeroed before they reach a product.  Only
// needed when the window leaves slots out or the tile runs past the last key.
__device__ __forceinline__ bool depth_tile_partial(long long n0, int L_cap, int slot_lo, int L_d, int T) {
  return slot_lo != 0 || L_d != L_cap || n0 + 32 > (long long)T * L_cap;
}
__device__ __forceinline__ uint32_t depth_tile_rows(long long n0, int L_cap, int slot_lo, int L_d, int T, int lane) {
  const uint32_t n = (uint32_t)n0 + (uint32_t)(lane & 31);
  const uint32_t slot = n % (uint32_t)L_cap;
  const bool ok = n / (uint32_t)L_cap < (uint32_t)T && slot - (uint32_t)slot_lo < (uint32_t)L_d;
  return (uint32_t)__ballot(ok);
}

// Query tile of workgroup slot s = blockIdx / (B * Hkv).  Longest tiles
// (latest positions, most keys) first; with `paired` set (a grid that the GPU
// runs in at most two rounds, two workgroups per compute unit) the second
// half of the slots takes the tiles in ascending order instead, so that the
// two workgroups that share a compute unit -- slots s and s + ntiles / 2 --
// have lengths adding up to about the same for every compute unit.
__device__ __forceinline__ int query_tile(int s, int ntiles, int paired) {
  const int h = (ntiles + 1) / 2;
  if (!paired || s < h) return ntiles - 1 - s;
  return s - h;
}

// Online-softmax step over NV new scores (log2 units, masked ones -inf) held
// by this lane for its query; the other lane half holds the rest of the
// block.  Updates the running max m and sum l, rescales O^T, and turns sv
// into unnormalised probabilities 2^(s - m), rounded to the element type E
// that enters the P.V product, so that l sums exactly the weights applied.
template <typename E, int NV, int NDT>
__device__ __forceinline__ void online_update(float (&sv)[NV], float& m_run, float& l_run,
                                              f32x16 (&o)[NDT]) {
  float mx = sv[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) mx = fmaxf(mx, sv[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    sv[i] = (float)(E)__builtin_amdgcn_exp2f(sv[i] - m_new);
    sum += sv[i];
  }
  l_run = l_run * alpha + sum;
  m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
}

template <typename E, int D, int NW>
__global__ __launch_bounds__(NW * 64) void moda_fwd_kernel(FwdParams p) {
  using Frag = typename Traits<E>::Frag;
  constexpr int BN = 64;                 // keys per sequence block
  constexpr int VE = Traits<E>::VE;      // elements per 16 bytes
  constexpr int KLD = D + VE;            // LDS row stride of K (16 B pad)
  constexpr int VLD = BN + VE;           // LDS row stride of V^T (16 B pad)
  constexpr int NKC = D / 16;            // 16-wide k-chunks over d
  constexpr int NDT = D / 32;            // 32-row tiles of O^T over d
  constexpr int NT = NW * 64;            // threads
  constexpr int KCH = BN * D / VE;       // 16-byte chunks in a K block
  constexpr int K_PER_T = KCH / NT;
  constexpr int VUNITS = BN * D / (4 * VE);  // (4 keys x VE dims) units
  constexpr int V_PER_T = (VUNITS + NT - 1) / NT;
  static_assert(KCH % NT == 0 && (VUNITS % NT == 0 || VUNITS < NT), "tile / thread mismatch");

  __shared__ __attribute__((aligned(16))) E sK[BN * KLD];
  __shared__ __attribute__((aligned(16))) E sVt[D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;     // query column of this lane in S^T / O^T
  const int hh = lane >> 5;    // lane half

  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH;
  const int tile = query_tile((int)(blockIdx.x / BH), p.ntiles, p.paired);
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

  // ---- Q fragments (B operand of S^T = K Q^T) ----
  Frag qf[NKC];
  {
    const E* qp = reinterpret_cast<const E*>(p.q) + (((long long)b * T + t_row) * p.Hq + hq) * D + hh * 8;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qf[kc] = row_ok ? load_frag(qp + kc * 16) : zero_frag<Frag>();
  }

  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x16{};
  float m_run = -1e30f;   // running max, log2 units
  float l_run = 0.f;      // running sum (this lane's keys only)

  const long long kstride = (long long)p.Hkv * D;   // elements between positions
  const E* kbase = reinterpret_cast<const E*>(p.k) + ((long long)b * T * p.Hkv + kvh) * D;
  const E* vbase = reinterpret_cast<const E*>(p.v) + ((long long)b * T * p.Hkv + kvh) * D;

  // register staging for the next block
  u32x4 kreg[K_PER_T];
  u32x4 vreg[V_PER_T][4];

  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / VE), col = c % (D / VE);
      const int s = kb * BN + row;
      kreg[i] = s < T ? ld16(kbase + (long long)s * kstride + col * VE) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * NT;
      const int kg = u % (BN / 4), dc = u / (BN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = kb * BN + kg * 4 + r;
        vreg[i][r] = (u < VUNITS && s < T) ? ld16(vbase + (long long)s * kstride + dc * VE)
                                           : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / VE), col = c % (D / VE);
      st16(sK + row * KLD + col * VE, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * NT;
      const int kg = u % (BN / 4), dc = u / (BN / 4);
      if (u >= VUNITS) continue;
      if constexpr (sizeof(E) == 2) {
        // 4 keys x 8 dims -> 8 rows of V^T, 4 consecutive keys (8 bytes) each
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint32_t sel = s ? 0x07060302u : 0x05040100u;
            u32x2 val;
            val[0] = __builtin_amdgcn_perm(vreg[i][1][w], vreg[i][0][w], sel);
            val[1] = __builtin_amdgcn_perm(vreg[i][3][w], vreg[i][2][w], sel);
            *reinterpret_cast<u32x2*>(sVt + (dc * VE + 2 * w + s) * VLD + kg * 4) = val;
          }
        }
      } else {
        // 4 keys x 4 dims -> 4 rows of V^T, 4 consecutive keys (16 bytes) each
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 val = {vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
          st16(sVt + (dc * VE + e) * VLD + kg * 4, val);
        }
      }
    }
  };

  const int key_row = key_row_perm(n);
  const float sl2 = p.scale_log2;

  load_block(0);
  for (int kb = 0; kb < nblocks; ++kb) {
    __syncthreads();
    store_block();
    __syncthreads();
    if (kb + 1 < nblocks) load_block(kb + 1);

    if (wave_active && kb * BN <= tw_max) {
      float sv[32];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x16 acc = f32x16{};
        const E* krow = sK + (st * 32 + key_row) * KLD + hh * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) acc = mma16(load_frag(krow + kc * 16), qf[kc], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[st * 16 + r] = acc[r] * sl2;
      }
      if (kb * BN + BN - 1 > tw_min) {   // block crosses the diagonal of some row
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * BN + st * 32 + reg_key(r, hh) > t_row) sv[st * 16 + r] = -INFINITY;
      }
      online_update<E>(sv, m_run, l_run, o);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          Frag pf;
          to_frag(sv + st * 16 + c * 8, pf);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const E* vrow = sVt + (dt * 32 + n) * VLD + st * 32 + c * 16 + hh * 8;
            o[dt] = mma16(load_frag(vrow), pf, o[dt]);
          }
        }
      }
    }
  }

  // ---- depth fold: this wave's positions only ----
  if (wave_active && p.L_d > 0) {
    const int L_d = p.L_d, L_cap = p.L_cap, slot_lo = p.slot_lo;
    const long long nlo = (long long)tw_min * L_cap + slot_lo;
    const long long nhi = (long long)tw_max * L_cap + slot_lo + L_d;
    const E* kdb = reinterpret_cast<const E*>(p.kd) + (long long)bh * p.NKp * D;
    const E* vdb = reinterpret_cast<const E*>(p.vd) + (long long)bh * p.NKp * D;
    for (long long n0 = nlo & ~31LL; n0 < nhi; n0 += 32) {
      if (!depth_tile_used(n0, L_cap, slot_lo, L_d)) continue;
      f32x16 acc = f32x16{};
      if (p.q8) {
        const long long kr = (long long)bh * p.NKp + n0 + key_row;
        const int8_t* krow = reinterpret_cast<const int8_t*>(p.kd) + kr * D + hh * 8;
        const float ks = p.ksc[kr];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) acc = mma16(Dequant<E>::frag(krow + kc * 16, ks), qf[kc], acc);
      } else {
        const E* krow = kdb + (n0 + key_row) * D + hh * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) acc = mma16(load_frag(krow + kc * 16), qf[kc], acc);
      }
      float sv[16];
      const long long own_lo = (long long)t_row * L_cap + slot_lo - n0;   // this row's slots,
      const long long own_hi = own_lo + L_d;                              // relative to n0
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = reg_key(r, hh);
        sv[r] = (key >= own_lo && key < own_hi) ? acc[r] * sl2 : -INFINITY;
      }
      online_update<E>(sv, m_run, l_run, o);
      // rows of this tile that may be read (all of them unless the window
      // leaves slots out or the tile runs past the last key)
      const uint32_t rows_ok = depth_tile_partial(n0, L_cap, slot_lo, L_d, T)
                                   ? depth_tile_rows(n0, L_cap, slot_lo, L_d, T, lane) : 0xffffffffu;
      // V^T operand: 8 consecutive keys of head dimension dt*32 + n, gathered
      // from the key-major packed rows
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag pf;
        to_frag(sv + c * 8, pf);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          Frag vt;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const long long key = n0 + c * 16 + hh * 8 + j;
            if (p.q8) {
              const long long vr = (long long)bh * p.NKp + key;
              vt[j] = Dequant<E>::one(reinterpret_cast<const int8_t*>(p.vd)[vr * D + dt * 32 + n], p.vsc[vr]);
            } else {
              vt[j] = vdb[key * D + dt * 32 + n];
            }
            if (!((rows_ok >> (c * 16 + hh * 8 + j)) & 1u)) vt[j] = (E)0.f;
          }
          o[dt] = mma16(vt, pf, o[dt]);
        }
      }
    }
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    E* op = reinterpret_cast<E*>(p.out) + (((long long)b * T + t_row) * p.Hq + hq) * D;
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
