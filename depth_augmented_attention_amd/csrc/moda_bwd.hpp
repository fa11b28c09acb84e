// MoDA backward kernels for gfx950.
//
// The forward is one softmax over the causal sequence keys s <= t of the
// current layer joined with the depth slots of the same position t (mhpn.cn
// article "动态混合深度注意力机制MoDA技术解析", section 1.2 formula and section
// 2.2 masks).  Its gradients, for dO = dL/dout, with z the scaled scores,
// P = exp(z - lse) the probabilities the forward used and
// Delta = rowsum(dO * out) (the softmax Jacobian term sum_j P_j dP_j):
//   dV_j = sum_i P_ij dO_i          dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - Delta_i)  dQ_i = scale sum_j dS_ij k_j
//   dK_j = scale sum_i dS_ij q_i
// Four kernels, all on the caller's stream in this order:
//   moda_bwd_delta_kernel  -Delta and -lse*sqrt(d), two [B,Hq,T] planes of a
//                          float32 work buffer; they seed the dP and S
//                          accumulators of the kernels below, so that the
//                          products come out as dP - Delta and as scores
//                          already shifted by lse.
//   moda_bwd_dq_kernel     one workgroup per query tile (rows fold GQA as in
//                          the forward: row R is position R / G, head
//                          kvh*G + R % G); sweeps the causal key blocks like
//                          the forward, recomputing P from lse, and folds in
//                          the row's own depth slots; writes dq.
//   moda_bwd_dkdv_kernel   one workgroup per 128 sequence keys of one
//                          (b, kv head); sweeps every query row at or after
//                          the keys' positions (all G heads); writes dk_seq,
//                          dv_seq.  No atomics: each key has one writer.
//   moda_bwd_depth_kernel  one workgroup per (b, t, kv head): the depth slots
//                          of position t are seen only by the G heads at t
//                          (the depth mask), so their gradients are local to
//                          that group; writes dk_depth, dv_depth in the
//                          logical [B,T,L_d,Hkv,d] layout.
// The products run on the matrix cores with float32 accumulation in the
// transposed orientation of the forward (a lane owns one query, or one key);
// probabilities and dS enter them in the input precision.
#pragma once

#include <utility>

#include "moda_bwd_split.hpp"
#include "moda_common.hpp"
#include "moda_fwd.hpp"        // depth_tile_used
#include "moda_fwd_bf16.hpp"   // direct-to-LDS loads, LDS transpose reads

namespace moda {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* kd;      // packed depth keys   [B][Hkv][NKp][D] (dtype, or int8 codes when q8)
  const void* vd;      // packed depth values [B][Hkv][NKp][D]
  const float* ksc;    // q8: float32 scale per packed key row   [B][Hkv][NKp]
  const float* vsc;    // q8: float32 scale per packed value row [B][Hkv][NKp]
  int q8;              // depth KV stored as int8 codes + row scales
  const void* o;       // forward output [B,T,Hq,D]
  const void* dO;      // gradient of the output [B,T,Hq,D]
  const float* lse;    // forward lse [B,Hq,T] (natural log)
  float* work;         // [2][B,Hq,T]: -Delta, then -lse*sqrt(d); written by the first kernel
  long long BHT;       // B * Hq * T (plane size of work)
  void* dq;            // [B,T,Hq,D]
  void* dk;            // [B,T,Hkv,D]
  void* dv;
  void* dkd;           // [B,T,L_d,Hkv,D]
  void* dvd;
  int B, T, Hq, Hkv, G;
  int L_d, L_cap, slot_lo;
  int ntiles;          // query tiles per (b, kvh)
  int nktiles;         // key tiles per (b, kvh)
  long long NKp;
  float scale;         // 1 / sqrt(d)
  float scale_log2;    // log2(e) / sqrt(d)
  uint32_t g_magic;    // x / G == (x * g_magic) >> g_shift for 0 <= x < 2^31
  int g_shift;
  // row-split dK/dV (short sequences): each key tile's query blocks are cut
  // into chunks of kchunk blocks swept by separate workgroups
  float* part;         // fp32 partial dK / dV, 32768 floats per (chunk, b, kv head)
  int kchunk;          // query blocks per chunk, a multiple of 2G; 0: no split
  int kfull;           // full chunks over all key tiles of one (b, kv head)
  int kitems;          // chunks (full and remainder) of one (b, kv head)
  // grids of several rounds: the launch counter slots of the dQ and the
  // (unsplit) dK/dV kernels, [work items taken, waves done], zero before and
  // after each launch; null: work items in blockIdx order
  uint32_t* tick_dq;
  uint32_t* tick_kv;
};

// Work item of a workgroup, as (b, kv head) pair and index within that
// pair's tiles (0 = heaviest).  With a launch counter slot `tick` (one queue
// counter per pair, then the count of waves done): the workgroup takes the
// next tile of its home pair blockIdx % npairs -- the pair that blockIdx
// order would give it, so that each XCD (the GPU hands workgroups to its
// eight XCDs round-robin by blockIdx) keeps to the q / dO rows of few pairs in
// its L2 -- and once that pair's tiles are all taken, the next tile of the
// following pairs.  XCDs run at different speeds, so a fixed split of the
// grid leaves the fast ones idle at the end; here they take over the slow
// ones' last tiles.  Every workgroup finds a tile: the grid has exactly one
// workgroup per tile, so while one is still looking, some pair has a tile
// left.  Without a slot: blockIdx order.
struct WorkItem {
  int pair, index;
};
__device__ __forceinline__ WorkItem take_work_item(uint32_t* tick, int npairs, int per_pair, uint32_t* s_item) {
  if (!tick) return WorkItem{(int)(blockIdx.x % (uint32_t)npairs), (int)(blockIdx.x / (uint32_t)npairs)};
  if (threadIdx.x == 0) {
    int q = (int)(blockIdx.x % (uint32_t)npairs);
    uint32_t it = 0;
    for (int k = 0; k < npairs; ++k) {
      it = __hip_atomic_fetch_add(tick + q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (it < (uint32_t)per_pair) break;
      q = q + 1 == npairs ? 0 : q + 1;
    }
    *s_item = (uint32_t)q * (uint32_t)per_pair + it;
  }
  __syncthreads();
  const uint32_t v = *s_item;
  return WorkItem{(int)(v / (uint32_t)per_pair), (int)(v % (uint32_t)per_pair)};
}
// Each wave counts itself out once its work is written (in the slot's last
// word); the last wave of the launch returns the slot to zero (every
// workgroup has taken its tile before any of its waves gets here).
constexpr int kTickWords = 16;   // words per counter slot: up to 15 pairs, then the count
__device__ __forceinline__ void release_work_slot(uint32_t* tick, int npairs, int waves_per_group) {
  if (!tick || (threadIdx.x & 63) != 0) return;
  const uint32_t done = __hip_atomic_fetch_add(tick + kTickWords - 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (done == gridDim.x * (uint32_t)waves_per_group - 1u) {
    for (int q = 0; q < npairs; ++q) __hip_atomic_store(tick + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(tick + kTickWords - 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

constexpr float kLog2e = 1.4426950408889634f;


// Four rows x VE elements (v[r] = VE consecutive elements of row row0 + r,
// starting at element e0) written transposed: sT[(e0 + e) * LDT + row0 + r].
template <typename E, int LDT>
__device__ __forceinline__ void store_t4(E* sT, int e0, int row0, const u32x4 (&v)[4]) {
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t sel = s ? 0x07060302u : 0x05040100u;
        u32x2 val;
        val[0] = __builtin_amdgcn_perm(v[1][w], v[0][w], sel);
        val[1] = __builtin_amdgcn_perm(v[3][w], v[2][w], sel);
        *reinterpret_cast<u32x2*>(sT + (e0 + 2 * w + s) * LDT + row0) = val;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 val = {v[0][e], v[1][e], v[2][e], v[3][e]};
      st16(sT + (e0 + e) * LDT + row0, val);
    }
  }
}

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * out), one 16-byte chunk per thread; stores -Delta and
// -lse / scale (= -lse * sqrt(d)).
template <typename E, int D>
__global__ __launch_bounds__(256) void moda_bwd_delta_kernel(BwdParams p) {
  constexpr int VE = Traits<E>::VE;
  constexpr int CPR = D / VE;         // chunks per row (8 or 16)
  constexpr int RPB = 256 / CPR;      // rows per workgroup
  const long long rows = (long long)p.B * p.T * p.Hq;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  float s = 0.f;
  if (row < rows) {
    E o[VE], g[VE];
    *reinterpret_cast<u32x4*>(o) = ld16(reinterpret_cast<const E*>(p.o) + row * D + c * VE);
    *reinterpret_cast<u32x4*>(g) = ld16(reinterpret_cast<const E*>(p.dO) + row * D + c * VE);
#pragma unroll
    for (int e = 0; e < VE; ++e) s += (float)o[e] * (float)g[e];
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && c == 0) {
    const int h = (int)(row % p.Hq);
    const long long bt = row / p.Hq;
    const int t = (int)(bt % p.T);
    const int b = (int)(bt / p.T);
    const long long i = ((long long)b * p.Hq + h) * p.T + t;
    p.work[i] = -s;
    p.work[p.BHT + i] = -p.lse[i] / p.scale;
  }
}

// Depth slots of one wave's positions [tw_min, tw_max] for dQ: the same
// three products on 32-key tiles of the packed buffers, read straight from
// memory (key-major rows for the score and dP products; the key-transposed
// operand of dQ is gathered).  Rows see only their own position's slots.
template <typename E, int D, typename Frag>
__device__ __forceinline__ void dq_depth_fold(const BwdParams& p, int bh, int tw_min, int tw_max, int t_row,
                                              int n, int hh, int key_row, const Frag (&qf)[D / 16],
                                              const Frag (&df)[D / 16], float lse2, float dlt,
                                              f32x16 (&acc)[D / 32]) {
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  const float sl2 = p.scale_log2;
  const int L_d = p.L_d, L_cap = p.L_cap, slot_lo = p.slot_lo;
  const long long nlo = (long long)tw_min * L_cap + slot_lo;
  const long long nhi = (long long)tw_max * L_cap + slot_lo + L_d;
  const E* kdb = reinterpret_cast<const E*>(p.kd) + (long long)bh * p.NKp * D;
  const E* vdb = reinterpret_cast<const E*>(p.vd) + (long long)bh * p.NKp * D;
  // 8-bit depth KV: codes and row scales of this (b, kv head)
  const int8_t* kq8 = reinterpret_cast<const int8_t*>(p.kd) + (long long)bh * p.NKp * D;
  const int8_t* vq8 = reinterpret_cast<const int8_t*>(p.vd) + (long long)bh * p.NKp * D;
  const float* ks8 = p.q8 ? p.ksc + (long long)bh * p.NKp : nullptr;
  const float* vs8 = p.q8 ? p.vsc + (long long)bh * p.NKp : nullptr;
  for (long long n0 = nlo & ~31LL; n0 < nhi; n0 += 32) {
    if (!depth_tile_used(n0, L_cap, slot_lo, L_d)) continue;
    f32x16 s = f32x16{}, dp = f32x16{};
    if (p.q8) {
      const long long kr = n0 + key_row;
      const float ks = ks8[kr], vs = vs8[kr];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s = mma16(Dequant<E>::frag(kq8 + kr * D + hh * 8 + kc * 16, ks), qf[kc], s);
        dp = mma16(Dequant<E>::frag(vq8 + kr * D + hh * 8 + kc * 16, vs), df[kc], dp);
      }
    } else {
      const E* krow = kdb + (n0 + key_row) * D + hh * 8;
      const E* vrow = vdb + (n0 + key_row) * D + hh * 8;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s = mma16(load_frag(krow + kc * 16), qf[kc], s);
        dp = mma16(load_frag(vrow + kc * 16), df[kc], dp);
      }
    }
    const long long own_lo = (long long)t_row * L_cap + slot_lo - n0;
    const long long own_hi = own_lo + L_d;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = reg_key(r, hh);
      const bool own = key >= own_lo && key < own_hi;
      const float pr = __builtin_amdgcn_exp2f(own ? s[r] * sl2 - lse2 : -INFINITY);
      // a masked key contributes exactly 0 (its dP may be non-finite when the
      // slot is unread)
      ds[r] = own ? pr * (dp[r] - dlt) : 0.f;
    }
    // keys of unread slots (and padding) are zeroed in the dQ operand: their
    // dS is 0, and 0 * x would still carry a non-finite x into dQ
    const uint32_t rows_ok = depth_tile_partial(n0, L_cap, slot_lo, L_d, p.T)
                                 ? depth_tile_rows(n0, L_cap, slot_lo, L_d, p.T, n + 32 * hh) : 0xffffffffu;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      Frag f;
      to_frag(ds + c * 8, f);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        Frag kt;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const long long r = n0 + c * 16 + hh * 8 + j;
          kt[j] = p.q8 ? Dequant<E>::one(kq8[r * D + dt * 32 + n], ks8[r]) : kdb[r * D + dt * 32 + n];
          if (!((rows_ok >> (c * 16 + hh * 8 + j)) & 1u)) kt[j] = (E)0.f;
        }
        acc[dt] = mma16(kt, f, acc[dt]);
      }
    }
  }
}

// dq = scale * dQ^T accumulator of one lane's row.
template <typename E, int D>
__device__ __forceinline__ void dq_store(const BwdParams& p, int b, int t_row, int hq, int hh,
                                         const f32x16 (&acc)[D / 32]) {
  const float sc = p.scale;
  E* op = reinterpret_cast<E*>(p.dq) + (((long long)b * p.T + t_row) * p.Hq + hq) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      store4(op + dt * 32 + g4 * 8 + hh * 4, acc[dt][g4 * 4 + 0] * sc, acc[dt][g4 * 4 + 1] * sc,
             acc[dt][g4 * 4 + 2] * sc, acc[dt][g4 * 4 + 3] * sc);
}

// ---------------------------------------------------------------------------
// dQ: per query tile, S^T = K Q^T and dP^T = V dO^T per 32-key half, then
// dQ^T += K^T dS^T.  K is staged key-major (score operand) and transposed
// (dQ operand); V key-major.
template <typename E, int D, int NW>
__global__ __launch_bounds__(NW * 64) void moda_bwd_dq_kernel(BwdParams p) {
  using Frag = typename Traits<E>::Frag;
  constexpr int BN = 64;
  constexpr int VE = Traits<E>::VE;
  constexpr int KLD = D + VE;          // key-major row stride (16 B pad)
  constexpr int TLD = BN + VE;         // transposed row stride (16 B pad)
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NT = NW * 64;
  constexpr int NU = BN * D / (4 * VE);   // units of 4 rows x 16 bytes per block
  constexpr int UPT = (NU + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) E sK[BN * KLD];
  __shared__ __attribute__((aligned(16))) E sV[BN * KLD];
  __shared__ __attribute__((aligned(16))) E sKt[D * TLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH;
  const int tile = p.ntiles - 1 - (int)(blockIdx.x / BH);   // heaviest first
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
  const int nblocks = (int)(Rlast / G) / BN + 1;

  const long long qrow = (((long long)b * T + t_row) * p.Hq + hq) * D + hh * 8;
  Frag qf[NKC], df[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    qf[kc] = row_ok ? load_frag(reinterpret_cast<const E*>(p.q) + qrow + kc * 16) : zero_frag<Frag>();
    df[kc] = row_ok ? load_frag(reinterpret_cast<const E*>(p.dO) + qrow + kc * 16) : zero_frag<Frag>();
  }
  const long long lrow = ((long long)b * p.Hq + hq) * T + t_row;
  const float lse2 = row_ok ? p.lse[lrow] * kLog2e : INFINITY;   // P = 0 on rows past the end
  const float dlt = row_ok ? -p.work[lrow] : 0.f;
  const float sl2 = p.scale_log2;

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16{};

  const long long kstride = (long long)p.Hkv * D;
  const E* kbase = reinterpret_cast<const E*>(p.k) + ((long long)b * T * p.Hkv + kvh) * D;
  const E* vbase = reinterpret_cast<const E*>(p.v) + ((long long)b * T * p.Hkv + kvh) * D;

  u32x4 kreg[UPT][4], vreg[UPT][4];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      const int rg = u % (BN / 4), dc = u / (BN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = kb * BN + rg * 4 + r;
        const bool ok = u < NU && s < T;
        kreg[i][r] = ok ? ld16(kbase + (long long)s * kstride + dc * VE) : u32x4{0, 0, 0, 0};
        vreg[i][r] = ok ? ld16(vbase + (long long)s * kstride + dc * VE) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= NU) continue;
      const int rg = u % (BN / 4), dc = u / (BN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st16(sK + (rg * 4 + r) * KLD + dc * VE, kreg[i][r]);
        st16(sV + (rg * 4 + r) * KLD + dc * VE, vreg[i][r]);
      }
      store_t4<E, TLD>(sKt, dc * VE, rg * 4, kreg[i]);
    }
  };

  const int key_row = key_row_perm(n);

  load_block(0);
  for (int kb = 0; kb < nblocks; ++kb) {
    __syncthreads();
    store_block();
    __syncthreads();
    if (kb + 1 < nblocks) load_block(kb + 1);
    if (!(wave_active && kb * BN <= tw_max)) continue;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const E* krow = sK + (st * 32 + key_row) * KLD + hh * 8;
      const E* vrow = sV + (st * 32 + key_row) * KLD + hh * 8;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s = mma16(load_frag(krow + kc * 16), qf[kc], s);
        dp = mma16(load_frag(vrow + kc * 16), df[kc], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * BN + st * 32 + reg_key(r, hh);
        const float pr = __builtin_amdgcn_exp2f(key <= t_row ? s[r] * sl2 - lse2 : -INFINITY);
        ds[r] = pr * (dp[r] - dlt);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag f;
        to_frag(ds + c * 8, f);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          acc[dt] = mma16(load_frag(sKt + (dt * 32 + n) * TLD + st * 32 + c * 16 + hh * 8), f, acc[dt]);
      }
    }
  }

  if (wave_active && p.L_d > 0)
    dq_depth_fold<E, D>(p, bh, tw_min, tw_max, t_row, n, hh, key_row, qf, df, lse2, dlt, acc);
  if (row_ok) dq_store<E, D>(p, b, t_row, hq, hh, acc);
}

// ---------------------------------------------------------------------------
// dK, dV of the sequence keys: per 32*NW keys of one (b, kvh), every query row
// at or after the keys' first position.  A lane owns one key: S = Q K^T and
// dP = dO V^T per 32-row half (queries down), then dV^T += dO^T P and
// dK^T += Q^T dS.  Q and dO are staged row-major (score operands) and
// transposed (gradient operands).
template <typename E, int D, int NW>
__global__ __launch_bounds__(NW * 64) void moda_bwd_dkdv_kernel(BwdParams p) {
  using Frag = typename Traits<E>::Frag;
  constexpr int QB = 64;               // query rows per block
  constexpr int VE = Traits<E>::VE;
  constexpr int QLD = D + VE;
  constexpr int TLD = QB + VE;
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NT = NW * 64;
  constexpr int NU = QB * D / (4 * VE);
  constexpr int UPT = (NU + NT - 1) / NT;
  static_assert(QB <= NT, "per-row arrays are filled one row per thread");

  __shared__ __attribute__((aligned(16))) E sQ[QB * QLD];
  __shared__ __attribute__((aligned(16))) E sO[QB * QLD];
  __shared__ __attribute__((aligned(16))) E sQt[D * TLD];
  __shared__ __attribute__((aligned(16))) E sOt[D * TLD];
  __shared__ __attribute__((aligned(16))) float sL[QB];
  __shared__ __attribute__((aligned(16))) float sDl[QB];
  __shared__ __attribute__((aligned(16))) int sTq[QB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH;
  const int ktile = (int)(blockIdx.x / BH);     // earliest keys (most rows) first
  const int b = bh / p.Hkv;
  const int kvh = bh % p.Hkv;
  const int G = p.G;
  const int T = p.T;
  const int Hq = p.Hq;
  const int TG = T * G;   // < 2^31 (checked at the boundary)

  const int kt0 = ktile * (NW * 32);
  const int wkey0 = kt0 + wave * 32;
  const int key = wkey0 + n;
  const bool key_ok = key < T;
  const bool wave_keys = wkey0 < T;

  const long long kstride = (long long)p.Hkv * D;
  Frag kf[NKC], vf[NKC];
  {
    const long long krow = ((long long)b * T + (key_ok ? key : 0)) * kstride + (long long)kvh * D + hh * 8;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      kf[kc] = key_ok ? load_frag(reinterpret_cast<const E*>(p.k) + krow + kc * 16) : zero_frag<Frag>();
      vf[kc] = key_ok ? load_frag(reinterpret_cast<const E*>(p.v) + krow + kc * 16) : zero_frag<Frag>();
    }
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  const int rb0 = kt0 * G / QB * QB;   // first block with a row at position >= kt0
  const int nqb = (TG - rb0 + QB - 1) / QB;
  const E* qg = reinterpret_cast<const E*>(p.q);
  const E* og = reinterpret_cast<const E*>(p.dO);

  u32x4 qreg[UPT][4], oreg[UPT][4];
  float l_reg = INFINITY, d_reg = 0.f;
  int t_reg = -1;
  auto load_block = [&](int Rb) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      const int rg = u % (QB / 4), dc = u / (QB / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int Rr = Rb + rg * 4 + r;
        const bool ok = u < NU && Rr < TG;
        const int t = div_g(Rr, p.g_magic, p.g_shift);
        const long long off = ok ? (((long long)b * T + t) * Hq + kvh * G + (Rr - t * G)) * D + dc * VE : 0;
        qreg[i][r] = ok ? ld16(qg + off) : u32x4{0, 0, 0, 0};
        oreg[i][r] = ok ? ld16(og + off) : u32x4{0, 0, 0, 0};
      }
    }
    if (tid < QB) {
      const int Rr = Rb + tid;
      if (Rr < TG) {
        const int t = div_g(Rr, p.g_magic, p.g_shift);
        const long long li = ((long long)b * Hq + kvh * G + (Rr - t * G)) * T + t;
        l_reg = p.lse[li] * kLog2e;
        d_reg = -p.work[li];
        t_reg = t;
      } else {
        l_reg = INFINITY;
        d_reg = 0.f;
        t_reg = -1;
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= NU) continue;
      const int rg = u % (QB / 4), dc = u / (QB / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st16(sQ + (rg * 4 + r) * QLD + dc * VE, qreg[i][r]);
        st16(sO + (rg * 4 + r) * QLD + dc * VE, oreg[i][r]);
      }
      store_t4<E, TLD>(sQt, dc * VE, rg * 4, qreg[i]);
      store_t4<E, TLD>(sOt, dc * VE, rg * 4, oreg[i]);
    }
    if (tid < QB) {
      sL[tid] = l_reg;
      sDl[tid] = d_reg;
      sTq[tid] = t_reg;
    }
  };

  const int qperm = key_row_perm(n);   // operand row m holds query row pi(m)
  const float sl2 = p.scale_log2;

  load_block(rb0);
  for (int qb = 0; qb < nqb; ++qb) {
    const int Rb = rb0 + qb * QB;
    __syncthreads();
    store_block();
    __syncthreads();
    if (qb + 1 < nqb) load_block(Rb + QB);
    if (!wave_keys) continue;
    const int Rend = Rb + QB < TG ? Rb + QB : TG;
    if (div_g(Rend - 1, p.g_magic, p.g_shift) < wkey0) continue;   // every row of the block precedes this wave's keys
#pragma unroll
    for (int sub = 0; sub < QB / 32; ++sub) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const E* qrow = sQ + (sub * 32 + qperm) * QLD + hh * 8;
      const E* orow = sO + (sub * 32 + qperm) * QLD + hh * 8;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s = mma16(load_frag(qrow + kc * 16), kf[kc], s);
        dp = mma16(load_frag(orow + kc * 16), vf[kc], dp);
      }
      // the lane's 16 rows are two runs of 8: sub*32 + 16c + 8hh + (0..7)
      float pv[16], ds[16];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int q0 = sub * 32 + 16 * c + 8 * hh;
        const f32x4 la = *reinterpret_cast<const f32x4*>(sL + q0), lb = *reinterpret_cast<const f32x4*>(sL + q0 + 4);
        const f32x4 da = *reinterpret_cast<const f32x4*>(sDl + q0), db = *reinterpret_cast<const f32x4*>(sDl + q0 + 4);
        const u32x4 ta = *reinterpret_cast<const u32x4*>(sTq + q0), tb = *reinterpret_cast<const u32x4*>(sTq + q0 + 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * c + j;
          const float lr = j < 4 ? la[j] : lb[j - 4];
          const float dr = j < 4 ? da[j] : db[j - 4];
          const int tr = (int)(j < 4 ? ta[j] : tb[j - 4]);
          // masked entries get exponent -inf (select on the argument, no branch)
          const float x = tr >= key ? s[r] * sl2 - lr : -INFINITY;
          const float pr = __builtin_amdgcn_exp2f(x);
          pv[r] = pr;
          ds[r] = pr * (dp[r] - dr);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        Frag fp, fd;
        to_frag(pv + c * 8, fp);
        to_frag(ds + c * 8, fd);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int off = (dt * 32 + n) * TLD + sub * 32 + c * 16 + hh * 8;
          dv[dt] = mma16(load_frag(sOt + off), fp, dv[dt]);
          dk[dt] = mma16(load_frag(sQt + off), fd, dk[dt]);
        }
      }
    }
  }

  if (key_ok) {
    const float sc = p.scale;
    const long long orow = (((long long)b * T + key) * p.Hkv + kvh) * D;
    E* dkp = reinterpret_cast<E*>(p.dk) + orow;
    E* dvp = reinterpret_cast<E*>(p.dv) + orow;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int e = dt * 32 + g4 * 8 + hh * 4;
        store4(dkp + e, dk[dt][g4 * 4 + 0] * sc, dk[dt][g4 * 4 + 1] * sc, dk[dt][g4 * 4 + 2] * sc,
               dk[dt][g4 * 4 + 3] * sc);
        store4(dvp + e, dv[dt][g4 * 4 + 0], dv[dt][g4 * 4 + 1], dv[dt][g4 * 4 + 2], dv[dt][g4 * 4 + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// Depth-slot gradients of one (b, t, kv head): the G query heads at t against
// the L_d slots of t, in float32 on the vector units (the block is
// G x L_d x d, a few hundred thousand multiply-adds).  Slots in chunks of LC,
// heads in chunks of GC.
template <typename E, int D>
__global__ __launch_bounds__(256) void moda_bwd_depth_kernel(BwdParams p) {
  constexpr int GC = 8, LC = 32, LDF = D + 1;   // odd row stride: conflict-free column reads
  constexpr int EPT = D / 8;                    // outputs per thread and tensor: (slot tid/8, dims tid%8 + 8i)
  static_assert(GC * LC == 256, "one (head, slot) pair per thread");
  __shared__ float sq[GC * LDF], sdo[GC * LDF], sk[LC * LDF], sv[LC * LDF];
  __shared__ float sP[GC * LC], sdS[GC * LC], sLs[GC], sDl[GC];

  const int tid = threadIdx.x;
  const int Hkv = p.Hkv, T = p.T, Hq = p.Hq, G = p.G, L_d = p.L_d;
  const int kvh = (int)(blockIdx.x % Hkv);
  const long long bt = blockIdx.x / Hkv;
  const int t = (int)(bt % T);
  const int b = (int)(bt / T);
  const long long bh = (long long)b * Hkv + kvh;
  const E* kdb = reinterpret_cast<const E*>(p.kd) + bh * p.NKp * D;
  const E* vdb = reinterpret_cast<const E*>(p.vd) + bh * p.NKp * D;
  const int8_t* kq8 = reinterpret_cast<const int8_t*>(p.kd) + bh * p.NKp * D;   // q8 codes
  const int8_t* vq8 = reinterpret_cast<const int8_t*>(p.vd) + bh * p.NKp * D;
  const float* ks8 = p.q8 ? p.ksc + bh * p.NKp : nullptr;                      // q8 row scales
  const float* vs8 = p.q8 ? p.vsc + bh * p.NKp : nullptr;
  const E* qg = reinterpret_cast<const E*>(p.q);
  const E* og = reinterpret_cast<const E*>(p.dO);
  const float scale = p.scale;

  for (int j0 = 0; j0 < L_d; j0 += LC) {
    const int nj = L_d - j0 < LC ? L_d - j0 : LC;
    __syncthreads();
    // keys: rows of the packed keys, dims fastest
    for (int i = tid; i < LC * D; i += 256) {
      const int j = i / D, e = i % D;
      float kv = 0.f;
      if (j < nj) {
        const long long r = (long long)t * p.L_cap + p.slot_lo + j0 + j;
        kv = p.q8 ? (float)Dequant<E>::one(kq8[r * D + e], ks8[r]) : (float)kdb[r * D + e];
      }
      sk[j * LDF + e] = kv;
    }
    // values: rows of the packed values, dims fastest
    for (int i = tid; i < LC * D; i += 256) {
      const int j = i / D, e = i % D;
      float vv = 0.f;
      if (j < nj) {
        const long long r = (long long)t * p.L_cap + p.slot_lo + j0 + j;
        vv = p.q8 ? (float)Dequant<E>::one(vq8[r * D + e], vs8[r]) : (float)vdb[r * D + e];
      }
      sv[j * LDF + e] = vv;
    }
    float accK[EPT], accV[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) { accK[i] = 0.f; accV[i] = 0.f; }

    for (int g0 = 0; g0 < G; g0 += GC) {
      const int ng = G - g0 < GC ? G - g0 : GC;
      __syncthreads();
      for (int i = tid; i < GC * D; i += 256) {
        const int g = i / D, e = i % D;
        float qv = 0.f, ov = 0.f;
        if (g < ng) {
          const long long row = (((long long)b * T + t) * Hq + kvh * G + g0 + g) * D + e;
          qv = (float)qg[row];
          ov = (float)og[row];
        }
        sq[g * LDF + e] = qv;
        sdo[g * LDF + e] = ov;
      }
      if (tid < GC) {
        const bool ok = tid < ng;
        const long long li = ((long long)b * Hq + kvh * G + g0 + tid) * T + t;
        sLs[tid] = ok ? p.lse[li] : 0.f;
        sDl[tid] = ok ? -p.work[li] : 0.f;
      }
      __syncthreads();
      {
        const int g = tid / LC, j = tid % LC;
        float s = 0.f, dp = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; ++e) {
          s += sq[g * LDF + e] * sk[j * LDF + e];
          dp += sdo[g * LDF + e] * sv[j * LDF + e];
        }
        const bool ok = g < ng && j < nj;
        const float pr = ok ? __builtin_amdgcn_exp2f((s * scale - sLs[g]) * kLog2e) : 0.f;
        sP[g * LC + j] = pr;
        sdS[g * LC + j] = pr * (dp - sDl[g]);
      }
      __syncthreads();
      {
        const int j = tid / 8, e0 = tid % 8;
#pragma unroll
        for (int g = 0; g < GC; ++g) {
          const float pp = sP[g * LC + j], dd = sdS[g * LC + j];
#pragma unroll
          for (int i = 0; i < EPT; ++i) {
            accV[i] += pp * sdo[g * LDF + e0 + 8 * i];
            accK[i] += dd * sq[g * LDF + e0 + 8 * i];
          }
        }
      }
    }
    {
      const int j = tid / 8, e0 = tid % 8;
      if (j < nj) {
        const long long orow = ((((long long)b * T + t) * L_d + j0 + j) * Hkv + kvh) * D;
        E* dkp = reinterpret_cast<E*>(p.dkd) + orow;
        E* dvp = reinterpret_cast<E*>(p.dvd) + orow;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          dkp[e0 + 8 * i] = (E)(accK[i] * scale);
          dvp[e0 + 8 * i] = (E)accV[i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, d = 128: dK, dV of the sequence keys laid out for the gfx950 memory
// path (same computation as moda_bwd_dkdv_kernel).
//   * Q and dO blocks of 64 rows, with their lse and Delta, go from memory
//     straight into LDS with the direct global->LDS loads (two stages, one
//     barrier per block); rows of the GQA fold are gathered by per-lane
//     offsets, rows past the end read as zeros.  When G divides 64 (GP)
//     every block starts at a whole position, so those offsets are lane
//     constants and the block's position moves the buffer base; otherwise
//     each block's offsets take a multiply-shift division by G.
//   * One copy of each block serves both products: row-major reads for
//     S = Q K^T and dP = dO V^T, and LDS transpose reads (ds_read_b64_tr_b16,
//     through the compiler builtin; the two stages are separate arrays, so
//     reads of one are not held back by loads in flight into the other) for
//     the Q^T and dO^T operands of dK^T and dV^T.  The 16-byte chunk index
//     is XOR-swizzled with 4 (row & 3) + ((row >> 2) & 3), which keeps both
//     access patterns free of bank conflicts: any 16 consecutive rows get 16
//     distinct chunks (row reads), and any 4 consecutive rows get 4 distinct
//     64-byte segments (transpose reads).
//   * The causal mask needs no division: row R (position R / G) sees key s
//     iff R >= s * G.
namespace bwdbf16 {

// physical 16-byte chunk of logical chunk c in row r of a block
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// lane-constant LDS byte offsets of the transpose reads of a 16-row chunk of a
// swizzled [rows][128] bf16 block: 16-lane group q16, lane j16 reads row
// 8 (q16 / 2) + j16 / 4 (+4 for the second half of each fragment), logical
// chunk 4 dt + 2 (q16 & 1) + (j16 & 3) / 2, half j16 & 1; a[2 dt + k4].
__device__ __forceinline__ void tr_offsets(int lane, uint32_t base, uint32_t (&a)[8]) {
  const int q16 = lane >> 4, j16 = lane & 15;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int k4 = 0; k4 < 2; ++k4) {
      const int r = 8 * (q16 >> 1) + (j16 >> 2) + 4 * k4;
      const int lc = 4 * dt + 2 * (q16 & 1) + ((j16 & 3) >> 1);
      a[2 * dt + k4] = base + (uint32_t)(r * 256 + ((lc ^ swz(r)) * 16) + (j16 & 1) * 8);
    }
}

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* ldst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)ldst, 4, voff, 0, 0, 0);
}

}  // namespace bwdbf16

template <int D, bool GP, bool SPLIT = false>
__global__ __launch_bounds__(256) void moda_bwd_dkdv_bf16_kernel(BwdParams p) {
  static_assert(D == 128, "built for head size 128");
  using namespace bwdbf16;
  constexpr int NW = 4;
  constexpr int QB = 64;                       // query rows per block
  constexpr int NSUB = QB / 32;                // 32-row sub-blocks per block
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE_B = QB * D * 2;           // bytes of a Q (or dO) block
  constexpr int OFF_O = TILE_B;                // dO block within a stage
  constexpr int OFF_L = 2 * TILE_B;            // lse[QB] within a stage
  constexpr int OFF_D = 2 * TILE_B + QB * 4;   // Delta[QB] within a stage
  constexpr int STAGE = 2 * TILE_B + 2 * QB * 4;
  constexpr int LOADS = QB * D / 8 / (NW * 64);   // 16-byte loads per lane per tensor per block
  constexpr uint32_t OOB = 0x80000000u;         // an offset past every buffer's range: reads zeros

  // the two stages as separate arrays, so that loads from one provably do not
  // alias the direct-to-LDS writes in flight into the other
  __shared__ __attribute__((aligned(1024))) char smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.Hkv;
  // work item: key tiles of each (b, kv head) pair, earliest keys (most
  // rows, the heaviest) first
  uint32_t* const tick = SPLIT ? nullptr : p.tick_kv;
  __shared__ uint32_t s_item;
  const WorkItem wi = take_work_item(tick, BH, SPLIT ? p.kitems : p.nktiles, &s_item);
  const int bh = wi.pair;
  // SPLIT: blocks [q_lo, q_hi) of the tile's sweep (chunks of the row-split
  // map); otherwise every block
  int ktile = wi.index, q_lo = 0, q_hi = 0, nchunks = 1;
  if constexpr (SPLIT) {
    const BwdChunkMap cm(p.T, p.G, p.kchunk, p.nktiles);
    const int chunk = ktile;
    if (chunk < p.kfull) {
      ktile = cm.full_tile(chunk);
      q_lo = (chunk - cm.prefix(ktile)) * p.kchunk;
      q_hi = q_lo + p.kchunk;
    } else {
      ktile = cm.rem_tile(chunk - p.kfull);
      if (ktile < 0) return;                    // past the map (not launched)
      q_lo = cm.nf(ktile) * p.kchunk;
      q_hi = cm.nqb(ktile);
    }
    nchunks = cm.nchunks(ktile);
  }
  const int b = bh / p.Hkv;
  const int kvh = bh % p.Hkv;
  const int G = p.G;
  const int T = p.T;
  const int Hq = p.Hq;
  const int TG = T * G;

  const int kt0 = ktile * (NW * 32);
  const int wkey0 = kt0 + wave * 32;
  const int key = wkey0 + n;
  const bool key_ok = key < T;
  const int keyG = key * G;                     // rows R >= keyG see this key

  const long long kstride = (long long)p.Hkv * D;
  bf16x8 kf[NKC], vf[NKC];
  {
    const long long krow = ((long long)b * T + (key_ok ? key : 0)) * kstride + (long long)kvh * D + hh * 8;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      kf[kc] = key_ok ? load_frag(reinterpret_cast<const bf16*>(p.k) + krow + kc * 16) : bf16x8{};
      vf[kc] = key_ok ? load_frag(reinterpret_cast<const bf16*>(p.v) + krow + kc * 16) : bf16x8{};
    }
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  // raw buffers over this (b, kv head)'s rows: q / dO from position 0, head kvh*G;
  // lse / Delta from head kvh*G of batch b
  const long long qbase = ((long long)b * T * Hq + (long long)kvh * G) * D;
  const long long lbase = ((long long)b * Hq + (long long)kvh * G) * T;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const bf16*>(p.q) + qbase), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const bf16*>(p.dO) + qbase), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.work + lbase), (short)0, 0x7fffffff, kBufferWord3);          // -Delta
  const __amdgpu_buffer_rsrc_t rl2 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.work + p.BHT + lbase), (short)0, 0x7fffffff, kBufferWord3);  // -lse * sqrt(d)

  // GP (G divides QB): every block starts at a whole position Rb / G, so row
  // r of a block is position Rb / G + r / G, head r % G -- a lane-constant
  // offset plus the block's position, which goes into the buffer base.
  uint32_t qoff[LOADS], loff = 0;
  if constexpr (GP) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = 4 * (i * NW + wave) + (lane >> 4);
      const int lc = (lane & 15) ^ swz(r);
      qoff[i] = (uint32_t)((((r / G) * Hq + r % G) * D + lc * 8) * 2);
    }
    const int r = wave * 64 + lane;             // lse / Delta row (waves < QB / 64)
    loff = (uint32_t)(((r % G) * T + r / G) * 4);
  }
  const int log2g = p.g_shift - 31;             // log2 G when G is a power of two

  // block of rows [Rb, Rb + 64) -> stage st
  auto load_block = [&](int Rb, int st) {
    char* sb = st ? smem1 : smem0;
    if constexpr (GP) {
      const int lim = TG - Rb;                  // rows r < lim of the block exist
      const long long tb = (long long)(Rb >> log2g);
      const __amdgpu_buffer_rsrc_t bq = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(reinterpret_cast<const bf16*>(p.q) + qbase + tb * Hq * D), (short)0, 0x7fffffff, kBufferWord3);
      const __amdgpu_buffer_rsrc_t bo = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(reinterpret_cast<const bf16*>(p.dO) + qbase + tb * Hq * D), (short)0, 0x7fffffff, kBufferWord3);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int sp = i * NW + wave;
        const uint32_t off = 4 * sp + (lane >> 4) < lim ? qoff[i] : OOB;
        dma16(bq, off, sb + sp * 1024);
        dma16(bo, off, sb + OFF_O + sp * 1024);
      }
      if (wave < QB / 64) {
        const uint32_t off = wave * 64 + lane < lim ? loff : OOB;
        const __amdgpu_buffer_rsrc_t bl = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.work + p.BHT + lbase + tb), (short)0, 0x7fffffff, kBufferWord3);
        const __amdgpu_buffer_rsrc_t bd = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.work + lbase + tb), (short)0, 0x7fffffff, kBufferWord3);
        dma4(bl, off, sb + OFF_L + wave * 256);
        dma4(bd, off, sb + OFF_D + wave * 256);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int sp = i * NW + wave;           // 4-row span of the block
        const int r = 4 * sp + (lane >> 4);
        const int R = Rb + r;
        const int t = div_g(R, p.g_magic, p.g_shift);
        const int lc = (lane & 15) ^ swz(r);
        const uint32_t off = R < TG ? (uint32_t)(((t * Hq + (R - t * G)) * D + lc * 8) * 2) : OOB;
        dma16(rq, off, sb + sp * 1024);
        dma16(ro, off, sb + OFF_O + sp * 1024);
      }
      if (wave < QB / 64) {
        const int R = Rb + wave * 64 + lane;
        const int t = div_g(R, p.g_magic, p.g_shift);
        const uint32_t off = R < TG ? (uint32_t)(((R - t * G) * T + t) * 4) : OOB;
        dma4(rl2, off, sb + OFF_L + wave * 256);
        dma4(rd, off, sb + OFF_D + wave * 256);
      }
    }
  };

  // lane-constant LDS byte offsets within a block
  //  row-major reads: operand row m holds block row pi(m) (+32 for the second half)
  const int qperm = key_row_perm(n);
  uint32_t roff[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) roff[kc] = (uint32_t)(qperm * 256 + (((2 * kc + hh) ^ swz(qperm)) * 16));
  uint32_t tro[8];   // transpose-read byte offsets within a block
  tr_offsets(lane, 0u, tro);

  const float sl2 = p.scale_log2;
  const int rb0 = kt0 * G / QB * QB;            // first block with a row at position >= kt0
  const int nqb = (TG - rb0 + QB - 1) / QB;
  if constexpr (!SPLIT) q_hi = nqb;

  // S and dP of 32-row sub-block `sub` of the block in stage ST, their
  // accumulators seeded with -lse*sqrt(d) and -Delta of each row: s holds
  // S - lse*sqrt(d) and dp holds dP - Delta.  The lane's 16 rows are two runs
  // of 8: sub*32 + 16c + 8hh + (0..7).
  auto products = [&]<int ST, int sub>(f32x16& s, f32x16& dp) {
    const char* sb = ST ? smem1 : smem0;
    bf16x8 qa[NKC], oa[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      qa[kc] = *reinterpret_cast<const bf16x8*>(sb + sub * 32 * 256 + roff[kc]);
      oa[kc] = *reinterpret_cast<const bf16x8*>(sb + OFF_O + sub * 32 * 256 + roff[kc]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q0 = sub * 32 + 16 * c + 8 * hh;
      const f32x4* lp = reinterpret_cast<const f32x4*>(sb + OFF_L + q0 * 4);
      const f32x4* dpp = reinterpret_cast<const f32x4*>(sb + OFF_D + q0 * 4);
      const f32x4 la = lp[0], lb = lp[1], da = dpp[0], db = dpp[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[8 * c + j] = la[j];
        s[8 * c + 4 + j] = lb[j];
        dp[8 * c + j] = da[j];
        dp[8 * c + 4 + j] = db[j];
      }
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      s = mma16(qa[kc], kf[kc], s);
      dp = mma16(oa[kc], vf[kc], dp);
    }
  };
  // P = 2^((S - lse sqrt(d)) log2(e) / sqrt(d)) and dS = P (dP - Delta) as
  // bf16 operand fragments; MASKED applies the causal condition
  // R >= key * G (rows past the end need no mask: their q and dO are zero, so
  // they add nothing)
  auto softmax = [&]<int sub, bool MASKED>(int Rb, const f32x16& s, const f32x16& dp, bf16x8 (&pf)[2],
                                           bf16x8 (&df)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * c + j;
        float x = s[r] * sl2;
        if constexpr (MASKED) x = Rb + sub * 32 + 16 * c + 8 * hh + j >= keyG ? x : -INFINITY;
        const float pr = __builtin_amdgcn_exp2f(x);
        pf[c][j] = (bf16)pr;
        df[c][j] = (bf16)(pr * dp[r]);
      }
    }
  };
  // Q^T and dO^T operand fragments of one sub-block (transpose reads), read
  // ahead of the softmax whose outputs they multiply
  auto tload = [&]<int ST, int sub>(bf16x8 (&qt)[2 * NDT], bf16x8 (&ot)[2 * NDT]) {
    const char* sb = ST ? smem1 : smem0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const char* qb = sb + sub * 32 * 256 + c * 4096;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + tro[2 * dt]));
        const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + tro[2 * dt + 1]));
        const s16x4 o0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + OFF_O + tro[2 * dt]));
        const s16x4 o1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + OFF_O + tro[2 * dt + 1]));
        const s16x4 pq[2] = {q0, q1}, po[2] = {o0, o1};
        qt[c * NDT + dt] = *reinterpret_cast<const bf16x8*>(pq);
        ot[c * NDT + dt] = *reinterpret_cast<const bf16x8*>(po);
      }
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS over one sub-block
  auto update = [&](const bf16x8 (&qt)[2 * NDT], const bf16x8 (&ot)[2 * NDT], const bf16x8 (&pf)[2],
                    const bf16x8 (&df)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        dv[dt] = mma16(ot[c * NDT + dt], pf[c], dv[dt]);
        dk[dt] = mma16(qt[c * NDT + dt], df[c], dk[dt]);
      }
  };
  // all sub-blocks, the products of the next issued before the softmax of
  // the current so that matrix and vector work overlap within the wave
  auto compute = [&]<int ST, bool MASKED>(int Rb) {
    f32x16 s[2], dp[2];
    products.template operator()<ST, 0>(s[0], dp[0]);
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ([&] {
        bf16x8 qt[2 * NDT], ot[2 * NDT];
        tload.template operator()<ST, I>(qt, ot);
        if constexpr (I + 1 < NSUB) products.template operator()<ST, I + 1>(s[(I + 1) & 1], dp[(I + 1) & 1]);
        bf16x8 pf[2], df[2];
        softmax.template operator()<I, MASKED>(Rb, s[I & 1], dp[I & 1], pf, df);
        update(qt, ot, pf, df);
      }(), ...);
    }(std::make_integer_sequence<int, NSUB>{});
  };

  auto block = [&]<int ST>(int qb) {
    // blocks are swept from the last rows back to the keys' first position, so
    // that the workgroups of all key tiles read the same rows at about the
    // same time (they share them in L2) and the masked blocks come last
    const int Rb = rb0 + (nqb - 1 - qb) * QB;
    if (qb + 1 < q_hi) load_block(Rb - QB, ST ^ 1);
    if (Rb + QB - 1 >= wkey0 * G) {             // some row of the block sees some key of this wave
      if (Rb >= (wkey0 + 31) * G)               // every row sees every key of this wave
        compute.template operator()<ST, false>(Rb);
      else
        compute.template operator()<ST, true>(Rb);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  load_block(rb0 + (nqb - 1 - q_lo) * QB, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int qb = q_lo;
  for (; qb + 1 < q_hi; qb += 2) {
    block.template operator()<0>(qb);
    block.template operator()<1>(qb + 1);
  }
  if (qb < q_hi) block.template operator()<0>(qb);

  if (SPLIT && nchunks > 1) {
    // partial sums in the accumulators' own layout, [wave][dK, dV][dt][4][lane][4]
    // floats (whole 1 KB rows per store), added up by moda_bwd_dkdv_reduce_kernel
    float* pp = p.part + (size_t)blockIdx.x * 32768 + wave * 8192 + lane * 4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 k4 = {dk[dt][g4 * 4 + 0], dk[dt][g4 * 4 + 1], dk[dt][g4 * 4 + 2], dk[dt][g4 * 4 + 3]};
        const f32x4 v4 = {dv[dt][g4 * 4 + 0], dv[dt][g4 * 4 + 1], dv[dt][g4 * 4 + 2], dv[dt][g4 * 4 + 3]};
        *reinterpret_cast<f32x4*>(pp + (dt * 4 + g4) * 256) = k4;
        *reinterpret_cast<f32x4*>(pp + (16 + dt * 4 + g4) * 256) = v4;
      }
  } else if (key_ok) {
    const float sc = p.scale;
    const long long orow = (((long long)b * T + key) * p.Hkv + kvh) * D;
    bf16* dkp = reinterpret_cast<bf16*>(p.dk) + orow;
    bf16* dvp = reinterpret_cast<bf16*>(p.dv) + orow;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int e = dt * 32 + g4 * 8 + hh * 4;
        store4(dkp + e, dk[dt][g4 * 4 + 0] * sc, dk[dt][g4 * 4 + 1] * sc, dk[dt][g4 * 4 + 2] * sc,
               dk[dt][g4 * 4 + 3] * sc);
        store4(dvp + e, dv[dt][g4 * 4 + 0], dv[dt][g4 * 4 + 1], dv[dt][g4 * 4 + 2], dv[dt][g4 * 4 + 3]);
      }
  }
  release_work_slot(tick, BH, NW);
}

// Row-split dK/dV: the sum of a key tile's partial sums, in chunk order (its
// full chunks, then its remainder chunk), scaled and stored like the unsplit
// kernel's epilogue.  One workgroup per (key tile, b, kv head); tiles swept by
// a single chunk were stored by the dK/dV kernel itself.
template <int D>
__global__ __launch_bounds__(256) void moda_bwd_dkdv_reduce_kernel(BwdParams p) {
  static_assert(D == 128, "built for head size 128");
  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH;
  const int kt = (int)(blockIdx.x / BH);
  const BwdChunkMap cm(p.T, p.G, p.kchunk, p.nktiles);
  const int nf = cm.nf(kt);
  const bool has_rem = cm.rem(kt) > 0;
  if (nf + (has_rem ? 1 : 0) <= 1) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const size_t first = (size_t)cm.prefix(kt) * BH + bh;             // slot of full chunk 0
  const size_t last = ((size_t)p.kfull + cm.rem_rank(kt)) * BH + bh;  // slot of the remainder
  const float* base = p.part + wave * 8192 + lane * 4;
  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto add = [&](size_t slot) {
    const float* src = base + slot * 32768;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] += *reinterpret_cast<const f32x4*>(src + i * 256);
  };
  for (int c = 0; c < nf; ++c) add(first + (size_t)c * BH);
  if (has_rem) add(last);

  const int key = kt * 128 + wave * 32 + (lane & 31);
  if (key >= p.T) return;
  const int hh = lane >> 5;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const float sc = p.scale;
  const long long orow = (((long long)b * p.T + key) * p.Hkv + kvh) * D;
  bf16* dkp = reinterpret_cast<bf16*>(p.dk) + orow;
  bf16* dvp = reinterpret_cast<bf16*>(p.dv) + orow;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int e = dt * 32 + g4 * 8 + hh * 4;
      const f32x4 k4 = acc[dt * 4 + g4], v4 = acc[16 + dt * 4 + g4];
      store4(dkp + e, k4[0] * sc, k4[1] * sc, k4[2] * sc, k4[3] * sc);
      store4(dvp + e, v4[0], v4[1], v4[2], v4[3]);
    }
}

// ---------------------------------------------------------------------------
// bf16, d = 128: dQ laid out like moda_bwd_dkdv_bf16_kernel (same computation
// as moda_bwd_dq_kernel): K and V blocks of 64 keys go straight into two LDS
// stages; one swizzled copy of K serves the row-major score operand and, via
// transpose reads, the K^T operand of dQ^T += K^T dS^T.
// The depth slots' share of dQ for the bf16 d = 128 kernel: as dq_depth_fold,
// with the key-transposed operand of dQ^T += K^T dS^T read from LDS.  The key
// rows loaded for the score products go to this wave's 8 KB region of the
// free LDS stages (swizzled like a sequence K block, unread slots as zero
// rows), to be read back with the transpose reads of the sequence sweep --
// instead of gathering 64 single elements per lane from memory.
template <int D>
__device__ __forceinline__ void dq_depth_fold_bf16(const BwdParams& p, int bh, int tw_min, int tw_max, int t_row,
                                                   int n, int hh, int key_row, const bf16x8 (&qf)[D / 16],
                                                   const bf16x8 (&df)[D / 16], float lse2, float dlt,
                                                   f32x16 (&acc)[D / 32], char* region,
                                                   const uint32_t (&tro)[8]) {
  using namespace bwdbf16;
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  const float sl2 = p.scale_log2;
  const int L_d = p.L_d, L_cap = p.L_cap, slot_lo = p.slot_lo;
  const long long nlo = (long long)tw_min * L_cap + slot_lo;
  const long long nhi = (long long)tw_max * L_cap + slot_lo + L_d;
  const bf16* kdb = reinterpret_cast<const bf16*>(p.kd) + (long long)bh * p.NKp * D;
  const bf16* vdb = reinterpret_cast<const bf16*>(p.vd) + (long long)bh * p.NKp * D;
  const int8_t* kq8 = reinterpret_cast<const int8_t*>(p.kd) + (long long)bh * p.NKp * D;
  const int8_t* vq8 = reinterpret_cast<const int8_t*>(p.vd) + (long long)bh * p.NKp * D;
  const float* ks8 = p.q8 ? p.ksc + (long long)bh * p.NKp : nullptr;
  const float* vs8 = p.q8 ? p.vsc + (long long)bh * p.NKp : nullptr;
  const int sw = swz(key_row);
  for (long long n0 = nlo & ~31LL; n0 < nhi; n0 += 32) {
    if (!depth_tile_used(n0, L_cap, slot_lo, L_d)) continue;
    bf16x8 kf[NKC];
    f32x16 s = f32x16{}, dp = f32x16{};
    const long long kr = n0 + key_row;
    if (p.q8) {
      const float ks = ks8[kr], vs = vs8[kr];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        kf[kc] = Dequant<bf16>::frag(kq8 + kr * D + hh * 8 + kc * 16, ks);
        s = mma16(kf[kc], qf[kc], s);
        dp = mma16(Dequant<bf16>::frag(vq8 + kr * D + hh * 8 + kc * 16, vs), df[kc], dp);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        kf[kc] = load_frag(kdb + kr * D + hh * 8 + kc * 16);
        s = mma16(kf[kc], qf[kc], s);
        dp = mma16(load_frag(vdb + kr * D + hh * 8 + kc * 16), df[kc], dp);
      }
    }
    const long long own_lo = (long long)t_row * L_cap + slot_lo - n0;
    const long long own_hi = own_lo + L_d;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = reg_key(r, hh);
      const bool own = key >= own_lo && key < own_hi;
      const float pr = __builtin_amdgcn_exp2f(own ? s[r] * sl2 - lse2 : -INFINITY);
      // a masked key contributes exactly 0 (its dP may be non-finite when the
      // slot is unread)
      ds[r] = own ? pr * (dp[r] - dlt) : 0.f;
    }
    // this lane's key row into the region (row key_row, 16-byte chunks
    // 2 kc + hh); keys of unread slots (and padding) as zero rows: their dS is
    // 0, and 0 * x would still carry a non-finite x into dQ
    const uint32_t rows_ok = depth_tile_partial(n0, L_cap, slot_lo, L_d, p.T)
                                 ? depth_tile_rows(n0, L_cap, slot_lo, L_d, p.T, n + 32 * hh) : 0xffffffffu;
    const bool row_ok = (rows_ok >> key_row) & 1u;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(&kf[kc]) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(region + key_row * 256 + (((2 * kc + hh) ^ sw) * 16)) = v;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (bf16)ds[c * 8 + j];
      const char* kb = region + c * 16 * 256;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + tro[2 * dt]));
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + tro[2 * dt + 1]));
        const s16x4 pr[2] = {r0, r1};
        acc[dt] = mma16(*reinterpret_cast<const bf16x8*>(pr), f, acc[dt]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moda_bwd_dq_bf16_kernel(BwdParams p) {
  static_assert(D == 128, "built for head size 128");
  using namespace bwdbf16;
  constexpr int NW = 4;
  constexpr int BN = 64;
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE_B = BN * D * 2;
  constexpr int OFF_V = TILE_B;
  constexpr int STAGE = 2 * TILE_B;
  constexpr int LOADS = BN * D / 8 / (NW * 64);

  // the two stages as separate arrays (loads from one provably do not alias
  // the direct-to-LDS writes in flight into the other)
  __shared__ __attribute__((aligned(1024))) char smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.Hkv;
  // work item: query tiles of each (b, kv head) pair, heaviest first
  __shared__ uint32_t s_item;
  const WorkItem wi = take_work_item(p.tick_dq, BH, p.ntiles, &s_item);
  const int bh = wi.pair;
  const int tile = p.ntiles - 1 - wi.index;
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
  const int nblocks = (int)(Rlast / G) / BN + 1;

  const long long qrow = (((long long)b * T + t_row) * p.Hq + hq) * D + hh * 8;
  bf16x8 qf[NKC], df[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    qf[kc] = row_ok ? load_frag(reinterpret_cast<const bf16*>(p.q) + qrow + kc * 16) : bf16x8{};
    df[kc] = row_ok ? load_frag(reinterpret_cast<const bf16*>(p.dO) + qrow + kc * 16) : bf16x8{};
  }
  const long long lrow = ((long long)b * p.Hq + hq) * T + t_row;
  const float lse2 = row_ok ? p.lse[lrow] * kLog2e : INFINITY;
  const float dlt = row_ok ? -p.work[lrow] : 0.f;
  const float sl2 = p.scale_log2;
  f32x16 dp0;                                   // dP accumulators start at -Delta
#pragma unroll
  for (int r = 0; r < 16; ++r) dp0[r] = -dlt;

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16{};

  const long long kstride = (long long)p.Hkv * D;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long long)b * T * p.Hkv + kvh) * D;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long long)b * T * p.Hkv + kvh) * D;
  const int row_bytes = (int)kstride * 2;
  // span sp of a block is loaded by wave sp % NW: lane l fills row 4 sp + l / 16,
  // physical chunk l % 16 (logical chunk l % 16 ^ swz(row))
  uint32_t off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int sp = i * NW + wave;
    const int r = 4 * sp + (lane >> 4);
    off[i] = (uint32_t)(r * row_bytes + (((lane & 15) ^ swz(r)) * 16));
  }
  auto block_rsrc = [&](const bf16* head, int blk) {
    const int valid = T - blk * BN;   // >= 1 for every loaded block; rows past it read zeros
    const int bytes = valid >= BN ? BN * row_bytes : (valid - 1) * row_bytes + D * 2;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(head) + (long long)blk * BN * row_bytes), (short)0, bytes,
        kBufferWord3);
  };
  auto load_block = [&](int blk, int st) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, blk), rv = block_rsrc(vbase, blk);
    char* sb = st ? smem1 : smem0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      dma16(rk, off[i], sb + (i * NW + wave) * 1024);
      dma16(rv, off[i], sb + OFF_V + (i * NW + wave) * 1024);
    }
  };

  const int key_row = key_row_perm(n);
  uint32_t roff[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) roff[kc] = (uint32_t)(key_row * 256 + (((2 * kc + hh) ^ swz(key_row)) * 16));
  uint32_t tro[8];   // transpose-read byte offsets within a block
  tr_offsets(lane, 0u, tro);

  auto block = [&]<int ST>(int j) {
    if (j + 1 < nblocks) load_block(j + 1, ST ^ 1);
    if (wave_active && j * BN <= tw_max) {
      const char* sb = ST ? smem1 : smem0;
      auto half = [&]<int H>() {
        bf16x8 ka[NKC], va[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          ka[kc] = *reinterpret_cast<const bf16x8*>(sb + H * 32 * 256 + roff[kc]);
          va[kc] = *reinterpret_cast<const bf16x8*>(sb + OFF_V + H * 32 * 256 + roff[kc]);
        }
        f32x16 s = f32x16{}, dp = dp0;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          s = mma16(ka[kc], qf[kc], s);
          dp = mma16(va[kc], df[kc], dp);
        }
        bf16x8 dsf[2];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], sl2, -lse2);
        // the causal mask only where some key of the half lies past some row
        // of the wave (a wave-uniform branch)
        if (j * BN + H * 32 + 31 > tw_min) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            x[r] = j * BN + H * 32 + reg_key(r, hh) <= t_row ? x[r] : -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(x[r]);
          dsf[r >> 3][r & 7] = (bf16)(pr * dp[r]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const char* kb = sb + H * 32 * 256 + c * 16 * 256;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + tro[2 * dt]));
            const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + tro[2 * dt + 1]));
            const s16x4 pr[2] = {r0, r1};
            acc[dt] = mma16(*reinterpret_cast<const bf16x8*>(pr), dsf[c], acc[dt]);
          }
        }
      };
      half.template operator()<0>();
      half.template operator()<1>();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  load_block(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int j = 0;
  for (; j + 1 < nblocks; j += 2) {
    block.template operator()<0>(j);
    block.template operator()<1>(j + 1);
  }
  if (j < nblocks) block.template operator()<0>(j);

  if (wave_active && p.L_d > 0)
    dq_depth_fold_bf16<D>(p, bh, tw_min, tw_max, t_row, n, hh, key_row, qf, df, lse2, dlt, acc, smem0 + wave * 8192, tro);
  if (row_ok) dq_store<bf16, D>(p, b, t_row, hq, hh, acc);
  release_work_slot(p.tick_dq, BH, NW);
}

// ---------------------------------------------------------------------------
// bf16, d = 128, G dividing 32: depth-slot gradients on the matrix cores.
// A wave owns 32 folded rows, i.e. 32 / G whole positions, so every depth slot
// of those positions is seen only by this wave's rows: the wave stages its
// rows of q and dO in its own LDS region (swizzled as in the dK/dV kernel) and
// sweeps the 32-key tiles of the packed depth buffers that hold its
// positions' slots -- S = Q K_d^T and dP = dO V_d^T with a lane per key (the
// accumulators seeded with -lse*sqrt(d) and -Delta), P and dS masked to
// "same position, slot in the window", then dV_d^T += dO^T P and
// dK_d^T += Q^T dS -- and writes the keys of its own positions in the logical
// [B,T,L_d,Hkv,d] layout.  No barriers: each wave touches only its own LDS.
template <int D>
__global__ __launch_bounds__(256) void moda_bwd_depth_bf16_kernel(BwdParams p) {
  static_assert(D == 128, "built for head size 128");
  using namespace bwdbf16;
  constexpr int NW = 4;
  constexpr int NKC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int REG = 32 * D * 2;                 // bytes of one wave's 32 rows

  __shared__ __attribute__((aligned(1024))) char sQ[NW * REG];
  __shared__ __attribute__((aligned(1024))) char sO[NW * REG];
  __shared__ __attribute__((aligned(16))) float sL[NW * 32];
  __shared__ __attribute__((aligned(16))) float sD[NW * 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH;
  const int tile = (int)(blockIdx.x / BH);
  const int b = bh / p.Hkv;
  const int kvh = bh % p.Hkv;
  const int G = p.G, T = p.T, Hq = p.Hq;
  const int TG = T * G;
  const int Rw = tile * (NW * 32) + wave * 32;
  if (Rw >= TG) return;
  const int tw_min = div_g(Rw, p.g_magic, p.g_shift);
  const int tw_max = div_g((Rw + 31 < TG ? Rw + 31 : TG - 1), p.g_magic, p.g_shift);

  char* wq = sQ + wave * REG;
  char* wo = sO + wave * REG;
  float* wl = sL + wave * 32;
  float* wd = sD + wave * 32;
  {
    const bf16* qg = reinterpret_cast<const bf16*>(p.q);
    const bf16* og = reinterpret_cast<const bf16*>(p.dO);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), lc = lane & 15;
      const int R = Rw + r;
      u32x4 qv = {0, 0, 0, 0}, ov = {0, 0, 0, 0};
      if (R < TG) {
        const int t = div_g(R, p.g_magic, p.g_shift);
        const long long off = (((long long)b * T + t) * Hq + kvh * G + (R - t * G)) * D + lc * 8;
        qv = ld16(qg + off);
        ov = ld16(og + off);
      }
      st16(wq + r * 256 + ((lc ^ swz(r)) * 16), qv);
      st16(wo + r * 256 + ((lc ^ swz(r)) * 16), ov);
    }
    if (lane < 32) {
      const int R = Rw + lane;
      float l = 0.f, dl = 0.f;
      if (R < TG) {
        const int t = div_g(R, p.g_magic, p.g_shift);
        const long long li = ((long long)b * Hq + kvh * G + (R - t * G)) * T + t;
        l = p.work[p.BHT + li];     // -lse * sqrt(d)
        dl = p.work[li];            // -Delta
      }
      wl[lane] = l;
      wd[lane] = dl;
    }
  }

  const int qperm = key_row_perm(n);
  uint32_t roff[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) roff[kc] = (uint32_t)(qperm * 256 + (((2 * kc + hh) ^ swz(qperm)) * 16));
  uint32_t tro[8];
  tr_offsets(lane, 0u, tro);
  const float sl2 = p.scale_log2, sc = p.scale;
  const int L_d = p.L_d, L_cap = p.L_cap, slot_lo = p.slot_lo;
  const bf16* kdb = reinterpret_cast<const bf16*>(p.kd) + (long long)bh * p.NKp * D;
  const bf16* vdb = reinterpret_cast<const bf16*>(p.vd) + (long long)bh * p.NKp * D;
  const long long nlo = (long long)tw_min * L_cap + slot_lo;
  const long long nhi = (long long)tw_max * L_cap + slot_lo + L_d;

  for (long long n0 = nlo & ~31LL; n0 < nhi; n0 += 32) {
    if (!depth_tile_used(n0, L_cap, slot_lo, L_d)) continue;
    const long long key = n0 + n;
    const int tk = (int)(key / L_cap);
    const int slot = (int)(key - (long long)tk * L_cap) - slot_lo;
    const bool key_ok = tk < T && slot >= 0 && slot < L_d;
    const int r_lo = tk * G;                      // rows [r_lo, r_lo + G) sit at position tk
    bf16x8 kf[NKC], vf[NKC];
    if (p.q8) {
      const long long r = (long long)bh * p.NKp + key;
      const int8_t* kq = reinterpret_cast<const int8_t*>(p.kd) + r * D + hh * 8;
      const int8_t* vq = reinterpret_cast<const int8_t*>(p.vd) + r * D + hh * 8;
      const float ks = p.ksc[r], vs = p.vsc[r];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        kf[kc] = dequant_frag_bf16(kq + kc * 16, ks);
        vf[kc] = dequant_frag_bf16(vq + kc * 16, vs);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        kf[kc] = load_frag(kdb + key * D + kc * 16 + hh * 8);
        vf[kc] = load_frag(vdb + key * D + kc * 16 + hh * 8);
      }
    }
    f32x16 s, dp;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x4* lp = reinterpret_cast<const f32x4*>(wl + 16 * c + 8 * hh);
      const f32x4* dpp = reinterpret_cast<const f32x4*>(wd + 16 * c + 8 * hh);
      const f32x4 la = lp[0], lb = lp[1], da = dpp[0], db = dpp[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[8 * c + j] = la[j];
        s[8 * c + 4 + j] = lb[j];
        dp[8 * c + j] = da[j];
        dp[8 * c + 4 + j] = db[j];
      }
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      s = mma16(*reinterpret_cast<const bf16x8*>(wq + roff[kc]), kf[kc], s);
      dp = mma16(*reinterpret_cast<const bf16x8*>(wo + roff[kc]), vf[kc], dp);
    }
    bf16x8 pf[2], df[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * c + j;
        const int R = Rw + 16 * c + 8 * hh + j;
        const float x = (key_ok && R >= r_lo && R < r_lo + G) ? s[r] * sl2 : -INFINITY;
        const float pr = __builtin_amdgcn_exp2f(x);
        pf[c][j] = (bf16)pr;
        df[c][j] = (bf16)(pr * dp[r]);
      }
    f32x16 dk[NDT], dv[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const char* qb = wq + c * 16 * 256;
        const char* ob = wo + c * 16 * 256;
        const s16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + tro[2 * dt]));
        const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + tro[2 * dt + 1]));
        const s16x4 o0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ob + tro[2 * dt]));
        const s16x4 o1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ob + tro[2 * dt + 1]));
        const s16x4 pq[2] = {q0, q1}, po[2] = {o0, o1};
        dv[dt] = mma16(*reinterpret_cast<const bf16x8*>(po), pf[c], dv[dt]);
        dk[dt] = mma16(*reinterpret_cast<const bf16x8*>(pq), df[c], dk[dt]);
      }
    if (key_ok && tk >= tw_min && tk <= tw_max) {
      const long long orow = ((((long long)b * T + tk) * L_d + slot) * p.Hkv + kvh) * D;
      bf16* dkp = reinterpret_cast<bf16*>(p.dkd) + orow;
      bf16* dvp = reinterpret_cast<bf16*>(p.dvd) + orow;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int e = dt * 32 + g4 * 8 + hh * 4;
          store4(dkp + e, dk[dt][g4 * 4 + 0] * sc, dk[dt][g4 * 4 + 1] * sc, dk[dt][g4 * 4 + 2] * sc,
                 dk[dt][g4 * 4 + 3] * sc);
          store4(dvp + e, dv[dt][g4 * 4 + 0], dv[dt][g4 * 4 + 1], dv[dt][g4 * 4 + 2], dv[dt][g4 * 4 + 3]);
        }
    }
  }
}

}  // namespace moda
