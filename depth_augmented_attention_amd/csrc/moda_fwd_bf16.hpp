// Fused MoDA forward, bf16 inputs, for gfx950 (CDNA4).
//
// Same computation and row folding as the generic kernel in moda_fwd.hpp (see
// the description there); this variant is laid out for the gfx950 memory path
// and for overlapping matrix-core and vector work:
//   * K and V blocks go from HBM straight into LDS with the direct
//     global->LDS 16-byte loads (no staging registers, no LDS store
//     instructions).  Scores run half a block ahead of the softmax: while
//     the softmax and P.V of one 32-key half run, the scores of the next half
//     are already being formed on the matrix cores, so a wave always has
//     independent matrix and vector work (K is loaded half a block further
//     ahead than V).  Two LDS stages each for K and V; one workgroup barrier
//     per 64-key block.
//   * V stays key-major in LDS; the P.V product reads it with the LDS
//     transpose load (ds_read_b64_tr_b16), which hands each lane four
//     consecutive keys of one head dimension -- the operand order the matrix
//     cores want -- without any shuffles.  A half-block's V fragments are
//     read before its softmax starts, so the LDS latency is spent under the
//     vector work instead of in front of each P.V product.
//   * LDS rows are 256 bytes with no padding; bank conflicts are avoided by an
//     XOR swizzle of the 16-byte chunk index (K: chunk ^ (row & 15);
//     V: chunk ^ 4 * (row & 3)), chosen so that every 16-lane K read and every
//     32-lane transposed V read touches 64 distinct banks.
//   * Eight waves (256 query rows) per workgroup and at most 256 registers per
//     wave: two waves per SIMD, and each K/V block staged in LDS serves 256
//     rows (one workgroup per compute unit; +3% over four-wave workgroups
//     with two per compute unit).  Grids too small to fill the GPU twice over
//     with 256-row tiles use four-wave workgroups (128 rows) instead.  The
//     eight-wave grids take their tiles from a per-launch counter in the
//     order their workgroups start (see the work-item code below).
//   * Probabilities are taken against the running max without forming the
//     block's row max first; only when a lane's sum of them exceeds 2^8 (a
//     score rose well above the max, or the first block) is the row max
//     formed, the max moved, O rescaled and the probabilities recomputed.
//     This changes nothing in exact arithmetic (out = O / l and lse =
//     m + log2 l use the same m), keeps every probability below 2^8, and
//     drops the max reduction from the common path.  Row sums come from the
//     same bf16 probabilities that feed the P.V product (v_dot2_f32_bf16).
//   * The causal mask is only evaluated in the last few blocks of a tile.
//   * The depth slots of a wave's positions are folded in after the sweep,
//     one 32-key depth tile at a time, with the tile's key fragments and
//     value rows loaded together (one round trip to memory per tile) and the
//     values transposed through the wave's own LDS region.
//   * Split key ranges (SPLIT, four-wave tiles, grids of at most two
//     workgroups per compute unit): a causal grid's longest tile sweeps about
//     twice the key blocks of the average one, and on a small grid it alone
//     sets the time.  With a workspace, each of the nsplit longest tiles of a
//     (b, kv head) -- tile i, paired with the short tile j = ntiles - 1 - i --
//     is swept by two workgroups: part 0 over key blocks [0, h) plus the
//     depth slots, part 1 over [h, nb_i), h = (nb_i - nb_j) / 2.  Parts run
//     first, then the short tiles longest first; a compute unit whose part 0
//     ends early takes the next short tile, so part 0 + short tile and part 1
//     each come to about (nb_i + nb_j) / 2 blocks.  The depth fold goes with
//     part 0 because parts 0 end at spread-out times (h varies with the tile)
//     while parts 1 all end together: folded at the end of part 1, every
//     compute unit would fetch its depth slots at once, at the end of the
//     kernel, bound by HBM; spread out, each fold runs beside another
//     workgroup's sweep.  Each wave of a part writes
//     its running state (O, m, l per lane) to the workspace, and the second
//     wave of the pair to arrive (a device-wide counter) merges the other's
//     state into its own -- m = max(m0, m1), O = 2^(m0 - m) O0 + 2^(m1 - m) O1,
//     l likewise: the same online-softmax recurrence over the union of the
//     two key sets, exact in real arithmetic -- writes out and lse, and
//     clears the counter for the next launch.
//   * Key split inside the workgroup (KS, grids of at most one round of
//     eight-wave workgroups over 128-row tiles): the two sets of four waves
//     share a tile's rows, sweep one half of its key blocks each (with their
//     own LDS stages) and take alternate depth tiles; set 1 hands its state
//     to set 0 through LDS, which merges it with the same recurrence and
//     writes the output.  No workspace, and one barrier count for both sets
//     (the set with one block fewer takes one barrier more).
#pragma once

#include "moda_common.hpp"
#include "moda_fwd.hpp"

namespace moda {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Third word of a raw buffer descriptor on gfx9-family GPUs (32-bit data
// format, no swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per lane from a raw buffer straight into LDS: lane l's data lands
// at ldst + 16 l (ldst is wave-uniform).  Out-of-range offsets read zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* ldst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)ldst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One V^T operand fragment through two LDS transpose reads
// (ds_read_b64_tr_b16): p is this lane's byte address of its first row; the
// second row is 4 rows (1024 bytes) further.  Each read hands the lane four
// consecutive rows (keys) of one column (head dimension).
__device__ __forceinline__ bf16x8 tr_frag(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 1024));
  const s16x4 pr[2] = {r0, r1};
  return *reinterpret_cast<const bf16x8*>(pr);
}

// Floats of one wave's partial state in the split-key workspace: 64 O^T
// accumulator values, m and l for each of the 64 lanes.
constexpr int kSplitState = 66;

// NW waves per workgroup (32 query rows each): 8, or 4 for small grids;
// SPLIT: key ranges of the longest tiles split over two workgroups.
// KS (eight waves, small grids): the two sets of four waves share one
// 128-row tile and split its key blocks and its depth tiles between them,
// each set with its own LDS stages, and meet through LDS at the end -- one
// workgroup per compute unit that sweeps a long tile's keys twice as fast.
template <int D, int NW, bool SPLIT = false, bool KS = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moda_fwd_bf16_kernel(FwdParams p) {
  static_assert(D == 128, "the bf16 fast path is built for head size 128");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(!KS || (NW == 8 && !SPLIT), "the key split is an eight-wave layout");
  constexpr int NR = KS ? 4 : NW;         // 32-row groups of a tile
  constexpr int NS = KS ? 2 : 1;          // sets of LDS stages
  constexpr int BN = 64;                  // keys per sequence block
  constexpr int NKC = D / 16;             // 16-wide k-chunks over d
  constexpr int NDT = D / 32;             // 32-row tiles of O^T over d
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int TILE = BN * D;            // elements of one K (or V) block
  constexpr int SPANS = TILE / 512;        // 1 KB spans per block
  constexpr int LOADS = (SPANS + NR - 1) / NR;   // the waves of a stage set load its blocks

  // Each K stage as two 32-row halves and each V stage as one array, all
  // separate objects: in every block the loads in flight go to (K stage ST,
  // half 0), (K stage ST^1, half 1) and V stage ST^1 while the reads come from
  // the other three, so the compiler can see that no read waits for them.
  __shared__ __attribute__((aligned(1024))) bf16 smemK00[NS * TILE / 2];
  __shared__ __attribute__((aligned(1024))) bf16 smemK01[NS * TILE / 2];
  __shared__ __attribute__((aligned(1024))) bf16 smemK10[NS * TILE / 2];
  __shared__ __attribute__((aligned(1024))) bf16 smemK11[NS * TILE / 2];
  __shared__ __attribute__((aligned(1024))) bf16 smemV0[NS * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 smemV1[NS * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int rw = KS ? (wave & 3) : wave;  // row group of the tile
  const int kh = KS ? (wave >> 2) : 0;    // key half (stage set) of the wave

  // Work item of this workgroup.  Eight-wave grids of several rounds take
  // it from a launch counter in the order workgroups start (the longest
  // tiles still first), not from blockIdx: the GPU hands workgroups to its
  // eight XCDs round-robin by blockIdx, and XCDs run at different speeds
  // (on one MI355X the odd ones took 3.5% longer over the same tiles), so a
  // fixed split of the grid leaves the fast XCDs idle while the slow ones
  // finish; drawn from the counter, each XCD takes work while it has time.
  constexpr bool DYN = NW == 8 && !KS && !SPLIT;
  uint32_t wg = blockIdx.x;
  if constexpr (DYN) {
    if (p.tick) {
      __shared__ uint32_t s_wg;
      if (tid == 0) s_wg = __hip_atomic_fetch_add(p.tick, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      wg = s_wg;
    }
  }

  const int BH = p.B * p.Hkv;
  // counter order: one (b, kv head) after another, so that the workgroups
  // running at one time share the K/V blocks of one head in each XCD's L2
  // (with blockIdx order each XCD keeps to one head by itself)
  const int bh = DYN && p.tick ? (int)(wg / (uint32_t)p.ntiles) : (int)(wg % (uint32_t)BH);
  // part 0 / 1 of a split tile, or -1 for a whole tile
  int tile, part = -1;
  if constexpr (SPLIT) {
    const int slot = (int)(blockIdx.x / BH), H = p.nsplit;
    if (slot < 2 * H) {
      part = slot < H ? 1 : 0;
      tile = p.ntiles - 1 - (slot < H ? slot : slot - H);
    } else {
      tile = p.ntiles - 1 - H - (slot - 2 * H);
    }
  } else if (DYN && p.tick) {
    tile = p.ntiles - 1 - (int)(wg % (uint32_t)p.ntiles);
  } else {
    tile = query_tile((int)(wg / (uint32_t)BH), p.ntiles, p.paired);
  }
  const int b = bh / p.Hkv;
  const int kvh = bh % p.Hkv;
  const int G = p.G;
  const int T = p.T;
  const long long TG = (long long)T * G;

  const long long R0 = (long long)tile * (NR * 32);
  const long long Rw = R0 + rw * 32;
  const long long R = Rw + n;
  const bool row_ok = R < TG;
  const bool wave_active = Rw < TG;
  const int t_row = row_ok ? (int)(R / G) : T - 1;
  const int hq = kvh * G + (row_ok ? (int)(R % G) : 0);
  const int tw_min = wave_active ? (int)(Rw / G) : T - 1;
  const int tw_max = wave_active ? (int)((Rw + 31 < TG ? Rw + 31 : TG - 1) / G) : T - 1;
  const long long Rlast = (R0 + NR * 32 < TG ? R0 + NR * 32 : TG) - 1;
  const int t_first = (int)(R0 / G);
  const int t_last = (int)(Rlast / G);
  const int nblocks = t_last / BN + 1;
  // blocks [0, jm) have every key <= every row's position: no mask needed
  const int jm = (t_first + 1) / BN < nblocks ? (t_first + 1) / BN : nblocks;
  // key blocks [jlo, jhi) swept by this workgroup
  int jlo = 0, jhi = nblocks;
  if constexpr (KS) {
    // set 0 the first half of the key blocks, set 1 the rest (and the masked ones)
    if (kh == 0) jhi = nblocks / 2;
    else jlo = nblocks / 2;
  }
  if constexpr (SPLIT) {
    if (part >= 0) {
      const int j_tile = p.ntiles - 1 - tile;          // the short partner tile
      const long long Rj = ((long long)j_tile + 1) * (NW * 32);
      const int nbj = (int)(((Rj < TG ? Rj : TG) - 1) / G) / BN + 1;
      int h = (nblocks - nbj) / 2;
      h = h < 0 ? 0 : (h > jm ? jm : h);
      if (part == 0) jhi = h;
      else jlo = h;
    }
  }

  bf16x8 qf[NKC];
  {
    const bf16* qp = reinterpret_cast<const bf16*>(p.q) + (((long long)b * T + t_row) * p.Hq + hq) * D + hh * 8;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qf[kc] = row_ok ? load_frag(qp + kc * 16) : bf16x8{};
  }

  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x16{};
  float m_run = -1e30f;   // running max (log2 units of the scaled scores)
  float l_run = 0.f;      // running sum over this lane's keys

  const long long kstride = (long long)p.Hkv * D;
  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long long)b * T * p.Hkv + kvh) * D;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long long)b * T * p.Hkv + kvh) * D;

  // Direct loads.  A K or V block is 64 rows of 256 bytes = 16 spans of 1 KB.
  // Span sp is written by one wave-wide load: lane l fills 16-byte position
  // l, i.e. row r = 4 sp + l / 16, physical chunk l % 16, which holds the
  // logical chunk physical ^ swizzle(r).  Byte offsets are lane constants
  // relative to the block's first row; the block base lives in the (scalar)
  // buffer descriptor.
  uint32_t offk[LOADS], offv[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int sp = i * NR + rw;
    const int r = sp * 4 + lane / 16;
    const int pc = lane % 16;
    offk[i] = (uint32_t)(r * (int)kstride + (pc ^ (r & 15)) * 8) * 2u;
    offv[i] = (uint32_t)(r * (int)kstride + (pc ^ (4 * (r & 3))) * 8) * 2u;
  }
  const int row_bytes = (int)kstride * 2;
  // Block blk of one head (K or V) as a raw buffer: rows past the end of the
  // sequence are out of range and arrive in LDS as zeros.
  auto block_rsrc = [&](const bf16* head, int blk) {
    const int valid = T - blk * BN;     // >= 1 for every block that is loaded
    const int bytes = valid >= BN ? BN * row_bytes : (valid - 1) * row_bytes + D * 2;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(head) + (long long)blk * BN * row_bytes), (short)0, bytes,
        kBufferWord3);
  };
  // load spans [S_LO, S_HI) of block blk: slot i covers span i*NW + wave,
  // which lands at span (i*NW + wave - S_LO) of lbase.  The range is a whole
  // number of rounds of the waves, so the slots a wave loads are known at
  // compile time (no branch per load: fewer basic blocks in the sweep for
  // the scheduler to work across)
  auto dma_rows = [&]<int S_LO, int S_HI>(const bf16* head, int blk, const uint32_t (&off)[LOADS], bf16* lbase) {
    static_assert(S_LO % NR == 0 && S_HI % NR == 0, "span ranges are whole rounds of the waves");
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(head, blk);
#pragma unroll
    for (int i = S_LO / NR; i < S_HI / NR; ++i) dma16(rs, off[i], lbase + (i * NR + rw - S_LO) * 512);
  };

  const int klast = jhi - 1;
  auto clampb = [&](int blk) { return blk <= klast ? blk : klast; };
  // K stage st, half h (rows 32h .. 32h+31 of the block)
  auto khalf = [&](int st, int h) -> bf16* {
    return (st ? (h ? smemK11 : smemK10) : (h ? smemK01 : smemK00)) + (KS ? kh * (TILE / 2) : 0);
  };
  auto vst = [&](int st) { return (st ? smemV1 : smemV0) + (KS ? kh * TILE : 0); };

  // Lane-constant LDS byte offsets.
  //  K operand row r = pi(n) of a 32-row half: chunk (2kc + hh) ^ (r & 15);
  //  pi(n) < 32 and (r & 15) is the same for the second half (rows + 32).
  const int key_row = key_row_perm(n);
  uint32_t koff[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    koff[kc] = (uint32_t)(key_row * D + (((2 * kc + hh) ^ (key_row & 15)) * 8)) * 2u;
  //  V transposed reads: 16-lane group q16, lane j16 reads row
  //  c16 + 8*(q16/2) + j16/4 (+4), logical chunk 4dt + 2(q16&1) + (j16&3)/2,
  //  half (j16&1); the swizzle XORs the chunk with 4*(row & 3) = 4*(j16/4).
  const int q16 = lane >> 4, j16 = lane & 15;
  uint32_t va[NDT];   // byte offsets within a V block (second row of a fragment: +1024)
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int r = 8 * (q16 >> 1) + (j16 >> 2);
    const int chunk = (4 * dt + 2 * (q16 & 1) + ((j16 & 3) >> 1)) ^ (4 * (j16 >> 2));
    va[dt] = (uint32_t)(r * D + chunk * 8 + (j16 & 1) * 4) * 2u;
  }
  const float sl2 = p.scale_log2;

  // S^T of one 32-key half-block (rows h*32.. of K stage ST) x this wave's 32 rows
  auto qk = [&]<int ST, int H>(float (&s)[16]) {
    const char* kb0 = reinterpret_cast<const char*>(khalf(ST, H));
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      acc = mma16(*reinterpret_cast<const bf16x8*>(kb0 + koff[kc]), qf[kc], acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = acc[i];
  };

  // Softmax of one 32-key half-block (keys key0 + reg_key(i, hh)): returns the
  // bf16 probabilities and whether O has to be rescaled by alpha first.
  // Probabilities are first taken against the current running max; only when
  // a lane's sum of them exceeds 2^8 (a score rose well above the max, or the
  // first half) is the row max formed, the max moved, and the probabilities
  // recomputed.  Exact in real arithmetic either way; keeps them < 2^8.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  auto exps = [&](const float (&s)[16], float neg_m, bf16x8 (&pf)[2]) {
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pf[c][j] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[c * 8 + j], sl2, neg_m));
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 pr = {pf[c][j], pf[c][j + 1]};
        sum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, sum, false);
      }
    }
    return sum;
  };
  auto softmax = [&]<bool MASKED>(float (&s)[16], int key0, bf16x8 (&pf)[2], float& alpha) -> bool {
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s[i] = key0 + reg_key(i, hh) > t_row ? -INFINITY : s[i];
    }
    float sum = exps(s, -m_run, pf);
    const bool need = __any(!(sum <= 256.f));
    alpha = 1.f;
    if (need) {
      // only rows whose own max rose by more than 2^8 move it; the others
      // recompute the same values with alpha = 1 (bit-identical)
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
      const float m_new = mx > m_run + 8.f ? mx : m_run;
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      sum = exps(s, -m_new, pf);
    }
    l_run = l_run * alpha + sum;
    return need;
  };

  // V^T operand fragments of one 32-key half-block H of V stage ST, read ahead
  // of the softmax whose probabilities they multiply
  auto vload = [&]<int ST, int H>(bf16x8 (&vf)[2 * NDT]) {
    const char* vb = reinterpret_cast<const char*>((ST ? smemV1 : smemV0) + (KS ? kh * TILE : 0)) + H * 32 * D * 2;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vf[c * NDT + dt] = tr_frag(vb + c * 16 * D * 2 + va[dt]);
  };
  // O += P V
  auto pv = [&](const bf16x8 (&vf)[2 * NDT], const bf16x8 (&pf)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] = mma16(vf[c * NDT + dt], pf[c], o[dt]);
  };

  auto rescale = [&](float alpha) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
  };

  // ---- prologue: K(jlo) both halves, K(jlo+1) first half, V(jlo) ----
  // (stage of block j: (j - jlo) & 1)
  const bool sweep = jlo < jhi;                     // uniform over the stage set
  float s_a[16], s_b[16];
  if constexpr (KS) {
    // both stage sets take every barrier, a set without blocks too
    if (sweep) {
      dma_rows.template operator()<0, 8>(kbase, jlo, offk, khalf(0, 0));
      dma_rows.template operator()<8, 16>(kbase, jlo, offk, khalf(0, 1));
      dma_rows.template operator()<0, 8>(kbase, clampb(jlo + 1), offk, khalf(1, 0));
      dma_rows.template operator()<0, 16>(vbase, jlo, offv, vst(0));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (sweep) qk.template operator()<0, 0>(s_a);
    __syncthreads();
  } else if (sweep) {
    dma_rows.template operator()<0, 8>(kbase, jlo, offk, khalf(0, 0));
    dma_rows.template operator()<8, 16>(kbase, jlo, offk, khalf(0, 1));
    dma_rows.template operator()<0, 8>(kbase, clampb(jlo + 1), offk, khalf(1, 0));
    dma_rows.template operator()<0, 16>(vbase, jlo, offv, vst(0));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    qk.template operator()<0, 0>(s_a);
    __syncthreads();   // every wave has read K(jlo) rows 0-31 before K(jlo+2) overwrites them
  }

  // One 64-key block j (ST = j & 1): half 0 (scores in s_a), half 1 (s_b).
  //   loads:  K(j+2) rows 0-31 -> K stage ST,   K(j+1) rows 32-63 -> K stage ST^1,
  //           V(j+1) -> V stage ST^1   (each region was last read before the
  //           previous barrier)
  //   half 0: s_b = QK(K(j) rows 32-63) while softmax(s_a); P.V with V(j) rows 0-31
  //   half 1: s_a = QK(K(j+1) rows 0-31) while softmax(s_b); P.V with V(j) rows 32-63
  auto block = [&]<bool MASKED, int ST>(int j) {
    dma_rows.template operator()<0, 8>(kbase, clampb(j + 2), offk, khalf(ST, 0));
    dma_rows.template operator()<8, 16>(kbase, clampb(j + 1), offk, khalf(ST ^ 1, 1));
    dma_rows.template operator()<0, 16>(vbase, clampb(j + 1), offv, vst(ST ^ 1));
    bf16x8 pf[2], vf[2 * NDT];
    float alpha;
    bool need;
    vload.template operator()<ST, 0>(vf);
    qk.template operator()<ST, 1>(s_b);
    need = softmax.template operator()<MASKED>(s_a, j * BN, pf, alpha);
    if (need) rescale(alpha);
    pv(vf, pf);
    vload.template operator()<ST, 1>(vf);
    qk.template operator()<ST ^ 1, 0>(s_a);
    need = softmax.template operator()<MASKED>(s_b, j * BN + 32, pf, alpha);
    if (need) rescale(alpha);
    pv(vf, pf);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  const int jmm = jm < jhi ? jm : jhi;   // unmasked blocks of this range end here
  int j = jlo;
  for (; j + 1 < jmm; j += 2) {
    block.template operator()<false, 0>(j);
    block.template operator()<false, 1>(j + 1);
  }
  if (j < jmm) { block.template operator()<false, 0>(j); ++j; }
  if (j < jhi && ((j - jlo) & 1)) { block.template operator()<true, 1>(j); ++j; }
  for (; j + 1 < jhi; j += 2) {
    block.template operator()<true, 0>(j);
    block.template operator()<true, 1>(j + 1);
  }
  if (j < jhi) { block.template operator()<true, 0>(j); ++j; }
  if constexpr (KS) {
    // set 1 sweeps at most one block more than set 0: set 0 takes its barrier
    if (kh == 0 && nblocks - 2 * (nblocks / 2) > 0) __syncthreads();
  }

  // ---- depth fold: this wave's positions only (see moda_fwd.hpp) ----
  if (wave_active && p.L_d > 0 && part != 1) {
    const int L_d = p.L_d, L_cap = p.L_cap, slot_lo = p.slot_lo;
    const long long nlo = (long long)tw_min * L_cap + slot_lo;
    const long long nhi = (long long)tw_max * L_cap + slot_lo + L_d;
    const bf16* kdb = reinterpret_cast<const bf16*>(p.kd) + (long long)bh * p.NKp * D;
    const bf16* vdb = reinterpret_cast<const bf16*>(p.vd) + (long long)bh * p.NKp * D;
    // the stages are free after the last barrier of the sweep: each wave takes
    // 32 rows (8 KB) of them -- the four K halves, then the halves of the two
    // V stages -- for its depth values
    bf16* vwave = wave < 4 ? khalf(wave >> 1, wave & 1) : ((wave < 6 ? smemV0 : smemV1) + (wave & 1) * 32 * D);
    static_assert(NW <= 8, "one 8 KB region per wave in the 64 KB of stages");
    for (long long n0 = nlo & ~31LL; n0 < nhi; n0 += 32) {
      if (!depth_tile_used(n0, L_cap, slot_lo, L_d)) continue;
      if constexpr (KS) {
        if ((int)(((n0 - (nlo & ~31LL)) >> 5) & 1) != kh) continue;   // the sets take alternate tiles
      }
      // K operand fragments (rows n0 + key_row) and this lane's share of the
      // 32 value rows (row n0 + 4 i + lane / 16, chunk lane % 16), loaded
      // together: one round trip to memory per tile
      bf16x8 kfr[NKC];
      u32x4 vr[8];
      if (p.q8) {
        // tile base (wave-uniform) plus 32-bit lane offsets
        const long long r0 = (long long)bh * p.NKp + n0;
        const int8_t* kt = reinterpret_cast<const int8_t*>(p.kd) + r0 * D;
        const int8_t* vt = reinterpret_cast<const int8_t*>(p.vd) + r0 * D;
        const float* kst = p.ksc + r0;
        const float* vst_ = p.vsc + r0;
        u32x2 kc8[NKC], vc8[8];
        float vs[8];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          kc8[kc] = *reinterpret_cast<const u32x2*>(kt + (uint32_t)(key_row * D + hh * 8 + kc * 16));
        const float ks = kst[key_row];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 4 * i + (lane >> 4);
          vc8[i] = *reinterpret_cast<const u32x2*>(vt + (uint32_t)(r * D + (lane & 15) * 8));
          vs[i] = vst_[r];
        }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kfr[kc] = dequant_frag_bf16(reinterpret_cast<const int8_t*>(&kc8[kc]), ks);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8 f = dequant_frag_bf16(reinterpret_cast<const int8_t*>(&vc8[i]), vs[i]);
          vr[i] = *reinterpret_cast<const u32x4*>(&f);
        }
      } else {
        // tile base (wave-uniform) plus 32-bit lane offsets
        const bf16* kt = kdb + n0 * D;
        const bf16* vt = vdb + n0 * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kfr[kc] = load_frag(kt + (uint32_t)(key_row * D + hh * 8 + kc * 16));
#pragma unroll
        for (int i = 0; i < 8; ++i) vr[i] = ld16(vt + (uint32_t)((4 * i + (lane >> 4)) * D + (lane & 15) * 8));
      }
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) acc = mma16(kfr[kc], qf[kc], acc);
      // value rows of unread slots (and padding) are zeroed: their weight is
      // 0, and 0 * x would still carry a non-finite x into O
      if (depth_tile_partial(n0, L_cap, slot_lo, L_d, T)) {
        const uint32_t rows_ok = depth_tile_rows(n0, L_cap, slot_lo, L_d, T, lane) >> (lane >> 4);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (!((rows_ok >> (4 * i)) & 1u)) vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
      // the value rows go to this wave's LDS region with the V-stage swizzle,
      // to be read back with the same transpose reads as the sequence blocks
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        st16(vwave + r * D + (((lane & 15) ^ (4 * (r & 3))) * 8), vr[i]);
      }
      // same arithmetic as a sequence half-block: masked raw scores, one FMA
      // into exp2; the max is exact here (these tiles are few) and the sum is
      // taken over the bf16-rounded probabilities that enter P.V
      float sv[16];
      // this row's window relative to the tile (small: the wave's rows span a
      // few positions around the tile)
      // (key reg_key(i, hh) = 16 (i >> 3) + 8 hh + (i & 7): the lane's 8 hh
      // moves to the bounds, so that each register compares with a constant)
      const int own_lo = (int)((long long)t_row * L_cap + slot_lo - n0) - 8 * hh;
      const int own_hi = own_lo + L_d;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 16 * (i >> 3) + (i & 7);
        sv[i] = (key >= own_lo && key < own_hi) ? acc[i] : -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
      if (__any(mx > m_run)) {
        const float m_new = fmaxf(mx, m_run);   // per row: alpha == 1 where it stays
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        rescale(alpha);
        m_run = m_new;
      }
      bf16x8 pf[2];
      l_run += exps(sv, -m_run, pf);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          o[dt] = mma16(tr_frag(reinterpret_cast<const char*>(vwave) + c * 16 * D * 2 + va[dt]), pf[c], o[dt]);
    }
  }

  if constexpr (KS) {
    // set 1 hands its state (O, m, l per lane) to set 0 through LDS, which
    // merges it as the online-softmax recurrence over the union of the two
    // key sets (set 0's values first, so the result does not depend on
    // timing) and writes the output.  The stages are free once every fold
    // is done.
    __syncthreads();
    float* so = reinterpret_cast<float*>((rw & 1 ? smemV1 : smemV0) + (rw < 2 ? TILE : 0));
    float* sm = reinterpret_cast<float*>(smemK00) + rw * 128;
    if (kh == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) so[(dt * 16 + i) * 64 + lane] = o[dt][i];
      sm[lane] = m_run;
      sm[64 + lane] = l_run;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m_o = sm[lane], l_o = sm[64 + lane];
    const float m_new = fmaxf(m_run, m_o);
    const float a = __builtin_amdgcn_exp2f(m_run - m_new), c = __builtin_amdgcn_exp2f(m_o - m_new);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = __builtin_fmaf(a, o[dt][i], c * so[(dt * 16 + i) * 64 + lane]);
    l_run = __builtin_fmaf(a, l_run, c * l_o);
    m_run = m_new;
  }

  if constexpr (SPLIT) {
    if (part >= 0) {
      // this wave's state to the workspace; the second of the two waves
      // (parts 0 and 1, same rows) to arrive merges and writes the output
      //
      // The two parts usually run on different XCDs, each with its own L2.
      // A device-scope fence would write back and invalidate the whole L2 of
      // the XCD (and with it the K/V blocks that its other workgroups still
      // read), so the state goes through device-coherent accesses instead:
      // relaxed device-scope atomic stores and loads (they bypass the stale
      // L2 copies), and the counter.  The wait for every store to complete
      // before the counter is incremented, and the second arrival's loads
      // issued only after its increment has returned, order the two.
      const int st = bh * p.nsplit + (p.ntiles - 1 - tile);
      float* mine = p.ws + ((long long)(st * 2 + part) * NW + wave) * (kSplitState * 64) + lane;
      float* other = p.ws + ((long long)(st * 2 + (part ^ 1)) * NW + wave) * (kSplitState * 64) + lane;
      auto put = [](float* a, float v) { __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      auto get = [](float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) put(mine + (dt * 16 + i) * 64, o[dt][i]);
      put(mine + 64 * 64, m_run);
      put(mine + 65 * 64, l_run);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every store of the state has completed
      uint32_t ticket = 0;
      if (lane == 0)
        ticket = __hip_atomic_fetch_add(p.cnt + st * NW + wave, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ticket = __builtin_amdgcn_readfirstlane(ticket);
      if (ticket == 0) return;                  // the other part merges
      asm volatile("" ::: "memory");            // its state is read only now
      // the merge is written in terms of part 0 and part 1 whichever of them
      // arrives second (x = fma(s0, x0, s1 * x1)), so repeated calls agree
      // bit for bit
      const float m_o = get(other + 64 * 64), l_o = get(other + 65 * 64);
      const float m_new = fmaxf(m_run, m_o);
      const float a = __builtin_amdgcn_exp2f(m_run - m_new), c = __builtin_amdgcn_exp2f(m_o - m_new);
      const bool p0 = part == 0;
      const float s0 = p0 ? a : c, s1 = p0 ? c : a;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = o[dt][i], y = get(other + (dt * 16 + i) * 64);
          o[dt][i] = __builtin_fmaf(s0, p0 ? x : y, s1 * (p0 ? y : x));
        }
      l_run = __builtin_fmaf(s0, p0 ? l_run : l_o, s1 * (p0 ? l_o : l_run));
      m_run = m_new;
      if (lane == 0) __hip_atomic_store(p.cnt + st * NW + wave, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  // The output address is formed anew here rather than kept from the Q load
  // through the sweep (a 64-bit value the register allocator would otherwise
  // park in scratch), and the lane half comes from the lane count.
  int t_out = t_row, h_out = hq;
  asm volatile("" : "+v"(t_out), "+v"(h_out));
  const int hh_out = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
  if (row_ok) {
    const float inv = 1.f / l_tot;
    bf16* op = reinterpret_cast<bf16*>(p.out) + (((long long)b * T + t_out) * p.Hq + h_out) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        store4(op + dt * 32 + g4 * 8 + hh_out * 4, o[dt][g4 * 4 + 0] * inv, o[dt][g4 * 4 + 1] * inv,
               o[dt][g4 * 4 + 2] * inv, o[dt][g4 * 4 + 3] * inv);
    if (hh_out == 0 && p.lse)
      p.lse[((long long)b * p.Hq + h_out) * T + t_out] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
  if constexpr (DYN) {
    // every wave counts itself out; the last of the launch returns the
    // counter slot to zero for the next launch that draws it (every
    // workgroup has taken its work item before any of its waves gets here)
    if (p.tick && lane == 0) {
      const uint32_t done = __hip_atomic_fetch_add(p.tick + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == gridDim.x * (uint32_t)NW - 1u) {
        __hip_atomic_store(p.tick, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.tick + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace moda
