// C ABI of libmoda.so (declared in include/moda.h): argument validation,
// kernel selection and launch on the caller's stream.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <atomic>
#include <mutex>

#include "moda.h"
#include "moda_bwd.hpp"
#include "moda_fwd.hpp"
#include "moda_fwd_bf16.hpp"
#include "moda_pack.hpp"

namespace {

// Products of sizes (all >= 0), saturated at LLONG_MAX instead of
// overflowing: validation compares them with limits, so a saturated product
// is rejected like any other too-large one.
long long smul(long long a, long long b) {
  if (a == 0 || b == 0) return 0;
  return a > LLONG_MAX / b ? LLONG_MAX : a * b;
}
long long smul(long long a, long long b, long long c) { return smul(smul(a, b), c); }
long long smul(long long a, long long b, long long c, long long e) { return smul(smul(a, b, c), e); }
// ceil(x / y) for x >= 0, y > 0, without overflow
long long cdiv(long long x, long long y) { return x / y + (x % y != 0); }

constexpr int kWaves = 4;          // waves per workgroup of the forward kernels

// Waves per workgroup of the forward for (dtype, d, shape): the bf16 d = 128
// kernel takes 8 waves (256 rows) when that still gives at least two
// workgroups per compute unit of a 256-CU GPU, else 4 (128 rows) like the
// generic kernel.
constexpr long long kCUs = 256;     // compute units of an MI355X
int fwd_waves(int dtype, int d, long long rows, long long BH) {
  if (dtype == MODA_BF16 && d == 128 && smul((rows + 255) / 256, BH) >= 2 * kCUs) return 8;
  return kWaves;
}


// Multiply-shift constants of moda::div_g for the divisor x >= 1:
// magic = ceil(2^(31+s) / x), s = ceil(log2 x), shift = 31 + s.
void div_magic(int x, uint32_t* magic, int* shift) {
  int sh = 0;
  while ((1LL << sh) < x) ++sh;
  const unsigned long long num = 1ULL << (31 + sh);
  *magic = (uint32_t)((num + (unsigned long long)x - 1) / (unsigned long long)x);
  *shift = 31 + sh;
}

bool valid_dtype(int dtype) { return dtype == MODA_F32 || dtype == MODA_BF16; }
bool supported_d(int d) { return d == 64 || d == 128; }

long long padded_depth_keys(int T, int L_d) {
  const long long n = (long long)T * L_d;
  return (n + 31) / 32 * 32;
}

// Split key ranges for the bf16 d = 128 kernel on grids of at most two
// workgroups per compute unit (four-wave tiles): the longest half of the
// query tiles of each (b, kv head) is swept by two workgroups each (see
// moda_fwd_bf16.hpp).  Workspace: the arrival counters in a header of fixed
// size (the most (split tile, wave) pairs any shape has: a grid of at most
// 2 * kCUs tiles splits at most kCUs of them, 4 waves each), so that the
// counters of one shape never overlap the partial states of another that
// used the same workspace before; then the partial states of both parts of
// every wave.
constexpr long long kSplitCntBytes = 2 * kCUs / 2 * 4 * 4;
// Grids of the bf16 d = 128 kernel that fit in one round of one eight-wave
// workgroup per compute unit over 128-row tiles: the key-split layout, whose
// two sets of four waves split each tile's key blocks (and depth tiles).
// With a second round the two rounds' depth folds come one after the other,
// and at T = 4K, G = 8, Hkv = 2 that costs more than the split saves.
bool fwd_key_split(int dtype, int d, long long rows, long long BH) {
  return dtype == MODA_BF16 && d == 128 && fwd_waves(dtype, d, rows, BH) == 4 &&
         smul((rows + 127) / 128, BH) <= kCUs && rows > 128;
}

struct SplitPlan {
  int nsplit = 0;          // split tiles per (b, kv head)
  long long cnt_bytes = 0; // counter header
  long long bytes = 0;     // whole workspace
};
SplitPlan split_plan(int dtype, int d, long long rows, long long BH) {
  SplitPlan sp;
  if (fwd_waves(dtype, d, rows, BH) != 4 || dtype != MODA_BF16 || d != 128) return sp;
  if (fwd_key_split(dtype, d, rows, BH)) return sp;   // split inside the workgroup instead
  const long long ntiles = (rows + 127) / 128;
  if (smul(ntiles, BH) > 2 * kCUs || ntiles < 2) return sp;
  sp.nsplit = (int)(ntiles / 2);
  const long long units = BH * sp.nsplit * 4;    // (split tile, wave) pairs, <= kSplitCntBytes / 4
  sp.cnt_bytes = kSplitCntBytes;
  sp.bytes = sp.cnt_bytes + units * 2 * moda::kSplitState * 64 * 4;
  return sp;
}

// Which dK/dV kernel the backward runs for bf16 with d = 128: the kernel laid
// out for the gfx950 memory path addresses one kv head's lse rows with 32-bit
// offsets, and with G not dividing 64 also one batch's q / dO rows (with G
// dividing 64 those offsets stay within one 64-row block).
enum class DkdvForm { generic, whole_positions, any_g };
DkdvForm dkdv_form(int dtype, int d, int T, int G, int Hq) {
  if (dtype != MODA_BF16 || d != 128) return DkdvForm::generic;
  const bool lse32 = (long long)T * G * 4 < 0x7fffffffLL;
  const bool q32 = (long long)T * Hq * d * 2 < 0x7fffffffLL;
  if (lse32 && 64 % G == 0) return DkdvForm::whole_positions;
  if (lse32 && q32) return DkdvForm::any_g;
  return DkdvForm::generic;
}

// The backward's workspace (moda_bwd_ws): the work buffer (2 * B * Hq * T
// floats, padded to 256 bytes), then, when the dK/dV rows are split, 128 KiB
// of float32 partial sums per (chunk, b, kv head).  One dK/dV workgroup runs
// per compute unit.
struct BwdWsPlan {
  moda::BwdSplitPlan split;
  long long work_bytes = 0;
  long long bytes = 0;
};
BwdWsPlan bwd_ws_plan(int B, int T, int Hq, int Hkv, int d, int dtype) {
  BwdWsPlan wp;
  const int G = Hq / Hkv;
  const long long work = smul(2LL * B, Hq, T, 4);
  if (work > LLONG_MAX / 2) {                   // saturated: no such buffer
    wp.work_bytes = wp.bytes = LLONG_MAX;
    return wp;
  }
  wp.work_bytes = (work + 255) / 256 * 256;
  if (dkdv_form(dtype, d, T, G, Hq) != DkdvForm::generic)
    wp.split = moda::bwd_split_plan(T, G, (long long)B * Hkv, (int)cdiv(T, 128), (int)kCUs);
  const long long part = smul((long long)B * Hkv, wp.split.items, 32768 * 4);
  wp.bytes = part > LLONG_MAX - wp.work_bytes ? LLONG_MAX : wp.work_bytes + part;
  return wp;
}

template <typename E, int D>
hipError_t launch_fwd(const moda::FwdParams& p, unsigned grid, int nw, hipStream_t s) {
  if constexpr (sizeof(E) == 2 && D == 128) {
    if (p.nsplit > 0)
      hipLaunchKernelGGL((moda::moda_fwd_bf16_kernel<D, 4, true>), dim3(grid), dim3(4 * 64), 0, s, p);
    else if (nw == -8)
      hipLaunchKernelGGL((moda::moda_fwd_bf16_kernel<D, 8, false, true>), dim3(grid), dim3(8 * 64), 0, s, p);
    else if (nw == 8)
      hipLaunchKernelGGL((moda::moda_fwd_bf16_kernel<D, 8>), dim3(grid), dim3(8 * 64), 0, s, p);
    else
      hipLaunchKernelGGL((moda::moda_fwd_bf16_kernel<D, 4>), dim3(grid), dim3(4 * 64), 0, s, p);
  } else {
    hipLaunchKernelGGL((moda::moda_fwd_kernel<E, D, kWaves>), dim3(grid), dim3(kWaves * 64), 0, s, p);
  }
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_append(const moda::AppendParams& p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((moda::moda_append_depth_kernel<E, D>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_pack(const moda::PackParams& p, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((moda::moda_pack_depth_kernel<E, D>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_bwd(const moda::BwdParams& p, hipStream_t s) {
  constexpr int ve = 16 / sizeof(E);
  const long long rows = (long long)p.B * p.T * p.Hq;
  const long long rpb = 256 / (D / ve);
  hipLaunchKernelGGL((moda::moda_bwd_delta_kernel<E, D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, s, p);
  // each launch is checked before the next, so that a failed launch is not
  // hidden behind the ones after it
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned BH = (unsigned)(p.B * p.Hkv);
  if constexpr (sizeof(E) == 2 && D == 128)
    hipLaunchKernelGGL((moda::moda_bwd_dq_bf16_kernel<D>), dim3(BH * p.ntiles), dim3(kWaves * 64), 0, s, p);
  else
    hipLaunchKernelGGL((moda::moda_bwd_dq_kernel<E, D, kWaves>), dim3(BH * p.ntiles), dim3(kWaves * 64), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (sizeof(E) == 2 && D == 128) {
    const DkdvForm form = dkdv_form(MODA_BF16, D, p.T, p.G, p.Hq);
    if (p.kchunk > 0) {
      // row-split: chunk_items workgroups per (b, kv head), then the sums
      const unsigned grid = BH * (unsigned)p.kitems;
      if (form == DkdvForm::whole_positions)
        hipLaunchKernelGGL((moda::moda_bwd_dkdv_bf16_kernel<D, true, true>), dim3(grid), dim3(kWaves * 64), 0, s, p);
      else
        hipLaunchKernelGGL((moda::moda_bwd_dkdv_bf16_kernel<D, false, true>), dim3(grid), dim3(kWaves * 64), 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_reduce_kernel<D>), dim3(BH * p.nktiles), dim3(256), 0, s, p);
    } else if (form == DkdvForm::whole_positions) {
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_bf16_kernel<D, true>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
    } else if (form == DkdvForm::any_g) {
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_bf16_kernel<D, false>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
    } else {
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_kernel<E, D, kWaves>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
    }
  } else {
    hipLaunchKernelGGL((moda::moda_bwd_dkdv_kernel<E, D, kWaves>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.L_d > 0) {
    // whole positions per 32-row wave (G divides 32): the matrix-core depth kernel
    if (sizeof(E) == 2 && D == 128 && 32 % p.G == 0)
      hipLaunchKernelGGL((moda::moda_bwd_depth_bf16_kernel<128>), dim3(BH * p.ntiles), dim3(kWaves * 64), 0, s, p);
    else
      hipLaunchKernelGGL((moda::moda_bwd_depth_kernel<E, D>), dim3((unsigned)((long long)p.T * BH)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

const char* moda_status_string(int status) {
  switch (status) {
    case MODA_OK: return "MODA_OK";
    case MODA_ERR_NULL: return "MODA_ERR_NULL: a required pointer is NULL";
    case MODA_ERR_SHAPE: return "MODA_ERR_SHAPE: a size is out of range or inconsistent";
    case MODA_ERR_DTYPE: return "MODA_ERR_DTYPE: unknown dtype";
    case MODA_ERR_UNSUPPORTED: return "MODA_ERR_UNSUPPORTED: head size must be 64 or 128";
    case MODA_ERR_HIP: return "MODA_ERR_HIP: the HIP runtime reported an error";
    case MODA_ERR_WORKSPACE:
      return "MODA_ERR_WORKSPACE: the workspace is NULL, misaligned or too small (moda_fwd_workspace_bytes), "
             "or the sizes need more than the static scratch of moda_bwd_noalloc (B * Hq * T > 4194304)";
    default: return "unknown moda_status";
  }
}

long long moda_depth_packed_elems(int B, int T, int Hkv, int d, int L_d) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || L_d < 0) return -1;
  if ((long long)T * L_d > 0x7fffffffLL - 32) return -1;           // packed key index is 31-bit
  const long long n = smul(B, Hkv, padded_depth_keys(T, L_d), d);
  return n == LLONG_MAX ? -1 : n;
}

int moda_pack_depth(const void* k_depth, const void* v_depth, void* k_packed, void* v_packed,
                    int B, int T, int Hkv, int d, int L_d, int dtype, void* stream) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || L_d < 0) return MODA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (L_d == 0) return MODA_OK;
  if (!k_depth || !v_depth || !k_packed || !v_packed) return MODA_ERR_NULL;
  if ((long long)T * L_d > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;
  moda::PackParams p{k_depth, v_depth, k_packed, v_packed, B, T, Hkv, L_d, padded_depth_keys(T, L_d)};
  const int ve = dtype == MODA_BF16 ? 8 : 4;
  const long long grid = cdiv(smul(B, Hkv, p.NKp, d / ve), 256);
  if (grid > 0x7fffffffLL) return MODA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_pack<moda::bf16, 128>(p, (unsigned)grid, s) : launch_pack<moda::bf16, 64>(p, (unsigned)grid, s);
  else
    e = d == 128 ? launch_pack<float, 128>(p, (unsigned)grid, s) : launch_pack<float, 64>(p, (unsigned)grid, s);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

// Launch counters of the grids of several rounds (the eight-wave forward,
// the backward's dQ and dK/dV kernels: work items drawn in the order
// workgroups start): a ring of slots in a file-scope device array, one copy
// per GPU, zero at load; each launch takes the next slot and leaves it at
// zero when it ends, so launches in flight at the same time on one GPU (other
// streams) use different slots as long as fewer than kTickSlots of them
// overlap.  The per-device address comes from hipGetSymbolAddress, once per
// device; without it a grid keeps the blockIdx order.
constexpr int kMaxDevices = 64;   // GPUs per process the per-device state is kept for
constexpr int kTickSlots = 1024;
static __device__ __align__(256) uint32_t work_tick[moda::kTickWords * kTickSlots];
static std::mutex g_tick_mu;
static uint32_t* g_tick_ptr[kMaxDevices] = {};
static std::atomic<uint32_t> g_tick_next{0};

static uint32_t* tick_slot() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint32_t* base;
  {
    std::lock_guard<std::mutex> lock(g_tick_mu);
    if (!g_tick_ptr[dev]) {
      void* a = nullptr;
      if (hipGetSymbolAddress(&a, HIP_SYMBOL(work_tick)) != hipSuccess || !a) return nullptr;
      g_tick_ptr[dev] = static_cast<uint32_t*>(a);
    }
    base = g_tick_ptr[dev];
  }
  return base + moda::kTickWords * (g_tick_next.fetch_add(1, std::memory_order_relaxed) % kTickSlots);
}

static int fwd_impl(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, const float* k_scale, const float* v_scale, int q8, void* out,
                    float* lse, int B, int T, int Hq, int Hkv, int d, int L_cap, int slot_lo, int slot_hi,
                    int dtype, void* stream, void* work = nullptr, long long work_bytes = 0) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1 || L_cap < 0) return MODA_ERR_SHAPE;
  if (slot_lo < 0 || slot_hi < slot_lo || slot_hi > L_cap) return MODA_ERR_SHAPE;
  if ((long long)T * L_cap > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;   // packed key index is 31-bit
  if (Hq % Hkv != 0) return MODA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (!q || !k_seq || !v_seq || !out) return MODA_ERR_NULL;
  const int L_d = slot_hi - slot_lo;
  if (L_d > 0 && (!k_depth || !v_depth)) return MODA_ERR_NULL;
  if (L_d > 0 && q8 && (!k_scale || !v_scale)) return MODA_ERR_NULL;
  const int G = Hq / Hkv;
  const long long rows = (long long)T * G;
  int nw = fwd_waves(dtype, d, rows, (long long)B * Hkv);
  const bool ks = fwd_key_split(dtype, d, rows, (long long)B * Hkv);
  const int tile_rows = 32 * nw;   // 128 for the key-split layout too
  const long long ntiles = (rows + tile_rows - 1) / tile_rows;
  const long long grid = smul(ntiles, B, Hkv);
  if (grid > 0x7fffffffLL || rows > 0x7fffffffLL) return MODA_ERR_SHAPE;

  moda::FwdParams p;
  p.q = q; p.k = k_seq; p.v = v_seq; p.kd = k_depth; p.vd = v_depth;
  p.ksc = k_scale; p.vsc = v_scale; p.q8 = q8;
  p.out = out; p.lse = lse;
  p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.G = G;
  p.L_d = L_d; p.L_cap = L_cap > 0 ? L_cap : 1; p.slot_lo = slot_lo;
  p.ntiles = (int)ntiles;
  // at most two workgroups per compute unit for the whole grid: pair long
  // tiles with short ones (with more rounds, longest first balances by itself)
  p.paired = !ks && grid <= 2 * kCUs && B * Hkv <= kCUs && kCUs % (B * Hkv) == 0;
  p.NKp = padded_depth_keys(T, L_cap);
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  p.nsplit = 0;
  p.ws = nullptr;
  p.cnt = nullptr;
  long long launch_grid = grid;
  if (work) {
    const SplitPlan sp = split_plan(dtype, d, rows, (long long)B * Hkv);
    if (sp.nsplit > 0) {
      if (work_bytes < sp.bytes || (reinterpret_cast<uintptr_t>(work) & 255)) return MODA_ERR_WORKSPACE;
      p.nsplit = sp.nsplit;
      p.cnt = reinterpret_cast<uint32_t*>(work);
      p.ws = reinterpret_cast<float*>(reinterpret_cast<char*>(work) + sp.cnt_bytes);
      launch_grid = (ntiles + sp.nsplit) * B * Hkv;
    }
  }
  if (ks && p.nsplit == 0) nw = -8;   // (launch_fwd: the key-split instantiation)
  p.tick = nullptr;
  if (dtype == MODA_BF16 && d == 128 && nw == 8 && launch_grid > kCUs && launch_grid * 8 < 0xffffffffLL)
    p.tick = tick_slot();

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_fwd<moda::bf16, 128>(p, (unsigned)launch_grid, nw, s) : launch_fwd<moda::bf16, 64>(p, (unsigned)grid, nw, s);
  else
    e = d == 128 ? launch_fwd<float, 128>(p, (unsigned)grid, nw, s) : launch_fwd<float, 64>(p, (unsigned)grid, nw, s);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_fwd_window(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, void* out, float* lse, int B, int T, int Hq, int Hkv, int d,
                    int L_cap, int slot_lo, int slot_hi, int dtype, void* stream) {
  return fwd_impl(q, k_seq, v_seq, k_depth, v_depth, nullptr, nullptr, 0, out, lse, B, T, Hq, Hkv, d,
                  L_cap, slot_lo, slot_hi, dtype, stream);
}

int moda_fwd_window_q8(const void* q, const void* k_seq, const void* v_seq, const int8_t* k_q,
                       const int8_t* v_q, const float* k_scale, const float* v_scale, void* out,
                       float* lse, int B, int T, int Hq, int Hkv, int d, int L_cap, int slot_lo,
                       int slot_hi, int dtype, void* stream) {
  return fwd_impl(q, k_seq, v_seq, k_q, v_q, k_scale, v_scale, 1, out, lse, B, T, Hq, Hkv, d, L_cap,
                  slot_lo, slot_hi, dtype, stream);
}

int moda_append_depth_q8(const void* k_new, const void* v_new, int8_t* k_q, int8_t* v_q,
                         float* k_scale, float* v_scale, int B, int T, int Hkv, int d, int L_cap,
                         int slot, int dtype, void* stream) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || L_cap < 1) return MODA_ERR_SHAPE;
  if (slot < 0 || slot >= L_cap) return MODA_ERR_SHAPE;
  if ((long long)T * L_cap > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;   // packed key index is 31-bit
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !k_q || !v_q || !k_scale || !v_scale) return MODA_ERR_NULL;
  moda::AppendQ8Params p{k_new, v_new, k_q, v_q, k_scale, v_scale, B, T, Hkv, L_cap, slot,
                         padded_depth_keys(T, L_cap)};
  const long long rows = smul(B, T, Hkv);
  const long long rpb = 256 / (d / moda::kQ8Elems);
  const long long grid = cdiv(rows, rpb);
  if (grid > 0x7fffffffLL) return MODA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == MODA_BF16) {
    if (d == 128) hipLaunchKernelGGL((moda::moda_append_depth_q8_kernel<moda::bf16, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((moda::moda_append_depth_q8_kernel<moda::bf16, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
  } else {
    if (d == 128) hipLaunchKernelGGL((moda::moda_append_depth_q8_kernel<float, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((moda::moda_append_depth_q8_kernel<float, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_fwd_q8(const void* q, const void* k_seq, const void* v_seq, const int8_t* k_q,
                const int8_t* v_q, const float* k_scale, const float* v_scale, void* out, float* lse,
                int B, int T, int Hq, int Hkv, int d, int L_d, int dtype, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return fwd_impl(q, k_seq, v_seq, k_q, v_q, k_scale, v_scale, 1, out, lse, B, T, Hq, Hkv, d, L_d, 0,
                  L_d, dtype, stream);
}

int moda_pack_depth_q8(const void* k_depth, const void* v_depth, int8_t* k_q, int8_t* v_q,
                       float* k_scale, float* v_scale, int B, int T, int Hkv, int d, int L_d, int dtype,
                       void* stream) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || L_d < 0) return MODA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (L_d == 0) return MODA_OK;
  if (!k_depth || !v_depth || !k_q || !v_q || !k_scale || !v_scale) return MODA_ERR_NULL;
  if ((long long)T * L_d > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;
  moda::PackQ8Params p{k_depth, v_depth, k_q, v_q, k_scale, v_scale, B, T, Hkv, L_d, padded_depth_keys(T, L_d)};
  div_magic(L_d, &p.ld_magic, &p.ld_shift);
  // blocks of rows x (b, kv head) planes, planes fastest; launches of at most
  // 2^31 - 1 workgroups
  const long long rpb = 2 * (256 / (d / moda::kQ8Elems));     // two rows per lane group
  const long long nrb = (p.NKp + rpb - 1) / rpb;
  const long long planes = (long long)B * Hkv;
  if (planes > 0x7fffffffLL) return MODA_ERR_SHAPE;
  const long long per = 0x7fffffffLL / planes;                  // row blocks per launch
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (long long rb0 = 0; rb0 < nrb; rb0 += per) {
    p.rb0 = rb0;
    const dim3 grid((unsigned)((nrb - rb0 < per ? nrb - rb0 : per) * planes));
    if (dtype == MODA_BF16) {
      if (d == 128) hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<moda::bf16, 128>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<moda::bf16, 64>), grid, dim3(256), 0, s, p);
    } else {
      if (d == 128) hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<float, 128>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<float, 64>), grid, dim3(256), 0, s, p);
    }
    if (hipGetLastError() != hipSuccess) return MODA_ERR_HIP;
  }
  return MODA_OK;
}

int moda_fwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
             const void* v_depth, void* out, float* lse, int B, int T, int Hq, int Hkv, int d,
             int L_d, int dtype, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return moda_fwd_window(q, k_seq, v_seq, k_depth, v_depth, out, lse, B, T, Hq, Hkv, d, L_d, 0, L_d,
                         dtype, stream);
}

long long moda_fwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d, int dtype) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0) return -1;
  if (!valid_dtype(dtype)) return -1;
  if (!supported_d(d)) return 0;
  return split_plan(dtype, d, (long long)T * (Hq / Hkv), (long long)B * Hkv).bytes;
}

int moda_fwd_ws(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                const void* v_depth, void* out, float* lse, int B, int T, int Hq, int Hkv, int d,
                int L_d, int dtype, void* work, long long work_bytes, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  if (!work) return MODA_ERR_WORKSPACE;
  return fwd_impl(q, k_seq, v_seq, k_depth, v_depth, nullptr, nullptr, 0, out, lse, B, T, Hq, Hkv, d, L_d, 0,
                  L_d, dtype, stream, work, work_bytes);
}

int moda_append_depth(const void* k_new, const void* v_new, void* k_packed, void* v_packed, int B,
                      int T, int Hkv, int d, int L_cap, int slot, int dtype, void* stream) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || L_cap < 1) return MODA_ERR_SHAPE;
  if (slot < 0 || slot >= L_cap) return MODA_ERR_SHAPE;
  if ((long long)T * L_cap > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;   // packed key index is 31-bit
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !k_packed || !v_packed) return MODA_ERR_NULL;
  moda::AppendParams p{k_new, v_new, k_packed, v_packed, B, T, Hkv, L_cap, slot, padded_depth_keys(T, L_cap)};
  const int ve = dtype == MODA_BF16 ? 8 : 4;
  const long long threads = smul(B, T, Hkv, d / ve);
  const long long grid = cdiv(threads, 256);
  if (grid > 0x7fffffffLL) return MODA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_append<moda::bf16, 128>(p, (unsigned)grid, s) : launch_append<moda::bf16, 64>(p, (unsigned)grid, s);
  else
    e = d == 128 ? launch_append<float, 128>(p, (unsigned)grid, s) : launch_append<float, 64>(p, (unsigned)grid, s);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

// The backward's work buffer for callers that cannot allocate
// (moda_bwd_noalloc): a file-scope device array, one copy per GPU, held until
// the process ends.  Host code never uses its name as an address: the
// per-device address comes from hipGetSymbolAddress, taken once per device on
// the first call there with that device current.
constexpr long long kScratchFloats = 8LL << 20;                  // 32 MiB: B * Hq * T <= 4M rows
static __device__ __align__(256) float scratch[kScratchFloats];
static std::mutex g_scratch_mu;
static float* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch, or an error status.
static int device_scratch(float** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MODA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return MODA_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<float*>(a);
  }
  *ptr = g_scratch_ptr[dev];
  return MODA_OK;
}

// work == nullptr with use_scratch: the work buffer is the device's static
// scratch (checked against its size after the other arguments).  With use_ws
// the work buffer and the row-split dK/dV partial sums come from the caller's
// workspace ws of ws_bytes bytes (bwd_ws_plan).
static int bwd_impl(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, const float* k_scale, const float* v_scale, int q8,
                    const void* out, const float* lse, const void* dout, void* dq,
                    void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, float* work, int B,
                    int T, int Hq, int Hkv, int d, int L_cap, int slot_lo, int slot_hi, int dtype,
                    void* stream, bool use_scratch = false, void* ws = nullptr, long long ws_bytes = 0,
                    bool use_ws = false) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1 || L_cap < 0) return MODA_ERR_SHAPE;
  if (slot_lo < 0 || slot_hi < slot_lo || slot_hi > L_cap) return MODA_ERR_SHAPE;
  if ((long long)T * L_cap > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;   // packed key index is 31-bit
  if (Hq % Hkv != 0) return MODA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (!q || !k_seq || !v_seq || !out || !lse || !dout || !dq || !dk_seq || !dv_seq ||
      (!work && !use_scratch && !use_ws))
    return MODA_ERR_NULL;
  const int L_d = slot_hi - slot_lo;
  if (L_d > 0 && (!k_depth || !v_depth || !dk_depth || !dv_depth)) return MODA_ERR_NULL;
  if (L_d > 0 && q8 && (!k_scale || !v_scale)) return MODA_ERR_NULL;
  const int G = Hq / Hkv;
  const long long rows = (long long)T * G;
  const long long ntiles = (rows + 32 * kWaves - 1) / (32 * kWaves);
  const long long nktiles = ((long long)T + 32 * kWaves - 1) / (32 * kWaves);
  const long long BH = (long long)B * Hkv;
  if (smul(ntiles, BH) > 0x7fffffffLL || smul(T, BH) > 0x7fffffffLL || rows > 0x7fffffffLL ||
      smul(B, T, Hq) > 0x7fffffffLL * 4)
    return MODA_ERR_SHAPE;

  if (use_scratch) {
    if (2LL * B * Hq * T > kScratchFloats) return MODA_ERR_WORKSPACE;
    const int st = device_scratch(&work);
    if (st != MODA_OK) return st;
  }
  moda::BwdSplitPlan split;
  float* part = nullptr;
  if (use_ws) {
    const BwdWsPlan wp = bwd_ws_plan(B, T, Hq, Hkv, d, dtype);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < wp.bytes) return MODA_ERR_WORKSPACE;
    if (smul(BH, wp.split.items) > 0x7fffffffLL) return MODA_ERR_SHAPE;
    work = static_cast<float*>(ws);
    split = wp.split;
    if (split.C > 0) part = reinterpret_cast<float*>(static_cast<char*>(ws) + wp.work_bytes);
  }

  moda::BwdParams p;
  p.q = q; p.k = k_seq; p.v = v_seq; p.kd = k_depth; p.vd = v_depth;
  p.ksc = k_scale; p.vsc = v_scale; p.q8 = q8;
  p.o = out; p.dO = dout; p.lse = lse; p.work = work; p.BHT = (long long)B * Hq * T;
  p.dq = dq; p.dk = dk_seq; p.dv = dv_seq; p.dkd = dk_depth; p.dvd = dv_depth;
  p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.G = G;
  p.L_d = L_d; p.L_cap = L_cap > 0 ? L_cap : 1; p.slot_lo = slot_lo;
  p.ntiles = (int)ntiles;
  p.nktiles = (int)nktiles;
  p.NKp = padded_depth_keys(T, L_cap);
  p.scale = (float)(1.0 / sqrt((double)d));
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  div_magic(G, &p.g_magic, &p.g_shift);
  p.part = part;
  p.kchunk = split.C;
  p.kfull = split.full;
  p.kitems = split.items;
  // grids of several rounds take their work items from launch counters
  // (one queue per (b, kv head) pair, at most kTickWords - 1 pairs): dQ (two
  // workgroups per compute unit) and the unsplit bf16 dK/dV kernel (one per
  // compute unit)
  p.tick_dq = p.tick_kv = nullptr;
  if (dtype == MODA_BF16 && d == 128 && (long long)B * Hkv <= moda::kTickWords - 1) {
    const long long gq = (long long)B * Hkv * ntiles, gk = (long long)B * Hkv * nktiles;
    if (gq > 2 * kCUs && gq * 4 < 0xffffffffLL) p.tick_dq = tick_slot();
    if (split.C == 0 && dkdv_form(dtype, d, T, G, Hq) != DkdvForm::generic && gk > kCUs && gk * 4 < 0xffffffffLL)
      p.tick_kv = tick_slot();
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_bwd<moda::bf16, 128>(p, s) : launch_bwd<moda::bf16, 64>(p, s);
  else
    e = d == 128 ? launch_bwd<float, 128>(p, s) : launch_bwd<float, 64>(p, s);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_bwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
             const void* v_depth, const void* out, const float* lse, const void* dout, void* dq,
             void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, float* work, int B, int T,
             int Hq, int Hkv, int d, int L_d, int dtype, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return bwd_impl(q, k_seq, v_seq, k_depth, v_depth, nullptr, nullptr, 0, out, lse, dout, dq, dk_seq,
                  dv_seq, dk_depth, dv_depth, work, B, T, Hq, Hkv, d, L_d, 0, L_d, dtype, stream);
}

long long moda_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d, int dtype) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0) return -1;
  if (!valid_dtype(dtype)) return -1;
  const long long n = bwd_ws_plan(B, T, Hq, Hkv, d, dtype).bytes;
  return n == LLONG_MAX ? -1 : n;
}

int moda_bwd_ws(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                const void* v_depth, const void* out, const float* lse, const void* dout, void* dq,
                void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, int B, int T, int Hq,
                int Hkv, int d, int L_d, int dtype, void* work, long long work_bytes, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return bwd_impl(q, k_seq, v_seq, k_depth, v_depth, nullptr, nullptr, 0, out, lse, dout, dq, dk_seq,
                  dv_seq, dk_depth, dv_depth, nullptr, B, T, Hq, Hkv, d, L_d, 0, L_d, dtype, stream, false,
                  work, work_bytes, true);
}

int moda_bwd_noalloc(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                     const void* v_depth, const void* out, const float* lse, const void* dout, void* dq,
                     void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, int B, int T, int Hq,
                     int Hkv, int d, int L_d, int dtype, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return bwd_impl(q, k_seq, v_seq, k_depth, v_depth, nullptr, nullptr, 0, out, lse, dout, dq, dk_seq,
                  dv_seq, dk_depth, dv_depth, nullptr, B, T, Hq, Hkv, d, L_d, 0, L_d, dtype, stream, true);
}

int moda_bwd_window(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, const void* out, const float* lse, const void* dout, void* dq,
                    void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, float* work, int B,
                    int T, int Hq, int Hkv, int d, int L_cap, int slot_lo, int slot_hi, int dtype,
                    void* stream) {
  return bwd_impl(q, k_seq, v_seq, k_depth, v_depth, nullptr, nullptr, 0, out, lse, dout, dq, dk_seq,
                  dv_seq, dk_depth, dv_depth, work, B, T, Hq, Hkv, d, L_cap, slot_lo, slot_hi, dtype,
                  stream);
}

int moda_bwd_q8(const void* q, const void* k_seq, const void* v_seq, const int8_t* k_q, const int8_t* v_q,
                const float* k_scale, const float* v_scale, const void* out, const float* lse,
                const void* dout, void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth,
                float* work, int B, int T, int Hq, int Hkv, int d, int L_d, int dtype, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return bwd_impl(q, k_seq, v_seq, k_q, v_q, k_scale, v_scale, 1, out, lse, dout, dq, dk_seq, dv_seq,
                  dk_depth, dv_depth, work, B, T, Hq, Hkv, d, L_d, 0, L_d, dtype, stream);
}

int moda_bwd_window_q8(const void* q, const void* k_seq, const void* v_seq, const int8_t* k_q,
                       const int8_t* v_q, const float* k_scale, const float* v_scale, const void* out,
                       const float* lse, const void* dout, void* dq, void* dk_seq, void* dv_seq,
                       void* dk_depth, void* dv_depth, float* work, int B, int T, int Hq, int Hkv, int d,
                       int L_cap, int slot_lo, int slot_hi, int dtype, void* stream) {
  return bwd_impl(q, k_seq, v_seq, k_q, v_q, k_scale, v_scale, 1, out, lse, dout, dq, dk_seq, dv_seq,
                  dk_depth, dv_depth, work, B, T, Hq, Hkv, d, L_cap, slot_lo, slot_hi, dtype, stream);
}

}  // extern "C"
