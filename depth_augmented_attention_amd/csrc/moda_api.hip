// C ABI of libmoda.so (declared in include/moda.h): argument validation,
// kernel selection and launch on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>

#include "moda.h"
#include "moda_bwd.hpp"
#include "moda_fwd.hpp"
#include "moda_fwd_bf16.hpp"
#include "moda_pack.hpp"

namespace {

constexpr int kWaves = 4;          // waves per workgroup of the forward kernels

// Waves per workgroup of the forward for (dtype, d, shape): the bf16 d = 128
// kernel takes 8 waves (256 rows) when that still gives at least two
// workgroups per compute unit of a 256-CU GPU, else 4 (128 rows) like the
// generic kernel.
constexpr long long kCUs = 256;     // compute units of an MI355X
int fwd_waves(int dtype, int d, long long rows, long long BH) {
  if (dtype == MODA_BF16 && d == 128 && (rows + 255) / 256 * BH >= 2 * kCUs) return 8;
  return kWaves;
}

bool valid_dtype(int dtype) { return dtype == MODA_F32 || dtype == MODA_BF16; }
bool supported_d(int d) { return d == 64 || d == 128; }

long long padded_depth_keys(int T, int L_d) {
  const long long n = (long long)T * L_d;
  return (n + 31) / 32 * 32;
}

template <typename E, int D>
hipError_t launch_fwd(const moda::FwdParams& p, unsigned grid, int nw, hipStream_t s) {
  if constexpr (sizeof(E) == 2 && D == 128) {
    if (nw == 8)
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
  // the bf16 d=128 kernel addresses one kv head's lse rows with 32-bit
  // offsets; with G not dividing 64 also one batch's q / dO rows (with G
  // dividing 64 those offsets stay within one 64-row block)
  const bool lse32 = (long long)p.T * p.G * 4 < 0x7fffffffLL;
  const bool q32 = (long long)p.T * p.Hq * D * 2 < 0x7fffffffLL;
  if constexpr (sizeof(E) == 2 && D == 128) {
    if (lse32 && 64 % p.G == 0)
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_bf16_kernel<D, true>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
    else if (lse32 && q32)
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_bf16_kernel<D, false>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
    else
      hipLaunchKernelGGL((moda::moda_bwd_dkdv_kernel<E, D, kWaves>), dim3(BH * p.nktiles), dim3(kWaves * 64), 0, s, p);
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
    default: return "unknown moda_status";
  }
}

long long moda_depth_packed_elems(int B, int T, int Hkv, int d, int L_d) {
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || L_d < 0) return -1;
  return (long long)B * Hkv * padded_depth_keys(T, L_d) * d;
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
  const long long grid = ((long long)B * Hkv * p.NKp * (d / ve) + 255) / 256;
  if (grid > 0x7fffffffLL) return MODA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_pack<moda::bf16, 128>(p, (unsigned)grid, s) : launch_pack<moda::bf16, 64>(p, (unsigned)grid, s);
  else
    e = d == 128 ? launch_pack<float, 128>(p, (unsigned)grid, s) : launch_pack<float, 64>(p, (unsigned)grid, s);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

static int fwd_impl(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, const float* k_scale, const float* v_scale, int q8, void* out,
                    float* lse, int B, int T, int Hq, int Hkv, int d, int L_cap, int slot_lo, int slot_hi,
                    int dtype, void* stream) {
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
  const int nw = fwd_waves(dtype, d, rows, (long long)B * Hkv);
  const int tile_rows = 32 * nw;
  const long long ntiles = (rows + tile_rows - 1) / tile_rows;
  const long long grid = ntiles * B * Hkv;
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
  p.paired = grid <= 2 * kCUs && B * Hkv <= kCUs && kCUs % (B * Hkv) == 0;
  p.NKp = padded_depth_keys(T, L_cap);
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_fwd<moda::bf16, 128>(p, (unsigned)grid, nw, s) : launch_fwd<moda::bf16, 64>(p, (unsigned)grid, nw, s);
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
  const long long rows = (long long)B * T * Hkv;
  const long long rpb = 256 / (d / 8);
  const long long grid = (rows + rpb - 1) / rpb;
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
  const long long rows = (long long)B * Hkv * p.NKp;
  const long long rpb = 256 / (d / 8);
  const long long grid = (rows + rpb - 1) / rpb;
  if (grid > 0x7fffffffLL) return MODA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == MODA_BF16) {
    if (d == 128) hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<moda::bf16, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<moda::bf16, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
  } else {
    if (d == 128) hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<float, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((moda::moda_pack_depth_q8_kernel<float, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_fwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
             const void* v_depth, void* out, float* lse, int B, int T, int Hq, int Hkv, int d,
             int L_d, int dtype, void* stream) {
  if (L_d < 0) return MODA_ERR_SHAPE;
  return moda_fwd_window(q, k_seq, v_seq, k_depth, v_depth, out, lse, B, T, Hq, Hkv, d, L_d, 0, L_d,
                         dtype, stream);
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
  const long long threads = (long long)B * T * Hkv * (d / ve);
  const long long grid = (threads + 255) / 256;
  if (grid > 0x7fffffffLL) return MODA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == MODA_BF16)
    e = d == 128 ? launch_append<moda::bf16, 128>(p, (unsigned)grid, s) : launch_append<moda::bf16, 64>(p, (unsigned)grid, s);
  else
    e = d == 128 ? launch_append<float, 128>(p, (unsigned)grid, s) : launch_append<float, 64>(p, (unsigned)grid, s);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

static int bwd_impl(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                    const void* v_depth, const float* k_scale, const float* v_scale, int q8,
                    const void* out, const float* lse, const void* dout, void* dq,
                    void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, float* work, int B,
                    int T, int Hq, int Hkv, int d, int L_cap, int slot_lo, int slot_hi, int dtype,
                    void* stream) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 1 || L_cap < 0) return MODA_ERR_SHAPE;
  if (slot_lo < 0 || slot_hi < slot_lo || slot_hi > L_cap) return MODA_ERR_SHAPE;
  if ((long long)T * L_cap > 0x7fffffffLL - 32) return MODA_ERR_SHAPE;   // packed key index is 31-bit
  if (Hq % Hkv != 0) return MODA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return MODA_ERR_DTYPE;
  if (!supported_d(d)) return MODA_ERR_UNSUPPORTED;
  if (!q || !k_seq || !v_seq || !out || !lse || !dout || !dq || !dk_seq || !dv_seq || !work)
    return MODA_ERR_NULL;
  const int L_d = slot_hi - slot_lo;
  if (L_d > 0 && (!k_depth || !v_depth || !dk_depth || !dv_depth)) return MODA_ERR_NULL;
  if (L_d > 0 && q8 && (!k_scale || !v_scale)) return MODA_ERR_NULL;
  const int G = Hq / Hkv;
  const long long rows = (long long)T * G;
  const long long ntiles = (rows + 32 * kWaves - 1) / (32 * kWaves);
  const long long nktiles = ((long long)T + 32 * kWaves - 1) / (32 * kWaves);
  const long long BH = (long long)B * Hkv;
  if (ntiles * BH > 0x7fffffffLL || (long long)T * BH > 0x7fffffffLL || rows > 0x7fffffffLL ||
      (long long)B * T * Hq > 0x7fffffffLL * 4)
    return MODA_ERR_SHAPE;

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
  {
    int sh = 0;
    while ((1LL << sh) < G) ++sh;                                 // ceil(log2 G)
    const unsigned long long num = 1ULL << (31 + sh);
    p.g_magic = (uint32_t)((num + (unsigned long long)G - 1) / (unsigned long long)G);
    p.g_shift = 31 + sh;
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
