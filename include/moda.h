/*
 * moda.h -- C ABI of libmoda.so: the forward pass of Mixture-of-Depths
 * Attention (MoDA) on AMD Instinct MI355X (gfx950).
 *
 * The operation (mhpn.cn article "动态混合深度注意力机制MoDA技术解析", section
 * 1.2, MoDA attention formula; section 2.2, dual masks; gist.science (de)
 * "Mixture-of-Depths Attention", Technische Zusammenfassung section 2,
 * Read-Step and Unified Softmax):
 *
 *   for every batch b, position t, query head h (kv head kvh = h / G,
 *   G = Hq / Hkv):
 *     keys   = [ k_seq[b, 0..t, kvh, :] ; k_depth[b, t, 0..L_d-1, kvh, :] ]
 *     values = [ v_seq[b, 0..t, kvh, :] ; v_depth[b, t, 0..L_d-1, kvh, :] ]
 *     z      = keys . q[b, t, h, :] / sqrt(d)
 *     out[b, t, h, :] = softmax(z) . values          (one softmax over both)
 *     lse[b, h, t]    = log(sum(exp(z)))             (natural log)
 *
 * i.e. causal sequence attention (s <= t) of the current layer joined with the
 * L_d depth slots that earlier layers wrote for the SAME position t.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers (HIP device memory of the current
 *     device), owned by the caller.  The library allocates nothing.  Its only
 *     state between calls is in its own static device memory: the launch
 *     counters of long grids (see moda_fwd; each launch takes its own and
 *     returns it to zero) and moda_bwd_noalloc's work array.  Calls on
 *     different streams may run concurrently (moda_bwd_noalloc aside).
 *   - Tensors are dense, row-major, in the layouts stated per argument
 *     (no strides).  Element type is `dtype` (MODA_F32 or MODA_BF16) except
 *     lse, which is always float32.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  It must belong to the current device, which holds the
 *     tensors (the library's per-device state is the current device's).  Every call only enqueues work and returns; results are ready
 *     after the stream is synchronised.
 *   - Arguments are validated before any HIP call is made.  A failed
 *     validation returns a nonzero moda_status and enqueues nothing.  A
 *     failed kernel launch returns MODA_ERR_HIP.  Faults inside a kernel
 *     surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Supported: dtype MODA_F32 or MODA_BF16, head size d = 64 or 128,
 *     any B, T >= 1, Hkv >= 1 with Hq a multiple of Hkv (G = 1 .. Hq),
 *     L_d >= 0.  Inputs are expected to be finite.
 *   - Packed depth keys are indexed n = t * L + slot with 31-bit integers:
 *     every call that takes a depth count or capacity L (L_d or L_cap)
 *     returns MODA_ERR_SHAPE when T * L exceeds 2^31 - 33.
 */
#ifndef MODA_H
#define MODA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MODA_F32 = 0,
  MODA_BF16 = 1
} moda_dtype;

typedef enum {
  MODA_OK = 0,
  MODA_ERR_NULL = 1,        /* a required pointer is NULL                   */
  MODA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent      */
  MODA_ERR_DTYPE = 3,       /* unknown dtype                                */
  MODA_ERR_UNSUPPORTED = 4, /* valid but not built (head size not 64/128)   */
  MODA_ERR_HIP = 5,         /* the HIP runtime reported an error on launch  */
  MODA_ERR_WORKSPACE = 6    /* workspace NULL, misaligned or too small, or
                               sizes beyond moda_bwd_noalloc's scratch      */
} moda_status;

/*
 * Number of ELEMENTS of each packed depth tensor (the packed keys and the
 * packed values have the same size): B * Hkv * NKp * d where NKp is T * L_d
 * rounded up to a multiple of 32.  Returns -1 for invalid sizes, 0 when
 * L_d == 0.
 */
long long moda_depth_packed_elems(int B, int T, int Hkv, int d, int L_d);

/*
 * moda_pack_depth -- repack the depth KV into the kernel's layout.
 *
 * The depth slots of one token position are the K/V that the L_d earlier
 * layers wrote for that position (gist.science (de), section 2, Read-Step and
 * Write-Step).  The pages flatten depth KV along one T x L axis so that it can
 * be read block-wise, and store the slots of one position contiguously
 * (gist.science (de), section 2, Flash-Compatible Layout; mhpn.cn article,
 * section 2.1, chunked contiguous storage).  This call produces that layout
 * for each (b, kv head):
 *
 *   k_depth, v_depth : in,  logical [B, T, L_d, Hkv, d], dtype
 *   k_packed         : out, [B, Hkv, NKp, d]   key n = t * L_d + j
 *   v_packed         : out, [B, Hkv, NKp, d]   value n = t * L_d + j
 *   Keys n >= T * L_d (padding up to NKp) are written as zeros.  T * L_d
 *   must stay below 2^31 - 32.
 *   Each packed buffer holds moda_depth_packed_elems(...) elements.
 *
 * With L_d == 0 nothing is enqueued and all four pointers may be NULL.
 * The packed buffers must not overlap the inputs.
 */
int moda_pack_depth(const void* k_depth, const void* v_depth,
                    void* k_packed, void* v_packed,
                    int B, int T, int Hkv, int d, int L_d, int dtype,
                    void* stream);

/*
 * moda_fwd -- fused MoDA forward.
 *
 *   q        : in,  [B, T, Hq, d]  dtype
 *   k_seq    : in,  [B, T, Hkv, d] dtype   (current layer's sequence keys)
 *   v_seq    : in,  [B, T, Hkv, d] dtype
 *   k_depth  : in,  packed keys   from moda_pack_depth (NULL iff L_d == 0)
 *   v_depth  : in,  packed values from moda_pack_depth (NULL iff L_d == 0)
 *   out      : out, [B, T, Hq, d]  dtype   (rounded to nearest even for bf16)
 *   lse      : out, [B, Hq, T] float32, natural-log sum of exp of the scaled
 *              scores; may be NULL to skip it
 *   B, T, Hq, Hkv, d, L_d, dtype : sizes as above
 *
 * Scores are computed with float32 accumulation; softmax statistics and the
 * output accumulator are float32.  With L_d == 0 the call is causal GQA
 * attention, run by the same kernel.  out must not overlap any input.
 *
 * Grids of several rounds (bf16, d = 128, at least 131072 query rows
 * B * T * Hq) hand out their query tiles through a launch counter, so that
 * faster parts of the GPU take more tiles: the library keeps a ring of 1024
 * such counters per GPU in its own device memory (8 KiB, nothing allocated
 * per call), one per launch, each back at zero when its launch ends.  Up to
 * 1024 launches that use them (this call, moda_fwd_window and the 8-bit
 * variants; the backward calls' long grids with B * Hkv <= 15) may run at the
 * same time on one GPU, on any streams; results do not depend on the order
 * in which tiles are taken.  A launch recorded into a HIP graph keeps the
 * counter it was given: replays of one graph must not overlap each other.
 */
int moda_fwd(const void* q, const void* k_seq, const void* v_seq,
             const void* k_depth, const void* v_depth,
             void* out, float* lse,
             int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
             void* stream);

/*
 * moda_fwd_workspace_bytes -- size in bytes of the workspace that moda_fwd_ws
 * uses for these sizes, or -1 for invalid sizes.  0 when no query tile is
 * split across workgroups: grids of more than two workgroups per compute
 * unit (about T * Hq / Hkv * B * Hkv > 65536 rows), grids small enough for
 * one round of eight-wave workgroups over 128-row tiles (at most 256 such
 * tiles: there moda_fwd itself splits each tile's keys between the two
 * halves of its workgroup), shapes other than bf16 with d = 128.
 * The size depends on B, T, G = Hq / Hkv and Hkv only: a 4096-byte header
 * of arrival counters (the same for every shape), then 2 * 66 * 64 * 4 =
 * 33792 bytes per (split tile, wave) for the two parts' states.  Splitting
 * applies to grids of at most 512 workgroups (at most 1024 (split tile,
 * wave) pairs), so it is at most 4096 + 1024 * 33792 bytes (33 MiB) for any
 * shape.
 */
long long moda_fwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d, int dtype);

/*
 * moda_fwd_ws -- moda_fwd with a workspace, for short sequences.
 *
 * The causal mask gives the query tile at the end of the sequence about
 * twice the keys of the average tile, and on a grid too small to fill the GPU
 * more than twice over that tile alone sets the run time; the pages single out
 * short sequences as the costly case for the depth slots (mhpn.cn article
 * "动态混合深度注意力机制MoDA技术解析", section 3.1, Table 2 discussion: extra
 * time 25.86% at 4K against 2.73% at 64K).  Here the key range of each of the
 * longer half of the tiles is split over two workgroups whose partial
 * softmax states (running max m, sum l, unnormalised output O) are merged
 * exactly as one online softmax over the union of the two key sets -- the
 * identity behind the Unified Softmax of gist.science (de) "Mixture-of-Depths
 * Attention", Technische Zusammenfassung section 2.
 *
 *   q ... dtype, stream : as for moda_fwd
 *   work       : device scratch owned by the caller, at least
 *                moda_fwd_workspace_bytes(B, T, Hq, Hkv, d, dtype) bytes,
 *                256-byte aligned.  Zero-fill it once before its first use;
 *                every call leaves it ready for the next one (its arrival
 *                counters return to zero).  Calls that share a workspace
 *                must not run at the same time (same stream, or ordered by
 *                events).
 *   work_bytes : size of work in bytes
 * Errors: MODA_ERR_WORKSPACE when work is NULL, not 256-byte aligned or too
 * small (when the size needed is 0 any work pointer is accepted and unused);
 * otherwise as for moda_fwd.  Results equal moda_fwd's within floating-point
 * rounding (the merge reorders the sums of split tiles).
 */
int moda_fwd_ws(const void* q, const void* k_seq, const void* v_seq,
                const void* k_depth, const void* v_depth,
                void* out, float* lse,
                int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
                void* work, long long work_bytes, void* stream);

/*
 * moda_fwd_window -- fused forward over a window of depth slots.
 *
 * The depth stream can hold more slots than one layer reads: a buffer packed
 * with L_cap slots per position (by moda_pack_depth with L_d = L_cap, or by
 * moda_append_depth), of which this call reads slots slot_lo .. slot_hi-1 of
 * each position.  This is the bounded depth-KV slot cache (sliding window or
 * selected range) that gist.science (de) "Mixture-of-Depths Attention",
 * Technische Zusammenfassung section 5, proposes for very deep models, and the
 * read side of the write step below (layer l reads slots 0 .. l-1).
 *
 *   k_depth, v_depth : packed buffers with L_cap slots per position, i.e.
 *                      moda_depth_packed_elems(B, T, Hkv, d, L_cap) elements
 *                      each; slots outside the window and the padding rows
 *                      are never read into a product, so they may hold
 *                      anything (a buffer being filled by the write step
 *                      needs no zero fill); NULL allowed iff
 *                      slot_lo == slot_hi
 *   L_cap            : slots per position in the packed buffers (>= 0)
 *   slot_lo, slot_hi : 0 <= slot_lo <= slot_hi <= L_cap
 *   all other arguments as for moda_fwd.
 *
 * moda_fwd(..., L_d, ...) is moda_fwd_window(..., L_cap = L_d, 0, L_d, ...).
 */
int moda_fwd_window(const void* q, const void* k_seq, const void* v_seq,
                    const void* k_depth, const void* v_depth,
                    void* out, float* lse,
                    int B, int T, int Hq, int Hkv, int d,
                    int L_cap, int slot_lo, int slot_hi, int dtype,
                    void* stream);

/*
 * moda_append_depth -- the write step: store one layer's K/V of every
 * position into slot `slot` of packed depth buffers with L_cap slots per
 * position (gist.science (de) "Mixture-of-Depths Attention", Technische
 * Zusammenfassung section 2, Write-Step: a layer appends its KV pairs to the
 * depth stream that later layers read).
 *
 *   k_new, v_new     : in,  [B, T, Hkv, d] dtype (this layer's keys / values)
 *   k_packed, v_packed : in/out, packed buffers of
 *                      moda_depth_packed_elems(B, T, Hkv, d, L_cap) elements;
 *                      only the entries of slot `slot` are written
 *   0 <= slot < L_cap.
 *
 * Appending slots 0 .. L-1 in turn into zero-filled buffers gives exactly the
 * bytes that moda_pack_depth produces for the same L = L_cap slots.
 */
int moda_append_depth(const void* k_new, const void* v_new,
                      void* k_packed, void* v_packed,
                      int B, int T, int Hkv, int d, int L_cap, int slot, int dtype,
                      void* stream);

/*
 * moda_pack_depth_q8 -- moda_pack_depth with 8-bit depth KV.
 *
 * The mhpn.cn article (section 4.2, memory optimisation) suggests 8-bit
 * quantisation for the depth KV of deep models; the format is not given.
 * Here: symmetric int8 per packed row (one key or value vector of d
 * elements) with one float32 scale, decided in float32:
 *   scale = max|x| / 127,  code = rint(x / scale) clamped to [-127, 127]
 *   (ties to even; an all-zero row has scale 0 and codes 0),
 *   dequantised value = scale * code.
 *
 *   k_depth, v_depth : in,  logical [B, T, L_d, Hkv, d], dtype
 *   k_q, v_q         : out, int8 [B, Hkv, NKp, d], the packed order of
 *                      moda_pack_depth (moda_depth_packed_elems(...) bytes each)
 *   k_scale, v_scale : out, float32 [B, Hkv, NKp] (elems / d floats each)
 *   Padding rows (n >= T * L_d) get scale 0 and codes 0.
 * With L_d == 0 nothing is enqueued and the pointers may be NULL.
 */
int moda_pack_depth_q8(const void* k_depth, const void* v_depth,
                       int8_t* k_q, int8_t* v_q, float* k_scale, float* v_scale,
                       int B, int T, int Hkv, int d, int L_d, int dtype,
                       void* stream);

/*
 * moda_fwd_q8 -- moda_fwd reading 8-bit depth KV from moda_pack_depth_q8.
 * The depth keys and values are dequantised (scale * code, rounded to dtype)
 * in registers before the matrix products; the result is the MoDA forward of
 * the dequantised depth KV.  Arguments as for moda_fwd, with the packed
 * buffers replaced by the int8 codes and float32 row scales (NULL iff
 * L_d == 0).
 */
int moda_fwd_q8(const void* q, const void* k_seq, const void* v_seq,
                const int8_t* k_q, const int8_t* v_q,
                const float* k_scale, const float* v_scale,
                void* out, float* lse,
                int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
                void* stream);

/*
 * moda_bwd -- gradients of the MoDA forward (moda_fwd with the same L_d).
 *
 * The pages present the kernel for training pipelines (gist.science (de)
 * "Mixture-of-Depths Attention", section 5, Praktische Anwendbarkeit); the
 * gradients are the derivatives of the forward's definition (mhpn.cn
 * article, section 1.2 formula, section 2.2 masks).  With P = exp(z - lse),
 * Delta = rowsum(dout * out), dP = dout . v, dS = P (dP - Delta):
 *   dq = dS . keys / sqrt(d);  dk = dS^T . q / sqrt(d);  dv = P^T . dout,
 * summed over every query row (all G heads of the kv head) that sees the key.
 *
 *   q, k_seq, v_seq  : in, as for moda_fwd
 *   k_depth, v_depth : in, packed buffers from moda_pack_depth (NULL iff L_d == 0)
 *   out, lse         : in, results of moda_fwd on these inputs (lse required)
 *   dout             : in,  [B, T, Hq, d]  dtype, gradient of out
 *   dq               : out, [B, T, Hq, d]  dtype
 *   dk_seq, dv_seq   : out, [B, T, Hkv, d] dtype
 *   dk_depth, dv_depth : out, [B, T, L_d, Hkv, d] dtype -- the LOGICAL depth
 *                      layout, slot j being the j-th earlier layer's K/V
 *                      (NULL iff L_d == 0)
 *   work             : scratch, 2 * B * Hq * T float32, owned by the caller
 *                      (after the call: -Delta, then -lse * sqrt(d), each
 *                      [B, Hq, T])
 * Every output element is written (no accumulation into existing contents).
 * Products use float32 accumulation; P and dS enter them in dtype.  All
 * outputs must be distinct and must not overlap any input.  With bf16,
 * d = 128, B * Hkv <= 15 and grids of several rounds, the dQ and dK/dV
 * kernels take their tiles from the launch counters described at moda_fwd
 * (no allocation; results independent of the order).
 */
int moda_bwd(const void* q, const void* k_seq, const void* v_seq,
             const void* k_depth, const void* v_depth,
             const void* out, const float* lse, const void* dout,
             void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth,
             float* work,
             int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
             void* stream);

/*
 * moda_bwd_workspace_bytes -- size in bytes of the workspace that moda_bwd_ws
 * uses for these sizes, or -1 for invalid sizes.  Always at least the work
 * buffer, 2 * B * Hq * T float32 rounded up to 256 bytes; on short sequences
 * with bf16 and d = 128 (about B * Hkv * T / 128 < 410 key tiles) another
 * 131072 bytes per chunk of the row-split dK / dV (described at moda_bwd_ws),
 * of which there are at most 256 + B * Hkv * ceil(T / 128).
 */
long long moda_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int d, int dtype);

/*
 * moda_bwd_ws -- moda_bwd with a workspace, for short sequences.
 *
 * moda_bwd gives each tile of 128 keys (per batch and kv head) one
 * workgroup, which sweeps every query row that sees its keys; under the
 * causal mask (mhpn.cn article, section 2.2) the first tile meets all T * G
 * rows and the last only its own, and when the grid does not fill the GPU
 * the first tiles alone set the run time (the pages name short sequences as
 * the costly case: mhpn.cn article "动态混合深度注意力机制MoDA技术解析",
 * section 3.1, Table 2 discussion).  Here each tile's rows are cut into
 * chunks swept by separate workgroups, all chunks about the average work of
 * a compute unit; dk and dv being sums over rows (the formulas at moda_bwd),
 * each chunk's float32 partial sums go to the workspace and a second kernel
 * adds them up in a fixed order.  Other shapes, and dtype / d other than
 * bf16 / 128, run as moda_bwd.
 *
 *   q ... dv_depth, B ... dtype, stream : as for moda_bwd
 *   work       : device scratch owned by the caller, at least
 *                moda_bwd_workspace_bytes(B, T, Hq, Hkv, d, dtype) bytes,
 *                256-byte aligned, any contents (every byte read is first
 *                written by the same call).  Its first 2 * B * Hq * T floats
 *                end as moda_bwd's work buffer does.  Calls that share a
 *                workspace must not run at the same time.
 *   work_bytes : size of work in bytes
 * Errors: MODA_ERR_WORKSPACE when work is NULL, not 256-byte aligned or too
 * small; otherwise as for moda_bwd.  Results equal moda_bwd's within
 * floating-point rounding (the split reorders the sums of dk and dv); they
 * are the same from call to call.
 */
int moda_bwd_ws(const void* q, const void* k_seq, const void* v_seq,
                const void* k_depth, const void* v_depth,
                const void* out, const float* lse, const void* dout,
                void* dq, void* dk_seq, void* dv_seq,
                void* dk_depth, void* dv_depth,
                int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
                void* work, long long work_bytes, void* stream);

/*
 * moda_bwd_noalloc -- moda_bwd without the work argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * training loops, harnesses that forbid hipMalloc).  The work buffer is
 * instead a static device array inside the library, one per GPU, held until
 * the process ends: 32 MiB, enough for B * Hq * T <= 4194304 (4M); larger
 * sizes return MODA_ERR_WORKSPACE before anything is enqueued.  The call
 * allocates nothing (no hipMalloc / hipFree); its first call on a GPU looks up
 * that GPU's copy of the array.  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (concurrent streams, or
 * threads) race: order them, or use moda_bwd with a buffer each.  The array
 * keeps the last call's -Delta and -lse * sqrt(d) (nothing needs clearing:
 * each call writes all it reads).  Other arguments, results and errors as for
 * moda_bwd; the results are bit for bit those of moda_bwd.
 */
int moda_bwd_noalloc(const void* q, const void* k_seq, const void* v_seq,
                     const void* k_depth, const void* v_depth,
                     const void* out, const float* lse, const void* dout,
                     void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth,
                     int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
                     void* stream);

/*
 * moda_bwd_window -- moda_bwd for the forward moda_fwd_window(..., L_cap,
 * slot_lo, slot_hi, ...): the packed buffers hold L_cap slots per position and
 * the gradients of slots slot_lo .. slot_hi-1 are written to dk_depth /
 * dv_depth, logical [B, T, slot_hi - slot_lo, Hkv, d] (NULL iff the window is
 * empty).  Other arguments as for moda_bwd; moda_bwd(..., L_d, ...) is
 * moda_bwd_window(..., L_cap = L_d, 0, L_d, ...).
 */
int moda_bwd_window(const void* q, const void* k_seq, const void* v_seq,
                    const void* k_depth, const void* v_depth,
                    const void* out, const float* lse, const void* dout,
                    void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth,
                    float* work,
                    int B, int T, int Hq, int Hkv, int d,
                    int L_cap, int slot_lo, int slot_hi, int dtype,
                    void* stream);

/*
 * moda_fwd_window_q8 -- moda_fwd_window over 8-bit depth KV: the codes and
 * scales of a buffer with L_cap slots per position (moda_pack_depth_q8 with
 * L_d = L_cap, or moda_append_depth_q8), reading slots slot_lo .. slot_hi-1.
 */
int moda_fwd_window_q8(const void* q, const void* k_seq, const void* v_seq,
                       const int8_t* k_q, const int8_t* v_q,
                       const float* k_scale, const float* v_scale,
                       void* out, float* lse,
                       int B, int T, int Hq, int Hkv, int d,
                       int L_cap, int slot_lo, int slot_hi, int dtype,
                       void* stream);

/*
 * moda_append_depth_q8 -- the write step into 8-bit packed buffers: one
 * layer's K/V [B, T, Hkv, d] quantised (as moda_pack_depth_q8 does each row)
 * into slot `slot` of int8 buffers with L_cap slots per position and their
 * row scales.  0 <= slot < L_cap.  Appending slots 0 .. L-1 into zero-filled
 * buffers gives bit for bit what moda_pack_depth_q8 produces for L slots.
 */
int moda_append_depth_q8(const void* k_new, const void* v_new,
                         int8_t* k_q, int8_t* v_q, float* k_scale, float* v_scale,
                         int B, int T, int Hkv, int d, int L_cap, int slot, int dtype,
                         void* stream);

/*
 * moda_bwd_q8 -- moda_bwd for moda_fwd_q8: the depth keys and values are read
 * as int8 codes and float32 row scales (moda_pack_depth_q8) and dequantised
 * (scale * code, rounded to dtype) as in the forward; dk_depth / dv_depth are
 * the gradients with respect to those dequantised keys and values (the
 * quantisation itself is not differentiated), in the logical layout of
 * moda_bwd.  mhpn.cn article, section 4.2 (8-bit depth KV) for the storage;
 * the derivatives as for moda_bwd.  Other arguments and errors as for
 * moda_bwd; k_scale / v_scale NULL iff L_d == 0.
 */
int moda_bwd_q8(const void* q, const void* k_seq, const void* v_seq,
                const int8_t* k_q, const int8_t* v_q,
                const float* k_scale, const float* v_scale,
                const void* out, const float* lse, const void* dout,
                void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth,
                float* work,
                int B, int T, int Hq, int Hkv, int d, int L_d, int dtype,
                void* stream);

/*
 * moda_bwd_window_q8 -- moda_bwd_window over 8-bit depth KV (the buffers of
 * moda_fwd_window_q8 with L_cap slots per position): gradients of slots
 * slot_lo .. slot_hi-1, logical [B, T, slot_hi - slot_lo, Hkv, d].
 */
int moda_bwd_window_q8(const void* q, const void* k_seq, const void* v_seq,
                       const int8_t* k_q, const int8_t* v_q,
                       const float* k_scale, const float* v_scale,
                       const void* out, const float* lse, const void* dout,
                       void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth,
                       float* work,
                       int B, int T, int Hq, int Hkv, int d,
                       int L_cap, int slot_lo, int slot_hi, int dtype,
                       void* stream);

/* Static, human-readable name of a moda_status value. */
const char* moda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MODA_H */
