/*
 * fa.h - C ABI of the exact-attention library (libfa.so), gfx950: the
 * forward pass (plain, local window, strided views, split-KV) and the
 * backward pass, plus host-only queries.
 *
 * The operation is exact softmax attention computed tile by tile with the
 * online-softmax recurrence, so the N x N score matrix is never written to
 * memory:
 *
 *   S = scale * Q K^T            (per batch b and head h)
 *   S_ij = -inf where causal and j > i (lower-triangular mask), or outside
 *          the local window of fa_fwd_window
 *   O = softmax_rows(S) V,  LSE_i = ln sum_j exp(S_ij)
 *
 * Sources: the standard three-step form and its [batch, heads, seq, head_dim]
 * layout and -inf mask are section 1.1 of "2.3 FlashAttention and IO-aware
 * attention" (aiknowledge.cn); the blockwise recurrence (running max m,
 * running sum l, rescale of the output accumulator, final O / l) is
 * ``flash_attention_forward`` on the flash_attention.py teaching page
 * (forceinjection.github.io); the scale and causal arguments mirror
 * ``softmax_scale`` / ``causal`` of the packed call in section 5.2 of the
 * flash-attn 2.8.3 build guide (intelliparadigm.com). LSE is the row
 * statistic m + ln l that the recurrence carries; it is written so that a
 * backward pass or a merge of partial results can use it.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. lse is always float32. */
typedef enum {
    FA_F16 = 0,  /* IEEE binary16 */
    FA_BF16 = 1, /* bfloat16 */
    FA_F32 = 2   /* IEEE binary32; computed in fp32 end to end */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,    /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,   /* a size is negative or too large */
    FA_ERR_HEADDIM = -3, /* d is not 64, 128 or 256 */
    FA_ERR_DTYPE = -4,   /* dtype is not an fa_dtype */
    FA_ERR_ALIGN = -5,   /* a row of q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_ARG = -6,     /* causal not 0/1, scale not finite, or an output overlaps */
    FA_ERR_LAUNCH = -7,  /* the HIP runtime rejected the kernel launch */
    FA_ERR_SCRATCH = -8  /* fa_fwd_kv_noalloc: the partial results exceed its static scratch buffer */
} fa_status;

/*
 * fa_fwd - enqueue one attention forward pass on `stream`.
 *
 * q, k, v  device pointers, [B, H, N, d] contiguous (d fastest), element type
 *          `dtype`. Read only; they may alias one another.
 * o        device pointer, [B, H, N, d] contiguous, element type `dtype`;
 *          written with O rounded to nearest even.
 * lse      device pointer, [B, H, N] contiguous float32; written with the
 *          natural-log LSE of each query row.
 * B, H, N  batch, heads, sequence length (queries and keys have the same N).
 * d        head dimension: 64, 128 or 256.
 * scale    multiplies Q K^T before the softmax; finite (0 gives uniform
 *          weights). Callers wanting the usual default pass 1/sqrt(d).
 * causal   0: every key is visible; 1: query i sees keys j <= i.
 * stream   a hipStream_t, or NULL for the default stream.
 *
 * Ownership: the caller allocates and owns every buffer. The library
 * allocates nothing for this call, which keeps no state between calls and is
 * reentrant.
 * o and lse must not overlap q, k or v.
 *
 * Synchronisation: asynchronous. The kernel is enqueued and the call returns;
 * a fault inside it surfaces at the caller's next synchronisation.
 *
 * Errors: all argument checks run on the host before any HIP call, and a
 * failed check returns its negative fa_status without touching the GPU. If
 * B*H*N == 0 the call returns FA_OK without launching (pointers are then not
 * checked). FA_ERR_LAUNCH is returned if the runtime reports an error right
 * after the launch.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_fwd_window - fa_fwd with a local-attention window: query i sees key j
 * only if i - window_left <= j <= i + window_right. A side of -1 is
 * unbounded, so (-1, -1) is exactly fa_fwd; with causal = 1 the window and
 * the causal mask intersect (window_right then has no effect).
 *
 * Source: the packed call in section 10.1 of the flash-attn 2.8.3 build
 * guide (intelliparadigm.com) lists window_size=(-1, -1) as the local
 * attention window without defining it; the bounds above are this library's
 * reading of it (the same one its oracle implements). Every query row keeps
 * its own key, so no row is empty.
 *
 * Arguments, layout, ownership, synchronisation and errors as fa_fwd;
 * additionally FA_ERR_ARG if window_left or window_right is below -1.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal,
                  int window_left, int window_right, int dtype, void* stream);

/*
 * fa_fwd_strided - fa_fwd_window on strided views, so that the head slices
 * of a packed tensor are read and written in place. The packed layouts are
 * those of the user calls of sections 5.2 and 10.1 of the flash-attn 2.8.3
 * build guide (intelliparadigm.com): qkv as [B, N, 3, H, d], and q, k, v or
 * o as [B, N, H, d].
 *
 * strides  host pointer to 12 element strides, or NULL for contiguous
 *          [B, H, N, d] operands: (batch, head, row) for q, then k, v and o,
 *          i.e. element (b, h, i, c) of q is q[b*s[0] + h*s[1] + i*s[2] + c].
 *          The head dimension itself is always contiguous. Read during the
 *          call only. Examples (element strides): contiguous [B, H, N, d]:
 *          (H*N*d, N*d, d); a [B, N, H, d] tensor: (N*H*d, d, H*d); slice t
 *          of a packed [B, N, 3, H, d] tensor, whose base is qkv + t*H*d:
 *          (3*N*H*d, d, 3*H*d).
 *
 * Requirements, checked on the host before any HIP call:
 *  - strides >= 0 and row strides >= d (FA_ERR_SHAPE); a row stride of at
 *    most 32 MiB in bytes (FA_ERR_SHAPE); the stride of a dimension of
 *    extent 1 is ignored;
 *  - every row start 16-byte aligned: base pointer and strides times the
 *    element size multiples of 16 (FA_ERR_ALIGN);
 *  - inputs may overlap one another (a head stride of 0 shares one K or V
 *    among all heads); o must not overlap itself (each stride, taken in
 *    increasing order over dimensions of extent > 1, at least the extent
 *    of the smaller ones) nor share a byte with q, k or v, and lse (still a
 *    contiguous [B, H, N] float32 array) must not overlap any of them
 *    (FA_ERR_ARG). Two operands whose extents overlap are accepted as
 *    disjoint when they have the same row stride P, batch strides that are
 *    multiples of P, and disjoint byte sets modulo P (the slices of one
 *    packed tensor); other overlapping extents are rejected.
 *
 * Everything else as fa_fwd_window, which is this call with strides = NULL.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   const long long* strides, int B, int H, int N, int d, float scale,
                   int causal, int window_left, int window_right, int dtype, void* stream);

/*
 * fa_fwd_splitkv - fa_fwd_strided with the key range of every query tile
 * split into num_splits parts that run as separate workgroups, for shapes
 * whose B * H * N gives too few workgroups to fill the GPU (small batches,
 * few heads, short sequences). Each part writes its partial result over its
 * keys, and a merge kernel combines them:
 *   LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
 * where O_s and LSE_s are the attention output and LSE over the part's keys
 * alone. This follows from the definition: the softmax over a union of
 * disjoint key sets is the LSE-weighted mix of the softmaxes over each set.
 * The use is the long-context inference of section 11.2 of the flash-attn
 * 2.8.3 build guide (intelliparadigm.com); the pages give no procedure.
 *
 * num_splits  0: the library chooses (fa_fwd_num_splits); 1: no split (the
 *             fa_fwd_strided kernel, workspace unused and may be NULL);
 *             2 .. 64: that many parts. Part s of a query tile whose key
 *             tiles (64 keys each) are t_0 .. t_0 + n - 1 covers tiles
 *             t_0 + floor(n s / S) .. t_0 + floor(n (s + 1) / S) - 1.
 * workspace   device pointer, 16-byte aligned, of at least
 *             fa_fwd_splitkv_workspace(...) bytes, owned by the caller, not
 *             overlapping any operand; written, its previous contents
 *             ignored. Layout: the parts' O_s as float32 [S, B*H, N, d],
 *             then their LSE_s as float32 [S, B*H, N] (a part with no
 *             visible key of a row holds O_s = 0, LSE_s = -inf there).
 * workspace_bytes  its size.
 *
 * The result equals fa_fwd_strided's up to rounding (the parts are kept in
 * float32 and O is rounded once, in the merge). Two kernels are enqueued on
 * stream in order. Other arguments and errors as fa_fwd_strided; in
 * addition FA_ERR_ARG for num_splits outside 0 .. 64, a workspace that is
 * too small or overlaps an operand, FA_ERR_NULL / FA_ERR_ALIGN for a
 * missing or misaligned workspace when more than one part runs.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   const long long* strides, void* workspace, long long workspace_bytes,
                   int num_splits, int B, int H, int N, int d, float scale, int causal,
                   int window_left, int window_right, int dtype, void* stream);

/*
 * fa_fwd_kv - the general forward: fa_fwd_splitkv with N query rows against
 * Nk key/value rows, for new tokens attending to a key/value cache (the
 * inference use of section 11.2 of the flash-attn 2.8.3 build guide,
 * intelliparadigm.com, which gives no definition for unequal lengths).
 *
 * q, o, lse have N rows per (b, h); k and v have Nk rows (their strides, in
 * the strides array as for fa_fwd_strided, describe [B, H, Nk, d] views).
 * The N queries are the last N positions of the Nk-long sequence: query
 * row i sits at position p = i + Nk - N, and the causal mask (key j <= p)
 * and the window (p - window_left <= j <= p + window_right) apply to p. With
 * N = Nk this is fa_fwd_splitkv. A decode step is N = 1 (or a few rows)
 * against a long Nk, typically with num_splits = 0 so that the key range is
 * spread over the GPU.
 *
 * Errors as fa_fwd_splitkv, and: FA_ERR_SHAPE for Nk < 0 or too large;
 * FA_ERR_ARG when some query row would see no key: Nk = 0 (with N > 0), or
 * N > Nk together with a causal mask or a window (rows before the first key
 * position). Workspace bytes depend on N only (fa_fwd_splitkv_workspace).
 */
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              const long long* strides, void* workspace, long long workspace_bytes,
              int num_splits, int B, int H, int N, int Nk, int d, float scale, int causal,
              int window_left, int window_right, int dtype, void* stream);

/*
 * fa_fwd_kv_noalloc - fa_fwd_kv without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): with more than one part
 * the partial results go to a static device array of the library,
 * FA_NOALLOC_SCRATCH_BYTES long, instead of a caller workspace. The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller still passes q, k, v, o and lse.
 *
 * The array exists once per GPU the library runs on (each GPU holds its
 * own copy, looked up on the first call on that device, with that device
 * current) and is held until the process ends. Every call on one GPU shares
 * it: calls that overlap in time on one GPU (on different streams, or from
 * different threads) race on it and must be ordered by the caller. Its
 * previous contents never matter: every element a call reads is written by
 * that call first. `stream` must belong to the current device.
 *
 * Arguments, result and errors as fa_fwd_kv, and: FA_ERR_SCRATCH (before
 * any HIP call) when the parts' partial results, 4 * S * B * H * N * (d + 1)
 * bytes for S parts (fa_fwd_splitkv_workspace), exceed
 * FA_NOALLOC_SCRATCH_BYTES; FA_ERR_LAUNCH if the device or the array's
 * address cannot be obtained.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64ll << 20)
int fa_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      const long long* strides, int num_splits, int B, int H, int N, int Nk, int d,
                      float scale, int causal, int window_left, int window_right, int dtype,
                      void* stream);

/*
 * fa_fwd_num_splits - host-only: the number of parts fa_fwd_splitkv uses
 * for num_splits = 0: 1 when the plain grid already fills half the GPU;
 * otherwise, while each part of the widest query tile keeps at least 16 key
 * tiles (causal) or 32 (not causal): enough parts to fill the GPU's
 * resident workgroup slots (at most 16), or, with fewer query rows than
 * half a query tile (a decode step, bound by streaming K and V), about one
 * workgroup per compute unit (at most 64). Writes it to *num_splits;
 * returns the shape checks' status.
 *
 * fa_fwd_splitkv_workspace - host-only: the workspace bytes fa_fwd_splitkv
 * needs for num_splits parts (0 for num_splits = 1): 4 * S * B * H * N *
 * (d + 1). FA_ERR_ARG for num_splits outside 1 .. 64.
 */
int fa_fwd_num_splits(int B, int H, int N, int d, int causal, int window_left,
                      int window_right, int dtype, int* num_splits);
/* fa_fwd_kv_num_splits - the same for N query rows against Nk keys (fa_fwd_kv). */
int fa_fwd_kv_num_splits(int B, int H, int N, int Nk, int d, int causal, int window_left,
                         int window_right, int dtype, int* num_splits);
int fa_fwd_splitkv_workspace(int B, int H, int N, int d, int num_splits, long long* bytes);

/*
 * fa_bwd - enqueue the backward pass: the gradients dq, dk, dv of a loss
 * whose gradient with respect to o is dout, for the forward pass fa_fwd_window
 * computed with the same q, k, v, scale, causal and window.
 *
 * Operation (per batch b and head h; masked keys excluded as in the
 * forward): P = exp(S - LSE) with S = scale q k^T, recomputed from q, k and
 * the forward's lse rather than stored (the recomputation of section 9.2 of
 * the flash-attn 2.8.3 build guide, intelliparadigm.com); then
 *   dv = P^T dout,  dP = dout v^T,  delta_i = sum_c dout_ic o_ic,
 *   dS = P * (dP - delta),  dq = scale dS k,  dk = scale dS^T q,
 * the chain rule of the forward definition.
 *
 * q, k, v, o  device pointers, [B, H, N, d] contiguous, element type dtype:
 *             the forward's inputs and output. Read only.
 * lse         device pointer, [B, H, N] float32: the forward's lse. Read only.
 * dout        device pointer, [B, H, N, d] contiguous, dtype: dLoss/do.
 * dq, dk, dv  device pointers, [B, H, N, d] contiguous, dtype; written
 *             (accumulated in float32, rounded to nearest even once).
 * delta       device pointer, [B, H, N] float32; written with delta_i (it is
 *             both a result and the scratch the kernels share).
 * B, H, N, scale, causal, window_left, window_right, stream: as fa_fwd_window.
 * d           64, 128 or 256.
 * dtype       FA_F16 or FA_BF16 (fp32 is not supported by the backward).
 *
 * Ownership, synchronisation and errors as fa_fwd: the caller owns every
 * buffer, nothing is allocated, and two kernels are enqueued on stream in
 * order (dq, which also writes delta, then dk/dv, which reads it); the
 * result does not depend on
 * scheduling (no atomics). The outputs dq, dk, dv, delta must not overlap
 * each other or any input (FA_ERR_ARG). FA_ERR_HEADDIM for d other than 64,
 * 128 or 256, FA_ERR_DTYPE for fp32 or an unknown dtype; all pointers 16-byte
 * aligned except lse and delta (4-byte).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, float scale, int causal,
           int window_left, int window_right, int dtype, void* stream);

/*
 * fa_bwd_strided - fa_bwd on strided views (the layouts of fa_fwd_strided),
 * so that the gradient of a packed [B, N, 3, H, d] qkv is written in place.
 *
 * strides  host pointer to 24 element strides, or NULL for contiguous
 *          operands: (batch, head, row) for q, k, v, o, dout, dq, dk, dv in
 *          this order. lse and delta stay contiguous [B, H, N] float32.
 *
 * The stride, alignment and extent rules of fa_fwd_strided apply to all
 * eight operands. dq, dk and dv must each be free of self-overlap and share
 * no byte with any other operand; delta must overlap nothing. The slices
 * of one packed gradient tensor pass this test.
 *
 * Everything else as fa_bwd, which is this call with strides = NULL.
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* delta,
                   const long long* strides, int B, int H, int N, int d, float scale,
                   int causal, int window_left, int window_right, int dtype, void* stream);

/*
 * fa_fwd_strided_check, fa_bwd_strided_check - host-only validation: return
 * the status that fa_fwd_strided / fa_bwd_strided (same arguments, without
 * the stream) would return from their argument checks, without any HIP call
 * or launch. The pointers are only compared, never dereferenced. A caller
 * can use them to find out up front whether a layout is accepted.
 */
int fa_fwd_strided_check(const void* q, const void* k, const void* v, void* o, float* lse,
                         const long long* strides, int B, int H, int N, int d, float scale,
                         int causal, int window_left, int window_right, int dtype);
int fa_bwd_strided_check(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* delta, const long long* strides, int B, int H, int N, int d,
                         float scale, int causal, int window_left, int window_right, int dtype);

/* Static text for a status code (never NULL). */
const char* fa_strerror(int status);

/*
 * fa_fwd_grid - host-only query of the launch shape fa_fwd would use:
 * writes the number of workgroups and the query rows of one query tile,
 * the unit the work is divided into (128 rows for 16-bit inputs, 64 for
 * fp32; split-KV partitions each tile's key range). A workgroup runs one
 * tile, except in the balanced causal grid (16-bit, causal, d = 64, at
 * least two tiles), where workgroup p runs tiles nqt - 1 - p and p of its
 * head so that all workgroups do the same work. Returns the same status
 * fa_fwd's argument checks would (pointers excepted). Used to relate
 * kernel timings to work units; makes no HIP call.
 */
int fa_fwd_grid(int B, int H, int N, int d, int causal, int dtype,
                long long* workgroups, int* rows_per_workgroup);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
