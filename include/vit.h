/*
 * vit.h -- C ABI of libvit.so: packed varlen (block-diagonal) multi-head
 * attention for vision encoder towers on AMD Instinct MI355X (gfx950).
 *
 * The operation.  Tokens of many images are packed into one [T, H, D] tensor;
 * int32 cu_seqlens[N+1] marks the boundaries (segment i owns tokens
 * [cu_seqlens[i], cu_seqlens[i+1])) and every segment attends only to itself,
 * non-causally, with no KV cache.  This is what the eager dense-mask and
 * per-segment forms (vLLM page vllm.models.dots3_note.nvidia.vision_attention,
 * VisionAttention.forward and VisionAttentionV2.forward) and the varlen backends
 * (tokenspeed page mm_encoder_attention.py, vision_attn_triton / vision_attn_fa3 /
 * vision_attn_fa4, which pass the same cu_seqlens for queries and keys) compute.
 * A pre-pass applies the Q/K RMSNorm and the 2D rotary embedding in place.
 *
 * Conventions shared by every entry point:
 *  - Status: every int-returning call returns VIT_OK (0) or a VIT_ERR_* code;
 *    on error vit_last_error() returns a message (thread-local, valid until the
 *    next call on the same thread).  Argument errors are detected on the host
 *    before anything is enqueued.
 *  - Memory: every pointer argument is device memory owned by the caller unless
 *    stated otherwise; the library never frees or retains caller pointers.
 *    Tensor pointers must be 16-byte aligned.
 *  - Layout: q, k, v, out are [T, H, D] row-major, element (t, h, d) at
 *    (t*H + h)*D + d, unless a call takes token strides (see "Token strides"
 *    below): then element (t, h, d) is at t*stride + h*D + d.
 *  - Streams: work is enqueued asynchronously on `stream` (0 = the default
 *    stream of the current device); the library never makes the host wait,
 *    except in vit_device_error() and vit_release().
 *  - Device-side validation of cu_seqlens (see vit_varlen_worklist) never
 *    reads or writes outside the segments it accepts.
 *  - The caller guarantees that q, k, v and out hold at least cu_seqlens[N]
 *    rows; the library cannot check this without a device-to-host sync.
 */
#ifndef VIT_H_
#define VIT_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vit_status {
  VIT_OK = 0,
  VIT_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, non-finite value */
  VIT_ERR_UNSUPPORTED = 2, /* head dim or size outside the supported set */
  VIT_ERR_HIP = 3          /* a HIP runtime call failed; the message names it */
};

enum vit_dtype {
  VIT_F32 = 0,  /* IEEE binary32 */
  VIT_BF16 = 1  /* bfloat16 (8-bit exponent, 7-bit fraction) */
};

/* Which elements the 2D rotary embedding pairs (see vit_qk_norm_rope_ex). */
enum vit_rope_mode {
  VIT_ROPE_NEOX = 0,   /* rotate-half: pairs (m, m + D/2) */
  VIT_ROPE_COMPLEX = 1 /* complex form: pairs (2j, 2j + 1) */
};

/* Attention flags (the `flags` argument of the _ex, planned and dense-batch calls). */
enum vit_attn_flags {
  /* Query a of a segment sees keys 0..a of that segment only.  _VisionAttentionBase
   * on the vLLM page carries is_causal (the encoders pass False); equal query
   * and key lengths, so the diagonal starts at the segment's first token. */
  VIT_ATTN_CAUSAL = 1
};

/* Device-side error bits of one work-list build (vit_varlen_worklist), OR-ed. */
enum vit_worklist_error {
  VIT_WL_ERR_CU0 = 1,      /* cu_seqlens[0] != 0: the list is empty */
  VIT_WL_ERR_NEGATIVE = 2, /* some cu_seqlens[i+1] < cu_seqlens[i]: that segment is skipped */
  VIT_WL_ERR_TOO_LONG = 4, /* some segment longer than max_seqlen: that segment is skipped */
  VIT_WL_ERR_CAPACITY = 8  /* more items than cap: the list is empty */
};

/*
 * Q/K RMSNorm followed by 2D rotary embedding, in place on q and k.
 *
 * Norm: vLLM page vllm.models.dots3_note.nvidia.vision_attention, class
 * _RMSNorm -- y = x * rsqrt(mean_d x^2 + eps) * w_d, the mean taken in fp32
 * over the head dim of each (token, head) row; q uses q_weight and k uses
 * k_weight, one [D] vector shared by all heads (_VisionAttentionBase).
 * Rotary: VisionRotaryEmbedding on the same page gives the 1-D table
 * inv_freq[j] = theta^(-2j/dim); here dim = D/2, so j < D/4.  Token t at grid
 * position (row, col) gets angles a_m = row*inv_freq[m] for m < D/4 and
 * a_m = col*inv_freq[m - D/4] for D/4 <= m < D/2, and each pair (m, m + D/2) is
 * rotated by a_m (rotate-half with the cosine widened by concatenation, as the
 * native rotary branch of MultimodalEncoderAttention.forward on the tokenspeed
 * page mm_encoder_attention.py applies it).  The norm comes first, then the
 * rotary (_qkv_with_rope).  Arithmetic is fp32; results are rounded once to the
 * tensor dtype (nearest, ties to even).
 *
 *  q, k          [total_tokens, H, D] of `dtype`, updated in place.  q may be
 *                NULL: only k is processed (q's half is then done inside the
 *                attention by vit_varlen_attn_planned_qnorm_rope).
 *  pos           int32 [total_tokens, 2] (row, col); NULL = no rotary.
 *  theta         rotary base, finite and > 0 (10000 in the pages).
 *  q_weight,
 *  k_weight      fp32 [D]; both NULL = no norm; exactly one NULL is an error
 *                (with q NULL: q_weight must be NULL, k_weight optional).
 *  eps           >= 0 (1e-6 in the pages).
 *  D             a multiple of 8 in [8, 256].
 * total_tokens == 0 is a no-op.
 */
int vit_qk_norm_rope(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                     int dtype, const int32_t* pos, float theta, const float* q_weight,
                     const float* k_weight, float eps, hipStream_t stream);

/*
 * Token strides.  The strided entry points below take `strides`, an int64
 * array of elements between consecutive tokens of each tensor (in the order
 * the call names: q, k for the pre-pass; q, k, v, out for attention), or
 * null for contiguous [T, H, D] (H * D).  Within a token the H head rows stay
 * contiguous (head h at offset h * D).  This reads q, k and v straight out of
 * a packed [T, 3, H, D] QKV projection (stride 3 * H * D; the views both
 * pages take: reshape(seq, 3, H, D) / unbind in _VisionAttentionBase on the
 * vLLM page, qkv.split along the last dim in MultimodalEncoderAttention on
 * the tokenspeed page) and writes out into a wider [T, >= H * D] buffer.
 * Each stride must be >= H * D, < 2^26, and keep rows 16-byte aligned (a
 * multiple of 8 elements for bf16, 4 for fp32); VIT_ERR_INVALID_ARG otherwise.
 */

/* vit_qk_norm_rope on strided q and k (strides[0], strides[1]). */
int vit_qk_norm_rope_strided(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                             int dtype, const int32_t* pos, float theta, const float* q_weight,
                             const float* k_weight, float eps, const int64_t* strides,
                             hipStream_t stream);

/*
 * vit_qk_norm_rope_strided with a choice of rotary pairing, rope_mode:
 *  VIT_ROPE_NEOX     rotate-half, pairs (m, m + D/2) (as vit_qk_norm_rope);
 *  VIT_ROPE_COMPLEX  the complex form that position_embedding_mode
 *                    "complex_rope" selects in MultimodalEncoderAttention on
 *                    the tokenspeed page (packed_qkv_complex_rotary, whose
 *                    body the page does not show): elements (2j, 2j + 1) form
 *                    the complex number x[2j] + i x[2j+1], multiplied by
 *                    exp(i a_j) with the same D/2 angles a_j (row table for
 *                    j < D/4, column table after).
 * Any other rope_mode: VIT_ERR_INVALID_ARG.  Other arguments, layout and
 * errors as for vit_qk_norm_rope_strided.
 */
int vit_qk_norm_rope_ex(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                        int dtype, const int32_t* pos, float theta, const float* q_weight,
                        const float* k_weight, float eps, int rope_mode, const int64_t* strides,
                        hipStream_t stream);

/*
 * vit_qk_norm_rope_ex followed by vit_varlen_worklist, in one kernel launch: the
 * two are independent, so one extra workgroup of the pre-pass launch builds
 * the work-list while the others normalise and rotate q and k.  Arguments,
 * results and errors are exactly those of the two calls (checked before
 * anything is enqueued).  A list whose build needs more than 24 KiB of LDS
 * (num_seqs > 2048) gets a launch of its own, as does a list when the
 * pre-pass has nothing to do.
 */
int vit_qk_norm_rope_worklist(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                              int dtype, const int32_t* pos, float theta, const float* q_weight,
                              const float* k_weight, float eps, int rope_mode,
                              const int64_t* strides, const int32_t* cu_seqlens, int num_seqs,
                              int max_seqlen, int block_m, int32_t* items, int64_t cap,
                              int32_t* meta, hipStream_t stream);

/*
 * vit_qk_norm_rope_worklist out of place: q and k receive the normalised and
 * rotated rows of q_src and k_src, which are only read.  This is the form the
 * step takes on the vLLM page (_qkv_with_rope in _VisionAttentionBase): the
 * norm and the rotary make new q and k from the views of the QKV projection's
 * output, which stays as it was.  With neither norm nor rotary requested the
 * rows are copied.
 *
 *  q_src, k_src  [total_tokens, H, D] of `dtype`, token strides src_strides[0]
 *                and src_strides[1] (null: contiguous); q_src is null exactly
 *                when q is.
 *  q, k          the outputs, token strides strides[0], strides[1].  Each is
 *                either its own source (the same pointer and stride: the
 *                in-place call) or shares no byte with q_src or k_src; other
 *                overlaps are VIT_ERR_INVALID_ARG.
 *  cu_seqlens, items, meta
 *                all null: no work-list is built (num_seqs, max_seqlen,
 *                block_m and cap are then ignored); all given: as for
 *                vit_qk_norm_rope_worklist; a mix is VIT_ERR_INVALID_ARG.
 * Everything else as for vit_qk_norm_rope_worklist, and errors as for it
 * (checked before anything is enqueued).
 */
int vit_qk_norm_rope_into(const void* q_src, const void* k_src, const int64_t* src_strides,
                          void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                          int dtype, const int32_t* pos, float theta, const float* q_weight,
                          const float* k_weight, float eps, int rope_mode, const int64_t* strides,
                          const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int block_m,
                          int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream);

/*
 * Varlen attention, bf16 in and out, fp32 accumulation and softmax.
 *
 * For every segment i, head h and query a in the segment:
 *   out[a,h,:] = sum_b softmax_b(scale * <q[a,h,:], k[b,h,:]>) v[b,h,:],
 * b ranging over the same segment (VisionAttentionV2.forward on the vLLM page;
 * flash_attn_varlen_func with cu_seqlens_q = cu_seqlens_k on the tokenspeed page).
 * The tokenspeed page defaults the scale to head_size^-0.5 when the caller
 * passes none; here it is always explicit, and any finite value is accepted,
 * zero and negative ones included (scale 0 gives every key of the segment the
 * same weight, so each row is the mean of its segment's v rows: a closed form
 * the tests use).
 *
 *  q, k, v       bf16 [T, H, D], T = cu_seqlens[num_seqs].
 *  cu_seqlens    int32 [num_seqs + 1] on the device.
 *  num_seqs      N >= 0, at most 8192.
 *  max_seqlen    an upper bound on every segment length, supplied by the
 *                caller so no device-to-host sync is needed (the capture-safe
 *                path of _varlen_metadata on the tokenspeed page); longer
 *                segments are skipped and flagged (VIT_WL_ERR_TOO_LONG).
 *                (max_seqlen + 64) * token stride * 2 must not exceed 2^30
 *                bytes, the span the kernel addresses with 32-bit buffer
 *                offsets (VIT_ERR_UNSUPPORTED otherwise).
 *  head_dim      one of 32, 64, 80, 96, 128.
 *  out           bf16 [T, H, D]; must not alias q, k or v.  Rows of skipped
 *                segments are left untouched.
 * Builds the work-list in library-owned scratch (one buffer per device and
 * stream, kept until vit_release), then runs the attention kernel.  When a
 * call needs more capacity than the stream's buffer has, the buffer is
 * replaced with stream-ordered allocation on `stream` (hipFreeAsync of the
 * old one, hipMallocAsync of a larger one): the host never waits, and the
 * old buffer is released after the stream's earlier work.  Callers that must
 * not allocate at all use vit_varlen_attn_noalloc.  num_seqs == 0 or
 * max_seqlen == 0 is a no-op.
 */
int vit_varlen_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                    int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                    void* out, hipStream_t stream);

/* Same operation and parameters with fp32 q, k, v, out; fp32 arithmetic throughout. */
int vit_varlen_attn_f32(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                        int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                        void* out, hipStream_t stream);

/*
 * vit_varlen_attn (dtype VIT_BF16) or vit_varlen_attn_f32 (VIT_F32) that also
 * writes each row's log-sum-exp of scores, natural log:
 *   lse[a, h] = log sum_b exp(scale * <q[a,h,:], k[b,h,:]>), b over a's segment
 * -- the second result the tokenspeed page's FA4 varlen call returns next to
 * the output (vision_attn_fa4) and that its cuDNN prefill call is asked for
 * (return_lse in vision_attn_flashinfer_cudnn).  It lets partial results over
 * key ranges be merged.
 *  lse   fp32 [T, H] on the device, token-major like out, 4-byte aligned, not
 *        aliasing q, k, v or out; rows outside the accepted segments are left
 *        untouched.  Null: only out is written.
 */
int vit_varlen_attn_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                        int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                        int dtype, void* out, float* lse, hipStream_t stream);

/* vit_varlen_attn_lse on strided q, k, v and out (strides[0..3]; see above). */
int vit_varlen_attn_strided(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                            int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                            int dtype, void* out, float* lse, const int64_t* strides,
                            hipStream_t stream);

/*
 * The general form: vit_varlen_attn_strided plus `flags` (enum
 * vit_attn_flags; 0 = non-causal, exactly vit_varlen_attn_strided).  Unknown
 * flag bits: VIT_ERR_INVALID_ARG.  With VIT_ATTN_CAUSAL a work item visits
 * only the key tiles up to its last query row.
 */
int vit_varlen_attn_ex(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                       int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                       int dtype, int flags, void* out, float* lse, const int64_t* strides,
                       hipStream_t stream);

/*
 * vit_varlen_attn_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same operation, arguments, layout and errors as
 * vit_varlen_attn_ex, and the same kernels; the work-list is built in a fixed
 * device array of the library instead of the per-stream scratch, so the call
 * makes no device or host allocation (no hipMalloc, hipFree or stream-ordered
 * allocation).
 *  - Limit: num_seqs * ceil(max_seqlen / vit_attn_block_m(num_heads, head_dim,
 *    dtype)) at most 262144 work items (the array holds 4 MiB of items);
 *    larger calls return VIT_ERR_UNSUPPORTED with nothing enqueued.
 *  - The array exists once per GPU, from the library's load until the process
 *    ends, and every call on that GPU uses it: calls that overlap in time on
 *    one GPU (other streams, other threads) race on it and can compute wrong
 *    results, so serialise them.  Each call rewrites the list count, the error
 *    bits and every item it reads, so nothing has to be cleared between calls.
 *  - Bad segments are skipped as vit_varlen_attn_ex skips them; the error
 *    bits stay in the array and vit_device_error does not report them (build
 *    a list with vit_varlen_worklist to read them).
 */
int vit_varlen_attn_noalloc(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                            int num_heads, int head_dim, float scale, int dtype, int flags,
                            void* out, float* lse, const int64_t* strides, hipStream_t stream);

/*
 * Attention over a uniform batch: `batch` segments of `seq_len` tokens each,
 * segment i covering tokens [i * seq_len, (i + 1) * seq_len).  This is the
 * case _varlen_metadata on the tokenspeed page fills in when cu_seqlens is
 * None (arange(0, (bsz + 1) * seq_len, seq_len)); the result is that of
 * vit_varlen_attn_strided on those cu_seqlens, bit for bit.  No cu_seqlens,
 * work-list or scratch exists: each workgroup derives its segment and q-tile
 * from its index, so the call allocates nothing and reads no metadata.
 *  q, k, v, out, lse, strides, dtype, scale, flags   as for vit_varlen_attn_ex
 *                (T = batch * seq_len rows).
 *  batch, seq_len   >= 0 (either 0: no-op); batch * seq_len must fit in int32
 *                and (seq_len + 64) * token stride * 2 must not exceed 2^30
 *                bytes (VIT_ERR_UNSUPPORTED otherwise).
 */
int vit_dense_batch_attn(const void* q, const void* k, const void* v, int batch, int seq_len,
                         int num_heads, int head_dim, float scale, int dtype, int flags,
                         void* out, float* lse, const int64_t* strides, hipStream_t stream);

/*
 * Query rows per (segment, q-tile) work item of the attention kernel for this
 * shape and dtype, or a negative VIT_ERR_* code for an unsupported shape.
 */
int vit_attn_block_m(int num_heads, int head_dim, int dtype);

/* Work-list capacity (items) for num_seqs segments no longer than max_seqlen:
 * num_seqs * ceil(max_seqlen / block_m); -1 on bad arguments. */
int64_t vit_worklist_capacity(int num_seqs, int max_seqlen, int block_m);

/*
 * Work-list builder.  The pages hand cu_seqlens straight to their kernels and
 * show no scheduler; this list is the library's own schedule:
 *  - segment i has len_i = cu_seqlens[i+1] - cu_seqlens[i];
 *  - segments with len_i > 0 that pass validation (enum vit_worklist_error)
 *    are ordered by len_i descending, ties by i ascending (longest first);
 *  - each contributes items (i, j) for j = 0 .. ceil(len_i / block_m) - 1.
 *  items   int32 [cap, 4], 16-byte aligned: row r < count is (segment, q-tile,
 *          cu_seqlens[segment], length of the segment); rows count ..
 *          min(cap, count + 2048) - 1 get segment = -1, so the attention
 *          kernel reads one 16-byte item per work unit and stops at the first
 *          marked row, without reading the count or cu_seqlens first.
 *  cap     >= vit_worklist_capacity(num_seqs, max_seqlen, block_m).
 *  meta    int32 [2]: meta[0] = count, meta[1] = error bits, both written.
 * Runs entirely on the device (no host sync).  num_seqs at most 8192.
 * The count and the error bits share one caller buffer, and cap is int64, so
 * capacities past 2^31 items are expressible; the capacity is still bounded by
 * 2^30 items (VIT_ERR_UNSUPPORTED beyond).
 */
int vit_varlen_worklist(const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int block_m,
                        int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream);

/*
 * Attention over a work-list built by vit_varlen_worklist with
 * block_m = vit_attn_block_m(num_heads, head_dim, dtype) for the same
 * cu_seqlens.  Lets one list serve every layer of an encoder tower.
 * dtype selects the bf16 (VIT_BF16) or fp32 (VIT_F32) kernel; lse is as for
 * vit_varlen_attn_lse (null: not written); strides as for
 * vit_varlen_attn_strided (null: contiguous); flags as for vit_varlen_attn_ex;
 * cap is the capacity the list was built with; the other arguments are those
 * of vit_varlen_attn.  The
 * list's max_seqlen must satisfy the bound vit_varlen_attn checks: the bf16
 * kernel skips a segment beyond the 32-bit offset span (this call cannot see
 * max_seqlen, so it is not rejected here).
 */
int vit_varlen_attn_planned(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, const int32_t* items, int64_t cap,
                            const int32_t* meta, int num_heads, int head_dim, float scale,
                            int dtype, int flags, void* out, float* lse, const int64_t* strides,
                            hipStream_t stream);

/*
 * vit_varlen_attn_planned with the Q half of the pre-pass done inside the
 * attention kernel: each work item applies RMSNorm (q_weight, eps; null
 * q_weight: none) and then the 2D rotary (pos, theta, rope_mode; null pos:
 * none) to its query rows in registers, as vit_qk_norm_rope_ex does to q,
 * and feeds the result to the MFMAs.  q in memory is not modified.  This is
 * _qkv_with_rope (vLLM page: norm, then rotary) with q's read and write of the
 * separate pre-pass removed; k is still prepared by vit_qk_norm_rope_ex (or
 * vit_qk_norm_rope_worklist, or vit_qk_norm_rope_into) called with q = null.
 *  pos        int32 [T, 2] (row, col), 8-byte aligned, or null.
 *  q_weight   fp32 [D], 16-byte aligned, or null.
 *  theta, eps, rope_mode   as for vit_qk_norm_rope_ex (checked when used).
 * The rotary angle is reduced to a fraction of a turn exactly and evaluated
 * with the hardware sine and cosine, so results match the separate pre-pass
 * within the attention tolerance, not bit for bit.  Other arguments, layout
 * and errors as for vit_varlen_attn_planned; head_dim at most 128.
 */
int vit_varlen_attn_planned_qnorm_rope(
    const void* q, const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* items,
    int64_t cap, const int32_t* meta, int num_heads, int head_dim, float scale, int dtype,
    int flags, const int32_t* pos, float theta, const float* q_weight, float eps, int rope_mode,
    void* out, float* lse, const int64_t* strides, hipStream_t stream);

/*
 * vit_varlen_attn_planned with the whole pre-pass done inside the attention
 * kernel, on q and on k: each work item normalises and rotates its query
 * rows as vit_varlen_attn_planned_qnorm_rope does, and every K tile it
 * visits is normalised (k_weight) and rotated in LDS before its scores are
 * formed, so neither q nor k is read and written by a separate pre-pass.
 * This is _qkv_with_rope (vLLM page: the q and k norms, then rotary on both)
 * fused into the attention's tile loads, as the FA4 route on the tokenspeed
 * page (MultimodalEncoderAttention.forward) fuses the rotary into the QKV
 * split.  q and k in memory are not modified.
 *  pos                  int32 [T, 2] (row, col), 8-byte aligned, or null.
 *  q_weight, k_weight   fp32 [D], 16-byte aligned; both null (no norm) or
 *                       both given, else VIT_ERR_INVALID_ARG.
 *  theta, eps, rope_mode   as for vit_qk_norm_rope_ex (checked when used).
 * Each unit transforms every K tile it visits, so a segment's keys are
 * transformed once per q-tile of that segment (block_m rows each): the call
 * pays where segments are short (one or two q-tiles).  Angles are reduced to
 * a fraction of a turn exactly; the bf16 kernel then takes the hardware sine
 * and cosine, the fp32 kernel sincosf.  Results match the separate pre-pass
 * within the attention tolerance, not bit for bit.  Other arguments, layout
 * and errors as for vit_varlen_attn_planned.
 */
int vit_varlen_attn_planned_qk_norm_rope(
    const void* q, const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* items,
    int64_t cap, const int32_t* meta, int num_heads, int head_dim, float scale, int dtype,
    int flags, const int32_t* pos, float theta, const float* q_weight, const float* k_weight,
    float eps, int rope_mode, void* out, float* lse, const int64_t* strides, hipStream_t stream);

/*
 * Reads (and with reset != 0 clears) the work-list error bits (enum
 * vit_worklist_error) left in the library's scratch by the most recent call
 * that builds its own work-list (vit_varlen_attn, _f32, _lse, _strided, _ex)
 * on the current device and `stream`.  Synchronises that stream.  *err = 0 if
 * no such call has run yet.  Calls on a caller's list report in its meta[1];
 * vit_dense_batch_attn has no list and no error bits.
 */
int vit_device_error(hipStream_t stream, int32_t* err, int reset);

/* Message of the last failed call on this thread ("" if none). */
const char* vit_last_error(void);

/*
 * Timing hook for profilers and benchmarks.  The next call on this host thread
 * of vit_qk_norm_rope, vit_qk_norm_rope_worklist (its combined launch),
 * vit_varlen_worklist, vit_varlen_attn_planned,
 * vit_varlen_attn or vit_varlen_attn_f32 records `start` when its kernel's
 * dispatch begins and `stop` when that kernel ends (hipExtLaunchKernel's
 * dispatch timestamps: the kernel alone, without launch gaps); the hook is
 * then cleared, whether that call succeeds or not.  For vit_varlen_attn and
 * vit_varlen_attn_f32 the timed kernel is the attention kernel, not the
 * work-list build they launch first.  A call that launches no kernel records
 * both events back to back on its stream.
 *  start, stop: events created with timing enabled, owned by the caller, or
 *               both null to clear the hook.
 * Returns VIT_ERR_INVALID_ARG when exactly one of them is null.
 */
int vit_time_next_kernel(hipEvent_t start, hipEvent_t stop);

/* Frees all library-owned scratch on every device (waits for each device first). */
void vit_release(void);

#ifdef __cplusplus
}
#endif

#endif /* VIT_H_ */
