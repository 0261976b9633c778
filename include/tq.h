/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant-style KV-cache codec.
 *
 * The method is the KV leg of the mlx-bun TurboQuant design pages
 * ("Algorithm (vllm-metal reference semantics, exact)" on the TurboQuant
 * page; "Algorithm" on the TurboQuant KV design page).  Per token and per
 * kv-head, head_dim is split into groups of 32:
 *   keys   -- no rotation; asymmetric affine per group, fp16 scale and zero;
 *             signed int8 at 8 bits, packed unsigned at 2/4/5 bits;
 *   values -- y = FWHT(x * signs) / sqrt(d); per-group RMS scale (fp16);
 *             Lloyd-Max index of y / (scale + 1e-8); packed bitstream.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All data pointers are DEVICE pointers unless stated; the caller owns
 *   every buffer.  The library allocates nothing and keeps no mutable
 *   state; calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *   default stream) and may be made from several host threads.
 * - bf16 and fp16 travel as raw 16-bit patterns (uint16_t).
 * - Rows.  One (token, kv-head) pair is a "row".  A bf16 row is head_dim
 *   contiguous elements; a plane row is tq_plane_row_bytes() contiguous
 *   bytes.  tq_rows addresses rows as
 *       row(s, t, h) = s*seq_stride + t*tok_stride + h*head_stride
 *   counted in rows of the buffer it describes, so a contiguous
 *   [L, T, H, d] tensor has (n_seq, n_tok, n_head) = (L, T, H) and strides
 *   (T*H, H, 1), and a [B, H, N_cap] cache window has strides (H*N_cap, 1, N_cap).
 * - Alignment: bf16 tensors, the sign vector, the workspace and the query /
 *   output of the decode call are 16-byte aligned; the packed planes k_q and
 *   v_q are 8-byte aligned; the fp16 planes are 2-byte aligned.  Plane row
 *   lengths keep these for any row offset.  Input and output buffers must
 *   not overlap.
 * - Counts: a codec or cache call serves fewer than 2^31 rows, each count
 *   of a tq_rows below 2^31; an attention call fewer than 2^30 query rows
 *   (batch x queries x query heads).  Larger calls are TQ_E_SHAPE.
 * - Validation runs on the host before any launch; on error nothing is
 *   launched and a negative TQ_E_* code is returned.  Zero rows is a no-op.
 *   Device faults surface at the caller's next synchronisation.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_OK 0
#define TQ_E_HEAD_DIM (-1)  /* head_dim not served by the call (see each call)   */
#define TQ_E_BITS (-2)      /* bit widths not served by the call (see each call) */
#define TQ_E_NULL (-3)      /* a required pointer is NULL                        */
#define TQ_E_SHAPE (-4)     /* negative count/stride, mismatched counts, Hq % Hkv */
#define TQ_E_ALIGN (-5)     /* a base pointer breaks the alignment rules below   */
#define TQ_E_WORKSPACE (-6) /* decode workspace missing or too small             */
#define TQ_E_HIP (-7)       /* the HIP runtime reported a launch error           */
#define TQ_E_PLANE (-8)     /* plane index out of range                          */
#define TQ_E_OVERLAP (-9)   /* an output buffer overlaps an input or itself      */

/* Quantization scheme, validated on every call.  The pages' served sets:
 * head_dim in {64,128,256,512}; k_bits in {2,4,5,8}; v_bits in {2,3,4,5,8}
 * (TurboQuant page, "Algorithm" and the scheme list under "Architecture"). */
typedef struct {
  int32_t head_dim;
  int32_t k_bits;
  int32_t v_bits;
} tq_scheme;

/* The five planes of a quantized cache, addressed by the same row index.
 * Per row (d = head_dim, G = d/32):
 *   k_q     : k_bits == 8 -> int8[d]; else uint8[d*k_bits/8] packed stream
 *   k_scale : fp16[G]     k_zero : fp16[G]
 *   v_q     : uint8[d*v_bits/8] packed stream
 *   v_scale : fp16[G]
 * Packed streams are little-endian: element i occupies stream bits
 * [i*b, i*b+b), index LSB first; stream bit n is bit n%8 of byte n/8
 * (TurboQuant page, "Algorithm", values bullet "Pack"). */
typedef struct {
  void* k_q;
  void* k_scale;
  void* k_zero;
  void* v_q;
  void* v_scale;
} tq_planes;

enum { TQ_PLANE_K_Q = 0, TQ_PLANE_K_SCALE, TQ_PLANE_K_ZERO, TQ_PLANE_V_Q, TQ_PLANE_V_SCALE };

typedef struct {
  int64_t n_seq, n_tok, n_head;
  int64_t seq_stride, tok_stride, head_stride;
} tq_rows;

/* TQ_OK or TQ_E_HEAD_DIM / TQ_E_BITS for the scheme (host only, pure). */
int32_t tq_check_scheme(const tq_scheme* scheme);

/* Bytes per row of one plane (TQ_PLANE_*), or a negative TQ_E_* code.
 * k8v3 at d=128 totals 200 bytes against 512 of bf16 K+V (TurboQuant page,
 * "Algorithm", bytes paragraph).  Host only, pure. */
int64_t tq_plane_row_bytes(const tq_scheme* scheme, int32_t plane);

/* Sum of the five planes' row bytes, or a negative TQ_E_* code: the bytes
 * one token-head occupies in the cache, 200 at k8v3 d=128 (TurboQuant page,
 * "Algorithm", bytes paragraph; TurboQuant KV design page, "Algorithm").
 * Host only, pure. */
int64_t tq_row_bytes(const tq_scheme* scheme);

/* Copies the library's value codebook for `bits` in {1,2,3,4,5,8} into host
 * arrays: 2^bits ascending float32 centroids and 2^bits - 1 ascending
 * boundaries.  The 3-bit table is the one the pages print; the others are
 * the Lloyd-Max fixed points for N(0,1) rounded to float32 (TurboQuant page,
 * "Algorithm", values bullet).  Host only.  Returns TQ_OK or TQ_E_BITS. */
int32_t tq_codebook(int32_t bits, float* centroids, float* boundaries);

/* Quantize K and V rows into the five planes.
 *   k_bf16, v_bf16 : bf16 rows addressed by *in_rows
 *   signs          : int8[head_dim] of +1/-1, the value sign vector
 *   out            : planes addressed by *out_rows (same n_seq/n_tok/n_head)
 * Keys (TurboQuant page, "Algorithm", keys bullets), per 32-group in fp32:
 *   k_bits = 8      scale = (max-min)/254, zero = round((max+min)/(2 scale)),
 *                   idx = clip(round(x/scale - zero), -127, 127)
 *   k_bits in 2,4,5 scale = (max-min)/(2^b-1), zero = round(min/scale),
 *                   idx = clip(round(x/scale - zero), 0, 2^b-1)
 *   scale and zero are stored as fp16 after the index is formed.
 * Values (same section, values bullets): y = FWHT(x*signs)/sqrt(d);
 *   scale = sqrt(mean(y^2)) per group; idx = #{boundaries < y/(scale+1e-8)}.
 *   For 2, 3 and 4 value bits the index is found without dividing, so it may
 *   differ by one where y/(scale+1e-8) lies within 5e-7 of a boundary (exact
 *   equality included), inside the tie window the pages allow; 5- and 8-bit
 *   values and all keys are exact.
 * Edge semantics: min/max propagate NaN (and order -0 below +0); round is
 * half-to-even; clip sends NaN to the low end; a constant key group gives
 * scale 0 and zero +-Inf (NaN for an all-zero group); any NaN stored as
 * fp16 is 0x7E00.  Returns TQ_OK or a TQ_E_* code. */
int32_t tq_quantize_kv(const tq_scheme* scheme, const uint16_t* k_bf16, const uint16_t* v_bf16,
                       const tq_rows* in_rows, const int8_t* signs, const tq_planes* out,
                       const tq_rows* out_rows, void* stream);

/* Dequantize planes back to bf16 rows (either output may be NULL to skip it).
 *   keys   : k_hat = (float(idx) + float(zero16)) * float(scale16)
 *            (f32 add before the multiply; TurboQuant page, packed-value decode
 *            section on the joint K/V decoder)
 *   values : signs * FWHT(centroid[idx] * float(scale16)) / sqrt(d), the
 *            transform first and the signs last (TurboQuant KV design page,
 *            "Algorithm", dequant bullet)
 * Outputs round to nearest even; NaN is written as 0x7FC0. */
int32_t tq_dequantize_kv(const tq_scheme* scheme, const tq_planes* in, const tq_rows* in_rows,
                         const int8_t* signs, uint16_t* k_bf16, uint16_t* v_bf16,
                         const tq_rows* out_rows, void* stream);

/* Append new tokens into a [batch, kv-head, capacity] cache at per-sequence
 * positions: only the appended tokens are quantized, the rest of the cache is
 * untouched (TurboQuant page, "Architecture in mlx-bun": the cache's
 * update quantizes just the newly appended tokens into packed storage).
 *   k_bf16, v_bf16 : [batch, n_new, n_kv_heads, head_dim], contiguous
 *   cache          : planes; row(b, g, t) = b*seq_stride_rows + g*head_stride_rows + t
 *   positions      : device int32[batch]; token j of sequence b goes to cache
 *                    token positions[b] + j, and is written only when
 *                    0 <= positions[b] + j < capacity (others are dropped)
 * Quantization is exactly that of tq_quantize_kv.  Returns TQ_OK or TQ_E_*. */
int32_t tq_append_kv(const tq_scheme* scheme, const uint16_t* k_bf16, const uint16_t* v_bf16, int32_t batch,
                     int32_t n_new, int32_t n_kv_heads, const int8_t* signs, const tq_planes* cache,
                     int64_t seq_stride_rows, int64_t head_stride_rows, const int32_t* positions,
                     int32_t capacity, void* stream);

/* Fetch the active window of every (sequence, kv head) as bf16 (TurboQuant
 * page, "Architecture in mlx-bun": the cache returns its dequantized bf16
 * active window; "Deferred inverse FWHT": the V window may stay in the
 * rotated domain so that attention un-rotates its output once).
 *   cache          : planes addressed as in tq_append_kv
 *   capacity       : cache tokens per (sequence, kv head); no cache row at or
 *                    past it is read
 *   lens           : device int32[batch]; tokens t < min(lens[b], capacity)
 *                    are live
 *   window         : tokens per output row block (>= every lens[b] the caller
 *                    wants whole, and may exceed the capacity); output rows
 *                    that are not live are written as +0
 *   values_rotated : 0 -> V as tq_dequantize_kv (signs needed);
 *                    1 -> V rows are centroid[idx] * scale16 rounded to bf16,
 *                    no transform and no signs (signs may be NULL)
 *   k_bf16, v_bf16 : [batch, n_kv_heads, window, head_dim], either may be NULL
 * Keys are always dequantized as in tq_dequantize_kv.  Returns TQ_OK or TQ_E_*. */
int32_t tq_fetch_kv(const tq_scheme* scheme, const tq_planes* cache, int32_t batch, int32_t n_kv_heads,
                    int64_t seq_stride_rows, int64_t head_stride_rows, int32_t capacity, const int32_t* lens,
                    int32_t window, const int8_t* signs, int32_t values_rotated, uint16_t* k_bf16,
                    uint16_t* v_bf16, void* stream);

/* Cache capacity grows in steps of this many tokens (campaign execution-log
 * page, the KV append dispatch probe: growth happens at 256-step
 * boundaries). */
#define TQ_CAPACITY_STEP 256

/* The capacity a cache that must hold `tokens` tokens grows to: the smallest
 * multiple of TQ_CAPACITY_STEP that is >= tokens (0 for 0).  Returns
 * TQ_E_SHAPE for a negative count or a result past INT32_MAX.  Host only. */
int64_t tq_grown_capacity(int64_t tokens);

/* Re-lay a [batch, kv-head, capacity] cache at another capacity (campaign
 * execution-log page, the KV append dispatch probe: a cache that grows
 * allocates zero padding and concatenates its old storage in front of it).
 * For every sequence b < batch, kv head g < n_kv_heads and plane:
 *   dst row t = src row t          t < min(src_capacity, dst_capacity)
 *   dst row t = zero bytes         min(...) <= t < dst_capacity
 * so dst_capacity > src_capacity grows the cache and a smaller one trims it
 * (rows past dst_capacity are dropped).  Source rows past the kept ones are
 * not read.
 *   src, dst       : planes; row(b, g, t) = b*seq_stride_rows + g*head_stride_rows + t
 *                    with each side's own strides (rows of its own planes)
 *   dst strides    : each (b, g) segment of dst_capacity rows must sit apart:
 *                    over the axes of extent > 1, the smaller stride s1 (axis
 *                    extent n1) is >= dst_capacity and the larger is
 *                    >= (n1 - 1) * s1 + dst_capacity.  [batch, kv-head,
 *                    capacity] and [kv-head, batch, capacity], padded or not,
 *                    qualify.
 * No byte any dst plane writes may lie in a src plane's read range or in
 * another dst plane (TQ_E_OVERLAP): the call copies, it does not move rows
 * in place.  A plane whose bases and segment offsets are all 16-byte aligned
 * (any capacity that is a multiple of 16 at the usual strides) is copied
 * 16 bytes per lane, otherwise 2 bytes per lane.  Returns TQ_OK or a TQ_E_*
 * code. */
int32_t tq_grow_kv(const tq_scheme* scheme, int32_t batch, int32_t n_kv_heads, const tq_planes* src,
                   int64_t src_seq_stride_rows, int64_t src_head_stride_rows, int32_t src_capacity,
                   const tq_planes* dst, int64_t dst_seq_stride_rows, int64_t dst_head_stride_rows,
                   int32_t dst_capacity, void* stream);

/* Un-rotate bf16 rows: out = bf16(signs * FWHT(in) / sqrt(d)), the transform
 * first and the signs last -- the inverse of the value rotation.  This is
 * what an attention site that consumed a rotated V window (tq_fetch_kv with
 * values_rotated) applies to its output rows, once per query row (TurboQuant
 * page, "Deferred inverse FWHT").
 *   in_bf16, out_bf16 : bf16 rows addressed by *in_rows / *out_rows (same
 *                       counts); the same buffer and row map may be given
 *                       for both (in place)
 *   signs             : int8[head_dim] of +1/-1, the cache's sign vector
 * Arithmetic is float32 in the butterfly order of the quantizer; NaN is
 * written as 0x7FC0.  Returns TQ_OK, TQ_E_HEAD_DIM, TQ_E_NULL, TQ_E_ALIGN or
 * TQ_E_SHAPE. */
int32_t tq_unrotate_rows(int32_t head_dim, const uint16_t* in_bf16, const tq_rows* in_rows, const int8_t* signs,
                         uint16_t* out_bf16, const tq_rows* out_rows, void* stream);

/* Workspace bytes tq_decode_attn_quant needs for these sizes (host only);
 * 0 when the arguments are invalid.  The workspace holds one (m, l,
 * rotated-domain accumulator) partial per query row and context split; the
 * combine merges them and applies the inverse rotation once per row
 * (TurboQuant page, "Deferred inverse FWHT"). */
size_t tq_decode_attn_workspace_bytes(const tq_scheme* scheme, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t max_ctx);

/* Fused dequant-on-fetch GQA decode attention over a quantized cache, one
 * query per sequence.  For batch b and query head h (kv head
 * g = h / (n_q_heads / n_kv_heads)):
 *   s_t = softmax_scale * q . k_hat_t           (t < ctx_lens[b])
 *   a   = sum_t softmax(s)_t * z_t               z = centroid[idx] * scale16
 *   out = signs * FWHT(a) / sqrt(d)             (bf16)
 * i.e. values are accumulated in the rotated domain and un-rotated once per
 * output row (TurboQuant page, "Deferred inverse FWHT").
 *   q_bf16    : [batch, n_q_heads, head_dim]
 *   cache     : planes; row(b, g, t) = b*seq_stride_rows + g*head_stride_rows + t
 *   ctx_lens  : device int32[batch]; values are clamped to [0, max_ctx] and a
 *               sequence with 0 tokens gets an all-zero output row
 *   max_ctx   : cache capacity in tokens (>= 1); sizes the launch
 *   out_bf16  : [batch, n_q_heads, head_dim]
 *   workspace : device scratch of >= tq_decode_attn_workspace_bytes() bytes
 * Planes may hold any finite scale and zero (fractions and subnormals
 * included): keys enter as (idx + zero16) * scale16 in float32.  A NaN or
 * infinite scale or zero in a visible row makes the result unspecified
 * (the dequantize and fetch calls define those cases bit for bit). */
int32_t tq_decode_attn_quant(const tq_scheme* scheme, const uint16_t* q_bf16, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache,
                             int64_t seq_stride_rows, int64_t head_stride_rows,
                             const int32_t* ctx_lens, int32_t max_ctx, float softmax_scale,
                             const int8_t* signs, uint16_t* out_bf16, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Multi-query form of tq_decode_attn_quant: n_queries >= 1 query tokens per
 * sequence, each attending causally to the cache (the speculative / chunked
 * decode shape; the pages' attention research runs GQA 6 at d = 256 over the
 * quantized cache, TurboQuant page, "Packed-value decode fusion
 * investigation").  Query m of sequence b is the cached token at position
 * ctx_lens[b] - n_queries + m (the new tokens are already appended) and sees
 * tokens t <= that position:
 *   s_t = softmax_scale * q_{b,m,h} . k_hat_t      (t < ctx_lens[b] - n_queries + 1 + m)
 *   out_{b,m,h} = signs * FWHT(sum_t softmax(s)_t z_t) / sqrt(d)
 * A query with no visible token gets an all-zero row.
 *   q_bf16, out_bf16 : [batch, n_queries, n_q_heads, head_dim]
 *   workspace        : >= tq_attn_quant_workspace_bytes() bytes, 16-byte aligned
 * Everything else as tq_decode_attn_quant, which is this call with
 * n_queries = 1.  Returns TQ_OK or a TQ_E_* code. */
size_t tq_attn_quant_workspace_bytes(const tq_scheme* scheme, int32_t batch, int32_t n_queries, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t max_ctx);
int32_t tq_attn_quant(const tq_scheme* scheme, const uint16_t* q_bf16, int32_t batch, int32_t n_queries,
                      int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache, int64_t seq_stride_rows,
                      int64_t head_stride_rows, const int32_t* ctx_lens, int32_t max_ctx, float softmax_scale,
                      const int8_t* signs, uint16_t* out_bf16, void* workspace, size_t workspace_bytes,
                      void* stream);

/* tq_attn_quant for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the split partials kept in the
 * library's own device scratch instead of a caller workspace.  The scratch
 * is a static device array of TQ_NOALLOC_SCRATCH_BYTES bytes, one copy per
 * GPU, held from the library's load to the end of the process; its address is
 * looked up on the first call made with each device current.  `stream` must
 * belong to the calling thread's current device.  A problem whose partials
 * need more than TQ_NOALLOC_SCRATCH_BYTES (tq_attn_quant_workspace_bytes) is
 * rejected with TQ_E_WORKSPACE before anything is launched.  Calls that
 * overlap on one GPU (other streams, other host threads) share the scratch
 * and race; order them.  The call itself allocates nothing.  Returns TQ_OK
 * or a TQ_E_* code (TQ_E_HIP if the scratch cannot be located). */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t tq_attn_quant_noalloc(const tq_scheme* scheme, const uint16_t* q_bf16, int32_t batch, int32_t n_queries,
                              int32_t n_q_heads, int32_t n_kv_heads, const tq_planes* cache,
                              int64_t seq_stride_rows, int64_t head_stride_rows, const int32_t* ctx_lens,
                              int32_t max_ctx, float softmax_scale, const int8_t* signs, uint16_t* out_bf16,
                              void* stream);

/* ---------------------------------------------------------------------------
 * Paper variant (TurboQuant KV design pages, "Oracle chain": the paper's own
 * codec -- a dense random rotation from the QR decomposition of a Gaussian
 * matrix, no groups, the same codec for keys and values, an optional QJL
 * residual stage; the third design listed there supplies the whole-vector
 * norm and the MSE / Prod split).  Per row x of head_dim d:
 *   norm = ||x||_2;  y = P x;  idx_i = #{boundaries < sqrt(d) * y_i / norm}
 *   (the N(0,1) Lloyd-Max table of `bits`, tq_codebook; a zero row codes
 *   u = 0).  With qjl = 1:  rho = y - norm * c[idx] / sqrt(d);
 *   gamma = ||rho||_2;  q_i = [(S rho)_i >= 0].
 * Dequantization: y_hat = norm * c[idx] / sqrt(d)
 *   (+ sqrt(pi/2) / d * gamma * S^T (2q - 1) with qjl);  x_hat = P^T y_hat.
 * P (the rotation) and S (the Gaussian projection) are caller-drawn d x d
 * bf16 matrices, row-major, 16-byte aligned device arrays.  Products are
 * float32 sums of exact bf16 products; float32 operands (residual,
 * reconstruction) enter as bf16 hi + lo pairs.  Served: d in {64, 128, 256},
 * bits in {1, 2, 3, 4}, qjl only for d <= 128 (the matrices stay resident in
 * one compute unit's LDS).  Inputs are finite, and a row is zero or has
 * ||x||^2 in the normal float32 range [2^-126, 2^128).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t head_dim;
  int32_t bits;  /* MSE index width */
  int32_t qjl;   /* 0 or 1: add the QJL residual stage */
} tq_dense_scheme;

/* Planes of the paper variant, addressed by one row index.  Per row:
 *   idx   : uint8[d*bits/8], the packed little-endian bitstream of tq_planes
 *   norm  : float32
 *   qjl   : uint8[d/8], bit i of the stream = q_i (qjl schemes only)
 *   gamma : float32 (qjl schemes only)
 * idx and qjl are 8-byte aligned, norm and gamma 4-byte aligned. */
typedef struct {
  void* idx;
  float* norm;
  void* qjl;
  float* gamma;
} tq_dense_planes;

enum { TQ_DENSE_IDX = 0, TQ_DENSE_NORM, TQ_DENSE_QJL, TQ_DENSE_GAMMA };

/* TQ_OK, TQ_E_NULL, TQ_E_HEAD_DIM (d not in {64,128,256}, or qjl with
 * d > 128) or TQ_E_BITS (bits not in 1..4, qjl not 0/1).  Host only. */
int32_t tq_dense_check_scheme(const tq_dense_scheme* scheme);

/* Bytes per row of plane TQ_DENSE_* (0 for the QJL planes of a scheme
 * without them), or a negative TQ_E_* code.  Host only. */
int64_t tq_dense_plane_row_bytes(const tq_dense_scheme* scheme, int32_t plane);

/* Quantize bf16 rows (addressed by *in_rows) into the planes (addressed by
 * *out_rows, same counts).  proj may be NULL unless scheme->qjl.
 * Returns TQ_OK or a TQ_E_* code. */
int32_t tq_dense_quantize(const tq_dense_scheme* scheme, const uint16_t* x_bf16, const tq_rows* in_rows,
                          const uint16_t* rot_bf16, const uint16_t* proj_bf16, const tq_dense_planes* out,
                          const tq_rows* out_rows, void* stream);

/* Rebuild bf16 rows x_hat (round to nearest even, NaN as 0x7FC0) from the
 * planes.  Returns TQ_OK or a TQ_E_* code. */
int32_t tq_dense_dequantize(const tq_dense_scheme* scheme, const tq_dense_planes* in, const tq_rows* in_rows,
                            const uint16_t* rot_bf16, const uint16_t* proj_bf16, uint16_t* x_bf16,
                            const tq_rows* out_rows, void* stream);

/* ---- Checked build (for tests and debugging; no passage defines it).
 * libtq_check.so is these sources built with TQ_CHECK: every kernel tests
 * the global rows, records and byte offsets it derives against the extents
 * the host computes for each buffer from the call's own arguments (row
 * maps, capacities, counts, workspace geometry).  A failed test sets a bit
 * in a device flag word (no trap) and keeps the access in range: a store is
 * dropped, a load reads the buffer's first row.  Host only. */

/* Waits for the current device, then returns the OR of the flag bits set
 * since the last call (0: every access was in range) and clears them.
 * Returns -1 in the library built without TQ_CHECK, TQ_E_HIP if the device
 * could not be read. */
int64_t tq_check_flags(void);

/* Positive control of the checks: every extent handed to the kernels is
 * reduced by `margin` rows (bytes for tq_grow_kv) until set back to 0, so
 * that a call covering its buffers to the end must set flags.  Process-wide.
 * Returns TQ_OK, TQ_E_SHAPE for a negative margin, or -1 in the library
 * built without TQ_CHECK. */
int64_t tq_check_set_margin(int64_t margin);

/* Static description of a status code (the TQ_E_* codes above; the pages
 * ask that unsupported head dims be refused up front, TurboQuant page,
 * "Architecture in mlx-bun").  Host only. */
const char* tq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
