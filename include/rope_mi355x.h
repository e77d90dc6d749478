/*
 * rope_mi355x.h -- C ABI of the MI355X (gfx950) rotary position embedding
 * library: a cos/sin table build, a standalone in-place RoPE for ragged
 * continuous batches, and a fused RoPE + softmax attention forward with an
 * offset-causal mask.
 *
 * Pages cited (by title and section):
 *   [RF] "RoPE and FlashAttention: relative positions and online softmax"
 *   [TR] "Write Triton Rope Kernel"
 *   [PK] "RoPE + PoPE Attention Kernels" (README of pope-memory-optimal)
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer, allocated, owned and freed
 *     by the caller.  The library allocates no memory and keeps no state
 *     beyond a per-device cache of device properties; it is thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; no call synchronises.
 *   - Each call returns ROPE_OK (0) or an error status.  Every host-visible
 *     argument is validated before any HIP call is made, so argument errors
 *     are reported without a device and nothing is enqueued on error.
 *     ROPE_ERR_HIP reports a failed kernel launch (hipGetLastError).
 *   - Element types: ROPE_BF16 (bfloat16 storage) and ROPE_F16 (IEEE
 *     binary16 storage, [TR] "Inputs the agent should gather first", item 5)
 *     everywhere; ROPE_F32 for rope_apply and the fused forward.  All rotation and softmax arithmetic is
 *     fp32; cos/sin tables are always fp32 ([TR] "Kernel design rules": fp32
 *     trig, upcast after load, cast at store, rounding to nearest even).
 *   - Pairing layouts ([TR] "Inputs the agent should gather first", item 1):
 *       ROPE_NEOX: half split, pair (i, i + rot_dim/2), i < rot_dim/2;
 *       ROPE_GPTJ: adjacent pairs (2i, 2i+1), i < rot_dim/2.
 *     Pair i at position p is rotated by angle p * theta_i with
 *     theta_i = base^(-2i/rot_dim):  a' = a cos - b sin,  b' = a sin + b cos
 *     ([RF] sections 1-2; [TR] "Required reasoning process", steps 1 and 6).
 *     Dims at or past rot_dim are never modified ([TR] "Correctness
 *     requirements": the unrotated tail is bit-identical).
 *   - cos/sin tables: fp32 [table_rows, rot_dim/2], row stride rot_dim/2,
 *     row p holds cos(p theta_i) / sin(p theta_i).
 */
#ifndef ROPE_MI355X_H
#define ROPE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* pairing layouts */
#define ROPE_NEOX 0
#define ROPE_GPTJ 1

/* element types */
#define ROPE_BF16 0
#define ROPE_F32 1
#define ROPE_F16 2

/* status codes */
#define ROPE_OK 0
#define ROPE_ERR_NULL 1          /* a required pointer is NULL */
#define ROPE_ERR_SHAPE 2         /* odd or out-of-range dims, non-positive sizes, bad strides */
#define ROPE_ERR_BASE 3          /* base or position divisor <= 0 (or not finite) */
#define ROPE_ERR_UNSUPPORTED 4   /* dtype / head_dim / rot_dim / layout combination not built */
#define ROPE_ERR_EMPTY_ROW 5     /* causal with q_pos_offset < k_pos_offset: a query sees no key */
#define ROPE_ERR_TABLE_RANGE 6   /* table_rows too small for the positions the call uses */
#define ROPE_ERR_HIP 7           /* a HIP launch failed */
#define ROPE_ERR_ALIGN 8         /* a pointer or stride breaks the required alignment */
#define ROPE_ERR_SCRATCH 9       /* the call needs more scratch than the library's static array */

/* Human-readable name of a status code (static storage, never NULL). */
const char *rope_status_str(int status);

/*
 * rope_tables_build -- fill fp32 cos/sin tables for positions 0..max_pos-1.
 *
 * Defines the table of [TR] "Correctness requirements" (theta_i =
 * base^(-2i/rot_dim), angle = position * theta_i, fp32 storage) with the
 * angle formed in fp64 as [RF] section 2 does, then each of cos and sin
 * rounded once to fp32.  The frequency denominator is rot_dim, so the table
 * of a partial RoPE has rot_dim/2 columns.
 *
 *   base        > 0, finite                          (else ROPE_ERR_BASE)
 *   rot_dim     even, 2..1024                        (else ROPE_ERR_SHAPE)
 *   max_pos     1..2^31-1 rows                       (else ROPE_ERR_SHAPE)
 *   cos_out,    device fp32 [max_pos, rot_dim/2] each, written whole
 *   sin_out
 * Off the hot path: build once per (base, rot_dim, max_pos) and keep the
 * tables as device buffers ([RF] section 2).
 */
int rope_tables_build(double base, int rot_dim, int64_t max_pos,
                      float *cos_out, float *sin_out, void *stream);

/*
 * rope_tables_build_scaled -- the same tables under position interpolation
 * ([RF] section 3: positions are divided by an extension factor before the
 * angle is formed): row p holds cos((p / pos_divisor) theta_i) and
 * sin((p / pos_divisor) theta_i), the quotient and the angle in fp64, each
 * value rounded once to fp32.  pos_divisor = 1 gives exactly the tables of
 * rope_tables_build.  A larger base (NTK-aware scaling, [RF] section 3) is
 * the base argument itself.  Every kernel that reads a table (rope_apply,
 * rope_flash_attn_fwd, rope_decode_attn_fwd) then rotates at the divided
 * positions; masks and cache rows keep the integer positions.
 *
 *   pos_divisor > 0, finite                          (else ROPE_ERR_BASE)
 *   other arguments as rope_tables_build.
 */
int rope_tables_build_scaled(double base, int rot_dim, int64_t max_pos, double pos_divisor,
                             float *cos_out, float *sin_out, void *stream);

/*
 * rope_apply -- standalone RoPE on Q and K of a ragged continuous batch, in
 * place, both tensors in one launch ([TR] "Required reasoning process"
 * steps 2-10 and "Performance requirements": per-token positions, GQA head
 * counts, partial rot_dim, combined Q+K launch; [TR] "Kernel design rules":
 * in-place is race-free because each pair is loaded before it is stored).
 *
 *   q           [n_tokens, h_q heads, head_dim] elements of `dtype`, element
 *               (t, h, d) at q[t*q_stride_tok + h*q_stride_head + d]; the
 *               first rot_dim dims of every (t, h) row are rotated in place.
 *               May be NULL when h_q == 0.
 *   k           same for the h_kv key heads (may be NULL when h_kv == 0).
 *               V is never passed: it is not rotated ([RF] section 1).
 *   strides     in elements; need stride_head >= head_dim and
 *               stride_tok >= heads * stride_head (rows do not overlap).
 *   positions   int32 [n_tokens]: absolute position of each token, read per
 *               token, never derived from the token index ([TR] step 3).
 *               Values outside [0, table_rows) are clamped into that range on
 *               the device (no access leaves the table); such tokens receive
 *               the rotation of the clamped position.
 *   cos_tab,    fp32 [table_rows, rot_dim/2] (see rope_tables_build).
 *   sin_tab
 *   head_dim    even, 2..1024; rot_dim even, 2..head_dim.
 *   layout      ROPE_NEOX or ROPE_GPTJ;  dtype ROPE_BF16, ROPE_F32 or ROPE_F16.
 * n_tokens == 0, or h_q == h_kv == 0, is a no-op returning ROPE_OK.
 * Any alignment is accepted; 16-byte-aligned rows whose rotated span is a
 * whole number of 16-byte vectors take the vectorised path.
 */
int rope_apply(void *q, int64_t q_stride_tok, int64_t q_stride_head, int h_q,
               void *k, int64_t k_stride_tok, int64_t k_stride_head, int h_kv,
               const int32_t *positions, int64_t n_tokens,
               const float *cos_tab, const float *sin_tab, int64_t table_rows,
               int head_dim, int rot_dim, int layout, int dtype, void *stream);

/*
 * rope_flash_attn_fwd -- fused RoPE + softmax attention forward.
 *
 * Computes O = softmax(scale * rope(Q) rope(K)^T + mask) V per (batch, head)
 * ([RF] section 4 for the operation, section 5 for the online-softmax
 * recurrence it is evaluated with, section 2 for offset positions).  Query i
 * sits at position q_pos_offset + i and key j at k_pos_offset + j; Q and K
 * rows are rotated at those positions inside the kernel (each K tile once as
 * it is staged, no rotated copy written to memory: [PK] "Why
 * memory_optimized_pope is much slower but uses much less memory"); V is
 * never rotated.  With causal != 0, key j is visible to query i iff
 * k_pos_offset + j <= q_pos_offset + i (the offset mask of [RF] section 6
 * for cached/chunked queries); causal == 0 shows every key to every query.
 *
 *   q, o        [B, H, Sq, head_dim], contiguous, element type `dtype`;
 *               o is written whole and must not alias q, k or v.
 *   lse         optional fp32 [B, H, Sq], 4-byte aligned, not aliasing the
 *               other arrays: when non-NULL, lse[b, h, i] receives the
 *               natural-log log-sum-exp of query row i's scaled scores over
 *               its visible keys, the saved row normalisation from which
 *               rope_flash_attn_bwd recomputes the probabilities ([RF]
 *               section 5: backward reconstructs P from Q/K and saved row
 *               statistics).
 *   k, v        [B, H_kv, Sk, head_dim], contiguous.  H_kv >= 1 divides H;
 *               query head h reads key/value head h / (H / H_kv): H_kv == H
 *               is multi-head attention, H_kv < H grouped-query attention
 *               (the two head counts of [TR] "Inputs the agent should gather
 *               first", item 3; [RF] section 7 names GQA as the lever on
 *               cache bytes).  H % H_kv != 0 is ROPE_ERR_SHAPE.
 *   cos_tab,    fp32 [table_rows, rot_dim/2]; need
 *   sin_tab     table_rows >= max(q_pos_offset + Sq, k_pos_offset + Sk)
 *               (else ROPE_ERR_TABLE_RANGE).
 *   rot_dim     0 (no rotation: plain attention; tables may be NULL) or a
 *               multiple of 32 up to head_dim.
 *   head_dim    64 or 128.
 *   softmax_scale  <= 0 selects 1/sqrt(head_dim).
 *   offsets     >= 0.  With causal != 0, q_pos_offset < k_pos_offset would
 *               leave query 0 with no visible key: ROPE_ERR_EMPTY_ROW
 *               ([RF] section 5 rejects such rows).
 * Requires 16-byte-aligned q, k, v, o (else ROPE_ERR_ALIGN).
 * dtype ROPE_BF16, ROPE_F16 (the same kernels on the fp16 matrix cores) or
 * ROPE_F32.  Accumulation and softmax are fp32; for the 16-bit types the
 * rotated Q/K and the probabilities enter the matrix cores rounded to the
 * storage type.
 *
 *   workspace   optional device scratch, workspace_bytes long, 16-byte
 *               aligned, contents irrelevant.  With at least
 *               rope_flash_attn_workspace_size() bytes, a head-dim-128
 *               16-bit workload with fewer work items (query-row blocks of
 *               one head group) than the device has CUs has the key tiles
 *               of each item cut into segments, one workgroup each; a cut
 *               item's segments leave fp32 partial states (unnormalised
 *               output rows, reference max and sum) in the workspace, and a
 *               second kernel enqueued right after on the same stream
 *               merges them (each state rescaled to the larger max, as
 *               [RF] section 5 rescales earlier contributions when the
 *               running max rises).  Calls that share one workspace
 *               must not run concurrently.  NULL / too small: one
 *               workgroup per item (same result up to floating-point
 *               rounding order).  Head dim 64 and fp32 use no workspace.
 */
int rope_flash_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim,
                        int64_t q_pos_offset, int64_t k_pos_offset,
                        const float *cos_tab, const float *sin_tab, int64_t table_rows,
                        int rot_dim, int layout, int causal, float softmax_scale,
                        int dtype, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * rope_flash_attn_workspace_size -- bytes of workspace rope_flash_attn_fwd
 * can use for these shapes on the current device, whatever H_kv (0: it
 * would use none).
 * Returns minus a status code for arguments rope_flash_attn_fwd would reject
 * on shape grounds.  Makes no device allocation.
 */
int64_t rope_flash_attn_workspace_size(int B, int H, int64_t Sq, int64_t Sk, int head_dim,
                                       int64_t q_pos_offset, int64_t k_pos_offset, int causal,
                                       int dtype);

/*
 * rope_flash_attn_bwd -- gradients of rope_flash_attn_fwd: given q, k, v,
 * the forward's output o and row statistics lse, and the upstream gradient
 * dout, write dq, dk and dv ([RF] section 5: the backward recomputes the
 * probabilities from Q, K and the saved row normalisation instead of storing
 * them; section 8, item 4).  With Q' = R(q_pos) Q, K' = R(k_pos) K and
 * P = exp(scale Q' K'^T - lse) under the same mask as the forward:
 *   dv = P^T dout,  dS = P * (dout V^T - rowsum(dout * o)),
 *   dq = R(q_pos)^T (scale dS K'),  dk = R(k_pos)^T (scale dS^T Q'),
 * R^T being the rotation by the opposite angle; dk and dv of a key/value
 * head sum over the query heads that read it.  V is never rotated.
 *
 *   q, o, dout  [B, H, Sq, head_dim], contiguous; o and lse from
 *               rope_flash_attn_fwd with the same arguments.
 *   k, v        [B, H_kv, Sk, head_dim], contiguous (H_kv divides H).
 *   lse         fp32 [B, H, Sq], 4-byte aligned.
 *   dq          [B, H, Sq, head_dim], written whole.
 *   dk, dv      [B, H_kv, Sk, head_dim], written whole (keys no query
 *               sees get zeros).
 *   The three outputs must not alias each other or any input
 *   (ROPE_ERR_SHAPE).
 *   other arguments as rope_flash_attn_fwd; dtype ROPE_BF16 or ROPE_F16 (all
 *   tensors of that type), head_dim 64 or 128, rot_dim 0 or a multiple of 32
 *   (else ROPE_ERR_UNSUPPORTED).
 *   workspace   device scratch of at least rope_flash_attn_bwd_workspace_size()
 *               bytes, 16-byte aligned, contents irrelevant (per-row
 *               rowsum(dout * o); with rotation, also q rotated and scaled
 *               and k rotated, once, in the storage type).  Calls that share
 *               a workspace must not run concurrently.
 * Two kernels are enqueued on `stream`: the row sums (with rot_dim > 0 in
 * the same launch as the rotation of q and k into the workspace), then
 * dk/dv and dq in one launch.
 * Accumulation is fp32; the rotated Q/K, dout, V, P and dS enter the matrix
 * cores rounded to the storage type.
 */
int rope_flash_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                        const float *lse, void *dq, void *dk, void *dv,
                        int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim,
                        int64_t q_pos_offset, int64_t k_pos_offset,
                        const float *cos_tab, const float *sin_tab, int64_t table_rows,
                        int rot_dim, int layout, int causal, float softmax_scale, int dtype,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * rope_flash_attn_bwd_workspace_size -- bytes of workspace rope_flash_attn_bwd
 * needs for these shapes: B * H * Sq * 4 rounded up to a multiple of 256,
 * plus, when rot_dim > 0, B * H * Sq * head_dim * 2 and
 * B * H_kv * Sk * head_dim * 2, each rounded up to a multiple of 256.
 * Minus a status code for shapes or types it would reject (H_kv must divide
 * H, 0 <= rot_dim <= head_dim).  No HIP call.
 */
int64_t rope_flash_attn_bwd_workspace_size(int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim,
                                           int rot_dim, int dtype);

/*
 * rope_decode_attn_fwd -- one decode step over a key/value cache: rotate the
 * new query and key of each request at its cache position, append the
 * rotated key and the unrotated value to the cache, and attend over the
 * cache with the offset mask, never rotating a cached key again ([RF]
 * section 2 for this decoder flow, section 6 for the offset mask; [TR]
 * "Performance requirements" for doing the decode rotation inside the
 * attention launch).
 *
 * Request b's new token sits at position L = cache_lens[b], the number of
 * keys already cached: rows 0..L-1 of the cache hold keys rotated at their
 * positions (by earlier steps, or by rope_apply after a prefill).  The call
 * writes rope(k_new[b], L) to k_cache[b, :, L] and v_new[b] to
 * v_cache[b, :, L], and
 *   o[b, h] = softmax(scale * rope(q[b, h], L) . k_cache[b, h / (H/H_kv), 0..L])
 *             . v_cache[b, h / (H/H_kv), 0..L]
 * (all L + 1 keys are visible to the new query).
 *
 *   q, o        [B, H, head_dim], one new query per request; o is
 *               written whole and must not alias the other arrays.
 *   k_new,      [B, H_kv, head_dim]; H_kv divides H, H / H_kv <= 8.
 *   v_new
 *   k_cache,    [B, H_kv, S_max, head_dim], contiguous; written at row
 *   v_cache     L of each (b, head) only.
 *   cache_lens  device int32 [B].  A value outside [0, S_max), or (rot_dim >
 *               0) outside [0, table_rows), is detected on the device: that
 *               request's o rows are set to NaN and its cache is neither read
 *               nor written.
 *   cos_tab,    fp32 [table_rows, rot_dim/2] (see rope_tables_build).
 *   sin_tab
 *   rot_dim     0 (no rotation; tables may be NULL) or even, 2..head_dim.
 *   head_dim    64 or 128;  layout ROPE_NEOX or ROPE_GPTJ;  dtype ROPE_BF16
 *               or ROPE_F16 (q, k_new, v_new, caches and o all of it).
 *   softmax_scale  <= 0 selects 1/sqrt(head_dim).
 *   workspace   device scratch of at least rope_decode_workspace_size()
 *               bytes, 16-byte aligned, contents irrelevant: the fp32
 *               partial states of the pieces each (request, key/value head)
 *               is cut into (the cache passes are shared out evenly over a
 *               fixed set of workgroups) and a table of where they lie,
 *               merged by a second kernel enqueued right after on the same
 *               stream.  Calls that share a workspace must not run
 *               concurrently.
 * Shapes past 2^31 - 1 passes of 64 cached positions over all (request,
 * key/value head) pairs, i.e. B * H_kv * (S_max / 64 + 1), are rejected with
 * ROPE_ERR_SHAPE.
 * Requires 16-byte-aligned q, k_new, v_new, caches, o (else ROPE_ERR_ALIGN).
 */
int rope_decode_attn_fwd(const void *q, const void *k_new, const void *v_new,
                         void *k_cache, void *v_cache, const int32_t *cache_lens, void *o,
                         int B, int H, int H_kv, int64_t S_max, int head_dim,
                         const float *cos_tab, const float *sin_tab, int64_t table_rows,
                         int rot_dim, int layout, float softmax_scale, int dtype,
                         void *workspace, int64_t workspace_bytes, void *stream);

/*
 * rope_decode_workspace_size -- bytes of workspace rope_decode_attn_fwd needs
 * for these shapes, or minus a status code for shapes it would reject:
 * (B * H_kv + 1024) * (H / H_kv) * (head_dim + 2) * 4 rounded up to a
 * multiple of 256, plus B * H_kv * 8; the same on every device, independent
 * of S_max.  Makes no device allocation and no HIP call.
 */
int64_t rope_decode_workspace_size(int B, int H, int H_kv, int64_t S_max, int head_dim);

/*
 * Bytes of the library's static decode scratch: one array of this size in
 * each GPU's memory, held from the first rope_decode_attn_fwd_noalloc call on
 * that GPU until the process ends.
 */
#define ROPE_DECODE_SCRATCH_BYTES (8 << 20)

/*
 * rope_decode_attn_fwd_noalloc -- rope_decode_attn_fwd without a workspace
 * argument, for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  It allocates nothing (no hipMalloc, hipFree or allocating
 * library call); the partial states and the piece table live in a static
 * device array of ROPE_DECODE_SCRATCH_BYTES per GPU, whose address the
 * first call on a device looks up once (with that device current).
 *
 * Arguments, results and errors are those of rope_decode_attn_fwd, plus
 * ROPE_ERR_SCRATCH, returned before any HIP call, when
 * rope_decode_workspace_size() for the shapes exceeds
 * ROPE_DECODE_SCRATCH_BYTES (for head_dim 128, B * H_kv up to 2997 fits
 * with H / H_kv = 4, up to 990 with H / H_kv = 8).  ROPE_ERR_HIP if the
 * array's address cannot be obtained.
 * Nothing in the array needs clearing between calls: every byte a call
 * reads was written earlier in that call.  All calls on one GPU share the
 * array, so calls that may overlap in time on one GPU (different streams,
 * or host threads) race and must be serialised by the caller.
 */
int rope_decode_attn_fwd_noalloc(const void *q, const void *k_new, const void *v_new,
                                 void *k_cache, void *v_cache, const int32_t *cache_lens, void *o,
                                 int B, int H, int H_kv, int64_t S_max, int head_dim,
                                 const float *cos_tab, const float *sin_tab, int64_t table_rows,
                                 int rot_dim, int layout, float softmax_scale, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_MI355X_H */
