/*
 * rope_calib.h -- C ABI of librope_calib.so: measurement kernels that give
 * what plain kernels of the same shape of work reach on the GPU, so that
 * the library's measured rates can be read against an attainable ceiling
 * as well as against the published peaks.  Nothing here is on the RoPE
 * path; the benchmark and the tests are the only callers.
 *
 * Pages cited (by title and section):
 *   [RF] "RoPE and FlashAttention: relative positions and online softmax"
 *   [TR] "Write Triton Rope Kernel"
 *
 * Conventions: pointers are DEVICE pointers owned by the caller; `stream` is
 * a hipStream_t passed as void*; nothing is allocated and no call
 * synchronises.  Arguments are checked before any HIP call; on error nothing
 * is enqueued.
 */
#ifndef ROPE_CALIB_H
#define ROPE_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROPE_CALIB_OK 0
#define ROPE_CALIB_ERR_NULL 1    /* a required pointer is NULL */
#define ROPE_CALIB_ERR_SHAPE 2   /* a size, count or variant outside what the kernel takes */
#define ROPE_CALIB_ERR_HIP 7     /* the launch failed */

/*
 * rope_calib_stream_inplace -- in-place read-modify-write of n_vec 16-byte
 * vectors: each is loaded, 1 is added to each of its four 32-bit words, and
 * it is stored back (non-temporal loads and stores, one vector per thread).
 * Touched vector v sits at vector index (v / span_vecs) * row_vecs +
 * v % span_vecs of buf, so span_vecs == row_vecs streams a contiguous range
 * and span_vecs < row_vecs the first span_vecs vectors of each row -- the
 * access of an in-place RoPE over the rotated span of each head row ([TR]
 * "Performance requirements": one read and one write of the rotated span).
 *
 *   buf        16-byte aligned, at least ceil(n_vec / span_vecs) * row_vecs
 *              vectors (the caller guarantees the size)
 *   n_vec      > 0
 *   row_vecs, span_vecs   powers of two, span_vecs <= row_vecs <= 2^20
 * Moves 32 * n_vec bytes (read + write).
 */
int rope_calib_stream_inplace(void *buf, int64_t n_vec, int row_vecs, int span_vecs, void *stream);

/*
 * rope_calib_stream_read -- read n_vec 16-byte vectors of buf once
 * (non-temporal loads, one vector per thread), the traffic of a decode step
 * walking its key/value cache ([RF] section 7).  A vector whose four 32-bit
 * words all equal `key` writes its index to *hit (several such vectors: one
 * of their indices); *hit is left alone otherwise.  Reads 16 * n_vec bytes.
 *
 *   buf     16-byte aligned, n_vec vectors
 *   n_vec   > 0 (grid within 2^32 - 1 work-items)
 *   hit     one int64
 */
int rope_calib_stream_read(const void *buf, int64_t n_vec, uint32_t key, int64_t *hit, void *stream);

/*
 * rope_calib_attn_loop -- the inner step of a flash-attention forward with
 * nothing around it ([RF] section 5: scores, exponentials, row sums, P V),
 * repeated `iters` times by every wave on one K tile and one V tile held in
 * LDS: per wave and iteration S = K Q^T for 64 keys x 32 query rows on
 * v_mfma_f32_32x32x16_bf16, P = exp2(S) rounded to bf16, the row sums of the
 * rounded P (v_dot2_f32_bf16), a wave-level fast-path check (any row sum
 * above 8192 halves O), and O^T += V^T P^T on the matrix cores (V^T from
 * transposing LDS reads).  No global traffic, barrier or rotation in the
 * loop.  4 * 64 * 32 * head_dim flops per wave and iteration.
 *
 *   head_dim        64 (waves_per_simd 1..4) or 128 (waves_per_simd 1..2)
 *   waves_per_simd  workgroup of 256 * waves_per_simd threads, one per CU
 *                   (the kernel reserves 90 KB of LDS)
 *   pipelined       0: scores, probabilities, P V in order per iteration;
 *                   1: the next iteration's scores issued with this one's
 *                   exponentials (two score sets live)
 *   iters           > 0, even
 *   workgroups      > 0
 *   k_tile          bf16 [64][head_dim + 8] (row pitch head_dim + 8)
 *   v_tile          bf16 [64][head_dim]; 16-byte chunk c of row r is stored
 *                   at chunk c ^ 4((r >> 1) & 1) of that row
 *   q_rows          bf16 [128 * waves_per_simd][head_dim]: rows 32w .. 32w+31
 *                   are wave w's query rows
 *   out             fp32 [workgroups][256 * waves_per_simd][head_dim / 2 + 4]:
 *                   thread t's O^T accumulators (element r of 32-dim block b
 *                   is dim 32b + 8(r/4) + 4(lane/32) + r%4 of query row
 *                   lane%32 of its wave) then its 4 partial row sums (the
 *                   row's sum is the total over lanes l and l + 32)
 *   cycles          int64 [workgroups][4 * waves_per_simd] s_memtime ticks of
 *                   each wave's loop, or NULL
 */
int rope_calib_attn_loop(int head_dim, int waves_per_simd, int pipelined, int iters, int workgroups,
                         const void *k_tile, const void *v_tile, const void *q_rows, float *out,
                         int64_t *cycles, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_CALIB_H */
