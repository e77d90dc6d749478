// calib.hip -- measurement kernels for reading the library's rates against
// what plain kernels of the same shape of work reach on this GPU.  Nothing
// here is on the RoPE path; bench.py times these beside the real kernels.
//
//  * stream_inplace_kernel: an in-place read-modify-write stream of 16-byte
//    vectors (non-temporal loads and stores, one vector per thread), either
//    contiguous or touching the first `span` vectors of every `row` -- the
//    access pattern of an in-place RoPE that rotates part of each head row
//    ("Write Triton Rope Kernel", "Performance requirements": the op is a
//    pure stream of the rotated span, read once and written once).
//  * stream_read_kernel: a read-only stream of 16-byte vectors (non-temporal
//    loads, one vector per thread), the access of a decode step walking its
//    key/value cache once ("RoPE and FlashAttention", section 7: decoding
//    reads the cached keys and values);
//  * attn_loop_kernel: the inner step of a flash-attention forward with
//    nothing around it ("RoPE and FlashAttention", section 5: scores, the
//    exponentials against a reference, row sums, the P V update), on one K
//    tile and one V tile held in LDS for the whole run, with no global
//    traffic, no barriers and no rotation: per wave and iteration, S = K Q^T
//    for 64 keys x 32 queries on the matrix cores, P = exp2(S) rounded to
//    bf16 with its row sums (v_dot2_f32_bf16), the wave-level check a
//    softmax fast path needs, and O^T += V^T P^T on the matrix cores.  Its
//    rate bounds any kernel that runs this step per (query, key tile) on
//    this GPU, whatever it does around it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rope_calib.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------------------
// In-place stream.  Vector v of the touched set sits at vector
// (v >> span_log2) << row_log2 | (v & (span - 1)) of the buffer.
__global__ __launch_bounds__(256) void stream_inplace_kernel(u32x4 *buf, int64_t n_vec, int row_log2,
                                                             int span_log2)
{
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= n_vec) return;
    const int64_t at = ((v >> span_log2) << row_log2) | (v & ((1 << span_log2) - 1));
    u32x4 x = __builtin_nontemporal_load(buf + at);
    x += 1u;
    __builtin_nontemporal_store(x, buf + at);
}

// Read-only stream: each thread loads one vector; a vector equal to `key`
// (all four words) writes its index to *hit, so the loads cannot be dropped
// and a test can find a planted vector.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, int64_t n_vec, uint32_t key,
                                                          int64_t *hit)
{
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= n_vec) return;
    const u32x4 x = __builtin_nontemporal_load(buf + v);
    if (x.x == key && x.y == key && x.z == key && x.w == key) *hit = v;
}

// ---------------------------------------------------------------------------
// Attention inner step.  D: head dim (64 or 128); NT = 256 x waves per SIMD;
// PIPE: the scores of the next iteration are issued before this
// iteration's exponentials (two score sets live), interleaved one matrix
// instruction per nine vector instructions; otherwise each iteration runs
// scores, probabilities, P V in order and the other waves of the SIMD fill
// the gaps.
constexpr int BN = 64;                        // keys per tile
constexpr int LDS_BYTES = 92160;              // > 80 KB: one workgroup per CU
constexpr float FAST_LIMIT = 8192.0f;         // row-sum bound of a softmax fast path

__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
}

template <int D, int NT, int WPE, bool PIPE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))
void attn_loop_kernel(const uint16_t *k_tile, const uint16_t *v_tile, const uint16_t *q_rows, float *out,
                      long long *cycles, int iters)
{
    constexpr int KP = D + 8;                 // K row pitch in LDS (bf16)
    constexpr int KE = BN * KP, VE = BN * D;
    constexpr int DT = D / 16, DB = D / 32;   // k-steps of S; 32-dim blocks of O^T
    constexpr int NO = 16 * DB + 4;           // floats written per thread
    static_assert(2 * (KE + VE) <= LDS_BYTES, "tiles fit the LDS block");
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_BYTES / 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    for (int i = tid; i < KE + VE; i += NT) lds[i] = i < KE ? k_tile[i] : v_tile[i - KE];
    __syncthreads();
    const uint16_t *kl = lds, *vl = lds + KE;

    // Q rows of this wave as the B operand of S = K Q^T: lane (l32, hh)
    // holds row l32, dims 16t + 8hh .. +7
    bf16x8 qf[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
        qf[t] = *reinterpret_cast<const bf16x8 *>(q_rows + (wave * 32 + l32) * D + 16 * t + 8 * hh);
    // V^T operand from transposing reads of the row-major V tile: in each
    // 16-lane group, source lane 4j + b points at V[key0 + j][dim0 + 4b]
    const int g16 = lane >> 4, lp = lane & 15;
    const int tr_row = lp >> 2, tr_col = 4 * (lp & 3) + 16 * (g16 & 1);
    const int tr_key = 4 * (g16 >> 1) + tr_row;

    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = (f32x16){};
    float l[4] = {0.f, 0.f, 0.f, 0.f};

    auto scores = [&](f32x16 (&s)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = (f32x16){};
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kl + (kb * 32 + l32) * KP + 16 * t + 8 * hh);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
            }
        }
    };
    // accumulator element 8mm + s of key block kb <-> slot s of P operand (kb, mm)
    auto probs = [&](const f32x16 (&s)[2], bf16x8 (&pb)[2][2], float (&lt)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) lt[u] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                uint32_t w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    w[u] = pack_bf16(__builtin_amdgcn_exp2f(s[kb][8 * mm + 2 * u]),
                                     __builtin_amdgcn_exp2f(s[kb][8 * mm + 2 * u + 1]));
#pragma unroll
                for (int u = 0; u < 4; ++u) lt[u] = sum_bf16x2(w[u], lt[u]);
                pb[kb][mm] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            }
    };
    auto check = [&](const float (&lt)[4]) {
        const float lmax = fmaxf(fmaxf(lt[0], lt[1]), fmaxf(lt[2], lt[3]));
        asm volatile("" ::"v"(lmax));
        if (__builtin_amdgcn_ballot_w64(!(lmax <= FAST_LIMIT)) != 0) {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][r] *= 0.5f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) l[u] += lt[u];
    };
    auto pv = [&](const bf16x8 (&pb)[2][2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int bd = 0; bd < DB; ++bd) {
                    // rows of the V tile are unpadded; chunk c of row r sits at c ^ 4((r >> 1) & 1)
                    const int col = 8 * ((4 * bd + (tr_col >> 3)) ^ (4 * ((tr_row >> 1) & 1))) + (tr_col & 7);
                    const uint16_t *src = vl + (32 * kb + 16 * mm + tr_key) * D + col;
                    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
                    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + 8 * D));
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, (short __attribute__((ext_vector_type(8)))){x0[0], x0[1], x0[2], x0[3], x1[0],
                                                                            x1[1], x1[2], x1[3]});
                    o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][mm], o[bd], 0, 0, 0);
                }
    };

    __syncthreads();
    const long long t0 = __builtin_amdgcn_s_memtime();
    if constexpr (!PIPE) {
        for (int it = 0; it < iters; ++it) {
            f32x16 s[2];
            bf16x8 pb[2][2];
            float lt[4];
            scores(s);
            probs(s, pb, lt);
            check(lt);
            pv(pb);
        }
    } else {
        f32x16 sa[2], sb[2];
        scores(sa);
        auto step = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
            bf16x8 pb[2][2];
            float lt[4];
            scores(nxt);
            probs(cur, pb, lt);
#pragma unroll
            for (int i = 0; i < 2 * DT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 72 / (2 * DT) + 1, 0);   // vector ALU
            }
            check(lt);
            pv(pb);
        };
        for (int it = 0; it < iters; it += 2) {   // iters is even
            step(sa, sb);
            step(sb, sa);
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();

    float *dst = out + ((int64_t)blockIdx.x * NT + tid) * NO;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[16 * b + r] = o[b][r];
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[16 * DB + u] = l[u];
    if (cycles && lane == 0) cycles[(int64_t)blockIdx.x * (NT / 64) + wave] = t1 - t0;
}

template <int D, int WPE, bool PIPE>
int launch_loop(int iters, int workgroups, const void *k, const void *v, const void *q, float *out,
                int64_t *cycles, hipStream_t stream)
{
    constexpr int NT = 256 * WPE;
    hipLaunchKernelGGL((attn_loop_kernel<D, NT, WPE, PIPE>), dim3(workgroups), dim3(NT), 0, stream,
                       static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                       static_cast<const uint16_t *>(q), out, reinterpret_cast<long long *>(cycles), iters);
    return hipGetLastError() == hipSuccess ? ROPE_CALIB_OK : ROPE_CALIB_ERR_HIP;
}

template <int D, int WPE>
int launch_pipe(int pipelined, int iters, int workgroups, const void *k, const void *v, const void *q,
                float *out, int64_t *cycles, hipStream_t stream)
{
    return pipelined ? launch_loop<D, WPE, true>(iters, workgroups, k, v, q, out, cycles, stream)
                     : launch_loop<D, WPE, false>(iters, workgroups, k, v, q, out, cycles, stream);
}

int log2_exact(int x)
{
    int n = 0;
    while ((1 << n) < x) ++n;
    return (1 << n) == x ? n : -1;
}

}  // namespace

extern "C" int rope_calib_stream_inplace(void *buf, int64_t n_vec, int row_vecs, int span_vecs, void *stream)
{
    if (!buf) return ROPE_CALIB_ERR_NULL;
    const int rl = log2_exact(row_vecs), sl = log2_exact(span_vecs);
    if (n_vec <= 0 || rl < 0 || sl < 0 || span_vecs > row_vecs || rl > 20) return ROPE_CALIB_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return ROPE_CALIB_ERR_SHAPE;
    const int64_t blocks = (n_vec + 255) / 256;
    if (blocks > 0xffffffffLL / 256) return ROPE_CALIB_ERR_SHAPE;
    hipLaunchKernelGGL(stream_inplace_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4 *>(buf), n_vec, rl, sl);
    return hipGetLastError() == hipSuccess ? ROPE_CALIB_OK : ROPE_CALIB_ERR_HIP;
}

extern "C" int rope_calib_stream_read(const void *buf, int64_t n_vec, uint32_t key, int64_t *hit,
                                     void *stream)
{
    if (!buf || !hit) return ROPE_CALIB_ERR_NULL;
    if (n_vec <= 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return ROPE_CALIB_ERR_SHAPE;
    const int64_t blocks = (n_vec + 255) / 256;
    if (blocks > 0xffffffffLL / 256) return ROPE_CALIB_ERR_SHAPE;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf), n_vec, key, hit);
    return hipGetLastError() == hipSuccess ? ROPE_CALIB_OK : ROPE_CALIB_ERR_HIP;
}

extern "C" int rope_calib_attn_loop(int head_dim, int waves_per_simd, int pipelined, int iters, int workgroups,
                                    const void *k_tile, const void *v_tile, const void *q_rows, float *out,
                                    int64_t *cycles, void *stream)
{
    if (!k_tile || !v_tile || !q_rows || !out) return ROPE_CALIB_ERR_NULL;
    if (iters <= 0 || iters % 2 != 0 || workgroups <= 0) return ROPE_CALIB_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (head_dim == 64) {
        switch (waves_per_simd) {
        case 1: return launch_pipe<64, 1>(pipelined, iters, workgroups, k_tile, v_tile, q_rows, out, cycles, s);
        case 2: return launch_pipe<64, 2>(pipelined, iters, workgroups, k_tile, v_tile, q_rows, out, cycles, s);
        case 3: return launch_pipe<64, 3>(pipelined, iters, workgroups, k_tile, v_tile, q_rows, out, cycles, s);
        case 4: return launch_pipe<64, 4>(pipelined, iters, workgroups, k_tile, v_tile, q_rows, out, cycles, s);
        default: return ROPE_CALIB_ERR_SHAPE;
        }
    }
    if (head_dim == 128) {
        switch (waves_per_simd) {
        case 1: return launch_pipe<128, 1>(pipelined, iters, workgroups, k_tile, v_tile, q_rows, out, cycles, s);
        case 2: return launch_pipe<128, 2>(pipelined, iters, workgroups, k_tile, v_tile, q_rows, out, cycles, s);
        default: return ROPE_CALIB_ERR_SHAPE;
        }
    }
    return ROPE_CALIB_ERR_SHAPE;
}
