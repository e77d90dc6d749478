// flash_fwd_f32.hip -- fused RoPE + softmax attention forward for fp32
// inputs, on the vector ALUs.
//
// Same operation and recurrence as the bf16 matrix-core kernel (see
// flash_fwd_bf16.hip): Q and each staged K tile rotated at their absolute
// positions, online softmax over key tiles ("RoPE and FlashAttention:
// relative positions and online softmax", section 5), offset-causal mask
// (section 6), output normalised once at the end.  fp32 inputs keep fp32
// products here (no bf16 rounding), so the result stays within fp32
// rounding of the exact forward.
//
// Layout: a 256-thread block owns 64 query rows; four adjacent lanes share a
// row, each holding a quarter of the head dims; a score is a 4-lane
// reduction.  K/V tiles of 32 keys are staged, rotated, in LDS.
#include "common.hpp"

namespace {

constexpr int BM = 64;
constexpr int BN = 32;

struct F32Params {
    const float *q, *k, *v;
    float *o;
    float *lse;     // [BH, Sq] natural-log log-sum-exp of each row's scores, or null
    int BH;
    int kv_group;   // query heads per key/value head: K/V head of bh is bh / kv_group
    int64_t Sq, Sk, q_off, k_off;
    const float *cos_tab, *sin_tab;
    int rot_dim;
    float sl2;      // softmax scale * log2(e)
    int causal;
    int n_qtiles;
};

// Rotate the rot_dim leading dims of `rows` rows held in LDS (pitch D) in
// place.  Row r sits at position pos0 + r.  Each pair is owned by one thread.
template <int D, int LAYOUT>
__device__ void rotate_rows_lds(float *buf, int rows, int64_t pos0, int64_t valid_rows,
                                const float *cos_tab, const float *sin_tab, int rot_dim)
{
    const int half = rot_dim / 2;
    const int pairs = rows * half;
    for (int e = threadIdx.x; e < pairs; e += blockDim.x) {
        const int r = e / half, i = e % half;
        if (r >= valid_rows) continue;
        const int64_t pos = pos0 + r;
        const float c = cos_tab[pos * half + i], s = sin_tab[pos * half + i];
        const int a = LAYOUT == 1 ? 2 * i : i;
        const int b = LAYOUT == 1 ? 2 * i + 1 : i + half;
        const float xa = buf[r * D + a], xb = buf[r * D + b];
        buf[r * D + a] = xa * c - xb * s;
        buf[r * D + b] = xa * s + xb * c;
    }
}

template <int D, int LAYOUT, bool ROT>
__global__ __launch_bounds__(256) void flash_fwd_f32_kernel(F32Params p)
{
    constexpr int DP = D / 4;   // dims per lane
    __shared__ float Qs[BM * D];
    __shared__ float Ks[BN * D];
    __shared__ float Vs[BN * D];

    const int tid = threadIdx.x;
    const int row = tid / 4, part = tid % 4;
    const int bh = blockIdx.x % p.BH;
    const int rank = blockIdx.x / p.BH;
    const int qtile = p.causal ? p.n_qtiles - 1 - rank : rank;
    const int64_t q0 = (int64_t)qtile * BM;
    const float *qh = p.q + (int64_t)bh * p.Sq * D;
    const float *kh = p.k + (int64_t)(bh / p.kv_group) * p.Sk * D;
    const float *vh = p.v + (int64_t)(bh / p.kv_group) * p.Sk * D;
    const int64_t q_valid = p.Sq - q0 < BM ? p.Sq - q0 : BM;

    // Q tile: copy, rotate in LDS, take this lane's slice.
    for (int e = tid; e < BM * D; e += 256) {
        const int r = e / D;
        Qs[e] = r < q_valid ? qh[(q0 + r) * D + e % D] : 0.f;
    }
    __syncthreads();
    if constexpr (ROT) {
        rotate_rows_lds<D, LAYOUT>(Qs, BM, p.q_off + q0, q_valid, p.cos_tab, p.sin_tab, p.rot_dim);
        __syncthreads();
    }
    float qv[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) qv[d] = Qs[row * D + part * DP + d];

    const int64_t qi = q0 + row;
    const int64_t n_kt = (p.Sk + BN - 1) / BN;
    int64_t kt_end = n_kt;
    if (p.causal) {
        const int64_t jmax = p.q_off + q0 + q_valid - 1 - p.k_off;
        kt_end = jmax / BN + 1 < n_kt ? jmax / BN + 1 : n_kt;
    }

    float m_run = -INFINITY, l_run = 0.f;
    float acc[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = 0.f;

    for (int64_t kt = 0; kt < kt_end; ++kt) {
        const int64_t j0 = kt * BN;
        const int64_t k_valid = p.Sk - j0 < BN ? p.Sk - j0 : BN;
        __syncthreads();   // previous tile fully consumed
        for (int e = tid; e < BN * D; e += 256) {
            const int r = e / D;
            const bool ok = r < k_valid;
            Ks[e] = ok ? kh[(j0 + r) * D + e % D] : 0.f;
            Vs[e] = ok ? vh[(j0 + r) * D + e % D] : 0.f;
        }
        __syncthreads();
        if constexpr (ROT) {
            rotate_rows_lds<D, LAYOUT>(Ks, BN, p.k_off + j0, k_valid, p.cos_tab, p.sin_tab, p.rot_dim);
            __syncthreads();
        }
        float s[BN];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float part_dot = 0.f;
#pragma unroll
            for (int d = 0; d < DP; ++d) part_dot += qv[d] * Ks[j * D + part * DP + d];
            part_dot += __shfl_xor(part_dot, 1);
            part_dot += __shfl_xor(part_dot, 2);
            const int64_t jg = j0 + j;
            const bool ok = j < k_valid && (!p.causal || p.k_off + jg <= p.q_off + qi);
            s[j] = ok ? part_dot * p.sl2 : -INFINITY;
            mt = fmaxf(mt, s[j]);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int d = 0; d < DP; ++d) acc[d] *= alpha;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            const float pj = __builtin_amdgcn_exp2f(s[j] - m_use);
            lsum += pj;
#pragma unroll
            for (int d = 0; d < DP; ++d) acc[d] += pj * Vs[j * D + part * DP + d];
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
    }

    if (qi < p.Sq) {
        const float inv = 1.f / l_run;
        float *orow = p.o + ((int64_t)bh * p.Sq + qi) * D + part * DP;
#pragma unroll
        for (int d = 0; d < DP; ++d) orow[d] = acc[d] * inv;
        if (p.lse && part == 0) p.lse[(int64_t)bh * p.Sq + qi] = (m_run + log2f(l_run)) * 0.6931471805599453f;
    }
}

template <int D, int LAYOUT, bool ROT>
int launch(const FlashArgs &a, hipStream_t stream)
{
    F32Params p;
    p.q = static_cast<const float *>(a.q);
    p.k = static_cast<const float *>(a.k);
    p.v = static_cast<const float *>(a.v);
    p.o = static_cast<float *>(a.o);
    p.lse = a.lse;
    p.BH = a.B * a.H;
    p.kv_group = a.H / a.H_kv;
    p.Sq = a.Sq; p.Sk = a.Sk; p.q_off = a.q_off; p.k_off = a.k_off;
    p.cos_tab = a.cos_tab; p.sin_tab = a.sin_tab; p.rot_dim = a.rot_dim;
    p.sl2 = a.scale * 1.4426950408889634f;
    p.causal = a.causal;
    p.n_qtiles = (int)((a.Sq + BM - 1) / BM);
    const int64_t blocks = (int64_t)p.BH * p.n_qtiles;
    if (!rope_grid_fits(blocks, 256)) return ROPE_LAUNCH_SHAPE;
    hipLaunchKernelGGL((flash_fwd_f32_kernel<D, LAYOUT, ROT>), dim3((unsigned)blocks), dim3(256),
                       0, stream, p);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

}  // namespace

int rope_launch_flash_f32(const FlashArgs &a, hipStream_t stream)
{
    const bool rot = a.rot_dim > 0;
    if (a.head_dim == 64) {
        if (!rot) return launch<64, 0, false>(a, stream);
        return a.layout == 0 ? launch<64, 0, true>(a, stream) : launch<64, 1, true>(a, stream);
    }
    if (!rot) return launch<128, 0, false>(a, stream);
    return a.layout == 0 ? launch<128, 0, true>(a, stream) : launch<128, 1, true>(a, stream);
}
