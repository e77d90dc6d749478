// decode_bf16.hip -- one decode step over a key/value cache, bf16, gfx950.
//
// For each request b the new token sits at position L = lens[b] (the number
// of keys already cached).  Inside a decoder the step rotates the new query
// and key at that position, appends the rotated key and the unrotated value to
// the cache, and attends over the cache with the offset mask, never rotating
// a cached key again ("RoPE and FlashAttention: relative positions and online
// softmax", section 2 for the decoder flow, section 6 for the offset mask; the
// Triton RoPE skill page, "Performance requirements", for doing the decode
// rotation inside the attention launch).
//
// The work is bound by reading the cache once, so the kernel is laid out for
// HBM streaming rather than for the matrix cores: a workgroup takes one
// request, one key/value head and a contiguous range of CW cached positions
// for all G query heads that share the key/value head, reads each 16-byte
// chunk of K and V once with coalesced buffer loads, and forms scores and
// P V on the vector ALU in fp32.  Ranges of one (request, key/value head) are
// combined by a second kernel (running max and sum rescaling, the merge rule
// of section 5 of the same page).
#include "common.hpp"

namespace {

using rope::bf16_to_f32;
using rope::f32_to_bf16;

constexpr int SUB = 128;          // keys per pass of the workgroup
constexpr int NSUB = 4;           // passes per workgroup
constexpr int CW = SUB * NSUB;    // cached positions per workgroup
constexpr int GMAX = 8;           // query heads per key/value head, at most

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_FLAGS = 0x00020000;   // untyped 32-bit buffer (gfx9 family)

struct DecodeParams {
    const uint16_t *q;          // [B, H, D]       new queries, unrotated
    const uint16_t *k_new;      // [B, Hkv, D]     new keys, unrotated
    const uint16_t *v_new;      // [B, Hkv, D]
    uint16_t *k_cache;          // [B, Hkv, S_max, D], rows < L rotated
    uint16_t *v_cache;          // [B, Hkv, S_max, D]
    const int32_t *lens;        // [B]
    const float *cos_tab, *sin_tab;   // [table_rows, rot_dim / 2]
    float *part;                // [B * H][n_chunks][D + 2]: m, l, O (unnormalised)
    uint16_t *o;                // [B, H, D]
    int64_t table_rows, S_max;
    int B, H, Hkv, G, rot_dim, n_chunks;
    float sl2;                  // softmax scale * log2(e)
};

// A buffer resource over `rows` rows of ROW_BYTES from base: loads past them
// (and with rows <= 0, all loads) return zeros and touch no memory.
template <int ROW_BYTES>
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int rows)
{
    const uint32_t n = rows <= 0 ? 0u : (uint32_t)rows * ROW_BYTES;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, RSRC_FLAGS);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// The two dims of rotation pair i (i < rot_dim / 2): NeoX pairs dim i with
// i + rot_dim/2, GPT-J pairs 2i with 2i + 1; pair indices past rot_dim/2
// stand for the untouched dims rot_dim + 2(i - rot_dim/2) and the next one.
template <int LAYOUT>
__device__ __forceinline__ void pair_dims(int i, int rot_dim, int &a, int &b)
{
    const int rh = rot_dim / 2;
    if (i >= rh) {
        a = rot_dim + 2 * (i - rh);
        b = a + 1;
    } else if (LAYOUT == 0) {
        a = i;
        b = i + rh;
    } else {
        a = 2 * i;
        b = 2 * i + 1;
    }
}

// Sum over groups of W consecutive lanes (W a power of two up to 64): every
// lane of a group ends with the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1) x += __shfl_xor(x, m);
    return x;
}
template <int W>
__device__ __forceinline__ float group_max(float x)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// One workgroup: request b, key/value head kvh, cached positions
// [c CW, (c + 1) CW) of the L + 1 keys the new query sees (the last one is the
// new key, taken from LDS and, by the workgroup whose range holds it,
// appended to the cache).  GT: G rounded up to a power of two.
template <int D, int LAYOUT, bool ROT, int GT>
__global__ __launch_bounds__(256) void decode_chunk_kernel(DecodeParams p)
{
    constexpr int LPR = D / 8;          // lanes per key row (16 bytes each)
    constexpr int KPI = 64 / LPR;       // keys per wave load
    constexpr int KPW = SUB / 4;        // keys per wave and pass
    constexpr int NI = KPW / KPI;       // loads per wave and pass, for K and for V
    static_assert(GT <= LPR && GT <= GMAX, "a lane of each row group writes one query's score");

    __shared__ __attribute__((aligned(16))) float q_lds[GT][D];    // rotated, scaled queries
    __shared__ float s_lds[GT][SUB];                               // scores, then probabilities
    __shared__ __attribute__((aligned(16))) uint16_t knew_lds[D];  // new key, rotated, bf16
    __shared__ __attribute__((aligned(16))) uint16_t vnew_lds[D];
    __shared__ float m_run[GT], l_run[GT], alpha_lds[GT];
    __shared__ __attribute__((aligned(16))) float o_lds[4][GT][D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x % p.n_chunks;
    const int bk = blockIdx.x / p.n_chunks;   // b * Hkv + kvh
    const int b = bk / p.Hkv, kvh = bk % p.Hkv;
    const int G = p.G;
    const int L = p.lens[b];
    // a length outside the cache (or the table) leaves the request to the
    // merge kernel, which writes NaN rows; nothing is read or written here
    if (L < 0 || (int64_t)L >= p.S_max || (ROT && (int64_t)L >= p.table_rows)) return;
    const int n = L + 1;                      // visible keys, the new one included
    const int k0 = c * CW;
    if (k0 >= n) return;

    // ---- the new query rows and key at position L ----
    const int rh = p.rot_dim / 2;
    const float *crow = ROT ? p.cos_tab + (int64_t)L * rh : nullptr;
    const float *srow = ROT ? p.sin_tab + (int64_t)L * rh : nullptr;
    for (int idx = tid; idx < G * (D / 2); idx += 256) {
        const int g = idx / (D / 2), i = idx % (D / 2);
        int da, db;
        pair_dims<LAYOUT>(i, ROT ? p.rot_dim : 0, da, db);
        const uint16_t *qr = p.q + ((int64_t)b * p.H + kvh * G + g) * D;
        const float xa = bf16_to_f32(qr[da]), xb = bf16_to_f32(qr[db]);
        float ya = xa, yb = xb;
        if (ROT && i < rh) {
            const float cs = crow[i], sn = srow[i];
            ya = xa * cs - xb * sn;
            yb = xa * sn + xb * cs;
        }
        q_lds[g][da] = ya * p.sl2;
        q_lds[g][db] = yb * p.sl2;
    }
    const bool last = n - k0 <= CW;           // this range holds position L
    if (last) {
        const int64_t crow_off = ((int64_t)bk * p.S_max + L) * D;
        for (int i = tid; i < D / 2; i += 256) {
            int da, db;
            pair_dims<LAYOUT>(i, ROT ? p.rot_dim : 0, da, db);
            const uint16_t *kr = p.k_new + (int64_t)bk * D;
            const float xa = bf16_to_f32(kr[da]), xb = bf16_to_f32(kr[db]);
            float ya = xa, yb = xb;
            if (ROT && i < rh) {
                const float cs = crow[i], sn = srow[i];
                ya = xa * cs - xb * sn;
                yb = xa * sn + xb * cs;
            }
            const uint16_t ba = f32_to_bf16(ya), bb = f32_to_bf16(yb);
            knew_lds[da] = ba;
            knew_lds[db] = bb;
            p.k_cache[crow_off + da] = ba;
            p.k_cache[crow_off + db] = bb;
        }
        for (int d = tid; d < D; d += 256) {
            const uint16_t v = p.v_new[(int64_t)bk * D + d];
            vnew_lds[d] = v;
            p.v_cache[crow_off + d] = v;
        }
    }
    if (tid < GT) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.f;
    }
    __syncthreads();

    const int sub = lane % LPR;               // 16-byte chunk of the row this lane reads
    float oacc[GT][8];
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[g][e] = 0.f;

    const int64_t slice = (int64_t)bk * p.S_max;   // row of (b, kvh, position 0)
    for (int s = 0; s < NSUB; ++s) {
        const int ks = k0 + s * SUB;
        if (ks >= n) break;
        // cached rows [ks, min(L, ks + SUB)); the row at L reads as zero here
        const int rows = L - ks < SUB ? L - ks : SUB;
        const rsrc_t krs = make_rsrc<2 * D>(p.k_cache + (slice + ks) * D, rows);
        const rsrc_t vrs = make_rsrc<2 * D>(p.v_cache + (slice + ks) * D, rows);
        uint4 kd[NI], vd[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = wave * KPW + i * KPI + lane / LPR;
            kd[i] = bload16(krs, 2 * (key * D + 8 * sub));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = wave * KPW + i * KPI + lane / LPR;
            vd[i] = bload16(vrs, 2 * (key * D + 8 * sub));
        }
        // scores of the wave's keys, one per lane group
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = wave * KPW + i * KPI + lane / LPR;
            const int pos = ks + key;
            uint4 w = kd[i];
            if (pos == L) w = *reinterpret_cast<const uint4 *>(knew_lds + 8 * sub);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = rope::bf16lo_to_f32(u[e]);
                kf[2 * e + 1] = rope::bf16hi_to_f32(u[e]);
            }
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float4 qa = *reinterpret_cast<const float4 *>(&q_lds[g][8 * sub]);
                const float4 qb = *reinterpret_cast<const float4 *>(&q_lds[g][8 * sub + 4]);
                float acc = qa.x * kf[0];
                acc = fmaf(qa.y, kf[1], acc);
                acc = fmaf(qa.z, kf[2], acc);
                acc = fmaf(qa.w, kf[3], acc);
                acc = fmaf(qb.x, kf[4], acc);
                acc = fmaf(qb.y, kf[5], acc);
                acc = fmaf(qb.z, kf[6], acc);
                acc = fmaf(qb.w, kf[7], acc);
                acc = group_sum<LPR>(acc);
                if (sub == g && g < G) s_lds[g][key] = pos < n ? acc : -INFINITY;
            }
        }
        __syncthreads();
        // running max and sum per query: wave w takes queries w and w + 4
#pragma unroll
        for (int gg = 0; gg < (GT + 3) / 4; ++gg) {
            const int g = wave + 4 * gg;
            if (g < G) {
                const float s0 = s_lds[g][lane], s1 = s_lds[g][lane + 64];
                const float cmax = group_max<64>(fmaxf(s0, s1));
                const float m_old = m_run[g];
                const float m_new = fmaxf(m_old, cmax);   // finite: the pass has a visible key
                const float p0 = __builtin_amdgcn_exp2f(s0 - m_new), p1 = __builtin_amdgcn_exp2f(s1 - m_new);
                s_lds[g][lane] = p0;
                s_lds[g][lane + 64] = p1;
                const float psum = group_sum<64>(p0 + p1);
                if (lane == 0) {
                    const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);   // 0 on the first pass
                    alpha_lds[g] = alpha;
                    l_run[g] = l_run[g] * alpha + psum;
                    m_run[g] = m_new;
                }
            }
        }
        __syncthreads();
        // O += P V for the wave's keys, after rescaling to the new maxima
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float a = g < G ? alpha_lds[g] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[g][e] *= a;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = wave * KPW + i * KPI + lane / LPR;
            const int pos = ks + key;
            uint4 w = vd[i];
            if (pos == L) w = *reinterpret_cast<const uint4 *>(vnew_lds + 8 * sub);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
            float vf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[2 * e] = rope::bf16lo_to_f32(u[e]);
                vf[2 * e + 1] = rope::bf16hi_to_f32(u[e]);
            }
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float pg = g < G ? s_lds[g][key] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[g][e] = fmaf(pg, vf[e], oacc[g][e]);
            }
        }
        __syncthreads();   // s_lds is rewritten by the next pass
    }

    // ---- the range's partial state: O summed over lane groups and waves ----
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = oacc[g][e];
#pragma unroll
            for (int m = LPR; m < 64; m <<= 1) x += __shfl_xor(x, m);
            oacc[g][e] = x;
        }
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float4 *dst = reinterpret_cast<float4 *>(&o_lds[wave][g][8 * lane]);
            dst[0] = make_float4(oacc[g][0], oacc[g][1], oacc[g][2], oacc[g][3]);
            dst[1] = make_float4(oacc[g][4], oacc[g][5], oacc[g][6], oacc[g][7]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        const float v = (o_lds[0][g][d] + o_lds[1][g][d]) + (o_lds[2][g][d] + o_lds[3][g][d]);
        float *dst = p.part + (((int64_t)b * p.H + kvh * G + g) * p.n_chunks + c) * (D + 2);
        dst[2 + d] = v;
        if (d == 0) {
            dst[0] = m_run[g];
            dst[1] = l_run[g];
        }
    }
}

// Output row (b, h): the ranges' partial states merged (maxima aligned, sums
// and rows rescaled), O / l rounded to bf16.  A request whose length lies
// outside the cache or the table gets a row of NaN.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int rot)
{
    constexpr int CL = 256 / D;   // ranges summed in parallel per dim
    __shared__ float red[256];
    __shared__ float mx;
    const int bh = blockIdx.x, b = bh / p.H, tid = threadIdx.x;
    const int L = p.lens[b];
    uint16_t *orow = p.o + (int64_t)bh * D;
    if (L < 0 || (int64_t)L >= p.S_max || (rot > 0 && (int64_t)L >= p.table_rows)) {
        for (int d = tid; d < D; d += 256) orow[d] = 0x7fc0;   // bf16 quiet NaN
        return;
    }
    const int nc = (L + 1 + CW - 1) / CW;
    const float *part = p.part + (int64_t)bh * p.n_chunks * (D + 2);
    // largest range maximum
    float m = -INFINITY;
    for (int c = tid; c < nc; c += 256) m = fmaxf(m, part[(int64_t)c * (D + 2)]);
    red[tid] = m;
    __syncthreads();
    if (tid < 64) {
        float x = fmaxf(fmaxf(red[tid], red[tid + 64]), fmaxf(red[tid + 128], red[tid + 192]));
        x = group_max<64>(x);
        if (tid == 0) mx = x;
    }
    __syncthreads();
    const float M = mx;
    // thread (d, j) sums dim d over ranges j, j + CL, ...; the sums l ride along
    const int d = tid % D, j = tid / D;
    float acc = 0.f, lsum = 0.f;
    for (int c = j; c < nc; c += CL) {
        const float *pc = part + (int64_t)c * (D + 2);
        const float w = __builtin_amdgcn_exp2f(pc[0] - M);
        acc = fmaf(pc[2 + d], w, acc);
        lsum = fmaf(pc[1], w, lsum);
    }
    __syncthreads();
    red[tid] = acc;
    __syncthreads();
    if (j == 0) {
        float o = 0.f;
#pragma unroll
        for (int jj = 0; jj < CL; ++jj) o += red[jj * D + d];
        acc = o;
    }
    __syncthreads();
    red[tid] = lsum;   // the same l sum in every dim lane of range group j
    __syncthreads();
    if (j == 0) {
        float l = 0.f;
#pragma unroll
        for (int jj = 0; jj < CL; ++jj) l += red[jj * D];
        orow[d] = f32_to_bf16(acc / l);
    }
}

template <int D, int LAYOUT, bool ROT>
int launch_gt(const DecodeParams &p, unsigned grid, hipStream_t stream)
{
    if (p.G <= 1)
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 1>), dim3(grid), dim3(256), 0, stream, p);
    else if (p.G <= 2)
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 2>), dim3(grid), dim3(256), 0, stream, p);
    else if (p.G <= 4)
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 4>), dim3(grid), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 8>), dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

template <int D>
int launch_d(const DecodeParams &p, int layout, hipStream_t stream)
{
    const unsigned grid = (unsigned)((int64_t)p.B * p.Hkv * p.n_chunks);
    int rc;
    if (p.rot_dim == 0) rc = launch_gt<D, 0, false>(p, grid, stream);
    else if (layout == 0) rc = launch_gt<D, 0, true>(p, grid, stream);
    else rc = launch_gt<D, 1, true>(p, grid, stream);
    if (rc != ROPE_LAUNCH_OK) return rc;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(p.B * p.H)), dim3(256), 0, stream, p,
                       p.rot_dim);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

}  // namespace

int64_t rope_decode_ranges(int64_t S_max) { return (S_max + CW - 1) / CW; }

int rope_launch_decode_bf16(const DecodeArgs &a, hipStream_t stream)
{
    DecodeParams p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k_new = static_cast<const uint16_t *>(a.k_new);
    p.v_new = static_cast<const uint16_t *>(a.v_new);
    p.k_cache = static_cast<uint16_t *>(a.k_cache);
    p.v_cache = static_cast<uint16_t *>(a.v_cache);
    p.lens = a.cache_lens;
    p.cos_tab = a.cos_tab;
    p.sin_tab = a.sin_tab;
    p.part = static_cast<float *>(a.workspace);
    p.o = static_cast<uint16_t *>(a.o);
    p.table_rows = a.table_rows;
    p.S_max = a.S_max;
    p.B = a.B;
    p.H = a.H;
    p.Hkv = a.H_kv;
    p.G = a.H / a.H_kv;
    p.rot_dim = a.rot_dim;
    p.n_chunks = (int)rope_decode_ranges(a.S_max);
    p.sl2 = a.scale * 1.4426950408889634f;
    return a.head_dim == 64 ? launch_d<64>(p, a.layout, stream) : launch_d<128>(p, a.layout, stream);
}
