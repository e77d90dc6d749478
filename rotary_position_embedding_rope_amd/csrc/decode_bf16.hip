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
// HBM streaming: a workgroup takes one request, one key/value head and a
// contiguous range of CW cached positions for all G query heads that share
// the key/value head, and reads each 16-byte chunk of K and V once with
// coalesced buffer loads, two passes ahead of the one being computed.
// Scores come from the matrix cores, P V from the vector ALU in fp32.
// Ranges of one (request, key/value head) are combined by a second kernel
// (running max and sum rescaling, the merge rule of section 5 of the same
// page).
#include "common.hpp"

namespace {

using rope::bf16_to_f32;
using rope::bf16x8_t;
using rope::f32_to_bf16;
using rope::f32x4_t;

constexpr int SUB = 64;           // keys per pass of the workgroup
constexpr int NSUB = 8;           // passes per workgroup
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

// Orders the LDS accesses of the lanes of one wave around it: writes before
// it are seen by reads after it in any lane of the wave (lanes are separate
// threads; without this the compiler may move a read across another lane's
// write).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint4 pick(bool c, uint4 a, uint4 b)
{
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
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
//
// A pass takes SUB keys, 16 per wave.  Scores come from the matrix cores:
// S (16 keys x 16 query slots) = K Q'^T over D/32 steps of
// v_mfma_f32_16x16x32_bf16, K straight from the loads in the A-operand
// layout (lane l: key l%16, dims 8(l/16) .. +7 of each 32-dim step), Q'
// (rotated, scaled, rounded to bf16) as the B operand, query slots past G
// zero.  P V runs on the vector ALU, each key row split over D/8 lanes.  The
// loads of passes s+1 and s+2 are in flight while pass s is computed.  Each
// wave runs its own online softmax over its keys; the four waves are merged
// once at the end.
template <int D, int LAYOUT, bool ROT, int GT>
__global__ __launch_bounds__(256) void decode_chunk_kernel(DecodeParams p)
{
    constexpr int LPR = D / 8;          // lanes per value row (16 bytes each)
    constexpr int KPI = 64 / LPR;       // value rows per wave load
    constexpr int KPW = SUB / 4;        // keys per wave and pass (16)
    constexpr int NV = KPW / KPI;       // value loads per wave and pass
    constexpr int NT = D / 32;          // score MFMA steps (and key loads) per pass
    static_assert(KPW == 16, "one 16-key score block per wave and pass");
    static_assert(GT <= 16 && GT <= GMAX, "query slots of the score block");

    __shared__ __attribute__((aligned(16))) float q_lds[GT][D];    // rotated, scaled queries
    __shared__ __attribute__((aligned(16))) float p_lds[4][GT][KPW];   // per wave: probabilities
    __shared__ float a_lds[4][GT];                                 // per wave: rescale factors
    __shared__ float ml_lds[4][2][GT];                             // per wave: max and sum
    __shared__ __attribute__((aligned(16))) uint16_t knew_lds[D];  // new key, rotated, bf16
    __shared__ __attribute__((aligned(16))) uint16_t vnew_lds[D];
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

    // ---- loads of one pass (issued early) ----
    const int64_t slice = (int64_t)bk * p.S_max;   // row of (b, kvh, position 0)
    const int kl = lane % 16, kq = lane / 16;      // score layout: key, dim quarter
    const int vrow = lane / LPR, vsub = lane % LPR; // value layout: row, 16-byte chunk
    auto issue = [&](int s, uint4 (&kd)[NT], uint4 (&vd)[NV]) {
        const int ks = k0 + s * SUB;
        // cached rows [ks, min(L, ks + SUB)); the row at L reads as zero here
        const int rows = L - ks < SUB ? L - ks : SUB;
        const rsrc_t krs = make_rsrc<2 * D>(p.k_cache + (slice + ks) * D, rows);
        const rsrc_t vrs = make_rsrc<2 * D>(p.v_cache + (slice + ks) * D, rows);
        const int kkey = wave * KPW + kl;
#pragma unroll
        for (int t = 0; t < NT; ++t) kd[t] = bload16(krs, 2 * (kkey * D + 32 * t + 8 * kq));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int key = wave * KPW + i * KPI + vrow;
            vd[i] = bload16(vrs, 2 * (key * D + 8 * vsub));
        }
    };
    // three register sets: the loads of passes s+1 and s+2 are in flight
    // while pass s is computed
    uint4 kd0[NT], vd0[NV], kd1[NT], vd1[NV], kd2[NT], vd2[NV];
    auto valid = [&](int s) { return s < NSUB && k0 + s * SUB < n; };
    issue(0, kd0, vd0);
    if (valid(1)) issue(1, kd1, vd1);

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
    for (int idx = G * D + tid; idx < GT * D; idx += 256) q_lds[idx / D][idx % D] = 0.f;
    const bool last = n - k0 <= CW;           // this range holds position L
    if (last) {
        const int64_t crow_off = (slice + L) * D;
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
    __syncthreads();

    // Q' as the B operand: lane l holds query slot l%16, dims 32t + 8(l/16) + j
    bf16x8_t qb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            qb[t][jj] = (__bf16)(kl < GT ? q_lds[kl][32 * t + 8 * kq + jj] : 0.f);
    }

    float oacc[GT][8];
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[g][e] = 0.f;

    // Each wave keeps its own running max and sum over its keys, for query
    // slot kl in lanes kl, kl+16, kl+32, kl+48 (MFMA layout); the waves'
    // states are merged once, at the end, so the passes need no barrier.
    float m_run = -INFINITY, l_run = 0.f;
    auto pass = [&](int s, const uint4 (&kd)[NT], const uint4 (&vd)[NV]) {
        const int ks = k0 + s * SUB;
        // scores of the wave's 16 keys for all query slots
        const int kpos = ks + wave * KPW + kl;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const bool knew = kpos == L;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // the new key's chunk is read every time and picked by value (a
            // conditional pointer would send the loaded rows through memory)
            const uint4 kn = *reinterpret_cast<const uint4 *>(knew_lds + 32 * t + 8 * kq);
            const uint4 w = pick(knew, kn, kd[t]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w), qb[t], acc,
                                                          0, 0, 0);
        }
        // accumulator element r of lane l: key 4(l/16) + r of the block, query slot l%16
        float sc[4];
        float mb = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sc[r] = ks + wave * KPW + 4 * kq + r < n ? acc[r] : -INFINITY;
            mb = fmaxf(mb, sc[r]);
        }
        mb = fmaxf(mb, __shfl_xor(mb, 16));
        mb = fmaxf(mb, __shfl_xor(mb, 32));
        const float m_new = fmaxf(m_run, mb);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;   // no visible key yet: all p are 0
        float ps = 0.f, pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = __builtin_amdgcn_exp2f(sc[r] - m_use);
            ps += pr[r];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // 0 before the first visible key
        l_run = l_run * alpha + ps;
        m_run = m_new;
        // probabilities and rescale factors to the value layout, through the
        // wave's own LDS (no other wave reads them)
        wave_sync();   // the previous pass's reads are done
        if (kl < GT) {
            *reinterpret_cast<float4 *>(&p_lds[wave][kl][4 * kq]) = make_float4(pr[0], pr[1], pr[2], pr[3]);
            if (kq == 0) a_lds[wave][kl] = alpha;
        }
        wave_sync();
        // O += P V for the wave's keys, after rescaling to the new maxima
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float a = a_lds[wave][g];
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[g][e] *= a;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int key = i * KPI + vrow;   // within the wave's block
            const uint4 vn = *reinterpret_cast<const uint4 *>(vnew_lds + 8 * vsub);
            const uint4 w = pick(ks + wave * KPW + key == L, vn, vd[i]);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
            float vf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[2 * e] = rope::bf16lo_to_f32(u[e]);
                vf[2 * e + 1] = rope::bf16hi_to_f32(u[e]);
            }
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float pg = p_lds[wave][g][key];
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[g][e] = fmaf(pg, vf[e], oacc[g][e]);
            }
        }
    };
    for (int s = 0; s < NSUB; s += 3) {
        if (!valid(s)) break;
        if (valid(s + 2)) issue(s + 2, kd2, vd2);
        pass(s, kd0, vd0);
        if (!valid(s + 1)) break;
        if (valid(s + 3)) issue(s + 3, kd0, vd0);
        pass(s + 1, kd1, vd1);
        if (!valid(s + 2)) break;
        if (valid(s + 4)) issue(s + 4, kd1, vd1);
        pass(s + 2, kd2, vd2);
    }

    // ---- the range's partial state: the four waves' states merged ----
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
    if (kq == 0 && kl < GT) {
        ml_lds[wave][0][kl] = m_run;
        ml_lds[wave][1][kl] = l_run;
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][0][g]);   // finite: wave 0 sees key k0
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = __builtin_amdgcn_exp2f(ml_lds[w][0][g] - M);   // 0 for a wave with no visible key
            o = fmaf(o_lds[w][g][d], f, o);
            l = fmaf(ml_lds[w][1][g], f, l);
        }
        float *dst = p.part + (((int64_t)b * p.H + kvh * G + g) * p.n_chunks + c) * (D + 2);
        dst[2 + d] = o;
        if (d == 0) {
            dst[0] = M;
            dst[1] = l;
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
