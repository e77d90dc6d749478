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
// HBM streaming.  The cached positions of every (request, key/value head)
// slice are cut into passes of 64 keys; the passes of all slices, in slice
// order, are split into equal contiguous runs, one per workgroup of a grid
// sized to the machine (stream-K style), so every workgroup moves the same
// number of bytes whatever the mix of lengths, and its loads stay two passes
// ahead of its arithmetic across slice boundaries.  A workgroup serves all G
// query heads that share the slice's key/value head and reads each 16-byte
// chunk of K and V once, with coalesced buffer loads.  Scores come from the
// matrix cores, P V from the vector ALU in fp32.  Each workgroup leaves one
// partial state per slice it touched; a second kernel combines the partial
// states of a slice (running max and sum rescaling, the merge rule of
// section 5 of the same page).
#include <atomic>

#include "common.hpp"
#include "rope_mi355x.h"

namespace {

using rope::elt_to_f32;
using rope::f32_to_elt;
using rope::Ty;
using rope::f32x4_t;

constexpr int SUB = 64;           // keys per pass of the workgroup
constexpr int GMAX = 8;           // query heads per key/value head, at most
constexpr int WG_PER_CU = 2;      // resident workgroups per compute unit (<= 256 registers)
constexpr int NW_MAX = 1024;      // chunk workgroups at most (the workspace is sized for it)

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
    float *part;                // [B * Hkv + nw][G][D + 2]: m, l, O (unnormalised)
    int2 *seg;                  // [B * Hkv]: first workgroup and number of pieces
    uint16_t *o;                // [B, H, D]
    int64_t table_rows, S_max;
    int B, H, Hkv, G, rot_dim, nw;
    float sl2;                  // softmax scale * log2(e)
};

// Passes of request with cached length L: the L + 1 keys the new query sees,
// 64 at a time; none for a length outside the cache (or the table).
template <bool ROT>
__device__ __forceinline__ int passes_of(const DecodeParams &p, int L)
{
    if (L < 0 || (int64_t)L >= p.S_max || (ROT && (int64_t)L >= p.table_rows)) return 0;
    return L / SUB + 1;
}

// Workgroup w of nw owns global passes [w P / nw, (w + 1) P / nw); the one
// that owns pass x is the largest w with w P / nw <= x.
__device__ __forceinline__ int owner_of(int64_t x, int64_t P, int nw)
{
    return (int)(((x + 1) * nw - 1) / P);
}

// A buffer resource over `rows` rows of ROW_BYTES from base: loads past them
// (and with rows <= 0, all loads) return zeros and touch no memory.
template <int ROW_BYTES>
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int rows)
{
    const uint32_t n = rows <= 0 ? 0u : (uint32_t)rows * ROW_BYTES;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, RSRC_FLAGS);
}
// Cached K and V rows are read once per step: the loads carry the
// non-temporal hint (cache policy 2, "nt"), so the stream does not displace
// other lines from the L2 and the last-level cache (5.36 -> 5.91 TB/s on
// 16 requests of 1k-32k cached tokens).
constexpr int STREAM_POLICY = 2;
__device__ __forceinline__ uint4 bload16(rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, STREAM_POLICY));
}
__device__ __forceinline__ void bload(rsrc_t r, int byte_off, uint4 &x) { x = bload16(r, byte_off); }
__device__ __forceinline__ void bload(rsrc_t r, int byte_off, uint2 &x)
{
    x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, STREAM_POLICY));
}

// The value-side shape of the chunk kernel.  Each lane of the P V product
// holds DPL dims of one value row for all query slots: 8 dims (16-byte
// loads), except with 8 query heads at D = 128, where 8 x 8 fp32 sums per
// lane would leave room for only one workgroup per compute unit; there a
// lane takes 4 dims (8-byte loads) and the loads run one pass ahead instead
// of two, which brings the kernel under 256 registers.
template <int D, int GT>
struct ChunkShape {
    static constexpr bool WIDE = GT == 8 && D == 128;
    static constexpr int DPL = WIDE ? 4 : 8;     // value dims per lane
    static constexpr int NSET = WIDE ? 2 : 3;    // register sets of loads (passes in flight + 1)
};
template <int DPL> struct VChunk { using type = uint4; };
template <> struct VChunk<4> { using type = uint2; };

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
__device__ __forceinline__ uint2 pick(bool c, uint2 a, uint2 b)
{
    return make_uint2(c ? a.x : b.x, c ? a.y : b.y);
}

// A run of passes.  The workgroup walks its passes in order with two cursors
// (one for the loads, two passes ahead, one for the arithmetic); a slice's
// passes inside the run form a piece, computed with the slice's rotated
// queries and finished by writing the piece's partial state to slot
// slice + w.  These slots are distinct: a workgroup touches each slice at most
// once and later slices only through later workgroups.  The workgroup that
// owns a slice's first pass records where its pieces lie; the one that owns
// its last pass (the pass holding position L) rotates and appends the new key
// and value.  GT: G rounded up to a power of two.
//
// A pass takes SUB keys, 16 per wave.  Scores come from the matrix cores:
// S (16 keys x 16 query slots) = K Q'^T over D/32 steps of
// v_mfma_f32_16x16x32_bf16, K straight from the loads in the A-operand
// layout (lane l: key l%16, dims 8(l/16) .. +7 of each 32-dim step), Q'
// (rotated, scaled, rounded to bf16) as the B operand, query slots past G
// zero.  P V runs on the vector ALU, each key row split over D/DPL lanes.  Each
// wave runs its own online softmax over its keys; the four waves are merged
// once per piece.
template <int D, int LAYOUT, bool ROT, int GT, typename E>
__global__ __launch_bounds__(256) void decode_chunk_kernel(DecodeParams p)
{
    using V8 = typename Ty<E>::v8;
    using Shape = ChunkShape<D, GT>;
    constexpr int DPL = Shape::DPL;
    using VC = typename VChunk<DPL>::type;
    constexpr int LPR = D / DPL;        // lanes per value row (DPL dims each)
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
    __shared__ __attribute__((aligned(16))) uint16_t knew_lds[D];  // new key, rotated, rounded to E
    __shared__ __attribute__((aligned(16))) uint16_t vnew_lds[D];
    __shared__ __attribute__((aligned(16))) float o_lds[4][GT][D];
    __shared__ int red_lds[4];
    __shared__ int found_lds[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = blockIdx.x;
    const int G = p.G;

    // ---- the run: total passes, then the slice holding the first one ----
    int mine = 0;
    for (int b = tid; b < p.B; b += 256) mine += passes_of<ROT>(p, p.lens[b]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) mine += __shfl_xor(mine, m);
    if (lane == 0) red_lds[wave] = mine;
    if (tid == 0) found_lds[0] = -1;
    __syncthreads();
    const int64_t P = (int64_t)p.Hkv *
                      __builtin_amdgcn_readfirstlane(red_lds[0] + red_lds[1] + red_lds[2] + red_lds[3]);
    // with fewer passes than workgroups only the first P take part, so every
    // run is non-empty and a slice's pieces lie in consecutive workgroups
    const int nw = P < p.nw ? (int)P : p.nw;
    if (w >= nw) return;
    const int64_t lo = (int64_t)w * P / nw, hi = (int64_t)(w + 1) * P / nw;
    if (wave == 0) {
        // request b covers global passes [Hkv pre(b), Hkv pre(b + 1)), pre = passes before b
        int64_t base = 0;
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int b = b0 + lane;
            const int np = b < p.B ? passes_of<ROT>(p, p.lens[b]) : 0;
            int inc = np;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const int y = __shfl_up(inc, m);
                if (lane >= m) inc += y;
            }
            const int64_t start = base + (int64_t)p.Hkv * (inc - np);
            const bool hit = np > 0 && lo >= start && lo < start + (int64_t)p.Hkv * np;
            const uint64_t bal = __ballot(hit);
            if (bal) {
                if (hit) {
                    found_lds[0] = b;
                    found_lds[1] = (int)(lo - start);   // < Hkv * np: fits
                }
                break;
            }
            base += (int64_t)p.Hkv * __shfl(inc, 63);
        }
    }
    __syncthreads();

    struct Cursor {
        int b, kvh, s, np, L;   // request, key/value head, pass in the slice, passes, length
        int64_t pstart;         // global index of the slice's first pass
    };
    Cursor c0;
    c0.b = __builtin_amdgcn_readfirstlane(found_lds[0]);
    if (c0.b < 0) return;   // not reached: lo < P lies in some request
    {
        const int off = __builtin_amdgcn_readfirstlane(found_lds[1]);
        c0.L = p.lens[c0.b];
        c0.np = passes_of<ROT>(p, c0.L);
        if (c0.np <= 0) return;   // not reached either
        c0.kvh = off / c0.np;
        c0.s = off % c0.np;
        c0.pstart = lo - c0.s;
    }
    // the next pass in slice order (only called while one exists)
    auto advance = [&](Cursor &c) {
        if (++c.s < c.np) return;
        c.pstart += c.np;
        c.s = 0;
        if (++c.kvh < p.Hkv) return;
        c.kvh = 0;
        while (c.b + 1 < p.B) {
            ++c.b;
            c.L = p.lens[c.b];
            c.np = passes_of<ROT>(p, c.L);
            if (c.np > 0) break;
        }
    };

    // ---- loads of one pass (issued two passes early) ----
    const int kl = lane % 16, kq = lane / 16;      // score layout: key, dim quarter
    const int vrow = lane / LPR, vsub = lane % LPR; // value layout: row, 16-byte chunk
    auto issue = [&](const Cursor &c, uint4 (&kd)[NT], VC (&vd)[NV]) {
        const int ks = c.s * SUB;
        const int64_t slice = ((int64_t)c.b * p.Hkv + c.kvh) * p.S_max;
        // cached rows [ks, min(L, ks + SUB)); the row at L reads as zero here
        const int rows = c.L - ks < SUB ? c.L - ks : SUB;
        const rsrc_t krs = make_rsrc<2 * D>(p.k_cache + (slice + ks) * D, rows);
        const rsrc_t vrs = make_rsrc<2 * D>(p.v_cache + (slice + ks) * D, rows);
        const int kkey = wave * KPW + kl;
#pragma unroll
        for (int t = 0; t < NT; ++t) kd[t] = bload16(krs, 2 * (kkey * D + 32 * t + 8 * kq));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int key = wave * KPW + i * KPI + vrow;
            bload(vrs, 2 * (key * D + DPL * vsub), vd[i]);
        }
    };

    V8 qb[NT];
    float oacc[GT][DPL];
    float m_run = -INFINITY, l_run = 0.f;

    // ---- start of a piece: the slice's queries (and new key) at position L ----
    auto setup = [&](const Cursor &c) {
        __syncthreads();   // the previous piece is done with the LDS
        const int rh = p.rot_dim / 2;
        const int L = c.L;
        const int bk = c.b * p.Hkv + c.kvh;
        const float *crow = ROT ? p.cos_tab + (int64_t)L * rh : nullptr;
        const float *srow = ROT ? p.sin_tab + (int64_t)L * rh : nullptr;
        for (int idx = tid; idx < G * (D / 2); idx += 256) {
            const int g = idx / (D / 2), i = idx % (D / 2);
            int da, db;
            pair_dims<LAYOUT>(i, ROT ? p.rot_dim : 0, da, db);
            const uint16_t *qr = p.q + ((int64_t)c.b * p.H + c.kvh * G + g) * D;
            const float xa = elt_to_f32<E>(qr[da]), xb = elt_to_f32<E>(qr[db]);
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
        if (c.pstart + c.np - 1 < hi) {   // this run holds the slice's last pass
            const int64_t crow_off = ((int64_t)bk * p.S_max + L) * D;
            for (int i = tid; i < D / 2; i += 256) {
                int da, db;
                pair_dims<LAYOUT>(i, ROT ? p.rot_dim : 0, da, db);
                const uint16_t *kr = p.k_new + (int64_t)bk * D;
                const float xa = elt_to_f32<E>(kr[da]), xb = elt_to_f32<E>(kr[db]);
                float ya = xa, yb = xb;
                if (ROT && i < rh) {
                    const float cs = crow[i], sn = srow[i];
                    ya = xa * cs - xb * sn;
                    yb = xa * sn + xb * cs;
                }
                const uint16_t ba = f32_to_elt<E>(ya), bb = f32_to_elt<E>(yb);
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
        if (c.s == 0 && tid == 0)   // this run holds the slice's first pass
            p.seg[bk] = make_int2(w, owner_of(c.pstart + c.np - 1, P, nw) - w + 1);
        __syncthreads();
        // Q' as the B operand: lane l holds query slot l%16, dims 32t + 8(l/16) + j
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                qb[t][jj] = (E)(kl < GT ? q_lds[kl][32 * t + 8 * kq + jj] : 0.f);
        }
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
            for (int e = 0; e < DPL; ++e) oacc[g][e] = 0.f;
        m_run = -INFINITY;
        l_run = 0.f;
    };

    // Each wave keeps its own running max and sum over its keys, for query
    // slot kl in lanes kl, kl+16, kl+32, kl+48 (MFMA layout); the waves'
    // states are merged once per piece, so the passes need no barrier.
    auto pass = [&](const Cursor &c, const uint4 (&kd)[NT], const VC (&vd)[NV]) {
        const int ks = c.s * SUB;
        const int L = c.L, n = L + 1;
        // scores of the wave's 16 keys for all query slots
        const int kpos = ks + wave * KPW + kl;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const bool knew = kpos == L;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // the new key's chunk is read every time and picked by value (a
            // conditional pointer would send the loaded rows through memory)
            const uint4 kn = *reinterpret_cast<const uint4 *>(knew_lds + 32 * t + 8 * kq);
            const uint4 wv = pick(knew, kn, kd[t]);
            acc = Ty<E>::mfma16(__builtin_bit_cast(V8, wv), qb[t], acc);
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
            for (int e = 0; e < DPL; ++e) oacc[g][e] *= a;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int key = i * KPI + vrow;   // within the wave's block
            const VC vn = *reinterpret_cast<const VC *>(vnew_lds + DPL * vsub);
            const VC wv = pick(ks + wave * KPW + key == L, vn, vd[i]);
            const uint32_t *u = reinterpret_cast<const uint32_t *>(&wv);
            float vf[DPL];
#pragma unroll
            for (int e = 0; e < DPL / 2; ++e) {
                vf[2 * e] = Ty<E>::lo(u[e]);
                vf[2 * e + 1] = Ty<E>::hi(u[e]);
            }
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float pg = p_lds[wave][g][key];
#pragma unroll
                for (int e = 0; e < DPL; ++e) oacc[g][e] = fmaf(pg, vf[e], oacc[g][e]);
            }
        }
    };

    // ---- end of a piece: the four waves' states merged into slot slice + w ----
    auto finish = [&](const Cursor &c) {
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                float x = oacc[g][e];
#pragma unroll
                for (int m = LPR; m < 64; m <<= 1) x += __shfl_xor(x, m);
                oacc[g][e] = x;
            }
        if (lane < LPR) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                float4 *dst = reinterpret_cast<float4 *>(&o_lds[wave][g][DPL * lane]);
#pragma unroll
                for (int e = 0; e < DPL; e += 4)
                    dst[e / 4] = make_float4(oacc[g][e], oacc[g][e + 1], oacc[g][e + 2], oacc[g][e + 3]);
            }
        }
        if (kq == 0 && kl < GT) {
            ml_lds[wave][0][kl] = m_run;
            ml_lds[wave][1][kl] = l_run;
        }
        __syncthreads();
        const int64_t slot = (int64_t)c.b * p.Hkv + c.kvh + w;
        for (int idx = tid; idx < G * D; idx += 256) {
            const int g = idx / D, d = idx % D;
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v) M = fmaxf(M, ml_lds[v][0][g]);   // finite: wave 0's first key is visible
            float o = 0.f, l = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float f = __builtin_amdgcn_exp2f(ml_lds[v][0][g] - M);   // 0 for a wave with no visible key
                o = fmaf(o_lds[v][g][d], f, o);
                l = fmaf(ml_lds[v][1][g], f, l);
            }
            float *dst = p.part + (slot * G + g) * (D + 2);
            dst[2 + d] = o;
            if (d == 0) {
                dst[0] = M;
                dst[1] = l;
            }
        }
    };

    const int npass = (int)(hi - lo);
    auto step = [&](int t, Cursor &c, const uint4 (&kd)[NT], const VC (&vd)[NV]) {
        if (t == 0 || c.s == 0) setup(c);
        pass(c, kd, vd);
        if (t == npass - 1 || c.s == c.np - 1) finish(c);
        if (t + 1 < npass) advance(c);
    };

    Cursor ci = c0, cc = c0;
    if constexpr (Shape::NSET == 2) {
        // two register sets: the loads of pass t+1 are in flight while pass t
        // is computed
        uint4 kd0[NT], kd1[NT];
        VC vd0[NV], vd1[NV];
        issue(ci, kd0, vd0);
        for (int t = 0; t < npass; t += 2) {
            if (t + 1 < npass) {
                advance(ci);
                issue(ci, kd1, vd1);
            }
            step(t, cc, kd0, vd0);
            if (t + 1 >= npass) break;
            if (t + 2 < npass) {
                advance(ci);
                issue(ci, kd0, vd0);
            }
            step(t + 1, cc, kd1, vd1);
        }
        return;
    }
    // three register sets: the loads of passes t+1 and t+2 are in flight
    // while pass t is computed
    uint4 kd0[NT], kd1[NT], kd2[NT];
    VC vd0[NV], vd1[NV], vd2[NV];
    issue(ci, kd0, vd0);
    if (npass > 1) {
        advance(ci);
        issue(ci, kd1, vd1);
    }
    for (int t = 0; t < npass; t += 3) {
        if (t + 2 < npass) {
            advance(ci);
            issue(ci, kd2, vd2);
        }
        step(t, cc, kd0, vd0);
        if (t + 1 >= npass) break;
        if (t + 3 < npass) {
            advance(ci);
            issue(ci, kd0, vd0);
        }
        step(t + 1, cc, kd1, vd1);
        if (t + 2 >= npass) break;
        if (t + 4 < npass) {
            advance(ci);
            issue(ci, kd1, vd1);
        }
        step(t + 2, cc, kd2, vd2);
    }
}

// Output row (b, h): the partial states of the pieces of its slice merged
// (maxima aligned, sums and rows rescaled), O / l rounded to bf16.  A request
// whose length lies outside the cache or the table gets a row of NaN.
//
// D/2 lanes take one piece (two dims each, 8-byte loads), so 256 threads read
// RP = 512/D pieces at a time; each thread walks its pieces U at a time with
// all U loads issued before any is used, keeping a running (max, sum, row)
// that it rescales whenever a larger piece maximum arrives.  The RP running
// states are then merged through LDS by the same rule.
template <int D, typename E>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int rot)
{
    constexpr int LR = D / 2;        // lanes per piece
    constexpr int RP = 256 / LR;     // pieces read at a time
    constexpr int U = 8;             // pieces per thread in flight
    __shared__ float2 red_o[RP][LR];
    __shared__ float red_m[RP], red_l[RP];
    const int bh = blockIdx.x, b = bh / p.H, tid = threadIdx.x;
    const int L = p.lens[b];
    uint16_t *orow = p.o + (int64_t)bh * D;
    if (L < 0 || (int64_t)L >= p.S_max || (rot > 0 && (int64_t)L >= p.table_rows)) {
        for (int d = tid; d < D; d += 256) orow[d] = Ty<E>::QNAN;
        return;
    }
    const int h = bh % p.H, sl = b * p.Hkv + h / p.G;
    const int2 sg = p.seg[sl];   // first workgroup, pieces (>= 1, each with a finite max)
    const int nc = sg.y;
    const float *part = p.part + (((int64_t)sl + sg.x) * p.G + h % p.G) * (D + 2);
    const int64_t pstride = (int64_t)p.G * (D + 2);   // from one piece to the next
    const int r0 = tid / LR, d2 = tid % LR;
    float M = -INFINITY, l = 0.f;
    float2 acc = make_float2(0.f, 0.f);
    for (int c0 = r0; c0 < nc; c0 += RP * U) {
        float mc[U], lc[U];
        float2 oc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // pieces past nc re-read the last one and are given no weight
            const int c = c0 + u * RP < nc ? c0 + u * RP : nc - 1;
            const float *pc = part + c * pstride;
            mc[u] = pc[0];
            lc[u] = pc[1];
            oc[u] = *reinterpret_cast<const float2 *>(pc + 2 + 2 * d2);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u * RP >= nc) break;
            const float mn = fmaxf(M, mc[u]);
            const float a = __builtin_amdgcn_exp2f(M - mn);   // 0 while M is -inf
            const float w = __builtin_amdgcn_exp2f(mc[u] - mn);
            acc.x = fmaf(oc[u].x, w, acc.x * a);
            acc.y = fmaf(oc[u].y, w, acc.y * a);
            l = fmaf(lc[u], w, l * a);
            M = mn;
        }
    }
    red_o[r0][d2] = acc;
    if (d2 == 0) {
        red_m[r0] = M;
        red_l[r0] = l;
    }
    __syncthreads();
    if (tid < LR) {
        float Mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < RP; ++r) Mx = fmaxf(Mx, red_m[r]);   // finite: piece 0 is read by r0 = 0
        float ox = 0.f, oy = 0.f, ls = 0.f;
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float f = __builtin_amdgcn_exp2f(red_m[r] - Mx);   // 0 for a group with no piece
            ox = fmaf(red_o[r][tid].x, f, ox);
            oy = fmaf(red_o[r][tid].y, f, oy);
            ls = fmaf(red_l[r], f, ls);
        }
        const uint32_t pk = Ty<E>::pack2(ox / ls, oy / ls);
        reinterpret_cast<uint32_t *>(orow)[tid] = pk;
    }
}

template <int D, int LAYOUT, bool ROT, typename E>
int launch_gt(const DecodeParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)p.nw);
    if (p.G <= 1)
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 1, E>), grid, dim3(256), 0, stream, p);
    else if (p.G <= 2)
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 2, E>), grid, dim3(256), 0, stream, p);
    else if (p.G <= 4)
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 4, E>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_chunk_kernel<D, LAYOUT, ROT, 8, E>), grid, dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

template <int D, typename E>
int launch_d(const DecodeParams &p, int layout, hipStream_t stream)
{
    if (!rope_grid_fits(p.nw, 256) || !rope_grid_fits((int64_t)p.B * p.H, 256)) return ROPE_LAUNCH_SHAPE;
    int rc;
    if (p.rot_dim == 0) rc = launch_gt<D, 0, false, E>(p, stream);
    else if (layout == 0) rc = launch_gt<D, 0, true, E>(p, stream);
    else rc = launch_gt<D, 1, true, E>(p, stream);
    if (rc != ROPE_LAUNCH_OK) return rc;
    hipLaunchKernelGGL((decode_merge_kernel<D, E>), dim3((unsigned)(p.B * p.H)), dim3(256), 0, stream, p,
                       p.rot_dim);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

// Workgroups of the chunk kernel on the current device (0 on error).
int decode_workgroups()
{
    const int n = WG_PER_CU * rope_device_cu_count();
    return n < NW_MAX ? n : NW_MAX;
}

// Partial states for up to NW_MAX workgroups, then the piece table from a
// 256-byte boundary.
int64_t part_bytes(int B, int H, int H_kv, int head_dim)
{
    const int64_t n = ((int64_t)B * H_kv + NW_MAX) * (H / H_kv) * (head_dim + 2) * 4;
    return (n + 255) / 256 * 256;
}

}  // namespace

// Static scratch of the allocation-free decode entry point: partial states
// and piece table, one copy per GPU.  Host code never uses this name as an
// address (on the host it is a stand-in symbol); it asks HIP for the
// device copy's address and keeps that per device.
static __device__ __align__(256) unsigned char scratch[ROPE_DECODE_SCRATCH_BYTES];

namespace {
std::atomic<void *> g_scratch[64];
}  // namespace

void *rope_decode_static_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        // with `dev` current: its own copy of the array
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

int64_t rope_decode_max_passes(int B, int H_kv, int64_t S_max)
{
    return (int64_t)B * H_kv * (S_max / SUB + 1);
}

int64_t rope_decode_workspace_bytes(int B, int H, int H_kv, int head_dim)
{
    return part_bytes(B, H, H_kv, head_dim) + (int64_t)B * H_kv * 8;
}

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
    p.nw = decode_workgroups();
    if (p.nw <= 0) return ROPE_LAUNCH_ERR;
    p.part = static_cast<float *>(a.workspace);
    p.seg = reinterpret_cast<int2 *>(static_cast<char *>(a.workspace) +
                                     part_bytes(a.B, a.H, a.H_kv, a.head_dim));
    p.o = static_cast<uint16_t *>(a.o);
    p.table_rows = a.table_rows;
    p.S_max = a.S_max;
    p.B = a.B;
    p.H = a.H;
    p.Hkv = a.H_kv;
    p.G = a.H / a.H_kv;
    p.rot_dim = a.rot_dim;
    p.sl2 = a.scale * 1.4426950408889634f;
    // dtype 0 (bf16) or 2 (fp16): the same kernels over either 16-bit type
    if (a.dtype == 2)
        return a.head_dim == 64 ? launch_d<64, _Float16>(p, a.layout, stream) : launch_d<128, _Float16>(p, a.layout, stream);
    return a.head_dim == 64 ? launch_d<64, __bf16>(p, a.layout, stream) : launch_d<128, __bf16>(p, a.layout, stream);
}
