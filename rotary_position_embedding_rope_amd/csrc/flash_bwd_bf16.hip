// flash_bwd_bf16.hip -- backward of the fused RoPE + softmax attention on the
// gfx950 matrix cores (bf16 inputs and gradients, fp32 accumulation).
//
// What it computes: for O = softmax(scale * rope(Q) rope(K)^T + mask) V and an
// upstream gradient dO, the gradients dQ, dK, dV ("RoPE and FlashAttention:
// relative positions and online softmax", section 5: the backward rebuilds
// the probabilities from Q, K and the saved row statistics instead of keeping
// the probability matrix; section 8, item 4: it recomputes the scores).  With
// Q' = R(q_pos) Q and K' = R(k_pos) K:
//   P = exp(S - lse)             S = scale Q' K'^T, lse saved by the forward
//   dV  = P^T dO                 (summed over the query heads of a group)
//   dP  = dO V^T,  dS = P * (dP - delta),  delta_i = dO_i . O_i
//   dQ' = scale dS K',   dK' = scale dS^T Q'
//   dQ = R(q_pos)^T dQ', dK = R(k_pos)^T dK'   (rotation by the opposite angle)
// V is never rotated (section 1).  Query i sits at q_off + i, key j at
// k_off + j; with the causal mask key j is visible iff k_off + j <= q_off + i
// (section 6).
//
// Two kernels, enqueued in order on the caller's stream: bwd_rotate_kernel
// (Q' = rope(Q) * scale * log2(e) and K' = rope(K), once, rounded, into the
// workspace, and delta = rowsum(dO * O) into the workspace; without rotation
// bwd_delta_kernel computes delta alone); then bwd_main_kernel, whose
// workgroups are of two kinds:
//   * bwd_dkv_kernel: a workgroup owns 128 keys of one (batch, key/value
//     head), 32 per wave; K' and V sit in registers as
//     matrix-core operands while the workgroup walks the query rows that see
//     them, 32 at a time, for every query head of the group: Q' and dO are
//     staged in LDS as plain copies, one tile ahead, and
//     dK^T, dV^T accumulate in registers, so the head-group sum needs no
//     atomics;
//   * bwd_dq_kernel: a workgroup owns 128 query rows of one head, 32 per
//     wave; Q' and dO sit in registers while K' and V
//     tiles of 32 keys stream through LDS, one tile ahead; dQ^T accumulates
//     in registers.
// Every product is v_mfma_f32_32x32x16_bf16.  Score tiles are laid out so
// that their accumulator doubles as the next product's operand: a lane owns
// one column (a key in the dK/dV kernel, a query in the dQ kernel), and P and
// dS leave the accumulator in the B-operand layout of the transposed product;
// the matching A operand (dO^T, Q'^T or K'^T) comes from ds_read_b64_tr_b16
// reads of the row-major LDS tile.  The un-rotation of dQ' and dK' happens in
// registers, with the table rows of the positions a lane owns, before the
// single bf16 store.
#include "common.hpp"

namespace {

using rope::f32x16_t;
using rope::Ty;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int WROWS = 32;            // rows (keys or queries) a wave owns
constexpr int WG_ROWS = 4 * WROWS;   // rows a workgroup owns
constexpr int TILE = 32;             // rows of a staged tile

struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;   // q, o, dout [BH, Sq, D]; k, v [B*Hkv, Sk, D]
    const float *lse;                       // [BH, Sq], natural log
    float *delta;                           // [BH, Sq] (workspace)
    uint16_t *dq, *dk, *dv;
    const float *cos_tab, *sin_tab;         // [table_rows, rot/2]
    int64_t Sq, Sk, q_off, k_off;
    int B, H, Hkv, kv_group, causal;
    int n_qtiles, n_ktiles;                 // 128-row tiles of the dQ and dK/dV kernels
    float scale, sl2;                       // softmax scale; scale * log2(e)
};

// E: the 16-bit storage type (__bf16 or _Float16); V8<E>: 8 of them, the
// matrix-core operand.
template <typename E> using V8 = typename Ty<E>::v8;

template <typename E>
__device__ __forceinline__ void unpack8(const uint4 w, float (&x)[8])
{
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = Ty<E>::lo(u[i]);
        x[2 * i + 1] = Ty<E>::hi(u[i]);
    }
}
template <typename E>
__device__ __forceinline__ uint4 pack8(const float (&x)[8])
{
    return make_uint4(Ty<E>::pack2(x[0], x[1]), Ty<E>::pack2(x[2], x[3]), Ty<E>::pack2(x[4], x[5]),
                      Ty<E>::pack2(x[6], x[7]));
}
template <typename E>
__device__ __forceinline__ V8<E> to_v8(const float (&x)[8])
{
    return __builtin_bit_cast(V8<E>, pack8<E>(x));
}
template <typename E>
__device__ __forceinline__ f32x16_t mfma(V8<E> a, V8<E> b, f32x16_t c)
{
    return Ty<E>::mfma(a, b, c);
}

// Staging of row-major [ROWS][D] bf16 tiles into LDS, in units a thread loads
// into registers one tile ahead and writes (rotated, scaled, rounded) after
// the tile before it is consumed.  A unit is 8 dims copied, or a GPT-J chunk
// of 4 pairs, or a NeoX low chunk with its partner chunk rot/2 dims later.
template <int D, int LAYOUT, int ROTD>
struct Geo {
    static constexpr int NROT = ROTD == 0 ? 0 : (LAYOUT == 0 ? ROTD / 16 : ROTD / 8);
    static constexpr int NTAIL = (D - ROTD) / 8;
    static constexpr int UPR = NROT + NTAIL;   // units per row
};

struct Unit {
    uint4 a, b;                 // the chunk; NeoX: its partner chunk
    float4 c0, c1, s0, s1;      // cos / sin of the unit's frequencies
};

template <int D, int LAYOUT, int ROTD, int ROWS, int NTH, typename E>
struct Stager {
    using G = Geo<D, LAYOUT, ROTD>;
    static constexpr int NU = (ROWS * G::UPR + NTH - 1) / NTH;
    Unit u[NU];

    // rows [0, valid) of src (row r at src + r D, position pos0 + r); the
    // other rows stage as zeros
    __device__ __forceinline__ void fetch(const uint16_t *src, int valid, int64_t pos0, const float *cos_tab,
                                          const float *sin_tab, int tid)
    {
#pragma unroll
        for (int n = 0; n < NU; ++n) {
            const int id = tid + NTH * n;
            const int r = id / G::UPR, k = id % G::UPR;
            Unit &x = u[n];
            x.a = x.b = make_uint4(0, 0, 0, 0);
            x.c0 = x.c1 = x.s0 = x.s1 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (id >= ROWS * G::UPR || r >= valid) continue;
            const uint16_t *row = src + (int64_t)r * D;
            if (k < G::NROT) {
                const float *cr = cos_tab + (pos0 + r) * (ROTD / 2);
                const float *sr = sin_tab + (pos0 + r) * (ROTD / 2);
                if constexpr (LAYOUT == 0) {
                    x.a = *reinterpret_cast<const uint4 *>(row + 8 * k);
                    x.b = *reinterpret_cast<const uint4 *>(row + 8 * k + ROTD / 2);
                    x.c0 = *reinterpret_cast<const float4 *>(cr + 8 * k);
                    x.c1 = *reinterpret_cast<const float4 *>(cr + 8 * k + 4);
                    x.s0 = *reinterpret_cast<const float4 *>(sr + 8 * k);
                    x.s1 = *reinterpret_cast<const float4 *>(sr + 8 * k + 4);
                } else {
                    x.a = *reinterpret_cast<const uint4 *>(row + 8 * k);
                    x.c0 = *reinterpret_cast<const float4 *>(cr + 4 * k);
                    x.s0 = *reinterpret_cast<const float4 *>(sr + 4 * k);
                }
            } else {
                x.a = *reinterpret_cast<const uint4 *>(row + ROTD + 8 * (k - G::NROT));
            }
        }
    }

    // the fetched units of rows [0, rows), rotated and multiplied by mul,
    // to dst (row pitch P)
    template <int P>
    __device__ __forceinline__ void store(uint16_t *dst, float mul, int tid, int rows = ROWS) const
    {
#pragma unroll
        for (int n = 0; n < NU; ++n) {
            const int id = tid + NTH * n;
            if (id >= ROWS * G::UPR) continue;
            const int r = id / G::UPR, k = id % G::UPR;
            if (r >= rows) continue;
            const Unit &x = u[n];
            uint16_t *row = dst + r * P;
            float a[8];
            unpack8<E>(x.a, a);
            if (k < G::NROT) {
                if constexpr (LAYOUT == 0) {
                    float b[8], lo[8], hi[8];
                    unpack8<E>(x.b, b);
                    const float c[8] = {x.c0.x, x.c0.y, x.c0.z, x.c0.w, x.c1.x, x.c1.y, x.c1.z, x.c1.w};
                    const float s[8] = {x.s0.x, x.s0.y, x.s0.z, x.s0.w, x.s1.x, x.s1.y, x.s1.z, x.s1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        lo[e] = (a[e] * c[e] - b[e] * s[e]) * mul;
                        hi[e] = (a[e] * s[e] + b[e] * c[e]) * mul;
                    }
                    *reinterpret_cast<uint4 *>(row + 8 * k) = pack8<E>(lo);
                    *reinterpret_cast<uint4 *>(row + 8 * k + ROTD / 2) = pack8<E>(hi);
                } else {
                    const float c[4] = {x.c0.x, x.c0.y, x.c0.z, x.c0.w};
                    const float s[4] = {x.s0.x, x.s0.y, x.s0.z, x.s0.w};
                    float y[8];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        y[2 * m] = (a[2 * m] * c[m] - a[2 * m + 1] * s[m]) * mul;
                        y[2 * m + 1] = (a[2 * m] * s[m] + a[2 * m + 1] * c[m]) * mul;
                    }
                    *reinterpret_cast<uint4 *>(row + 8 * k) = pack8<E>(y);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] *= mul;
                *reinterpret_cast<uint4 *>(row + ROTD + 8 * (k - G::NROT)) = pack8<E>(a);
            }
        }
    }
};

// A row owned by a lane as a B operand of the 32x32x16 products: lane half hh
// holds dims 16 s + 8 hh .. + 7 of step s, rotated at pos (NeoX partners sit
// rot/32 steps later in the same lane; GPT-J pairs are adjacent), multiplied
// by mul and rounded to bf16.  An invalid row is zero.
template <int D, int LAYOUT, int ROTD, typename E>
__device__ __forceinline__ void row_operand(const uint16_t *row, bool valid, int64_t pos, float mul,
                                            const float *cos_tab, const float *sin_tab, int hh,
                                            V8<E> (&out)[D / 16])
{
    constexpr int NS = D / 16;
    float x[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const uint4 w = valid ? *reinterpret_cast<const uint4 *>(row + 16 * s + 8 * hh) : make_uint4(0, 0, 0, 0);
        unpack8<E>(w, x[s]);
    }
    if constexpr (ROTD > 0) {
        if (valid) {
            const float *cr = cos_tab + pos * (ROTD / 2), *sr = sin_tab + pos * (ROTD / 2);
            if constexpr (LAYOUT == 0) {
                constexpr int M = ROTD / 32;
#pragma unroll
                for (int s = 0; s < M; ++s) {
                    const float4 c0 = *reinterpret_cast<const float4 *>(cr + 16 * s + 8 * hh);
                    const float4 c1 = *reinterpret_cast<const float4 *>(cr + 16 * s + 8 * hh + 4);
                    const float4 s0 = *reinterpret_cast<const float4 *>(sr + 16 * s + 8 * hh);
                    const float4 s1 = *reinterpret_cast<const float4 *>(sr + 16 * s + 8 * hh + 4);
                    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float lo = x[s][e], hi = x[s + M][e];
                        x[s][e] = lo * c[e] - hi * sn[e];
                        x[s + M][e] = lo * sn[e] + hi * c[e];
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < ROTD / 16; ++s) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(cr + 8 * s + 4 * hh);
                    const float4 s4 = *reinterpret_cast<const float4 *>(sr + 8 * s + 4 * hh);
                    const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float a = x[s][2 * m], b = x[s][2 * m + 1];
                        x[s][2 * m] = a * c[m] - b * sn[m];
                        x[s][2 * m + 1] = a * sn[m] + b * c[m];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] *= mul;
        out[s] = to_v8<E>(x[s]);
    }
}

// acc[bd][4 i + j] holds dim 32 bd + 8 i + 4 hh + j of one row: rotate it
// back by the angle of position pos (R^T: lo = lo' c + hi' s, hi = hi' c - lo' s).
template <int D, int LAYOUT, int ROTD>
__device__ __forceinline__ void unrotate(f32x16_t (&acc)[D / 32], int64_t pos, const float *cos_tab,
                                         const float *sin_tab, int hh)
{
    if constexpr (ROTD > 0) {
        const float *cr = cos_tab + pos * (ROTD / 2), *sr = sin_tab + pos * (ROTD / 2);
        if constexpr (LAYOUT == 0) {
#pragma unroll
            for (int bd = 0; bd < D / 32; ++bd)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (32 * bd + 8 * i >= ROTD / 2) continue;   // not a low dim
                    constexpr int HALF = ROTD / 2;
                    const int dp = 32 * bd + 8 * i + HALF;        // partner of the block's first dim
                    const int bp = dp / 32, ip = (dp % 32) / 8;
                    const float4 c4 = *reinterpret_cast<const float4 *>(cr + 32 * bd + 8 * i + 4 * hh);
                    const float4 s4 = *reinterpret_cast<const float4 *>(sr + 32 * bd + 8 * i + 4 * hh);
                    const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float lo = acc[bd][4 * i + j], hi = acc[bp][4 * ip + j];
                        acc[bd][4 * i + j] = lo * c[j] + hi * sn[j];
                        acc[bp][4 * ip + j] = hi * c[j] - lo * sn[j];
                    }
                }
        } else {
#pragma unroll
            for (int bd = 0; bd < ROTD / 32; ++bd)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float2 c2 = *reinterpret_cast<const float2 *>(cr + 16 * bd + 4 * i + 2 * hh);
                    const float2 s2 = *reinterpret_cast<const float2 *>(sr + 16 * bd + 4 * i + 2 * hh);
                    const float c[2] = {c2.x, c2.y}, sn[2] = {s2.x, s2.y};
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const float a = acc[bd][4 * i + 2 * m], b = acc[bd][4 * i + 2 * m + 1];
                        acc[bd][4 * i + 2 * m] = a * c[m] + b * sn[m];
                        acc[bd][4 * i + 2 * m + 1] = b * c[m] - a * sn[m];
                    }
                }
        }
    }
}

// One row (acc layout above), times mul, rounded to bf16, 8-byte stores.
template <int D, typename E>
__device__ __forceinline__ void store_row(uint16_t *row, const f32x16_t (&acc)[D / 32], float mul, int hh)
{
#pragma unroll
    for (int bd = 0; bd < D / 32; ++bd)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint2 w;
            w.x = Ty<E>::pack2(acc[bd][4 * i] * mul, acc[bd][4 * i + 1] * mul);
            w.y = Ty<E>::pack2(acc[bd][4 * i + 2] * mul, acc[bd][4 * i + 3] * mul);
            *reinterpret_cast<uint2 *>(row + 32 * bd + 8 * i + 4 * hh) = w;
        }
}

// The A operand of a transposed product from a row-major LDS tile T (pitch P):
// lane l gets column 32 bd + l % 32 of rows 16 mm + 4 (l / 32) + {0..3} and
// the same + 8 -- the row order in which a score accumulator's rows 8 i +
// 4 (l / 32) + j, i = 2 mm, 2 mm + 1, leave as a B operand.
template <int P, typename E>
__device__ __forceinline__ V8<E> tr_operand(const uint16_t *T, int mm, int bd, int tr_row0, int tr_col)
{
    const uint16_t *src = T + (16 * mm + tr_row0) * P + 32 * bd + tr_col;
    const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)src);
    const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(src + 8 * P));
    return __builtin_bit_cast(V8<E>, (short __attribute__((ext_vector_type(8)))){
                                            x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
}

// rows 8 mm .. 8 mm + 7 of a score accumulator, rounded: the B operand of
// 16-row step mm
template <typename E>
__device__ __forceinline__ V8<E> acc_operand(const float (&v)[16], int mm)
{
    const float x[8] = {v[8 * mm], v[8 * mm + 1], v[8 * mm + 2], v[8 * mm + 3],
                        v[8 * mm + 4], v[8 * mm + 5], v[8 * mm + 6], v[8 * mm + 7]};
    return to_v8<E>(x);
}

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O), D/8 lanes per row.
template <int D, typename E>
__device__ __forceinline__ void delta_rows(const uint16_t *o, const uint16_t *dout, float *delta, int64_t rows,
                                           int64_t blk)
{
    constexpr int LPR = D / 8, RPB = 256 / LPR;
    const int64_t r = blk * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (r < rows) {
        float a[8], b[8];
        unpack8<E>(*reinterpret_cast<const uint4 *>(o + r * D + 8 * c), a);
        unpack8<E>(*reinterpret_cast<const uint4 *>(dout + r * D + 8 * c), b);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(a[e], b[e], acc);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (c == 0 && r < rows) delta[r] = acc;
}

template <int D, typename E>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t *o, const uint16_t *dout, float *delta,
                                                        int64_t rows)
{
    delta_rows<D, E>(o, dout, delta, rows, blockIdx.x);
}

// The rotated operands, once: row i of q rotated at q_off + i, multiplied by
// scale log2(e) and rounded to E; row j of k rotated at k_off + j and
// rounded.  One 32-row tile of one head per workgroup, query tiles first.
// The main kernel then stages these rows as plain copies, instead of
// rotating a query tile again for every key tile that sees it (and a key
// tile for every query tile).
// The same launch computes the row sums: blocks past the rotation tiles run
// bwd_delta_kernel's rows.
template <int D, int LAYOUT, int ROTD, typename E>
__global__ __launch_bounds__(256) void bwd_rotate_kernel(BwdParams p, const uint16_t *q, const uint16_t *k,
                                                         uint16_t *qr, uint16_t *kr)
{
    const int64_t tq = (p.Sq + TILE - 1) / TILE, tk = (p.Sk + TILE - 1) / TILE;
    const int64_t nq = (int64_t)p.B * p.H * tq, nrot = nq + (int64_t)p.B * p.Hkv * tk;
    int64_t blk = blockIdx.x;
    if (blk >= nrot) {
        delta_rows<D, E>(p.o, p.dout, p.delta, (int64_t)p.B * p.H * p.Sq, blk - nrot);
        return;
    }
    const bool isq = blk < nq;
    if (!isq) blk -= nq;
    const int64_t t = isq ? tq : tk, S = isq ? p.Sq : p.Sk;
    const int64_t head = blk / t, i = (blk % t) * TILE;
    const int64_t off = (head * S + i) * D;
    const int rows = S - i < TILE ? (int)(S - i) : TILE;
    Stager<D, LAYOUT, ROTD, TILE, 256, E> st;
    st.fetch((isq ? q : k) + off, rows, (isq ? p.q_off : p.k_off) + i, p.cos_tab, p.sin_tab, threadIdx.x);
    st.template store<D>((isq ? qr : kr) + off, isq ? p.sl2 : 1.f, threadIdx.x, rows);
}

// The halves of a workgroup: NH = 2 for D = 64 (8 waves, two per SIMD: the
// halves take alternate 32-row steps and are summed at the end), NH = 1 for
// D = 128 (its accumulators leave room for one wave per SIMD).
template <int D> struct Halves { static constexpr int NH = D == 64 ? 2 : 1; };

// Half 1's accumulators added into half 0's through LDS (`buf`, at least
// 4 waves x 64 lanes x 16 floats), one block of 16 at a time; ends with the
// sum in half 0.
template <int DB>
__device__ __forceinline__ void fold_halves(f32x16_t (&acc)[DB], float *buf, int half, int wv, int lane)
{
#pragma unroll
    for (int bd = 0; bd < DB; ++bd) {
        __syncthreads();
        if (half == 1)
#pragma unroll
            for (int r = 0; r < 16; ++r) buf[(wv * 16 + r) * 64 + lane] = acc[bd][r];
        __syncthreads();
        if (half == 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[bd][r] += buf[(wv * 16 + r) * 64 + lane];
    }
}

// LDS of a workgroup: two double-buffered [ROWS][D + 8] bf16 tiles and two
// double-buffered rows of ROWS floats.
template <int D>
struct Lds {
    static constexpr int ROWS = TILE * Halves<D>::NH, P = D + 8;
    static constexpr int TILE_ELEMS = ROWS * P;
    static constexpr int BYTES = 4 * TILE_ELEMS * 2 + 4 * ROWS * 4;
    static_assert(2 * TILE_ELEMS * 2 >= 4 * 64 * 16 * 4 || Halves<D>::NH == 1, "LDS for the fold");
};

// ---------------------------------------------------------------------------
// dK, dV: 128 keys of one (batch, key/value head) per workgroup; blk orders
// the tiles heaviest first (with the causal mask the first keys see the most
// queries).
template <int D, int LAYOUT, int ROTD, typename E>
__device__ __forceinline__ void dkv_block(const BwdParams &p, int blk, unsigned char *smem)
{
    constexpr int NH = Halves<D>::NH, NTH = 256 * NH, ROWS = TILE * NH;
    constexpr int P = D + 8;   // LDS row pitch (bf16)
    constexpr int NS = D / 16, DB = D / 32, TE = Lds<D>::TILE_ELEMS;
    uint16_t(*q_lds)[TE] = reinterpret_cast<uint16_t(*)[TE]>(smem);
    uint16_t(*do_lds)[TE] = reinterpret_cast<uint16_t(*)[TE]>(smem + 2 * TE * 2);
    float(*lse_lds)[ROWS] = reinterpret_cast<float(*)[ROWS]>(smem + 4 * TE * 2);
    float(*dl_lds)[ROWS] = reinterpret_cast<float(*)[ROWS]>(smem + 4 * TE * 2 + 2 * ROWS * 4);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = wave >> 2, wv = wave & 3;   // this wave's half and its place in it
    const int l32 = lane & 31, hh = lane >> 5;
    const int BKV = p.B * p.Hkv;
    const int bkv = blk % BKV;
    const int kt = blk / BKV;
    const int b = bkv / p.Hkv, kvh = bkv % p.Hkv;
    const int64_t key = (int64_t)kt * WG_ROWS + wv * WROWS + l32;   // this lane's key
    const bool kvalid = key < p.Sk;
    const int g16 = lane >> 4, lp = lane & 15;
    const int tr_row0 = 4 * (g16 >> 1) + (lp >> 2), tr_col = 4 * (lp & 3) + 16 * (g16 & 1);

    V8<E> kb[NS], vb[NS];
    const uint16_t *krow = p.k + ((int64_t)bkv * p.Sk + key) * D;
    const uint16_t *vrow = p.v + ((int64_t)bkv * p.Sk + key) * D;
    row_operand<D, 0, 0, E>(krow, kvalid, 0, 1.f, nullptr, nullptr, hh, kb);   // rotated beforehand
    row_operand<D, 0, 0, E>(vrow, kvalid, 0, 1.f, nullptr, nullptr, hh, vb);
    f32x16_t dk[DB], dv[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dk[i] = dv[i] = (f32x16_t){};

    // query rows that see a key of this tile start at k_off + first key - q_off
    int64_t i0 = 0;
    if (p.causal) {
        i0 = p.k_off + (int64_t)kt * WG_ROWS - p.q_off;
        if (i0 < 0) i0 = 0;
        i0 = i0 / ROWS * ROWS;
    }
    const int nsteps = i0 < p.Sq ? (int)((p.Sq - i0 + ROWS - 1) / ROWS) : 0;
    const int total = nsteps * p.kv_group;

    Stager<D, 0, 0, ROWS, NTH, E> qst;   // rotated and scaled beforehand (or scaled at staging)
    Stager<D, 0, 0, ROWS, NTH, E> dost;
    float lse_r = 0.f, dl_r = 0.f;   // thread tid < ROWS: row tid of the tile
    auto fetch = [&](int t) {
        const int g = t / nsteps;
        const int64_t i = i0 + (int64_t)(t % nsteps) * ROWS;
        const int64_t bh = (int64_t)b * p.H + kvh * p.kv_group + g;
        const int valid = p.Sq - i < ROWS ? (int)(p.Sq - i) : ROWS;
        qst.fetch(p.q + (bh * p.Sq + i) * D, valid, 0, nullptr, nullptr, tid);
        dost.fetch(p.dout + (bh * p.Sq + i) * D, valid, 0, nullptr, nullptr, tid);
        if (tid < ROWS) {
            const bool ok = tid < valid;
            lse_r = ok ? p.lse[bh * p.Sq + i + tid] * LOG2E : INFINITY;   // invalid rows: P = 0
            dl_r = ok ? p.delta[bh * p.Sq + i + tid] : 0.f;
        }
    };
    auto store = [&](int buf) {
        qst.template store<P>(q_lds[buf], ROTD > 0 ? 1.f : p.sl2, tid);
        dost.template store<P>(do_lds[buf], 1.f, tid);
        if (tid < ROWS) {
            lse_lds[buf][tid] = lse_r;
            dl_lds[buf][tid] = dl_r;
        }
    };

    if (total > 0) {
        fetch(0);
        store(0);
        if (total > 1) fetch(1);
        __syncthreads();
    }
    for (int t = 0; t < total; ++t) {
        const int buf = t & 1;
        // this half's 32 rows of the tile
        const int64_t i = i0 + (int64_t)(t % nsteps) * ROWS + TILE * half;
        const uint16_t *qt_lds = q_lds[buf] + TILE * half * P, *dot_lds = do_lds[buf] + TILE * half * P;
        const float *lse_h = lse_lds[buf] + TILE * half, *dl_h = dl_lds[buf] + TILE * half;
        // S - lse (queries x keys) and dP - delta = dO V^T - delta, the
        // accumulators seeded with the row statistics: a lane owns key
        // column l32, its accumulator element 4 ii + j row 8 ii + 4 hh + j
        f32x16_t s, dp;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const float4 l4 = *reinterpret_cast<const float4 *>(lse_h + 8 * ii + 4 * hh);
            const float4 d4 = *reinterpret_cast<const float4 *>(dl_h + 8 * ii + 4 * hh);
            s[4 * ii] = -l4.x; s[4 * ii + 1] = -l4.y; s[4 * ii + 2] = -l4.z; s[4 * ii + 3] = -l4.w;
            dp[4 * ii] = -d4.x; dp[4 * ii + 1] = -d4.y; dp[4 * ii + 2] = -d4.z; dp[4 * ii + 3] = -d4.w;
        }
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const V8<E> aq = *reinterpret_cast<const V8<E> *>(qt_lds + l32 * P + 16 * st + 8 * hh);
            s = mfma<E>(aq, kb[st], s);
            const V8<E> ao = *reinterpret_cast<const V8<E> *>(dot_lds + l32 * P + 16 * st + 8 * hh);
            dp = mfma<E>(ao, vb[st], dp);
        }
        float pv[16], dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(s[r]);
        // the mask only where the diagonal crosses the wave's 32 x 32 block
        // (a wave-uniform test): row offset r sees this lane's key iff r >= thr
        if (p.causal && p.k_off + kt * (int64_t)WG_ROWS + wv * WROWS + WROWS - 1 > p.q_off + i) {
            const int64_t t64 = p.k_off + key - p.q_off - i;
            const int thr = t64 < -1 ? -1 : (t64 > WROWS ? WROWS : (int)t64);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + 4 * hh + (r & 3) < thr) pv[r] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dsv[r] = pv[r] * dp[r];
        // dV^T += dO^T P,  dK^T += Q'^T dS
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const V8<E> bp = acc_operand<E>(pv, mm), bs = acc_operand<E>(dsv, mm);
#pragma unroll
            for (int bd = 0; bd < DB; ++bd) {
                dv[bd] = mfma<E>(tr_operand<P, E>(dot_lds, mm, bd, tr_row0, tr_col), bp, dv[bd]);
                dk[bd] = mfma<E>(tr_operand<P, E>(qt_lds, mm, bd, tr_row0, tr_col), bs, dk[bd]);
            }
        }
        if (t + 1 < total) store(buf ^ 1);
        if (t + 2 < total) fetch(t + 2);
        __syncthreads();
    }

    if constexpr (NH == 2) {
        float *xbuf = reinterpret_cast<float *>(smem);
        fold_halves<DB>(dk, xbuf, half, wv, lane);
        fold_halves<DB>(dv, xbuf, half, wv, lane);
    }
    if (half != 0 || !kvalid) return;
    // dK' = scale dS^T Q' = ln 2 * (dS^T (scale log2(e) Q')), then back to K's frame
    unrotate<D, LAYOUT, ROTD>(dk, p.k_off + key, p.cos_tab, p.sin_tab, hh);
    store_row<D, E>(p.dk + ((int64_t)bkv * p.Sk + key) * D, dk, LN2, hh);
    store_row<D, E>(p.dv + ((int64_t)bkv * p.Sk + key) * D, dv, 1.f, hh);
}

// ---------------------------------------------------------------------------
// dQ: 128 query rows of one (batch, head) per workgroup; blk orders the tiles
// heaviest first (with the causal mask the last rows see the most keys).
template <int D, int LAYOUT, int ROTD, typename E>
__device__ __forceinline__ void dq_block(const BwdParams &p, int blk, unsigned char *smem)
{
    constexpr int NH = Halves<D>::NH, NTH = 256 * NH, ROWS = TILE * NH;
    constexpr int P = D + 8;
    constexpr int NS = D / 16, DB = D / 32, TE = Lds<D>::TILE_ELEMS;
    uint16_t(*k_lds)[TE] = reinterpret_cast<uint16_t(*)[TE]>(smem);
    uint16_t(*v_lds)[TE] = reinterpret_cast<uint16_t(*)[TE]>(smem + 2 * TE * 2);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = wave >> 2, wv = wave & 3;
    const int l32 = lane & 31, hh = lane >> 5;
    const int BH = p.B * p.H;
    const int bh = blk % BH;
    const int qt = p.n_qtiles - 1 - blk / BH;
    const int64_t qi = (int64_t)qt * WG_ROWS + wv * WROWS + l32;   // this lane's query row
    const bool qvalid = qi < p.Sq;
    const int64_t bkv = bh / p.kv_group;
    const int g16 = lane >> 4, lp = lane & 15;
    const int tr_row0 = 4 * (g16 >> 1) + (lp >> 2), tr_col = 4 * (lp & 3) + 16 * (g16 & 1);

    V8<E> qb[NS], ob[NS];
    row_operand<D, 0, 0, E>(p.q + ((int64_t)bh * p.Sq + qi) * D, qvalid, 0, ROTD > 0 ? 1.f : p.sl2, nullptr,
                            nullptr, hh, qb);
    row_operand<D, 0, 0, E>(p.dout + ((int64_t)bh * p.Sq + qi) * D, qvalid, 0, 1.f, nullptr, nullptr, hh, ob);
    const float lse2 = qvalid ? p.lse[(int64_t)bh * p.Sq + qi] * LOG2E : INFINITY;
    const float dl = qvalid ? p.delta[(int64_t)bh * p.Sq + qi] : 0.f;
    f32x16_t dq[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dq[i] = (f32x16_t){};

    // keys the tile's last row sees
    int64_t nk = p.Sk;
    if (p.causal) {
        const int64_t last = (int64_t)qt * WG_ROWS + WG_ROWS - 1 < p.Sq ? (int64_t)qt * WG_ROWS + WG_ROWS - 1 : p.Sq - 1;
        const int64_t vis = p.q_off + last - p.k_off + 1;
        nk = vis < nk ? vis : nk;
    }
    const int total = nk > 0 ? (int)((nk + ROWS - 1) / ROWS) : 0;

    Stager<D, 0, 0, ROWS, NTH, E> kst;   // rotated beforehand
    Stager<D, 0, 0, ROWS, NTH, E> vst;
    const uint16_t *kh = p.k + bkv * p.Sk * D, *vh = p.v + bkv * p.Sk * D;
    auto fetch = [&](int t) {
        const int64_t j = (int64_t)t * ROWS;
        const int valid = p.Sk - j < ROWS ? (int)(p.Sk - j) : ROWS;
        kst.fetch(kh + j * D, valid, 0, nullptr, nullptr, tid);
        vst.fetch(vh + j * D, valid, 0, nullptr, nullptr, tid);
    };
    auto store = [&](int buf) {
        kst.template store<P>(k_lds[buf], 1.f, tid);
        vst.template store<P>(v_lds[buf], 1.f, tid);
    };

    if (total > 0) {
        fetch(0);
        store(0);
        if (total > 1) fetch(1);
        __syncthreads();
    }
    for (int t = 0; t < total; ++t) {
        const int buf = t & 1;
        // this half's 32 keys of the tile
        const int64_t j0 = (int64_t)t * ROWS + TILE * half;
        const uint16_t *kt_lds = k_lds[buf] + TILE * half * P, *vt_lds = v_lds[buf] + TILE * half * P;
        // S^T - lse and dP^T - delta (keys x queries), the accumulators
        // seeded with this lane's row statistics: a lane owns query column l32
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = -lse2;
            dp[r] = -dl;
        }
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const V8<E> ak = *reinterpret_cast<const V8<E> *>(kt_lds + l32 * P + 16 * st + 8 * hh);
            s = mfma<E>(ak, qb[st], s);
            const V8<E> av = *reinterpret_cast<const V8<E> *>(vt_lds + l32 * P + 16 * st + 8 * hh);
            dp = mfma<E>(av, ob[st], dp);
        }
        float pr[16], dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r]);
        // key offset c of the block is visible iff c <= lim: the mask only
        // where the diagonal or the end of the keys crosses the wave's block
        // (a wave-uniform test)
        if (j0 + WROWS > p.Sk ||
            (p.causal && p.k_off + j0 + WROWS - 1 > p.q_off + (int64_t)qt * WG_ROWS + wv * WROWS)) {
            int64_t l64 = p.Sk - 1 - j0;
            if (p.causal && p.q_off + qi - p.k_off - j0 < l64) l64 = p.q_off + qi - p.k_off - j0;
            const int lim = l64 < -1 ? -1 : (l64 > WROWS ? WROWS : (int)l64);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + 4 * hh + (r & 3) > lim) pr[r] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dsv[r] = pr[r] * dp[r];
        // dQ^T += K'^T dS
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const V8<E> bs = acc_operand<E>(dsv, mm);
#pragma unroll
            for (int bd = 0; bd < DB; ++bd)
                dq[bd] = mfma<E>(tr_operand<P, E>(kt_lds, mm, bd, tr_row0, tr_col), bs, dq[bd]);
        }
        if (t + 1 < total) store(buf ^ 1);
        if (t + 2 < total) fetch(t + 2);
        __syncthreads();
    }

    if constexpr (NH == 2) fold_halves<DB>(dq, reinterpret_cast<float *>(smem), half, wv, lane);
    if (half != 0 || !qvalid) return;
    // dQ' = scale dS K', then back to Q's frame
    unrotate<D, LAYOUT, ROTD>(dq, p.q_off + qi, p.cos_tab, p.sin_tab, hh);
    store_row<D, E>(p.dq + ((int64_t)bh * p.Sq + qi) * D, dq, p.scale, hh);
}

// dK/dV and dQ workgroups in one launch: the two lists, each heaviest first,
// interleaved, so that light tiles of one fill in around heavy tiles of the
// other (with the causal mask the heavy dK/dV tiles are the light dQ tiles).
template <int D, int LAYOUT, int ROTD, typename E>
__global__ __launch_bounds__(256 * Halves<D>::NH) void bwd_main_kernel(BwdParams p, int n_dkv, int n_dq)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[Lds<D>::BYTES];
    const int blk = blockIdx.x;
    const int m = n_dkv < n_dq ? n_dkv : n_dq;
    if (blk < 2 * m) {
        if (blk & 1) dq_block<D, LAYOUT, ROTD, E>(p, blk >> 1, smem);
        else dkv_block<D, LAYOUT, ROTD, E>(p, blk >> 1, smem);
    } else if (n_dkv > n_dq) {
        dkv_block<D, LAYOUT, ROTD, E>(p, blk - m, smem);
    } else {
        dq_block<D, LAYOUT, ROTD, E>(p, blk - m, smem);
    }
}

template <int D, int LAYOUT, int ROTD, typename E>
int launch_all(BwdParams p, uint16_t *qr, uint16_t *kr, hipStream_t stream)
{
    const int64_t rows = (int64_t)p.B * p.H * p.Sq;
    constexpr int RPB = 256 / (D / 8);
    const int64_t ndelta = (rows + RPB - 1) / RPB;
    constexpr int NTH = 256 * Halves<D>::NH;
    const int64_t n_dkv = (int64_t)p.B * p.Hkv * p.n_ktiles, n_dq = (int64_t)p.B * p.H * p.n_qtiles;
    const int64_t nrot = ROTD > 0 ? (int64_t)p.B * p.H * ((p.Sq + TILE - 1) / TILE) +
                                        (int64_t)p.B * p.Hkv * ((p.Sk + TILE - 1) / TILE)
                                  : 0;
    if (!rope_grid_fits(nrot + ndelta, 256) || !rope_grid_fits(n_dkv + n_dq, NTH)) return ROPE_LAUNCH_SHAPE;
    if constexpr (ROTD > 0) {
        // rotation tiles, then the row sums, in one launch
        hipLaunchKernelGGL((bwd_rotate_kernel<D, LAYOUT, ROTD, E>), dim3((unsigned)(nrot + ndelta)), dim3(256), 0,
                           stream, p, p.q, p.k, qr, kr);
        if (hipGetLastError() != hipSuccess) return ROPE_LAUNCH_ERR;
        p.q = qr;
        p.k = kr;
    } else {
        hipLaunchKernelGGL((bwd_delta_kernel<D, E>), dim3((unsigned)ndelta), dim3(256), 0, stream, p.o, p.dout,
                           p.delta, rows);
        if (hipGetLastError() != hipSuccess) return ROPE_LAUNCH_ERR;
    }
    hipLaunchKernelGGL((bwd_main_kernel<D, LAYOUT, ROTD, E>), dim3((unsigned)(n_dkv + n_dq)), dim3(NTH), 0, stream,
                       p, (int)n_dkv, (int)n_dq);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

template <int D, int ROTD, typename E>
int launch_rot(const BwdParams &p, int layout, uint16_t *qr, uint16_t *kr, hipStream_t stream)
{
    if constexpr (ROTD == 0) return launch_all<D, 0, 0, E>(p, qr, kr, stream);
    else
        return layout == 0 ? launch_all<D, 0, ROTD, E>(p, qr, kr, stream)
                           : launch_all<D, 1, ROTD, E>(p, qr, kr, stream);
}

template <typename E>
int launch_typed(const BwdParams &p, int head_dim, int rot_dim, int layout, uint16_t *qr, uint16_t *kr,
                 hipStream_t stream)
{
    if (head_dim == 64) {
        switch (rot_dim) {
        case 0: return launch_rot<64, 0, E>(p, layout, qr, kr, stream);
        case 32: return launch_rot<64, 32, E>(p, layout, qr, kr, stream);
        case 64: return launch_rot<64, 64, E>(p, layout, qr, kr, stream);
        default: return ROPE_LAUNCH_ERR;
        }
    }
    switch (rot_dim) {
    case 0: return launch_rot<128, 0, E>(p, layout, qr, kr, stream);
    case 32: return launch_rot<128, 32, E>(p, layout, qr, kr, stream);
    case 64: return launch_rot<128, 64, E>(p, layout, qr, kr, stream);
    case 96: return launch_rot<128, 96, E>(p, layout, qr, kr, stream);
    case 128: return launch_rot<128, 128, E>(p, layout, qr, kr, stream);
    default: return ROPE_LAUNCH_ERR;
    }
}

}  // namespace

// The row sums dO.O (fp32), then, with rotation, the rotated copies of q and
// k (E), each from a 256-byte boundary.
namespace {
int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }
}
int64_t rope_flash_bwd_workspace_bytes(int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim, int rot_dim)
{
    int64_t n = round256((int64_t)B * H * Sq * 4);
    if (rot_dim > 0) n += round256((int64_t)B * H * Sq * head_dim * 2) + round256((int64_t)B * H_kv * Sk * head_dim * 2);
    return n;
}

int rope_launch_flash_bwd_bf16(const FlashBwdArgs &a, hipStream_t stream)
{
    BwdParams p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<const uint16_t *>(a.o);
    p.dout = static_cast<const uint16_t *>(a.dout);
    p.lse = a.lse;
    p.delta = static_cast<float *>(a.workspace);
    char *const ws = static_cast<char *>(a.workspace);
    const int64_t q_at = round256((int64_t)a.B * a.H * a.Sq * 4);
    uint16_t *const qr = reinterpret_cast<uint16_t *>(ws + q_at);
    uint16_t *const kr = reinterpret_cast<uint16_t *>(ws + q_at + round256((int64_t)a.B * a.H * a.Sq * a.head_dim * 2));
    p.dq = static_cast<uint16_t *>(a.dq);
    p.dk = static_cast<uint16_t *>(a.dk);
    p.dv = static_cast<uint16_t *>(a.dv);
    p.cos_tab = a.cos_tab;
    p.sin_tab = a.sin_tab;
    p.Sq = a.Sq; p.Sk = a.Sk; p.q_off = a.q_off; p.k_off = a.k_off;
    p.B = a.B; p.H = a.H; p.Hkv = a.H_kv; p.kv_group = a.H / a.H_kv; p.causal = a.causal;
    p.n_qtiles = (int)((a.Sq + WG_ROWS - 1) / WG_ROWS);
    p.n_ktiles = (int)((a.Sk + WG_ROWS - 1) / WG_ROWS);
    p.scale = a.scale;
    p.sl2 = a.scale * LOG2E;
    // dtype 0 (bf16) or 2 (fp16): the same kernels over either 16-bit type
    return a.dtype == 2 ? launch_typed<_Float16>(p, a.head_dim, a.rot_dim, a.layout, qr, kr, stream)
                        : launch_typed<__bf16>(p, a.head_dim, a.rot_dim, a.layout, qr, kr, stream);
}
