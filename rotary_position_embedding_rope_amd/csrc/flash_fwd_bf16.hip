// flash_fwd_bf16.hip -- fused RoPE + softmax attention forward on the gfx950
// matrix cores (bf16 inputs, fp32 accumulation).
//
// Operation: O = softmax(scale * rope(Q) rope(K)^T + mask) V per (batch,
// head) ("RoPE and FlashAttention: relative positions and online softmax",
// section 4), evaluated with the online-softmax recurrence of section 5
// (running max m, denominator l, unnormalised numerator; rescale when the
// max rises; a key tile with no visible key leaves a row untouched; divide
// once at the end).  Query i sits at position q_off + i, key j at k_off + j;
// with the causal mask, key j is visible iff k_off + j <= q_off + i
// (section 6's offset mask).  Rotation pairs and formula: "Write Triton Rope
// Kernel", "Required reasoning process" steps 1 and 6.
//
// Work decomposition (FlashAttention-2 style, the same page's section 7: a
// query-block outer loop, key/value inner loop, output written once):
//   * a workgroup owns 128 query rows of one (batch, head): two 64-row
//     halves.  With the causal mask these are half-tiles r and n - 1 - r of
//     the query range, a light and a heavy one, so all workgroups see about
//     the same number of key tiles (the causal triangle is folded instead of
//     leaving the last query tiles as the critical path); otherwise they are
//     128 consecutive rows.  Two key groups of 4 waves walk interleaved key
//     tiles over the same rows and are merged through LDS at the end, each
//     group merging and storing one 32-dim half of O.  Every SIMD runs two
//     waves, one per half, so one wave's softmax overlaps the other's
//     matrix-core work and the heavy half's tiles are spread over all four
//     SIMDs;
//   * in each group a wave owns 32 query rows; the key loop stops at the
//     last tile a query of the workgroup can see, tiles past a wave's last
//     query are skipped by that wave (it keeps staging for the others), and
//     the element mask runs only on tiles straddling the diagonal or the
//     ragged end;
//   * all workgroups of one head go to one XCD (block index modulo the head
//     count), so a head's K/V stay in one L2.
//
// Data path of a group:
//   * Q: in group 0 each lane loads its query row's dims straight into the
//     matrix-core operand layout, rotates them in fp32 at q_off + i,
//     multiplies by scale*log2(e), rounds to bf16 and keeps the tile in
//     registers; it also leaves it in LDS, where the group-1 wave holding
//     the same rows picks it up after the first barrier (each query row is
//     loaded and rotated once per workgroup).
//   * K: every visited tile is loaded from HBM once (into registers, a tile
//     ahead), rotated in fp32 at its key positions, rounded to bf16 and
//     written to LDS -- rotated once per staging, never written back to HBM
//     ("RoPE + PoPE Attention Kernels": recompute instead of materialising
//     rotated [B,H,S,D] tensors).  V goes unrotated from HBM straight into
//     LDS (buffer loads with the LDS bit), row-major with swizzled 16-byte
//     chunks.  Two K and two V buffers per group; one barrier per tile.
//   * S = K Q'^T on v_mfma_f32_32x32x16_bf16: a lane owns one query column,
//     so row max / row sum are in-lane plus one v_permlane32_swap.
//     P = exp2(S - m) against a per-row reference m that stays 0 while the
//     row's scores (log2 units) lie in [-64, 8], so the common path needs
//     no per-score subtraction.
//   * The reference is raised lazily: only when a row's scores exceed it by
//     more than 8 (or its first visible scores all lie below -64) is it
//     raised to the row max and O, l rescaled -- exact in real arithmetic
//     since numerator and denominator share the reference.
//   * P is rounded to bf16; its row sums use v_dot2_f32_bf16 on those same
//     bf16 values, so numerator and denominator see identical weights.  P
//     leaves the accumulator already in the B-operand layout of
//     O^T = V^T P^T; the V^T operand comes from ds_read_b64_tr_b16
//     transposing reads of the row-major V tile.
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace {

using rope::bf16x8_t;
using rope::f32x16_t;
using rope::pack_bf16x2;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int WAVES_PER_GROUP = 4;
constexpr int BM = 32 * WAVES_PER_GROUP;   // queries per workgroup
constexpr int KPAD = 8;                     // K LDS row pitch = D + 8 bf16
constexpr float LAZY_THRESHOLD = 8.0f;      // log2 headroom before the reference max is raised
constexpr float LN2 = 0.6931471805599453f;

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;         // [BH, Sq] natural-log log-sum-exp of each row's scores, or null
    int BH;
    int kv_group;       // query heads per key/value head: K/V head of bh is bh / kv_group
    int64_t Sq, Sk, q_off, k_off;
    const float *cos_tab, *sin_tab;
    int64_t table_rows;
    int rot_dim;
    float sl2;          // softmax scale * log2(e)
    int causal;
    int64_t n_qtiles;
    int64_t n_half;     // 64-row halves of the query range
    int64_t n_kt;       // key tiles
    int tile_n;         // keys per tile
};

// ---- schedule arithmetic (host and device) ----

// Key tiles seen by query rows up to `last` (all key tiles when not causal).
__host__ __device__ inline int64_t row_visits(const Params &p, int64_t last)
{
    if (!p.causal) return p.n_kt;
    const int64_t v = (p.q_off + last - p.k_off) / p.tile_n + 1;
    return v < p.n_kt ? v : p.n_kt;
}

using rope::Ty;

template <typename E>
__device__ __forceinline__ void unpack8(uint4 w, float (&x)[8])
{
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = Ty<E>::lo(ws[i]);
        x[2 * i + 1] = Ty<E>::hi(ws[i]);
    }
}
template <typename E>
__device__ __forceinline__ uint4 pack8(const float (&x)[8])
{
    return make_uint4(Ty<E>::pack2(x[0], x[1]), Ty<E>::pack2(x[2], x[3]), Ty<E>::pack2(x[4], x[5]),
                      Ty<E>::pack2(x[6], x[7]));
}

// Rotate pairs (a[i], b[i]) by (c[i], s[i]): a' = a c - b s, b' = a s + b c.
template <int N>
__device__ __forceinline__ void rotate_pairs(float *a, float *b, const float *c, const float *s)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float x = a[i], y = b[i];
        a[i] = x * c[i] - y * s[i];
        b[i] = x * s[i] + y * c[i];
    }
}

// Instruction order of one iteration's block for the scheduler: matrix op
// I, then the LDS reads of the matrix op two further on (two for a P V op,
// one for a score op), then NVA vector-ALU instructions.
template <int I, int NPV, int NMF, int NVA>
__device__ __forceinline__ void sched_mix()
{
    if constexpr (I < NMF) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one MFMA
        if constexpr (I + 2 < NPV)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // LDS reads
        else if constexpr (I + 2 < NMF)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NVA, 0);       // vector ALU
        sched_mix<I + 1, NPV, NMF, NVA>();
    }
}

// Reductions with the lane 32 apart (the other half of the same query
// column).  v_permlane32_swap leaves {own, partner} in its two results on
// every lane, so the symmetric max / sum is the same on both halves.
__device__ __forceinline__ float max_with_partner(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer access: one descriptor per tensor slice, carrying the slice's
// exact byte length.  A load at or past that length returns zeros, so a
// ragged last tile needs no per-lane row checks and no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_FLAGS = 0x00020000;   // untyped 32-bit buffer (gfx9 family)

// `rows` rows of `row_bytes` bytes from `base` (rows <= 0: empty; lengths
// past 4 GiB are capped, far beyond the few KiB one tile addresses).
template <int ROW_BYTES>
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int rows)
{
    constexpr int MAX_ROWS = (int)(0xffffffffu / ROW_BYTES);
    const uint32_t n = rows <= 0 ? 0u : (rows >= MAX_ROWS ? 0xffffffffu : (uint32_t)rows * ROW_BYTES);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, RSRC_FLAGS);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ float4 bload16f(rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Per-thread staging plan for K tiles (fixed across tiles).  A slot is two
// 8-dim chunks of one key row, D/16 slots per row:
//   NeoX: a rotated pair of chunks (lo at 8c, hi at 8c + rot/2), or two
//         copied chunks past rot_dim;
//   GPT-J: 16 consecutive dims (8 whole pairs), rotated or copied (rot_dim
//         is a multiple of 32, so a slot is never split);
//   no rotation: 16 consecutive dims, copied.
template <int D, int LAYOUT, bool ROT, int BN>
struct KPlan {
    static constexpr bool NEOX_SLOT = ROT && LAYOUT == 0;
    static constexpr int SLOTS_PER_ROW = D / 16;
    static constexpr int SLOTS = BN * SLOTS_PER_ROW;
    static constexpr int ITEMS = (SLOTS + 255) / 256;   // per thread (the last may be empty)
};

struct KItem {
    int row, mode, o0, o1, to;
};

// Row sums of one tile's probabilities (this lane's keys) up to this bound
// are taken without looking at the row max: every probability is then at
// most 2^13, far from fp32/bf16 overflow, and the reference the scores are
// measured against only ever rises.  A larger sum sends the tile to the
// exact path (true row max, lazy rescale).
constexpr float FAST_SUM_LIMIT = 8192.0f;

// D: head dim (64); BN: keys per tile (64); NG: groups of 4 waves per
// workgroup (2): the groups take the same rows and alternate key tiles;
// FULL: rot_dim == D (every K slot rotates).
template <int D, int LAYOUT, bool ROT, bool FULL, int NG, int BN, typename E>
__global__ __launch_bounds__(256 * NG) __attribute__((amdgpu_waves_per_eu(2)))
void flash_fwd_bf16_kernel(Params p)
{
    using TT = Ty<E>;
    using v8 = typename TT::v8;
    static_assert(D == 64 && NG == 2 && BN == 64, "built for head dim 64, two key groups, 64-key tiles");
    using Plan = KPlan<D, LAYOUT, ROT, BN>;
    constexpr int NKB = BN / 32;                    // 32-key blocks per tile
    constexpr int KP = D + KPAD;                    // K LDS row pitch
    // value tiles go from HBM straight into LDS (buffer loads with the LDS
    // bit), unpadded and swizzled (dma_v)
    constexpr int K_ELEMS = BN * KP, V_ELEMS = BN * D;
    constexpr int NST = 256;                        // staging threads per tile: a group
    constexpr int KI = (Plan::SLOTS + NST - 1) / NST;   // K slots per thread per tile
    constexpr int DT = D / 16;                      // k-steps of the QK^T product
    constexpr int DB = D / 32;                      // 32-row blocks of O^T
    constexpr int NBUF = NG;                        // buffer sets (one per key stream)
    constexpr int NVB = 2;                          // V buffers per set

    // [stream][buffer] K tiles, then [stream][buffer] V tiles.  K runs one
    // tile ahead of V: while tile t's probabilities are formed, the scores of
    // the next tile are computed from the other K buffer.  Then the rotated
    // query operand of the workgroup's rows, [wave][k-step][lane] 16 bytes
    // each: group 0 forms it, group 1 (same rows) reads it.
    constexpr int KV_ELEMS = NBUF * (2 * K_ELEMS + NVB * V_ELEMS);
    constexpr int QX_ELEMS = WAVES_PER_GROUP * DT * 64 * 8;
    __shared__ __attribute__((aligned(16))) uint16_t lds[KV_ELEMS + QX_ELEMS];

    const int tid = threadIdx.x;
    // group and wave are uniform across a wave; saying so keeps every
    // tile-level quantity (and the buffer descriptors) in scalar registers
    const int group = __builtin_amdgcn_readfirstlane(tid >> 8);
    const int gtid = tid & 255;                     // thread index inside the group
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(gtid >> 6);   // wave inside the group
    const int l32 = lane & 31, hh = lane >> 5;
    const int rh = p.rot_dim / 2;   // table row stride
    const int stream = group;
    auto kbuf = [&](int b) { return lds + (stream * 2 + b) * K_ELEMS; };
    auto vbuf = [&](int b) { return lds + NBUF * 2 * K_ELEMS + (stream * NVB + b) * V_ELEMS; };
    auto vslot = [&](int j) { return j & 1; };   // V buffer of tile T(j)

    // ---------------- staging plans ----------------
    // A K item is one slot of a key row: mode -1 no slot, 0 copy, 1 NeoX
    // rotate (lo, hi), 2 GPT-J rotate; o0/o1 = element offsets of its two
    // chunks inside a K tile, to = offset of its cos/sin slice inside the
    // tile's block of table rows.  A V item is one 16-byte chunk.
    auto k_item = [&](int item) {
        KItem it;
        int row = item / Plan::SLOTS_PER_ROW;
        int slot = item % Plan::SLOTS_PER_ROW;
        if constexpr (D == 64) {
            // 16 consecutive items (one pass of a 128-bit LDS write) take 4
            // slots of 4 rows chosen so that their chunks cover the 64 banks
            // once (row pitch 36 dwords): rows r + {0, 4, 8, 12} when the
            // chunks sit at dword 4 slot (+16), rows r + {0, 1, 8, 9} when
            // they sit at dword 8 slot (+4).  A wave still covers 16 whole
            // rows, so the global loads are unchanged.
            const int q = item >> 4, k = item & 15;
            slot = k & 3;
            if constexpr (Plan::NEOX_SLOT && FULL)
                row = 16 * (q >> 2) + (q & 3) + 4 * (k >> 2);
            else
                row = 16 * (q >> 2) + 2 * (q & 3) + ((k >> 2) & 1) + 8 * (k >> 3);
        }
        int d0 = 0, d1 = 0;
        it.row = row;
        if (item >= Plan::SLOTS) {
            it.mode = -1;
        } else if constexpr (Plan::NEOX_SLOT) {
            const int rslots = p.rot_dim / 16;
            if (slot < rslots) {
                it.mode = 1;                            // rotate (lo, hi)
                d0 = 8 * slot;
                d1 = 8 * slot + rh;
            } else {
                it.mode = 0;                            // copy two chunks
                d0 = p.rot_dim + 16 * (slot - rslots);
                d1 = d0 + 8;
            }
        } else {
            it.mode = (ROT && 16 * slot < p.rot_dim) ? 2 : 0;
            d0 = 16 * slot;
            d1 = d0 + 8;
        }
        it.o0 = row * D + d0;
        it.o1 = row * D + d1;
        it.to = row * rh + (LAYOUT == 0 ? d0 : d0 / 2);
        return it;
    };
    // Plan A: the threads of a key stream share the staging of a tile.
    KItem kpa[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) kpa[i] = k_item(gtid + NST * i);

    // V^T operand addressing for ds_read_b64_tr_b16: in each 16-lane group
    // the source lane 4j + b points at V[key0 + j][dim0 + 4b]; the receiving
    // lane l' then holds V[key0 .. key0+3][dim0 + l'].
    const int g16 = lane >> 4, lp = lane & 15;
    const int tr_row = lp >> 2, tr_col = 4 * (lp & 3) + 16 * (g16 & 1);
    const int tr_key = 4 * (g16 >> 1) + tr_row;   // + 32kb + 16mm (+ 8)
    // V layout: column offset of dims 32 bd + tr_col in a key row whose
    // chunks are swizzled by 4 ((key >> 1) & 1) (the key's low bits are tr_row)
    int vcol[D / 32];
#pragma unroll
    for (int bd = 0; bd < D / 32; ++bd)
        vcol[bd] = 8 * ((4 * bd + (tr_col >> 3)) ^ (4 * ((tr_row >> 1) & 1))) + (tr_col & 7);

    // One segment: key tiles [kb, ke) of the 128 query rows made of two
    // 64-row halves starting at rowA and rowB (rowB >= Sq: no second half)
    // of head `bh`, every key tile those rows see.
    // Wave w of group 0 takes half (w >> 1) & 1, rows 32 (w & 1) of it; group
    // 1 takes the other half on each SIMD, so a SIMD's two waves work on
    // different halves.
    auto segment = [&](int bh, int64_t rowA, int64_t rowB, int64_t kb, int64_t ke) {
        const int half = ((wave >> 1) ^ group) & 1;
        const int64_t wq0 = (half ? rowB : rowA) + 32 * (wave & 1);   // first row of this wave
        const uint16_t *qh = p.q + (int64_t)bh * p.Sq * D;
        // (b H + h) / G = b H_kv + h / G: the key/value head of query head h
        const uint16_t *kh = p.k + (int64_t)(bh / p.kv_group) * p.Sk * D;
        const uint16_t *vh = p.v + (int64_t)(bh / p.kv_group) * p.Sk * D;
        const int sk32 = (int)p.Sk;
        // cos/sin rows of this segment's keys start at position k_off; table
        // rows from there on, capped at the int range
        const float *ctab = ROT ? p.cos_tab + p.k_off * rh : nullptr;
        const float *stab = ROT ? p.sin_tab + p.k_off * rh : nullptr;
        const int64_t trk = p.table_rows - p.k_off;
        const int tab_rows_k = (int)(trk < 0x7fffffffLL ? trk : 0x7fffffffLL);

        // Group g takes tiles kb + g, kb + g + NG, ...: iteration j of the
        // group handles tile T(j) = kb + j NG + g, whose K sits in K buffer
        // j & 1 and whose V sits in V buffer j & 1.
        constexpr int TS = NG;   // tile stride of a key stream
        const int n_iter = (int)((ke - kb + TS - 1) / TS);
        const int t0 = (int)kb + group;
        const int tend = (int)ke;
        auto T = [&](int j) { return t0 + j * TS; };

        // ---- K/V loads and staging ----
        // Global loads of key tile kt's K items (with their table rows) and
        // of value tile kt's V items into the given registers.  Rows past Sk
        // (and table rows past the table) read as zeros.
        auto fetch_k = [&](int kt, const auto &ki, auto &r0, auto &r1, auto &c, auto &s) {
            constexpr int N = sizeof(ki) / sizeof(ki[0]);
            const int j0 = kt * BN;
            const rsrc_t krs = make_rsrc<2 * D>(kh + (int64_t)j0 * D, sk32 - j0);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (ki[i].mode < 0) continue;
                r0[i] = bload16(krs, 2 * ki[i].o0);
                r1[i] = bload16(krs, 2 * ki[i].o1);
            }
            if constexpr (ROT) {
                // table rows are rot_dim/2 floats; descriptors count 16-byte
                // units (rh is a multiple of 16)
                const int left = tab_rows_k - j0;   // a tile reads at most BN of them
                const int trows = (left < BN ? left : BN) * (rh / 4);
                const rsrc_t crs = make_rsrc<16>(ctab + (int64_t)j0 * rh, trows);
                const rsrc_t srs = make_rsrc<16>(stab + (int64_t)j0 * rh, trows);
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    if (ki[i].mode < 0) continue;
                    const int to = 4 * ki[i].to;
                    *reinterpret_cast<float4 *>(c[i]) = bload16f(crs, to);
                    *reinterpret_cast<float4 *>(s[i]) = bload16f(srs, to);
                    *reinterpret_cast<float4 *>(c[i] + 4) = bload16f(crs, to + 16);
                    *reinterpret_cast<float4 *>(s[i] + 4) = bload16f(srs, to + 16);
                }
            }
        };
        // Blocks [blk0, blk0 + NBLK) of value tile kt straight into V
        // buffer b.  A block is 8 rows = 1 KB of LDS, written by one buffer
        // load of the wave: lane q (LDS bytes 16q .. 16q+15 of the block)
        // takes row q/8 of the block and 16-byte chunk (q%8) ^ 4((q/16)&1)
        // of that row, so that the 4 keys a transposing read of P V fetches
        // at once sit in 4 different 16-bank groups.  Rows past Sk (and
        // tiles past the segment) are written as zeros.  The loads complete
        // asynchronously: the issuing wave waits for them (vmcnt) before the
        // barrier that hands the tile over.
        auto dma_v = [&](int kt, int b, int blk0, auto NBLK) {
            const int j0 = kt * BN;
            const int rows = kt < tend ? sk32 - j0 : 0;
            const rsrc_t vrs = make_rsrc<2 * D>(vh + (int64_t)j0 * D, rows);
            const int r = lane >> 3, c = (lane & 7) ^ (4 * ((r >> 1) & 1));
#pragma unroll
            for (int i = 0; i < decltype(NBLK)::value; ++i) {
                const int blk = blk0 + i;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    vrs, (__attribute__((address_space(3))) void *)(vbuf(b) + blk * 8 * D), 16,
                    2 * ((8 * blk + r) * D + 8 * c), 0, 0, 0);
            }
        };
        // Rotate fetched K items in fp32 at their key positions, round to
        // bf16 and write them to K buffer b; write fetched V items to V
        // buffer b.
        auto stage_k = [&](int b, const auto &ki, const auto &r0, const auto &r1, const auto &c,
                           const auto &s) {
            constexpr int N = sizeof(ki) / sizeof(ki[0]);
            uint16_t *kdst = kbuf(b);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (ki[i].mode < 0) continue;
                // LDS rows have pitch KP; the chunk offsets inside a row are
                // o - row * D.
                uint16_t *row = kdst + ki[i].row * (KP - D);
                uint4 w0 = r0[i], w1 = r1[i];
                // slots past rot_dim rotate by angle 0 (cos 1, sin 0), which
                // gives back their input values
                const bool rot_slot = FULL || ki[i].mode != 0;
                if constexpr (ROT && LAYOUT == 0) {
                    float lo[8], hi[8], cc[8], ss[8];
                    unpack8<E>(r0[i], lo);
                    unpack8<E>(r1[i], hi);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        cc[u] = rot_slot ? c[i][u] : 1.f;
                        ss[u] = rot_slot ? s[i][u] : 0.f;
                    }
                    rotate_pairs<8>(lo, hi, cc, ss);
                    w0 = pack8<E>(lo);
                    w1 = pack8<E>(hi);
                } else if constexpr (ROT && LAYOUT == 1) {
                    // chunk h holds pairs 4h .. 4h+3 of the slot's 8
                    float x[2][8];
                    unpack8<E>(r0[i], x[0]);
                    unpack8<E>(r1[i], x[1]);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float a[4], bb[4], cc[4], ss[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            a[u] = x[h][2 * u]; bb[u] = x[h][2 * u + 1];
                            cc[u] = rot_slot ? c[i][4 * h + u] : 1.f;
                            ss[u] = rot_slot ? s[i][4 * h + u] : 0.f;
                        }
                        rotate_pairs<4>(a, bb, cc, ss);
#pragma unroll
                        for (int u = 0; u < 4; ++u) { x[h][2 * u] = a[u]; x[h][2 * u + 1] = bb[u]; }
                    }
                    w0 = pack8<E>(x[0]);
                    w1 = pack8<E>(x[1]);
                }
                *reinterpret_cast<uint4 *>(row + ki[i].o0) = w0;
                *reinterpret_cast<uint4 *>(row + ki[i].o1) = w1;
            }
        };

        // Plan A registers: one K tile of this group in flight.
        uint4 kr0[KI], kr1[KI];
        float kc[KI][8], ks[KI][8];
        // The first two key tiles, the query rows and their table rows are
        // all requested before any of them is used, so their latencies
        // overlap (rows past Sq, or past the table, read as zeros).
        v8 qf[DT];
        {
            uint4 pr0[KI], pr1[KI];
            float pc[KI][8], ps[KI][8];
            if (T(0) < tend) {
                fetch_k(T(0), kpa, kr0, kr1, kc, ks);
                dma_v(T(0), 0, 2 * wave, std::integral_constant<int, 2>{});
            }
            if (T(1) < tend) fetch_k(T(1), kpa, pr0, pr1, pc, ps);

            // ---- Q: load, rotate, scale, keep as MFMA B operand ----
            // Group 0 only: group 1 holds the same rows (its wave w those of
            // group 0's wave w ^ 2) and reads the operand from LDS after
            // the first barrier.
            if (group == 0) {
                const int64_t qleft = p.Sq - wq0;
                const rsrc_t qrs = make_rsrc<2 * D>(qh + wq0 * D, (int)(qleft < 0 ? 0 : (qleft > 32 ? 32 : qleft)));
                float qv[DT][8];
#pragma unroll
                for (int t = 0; t < DT; ++t) unpack8<E>(bload16(qrs, 2 * (l32 * D + 16 * t + 8 * hh)), qv[t]);
                if constexpr (ROT) {
                    const int64_t tleft = p.table_rows - (p.q_off + wq0);
                    const int trows = (int)(tleft < 0 ? 0 : (tleft > 32 ? 32 : tleft)) * (rh / 4);
                    const rsrc_t qcs = make_rsrc<16>(p.cos_tab + (p.q_off + wq0) * rh, trows);
                    const rsrc_t qss = make_rsrc<16>(p.sin_tab + (p.q_off + wq0) * rh, trows);
                    const int tb = 4 * l32 * rh;   // byte offset of this lane's table row
                    if constexpr (LAYOUT == 0) {
                        // lane holds dims 16t + 8hh + s; the partner of
                        // 16t+8hh+s is 16(t + rot/32) + 8hh + s, in the same
                        // lane (rot_dim is a multiple of 32: tr <= DT/2).
                        const int tr = p.rot_dim / 32;
#pragma unroll
                        for (int t = 0; t < DT / 2; ++t) {
                            if (t < tr) {
                                const int f0 = 4 * (16 * t + 8 * hh);
                                float c[8], s[8];
                                *reinterpret_cast<float4 *>(c) = bload16f(qcs, tb + f0);
                                *reinterpret_cast<float4 *>(c + 4) = bload16f(qcs, tb + f0 + 16);
                                *reinterpret_cast<float4 *>(s) = bload16f(qss, tb + f0);
                                *reinterpret_cast<float4 *>(s + 4) = bload16f(qss, tb + f0 + 16);
                                // registers are only indexed with compile-time constants
#pragma unroll
                                for (int u = 1; u <= DT / 2; ++u)
                                    if (u == tr) rotate_pairs<8>(qv[t], qv[t + u], c, s);
                            }
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < DT; ++t) {
                            if (16 * t < p.rot_dim) {
                                const int f0 = 4 * (8 * t + 4 * hh);
                                float c[4], s[4], a[4], b[4];
                                *reinterpret_cast<float4 *>(c) = bload16f(qcs, tb + f0);
                                *reinterpret_cast<float4 *>(s) = bload16f(qss, tb + f0);
#pragma unroll
                                for (int u = 0; u < 4; ++u) { a[u] = qv[t][2 * u]; b[u] = qv[t][2 * u + 1]; }
                                rotate_pairs<4>(a, b, c, s);
#pragma unroll
                                for (int u = 0; u < 4; ++u) { qv[t][2 * u] = a[u]; qv[t][2 * u + 1] = b[u]; }
                            }
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < DT; ++t) {
#pragma unroll
                    for (int s = 0; s < 8; ++s) qf[t][s] = (E)(qv[t][s] * p.sl2);
                    *reinterpret_cast<v8 *>(lds + KV_ELEMS + ((wave * DT + t) * 64 + lane) * 8) = qf[t];
                }
            }
            if (T(0) < tend) stage_k(0, kpa, kr0, kr1, kc, ks);
            if (T(1) < tend) stage_k(1, kpa, pr0, pr1, pc, ps);
        }
        const int64_t qrow = wq0 + l32;
        const bool qvalid = qrow < p.Sq;

        const int64_t wq_last = (wq0 + 31 < p.Sq ? wq0 + 31 : p.Sq - 1);
        const bool wave_has_rows = wq0 < p.Sq;
        // Per-wave tile bounds, so the tile loop needs no 64-bit position
        // arithmetic: this wave computes tiles [0, kt_end) and masks tiles
        // from kt_mask on (the one straddling its diagonal, or the ragged
        // last tile); lane key limit: key j is visible iff j <= lim_base.
        const int kt_end = wave_has_rows ? (int)row_visits(p, wq_last) : 0;
        int kt_mask = (int)(p.Sk / BN);            // the ragged tile, or n_kt if none
        int lim_base = (int)(p.Sk - 1);
        if (p.causal) {
            const int64_t delta = p.q_off - p.k_off;   // >= 0
            const int64_t x = delta + wq0 + 1 - BN;
            const int64_t kc0 = x < 0 ? 0 : x / BN + 1;
            if (kc0 < kt_mask) kt_mask = (int)kc0;
            const int64_t c = delta + qrow;
            if (c < lim_base) lim_base = (int)c;
        }

        // ---- running state ----
        f32x16_t oacc[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) oacc[b] = (f32x16_t){};
        // Reference of this lane's query row (base 2, scaled scores), equal
        // in lanes l and l^32: probabilities are exp2(S - m_ref).  It stays 0
        // while the row's scores sit in [-64, 8] (no subtraction needed) and
        // is raised lazily to the row max when a score exceeds it by more
        // than the lazy threshold (or a row's first scores all lie below
        // -64).  m_set: the row has seen a visible key; all_set / ref_zero:
        // every row of the wave has / has a zero reference.
        float m_ref = 0.f;
        bool m_set = false, all_set = false, ref_zero = true;
        float l_acc[4] = {0.f, 0.f, 0.f, 0.f};   // partial row sums (this lane's keys)

        // S = K Q'^T of the tile in K buffer b: NKB 32-key blocks x 32
        // queries.  Accumulator element r of block kb2 <-> key
        // 32kb2 + 8(r/4) + 4hh + r%4 of the tile.
        auto qk = [&](int b, f32x16_t (&s)[NKB]) {
            const uint16_t *kl = kbuf(b);
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2) {
                s[kb2] = (f32x16_t){};
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const v8 a = *reinterpret_cast<const v8 *>(
                        kl + (kb2 * 32 + l32) * KP + 16 * t + 8 * hh);
                    s[kb2] = TT::mfma(a, qf[t], s[kb2]);
                }
            }
        };
        // P = exp2(S - m_ref) (SUB) or exp2(S) (every reference zero),
        // rounded to bf16 in the B-operand layout of O^T += V^T P^T, and this
        // lane's partial row sums of those bf16 values.  For key sub-step mm
        // of block kb2, slot s holds accumulator element 8mm + s.
        auto probs = [&](const f32x16_t (&s)[NKB], v8 (&pb)[NKB][2], float (&lt)[4], auto SUB) {
#pragma unroll
            for (int u = 0; u < 4; ++u) lt[u] = 0.f;
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    uint32_t wv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        float x0 = s[kb2][8 * mm + 2 * u], x1 = s[kb2][8 * mm + 2 * u + 1];
                        if constexpr (decltype(SUB)::value) {
                            x0 -= m_ref;
                            x1 -= m_ref;
                        }
                        wv[u] = TT::pack2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        lt[u] = TT::sum2(wv[u], lt[u]);
                    pb[kb2][mm] = __builtin_bit_cast(v8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
                }
        };
        using sub_on = std::integral_constant<bool, true>;
        using sub_off = std::integral_constant<bool, false>;
        // The exact path for tile kt: element mask (diagonal or ragged
        // tile), row max, lazy raise of the reference (rescaling O and l),
        // probabilities.
        auto exact = [&](int kt, f32x16_t (&s)[NKB], v8 (&pb)[NKB][2], float (&lt)[4]) {
            if (kt >= kt_mask) {
                // key kt*BN + kk is visible iff kk <= lim (kk: index inside the tile)
                const int lim0 = lim_base - kt * BN;
                const int lim = lim0 < -1 ? -1 : (lim0 > BN ? BN : lim0);
                const int lim_h = lim - 4 * hh;
#pragma unroll
                for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = 32 * kb2 + 8 * (r / 4) + (r % 4);
                        if (kk > lim_h) s[kb2][r] = -INFINITY;
                    }
            }
            // row max of S (tree), combined with the other half of the column
            float mx[4 * NKB];
#pragma unroll
            for (int u = 0; u < 4 * NKB; ++u)
                mx[u] = fmaxf(fmaxf(s[u >> 2][4 * (u & 3)], s[u >> 2][4 * (u & 3) + 1]),
                              fmaxf(s[u >> 2][4 * (u & 3) + 2], s[u >> 2][4 * (u & 3) + 3]));
#pragma unroll
            for (int wd = 2 * NKB; wd >= 1; wd >>= 1)
#pragma unroll
                for (int u = 0; u < wd; ++u) mx[u] = fmaxf(mx[u], mx[u + wd]);
            const float rmax = max_with_partner(mx[0]);
            // raise the reference when the row's scores exceed it by more
            // than the lazy threshold, or when a row's first visible scores
            // all lie below -64 (they would underflow against 0)
            const bool need = rmax - m_ref > LAZY_THRESHOLD || (!m_set && rmax > -INFINITY && rmax < -64.f);
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                const float m_new = need ? rmax : m_ref;
                const float alpha = m_set ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
#pragma unroll
                for (int u = 0; u < 4; ++u) l_acc[u] *= alpha;
                m_ref = m_new;
                ref_zero = __builtin_amdgcn_ballot_w64(m_ref != 0.f) == 0;
            }
            m_set = m_set || rmax > -INFINITY;
            all_set = __builtin_amdgcn_ballot_w64(!m_set) == 0;
            probs(s, pb, lt, sub_on{});
        };
        // O^T += V^T P^T with V from V buffer b.
        auto pv = [&](const v8 (&pb)[NKB][2], int b) {
            const uint16_t *v_lds = vbuf(b);
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                    for (int bd = 0; bd < DB; ++bd) {
                        const int key0 = 32 * kb2 + 16 * mm + tr_key;
                        const uint16_t *src = v_lds + key0 * D + vcol[bd];
                        const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)src);
                        const s16x4_t x1 =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(src + 8 * D));
                        const v8 a = __builtin_bit_cast(
                            v8, (short __attribute__((ext_vector_type(8)))){
                                          x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
                        oacc[bd] = TT::mfma(a, pb[kb2][mm], oacc[bd]);
                    }
        };

        // Phase 1 (plan A), iterations [0, j_split), every wave of the group
        // sharing the staging.  Iteration j (tile T(j)): load V(j+1) straight
        // into LDS; compute the scores of tile j+1 (its K was staged one
        // iteration earlier) on the matrix cores while forming tile j's
        // probabilities from the scores computed one iteration earlier; then
        // add tile j's P V while rotating and staging K(j+2) into the buffer
        // iteration j-1 finished reading; then fetch K(j+3) into registers.
        //
        // Phase 2 (plan B), [j_split, n_iter): the tiles left are seen only
        // by the heavy half's rows.  The light half's two waves stage their
        // K tiles (K(j+2) in iteration j), loading two tiles ahead, and load
        // the V tiles (V(j+1) in iteration j) straight into LDS; the heavy
        // half's waves only compute, so their dependency chain holds no
        // memory operation.
        //
        // One barrier per iteration; every wave of the workgroup runs the
        // same number of iterations, plus one at the end.
        const int c_end = kt_end < tend ? kt_end : tend;   // this wave computes tiles [t0, c_end)
        int j_end = c_end > t0 ? (c_end - t0 + TS - 1) / TS : 0;
        if (j_end > n_iter) j_end = n_iter;
        int j_split = n_iter;
        if (rowB < p.Sq) {
            const int64_t lastA = rowA + 63 < p.Sq ? rowA + 63 : p.Sq - 1;
            const int light_end = (int)row_visits(p, lastA);   // light rows see tiles < light_end
            const int js = light_end > t0 ? (light_end - t0 + TS - 1) / TS : 0;
            if (js < j_split) j_split = js;
        }
        const bool light = half == 0;

        // The loads staged in iteration j are issued at the end of
        // iteration j-1 (here for j = 0), ahead of the barrier.
        auto fetch_next = [&](int j) {
            if (T(j + 2) < tend) fetch_k(T(j + 2), kpa, kr0, kr1, kc, ks);
        };
        // Right after the barrier that starts iteration j each wave
        // loads its share of V(j+1) into V buffer (j+1) & 1, whose V(j-1) was
        // read in iteration j-1; before the barrier that ends iteration j it
        // waits for all its vector-memory loads (vmcnt 0), so the tile is
        // complete when iteration j+1 reads it.  4 waves share a tile: 2
        // blocks each; 2 waves: 4 blocks each.
        auto wait_vm0 = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0); expcnt, lgkmcnt: no wait
            __builtin_amdgcn_sched_barrier(0);
        };
        auto dma_next = [&](int j, int blk0, auto NBLK) { dma_v(T(j + 1), (j + 1) & 1, blk0, NBLK); };
        auto wait_dma = [&]() { wait_vm0(); };
        using blk2 = std::integral_constant<int, 2>;
        using blk4 = std::integral_constant<int, 4>;
        wait_dma();   // V(0)
        if (j_split > 0) fetch_next(0);
        __syncthreads();
        if (group == 1) {
#pragma unroll
            for (int t = 0; t < DT; ++t)
                qf[t] = *reinterpret_cast<const v8 *>(lds + KV_ELEMS + (((wave ^ 2) * DT + t) * 64 + lane) * 8);
        }
        // scores S[j & 1] of tile j
        f32x16_t S0[NKB], S1[NKB];
        if (j_end > 0) qk(0, S0);

        auto stage_next = [&](int j) { stage_k(j & 1, kpa, kr0, kr1, kc, ks); };
        // tile j's probabilities on the fast path (exact path if needed);
        // `mfma` issues the matrix-core work they are interleaved with
        auto softmax = [&](int j, f32x16_t (&sc)[NKB], v8 (&pb)[NKB][2], auto mfma, auto NMF,
                           auto NPV) {
            const int kt = T(j);
            float lt[4];
            constexpr int nmf = decltype(NMF)::value, npv = decltype(NPV)::value;
            auto block = [&](auto SUB) {
                mfma();
                probs(sc, pb, lt, SUB);
                __builtin_amdgcn_sched_group_barrier(0x100, npv > 0 ? 4 : 2, 0);   // LDS reads
                sched_mix<0, npv, nmf, 72 / nmf + 1>();
            };
            if (ref_zero) block(sub_off{});
            else block(sub_on{});
            const float lmax = fmaxf(fmaxf(lt[0], lt[1]), fmaxf(lt[2], lt[3]));
            // the fast path's values exist before the branch on them
            asm volatile("" ::"v"(lmax));
            const bool big = !(lmax <= FAST_SUM_LIMIT);
            if (!all_set || kt >= kt_mask || __builtin_amdgcn_ballot_w64(big) != 0)
                exact(kt, sc, pb, lt);
#pragma unroll
            for (int u = 0; u < 4; ++u) l_acc[u] += lt[u];
        };
        using i_qk = std::integral_constant<int, NKB * DT>;
        using i_zero = std::integral_constant<int, 0>;
        // phase-1 iteration
        auto step_a = [&](int j, f32x16_t (&sc)[NKB], f32x16_t (&sn)[NKB]) {
            __syncthreads();   // K(j+1), V(j) staged; buffers of iteration j-1 free
            dma_next(j, 2 * wave, blk2{});
            v8 pb[NKB][2];
            softmax(j, sc, pb, [&]() { qk((j + 1) & 1, sn); }, i_qk{}, i_zero{});
            // tile j's P V on the matrix cores, interleaved with staging
            pv(pb, vslot(j));
            stage_next(j);
#pragma unroll
            for (int i = 0; i < 2 * NKB * DB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 64 / (2 * NKB * DB), 0);   // vector ALU
            }
            wait_dma();   // V(j+1)
            if (j + 1 < j_split) fetch_next(j + 1);
        };
        // phase-2 iteration of a heavy wave: the pair loads V(j+1) (4
        // blocks per wave, from block pblk)
        auto step_b = [&](int j, f32x16_t (&sc)[NKB], f32x16_t (&sn)[NKB]) {
            __syncthreads();   // K(j+1), V(j) staged
            v8 pb[NKB][2];
            softmax(j, sc, pb, [&]() { qk((j + 1) & 1, sn); }, i_qk{}, i_zero{});
            pv(pb, vslot(j));
        };

        // ---- phase 1 ----
        int j = 0;
        {
            const int je1 = j_end < j_split ? j_end : j_split;
            for (; j + 1 < je1; j += 2) {
                step_a(j, S0, S1);
                step_a(j + 1, S1, S0);
            }
            if (j < je1) {
                step_a(j, S0, S1);
                ++j;
            }
        }
        for (; j < j_split; ++j) {
            __syncthreads();
            dma_next(j, 2 * wave, blk2{});
            stage_next(j);
            wait_dma();
            if (j + 1 < j_split) fetch_next(j + 1);
        }
        // ---- phase 2 ----
        {
            if (j_split < n_iter) {
                // Iteration j stages K(j+2) and loads V(j+1), as in phase 1,
                // both by the light pair's 128 threads: the K tiles with their
                // rotation, two register sets deep (K(j+2) staged while
                // K(j+4) loads), the V tiles straight into LDS.
                constexpr int KIB = (Plan::SLOTS + 127) / 128;
                const int ptid = (wave & 1) * 64 + lane;   // thread index inside the pair
                if (light) {
                    KItem kpb[KIB];
#pragma unroll
                    for (int i = 0; i < KIB; ++i) kpb[i] = k_item(ptid + 128 * i);
                    uint4 a0[KIB], a1[KIB], b0[KIB], b1[KIB];
                    float ac[KIB][8], as[KIB][8], bc[KIB][8], bs[KIB][8];
                    auto fetch_b = [&](int jj, auto &r0, auto &r1, auto &c, auto &s) {
                        if (T(jj + 2) < tend) fetch_k(T(jj + 2), kpb, r0, r1, c, s);
                    };
                    const int pblk = 4 * (wave & 1);
                    // V(jj+1) straight into LDS (4 blocks per wave), then the
                    // K loads two tiles ahead; before the next barrier wait
                    // for all but those K loads (vector-memory operations
                    // complete in order), so V(jj+1) is complete
                    constexpr int KB_LOADS = KIB * (2 + (ROT ? 4 : 0));
                    auto wait_v = [&](int jj) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (T(jj + 2) < tend)
                            __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8) | (KB_LOADS & 15) | ((KB_LOADS >> 4) << 14));
                        else
                            __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
                        __builtin_amdgcn_sched_barrier(0);
                    };
                    fetch_b(j, a0, a1, ac, as);
                    fetch_b(j + 1, b0, b1, bc, bs);
                    for (; j < n_iter; j += 2) {
                        __syncthreads();
                        dma_next(j, pblk, blk4{});
                        stage_k(j & 1, kpb, a0, a1, ac, as);
                        __builtin_amdgcn_sched_barrier(0);
                        fetch_b(j + 2, a0, a1, ac, as);
                        wait_v(j + 2);
                        if (j + 1 < n_iter) {
                            __syncthreads();
                            dma_next(j + 1, pblk, blk4{});
                            stage_k((j + 1) & 1, kpb, b0, b1, bc, bs);
                            __builtin_amdgcn_sched_barrier(0);
                            fetch_b(j + 3, b0, b1, bc, bs);
                            wait_v(j + 3);
                        }
                    }
                    j = n_iter;
                } else {
                    auto run = [&](f32x16_t (&A)[NKB], f32x16_t (&B)[NKB]) {
                        // iterations [j, j_end); tile j's scores in A
                        for (; j + 1 < j_end; j += 2) {
                            step_b(j, A, B);
                            step_b(j + 1, B, A);
                        }
                        if (j < j_end) {
                            step_b(j, A, B);
                            ++j;
                        }
                    };
                    if (j & 1) run(S1, S0);
                    else run(S0, S1);
                    for (; j < n_iter; ++j) __syncthreads();
                }
            }
        }
        wait_dma();   // the value loads of tiles past the segment
        __syncthreads();   // all tiles consumed

        // ---- per-segment epilogue ----
        // The two groups hold the same rows (group 1's wave w those of group
        // 0's wave w ^ 2) over alternate key tiles.  Each group merges and
        // stores one 32-dim block of O (group g block g): it hands the other
        // block with its (m, l) to the partner wave through LDS, and both
        // form the merged (m, l) by the same expression, so both halves of a
        // row divide by the same l.
        static_assert(DB == 2, "one 32-dim block of O per group");
        const float l_own = sum_with_partner((l_acc[0] + l_acc[1]) + (l_acc[2] + l_acc[3]));
        const float m_own = m_set ? m_ref : -INFINITY;
        float *xfer = reinterpret_cast<float *>(lds);
        const int pair = group == 0 ? wave : (wave ^ 2);   // group 0's wave of these rows
        constexpr int NX = 16 + 2;                         // floats handed over per lane
        {
            float *dst = xfer + ((group * WAVES_PER_GROUP + pair) * NX) * 64 + lane;
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[r * 64] = group == 0 ? oacc[1][r] : oacc[0][r];
            dst[16 * 64] = m_own;
            dst[17 * 64] = l_own;
        }
        __syncthreads();
        const float *src = xfer + (((group ^ 1) * WAVES_PER_GROUP + pair) * NX) * 64 + lane;
        const float m_oth = src[16 * 64], l_oth = src[17 * 64];
        // A: group 0's state, B: group 1's
        const float mA = group == 0 ? m_own : m_oth, mB = group == 0 ? m_oth : m_own;
        const float lA = group == 0 ? l_own : l_oth, lB = group == 0 ? l_oth : l_own;
        const float m_fin = fmaxf(mA, mB);
        const float aA = mA == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mA - m_fin);
        const float aB = mB == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mB - m_fin);
        const float l_tot = lA * aA + lB * aB;
        const float a_own = group == 0 ? aA : aB, a_oth = group == 0 ? aB : aA;

        // merge block b of O with the partner's, scale by 1/l, round, store
        auto merge_store = [&](auto B) {
            constexpr int b = decltype(B)::value;
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[b][r] = oacc[b][r] * a_own + src[r * 64] * a_oth;
            if (!qvalid) return;
            const float inv = 1.f / l_tot;
            uint16_t *orow = p.o + ((int64_t)bh * p.Sq + qrow) * D;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * b + 8 * g + 4 * hh;
                uint2 wv;
                wv.x = TT::pack2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
                wv.y = TT::pack2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + d0) = wv;
            }
        };
        if (group == 0) {
            merge_store(std::integral_constant<int, 0>{});
            // scores are in log2 units against the reference m_fin
            if (p.lse && hh == 0 && qvalid) p.lse[(int64_t)bh * p.Sq + qrow] = (m_fin + log2f(l_tot)) * LN2;
        } else {
            merge_store(std::integral_constant<int, 1>{});
        }
    };

    // A head's workgroups share an XCD (block index modulo the head count).
    // Causal: workgroup r takes 64-row half-tiles r and n_half - 1 - r, a
    // light and a heavy one, so every workgroup sees about the same number
    // of key tiles.  Otherwise: 128 consecutive rows.
    const int bh = blockIdx.x % p.BH;
    const int64_t rank = blockIdx.x / p.BH;
    int64_t rowA, rowB;
    if (p.causal) {
        const int64_t hb = p.n_half - 1 - rank;
        rowA = 64 * rank;
        rowB = hb > rank ? 64 * hb : p.Sq;
    } else {
        rowA = rank * BM;
        rowB = rowA + 64;
    }
    const int64_t last = (rowB < p.Sq ? rowB : rowA) + 63;
    segment(bh, rowA, rowB, 0, row_visits(p, last < p.Sq ? last : p.Sq - 1));
}

// Tile shape: two key groups (8 waves, two per SIMD) of 64-key tiles.
constexpr int D64_NG = 2, D64_BN = 64;

template <int LAYOUT, bool ROT, bool FULL, typename E>
int launch(const FlashArgs &a, hipStream_t stream)
{
    constexpr int D = 64, NG = D64_NG, BN = D64_BN;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.cos_tab = a.cos_tab; p.sin_tab = a.sin_tab; p.rot_dim = a.rot_dim;
    p.table_rows = a.table_rows;
    p.sl2 = a.scale * 1.4426950408889634f;
    p.BH = a.B * a.H;
    p.kv_group = a.H / a.H_kv;
    p.Sq = a.Sq; p.Sk = a.Sk; p.q_off = a.q_off; p.k_off = a.k_off;
    p.causal = a.causal;
    p.n_qtiles = (a.Sq + BM - 1) / BM;
    p.n_half = (a.Sq + 63) / 64;
    p.tile_n = BN;
    p.n_kt = (a.Sk + BN - 1) / BN;
    const int64_t blocks = (int64_t)p.BH * (p.causal ? (p.n_half + 1) / 2 : p.n_qtiles);
    if (!rope_grid_fits(blocks, 256 * NG)) return ROPE_LAUNCH_SHAPE;
    hipLaunchKernelGGL((flash_fwd_bf16_kernel<D, LAYOUT, ROT, FULL, NG, BN, E>), dim3((unsigned)blocks),
                       dim3(256 * NG), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

template <typename E>
int launch_e(const FlashArgs &a, hipStream_t stream)
{
    if (a.rot_dim == 0) return launch<1, false, false, E>(a, stream);
    const bool full = a.rot_dim == 64;
    if (a.layout == 0) return full ? launch<0, true, true, E>(a, stream) : launch<0, true, false, E>(a, stream);
    return full ? launch<1, true, true, E>(a, stream) : launch<1, true, false, E>(a, stream);
}

}  // namespace

// dtype 0 (bf16) or 2 (fp16): the same kernels over either 16-bit type.
// Head dim 64 runs the kernel above, 128 the two-team kernel of
// flash_fwd_pp.hip.
int rope_launch_flash_bf16(const FlashArgs &a, hipStream_t stream)
{
    const int rc = rope_launch_flash_pp(a, stream);
    if (rc >= 0) return rc;
    if (a.head_dim != 64) return ROPE_LAUNCH_SHAPE;
    return a.dtype == 2 ? launch_e<_Float16>(a, stream) : launch_e<__bf16>(a, stream);
}

// Only the split-key schedule of the head-dim-128 kernel uses a workspace.
int64_t rope_flash_bf16_workspace_bytes(const FlashArgs &a)
{
    if (a.head_dim == 128 && (a.dtype == 0 || a.dtype == 2)) return rope_flash_pp_workspace_bytes(a);
    return 0;
}

namespace {
std::atomic<int> g_cu_count[64];
}  // namespace

int rope_device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
