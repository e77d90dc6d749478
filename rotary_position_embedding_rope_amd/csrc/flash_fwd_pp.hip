// flash_fwd_pp.hip -- fused RoPE + softmax attention forward, head dim 128,
// on the gfx950 matrix cores: two teams of four waves in ping-pong.
//
// Operation: O = softmax(scale * rope(Q) rope(K)^T + mask) V per (batch,
// head) ("RoPE and FlashAttention: relative positions and online softmax",
// section 4), evaluated with section 5's online-softmax recurrence; query i
// sits at q_off + i, key j at k_off + j, and with the causal mask key j is
// visible iff k_off + j <= q_off + i (section 6's offset mask).  Rotation
// pairs and formula: "Write Triton Rope Kernel", "Required reasoning
// process" steps 1 and 6; V is never rotated.
//
// Work decomposition.  A workgroup of 512 threads owns 256 query rows that
// read the same key/value head: G query heads of one key/value head (G the
// largest of 1, 2, 4, 8 dividing the query heads per key/value head) times
// a block of 256 / G consecutive query rows, the same rows in each head, so
// every wave walks nearly the same key range.  Waves 8/G apart take
// consecutive heads; a wave owns 32 query rows.  With G = 1 that is two
// 128-row query tiles of one head (team 0 = waves 0-3 the lower one); with
// grouped-query attention a staged key tile serves G query heads at once
// ("Write Triton Rope Kernel", "Inputs the agent should gather first", item
// 3: query and key head counts differ and share one table).  Under the
// causal mask the row blocks with the most keys are launched first.  All
// waves walk the same key tiles (BN = 64 keys by default, 32 also
// compiles), so each key tile is loaded, rotated and staged in LDS once
// for 256 query rows.
//
// Ping-pong.  The two waves of one SIMD belong to different teams.  Time is
// cut into phases separated by workgroup barriers; in each phase one team
// runs its matrix-core step (S(k) = K(k) Q'^T and O += P(k-1) V(k-1), with
// the staging of the next key tile's half interleaved between the matrix
// instructions) while the other team runs the vector-ALU step of its
// previous tile (online softmax: probabilities, row sums, lazy reference
// max).  Team 1 runs one phase behind team 0, so on every SIMD one wave
// keeps the matrix core busy while the other does the exponentials.
//
//   phase 2k:   team 0 matrix step k,   team 1 softmax of tile k-1
//   phase 2k+1: team 0 softmax of k,    team 1 matrix step k
//
// LDS rings: K tiles in 2 slots (tile k is read in phases 2k and 2k+1 and
// staged in phases 2k-2 (team 0: the first half of its keys) and 2k-1
// (team 1: the second half)); V tiles in 3 slots (tile k is read in phases
// 2k+2 and 2k+3, loaded by buffer loads straight into LDS in phases 2k-2 and
// 2k-1).  K is rotated in fp32 at its key positions from the fp32 table and
// rounded to the storage type once per staging; no rotated tensor reaches
// HBM.
//
// Every wave runs the same straight-line loop whatever its row range: a
// wave past its last visible tile multiplies a zero P, so no branch splits
// the matrix accumulators (which would double their registers).
//
// Softmax (section 5's recurrence with a free reference, exact in real
// arithmetic): probabilities are exp2(S - m) with S in log2 units (Q carries
// scale * log2 e) and a per-row reference m that stays 0 while the row's
// scores stay below 8 and above -64; it is raised lazily to the row max when
// a score exceeds it by more than 8, rescaling O and l.  Row sums are taken
// from the same bf16-rounded probabilities the P V product uses.
#include <type_traits>

#include "common.hpp"

namespace {

using rope::f32x16_t;
using rope::Ty;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int PP_NKS = 2;            // K slots
constexpr int PP_NVS = 3;            // V slots
#ifndef ROPE_PP_BN
#define ROPE_PP_BN 64
#endif
#ifndef ROPE_PP_PF
#define ROPE_PP_PF 3
#endif
constexpr int PP_PF = ROPE_PP_PF;   // LDS operand reads in flight ahead of the matrix instruction

// Tile geometry for head dim D (64 or 128) and BN keys per tile (32 or 64).
// Each team stages half of a tile's keys; a staging unit is two CH-dim
// chunks of one key row.  V rows are D / 8 chunks of 16 bytes, RPB rows to
// a 1 KB block of the loads straight into LDS.
template <int D, int BN> struct PPShape {
    static constexpr int NKB = BN / 32;           // 32-key blocks per tile
    static constexpr int HALF = BN / 2;           // keys a team stages per tile
    static constexpr int UPR = 256 / HALF;        // staging units per key row
    static constexpr int CH = D / (2 * UPR);      // dims per chunk (2, 4 or 8)
    static constexpr int NTRIG = CH >= 4 ? CH / 4 : 1;   // cos (and sin) loads per unit
    static constexpr int KP = D + 8;              // K LDS row pitch (elements)
    static constexpr int CPR = D / 8;             // 16-byte chunks per V row
    static constexpr int RPB = 64 / CPR;          // V rows per 1 KB block
    static constexpr int VBW = HALF / RPB / 4;    // 1 KB value blocks per wave per tile
    // vector-memory loads per matrix step (K chunks, cos/sin with rotation, V)
    template <bool ROT> static constexpr int nload() { return 2 + (ROT ? 2 * NTRIG : 0) + VBW; }
    static constexpr int K_ELEMS = BN * KP;
    static constexpr int V_ELEMS = BN * D;
    static constexpr int LDS_BYTES = 2 * (PP_NKS * K_ELEMS + PP_NVS * V_ELEMS);
    static_assert(CH >= 4 && VBW >= 1, "tile shape");
};
// Position of 16-byte chunk c of V row `row` in LDS: c ^ vswz(row).  Every
// four consecutive keys of a transposing read then fall in different bank
// groups (D = 128: rows are 256 bytes, so the row's low two bits pick a
// quarter; D = 64: 128-byte rows, rows 2 and 3 of four take the other half).
template <int D>
__device__ __forceinline__ int vswz(int row)
{
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}
constexpr float PP_LAZY = 8.0f;      // log2 headroom before the reference is raised
constexpr int PP_MAXSEG = 8;         // key segments per row block at most (split schedule)
constexpr float PP_LN2 = 0.6931471805599453f;
constexpr int RSRC_FLAGS = 0x00020000;

struct PPParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int BH, kv_group;
    int Sq, Sk;
    int64_t q_off, k_off;
    const float *cos_tab, *sin_tab;
    int64_t table_rows;
    int rot_dim;
    float sl2;
    int causal;
    int g_log2;  // log2 G: G query heads of one key/value head per workgroup
    int n_hg;    // head groups: BH / G
    int n_rb;    // row blocks of 256 / G query rows
    int n_kt;    // key tiles
    // split keys: the key tiles of a workgroup's query rows are cut into
    // segments of seg_tiles tiles (nseg at most); segments of a cut row
    // block leave fp32 partial states in ws, merged by flash_pp_merge_kernel
    int seg_tiles, nseg;
    float *ws;
};

// A buffer descriptor over `rows` rows of ROW_BYTES from `base` (wave-uniform
// arguments; loads at or past the end return zeros).  The record count is
// made explicitly scalar so the descriptor never lands in vector registers.
template <int ROW_BYTES>
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int rows)
{
    constexpr int MAX_ROWS = (int)(0xffffffffu / ROW_BYTES);
    const uint32_t n = rows <= 0 ? 0u : (rows >= MAX_ROWS ? 0xffffffffu : (uint32_t)rows * ROW_BYTES);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)n), RSRC_FLAGS);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, int off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float4 bload16f(rsrc_t r, int off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
[[maybe_unused]] __device__ __forceinline__ uint2 bload8(rsrc_t r, int off)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

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

// 16 bytes per lane from global memory straight into LDS: lane i writes LDS
// bytes lds_byte + 16 i .. +15 with the bytes at voff of the buffer.  Written
// out here rather than through the compiler's builtin, which makes every later
// LDS access of the wave wait for all its outstanding loads (it cannot tell
// the slots apart); the issuing wave waits for these loads (vmcnt) before the
// barrier that hands their tile over.  No register receives data.
typedef int sgpr4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16(sgpr4_t rs, uint32_t voff, uint32_t lds_byte)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(lds_byte)
                 : "memory", "m0");
}
// The same descriptor as make_rsrc, as four scalar dwords (untyped buffer,
// stride 0).
__device__ __forceinline__ sgpr4_t rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    sgpr4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = RSRC_FLAGS;
    return r;
}

// Workgroup barrier after this wave's LDS writes have completed.  Unlike
// __syncthreads() it does not wait for the wave's loads straight into LDS
// (the fence would turn that into a full vmcnt(0) at every barrier); those
// are waited for explicitly before the barrier that hands their tile over.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Key tiles (of BN) visible to query rows up to `last` (all when not causal).
template <int BN>
__device__ __forceinline__ int tiles_seen(const PPParams &p, int last)
{
    if (!p.causal) return p.n_kt;
    const int64_t v = (p.q_off + last - p.k_off) / BN + 1;
    return v < p.n_kt ? (int)v : p.n_kt;
}

// Key tiles of row block rb (rows rb R .. rb R + R - 1, R = 256 / G): those
// its last row sees.
template <int BN>
__device__ __forceinline__ int block_tiles(const PPParams &p, int rb)
{
    const int R = 256 >> p.g_log2;
    const int last = rb * R + R - 1 < p.Sq ? rb * R + R - 1 : p.Sq - 1;
    return tiles_seen<BN>(p, last);
}

// PING: ping-pong schedule (team 1 one phase behind team 0, two barriers per
// key tile); otherwise both teams run each step together (one barrier per
// tile).  SPLIT: the workgroup takes one key segment of its row block.
template <int D, int BN, bool PING, bool SPLIT, int LAYOUT, bool ROT, bool FULL, typename E>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void flash_fwd_pp_kernel(PPParams p)
{
    using SH = PPShape<D, BN>;
    constexpr int KP = SH::KP;
    constexpr int DT = D / 16;          // k-steps of Q K^T
    constexpr int DB = D / 32;          // 32-dim blocks of O^T
    constexpr int NKB = SH::NKB, CH = SH::CH, UPR = SH::UPR;
    constexpr int NS = NKB * DT;        // score products per tile
    constexpr int NPV = NKB * 2 * DB;   // P V products per tile
    using TT = Ty<E>;
    using v8 = typename TT::v8;

    __shared__ __attribute__((aligned(16))) uint16_t lds[SH::LDS_BYTES / 2];
    auto kslot = [&](int k) { return lds + (k % PP_NKS) * SH::K_ELEMS; };
    auto vslot = [&](int k) { return lds + PP_NKS * SH::K_ELEMS + ((k + PP_NVS) % PP_NVS) * SH::V_ELEMS; };

    const int tid = threadIdx.x;
    const int team = __builtin_amdgcn_readfirstlane(tid >> 8);
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);   // wave inside the team
    const int st = tid & 255;                                          // thread inside the team
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int rh = p.rot_dim / 2;   // table row stride (floats)

    // ---- work item: (head group, row block, key segment) ----
    // Block index mod n_hg selects the head group, so one key/value head's
    // workgroups share an XCD (and its L2) when n_hg is a multiple of 8.
    const int hg = blockIdx.x % p.n_hg;
    const int r = (blockIdx.x / p.n_hg) % p.n_rb;
    const int seg = SPLIT ? (int)(blockIdx.x / p.n_hg / p.n_rb) : 0;
    const int rb = p.causal ? p.n_rb - 1 - r : r;   // the most keys first
    const int item = hg * p.n_rb + rb;
    // wave gw of the workgroup: head gw >> (3 - g_log2) of the group, rows
    // 32 (gw mod 8/G) of the block (wave-uniform: keeps descriptors scalar)
    const int gw = 4 * team + wave;
    const int wlog = 3 - p.g_log2;
    const int bh = __builtin_amdgcn_readfirstlane((hg << p.g_log2) + (gw >> wlog));   // batch*head
    const int row0 = __builtin_amdgcn_readfirstlane(rb * (256 >> p.g_log2) + 32 * (gw & ((1 << wlog) - 1)));
    const bool wave_rows = row0 < p.Sq;
    const int wlast = row0 + 31 < p.Sq ? row0 + 31 : p.Sq - 1;
    // tiles this wave computes, and the workgroup's staging range
    const int w_end = wave_rows ? tiles_seen<BN>(p, wlast) : 0;
    const int k_all = block_tiles<BN>(p, rb);
    // this workgroup's key tiles [k_beg, k_end): its segment of the row block's
    int k_beg = 0, k_end = k_all;
    bool partial = false;   // the row block is cut: leave a partial state
    if constexpr (SPLIT) {
        k_beg = seg * p.seg_tiles;
        if (k_beg >= k_all) return;   // no segment here (uniform over the workgroup)
        k_end = k_beg + p.seg_tiles < k_all ? k_beg + p.seg_tiles : k_all;
        partial = k_all > p.seg_tiles;
    }
    const int w_stop = w_end < k_end ? w_end : k_end;   // softmax only below this tile
    // first tile needing the element mask (diagonal or ragged end), and the
    // lane's key limit: key j of the segment is visible iff j <= lim_base
    const int qrow = row0 + l32;
    int w_mask = p.Sk / BN;
    int lim_base = p.Sk - 1;
    if (p.causal) {
        const int64_t delta = p.q_off - p.k_off;   // >= 0 (validated)
        const int64_t x = delta + row0 + 1 - BN;
        const int64_t kc0 = x < 0 ? 0 : x / BN + 1;
        if (kc0 < w_mask) w_mask = (int)kc0;
        const int64_t c = delta + qrow;
        if (c < lim_base) lim_base = (int)c;
    }

    const uint16_t *qh = p.q + (int64_t)bh * p.Sq * D;
    const uint16_t *kh = p.k + (int64_t)(bh / p.kv_group) * p.Sk * D;
    const uint16_t *vh = p.v + (int64_t)(bh / p.kv_group) * p.Sk * D;
    const float *ctab = ROT ? p.cos_tab + p.k_off * rh : nullptr;
    const float *stab = ROT ? p.sin_tab + p.k_off * rh : nullptr;
    const int64_t trk = p.table_rows - p.k_off;
    const int tab_rows_k = (int)(trk < 0x7fffffffLL ? trk : 0x7fffffffLL);

    // ---- K staging plan: this thread's unit of its team's half tile ----
    // Team 0 stages the first HALF keys of a tile, team 1 the rest.  A unit
    // is two CH-dim chunks of one key row: NeoX, dims CH u and their
    // partners CH u + rot/2; GPT-J, 2 CH consecutive dims (CH whole pairs);
    // past rot_dim, 2 CH consecutive dims copied.  It uses table columns
    // CH u .. CH u + CH - 1.
    const int krow = team * SH::HALF + st / UPR;
    const int ku = st % UPR;
    int kd0, kd1;
    bool krot;
    if constexpr (ROT && LAYOUT == 0) {
        const int ru = p.rot_dim / (2 * CH);   // rotated units per row
        krot = ku < ru;
        kd0 = krot ? CH * ku : p.rot_dim + 2 * CH * (ku - ru);
        kd1 = krot ? kd0 + rh : kd0 + CH;
    } else {
        krot = ROT && 2 * CH * ku < p.rot_dim;
        kd0 = 2 * CH * ku;
        kd1 = kd0 + CH;
    }
    const int kto = 4 * CH * ku;   // byte offset of the unit's table columns in a row

    uint32_t sk0[CH / 2], sk1[CH / 2];   // raw K chunks of the unit in flight
    float sc[CH], ss[CH];                // their cos / sin
    auto fetch_k = [&](int kt) {
        const int j0 = kt * BN;
        const rsrc_t krs = make_rsrc<2 * D>(kh + (int64_t)j0 * D, kt < k_end ? p.Sk - j0 : 0);
        if constexpr (CH == 8) {
            *reinterpret_cast<uint4 *>(sk0) = bload16(krs, 2 * (krow * D + kd0));
            *reinterpret_cast<uint4 *>(sk1) = bload16(krs, 2 * (krow * D + kd1));
        } else {
            *reinterpret_cast<uint2 *>(sk0) = bload8(krs, 2 * (krow * D + kd0));
            *reinterpret_cast<uint2 *>(sk1) = bload8(krs, 2 * (krow * D + kd1));
        }
        if constexpr (ROT) {
            const int left = tab_rows_k - j0;
            const int trows = (left < BN ? left : BN) * (rh / 4);
            const rsrc_t crs = make_rsrc<16>(ctab + (int64_t)j0 * rh, trows);
            const rsrc_t srs = make_rsrc<16>(stab + (int64_t)j0 * rh, trows);
            const int to = 4 * krow * rh + kto;
#pragma unroll
            for (int i = 0; i < SH::NTRIG; ++i) {
                *reinterpret_cast<float4 *>(sc + 4 * i) = bload16f(crs, to + 16 * i);
                *reinterpret_cast<float4 *>(ss + 4 * i) = bload16f(srs, to + 16 * i);
            }
        }
    };
    // Rotate the fetched unit in fp32 and round to the storage type, then
    // write both chunks to K slot kt.  Dword i of the two chunks holds two
    // rotation pairs (x, y) -> (x c - y s, x s + y c): NeoX, element e of
    // chunk 0 with element e of chunk 1 (frequency CH u + 2i + e); GPT-J, the
    // two elements of one chunk's dword (chunk h: frequency CH u + CH/2 h + i).
    // The work is cut into NSUB substeps, four per dword (unpack, products,
    // fused sums, packing), so that only a few vector instructions sit
    // between consecutive matrix instructions.
    constexpr int NSUB = ROT ? 2 * CH : 0;
    static_assert(NSUB + 2 < NPV + NS, "staging fits in the matrix step");
    uint32_t sx0[CH / 2], sx1[CH / 2];
    float rin[CH / 2][4], rpr[CH / 2][4], rout[CH / 2][4];   // x0 y0 x1 y1 / y0 s0, y1 s1, x0 s0, x1 s1 / results
    auto trig = [&](int i, int e, float &c, float &sn) {
        const int f = LAYOUT == 0 ? 2 * i + e : (CH / 2) * e + i;
        c = (FULL || krot) ? sc[f] : 1.f;
        sn = (FULL || krot) ? ss[f] : 0.f;
    };
    auto stage_sub = [&](int sub) {
        if constexpr (ROT) {
            const int i = sub / 4;
            float c0, s0, c1, s1;
            trig(i, 0, c0, s0);
            trig(i, 1, c1, s1);
            switch (sub % 4) {
            case 0: {
                const uint32_t a = sk0[i], b = sk1[i];
                if constexpr (LAYOUT == 0) {
                    rin[i][0] = TT::lo(a); rin[i][1] = TT::lo(b); rin[i][2] = TT::hi(a); rin[i][3] = TT::hi(b);
                } else {
                    rin[i][0] = TT::lo(a); rin[i][1] = TT::hi(a); rin[i][2] = TT::lo(b); rin[i][3] = TT::hi(b);
                }
                break;
            }
            case 1:
                rpr[i][0] = rin[i][1] * s0;
                rpr[i][1] = rin[i][3] * s1;
                rpr[i][2] = rin[i][0] * s0;
                rpr[i][3] = rin[i][2] * s1;
                break;
            case 2:
                rout[i][0] = __builtin_fmaf(rin[i][0], c0, -rpr[i][0]);
                rout[i][1] = __builtin_fmaf(rin[i][1], c0, rpr[i][2]);
                rout[i][2] = __builtin_fmaf(rin[i][2], c1, -rpr[i][1]);
                rout[i][3] = __builtin_fmaf(rin[i][3], c1, rpr[i][3]);
                break;
            default:
                if constexpr (LAYOUT == 0) {
                    sx0[i] = TT::pack2(rout[i][0], rout[i][2]);
                    sx1[i] = TT::pack2(rout[i][1], rout[i][3]);
                } else {
                    sx0[i] = TT::pack2(rout[i][0], rout[i][1]);
                    sx1[i] = TT::pack2(rout[i][2], rout[i][3]);
                }
                break;
            }
        }
    };
    auto stage_write = [&](int kt) {
        if constexpr (!ROT) {
#pragma unroll
            for (int i = 0; i < CH / 2; ++i) {
                sx0[i] = sk0[i];
                sx1[i] = sk1[i];
            }
        }
        uint16_t *dst = kslot(kt) + krow * KP;
        if constexpr (CH == 8) {
            *reinterpret_cast<uint4 *>(dst + kd0) = make_uint4(sx0[0], sx0[1], sx0[2], sx0[3]);
            *reinterpret_cast<uint4 *>(dst + kd1) = make_uint4(sx1[0], sx1[1], sx1[2], sx1[3]);
        } else {
            *reinterpret_cast<uint2 *>(dst + kd0) = make_uint2(sx0[0], sx0[1]);
            *reinterpret_cast<uint2 *>(dst + kd1) = make_uint2(sx1[0], sx1[1]);
        }
    };
    auto stage_k = [&](int kt) {
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) stage_sub(sub);
        stage_write(kt);
    };
    // V tile kt, this team's half of its keys, straight into LDS: blocks of
    // 1 KB (RPB rows), VBW per wave, each row's chunks swizzled by vswz.
    // Tiles past the range load nothing (zero records) and fill their slot,
    // which is free by then, with zeros.
    const uint32_t lds_byte0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
    auto dma_v = [&](int kt) {
        const int j0 = kt * BN;
        const int rows = kt < k_end ? p.Sk - j0 : 0;
        const uint32_t bytes = rows <= 0 ? 0u : (rows >= (int)(0xffffffffu / (2 * D)) ? 0xffffffffu : (uint32_t)rows * (2 * D));
        const sgpr4_t vrs = rsrc_words(vh + (int64_t)j0 * D, bytes);
#pragma unroll
        for (int i = 0; i < SH::VBW; ++i) {
            const int blk = team * (SH::HALF / SH::RPB) + wave * SH::VBW + i;   // 1 KB block of the tile
            const int rr = SH::RPB * blk + lane / SH::CPR;                     // key row
            const int cq = (lane % SH::CPR) ^ vswz<D>(rr);
            const uint32_t dst = lds_byte0 + 2 * (uint32_t)((vslot(kt) - lds) + blk * 512);
            dma16(vrs, 2 * (rr * D + 8 * cq), __builtin_amdgcn_readfirstlane(dst));
        }
    };

    // ---- Q: load, rotate at q_off + row, scale by scale*log2 e, keep as
    // the B operand of S = K Q'^T (lane: query l32, dims 16t + 8hh + 0..7)
    v8 qf[DT];
    {
        const int qleft = p.Sq - row0;
        const rsrc_t qrs = make_rsrc<2 * D>(qh + (int64_t)row0 * D, qleft < 0 ? 0 : (qleft > 32 ? 32 : qleft));
        float qv[DT][8];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const uint4 w = bload16(qrs, 2 * (l32 * D + 16 * t + 8 * hh));
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qv[t][2 * i] = TT::lo(ws[i]);
                qv[t][2 * i + 1] = TT::hi(ws[i]);
            }
        }
        if constexpr (ROT) {
            const int64_t tleft = p.table_rows - (p.q_off + row0);
            const int trows = (int)(tleft < 0 ? 0 : (tleft > 32 ? 32 : tleft)) * (rh / 4);
            const rsrc_t qcs = make_rsrc<16>(p.cos_tab + (p.q_off + row0) * rh, trows);
            const rsrc_t qss = make_rsrc<16>(p.sin_tab + (p.q_off + row0) * rh, trows);
            const int tb = 4 * l32 * rh;
            if constexpr (LAYOUT == 0) {
                // dims 16t + 8hh + u pair with 16(t + rot/32) + 8hh + u (same lane)
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
#pragma unroll
                        for (int u = 1; u <= DT / 2; ++u)
                            if (u == tr) {
#pragma unroll
                                for (int i = 0; i < 8; ++i) {
                                    const float x = qv[t][i], y = qv[t + u][i];
                                    qv[t][i] = x * c[i] - y * s[i];
                                    qv[t + u][i] = x * s[i] + y * c[i];
                                }
                            }
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    if (16 * t < p.rot_dim) {
                        const int f0 = 4 * (8 * t + 4 * hh);
                        float c[4], s[4];
                        *reinterpret_cast<float4 *>(c) = bload16f(qcs, tb + f0);
                        *reinterpret_cast<float4 *>(s) = bload16f(qss, tb + f0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = qv[t][2 * i], y = qv[t][2 * i + 1];
                            qv[t][2 * i] = x * c[i] - y * s[i];
                            qv[t][2 * i + 1] = x * s[i] + y * c[i];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[t][i] = (E)(qv[t][i] * p.sl2);
    }

    // ---- prologue: K(k_beg) staged, this team's half of K(k_beg + 1) and
    // V(k_beg) in flight.  Every matrix step then issues the same number of
    // vector-memory loads per wave (nload: its V half, then its K half; past
    // the key range they read zero records), so the waits below can count
    // them.
    fetch_k(k_beg);
    stage_k(k_beg);
    fetch_k(k_beg + 1);
    dma_v(k_beg);
    {
        // the slot of V(k_beg - 1), which the first step multiplies by the
        // zero P(k_beg - 1)
        uint4 *z = reinterpret_cast<uint4 *>(vslot(k_beg - 1));
#pragma unroll
        for (int i = 0; i < SH::V_ELEMS / 8 / 512; ++i) z[tid + 512 * i] = make_uint4(0, 0, 0, 0);
    }

    // ---- running state ----
    f32x16_t oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = (f32x16_t){};
    f32x16_t sacc[NKB];
    v8 pb[NKB][2];   // P(k-1); zero before the first tile
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) pb[kb][mm] = __builtin_bit_cast(v8, make_uint4(0, 0, 0, 0));
    float m_ref = 0.f;
    bool m_set = false, all_set = false, ref_zero = true;
    float l_acc[4] = {0.f, 0.f, 0.f, 0.f};

    // V^T operand addressing (ds_read_b64_tr_b16): in each 16-lane group,
    // lane 4j + b points at V[key0 + j][dim0 + 4b]; the receiving lane then
    // holds V[key0 .. key0+3][dim0 + its index].  Key k of the tile maps to
    // row k, whose 16-byte chunk c sits at c ^ vswz(k).  The lane's key is
    // tr_key + 32 kb + 16 mm (+ 8), all multiples of 8 apart from tr_key,
    // which leave vswz unchanged, so a lane needs one base per 32-dim block
    // and the key steps are immediate offsets.
    const int g16 = lane >> 4, lp = lane & 15;
    const int tr_key = 4 * (g16 >> 1) + (lp >> 2);
    const int tr_dim = 4 * (lp & 3) + 16 * (g16 & 1);
    int vbase[DB];   // element offsets inside a V slot
#pragma unroll
    for (int bd = 0; bd < DB; ++bd)
        vbase[bd] = tr_key * D + 8 * ((4 * bd + (tr_dim >> 3)) ^ vswz<D>(tr_key)) + (tr_dim & 7);
    const int kbase = l32 * KP + 8 * hh;   // K operand: row l32, dims 8 hh (+ 32 kb rows, 16 t dims)

    // The operand stream of matrix step k: NPV P V operands (V^T of tile k-1,
    // keys 32 kb + 16 mm, dims 32 bd for product j with bd = j % DB,
    // mm = (j / DB) % 2, kb = j / (2 DB)), then NS score operands (K of tile
    // k, keys 32 (j / DT), dims 16 (j % DT)).  Reads run PP_PF operands ahead
    // of the matrix instruction in the ring buf; the first PP_PF of step k are
    // read during the softmax phase before it, when V(k-1) is complete.
    v8 buf[PP_PF];
    auto pv_bases = [&](int k, int (&vb)[DB]) {
#pragma unroll
        for (int bd = 0; bd < DB; ++bd) {
            // per-lane bases of this step, opaque to the optimiser so that
            // the key steps stay immediate offsets of the reads
            vb[bd] = vbase[bd] + (int)(vslot(k - 1) - lds);
            asm volatile("" : "+v"(vb[bd]));
        }
    };
    auto pv_operand = [&](const int (&vb)[DB], int j) {
        const uint16_t *src = lds + vb[j % DB] + (32 * (j / (2 * DB)) + 16 * ((j / DB) & 1)) * D;
        const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)src);
        const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(src + 8 * D));
        return __builtin_bit_cast(v8, (short __attribute__((ext_vector_type(8)))){x0[0], x0[1], x0[2], x0[3], x1[0],
                                                                                 x1[1], x1[2], x1[3]});
    };
    auto prefetch_pv = [&](int k) {
        int vb[DB];
        pv_bases(k, vb);
#pragma unroll
        for (int i = 0; i < PP_PF; ++i)
            if (i < NPV) buf[i] = pv_operand(vb, i);
    };

    // Matrix-core step k: O += P(k-1) V(k-1), then S(k) = K(k) Q'^T (P is
    // dead before S is written, so the two can share registers).  Scheduling
    // fences keep the order written: the rotation of this team's half of
    // tile k+1 between the P V products and its LDS writes after them; the
    // loads of V(k+1) and of its half of tile k+2 between the score
    // products.  Step 0 multiplies the zero P(-1) by the zero-filled slot of
    // V(-1); a wave past its last tile multiplies zeros (its P is zero), so
    // every wave runs the same straight-line code.  The wave runs at raised
    // priority so its matrix instructions issue ahead of the other team's
    // softmax on the same SIMD.
    auto mfma_step = [&](int k) {
        __builtin_amdgcn_s_setprio(1);
        int vb[DB];
        pv_bases(k, vb);
        int kb0 = kbase + (int)(kslot(k) - lds);
        asm volatile("" : "+v"(kb0));
        const uint16_t *kl = lds + kb0;
        auto operand = [&](int j) {
            if (j < NPV) return pv_operand(vb, j);
            const int i = j - NPV;
            return *reinterpret_cast<const v8 *>(kl + (i / DT) * 32 * KP + 16 * (i % DT));
        };
#pragma unroll
        for (int j = 0; j < NPV + NS; ++j) {
            if (j < NPV) {
                oacc[j % DB] = TT::mfma(buf[j % PP_PF], pb[j / (2 * DB)][(j / DB) & 1], oacc[j % DB]);
            } else {
                const int i = j - NPV, kb = i / DT;
                sacc[kb] = TT::mfma(buf[j % PP_PF], qf[i % DT], (i % DT) ? sacc[kb] : (f32x16_t){});
            }
            if (j + PP_PF < NPV + NS) buf[j % PP_PF] = operand(j + PP_PF);
            if (j < NSUB) stage_sub(j);
            if (j == NSUB + 1) stage_write(k + 1);
            // V first: the rotation of K(k+2) in the next step then waits only
            // on loads the compiler issued after it
            if (j == NPV + 1) dma_v(k + 1);
            if (j == NPV + 2) fetch_k(k + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Probabilities of the scores in sacc, against the reference (SUB) or
    // with every reference zero, exponentiated in place (all exponentials
    // issue before the first use of one), then rounded to the storage type
    // in the B-operand layout of O^T += V^T P^T, with this lane's partial
    // row sums.
    auto probs = [&](float (&lt)[4], auto SUB) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float x = sacc[kb][rr];
                if constexpr (decltype(SUB)::value) x -= m_ref;
                sacc[kb][rr] = __builtin_amdgcn_exp2f(x);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) lt[u] = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                uint32_t wv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) wv[u] = TT::pack2(sacc[kb][8 * mm + 2 * u], sacc[kb][8 * mm + 2 * u + 1]);
#pragma unroll
                for (int u = 0; u < 4; ++u) lt[u] = TT::sum2(wv[u], lt[u]);
                pb[kb][mm] = __builtin_bit_cast(v8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
            }
    };
    using sub_on = std::integral_constant<bool, true>;
    using sub_off = std::integral_constant<bool, false>;

    // this lane's largest score of the tile
    auto lane_max = [&]() {
        float mx[4 * NKB];
#pragma unroll
        for (int u = 0; u < 4 * NKB; ++u)
            mx[u] = fmaxf(fmaxf(sacc[u >> 2][4 * (u & 3)], sacc[u >> 2][4 * (u & 3) + 1]),
                          fmaxf(sacc[u >> 2][4 * (u & 3) + 2], sacc[u >> 2][4 * (u & 3) + 3]));
#pragma unroll
        for (int wd = 2 * NKB; wd >= 1; wd >>= 1)
#pragma unroll
            for (int u = 0; u < wd; ++u) mx[u] = fmaxf(mx[u], mx[u + wd]);
        return mx[0];
    };

    // Vector-ALU step k: the online softmax of S(k).  Once every row of the
    // wave has a reference, a tile without masked keys whose scores all
    // stay within PP_LAZY of the reference takes the probabilities directly;
    // otherwise the exact path masks, takes the row max and raises the
    // reference where needed (rescaling O and l) first.
    float m_lim = PP_LAZY;   // m_ref + PP_LAZY
    auto softmax_step = [&](int k) {
        if (k >= w_stop) {
            // past this wave's keys or the segment: P = 0, so the next P V
            // product adds nothing
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) pb[kb][mm] = __builtin_bit_cast(v8, make_uint4(0, 0, 0, 0));
            return;
        }
        bool fast = all_set && k < w_mask;
        if (fast) fast = __builtin_amdgcn_ballot_w64(lane_max() > m_lim) == 0;
        if (!fast) {
            {
                // the mask (a no-op before tile w_mask, where every key of
                // the tile is visible to every row of the wave)
                const int lim0 = lim_base - k * BN;
                const int lim = (lim0 < -1 ? -1 : (lim0 > BN ? BN : lim0)) - 4 * hh;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr)
                        if (32 * kb + 8 * (rr / 4) + (rr % 4) > lim) sacc[kb][rr] = -INFINITY;
            }
            const float rmax = max_with_partner(lane_max());
            const bool need = rmax - m_ref > PP_LAZY || (!m_set && rmax > -INFINITY && rmax < -64.f);
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                const float m_new = need ? rmax : m_ref;
                const float alpha = m_set ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) oacc[b][rr] *= alpha;
#pragma unroll
                for (int u = 0; u < 4; ++u) l_acc[u] *= alpha;
                m_ref = m_new;
                m_lim = m_ref + PP_LAZY;
                ref_zero = __builtin_amdgcn_ballot_w64(m_ref != 0.f) == 0;
            }
            m_set = m_set || rmax > -INFINITY;
            all_set = __builtin_amdgcn_ballot_w64(!m_set) == 0;
        }
        float lt[4];
        if (ref_zero) probs(lt, sub_off{});
        else probs(lt, sub_on{});
#pragma unroll
        for (int u = 0; u < 4; ++u) l_acc[u] += lt[u];
    };

    __syncthreads();   // K(k_beg) staged, the slot of V(k_beg - 1) zeroed

    // Ping-pong: both teams run the same sequence, matrix step k, barrier,
    // softmax k, barrier; team 1 passes one barrier first, so it runs one
    // phase behind: phase 2k holds team 0's matrix step k and team 1's
    // softmax k-1, phase 2k+1 team 0's softmax k and team 1's matrix step k.
    // K(k+1) is staged in phases 2k (team 0's half) and 2k+1 (team 1's) and
    // first read in phase 2k+2.  V(k), loaded by the matrix steps k-1, is
    // first read in phase 2k+2; waiting at the end of matrix step k until at
    // most the loads of that step are outstanding completes V(k) by the
    // end of phase 2k (team 0) or 2k+1 (team 1).
    // Together (not PING): every wave runs matrix step k, waits, passes one
    // barrier, then runs softmax k; the barrier hands over K(k+1) and V(k),
    // and the reads of K(k) and V(k-1) all precede it, so their slots may be
    // refilled in step k+1.
    auto wait_older_loads = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(SH::template nload<ROT>() | (7 << 4) | (15 << 8));   // vmcnt(loads of one step)
        __builtin_amdgcn_sched_barrier(0);
    };
    prefetch_pv(k_beg);
    if constexpr (PING) {
        if (team == 1) lds_barrier();
        for (int k = k_beg; k <= k_end; ++k) {
            mfma_step(k);
            wait_older_loads();
            lds_barrier();
            prefetch_pv(k + 1);   // V(k): complete since the phase before
            softmax_step(k);
            lds_barrier();
        }
        if (team == 0) lds_barrier();
    } else {
        for (int k = k_beg; k <= k_end; ++k) {
            mfma_step(k);
            wait_older_loads();
            lds_barrier();
            prefetch_pv(k + 1);   // V(k): complete before the barrier
            softmax_step(k);
        }
    }

    if (!wave_rows || qrow >= p.Sq) return;
    const float l_tot = sum_with_partner((l_acc[0] + l_acc[1]) + (l_acc[2] + l_acc[3]));
    if (SPLIT && partial) {
        // ---- partial state of this segment: unnormalised O, reference m
        // (-inf when no key of the segment was visible) and row sum l, as
        // [D + 2][256 rows] fp32 for the merge kernel's coalesced reads
        const int rr = 32 * gw + l32;
        float *blk = p.ws + ((int64_t)item * p.nseg + seg) * (int64_t)(D + 2) * 256;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) blk[(32 * b + 8 * g + 4 * hh + e) * 256 + rr] = oacc[b][4 * g + e];
        if (hh == 0) {
            blk[D * 256 + rr] = m_set ? m_ref : -INFINITY;
            blk[(D + 1) * 256 + rr] = l_tot;
        }
        return;
    }

    // ---- epilogue: O / l, one store per element; lse on request ----
    const float inv = 1.f / l_tot;
    uint16_t *orow = p.o + ((int64_t)bh * p.Sq + qrow) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * b + 8 * g + 4 * hh;
            uint2 wv;
            wv.x = TT::pack2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
            wv.y = TT::pack2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
            *reinterpret_cast<uint2 *>(orow + d0) = wv;
        }
    if (p.lse && hh == 0) p.lse[(int64_t)bh * p.Sq + qrow] = ((m_set ? m_ref : -INFINITY) + log2f(l_tot)) * PP_LN2;
}

// Merges the segments of every cut row block: one workgroup per (head group,
// row block, 8-dim chunk of the output), one thread per query row (thread t:
// head t / R of the group, row t mod R of the block, R = 256 / G).  With M the
// largest reference of the row's segments,
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, which is exact in real
// arithmetic (each segment's O_s and l_s are measured against its own
// reference m_s).  All loads of a thread are independent and issued
// together (at most PP_MAXSEG segments).  Runs after the main kernel on the
// same stream.
template <int D, int BN, typename E>
__global__ __launch_bounds__(256) void flash_pp_merge_kernel(PPParams p)
{
    using TT = Ty<E>;
    constexpr int NC = D / 8;
    const int hg = blockIdx.x % p.n_hg;
    const int rb = (blockIdx.x / p.n_hg) / NC;
    const int c8 = 8 * ((blockIdx.x / p.n_hg) % NC);
    const int k_all = block_tiles<BN>(p, rb);
    if (k_all <= p.seg_tiles) return;   // written by the main kernel
    const int ns = (k_all + p.seg_tiles - 1) / p.seg_tiles;
    const int t = threadIdx.x;
    const int rlog = 8 - p.g_log2;   // log2 R
    const int bh = (hg << p.g_log2) + (t >> rlog);
    const int qrow = (rb << rlog) + (t & ((1 << rlog) - 1));
    if (qrow >= p.Sq) return;
    const float *blk0 = p.ws + ((int64_t)hg * p.n_rb + rb) * p.nseg * (int64_t)(D + 2) * 256 + t;
    const int64_t sstride = (int64_t)(D + 2) * 256;
    float m[PP_MAXSEG], l[PP_MAXSEG], o[PP_MAXSEG][8];
#pragma unroll
    for (int sg = 0; sg < PP_MAXSEG; ++sg) {
        m[sg] = -INFINITY;
        l[sg] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[sg][e] = 0.f;
        if (sg < ns) {
            const float *b = blk0 + sg * sstride;
            m[sg] = b[D * 256];
            l[sg] = b[(D + 1) * 256];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[sg][e] = b[(c8 + e) * 256];
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int sg = 0; sg < PP_MAXSEG; ++sg) M = fmaxf(M, m[sg]);
    float lsum = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sg = 0; sg < PP_MAXSEG; ++sg) {
        // segments without a visible key (m = -inf, l = 0, O = 0) add nothing
        const float w = m[sg] > -INFINITY ? __builtin_amdgcn_exp2f(m[sg] - M) : 0.f;
        lsum += w * l[sg];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * o[sg][e];
    }
    const float inv = 1.f / lsum;
    uint4 wv;
    wv.x = TT::pack2(acc[0] * inv, acc[1] * inv);
    wv.y = TT::pack2(acc[2] * inv, acc[3] * inv);
    wv.z = TT::pack2(acc[4] * inv, acc[5] * inv);
    wv.w = TT::pack2(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4 *>(p.o + ((int64_t)bh * p.Sq + qrow) * D + c8) = wv;
    if (p.lse && c8 == 0) p.lse[(int64_t)bh * p.Sq + qrow] = (M + log2f(lsum)) * PP_LN2;
}

#ifndef ROPE_PP_PING64
#define ROPE_PP_PING64 1
#endif
// Schedule per head dim: ping-pong (true) or together.
template <int D> constexpr bool pp_ping() { return D == 128 ? true : (ROPE_PP_PING64 != 0); }

// Host half: kernel parameters, and the split plan (seg_tiles = 0: none).
// Row block rb (of each head group) sees k_all(rb) key tiles; when the work
// items (head groups times row blocks) are fewer than the CUs, the smallest
// segment length C is chosen whose segment count, n_hg times the sum over
// row blocks of ceil(k_all / C), still fits one workgroup per CU.
struct PPPlan {
    PPParams p;
    int64_t ws_bytes;   // workspace the split needs (0: no split)
};

// log2 of G, the query heads per workgroup: the largest of 1, 2, 4, 8 that
// divides the query heads per key/value head.
inline int pp_group_log2(int kv_group)
{
    int g = 0;
    while (g < 3 && kv_group % (2 << g) == 0) ++g;
    return g;
}

// g_log2 < 0: G from the head counts of `a`.
template <int D>
PPPlan pp_plan(const FlashArgs &a, int g_log2 = -1)
{
    constexpr int BN = ROPE_PP_BN;
    PPPlan pl;
    PPParams &p = pl.p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.BH = a.B * a.H;
    p.kv_group = a.H_kv > 0 ? a.H / a.H_kv : 1;
    p.Sq = (int)a.Sq;
    p.Sk = (int)a.Sk;
    p.q_off = a.q_off;
    p.k_off = a.k_off;
    p.cos_tab = a.cos_tab;
    p.sin_tab = a.sin_tab;
    p.table_rows = a.table_rows;
    p.rot_dim = a.rot_dim;
    p.sl2 = a.scale * 1.4426950408889634f;
    p.causal = a.causal;
    p.g_log2 = g_log2 >= 0 ? g_log2 : pp_group_log2(p.kv_group);
    const int R = 256 >> p.g_log2;   // query rows per head in a workgroup
    p.n_hg = p.BH >> p.g_log2;
    p.n_rb = (int)((a.Sq + R - 1) / R);
    p.n_kt = (int)((a.Sk + BN - 1) / BN);
    p.seg_tiles = 0;
    p.nseg = 1;
    p.ws = nullptr;
    pl.ws_bytes = 0;
    const int cus = rope_device_cu_count();
    const int64_t items = (int64_t)p.n_hg * p.n_rb;
    if (cus <= 0 || items >= cus) return pl;
    auto k_all = [&](int rb) {
        const int64_t last = (int64_t)rb * R + R - 1 < a.Sq ? (int64_t)rb * R + R - 1 : a.Sq - 1;
        if (!a.causal) return p.n_kt;
        const int64_t v = (a.q_off + last - a.k_off) / BN + 1;
        return (int)(v < p.n_kt ? v : p.n_kt);
    };
    int kmax = 0;
    for (int rb = 0; rb < p.n_rb; ++rb) kmax = k_all(rb) > kmax ? k_all(rb) : kmax;
    int C = kmax;
    for (int c = (kmax + PP_MAXSEG - 1) / PP_MAXSEG; c < kmax; ++c) {
        int64_t n = 0;
        for (int rb = 0; rb < p.n_rb; ++rb) n += (k_all(rb) + c - 1) / c;
        if (n * p.n_hg <= cus) {
            C = c;
            break;
        }
    }
    if (C >= kmax) return pl;
    p.seg_tiles = C;
    p.nseg = (kmax + C - 1) / C;
    pl.ws_bytes = items * p.nseg * (int64_t)(D + 2) * 256 * 4;
    return pl;
}

template <int D, bool SPLIT, int LAYOUT, bool ROT, bool FULL, typename E>
int launch(const PPParams &p, hipStream_t stream)
{
    constexpr int BN = ROPE_PP_BN;
    const int64_t items = (int64_t)p.n_hg * p.n_rb;
    const int64_t blocks = items * (SPLIT ? p.nseg : 1);
    if (!rope_grid_fits(blocks, 512) || !rope_grid_fits(items * (D / 8), 256)) return ROPE_LAUNCH_SHAPE;
    hipLaunchKernelGGL((flash_fwd_pp_kernel<D, BN, pp_ping<D>(), SPLIT, LAYOUT, ROT, FULL, E>), dim3((unsigned)blocks),
                       dim3(512), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return ROPE_LAUNCH_ERR;
    if (SPLIT) {
        hipLaunchKernelGGL((flash_pp_merge_kernel<D, BN, E>), dim3((unsigned)(items * (D / 8))), dim3(256), 0,
                           stream, p);
        if (hipGetLastError() != hipSuccess) return ROPE_LAUNCH_ERR;
    }
    return ROPE_LAUNCH_OK;
}

template <int D, bool SPLIT, typename E>
int launch_r(const PPParams &p, int layout, hipStream_t stream)
{
    if (p.rot_dim == 0) return launch<D, SPLIT, 1, false, false, E>(p, stream);
    const bool full = p.rot_dim == D;
    if (layout == 0)
        return full ? launch<D, SPLIT, 0, true, true, E>(p, stream) : launch<D, SPLIT, 0, true, false, E>(p, stream);
    return full ? launch<D, SPLIT, 1, true, true, E>(p, stream) : launch<D, SPLIT, 1, true, false, E>(p, stream);
}

template <int D, typename E>
int launch_d(const FlashArgs &a, hipStream_t stream)
{
    PPPlan pl = pp_plan<D>(a);
    const bool split = pl.ws_bytes > 0 && a.workspace != nullptr && a.workspace_bytes >= pl.ws_bytes;
    if (split) {
        pl.p.ws = static_cast<float *>(a.workspace);
        return launch_r<D, true, E>(pl.p, a.layout, stream);
    }
    pl.p.seg_tiles = 0;
    pl.p.nseg = 1;
    return launch_r<D, false, E>(pl.p, a.layout, stream);
}

}  // namespace

// Head dim 128, 16-bit storage.  Returns -1 (nothing launched) for shapes
// it does not take.  (The kernel also compiles for head dim 64, where it
// measured slower than the row-split kernel of flash_fwd_bf16.hip on the
// causal 1x8xSx64 shapes: with the softmax twice the matrix work per tile,
// neither schedule hides it.)
int rope_launch_flash_pp(const FlashArgs &a, hipStream_t stream)
{
    if (a.head_dim != 128 || (a.dtype != 0 && a.dtype != 2)) return -1;
    return a.dtype == 2 ? launch_d<128, _Float16>(a, stream) : launch_d<128, __bf16>(a, stream);
}

// H_kv == 0: the key/value head count is not known yet; the bytes then
// cover every head grouping a divisor of H can give.
int64_t rope_flash_pp_workspace_bytes(const FlashArgs &a)
{
    if (a.head_dim != 128 || (a.dtype != 0 && a.dtype != 2)) return 0;
    if (a.H_kv > 0) return pp_plan<128>(a).ws_bytes;
    int64_t most = 0;
    for (int g = 0; g <= 3; ++g)
        if (a.H % (1 << g) == 0) {
            const int64_t b = pp_plan<128>(a, g).ws_bytes;
            most = b > most ? b : most;
        }
    return most;
}
