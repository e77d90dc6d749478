// rope_apply.hip -- standalone in-place RoPE over a ragged continuous batch.
//
// What it computes ("Write Triton Rope Kernel", "Required reasoning process"
// steps 3-10): for every token t and every Q head and K head, the first
// rot_dim dims of the row are rotated pairwise at the token's own position
// positions[t], reading the fp32 cos/sin row of that position; rotation in
// fp32, result rounded back to the storage type; dims >= rot_dim are not
// touched.  NeoX pairs (i, i + rot_dim/2); GPT-J pairs (2i, 2i+1).
//
// MI355X design: the op moves 2 * (H_q + H_kv) * rot_dim * elt bytes per
// token and does ~7 flops per pair, so it is HBM-bound ("Performance
// requirements": fully memory-bound).  One launch covers Q and K.  Two
// kernels:
//   - rope_apply_rows_kernel, for 16-byte aligned rows whose rotated span is
//     a power-of-two number of 16-byte vectors (the common head sizes): lanes
//     cover each row's rotated span contiguously, NeoX partners are swapped
//     between lanes, and each thread keeps several heads' loads in flight;
//     row data moves with non-temporal loads and stores.
//   - rope_apply_kernel for everything else (unaligned strides, odd spans,
//     very many heads): a thread owns one chunk column (NeoX: a low chunk and
//     its partner high chunk; GPT-J: a chunk of whole adjacent pairs) for one
//     token, loads that chunk's cos/sin once, and walks a strided subset of
//     the token's heads.
// In both, each element is loaded before it is stored by the same thread (the
// lane exchange happens between a pair's load and its stores), so the
// in-place update is race-free.
#include "common.hpp"

namespace {

using rope::bf16hi_to_f32;
using rope::bf16lo_to_f32;
using rope::pack_bf16x2;

// Storage types: uint16_t holds bf16 bit patterns, _Float16 is IEEE binary16,
// float is fp32.  Widening is exact; narrowing rounds to nearest even.
template <typename T> struct Elt;
template <> struct Elt<uint16_t> {
    static __device__ __forceinline__ float lo(uint32_t w) { return bf16lo_to_f32(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return bf16hi_to_f32(w); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
    static __device__ __forceinline__ float get(uint16_t v) { return rope::bf16_to_f32(v); }
    static __device__ __forceinline__ uint16_t put(float x) { return rope::f32_to_bf16(x); }
};
template <> struct Elt<_Float16> {
    static __device__ __forceinline__ float lo(uint32_t w) { return rope::f16lo_to_f32(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return rope::f16hi_to_f32(w); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return rope::pack_f16x2(a, b); }
    static __device__ __forceinline__ float get(_Float16 v) { return (float)v; }
    static __device__ __forceinline__ _Float16 put(float x) { return (_Float16)x; }
};
template <> struct Elt<float> {
    static __device__ __forceinline__ float get(float v) { return v; }
    static __device__ __forceinline__ float put(float x) { return x; }
};

// V contiguous elements of T <-> float[V].
template <typename T, int V>
struct Access {
    static __device__ __forceinline__ void load(const T *p, float (&x)[V])
    {
        if constexpr (sizeof(T) == 2 && V == 8) {
            const uint4 w = *reinterpret_cast<const uint4 *>(p);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = Elt<T>::lo(ws[i]);
                x[2 * i + 1] = Elt<T>::hi(ws[i]);
            }
        } else if constexpr (sizeof(T) == 4 && V == 4) {
            const float4 w = *reinterpret_cast<const float4 *>(p);
            x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) x[i] = Elt<T>::get(p[i]);
        }
    }
    static __device__ __forceinline__ void store(T *p, const float (&x)[V])
    {
        if constexpr (sizeof(T) == 2 && V == 8) {
            uint4 w;
            w.x = Elt<T>::pack(x[0], x[1]);
            w.y = Elt<T>::pack(x[2], x[3]);
            w.z = Elt<T>::pack(x[4], x[5]);
            w.w = Elt<T>::pack(x[6], x[7]);
            *reinterpret_cast<uint4 *>(p) = w;
        } else if constexpr (sizeof(T) == 4 && V == 4) {
            *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) p[i] = Elt<T>::put(x[i]);
        }
    }
};

template <int N>
__device__ __forceinline__ void load_f32(const float *p, float (&x)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 w = *reinterpret_cast<const float4 *>(p + i);
            x[i] = w.x; x[i + 1] = w.y; x[i + 2] = w.z; x[i + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = p[i];
    }
}

struct ApplyGeom {
    int chunks;          // chunk columns per row
    int chunk_lanes;     // threads across the chunk columns (min(chunks, 256))
    int head_slots;      // threads per (token, chunk column) walking the heads
    int tokens_per_block;
};

// LAYOUT 0 = NeoX, 1 = GPT-J.  V = elements per access.  VEC_TABLE: the
// table row slice of a chunk may be read with 16-byte loads.
template <typename T, int LAYOUT, int V, bool VEC_TABLE>
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeApplyArgs a, ApplyGeom g)
{
    constexpr int NF = LAYOUT == 0 ? V : V / 2;   // frequencies per chunk
    const int tid = threadIdx.x;
    const int chunk0 = tid % g.chunk_lanes;
    const int r = tid / g.chunk_lanes;
    const int head_sub = r % g.head_slots;
    const int tok_local = r / g.head_slots;
    if (tok_local >= g.tokens_per_block) return;
    const int64_t token = (int64_t)blockIdx.x * g.tokens_per_block + tok_local;
    if (token >= a.n_tokens) return;

    const int half = a.rot_dim / 2;
    int64_t pos = a.positions[token];
    pos = pos < 0 ? 0 : (pos >= a.table_rows ? a.table_rows - 1 : pos);

    const int heads = a.h_q + a.h_kv;
    T *const qbase = static_cast<T *>(a.q) + token * a.q_stride_tok;
    T *const kbase = static_cast<T *>(a.k) + token * a.k_stride_tok;

    for (int chunk = chunk0; chunk < g.chunks; chunk += g.chunk_lanes) {
    const int f0 = LAYOUT == 0 ? chunk * V : chunk * (V / 2);
    float c[NF], s[NF];
    if constexpr (VEC_TABLE) {
        load_f32<NF>(a.cos_tab + pos * half + f0, c);
        load_f32<NF>(a.sin_tab + pos * half + f0, s);
    } else {
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            c[i] = a.cos_tab[pos * half + f0 + i];
            s[i] = a.sin_tab[pos * half + f0 + i];
        }
    }

#pragma unroll 2
    for (int h = head_sub; h < heads; h += g.head_slots) {
        T *row = h < a.h_q ? qbase + (int64_t)h * a.q_stride_head
                           : kbase + (int64_t)(h - a.h_q) * a.k_stride_head;
        if constexpr (LAYOUT == 0) {
            T *lo_p = row + chunk * V;
            T *hi_p = lo_p + half;
            float lo[V], hi[V];
            Access<T, V>::load(lo_p, lo);
            Access<T, V>::load(hi_p, hi);
            float olo[V], ohi[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                olo[i] = lo[i] * c[i] - hi[i] * s[i];
                ohi[i] = lo[i] * s[i] + hi[i] * c[i];
            }
            Access<T, V>::store(lo_p, olo);
            Access<T, V>::store(hi_p, ohi);
        } else {
            T *p = row + chunk * V;
            float x[V];
            Access<T, V>::load(p, x);
            float y[V];
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                y[2 * i] = x[2 * i] * c[i] - x[2 * i + 1] * s[i];
                y[2 * i + 1] = x[2 * i] * s[i] + x[2 * i + 1] * c[i];
            }
            Access<T, V>::store(p, y);
        }
    }
    }
}

template <typename T, int LAYOUT, int V, bool VT>
int launch(const RopeApplyArgs &a, hipStream_t stream)
{
    ApplyGeom g;
    const int half = a.rot_dim / 2;
    g.chunks = LAYOUT == 0 ? half / V : a.rot_dim / V;
    g.chunk_lanes = g.chunks < 256 ? g.chunks : 256;
    const int heads = a.h_q + a.h_kv;
    // Head slots: a power of two with chunk_lanes * slots <= 64 (at most one
    // wave per token) and no more slots than heads.
    int slots = 1;
    while (slots * 2 * g.chunk_lanes <= 64 && slots * 2 <= heads) slots *= 2;
    g.head_slots = slots;
    const int per_token = g.chunk_lanes * g.head_slots;
    g.tokens_per_block = 256 / per_token;
    const int threads = g.tokens_per_block * per_token;
    const int64_t blocks = (a.n_tokens + g.tokens_per_block - 1) / g.tokens_per_block;
    if (!rope_grid_fits(blocks, threads)) return ROPE_LAUNCH_SHAPE;
    hipLaunchKernelGGL((rope_apply_kernel<T, LAYOUT, V, VT>), dim3((unsigned)blocks),
                       dim3(threads), 0, stream, a, g);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of T <-> float[16 / sizeof(T)].
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4_t w, float (&x)[16 / sizeof(T)])
{
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = Elt<T>::lo(w[i]); x[2 * i + 1] = Elt<T>::hi(w[i]); }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
    }
}
template <typename T>
__device__ __forceinline__ u32x4_t pack16(const float (&y)[16 / sizeof(T)])
{
    u32x4_t w;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = Elt<T>::pack(y[2 * i], y[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(y[i]);
    }
    return w;
}

// Row-contiguous path (16-byte aligned rows, the rotated span a power-of-two
// number L of 16-byte vectors): lane j of a group of L lanes covers elements
// [VE*j, VE*j + VE) of one row's rotated span, so every load instruction
// reads whole contiguous spans.  NeoX: lanes j < L/2 hold low-half chunks,
// the others their high-half partners; the two lanes of a pair swap their
// chunks (lane xor L/2, inside one wave because L divides 64) and each
// computes its own half.  GPT-J: whole adjacent pairs per lane.  Group g
// serves token g / slots and its heads hs, hs + slots, ... (hs = g % slots),
// in batches of BATCH rows whose loads are all issued before any store; the
// first batch is issued before the position and cos/sin loads.
// UNIFORM: each wave serves a single token (slots * L a multiple of 64), so
// the token index, its position and its table row address are scalar.  Loads
// are never predicated (lanes past the end read a clamped, valid row and
// store nothing), so no load waits on another.  Row data is streamed once:
// loads and stores carry the non-temporal hint; the cos/sin rows, shared by
// a token's heads, are ordinary cached loads.
template <typename T, int LAYOUT, int L, int BATCH, bool UNIFORM>
__global__ __launch_bounds__(256) void rope_apply_rows_kernel(RopeApplyArgs a, int64_t q_sh, int64_t k_sh,
                                                              int head_slots, int heads_per_thread,
                                                              int64_t groups)
{
    constexpr int VE = 16 / sizeof(T);                    // elements per 16-byte vector
    constexpr int NF = LAYOUT == 0 ? VE : VE / 2;         // frequencies per lane
    const int j = threadIdx.x % L;
    int64_t group = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / L;
    const bool live = group < groups;   // no early return: shuffles below
    if (!live) group = groups - 1;
    int64_t token = group / head_slots;
    if constexpr (UNIFORM) {
        const uint64_t t = (uint64_t)token;
        token = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(t >> 32)) << 32) |
                          __builtin_amdgcn_readfirstlane((uint32_t)t));
    }
    const int hs = (int)(group - token * head_slots);
    const int half = a.rot_dim / 2;
    const int heads = a.h_q + a.h_kv;

    T *const qbase = static_cast<T *>(a.q) + token * a.q_stride_tok + VE * j;
    T *const kbase = static_cast<T *>(a.k) + token * a.k_stride_tok + VE * j;
    u32x4_t *rows[BATCH];
    bool ok[BATCH];
    u32x4_t raw[BATCH];
    auto issue = [&](int u0) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            int h = hs + (u0 + u) * head_slots;
            ok[u] = live && h < heads;
            h = h < heads ? h : heads - 1;
            rows[u] = reinterpret_cast<u32x4_t *>(h < a.h_q ? qbase + (int64_t)h * q_sh
                                                            : kbase + (int64_t)(h - a.h_q) * k_sh);
            raw[u] = __builtin_nontemporal_load(rows[u]);
        }
    };
    issue(0);   // the first rows are in flight while the position and cos/sin resolve
    __builtin_amdgcn_sched_barrier(0);   // keep them ahead of the position lookup

    int64_t pos = a.positions[token];
    pos = pos < 0 ? 0 : (pos >= a.table_rows ? a.table_rows - 1 : pos);
    const int f0 = LAYOUT == 0 ? VE * (j % (L / 2)) : (VE / 2) * j;
    float c[NF], s[NF];
    load_f32<NF>(a.cos_tab + pos * half + f0, c);
    load_f32<NF>(a.sin_tab + pos * half + f0, s);

    for (int u0 = 0; u0 < heads_per_thread; u0 += BATCH) {   // uniform trip count
        if (u0 > 0) issue(u0);
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            float x[VE], y[VE];
            unpack16<T>(raw[u], x);
            if constexpr (LAYOUT == 0) {
                // partner chunk from lane j ^ L/2 (every lane executes the shuffles)
                u32x4_t pr;
#pragma unroll
                for (int i = 0; i < 4; ++i) pr[i] = __shfl_xor(raw[u][i], L / 2);
                float z[VE];
                unpack16<T>(pr, z);
                const bool lo = j < L / 2;
#pragma unroll
                for (int i = 0; i < VE; ++i)   // lo: a c - b s (b = partner); hi: b c + a s (a = partner)
                    y[i] = lo ? x[i] * c[i] - z[i] * s[i] : z[i] * s[i] + x[i] * c[i];
            } else {
#pragma unroll
                for (int i = 0; i < VE / 2; ++i) {
                    y[2 * i] = x[2 * i] * c[i] - x[2 * i + 1] * s[i];
                    y[2 * i + 1] = x[2 * i] * s[i] + x[2 * i + 1] * c[i];
                }
            }
            if (ok[u]) __builtin_nontemporal_store(pack16<T>(y), rows[u]);
        }
    }
}

// Row loads in flight per thread.  5 keeps a thread at 60 VGPRs (8 waves per
// SIMD, so a 40-head batch of 8192 tokens is resident in one round) and
// measured ahead of 2, 3 and 4 on that workload.
constexpr int kRowsBatch = 5;

// Head slots of the row-contiguous path: groups of one token fill whole
// waves where the heads allow it (slots * L a multiple of 64: the wave's
// position and cos/sin loads are uniform); more slots (2x, 4x, ...) while the
// grid is too small to fill the GPU and threads would walk more than one
// batch of heads.
int rows_slots(int heads, int L, int64_t n_tokens)
{
    int slots = 64 / L;
    if (slots >= heads) return heads;
    const int64_t fill = 256 * 4 * 8 * 64;   // CUs x SIMDs x waves x lanes
    while (slots * 2 <= heads && (heads + slots - 1) / slots > kRowsBatch &&
           n_tokens * slots * L < fill)
        slots *= 2;
    return slots;
}

template <typename T, int LAYOUT, int L>
int launch_rows(const RopeApplyArgs &a, hipStream_t stream)
{
    const int heads = a.h_q + a.h_kv;
    const int slots = rows_slots(heads, L, a.n_tokens);
    const int hpt = (heads + slots - 1) / slots;
    const int64_t groups = a.n_tokens * slots;
    const int64_t blocks = (groups * L + 255) / 256;
    if (!rope_grid_fits(blocks, 256)) return -1;   // the general kernel checks its own grid
    if ((slots * L) % 64 == 0)
        hipLaunchKernelGGL((rope_apply_rows_kernel<T, LAYOUT, L, kRowsBatch, true>), dim3((unsigned)blocks),
                           dim3(256), 0, stream, a, a.q_stride_head, a.k_stride_head, slots, hpt, groups);
    else
        hipLaunchKernelGGL((rope_apply_rows_kernel<T, LAYOUT, L, kRowsBatch, false>), dim3((unsigned)blocks),
                           dim3(256), 0, stream, a, a.q_stride_head, a.k_stride_head, slots, hpt, groups);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

template <typename T, int LAYOUT>
int dispatch_rows(const RopeApplyArgs &a, int L, hipStream_t stream)
{
    switch (L) {
    case 2: return launch_rows<T, LAYOUT, 2>(a, stream);
    case 4: return launch_rows<T, LAYOUT, 4>(a, stream);
    case 8: return launch_rows<T, LAYOUT, 8>(a, stream);
    case 16: return launch_rows<T, LAYOUT, 16>(a, stream);
    case 32: return launch_rows<T, LAYOUT, 32>(a, stream);
    default: return -1;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T>
int launch_typed(const RopeApplyArgs &a, hipStream_t stream)
{
    constexpr int elt = (int)sizeof(T);
    constexpr int V = 16 / elt;
    const int half = a.rot_dim / 2;
    const bool neox = a.layout == 0;
    // 16-byte path: row starts 16-byte aligned for every token/head, and the
    // rotated span splits into whole 16-byte chunks.
    bool vec = (neox ? half % V == 0 : a.rot_dim % V == 0);
    if (a.h_q > 0)
        vec = vec && aligned16(a.q) && (a.q_stride_tok * elt) % 16 == 0 && (a.q_stride_head * elt) % 16 == 0;
    if (a.h_kv > 0)
        vec = vec && aligned16(a.k) && (a.k_stride_tok * elt) % 16 == 0 && (a.k_stride_head * elt) % 16 == 0;
    // cos/sin rows: 16-byte loads need a 16-byte-aligned row slice per chunk.
    const bool vt = vec && aligned16(a.cos_tab) && aligned16(a.sin_tab) && (half * 4) % 16 == 0 &&
                    (neox ? (V * 4) % 16 == 0 : ((V / 2) * 4) % 16 == 0);
    // row-contiguous path: 16-byte aligned rows and table, the rotated span a
    // power-of-two number of 16-byte vectors, 16-byte table slices per lane
    if (vec && vt) {
        const int L = a.rot_dim / V;
        const bool pow2 = L >= 2 && L <= 32 && (L & (L - 1)) == 0;
        if (pow2) {
            const int rc = neox ? dispatch_rows<T, 0>(a, L, stream) : dispatch_rows<T, 1>(a, L, stream);
            if (rc >= 0) return rc;
        }
    }
    if constexpr (elt == 2) {
        if (neox) {
            if (vec) return vt ? launch<T, 0, 8, true>(a, stream) : launch<T, 0, 8, false>(a, stream);
            return launch<T, 0, 1, false>(a, stream);
        }
        if (vec) return vt ? launch<T, 1, 8, true>(a, stream) : launch<T, 1, 8, false>(a, stream);
        return launch<T, 1, 2, false>(a, stream);
    } else {
        if (neox) {
            if (vec) return vt ? launch<T, 0, 4, true>(a, stream) : launch<T, 0, 4, false>(a, stream);
            return launch<T, 0, 1, false>(a, stream);
        }
        if (vec) return launch<T, 1, 4, false>(a, stream);   // 2 frequencies per chunk
        return launch<T, 1, 2, false>(a, stream);
    }
}

}  // namespace

int rope_launch_apply(const RopeApplyArgs &a, hipStream_t stream)
{
    switch (a.dtype) {
    case 0: return launch_typed<uint16_t>(a, stream);
    case 1: return launch_typed<float>(a, stream);
    case 2: return launch_typed<_Float16>(a, stream);
    default: return ROPE_LAUNCH_ERR;
    }
}
