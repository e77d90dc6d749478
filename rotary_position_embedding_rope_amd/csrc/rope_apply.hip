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
// requirements": fully memory-bound).  One launch covers Q and K.  A thread
// owns one 16-byte chunk column (NeoX: a low chunk and its partner high
// chunk, which is the pair layout the rotation needs, so no lane exchange;
// GPT-J: a chunk of whole adjacent pairs) for one token, loads that chunk's
// cos/sin once, and walks a strided subset of that token's heads.  Lanes of a
// wave cover consecutive chunks of several head rows, so each load
// instruction reads whole row segments.  Each element is loaded before it is
// stored by the same thread, so the in-place update is race-free.
#include "common.hpp"

namespace {

using rope::bf16hi_to_f32;
using rope::bf16lo_to_f32;
using rope::pack_bf16x2;

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
                x[2 * i] = bf16lo_to_f32(ws[i]);
                x[2 * i + 1] = bf16hi_to_f32(ws[i]);
            }
        } else if constexpr (sizeof(T) == 4 && V == 4) {
            const float4 w = *reinterpret_cast<const float4 *>(p);
            x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if constexpr (sizeof(T) == 2) x[i] = rope::bf16_to_f32(p[i]);
                else x[i] = p[i];
            }
        }
    }
    static __device__ __forceinline__ void store(T *p, const float (&x)[V])
    {
        if constexpr (sizeof(T) == 2 && V == 8) {
            uint4 w;
            w.x = pack_bf16x2(x[0], x[1]);
            w.y = pack_bf16x2(x[2], x[3]);
            w.z = pack_bf16x2(x[4], x[5]);
            w.w = pack_bf16x2(x[6], x[7]);
            *reinterpret_cast<uint4 *>(p) = w;
        } else if constexpr (sizeof(T) == 4 && V == 4) {
            *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if constexpr (sizeof(T) == 2) p[i] = rope::f32_to_bf16(x[i]);
                else p[i] = x[i];
            }
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
    hipLaunchKernelGGL((rope_apply_kernel<T, LAYOUT, V, VT>), dim3((unsigned)blocks),
                       dim3(threads), 0, stream, a, g);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int rope_launch_apply(const RopeApplyArgs &a, hipStream_t stream)
{
    const bool bf16 = a.dtype == 0;
    const int elt = bf16 ? 2 : 4;
    const int V = 16 / elt;
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
    if (bf16) {
        if (neox) {
            if (vec) return vt ? launch<uint16_t, 0, 8, true>(a, stream) : launch<uint16_t, 0, 8, false>(a, stream);
            return launch<uint16_t, 0, 1, false>(a, stream);
        }
        if (vec) return vt ? launch<uint16_t, 1, 8, true>(a, stream) : launch<uint16_t, 1, 8, false>(a, stream);
        return launch<uint16_t, 1, 2, false>(a, stream);
    }
    if (neox) {
        if (vec) return vt ? launch<float, 0, 4, true>(a, stream) : launch<float, 0, 4, false>(a, stream);
        return launch<float, 0, 1, false>(a, stream);
    }
    if (vec) return launch<float, 1, 4, false>(a, stream);   // 2 frequencies per chunk
    return launch<float, 1, 2, false>(a, stream);
}
