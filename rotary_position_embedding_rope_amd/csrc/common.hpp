// common.hpp -- device helpers shared by the gfx950 kernels of this library:
// bf16 <-> fp32 conversion, vector types for 16-byte accesses, and the
// launcher interface that abi.cpp calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rope {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// bf16 storage is handled as raw uint16 bit patterns; widening is exact.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 values rounded to nearest-even bf16 (v_cvt_pk_bf16_f32), packed
// low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
// IEEE binary16 halves of a 32-bit word; two fp32 values rounded to nearest
// even binary16 and packed (low half first).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16lo_to_f32(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16hi_to_f32(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// The 16-bit storage types: bf16 and IEEE fp16.  Each gives the widening of
// the low / high half of a 32-bit word, the rounding (to nearest even) of two
// floats into one word, the matrix-core products of its type (32x32x16 and
// 16x16x32), the sum of a word's two halves into an fp32 accumulator (one
// v_dot2 against (1, 1)) and the bits of a quiet NaN.
template <typename E> struct Ty;
template <> struct Ty<__bf16> {
    using v8 = bf16x8_t;
    static __device__ __forceinline__ float lo(uint32_t w) { return bf16lo_to_f32(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return bf16hi_to_f32(w); }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
    static __device__ __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mfma16(v8 a, v8 b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(uint32_t w, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                               __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
    }
    static constexpr uint16_t QNAN = 0x7fc0;
};
template <> struct Ty<_Float16> {
    using v8 = f16x8_t;
    static __device__ __forceinline__ float lo(uint32_t w) { return f16lo_to_f32(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return f16hi_to_f32(w); }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_f16x2(a, b); }
    static __device__ __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mfma16(v8 a, v8 b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(uint32_t w, float acc)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3c003c00u),
                                      acc, false);
    }
    static constexpr uint16_t QNAN = 0x7e00;
};

// One 16-bit element of type E <-> fp32 (bits held in a uint16_t).
template <typename E>
__device__ __forceinline__ float elt_to_f32(uint16_t b) { return Ty<E>::lo((uint32_t)b); }
template <typename E>
__device__ __forceinline__ uint16_t f32_to_elt(float x) { return (uint16_t)(Ty<E>::pack2(x, 0.f) & 0xffffu); }


}  // namespace rope

// Status values returned by the launchers (mirror include/rope_mi355x.h).
#define ROPE_LAUNCH_OK 0
#define ROPE_LAUNCH_SHAPE 2   // the grid would not fit one launch: nothing was enqueued
#define ROPE_LAUNCH_ERR 7

// A 1-D launch holds at most 2^32 - 1 work-items in all (grid blocks times
// block threads); launchers check every grid of a call before the first
// launch and return ROPE_LAUNCH_SHAPE when one does not fit.
inline bool rope_grid_fits(int64_t blocks, int threads)
{
    return blocks >= 1 && threads >= 1 && blocks <= (int64_t)0xffffffffLL / threads;
}

// Host launchers, one per kernel family.  Arguments are validated by abi.cpp
// before these are called; each returns ROPE_LAUNCH_OK, ROPE_LAUNCH_SHAPE
// (before any launch) or ROPE_LAUNCH_ERR.
int rope_launch_tables(double base, int rot_dim, int64_t max_pos, double pos_div, float *cos_out,
                       float *sin_out, hipStream_t stream);

struct RopeApplyArgs {
    void *q;
    int64_t q_stride_tok, q_stride_head;
    int h_q;
    void *k;
    int64_t k_stride_tok, k_stride_head;
    int h_kv;
    const int32_t *positions;
    int64_t n_tokens;
    const float *cos_tab, *sin_tab;
    int64_t table_rows;
    int head_dim, rot_dim, layout, dtype;
};
int rope_launch_apply(const RopeApplyArgs &a, hipStream_t stream);

struct FlashArgs {
    const void *q, *k, *v;
    void *o;
    int B, H, H_kv;   // query heads, key/value heads (H_kv divides H)
    int64_t Sq, Sk;
    int head_dim;
    int64_t q_off, k_off;
    const float *cos_tab, *sin_tab;
    int64_t table_rows;
    int rot_dim, layout, causal;
    float scale;   // already resolved (> 0)
    int dtype;
    float *lse;                // [B, H, Sq] log-sum-exp of each query row, or NULL
    void *workspace;           // zero-filled scratch for the balanced schedule, or NULL
    int64_t workspace_bytes;
};
int rope_launch_flash_bf16(const FlashArgs &a, hipStream_t stream);
// Workspace bytes the bf16 launch would use for these shapes on the current
// device (0: the launch needs none).
int64_t rope_flash_bf16_workspace_bytes(const FlashArgs &a);
int rope_launch_flash_f32(const FlashArgs &a, hipStream_t stream);
// Head dim 128 (bf16 / fp16): the two-team kernel of flash_fwd_pp.hip;
// -1 when it does not take the shape (nothing launched).
int rope_launch_flash_pp(const FlashArgs &a, hipStream_t stream);
// Workspace bytes its split-key schedule would use (0: none).
int64_t rope_flash_pp_workspace_bytes(const FlashArgs &a);

struct FlashBwdArgs {
    const void *q, *k, *v, *o, *dout;   // q, o, dout [B, H, Sq, D]; k, v [B, H_kv, Sk, D]
    const float *lse;                   // [B, H, Sq] from the forward
    void *dq, *dk, *dv;
    int B, H, H_kv;
    int64_t Sq, Sk;
    int head_dim;
    int64_t q_off, k_off;
    const float *cos_tab, *sin_tab;
    int rot_dim, layout, causal;
    float scale;                        // already resolved (> 0)
    int dtype;                          // 0 bf16, 2 fp16
    void *workspace;                    // rope_flash_bwd_workspace_bytes() bytes
};
int rope_launch_flash_bwd_bf16(const FlashBwdArgs &a, hipStream_t stream);
int64_t rope_flash_bwd_workspace_bytes(int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim, int rot_dim);

struct DecodeArgs {
    const void *q, *k_new, *v_new;   // [B, H, D], [B, H_kv, D], [B, H_kv, D]
    void *k_cache, *v_cache;         // [B, H_kv, S_max, D]
    const int32_t *cache_lens;       // [B]
    void *o;                         // [B, H, D]
    int B, H, H_kv;
    int64_t S_max;
    int head_dim;
    const float *cos_tab, *sin_tab;
    int64_t table_rows;
    int rot_dim, layout;
    float scale;                     // already resolved (> 0)
    int dtype;                       // 0 bf16, 2 fp16
    void *workspace;                 // rope_decode_workspace_bytes() bytes
};
int rope_launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);
// Workspace bytes of one decode step (any device).
int64_t rope_decode_workspace_bytes(int B, int H, int H_kv, int head_dim);
// Passes of 64 cached positions the step may walk: an upper bound the host
// checks so that device-side pass counts fit in 32 bits.
int64_t rope_decode_max_passes(int B, int H_kv, int64_t S_max);
// The current device's copy of the static decode scratch
// (ROPE_DECODE_SCRATCH_BYTES), looked up on the first call per device;
// nullptr if HIP cannot give its address.
void *rope_decode_static_scratch();

// Compute units of the current device (cached per device; 0 on error).
int rope_device_cu_count();
