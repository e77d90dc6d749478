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
// Work decomposition (FlashAttention-2 style, section 7 of the same page: a
// query-block outer loop, key/value inner loop, output written once):
//   * one 256-thread workgroup per (batch*head, 128-query tile); each of its
//     4 waves owns 32 query rows;
//   * the key loop walks 64-key tiles, stopping at the last tile a query of
//     the workgroup can see; tiles past a wave's last query are skipped by
//     that wave; the element mask runs only on tiles straddling the diagonal
//     or the ragged end;
//   * heaviest query tiles are dispatched first and all tiles of one head are
//     issued to the same XCD (block index modulo the head count), so a head's
//     K/V stay in one L2.
//
// Data path per workgroup:
//   * Q: each lane loads its query row's dims straight into the matrix-core
//     operand layout, rotates in fp32 at q_off + i, rounds to bf16 and keeps
//     the tile in registers for the whole key loop.
//   * K: every visited tile is loaded once from HBM by all 256 threads,
//     rotated in fp32 at its key positions, rounded to bf16 and written to
//     LDS -- each key tile is rotated once per staging and no rotated copy
//     ever reaches HBM ("RoPE + PoPE Attention Kernels": recompute instead
//     of materialising rotated [B,H,S,D] tensors).  V is staged unrotated,
//     transposed, into LDS.  Two LDS buffers: tile t+1 is fetched into
//     registers while tile t is consumed, then written to the other buffer;
//     one barrier per tile.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a lane owns one query column,
//     so the row max / row sum of the softmax are 32 in-lane values plus one
//     exchange with the lane 32 apart.  The probabilities come out of the
//     accumulator already in the B-operand layout of the next product:
//     O^T = V^T P^T needs no LDS round trip for P.
//   * Softmax in base 2 with scale*log2(e) applied to the fp32 scores.
#include "common.hpp"

namespace {

using rope::bf16x8_t;
using rope::f32x16_t;
using rope::pack_bf16x2;

constexpr int NWAVES = 4;
constexpr int BM = 32 * NWAVES;   // queries per workgroup
constexpr int BN = 64;            // keys per tile
constexpr int KPAD = 8;           // K LDS row pitch = D + KPAD bf16 (16-byte aligned rows)
constexpr int VPAD = 4;           // V^T LDS row pitch = BN + VPAD bf16 (8-byte aligned rows)

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    int BH;
    int64_t Sq, Sk, q_off, k_off;
    const float *cos_tab, *sin_tab;
    int rot_dim;
    float sl2;          // softmax scale * log2(e)
    int causal;
    int n_qtiles;
};

__device__ __forceinline__ void unpack8(uint4 w, float (&x)[8])
{
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = rope::bf16lo_to_f32(ws[i]);
        x[2 * i + 1] = rope::bf16hi_to_f32(ws[i]);
    }
}
__device__ __forceinline__ uint4 pack8(const float (&x)[8])
{
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// Rotate the pair (a[i], b[i]) by (c[i], s[i]) for i < N: a' = a c - b s,
// b' = a s + b c.
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

// Per-thread staging plan for K tiles (fixed across tiles).
//   NeoX: a slot is two 8-dim chunks -- either a rotated pair of chunks
//         (lo at 8c, hi at 8c + rot/2) or two copied chunks past rot_dim.
//         D/16 slots per key row.
//   GPT-J / no rotation: a slot is one 8-dim chunk, rotated (whole pairs)
//         or copied.  D/8 slots per key row.
template <int D, int LAYOUT, bool ROT>
struct KPlan {
    static constexpr bool NEOX_SLOT = ROT && LAYOUT == 0;
    static constexpr int SLOTS_PER_ROW = NEOX_SLOT ? D / 16 : D / 8;
    static constexpr int ITEMS = BN * SLOTS_PER_ROW / (NWAVES * 64);
};

template <int D, int LAYOUT, bool ROT>
__global__ __launch_bounds__(256) void flash_fwd_bf16_kernel(Params p)
{
    using Plan = KPlan<D, LAYOUT, ROT>;
    constexpr int KP = D + KPAD;
    constexpr int VP = BN + VPAD;
    constexpr int KI = Plan::ITEMS;                 // K slots per thread per tile
    constexpr int VI = (BN / 2) * (D / 8) / 256;    // V items per thread per tile
    constexpr int DT = D / 16;                      // k-steps of the QK^T product
    constexpr int DB = D / 32;                      // 32-row blocks of O^T

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int bh = blockIdx.x % p.BH;
    const int rank = blockIdx.x / p.BH;
    const int qtile = p.causal ? p.n_qtiles - 1 - rank : rank;
    const int64_t q0 = (int64_t)qtile * BM;
    const uint16_t *qh = p.q + (int64_t)bh * p.Sq * D;
    const uint16_t *kh = p.k + (int64_t)bh * p.Sk * D;
    const uint16_t *vh = p.v + (int64_t)bh * p.Sk * D;
    const int rh = p.rot_dim / 2;   // table row stride

    // ---------------- Q: load, rotate, keep as MFMA B operand ----------------
    const int64_t qrow = q0 + wave * 32 + l32;
    const bool qvalid = qrow < p.Sq;
    bf16x8_t qf[DT];
    {
        float qv[DT][8];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (qvalid) w = *reinterpret_cast<const uint4 *>(qh + qrow * D + 16 * t + 8 * hh);
            unpack8(w, qv[t]);
        }
        if constexpr (ROT) {
            if (qvalid) {
                const int64_t pos = p.q_off + qrow;
                const float *crow = p.cos_tab + pos * rh;
                const float *srow = p.sin_tab + pos * rh;
                if constexpr (LAYOUT == 0) {
                    // lane holds dims 16t + 8hh + s; partner of 16t+8hh+s is
                    // 16(t + rot/32) + 8hh + s, in the same lane.
                    // (rot_dim is a multiple of 32, so tr = rot_dim/32 <= DT/2.)
                    const int tr = p.rot_dim / 32;
#pragma unroll
                    for (int t = 0; t < DT / 2; ++t) {
                        if (t < tr) {
                            const int f0 = 16 * t + 8 * hh;
                            float c[8], s[8];
                            *reinterpret_cast<float4 *>(c) = ld4(crow + f0);
                            *reinterpret_cast<float4 *>(c + 4) = ld4(crow + f0 + 4);
                            *reinterpret_cast<float4 *>(s) = ld4(srow + f0);
                            *reinterpret_cast<float4 *>(s + 4) = ld4(srow + f0 + 4);
                            // the partner chunk is t + tr; registers are only
                            // indexed with compile-time constants
#pragma unroll
                            for (int u = 1; u <= DT / 2; ++u)
                                if (u == tr) rotate_pairs<8>(qv[t], qv[t + u], c, s);
                        }
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        if (16 * t < p.rot_dim) {
                            const int f0 = 8 * t + 4 * hh;
                            float c[4], s[4], a[4], b[4];
                            *reinterpret_cast<float4 *>(c) = ld4(crow + f0);
                            *reinterpret_cast<float4 *>(s) = ld4(srow + f0);
#pragma unroll
                            for (int u = 0; u < 4; ++u) { a[u] = qv[t][2 * u]; b[u] = qv[t][2 * u + 1]; }
                            rotate_pairs<4>(a, b, c, s);
#pragma unroll
                            for (int u = 0; u < 4; ++u) { qv[t][2 * u] = a[u]; qv[t][2 * u + 1] = b[u]; }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[t][s] = (__bf16)qv[t][s];
        }
    }

    // ---------------- key loop bounds ----------------
    const int64_t q_valid = p.Sq - q0 < BM ? p.Sq - q0 : BM;
    const int64_t n_kt = (p.Sk + BN - 1) / BN;
    int64_t kt_end = n_kt;
    if (p.causal) {
        const int64_t jmax = p.q_off + q0 + q_valid - 1 - p.k_off;
        kt_end = jmax / BN + 1 < n_kt ? jmax / BN + 1 : n_kt;
    }
    // this wave's query range
    const int64_t wq0 = q0 + wave * 32;
    const int64_t wq_last = (wq0 + 31 < p.Sq ? wq0 + 31 : p.Sq - 1);
    const bool wave_has_rows = wq0 < p.Sq;

    // ---------------- staging plan ----------------
    int k_row[KI], k_mode[KI], k_d0[KI], k_d1[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int item = tid + 256 * i;
        const int row = item / Plan::SLOTS_PER_ROW;
        const int slot = item % Plan::SLOTS_PER_ROW;
        k_row[i] = row;
        if constexpr (Plan::NEOX_SLOT) {
            const int rslots = p.rot_dim / 16;
            if (slot < rslots) {
                k_mode[i] = 1;                            // rotate (lo, hi)
                k_d0[i] = 8 * slot;
                k_d1[i] = 8 * slot + rh;
            } else {
                k_mode[i] = 0;                            // copy two chunks
                k_d0[i] = p.rot_dim + 16 * (slot - rslots);
                k_d1[i] = k_d0[i] + 8;
            }
        } else {
            k_mode[i] = (ROT && 8 * slot < p.rot_dim) ? 2 : 0;
            k_d0[i] = 8 * slot;
            k_d1[i] = 0;
        }
    }
    int v_kp[VI], v_c[VI];
#pragma unroll
    for (int i = 0; i < VI; ++i) {
        const int item = tid + 256 * i;
        v_kp[i] = item / (D / 8);
        v_c[i] = item % (D / 8);
    }

    // prefetch registers
    uint4 kr0[KI], kr1[KI];
    float kc[KI][8], ks[KI][8];
    uint4 vr0[VI], vr1[VI];

    auto fetch = [&](int64_t kt) {
        const int64_t j0 = kt * BN;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int64_t j = j0 + k_row[i];
            const bool ok = j < p.Sk;
            const uint16_t *src = kh + j * D;
            kr0[i] = ok ? *reinterpret_cast<const uint4 *>(src + k_d0[i]) : make_uint4(0, 0, 0, 0);
            if constexpr (Plan::NEOX_SLOT)
                kr1[i] = ok ? *reinterpret_cast<const uint4 *>(src + k_d1[i]) : make_uint4(0, 0, 0, 0);
            if constexpr (ROT) {
                if (ok && k_mode[i] != 0) {
                    const int64_t pos = p.k_off + j;
                    const int f0 = LAYOUT == 0 ? k_d0[i] : k_d0[i] / 2;
                    const float *cr = p.cos_tab + pos * rh + f0;
                    const float *sr = p.sin_tab + pos * rh + f0;
                    *reinterpret_cast<float4 *>(kc[i]) = ld4(cr);
                    *reinterpret_cast<float4 *>(ks[i]) = ld4(sr);
                    if constexpr (LAYOUT == 0) {
                        *reinterpret_cast<float4 *>(kc[i] + 4) = ld4(cr + 4);
                        *reinterpret_cast<float4 *>(ks[i] + 4) = ld4(sr + 4);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const int64_t j = j0 + 2 * v_kp[i];
            const uint16_t *src = vh + j * D + 8 * v_c[i];
            vr0[i] = j < p.Sk ? *reinterpret_cast<const uint4 *>(src) : make_uint4(0, 0, 0, 0);
            vr1[i] = j + 1 < p.Sk ? *reinterpret_cast<const uint4 *>(src + D) : make_uint4(0, 0, 0, 0);
        }
    };

    auto stage = [&](int buf) {
        uint16_t *kdst = Ks[buf];
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            uint16_t *row = kdst + k_row[i] * KP;
            if (k_mode[i] == 1) {
                float lo[8], hi[8];
                unpack8(kr0[i], lo);
                unpack8(kr1[i], hi);
                rotate_pairs<8>(lo, hi, kc[i], ks[i]);
                *reinterpret_cast<uint4 *>(row + k_d0[i]) = pack8(lo);
                *reinterpret_cast<uint4 *>(row + k_d1[i]) = pack8(hi);
            } else if (k_mode[i] == 2) {
                float x[8], a[4], b[4];
                unpack8(kr0[i], x);
#pragma unroll
                for (int u = 0; u < 4; ++u) { a[u] = x[2 * u]; b[u] = x[2 * u + 1]; }
                rotate_pairs<4>(a, b, kc[i], ks[i]);
#pragma unroll
                for (int u = 0; u < 4; ++u) { x[2 * u] = a[u]; x[2 * u + 1] = b[u]; }
                *reinterpret_cast<uint4 *>(row + k_d0[i]) = pack8(x);
            } else {
                *reinterpret_cast<uint4 *>(row + k_d0[i]) = kr0[i];
                if constexpr (Plan::NEOX_SLOT) *reinterpret_cast<uint4 *>(row + k_d1[i]) = kr1[i];
            }
        }
        // V^T: element (dim d, key j) at Vt[d * VP + j]; a thread writes the
        // two keys (2kp, 2kp+1) of 8 dims as 8 packed dwords.
        uint16_t *vdst = Vt[buf];
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const uint32_t a[4] = {vr0[i].x, vr0[i].y, vr0[i].z, vr0[i].w};
            const uint32_t b[4] = {vr1[i].x, vr1[i].y, vr1[i].z, vr1[i].w};
            uint16_t *col = vdst + (8 * v_c[i]) * VP + 2 * v_kp[i];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                *reinterpret_cast<uint32_t *>(col + (2 * u) * VP) = (a[u] & 0xffffu) | (b[u] << 16);
                *reinterpret_cast<uint32_t *>(col + (2 * u + 1) * VP) = (a[u] >> 16) | (b[u] & 0xffff0000u);
            }
        }
    };

    // ---------------- running state ----------------
    f32x16_t oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = (f32x16_t){};
    float m_run = -INFINITY;   // running max (scaled, base 2), same in lanes l and l^32
    float l_part = 0.f;        // this lane's share of the running denominator

    fetch(0);
    stage(0);

    for (int64_t kt = 0; kt < kt_end; ++kt) {
        const int buf = (int)(kt & 1);
        __syncthreads();   // tile kt staged; tile kt-1 fully consumed
        const bool more = kt + 1 < kt_end;
        if (more) fetch(kt + 1);

        const int64_t j0 = kt * BN;
        const bool wave_active =
            wave_has_rows && (!p.causal || p.k_off + j0 <= p.q_off + wq_last);
        if (wave_active) {
            const uint16_t *kb_lds = Ks[buf];
            const uint16_t *vt_lds = Vt[buf];
            // S^T = K Q^T: two 32-key blocks x 32 queries.
            f32x16_t sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = (f32x16_t){};
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                        kb_lds + (kb * 32 + l32) * KP + 16 * t + 8 * hh);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], sacc[kb], 0, 0, 0);
                }
            }
            // accumulator element r of block kb <-> key j0 + 32kb + 8(r/4) + 4hh + r%4
            const bool need_mask = (j0 + BN > p.Sk) ||
                                   (p.causal && p.k_off + j0 + BN - 1 > p.q_off + wq0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t j = j0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
                        const bool ok = j < p.Sk && (!p.causal || p.k_off + j <= p.q_off + qrow);
                        if (!ok) sacc[kb][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx * p.sl2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.sl2, -m_use));
                    sacc[kb][r] = pr;
                    lsum += pr;
                }
            l_part = l_part * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

            // O^T += V^T P^T.  For key sub-step mm of block kb, B-operand slot
            // s holds accumulator element 8mm + s, i.e. key
            // 32kb + 16mm + 8(s/4) + 4hh + s%4; the A operand takes the same
            // keys from V^T row d: two runs of 4 contiguous keys.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    bf16x8_t pb;
#pragma unroll
                    for (int s = 0; s < 8; ++s) pb[s] = (__bf16)sacc[kb][8 * mm + s];
#pragma unroll
                    for (int b = 0; b < DB; ++b) {
                        const uint16_t *vrow = vt_lds + (32 * b + l32) * VP + 32 * kb + 16 * mm + 4 * hh;
                        const uint2 x0 = *reinterpret_cast<const uint2 *>(vrow);
                        const uint2 x1 = *reinterpret_cast<const uint2 *>(vrow + 8);
                        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(x0.x, x0.y, x1.x, x1.y));
                        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[b], 0, 0, 0);
                    }
                }
        }
        if (more) stage(buf ^ 1);
    }

    // ---------------- epilogue: O = O_acc / l ----------------
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (qvalid) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = p.o + ((int64_t)bh * p.Sq + qrow) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * b + 8 * g + 4 * hh;
                uint2 w;
                w.x = pack_bf16x2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
                w.y = pack_bf16x2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + d0) = w;
            }
    }
}

template <int D, int LAYOUT, bool ROT>
int launch(const FlashArgs &a, hipStream_t stream)
{
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.BH = a.B * a.H;
    p.Sq = a.Sq; p.Sk = a.Sk; p.q_off = a.q_off; p.k_off = a.k_off;
    p.cos_tab = a.cos_tab; p.sin_tab = a.sin_tab; p.rot_dim = a.rot_dim;
    p.sl2 = a.scale * 1.4426950408889634f;
    p.causal = a.causal;
    p.n_qtiles = (int)((a.Sq + BM - 1) / BM);
    const int64_t blocks = (int64_t)p.BH * p.n_qtiles;
    hipLaunchKernelGGL((flash_fwd_bf16_kernel<D, LAYOUT, ROT>), dim3((unsigned)blocks), dim3(256),
                       0, stream, p);
    return hipGetLastError() == hipSuccess ? ROPE_LAUNCH_OK : ROPE_LAUNCH_ERR;
}

}  // namespace

int rope_launch_flash_bf16(const FlashArgs &a, hipStream_t stream)
{
    const bool rot = a.rot_dim > 0;
    if (a.head_dim == 64) {
        if (!rot) return launch<64, 1, false>(a, stream);
        return a.layout == 0 ? launch<64, 0, true>(a, stream) : launch<64, 1, true>(a, stream);
    }
    if (!rot) return launch<128, 1, false>(a, stream);
    return a.layout == 0 ? launch<128, 0, true>(a, stream) : launch<128, 1, true>(a, stream);
}
