// abi.cpp -- the extern "C" entry points of include/rope_mi355x.h.
//
// Every entry point validates all host-visible arguments first and returns a
// status without touching HIP when one is wrong; only then does it pick a
// kernel instantiation and enqueue it on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "common.hpp"
#include "rope_mi355x.h"

namespace {

// Bound on the block counts the launchers form in 32-bit arithmetic; each
// launcher also checks its exact grid against the 2^32 - 1 work-item limit
// of one launch (ROPE_ERR_SHAPE when it does not fit).
constexpr int64_t kMaxGrid = 2147483647;

bool aligned(const void *p, unsigned bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// Launcher status -> API status.
int api_status(int rc)
{
    return rc == ROPE_LAUNCH_OK ? ROPE_OK : (rc == ROPE_LAUNCH_SHAPE ? ROPE_ERR_SHAPE : ROPE_ERR_HIP);
}

// Bytes of a dense tensor with these dims and element size (saturating at
// INT64_MAX, so an absurd shape still compares as "large").
int64_t bytes_of(std::initializer_list<int64_t> dims, int64_t elt)
{
    int64_t n = elt;
    for (int64_t d : dims) {
        if (d <= 0) return 0;
        if (n > INT64_MAX / d) return INT64_MAX;
        n *= d;
    }
    return n;
}

// Whether two byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    const uintptr_t xe = (uint64_t)na > UINTPTR_MAX - x ? UINTPTR_MAX : x + (uintptr_t)na;
    const uintptr_t ye = (uint64_t)nb > UINTPTR_MAX - y ? UINTPTR_MAX : y + (uintptr_t)nb;
    return x < ye && y < xe;
}

struct Span {
    const void *p;
    int64_t n;
};
// Whether any written range overlaps another written range or a read range.
bool any_overlap(std::initializer_list<Span> writes, std::initializer_list<Span> reads)
{
    for (auto w = writes.begin(); w != writes.end(); ++w) {
        for (auto w2 = w + 1; w2 != writes.end(); ++w2)
            if (overlaps(w->p, w->n, w2->p, w2->n)) return true;
        for (const Span &r : reads)
            if (overlaps(w->p, w->n, r.p, r.n)) return true;
    }
    return false;
}

int elt_size(int dtype) { return dtype == ROPE_F32 ? 4 : 2; }

// dtypes of the fused forward and rope_apply
bool valid_dtype(int dtype) { return dtype == ROPE_BF16 || dtype == ROPE_F32 || dtype == ROPE_F16; }
bool valid_apply_dtype(int dtype) { return valid_dtype(dtype); }
bool valid_layout(int layout) { return layout == ROPE_NEOX || layout == ROPE_GPTJ; }

// Rows (t, h) of one tensor must not overlap: stride_head >= head_dim when
// there is more than one head, and a token's heads fit inside stride_tok
// when there is more than one token.
bool strides_ok(int64_t st_tok, int64_t st_head, int heads, int head_dim, int64_t n_tokens)
{
    if (heads == 0) return true;
    if (heads > 1 && st_head < head_dim) return false;
    if (st_head < 0 || st_tok < 0) return false;
    const int64_t row_span = (int64_t)(heads - 1) * st_head + head_dim;
    if (n_tokens > 1 && st_tok < row_span) return false;
    return true;
}

}  // namespace

extern "C" {

const char *rope_status_str(int status)
{
    switch (status) {
    case ROPE_OK: return "ok";
    case ROPE_ERR_NULL: return "a required pointer is NULL";
    case ROPE_ERR_SHAPE: return "invalid shape, dimension, offset or stride";
    case ROPE_ERR_BASE: return "base (and position divisor) must be positive and finite";
    case ROPE_ERR_UNSUPPORTED: return "unsupported dtype / head_dim / rot_dim / layout combination";
    case ROPE_ERR_EMPTY_ROW: return "a query row sees no key (causal with q_pos_offset < k_pos_offset)";
    case ROPE_ERR_TABLE_RANGE: return "cos/sin table has too few rows for the positions used";
    case ROPE_ERR_HIP: return "HIP kernel launch failed";
    case ROPE_ERR_ALIGN: return "pointer or stride breaks the required alignment";
    case ROPE_ERR_SCRATCH: return "the call needs more scratch than the static decode array holds";
    default: return "unknown status";
    }
}

int rope_tables_build(double base, int rot_dim, int64_t max_pos, float *cos_out,
                      float *sin_out, void *stream)
{
    return rope_tables_build_scaled(base, rot_dim, max_pos, 1.0, cos_out, sin_out, stream);
}

int rope_tables_build_scaled(double base, int rot_dim, int64_t max_pos, double pos_divisor,
                             float *cos_out, float *sin_out, void *stream)
{
    if (!(base > 0.0) || !std::isfinite(base)) return ROPE_ERR_BASE;
    if (!(pos_divisor > 0.0) || !std::isfinite(pos_divisor)) return ROPE_ERR_BASE;
    if (rot_dim < 2 || rot_dim > 1024 || rot_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (max_pos < 1 || max_pos > 2147483647) return ROPE_ERR_SHAPE;
    if (!cos_out || !sin_out) return ROPE_ERR_NULL;
    if (!aligned(cos_out, 4) || !aligned(sin_out, 4)) return ROPE_ERR_ALIGN;
    if (overlaps(cos_out, bytes_of({max_pos, rot_dim / 2}, 4), sin_out, bytes_of({max_pos, rot_dim / 2}, 4)))
        return ROPE_ERR_SHAPE;
    return api_status(rope_launch_tables(base, rot_dim, max_pos, pos_divisor, cos_out, sin_out,
                                         static_cast<hipStream_t>(stream)));
}

int rope_apply(void *q, int64_t q_stride_tok, int64_t q_stride_head, int h_q,
               void *k, int64_t k_stride_tok, int64_t k_stride_head, int h_kv,
               const int32_t *positions, int64_t n_tokens,
               const float *cos_tab, const float *sin_tab, int64_t table_rows,
               int head_dim, int rot_dim, int layout, int dtype, void *stream)
{
    if (head_dim < 2 || head_dim > 1024 || head_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (rot_dim < 2 || rot_dim > head_dim || rot_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (n_tokens < 0 || n_tokens > 2147483647 || h_q < 0 || h_kv < 0 || h_q + h_kv > 65536)
        return ROPE_ERR_SHAPE;
    if (!valid_layout(layout) || !valid_apply_dtype(dtype)) return ROPE_ERR_UNSUPPORTED;
    if (!strides_ok(q_stride_tok, q_stride_head, h_q, head_dim, n_tokens) ||
        !strides_ok(k_stride_tok, k_stride_head, h_kv, head_dim, n_tokens))
        return ROPE_ERR_SHAPE;
    if (n_tokens == 0 || h_q + h_kv == 0) return ROPE_OK;
    if ((h_q > 0 && !q) || (h_kv > 0 && !k) || !positions || !cos_tab || !sin_tab)
        return ROPE_ERR_NULL;
    if (table_rows < 1) return ROPE_ERR_TABLE_RANGE;
    const unsigned es = (unsigned)elt_size(dtype);
    if ((h_q > 0 && !aligned(q, es)) || (h_kv > 0 && !aligned(k, es)) || !aligned(positions, 4) ||
        !aligned(cos_tab, 4) || !aligned(sin_tab, 4))
        return ROPE_ERR_ALIGN;

    RopeApplyArgs a;
    a.q = q; a.q_stride_tok = q_stride_tok; a.q_stride_head = q_stride_head; a.h_q = h_q;
    a.k = k; a.k_stride_tok = k_stride_tok; a.k_stride_head = k_stride_head; a.h_kv = h_kv;
    a.positions = positions; a.n_tokens = n_tokens;
    a.cos_tab = cos_tab; a.sin_tab = sin_tab; a.table_rows = table_rows;
    a.head_dim = head_dim; a.rot_dim = rot_dim; a.layout = layout; a.dtype = dtype;
    return api_status(rope_launch_apply(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Shape checks shared by the forward and its workspace query.
int check_fwd_shape(int B, int H, int64_t Sq, int64_t Sk, int head_dim, int64_t q_pos_offset,
                    int64_t k_pos_offset, int causal, int dtype)
{
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ROPE_ERR_SHAPE;
    if (Sq > 2147483647 || Sk > 2147483647) return ROPE_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (q_pos_offset < 0 || k_pos_offset < 0) return ROPE_ERR_SHAPE;
    if (!valid_dtype(dtype)) return ROPE_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return ROPE_ERR_UNSUPPORTED;
    const int64_t tiles = (Sq + 63) / 64;
    if ((int64_t)B * H > kMaxGrid || (int64_t)B * H * tiles > kMaxGrid) return ROPE_ERR_SHAPE;
    if (causal && q_pos_offset < k_pos_offset) return ROPE_ERR_EMPTY_ROW;
    return ROPE_OK;
}

}  // namespace

int64_t rope_flash_attn_workspace_size(int B, int H, int64_t Sq, int64_t Sk, int head_dim,
                                       int64_t q_pos_offset, int64_t k_pos_offset, int causal,
                                       int dtype)
{
    const int st = check_fwd_shape(B, H, Sq, Sk, head_dim, q_pos_offset, k_pos_offset, causal, dtype);
    if (st != ROPE_OK) return -st;
    if (dtype == ROPE_F32) return 0;
    FlashArgs a = {};
    // H_kv 0: enough for any key/value head count (the head grouping of the
    // split schedule depends on it)
    a.B = B; a.H = H; a.H_kv = 0; a.Sq = Sq; a.Sk = Sk; a.head_dim = head_dim;
    a.q_off = q_pos_offset; a.k_off = k_pos_offset; a.causal = causal ? 1 : 0; a.dtype = dtype;
    return rope_flash_bf16_workspace_bytes(a);
}

int rope_flash_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim,
                        int64_t q_pos_offset, int64_t k_pos_offset,
                        const float *cos_tab, const float *sin_tab, int64_t table_rows,
                        int rot_dim, int layout, int causal, float softmax_scale,
                        int dtype, void *workspace, int64_t workspace_bytes, void *stream)
{
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ROPE_ERR_SHAPE;
    if (H_kv < 1 || H % H_kv != 0) return ROPE_ERR_SHAPE;
    if (Sq > 2147483647 || Sk > 2147483647) return ROPE_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (rot_dim < 0 || rot_dim > head_dim || rot_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (q_pos_offset < 0 || k_pos_offset < 0) return ROPE_ERR_SHAPE;
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale)) return ROPE_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_layout(layout)) return ROPE_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return ROPE_ERR_UNSUPPORTED;
    if (rot_dim % 32 != 0) return ROPE_ERR_UNSUPPORTED;
    // grid size: one block per (batch*head, query tile); the fp32 kernel uses
    // 64-query tiles, the bf16 kernel 128.
    const int64_t tiles = (Sq + 63) / 64;
    if ((int64_t)B * H > kMaxGrid || (int64_t)B * H * tiles > kMaxGrid) return ROPE_ERR_SHAPE;
    if (!q || !k || !v || !o) return ROPE_ERR_NULL;
    if (rot_dim > 0 && (!cos_tab || !sin_tab)) return ROPE_ERR_NULL;
    {
        // o, lse and the workspace are written: none may overlap another or an input
        const int64_t es = elt_size(dtype);
        const int64_t nq = bytes_of({B, H, Sq, head_dim}, es), nk = bytes_of({B, H_kv, Sk, head_dim}, es);
        const int64_t nt = rot_dim > 0 ? bytes_of({table_rows, rot_dim / 2}, 4) : 0;
        if (any_overlap({{o, nq}, {lse, lse ? bytes_of({B, H, Sq}, 4) : 0}, {workspace, workspace_bytes}},
                        {{q, nq}, {k, nk}, {v, nk}, {cos_tab, nt}, {sin_tab, nt}}))
            return ROPE_ERR_SHAPE;
    }
    if (causal && q_pos_offset < k_pos_offset) return ROPE_ERR_EMPTY_ROW;
    if (rot_dim > 0) {
        const int64_t need_q = q_pos_offset + Sq, need_k = k_pos_offset + Sk;
        if (table_rows < need_q || table_rows < need_k) return ROPE_ERR_TABLE_RANGE;
        if (!aligned(cos_tab, 16) || !aligned(sin_tab, 16)) return ROPE_ERR_ALIGN;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return ROPE_ERR_ALIGN;
    if (lse && !aligned(lse, 4)) return ROPE_ERR_ALIGN;
    if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return ROPE_ERR_SHAPE;
    if (workspace && !aligned(workspace, 16)) return ROPE_ERR_ALIGN;

    FlashArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.B = B; a.H = H; a.H_kv = H_kv; a.Sq = Sq; a.Sk = Sk; a.head_dim = head_dim;
    a.q_off = q_pos_offset; a.k_off = k_pos_offset;
    a.cos_tab = cos_tab; a.sin_tab = sin_tab; a.table_rows = table_rows;
    a.rot_dim = rot_dim; a.layout = layout; a.causal = causal ? 1 : 0;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    a.dtype = dtype;
    a.lse = lse;
    a.workspace = workspace;
    a.workspace_bytes = workspace ? workspace_bytes : 0;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return api_status(dtype == ROPE_F32 ? rope_launch_flash_f32(a, s) : rope_launch_flash_bf16(a, s));
}

int64_t rope_flash_attn_bwd_workspace_size(int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim,
                                           int rot_dim, int dtype)
{
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0) return -ROPE_ERR_SHAPE;
    if (Sq < 1 || Sk < 1 || Sq > 2147483647 || Sk > 2147483647) return -ROPE_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0) return -ROPE_ERR_SHAPE;
    if (rot_dim < 0 || rot_dim > head_dim || rot_dim % 2 != 0) return -ROPE_ERR_SHAPE;
    if ((dtype != ROPE_BF16 && dtype != ROPE_F16) || (head_dim != 64 && head_dim != 128))
        return -ROPE_ERR_UNSUPPORTED;
    return rope_flash_bwd_workspace_bytes(B, H, H_kv, Sq, Sk, head_dim, rot_dim);
}

int rope_flash_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                        const float *lse, void *dq, void *dk, void *dv,
                        int B, int H, int H_kv, int64_t Sq, int64_t Sk, int head_dim,
                        int64_t q_pos_offset, int64_t k_pos_offset,
                        const float *cos_tab, const float *sin_tab, int64_t table_rows,
                        int rot_dim, int layout, int causal, float softmax_scale, int dtype,
                        void *workspace, int64_t workspace_bytes, void *stream)
{
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ROPE_ERR_SHAPE;
    if (H_kv < 1 || H % H_kv != 0) return ROPE_ERR_SHAPE;
    if (Sq > 2147483647 || Sk > 2147483647) return ROPE_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (rot_dim < 0 || rot_dim > head_dim || rot_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (q_pos_offset < 0 || k_pos_offset < 0) return ROPE_ERR_SHAPE;
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale)) return ROPE_ERR_SHAPE;
    if (!valid_layout(layout) || (dtype != ROPE_BF16 && dtype != ROPE_F16)) return ROPE_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return ROPE_ERR_UNSUPPORTED;
    if (rot_dim % 32 != 0) return ROPE_ERR_UNSUPPORTED;
    // grids of 128-row tiles; the key/value kernel walks (Sq / 32 + 1) * (H / H_kv) steps
    if ((int64_t)B * H * ((Sq + 127) / 128) > kMaxGrid || (int64_t)B * H_kv * ((Sk + 127) / 128) > kMaxGrid ||
        (Sq / 32 + 1) * (int64_t)(H / H_kv) > 2147483647)
        return ROPE_ERR_SHAPE;
    // the pre-pass: one block per 32-row tile of q and of k, then one per 16
    // (D = 128) or 32 rows of the row sums
    if (rot_dim > 0 && (int64_t)B * H * ((Sq + 31) / 32) + (int64_t)B * H_kv * ((Sk + 31) / 32) +
                               ((int64_t)B * H * Sq + 15) / 16 > kMaxGrid)
        return ROPE_ERR_SHAPE;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return ROPE_ERR_NULL;
    if (rot_dim > 0 && (!cos_tab || !sin_tab)) return ROPE_ERR_NULL;
    {
        // dq, dk, dv and the workspace are written: none may overlap another or an input
        const int64_t es = elt_size(dtype);
        const int64_t nq = bytes_of({B, H, Sq, head_dim}, es), nk = bytes_of({B, H_kv, Sk, head_dim}, es);
        const int64_t nt = rot_dim > 0 ? bytes_of({table_rows, rot_dim / 2}, 4) : 0;
        if (any_overlap({{dq, nq}, {dk, nk}, {dv, nk}, {workspace, workspace_bytes}},
                        {{q, nq}, {k, nk}, {v, nk}, {o, nq}, {dout, nq}, {lse, bytes_of({B, H, Sq}, 4)},
                         {cos_tab, nt}, {sin_tab, nt}}))
            return ROPE_ERR_SHAPE;
    }
    if (causal && q_pos_offset < k_pos_offset) return ROPE_ERR_EMPTY_ROW;
    if (rot_dim > 0) {
        if (table_rows < q_pos_offset + Sq || table_rows < k_pos_offset + Sk) return ROPE_ERR_TABLE_RANGE;
        if (!aligned(cos_tab, 16) || !aligned(sin_tab, 16)) return ROPE_ERR_ALIGN;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16) || !aligned(lse, 4))
        return ROPE_ERR_ALIGN;
    if (workspace_bytes < rope_flash_bwd_workspace_bytes(B, H, H_kv, Sq, Sk, head_dim, rot_dim))
        return ROPE_ERR_SHAPE;

    FlashBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.H = H; a.H_kv = H_kv; a.Sq = Sq; a.Sk = Sk; a.head_dim = head_dim;
    a.q_off = q_pos_offset; a.k_off = k_pos_offset;
    a.cos_tab = cos_tab; a.sin_tab = sin_tab;
    a.rot_dim = rot_dim; a.layout = layout; a.causal = causal ? 1 : 0;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    a.dtype = dtype;
    a.workspace = workspace;
    return api_status(rope_launch_flash_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

namespace {

int decode_checked(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                   const int32_t *cache_lens, void *o, int B, int H, int H_kv, int64_t S_max, int head_dim,
                   const float *cos_tab, const float *sin_tab, int64_t table_rows, int rot_dim, int layout,
                   float softmax_scale, int dtype, void *workspace, int64_t workspace_bytes, void *stream);

int check_decode_shape(int B, int H, int H_kv, int64_t S_max, int head_dim)
{
    if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || S_max < 1) return ROPE_ERR_SHAPE;
    if (S_max > 2147483647) return ROPE_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return ROPE_ERR_UNSUPPORTED;
    if (H / H_kv > 8) return ROPE_ERR_UNSUPPORTED;
    // pass counts are 32-bit on the device; one merge workgroup per (request, head)
    if (rope_decode_max_passes(B, H_kv, S_max) > 2147483647 || (int64_t)B * H > kMaxGrid)
        return ROPE_ERR_SHAPE;
    return ROPE_OK;
}

}  // namespace

int64_t rope_decode_workspace_size(int B, int H, int H_kv, int64_t S_max, int head_dim)
{
    const int st = check_decode_shape(B, H, H_kv, S_max, head_dim);
    if (st != ROPE_OK) return -st;
    return rope_decode_workspace_bytes(B, H, H_kv, head_dim);
}

int rope_decode_attn_fwd(const void *q, const void *k_new, const void *v_new,
                         void *k_cache, void *v_cache, const int32_t *cache_lens, void *o,
                         int B, int H, int H_kv, int64_t S_max, int head_dim,
                         const float *cos_tab, const float *sin_tab, int64_t table_rows,
                         int rot_dim, int layout, float softmax_scale, int dtype,
                         void *workspace, int64_t workspace_bytes, void *stream)
{
    const int st = check_decode_shape(B, H, H_kv, S_max, head_dim);
    if (st != ROPE_OK) return st;
    if (!workspace) return ROPE_ERR_NULL;
    return decode_checked(q, k_new, v_new, k_cache, v_cache, cache_lens, o, B, H, H_kv, S_max, head_dim, cos_tab,
                          sin_tab, table_rows, rot_dim, layout, softmax_scale, dtype, workspace, workspace_bytes,
                          stream);
}

int rope_decode_attn_fwd_noalloc(const void *q, const void *k_new, const void *v_new,
                                 void *k_cache, void *v_cache, const int32_t *cache_lens, void *o,
                                 int B, int H, int H_kv, int64_t S_max, int head_dim,
                                 const float *cos_tab, const float *sin_tab, int64_t table_rows,
                                 int rot_dim, int layout, float softmax_scale, int dtype, void *stream)
{
    const int st = check_decode_shape(B, H, H_kv, S_max, head_dim);
    if (st != ROPE_OK) return st;
    // before any HIP call: the static array must hold what the shapes need
    if (rope_decode_workspace_bytes(B, H, H_kv, head_dim) > (int64_t)ROPE_DECODE_SCRATCH_BYTES)
        return ROPE_ERR_SCRATCH;
    // workspace nullptr: decode_checked looks up the current device's copy
    // of the static array after every host-side check has passed
    return decode_checked(q, k_new, v_new, k_cache, v_cache, cache_lens, o, B, H, H_kv, S_max, head_dim, cos_tab,
                          sin_tab, table_rows, rot_dim, layout, softmax_scale, dtype, nullptr,
                          (int64_t)ROPE_DECODE_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {

// rope_decode_attn_fwd after the shape check: arguments, overlap and
// alignment checks, then the launch on `workspace`, or (workspace nullptr)
// on the static decode scratch, whose address is looked up only after the
// host-side checks
int decode_checked(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                   const int32_t *cache_lens, void *o, int B, int H, int H_kv, int64_t S_max, int head_dim,
                   const float *cos_tab, const float *sin_tab, int64_t table_rows, int rot_dim, int layout,
                   float softmax_scale, int dtype, void *workspace, int64_t workspace_bytes, void *stream)
{
    if (rot_dim < 0 || rot_dim > head_dim || rot_dim % 2 != 0) return ROPE_ERR_SHAPE;
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale)) return ROPE_ERR_SHAPE;
    if (!valid_layout(layout)) return ROPE_ERR_UNSUPPORTED;
    if (dtype != ROPE_BF16 && dtype != ROPE_F16) return ROPE_ERR_UNSUPPORTED;
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_lens || !o) return ROPE_ERR_NULL;
    if (rot_dim > 0 && (!cos_tab || !sin_tab)) return ROPE_ERR_NULL;
    if (rot_dim > 0 && table_rows < 1) return ROPE_ERR_TABLE_RANGE;
    if (workspace_bytes < rope_decode_workspace_bytes(B, H, H_kv, head_dim)) return ROPE_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(o, 16) || !aligned(cache_lens, 4))
        return ROPE_ERR_ALIGN;
    if (rot_dim > 0 && (!aligned(cos_tab, 4) || !aligned(sin_tab, 4))) return ROPE_ERR_ALIGN;
    if (workspace == nullptr) {
        workspace = rope_decode_static_scratch();
        if (workspace == nullptr) return ROPE_ERR_HIP;
    }
    if (!aligned(workspace, 16)) return ROPE_ERR_ALIGN;
    {
        // o, the caches (rows L are written) and the workspace: none may
        // overlap another or an input
        const int64_t es = elt_size(dtype);
        const int64_t nq = bytes_of({B, H, head_dim}, es), nn = bytes_of({B, H_kv, head_dim}, es);
        const int64_t nc = bytes_of({B, H_kv, S_max, head_dim}, es);
        const int64_t nt = rot_dim > 0 ? bytes_of({table_rows, rot_dim / 2}, 4) : 0;
        if (any_overlap({{o, nq}, {k_cache, nc}, {v_cache, nc}, {workspace, workspace_bytes}},
                        {{q, nq}, {k_new, nn}, {v_new, nn}, {cache_lens, bytes_of({B}, 4)}, {cos_tab, nt},
                         {sin_tab, nt}}))
            return ROPE_ERR_SHAPE;
    }

    DecodeArgs a;
    a.q = q; a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
    a.cache_lens = cache_lens; a.o = o;
    a.B = B; a.H = H; a.H_kv = H_kv; a.S_max = S_max; a.head_dim = head_dim;
    a.cos_tab = cos_tab; a.sin_tab = sin_tab; a.table_rows = rot_dim > 0 ? table_rows : 0;
    a.rot_dim = rot_dim; a.layout = layout;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    a.dtype = dtype;
    a.workspace = workspace;
    return api_status(rope_launch_decode_bf16(a, static_cast<hipStream_t>(stream)));
}

}  // namespace
