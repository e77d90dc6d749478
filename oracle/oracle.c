/*
 * oracle.c -- plain, slow, obviously-correct fp64 CPU reference for rotary
 * position embedding (RoPE) and for softmax attention over rotated queries
 * and keys.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load or call this file.  It shares no
 * code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * Sources (cited by page title and section):
 *   [RF] "RoPE and FlashAttention: relative positions and online softmax"
 *        section 1 (RoPE from a relative-position requirement: pair rotation,
 *        frequency schedule, Q and K rotated but never V), section 2
 *        (offset-aware RoPE: absolute positions, fp64 angle construction),
 *        section 4 (naive attention S = QK^T/sqrt(d), P = softmax(S), O = PV),
 *        section 5 (masked rows; a row with no valid key is rejected).
 *   [TR] "Write Triton Rope Kernel", sections "Inputs the agent should gather
 *        first" (GPT-NeoX half-split vs GPT-J adjacent-pair layout, partial
 *        RoPE on the first rot_dim dims, per-token positions) and
 *        "Required reasoning process" steps 1, 6 and 8 (the rotation formulas
 *        and their sign convention).
 *
 * Readings where the pages are silent or disagree (each stated once here):
 *   - Frequency denominator under partial RoPE is rot_dim, not head_dim:
 *     theta_i = base^(-2 i / rot_dim), i in [0, rot_dim/2).
 *   - Half-split partial RoPE pairs (i, i + rot_dim/2) for i < rot_dim/2; the
 *     dims [rot_dim, head_dim) are copied unchanged.
 *   - Angles and trig are carried in fp64 here; no rounding to the input type.
 *   - Softmax scale defaults to 1/sqrt(head_dim) (head_dim, not rot_dim).
 *   - Offset mask: query i sits at q_off + i, key j at k_off + j; with causal
 *     set, key j is visible to query i iff k_off + j <= q_off + i.
 *   - Position interpolation ([RF] section 3: positions divided by an
 *     extension factor) rotates a row at position p by the angle
 *     (p / pos_div) theta_i; the mask still compares the integer positions.
 *     pos_div = 1 is plain RoPE.
 *
 * Build: gcc -O2 -std=c99 -fopenmp -ffp-contract=off -shared -fPIC -lm
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_NEOX = 0, OR_GPTJ = 1 };
enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_EMPTY_ROW = 2, OR_ERR_NOMEM = 3 };

/* Threads an OpenMP region of the oracle uses (reported with its timings). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* Threads later parallel regions use (n >= 1); for single-thread timings. */
void oracle_set_threads(int n) { if (n >= 1) omp_set_num_threads(n); }

/* theta_i = base^(-2i/rot_dim): one frequency per rotated pair; the first
 * frequency is 1 for every base.  [RF] section 1; [TR] "Correctness
 * requirements" (table build). */
static double pair_frequency(double base, int i, int rot_dim)
{
    return pow(base, -2.0 * (double)i / (double)rot_dim);
}

/* The two coordinates that form pair i.  GPT-J rotates adjacent pairs
 * (2i, 2i+1); GPT-NeoX rotates the halves (i, i + rot_dim/2).  [TR] "Inputs
 * the agent should gather first", item 1; [RF] section 1. */
static void pair_slots(int layout, int i, int rot_dim, int *a, int *b)
{
    if (layout == OR_GPTJ) {
        *a = 2 * i;
        *b = 2 * i + 1;
    } else {
        *a = i;
        *b = i + rot_dim / 2;
    }
}

/* Rotate one row of head_dim values sitting at absolute position pos.
 * Each pair (xa, xb) becomes (xa cos - xb sin, xa sin + xb cos) with angle
 * pos * theta_i.  Dims at or past rot_dim pass through.  [TR] "Required
 * reasoning process" steps 1 and 6; [RF] section 1. */
static void rotate_row(const double *x, double *y, int head_dim, int rot_dim,
                       double pos, double base, int layout)
{
    for (int d = rot_dim; d < head_dim; ++d)
        y[d] = x[d];
    for (int i = 0; i < rot_dim / 2; ++i) {
        double ang = pos * pair_frequency(base, i, rot_dim);
        double c = cos(ang), s = sin(ang);
        int a, b;
        pair_slots(layout, i, rot_dim, &a, &b);
        double xa = x[a], xb = x[b];
        y[a] = xa * c - xb * s;
        y[b] = xa * s + xb * c;
    }
}

static int rope_args_ok(int head_dim, int rot_dim, double base, int layout)
{
    if (head_dim <= 0 || head_dim % 2 != 0) return 0;
    if (rot_dim < 0 || rot_dim % 2 != 0 || rot_dim > head_dim) return 0;
    if (!(base > 0.0)) return 0;
    if (layout != OR_NEOX && layout != OR_GPTJ) return 0;
    return 1;
}

/* Rotate n_rows rows of x ([n_rows, head_dim], contiguous) at the given
 * per-row positions.  rot_dim == 0 copies.  Per-token positions come from the
 * caller, never from the row index: [TR] "Required reasoning process" step 3. */
int oracle_rope(const double *x, double *y, int64_t n_rows, int head_dim,
                int rot_dim, const double *positions, double base, int layout)
{
    if (!rope_args_ok(head_dim, rot_dim, base, layout) || n_rows < 0) return OR_ERR_ARG;
    if (n_rows > 0 && (!x || !y || !positions)) return OR_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r)
        rotate_row(x + r * head_dim, y + r * head_dim, head_dim, rot_dim,
                   positions[r], base, layout);
    return OR_OK;
}

/* The exact trig a cos/sin table approximates: cos_out[p][i] = cos(a),
 * sin_out[p][i] = sin(a) with a = (p / pos_div) theta_i, rows of rot_dim/2
 * values.  [RF] section 2 (angles formed in fp64), section 3 (position
 * interpolation divides the position); [TR] "Correctness requirements"
 * (table build). */
int oracle_trig(double base, int rot_dim, int64_t n_pos, double pos_div, double *cos_out,
                double *sin_out)
{
    if (rot_dim <= 0 || rot_dim % 2 != 0 || !(base > 0.0) || n_pos < 0) return OR_ERR_ARG;
    if (!(pos_div > 0.0) || !isfinite(pos_div)) return OR_ERR_ARG;
    if (n_pos > 0 && (!cos_out || !sin_out)) return OR_ERR_ARG;
    const int half = rot_dim / 2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < n_pos; ++p)
        for (int i = 0; i < half; ++i) {
            double ang = ((double)p / pos_div) * pair_frequency(base, i, rot_dim);
            cos_out[p * half + i] = cos(ang);
            sin_out[p * half + i] = sin(ang);
        }
    return OR_OK;
}

/* Number of keys query i may attend to.  Keys sit at contiguous positions, so
 * the visible set is a prefix [0, n) of the key rows. */
static int64_t visible_keys(int64_t i, int64_t Sk, int64_t q_off, int64_t k_off, int causal)
{
    if (!causal) return Sk;
    int64_t last = q_off + i - k_off;    /* largest visible key index */
    if (last < 0) return 0;
    return last + 1 < Sk ? last + 1 : Sk;
}

/* One output row of naive attention over n visible keys:
 * s_j = scale * (qr . kr_j), p = softmax(s), out = sum_j p_j v_j.
 * [RF] section 4 (S = QK^T/sqrt(d), P = softmax(S), O = PV). */
static void attend_row(const double *qr, const double *kr, const double *v,
                       int64_t n, int D, int Dv, double scale, double *scores,
                       double *out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += qr[d] * kr[j * D + d];
        s *= scale;
        scores[j] = s;
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }
    for (int e = 0; e < Dv; ++e) out[e] = 0.0;
    for (int64_t j = 0; j < n; ++j)
        for (int e = 0; e < Dv; ++e) out[e] += scores[j] * v[j * Dv + e];
    for (int e = 0; e < Dv; ++e) out[e] /= l;
}

static int attn_args_ok(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int D, int Dv,
                        int rot_dim, double base, int layout)
{
    if (B <= 0 || H <= 0 || Sq <= 0 || Sk <= 0 || Dv <= 0) return 0;
    if (Hkv <= 0 || H % Hkv != 0) return 0;
    if (rot_dim == 0) return D > 0 && D % 2 == 0;
    return rope_args_ok(D, rot_dim, base, layout);
}

/* Full attention forward.  q [B,H,Sq,D], k [B,Hkv,Sk,D], v [B,Hkv,Sk,Dv],
 * o [B,H,Sq,Dv], all contiguous fp64.  Query head h of batch b attends to key
 * and value head h / (H / Hkv) of batch b (Hkv divides H; Hkv == H is plain
 * multi-head attention, fewer key heads are shared by consecutive query
 * heads: [TR] "Inputs the agent should gather first", item 3, and "Required
 * reasoning process", step 10, for the two head counts).  Query i has
 * position q_off + i and key j position k_off + j; Q and K are rotated at
 * those positions (rot_dim == 0: no rotation), V is never rotated ([RF]
 * section 1); with position interpolation the rotation angles use the
 * positions divided by pos_div ([RF] section 3).  scale <= 0 selects
 * 1/sqrt(D).  A query with no visible key is rejected ([RF] section 5). */
int oracle_attention(const double *q, const double *k, const double *v, double *o,
                     int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int D, int Dv,
                     int64_t q_off, int64_t k_off, int rot_dim, double base, double pos_div,
                     int layout, int causal, double scale)
{
    if (!attn_args_ok(B, H, Hkv, Sq, Sk, D, Dv, rot_dim, base, layout)) return OR_ERR_ARG;
    if (!(pos_div > 0.0) || !isfinite(pos_div)) return OR_ERR_ARG;
    if (!q || !k || !v || !o) return OR_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int64_t i = 0; i < Sq; ++i)
        if (visible_keys(i, Sk, q_off, k_off, causal) == 0) return OR_ERR_EMPTY_ROW;

    const int64_t nq = B * H * Sq, nk = B * Hkv * Sk, group = H / Hkv;
    double *qr = malloc(sizeof(double) * (size_t)(nq * D));
    double *kr = malloc(sizeof(double) * (size_t)(nk * D));
    if (!qr || !kr) { free(qr); free(kr); return OR_ERR_NOMEM; }

    /* Rotate every Q and K row once, at its absolute position. */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nq; ++r)
        rotate_row(q + r * D, qr + r * D, D, rot_dim, (double)(q_off + r % Sq) / pos_div, base,
                   layout);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nk; ++r)
        rotate_row(k + r * D, kr + r * D, D, rot_dim, (double)(k_off + r % Sk) / pos_div, base,
                   layout);

    int status = OR_OK;
#pragma omp parallel
    {
        double *scores = malloc(sizeof(double) * (size_t)Sk);
        if (!scores) {
#pragma omp atomic write
            status = OR_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nq; ++r) {
                int64_t bh = r / Sq, i = r % Sq;
                int64_t kvh = bh / group;   /* (b * H + h) / group = b * Hkv + h / group */
                int64_t n = visible_keys(i, Sk, q_off, k_off, causal);
                attend_row(qr + r * D, kr + kvh * Sk * D, v + kvh * Sk * Dv, n, D, Dv,
                           scale, scores, o + r * Dv);
            }
            free(scores);
        }
    }
    free(qr);
    free(kr);
    return status;
}

/* Selected rows of the same forward, for spot checks at sizes the full
 * oracle cannot finish quickly.  rows holds n_rows (b, h, i) triples; row r of
 * o_rows ([n_rows, Dv]) receives output row (b, h, i).  Each selected row
 * rotates its own query and visible keys. */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int D, int Dv,
                          int64_t q_off, int64_t k_off, int rot_dim, double base, double pos_div,
                          int layout, int causal, double scale,
                          const int64_t *rows, int64_t n_rows, double *o_rows)
{
    if (!attn_args_ok(B, H, Hkv, Sq, Sk, D, Dv, rot_dim, base, layout)) return OR_ERR_ARG;
    if (!(pos_div > 0.0) || !isfinite(pos_div)) return OR_ERR_ARG;
    if (!q || !k || !v || (n_rows > 0 && (!rows || !o_rows)) || n_rows < 0) return OR_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Sq) return OR_ERR_ARG;
        if (visible_keys(i, Sk, q_off, k_off, causal) == 0) return OR_ERR_EMPTY_ROW;
    }
    int status = OR_OK;
#pragma omp parallel
    {
        double *qr = malloc(sizeof(double) * (size_t)D);
        double *kr = malloc(sizeof(double) * (size_t)(Sk * D));
        double *scores = malloc(sizeof(double) * (size_t)Sk);
        if (!qr || !kr || !scores) {
#pragma omp atomic write
            status = OR_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
                int64_t bh = b * H + h, kvh = b * Hkv + h / (H / Hkv);
                int64_t n = visible_keys(i, Sk, q_off, k_off, causal);
                rotate_row(q + (bh * Sq + i) * D, qr, D, rot_dim, (double)(q_off + i) / pos_div, base,
                           layout);
                for (int64_t j = 0; j < n; ++j)
                    rotate_row(k + (kvh * Sk + j) * D, kr + j * D, D, rot_dim,
                               (double)(k_off + j) / pos_div, base, layout);
                attend_row(qr, kr, v + kvh * Sk * Dv, n, D, Dv, scale, scores, o_rows + r * Dv);
            }
        }
        free(qr);
        free(kr);
        free(scores);
    }
    return status;
}

/* Row-wise log-sum-exp of the same forward's scores, natural log:
 * lse[b, h, i] = log sum_j exp(s_ij) over the visible keys, the quantity a
 * blocked forward keeps (running max plus log of the running sum) so that a
 * backward pass can recompute p_ij = exp(s_ij - lse_i) ([RF] section 5: the
 * (m, l) state; its last row of questions: backward recomputes P from saved
 * row statistics). */
int oracle_attention_lse(const double *q, const double *k, double *lse,
                         int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int D,
                         int64_t q_off, int64_t k_off, int rot_dim, double base, double pos_div,
                         int layout, int causal, double scale)
{
    if (!attn_args_ok(B, H, Hkv, Sq, Sk, D, 1, rot_dim, base, layout)) return OR_ERR_ARG;
    if (!(pos_div > 0.0) || !isfinite(pos_div)) return OR_ERR_ARG;
    if (!q || !k || !lse) return OR_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int64_t i = 0; i < Sq; ++i)
        if (visible_keys(i, Sk, q_off, k_off, causal) == 0) return OR_ERR_EMPTY_ROW;
    const int64_t nq = B * H * Sq, nk = B * Hkv * Sk, group = H / Hkv;
    /* Rotate every K row once, at its absolute position. */
    double *kr = malloc(sizeof(double) * (size_t)(nk * D));
    if (!kr) return OR_ERR_NOMEM;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nk; ++r)
        rotate_row(k + r * D, kr + r * D, D, rot_dim, (double)(k_off + r % Sk) / pos_div, base,
                   layout);
    int status = OR_OK;
#pragma omp parallel
    {
        double *qr = malloc(sizeof(double) * (size_t)D);
        if (!qr) {
#pragma omp atomic write
            status = OR_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nq; ++r) {
                int64_t bh = r / Sq, i = r % Sq, kvh = bh / group;
                int64_t n = visible_keys(i, Sk, q_off, k_off, causal);
                const double *krh = kr + kvh * Sk * D;
                rotate_row(q + r * D, qr, D, rot_dim, (double)(q_off + i) / pos_div, base, layout);
                double m = -INFINITY;
                for (int64_t j = 0; j < n; ++j) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += qr[d] * krh[j * D + d];
                    s *= scale;
                    if (s > m) m = s;
                }
                double l = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += qr[d] * krh[j * D + d];
                    l += exp(s * scale - m);
                }
                lse[r] = m + log(l);
            }
        }
        free(qr);
    }
    free(kr);
    return status;
}

/* Gradients of the same forward, o = attention(q, k, v), for an upstream
 * gradient dout [B, H, Sq, Dv], by the chain rule through each step of the
 * forward ([RF] section 5's last questions: the backward recomputes the
 * probabilities and needs, per query row, the sum of p times its upstream
 * score gradient):
 *   qr_i = R(q_pos_i) q_i, kr_j = R(k_pos_j) k_j    (rotation; V unrotated)
 *   s_ij = scale qr_i . kr_j,  p_ij = softmax over the visible j
 *   dv_j   = sum_i p_ij dout_i
 *   dp_ij  = dout_i . v_j
 *   ds_ij  = p_ij (dp_ij - sum_j' p_ij' dp_ij')
 *   dqr_i  = scale sum_j ds_ij kr_j,   dq_i = R(q_pos_i)^T dqr_i
 *   dkr_j  = scale sum_i ds_ij qr_i,   dk_j = R(k_pos_j)^T dkr_j
 * R(pos)^T is the rotation by the opposite angle.  A key/value head's dk and
 * dv sum over every query head that reads it and every query row.
 *
 * Two passes, so that each thread owns the rows it writes:
 *   1. per query row i: its softmax statistics (max m_i, sum l_i), the row
 *      correction c_i = sum_j p_ij dp_ij, and dq_i;
 *   2. per key row j of a key/value head: dk_j and dv_j, summing over the
 *      query rows of every query head that reads it, with p_ij rebuilt as
 *      exp(s_ij - m_i) / l_i from the same scores and statistics. */
int oracle_attention_bwd(const double *q, const double *k, const double *v, const double *dout,
                         double *dq, double *dk, double *dv,
                         int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int D, int Dv,
                         int64_t q_off, int64_t k_off, int rot_dim, double base, double pos_div,
                         int layout, int causal, double scale)
{
    if (!attn_args_ok(B, H, Hkv, Sq, Sk, D, Dv, rot_dim, base, layout)) return OR_ERR_ARG;
    if (!(pos_div > 0.0) || !isfinite(pos_div)) return OR_ERR_ARG;
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return OR_ERR_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int64_t i = 0; i < Sq; ++i)
        if (visible_keys(i, Sk, q_off, k_off, causal) == 0) return OR_ERR_EMPTY_ROW;

    const int64_t nq = B * H * Sq, nk = B * Hkv * Sk, group = H / Hkv;
    double *qr = malloc(sizeof(double) * (size_t)(nq * D));
    double *kr = malloc(sizeof(double) * (size_t)(nk * D));
    double *row_m = malloc(sizeof(double) * (size_t)nq);
    double *row_l = malloc(sizeof(double) * (size_t)nq);
    double *row_c = malloc(sizeof(double) * (size_t)nq);
    if (!qr || !kr || !row_m || !row_l || !row_c) {
        free(qr); free(kr); free(row_m); free(row_l); free(row_c);
        return OR_ERR_NOMEM;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nq; ++r)
        rotate_row(q + r * D, qr + r * D, D, rot_dim, (double)(q_off + r % Sq) / pos_div, base,
                   layout);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nk; ++r)
        rotate_row(k + r * D, kr + r * D, D, rot_dim, (double)(k_off + r % Sk) / pos_div, base,
                   layout);

    int status = OR_OK;
    /* Pass 1: per query row, its statistics, its correction and dq. */
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * (size_t)Sk);
        double *dp = malloc(sizeof(double) * (size_t)Sk);
        double *dqr = malloc(sizeof(double) * (size_t)D);
        if (!p || !dp || !dqr) {
#pragma omp atomic write
            status = OR_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nq; ++r) {
                const int64_t bh = r / Sq, i = r % Sq;
                const int64_t kvh = bh / group;   /* (b * H + h) / group = b * Hkv + h / group */
                const double *krh = kr + kvh * Sk * D, *vh = v + kvh * Sk * Dv;
                const double *qri = qr + r * D, *doi = dout + r * Dv;
                const int64_t n = visible_keys(i, Sk, q_off, k_off, causal);
                double m = -INFINITY;
                for (int64_t j = 0; j < n; ++j) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += qri[d] * krh[j * D + d];
                    p[j] = s * scale;
                    if (p[j] > m) m = p[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    p[j] = exp(p[j] - m);
                    l += p[j];
                }
                double pdp = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    p[j] /= l;
                    double t = 0.0;
                    for (int e = 0; e < Dv; ++e) t += doi[e] * vh[j * Dv + e];
                    dp[j] = t;
                    pdp += p[j] * t;
                }
                for (int d = 0; d < D; ++d) dqr[d] = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    const double ds = p[j] * (dp[j] - pdp);
                    for (int d = 0; d < D; ++d) dqr[d] += scale * ds * krh[j * D + d];
                }
                rotate_row(dqr, dq + r * D, D, rot_dim, -(double)(q_off + i) / pos_div, base,
                           layout);
                row_m[r] = m;
                row_l[r] = l;
                row_c[r] = pdp;
            }
        }
        free(p);
        free(dp);
        free(dqr);
    }
    /* Pass 2: per key row, dk and dv over every query row that sees it. */
    if (status == OR_OK) {
#pragma omp parallel
        {
            double *dkr = malloc(sizeof(double) * (size_t)D);
            if (!dkr) {
#pragma omp atomic write
                status = OR_ERR_NOMEM;
            } else {
#pragma omp for schedule(dynamic, 16)
                for (int64_t kr_row = 0; kr_row < nk; ++kr_row) {
                    const int64_t kvh = kr_row / Sk, j = kr_row % Sk, b = kvh / Hkv;
                    const double *krj = kr + kr_row * D, *vj = v + kr_row * Dv;
                    double *dvj = dv + kr_row * Dv;
                    for (int d = 0; d < D; ++d) dkr[d] = 0.0;
                    for (int e = 0; e < Dv; ++e) dvj[e] = 0.0;
                    for (int64_t g = 0; g < group; ++g) {
                        const int64_t bh = b * H + (kvh % Hkv) * group + g;
                        for (int64_t i = 0; i < Sq; ++i) {
                            if (j >= visible_keys(i, Sk, q_off, k_off, causal)) continue;
                            const int64_t r = bh * Sq + i;
                            const double *qri = qr + r * D, *doi = dout + r * Dv;
                            double s = 0.0;
                            for (int d = 0; d < D; ++d) s += qri[d] * krj[d];
                            const double pij = exp(s * scale - row_m[r]) / row_l[r];
                            double dpij = 0.0;
                            for (int e = 0; e < Dv; ++e) dpij += doi[e] * vj[e];
                            const double ds = pij * (dpij - row_c[r]);
                            for (int d = 0; d < D; ++d) dkr[d] += scale * ds * qri[d];
                            for (int e = 0; e < Dv; ++e) dvj[e] += pij * doi[e];
                        }
                    }
                    rotate_row(dkr, dk + kr_row * D, D, rot_dim, -(double)(k_off + j) / pos_div, base,
                               layout);
                }
            }
            free(dkr);
        }
    }
    free(qr);
    free(kr);
    free(row_m);
    free(row_l);
    free(row_c);
    return status;
}
