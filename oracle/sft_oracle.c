/*
 * sft_oracle.c -- plain, slow CPU oracle of the sparse-first fine-tuning step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists so that the GPU library can be
 * checked against an independent, obviously-correct statement of what the
 * step computes.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header, table or helper
 * with the HIP library, and the HIP library never calls it.
 *
 * Source of the method: the page "Sparse-First Fine-Tuning: Full-Weight
 * Training at the Cost of the Active Set" (tensorwirelabs.com), sections 2.1
 * (observing activity), 2.2 (masked backward pass), 2.3 (sparse state and int8
 * weights) and 2.4 (the coupled update).  Adam is the textbook step with bias
 * correction, as that page's section 2.4 names it and as the SparseLeaf blog
 * post (di-zhang-llm.github.io, section 4 "SparseLeaf Adam") restates it after
 * Kingma and Ba.  Where the pages lost an equation the reading taken is stated
 * at the function that depends on it.
 *
 * Arithmetic rules, chosen so that a careful GPU implementation can match the
 * integer and quantised results bit for bit:
 *   - IEEE-754 binary32, round-to-nearest-even, no fused multiply-add (built
 *     with -ffp-contract=off), no fast-math, denormals kept;
 *   - every fp32->fp16 and fp32->bf16 conversion is written out below from the
 *     IEEE definition (round to nearest, ties to even, subnormals kept);
 *   - the weight-gradient sums (a plain dot product over tokens) are taken in
 *     fp64 and rounded to fp32 once.
 *
 * The element-sparse variant of the SparseLeaf blog post (gradients of K
 * selected connections and their coordinate Adam step) is stated at the end.
 *
 * Parity pins: every exported function is checked in tests/test_oracle_pins.py
 * against closed forms, library routines or brute force.  The coupled mixing
 * schedule (the lost equations of section 2.4) is not part of this file: the
 * mix coefficients are inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Number formats, from the IEEE-754 definitions.                            */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of a binary32: widening is exact. */
ORACLE_API float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
ORACLE_API float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int frac = h & 1023;
    double mag;
    if (e == 0)
        mag = ldexp((double)frac, -24);                  /* subnormal: frac * 2^-24 */
    else if (e == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), e - 25);      /* (1.frac) * 2^(e-15) */
    return (float)(sign ? -mag : mag);
}

/*
 * Round |x| to an integer number of units of 2^lsb_exp, ties to even.  The
 * scaling by a power of two is exact in double for every binary32 input and
 * nearbyint() rounds to nearest-even in the default rounding mode.
 */
static double round_to_units(double ax, int lsb_exp)
{
    return nearbyint(ldexp(ax, -lsb_exp));
}

/* fp32 -> binary16, round to nearest even, subnormals kept, overflow to inf. */
ORACLE_API uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs((double)x);
    if (isnan(x))
        return sign | 0x7e00;
    if (isinf(x))
        return sign | 0x7c00;
    if (ax < ldexp(1.0, -14)) {
        /* subnormal range: the unit is 2^-24; 1024 units is the smallest normal */
        double n = round_to_units(ax, -24);
        return sign | (uint16_t)n;
    }
    int e;
    frexp(ax, &e);                 /* ax = f * 2^e with f in [0.5, 1) */
    int exp2 = e - 1;              /* ax in [2^exp2, 2^(exp2+1)) */
    double n = round_to_units(ax, exp2 - 10);   /* 11 significant bits */
    if (n >= 2048.0) {             /* rounded up into the next binade */
        n = 1024.0;
        exp2 += 1;
    }
    if (exp2 + 15 >= 31)
        return sign | 0x7c00;      /* overflow */
    return sign | (uint16_t)(((exp2 + 15) << 10) | ((int)n - 1024));
}

/* fp32 -> bf16 (8 significant bits, binary32 exponent range), RNE. */
ORACLE_API uint16_t oracle_f32_to_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs((double)x);
    if (isnan(x))
        return sign | 0x7fc0;
    if (isinf(x))
        return sign | 0x7f80;
    if (ax < ldexp(1.0, -126)) {
        double n = round_to_units(ax, -133);           /* unit 2^-133 */
        return sign | (uint16_t)n;                     /* 128 units = smallest normal */
    }
    int e;
    frexp(ax, &e);
    int exp2 = e - 1;
    double n = round_to_units(ax, exp2 - 7);
    if (n >= 256.0) {
        n = 128.0;
        exp2 += 1;
    }
    if (exp2 + 127 >= 255)
        return sign | 0x7f80;
    return sign | (uint16_t)(((exp2 + 127) << 7) | ((int)n - 128));
}

/*
 * Scaled fp16 storage of a row of Adam moments (section 2.3 keeps m and v in
 * fp16).  Plain fp16 loses small moments: (1 - beta2) g^2 falls below the
 * smallest fp16 subnormal (2^-24) once |g| is under about 5e-3 and large ones
 * overflow (v above 65504 once |g| passes about 256).  Reading: each slot
 * stores its row of m (and of v) as fp16 values of m * 2^e with one exponent
 * e per row and moment, e chosen at every update so that the row's largest
 * magnitude lands in [2^14, 2^15): the row keeps fp16's 11 significant bits
 * across any range of gradients.  e = 15 - k for the row maximum in
 * [2^(k-1), 2^k), limited to [-112, 125] so that both 2^e and 2^-e are
 * normal binary32 numbers; an all-zero row takes e = 0.  Scaling by a power
 * of two is exact in double; the fp16 rounding is to nearest even and
 * saturates at the largest finite value (65504) instead of overflowing.
 */
#define MOMENT_EXP_MIN (-112)
#define MOMENT_EXP_MAX 125

ORACLE_API int oracle_moment_exponent(float amax)
{
    if (!(amax > 0.0f))
        return 0;
    int k;
    frexp((double)amax, &k);       /* amax in [2^(k-1), 2^k) */
    int e = 15 - k;
    if (e < MOMENT_EXP_MIN)
        e = MOMENT_EXP_MIN;
    if (e > MOMENT_EXP_MAX)
        e = MOMENT_EXP_MAX;
    return e;
}

/* fp16 bits of x * 2^e (round to nearest even, saturating at +-65504). */
ORACLE_API uint16_t oracle_moment_encode(float x, int e)
{
    double y = ldexp((double)x, e);
    uint16_t h;
    if (y >= 65504.0)
        h = 0x7bff;
    else if (y <= -65504.0)
        h = 0xfbff;
    else
        h = oracle_f32_to_f16((float)y);   /* y is a binary32 value or rounds to f16 zero below 2^-126 */
    return h;
}

/* The stored moment: fp16 value times 2^-e (exact in binary32 for e in range). */
ORACLE_API float oracle_moment_decode(uint16_t h, int e)
{
    return (float)ldexp((double)oracle_f16_to_f32(h), -e);
}

/* ------------------------------------------------------------------------ */
/* Section 2.1: the conductor and the row tracker.                           */
/* ------------------------------------------------------------------------ */

/*
 * One charge recurrence step for a whole matrix, given each row's weight for
 * the window (hit count, or output magnitude) and the window's largest weight.
 * Section 2.1: at the end of an observation window every charge is halved
 * and gains half of the row's share (its weight over the busiest row's); a
 * row is active while its charge is at least 0.01.  Readings: fp32 charges,
 * an empty window (largest weight 0) only halves the charges, the threshold
 * is inclusive.
 */
static void charge_step(float *ch, int64_t rows, const double *weight, double wmax,
                        uint8_t *active)
{
    for (int64_t r = 0; r < rows; ++r) {
        float share = 0.0f;
        if (wmax > 0.0)
            share = (float)weight[r] / (float)wmax;
        ch[r] = 0.5f * ch[r] + 0.5f * share;
        active[r] = ch[r] >= 0.01f ? 1 : 0;
    }
}

/* Conductor (section 2.1): weights are the window's token hit counts. */
ORACLE_API int oracle_conductor_window(float *ch, int64_t rows, const int32_t *tokens,
                                       int64_t n_tokens, uint8_t *active)
{
    for (int64_t i = 0; i < n_tokens; ++i)
        if (tokens[i] < 0 || tokens[i] >= rows)
            return -1;
    double *hits = calloc((size_t)(rows > 0 ? rows : 1), sizeof(double));
    if (!hits)
        return -2;
    for (int64_t i = 0; i < n_tokens; ++i)
        hits[tokens[i]] += 1.0;
    double busiest = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        if (hits[r] > busiest)
            busiest = hits[r];
    charge_step(ch, rows, hits, busiest, active);
    free(hits);
    return 0;
}

/* Row tracker (section 2.1): weights are the rows' output magnitudes (>= 0). */
ORACLE_API int oracle_tracker_window(float *ch, int64_t rows, const float *magnitude,
                                     uint8_t *active)
{
    double *w = malloc((size_t)(rows > 0 ? rows : 1) * sizeof(double));
    if (!w)
        return -2;
    double wmax = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        if (!(magnitude[r] >= 0.0f)) {
            free(w);
            return -1;
        }
        w[r] = magnitude[r];
        if (w[r] > wmax)
            wmax = w[r];
    }
    charge_step(ch, rows, w, wmax, active);
    free(w);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Mask bookkeeping: tiles of 32 rows (section 2.2), moment slots (2.3).      */
/* ------------------------------------------------------------------------ */

/*
 * bits[j] bit i is the mask of row 32*j+i; active_rows lists the active rows
 * in ascending order; active_tiles lists the tiles with any active row.
 */
ORACLE_API void oracle_plan_rows(const uint8_t *active, int64_t rows, uint32_t *bits,
                                 int32_t *active_rows, int64_t *n_active,
                                 int32_t *active_tiles, int64_t *n_tiles)
{
    int64_t tiles = (rows + 31) / 32;
    int64_t na = 0, nt = 0;
    for (int64_t j = 0; j < tiles; ++j) {
        uint32_t word = 0;
        for (int i = 0; i < 32; ++i) {
            int64_t r = 32 * j + i;
            if (r < rows && active[r]) {
                word |= (uint32_t)1 << i;
                active_rows[na++] = (int32_t)r;
            }
        }
        bits[j] = word;
        if (word)
            active_tiles[nt++] = (int32_t)j;
    }
    *n_active = na;
    *n_tiles = nt;
}

/* Token positions of every active embedding row, rows and positions ascending. */
ORACLE_API void oracle_plan_embedding(const int32_t *active_rows, int64_t n_active,
                                      const int32_t *tokens, int64_t n_tokens,
                                      int32_t *row_ptr, int32_t *positions, int64_t *nnz)
{
    int64_t n = 0;
    row_ptr[0] = 0;
    for (int64_t k = 0; k < n_active; ++k) {
        for (int64_t t = 0; t < n_tokens; ++t)
            if (tokens[t] == active_rows[k])
                positions[n++] = (int32_t)t;
        row_ptr[k + 1] = (int32_t)n;
    }
    *nnz = n;
}

/*
 * Moment slots (section 2.3: the moments exist only for active rows).
 * Reading: a row keeps its slot while it stays active; a row that became
 * inactive frees its slot; a newly active row takes the lowest free slot and
 * starts from zero moments and a zero step count (fresh = 1).
 * row_slot[R] is the persistent map row -> slot (-1 = none).
 */
ORACLE_API int oracle_slots_update(int32_t *row_slot, int64_t rows, int64_t n_slots,
                                   const int32_t *active_rows, int64_t n_active,
                                   int32_t *slot, uint8_t *fresh)
{
    if (n_active > n_slots)
        return -1;
    uint8_t *is_active = calloc((size_t)(rows > 0 ? rows : 1), 1);
    uint8_t *used = calloc((size_t)(n_slots > 0 ? n_slots : 1), 1);
    if (!is_active || !used) {
        free(is_active);
        free(used);
        return -2;
    }
    for (int64_t k = 0; k < n_active; ++k)
        is_active[active_rows[k]] = 1;
    for (int64_t r = 0; r < rows; ++r) {
        if (!is_active[r])
            row_slot[r] = -1;
        else if (row_slot[r] >= 0)
            used[row_slot[r]] = 1;
    }
    for (int64_t k = 0; k < n_active; ++k) {
        int32_t r = active_rows[k];
        if (row_slot[r] >= 0) {
            slot[k] = row_slot[r];
            fresh[k] = 0;
            continue;
        }
        int64_t s = 0;
        while (used[s])
            ++s;
        used[s] = 1;
        row_slot[r] = (int32_t)s;
        slot[k] = (int32_t)s;
        fresh[k] = 1;
    }
    free(is_active);
    free(used);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Section 2.2: the masked weight gradient.                                 */
/* ------------------------------------------------------------------------ */

/*
 * dW = dY^T X restricted to the active output rows: for the k-th active row r,
 *   dW_act[k, c] = sum_t dY[t, r] * X[t, c],
 * each sum taken in fp64 and rounded to fp32 once.  Inactive rows produce no
 * output at all.  dY is bf16 [T x R], X is bf16 [T x C], both row-major.
 */
ORACLE_API void oracle_masked_dw(const uint16_t *dY, int64_t T, int64_t R, const uint16_t *X,
                                 int64_t C, const int32_t *active_rows, int64_t n_active,
                                 float *dW_act)
{
    for (int64_t k = 0; k < n_active; ++k) {
        int64_t r = active_rows[k];
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += (double)oracle_bf16_to_f32(dY[t * R + r]) *
                       (double)oracle_bf16_to_f32(X[t * C + c]);
            dW_act[k * C + c] = (float)acc;
        }
    }
}

/*
 * The embedding's weight gradient is the same product with a one-hot input:
 * row r of the gradient is the sum of dY over the positions whose token is r.
 * Summed in fp64 and rounded once, as above.  dY is bf16 [T x d].
 */
ORACLE_API void oracle_embedding_dw(const uint16_t *dY, int64_t T, int64_t d,
                                    const int32_t *tokens, const int32_t *active_rows,
                                    int64_t n_active, float *dW_act)
{
    for (int64_t k = 0; k < n_active; ++k) {
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                if (tokens[t] == active_rows[k])
                    acc += (double)oracle_bf16_to_f32(dY[t * d + c]);
            dW_act[k * d + c] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Sections 2.3-2.4: the sparse int8 + residual Adam update.                 */
/* ------------------------------------------------------------------------ */

/* Adam bias corrections 1 - beta^t, computed in fp64 and rounded once. */
ORACLE_API void oracle_bias_table(float beta1, float beta2, int32_t t_max, float *bc1,
                                  float *bc2)
{
    bc1[0] = 0.0f;
    bc2[0] = 0.0f;
    for (int32_t t = 1; t <= t_max; ++t) {
        bc1[t] = (float)(1.0 - pow((double)beta1, (double)t));
        bc2[t] = (float)(1.0 - pow((double)beta2, (double)t));
    }
}

typedef struct {
    int64_t R, C, n_active;
    const int32_t *active_rows; /* [n_active], ascending */
    const int32_t *slot;        /* [n_active], moment slot of each active row */
    const uint8_t *fresh;       /* [n_active] or NULL: 1 = moments start at zero */
    const float *G;             /* [n_active x C] gradient of the active rows */
    int8_t *q;                  /* [R x C] */
    float *s;                   /* [R] */
    float *delta;               /* [R x C] */
    uint16_t *m, *v;            /* fp16 [n_slots x C], scaled by 2^mv_exp (see above) */
    int32_t *t;                 /* [n_slots] */
    int8_t *mv_exp;             /* [n_slots x 2]: exponent of the slot's m row, of its v row */
    int64_t n_slots;
    uint16_t *w_live;           /* bf16 [R x C] or NULL */
} oracle_mat;

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
} oracle_adam;

/*
 * Update one active row of a matrix with the (effective) gradient g[C].
 *
 * Section 2.3: storage is an int8 code q, a scale s per row and an fp32
 * residual delta; the fp32 weight w = s*q + delta is rebuilt, stepped and
 * split again into q and delta; m and v live in fp16.  The
 * equation of the quantiser is lost; the reading is: w is rebuilt with two
 * roundings (product, then sum), the new scale is the row's largest |w'| over
 * 127, q' = clamp(rint(w'/s'), -127, 127) and delta' = w' - s'*q' (exact by
 * Sterbenz's lemma, so s'*q' + delta' gives w' back); a zero row keeps q' = 0
 * and delta' = w'.
 *
 * Section 2.4 / Kingma-Ba Adam with bias correction: fp32 moments decoded
 * from the stored scaled fp16 rows drive the step, the new moments are
 * stored as scaled fp16 rows (exponents from the new rows' maxima).  The step
 * is lr * mhat / (sqrt(vhat) + eps) with mhat = m / (1 - beta1^t) and
 * vhat = v / (1 - beta2^t).  Reading of the rounding order: the two bias
 * corrections are per-row factors, k1 = lr / bc1 and k2 = 1 / sqrt(bc2)
 * (fp32, bc1 and bc2 as below), applied as multiplications, which is the
 * reordering Kingma and Ba themselves give for an efficient step: per
 * element u = (k1 * m) / (sqrt(v) * k2 + eps), one division and one square
 * root.  Decoupled weight decay multiplies w by (1 - lr*lambda) before the
 * step (by 1, exactly, when lambda = 0).
 *
 * Requantisation reading: q' = clamp(rint(w' * r), -127, 127) with r = 1/s'
 * the row's reciprocal scale (fp32); only if r overflows (s' below 2^-128)
 * does the row divide, q' = rint(w' / s').  Either way q' is a nearest code of
 * w'/s' (to within the reciprocal's rounding near a .5 tie) and
 * delta' = w' - s'*q' stays exact.
 */
static void update_row(oracle_mat *M, int64_t k, const float *g, const oracle_adam *hp,
                       float *wnew, float *mnew, float *vnew)
{
    int64_t C = M->C;
    int64_t r = M->active_rows[k];
    int64_t sl = M->slot[k];
    int fresh = M->fresh ? M->fresh[k] : 0;
    int32_t step = (fresh ? 0 : M->t[sl]) + 1;
    float bc1 = (float)(1.0 - pow((double)hp->beta1, (double)step));
    float bc2 = (float)(1.0 - pow((double)hp->beta2, (double)step));
    float k1 = hp->lr / bc1;               /* per-row factors of the bias corrections */
    float sbc2 = sqrtf(bc2);
    float k2 = 1.0f / sbc2;
    float c1 = 1.0f - hp->beta1;
    float c2 = 1.0f - hp->beta2;
    float lrwd = hp->lr * hp->weight_decay;
    float decay = 1.0f - lrwd;
    float s_old = M->s[r];
    int em_old = fresh ? 0 : M->mv_exp[2 * sl];
    int ev_old = fresh ? 0 : M->mv_exp[2 * sl + 1];

    for (int64_t c = 0; c < C; ++c) {
        int64_t e = r * C + c;
        float sq = s_old * (float)M->q[e];
        float w = sq + M->delta[e];
        float m_old = fresh ? 0.0f : oracle_moment_decode(M->m[sl * C + c], em_old);
        float v_old = fresh ? 0.0f : oracle_moment_decode(M->v[sl * C + c], ev_old);
        float gc = g[c];
        float m_a = hp->beta1 * m_old;
        float m_b = c1 * gc;
        float m = m_a + m_b;
        float gg = gc * gc;
        float v_a = hp->beta2 * v_old;
        float v_b = c2 * gg;
        float v = v_a + v_b;
        mnew[c] = m;
        vnew[c] = v;
        float sv = sqrtf(v);
        float sk = sv * k2;
        float den = sk + hp->eps;
        float num = k1 * m;
        float u = num / den;
        float w1 = w * decay;
        wnew[c] = w1 - u;
    }
    M->t[sl] = step;

    /* the moments leave as scaled fp16 rows */
    float mmax = 0.0f, vmax = 0.0f;
    for (int64_t c = 0; c < C; ++c) {
        if (fabsf(mnew[c]) > mmax)
            mmax = fabsf(mnew[c]);
        if (fabsf(vnew[c]) > vmax)
            vmax = fabsf(vnew[c]);
    }
    int em = oracle_moment_exponent(mmax);
    int ev = oracle_moment_exponent(vmax);
    M->mv_exp[2 * sl] = (int8_t)em;
    M->mv_exp[2 * sl + 1] = (int8_t)ev;
    for (int64_t c = 0; c < C; ++c) {
        M->m[sl * C + c] = oracle_moment_encode(mnew[c], em);
        M->v[sl * C + c] = oracle_moment_encode(vnew[c], ev);
    }

    float amax = 0.0f;
    for (int64_t c = 0; c < C; ++c)
        if (fabsf(wnew[c]) > amax)
            amax = fabsf(wnew[c]);
    float s_new = amax / 127.0f;
    float rs = s_new != 0.0f ? 1.0f / s_new : 0.0f;
    int by_division = s_new != 0.0f && isinf(rs);
    M->s[r] = s_new;
    for (int64_t c = 0; c < C; ++c) {
        int64_t e = r * C + c;
        float qf = 0.0f;
        if (s_new != 0.0f) {
            float x = by_division ? wnew[c] / s_new : wnew[c] * rs;
            qf = rintf(x);
            if (qf > 127.0f)
                qf = 127.0f;
            if (qf < -127.0f)
                qf = -127.0f;
        }
        float sq = s_new * qf;
        float d = wnew[c] - sq;
        M->q[e] = (int8_t)qf;
        M->delta[e] = d;
        if (M->w_live) {
            float back = sq + d;
            M->w_live[e] = oracle_f32_to_bf16(back);
        }
    }
}

static int check_mat(const oracle_mat *M)
{
    if (M->C <= 0 || M->R < 0 || M->n_active < 0)
        return -1;
    for (int64_t k = 0; k < M->n_active; ++k) {
        if (M->active_rows[k] < 0 || M->active_rows[k] >= M->R)
            return -1;
        if (k > 0 && M->active_rows[k] <= M->active_rows[k - 1])
            return -1;
        if (M->slot[k] < 0 || M->slot[k] >= M->n_slots)
            return -1;
    }
    return 0;
}

/* Plain (uncoupled) update of every active row: section 2.4's plain Adam step. */
ORACLE_API int oracle_sparse_update(oracle_mat *M, const oracle_adam *hp)
{
    if (check_mat(M))
        return -1;
    float *wnew = malloc((size_t)M->C * sizeof(float));
    float *mnew = malloc((size_t)M->C * sizeof(float));
    float *vnew = malloc((size_t)M->C * sizeof(float));
    if (!wnew || !mnew || !vnew) {
        free(wnew); free(mnew); free(vnew);
        return -2;
    }
    for (int64_t k = 0; k < M->n_active; ++k)
        update_row(M, k, M->G + k * M->C, hp, wnew, mnew, vnew);
    free(wnew); free(mnew); free(vnew);
    return 0;
}

/*
 * Coupled update of a pair (A, B) of equally shaped matrices, section 2.4:
 * the step of each matrix also sees its partner's gradient.  The lost equations give
 * the effective gradients as a blend of the two clipped gradients; with the
 * blend weights given as inputs (own weight a_own, cross weight a_cross, clip
 * factors clip_a and clip_b) the reading is
 *   gA~ = a_own * (clip_a * gA) + a_cross * (clip_b * gB)
 *   gB~ = a_own * (clip_b * gB) + a_cross * (clip_a * gA),
 * each product and the sum rounded in fp32, over the union of the two masks;
 * a matrix whose row is inactive contributes a zero gradient and its own row
 * is not updated.  Each effective gradient then drives the step above.
 */
ORACLE_API int oracle_coupled_update(oracle_mat *A, oracle_mat *B, float a_own, float a_cross,
                                     float clip_a, float clip_b, const oracle_adam *hp)
{
    if (check_mat(A) || check_mat(B) || A->R != B->R || A->C != B->C)
        return -1;
    int64_t C = A->C;
    float *ga = malloc((size_t)C * sizeof(float));
    float *gb = malloc((size_t)C * sizeof(float));
    float *ea = malloc((size_t)C * sizeof(float));
    float *eb = malloc((size_t)C * sizeof(float));
    float *wnew = malloc((size_t)C * sizeof(float));
    float *mnew = malloc((size_t)C * sizeof(float));
    float *vnew = malloc((size_t)C * sizeof(float));
    if (!ga || !gb || !ea || !eb || !wnew || !mnew || !vnew) {
        free(ga); free(gb); free(ea); free(eb); free(wnew); free(mnew); free(vnew);
        return -2;
    }
    int64_t ia = 0, ib = 0;
    while (ia < A->n_active || ib < B->n_active) {
        int64_t ra = ia < A->n_active ? A->active_rows[ia] : INT64_MAX;
        int64_t rb = ib < B->n_active ? B->active_rows[ib] : INT64_MAX;
        int64_t r = ra < rb ? ra : rb;
        int has_a = ra == r, has_b = rb == r;
        for (int64_t c = 0; c < C; ++c) {
            ga[c] = has_a ? A->G[ia * C + c] : 0.0f;
            gb[c] = has_b ? B->G[ib * C + c] : 0.0f;
        }
        for (int64_t c = 0; c < C; ++c) {
            float ca = clip_a * ga[c];
            float cb = clip_b * gb[c];
            float own_a = a_own * ca, cross_a = a_cross * cb;
            float own_b = a_own * cb, cross_b = a_cross * ca;
            ea[c] = own_a + cross_a;
            eb[c] = own_b + cross_b;
        }
        if (has_a)
            update_row(A, ia++, ea, hp, wnew, mnew, vnew);
        if (has_b)
            update_row(B, ib++, eb, hp, wnew, mnew, vnew);
    }
    free(ga); free(gb); free(ea); free(eb); free(wnew); free(mnew); free(vnew);
    return 0;
}

/*
 * Section 2.3's sparse write-back: the live bf16 weights of the active rows
 * are rebuilt from the stored state, w = s*q + delta (two roundings), and
 * converted to bf16; every other row is left untouched.
 */
ORACLE_API void oracle_masked_writeback(const int8_t *q, const float *s, const float *delta,
                                        int64_t R, int64_t C, const int32_t *active_rows,
                                        int64_t n_active, uint16_t *w_live)
{
    (void)R;
    for (int64_t k = 0; k < n_active; ++k) {
        int64_t r = active_rows[k];
        for (int64_t c = 0; c < C; ++c) {
            float sq = s[r] * (float)q[r * C + c];
            float w = sq + delta[r * C + c];
            w_live[r * C + c] = oracle_f32_to_bf16(w);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* SparseLeaf: gradients and Adam of K selected connections.                */
/* ------------------------------------------------------------------------ */

/*
 * The blog post "SparseLeaf: synaptic sparse fine-tuning" (di-zhang-llm.github
 * .io), section "Weight gradients: write the selected results directly": for
 * Y = X W^T and D = dL/dY, each selected connection (i_k, j_k) receives the
 * dot product over token positions of column i_k of D and column j_k of X,
 * written into a length-K buffer.  D is bf16 [T x m], X bf16 [T x n]; summed
 * in fp64 and rounded to fp32 once, like the masked dW above.
 */
ORACLE_API void oracle_leaf_grad(const uint16_t *D, const uint16_t *X, int64_t T, int64_t m,
                                 int64_t n, const int32_t *rows, const int32_t *cols, int64_t K,
                                 float *g)
{
    for (int64_t k = 0; k < K; ++k) {
        int64_t i = rows[k], j = cols[k];
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t)
            acc += (double)oracle_bf16_to_f32(D[t * m + i]) * (double)oracle_bf16_to_f32(X[t * n + j]);
        g[k] = (float)acc;
    }
}

/*
 * SparseLeaf Adam (same post, section "The optimizer"): theta, m and v start
 * at zero; at step t >= 1 the moments of each selected coordinate follow
 * Adam, are bias-corrected with 1 - beta^t and move theta by
 * lr * mhat / (sqrt(vhat) + eps), all elementwise.  The post's memory ledger
 * keeps an fp32 master theta and fp32 moments and computes with a bf16 copy
 * of theta.  Reading: the same fp32 rounding steps as update_row above (no
 * weight decay, which the post's step does not have), theta_bf16 = RNE(theta).
 */
ORACLE_API void oracle_leaf_adam(int64_t K, const float *g, float *theta, float *m, float *v,
                                 uint16_t *theta_bf16, int32_t step, float lr, float beta1,
                                 float beta2, float eps)
{
    float bc1 = (float)(1.0 - pow((double)beta1, (double)step));
    float bc2 = (float)(1.0 - pow((double)beta2, (double)step));
    float c1 = 1.0f - beta1;
    float c2 = 1.0f - beta2;
    for (int64_t k = 0; k < K; ++k) {
        float gk = g[k];
        float m_a = beta1 * m[k];
        float m_b = c1 * gk;
        float mk = m_a + m_b;
        float gg = gk * gk;
        float v_a = beta2 * v[k];
        float v_b = c2 * gg;
        float vk = v_a + v_b;
        float mhat = mk / bc1;
        float vhat = vk / bc2;
        float denom = sqrtf(vhat) + eps;
        float ratio = mhat / denom;
        float u = lr * ratio;
        m[k] = mk;
        v[k] = vk;
        theta[k] = theta[k] - u;
        if (theta_bf16)
            theta_bf16[k] = oracle_f32_to_bf16(theta[k]);
    }
}

/* Array forms of the conversions above (for tests that convert many values). */
ORACLE_API void oracle_moment_encode_array(const float *x, int64_t n, int e, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_moment_encode(x[i], e);
}

ORACLE_API void oracle_moment_decode_array(const uint16_t *h, int64_t n, int e, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_moment_decode(h[i], e);
}

ORACLE_API void oracle_f32_to_f16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_f16(x[i]);
}

ORACLE_API void oracle_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(x[i]);
}

ORACLE_API void oracle_f16_to_f32_array(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f32(h[i]);
}

ORACLE_API void oracle_bf16_to_f32_array(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f32(h[i]);
}
