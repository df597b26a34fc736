// sft_host.cpp -- host side of the sparse-first step: the error channel, the
// conductor and row tracker, row plans, embedding CSR, moment slots and the
// Adam bias-correction table.
//
// Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
// Active Set", section 2.1 (the conductor holds a charge per row; at each
// window's end the charge is halved and half of the row's hit count relative
// to the window's busiest row is added; a row counts as active while its
// charge is at least 0.01; the row tracker runs the same recurrence on output
// magnitudes; the CPU derives the masks once per step) and section 2.2 (the
// mask is tested 32 rows at a time).  These run on the CPU by design: the page keeps mask decisions on the
// host, one step ahead of the GPU.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "sft_internal.h"

namespace sft {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

namespace {

// Charge recurrence over `rows` given each row's window weight (hit count or
// magnitude) and the window's largest weight.  fp32 throughout: the halving
// and the half share are exact, the sum rounds once.
void charge_update(float *ch, int64_t rows, const float *weight, float wmax, uint8_t *active) {
    for (int64_t r = 0; r < rows; ++r) {
        const float share = wmax > 0.0f ? weight[r] / wmax : 0.0f;
        const float next = 0.5f * ch[r] + 0.5f * share;
        ch[r] = next;
        active[r] = next >= 0.01f;
    }
}

}  // namespace
}  // namespace sft

using namespace sft;

extern "C" {

const char *sft_last_error(void) { return g_last_error.c_str(); }

int sft_abi_version(void) { return SFT_ABI_VERSION; }

int sft_conductor_window(float *ch, int64_t rows, const int32_t *tokens, int64_t n_tokens,
                         uint8_t *active) {
    clear_error();
    SFT_CHECK(rows >= 0 && n_tokens >= 0, SFT_EINVAL, "conductor: negative size");
    SFT_CHECK(rows == 0 || (ch && active), SFT_EINVAL, "conductor: null charge/mask array");
    SFT_CHECK(n_tokens == 0 || tokens, SFT_EINVAL, "conductor: null tokens");
    // Hit counts are exact in fp32 up to 2^24 tokens per window.
    SFT_CHECK(n_tokens <= (int64_t(1) << 24), SFT_ENOTSUP, "conductor: window over 2^24 tokens");
    std::vector<float> hits(static_cast<size_t>(rows), 0.0f);
    for (int64_t i = 0; i < n_tokens; ++i) {
        const int32_t tok = tokens[i];
        SFT_CHECK(tok >= 0 && tok < rows, SFT_EINVAL, "conductor: token %d at %lld out of [0, %lld)",
                  tok, (long long)i, (long long)rows);
    }
    for (int64_t i = 0; i < n_tokens; ++i) hits[tokens[i]] += 1.0f;
    float busiest = 0.0f;
    for (float h : hits) busiest = std::max(busiest, h);
    charge_update(ch, rows, hits.data(), busiest, active);
    return SFT_OK;
}

int sft_tracker_window(float *ch, int64_t rows, const float *magnitude, uint8_t *active) {
    clear_error();
    SFT_CHECK(rows >= 0, SFT_EINVAL, "tracker: negative size");
    SFT_CHECK(rows == 0 || (ch && magnitude && active), SFT_EINVAL, "tracker: null array");
    float wmax = 0.0f;
    for (int64_t r = 0; r < rows; ++r) {
        SFT_CHECK(magnitude[r] >= 0.0f && std::isfinite(magnitude[r]), SFT_EINVAL,
                  "tracker: magnitude[%lld] is negative or not finite", (long long)r);
        wmax = std::max(wmax, magnitude[r]);
    }
    charge_update(ch, rows, magnitude, wmax, active);
    return SFT_OK;
}

int sft_plan_rows(const uint8_t *active, sft_plan *plan) {
    clear_error();
    SFT_CHECK(plan, SFT_EINVAL, "plan_rows: null plan");
    const int64_t rows = plan->rows;
    SFT_CHECK(rows >= 0 && rows < (int64_t(1) << 31), SFT_EINVAL, "plan_rows: rows out of range");
    SFT_CHECK(rows == 0 || (active && plan->tile_bits && plan->active_rows && plan->active_tiles),
              SFT_EINVAL, "plan_rows: null array");
    const int64_t tiles = (rows + 31) / 32;
    int64_t na = 0, nt = 0;
    for (int64_t j = 0; j < tiles; ++j) {
        const int64_t lo = 32 * j;
        const int64_t hi = std::min<int64_t>(lo + 32, rows);
        uint32_t word = 0;
        for (int64_t r = lo; r < hi; ++r) {
            if (active[r]) {
                word |= 1u << (r - lo);
                plan->active_rows[na++] = static_cast<int32_t>(r);
            }
        }
        plan->tile_bits[j] = word;
        if (word) {
            if (plan->active_bits) plan->active_bits[nt] = word;
            if (plan->tile_first) plan->tile_first[nt] = static_cast<int32_t>(na - __builtin_popcount(word));
            plan->active_tiles[nt++] = static_cast<int32_t>(j);
        }
    }
    plan->n_active = na;
    plan->n_active_tiles = nt;
    return SFT_OK;
}

int sft_plan_embedding(const sft_plan *plan, const int32_t *tokens, int64_t n_tokens,
                       int32_t *row_ptr, int32_t *positions, int64_t positions_cap, int64_t *nnz) {
    clear_error();
    SFT_CHECK(plan && row_ptr && nnz, SFT_EINVAL, "plan_embedding: null argument");
    SFT_CHECK(n_tokens >= 0 && n_tokens < (int64_t(1) << 31), SFT_EINVAL,
              "plan_embedding: n_tokens out of range");
    SFT_CHECK(n_tokens == 0 || tokens, SFT_EINVAL, "plan_embedding: null tokens");
    const int64_t rows = plan->rows, na = plan->n_active;
    SFT_CHECK(na == 0 || plan->active_rows, SFT_EINVAL, "plan_embedding: null active_rows");
    // Row -> position in the active list (-1 = inactive), then a counting sort
    // of the token positions by row; a stable pass keeps positions ascending.
    std::vector<int32_t> index(static_cast<size_t>(rows), -1);
    for (int64_t k = 0; k < na; ++k) index[plan->active_rows[k]] = static_cast<int32_t>(k);
    std::vector<int64_t> count(static_cast<size_t>(na) + 1, 0);
    for (int64_t t = 0; t < n_tokens; ++t) {
        const int32_t tok = tokens[t];
        SFT_CHECK(tok >= 0 && tok < rows, SFT_EINVAL, "plan_embedding: token %d out of range", tok);
        if (index[tok] >= 0) ++count[index[tok] + 1];
    }
    for (int64_t k = 0; k < na; ++k) count[k + 1] += count[k];
    SFT_CHECK(count[na] <= positions_cap, SFT_ECAPACITY,
              "plan_embedding: %lld positions exceed capacity %lld", (long long)count[na],
              (long long)positions_cap);
    SFT_CHECK(count[na] == 0 || positions, SFT_EINVAL, "plan_embedding: null positions");
    for (int64_t k = 0; k <= na; ++k) row_ptr[k] = static_cast<int32_t>(count[k]);
    std::vector<int64_t> fill(count.begin(), count.end() - 1);
    for (int64_t t = 0; t < n_tokens; ++t) {
        const int32_t k = index[tokens[t]];
        if (k >= 0) positions[fill[k]++] = static_cast<int32_t>(t);
    }
    *nnz = count[na];
    return SFT_OK;
}

int sft_slots_update(int32_t *row_slot, int64_t rows, int64_t n_slots, const int32_t *active_rows,
                     int64_t n_active, int32_t *slot, uint8_t *fresh) {
    clear_error();
    SFT_CHECK(rows >= 0 && n_slots >= 0 && n_active >= 0, SFT_EINVAL, "slots: negative size");
    SFT_CHECK(rows == 0 || row_slot, SFT_EINVAL, "slots: null row_slot");
    SFT_CHECK(n_active == 0 || (active_rows && slot && fresh), SFT_EINVAL, "slots: null array");
    SFT_CHECK(n_active <= n_slots, SFT_ECAPACITY, "slots: %lld active rows exceed %lld slots",
              (long long)n_active, (long long)n_slots);
    for (int64_t k = 0; k < n_active; ++k) {
        SFT_CHECK(active_rows[k] >= 0 && active_rows[k] < rows, SFT_EINVAL,
                  "slots: active row %d out of range", active_rows[k]);
        SFT_CHECK(k == 0 || active_rows[k] > active_rows[k - 1], SFT_EINVAL,
                  "slots: active rows not strictly ascending at %lld", (long long)k);
    }
    for (int64_t r = 0; r < rows; ++r)
        SFT_CHECK(row_slot[r] >= -1 && row_slot[r] < n_slots, SFT_EINVAL,
                  "slots: row_slot[%lld] = %d out of range", (long long)r, row_slot[r]);
    // Walk rows and the sorted active list together: rows that left the set
    // free their slot; survivors mark theirs as taken.
    std::vector<uint8_t> taken(static_cast<size_t>(n_slots), 0);
    int64_t k = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const bool on = k < n_active && active_rows[k] == r;
        if (on) ++k;
        if (!on) row_slot[r] = -1;
        else if (row_slot[r] >= 0) taken[row_slot[r]] = 1;
    }
    int64_t next_free = 0;
    for (int64_t i = 0; i < n_active; ++i) {
        const int32_t r = active_rows[i];
        if (row_slot[r] >= 0) {
            slot[i] = row_slot[r];
            fresh[i] = 0;
            continue;
        }
        while (taken[next_free]) ++next_free;  // lowest free slot (ascending scan)
        taken[next_free] = 1;
        row_slot[r] = static_cast<int32_t>(next_free);
        slot[i] = static_cast<int32_t>(next_free);
        fresh[i] = 1;
    }
    return SFT_OK;
}

int sft_bias_table(float beta1, float beta2, int32_t t_max, float *bc1, float *bc2) {
    clear_error();
    SFT_CHECK(bc1 && bc2, SFT_EINVAL, "bias_table: null array");
    SFT_CHECK(t_max >= 1, SFT_EINVAL, "bias_table: t_max < 1");
    SFT_CHECK(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f, SFT_EINVAL,
              "bias_table: beta outside [0, 1)");
    bc1[0] = 0.0f;
    bc2[0] = 0.0f;
    // Powers by repeated fp64 multiplication would drift from pow(); use pow()
    // on the fp32 betas widened to double, then round once.
    for (int32_t t = 1; t <= t_max; ++t) {
        bc1[t] = static_cast<float>(1.0 - std::pow(static_cast<double>(beta1), t));
        bc2[t] = static_cast<float>(1.0 - std::pow(static_cast<double>(beta2), t));
    }
    return SFT_OK;
}

// Checkpoint-and-rewind controller (section 2.6); the readings it implements
// are stated with the declaration.  All arithmetic in double.
int sft_rewind_init(sft_rewind *st) {
    clear_error();
    SFT_CHECK(st, SFT_EINVAL, "rewind_init: null state");
    std::memset(st, 0, sizeof(*st));
    st->save_within = 0.10;
    st->rise_above = 0.15;
    st->watch_steps = 10;
    st->max_recoveries = 3;
    st->min_loss = HUGE_VAL;
    st->checkpoint_step = -1;
    st->min_step = -1;
    return SFT_OK;
}

namespace {
// The minimum's copy becomes the checkpoint, with the minimum's loss.
int32_t rewind_accept(sft_rewind *st) {
    st->has_checkpoint = 1;
    st->checkpoint_loss = st->min_loss;
    st->checkpoint_step = st->min_step;
    return SFT_REWIND_PROMOTE;
}
}  // namespace

int sft_rewind_observe(sft_rewind *st, double loss, int32_t *action) {
    clear_error();
    SFT_CHECK(st && action, SFT_EINVAL, "rewind_observe: null pointer");
    SFT_CHECK(st->save_within >= 0.0 && st->rise_above >= 0.0, SFT_EINVAL,
              "rewind_observe: save_within and rise_above must be >= 0");
    SFT_CHECK(st->watch_steps >= 1 && st->max_recoveries >= 0, SFT_EINVAL,
              "rewind_observe: watch_steps < 1 or max_recoveries < 0");
    const double x = std::isfinite(loss) ? loss : HUGE_VAL;
    const int64_t k = st->step++;
    int32_t act = 0;
    // the end of an open watch
    if (st->watch_left > 0 && --st->watch_left == 0) {
        if (x > (1.0 + st->rise_above) * st->min_loss && st->recoveries < st->max_recoveries) {
            ++st->recoveries;
            st->watch_left = st->watch_steps;
            *action = SFT_REWIND_RESTORE;
            return SFT_OK;
        }
        act |= rewind_accept(st);
    }
    // a new minimum; one still being watched is accepted first
    if (x < st->min_loss) {
        if (st->watch_left > 0) act |= rewind_accept(st);
        st->min_loss = x;
        st->min_step = k;
        st->watch_left = st->watch_steps;
        st->recoveries = 0;
        act |= SFT_REWIND_SAVE_MIN;
    }
    // the refresh: never during a watch, never above the rise bound
    if (x != HUGE_VAL &&
        (!st->has_checkpoint || (st->watch_left == 0 && x <= (1.0 + st->save_within) * st->checkpoint_loss &&
                                 x <= (1.0 + st->rise_above) * st->min_loss))) {
        st->has_checkpoint = 1;
        st->checkpoint_loss = x;
        st->checkpoint_step = k;
        act |= SFT_REWIND_SAVE;
    }
    *action = act;
    return SFT_OK;
}

// The coupled update's scalar schedule; the readings it implements are
// stated with the declaration.  Double precision throughout.
namespace {
constexpr int32_t kFib[8] = {1, 1, 2, 3, 5, 8, 13, 21};
}

int sft_helix_init(sft_helix *h) {
    clear_error();
    SFT_CHECK(h, SFT_EINVAL, "helix_init: null state");
    std::memset(h, 0, sizeof(*h));
    h->decay_len = 10.0;
    h->up_threshold = 1e-4;
    h->rung_deg = 36.0;
    h->M = 1.833;
    h->mu = 1.0;
    h->mod_plus = 0.10;
    h->mod_minus = 0.05;
    return SFT_OK;
}

int sft_helix_step(sft_helix *h, double loss, int32_t rewind, int32_t *stride, double *phase_deg) {
    clear_error();
    SFT_CHECK(h && std::isfinite(loss), SFT_EINVAL, "helix_step: null state or non-finite loss");
    SFT_CHECK(h->decay_len > 0.0 && h->rung >= 0 && h->rung < 8, SFT_EINVAL, "helix_step: bad settings or rung");
    const double r = std::exp(-1.0 / h->decay_len);
    if (h->has_loss) {
        const double d = h->last_loss - loss;
        h->trend_sum = d + r * h->trend_sum;
        h->trend_w = 1.0 + r * h->trend_w;
        const double trend = h->trend_sum / h->trend_w;
        h->smooth_sum = trend + r * h->smooth_sum;
        h->smooth_w = 1.0 + r * h->smooth_w;
    }
    h->last_loss = loss;
    h->has_loss = 1;
    const double smooth = h->smooth_w > 0.0 ? h->smooth_sum / h->smooth_w : 0.0;
    if (rewind)
        h->rung = 0;
    else if (smooth > h->up_threshold)
        h->rung = std::min(h->rung + 1, 7);
    else if (smooth < 0.0)
        h->rung = std::max(h->rung - 1, 0);
    h->rotation += h->rung_deg * kFib[h->rung];
    if (stride) *stride = kFib[h->rung];
    if (phase_deg) *phase_deg = std::fmod(h->rotation, 360.0);
    return SFT_OK;
}

int sft_helix_coupling(const sft_helix *h, double b, double psi_deg, double *a_own, double *a_cross) {
    clear_error();
    SFT_CHECK(h && a_own && a_cross && std::isfinite(b) && std::isfinite(psi_deg), SFT_EINVAL,
              "helix_coupling: null pointer or non-finite b / psi");
    const double R = h->rotation;
    const double wp = 1.0 + h->mod_plus * std::cos(2.0 * M_PI * R / 360.0);
    const double wm = 1.0 + h->mod_minus * std::cos(2.0 * M_PI * R / 3600.0);
    SFT_CHECK(h->M > 0.0 && h->mu > 0.0 && wp > 0.0 && wm > 0.0, SFT_EINVAL,
              "helix_coupling: channel weights must be positive");
    const double e = (1.0 + std::cos((std::fmod(R, 360.0) + psi_deg) * (M_PI / 180.0))) / 2.0;
    const double sec = h->mu * wm * (1.0 - e);
    *a_own = 1.0;
    *a_cross = b * sec / (h->M * wp * e + sec);
    return SFT_OK;
}

}  // extern "C"