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
#include <emmintrin.h>

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
// magnitude) and the window's largest weight; returns the active rows'
// count.  fp32 throughout: the halving and the half share are exact, the sum
// rounds once.  Straight-line, so that the compiler vectorises it.
__attribute__((target_clones("avx2", "default")))
int64_t charge_update(float *__restrict__ ch, int64_t rows, const float *__restrict__ weight, float wmax,
                      uint8_t *__restrict__ active) {
    int32_t na = 0;
    if (wmax > 0.0f) {
        for (int64_t r = 0; r < rows; ++r) {
            const float share = weight[r] / wmax;
            const float next = 0.5f * ch[r] + 0.5f * share;
            ch[r] = next;
            const bool on = next >= 0.01f;
            active[r] = on;
            na += on;
        }
    } else {
        for (int64_t r = 0; r < rows; ++r) {
            const float next = 0.5f * ch[r] + 0.5f * 0.0f;
            ch[r] = next;
            const bool on = next >= 0.01f;
            active[r] = on;
            na += on;
        }
    }
    return na;
}

// The tracker's window: magnitudes must be finite and not below zero (-0
// passes); returns the first bad index or -1.  The largest magnitude comes
// from the integer order of the bit patterns with the sign cleared, which
// is the order of the values for the magnitudes that pass.
__attribute__((target_clones("avx2", "default")))
int64_t magnitude_max(const float *__restrict__ mag, int64_t rows, float *wmax) {
    uint32_t mx = 0, bad = 0;
    for (int64_t r = 0; r < rows; ++r) {
        uint32_t b;
        std::memcpy(&b, mag + r, 4);
        const uint32_t a = b & 0x7fffffffu;
        bad |= static_cast<uint32_t>(a >= 0x7f800000u) | static_cast<uint32_t>(b > 0x80000000u);
        mx = a > mx ? a : mx;
    }
    if (bad) {
        for (int64_t r = 0; r < rows; ++r)
            if (!(mag[r] >= 0.0f && std::isfinite(mag[r]))) return r;
    }
    std::memcpy(wmax, &mx, 4);
    return -1;
}

// 32 mask bytes (nonzero = active) as a bit word, bit i = byte i.
inline uint32_t mask_word(const uint8_t *a) {
    const __m128i z = _mm_setzero_si128();
    const uint32_t lo = static_cast<uint32_t>(_mm_movemask_epi8(
        _mm_cmpeq_epi8(_mm_loadu_si128(reinterpret_cast<const __m128i *>(a)), z)));
    const uint32_t hi = static_cast<uint32_t>(_mm_movemask_epi8(
        _mm_cmpeq_epi8(_mm_loadu_si128(reinterpret_cast<const __m128i *>(a + 16)), z)));
    return ~(lo | (hi << 16));
}

// The row plan of a mask (tile words, active rows, active tiles, their words
// and first indices); the last tile may be partial.
void plan_core(const uint8_t *__restrict__ active, int64_t rows, uint32_t *tile_bits, int32_t *active_rows,
               int32_t *active_tiles, uint32_t *active_bits, int32_t *tile_first, int64_t *n_active,
               int64_t *n_tiles) {
    const int64_t tiles = (rows + 31) / 32, full = rows / 32;
    int64_t na = 0, nt = 0;
    for (int64_t j = 0; j < tiles; ++j) {
        uint32_t word;
        if (j < full) {
            word = mask_word(active + 32 * j);
        } else {
            word = 0;
            for (int64_t r = 32 * j; r < rows; ++r) word |= (active[r] ? 1u : 0u) << (r - 32 * j);
        }
        if (tile_bits) tile_bits[j] = word;
        if (!word) continue;
        if (active_bits) active_bits[nt] = word;
        if (tile_first) tile_first[nt] = static_cast<int32_t>(na);
        active_tiles[nt++] = static_cast<int32_t>(j);
        for (uint32_t w = word; w; w &= w - 1)
            active_rows[na++] = static_cast<int32_t>(32 * j + __builtin_ctz(w));
    }
    *n_active = na;
    *n_tiles = nt;
}

// First row_slot entry outside [-1, n_slots), or -1.
int64_t row_slot_bad(const int32_t *__restrict__ row_slot, int64_t rows, int64_t n_slots) {
    // n_slots < 2^31: compare in 32 bits (vectorises without widening)
    const int32_t ns = static_cast<int32_t>(std::min<int64_t>(n_slots, INT32_MAX));
    const uint32_t wide = n_slots > INT32_MAX;   // every int32 slot >= -1 is then in range
    uint32_t bad = 0;
    for (int64_t r = 0; r < rows; ++r)
        bad |= static_cast<uint32_t>(row_slot[r] < -1) | (static_cast<uint32_t>(row_slot[r] >= ns) & ~wide);
    if (bad) {
        for (int64_t r = 0; r < rows; ++r)
            if (row_slot[r] < -1 || int64_t(row_slot[r]) >= n_slots) return r;
    }
    return -1;
}

// Rows that hold a slot (row_slot >= 0), ascending, 16 rows at a time
// (usually few: only last step's active rows hold one): fn(r) for each.
template <typename Fn>
void for_held_rows(const int32_t *row_slot, int64_t rows, Fn &&fn) {
    int64_t r = 0;
    for (; r + 16 <= rows; r += 16) {
        const __m128i *p = reinterpret_cast<const __m128i *>(row_slot + r);
        const int neg = _mm_movemask_ps(_mm_castsi128_ps(_mm_loadu_si128(p))) |
                        (_mm_movemask_ps(_mm_castsi128_ps(_mm_loadu_si128(p + 1))) << 4) |
                        (_mm_movemask_ps(_mm_castsi128_ps(_mm_loadu_si128(p + 2))) << 8) |
                        (_mm_movemask_ps(_mm_castsi128_ps(_mm_loadu_si128(p + 3))) << 12);
        for (int held = ~neg & 0xffff; held; held &= held - 1) fn(r + __builtin_ctz(held));
    }
    for (; r < rows; ++r)
        if (row_slot[r] >= 0) fn(r);
}

// Slots of the active rows once the rows that left the set have released
// theirs: survivors keep their slot, newcomers take the lowest free slots in
// the list's (ascending row) order and are flagged fresh.  `taken` becomes a
// bit set of n_slots bits.
void assign_slots(int32_t *row_slot, int64_t n_slots, const int32_t *active_rows, int64_t n_active, int32_t *slot,
                  uint8_t *fresh, std::vector<uint64_t> &taken) {
    taken.assign(static_cast<size_t>((n_slots + 63) / 64), 0);
    for (int64_t i = 0; i < n_active; ++i) {
        const int32_t s = row_slot[active_rows[i]];
        if (s >= 0) taken[s >> 6] |= uint64_t(1) << (s & 63);
    }
    size_t word = 0;
    for (int64_t i = 0; i < n_active; ++i) {
        const int32_t r = active_rows[i];
        if (row_slot[r] >= 0) {
            slot[i] = row_slot[r];
            fresh[i] = 0;
            continue;
        }
        while (taken[word] == ~uint64_t(0)) ++word;   // lowest free slot (ascending scan)
        const int b = __builtin_ctzll(~taken[word]);
        taken[word] |= uint64_t(1) << b;
        const int32_t s = static_cast<int32_t>(64 * word + b);
        row_slot[r] = s;
        slot[i] = s;
        fresh[i] = 1;
    }
}

// The slots given the row mask (nonzero = active) and its active rows.
void slots_core(int32_t *__restrict__ row_slot, int64_t rows, int64_t n_slots, const uint8_t *__restrict__ active,
                const int32_t *active_rows, int64_t n_active, int32_t *slot, uint8_t *fresh,
                std::vector<uint64_t> &taken) {
    for_held_rows(row_slot, rows, [&](int64_t r) {
        if (!active[r]) row_slot[r] = -1;
    });
    assign_slots(row_slot, n_slots, active_rows, n_active, slot, fresh, taken);
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
    static thread_local std::vector<float> hits_tls;
    std::vector<float> &hits = hits_tls;
    hits.assign(static_cast<size_t>(rows), 0.0f);
    for (int64_t i = 0; i < n_tokens; ++i) {
        const int32_t tok = tokens[i];
        SFT_CHECK(tok >= 0 && tok < rows, SFT_EINVAL, "conductor: token %d at %lld out of [0, %lld)",
                  tok, (long long)i, (long long)rows);
    }
    // counts are exact in fp32 (at most 2^24), so the running maximum of the
    // incremented counts is the window's busiest row
    float *const h = hits.data();
    float busiest = 0.0f;
    for (int64_t i = 0; i < n_tokens; ++i) {
        const float c = h[tokens[i]] + 1.0f;
        h[tokens[i]] = c;
        busiest = std::max(busiest, c);
    }
    charge_update(ch, rows, h, busiest, active);
    return SFT_OK;
}

int sft_tracker_window(float *ch, int64_t rows, const float *magnitude, uint8_t *active) {
    clear_error();
    SFT_CHECK(rows >= 0, SFT_EINVAL, "tracker: negative size");
    SFT_CHECK(rows == 0 || (ch && magnitude && active), SFT_EINVAL, "tracker: null array");
    float wmax = 0.0f;
    const int64_t bad = magnitude_max(magnitude, rows, &wmax);
    SFT_CHECK(bad < 0, SFT_EINVAL, "tracker: magnitude[%lld] is negative or not finite", (long long)bad);
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
    plan_core(active, rows, plan->tile_bits, plan->active_rows, plan->active_tiles, plan->active_bits,
              plan->tile_first, &plan->n_active, &plan->n_active_tiles);
    return SFT_OK;
}

int64_t sft_plan_layer_words(const sft_layer_mat *mats, int32_t n_mats) {
    if (n_mats < 0 || (n_mats > 0 && !mats)) return -1;
    int64_t words = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const int64_t R = mats[i].rows;
        if (R < 0 || R >= (int64_t(1) << 31)) return -1;
        const int64_t tiles = (R + 31) / 32;
        words += 2 * R + (R + 3) / 4 + 3 * tiles + 6 * 3;   // six sections, each padded to 4 words
    }
    return words;
}

int sft_plan_layer(sft_layer_mat *mats, int32_t n_mats, int32_t *packed, int64_t packed_cap,
                   int64_t *packed_len) {
    clear_error();
    SFT_CHECK(n_mats >= 0 && (n_mats == 0 || mats) && packed_len, SFT_EINVAL, "plan_layer: null argument");
    const int64_t need = sft_plan_layer_words(mats, n_mats);
    SFT_CHECK(need >= 0, SFT_EINVAL, "plan_layer: rows out of range");
    SFT_CHECK(packed_cap >= need, SFT_ECAPACITY, "plan_layer: packed holds %lld words, %lld needed",
              (long long)packed_cap, (long long)need);
    SFT_CHECK(need == 0 || (packed && sft::aligned16(packed)), packed ? SFT_EALIGN : SFT_EINVAL,
              "plan_layer: packed null or not 16-byte aligned");
    // Everything is checked, and every mask formed, before any state changes:
    // the new charges go straight to the caller's arrays only when no matrix
    // can have more active rows than slots; otherwise they are staged.
    static thread_local std::vector<float> next_tls;
    static thread_local std::vector<uint8_t> act_tls;
    static thread_local std::vector<uint64_t> taken_tls;
    std::vector<float> &next = next_tls;
    std::vector<uint8_t> &act_v = act_tls;
    std::vector<uint64_t> &taken = taken_tls;
    int64_t total = 0;
    bool direct = true;
    for (int32_t i = 0; i < n_mats; ++i) {
        total += mats[i].rows;
        direct = direct && mats[i].n_slots >= mats[i].rows;
    }
    act_v.resize(static_cast<size_t>(total) + 32);
    uint8_t *const act = act_v.data();
    if (!direct) next.resize(static_cast<size_t>(total));
    float *const nxt = next.data();
    float wmax[64];
    float *wm = wmax;
    std::vector<float> wmax_many;
    if (n_mats > 64) {
        wmax_many.resize(static_cast<size_t>(n_mats));
        wm = wmax_many.data();
    }
    for (int32_t i = 0; i < n_mats; ++i) {
        const sft_layer_mat &m = mats[i];
        const int64_t R = m.rows;
        SFT_CHECK(m.n_slots >= 0 && m.n_slots < (int64_t(1) << 31), SFT_EINVAL, "plan_layer: matrix %d: bad n_slots", i);
        SFT_CHECK(R == 0 || (m.charge && m.magnitude && m.row_slot), SFT_EINVAL, "plan_layer: matrix %d: null array", i);
        const int64_t bad = magnitude_max(m.magnitude, R, &wm[i]);
        SFT_CHECK(bad < 0, SFT_EINVAL, "plan_layer: matrix %d: magnitude[%lld] is negative or not finite", i,
                  (long long)bad);
        const int64_t bs = row_slot_bad(m.row_slot, R, m.n_slots);
        SFT_CHECK(bs < 0, SFT_EINVAL, "plan_layer: matrix %d: row_slot[%lld] out of range", i, (long long)bs);
    }
    int64_t base = 0;
    if (!direct) {
        for (int32_t i = 0; i < n_mats; ++i) {
            const sft_layer_mat &m = mats[i];
            const int64_t R = m.rows;
            std::memcpy(nxt + base, m.charge, static_cast<size_t>(R) * 4);
            const int64_t na = charge_update(nxt + base, R, m.magnitude, wm[i], act + base);
            SFT_CHECK(na <= m.n_slots, SFT_ECAPACITY, "plan_layer: matrix %d: %lld active rows exceed %lld slots", i,
                      (long long)na, (long long)m.n_slots);
            base += R;
        }
    }
    int64_t off = 0;
    base = 0;
    auto section = [&](int64_t words) {
        const int64_t at = off;
        off += (words + 3) & ~int64_t(3);
        return at;
    };
    for (int32_t i = 0; i < n_mats; ++i) {
        sft_layer_mat &m = mats[i];
        const int64_t R = m.rows, tiles = (R + 31) / 32;
        if (direct) charge_update(m.charge, R, m.magnitude, wm[i], act + base);
        else std::memcpy(m.charge, nxt + base, static_cast<size_t>(R) * 4);
        const uint8_t *a = act + base;
        // sections: rows | tiles | bits | first, sized by the counts below
        int32_t *rows_out = packed + off;
        int64_t na = 0, nt = 0;
        // rows go first at `off`; tiles, bits and first after the rows' padded
        // length, which is known once the plan is built: plan into a staging
        // area at the end of the matrix's worst-case space, then move.
        int32_t *tiles_tmp = packed + off + ((R + 3) & ~int64_t(3));
        int32_t *bits_tmp = tiles_tmp + ((tiles + 3) & ~int64_t(3));
        int32_t *first_tmp = bits_tmp + ((tiles + 3) & ~int64_t(3));
        plan_core(a, R, nullptr, rows_out, tiles_tmp, reinterpret_cast<uint32_t *>(bits_tmp), first_tmp, &na, &nt);
        m.n_active = na;
        m.n_active_tiles = nt;
        m.off_rows = section(na);
        m.off_tiles = section(nt);
        std::memmove(packed + m.off_tiles, tiles_tmp, static_cast<size_t>(nt) * 4);
        m.off_bits = section(nt);
        std::memmove(packed + m.off_bits, bits_tmp, static_cast<size_t>(nt) * 4);
        m.off_first = section(nt);
        std::memmove(packed + m.off_first, first_tmp, static_cast<size_t>(nt) * 4);
        m.off_slot = section(na);
        m.off_fresh = section((na + 3) / 4);
        int32_t *slot = packed + m.off_slot;
        uint8_t *fresh = reinterpret_cast<uint8_t *>(packed + m.off_fresh);
        slots_core(m.row_slot, R, m.n_slots, a, packed + m.off_rows, na, slot, fresh, taken);
        for (int64_t k = na; k < 4 * ((na + 3) / 4); ++k) fresh[k] = 0;
        base += R;
    }
    *packed_len = off;
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
    static thread_local std::vector<int32_t> index_tls;
    static thread_local std::vector<int64_t> count_tls, fill_tls;
    std::vector<int32_t> &index = index_tls;
    std::vector<int64_t> &count = count_tls;
    index.assign(static_cast<size_t>(rows), -1);
    for (int64_t k = 0; k < na; ++k) index[plan->active_rows[k]] = static_cast<int32_t>(k);
    count.assign(static_cast<size_t>(na) + 1, 0);
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
    std::vector<int64_t> &fill = fill_tls;
    fill.assign(count.begin(), count.end() - 1);
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
    const int64_t bs = row_slot_bad(row_slot, rows, n_slots);
    SFT_CHECK(bs < 0, SFT_EINVAL, "slots: row_slot[%lld] = %d out of range", (long long)bs,
              bs < 0 ? 0 : row_slot[bs]);
    // Rows holding a slot that are not in the (ascending) list release it:
    // the held rows and the list are walked together.
    int64_t k = 0;
    for_held_rows(row_slot, rows, [&](int64_t r) {
        while (k < n_active && active_rows[k] < r) ++k;
        if (!(k < n_active && active_rows[k] == r)) row_slot[r] = -1;
    });
    static thread_local std::vector<uint64_t> taken_tls;
    assign_slots(row_slot, n_slots, active_rows, n_active, slot, fresh, taken_tls);
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