/*
 * sft.h -- C ABI of the sparse-first fine-tuning hot path for AMD MI355X (gfx950).
 *
 * The method is the one described on the page "Sparse-First Fine-Tuning:
 * Full-Weight Training at the Cost of the Active Set" (tensorwirelabs.com).
 * One training step of a weight matrix W [R x C] (rows = output features):
 *
 *   1. masks, once per step, on the host (section 2.1): the conductor for the
 *      embedding, a row tracker for every projection;            -> sft_conductor_window,
 *                                                                     sft_tracker_window,
 *                                                                     sft_plan_rows,
 *                                                                     sft_plan_embedding,
 *                                                                     sft_slots_update,
 *                                                                     sft_plan_layer (all
 *                                                                     three, per layer)
 *   2. the masked weight gradient dW = dY^T X, skipping 32-row tiles with no
 *      active row (section 2.2);                                  -> sft_masked_dw,
 *                                                                     sft_embedding_dw
 *   3. the sparse update of the int8 weight q, per-row scale s and fp32
 *      residual delta with fp16 Adam moments kept only for active rows
 *      (sections 2.3 and 2.4; pairs of matrices take the coupled update);
 *                                                                  -> sft_sparse_update,
 *                                                                     sft_coupled_update
 *   4. the sparse write-back of the live bf16 weights (section 2.3).
 *                                                                  -> sft_masked_writeback,
 *                                                                     sft_masked_writeback_many
 *                                                                     (or fused into 3)
 *   The mixing coefficients of the coupled update come from a host schedule
 *   (sections 2.4, 2.5):                                         -> sft_helix_init,
 *                                                                     sft_helix_step,
 *                                                                     sft_helix_coupling
 *   5. checkpoint and rewind (section 2.6): a host controller decides from
 *      the loss when to save the active rows and when to restore them;
 *                                                                  -> sft_rewind_init,
 *                                                                     sft_rewind_observe,
 *                                                                     sft_rows_save,
 *                                                                     sft_rows_restore
 *   Measurement probes (sustained bandwidth and matrix-core rate) are
 *   declared apart, in sft_probe.h.
 *   The element-sparse variant of the blog post "SparseLeaf: synaptic sparse
 *   fine-tuning" (K selected connections of a frozen weight train their own
 *   increments): their gradients and their Adam step.
 *                                                                  -> sft_leaf_grad,
 *                                                                     sft_leaf_grad_workspace,
 *                                                                     sft_leaf_adam
 *
 * Conventions shared by every call:
 *   - Status: every entry point returns SFT_OK (0) or a negative SFT_E* code,
 *     never throws and never aborts.  The message of the last failure on the
 *     calling thread is returned by sft_last_error().
 *   - Ownership: the caller owns every buffer.  The library keeps no pointer
 *     after a call returns and allocates no device memory.
 *   - Host calls (section "host") run synchronously on plain host arrays.
 *   - Device calls (section "device") take device pointers, validate host-side
 *     scalars and pointer alignment, enqueue their kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and return
 *     without synchronising.  They never copy anything back to the host
 *     (section 2.6 of the page: no readback happens while a step runs),
 *     so a fault inside a kernel surfaces at the caller's next synchronisation.
 *     Inputs must stay alive until the stream work completes.
 *   - Layouts: row-major and contiguous.  bf16 and fp16 values are passed as
 *     their 16-bit patterns (uint16_t).  Device base pointers must be 16-byte
 *     aligned and C must be a multiple of 8 (16-byte vector access).
 *   - Row lists (active_rows) are strictly ascending and < R.  Row k of a
 *     compact gradient (dW_act, G) belongs to active_rows[k].
 *   - Counts (n_active, n_active_tiles, nnz) are host scalars taken from the
 *     host plan; the GPU never reports a count back.
 *   - Thread safety: every call is re-entrant; the only per-thread state is
 *     the last-error message.
 */
#ifndef SFT_H
#define SFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFT_ABI_VERSION 14

enum {
    SFT_OK = 0,
    SFT_EINVAL = -1,    /* null pointer, negative size, bad value, unsorted row list */
    SFT_ESHAPE = -2,    /* inconsistent shapes (e.g. C not a multiple of 8)           */
    SFT_EALIGN = -3,    /* a device pointer is not 16-byte aligned                     */
    SFT_ECAPACITY = -4, /* an output or slot table is too small, or workspace too small */
    SFT_EHIP = -5,      /* the HIP runtime reported an error at launch                 */
    SFT_ENOTSUP = -6    /* a size beyond what the kernels support                     */
};

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char *sft_last_error(void);

/* SFT_ABI_VERSION of the built library. */
int sft_abi_version(void);

/* ======================================================================= */
/* host: masks and plans (CPU, synchronous, plain host arrays)              */
/* ======================================================================= */

/*
 * The conductor (section 2.1): one observation window over `rows` embedding
 * rows.  For every row, hits_r = number of tokens equal to r; with H the
 * largest hit count, the row's charge becomes ch_r/2 + (hits_r/H)/2 (fp32;
 * an empty window only halves the charges) and active[r] = (ch_r >= 0.01).
 *   ch       [rows] fp32, in/out: charges (start at 0)
 *   tokens   [n_tokens] token ids, each in [0, rows)
 *   active   [rows] out: 1 = active, 0 = inactive
 * Errors: SFT_EINVAL for a null pointer, rows < 0, n_tokens < 0 or a token
 * out of range (checked before anything is written).
 */
int sft_conductor_window(float *ch, int64_t rows, const int32_t *tokens, int64_t n_tokens,
                         uint8_t *active);

/*
 * The row tracker (section 2.1): the same recurrence as the conductor with the
 * rows' output magnitudes from the forward pass in place of hit counts.
 *   magnitude [rows] fp32, each >= 0 and finite
 * Errors: SFT_EINVAL for a null pointer, rows < 0, or a negative/NaN magnitude.
 */
int sft_tracker_window(float *ch, int64_t rows, const float *magnitude, uint8_t *active);

/*
 * Row plan of one mask (section 2.2: the mask is tested 32 rows at a time).
 * Caller-allocated arrays; the call fills the counts.
 *   tile_bits    [ceil(rows/32)]  bit i of word j = mask of row 32*j+i (bits >= rows are 0)
 *   active_rows  [rows]           ascending active rows (first n_active valid)
 *   active_tiles [ceil(rows/32)]  ascending tiles with an active row (first n_active_tiles valid)
 *   active_bits  [ceil(rows/32)]  tile_bits of each active tile (first n_active_tiles valid)
 *   tile_first   [ceil(rows/32)]  index in active_rows of each active tile's first active row
 */
typedef struct sft_plan {
    int64_t rows;           /* in  */
    int64_t n_active;       /* out */
    int64_t n_active_tiles; /* out */
    uint32_t *tile_bits;
    int32_t *active_rows;
    int32_t *active_tiles;
    uint32_t *active_bits;
    int32_t *tile_first;
} sft_plan;

/* Errors: SFT_EINVAL for null pointers or rows < 0 or rows >= 2^31.
 * active_bits and tile_first may be NULL (not filled). */
int sft_plan_rows(const uint8_t *active, sft_plan *plan);

/*
 * The embedding's masked backward pass needs, per active row, the token
 * positions that looked it up (section 2.2: the embedding's input is one-hot,
 * so a row's gradient sums dY over its token's positions; section 2.1: the
 * conductor's mask chooses the rows).
 * Token positions of the active embedding rows, as CSR: the positions t with
 * tokens[t] == plan->active_rows[k] are positions[row_ptr[k] .. row_ptr[k+1]),
 * ascending.  row_ptr has n_active + 1 entries; positions has capacity
 * `positions_cap` (n_tokens always suffices); *nnz receives the total.
 * Errors: SFT_EINVAL (null / token out of range), SFT_ECAPACITY (positions_cap).
 */
int sft_plan_embedding(const sft_plan *plan, const int32_t *tokens, int64_t n_tokens,
                       int32_t *row_ptr, int32_t *positions, int64_t positions_cap,
                       int64_t *nnz);

/*
 * Moment slots (section 2.3: m and v exist only for active rows).  row_slot
 * [rows] is the persistent map row -> slot (-1 = none; start all -1).  Rows no
 * longer active free their slot; rows still active keep theirs; a newly active
 * row takes the lowest free slot and is flagged fresh (its moments and step
 * count start from zero; the update kernels then ignore the stored values).
 *   slot  [n_active] out, fresh [n_active] out (1 = fresh)
 * Errors: SFT_EINVAL (null, unsorted rows), SFT_ECAPACITY (n_active > n_slots;
 * checked before anything is written).
 */
int sft_slots_update(int32_t *row_slot, int64_t rows, int64_t n_slots,
                     const int32_t *active_rows, int64_t n_active, int32_t *slot,
                     uint8_t *fresh);

/*
 * One step's host plan of the matrices of a layer in one call: section 2.1
 * (the CPU derives every mask once per step, a step ahead of the GPU, and
 * ships them in one transfer), section 2.2 (32-row tiles) and section 2.3
 * (moment slots of the active rows).  For each matrix, in order: the row
 * tracker's window over the matrix's output magnitudes (exactly
 * sft_tracker_window), the row plan of the resulting mask (exactly
 * sft_plan_rows) and its moment slots (exactly sft_slots_update).  The
 * results go one after another into `packed`, host int32 words meant for a
 * single copy to the device; each matrix's sections start on a 16-byte
 * boundary of `packed`, at the word offsets returned in its entry:
 *   off_rows   active rows [n_active]
 *   off_tiles  active tiles [n_active_tiles]
 *   off_bits   their row bits [n_active_tiles] (uint32)
 *   off_first  index of each active tile's first active row [n_active_tiles]
 *   off_slot   moment slot of each active row [n_active]
 *   off_fresh  fresh flags, one byte per active row (uint8, zero-padded to
 *              whole words)
 * packed must be 16-byte aligned and hold sft_plan_layer_words(mats)
 * words; *packed_len receives the words used.  Every input is checked and
 * every mask formed before any state changes: on an error no charge, row
 * slot or packed word has been written.
 * Errors: SFT_EINVAL (null arrays, bad sizes, a negative or non-finite
 * magnitude, a row_slot entry outside [-1, n_slots)), SFT_EALIGN,
 * SFT_ECAPACITY (packed too small, or more active rows than slots).
 */
typedef struct sft_layer_mat {
    int64_t rows;              /* in: R, below 2^31                          */
    int64_t n_slots;           /* in: moment slots of the matrix             */
    float *charge;             /* in/out [rows]: the row tracker's charge    */
    const float *magnitude;    /* in [rows]: this window's output magnitudes */
    int32_t *row_slot;         /* in/out [rows]: row -> slot (-1 = none)     */
    int64_t n_active;          /* out */
    int64_t n_active_tiles;    /* out */
    int64_t off_rows, off_tiles, off_bits, off_first, off_slot, off_fresh;   /* out, in words */
} sft_layer_mat;

/* Words of `packed` that sft_plan_layer needs for these matrices (only
 * `rows` is read), or -1 for a bad argument. */
int64_t sft_plan_layer_words(const sft_layer_mat *mats, int32_t n_mats);

int sft_plan_layer(sft_layer_mat *mats, int32_t n_mats, int32_t *packed, int64_t packed_cap,
                   int64_t *packed_len);

/*
 * Section 2.6 and Figure 2 (the step's masks go to the GPU once per step):
 * copies `bytes` bytes of a plan in pinned host memory (`src`, allocated by
 * hipHostMalloc or an allocator built on it, such as torch's pin_memory) to
 * device memory `dst`, by a kernel on `stream` that reads the host buffer
 * over the bus.  Asynchronous like a copy on the stream: src must stay
 * unchanged until the stream has passed the call.  bytes is a multiple of 4
 * (plans are int32 words); dst and src are 16-byte aligned.
 * Errors: SFT_EINVAL (null, or src not pinned host memory), SFT_ESHAPE
 * (bytes % 4), SFT_EALIGN, SFT_ENOTSUP (bytes >= 2^31), SFT_EHIP.
 */
int sft_plan_upload(void *dst, const void *src, size_t bytes, void *stream);

/*
 * Adam bias corrections (section 2.4: Adam with its bias correction):
 * bc1[t] = fl32(1 - beta1^t), bc2[t] = fl32(1 - beta2^t) for
 * t = 1..t_max, computed in fp64 and rounded once; bc1[0] = bc2[0] = 0.
 * The arrays hold t_max + 1 floats.  The update kernels read entry
 * min(t, t_max); choose t_max so that the entries have reached 1.0f (about
 * 17,000 for beta2 = 0.999) or the step count never exceeds it.
 * Errors: SFT_EINVAL (null, t_max < 1, beta outside [0, 1)).
 */
int sft_bias_table(float beta1, float beta2, int32_t t_max, float *bc1, float *bc2);

/*
 * Checkpoint-and-rewind controller (section 2.6; section 4.2 reports its one
 * rewind: at step 356 the loss had rebounded past the threshold and the
 * checkpoint of step 336 came back).  Two row copies are kept: the checkpoint
 * (what a restore brings back) and the copy of the lowest loss so far (the
 * minimum), which becomes the checkpoint once the minimum is accepted.  Each
 * new minimum is watched for 10 steps; a loss more than 15% above it when the
 * watch ends brings the checkpoint back, restarts the phase stride at 1 and
 * drops the step (up to 3 times for one minimum); otherwise the minimum is
 * accepted and becomes the checkpoint.  Outside a watch the checkpoint is
 * refreshed while the loss stays within 10% of the checkpoint's loss.
 * Readings of the prose, exactly as implemented (loss = the loss the rows
 * held by the caller produced, a double; comparisons in double; the step
 * counter k counts observations from 0):
 *   - the end of a watch comes first: each step decrements watch_left; the
 *     step that brings it to 0 ends the watch: if loss > (1 + rise_above) *
 *     min_loss and recoveries < max_recoveries, the action is
 *     SFT_REWIND_RESTORE alone, recoveries grows by one and the watch
 *     re-opens on the same minimum (the step is dropped: nothing else
 *     happens on it); otherwise the minimum is accepted (SFT_REWIND_PROMOTE:
 *     checkpoint_loss = min_loss, checkpoint_step = min_step);
 *   - then a new minimum, a loss below every loss seen so far: if a watch is
 *     still open its minimum is accepted first (SFT_REWIND_PROMOTE: the loss
 *     fell below it, so it did not rise); then min_loss = loss, min_step = k,
 *     watch_left = watch_steps, recoveries = 0, action SFT_REWIND_SAVE_MIN;
 *   - then the refresh, SFT_REWIND_SAVE (checkpoint_loss = loss,
 *     checkpoint_step = k): when there is no checkpoint yet, or when no watch
 *     is open, loss <= (1 + save_within) * checkpoint_loss and
 *     loss <= (1 + rise_above) * min_loss;
 *   - a NaN or infinite loss counts as +infinity: never a minimum, never
 *     copied, always a rise.
 * The caller keeps two copy buffers (sft_ckpt_mat) and applies a step's
 * bits before the step's update, in this order: SFT_REWIND_PROMOTE (the
 * minimum's buffer, with its row list, becomes the checkpoint's and the old
 * checkpoint buffer becomes the minimum's: no copy is made),
 * SFT_REWIND_SAVE_MIN (sft_rows_save of the active rows into the minimum's
 * buffer), SFT_REWIND_SAVE (sft_rows_save into the checkpoint's buffer).  On
 * SFT_REWIND_RESTORE it calls sft_rows_restore with the checkpoint's buffer,
 * resets its phase stride to 1 and does not apply the step's update.
 * sft_rewind_init sets the page's values (0.10, 0.15, 10 steps, 3 recoveries)
 * and an empty state; the settings may be changed before the first
 * observation.
 */
enum {
    SFT_REWIND_SAVE = 1,      /* copy the rows into the checkpoint              */
    SFT_REWIND_RESTORE = 2,   /* bring the checkpoint back, drop the step       */
    SFT_REWIND_SAVE_MIN = 4,  /* copy the rows into the minimum's copy          */
    SFT_REWIND_PROMOTE = 8    /* the minimum's copy becomes the checkpoint      */
};

typedef struct sft_rewind {
    double save_within;       /* 0.10 */
    double rise_above;        /* 0.15 */
    int32_t watch_steps;      /* 10 */
    int32_t max_recoveries;   /* 3 */
    /* state */
    int32_t has_checkpoint;
    int32_t watch_left;       /* 0 = no watch open */
    int32_t recoveries;       /* restores since the current minimum */
    int32_t reserved;
    double checkpoint_loss;   /* loss of the rows the checkpoint holds */
    double min_loss;          /* +inf before the first finite loss */
    int64_t step;             /* observations so far */
    int64_t checkpoint_step;  /* step whose rows the checkpoint holds (-1: none) */
    int64_t min_step;         /* step whose rows the minimum's copy holds (-1: none) */
} sft_rewind;

/* Errors: SFT_EINVAL (null). */
int sft_rewind_init(sft_rewind *st);

/*
 * Feeds one step's loss; *action = an OR of the SFT_REWIND_* bits (0 = none).
 * Errors: SFT_EINVAL (null pointers, save_within or rise_above negative or
 * NaN, watch_steps < 1, max_recoveries < 0); the state is then unchanged.
 */
int sft_rewind_observe(sft_rewind *st, double loss, int32_t *action);

/*
 * The coupled update's scalar schedule (sections 2.4, 2.5, 2.6, 2.8), host
 * side: a loss trend, a Fibonacci stride, the phase it advances, and the
 * mixing coefficients a_own / a_cross that sft_coupled_update takes.  The
 * page's equations are lost; the readings implemented are:
 *   - trend = sum_i r^i dL(t-i) / sum_i r^i over the steps seen, r =
 *     exp(-1/decay_len), dL(t) = L(t-1) - L(t) (none for the first loss);
 *     smooth = the same mean over the series of trends;
 *   - each step the rung (0..7 on 1, 1, 2, 3, 5, 8, 13, 21) goes up by one if
 *     smooth > up_threshold, down by one if smooth < 0, else stays; a rewind
 *     sets it to 0 instead; stride = the rung's Fibonacci number;
 *   - rotation += rung_deg * stride (degrees); phase = fmod(rotation, 360);
 *   - channel weights w+ = 1 + mod_plus cos(2 pi rotation / 360) and
 *     w- = 1 + mod_minus cos(2 pi rotation / 3600);
 *   - exposure e = (1 + cos(phase + psi)) / 2 (psi, the slow phase term, is
 *     the caller's: the page's elliptic-curve walk is not specified),
 *     a_own = 1, a_cross = b mu w- (1 - e) / (M w+ e + mu w- (1 - e));
 *   - double precision throughout.
 * sft_helix_init sets decay_len 10, up_threshold 1e-4 (loss units), rung_deg
 * 36, M 1.833, mu 1, mod_plus 0.10, mod_minus 0.05 and an empty state.
 */
typedef struct sft_helix {
    double decay_len, up_threshold, rung_deg, M, mu, mod_plus, mod_minus;
    /* state */
    double trend_sum, trend_w, smooth_sum, smooth_w, last_loss, rotation;
    int32_t has_loss, rung;
} sft_helix;

/* Errors: SFT_EINVAL (null). */
int sft_helix_init(sft_helix *h);

/* One step with the loss the caller has (rewind != 0: the step was dropped by
 * a restore); *stride and *phase_deg (either may be NULL) receive the new
 * values.  Errors: SFT_EINVAL (null state, non-finite loss, decay_len <= 0). */
int sft_helix_step(sft_helix *h, double loss, int32_t rewind, int32_t *stride, double *phase_deg);

/* The pair coefficients at the current phase for coupling strength b (0.6
 * gate-up, 0.4 attention pairs on the page).  Errors: SFT_EINVAL (null
 * pointers, b or psi not finite, M, mu or a channel weight not positive). */
int sft_helix_coupling(const sft_helix *h, double b, double psi_deg, double *a_own, double *a_cross);

/* ======================================================================= */
/* device: the masked backward pass (section 2.2)                           */
/* ======================================================================= */

/*
 * One matrix of a masked-dW group.  dY is bf16 [T x R] (gradient at the
 * matrix's output); the plan arrays are device copies of an sft_plan of this
 * matrix's mask; dW_act is fp32 [n_active x C], row k = the k-th active row.
 * active_rows is read by the packed layout only, the tile arrays by the tile
 * layout only (the other pointers may be NULL).
 */
typedef struct sft_dw_mat {
    const uint16_t *dY;
    int64_t R;
    const int32_t *active_rows;  /* device [n_active] */
    const int32_t *active_tiles; /* device [n_active_tiles] */
    const uint32_t *active_bits; /* device [n_active_tiles] */
    const int32_t *tile_first;   /* device [n_active_tiles] */
    int64_t n_active;            /* host scalar */
    int64_t n_active_tiles;      /* host scalar */
    float *dW_act;               /* device [n_active x C] */
} sft_dw_mat;

/*
 * How a group's rows are laid out on the matrix cores (the result is the
 * same, bit for bit, for integer-exact inputs and within fp32 summation order
 * otherwise):
 *   SFT_DW_TILES   every active 32-row tile is multiplied whole and its
 *                  inactive rows are dropped at the store (section 2.2 as
 *                  the page states it);
 *   SFT_DW_PACKED  the active rows of the group are packed 32 to a tile
 *                  before the product, so a tile with one active row costs
 *                  1/32 of a whole tile.  Inactive tiles are skipped in both.
 */
enum { SFT_DW_TILES = 0, SFT_DW_PACKED = 1 };

/* Matrices that read the same layer input X (bf16 [T x C]), e.g. q/k/v. */
typedef struct sft_dw_group {
    const uint16_t *X;
    int64_t T, C;
    int32_t n_mats;
    int32_t layout;         /* SFT_DW_TILES or SFT_DW_PACKED */
    const sft_dw_mat *mats; /* host array of n_mats */
} sft_dw_group;

/*
 * Section 2.2 (only active 32-row tiles reach the matrix cores, so the
 * scratch scales with the active rows, never with R).
 * Workspace bytes sft_masked_dw needs for these groups: the gathered dY
 * columns of the active rows (the matrix-core operand, token-contiguous),
 * their output map, and the split-K partial rows when the token axis is
 * split to fill the GPU.
 * Returns (size_t)-1 and sets the error message on invalid groups.
 */
size_t sft_masked_dw_workspace(const sft_dw_group *groups, int32_t n_groups);

/*
 * dW_act[k, c] = sum_t dY[t, r_k] * X[t, c] for every active row r_k of every
 * matrix (bf16 inputs, fp32 accumulation on the matrix cores, fp32 output).
 * Each 32-row tile with no active row is skipped before any load of dY or X;
 * inside an active tile only the active rows are written (section 2.2).
 * Matrices of one group share every load of X.
 *   ws / ws_bytes  device scratch of at least sft_masked_dw_workspace()
 *                  bytes (16-byte aligned; no initialisation needed).  Calls
 *                  that share a workspace must be ordered on one stream.
 * Limits: 1 <= T <= 2^24, C % 8 == 0, C <= 2^24, T * C < 2^31, R < 2^31,
 * n_active < 2^24, at most 16 matrices per group, fewer than 2^31 (output
 * tile, 64-token chunk) iterations per launch of 8 groups.  Results are deterministic
 * (a fixed summation order for every launch configuration the same inputs
 * produce).
 * Errors: SFT_EINVAL, SFT_ESHAPE, SFT_EALIGN, SFT_ECAPACITY (ws too small),
 * SFT_ENOTSUP (beyond the limits above), SFT_EHIP.
 */
int sft_masked_dw(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * The embedding's masked weight gradient (section 2.2: the same product with
 * a one-hot input): dW_act[k, c] = sum over positions t of row k of dY[t, c],
 * with the CSR from sft_plan_embedding (device copies).  Summed in fp64 and
 * rounded to fp32 once.
 *   dY [T x d] bf16, row_ptr [n_active+1], positions [nnz], dW_act [n_active x d] fp32
 * Limits: d % 8 == 0.  Errors: SFT_EINVAL, SFT_ESHAPE, SFT_EALIGN, SFT_EHIP.
 */
int sft_embedding_dw(const uint16_t *dY, int64_t T, int64_t d, const int32_t *row_ptr,
                     const int32_t *positions, int64_t n_active, float *dW_act, void *stream);

/* ======================================================================= */
/* device: the sparse update and write-back (sections 2.3 and 2.4)          */
/* ======================================================================= */

/* Adam hyper-parameters; bc1/bc2 are device copies of sft_bias_table(). */
typedef struct sft_adam {
    float lr, beta1, beta2, eps;
    float weight_decay; /* decoupled (AdamW order: decay, then step); 0 = none */
    const float *bc1;   /* device [t_max + 1] */
    const float *bc2;   /* device [t_max + 1] */
    int32_t t_max;
} sft_adam;

/*
 * One matrix's optimizer state and the gradient of its active rows.
 *   q      int8 [R x C], s fp32 [R], delta fp32 [R x C]: w = s*q + delta
 *   m, v   fp16 [n_slots x C], t int32 [n_slots]: moments and step count per slot
 *   mv_exp int8 [n_slots x 2]: the exponents of each slot's m row and v row.
 *          The fp16 moments (section 2.3) are stored scaled: the value h of
 *          a row with exponent e stands for h * 2^-e.  Every update picks e
 *          from the new row's largest magnitude so that it lands in
 *          [2^14, 2^15) (e = 15 - k for a maximum in [2^(k-1), 2^k), limited
 *          to [-112, 125]; 0 for an all-zero row), rounds to nearest even and
 *          saturates at 65504, so that small and large gradients alike keep
 *          fp16's 11 significant bits instead of flushing to zero or
 *          overflowing.  A fresh slot ignores the stored values.
 *   G      fp32 [n_active x C] (row k = active_rows[k]), e.g. dW_act
 *   slot   [n_active] slot of each active row; fresh [n_active] or NULL
 *   w_live bf16 [R x C] live weights, or NULL for no fused write-back
 */
typedef struct sft_upd_mat {
    int64_t R, C, n_active, n_slots;
    const int32_t *active_rows;
    const int32_t *slot;
    const uint8_t *fresh;
    const float *G;
    int8_t *q;
    float *s;
    float *delta;
    uint16_t *m;
    uint16_t *v;
    int32_t *t;
    int8_t *mv_exp;
    uint16_t *w_live;
} sft_upd_mat;

/*
 * Plain sparse update of every active row of n_mats matrices, in one launch
 * (section 2.3; section 2.4's plain Adam step for unpaired matrices).  Per
 * active row: rebuild w = fl(fl(s*q) + delta) in registers, take the Adam step
 * (fp32 moments decoded from the stored scaled fp16 rows, new moments stored
 * as scaled fp16 rows with new exponents; the step lr*mhat/(sqrt(vhat)+eps)
 * with the bias corrections bc1, bc2 from the table applied as the per-row
 * factors k1 = lr/bc1 and k2 = 1/sqrt(bc2): u = (k1*m)/(sqrt(v)*k2 + eps);
 * decoupled weight decay first, w*(1 - lr*weight_decay)), then requantise
 * the row: s' = max|w'|/127, q' = clamp(rint(w' * (1/s')), -127, 127) (a
 * row whose reciprocal scale overflows divides by s'),
 * delta' = w' - s'*q' (exact, so s'*q' + delta' rebuilds w'); a row with
 * s' = 0 stores q' = 0, delta' = w'.  With w_live set, the row's live weights
 * are rewritten as bf16(w') in the same pass.  Rows not listed are neither
 * read nor written.  Arithmetic is IEEE fp32 with no contraction.
 * Limits: C % 8 == 0, C <= 65536.
 * Errors: SFT_EINVAL, SFT_ESHAPE, SFT_EALIGN, SFT_ENOTSUP, SFT_EHIP.
 */
int sft_sparse_update(const sft_upd_mat *mats, int32_t n_mats, const sft_adam *hp, void *stream);

/*
 * sft_masked_dw followed by sft_sparse_update on its gradients, with the
 * fix-up of split output tiles folded into the update (sections 2.2, 2.3):
 * each updated row reads its gradient as the sum, in slice order, of the
 * partial rows the product left in the workspace -- the same additions as
 * sft_masked_dw's -- so every result is bit-identical to the two calls.
 *   groups, ws, ws_bytes  as for sft_masked_dw (the same workspace size)
 *   mats / n_mats         one update matrix per dW matrix, in the order of
 *                         the groups and their matrices; mats[i].G must be
 *                         the dW matrix's dW_act, and active_rows, n_active,
 *                         R and C must be the same
 * On return dW_act holds only the tiles that one slice computed whole (the
 * rest stayed in the workspace); its contents are otherwise unspecified.
 * When the groups need more than one product launch, the call runs
 * sft_masked_dw and sft_sparse_update instead.
 * Errors: those of sft_masked_dw and sft_sparse_update; SFT_EINVAL when the
 * update matrices do not match the dW matrices.
 */
int sft_masked_dw_update(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes,
                         const sft_upd_mat *mats, int32_t n_mats, const sft_adam *hp, void *stream);

/*
 * sft_masked_dw_update for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call with the workspace taken from a scratch array
 * the library holds on each device (sft_noalloc_scratch_bytes() bytes, 96 MiB,
 * held until the process ends; its address is looked up once per device on
 * the first call there).  The call allocates nothing.  It uses the current
 * device's array; `stream` must belong to the current device.  Every call on
 * one device shares that array: calls that overlap on one device (different
 * streams, or host threads) race, so order them on one stream.  Results are
 * bit-identical to sft_masked_dw_update.
 * Errors: those of sft_masked_dw_update; SFT_ECAPACITY when the groups need
 * more workspace (sft_masked_dw_workspace) than the array holds; SFT_EHIP
 * if the array's address cannot be found.
 */
size_t sft_noalloc_scratch_bytes(void);
int sft_masked_dw_update_noalloc(const sft_dw_group *groups, int32_t n_groups, const sft_upd_mat *mats,
                                 int32_t n_mats, const sft_adam *hp, void *stream);

/*
 * A coupled pair (section 2.4: gate-up, query-output, key-value).  a and b
 * have equal R and C.  Over the union of the two row lists, the effective
 * gradients are
 *   gA~ = a_own * (clipA * gA) + a_cross * (clipB * gB)
 *   gB~ = a_own * (clipB * gB) + a_cross * (clipA * gA)
 * (fp32, each product and the sum rounded), where a matrix whose row is not in
 * its list contributes a zero gradient; then each matrix whose row is listed
 * takes the plain update above with its effective gradient.  The blend
 * weights a_own/a_cross come from the caller's phase schedule; clip points to
 * a device float[2] {clipA, clipB}, or is NULL for {1, 1}.
 */
/* The union of the two row lists is never formed: each matrix's rows are
 * updated by their own workgroups, which find the partner's row (if any) by a
 * binary search of the partner's ascending active_rows on the device. */
typedef struct sft_pair {
    sft_upd_mat a, b;
    float a_own, a_cross;
    const float *clip;
} sft_pair;

/*
 * All pairs in one launch.  hp->weight_decay is the effective decay (the page
 * scales it by cos(alpha) of the pitch angle; the caller applies that factor).
 * Errors: as sft_sparse_update.
 */
int sft_coupled_update(const sft_pair *pairs, int32_t n_pairs, const sft_adam *hp, void *stream);

/*
 * The sparse write-back (section 2.3): w_live[r, c] = bf16(fl(fl(s[r]*q[r,c]) +
 * delta[r,c])) for the listed rows only; every other row is left untouched.
 *   q int8 [R x C], s fp32 [R], delta fp32 [R x C], w_live bf16 [R x C]
 * Limits: C % 8 == 0.  Errors: SFT_EINVAL, SFT_ESHAPE, SFT_EALIGN, SFT_EHIP.
 */
int sft_masked_writeback(const int8_t *q, const float *s, const float *delta, int64_t R,
                         int64_t C, const int32_t *active_rows, int64_t n_active,
                         uint16_t *w_live, void *stream);

/* One matrix of sft_masked_writeback_many: the arguments of
 * sft_masked_writeback, with the same layouts and limits. */
typedef struct {
    const int8_t *q;            /* int8 [R x C]                     */
    const float *s;             /* fp32 [R]                         */
    const float *delta;         /* fp32 [R x C]                     */
    int64_t R, C;
    const int32_t *active_rows; /* device, ascending, [n_active]    */
    int64_t n_active;
    uint16_t *w_live;           /* bf16 [R x C], written on the listed rows only */
} sft_wb_mat;

/*
 * The sparse write-back (section 2.3) of several matrices in one launch (16
 * matrices per launch; more take more launches): each matrix's listed rows
 * get exactly what sft_masked_writeback writes.  Matrices with no active row
 * are skipped.  The caller owns every buffer; the library keeps no pointer.
 * Errors: SFT_EINVAL (bad sizes, null pointer), SFT_ESHAPE (C % 8 != 0),
 * SFT_EALIGN, SFT_ENOTSUP (2^31 rows or more in one launch), SFT_EHIP; a
 * failed check launches nothing.
 */
int sft_masked_writeback_many(const sft_wb_mat *mats, int32_t n_mats, void *stream);

/* ======================================================================= */
/* device: active-row checkpoints (section 2.6)                             */
/* ======================================================================= */

/*
 * One matrix's part of a checkpoint (section 2.6: the copy holds the active
 * rows only, so it is the size of the active set).  The live state
 * is laid out as in sft_upd_mat; the checkpoint buffers are caller-owned
 * device arrays whose row k belongs to rows[k].
 *   rows  [n_rows] strictly ascending, < R (device)
 *   slot  [n_rows] the moment slot of each row, in [0, n_slots) (device):
 *         at save the slot the moments are read from, at restore the slot
 *         they are written to (the same array unless slots were reassigned)
 *   q, s, delta, m, v, t, mv_exp   live state: int8 [R x C], fp32 [R],
 *                          fp32 [R x C], fp16 [n_slots x C] twice, int32
 *                          [n_slots], int8 [n_slots x 2] (as in sft_upd_mat)
 *   w_live                 bf16 [R x C]; restore rebuilds the restored rows
 *                          as in sft_masked_writeback; NULL = no live copy
 *   ck_q [n_rows x C] int8, ck_s [n_rows] fp32, ck_delta [n_rows x C] fp32,
 *   ck_m, ck_v [n_rows x C] fp16, ck_t [n_rows] int32, ck_mv_exp [n_rows x 2] int8
 */
typedef struct sft_ckpt_mat {
    int64_t R, C, n_rows, n_slots;
    const int32_t *rows;
    const int32_t *slot;
    int8_t *q;
    float *s;
    float *delta;
    uint16_t *m;
    uint16_t *v;
    int32_t *t;
    int8_t *mv_exp;
    uint16_t *w_live;
    int8_t *ck_q;
    float *ck_s;
    float *ck_delta;
    uint16_t *ck_m;
    uint16_t *ck_v;
    int32_t *ck_t;
    int8_t *ck_mv_exp;
} sft_ckpt_mat;

/*
 * Copies the listed rows of every matrix (q, s, delta and the moments, step
 * count and moment exponents of their slots) into the checkpoint buffers, bit for bit; one
 * launch for all matrices.  Rows not listed and the live state are not
 * touched.
 * Limits: C % 8 == 0, fewer than 2^31 rows in all.
 * Errors: SFT_EINVAL (null pointers, negative sizes, n_rows above R or
 * n_slots), SFT_ESHAPE (C % 8), SFT_EALIGN (a row-major buffer not 16-byte
 * aligned), SFT_ENOTSUP (beyond the limits), SFT_EHIP.  Nothing is launched
 * when a check fails.
 */
int sft_rows_save(const sft_ckpt_mat *mats, int32_t n_mats, void *stream);

/*
 * The inverse copy: writes the checkpointed q, s, delta rows back to their
 * rows and the moments, step counts and exponents back to slot[k], bit for bit, and
 * rebuilds those rows of w_live (bf16 of fl(s*q) + delta, as
 * sft_masked_writeback) when w_live is set.  Rows not listed are not
 * touched.  Limits and errors: as sft_rows_save.
 */
int sft_rows_restore(const sft_ckpt_mat *mats, int32_t n_mats, void *stream);

/* ======================================================================= */
/* device: SparseLeaf connection gradients and Adam                          */
/* ======================================================================= */

/*
 * One weight of the SparseLeaf variant (blog post "SparseLeaf: synaptic
 * sparse fine-tuning", section "Weight gradients: write the selected results
 * directly"): for Y = X W^T, D = dL/dY and K selected coordinates (i_k, j_k)
 * of the m x n weight, grad[k] = sum over tokens t of D[t, i_k] * X[t, j_k].
 *   dY   bf16 [T x m], X bf16 [T x n] (row-major, 16-byte aligned)
 *   rows [K] i_k in [0, m), cols [K] j_k in [0, n) (device; any order,
 *        coordinates distinct)
 *   grad [K] fp32 out
 * Summed in fp32 over token ranges (any association), the ranges added in a
 * fixed order: deterministic for a given launch configuration.
 */
typedef struct sft_leaf_mat {
    const uint16_t *dY;
    const uint16_t *X;
    int64_t m, n, K;
    const int32_t *rows;
    const int32_t *cols;
    float *grad;
} sft_leaf_mat;

/* Workspace bytes sft_leaf_grad needs for these matrices and T tokens, or
 * (size_t)-1 on invalid input (message in sft_last_error). */
size_t sft_leaf_grad_workspace(const sft_leaf_mat *mats, int32_t n_mats, int64_t T);

/*
 * The gradients of every matrix's selected connections, all matrices in one
 * launch (plus one short reduction launch).  T = 0 gives zero gradients.
 *   ws / ws_bytes  device scratch of at least sft_leaf_grad_workspace()
 *                  bytes (16-byte aligned; no initialisation needed); calls
 *                  sharing it must be ordered on one stream.
 * Limits: m and n multiples of 8, m <= 65536, n <= 65536, m + n <= 65536,
 * K < 2^31.
 * Errors: SFT_EINVAL (null pointers, negative sizes), SFT_ESHAPE (m or n not
 * a multiple of 8), SFT_EALIGN, SFT_ECAPACITY (workspace too small),
 * SFT_ENOTSUP (beyond the limits), SFT_EHIP.
 */
int sft_leaf_grad(const sft_leaf_mat *mats, int32_t n_mats, int64_t T, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * SparseLeaf Adam (same post, section "The optimizer") on the K increments of
 * one or more weights at step `step` (>= 1, the same for every coordinate: the
 * support is fixed and trains every step); theta, m, v start at zero.
 *   m = beta1*m + (1-beta1)*g,  v = beta2*v + (1-beta2)*g^2,
 *   theta -= lr * (m / bc1[step]) / (sqrt(v / bc2[step]) + eps)
 * in fp32 with every product, sum, quotient and square root rounded on its
 * own (bc1/bc2 from sft_bias_table); theta_bf16 (optional) receives
 * RNE-bf16(theta), the copy used for computation.
 *   grad, theta, m, v [K] fp32; theta_bf16 [K] bf16 or NULL
 * Errors: SFT_EINVAL (null pointers, step outside [1, t_max], nonzero
 * weight_decay: this step has none), SFT_EHIP.
 */
typedef struct sft_leaf_vec {
    int64_t K;
    const float *grad;
    float *theta;
    float *m;
    float *v;
    uint16_t *theta_bf16;
} sft_leaf_vec;

int sft_leaf_adam(const sft_leaf_vec *vecs, int32_t n_vecs, int32_t step, const sft_adam *hp,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SFT_H */
