// sft_internal.h -- helpers shared by the library's translation units
// (error channel and argument checks).  Not part of the public ABI.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "sft.h"

namespace sft {

// Records the message of a failure for sft_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message at the start of a call.
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (256 if the runtime cannot say).
int num_cus();

// Where one matrix's dW rows are after a masked-dW launch that left its cut
// output tiles as partial sums (for the update that adds them itself).
// Partial slot s holds rows [prow][col] of an output tile, row-major, at
// part + s * slot_floats; slice v's first segment uses slot 2v, its last
// segment slot 2v + 1.  A tile one slice covers whole is in dW.
struct DwRowSrc {
    const float *part;
    const float *dW;          // the matrix's dW_act
    const int32_t *tiles;     // active tiles (tile layout), else null
    int64_t n_tiles;
    int64_t slot_floats;
    int64_t it_begin;         // first (output tile, chunk) iteration of the matrix's group
    int64_t P, Q;             // slices of the launch; its rounds of `rnd` chunks
    int32_t bn, rnd;          // columns per output tile, chunks per round
    int32_t chunks, n_nblk, n_ptiles, n_mblk;
    int32_t row_begin;        // first packed row of the matrix in its group
    int32_t layout;           // SFT_DW_TILES or SFT_DW_PACKED
    int32_t nb_major;         // output tiles numbered column block by column block
    int32_t team;             // team slicing: slices wg_begin + t * n_mblk + M-block, t < n_team
    int32_t wg_begin, n_team;
};

// Gather and product of sft_masked_dw without the fix-up, partial tiles
// row-major; src[i] describes the i-th matrix of the groups in order (part
// null for matrices with no active row).  Sets *done = false and launches
// nothing when the call needs more than one launch.  Sets *whole when the
// launch wrote every tile whole into dW_act (no partial sums to add).
int masked_dw_partials(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes, void *stream,
                       DwRowSrc *src, bool *done, bool *whole);

}  // namespace sft

#define SFT_CHECK(cond, code, ...)               \
    do {                                         \
        if (!(cond))                             \
            return ::sft::fail((code), __VA_ARGS__); \
    } while (0)
