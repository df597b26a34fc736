// sft_dw.hip -- the masked weight gradient dW = dY^T X on the gfx950 matrix
// cores, and the embedding's masked gradient.
//
// Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
// Active Set", section 2.2: dW of a linear layer is dY^T times the layer's
// input; the row mask is tested 32 output rows at a time, 32 rows with no
// active one are skipped before any load, multiply or store, and inside an
// active tile the inactive rows
// are dropped before the final write.  For the embedding the input is one-hot,
// so a row's gradient is the sum of dY over the positions of its token.
//
// Masked dW design (MI355X), three kernels on the caller's stream:
//   1. Gather.  Only active 32-row tiles are visited.  The dY columns of the
//      rows to multiply -- every row of each active tile (tile layout) or the
//      active rows packed 32 to a tile (packed layout) -- are copied into a
//      token-contiguous operand buffer laid out as the 32x32x16 MFMA reads
//      its operand: [tile][token/8][row][8 tokens], so one k-step of one tile
//      is 1 KB and lane l reads bytes 16l..16l+15.  Each packed row's
//      destination (matrix, row of dW_act) or -1 goes to a row map.
//   2. Product.  Matrices that read the same X (q/k/v; gate/up) form a group;
//      up to 4 packed tiles of a group (an M-block) share every load of an X
//      block of 64 tokens x 256 columns.  X is the dominant HBM stream.  It
//      goes from HBM straight into a 4-stage LDS ring (buffer_load ... lds,
//      16 bytes per lane, 512 contiguous bytes a row), so 3 chunks (96 KB)
//      are in flight per CU, and the MFMA operand is read from the
//      [token][column] layout with ds_read_b64_tr_b16.  The dY operand goes
//      from the gather buffer straight into registers, 3 chunks ahead.  Two
//      waves share a packed tile, each taking four of its eight 32-column
//      blocks.  The launch is persistent and
//      stream-K: one 8-wave workgroup per CU takes an equal slice of the
//      (output tile, chunk) iteration space; or, where the tiles line up with
//      the CUs, tile-aligned slices, team slices (groups of three or more
//      M-blocks), or narrow whole tiles (128 columns x 128-token chunks, one
//      tile per workgroup, no partial sums at all; a group of more than 4
//      packed tiles there takes M-blocks of up to 8 with one wave per packed
//      tile, over 64 or 128 columns).
//   3. Fix-up.  Output tiles cut by slice boundaries leave partial sums in
//      scratch; this kernel adds them in slice order (deterministic; the
//      kernel boundary orders the stores, so no device-scope fence is needed
//      -- such a fence writes back and invalidates an XCD's L2).  Narrow
//      launches have nothing to add and skip it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "sft_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const bf16x8 gbf16x8;

constexpr int kBN = 256;             // columns per output tile: 8 MFMA column blocks of 32
constexpr int kMaxTiles = 4;         // packed tiles per M-block
constexpr int kBK = 64;              // tokens per chunk: 4 MFMA k-steps of 16
// Narrow output tiles (launches where every workgroup takes one whole tile):
// 128 columns, chunks of 128 tokens (the same 32 KB of X a chunk).
constexpr int kBNn = 128, kBKn = 128;
static_assert(kBK * kBN == kBKn * kBNn, "one X stage size for both tile shapes");
// Narrow tiles of one wave per packed tile (a group of more than 4 packed
// tiles in a narrow launch): M-blocks of up to 8 packed tiles, the same
// 128-token chunks, over 64 columns (16 KB of X a chunk; as many workgroups as
// two 4-tile M-blocks of 128 columns, and the X read once) or 128.
constexpr int kBNw = 64, kMaxTilesW = 8;
constexpr int kRound = 4;            // chunks per pipeline round (segments are whole rounds)
constexpr int kThreads = 512;        // 8 waves
constexpr int kXStages = 4;          // X ring depth
constexpr int kXAhead = kXStages - 1;
constexpr int kXStageBytes = kBK * kBN * 2;   // 32 KB
constexpr int kAAhead = 3;           // chunks of the dY operand in flight (registers)
constexpr int kMaxGroups = 8;
constexpr int kMaxMats = 16;
constexpr int kMaxSegs = 16;         // output tiles touched by one slice
constexpr int kXcds = 8;
constexpr int kTeamMblk = 3;         // team slicing when a group has this many M-blocks (2 measured slower)
constexpr int64_t kSlotFloats = int64_t(kMaxTiles) * 32 * kBN;   // one partial output tile
constexpr int kGatherTokens = 64;
constexpr uint32_t kOutside = 0x80000000u;   // buffer offset beyond every resource size
// Memory instructions a wave issues per chunk: 4 operand loads + 4 X copies.
constexpr int kLoadsA = 4, kCopiesX = 4;
// Stores a wave issues per segment epilogue: 4 column blocks x 4 float4.
constexpr int kEpiStores = 16;
// Loads a wave may leave in flight when chunk j's data must have landed: the
// operand loads and copies of chunks j+1 and j+2 (issued after those of
// chunk j, which go out together, operands first, kAAhead = kXAhead chunks
// ahead).
static_assert(kAAhead == kXAhead, "operands and X travel together");
constexpr int kInFlight = (kXAhead - 1) * (kLoadsA + kCopiesX);

struct DwMatDev {
    const uint16_t *dY;
    const int32_t *rows;    // active rows (packed layout)
    const int32_t *tiles;   // active tiles (tile layout)
    const uint32_t *abits;  // their row bits
    const int32_t *first;   // index of their first active row
    float *out;
    int64_t R;
    int32_t row_begin;      // first packed row of the matrix in its group
};

struct DwGroupDev {
    const uint16_t *X;
    uint16_t *at;           // gathered operand [n_ptiles][Tp/8][32][8] bf16
    int32_t *rowmap;        // [n_ptiles*32]: (matrix << 24) | row of dW_act, or -1
    int64_t T, C;
    int32_t Tp;             // tokens rounded up to whole rounds (of 256 tokens; 512 for narrow tiles)
    int32_t layout;
    int32_t mat_begin, n_mats;
    int32_t n_rows, n_ptiles, n_mblk, n_nblk, chunks;
    int32_t ptile_begin;    // first packed tile in the launch's numbering
    int32_t nb_major;       // output tiles numbered column block by column block (3+ M-blocks)
    int32_t keep_x;         // X copies allocate in L2 (other M-blocks read the same X soon)
    int32_t wg_begin;       // team slicing: first slice of the group's teams
    int32_t n_team;         // team slicing: teams of n_mblk slices each
    int32_t wt;             // narrow launch, one wave per packed tile and M-blocks of up to 8 tiles: 1: 64-column
                            // tiles, 2: 128-column tiles (0: two waves per packed tile, M-blocks of up to 4)
    int64_t it_begin;       // first global iteration of this group
    int64_t otile_begin;    // first output tile (launch numbering)
};

struct DwParams {
    DwGroupDev g[kMaxGroups];
    DwMatDev m[kMaxMats];
    int32_t n_groups;
    int32_t n_wg;           // slices (= workgroups of the product)
    int32_t xcd_blocked;    // neighbouring slices on one XCD (else slice = workgroup index)
    int32_t teams;          // team slicing (per group) instead of slices of the iteration space
    int32_t narrow;         // narrow output tiles, one whole tile per workgroup (no partial sums)
    int64_t iters;          // total (output tile, chunk) iterations, a multiple of kRound
    float *part;            // [2 * n_wg] partial tiles of kSlotFloats
    int32_t part_rows;      // partial tiles row-major (1) or in MFMA fragment order (0)
    float *sink;            // [n_wg * 8] x 16 floats: target of masked-off stores
};

struct Seg {
    int32_t g, nb, mt, p0;
    int32_t k0;     // first chunk of the output tile in this slice
    int32_t j0;     // first local iteration of the segment
    int32_t len;    // chunks (whole rounds)
    int32_t slot;   // -1: whole tile (final output); else partial slot
};

// floor(n / d) for 0 <= n, d < 2^53 through one correctly rounded fp64
// division (a few instructions where a 64-bit integer division is a long
// scalar routine): n/d = k + f with f <= 1 - 1/d, and the rounding error is
// at most (n/d)*2^-53 < 1/d, so the rounded quotient stays below k + 1.
__device__ __forceinline__ int64_t floordiv53(int64_t n, int64_t d) {
    return static_cast<int64_t>(static_cast<double>(n) / static_cast<double>(d));
}

// Packed tiles [lo(b), lo(b+1)) form M-block b: balanced blocks of at most
// kMaxTiles (b * n_ptiles < 2^48).
__device__ __forceinline__ int32_t mblk_lo(const DwGroupDev &G, int32_t b) {
    return static_cast<int32_t>(floordiv53(static_cast<int64_t>(b) * G.n_ptiles, G.n_mblk));
}

// M-block and column block of output tile t of a group.  A group of three or
// more M-blocks numbers its tiles column block by column block (under
// stream-K slicing, which such groups fall back to when their teams do not
// fit the CUs, all M-blocks of one column block then take neighbouring
// slices: one XCD, at about the same time, X from L2 after the first); other
// groups number them M-block by M-block.  The fix-up's grid follows the
// same numbering.
// Returns (M-block, column block).
__device__ __forceinline__ int2 tile_pos(const DwGroupDev &G, int32_t t) {
    const int32_t q = t / (G.nb_major ? G.n_mblk : G.n_nblk);
    const int32_t r = t - q * (G.nb_major ? G.n_mblk : G.n_nblk);
    return G.nb_major ? make_int2(r, q) : make_int2(q, r);
}

// ---------------------------------------------------------------- gather

// One workgroup per (packed tile, 64 tokens) (measured faster than 128 or
// 256: more waves in flight for the scattered reads).  When the tile's 32
// rows are one run of consecutive dY columns starting on a 16-byte boundary
// (whole tiles, and packed rows of a clustered mask), each token's 32 values
// are 64 contiguous bytes: four lanes load them with 16-byte loads (one load
// per thread) into a [token][row] LDS block.  Otherwise thread (row i, token
// t%8) loads one bf16 per 8 tokens into a [row][token] block.  Either block is
// then written as 16-byte runs of 8 tokens of one row.  Rows without a
// source, tokens past T and the padding up to Tp are zero.
__global__ __launch_bounds__(256) void k_dw_gather(const DwParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t tile_t[32][kGatherTokens + 8];
    __shared__ __attribute__((aligned(16))) uint16_t tile_r[kGatherTokens][32];
    __shared__ const uint16_t *s_src[32];
    __shared__ int64_t s_pitch[32];
    __shared__ int32_t s_run;
    const int32_t gp = blockIdx.x;
    int gi = 0;
    while (gi + 1 < p.n_groups && gp >= p.g[gi + 1].ptile_begin) ++gi;
    const DwGroupDev &G = p.g[gi];
    const int32_t pt = gp - G.ptile_begin;
    const int32_t t0 = blockIdx.y * kGatherTokens;
    if (t0 >= G.Tp) return;
    const int tid = threadIdx.x;
    if (tid < 32) {
        const int32_t j = pt * 32 + tid;   // packed row of the group
        const uint16_t *src = nullptr;
        int64_t pitch = 0;
        int32_t code = -1;
        if (j < G.n_rows) {
            int mi = G.mat_begin;
            while (mi + 1 < G.mat_begin + G.n_mats && j >= p.m[mi + 1].row_begin) ++mi;
            const DwMatDev &M = p.m[mi];
            const int32_t jr = j - M.row_begin;
            int64_t col = -1;
            if (G.layout == SFT_DW_PACKED) {
                col = M.rows[jr];
                code = (mi << 24) | jr;
            } else {
                const int32_t tt = jr >> 5, i = jr & 31;
                const uint32_t bits = M.abits[tt];
                const int64_t r = 32 * static_cast<int64_t>(M.tiles[tt]) + i;
                if (r < M.R) col = r;
                if ((bits >> i) & 1u) code = (mi << 24) | (M.first[tt] + __builtin_popcount(bits & ((1u << i) - 1u)));
            }
            if (col >= 0) {
                src = M.dY + col;
                pitch = M.R;
            }
        }
        s_src[tid] = src;
        s_pitch[tid] = pitch;
        if (blockIdx.y == 0) G.rowmap[pt * 32 + tid] = code;
        // one run: every row present, rows consecutive columns of one matrix,
        // the first on a 16-byte boundary (and so every token's 64 bytes)
        const uint16_t *src0 = reinterpret_cast<const uint16_t *>(
            __shfl(reinterpret_cast<uintptr_t>(src), 0, 32));
        const int64_t pitch0 = __shfl(pitch, 0, 32);
        const bool mine = src && src == src0 + tid && pitch == pitch0;
        const bool all = __all(mine ? 1 : 0);   // lanes 32..63 of wave 0 are inactive here
        if (tid == 0)
            s_run = all && (reinterpret_cast<uintptr_t>(src0) & 15u) == 0 && (pitch0 & 7) == 0;
    }
    __syncthreads();
    uint16_t *dst = G.at + (static_cast<int64_t>(pt) * (G.Tp / 8) + t0 / 8) * 256;
    if (s_run) {
        static_assert(kGatherTokens * 4 == 256, "four lanes per token");
        const int tk = tid >> 2, part = tid & 3;
        const int64_t t = t0 + tk;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < G.T) v = *reinterpret_cast<const uint4 *>(s_src[0] + t * s_pitch[0] + 8 * part);
        *reinterpret_cast<uint4 *>(&tile_r[tk][8 * part]) = v;
        __syncthreads();
        const int oct = tid >> 5, r = tid & 31;
        if (t0 + 8 * oct < G.Tp) {
            uint16_t o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = tile_r[8 * oct + e][r];
            uint4 pack;
            pack.x = o[0] | (static_cast<uint32_t>(o[1]) << 16);
            pack.y = o[2] | (static_cast<uint32_t>(o[3]) << 16);
            pack.z = o[4] | (static_cast<uint32_t>(o[5]) << 16);
            pack.w = o[6] | (static_cast<uint32_t>(o[7]) << 16);
            *reinterpret_cast<uint4 *>(dst + (oct * 32 + r) * 8) = pack;
        }
        return;
    }
    const int i = tid & 31, tt = tid >> 5;
    const uint16_t *src = s_src[i];
    const int64_t pitch = s_pitch[i];
    uint16_t v[kGatherTokens / 8];
#pragma unroll
    for (int q = 0; q < kGatherTokens / 8; ++q) {
        const int64_t t = t0 + 8 * q + tt;
        v[q] = (src && t < G.T) ? src[t * pitch] : uint16_t(0);
    }
#pragma unroll
    for (int q = 0; q < kGatherTokens / 8; ++q) tile_t[i][8 * q + tt] = v[q];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGatherTokens / 64; ++u) {
        const int gidx = tid + 256 * u;
        const int oct = gidx >> 5, r = gidx & 31;
        if (t0 + 8 * oct < G.Tp)
            *reinterpret_cast<uint4 *>(dst + (oct * 32 + r) * 8) = *reinterpret_cast<const uint4 *>(&tile_t[r][8 * oct]);
    }
}

// ---------------------------------------------------------------- product

// Slice of workgroup v: global iterations [lo, hi), on whole rounds (output
// tiles are whole rounds too, so every segment is whole rounds).
// Slice v starts at round floor(v * Q / n_wg), Q = iters / kRound rounds.
__device__ __forceinline__ int64_t slice_lo(const DwParams &p, int64_t v) {
    return kRound * floordiv53(v * (p.iters / kRound), p.n_wg);
}

// The X ring: one LDS variable per stage.  The compiler's wait insertion can
// then tell a transposing read of one stage from the direct-to-LDS copies in
// flight into the others (distinct variables get distinct alias scopes); with
// one array it would wait for every copy before every read.  Stage indices
// are compile-time constants in the unrolled round below.
__shared__ __attribute__((aligned(1024))) uint8_t xs0[kXStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t xs1[kXStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t xs2[kXStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t xs3[kXStageBytes];

template <int S>
__device__ __forceinline__ uint8_t *xstage() {
    static_assert(S >= 0 && S < kXStages, "stage");
    if constexpr (S == 0) return xs0;
    else if constexpr (S == 1) return xs1;
    else if constexpr (S == 2) return xs2;
    else return xs3;
}

template <int V>
using ic = std::integral_constant<int, V>;

// Slice of workgroup b: the 32 workgroups of an XCD (the hardware deals
// workgroup i to XCD i mod 8) take neighbouring slices, which share dY
// operand rows and X blocks in that XCD's L2.
__device__ __forceinline__ int64_t slice_of(const DwParams &p) {
    const int64_t b = blockIdx.x;
    return (p.xcd_blocked && p.n_wg % kXcds == 0) ? (b % kXcds) * (p.n_wg / kXcds) + b / kXcds : b;
}

// Wave-uniform copy of a value every lane holds alike (so that it lives in
// scalar registers and buffer resources need no per-lane loop).
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// 16 bytes per lane from buffer r at byte offset voff into LDS at lds +
// 16*lane; offsets at or beyond the buffer's size read as zero.  keep: an
// ordinary cached load (X that other M-blocks read again soon); otherwise
// non-temporal (X read once).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds, bool keep) {
    if (keep)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(lds), 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(lds), 16, voff, 0, 0, 2);
}

__device__ __forceinline__ short4v lds_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v *)(p));
}

// s_waitcnt vmcnt(n) leaving the other counters free (gfx9 encoding).
#define SFT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
// s_waitcnt lgkmcnt(0) leaving vmcnt and expcnt free.
#define SFT_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Output tile = (M-block, 256 columns) of a group; a chunk is 64 tokens.
//
// Per chunk j every wave: waits until its own copies and operand loads of
// chunk j have landed (an exact s_waitcnt: every wave issues the same memory
// instructions in the same order every chunk, masked-off work included), joins
// a bare s_barrier (all copies of chunk j landed; all reads of chunk j-1
// done), issues the operand loads of chunk j+3 and, between its MFMA k-steps,
// the X copies of chunk j+3 into the stage chunk j-1 used.  Segment epilogues
// store unconditionally too (masked-off lanes write to a per-wave sink), so
// the compiler's own waits stay exact as well.
//
// kKeep: the cache policy of the launch's X copies, when every group has the
// same (0 non-temporal, 1 cached), or 2: each group's own (a branch per copy).
//
// kNarrow: output tile = (M-block, 128 columns), a chunk is 128 tokens, and
// every workgroup takes one whole tile (never a partial slot).  The two waves
// of a packed tile then split each chunk's tokens (64 each) rather than its
// columns, so each loads only its own half of the operand; at the end they
// add their sums through LDS and store the tile straight into dW_act.  Odd
// workgroups start halfway along the token axis and wrap (two segments of the
// one tile), so that the launch reads two token ranges at a time.  kNarrow 2
// is the same with the 128-column one-wave body compiled in (kWt below).
//
// kWt (narrow launches only, chosen per workgroup by its group's wt flag):
// output tile = (M-block of up to 8 packed tiles, 64 columns for kWt 1 or 128
// for kWt 2), a chunk is 128 tokens; wave w takes packed tile w over the
// whole chunk (all 128 tokens, every 32-column block of the tile) and stores
// its 32-row sums straight into dW_act.
__shared__ int32_t codes[kMaxSegs][kMaxTiles * 32];
__shared__ DwGroupDev gs[kMaxGroups];   // the group table, indexable at run time
__shared__ float *outp[kMaxMats];
__shared__ Seg segs[kMaxSegs];
__shared__ int32_t s_nseg;
static_assert(kMaxTilesW * 32 <= kMaxSegs * kMaxTiles * 32, "output map of an 8-tile M-block");

template <int kKeep, int kNarrow, int kWt>
__device__ __forceinline__ void masked_dw_body(const DwParams &p, const int64_t v, const int nseg);

template <int kKeep, int kNarrow>
__global__ __launch_bounds__(kThreads, 1) void k_masked_dw(const DwParams p) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int64_t v = slice_of(p);
    const int64_t it_lo = p.teams ? 0 : slice_lo(p, v), it_hi = p.teams ? 1 : slice_lo(p, v + 1);
    if (it_lo >= it_hi) return;

    // ---- the group table, for run-time indexing (one wave per entry, constant
    // indices only: a run-time index into the kernel argument would make the
    // compiler copy it to scratch)
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g)
        if (wave == g && lane == 0) gs[g] = p.g[g];
#pragma unroll
    for (int m = 0; m < kMaxMats; ++m)
        if (wave == (m & 7) && lane == 1 + (m >> 3)) outp[m] = p.m[m].out;

    // ---- meanwhile wave 0 builds the slice's segments (one per output tile it
    // touches) from the kernel argument: wave-uniform control flow, so the
    // table reads are scalar loads.  32-bit arithmetic (the host keeps the
    // iteration count below 2^31).
    if (wave == 0 && p.teams) {
        // Team slicing: the slices of group g form n_team teams of n_mblk;
        // member mb of team t takes M-block mb over the team's share
        // [floor(t*Q/n_team), floor((t+1)*Q/n_team)) of the group's Q =
        // n_nblk * R column-block rounds, column block by column block, so
        // the members read the same X at about the same time.
        int gi = 0;
        while (gi + 1 < p.n_groups && v >= p.g[gi + 1].wg_begin) ++gi;
        const DwGroupDev &G = p.g[gi];
        const int32_t w = static_cast<int32_t>(v) - G.wg_begin;
        int n = 0;
        if (w < G.n_team * G.n_mblk) {
            const int32_t t = w / G.n_mblk, mb = w - t * G.n_mblk;
            const int32_t R = G.chunks / kRound;
            const int64_t Q = static_cast<int64_t>(G.n_nblk) * R;
            int32_t u = static_cast<int32_t>(floordiv53(t * Q, G.n_team));
            const int32_t hi = static_cast<int32_t>(floordiv53((t + 1) * Q, G.n_team));
            const int32_t p0 = mblk_lo(G, mb), mt = mblk_lo(G, mb + 1) - p0;
            int32_t j = 0;
            while (u < hi && n < kMaxSegs) {
                const int32_t nb = u / R, r0 = u - nb * R;
                const int32_t end = min((nb + 1) * R, hi);
                Seg sg;
                sg.g = gi;
                sg.nb = nb;
                sg.p0 = p0;
                sg.mt = mt;
                sg.k0 = r0 * kRound;
                sg.j0 = j;
                sg.len = (end - u) * kRound;
                const bool whole = (r0 == 0 && end == (nb + 1) * R);
                sg.slot = whole ? -1 : (n == 0 ? static_cast<int32_t>(2 * v) : static_cast<int32_t>(2 * v + 1));
                if (lane == 0) segs[n] = sg;
                ++n;
                j += sg.len;
                u = end;
            }
        }
        if (lane == 0) s_nseg = n;
    } else if (wave == 0) {
        int32_t it = static_cast<int32_t>(it_lo);
        const int32_t hi = static_cast<int32_t>(it_hi);
        int n = 0;
        int32_t j = 0;
        while (it < hi && n < kMaxSegs) {
            int gi = 0;
            while (gi + 1 < p.n_groups && it >= static_cast<int32_t>(p.g[gi + 1].it_begin)) ++gi;
            const DwGroupDev &G = p.g[gi];
            const int32_t rel = it - static_cast<int32_t>(G.it_begin);
            const int32_t tile = rel / G.chunks;
            const int32_t k0 = rel - tile * G.chunks;
            const int32_t tile_end = static_cast<int32_t>(G.it_begin) + (tile + 1) * G.chunks;
            const int32_t end = min(tile_end, hi);
            const int2 pos = tile_pos(G, tile);
            const int32_t mb = pos.x;
            Seg sg;
            sg.g = gi;
            sg.nb = pos.y;
            sg.p0 = mblk_lo(G, mb);
            sg.mt = mblk_lo(G, mb + 1) - sg.p0;
            sg.k0 = k0;
            sg.j0 = j;
            sg.len = end - it;
            const bool whole = (k0 == 0 && end == tile_end);
            sg.slot = whole ? -1 : (n == 0 ? static_cast<int32_t>(2 * v) : static_cast<int32_t>(2 * v + 1));
            if (lane == 0) segs[n] = sg;
            ++n;
            j += sg.len;
            it = end;
        }
        if constexpr (kNarrow) {
            // odd workgroups: the second half of the tile's token axis first
            if ((v & 1) && n == 1 && segs[0].len >= 2 * kRound) {
                Seg a = segs[0], b = segs[0];
                const int32_t h = (a.len / kRound / 2) * kRound;
                a.k0 = h;
                a.len = b.len - h;
                b.k0 = 0;
                b.j0 = a.len;
                b.len = h;
                if (lane == 0) {
                    segs[0] = a;
                    segs[1] = b;
                }
                n = 2;
            }
        }
        if (lane == 0) s_nseg = n;
    }
    __syncthreads();
    const int nseg = s_nseg;
    if (nseg == 0) return;   // an idle slice (team slicing pads the grid to whole XCDs)
    if constexpr (kNarrow) {
        // kNarrow 2: the launch has 128-column one-wave tiles, whose body
        // needs more registers than the others (252 against 204 VGPRs), so
        // it is compiled into this instantiation only
        const int32_t wt = __builtin_amdgcn_readfirstlane(gs[segs[0].g].wt);
        if (wt == 1) {
            masked_dw_body<kKeep, 1, 1>(p, v, nseg);
        } else if constexpr (kNarrow == 2) {
            if (wt == 2) masked_dw_body<kKeep, 1, 2>(p, v, nseg);
            else masked_dw_body<kKeep, 1, 0>(p, v, nseg);
        } else {
            masked_dw_body<kKeep, 1, 0>(p, v, nseg);
        }
    } else {
        masked_dw_body<kKeep, 0, 0>(p, v, nseg);
    }
}

template <int kKeep, int kNarrow, int kWt>
__device__ __forceinline__ void masked_dw_body(const DwParams &p, const int64_t v, const int nseg) {
    static_assert(!kWt || kNarrow, "one wave per tile only in narrow launches");
    constexpr int BN = kWt == 1 ? kBNw : kNarrow ? kBNn : kBN;   // columns per output tile
    constexpr int BK = kNarrow ? kBKn : kBK;                // tokens per chunk
    constexpr int kRowLanes = BN / 8;          // 16-byte column groups (lanes) per X row
    constexpr int kCopyRows = 64 / kRowLanes;  // X rows per wave copy
    // per wave and chunk: operand loads (1 KB each), X copies (1 KB each),
    // 32-column blocks and 16-token k-steps
    // (a wide tile's two waves of a packed tile split its columns)
    constexpr int LA = kWt ? 8 : kLoadsA, CX = BK * BN * 2 / (8 * 1024), NC = kNarrow ? BN / 32 : BN / 64,
                  KS = kWt ? 8 : 4;
    static_assert(CX * 8 * 1024 == BK * BN * 2 && KS % CX == 0, "a chunk's X is its waves' copies");
    constexpr int IF = (kXAhead - 1) * (LA + CX);   // loads in flight while chunk j is consumed
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t J = segs[nseg - 1].j0 + segs[nseg - 1].len;
    float *const sink = p.sink + (v * 8 + wave) * 16;

    // ---- X copies.  A chunk is BK token rows x BN columns (64 x 256, 512
    // bytes a row; narrow 128 x 128, 256 bytes a row); copy k (k = 0..3) of a
    // wave holds the kCopyRows rows from kCopyRows*q, q = wave + 8k.  Lane slot
    // l%kRowLanes of row kCopyRows*q + l/kRowLanes holds the 16-byte column
    // group (l%kRowLanes) ^ 2*(row%4) (a swizzle that makes the transposing
    // reads of 4 consecutive rows hit distinct banks).  The buffer resource's base
    // advances by one chunk per chunk (scalar work); rows past T fall beyond
    // its size and columns past C get an offset beyond any size, so the range
    // check turns them into zeros.
    // The next segment's first chunk is kept in a register (a chunk only
    // compares against it), and a chunk's copies share one buffer resource.
    int sx = 0;
    const uint8_t *x_base = nullptr;
    int64_t x_rem = 0, x_stride = 0;
    int32_t x_j0 = 0, x_next = 0;
    bool x_keep = kKeep == 1;
    uint32_t x_voff[CX];
    auto describe_x = [&](int sg) __attribute__((always_inline)) {
        const Seg &S = segs[sg];
        const DwGroupDev &G = gs[S.g];
        const int64_t C = G.C, c0 = static_cast<int64_t>(S.nb) * BN, r0 = static_cast<int64_t>(S.k0) * BK;
        x_base = reinterpret_cast<const uint8_t *>(uniform64(reinterpret_cast<uint64_t>(G.X + r0 * C + c0)));
        x_rem = static_cast<int64_t>(uniform64(static_cast<uint64_t>((G.T - r0) * C * 2 - c0 * 2)));
        x_stride = static_cast<int64_t>(uniform64(static_cast<uint64_t>(BK * C * 2)));
        x_j0 = __builtin_amdgcn_readfirstlane(S.j0);
        x_next = __builtin_amdgcn_readfirstlane(sg + 1 < nseg ? segs[sg + 1].j0 : J);
        if constexpr (kKeep == 2) x_keep = __builtin_amdgcn_readfirstlane(G.keep_x) != 0;
#pragma unroll
        for (int k = 0; k < CX; ++k) {
            const int row_in = kCopyRows * (wave + 8 * k) + lane / kRowLanes;
            const int grp = (lane % kRowLanes) ^ (2 * (row_in & 3));
            x_voff[k] = (c0 + 8 * grp < C) ? static_cast<uint32_t>((row_in * C + 8 * grp) * 2) : kOutside;
        }
    };
    auto advance_x = [&](int32_t jx) __attribute__((always_inline)) {
        if (jx >= x_next && jx < J) {
            ++sx;
            describe_x(sx);
        }
    };
    // the buffer resource of chunk jx's X (size 0 past the slice)
    auto x_rsrc = [&](int32_t jx) __attribute__((always_inline)) {
        const int64_t off = static_cast<int64_t>(jx - x_j0) * x_stride;
        const int64_t rem = jx < J ? x_rem - off : 0;
        const int32_t size = static_cast<int32_t>(rem <= 0 ? 0 : (rem > 0x7fffffff ? 0x7fffffff : rem));
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(x_base + (jx < J ? off : 0)),
                                                 static_cast<short>(0), size, 0x00020000);
    };
    auto issue_x = [&](__amdgpu_buffer_rsrc_t r, int k, uint8_t *stage) __attribute__((always_inline)) {
        dma16(r, x_voff[k], stage + (wave + 8 * k) * 1024, x_keep);
    };

    // ---- wave layout: wave w takes packed tile w/2 of the M-block and the
    // column half w%2 (four 32-column blocks); narrow: all four column blocks
    // of the tile and the token half w%2 of each chunk.  Waves past the
    // M-block's tiles only copy.
    const int tw = kWt ? wave : wave >> 1, ch = kWt ? 0 : wave & 1;

    // ---- dY operand: 4 KB per (packed tile, 64 tokens); k-step kk is the
    // 1 KB at 512*kk elements, lane l's 16 bytes at 8*l.  A narrow chunk's
    // wave loads the 4 KB of its token half.  Loads go through a buffer
    // resource whose size is 0 for waves without a tile and for chunks past
    // the slice: the load is still issued (every wave issues the same memory
    // instructions every chunk) but touches no memory.
    int sa = 0;
    const uint16_t *a_base = nullptr;
    int32_t a_j0 = 0, a_next = 0;
    bool a_live = false;
    auto describe_a = [&](int sg) __attribute__((always_inline)) {
        const Seg &S = segs[sg];
        const DwGroupDev &G = gs[S.g];
        a_next = __builtin_amdgcn_readfirstlane(sg + 1 < nseg ? segs[sg + 1].j0 : J);
        a_live = tw < S.mt;
        a_base = reinterpret_cast<const uint16_t *>(uniform64(reinterpret_cast<uint64_t>(
            G.at + (static_cast<int64_t>(S.p0 + (a_live ? tw : 0)) * (G.Tp / 8) + (BK / 8) * static_cast<int64_t>(S.k0)) * 256 +
            (kNarrow && !kWt ? 2048 * ch : 0))));
        a_j0 = __builtin_amdgcn_readfirstlane(S.j0);
    };
    auto issue_a = [&](int32_t ja, bf16x8 (&buf)[LA]) __attribute__((always_inline)) {
        if (ja >= a_next && ja < J) {
            ++sa;
            describe_a(sa);
        }
        const bool live = a_live && ja < J;
        const uint16_t *base = a_base + (live ? static_cast<int64_t>(ja - a_j0) * (BK / 8) * 256 : 0);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(base), static_cast<short>(0), live ? 1024 * LA : 0, 0x00020000);
#pragma unroll
        for (int kk = 0; kk < LA; ++kk)
            buf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane + 1024 * kk, 0, 0));
    };

    // ---- operand reads of X: lane l takes column l%32 of a 32-column block,
    // tokens 8*(l/32) + 0..7 of a k-step, by two transposing reads of 4 rows.
    // Column group g of token row r sits at group g ^ 2*(r%4); here r%4 =
    // (l%16)/4 for every row a lane reads.
    const int s16 = lane & 15;
    const int trow = 8 * (lane >> 5) + (s16 >> 2);
    const int xcp = ((lane >> 4) & 1) * 16 + 4 * (s16 & 3);   // column inside a 32-column block
    int xo[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int cb = kNarrow ? c : 4 * ch + c;
        xo[c] = 8 * ((4 * cb + (xcp >> 3)) ^ (2 * (s16 >> 2))) + (xcp & 7);
    }

    // Accumulators: acc[c] = X-block^T . dY-tile for the wave's c-th column
    // block, so lane l register r holds column 8*(r/4) + 4*(l/32) + r%4 of the
    // block for packed row l%32: four consecutive columns per register quad,
    // stored as one float4.
    floatx16 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;

    auto wait_vm = [](int n) __attribute__((always_inline)) {
        if (n == IF) SFT_WAIT_VMCNT(IF);
        else SFT_WAIT_VMCNT(IF + kEpiStores);
    };

    // One chunk, u = jj mod 4 (a constant): reads stage u and A buffer u; the
    // operand loads and copies of chunk jj+3 go to buffer (u+3)%4 and stage
    // (u+3)%4 (chunk jj-1's), one copy after each k-step.
    bf16x8 ab[kAAhead + 1][LA];
    auto step = [&](auto u_tag, int32_t jj, int n_wait, bool active) __attribute__((always_inline)) {
        constexpr int U = decltype(u_tag)::value;
        const uint16_t *X = reinterpret_cast<const uint16_t *>(xstage<U>());
        uint8_t *st_dma = xstage<(U + kXAhead) % kXStages>();
        const bf16x8 (&a)[LA] = ab[U % (kAAhead + 1)];
        SFT_WAIT_LGKM0();
        wait_vm(n_wait);
        __builtin_amdgcn_s_barrier();
        issue_a(jj + kAAhead, ab[(U + kAAhead) % (kAAhead + 1)]);
        const int32_t jx = jj + kXAhead;
        advance_x(jx);
        const __amdgpu_buffer_rsrc_t xr = x_rsrc(jx);
        auto bfrag = [&](int kk, bf16x8 (&b)[NC]) __attribute__((always_inline)) {
            const int r0 = (kNarrow && !kWt ? 64 * ch : 0) + 16 * kk + trow;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const short4v lo = lds_tr16(X + r0 * BN + xo[c]);
                const short4v hi = lds_tr16(X + (r0 + 4) * BN + xo[c]);
                b[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        // The X copies are issued on every path (only the MFMA work is
        // conditional), so the compiler's count of operations in flight is
        // exact; they sit between k-steps to overlap the matrix cores.  The
        // fragments alternate between two register sets (k-step kk reads set
        // kk%2 while set (kk+1)%2 fills), with no copies between them.
        // Copy k follows k-step k*KS/CX (every k-step; one wave per tile:
        // k-steps 0 and 4 of 8).
        bf16x8 bf[2][NC];
        if (active) bfrag(0, bf[0]);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (active) {
                if (kk < KS - 1) bfrag(kk + 1, bf[(kk + 1) & 1]);
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[kk & 1][c], a[kk], acc[c], 0, 0, 0);
            }
            if (kk % (KS / CX) == 0) {
                __builtin_amdgcn_sched_barrier(0);
                issue_x(xr, kk / (KS / CX), st_dma);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    static_assert(LA == KS && kRound == kXStages, "one operand load per k-step; stages rotate once a round");
    // A round of 4 chunks; the first three wait for `extra` more operations.
    auto round4 = [&](int32_t jq, bool active, int extra) __attribute__((always_inline)) {
        step(ic<0>{}, jq + 0, IF + extra, active);
        step(ic<1>{}, jq + 1, IF + extra, active);
        step(ic<2>{}, jq + 2, IF + extra, active);
        step(ic<3>{}, jq + 3, IF, active);
    };

    // Segment epilogue: every wave issues 16 float4 stores (masked-off lanes
    // write to the sink).  A whole tile goes to dW_act through the row map,
    // row-major.  A partial one goes to its slot in fragment order: store q
    // of wave (tw, ch) fills the 1 KB fragment (tw*2 + ch)*16 + q, lane l's
    // 16 bytes at 16*l, so each of those stores is one contiguous kilobyte;
    // or, for an update that reads its rows from the slots, row-major.
    auto epilogue = [&](int sg) __attribute__((always_inline)) {
      if constexpr (!kNarrow) {
        const Seg &S = segs[sg];
        const DwGroupDev &G = gs[S.g];
        const int h = lane >> 5;
        const int32_t code = tw < S.mt ? codes[sg][tw * 32 + (lane & 31)] : -1;
        const int64_t c0 = static_cast<int64_t>(S.nb) * kBN;
        const bool part = S.slot >= 0;
        const bool frag = part && !p.part_rows;
        float *base = sink;
        if (code >= 0)
            base = frag ? p.part + S.slot * kSlotFloats + ((tw * 2 + ch) * kEpiStores * 64 + lane) * 4
                 : part ? p.part + S.slot * kSlotFloats + (tw * 32 + (lane & 31)) * kBN + 128 * ch + 4 * h
                        : outp[code >> 24] + static_cast<int64_t>(code & 0xFFFFFF) * G.C + c0 + 128 * ch + 4 * h;
#pragma unroll
        for (int q = 0; q < kEpiStores; ++q) {
            const int c = q / 4, a = q % 4;
            const bool ok = code >= 0 && (part || c0 + 32 * (4 * ch + c) + 8 * a + 4 * h < G.C);
            const int off = frag ? 256 * q : 32 * c + 8 * a;
            auto *dst = reinterpret_cast<__attribute__((address_space(1))) f32x4 *>(
                reinterpret_cast<uintptr_t>(ok ? base + off : sink));
            *dst = f32x4{acc[c][4 * a], acc[c][4 * a + 1], acc[c][4 * a + 2], acc[c][4 * a + 3]};
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
      }
    };

    // Narrow epilogue (the workgroup's one tile): waves 2t and 2t+1 summed
    // tile t over the two token halves of every chunk.  Once every copy has
    // landed the X ring is free: each wave leaves its 32 x 128 partial there
    // row-major (16 KB; the 16-byte groups of row r swizzled by r%16, so that
    // the writes of a fragment and the reads of a row hit distinct banks), and
    // after a barrier wave 2t+h adds the two partials of rows 16h..16h+15 and
    // stores them two rows (1 KB) an instruction.  Two addends: the sum does
    // not depend on which wave adds.
    auto epilogue_narrow = [&](int sg) __attribute__((always_inline)) {
      if constexpr (kNarrow && !kWt) {
        const Seg &S = segs[sg];
        const DwGroupDev &G = gs[S.g];
        SFT_WAIT_VMCNT(0);
        __syncthreads();
        auto region = [&](int w) __attribute__((always_inline)) {
            uint8_t *st = w < 2 ? xstage<0>() : w < 4 ? xstage<1>() : w < 6 ? xstage<2>() : xstage<3>();
            return reinterpret_cast<float *>(st) + (w & 1) * (32 * kBNn);
        };
        {
            float *const mine = region(wave);
            const int r = lane & 31, h = lane >> 5;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int g = 8 * c + 2 * a + h;
                    *reinterpret_cast<f32x4 *>(mine + r * kBNn + 4 * (g ^ (r & 15))) =
                        f32x4{acc[c][4 * a], acc[c][4 * a + 1], acc[c][4 * a + 2], acc[c][4 * a + 3]};
                }
        }
        __syncthreads();
        const float *const p0 = region(2 * tw), *const p1 = region(2 * tw + 1);
        const int64_t c0 = static_cast<int64_t>(S.nb) * BN;
        const int g = lane & 31;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 16 * ch + 2 * i + (lane >> 5);
            const int o = r * kBNn + 4 * (g ^ (r & 15));
            const f32x4 x = *reinterpret_cast<const f32x4 *>(p0 + o);
            const f32x4 y = *reinterpret_cast<const f32x4 *>(p1 + o);
            const int32_t code = tw < S.mt ? codes[sg][tw * 32 + r] : -1;
            if (code >= 0 && c0 + 4 * g < G.C) {
                float *dst = outp[code >> 24] + static_cast<int64_t>(code & 0xFFFFFF) * G.C + c0 + 4 * g;
                *reinterpret_cast<__attribute__((address_space(1))) f32x4 *>(reinterpret_cast<uintptr_t>(dst)) = x + y;
            }
        }
      }
    };

    // One wave per tile: wave w holds packed tile w's 32 x BN sums over the
    // whole token axis; each lane stores 4 consecutive columns of its row at
    // a time (a lane pair covers 8 columns a store) straight into dW_act.  No
    // wave adds another's sums.
    auto epilogue_wt = [&](int sg) __attribute__((always_inline)) {
      if constexpr (kWt) {
        const Seg &S = segs[sg];
        const DwGroupDev &G = gs[S.g];
        SFT_WAIT_VMCNT(0);   // the copies past the slice (zeros into LDS) land before the workgroup ends
        const int h = lane >> 5;
        const int32_t code = tw < S.mt ? (&codes[0][0])[tw * 32 + (lane & 31)] : -1;
        const int64_t c0 = static_cast<int64_t>(S.nb) * BN;
        if (code >= 0) {
            float *const row = outp[code >> 24] + static_cast<int64_t>(code & 0xFFFFFF) * G.C;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int64_t col = c0 + 32 * c + 8 * a + 4 * h;
                    if (col < G.C)
                        *reinterpret_cast<__attribute__((address_space(1))) f32x4 *>(
                            reinterpret_cast<uintptr_t>(row + col)) =
                            f32x4{acc[c][4 * a], acc[c][4 * a + 1], acc[c][4 * a + 2], acc[c][4 * a + 3]};
                }
        }
      }
    };

    // ---- the output map of the slice's first four segments (thread t: entry
    // t%128 of segment t/128; one wave per tile: entry t of the one tile's
    // map, up to 8 packed tiles), loaded ahead of the prologue so that the wait
    // for it covers these loads only; written to LDS behind the prologue, and
    // read only by epilogues, after the first chunk's barrier.
    const int csg = kWt ? 0 : tid >> 7, crow = kWt ? tid : tid & 127;
    int32_t cval = -1;
    if (csg < nseg) {
        const int32_t gsg = __builtin_amdgcn_readfirstlane(segs[csg].g);
        // (a global, not flat, load: flat loads count in lgkmcnt too, and every
        // LDS access of the prologue would then wait for this one)
        if (crow < segs[csg].mt * 32)
            cval = *reinterpret_cast<__attribute__((address_space(1))) const int32_t *>(
                reinterpret_cast<uintptr_t>(gs[gsg].rowmap + segs[csg].p0 * 32 + crow));
    }

    // ---- prologue: operands and X copies of chunks 0..2, in the order the
    // steady state issues them.
    describe_x(0);
    describe_a(0);
    auto prologue = [&](auto s_tag) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;
        issue_a(S, ab[S]);
        advance_x(S);
        const __amdgpu_buffer_rsrc_t xr = x_rsrc(S);
#pragma unroll
        for (int k = 0; k < CX; ++k) issue_x(xr, k, xstage<S>());
    };
    static_assert(kXAhead == 3, "prologue order");
    prologue(ic<0>{});
    prologue(ic<1>{});
    prologue(ic<2>{});

    static_assert(kThreads / (kMaxTiles * 32) == 4 && kMaxSegs >= 4, "four segments' output map per pass");
    if constexpr (kWt) {
        if (tid < kMaxTilesW * 32) (&codes[0][0])[tid] = cval;
    } else {
        codes[csg][crow] = cval;
    }
    if (!kNarrow && nseg > 4) {   // rare: slices across more than four output tiles
        for (int sg = 4; sg < nseg; ++sg) {
            const int32_t gsg = __builtin_amdgcn_readfirstlane(segs[sg].g);
            const int32_t *map = gs[gsg].rowmap + segs[sg].p0 * 32;
            const int32_t n = segs[sg].mt * 32;
            for (int r = tid; r < kMaxTiles * 32; r += kThreads) codes[sg][r] = r < n ? map[r] : -1;
        }
        __syncthreads();
    }

    // ---- the segments.  The first round of every segment but the first waits
    // for 16 more memory operations in its first three chunks (the previous
    // epilogue's stores sit behind their loads); the first segment's code is
    // separate, so that each loop sees one state of the operations in flight.
    auto segment = [&](int sg, auto first_tag) __attribute__((always_inline)) {
        const int32_t j0 = segs[sg].j0, len = segs[sg].len;
        const bool active = tw < segs[sg].mt;
        round4(j0, active, decltype(first_tag)::value ? 0 : kEpiStores);
        for (int32_t jq = j0 + kRound; jq < j0 + len; jq += kRound) round4(jq, active, 0);
        epilogue(sg);
    };
    if constexpr (kNarrow) {
        // one tile (the host plans narrow launches that way), in one or two
        // segments
        const bool active = tw < segs[0].mt;
        round4(0, active, 0);
        for (int32_t jq = kRound; jq < J; jq += kRound) round4(jq, active, 0);
        if constexpr (kWt) epilogue_wt(0);
        else epilogue_narrow(0);
        return;
    } else {
        segment(0, ic<1>{});
        for (int sg = 1; sg < nseg; ++sg) segment(sg, ic<0>{});
    }
    // Copies past the slice are still in flight (they write zeros to LDS):
    // drain them before the workgroup's LDS can be handed to another (the
    // last epilogue's stores, issued after them, may stay in flight).
    SFT_WAIT_VMCNT(kEpiStores);
}

// Combination of the partial tiles: an output tile cut by slice boundaries
// is the sum of its slices' partial rows, added in slice order.  One
// workgroup per (output tile, 32 packed rows); a lane adds 4 columns of 8
// rows.  The tile bookkeeping is wave-uniform; a lane issues its row-map
// loads and the partial loads of its rows for the first four slices
// together, so the kernel is one memory round trip for tiles cut up to
// four ways.
__global__ __launch_bounds__(256) void k_dw_fixup(const DwParams p) {
    const int64_t ot = blockIdx.x;
    int gi = 0;
    while (gi + 1 < p.n_groups && ot >= p.g[gi + 1].otile_begin) ++gi;
    const DwGroupDev &G = p.g[gi];
    const int32_t tile = static_cast<int32_t>(ot - G.otile_begin);
    const int2 pos = tile_pos(G, tile);
    const int32_t mb = pos.x, nb = pos.y;
    // The tile is rounds [a, b) of a space of Q rounds cut into P equal
    // ranges: the launch's iterations and its slices, or (team slicing) the
    // group's column-block rounds and its teams, range i being slice
    // base + i * stride.  Range i starts at or before round r exactly when
    // floor(i * Q / P) < r + 1, i.e. when i <= ((r + 1) * P - 1) / Q.
    int64_t a, b, Q, P;
    int32_t base = 0, stride = 1;
    if (p.teams) {
        const int32_t R = G.chunks / kRound;
        a = static_cast<int64_t>(nb) * R;
        b = a + R;
        Q = static_cast<int64_t>(G.n_nblk) * R;
        P = G.n_team;
        base = G.wg_begin + mb;
        stride = G.n_mblk;
    } else {
        a = (G.it_begin + static_cast<int64_t>(tile) * G.chunks) / kRound;
        b = a + G.chunks / kRound;
        Q = p.iters / kRound;
        P = p.n_wg;
    }
    const int32_t v_first = static_cast<int32_t>(floordiv53((a + 1) * P - 1, Q));
    const int32_t v_last = static_cast<int32_t>(floordiv53(b * P - 1, Q));
    if (v_first == v_last) return;  // the tile lies inside one range: written directly
    const int32_t p0 = mblk_lo(G, mb), mt = mblk_lo(G, mb + 1) - p0;
    const int tw = blockIdx.y;
    if (tw >= mt) return;   // past the M-block's packed tiles
    // The first slice started before the tile (its last segment: odd slot)
    // unless it starts at round a; every later one starts inside the tile
    // (first segment: even slot).
    const bool first_odd = floordiv53(static_cast<int64_t>(v_first) * Q, P) < a;
    // Partial slots hold the product's fragments: fragment f = (tw*2 + ch)*16
    // + 4*c + a (1 KB), lane l's 4 floats at 4*l, are columns
    // 32*(4*ch + c) + 8*a + 4*(l/32) .. +3 of packed row tw*32 + l%32.  Thread
    // t takes lane t%64 of fragments tw*32 + t/64 + 4*i, i = 0..7: one row,
    // eight 4-column pieces, all loads before the sums.
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const int32_t code = G.rowmap[p0 * 32 + tw * 32 + (lane & 31)];
    const float *part = p.part + (tw * 32 + (threadIdx.x >> 6)) * 256 + lane * 4;
    constexpr int kRows = 8;
    float4 x[4][kRows];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int32_t vv = v_first + c;
        const int64_t sv = base + static_cast<int64_t>(vv) * stride;
        const int64_t slot = (c == 0 && first_odd) ? 2 * sv + 1 : 2 * sv;
        if (vv <= v_last) {
#pragma unroll
            for (int i = 0; i < kRows; ++i)
                x[c][i] = *reinterpret_cast<const float4 *>(part + slot * kSlotFloats + 4 * i * 256);
        }
    }
    float4 sum[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        sum[i] = x[0][i];
#pragma unroll
        for (int c = 1; c < 4; ++c) {
            if (v_first + c <= v_last) {
                sum[i].x += x[c][i].x;
                sum[i].y += x[c][i].y;
                sum[i].z += x[c][i].z;
                sum[i].w += x[c][i].w;
            }
        }
    }
    for (int32_t vv = v_first + 4; vv <= v_last; ++vv) {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const float4 y = *reinterpret_cast<const float4 *>(
                part + 2 * (base + static_cast<int64_t>(vv) * stride) * kSlotFloats + 4 * i * 256);
            sum[i].x += y.x;
            sum[i].y += y.y;
            sum[i].z += y.z;
            sum[i].w += y.w;
        }
    }
    if (code < 0) return;
    float *out = p.m[code >> 24].out + static_cast<int64_t>(code & 0xFFFFFF) * G.C + static_cast<int64_t>(nb) * kBN;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int f = (threadIdx.x >> 6) + 4 * i;   // (ch*4 + c)*4 + a
        const int cl = 32 * (f >> 2) + 8 * (f & 3) + 4 * h;   // block ch*4 + c, piece a, half h
        if (static_cast<int64_t>(nb) * kBN + cl < G.C) *reinterpret_cast<float4 *>(out + cl) = sum[i];
    }
}

// ---------------------------------------------------------------- embedding

constexpr int kEmbThreads = 512;   // 8 waves split a row's positions (measured faster than 4 or 16)
constexpr int kEmbVec = 4;         // columns per lane (8-byte loads)
constexpr int kEmbCols = 64 * kEmbVec;   // columns per workgroup
constexpr int kEmbBatch = 32;      // positions whose dY loads a wave keeps in flight

// One workgroup per (active row, 256 columns).  Wave w sums the w-th of 8
// contiguous shares of the row's positions (fp64, in position order).  The
// wave reads up to 64 of its positions with one vector load, takes them from
// the lanes one by one (wave-uniform), and issues the dY loads of 32
// positions together before adding them, so a hot row (hundreds of hits)
// costs a few memory round trips per wave rather than one per position.
// The 8 wave sums are added in wave order and rounded to fp32 once.
__global__ __launch_bounds__(kEmbThreads) void k_embedding_dw(const uint16_t *__restrict__ dY,
                                                              int64_t d,
                                                              const int32_t *__restrict__ row_ptr,
                                                              const int32_t *__restrict__ positions,
                                                              float *__restrict__ dW_act) {
    __shared__ double part[kEmbThreads / 64][kEmbCols];
    const int64_t k = blockIdx.y;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kEmbCols;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t col = c0 + lane * kEmbVec;
    const bool in = col < d;
    const int64_t lo = row_ptr[k], n = row_ptr[k + 1] - lo;
    const int64_t a = lo + n * wave / (kEmbThreads / 64), b = lo + n * (wave + 1) / (kEmbThreads / 64);
    double acc[kEmbVec] = {0, 0, 0, 0};
    for (int64_t base = a; base < b; base += 64) {
        const int m = static_cast<int>(b - base < 64 ? b - base : 64);
        const int32_t pv = lane < m ? positions[base + lane] : 0;
        for (int j0 = 0; j0 < m; j0 += kEmbBatch) {
            uint2 v[kEmbBatch];
#pragma unroll
            for (int j = 0; j < kEmbBatch; ++j) {
                v[j] = make_uint2(0, 0);
                if (j0 + j < m) {
                    const int64_t t = __builtin_amdgcn_readlane(pv, j0 + j);
                    if (in) v[j] = *reinterpret_cast<const uint2 *>(dY + t * d + col);
                }
            }
#pragma unroll
            for (int j = 0; j < kEmbBatch; ++j) {
                if (j0 + j < m) {
                    const uint32_t w[2] = {v[j].x, v[j].y};
#pragma unroll
                    for (int e = 0; e < kEmbVec; ++e) {
                        const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
                        acc[e] += static_cast<double>(__uint_as_float(bits));
                    }
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < kEmbVec; ++e) part[wave][lane * kEmbVec + e] = acc[e];
    __syncthreads();
    // Fixed-order combination of the wave partials (fp64), one rounding.
    for (int c = threadIdx.x; c < kEmbCols; c += kEmbThreads) {
        if (c0 + c >= d) continue;
        double s = part[0][c];
        for (int w = 1; w < kEmbThreads / 64; ++w) s += part[w][c];
        dW_act[k * d + c0 + c] = static_cast<float>(s);
    }
}

// ---------------------------------------------------------------- host side

struct Launch {
    DwParams p;
    int64_t out_tiles = 0;
    int32_t gather_tiles = 0;    // packed tiles of the launch (gather grid x)
    int32_t gather_blocks = 0;   // 256-token blocks of the longest group (gather grid y)
    size_t at_bytes = 0;         // gathered operands + row maps of the launch
    std::vector<size_t> at_off, map_off;   // per group, inside that region
};

struct Plan {
    std::vector<Launch> launches;
    bool too_big = false;      // a launch would exceed 2^31 (tile, chunk) iterations
    size_t part_bytes = 0, sink_bytes = 0, at_bytes = 0;
    size_t ws_bytes() const { return part_bytes + sink_bytes + at_bytes; }
};

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }


bool group_live(const sft_dw_group &g) {
    for (int32_t mi = 0; mi < g.n_mats; ++mi)
        if (g.mats[mi].n_active_tiles) return true;
    return false;
}

int validate(const sft_dw_group *groups, int32_t n_groups) {
    SFT_CHECK(n_groups >= 0 && (n_groups == 0 || groups), SFT_EINVAL, "sft_masked_dw: bad group list");
    for (int32_t gi = 0; gi < n_groups; ++gi) {
        const sft_dw_group &g = groups[gi];
        SFT_CHECK(g.n_mats >= 0 && (g.n_mats == 0 || g.mats), SFT_EINVAL,
                  "sft_masked_dw: group %d has a bad matrix list", gi);
        SFT_CHECK(g.n_mats <= kMaxMats, SFT_ENOTSUP, "sft_masked_dw: group %d has more than %d matrices",
                  gi, kMaxMats);
        SFT_CHECK(g.layout == SFT_DW_TILES || g.layout == SFT_DW_PACKED, SFT_EINVAL,
                  "sft_masked_dw: group %d has unknown layout %d", gi, g.layout);
        if (!group_live(g)) continue;
        SFT_CHECK(g.T >= 1 && g.T <= (int64_t(1) << 24) && g.C > 0, g.T > (int64_t(1) << 24) ? SFT_ENOTSUP : SFT_EINVAL,
                  "sft_masked_dw: group %d has T=%lld C=%lld", gi, (long long)g.T, (long long)g.C);
        SFT_CHECK(g.C % 8 == 0, SFT_ESHAPE, "sft_masked_dw: C=%lld is not a multiple of 8", (long long)g.C);
        SFT_CHECK(g.T * g.C < (int64_t(1) << 31), SFT_ENOTSUP, "sft_masked_dw: group %d: T*C reaches 2^31", gi);
        // (a chunk's X copy offsets, up to 63 rows of C columns, stay 32-bit)
        SFT_CHECK(g.C <= (int64_t(1) << 24), SFT_ENOTSUP, "sft_masked_dw: group %d: C above 2^24", gi);
        SFT_CHECK(g.X && sft::aligned16(g.X), g.X ? SFT_EALIGN : SFT_EINVAL,
                  "sft_masked_dw: group %d X null or not 16-byte aligned", gi);
        for (int32_t mi = 0; mi < g.n_mats; ++mi) {
            const sft_dw_mat &m = g.mats[mi];
            SFT_CHECK(m.R > 0 && m.R < (int64_t(1) << 31) && m.n_active >= 0 && m.n_active_tiles >= 0,
                      SFT_EINVAL, "sft_masked_dw: matrix %d/%d has bad sizes", gi, mi);
            SFT_CHECK(m.n_active_tiles <= (m.R + 31) / 32 && m.n_active <= m.R &&
                          m.n_active >= m.n_active_tiles && (m.n_active == 0) == (m.n_active_tiles == 0),
                      SFT_EINVAL, "sft_masked_dw: matrix %d/%d has inconsistent counts", gi, mi);
            SFT_CHECK(m.n_active < (int64_t(1) << 24), SFT_ENOTSUP,
                      "sft_masked_dw: matrix %d/%d has 2^24 or more active rows", gi, mi);
            if (m.n_active_tiles == 0) continue;
            SFT_CHECK(m.dY && m.dW_act, SFT_EINVAL, "sft_masked_dw: matrix %d/%d has a null pointer", gi, mi);
            if (g.layout == SFT_DW_PACKED)
                SFT_CHECK(m.active_rows, SFT_EINVAL, "sft_masked_dw: matrix %d/%d: packed layout needs active_rows",
                          gi, mi);
            else
                SFT_CHECK(m.active_tiles && m.active_bits && m.tile_first, SFT_EINVAL,
                          "sft_masked_dw: matrix %d/%d: tile layout needs the tile arrays", gi, mi);
            SFT_CHECK(sft::aligned16(m.dW_act), SFT_EALIGN, "sft_masked_dw: matrix %d/%d dW_act not 16-byte aligned",
                      gi, mi);
        }
    }
    return SFT_OK;
}

// Launch decomposition, shared by the workspace query and the launch.
// Workspace: [partial slots][store sink][gathered operands + row maps of one
// launch] (launches run in stream order, so they reuse the last region).
// Shapes of a group in a narrow launch (DwGroupDev::wt): 0, M-blocks of up
// to 4 packed tiles and 128-column tiles, two waves per packed tile; 1 and 2,
// M-blocks of up to 8 packed tiles, one wave per packed tile, over 64 or 128
// columns.  Returns the group's output tiles (= workgroups) in that shape.
int64_t narrow_tiles(const DwGroupDev &d, int wt) {
    const int64_t mb = wt ? (d.n_ptiles + kMaxTilesW - 1) / kMaxTilesW : (d.n_ptiles + kMaxTiles - 1) / kMaxTiles;
    const int64_t bn = wt == 1 ? kBNw : kBNn;
    return mb * ((d.C + bn - 1) / bn);
}

// Narrow shapes for the launch's groups: groups of up to 4 packed tiles take
// shape 0, the others shape 1 (their X read once per 8 packed tiles, with as
// many workgroups as two 4-tile M-blocks of 128 columns); while the tiles
// outnumber the CUs, the shape-1 group with the most tiles moves to shape 2
// (half its workgroups, each with twice the columns).  A narrow launch needs
// every group on the same rounds and between half the CUs and all of them
// busy; where a group has 3 or more M-blocks of 4 packed tiles (team slicing
// otherwise), also two rounds of workgroups that keep at least 70% of the
// CUs busy over both (5% rows: 374 tiles, measured faster than team slices).
// Returns false if no such assignment exists.
bool narrow_shapes(const DwParams &p, int cus, int32_t *wt) {
    int64_t n = 0;
    bool same = true, many = false;
    for (int32_t g = 0; g < p.n_groups; ++g) {
        const DwGroupDev &d = p.g[g];
        wt[g] = d.n_ptiles > kMaxTiles ? 1 : 0;
        n += narrow_tiles(d, wt[g]);
        many = many || d.n_ptiles > (kTeamMblk - 1) * kMaxTiles;
        same = same && (d.T + kRound * kBKn - 1) / (kRound * kBKn) ==
                           (p.g[0].T + kRound * kBKn - 1) / (kRound * kBKn);
    }
    while (n > cus) {
        int32_t best = -1;
        for (int32_t g = 0; g < p.n_groups; ++g)
            if (wt[g] == 1 && (best < 0 || narrow_tiles(p.g[g], 1) > narrow_tiles(p.g[best], 1))) best = g;
        if (best < 0) break;
        n += narrow_tiles(p.g[best], 2) - narrow_tiles(p.g[best], 1);
        wt[best] = 2;
    }
    return same && ((n <= cus && 2 * n >= int64_t(cus)) || (many && n <= 2 * cus && 10 * n >= 14 * int64_t(cus)));
}

Plan make_plan(const sft_dw_group *groups, int32_t n_groups, int cus = sft::num_cus()) {
    Plan plan;
    int32_t gi = 0;
    while (gi < n_groups) {
        Launch L;
        DwParams &p = L.p;
        p = DwParams{};
        int32_t nm = 0, ptiles = 0;
        int64_t iters = 0, otiles = 0, min_chunks = INT64_MAX;
        size_t at = 0;
        // Output-tile geometry of the launch's groups: wide (256 columns,
        // 64-token chunks) or narrow (128 columns, 128-token chunks).
        int32_t wt_of[kMaxGroups] = {};
        auto lay = [&](bool narrow) {
            const int64_t bk = narrow ? kBKn : kBK;
            iters = otiles = 0;
            min_chunks = INT64_MAX;
            at = 0;
            L.at_off.clear();
            L.map_off.clear();
            L.gather_blocks = 0;
            for (int32_t g = 0; g < p.n_groups; ++g) {
                DwGroupDev &d = p.g[g];
                d.wt = narrow ? wt_of[g] : 0;
                d.n_mblk = d.wt ? (d.n_ptiles + kMaxTilesW - 1) / kMaxTilesW : (d.n_ptiles + kMaxTiles - 1) / kMaxTiles;
                d.nb_major = !narrow && d.n_mblk >= 3 ? 1 : 0;
                const int64_t bn = d.wt == 1 ? kBNw : narrow ? kBNn : kBN;
                d.n_nblk = static_cast<int32_t>((d.C + bn - 1) / bn);
                d.chunks = static_cast<int32_t>(((d.T + kRound * bk - 1) / (kRound * bk)) * kRound);
                d.Tp = static_cast<int32_t>(d.chunks * bk);
                d.it_begin = iters;
                d.otile_begin = otiles;
                const int64_t ot = int64_t(d.n_mblk) * d.n_nblk;
                otiles += ot;
                iters += ot * d.chunks;
                min_chunks = std::min<int64_t>(min_chunks, d.chunks);
                L.at_off.push_back(at);
                at += round256(size_t(d.n_ptiles) * 32 * size_t(d.Tp) * 2);
                L.map_off.push_back(at);
                at += round256(size_t(d.n_ptiles) * 32 * 4);
                L.gather_blocks = std::max(L.gather_blocks, d.Tp / kGatherTokens);
            }
            p.narrow = narrow ? 1 : 0;
        };
        while (gi < n_groups && p.n_groups < kMaxGroups) {
            const sft_dw_group &g = groups[gi];
            if (!group_live(g)) {
                ++gi;
                continue;
            }
            int32_t live = 0;
            for (int32_t mi = 0; mi < g.n_mats; ++mi) live += g.mats[mi].n_active_tiles ? 1 : 0;
            if (nm + live > kMaxMats) break;
            ++gi;
            DwGroupDev &d = p.g[p.n_groups++];
            d.X = g.X;
            d.T = g.T;
            d.C = g.C;
            d.layout = g.layout;
            d.mat_begin = nm;
            d.n_mats = 0;
            int64_t rows = 0;
            for (int32_t mi = 0; mi < g.n_mats; ++mi) {
                const sft_dw_mat &m = g.mats[mi];
                if (m.n_active_tiles == 0) continue;
                DwMatDev &dm = p.m[nm++];
                ++d.n_mats;
                dm.dY = m.dY;
                dm.rows = m.active_rows;
                dm.tiles = m.active_tiles;
                dm.abits = m.active_bits;
                dm.first = m.tile_first;
                dm.out = m.dW_act;
                dm.R = m.R;
                dm.row_begin = static_cast<int32_t>(rows);
                rows += g.layout == SFT_DW_PACKED ? m.n_active : 32 * m.n_active_tiles;
            }
            d.n_rows = static_cast<int32_t>(rows);
            d.n_ptiles = static_cast<int32_t>((rows + 31) / 32);
            d.n_mblk = (d.n_ptiles + kMaxTiles - 1) / kMaxTiles;
            d.nb_major = d.n_mblk >= 3 ? 1 : 0;
            d.ptile_begin = ptiles;
            ptiles += d.n_ptiles;
        }
        if (p.n_groups == 0) break;
        lay(false);
        if (iters >= (int64_t(1) << 31)) {
            plan.too_big = true;
            break;
        }
        // Slices aligned to the output tiles when that keeps most CUs busy:
        // if every tile has the same number of rounds and f (dividing it) times
        // the tile count fits the CUs with at least 3/4 of them at work, each
        // workgroup takes exactly 1/f of one tile -- every tile cut f ways at
        // the same places, the fewest partial sums for that many workgroups,
        // one segment each, equal work -- with workgroup index = slice (on
        // MI355X this spread of the groups over the XCDs measured faster than
        // keeping neighbouring slices on one XCD).  Otherwise one workgroup per
        // CU over the whole (tile, chunk) space (stream-K), neighbouring
        // slices on one XCD; more workgroups (whole rounds) only if a slice
        // would cross more output tiles than the kernel tracks; never more
        // slices than rounds (so none is empty).  The slice arithmetic runs in
        // fp64 on the GPU, exact while P * Q < 2^53.
        //
        // Team slicing when a group has three or more M-blocks: group g gets
        // n_team teams of n_mblk workgroups, member mb of a team doing
        // M-block mb over the team's range of column-block rounds, so the
        // members read each X chunk together (one XCD, neighbouring slices)
        // and all but the first find it in L2.  Each group starts with the
        // fewest teams whose ranges touch at most kMaxSegs - 1 column blocks;
        // a team is then added, while the CUs last, to the group whose
        // members have the most rounds each (never more teams than rounds).
        int64_t P = 0;
        // Narrow whole tiles first, when the groups' shapes keep at least half
        // of the CUs busy with one workgroup per tile: each workgroup then takes
        // one whole tile over the whole token axis, with no partial sums and no
        // fix-up (the tile halves of the wide shape leave every tile in two
        // partial slots, 16 bytes per element written and read again, where
        // narrow tiles write the 4-byte result once; at 0.5% rows, 182 narrow
        // tiles measured faster than stream-K over all 256 CUs).
        if (narrow_shapes(p, cus, wt_of)) {
            lay(true);
            P = otiles;
        }
        bool teams = false;
        for (int32_t g = 0; g < p.n_groups && !p.narrow; ++g) teams = teams || p.g[g].n_mblk >= kTeamMblk;
        if (teams) {
            int64_t T[kMaxGroups], Qg[kMaxGroups], tot = 0;
            for (int32_t g = 0; g < p.n_groups; ++g) {
                const DwGroupDev &d = p.g[g];
                Qg[g] = int64_t(d.n_nblk) * (d.chunks / kRound);
                T[g] = std::min<int64_t>(Qg[g], (d.n_nblk + kMaxSegs - 3) / (kMaxSegs - 2));
                tot += T[g] * d.n_mblk;
            }
            teams = tot <= cus;
            while (teams) {
                int32_t best = -1;
                for (int32_t g = 0; g < p.n_groups; ++g) {
                    if (T[g] >= Qg[g] || tot + p.g[g].n_mblk > cus) continue;
                    if (best < 0 || Qg[g] * T[best] > Qg[best] * T[g]) best = g;
                }
                if (best < 0) break;
                ++T[best];
                tot += p.g[best].n_mblk;
            }
            if (teams) {
                int32_t wb = 0;
                for (int32_t g = 0; g < p.n_groups; ++g) {
                    p.g[g].wg_begin = wb;
                    p.g[g].n_team = static_cast<int32_t>(T[g]);
                    wb += static_cast<int32_t>(T[g]) * p.g[g].n_mblk;
                }
                P = ((tot + kXcds - 1) / kXcds) * kXcds;   // idle slices up to whole XCDs
            }
        }
        p.teams = teams ? 1 : 0;
        for (int32_t g = 0; g < p.n_groups; ++g)
            p.g[g].keep_x = teams ? (p.g[g].n_mblk >= 2) : p.g[g].nb_major;
        int64_t rt = p.g[0].chunks / kRound;
        for (int32_t g = 1; g < p.n_groups; ++g)
            if (p.g[g].chunks / kRound != rt) rt = 0;
        for (int64_t f = rt; f >= 1 && !teams && !p.narrow; --f) {
            if (rt % f || f * otiles > cus) continue;
            if (4 * f * otiles >= 3 * int64_t(cus)) P = f * otiles;
            break;
        }
        p.xcd_blocked = teams || P == 0;
        if (P == 0) {
            P = cus;
            const int64_t need = (iters + (kMaxSegs - 2) * min_chunks - 1) / ((kMaxSegs - 2) * min_chunks);
            if (need > P) P = ((need + cus - 1) / cus) * cus;
            P = std::min<int64_t>(P, iters / kRound);
            if (P >= kXcds) P -= P % kXcds;
        }
        if (P * (iters / kRound) >= (int64_t(1) << 53)) {
            plan.too_big = true;
            break;
        }
        p.n_wg = static_cast<int32_t>(P);
        p.iters = iters;
        L.out_tiles = otiles;
        L.gather_tiles = ptiles;
        L.at_bytes = at;
        if (!p.narrow)
            plan.part_bytes = std::max(plan.part_bytes, round256(size_t(2 * P) * size_t(kSlotFloats) * sizeof(float)));
        plan.sink_bytes = std::max(plan.sink_bytes, round256(size_t(P) * 8 * 16 * sizeof(float)));
        plan.at_bytes = std::max(plan.at_bytes, at);
        plan.launches.push_back(L);
    }
    return plan;
}

// The product with its X copies' cache policy fixed when every group of the
// launch has the same one.
void launch_product(const DwParams &p, hipStream_t st) {
    bool any = false, all = true;
    for (int32_t g = 0; g < p.n_groups; ++g) {
        any = any || p.g[g].keep_x;
        all = all && p.g[g].keep_x;
    }
    const dim3 grid(static_cast<uint32_t>(p.n_wg)), block(kThreads);
    bool wide_wt = false;
    for (int32_t g = 0; g < p.n_groups; ++g) wide_wt = wide_wt || p.g[g].wt == 2;
    if (p.narrow && wide_wt) {
        if (!any) hipLaunchKernelGGL((k_masked_dw<0, 2>), grid, block, 0, st, p);
        else if (all) hipLaunchKernelGGL((k_masked_dw<1, 2>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((k_masked_dw<2, 2>), grid, block, 0, st, p);
    } else if (p.narrow) {
        if (!any) hipLaunchKernelGGL((k_masked_dw<0, 1>), grid, block, 0, st, p);
        else if (all) hipLaunchKernelGGL((k_masked_dw<1, 1>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((k_masked_dw<2, 1>), grid, block, 0, st, p);
    } else {
        if (!any) hipLaunchKernelGGL((k_masked_dw<0, 0>), grid, block, 0, st, p);
        else if (all) hipLaunchKernelGGL((k_masked_dw<1, 0>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((k_masked_dw<2, 0>), grid, block, 0, st, p);
    }
}

void bind_workspace(Plan &plan, void *ws) {
    uint8_t *base = static_cast<uint8_t *>(ws);
    for (Launch &L : plan.launches) {
        L.p.part = reinterpret_cast<float *>(base);
        L.p.sink = reinterpret_cast<float *>(base + plan.part_bytes);
        uint8_t *at = base + plan.part_bytes + plan.sink_bytes;
        for (int32_t g = 0; g < L.p.n_groups; ++g) {
            L.p.g[g].at = reinterpret_cast<uint16_t *>(at + L.at_off[g]);
            L.p.g[g].rowmap = reinterpret_cast<int32_t *>(at + L.map_off[g]);
        }
    }
}

}  // namespace

namespace sft {

int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int masked_dw_partials(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes, void *stream,
                       DwRowSrc *src, bool *done, bool *whole) {
    *done = false;
    *whole = false;
    if (int rc = validate(groups, n_groups)) return rc;
    Plan plan = make_plan(groups, n_groups);
    SFT_CHECK(!plan.too_big, SFT_ENOTSUP, "sft_masked_dw: a launch beyond 2^31 (tile, chunk) iterations");
    if (plan.launches.size() != 1) return SFT_OK;
    SFT_CHECK(ws_bytes >= plan.ws_bytes(), SFT_ECAPACITY, "sft_masked_dw: workspace %zu < %zu bytes", ws_bytes,
              plan.ws_bytes());
    SFT_CHECK(ws && aligned16(ws), SFT_EINVAL, "sft_masked_dw: workspace null or not 16-byte aligned");
    bind_workspace(plan, ws);
    Launch &L = plan.launches[0];
    L.p.part_rows = 1;
    // the matrices in input order: live groups and their matrices with active
    // tiles were taken in this order by the plan
    int32_t dg = 0, dm = 0, i = 0;
    for (int32_t gi = 0; gi < n_groups; ++gi) {
        const sft_dw_group &g = groups[gi];
        const bool live = group_live(g);
        for (int32_t mi = 0; mi < g.n_mats; ++mi, ++i) {
            DwRowSrc &r = src[i];
            r = DwRowSrc{};
            if (!live || g.mats[mi].n_active_tiles == 0) continue;
            const DwGroupDev &G = L.p.g[dg];
            const DwMatDev &M = L.p.m[dm++];
            r.part = L.p.part;
            r.dW = M.out;
            r.tiles = g.layout == SFT_DW_TILES ? g.mats[mi].active_tiles : nullptr;
            r.n_tiles = g.mats[mi].n_active_tiles;
            r.slot_floats = kSlotFloats;
            r.it_begin = G.it_begin;
            r.P = L.p.n_wg;
            r.Q = L.p.iters / kRound;
            r.bn = kBN;
            r.rnd = kRound;
            r.chunks = G.chunks;
            r.n_nblk = G.n_nblk;
            r.nb_major = G.nb_major;
            r.team = L.p.teams;
            r.wg_begin = G.wg_begin;
            r.n_team = G.n_team;
            r.n_ptiles = G.n_ptiles;
            r.n_mblk = G.n_mblk;
            r.row_begin = M.row_begin;
            r.layout = G.layout;
        }
        if (live) ++dg;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_dw_gather, dim3(static_cast<uint32_t>(L.gather_tiles), static_cast<uint32_t>(L.gather_blocks)),
                       dim3(256), 0, st, L.p);
    hipError_t e = hipGetLastError();
    SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: gather launch failed: %s", hipGetErrorString(e));
    launch_product(L.p, st);
    e = hipGetLastError();
    SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: launch failed: %s", hipGetErrorString(e));
    *done = true;
    *whole = L.p.narrow != 0;
    return SFT_OK;
}

}  // namespace sft

extern "C" {

size_t sft_masked_dw_workspace(const sft_dw_group *groups, int32_t n_groups) {
    sft::clear_error();
    if (validate(groups, n_groups) != SFT_OK) return static_cast<size_t>(-1);
    const Plan plan = make_plan(groups, n_groups);
    if (plan.too_big) {
        sft::fail(SFT_ENOTSUP, "sft_masked_dw: a launch beyond 2^31 (tile, chunk) iterations");
        return static_cast<size_t>(-1);
    }
    return plan.ws_bytes();
}

int sft_probe_dw_plan(const sft_dw_group *groups, int32_t n_groups, int32_t cus, int32_t *out, int32_t cap) {
    sft::clear_error();
    SFT_CHECK(cus >= 0 && cap >= 0 && (cap == 0 || out), SFT_EINVAL, "sft_probe_dw_plan: bad arguments");
    if (int rc = validate(groups, n_groups)) return rc;
    const Plan plan = cus ? make_plan(groups, n_groups, cus) : make_plan(groups, n_groups);
    SFT_CHECK(!plan.too_big, SFT_ENOTSUP, "sft_probe_dw_plan: a launch beyond 2^31 (tile, chunk) iterations");
    int32_t n = 0;
    auto put = [&](int64_t x) {
        if (n < cap) out[n] = static_cast<int32_t>(x);
        ++n;
    };
    for (const Launch &L : plan.launches) {
        const DwParams &p = L.p;
        put(p.narrow ? 3 : p.teams ? 2 : p.xcd_blocked ? 0 : 1);
        put(p.n_wg);
        put(p.n_groups);
        for (int32_t g = 0; g < p.n_groups; ++g) {
            put(p.g[g].wt);
            put(p.g[g].n_mblk);
            put(p.g[g].n_nblk);
        }
    }
    return n;
}

int sft_masked_dw(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes, void *stream) {
    sft::clear_error();
    if (int rc = validate(groups, n_groups)) return rc;
    Plan plan = make_plan(groups, n_groups);
    SFT_CHECK(!plan.too_big, SFT_ENOTSUP, "sft_masked_dw: a launch beyond 2^31 (tile, chunk) iterations");
    if (plan.launches.empty()) return SFT_OK;
    SFT_CHECK(ws_bytes >= plan.ws_bytes(), SFT_ECAPACITY, "sft_masked_dw: workspace %zu < %zu bytes", ws_bytes,
              plan.ws_bytes());
    SFT_CHECK(ws && sft::aligned16(ws), SFT_EINVAL, "sft_masked_dw: workspace null or not 16-byte aligned");
    bind_workspace(plan, ws);
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (const Launch &L : plan.launches) {
        hipLaunchKernelGGL(k_dw_gather, dim3(static_cast<uint32_t>(L.gather_tiles), static_cast<uint32_t>(L.gather_blocks)),
                           dim3(256), 0, st, L.p);
        hipError_t e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: gather launch failed: %s", hipGetErrorString(e));
        launch_product(L.p, st);
        e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: launch failed: %s", hipGetErrorString(e));
        if (L.p.narrow) continue;   // whole tiles only: nothing to add up
        hipLaunchKernelGGL(k_dw_fixup, dim3(static_cast<uint32_t>(L.out_tiles), kMaxTiles), dim3(256), 0, st,
                           L.p);
        e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: fix-up launch failed: %s", hipGetErrorString(e));
    }
    return SFT_OK;
}

int sft_embedding_dw(const uint16_t *dY, int64_t T, int64_t d, const int32_t *row_ptr,
                     const int32_t *positions, int64_t n_active, float *dW_act, void *stream) {
    sft::clear_error();
    SFT_CHECK(T >= 0 && d > 0 && n_active >= 0, SFT_EINVAL, "sft_embedding_dw: bad sizes");
    SFT_CHECK(d % 8 == 0, SFT_ESHAPE, "sft_embedding_dw: d=%lld is not a multiple of 8", (long long)d);
    if (n_active == 0) return SFT_OK;
    SFT_CHECK(dY && row_ptr && positions && dW_act, SFT_EINVAL, "sft_embedding_dw: null pointer");
    SFT_CHECK(sft::aligned16(dY) && sft::aligned16(dW_act), SFT_EALIGN,
              "sft_embedding_dw: dY or dW_act not 16-byte aligned");
    SFT_CHECK(n_active <= 65535, SFT_ENOTSUP, "sft_embedding_dw: more than 65535 active rows");
    const dim3 grid(static_cast<uint32_t>((d + kEmbCols - 1) / kEmbCols), static_cast<uint32_t>(n_active));
    hipLaunchKernelGGL(k_embedding_dw, grid, dim3(kEmbThreads), 0, static_cast<hipStream_t>(stream), dY, d,
                       row_ptr, positions, dW_act);
    const hipError_t e = hipGetLastError();
    SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_embedding_dw: launch failed: %s", hipGetErrorString(e));
    return SFT_OK;
}

}  // extern "C"
