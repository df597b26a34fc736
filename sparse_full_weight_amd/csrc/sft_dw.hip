// sft_dw.hip -- the masked weight gradient dW = dY^T X on the gfx950 matrix
// cores, and the embedding's masked gradient.
//
// Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
// Active Set", section 2.2: the weight gradient of a projection is the
// transposed product of the output gradient and the layer input; the mask is
// checked per tile of 32 output rows, a tile with no active row costs no load,
// no accumulation and no write, and inside an active tile the inactive rows
// are dropped before the final write.  For the embedding the input is one-hot,
// so a row's gradient is the sum of dY over the positions of its token.
//
// Masked dW design (MI355X):
//   * Only active tiles are ever scheduled: the work list is built from the
//     active tile lists, so a skipped tile is never visited.
//   * Matrices that read the same input X (q/k/v; gate/up) form one group; up
//     to 8 active tiles of a group (an M-block of 256 rows) share every load
//     of an X block.  X is the dominant HBM stream at ~1% density and is read
//     once per M-block instead of once per matrix.
//   * Output tiles are (M-block, 128 columns of C); each is a sequence of
//     64-token chunks.  The launch is persistent and stream-K: one 8-wave
//     workgroup per CU takes an equal contiguous slice of the whole
//     (tile, chunk) iteration space, so every CU streams the same number of X
//     bytes whatever the tile counts.  Tiles cut by a slice boundary are
//     written as partial sums to scratch and combined by a second small
//     kernel in slice order (deterministic; the kernel boundary orders the
//     stores, so no device-scope fence is needed -- such a fence writes back
//     and invalidates an XCD's L2, and one per workgroup serialised badly).
//   * Per chunk each lane loads one 8x8 bf16 block (eight 16-byte rows of
//     tokens), transposes it in registers so that tokens (the reduction
//     axis) become contiguous, and stores it to LDS with 16-byte writes.  The
//     LDS row pitch is 9 granules of 16 bytes: the 8 lanes of a store phase
//     (same columns, token groups 0..7) and the 8 lanes of an operand read
//     phase (8 consecutive rows) then hit 8 distinct bank groups.  LDS is
//     double-buffered and two further chunks are in flight in registers.
//   * v_mfma_f32_32x32x16_bf16 consumes 16-byte LDS fragments; wave w owns
//     columns 32*(w%4) and half of the M-block's tiles.
//   * Slices are laid out so that the 32 workgroups of one XCD (the hardware
//     dispatches workgroup i to XCD i mod 8) take neighbouring slices, which
//     share the M-block's dY columns in that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "sft_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const uint16_t gu16;

constexpr int kBN = 128;           // columns per output tile (4 column slices of 32)
constexpr int kMaxTiles = 8;       // 32-row tiles per M-block
constexpr int kBK = 64;            // tokens per chunk
constexpr int kLdk = 72;           // LDS row pitch (elements): 9 granules of 16 B
constexpr int kThreads = 512;      // 8 waves
constexpr int kStageRows = kMaxTiles * 32 + kBN;
constexpr int kStageElems = kStageRows * kLdk;
constexpr int kMaxGroups = 8;
constexpr int kMaxMats = 16;
constexpr int kMaxSegs = 16;       // tiles touched by one slice
constexpr int kXcds = 8;
constexpr int64_t kSlotFloats = int64_t(kMaxTiles) * 32 * kBN;  // one partial tile

struct DwMatDev {
    const uint16_t *dY;
    int64_t R;
    const int32_t *tiles;   // active tiles
    const uint32_t *abits;  // their row bits
    const int32_t *first;   // index of their first active row
    int64_t n_active;
    float *out;
    int32_t n_tiles;
    int32_t tile_begin;  // offset in the group's concatenated tile list
};

struct DwGroupDev {
    const uint16_t *X;
    int64_t T, C;
    int32_t mat_begin, n_mats;
    int32_t n_tiles;     // active 32-row tiles of the group
    int32_t n_mblk, n_nblk, chunks;
    int64_t it_begin;    // first global iteration of this group
    int64_t otile_begin; // first output tile (global numbering)
};

struct DwParams {
    DwGroupDev g[kMaxGroups];
    DwMatDev m[kMaxMats];
    int32_t n_groups;
    int32_t n_wg;        // slices (= workgroups of the main launch)
    int64_t iters;       // total (tile, chunk) iterations
    float *part;         // [2 * n_wg] partial tiles of kSlotFloats
};

struct TileDesc {
    const uint16_t *dY;
    float *out;
    int64_t col0;   // first dY column (= first row of W) of the tile
    uint32_t R;
    uint32_t bits;
    int32_t first;  // index in the matrix's active-row list of the tile's first active row
};

struct Seg {
    int32_t g, mb, nb, mt;
    int32_t k0;     // first chunk of the tile in this slice
    int32_t j0;     // first local iteration of the segment
    int32_t len;    // chunks
    int32_t slot;   // -1: whole tile (final output); else partial slot
};

__device__ __forceinline__ uint4 gload16(const uint16_t *p) {
    const u32x4 v = *reinterpret_cast<gu32x4 *>(reinterpret_cast<uintptr_t>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t gload2(const uint16_t *p) {
    return *reinterpret_cast<gu16 *>(reinterpret_cast<uintptr_t>(p));
}

// 8x8 transpose of bf16: in[i] holds 8 consecutive columns of token row i;
// out[e] holds tokens 0..7 of column e.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t word = (e < 2) ? in[i].x : (e < 4) ? in[i].y : (e < 6) ? in[i].z : in[i].w;
            w[i] = (e & 1) ? (word >> 16) : (word & 0xffffu);
        }
        out[e].x = w[0] | (w[1] << 16);
        out[e].y = w[2] | (w[3] << 16);
        out[e].z = w[4] | (w[5] << 16);
        out[e].w = w[6] | (w[7] << 16);
    }
}

// Descriptor of tile `t` (0..mt-1) of M-block mb of group G.
__device__ TileDesc make_tile_desc(const DwParams &p, const DwGroupDev &G, int32_t mb, int t) {
    const int32_t gt = mb * kMaxTiles + t;
    int mi = G.mat_begin;
    while (mi + 1 < G.mat_begin + G.n_mats && gt >= p.m[mi + 1].tile_begin) ++mi;
    const DwMatDev &M = p.m[mi];
    const int32_t lt = gt - M.tile_begin;
    TileDesc d;
    d.dY = M.dY;
    d.out = M.out;
    d.col0 = 32 * static_cast<int64_t>(M.tiles[lt]);
    d.R = static_cast<uint32_t>(M.R);
    d.bits = M.abits[lt];
    d.first = M.first[lt];
    return d;
}

// Slice of workgroup v: global iterations [lo, hi).  Boundaries fall on
// even iterations (chunk counts are even too), so every segment is a whole
// number of chunk pairs -- the unit of the software pipeline below.
__device__ __forceinline__ int64_t slice_lo(const DwParams &p, int64_t v) {
    return 2 * (v * (p.iters / 2) / p.n_wg);
}

// One lane's share of a chunk: which 8 columns and 8 tokens it loads and
// where the transposed block goes in the stage buffer.  Offsets are 32-bit
// element counts (the host checks T*R and T*C < 2^31).
struct Task {
    const uint16_t *base;     // matrix base; masked-off lanes use X (>= 16 bytes, C % 8 == 0)
    uint32_t col;             // first column of the block (0 for masked-off lanes)
    uint32_t pitch;           // row pitch (elements)
    uint32_t t0;              // first token row
    uint32_t t_last;          // last valid token row (T - 1)
    uint32_t valid_cols;      // columns of the block inside the matrix (0: no task)
    int32_t dst;              // element offset in the stage buffer
};

// What a store needs to know about a block in flight.  The loaded registers
// are never touched before the store: masking them at load time would make
// the compiler wait for the loads right after issuing them.
struct Pending {
    int32_t dst;        // -1: no task
    uint32_t row_ok;    // bit i: token row i of the block is inside the matrix
    uint32_t valid_cols;
};

template <bool kVec>
__device__ __forceinline__ Pending load_task(const Task &k, uint4 (&ld)[8]) {
    Pending pd;
    pd.dst = k.valid_cols ? k.dst : -1;
    pd.valid_cols = k.valid_cols;
    pd.row_ok = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t t = k.t0 + i;
        pd.row_ok |= (t <= k.t_last) ? (1u << i) : 0u;
        // rows past the end re-read the last row; the store masks them
        const uint32_t off = min(t, k.t_last) * k.pitch + k.col;
        if (kVec) {
            ld[i] = gload16(k.base + off);
        } else {
            // rows not 16-byte aligned: element loads (this path packs at once)
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                e[q] = gload2(k.base + off + (static_cast<uint32_t>(q) < k.valid_cols ? q : 0));
            ld[i] = make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                               e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
        }
    }
    return pd;
}

__device__ __forceinline__ void store_task(uint4 (&ld)[8], const Pending &pd, uint16_t *stage) {
    if (pd.dst < 0) return;
    // zero what lies outside the matrix: token rows past T, columns past R
    uint32_t cm[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
        cm[w] = (2u * w < pd.valid_cols ? 0x0000ffffu : 0u) | (2u * w + 1 < pd.valid_cols ? 0xffff0000u : 0u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t rm = ((pd.row_ok >> i) & 1u) ? 0xffffffffu : 0u;
        ld[i].x &= rm & cm[0];
        ld[i].y &= rm & cm[1];
        ld[i].z &= rm & cm[2];
        ld[i].w &= rm & cm[3];
    }
    uint4 tr[8];
    transpose8x8(ld, tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4 *>(stage + pd.dst + e * kLdk) = tr[e];
}

// MFMAs of one chunk for one wave: NT tiles (from tile tb) x 32 columns.
template <int NT>
__device__ __forceinline__ void mma_chunk(const uint16_t *stage, int tb, int wave, int lane,
                                          floatx16 (&acc)[4]) {
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    const uint16_t *bptr = stage + (kMaxTiles * 32 + (wave & 3) * 32 + frag_row) * kLdk + frag_k;
    const uint16_t *aptr = stage + (tb * 32 + frag_row) * kLdk + frag_k;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(bptr + kk * 16);
        bf16x8 a[NT > 0 ? NT : 1];
#pragma unroll
        for (int t = 0; t < NT; ++t) a[t] = *reinterpret_cast<const bf16x8 *>(aptr + t * 32 * kLdk + kk * 16);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], b, acc[t], 0, 0, 0);
    }
}

// ---- shared by both masked-dW kernels -----------------------------------

// The slice's segments (one per tile it touches) and their tile descriptors,
// built once per workgroup into LDS.  Returns the slice's chunk count.
__device__ int32_t build_segments(const DwParams &p, int64_t v, int64_t it_lo, int64_t it_hi, Seg *segs,
                                  TileDesc (*tdesc)[kMaxTiles], int32_t *s_nseg) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        int64_t it = it_lo;
        int n = 0;
        int32_t j = 0;
        while (it < it_hi && n < kMaxSegs) {
            int gi = 0;
            while (gi + 1 < p.n_groups && it >= p.g[gi + 1].it_begin) ++gi;
            const DwGroupDev &G = p.g[gi];
            const int64_t rel = it - G.it_begin;
            const int32_t tile = static_cast<int32_t>(rel / G.chunks);
            const int32_t k0 = static_cast<int32_t>(rel % G.chunks);
            const int64_t tile_end = G.it_begin + static_cast<int64_t>(tile + 1) * G.chunks;
            const int64_t end = min(tile_end, it_hi);
            Seg sg;
            sg.g = gi;
            sg.mb = tile / G.n_nblk;
            sg.nb = tile % G.n_nblk;
            sg.mt = min(kMaxTiles, G.n_tiles - sg.mb * kMaxTiles);
            sg.k0 = k0;
            sg.j0 = j;
            sg.len = static_cast<int32_t>(end - it);
            const bool whole = (k0 == 0 && end == tile_end);
            sg.slot = whole ? -1 : (n == 0 ? static_cast<int32_t>(2 * v) : static_cast<int32_t>(2 * v + 1));
            segs[n++] = sg;
            j += sg.len;
            it = end;
        }
        *s_nseg = n;
    }
    __syncthreads();
    const int nseg = *s_nseg;
    for (int x = tid; x < nseg * kMaxTiles; x += blockDim.x) {
        const int sg = x / kMaxTiles, t = x % kMaxTiles;
        if (t < segs[sg].mt) tdesc[sg][t] = make_tile_desc(p, p.g[segs[sg].g], segs[sg].mb, t);
    }
    __syncthreads();
    return segs[nseg - 1].j0 + segs[nseg - 1].len;
}

// Epilogue of a segment for one wave: nt tiles (from tile tb) x 32 columns.
// Accumulator layout of the 32x32 MFMA: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.  A whole tile goes to dW_act; a
// partial one to its slot, as compact active rows (row c = c-th active row of
// the M-block).  The accumulators are cleared for the next segment.
__device__ __forceinline__ void segment_epilogue(const DwParams &p, const Seg &S, const TileDesc *td, int nt,
                                                 int tb, int wave, int lane, floatx16 (&acc)[4]) {
    const DwGroupDev &G = p.g[S.g];
    const int cl = (wave & 3) * 32 + (lane & 31);        // column inside the tile
    const int64_t col = static_cast<int64_t>(S.nb) * kBN + cl;
    const int row_base = 4 * (lane >> 5);
    int prefix = 0;                                       // active rows of tiles before tb
    for (int t = 0; t < tb; ++t) prefix += __builtin_popcount(td[t].bits);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (t < nt) {
            const TileDesc &d = td[tb + t];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + row_base + (r & 3);
                if ((d.bits >> i) & 1u) {
                    const int below = __builtin_popcount(d.bits & ((1u << i) - 1u));
                    if (S.slot < 0) {
                        if (col < G.C) d.out[static_cast<int64_t>(d.first + below) * G.C + col] = acc[t][r];
                    } else {
                        p.part[S.slot * kSlotFloats + (prefix + below) * kBN + cl] = acc[t][r];
                    }
                }
            }
            prefix += __builtin_popcount(d.bits);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    }
}

// Slice of workgroup b: the 32 workgroups of an XCD take neighbouring slices.
__device__ __forceinline__ int64_t slice_of(const DwParams &p) {
    const int64_t b = blockIdx.x;
    return (p.n_wg % kXcds == 0) ? (b % kXcds) * (p.n_wg / kXcds) + b / kXcds : b;
}

// ---- register-staged kernel: rows of dY that are not 16-byte aligned ------
// (R % 8 != 0).  Each lane loads an 8x8 block into registers (element loads),
// transposes it and writes it to LDS.

template <bool kVecA>
__global__ __launch_bounds__(kThreads, 1) void k_masked_dw_reg(const DwParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t stage[2][kStageElems];
    __shared__ Seg segs[kMaxSegs];
    __shared__ TileDesc tdesc[kMaxSegs][kMaxTiles];
    __shared__ int32_t s_nseg;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t v = slice_of(p);
    const int64_t it_lo = slice_lo(p, v), it_hi = slice_lo(p, v + 1);
    if (it_lo >= it_hi) return;
    const int32_t J = build_segments(p, v, it_lo, it_hi, segs, tdesc, &s_nseg);
    const int nseg = s_nseg;

    // ---- this lane's load task for local iteration j
    const int tg = tid & 7;   // token group: the 8 lanes of a store phase cover tokens 0..63
    const int cg = tid >> 3;  // column group (8 columns)
    // j lies in segment s0 or in one of the next two (lookahead is at most 4
    // chunks and segments are at least 2 long); no loop here, so that the
    // compiler keeps exact counts of the loads in flight.
    auto make_task = [&](int32_t j, int s0) {
        int s = s0;
        s += (s + 1 < nseg && j >= segs[s + 1].j0) ? 1 : 0;
        s += (s + 1 < nseg && j >= segs[s + 1].j0) ? 1 : 0;
        const Seg &S = segs[s];
        const DwGroupDev &G = p.g[S.g];
        Task k;
        k.base = G.X;
        k.col = 0;
        k.pitch = 0;
        k.t_last = static_cast<uint32_t>(G.T) - 1;
        k.t0 = static_cast<uint32_t>(S.k0 + (j - S.j0)) * kBK + tg * 8;
        k.valid_cols = 0;
        k.dst = -1;
        if (j < J) {
            if (cg < 4 * S.mt) {
                const TileDesc &d = tdesc[s][cg >> 2];
                const uint32_t col = static_cast<uint32_t>(d.col0) + (cg & 3) * 8;
                if (col < d.R) {
                    k.base = d.dY;
                    k.col = col;
                    k.pitch = d.R;
                    k.valid_cols = min(8u, d.R - col);
                    k.dst = (cg * 8) * kLdk + tg * 8;
                }
            } else if (cg < 4 * S.mt + kBN / 8) {
                const int cb = cg - 4 * S.mt;
                const uint32_t col = static_cast<uint32_t>(S.nb) * kBN + cb * 8;
                if (col < static_cast<uint32_t>(G.C)) {
                    k.col = col;
                    k.pitch = static_cast<uint32_t>(G.C);
                    k.valid_cols = 8;
                    k.dst = (kMaxTiles * 32 + cb * 8) * kLdk + tg * 8;
                }
            }
        }
        return k;
    };

    floatx16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

    // ---- software pipeline, one chunk pair at a time: both chunks of a pair
    // are transposed into the two stage buffers, then the loads of the next
    // pair are issued, then both chunks are multiplied while those loads are
    // in flight.  Loads are issued unconditionally (past the end of the slice
    // they read a safe address and are masked), and sched_barrier keeps every
    // group of loads in place, so the only wait on loads is the one at the
    // stores, which needs them all.
    uint4 ld0[8], ld1[8];
    Pending pd0 = load_task<kVecA>(make_task(0, 0), ld0);
    __builtin_amdgcn_sched_barrier(0);
    Pending pd1 = load_task<kVecA>(make_task(1, 0), ld1);
    __builtin_amdgcn_sched_barrier(0);

    auto pairs = [&](auto nt_tag, int tb, int seg, int32_t j, int32_t n) {
        constexpr int NT = decltype(nt_tag)::value;
        for (int32_t c = 0; c < n; c += 2, j += 2) {
            store_task(ld0, pd0, stage[0]);
            store_task(ld1, pd1, stage[1]);
            __builtin_amdgcn_sched_barrier(0);
            pd0 = load_task<kVecA>(make_task(j + 2, seg), ld0);
            __builtin_amdgcn_sched_barrier(0);
            pd1 = load_task<kVecA>(make_task(j + 3, seg), ld1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            mma_chunk<NT>(stage[0], tb, wave, lane, acc);
            mma_chunk<NT>(stage[1], tb, wave, lane, acc);
            __syncthreads();
        }
    };

    for (int s = 0; s < nseg; ++s) {
        const Seg &S = segs[s];
        const int half = wave >> 2;
        const int nt = half ? S.mt / 2 : (S.mt + 1) / 2;   // this wave's tiles
        const int tb = half ? (S.mt + 1) / 2 : 0;
        switch (nt) {
            // Two loop bodies only (more instantiations make the register
            // allocator spill): a wave with fewer tiles multiplies rows it
            // then ignores -- cheap, as such blocks are bound by HBM anyway.
            case 0:
            case 1:
            case 2: pairs(std::integral_constant<int, 2>{}, tb, s, S.j0, S.len); break;
            default: pairs(std::integral_constant<int, 4>{}, tb, s, S.j0, S.len); break;
        }
        segment_epilogue(p, S, tdesc[s], nt, tb, wave, lane, acc);
    }
}

// ---- DMA kernel (every dY row 16-byte aligned, the common case) ----------
//
// Chunks go from HBM straight into a 3-stage LDS ring with the gfx950
// global_load_lds_dwordx4 (lane l's 16 bytes land at base + 16*l), without
// passing through registers, so two chunks are always in flight.  The MFMA
// operands are read from the untransposed [token][column] layout with
// ds_read_b64_tr_b16: in each group of 16 lanes, output lane 4a+b receives
// element b of source lane 4e+a as its element e; when the 16 lanes point at
// a 4-token x 16-column block, lane i receives column i for 4 consecutive
// tokens, and two such reads give the 32x32x16 operand of a lane (column
// l%32, tokens 8*(l/32) + 0..7).
//
// Stage layout (48 KB): 8 dY tiles x [64 tokens][32 columns] (4 KB each),
// then X as [64 tokens][128 columns] (16 KB) with the 16-byte column groups
// of token row r stored at group g ^ (2*(r%4)), which makes the transposing
// reads of 4 consecutive rows hit distinct banks.  Lanes outside the
// matrices (tokens >= T, columns >= R or C) copy 16 zero bytes.
//
// Per chunk j each wave: waits for its own copies of chunk j (vmcnt), joins a
// barrier (all copies of chunk j landed; all reads of chunk j-1 finished),
// issues the copies of chunk j+2 into the stage of chunk j-1, then multiplies
// chunk j.  The waits are explicit (s_waitcnt with an immediate count) and the
// barrier is a bare s_barrier: __syncthreads() carries a release fence that
// would wait for every copy in flight.

constexpr int kStages = 3;
constexpr int kStageBytes = 48 * 1024;
constexpr int kXOff = kMaxTiles * 4096;   // byte offset of the X block in a stage

__device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0, 0, 0, 0};

typedef short short4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const __attribute__((address_space(1))) void *>(reinterpret_cast<uintptr_t>(src)),
        reinterpret_cast<__attribute__((address_space(3))) void *>(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds))),
        16, 0, 0);
}

// Wave-uniform copies of values every lane holds alike (so that they live in
// scalar registers and buffer resources need no per-lane loop).
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// 16 bytes per lane from a raw buffer [base, base + size) at byte offset
// voff into LDS at lds + 16*lane; offsets at or beyond size read as zero.
__device__ __forceinline__ void dma16_buf(const uint8_t *base, int32_t size, uint32_t voff, void *lds) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), static_cast<short>(0), size, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, reinterpret_cast<__attribute__((address_space(3))) void *>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds))),
        16, voff, 0, 0, 0);
}

__device__ __forceinline__ short4v lds_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) short4v *>(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p))));
}

// s_waitcnt vmcnt(n) leaving the other counters free (gfx9 encoding).
#define SFT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
// s_waitcnt lgkmcnt(0) leaving vmcnt and expcnt free.
#define SFT_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 0: SFT_WAIT_VMCNT(0); break;
        case 1: SFT_WAIT_VMCNT(1); break;
        case 2: SFT_WAIT_VMCNT(2); break;
        case 3: SFT_WAIT_VMCNT(3); break;
        case 4: SFT_WAIT_VMCNT(4); break;
        case 5: SFT_WAIT_VMCNT(5); break;
        default: SFT_WAIT_VMCNT(6); break;
    }
}

// Copies one wave issues for a chunk of an M-block of mt tiles: the chunk is
// 4*mt + 16 copies of 1 KB, dealt round-robin to the 8 waves.
__device__ __forceinline__ int copies_of_wave(int mt, int wave) { return (4 * mt + 16 - wave + 7) / 8; }

// MFMAs of one chunk for one wave: NT tiles (from tile tb) x 32 columns.
// after_step(kk) runs after the MFMAs of k-step kk are issued: the caller
// issues the next chunks' copies there, so that the vector-memory pipe and
// the matrix cores work at the same time.
template <int NT, typename AfterStep>
__device__ __forceinline__ void mma_chunk_tr(const uint8_t *st, int tb, int wave, int lane, floatx16 (&acc)[4],
                                             AfterStep after_step) {
    const int s16 = lane & 15;
    const int half_col = ((lane >> 4) & 1) * 16;          // 16-column half of the 32
    const int trow = 8 * (lane >> 5) + (s16 >> 2);          // token row inside a k-step, before +4h
    const int c4 = 4 * (s16 & 3);
    const uint16_t *A = reinterpret_cast<const uint16_t *>(st);
    const uint16_t *X = reinterpret_cast<const uint16_t *>(st + kXOff);
    // X: logical column = 32*(wave%4) + half_col + c4, group g = column / 8,
    // stored at group g ^ (2*(row%4)); row%4 = s16 >> 2 for every row read here.
    const int xcol = 32 * (wave & 3) + half_col + c4;
    const int xoff = 8 * ((xcol >> 3) ^ (2 * (s16 >> 2))) + (xcol & 7);
    const uint16_t *Ab = A + tb * 2048 + half_col + c4;
    auto frags = [&](int kk, bf16x8 &b, bf16x8 (&a)[NT > 0 ? NT : 1]) {
        const int r0 = 16 * kk + trow;                      // tokens r0 (h = 0) and r0 + 4 (h = 1)
        const short4v blo = lds_tr16(X + r0 * kBN + xoff);
        const short4v bhi = lds_tr16(X + (r0 + 4) * kBN + xoff);
        b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const short4v lo = lds_tr16(Ab + t * 2048 + r0 * 32);
            const short4v hi = lds_tr16(Ab + t * 2048 + (r0 + 4) * 32);
            a[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    bf16x8 b_cur, a_cur[NT > 0 ? NT : 1];
    frags(0, b_cur, a_cur);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
        bf16x8 b_nxt, a_nxt[NT > 0 ? NT : 1];
        if (kk + 1 < kBK / 16) frags(kk + 1, b_nxt, a_nxt);   // next k-step's fragments in flight
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_cur[t], b_cur, acc[t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        after_step(kk);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < kBK / 16) {
            b_cur = b_nxt;
#pragma unroll
            for (int t = 0; t < NT; ++t) a_cur[t] = a_nxt[t];
        }
    }
}

__global__ __launch_bounds__(kThreads, 1) void k_masked_dw_dma(const DwParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * kStageBytes];
    __shared__ Seg segs[kMaxSegs];
    __shared__ TileDesc tdesc[kMaxSegs][kMaxTiles];
    __shared__ int32_t s_nseg;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t v = slice_of(p);
    const int64_t it_lo = slice_lo(p, v), it_hi = slice_lo(p, v + 1);
    if (it_lo >= it_hi) return;
    const int32_t J = build_segments(p, v, it_lo, it_hi, segs, tdesc, &s_nseg);
    const int nseg = s_nseg;

    // Copies of local chunk j (segment hint s0: j is in s0 or the next segment).
    // Returns the number of copies this wave issued.
    auto issue = [&](int32_t j, int s0) -> int {
        if (j >= J) return 0;
        int sg = s0;
        sg += (sg + 1 < nseg && j >= segs[sg + 1].j0) ? 1 : 0;
        const Seg &S = segs[sg];
        const DwGroupDev &G = p.g[S.g];
        const uint32_t T = static_cast<uint32_t>(G.T);
        const uint32_t t0 = static_cast<uint32_t>(S.k0 + (j - S.j0)) * kBK;
        uint8_t *st = ring + (j % kStages) * kStageBytes;
        const int nq = 4 * S.mt + 16;
        int n = 0;
        for (int q = wave; q < nq; q += 8, ++n) {
            const void *src = g_zero16;
            uint8_t *dst;
            if (q < 4 * S.mt) {
                // dY tile q/4, token rows 16*(q%4) + lane/4, 16-byte quarter lane%4
                const TileDesc &d = tdesc[sg][q >> 2];
                const uint32_t row = t0 + 16 * (q & 3) + (lane >> 2);
                const int64_t col = d.col0 + 8 * (lane & 3);
                if (row < T && col < d.R) src = d.dY + static_cast<uint64_t>(row) * d.R + col;
                dst = st + (q >> 2) * 4096 + (q & 3) * 1024;
            } else {
                // X rows 4*b + lane/16; lane's slot lane%16 holds column group (lane%16) ^ 2*(row%4)
                const int bq = q - 4 * S.mt;
                const uint32_t row = t0 + 4 * bq + (lane >> 4);
                const int grp = (lane & 15) ^ (2 * (lane >> 4));
                const int64_t col = static_cast<int64_t>(S.nb) * kBN + 8 * grp;
                if (row < T && col < G.C) src = G.X + static_cast<uint64_t>(row) * static_cast<uint64_t>(G.C) + col;
                dst = st + kXOff + bq * 1024;
            }
            dma16(src, dst);   // lane l lands at dst + 16*l
        }
        return n;
    };

    // Per-segment copy descriptors of this wave.  Each copy reads through a
    // buffer resource whose base and size advance by one chunk per chunk
    // (scalar work only); a lane's offset inside the chunk is fixed for the
    // segment.  Rows past T fall beyond the resource's size and columns past
    // R or C get an offset beyond any size, so the hardware range check turns
    // them into zeros.
    constexpr int kMaxCopies = (4 * kMaxTiles + 16 + 7) / 8;   // per wave and chunk
    constexpr uint32_t kOutside = 0x80000000u;                   // >= every resource size
    const uint8_t *cp_base[kMaxCopies];   // uniform: chunk 0 of the segment
    int64_t cp_rem[kMaxCopies];           // uniform: bytes from cp_base to the end of the matrix
    int64_t cp_stride[kMaxCopies];        // uniform: bytes per chunk
    uint32_t cp_dst[kMaxCopies];          // uniform: byte offset in the stage
    uint32_t cp_voff[kMaxCopies];         // per lane: byte offset inside the chunk
    int n_cp = 0;
    auto describe = [&](int sg) {
        const Seg &S = segs[sg];
        const DwGroupDev &G = p.g[S.g];
        const int64_t T = G.T;
        const int64_t r0 = static_cast<int64_t>(S.k0) * kBK;
        const int nq = 4 * S.mt + 16;
        n_cp = 0;
#pragma unroll
        for (int k = 0; k < kMaxCopies; ++k) {
            const int q = wave + 8 * k;
            cp_base[k] = reinterpret_cast<const uint8_t *>(G.X);
            cp_rem[k] = 0;
            cp_stride[k] = 0;
            cp_dst[k] = 0;
            cp_voff[k] = kOutside;
            if (q < nq) {
                ++n_cp;
                if (q < 4 * S.mt) {
                    const TileDesc &d = tdesc[sg][q >> 2];
                    const int64_t R = d.R;
                    const int row_in = 16 * (q & 3) + (lane >> 2);
                    const int col_in = 8 * (lane & 3);
                    cp_base[k] = reinterpret_cast<const uint8_t *>(d.dY + r0 * R + d.col0);
                    cp_rem[k] = (T - r0) * R * 2 - d.col0 * 2;
                    cp_stride[k] = static_cast<int64_t>(kBK) * R * 2;
                    cp_dst[k] = (q >> 2) * 4096 + (q & 3) * 1024;
                    if (d.col0 + col_in < R) cp_voff[k] = static_cast<uint32_t>((row_in * R + col_in) * 2);
                } else {
                    const int bq = q - 4 * S.mt;
                    const int64_t C = G.C;
                    const int64_t c0 = static_cast<int64_t>(S.nb) * kBN;
                    const int row_in = 4 * bq + (lane >> 4);
                    const int grp = (lane & 15) ^ (2 * (lane >> 4));   // X swizzle
                    cp_base[k] = reinterpret_cast<const uint8_t *>(G.X + r0 * C + c0);
                    cp_rem[k] = (T - r0) * C * 2 - c0 * 2;
                    cp_stride[k] = static_cast<int64_t>(kBK) * C * 2;
                    cp_dst[k] = kXOff + bq * 1024;
                    if (c0 + 8 * grp < C) cp_voff[k] = static_cast<uint32_t>((row_in * C + 8 * grp) * 2);
                }
            }
            cp_base[k] = reinterpret_cast<const uint8_t *>(uniform64(reinterpret_cast<uint64_t>(cp_base[k])));
            cp_rem[k] = static_cast<int64_t>(uniform64(static_cast<uint64_t>(cp_rem[k])));
            cp_stride[k] = static_cast<int64_t>(uniform64(static_cast<uint64_t>(cp_stride[k])));
            cp_dst[k] = __builtin_amdgcn_readfirstlane(cp_dst[k]);
        }
        n_cp = __builtin_amdgcn_readfirstlane(n_cp);
    };
    // Copies [k_lo, k_hi) of chunk c (0-based inside the described segment) into stage `st`.
    auto issue_fast = [&](int32_t c, uint8_t *st, int k_lo, int k_hi) -> int {
#pragma unroll
        for (int k = 0; k < kMaxCopies; ++k) {
            if (k >= k_lo && k < k_hi && k < n_cp) {
                const int64_t off = static_cast<int64_t>(c) * cp_stride[k];
                const int64_t rem = cp_rem[k] - off;
                const int32_t size = static_cast<int32_t>(rem <= 0 ? 0 : (rem > 0x7fffffff ? 0x7fffffff : rem));
                dma16_buf(cp_base[k] + off, size, cp_voff[k], st + cp_dst[k]);
            }
        }
        return n_cp;
    };

    floatx16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

    int n_next = issue(0, 0);      // copies of chunk j+1 still allowed in flight at the wait
    n_next = issue(1, 0);
    auto run = [&](auto nt_tag, int tb, int sg, int32_t j0, int32_t len) {
        constexpr int NT = decltype(nt_tag)::value;
        for (int32_t j = j0; j < j0 + len; ++j) {
            // chunk j landed for this wave (only chunk j+1's copies may remain), and
            // every read of chunk j-1 done; then the whole workgroup agrees.
            SFT_WAIT_LGKM0();
            wait_vmcnt(n_next);
            __builtin_amdgcn_s_barrier();
            uint8_t *st2 = ring + ((j + 2) % kStages) * kStageBytes;
            const bool fast = j + 2 < j0 + len;
            if (!fast) n_next = issue(j + 2, sg);   // crosses into the next segment (rare)
            // copies of chunk j+2 spread over the four k-steps: 2, 2, 1, 1
            mma_chunk_tr<NT>(ring + (j % kStages) * kStageBytes, tb, wave, lane, acc, [&](int kk) {
                if (!fast) return;
                const int lo = kk < 2 ? 2 * kk : kk + 2, hi = kk < 2 ? 2 * kk + 2 : kk + 3;
                issue_fast(j + 2 - j0, st2, lo, hi);
            });
            if (fast) n_next = n_cp;
        }
    };
    for (int sg = 0; sg < nseg; ++sg) {
        const Seg &S = segs[sg];
        describe(sg);
        const int half = wave >> 2;
        const int nt = half ? S.mt / 2 : (S.mt + 1) / 2;   // this wave's tiles
        const int tb = half ? (S.mt + 1) / 2 : 0;
        switch (nt) {
            case 0:
            case 1:
            case 2: run(std::integral_constant<int, 2>{}, tb, sg, S.j0, S.len); break;
            default: run(std::integral_constant<int, 4>{}, tb, sg, S.j0, S.len); break;
        }
        segment_epilogue(p, S, tdesc[sg], nt, tb, wave, lane, acc);
    }
}

// Combination of the partial tiles: an output tile cut by slice boundaries
// is the sum of its slices' partial rows, added in slice order.  One
// workgroup per (tile, 8 compact rows); a lane adds 4 columns.
__global__ __launch_bounds__(256) void k_dw_fixup(const DwParams p) {
    const int64_t ot = blockIdx.x;
    int gi = 0;
    while (gi + 1 < p.n_groups && ot >= p.g[gi + 1].otile_begin) ++gi;
    const DwGroupDev &G = p.g[gi];
    const int32_t tile = static_cast<int32_t>(ot - G.otile_begin);
    const int64_t A = G.it_begin + static_cast<int64_t>(tile) * G.chunks;   // first iteration
    const int64_t B = A + G.chunks;                                           // one past the last
    // slices covering [A, B): slice v starts at 2*floor(v*PI/P), PI = iters/2
    // (A and B are even)
    const int64_t PI = p.iters / 2, P = p.n_wg;
    const int64_t v_first = ((A / 2 + 1) * P - 1) / PI;
    const int64_t v_last = ((B / 2) * P - 1) / PI;
    if (v_first == v_last) return;  // the tile lies inside one slice: written directly
    const int32_t mb = tile / G.n_nblk, nb = tile % G.n_nblk;
    const int32_t mt = min(kMaxTiles, G.n_tiles - mb * kMaxTiles);
    __shared__ TileDesc td[kMaxTiles];
    __shared__ int32_t pre[kMaxTiles + 1];
    if (threadIdx.x < mt) td[threadIdx.x] = make_tile_desc(p, G, mb, threadIdx.x);
    __syncthreads();
    if (threadIdx.x == 0) {
        pre[0] = 0;
        for (int t = 0; t < mt; ++t) pre[t + 1] = pre[t] + __builtin_popcount(td[t].bits);
    }
    __syncthreads();
    const int c = blockIdx.y * 8 + (threadIdx.x >> 5);   // compact active row of the M-block
    if (c >= pre[mt]) return;
    const int cl = (threadIdx.x & 31) * 4;                // first of this lane's 4 columns
    const int64_t col = static_cast<int64_t>(nb) * kBN + cl;
    if (col >= G.C) return;
    int t = 0;
    while (t + 1 < mt && c >= pre[t + 1]) ++t;
    const int64_t k = td[t].first + (c - pre[t]);        // output row in dW_act
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t vv = v_first; vv <= v_last; ++vv) {
        const int64_t slot = (slice_lo(p, vv) >= A) ? 2 * vv : 2 * vv + 1;
        const float4 x = *reinterpret_cast<const float4 *>(p.part + slot * kSlotFloats + c * kBN + cl);
        if (vv == v_first) {
            sum = x;
        } else {
            sum.x += x.x;
            sum.y += x.y;
            sum.z += x.z;
            sum.w += x.w;
        }
    }
    *reinterpret_cast<float4 *>(td[t].out + k * G.C + col) = sum;
}

// ---------------------------------------------------------------- embedding

constexpr int kEmbThreads = 1024;  // 16 waves split a row's positions
constexpr int kEmbCols = 512;      // columns per workgroup: 64 lanes x 8

__global__ __launch_bounds__(kEmbThreads) void k_embedding_dw(const uint16_t *__restrict__ dY,
                                                              int64_t d,
                                                              const int32_t *__restrict__ row_ptr,
                                                              const int32_t *__restrict__ positions,
                                                              float *__restrict__ dW_act) {
    __shared__ double part[kEmbThreads / 64][kEmbCols];
    const int64_t k = blockIdx.y;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kEmbCols;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col = c0 + lane * 8;
    const int32_t lo = row_ptr[k], hi = row_ptr[k + 1];
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col < d) {
        for (int32_t i = lo + wave; i < hi; i += kEmbThreads / 64) {
            const int64_t t = positions[i];
            const uint4 v = *reinterpret_cast<const uint4 *>(dY + t * d + col);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
                acc[e] += static_cast<double>(__uint_as_float(bits));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave][lane * 8 + e] = acc[e];
    __syncthreads();
    // Fixed-order combination of the 16 wave partials (fp64), one rounding.
    for (int c = threadIdx.x; c < kEmbCols; c += kEmbThreads) {
        if (c0 + c >= d) continue;
        double s = part[0][c];
        for (int w = 1; w < kEmbThreads / 64; ++w) s += part[w][c];
        dW_act[k * d + c0 + c] = static_cast<float>(s);
    }
}

// ---------------------------------------------------------------- host side

struct Plan {
    std::vector<DwParams> launches;
    std::vector<int64_t> out_tiles;
    size_t ws_bytes = 0;
};

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

int validate(const sft_dw_group *groups, int32_t n_groups) {
    SFT_CHECK(n_groups >= 0 && (n_groups == 0 || groups), SFT_EINVAL, "sft_masked_dw: bad group list");
    for (int32_t gi = 0; gi < n_groups; ++gi) {
        const sft_dw_group &g = groups[gi];
        SFT_CHECK(g.n_mats >= 0 && (g.n_mats == 0 || g.mats), SFT_EINVAL,
                  "sft_masked_dw: group %d has a bad matrix list", gi);
        SFT_CHECK(g.n_mats <= kMaxMats, SFT_ENOTSUP, "sft_masked_dw: group %d has more than %d matrices",
                  gi, kMaxMats);
        int64_t tiles = 0;
        for (int32_t mi = 0; mi < g.n_mats; ++mi) tiles += g.mats[mi].n_active_tiles;
        if (tiles == 0) continue;
        SFT_CHECK(g.T >= 1 && g.T < (int64_t(1) << 31) && g.C > 0, SFT_EINVAL,
                  "sft_masked_dw: group %d has T=%lld C=%lld", gi, (long long)g.T, (long long)g.C);
        SFT_CHECK(g.C % 8 == 0, SFT_ESHAPE, "sft_masked_dw: C=%lld is not a multiple of 8", (long long)g.C);
        SFT_CHECK(g.X && sft::aligned16(g.X), g.X ? SFT_EALIGN : SFT_EINVAL,
                  "sft_masked_dw: group %d X null or not 16-byte aligned", gi);
        for (int32_t mi = 0; mi < g.n_mats; ++mi) {
            const sft_dw_mat &m = g.mats[mi];
            SFT_CHECK(m.R > 0 && m.R < (int64_t(1) << 31) && m.n_active >= 0 && m.n_active_tiles >= 0,
                      SFT_EINVAL, "sft_masked_dw: matrix %d/%d has bad sizes", gi, mi);
            SFT_CHECK(m.n_active_tiles <= (m.R + 31) / 32 && m.n_active <= m.R &&
                          m.n_active >= m.n_active_tiles && (m.n_active == 0) == (m.n_active_tiles == 0),
                      SFT_EINVAL, "sft_masked_dw: matrix %d/%d has inconsistent counts", gi, mi);
            if (m.n_active_tiles == 0) continue;
            SFT_CHECK(m.dY && m.active_tiles && m.active_bits && m.tile_first && m.dW_act, SFT_EINVAL,
                      "sft_masked_dw: matrix %d/%d has a null pointer", gi, mi);
            SFT_CHECK(g.T * m.R < (int64_t(1) << 31) && g.T * g.C < (int64_t(1) << 31), SFT_ENOTSUP,
                      "sft_masked_dw: matrix %d/%d: T*R or T*C reaches 2^31 elements", gi, mi);
            SFT_CHECK(sft::aligned16(m.dY) && sft::aligned16(m.dW_act), SFT_EALIGN,
                      "sft_masked_dw: matrix %d/%d dY or dW_act not 16-byte aligned", gi, mi);
        }
    }
    return SFT_OK;
}

// Launch decomposition, shared by the workspace query and the launch.
Plan make_plan(const sft_dw_group *groups, int32_t n_groups, void *ws) {
    Plan plan;
    const int cus = num_cus();
    int32_t gi = 0;
    while (gi < n_groups) {
        DwParams p{};
        int32_t nm = 0;
        int64_t iters = 0, otiles = 0, min_chunks = INT64_MAX;
        while (gi < n_groups && p.n_groups < kMaxGroups) {
            const sft_dw_group &g = groups[gi];
            int32_t live_mats = 0;
            int64_t tiles = 0;
            for (int32_t mi = 0; mi < g.n_mats; ++mi)
                if (g.mats[mi].n_active_tiles) {
                    ++live_mats;
                    tiles += g.mats[mi].n_active_tiles;
                }
            if (tiles == 0) {
                ++gi;
                continue;
            }
            if (nm + live_mats > kMaxMats) break;
            ++gi;
            DwGroupDev &d = p.g[p.n_groups++];
            d.X = g.X;
            d.T = g.T;
            d.C = g.C;
            d.mat_begin = nm;
            d.n_mats = 0;
            int32_t tb = 0;
            for (int32_t mi = 0; mi < g.n_mats; ++mi) {
                const sft_dw_mat &m = g.mats[mi];
                if (m.n_active_tiles == 0) continue;
                DwMatDev &dm = p.m[nm++];
                ++d.n_mats;
                dm.dY = m.dY;
                dm.R = m.R;
                dm.tiles = m.active_tiles;
                dm.abits = m.active_bits;
                dm.first = m.tile_first;
                dm.n_active = m.n_active;
                dm.out = m.dW_act;
                dm.n_tiles = static_cast<int32_t>(m.n_active_tiles);
                dm.tile_begin = tb;
                tb += dm.n_tiles;
            }
            d.n_tiles = tb;
            d.n_mblk = (tb + kMaxTiles - 1) / kMaxTiles;
            d.n_nblk = static_cast<int32_t>((g.C + kBN - 1) / kBN);
            d.chunks = static_cast<int32_t>(((g.T + 2 * kBK - 1) / (2 * kBK)) * 2);  // even
            d.it_begin = iters;
            d.otile_begin = otiles;
            const int64_t ot = int64_t(d.n_mblk) * d.n_nblk;
            otiles += ot;
            iters += ot * d.chunks;
            min_chunks = std::min<int64_t>(min_chunks, d.chunks);
        }
        if (p.n_groups == 0) break;
        // One workgroup per CU; more (whole rounds) only if a slice would cross
        // more tiles than the kernel tracks; never more slices than iterations.
        int64_t P = cus;
        const int64_t need = (iters + (kMaxSegs - 2) * min_chunks - 1) / ((kMaxSegs - 2) * min_chunks);
        if (need > P) P = ((need + cus - 1) / cus) * cus;
        P = std::min<int64_t>(P, iters / 2);
        if (P >= kXcds) P -= P % kXcds;
        p.n_wg = static_cast<int32_t>(P);
        p.iters = iters;
        plan.launches.push_back(p);
        plan.out_tiles.push_back(otiles);
        plan.ws_bytes = std::max(plan.ws_bytes, size_t(2 * P) * size_t(kSlotFloats) * sizeof(float));
    }
    for (DwParams &p : plan.launches) p.part = static_cast<float *>(ws);
    return plan;
}

}  // namespace

extern "C" {

size_t sft_masked_dw_workspace(const sft_dw_group *groups, int32_t n_groups) {
    sft::clear_error();
    if (validate(groups, n_groups) != SFT_OK) return static_cast<size_t>(-1);
    return make_plan(groups, n_groups, nullptr).ws_bytes;
}

int sft_masked_dw(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes, void *stream) {
    sft::clear_error();
    if (int rc = validate(groups, n_groups)) return rc;
    Plan plan = make_plan(groups, n_groups, ws);
    SFT_CHECK(ws_bytes >= plan.ws_bytes, SFT_ECAPACITY, "sft_masked_dw: workspace %zu < %zu bytes",
              ws_bytes, plan.ws_bytes);
    SFT_CHECK(plan.ws_bytes == 0 || (ws && sft::aligned16(ws)), SFT_EINVAL,
              "sft_masked_dw: workspace null or not 16-byte aligned");
    bool all_vec = true;
    for (int32_t gi = 0; gi < n_groups; ++gi)
        for (int32_t mi = 0; mi < groups[gi].n_mats; ++mi)
            if (groups[gi].mats[mi].n_active_tiles && groups[gi].mats[mi].R % 8) all_vec = false;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (size_t li = 0; li < plan.launches.size(); ++li) {
        const DwParams &p = plan.launches[li];
        const dim3 grid(static_cast<uint32_t>(p.n_wg));
        if (all_vec)
            hipLaunchKernelGGL(k_masked_dw_dma, grid, dim3(kThreads), 0, st, p);
        else
            hipLaunchKernelGGL(k_masked_dw_reg<false>, grid, dim3(kThreads), 0, st, p);
        hipError_t e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: launch failed: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(k_dw_fixup, dim3(static_cast<uint32_t>(plan.out_tiles[li]), kMaxTiles * 32 / 8), dim3(256),
                           0, st, p);
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
