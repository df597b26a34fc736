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
//   * Only active tiles are ever scheduled: the grid is built from the active
//     tile lists, so a skipped tile is never even visited.
//   * Matrices that read the same input X (q/k/v; gate/up) form one group; up
//     to 8 active tiles of a group (256 rows) share every load of an X block,
//     which is what makes the product cheap at ~1% density: X is the dominant
//     HBM stream and is read once per group instead of once per matrix.
//   * A workgroup (4 wave64s) owns an M-block of up to 8 tiles x 128 columns
//     of C and a range of tokens.  Per 64-token chunk each lane loads 8x8
//     bf16 blocks (eight 16-byte rows), transposes them in registers so that
//     tokens (the reduction axis) become contiguous, and writes them to LDS
//     with 16-byte stores; the MFMA v_mfma_f32_32x32x16_bf16 then reads its
//     operand fragments as 16-byte LDS loads.  The next chunk's global loads
//     are in flight while the current chunk is multiplied.
//   * Few active tiles means few workgroups, so the token axis is split
//     (split-K) until the launch fills the 256 CUs.  Partial tiles go to a
//     workspace; the last workgroup of a tile to arrive (an atomic counter)
//     adds all partials in split order, so the result does not depend on
//     timing, and resets the counter for the next call.
//   * Units are ordered so that consecutive ones, which share the same dY
//     slice, land on the same XCD (its private L2): the hardware dispatches
//     workgroup i to XCD i mod 8, and unit = (i mod 8) * per_xcd + i / 8.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "sft_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 32;              // tokens per chunk
constexpr int kBN = 128;             // columns per N-block (4 waves x 32)
constexpr int kMaxTiles = 8;         // 32-row tiles per M-block
constexpr int kLdk = kBK + 8;        // LDS pitch (elements): 80-B rows keep 16-B fragment reads conflict-free
constexpr int kThreads = 256;
constexpr int kMaxGroups = 8;
constexpr int kMaxMats = 16;
constexpr int kXcds = 8;
constexpr int64_t kPartStride = int64_t(kMaxTiles) * 32 * kBN;  // floats per partial tile

struct DwMatDev {
    const uint16_t *dY;
    int64_t R;
    const uint32_t *bits;
    const int32_t *rows;
    const int32_t *tiles;
    int64_t n_active;
    float *out;
    int32_t n_tiles;
    int32_t tile_begin;  // offset in the group's concatenated tile list
    int32_t vec;         // R % 8 == 0: 16-byte loads of dY
};

struct DwGroupDev {
    const uint16_t *X;
    int64_t T, C;
    int32_t mat_begin, n_mats;
    int32_t n_tiles, n_mblk, n_nblk, n_split, chunks;
    int64_t unit_begin;      // first unit of this group
    int64_t out_tile_begin;  // first (mblock, nblock) output tile of this group (counter index)
    int64_t part_offset;     // floats: this group's partial tiles in the workspace
};

struct DwParams {
    DwGroupDev g[kMaxGroups];
    DwMatDev m[kMaxMats];
    int32_t n_groups;
    int64_t n_units;
    int64_t per_xcd;
    uint32_t *counters;  // [output tiles of the call], zero between calls
    float *partials;     // per split group: [mblk*nblk][n_split][kPartStride]
};

struct TileDesc {
    const uint16_t *dY;
    int64_t R;
    float *out;
    int64_t col0;   // first dY column (= first row of W) of the tile
    uint32_t bits;
    int32_t first;  // index in the matrix's active-row list of the tile's first active row
    int32_t vec;
};

// First index k with rows[k] >= key.
__device__ __forceinline__ int32_t lower_bound_rows(const int32_t *rows, int64_t n, int64_t key) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (rows[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    return static_cast<int32_t>(lo);
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

template <bool kVecA>
__global__ __launch_bounds__(kThreads, 2) void k_masked_dw(const DwParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t As[kMaxTiles * 32 * kLdk];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdk];
    __shared__ TileDesc tdesc[kMaxTiles];
    __shared__ int32_t s_last;

    // ---- which unit: XCD-contiguous order
    const int64_t b = blockIdx.x;
    const int64_t unit = (b % kXcds) * p.per_xcd + b / kXcds;
    if (unit >= p.n_units) return;
    int gi = 0;
    while (gi + 1 < p.n_groups && unit >= p.g[gi + 1].unit_begin) ++gi;
    const DwGroupDev &G = p.g[gi];
    int64_t u = unit - G.unit_begin;
    const int32_t nb = static_cast<int32_t>(u % G.n_nblk);
    u /= G.n_nblk;
    const int32_t sp = static_cast<int32_t>(u % G.n_split);
    const int32_t mb = static_cast<int32_t>(u / G.n_split);
    const int32_t t_lo = mb * kMaxTiles;
    const int32_t mt = min(kMaxTiles, G.n_tiles - t_lo);
    const int64_t n0 = static_cast<int64_t>(nb) * kBN;
    const int32_t c_begin = static_cast<int32_t>((static_cast<int64_t>(sp) * G.chunks) / G.n_split);
    const int32_t c_end = static_cast<int32_t>((static_cast<int64_t>(sp + 1) * G.chunks) / G.n_split);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (tid < mt) {
        const int32_t gt = t_lo + tid;
        int mi = G.mat_begin;
        while (mi + 1 < G.mat_begin + G.n_mats && gt >= p.m[mi + 1].tile_begin) ++mi;
        const DwMatDev &M = p.m[mi];
        const int32_t j = M.tiles[gt - M.tile_begin];
        TileDesc d;
        d.dY = M.dY;
        d.R = M.R;
        d.out = M.out;
        d.col0 = 32 * static_cast<int64_t>(j);
        d.bits = M.bits[j];
        d.first = lower_bound_rows(M.rows, M.n_active, d.col0);
        d.vec = M.vec;
        tdesc[tid] = d;
    }
    __syncthreads();

    const int64_t T = G.T, C = G.C;
    const uint16_t *X = G.X;
    // One 8x8 (8 columns x 8 tokens) block per lane and chunk: the A side has
    // mt tiles x 4 column groups x 4 token groups, the B side 16 x 4.
    const int n_a = 16 * mt;
    const int n_tasks = n_a + 64;
    const int task = tid;
    const bool has_task = task < n_tasks;
    const int tg = task & 3;  // token group fastest: LDS stores spread over banks
    const bool is_a = task < n_a;
    const int cg = is_a ? (task >> 2) : ((task - n_a) >> 2);
    // Element offsets fit 32 bits (the host checks T*R and T*C < 2^31).
    const uint16_t *src_base;
    uint32_t src_pitch;
    bool col_ok;
    uint32_t valid_cols = 8;  // unaligned dY rows: columns of the granule inside R
    if (is_a) {
        const TileDesc &d = tdesc[cg >> 2];
        const int64_t col = d.col0 + (cg & 3) * 8;
        src_base = d.dY + col;
        src_pitch = static_cast<uint32_t>(d.R);
        col_ok = col < d.R;
        if (!kVecA && col_ok) valid_cols = static_cast<uint32_t>(min<int64_t>(8, d.R - col));
    } else {
        const int64_t col = n0 + cg * 8;
        src_base = X + col;
        src_pitch = static_cast<uint32_t>(C);
        col_ok = col < C;
    }
    uint16_t *lds_dst = (is_a ? As : Bs) + (cg * 8) * kLdk + tg * 8;

    uint4 ld[8];
    auto load_chunk = [&](int32_t chunk) {
        const uint32_t t0 = static_cast<uint32_t>(chunk) * kBK + tg * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t t = t0 + i;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (has_task && col_ok && t < T) {
                const uint16_t *src = src_base + t * src_pitch;
                if (kVecA || !is_a) {
                    v = *reinterpret_cast<const uint4 *>(src);
                } else {
                    uint16_t e[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) e[q] = (static_cast<uint32_t>(q) < valid_cols) ? src[q] : 0;
                    v.x = e[0] | (uint32_t(e[1]) << 16);
                    v.y = e[2] | (uint32_t(e[3]) << 16);
                    v.z = e[4] | (uint32_t(e[5]) << 16);
                    v.w = e[6] | (uint32_t(e[7]) << 16);
                }
            }
            ld[i] = v;
        }
    };
    auto store_chunk = [&]() {
        if (!has_task) return;
        uint4 tr[8];
        transpose8x8(ld, tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4 *>(lds_dst + e * kLdk) = tr[e];
    };

    floatx16 acc[kMaxTiles];
#pragma unroll
    for (int tm = 0; tm < kMaxTiles; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tm][r] = 0.0f;

    const int frag_row = lane & 31;           // row (A) / column (B) of the fragment
    const int frag_k = (lane >> 5) * 8;       // first of the lane's 8 tokens
    if (c_begin < c_end) load_chunk(c_begin);
    for (int32_t chunk = c_begin; chunk < c_end; ++chunk) {
        __syncthreads();
        store_chunk();
        __syncthreads();
        if (chunk + 1 < c_end) load_chunk(chunk + 1);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const bf16x8 bfrag = *reinterpret_cast<const bf16x8 *>(
                Bs + (wave * 32 + frag_row) * kLdk + kk * 16 + frag_k);
#pragma unroll
            for (int tm = 0; tm < kMaxTiles; ++tm) {
                if (tm < mt) {
                    const bf16x8 afrag = *reinterpret_cast<const bf16x8 *>(
                        As + (tm * 32 + frag_row) * kLdk + kk * 16 + frag_k);
                    acc[tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, bfrag, acc[tm], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue.  Accumulator layout of the 32x32 MFMA: lane l, register r
    // holds row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the tile.
    const int64_t col = n0 + wave * 32 + (lane & 31);
    const int row_base = 4 * (lane >> 5);
    if (G.n_split == 1) {
#pragma unroll
        for (int tm = 0; tm < kMaxTiles; ++tm) {
            if (tm >= mt) continue;
            const TileDesc &d = tdesc[tm];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + row_base + (r & 3);
                if (((d.bits >> i) & 1u) && col < C) {
                    const int k = d.first + __builtin_popcount(d.bits & ((1u << i) - 1u));
                    d.out[static_cast<int64_t>(k) * C + col] = acc[tm][r];
                }
            }
        }
        return;
    }

    // split-K: publish the partial tile, count arrivals, the last one reduces.
    const int64_t out_tile = G.out_tile_begin + static_cast<int64_t>(mb) * G.n_nblk + nb;
    float *part = p.partials + G.part_offset +
                  (static_cast<int64_t>(mb) * G.n_nblk + nb) * G.n_split * kPartStride;
    const int pcol = wave * 32 + (lane & 31);
#pragma unroll
    for (int tm = 0; tm < kMaxTiles; ++tm) {
        if (tm >= mt) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + row_base + (r & 3);
            part[sp * kPartStride + (tm * 32 + i) * kBN + pcol] = acc[tm][r];
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(p.counters + out_tile, 1u);
        s_last = (prev == static_cast<uint32_t>(G.n_split - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int tm = 0; tm < kMaxTiles; ++tm) {
        if (tm >= mt) continue;
        const TileDesc &d = tdesc[tm];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + row_base + (r & 3);
            float sum = 0.0f;
            for (int s = 0; s < G.n_split; ++s) {
                const float v = (s == sp) ? acc[tm][r]
                                          : __builtin_nontemporal_load(
                                                part + s * kPartStride + (tm * 32 + i) * kBN + pcol);
                sum = (s == 0) ? v : sum + v;
            }
            if (((d.bits >> i) & 1u) && col < C) {
                const int k = d.first + __builtin_popcount(d.bits & ((1u << i) - 1u));
                d.out[static_cast<int64_t>(k) * C + col] = sum;
            }
        }
    }
    if (tid == 0) atomicExch(p.counters + out_tile, 0u);
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
    std::vector<int64_t> grid;
    size_t cnt_bytes = 0;
    size_t ws_bytes = 0;
};

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
            SFT_CHECK(m.dY && m.tile_bits && m.active_rows && m.active_tiles && m.dW_act, SFT_EINVAL,
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
Plan make_plan(const sft_dw_group *groups, int32_t n_groups) {
    Plan plan;
    struct G {
        const sft_dw_group *g;
        int64_t tiles, mblk, nblk, chunks;
    };
    std::vector<G> live;
    int64_t pairs = 0;
    for (int32_t gi = 0; gi < n_groups; ++gi) {
        int64_t tiles = 0;
        for (int32_t mi = 0; mi < groups[gi].n_mats; ++mi) tiles += groups[gi].mats[mi].n_active_tiles;
        if (tiles == 0) continue;
        G g{&groups[gi], tiles, (tiles + kMaxTiles - 1) / kMaxTiles, (groups[gi].C + kBN - 1) / kBN,
            (groups[gi].T + kBK - 1) / kBK};
        pairs += g.mblk * g.nblk;
        live.push_back(g);
    }
    if (live.empty()) return plan;
    // Split the token axis until ~2 workgroups per CU exist (two fit at once),
    // keeping at least 4 chunks (256 tokens) per split.
    const int64_t target = 2 * 256;
    int64_t max_chunks = 0;
    for (const G &g : live) max_chunks = std::max(max_chunks, g.chunks);
    int64_t split = std::max<int64_t>(1, (target + pairs - 1) / pairs);
    split = std::min(split, std::max<int64_t>(1, max_chunks / 4));

    size_t part_floats = 0;
    int64_t out_tiles = 0;
    size_t gidx = 0;
    while (gidx < live.size()) {
        DwParams p{};
        int64_t units = 0;
        int32_t nm = 0;
        while (gidx < live.size() && p.n_groups < kMaxGroups &&
               nm + live[gidx].g->n_mats <= kMaxMats) {
            const G &g = live[gidx++];
            DwGroupDev &d = p.g[p.n_groups++];
            d.X = g.g->X;
            d.T = g.g->T;
            d.C = g.g->C;
            d.mat_begin = nm;
            d.n_mats = 0;
            int32_t tb = 0;
            for (int32_t mi = 0; mi < g.g->n_mats; ++mi) {
                const sft_dw_mat &m = g.g->mats[mi];
                if (m.n_active_tiles == 0) continue;
                DwMatDev &dm = p.m[nm++];
                ++d.n_mats;
                dm.dY = m.dY;
                dm.R = m.R;
                dm.bits = m.tile_bits;
                dm.rows = m.active_rows;
                dm.tiles = m.active_tiles;
                dm.n_active = m.n_active;
                dm.out = m.dW_act;
                dm.n_tiles = static_cast<int32_t>(m.n_active_tiles);
                dm.tile_begin = tb;
                dm.vec = (m.R % 8 == 0) ? 1 : 0;
                tb += dm.n_tiles;
            }
            d.n_tiles = tb;
            d.n_mblk = static_cast<int32_t>(g.mblk);
            d.n_nblk = static_cast<int32_t>(g.nblk);
            d.chunks = static_cast<int32_t>(g.chunks);
            d.n_split = static_cast<int32_t>(std::min<int64_t>(split, g.chunks));
            d.unit_begin = units;
            d.out_tile_begin = out_tiles;
            d.part_offset = static_cast<int64_t>(part_floats);
            units += g.mblk * g.nblk * d.n_split;
            if (d.n_split > 1) part_floats += size_t(g.mblk * g.nblk) * d.n_split * kPartStride;
            out_tiles += g.mblk * g.nblk;
        }
        p.n_units = units;
        p.per_xcd = (units + kXcds - 1) / kXcds;
        plan.launches.push_back(p);
        plan.grid.push_back(p.per_xcd * kXcds);
    }
    // Workspace: counters for every output tile (256-B aligned), then partials.
    plan.cnt_bytes = ((size_t(out_tiles) * 4 + 255) / 256) * 256;
    plan.ws_bytes = part_floats == 0 ? 0 : plan.cnt_bytes + part_floats * sizeof(float);
    return plan;
}

}  // namespace

extern "C" {

size_t sft_masked_dw_workspace(const sft_dw_group *groups, int32_t n_groups) {
    sft::clear_error();
    if (validate(groups, n_groups) != SFT_OK) return static_cast<size_t>(-1);
    return make_plan(groups, n_groups).ws_bytes;
}

int sft_masked_dw(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes, void *stream) {
    sft::clear_error();
    if (int rc = validate(groups, n_groups)) return rc;
    Plan plan = make_plan(groups, n_groups);
    SFT_CHECK(ws_bytes >= plan.ws_bytes, SFT_ECAPACITY, "sft_masked_dw: workspace %zu < %zu bytes",
              ws_bytes, plan.ws_bytes);
    bool all_vec = true;
    for (int32_t gi = 0; gi < n_groups; ++gi)
        for (int32_t mi = 0; mi < groups[gi].n_mats; ++mi)
            if (groups[gi].mats[mi].n_active_tiles && groups[gi].mats[mi].R % 8) all_vec = false;
    SFT_CHECK(plan.ws_bytes == 0 || (ws && sft::aligned16(ws)), SFT_EINVAL,
              "sft_masked_dw: workspace null or not 16-byte aligned");
    uint32_t *counters = plan.ws_bytes ? static_cast<uint32_t *>(ws) : nullptr;
    float *partials =
        plan.ws_bytes ? reinterpret_cast<float *>(static_cast<char *>(ws) + plan.cnt_bytes) : nullptr;
    for (size_t li = 0; li < plan.launches.size(); ++li) {
        DwParams &p = plan.launches[li];
        p.counters = counters;
        p.partials = partials;
        SFT_CHECK(plan.grid[li] < (int64_t(1) << 31), SFT_ENOTSUP, "sft_masked_dw: grid too large");
        if (all_vec)
            hipLaunchKernelGGL(k_masked_dw<true>, dim3(static_cast<uint32_t>(plan.grid[li])), dim3(kThreads),
                               0, static_cast<hipStream_t>(stream), p);
        else
            hipLaunchKernelGGL(k_masked_dw<false>, dim3(static_cast<uint32_t>(plan.grid[li])), dim3(kThreads),
                               0, static_cast<hipStream_t>(stream), p);
        const hipError_t e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_masked_dw: launch failed: %s", hipGetErrorString(e));
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
