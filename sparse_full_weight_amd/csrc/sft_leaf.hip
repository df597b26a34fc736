// sft_leaf.hip -- gradients and Adam step of K selected connections, for
// gfx950.
//
// Method: the blog post "SparseLeaf: synaptic sparse fine-tuning"
// (di-zhang-llm.github.io).  A fixed support of K coordinates (i_k, j_k) of a
// frozen m x n weight carries trainable increments theta.  For Y = X W^T and
// D = dL/dY the backward pass gives each increment the dot product over token
// positions of column i_k of D and column j_k of X, written into a length-K
// buffer (section "Weight gradients: write the selected results directly");
// the increments then take Adam's step coordinate by coordinate, starting
// from theta = m = v = 0 (section "The optimizer"), with an fp32 master copy,
// fp32 moments and a bf16 copy for computation (the post's tensor ledger).
//
// Gradient kernel shape: every coordinate needs one column of D and one of X
// over all tokens, and a support spread over the matrix touches every cache
// line of both, so the kernel reads each token row of D and X once per pass:
// a workgroup takes a range of tokens, stages a few token pairs' full rows of
// D and X in LDS (16-byte coalesced loads, two tokens of a column in one
// dword) and lets each lane add, for its coordinates, one bf16 dot2 per token
// pair.  The lane's coordinates (packed row/column indices) and their
// accumulators stay in registers for the whole token range, up to 28 per lane
// (28672 per workgroup); matrices with more coordinates take several passes,
// each re-reading its rows.  Each workgroup leaves one partial sum per
// coordinate; a second kernel adds the partials of the token ranges in a
// fixed order, so the result does not depend on timing.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "sft_internal.h"

namespace {

constexpr int kLeafThreads = 1024;                   // 16 waves: 4 a SIMD to cover LDS latency
constexpr int kLeafMats = 16;                        // matrices per launch (kernel-argument size)
constexpr int kLeafStageWords = 16384;               // 64 KB of LDS: one dword = one column of two tokens
constexpr int kLeafMaxPairs = 4;                     // token pairs staged at once
constexpr int kLeafSlots = 4;                        // 16-byte chunk pairs a lane stages per batch
constexpr int kLeafAccs[] = {12, 16, 20, 24, 28};    // coordinates per lane and pass the kernel is built for

struct LeafMatDev {
    const uint16_t *D;
    const uint16_t *X;
    const int32_t *rows;
    const int32_t *cols;
    float *part;          // [S x K] partial sums, token range s at row s
    float *grad;          // [K]
    int64_t m, n, K;
    int64_t wg_begin;     // first workgroup of this matrix
    int32_t S;            // token ranges
    int32_t P;            // coordinate passes of kAcc * kLeafThreads coordinates
    int32_t tp;           // token pairs per LDS batch
    int32_t slot[kLeafSlots];   // per lane slot: pair | (1 << 8 if X) | (chunk step << 16), or -1
};

struct LeafParams {
    LeafMatDev mat[kLeafMats];
    int32_t n_mats;
    int64_t T;
};

__device__ __forceinline__ float bf16_bits(uint32_t h) { return __uint_as_float(h << 16); }

// A native 16-byte vector: an array of these stays in registers, where an
// array of the HIP uint4 struct was kept in scratch memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Workgroup (matrix, token range s, coordinate pass p).  Lane l owns
// coordinates k = p*kAcc*1024 + a*1024 + l, a = 0..kAcc-1.
//
// LDS holds tp token pairs: D as [pair][m] and X as [pair][n] dwords, the
// dword of (pair, column) holding that column's bf16 values of the pair's two
// tokens, so one 32-bit read per operand and one bf16 dot2 add two tokens'
// products to a coordinate.  Staging: lane l loads 16-byte chunks (8 columns)
// of both rows of a pair, chunk l + 1024u of D's or X's rows as the slot table
// says, interleaves them (v_perm) into 8 dwords and writes them as 32
// contiguous bytes.  A pair past the token range is zero; so is the second
// token of a pair that has only one.  The next batch is loaded into registers
// while the current one is multiplied.
template <int kAcc>
__global__ __launch_bounds__(kLeafThreads) void k_leaf_grad(const LeafParams p) {
    __shared__ __attribute__((aligned(16))) uint32_t stage[kLeafStageWords];
    const int64_t wg = blockIdx.x;
    int mi = 0;
    while (mi + 1 < p.n_mats && wg >= p.mat[mi + 1].wg_begin) ++mi;
    const LeafMatDev &M = p.mat[mi];
    const int64_t local = wg - M.wg_begin;
    const int64_t s = local % M.S, pass = local / M.S;
    const int64_t t_lo = s * p.T / M.S, t_hi = (s + 1) * p.T / M.S;
    const int tid = threadIdx.x;
    const int64_t m = M.m, n = M.n, K = M.K;
    const int tp = M.tp;
    const int64_t k0 = pass * int64_t(kAcc) * kLeafThreads + tid;

    // coordinates: row in the high half, column in the low half (m, n <= 65536).
    // Buffer loads with the coordinate's offset in a scalar register (one
    // vector offset for all of them, no per-load address registers); past K
    // they read 0, a valid index whose sum is never stored.
    const int32_t kbytes = static_cast<int32_t>(K * 4);
    const __amdgpu_buffer_rsrc_t rrows =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(M.rows), static_cast<short>(0), kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rcols =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(M.cols), static_cast<short>(0), kbytes, 0x00020000);
    const int32_t vo = tid * 4;
    const int32_t so = static_cast<int32_t>(pass * int64_t(kAcc) * kLeafThreads * 4);
    uint32_t idx[kAcc];
    float acc[kAcc];
#pragma unroll
    for (int a = 0; a < kAcc; ++a)
        idx[a] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rrows, vo, so + a * kLeafThreads * 4, 0))
                 << 16;
#pragma unroll
    for (int a = 0; a < kAcc; ++a) {
        idx[a] |= static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rcols, vo, so + a * kLeafThreads * 4, 0));
        acc[a] = 0.0f;
    }

    // the lane's staging slots (fixed for the matrix): chunk c of rows
    // (2*pair, 2*pair + 1) of the batch, of D or of X
    const int64_t m8 = m / 8, n8 = n / 8;
    int32_t c_of[kLeafSlots];   // < 2^31: m/8, n/8 <= 8192
    int pair_of[kLeafSlots], is_x[kLeafSlots];
    bool live[kLeafSlots];
#pragma unroll
    for (int q = 0; q < kLeafSlots; ++q) {
        const int32_t d = M.slot[q];
        pair_of[q] = d & 0xff;
        is_x[q] = (d >> 8) & 1;
        c_of[q] = tid + (d >> 16) * kLeafThreads;
        live[q] = d >= 0 && c_of[q] < (is_x[q] ? n8 : m8);
    }
    u32x4 lo[kLeafSlots], hi[kLeafSlots];
    auto fetch = [&](int64_t t0) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < kLeafSlots; ++q) {
            const int64_t r0 = t0 + 2 * pair_of[q], r1 = r0 + 1;
            const uint16_t *base = is_x[q] ? M.X : M.D;
            const int64_t len = is_x[q] ? n : m;
            // loads always (clamped to row t_lo, chunk 0); out-of-range halves become zero below
            const bool ok0 = live[q] && r0 < t_hi, ok1 = live[q] && r1 < t_hi;
            lo[q] = *reinterpret_cast<const u32x4 *>(base + (ok0 ? r0 * len + 8 * c_of[q] : t_lo * len));
            hi[q] = *reinterpret_cast<const u32x4 *>(base + (ok1 ? r1 * len + 8 * c_of[q] : t_lo * len));
            if (!ok0) lo[q] = u32x4{0, 0, 0, 0};
            if (!ok1) hi[q] = u32x4{0, 0, 0, 0};
        }
    };
    auto put = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < kLeafSlots; ++q) {
            if (!live[q]) continue;
            // dword 2e: column 2e of both tokens; dword 2e+1: column 2e+1
            u32x4 w0, w1;
            w0.x = __builtin_amdgcn_perm(hi[q].x, lo[q].x, 0x05040100u);
            w0.y = __builtin_amdgcn_perm(hi[q].x, lo[q].x, 0x07060302u);
            w0.z = __builtin_amdgcn_perm(hi[q].y, lo[q].y, 0x05040100u);
            w0.w = __builtin_amdgcn_perm(hi[q].y, lo[q].y, 0x07060302u);
            w1.x = __builtin_amdgcn_perm(hi[q].z, lo[q].z, 0x05040100u);
            w1.y = __builtin_amdgcn_perm(hi[q].z, lo[q].z, 0x07060302u);
            w1.z = __builtin_amdgcn_perm(hi[q].w, lo[q].w, 0x05040100u);
            w1.w = __builtin_amdgcn_perm(hi[q].w, lo[q].w, 0x07060302u);
            uint32_t *dst = stage + (is_x[q] ? tp * m + pair_of[q] * n : pair_of[q] * m) + 8 * c_of[q];
            reinterpret_cast<u32x4 *>(dst)[0] = w0;
            reinterpret_cast<u32x4 *>(dst)[1] = w1;
        }
    };

    const uint32_t *const sd = stage;            // [tp][m]
    const uint32_t *const sx = stage + tp * m;   // [tp][n]
    const int64_t batch = 2 * int64_t(tp);
    if (t_lo < t_hi) fetch(t_lo);
    for (int64_t t0 = t_lo; t0 < t_hi; t0 += batch) {
        __syncthreads();   // the previous batch has been read
        put();
        __syncthreads();
        const int pairs = static_cast<int>((t_hi - t0 + 1) / 2 < tp ? (t_hi - t0 + 1) / 2 : tp);
        if (t0 + batch < t_hi) fetch(t0 + batch);   // in flight while this batch is multiplied
        // pair by pair, every coordinate of the lane: a coordinate costs its
        // packed index and its accumulator across the loop (the empty asm
        // makes the index opaque at each pair, so the compiler unpacks it
        // there rather than keeping every coordinate's unpacked offsets live)
        for (int r = 0; r < pairs; ++r) {
            const uint32_t *const dr = sd + r * m;
            const uint32_t *const xr = sx + r * n;
#pragma unroll
            for (int a = 0; a < kAcc; ++a) {
                uint32_t w = idx[a];
                asm volatile("" : "+v"(w));
                acc[a] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, dr[w >> 16]),
                                                         __builtin_bit_cast(bf16x2, xr[w & 0xffffu]), acc[a], false);
            }
        }
    }
#pragma unroll
    for (int a = 0; a < kAcc; ++a) {
        const int64_t k = k0 + int64_t(a) * kLeafThreads;
        if (k < K) M.part[s * K + k] = acc[a];
    }
}

// g[k] = sum over token ranges s = 0..S-1 of part[s][k], in that order.
__global__ __launch_bounds__(256) void k_leaf_reduce(const LeafParams p) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    int mi = 0;
    int64_t base = 0;
    while (mi < p.n_mats && gid >= base + p.mat[mi].K) {
        base += p.mat[mi].K;
        ++mi;
    }
    if (mi >= p.n_mats) return;
    const LeafMatDev &M = p.mat[mi];
    const int64_t k = gid - base;
    float g = 0.0f;
    for (int32_t s = 0; s < M.S; ++s) g += M.part[s * M.K + k];
    M.grad[k] = g;
}

// SparseLeaf Adam, one lane per coordinate; the same fp32 rounding steps as
// the row update (no weight decay, which this step does not have).
struct LeafVecDev {
    const float *grad;
    float *theta, *m, *v;
    uint16_t *theta_bf16;
    int64_t K;
    int64_t begin;        // first coordinate of this vector in the launch
};

struct LeafAdamParams {
    LeafVecDev vec[kLeafMats];
    int32_t n_vecs;
    int32_t step;
    float lr, beta1, beta2, eps, c1, c2;
    const float *bc1, *bc2;
};

__global__ __launch_bounds__(256) void k_leaf_adam(const LeafAdamParams p) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    int vi = 0;
    while (vi + 1 < p.n_vecs && gid >= p.vec[vi + 1].begin) ++vi;
    const LeafVecDev &V = p.vec[vi];
    const int64_t k = gid - V.begin;
    if (k >= V.K) return;
    const float bc1 = p.bc1[p.step], bc2 = p.bc2[p.step];
    const float g = V.grad[k];
    const float m_a = p.beta1 * V.m[k];
    const float m_b = p.c1 * g;
    const float mk = m_a + m_b;
    const float gg = g * g;
    const float v_a = p.beta2 * V.v[k];
    const float v_b = p.c2 * gg;
    const float vk = v_a + v_b;
    const float mhat = mk / bc1;
    const float vhat = vk / bc2;
    const float denom = __builtin_sqrtf(vhat) + p.eps;
    const float ratio = mhat / denom;
    const float u = p.lr * ratio;
    const float th = V.theta[k] - u;
    V.m[k] = mk;
    V.v[k] = vk;
    V.theta[k] = th;
    if (V.theta_bf16) V.theta_bf16[k] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(th));
}

struct LeafPlan {
    std::vector<LeafParams> launches;
    std::vector<int> acc;            // kAcc of each launch
    std::vector<int64_t> wgs;        // workgroups of each launch
    std::vector<int64_t> coords;     // coordinates of each launch (reduce grid)
    size_t ws_bytes = 0;
};

constexpr size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int check_leaf(const sft_leaf_mat *mats, int32_t n_mats, int64_t T, const char *who) {
    SFT_CHECK(n_mats >= 0 && (n_mats == 0 || mats), SFT_EINVAL, "%s: bad matrix list", who);
    SFT_CHECK(T >= 0, SFT_EINVAL, "%s: T < 0", who);
    for (int32_t i = 0; i < n_mats; ++i) {
        const sft_leaf_mat &L = mats[i];
        SFT_CHECK(L.m > 0 && L.n > 0 && L.K >= 0, SFT_EINVAL, "%s: matrix %d: bad sizes", who, i);
        SFT_CHECK(L.m % 8 == 0 && L.n % 8 == 0, SFT_ESHAPE, "%s: matrix %d: m and n must be multiples of 8", who, i);
        SFT_CHECK(L.m <= 65536 && L.n <= 65536 && L.m + L.n <= kLeafStageWords, SFT_ENOTSUP,
                  "%s: matrix %d: m=%lld n=%lld beyond m, n <= 65536 and m + n <= %d", who, i, (long long)L.m,
                  (long long)L.n, kLeafStageWords);
        SFT_CHECK(L.K < (int64_t(1) << 29), SFT_ENOTSUP, "%s: matrix %d: K >= 2^29", who, i);
        if (L.K == 0) continue;
        SFT_CHECK(L.rows && L.cols && L.grad && (T == 0 || (L.dY && L.X)), SFT_EINVAL,
                  "%s: matrix %d: null device pointer", who, i);
        SFT_CHECK(T == 0 || (sft::aligned16(L.dY) && sft::aligned16(L.X)), SFT_EALIGN,
                  "%s: matrix %d: dY or X not 16-byte aligned", who, i);
    }
    return SFT_OK;
}

// Decomposition: coordinates per pass kAcc*1024, kAcc one of kLeafAccs (28
// is the most that fit the 128 registers of a 1024-lane workgroup without
// spilling), the one with the least work over the launch: every lane works
// all kAcc of its coordinate slots whether or not they hold a coordinate, so
// a matrix costs passes x kAcc slots per token pair, plus its staging; token
// ranges per matrix in proportion to that cost (passes x (staged row length
// / 4 + kAcc*1024) per token), about one workgroup per CU in all, each range
// at least one LDS batch long.
LeafPlan leaf_plan(const sft_leaf_mat *mats, int32_t n_mats, int64_t T) {
    LeafPlan plan;
    const int cus = sft::num_cus();
    int32_t i = 0;
    size_t ws = 0;
    while (i < n_mats) {
        LeafParams p{};
        p.T = T;
        std::vector<int32_t> idx;
        while (i < n_mats && static_cast<int32_t>(idx.size()) < kLeafMats) {
            if (mats[i].K > 0) idx.push_back(i);
            ++i;
        }
        if (idx.empty()) break;
        // a matrix's work per token for kAcc a: passes x (staging + slots)
        auto work = [&](const sft_leaf_mat &L, int a) {
            const int64_t pp = int64_t(a) * kLeafThreads, passes = (L.K + pp - 1) / pp;
            return double(passes) * (double(L.m + L.n) / 4.0 + double(pp));
        };
        int acc = kLeafAccs[0];
        double best = -1.0;
        for (int a : kLeafAccs) {
            double w = 0.0;
            for (int32_t j : idx) w += work(mats[j], a);
            if (best < 0.0 || w < best) best = w, acc = a;
        }
        const int64_t per_pass = int64_t(acc) * kLeafThreads;
        const double cost = best;
        int64_t wgs = 0, coords = 0;
        for (int32_t j : idx) {
            const sft_leaf_mat &L = mats[j];
            LeafMatDev &d = p.mat[p.n_mats++];
            d.D = L.dY;
            d.X = L.X;
            d.rows = L.rows;
            d.cols = L.cols;
            d.grad = L.grad;
            d.m = L.m;
            d.n = L.n;
            d.K = L.K;
            d.P = static_cast<int32_t>((L.K + per_pass - 1) / per_pass);
            // token pairs per batch: as many as LDS and the lane's staging
            // slots allow (a pair needs ceil(m/8/1024) + ceil(n/8/1024) slots)
            const int64_t ud = (L.m / 8 + kLeafThreads - 1) / kLeafThreads, ux = (L.n / 8 + kLeafThreads - 1) / kLeafThreads;
            int64_t tp = std::min<int64_t>(kLeafMaxPairs, kLeafStageWords / (L.m + L.n));
            tp = std::max<int64_t>(1, std::min<int64_t>(tp, kLeafSlots / (ud + ux)));
            d.tp = static_cast<int32_t>(tp);
            int q = 0;
            for (int32_t pr = 0; pr < d.tp; ++pr) {
                for (int64_t u = 0; u < ud; ++u) d.slot[q++] = pr | int32_t(u << 16);
                for (int64_t u = 0; u < ux; ++u) d.slot[q++] = pr | (1 << 8) | int32_t(u << 16);
            }
            for (; q < kLeafSlots; ++q) d.slot[q] = -1;
            const double share = work(L, acc) / cost;
            int64_t S = static_cast<int64_t>(share * cus / d.P + 0.5);
            S = std::max<int64_t>(1, std::min<int64_t>(S, (T + 2 * tp - 1) / (2 * tp)));
            d.S = static_cast<int32_t>(S);
            d.wg_begin = wgs;
            wgs += S * d.P;
            coords += L.K;
            ws = round256(ws);
            d.part = reinterpret_cast<float *>(ws);   // offset, bound to the workspace later
            ws += size_t(S) * size_t(L.K) * sizeof(float);
        }
        plan.launches.push_back(p);
        plan.acc.push_back(acc);
        plan.wgs.push_back(wgs);
        plan.coords.push_back(coords);
    }
    plan.ws_bytes = round256(ws);
    return plan;
}

}  // namespace

extern "C" {

size_t sft_leaf_grad_workspace(const sft_leaf_mat *mats, int32_t n_mats, int64_t T) {
    sft::clear_error();
    if (check_leaf(mats, n_mats, T, "sft_leaf_grad_workspace")) return static_cast<size_t>(-1);
    return leaf_plan(mats, n_mats, T).ws_bytes;
}

int sft_leaf_grad(const sft_leaf_mat *mats, int32_t n_mats, int64_t T, void *ws, size_t ws_bytes, void *stream) {
    sft::clear_error();
    if (int rc = check_leaf(mats, n_mats, T, "sft_leaf_grad")) return rc;
    LeafPlan plan = leaf_plan(mats, n_mats, T);
    if (plan.launches.empty()) return SFT_OK;
    SFT_CHECK(ws_bytes >= plan.ws_bytes, SFT_ECAPACITY, "sft_leaf_grad: workspace %zu < %zu bytes", ws_bytes,
              plan.ws_bytes);
    SFT_CHECK(ws && sft::aligned16(ws), SFT_EINVAL, "sft_leaf_grad: workspace null or not 16-byte aligned");
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (size_t l = 0; l < plan.launches.size(); ++l) {
        LeafParams &p = plan.launches[l];
        for (int32_t j = 0; j < p.n_mats; ++j)
            p.mat[j].part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                      reinterpret_cast<uintptr_t>(p.mat[j].part));
        if (T > 0) {
            const dim3 grid(static_cast<uint32_t>(plan.wgs[l]));
            switch (plan.acc[l]) {
                case 12: hipLaunchKernelGGL(k_leaf_grad<12>, grid, dim3(kLeafThreads), 0, st, p); break;
                case 16: hipLaunchKernelGGL(k_leaf_grad<16>, grid, dim3(kLeafThreads), 0, st, p); break;
                case 20: hipLaunchKernelGGL(k_leaf_grad<20>, grid, dim3(kLeafThreads), 0, st, p); break;
                case 24: hipLaunchKernelGGL(k_leaf_grad<24>, grid, dim3(kLeafThreads), 0, st, p); break;
                default: hipLaunchKernelGGL(k_leaf_grad<28>, grid, dim3(kLeafThreads), 0, st, p); break;
            }
            hipError_t e = hipGetLastError();
            SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_leaf_grad: launch failed: %s", hipGetErrorString(e));
        } else {
            for (int32_t j = 0; j < p.n_mats; ++j) p.mat[j].S = 0;   // no tokens: every gradient is 0
        }
        hipLaunchKernelGGL(k_leaf_reduce, dim3(static_cast<uint32_t>((plan.coords[l] + 255) / 256)), dim3(256), 0,
                           st, p);
        const hipError_t e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_leaf_grad: reduce launch failed: %s", hipGetErrorString(e));
    }
    return SFT_OK;
}

int sft_leaf_adam(const sft_leaf_vec *vecs, int32_t n_vecs, int32_t step, const sft_adam *hp, void *stream) {
    sft::clear_error();
    SFT_CHECK(n_vecs >= 0 && (n_vecs == 0 || vecs), SFT_EINVAL, "sft_leaf_adam: bad vector list");
    SFT_CHECK(hp && hp->bc1 && hp->bc2, SFT_EINVAL, "sft_leaf_adam: missing Adam parameters or bias table");
    SFT_CHECK(step >= 1 && step <= hp->t_max, SFT_EINVAL, "sft_leaf_adam: step %d outside [1, t_max=%d]", step,
              hp->t_max);
    SFT_CHECK(hp->weight_decay == 0.0f, SFT_EINVAL, "sft_leaf_adam: the SparseLeaf step has no weight decay");
    for (int32_t i = 0; i < n_vecs; ++i) {
        const sft_leaf_vec &v = vecs[i];
        SFT_CHECK(v.K >= 0 && v.K < (int64_t(1) << 31), SFT_EINVAL, "sft_leaf_adam: vector %d: bad K", i);
        if (v.K == 0) continue;
        SFT_CHECK(v.grad && v.theta && v.m && v.v, SFT_EINVAL, "sft_leaf_adam: vector %d: null pointer", i);
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    LeafAdamParams p{};
    p.step = step;
    p.lr = hp->lr;
    p.beta1 = hp->beta1;
    p.beta2 = hp->beta2;
    p.eps = hp->eps;
    p.c1 = 1.0f - hp->beta1;
    p.c2 = 1.0f - hp->beta2;
    p.bc1 = hp->bc1;
    p.bc2 = hp->bc2;
    int64_t total = 0;
    auto flush = [&]() -> int {
        if (p.n_vecs == 0) return SFT_OK;
        hipLaunchKernelGGL(k_leaf_adam, dim3(static_cast<uint32_t>((total + 255) / 256)), dim3(256), 0, st, p);
        const hipError_t e = hipGetLastError();
        SFT_CHECK(e == hipSuccess, SFT_EHIP, "sft_leaf_adam: launch failed: %s", hipGetErrorString(e));
        p.n_vecs = 0;
        total = 0;
        return SFT_OK;
    };
    for (int32_t i = 0; i < n_vecs; ++i) {
        if (vecs[i].K == 0) continue;
        if (p.n_vecs == kLeafMats)
            if (int rc = flush()) return rc;
        LeafVecDev &d = p.vec[p.n_vecs++];
        d.grad = vecs[i].grad;
        d.theta = vecs[i].theta;
        d.m = vecs[i].m;
        d.v = vecs[i].v;
        d.theta_bf16 = vecs[i].theta_bf16;
        d.K = vecs[i].K;
        d.begin = total;
        total += vecs[i].K;
    }
    return flush();
}

}  // extern "C"
