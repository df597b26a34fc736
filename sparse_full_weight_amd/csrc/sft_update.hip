// sft_update.hip -- the sparse int8 + residual Adam update, the coupled pair
// update and the masked write-back, for gfx950.
//
// Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
// Active Set", section 2.3 (storage is an int8 code q per weight, a scale s
// per row and an fp32 residual delta; the fp32 weight exists only in
// registers while the update steps it, and leaves as a fresh q and delta;
// fp16 moments are kept for active rows alone; rows outside the mask are not
// touched; the mask also selects the live rows to rebuild) and section 2.4
// (paired matrices mix their clipped gradients; each mixed gradient takes a
// textbook Adam step with bias correction; matrices without a partner take
// the plain step).
//
// Kernel shape: one workgroup per active row, all matrices of a call in one
// launch.  A row is streamed once: each lane owns 4-column chunks
// (16-byte loads of gradient and residual, 4 bytes of q, 8 bytes of each
// moment), keeps the new weights and moments in registers, reduces the row's
// maxima of |w'|, |m| and v across the wavefront (cross-lane shuffles) and
// across wavefronts (LDS), then requantises, scales the moments and stores.
// The work is bound by HBM bandwidth: per active element it reads 13 bytes
// and writes 11 (with the fused write-back).
//
// Arithmetic is IEEE fp32 without contraction: every product and sum below
// rounds on its own, divisions and square roots are correctly rounded (the
// compiler's default for HIP), fp32->fp16 and fp32->bf16 conversions round to
// nearest even, denormals are kept.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <numeric>
#include <vector>

#include "sft_internal.h"

namespace {

constexpr int kMaxMats = 16;
constexpr int kMaxFused = 8;   // matrices per fused-update launch (kernel-argument size)

struct UpdMatDev {
    const int32_t *rows;
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
    int64_t C;
    int64_t n_active;
    int64_t row_begin;  // first workgroup of this matrix
    int32_t per_wg;     // rows per workgroup (1, or 2 on the halves of a 1024-lane workgroup)
};

struct AdamDev {
    float lr, beta1, beta2, eps, wd;
    float c1, c2, decay;  // 1-beta1, 1-beta2, 1-lr*wd (host fp32)
    const float *bc1;
    const float *bc2;
    int32_t t_max;
};

struct UpdParams {
    UpdMatDev mat[kMaxMats];
    int32_t n_mats;
    AdamDev hp;
};

// Coupled pair: the partner's gradient is looked up by row.
struct PairDev {
    UpdMatDev self;        // the matrix this workgroup updates
    const int32_t *prow;   // partner's active rows
    const float *pG;       // partner's gradient rows
    int64_t pn;            // partner's n_active
    float a_own, a_cross;
    const float *clip;     // {clip_self_first? see below} device [2] or null
    int32_t self_is_b;     // 0: self is `a` of the pair, 1: self is `b`
};

struct PairParams {
    PairDev side[kMaxMats];
    int32_t n_sides;
    AdamDev hp;
};

__device__ __forceinline__ float h2f(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint16_t f2h(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ uint16_t f2bf(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Wave-uniform copy of a value every lane of the wave holds alike (a row's
// address: a wavefront never spans two rows).
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// A raw buffer over the `bytes` bytes at p (the same for every lane of the
// wave): loads at or past the end read zero and touch no memory.  The row
// loads below go through such buffers, with no branch around them, so that
// the compiler's waits can count them one chunk at a time.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buf(const void *p, int64_t bytes) {
    void *u = reinterpret_cast<void *>(uniform64(reinterpret_cast<uint64_t>(p)));
    const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
    return __builtin_amdgcn_make_buffer_rsrc(u, static_cast<short>(0), n, 0x00020000);
}
__device__ __forceinline__ float4 ld_f4(__amdgpu_buffer_rsrc_t r, int64_t byte_off) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<uint32_t>(byte_off), 0, 0));
}

// Largest values over the workgroup (three non-negative floats at once), via
// the integer order of their bit patterns: wave64 shuffles, then one LDS word
// per wave and value.  The workgroup may hold several rows of kLanes lanes
// each: the maxima are taken over the waves of the calling lane's row.
template <int kThreads, int kLanes>
__device__ __forceinline__ void block_max3_nonneg(float &x0, float &x1, float &x2, float (*lds)[kThreads / 64]) {
    uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1), u2 = __float_as_uint(x2);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        u0 = max(u0, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u0), off, 64)));
        u1 = max(u1, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u1), off, 64)));
        u2 = max(u2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(u2), off, 64)));
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        lds[0][wave] = __uint_as_float(u0);
        lds[1][wave] = __uint_as_float(u1);
        lds[2][wave] = __uint_as_float(u2);
    }
    __syncthreads();
    const int w0 = (static_cast<int>(threadIdx.x) / kLanes) * (kLanes / 64);
    float r0 = lds[0][w0], r1 = lds[1][w0], r2 = lds[2][w0];
#pragma unroll
    for (int w = 1; w < kLanes / 64; ++w) {
        r0 = fmaxf(r0, lds[0][w0 + w]);
        r1 = fmaxf(r1, lds[1][w0 + w]);
        r2 = fmaxf(r2, lds[2][w0 + w]);
    }
    x0 = r0;
    x1 = r1;
    x2 = r2;
}

// Scaled fp16 moment rows (the storage of section 2.3's fp16 moments): a row
// is stored as fp16 values of x * 2^e, one exponent e per row and moment,
// chosen from the new row's largest magnitude so that it lands in
// [2^14, 2^15): e = 141 - (biased exponent of the maximum), limited to
// [-112, 125] so that 2^e and 2^-e are normal floats; an all-zero row takes
// e = 0.  Scaling by 2^e is exact (a result below 2^-126 rounds to fp16 zero
// either way), the fp16 rounding is to nearest even, saturating at 65504.
constexpr int kExpMin = -112, kExpMax = 125;

__device__ __forceinline__ float pow2f(int e) {   // e in [-126, 127]
    return __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
}
__device__ __forceinline__ int moment_exp(float amax) {
    if (!(amax > 0.0f)) return 0;
    const int biased = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
    return min(kExpMax, max(kExpMin, 141 - biased));
}
__device__ __forceinline__ uint16_t moment_enc(float x, float scale) {
    return f2h(fminf(fmaxf(x * scale, -65504.0f), 65504.0f));
}

// Update one active row (index k of matrix M).  `gr` supplies the effective
// gradient of a 4-column chunk in two parts: gr.load(c) issues the chunk's
// gradient loads, gr.combine(raw, c, g) forms the gradient from them.
//
// Pass 1 loads the row (every load of a batch of chunks before any
// arithmetic), takes the Adam step and reduces the row's maxima of |w'|,
// |m| and v; pass 2 requantises w' and stores q, delta, the live weights and
// the moments scaled by their new exponents.  Rows of up to 16384 columns
// keep w', m and v in registers between the passes; wider rows (kChunks > 4)
// load and compute the row again in pass 2 (the same operations, so the same
// values).
//
// The workgroup holds kPer rows, each on kThreads/kPer consecutive lanes; in
// a workgroup of two rows whose second one does not exist (odd row count)
// those lanes pass valid = false and only take part in the barrier.
template <int kThreads, int kChunks, int kPer, typename Grad>
__device__ __forceinline__ void update_row(const UpdMatDev &M, int64_t k, bool valid, const AdamDev &hp,
                                           const Grad &gr) {
    constexpr int kLanes = kThreads / kPer;
    constexpr bool kKeep = kChunks <= 4;
    constexpr int kKept = kKeep ? kChunks : 1;
    const int lt = static_cast<int>(threadIdx.x) % kLanes;
    __shared__ float red[3][kThreads / 64];
    const int64_t C = valid ? M.C : 0;
    // The row's bookkeeping, none of it under a branch (a missing second row
    // of a pair reads the list's first entry and ignores it): the row and its
    // slot address the row's data; the fresh flag, the row's scale and the
    // slot's step count and moment exponents are loaded next but first used
    // after the row's data loads have gone out (the waits count loads in
    // issue order, so a use before them would hold them back).  A fresh
    // row's stored moments are loaded like any other and replaced by zeros.
    const int64_t kk = valid ? k : 0;
    const int64_t r_ld = M.rows[kk];
    const int64_t sl_ld = M.slot[kk];
    const int64_t r = valid ? r_ld : 0;
    const int64_t sl = valid ? sl_ld : 0;
    // The fresh flag and the exponents are read per lane, at an index plus a
    // lane count that is zero in every lane: as vector values they are not
    // moved to scalar registers, and so not waited for, where they are
    // loaded.  The scale, the step count and the bias corrections of both
    // cases (a continuing row's step t + 1, a fresh row's step 1) come
    // through scalar loads, which have a counter of their own.
    const int64_t z = static_cast<int64_t>(__builtin_amdgcn_mbcnt_lo(0u, 0u));
    // (no list of fresh flags: an empty buffer, which reads zero, not a branch)
    const uint8_t fresh_ld = static_cast<uint8_t>(__builtin_amdgcn_raw_buffer_load_b8(
        row_buf(M.fresh, M.fresh ? M.n_active : 0), static_cast<uint32_t>(kk + z), 0, 0));
    const int8_t em_ld = M.mv_exp[2 * sl + z], ev_ld = M.mv_exp[2 * sl + 1 + z];
    const float s_ld = M.s[r];
    const int32_t t_ld = M.t[sl];
    // (a fresh row's slot holds a stale count: keep the index inside the table)
    const int32_t ti_cont = t_ld < 0 ? 1 : (t_ld < hp.t_max ? t_ld + 1 : hp.t_max);
    const float bc1_cont = hp.bc1[ti_cont], bc2_cont = hp.bc2[ti_cont];
    const float bc1_fresh = hp.bc1[1], bc2_fresh = hp.bc2[1];
    const int8_t *__restrict__ qrow = M.q + r * C;
    const float *__restrict__ drow = M.delta + r * C;
    uint16_t *mrow = M.m + sl * C;
    uint16_t *vrow = M.v + sl * C;

    struct RowState {
        float s_old, dec_m, dec_v, k1, k2;
        int32_t step;
    };
    auto row_state = [&]() __attribute__((always_inline)) {
        const bool fresh = valid && fresh_ld != 0;
        RowState rs;
        rs.s_old = valid ? s_ld : 0.0f;
        const int32_t t_old = (fresh || !valid) ? 0 : t_ld;
        rs.dec_m = pow2f((fresh || !valid) ? 0 : -static_cast<int>(em_ld));
        rs.dec_v = pow2f((fresh || !valid) ? 0 : -static_cast<int>(ev_ld));
        rs.step = t_old + 1;
        // the bias corrections as per-row factors: u = (k1*m) / (sqrt(v)*k2 + eps)
        const float bc1 = !valid ? 1.0f : (fresh ? bc1_fresh : bc1_cont);
        const float bc2 = !valid ? 1.0f : (fresh ? bc2_fresh : bc2_cont);
        rs.k1 = hp.lr / bc1;
        const float sbc2 = __builtin_sqrtf(bc2);
        rs.k2 = 1.0f / sbc2;
        return rs;
    };

    // Wide rows on 1024-lane workgroups go in batches of chunks (registers).
    constexpr int kBatch = Grad::template batch<kThreads, kChunks>();
    static_assert(kChunks % kBatch == 0, "batch");
    float wn[kKept][4], mn[kKept][4], vn[kKept][4];
    float amax = 0.0f, mmax = 0.0f, vmax = 0.0f;

    // The row's buffers: columns past C (or a whole missing row) read as zero.
    const __amdgpu_buffer_rsrc_t bq = row_buf(qrow, C), bd = row_buf(drow, 4 * C);
    const __amdgpu_buffer_rsrc_t bm = row_buf(mrow, 2 * C), bv = row_buf(vrow, 2 * C);

    // Loads and Adam step of chunks [b0, b0 + kBatch): fn(j, e, w', m, v) per element.
    auto step_batch = [&](int b0, auto &&fn) __attribute__((always_inline)) {
        typename Grad::Raw graw[kBatch];
        char4 qv[kBatch];
        float4 dv[kBatch];
        ushort4 mv[kBatch], vv[kBatch];
#pragma unroll
        for (int jb = 0; jb < kBatch; ++jb) {
            const int j = b0 + jb;
            const int64_t c = 4 * (static_cast<int64_t>(lt) + static_cast<int64_t>(j) * kLanes);
            graw[jb] = gr.load(c);
            qv[jb] = __builtin_bit_cast(char4, __builtin_amdgcn_raw_buffer_load_b32(bq, static_cast<uint32_t>(c), 0, 0));
            dv[jb] = ld_f4(bd, 4 * c);
            mv[jb] = __builtin_bit_cast(ushort4, __builtin_amdgcn_raw_buffer_load_b64(bm, static_cast<uint32_t>(2 * c), 0, 0));
            vv[jb] = __builtin_bit_cast(ushort4, __builtin_amdgcn_raw_buffer_load_b64(bv, static_cast<uint32_t>(2 * c), 0, 0));
        }
        const RowState rs = row_state();
        const float s_old = rs.s_old, dec_m = rs.dec_m, dec_v = rs.dec_v, k1 = rs.k1, k2 = rs.k2;
        const bool zero_mv = !valid || fresh_ld != 0;   // a fresh row's moments start from zero
#pragma unroll
        for (int jb = 0; jb < kBatch; ++jb) {
            const int j = b0 + jb;
            const int64_t c = 4 * (static_cast<int64_t>(lt) + static_cast<int64_t>(j) * kLanes);
            if (c < C) {
                float g[4];
                gr.combine(graw[jb], c, g);
                const float qf[4] = {static_cast<float>(qv[jb].x), static_cast<float>(qv[jb].y),
                                     static_cast<float>(qv[jb].z), static_cast<float>(qv[jb].w)};
                const float df[4] = {dv[jb].x, dv[jb].y, dv[jb].z, dv[jb].w};
                const ushort4 mz = zero_mv ? make_ushort4(0, 0, 0, 0) : mv[jb];
                const ushort4 vz = zero_mv ? make_ushort4(0, 0, 0, 0) : vv[jb];
                const uint16_t mh[4] = {mz.x, mz.y, mz.z, mz.w};
                const uint16_t vh[4] = {vz.x, vz.y, vz.z, vz.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sq = s_old * qf[e];
                    const float w = sq + df[e];
                    const float m_old = h2f(mh[e]) * dec_m;
                    const float v_old = h2f(vh[e]) * dec_v;
                    const float m_a = hp.beta1 * m_old;
                    const float m_b = hp.c1 * g[e];
                    const float m = m_a + m_b;
                    const float gg = g[e] * g[e];
                    const float v_a = hp.beta2 * v_old;
                    const float v_b = hp.c2 * gg;
                    const float v = v_a + v_b;
                    const float sv = __builtin_sqrtf(v);
                    const float sk = sv * k2;
                    const float den = sk + hp.eps;
                    const float num = k1 * m;
                    const float u = num / den;
                    const float w1 = w * hp.decay;   // decay = 1 - lr*lambda (1 exactly without decay)
                    fn(j, e, w1 - u, m, v);
                }
            }
        }
    };

    // pass 1
#pragma unroll
    for (int b0 = 0; b0 < kChunks; b0 += kBatch)
        step_batch(b0, [&](int j, int e, float w, float m, float v) __attribute__((always_inline)) {
            if constexpr (kKeep) {
                wn[j][e] = w;
                mn[j][e] = m;
                vn[j][e] = v;
            }
            amax = fmaxf(amax, fabsf(w));
            mmax = fmaxf(mmax, fabsf(m));
            vmax = fmaxf(vmax, fabsf(v));
        });
    block_max3_nonneg<kThreads, kLanes>(amax, mmax, vmax, red);
    const float s_new = amax / 127.0f;
    const int em = moment_exp(mmax), ev = moment_exp(vmax);
    const float enc_m = pow2f(em), enc_v = pow2f(ev);
    if (lt == 0 && valid) {
        M.s[r] = s_new;
        M.t[sl] = row_state().step;
        M.mv_exp[2 * sl] = static_cast<int8_t>(em);
        M.mv_exp[2 * sl + 1] = static_cast<int8_t>(ev);
    }

    // pass 2: codes by the reciprocal scale (a row whose reciprocal overflows
    // divides; an all-zero row keeps zero codes), uniform per row
    const float rs = s_new != 0.0f ? 1.0f / s_new : 0.0f;
    const int mode = s_new == 0.0f ? 0 : (__builtin_isinf(rs) ? 2 : 1);
    int8_t *qout = M.q + r * C;
    float *dout = M.delta + r * C;
    uint16_t *wl = M.w_live ? M.w_live + r * C : nullptr;
    auto store_chunk = [&](auto mode_tag, int j, const float (&w4)[4], const float (&m4)[4], const float (&v4)[4])
        __attribute__((always_inline)) {
        constexpr int kMode = decltype(mode_tag)::value;
        const int64_t c = 4 * (static_cast<int64_t>(lt) + static_cast<int64_t>(j) * kLanes);
        if (c >= C) return;
        float qf[4], d[4];
        uint16_t b[4], mo[4], vo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float qq = 0.0f;
            if constexpr (kMode != 0) {
                const float x = kMode == 1 ? w4[e] * rs : w4[e] / s_new;
                qq = __builtin_rintf(x);
                qq = fminf(fmaxf(qq, -127.0f), 127.0f);
            }
            const float sq = s_new * qq;
            d[e] = w4[e] - sq;
            qf[e] = qq;
            const float back = sq + d[e];
            b[e] = f2bf(back);
            mo[e] = moment_enc(m4[e], enc_m);
            vo[e] = moment_enc(v4[e], enc_v);
        }
        *reinterpret_cast<char4 *>(qout + c) =
            make_char4(static_cast<signed char>(qf[0]), static_cast<signed char>(qf[1]),
                       static_cast<signed char>(qf[2]), static_cast<signed char>(qf[3]));
        *reinterpret_cast<float4 *>(dout + c) = make_float4(d[0], d[1], d[2], d[3]);
        if (wl) *reinterpret_cast<ushort4 *>(wl + c) = make_ushort4(b[0], b[1], b[2], b[3]);
        *reinterpret_cast<ushort4 *>(mrow + c) = make_ushort4(mo[0], mo[1], mo[2], mo[3]);
        *reinterpret_cast<ushort4 *>(vrow + c) = make_ushort4(vo[0], vo[1], vo[2], vo[3]);
    };
    auto pass2 = [&](auto mode_tag) __attribute__((always_inline)) {
        if constexpr (kKeep) {
#pragma unroll
            for (int j = 0; j < kChunks; ++j) store_chunk(mode_tag, j, wn[j], mn[j], vn[j]);
        } else {
            // Pass 1 read every load of the row before the barrier, so the
            // stores below cannot overtake a load of the same address.
#pragma unroll
            for (int b0 = 0; b0 < kChunks; b0 += kBatch) {
                float w4[kBatch][4], m4[kBatch][4], v4[kBatch][4];
                step_batch(b0, [&](int j, int e, float w, float m, float v) __attribute__((always_inline)) {
                    w4[j - b0][e] = w;
                    m4[j - b0][e] = m;
                    v4[j - b0][e] = v;
                });
#pragma unroll
                for (int jb = 0; jb < kBatch; ++jb) store_chunk(mode_tag, b0 + jb, w4[jb], m4[jb], v4[jb]);
            }
        }
    };
    if (mode == 1) pass2(std::integral_constant<int, 1>{});
    else if (mode == 0) pass2(std::integral_constant<int, 0>{});
    else pass2(std::integral_constant<int, 2>{});
}

// Plain update: the gradient is the matrix's own dW row.
// Launch shapes that may take rows two to a workgroup (see assign_wgs).
template <int kThreads, int kChunks>
constexpr bool kPairs = kThreads == 1024 && kChunks == 4;

// Runs fn(integral_constant<kPer>) with the matrix's rows per workgroup.
template <int kThreads, int kChunks, typename Fn>
__device__ __forceinline__ void with_rows_per_wg(const UpdMatDev &M, Fn &&fn) {
    if constexpr (kPairs<kThreads, kChunks>) {
        if (M.per_wg == 2) {
            fn(std::integral_constant<int, 2>{});
            return;
        }
    }
    fn(std::integral_constant<int, 1>{});
}

// Chunks whose loads go out together, within the register budget (1024-lane
// workgroups have at most 128 registers a lane).
template <int kThreads, int kChunks>
constexpr int plain_batch() { return kThreads >= 1024 ? (kChunks >= 16 ? 2 : 4) : kChunks; }

struct OwnGrad {
    template <int kThreads, int kChunks>
    static constexpr int batch() { return plain_batch<kThreads, kChunks>(); }
    typedef float4 Raw;
    __amdgpu_buffer_rsrc_t row;   // the dW row (C floats; empty for a missing row)
    __device__ __forceinline__ Raw load(int64_t c) const { return ld_f4(row, 4 * c); }
    __device__ __forceinline__ void combine(const Raw &x, int64_t, float *g) const {
        g[0] = x.x;
        g[1] = x.y;
        g[2] = x.z;
        g[3] = x.w;
    }
};

template <int kThreads, int kChunks>
__global__ __launch_bounds__(kThreads) void k_sparse_update(const UpdParams p) {
    const int64_t wg = blockIdx.x;
    int mi = 0;
    while (mi + 1 < p.n_mats && wg >= p.mat[mi + 1].row_begin) ++mi;
    const UpdMatDev &M = p.mat[mi];
    with_rows_per_wg<kThreads, kChunks>(M, [&](auto per) __attribute__((always_inline)) {
        constexpr int kPer = decltype(per)::value;
        const int64_t k = (wg - M.row_begin) * kPer + static_cast<int>(threadIdx.x) / (kThreads / kPer);
        const bool valid = k < M.n_active;
        update_row<kThreads, kChunks, kPer>(M, k, valid, p.hp,
                                            OwnGrad{row_buf(M.G + (valid ? k : 0) * M.C, valid ? 4 * M.C : 0)});
    });
}

// Coupled update: the blend of the clipped own and partner gradients (a row
// missing from the partner's active set contributes zero).
struct PairGrad {
    // two float4 gradient loads per chunk: half the plain batch on wide rows
    template <int kThreads, int kChunks>
    static constexpr int batch() { return kThreads >= 1024 ? (kChunks >= 8 ? 2 : 4) : kChunks; }
    struct Raw {
        float4 own, part;
    };
    __amdgpu_buffer_rsrc_t own_row;
    __amdgpu_buffer_rsrc_t part_row;   // empty: the partner's row is inactive (reads zero)
    float c_self, c_part, a_own, a_cross;
    __device__ __forceinline__ Raw load(int64_t c) const {
        Raw x;
        x.own = ld_f4(own_row, 4 * c);
        x.part = ld_f4(part_row, 4 * c);
        return x;
    }
    __device__ __forceinline__ void combine(const Raw &x, int64_t, float *g) const {
        const float sa[4] = {x.own.x, x.own.y, x.own.z, x.own.w};
        const float pa[4] = {x.part.x, x.part.y, x.part.z, x.part.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float cs = c_self * sa[e];
            const float cp = c_part * pa[e];
            const float own = a_own * cs;
            const float cross = a_cross * cp;
            g[e] = own + cross;
        }
    }
};

// Index of `row` in an ascending list of distinct rows, or -1, found by the
// 64 lanes of a wave together (every lane of the wave gets the answer): each
// round reads 64 evenly spaced entries of the remaining range and keeps the
// stretch between the last entry <= row and the next, so a list of up to
// 64^m entries takes m dependent loads.  Called with the whole wave active.
__device__ __forceinline__ int64_t find_row_wave(const int32_t *rows, int64_t n, int64_t row) {
    const int lane = static_cast<int>(threadIdx.x & 63);
    int64_t lo = 0, hi = n;   // row, if listed, is in [lo, hi)
    while (hi - lo > 64) {
        const int64_t step = (hi - lo + 63) / 64;
        const int64_t idx = lo + lane * step;
        const bool le = idx < hi && rows[idx] <= row;
        const int cnt = __popcll(__ballot(le));   // a prefix of the lanes (the list ascends)
        if (cnt == 0) return -1;
        lo = lo + static_cast<int64_t>(cnt - 1) * step;
        hi = min(hi, lo + step);
    }
    const int64_t idx = lo + lane;
    const bool hit = idx < hi && rows[idx] == row;
    const uint64_t b = __ballot(hit);
    return b ? lo + __ffsll(static_cast<unsigned long long>(b)) - 1 : -1;
}

template <int kThreads, int kChunks>
__global__ __launch_bounds__(kThreads) void k_coupled_update(const PairParams p) {
    const int64_t wg = blockIdx.x;
    int si = 0;
    while (si + 1 < p.n_sides && wg >= p.side[si + 1].self.row_begin) ++si;
    const PairDev &S = p.side[si];
    const UpdMatDev &M = S.self;
    with_rows_per_wg<kThreads, kChunks>(M, [&](auto per) __attribute__((always_inline)) {
        constexpr int kPer = decltype(per)::value;
        const int64_t k = (wg - M.row_begin) * kPer + static_cast<int>(threadIdx.x) / (kThreads / kPer);
        const bool valid = k < M.n_active;
        const int64_t r = valid ? M.rows[k] : 0;
        const int64_t pk = valid ? find_row_wave(S.prow, S.pn, r) : -1;
        const float clip_a = S.clip ? S.clip[0] : 1.0f;
        const float clip_b = S.clip ? S.clip[1] : 1.0f;
        PairGrad gr;
        gr.own_row = row_buf(M.G + (valid ? k : 0) * M.C, valid ? 4 * M.C : 0);
        gr.part_row = row_buf(pk >= 0 ? S.pG + pk * M.C : M.G, pk >= 0 ? 4 * M.C : 0);
        gr.c_self = S.self_is_b ? clip_b : clip_a;
        gr.c_part = S.self_is_b ? clip_a : clip_b;
        gr.a_own = S.a_own;
        gr.a_cross = S.a_cross;
        update_row<kThreads, kChunks, kPer>(M, k, valid, p.hp, gr);
    });
}

// One live row r: w_live[r, c] = bf16(fl(fl(s[r] * q[r, c]) + delta[r, c])),
// 8 columns per lane and step, 256 lanes.
__device__ __forceinline__ void writeback_row(const int8_t *__restrict__ q, const float *__restrict__ s,
                                              const float *__restrict__ delta, int64_t C, int64_t r,
                                              uint16_t *__restrict__ w_live) {
    const float sr = s[r];
    const int8_t *qr = q + r * C;
    const float *dr = delta + r * C;
    uint16_t *wr = w_live + r * C;
    for (int64_t c = 8 * static_cast<int64_t>(threadIdx.x); c < C; c += 8 * 256) {
        const int2 qv = *reinterpret_cast<const int2 *>(qr + c);
        const float4 d0 = *reinterpret_cast<const float4 *>(dr + c);
        const float4 d1 = *reinterpret_cast<const float4 *>(dr + c + 4);
        const int8_t *qb = reinterpret_cast<const int8_t *>(&qv);
        const float df[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        uint16_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sq = sr * static_cast<float>(qb[e]);
            const float w = sq + df[e];
            o[e] = f2bf(w);
        }
        uint4 pack;
        pack.x = o[0] | (static_cast<uint32_t>(o[1]) << 16);
        pack.y = o[2] | (static_cast<uint32_t>(o[3]) << 16);
        pack.z = o[4] | (static_cast<uint32_t>(o[5]) << 16);
        pack.w = o[6] | (static_cast<uint32_t>(o[7]) << 16);
        *reinterpret_cast<uint4 *>(wr + c) = pack;
    }
}

__global__ __launch_bounds__(256) void k_masked_writeback(const int8_t *__restrict__ q,
                                                          const float *__restrict__ s,
                                                          const float *__restrict__ delta, int64_t C,
                                                          const int32_t *__restrict__ rows,
                                                          uint16_t *__restrict__ w_live) {
    writeback_row(q, s, delta, C, rows[blockIdx.x], w_live);
}

// Several matrices in one launch: workgroup b takes row b - row_begin of the
// matrix whose range [row_begin, row_begin + n_active) holds b.
struct WbMatDev {
    const int8_t *q;
    const float *s;
    const float *delta;
    const int32_t *rows;
    uint16_t *w_live;
    int64_t C;
    int64_t row_begin;
};

struct WbParams {
    WbMatDev mat[kMaxMats];
    int32_t n_mats;
};

__global__ __launch_bounds__(256) void k_masked_writeback_many(const WbParams p) {
    const int64_t b = blockIdx.x;
    int mi = 0;
    while (mi + 1 < p.n_mats && b >= p.mat[mi + 1].row_begin) ++mi;
    const WbMatDev &M = p.mat[mi];
    writeback_row(M.q, M.s, M.delta, M.C, M.rows[b - M.row_begin], M.w_live);
}

// ---- Active-row checkpoints (section 2.6: only the active rows are copied).
constexpr int kCkMats = 16;      // matrices per launch (kernel-argument size)
constexpr int kCkThreads = 256;
constexpr int kCkBatch = 4;      // 8-column chunks per lane whose loads are in flight together

struct CkMatDev {
    sft_ckpt_mat m;
    int64_t row_begin;   // first workgroup (= checkpointed row) of this matrix
};

struct CkParams {
    CkMatDev mat[kCkMats];
    int32_t n_mats;
};

// One workgroup per checkpointed row.  Per 8-column chunk the row's q
// (8 bytes) and delta (32 bytes) and its slot's m and v (16 bytes each) go
// live -> checkpoint (save) or back (restore); a restore also rebuilds the
// row's live bf16 weights from the restored values, as the write-back does.
// Lane l takes chunks l, l + 256, ...; it issues the loads of 4 chunks before
// its stores.  The row's s and its slot's t and moment exponents are copied
// by lane 0.
template <bool kRestore>
__global__ __launch_bounds__(kCkThreads) void k_rows_copy(const CkParams p) {
    const int64_t wg = blockIdx.x;
    int mi = 0;
    while (mi + 1 < p.n_mats && wg >= p.mat[mi + 1].row_begin) ++mi;
    const sft_ckpt_mat &M = p.mat[mi].m;
    const int64_t k = wg - p.mat[mi].row_begin;
    const int64_t r = M.rows[k], sl = M.slot[k], C = M.C;
    int8_t *const lq = M.q + r * C, *const cq = M.ck_q + k * C;
    float *const ld = M.delta + r * C, *const cd = M.ck_delta + k * C;
    uint16_t *const lm = M.m + sl * C, *const cm = M.ck_m + k * C;
    uint16_t *const lv = M.v + sl * C, *const cv = M.ck_v + k * C;
    const int8_t *const q_src = kRestore ? cq : lq;
    int8_t *const q_dst = kRestore ? lq : cq;
    const float *const d_src = kRestore ? cd : ld;
    float *const d_dst = kRestore ? ld : cd;
    const uint16_t *const m_src = kRestore ? cm : lm;
    uint16_t *const m_dst = kRestore ? lm : cm;
    const uint16_t *const v_src = kRestore ? cv : lv;
    uint16_t *const v_dst = kRestore ? lv : cv;
    uint16_t *const w = (kRestore && M.w_live) ? M.w_live + r * C : nullptr;
    const float s_row = kRestore ? M.ck_s[k] : 0.0f;
    if (threadIdx.x == 0) {
        if (kRestore) {
            M.s[r] = s_row;
            M.t[sl] = M.ck_t[k];
            M.mv_exp[2 * sl] = M.ck_mv_exp[2 * k];
            M.mv_exp[2 * sl + 1] = M.ck_mv_exp[2 * k + 1];
        } else {
            M.ck_s[k] = M.s[r];
            M.ck_t[k] = M.t[sl];
            M.ck_mv_exp[2 * k] = M.mv_exp[2 * sl];
            M.ck_mv_exp[2 * k + 1] = M.mv_exp[2 * sl + 1];
        }
    }
    // One 8-column chunk in registers.  The four chunks of a batch are named
    // variables, not an array: an array here was placed in LDS and scratch.
    struct Chunk {
        uint2 q;
        float4 d0, d1;
        uint4 m, v;
    };
    auto load = [&](int64_t c) __attribute__((always_inline)) {
        Chunk x;
        x.q = *reinterpret_cast<const uint2 *>(q_src + c);
        x.d0 = *reinterpret_cast<const float4 *>(d_src + c);
        x.d1 = *reinterpret_cast<const float4 *>(d_src + c + 4);
        x.m = *reinterpret_cast<const uint4 *>(m_src + c);
        x.v = *reinterpret_cast<const uint4 *>(v_src + c);
        return x;
    };
    auto store = [&](int64_t c, const Chunk &x) __attribute__((always_inline)) {
        if (c >= C) return;
        *reinterpret_cast<uint2 *>(q_dst + c) = x.q;
        *reinterpret_cast<float4 *>(d_dst + c) = x.d0;
        *reinterpret_cast<float4 *>(d_dst + c + 4) = x.d1;
        *reinterpret_cast<uint4 *>(m_dst + c) = x.m;
        *reinterpret_cast<uint4 *>(v_dst + c) = x.v;
        if (w) {
            const float df[8] = {x.d0.x, x.d0.y, x.d0.z, x.d0.w, x.d1.x, x.d1.y, x.d1.z, x.d1.w};
            uint32_t o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t word = e < 4 ? x.q.x : x.q.y;
                const int8_t qe = static_cast<int8_t>((word >> (8 * (e & 3))) & 0xffu);
                const float sq = s_row * static_cast<float>(qe);
                o[e] = f2bf(sq + df[e]);
            }
            *reinterpret_cast<uint4 *>(w + c) =
                make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16));
        }
    };
    static_assert(kCkBatch == 4, "the batch below is spelled out for four chunks");
    constexpr int64_t kStep = 8 * kCkThreads;
    for (int64_t c0 = 8 * static_cast<int64_t>(threadIdx.x); c0 < C; c0 += kStep * kCkBatch) {
        // chunks past the row read chunk c0 again (in bounds) and store nothing
        const int64_t c1 = c0 + kStep, c2 = c0 + 2 * kStep, c3 = c0 + 3 * kStep;
        const Chunk x0 = load(c0);
        const Chunk x1 = load(c1 < C ? c1 : c0);
        const Chunk x2 = load(c2 < C ? c2 : c0);
        const Chunk x3 = load(c3 < C ? c3 : c0);
        store(c0, x0);
        store(c1, x1);
        store(c2, x2);
        store(c3, x3);
    }
}

// Update fused with the masked-dW fix-up: the gradient of a 256-column block
// of the row is the sum, in slice order, of the partial rows the slices that
// cut its output tile left (the same additions as the fix-up kernel's), or
// the dW_act row where one slice covered the tile.  tab[nb] = (first slice,
// slices | first-slot-odd << 16), built per workgroup; the slices are
// `stride` apart (team slicing: one per team).
struct FusedGrad {
    // (two partial rows per chunk loaded with the row; a block cut more ways
    // adds the rest from memory while the step combines them, which keeps a
    // 1024-lane batch of four chunks within the registers)
    template <int kThreads, int kChunks>
    static constexpr int batch() { return kThreads >= 1024 ? (kChunks >= 8 ? 2 : 4) : kChunks; }
    struct Raw {
        float4 x[2];
        int32_t n, v0, cl;   // partial rows of the chunk's column block, their first slice, column in the block
        bool odd;
    };
    const float *part;
    const float *dw_row;      // the row in dW_act
    int64_t row_bytes;        // its bytes (0 for a missing row)
    int64_t cols;             // its columns (0 for a missing row)
    const int2 *tab;          // LDS, entries for the column blocks below cols only
    int64_t slot_floats;
    int32_t bn, prow, stride;
    __device__ __forceinline__ const float *slot_row(int32_t v0, int32_t i, bool odd) const {
        const int64_t sv = v0 + static_cast<int64_t>(i) * stride;
        const int64_t slot = (i == 0 && odd) ? 2 * sv + 1 : 2 * sv;
        return part + slot * slot_floats + static_cast<int64_t>(prow) * bn;
    }
    // A wave's 64 lanes take 256 consecutive columns starting on a multiple
    // of 256 (4 columns a lane), and the product's output tiles are 256
    // columns wide (bn), so the chunk's column block, and with it every
    // partial row's address, is the same across the wave.  A block that
    // starts at or past the row's end has no table entry: it reads nothing
    // (every buffer empty, based at the partial array).
    __device__ __forceinline__ Raw load(int64_t c) const {
        const int nb = static_cast<int>(c / bn);
        const bool in = static_cast<int64_t>(nb) * bn < cols;
        Raw r;
        r.cl = static_cast<int>(c - static_cast<int64_t>(nb) * bn);
        const int2 t = in ? tab[nb] : make_int2(0, 0);
        r.v0 = __builtin_amdgcn_readfirstlane(t.x);
        const int32_t ty = __builtin_amdgcn_readfirstlane(t.y);
        r.n = ty & 0xFFFF;
        r.odd = (ty >> 16) != 0;
        // one slice covered the tile: the dW row itself; else the partial rows
        const bool whole = r.n == 1;
        r.x[0] = ld_f4(row_buf(whole ? dw_row : slot_row(r.v0, 0, r.odd), whole ? row_bytes : (in ? 4 * bn : 0)),
                       whole ? 4 * c : 4 * r.cl);
        r.x[1] = ld_f4(row_buf(slot_row(r.v0, 1, false), 1 < r.n ? 4 * bn : 0), 4 * r.cl);
        return r;
    }
    __device__ __forceinline__ void combine(const Raw &r, int64_t, float *g) const {
        float4 sum = r.x[0];
        if (1 < r.n) {
            sum.x += r.x[1].x;
            sum.y += r.x[1].y;
            sum.z += r.x[1].z;
            sum.w += r.x[1].w;
        }
        for (int i = 2; i < r.n; ++i) {
            const float4 y = *reinterpret_cast<const float4 *>(slot_row(r.v0, i, false) + r.cl);
            sum.x += y.x;
            sum.y += y.y;
            sum.z += y.z;
            sum.w += y.w;
        }
        g[0] = sum.x;
        g[1] = sum.y;
        g[2] = sum.z;
        g[3] = sum.w;
    }
};

struct FusedParams {
    UpdMatDev mat[kMaxFused];
    sft::DwRowSrc src[kMaxFused];
    int32_t n_mats;
    AdamDev hp;
};

// floor(n / d) for 0 <= n, d < 2^53 (one correctly rounded fp64 division:
// the rounding error stays below the distance 1/d to the next integer).
__device__ __forceinline__ int64_t floordiv53(int64_t n, int64_t d) {
    return static_cast<int64_t>(static_cast<double>(n) / static_cast<double>(d));
}

template <int kThreads, int kChunks>
__global__ __launch_bounds__(kThreads) void k_fused_update(const FusedParams p) {
    __shared__ int2 tab[2][256];
    const int64_t wg = blockIdx.x;
    int mi = 0;
    while (mi + 1 < p.n_mats && wg >= p.mat[mi + 1].row_begin) ++mi;
    const UpdMatDev &M = p.mat[mi];
    const sft::DwRowSrc &S = p.src[mi];
    with_rows_per_wg<kThreads, kChunks>(M, [&](auto per) __attribute__((always_inline)) {
        constexpr int kPer = decltype(per)::value, kLanes = kThreads / kPer;
        const int sub = static_cast<int>(threadIdx.x) / kLanes, lt = static_cast<int>(threadIdx.x) % kLanes;
        const int64_t k = (wg - M.row_begin) * kPer + sub;
        const bool valid = k < M.n_active;
        const int64_t kk = valid ? k : 0;
        // the row's packed row j in its group, its M-block and its row in the
        // M-block's packed rows
        int64_t j = S.row_begin + kk;
        if (S.tiles) {   // tile layout: 32 rows per active tile
            const int32_t r = M.rows[kk];
            int64_t lo = 0, hi = S.n_tiles;
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (S.tiles[mid] < (r >> 5)) lo = mid + 1;
                else hi = mid;
            }
            j = S.row_begin + 32 * lo + (r & 31);
        }
        const int64_t ptile = j >> 5;
        auto mlo = [&](int64_t bb) __attribute__((always_inline)) { return floordiv53(bb * S.n_ptiles, S.n_mblk); };
        int64_t mb = floordiv53(ptile * S.n_mblk, S.n_ptiles);
        while (mb > 0 && mlo(mb) > ptile) --mb;
        while (mb + 1 < S.n_mblk && mlo(mb + 1) <= ptile) ++mb;
        const int32_t prow = static_cast<int32_t>(j - 32 * mlo(mb));
        // slices over each output tile (M-block mb, column block nb): the
        // tile is rounds [a, b) of Q rounds cut into P equal ranges, range i
        // starting at round floor(i * Q / P) -- the launch's iterations and
        // slices, or (team slicing) the group's column-block rounds and teams,
        // range i being slice wg_begin + i * n_mblk + mb
        const int64_t R = S.chunks / S.rnd;
        const int64_t Q = S.team ? S.n_nblk * R : S.Q, P = S.team ? S.n_team : S.P;
        const int64_t base = S.team ? S.wg_begin + mb : 0, stride = S.team ? S.n_mblk : 1;
        for (int nb = lt; nb < S.n_nblk; nb += kLanes) {
            const int64_t tile = S.nb_major ? nb * static_cast<int64_t>(S.n_mblk) + mb : mb * S.n_nblk + nb;
            const int64_t a = S.team ? nb * R : (S.it_begin + tile * static_cast<int64_t>(S.chunks)) / S.rnd;
            const int64_t b = a + R;
            const int64_t v0 = floordiv53((a + 1) * P - 1, Q);
            const int64_t v1 = floordiv53(b * P - 1, Q);
            const bool odd = floordiv53(v0 * Q, P) < a;
            tab[sub][nb] = make_int2(static_cast<int>(base + v0 * stride),
                                     static_cast<int>(v1 - v0 + 1) | (odd ? 0x10000 : 0));
        }
        __syncthreads();
        FusedGrad gr;
        gr.part = S.part;
        gr.dw_row = S.dW + kk * M.C;
        gr.row_bytes = valid ? 4 * M.C : 0;
        gr.cols = valid ? M.C : 0;
        gr.tab = tab[sub];
        gr.slot_floats = S.slot_floats;
        gr.bn = S.bn;
        gr.prow = prow;
        gr.stride = S.team ? S.n_mblk : 1;
        update_row<kThreads, kChunks, kPer>(M, k, valid, p.hp, gr);
    });
}

// ---------------------------------------------------------------- host side

int check_mat(const sft_upd_mat &m, const char *who) {
    SFT_CHECK(m.R >= 0 && m.C > 0 && m.n_active >= 0 && m.n_slots >= 0, SFT_EINVAL,
              "%s: bad sizes (R=%lld C=%lld n_active=%lld)", who, (long long)m.R, (long long)m.C,
              (long long)m.n_active);
    SFT_CHECK(m.C % 8 == 0, SFT_ESHAPE, "%s: C=%lld is not a multiple of 8", who, (long long)m.C);
    SFT_CHECK(m.C <= 65536, SFT_ENOTSUP, "%s: C=%lld above 65536", who, (long long)m.C);
    SFT_CHECK(m.n_active <= m.R && m.n_active <= m.n_slots, SFT_ECAPACITY,
              "%s: n_active=%lld exceeds R or n_slots", who, (long long)m.n_active);
    if (m.n_active == 0) return SFT_OK;
    SFT_CHECK(m.active_rows && m.slot && m.G && m.q && m.s && m.delta && m.m && m.v && m.t && m.mv_exp,
              SFT_EINVAL, "%s: null device pointer", who);
    SFT_CHECK(sft::aligned16(m.G) && sft::aligned16(m.q) && sft::aligned16(m.delta) &&
                  sft::aligned16(m.m) && sft::aligned16(m.v) &&
                  (!m.w_live || sft::aligned16(m.w_live)),
              SFT_EALIGN, "%s: a row-major device buffer is not 16-byte aligned", who);
    return SFT_OK;
}

int check_hp(const sft_adam *hp, const char *who) {
    SFT_CHECK(hp && hp->bc1 && hp->bc2 && hp->t_max >= 1, SFT_EINVAL,
              "%s: missing Adam parameters or bias table", who);
    return SFT_OK;
}

AdamDev make_adam(const sft_adam &hp) {
    AdamDev a;
    a.lr = hp.lr;
    a.beta1 = hp.beta1;
    a.beta2 = hp.beta2;
    a.eps = hp.eps;
    a.wd = hp.weight_decay;
    a.c1 = 1.0f - hp.beta1;
    a.c2 = 1.0f - hp.beta2;
    const float lrwd = hp.lr * hp.weight_decay;
    a.decay = 1.0f - lrwd;
    a.bc1 = hp.bc1;
    a.bc2 = hp.bc2;
    a.t_max = hp.t_max;
    return a;
}

UpdMatDev make_mat(const sft_upd_mat &m, int64_t row_begin) {
    UpdMatDev d;
    d.rows = m.active_rows;
    d.slot = m.slot;
    d.fresh = m.fresh;
    d.G = m.G;
    d.q = m.q;
    d.s = m.s;
    d.delta = m.delta;
    d.m = m.m;
    d.v = m.v;
    d.t = m.t;
    d.mv_exp = m.mv_exp;
    d.w_live = m.w_live;
    d.C = m.C;
    d.n_active = m.n_active;
    d.row_begin = row_begin;
    d.per_wg = 1;
    return d;
}

// Rows per workgroup and workgroup offsets of a launch's matrices.  With
// 1024 lanes (some row wider than 4096 columns) a workgroup holds a CU by
// itself; when single rows would outnumber the CUs, rows of up to 8192
// columns go two to a workgroup (512 lanes each), so that the launch is one
// wave of workgroups.  Returns the workgroup count.
int64_t assign_wgs(UpdMatDev *const *mats, int32_t n, int64_t maxC) {
    int64_t rows = 0;
    for (int32_t i = 0; i < n; ++i) rows += mats[i]->n_active;
    const bool pair = maxC > 256 * 4 * 4 && maxC <= 1024 * 4 * 4 && rows > sft::num_cus();
    int64_t n_wg = 0;
    for (int32_t i = 0; i < n; ++i) {
        UpdMatDev &d = *mats[i];
        d.per_wg = (pair && d.C <= 512 * 4 * 4) ? 2 : 1;
        d.row_begin = n_wg;
        n_wg += (d.n_active + d.per_wg - 1) / d.per_wg;
    }
    return n_wg;
}

// Chunks of 4 columns per lane: the smallest instantiated count covering C.
// Rows up to 4096 columns take 256 lanes (several workgroups share a CU);
// wider ones take 1024 lanes, one workgroup a CU, so that a wide row's
// arithmetic has all four SIMDs to itself (with 256 lanes it shared its CU
// with a narrow row and set the kernel's length).
template <typename Params, template <int, int> class Launch>
int dispatch(int64_t maxC, int64_t n_wg, const Params &p, hipStream_t stream) {
    if (maxC <= 256 * 4 * 4) return Launch<256, 4>::go(n_wg, p, stream);
    if (maxC <= 1024 * 4 * 4) return Launch<1024, 4>::go(n_wg, p, stream);
    if (maxC <= 1024 * 4 * 8) return Launch<1024, 8>::go(n_wg, p, stream);
    return Launch<1024, 16>::go(n_wg, p, stream);
}

// Launches of a list of matrices sorted widest first: at most `per_launch`
// matrices each; and when the matrices of at most 4096 columns have more
// than two rows per CU, they take launches of their own: their 256-lane
// workgroups then share CUs several at a time, and the load and store phases
// of different rows interleave, where as 1024-lane workgroups beside wide rows
// each CU would run one row (or pair) at a time in lock step.  Returns the
// first index of each launch, and the end.
std::vector<int32_t> launch_cuts(const std::vector<int64_t> &width, const std::vector<int64_t> &rows,
                                 int32_t per_launch) {
    const int32_t n = static_cast<int32_t>(width.size());
    int64_t narrow = 0;
    for (int32_t i = 0; i < n; ++i)
        if (width[i] <= 256 * 4 * 4) narrow += rows[i];
    const bool split = narrow > 2 * int64_t(sft::num_cus());
    std::vector<int32_t> cuts;
    for (int32_t i = 0; i < n; ++i) {
        const bool boundary = i > 0 && split && width[i - 1] > 256 * 4 * 4 && width[i] <= 256 * 4 * 4;
        if (i == 0 || boundary || i - cuts.back() == per_launch) cuts.push_back(i);
    }
    cuts.push_back(n);
    return cuts;
}

int launch_status(const char *who) {
    const hipError_t e = hipGetLastError();
    SFT_CHECK(e == hipSuccess, SFT_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return SFT_OK;
}

template <int T, int N>
struct LaunchUpd {
    static int go(int64_t n_wg, const UpdParams &p, hipStream_t s) {
        hipLaunchKernelGGL((k_sparse_update<T, N>), dim3(static_cast<uint32_t>(n_wg)), dim3(T), 0, s, p);
        return launch_status("sft_sparse_update");
    }
};

template <int T, int N>
struct LaunchFused {
    static int go(int64_t n_wg, const FusedParams &p, hipStream_t s) {
        hipLaunchKernelGGL((k_fused_update<T, N>), dim3(static_cast<uint32_t>(n_wg)), dim3(T), 0, s, p);
        return launch_status("sft_masked_dw_update");
    }
};

template <int T, int N>
struct LaunchPair {
    static int go(int64_t n_wg, const PairParams &p, hipStream_t s) {
        hipLaunchKernelGGL((k_coupled_update<T, N>), dim3(static_cast<uint32_t>(n_wg)), dim3(T), 0, s, p);
        return launch_status("sft_coupled_update");
    }
};

}  // namespace

extern "C" {

int sft_sparse_update(const sft_upd_mat *mats, int32_t n_mats, const sft_adam *hp, void *stream) {
    sft::clear_error();
    SFT_CHECK(n_mats >= 0 && (n_mats == 0 || mats), SFT_EINVAL, "sft_sparse_update: bad matrix list");
    if (int rc = check_hp(hp, "sft_sparse_update")) return rc;
    for (int32_t i = 0; i < n_mats; ++i)
        if (int rc = check_mat(mats[i], "sft_sparse_update")) return rc;
    const AdamDev a = make_adam(*hp);
    // Widest rows first: they are the longest workgroups, and going out
    // first they get CUs of their own before the narrow rows fill the rest.
    std::vector<int32_t> order(static_cast<size_t>(n_mats));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return mats[x].C > mats[y].C; });
    // Matrices go out in batches of kMaxMats per launch (kernel-argument table),
    // narrow ones apart when they are many (launch_cuts).
    std::vector<int64_t> wid, nr;
    for (const int32_t i : order) {
        wid.push_back(mats[i].C);
        nr.push_back(mats[i].n_active);
    }
    const std::vector<int32_t> cuts = launch_cuts(wid, nr, kMaxMats);
    for (size_t ci = 0; ci + 1 < cuts.size(); ++ci) {
        UpdParams p{};
        p.hp = a;
        int64_t n_wg = 0, maxC = 0;
        int32_t n = 0;
        UpdMatDev *list[kMaxMats];
        for (int32_t oi = cuts[ci]; oi < cuts[ci + 1]; ++oi) {
            const int32_t i = order[static_cast<size_t>(oi)];
            if (mats[i].n_active == 0) continue;
            p.mat[n] = make_mat(mats[i], 0);
            list[n] = &p.mat[n];
            ++n;
            maxC = std::max<int64_t>(maxC, mats[i].C);
        }
        p.n_mats = n;
        n_wg = assign_wgs(list, n, maxC);
        if (n_wg == 0) continue;
        SFT_CHECK(n_wg < (int64_t(1) << 31), SFT_ENOTSUP, "sft_sparse_update: too many rows");
        if (int rc = dispatch<UpdParams, LaunchUpd>(maxC, n_wg, p, static_cast<hipStream_t>(stream)))
            return rc;
    }
    return SFT_OK;
}

int sft_coupled_update(const sft_pair *pairs, int32_t n_pairs, const sft_adam *hp, void *stream) {
    sft::clear_error();
    SFT_CHECK(n_pairs >= 0 && (n_pairs == 0 || pairs), SFT_EINVAL, "sft_coupled_update: bad pair list");
    if (int rc = check_hp(hp, "sft_coupled_update")) return rc;
    for (int32_t i = 0; i < n_pairs; ++i) {
        const sft_pair &pr = pairs[i];
        if (int rc = check_mat(pr.a, "sft_coupled_update")) return rc;
        if (int rc = check_mat(pr.b, "sft_coupled_update")) return rc;
        SFT_CHECK(pr.a.R == pr.b.R && pr.a.C == pr.b.C, SFT_ESHAPE,
                  "sft_coupled_update: pair %d has unequal shapes", i);
    }
    const AdamDev a = make_adam(*hp);
    // Each side of each pair is a list of workgroups (one per active row of that
    // side); kMaxMats sides per launch.
    PairParams p{};
    p.hp = a;
    int64_t n_wg = 0, maxC = 0;
    auto flush = [&]() -> int {
        if (n_wg == 0) return SFT_OK;
        UpdMatDev *list[kMaxMats];
        for (int32_t i = 0; i < p.n_sides; ++i) list[i] = &p.side[i].self;
        n_wg = assign_wgs(list, p.n_sides, maxC);
        SFT_CHECK(n_wg < (int64_t(1) << 31), SFT_ENOTSUP, "sft_coupled_update: too many rows");
        const int rc = dispatch<PairParams, LaunchPair>(maxC, n_wg, p, static_cast<hipStream_t>(stream));
        p = PairParams{};
        p.hp = a;
        n_wg = 0;
        maxC = 0;
        return rc;
    };
    // Sides with the widest rows first (as in sft_sparse_update).
    std::vector<int32_t> order(static_cast<size_t>(2 * n_pairs));
    std::iota(order.begin(), order.end(), 0);
    auto width = [&](int32_t k) { return (k & 1) ? pairs[k >> 1].b.C : pairs[k >> 1].a.C; };
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return width(x) > width(y); });
    // narrow sides apart when they are many (as launch_cuts does)
    std::vector<int64_t> wid, nr;
    for (const int32_t k : order) {
        wid.push_back(width(k));
        nr.push_back((k & 1) ? pairs[k >> 1].b.n_active : pairs[k >> 1].a.n_active);
    }
    const std::vector<int32_t> cuts = launch_cuts(wid, nr, static_cast<int32_t>(order.size()) + 1);
    size_t next_cut = 1;
    for (size_t oi = 0; oi < order.size(); ++oi) {
        const int32_t k = order[oi];
        const sft_pair &pr = pairs[k >> 1];
        if (next_cut + 1 < cuts.size() && static_cast<int32_t>(oi) == cuts[next_cut]) {
            ++next_cut;
            if (int rc = flush()) return rc;
        }
        {
            const int side = k & 1;
            const sft_upd_mat &self = side ? pr.b : pr.a;
            const sft_upd_mat &partner = side ? pr.a : pr.b;
            if (self.n_active == 0) continue;
            if (p.n_sides == kMaxMats)
                if (int rc = flush()) return rc;
            PairDev &d = p.side[p.n_sides++];
            d.self = make_mat(self, n_wg);
            d.prow = partner.active_rows;
            d.pG = partner.G;
            d.pn = partner.n_active;
            d.a_own = pr.a_own;
            d.a_cross = pr.a_cross;
            d.clip = pr.clip;
            d.self_is_b = side;
            n_wg += self.n_active;
            maxC = std::max<int64_t>(maxC, self.C);
        }
    }
    return flush();
}

int sft_masked_dw_update(const sft_dw_group *groups, int32_t n_groups, void *ws, size_t ws_bytes,
                         const sft_upd_mat *mats, int32_t n_mats, const sft_adam *hp, void *stream) {
    sft::clear_error();
    SFT_CHECK(n_groups >= 0 && (n_groups == 0 || groups), SFT_EINVAL, "sft_masked_dw_update: bad group list");
    int32_t total = 0;
    for (int32_t g = 0; g < n_groups; ++g) {
        SFT_CHECK(groups[g].n_mats >= 0 && (groups[g].n_mats == 0 || groups[g].mats), SFT_EINVAL,
                  "sft_masked_dw_update: group %d has a bad matrix list", g);
        total += groups[g].n_mats;
    }
    SFT_CHECK(n_mats == total && (n_mats == 0 || mats), SFT_EINVAL,
              "sft_masked_dw_update: %d update matrices for %d dW matrices", n_mats, total);
    if (int rc = check_hp(hp, "sft_masked_dw_update")) return rc;
    for (int32_t i = 0, g = 0; g < n_groups; ++g) {
        for (int32_t m = 0; m < groups[g].n_mats; ++m, ++i) {
            if (int rc = check_mat(mats[i], "sft_masked_dw_update")) return rc;
            const sft_dw_mat &d = groups[g].mats[m];
            SFT_CHECK(mats[i].C == groups[g].C && mats[i].n_active == d.n_active && mats[i].R == d.R &&
                          (d.n_active == 0 || (mats[i].G == d.dW_act && mats[i].active_rows == d.active_rows)),
                      SFT_EINVAL, "sft_masked_dw_update: update matrix %d does not match its dW matrix", i);
        }
    }
    std::vector<sft::DwRowSrc> src(static_cast<size_t>(total));
    bool done = false, whole = false;
    if (int rc = sft::masked_dw_partials(groups, n_groups, ws, ws_bytes, stream, src.data(), &done, &whole))
        return rc;
    if (!done) {   // the product needs more than one launch: the two calls
        if (int rc = sft_masked_dw(groups, n_groups, ws, ws_bytes, stream)) return rc;
        return sft_sparse_update(mats, n_mats, hp, stream);
    }
    if (whole) return sft_sparse_update(mats, n_mats, hp, stream);   // dW_act holds every row whole
    const AdamDev a = make_adam(*hp);
    std::vector<int32_t> order(static_cast<size_t>(n_mats));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return mats[x].C > mats[y].C; });
    std::vector<int64_t> wid, nr;
    for (const int32_t i : order) {
        wid.push_back(mats[i].C);
        nr.push_back(mats[i].n_active);
    }
    const std::vector<int32_t> cuts = launch_cuts(wid, nr, kMaxFused);
    for (size_t ci = 0; ci + 1 < cuts.size(); ++ci) {
        FusedParams p{};
        p.hp = a;
        int64_t n_wg = 0, maxC = 0;
        int32_t n = 0;
        UpdMatDev *list[kMaxFused];
        for (int32_t oi = cuts[ci]; oi < cuts[ci + 1]; ++oi) {
            const int32_t i = order[static_cast<size_t>(oi)];
            if (mats[i].n_active == 0) continue;
            p.mat[n] = make_mat(mats[i], 0);
            p.src[n] = src[static_cast<size_t>(i)];
            list[n] = &p.mat[n];
            ++n;
            maxC = std::max<int64_t>(maxC, mats[i].C);
        }
        p.n_mats = n;
        n_wg = assign_wgs(list, n, maxC);
        if (n_wg == 0) continue;
        SFT_CHECK(n_wg < (int64_t(1) << 31), SFT_ENOTSUP, "sft_masked_dw_update: too many rows");
        if (int rc = dispatch<FusedParams, LaunchFused>(maxC, n_wg, p, static_cast<hipStream_t>(stream)))
            return rc;
    }
    return SFT_OK;
}

}  // extern "C"

namespace {

// The allocation-free variant's workspace: one array per device, held for the
// life of the process.  Host code never passes `scratch` itself to a kernel
// (in host code the name stands for a host-side shadow); it passes the device
// address hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = size_t(96) << 20;
constexpr int kScratchDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

int scratch_address(void **out, const char *who) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    SFT_CHECK(e == hipSuccess, SFT_EHIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
    SFT_CHECK(dev >= 0 && dev < kScratchDevices, SFT_ENOTSUP, "%s: device %d beyond the %d supported", who, dev,
              kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        SFT_CHECK(r == hipSuccess && ptr, SFT_EHIP, "%s: hipGetSymbolAddress of the scratch array failed: %s", who,
                  hipGetErrorString(r));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SFT_OK;
}

}  // namespace

extern "C" {

size_t sft_noalloc_scratch_bytes(void) { return kScratchBytes; }

int sft_masked_dw_update_noalloc(const sft_dw_group *groups, int32_t n_groups, const sft_upd_mat *mats,
                                 int32_t n_mats, const sft_adam *hp, void *stream) {
    sft::clear_error();
    const size_t need = sft_masked_dw_workspace(groups, n_groups);
    if (need == static_cast<size_t>(-1)) return SFT_EINVAL;   // message set by the size call
    SFT_CHECK(need <= kScratchBytes, SFT_ECAPACITY,
              "sft_masked_dw_update_noalloc: the groups need %zu workspace bytes, above the %zu-byte scratch "
              "array; use sft_masked_dw_update with a workspace", need, kScratchBytes);
    void *ws = nullptr;
    if (int rc = scratch_address(&ws, "sft_masked_dw_update_noalloc")) return rc;
    return sft_masked_dw_update(groups, n_groups, ws, kScratchBytes, mats, n_mats, hp, stream);
}

int sft_masked_writeback(const int8_t *q, const float *s, const float *delta, int64_t R, int64_t C,
                         const int32_t *active_rows, int64_t n_active, uint16_t *w_live, void *stream) {
    sft::clear_error();
    SFT_CHECK(R >= 0 && C > 0 && n_active >= 0 && n_active <= R, SFT_EINVAL,
              "sft_masked_writeback: bad sizes");
    SFT_CHECK(C % 8 == 0, SFT_ESHAPE, "sft_masked_writeback: C=%lld is not a multiple of 8", (long long)C);
    if (n_active == 0) return SFT_OK;
    SFT_CHECK(q && s && delta && active_rows && w_live, SFT_EINVAL, "sft_masked_writeback: null pointer");
    SFT_CHECK(sft::aligned16(q) && sft::aligned16(delta) && sft::aligned16(w_live), SFT_EALIGN,
              "sft_masked_writeback: buffer not 16-byte aligned");
    SFT_CHECK(n_active < (int64_t(1) << 31), SFT_ENOTSUP, "sft_masked_writeback: too many rows");
    hipLaunchKernelGGL(k_masked_writeback, dim3(static_cast<uint32_t>(n_active)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), q, s, delta, C, active_rows, w_live);
    return launch_status("sft_masked_writeback");
}

int sft_masked_writeback_many(const sft_wb_mat *mats, int32_t n_mats, void *stream) {
    sft::clear_error();
    SFT_CHECK(n_mats >= 0 && (n_mats == 0 || mats), SFT_EINVAL, "sft_masked_writeback_many: bad matrix list");
    for (int32_t i = 0; i < n_mats; ++i) {
        const sft_wb_mat &m = mats[i];
        SFT_CHECK(m.R >= 0 && m.C > 0 && m.n_active >= 0 && m.n_active <= m.R, SFT_EINVAL,
                  "sft_masked_writeback_many: matrix %d: bad sizes", i);
        SFT_CHECK(m.C % 8 == 0, SFT_ESHAPE, "sft_masked_writeback_many: matrix %d: C=%lld is not a multiple of 8", i,
                  (long long)m.C);
        if (m.n_active == 0) continue;
        SFT_CHECK(m.q && m.s && m.delta && m.active_rows && m.w_live, SFT_EINVAL,
                  "sft_masked_writeback_many: matrix %d: null pointer", i);
        SFT_CHECK(sft::aligned16(m.q) && sft::aligned16(m.delta) && sft::aligned16(m.w_live), SFT_EALIGN,
                  "sft_masked_writeback_many: matrix %d: buffer not 16-byte aligned", i);
    }
    // Matrices go out in batches of kMaxMats per launch (kernel-argument table).
    for (int32_t base = 0; base < n_mats; base += kMaxMats) {
        WbParams p{};
        int64_t n_wg = 0;
        for (int32_t i = base; i < std::min(n_mats, base + kMaxMats); ++i) {
            const sft_wb_mat &m = mats[i];
            if (m.n_active == 0) continue;
            p.mat[p.n_mats++] = WbMatDev{m.q, m.s, m.delta, m.active_rows, m.w_live, m.C, n_wg};
            n_wg += m.n_active;
        }
        if (n_wg == 0) continue;
        SFT_CHECK(n_wg < (int64_t(1) << 31), SFT_ENOTSUP, "sft_masked_writeback_many: too many rows");
        hipLaunchKernelGGL(k_masked_writeback_many, dim3(static_cast<uint32_t>(n_wg)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), p);
        if (int rc = launch_status("sft_masked_writeback_many")) return rc;
    }
    return SFT_OK;
}

}  // extern "C"

namespace {

// Validation and batched launches shared by sft_rows_save / sft_rows_restore.
int rows_copy(const sft_ckpt_mat *mats, int32_t n_mats, void *stream, bool restore, const char *who) {
    sft::clear_error();
    SFT_CHECK(n_mats >= 0 && (n_mats == 0 || mats), SFT_EINVAL, "%s: bad matrix list", who);
    int64_t total = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const sft_ckpt_mat &m = mats[i];
        SFT_CHECK(m.R >= 0 && m.C > 0 && m.n_rows >= 0 && m.n_slots >= 0, SFT_EINVAL,
                  "%s: matrix %d: bad sizes (R=%lld C=%lld n_rows=%lld)", who, i, (long long)m.R,
                  (long long)m.C, (long long)m.n_rows);
        SFT_CHECK(m.n_rows <= m.R && m.n_rows <= m.n_slots, SFT_EINVAL,
                  "%s: matrix %d: n_rows=%lld exceeds R or n_slots", who, i, (long long)m.n_rows);
        SFT_CHECK(m.C % 8 == 0, SFT_ESHAPE, "%s: matrix %d: C=%lld is not a multiple of 8", who, i,
                  (long long)m.C);
        if (m.n_rows == 0) continue;
        SFT_CHECK(m.rows && m.slot && m.q && m.s && m.delta && m.m && m.v && m.t && m.mv_exp && m.ck_q &&
                      m.ck_s && m.ck_delta && m.ck_m && m.ck_v && m.ck_t && m.ck_mv_exp,
                  SFT_EINVAL, "%s: matrix %d: null device pointer", who, i);
        SFT_CHECK(sft::aligned16(m.q) && sft::aligned16(m.delta) && sft::aligned16(m.m) && sft::aligned16(m.v) &&
                      sft::aligned16(m.ck_q) && sft::aligned16(m.ck_delta) && sft::aligned16(m.ck_m) &&
                      sft::aligned16(m.ck_v) && (!m.w_live || sft::aligned16(m.w_live)),
                  SFT_EALIGN, "%s: matrix %d: a row-major buffer is not 16-byte aligned", who, i);
        total += m.n_rows;
    }
    SFT_CHECK(total < (int64_t(1) << 31), SFT_ENOTSUP, "%s: %lld rows in one call", who, (long long)total);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    CkParams p{};
    int64_t rows = 0;
    auto flush = [&]() -> int {
        if (p.n_mats == 0) return SFT_OK;
        if (restore)
            hipLaunchKernelGGL(k_rows_copy<true>, dim3(static_cast<uint32_t>(rows)), dim3(kCkThreads), 0, st, p);
        else
            hipLaunchKernelGGL(k_rows_copy<false>, dim3(static_cast<uint32_t>(rows)), dim3(kCkThreads), 0, st, p);
        const int rc = launch_status(who);
        p = CkParams{};
        rows = 0;
        return rc;
    };
    for (int32_t i = 0; i < n_mats; ++i) {
        if (mats[i].n_rows == 0) continue;
        if (p.n_mats == kCkMats)
            if (int rc = flush()) return rc;
        p.mat[p.n_mats].m = mats[i];
        p.mat[p.n_mats].row_begin = rows;
        ++p.n_mats;
        rows += mats[i].n_rows;
    }
    return flush();
}

}  // namespace

extern "C" {

int sft_rows_save(const sft_ckpt_mat *mats, int32_t n_mats, void *stream) {
    return rows_copy(mats, n_mats, stream, false, "sft_rows_save");
}

int sft_rows_restore(const sft_ckpt_mat *mats, int32_t n_mats, void *stream) {
    return rows_copy(mats, n_mats, stream, true, "sft_rows_restore");
}

}  // extern "C"
