// sft_probe.hip -- measurement probes: the HBM read and copy rates and the
// dense bf16 matrix-core rate this MI355X actually sustains, measured beside
// the published peaks (8 TB/s, 2.5 PFLOP/s) that the kernels' roofline
// fractions are taken against.
//
// - read: every lane streams 16-byte loads, four in flight, over a grid of
//   8 workgroups per CU, and folds them into one XOR per lane (written to a
//   sink so the loads cannot be dropped);
// - copy: the same loop writing each chunk to a second buffer;
// - mfma: each wave issues v_mfma_f32_32x32x16_bf16 back to back on four
//   independent accumulator sets (no waits between dependent instructions),
//   operands in registers, for `iters` rounds; the sums leave through `out`.
#include <hip/hip_runtime.h>

#include "sft_internal.h"
#include "sft_probe.h"

namespace {

constexpr int kProbeThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const u32x4 *__restrict__ src, int64_t n16,
                                                              uint32_t *__restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
    u32x4 acc = {0, 0, 0, 0};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kProbeThreads) void k_probe_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                              int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + stride);
        __builtin_nontemporal_store(c, dst + i + 2 * stride);
        __builtin_nontemporal_store(d, dst + i + 3 * stride);
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Operands: every bf16 of A and B is 1/16 (exact), so each MFMA adds
// 16 * (1/16)^2 = 1/16 to every accumulator element: after `iters` rounds an
// element of each of the four sets holds iters/16, exact while iters < 2^28.
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(int64_t iters, float *__restrict__ out) {
    const bf16x8 a = {0.0625, 0.0625, 0.0625, 0.0625, 0.0625, 0.0625, 0.0625, 0.0625};
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c3, 0, 0, 0);
    }
    const f32x16 s = c0 + c1 + c2 + c3;
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) t += s[e];
    out[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = t;
}

int launch_status(const char *who) {
    const hipError_t e = hipGetLastError();
    SFT_CHECK(e == hipSuccess, SFT_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return SFT_OK;
}

}  // namespace

extern "C" {

int sft_probe_grid(void) { return sft::num_cus() * 8; }

int sft_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    sft::clear_error();
    SFT_CHECK(buf && sink && sft::aligned16(buf) && bytes % 16 == 0, SFT_EINVAL,
              "sft_probe_read: null or unaligned buffer, or size not a multiple of 16");
    hipLaunchKernelGGL(k_probe_read, dim3(sft_probe_grid()), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(buf), static_cast<int64_t>(bytes / 16), sink);
    return launch_status("sft_probe_read");
}

int sft_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    sft::clear_error();
    SFT_CHECK(src && dst && sft::aligned16(src) && sft::aligned16(dst) && bytes % 16 == 0, SFT_EINVAL,
              "sft_probe_copy: null or unaligned buffer, or size not a multiple of 16");
    hipLaunchKernelGGL(k_probe_copy, dim3(sft_probe_grid()), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), static_cast<int64_t>(bytes / 16));
    return launch_status("sft_probe_copy");
}

int sft_probe_mfma(int64_t iters, float *out, void *stream) {
    sft::clear_error();
    SFT_CHECK(out && iters >= 0 && iters < (int64_t(1) << 28), SFT_EINVAL, "sft_probe_mfma: bad arguments");
    hipLaunchKernelGGL(k_probe_mfma, dim3(sft_probe_grid()), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                       iters, out);
    return launch_status("sft_probe_mfma");
}

}  // extern "C"
