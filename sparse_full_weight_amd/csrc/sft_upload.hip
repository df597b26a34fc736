// sft_upload.hip -- the step's plan shipped to the device by a kernel that
// reads it straight from pinned host memory, on the caller's stream.
//
// Method: "Sparse-First Fine-Tuning: Full-Weight Training at the Cost of the
// Active Set", section 2.6 and Figure 2: the CPU derives the step's masks a
// step ahead and the GPU receives them once per step, with nothing copied
// back.  The plan of a 7B-shaped layer at 1% rows is a few KB, so the copy is
// one PCIe round trip; doing it in a kernel of its own keeps it in the
// stream's order without the runtime's copy path (whose host-to-device
// copies, issued from several streams at once, stalled for milliseconds at
// a time).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "sft_internal.h"

namespace {

constexpr int kUpThreads = 256;
constexpr int kUpMaxBlocks = 64;

// dst[i] = src[i] for the n16 16-byte words, then the tail's 4-byte words
// (grid-stride; src is the device address of the pinned host buffer).
__global__ __launch_bounds__(kUpThreads) void k_plan_upload(uint4 *__restrict__ dst, const uint4 *__restrict__ src,
                                                           int64_t n16, int64_t tail) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kUpThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kUpThreads + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
    if (blockIdx.x == 0 && threadIdx.x < tail)
        reinterpret_cast<uint32_t *>(dst + n16)[threadIdx.x] = reinterpret_cast<const uint32_t *>(src + n16)[threadIdx.x];
}

}  // namespace

extern "C" int sft_plan_upload(void *dst, const void *src, size_t bytes, void *stream) {
    sft::clear_error();
    if (bytes == 0) return SFT_OK;
    SFT_CHECK(dst && src, SFT_EINVAL, "sft_plan_upload: null pointer");
    SFT_CHECK(bytes % 4 == 0, SFT_ESHAPE, "sft_plan_upload: %zu bytes is not whole 4-byte words", bytes);
    SFT_CHECK(bytes < (size_t(1) << 31), SFT_ENOTSUP, "sft_plan_upload: %zu bytes reach 2^31", bytes);
    SFT_CHECK(sft::aligned16(dst) && sft::aligned16(src), SFT_EALIGN,
              "sft_plan_upload: dst or src not 16-byte aligned");
    void *dsrc = nullptr;
    const hipError_t e = hipHostGetDevicePointer(&dsrc, const_cast<void *>(src), 0);
    if (e != hipSuccess || !dsrc) {
        (void)hipGetLastError();   // the failed lookup is ours to report: clear it for the caller's next call
        return sft::fail(SFT_EINVAL, "sft_plan_upload: src is not pinned host memory (%s)", hipGetErrorString(e));
    }
    const int64_t n16 = static_cast<int64_t>(bytes / 16), tail = static_cast<int64_t>((bytes % 16) / 4);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(kUpMaxBlocks, (n16 + kUpThreads - 1) / kUpThreads));
    hipLaunchKernelGGL(k_plan_upload, dim3(static_cast<uint32_t>(blocks)), dim3(kUpThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint4 *>(dst), static_cast<const uint4 *>(dsrc),
                       n16, tail);
    const hipError_t le = hipGetLastError();
    SFT_CHECK(le == hipSuccess, SFT_EHIP, "sft_plan_upload: launch failed: %s", hipGetErrorString(le));
    return SFT_OK;
}
