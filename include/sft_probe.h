/*
 * sft_probe.h -- measurement probes of libsft (not part of the training
 * step): what the device sustains, measured beside the published peaks that
 * the hot path's roofline fractions are quoted against.
 */
#ifndef SFT_PROBE_H
#define SFT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "sft.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * What this device sustains, measured beside the published peaks that the
 * kernels' roofline fractions use.  Each launches sft_probe_grid()
 * workgroups of 256 lanes (8 per CU) and returns without synchronising.
 *   sft_probe_read: streams `bytes` (a multiple of 16, 16-byte aligned) with
 *     16-byte non-temporal loads and writes one XOR per lane to sink
 *     [sft_probe_grid() * 256] (the XOR of sink equals the XOR of the buffer's
 *     32-bit words);
 *   sft_probe_copy: copies `bytes` from src to dst the same way;
 *   sft_probe_mfma: each wave issues 4 * iters v_mfma_f32_32x32x16_bf16 on
 *     register operands (every input 1/16) and writes each lane's sum to out
 *     [sft_probe_grid() * 256], which equals 4 * iters (iters < 2^22 keeps it
 *     exact); work = sft_probe_grid() * 4 waves * 4 * iters * 32768 FLOP.
 * Errors: SFT_EINVAL (null or unaligned pointers, bad sizes), SFT_EHIP.
 */
int sft_probe_grid(void);
int sft_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
int sft_probe_copy(const void *src, void *dst, size_t bytes, void *stream);
int sft_probe_mfma(int64_t iters, float *out, void *stream);

/*
 * How sft_masked_dw would launch these groups (host only: nothing runs on the
 * device and no device pointer is read; the groups' pointers need only be
 * non-null where sft_masked_dw requires them).  cus: the compute units to
 * plan for (0: this device's count).  Writes, for each product launch in
 * order, its kind (0 stream-K slices, 1 slices aligned to the output tiles,
 * 2 team slices, 3 narrow whole tiles), its workgroups with work, its group
 * count, then per group the narrow tile shape (0 two waves per packed tile,
 * 1 one wave per packed tile over 64 columns, 2 over 128 columns; 0 outside
 * narrow launches), its M-blocks and its column blocks; at most `cap` values
 * go to out.  Returns the number of values (more than cap if out was too
 * short), or an error code (< 0): SFT_EINVAL (bad groups or arguments),
 * SFT_ENOTSUP (a launch beyond 2^31 iterations).
 */
int sft_probe_dw_plan(const sft_dw_group *groups, int32_t n_groups, int32_t cus, int32_t *out, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* SFT_PROBE_H */
