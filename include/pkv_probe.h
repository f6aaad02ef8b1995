/*
 * pkv_probe.h -- measurement probe of libpagedkv.so (not part of the decode
 * path): the streaming-read bandwidth the device's HBM delivers to a plain
 * read, the reference next to which the decode kernels' KV-read rate is
 * reported.  Decode reads every cached byte once per step, so its speed is
 * a bandwidth question ([B] "KV Cache Engineering: PagedAttention,
 * Continuous Batching, Attention Variants, and the Bandwidth Wall", "Two
 * Costs: Capacity and Bandwidth").
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_stream_read -- read `bytes` bytes of the device buffer `buf` once.
 * `waves` waves (64 lanes each, 4 per work-group) each read one contiguous
 * chunk of bytes / waves bytes with 16-byte non-temporal loads, 8 per lane
 * in flight; the loaded words are folded into a checksum that is written
 * to sink[0..63] only in the (practically impossible) case that it equals
 * a fixed constant, so sink is a 256-byte device buffer that is almost
 * never written.  Enqueued on `stream`; nothing is allocated.
 *
 *  buf   : device pointer, 16-byte aligned (caller-owned, read only)
 *  bytes : > 0, a multiple of waves * 8192
 *  waves : > 0, a multiple of 4
 *  sink  : device pointer to 64 uint32 (caller-owned)
 * Returns PKV_OK, PKV_EINVAL for a null / misaligned pointer or sizes that
 * break the rules above, PKV_ELAUNCH if the launch failed.
 */
int pkv_stream_read(const void* buf, int64_t bytes, int32_t waves, uint32_t* sink,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
