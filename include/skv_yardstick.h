/* skv_yardstick.h — a streaming-read yardstick beside the decode-step
 * library (libskv_yardstick.so; not part of libsparsekv).
 *
 * skv_read_probe reads `bytes` (a multiple of 16) of the device buffer buf
 * once, with n_wg workgroups of 256 threads issuing 16-byte loads, and writes
 * one folded word per workgroup to sink (device [n_wg]) so no load is dead.
 * Its duration measures what a plain read reaches on the device, the second
 * yardstick beside the published HBM peak for the decode step's rooflines.
 * Asynchronous on stream.  Returns 0, 1 on a bad argument (null pointer,
 * size not a positive multiple of 16, n_wg < 1) or 4 if the launch failed.
 */
#ifndef SKV_YARDSTICK_H
#define SKV_YARDSTICK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t skv_read_probe(const void* buf, size_t bytes, int32_t n_wg, uint32_t* sink,
                       hipStream_t stream);

/* skv_read_probe with nontemporal != 0: the loads are marked non-temporal
 * (data read once, not kept in the caches). */
int32_t skv_read_probe_ex(const void* buf, size_t bytes, int32_t n_wg, int32_t nontemporal,
                          uint32_t* sink, hipStream_t stream);

/* Reads n_pieces 4 KB pieces of buf (device, at least 4096 n_pieces bytes)
 * in the order given by order[0 .. n_pieces) (device int32 piece indices,
 * each in [0, n_pieces)), one piece per wave at a time, four in flight per
 * wave, with n_wg workgroups of 256 threads; one folded word per workgroup
 * to sink.  The access pattern of a scan over 4 KB runs in permuted block
 * order.  Returns 0, 1 on a bad argument or 4 if the launch failed. */
int32_t skv_read_pieces(const void* buf, const int32_t* order, int64_t n_pieces, int32_t n_wg,
                        uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SKV_YARDSTICK_H */
