/*
 * oscar_probe.h - HBM read-bandwidth probe of liboscar.so.
 *
 * Measurement support, not part of the decode path: the history kernel is
 * bound by how fast HBM delivers its pages, so its roofline fraction is
 * reported against the published peak and against the rate this probe
 * reaches on the same device.  Same conventions as oscar.h (caller-owned
 * device memory, asynchronous on `stream`, OSCAR_* return codes with the
 * message in oscar_last_error()).
 */
#ifndef OSCAR_PROBE_H
#define OSCAR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `buf` once, as 16-byte loads
 * (non-temporal when `nontemporal` is non-zero, the kind the history kernel
 * uses for its code words) spread over every compute unit, eight loads in
 * flight per lane.  The loaded words are XOR-reduced per lane and `sink`
 * (device, one uint32) is written only when a lane's reduction equals a
 * fixed constant, so the loads cannot be elided and nearly nothing is
 * written.  buf must be 16-byte aligned and bytes a multiple of 16;
 * OSCAR_EINVAL otherwise.  Time it with events around the call. */
int oscar_probe_read(const void* buf, size_t bytes, int32_t nontemporal, uint32_t* sink, void* stream);

/* The history kernel's access pattern without its arithmetic: `waves`
 * one-wave workgroups, each reading its own contiguous bytes / waves share
 * front to back in 4096-byte blocks (four 16-byte loads per lane, each 1 KB
 * across the wave), four blocks in flight.  Loads are non-temporal when
 * `nontemporal` is non-zero; `sink` as above.  buf must be 16-byte aligned,
 * waves > 0 and bytes a multiple of waves x 4096; OSCAR_EINVAL otherwise. */
int oscar_probe_read_blocks(const void* buf, size_t bytes, int32_t nontemporal, int32_t waves, uint32_t* sink,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_PROBE_H */
