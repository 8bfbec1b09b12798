/*
 * ifa_probe.h — measurement utility of libifadecode (not an attention operation).
 *
 * The decode kernels are bound by HBM reads.  Their achieved bandwidth is
 * reported against MI355X's published peak and against the practical read
 * ceiling of the device, which this probe measures: it streams a buffer the
 * way the decode kernels stream K/V (16 bytes per lane, nontemporal, eight
 * loads in flight per lane, coalesced) and computes nothing else.
 */
#ifndef IFA_PROBE_H
#define IFA_PROBE_H

#include <stddef.h>

#include "ifa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes of device memory at `src` once, on `stream`, and
 * returns without waiting.  src: caller-owned device memory, 16-byte aligned;
 * bytes: a positive multiple of 16; sink: caller-owned device memory of at
 * least 4 bytes, which the kernel may write (its content is meaningless).
 * Returns IFA_ERR_PARAM_NULLPTR for a NULL src or sink,
 * IFA_ERR_PARAM_INVALID for a size or alignment outside that, and
 * IFA_ERR_RUNTIME when the HIP launch fails; nothing is launched on an error.
 */
int ifa_read_probe(const void *src, size_t bytes, void *sink, ifa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* IFA_PROBE_H */
