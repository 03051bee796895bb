/*
 * tq_probe.h -- measurement aid beside libtq (libtq_probe.so), not part of the method.
 *
 * Error codes are tq.h's. The call is asynchronous on stream (a hipStream_t, or null for the
 * default stream); buf and sink are device pointers owned by the caller.
 */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads bytes (a multiple of 16) of buf with a plain streaming kernel, so that the decode's
 * HBM rate can be set against the read rate a simple kernel reaches on the same GPU.
 * sink: device scratch of >= CUs * 1024 * 4 bytes (TQ_ENOSPC otherwise; 2 MiB always
 * suffices), overwritten with the XOR of the words each thread read. TQ_EINVAL for a null
 * pointer or a size not a multiple of 16; TQ_EDEVICE if the launch fails. */
int tq_stream_read_probe(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
