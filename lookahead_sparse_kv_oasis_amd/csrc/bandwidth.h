// Measurement helper, not part of the decode path: a streaming read of device
// memory that gives the box's own HBM read rate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oasis {

// Streaming read of bytes (a multiple of 16) at buf by `workgroups`
// workgroups; sink[w] receives the XOR of the 32-bit words workgroup w read.
hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int workgroups,
                              hipStream_t st);

}  // namespace oasis
