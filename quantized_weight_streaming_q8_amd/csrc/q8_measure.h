// q8_measure.h -- the read-ceiling kernel's launcher (see q8_measure.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Plain read of `bytes` (a multiple of 16) at buf, 16-byte aligned; sink
// holds kStreamSinkWords uint32.
constexpr int kStreamSinkWords = 1024;
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace q8
