// Measurement helpers of libaql.so (internal; not part of the method): the
// attainable read and int8 MFMA ceilings. Declared apart from common.h so that
// the linears' shared header does not change with them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aql {

hipError_t launch_measure_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_measure_mfma_i8(int64_t iters, int32_t *sink, hipStream_t st);

}  // namespace aql
