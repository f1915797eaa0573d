// Host-side helpers shared by the entry points of libmxq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_device.hpp"
#include "quant_out.hpp"

namespace mxq {

mxq_status check_qconfig(const mxq_qconfig *cfg);
mxq_status check_qtensor_out(const mxq_qtensor *t, int32_t grid, int64_t k);
QKnobs make_knobs(const mxq_qconfig *cfg);

// Launch of the column-wise-only quantize kernel (quantize_col.hip).
struct ColLaunch {
    const uint16_t *x;
    int64_t rows, cols, ld;
    OutDesc out;
    int vec;  // x 8-byte aligned and ld % 4 == 0: 64-bit loads
    QKnobs kn;
    hipStream_t s;
};
hipError_t launch_quant_col(int grid, int round, int hn, const ColLaunch &q);

}  // namespace mxq
