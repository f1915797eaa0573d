// Host-side helpers shared by the entry points of libmxq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"
#include "mxq_device.hpp"

namespace mxq {

mxq_status check_qconfig(const mxq_qconfig *cfg);
mxq_status check_qtensor_out(const mxq_qtensor *t, int32_t grid, int64_t k);
QKnobs make_knobs(const mxq_qconfig *cfg);

}  // namespace mxq
