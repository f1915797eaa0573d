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

// One job of a batched column-wise launch: a ColLaunch's tensor plus its
// rounding and its range of 128 x 128 tiles (gx tiles per tile row, the
// first at workgroup `first`).
struct ColJob {
    const uint16_t *x;
    int64_t rows, cols, ld;
    OutDesc out;
    QKnobs kn;
    int64_t first;
    int64_t gx;
    int32_t vec;
    int32_t round;
};
constexpr int kColBatchMax = 8;
constexpr int kBatchMixed = 2;  // a batch launch with both SR and RTNE jobs
struct ColBatch {
    ColJob job[kColBatchMax];
    int32_t n;
};
// Launch of the batched kernel: every job of b shares the grid family, the
// rotation size hn and the column code format fmt; `tiles` = the jobs' total.
hipError_t launch_quant_col_batch(int grid, int hn, int fmt, const ColBatch &b, int64_t tiles,
                                  hipStream_t s);

// Launch of the row-wise-only quantize kernel (two lanes per block).
struct RowLaunch {
    const uint16_t *x;
    uint64_t nblocks;  // rows * cols / 32
    uint32_t nbr;      // blocks per row
    int64_t ld;
    int dense;         // ld == cols
    int vec;           // x 16-byte aligned and ld % 8 == 0: 128-bit loads
    OutDesc out;
    QKnobs kn;
    hipStream_t s;
};
hipError_t launch_quant_row16(int grid, int round, int hn, const RowLaunch &q);

// Launch of the kernel that writes both outputs from one read.
struct DualLaunch {
    const uint16_t *x;
    int64_t rows, cols, ld;
    OutDesc rout, cout;
    int vec;  // x 8-byte aligned and ld % 4 == 0: 64-bit loads
    QKnobs kn;
    hipStream_t s;
};
hipError_t launch_quant_dual16(int grid, int round, int hn, const DualLaunch &q);

// Statistics (dequant_stats.hip): the argument checks of mxq_bias_stats other
// than the workspace's, the workspace it needs, and the launch of its kernels
// with the workgroup partials in `part`.
mxq_status check_stats(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                       int64_t ld_x, int32_t axis, const mxq_qtensor *q, const mxq_stats *out);
size_t stats_workspace_bytes(int64_t rows, int64_t cols, int32_t axis);
mxq_status launch_stats(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                        int64_t ld_x, int32_t axis, const mxq_qtensor *q, mxq_stats *out,
                        double *part, hipStream_t s);

}  // namespace mxq
