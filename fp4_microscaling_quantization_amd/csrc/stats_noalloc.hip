// mxq_bias_stats_noalloc: mxq_bias_stats with its workspace in a static
// device array, for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` holds the statistics kernels' workgroup partials: at
// most 1024 workgroups x 25 eight-byte sums = 204800 bytes, the largest
// workspace mxq_bias_stats ever asks for (its workgroup count is capped).
// Each GPU the library runs on holds its own copy until the process ends.
// In host code the name `scratch` is only a stand-in for the symbol, never a
// device address: the address is taken once per device with
// hipGetSymbolAddress (with that device current) and cached, and only that
// address is handed to the kernels.  The kernels write every partial slot the
// final reduction reads, so nothing needs clearing between calls.  Calls
// that overlap on one GPU share the array and race.
#include <mutex>

#include "mxq_host.hpp"

static constexpr size_t kScratchBytes = 204800;

static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
double *g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call on each device).
mxq_status scratch_address(double **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MXQ_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MXQ_ERR_DEVICE;
        g_ptr[dev] = static_cast<double *>(p);
    }
    *out = g_ptr[dev];
    return MXQ_OK;
}

}  // namespace

extern "C" mxq_status mxq_bias_stats_noalloc(const mxq_qconfig *cfg, const void *x, int64_t rows,
                                             int64_t cols, int64_t ld_x, int32_t axis,
                                             const mxq_qtensor *q, mxq_stats *out, void *stream)
{
    const mxq_status st = mxq::check_stats(cfg, x, rows, cols, ld_x, axis, q, out);
    if (st)
        return st;
    if (mxq::stats_workspace_bytes(rows, cols, axis) > kScratchBytes)
        return MXQ_ERR_WORKSPACE;
    double *part = nullptr;
    const mxq_status sa = scratch_address(&part);
    if (sa)
        return sa;
    return mxq::launch_stats(cfg, x, rows, cols, ld_x, axis, q, out, part,
                             static_cast<hipStream_t>(stream));
}
