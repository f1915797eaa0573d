// Output placement shared by the quantize kernels: where block (line, jb) of
// a quantized tensor goes in MXQ_LAYOUT_ROWS or MXQ_LAYOUT_MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"

namespace mxq {

// Where an output's blocks go (MXQ_LAYOUT_ROWS or MXQ_LAYOUT_MFMA).
struct OutDesc {
    uint8_t *codes;
    uint8_t *scales;
    int fmt;
    int layout;
    uint64_t nbk;     // blocks per line
    uint64_t ntiles;  // 16-line tiles (MFMA layout)
};

__device__ __forceinline__ uint64_t code_offset(const OutDesc &o, uint64_t line, uint64_t jb, int bb)
{
    if (o.layout == MXQ_LAYOUT_ROWS)
        return (line * o.nbk + jb) * bb;
    // [step = jb / 4][tile = line / 16][lane = 16 (jb % 4) + line % 16]
    return (((jb >> 2) * o.ntiles + (line >> 4)) * 64 + 16 * (jb & 3) + (line & 15)) * bb;
}

__device__ __forceinline__ uint64_t scale_offset(const OutDesc &o, uint64_t line, uint64_t jb)
{
    if (o.layout == MXQ_LAYOUT_ROWS)
        return line * o.nbk + jb;
    // [group = jb / 16][tile][lane] words, byte = step within the group
    return (((jb >> 4) * o.ntiles + (line >> 4)) * 64 + 16 * (jb & 3) + (line & 15)) * 4 +
           ((jb >> 2) & 3);
}

}  // namespace mxq
