// Device helpers shared by the forward kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace sa {

constexpr int kXcds = 8;  // MI355X: 8 accelerator dies, each with its own L2

// Workgroups are handed to the dies round-robin (block b runs on die b % 8).
// Remap block ids so that each die walks one contiguous slice of the work
// list -- whole heads, query blocks in plan order -- which keeps the K/V
// tiles that neighbouring query blocks share inside that die's L2.
// Returns the logical work index in [0, total).
__device__ __forceinline__ int xcd_slice_index(int block, int total) {
    const int q = total / kXcds, r = total % kXcds;
    const int die = block % kXcds, local = block / kXcds;
    return die * q + min(die, r) + local;
}

// Dilated windows: bit x of the result is set iff key k0 + x is on query
// qi's grid, qi - (k0 + x) = 0 (mod g).  pat has bits 0, g, 2g, ... below 64;
// qres = qi mod g and k0res = k0 mod g.
__device__ __forceinline__ uint64_t grid_word(uint64_t pat, int g, int qres, int k0res) {
    int start = qres - k0res;
    if (start < 0) start += g;
    return start < 64 ? pat << start : 0ull;
}

}  // namespace sa
