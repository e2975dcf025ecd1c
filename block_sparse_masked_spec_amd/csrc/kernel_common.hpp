// Device helpers shared by the forward and backward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace sa {

constexpr int kXcds = 8;  // MI355X: 8 accelerator dies, each with its own L2

// The plan is written before the launch and only read by the kernel, so it
// can be read through the constant address space: uniform reads become
// scalar loads, which do not share a wait counter with the tile loads.
template <typename T>
__device__ __forceinline__ T ldc(const T* p, int i) {
    return ((const __attribute__((address_space(4))) T*)p)[i];
}

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

// Block mode: bit x is set iff key k0 + x lies in one of the allowed key-block
// intervals [iv[2t], iv[2t+1]) (in blocks of size blk) of query block qblk.
__device__ __forceinline__ uint64_t block_word(int blk, const int32_t* ptr, const int32_t* iv,
                                               int qblk, int k0) {
    uint64_t w = 0;
    for (int t = ptr[qblk]; t < ptr[qblk + 1]; ++t) {
        const long lo = long(iv[2 * t]) * blk - k0, hi = long(iv[2 * t + 1]) * blk - k0;
        if (hi > 0 && lo < 64) {
            const int l0 = lo < 0 ? 0 : int(lo), h0 = hi > 64 ? 64 : int(hi);
            w |= (h0 >= 64 ? ~0ull : ((1ull << h0) - 1ull)) & ~((1ull << l0) - 1ull);
        }
    }
    return w;
}

// Bits [0, n) set, n clamped to [0, 64].
__device__ __forceinline__ uint64_t low_bits(int n) {
    return n <= 0 ? 0ull : (n >= 64 ? ~0ull : ((1ull << n) - 1ull));
}

// Allowed keys of query qi among the 64 keys starting at k0, as a bit word:
// (band OR column keys OR block-mode key blocks OR a global query row) AND
// key < T AND the causal cut.  colw is the column-key bit word of the tile;
// the band is the distance range thinned to the dilation grid (qres = qi mod
// g, k0res = k0 mod g, both 0 when g = 1); qblk is the query's block in
// block mode, where the token band is empty.
__device__ __forceinline__ uint64_t allowed_word(const FwdArgs& a, int qi, int k0, bool rowg,
                                                 uint64_t colw, int qres, int k0res, int qblk) {
    uint64_t w = rowg ? ~0ull : colw;
    const long lo = long(qi) - a.band_back - k0;           // first band offset
    const long hi = long(qi) + long(a.band_fwd) - k0 + 1;  // one past the last
    if (!rowg && hi > 0 && lo < 64) {
        const int l0 = lo < 0 ? 0 : int(lo), h0 = hi > 64 ? 64 : int(hi);
        uint64_t band = low_bits(h0) & ~low_bits(l0);
        if (a.dil != 1) band &= grid_word(a.dil_pat, a.dil, qres, k0res);
        w |= band;
    }
    if (a.blk > 0 && !rowg) w |= block_word(a.blk, a.blk_ptr, a.blk_iv, qblk, k0);
    w &= low_bits(a.T - k0);
    if (a.causal) w &= low_bits(qi - k0 + 1);
    return w;
}

// The same rule read by key: bit x is set iff query q0 + x may read key j.
// colj: key j is a strided or global column key; roww: bit x set iff query
// q0 + x is a global row.
__device__ __forceinline__ uint64_t allowed_word_T(const FwdArgs& a, int j, int q0, bool colj,
                                                   uint64_t roww) {
    uint64_t w = colj ? ~0ull : roww;
    if (!colj) {
        // band: i - j in [-fwd, back], i.e. x in [j - fwd - q0, j + back - q0]
        const long lo = long(j) - a.band_fwd - q0;
        const long hi = long(j) + long(a.band_back) - q0 + 1;
        if (hi > 0 && lo < 64) {
            const int l0 = lo < 0 ? 0 : int(lo), h0 = hi > 64 ? 64 : int(hi);
            uint64_t band = low_bits(h0) & ~low_bits(l0);
            if (a.dil != 1) band &= grid_word(a.dil_pat, a.dil, j % a.dil, q0 % a.dil);
            w |= band;
        }
        if (a.blk > 0) {  // query blocks of the tile whose intervals hold key block j / blk
            const int kbj = j / a.blk;
            const int qe = min(q0 + 64, a.T);
            for (int qb = q0 / a.blk; qb * a.blk < qe; ++qb) {
                bool hit = false;
                for (int t = a.blk_ptr[qb]; t < a.blk_ptr[qb + 1]; ++t)
                    hit |= a.blk_iv[2 * t] <= kbj && kbj < a.blk_iv[2 * t + 1];
                if (hit) {
                    const int l0 = max(qb * a.blk, q0) - q0, h0 = min((qb + 1) * a.blk, qe) - q0;
                    w |= low_bits(h0) & ~low_bits(l0);
                }
            }
        }
    }
    w &= low_bits(a.T - q0);
    if (a.causal) w &= ~low_bits(j - q0);  // i >= j
    return w;
}

}  // namespace sa
