// MFMA tile helpers shared by the generic forward and the backward kernels
// (gfx950): per element type, the 32x32 MFMA flavour and its lane fragments;
// per head size, the LDS tile geometry; and the staging of 64-row tiles into
// LDS, row-major or transposed.
//
// Fragment conventions (32x32 MFMA, "k" the contracted dimension): an A or B
// fragment of lane l covers MFMA row/column l % 32 and the k-elements
// [VPL * (l / 32), VPL * (l / 32) + VPL) of one k-step; the f32x16
// accumulator register r of lane l is row (r / 4) * 8 + (l / 32) * 4 + r % 4,
// column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.hpp"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
static_assert(kBQ == kWaves * 32, "one 32-query MFMA column block per wave");
static_assert(kBK == 64, "column bit words cover exactly one key tile");

// Per element type: MFMA flavour, lane fragment and 16-byte chunk views.
template <typename E>
struct Ops;

template <>
struct Ops<__bf16> {
    static constexpr int VPL = 8;  // elements per lane per MFMA k-step
    using frag = bf16x8;
    using chunk = bf16x8;  // one 16-byte global chunk
    using quad = bf16x4;   // 4 keys of one transposed V row
    __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // Scores rb .. rb+7 of one 32-key block as a B fragment.
    template <int RB>
    __device__ static frag pack(const f32x16& s) {
        frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(s[RB + e]);
        return r;
    }
    __device__ static frag zero() { return frag{}; }
};

template <>
struct Ops<float> {
    static constexpr int VPL = 1;
    using frag = float;
    using chunk = f32x4;
    using quad = f32x4;
    __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    template <int RB>
    __device__ static frag pack(const f32x16& s) {
        return s[RB];
    }
    __device__ static frag zero() { return 0.f; }
};

template <typename E, int D>
struct Shape {
    static constexpr int EPC = 16 / sizeof(E);        // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;               // chunks per K/V row
    static constexpr int KLD = D + EPC;               // K row stride (16-byte pad)
    static constexpr int NDB = D >= 32 ? D / 32 : 1;  // 32-row blocks of d
    static constexpr int VROWS = NDB * 32;            // rows of the V^T tile
    static constexpr int VLD = kBK + EPC;             // V^T row stride (16-byte pad)
    static constexpr int VPL = Ops<E>::VPL;
    static constexpr int KSTEP = 2 * VPL;             // MFMA k per instruction
    static constexpr int NKS = D / KSTEP;             // k-steps of S^T = K Q^T
    static constexpr int PKS = kBK / KSTEP;           // k-steps of O^T += V^T P^T
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// MFMA row m of a 32-key block holds key swap23(m) of that block.
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Stage 64 rows of a [T][d] tensor row-major into dst (row stride KLD).
// key_of(row) gives the source row of tile row `row`, or -1 for an unused row
// (filled with zeros).
template <typename E, int D, typename KeyOf>
__device__ __forceinline__ void stage_rows(E* dst, const E* src, KeyOf key_of, int tid) {
    using S = Shape<E, D>;
    using chunk = typename Ops<E>::chunk;
#pragma unroll
    for (int c = tid; c < kBK * S::CPR; c += kThreads) {
        const int row = c / S::CPR, col = c % S::CPR;
        const int key = key_of(row);
        chunk v{};
        if (key >= 0) v = *reinterpret_cast<const chunk*>(src + size_t(key) * D + col * S::EPC);
        *reinterpret_cast<chunk*>(dst + row * S::KLD + col * S::EPC) = v;
    }
}

// Stage the same 64 rows transposed: dst[e][row] (row stride VLD), so that a
// lane reads several consecutive rows of one column with one load.
template <typename E, int D, typename KeyOf>
__device__ __forceinline__ void stage_cols(E* dst, const E* src, KeyOf key_of, int tid) {
    using S = Shape<E, D>;
    using chunk = typename Ops<E>::chunk;
    using quad = typename Ops<E>::quad;
#pragma unroll
    for (int b = tid; b < (kBK / 4) * S::CPR; b += kThreads) {
        const int rg = b % (kBK / 4), col = b / (kBK / 4);
        chunk x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key_of(rg * 4 + i);
            x[i] = chunk{};
            if (key >= 0) x[i] = *reinterpret_cast<const chunk*>(src + size_t(key) * D + col * S::EPC);
        }
#pragma unroll
        for (int e = 0; e < S::EPC; ++e) {
            quad q;
            q[0] = x[0][e];
            q[1] = x[1][e];
            q[2] = x[2][e];
            q[3] = x[3][e];
            *reinterpret_cast<quad*>(dst + (col * S::EPC + e) * S::VLD + rg * 4) = q;
        }
    }
}

// Stage one 64-key tile: K row-major, V transposed.
template <typename E, int D, typename KeyOf>
__device__ __forceinline__ void stage(E* k_lds, E* vt_lds, const E* Kp, const E* Vp,
                                      KeyOf key_of, int tid) {
    stage_rows<E, D>(k_lds, Kp, key_of, tid);
    stage_cols<E, D>(vt_lds, Vp, key_of, tid);
}

}  // namespace
}  // namespace sa
