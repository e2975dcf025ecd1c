// Fused forward kernel of masked sparse attention for gfx950 (MI355X).
//
// Computes, per query i, the softmax over the allowed set S_i only and the
// weighted sum of values ("Sparse attention", glossary.selfmadequant.com,
// section "Choose the available reads"), streaming over the live key tiles of
// the host plan so that excluded tiles are never loaded ("Sparse and
// sliding-window attention", getnybble.com, section "Implementation"; the
// streaming, rescaled softmax is the FlashAttention idea both that page and
// "Attention variants" section 1 mention, derived here from the definition).
//
// Work decomposition
//   * one workgroup = 4 wavefronts = one (batch*head, 128-query block);
//     wave w owns query rows q0 + 32w .. q0 + 32w + 31, one query per lane
//     column (lane % 32), the two lane halves (lane / 32) split the keys;
//   * per 64-key tile: K (row-major) and V (transposed) are staged in LDS;
//     S^T = K * Q^T on 32x32 MFMA (keys are the MFMA rows, queries the
//     columns) so every per-query quantity -- running max, running sum,
//     rescale factor -- lives in one lane; a row reduction is an in-lane
//     reduction plus one exchange between the lane halves;
//   * O^T += V^T * P^T on 32x32 MFMA, P rounded to the input type;
//   * keys are loaded into MFMA rows in a permuted order (bits 2 and 3 of the
//     row index swapped) so that the 8 scores a lane holds for one PV k-step
//     are 8 consecutive keys, read from V^T with one 16-byte LDS load.
//
// Masking: tiles the plan marks FULL run with no mask code; other in-place
// tiles evaluate the rule (causal cut, band distance, strided/global column
// bits, global row bit); gathered tiles only mask their unused slots.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.hpp"
#include "kernel_common.hpp"
#include "mfma_tiles.hpp"

namespace sa {
namespace {

enum { MASK_NONE = 0, MASK_RULE = 1, MASK_SLOTS = 2 };

template <typename E, int D>
struct WaveState {
    using S = Shape<E, D>;
    using O = Ops<E>;
    typename O::frag qf[S::NKS];
    f32x16 acc[S::NDB];
    float m_run;  // running max of the log2-scaled scores
    float l_run;  // running sum over this lane half's keys

    // One 64-key tile.  MODE selects the mask; k0 is the tile's first key
    // (MASK_RULE) and cnt its number of used slots (MASK_SLOTS).
    template <int MODE>
    __device__ __forceinline__ void step(const E* k_lds, const E* vt_lds, const FwdArgs& a, int n,
                                         int h, int qi, bool rowg, int k0, int cnt) {
        f32x16 s[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x16{};
            const E* kr = k_lds + (blk * 32 + swap23(n)) * S::KLD + h * S::VPL;
#pragma unroll
            for (int ks = 0; ks < S::NKS; ++ks)
                s[blk] = O::mma(*reinterpret_cast<const typename O::frag*>(kr + ks * S::KSTEP),
                                qf[ks], s[blk]);
        }
        if (MODE == MASK_RULE) {
            // One allowed-key word per lane, then a select per score.
            const uint64_t aw = allowed_word(
                a, qi, k0, rowg, a.colbits[k0 >> 6], a.dil == 1 ? 0 : qi % a.dil,
                a.dil == 1 ? 0 : k0 % a.dil, a.blk > 0 ? min(qi, a.T - 1) / a.blk : 0);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ko = blk * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                    s[blk][r] = ((aw >> ko) & 1) ? s[blk][r] : -INFINITY;
                }
        } else if (MODE == MASK_SLOTS) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ko = blk * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
                    if (ko >= cnt) s[blk][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[blk][r], a.scale_log2, -m_new));
                s[blk][r] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) acc[db] *= alpha;
        // O^T += V^T P^T, one MFMA k-step at a time.
        static_for<0, S::PKS>([&](auto kk_c) {
            constexpr int kk = decltype(kk_c)::value;
            constexpr int blk = (kk * S::VPL) >> 4;  // 32-key block of the scores
            constexpr int rb = (kk * S::VPL) & 15;   // first score register
            constexpr int koff = blk * 32 + (rb >> 3) * 16 + (rb & 7);
            const typename O::frag pf = O::template pack<rb>(s[blk]);
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
                const E* vr = vt_lds + (db * 32 + n) * S::VLD + koff + h * 8;
                acc[db] = O::mma(*reinterpret_cast<const typename O::frag*>(vr), pf, acc[db]);
            }
        });
    }
};

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void sa_fwd_kernel(FwdArgs a) {
    using S = Shape<E, D>;
    using O = Ops<E>;
    __shared__ __attribute__((aligned(16))) E k_lds[kBK * S::KLD];
    __shared__ __attribute__((aligned(16))) E vt_lds[S::VROWS * S::VLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int work = xcd_slice_index(blockIdx.x, gridDim.x);
    const int n_qb = gridDim.x / a.BH;
    const int bh = work / n_qb;
    const int qb = a.qb_order[work % n_qb];
    const int T = a.T;
    const size_t base = size_t(bh) * size_t(T) * D;
    const E* Qp = static_cast<const E*>(a.Q) + base;
    const E* Kp = static_cast<const E*>(a.K) + base;
    const E* Vp = static_cast<const E*>(a.V) + base;
    E* Op = static_cast<E*>(a.O) + base;
    const int qi = qb * kBQ + wave * 32 + n;

    if (D < 32) {  // rows of V^T past d stay zero for the whole kernel
        for (int x = tid; x < (S::VROWS - D) * S::VLD; x += kThreads)
            vt_lds[D * S::VLD + x] = static_cast<E>(0.f);
    }

    WaveState<E, D> st;
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
        st.qf[ks] = O::zero();
        if (qi < T)
            st.qf[ks] = *reinterpret_cast<const typename O::frag*>(
                Qp + size_t(qi) * D + ks * S::KSTEP + h * S::VPL);
    }
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) st.acc[db] = f32x16{};
    st.m_run = -1e30f;
    st.l_run = 0.f;
    const bool rowg = qi < T && ((a.rowbits[qi >> 5] >> (qi & 31)) & 1u);

    // In-place key tiles, run by run.
    for (int r = a.run_ptr[qb]; r < a.run_ptr[qb + 1]; ++r) {
        const int kb0 = a.runs[2 * r];
        const int w1 = a.runs[2 * r + 1];
        const int kb1 = w1 & 0x7fffffff;
        const bool masked = w1 < 0;
        for (int kb = kb0; kb < kb1; ++kb) {
            const int k0 = kb * kBK;
            __syncthreads();
            stage<E, D>(k_lds, vt_lds, Kp, Vp,
                        [&](int row) { return k0 + row < T ? k0 + row : -1; }, tid);
            __syncthreads();
            if (masked)
                st.template step<MASK_RULE>(k_lds, vt_lds, a, n, h, qi, rowg, k0, kBK);
            else
                st.template step<MASK_NONE>(k_lds, vt_lds, a, n, h, qi, rowg, k0, kBK);
        }
    }
    // Gathered strided/global keys.
    {
        const int a0 = a.gseg[4 * qb], a1 = a.gseg[4 * qb + 1];
        const int b0 = a.gseg[4 * qb + 2], b1 = a.gseg[4 * qb + 3];
        const int na = a1 - a0, total = na + (b1 - b0);
        for (int g = 0; g < total; g += kBK) {
            const int cnt = min(kBK, total - g);
            __syncthreads();
            stage<E, D>(k_lds, vt_lds, Kp, Vp,
                        [&](int row) {
                            const int sl = g + row;
                            if (row >= cnt) return -1;
                            return a.colkeys[sl < na ? a0 + sl : b0 + (sl - na)];
                        },
                        tid);
            __syncthreads();
            st.template step<MASK_SLOTS>(k_lds, vt_lds, a, n, h, qi, rowg, 0, cnt);
        }
    }

    // Epilogue: O = acc / l, both lane halves' sums combined.
    const float lt = st.l_run + __shfl_xor(st.l_run, 32);
    const float inv = 1.f / lt;
    if (a.lse && qi < T && h == 0)  // log-sum-exp: the scores are in log2 units
        a.lse[size_t(bh) * size_t(T) + size_t(qi)] = (st.m_run + __log2f(lt)) * 0.6931471805599453f;
    if (qi < T) {
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + g * 8 + h * 4;
                if (d0 < D) {
                    typename O::quad q;
#pragma unroll
                    for (int e = 0; e < 4; ++e) q[e] = static_cast<E>(st.acc[db][g * 4 + e] * inv);
                    *reinterpret_cast<typename O::quad*>(Op + size_t(qi) * D + d0) = q;
                }
            }
    }
}

template <typename E, int D>
int launch_t(const FwdArgs& a, int64_t grid, void* stream) {
    hipLaunchKernelGGL((sa_fwd_kernel<E, D>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace

int launch_fwd(int dtype, int d, const FwdArgs& a, int64_t grid, void* stream) {
    if (grid < 1) return SA_ERR_SHAPE;
    if (a.bq != kBQ) return SA_ERR_UNSUPPORTED;  // 128-row query blocks only
    if (dtype == SA_DTYPE_BF16) {
        switch (d) {
            case 16: return launch_t<__bf16, 16>(a, grid, stream);
            case 32: return launch_t<__bf16, 32>(a, grid, stream);
            case 64: return launch_t<__bf16, 64>(a, grid, stream);
            case 128: return launch_t<__bf16, 128>(a, grid, stream);
        }
    } else if (dtype == SA_DTYPE_F32) {
        switch (d) {
            case 16: return launch_t<float, 16>(a, grid, stream);
            case 32: return launch_t<float, 32>(a, grid, stream);
            case 64: return launch_t<float, 64>(a, grid, stream);
            case 128: return launch_t<float, 128>(a, grid, stream);
        }
    }
    return SA_ERR_UNSUPPORTED;
}

}  // namespace sa
