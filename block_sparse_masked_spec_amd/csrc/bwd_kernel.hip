// Backward pass of masked sparse attention for gfx950 (MI355X): dQ, dK, dV.
//
// The pages define the forward only ("Sparse attention", glossary.selfmadequant.com,
// section "Choose the available reads": a softmax renormalised over S_i); the
// backward is its gradient by the chain rule.  With p_ij the softmax weights
// (recomputed from the saved log-sum-exp), dp_ij = dO_i . v_j and
// D_i = dO_i . o_i:
//   ds_ij = p_ij (dp_ij - D_i),  dQ_i = sum_j ds_ij k_j / sqrt(d),
//   dK_j = sum_i ds_ij q_i / sqrt(d),  dV_j = sum_i p_ij dO_i.
// Only allowed pairs are visited, tile by tile, as in the forward.
//
// Two kernels, no atomics (sa_bwd_dq_kernel / sa_bwd_dkv_kernel for fp32 and
// small d; the _dma pair further down for bf16 d = 64, 128, same work):
//   * sa_bwd_dq_kernel: one workgroup per (head, 128-query block), walking
//     the forward plan (in-place key tiles, then gathered strided/global
//     keys).  Per 64-key tile: S^T = K Q^T and dP^T = V dO^T on MFMA (keys
//     are the MFMA rows, one query per lane column), the mask, P, dS, then
//     dQ^T += K^T dS^T.  It also writes D_i for the second kernel.
//   * sa_bwd_dkv_kernel: one workgroup per (head, 128-key block), walking
//     the 64-query tiles that meet the block.  The roles swap: S = Q K^T and
//     dP = dO V^T with queries as the MFMA rows and one key per lane column,
//     then dV^T += dO^T P and dK^T += Q^T dS.
// Rows go into the MFMA in the permuted order of the forward (bits 2 and 3
// swapped) so that the 8 values a lane holds for one k-step of the second
// product are 8 consecutive rows, read from the transposed tile at once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"
#include "kernel_common.hpp"
#include "mfma_tiles.hpp"

namespace sa {
namespace {

enum { BMASK_NONE = 0, BMASK_RULE = 1, BMASK_SLOTS = 2 };

constexpr float kLog2e = 1.4426950408889634f;

// Fragments of 32 rows of a [T][d] tensor for this lane (row `row`, the
// lane half's k-slices), zero past T.
template <typename E, int D>
__device__ __forceinline__ void load_frags(typename Ops<E>::frag* f, const E* base, int row, int T,
                                           int h) {
    using S = Shape<E, D>;
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
        f[ks] = Ops<E>::zero();
        if (row < T)
            f[ks] = *reinterpret_cast<const typename Ops<E>::frag*>(base + size_t(row) * D +
                                                                   ks * S::KSTEP + h * S::VPL);
    }
}

// Dot product of two fragment sets (this lane's half of a row), in fp32.
template <typename E, int D>
__device__ __forceinline__ float frag_dot(const typename Ops<E>::frag* x,
                                          const typename Ops<E>::frag* y) {
    using S = Shape<E, D>;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
        if constexpr (S::VPL == 1) {
            acc += static_cast<float>(x[ks]) * static_cast<float>(y[ks]);
        } else {
#pragma unroll
            for (int e = 0; e < S::VPL; ++e) acc += static_cast<float>(x[ks][e]) * static_cast<float>(y[ks][e]);
        }
    }
    return acc;
}

// Two 32-row products of one 64-row tile: out[blk] = rows(tile) . frag^T.
template <typename E, int D>
__device__ __forceinline__ void tile_product(f32x16* out, const E* rows_lds,
                                             const typename Ops<E>::frag* f, int n, int h) {
    using S = Shape<E, D>;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        out[blk] = f32x16{};
        const E* r = rows_lds + (blk * 32 + swap23(n)) * S::KLD + h * S::VPL;
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks)
            out[blk] = Ops<E>::mma(*reinterpret_cast<const typename Ops<E>::frag*>(r + ks * S::KSTEP),
                                   f[ks], out[blk]);
    }
}

// acc[db] += cols(tile)^T . x, with x the 64 tile rows held as two 32-row
// score blocks of this lane's column (rounded to E for the MFMA).
template <typename E, int D>
__device__ __forceinline__ void tile_accumulate(f32x16* acc, const E* cols_lds, const f32x16* x,
                                                int n, int h) {
    using S = Shape<E, D>;
    static_for<0, S::PKS>([&](auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
        constexpr int blk = (kk * S::VPL) >> 4;
        constexpr int rb = (kk * S::VPL) & 15;
        constexpr int off = blk * 32 + (rb >> 3) * 16 + (rb & 7);
        const typename Ops<E>::frag xf = Ops<E>::template pack<rb>(x[blk]);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db) {
            const E* c = cols_lds + (db * 32 + n) * S::VLD + off + h * 8;
            acc[db] = Ops<E>::mma(*reinterpret_cast<const typename Ops<E>::frag*>(c), xf, acc[db]);
        }
    });
}

// Tile row of score register r in block blk for lane half h.
__device__ __forceinline__ int reg_row(int blk, int r, int h) {
    return blk * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
}

// Store a d x 32 accumulator (row = d index, column = this lane's row) times
// `mul` into row `row` of a [T][d] tensor.
template <typename E, int D>
__device__ __forceinline__ void store_rows(E* dst, const f32x16* acc, int row, int h, float mul) {
    using S = Shape<E, D>;
#pragma unroll
    for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = db * 32 + g * 8 + h * 4;
            if (d0 < D) {
                typename Ops<E>::quad q;
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = static_cast<E>(acc[db][g * 4 + e] * mul);
                *reinterpret_cast<typename Ops<E>::quad*>(dst + size_t(row) * D + d0) = q;
            }
        }
}

// Row `row` of a [rows][D] fp32 block, same element mapping as store_rows
// (a partial result of a split work item, unscaled).
template <int D>
__device__ __forceinline__ void store_rows_f32(float* dst, const f32x16* acc, int row, int h) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float4 q;
            q.x = acc[db][g * 4];
            q.y = acc[db][g * 4 + 1];
            q.z = acc[db][g * 4 + 2];
            q.w = acc[db][g * 4 + 3];
            *reinterpret_cast<float4*>(dst + size_t(row) * D + db * 32 + g * 8 + h * 4) = q;
        }
}

// ---------------------------------------------------------------- dQ kernel
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void sa_bwd_dq_kernel(BwdArgs b) {
    using S = Shape<E, D>;
    using F = typename Ops<E>::frag;
    const FwdArgs& a = b.f;
    __shared__ __attribute__((aligned(16))) E k_lds[kBK * S::KLD];
    __shared__ __attribute__((aligned(16))) E v_lds[kBK * S::KLD];
    __shared__ __attribute__((aligned(16))) E kt_lds[S::VROWS * S::VLD];

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
    const E* Op = static_cast<const E*>(a.O) + base;
    const E* Gp = static_cast<const E*>(b.dO) + base;
    const int qi = qb * kBQ + wave * 32 + n;

    if (D < 32) {  // rows of the transposed tile past d stay zero
        for (int x = tid; x < (S::VROWS - D) * S::VLD; x += kThreads)
            kt_lds[D * S::VLD + x] = static_cast<E>(0.f);
    }

    F qf[S::NKS], gf[S::NKS];
    load_frags<E, D>(qf, Qp, qi, T, h);
    load_frags<E, D>(gf, Gp, qi, T, h);
    float Dq;
    {
        F of[S::NKS];
        load_frags<E, D>(of, Op, qi, T, h);
        const float part = frag_dot<E, D>(gf, of);
        Dq = part + __shfl_xor(part, 32);
    }
    if (qi < T && h == 0) b.Dw[size_t(bh) * size_t(T) + size_t(qi)] = Dq;
    const float lse2 = qi < T ? b.lse[size_t(bh) * size_t(T) + size_t(qi)] * kLog2e : 0.f;
    const bool rowg = qi < T && ((a.rowbits[qi >> 5] >> (qi & 31)) & 1u);
    const int qres = a.dil == 1 ? 0 : qi % a.dil;
    const int qblk = a.blk > 0 ? min(qi, T - 1) / a.blk : 0;

    f32x16 acc[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) acc[db] = f32x16{};

    auto tile = [&](int mode, int k0, int cnt) {
        f32x16 s[2], dp[2];
        tile_product<E, D>(s, k_lds, qf, n, h);
        tile_product<E, D>(dp, v_lds, gf, n, h);
        uint64_t aw = ~0ull;
        if (mode == BMASK_RULE)
            aw = allowed_word(a, qi, k0, rowg, a.colbits[k0 >> 6], qres,
                              a.dil == 1 ? 0 : k0 % a.dil, qblk);
        else if (mode == BMASK_SLOTS)
            aw = low_bits(cnt);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool ok = (aw >> reg_row(blk, r, h)) & 1;
                const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[blk][r], a.scale_log2, -lse2)) : 0.f;
                s[blk][r] = p * (dp[blk][r] - Dq);  // dS
            }
        tile_accumulate<E, D>(acc, kt_lds, s, n, h);
    };

    // In-place key tiles, run by run.
    for (int r = a.run_ptr[qb]; r < a.run_ptr[qb + 1]; ++r) {
        const int kb0 = a.runs[2 * r];
        const int w1 = a.runs[2 * r + 1];
        const int kb1 = w1 & 0x7fffffff;
        const bool masked = w1 < 0;
        for (int kb = kb0; kb < kb1; ++kb) {
            const int k0 = kb * kBK;
            auto key_of = [&](int row) { return k0 + row < T ? k0 + row : -1; };
            __syncthreads();
            stage_rows<E, D>(k_lds, Kp, key_of, tid);
            stage_rows<E, D>(v_lds, Vp, key_of, tid);
            stage_cols<E, D>(kt_lds, Kp, key_of, tid);
            __syncthreads();
            tile(masked ? BMASK_RULE : BMASK_NONE, k0, kBK);
        }
    }
    // Gathered strided/global keys.
    {
        const int a0 = a.gseg[4 * qb], a1 = a.gseg[4 * qb + 1];
        const int b0 = a.gseg[4 * qb + 2], b1 = a.gseg[4 * qb + 3];
        const int na = a1 - a0, total = na + (b1 - b0);
        for (int g = 0; g < total; g += kBK) {
            const int cnt = min(kBK, total - g);
            auto key_of = [&](int row) {
                const int sl = g + row;
                if (row >= cnt) return -1;
                return a.colkeys[sl < na ? a0 + sl : b0 + (sl - na)];
            };
            __syncthreads();
            stage_rows<E, D>(k_lds, Kp, key_of, tid);
            stage_rows<E, D>(v_lds, Vp, key_of, tid);
            stage_cols<E, D>(kt_lds, Kp, key_of, tid);
            __syncthreads();
            tile(BMASK_SLOTS, 0, cnt);
        }
    }
    if (qi < T) store_rows<E, D>(static_cast<E*>(b.dQ) + base, acc, qi, h, b.scale);
}

// -------------------------------------------------------------- dK/dV kernel
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void sa_bwd_dkv_kernel(BwdArgs b) {
    using S = Shape<E, D>;
    using F = typename Ops<E>::frag;
    const FwdArgs& a = b.f;
    static_assert(kBKB == kWaves * 32, "one 32-key MFMA column block per wave");
    static_assert(kBQB == kBK, "query tiles use the 64-row tile geometry");
    __shared__ __attribute__((aligned(16))) E q_lds[kBQB * S::KLD];
    __shared__ __attribute__((aligned(16))) E g_lds[kBQB * S::KLD];
    __shared__ __attribute__((aligned(16))) E qt_lds[S::VROWS * S::VLD];
    __shared__ __attribute__((aligned(16))) E gt_lds[S::VROWS * S::VLD];
    __shared__ __attribute__((aligned(16))) float lse_s[kBQB];
    __shared__ __attribute__((aligned(16))) float d_s[kBQB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int work = xcd_slice_index(blockIdx.x, gridDim.x);
    const int bh = work / b.n_kb;
    const int kb = b.kb_order[work % b.n_kb];
    const int T = a.T;
    const size_t base = size_t(bh) * size_t(T) * D;
    const E* Qp = static_cast<const E*>(a.Q) + base;
    const E* Kp = static_cast<const E*>(a.K) + base;
    const E* Vp = static_cast<const E*>(a.V) + base;
    const E* Gp = static_cast<const E*>(b.dO) + base;
    const float* Lp = b.lse + size_t(bh) * size_t(T);
    const float* Dp = b.Dw + size_t(bh) * size_t(T);
    const int kj = kb * kBKB + wave * 32 + n;  // this lane's key

    if (D < 32) {
        for (int x = tid; x < (S::VROWS - D) * S::VLD; x += kThreads) {
            qt_lds[D * S::VLD + x] = static_cast<E>(0.f);
            gt_lds[D * S::VLD + x] = static_cast<E>(0.f);
        }
    }

    F kf[S::NKS], vf[S::NKS];
    load_frags<E, D>(kf, Kp, kj, T, h);
    load_frags<E, D>(vf, Vp, kj, T, h);
    const bool colj = kj < T && ((a.colbits[kj >> 6] >> (kj & 63)) & 1);

    f32x16 dk[S::NDB], dv[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) dk[db] = dv[db] = f32x16{};

    for (int r = b.kb_ptr[kb]; r < b.kb_ptr[kb + 1]; ++r) {
        const int qt0 = b.kb_runs[2 * r];
        const int w1 = b.kb_runs[2 * r + 1];
        const int qt1 = w1 & 0x7fffffff;
        const bool masked = w1 < 0;
        for (int qt = qt0; qt < qt1; ++qt) {
            const int q0 = qt * kBQB;
            auto row_of = [&](int row) { return q0 + row < T ? q0 + row : -1; };
            __syncthreads();
            stage_rows<E, D>(q_lds, Qp, row_of, tid);
            stage_rows<E, D>(g_lds, Gp, row_of, tid);
            stage_cols<E, D>(qt_lds, Qp, row_of, tid);
            stage_cols<E, D>(gt_lds, Gp, row_of, tid);
            if (tid < kBQB) {
                const int i = q0 + tid;
                lse_s[tid] = i < T ? Lp[i] * kLog2e : 0.f;
                d_s[tid] = i < T ? Dp[i] : 0.f;
            }
            __syncthreads();

            f32x16 s[2], dp[2];
            tile_product<E, D>(s, q_lds, kf, n, h);
            tile_product<E, D>(dp, g_lds, vf, n, h);
            uint64_t aw = ~0ull;
            if (masked) {
                uint64_t roww = 0;
                const int w0 = q0 >> 5, nw = (T + 31) >> 5;
                if (w0 < nw) roww = a.rowbits[w0];
                if (w0 + 1 < nw) roww |= uint64_t(a.rowbits[w0 + 1]) << 32;
                aw = kj < T ? allowed_word_T(a, kj, q0, colj, roww) : 0ull;
            }
            f32x16 p[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r4 = 0; r4 < 16; r4 += 4) {
                    const int x0 = reg_row(blk, r4, h);  // 4 consecutive rows
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + x0);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(d_s + x0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = (aw >> (x0 + e)) & 1;
                        const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(s[blk][r4 + e], a.scale_log2, -l4[e])) : 0.f;
                        p[blk][r4 + e] = pv;
                        s[blk][r4 + e] = pv * (dp[blk][r4 + e] - d4[e]);  // dS
                    }
                }
            tile_accumulate<E, D>(dv, gt_lds, p, n, h);
            tile_accumulate<E, D>(dk, qt_lds, s, n, h);
        }
    }
    if (kj < T) {
        store_rows<E, D>(static_cast<E*>(b.dK) + base, dk, kj, h, b.scale);
        store_rows<E, D>(static_cast<E*>(b.dV) + base, dv, kj, h, 1.f);
    }
}

// ------------------------------------------- bf16: tiles by direct loads
// For bf16 (d = 64, 128) the two kernels below (sa_bwd_dq_dma_kernel,
// sa_bwd_dkv_dma_kernel) fill unpadded, XOR-swizzled row-major LDS tiles
// with buffer loads straight into LDS (16 bytes per lane, 1 KiB per instruction),
// double-buffered so that the next tile's loads run under the current
// tile's MFMAs.  The transposed operands (K^T, Q^T, dO^T) are read from the
// same row-major tiles with transposing LDS reads, so no transposed copy is
// staged.  Each 64-row tile is processed as two 32-row halves.

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lptr_t;
typedef __attribute__((address_space(3))) s16x4* lptr_s16x4_t;
__device__ __forceinline__ lptr_t as_lds(void* p) { return (lptr_t)p; }
__device__ __forceinline__ lptr_s16x4_t as_lds_s16x4(const void* p) { return (lptr_s16x4_t)(void*)p; }

// End of a tile: this wave's direct loads have landed and every wave is done
// with the current buffers; the scheduling barriers keep LDS reads on their
// side of the barrier.
__device__ __forceinline__ void dma_tile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// Tiles are 64 rows of D bf16 with no padding; the 16-byte chunk c of row r
// sits at chunk position c ^ swz(r) of that row.  The XOR pattern (a linear
// map of the row's low four bits) keeps both read patterns free of bank
// conflicts: the 16-byte row reads of the first product (8 or 16 lanes on
// distinct rows) and the 8-byte transposing reads (4 rows x 2 chunks per 16
// lanes).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128)
        return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 3 : 0);
    else
        return ((r & 1) ? 2 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 3 : 0);
}

// This wave's share of the loads of one 64-row tile of two [T][d] tensors,
// by buffer loads into LDS: LDS chunk position p of row r receives source
// chunk p ^ swz(r).  The rows of one wave's pieces are NW * RPI apart (a
// multiple of 16, so every piece of a lane has the same swizzled chunk), and
// a piece's byte offset from the tile's first row is the first piece's plus
// a scalar step.  Issuing a tile of consecutive rows then takes a lane's
// first row r0 and that offset (a few instructions from the lane id), with
// the tile's first row and the step as scalar offsets.  A tile past T clamps
// its rows to T - 1 per lane, and a tile of listed rows takes per-lane
// offsets.
template <int D, int NW>
struct DmaTile {
    static constexpr int CPR = D / 8;     // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;  // rows per instruction
    static constexpr int NJ = CPR / NW;   // instructions per wave and tensor
    static constexpr int ROWB = D * 2;    // bytes per row
    static constexpr int STEP = NW * RPI;
    static_assert(STEP % 16 == 0, "pieces of one lane share their swizzle");
    int wave, lane;

    __device__ __forceinline__ DmaTile(int wave_, int lane_) : wave(wave_), lane(lane_) {}
    __device__ __forceinline__ int first_row() const { return wave * RPI + lane / CPR; }
    __device__ __forceinline__ int first_off(int r0) const {
        return r0 * ROWB + ((lane % CPR) ^ swz<D>(r0)) * 16;
    }
    template <typename VOff, typename SOff>
    __device__ __forceinline__ void put(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, __bf16* da,
                                        __bf16* db, VOff vo, SOff so) const {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int lds = (wave + j * NW) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, as_lds(reinterpret_cast<char*>(da) + lds), 16, vo(j),
                                                     so(j), 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, as_lds(reinterpret_cast<char*>(db) + lds), 16, vo(j),
                                                     so(j), 0, 0);
        }
    }
    // Rows k0 .. k0 + 63, those past T clamped to row T - 1.
    __device__ __forceinline__ void rows_from(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, __bf16* da,
                                              __bf16* db, int k0, int T) const {
        const int r0 = first_row(), off0 = first_off(r0);
        if (k0 + 64 <= T) {
            put(ra, rb, da, db, [&](int) { return off0; }, [&](int j) { return (k0 + j * STEP) * ROWB; });
            asm volatile("; tile loads issued: in place" ::: "memory");
        } else {
            put(ra, rb, da, db,
                [&](int j) { return off0 + (min(k0 + r0 + j * STEP, T - 1) - r0) * ROWB; },
                [&](int) { return 0; });
            asm volatile("; tile loads issued: past T" ::: "memory");
        }
    }
    // Tile row r comes from source row row_of(r) (a valid row).
    template <typename RowOf>
    __device__ __forceinline__ void rows_listed(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                                __bf16* da, __bf16* db, RowOf row_of) const {
        const int r0 = first_row(), off0 = first_off(r0);
        int vo[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) vo[j] = off0 + (row_of(r0 + j * STEP) - r0) * ROWB;
        put(ra, rb, da, db, [&](int j) { return vo[j]; }, [&](int) { return 0; });
        asm volatile("; tile loads issued: listed rows" ::: "memory");
    }
};

// Buffer resource over the n bytes at p (raw addressing, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

// Product of rows blk*32 .. blk*32+31 of a swizzled 64-row tile with this
// lane's fragments: out = rows . frag^T (rows are MFMA rows in the permuted
// order, one column per lane).
template <int D, bool PRE = false>
__device__ __forceinline__ f32x16 half_product(const __bf16* tile, const bf16x8* f, int blk, int n,
                                               int h) {
    const int rr = swap23(n);
    const int x = h ^ swz<D>(rr);  // chunk 2 ks + h lands at 2 ks ^ x
    const __bf16* r = tile + (blk * 32 + rr) * D;
    f32x16 out = f32x16{};
    if constexpr (PRE) {
        bf16x8 a[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(r + ((2 * ks) ^ x) * 8);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], f[ks], out, 0, 0, 0);
    } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *reinterpret_cast<const bf16x8*>(r + ((2 * ks) ^ x) * 8), f[ks], out, 0, 0, 0);
    }
    return out;
}

// acc[db] += rows(blk half of the tile)^T . x, the transposed operand read
// from the swizzled row-major tile: for lane l of 16-lane group g
// (i = l % 16), read 4 columns starting at db*32 + (g%2)*16 + 4*(i%4) of
// tile row off + (l/32)*8 + i/4 (and 4 rows further); the hardware
// transposes within the group so that lane l holds 8 consecutive rows of
// column db*32 + l%32.  x holds the half's 32 rows of this lane's column.
template <int D, bool PRE = false>
__device__ __forceinline__ void half_accumulate_tr(f32x16* acc, const __bf16* tile, const f32x16& x,
                                                   int blk, int lane) {
    using S = Shape<__bf16, D>;
    const int h = lane >> 5, i = lane & 15, g = (lane >> 4) & 1;
    const int r_lo = h * 8 + (i >> 2);                   // row within a 16-row group
    const int cl = g * 2 + ((i & 3) >> 1);               // chunk within a 32-column block
    const int half = (i & 1) * 4;                        // element offset in the chunk
    const int y_lo = cl ^ swz<D>(r_lo), y_hi = cl ^ swz<D>(r_lo + 4);
    if constexpr (PRE) {
        bf16x8 af[2][S::NDB];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
                const int off = blk * 32 + q * 16;
                const __bf16* p0 = tile + (off + r_lo) * D + ((db * 4) ^ y_lo) * 8 + half;
                const __bf16* p1 = tile + (off + r_lo + 4) * D + ((db * 4) ^ y_hi) * 8 + half;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(p0));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(p1));
                af[q][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, 2>([&](auto rb_c) {
            constexpr int rb = decltype(rb_c)::value * 8;
            const bf16x8 xf = Ops<__bf16>::template pack<rb>(x);
#pragma unroll
            for (int db = 0; db < S::NDB; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb >> 3][db], xf, acc[db], 0, 0, 0);
        });
    } else {
        static_for<0, 2>([&](auto rb_c) {
            constexpr int rb = decltype(rb_c)::value * 8;
            const int off = blk * 32 + (rb >> 3) * 16;
            const bf16x8 xf = Ops<__bf16>::template pack<rb>(x);
    #pragma unroll
            for (int db = 0; db < S::NDB; ++db) {
                const __bf16* p0 = tile + (off + r_lo) * D + ((db * 4) ^ y_lo) * 8 + half;
                const __bf16* p1 = tile + (off + r_lo + 4) * D + ((db * 4) ^ y_hi) * 8 + half;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(p0));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(p1));
                const bf16x8 af =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf, acc[db], 0, 0, 0);
            }
        });
    }
}

// Tiles of one query block of the forward plan: runs of in-place key tiles,
// then gathered strided/global keys in chunks of 64.
struct BwdCursor {
    int run, run_end, kb, kb_end;
    bool masked;
    int gi, g_total;
    __device__ bool inplace() const { return run < run_end; }
    __device__ bool done() const { return !inplace() && gi >= g_total; }
};

__device__ __forceinline__ void bcur_enter(BwdCursor& c, const FwdArgs& a) {
    if (c.run < c.run_end) {
        c.kb = ldc(a.runs, 2 * c.run);
        const int w = ldc(a.runs, 2 * c.run + 1);
        c.kb_end = w & 0x7fffffff;
        c.masked = w < 0;
    }
}

__device__ __forceinline__ void bcur_advance(BwdCursor& c, const FwdArgs& a) {
    if (c.inplace()) {
        if (++c.kb >= c.kb_end) {
            ++c.run;
            bcur_enter(c, a);
        }
    } else {
        c.gi += kBK;
    }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void sa_bwd_dq_dma_kernel(BwdArgs b) {
    using E = __bf16;
    using S = Shape<E, D>;
    using F = typename Ops<E>::frag;
    const FwdArgs& a = b.f;
    constexpr int TILE = kBK * D;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int work = xcd_slice_index(blockIdx.x, gridDim.x);
    const int n_items = gridDim.x / a.BH;
    const int bh = work / n_items;
    // The work item (a query block or one key range of it) from its record.
    const int32_t* rec = a.item_rec + size_t(work % n_items) * kItemRec;
    const int qb = ldc(rec, REC_QB);
    const int T = a.T;
    const size_t base = size_t(bh) * size_t(T) * D;
    const E* Qp = static_cast<const E*>(a.Q) + base;
    const E* Kp = static_cast<const E*>(a.K) + base;
    const E* Vp = static_cast<const E*>(a.V) + base;
    const E* Op = static_cast<const E*>(a.O) + base;
    const E* Gp = static_cast<const E*>(b.dO) + base;
    const int qi = qb * (NW * 32) + wave * 32 + n;

    F qf[S::NKS], gf[S::NKS];
    load_frags<E, D>(qf, Qp, qi, T, h);
    load_frags<E, D>(gf, Gp, qi, T, h);
    float Dq;
    {
        F of[S::NKS];
        load_frags<E, D>(of, Op, qi, T, h);
        const float part = frag_dot<E, D>(gf, of);
        Dq = part + __shfl_xor(part, 32);
    }
    if (qi < T && h == 0) b.Dw[size_t(bh) * size_t(T) + size_t(qi)] = Dq;
    const float lse2 = qi < T ? b.lse[size_t(bh) * size_t(T) + size_t(qi)] * kLog2e : 0.f;
    // A 32-query group's global-row bits: one word, through the scalar cache.
    const bool rowg =
        qi < T && ((ldc(a.rowbits, min(qb * (NW * 32) + wave * 32, T - 1) >> 5) >> n) & 1u);
    const int qres = a.dil == 1 ? 0 : qi % a.dil;
    const int qblk = a.blk > 0 ? min(qi, T - 1) / a.blk : 0;

    f32x16 acc[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) acc[db] = f32x16{};

    const int ga0 = ldc(rec, REC_GA0), ga1 = ldc(rec, REC_GA1);
    const int gb0 = ldc(rec, REC_GB0), gb1 = ldc(rec, REC_GB1);
    const int gna = ga1 - ga0, gtot = gna + (gb1 - gb0);
    auto gkey = [&](int slot) { return a.colkeys[slot < gna ? ga0 + slot : gb0 + (slot - gna)]; };

    // Every row of the sequence lies in its T * D * 2 bytes (at most 1 GiB).
    const DmaTile<D, NW> dt(wave, lane);
    const __amdgpu_buffer_rsrc_t krs = raw_rsrc(Kp, T * D * 2), vrs = raw_rsrc(Vp, T * D * 2);
    auto issue = [&](const BwdCursor& c, E* kd, E* vd) {
        if (c.inplace()) {
            dt.rows_from(krs, vrs, kd, vd, c.kb * kBK, T);
        } else {
            const int g0 = c.gi;
            dt.rows_listed(krs, vrs, kd, vd, [&](int r) { return gkey(min(g0 + r, gtot - 1)); });
        }
    };
    auto compute = [&](const BwdCursor& c, const E* kt, const E* vt) {
        // The tile's allowed keys, and whether any is missing (wave-uniform:
        // full tiles skip the per-score test).
        uint64_t aw = ~0ull;
        bool msk;
        if (c.inplace()) {
            const int k0 = c.kb * kBK;
            msk = c.masked;
            if (c.masked)
                aw = allowed_word(a, qi, k0, rowg, ldc(a.colbits, k0 >> 6), qres,
                                  a.dil == 1 ? 0 : k0 % a.dil, qblk);
        } else {
            msk = gtot - c.gi < kBK;
            aw = low_bits(gtot - c.gi);
        }
        // Key reg_row(blk, r, h) of the tile is bit reg_row(blk, r, 0) of
        // awh: one shift per tile, constant bit positions per score.
        const uint64_t awh = aw >> (h * 8);
        // One 32-key half at a time: S^T, dP^T, dS^T, then dQ^T += K^T dS^T.
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x16 sv = half_product<D>(kt, qf, blk, n, h);
            const f32x16 dp = half_product<D>(vt, gf, blk, n, h);
            if (msk) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool ok = (awh >> reg_row(blk, r, 0)) & 1;
                    const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sv[r], a.scale_log2, -lse2)) : 0.f;
                    sv[r] = p * (dp[r] - Dq);  // dS
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sv[r], a.scale_log2, -lse2));
                    sv[r] = p * (dp[r] - Dq);  // dS
                }
            }
            half_accumulate_tr<D>(acc, kt, sv, blk, lane);
        }
    };

    // Tile t computes from slot t % 2 while tile t + 1 loads into the other.
    const int first_end = ldc(rec, REC_FIRST_END);
    BwdCursor cur{ldc(rec, REC_RUN_BEGIN), ldc(rec, REC_RUN_END), ldc(rec, REC_FIRST_KB),
                  first_end & 0x7fffffff, first_end < 0, 0, gtot};
    if constexpr (D == 64) {
        // Two slots as distinct objects, indexed statically (the loop is
        // unrolled by two), so the compiler can tell the prefetch into one
        // from the reads of the other and keeps the prefetch in flight.
        __shared__ __attribute__((aligned(1024))) E kbuf0[TILE];
        __shared__ __attribute__((aligned(1024))) E vbuf0[TILE];
        __shared__ __attribute__((aligned(1024))) E kbuf1[TILE];
        __shared__ __attribute__((aligned(1024))) E vbuf1[TILE];
        if (!cur.done()) issue(cur, kbuf0, vbuf0);
        dma_tile_barrier();
        while (!cur.done()) {
            BwdCursor nxt = cur;
            bcur_advance(nxt, a);
            if (!nxt.done()) issue(nxt, kbuf1, vbuf1);
            compute(cur, kbuf0, vbuf0);
            dma_tile_barrier();
            if (nxt.done()) break;
            cur = nxt;
            bcur_advance(nxt, a);
            if (!nxt.done()) issue(nxt, kbuf0, vbuf0);
            compute(cur, kbuf1, vbuf1);
            dma_tile_barrier();
            cur = nxt;
        }
    } else {
        // d = 128: the slot is chosen at run time, so a tile's reads of its
        // slot also wait for the loads into the other one, which the second
        // wave of the SIMD covers.  Two static slots and an unrolled loop fit
        // in 247 registers at two waves per SIMD but measured no faster.
        __shared__ __attribute__((aligned(1024))) E kbuf[2 * TILE];
        __shared__ __attribute__((aligned(1024))) E vbuf[2 * TILE];
        int slot = 0;
        if (!cur.done()) issue(cur, kbuf, vbuf);
        dma_tile_barrier();
        while (!cur.done()) {
            BwdCursor nxt = cur;
            bcur_advance(nxt, a);
            if (!nxt.done()) issue(nxt, kbuf + (slot ^ 1) * TILE, vbuf + (slot ^ 1) * TILE);
            compute(cur, kbuf + slot * TILE, vbuf + slot * TILE);
            dma_tile_barrier();
            cur = nxt;
            slot ^= 1;
        }
    }
    const int part = ldc(rec, REC_PART);
    if (part >= 0)  // one key range of a split block: unscaled partial
        store_rows_f32<D>(b.dq_part + (size_t(bh) * a.n_parts + part) * (NW * 32) * D, acc,
                          qi - qb * (NW * 32), h);
    else if (qi < T)
        store_rows<E, D>(static_cast<E*>(b.dQ) + base, acc, qi, h, b.scale);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, D == 64 ? 2 : 1) void sa_bwd_dkv_dma_kernel(BwdArgs b) {
    using E = __bf16;
    using S = Shape<E, D>;
    using F = typename Ops<E>::frag;
    const FwdArgs& a = b.f;
    // Two slots as distinct objects, indexed statically (see the dQ kernel).
    constexpr int TILE = kBQB * D;
    __shared__ __attribute__((aligned(1024))) E qbuf0[TILE];
    __shared__ __attribute__((aligned(1024))) E gbuf0[TILE];
    __shared__ __attribute__((aligned(1024))) E qbuf1[TILE];
    __shared__ __attribute__((aligned(1024))) E gbuf1[TILE];
    __shared__ __attribute__((aligned(256))) float lbuf0[kBQB], dbuf0[kBQB], lbuf1[kBQB], dbuf1[kBQB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int work = xcd_slice_index(blockIdx.x, gridDim.x);
    const int n_items = gridDim.x / a.BH;
    const int bh = work / n_items;
    const int it = ldc(b.kb_order, work % n_items);  // a key block or one query range of it
    const int kb = ldc(b.kv_item_kb, it);
    // Gathered block kb - n_kb: keys f.colkeys[slot]; a band block skips its
    // column keys when they are gathered.
    const bool gath = kb >= b.n_kb;
    const int T = a.T;
    const size_t base = size_t(bh) * size_t(T) * D;
    const E* Qp = static_cast<const E*>(a.Q) + base;
    const E* Kp = static_cast<const E*>(a.K) + base;
    const E* Vp = static_cast<const E*>(a.V) + base;
    const E* Gp = static_cast<const E*>(b.dO) + base;
    const float* Lp = b.lse + size_t(bh) * size_t(T);
    const float* Dp = b.Dw + size_t(bh) * size_t(T);
    const int gslot = (kb - b.n_kb) * (NW * 32) + wave * 32 + n;
    const int kj = gath ? a.colkeys[min(gslot, b.kv_n_col - 1)] : kb * (NW * 32) + wave * 32 + n;

    F kf[S::NKS], vf[S::NKS];
    load_frags<E, D>(kf, Kp, kj, T, h);
    load_frags<E, D>(vf, Vp, kj, T, h);
    const bool colj = kj < T && ((a.colbits[kj >> 6] >> (kj & 63)) & 1);
    // This lane's key takes part: gathered keys inside the list; band keys
    // below T, column keys only when they are not gathered.
    const bool mine = gath ? gslot < b.kv_n_col : (kj < T && !(colj && b.kv_n_gkb > 0));

    f32x16 dk[S::NDB], dv[S::NDB];
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) dk[db] = dv[db] = f32x16{};

    // Query tiles of this item: run r, tile qt.
    int r = ldc(b.kb_ptr, it);
    const int r_end = ldc(b.kb_ptr, it + 1);
    int qt = 0, qt_end = 0;
    bool masked = false;
    auto enter = [&]() {
        if (r < r_end) {
            qt = ldc(b.kb_runs, 2 * r);
            const int w = ldc(b.kb_runs, 2 * r + 1);
            qt_end = w & 0x7fffffff;
            masked = w < 0;
        }
    };
    enter();
    // Query tiles and their LSE and D values by buffer loads.  (The
    // flat-encoded global->LDS loads count against both wait counters, and
    // the compiler turns every LDS wait behind one into a full drain.)
    const DmaTile<D, NW> dt(wave, lane);
    const __amdgpu_buffer_rsrc_t qrs = raw_rsrc(Qp, T * D * 2), grs = raw_rsrc(Gp, T * D * 2);
    const __amdgpu_buffer_rsrc_t lrs = raw_rsrc(Lp, T * 4), drs = raw_rsrc(Dp, T * 4);
    auto issue = [&](int q0, E* qd, E* gd, float* lsd, float* dsd) {
        dt.rows_from(qrs, grs, qd, gd, q0, T);
        if (wave == 0) {
            const int i = min(q0 + lane, T - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, as_lds(lsd), 4, i * 4, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, as_lds(dsd), 4, i * 4, 0, 0, 0);
        }
    };
    auto compute = [&](int q0, bool msk, const E* qt_l, const E* gt_l, const float* ls, const float* dsv) {
        uint64_t aw = ~0ull;
        if (msk) {
            uint64_t roww = 0;
            const int w0 = q0 >> 5, nw = (T + 31) >> 5;
            if (w0 < nw) roww = ldc(a.rowbits, w0);
            if (w0 + 1 < nw) roww |= uint64_t(ldc(a.rowbits, w0 + 1)) << 32;
            aw = mine ? allowed_word_T(a, kj, q0, colj, roww) : 0ull;
        }
        // S and dP for both 32-query halves, then per half P and dS,
        // dV^T += dO^T P and dK^T += Q^T dS.
        f32x16 svs[2], dps[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            svs[blk] = half_product<D, D == 128>(qt_l, kf, blk, n, h);
            dps[blk] = half_product<D, D == 128>(gt_l, vf, blk, n, h);
        }
        // Query reg_row(blk, r, h) of the tile is bit reg_row(blk, r, 0) of
        // awh: one shift per tile, constant bit positions per score.
        const uint64_t awh = aw >> (h * 8);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x16& sv = svs[blk];
            f32x16& dp = dps[blk];
            if (msk) {
#pragma unroll
                for (int r4 = 0; r4 < 16; r4 += 4) {
                    const int x0 = reg_row(blk, r4, h);
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + x0);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dsv + x0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = (awh >> (reg_row(blk, r4, 0) + e)) & 1;
                        const float pv =
                            ok ? __builtin_amdgcn_exp2f(fmaf(sv[r4 + e], a.scale_log2, -l4[e] * kLog2e)) : 0.f;
                        sv[r4 + e] = pv;
                        dp[r4 + e] = pv * (dp[r4 + e] - d4[e]);  // dS
                    }
                }
            } else {  // wave-uniform: a full tile skips the per-score test
#pragma unroll
                for (int r4 = 0; r4 < 16; r4 += 4) {
                    const int x0 = reg_row(blk, r4, h);
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + x0);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dsv + x0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pv = __builtin_amdgcn_exp2f(fmaf(sv[r4 + e], a.scale_log2, -l4[e] * kLog2e));
                        sv[r4 + e] = pv;
                        dp[r4 + e] = pv * (dp[r4 + e] - d4[e]);  // dS
                    }
                }
            }
            half_accumulate_tr<D, D == 128>(dv, gt_l, sv, blk, lane);
            half_accumulate_tr<D, D == 128>(dk, qt_l, dp, blk, lane);
        }
        // At d = 128 (one wave per SIMD) the MFMAs of the second half's
        // products and of both halves' accumulations are interleaved with
        // the softmax arithmetic, so the matrix pipe and the vector ALU of
        // the one wave run together.
        if constexpr (D == 128) {
#pragma unroll
            for (int i = 0; i < 48; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
            }
        }
    };

    // The (run, tile) sequence: tile t computes from slot t % 2 while tile
    // t + 1 loads into the other.
    bool have = r < r_end;
    int cq = qt;
    bool cm = masked;
    auto step_next = [&]() {  // advance to the next tile; false when none
        if (++qt >= qt_end) {
            ++r;
            if (r >= r_end) return false;
            enter();
        }
        return true;
    };
    if (have) issue(cq * kBQB, qbuf0, gbuf0, lbuf0, dbuf0);
    dma_tile_barrier();
    if constexpr (D == 64) {
        // Two waves per SIMD leave no registers for a second copy of the
        // loop body: the slot is chosen at run time (each tile's reads then
        // wait for the next tile's loads, which the other wave covers).
        int slot = 0;
        while (have) {
            const bool nh = step_next();
            const int nq = qt;
            const bool nm = masked;
            if (nh) {
                if (slot)
                    issue(nq * kBQB, qbuf0, gbuf0, lbuf0, dbuf0);
                else
                    issue(nq * kBQB, qbuf1, gbuf1, lbuf1, dbuf1);
            }
            compute(cq * kBQB, cm, slot ? qbuf1 : qbuf0, slot ? gbuf1 : gbuf0, slot ? lbuf1 : lbuf0,
                    slot ? dbuf1 : dbuf0);
            dma_tile_barrier();
            have = nh;
            cq = nq;
            cm = nm;
            slot ^= 1;
        }
    }
    while (D != 64 && have) {
        bool nh = step_next();
        int nq = qt;
        bool nm = masked;
        if (nh) issue(nq * kBQB, qbuf1, gbuf1, lbuf1, dbuf1);
        compute(cq * kBQB, cm, qbuf0, gbuf0, lbuf0, dbuf0);
        dma_tile_barrier();
        if (!nh) break;
        cq = nq;
        cm = nm;
        nh = step_next();
        nq = qt;
        nm = masked;
        if (nh) issue(nq * kBQB, qbuf0, gbuf0, lbuf0, dbuf0);
        compute(cq * kBQB, cm, qbuf1, gbuf1, lbuf1, dbuf1);
        dma_tile_barrier();
        have = nh;
        cq = nq;
        cm = nm;
    }
    const int part = b.kv_item_part ? ldc(b.kv_item_part, it) : -1;
    if (part >= 0) {  // one query range of a split key block: unscaled partials
        const size_t slot = (size_t(bh) * b.kv_n_parts + part) * (NW * 32) * D;
        const size_t half = size_t(a.BH) * b.kv_n_parts * (NW * 32) * D;
        // row of this lane's key in the block (band or gathered)
        store_rows_f32<D>(b.kv_part + slot, dk, wave * 32 + n, h);
        store_rows_f32<D>(b.kv_part + half + slot, dv, wave * 32 + n, h);
    } else if (mine) {
        store_rows<E, D>(static_cast<E*>(b.dK) + base, dk, kj, h, b.scale);
        store_rows<E, D>(static_cast<E*>(b.dV) + base, dv, kj, h, 1.f);
    }
}

// Sum the partials of the split blocks into the bf16 output: rows of block
// split_blk[s] get mul * the sum over slots [split_ptr[s], split_ptr[s+1])
// of part[bh][slot][row][:].  Row r of block blk is output row blk * rows
// + r (skipped if colbits marks it a column key), or, for a gathered block
// blk >= n_band, output row colkeys[(blk - n_band) * rows + r] while that
// is below n_col.  One thread per (row, 4 columns).
template <int D>
__global__ __launch_bounds__(256) void sa_bwd_sum_parts_kernel(const float* part, int n_parts, int rows,
                                                                const int32_t* split_blk,
                                                                const int32_t* split_ptr, int n_split,
                                                                __bf16* dst, int T, float mul,
                                                                const uint64_t* colbits,
                                                                const int32_t* colkeys, int n_col,
                                                                int n_band) {
    constexpr int C = D / 4, RPW = 256 / C;
    const int per_blk = rows / RPW;
    const int x = blockIdx.x % per_blk, y = blockIdx.x / per_blk;
    const int bh = y / n_split, sidx = y % n_split;
    const int r = x * RPW + threadIdx.x / C, c = threadIdx.x % C;
    const int blk = split_blk[sidx];
    int row;
    if (blk >= n_band) {
        const int slot = (blk - n_band) * rows + r;
        if (slot >= n_col) return;
        row = colkeys[slot];
    } else {
        row = blk * rows + r;
        if (row >= T || (colbits && ((colbits[row >> 6] >> (row & 63)) & 1))) return;
    }
    float4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int p = split_ptr[sidx]; p < split_ptr[sidx + 1]; ++p) {
        const float4 v =
            *reinterpret_cast<const float4*>(part + ((size_t(bh) * n_parts + p) * rows + r) * D + c * 4);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    typename Ops<__bf16>::quad q;
    q[0] = static_cast<__bf16>(sum.x * mul);
    q[1] = static_cast<__bf16>(sum.y * mul);
    q[2] = static_cast<__bf16>(sum.z * mul);
    q[3] = static_cast<__bf16>(sum.w * mul);
    *reinterpret_cast<typename Ops<__bf16>::quad*>(dst + (size_t(bh) * T + row) * D + c * 4) = q;
}

template <typename E, int D>
int launch_b(const BwdArgs& b, void* stream) {
    const unsigned g1 = static_cast<unsigned>(int64_t(b.f.BH) * ((b.f.T + kBQ - 1) / kBQ));
    hipLaunchKernelGGL((sa_bwd_dq_kernel<E, D>), dim3(g1), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), b);
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    const unsigned g2 = static_cast<unsigned>(int64_t(b.f.BH) * b.n_kb);
    hipLaunchKernelGGL((sa_bwd_dkv_kernel<E, D>), dim3(g2), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), b);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// NW waves per workgroup: 4 (128-query and 128-key blocks) or 2 (the 64-row
// plans of block mode).
template <int D, int NW>
int launch_b_dma(const BwdArgs& b, void* stream) {
    constexpr int ROWS = NW * 32;  // query rows of a dQ block, keys of a dK/dV block
    const auto st = static_cast<hipStream_t>(stream);
    auto sum_parts = [&](const float* part, int n_parts, const int32_t* blk, const int32_t* ptr, int n_split,
                         void* dst, float mul, bool kv) {
        const int64_t g = int64_t(b.f.BH) * n_split * (ROWS / (256 / (D / 4)));
        if (g > INT32_MAX) return SA_ERR_SHAPE;
        const bool gathered = kv && b.kv_n_gkb > 0;
        hipLaunchKernelGGL((sa_bwd_sum_parts_kernel<D>), dim3(static_cast<unsigned>(g)), dim3(256), 0, st, part,
                           n_parts, ROWS, blk, ptr, n_split, static_cast<__bf16*>(dst), b.f.T, mul,
                           gathered ? b.f.colbits : nullptr, b.f.colkeys, b.kv_n_col,
                           gathered ? b.n_kb : INT32_MAX);
        return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
    };
    const unsigned g1 = static_cast<unsigned>(int64_t(b.f.BH) * b.n_q_items);
    hipLaunchKernelGGL((sa_bwd_dq_dma_kernel<D, NW>), dim3(g1), dim3(NW * 64), 0, st, b);
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    if (b.f.n_parts > 0) {
        const int rc =
            sum_parts(b.dq_part, b.f.n_parts, b.dq_split_qb, b.dq_split_ptr, b.dq_n_split, b.dQ, b.scale, false);
        if (rc != SA_OK) return rc;
    }
    const unsigned g2 = static_cast<unsigned>(int64_t(b.f.BH) * b.n_kv_items);
    hipLaunchKernelGGL((sa_bwd_dkv_dma_kernel<D, NW>), dim3(g2), dim3(NW * 64), 0, st, b);
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    if (b.kv_n_parts > 0) {
        const size_t half = size_t(b.f.BH) * b.kv_n_parts * ROWS * D;
        int rc = sum_parts(b.kv_part, b.kv_n_parts, b.kv_split_kb, b.kv_split_ptr, b.kv_n_split, b.dK, b.scale,
                           true);
        if (rc == SA_OK)
            rc = sum_parts(b.kv_part + half, b.kv_n_parts, b.kv_split_kb, b.kv_split_ptr, b.kv_n_split, b.dV, 1.f,
                           true);
        if (rc != SA_OK) return rc;
    }
    return SA_OK;
}

}  // namespace

int launch_bwd(int dtype, int d, const BwdArgs& b, void* stream) {
    if (b.f.bq != kBQ && !(b.f.bq == 64 && dtype == SA_DTYPE_BF16 && d == 64)) return SA_ERR_UNSUPPORTED;
    if (dtype == SA_DTYPE_BF16) {
        switch (d) {
            case 16: return launch_b<__bf16, 16>(b, stream);
            case 32: return launch_b<__bf16, 32>(b, stream);
            case 64: return b.f.bq == 64 ? launch_b_dma<64, 2>(b, stream) : launch_b_dma<64, 4>(b, stream);
            case 128: return launch_b_dma<128, 4>(b, stream);
        }
    } else if (dtype == SA_DTYPE_F32) {
        switch (d) {
            case 16: return launch_b<float, 16>(b, stream);
            case 32: return launch_b<float, 32>(b, stream);
            case 64: return launch_b<float, 64>(b, stream);
            case 128: return launch_b<float, 128>(b, stream);
        }
    }
    return SA_ERR_UNSUPPORTED;
}

}  // namespace sa
