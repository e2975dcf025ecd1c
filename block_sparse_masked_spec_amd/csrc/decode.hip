// Windowed decode for gfx950 (MI355X): a few new query tokens per sequence
// against a ring-buffer KV cache that holds only the last C positions.
//
// A sliding-window layer needs only its last w keys and values at inference
// time ("Sparse and sliding-window attention", getnybble.com, section
// "Sliding window attention"; "Attention variants", sreshtalluri.github.io,
// section 1 and section 3 "Worked example: KV cache for a long context").
// Each new query i reads the allowed keys j of the mask rule among the live
// cache positions; the result is the same softmax-renormalised sum as the
// forward ("Sparse attention", glossary.selfmadequant.com, "Choose the
// available reads").
//
// The work is HBM-bound: every live K and V row is read once per step while
// the arithmetic per row is a handful of dot products.  So:
//   * one workgroup per (sequence, KV head, query chunk, key split) handles
//     every query head that shares that KV head (grouped-query attention),
//     so each K/V byte crosses HBM once;
//   * d/8 lanes read one key row (16 bytes each, one coalesced row per lane
//     group); the partial dot products are summed across the group with DPP
//     moves (no LDS), leaving the score in every lane of the group;
//   * each lane group keeps a running max, sum and its d/8-slice of the
//     accumulator per query (online softmax in base 2);
//   * groups, then waves, then key splits are merged with the usual
//     (max, sum, acc) rescaling; splits go through a small fp32 workspace and
//     a second kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.hpp"

namespace sa {

// Scratch of the allocation-free decode entry point: the key-split partials
// live in this file-scope device array instead of the library workspace.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code the name `scratch` is only a stand-in for the symbol, never a
// device address: the address (different on each GPU) comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_addr[kMaxDevices] = {};  // per device, filled on first use

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kUnroll = 2;  // keys per lane group per chunk (two chunks in flight)

// Sum over aligned groups of LPR lanes (LPR in {2, 4, 8, 16}); every lane of
// the group receives the total.  Quad permutes swap neighbours (xor 1, xor
// 2); the half-row and row mirrors then pair the quads and the halves.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    if (LPR >= 4)
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    if (LPR >= 8)
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    if (LPR >= 16)
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Merge state (m2, l2, a2) into (m, l, a): both are partial softmax sums in
// base 2 over disjoint key sets.
__device__ __forceinline__ void merge_into(float& m, float& l, float* a, float m2, float l2,
                                           const float* a2, int n) {
    const float mn = fmaxf(m, m2);
    const float s1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float s2 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
    l = l * s1 + l2 * s2;
    for (int e = 0; e < n; ++e) a[e] = a[e] * s1 + a2[e] * s2;
    m = mn;
}

template <int D, int NQ>
__global__ __launch_bounds__(kDecThreads) void sa_decode_kernel(DecodeArgs a) {
    constexpr int EPL = D >= 128 ? 16 : 8;  // elements of a key row per lane
    constexpr int NW = EPL / 2;             // packed bf16 pairs per lane
    constexpr int LPR = D / EPL;            // lanes per key row
    constexpr int GPW = 64 / LPR;           // key rows per wave step
    constexpr int STEP = GPW * kDecWaves;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / LPR, sub = lane % LPR;
    // Grid (KV head x query chunk, sequence, key split): the workgroups
    // dispatched together hold the same key range of many sequences, which
    // streams about 2% faster than the splits of one sequence side by side.
    const int split = blockIdx.z;
    const int kvh = blockIdx.x % a.Hkv, qchunk = blockIdx.x / a.Hkv;
    const int b = blockIdx.y;
    const int nq_all = a.G * a.n_new;
    const int q0 = qchunk * NQ;
    const int nq = min(NQ, nq_all - q0);

    // Positions: the new tokens are pos-n_new+1 .. pos; the cache holds
    // max(0, pos-C+1) .. pos.
    const int pos = a.pos[b];
    const int i_first = pos - a.n_new + 1;
    long lo = long(pos) - a.C + 1;
    if (lo < 0) lo = 0;
    if (a.reach != INT32_MAX && long(i_first) - a.reach > lo) lo = long(i_first) - a.reach;
    // Keys visited: lo, lo + ks, ... <= pos.  With one new token and a
    // dilation g, only keys on its grid (j = pos mod g) are visited.
    const int ks = (a.n_new == 1 && a.dil > 1) ? a.dil : 1;
    if (ks > 1) lo += ((long(pos) - lo) % ks);  // first key on the grid
    const long nkeys = pos >= lo ? (long(pos) - lo) / ks + 1 : 0;
    const long chunk = (nkeys + a.nsplit - 1) / a.nsplit;
    const long kbeg = min(nkeys, long(split) * chunk), kend = min(nkeys, kbeg + chunk);
    // With one new token every visited key is allowed (the range and the
    // grid come from the rule); several new tokens need the rule per key.
    const bool rule = a.n_new > 1;

    const size_t kvbase = (size_t(b) * a.Hkv + kvh) * size_t(a.C) * D;
    const __bf16* Kc = static_cast<const __bf16*>(a.K) + kvbase + sub * EPL;
    const __bf16* Vc = static_cast<const __bf16*>(a.V) + kvbase + sub * EPL;
    const int slot0 = int(lo % a.C);

    // Queries of this chunk: query q = gh * n_new + t reads with head
    // kvh * G + gh at position i_first + t.  Packed bf16 pairs of this lane's
    // d-slice.
    uint32_t qw[NQ][NW];
    int qpos[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int qq = q0 + min(q, nq - 1);
        const int gh = qq / a.n_new, t = qq % a.n_new;
        const int h = kvh * a.G + gh;
        const uint4* src = reinterpret_cast<const uint4*>(
            static_cast<const __bf16*>(a.Q) + ((size_t(b) * a.H + h) * a.n_new + t) * D + sub * EPL);
#pragma unroll
        for (int c = 0; c < NW / 4; ++c) {
            const uint4 w = src[c];
            qw[q][4 * c] = w.x;
            qw[q][4 * c + 1] = w.y;
            qw[q][4 * c + 2] = w.z;
            qw[q][4 * c + 3] = w.w;
        }
        qpos[q] = q < nq ? i_first + t : -1;  // -1: padding query, never allowed
    }

    float m[NQ], l[NQ], acc[NQ][EPL];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        m[q] = -INFINITY;
        l[q] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[q][e] = 0.f;
    }

    // Chunks of kUnroll keys per lane group.  Software-pipelined: the loads
    // of the next chunk are issued before the current one is scored, so each
    // wave keeps memory requests in flight while it computes.
    struct Chunk {
        uint32_t kr[kUnroll][NW], vr[kUnroll][NW];
        int jj[kUnroll];
    };
    auto load = [&](Chunk& c, long k) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const long kk = min(k + long(u) * STEP, kend - 1);  // clamp: a valid row, dropped below
            c.jj[u] = k + long(u) * STEP < kend ? int(lo + kk * ks) : -1;
            // kk * ks <= pos - lo < C, so one wrap at most
            int slot = slot0 + int(kk * ks);
            if (slot >= a.C) slot -= a.C;
            const uint4* kp = reinterpret_cast<const uint4*>(Kc + size_t(slot) * D);
            const uint4* vp = reinterpret_cast<const uint4*>(Vc + size_t(slot) * D);
#pragma unroll
            for (int x = 0; x < NW / 4; ++x) {
                const uint4 kx = kp[x], vx = vp[x];
                c.kr[u][4 * x] = kx.x; c.kr[u][4 * x + 1] = kx.y; c.kr[u][4 * x + 2] = kx.z; c.kr[u][4 * x + 3] = kx.w;
                c.vr[u][4 * x] = vx.x; c.vr[u][4 * x + 1] = vx.y; c.vr[u][4 * x + 2] = vx.z; c.vr[u][4 * x + 3] = vx.w;
            }
        }
    };
    auto compute = [&](const Chunk& c) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float s[kUnroll];
            float cmax = -INFINITY;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float x = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) x = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(qw[q][w]), as_bf2(c.kr[u][w]), x, false);
                x = group_sum<LPR>(x) * a.scale_log2;
                const int j = c.jj[u];
                bool ok = j >= 0;
                if (rule) {  // causal, inside the band, on the dilation grid
                    const int gap = qpos[q] - j;
                    ok = ok && qpos[q] >= 0 && gap >= 0 && gap <= a.reach && (a.dil == 1 || gap % a.dil == 0);
                }
                s[u] = ok ? x : -INFINITY;
                cmax = fmaxf(cmax, s[u]);
            }
            if (cmax > m[q]) {  // the running max grows: rescale (rare once warm)
                const float sc = __builtin_amdgcn_exp2f(m[q] - cmax);  // 0 while m is -inf
                l[q] *= sc;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[q][e] *= sc;
                m[q] = cmax;
            }
            // Weights are rounded to bf16 and both the sum and the values use
            // the rounded ones.  acc[2w] += p * v_lo and acc[2w+1] += p * v_hi
            // are dot products of (p, 0) and (0, p) with the packed pair.
            if (m[q] == -INFINITY) continue;  // no allowed key yet
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const __bf16 pb = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[u] - m[q]));
                l[q] += static_cast<float>(pb);
                const uint32_t pw = __builtin_bit_cast(uint16_t, pb);
                const bf16x2 plo = as_bf2(pw), phi = as_bf2(pw << 16);
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    acc[q][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(plo, as_bf2(c.vr[u][w]), acc[q][2 * w], false);
                    acc[q][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(phi, as_bf2(c.vr[u][w]), acc[q][2 * w + 1], false);
                }
            }
        }
    };
    const long stride = long(STEP) * kUnroll;
    long k = kbeg + wave * GPW + grp;
    if (k < kend) {
        Chunk c0, c1;
        load(c0, k);
        for (;;) {
            const long k1 = k + stride;
            if (k1 < kend) load(c1, k1);
            compute(c0);
            if (k1 >= kend) break;
            const long k2 = k1 + stride;
            if (k2 < kend) load(c0, k2);
            compute(c1);
            if (k2 >= kend) break;
            k = k2;
        }
    }

    // Merge the lane groups of the wave: partners differ in the lane bits
    // above the group's own.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float m2 = __shfl_xor(m[q], off);
            const float l2 = __shfl_xor(l[q], off);
            float a2[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(acc[q][e], off);
            merge_into(m[q], l[q], acc[q], m2, l2, a2, EPL);
        }
    }

    // Merge the waves through LDS: wave w's group 0 publishes its state.
    __shared__ float sm[kDecWaves][NQ], sl[kDecWaves][NQ];
    __shared__ float sa[kDecWaves][NQ][D];
    if (grp == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sa[wave][q][sub * EPL + e] = acc[q][e];
            if (sub == 0) {
                sm[wave][q] = m[q];
                sl[wave][q] = l[q];
            }
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < NQ * D; x += kDecThreads) {
        const int q = x / D, e = x % D;
        if (q >= nq) continue;
        float M = -INFINITY;
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm[w][q]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int w = 0; w < kDecWaves; ++w) {
                const float s = exp2f(sm[w][q] - M);
                L += sl[w][q] * s;
                A += sa[w][q][e] * s;
            }
        }
        const int qq = q0 + q, gh = qq / a.n_new, t = qq % a.n_new;
        const size_t row = (size_t(b) * a.H + kvh * a.G + gh) * a.n_new + t;
        if (a.nsplit == 1) {
            static_cast<__bf16*>(a.O)[row * D + e] = static_cast<__bf16>(L > 0.f ? A / L : 0.f);
        } else {
            float* p = a.part + (row * a.nsplit + split) * (D + 2);
            p[2 + e] = A;
            if (e == 0) {
                p[0] = M;
                p[1] = L;
            }
        }
    }
}

// Combine the key splits of one query row: O = sum_s A_s 2^(M_s - M) /
// sum_s L_s 2^(M_s - M).
template <int D>
__global__ __launch_bounds__(128) void sa_decode_merge_kernel(DecodeArgs a) {
    const size_t row = blockIdx.x;
    const float* p = a.part + row * a.nsplit * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, p[s * (D + 2)]);
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < a.nsplit; ++s) {
                const float* ps = p + s * (D + 2);
                const float w = exp2f(ps[0] - M);
                L += ps[1] * w;
                A += ps[2 + e] * w;
            }
        }
        static_cast<__bf16*>(a.O)[row * D + e] = static_cast<__bf16>(L > 0.f ? A / L : 0.f);
    }
}

template <int D, int NQ>
int launch_dec(const DecodeArgs& a, int nqchunks, void* stream) {
    const dim3 grid(a.Hkv * nqchunks, a.B, a.nsplit);
    hipLaunchKernelGGL((sa_decode_kernel<D, NQ>), grid, dim3(kDecThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    if (a.nsplit > 1) {
        const unsigned rows = static_cast<unsigned>(size_t(a.B) * a.H * a.n_new);
        hipLaunchKernelGGL((sa_decode_merge_kernel<D>), dim3(rows), dim3(D < 128 ? D : 128), 0,
                           static_cast<hipStream_t>(stream), a);
        if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
    }
    return SA_OK;
}

template <int D>
int launch_dec_d(const DecodeArgs& a, void* stream) {
    const int nq_all = a.G * a.n_new;
    if (nq_all == 1) return launch_dec<D, 1>(a, 1, stream);
    if (nq_all == 2) return launch_dec<D, 2>(a, 1, stream);
    if (nq_all <= 4) return launch_dec<D, 4>(a, 1, stream);
    return launch_dec<D, 8>(a, (nq_all + 7) / 8, stream);
}

}  // namespace

int decode_scratch(size_t bytes, float** out) {
    if (bytes > kDecodeScratchBytes) return SA_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        // Once per device, with that device current.
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return SA_ERR_HIP;
        }
        scratch_addr[dev] = static_cast<float*>(p);
    }
    *out = scratch_addr[dev];
    return SA_OK;
}

int launch_decode(int d, const DecodeArgs& a, void* stream) {
    switch (d) {
        case 16: return launch_dec_d<16>(a, stream);
        case 32: return launch_dec_d<32>(a, stream);
        case 64: return launch_dec_d<64>(a, stream);
        case 128: return launch_dec_d<128>(a, stream);
        default: return SA_ERR_UNSUPPORTED;
    }
}

}  // namespace sa
