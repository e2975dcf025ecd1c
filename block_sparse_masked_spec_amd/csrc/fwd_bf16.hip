// Fast path of the fused forward kernel: bf16, head dim 64 or 128, gfx950.
//
// Same operation and tile plan as the generic kernel (fwd_kernel.hip): the
// softmax over S_i only ("Sparse attention", glossary.selfmadequant.com,
// "Choose the available reads"), live key tiles only ("Sparse and
// sliding-window attention", getnybble.com, "Implementation").  What differs
// is how a tile is fed to the matrix cores:
//
//   * a workgroup of NW wavefronts covers the query block of 128 rows; each
//     wave owns 32 queries (16 on the 64-row plans and on small grids, see
//     below).  At d = 64 they are one
//     32-wide MFMA column block (v_mfma_f32_32x32x16_bf16, NG groups of 32;
//     the launches use NG = 1).  At d = 128 they are two 16-query blocks of
//     v_mfma_f32_16x16x32_bf16: the same work in twice as many MFMAs of half
//     the length, which gives the scheduler finer interleave points (1-4%
//     faster there; 5-15% slower at d = 64).  Either way a wave needs at most
//     256 registers, so two waves share each SIMD and one wave's softmax can
//     run while the other's matrix products do;
//   * LDS holds each K and V tile "fragment-major": for every MFMA k-step,
//     the 64 lanes' operand pieces are stored contiguously in lane order.
//     Every fragment read is then lane_base + a compile-time offset and 32
//     lanes read 512 consecutive bytes (no bank conflicts, one address
//     register).  The permutation is done for free on the load side: the
//     tiles are filled by direct global->LDS loads (16 bytes per lane, no
//     register staging), each lane choosing its global source;
//   * two LDS buffers: tile t+1 is loaded while tile t is computed;
//   * V^T fragments come from transposed LDS reads (ds_read_b64_tr_b16):
//     within each 16-lane group, output lane j element e is element j%4 of
//     the 8-byte piece addressed by lane 4e + j/4 (checked on the hardware,
//     as are the 16x16x32 operand layouts and permlane16_swap's pairing);
//   * the running max moves only when a score exceeds it by more than 2^8
//     (log2 domain), so the accumulator rescale is almost never paid --
//     exact either way, since every weight of a row uses the same reference;
//   * row sums add the bf16-rounded weights with v_dot2 (the same values the
//     PV MFMA consumes);
//   * a workgroup runs one work item of the plan: a query block, or one
//     key range of a block far heavier than the mean (a block of global
//     rows), whose unnormalised result a merge kernel combines with the
//     block's other ranges.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.hpp"
#include "kernel_common.hpp"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
static_assert(sizeof(i32x16) == sizeof(int32_t) * kItemRec, "one item record");

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
typedef __attribute__((address_space(3))) s16x4* lptr_s16x4_t;
__device__ __forceinline__ gptr_t as_global(const void* p) { return (gptr_t)p; }
__device__ __forceinline__ lptr_t as_lds(void* p) { return (lptr_t)p; }
__device__ __forceinline__ lptr_s16x4_t as_lds_s16x4(const void* p) { return (lptr_s16x4_t)(void*)p; }

constexpr float kLazyTau = 8.0f;  // log2-domain slack before the max moves
static_assert(kBK == 64, "one column-bit word per key tile");

__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Tile shapes.  M16 selects the 16x16x32 MFMA (v_mfma_f32_16x16x32_bf16,
// used at d = 128), else the 32x32x16 one (d = 64); both run 2 products of
// the same cost per tile, with different fragment layouts.
template <int D, int NW, bool M16>
struct Lay {
    static constexpr int TILE = kBK * D * 2;           // bytes per K or V tile
    static constexpr int LOADS = TILE / 1024;          // 1 KiB wave-wide loads per tile
    static constexpr int LOADS_PER_WAVE = LOADS / NW;
    static constexpr int NKS = M16 ? D / 32 : D / 16;  // k-steps of S^T = K Q^T
    static constexpr int NDB = M16 ? D / 16 : D / 32;  // row blocks of O^T
    static constexpr int NKB = M16 ? 4 : 2;            // key blocks of a tile (16 or 32 keys)
    static_assert(LOADS == NKB * NKS && LOADS == (M16 ? 2 : 4) * NDB, "one 1 KiB block per fragment");
    static_assert(LOADS % NW == 0, "loads split evenly over the waves");
};

// Where the next tile comes from: a run of in-place key tiles or a slice of
// the gathered column keys.
struct Cursor {
    int run, run_end, kb, kb_end;
    bool masked;
    int gi, g_total;
    __device__ bool done() const { return run >= run_end && gi >= g_total; }
    __device__ bool inplace() const { return run < run_end; }
};

__device__ __forceinline__ void cursor_enter_run(Cursor& c, const FwdArgs& a) {
    if (c.run < c.run_end) {
        c.kb = ldc(a.runs, 2 * c.run);
        const int w = ldc(a.runs, 2 * c.run + 1);
        c.kb_end = w & 0x7fffffff;
        c.masked = w < 0;
    }
}

__device__ __forceinline__ void cursor_advance(Cursor& c, const FwdArgs& a) {
    if (c.run < c.run_end) {
        if (++c.kb == c.kb_end) {
            ++c.run;
            cursor_enter_run(c, a);
        }
    } else {
        c.gi += kBK;
    }
}

// Allowed keys of query qi in the tile at k0 (allowed_word with the tile's
// column bits read through the scalar cache).
__device__ __forceinline__ uint64_t rule_word(const FwdArgs& a, int qi, int k0, bool rowg,
                                              int qres, int k0res, int qblk) {
    return allowed_word(a, qi, k0, rowg, ldc(a.colbits, k0 >> 6), qres, k0res, qblk);
}

// 32x32x16 K tile layout: 1 KiB block (b, ks) = b * NKS + ks holds, at byte lane*16,
// the A fragment of lane (n = lane%32, h = lane/32) for key block b and
// k-step ks: K[b*32 + swap23(n)][ks*16 + h*8 .. +8].  Rows enter the MFMA in
// swap23 order so that a lane's 8 scores of one PV k-step are 8 consecutive
// keys (register r of block b then holds key b*32 + (r/8)*16 + h*8 + r%8).
//
// 32x32x16 V tile layout: 1 KiB block (kk, db) = kk * NDB + db holds two 512-byte
// halves rd = 0, 1; transposed-read lane l reads 8 bytes at rd*512 + l*8:
// V[kk*16 + h*8 + (l%16)/4 + 4*rd][db*32 + ((l/16)%2)*16 + (l%4)*4 .. +4].
// After the transposed read, lane (n, h) holds V^T[db*32 + n][kk*16 + h*8 +
// e] for e = 0..7 (rd = 0 gives e < 4) -- the A fragment of O^T += V^T P^T.

// 16x16x32 K tile layout: 1 KiB block (kb, ks) = kb * NKS + ks holds lane
// l's A fragment, K[row(kb, l%16)][ks*32 + 8*(l/16) .. +8], with row(kb, r)
// = (kb/2)*32 + 8*(r/4) + 4*(kb%2) + r%4: the four score rows that lane group
// g = l/16 holds of blocks 2kk and 2kk+1 are then keys kk*32 + 8g .. +8, the
// B fragment of the PV product for that 32-key step.
//
// 16x16x32 V tile layout: 1 KiB block (kk, db) = kk * NDB + db holds two
// 512-byte halves rd; transposed-read lane l = 16g + 4e + q reads 8 bytes at
// rd*512 + l*8: V[kk*32 + 8g + 4rd + e][db*16 + 4q .. +4].  After the two
// transposed reads lane (16g + j) holds V^T[db*16 + j][kk*32 + 8g + e], e =
// 0..7 -- the A fragment of O^T += V^T P^T.

// Tile row (key slot 0..63) that load gi of a tile, lane `lane`, copies, and
// the element offset within that key's row.
template <int D, bool M16>
__device__ __forceinline__ void k_piece(int gi, int lane, int* row, int* col) {
    if constexpr (M16) {
        constexpr int NKS = D / 32;
        const int kb = gi / NKS, ks = gi % NKS, r = lane & 15;
        *row = (kb >> 1) * 32 + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3);
        *col = ks * 32 + 8 * (lane >> 4);
    } else {
        constexpr int NKS = D / 16;
        *row = (gi / NKS) * 32 + swap23(lane & 31);
        *col = (gi % NKS) * 16 + (lane >> 5) * 8;
    }
}
template <int D, bool M16>
__device__ __forceinline__ void v_piece(int gi, int lane, int* row, int* col) {
    if constexpr (M16) {
        constexpr int NDB = D / 16;
        const int kk = gi / NDB, db = gi % NDB;
        const int rd = lane >> 5, l0 = 2 * (lane & 31);
        const int g = l0 >> 4, e = (l0 & 15) >> 2, q = l0 & 3;
        *row = kk * 32 + 8 * g + 4 * rd + e;
        *col = db * 16 + 4 * q;
    } else {
        constexpr int NDB = D / 32;
        const int kk = gi / NDB, db = gi % NDB;
        const int rd = lane >> 5, l0 = 2 * (lane & 31);
        const int g = l0 >> 4, L = l0 & 15, h = l0 >> 5;
        *row = kk * 16 + h * 8 + (L >> 2) + 4 * rd;
        *col = db * 32 + (g & 1) * 16 + (L & 3) * 4;
    }
}

// The direct loads of one K tile and one V tile (this wave's share), as
// buffer loads into LDS.  A lane's piece of an in-place tile sits at a fixed
// byte offset from the tile's first row (computed once), and the tile's
// first row is a scalar offset: issuing a tile costs no vector arithmetic.
// Only a tile that runs past T takes per-lane offsets, with its missing rows
// clamped to row T - 1 (the mask gives them zero weight), and so do
// gathered tiles, whose keys are read from the plan before the first load is
// issued (no wait lands between the loads).  Each kind of tile issues its
// own loads: were the paths joined before the loads, the in-place path would
// inherit the wait on the gathered path's key reads -- and, since vector
// loads complete in order, on every load in flight.  The marker after each
// path's loads keeps the compiler from merging them.
template <int D, int NW, bool M16>
struct TileLoad {
    using L = Lay<D, NW, M16>;
    __amdgpu_buffer_rsrc_t krsrc, vrsrc;
    int rowb;                                  // bytes between key rows
    int wave;
    int kr[L::LOADS_PER_WAVE], vr[L::LOADS_PER_WAVE];      // tile row of each piece
    int koff[L::LOADS_PER_WAVE], voff[L::LOADS_PER_WAVE];  // byte offset in the tile

    __device__ __forceinline__ TileLoad(const __bf16* Kp, const __bf16* Vp, int T, size_t rs, int wave_,
                                        int lane)
        : rowb(int(rs) * 2), wave(wave_) {
        // The sequence's rows span at most T * rs elements (at most 1 GiB for
        // T <= SA_MAX_T), so every offset fits the buffer's 32 bits.
        const int bytes = int(size_t(T) * rs * 2);
        krsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Kp), 0, bytes, 0x00020000);
        vrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Vp), 0, bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < L::LOADS_PER_WAVE; ++i) {
            const int gi = wave * L::LOADS_PER_WAVE + i;
            int kc, vc;
            k_piece<D, M16>(gi, lane, &kr[i], &kc);
            v_piece<D, M16>(gi, lane, &vr[i], &vc);
            koff[i] = kr[i] * rowb + kc * 2;
            voff[i] = vr[i] * rowb + vc * 2;
        }
    }

    __device__ __forceinline__ void put(char* kdst, char* vdst, const int (&ko)[L::LOADS_PER_WAVE],
                                        const int (&vo)[L::LOADS_PER_WAVE], int soff) const {
#pragma unroll
        for (int i = 0; i < L::LOADS_PER_WAVE; ++i) {
            const int gi = wave * L::LOADS_PER_WAVE + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, as_lds(kdst + gi * 1024), 16, ko[i], soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, as_lds(vdst + gi * 1024), 16, vo[i], soff, 0, 0);
        }
    }

    __device__ __forceinline__ void issue(const Cursor& c, const FwdArgs& a, char* kdst, char* vdst, int T,
                                          int ga0, int gna, int gb0) const {
        int ko[L::LOADS_PER_WAVE], vo[L::LOADS_PER_WAVE];
        if (c.inplace()) {
            const int k0 = c.kb * kBK;
            if (k0 + kBK <= T) {
                put(kdst, vdst, koff, voff, k0 * rowb);
                asm volatile("; tile loads issued: in place" ::: "memory");
            } else {
#pragma unroll
                for (int i = 0; i < L::LOADS_PER_WAVE; ++i) {
                    ko[i] = koff[i] + (min(k0 + kr[i], T - 1) - kr[i]) * rowb;
                    vo[i] = voff[i] + (min(k0 + vr[i], T - 1) - vr[i]) * rowb;
                }
                put(kdst, vdst, ko, vo, 0);
                asm volatile("; tile loads issued: past T" ::: "memory");
            }
        } else {
#pragma unroll
            for (int i = 0; i < L::LOADS_PER_WAVE; ++i) {
                const int ks = min(c.gi + kr[i], c.g_total - 1), vs = min(c.gi + vr[i], c.g_total - 1);
                const int kkey = a.colkeys[ks < gna ? ga0 + ks : gb0 + (ks - gna)];
                const int vkey = a.colkeys[vs < gna ? ga0 + vs : gb0 + (vs - gna)];
                ko[i] = koff[i] + (kkey - kr[i]) * rowb;
                vo[i] = voff[i] + (vkey - vr[i]) * rowb;
            }
            put(kdst, vdst, ko, vo, 0);
            asm volatile("; tile loads issued: gathered keys" ::: "memory");
        }
    }
};

// End of a tile: this wave's direct loads of the next tile have landed and
// every wave has finished the current one.  Only vmcnt is drained (the
// scalar plan reads already in flight for later tiles may stay in flight);
// the scheduling barriers keep every LDS read of the current tile before
// the barrier and every read of the next tile after it.
__device__ __forceinline__ void tile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left alone
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// 32x32x16 tiles: the wave's queries as NG groups of 32, one per lane column
// (lane l holds query l%32 of each group).
template <int D, int NG, int NW>
struct WaveState {
    using L = Lay<D, NW, false>;
    static constexpr int NQ = NG;     // queries per lane
    static constexpr int SLOT = 32;   // queries per group
    bf16x8 qf[NG][L::NKS];   // Q^T fragments of the wave's query groups
    f32x16 acc[NG][L::NDB];  // O^T accumulators
    float m_run[NG], l_run[NG];

    static __device__ __forceinline__ int query(int lane) { return lane & 31; }
    // one lane per query writes the row's LSE or partial max and sum
    static __device__ __forceinline__ bool owns_row(int lane) { return lane < 32; }
    __device__ __forceinline__ void load_q(int g, const __bf16* Qp, int qi, size_t rs, int T, int lane) {
#pragma unroll
        for (int ks = 0; ks < L::NKS; ++ks) {
            qf[g][ks] = bf16x8{};
            if (qi < T) qf[g][ks] = *reinterpret_cast<const bf16x8*>(Qp + size_t(qi) * rs + ks * 16 + (lane >> 5) * 8);
        }
#pragma unroll
        for (int db = 0; db < L::NDB; ++db) acc[g][db] = f32x16{};
        m_run[g] = -1e30f;
        l_run[g] = 0.f;
    }
    // l over both lane halves
    __device__ __forceinline__ float row_sum(int g) const {
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[g]), __float_as_uint(l_run[g]),
                                                         false, false);
        return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    // f(d0, four accumulator values of output columns d0 .. d0+3)
    template <typename F>
    __device__ __forceinline__ void outputs(int g, int lane, F f) const {
#pragma unroll
        for (int db = 0; db < L::NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[g][db][r4 * 4 + e];
                f(db * 32 + r4 * 8 + (lane >> 5) * 4, v);
            }
    }

    // One 64-key tile.  With `masked`, allowed[g] has bit k set iff key k of
    // the tile is allowed for this lane's query of group g.
    __device__ __forceinline__ void tile(const char* kt, const char* vt, const FwdArgs& a, int lane,
                                         bool masked, const uint64_t (&allowed)[NG]) {
        const int h = lane >> 5;
        f32x16 s[NG][2];  // [query group][32-key block]
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int b = 0; b < 2; ++b) s[g][b] = f32x16{};
        // S^T = K Q^T: one K fragment feeds every query group of the wave.
        // All of the tile's K fragments are read first, then the MFMAs run
        // (the fragment registers are free again before the V^T reads);
        // otherwise the scheduler spreads the V^T reads between the QK MFMAs
        // and every later K fragment waits for all of them.
        bf16x8 kfa[2 * L::NKS];
#pragma unroll
        for (int i = 0; i < 2 * L::NKS; ++i) kfa[i] = *reinterpret_cast<const bf16x8*>(kt + i * 1024 + lane * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * L::NKS; ++i)
#pragma unroll
            for (int g = 0; g < NG; ++g)
                s[g][i / L::NKS] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfa[i], qf[g][i % L::NKS], s[g][i / L::NKS], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // V^T fragment i (two transposed reads).  With one query group the
        // whole tile's fragments are read here, so that they arrive while
        // the softmax runs; with two there is no room and each is read just
        // before its products.
        auto vt_frag = [&](int i) {
            const char* blk = vt + i * 1024 + lane * 8;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(blk));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(blk + 512));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr bool kEarlyV = NG == 1;
        bf16x8 vfa[kEarlyV ? 4 * L::NDB : 1];
        if constexpr (kEarlyV) {
#pragma unroll
            for (int i = 0; i < 4 * L::NDB; ++i) vfa[i] = vt_frag(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pf[NG][4];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (masked) {
                // Register r of block b holds key b*32 + (r/8)*16 + h*8 + r%8.
                const uint64_t mine = allowed[g] >> (h * 8);
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int bit = b * 32 + (r >> 3) * 16 + (r & 7);
                        if (!((mine >> bit) & 1)) s[g][b][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[g][b][r]);
            {
                const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                 __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
            }
            const float ms = mx * a.scale_log2;
            if (__any(ms > m_run[g] + kLazyTau)) {
                const float m_new = fmaxf(m_run[g], ms);
                const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
                m_run[g] = m_new;
                l_run[g] *= alpha;
#pragma unroll
                for (int db = 0; db < L::NDB; ++db) acc[g][db] *= alpha;
            }
            const float mneg = -m_run[g];
            bf16x2 ones;
            ones[0] = static_cast<__bf16>(1.0f);
            ones[1] = static_cast<__bf16>(1.0f);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pf[g][kk][e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(
                        fmaf(s[g][kk >> 1][(kk & 1) * 8 + e], a.scale_log2, mneg)));
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    bf16x2 pair;
                    pair[0] = pf[g][kk][e];
                    pair[1] = pf[g][kk][e + 1];
                    l_run[g] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, l_run[g], false);
                }
            }
        }
        // O^T += V^T P^T: one V^T fragment feeds every query group of the wave.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int db = 0; db < L::NDB; ++db) {
                bf16x8 vf;
                if constexpr (kEarlyV)
                    vf = vfa[kk * L::NDB + db];
                else
                    vf = vt_frag(kk * L::NDB + db);
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    acc[g][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[g][kk], acc[g][db], 0, 0, 0);
            }
    }
};

// 16x16x32 tiles: the wave's queries as NQB blocks of 16 (two at d = 128;
// one in the 16-query waves of small grids); lane l holds query l%16 of
// each block, and lane group g = l/16 holds score rows 4g .. 4g+3 of each
// 16-key block (keys of the tile as the K layout orders them).
template <int D, int NW, int NQB>
struct WaveState16 {
    using L = Lay<D, NW, true>;
    static constexpr int NQ = NQB;    // queries per lane (16-query blocks per wave)
    static constexpr int SLOT = 16;   // queries per block
    bf16x8 qf[NQ][L::NKS];   // Q^T fragments (B operands)
    f32x4 acc[L::NDB][NQ];   // O^T accumulators
    float m_run[NQ], l_run[NQ];

    static __device__ __forceinline__ int query(int lane) { return lane & 15; }
    static __device__ __forceinline__ bool owns_row(int lane) { return lane < 16; }
    __device__ __forceinline__ void load_q(int qh, const __bf16* Qp, int qi, size_t rs, int T, int lane) {
#pragma unroll
        for (int ks = 0; ks < L::NKS; ++ks) {
            qf[qh][ks] = bf16x8{};
            if (qi < T) qf[qh][ks] = *reinterpret_cast<const bf16x8*>(Qp + size_t(qi) * rs + ks * 32 + (lane >> 4) * 8);
        }
#pragma unroll
        for (int db = 0; db < L::NDB; ++db) acc[db][qh] = f32x4{};
        m_run[qh] = -1e30f;
        l_run[qh] = 0.f;
    }
    // l over the four lane groups that share the query
    __device__ __forceinline__ float row_sum(int qh) const {
        const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run[qh]), __float_as_uint(l_run[qh]),
                                                          false, false);
        const float x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
        const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
    }
    template <typename F>
    __device__ __forceinline__ void outputs(int qh, int lane, F f) const {
#pragma unroll
        for (int db = 0; db < L::NDB; ++db) f(db * 16 + (lane >> 4) * 4, acc[db][qh]);
    }

    // One 64-key tile.  With `masked`, allowed[qh] has bit k set iff key k
    // of the tile is allowed for this lane's query of block qh.
    __device__ __forceinline__ void tile(const char* kt, const char* vt, const FwdArgs& a, int lane,
                                         bool masked, const uint64_t (&allowed)[NQ]) {
        const int g = lane >> 4;
        f32x4 s[4][NQ];  // [16-key block][query block]
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qh = 0; qh < NQ; ++qh) s[kb][qh] = f32x4{};
        // S^T = K Q^T: each K fragment feeds both query blocks.  All of the
        // tile's K fragments are read first, then the MFMAs run.
        bf16x8 kfa[4 * L::NKS];
#pragma unroll
        for (int i = 0; i < 4 * L::NKS; ++i) kfa[i] = *reinterpret_cast<const bf16x8*>(kt + i * 1024 + lane * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4 * L::NKS; ++i)
#pragma unroll
            for (int qh = 0; qh < NQ; ++qh)
                s[i / L::NKS][qh] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfa[i], qf[qh][i % L::NKS], s[i / L::NKS][qh], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // Every V^T fragment of the tile, read while the softmax runs.
        bf16x8 vfa[2 * L::NDB];
#pragma unroll
        for (int i = 0; i < 2 * L::NDB; ++i) {
            const char* blk = vt + i * 1024 + lane * 8;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(blk));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds_s16x4(blk + 512));
            vfa[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 pf[NQ][2];  // [query block][32-key step]
#pragma unroll
        for (int qh = 0; qh < NQ; ++qh) {
            if (masked) {
                // score t of block kb is key (kb/2)*32 + 8g + 4*(kb%2) + t
                const uint64_t mine = allowed[qh] >> (8 * g);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int bit = (kb >> 1) * 32 + 4 * (kb & 1) + t;
                        if (!((mine >> bit) & 1)) s[kb][qh][t] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int t = 0; t < 4; ++t) mx = fmaxf(mx, s[kb][qh][t]);
            {  // over the four lane groups of the query
                const auto p16 =
                    __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
                const auto p32 =
                    __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
            }
            const float ms = mx * a.scale_log2;
            if (__any(ms > m_run[qh] + kLazyTau)) {
                const float m_new = fmaxf(m_run[qh], ms);
                const float alpha = __builtin_amdgcn_exp2f(m_run[qh] - m_new);
                m_run[qh] = m_new;
                l_run[qh] *= alpha;
#pragma unroll
                for (int db = 0; db < L::NDB; ++db) acc[db][qh] *= alpha;
            }
            const float mneg = -m_run[qh];
            bf16x2 ones;
            ones[0] = static_cast<__bf16>(1.0f);
            ones[1] = static_cast<__bf16>(1.0f);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pf[qh][kk][e] = static_cast<__bf16>(
                        __builtin_amdgcn_exp2f(fmaf(s[2 * kk + (e >> 2)][qh][e & 3], a.scale_log2, mneg)));
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    bf16x2 pair;
                    pair[0] = pf[qh][kk][e];
                    pair[1] = pf[qh][kk][e + 1];
                    l_run[qh] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, l_run[qh], false);
                }
            }
        }
        // O^T += V^T P^T: each V^T fragment feeds both query blocks.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < L::NDB; ++db)
#pragma unroll
                for (int qh = 0; qh < NQ; ++qh)
                    acc[db][qh] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfa[kk * L::NDB + db], pf[qh][kk], acc[db][qh], 0, 0, 0);
    }
};

// Waves per SIMD to ask the compiler for: two when a wave holds one query
// group (fits in 256 registers), else one.
template <int NG>
struct Occupancy {
    static constexpr int kWavesPerSimd = NG == 1 ? 2 : 1;
};

// QW: queries per wave.  32: NG groups of 32 (d = 64) or two 16-query
// blocks (d = 128); 16: one 16-query block per wave, at d = 64 on the 64-row
// plans (four waves: block mode with 64-key blocks, and token-level calls
// whose 128-row blocks would not give every CU a workgroup) and on grids of
// up to 512 128-row blocks (eight waves), where 32-query waves would leave
// SIMDs with one wave.
template <int D, int NG, int NW, bool SUB, int QW>
__global__ __launch_bounds__(NW * 64, Occupancy<NG>::kWavesPerSimd) void sa_fwd_bf16_kernel(FwdArgs a) {
    constexpr int BQ = NW * NG * QW;  // waves x queries per wave = one query block
    static_assert(BQ == kBQ || BQ == 64, "query blocks of the plans: 128 or 64 rows");
    // d = 128 runs the 16x16x32 tiles (measured 1-4% faster there), d = 64
    // the 32x32x16 ones (the 16x16x32 form measured 5-15% slower at d = 64)
    // except in the 16-query waves.
    constexpr bool M16 = D == 128 || QW == 16;
    static_assert(!M16 || NG == 1, "16x16x32 tiles: one query group per wave");
    using L = Lay<D, NW, M16>;
    using WS = std::conditional_t<M16, WaveState16<D, NW, QW / 16>, WaveState<D, NG, NW>>;
    constexpr int NQ = WS::NQ;

    // The wave index is uniform across the wave; readfirstlane lets the
    // compiler keep it, and every address derived from it, in scalar registers.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int work = xcd_slice_index(blockIdx.x, gridDim.x);
    const int n_items = gridDim.x / a.BH;
    const int bh = work / n_items;
    // The work item (a query block or part of one): its whole record in one
    // scalar load, so the first tile's loads wait on a single read.
    const i32x16 rec = ldc(reinterpret_cast<const i32x16*>(a.item_rec), work % n_items);
    const int qb = rec[REC_QB];
    const int T = a.T;
    // Row stride and base of this sequence; with SUB, sequence bh is residue
    // class bh % sub of the full sequence bh / sub.
    const size_t rs = SUB ? size_t(a.sub) * D : size_t(D);
    const size_t base = SUB ? (size_t(bh / a.sub) * size_t(T) * a.sub + size_t(bh % a.sub)) * D
                            : size_t(bh) * size_t(T) * D;
    const __bf16* Qp = static_cast<const __bf16*>(a.Q) + base;
    const __bf16* Kp = static_cast<const __bf16*>(a.K) + base;
    const __bf16* Vp = static_cast<const __bf16*>(a.V) + base;
    __bf16* Op = static_cast<__bf16*>(a.O) + base;
    const int q_base = qb * BQ + wave * NG * QW;
    const TileLoad<D, NW, M16> ld(Kp, Vp, T, rs, wave, lane);

    // Lane `lane` holds query qi(x) of each of its NQ query slots.
    auto qi_of = [&](int x) { return q_base + x * WS::SLOT + WS::query(lane); };
    WS st;
    bool rowg[NQ];
    int qres[NQ];  // query index mod the dilation
    int qblk[NQ];  // block mode: the query's block (padding rows use the last row's)
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
        const int qi = qi_of(x);
        st.load_q(x, Qp, qi, rs, T, lane);
        // A slot's queries share one word of the global-row bits (read
        // through the scalar cache, so it adds no wait on the Q loads).
        const uint32_t rw = ldc(a.rowbits, min(q_base + x * WS::SLOT, T - 1) >> 5);
        rowg[x] = qi < T && ((rw >> (qi & 31)) & 1u);
        qres[x] = a.dil == 1 ? 0 : qi % a.dil;
        qblk[x] = a.blk > 0 ? min(qi, T - 1) / a.blk : 0;
    }

    const int ga0 = rec[REC_GA0], gna = rec[REC_GA1] - ga0, gb0 = rec[REC_GB0];
    Cursor cur{rec[REC_RUN_BEGIN], rec[REC_RUN_END], rec[REC_FIRST_KB], rec[REC_FIRST_END] & 0x7fffffff,
               rec[REC_FIRST_END] < 0, 0, gna + (rec[REC_GB1] - gb0)};

    auto run_tile = [&](const Cursor& c, const char* kt, const char* vt) {
        // A full chunk of gathered keys needs no mask: only a chunk's unused
        // slots are masked.  The 16x16x32 kernels mask every gathered tile
        // all the same: skipping it there measured slower on layers without
        // any gathered tile (the code moves).
        const bool masked = c.inplace() ? c.masked : M16 || c.g_total - c.gi < kBK;
        uint64_t allowed[NQ];
        const int k0res = a.dil == 1 ? 0 : (c.kb * kBK) % a.dil;
#pragma unroll
        for (int x = 0; x < NQ; ++x) {
            allowed[x] = ~0ull;
            if (masked)
                allowed[x] = c.inplace() ? rule_word(a, qi_of(x), c.kb * kBK, rowg[x], qres[x], k0res, qblk[x])
                                         : low_bits(min(kBK, c.g_total - c.gi));
        }
        st.tile(kt, vt, a, lane, masked, allowed);
    };

    // Two buffers as distinct objects, indexed statically (the loop below is
    // unrolled by two), so the compiler can tell the prefetch into one from
    // the reads of the other and keeps the prefetch in flight.
    __shared__ __attribute__((aligned(1024))) char kbuf0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char kbuf1[L::TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf1[L::TILE];
    if (!cur.done()) ld.issue(cur, a, kbuf0, vbuf0, T, ga0, gna, gb0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed
    __syncthreads();                // ... and the other waves'
    while (!cur.done()) {
        Cursor nxt = cur;
        cursor_advance(nxt, a);
        if (!nxt.done()) ld.issue(nxt, a, kbuf1, vbuf1, T, ga0, gna, gb0);
        run_tile(cur, kbuf0, vbuf0);
        tile_barrier();
        if (nxt.done()) break;
        cur = nxt;
        cursor_advance(nxt, a);
        if (!nxt.done()) ld.issue(nxt, a, kbuf0, vbuf0, T, ga0, gna, gb0);
        run_tile(cur, kbuf1, vbuf1);
        tile_barrier();
        cur = nxt;
    }

    // Epilogue: O = acc / l (l summed over the lanes that share the query),
    // or -- for one part of a split block -- acc, the running max and l into
    // the item's slot.
    const int part = rec[REC_PART];
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
        const int qi = qi_of(x);
        const float lt = st.row_sum(x);
        if (part >= 0) {
            const size_t slot = (size_t(bh) * a.n_parts + part) * BQ + (qi - qb * BQ);
            float* po = a.part + slot * D;
            st.outputs(x, lane, [&](int d0, const f32x4& v) {
                float4 q;
                q.x = v[0];
                q.y = v[1];
                q.z = v[2];
                q.w = v[3];
                *reinterpret_cast<float4*>(po + d0) = q;
            });
            if (WS::owns_row(lane)) {
                float2 ml;
                ml.x = st.m_run[x];
                ml.y = lt;
                reinterpret_cast<float2*>(a.part + size_t(a.BH) * a.n_parts * BQ * D)[slot] = ml;
            }
            continue;
        }
        const float inv = 1.f / lt;
        if (a.lse && qi < T && WS::owns_row(lane)) {  // log-sum-exp: the scores are in log2 units
            const size_t row = SUB ? size_t(bh / a.sub) * size_t(T) * a.sub + size_t(bh % a.sub) +
                                         size_t(qi) * a.sub
                                   : size_t(bh) * size_t(T) + size_t(qi);
            a.lse[row] = (st.m_run[x] + __log2f(lt)) * 0.6931471805599453f;
        }
        if (qi < T)
            st.outputs(x, lane, [&](int d0, const f32x4& v) {
                bf16x4 q;
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = static_cast<__bf16>(v[e] * inv);
                *reinterpret_cast<bf16x4*>(Op + size_t(qi) * rs + d0) = q;
            });
    }
}

// Merge of a split block's partial slots: one thread per (row, 4 columns),
// 256 / (D/4) rows per workgroup.  With m_p and l_p the part's reference max
// (log2 units) and row sum and acc_p its unnormalised output, the row's
// result is sum_p 2^(m_p - m) acc_p / sum_p 2^(m_p - m) l_p for
// m = max_p m_p: the online softmax's own rescaling, applied across parts (a
// part without an allowed key for the row has l_p = 0, acc_p = 0).
template <int D>
struct MergeShape {
    static constexpr int C = D / 4;      // float4 pieces per row
    static constexpr int RPW = 256 / C;  // rows per workgroup
};

template <int D>
__global__ __launch_bounds__(256) void sa_fwd_merge_kernel(FwdArgs a, const int32_t* split_qb,
                                                            const int32_t* split_ptr, int n_split) {
    using M = MergeShape<D>;
    const int BQ = a.bq, T = a.T;
    const int per_blk = BQ / M::RPW;  // workgroups per split block
    const int x = blockIdx.x % per_blk, y = blockIdx.x / per_blk;
    const int bh = y / n_split, sidx = y % n_split;
    const int r = x * M::RPW + threadIdx.x / M::C, c = threadIdx.x % M::C;
    const int qb = split_qb[sidx], p0 = split_ptr[sidx], p1 = split_ptr[sidx + 1];
    const int qi = qb * BQ + r;
    if (qi >= T) return;
    const float2* pml = reinterpret_cast<const float2*>(a.part + size_t(a.BH) * a.n_parts * BQ * D);
    const size_t slot0 = size_t(bh) * a.n_parts * BQ + r;  // slot of part p: slot0 + p * BQ
    float m = -INFINITY;
    for (int p = p0; p < p1; ++p) m = fmaxf(m, pml[slot0 + size_t(p) * BQ].x);
    float l = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    for (int p = p0; p < p1; ++p) {
        const size_t slot = slot0 + size_t(p) * BQ;
        const float2 ml = pml[slot];
        const float w = __builtin_amdgcn_exp2f(ml.x - m);
        const float4 v = *reinterpret_cast<const float4*>(a.part + slot * D + c * 4);
        l = fmaf(w, ml.y, l);
        o0 = fmaf(w, v.x, o0);
        o1 = fmaf(w, v.y, o1);
        o2 = fmaf(w, v.z, o2);
        o3 = fmaf(w, v.w, o3);
    }
    const float inv = 1.f / l;
    bf16x4 q;
    q[0] = static_cast<__bf16>(o0 * inv);
    q[1] = static_cast<__bf16>(o1 * inv);
    q[2] = static_cast<__bf16>(o2 * inv);
    q[3] = static_cast<__bf16>(o3 * inv);
    __bf16* Op = static_cast<__bf16*>(a.O) + size_t(bh) * size_t(T) * D;
    *reinterpret_cast<bf16x4*>(Op + size_t(qi) * D + c * 4) = q;
    if (a.lse && c == 0) a.lse[size_t(bh) * T + qi] = (m + __log2f(l)) * 0.6931471805599453f;
}

#ifndef SA_FWD_SMALL_GRID
#define SA_FWD_SMALL_GRID 512
#endif

template <int D, int NG, int NW, bool SUB = false, int QW = 32>
int launch_t(const FwdArgs& a, int64_t grid, void* stream) {
    hipLaunchKernelGGL((sa_fwd_bf16_kernel<D, NG, NW, SUB, QW>), dim3(static_cast<unsigned>(grid)),
                       dim3(NW * 64), 0, static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace

int launch_fwd_merge(int d, const FwdArgs& a, const int32_t* split_qb, const int32_t* split_ptr,
                     int32_t n_split, void* stream) {
    if (n_split <= 0 || a.sub != 1) return SA_ERR_UNSUPPORTED;
    auto go = [&](auto kernel, int rpw) {
        if (a.bq % rpw) return SA_ERR_UNSUPPORTED;
        const int64_t g = int64_t(a.BH) * n_split * (a.bq / rpw);
        if (g > INT32_MAX) return SA_ERR_SHAPE;
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(g)), dim3(256), 0, static_cast<hipStream_t>(stream),
                           a, split_qb, split_ptr, n_split);
        return SA_OK;
    };
    int rc = d == 128 ? go(sa_fwd_merge_kernel<128>, MergeShape<128>::RPW)
             : d == 64 ? go(sa_fwd_merge_kernel<64>, MergeShape<64>::RPW)
                       : SA_ERR_UNSUPPORTED;
    if (rc != SA_OK) return rc;
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// Returns SA_ERR_UNSUPPORTED when (dtype, d) has no fast path.
int launch_fwd_fast(int dtype, int d, const FwdArgs& a, int64_t grid, void* stream) {
    if (dtype != SA_DTYPE_BF16) return SA_ERR_UNSUPPORTED;
    if (a.sub > 1 && a.bq != kBQ) return SA_ERR_UNSUPPORTED;
    if (a.sub > 1) {  // interleaved subsequences: strided rows
        if (d == 128) return launch_t<128, 1, 4, true>(a, grid, stream);
        if (d == 64) return launch_t<64, 1, 4, true>(a, grid, stream);
        return SA_ERR_UNSUPPORTED;
    }
    // 64-row plans (block mode with 64-key blocks, and token-level calls
    // too small to fill the GPU): four 16-query waves per block.
    if (a.bq == 64) return d == 64 ? launch_t<64, 1, 4, false, 16>(a, grid, stream) : SA_ERR_UNSUPPORTED;
    if (d == 128) return launch_t<128, 1, 4>(a, grid, stream);
    if (d == 64 && grid <= SA_FWD_SMALL_GRID) return launch_t<64, 1, 8, false, 16>(a, grid, stream);
    if (d == 64) return launch_t<64, 1, 4>(a, grid, stream);
    return SA_ERR_UNSUPPORTED;
}

}  // namespace sa
