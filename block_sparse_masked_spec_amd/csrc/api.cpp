// C-ABI of libsparse_attn.so: argument checks, the per-device plan cache
// and the launch.  Every function is declared and documented in
// include/sparse_attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include "internal.hpp"

#define SA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using sa::DevicePlan;
using sa::HostPlan;
using sa::MaskRule;

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int check_globals(const sa_mask& m, int64_t T) {
    for (int k = 0; k < m.n_global; ++k)
        if (m.global_hi[k] > T) return SA_ERR_RANGE;
    return SA_OK;
}

// Parse + range-check; the common front half of every spec-taking call.
int parse_for(const char* spec, int T, sa_mask* m) {
    if (!spec) return SA_ERR_NULL;
    if (T < 1 || T > SA_MAX_T) return SA_ERR_SHAPE;
    int rc = sa::parse_mask_spec(spec, m);
    if (rc != SA_OK) return rc;
    return check_globals(*m, T);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

class PlanCache {
  public:
    // Returns SA_OK and a device plan for (spec, T) on the current device.
    int get(const sa_mask& m, int T, DevicePlan* out) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
        std::string key = sa::canonical_spec(m) + "|T=" + std::to_string(T) + "|bq=" +
                          std::to_string(sa::kBQ) + "|bk=" + std::to_string(sa::kBK) +
                          "|dev=" + std::to_string(dev);
        std::lock_guard<std::mutex> lock(mu_);
        auto it = plans_.find(key);
        if (it != plans_.end()) {
            *out = it->second.plan;
            return SA_OK;
        }
        HostPlan hp = sa::build_plan(MaskRule(m, T), sa::kBQ, sa::kBK);
        DevicePlan dp;
        dp.n_qb = hp.n_qb;
        size_t off = 0;
        auto section = [&](size_t bytes, size_t* where) {
            off = align_up(off, 16);
            *where = off;
            off += bytes;
        };
        section(hp.qb_order.size() * 4, &dp.off_qb_order);
        section(hp.run_ptr.size() * 4, &dp.off_run_ptr);
        section(hp.runs.size() * 4, &dp.off_runs);
        section(hp.gseg.size() * 4, &dp.off_gseg);
        section(hp.colkeys.size() * 4, &dp.off_colkeys);
        section(hp.colbits.size() * 8, &dp.off_colbits);
        section(hp.rowbits.size() * 4, &dp.off_rowbits);
        dp.bytes = align_up(off, 16) + 16;
        std::vector<unsigned char> host(dp.bytes, 0);
        auto put = [&](size_t where, const void* src, size_t bytes) {
            if (bytes) std::memcpy(host.data() + where, src, bytes);
        };
        put(dp.off_qb_order, hp.qb_order.data(), hp.qb_order.size() * 4);
        put(dp.off_run_ptr, hp.run_ptr.data(), hp.run_ptr.size() * 4);
        put(dp.off_runs, hp.runs.data(), hp.runs.size() * 4);
        put(dp.off_gseg, hp.gseg.data(), hp.gseg.size() * 4);
        put(dp.off_colkeys, hp.colkeys.data(), hp.colkeys.size() * 4);
        put(dp.off_colbits, hp.colbits.data(), hp.colbits.size() * 8);
        put(dp.off_rowbits, hp.rowbits.data(), hp.rowbits.size() * 4);
        if (hipMalloc(&dp.base, dp.bytes) != hipSuccess) {
            (void)hipGetLastError();
            return SA_ERR_NOMEM;
        }
        if (hipMemcpy(dp.base, host.data(), dp.bytes, hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(dp.base);
            return SA_ERR_HIP;
        }
        plans_.emplace(key, Entry{dp, dev});
        *out = dp;
        return SA_OK;
    }

    void release() {
        std::lock_guard<std::mutex> lock(mu_);
        int cur = 0;
        bool have_cur = hipGetDevice(&cur) == hipSuccess;
        for (auto& kv : plans_) {
            if (hipSetDevice(kv.second.device) == hipSuccess) (void)hipFree(kv.second.plan.base);
        }
        if (have_cur) (void)hipSetDevice(cur);
        plans_.clear();
    }

  private:
    struct Entry {
        DevicePlan plan;
        int device;
    };
    std::mutex mu_;
    std::unordered_map<std::string, Entry> plans_;
};

PlanCache& cache() {
    static PlanCache* c = new PlanCache();  // never destroyed: no teardown-order issues
    return *c;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int forward(int dtype, const void* Q, const void* K, const void* V, void* O, int B, int H, int T,
            int d, const char* spec, void* stream) {
    if (!Q || !K || !V || !O || !spec) return SA_ERR_NULL;
    if (B < 1 || H < 1 || T < 1 || T > SA_MAX_T) return SA_ERR_SHAPE;
    if (!supported_d(d)) return SA_ERR_UNSUPPORTED;
    const int64_t BH = int64_t(B) * H;
    const int64_t n_qb = (int64_t(T) + sa::kBQ - 1) / sa::kBQ;
    if (BH > INT32_MAX || BH * n_qb > INT32_MAX) return SA_ERR_SHAPE;
    for (const void* p : {Q, K, V, static_cast<const void*>(O)})
        if (reinterpret_cast<uintptr_t>(p) % 16) return SA_ERR_ALIGN;
    const size_t esz = dtype == SA_DTYPE_BF16 ? 2 : 4;
    const size_t bytes = size_t(BH) * size_t(T) * size_t(d) * esz;
    if (overlaps(O, bytes, Q, bytes) || overlaps(O, bytes, K, bytes) || overlaps(O, bytes, V, bytes))
        return SA_ERR_ALIAS;
    sa_mask m;
    int rc = parse_for(spec, T, &m);
    if (rc != SA_OK) return rc;
    // Pure dilated windows run as `sub` interleaved plain windows.
    const int sub = sa::residue_split(m, T, d, dtype) ? m.dilation : 1;
    if (sub > 1) m.dilation = 1;
    const int Ts = T / sub;
    if (BH * sub * ((int64_t(Ts) + sa::kBQ - 1) / sa::kBQ) > INT32_MAX) return SA_ERR_SHAPE;
    DevicePlan dp;
    rc = cache().get(m, Ts, &dp);
    if (rc != SA_OK) return rc;
    sa::FwdArgs a;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.T = Ts;
    a.BH = static_cast<int32_t>(BH * sub);
    a.sub = sub;
    a.causal = m.causal;
    // Band distances (as MaskRule::band_back/band_fwd) and the dilation grid.
    a.band_back = sa::band_reach32(m);
    a.band_fwd = m.causal ? 0 : a.band_back;
    a.dil = m.dilation > 1 ? m.dilation : 1;
    a.dil_pat = 0;
    for (int x = 0; x < 64; x += a.dil) a.dil_pat |= uint64_t(1) << x;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
    auto* base = static_cast<unsigned char*>(dp.base);
    a.qb_order = reinterpret_cast<const int32_t*>(base + dp.off_qb_order);
    a.run_ptr = reinterpret_cast<const int32_t*>(base + dp.off_run_ptr);
    a.runs = reinterpret_cast<const int32_t*>(base + dp.off_runs);
    a.gseg = reinterpret_cast<const int32_t*>(base + dp.off_gseg);
    a.colkeys = reinterpret_cast<const int32_t*>(base + dp.off_colkeys);
    a.colbits = reinterpret_cast<const uint64_t*>(base + dp.off_colbits);
    a.rowbits = reinterpret_cast<const uint32_t*>(base + dp.off_rowbits);
    const int64_t grid = int64_t(a.BH) * dp.n_qb;
    int lrc = sa::launch_fwd_fast(dtype, d, a, grid, stream);
    if (lrc == SA_ERR_UNSUPPORTED && sub == 1) lrc = sa::launch_fwd(dtype, d, a, grid, stream);
    return lrc;
}

template <typename F>
int guarded(F&& f) {
    try {
        return f();
    } catch (const std::bad_alloc&) {
        return SA_ERR_NOMEM;
    } catch (...) {
        return SA_ERR_HIP;
    }
}

}  // namespace

SA_EXPORT int sparse_attn_fwd(const void* Q, const void* K, const void* V, void* O, int B, int H,
                              int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] { return forward(SA_DTYPE_BF16, Q, K, V, O, B, H, T, d, mask_spec, stream); });
}

SA_EXPORT int sparse_attn_fwd_f32(const void* Q, const void* K, const void* V, void* O, int B,
                                  int H, int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] { return forward(SA_DTYPE_F32, Q, K, V, O, B, H, T, d, mask_spec, stream); });
}

SA_EXPORT int sparse_attn_parse(const char* mask_spec, sa_mask* out) {
    return guarded([&] { return sa::parse_mask_spec(mask_spec, out); });
}

SA_EXPORT int sparse_attn_count(const char* mask_spec, int T, int64_t* allowed_cells,
                                int32_t* row_counts) {
    return guarded([&] {
        if (!allowed_cells) return SA_ERR_NULL;
        sa_mask m;
        int rc = parse_for(mask_spec, T, &m);
        if (rc != SA_OK) return rc;
        MaskRule rule(m, T);
        int64_t total = 0;
        for (int64_t i = 0; i < T; ++i) {
            int64_t c = rule.allowed_in(i, 0, T);
            if (row_counts) row_counts[i] = static_cast<int32_t>(c);
            total += c;
        }
        *allowed_cells = total;
        return SA_OK;
    });
}

SA_EXPORT int sparse_attn_tile_map(const char* mask_spec, int T, int bq, int bk, uint8_t* map) {
    return guarded([&] {
        if (!map) return SA_ERR_NULL;
        if (bq < 1 || bk < 1) return SA_ERR_SHAPE;
        sa_mask m;
        int rc = parse_for(mask_spec, T, &m);
        if (rc != SA_OK) return rc;
        MaskRule rule(m, T);
        const int64_t nqb = (int64_t(T) + bq - 1) / bq, nkb = (int64_t(T) + bk - 1) / bk;
        for (int64_t qb = 0; qb < nqb; ++qb)
            for (int64_t kb = 0; kb < nkb; ++kb)
                map[qb * nkb + kb] = static_cast<uint8_t>(
                    rule.classify(qb * bq, (qb + 1) * bq, kb * bk, (kb + 1) * bk));
        return SA_OK;
    });
}

SA_EXPORT int sparse_attn_tile_shape(int d, int dtype, int* bq, int* bk) {
    if (!bq || !bk) return SA_ERR_NULL;
    if (!supported_d(d) || (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F32))
        return SA_ERR_UNSUPPORTED;
    *bq = sa::kBQ;
    *bk = sa::kBK;
    return SA_OK;
}

SA_EXPORT int sparse_attn_plan_info(const char* mask_spec, int T, int d, int dtype,
                                    sa_plan_info* info) {
    return guarded([&] {
        if (!info) return SA_ERR_NULL;
        int bq = 0, bk = 0;
        int rc = sparse_attn_tile_shape(d, dtype, &bq, &bk);
        if (rc != SA_OK) return rc;
        sa_mask m;
        rc = parse_for(mask_spec, T, &m);
        if (rc != SA_OK) return rc;
        MaskRule rule(m, T);
        // The plan the forward runs: for a residue split, one subsequence's.
        const int sub = sa::residue_split(m, T, d, dtype) ? m.dilation : 1;
        sa_mask mp = m;
        if (sub > 1) mp.dilation = 1;
        MaskRule prule(mp, T / sub);
        HostPlan hp = sa::build_plan(prule, bq, bk);
        std::memset(info, 0, sizeof(*info));
        info->bq = bq;
        info->bk = bk;
        info->n_qb = hp.n_qb;
        info->n_kb = hp.n_kb;
        info->subsequences = sub;
        info->inplace_tiles = hp.inplace_tiles * sub;
        info->masked_tiles = hp.masked_tiles * sub;
        info->gathered_tiles = hp.gathered_tiles * sub;
        info->gathered_keys = hp.gathered_keys * sub;
        info->executed_cells = int64_t(bq) * bk * (hp.inplace_tiles + hp.gathered_tiles) * sub;
        int64_t total = 0;
        for (int64_t i = 0; i < T; ++i) total += rule.allowed_in(i, 0, T);
        info->allowed_cells = total;
        return SA_OK;
    });
}

SA_EXPORT const char* sparse_attn_strerror(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_SPEC: return "mask spec does not parse";
        case SA_ERR_RANGE: return "a global index is not below T";
        case SA_ERR_SHAPE: return "bad shape (B, H or T < 1, T too large, or bad tile shape)";
        case SA_ERR_UNSUPPORTED: return "unsupported head dim or dtype (d must be 16, 32, 64 or 128)";
        case SA_ERR_NULL: return "a required pointer is NULL";
        case SA_ERR_ALIAS: return "output overlaps an input";
        case SA_ERR_HIP: return "HIP runtime or launch error";
        case SA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case SA_ERR_NOMEM: return "allocation failed";
        default: return "unknown status";
    }
}

SA_EXPORT void sparse_attn_release_cache(void) {
    try {
        cache().release();
    } catch (...) {
    }
}
