// C-ABI of libsparse_attn.so: argument checks, the per-device plan cache
// and the launch.  Every function is declared and documented in
// include/sparse_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <sstream>
#include <string>
#include <thread>
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

// Largest workspace the split partials may take.
constexpr size_t kMaxSplitWorkspace = size_t(1) << 30;

// Tile cap of the fast path's work items: automatic, or SA_FWD_SPLIT_TILES=n
// (n > 0) to split every query block above n tiles.
int64_t split_cap() {
    const char* e = getenv("SA_FWD_SPLIT_TILES");
    const long long n = e ? atoll(e) : 0;
    return n > 0 ? n : sa::kSplitAuto;
}

// One device plan: its device copy, the pinned host copy it was uploaded
// from (kept alive by the entry) and the event that marks the end of the
// upload on the stream of the call that built it.
struct Upload {
    void* dev_base = nullptr;
    void* host = nullptr;
    hipEvent_t done = nullptr;
    bool complete = false;
    int device = 0;

    // Make `stream` wait for the upload (a no-op once it has completed).
    int order_after(void* stream) {
        if (complete) return SA_OK;
        const hipError_t q = hipEventQuery(done);
        if (q == hipSuccess) {
            complete = true;
            return SA_OK;
        }
        if (q != hipErrorNotReady) return SA_ERR_HIP;
        return hipStreamWaitEvent(static_cast<hipStream_t>(stream), done, 0) == hipSuccess ? SA_OK
                                                                                            : SA_ERR_HIP;
    }

    void free_all() {
        if (done) (void)hipEventDestroy(done);
        if (host) (void)hipHostFree(host);
        if (dev_base) (void)hipFree(dev_base);
        done = nullptr;
        host = nullptr;
        dev_base = nullptr;
    }
};

// Copy `bytes` of host plan data to a new device allocation, stream-ordered:
// a pinned staging buffer, hipMemcpyAsync on `stream`, an event after it.
int upload(const std::vector<unsigned char>& data, void* stream, int device, Upload* up) {
    Upload u;
    u.device = device;
    const size_t bytes = data.size();
    if (hipHostMalloc(&u.host, bytes, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        return SA_ERR_NOMEM;
    }
    std::memcpy(u.host, data.data(), bytes);
    if (hipMalloc(&u.dev_base, bytes) != hipSuccess) {
        (void)hipGetLastError();
        u.dev_base = nullptr;
        u.free_all();
        return SA_ERR_NOMEM;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipEventCreateWithFlags(&u.done, hipEventDisableTiming) != hipSuccess ||
        hipMemcpyAsync(u.dev_base, u.host, bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipEventRecord(u.done, s) != hipSuccess) {
        (void)hipGetLastError();
        // Nothing may still read the staging buffer once we free it.
        (void)hipStreamSynchronize(s);
        u.free_all();
        return SA_ERR_HIP;
    }
    *up = u;
    return SA_OK;
}

class PlanCache {
  public:
    // Returns SA_OK and a device plan for (spec, T, bq) on the current device;
    // split_cap as build_plan's.  A plan built by this call is uploaded on
    // `stream`; a plan built earlier on another stream is waited for.
    int get(const sa_mask& m, int T, int bq, int64_t split_cap, void* stream, DevicePlan* out) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
        std::string key = sa::canonical_spec(m) + "|T=" + std::to_string(T) + "|bq=" +
                          std::to_string(bq) + "|bk=" + std::to_string(sa::kBK) +
                          "|split=" + std::to_string(split_cap) + "|dev=" + std::to_string(dev);
        std::lock_guard<std::mutex> lock(mu_);
        auto it = plans_.find(key);
        if (it != plans_.end()) {
            *out = it->second.plan;
            return it->second.up.order_after(stream);
        }
        HostPlan hp = sa::build_plan(MaskRule(m, T), bq, sa::kBK, split_cap);
        DevicePlan dp;
        dp.n_qb = hp.n_qb;
        dp.n_items = hp.n_items;
        dp.n_parts = hp.n_parts;
        dp.n_split = static_cast<int32_t>(hp.split_qb.size());
        size_t off = 0;
        auto section = [&](size_t bytes, size_t* where, size_t align = 16) {
            off = align_up(off, align);
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
        section(hp.blk_ptr.size() * 4, &dp.off_blk_ptr);
        section(hp.blk_iv.size() * 4, &dp.off_blk_iv);
        section(hp.item_qb.size() * 4, &dp.off_item_qb);
        section(hp.item_part.size() * 4, &dp.off_item_part);
        section(hp.split_qb.size() * 4, &dp.off_split_qb);
        section(hp.split_ptr.size() * 4, &dp.off_split_ptr);
        section(hp.item_rec.size() * 4, &dp.off_item_rec, sizeof(int32_t) * sa::kItemRec);
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
        put(dp.off_blk_ptr, hp.blk_ptr.data(), hp.blk_ptr.size() * 4);
        put(dp.off_blk_iv, hp.blk_iv.data(), hp.blk_iv.size() * 4);
        put(dp.off_item_qb, hp.item_qb.data(), hp.item_qb.size() * 4);
        put(dp.off_item_part, hp.item_part.data(), hp.item_part.size() * 4);
        put(dp.off_split_qb, hp.split_qb.data(), hp.split_qb.size() * 4);
        put(dp.off_split_ptr, hp.split_ptr.data(), hp.split_ptr.size() * 4);
        put(dp.off_item_rec, hp.item_rec.data(), hp.item_rec.size() * 4);
        Upload up;
        int rc = upload(host, stream, dev, &up);
        if (rc != SA_OK) return rc;
        dp.base = up.dev_base;
        plans_.emplace(key, Entry{dp, up});
        *out = dp;
        return SA_OK;
    }

    // The backward plan (key blocks -> query tiles) for (spec, T).
    int get_bwd(const sa_mask& m, int T, int bkb, int64_t split_cap, bool gather, void* stream,
                sa::BwdDevicePlan* out) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
        std::string key = sa::canonical_spec(m) + "|T=" + std::to_string(T) + "|bwd|bkb=" +
                          std::to_string(bkb) + "|split=" + std::to_string(split_cap) +
                          (gather ? "|gather" : "") + "|dev=" + std::to_string(dev);
        std::lock_guard<std::mutex> lock(mu_);
        auto it = bwd_.find(key);
        if (it != bwd_.end()) {
            *out = it->second.plan;
            return it->second.up.order_after(stream);
        }
        sa::BwdHostPlan hp = sa::build_bwd_plan(MaskRule(m, T), bkb, split_cap, gather);
        sa::BwdDevicePlan dp;
        dp.n_kb = hp.n_kb;
        dp.n_items = hp.n_items;
        dp.n_parts = hp.n_parts;
        dp.n_split = static_cast<int32_t>(hp.split_kb.size());
        dp.n_gkb = hp.n_gkb;
        dp.n_col = hp.n_col;
        size_t off = 0;
        auto section = [&](size_t bytes, size_t* where) {
            off = align_up(off, 16);
            *where = off;
            off += bytes;
        };
        section(hp.kb_order.size() * 4, &dp.off_order);
        section(hp.kb_ptr.size() * 4, &dp.off_ptr);
        section(hp.kb_runs.size() * 4, &dp.off_runs);
        section(hp.item_kb.size() * 4, &dp.off_item_kb);
        section(hp.item_part.size() * 4, &dp.off_item_part);
        section(hp.split_kb.size() * 4, &dp.off_split_kb);
        section(hp.split_ptr.size() * 4, &dp.off_split_ptr);
        dp.bytes = align_up(off, 16) + 16;
        std::vector<unsigned char> host(dp.bytes, 0);
        auto put = [&](size_t where, const void* src, size_t bytes) {
            if (bytes) std::memcpy(host.data() + where, src, bytes);
        };
        put(dp.off_order, hp.kb_order.data(), hp.kb_order.size() * 4);
        put(dp.off_ptr, hp.kb_ptr.data(), hp.kb_ptr.size() * 4);
        put(dp.off_runs, hp.kb_runs.data(), hp.kb_runs.size() * 4);
        put(dp.off_item_kb, hp.item_kb.data(), hp.item_kb.size() * 4);
        put(dp.off_item_part, hp.item_part.data(), hp.item_part.size() * 4);
        put(dp.off_split_kb, hp.split_kb.data(), hp.split_kb.size() * 4);
        put(dp.off_split_ptr, hp.split_ptr.data(), hp.split_ptr.size() * 4);
        Upload up;
        int rc = upload(host, stream, dev, &up);
        if (rc != SA_OK) return rc;
        dp.base = up.dev_base;
        bwd_.emplace(key, BwdEntry{dp, up});
        *out = dp;
        return SA_OK;
    }

    void release() {
        std::lock_guard<std::mutex> lock(mu_);
        int cur = 0;
        bool have_cur = hipGetDevice(&cur) == hipSuccess;
        for (auto& kv : plans_)
            if (hipSetDevice(kv.second.up.device) == hipSuccess) kv.second.up.free_all();
        for (auto& kv : bwd_)
            if (hipSetDevice(kv.second.up.device) == hipSuccess) kv.second.up.free_all();
        if (have_cur) (void)hipSetDevice(cur);
        plans_.clear();
        bwd_.clear();
    }

  private:
    struct Entry {
        DevicePlan plan;
        Upload up;
    };
    struct BwdEntry {
        sa::BwdDevicePlan plan;
        Upload up;
    };
    std::mutex mu_;
    std::unordered_map<std::string, Entry> plans_;
    std::unordered_map<std::string, BwdEntry> bwd_;
};

PlanCache& cache() {
    static PlanCache* c = new PlanCache();  // never destroyed: no teardown-order issues
    return *c;
}

// fp32 scratch (split partials, the backward's row dots, decode's key-split
// partials), one buffer per (device, stream).  hipStreamPerThread names a
// different stream in every host thread, so its buffers are also keyed by
// thread.  A buffer only grows; before the old one is freed, the one stream
// that uses it is synchronised (work queued on it may still read it).  The
// caller holds the entry's lock from get() until its launches are enqueued,
// so two host threads that share a stream cannot free a buffer under each
// other.
class Workspace {
  public:
    int get(size_t bytes, void* stream, float** out, std::unique_lock<std::mutex>* hold) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
        std::string key = std::to_string(dev) + "/" + std::to_string(reinterpret_cast<uintptr_t>(stream));
        if (static_cast<hipStream_t>(stream) == hipStreamPerThread) {
            std::ostringstream tid;
            tid << std::this_thread::get_id();
            key += "/" + tid.str();
        }
        Entry* e = nullptr;
        {
            std::lock_guard<std::mutex> lock(mu_);
            std::unique_ptr<Entry>& slot = bufs_[key];
            if (!slot) slot.reset(new Entry());
            e = slot.get();
        }
        std::unique_lock<std::mutex> lk(e->mu);
        e->device = dev;
        if (e->bytes < bytes) {
            if (e->base) {
                if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SA_ERR_HIP;
                (void)hipFree(e->base);
                e->base = nullptr;
                e->bytes = 0;
            }
            if (hipMalloc(&e->base, bytes) != hipSuccess) {
                (void)hipGetLastError();
                e->base = nullptr;
                return SA_ERR_NOMEM;
            }
            e->bytes = bytes;
        }
        *out = static_cast<float*>(e->base);
        *hold = std::move(lk);
        return SA_OK;
    }

    void release() {
        std::lock_guard<std::mutex> lock(mu_);
        int cur = 0;
        bool have_cur = hipGetDevice(&cur) == hipSuccess;
        for (auto& kv : bufs_) {
            std::lock_guard<std::mutex> lk(kv.second->mu);
            if (kv.second->base && hipSetDevice(kv.second->device) == hipSuccess)
                (void)hipFree(kv.second->base);
            kv.second->base = nullptr;
            kv.second->bytes = 0;
        }
        if (have_cur) (void)hipSetDevice(cur);
    }

  private:
    struct Entry {
        std::mutex mu;
        void* base = nullptr;
        size_t bytes = 0;
        int device = 0;
    };
    std::mutex mu_;
    std::unordered_map<std::string, std::unique_ptr<Entry>> bufs_;
};

Workspace& workspace() {
    static Workspace* w = new Workspace();
    return *w;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Compute units of one MI355X.
constexpr int64_t kCUs = 256;

// Query rows per tile of the forward for a call of BH sequences of T rows
// (T of one subsequence when a residue split runs `sub` of them).  A
// token-level bf16 d = 64 call whose 128-row blocks would not give every CU
// a workgroup runs 64-row blocks instead, four 16-query waves each: twice
// the workgroups, so that each CU holds two whose barriers are independent
// and one's waits are filled by the other's work (with one eight-wave
// workgroup per CU, both waves of a SIMD wait at the same barrier).
int fwd_query_block_bh(const sa_mask& m, int d, int dtype, int64_t BH, int64_t T, int sub) {
    const int bq = sa::fwd_query_block(m, d, dtype);
    if (bq == sa::kBQ && m.block == 0 && dtype == SA_DTYPE_BF16 && d == 64 && sub == 1 && BH >= 1 &&
        BH <= kCUs && BH * ((T + sa::kBQ - 1) / sa::kBQ) <= kCUs)
        return 64;
    return bq;
}

int forward(int dtype, const void* Q, const void* K, const void* V, void* O, int B, int H, int T,
            int d, const char* spec, void* stream, float* lse = nullptr) {
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
    if (lse) {
        const size_t lbytes = size_t(BH) * size_t(T) * sizeof(float);
        if (reinterpret_cast<uintptr_t>(lse) % 4) return SA_ERR_ALIGN;
        for (const void* p : {Q, K, V, static_cast<const void*>(O)})
            if (overlaps(lse, lbytes, p, bytes)) return SA_ERR_ALIAS;
    }
    sa_mask m;
    int rc = parse_for(spec, T, &m);
    if (rc != SA_OK) return rc;
    // Pure dilated windows run as `sub` interleaved plain windows.
    const int sub = sa::residue_split(m, T, d, dtype) ? m.dilation : 1;
    if (sub > 1) m.dilation = 1;
    const int Ts = T / sub;
    const int bq = fwd_query_block_bh(m, d, dtype, BH, Ts, sub);
    // Only the bf16 fast path runs split plans (and leaves them for the
    // merge kernel).
    const bool fast = sa::fwd_fast_path(dtype, d, bq, sub);
    DevicePlan dp;
    rc = cache().get(m, Ts, bq, fast && sub == 1 ? split_cap() : 0, stream, &dp);
    if (rc != SA_OK) return rc;
    // Partial slots grow with B*H: past kMaxSplitWorkspace the unsplit plan
    // runs instead (slower on blocks of global rows, same result).
    const size_t pbytes = size_t(BH) * size_t(dp.n_parts) * bq * (size_t(d) + 2) * sizeof(float);
    if (dp.n_parts > 0 && pbytes > kMaxSplitWorkspace) {
        rc = cache().get(m, Ts, bq, 0, stream, &dp);
        if (rc != SA_OK) return rc;
    }
    if (BH * sub * int64_t(dp.n_items) > INT32_MAX) return SA_ERR_SHAPE;
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
    a.blk = static_cast<int32_t>(m.block);
    a.blk_ptr = reinterpret_cast<const int32_t*>(base + dp.off_blk_ptr);
    a.blk_iv = reinterpret_cast<const int32_t*>(base + dp.off_blk_iv);
    a.lse = lse;
    a.bq = bq;
    a.item_qb = reinterpret_cast<const int32_t*>(base + dp.off_item_qb);
    a.item_part = dp.n_parts > 0 ? reinterpret_cast<const int32_t*>(base + dp.off_item_part) : nullptr;
    a.item_rec = reinterpret_cast<const int32_t*>(base + dp.off_item_rec);
    a.part = nullptr;
    a.n_parts = dp.n_parts;
    std::unique_lock<std::mutex> ws_hold;
    if (dp.n_parts > 0) {
        rc = workspace().get(pbytes, stream, &a.part, &ws_hold);
        if (rc != SA_OK) return rc;
    }
    const int64_t grid = int64_t(a.BH) * dp.n_items;
    if (!fast) return sub == 1 ? sa::launch_fwd(dtype, d, a, grid, stream) : SA_ERR_UNSUPPORTED;
    int lrc = sa::launch_fwd_fast(dtype, d, a, grid, stream);
    if (lrc != SA_OK || dp.n_parts == 0) return lrc;
    return sa::launch_fwd_merge(d, a, reinterpret_cast<const int32_t*>(base + dp.off_split_qb),
                                reinterpret_cast<const int32_t*>(base + dp.off_split_ptr), dp.n_split,
                                stream);
}

// Forward arguments for (spec, T, d): parse, plan lookup and the rule fields.
// Used by the backward, which runs on the token-level plan (no residue split).
int backward(int dtype, const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* lse, void* dQ, void* dK, void* dV, int B, int H, int T, int d,
             const char* spec, void* stream) {
    if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || !spec) return SA_ERR_NULL;
    if (B < 1 || H < 1 || T < 1 || T > SA_MAX_T) return SA_ERR_SHAPE;
    if (!supported_d(d)) return SA_ERR_UNSUPPORTED;
    const int64_t BH = int64_t(B) * H;
    const int64_t n_qb = (int64_t(T) + 64 - 1) / 64;    // the finer of the two plan shapes
    const int64_t n_kb = (int64_t(T) + 64 - 1) / 64;
    if (BH > INT32_MAX || BH * n_qb > INT32_MAX || BH * n_kb > INT32_MAX) return SA_ERR_SHAPE;
    for (const void* p : {Q, K, V, O, dO, static_cast<const void*>(dQ), static_cast<const void*>(dK),
                          static_cast<const void*>(dV)})
        if (reinterpret_cast<uintptr_t>(p) % 16) return SA_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(lse) % 4) return SA_ERR_ALIGN;
    const size_t esz = dtype == SA_DTYPE_BF16 ? 2 : 4;
    const size_t bytes = size_t(BH) * size_t(T) * size_t(d) * esz;
    const size_t lbytes = size_t(BH) * size_t(T) * sizeof(float);
    const void* outs[3] = {dQ, dK, dV};
    for (int x = 0; x < 3; ++x) {
        for (const void* p : {Q, K, V, O, dO})
            if (overlaps(outs[x], bytes, p, bytes)) return SA_ERR_ALIAS;
        if (overlaps(outs[x], bytes, lse, lbytes)) return SA_ERR_ALIAS;
        for (int y = x + 1; y < 3; ++y)
            if (overlaps(outs[x], bytes, outs[y], bytes)) return SA_ERR_ALIAS;
    }
    sa_mask m;
    int rc = parse_for(spec, T, &m);
    if (rc != SA_OK) return rc;
    // With the forward's 64-row plans (block mode, 64-key blocks, bf16 d=64)
    // the backward uses 64-query blocks and 64-key blocks as well.
    const int bq = sa::fwd_query_block(m, d, dtype);
    const int bkb = bq == 64 ? 64 : sa::kBKB;
    // The bf16 d = 64 / 128 kernels run split plans (heavy query blocks and
    // heavy key blocks as several items); the generic kernels do not.
    const bool dma = dtype == SA_DTYPE_BF16 && (d == 64 || d == 128);
    const int64_t cap = dma ? split_cap() : 0;
    DevicePlan dp;
    rc = cache().get(m, T, bq, cap, stream, &dp);
    if (rc != SA_OK) return rc;
    sa::BwdDevicePlan bp;
    rc = cache().get_bwd(m, T, bkb, cap, dma, stream, &bp);
    if (rc != SA_OK) return rc;
    // Workspace: row dots D_i, then dQ partials, then dK and dV partials
    // (each section 256-byte aligned).  Past kMaxSplitWorkspace of partials
    // the unsplit plans run instead.
    auto sized = [&](const DevicePlan& f, const sa::BwdDevicePlan& k, size_t* q_off, size_t* kv_off) {
        size_t off = align_up(lbytes, 256);
        *q_off = off;
        off += align_up(size_t(BH) * size_t(f.n_parts) * bq * size_t(d) * sizeof(float), 256);
        *kv_off = off;
        off += 2 * size_t(BH) * size_t(k.n_parts) * bkb * size_t(d) * sizeof(float);
        return off;
    };
    size_t q_off = 0, kv_off = 0;
    size_t wbytes = sized(dp, bp, &q_off, &kv_off);
    if (wbytes - align_up(lbytes, 256) > kMaxSplitWorkspace) {
        rc = cache().get(m, T, bq, 0, stream, &dp);
        if (rc == SA_OK) rc = cache().get_bwd(m, T, bkb, 0, dma, stream, &bp);
        if (rc != SA_OK) return rc;
        wbytes = sized(dp, bp, &q_off, &kv_off);
    }
    float* Dw = nullptr;
    std::unique_lock<std::mutex> ws_hold;
    rc = workspace().get(wbytes, stream, &Dw, &ws_hold);
    if (rc != SA_OK) return rc;

    sa::BwdArgs b;
    sa::FwdArgs& a = b.f;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = const_cast<void*>(O);
    a.T = T;
    a.BH = static_cast<int32_t>(BH);
    a.sub = 1;
    a.causal = m.causal;
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
    a.blk = static_cast<int32_t>(m.block);
    a.blk_ptr = reinterpret_cast<const int32_t*>(base + dp.off_blk_ptr);
    a.blk_iv = reinterpret_cast<const int32_t*>(base + dp.off_blk_iv);
    a.lse = nullptr;
    a.bq = bq;
    a.item_qb = reinterpret_cast<const int32_t*>(base + dp.off_item_qb);
    a.item_part = dp.n_parts > 0 ? reinterpret_cast<const int32_t*>(base + dp.off_item_part) : nullptr;
    a.item_rec = reinterpret_cast<const int32_t*>(base + dp.off_item_rec);
    a.part = nullptr;
    a.n_parts = dp.n_parts;
    b.dO = dO;
    b.lse = lse;
    b.dQ = dQ;
    b.dK = dK;
    b.dV = dV;
    b.Dw = Dw;
    b.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    auto* bb = static_cast<unsigned char*>(bp.base);
    b.kb_order = reinterpret_cast<const int32_t*>(bb + bp.off_order);
    b.kb_ptr = reinterpret_cast<const int32_t*>(bb + bp.off_ptr);
    b.kb_runs = reinterpret_cast<const int32_t*>(bb + bp.off_runs);
    b.n_kb = bp.n_kb;
    b.n_q_items = dp.n_items;
    b.n_kv_items = bp.n_items;
    auto* wb = reinterpret_cast<unsigned char*>(Dw);
    b.dq_part = dp.n_parts > 0 ? reinterpret_cast<float*>(wb + q_off) : nullptr;
    b.dq_split_qb = reinterpret_cast<const int32_t*>(base + dp.off_split_qb);
    b.dq_split_ptr = reinterpret_cast<const int32_t*>(base + dp.off_split_ptr);
    b.dq_n_split = dp.n_split;
    b.kv_item_kb = reinterpret_cast<const int32_t*>(bb + bp.off_item_kb);
    b.kv_item_part = bp.n_parts > 0 ? reinterpret_cast<const int32_t*>(bb + bp.off_item_part) : nullptr;
    b.kv_part = bp.n_parts > 0 ? reinterpret_cast<float*>(wb + kv_off) : nullptr;
    b.kv_split_kb = reinterpret_cast<const int32_t*>(bb + bp.off_split_kb);
    b.kv_split_ptr = reinterpret_cast<const int32_t*>(bb + bp.off_split_ptr);
    b.kv_n_split = bp.n_split;
    b.kv_n_parts = bp.n_parts;
    b.kv_n_gkb = bp.n_gkb;
    b.kv_n_col = bp.n_col;
    if (BH * int64_t(std::max(dp.n_items, bp.n_items)) > INT32_MAX) return SA_ERR_SHAPE;
    return sa::launch_bwd(dtype, d, b, stream);
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

// Decode: validation, key-split choice and launch.
int decode_mask(const char* spec, int n_new, sa_mask* m, int64_t* min_rows) {
    if (!spec) return SA_ERR_NULL;
    int rc = sa::parse_mask_spec(spec, m);
    if (rc != SA_OK) return rc;
    // Landmark and global keys would need a cache of their own.
    if (!m->causal || m->stride != 0 || m->n_global != 0) return SA_ERR_UNSUPPORTED;
    const int64_t r = sa::band_reach(*m);
    *min_rows = r < 0 ? 0 : r + n_new;
    return SA_OK;
}

// Validation and launch arguments of a decode call; *part_bytes receives the
// size of the key-split partials the launch needs (0 with one split).
int decode_prepare(const void* Q, const void* K, const void* V, void* O, const int32_t* pos,
                   int B, int H, int Hkv, int n_new, int C, int d, const char* spec,
                   sa::DecodeArgs* out, size_t* part_bytes) {
    if (!Q || !K || !V || !O || !pos || !spec) return SA_ERR_NULL;
    if (B < 1 || H < 1 || Hkv < 1 || n_new < 1 || C < 1 || C > SA_MAX_T || H % Hkv != 0 ||
        B > 65535)
        return SA_ERR_SHAPE;
    if (!supported_d(d)) return SA_ERR_UNSUPPORTED;
    for (const void* p : {Q, K, V, static_cast<const void*>(O)})
        if (reinterpret_cast<uintptr_t>(p) % 16) return SA_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(pos) % 4) return SA_ERR_ALIGN;
    sa_mask m;
    int64_t min_rows = 0;
    int rc = decode_mask(spec, n_new, &m, &min_rows);
    if (rc != SA_OK) return rc;
    if (min_rows > C) return SA_ERR_SHAPE;  // the cache cannot hold every allowed key
    const int G = H / Hkv;
    const int64_t nq_all = int64_t(G) * n_new;
    const int64_t nqchunks = nq_all <= 8 ? 1 : (nq_all + 7) / 8;
    if (int64_t(Hkv) * nqchunks > 65535) return SA_ERR_SHAPE;
    const size_t qbytes = size_t(B) * H * n_new * d * 2, kvbytes = size_t(B) * Hkv * C * d * 2;
    if (overlaps(O, qbytes, Q, qbytes) || overlaps(O, qbytes, K, kvbytes) ||
        overlaps(O, qbytes, V, kvbytes))
        return SA_ERR_ALIAS;

    sa::DecodeArgs& a = *out;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.pos = pos;
    a.part = nullptr;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.G = G;
    a.n_new = n_new;
    a.C = C;
    a.reach = sa::band_reach32(m);
    a.dil = m.dilation > 1 ? m.dilation : 1;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
    // Key splits: enough workgroups to fill the chip once -- 512, two per
    // CU, what the kernel keeps resident at d = 128 -- each with at least 256
    // keys. More splits only add rounds of workgroups, partial rows and the
    // merge: at 64 sequences x 8 KV heads (512 groups, no split) decode
    // streams 5.45 TB/s against 4.87 with four splits each.
    int64_t keys = min_rows > 0 ? std::min<int64_t>(C, min_rows) : C;
    if (n_new == 1 && a.dil > 1) keys = (keys + a.dil - 1) / a.dil;
    const int64_t groups = int64_t(B) * Hkv * nqchunks;
    int64_t nsplit = (512 + groups - 1) / groups;
    nsplit = std::max<int64_t>(1, std::min<int64_t>(nsplit, (keys + 255) / 256));
    a.nsplit = static_cast<int32_t>(nsplit);
    *part_bytes = a.nsplit > 1 ? size_t(B) * H * n_new * size_t(a.nsplit) * (d + 2) * sizeof(float) : 0;
    return SA_OK;
}

int decode(const void* Q, const void* K, const void* V, void* O, const int32_t* pos, int B,
           int H, int Hkv, int n_new, int C, int d, const char* spec, void* stream) {
    sa::DecodeArgs a;
    size_t bytes = 0;
    int rc = decode_prepare(Q, K, V, O, pos, B, H, Hkv, n_new, C, d, spec, &a, &bytes);
    if (rc != SA_OK) return rc;
    std::unique_lock<std::mutex> ws_hold;
    if (bytes > 0) {
        rc = workspace().get(bytes, stream, &a.part, &ws_hold);
        if (rc != SA_OK) return rc;
    }
    return sa::launch_decode(d, a, stream);
}

// The same decode with the partials in the library's static per-device
// scratch array: no allocation on any path.
int decode_noalloc(const void* Q, const void* K, const void* V, void* O, const int32_t* pos,
                   int B, int H, int Hkv, int n_new, int C, int d, const char* spec, void* stream) {
    sa::DecodeArgs a;
    size_t bytes = 0;
    int rc = decode_prepare(Q, K, V, O, pos, B, H, Hkv, n_new, C, d, spec, &a, &bytes);
    if (rc != SA_OK) return rc;
    if (bytes > 0) {
        rc = sa::decode_scratch(bytes, &a.part);
        if (rc != SA_OK) return rc;
    }
    return sa::launch_decode(d, a, stream);
}

SA_EXPORT int sparse_attn_fwd(const void* Q, const void* K, const void* V, void* O, int B, int H,
                              int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] { return forward(SA_DTYPE_BF16, Q, K, V, O, B, H, T, d, mask_spec, stream); });
}

SA_EXPORT int sparse_attn_fwd_f32(const void* Q, const void* K, const void* V, void* O, int B,
                                  int H, int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] { return forward(SA_DTYPE_F32, Q, K, V, O, B, H, T, d, mask_spec, stream); });
}

SA_EXPORT int sparse_attn_fwd_lse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                  int B, int H, int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] {
        if (!LSE) return SA_ERR_NULL;
        return forward(SA_DTYPE_BF16, Q, K, V, O, B, H, T, d, mask_spec, stream, LSE);
    });
}

SA_EXPORT int sparse_attn_fwd_lse_f32(const void* Q, const void* K, const void* V, void* O,
                                      float* LSE, int B, int H, int T, int d, const char* mask_spec,
                                      void* stream) {
    return guarded([&] {
        if (!LSE) return SA_ERR_NULL;
        return forward(SA_DTYPE_F32, Q, K, V, O, B, H, T, d, mask_spec, stream, LSE);
    });
}

SA_EXPORT int sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                              int H, int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] {
        return backward(SA_DTYPE_BF16, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, T, d, mask_spec,
                        stream);
    });
}

SA_EXPORT int sparse_attn_bwd_f32(const void* Q, const void* K, const void* V, const void* O,
                                  const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                  int B, int H, int T, int d, const char* mask_spec, void* stream) {
    return guarded([&] {
        return backward(SA_DTYPE_F32, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, T, d, mask_spec,
                        stream);
    });
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

SA_EXPORT int sparse_attn_tile_shape(const char* mask_spec, int d, int dtype, int* bq, int* bk) {
    return guarded([&] {
        if (!bq || !bk) return SA_ERR_NULL;
        if (!supported_d(d) || (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F32))
            return SA_ERR_UNSUPPORTED;
        sa_mask m;
        std::memset(&m, 0, sizeof(m));
        if (mask_spec) {
            int rc = sa::parse_mask_spec(mask_spec, &m);
            if (rc != SA_OK) return rc;
        }
        // The same choice the forward makes (a residue split keeps the
        // plain window's tiles).
        *bq = sa::fwd_query_block(m, d, dtype);
        *bk = sa::kBK;
        return SA_OK;
    });
}

namespace {

// The plan of a forward call of BH sequences (BH < 0: a call whose grid
// fills the chip, the plan sparse_attn_plan_info describes).
int plan_info_for(const char* mask_spec, int64_t BH, int T, int d, int dtype, sa_plan_info* info) {
    if (!info) return SA_ERR_NULL;
    int bq = 0, bk = 0;
    int rc = sparse_attn_tile_shape(mask_spec, d, dtype, &bq, &bk);
    if (rc != SA_OK) return rc;
    sa_mask m;
    rc = parse_for(mask_spec, T, &m);
    if (rc != SA_OK) return rc;
    MaskRule rule(m, T);
    // The plan the forward runs: for a residue split, one subsequence's.
    const int sub = sa::residue_split(m, T, d, dtype) ? m.dilation : 1;
    sa_mask mp = m;
    if (sub > 1) mp.dilation = 1;
    if (BH >= 0) bq = fwd_query_block_bh(mp, d, dtype, BH, T / sub, sub);
    MaskRule prule(mp, T / sub);
    HostPlan hp = sa::build_plan(prule, bq, bk,
                                 sub == 1 && sa::fwd_fast_path(dtype, d, bq, sub) ? split_cap() : 0);
    std::memset(info, 0, sizeof(*info));
    info->bq = bq;
    info->bk = bk;
    info->n_qb = hp.n_qb;
    info->n_kb = hp.n_kb;
    info->subsequences = sub;
    info->split_parts = hp.n_parts;
    info->inplace_tiles = hp.inplace_tiles * sub;
    info->masked_tiles = hp.masked_tiles * sub;
    info->gathered_tiles = hp.gathered_tiles * sub;
    info->gathered_keys = hp.gathered_keys * sub;
    info->executed_cells = int64_t(bq) * bk * (hp.inplace_tiles + hp.gathered_tiles) * sub;
    int64_t total = 0;
    for (int64_t i = 0; i < T; ++i) total += rule.allowed_in(i, 0, T);
    info->allowed_cells = total;
    return SA_OK;
}

}  // namespace

SA_EXPORT int sparse_attn_plan_info(const char* mask_spec, int T, int d, int dtype,
                                    sa_plan_info* info) {
    return guarded([&] { return plan_info_for(mask_spec, -1, T, d, dtype, info); });
}

SA_EXPORT int sparse_attn_plan_info_bh(const char* mask_spec, int B, int H, int T, int d, int dtype,
                                       sa_plan_info* info) {
    return guarded([&] {
        if (B < 1 || H < 1) return SA_ERR_SHAPE;
        return plan_info_for(mask_spec, int64_t(B) * H, T, d, dtype, info);
    });
}

SA_EXPORT const char* sparse_attn_strerror(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_SPEC: return "mask spec does not parse";
        case SA_ERR_RANGE: return "a global index is not below T, or phase is not below stride";
        case SA_ERR_SHAPE: return "bad shape (B, H or T < 1, T too large, or bad tile shape)";
        case SA_ERR_UNSUPPORTED: return "unsupported head dim or dtype (d must be 16, 32, 64 or 128)";
        case SA_ERR_NULL: return "a required pointer is NULL";
        case SA_ERR_ALIAS: return "output overlaps an input";
        case SA_ERR_HIP: return "HIP runtime or launch error";
        case SA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case SA_ERR_NOMEM: return "allocation failed";
        case SA_ERR_SCRATCH: return "the call needs more than the static decode scratch holds";
        default: return "unknown status";
    }
}

SA_EXPORT int sparse_attn_decode(const void* Q, const void* K_cache, const void* V_cache, void* O,
                                 const int32_t* pos, int B, int H, int Hkv, int n_new, int C,
                                 int d, const char* mask_spec, void* stream) {
    return guarded([&] {
        return decode(Q, K_cache, V_cache, O, pos, B, H, Hkv, n_new, C, d, mask_spec, stream);
    });
}

SA_EXPORT int sparse_attn_decode_noalloc(const void* Q, const void* K_cache, const void* V_cache,
                                         void* O, const int32_t* pos, int B, int H, int Hkv,
                                         int n_new, int C, int d, const char* mask_spec,
                                         void* stream) {
    return guarded([&] {
        return decode_noalloc(Q, K_cache, V_cache, O, pos, B, H, Hkv, n_new, C, d, mask_spec, stream);
    });
}

SA_EXPORT int sparse_attn_decode_cache_rows(const char* mask_spec, int n_new, int64_t* rows) {
    return guarded([&] {
        if (!rows) return SA_ERR_NULL;
        if (n_new < 1) return SA_ERR_SHAPE;
        sa_mask m;
        return decode_mask(mask_spec, n_new, &m, rows);
    });
}

SA_EXPORT void sparse_attn_release_cache(void) {
    try {
        cache().release();
        workspace().release();
    } catch (...) {
    }
}
