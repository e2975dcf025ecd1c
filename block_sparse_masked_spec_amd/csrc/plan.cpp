// Host planner: allowed-pair counts, exact tile classes and the execution
// plan of the fused kernel.
//
// Tile skipping follows "Sparse and sliding-window attention" (getnybble.com,
// section "Implementation": skip tiles outside the band) and "Attention
// variants" (sreshtalluri.github.io, section 4 "Use the library": skip fully
// masked blocks).  Strided and global columns would make every key tile
// non-empty, so the plan runs them apart: for each query block, the key
// tiles that meet the band (or every tile, if the block holds a global row)
// run in place, and the strided/global keys outside those tiles are
// gathered into dense tiles of their own.
#include <algorithm>
#include <numeric>

#include "internal.hpp"

namespace sa {

std::vector<int64_t> random_key_blocks(const sa_mask& m, int64_t nkb, int64_t qb) {
    std::vector<int64_t> out;
    if (m.n_random <= 0) return out;
    if (nkb <= m.n_random) {
        for (int64_t kb = 0; kb < nkb; ++kb) out.push_back(kb);
        return out;
    }
    // SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): add the golden gamma,
    // then two xor-shift-multiply rounds and a final xor-shift.
    uint64_t state = (uint64_t(m.seed) << 32) | uint64_t(qb);
    for (int64_t draw = 0; draw < 64 * int64_t(m.n_random) && int64_t(out.size()) < m.n_random;
         ++draw) {
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        const int64_t kb = int64_t((z >> 32) % uint64_t(nkb));
        if (std::find(out.begin(), out.end(), kb) == out.end()) out.push_back(kb);
    }
    return out;
}

MaskRule::MaskRule(const sa_mask& m, int64_t T)
    : m_(m), T_(T), g_(m.dilation > 1 ? m.dilation : 1), colpre_(T + 1, 0), rowpre_(T + 1, 0) {
    if (m.block > 0) {  // block mode: merged intervals of allowed key blocks per query block
        S_ = m.block;
        const int64_t nb = (T + S_ - 1) / S_;
        iv_ptr_.push_back(0);
        for (int64_t qb = 0; qb < nb; ++qb) {
            std::vector<std::pair<int64_t, int64_t>> iv;
            iv.emplace_back(std::max<int64_t>(0, qb - m.radius), std::min<int64_t>(nb, qb + m.radius + 1));
            for (int64_t kb : random_key_blocks(m, nb, qb)) iv.emplace_back(kb, kb + 1);
            std::sort(iv.begin(), iv.end());
            int64_t n0 = static_cast<int64_t>(ivals_.size());
            for (const auto& x : iv) {
                const int64_t n = static_cast<int64_t>(ivals_.size());
                if (n > n0 && x.first <= ivals_[n - 1])
                    ivals_[n - 1] = static_cast<int32_t>(std::max<int64_t>(ivals_[n - 1], x.second));
                else {
                    ivals_.push_back(static_cast<int32_t>(x.first));
                    ivals_.push_back(static_cast<int32_t>(x.second));
                }
            }
            iv_ptr_.push_back(static_cast<int32_t>(ivals_.size() / 2));
        }
    }
    std::vector<uint8_t> glob(T, 0);
    for (int k = 0; k < m.n_global; ++k)
        for (int64_t x = m.global_lo[k]; x < m.global_hi[k] && x < T; ++x) glob[x] = 1;
    for (int64_t j = 0; j < T; ++j) {
        bool strided = m.stride > 0 && (j % m.stride) == m.phase;
        colpre_[j + 1] = colpre_[j] + ((strided || glob[j]) ? 1 : 0);
        rowpre_[j + 1] = rowpre_[j] + (glob[j] ? 1 : 0);
    }
    if (g_ > 1) {
        colres_.assign(T, 0);
        for (int64_t j = 0; j < T; ++j)
            colres_[j] = (j >= g_ ? colres_[j - g_] : 0) + (col_key(j) ? 1 : 0);
    }
}

int64_t MaskRule::band_lo(int64_t i) const {
    if (S_ > 0) return 0;  // block mode: the plan scans every key tile
    const int64_t r = band_reach(m_);
    return r < 0 ? 0 : std::max<int64_t>(0, i - r);
}

int64_t MaskRule::band_hi(int64_t i) const {
    if (S_ > 0) return T_ - 1;
    if (m_.causal) return i;
    const int64_t r = band_reach(m_);
    return r < 0 ? T_ - 1 : std::min<int64_t>(T_ - 1, i + r);
}

int32_t MaskRule::band_back() const { return band_reach32(m_); }

int32_t MaskRule::band_fwd() const {
    if (m_.causal) return 0;
    return band_back();
}

int64_t MaskRule::on_grid(int64_t i, int64_t a, int64_t b) const {
    if (a >= b) return 0;
    const int64_t first = a + (((i - a) % g_) + g_) % g_;
    return first >= b ? 0 : (b - 1 - first) / g_ + 1;
}

int64_t MaskRule::col_keys_on_grid(int64_t i, int64_t a, int64_t b) const {
    if (g_ == 1) return col_keys_in(a, b);
    const int64_t n = on_grid(i, a, b);
    if (n == 0) return 0;
    const int64_t first = a + (((i - a) % g_) + g_) % g_, last = first + (n - 1) * g_;
    return colres_[last] - (first >= g_ ? colres_[first - g_] : 0);
}

int64_t MaskRule::allowed_in(int64_t i, int64_t a, int64_t b) const {
    a = std::max<int64_t>(a, 0);
    b = std::min<int64_t>(b, key_limit(i) + 1);  // causal cut
    if (a >= b) return 0;
    if (row_global(i)) return b - a;
    if (S_ > 0) {  // block mode: keys of the allowed key blocks, plus column keys elsewhere
        const int64_t qb = i / S_;
        int64_t n = col_keys_in(a, b);
        for (int32_t t = iv_ptr_[qb]; t < iv_ptr_[qb + 1]; ++t) {
            const int64_t lo = std::max(a, int64_t(ivals_[2 * t]) * S_);
            const int64_t hi = std::min(b, int64_t(ivals_[2 * t + 1]) * S_);
            if (lo < hi) n += (hi - lo) - col_keys_in(lo, hi);
        }
        return n;
    }
    int64_t lo = std::max(a, band_lo(i)), hi = std::min(b, band_hi(i) + 1);
    if (lo >= hi) return col_keys_in(a, b);
    return on_grid(i, lo, hi) + col_keys_in(a, b) - col_keys_on_grid(i, lo, hi);
}

int MaskRule::classify(int64_t q0, int64_t q1, int64_t k0, int64_t k1) const {
    q1 = std::min(q1, T_);
    k1 = std::min(k1, T_);
    if (q0 >= q1 || k0 >= k1) return SA_TILE_EMPTY;
    if (S_ > 0 && rows_global_in(q0, q1) == 0 && col_keys_in(k0, k1) == 0) {
        // Block mode: empty unless some query block of the rows allows a key
        // block that meets the tile.
        bool meets = false;
        for (int64_t qb = q0 / S_; qb <= (q1 - 1) / S_ && !meets; ++qb)
            for (int32_t t = iv_ptr_[qb]; t < iv_ptr_[qb + 1]; ++t)
                meets |= int64_t(ivals_[2 * t]) * S_ < k1 && k0 < int64_t(ivals_[2 * t + 1]) * S_;
        if (!meets) return SA_TILE_EMPTY;
    }
    if (S_ == 0 && rows_global_in(q0, q1) == 0) {
        // Band ends are monotone in i: the first row has the lowest upper
        // end, the last row the highest lower end.
        if (g_ == 1 && k0 >= band_lo(q1 - 1) && k1 - 1 <= band_hi(q0)) return SA_TILE_FULL;
        bool misses_band = k1 - 1 < band_lo(q0) || k0 > band_hi(q1 - 1);
        if (misses_band && col_keys_in(k0, std::min(k1, key_limit(q1 - 1) + 1)) == 0)
            return SA_TILE_EMPTY;
    }
    const int64_t cells = (q1 - q0) * (k1 - k0);
    int64_t allowed = 0;
    for (int64_t i = q0; i < q1; ++i) allowed += allowed_in(i, k0, k1);
    return allowed == 0 ? SA_TILE_EMPTY : (allowed == cells ? SA_TILE_FULL : SA_TILE_PARTIAL);
}

namespace {

// The tiles of one query block: in-place runs, then its gathered keys
// (segments [a0, a1) and [b0, b1) of colkeys, taken in that order).
struct BlockTiles {
    std::vector<int32_t> runs;  // pairs, as HostPlan::runs
    int32_t a0 = 0, a1 = 0, b0 = 0, b1 = 0;
    int64_t inplace = 0, gathered = 0;
    int64_t work() const { return inplace + gathered; }
};

// Emit tiles [t0, t1) of block `bt` (in-place tiles first, then gathered
// tiles of bk keys) as one work item's runs and gather segments.
void emit_item(const BlockTiles& bt, int64_t t0, int64_t t1, int32_t bk, HostPlan& p) {
    int64_t t = 0;  // tile index of the current run's first tile
    for (size_t r = 0; r < bt.runs.size(); r += 2) {
        const int32_t kb0 = bt.runs[r], end = bt.runs[r + 1];
        const int32_t kb1 = end & 0x7fffffff, flag = end & int32_t(0x80000000u);
        const int64_t lo = std::max<int64_t>(t0, t), hi = std::min<int64_t>(t1, t + (kb1 - kb0));
        if (lo < hi) {
            p.runs.push_back(static_cast<int32_t>(kb0 + (lo - t)));
            p.runs.push_back(static_cast<int32_t>(kb0 + (hi - t)) | flag);
        }
        t += kb1 - kb0;
    }
    p.run_ptr.push_back(static_cast<int32_t>(p.runs.size() / 2));
    // Gathered tiles [g0, g1) of the block, as a range of its key list.
    const int64_t na = bt.a1 - bt.a0, nk = na + (bt.b1 - bt.b0);
    const int64_t g0 = std::max<int64_t>(t0 - bt.inplace, 0), g1 = std::max<int64_t>(t1 - bt.inplace, 0);
    const int64_t s = std::min(g0 * bk, nk), e = std::min(g1 * bk, nk);
    p.gseg.push_back(static_cast<int32_t>(bt.a0 + std::min(s, na)));
    p.gseg.push_back(static_cast<int32_t>(bt.a0 + std::min(e, na)));
    p.gseg.push_back(static_cast<int32_t>(bt.b0 + std::max(s, na) - na));
    p.gseg.push_back(static_cast<int32_t>(bt.b0 + std::max(e, na) - na));
}

}  // namespace

HostPlan build_plan(const MaskRule& rule, int32_t bq, int32_t bk, int64_t split_cap) {
    HostPlan p;
    const int64_t T = rule.T();
    p.bq = bq;
    p.bk = bk;
    p.n_qb = static_cast<int32_t>((T + bq - 1) / bq);
    p.n_kb = static_cast<int32_t>((T + bk - 1) / bk);
    p.colbits.assign((T + 63) / 64, 0);
    p.rowbits.assign((T + 31) / 32, 0);
    for (int64_t j = 0; j < T; ++j) {
        if (rule.col_key(j)) {
            p.colkeys.push_back(static_cast<int32_t>(j));
            p.colbits[j >> 6] |= uint64_t(1) << (j & 63);
        }
        if (rule.row_global(j)) p.rowbits[j >> 5] |= uint32_t(1) << (j & 31);
    }
    p.blk_ptr = rule.iv_ptr();
    p.blk_iv = rule.ivals();
    std::vector<BlockTiles> blocks(p.n_qb);
    int64_t total_work = 0;
    for (int32_t qb = 0; qb < p.n_qb; ++qb) {
        BlockTiles& bt = blocks[qb];
        const int64_t q0 = int64_t(qb) * bq, q1 = std::min<int64_t>(T, q0 + bq);
        int64_t klo, khi;
        if (rule.rows_global_in(q0, q1) > 0) {
            klo = 0;
            khi = rule.key_limit(q1 - 1);
        } else {
            klo = rule.band_lo(q0);
            khi = rule.band_hi(q1 - 1);
        }
        const int64_t kb_lo = klo / bk, kb_hi = khi / bk + 1;
        bool open = false;
        for (int64_t kb = kb_lo; kb < kb_hi; ++kb) {
            const int cls = rule.classify(q0, q1, kb * bk, (kb + 1) * bk);
            if (cls == SA_TILE_EMPTY) {
                open = false;
                continue;
            }
            const bool need_mask = !(cls == SA_TILE_FULL && (kb + 1) * bk <= T);
            const int32_t flag = need_mask ? int32_t(0x80000000u) : 0;
            if (open && (bt.runs.back() & int32_t(0x80000000u)) == flag &&
                (bt.runs.back() & 0x7fffffff) == kb) {
                bt.runs.back() = int32_t(kb + 1) | flag;
            } else {
                bt.runs.push_back(static_cast<int32_t>(kb));
                bt.runs.push_back(int32_t(kb + 1) | flag);
                open = true;
            }
            ++bt.inplace;
            p.masked_tiles += need_mask ? 1 : 0;
        }
        // Gathered keys: strided/global keys outside [kb_lo*bk, kb_hi*bk)
        // that some row of the block may read.  Below the block's band every
        // such key precedes every row (causal holds); above it only bidir
        // rows read, and they read all of them.
        const int64_t limit = rule.key_limit(q1 - 1);
        auto first_at_or_after = [&](int64_t key) {
            return static_cast<int32_t>(
                std::lower_bound(p.colkeys.begin(), p.colkeys.end(), key) - p.colkeys.begin());
        };
        bt.a0 = 0;
        bt.a1 = first_at_or_after(kb_lo * bk);
        bt.b0 = first_at_or_after(kb_hi * bk);
        bt.b1 = std::max(bt.b0, first_at_or_after(limit + 1));
        const int64_t nkeys = int64_t(bt.a1 - bt.a0) + (bt.b1 - bt.b0);
        bt.gathered = (nkeys + bk - 1) / bk;
        p.inplace_tiles += bt.inplace;
        p.gathered_tiles += bt.gathered;
        p.gathered_keys += nkeys;
        total_work += bt.work();
    }
    // Work items.  A block whose tile count is far above the mean (a block
    // of global rows reads every key tile) would run alone long after the
    // rest: a split plan makes it ceil(work / cap) items over consecutive
    // tile ranges, each leaving an unnormalised partial result that a second
    // kernel merges.
    const int64_t mean = p.n_qb ? (total_work + p.n_qb - 1) / p.n_qb : 0;
    const int64_t cap = split_cap == kSplitAuto ? std::max<int64_t>(kSplitMinTiles, 2 * mean)
                        : split_cap > 0         ? split_cap
                                                : INT64_MAX;
    std::vector<int64_t> item_work;
    p.run_ptr.push_back(0);
    p.split_ptr.push_back(0);
    for (int32_t qb = 0; qb < p.n_qb; ++qb) {
        const BlockTiles& bt = blocks[qb];
        const int64_t w = bt.work();
        const int64_t parts = w > cap ? (w + cap - 1) / cap : 1;
        for (int64_t x = 0; x < parts; ++x) {
            const int64_t t0 = w * x / parts, t1 = w * (x + 1) / parts;
            emit_item(bt, t0, t1, bk, p);
            p.item_qb.push_back(qb);
            p.item_part.push_back(parts > 1 ? p.n_parts++ : -1);
            item_work.push_back(t1 - t0);
        }
        if (parts > 1) {
            p.split_qb.push_back(qb);
            p.split_ptr.push_back(p.n_parts);
        }
    }
    p.n_items = static_cast<int32_t>(p.item_qb.size());
    p.qb_order.resize(p.n_items);
    std::iota(p.qb_order.begin(), p.qb_order.end(), 0);
    std::stable_sort(p.qb_order.begin(), p.qb_order.end(),
                     [&](int32_t x, int32_t y) { return item_work[x] > item_work[y]; });
    p.item_rec.assign(size_t(p.n_items) * kItemRec, 0);
    for (int32_t w = 0; w < p.n_items; ++w) {
        const int32_t it = p.qb_order[w];
        int32_t* r = p.item_rec.data() + size_t(w) * kItemRec;
        r[REC_QB] = p.item_qb[it];
        r[REC_PART] = p.item_part[it];
        r[REC_RUN_BEGIN] = p.run_ptr[it];
        r[REC_RUN_END] = p.run_ptr[it + 1];
        for (int x = 0; x < 4; ++x) r[REC_GA0 + x] = p.gseg[4 * size_t(it) + x];
        if (r[REC_RUN_BEGIN] < r[REC_RUN_END]) {
            r[REC_FIRST_KB] = p.runs[2 * size_t(r[REC_RUN_BEGIN])];
            r[REC_FIRST_END] = p.runs[2 * size_t(r[REC_RUN_BEGIN]) + 1];
        }
    }
    return p;
}

BwdHostPlan build_bwd_plan(const MaskRule& rule, int32_t bkb, int64_t split_cap, bool gather_cols) {
    BwdHostPlan p;
    const int64_t T = rule.T();
    p.n_kb = static_cast<int32_t>((T + bkb - 1) / bkb);
    p.n_qt = static_cast<int32_t>((T + kBQB - 1) / kBQB);
    const bool any_global_row = rule.rows_global_in(0, T) > 0;
    const int64_t back = rule.band_back(), fwd = rule.band_fwd();
    // A column key is allowed for every row its causal limit lets read it,
    // so in the band blocks it would make every query tile live.  With
    // gather_cols the column keys run as dense blocks of their own (every
    // query tile from the first that may read them), and the band blocks
    // count and execute only their other keys.
    std::vector<int32_t> colkeys;
    if (gather_cols)
        for (int64_t j = 0; j < T; ++j)
            if (rule.col_key(j)) colkeys.push_back(static_cast<int32_t>(j));
    p.n_col = static_cast<int32_t>(colkeys.size());
    p.n_gkb = static_cast<int32_t>((colkeys.size() + bkb - 1) / bkb);
    std::vector<std::vector<int32_t>> block_runs(p.n_kb + p.n_gkb);
    std::vector<int64_t> work(p.n_kb + p.n_gkb, 0);
    for (int32_t kb = 0; kb < p.n_kb; ++kb) {
        std::vector<int32_t>& runs = block_runs[kb];
        const int64_t k0 = int64_t(kb) * bkb, k1 = std::min<int64_t>(T, k0 + bkb);
        // Query tiles that can hold allowed pairs: every tile when some row is
        // global, the block has column keys (not gathered) or in block mode;
        // else the rows whose band meets the block.
        int64_t qlo = 0, qhi = T - 1;
        if (!any_global_row && (gather_cols || rule.col_keys_in(k0, k1) == 0) && rule.block() == 0) {
            qlo = fwd >= T ? 0 : std::max<int64_t>(0, k0 - fwd);
            qhi = back >= T ? T - 1 : std::min<int64_t>(T - 1, k1 - 1 + back);
            if (rule.causal()) qlo = std::max(qlo, k0);
        }
        bool open = false;
        int64_t tiles = 0;
        for (int64_t qt = qlo / kBQB; qt <= qhi / kBQB && qt < p.n_qt; ++qt) {
            const int64_t q0 = qt * kBQB, q1 = std::min<int64_t>(T, q0 + kBQB);
            int cls;
            if (gather_cols && rule.col_keys_in(k0, k1) > 0) {  // count the block's other keys
                int64_t n = 0;
                for (int64_t i = q0; i < q1; ++i) n += rule.allowed_noncol_in(i, k0, k1);
                cls = n == 0 ? SA_TILE_EMPTY : (n == (q1 - q0) * (k1 - k0) ? SA_TILE_FULL : SA_TILE_PARTIAL);
            } else {
                cls = rule.classify(q0, q1, k0, k1);
            }
            if (cls == SA_TILE_EMPTY) {
                open = false;
                continue;
            }
            const bool need_mask = !(cls == SA_TILE_FULL && q0 + kBQB <= T && k0 + bkb <= T);
            const int32_t flag = need_mask ? int32_t(0x80000000u) : 0;
            if (open && (runs.back() & int32_t(0x80000000u)) == flag && (runs.back() & 0x7fffffff) == qt) {
                runs.back() = int32_t(qt + 1) | flag;
            } else {
                runs.push_back(static_cast<int32_t>(qt));
                runs.push_back(int32_t(qt + 1) | flag);
                open = true;
            }
            ++tiles;
            p.masked_tiles += need_mask ? 1 : 0;
        }
        p.tiles += tiles;
        work[kb] = tiles;
    }
    // Gathered blocks: every query tile from the first row that may read the
    // block's first key, each evaluating the rule (causal limit, ragged ends).
    for (int32_t c = 0; c < p.n_gkb; ++c) {
        const int64_t first = rule.causal() ? colkeys[size_t(c) * bkb] / kBQB : 0;
        if (first < p.n_qt) {
            block_runs[p.n_kb + c] = {static_cast<int32_t>(first), p.n_qt | int32_t(0x80000000u)};
            work[p.n_kb + c] = p.n_qt - first;
            p.tiles += p.n_qt - first;
            p.masked_tiles += p.n_qt - first;
        }
    }
    // Work items, as in build_plan: key blocks far above the mean become
    // ceil(tiles / cap) items over consecutive ranges of their query tiles.
    const int32_t n_blocks = p.n_kb + p.n_gkb;
    const int64_t mean = n_blocks ? (p.tiles + n_blocks - 1) / n_blocks : 0;
    const int64_t cap = split_cap == kSplitAuto ? std::max<int64_t>(kSplitMinTiles, 2 * mean)
                        : split_cap > 0         ? split_cap
                                                : INT64_MAX;
    std::vector<int64_t> item_work;
    p.kb_ptr.push_back(0);
    p.split_ptr.push_back(0);
    for (int32_t kb = 0; kb < n_blocks; ++kb) {
        const std::vector<int32_t>& runs = block_runs[kb];
        const int64_t w = work[kb];
        const int64_t parts = w > cap ? (w + cap - 1) / cap : 1;
        for (int64_t x = 0; x < parts; ++x) {
            const int64_t t0 = w * x / parts, t1 = w * (x + 1) / parts;
            int64_t t = 0;
            for (size_t r = 0; r < runs.size(); r += 2) {
                const int32_t q0 = runs[r], end = runs[r + 1];
                const int32_t q1 = end & 0x7fffffff, flag = end & int32_t(0x80000000u);
                const int64_t lo = std::max(t0, t), hi = std::min(t1, t + (q1 - q0));
                if (lo < hi) {
                    p.kb_runs.push_back(static_cast<int32_t>(q0 + (lo - t)));
                    p.kb_runs.push_back(static_cast<int32_t>(q0 + (hi - t)) | flag);
                }
                t += q1 - q0;
            }
            p.kb_ptr.push_back(static_cast<int32_t>(p.kb_runs.size() / 2));
            p.item_kb.push_back(kb);
            p.item_part.push_back(parts > 1 ? p.n_parts++ : -1);
            item_work.push_back(t1 - t0);
        }
        if (parts > 1) {
            p.split_kb.push_back(kb);
            p.split_ptr.push_back(p.n_parts);
        }
    }
    p.n_items = static_cast<int32_t>(p.item_kb.size());
    p.kb_order.resize(p.n_items);
    std::iota(p.kb_order.begin(), p.kb_order.end(), 0);
    std::stable_sort(p.kb_order.begin(), p.kb_order.end(),
                     [&](int32_t x, int32_t y) { return item_work[x] > item_work[y]; });
    return p;
}

}  // namespace sa
