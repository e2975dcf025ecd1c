// Host-side check of the forward plan's work items (built with g++ by
// tests/test_plan_items.py; no GPU).  For random mask specs, lengths, tile
// heights and split caps it builds the plan twice -- one item per query
// block, and split -- and checks that the split items of each block, taken in
// order, hold exactly the block's in-place tiles (with their mask flags) and
// its gathered key list, that gathered cuts fall on whole tiles, that the
// partial slots and the merge lists agree, and that the item order is a
// permutation, heaviest first; the backward plan's key-block items the same
// way.  Prints "ok <cases>" and exits 0, or prints
// the first mismatch and exits 1.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../block_sparse_masked_spec_amd/csrc/internal.hpp"

namespace {

struct Lcg {
    uint64_t s;
    uint32_t next() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return uint32_t(s >> 33);
    }
    int below(int n) { return int(next() % uint32_t(n)); }
};

std::string random_spec(Lcg& r, int T) {
    std::string s;
    const int mode = r.below(3);
    if (mode == 2) {
        const int blk = r.below(2) ? 64 : 32 * (1 + r.below(4));
        s = "blocks;block=" + std::to_string(blk) + ";radius=" + std::to_string(r.below(3)) +
            ";random=" + std::to_string(r.below(4)) + ";seed=" + std::to_string(r.below(100));
    } else if (mode == 1) {
        s = "bidir";
        if (r.below(4)) s += ";radius=" + std::to_string(r.below(300));
    } else {
        s = "causal;window=" + std::to_string(r.below(5) ? 1 + r.below(400) : 0);
        if (r.below(4) == 0) s += ";dilation=" + std::to_string(1 + r.below(3));
    }
    if (r.below(2)) {
        const int st = 2 + r.below(40);
        s += ";stride=" + std::to_string(st) + ";phase=" + std::to_string(r.below(st));
    }
    const int ng = r.below(3);
    if (ng) {
        s += ";global=";
        for (int k = 0; k < ng; ++k) {
            const int a = r.below(T), b = a + 1 + r.below(std::max(1, T / 8));
            s += (k ? "," : "") + std::to_string(a) + ":" + std::to_string(std::min(b, T));
        }
    }
    return s;
}

// The tiles of item `it` (or block `it` of an unsplit plan): in-place
// (kb | flag) words, then its gathered key indices into colkeys.
void expand(const sa::HostPlan& p, int it, std::vector<int32_t>& inplace, std::vector<int32_t>& keys) {
    for (int r = p.run_ptr[it]; r < p.run_ptr[it + 1]; ++r) {
        const int32_t kb0 = p.runs[2 * r], end = p.runs[2 * r + 1];
        const int32_t flag = end & int32_t(0x80000000u);
        for (int32_t kb = kb0; kb < (end & 0x7fffffff); ++kb) inplace.push_back(kb | flag);
    }
    const int32_t* g = &p.gseg[4 * size_t(it)];
    for (int32_t x = g[0]; x < g[1]; ++x) keys.push_back(x);
    for (int32_t x = g[2]; x < g[3]; ++x) keys.push_back(x);
}

int fail(const std::string& what, const std::string& spec, int T, int bq, int64_t cap) {
    std::printf("mismatch: %s (spec %s, T=%d, bq=%d, cap=%lld)\n", what.c_str(), spec.c_str(), T, bq,
                static_cast<long long>(cap));
    return 1;
}

int check(const std::string& spec, int T, int bq, int64_t cap) {
    sa_mask m;
    if (sa::parse_mask_spec(spec.c_str(), &m) != SA_OK) return fail("spec does not parse", spec, T, bq, cap);
    const sa::MaskRule rule(m, T);
    const sa::HostPlan one = sa::build_plan(rule, bq, sa::kBK, 0);
    const sa::HostPlan sp = sa::build_plan(rule, bq, sa::kBK, cap);
    if (one.n_items != one.n_qb || one.n_parts != 0) return fail("unsplit plan has split items", spec, T, bq, cap);
    if (sp.n_qb != one.n_qb || sp.inplace_tiles != one.inplace_tiles || sp.gathered_tiles != one.gathered_tiles)
        return fail("totals differ", spec, T, bq, cap);
    // The cap in force: automatic caps follow the mean block.
    int64_t total = 0;
    for (int qb = 0; qb < one.n_qb; ++qb) {
        std::vector<int32_t> in, keys;
        expand(one, qb, in, keys);
        total += int64_t(in.size()) + int64_t((keys.size() + sa::kBK - 1) / sa::kBK);
    }
    const int64_t mean = (total + one.n_qb - 1) / one.n_qb;
    const int64_t eff = cap == sa::kSplitAuto ? std::max<int64_t>(sa::kSplitMinTiles, 2 * mean) : cap;
    // Items of each block, in index order.
    int it = 0, parts = 0;
    std::vector<int64_t> work(sp.n_items, 0);
    for (int qb = 0; qb < one.n_qb; ++qb) {
        std::vector<int32_t> want_in, want_keys, got_in, got_keys;
        expand(one, qb, want_in, want_keys);
        const int first = it;
        while (it < sp.n_items && sp.item_qb[it] == qb) {
            const size_t before = got_keys.size();
            const size_t in_before = got_in.size();
            expand(sp, it, got_in, got_keys);
            const size_t nk = got_keys.size() - before;
            work[it] = int64_t(got_in.size() - in_before) + int64_t((nk + sa::kBK - 1) / sa::kBK);
            if (work[it] < 1) return fail("empty item", spec, T, bq, cap);
            // a cut inside the gathered list must fall on a whole tile
            const bool more_keys_follow = got_keys.size() < want_keys.size();
            if (more_keys_follow && nk % sa::kBK) return fail("gathered cut inside a tile", spec, T, bq, cap);
            ++it;
        }
        const int n = it - first;
        if (n == 0) return fail("block without items", spec, T, bq, cap);
        if (got_in != want_in) return fail("in-place tiles differ", spec, T, bq, cap);
        if (got_keys != want_keys) return fail("gathered keys differ", spec, T, bq, cap);
        const int64_t w = int64_t(want_in.size()) + int64_t((want_keys.size() + sa::kBK - 1) / sa::kBK);
        const int64_t expect = w > eff ? (w + eff - 1) / eff : 1;
        if (n != expect) return fail("item count", spec, T, bq, cap);
        for (int x = first; x < it; ++x) {
            const int32_t want = n > 1 ? parts + (x - first) : -1;
            if (sp.item_part[x] != want) return fail("partial slot", spec, T, bq, cap);
        }
        if (n > 1) {
            size_t s = 0;
            while (s < sp.split_qb.size() && sp.split_qb[s] != qb) ++s;
            if (s == sp.split_qb.size() || sp.split_ptr[s] != parts || sp.split_ptr[s + 1] != parts + n)
                return fail("merge list", spec, T, bq, cap);
            parts += n;
        }
    }
    if (it != sp.n_items || parts != sp.n_parts) return fail("item or part count", spec, T, bq, cap);
    std::vector<char> seen(sp.n_items, 0);
    for (int x = 0; x < sp.n_items; ++x) {
        const int32_t o = sp.qb_order[x];
        if (o < 0 || o >= sp.n_items || seen[o]) return fail("order is not a permutation", spec, T, bq, cap);
        seen[o] = 1;
        if (x > 0 && work[sp.qb_order[x - 1]] < work[o]) return fail("order not heaviest first", spec, T, bq, cap);
        // The fast kernel reads item x of the launch from its record alone.
        if (sp.item_rec.size() != size_t(sp.n_items) * sa::kItemRec) return fail("record count", spec, T, bq, cap);
        const int32_t* r = sp.item_rec.data() + size_t(x) * sa::kItemRec;
        bool ok = r[sa::REC_QB] == sp.item_qb[o] && r[sa::REC_PART] == sp.item_part[o] &&
                  r[sa::REC_RUN_BEGIN] == sp.run_ptr[o] && r[sa::REC_RUN_END] == sp.run_ptr[o + 1];
        for (int g = 0; g < 4; ++g) ok = ok && r[sa::REC_GA0 + g] == sp.gseg[4 * size_t(o) + g];
        if (sp.run_ptr[o] < sp.run_ptr[o + 1])
            ok = ok && r[sa::REC_FIRST_KB] == sp.runs[2 * size_t(sp.run_ptr[o])] &&
                 r[sa::REC_FIRST_END] == sp.runs[2 * size_t(sp.run_ptr[o]) + 1];
        else
            ok = ok && r[sa::REC_FIRST_KB] == 0 && r[sa::REC_FIRST_END] == 0;
        if (!ok) return fail("item record differs from the plan arrays", spec, T, bq, cap);
    }
    return 0;
}

// The backward plan: the items of each key block, in order, hold exactly
// the block's query-tile runs (with their mask flags).
int check_bwd(const std::string& spec, int T, int bkb, int64_t cap, bool gather) {
    sa_mask m;
    if (sa::parse_mask_spec(spec.c_str(), &m) != SA_OK) return fail("spec does not parse", spec, T, bkb, cap);
    const sa::MaskRule rule(m, T);
    const sa::BwdHostPlan one = sa::build_bwd_plan(rule, bkb, 0, gather);
    const sa::BwdHostPlan sp = sa::build_bwd_plan(rule, bkb, cap, gather);
    if (one.n_items != one.n_kb + one.n_gkb || one.n_parts != 0)
        return fail("bwd: unsplit plan has split items", spec, T, bkb, cap);
    // Every allowed pair (i, j) lies in a listed tile: query tile i / 64 of
    // key block j / bkb, or, for a gathered column key, of its gathered block.
    if (T <= 300) {
        std::vector<std::vector<char>> live(one.n_kb + one.n_gkb, std::vector<char>(one.n_qt, 0));
        for (int blk = 0; blk < one.n_kb + one.n_gkb; ++blk)
            for (int r = one.kb_ptr[blk]; r < one.kb_ptr[blk + 1]; ++r)
                for (int32_t q = one.kb_runs[2 * r]; q < (one.kb_runs[2 * r + 1] & 0x7fffffff); ++q) live[blk][q] = 1;
        int ci = 0;
        for (int64_t j = 0; j < T; ++j) {
            const bool gathered = gather && rule.col_key(j);
            const int blk = gathered ? one.n_kb + ci / bkb : int(j / bkb);
            for (int64_t i = 0; i < T; ++i)
                if (rule.allowed_in(i, j, j + 1) && !live[blk][i / sa::kBQB])
                    return fail("bwd: allowed pair outside the plan", spec, T, bkb, cap);
            ci += gathered ? 1 : 0;
        }
        if (ci != one.n_col) return fail("bwd: column key count", spec, T, bkb, cap);
    }
    if (sp.tiles != one.tiles || sp.masked_tiles != one.masked_tiles) return fail("bwd: totals differ", spec, T, bkb, cap);
    auto tiles_of = [](const sa::BwdHostPlan& p, int it) {
        std::vector<int32_t> out;
        for (int r = p.kb_ptr[it]; r < p.kb_ptr[it + 1]; ++r) {
            const int32_t q0 = p.kb_runs[2 * r], end = p.kb_runs[2 * r + 1];
            for (int32_t q = q0; q < (end & 0x7fffffff); ++q) out.push_back(q | (end & int32_t(0x80000000u)));
        }
        return out;
    };
    const int nb = one.n_kb + one.n_gkb;
    const int64_t mean = nb ? (one.tiles + nb - 1) / nb : 0;
    const int64_t eff = cap == sa::kSplitAuto ? std::max<int64_t>(sa::kSplitMinTiles, 2 * mean) : cap;
    int it = 0, parts = 0;
    std::vector<int64_t> work(sp.n_items, 0);
    for (int kb = 0; kb < nb; ++kb) {
        const std::vector<int32_t> want = tiles_of(one, kb);
        std::vector<int32_t> got;
        const int first = it;
        while (it < sp.n_items && sp.item_kb[it] == kb) {
            const std::vector<int32_t> t = tiles_of(sp, it);
            work[it] = int64_t(t.size());
            if (t.empty() && !want.empty()) return fail("bwd: empty item", spec, T, bkb, cap);
            got.insert(got.end(), t.begin(), t.end());
            ++it;
        }
        const int n = it - first;
        if (n == 0) return fail("bwd: block without items", spec, T, bkb, cap);
        if (got != want) return fail("bwd: query tiles differ", spec, T, bkb, cap);
        const int64_t w = int64_t(want.size());
        if (n != (w > eff ? (w + eff - 1) / eff : 1)) return fail("bwd: item count", spec, T, bkb, cap);
        for (int x = first; x < it; ++x)
            if (sp.item_part[x] != (n > 1 ? parts + (x - first) : -1)) return fail("bwd: partial slot", spec, T, bkb, cap);
        if (n > 1) {
            size_t s = 0;
            while (s < sp.split_kb.size() && sp.split_kb[s] != kb) ++s;
            if (s == sp.split_kb.size() || sp.split_ptr[s] != parts || sp.split_ptr[s + 1] != parts + n)
                return fail("bwd: merge list", spec, T, bkb, cap);
            parts += n;
        }
    }
    if (it != sp.n_items || parts != sp.n_parts) return fail("bwd: item or part count", spec, T, bkb, cap);
    std::vector<char> seen(sp.n_items, 0);
    for (int x = 0; x < sp.n_items; ++x) {
        const int32_t o = sp.kb_order[x];
        if (o < 0 || o >= sp.n_items || seen[o]) return fail("bwd: order is not a permutation", spec, T, bkb, cap);
        seen[o] = 1;
        if (x > 0 && work[sp.kb_order[x - 1]] < work[o]) return fail("bwd: order not heaviest first", spec, T, bkb, cap);
    }
    return 0;
}

// Parser robustness: random strings over the grammar's alphabet and single-
// character mutations of valid specs must parse to SA_OK, SA_ERR_SPEC or
// SA_ERR_RANGE (never crash or read out of bounds -- the sanitizer build of
// this program checks that); a spec that parses must survive the round trip
// through its canonical text unchanged.
int fuzz_parser(Lcg& r, int n) {
    static const char alphabet[] = "causlbidrwnophetgkzfm=;:,0123456789 -x";
    const char* seeds[] = {"causal;window=4096", "bidir;radius=256;stride=16;phase=0;global=0:128",
                           "blocks;block=64;radius=1;random=3;seed=0;global=0:128",
                           "causal;window=9;dilation=2;stride=5;phase=4;global=3,7:9"};
    for (int c = 0; c < n; ++c) {
        std::string s;
        if (c % 2) {
            const int len = r.below(60);
            for (int k = 0; k < len; ++k) s += alphabet[r.below(int(sizeof(alphabet)) - 1)];
        } else {
            s = seeds[r.below(4)];
            const int edits = 1 + r.below(3);
            for (int e = 0; e < edits && !s.empty(); ++e) {
                const int at = r.below(int(s.size()));
                switch (r.below(3)) {
                    case 0: s[at] = alphabet[r.below(int(sizeof(alphabet)) - 1)]; break;
                    case 1: s.erase(at, 1); break;
                    default: s.insert(s.begin() + at, alphabet[r.below(int(sizeof(alphabet)) - 1)]);
                }
            }
        }
        sa_mask m;
        const int rc = sa::parse_mask_spec(s.c_str(), &m);
        if (rc != SA_OK && rc != SA_ERR_SPEC && rc != SA_ERR_RANGE) {
            std::printf("parser: status %d for \"%s\"\n", rc, s.c_str());
            return 1;
        }
        if (rc != SA_OK) continue;
        sa_mask back;
        const std::string canon = sa::canonical_spec(m);
        if (sa::parse_mask_spec(canon.c_str(), &back) != SA_OK || sa::canonical_spec(back) != canon) {
            std::printf("parser: round trip of \"%s\" via \"%s\"\n", s.c_str(), canon.c_str());
            return 1;
        }
    }
    return 0;
}

}  // namespace

int main() {
    Lcg r{12345};
    int cases = 0;
    // fixed cases: the Longformer 16K layer and a global block mid-sequence
    const struct {
        const char* spec;
        int T, bq;
    } fixed[] = {{"bidir;radius=256;stride=16;phase=0;global=0:128", 16384, 128},
                 {"causal;window=64;global=3000:3050", 5000, 128},
                 {"blocks;block=64;radius=1;random=3;seed=0;global=0:128", 4096, 64}};
    for (const auto& f : fixed)
        for (int64_t cap : {int64_t(sa::kSplitAuto), int64_t(1), int64_t(7), int64_t(60)}) {
            if (check(f.spec, f.T, f.bq, cap)) return 1;
            if (check_bwd(f.spec, f.T, f.bq == 64 ? 64 : 128, cap, false)) return 1;
            if (check_bwd(f.spec, f.T, f.bq == 64 ? 64 : 128, cap, true)) return 1;
            cases += 3;
        }
    for (int n = 0; n < 400; ++n) {
        const int T = 1 + r.below(n < 200 ? 700 : 3000);
        const std::string spec = random_spec(r, T);
        const int bq = r.below(2) ? 128 : 64;
        const int64_t caps[] = {sa::kSplitAuto, 1, 2, 3, 5, 16};
        const int64_t cap = caps[r.below(6)];
        if (check(spec, T, bq, cap)) return 1;
        if (check_bwd(spec, T, bq == 64 ? 64 : 128, cap, false)) return 1;
        if (check_bwd(spec, T, bq == 64 ? 64 : 128, cap, true)) return 1;
        cases += 3;
    }
    if (fuzz_parser(r, 20000)) return 1;
    std::printf("ok %d\n", cases);
    return 0;
}
