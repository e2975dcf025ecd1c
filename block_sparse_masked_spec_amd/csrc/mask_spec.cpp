// Mask-spec parser: spec text -> sa_mask.
//
// The spec names the rules of "Attention variants" (sreshtalluri.github.io),
// section 1 "Intuition" and section 4 "Build it from scratch": a causal or
// bidirectional base, a local window (causal, counting the query) or radius
// (bidirectional), strided landmark columns with a phase, and global tokens;
// plus a dilation of the local window (section 6, the dilated-mask exercise),
// and a block mode for BigBird ("Sparse and sliding-window attention",
// section "Block-sparse attention: BigBird").
// The grammar is documented in include/sparse_attn.h.
#include "internal.hpp"

#include <algorithm>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

namespace sa {
namespace {

class Cursor {
  public:
    explicit Cursor(std::string s) : s_(std::move(s)) {}
    bool done() const { return pos_ >= s_.size(); }
    char peek() const { return done() ? '\0' : s_[pos_]; }
    bool eat(char c) {
        if (peek() != c) return false;
        ++pos_;
        return true;
    }
    bool word(std::string* out) {
        size_t b = pos_;
        while (!done() && ((s_[pos_] >= 'a' && s_[pos_] <= 'z') || s_[pos_] == '_')) ++pos_;
        *out = s_.substr(b, pos_ - b);
        return pos_ > b;
    }
    // Non-negative decimal below 2^31.
    bool number(int64_t* out) {
        size_t b = pos_;
        int64_t v = 0;
        while (!done() && s_[pos_] >= '0' && s_[pos_] <= '9') {
            v = v * 10 + (s_[pos_] - '0');
            if (v > INT32_MAX) return false;
            ++pos_;
        }
        *out = v;
        return pos_ > b;
    }

  private:
    std::string s_;
    size_t pos_ = 0;
};

std::string strip_spaces(const char* text) {
    std::string s;
    for (const char* p = text; *p; ++p)
        if (*p != ' ' && *p != '\t' && *p != '\n' && *p != '\r') s.push_back(*p);
    return s;
}

bool parse_globals(Cursor& c, std::vector<std::pair<int64_t, int64_t>>* ranges) {
    do {
        int64_t a = 0, b = 0;
        if (!c.number(&a)) return false;
        if (c.eat(':')) {
            if (!c.number(&b) || b <= a) return false;
        } else {
            b = a + 1;
        }
        ranges->emplace_back(a, b);
    } while (c.eat(','));
    return true;
}

}  // namespace

int parse_mask_spec(const char* text, sa_mask* out) {
    if (!text || !out) return SA_ERR_NULL;
    Cursor c(strip_spaces(text));
    std::string mode;
    if (!c.word(&mode)) return SA_ERR_SPEC;
    sa_mask m;
    std::memset(&m, 0, sizeof(m));
    const bool blocks = mode == "blocks";
    if (mode == "causal")
        m.causal = 1;
    else if (mode == "bidir" || blocks)
        m.causal = 0;
    else
        return SA_ERR_SPEC;

    m.dilation = 1;
    bool seen_window = false, seen_radius = false, seen_stride = false, seen_phase = false,
         seen_global = false, seen_dilation = false, seen_block = false, seen_random = false,
         seen_seed = false;
    std::vector<std::pair<int64_t, int64_t>> ranges;
    while (c.eat(';')) {
        std::string key;
        if (!c.word(&key) || !c.eat('=')) return SA_ERR_SPEC;
        if (key == "global") {
            if (seen_global || !parse_globals(c, &ranges)) return SA_ERR_SPEC;
            seen_global = true;
            continue;
        }
        int64_t v = 0;
        if (!c.number(&v)) return SA_ERR_SPEC;
        const bool block_only = key == "block" || key == "random" || key == "seed";
        const bool token_only = key == "window" || key == "dilation";
        if ((block_only && !blocks) || (token_only && blocks)) return SA_ERR_SPEC;
        if (key == "block") {
            if (seen_block || v < 1) return SA_ERR_SPEC;
            seen_block = true;
            m.block = v;
        } else if (key == "random") {
            if (seen_random || v > 4096) return SA_ERR_SPEC;
            seen_random = true;
            m.n_random = static_cast<int32_t>(v);
        } else if (key == "seed") {
            if (seen_seed) return SA_ERR_SPEC;
            seen_seed = true;
            m.seed = static_cast<uint32_t>(v);
        } else if (key == "window") {
            if (seen_window || !m.causal) return SA_ERR_SPEC;
            seen_window = true;
            m.window = v;
        } else if (key == "radius") {
            if (seen_radius || m.causal) return SA_ERR_SPEC;
            seen_radius = true;
            m.has_radius = 1;
            m.radius = v;
        } else if (key == "stride") {
            if (seen_stride) return SA_ERR_SPEC;
            seen_stride = true;
            m.stride = v;
        } else if (key == "phase") {
            if (seen_phase) return SA_ERR_SPEC;
            seen_phase = true;
            m.phase = v;
        } else if (key == "dilation") {
            if (seen_dilation || v < 1) return SA_ERR_SPEC;
            seen_dilation = true;
            m.dilation = static_cast<int32_t>(v);
        } else {
            return SA_ERR_SPEC;
        }
    }
    if (!c.done()) return SA_ERR_SPEC;
    if (blocks) {
        if (!seen_block) return SA_ERR_SPEC;
        m.has_radius = 1;  // radius counts blocks; absent = 0 (the query's own block)
    }
    if (seen_phase && m.stride == 0) return SA_ERR_SPEC;
    if (m.stride > 0 && m.phase >= m.stride) return SA_ERR_RANGE;  // well-formed, out of range

    // Sort and merge overlapping or touching ranges.
    std::sort(ranges.begin(), ranges.end());
    std::vector<std::pair<int64_t, int64_t>> merged;
    for (const auto& r : ranges) {
        if (!merged.empty() && r.first <= merged.back().second)
            merged.back().second = std::max(merged.back().second, r.second);
        else
            merged.push_back(r);
    }
    if (merged.size() > SA_MAX_GLOBAL_RANGES) return SA_ERR_SPEC;
    m.n_global = static_cast<int32_t>(merged.size());
    for (size_t k = 0; k < merged.size(); ++k) {
        m.global_lo[k] = merged[k].first;
        m.global_hi[k] = merged[k].second;
    }
    *out = m;
    return SA_OK;
}

std::string canonical_spec(const sa_mask& m) {
    std::string s = m.causal ? "causal" : (m.block > 0 ? "blocks" : "bidir");
    if (m.block > 0)
        s += ";block=" + std::to_string(m.block) + ";random=" + std::to_string(m.n_random) +
             ";seed=" + std::to_string(m.seed);
    if (m.causal) s += ";window=" + std::to_string(m.window);
    if (!m.causal && m.has_radius) s += ";radius=" + std::to_string(m.radius);
    if (m.dilation != 1) s += ";dilation=" + std::to_string(m.dilation);
    if (m.stride) s += ";stride=" + std::to_string(m.stride) + ";phase=" + std::to_string(m.phase);
    if (m.n_global) {
        s += ";global=";
        for (int k = 0; k < m.n_global; ++k) {
            if (k) s += ",";
            s += std::to_string(m.global_lo[k]) + ":" + std::to_string(m.global_hi[k]);
        }
    }
    return s;
}

}  // namespace sa
