// Internal declarations shared by the host planner, the C-ABI and the
// kernel launcher.  Not installed; the public interface is sparse_attn.h.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/sparse_attn.h"

namespace sa {

int parse_mask_spec(const char* text, sa_mask* out);
std::string canonical_spec(const sa_mask& m);

// The mask rule of sparse_attn.h for one sequence length, with prefix counts
// of "column-rule" keys (strided or global) and of global rows so that the
// number of allowed keys of any row inside any key range is O(1).
class MaskRule {
  public:
    MaskRule(const sa_mask& m, int64_t T);

    int64_t T() const { return T_; }
    bool causal() const { return m_.causal != 0; }
    bool row_global(int64_t i) const { return rowpre_[i + 1] != rowpre_[i]; }
    bool col_key(int64_t j) const { return colpre_[j + 1] != colpre_[j]; }
    int64_t rows_global_in(int64_t a, int64_t b) const { return rowpre_[b] - rowpre_[a]; }
    int64_t col_keys_in(int64_t a, int64_t b) const {  // keys in [a, b)
        return a >= b ? 0 : colpre_[b] - colpre_[a];
    }
    // Inclusive band [lo, hi] of row i, clipped to [0, T-1].  Both ends are
    // non-decreasing in i.
    int64_t band_lo(int64_t i) const;
    int64_t band_hi(int64_t i) const;
    // Largest key a row may read at all (the causal limit).
    int64_t key_limit(int64_t i) const { return causal() ? i : T_ - 1; }
    // Allowed keys of row i within [a, b).
    int64_t allowed_in(int64_t i, int64_t a, int64_t b) const;
    // SA_TILE_* for rows [q0, q1) x keys [k0, k1), judged on in-range cells.
    int classify(int64_t q0, int64_t q1, int64_t k0, int64_t k1) const;
    // Distance bounds of the band: key j is in row i's band iff
    // i - j <= back and j - i <= fwd (saturated to INT32_MAX when unlimited).
    int32_t band_back() const;
    int32_t band_fwd() const;
    const std::vector<int64_t>& colpre() const { return colpre_; }

  private:
    sa_mask m_;
    int64_t T_;
    std::vector<int64_t> colpre_;  // T + 1 entries
    std::vector<int64_t> rowpre_;  // T + 1 entries
};

// Execution plan for one (spec, T, tile shape).  All counts per (b, h).
struct HostPlan {
    int32_t bq = 0, bk = 0, n_qb = 0, n_kb = 0;
    std::vector<int32_t> qb_order;  // query blocks, most work first
    std::vector<int32_t> run_ptr;   // n_qb + 1
    std::vector<int32_t> runs;      // pairs: kb_begin, kb_end | (needs_mask << 31)
    std::vector<int32_t> gseg;      // 4 per qb: [a0, a1) and [b0, b1) into colkeys
    std::vector<int32_t> colkeys;   // sorted keys that are strided or global
    std::vector<uint64_t> colbits;  // bit j%64 of word j/64: key j is a colkey
    std::vector<uint32_t> rowbits;  // bit i%32 of word i/32: row i is global
    int64_t inplace_tiles = 0, masked_tiles = 0, gathered_tiles = 0, gathered_keys = 0;
};

HostPlan build_plan(const MaskRule& rule, int32_t bq, int32_t bk);

// Device-resident plan: one allocation, section offsets in bytes.
struct DevicePlan {
    void* base = nullptr;
    size_t bytes = 0;
    int32_t n_qb = 0;
    size_t off_qb_order = 0, off_run_ptr = 0, off_runs = 0, off_gseg = 0, off_colkeys = 0,
           off_colbits = 0, off_rowbits = 0;
};

// Kernel arguments (passed by value).
struct FwdArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    int32_t T;
    int32_t BH;
    int32_t causal;
    int32_t band_back;
    int32_t band_fwd;
    float scale_log2;  // log2(e) / sqrt(d)
    const int32_t* qb_order;
    const int32_t* run_ptr;
    const int32_t* runs;
    const int32_t* gseg;
    const int32_t* colkeys;
    const uint64_t* colbits;
    const uint32_t* rowbits;
};

constexpr int kBQ = 128;
constexpr int kBK = 64;

// Launch the fused forward kernel; returns SA_OK or SA_ERR_HIP.
int launch_fwd(int dtype, int d, const FwdArgs& args, int64_t grid, void* stream);
// The bf16 fast path (d = 64 or 128); SA_ERR_UNSUPPORTED for other shapes.
int launch_fwd_fast(int dtype, int d, const FwdArgs& args, int64_t grid, void* stream);

}  // namespace sa
