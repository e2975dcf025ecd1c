// Internal declarations shared by the host planner, the C-ABI and the
// kernel launcher.  Not installed; the public interface is sparse_attn.h.
#pragma once

#include <stdint.h>

#include <algorithm>

#include <string>
#include <vector>

#include "../../include/sparse_attn.h"

namespace sa {

int parse_mask_spec(const char* text, sa_mask* out);
std::string canonical_spec(const sa_mask& m);

// How far the local band reaches from the query, in keys: (w-1)g behind it
// in causal mode, rg on each side in bidir mode (g = dilation); -1 when the
// band is unlimited.
inline int64_t band_reach(const sa_mask& m) {
    if (m.block > 0) return -2;  // block mode: no token band (see band_reach32)
    const int64_t g = m.dilation > 1 ? m.dilation : 1;
    if (m.causal) return m.window == 0 ? -1 : (m.window - 1) * g;
    return m.has_radius ? m.radius * g : -1;
}

// band_reach as the kernels take it: INT32_MAX stands for unlimited (any
// reach >= T is the same band).
inline int32_t band_reach32(const sa_mask& m) {
    const int64_t r = band_reach(m);
    if (r == -2) return -1;  // empty band: i - j <= -1 and j - i <= -1 never hold
    return r < 0 || r > INT32_MAX ? INT32_MAX : static_cast<int32_t>(r);
}

// Random key blocks of query block qb in block mode ("Rand(qb)" of
// sparse_attn.h): SplitMix64 from state (seed << 32) | qb, block (x >> 32)
// mod nkb per output, repeats skipped, at most 64 R draws.
std::vector<int64_t> random_key_blocks(const sa_mask& m, int64_t nkb, int64_t qb);

// The mask rule of sparse_attn.h for one sequence length, with prefix counts
// of "column-rule" keys (strided or global) and of global rows so that the
// number of allowed keys of any row inside any key range is O(1).
class MaskRule {
  public:
    MaskRule(const sa_mask& m, int64_t T);

    int64_t T() const { return T_; }
    bool causal() const { return m_.causal != 0; }
    int64_t dilation() const { return g_; }
    int64_t block() const { return S_; }
    // Block mode: allowed key-block intervals [kb0, kb1) of query block qb,
    // sorted and disjoint: ivals()[2t], ivals()[2t+1] for t in
    // [iv_ptr()[qb], iv_ptr()[qb + 1]).
    const std::vector<int32_t>& iv_ptr() const { return iv_ptr_; }
    const std::vector<int32_t>& ivals() const { return ivals_; }
    bool row_global(int64_t i) const { return rowpre_[i + 1] != rowpre_[i]; }
    bool col_key(int64_t j) const { return colpre_[j + 1] != colpre_[j]; }
    int64_t rows_global_in(int64_t a, int64_t b) const { return rowpre_[b] - rowpre_[a]; }
    int64_t col_keys_in(int64_t a, int64_t b) const {  // keys in [a, b)
        return a >= b ? 0 : colpre_[b] - colpre_[a];
    }
    // Inclusive extent [lo, hi] of row i's band, clipped to [0, T-1].  Both
    // ends are non-decreasing in i.  With dilation g > 1 only the keys of the
    // extent with j = i (mod g) are in the band.
    int64_t band_lo(int64_t i) const;
    int64_t band_hi(int64_t i) const;
    // Largest key a row may read at all (the causal limit).
    int64_t key_limit(int64_t i) const { return causal() ? i : T_ - 1; }
    // Allowed keys of row i within [a, b).
    int64_t allowed_in(int64_t i, int64_t a, int64_t b) const;
    // Of those, the ones that are not column (strided or global) keys.
    int64_t allowed_noncol_in(int64_t i, int64_t a, int64_t b) const {
        const int64_t lo = std::max<int64_t>(a, 0), hi = std::min<int64_t>(b, key_limit(i) + 1);
        return lo >= hi ? 0 : allowed_in(i, a, b) - col_keys_in(lo, hi);
    }
    // SA_TILE_* for rows [q0, q1) x keys [k0, k1), judged on in-range cells.
    int classify(int64_t q0, int64_t q1, int64_t k0, int64_t k1) const;
    // Distance bounds of the band: key j is in row i's band iff
    // i - j <= back, j - i <= fwd (saturated to INT32_MAX when unlimited)
    // and i - j = 0 (mod g).
    int32_t band_back() const;
    int32_t band_fwd() const;
    const std::vector<int64_t>& colpre() const { return colpre_; }

  private:
    // Keys j in [a, b) with j = i (mod g), and the column keys among them.
    int64_t on_grid(int64_t i, int64_t a, int64_t b) const;
    int64_t col_keys_on_grid(int64_t i, int64_t a, int64_t b) const;

    sa_mask m_;
    int64_t T_;
    int64_t g_;                    // dilation
    std::vector<int64_t> colpre_;  // T + 1 entries
    std::vector<int64_t> rowpre_;  // T + 1 entries
    std::vector<int64_t> colres_;  // g > 1: column keys k <= j with k = j (mod g)
    int64_t S_ = 0;                // block size (block mode) or 0
    std::vector<int32_t> iv_ptr_, ivals_;
};

// Execution plan for one (spec, T, tile shape).  All counts per (b, h).
// The kernels run work items: each is one query block, or -- for a block
// whose tile count is far above the mean -- one range of its tiles, whose
// unnormalised result goes to a partial slot that a merge kernel combines.
struct HostPlan {
    int32_t bq = 0, bk = 0, n_qb = 0, n_kb = 0;
    int32_t n_items = 0;            // work items (n_qb when nothing is split)
    int32_t n_parts = 0;            // items that write partial slots
    std::vector<int32_t> qb_order;  // work items, most work first
    std::vector<int32_t> run_ptr;   // n_items + 1
    std::vector<int32_t> runs;      // pairs: kb_begin, kb_end | (needs_mask << 31)
    std::vector<int32_t> gseg;      // 4 per item: [a0, a1) and [b0, b1) into colkeys
    std::vector<int32_t> item_qb;   // query block of each item
    std::vector<int32_t> item_part; // -1 (writes O) or the item's partial slot
    std::vector<int32_t> split_qb;  // the split query blocks ...
    std::vector<int32_t> split_ptr; // ... and their slots [split_ptr[s], split_ptr[s+1])
    std::vector<int32_t> colkeys;   // sorted keys that are strided or global
    std::vector<uint64_t> colbits;  // bit j%64 of word j/64: key j is a colkey
    std::vector<uint32_t> rowbits;  // bit i%32 of word i/32: row i is global
    std::vector<int32_t> blk_ptr;   // block mode: copies of MaskRule::iv_ptr/ivals
    std::vector<int32_t> blk_iv;
    // The fast kernel's view of the items: kItemRec ints per item, in
    // qb_order's order, so that one scalar load gives a workgroup all of it
    // (see ItemRec for the fields).
    std::vector<int32_t> item_rec;
    int64_t inplace_tiles = 0, masked_tiles = 0, gathered_tiles = 0, gathered_keys = 0;
};

// Fields of one item record.  FIRST_KB / FIRST_END repeat the item's first
// run (FIRST_END carries the run's mask flag in bit 31), so the first tile
// can be addressed without a dependent read; both are 0 when the item has
// no in-place run.
enum ItemRec : int {
    REC_QB = 0,
    REC_PART,
    REC_RUN_BEGIN,
    REC_RUN_END,
    REC_GA0,
    REC_GA1,
    REC_GB0,
    REC_GB1,
    REC_FIRST_KB,
    REC_FIRST_END,
};
constexpr int kItemRec = 16;

// split_cap: 0 = one item per query block; kSplitAuto = split blocks above
// max(kSplitMinTiles, twice the mean tile count); n > 0 = split blocks above
// n tiles.  A block of w > cap tiles becomes ceil(w / cap) items.
constexpr int64_t kSplitMinTiles = 16;
constexpr int64_t kSplitAuto = -1;
HostPlan build_plan(const MaskRule& rule, int32_t bq, int32_t bk, int64_t split_cap = 0);

// Device-resident plan: one allocation, section offsets in bytes.
struct DevicePlan {
    void* base = nullptr;
    size_t bytes = 0;
    int32_t n_qb = 0, n_items = 0, n_parts = 0, n_split = 0;
    size_t off_qb_order = 0, off_run_ptr = 0, off_runs = 0, off_gseg = 0, off_colkeys = 0,
           off_colbits = 0, off_rowbits = 0, off_blk_ptr = 0, off_blk_iv = 0, off_item_qb = 0,
           off_item_part = 0, off_split_qb = 0, off_split_ptr = 0, off_item_rec = 0;
};

// Device-resident backward plan (one allocation).
struct BwdDevicePlan {
    void* base = nullptr;
    size_t bytes = 0;
    int32_t n_kb = 0, n_items = 0, n_parts = 0, n_split = 0, n_gkb = 0, n_col = 0;
    size_t off_order = 0, off_ptr = 0, off_runs = 0, off_item_kb = 0, off_item_part = 0,
           off_split_kb = 0, off_split_ptr = 0;
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
    int32_t dil;       // dilation g >= 1
    uint64_t dil_pat;  // bits 0, g, 2g, ... below 64
    // Block mode: query block i / blk of query i may read the key blocks in
    // the intervals blk_iv[2t], blk_iv[2t+1] for t in [blk_ptr[qb], blk_ptr[qb+1]).
    int32_t blk;  // 0 = token mode
    const int32_t* blk_ptr;
    const int32_t* blk_iv;
    // Interleaved subsequences: with sub > 1 each of the BH sequences above is
    // one residue class r of a sequence of T * sub rows (rows r, r + sub, ...),
    // BH counts (b, h, r) triples, and rows sit sub * d elements apart.
    int32_t sub;
    float scale_log2;  // log2(e) / sqrt(d)
    const int32_t* qb_order;
    const int32_t* run_ptr;
    const int32_t* runs;
    const int32_t* gseg;
    const int32_t* colkeys;
    const uint64_t* colbits;
    const uint32_t* rowbits;
    float* lse;  // optional [BH][T] output: natural-log sum of exp of the row's scores
    int32_t bq;  // query rows per tile of the plan (kBQ, or 64: fast path only)
    // Split plans (fast path only): item -> query block and partial slot.
    // part holds [BH][n_parts][bq][d] fp32 unnormalised outputs, then
    // [BH][n_parts][bq] float2 (running max in log2 units, row sum).
    const int32_t* item_qb;    // null: item = query block
    const int32_t* item_part;  // null: no partial slots
    const int32_t* item_rec;   // kItemRec ints per item, in qb_order's order
    float* part;
    int32_t n_parts;
};

constexpr int kBQ = 128;
constexpr int kBK = 64;

// Backward plan: for each block of kBKB keys, runs of the kBQB-query tiles
// that hold allowed pairs with it (the forward plan read by key).
constexpr int kBKB = 128;  // keys per dK/dV workgroup
constexpr int kBQB = 64;   // queries per tile it visits

// Work items as in HostPlan: a key block, or one range of the query tiles
// of a key block far heavier than the mean (the key block of a global
// column), whose partial dK and dV a merge kernel sums.
struct BwdHostPlan {
    int32_t n_kb = 0, n_qt = 0;
    // With gathered column keys: key blocks n_kb .. n_kb + n_gkb - 1 are
    // blocks of the sorted column-key list (n_col keys), and the band blocks
    // leave their column keys to them.
    int32_t n_gkb = 0, n_col = 0;
    int32_t n_items = 0, n_parts = 0;
    std::vector<int32_t> kb_order;   // work items, most work first
    std::vector<int32_t> kb_ptr;     // n_items + 1
    std::vector<int32_t> kb_runs;    // pairs: qt_begin, qt_end | (needs_mask << 31)
    std::vector<int32_t> item_kb;    // key block of each item
    std::vector<int32_t> item_part;  // -1 or the item's partial slot
    std::vector<int32_t> split_kb;   // split key blocks and their slots
    std::vector<int32_t> split_ptr;  // [split_ptr[s], split_ptr[s+1])
    int64_t tiles = 0, masked_tiles = 0;
};

// Key blocks of bkb keys (kBKB, or 64 with the forward's 64-row plans);
// split_cap as build_plan's; gather_cols: run the column keys as gathered
// key blocks (bf16 d = 64 / 128 kernels).
BwdHostPlan build_bwd_plan(const MaskRule& rule, int32_t bkb, int64_t split_cap = 0,
                           bool gather_cols = false);

// Backward arguments: the forward's (rule, plan, Q, K, V, O) plus gradients,
// the saved log-sum-exp and the transposed plan.
struct BwdArgs {
    FwdArgs f;           // f.Q, f.K, f.V, f.O, rule and forward plan; f.lse unused
    const void* dO;      // [BH][T][d]
    const float* lse;    // [BH][T] natural-log sum of exp, from the forward
    void* dQ;            // [BH][T][d] outputs, input dtype
    void* dK;
    void* dV;
    float* Dw;           // [BH][T] workspace: D_i = dO_i . O_i
    float scale;         // 1 / sqrt(d)
    const int32_t* kb_order;
    const int32_t* kb_ptr;
    const int32_t* kb_runs;
    int32_t n_kb;
    // Split work items (bf16 d = 64 / 128 kernels only).  dQ: f.item_qb,
    // f.item_part and f.n_parts of the forward plan; partials [BH][n_parts]
    // [bq][d] fp32 in dq_part.  dK/dV: kv_item_kb, kv_item_part; partials
    // [BH][kv_n_parts][bkb][d] fp32 for dK, then the same for dV, in kv_part.
    int32_t n_q_items, n_kv_items;
    float* dq_part;
    const int32_t* dq_split_qb;
    const int32_t* dq_split_ptr;
    int32_t dq_n_split;
    const int32_t* kv_item_kb;    // null: item = key block
    const int32_t* kv_item_part;  // null: no partial slots
    float* kv_part;
    const int32_t* kv_split_kb;
    const int32_t* kv_split_ptr;
    int32_t kv_n_split, kv_n_parts;
    // Gathered column keys (kv_n_gkb > 0): items with key block kb >= n_kb
    // run keys f.colkeys[(kb - n_kb) * bkb ...] (kv_n_col keys in all), and
    // band blocks skip their column keys.
    int32_t kv_n_gkb, kv_n_col;
};

int launch_bwd(int dtype, int d, const BwdArgs& args, void* stream);

// Decode arguments (passed by value): n_new query tokens per sequence against
// ring-buffer caches [B][Hkv][C][d]; position t lives in slot t mod C.
struct DecodeArgs {
    const void* Q;         // [B][H][n_new][d] bf16
    const void* K;         // [B][Hkv][C][d] bf16
    const void* V;         // [B][Hkv][C][d] bf16
    void* O;               // [B][H][n_new][d] bf16
    const int32_t* pos;    // [B] position of each sequence's last new token
    float* part;           // nsplit > 1: [B*H*n_new][nsplit][d+2] fp32 (m, l, acc)
    int32_t B, H, Hkv, G;  // G = H / Hkv query heads per KV head
    int32_t n_new, C, nsplit;
    int32_t reach;         // band reach (w-1)g, INT32_MAX = unlimited
    int32_t dil;           // dilation g
    float scale_log2;      // log2(e) / sqrt(d)
};

int launch_decode(int d, const DecodeArgs& args, void* stream);

// Size of the static scratch array of the allocation-free decode entry point
// (one per GPU, for the key-split partials).
constexpr size_t kDecodeScratchBytes = size_t(SA_DECODE_SCRATCH_BYTES);
// That array's device address on the current device (looked up once per
// device); SA_ERR_SCRATCH when `bytes` exceeds kDecodeScratchBytes.
int decode_scratch(size_t bytes, float** out);

// A pure dilated window (no strided or global keys) links only rows of equal
// residue mod g, and within a residue class it is the plain window.  When T
// is a multiple of g the forward then runs as g interleaved plain-window
// sequences of T/g rows each (the bf16 fast path only).
inline bool residue_split(const sa_mask& m, int T, int d, int dtype) {
    return m.dilation > 1 && m.stride == 0 && m.n_global == 0 && T % m.dilation == 0 &&
           dtype == SA_DTYPE_BF16 && (d == 64 || d == 128);
}

// Query rows per tile of the forward plan.  Block mode with 64-key blocks
// runs 64-query tiles on the bf16 d = 64 fast path: every tile then lies in
// one query block, whose key blocks (neighbours, random picks, globals) are
// whole tiles, instead of mixing two query blocks' random sets.
inline int fwd_query_block(const sa_mask& m, int d, int dtype) {
    return (m.block > 0 && m.block % 128 != 0 && m.block % 64 == 0 && dtype == SA_DTYPE_BF16 && d == 64)
               ? 64
               : kBQ;
}

// Whether the bf16 fast path runs (dtype, d) with bq-row tiles and `sub`
// interleaved subsequences; only its plans are split.
inline bool fwd_fast_path(int dtype, int d, int bq, int sub) {
    if (dtype != SA_DTYPE_BF16 || (d != 64 && d != 128)) return false;
    if (bq == 64) return d == 64 && sub == 1;
    return bq == kBQ;
}

// Launch the fused forward kernel; returns SA_OK or SA_ERR_HIP.
int launch_fwd(int dtype, int d, const FwdArgs& args, int64_t grid, void* stream);
// The bf16 fast path (d = 64 or 128); SA_ERR_UNSUPPORTED for other shapes.
int launch_fwd_fast(int dtype, int d, const FwdArgs& args, int64_t grid, void* stream);
// Merge the partial slots of the n_split split query blocks into O (and LSE).
int launch_fwd_merge(int d, const FwdArgs& args, const int32_t* split_qb, const int32_t* split_ptr,
                     int32_t n_split, void* stream);

}  // namespace sa
