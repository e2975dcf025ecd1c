/*
 * sparse_attn.h -- C-ABI of the masked sparse attention library (forward),
 * built for AMD MI355X (gfx950).  Library file: libsparse_attn.so.
 *
 * The operation ("Sparse attention", glossary.selfmadequant.com, section
 * "Choose the available reads"): for every batch b, head h and query i,
 *
 *     O[b,h,i,:] = sum_{j in S_i} a_ij V[b,h,j,:],
 *     a_ij = exp(Q_i.K_j / sqrt(d)) / sum_{l in S_i} exp(Q_i.K_l / sqrt(d)),
 *
 * a softmax renormalised over the allowed key set S_i only.  S_i comes from
 * a mask spec (grammar below).  Pairs outside S_i are skipped tile by tile
 * and never materialised ("Attention variants", sreshtalluri.github.io,
 * section 5: the speed comes from never loading fully masked blocks).
 *
 * Mask rule.  allowed(i,j) = C and (L or St or Gl), with
 *   C  = (j <= i) in causal mode, true in bidir mode
 *   L  = with dilation g (default 1) and gap = i - j, gap mod g == 0 and
 *        causal: window == 0 or gap < window * g   (the window counts the
 *        query itself: "Attention variants" section 1; "Sparse attention",
 *        octlm lab note, "A window, plus a few global columns")
 *        bidir : no radius given or |gap| <= radius * g ("Sparse
 *        Attention", ai360xpert.com, "Local windows"; "Attention variants"
 *        section 3)
 *        With g > 1 the w window keys are i, i-g, ..., i-(w-1)g: the dilated
 *        mask of "Attention variants" section 6 (knowledge check).
 *   St = stride > 0 and j mod stride == phase (strided landmark columns;
 *        phase 0 in the octlm lab note, stride-1 in "Attention variants")
 *   Gl = i in G or j in G (global tokens read and are read by everyone;
 *        in causal mode C still applies, "Attention variants" section 4).
 *
 * Block mode (BigBird: "Sparse and sliding-window attention", getnybble.com,
 * section "Block-sparse attention: BigBird", a window of 3 blocks, R random
 * blocks, G global blocks).  With block size S, qb = i / S and kb = j / S:
 *   allowed(i,j) = |qb - kb| <= radius or kb in Rand(qb) or St or Gl,
 * bidirectional.  Rand(qb) holds R distinct key blocks drawn uniformly from
 * all ceil(T/S) blocks (local and global ones included): SplitMix64 (Steele,
 * Lea and Flood, OOPSLA 2014) started from state (seed << 32) | qb, each
 * output x naming block (x >> 32) mod ceil(T/S); repeats are skipped, at most
 * 64 R draws are made, and with ceil(T/S) <= R every block is taken.
 *
 * Mask-spec grammar (whitespace ignored; integers are decimal, >= 0,
 * < 2^31; a key may appear once):
 *   spec   := ('causal' | 'bidir') (';' clause)*
 *           | 'blocks' ';' 'block=' INT (';' bclause)*
 *   clause := 'window=' INT        causal only; 0 = unlimited (full causal)
 *           | 'radius=' INT        bidir only; absent = unlimited
 *           | 'dilation=' INT      >= 1; local keys sit this far apart
 *           | 'stride=' INT        0 = no strided columns
 *           | 'phase='  INT        needs stride > 0 (else SA_ERR_SPEC);
 *                                  0 <= phase < stride (else SA_ERR_RANGE)
 *           | 'global=' R (',' R)* R := INT | INT ':' INT  (half-open, a < b)
 *   bclause := 'radius=' INT       in blocks; default 0 (own block)
 *           | 'random=' INT        random key blocks per query block, <= 4096
 *           | 'seed=' INT          default 0
 *           | 'stride=' INT | 'phase=' INT | 'global=' ...   as above
 *   ('block=' may stand anywhere among the block-mode clauses; S >= 1.)
 *
 * Tensor layout.  Q, K, V, O are dense row-major [B][H][T][d] device arrays
 * of one element type (bf16 for sparse_attn_fwd, fp32 for
 * sparse_attn_fwd_f32), 16-byte aligned ("q, k, v: [batch, heads, n,
 * d_head]", "Attention variants" section 4 "Use the library").  The scale
 * is 1/sqrt(d).  O has the input's element type; bf16 output is rounded to
 * nearest even from the fp32 accumulator.
 *
 * Ownership.  The caller owns Q, K, V and O; the library never allocates,
 * frees or keeps them.  The library owns a per-device cache of execution
 * plans (tile lists for one spec and T), built on first use and freed by
 * sparse_attn_release_cache(), and an fp32 workspace per (device, stream),
 * grown on demand: partial results when a plan splits a heavy block (bf16
 * forward and backward; at most 1 GiB, past that the unsplit plan runs),
 * the backward's row dots and decode's key-split partials.  Calls are
 * thread-safe; calls that share a stream use its workspace in stream order
 * (hipStreamPerThread has one workspace per host thread, since it names a
 * different stream in each).
 *
 * Tuning.  SA_FWD_SPLIT_TILES=n (n > 0) in the environment makes the bf16
 * d = 64 / 128 forward and backward split every query block (and, in the
 * backward's dK/dV pass, every key block) above n tiles into work items (the
 * default splits blocks above max(16, twice the mean)); the result is the
 * same up to rounding order.
 *
 * Streams.  Device work is enqueued on `stream` (a hipStream_t; NULL = the
 * null stream) of the current device; the call returns after the enqueue.
 * O is valid once the stream reaches that point.  A new plan is uploaded
 * with hipMemcpyAsync on the caller's stream from a pinned host buffer that
 * the plan cache keeps alive; a call on another stream that finds the plan
 * still in flight makes its stream wait for the upload (an event), so no
 * call blocks the host or the device.  Growing a workspace synchronises
 * only the stream that owns it (the old buffer may still be in use there).
 *
 * Errors.  Every call returns SA_OK or a negative status.  All checks run
 * before anything is enqueued, so on error O is untouched.  No C++
 * exception crosses this boundary.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SA_OK 0
#define SA_ERR_SPEC (-1)        /* mask spec does not parse */
#define SA_ERR_RANGE (-2)       /* a global index >= T, or phase >= stride */
#define SA_ERR_SHAPE (-3)       /* B, H or T < 1, T > SA_MAX_T, bad tile shape */
#define SA_ERR_UNSUPPORTED (-4) /* d not in {16, 32, 64, 128}, unknown dtype */
#define SA_ERR_NULL (-5)        /* a required pointer is NULL */
#define SA_ERR_ALIAS (-6)       /* O overlaps Q, K or V */
#define SA_ERR_HIP (-7)         /* a HIP runtime call or the launch failed */
#define SA_ERR_ALIGN (-8)       /* a tensor pointer is not 16-byte aligned */
#define SA_ERR_NOMEM (-9)       /* host or device allocation for a plan failed */
#define SA_ERR_SCRATCH (-10)    /* sparse_attn_decode_noalloc: the call needs more
                                   than the static scratch holds */

/* tile classes written by sparse_attn_tile_map */
#define SA_TILE_EMPTY 0   /* no allowed pair among the tile's in-range cells */
#define SA_TILE_FULL 1    /* every in-range cell allowed */
#define SA_TILE_PARTIAL 2 /* some, not all */

/* element types */
#define SA_DTYPE_BF16 0
#define SA_DTYPE_F32 1

#define SA_MAX_GLOBAL_RANGES 64
#define SA_MAX_T (1 << 22)

/* A parsed mask spec.  Global ranges are sorted, merged and half-open. */
typedef struct sa_mask {
    int32_t causal;     /* 1 = causal, 0 = bidir */
    int32_t has_radius; /* bidir: 1 if radius= was given */
    int64_t window;     /* causal: 0 = unlimited */
    int64_t radius;     /* bidir: valid if has_radius */
    int64_t stride;     /* 0 = none */
    int64_t phase;
    int32_t n_global;
    int32_t dilation;   /* >= 1 */
    int64_t global_lo[SA_MAX_GLOBAL_RANGES];
    int64_t global_hi[SA_MAX_GLOBAL_RANGES];
    int64_t block;      /* > 0: block mode with block size `block`; radius
                           then counts blocks */
    int32_t n_random;   /* block mode: random key blocks per query block */
    uint32_t seed;      /* block mode: random stream seed */
} sa_mask;

/* Summary of the plan the kernel runs for (spec, T, d, dtype).  Counts are
 * per (batch, head). */
typedef struct sa_plan_info {
    int32_t bq, bk;              /* tile shape */
    int32_t n_qb, n_kb;          /* query / key blocks (of one subsequence) */
    int32_t subsequences;        /* 1, or g when a pure dilated window (no
                                    stride, no globals, T % g == 0, bf16,
                                    d in {64, 128}) runs as g interleaved
                                    plain windows of T/g rows; the tile
                                    counts below are totals over all g */
    int32_t split_parts;         /* bf16 fast path: work items that hold one
                                    key range of a query block with far more
                                    tiles than the mean (a block of global
                                    rows); a merge kernel combines their
                                    partial results.  0 when none is split */
    int64_t inplace_tiles;       /* contiguous key tiles executed */
    int64_t masked_tiles;        /* of those, tiles that evaluate the rule */
    int64_t gathered_tiles;      /* tiles of gathered landmark/global keys */
    int64_t gathered_keys;       /* keys staged through gathered tiles */
    int64_t executed_cells;      /* bq * bk * (inplace + gathered tiles) */
    int64_t allowed_cells;       /* E = sum_i |S_i| */
} sa_plan_info;

/*
 * Forward pass, bf16 in and out.  Q, K, V, O: device pointers to
 * [B][H][T][d] bf16 (raw 16-bit storage).  d in {16, 32, 64, 128}.
 * mask_spec: NUL-terminated spec text.  stream: hipStream_t or NULL.
 * Returns SA_OK or SA_ERR_{NULL, SHAPE, UNSUPPORTED, ALIGN, ALIAS, SPEC,
 * RANGE, NOMEM, HIP}.
 */
int sparse_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                    int B, int H, int T, int d, const char* mask_spec,
                    void* stream);

/* Same as sparse_attn_fwd with fp32 tensors (fp32 MFMA, fp32 softmax). */
int sparse_attn_fwd_f32(const void* Q, const void* K, const void* V, void* O,
                        int B, int H, int T, int d, const char* mask_spec,
                        void* stream);

/*
 * Forward that also writes LSE: device float [B][H][T], the natural-log
 * log-sum-exp of each row's allowed scores, lse_i = log sum_{j in S_i}
 * exp(Q_i.K_j / sqrt(d)) (what the backward needs to rebuild the weights).
 * Otherwise as sparse_attn_fwd / sparse_attn_fwd_f32; LSE must be 4-byte
 * aligned and must not overlap Q, K, V or O (SA_ERR_ALIAS).
 */
int sparse_attn_fwd_lse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int B, int H, int T, int d, const char* mask_spec, void* stream);
int sparse_attn_fwd_lse_f32(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int B, int H, int T, int d, const char* mask_spec, void* stream);

/*
 * Backward pass: gradients of the forward for an upstream gradient dO.  The
 * pages define the forward only; this is its gradient by the chain rule
 * through the softmax over S_i ("Sparse attention", "Choose the available
 * reads").  With p_ij = exp(Q_i.K_j / sqrt(d) - LSE_i) for j in S_i,
 * dp_ij = dO_i.V_j, D_i = dO_i.O_i and ds_ij = p_ij (dp_ij - D_i):
 *   dQ_i = sum_j ds_ij K_j / sqrt(d),  dK_j = sum_i ds_ij Q_i / sqrt(d),
 *   dV_j = sum_i p_ij dO_i.
 * Q, K, V, O, dO (input dtype: bf16 for sparse_attn_bwd, fp32 for _f32) and
 * LSE (float) are the forward's tensors and its LSE output for the same
 * mask_spec; dQ, dK, dV are written in full ([B][H][T][d], input dtype).
 * Outputs must not overlap each other or any input (SA_ERR_ALIAS).  A
 * library-owned fp32 workspace of B*H*T floats per (device, stream) holds
 * D between the two kernels (shared with decode, grown on demand).
 * Returns SA_OK or SA_ERR_{NULL, SHAPE, UNSUPPORTED, ALIGN, ALIAS, SPEC,
 * RANGE, NOMEM, HIP}, validation before any device work.
 */
int sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int T, int d,
                    const char* mask_spec, void* stream);
int sparse_attn_bwd_f32(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                        int H, int T, int d, const char* mask_spec, void* stream);

/* Parse mask_spec into *out (host only).  SA_ERR_SPEC on any grammar
 * error, SA_ERR_RANGE for phase >= stride, SA_ERR_NULL on NULL arguments. */
int sparse_attn_parse(const char* mask_spec, sa_mask* out);

/*
 * Count allowed pairs for sequence length T (host only): *allowed_cells =
 * E = sum_i |S_i| ("Sparse attention", glossary.selfmadequant.com, "Six
 * tokens: count connections before claiming speed").  row_counts may be
 * NULL, else receives |S_i| for i in [0, T).  SA_ERR_RANGE if a global
 * index is >= T.
 */
int sparse_attn_count(const char* mask_spec, int T, int64_t* allowed_cells,
                      int32_t* row_counts);

/*
 * Classify every (query block, key block) tile of a T x T grid cut into
 * bq x bk tiles (host only).  map[qb * ceil(T/bk) + kb] receives
 * SA_TILE_EMPTY / FULL / PARTIAL, judged over the tile's in-range cells
 * (row and key < T).  Exact at any tile shape, not only the kernel's.
 */
int sparse_attn_tile_map(const char* mask_spec, int T, int bq, int bk,
                         uint8_t* map);

/* The tile shape (query rows bq x keys bk) the forward kernel uses for
 * mask_spec, head dim d and dtype (SA_DTYPE_*) in a call large enough to
 * fill the GPU; the same shape that sparse_attn_plan_info reports.
 * mask_spec may be NULL: the shape of the token-level specs (causal /
 * bidir), 128 x 64.  Block mode with a block size that is a multiple of 64
 * but not of 128 runs 64 x 64 tiles at bf16, d = 64 (every tile then lies in
 * one query block).  A smaller call can run other tiles: the shape of a
 * given call is the bq, bk that sparse_attn_plan_info_bh reports for its B,
 * H and T.  Host only.  Returns SA_OK or SA_ERR_{NULL, UNSUPPORTED, SPEC,
 * RANGE}. */
int sparse_attn_tile_shape(const char* mask_spec, int d, int dtype, int* bq, int* bk);

/* Describe the plan the kernel would run for (mask_spec, T, d, dtype) in a
 * call large enough to fill the GPU (host only; builds no device state).
 * Returns SA_OK or SA_ERR_{NULL, SHAPE, UNSUPPORTED, SPEC, RANGE}. */
int sparse_attn_plan_info(const char* mask_spec, int T, int d, int dtype,
                          sa_plan_info* info);

/* Describe the plan a forward call with these B, H, T, d, dtype runs (host
 * only; builds no device state).  It differs from sparse_attn_plan_info in
 * one case: a token-level (causal / bidir) bf16 call with d = 64, no residue
 * split and B * H * ceil(T / 128) <= 256 (the MI355X's compute units) runs
 * 64 x 64 tiles, so that every compute unit holds two independent
 * workgroups.  Returns SA_OK or SA_ERR_{NULL, SHAPE (B or H < 1, bad T),
 * UNSUPPORTED, SPEC, RANGE}. */
int sparse_attn_plan_info_bh(const char* mask_spec, int B, int H, int T, int d, int dtype,
                             sa_plan_info* info);

/*
 * Windowed decode, bf16: n_new new query tokens per sequence against a
 * ring-buffer KV cache that keeps only the last C positions ("Sparse and
 * sliding-window attention", getnybble.com, section "Sliding window
 * attention": the cache is capped at the window; "Attention variants",
 * section 1 and section 3 "Worked example: KV cache for a long context").
 *
 *   Q        device [B][H][n_new][d]: the new tokens, at positions
 *            pos[b]-n_new+1 .. pos[b] of sequence b.
 *   K_cache, V_cache  device [B][Hkv][C][d]: position t of sequence b, KV
 *            head k lives in row t mod C.  The new tokens' keys and values
 *            must already be written.  H is a multiple of Hkv; query head h
 *            reads KV head h / (H / Hkv) (grouped-query attention).
 *   O        device [B][H][n_new][d], written.
 *   pos      device int32 [B], read by the kernel (so a decode loop can
 *            advance it on the device); pos[b] >= n_new - 1.
 *   mask_spec  causal specs only, window (0 = unlimited) and dilation; a
 *            spec with strided or global keys is SA_ERR_UNSUPPORTED (those
 *            keys would need a cache of their own).
 *
 * Query i (absolute position) reads the live positions max(0, pos-C+1) ..
 * pos that the mask rule allows.  That equals the forward's row i when C is
 * at least sparse_attn_decode_cache_rows(spec, n_new) for a window, and when
 * no position has left the cache (pos < C) for an unlimited window.  C below
 * the window's need is SA_ERR_SHAPE.  A query with no live allowed key
 * gets O = 0.
 *
 * Long caches are split over several workgroups whose partial results go
 * through a library-owned fp32 workspace, one per (device, stream), grown on
 * demand (growing synchronises the device) and freed by
 * sparse_attn_release_cache.  Calls on one stream are ordered; calls on
 * different streams never share a workspace.  Returns SA_OK or SA_ERR_{NULL,
 * SHAPE, UNSUPPORTED, ALIGN, ALIAS, SPEC, NOMEM, HIP}; validation happens
 * before any device work.
 */
int sparse_attn_decode(const void* Q, const void* K_cache, const void* V_cache, void* O,
                       const int32_t* pos, int B, int H, int Hkv, int n_new, int C, int d,
                       const char* mask_spec, void* stream);

/*
 * Allocation-free windowed decode, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, layout, semantics and errors are those of
 * sparse_attn_decode, and the result is bit-identical to it (same kernels,
 * same key splits).  The difference: the key-split partials live in a static
 * device array of SA_DECODE_SCRATCH_BYTES per GPU (part of the library's
 * device code, so each GPU it is loaded on holds one until the process
 * ends), instead of the library workspace; no call on this path allocates or frees memory (hipMalloc,
 * hipFree, host containers).  The array's address on a device is looked up
 * on this entry point's first call on that device.
 *
 * A call needs B * H * n_new * nsplit * (d + 2) * 4 bytes of scratch when it
 * splits the cache over nsplit > 1 workgroups (nsplit = ceil(512 / groups)
 * for groups = B * Hkv * ceil(H / Hkv * n_new / 8) below 512, capped so each
 * split covers at least 256 keys; one split needs none).  That is at most
 * about 4.3 MB (d = 128, groups just below 512, eight queries each); a call
 * that needs more than SA_DECODE_SCRATCH_BYTES (4 MiB) returns SA_ERR_SCRATCH
 * before any device work -- for example B = 511, H = 8, Hkv = 1, n_new = 1,
 * d = 128 with a 4096-row window -- and can use sparse_attn_decode instead.  Every partial a call reads is written by the same call first, so
 * nothing has to start at zero.
 *
 * All calls on one GPU share that GPU's array: calls on one stream are
 * ordered, but calls that may overlap in time on one GPU (different streams,
 * or several host threads without a common stream) race on it and must not
 * be issued.
 */
#define SA_DECODE_SCRATCH_BYTES (4 << 20)
int sparse_attn_decode_noalloc(const void* Q, const void* K_cache, const void* V_cache, void* O,
                               const int32_t* pos, int B, int H, int Hkv, int n_new, int C,
                               int d, const char* mask_spec, void* stream);

/* Cache rows decode needs for mask_spec and n_new new tokens (host only):
 * (w-1)*g + n_new for a window w with dilation g -- for n_new = 1 and g = 1
 * the last w positions; 0 when the window is unlimited (the cache must then
 * hold the whole context).  SA_ERR_UNSUPPORTED for specs decode rejects. */
int sparse_attn_decode_cache_rows(const char* mask_spec, int n_new, int64_t* rows);

/* Static text for a status code. */
const char* sparse_attn_strerror(int status);

/* Free every cached plan and workspace on every device.  The caller
 * must make sure no launched kernel still uses them (synchronise first). */
void sparse_attn_release_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
