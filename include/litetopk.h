/*
 * litetopk.h -- C ABI of the MI355X (gfx950) fused Indexer-TopK library.
 *
 * The operation (LiteTopK pages, "Problem statement" and "Methodology"):
 * for every query of a prefill chunk, score every causal key and return the
 * exact top-k key indices, without writing the full score matrix to device
 * memory.  The method runs in three phases -- Sample, Filter, Select -- and
 * is exact: the returned set is the plain top-k of the scores (arXiv
 * abstract: "preserving exact top-k correctness").
 *
 * Scores (the pages name "relevance scores for all candidate tokens"; the
 * indexer form is the DSA-style indexer score):
 *   indexer    I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])   s <= pos[t]
 *   retrieval  I[t,s] = q[t,:] . x[s,:]                              all s
 * Ties at the k-th score go to the lower key index.
 *
 * Conventions for every entry point below:
 *  - All pointers are DEVICE pointers unless noted; the caller owns every
 *    buffer, including the workspace.  The library allocates nothing and
 *    keeps no state between calls except a cached per-device architecture
 *    check.
 *  - Arrays are row-major and contiguous.  q/k/db rows must start on a
 *    16-byte boundary (q, k and db themselves 16-byte aligned).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream), never synchronises the host, and returns an ltk_status.  No
 *    C++ exception crosses the ABI.  Calls on different streams must use
 *    different workspaces.
 *  - Host-side argument errors are reported before anything is enqueued.
 *    Data conditions are NOT errors: duplicate, out-of-range or non-causal
 *    sample entries are ignored; with no sample (n_sample == 0) the library
 *    samples min(3 topk, L, 16384) evenly spaced causal keys itself; a candidate
 *    buffer that overflows is recovered exactly on the device; rows with
 *    fewer than k valid keys are padded with -1 (score NaN).
 *  - Inputs must be finite (no NaN/Inf in q, k, w, scales).
 */
#ifndef LITETOPK_H
#define LITETOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LTK_OK = 0,
    LTK_EINVAL = -1,        /* bad argument (null pointer, size, alignment, option) */
    LTK_EUNSUPPORTED = -2,  /* unsupported (H, D, dtype) or device is not gfx950 */
    LTK_EWORKSPACE = -3,    /* ws_bytes smaller than litetopk_workspace_bytes() */
    LTK_EHIP = -4           /* a HIP runtime call or launch failed */
} ltk_status;

typedef enum {
    LTK_F32 = 0,            /* fp32 q/k */
    LTK_BF16 = 1,           /* bf16 q/k (bit patterns, round-to-nearest-even) */
    LTK_FP8_E4M3FN = 2      /* OCP e4m3fn q/k with fp32 per-token scales */
} ltk_dtype;

typedef enum {
    LTK_KIND_SCORE_SELECT = 0,   /* litetopk_score_select */
    LTK_KIND_RETRIEVE = 1,       /* litetopk_retrieve */
    LTK_KIND_UNFUSED = 2,        /* litetopk_unfused_score_select */
    LTK_KIND_NEXT_SAMPLE = 3,    /* litetopk_next_sample */
    LTK_KIND_UNFUSED_RETRIEVE = 4  /* litetopk_unfused_retrieve */
} ltk_kind;

/* Tuning options (HOST struct).  Pass NULL for the defaults; a zero field
 * also means "default".  None of them changes the result, only the work. */
typedef struct {
    int32_t nbins;          /* equal-width bins over the sample's score range; 1..1024, default 256 */
    int32_t refresh_every;  /* threshold refresh after every N candidate batches; default 1; <0 = never */
    int32_t l_splits;       /* key-range splits per query group; default: chosen to fill the GPU */
    int32_t sorted_output;  /* nonzero: each row ordered by (score desc, index asc), with or without
                               out_score; needs topk <= 8192 */
    int64_t cand_capacity;  /* candidate-buffer entries per query; default 16384 (retrieval
                               max(262144, 64 x topk); shared thresholds: L when T x L x 8 B <= 512 MiB,
                               else >= 256 per split) */
    void* scan_event_start; /* optional hipEvent_t recorded on `stream` just before the fused scan kernel */
    void* scan_event_stop;  /* optional hipEvent_t recorded just after it (profiling; NULL = none) */
    int32_t shared_threshold; /* indexer: key splits of a query share one threshold histogram in the
                                 workspace (decode: few queries over a long context); 0 = when the
                                 scan has >= 16 splits, > 0 = always, < 0 = never */
    int32_t flush_batch;    /* indexer: candidates per write-back batch of a wave's list, 32 or 64
                               (LiteTopK summary, Methodology > 2. Filtering: batches of 32 or 64);
                               default 64 */
} ltk_opts;

/* Optional counters (DEVICE struct, written by the call; pass NULL to skip). */
typedef struct {
    uint64_t cand_written;        /* candidates appended over all queries (incl. dropped ones) */
    uint64_t bytes_written;       /* bytes the call wrote to device memory for its rows: stored
                                     candidates (8 B each), sample scores (4 B per query and
                                     distinct sample key) and the outputs (4 B per index, 4 B per
                                     score when asked); the full score matrix would be 4 B per pair */
    uint32_t max_cand_per_query;  /* largest per-query candidate count */
    uint32_t overflow_rows;       /* rows recovered by the exact overflow fallback */
} ltk_stats;

/* Bytes of workspace a call of `kind` needs.  For LTK_KIND_RETRIEVE, H is
 * ignored and L is the database size N; for LTK_KIND_UNFUSED, topk, n_sample
 * and opts are ignored (it holds the full T x L fp32 score matrix and, for
 * fp8, 4 D + 4 bytes per query of linear-term operands); for
 * LTK_KIND_NEXT_SAMPLE only L counts (4 * L bytes of key counts and a fixed
 * 69,888 bytes more).  Returns 0 for invalid sizes. */
size_t litetopk_workspace_bytes(int32_t kind, int32_t T, int32_t H, int32_t D, int64_t L,
                                int32_t topk, int32_t n_sample, int32_t dtype, const ltk_opts* opts);

/* Fused indexer top-k of one prefill chunk (LiteTopK pages, "Methodology":
 * Sample -> Filter -> Select).
 *
 *  q        [T, H, D] queries (dtype); k [L, D] keys (dtype)
 *  q_scale  [T] fp32 per-query scales (fp8 only; NULL otherwise), finite and > 0
 *  k_scale  [L] fp32 per-key scales (fp8 only; NULL otherwise), finite and > 0
 *           (the kernels move both scales out of the ReLU, which is exact for
 *           positive scales only)
 *  w        [T, H] fp32 head weights (either sign)
 *           (with T == 0 the per-query arrays q, q_scale, w, pos and the
 *           outputs may be NULL: the call checks its sizes and returns 0)
 *  pos      [T] int32 query positions; keys 0..pos[t] (and < L) are valid
 *  T >= 0, 1 <= H <= 64, D in {64, 128}, 1 <= L <= 2^31 - 256 (key offsets
 *           past a tile's end stay in int32), 1 <= topk <= 65536
 *           (a decode or speculative-decode step is the same call with T = 1..8
 *           queries at the newest positions; the key range is then split over
 *           every CU and the splits share one threshold per query)
 *  sample   [n_sample] int32 key indices reused from the previous chunk's
 *           result (the pages reuse its top-3k); may be NULL if n_sample == 0.
 *           The first kernels of the call consume it, so it may overlap
 *           out_idx (a decode loop can keep its last results in one ring)
 *  out_idx  [T, topk] int32 result; -1 padded
 *  out_score[T, topk] fp32 scores of out_idx (NaN where padded), or NULL
 *  ws       workspace of ws_bytes >= litetopk_workspace_bytes(LTK_KIND_SCORE_SELECT, ...)
 *  stats    optional device counters, or NULL
 */
int litetopk_score_select(const void* q, const float* q_scale, const void* k, const float* k_scale,
                          const float* w, const int32_t* pos, int32_t T, int32_t H, int32_t D,
                          int64_t L, int32_t dtype, int32_t topk, const int32_t* sample,
                          int32_t n_sample, int32_t* out_idx, float* out_score, void* ws,
                          size_t ws_bytes, const ltk_opts* opts, ltk_stats* stats, void* stream);

/* litetopk_score_select for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops such as decode steps,
 * harnesses that forbid hipMalloc): the same arguments, checks, kernels and
 * results, without a workspace argument.  The workspace is a static device
 * array of the library, 96 MiB per GPU (held by each GPU the library runs on
 * until the process ends), shared by every call of this entry point on that
 * GPU: calls that may overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.  Each call clears what must
 * start at zero with its own kernels (no memset node).  Returns
 * LTK_EWORKSPACE, before enqueuing anything, when
 * litetopk_workspace_bytes(LTK_KIND_SCORE_SELECT, ...) exceeds 96 MiB: e.g.
 * a decode or speculative-decode step (T <= 8) over up to 1M keys fits, a
 * 1M-context 8,192-query prefill chunk does not.  The first call on a
 * device looks up the array's device address (hipGetSymbolAddress); no
 * call allocates. */
int litetopk_score_select_static(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                 const float* w, const int32_t* pos, int32_t T, int32_t H, int32_t D,
                                 int64_t L, int32_t dtype, int32_t topk, const int32_t* sample,
                                 int32_t n_sample, int32_t* out_idx, float* out_score,
                                 const ltk_opts* opts, ltk_stats* stats, void* stream);

/* Fused inner-product retrieval top-k (LiteTopK pages: the same primitive
 * serves vector retrieval; "Large-scale retrieval", k from 1,024).
 *
 *  q [T, D] queries, db [N, D] database rows, both dtype (LTK_BF16 only),
 *  D in {64, 128, 256, 512, 768}, 1 <= N <= 2^31 - 256; sample [n_sample] database
 *  rows used to estimate the score range (duplicates and out-of-range
 *  entries ignored).  opts->l_splits sets the number of database splits
 *  (LTK_EINVAL if a split would hold more than 2^26 rows).
 *  Other arguments as above.
 */
int litetopk_retrieve(const void* q, const void* db, int32_t T, int32_t D, int64_t N, int32_t dtype,
                      int32_t topk, const int32_t* sample, int32_t n_sample, int32_t* out_idx,
                      float* out_score, void* ws, size_t ws_bytes, const ltk_opts* opts,
                      ltk_stats* stats, void* stream);

/* Unfused comparison path (LiteTopK pages, "Problem statement": the
 * decoupled pipeline writes the full score matrix to device memory, then
 * radix-selects each row, reading the matrix several times).  Same
 * arguments and result as litetopk_score_select without the sample; the
 * workspace holds the T x L fp32 score matrix (and, for fp8, the per-query
 * linear-term operands that every fp8 pass shares). */
int litetopk_unfused_score_select(const void* q, const float* q_scale, const void* k,
                                  const float* k_scale, const float* w, const int32_t* pos,
                                  int32_t T, int32_t H, int32_t D, int64_t L, int32_t dtype,
                                  int32_t topk, int32_t* out_idx, float* out_score, void* ws,
                                  size_t ws_bytes, void* stream);

/* Unfused comparison path of retrieval (the same decoupled pipeline as
 * litetopk_unfused_score_select, for the inner-product score): the T x N
 * fp32 score matrix is written to the workspace, then each row is
 * radix-selected.  Arguments and result as litetopk_retrieve without the
 * sample and statistics; opts may set sorted_output and l_splits (others are
 * ignored).  ws_bytes >= litetopk_workspace_bytes(LTK_KIND_UNFUSED_RETRIEVE,
 * T, 1, D, N, topk, 0, dtype, NULL) = 4 T N bytes rounded up to 256 (33 GB
 * for 1,024 queries over 8M rows).  The scores are bit-identical to the
 * fused path's (same products in the same order). */
int litetopk_unfused_retrieve(const void* q, const void* db, int32_t T, int32_t D, int64_t N,
                              int32_t dtype, int32_t topk, int32_t* out_idx, float* out_score,
                              void* ws, size_t ws_bytes, const ltk_opts* opts, void* stream);

/* Sample for the next chunk (LiteTopK pages, "Sampling": the previous
 * chunk's top-3k tokens are reused as the next chunk's sample).  Ranks the
 * keys 0..L-1 by how many rows of prev_idx [T, topk] (int32, -1 entries
 * ignored) selected them, ties to the lower index, and writes the first
 * n_sample of them to out_sample [n_sample] (int32), in no particular order.
 * ws_bytes >= litetopk_workspace_bytes(LTK_KIND_NEXT_SAMPLE, 0, 0, 0, L, 1,
 * 0, 0, NULL): the key counts, a histogram of the count values and a few
 * words per workgroup.  Returns LTK_EWORKSPACE below that, and LTK_EINVAL
 * unless T >= 0, topk >= 1, 1 <= L <= 2^31 - 256 and 0 <= n_sample <= L. */
int litetopk_next_sample(const int32_t* prev_idx, int32_t T, int32_t topk, int64_t L, int32_t n_sample,
                         int32_t* out_sample, void* ws, size_t ws_bytes, void* stream);

/* LiteDSA packing (LiteTopK pages, arXiv abstract: the candidates that
 * neighbouring query tokens share are packed into one key/value list for
 * joint attention, and per-query masks keep each token's own top-k
 * membership).  Groups are the rows [g*group, (g+1)*group) of idx, the last
 * one possibly shorter; ngroups = ceil(T / group), cap = group * topk.
 *
 *  idx     [T, topk] int32 selected keys per query (a litetopk_score_select
 *          result; entries outside [0, L) are not keys)
 *  group   1..32 queries per group; group * topk <= 32768; L <= 2^26
 *  shared  [ngroups, cap] int32 out: per group its distinct keys in
 *          ascending order, then -1
 *  masks   [ngroups, cap] uint32 out: bit i of masks[g][j] is set when row
 *          g*group + i selected shared[g][j]; 0 past the list
 *  lens    [ngroups] int32 out: length of each group's list
 * Returns LTK_EUNSUPPORTED past the size limits above. */
int litetopk_dsa_pack(const int32_t* idx, int32_t T, int32_t topk, int64_t L, int32_t group,
                      int32_t* shared, uint32_t* masks, int32_t* lens, void* stream);

/* Gathers each group's shared key/value rows contiguously:
 * out[g][j] = kv[shared[g][j]] for j < lens[g] (rows of row_bytes, a multiple
 * of 16; kv [L, row_bytes] and out [ngroups, cap, row_bytes] 16-byte
 * aligned).  Rows past lens[g] are left untouched; an entry outside [0, L)
 * gives a zero row. */
int litetopk_dsa_gather(const void* kv, int64_t L, int64_t row_bytes, const int32_t* shared,
                        const int32_t* lens, int32_t ngroups, int32_t cap, void* out, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* litetopk_strerror(int status);

/* LTK_OK if the current HIP device is a gfx950, LTK_EUNSUPPORTED otherwise,
 * LTK_EHIP if there is no usable device. */
int litetopk_device_check(void);

#ifdef __cplusplus
}
#endif

#endif /* LITETOPK_H */
