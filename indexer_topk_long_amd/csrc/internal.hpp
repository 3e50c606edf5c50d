// internal.hpp -- host/device shared definitions of the library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "litetopk.h"
#include "split.hpp"

namespace ltk {

constexpr int kQPG = 8;              // queries per workgroup (4 waves x 2 queries)
constexpr int kStage = 128;          // staging entries per query in LDS (>= 64 + 32)
constexpr int kFlush = 64;           // default write-back batch (one wave64 of 8-byte entries)
constexpr int kDefaultBins = 256;
constexpr int kMaxBins = 1024;
constexpr int64_t kDefaultCcap = 16384;
constexpr int64_t kDefaultCcapRetrieve = 262144;
// Retrieval candidates per query by default: every database split keeps a
// fixed slice of the buffer (1,024 entries at 256 splits), and the total grows
// with k (a random 3k-row sample lets some 15k rows per query through at
// k = 1,024, 65k at k = 8,192; 512-entry slices overflowed at k = 2,048).
inline int64_t retrieve_default_ccap(int32_t topk) {
    const int64_t c = (int64_t)64 * topk;
    return c > kDefaultCcapRetrieve ? c : kDefaultCcapRetrieve;
}
constexpr int kMaxSortedK = 8192;
constexpr size_t kMaxLds = 160 * 1024;   // LDS one gfx950 workgroup may allocate

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Sample de-duplication: a bitmap over the keys, cut into chunks of
// 2^chunk_log2 words (at least 1024, doubled until there are at most 2048
// chunks); a counting pass popcounts every chunk so that the chunks compact
// in parallel.
inline int sample_chunk_log2(int64_t L) {
    const int64_t nw = (L + 31) / 32;
    int lg = 10;
    while ((nw + ((int64_t)1 << lg) - 1) >> lg > 2048) ++lg;
    return lg;
}
inline int sample_chunks(int64_t L) {
    const int lg = sample_chunk_log2(L);
    return (int)(((L + 31) / 32 + ((int64_t)1 << lg) - 1) >> lg);
}

// Workspace of one fused call.  The [zero_begin, zero_end) range is cleared
// by the first kernel of every call.
struct WsLayout {
    size_t tail, flags, thrf, ovfc, hist, bitmap, ccount, zero_begin, zero_end;
    size_t nu, meta, sample_u, sscore, qlin, qinv, ovfl, sgk, sgs, sgp, cand, total;
};

// Per-query linear-term operands of the fp8 score (four fp8 parts of D bytes
// and one fp32 scale per query; lin_d = D for fp8 inputs, else 0).
inline size_t qlin_bytes(int32_t T, int lin_d) { return (size_t)T * 4 * (size_t)lin_d; }

// Samples of at most this many entries are de-duplicated in one workgroup's
// LDS hash table, with no key bitmap (the bitmap and its chunk counts, the
// tail of the cleared range, then stay untouched).
constexpr int kHashSampleMax = 16384;

// Calls of at most kFrontMaxT queries whose sample has at most kFrontSampleMax
// slots run the sample steps (de-duplication, linear-term operands, scores) as
// one launch of front_parts workgroups per query, each taking the sample keys
// of one class (a hash of the key); score row t of sscore then holds
// one score per distinct key the query sees, at the slot of one of its
// entries, and NaN at every other slot.  One more launch turns the rows into
// statistics.  A workgroup's LDS holds the list of its keys (n_slots 64-bit
// entries) and a hash table of 2^front_log2_slots keys (more than the sample,
// as one class may hold every key).
constexpr int kFrontMaxT = 8;
// Calls of at least this many queries (prefill chunks) score their sample
// with the scan itself: the distinct sample keys' rows are copied into a
// contiguous array, which the scan's full-score form then covers.
constexpr int kSampleScanMinT = 2048;
inline bool sample_by_scan(int32_t T, int32_t n_slots) { return T >= kSampleScanMinT && n_slots > 0; }
inline size_t dtype_bytes(int dtype) { return dtype == 0 ? 4 : dtype == 1 ? 2 : 1; }   // fp32, bf16, fp8
constexpr int kFrontSampleMax = 6144;
// (fp32 queries of 128 dimensions in two head blocks leave that kernel too
// few registers: those calls keep the separate launches)
inline bool front_fits(int dtype, int D, int HB) { return !(dtype == 0 && D == 128 && HB == 2); }
inline bool front_path(int32_t T, int32_t n_slots, int dtype, int D, int H) {
    return T <= kFrontMaxT && n_slots <= kFrontSampleMax && front_fits(dtype, D, (H + 31) / 32);
}
inline int front_log2_parts(int32_t n_slots) {   // about 512 sample entries per workgroup, at most 16
    int lg = 0;
    while (lg < 4 && ((int64_t)512 << lg) < n_slots) ++lg;
    return lg;
}
inline int front_parts(int32_t n_slots) { return 1 << front_log2_parts(n_slots); }
inline int front_log2_slots(int32_t n_slots) {
    int lg = 10;
    while ((1 << lg) <= n_slots) ++lg;
    return lg;
}
inline size_t front_lds_bytes(int32_t n_slots) {
    return (size_t)n_slots * 8 + ((size_t)4 << front_log2_slots(n_slots));
}

// Sample slots of a call: the caller's sample size, or, with no sample,
// min(3 k, L, 16384) evenly spaced causal keys drawn by the library (the
// pages' sample is 3 k keys of the previous chunk's result).
inline int32_t sample_slots(int32_t n_sample, int32_t topk, int64_t L) {
    if (n_sample > 0) return n_sample;
    int64_t n = (int64_t)3 * topk;
    if (n > L) n = L;
    if (n > kHashSampleMax) n = kHashSampleMax;
    return (int32_t)n;
}

// hist_words: 32-bit counters of the histograms shared across workgroups
// (retrieval: T x (nbins + super-bins) + T x splits; indexer: T x nbins when
// its splits share thresholds, else 0).
inline WsLayout ws_layout(int32_t T, int64_t L, int32_t n_sample, int64_t ccap, size_t hist_words = 0,
                          int lin_d = 0, size_t gather_row_bytes = 0) {
    WsLayout w{};
    size_t o = 0;
    // cleared by the sample preparation of every call
    w.zero_begin = o;
    w.tail = o;   o = align_up(o + (size_t)T * 4, 256);
    w.flags = o;  o = align_up(o + (size_t)T * 4, 256);
    w.thrf = o;   o = align_up(o + (size_t)T * 4, 256);
    w.ovfc = o;   o = align_up(o + 64, 256);
    w.hist = o;   o = align_up(o + hist_words * 4, 256);
    w.bitmap = o; o = align_up(o + (size_t)((L + 31) / 32) * 4, 256);
    w.ccount = o; o = align_up(o + (size_t)sample_chunks(L) * 4, 256);
    w.zero_end = o;
    // written whole by the kernel that produces it (the de-duplicated sample
    // count is written by the sample preparation, which clears the range
    // above in other workgroups of the same launch)
    w.nu = o;       o = align_up(o + 64, 256);
    w.meta = o;     o = align_up(o + (size_t)T * sizeof(int32_t) * 4, 256);
    w.sample_u = o; o = align_up(o + (size_t)(n_sample > 0 ? n_sample : 1) * 4, 256);
    w.sscore = o;   o = align_up(o + (size_t)T * (size_t)(n_sample > 0 ? n_sample : 1) * 4, 256);
    w.qlin = o;     o = align_up(o + qlin_bytes(T, lin_d), 256);
    w.qinv = o;     o = align_up(o + (lin_d ? (size_t)T * 4 : 0), 256);
    w.ovfl = o;     o = align_up(o + (size_t)T * 4, 256);
    // the sample pass at prefill shape: the sample's key rows, their scales
    // and one causal bound per query, for the scan (gather_row_bytes = 0: none)
    const size_t ng = gather_row_bytes ? (size_t)(n_sample > 0 ? n_sample : 1) : 0;
    w.sgk = o;      o = align_up(o + ng * gather_row_bytes, 256);
    w.sgs = o;      o = align_up(o + ng * 4, 256);
    w.sgp = o;      o = align_up(o + (gather_row_bytes ? (size_t)T * 4 : 0), 256);
    w.cand = o;     o = align_up(o + (size_t)T * (size_t)ccap * 8, 256);
    w.total = o;
    return w;
}

// Everything a kernel of the fused indexer path needs.
struct IdxArgs {
    const uint8_t* q;        // [T, H, D]
    const float* q_scale;    // [T] (fp8) or null
    const uint8_t* k;        // [L, D]
    const float* k_scale;    // [L] (fp8) or null
    const float* w;          // [T, H]
    const int32_t* pos;      // [T]
    int T, H, L, topk, nbins;
    int n_sample;            // row stride of sscore
    int n_splits;            // key-range splits per query group (scan, unfused score)
    int s_splits;            // sample splits per query group (sample pass)
    int refresh_every;       // <= 0: never
    int sorted;
    int flush;               // candidates per write-back batch (32 or 64)
    int pass;                // 0: one pass (an overflowed row takes the exact fallback);
                             // 1: first pass of two (overflowed rows are listed for a rescan);
                             // 2: the rescan of the listed rows
    int64_t ccap;
    int front_parts;         // workgroups per query of the one-launch sample steps, or 0
    // workspace
    uint32_t* tail;
    uint32_t* flags;
    uint32_t* nu;
    uint32_t* bitmap;
    uint32_t* hist_g;        // [T][nbins] threshold histograms shared by the key splits, or null
    void* meta;              // Meta[T]
    int32_t* sample_u;
    float* sscore;
    uint2* cand;
    int* thr_fin;            // [T] final threshold bin of the first pass (max over the query's waves)
    int* ovf_list;           // [T] rows whose first-pass buffer overflowed
    uint32_t* ovf_count;     // number of them
    uint8_t* qlin;           // fp8: [T][4][D] parts of each query's q''/2 (linear term), else null
    float* qinv;             // fp8: [T] 1/S of those parts
    uint8_t* sg_k;           // sample pass by the scan: [n_sample][D] the sample's key rows, else null
    float* sg_scale;         // and their scales (fp8)
    int32_t* sg_pos;         // [T] n_sample - 1 (every row visible to every query)
    // outputs
    int32_t* out_idx;
    float* out_score;
    ltk_stats* stats;
    float* S;                // unfused: [T, L] score matrix
    hipEvent_t ev_scan_start, ev_scan_stop;   // optional, recorded around the scan launch
};

// Waves per workgroup of the retrieval scan (32 queries each, two waves per
// SIMD): 8, or 4 when a tile of 32 rows is fewer than 8 wave-wide 1 KB loads
// (D = 64).
constexpr int retr_waves(int D) { return (D / 16) % 8 == 0 ? 8 : 4; }
constexpr int retr_group_queries(int D) { return retr_waves(D) * 32; }

// Everything a kernel of the fused retrieval path needs.
struct RetrArgs {
    const uint8_t* q;        // [T, D] bf16
    const uint8_t* db;       // [N, D] bf16
    int T, N, topk, nbins, nsuper;
    int n_sample;            // row stride of sscore
    int n_splits, n_qgroups; // database splits x query groups (retr_group_queries(D) queries)
    int sorted;
    int64_t ccap;
    uint32_t* tail;
    uint32_t* flags;
    const uint32_t* nu;
    const int32_t* sample_u;
    float* sscore;
    void* meta;              // Meta[T]
    uint2* cand;
    uint32_t* hist_g;        // [T][nbins] shared fine histograms
    uint32_t* hist_c;        // [T][nsuper] shared super-bin histograms
    uint32_t* seg_cnt;       // [T][n_splits] candidates each split found (zeroed before the scan)
    int64_t cap_s;           // candidate slots per (query, split): ccap / n_splits
    float* S;                // unfused: [T, N] score matrix
    int32_t* out_idx;
    float* out_score;
    hipEvent_t ev_scan_start, ev_scan_stop;   // optional, recorded around the scan launch
};

// Host launchers (return hipSuccess or the first launch error).
hipError_t launch_prepare_sample(const IdxArgs& a, const int32_t* sample, int n_sample, const WsLayout& lay,
                                 uint8_t* ws, hipStream_t st);   // n_sample == 0: the library's own (a.n_sample keys)
// The sample of a call that takes the one-launch sample steps, and the
// workspace range its launch clears.
struct FrontArgs {
    const int32_t* sample;
    int n;
    uint32_t* zero;
    size_t n_zero;
};
hipError_t launch_indexer_fused(int dt, int D, int HB, const IdxArgs& a, const FrontArgs* front, hipStream_t st);
hipError_t launch_indexer_unfused(int dt, int D, int HB, const IdxArgs& a, hipStream_t st);
// Unfused workspace: the T x L fp32 score matrix, then (fp8) the linear-term parts.
inline size_t unfused_matrix_bytes(int32_t T, int64_t L) { return align_up((size_t)T * (size_t)L * 4, 256); }
inline size_t unfused_ws_bytes(int32_t T, int64_t L, int lin_d) {
    return unfused_matrix_bytes(T, L) + align_up(qlin_bytes(T, lin_d), 256) + align_up(lin_d ? (size_t)T * 4 : 0, 256);
}
hipError_t launch_sample_stats(const IdxArgs& a, hipStream_t st);
hipError_t launch_finalize(const IdxArgs& a, hipStream_t st);
hipError_t launch_retrieve(int D, const RetrArgs& a, const IdxArgs& fin, hipStream_t st);
// Unfused retrieval: the full score matrix (a.S), then the row select of sel
// (sel.S = a.S, sel.pos = null: every row is valid).
hipError_t launch_retrieve_unfused(int D, const RetrArgs& a, const IdxArgs& sel, hipStream_t st);
hipError_t launch_unfused_select(const IdxArgs& a, hipStream_t st);
constexpr int kDsaMaxEntries = 32768;   // G x k selections packed by one workgroup (LDS)
constexpr int64_t kDsaMaxKeys = (int64_t)1 << 26;   // key << 5 | row fits 31 bits
hipError_t launch_dsa_pack(const int32_t* idx, int T, int k, int L, int G, int32_t* shared, uint32_t* masks,
                           int32_t* lens, hipStream_t st);
hipError_t launch_dsa_gather(const void* kv, int L, size_t row_bytes, const int32_t* shared, const int32_t* lens,
                             int ngroups, int cap, void* out, hipStream_t st);
// Workspace of litetopk_next_sample, in 32-bit words: the key counts [L],
// a histogram of count values [kNsBins], a header, and the count of ties in
// each workgroup's key range [at most kNsBlocks].
constexpr int kNsBins = 16384;
constexpr int kNsBlocks = 1024;
struct NsLayout {
    size_t hist, hdr, ties, words;
};
inline NsLayout ns_layout(int64_t L) {
    NsLayout w{};
    w.hist = (size_t)((L + 63) / 64 * 64);
    w.hdr = w.hist + kNsBins;
    w.ties = w.hdr + 64;
    w.words = w.ties + kNsBlocks;
    return w;
}
// keys per workgroup: a multiple of 256, at least 4,096, at most kNsBlocks workgroups
inline int ns_chunk(int64_t L) {
    int64_t c = (L + kNsBlocks - 1) / kNsBlocks;
    c = (c + 255) / 256 * 256;
    return (int)(c < 4096 ? 4096 : c);
}
hipError_t launch_next_sample(const int32_t* prev_idx, size_t n, int L, int n_sample, int32_t* out,
                              uint32_t* counts, hipStream_t st);

}  // namespace ltk
