// api.hip -- the C ABI declared in include/litetopk.h: argument checks,
// workspace carving and kernel launches on the caller's stream.
#include <algorithm>
#include <atomic>
#include <string.h>

#include "internal.hpp"

namespace ltk {

static std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, -1 other

// Workspace of litetopk_score_select_static: a file-scope device array (each
// GPU the library runs on holds its own copy until the process ends).  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever passed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
static std::atomic<void*> g_scratch[64];

// Device address of this device's `scratch` (looked up on the first call on
// the device, with that device current).
static int static_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LTK_EHIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LTK_EHIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return LTK_OK;
}

static int device_check() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LTK_EHIP;
    if (dev >= 0 && dev < 64) {
        const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (c != 0) return c > 0 ? LTK_OK : LTK_EUNSUPPORTED;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LTK_EHIP;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? LTK_OK : LTK_EUNSUPPORTED;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Opts {
    int nbins, refresh_every, l_splits, sorted, shared, flush;
    int64_t ccap;
    bool ccap_given;
    hipEvent_t ev0, ev1;
};

static int resolve_opts(const ltk_opts* o, int64_t default_ccap, Opts& r) {
    r.nbins = kDefaultBins;
    r.refresh_every = 1;
    r.l_splits = 0;
    r.sorted = 0;
    r.shared = 0;
    r.flush = kFlush;
    r.ccap = default_ccap;
    r.ccap_given = false;
    r.ev0 = r.ev1 = nullptr;
    if (!o) return LTK_OK;
    r.ev0 = static_cast<hipEvent_t>(o->scan_event_start);
    r.ev1 = static_cast<hipEvent_t>(o->scan_event_stop);
    if (o->nbins < 0 || o->nbins > kMaxBins) return LTK_EINVAL;   // LDS holds 16 x nbins counters
    if (o->nbins) r.nbins = o->nbins;
    if (o->refresh_every) r.refresh_every = o->refresh_every;   // negative: never
    if (o->l_splits < 0 || o->l_splits > 4096) return LTK_EINVAL;
    r.l_splits = o->l_splits;
    r.sorted = o->sorted_output != 0;
    if (o->cand_capacity < 0 || o->cand_capacity > (int64_t)1 << 31) return LTK_EINVAL;
    if (o->cand_capacity) r.ccap = o->cand_capacity;
    r.ccap_given = o->cand_capacity != 0;
    r.shared = o->shared_threshold;
    if (o->flush_batch != 0 && o->flush_batch != 32 && o->flush_batch != 64) return LTK_EINVAL;
    if (o->flush_batch) r.flush = o->flush_batch;
    return LTK_OK;
}

// Head blocks of 32 on the MFMA M dimension.
static int head_blocks(int H) { return (H + 31) / 32; }

static int check_indexer_sizes(int32_t T, int32_t H, int32_t D, int64_t L, int32_t dtype, int32_t topk) {
    if (T < 0 || L < 1 || L > (int64_t)0x7fffff00 || topk < 1 || topk > 65536) return LTK_EINVAL;
    if (dtype < LTK_F32 || dtype > LTK_FP8_E4M3FN) return LTK_EINVAL;
    if (H < 1 || H > 64 || (D != 64 && D != 128)) return LTK_EUNSUPPORTED;
    return LTK_OK;
}

// Key splits of the fused scan: about 2048 workgroups of at least 16K keys;
// below one workgroup per CU (decode: a handful of queries), splits go down to
// 4K keys so that all 256 CUs stream the context.
static int auto_splits(int nqg, int64_t L, int requested) {
    if (requested > 0) return requested;
    int s = 1;
    while ((int64_t)nqg * s < 2048 && L / (s * 2) >= ((int64_t)nqg * s < 256 ? 4096 : 16384)) s *= 2;
    return s;
}

// Queries per scan workgroup: 8 waves x 1 query.
static int scan_qpg(int) { return 8; }

// Splits from which the fused scan shares one threshold histogram per query
// across its splits (the decode shape: few queries, hundreds of splits, no
// split holding k passing keys on its own).
constexpr int kSharedSplitMin = 16;

// What a fused indexer call will launch, fixed by its sizes and options
// alone, so that litetopk_workspace_bytes and the call agree.
struct IdxPlan {
    int n_splits;
    bool shared;     // shared per-query histograms in the workspace
    int64_t ccap;    // candidate slots per query
};
static IdxPlan indexer_plan(int32_t T, int64_t L, int32_t dtype, const Opts& o) {
    IdxPlan p;
    p.n_splits = auto_splits((T + scan_qpg(dtype) - 1) / scan_qpg(dtype), L, o.l_splits);
    p.shared = o.shared > 0 || (o.shared == 0 && p.n_splits >= kSharedSplitMin);
    // every split may write a few batches before the shared counts reach k; a
    // few queries over a context whose every key fits (T x L x 8 B <= 512 MiB)
    // get room for all of them, so no decode step ever overflows
    p.ccap = o.ccap;
    if (p.shared && !o.ccap_given)
        p.ccap = ((int64_t)T * L * 8 <= ((int64_t)512 << 20)) ? std::max<int64_t>(o.ccap, L)
                                                            : std::max<int64_t>(o.ccap, (int64_t)p.n_splits * 256);
    return p;
}

// Shared retrieval histograms: nbins fine counters + one per 16-bin super-bin, per query.
// Retrieval database splits: the caller's count, else about 2048 workgroups
// (4 waves x 64 queries each) of at least 2048 rows.
// A split holds at most 2^26 rows (the scan packs a row's offset in its
// split into 26 bits); a caller's count that leaves more is rejected.
constexpr int64_t kRetrMaxSplitRows = (int64_t)1 << 26;
static int retr_splits(int32_t T, int32_t D, int64_t N, int l_splits) {
    if (l_splits > 0) return l_splits;
    const int64_t nqg = (T + retr_group_queries(D) - 1) / retr_group_queries(D);
    int ns = 1;
    while ((nqg * ns < 2048 && N / ((int64_t)ns * 2) >= 2048) || (N + ns - 1) / ns > kRetrMaxSplitRows) ns *= 2;
    return ns;
}
// Zeroed shared counters of the retrieval scan: fine and super-bin
// histograms, then the per-(query, split) candidate counts.
static size_t retr_hist_words(int32_t T, int nbins, int ns) {
    return (size_t)T * (size_t)(nbins + (nbins + 15) / 16) + (size_t)T * (size_t)ns;
}

}  // namespace ltk

using namespace ltk;

extern "C" {

const char* litetopk_strerror(int status) {
    switch (status) {
        case LTK_OK: return "ok";
        case LTK_EINVAL: return "invalid argument";
        case LTK_EUNSUPPORTED: return "unsupported shape, dtype or device (gfx950 only)";
        case LTK_EWORKSPACE: return "workspace too small";
        case LTK_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int litetopk_device_check(void) { return device_check(); }

int litetopk_dsa_pack(const int32_t* idx, int32_t T, int32_t topk, int64_t L, int32_t group, int32_t* shared,
                      uint32_t* masks, int32_t* lens, void* stream) {
    if (T < 0 || topk < 1 || group < 1 || group > 32 || L < 1) return LTK_EINVAL;
    if (L > kDsaMaxKeys || (int64_t)group * topk > kDsaMaxEntries) return LTK_EUNSUPPORTED;
    if (T == 0) return LTK_OK;
    if (!idx || !shared || !masks || !lens) return LTK_EINVAL;
    int st;
    if ((st = device_check()) != LTK_OK) return st;
    if (launch_dsa_pack(idx, T, topk, (int)L, group, shared, masks, lens, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return LTK_EHIP;
    return LTK_OK;
}

int litetopk_dsa_gather(const void* kv, int64_t L, int64_t row_bytes, const int32_t* shared, const int32_t* lens,
                        int32_t ngroups, int32_t cap, void* out, void* stream) {
    if (L < 1 || L > (int64_t)0x7fffffff || row_bytes < 16 || row_bytes % 16 != 0 || ngroups < 0 || cap < 1)
        return LTK_EINVAL;
    if (ngroups == 0) return LTK_OK;
    if (!kv || !shared || !lens || !out || !aligned16(kv) || !aligned16(out)) return LTK_EINVAL;
    int st;
    if ((st = device_check()) != LTK_OK) return st;
    if (launch_dsa_gather(kv, (int)L, (size_t)row_bytes, shared, lens, ngroups, cap, out,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
        return LTK_EHIP;
    return LTK_OK;
}

size_t litetopk_workspace_bytes(int32_t kind, int32_t T, int32_t H, int32_t D, int64_t L, int32_t topk,
                                int32_t n_sample, int32_t dtype, const ltk_opts* opts) {
    if (kind == LTK_KIND_UNFUSED) {
        if (T < 0 || L < 1) return 0;
        return unfused_ws_bytes(T, L, dtype == LTK_FP8_E4M3FN ? D : 0);
    }
    if (kind == LTK_KIND_UNFUSED_RETRIEVE) {
        if (T < 0 || L < 1) return 0;
        return unfused_matrix_bytes(T, L);
    }
    if (kind == LTK_KIND_NEXT_SAMPLE) {
        if (L < 1 || L > (int64_t)0x7fffff00) return 0;
        return ns_layout(L).words * 4;
    }
    if (kind != LTK_KIND_SCORE_SELECT && kind != LTK_KIND_RETRIEVE) return 0;
    if (T < 0 || L < 1 || topk < 1 || n_sample < 0) return 0;
    Opts o;
    if (resolve_opts(opts, kind == LTK_KIND_RETRIEVE ? retrieve_default_ccap(topk) : kDefaultCcap, o) != LTK_OK)
        return 0;
    if (kind == LTK_KIND_RETRIEVE)
        return ws_layout(T, L, sample_slots(n_sample, topk, L), o.ccap,
                         retr_hist_words(T, o.nbins, retr_splits(T, D, L, o.l_splits))).total;
    (void)H;
    const IdxPlan p = indexer_plan(T, L, dtype, o);
    const int32_t n_slots = sample_slots(n_sample, topk, L);
    const size_t grb = sample_by_scan(T, n_slots) && !front_path(T, n_slots, dtype, D, H) ? (size_t)D * dtype_bytes(dtype) : 0;
    return ws_layout(T, L, n_slots, p.ccap, p.shared ? (size_t)T * o.nbins : 0, dtype == LTK_FP8_E4M3FN ? D : 0, grb).total;
}

int litetopk_score_select(const void* q, const float* q_scale, const void* k, const float* k_scale, const float* w,
                          const int32_t* pos, int32_t T, int32_t H, int32_t D, int64_t L, int32_t dtype,
                          int32_t topk, const int32_t* sample, int32_t n_sample, int32_t* out_idx, float* out_score,
                          void* ws, size_t ws_bytes, const ltk_opts* opts, ltk_stats* stats, void* stream) {
    int st = check_indexer_sizes(T, H, D, L, dtype, topk);
    if (st != LTK_OK) return st;
    if (n_sample < 0 || (n_sample > 0 && !sample)) return LTK_EINVAL;
    if (T > 0 && (!q || !k || !w || !pos || !out_idx || !ws)) return LTK_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(ws)) return LTK_EINVAL;
    const bool fp8 = dtype == LTK_FP8_E4M3FN;
    if (fp8 && ((T > 0 && !q_scale) || !k_scale)) return LTK_EINVAL;   // no queries: no query scales
    if (!fp8 && (q_scale || k_scale)) return LTK_EINVAL;
    Opts o;
    if ((st = resolve_opts(opts, kDefaultCcap, o)) != LTK_OK) return st;
    if (o.sorted && topk > kMaxSortedK) return LTK_EINVAL;
    const IdxPlan plan = indexer_plan(T, L, dtype, o);
    const int32_t n_slots = sample_slots(n_sample, topk, L);
    // few queries and a small sample: the sample steps take one launch
    const bool front = front_path(T, n_slots, dtype, D, H);
    const size_t grb = sample_by_scan(T, n_slots) && !front_path(T, n_slots, dtype, D, H) ? (size_t)D * dtype_bytes(dtype) : 0;
    const WsLayout lay = ws_layout(T, L, n_slots, plan.ccap, plan.shared ? (size_t)T * o.nbins : 0, fp8 ? D : 0, grb);
    if (ws_bytes < lay.total) return LTK_EWORKSPACE;
    if (T == 0) return LTK_OK;
    if ((st = device_check()) != LTK_OK) return st;

    uint8_t* wsb = static_cast<uint8_t*>(ws);
    IdxArgs a{};
    a.q = static_cast<const uint8_t*>(q);
    a.q_scale = q_scale;
    a.k = static_cast<const uint8_t*>(k);
    a.k_scale = k_scale;
    a.w = w;
    a.pos = pos;
    a.T = T;
    a.H = H;
    a.L = (int)L;
    a.topk = topk;
    a.nbins = o.nbins;
    a.n_sample = n_slots > 0 ? n_slots : 1;
    const int nqg = (T + kQPG - 1) / kQPG;
    a.n_splits = plan.n_splits;
    a.s_splits = 1;
    // sample splits: about 512 workgroups of >= 8 key blocks, down to one block
    // each while the queries alone fill fewer than 128 workgroups (decode)
    while (nqg * a.s_splits < 512 && (n_slots / 32) / (a.s_splits * 2) >= (nqg * a.s_splits < 128 ? 1 : 8))
        a.s_splits *= 2;
    a.refresh_every = o.refresh_every;
    a.sorted = o.sorted;
    a.flush = o.flush;
    a.ccap = plan.ccap;
    a.tail = reinterpret_cast<uint32_t*>(wsb + lay.tail);
    a.flags = reinterpret_cast<uint32_t*>(wsb + lay.flags);
    a.nu = reinterpret_cast<uint32_t*>(wsb + lay.nu);
    a.bitmap = reinterpret_cast<uint32_t*>(wsb + lay.bitmap);
    a.hist_g = plan.shared ? reinterpret_cast<uint32_t*>(wsb + lay.hist) : nullptr;
    a.meta = wsb + lay.meta;
    a.sample_u = reinterpret_cast<int32_t*>(wsb + lay.sample_u);
    a.sscore = reinterpret_cast<float*>(wsb + lay.sscore);
    a.front_parts = front ? front_parts(n_slots) : 0;
    a.sg_k = grb ? wsb + lay.sgk : nullptr;
    a.sg_scale = grb ? reinterpret_cast<float*>(wsb + lay.sgs) : nullptr;
    a.sg_pos = grb ? reinterpret_cast<int32_t*>(wsb + lay.sgp) : nullptr;
    a.cand = reinterpret_cast<uint2*>(wsb + lay.cand);
    a.thr_fin = reinterpret_cast<int*>(wsb + lay.thrf);
    a.ovf_list = reinterpret_cast<int*>(wsb + lay.ovfl);
    a.ovf_count = reinterpret_cast<uint32_t*>(wsb + lay.ovfc);
    // a row can overflow only when its buffer cannot hold every key: then the
    // overflowed rows are rescanned once, gated at their first pass's final
    // threshold bin
    a.pass = (plan.ccap < L) ? 1 : 0;
    a.qlin = fp8 ? wsb + lay.qlin : nullptr;
    a.qinv = fp8 ? reinterpret_cast<float*>(wsb + lay.qinv) : nullptr;
    a.out_idx = out_idx;
    a.out_score = out_score;
    a.stats = stats;
    a.S = nullptr;
    a.ev_scan_start = o.ev0;
    a.ev_scan_stop = o.ev1;

    hipStream_t s = static_cast<hipStream_t>(stream);
    FrontArgs fr{};
    if (front) {
        fr.sample = sample;
        fr.n = n_sample;
        fr.zero = reinterpret_cast<uint32_t*>(wsb + lay.zero_begin);
        fr.n_zero = (lay.bitmap - lay.zero_begin) / 4;   // the bitmap is not used
    } else if (launch_prepare_sample(a, sample, n_sample, lay, wsb, s) != hipSuccess) {
        return LTK_EHIP;
    }
    if (launch_indexer_fused(dtype, D, head_blocks(H), a, front ? &fr : nullptr, s) != hipSuccess) return LTK_EHIP;
    return LTK_OK;
}

int litetopk_score_select_static(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                 const float* w, const int32_t* pos, int32_t T, int32_t H, int32_t D, int64_t L,
                                 int32_t dtype, int32_t topk, const int32_t* sample, int32_t n_sample,
                                 int32_t* out_idx, float* out_score, const ltk_opts* opts, ltk_stats* stats,
                                 void* stream) {
    // the same checks and kernels as litetopk_score_select, on the static
    // workspace: a call that needs more than it holds is rejected before
    // anything is enqueued
    const size_t need = litetopk_workspace_bytes(LTK_KIND_SCORE_SELECT, T, H, D, L, topk, n_sample, dtype, opts);
    if (need == 0) {
        const int st = check_indexer_sizes(T, H, D, L, dtype, topk);
        return st != LTK_OK ? st : LTK_EINVAL;
    }
    if (need > kStaticScratchBytes) return LTK_EWORKSPACE;
    if (T == 0) {
        // no queries: litetopk_score_select checks the arguments and returns
        // before it touches any workspace (this aligned host word stands in)
        alignas(256) static unsigned char no_work[256];
        return litetopk_score_select(q, q_scale, k, k_scale, w, pos, T, H, D, L, dtype, topk, sample, n_sample,
                                     out_idx, out_score, no_work, need, opts, stats, stream);
    }
    int st = device_check();
    if (st != LTK_OK) return st;
    void* ws = nullptr;
    if ((st = static_scratch(&ws)) != LTK_OK) return st;
    return litetopk_score_select(q, q_scale, k, k_scale, w, pos, T, H, D, L, dtype, topk, sample, n_sample, out_idx,
                                 out_score, ws, kStaticScratchBytes, opts, stats, stream);
}

int litetopk_unfused_score_select(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                  const float* w, const int32_t* pos, int32_t T, int32_t H, int32_t D, int64_t L,
                                  int32_t dtype, int32_t topk, int32_t* out_idx, float* out_score, void* ws,
                                  size_t ws_bytes, void* stream) {
    int st = check_indexer_sizes(T, H, D, L, dtype, topk);
    if (st != LTK_OK) return st;
    if (T > 0 && (!q || !k || !w || !pos || !out_idx || !ws)) return LTK_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(ws)) return LTK_EINVAL;
    const bool fp8 = dtype == LTK_FP8_E4M3FN;
    if (fp8 && ((T > 0 && !q_scale) || !k_scale)) return LTK_EINVAL;   // no queries: no query scales
    if (!fp8 && (q_scale || k_scale)) return LTK_EINVAL;
    if (ws_bytes < unfused_ws_bytes(T, L, fp8 ? D : 0)) return LTK_EWORKSPACE;
    if (T == 0) return LTK_OK;
    if ((st = device_check()) != LTK_OK) return st;
    IdxArgs a{};
    a.q = static_cast<const uint8_t*>(q);
    a.q_scale = q_scale;
    a.k = static_cast<const uint8_t*>(k);
    a.k_scale = k_scale;
    a.w = w;
    a.pos = pos;
    a.T = T;
    a.H = H;
    a.L = (int)L;
    a.topk = topk;
    a.nbins = kDefaultBins;
    const int nqg = (T + kQPG - 1) / kQPG;
    a.n_splits = auto_splits(nqg, L, 0);
    a.out_idx = out_idx;
    a.out_score = out_score;
    a.S = static_cast<float*>(ws);
    if (fp8) {
        uint8_t* wsb = static_cast<uint8_t*>(ws);
        a.qlin = wsb + unfused_matrix_bytes(T, L);
        a.qinv = reinterpret_cast<float*>(a.qlin + align_up(qlin_bytes(T, D), 256));
    }
    if (launch_indexer_unfused(dtype, D, head_blocks(H), a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return LTK_EHIP;
    return LTK_OK;
}

int litetopk_next_sample(const int32_t* prev_idx, int32_t T, int32_t topk, int64_t L, int32_t n_sample,
                         int32_t* out_sample, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || topk < 1 || L < 1 || L > (int64_t)0x7fffff00 || n_sample < 0) return LTK_EINVAL;
    if (n_sample == 0) return LTK_OK;
    if ((T > 0 && !prev_idx) || !out_sample || !ws) return LTK_EINVAL;
    if ((int64_t)n_sample > L) return LTK_EINVAL;
    if (ws_bytes < ns_layout(L).words * 4) return LTK_EWORKSPACE;
    int st = device_check();
    if (st != LTK_OK) return st;
    if (launch_next_sample(prev_idx, (size_t)T * (size_t)topk, (int)L, n_sample, out_sample,
                           static_cast<uint32_t*>(ws), static_cast<hipStream_t>(stream)) != hipSuccess)
        return LTK_EHIP;
    return LTK_OK;
}

int litetopk_unfused_retrieve(const void* q, const void* db, int32_t T, int32_t D, int64_t N, int32_t dtype,
                              int32_t topk, int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                              const ltk_opts* opts, void* stream) {
    if (T < 0 || N < 1 || N > (int64_t)0x7fffff00 || topk < 1 || topk > 65536) return LTK_EINVAL;
    if (dtype != LTK_BF16) return dtype < LTK_F32 || dtype > LTK_FP8_E4M3FN ? LTK_EINVAL : LTK_EUNSUPPORTED;
    if (D != 64 && D != 128 && D != 256 && D != 512 && D != 768) return LTK_EUNSUPPORTED;
    if (T > 0 && (!q || !db || !out_idx || !ws)) return LTK_EINVAL;
    if (!aligned16(q) || !aligned16(db) || !aligned16(ws)) return LTK_EINVAL;
    Opts o;
    int st;
    if ((st = resolve_opts(opts, retrieve_default_ccap(topk), o)) != LTK_OK) return st;
    if (o.sorted && topk > kMaxSortedK) return LTK_EINVAL;
    const int ns = retr_splits(T, D, N, o.l_splits);
    if ((N + ns - 1) / ns > kRetrMaxSplitRows) return LTK_EINVAL;
    if (ws_bytes < unfused_matrix_bytes(T, N)) return LTK_EWORKSPACE;
    if (T == 0) return LTK_OK;
    if ((st = device_check()) != LTK_OK) return st;
    RetrArgs r{};
    r.q = static_cast<const uint8_t*>(q);
    r.db = static_cast<const uint8_t*>(db);
    r.T = T;
    r.N = (int)N;
    r.topk = topk;
    r.n_splits = ns;
    r.n_qgroups = (T + retr_group_queries(D) - 1) / retr_group_queries(D);
    r.S = static_cast<float*>(ws);
    r.ev_scan_start = o.ev0;
    r.ev_scan_stop = o.ev1;
    IdxArgs sel{};
    sel.T = T;
    sel.L = (int)N;
    sel.topk = topk;
    sel.sorted = o.sorted;
    sel.pos = nullptr;
    sel.S = r.S;
    sel.out_idx = out_idx;
    sel.out_score = out_score;
    if (launch_retrieve_unfused(D, r, sel, static_cast<hipStream_t>(stream)) != hipSuccess) return LTK_EHIP;
    return LTK_OK;
}

int litetopk_retrieve(const void* q, const void* db, int32_t T, int32_t D, int64_t N, int32_t dtype, int32_t topk,
                      const int32_t* sample, int32_t n_sample, int32_t* out_idx, float* out_score, void* ws,
                      size_t ws_bytes, const ltk_opts* opts, ltk_stats* stats, void* stream) {
    if (T < 0 || N < 1 || N > (int64_t)0x7fffff00 || topk < 1 || topk > 65536 || n_sample < 0) return LTK_EINVAL;
    if (dtype != LTK_BF16) return dtype < LTK_F32 || dtype > LTK_FP8_E4M3FN ? LTK_EINVAL : LTK_EUNSUPPORTED;
    if (D != 64 && D != 128 && D != 256 && D != 512 && D != 768) return LTK_EUNSUPPORTED;
    if (n_sample > 0 && !sample) return LTK_EINVAL;
    if (T > 0 && (!q || !db || !out_idx || !ws)) return LTK_EINVAL;
    if (!aligned16(q) || !aligned16(db) || !aligned16(ws)) return LTK_EINVAL;
    Opts o;
    int st;
    if ((st = resolve_opts(opts, retrieve_default_ccap(topk), o)) != LTK_OK) return st;
    if (o.sorted && topk > kMaxSortedK) return LTK_EINVAL;
    const int ns = retr_splits(T, D, N, o.l_splits);
    if ((N + ns - 1) / ns > kRetrMaxSplitRows) return LTK_EINVAL;
    const int32_t n_slots = sample_slots(n_sample, topk, N);
    const WsLayout lay = ws_layout(T, N, n_slots, o.ccap, retr_hist_words(T, o.nbins, ns));
    if (ws_bytes < lay.total) return LTK_EWORKSPACE;
    if (T == 0) return LTK_OK;
    if ((st = device_check()) != LTK_OK) return st;

    uint8_t* wsb = static_cast<uint8_t*>(ws);
    // the sample pass, finalize and the shared kernels take the indexer's argument block
    IdxArgs f{};
    f.T = T;
    f.H = 1;
    f.L = (int)N;
    f.topk = topk;
    f.nbins = o.nbins;
    f.n_sample = n_slots > 0 ? n_slots : 1;
    f.sorted = o.sorted;
    f.ccap = o.ccap;
    f.pos = nullptr;   // no causal mask
    f.tail = reinterpret_cast<uint32_t*>(wsb + lay.tail);
    f.flags = reinterpret_cast<uint32_t*>(wsb + lay.flags);
    f.nu = reinterpret_cast<uint32_t*>(wsb + lay.nu);
    f.bitmap = reinterpret_cast<uint32_t*>(wsb + lay.bitmap);
    f.meta = wsb + lay.meta;
    f.sample_u = reinterpret_cast<int32_t*>(wsb + lay.sample_u);
    f.sscore = reinterpret_cast<float*>(wsb + lay.sscore);
    f.cand = reinterpret_cast<uint2*>(wsb + lay.cand);
    f.out_idx = out_idx;
    f.out_score = out_score;
    f.stats = stats;

    RetrArgs r{};
    r.q = static_cast<const uint8_t*>(q);
    r.db = static_cast<const uint8_t*>(db);
    r.T = T;
    r.N = (int)N;
    r.topk = topk;
    r.nbins = o.nbins;
    r.nsuper = (o.nbins + 15) / 16;
    r.n_sample = f.n_sample;
    r.n_qgroups = (T + retr_group_queries(D) - 1) / retr_group_queries(D);
    r.n_splits = ns;
    r.cap_s = o.ccap / ns;
    r.sorted = o.sorted;
    r.ccap = o.ccap;
    r.tail = f.tail;
    r.flags = f.flags;
    r.nu = f.nu;
    r.sample_u = f.sample_u;
    r.sscore = f.sscore;
    r.meta = f.meta;
    r.cand = f.cand;
    r.hist_g = reinterpret_cast<uint32_t*>(wsb + lay.hist);
    r.hist_c = r.hist_g + (size_t)T * o.nbins;
    r.seg_cnt = r.hist_c + (size_t)T * r.nsuper;
    r.out_idx = out_idx;
    r.out_score = out_score;
    r.ev_scan_start = o.ev0;
    r.ev_scan_stop = o.ev1;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_prepare_sample(f, sample, n_sample, lay, wsb, s) != hipSuccess) return LTK_EHIP;
    if (launch_retrieve(D, r, f, s) != hipSuccess) return LTK_EHIP;
    return LTK_OK;
}

}  // extern "C"
