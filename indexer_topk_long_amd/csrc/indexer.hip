// indexer.hip -- the fused Indexer-TopK path for gfx950 and its unfused baseline.
//
// Phases (LiteTopK pages, "Methodology"):
//   Sample  : sample_prepare (de-duplicate the reused sample), sample_score
//             (score it on the matrix cores), sample_stats (score range,
//             equal-width bins, initial threshold bin = bin of the sample's
//             k-th largest score)
//   Filter  : scan_kernel -- MFMA scoring of every causal key, ReLU*w head
//             reduction, affine bin map, gate against the threshold bin,
//             wave-local candidate lists written back in batches of 64,
//             histogram of kept keys and a periodic top-down threshold refresh
//   Select  : finalize_kernel -- keys in bins above the final threshold bin
//             go straight out; an exact top-k runs only inside that bin
//   (overflow) fallback_kernel -- exact re-scoring radix select for rows whose
//             candidate buffer overflowed (not on the pages; keeps exactness)
// Unfused baseline (pages, "Problem statement"): the fused scan's scoring loop
// in its FULL form writes the whole T x L score matrix, then
// unfused_select_kernel radix-selects each row.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"
#include "kernels_common.hpp"

namespace ltk {

// ---------------------------------------------------------------------------
// small kernels of the sample pass
// ---------------------------------------------------------------------------

__global__ void zero_kernel(uint32_t* p, size_t n_words, ltk_stats* stats) {
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (size_t i = i0; i < n_words; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
    if (stats && i0 == 0) {
        stats->cand_written = 0;
        stats->bytes_written = 0;
        stats->max_cand_per_query = 0;
        stats->overflow_rows = 0;
    }
}

// Mark each in-range sample index in a bitmap over the keys (drops duplicates
// and out-of-range entries).
__global__ void sample_mark_kernel(const int32_t* sample, int n, int L, uint32_t* bitmap) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const int s = sample[i];
        if (s >= 0 && s < L) atomicOr(&bitmap[s >> 5], 1u << (s & 31));
    }
}

// Small samples: workgroup 0 (1024 threads) de-duplicates the sample through
// an LDS hash table (open addressing, at least twice as many slots as
// entries) into the list of distinct in-range keys, in no particular order;
// the other workgroups clear [zero_begin, zero_end) of the workspace.
constexpr uint32_t kHashEmpty = 0xffffffffu;

__global__ __launch_bounds__(1024) void sample_prep_kernel(const int32_t* sample, int n, int L, int log2_slots,
                                                           uint32_t* zero, size_t n_zero, ltk_stats* stats,
                                                           int32_t* out, uint32_t* nu, int n_own,
                                                           const int32_t* pos, int T) {
    const int tid = threadIdx.x;
    if (blockIdx.x > 0) {
        const size_t i0 = (size_t)(blockIdx.x - 1) * 1024 + tid;
        for (size_t i = i0; i < n_zero; i += (size_t)(gridDim.x - 1) * 1024) zero[i] = 0u;
        if (stats && i0 == 0) {
            stats->cand_written = 0;
            stats->bytes_written = 0;
            stats->max_cand_per_query = 0;
            stats->overflow_rows = 0;
        }
        return;
    }
    if (n == 0) {
        // no sample given: n_own evenly spaced keys below the largest causal
        // bound of the call's queries (every key without positions), ascending
        __shared__ int s_e[16];
        int e = pos ? 0 : L;
        if (pos)
            for (int t = tid; t < T; t += 1024) e = max(e, min(pos[t], L - 1) + 1);
        e = wave_max_i32(e);
        if (lane_id() == 0) s_e[tid >> 6] = e;
        __syncthreads();
        int kmax = 0;
        for (int w = 0; w < 16; ++w) kmax = max(kmax, s_e[w]);
        const int nw = min(n_own, kmax);
        for (int j = tid; j < nw; j += 1024) out[j] = (int32_t)(((int64_t)j * kmax) / nw);
        if (tid == 0) *nu = (uint32_t)nw;
        return;
    }
    extern __shared__ uint32_t tab[];   // [1 << log2_slots]
    __shared__ uint32_t s_n;
    const int slots = 1 << log2_slots, lane = lane_id();
    for (int i = tid; i < slots; i += 1024) tab[i] = kHashEmpty;
    if (tid == 0) s_n = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += 1024) {
        const int i = i0 + tid;
        bool fresh = false;
        uint32_t key = 0u;
        if (i < n) {
            const int s = sample[i];
            if (s >= 0 && s < L) {
                key = (uint32_t)s;
                uint32_t h = (key * 2654435761u) >> (32 - log2_slots);
                while (true) {   // terminates: fewer entries than slots
                    const uint32_t old = atomicCAS(&tab[h], kHashEmpty, key);
                    if (old == kHashEmpty) { fresh = true; break; }
                    if (old == key) break;
                    h = (h + 1u) & (uint32_t)(slots - 1);
                }
            }
        }
        const uint64_t m = __ballot(fresh);
        uint32_t base = 0u;
        if (lane == 0 && m) base = atomicAdd(&s_n, (uint32_t)__popcll(m));
        base = lane0_u32(base);
        if (fresh) out[base + mbcnt(m)] = (int32_t)key;
    }
    __syncthreads();
    if (tid == 0) *nu = s_n;
}

// Keys marked in each bitmap chunk (one workgroup per chunk).
__global__ __launch_bounds__(256) void sample_count_kernel(const uint32_t* bitmap, int nwords, int chunk_log2,
                                                           uint32_t* ccount) {
    __shared__ uint32_t s_red[4];
    const int c = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int w_end = min(nwords, (c + 1) << chunk_log2);
    uint32_t cnt = 0;
    for (int w = (c << chunk_log2) + tid; w < w_end; w += 256) cnt += __popc(bitmap[w]);
    cnt = wave_sum_u32(cnt);
    if (lane == 0) s_red[wave] = cnt;
    __syncthreads();
    if (tid == 0) ccount[c] = s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

// One workgroup per bitmap chunk writes the chunk's keys, in order, after the
// keys of all earlier chunks: the sorted list of distinct sample keys.  The
// last chunk's workgroup writes the total.
__global__ __launch_bounds__(256) void sample_compact_kernel(const uint32_t* bitmap, int nwords, int chunk_log2,
                                                             const uint32_t* ccount, int32_t* out, uint32_t* nu) {
    __shared__ uint32_t s_red[4], s_wsum[4];
    const int c = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    uint32_t part = 0;
    for (int i = tid; i < c; i += 256) part += ccount[i];
    part = wave_sum_u32(part);
    if (lane == 0) s_red[wave] = part;
    __syncthreads();
    const uint32_t off = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const uint32_t mine = ccount[c];
    if (c == (int)gridDim.x - 1 && tid == 0) *nu = off + mine;
    if (mine == 0) return;
    const int wpt = (1 << chunk_log2) >> 8;   // words per thread (>= 4)
    const int w0 = (c << chunk_log2) + tid * wpt;
    uint32_t cnt = 0;
    for (int j = 0; j < wpt; ++j)
        if (w0 + j < nwords) cnt += __popc(bitmap[w0 + j]);
    uint32_t incl = wave_scan_add_u32(cnt);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t o = off + incl - cnt;
    for (int w = 0; w < wave; ++w) o += s_wsum[w];
    for (int j = 0; j < wpt; ++j) {
        if (w0 + j >= nwords) break;
        uint32_t word = bitmap[w0 + j];
        while (word) {
            const int b = __ffs(word) - 1;
            out[o++] = (w0 + j) * 32 + b;
            word &= word - 1;
        }
    }
}

// ---------------------------------------------------------------------------
// per-wave query state: two queries per wave, one per 32-lane half
// ---------------------------------------------------------------------------

template <int DT, int D, int HB>
struct QueryRegs {
    HalfRow<DT, D> q[HB];
    float w[HB][16];
};

// Q rows (heads) of query t for this lane and the lane's head weights
// w'[h] = sigma_q[t] * w[t, h], halved for fp8 (zero for padded heads / queries).
template <int DT, int D, int HB>
__device__ __forceinline__ void load_query(QueryRegs<DT, D, HB>& r, const IdxArgs& a, int t) {
    const int lane = lane_id(), half = lane >> 5, row = lane & 31;
    constexpr int RB = D * DTraits<DT>::ESZ;  // bytes per row
    const bool tv = t < a.T;
    const float sq = (DT == DT_FP8 && tv) ? a.q_scale[t] : 1.0f;
#pragma unroll
    for (int m = 0; m < HB; ++m) {
        const int h = m * 32 + row;
        if (tv && h < a.H)
            load_half_row<DT, D>(r.q[m], a.q + ((size_t)t * a.H + h) * RB, half);
        else
            zero_half_row<DT, D>(r.q[m]);
        // the lane's 16 weights load unconditionally, so they issue back to
        // back and are waited for once (a load per condition would be waited
        // for one by one).  When all 16 heads exist they come from one row
        // address with immediate offsets (few registers); otherwise the head
        // index is clamped into the row.  Padded heads and queries then get
        // weight 0.
        const float* wq = a.w + (size_t)min(t, a.T - 1) * a.H;
        const int h0 = head_of(m, 0, half);
        float wv[16];
        if (h0 + 27 < a.H) {
#pragma unroll
            for (int i = 0; i < 16; ++i) wv[i] = wq[h0 + 8 * (i >> 2) + (i & 3)];
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) wv[i] = wq[min(h0 + 8 * (i >> 2) + (i & 3), a.H - 1)];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hh = head_of(m, i, half);
            // fp8 scores sum w'/2 |x| (abs_wsum): the halving is exact
            const float wh = (DT == DT_FP8) ? (sq * wv[i]) * 0.5f : sq * wv[i];
            r.w[m][i] = (tv && hh < a.H) ? wh : 0.0f;
        }
    }
}

template <int DT, int D>
__device__ __forceinline__ void load_key(HalfRow<DT, D>& f, const uint8_t* k, int key) {
    constexpr int RB = D * DTraits<DT>::ESZ;
    load_half_row<DT, D>(f, k + (size_t)key * RB, lane_id() >> 5);
}

// Scores of two slots; lane gets slot (lane>>5), key (lane&31) of that slot's block.
template <int DT, int D, int HB>
__device__ __forceinline__ float score_2slots(const QueryRegs<DT, D, HB>& qa, const HalfRow<DT, D>& ka,
                                              const QueryRegs<DT, D, HB>& qb, const HalfRow<DT, D>& kb) {
    v16f acca[HB], accb[HB];
    mfma_2slots<DT, D, HB>(qa.q, ka, qb.q, kb, acca, accb);
    if constexpr (DT == DT_FP8) {   // 1/2 sum w'|x|; the caller adds the linear term
        const float pa = abs_wsum<HB>(acca, qa.w);
        const float pb = abs_wsum<HB>(accb, qb.w);
        return combine_halves(pa, pb);
    }
    const float pa = relu_wsum<HB>(acca, qa.w);
    const float pb = relu_wsum<HB>(accb, qb.w);
    return combine_halves(pa, pb);
}

// End (exclusive) of the keys any query of the group [t0, t0+8) can see.
__device__ __forceinline__ int group_key_end(const IdxArgs& a, int t0) {
    const int lane = lane_id();
    const int t = t0 + (lane & 7);
    int e = (t < a.T) ? min(a.pos[t], a.L - 1) + 1 : 0;
    return wave_max_i32(max(e, 0));
}


// ---------------------------------------------------------------------------
// fp8 linear term: operands per query, and its products outside the scan
// ---------------------------------------------------------------------------

// One workgroup of 256 threads per query: q''/2 = sum_h (w'_h / 2) q_h over
// the query's heads (w' = sigma_q w as the head sum uses it), each thread
// summing 4 dimensions over every (256 / (D/4))-th head from one 32-bit load
// per head, the head groups then added in LDS; then four fp8 parts of
// (q''/2) * S with S = 2^(8 - e) putting the largest magnitude in [128, 256),
// each part taking the residue of the ones before it times 16.  Every fp8
// pass reads these same bytes, so all of them get the same linear term.
// The loads come first (qlin_load, every one issued before any is waited
// for), then the sums (qlin_partial, a barrier, qlin_finish), which every
// thread of a workgroup of at least 256 threads calls (the first 256 do the
// work, so that every launch adds in the same order).  lin, when given,
// receives a copy of the four parts in LDS, and store = false leaves the
// workspace copy to another workgroup.  qlin_finish returns 1/S (to every
// thread).
template <int D>
struct QlinIn {
    static constexpr int NQ = D / 4;          // 4-dimension groups
    static constexpr int HG = 256 / NQ;       // head groups
    static constexpr int NI = 64 / HG;        // heads per thread (at most 64 heads)
    uint32_t v[NI];
    float w[NI];
    float sq;
};

template <int D>
__device__ __forceinline__ void qlin_load(QlinIn<D>& in, const IdxArgs& a, int t) {
    using Q = QlinIn<D>;
    const int tid = threadIdx.x;
    const int dq = tid % Q::NQ, hg = (tid / Q::NQ) % Q::HG;
    in.sq = a.q_scale[t];
    const uint8_t* q = a.q + (size_t)t * a.H * D;
    const float* w = a.w + (size_t)t * a.H;
#pragma unroll
    for (int i = 0; i < Q::NI; ++i) {
        const int h = min(hg + i * Q::HG, a.H - 1);
        in.v[i] = *reinterpret_cast<const uint32_t*>(q + (size_t)h * D + 4 * dq);
        in.w[i] = w[h];
    }
}

template <int D>
struct QlinShared {
    float part[QlinIn<D>::HG][D];
    float wmax[4];
};

// Head-group partial sums into LDS (no barrier).
template <int D>
__device__ __forceinline__ void qlin_partial(const QlinIn<D>& in, const IdxArgs& a, QlinShared<D>& sh) {
    using Q = QlinIn<D>;
    const int tid = threadIdx.x;
    if (tid < 256) {
        const int dq = tid % Q::NQ, hg = tid / Q::NQ;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < Q::NI; ++i) {
            if (hg + i * Q::HG < a.H) {
                const float c = (in.sq * in.w[i]) * 0.5f;
                acc[0] = __builtin_fmaf(c, __builtin_amdgcn_cvt_f32_fp8((int)in.v[i], 0), acc[0]);
                acc[1] = __builtin_fmaf(c, __builtin_amdgcn_cvt_f32_fp8((int)in.v[i], 1), acc[1]);
                acc[2] = __builtin_fmaf(c, __builtin_amdgcn_cvt_f32_fp8((int)in.v[i], 2), acc[2]);
                acc[3] = __builtin_fmaf(c, __builtin_amdgcn_cvt_f32_fp8((int)in.v[i], 3), acc[3]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.part[hg][4 * dq + i] = acc[i];
    }
}

// The rest, after a barrier that follows qlin_partial: the head groups added,
// the scale, the four parts.  Synchronises the workgroup once.
template <int D>
__device__ float qlin_finish(const IdxArgs& a, int t, uint8_t* lin, bool store, QlinShared<D>& sh) {
    using Q = QlinIn<D>;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    float x = 0.0f;
    if (tid < D) {
#pragma unroll
        for (int g = 0; g < Q::HG; ++g) x += sh.part[g][tid];
    }
    if (tid < 256) {
        const float m = wave_max_f32(tid < D ? fabsf(x) : 0.0f);
        if (lane == 0) sh.wmax[wave] = m;
    }
    __syncthreads();
    const float mx = fmaxf(fmaxf(sh.wmax[0], sh.wmax[1]), fmaxf(sh.wmax[2], sh.wmax[3]));
    int e = 0;
    if (mx > 0.0f) frexpf(mx, &e);   // mx in [2^(e-1), 2^e)
    e = max(-100, min(e, 100));      // keeps S and 1/S finite and normal
    if (tid < D) {
        uint8_t* out = a.qlin + (size_t)t * 4 * D;
        float r = x * ldexpf(1.0f, 8 - e);   // exact: a power of two
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false) & 0xffu;
            if (store) out[p * D + tid] = (uint8_t)code;
            if (lin) lin[p * D + tid] = (uint8_t)code;
            r = (r - __builtin_amdgcn_cvt_f32_fp8((int)code, 0)) * 16.0f;   // exact residue, scaled
        }
    }
    const float inv = ldexpf(1.0f, e - 8);
    if (store && tid == 0) a.qinv[t] = inv;
    return inv;
}

template <int D>
__global__ __launch_bounds__(256) void qlin_kernel(IdxArgs a) {
    __shared__ QlinShared<D> sh;
    QlinIn<D> in;
    qlin_load<D>(in, a, blockIdx.x);
    qlin_partial<D>(in, a, sh);
    __syncthreads();
    (void)qlin_finish<D>(a, blockIdx.x, nullptr, true, sh);
}

// 32 fp8 values of row `row` (D bytes), dimensions [32 ks, 32 ks + 32); zero
// past D (D = 64 uses half of the instruction's 128 dimensions).
template <int D>
__device__ __forceinline__ void load_lin_frag(LinFrag& f, const uint8_t* row, int ks) {
    if (32 * ks < D) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + 32 * ks);
        f.v[0] = p[0];
        f.v[1] = p[1];
    } else {
        f.v[0] = f.v[1] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Linear-term operands of two queries ta (results in lanes 0-31) and tb
// (lanes 32-63) against one 32-key block, in the lane layout of
// score_2slots: two instructions, keys 0-15 with ta in rows 0-3 and tb in
// rows 8-11, keys 16-31 with ta in rows 4-7 and tb in rows 12-15, so that
// lane l finds its own (query, key) in one of the two results.  inv is 1/S
// of the lane's query.
struct LinPair {
    LinFrag a0, a1;
    float inv;
};

template <int D>
__device__ __forceinline__ void load_lin_pair(LinPair& p, const IdxArgs& a, int ta, int tb) {
    const int lane = lane_id(), r = lane & 15, ks = lane >> 4;
    auto part = [&](LinFrag& f, int t, int pp) {
        if (t < a.T) load_lin_frag<D>(f, a.qlin + ((size_t)t * 4 + pp) * D, ks);
        else f.v[0] = f.v[1] = u32x4{0u, 0u, 0u, 0u};
    };
    const int g = r >> 2, pp = r & 3;   // row group and part of this lane's operand row
    part(p.a0, g == 0 ? ta : g == 2 ? tb : a.T, pp);
    part(p.a1, g == 1 ? ta : g == 3 ? tb : a.T, pp);
    const int t = (lane < 32) ? ta : tb;
    p.inv = (t < a.T) ? a.qinv[t] : 0.0f;
}

// (q''/2 . k) * S for the lane's query of the pair and key row kA (lanes
// with (lane >> 4) even) or kB (odd): kA/kB hold the keys of columns
// (lane & 15) and 16 + (lane & 15) of the block.
template <int D>
__device__ __forceinline__ float lin_pair_t(const LinPair& p, const uint8_t* k, int kA, int kB) {
    const int ks = lane_id() >> 4;
    LinFrag b0, b1;
    load_lin_frag<D>(b0, k + (size_t)kA * D, ks);
    load_lin_frag<D>(b1, k + (size_t)kB * D, ks);
    const v4f c0 = lin_mfma(p.a0, b0), c1 = lin_mfma(p.a1, b1);
    return lin_combine((ks & 1) ? c1 : c0);
}

// One query against 64 consecutive keys (lane l: key base + l): the query's
// four parts in every row group, four instructions of 16 keys each.
template <int D>
__device__ __forceinline__ void load_lin_one(LinFrag& f, const IdxArgs& a, int t) {
    const int lane = lane_id();
    load_lin_frag<D>(f, a.qlin + ((size_t)t * 4 + (lane & 3)) * D, lane >> 4);
}
template <int D>
__device__ __forceinline__ float lin_one64_t(const LinFrag& aq, const uint8_t* k, int base, int L) {
    const int lane = lane_id(), ks = lane >> 4;
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        LinFrag b;
        load_lin_frag<D>(b, k + (size_t)min(base + 16 * i + (lane & 15), L - 1) * D, ks);
        const float ti = lin_combine(lin_mfma(aq, b));
        t = (ks == i) ? ti : t;
    }
    return t;
}

// ---------------------------------------------------------------------------
// Sample: score the de-duplicated sample keys
// ---------------------------------------------------------------------------

// Range, delta, histogram and initial threshold bin of query t (its Meta)
// from each thread's count of valid sample scores and their extremes; add(smin,
// delta) puts the thread's valid scores into the histogram sh (nbins words).
// All NW * 64 threads of the workgroup call it together (it synchronises them).
template <int NW, class Add>
__device__ void sample_meta(const IdxArgs& a, int t, uint32_t c, float mn, float mx, uint32_t* sh, Add add) {
    __shared__ float s_min[NW], s_max[NW];
    __shared__ uint32_t s_nv[NW];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    c = wave_sum_u32(c);
    for (int i = tid; i < a.nbins; i += NW * 64) sh[i] = 0u;
    mn = wave_min_f32(mn);
    mx = wave_max_f32(mx);
    if (lane == 0) {
        s_nv[wave] = c;
        s_min[wave] = mn;
        s_max[wave] = mx;
    }
    __syncthreads();
    int nv = 0;
    float smin = INFINITY, smax = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        nv += (int)s_nv[w];
        smin = fminf(smin, s_min[w]);
        smax = fmaxf(smax, s_max[w]);
    }
    if (nv == 0) {
        smin = 0.0f;
        smax = 1.0f;
    }
    float width = smax - smin;
    const float floor_w = 1e-6f * fmaxf(1.0f, fabsf(smax));
    if (!(width >= floor_w)) width = floor_w;
    const float delta = (float)a.nbins / width;
    add(smin, delta);
    __syncthreads();
    if (wave == 0) {
        int thr0 = 0;
        if (nv >= a.topk) thr0 = max(0, suffix_pick(sh, a.nbins, (uint32_t)a.topk).bin);
        if (lane == 0) {
            Meta m;
            m.smin = smin;
            m.delta = delta;
            m.thr0 = thr0;
            m.nvalid = nv;
            reinterpret_cast<Meta*>(a.meta)[t] = m;
        }
    }
    __syncthreads();   // sh and the partials are free for the next query
}

// Sample statistics of query t: valid sample keys (<= pos), range, delta,
// histogram and the initial threshold bin.  All NT threads of the workgroup
// call it together (it synchronises them); sh holds nbins words.
template <int NT>
__device__ void sample_stats_query(const IdxArgs& a, int t, uint32_t* sh) {
    const int tid = threadIdx.x;
    const int nu = (int)*a.nu;
    const int pos_t = a.pos ? min(a.pos[t], a.L - 1) : a.L - 1;   // no positions: every key is valid
    const float* S = a.sscore + (size_t)t * a.n_sample;
    // one pass: valid sample keys (<= pos_t; the list may be in any order)
    // and their score range; up to kStatsRegs scores per thread stay in
    // registers (NaN when invalid) for the histogram
    constexpr int kStatsRegs = 16;
    const bool in_regs = nu <= NT * kStatsRegs;
    float v[kStatsRegs];
    uint32_t c = 0;
    float mn = INFINITY, mx = -INFINITY;
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kStatsRegs; ++i) {
            // the score loads do not wait for the key loads (one round trip)
            const int j = tid + NT * i;
            const float sj = (j < nu) ? S[j] : NAN;
            const bool ok = j < nu && a.sample_u[j] <= pos_t;
            v[i] = ok ? sj : NAN;
            if (ok) {
                ++c;
                mn = fminf(mn, v[i]);
                mx = fmaxf(mx, v[i]);
            }
        }
    } else {
        for (int j = tid; j < nu; j += NT) {
            if (a.sample_u[j] <= pos_t) {
                ++c;
                mn = fminf(mn, S[j]);
                mx = fmaxf(mx, S[j]);
            }
        }
    }
    sample_meta<NT / 64>(a, t, c, mn, mx, sh, [&](float smin, float delta) {
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < kStatsRegs; ++i)
                if (!__builtin_isnan(v[i])) atomicAdd(&sh[bin_of(v[i], smin, delta, a.nbins)], 1u);
        } else {
            for (int j = tid; j < nu; j += NT)
                if (a.sample_u[j] <= pos_t) atomicAdd(&sh[bin_of(S[j], smin, delta, a.nbins)], 1u);
        }
    });
}

// One workgroup per query; 1,024 threads when the sample has more slots than
// 256 threads hold in registers.
template <int NT>
__global__ __launch_bounds__(NT) void sample_stats_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];  // [nbins]
    sample_stats_query<NT>(a, blockIdx.x, sh);
}

static void launch_stats_kernel(const IdxArgs& a, hipStream_t st) {
    if (a.n_sample > 256 * 16) sample_stats_kernel<1024><<<a.T, 1024, (size_t)a.nbins * 4, st>>>(a);
    else sample_stats_kernel<256><<<a.T, 256, (size_t)a.nbins * 4, st>>>(a);
}

template <int DT, int D, int HB>
__device__ __forceinline__ void sample_score_part(const IdxArgs& a, int qg, int sp) {
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;
    const int ta = qg * kQPG + 2 * wave, tb = ta + 1;
    const int nu = (int)*a.nu;
    if (nu == 0) return;
    const int nblk = (nu + 31) / 32;
    const int per = (nblk + a.s_splits - 1) / a.s_splits;
    const int b0 = sp * per, b1 = min(nblk, b0 + per);
    if (b0 >= b1) return;
    QueryRegs<DT, D, HB> ra, rb;
    load_query<DT, D, HB>(ra, a, ta);
    load_query<DT, D, HB>(rb, a, tb);
    const int t = half ? tb : ta;
    LinPair lp;
    if constexpr (DT == DT_FP8) load_lin_pair<D>(lp, a, ta, tb);
    if constexpr (HalfRow<DT, D>::NV > 4) {
        // wide fragments: no room for a second one
        for (int blk = b0; blk < b1; ++blk) {
            const int j = blk * 32 + (lane & 31);
            const int key = a.sample_u[min(j, nu - 1)];
            HalfRow<DT, D> kf;
            load_key<DT, D>(kf, a.k, key);
            float I = score_2slots<DT, D, HB>(ra, kf, rb, kf);
            if constexpr (DT == DT_FP8) I = I * a.k_scale[key];
            if (t < a.T && j < nu) a.sscore[(size_t)t * a.n_sample + j] = I;
        }
        return;
    }
    // the next block's key rows (and the one after's key indices) are in
    // flight while a block is scored
    auto key_at = [&](int blk) { return a.sample_u[min(blk * 32 + (lane & 31), nu - 1)]; };
    int key = key_at(b0);
    int key2 = (b0 + 1 < b1) ? key_at(b0 + 1) : key;
    HalfRow<DT, D> kf;
    load_key<DT, D>(kf, a.k, key);
    float ks = (DT == DT_FP8) ? a.k_scale[key] : 1.0f;
    for (int blk = b0; blk < b1; ++blk) {
        const int j = blk * 32 + (lane & 31);
        const HalfRow<DT, D> cur = kf;
        const float cks = ks;
        const int ckey = key;
        if (blk + 1 < b1) {
            key = key2;
            load_key<DT, D>(kf, a.k, key);
            if constexpr (DT == DT_FP8) ks = a.k_scale[key];
            if (blk + 2 < b1) key2 = key_at(blk + 2);
        }
        float I = score_2slots<DT, D, HB>(ra, cur, rb, cur);
        if constexpr (DT == DT_FP8) {
            // the block's keys of columns (lane & 15) and 16 + (lane & 15)
            const int kA = __shfl(ckey, lane & 15), kB = __shfl(ckey, 16 + (lane & 15));
            I = lin_score(lin_pair_t<D>(lp, a.k, kA, kB), lp.inv, I, cks);
        }
        if (t < a.T && j < nu) a.sscore[(size_t)t * a.n_sample + j] = I;
    }
}

// Sample pass at prefill shape: the de-duplicated sample keys' rows (and
// fp8 scales) copied into one contiguous array, row j from sample_u[j] (rows
// past the nu distinct keys repeat the last; their scores are never read),
// and a causal bound past every row for each query.  The scan's full-score
// form then scores every query against the array into the sample-score rows
// (launch_indexer_fused), with the scan's own arithmetic and tiles.
__global__ __launch_bounds__(256) void sample_gather_kernel(IdxArgs a, int rb) {
    const int nu = (int)*a.nu;
    const int chunks = rb / 16;
    const size_t total = (size_t)a.n_sample * chunks;
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < total; u += stride) {
        const int j = (int)(u / chunks), c = (int)(u % chunks);
        const int key = nu > 0 ? a.sample_u[min(j, nu - 1)] : 0;
        reinterpret_cast<u32x4*>(a.sg_k + (size_t)j * rb)[c] = reinterpret_cast<const u32x4*>(a.k + (size_t)key * rb)[c];
    }
    for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < (size_t)a.n_sample; j += stride) {
        const int key = nu > 0 ? a.sample_u[min((int)j, nu - 1)] : 0;
        if (a.k_scale) a.sg_scale[j] = a.k_scale[key];
    }
    for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < (size_t)a.T; t += stride) a.sg_pos[t] = a.n_sample - 1;
}

// Sample scores of a query group's queries, split over s_splits workgroups.
template <int DT, int D, int HB>
__global__ __launch_bounds__(256) void sample_score_kernel(IdxArgs a) {
    sample_score_part<DT, D, HB>(a, blockIdx.x / a.s_splits, blockIdx.x % a.s_splits);
}

// ---------------------------------------------------------------------------
// Sample, decode shape: the sample steps in one launch
// ---------------------------------------------------------------------------
//
// With few queries the steps above are each a launch of a few microseconds
// that leaves most of the GPU idle.  Here `parts` workgroups per query do all
// of them.  Workgroup (t, p) inserts the sample entries of class p
// (front_class of the key) that query t can see into its LDS hash table; the
// entry that inserts a key writes the key's score -- the arithmetic of the
// sample pass, so the same value -- to its slot of score row t, every other
// entry of the key writes NaN there.  The workgroup also writes NaN to the
// slots of the entries no class takes (empty, outside the context or past the
// query's position) that are p modulo parts.  The classes
// partition the keys, so each distinct key the query sees has exactly one
// score in the row.  Every workgroup of a query computes its fp8 linear-term
// operands the same way (p = 0 stores them).  The launch's other workgroups
// clear the workspace.

constexpr int kFrontThreads = 512;
constexpr int kFrontRegs = kFrontSampleMax / kFrontThreads;   // sample entries per thread

// Class of a sample key: a hash of it, so that keys in arithmetic progression
// spread over the classes (another multiplier than the hash table's, whose
// slot bits it would otherwise fix).
__device__ __forceinline__ int front_class(int key, int lgp) {
    return lgp ? (int)(((uint32_t)key * 0x85EBCA77u) >> (32 - lgp)) : 0;
}

template <int DT, int D, int HB>
__global__ __launch_bounds__(kFrontThreads) void front_kernel(IdxArgs a, const int32_t* sample, int n, int lgp,
                                                              int log2_slots, uint32_t* zero, size_t n_zero) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int parts = 1 << lgp;
    const int nq = a.T * parts;
    if ((int)blockIdx.x >= nq) {
        const size_t i0 = (size_t)(blockIdx.x - nq) * kFrontThreads + tid;
        for (size_t i = i0; i < n_zero; i += (size_t)(gridDim.x - nq) * kFrontThreads) zero[i] = 0u;
        if (a.stats && i0 == 0) {
            a.stats->cand_written = 0;
            a.stats->bytes_written = 0;
            a.stats->max_cand_per_query = 0;
            a.stats->overflow_rows = 0;
        }
        return;
    }
    const int t = blockIdx.x / parts, p = blockIdx.x % parts;
    extern __shared__ unsigned long long fs[];
    const int slots = 1 << log2_slots;
    unsigned long long* list = fs;                                  // key << 32 | its slot
    uint32_t* tab = reinterpret_cast<uint32_t*>(fs + a.n_sample);   // hash table of keys
    __shared__ uint32_t s_wn[kFrontThreads / 64];
    __shared__ __attribute__((aligned(16))) uint8_t lin_l[DT == DT_FP8 ? 4 * D : 16];
    __shared__ QlinShared<DT == DT_FP8 ? D : 64> qsh;
    const int pos_t = min(a.pos[t], a.L - 1);
    const int ns = a.n_sample;                                      // slots of the score row
    float* srow = a.sscore + (size_t)t * ns;
    // every load that depends on nothing goes out before the first wait (the
    // query's first: the code between its loads has branches)
    QlinIn<D> qin;
    if constexpr (DT == DT_FP8) qlin_load<D>(qin, a, t);
    QueryRegs<DT, D, HB> qr;
    load_query<DT, D, HB>(qr, a, t);
    int sv[kFrontRegs];
    int kmax = 0;   // no sample given: the largest causal bound of the call's queries
    if (n > 0) {
#pragma unroll
        for (int r = 0; r < kFrontRegs; ++r) {
            const int j = tid + kFrontThreads * r;
            sv[r] = (j < n) ? sample[j] : -1;
        }
    } else {
        for (int u = 0; u < a.T; ++u) kmax = max(kmax, min(a.pos[u], a.L - 1) + 1);
    }
    for (int i = tid; i < slots; i += kFrontThreads) tab[i] = kHashEmpty;
    __syncthreads();   // the empty table before any insertion
    if constexpr (DT == DT_FP8) qlin_partial<D>(qin, a, qsh);
    // entry r of this thread: slot i and key s.  With a sample: slot
    // tid + 512 r.  Without: ns evenly spaced keys below kmax (distinct and
    // ascending), or fewer, of which this workgroup takes the slots p modulo
    // parts.
    const int nw = min(ns, kmax);
    auto entry = [&](int r, int& i, int& s) {
        if (n > 0) {
            i = tid + kFrontThreads * r;
            s = sv[r];
        } else {
            i = p + parts * (tid + kFrontThreads * r);
            s = (i < nw) ? (int)(((int64_t)i * kmax) / nw) : -1;
        }
    };
    // the keys of the class in [0, pos_t]: the entry that inserts a key into
    // the hash table lists it with its slot, the key's other entries write NaN
    // there; so do the entries no class takes (empty, outside the context or
    // past the query's position) whose slot is p modulo parts
    uint32_t fresh = 0;   // bit r: entry r inserted its key
#pragma unroll
    for (int r = 0; r < kFrontRegs; ++r) {
        int i, s;
        entry(r, i, s);
        const bool vis = i < ns && s >= 0 && s <= pos_t;
        if (vis && (n == 0 || front_class(s, lgp) == p)) {
            const uint32_t key = (uint32_t)s;
            uint32_t h = (key * 2654435761u) >> (32 - log2_slots);
            bool ins = false;
            while (true) {   // terminates: fewer entries than slots
                const uint32_t old = atomicCAS(&tab[h], kHashEmpty, key);
                if (old == kHashEmpty) { ins = true; break; }
                if (old == key) break;
                h = (h + 1u) & (uint32_t)(slots - 1);
            }
            if (ins) fresh |= 1u << r;
            else srow[i] = NAN;
        } else if (i < ns && !vis && (i & (parts - 1)) == p) {
            srow[i] = NAN;
        }
    }
    const uint32_t c = (uint32_t)__builtin_popcount(fresh);
    const uint32_t incl = wave_scan_add_u32(c);
    if (lane == 63) s_wn[wave] = incl;
    __syncthreads();
    uint32_t o = incl - c, nu = 0;
#pragma unroll
    for (int w = 0; w < kFrontThreads / 64; ++w) {
        const uint32_t x = s_wn[w];
        o += (w < wave) ? x : 0u;
        nu += x;
    }
#pragma unroll
    for (int r = 0; r < kFrontRegs; ++r) {
        if (fresh & (1u << r)) {
            int i, s;
            entry(r, i, s);
            list[o++] = ((unsigned long long)s << 32) | (uint32_t)i;
        }
    }
    float inv = 0.0f;   // fp8: 1/S of the linear term
    if constexpr (DT == DT_FP8) inv = qlin_finish<D>(a, t, lin_l, p == 0, qsh);   // synchronises
    __syncthreads();   // the list and the linear-term parts
    // scores: wave w takes 64-key blocks w, w + 8, ... of the list as two
    // 32-key slots of the query (lane l: list entry 64 b + l); every load of
    // a block is issued before the first is waited for
    LinFrag aq;
    if constexpr (DT == DT_FP8) load_lin_frag<D>(aq, lin_l + (lane & 3) * D, lane >> 4);
    const int nblk = ((int)nu + 63) / 64;
    auto key_at = [&](int j) { return (int)(list[min(j, (int)nu - 1)] >> 32); };
    for (int b = wave; b < nblk; b += kFrontThreads / 64) {
        const int j = 64 * b + lane;
        const unsigned long long own = list[min(j, (int)nu - 1)];
        HalfRow<DT, D> ka, kb;
        load_key<DT, D>(ka, a.k, key_at(64 * b + (lane & 31)));
        load_key<DT, D>(kb, a.k, key_at(64 * b + 32 + (lane & 31)));
        float I;
        if constexpr (DT == DT_FP8) {
            // lane l's key is 64 b + 16 (l >> 4) + (l & 15): instruction i
            // covers keys 16 i .. 16 i + 15 of the block
            LinFrag kf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                load_lin_frag<D>(kf[i], a.k + (size_t)key_at(64 * b + 16 * i + (lane & 15)) * D, lane >> 4);
            const float ks = a.k_scale[(int)(own >> 32)];
            I = score_2slots<DT, D, HB>(qr, ka, qr, kb);
            float tl = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ti = lin_combine(lin_mfma(aq, kf[i]));
                tl = ((lane >> 4) == i) ? ti : tl;
            }
            I = lin_score(tl, inv, I, ks);
        } else {
            I = score_2slots<DT, D, HB>(qr, ka, qr, kb);
        }
        if (j < (int)nu) srow[(uint32_t)own] = I;
    }
}

// Statistics of query t from its score row of the one-launch sample steps
// (NaN: no key at that slot).
__global__ __launch_bounds__(kFrontThreads) void front_stats_kernel(IdxArgs a) {
    __shared__ uint32_t sh[kMaxBins];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float* srow = a.sscore + (size_t)t * a.n_sample;
    float v[kFrontRegs];
#pragma unroll
    for (int r = 0; r < kFrontRegs; ++r) {
        const int i = tid + kFrontThreads * r;
        v[r] = (i < a.n_sample) ? srow[i] : NAN;
    }
    uint32_t c = 0;
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < kFrontRegs; ++r) {
        if (!__builtin_isnan(v[r])) {
            ++c;
            mn = fminf(mn, v[r]);
            mx = fmaxf(mx, v[r]);
        }
    }
    sample_meta<kFrontThreads / 64>(a, t, c, mn, mx, sh, [&](float smin, float delta) {
#pragma unroll
        for (int r = 0; r < kFrontRegs; ++r)
            if (!__builtin_isnan(v[r])) atomicAdd(&sh[bin_of(v[r], smin, delta, a.nbins)], 1u);
    });
}

// ---------------------------------------------------------------------------
// Filter: the fused scan
// ---------------------------------------------------------------------------
//
// One workgroup = 8 waves sharing K tiles that are streamed into LDS with
// direct global->LDS loads (one tile scored while the next ones load), so
// the eight waves read each key from device memory once.  Each wave owns one
// query (at decode shape two or four waves share one) and scores it against
// 32-key slots.  Two waves per SIMD let one wave's VALU epilogue overlap the
// other's MFMAs.
//
// fp8 scores use the abs form of the head sum (abs_wsum) plus the linear
// term q''/2 . k on the matrix cores.  Each wave loads whole 16-key blocks of
// every tile; as soon as its own loads have landed it scores its blocks
// against the linear-term parts of all the workgroup's queries (four queries
// per v_mfma_f32_16x16x128_f8f6f4) and writes the results to an LDS row per
// query; the tile's barrier then publishes them to the query owners.

constexpr int kScanWaves = 8;
constexpr int kTileBytes = 32768;          // key bytes per tile at decode shape (R > 1) and for narrow rows
constexpr int kTileBytesWide = 65536;      // one wave per query, rows of 128 bytes or more
constexpr int kTileBytesWideFp8 = 49152;   // fp8: 384 keys, so that two stages and the linear-term rows fit
constexpr int kScanStagesWide = 2;         // wide tiles: one scored while the next loads
constexpr int kScanStages = 3;             // 32 KB tiles, one wave per query: one scored, two loading
constexpr int kScanStagesFew = 4;          // at decode shape (R > 1), where the key stream bounds the scan
constexpr int kLinPad = 16;                // floats of padding per linear-term row (spreads LDS banks)
constexpr int kSlotValuPerMfma = 8;        // fp8 prefill slots: head-sum VALU instructions issued behind each MFMA
constexpr int kLinLead = 2;                // fp8 prefill: the next tile's linear-term rows, this many slots before the tile's end

template <int DT, int D, int TB = kTileBytes>
struct TileGeom {
    static constexpr int RB = D * DTraits<DT>::ESZ;        // bytes per key row
    static constexpr int CPR = RB / 16;                    // 16-byte chunks per row
    static constexpr int TILE_BYTES = TB;
    static constexpr int TK = TB / RB;                     // keys per tile
    static constexpr int NINST = TK * CPR / 64;            // wave-wide 1 KB loads per tile
    static constexpr int PER_WAVE = NINST / kScanWaves;
    static constexpr int SCALE_BYTES = (DT == DT_FP8) ? TK * 4 : 0;
    static constexpr int STAGE_BYTES = TB + SCALE_BYTES;
    static_assert(NINST % kScanWaves == 0, "tile loads split evenly over the waves");
    static_assert(TK % 64 == 0, "per-key scales load in whole 64-lane wave loads");
    static constexpr int SCALE_INST = (DT == DT_FP8) ? TK / 64 : 0;       // wave loads of scales per tile
    static_assert(SCALE_INST <= kScanWaves, "at most one scale load per wave");
    // fp8 linear term: each wave loads (and then scores) whole 16-key blocks
    static constexpr bool LIN = DT == DT_FP8;
    static constexpr int IPB = (16 * RB >= 1024) ? 16 * RB / 1024 : 1;    // 1 KB loads per 16-key block
    static constexpr int LBW = TK / (16 * kScanWaves);                    // 16-key blocks per wave and tile
    static constexpr int LROW = TK + kLinPad;                              // floats per linear-term row
    static_assert(!LIN || (16 * RB >= 1024 && PER_WAVE % IPB == 0 && TK % (16 * kScanWaves) == 0),
                  "fp8 tiles split into whole 16-key blocks per wave");
};

// Tile size of a scan with R waves per query.  At one wave per query
// (prefill shape) the MFMA/VALU work bounds the scan, and each tile ends in a
// workgroup barrier at which every wave stops issuing, so the tiles are as
// large as two stages allow (64 KB, measured 1.5 % faster than 32 KB
// tiles with three stages; 48 KB for fp8, whose linear-term rows take LDS
// too).  WIDE needs rows of at least 128 bytes (at most 512 keys, whose
// scales take one wave load each) and LDS for two such stages, which the
// launch checks against the bin count.  Decode shapes keep 32 KB tiles.
template <int DT, int D, int R, bool WIDE>
struct ScanShape {
    static_assert(!WIDE || (R == 1 && D * DTraits<DT>::ESZ >= 128), "wide tiles: one wave per query, rows >= 128 B");
    static constexpr int TB = WIDE ? (DT == DT_FP8 ? kTileBytesWideFp8 : kTileBytesWide) : kTileBytes;
};

// Index of the wave's j-th 1 KB load of a tile.  fp8: wave w loads the rows
// of the 16-key blocks w, w + 8, w + 16, ... (IPB consecutive loads each), so
// that it can score them once its own loads have landed; otherwise the loads
// of the waves interleave.
template <class G>
__device__ __forceinline__ int load_inst(int wave, int j) {
    if constexpr (G::LIN) return G::IPB * (kScanWaves * (j / G::IPB) + wave) + j % G::IPB;
    else return wave + j * kScanWaves;
}

// Per-lane byte offsets, inside a tile, of the wave's share of the tile's
// direct loads (fixed for the whole kernel: row r of the tile, swizzled chunk).
template <int DT, int D, int TB>
struct TileOffsets {
    uint32_t key[TileGeom<DT, D, TB>::PER_WAVE];
};

template <int DT, int D, int TB>
__device__ __forceinline__ void tile_offsets(TileOffsets<DT, D, TB>& o, int wave, int lane) {
    using G = TileGeom<DT, D, TB>;
#pragma unroll
    for (int j = 0; j < G::PER_WAVE; ++j) {
        const int p = load_inst<G>(wave, j) * 64 + lane;
        const int r = p / G::CPR, pc = p % G::CPR;
        o.key[j] = (uint32_t)(r * G::RB + (pc ^ chunk_swz<G::RB, G::CPR>(r)) * 16);
    }
}

// Issue this wave's share of the direct loads of the tile starting at key0.
// A tile wholly inside the context loads from one wave-uniform base plus the
// precomputed lane offsets; the last, partial tile clamps its rows (keys past
// the context re-read the last one).  ASYNC: issued as inline assembly,
// ordered by the caller's own vmcnt waits (the builtin form makes the
// compiler drain every load before each barrier).
template <int DT, int D, int TB, bool ASYNC = false>
__device__ __forceinline__ void load_tile(const IdxArgs& a, const TileOffsets<DT, D, TB>& to, int key0, uint8_t* st,
                                          int wave, int lane) {
    using G = TileGeom<DT, D, TB>;
    if (tile_inside(key0, G::TK, a.L)) {
        const uint8_t* tb = a.k + (size_t)key0 * G::RB;
#pragma unroll
        for (int j = 0; j < G::PER_WAVE; ++j) {
            uint8_t* dst = st + load_inst<G>(wave, j) * 1024;
            if constexpr (ASYNC) lds_direct16_async(tb, to.key[j], dst);
            else lds_direct16(tb + to.key[j], dst);
        }
        if constexpr (DT == DT_FP8) {
            const float* sb = a.k_scale + key0;
#pragma unroll
            for (int j = wave; j < G::TK / 64; j += kScanWaves) {
                if constexpr (ASYNC) lds_direct4_async(sb, (uint32_t)(j * 256 + lane * 4), st + TB + j * 256);
                else lds_direct4(sb + j * 64 + lane, st + TB + j * 256);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < G::PER_WAVE; ++j) {
        const int inst = load_inst<G>(wave, j);
        const int p = inst * 64 + lane;
        const int r = p / G::CPR, pc = p % G::CPR;
        const int c = pc ^ chunk_swz<G::RB, G::CPR>(r);
        const int key = min(key0 + r, a.L - 1);
        if constexpr (ASYNC) lds_direct16_async(a.k + (size_t)key * G::RB + c * 16, st + inst * 1024);
        else lds_direct16(a.k + (size_t)key * G::RB + c * 16, st + inst * 1024);
    }
    if constexpr (DT == DT_FP8) {
#pragma unroll
        for (int j = wave; j < G::TK / 64; j += kScanWaves) {
            const int key = min(key0 + j * 64 + lane, a.L - 1);
            if constexpr (ASYNC) lds_direct4_async(a.k_scale + key, st + TB + j * 256);
            else lds_direct4(a.k_scale + key, st + TB + j * 256);
        }
    }
}

template <int DT, int D>
__device__ __forceinline__ void read_frag(HalfRow<DT, D>& f, const uint8_t* st, int r0, int lane) {
    using G = TileGeom<DT, D>;
    const int r = r0 + (lane & 31), h = lane >> 5;
#pragma unroll
    for (int i = 0; i < HalfRow<DT, D>::NV; ++i) {
        const int c = h * (G::CPR / 2) + i;
        f.v[i] = *reinterpret_cast<const u32x4*>(st + r * G::RB + ((c ^ chunk_swz<G::RB, G::CPR>(r)) * 16));
    }
}

// Linear-term operands of the workgroup's queries in LDS: NG groups of four
// queries x four parts, 16 rows of 128 bytes each (zero past D and for
// missing queries), rows 144 bytes apart: the 16 rows a fragment read touches
// then fall on distinct banks (a 128-byte stride put eight of them on one).
constexpr int kLinRowBytes = 144;
constexpr int kLinGroupBytes = 16 * kLinRowBytes;

// The linear term of the wave's own 16-key blocks of a tile (rows it loaded
// itself, so only its own loads need to have landed) for every query of the
// workgroup, into the LDS rows lb[query][key in tile].
template <int DT, int D, int TB, int QPG>
__device__ __forceinline__ void lin_phase(const uint8_t* st, const uint8_t* apart, float* lb, int wave, int lane) {
    using G = TileGeom<DT, D, TB>;
    constexpr int NG = (QPG + 3) / 4;
    const int r = lane & 15, ks = lane >> 4;
    LinFrag af[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const u32x4* p = reinterpret_cast<const u32x4*>(apart + g * kLinGroupBytes + r * kLinRowBytes + ks * 32);
        af[g].v[0] = p[0];
        af[g].v[1] = p[1];
    }
#pragma unroll
    for (int b = 0; b < G::LBW; ++b) {
        const int row = 16 * (wave + kScanWaves * b) + r;
        LinFrag bf;
        if (32 * ks < D) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = 2 * ks + i;
                bf.v[i] = *reinterpret_cast<const u32x4*>(st + row * G::RB + ((c ^ chunk_swz<G::RB, G::CPR>(row)) * 16));
            }
        } else {
            bf.v[0] = bf.v[1] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float tl = lin_combine(lin_mfma(af[g], bf));
            const int q = 4 * g + ks;
            if (q < QPG) lb[q * G::LROW + row] = tl;
        }
    }
}

// LDS the fused scan needs beyond its tile stages: per-wave histograms and
// staging lists, and for fp8 the linear-term operands and two buffers of
// linear-term rows.
template <int DT, int D, int TB, int QPG>
constexpr size_t scan_extra_lds(int nbins) {
    using G = TileGeom<DT, D, TB>;
    const size_t fixed = (size_t)kScanWaves * nbins * 4 + (size_t)kScanWaves * kStage * 8;
    if constexpr (!G::LIN) return fixed;
    return fixed + (size_t)((QPG + 3) / 4) * kLinGroupBytes + (size_t)2 * QPG * G::LROW * 4;
}

// R waves per query: a workgroup holds kScanWaves / R queries, and the R
// waves of a query take every R-th 64-key block of each tile.  R = 1 at
// prefill shape; a decode step of one to four queries uses R = 4 or 2, so
// that the waves score real queries instead of empty slots.
// FULL: the unfused baseline's scoring, the same loop writing every causal
// score to the T x L matrix instead of gating it.
template <int DT, int D, int HB, int R, bool WIDE, int NST, bool FULL = false>
__global__ __launch_bounds__(512) void scan_kernel(IdxArgs a) {
    using SS = ScanShape<DT, D, R, WIDE>;
    using G = TileGeom<DT, D, SS::TB>;
    constexpr bool ASYNC = true;   // loads as inline assembly from a uniform base (no per-load VALU)
    constexpr int QPG = kScanWaves / R;
    constexpr int NB = G::TK / 64;                                         // 64-key blocks per tile
    constexpr int NG = (QPG + 3) / 4;                                      // linear-term query groups
    static_assert(R >= 1 && NB % R == 0, "a tile's blocks split evenly over a query's waves");
    extern __shared__ __attribute__((aligned(16))) uint8_t shm[];
    const int nbins = a.nbins;
    uint8_t* tiles = shm;                                                  // NST stages
    uint32_t* hist = reinterpret_cast<uint32_t*>(shm + NST * G::STAGE_BYTES);  // [waves][nbins]
    uint2* stage = reinterpret_cast<uint2*>(hist + kScanWaves * nbins);    // [waves][kStage]
    uint8_t* apart = reinterpret_cast<uint8_t*>(stage + kScanWaves * kStage);      // fp8: [NG][16][128]
    float* lbuf = reinterpret_cast<float*>(apart + NG * kLinGroupBytes);            // fp8: [2][QPG][LROW]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
    const int qg = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
    const int t0 = qg * QPG;
    // the rescan pass takes its queries from the list of overflowed rows
    const int n_rows = (a.pass == 2) ? (int)__builtin_amdgcn_readfirstlane(*a.ovf_count) : a.T;
    if (t0 >= n_rows) return;                                             // the whole workgroup
    auto qmap = [&](int i) { return (a.pass == 2) ? (i < n_rows ? a.ovf_list[i] : a.T) : i; };
    const int t = qmap(t0 + wave / R);                                     // the wave's query
    TileOffsets<DT, D, SS::TB> toff;
    tile_offsets<DT, D, SS::TB>(toff, wave, lane);
    const int sub = wave % R;                                              // its blocks: sub, sub + R, ...
    const uint32_t k = (uint32_t)a.topk;
    uint32_t* hl = hist + wave * nbins;                                    // the wave's own counts
    uint2* stg = stage + wave * kStage;                                    // and staging list

    for (int i = lane; i < nbins; i += 64) hl[i] = 0u;

    // keys any query of the group can see, split into tile-aligned ranges
    int e = 0;
    for (int i = lane; i < QPG; i += 64) {
        const int tt = qmap(t0 + i);
        if (tt < a.T) e = max(e, min(a.pos[tt], a.L - 1) + 1);
    }
    const int kend = __builtin_amdgcn_readfirstlane(wave_max_i32(e));   // uniform: every lane holds the max
    const KeyRange kr = split_range(kend, a.n_splits, split, G::TK);
    const int k_lo = kr.lo, k_hi = kr.hi;

    const bool tv = t < a.T;
    const int my_pos = tv ? min(a.pos[t], a.L - 1) : -1;
    const int wave_end = min(k_hi, my_pos + 1);
    Meta m{0.0f, 1.0f, 0, 0};
    if (tv && !FULL) m = reinterpret_cast<const Meta*>(a.meta)[t];
    int thr = m.thr0;
    // rescan: gate at the first pass's final threshold bin (a refresh result,
    // so at most the true one)
    if (a.pass == 2 && tv) thr = max(thr, a.thr_fin[t]);
    float tau = (tv && !FULL) ? initial_gate(thr, m, nbins, a.topk) : -INFINITY;

    QueryRegs<DT, D, HB> ra;
    load_query<DT, D, HB>(ra, a, t);
    float inv_own = 0.0f;   // fp8: 1/S of the query's linear-term parts
    if constexpr (G::LIN) {
        // the workgroup's linear-term operands into LDS, 16 bytes per thread
        for (int i = threadIdx.x; i < NG * 16 * 8; i += kScanWaves * 64) {
            const int g = i / 128, r = (i / 8) % 16, c = i % 8;
            const int ql = 4 * g + (r >> 2), tq = qmap(t0 + ql);
            u32x4 v{0u, 0u, 0u, 0u};
            if (ql < QPG && tq < a.T && 16 * c < D)
                v = *reinterpret_cast<const u32x4*>(a.qlin + ((size_t)tq * 4 + (r & 3)) * D + 16 * c);
            *reinterpret_cast<u32x4*>(apart + g * kLinGroupBytes + r * kLinRowBytes + 16 * c) = v;
        }
        if (tv) inv_own = a.qinv[t];
    }
    if constexpr (ASYNC) drain_vm_loads();   // the loop's waits then cover tile loads only
    if constexpr (G::LIN) __syncthreads();   // operands in LDS before the first linear-term phase

    int cnt = 0;   // staged entries (wave-uniform)
    int fl = 0;    // batches written back

    const int fb = a.flush;   // write-back batch: 32 or 64 entries
    auto flush = [&]() {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&a.tail[t], (uint32_t)fb);
        base = lane0_u32(base);
        const uint2 en = stg[lane];
        if (lane < fb && (int64_t)base + lane < a.ccap) a.cand[(size_t)t * a.ccap + base + lane] = en;
        const int rem = cnt - fb;   // < 64: at most 63 + 64 entries were staged
        uint2 r{0u, 0u};
        if (lane < rem) r = stg[fb + lane];
        if (lane < rem) stg[lane] = r;
        cnt = rem;
        ++fl;
        uint32_t* hg = a.hist_g ? a.hist_g + (size_t)t * nbins : nullptr;
        if (hg) {
            // shared threshold: move the counts gathered since the last flush
            // into the query's histogram in device memory (the LDS copy then
            // holds only what this wave has not yet added there)
            for (int b = lane; b < nbins; b += 64) {
                const uint32_t v = hl[b];
                if (v) {
                    atomicAdd(&hg[b], v);
                    hl[b] = 0u;
                }
            }
        }
        wait_vm<0>();   // keep the in-flight vector-memory ops to tile loads only
        if (a.refresh_every > 0 && fl % a.refresh_every == 0) {
            // top-down recount (of every split's counts, when shared); a plain
            // overwrite that can only raise the threshold.  Counts cover real
            // causal keys only, so the new bin is at most the true one.
            if (hg)
                for (int b = lane; b < nbins; b += 64) hl[b] = __hip_atomic_load(&hg[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const SuffixPick p = suffix_pick(hl, nbins, k);
            if (hg)
                for (int b = lane; b < nbins; b += 64) hl[b] = 0u;
            if (p.bin > thr) {
                thr = p.bin;
                tau = tau_of(thr, m.smin, m.delta, nbins);
            }
        }
    };

    // Gate of 64 consecutive keys, lane l holding key base + l.  The causal
    // bound is a scalar lane mask (keys past the query's position), so the
    // common case costs one compare and a scalar AND.
    const int pos_u = __builtin_amdgcn_readfirstlane(my_pos);
    auto process = [&](float I, int base) {
        if constexpr (FULL) {   // unfused: every causal score to the matrix
            if (base + lane <= pos_u) a.S[(size_t)t * a.L + base + lane] = I;
            return;
        }
        const int lim = pos_u - base;   // lanes 0..lim are causal
        const uint64_t causal = lim >= 63 ? ~0ull : (lim < 0 ? 0ull : ((2ull << lim) - 1ull));
        const uint64_t mask = __builtin_amdgcn_ballot_w64(I >= tau) & causal;
        if (mask) {
            if ((mask >> lane) & 1ull) {
                atomicAdd(&hl[bin_of(I, m.smin, m.delta, nbins)], 1u);
                stg[cnt + mbcnt(mask)] = make_uint2((uint32_t)(base + lane), __float_as_uint(I));
            }
            cnt += __popcll(mask);
            while (cnt >= fb) flush();   // twice at most, with batches of 32
        }
    };

    constexpr int LPW_HI = G::PER_WAVE + (G::SCALE_INST > 0 ? 1 : 0);   // loads per tile, waves < SCALE_INST
    constexpr int LPW_LO = G::PER_WAVE;                                  // loads per tile, other waves
    // (issuing the first tiles before the query state measured 3 us slower at decode shape)
    const int ntiles = (k_hi > k_lo) ? (k_hi - k_lo + G::TK - 1) / G::TK : 0;
    static_assert(NST >= 2 && NST <= 4, "one to three tiles load while one is scored");
#pragma unroll
    for (int j = 0; j < NST - 1; ++j)
        if (j < ntiles) load_tile<DT, D, SS::TB, ASYNC>(a, toff, k_lo + j * G::TK, tiles + j * G::STAGE_BYTES, wave, lane);
    // The wave's own loads of tile i have landed once at most the loads of
    // the later tiles issued so far remain (vector-memory operations complete
    // in issue order; the candidate flushes drain their own).
    auto wait_tile = [&](int i) {
        const int later = min(NST - 2, ntiles - 1 - i);
        if (wave < G::SCALE_INST) {
            if (NST == 4 && later >= 2) wait_vm<2 * LPW_HI>(); else if (later >= 1) wait_vm<LPW_HI>(); else wait_vm<0>();
        } else {
            if (NST == 4 && later >= 2) wait_vm<2 * LPW_LO>(); else if (later >= 1) wait_vm<LPW_LO>(); else wait_vm<0>();
        }
    };
    // fp8 at prefill shape: the slot pipeline runs on across tiles.  A wave
    // computes the next tile's linear-term rows of its own key blocks
    // kLinLead slots before the end of the current tile, behind MFMAs in
    // flight (they go to the other row buffer, which nobody reads after the
    // barrier that starts the current tile), and the gate of a tile's last
    // pair waits for the next tile's first MFMAs.
    constexpr bool CONT = G::LIN && R == 1 && HalfRow<DT, D>::NV <= 4;   // the fp8 branch of the slot loop below
    auto lin_rows = [&](int i) { return lbuf + (size_t)(i & 1) * QPG * G::LROW; };
    float ga = 0.0f, gb = 0.0f, glin = 0.0f, gsk = 0.0f;   // the pair waiting for its gate
    int gkey = 0;                                          // and its first key
    bool gpend = false;
    if constexpr (CONT) {
        if (ntiles > 0) {
            wait_tile(0);
            lin_phase<DT, D, SS::TB, QPG>(tiles, apart, lin_rows(0), wave, lane);
        }
    }
    int sbuf = 0;   // stage holding tile `it`
    for (int it = 0; it < ntiles; ++it) {
        const uint8_t* st = tiles + sbuf * G::STAGE_BYTES;
        float* lrow = lin_rows(it);   // this tile's linear-term rows
        if constexpr (!CONT) {
            wait_tile(it);
            if constexpr (G::LIN) lin_phase<DT, D, SS::TB, QPG>(st, apart, lrow, wave, lane);
        }
        __syncthreads();
        const int key0 = k_lo + it * G::TK;
        const bool act = tv && key0 < wave_end;   // some key of this tile is visible to the wave's query
        if (it + NST - 1 < ntiles) {   // into the stage every wave finished scoring before the barrier
            const int nb = (sbuf + NST - 1) % NST;
            load_tile<DT, D, SS::TB, ASYNC>(a, toff, k_lo + (it + NST - 1) * G::TK, tiles + nb * G::STAGE_BYTES, wave, lane);
        }
        sbuf = (sbuf + 1) % NST;
        const float* sks = reinterpret_cast<const float*>(st + SS::TB);
        const float* lq = lrow + (wave / R) * G::LROW;                  // the wave's query's linear terms
        // the next tile's linear-term rows of this wave's own key blocks
        auto next_lin = [&]() {
            if (it + 1 < ntiles) {
                wait_tile(it + 1);
                lin_phase<DT, D, SS::TB, QPG>(tiles + sbuf * G::STAGE_BYTES, apart, lin_rows(it + 1), wave, lane);
            }
        };
        if (!act) {   // nothing of this tile is visible to the wave's query
            if constexpr (CONT) {
                if (gpend) {
                    process(lin_score(glin, inv_own, combine_halves(ga, gb), gsk), gkey);
                    gpend = false;
                }
                next_lin();
            }
            continue;
        }
        if constexpr (DT == DT_F32) {
            // fp32: a whole fragment is 16 registers per 16 dimensions and
            // the query's head blocks as many again per block, so the slots
            // are scored one after the other and each fragment is read and
            // consumed 16 dimensions at a time; holding it whole spills
            constexpr int NS = G::TK / 32 / R, NV = HalfRow<DT, D>::NV, PV = 2;
            const int h = lane >> 5;
            float pprev = 0.0f;
            for (int sl = 0; sl < NS; ++sl) {
                const int r0 = 64 * (sub + R * (sl >> 1)) + 32 * (sl & 1), r = r0 + (lane & 31);
                v16f acc[HB];
#pragma unroll
                for (int mm = 0; mm < HB; ++mm) acc[mm] = v16f{};
#pragma unroll
                for (int pc = 0; pc < NV / PV; ++pc) {
                    u32x4 kv[PV];
#pragma unroll
                    for (int i = 0; i < PV; ++i) {
                        const int c = h * (G::CPR / 2) + pc * PV + i;
                        kv[i] = *reinterpret_cast<const u32x4*>(st + r * G::RB + ((c ^ chunk_swz<G::RB, G::CPR>(r)) * 16));
                    }
#pragma unroll
                    for (int j = 0; j < 4 * PV; ++j)
#pragma unroll
                        for (int mm = 0; mm < HB; ++mm)
                            acc[mm] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                __uint_as_float(ra.q[mm].v[pc * PV + (j >> 2)][j & 3]), __uint_as_float(kv[j >> 2][j & 3]),
                                acc[mm], 0, 0, 0);
                }
                const float p = relu_wsum<HB>(acc, ra.w);
                if (sl & 1) process(combine_halves(pprev, p), key0 + r0 - 32);
                else pprev = p;
            }
        } else if constexpr (HalfRow<DT, D>::NV > 4) {
            // wide fragments (bf16/fp32 at D = 128): the same software pipeline
            // as below with one fragment buffer (a wide fragment takes twice
            // the registers): slot s+1's fragment is read just before its MFMAs,
            // which are issued before the ReLU*w reduction of slot s (2.4 %
            // faster at bf16 than scoring a block's two slots one after the
            // other); keys past the query's position fail the gate in process
            constexpr int NS = G::TK / 32 / R;
            auto row0 = [&](int j) { return 64 * (sub + R * (j >> 1)) + 32 * (j & 1); };
            HalfRow<DT, D> kf;
            v16f accC[HB], accN[HB];
            read_frag<DT, D>(kf, st, row0(0), lane);
            mfma_1slot<DT, D, HB>(ra.q, kf, accC);
            float pprev = 0.0f;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                if constexpr (R == 1) {   // priority falling through the tile, as in the fp8 loop
                    if (sl == 0) set_wave_prio(3);
                    else if (sl == NS / 2) set_wave_prio(2);
                    else if (sl == 3 * NS / 4) set_wave_prio(1);
                    else if (sl == NS - 1) set_wave_prio(0);
                }
                if (sl + 1 < NS) {
                    read_frag<DT, D>(kf, st, row0(sl + 1), lane);
                    mfma_1slot<DT, D, HB>(ra.q, kf, accN);
                }
                const float p = relu_wsum<HB>(accC, ra.w);
                if (sl & 1) {
                    const int r0 = row0(sl - 1);
                    process(combine_halves(pprev, p), key0 + r0);
                } else {
                    pprev = p;
                }
                if (sl + 1 < NS) {
#pragma unroll
                    for (int mm = 0; mm < HB; ++mm) accC[mm] = accN[mm];
                }
            }
        } else if constexpr (DT == DT_FP8 && R == 1) {
            // fp8 at prefill shape: the pipeline below, with each pair's gate
            // deferred into the next slot, just behind that slot's first
            // MFMA (for a tile's last pair: the next tile's).  The gate's
            // dependent chain (half exchange, linear term, key scale,
            // compare, ballot, branch) then runs while the matrix core
            // works, instead of leaving it idle at the end of every other
            // slot (which a wave running alone, after its SIMD partner
            // reached the tile's barrier, otherwise exposes).  A gate one
            // slot later sees a threshold at most one refresh staler: still
            // safe.
            constexpr int NS = G::TK / 32;
            constexpr int KS = HalfRow<DT, D>::KSTEPS;
            constexpr int VPM = kSlotValuPerMfma;
            auto row0 = [&](int j) { return 64 * (j >> 1) + 32 * (j & 1); };
            HalfRow<DT, D> kf[2];
            v16f accC[HB], accN[HB];
            read_frag<DT, D>(kf[0], st, row0(0), lane);
            mfma_1slot<DT, D, HB>(ra.q, kf[0], accC);
            if (NS > 1) read_frag<DT, D>(kf[1], st, row0(1), lane);
            float pprev = 0.0f;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                // A wave's priority falls as it works through the tile, so
                // that of the two waves sharing a SIMD the one behind issues
                // first.  Left to the oldest-first arbitration, one wave ran
                // ahead and then waited at the barrier for a quarter of the
                // tile while its partner finished alone.
                if (sl == 0) set_wave_prio(3);
                else if (sl == NS / 2) set_wave_prio(2);
                else if (sl == 3 * NS / 4) set_wave_prio(1);
                else if (sl == NS - 1) set_wave_prio(0);
                const HalfRow<DT, D>& kn = kf[(sl + 1) & 1];
                if (sl + 1 < NS) {
                    accN[0] = v16f{};
                    mfma_step<DT, D>(ra.q[0], kn, 0, accN[0]);
                }
                if (gpend) {
                    // the gate's chain starts here, not at the end of the
                    // previous slot: a region boundary behind the MFMA, and an
                    // empty asm that the chain's inputs pass through
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("" : "+v"(ga), "+v"(gb), "+v"(glin), "+v"(gsk));
                    process(lin_score(glin, inv_own, combine_halves(ga, gb), gsk), gkey);
                    gpend = false;
                }
                // the last slots' MFMAs are in flight: the next tile's
                // linear-term rows now, the head sums behind them
                if (sl == NS - kLinLead) next_lin();
                if (sl & 1) {   // this pair's linear terms and key scales, read early
                    const int gr0 = row0(sl - 1);
                    gkey = key0 + gr0;
                    glin = lq[gr0 + lane];
                    gsk = sks[gr0 + lane];
                }
                if (sl + 1 < NS) {
#pragma unroll
                    for (int mm = 1; mm < HB; ++mm) {
                        accN[mm] = v16f{};
                        mfma_step<DT, D>(ra.q[mm], kn, 0, accN[mm]);
                    }
#pragma unroll
                    for (int j = 1; j < KS; ++j)
#pragma unroll
                        for (int mm = 0; mm < HB; ++mm) mfma_step<DT, D>(ra.q[mm], kn, j, accN[mm]);
                    if (sl + 2 < NS) read_frag<DT, D>(kf[sl & 1], st, row0(sl + 2), lane);
                }
                const float p = abs_wsum<HB>(accC, ra.w);
                if (sl + 1 < NS) {
                    // issue order after the gate: the fragment reads two slots
                    // ahead, then VPM head-sum VALU instructions behind each of
                    // the slot's remaining MFMAs
                    if (sl & 1 || sl == 0) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // first MFMA
                    if (sl + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, HalfRow<DT, D>::NV, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
#pragma unroll
                    for (int g = 1; g < HB * KS; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
                    }
                }
                if (sl & 1) {
                    ga = pprev;
                    gb = p;
                    gpend = true;
                } else {
                    pprev = p;
                }
                if (sl + 1 < NS) {
#pragma unroll
                    for (int mm = 0; mm < HB; ++mm) accC[mm] = accN[mm];
                }
                __builtin_amdgcn_sched_barrier(0);   // each slot its own scheduling region
            }
        } else {
            // 32-key slots, software-pipelined: the MFMAs of slot s+1 are issued
            // before the head sum of slot s, so the matrix core and the VALU of
            // one wave overlap; two slots make one 64-key block.  The wave's
            // slot j is half (j & 1) of block sub + R * (j / 2).  Key fragments
            // are double-buffered: slot s+2's LDS reads go out after slot s+1's
            // MFMAs and land during slot s's reduction (0.5 % faster than
            // reading each fragment just before its MFMAs).
            constexpr int NS = G::TK / 32 / R;
            auto row0 = [&](int j) { return 64 * (sub + R * (j >> 1)) + 32 * (j & 1); };
            HalfRow<DT, D> kf[2];
            v16f accC[HB], accN[HB];
            read_frag<DT, D>(kf[0], st, row0(0), lane);
            mfma_1slot<DT, D, HB>(ra.q, kf[0], accC);
            if (NS > 1) read_frag<DT, D>(kf[1], st, row0(1), lane);
            float pprev = 0.0f;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                if (sl + 1 < NS) {
                    mfma_1slot<DT, D, HB>(ra.q, kf[(sl + 1) & 1], accN);
                    if (sl + 2 < NS) read_frag<DT, D>(kf[sl & 1], st, row0(sl + 2), lane);
                }
                float p;
                if constexpr (DT == DT_FP8) p = abs_wsum<HB>(accC, ra.w);
                else p = relu_wsum<HB>(accC, ra.w);
                if constexpr (DT == DT_FP8 && R == 1) {
                    // issue order of the slot: its first MFMA, the LDS reads
                    // of the fragment two slots ahead, then the head sum's VALU
                    // instructions spread behind the MFMAs.  Left to itself the
                    // scheduler sinks half of those reads to just before their
                    // MFMA, which then waits on LDS
                    if (sl + 1 < NS) {
                        constexpr int NM = HB * HalfRow<DT, D>::KSTEPS;
                        constexpr int VPM = kSlotValuPerMfma;
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                        if (sl + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, HalfRow<DT, D>::NV, 0);   // LDS reads
                        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
#pragma unroll
                        for (int g = 1; g < NM; ++g) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
                        }
                    }
                }
                if (sl & 1) {
                    const int r0 = row0(sl - 1);
                    float I = combine_halves(pprev, p);
                    if constexpr (DT == DT_FP8) I = lin_score(lq[r0 + lane], inv_own, I, sks[r0 + lane]);
                    process(I, key0 + r0);
                } else {
                    pprev = p;
                }
                if (sl + 1 < NS) {
#pragma unroll
                    for (int mm = 0; mm < HB; ++mm) accC[mm] = accN[mm];
                }
                // each slot is its own scheduling region: otherwise the head sum
                // of slot s+1 (no branch separates an even slot from the next)
                // is hoisted right behind its own MFMAs and waits for them
                if constexpr (DT == DT_FP8 && R == 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if constexpr (CONT) {   // the last tile's last pair
        if (gpend) process(lin_score(glin, inv_own, combine_halves(ga, gb), gsk), gkey);
    }
    // final partial batch
    if (cnt > 0) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&a.tail[t], (uint32_t)cnt);
        base = lane0_u32(base);
        if (lane < cnt) {
            const uint2 en = stg[lane];
            if ((int64_t)base + lane < a.ccap) a.cand[(size_t)t * a.ccap + base + lane] = en;
        }
    }
    // first of two passes: the query's final threshold bin, for a rescan
    if (a.pass == 1 && tv && lane == 0) atomicMax(&a.thr_fin[t], thr);
}

// ---------------------------------------------------------------------------
// Select: finalize
// ---------------------------------------------------------------------------

constexpr int kRankMax = 512;   // threshold-bin entries ranked in LDS by counting

// 32-bit LDS words of the select's counters: max(nbins, 256), rounded up to even.
__host__ __device__ inline int fin_words(int nbins) { return ((nbins > 256 ? nbins : 256) + 1) & ~1; }

// Score row of query t: the caller's out_score row, or, for a sorted output
// without scores, an LDS row (the sort needs the scores; nothing reads them
// afterwards), else none.
__device__ __forceinline__ float* score_row(const IdxArgs& a, int t, float* lds_row) {
    if (a.out_score) return a.out_score + (size_t)t * a.topk;
    return a.sorted ? lds_row : nullptr;
}

// Select of one row (LiteTopK pages, "Selection").  Returns true, with the
// row's overflow flag set, when the candidate buffer overflowed and the row
// must be recomputed.  LDS (sh): fin_words(nbins) counters, then kRankMax
// rank keys and candidate entries, then the sort keys of a sorted output and,
// without out_score, its scores.
__device__ bool finalize_row(const IdxArgs& a, int t, uint32_t* sh) {
    __shared__ int s_pick;
    __shared__ uint32_t s_above, s_cnt, s_ocnt, s_mcnt;
    const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
    const int k = a.topk;
    const uint32_t n = a.tail[t];
    int32_t* out = a.out_idx + (size_t)t * k;
    uint64_t* rk = reinterpret_cast<uint64_t*>(sh + fin_words(a.nbins));        // [kRankMax]
    uint2* rent = reinterpret_cast<uint2*>(rk + kRankMax);                        // [kRankMax]
    uint64_t* sort_keys = reinterpret_cast<uint64_t*>(rent + kRankMax);
    float* osc = score_row(a, t, reinterpret_cast<float*>(sort_keys + (a.sorted ? sort_p2(k) : 0)));
    if (tid == 0 && a.stats) {
        atomicAdd((unsigned long long*)&a.stats->cand_written, (unsigned long long)n);
        atomicMax(&a.stats->max_cand_per_query, n);
        // stored candidates (every pass), this query's sample scores (once),
        // its outputs (by the pass that writes them: not a first pass whose
        // overflowed row is rescanned)
        const bool ovf = (int64_t)n > a.ccap;
        const uint64_t stored = ovf ? (uint64_t)a.ccap : (uint64_t)n;
        // sample scores stored for this query: a whole row on the one-launch
        // path, else one per distinct in-range sample key
        const uint64_t nsc = a.front_parts ? (uint64_t)a.n_sample : (uint64_t)*a.nu;
        const uint64_t b = 8ull * stored + (a.pass != 2 ? 4ull * nsc : 0ull) +
                           ((ovf && a.pass == 1) ? 0ull : 4ull * (uint64_t)k * (a.out_score ? 2u : 1u));
        atomicAdd((unsigned long long*)&a.stats->bytes_written, (unsigned long long)b);
    }
    if ((int64_t)n > a.ccap) {   // the buffer overflowed: a rescan or the fallback recomputes this row
        if (tid == 0) {
            a.flags[t] = 1u;
            if (a.stats && a.pass != 2) atomicAdd(&a.stats->overflow_rows, 1u);
        }
        return true;
    }
    const uint2* c = a.cand + (size_t)t * a.ccap;
    if (n <= (uint32_t)k) {      // only when the row has at most k valid keys: keep them all
        for (uint32_t i = tid; i < n; i += 256) {
            out[i] = (int32_t)c[i].x;
            if (osc) osc[i] = __uint_as_float(c[i].y);
        }
        for (int i = (int)n + tid; i < k; i += 256) {
            out[i] = -1;
            if (osc) osc[i] = __builtin_nanf("");
        }
        if (a.sorted) sort_row_output(out, osc, k, sort_keys);
        return false;
    }
    const Meta m = reinterpret_cast<const Meta*>(a.meta)[t];
    const int nbins = a.nbins;
    // up to kSelRegs candidates per thread are read once and kept in registers
    constexpr int kSelRegs = 16;
    const bool in_regs = n <= 256u * kSelRegs;
    uint2 ce[kSelRegs];
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < kSelRegs; ++r) {
            const uint32_t i = tid + 256u * r;
            ce[r] = (i < n) ? c[i] : make_uint2(0u, 0u);
        }
    }
    uint32_t* hist = sh;
    for (int i = tid; i < nbins; i += 256) hist[i] = 0u;
    if (tid == 0) {
        s_ocnt = 0u;
        s_mcnt = 0u;
    }
    __syncthreads();
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < kSelRegs; ++r)
            if (tid + 256u * r < n) atomicAdd(&hist[bin_of(__uint_as_float(ce[r].y), m.smin, m.delta, nbins)], 1u);
    } else {
        for (uint32_t i = tid; i < n; i += 256)
            atomicAdd(&hist[bin_of(__uint_as_float(c[i].y), m.smin, m.delta, nbins)], 1u);
    }
    __syncthreads();
    if (wave == 0) {   // final threshold bin: top-down recount of the candidates' bins
        const SuffixPick p = suffix_pick(hist, nbins, (uint32_t)k);
        if (lane == 0) {
            s_pick = p.bin;
            s_above = p.above;
            s_cnt = hist[p.bin];
        }
    }
    __syncthreads();
    const int bstar = s_pick;
    const uint32_t above = s_above;
    const bool ranked = s_cnt <= (uint32_t)kRankMax;   // the threshold bin fits the LDS ranking
    // bins strictly above the final threshold bin go straight to the output;
    // a small threshold bin is gathered into LDS
    auto emit = [&](const uint2 e) {
        const float I = __uint_as_float(e.y);
        const int b = bin_of(I, m.smin, m.delta, nbins);
        if (b > bstar) {
            const uint32_t p = atomicAdd(&s_ocnt, 1u);
            if (p < (uint32_t)k) {
                out[p] = (int32_t)e.x;
                if (osc) osc[p] = I;
            }
        } else if (ranked && b == bstar) {
            const uint32_t p = atomicAdd(&s_mcnt, 1u);   // < kRankMax: the bin holds s_cnt entries
            if (p < (uint32_t)kRankMax) {
                rk[p] = rank_key(I, (int)e.x);
                rent[p] = e;
            }
        }
    };
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < kSelRegs; ++r)
            if (tid + 256u * r < n) emit(ce[r]);
    } else {
        for (uint32_t i = tid; i < n; i += 256) emit(c[i]);
    }
    if (ranked) {
        // exact top-(k - above) inside the threshold bin: an entry is taken when
        // fewer than k - above entries of the bin rank before it (score desc,
        // index asc; the keys are distinct)
        __syncthreads();
        const uint32_t mm = min(s_mcnt, (uint32_t)kRankMax), need = (uint32_t)k - above;
        for (uint32_t i = tid; i < mm; i += 256) {
            const uint64_t key = rk[i];
            uint32_t r = 0;
            for (uint32_t j = 0; j < mm; ++j) r += (rk[j] > key) ? 1u : 0u;
            if (r < need) {
                const uint2 e = rent[i];
                const uint32_t p = atomicAdd(&s_ocnt, 1u);
                if (p < (uint32_t)k) {
                    out[p] = (int32_t)e.x;
                    if (osc) osc[p] = __uint_as_float(e.y);
                }
            }
        }
        if (a.sorted) sort_row_output(out, osc, k, sort_keys);
        return false;
    }
    // larger threshold bins: radix select on (score desc, index asc)
    uint64_t P = 0ull, mask = 0ull;
    uint32_t need = (uint32_t)k - above;
    uint32_t* h256 = sh;   // reuses the histogram space (nbins is no longer needed)
    for (int shift = 56; shift >= 0; shift -= 8) {
        __syncthreads();
        for (int i = tid; i < 256; i += 256) h256[i] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < n; i += 256) {
            const uint2 e = c[i];
            const float I = __uint_as_float(e.y);
            if (bin_of(I, m.smin, m.delta, nbins) == bstar) {
                const uint64_t key = rank_key(I, (int)e.x);
                if ((key & mask) == P) atomicAdd(&h256[(uint32_t)(key >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        if (wave == 0) {
            const SuffixPick p = suffix_pick(h256, 256, need);
            if (lane == 0) {
                s_pick = p.bin;
                s_above = p.above;
                s_cnt = h256[p.bin];
            }
        }
        __syncthreads();
        const uint32_t d = (uint32_t)s_pick;
        P |= (uint64_t)d << shift;
        mask |= 0xffull << shift;
        need -= s_above;
        if (s_cnt == need) break;   // every entry with this prefix is taken
    }
    for (uint32_t i = tid; i < n; i += 256) {
        const uint2 e = c[i];
        const float I = __uint_as_float(e.y);
        if (bin_of(I, m.smin, m.delta, nbins) == bstar && (rank_key(I, (int)e.x) & mask) >= P) {
            const uint32_t p = atomicAdd(&s_ocnt, 1u);
            if (p < (uint32_t)k) {
                out[p] = (int32_t)e.x;
                if (osc) osc[p] = I;
            }
        }
    }
    if (a.sorted) sort_row_output(out, osc, k, sort_keys);
    return false;
}

// Retrieval select (its own fallback kernel re-scores overflowed rows).
__global__ __launch_bounds__(256) void finalize_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];
    finalize_row(a, blockIdx.x, sh);
}

// ---------------------------------------------------------------------------
// Exact row select by 8-bit radix digits over a stream of (key, score)
// (overflow fallback and unfused baseline)
// ---------------------------------------------------------------------------

// Scores recomputed on the matrix cores (overflow fallback): wave w covers
// keys [base + 64w, base + 64w + 64) as two 32-key slots of the same query.
template <int DT, int D, int HB>
struct RescoreSource {
    QueryRegs<DT, D, HB> r;
    LinFrag lq;   // fp8: the query's linear-term parts in every row group
    float inv;
    const uint8_t* k;
    const float* ks;
    int L;
    __device__ __forceinline__ void get(int base, int nvalid, int& key, float& I, bool& valid) {
        const int wave = threadIdx.x >> 6, lane = lane_id();
        const int kb0 = base + 64 * wave;
        HalfRow<DT, D> ka, kbf;
        load_key<DT, D>(ka, k, min(kb0 + (lane & 31), L - 1));
        load_key<DT, D>(kbf, k, min(kb0 + 32 + (lane & 31), L - 1));
        I = score_2slots<DT, D, HB>(r, ka, r, kbf);
        key = kb0 + lane;
        if constexpr (DT == DT_FP8) I = lin_score(lin_one64_t<D>(lq, k, kb0, L), inv, I, ks[min(key, L - 1)]);
        valid = key < nvalid;
    }
};

__device__ __forceinline__ float* row_select_scores(const IdxArgs& a, int t, uint32_t* sh) {
    return score_row(a, t, reinterpret_cast<float*>(sh + 256 + 2 * (a.sorted ? sort_p2(a.topk) : 0)));
}

// Indexer select: finalize.  A row whose candidate buffer overflowed is, in a
// first pass of two, listed for the rescan (its buffer emptied); in the rescan
// pass (rows taken from that list) or a single pass, it takes the exact
// select over re-computed scores in the same workgroup.
template <int DT, int D, int HB>
__global__ __launch_bounds__(256) void select_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];
    int t = blockIdx.x;
    if (a.pass == 2) {
        if (blockIdx.x >= *a.ovf_count) return;
        t = a.ovf_list[blockIdx.x];
    }
    if (!finalize_row(a, t, sh)) return;
    __syncthreads();   // every thread has read the row's candidate count
    if (a.pass == 1) {
        if (threadIdx.x == 0) {
            a.ovf_list[atomicAdd(a.ovf_count, 1u)] = t;
            a.tail[t] = 0u;
        }
        return;
    }
    RescoreSource<DT, D, HB> src;
    load_query<DT, D, HB>(src.r, a, t);
    if constexpr (DT == DT_FP8) {
        load_lin_one<D>(src.lq, a, t);
        src.inv = a.qinv[t];
    }
    src.k = a.k;
    src.ks = a.k_scale;
    src.L = a.L;
    const int nvalid = max(min(a.pos[t], a.L - 1) + 1, 0);
    int32_t* out = a.out_idx + (size_t)t * a.topk;
    float* osc = row_select_scores(a, t, sh);
    select_row(src, nvalid, a.topk, out, osc, sh);
    if (a.sorted) sort_row_output(out, osc, a.topk, reinterpret_cast<uint64_t*>(sh + 256));
}

// ---------------------------------------------------------------------------
// Unfused baseline
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void unfused_select_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];
    const int t = blockIdx.x;
    MemSource src{a.S + (size_t)t * a.L};
    const int nvalid = a.pos ? max(min(a.pos[t], a.L - 1) + 1, 0) : a.L;   // no positions: every key
    int32_t* out = a.out_idx + (size_t)t * a.topk;
    float* osc = row_select_scores(a, t, sh);
    select_row(src, nvalid, a.topk, out, osc, sh);
    if (a.sorted) sort_row_output(out, osc, a.topk, reinterpret_cast<uint64_t*>(sh + 256));
}

// ---------------------------------------------------------------------------
// sample carried to the next chunk: keys ranked by selection count
// ---------------------------------------------------------------------------

__global__ void count_selected_kernel(const int32_t* idx, size_t n, int L, uint32_t* counts) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const int s = idx[i];
        if (s >= 0 && s < L) atomicAdd(&counts[s], 1u);
    }
}

// The first n keys in (count descending, index ascending) order:
//  1. a histogram of the counts over kNsBins values (the last bin takes every
//     count from kNsBins - 1 up);
//  2. from the top of it, the threshold count c* of the n-th key, the number
//     `above` of keys with larger counts and the number of ties to take;
//  3. keys counted above c* go to slots [0, above) in any order, and the
//     first `need` keys counted exactly c*, in index order, to [above, n)
//     (each workgroup's share of them found from the ties of the workgroups
//     before it).
// Only when c* falls in the last bin, where counts are not told apart, does
// one workgroup rank the whole count array instead.
struct NsHeader {
    uint32_t cstar, above, need, fallback, slot;
};

__global__ __launch_bounds__(256) void ns_hist_kernel(const uint32_t* counts, int L, int chunk, uint32_t* hist) {
    __shared__ uint32_t s_zero;
    if (threadIdx.x == 0) s_zero = 0u;
    __syncthreads();
    const int k0 = blockIdx.x * chunk, k1 = min(L, k0 + chunk);
    uint32_t zeros = 0;
    for (int key = k0 + threadIdx.x; key < k1; key += 256) {
        const uint32_t c = counts[key];
        if (c == 0u) ++zeros;
        else atomicAdd(&hist[min(c, (uint32_t)(kNsBins - 1))], 1u);
    }
    zeros = wave_sum_u32(zeros);
    if (lane_id() == 0 && zeros) atomicAdd(&s_zero, zeros);
    __syncthreads();
    if (threadIdx.x == 0 && s_zero) atomicAdd(&hist[0], s_zero);
}

__global__ __launch_bounds__(1024) void ns_pick_kernel(const uint32_t* hist, int n, NsHeader* hdr) {
    constexpr int PER = kNsBins / 1024;
    __shared__ uint32_t s_wsum[16];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    // thread tid holds bins [kNsBins - PER (tid + 1), kNsBins - PER tid): the
    // scan runs from the top bin down
    const int hi = kNsBins - PER * tid;
    uint32_t h[PER], part = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        h[i] = hist[hi - 1 - i];
        part += h[i];
    }
    uint32_t incl = wave_scan_add_u32(part);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t run = incl - part;   // keys in the bins above this thread's
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
    const uint32_t nn = (uint32_t)n;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (run < nn && run + h[i] >= nn) {   // exactly one bin holds the n-th key
            const uint32_t c = (uint32_t)(hi - 1 - i);
            hdr->cstar = c;
            hdr->above = run;
            hdr->need = nn - run;
            hdr->fallback = (c == (uint32_t)(kNsBins - 1)) ? 1u : 0u;
        }
        run += h[i];
    }
}

// Keys counted above c* to their slots; the ties of each workgroup counted.
__global__ __launch_bounds__(256) void ns_above_kernel(const uint32_t* counts, int L, int chunk, NsHeader* hdr,
                                                       uint32_t* ties, int32_t* out) {
    __shared__ uint32_t s_t;
    if (hdr->fallback) return;
    const uint32_t cstar = hdr->cstar;
    if (threadIdx.x == 0) s_t = 0u;
    __syncthreads();
    const int k0 = blockIdx.x * chunk, k1 = min(L, k0 + chunk);
    uint32_t t = 0;
    for (int b = k0; b < k1; b += 256) {
        const int key = b + (int)threadIdx.x;
        const uint32_t c = key < k1 ? counts[key] : 0u;
        const bool up = key < k1 && c > cstar;
        t += (key < k1 && c == cstar) ? 1u : 0u;
        const uint64_t m = __ballot(up);
        if (m) {
            uint32_t base = 0u;
            if (lane_id() == 0) base = atomicAdd(&hdr->slot, (uint32_t)__popcll(m));
            base = lane0_u32(base);
            if (up) out[base + mbcnt(m)] = key;
        }
    }
    t = wave_sum_u32(t);
    if (lane_id() == 0 && t) atomicAdd(&s_t, t);
    __syncthreads();
    if (threadIdx.x == 0) ties[blockIdx.x] = s_t;
}

// The first `need` ties in index order to slots [above, n).
__global__ __launch_bounds__(256) void ns_ties_kernel(const uint32_t* counts, int L, int chunk, const NsHeader* hdr,
                                                      const uint32_t* ties, int32_t* out) {
    __shared__ uint32_t s_wsum[4], s_base;
    if (hdr->fallback) return;
    const uint32_t cstar = hdr->cstar, need = hdr->need, above = hdr->above;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    uint32_t before = 0;   // ties of the workgroups before this one
    for (int b = tid; b < (int)blockIdx.x; b += 256) before += ties[b];
    before = wave_sum_u32(before);
    if (lane == 0) s_wsum[wave] = before;
    __syncthreads();
    if (tid == 0) s_base = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
    uint32_t base = s_base;
    if (base >= need) return;
    const int k0 = blockIdx.x * chunk, k1 = min(L, k0 + chunk);
    for (int b = k0; b < k1 && base < need; b += 256) {
        const int key = b + tid;
        const bool tie = key < k1 && counts[key] == cstar;
        const uint64_t m = __ballot(tie);
        __syncthreads();   // s_wsum of the previous round read by every thread
        if (lane == 0) s_wsum[wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t r = base + (uint32_t)mbcnt(m);
        for (int w = 0; w < wave; ++w) r += s_wsum[w];
        if (tie && r < need) out[above + r] = key;
        base += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    }
}

// Counts past the histogram's range decide: one workgroup ranks them all
// (counts below 2^24 order exactly as fp32).
__global__ __launch_bounds__(256) void ns_fallback_kernel(uint32_t* counts, int L, int n, const NsHeader* hdr,
                                                          int32_t* out) {
    extern __shared__ uint32_t sh[];
    if (!hdr->fallback) return;
    for (int i = threadIdx.x; i < L; i += 256) reinterpret_cast<float*>(counts)[i] = (float)counts[i];
    __syncthreads();
    MemSource src{reinterpret_cast<const float*>(counts)};
    select_row(src, L, n, out, nullptr, sh);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <int V> using ic = std::integral_constant<int, V>;

template <class F>
static bool dispatch(int dt, int D, int HB, F&& f) {
#define LTK_CASE(DTV, DV, HBV) \
    if (dt == DTV && D == DV && HB == HBV) { f(ic<DTV>{}, ic<DV>{}, ic<HBV>{}); return true; }
    LTK_CASE(DT_F32, 64, 1) LTK_CASE(DT_F32, 64, 2) LTK_CASE(DT_F32, 128, 1) LTK_CASE(DT_F32, 128, 2)
    LTK_CASE(DT_BF16, 64, 1) LTK_CASE(DT_BF16, 64, 2) LTK_CASE(DT_BF16, 128, 1) LTK_CASE(DT_BF16, 128, 2)
    LTK_CASE(DT_FP8, 64, 1) LTK_CASE(DT_FP8, 64, 2) LTK_CASE(DT_FP8, 128, 1) LTK_CASE(DT_FP8, 128, 2)
#undef LTK_CASE
    return false;
}

// Waves per query of the fused scan: 4 for one or two queries, 2 for three or
// four, else 1; at most the number of 64-key blocks in a tile.  (Eight waves
// on one query, one 32-key slot each, measured slower at decode shape.)
static int scan_waves_per_query(int T, int nb) {
    const int r = (T <= 2) ? 4 : (T <= 4) ? 2 : 1;
    return std::min(r, nb);
}

// sort keys of a sorted row, and its LDS scores when there is no out_score
static size_t sort_lds(const IdxArgs& a) {
    if (!a.sorted) return 0;
    return (size_t)sort_p2(a.topk) * 8 + (a.out_score ? 0 : (size_t)a.topk * 4);
}

// finalize_row's LDS: counters, the threshold bin's rank keys and positions, sort keys and scores
static size_t fin_lds_bytes(const IdxArgs& a) {
    return (size_t)fin_words(a.nbins) * 4 + (size_t)kRankMax * 16 + sort_lds(a);
}

template <class K>
static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)bytes);
}

hipError_t launch_prepare_sample(const IdxArgs& a, const int32_t* sample, int n_sample, const WsLayout& lay,
                                 uint8_t* ws, hipStream_t st) {
    if (n_sample <= kHashSampleMax) {
        int lg = 10;
        while ((1 << lg) < 2 * n_sample) ++lg;
        const size_t nz = (lay.bitmap - lay.zero_begin) / 4;   // the bitmap is not used
        const int zb = (int)std::min<size_t>((nz + 1023) / 1024, 512);
        const size_t lds = (size_t)4 << lg;
        allow_lds(sample_prep_kernel, lds);
        sample_prep_kernel<<<1 + std::max(zb, 1), 1024, lds, st>>>(sample, n_sample, a.L, lg,
                                                                     reinterpret_cast<uint32_t*>(ws + lay.zero_begin),
                                                                     nz, a.stats, a.sample_u, a.nu, a.n_sample,
                                                                     a.pos, a.T);
        return hipGetLastError();
    }
    const size_t nz = (lay.zero_end - lay.zero_begin) / 4;
    const int zb = (int)std::min<size_t>((nz + 255) / 256, 2048);
    zero_kernel<<<std::max(zb, 1), 256, 0, st>>>(reinterpret_cast<uint32_t*>(ws + lay.zero_begin), nz, a.stats);
    const int lg = sample_chunk_log2(a.L);
    uint32_t* ccount = reinterpret_cast<uint32_t*>(ws + lay.ccount);
    const int nwords = (a.L + 31) / 32;
    if (n_sample > 0) {
        sample_mark_kernel<<<(n_sample + 255) / 256, 256, 0, st>>>(sample, n_sample, a.L, a.bitmap);
        sample_count_kernel<<<sample_chunks(a.L), 256, 0, st>>>(a.bitmap, nwords, lg, ccount);
    }
    sample_compact_kernel<<<sample_chunks(a.L), 256, 0, st>>>(a.bitmap, nwords, lg, ccount, a.sample_u, a.nu);
    return hipGetLastError();
}


// Launches the fused scan variant that fits: decode shapes (R > 1 waves per
// query) need room for four tile stages; else one wave per query, with wide
// tiles where they fit.  FULL (the unfused baseline) always takes one wave
// per query.  Returns false when no variant fits the LDS.
template <int DT_, int D_, int HB_, bool FULL>
static bool run_scan_variant(const IdxArgs& args, hipStream_t st) {
    constexpr int NB = TileGeom<DT_, D_>::TK / 64;
    auto scan_lds = [&](auto Rc, auto Wc, auto Nc) -> size_t {
        constexpr int R_ = decltype(Rc)::value, N_ = decltype(Nc)::value;
        constexpr bool W_ = decltype(Wc)::value;
        using SS = ScanShape<DT_, D_, R_, W_>;
        return (size_t)N_ * TileGeom<DT_, D_, SS::TB>::STAGE_BYTES +
               scan_extra_lds<DT_, D_, SS::TB, kScanWaves / R_>(args.nbins);
    };
    auto launch_scan = [&](auto Rc, auto Wc, auto Nc) {
        constexpr int R_ = decltype(Rc)::value, N_ = decltype(Nc)::value;
        constexpr bool W_ = decltype(Wc)::value;
        constexpr int QPG = kScanWaves / R_;
        const size_t lds = scan_lds(Rc, Wc, Nc);
        allow_lds(scan_kernel<DT_, D_, HB_, R_, W_, N_, FULL>, lds);
        if (args.ev_scan_start) (void)hipEventRecord(args.ev_scan_start, st);
        scan_kernel<DT_, D_, HB_, R_, W_, N_, FULL>
            <<<((args.T + QPG - 1) / QPG) * args.n_splits, kScanWaves * 64, lds, st>>>(args);
        if (args.ev_scan_stop) (void)hipEventRecord(args.ev_scan_stop, st);
    };
    if constexpr (!FULL) {
        const int Rw = scan_waves_per_query(args.T, NB);
        if constexpr (NB % 4 == 0) {
            if (Rw == 4 && scan_lds(ic<4>{}, std::false_type{}, ic<kScanStagesFew>{}) <= kMaxLds) {
                launch_scan(ic<4>{}, std::false_type{}, ic<kScanStagesFew>{});
                return true;
            }
        }
        if constexpr (NB % 2 == 0) {
            if (Rw == 2 && scan_lds(ic<2>{}, std::false_type{}, ic<kScanStagesFew>{}) <= kMaxLds) {
                launch_scan(ic<2>{}, std::false_type{}, ic<kScanStagesFew>{});
                return true;
            }
        }
    }
    // (fp32 at D = 128 keeps 32 KB tiles: its wide variant spills registers)
    if constexpr (TileGeom<DT_, D_>::RB >= 128 && !(DT_ == DT_F32 && D_ >= 128)) {
        if (scan_lds(ic<1>{}, std::true_type{}, ic<kScanStagesWide>{}) <= kMaxLds) {
            launch_scan(ic<1>{}, std::true_type{}, ic<kScanStagesWide>{});
            return true;
        }
    }
    if (scan_lds(ic<1>{}, std::false_type{}, ic<kScanStages>{}) <= kMaxLds) {
        launch_scan(ic<1>{}, std::false_type{}, ic<kScanStages>{});
        return true;
    }
    if (scan_lds(ic<1>{}, std::false_type{}, ic<2>{}) <= kMaxLds) {
        launch_scan(ic<1>{}, std::false_type{}, ic<2>{});
        return true;
    }
    return false;
}

hipError_t launch_indexer_fused(int dt, int D, int HB, const IdxArgs& a, const FrontArgs* front, hipStream_t st) {
    const int nqg = (a.T + kQPG - 1) / kQPG;
    hipError_t err = hipSuccess;
    const bool ok = dispatch(dt, D, HB, [&](auto DTc, auto Dc, auto HBc) {
        constexpr int DT_ = decltype(DTc)::value, D_ = decltype(Dc)::value, HB_ = decltype(HBc)::value;
        if (front) {
            // the caller checked front_fits for this combination
            if constexpr (!(DT_ == DT_F32 && D_ == 128 && HB_ == 2)) {
                const int parts = a.front_parts;
                const size_t lds = front_lds_bytes(a.n_sample);
                const int zb = (int)std::min<size_t>((front->n_zero + kFrontThreads - 1) / kFrontThreads, 512);
                allow_lds(front_kernel<DT_, D_, HB_>, lds);
                front_kernel<DT_, D_, HB_><<<a.T * parts + std::max(zb, 1), kFrontThreads, lds, st>>>(
                    a, front->sample, front->n, front_log2_parts(a.n_sample), front_log2_slots(a.n_sample),
                    front->zero, front->n_zero);
                front_stats_kernel<<<a.T, kFrontThreads, 0, st>>>(a);
            } else {
                err = hipErrorInvalidValue;
                return;
            }
        } else {
            if constexpr (DT_ == DT_FP8) qlin_kernel<D_><<<a.T, 256, 0, st>>>(a);
            if (a.sg_k != nullptr) {
                // prefill shape: the sample's rows gathered, then scored by
                // the scan's full-score form into the sample-score rows
                constexpr int RB = D_ * DTraits<DT_>::ESZ;
                sample_gather_kernel<<<256, 256, 0, st>>>(a, RB);
                IdxArgs b = a;
                b.k = a.sg_k;
                b.k_scale = (DT_ == DT_FP8) ? a.sg_scale : nullptr;
                b.L = a.n_sample;
                b.pos = a.sg_pos;
                b.S = a.sscore;          // row stride b.L = n_sample: the sample-score rows
                b.n_splits = 1;
                b.pass = 0;
                b.hist_g = nullptr;
                b.ev_scan_start = b.ev_scan_stop = nullptr;
                if (!run_scan_variant<DT_, D_, HB_, true>(b, st)) { err = hipErrorInvalidValue; return; }
            } else {
                sample_score_kernel<DT_, D_, HB_><<<nqg * a.s_splits, 256, 0, st>>>(a);
            }
            launch_stats_kernel(a, st);
        }
        auto run_scan = [&](const IdxArgs& args) { return run_scan_variant<DT_, D_, HB_, false>(args, st); };
        if (!run_scan(a)) { err = hipErrorInvalidValue; return; }
        const size_t sel_lds = std::max(fin_lds_bytes(a), row_select_lds(a.topk, a.sorted, a.out_score != nullptr));
        allow_lds(select_kernel<DT_, D_, HB_>, sel_lds);
        select_kernel<DT_, D_, HB_><<<a.T, 256, sel_lds, st>>>(a);
        if (a.pass == 1) {
            // rescan of the rows whose buffer overflowed, gated at their first
            // pass's final threshold bin; without the shared histograms, whose
            // first-pass counts would otherwise be counted twice
            IdxArgs b = a;
            b.pass = 2;
            b.hist_g = nullptr;
            b.ev_scan_start = b.ev_scan_stop = nullptr;
            if (!run_scan(b)) { err = hipErrorInvalidValue; return; }
            select_kernel<DT_, D_, HB_><<<a.T, 256, sel_lds, st>>>(b);
        }
        err = hipGetLastError();
    });
    return ok ? err : hipErrorInvalidValue;
}

hipError_t launch_unfused_select(const IdxArgs& a, hipStream_t st) {
    const size_t lds = row_select_lds(a.topk, a.sorted, a.out_score != nullptr);
    allow_lds(unfused_select_kernel, lds);
    unfused_select_kernel<<<a.T, 256, lds, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_sample_stats(const IdxArgs& a, hipStream_t st) {
    launch_stats_kernel(a, st);
    return hipGetLastError();
}

hipError_t launch_finalize(const IdxArgs& a, hipStream_t st) {
    const size_t fin_lds = fin_lds_bytes(a);
    allow_lds(finalize_kernel, fin_lds);
    finalize_kernel<<<a.T, 256, fin_lds, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_indexer_unfused(int dt, int D, int HB, const IdxArgs& a, hipStream_t st) {
    hipError_t err = hipSuccess;
    const bool ok = dispatch(dt, D, HB, [&](auto DTc, auto Dc, auto HBc) {
        constexpr int DT_ = decltype(DTc)::value, D_ = decltype(Dc)::value, HB_ = decltype(HBc)::value;
        if constexpr (DT_ == DT_FP8) qlin_kernel<D_><<<a.T, 256, 0, st>>>(a);
        if (!run_scan_variant<DT_, D_, HB_, true>(a, st)) { err = hipErrorInvalidValue; return; }
        const size_t lds = row_select_lds(a.topk, a.sorted, a.out_score != nullptr);
        allow_lds(unfused_select_kernel, lds);
        unfused_select_kernel<<<a.T, 256, lds, st>>>(a);
        err = hipGetLastError();
    });
    return ok ? err : hipErrorInvalidValue;
}

hipError_t launch_next_sample(const int32_t* prev_idx, size_t n, int L, int n_sample, int32_t* out,
                              uint32_t* ws, hipStream_t st) {
    const NsLayout lay = ns_layout(L);
    uint32_t* counts = ws;
    uint32_t* hist = ws + lay.hist;
    NsHeader* hdr = reinterpret_cast<NsHeader*>(ws + lay.hdr);
    uint32_t* ties = ws + lay.ties;
    const int chunk = ns_chunk(L), nb = (L + chunk - 1) / chunk;
    zero_kernel<<<std::max(1, std::min((int)((lay.ties + 255) / 256), 2048)), 256, 0, st>>>(ws, lay.ties, nullptr);
    if (n > 0) count_selected_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(prev_idx, n, L, counts);
    ns_hist_kernel<<<nb, 256, 0, st>>>(counts, L, chunk, hist);
    ns_pick_kernel<<<1, 1024, 0, st>>>(hist, n_sample, hdr);
    ns_above_kernel<<<nb, 256, 0, st>>>(counts, L, chunk, hdr, ties, out);
    ns_ties_kernel<<<nb, 256, 0, st>>>(counts, L, chunk, hdr, ties, out);
    ns_fallback_kernel<<<1, 256, 256 * 4, st>>>(counts, L, n_sample, hdr, out);
    return hipGetLastError();
}

}  // namespace ltk
