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
// Unfused baseline (pages, "Problem statement"): unfused_score_kernel writes
// the full T x L score matrix, unfused_select_kernel radix-selects each row.
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

// One workgroup of 1024 threads turns the bitmap into the sorted list of
// distinct sample keys.
__global__ __launch_bounds__(1024) void sample_compact_kernel(const uint32_t* bitmap, int nwords, int32_t* out,
                                                              uint32_t* nu) {
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t s_base;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    if (tid == 0) s_base = 0;
    __syncthreads();
    for (int w0 = 0; w0 < nwords; w0 += 1024) {
        const int i = w0 + tid;
        uint32_t word = (i < nwords) ? bitmap[i] : 0u;
        const uint32_t c = __popc(word);
        uint32_t incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint32_t before = s_base;
        uint32_t total = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wave) before += wsum[w];
            total += wsum[w];
        }
        uint32_t o = before + incl - c;
        while (word) {
            const int b = __ffs(word) - 1;
            out[o++] = i * 32 + b;
            word &= word - 1;
        }
        __syncthreads();
        if (tid == 0) s_base += total;
        __syncthreads();
    }
    if (tid == 0) *nu = s_base;
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
// w'[h] = sigma_q[t] * w[t, h] (zero for padded heads / queries).
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
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hh = head_of(m, i, half);
            r.w[m][i] = (tv && hh < a.H) ? sq * a.w[(size_t)t * a.H + hh] : 0.0f;
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
// Sample: score the de-duplicated sample keys
// ---------------------------------------------------------------------------

template <int DT, int D, int HB>
__global__ __launch_bounds__(256) void sample_score_kernel(IdxArgs a) {
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;
    const int qg = blockIdx.x / a.s_splits, sp = blockIdx.x % a.s_splits;
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
    for (int blk = b0; blk < b1; ++blk) {
        const int j = blk * 32 + (lane & 31);
        const int key = a.sample_u[min(j, nu - 1)];
        HalfRow<DT, D> kf;
        load_key<DT, D>(kf, a.k, key);
        float I = score_2slots<DT, D, HB>(ra, kf, rb, kf);
        if constexpr (DT == DT_FP8) I = I * a.k_scale[key];
        if (t < a.T && j < nu) a.sscore[(size_t)t * a.n_sample + j] = I;
    }
}

// Sample statistics of one query: valid sample keys (<= pos), range, delta,
// histogram and the initial threshold bin.
__global__ __launch_bounds__(256) void sample_stats_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];  // [nbins]
    __shared__ float s_min[4], s_max[4];
    __shared__ int s_nvalid;
    const int t = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int nu = (int)*a.nu;
    const int pos_t = a.pos ? min(a.pos[t], a.L - 1) : a.L - 1;   // no positions: every key is valid
    if (tid == 0) {  // number of sorted sample keys <= pos_t
        int lo = 0, hi = nu;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (a.sample_u[mid] <= pos_t) lo = mid + 1; else hi = mid;
        }
        s_nvalid = lo;
    }
    for (int i = tid; i < a.nbins; i += 256) sh[i] = 0u;
    __syncthreads();
    const int nv = s_nvalid;
    const float* S = a.sscore + (size_t)t * a.n_sample;
    float mn = INFINITY, mx = -INFINITY;
    for (int j = tid; j < nv; j += 256) {
        const float v = S[j];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off));
        mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    if (lane == 0) {
        s_min[wave] = mn;
        s_max[wave] = mx;
    }
    __syncthreads();
    float smin = fminf(fminf(s_min[0], s_min[1]), fminf(s_min[2], s_min[3]));
    float smax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    if (nv == 0) {
        smin = 0.0f;
        smax = 1.0f;
    }
    float width = smax - smin;
    const float floor_w = 1e-6f * fmaxf(1.0f, fabsf(smax));
    if (!(width >= floor_w)) width = floor_w;
    const float delta = (float)a.nbins / width;
    for (int j = tid; j < nv; j += 256) atomicAdd(&sh[bin_of(S[j], smin, delta, a.nbins)], 1u);
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
}

// ---------------------------------------------------------------------------
// Filter: the fused scan
// ---------------------------------------------------------------------------
//
// One workgroup = 8 waves sharing K tiles that are streamed into LDS with
// direct global->LDS loads (three 32 KB stages: one computed, two loading), so the
// eight waves read each key from device memory once.  fp8 waves own two
// queries (one per 32-lane half, both scored against the same 32 keys);
// bf16/fp32 waves own one query scored against two 32-key blocks.  Two waves
// per SIMD let one wave's VALU epilogue overlap the other's MFMAs.

constexpr int kScanWaves = 8;
constexpr int kTileBytes = 32768;
constexpr int kScanStages = 3;     // tiles in flight: compute one, two loading

template <int DT> struct ScanShape { static constexpr int QPW = 1; };

template <int DT, int D>
struct TileGeom {
    static constexpr int RB = D * DTraits<DT>::ESZ;        // bytes per key row
    static constexpr int CPR = RB / 16;                    // 16-byte chunks per row
    static constexpr int TK = kTileBytes / RB;             // keys per tile
    static constexpr int NINST = TK * CPR / 64;            // wave-wide 1 KB loads per tile
    static constexpr int PER_WAVE = NINST / kScanWaves;
    static constexpr int SCALE_BYTES = (DT == DT_FP8) ? TK * 4 : 0;
    static constexpr int STAGE_BYTES = kTileBytes + SCALE_BYTES;
    static_assert(NINST % kScanWaves == 0, "tile loads split evenly over the waves");
    static_assert(TK % 64 == 0, "per-key scales load in whole 64-lane wave loads");
    static constexpr int SCALE_INST = (DT == DT_FP8) ? TK / 64 : 0;       // wave loads of scales per tile
    static_assert(SCALE_INST <= kScanWaves, "at most one scale load per wave");
};

// Issue this wave's share of the direct loads of the tile starting at key0.
template <int DT, int D>
__device__ __forceinline__ void load_tile(const IdxArgs& a, int key0, uint8_t* st, int wave, int lane) {
    using G = TileGeom<DT, D>;
#pragma unroll
    for (int j = 0; j < G::PER_WAVE; ++j) {
        const int inst = wave + j * kScanWaves;
        const int p = inst * 64 + lane;
        const int r = p / G::CPR, pc = p % G::CPR;
        const int c = pc ^ chunk_swz<G::RB, G::CPR>(r);
        const int key = min(key0 + r, a.L - 1);
        lds_direct16(a.k + (size_t)key * G::RB + c * 16, st + inst * 1024);
    }
    if constexpr (DT == DT_FP8) {
        // one per-key scale per lane (keys past the context re-read the last one)
#pragma unroll
        for (int j = wave; j < G::TK / 64; j += kScanWaves) {
            const int key = min(key0 + j * 64 + lane, a.L - 1);
            lds_direct4(a.k_scale + key, st + kTileBytes + j * 256);
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

template <int DT, int D, int HB>
__global__ __launch_bounds__(512) void scan_kernel(IdxArgs a) {
    using G = TileGeom<DT, D>;
    constexpr int QPW = ScanShape<DT>::QPW;
    constexpr int QPG = kScanWaves * QPW;
    extern __shared__ __attribute__((aligned(16))) uint8_t shm[];
    const int nbins = a.nbins;
    uint8_t* tiles = shm;                                                  // kScanStages stages
    uint32_t* hist = reinterpret_cast<uint32_t*>(shm + kScanStages * G::STAGE_BYTES);  // [QPG][nbins]
    uint2* stage = reinterpret_cast<uint2*>(hist + QPG * nbins);           // [QPG][kStage]
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;
    const int qg = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
    const int t0 = qg * QPG;
    const int s0 = t0 + QPW * wave, s1 = s0 + (QPW - 1);                  // the wave's queries
    const int t = (QPW == 2 && half) ? s1 : s0;                           // this lane's query
    const int qi = QPW * wave + ((QPW == 2) ? half : 0);                  // its local index
    const uint32_t k = (uint32_t)a.topk;

    for (int i = lane; i < QPW * nbins; i += 64) hist[QPW * wave * nbins + i] = 0u;

    // keys any query of the group can see, split into tile-aligned ranges
    int e = 0;
    for (int i = lane; i < QPG; i += 64) {
        const int tt = t0 + i;
        if (tt < a.T) e = max(e, min(a.pos[tt], a.L - 1) + 1);
    }
    const int kend = wave_max_i32(e);
    const int per = ((kend + a.n_splits - 1) / a.n_splits + G::TK - 1) / G::TK * G::TK;
    const int k_lo = split * per, k_hi = min(kend, k_lo + per);

    const bool tv = t < a.T;
    const int my_pos = tv ? min(a.pos[t], a.L - 1) : -1;
    const int wave_end = min(k_hi, wave_max_i32(my_pos) + 1);
    Meta m{0.0f, 1.0f, 0, 0};
    if (tv) m = reinterpret_cast<const Meta*>(a.meta)[t];
    int thr = m.thr0;
    float tau = tv ? initial_gate(thr, m, nbins, a.topk) : -INFINITY;

    QueryRegs<DT, D, HB> ra, rb;
    load_query<DT, D, HB>(ra, a, s0);
    if constexpr (QPW == 2) load_query<DT, D, HB>(rb, a, s1);

    int cnt[QPW] = {};   // staged entries per query (wave-uniform)
    int fl[QPW] = {};    // batches written back per query
    const uint64_t lt_mask = (1ull << lane) - 1ull;

    auto flush = [&](int s) {
        const int tq = s0 + s;
        const int lq = QPW * wave + s;
        uint2* st = stage + lq * kStage;
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&a.tail[tq], (uint32_t)kFlush);
        base = __shfl(base, 0);
        const uint2 en = st[lane];
        if ((int64_t)base + lane < a.ccap) a.cand[(size_t)tq * a.ccap + base + lane] = en;
        const int rem = cnt[s] - kFlush;
        uint2 r{0u, 0u};
        if (lane < rem) r = st[kFlush + lane];
        if (lane < rem) st[lane] = r;
        cnt[s] = rem;
        ++fl[s];
        uint32_t* hl = hist + lq * nbins;
        uint32_t* hg = a.hist_g ? a.hist_g + (size_t)tq * nbins : nullptr;
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
        if (a.refresh_every > 0 && fl[s] % a.refresh_every == 0) {
            // top-down recount (of every split's counts, when shared); a plain
            // overwrite that can only raise the threshold.  Counts cover real
            // causal keys only, so the new bin is at most the true one.
            if (hg)
                for (int b = lane; b < nbins; b += 64) hl[b] = __hip_atomic_load(&hg[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const SuffixPick p = suffix_pick(hl, nbins, k);
            if (hg)
                for (int b = lane; b < nbins; b += 64) hl[b] = 0u;
            if (QPW == 1 || half == s) {
                if (p.bin > thr) {
                    thr = p.bin;
                    tau = tau_of(thr, m.smin, m.delta, nbins);
                }
            }
        }
    };

    auto process = [&](float I, int key) {
        const bool pass = (key <= my_pos) && (I >= tau);
        const uint64_t mask = __ballot(pass);
        if (mask) {
            if (pass) atomicAdd(&hist[qi * nbins + bin_of(I, m.smin, m.delta, nbins)], 1u);
            if constexpr (QPW == 2) {
                const uint32_t ma = (uint32_t)mask, mb = (uint32_t)(mask >> 32);
                if (pass) {
                    const int rank = __popcll(mask & lt_mask & (half ? 0xffffffff00000000ull : 0xffffffffull));
                    stage[qi * kStage + (half ? cnt[1] : cnt[0]) + rank] = make_uint2((uint32_t)key, __float_as_uint(I));
                }
                cnt[0] += __popc(ma);
                cnt[1] += __popc(mb);
                if (cnt[0] >= kFlush) flush(0);
                if (cnt[1] >= kFlush) flush(1);
            } else {
                if (pass) stage[qi * kStage + cnt[0] + mbcnt(mask)] = make_uint2((uint32_t)key, __float_as_uint(I));
                cnt[0] += __popcll(mask);
                if (cnt[0] >= kFlush) flush(0);
            }
        }
    };

    const int ntiles = (k_hi > k_lo) ? (k_hi - k_lo + G::TK - 1) / G::TK : 0;
    constexpr int LPW_HI = G::PER_WAVE + (G::SCALE_INST > 0 ? 1 : 0);   // loads per tile, waves < SCALE_INST
    constexpr int LPW_LO = G::PER_WAVE;                                  // loads per tile, other waves
    if (ntiles > 0) load_tile<DT, D>(a, k_lo, tiles, wave, lane);
    if (ntiles > 1) load_tile<DT, D>(a, k_lo + G::TK, tiles + G::STAGE_BYTES, wave, lane);
    int sbuf = 0;   // stage holding tile `it`
    for (int it = 0; it < ntiles; ++it) {
        if (it + 1 < ntiles) {   // tile it+1 may still be loading
            if (wave < G::SCALE_INST) wait_vm<LPW_HI>(); else wait_vm<LPW_LO>();
        } else {
            wait_vm<0>();
        }
        __syncthreads();
        if (it + 2 < ntiles) {
            const int nb = (sbuf + 2) % kScanStages;
            load_tile<DT, D>(a, k_lo + (it + 2) * G::TK, tiles + nb * G::STAGE_BYTES, wave, lane);
        }
        const int key0 = k_lo + it * G::TK;
        const uint8_t* st = tiles + sbuf * G::STAGE_BYTES;
        sbuf = (sbuf + 1) % kScanStages;
        const float* sks = reinterpret_cast<const float*>(st + kTileBytes);
        if constexpr (QPW == 2) {
#pragma unroll 1
            for (int blk = 0; blk < G::TK / 32; ++blk) {
                const int kb = key0 + 32 * blk;
                if (kb >= wave_end) break;
                HalfRow<DT, D> kf;
                read_frag<DT, D>(kf, st, 32 * blk, lane);
                float I = score_2slots<DT, D, HB>(ra, kf, rb, kf);
                if constexpr (DT == DT_FP8) I = I * sks[32 * blk + (lane & 31)];
                process(I, kb + (lane & 31));
            }
        } else if constexpr (HalfRow<DT, D>::NV > 4) {
            // wide fragments (bf16/fp32 at D = 128): the two 32-key slots of a
            // block one after the other, keeping one slot's registers live
#pragma unroll 1
            for (int blk = 0; blk < G::TK / 64; ++blk) {
                const int kb = key0 + 64 * blk;
                if (kb >= wave_end) break;
                HalfRow<DT, D> kf;
                v16f acc[HB];
                read_frag<DT, D>(kf, st, 64 * blk, lane);
                mfma_1slot<DT, D, HB>(ra.q, kf, acc);
                const float pa = relu_wsum<HB>(acc, ra.w);
                read_frag<DT, D>(kf, st, 64 * blk + 32, lane);
                mfma_1slot<DT, D, HB>(ra.q, kf, acc);
                const float pb = relu_wsum<HB>(acc, ra.w);
                float I = combine_halves(pa, pb);
                if constexpr (DT == DT_FP8) I = I * sks[64 * blk + lane];
                process(I, kb + lane);
            }
        } else {
            // 32-key slots, software-pipelined: the MFMAs of slot s+1 are issued
            // before the ReLU*w reduction of slot s, so the matrix core and the
            // VALU of one wave overlap; two slots make one 64-key block.
            constexpr int NS = G::TK / 32;
            HalfRow<DT, D> kf;
            v16f accC[HB], accN[HB];
            read_frag<DT, D>(kf, st, 0, lane);
            mfma_1slot<DT, D, HB>(ra.q, kf, accC);
            float pprev = 0.0f;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                if (sl + 1 < NS) {
                    read_frag<DT, D>(kf, st, 32 * (sl + 1), lane);
                    mfma_1slot<DT, D, HB>(ra.q, kf, accN);
                }
                const float p = relu_wsum<HB>(accC, ra.w);
                if (sl & 1) {
                    float I = combine_halves(pprev, p);
                    if constexpr (DT == DT_FP8) I = I * sks[32 * (sl - 1) + lane];
                    process(I, key0 + 32 * (sl - 1) + lane);
                } else {
                    pprev = p;
                }
                if (sl + 1 < NS) {
#pragma unroll
                    for (int m = 0; m < HB; ++m) accC[m] = accN[m];
                }
            }
        }
    }
    // final partial batches
#pragma unroll
    for (int s = 0; s < QPW; ++s) {
        if (cnt[s] > 0) {
            const int tq = s0 + s;
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&a.tail[tq], (uint32_t)cnt[s]);
            base = __shfl(base, 0);
            if (lane < cnt[s]) {
                const uint2 en = stage[(QPW * wave + s) * kStage + lane];
                if ((int64_t)base + lane < a.ccap) a.cand[(size_t)tq * a.ccap + base + lane] = en;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Select: finalize
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void finalize_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];   // [max(nbins, 256)] then (sorted) keys
    __shared__ int s_pick;
    __shared__ uint32_t s_above, s_cnt, s_ocnt;
    const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
    const int k = a.topk;
    const uint32_t n = a.tail[t];
    int32_t* out = a.out_idx + (size_t)t * k;
    float* osc = a.out_score ? a.out_score + (size_t)t * k : nullptr;
    uint64_t* sort_keys = reinterpret_cast<uint64_t*>(sh + ((max(a.nbins, 256) + 1) & ~1));
    if (tid == 0 && a.stats) {
        atomicAdd((unsigned long long*)&a.stats->cand_written, (unsigned long long)n);
        atomicMax(&a.stats->max_cand_per_query, n);
    }
    if ((int64_t)n > a.ccap) {   // the buffer overflowed: the fallback recomputes this row
        if (tid == 0) {
            a.flags[t] = 1u;
            if (a.stats) atomicAdd(&a.stats->overflow_rows, 1u);
        }
        return;
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
        return;
    }
    const Meta m = reinterpret_cast<const Meta*>(a.meta)[t];
    const int nbins = a.nbins;
    uint32_t* hist = sh;
    for (int i = tid; i < nbins; i += 256) hist[i] = 0u;
    if (tid == 0) s_ocnt = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += 256) atomicAdd(&hist[bin_of(__uint_as_float(c[i].y), m.smin, m.delta, nbins)], 1u);
    __syncthreads();
    if (wave == 0) {   // final threshold bin: top-down recount of the candidates' bins
        const SuffixPick p = suffix_pick(hist, nbins, (uint32_t)k);
        if (lane == 0) {
            s_pick = p.bin;
            s_above = p.above;
        }
    }
    __syncthreads();
    const int bstar = s_pick;
    const uint32_t above = s_above;
    // bins strictly above the final threshold bin go straight to the output
    for (uint32_t i = tid; i < n; i += 256) {
        const uint2 e = c[i];
        const float I = __uint_as_float(e.y);
        if (bin_of(I, m.smin, m.delta, nbins) > bstar) {
            const uint32_t p = atomicAdd(&s_ocnt, 1u);
            if (p < (uint32_t)k) {
                out[p] = (int32_t)e.x;
                if (osc) osc[p] = I;
            }
        }
    }
    // exact top-(k - above) inside the threshold bin: radix select on (score desc, index asc)
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
        if constexpr (DT == DT_FP8) I = I * ks[min(key, L - 1)];
        valid = key < nvalid;
    }
};

template <int DT, int D, int HB>
__global__ __launch_bounds__(256) void fallback_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];
    const int t = blockIdx.x;
    if (a.flags[t] == 0u) return;
    RescoreSource<DT, D, HB> src;
    load_query<DT, D, HB>(src.r, a, t);
    src.k = a.k;
    src.ks = a.k_scale;
    src.L = a.L;
    const int nvalid = max(min(a.pos[t], a.L - 1) + 1, 0);
    int32_t* out = a.out_idx + (size_t)t * a.topk;
    float* osc = a.out_score ? a.out_score + (size_t)t * a.topk : nullptr;
    select_row(src, nvalid, a.topk, out, osc, sh);
    if (a.sorted) sort_row_output(out, osc, a.topk, reinterpret_cast<uint64_t*>(sh + 256));
}

// ---------------------------------------------------------------------------
// Unfused baseline
// ---------------------------------------------------------------------------

template <int DT, int D, int HB>
__global__ __launch_bounds__(256) void unfused_score_kernel(IdxArgs a) {
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;
    const int qg = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
    const int ta = qg * kQPG + 2 * wave, tb = ta + 1;
    const int t = half ? tb : ta;
    const int per = (((a.L + a.n_splits - 1) / a.n_splits) + 31) & ~31;
    const int k_lo = split * per, k_hi = min(a.L, k_lo + per);
    QueryRegs<DT, D, HB> ra, rb;
    load_query<DT, D, HB>(ra, a, ta);
    load_query<DT, D, HB>(rb, a, tb);
    const int my_pos = (t < a.T) ? a.pos[t] : -1;
    for (int kb = k_lo; kb < k_hi; kb += 32) {
        const int key = kb + (lane & 31);
        HalfRow<DT, D> kf;
        load_key<DT, D>(kf, a.k, min(key, a.L - 1));
        float I = score_2slots<DT, D, HB>(ra, kf, rb, kf);
        if constexpr (DT == DT_FP8) I = I * a.k_scale[min(key, a.L - 1)];
        if (t < a.T && key < k_hi) a.S[(size_t)t * a.L + key] = (key <= my_pos) ? I : -INFINITY;
    }
}

__global__ __launch_bounds__(256) void unfused_select_kernel(IdxArgs a) {
    extern __shared__ uint32_t sh[];
    const int t = blockIdx.x;
    MemSource src{a.S + (size_t)t * a.L};
    const int nvalid = max(min(a.pos[t], a.L - 1) + 1, 0);
    int32_t* out = a.out_idx + (size_t)t * a.topk;
    float* osc = a.out_score ? a.out_score + (size_t)t * a.topk : nullptr;
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

// counts are < 2^24, so their fp32 values order exactly like the integers
__global__ void counts_to_f32_kernel(uint32_t* counts, int L) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < L) reinterpret_cast<float*>(counts)[i] = (float)counts[i];
}

__global__ __launch_bounds__(256) void select_counts_kernel(const float* counts, int L, int n, int32_t* out) {
    extern __shared__ uint32_t sh[];
    MemSource src{counts};
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

static size_t sort_lds(const IdxArgs& a) {
    if (!a.sorted) return 0;
    int p2 = 1;
    while (p2 < a.topk) p2 <<= 1;
    return (size_t)p2 * 8;
}

hipError_t launch_prepare_sample(const IdxArgs& a, const int32_t* sample, int n_sample, const WsLayout& lay,
                                 uint8_t* ws, hipStream_t st) {
    const size_t nz = (lay.zero_end - lay.zero_begin) / 4;
    const int zb = (int)std::min<size_t>((nz + 255) / 256, 2048);
    zero_kernel<<<std::max(zb, 1), 256, 0, st>>>(reinterpret_cast<uint32_t*>(ws + lay.zero_begin), nz, a.stats);
    if (n_sample > 0)
        sample_mark_kernel<<<(n_sample + 255) / 256, 256, 0, st>>>(sample, n_sample, a.L, a.bitmap);
    sample_compact_kernel<<<1, 1024, 0, st>>>(a.bitmap, (a.L + 31) / 32, a.sample_u, a.nu);
    return hipGetLastError();
}

template <class K>
static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)bytes);
}

hipError_t launch_indexer_fused(int dt, int D, int HB, const IdxArgs& a, hipStream_t st) {
    const int nqg = (a.T + kQPG - 1) / kQPG;
    hipError_t err = hipSuccess;
    const bool ok = dispatch(dt, D, HB, [&](auto DTc, auto Dc, auto HBc) {
        constexpr int DT_ = decltype(DTc)::value, D_ = decltype(Dc)::value, HB_ = decltype(HBc)::value;
        sample_score_kernel<DT_, D_, HB_><<<nqg * a.s_splits, 256, 0, st>>>(a);
        sample_stats_kernel<<<a.T, 256, (size_t)a.nbins * 4, st>>>(a);
        constexpr int QPG = kScanWaves * ScanShape<DT_>::QPW;
        const size_t scan_lds = kScanStages * (size_t)TileGeom<DT_, D_>::STAGE_BYTES + (size_t)QPG * a.nbins * 4 +
                                (size_t)QPG * kStage * 8;
        allow_lds(scan_kernel<DT_, D_, HB_>, scan_lds);
        if (a.ev_scan_start) (void)hipEventRecord(a.ev_scan_start, st);
        scan_kernel<DT_, D_, HB_><<<((a.T + QPG - 1) / QPG) * a.n_splits, kScanWaves * 64, scan_lds, st>>>(a);
        if (a.ev_scan_stop) (void)hipEventRecord(a.ev_scan_stop, st);
        const size_t fin_lds = (size_t)((std::max(a.nbins, 256) + 1) & ~1) * 4 + sort_lds(a);
        allow_lds(finalize_kernel, fin_lds);
        finalize_kernel<<<a.T, 256, fin_lds, st>>>(a);
        const size_t fb_lds = 256 * 4 + sort_lds(a);
        allow_lds(fallback_kernel<DT_, D_, HB_>, fb_lds);
        fallback_kernel<DT_, D_, HB_><<<a.T, 256, fb_lds, st>>>(a);
        err = hipGetLastError();
    });
    return ok ? err : hipErrorInvalidValue;
}

hipError_t launch_sample_stats(const IdxArgs& a, hipStream_t st) {
    sample_stats_kernel<<<a.T, 256, (size_t)a.nbins * 4, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_finalize(const IdxArgs& a, hipStream_t st) {
    const size_t fin_lds = (size_t)((std::max(a.nbins, 256) + 1) & ~1) * 4 + sort_lds(a);
    allow_lds(finalize_kernel, fin_lds);
    finalize_kernel<<<a.T, 256, fin_lds, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_indexer_unfused(int dt, int D, int HB, const IdxArgs& a, hipStream_t st) {
    const int nqg = (a.T + kQPG - 1) / kQPG;
    hipError_t err = hipSuccess;
    const bool ok = dispatch(dt, D, HB, [&](auto DTc, auto Dc, auto HBc) {
        constexpr int DT_ = decltype(DTc)::value, D_ = decltype(Dc)::value, HB_ = decltype(HBc)::value;
        unfused_score_kernel<DT_, D_, HB_><<<nqg * a.n_splits, 256, 0, st>>>(a);
        const size_t lds = 256 * 4 + sort_lds(a);
        allow_lds(unfused_select_kernel, lds);
        unfused_select_kernel<<<a.T, 256, lds, st>>>(a);
        err = hipGetLastError();
    });
    return ok ? err : hipErrorInvalidValue;
}

hipError_t launch_next_sample(const int32_t* prev_idx, size_t n, int L, int n_sample, int32_t* out,
                              uint32_t* counts, hipStream_t st) {
    zero_kernel<<<std::max(1, std::min((L + 255) / 256, 2048)), 256, 0, st>>>(counts, (size_t)L, nullptr);
    if (n > 0) count_selected_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(prev_idx, n, L, counts);
    counts_to_f32_kernel<<<(L + 255) / 256, 256, 0, st>>>(counts, L);
    select_counts_kernel<<<1, 256, 256 * 4, st>>>(reinterpret_cast<const float*>(counts), L, n_sample, out);
    return hipGetLastError();
}

}  // namespace ltk
