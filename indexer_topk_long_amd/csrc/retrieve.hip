// retrieve.hip -- fused inner-product retrieval top-k for gfx950.
//
// The same Sample -> Filter -> Select method as the indexer (LiteTopK pages,
// "Methodology"; the pages apply the primitive to vector retrieval), with
// the score I[t, s] = q[t] . x[s] of bf16 vectors (fp32 accumulation) and no
// causal mask.  Queries sit on the MFMA M dimension: one wave holds 32
// queries in registers and scores them against 32 database rows per tile,
// so every accumulator register is a (query, row) score and no head
// reduction is needed.  Database rows stream through LDS in 48 KB tiles
// (direct global->LDS loads, double-buffered) shared by the 4 waves of a
// workgroup (128 queries).
//
// The database is split across workgroups.  Their per-query histograms are
// one shared array in device memory: every kept candidate adds to it with an
// atomic, and a workgroup refreshes its threshold bins from the shared
// counts.  Counts only ever cover real database rows, so any refresh is at
// most the true threshold bin and the result stays exact; sharing lets the
// threshold rise even though no single split holds k matching rows.
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "internal.hpp"
#include "kernels_common.hpp"

namespace ltk {

constexpr int kRetrWaves = 4;             // waves per workgroup (one per SIMD: 32 queries of
                                          // D = 768 take 192 registers per lane)
constexpr int kRetrQ = 32;                // queries per wave (one MFMA M block)
constexpr int kRetrRows = 32;             // database rows per LDS tile
constexpr int kRetrRefreshCands = 64;     // candidates a wave adds before it refreshes
constexpr int kSuperBins = 16;            // fine bins per super-bin of the shared histogram

template <int D>
struct RetrGeom {
    static constexpr int RB = 2 * D;                       // bf16 row bytes
    static constexpr int CPR = RB / 16;                    // 16-byte chunks per row
    static constexpr int TILE = kRetrRows * RB;            // bytes per tile
    static constexpr int NINST = kRetrRows * CPR / 64;     // wave-wide 1 KB loads per tile
    static constexpr int KSTEPS = D / 16;                  // v_mfma_f32_32x32x16_bf16 steps
};

// Query block of 32 rows: lane holds row (lane & 31), half (lane >> 5).
template <int D>
__device__ __forceinline__ void load_qblock(HalfRow<DT_BF16, D>& f, const RetrArgs& a, int q0) {
    const int lane = lane_id();
    const int q = q0 + (lane & 31);
    if (q < a.T)
        load_half_row<DT_BF16, D>(f, a.q + (size_t)q * (2 * D), lane >> 5);
    else
        zero_half_row<DT_BF16, D>(f);
}

// Query of accumulator register r of this lane (32x32 MFMA result layout).
__device__ __forceinline__ int reg_query(int q0, int r, int half) { return q0 + 8 * (r >> 2) + 4 * half + (r & 3); }

// ---------------------------------------------------------------------------
// Sample: scores of the de-duplicated sample rows (rows read straight from
// device memory; the sample is small)
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void retr_sample_score_kernel(RetrArgs a) {
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;
    const int q0 = (blockIdx.x * 4 + wave) * kRetrQ;
    const int nu = (int)*a.nu;
    if (q0 >= a.T || nu == 0) return;
    HalfRow<DT_BF16, D> qf;
    load_qblock<D>(qf, a, q0);
    for (int j0 = blockIdx.y * 32; j0 < nu; j0 += 32 * gridDim.y) {
        const int j = j0 + (lane & 31);
        const int row = a.sample_u[min(j, nu - 1)];
        const u32x4* rp = reinterpret_cast<const u32x4*>(a.db + (size_t)row * (2 * D) + half * D);
        v16f acc = v16f{};
#pragma unroll
        for (int s = 0; s < RetrGeom<D>::KSTEPS; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf.v[s]),
                                                          __builtin_bit_cast(bf16x8, rp[s]), acc, 0, 0, 0);
        if (j < nu) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = reg_query(q0, r, half);
                if (q < a.T) a.sscore[(size_t)q * a.n_sample + j] = acc[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Filter: the fused scan over the database
// ---------------------------------------------------------------------------

template <int D>
__device__ __forceinline__ void retr_load_tile(const RetrArgs& a, int row0, uint8_t* st, int wave, int lane) {
    using G = RetrGeom<D>;
#pragma unroll
    for (int inst = wave; inst < G::NINST; inst += kRetrWaves) {
        const int p = inst * 64 + lane;
        const int r = p / G::CPR, pc = p % G::CPR;
        const int c = pc ^ chunk_swz<G::RB, G::CPR>(r);
        const int row = min(row0 + r, a.N - 1);
        lds_direct16(a.db + (size_t)row * G::RB + c * 16, st + inst * 1024);
    }
}

// Coherent (device-scope) read of a shared counter.
__device__ __forceinline__ uint32_t load_shared_count(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void retr_scan_kernel(RetrArgs a) {
    using G = RetrGeom<D>;
    extern __shared__ __attribute__((aligned(16))) uint8_t shm[];
    uint8_t* tiles = shm;                                                 // 2 stages
    float* tau_l = reinterpret_cast<float*>(shm + 2 * G::TILE);           // [waves][32 queries]
    float* stash = tau_l + kRetrWaves * kRetrQ;                            // [waves][16][64] scores
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;

    // (split, query group) from the block index so that the query groups of
    // one split are dispatched back to back on the same XCD (block i runs on
    // XCD i % 8): they stream the same database rows through one L2.
    const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
    const int split = (slot / a.n_qgroups) * 8 + xcd, qgroup = slot % a.n_qgroups;
    if (split >= a.n_splits) return;
    const int q0 = qgroup * (kRetrWaves * kRetrQ) + wave * kRetrQ;
    const int per = ((a.N + a.n_splits - 1) / a.n_splits + kRetrRows - 1) / kRetrRows * kRetrRows;
    const int r_lo = split * per, r_hi = min(a.N, r_lo + per);
    const int ntiles = (r_hi > r_lo) ? (r_hi - r_lo + kRetrRows - 1) / kRetrRows : 0;
    if (ntiles == 0) return;

    HalfRow<DT_BF16, D> qf;
    load_qblock<D>(qf, a, q0);
    const Meta* meta = reinterpret_cast<const Meta*>(a.meta);

    // thresholds of the wave's 32 queries: lane i < 32 owns query q0 + i
    int thr_own = 0;
    Meta m_own{0.0f, 1.0f, 0, 0};
    const bool own_valid = lane < 32 && q0 + lane < a.T;
    if (own_valid) {
        m_own = meta[q0 + lane];
        thr_own = m_own.thr0;
    }
    float* my_tau = tau_l + wave * kRetrQ;
    if (lane < 32) my_tau[lane] = own_valid ? tau_of(thr_own, m_own.smin, m_own.delta, a.nbins) : INFINITY;
    float tau[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) tau[r] = my_tau[reg_query(0, r, half)];
    int added = 0;   // candidates this wave added since its last refresh (wave-uniform)

    retr_load_tile<D>(a, r_lo, tiles, wave, lane);
    for (int it = 0; it < ntiles; ++it) {
        wait_vm<0>();
        __syncthreads();
        if (it + 1 < ntiles) retr_load_tile<D>(a, r_lo + (it + 1) * kRetrRows, tiles + ((it + 1) & 1) * G::TILE, wave, lane);
        const uint8_t* st = tiles + (it & 1) * G::TILE;
        const int rr = lane & 31;
        const int row = r_lo + it * kRetrRows + rr;
        // B fragments read from LDS four steps ahead of their MFMA; the
        // scheduling barriers keep the compiler from hoisting every read (the
        // 32 query rows already hold 2*D bytes of registers per lane)
        const uint8_t* rowp = st + rr * G::RB;
        const int sw = chunk_swz<G::RB, G::CPR>(rr);
        auto rd = [&](int s) {
            return *reinterpret_cast<const u32x4*>(rowp + (((half * (G::CPR / 2) + s) ^ sw) * 16));
        };
        constexpr int PF = G::KSTEPS < 4 ? G::KSTEPS : 4;
        u32x4 bq[PF];
#pragma unroll
        for (int s = 0; s < PF; ++s) bq[s] = rd(s);
        v16f acc = v16f{};
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf.v[s]),
                                                          __builtin_bit_cast(bf16x8, bq[s % PF]), acc, 0, 0, 0);
            if (s + PF < G::KSTEPS) bq[s % PF] = rd(s + PF);
            if (s % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
        }
        // gate: bit r of pm is set when the score in accumulator register r
        // reaches its query's threshold
        const bool rv = row < r_hi;
        uint32_t pm = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) pm |= (rv && acc[r] >= tau[r]) ? (1u << r) : 0u;
        if (__ballot(pm != 0u)) {
            // rare: keep the passing (row, score) pairs, register by register,
            // from a wave-private LDS copy of the scores (one loop body, no
            // per-register copies of the write-back code)
            float* sv = stash + wave * 16 * 64;
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r * 64 + lane] = acc[r];
#pragma unroll 1
            for (int r = 0; r < 16; ++r) {
                const bool pass = (pm >> r) & 1u;
                const uint64_t mask = __ballot(pass);
                if (!mask) continue;
                const float I = sv[r * 64 + lane];
#pragma unroll 1
                for (int h = 0; h < 2; ++h) {
                    const uint32_t mh = (uint32_t)(mask >> (32 * h));
                    if (!mh) continue;
                    const int q = reg_query(q0, r, h);
                    const int leader = 32 * h + __ffs(mh) - 1;
                    uint32_t base = 0;
                    if (lane == leader) base = atomicAdd(&a.tail[q], (uint32_t)__popc(mh));
                    base = __shfl(base, leader);
                    if (pass && half == h) {
                        const uint32_t p = base + (uint32_t)__popc(mh & ((1u << rr) - 1u));
                        if ((int64_t)p < a.ccap) a.cand[(size_t)q * a.ccap + p] = make_uint2((uint32_t)row, __float_as_uint(I));
                        const Meta mq = meta[q];
                        const int b = bin_of(I, mq.smin, mq.delta, a.nbins);
                        atomicAdd(&a.hist_g[(size_t)q * a.nbins + b], 1u);
                        atomicAdd(&a.hist_c[(size_t)q * a.nsuper + b / kSuperBins], 1u);
                    }
                }
                added += __popcll(mask);
            }
        }
        // refresh from the shared histograms once this wave has added enough
        // candidates: accumulate counts from the top bin down (super-bins
        // first, then the fine bins of the crossing super-bin), and overwrite
        // the wave's thresholds -- plain stores that can only raise them.
        // Every counter read is at most the number of real rows in its bin, so
        // the new threshold bin is at most the true one.
        if (added >= kRetrRefreshCands) {
            added = 0;
            int nt = thr_own;
            if (own_valid) {
                const uint32_t kk = (uint32_t)a.topk;
                const uint32_t* hc = a.hist_c + (size_t)(q0 + lane) * a.nsuper;
                const uint32_t* hf = a.hist_g + (size_t)(q0 + lane) * a.nbins;
                uint32_t cum = 0;
                int sup = -1;
                for (int hi = a.nsuper - 1; hi >= 0 && sup < 0; hi -= 16) {
                    uint32_t c[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) c[i] = (hi - i >= 0) ? load_shared_count(hc + hi - i) : 0u;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        if (sup < 0) {
                            if (cum + c[i] >= kk) sup = hi - i; else cum += c[i];
                        }
                    }
                }
                if (sup >= 0 && (sup + 1) * kSuperBins - 1 > thr_own) {
                    uint32_t f[kSuperBins];
#pragma unroll
                    for (int i = 0; i < kSuperBins; ++i) {
                        const int b = sup * kSuperBins + kSuperBins - 1 - i;
                        f[i] = (b < a.nbins) ? load_shared_count(hf + b) : 0u;
                    }
                    int found = -1;
#pragma unroll
                    for (int i = 0; i < kSuperBins; ++i) {
                        const int b = sup * kSuperBins + kSuperBins - 1 - i;
                        if (found < 0 && b < a.nbins) {
                            cum += f[i];
                            if (cum >= kk) found = b;
                        }
                    }
                    nt = max(thr_own, found);
                }
            }
            const bool changed = nt > thr_own;
            if (__ballot(changed)) {
                if (changed) {
                    thr_own = nt;
                    my_tau[lane] = tau_of(thr_own, m_own.smin, m_own.delta, a.nbins);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) tau[r] = my_tau[reg_query(0, r, half)];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Overflow fallback: exact radix select over re-computed scores of one query
// (the query is replicated into all 32 M rows, so every accumulator register
// of a lane holds the score of the lane's row; same arithmetic as the scan)
// ---------------------------------------------------------------------------

template <int D>
struct RetrRescoreSource {
    HalfRow<DT_BF16, D> qf;
    const uint8_t* db;
    int N;
    __device__ __forceinline__ void get(int base, int nvalid, int& key, float& I, bool& valid) {
        const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;
        const int kb0 = base + 64 * wave;
        const u32x4* ra = reinterpret_cast<const u32x4*>(db + (size_t)min(kb0 + (lane & 31), N - 1) * (2 * D) + half * D);
        const u32x4* rb = reinterpret_cast<const u32x4*>(db + (size_t)min(kb0 + 32 + (lane & 31), N - 1) * (2 * D) + half * D);
        v16f acca = v16f{}, accb = v16f{};
#pragma unroll
        for (int s = 0; s < RetrGeom<D>::KSTEPS; ++s) {
            acca = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf.v[s]),
                                                           __builtin_bit_cast(bf16x8, ra[s]), acca, 0, 0, 0);
            accb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf.v[s]),
                                                           __builtin_bit_cast(bf16x8, rb[s]), accb, 0, 0, 0);
        }
        I = half ? accb[0] : acca[0];
        key = kb0 + lane;
        valid = key < nvalid;
    }
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void retr_fallback_kernel(RetrArgs a) {
    extern __shared__ uint32_t sh[];
    const int t = blockIdx.x;
    if (a.flags[t] == 0u) return;
    RetrRescoreSource<D> src;
    load_half_row<DT_BF16, D>(src.qf, a.q + (size_t)t * (2 * D), lane_id() >> 5);
    src.db = a.db;
    src.N = a.N;
    int32_t* out = a.out_idx + (size_t)t * a.topk;
    float* osc = a.out_score ? a.out_score + (size_t)t * a.topk : nullptr;
    select_row(src, a.N, a.topk, out, osc, sh);
    if (a.sorted) sort_row_output(out, osc, a.topk, reinterpret_cast<uint64_t*>(sh + 256));
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------

template <int D>
static hipError_t launch_retrieve_d(const RetrArgs& a, const IdxArgs& fin, hipStream_t st) {
    using G = RetrGeom<D>;
    const int nqb = (a.T + kRetrQ - 1) / kRetrQ;
    dim3 sg((nqb + 3) / 4, std::max(1, std::min(64, (a.n_sample + 31) / 32)));
    retr_sample_score_kernel<D><<<sg, 256, 0, st>>>(a);
    hipError_t e = launch_sample_stats(fin, st);
    if (e != hipSuccess) return e;
    const size_t lds = 2 * (size_t)G::TILE + (size_t)kRetrWaves * kRetrQ * 4 + (size_t)kRetrWaves * 16 * 64 * 4;
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(retr_scan_kernel<D>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int nsplit_pad = (a.n_splits + 7) / 8 * 8;
    if (a.ev_scan_start) (void)hipEventRecord(a.ev_scan_start, st);
    retr_scan_kernel<D><<<nsplit_pad * a.n_qgroups, kRetrWaves * 64, lds, st>>>(a);
    if (a.ev_scan_stop) (void)hipEventRecord(a.ev_scan_stop, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_finalize(fin, st)) != hipSuccess) return e;
    int p2 = 1;
    while (p2 < a.topk) p2 <<= 1;
    const size_t fb_lds = 256 * 4 + (a.sorted ? (size_t)p2 * 8 : 0);
    if (fb_lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(retr_fallback_kernel<D>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)fb_lds);
    retr_fallback_kernel<D><<<a.T, 256, fb_lds, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_retrieve(int D, const RetrArgs& a, const IdxArgs& fin, hipStream_t st) {
    switch (D) {
        case 64: return launch_retrieve_d<64>(a, fin, st);
        case 128: return launch_retrieve_d<128>(a, fin, st);
        case 256: return launch_retrieve_d<256>(a, fin, st);
        case 512: return launch_retrieve_d<512>(a, fin, st);
        case 768: return launch_retrieve_d<768>(a, fin, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ltk
