// retrieve.hip -- fused inner-product retrieval top-k for gfx950.
//
// The same Sample -> Filter -> Select method as the indexer (LiteTopK pages,
// "Methodology"; the pages apply the primitive to vector retrieval), with
// the score I[t, s] = q[t] . x[s] of bf16 vectors (fp32 accumulation) and no
// causal mask.  Queries sit on the MFMA M dimension: one wave holds 32
// queries in registers and scores them against 32 database rows per tile, so
// every accumulator register is a (query, row) score and no head reduction
// is needed.  Database rows stream through LDS in tiles (direct global->LDS
// loads) shared by the 8 waves of a workgroup (256 queries), two waves per
// SIMD, so that one wave's candidate handling and refreshes overlap the
// other's MFMAs (4 waves at D = 64, whose tile is 4 loads).
//
// The database is split across workgroups.  Their per-query histograms are
// one shared array in device memory: every kept candidate adds to it with an
// atomic (no return value, so the wave does not wait), and a workgroup
// refreshes its threshold bins from the shared counts.  Candidates go to a
// fixed slice of the query's buffer per split, counted in LDS, so keeping one
// costs no round trip to device memory; a compaction pass then packs the
// slices of each query before the select.  Counts only ever cover real database rows, so any refresh is at
// most the true threshold bin and the result stays exact; sharing lets the
// threshold rise even though no single split holds k matching rows.
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "internal.hpp"
#include "kernels_common.hpp"

namespace ltk {

constexpr int kRetrQ = 32;                // queries per wave (one MFMA M block)
constexpr int kRetrQB = 1;                // query blocks per wave
constexpr int kRetrRows = 32;             // database rows per LDS tile
constexpr int kRetrRefreshCands = 128;    // candidates a wave adds before it refreshes
constexpr int kSuperBins = 16;            // fine bins per super-bin of the shared histogram

constexpr int kRetrStashRegs = 8;         // accumulator registers staged per rare-path round
constexpr int kRetrQueue = 128;           // candidate queue entries per wave (flushed 64 at a time)
constexpr int kRetrSplitRowsLog2 = 26;    // a split's rows fit 26 bits of a queue entry

template <int D>
struct RetrGeom {
    static constexpr int RB = 2 * D;                       // bf16 row bytes
    static constexpr int CPR = RB / 16;                    // 16-byte chunks per row
    static constexpr int TILE = kRetrRows * RB;            // bytes per tile
    static constexpr int NINST = kRetrRows * CPR / 64;     // wave-wide 1 KB loads per tile
    static constexpr int W = retr_waves(D);                // waves per workgroup (two per SIMD)
    static_assert(W * kRetrQ == retr_group_queries(D), "query group size as the host computes it");
    static constexpr int LPW = NINST / W;                  // loads per wave per tile
    static constexpr int KSTEPS = D / 16;                  // v_mfma_f32_32x32x16_bf16 steps
    static_assert(NINST % W == 0, "tile loads split evenly over the waves");
    // per wave: thresholds, candidate counts, bin-map origin and scale of its queries; score
    // stash; candidate queue
    static constexpr size_t FIXED_LDS = (size_t)W * kRetrQB * kRetrQ * 4 * 4 +
                                        (size_t)W * kRetrStashRegs * 64 * 4 + (size_t)W * kRetrQueue * 8;
    // tile stages: as many as fit (at most 4), so tiles are requested one to
    // three tiles ahead of their use (two at D = 768, where a tile of MFMA
    // work for the 8 waves takes ~2 us)
    static constexpr int NST = ((kMaxLds - FIXED_LDS) / TILE) < 4 ? (int)((kMaxLds - FIXED_LDS) / TILE) : 4;
    static_assert(NST >= 2, "at least double buffering");
    static constexpr size_t LDS = (size_t)NST * TILE + FIXED_LDS;
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

// Byte offset, within a tile, of this lane's 16-byte chunk in the wave's
// j-th 1 KB direct load (chunk p = 64*inst + lane holds chunk
// (p % CPR) ^ swz(row) of row p / CPR); the same for every tile.
template <int D>
__device__ __forceinline__ uint32_t retr_part_off(int wave, int lane, int j) {
    using G = RetrGeom<D>;
    const int inst = wave + j * RetrGeom<D>::W;
    const int p = inst * 64 + lane;
    const int r = p / G::CPR, pc = p % G::CPR;
    return (uint32_t)(r * G::RB + (pc ^ chunk_swz<G::RB, G::CPR>(r)) * 16);
}
// Source of the tile starting at row0: a wave-uniform base row and the
// largest in-bounds chunk offset from it.  Clamping a lane's offset to `lim`
// leaves every chunk of a row below N where it is (its offset is at most
// lim) and sends those of rows past the end (a ragged last tile, tiles
// requested past a split's last one) to the database's last chunk.
struct TileSrc {
    const uint8_t* base;
    uint32_t lim;
};
template <int D>
__device__ __forceinline__ TileSrc retr_tile_src(const RetrArgs& a, int row0) {
    const int r0 = min(row0, a.N - 1);
    const int64_t lim = (int64_t)(a.N - r0) * RetrGeom<D>::RB - 16;
    return {a.db + (size_t)r0 * RetrGeom<D>::RB, (uint32_t)min<int64_t>(lim, (int64_t)0xffffffffu)};
}
template <int D>
__device__ __forceinline__ void retr_load_part(const TileSrc& src, uint32_t off, uint8_t* st, int wave, int j) {
    lds_direct16_async(src.base, min(off, src.lim), st + (wave + j * RetrGeom<D>::W) * 1024);
}

// Coherent (device-scope) read of a shared counter.
__device__ __forceinline__ uint32_t load_shared_count(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FULL: the unfused comparison path -- every score goes to the T x N matrix
// a.S, with no sample, gate or candidates (the same MFMA order, so the same
// fp32 scores as the fused scan).
template <int D, bool FULL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void retr_scan_kernel(RetrArgs a) {
    using G = RetrGeom<D>;
    constexpr int QW = kRetrQB * kRetrQ;                                  // queries per wave
    constexpr int NR = kRetrQB * 16;                                      // score registers per lane and tile
    extern __shared__ __attribute__((aligned(16))) uint8_t shm[];
    uint8_t* tiles = shm;                                                 // G::NST stages
    float* tau_l = reinterpret_cast<float*>(shm + G::NST * G::TILE);      // [waves][QW queries]
    uint32_t* cnt_l = reinterpret_cast<uint32_t*>(tau_l + G::W * QW);   // [waves][QW]
    float* smin_l = reinterpret_cast<float*>(cnt_l + G::W * QW);        // [waves][QW]
    float* delta_l = smin_l + G::W * QW;                                 // [waves][QW]
    float* stash = delta_l + G::W * QW;                              // [waves][8][64] scores
    uint2* queue = reinterpret_cast<uint2*>(stash + G::W * kRetrStashRegs * 64);   // [waves][kRetrQueue]
    static_assert(QW <= 64, "a queue entry holds the query in 6 bits");
    const int wave = threadIdx.x >> 6, lane = lane_id(), half = lane >> 5;

    // (split, query group) from the block index so that the query groups of
    // one split are dispatched back to back on the same XCD (block i runs on
    // XCD i % 8): they stream the same database rows through one L2.
    const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
    const int split = (slot / a.n_qgroups) * 8 + xcd, qgroup = slot % a.n_qgroups;
    if (split >= a.n_splits) return;
    const int q0 = qgroup * (G::W * QW) + wave * QW;
    const KeyRange rr = split_range(a.N, a.n_splits, split, kRetrRows);
    const int r_lo = rr.lo, r_hi = rr.hi;
    const int ntiles = (r_hi > r_lo) ? (r_hi - r_lo + kRetrRows - 1) / kRetrRows : 0;
    if (ntiles == 0) return;

    // the wave's query blocks: every database-row fragment read from LDS feeds
    // one MFMA per block
    HalfRow<DT_BF16, D> qf[kRetrQB];
#pragma unroll
    for (int b = 0; b < kRetrQB; ++b) load_qblock<D>(qf[b], a, q0 + b * kRetrQ);
    drain_vm_loads();
    const Meta* meta = reinterpret_cast<const Meta*>(a.meta);

    // thresholds of the wave's queries: lane i owns query q0 + i
    int thr_own = 0;
    Meta m_own{0.0f, 1.0f, 0, 0};
    const bool own_lane = lane < QW;
    const bool own_valid = own_lane && q0 + lane < a.T;
    if (!FULL && own_valid) {
        m_own = meta[q0 + lane];
        thr_own = m_own.thr0;
    }
    float* my_tau = tau_l + wave * QW;
    uint32_t* my_cnt = cnt_l + wave * QW;
    if (own_lane) {
        my_tau[lane] = own_valid ? initial_gate(thr_own, m_own, a.nbins, a.topk) : INFINITY;
        my_cnt[lane] = 0u;
        smin_l[wave * QW + lane] = m_own.smin;
        delta_l[wave * QW + lane] = m_own.delta;
    }
    uint2* cand_base = a.cand + (size_t)split * a.cap_s;   // + q * ccap: this split's slice of query q
    // query (of the wave) of score register R: block R / 16, row of register R % 16
    auto rq = [&](int R) { return (R >> 4) * kRetrQ + reg_query(0, R & 15, half); };
    int added = 0;   // candidates this wave added since its last refresh (wave-uniform)

    uint32_t loff[G::LPW];
#pragma unroll
    for (int j = 0; j < G::LPW; ++j) loff[j] = retr_part_off<D>(wave, lane, j);
    constexpr int LEAD = G::NST - 1;   // tiles requested ahead of the one computed
#pragma unroll
    for (int t = 0; t < LEAD; ++t)
        if (t < ntiles) {
            const TileSrc src = retr_tile_src<D>(a, r_lo + t * kRetrRows);
#pragma unroll
            for (int j = 0; j < G::LPW; ++j) retr_load_part<D>(src, loff[j], tiles + t * G::TILE, wave, j);
        }
    // The wave's queued candidates: each lane takes one entry, claims a slot
    // of the query's slice with an LDS atomic, writes it and adds to the
    // shared histograms without waiting for a reply.
    uint2* my_q = queue + wave * kRetrQueue;
    int qn = 0;       // queued entries (wave-uniform)
    int vm_now = 0;   // vector-memory instructions the flushes of this tile issued (a lower bound)
    auto flush = [&]() {
        for (int b0 = 0; b0 < qn; b0 += 64) {
            if (b0 + lane < qn) {
                const uint2 e = my_q[b0 + lane];
                const int ql = (int)(e.y & 63u);
                const int q = q0 + ql;
                const uint32_t p = atomicAdd(&my_cnt[ql], 1u);
                if ((int64_t)p < a.cap_s) cand_base[(size_t)q * a.ccap + p] = make_uint2((uint32_t)r_lo + (e.y >> 6), e.x);
                const int b = bin_of(__uint_as_float(e.x), smin_l[wave * QW + ql], delta_l[wave * QW + ql], a.nbins);
                atomicAdd(&a.hist_g[(size_t)q * a.nbins + b], 1u);
                atomicAdd(&a.hist_c[(size_t)q * a.nsuper + b / kSuperBins], 1u);
            }
            vm_now += 2;   // two atomics per round (some lane is active)
        }
        qn = 0;
    };
    int sbuf = 0;   // stage of tile `it`
    int vm_prev1 = 0, vm_prev2 = 0;   // vector-memory instructions of the last two tiles' candidate paths
    for (int it = 0; it < ntiles; ++it) {
        // Wait for this tile's loads only: the loads of tiles it+1 .. it+LEAD-1
        // (those that exist) may still be in flight, and so may the
        // vector-memory instructions the last two tiles' candidate flushes
        // issued after this tile's loads (vm_prev1 + vm_prev2 is a lower bound
        // of their count).
        const int later = min(LEAD - 1, ntiles - 1 - it);
        if (later <= 0) wait_vm<0>();
        else if (later == 1) wait_vm_plus<G::LPW>(vm_prev1 + vm_prev2);
        else wait_vm_plus<2 * G::LPW>(vm_prev1 + vm_prev2);
        __syncthreads();   // every wave's share of tile `it` has landed; the stage of tile it-1 is free
        // the loads of tile it+LEAD go out spread over this tile's MFMAs (below):
        // issued back to back they hold the wave at the memory pipe before its
        // MFMAs.  They go out unconditionally (no branch between the MFMAs): past
        // the last tile they re-read clamped rows into a stage nothing reads, and
        // being the newest loads they never loosen the waits above.
        const TileSrc src_next = retr_tile_src<D>(a, r_lo + (it + LEAD) * kRetrRows);
        uint8_t* st_next = tiles + ((sbuf + LEAD) % G::NST) * G::TILE;
        const uint8_t* st = tiles + sbuf * G::TILE;
        sbuf = (sbuf + 1) % G::NST;
        const int rrow = lane & 31;
        const int row = r_lo + it * kRetrRows + rrow;
        // B fragments read from LDS two steps ahead of their MFMAs (the other
        // wave of the SIMD covers the rest of the latency); the
        // scheduling barriers keep the compiler from hoisting every read
        const uint8_t* rowp = st + rrow * G::RB;
        const int sw = chunk_swz<G::RB, G::CPR>(rrow);
        // When the half-row offset is a multiple of the swizzle span, the XOR
        // only touches the low bits of s: one XOR with a constant per read and
        // an immediate offset.  The XOR is opaque to the compiler (volatile
        // asm), which would otherwise keep one address register per step.
        constexpr int SPAN = G::CPR < 16 ? G::CPR : 16;
        typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
        const uint32_t lbase =
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(rowp + half * (G::CPR / 2) * 16);
        const uint32_t sw16 = (uint32_t)sw * 16u;
        auto rd = [&](int s) {
            if constexpr ((G::CPR / 2) % SPAN == 0) {
                uint32_t x;
                asm volatile("v_xor_b32 %0, %1, %2" : "=v"(x) : "n"((s & (SPAN - 1)) * 16), "v"(sw16));
                return *(reinterpret_cast<lds_u32x4*>((uintptr_t)(lbase + x)) + (s & ~(SPAN - 1)));
            } else {
                return *reinterpret_cast<const u32x4*>(rowp + (((half * (G::CPR / 2) + s) ^ sw) * 16));
            }
        };
        constexpr int PF = G::KSTEPS < 2 ? G::KSTEPS : 2;
        u32x4 bq[PF];
#pragma unroll
        for (int s = 0; s < PF; ++s) bq[s] = rd(s);
        v16f acc[kRetrQB];
#pragma unroll
        for (int b = 0; b < kRetrQB; ++b) acc[b] = v16f{};
        // issue priority falls through the tile (3, 2 over the MFMAs, 1 for the
        // gate and the candidates, 0 in a refresh): of the two waves of a
        // SIMD the one behind issues first
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            constexpr int LSTEP = G::KSTEPS / G::LPW;   // MFMA steps between this wave's tile loads
            if (s == 0) set_wave_prio(3);
            else if (s == G::KSTEPS / 2) set_wave_prio(2);
            if (s % LSTEP == 0 && s / LSTEP < G::LPW)
            {
                int ln;
                asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
                retr_load_part<D>(src_next, retr_part_off<D>(wave, ln, s / LSTEP), st_next, wave, s / LSTEP);
            }
#pragma unroll
            for (int b = 0; b < kRetrQB; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf[b].v[s]),
                                                                 __builtin_bit_cast(bf16x8, bq[s % PF]), acc[b], 0, 0, 0);
            if (s + PF < G::KSTEPS) bq[s % PF] = rd(s + PF);
            if (s % PF == PF - 1) __builtin_amdgcn_sched_barrier(0);
        }
        set_wave_prio(1);
        if constexpr (FULL) {
#pragma unroll
            for (int R = 0; R < NR; ++R) {
                const int q = q0 + rq(R);
                if (row < r_hi && q < a.T) a.S[(size_t)q * (size_t)a.N + row] = acc[R >> 4][R & 15];
            }
            continue;
        }
        // gate: one compare per register into a wave mask (scalar ORs); the
        // per-lane mask of passing registers (bit R of pm) only when some pass
        // (thresholds read from LDS: four queries' in one 16-byte read)
        float tau[NR];
#pragma unroll
        for (int R = 0; R < NR; R += 4) {
            const float4 t4 = *reinterpret_cast<const float4*>(my_tau + rq(R));
            tau[R] = t4.x; tau[R + 1] = t4.y; tau[R + 2] = t4.z; tau[R + 3] = t4.w;
        }
        vm_now = 0;
        uint64_t any = 0;
#pragma unroll
        for (int R = 0; R < NR; ++R) any |= __builtin_amdgcn_ballot_w64(acc[R >> 4][R & 15] >= tau[R]);
        if (any & __builtin_amdgcn_ballot_w64(row < r_hi)) {
            const bool rv = row < r_hi;
            uint32_t pm = 0;
#pragma unroll
            for (int R = 0; R < NR; ++R) pm |= (rv && acc[R >> 4][R & 15] >= tau[R]) ? (1u << R) : 0u;
            // candidates (a few per tile once the thresholds have risen): each
            // round every lane with passing registers appends its lowest one
            // to the wave's queue in LDS (score read back from a wave-private
            // copy of 8 registers, position from the round's ballot); full
            // queues are flushed 64 entries per instruction, so the vector-memory
            // traffic per tile stays a few instructions, not three per candidate
            float* sv = stash + wave * kRetrStashRegs * 64;
#pragma unroll
            for (int rb = 0; rb < NR; rb += kRetrStashRegs) {
                uint32_t pr = (pm >> rb) & ((1u << kRetrStashRegs) - 1u);
                if (__ballot(pr != 0u)) {
#pragma unroll
                    for (int r = 0; r < kRetrStashRegs; ++r) sv[r * 64 + lane] = acc[(rb + r) >> 4][(rb + r) & 15];
                    while (true) {
                        const uint64_t m = __ballot(pr != 0u);
                        if (!m) break;
                        const int n = __popcll(m);
                        if (qn + n > kRetrQueue) flush();
                        if (pr) {
                            const int reg = rb + __ffs(pr) - 1;
                            pr &= pr - 1u;
                            const uint32_t pos = (uint32_t)qn + __builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                            my_q[pos] = make_uint2(__float_as_uint(sv[(reg - rb) * 64 + lane]),
                                                   ((uint32_t)(row - r_lo) << 6) | (uint32_t)rq(reg));
                        }
                        qn += n;
                    }
                }
            }
            added += __popcll(__ballot(pm != 0u));   // lanes that kept a candidate (a lower bound)
        }
        // refresh from the shared histograms once this wave has added enough
        // candidates: accumulate counts from the top bin down (super-bins
        // first, then the fine bins of the crossing super-bin), and overwrite
        // the wave's thresholds -- plain stores that can only raise them.
        // Every counter read is at most the number of real rows in its bin, so
        // the new threshold bin is at most the true one.
        if (qn >= 64 || (qn > 0 && added >= kRetrRefreshCands)) flush();
        if (added >= kRetrRefreshCands) {
            added = 0;
            set_wave_prio(0);
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
            }
        }
        vm_prev2 = vm_prev1;
        vm_prev1 = min(vm_now, 64);
    }
    if constexpr (!FULL) flush();
    wait_vm<0>();   // loads issued past the last tile land before the workgroup ends
    // candidates this split found for each of the wave's queries (may exceed the slice)
    if (!FULL && own_valid) a.seg_cnt[(size_t)(q0 + lane) * a.n_splits + split] = my_cnt[lane];
}

// ---------------------------------------------------------------------------
// Compaction: pack the per-split slices of each query's candidate buffer into
// a prefix, in place.  Entry v of the packed order comes from slice s (the
// split holding it) at s * cap_s + (v - start of s) >= v, so rounds that stage
// a range of v in LDS, then write it back, never overwrite an entry a later
// round still has to read.  A slice that overflowed sends the query to the
// exact fallback (its tail is set past the buffer capacity).
// ---------------------------------------------------------------------------

constexpr int kCompactStage = 8192;   // entries staged per round (64 KB of LDS)

__global__ __launch_bounds__(256) void retr_compact_kernel(RetrArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t shm[];
    uint2* stage = reinterpret_cast<uint2*>(shm);                         // [kCompactStage]
    uint32_t* start = reinterpret_cast<uint32_t*>(stage + kCompactStage); // [n_splits + 1]
    __shared__ uint32_t s_part[256];
    __shared__ uint32_t s_total, s_over;
    const int t = blockIdx.x, tid = threadIdx.x, ns = a.n_splits;
    const uint32_t cap = (uint32_t)a.cap_s;
    const uint32_t* cnt = a.seg_cnt + (size_t)t * ns;
    // exclusive prefix of the kept counts: each thread sums a contiguous run of splits
    const int per = (ns + 255) / 256, lo = tid * per, hi = min(ns, lo + per);
    uint32_t run = 0, over = 0;
    uint64_t found = 0;
    for (int s = lo; s < hi; ++s) {
        const uint32_t c = cnt[s];
        found += c;
        over |= (c > cap) ? 1u : 0u;
        run += min(c, cap);
    }
    s_part[tid] = run;
    if (tid == 0) { s_total = 0u; s_over = 0u; }
    __syncthreads();
    if (over) atomicOr(&s_over, 1u);
    atomicAdd(&s_total, (uint32_t)min<uint64_t>(found, 0xffffffffull));
    if (tid == 0) {   // 256 partial sums, serially
        uint32_t acc = 0;
        for (int i = 0; i < 256; ++i) {
            const uint32_t v = s_part[i];
            s_part[i] = acc;
            acc += v;
        }
    }
    __syncthreads();
    uint32_t acc = s_part[tid];
    for (int s = lo; s < hi; ++s) {
        start[s] = acc;
        acc += min(cnt[s], cap);
    }
    if (tid == 255) start[ns] = acc;
    __syncthreads();
    const uint32_t kept = start[ns];
    if (s_over) {   // the fallback recomputes this row
        if (tid == 0) a.tail[t] = (uint32_t)max<int64_t>((int64_t)s_total, a.ccap + 1);
        return;
    }
    uint2* c = a.cand + (size_t)t * a.ccap;
    for (uint32_t r0 = 0; r0 < kept; r0 += kCompactStage) {
        const uint32_t r1 = min(kept, r0 + (uint32_t)kCompactStage);
        for (uint32_t v = r0 + tid; v < r1; v += 256) {
            int l = 0, h = ns;   // last split with start <= v
            while (h - l > 1) {
                const int m = (l + h) >> 1;
                if (start[m] <= v) l = m; else h = m;
            }
            stage[v - r0] = c[(size_t)l * cap + (v - start[l])];
        }
        __syncthreads();
        for (uint32_t v = r0 + tid; v < r1; v += 256) c[v] = stage[v - r0];
        __syncthreads();
    }
    if (tid == 0) a.tail[t] = kept;
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
    // a sorted row without out_score ranks by an LDS row of scores past the sort keys
    float* osc = a.out_score ? a.out_score + (size_t)t * a.topk
                             : (a.sorted ? reinterpret_cast<float*>(sh + 256 + 2 * sort_p2(a.topk)) : nullptr);
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
    const size_t lds = G::LDS;
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(retr_scan_kernel<D, false>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int nsplit_pad = (a.n_splits + 7) / 8 * 8;
    if (a.ev_scan_start) (void)hipEventRecord(a.ev_scan_start, st);
    retr_scan_kernel<D, false><<<nsplit_pad * a.n_qgroups, G::W * 64, lds, st>>>(a);
    if (a.ev_scan_stop) (void)hipEventRecord(a.ev_scan_stop, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t compact_lds = (size_t)kCompactStage * 8 + ((size_t)a.n_splits + 1) * 4;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(retr_compact_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)compact_lds);
    retr_compact_kernel<<<a.T, 256, compact_lds, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_finalize(fin, st)) != hipSuccess) return e;
    const size_t fb_lds = row_select_lds(a.topk, a.sorted, a.out_score != nullptr);
    if (fb_lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(retr_fallback_kernel<D>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)fb_lds);
    retr_fallback_kernel<D><<<a.T, 256, fb_lds, st>>>(a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_retrieve_unfused_d(const RetrArgs& a, const IdxArgs& sel, hipStream_t st) {
    using G = RetrGeom<D>;
    const size_t lds = G::LDS;
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(retr_scan_kernel<D, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int nsplit_pad = (a.n_splits + 7) / 8 * 8;
    if (a.ev_scan_start) (void)hipEventRecord(a.ev_scan_start, st);
    retr_scan_kernel<D, true><<<nsplit_pad * a.n_qgroups, G::W * 64, lds, st>>>(a);
    if (a.ev_scan_stop) (void)hipEventRecord(a.ev_scan_stop, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_unfused_select(sel, st);
}

hipError_t launch_retrieve_unfused(int D, const RetrArgs& a, const IdxArgs& sel, hipStream_t st) {
    switch (D) {
        case 64: return launch_retrieve_unfused_d<64>(a, sel, st);
        case 128: return launch_retrieve_unfused_d<128>(a, sel, st);
        case 256: return launch_retrieve_unfused_d<256>(a, sel, st);
        case 512: return launch_retrieve_unfused_d<512>(a, sel, st);
        case 768: return launch_retrieve_unfused_d<768>(a, sel, st);
        default: return hipErrorInvalidValue;
    }
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
