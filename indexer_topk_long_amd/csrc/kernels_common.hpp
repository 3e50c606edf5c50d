// kernels_common.hpp -- device helpers shared by the indexer and retrieval kernels.
#pragma once

#include <math.h>

#include "device.hpp"

namespace ltk {

// Wait until at most n of this wave's vector-memory operations are in flight.
// Vector-memory operations complete in issue order, so this means that
// everything but the n most recent (the next tile's loads) has landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// wait_vm<N + e> for a wave-uniform run-time count `extra` of further vector
// memory instructions known to have been issued after the awaited ones:
// e is the largest step of {0, 4, 8, 16, 32} not above extra (and with
// N + e <= 63), so the wait never allows more than extra beyond N.
template <int N>
__device__ __forceinline__ void wait_vm_plus(int extra) {
    if constexpr (N + 32 <= 63) {
        if (extra >= 32) { wait_vm<N + 32>(); return; }
    }
    if constexpr (N + 16 <= 63) {
        if (extra >= 16) { wait_vm<N + 16>(); return; }
    }
    if constexpr (N + 8 <= 63) {
        if (extra >= 8) { wait_vm<N + 8>(); return; }
    }
    if constexpr (N + 4 <= 63) {
        if (extra >= 4) { wait_vm<N + 4>(); return; }
    }
    wait_vm<N>();
}

// Wait, visibly to the compiler, until every vector-memory load issued so far
// has landed (s_waitcnt vmcnt(0); expcnt and lgkmcnt untouched).  Used once
// after the per-wave register loads that precede a streaming loop: the
// compiler's wait analysis merges the loop entry (those loads pending) with
// the back edge and otherwise re-inserts waits for them before their uses in
// every iteration, waits that then also stall on the tile loads in flight.
__device__ __forceinline__ void drain_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Issue priority of the calling wave (s_setprio takes an immediate; with a
// constant level, as in an unrolled loop, this folds to one instruction).
// The scans lower a wave's priority as it works through a tile, so that of
// the two waves sharing a SIMD the one behind issues first.
__device__ __forceinline__ void set_wave_prio(int level) {
    if (level >= 3) __builtin_amdgcn_s_setprio(3);
    else if (level == 2) __builtin_amdgcn_s_setprio(2);
    else if (level == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// XOR swizzle of the 16-byte chunks of a row.  LDS has 64 four-byte banks (a
// 256-byte bank line).  The MFMA fragment read of the scans is the half-row
// read: lane l takes row (l & 31), and the two 32-lane halves take different
// chunks, so consecutive lanes read consecutive rows at the same logical
// chunk.  XORing the chunk index with the row's position among the rows that
// share a bank-line slot spreads them over distinct 16-byte slots.  Measured
// on gfx950 this read costs 4 LDS cycles per 1 KB instruction, the same as a
// linear read; an unswizzled (or 32-bank-keyed) layout costs twice that.
template <int RB, int CPR>
__device__ __forceinline__ int chunk_swz(int r) {
    constexpr int RPL = (RB < 256) ? 256 / RB : 1;       // rows per 256-byte bank line
    constexpr int MASK = (CPR < 16 ? CPR : 16) - 1;
    return (r / RPL) & MASK;
}

// Direct global -> LDS copies (gfx950 global_load_lds): every lane moves 16
// (or 4) bytes, landing at lds + 16*lane (4*lane); lds must be wave-uniform.
__device__ __forceinline__ void lds_direct16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_direct4(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// The same 16-byte direct copy issued as inline assembly (M0 = LDS base, then
// the load).  The compiler treats a pending LDS DMA issued through the builtin
// as possibly aliasing every later LDS access: it drains all loads in flight
// (vmcnt(0)) before each barrier, so no more than one tile can be in flight
// across a barrier.  A kernel that streams several tiles ahead uses this form
// and orders the copies itself: wait_vm on all but the newest tiles' loads,
// then a barrier.  Vector memory operations complete in issue order, so the
// compiler's own vmcnt waits stay correct with these copies in flight.
__device__ __forceinline__ void lds_direct16_async(const void* g, void* lds) {
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(off) : "memory", "m0");
}
// The same copy from a wave-uniform base (SGPRs) plus a per-lane 32-bit byte
// offset, so that no per-load address arithmetic is needed.
// A wave-uniform 64-bit pointer in scalar registers.  The builtin returns a
// signed int: each half goes through uint32_t before widening, so the low
// half is zero-extended (a sign-extended low half would corrupt the high one).
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ void lds_direct16_async(const void* base, uint32_t off, void* lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(uniform_ptr(base)), "s"(m)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_direct4_async(const void* base, uint32_t off, void* lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(off), "s"(uniform_ptr(base)), "s"(m)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_direct4_async(const void* g, void* lds) {
    const uint32_t off = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(off) : "memory", "m0");
}

// Smallest fp32 score whose bin is >= thr (bin_of is monotone), found by
// bisection over the ordered float encoding: the gate I >= tau is then
// exactly the gate bin_of(I) >= thr, and the bin is only computed for keys
// that pass.
__device__ __forceinline__ float tau_of(int thr, float smin, float delta, int nbins) {
    if (thr <= 0) return -INFINITY;
    uint32_t lo = ord_f32(-3.402823466e38f), hi = ord_f32(3.402823466e38f);   // bin(lo) < thr <= bin(hi)
    while (hi - lo > 1u) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        if (bin_of(unord_f32(mid), smin, delta, nbins) >= thr) hi = mid; else lo = mid;
    }
    return unord_f32(hi);
}

// Initial gate of a query: the gate of its threshold bin, except that bin 0
// also counts every score below the sample's minimum (the bin map clamps them
// for counting).  When at least k valid sample keys scored >= smin, no key
// scoring below smin can be in the top-k, so bin 0 gates at smin itself.
// Sample and scan score a key bit-identically, so the sample's own keys pass.
__device__ __forceinline__ float initial_gate(int thr, const Meta& m, int nbins, int k) {
    if (thr <= 0) return (m.nvalid >= k) ? m.smin : -INFINITY;
    return tau_of(thr, m.smin, m.delta, nbins);
}

// Block-wide bitonic sort (descending) of n <= cap 64-bit keys in LDS.
__device__ inline void block_sort_desc(uint64_t* keys, int n) {
    int p2 = 1;
    while (p2 < n) p2 <<= 1;
    for (int i = n + threadIdx.x; i < p2; i += blockDim.x) keys[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= p2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < p2 / 2; i += blockDim.x) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = ((lo & size) == 0);
                const uint64_t x = keys[lo], y = keys[hi];
                if ((x < y) == desc) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// Power of two >= k: the sort keys of a sorted row.
__host__ __device__ inline int sort_p2(int k) {
    int p2 = 1;
    while (p2 < k) p2 <<= 1;
    return p2;
}

// LDS of an exact row select (select_row) followed by an optional sort:
// 256 digit counters, the sort keys, and, for a sorted output without
// out_score, an LDS row of the scores (the sort ranks by them).
__host__ __device__ inline size_t row_select_lds(int topk, bool sorted, bool with_scores) {
    if (!sorted) return 256 * 4;
    return 256 * 4 + (size_t)sort_p2(topk) * 8 + (with_scores ? 0 : (size_t)topk * 4);
}

// Order the k outputs of one row by (score desc, index asc).  osc holds the
// row's scores (the caller's output row, or an LDS row when the caller asked
// for indices only) and is rewritten in the same order.
__device__ inline void sort_row_output(int32_t* out, float* osc, int k, uint64_t* keys) {
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        const int idx = out[i];
        keys[i] = (idx >= 0) ? rank_key(osc[i], idx) : 0ull;
    }
    __syncthreads();
    block_sort_desc(keys, k);
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        const uint64_t key = keys[i];
        if (key == 0ull) {
            out[i] = -1;
            osc[i] = __builtin_nanf("");
        } else {
            out[i] = (int32_t)(0xffffffffu - (uint32_t)key);
            osc[i] = unord_f32((uint32_t)(key >> 32));
        }
    }
    __syncthreads();
}

// Scores re-read from the materialised row (unfused baseline).
struct MemSource {
    const float* row;
    __device__ __forceinline__ void get(int base, int nvalid, int& key, float& I, bool& valid) {
        key = base + (int)threadIdx.x;
        valid = key < nvalid;
        I = valid ? row[key] : 0.0f;
    }
};

template <class Src>
__device__ void select_row(Src& src, int nvalid, int k, int32_t* out, float* osc, uint32_t* h256) {
    __shared__ int s_pick;
    __shared__ uint32_t s_above, s_ocnt, s_taken, s_wc[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
    if (nvalid <= k) {   // every valid key is in the result
        for (int base = 0; base < nvalid; base += 256) {
            int key;
            float I;
            bool valid;
            src.get(base, nvalid, key, I, valid);
            if (valid) {
                out[key] = key;
                if (osc) osc[key] = I;
            }
        }
        for (int i = max(nvalid, 0) + tid; i < k; i += 256) {
            out[i] = -1;
            if (osc) osc[i] = __builtin_nanf("");
        }
        return;
    }
    uint32_t P = 0u, mask = 0u, need = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        __syncthreads();
        for (int i = tid; i < 256; i += 256) h256[i] = 0u;
        __syncthreads();
        for (int base = 0; base < nvalid; base += 256) {
            int key;
            float I;
            bool valid;
            src.get(base, nvalid, key, I, valid);
            const uint32_t u = ord_f32(I);
            if (valid && (u & mask) == P) atomicAdd(&h256[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            const SuffixPick p = suffix_pick(h256, 256, need);
            if (lane == 0) {
                s_pick = p.bin;
                s_above = p.above;
            }
        }
        __syncthreads();
        P |= (uint32_t)s_pick << shift;
        mask |= 0xffu << shift;
        need -= s_above;
    }
    // P is now the k-th largest score; `need` of its ties are taken, lowest index first
    const uint32_t ngt = (uint32_t)k - need;
    if (tid == 0) {
        s_ocnt = 0u;
        s_taken = 0u;
    }
    __syncthreads();
    for (int base = 0; base < nvalid; base += 256) {
        int key;
        float I;
        bool valid;
        src.get(base, nvalid, key, I, valid);
        const uint32_t u = ord_f32(I);
        const bool gt = valid && u > P;
        const bool eq = valid && u == P;
        if (gt) {
            const uint32_t p = atomicAdd(&s_ocnt, 1u);
            if (p < ngt) {
                out[p] = key;
                if (osc) osc[p] = I;
            }
        }
        const uint64_t em = __ballot(eq);
        if (lane == 0) s_wc[wave] = (uint32_t)__popcll(em);
        __syncthreads();
        uint32_t before = s_taken, total = 0;
        for (int w = 0; w < 4; ++w) {
            if (w < wave) before += s_wc[w];
            total += s_wc[w];
        }
        if (eq) {
            const uint32_t rank = before + (uint32_t)mbcnt(em);
            if (rank < need) {
                out[ngt + rank] = key;
                if (osc) osc[ngt + rank] = I;
            }
        }
        __syncthreads();
        if (tid == 0) s_taken += total;
    }
}

}  // namespace ltk
