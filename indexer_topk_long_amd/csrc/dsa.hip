// dsa.hip -- LiteDSA packing for gfx950.
//
// LiteTopK pages, arXiv abstract: LiteDSA packs the candidates that
// neighbouring query tokens have in common into one shared key/value list for
// joint attention, and per-query masks keep each token's own top-k membership.
//
// Pack: one workgroup of 1024 threads per group of G consecutive query rows.
// Neighbouring queries select mostly the same keys, so the group's distinct
// keys are few (about 4,700 of 32,768 selections at k = 2,048, G = 16):
//  1. every (key, row) selection goes into an LDS hash table of keys, whose
//     slot ORs the row's bit into the key's mask;
//  2. the distinct keys and their masks are put in ascending key order by a
//     counting sort on key-range buckets (a bitonic sort of (key, mask) pairs
//     where one bucket holds too many keys);
//  3. the list and masks are written out in order.
// A group with more distinct keys than half the table's slots is packed by
// sorting all of its G*k selections instead, each tagged with its row as
// key << 5 | row: equal keys are then adjacent, each run of one key becomes
// one list entry, and its mask is the OR of the run's row bits.
//
// Gather: the key/value rows of every group's list, copied contiguously in
// 16-byte vectors, so that the attention of the group reads each shared row
// once.
#include <algorithm>

#include "device.hpp"
#include "internal.hpp"

namespace ltk {

constexpr int kDsaThreads = 1024;
constexpr uint32_t kDsaEmpty = 0xffffffffu;   // above every key << 5 | row with key < 2^26
constexpr int kDsaPerThread = kDsaMaxEntries / kDsaThreads;

// Ascending bitonic sort of n (a power of two) values in LDS.
template <typename V>
__device__ inline void dsa_sort(V* v, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n / 2; i += kDsaThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const V x = v[lo], y = v[hi];
                if ((x > y) == up) {
                    v[lo] = y;
                    v[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// Sorted-selection path: all of the group's selections tagged with their row
// (v holds n2 >= G*k entries of LDS).
__device__ void dsa_pack_by_sort(uint32_t* v, const int32_t* src, int rows, int k, int L, int n2, int32_t* out_s,
                                 uint32_t* out_m, int cap, int32_t* len) {
    __shared__ uint32_t s_wsum[kDsaThreads / 64];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    for (int p = tid; p < n2; p += kDsaThreads) {
        uint32_t c = kDsaEmpty;
        if (p < rows * k) {
            const int s = src[p];
            if (s >= 0 && s < L) c = ((uint32_t)s << 5) | (uint32_t)(p / k);
        }
        v[p] = c;
    }
    __syncthreads();
    dsa_sort(v, n2);

    // thread tid owns the sorted positions [p0, p1); a run head is the first
    // entry of a key
    const int per = (n2 + kDsaThreads - 1) / kDsaThreads;
    const int p0 = min(tid * per, n2), p1 = min(p0 + per, n2);
    auto is_head = [&](int p) {
        const uint32_t x = v[p];
        return x != kDsaEmpty && (p == 0 || (v[p - 1] >> 5) != (x >> 5));
    };
    uint32_t heads = 0;
    for (int p = p0; p < p1; ++p) heads += is_head(p) ? 1u : 0u;
    uint32_t incl = wave_scan_add_u32(heads);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    uint32_t o = incl - heads, total = 0;
    for (int w = 0; w < kDsaThreads / 64; ++w) {
        if (w < wave) o += s_wsum[w];
        total += s_wsum[w];
    }
    for (int p = p0; p < p1; ++p) {
        if (!is_head(p)) continue;
        const uint32_t key = v[p] >> 5;
        uint32_t m = 0;
        for (int q = p; q < n2 && (v[q] >> 5) == key; ++q) m |= 1u << (v[q] & 31u);   // runs may cross p1
        out_s[o] = (int32_t)key;
        out_m[o] = m;
        ++o;
    }
    for (int j = (int)total + tid; j < cap; j += kDsaThreads) {
        out_s[j] = -1;
        out_m[j] = 0u;
    }
    if (tid == 0) *len = (int32_t)total;
}

constexpr int kDsaProbeMax = 256;   // probing steps before the group takes the sort path
constexpr int kDsaBatch = 4;        // selections a thread inserts together

__device__ __forceinline__ uint32_t dsa_slot(uint32_t key, int log2_slots) {
    return (key * 2654435761u) >> (32 - log2_slots);
}

constexpr int kDsaLog2SlotsMax = 14;   // hash slots: at most 16,384 (128 KB of keys and masks)
constexpr int kDsaSlotsPerThread = (1 << kDsaLog2SlotsMax) / kDsaThreads;
constexpr int kDsaBuckets = 4096;       // key-range buckets of the ranking pass
constexpr int kDsaBucketMax = 64;       // a fuller bucket sends the group to the bitonic sort


// Hash path (sh: 2 * slots + kDsaBuckets + 1 words of LDS).  Returns false,
// having written nothing, when the group has more distinct keys than half the
// slots.  The table stays at most half full, so that linear probing is short:
// a wave waits for its longest probe sequence, one LDS atomic per step.
//
// The distinct keys are then put in order by a counting sort on key-range
// buckets: each key's place is its bucket's start plus the number of smaller
// keys in its bucket.  A group with a bucket of more than kDsaBucketMax keys
// sorts its (key, mask) pairs bitonically instead.
__device__ bool dsa_pack_by_hash(uint32_t* sh, const int32_t* src, int rows, int k, int L, int log2_slots,
                                 int32_t* out_s, uint32_t* out_m, int cap, int32_t* len) {
    __shared__ uint32_t s_n, s_over, s_c, s_kmin, s_kmax;
    __shared__ uint32_t s_wsum[kDsaThreads / 64], s_wmax[kDsaThreads / 64];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int slots = 1 << log2_slots;
    const uint32_t limit = (uint32_t)(slots / 2);
    uint32_t* tk = sh;                     // keys
    uint32_t* tm = sh + slots;             // masks
    uint32_t* cnt = sh + 2 * slots;        // bucket counts, then bucket starts
    for (int i = tid; i < slots; i += kDsaThreads) {
        tk[i] = kDsaEmpty;
        tm[i] = 0u;
    }
    for (int i = tid; i <= kDsaBuckets; i += kDsaThreads) cnt[i] = 0u;
    if (tid == 0) {
        s_n = 0u;
        s_over = 0u;
        s_c = 0u;
        s_kmin = kDsaEmpty;
        s_kmax = 0u;
    }
    __syncthreads();
    // all of the thread's selections are loaded before the first insertion
    // (at most kDsaPerThread: G * k <= kDsaMaxEntries)
    const int total = rows * k;
    int32_t sel[kDsaPerThread];
#pragma unroll
    for (int r = 0; r < kDsaPerThread; ++r) {
        const int p = r * kDsaThreads + tid;
        sel[r] = (p < total) ? src[p] : -1;
    }
    uint32_t kmin = kDsaEmpty, kmax = 0u;
    // insertion, kDsaBatch selections of the thread at a time: their bucket
    // reads and CASes are independent, so a wave waits about one LDS round
    // trip per step rather than one per selection.  A key is inserted into the
    // first empty slot of the first bucket (4 slots, read as one 16-byte
    // word) along its probe sequence that has one; a CAS that loses its slot
    // to another key reads the same bucket again.  Slots never empty, so each
    // key lands in exactly one slot.
    const int log2_buckets = log2_slots - 2;
    const uint32_t bmask = (1u << log2_buckets) - 1u;
#pragma unroll
    for (int r0 = 0; r0 < kDsaPerThread; r0 += kDsaBatch) {
        if (__builtin_amdgcn_readfirstlane(*(volatile uint32_t*)&s_over) != 0) break;
        uint32_t key[kDsaBatch], bkt[kDsaBatch], pend = 0u, n_fresh = 0u;
#pragma unroll
        for (int b = 0; b < kDsaBatch; ++b) {
            const int s = sel[r0 + b];
            key[b] = (uint32_t)s;
            bkt[b] = dsa_slot((uint32_t)s, log2_buckets);
            if (s >= 0 && s < L) {
                pend |= 1u << b;
                kmin = min(kmin, (uint32_t)s);
                kmax = max(kmax, (uint32_t)s);
            }
        }
        for (int step = 0; pend != 0u; ++step) {
            if (step == kDsaProbeMax) {
                s_over = 1u;
                break;
            }
            u32x4 q[kDsaBatch];
#pragma unroll
            for (int b = 0; b < kDsaBatch; ++b)
                if (pend & (1u << b)) q[b] = *reinterpret_cast<const u32x4*>(tk + 4 * bkt[b]);
            uint32_t at[kDsaBatch], got[kDsaBatch];
#pragma unroll
            for (int b = 0; b < kDsaBatch; ++b) {
                at[b] = 4u;   // the slot found or claimed in the bucket; 4 = none
                got[b] = 0u;
                if (!(pend & (1u << b))) continue;
                const uint32_t v[4] = {q[b].x, q[b].y, q[b].z, q[b].w};
                uint32_t e = 4u;
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    if (v[i] == key[b]) at[b] = (uint32_t)i;
                    if (v[i] == kDsaEmpty) e = (uint32_t)i;
                }
                if (at[b] < 4u) {
                    got[b] = key[b];
                } else if (e < 4u) {
                    at[b] = e;
                    got[b] = atomicCAS(&tk[4 * bkt[b] + e], kDsaEmpty, key[b]);
                } else {
                    bkt[b] = (bkt[b] + 1u) & bmask;   // bucket full: the next one
                }
            }
#pragma unroll
            for (int b = 0; b < kDsaBatch; ++b) {
                if (!(pend & (1u << b)) || at[b] == 4u) continue;
                const bool fresh = got[b] == kDsaEmpty;
                if (fresh || got[b] == key[b]) {
                    atomicOr(&tm[4 * bkt[b] + at[b]], 1u << (uint32_t)(((r0 + b) * kDsaThreads + tid) / k));
                    n_fresh += fresh ? 1u : 0u;
                    pend &= ~(1u << b);
                }
            }
        }
        // the wave's new keys are counted together; past the limit the
        // group stops inserting (every wave polls the flag)
        n_fresh = wave_sum_u32(n_fresh);
        if (lane == 0 && n_fresh) {
            if (atomicAdd(&s_n, n_fresh) + n_fresh > limit) s_over = 1u;
        }
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
        atomicMin(&s_kmin, kmin);
        atomicMax(&s_kmax, kmax);
    }
    __syncthreads();
    const uint32_t n = s_n;
    if (s_over != 0u) return false;

    // the table's keys and masks move to registers (thread tid takes slots
    // tid, tid + 1024, ...) and are counted into buckets of
    // (key - kmin) >> shift, whose index is below kDsaBuckets
    const uint32_t lo = s_kmin, span = (n > 0u) ? s_kmax - lo : 0u;
    const int shift = max(0, (32 - __clz((int)span)) - 12);
    uint32_t mk[kDsaSlotsPerThread], mm[kDsaSlotsPerThread], mr[kDsaSlotsPerThread];
#pragma unroll
    for (int j = 0; j < kDsaSlotsPerThread; ++j) {
        const int i = j * kDsaThreads + tid;
        mk[j] = (i < slots) ? tk[i] : kDsaEmpty;
        mm[j] = (i < slots) ? tm[i] : 0u;
        mr[j] = 0u;
        if (mk[j] != kDsaEmpty) mr[j] = atomicAdd(&cnt[(mk[j] - lo) >> shift], 1u);
    }
    __syncthreads();   // the table is free from here on
    // exclusive scan of the counts (4 buckets per thread) and the largest bucket
    uint32_t c[kDsaBuckets / kDsaThreads], part = 0u, cmax = 0u;
#pragma unroll
    for (int i = 0; i < kDsaBuckets / kDsaThreads; ++i) {
        c[i] = cnt[(kDsaBuckets / kDsaThreads) * tid + i];
        part += c[i];
        cmax = max(cmax, c[i]);
    }
    uint32_t incl = wave_scan_add_u32(part);
    cmax = wave_max_u32(cmax);
    if (lane == 63) s_wsum[wave] = incl;
    if (lane == 0) s_wmax[wave] = cmax;
    __syncthreads();
    uint32_t run = incl - part, big = 0u;
    for (int w = 0; w < kDsaThreads / 64; ++w) {
        if (w < wave) run += s_wsum[w];
        big = max(big, s_wmax[w]);
    }
#pragma unroll
    for (int i = 0; i < kDsaBuckets / kDsaThreads; ++i) {
        cnt[(kDsaBuckets / kDsaThreads) * tid + i] = run;
        run += c[i];
    }
    if (tid == 0) cnt[kDsaBuckets] = n;
    __syncthreads();

    if (big <= (uint32_t)kDsaBucketMax) {
        // place each key in its bucket (sb), then rank it among the bucket's
        // keys; the ordered keys and masks go to ok and om (n <= slots / 2)
        uint32_t* sb = tk;
        uint32_t* ok = tm;
        uint32_t* om = tm + slots / 2;
#pragma unroll
        for (int j = 0; j < kDsaSlotsPerThread; ++j)
            if (mk[j] != kDsaEmpty) sb[cnt[(mk[j] - lo) >> shift] + mr[j]] = mk[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kDsaSlotsPerThread; ++j) {
            if (mk[j] == kDsaEmpty) continue;
            const uint32_t b = (mk[j] - lo) >> shift, b0 = cnt[b], b1 = cnt[b + 1];
            uint32_t less = 0u;
            for (uint32_t q = b0; q < b1; ++q) less += (sb[q] < mk[j]) ? 1u : 0u;
            ok[b0 + less] = mk[j];
            om[b0 + less] = mm[j];
        }
        __syncthreads();
        for (int j = tid; j < (int)n; j += kDsaThreads) {
            out_s[j] = (int32_t)ok[j];
            out_m[j] = om[j];
        }
    } else {
        // skewed keys: the (key, mask) pairs, compacted in any order and
        // padded to a power of two (at most slots / 2 of them: 64-bit values
        // in the table's place), sorted by key
        uint64_t* pv = reinterpret_cast<uint64_t*>(sh);
#pragma unroll
        for (int j = 0; j < kDsaSlotsPerThread; ++j) {
            const bool v = mk[j] != kDsaEmpty;
            const uint64_t m = __ballot(v);
            uint32_t base = 0u;
            if (lane == 0 && m) base = atomicAdd(&s_c, (uint32_t)__popcll(m));
            base = lane0_u32(base);
            if (v) pv[base + mbcnt(m)] = ((uint64_t)mk[j] << 32) | (uint64_t)mm[j];
        }
        int n2 = 1;
        while (n2 < (int)n) n2 <<= 1;
        for (int i = (int)n + tid; i < n2; i += kDsaThreads) pv[i] = ~0ull;
        __syncthreads();
        dsa_sort(pv, n2);
        for (int j = tid; j < (int)n; j += kDsaThreads) {
            const uint64_t x = pv[j];
            out_s[j] = (int32_t)(uint32_t)(x >> 32);
            out_m[j] = (uint32_t)x;
        }
    }
    for (int j = (int)n + tid; j < cap; j += kDsaThreads) {
        out_s[j] = -1;
        out_m[j] = 0u;
    }
    if (tid == 0) *len = (int32_t)n;
    return true;
}

__global__ __launch_bounds__(kDsaThreads) void dsa_pack_kernel(const int32_t* idx, int T, int k, int L, int G,
                                                               int n2, int log2_slots,
                                                               int32_t* shared, uint32_t* masks, int32_t* lens) {
    extern __shared__ uint32_t sh[];   // max(n2, 2 * slots + kDsaBuckets + 1) words
    const int g = blockIdx.x;
    const int t0 = g * G, rows = min(G, T - t0), cap = G * k;
    const int32_t* src = idx + (size_t)t0 * k;
    int32_t* out_s = shared + (size_t)g * cap;
    uint32_t* out_m = masks + (size_t)g * cap;
    if (dsa_pack_by_hash(sh, src, rows, k, L, log2_slots, out_s, out_m, cap, lens + g)) return;
    __syncthreads();
    dsa_pack_by_sort(sh, src, rows, k, L, n2, out_s, out_m, cap, lens + g);
}

__global__ __launch_bounds__(256) void dsa_gather_kernel(const uint8_t* kv, int L, size_t row_bytes,
                                                         const int32_t* shared, const int32_t* lens, int cap,
                                                         uint8_t* out) {
    const int g = blockIdx.x;
    const size_t units = row_bytes / 16;
    const size_t total = (size_t)min(max(lens[g], 0), cap) * units;
    for (size_t u = (size_t)blockIdx.y * 256 + threadIdx.x; u < total; u += (size_t)gridDim.y * 256) {
        const size_t j = u / units, c = u % units;
        const int s = shared[(size_t)g * cap + j];
        u32x4 val{0u, 0u, 0u, 0u};
        if (s >= 0 && s < L) val = reinterpret_cast<const u32x4*>(kv + (size_t)s * row_bytes)[c];
        reinterpret_cast<u32x4*>(out + ((size_t)g * cap + j) * row_bytes)[c] = val;
    }
}

hipError_t launch_dsa_pack(const int32_t* idx, int T, int k, int L, int G, int32_t* shared, uint32_t* masks,
                           int32_t* lens, hipStream_t st) {
    const int ng = (T + G - 1) / G;
    int n2 = 1;
    while (n2 < G * k) n2 <<= 1;
    // hash table: twice the selections, at most 16,384 slots
    int lg = 8;
    while ((1 << lg) < 2 * G * k && lg < kDsaLog2SlotsMax) ++lg;
    const size_t lds = (size_t)4 * std::max(n2, 2 * (1 << lg) + kDsaBuckets + 1);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dsa_pack_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    dsa_pack_kernel<<<ng, kDsaThreads, lds, st>>>(idx, T, k, L, G, n2, lg, shared, masks, lens);
    return hipGetLastError();
}

hipError_t launch_dsa_gather(const void* kv, int L, size_t row_bytes, const int32_t* shared, const int32_t* lens,
                             int ngroups, int cap, void* out, hipStream_t st) {
    const size_t per_group = (size_t)cap * (row_bytes / 16);
    const int ny = (int)std::max<size_t>(1, std::min<size_t>(64, per_group / (256 * 8)));
    dsa_gather_kernel<<<dim3(ngroups, ny), 256, 0, st>>>(static_cast<const uint8_t*>(kv), L, row_bytes, shared,
                                                         lens, cap, static_cast<uint8_t*>(out));
    return hipGetLastError();
}

}  // namespace ltk
