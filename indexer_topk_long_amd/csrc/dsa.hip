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
//  2. the distinct keys are compacted and sorted ascending (bitonic, in LDS);
//  3. each sorted key's mask is looked up in the table, and the list and
//     masks are written out in order.
// A group whose distinct keys would crowd the table (more than 3/4 of its
// slots) is packed by sorting all of its G*k selections instead, each tagged
// with its row as key << 5 | row: equal keys are then adjacent, each run of
// one key becomes one list entry, and its mask is the OR of the run's row
// bits.
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

// Ascending bitonic sort of n (a power of two) values in LDS.
__device__ inline void dsa_sort(uint32_t* v, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n / 2; i += kDsaThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint32_t x = v[lo], y = v[hi];
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
    uint32_t incl = heads;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
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

constexpr int kDsaProbeMax = 256;   // linear-probing steps before the group takes the sort path

__device__ __forceinline__ uint32_t dsa_slot(uint32_t key, int log2_slots) {
    return (key * 2654435761u) >> (32 - log2_slots);
}

// Hash path (sh: 2 * slots + sort_n words of LDS).  Returns false, having
// written nothing, when the group's distinct keys exceed 3/4 of the slots.
__device__ bool dsa_pack_by_hash(uint32_t* sh, const int32_t* src, int rows, int k, int L, int log2_slots,
                                 int sort_n, int32_t* out_s, uint32_t* out_m, int cap, int32_t* len) {
    __shared__ uint32_t s_n, s_over, s_c;
    const int tid = threadIdx.x, lane = lane_id();
    const int slots = 1 << log2_slots;
    const uint32_t limit = (uint32_t)min(sort_n, slots * 3 / 4);
    uint32_t* tk = sh;               // keys
    uint32_t* tm = sh + slots;       // masks
    uint32_t* sb = sh + 2 * slots;   // the distinct keys, then sorted
    for (int i = tid; i < slots; i += kDsaThreads) {
        tk[i] = kDsaEmpty;
        tm[i] = 0u;
    }
    if (tid == 0) {
        s_n = 0u;
        s_over = 0u;
        s_c = 0u;
    }
    __syncthreads();
    for (int p0 = 0; p0 < rows * k; p0 += kDsaThreads) {
        const int p = p0 + tid;
        bool fresh = false;
        if (p < rows * k && s_over == 0u) {
            const int s = src[p];
            if (s >= 0 && s < L) {
                const uint32_t key = (uint32_t)s, bit = 1u << (uint32_t)(p / k);
                uint32_t h = dsa_slot(key, log2_slots);
                for (int probe = 0;; ++probe) {
                    if (probe == kDsaProbeMax) {
                        s_over = 1u;
                        break;
                    }
                    const uint32_t old = atomicCAS(&tk[h], kDsaEmpty, key);
                    if (old == kDsaEmpty || old == key) {
                        atomicOr(&tm[h], bit);
                        fresh = old == kDsaEmpty;
                        break;
                    }
                    h = (h + 1u) & (uint32_t)(slots - 1);
                }
            }
        }
        const uint64_t f = __ballot(fresh);
        if (lane == 0 && f) {
            if (atomicAdd(&s_n, (uint32_t)__popcll(f)) + (uint32_t)__popcll(f) > limit) s_over = 1u;
        }
        __syncthreads();   // s_over seen by every wave before the next round
    }
    const uint32_t n = s_n;
    if (s_over != 0u) return false;
    // compact the distinct keys (any order), pad, sort
    for (int i0 = 0; i0 < slots; i0 += kDsaThreads) {
        const int i = i0 + tid;
        const uint32_t key = (i < slots) ? tk[i] : kDsaEmpty;
        const uint64_t m = __ballot(key != kDsaEmpty);
        uint32_t base = 0u;
        if (lane == 0 && m) base = atomicAdd(&s_c, (uint32_t)__popcll(m));
        base = __shfl(base, 0);
        if (key != kDsaEmpty) sb[base + mbcnt(m)] = key;
    }
    __syncthreads();
    int n2 = 1;
    while (n2 < (int)n) n2 <<= 1;
    for (int i = (int)n + tid; i < n2; i += kDsaThreads) sb[i] = kDsaEmpty;
    __syncthreads();
    dsa_sort(sb, n2);
    for (int j = tid; j < (int)n; j += kDsaThreads) {
        const uint32_t key = sb[j];
        uint32_t h = dsa_slot(key, log2_slots);
        while (tk[h] != key) h = (h + 1u) & (uint32_t)(slots - 1);   // present: inserted above
        out_s[j] = (int32_t)key;
        out_m[j] = tm[h];
    }
    for (int j = (int)n + tid; j < cap; j += kDsaThreads) {
        out_s[j] = -1;
        out_m[j] = 0u;
    }
    if (tid == 0) *len = (int32_t)n;
    return true;
}

__global__ __launch_bounds__(kDsaThreads) void dsa_pack_kernel(const int32_t* idx, int T, int k, int L, int G,
                                                               int n2, int log2_slots, int sort_n,
                                                               int32_t* shared, uint32_t* masks, int32_t* lens) {
    extern __shared__ uint32_t sh[];   // max(n2, 2 * slots + sort_n) words
    const int g = blockIdx.x;
    const int t0 = g * G, rows = min(G, T - t0), cap = G * k;
    const int32_t* src = idx + (size_t)t0 * k;
    int32_t* out_s = shared + (size_t)g * cap;
    uint32_t* out_m = masks + (size_t)g * cap;
    if (dsa_pack_by_hash(sh, src, rows, k, L, log2_slots, sort_n, out_s, out_m, cap, lens + g)) return;
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
    // hash table: twice the selections, at most 8,192 slots; the sort buffer
    // holds every distinct key the table may accept (3/4 of its slots)
    int lg = 8;
    while ((1 << lg) < 2 * G * k && lg < 13) ++lg;
    int sort_n = 1;
    while (sort_n < std::min(G * k, (1 << lg) * 3 / 4)) sort_n <<= 1;
    const size_t lds = (size_t)4 * std::max(n2, 2 * (1 << lg) + sort_n);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dsa_pack_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    dsa_pack_kernel<<<ng, kDsaThreads, lds, st>>>(idx, T, k, L, G, n2, lg, sort_n, shared, masks, lens);
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
