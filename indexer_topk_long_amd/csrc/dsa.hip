// dsa.hip -- LiteDSA packing for gfx950.
//
// LiteTopK pages, arXiv abstract: LiteDSA packs the candidates that
// neighbouring query tokens have in common into one shared key/value list for
// joint attention, and per-query masks keep each token's own top-k membership.
//
// Pack: one workgroup of 1024 threads per group of G consecutive query rows.
// The group's G*k selections, each tagged with its row as key << 5 | row, are
// sorted in LDS by a bitonic network, padded to a power of two with an
// all-ones value that sorts last.  Equal keys are then adjacent, so each run
// of one key becomes one entry of the shared list (ascending), and its mask
// is the OR of the run's row bits.  Output positions come from a block-wide
// prefix count of the run heads.
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

__global__ __launch_bounds__(kDsaThreads) void dsa_pack_kernel(const int32_t* idx, int T, int k, int L, int G,
                                                               int n2, int32_t* shared, uint32_t* masks,
                                                               int32_t* lens) {
    extern __shared__ uint32_t v[];   // [n2]
    __shared__ uint32_t s_wsum[kDsaThreads / 64];
    const int g = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int t0 = g * G, rows = min(G, T - t0), cap = G * k;
    const int32_t* src = idx + (size_t)t0 * k;
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
    int32_t* out_s = shared + (size_t)g * cap;
    uint32_t* out_m = masks + (size_t)g * cap;
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
    if (tid == 0) lens[g] = (int32_t)total;
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
    const size_t lds = (size_t)n2 * 4;
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dsa_pack_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    dsa_pack_kernel<<<ng, kDsaThreads, lds, st>>>(idx, T, k, L, G, n2, shared, masks, lens);
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
