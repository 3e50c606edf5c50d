// peak.hip -- achievable-peak microbenchmarks of one MI355X (gfx950), the
// measured denominators beside the vendor figures in the roofline.
//
//   ltkpeak_mfma(kind, valu_per_mfma, iters, ...)  fp8 or bf16 32x32 MFMAs,
//       eight independent accumulator chains per wave, two waves per SIMD on
//       every CU (the fused scan's occupancy), optionally with fp32 FMAs
//       (with an |x| source modifier, as in the scan's head sum) issued
//       behind each MFMA;
//   ltkpeak_read(...)  a streaming read of a device buffer (16 bytes per
//       lane per load, summed so that nothing is optimised away).
//
// Built into its own library (liblitkpeak.so); the fused Indexer-TopK
// library does not contain or call it.  C ABI: plain pointers and sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;   // independent accumulators per wave

// One MFMA per chain per step; VPM fp32 FMAs on a chain's accumulator
// registers are issued behind each MFMA (reading the previous step's result).
template <int KIND, int VPM>
__global__ __launch_bounds__(512) void mfma_loop(int iters, const uint32_t* seed, float* sink) {
    const int lane = threadIdx.x & 63;
    const uint32_t s = seed[lane];
    i32x8 a8, b8;
    u32x4 a4, b4;
    for (int i = 0; i < 8; ++i) {
        a8[i] = (int)(s * 2654435761u + i) & 0x3b3b3b3b;   // small finite fp8 values
        b8[i] = (int)(s * 40503u + 7 * i) & 0x3b3b3b3b;
    }
    for (int i = 0; i < 4; ++i) {
        a4[i] = (s * 2654435761u + i) & 0x3f803f80u;       // bf16 values near 1
        b4[i] = (s * 40503u + 7 * i) & 0x3f803f80u;
    }
    v16f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
    float p = 0.0f;
    const float w = __uint_as_float(0x3c000000u | (s & 0xff));
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (KIND == 0)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 0, 0, 0, 0, 0, 0);
            else
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                                 __builtin_bit_cast(bf16x8, b4), acc[c], 0, 0, 0);
            // read a chain finished a full round earlier
            const v16f& r = acc[(c + 1) % kChains];
#pragma unroll
            for (int v = 0; v < VPM; ++v) p = __builtin_fmaf(w, __builtin_fabsf(r[v & 15]), p);
        }
    }
    float t = p;
#pragma unroll
    for (int c = 0; c < kChains; ++c) t += acc[c][lane & 15];
    if (t == 1.2345f) sink[blockIdx.x] = t;   // keeps the work; never true for these inputs
}

__global__ __launch_bounds__(256) void read_loop(const u32x4* src, size_t n16, uint32_t* sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] + v[1] + v[2] + v[3];
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

template <int KIND>
hipError_t launch_mfma(int vpm, int blocks, int iters, const uint32_t* seed, float* sink, hipStream_t st) {
    switch (vpm) {
        case 0: mfma_loop<KIND, 0><<<blocks, 512, 0, st>>>(iters, seed, sink); break;
        case 4: mfma_loop<KIND, 4><<<blocks, 512, 0, st>>>(iters, seed, sink); break;
        case 8: mfma_loop<KIND, 8><<<blocks, 512, 0, st>>>(iters, seed, sink); break;
        case 16: mfma_loop<KIND, 16><<<blocks, 512, 0, st>>>(iters, seed, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

// MFMA loop: kind 0 = fp8 v_mfma_f32_32x32x64_f8f6f4 (131,072 flop each),
// kind 1 = bf16 v_mfma_f32_32x32x16_bf16 (32,768 flop each); valu_per_mfma in
// {0, 4, 8, 16}; `blocks` workgroups of 8 waves, each wave running iters x 8
// MFMAs.  seed: 64 device uint32; sink: `blocks` device floats (never
// written for the built-in inputs).  Returns 0, or -1 for bad arguments, -4
// for a launch error.  Flop of one call: blocks x 8 x iters x 8 x (flop per MFMA).
int ltkpeak_mfma(int kind, int valu_per_mfma, int blocks, int iters, const uint32_t* seed, float* sink,
                 void* stream) {
    if (blocks < 1 || iters < 1 || !seed || !sink || (kind != 0 && kind != 1)) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = kind == 0 ? launch_mfma<0>(valu_per_mfma, blocks, iters, seed, sink, st)
                                   : launch_mfma<1>(valu_per_mfma, blocks, iters, seed, sink, st);
    return e == hipSuccess ? 0 : (e == hipErrorInvalidValue ? -1 : -4);
}

// Streaming read of `bytes` (a multiple of 16) from the 16-byte-aligned
// device buffer src by `blocks` workgroups of 256 threads; sink: `blocks`
// device uint32.  Returns 0, -1 for bad arguments, -4 for a launch error.
int ltkpeak_read(const void* src, size_t bytes, int blocks, uint32_t* sink, void* stream) {
    if (!src || !sink || blocks < 1 || bytes % 16 != 0 || ((uintptr_t)src & 15u)) return -1;
    read_loop<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
