// device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// Score contraction on the matrix cores.  Heads sit on the MFMA M dimension
// and keys on N, so the head reduction of the DSA-style indexer score
// I[t,s] = sum_h w[t,h] * max(0, q[t,h].k[s]) stays inside each lane (the
// lane holds 16 heads of one key per 32x32 block), plus one exchange between
// the two 32-lane halves of the wave.  K (= head dimension) is split so that
// every lane reads one contiguous half of its row: the lane of half `h`
// holds elements [h*D/2, (h+1)*D/2) of row (lane & 31), and MFMA step j
// consumes the j-th EPL-element slice of that half for both operands.  The
// same slicing for A and B makes the dot product over D exact whatever the
// instruction's internal order of K, because both operands use it.
//
// All score arithmetic is written once here and shared by the sample pass,
// the fused scan, the overflow fallback and the unfused baseline, so a key
// gets bit-identical fp32 scores in all of them.  The library is compiled
// with -ffp-contract=off so that no pass fuses differently.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ltk {

enum DType { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct DTraits;
template <> struct DTraits<DT_F32> { static constexpr int ESZ = 4, EPL = 1; };    // v_mfma_f32_32x32x2_f32
template <> struct DTraits<DT_BF16> { static constexpr int ESZ = 2, EPL = 8; };   // v_mfma_f32_32x32x16_bf16
template <> struct DTraits<DT_FP8> { static constexpr int ESZ = 1, EPL = 32; };   // v_mfma_f32_32x32x64_f8f6f4

// One lane's share of a 32-row operand block: its contiguous half row.
template <int DT, int D>
struct HalfRow {
    static constexpr int ESZ = DTraits<DT>::ESZ;
    static constexpr int BYTES = D / 2 * ESZ;
    static constexpr int NV = BYTES / 16;
    static constexpr int KSTEPS = (D / 2) / DTraits<DT>::EPL;
    static_assert(BYTES % 16 == 0, "half rows are whole 16-byte vectors");
    u32x4 v[NV];
};

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

template <int DT, int D>
__device__ __forceinline__ void load_half_row(HalfRow<DT, D>& f, const uint8_t* row, int half) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + (size_t)half * HalfRow<DT, D>::BYTES);
#pragma unroll
    for (int i = 0; i < HalfRow<DT, D>::NV; ++i) f.v[i] = p[i];
}

template <int DT, int D>
__device__ __forceinline__ void zero_half_row(HalfRow<DT, D>& f) {
#pragma unroll
    for (int i = 0; i < HalfRow<DT, D>::NV; ++i) f.v[i] = u32x4{0u, 0u, 0u, 0u};
}

// acc += A_slice_j x B_slice_j
template <int DT, int D>
__device__ __forceinline__ void mfma_step(const HalfRow<DT, D>& a, const HalfRow<DT, D>& b, int j, v16f& acc) {
    if constexpr (DT == DT_F32) {
        const float av = __uint_as_float(a.v[j >> 2][j & 3]);
        const float bv = __uint_as_float(b.v[j >> 2][j & 3]);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    } else if constexpr (DT == DT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v[j]),
                                                      __builtin_bit_cast(bf16x8, b.v[j]), acc, 0, 0, 0);
    } else {
        const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(a.v[2 * j], a.v[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        const i32x8 bv = __builtin_bit_cast(i32x8, __builtin_shufflevector(b.v[2 * j], b.v[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        // format 0 = e4m3 for both operands; zero scales select the unscaled instruction
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
    }
}

// Two independent slots (query a x key block A, query b x key block B),
// HB head blocks each; the four MFMA chains are interleaved.
template <int DT, int D, int HB>
__device__ __forceinline__ void mfma_2slots(const HalfRow<DT, D> (&qa)[HB], const HalfRow<DT, D>& ka,
                                            const HalfRow<DT, D> (&qb)[HB], const HalfRow<DT, D>& kb,
                                            v16f (&acca)[HB], v16f (&accb)[HB]) {
#pragma unroll
    for (int m = 0; m < HB; ++m) {
        acca[m] = v16f{};
        accb[m] = v16f{};
    }
#pragma unroll
    for (int j = 0; j < HalfRow<DT, D>::KSTEPS; ++j) {
#pragma unroll
        for (int m = 0; m < HB; ++m) {
            mfma_step<DT, D>(qa[m], ka, j, acca[m]);
            mfma_step<DT, D>(qb[m], kb, j, accb[m]);
        }
    }
}

// One slot: query block q x one 32-key block (HB independent chains).
template <int DT, int D, int HB>
__device__ __forceinline__ void mfma_1slot(const HalfRow<DT, D> (&q)[HB], const HalfRow<DT, D>& kf, v16f (&acc)[HB]) {
#pragma unroll
    for (int m = 0; m < HB; ++m) acc[m] = v16f{};
#pragma unroll
    for (int j = 0; j < HalfRow<DT, D>::KSTEPS; ++j)
#pragma unroll
        for (int m = 0; m < HB; ++m) mfma_step<DT, D>(q[m], kf, j, acc[m]);
}

// Head of accumulator register r of a lane in half `half`, head block m:
// the 32x32 MFMA result row held by (lane, r) is 8*(r/4) + 4*half + (r%4).
__device__ __forceinline__ int head_of(int m, int r, int half) { return m * 32 + 8 * (r >> 2) + 4 * half + (r & 3); }

// max(0, x) of a finite float as one integer max on its bits: the bit
// pattern of a float read as int32 is negative exactly when the sign bit is
// set, so negative values and -0 become +0 and the rest pass unchanged.  (A
// float max would first quiet NaNs: two instructions per head instead of one.)
__device__ __forceinline__ float relu_bits(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// sum over the lane's heads of w * max(0, x), in a fixed order
template <int HB>
__device__ __forceinline__ float relu_wsum(const v16f (&acc)[HB], const float (&w)[HB][16]) {
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < HB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) p = __builtin_fmaf(w[m][r], relu_bits(acc[m][r]), p);
    return p;
}

// fp8 form of the head sum.  With w' the head weights,
//   sum_h w'_h max(0, x_h) = 1/2 sum_h w'_h x_h + 1/2 sum_h w'_h |x_h|
// for weights of either sign.  The second sum is one FMA per head (|x| is a
// free source modifier); the first is linear in the query, sum_h w'_h x_h =
// q''.k with q'' = sum_h w'_h q_h, and goes to the matrix cores (lin_* below).
// Here w holds w'/2, so this returns the lane's share of 1/2 sum w'|x|.
template <int HB>
__device__ __forceinline__ float abs_wsum(const v16f (&acc)[HB], const float (&w)[HB][16]) {
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < HB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) p = __builtin_fmaf(w[m][r], __builtin_fabsf(acc[m][r]), p);
    return p;
}

// The linear term on the matrix cores.  q''/2 of a query is held as four
// fp8 parts P_0..P_3 with q''/2 * S ~= P_0 + P_1/16 + P_2/256 + P_3/4096
// (S a power of two per query; each part carries the rounding residue of the
// ones before, scaled up by 16, so the four parts hold about 16 significant
// bits).  One v_mfma_f32_16x16x128_f8f6f4 scores 16 keys against 16 rows:
// four queries x four parts, row 4g + p = part p of query g.  Lane l holds
// row / key (l & 15), dimensions [32 (l >> 4), 32 (l >> 4) + 32) of both
// operands, and gets rows 4 (l >> 4) .. 4 (l >> 4) + 3 of key (l & 15): the
// four part products of one query and one key.
struct LinFrag {
    u32x4 v[2];   // 32 fp8 values of one row (or key) of the operand
};

__device__ __forceinline__ v4f lin_mfma(const LinFrag& a, const LinFrag& b) {
    const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(a.v[0], a.v[1], 0, 1, 2, 3, 4, 5, 6, 7));
    const i32x8 bv = __builtin_bit_cast(i32x8, __builtin_shufflevector(b.v[0], b.v[1], 0, 1, 2, 3, 4, 5, 6, 7));
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
}

// (q''/2 . k) * S from the four part products, in one fixed order.
__device__ __forceinline__ float lin_combine(const v4f& c) {
    float t = __builtin_fmaf(c[3], 0.0625f, c[2]);
    t = __builtin_fmaf(t, 0.0625f, c[1]);
    return __builtin_fmaf(t, 0.0625f, c[0]);
}

// fp8 score of one key: sigma_k * (1/2 q''.k + 1/2 sum w'|x|), the linear
// term t scaled back by 1/S.
__device__ __forceinline__ float lin_score(float t, float inv_s, float abs_half, float sk) {
    return __builtin_fmaf(t, inv_s, abs_half) * sk;
}

// Partial head sums of two slots -> lanes 0-31 get slot a's full sum for key
// (lane & 31), lanes 32-63 slot b's.  Both halves add (low heads + high heads).
__device__ __forceinline__ float combine_halves(float pa, float pb) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Affine bin map of the pages ("Filtering"): B = (I - s_min) * delta, clamped
// into [0, nbins-1] and floored.  Monotone non-decreasing in I.
__device__ __forceinline__ int bin_of(float I, float smin, float delta, int nbins) {
    float B = (I - smin) * delta;
    B = __builtin_fminf(__builtin_fmaxf(B, 0.0f), (float)(nbins - 1));
    return (int)B;
}

// Order-preserving map of a finite float to uint32 (-0 is folded onto +0).
__device__ __forceinline__ uint32_t ord_f32(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// 64-bit ranking key: score descending, then index ascending.
__device__ __forceinline__ uint64_t rank_key(float I, int idx) {
    return ((uint64_t)ord_f32(I) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

__device__ __forceinline__ int mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Cross-lane steps on the DPP network: row shifts inside 16-lane rows, then
// the row broadcasts of lane 15 and lane 31.  Each step costs a few cycles,
// where a shuffle (ds_bpermute) waits on the LDS crossbar.  Inclusive scans
// over the wave's 64 lanes (lane i gets op over lanes 0..i); every lane of
// the wave must be active.
template <int CTRL, int ROWM = 0xf, int BANKM = 0xf>
__device__ __forceinline__ int dpp_i32(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWM, BANKM, false);   // masked or outside lanes: old
}
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v, uint32_t ident, Op op) {
    const int id = (int)ident;
    v = op(v, (uint32_t)dpp_i32<0x111>(id, (int)v));         // row_shr:1
    v = op(v, (uint32_t)dpp_i32<0x112>(id, (int)v));         // row_shr:2
    v = op(v, (uint32_t)dpp_i32<0x114>(id, (int)v));         // row_shr:4
    v = op(v, (uint32_t)dpp_i32<0x118>(id, (int)v));         // row_shr:8
    v = op(v, (uint32_t)dpp_i32<0x142, 0xa>(id, (int)v));    // row_bcast:15 into rows 1, 3
    v = op(v, (uint32_t)dpp_i32<0x143, 0xc>(id, (int)v));    // row_bcast:31 into rows 2, 3
    return v;
}
__device__ __forceinline__ uint32_t wave_scan_add_u32(uint32_t v) {
    return wave_scan_u32(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}
__device__ __forceinline__ uint32_t lane63_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return lane63_u32(wave_scan_add_u32(v)); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return lane63_u32(wave_scan_u32(v, 0xffffffffu, [](uint32_t x, uint32_t y) { return x < y ? x : y; }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return lane63_u32(wave_scan_u32(v, 0u, [](uint32_t x, uint32_t y) { return x > y ? x : y; }));
}
__device__ __forceinline__ int wave_max_i32(int v) {
    return (int)lane63_u32(wave_scan_u32((uint32_t)v, 0x80000000u,
                                         [](uint32_t x, uint32_t y) { return (uint32_t)max((int)x, (int)y); }));
}
__device__ __forceinline__ float wave_min_f32(float v) {
    return __uint_as_float(lane63_u32(wave_scan_u32(__float_as_uint(v), __float_as_uint(INFINITY), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
    })));
}
__device__ __forceinline__ float wave_max_f32(float v) {
    return __uint_as_float(lane63_u32(wave_scan_u32(__float_as_uint(v), __float_as_uint(-INFINITY), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    })));
}
// lane 0's value in every lane (lane 0 active)
__device__ __forceinline__ uint32_t lane0_u32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

// Top-down accumulation of a histogram (one wave, all 64 lanes): the largest
// bin b with sum_{b' >= b} h[b'] >= k, and sum_{b' > b} h[b'].  Returns b = -1
// (above = total) when the total is below k.  Used for the initial threshold
// bin, the threshold refresh, the final threshold bin and radix digits.
struct SuffixPick { int bin; uint32_t above; };

__device__ __forceinline__ SuffixPick suffix_pick(const uint32_t* h, int nbins, uint32_t k) {
    const int lane = lane_id();
    const int per = (nbins + 63) >> 6;
    const int lo = lane * per;
    uint32_t local = 0;
    for (int i = 0; i < per; ++i)
        if (lo + i < nbins) local += h[lo + i];
    // entries in the bins of higher lanes: the total less the inclusive prefix
    const uint32_t pre = wave_scan_add_u32(local), total = lane63_u32(pre);
    uint32_t c = total - pre;
    int best = -1;
    uint32_t best_above = 0;
    for (int i = per - 1; i >= 0; --i) {
        const int b = lo + i;
        if (b < nbins) {
            const uint32_t hb = h[b];
            if (best < 0 && c + hb >= k) {
                best = b;
                best_above = c;
            }
            c += hb;
        }
    }
    const int bmax = wave_max_i32(best);
    // bins are split across lanes, so exactly one lane owns bmax
    uint32_t ab = wave_sum_u32((bmax >= 0 && best == bmax) ? best_above : 0u);
    if (bmax < 0) ab = total;
    return SuffixPick{bmax, ab};
}

// Per-query summary of the sample pass.
struct Meta {
    float smin;   // lower end of the sample's score range
    float delta;  // bins per unit score
    int thr0;     // initial threshold bin
    int nvalid;   // valid sample keys of this query
};

}  // namespace ltk
