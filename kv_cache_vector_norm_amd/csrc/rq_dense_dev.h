// Building blocks of the TurboQuant comparison path and of the PolarQuant
// rotation (gfx950): the dense session's device tables, the exact half-pair
// split of a rotation operand, and the slot-table quantiser in the
// rotation's accumulator scale (hyper.ai summary, Algorithms 1 and 2; README
// "How TurboQuant Works").
//
// Pi is held as an exact pair of halves, 16 Pi = P_hi + 2^-11 P_lo, and so is
// the other operand, 16 v = v_hi + 2^-11 v_lo; the three products that
// matter are folded into one fp32 accumulator by scaling v_hi by 2^11:
//   P_hi (2^11 v_hi) + P_hi v_lo + P_lo v_hi = 2^11 * 256 * (Pi v) + O(2^-22).
// Codes come from the rotor path's exact 256-slot quantiser with its
// thresholds scaled by 2^19, so the unscaled accumulators are compared
// directly.  The codec kernels are in rq_dense_codec_dev.h.
#pragma once

#include "rq_common_dev.h"
#include "rq_kernels.h"

namespace rqk {

struct DenseDev {
    const uint16_t* __restrict__ pi_hi;
    const uint16_t* __restrict__ pi_lo;
    const uint16_t* __restrict__ pit_hi;
    const uint16_t* __restrict__ pit_lo;
    const uint16_t* __restrict__ pi2_hi;
    const uint16_t* __restrict__ pi2_lo;
    const uint16_t* __restrict__ pit2_hi;
    const uint16_t* __restrict__ pit2_lo;
    const uint16_t* __restrict__ t2_hi;
    const uint16_t* __restrict__ t2_lo;
    const uint16_t* __restrict__ s_back;
    const float* __restrict__ thr;
    const float* __restrict__ cent;
    const uint16_t* __restrict__ s_rows;
    const uint16_t* __restrict__ s_cols;
    const u32x4_t* __restrict__ bins;
    float bin_a, bin_b;
    float qjl_scale;
};

constexpr float kRotScale = 1.0f / (2048.0f * 256.0f);   // undoes 2^11 * 16 * 16
constexpr float kDenseResidualScale = 4096.0f;

// fragment of a row-major 128 x 128 half matrix in global memory
__device__ __forceinline__ u32x4 gmat_frag(const uint16_t* __restrict__ m, int row, int chunk) {
    return *reinterpret_cast<const u32x4*>(m + row * 128 + chunk * 8);
}

// 16 v as halves: hi = half(16 v), lo = half((16 v - hi) 2^11), and 2^11 hi
// (the difference 16 v - hi is exact in fp32; scaling by 2^11 is exact).
__device__ __forceinline__ void split16(float v, uint32_t* h11, uint32_t* h, uint32_t* l) {
    const uint32_t hi = f2h(v * 16.0f);
    const float hf = h2f(hi);
    *h = hi;
    *l = f2h((v * 16.0f - hf) * 2048.0f);
    *h11 = f2h(hf * 2048.0f);
}

// acc[nt] += rotation of this lane's own 128-vector held as split pairs,
// for the 32 output rows of M tile MT; A fragments from `fa_hi`, `fa_lo`.
template <int MT, class FragHi, class FragLo>
__device__ __forceinline__ void rot_mfma(const uint32_t (&vh11)[64], const uint32_t (&vh)[64],
                                         const uint32_t (&vl)[64], FragHi fa_hi, FragLo fa_lo, int l,
                                         float (&own0)[16], float (&own1)[16]) {
    f32x16 a0 = {}, a1 = {};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int row = 32 * MT + (l & 31), chunk = 2 * kb + (l >> 5);
        const u32x4 ph = fa_hi(row, chunk);
        const u32x4 pl = fa_lo(row, chunk);
        u32x4 b11_0, b11_1, bh_0, bh_1, bl_0, bl_1;
        to_operands(u32x4{vh11[8 * kb], vh11[8 * kb + 1], vh11[8 * kb + 2], vh11[8 * kb + 3]},
                    u32x4{vh11[8 * kb + 4], vh11[8 * kb + 5], vh11[8 * kb + 6], vh11[8 * kb + 7]}, &b11_0, &b11_1);
        to_operands(u32x4{vh[8 * kb], vh[8 * kb + 1], vh[8 * kb + 2], vh[8 * kb + 3]},
                    u32x4{vh[8 * kb + 4], vh[8 * kb + 5], vh[8 * kb + 6], vh[8 * kb + 7]}, &bh_0, &bh_1);
        to_operands(u32x4{vl[8 * kb], vl[8 * kb + 1], vl[8 * kb + 2], vl[8 * kb + 3]},
                    u32x4{vl[8 * kb + 4], vl[8 * kb + 5], vl[8 * kb + 6], vl[8 * kb + 7]}, &bl_0, &bl_1);
        a0 = mfma(ph, b11_0, a0);
        a0 = mfma(ph, bl_0, a0);
        a0 = mfma(pl, bh_0, a0);
        a1 = mfma(ph, b11_1, a1);
        a1 = mfma(ph, bl_1, a1);
        a1 = mfma(pl, bh_1, a1);
    }
    from_accumulators(a0, a1, own0, own1);
}

__device__ __forceinline__ void put_pair(uint32_t (&arr)[64], int i, uint32_t h) {
    if (i & 1) arr[i >> 1] |= h << 16; else arr[i >> 1] = h;
}

// ------------------------------------------------------------ kernels --
// The slot table with thresholds and centroids in the rotation's
// accumulator scale (unit domain times 2^19 = 1 / kRotScale, exact).
__device__ __forceinline__ void dense_bins_to_lds(const DenseDev& P, u32x4* __restrict__ s) {
    const u32x4* src = reinterpret_cast<const u32x4*>(P.bins);
    for (int i = threadIdx.x; i < kBinSlots; i += blockDim.x) {
        const u32x4 e = src[i];
        const uint32_t e0 = e[0], e1 = e[1], e2 = e[2], e3 = e[3];
        constexpr float up = 1.0f / kRotScale;
        s[i] = u32x4{e0, __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, e1) * up),
                     __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, e2) * up),
                     __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, e3) * up)};
    }
}

// #{k : y > t_k} of y = acc * kRotScale through the slot table: the slot of
// fma(acc, bin_a * kRotScale, bin_b) equals that of fma(y, bin_a, bin_b)
// (power-of-two scalings are exact), and acc > 2^19 t equals y > t.  The
// table's elements go through scalars: hipcc turns a bit cast of an
// ext-vector element straight into one of element 0.
// In two steps, so that table reads can be issued ahead of their use: the
// byte offset of y's slot entry, then the code (and the centroid times
// 2^19, when the entry's c_lo, c_hi were read) from the entry.
__device__ __forceinline__ uint32_t dense_slot(float acc, float ba, float bb) {
    return __builtin_bit_cast(uint32_t, __builtin_fmaf(acc, ba, bb)) & 0xFF0u;
}
__device__ __forceinline__ uint32_t dense_decide(float acc, const u32x4& e, float* cv) {
    const uint32_t base = e[0], thr = e[1], c_lo = e[2], c_hi = e[3];
    const bool up = acc > __builtin_bit_cast(float, thr);
    *cv = __builtin_bit_cast(float, up ? c_hi : c_lo);
    return base + (up ? 1u : 0u);
}

// Centroid pair table: for codes (a, b), ptab[a + L b] = {hi[a] | hi[b] << 16,
// lo[a] | lo[b] << 16} with 16 c_k = hi[k] + 2^-11 lo[k]: one 8-byte read
// gives two slots' hi and lo operand halves.
template <int B>
__device__ __forceinline__ void dense_tables_to_lds(const DenseDev& P, uint2* ptab) {
    constexpr int L = 1 << B;
    for (int p = threadIdx.x; p < L * L; p += blockDim.x) {
        uint32_t h11a, ha, la, h11b, hb, lb;
        split16(P.cent[p & (L - 1)], &h11a, &ha, &la);
        split16(P.cent[p >> B], &h11b, &hb, &lb);
        ptab[p] = make_uint2(ha | (hb << 16), la | (lb << 16));
    }
}

}  // namespace rqk
