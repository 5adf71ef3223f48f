// TurboQuant comparison path for gfx950, two lanes per vector (templates;
// instantiated per bit width and mode in rq_dense_inst.hip): y = Pi x_u with
// a dense 128 x 128 random orthogonal Pi, per-coordinate Lloyd-Max codes,
// x~ = Pi^T y^, optionally with the QJL residual stage (hyper.ai summary,
// Algorithms 1 and 2; README "How TurboQuant Works").
//
// Mapping.  A wave owns a tile of 32 vectors; lanes v and v + 32 share vector
// v, lane half h holding coordinates 64 h .. 64 h + 63 (its 64 slots).  Every
// contraction is a 32x32x16 MFMA over the tile (N = the 32 vectors) whose
// two 8-element K halves are the two lane halves: K block kb is slots
// 8 kb .. 8 kb + 7 of both halves.  Pi, Pi^T, S and S^T are permuted on the
// host so that accumulator element r of M tile mt in half h is slot
// 16 mt + r of that half, so operands and results never leave their lane
// (the one-lane design moved every operand and result across lanes).  The
// record's 4 B code words split evenly too: half h packs its 64 codes into
// record words 2 B h .. 2 B h + 2 B - 1.
//
// Precision (as the one-lane design): 16 Pi = P_hi + 2^-11 P_lo and
// 16 v = v_hi + 2^-11 v_lo as exact half pairs, three products folded into
// one fp32 accumulator, P_hi (2^11 v_hi) + P_hi v_lo + P_lo v_hi =
// 2^19 (Pi v) + O(2^-22); codes from the rotor path's exact slot table with
// thresholds scaled by 2^19; the residual r enters S r as an exact hi + lo
// pair (S is exactly half).  Pi sits in LDS (the quantize side); Pi^T, S and
// S^T are read from L2.
#pragma once

#include "rq_dense_dev.h"
#include "rq_rotor_dev.h"
#include "rq_tile2_dev.h"

namespace rqk {

constexpr int kDenseSlots = 64;

template <bool F16>
constexpr int dense_half_bytes() { return F16 ? 128 : 256; }

// The lane's 64 input slots.
template <bool IN_F16>
struct DSlots;

template <>
struct DSlots<true> {
    uint32_t w[kDenseSlots / 2];
    __device__ void read(const char* tile, int vi, int h) {
        const u32x4* p = reinterpret_cast<const u32x4*>(tile + vi * row_bytes2<true>() + dense_half_bytes<true>() * h);
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4 q = p[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = q[e];
                w[4 * c + e] = x;
            }
        }
        wave_lds_sync();
    }
    __device__ float get(int j) const { return h2f((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu)); }
};

template <>
struct DSlots<false> {
    float v[kDenseSlots];
    __device__ void read(const char* tile, int vi, int h) {
        const u32x4* p = reinterpret_cast<const u32x4*>(tile + vi * row_bytes2<false>() + dense_half_bytes<false>() * h);
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const u32x4 q = p[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = q[e];
                v[4 * c + e] = __builtin_bit_cast(float, x);
            }
        }
        wave_lds_sync();
    }
    __device__ float get(int j) const { return v[j]; }
};

// Operands of K block kb from the 8 split slots (half pairs): 2^11 hi, lo, hi.
struct Split8 {
    u32x4 h11, lo, hi;
};

// acc[mt] += the product of the permuted matrix (A fragments fa_hi, fa_lo)
// with the three split operands of K block kb, for all four M tiles.
template <class FragHi, class FragLo>
__device__ __forceinline__ void dense_kblock(f32x16 (&acc)[4], const Split8& s, int kb, FragHi fa_hi, FragLo fa_lo,
                                             int l, int h) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int row = 32 * mt + (l & 31), chunk = 2 * kb + h;
        const u32x4 ph = fa_hi(row, chunk);
        const u32x4 pl = fa_lo(row, chunk);
        acc[mt] = mfma(ph, s.h11, acc[mt]);
        acc[mt] = mfma(ph, s.lo, acc[mt]);
        acc[mt] = mfma(pl, s.hi, acc[mt]);
    }
}

// x~ = Pi^T y^ of the lane's 64 slots (accumulator scale 2^19), y^ the
// centroids of the lane's codes; the same sequence in the quantiser's
// roundtrip and in the dequantiser.
template <int B>
__device__ __forceinline__ void dense_pit2(const DenseDev& P, const uint32_t* __restrict__ ctab,
                                           const uint32_t (&cw)[2 * B], f32x16 (&ax)[4], int l, int h) {
    constexpr int L = 1 << B;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ax[mt] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        Split8 s;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t c0 = get_code<B, 2 * B>(cw, 8 * kb + 2 * q);
            const uint32_t c1 = get_code<B, 2 * B>(cw, 8 * kb + 2 * q + 1);
            const uint32_t e0 = ctab[c0], e1 = ctab[c1];        // lo 16 bits: hi half, hi 16 bits: 2^11 hi
            const uint32_t o0 = ctab[L + c0], o1 = ctab[L + c1];  // lo half
            s.hi[q] = (e0 & 0xFFFFu) | (e1 << 16);
            s.h11[q] = (e0 >> 16) | (e1 & 0xFFFF0000u);
            s.lo[q] = o0 | (o1 << 16);
        }
        dense_kblock(
            ax, s, kb, [&](int row, int chunk) { return gmat_frag(P.pit2_hi, row, chunk); },
            [&](int row, int chunk) { return gmat_frag(P.pit2_lo, row, chunk); }, l, h);
    }
}

// S^T sigma of the lane's slots from its two sign words (sign indices
// 64 h .. 64 h + 63); the same sequence in the roundtrip and the dequantiser.
__device__ __forceinline__ void dense_back2(const DenseDev& P, uint32_t sw0, uint32_t sw1, f32x16 (&acc)[4], int l,
                                            int h) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
    // K blocks in order, their +-1 operands formed two at a time
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
        u32x4 sig[2];
        const uint32_t w = kp < 2 ? sw0 : sw1;
        sigma16((w >> (16 * (kp & 1))) & 0xFFFFu, sig[0], sig[1]);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = mfma(gmat_frag(P.s_back, 32 * mt + (l & 31), 2 * (2 * kp + c) + h), sig[c], acc[mt]);
    }
}

// Output slots of the lane: n^ x~ (MSE) or n^ (x~ + k (S^T sigma)) (QJL),
// x~ = ax * kRotScale, as pairs into the lane's part of its LDS row.
template <bool QJL, bool OUT_F16>
__device__ __forceinline__ void dense_out2(const f32x16 (&ax)[4], const f32x16 (&aq)[4], float k, float nhat,
                                           char* rowo) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float xv[16], qv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = ax[mt][r];
            xv[r] = e * kRotScale;
            if constexpr (QJL) {
                const float f = aq[mt][r];
                qv[r] = f;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float v0 = xv[r], v1 = xv[r + 1];
            if constexpr (QJL) {
                v0 = __builtin_fmaf(k, qv[r], v0);
                v1 = __builtin_fmaf(k, qv[r + 1], v1);
            }
            out_pair<OUT_F16>(rowo, (16 * mt + r) >> 1, nhat * v0, nhat * v1);
        }
    }
}

// ------------------------------------------------------------ kernels --
template <int B, bool QJL, bool IN_F16, bool OUT_F16, bool ROUNDTRIP, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void tq_quant_kernel(DenseDev P, const char* __restrict__ x,
                                                              int64_t ldx_bytes, int64_t n,
                                                              uint32_t* __restrict__ codes,
                                                              uint16_t* __restrict__ norms,
                                                              uint32_t* __restrict__ signs,
                                                              uint16_t* __restrict__ rnorms, char* __restrict__ y,
                                                              int64_t ldy_bytes) {
    constexpr int LW = 2 * B;   // record words of one lane half
    constexpr int W = 4 * B;    // record words per vector
    constexpr int NT = 64 * WAVES;
    constexpr int RBI = row_bytes2<IN_F16>(), RBO = row_bytes2<OUT_F16>();
    constexpr int TB = 32 * (RBI > RBO ? RBI : RBO);
    constexpr int SW = 32 * W > 128 ? 32 * W : 128;
    struct Lds {
        u32x4 bins[kBinSlots];      // slot table (LDS address 0), thresholds and centroids times 2^19
        u32x4 pih[128 * 16];
        u32x4 pil[128 * 16];
        uint32_t ctab[32];
        u32x4 tiles[WAVES][TB / 16];
        uint32_t stage[WAVES][SW];
    };
    __shared__ Lds lds;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (n + 31) / 32;
    const int64_t tstep = static_cast<int64_t>(gridDim.x) * WAVES;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * WAVES + wave;
    Tile2Regs<true> nx;
    if constexpr (IN_F16) {
        if (t0 < ntiles) tile2_fetch<true>(x, ldx_bytes, t0 * 32, n, nx, lane_id());
    }
    dense_tables_to_lds<B>(P, lds.ctab);
    dense_bins_to_lds(P, lds.bins);
    mat_to_lds<NT>(P.pi2_hi, lds.pih);
    mat_to_lds<NT>(P.pi2_lo, lds.pil);
    __syncthreads();
    const float ba = P.bin_a * kRotScale, bb = P.bin_b;
    const char* binc = reinterpret_cast<const char*>(lds.bins);
    char* tile = reinterpret_cast<char*>(lds.tiles[wave]);
    uint32_t* stw = lds.stage[wave];

    for (int64_t t = t0; t < ntiles; t += tstep) {
        const int64_t base = t * 32;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int h = l >> 5, vi = l & 31;
        DSlots<IN_F16> in;
        if constexpr (IN_F16) {
            tile2_put<true>(nx, tile, l);
            in.read(tile, vi, h);
            if (t + tstep < ntiles) tile2_fetch<true>(x, ldx_bytes, (t + tstep) * 32, n, nx, l);
        } else {
            Tile2Regs<false> r;
            tile2_fetch<false>(x, ldx_bytes, base, n, r, l);
            tile2_put<false>(r, tile, l);
            in.read(tile, vi, h);
        }
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < kDenseSlots; ++j) {
            const float v = in.get(j);
            ss = __builtin_fmaf(v, v, ss);
        }
        ss = ss + other_half(ss, h);
        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);

        // y = Pi x_u, K blocks outermost
        f32x16 ay[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) ay[mt] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            Split8 s;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t a0, b0, c0, a1, b1, c1;
                split16(in.get(8 * kb + 2 * q) * inv, &a0, &b0, &c0);
                split16(in.get(8 * kb + 2 * q + 1) * inv, &a1, &b1, &c1);
                s.h11[q] = a0 | (a1 << 16);
                s.hi[q] = b0 | (b1 << 16);
                s.lo[q] = c0 | (c1 << 16);
            }
            dense_kblock(
                ay, s, kb, [&](int row, int chunk) { return mat_frag(lds.pih, row, chunk); },
                [&](int row, int chunk) { return mat_frag(lds.pil, row, chunk); }, l, h);
        }
        uint32_t cw[LW];
#pragma unroll
        for (int k = 0; k < LW; ++k) cw[k] = 0u;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = ay[mt][r];
                put_code<B, LW>(cw, 16 * mt + r, dense_code(e, ba, bb, binc));
            }

        // x~ = Pi^T y^ (roundtrip or QJL), then with QJL the residual, S r
        // and the sign words
        f32x16 ax[4];
        uint32_t sw0 = 0u, sw1 = 0u, gh = 0u;
        float ghat = 0.0f;
        if constexpr (ROUNDTRIP || QJL) dense_pit2<B>(P, lds.ctab, cw, ax, l, h);
        if constexpr (QJL) {
            f32x16 za[4];
#pragma unroll
            for (int mz = 0; mz < 4; ++mz) za[mz] = f32x16{};
            float gam2 = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const int mt = kb >> 1, c = kb & 1;
                u32x4 rh, rl;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float rr[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int r = 8 * c + 2 * q + e;
                        const float xe = ax[mt][r];
                        rr[e] = in.get(16 * mt + r) * inv - xe * kRotScale;
                        gam2 = __builtin_fmaf(rr[e], rr[e], gam2);
                    }
                    uint32_t h0, l0, h1, l1;
                    split_h(rr[0] * kDenseResidualScale, &h0, &l0);
                    split_h(rr[1] * kDenseResidualScale, &h1, &l1);
                    rh[q] = h0 | (h1 << 16);
                    rl[q] = l0 | (l1 << 16);
                }
#pragma unroll
                for (int mz = 0; mz < 4; ++mz) {
                    const u32x4 a = gmat_frag(P.s_fwd, 32 * mz + (l & 31), 2 * kb + h);
                    za[mz] = mfma(a, rh, za[mz]);
                    za[mz] = mfma(a, rl, za[mz]);
                }
            }
            gam2 = gam2 + other_half(gam2, h);
            const float gam = __builtin_sqrtf(gam2);
            gh = f2h(gam);
            ghat = h2f(gh);
            // sign words 2 h, 2 h + 1: bit r of M tile 2 w + p at 16 p + r = [z >= 0]
            // (an accumulator that starts at +0 never ends at -0)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                uint32_t pb = 0u;
#pragma unroll
                for (int mt = 2 * w + 1; mt >= 2 * w; --mt)
#pragma unroll
                    for (int r = 15; r >= 0; --r) {
                        const float e = za[mt][r];
                        pb = __builtin_amdgcn_alignbit(pb, __builtin_bit_cast(uint32_t, e), 31);
                    }
                if (w == 0) sw0 = ~pb;
                else sw1 = ~pb;
            }
        }

        // record
        half_store2(norms, base, n, nh, vi);
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < LW; ++k) stw[vi * W + LW * h + k] = cw[k];
        words2_store<W>(codes, base, n, stw, l);
        if constexpr (QJL) {
            half_store2(rnorms, base, n, gh, vi);
            wave_lds_sync();
            stw[vi * 4 + 2 * h] = sw0;
            stw[vi * 4 + 2 * h + 1] = sw1;
            words2_store<4>(signs, base, n, stw, l);
        }

        // The reconstruction is exactly what tq_dequant_kernel forms from the
        // record just written.
        if constexpr (ROUNDTRIP) {
            f32x16 aq[4];
            if constexpr (QJL) dense_back2(P, sw0, sw1, aq, l, h);
            char* rowo = tile + vi * RBO + dense_half_bytes<OUT_F16>() * h;
            wave_lds_sync();
            dense_out2<QJL, OUT_F16>(ax, aq, P.qjl_scale * ghat, nhat, rowo);
            tile2_store<OUT_F16>(y, ldy_bytes, base, n, tile, l);
        }
    }
}

template <int B, bool QJL, bool OUT_F16>
__global__ __launch_bounds__(256) void tq_dequant_kernel(DenseDev P, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ norms,
                                                         const uint32_t* __restrict__ signs,
                                                         const uint16_t* __restrict__ rnorms, int64_t n,
                                                         char* __restrict__ y, int64_t ldy_bytes) {
    constexpr int LW = 2 * B;
    constexpr int W = 4 * B;
    constexpr int RBO = row_bytes2<OUT_F16>();
    constexpr int SW = 32 * W > 128 ? 32 * W : 128;
    struct Lds {
        uint32_t ctab[32];
        u32x4 tiles[4][32 * RBO / 16];
        uint32_t stage[4][SW];
    };
    __shared__ Lds lds;
    dense_tables_to_lds<B>(P, lds.ctab);
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    char* tile = reinterpret_cast<char*>(lds.tiles[wave]);
    uint32_t* stw = lds.stage[wave];
    const int64_t ntiles = (n + 31) / 32;
    for (int64_t t = blockIdx.x * 4LL + wave; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 32;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int h = l >> 5, vi = l & 31;
        words2_load<W>(codes, base, n, stw, l);
        uint32_t cw[LW];
#pragma unroll
        for (int k = 0; k < LW; ++k) cw[k] = stw[vi * W + LW * h + k];
        const float nhat = h2f(half_load2(norms, base, n, vi));
        uint32_t sw0 = 0u, sw1 = 0u;
        float ghat = 0.0f;
        if constexpr (QJL) {
            words2_load<4>(signs, base, n, stw, l);   // the code words are in registers
            sw0 = stw[vi * 4 + 2 * h];
            sw1 = stw[vi * 4 + 2 * h + 1];
            ghat = h2f(half_load2(rnorms, base, n, vi));
        }
        f32x16 ax[4], aq[4];
        dense_pit2<B>(P, lds.ctab, cw, ax, l, h);
        if constexpr (QJL) dense_back2(P, sw0, sw1, aq, l, h);
        char* rowo = tile + vi * RBO + dense_half_bytes<OUT_F16>() * h;
        wave_lds_sync();
        dense_out2<QJL, OUT_F16>(ax, aq, P.qjl_scale * ghat, nhat, rowo);
        tile2_store<OUT_F16>(y, ldy_bytes, base, n, tile, l);
    }
}

// ----------------------------------------------------------- launchers --
// fp16 input and output: eight-wave workgroups sharing one LDS copy of Pi
// (two waves per SIMD); fp32 tiles need four waves' LDS.
template <int B, bool QJL>
hipError_t launch_tq_quant(const DenseDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                           uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                           int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    const char* xc = static_cast<const char*>(x);
    char* yc = static_cast<char*>(y);
    auto grid = [n](int waves) {
        const int64_t ntiles = (n + 31) / 32;
        const int64_t blocks = (ntiles + waves - 1) / waves;
        return static_cast<int>(blocks < 256 ? (blocks > 0 ? blocks : 1) : 256);
    };
#define TQ_LAUNCH(IF, OF, RT, WV)                                                                                   \
    hipLaunchKernelGGL((tq_quant_kernel<B, QJL, IF, OF, RT, WV>), dim3(grid(WV)), dim3(64 * WV), 0, s, P, xc,      \
                       ldx_bytes, n, codes, norms, signs, rnorms, yc, ldy_bytes)
    if (!roundtrip) {
        if (in_f16) TQ_LAUNCH(true, true, false, 8);
        else TQ_LAUNCH(false, true, false, 4);
    } else if (in_f16) {
        if (out_f16) TQ_LAUNCH(true, true, true, 8);
        else TQ_LAUNCH(true, false, true, 4);
    } else {
        if (out_f16) TQ_LAUNCH(false, true, true, 4);
        else TQ_LAUNCH(false, false, true, 4);
    }
#undef TQ_LAUNCH
    return hipGetLastError();
}

template <int B, bool QJL>
hipError_t launch_tq_dequant(const DenseDev& P, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                             const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                             hipStream_t s) {
    const int64_t ntiles = (n + 31) / 32;
    const int64_t blocks = (ntiles + 3) / 4;
    const int grid = static_cast<int>(blocks < 256 * 2 ? (blocks > 0 ? blocks : 1) : 256 * 2);
    char* yc = static_cast<char*>(y);
    if (out_f16)
        hipLaunchKernelGGL((tq_dequant_kernel<B, QJL, true>), dim3(grid), dim3(256), 0, s, P, codes, norms, signs,
                           rnorms, n, yc, ldy_bytes);
    else
        hipLaunchKernelGGL((tq_dequant_kernel<B, QJL, false>), dim3(grid), dim3(256), 0, s, P, codes, norms, signs,
                           rnorms, n, yc, ldy_bytes);
    return hipGetLastError();
}

}  // namespace rqk
