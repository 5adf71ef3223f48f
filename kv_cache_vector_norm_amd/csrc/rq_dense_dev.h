// TurboQuant comparison path for gfx950: y = Pi x_u with a dense 128 x 128
// random orthogonal Pi, per-coordinate Lloyd-Max codes on 128 coordinates,
// x~ = Pi^T y^, optionally with the QJL residual stage (hyper.ai summary,
// Algorithms 1 and 2; README "How TurboQuant Works").
//
// Both rotations are 32x32x16 MFMA contractions over a tile of 64 vectors
// (one vector per lane, as in the rotor kernels).  Pi is held as an exact
// pair of halves, 16 Pi = P_hi + 2^-11 P_lo, and so is the other operand,
// 16 v = v_hi + 2^-11 v_lo; the three products that matter are folded into
// one fp32 accumulator by scaling v_hi by 2^11:
//   P_hi (2^11 v_hi) + P_hi v_lo + P_lo v_hi = 2^11 * 256 * (Pi v) + O(2^-22).
// The residual projection S r reuses the rotor path's exact scheme (S is
// exactly half; r enters as hi + lo).  Pi feeds the quantize side from LDS;
// Pi^T, S and S^T come from global memory (L2 resident), which keeps LDS
// within one four-wave workgroup per CU.  Codes come from the rotor path's
// exact 256-slot quantiser, with its thresholds scaled by 2^19 so that the
// unscaled accumulators are compared directly.  With QJL, each 32-row tile
// of x~_u = Pi^T y^ is turned into its two K blocks of the residual at once
// and multiplied by S, so the split residual is never held whole.
#pragma once

#include "rq_common_dev.h"
#include "rq_kernels.h"

namespace rqk {

struct DenseDev {
    const uint16_t* __restrict__ pi_hi;
    const uint16_t* __restrict__ pi_lo;
    const uint16_t* __restrict__ pit_hi;
    const uint16_t* __restrict__ pit_lo;
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

// rot_mfma for all four M tiles with the K blocks outermost: split(kb, h11,
// h, lo) forms the 16 split coordinates of block kb (as 8 half pairs each),
// which feed every tile, so the 128 split coordinates are never live at
// once.  Per tile the MFMA order is rot_mfma's.
template <class Split, class FragHi, class FragLo>
__device__ __forceinline__ void rot4_mfma(Split split, FragHi fa_hi, FragLo fa_lo, int l, f32x16 (&ax0)[4],
                                          f32x16 (&ax1)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        ax0[mt] = f32x16{};
        ax1[mt] = f32x16{};
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        uint32_t h11[8], h[8], lo[8];
        split(kb, h11, h, lo);
        u32x4 b11_0, b11_1, bh_0, bh_1, bl_0, bl_1;
        to_operands(u32x4{h11[0], h11[1], h11[2], h11[3]}, u32x4{h11[4], h11[5], h11[6], h11[7]}, &b11_0, &b11_1);
        to_operands(u32x4{h[0], h[1], h[2], h[3]}, u32x4{h[4], h[5], h[6], h[7]}, &bh_0, &bh_1);
        to_operands(u32x4{lo[0], lo[1], lo[2], lo[3]}, u32x4{lo[4], lo[5], lo[6], lo[7]}, &bl_0, &bl_1);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int row = 32 * mt + (l & 31), chunk = 2 * kb + (l >> 5);
            const u32x4 ph = fa_hi(row, chunk);
            const u32x4 pl = fa_lo(row, chunk);
            ax0[mt] = mfma(ph, b11_0, ax0[mt]);
            ax0[mt] = mfma(ph, bl_0, ax0[mt]);
            ax0[mt] = mfma(pl, bh_0, ax0[mt]);
            ax1[mt] = mfma(ph, b11_1, ax1[mt]);
            ax1[mt] = mfma(ph, bl_1, ax1[mt]);
            ax1[mt] = mfma(pl, bh_1, ax1[mt]);
        }
    }
}

// coordinate index of own register (h, r) in M tile MT
__device__ __forceinline__ constexpr int own_coord(int mt, int h, int r) { return 32 * mt + own_row(h, r); }

// Pi^T y^ for all four 32-row M tiles with the K blocks outermost: each
// block's 16 centroid halves (ctab: lo 16 bits = hi half, hi 16 bits =
// 2^11 hi; ctab[L + k] = lo) are formed once and feed every tile, so the
// 128 split coordinates are never live at once.  Per tile the MFMA order is
// that of rot_mfma (K blocks 0..7, the same three products each).
template <int B>
__device__ __forceinline__ void dense_pit_tiles(const DenseDev& P, const uint32_t* __restrict__ ctab,
                                                const uint32_t (&cw)[(128 * B + 31) / 32], int l,
                                                f32x16 (&ax0)[4], f32x16 (&ax1)[4]) {
    constexpr int W = (128 * B + 31) / 32;
    constexpr int L = 1 << B;
    rot4_mfma(
        [&](int kb, uint32_t (&yh11)[8], uint32_t (&yh)[8], uint32_t (&yl)[8]) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t code = get_code<B, W>(cw, 16 * kb + i);
                const uint32_t e = ctab[code];
                const uint32_t eh = e & 0xFFFFu, e11 = e >> 16, el = ctab[L + code];
                if (i & 1) {
                    yh[i >> 1] |= eh << 16;
                    yh11[i >> 1] |= e11 << 16;
                    yl[i >> 1] |= el << 16;
                } else {
                    yh[i >> 1] = eh;
                    yh11[i >> 1] = e11;
                    yl[i >> 1] = el;
                }
            }
        },
        [&](int row, int chunk) { return gmat_frag(P.pit_hi, row, chunk); },
        [&](int row, int chunk) { return gmat_frag(P.pit_lo, row, chunk); }, l, ax0, ax1);
}

// The output of one record from its Pi^T y^ accumulators (dense_pit_tiles):
// plus the QJL term k S^T sigma per tile, times the norm.
template <bool QJL, class Out, class SColFrag, class Done>
__device__ __forceinline__ void dense_finish_vec(const DenseDev& P, const f32x16 (&ax0)[4], const f32x16 (&ax1)[4],
                                                 float nhat, float ghat, const uint32_t (&sw)[4], SColFrag scol,
                                                 Out& out, int l, Done done) {
    const float k = P.qjl_scale * ghat;
    auto tile = [&](auto mt_c) {
        constexpr int MT = decltype(mt_c)::value;
        float x0[16], x1[16];
        from_accumulators(ax0[MT], ax1[MT], x0, x1);
        float q0[16], q1[16];
        if constexpr (QJL) {
            f32x16 a0 = {}, a1 = {};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const uint32_t word = sw[kb >> 1] >> (16 * (kb & 1));
                u32x4 op0, op1;
                u32x4 s0, s1;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t b = word >> (2 * p);
                    s0[p] = 0xBC00BC00u ^ ((b & 1u) << 15) ^ (((b >> 1) & 1u) << 31);
                    const uint32_t c = word >> (8 + 2 * p);
                    s1[p] = 0xBC00BC00u ^ ((c & 1u) << 15) ^ (((c >> 1) & 1u) << 31);
                }
                to_operands(s0, s1, &op0, &op1);
                const u32x4 a = scol(32 * MT + (l & 31), 2 * kb + (l >> 5));
                a0 = mfma(a, op0, a0);
                a1 = mfma(a, op1, a1);
            }
            from_accumulators(a0, a1, q0, q1);
        }
        // coordinates of this tile in increasing order
#pragma unroll
        for (int il = 0; il < 32; ++il) {
            const int b8 = il >> 3, w = il & 7;
            const float xv = (w < 4 ? x0[4 * b8 + w] : x1[4 * b8 + w - 4]) * kRotScale;
            float v = xv;
            if constexpr (QJL) v = __builtin_fmaf(k, w < 4 ? q0[4 * b8 + w] : q1[4 * b8 + w - 4], xv);
            out.set(32 * MT + il, nhat * v);
        }
        done(MT);
    };
    tile(std::integral_constant<int, 0>{});
    tile(std::integral_constant<int, 1>{});
    tile(std::integral_constant<int, 2>{});
    tile(std::integral_constant<int, 3>{});
}

template <int B, bool QJL, class Out, class SColFrag, class Done>
__device__ __forceinline__ void dense_dequant_vec(const DenseDev& P, const uint32_t* __restrict__ ctab,
                                                  const uint32_t (&cw)[(128 * B + 31) / 32], float nhat, float ghat,
                                                  const uint32_t (&sw)[4], SColFrag scol, Out& out, int l, Done done) {
    // x~ = Pi^T y^, y^ = c[code]
    f32x16 ax0[4], ax1[4];
    dense_pit_tiles<B>(P, ctab, cw, l, ax0, ax1);
    dense_finish_vec<QJL>(P, ax0, ax1, nhat, ghat, sw, scol, out, l, done);
}

// ------------------------------------------------------------ kernels --
template <int WAVES>
struct DenseLds {
    u32x4 bins[kBinSlots];      // slot table (LDS address 0), thresholds and centroids times 2^19
    u32x4 tiles[WAVES][kTileBytes / 16];
    u32x4 pih[128 * 16];
    u32x4 pil[128 * 16];
    uint32_t ctab[32];
    float thr[16];
};

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
// (power-of-two scalings are exact), and acc > 2^19 t equals y > t.
__device__ __forceinline__ uint32_t dense_code(float acc, float ba, float bb, const char* __restrict__ bins) {
    const uint32_t off = __builtin_bit_cast(uint32_t, __builtin_fmaf(acc, ba, bb)) & 0xFF0u;
    const uint2 e = *reinterpret_cast<const uint2*>(bins + off);   // {base code, boundary in the slot}
    return e.x + (acc > __builtin_bit_cast(float, e.y) ? 1u : 0u);
}

template <int B>
__device__ __forceinline__ void dense_tables_to_lds(const DenseDev& P, uint32_t* ctab, float* thr) {
    constexpr int L = 1 << B;
    if (threadIdx.x < L) {
        uint32_t h11, h, l;
        split16(P.cent[threadIdx.x], &h11, &h, &l);
        ctab[threadIdx.x] = h | (h11 << 16);
        ctab[L + threadIdx.x] = l;
    }
    if (threadIdx.x < L - 1) thr[threadIdx.x] = P.thr[threadIdx.x];
}

template <int B, bool QJL, bool IN_F16, bool OUT_F16, bool ROUNDTRIP, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void tq_quant_kernel(DenseDev P, const char* __restrict__ x,
                                                              int64_t ldx_bytes, int64_t n,
                                                              uint32_t* __restrict__ codes,
                                                              uint16_t* __restrict__ norms,
                                                              uint32_t* __restrict__ signs,
                                                              uint16_t* __restrict__ rnorms, char* __restrict__ y,
                                                              int64_t ldy_bytes) {
    constexpr int W = (128 * B + 31) / 32;
    __shared__ DenseLds<WAVES> sm;
    dense_tables_to_lds<B>(P, sm.ctab, sm.thr);
    dense_bins_to_lds(P, sm.bins);
    mat_to_lds<WAVES * 64>(P.pi_hi, sm.pih);
    mat_to_lds<WAVES * 64>(P.pi_lo, sm.pil);
    __syncthreads();
    const float ba = P.bin_a * kRotScale, bb = P.bin_b;
    const char* binc = reinterpret_cast<const char*>(sm.bins);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* tile = sm.tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
    const bool single = ntiles <= kSimds;   // at most one tile per SIMD: output leaves in quarters
    for (int64_t t = blockIdx.x * (int64_t)WAVES + wave; t < ntiles; t += gridDim.x * (int64_t)WAVES) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;

        // load, norm (same arithmetic as the rotor path).  fp16 input stays in
        // the wave's LDS tile until the residual step (nothing writes the tile
        // before the record is staged) and is read from there where it is
        // used, so no input registers are held across the rotations.
        if constexpr (IN_F16) {
            tile_load(x, ldx_bytes, base, n, 0, tile, l);
            wave_lds_sync();
        }
        auto xword = [&](int k) -> uint32_t {
            const u32x4 q = tile[swz(l, k >> 2)];
            return q[k & 3];
        };
        float xf32[IN_F16 ? 1 : 128];
        if constexpr (!IN_F16) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                tile_load(x, ldx_bytes, base, n, 256 * h, tile, l);
                wave_lds_sync();
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const u32x4 q = tile[swz(l, c)];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t qe = q[e];
                        xf32[64 * h + 4 * c + e] = __builtin_bit_cast(float, qe);
                    }
                }
            }
        }
        auto xget = [&](int i) -> float {
            if constexpr (IN_F16) {
                const uint32_t w = xword(i >> 1);
                return h2f((i & 1) ? (w >> 16) : (w & 0xFFFFu));
            } else {
                return xf32[i];
            }
        };
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
            const float v = xget(i);
            ss = __builtin_fmaf(v, v, ss);
        }

        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);

        // y = Pi x_u
        uint32_t cw[W];
#pragma unroll
        for (int k = 0; k < W; ++k) cw[k] = 0u;
        if constexpr (QJL) {
            // the K blocks outermost (the residual step that follows needs the
            // registers)
            f32x16 ay0[4], ay1[4];
            rot4_mfma(
                [&](int kb, uint32_t (&vh11)[8], uint32_t (&vh)[8], uint32_t (&vl)[8]) {
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        uint32_t a0, b0, c0, a1, b1, c1;
                        split16(xget(16 * kb + i) * inv, &a0, &b0, &c0);
                        split16(xget(16 * kb + i + 1) * inv, &a1, &b1, &c1);
                        vh11[i >> 1] = a0 | (a1 << 16);
                        vh[i >> 1] = b0 | (b1 << 16);
                        vl[i >> 1] = c0 | (c1 << 16);
                    }
                },
                [&](int row, int chunk) { return mat_frag(sm.pih, row, chunk); },
                [&](int row, int chunk) { return mat_frag(sm.pil, row, chunk); }, l, ay0, ay1);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float y0[16], y1[16];
                from_accumulators(ay0[mt], ay1[mt], y0, y1);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    put_code<B, W>(cw, 32 * mt + own_row(0, r), dense_code(y0[r], ba, bb, binc));
                    put_code<B, W>(cw, 32 * mt + own_row(1, r), dense_code(y1[r], ba, bb, binc));
                }
            }
        } else {
            // all 128 split coordinates, then one M tile at a time (each tile's
            // codes are formed while the next tile's MFMAs run)
            uint32_t vh11[64], vh[64], vl[64];
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                uint32_t a, b, c;
                split16(xget(i) * inv, &a, &b, &c);
                put_pair(vh11, i, a);
                put_pair(vh, i, b);
                put_pair(vl, i, c);
            }
            auto tile_q = [&](auto mt_c) {
                constexpr int MT = decltype(mt_c)::value;
                float y0[16], y1[16];
                rot_mfma<MT>(
                    vh11, vh, vl, [&](int row, int chunk) { return mat_frag(sm.pih, row, chunk); },
                    [&](int row, int chunk) { return mat_frag(sm.pil, row, chunk); }, l, y0, y1);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    put_code<B, W>(cw, own_coord(MT, 0, r), dense_code(y0[r], ba, bb, binc));
                    put_code<B, W>(cw, own_coord(MT, 1, r), dense_code(y1[r], ba, bb, binc));
                }
            };
            tile_q(std::integral_constant<int, 0>{});
            tile_q(std::integral_constant<int, 1>{});
            tile_q(std::integral_constant<int, 2>{});
            tile_q(std::integral_constant<int, 3>{});
        }

        uint32_t sw[4] = {0u, 0u, 0u, 0u};
        uint32_t gh = 0u;
        float ghat = 0.0f;
        if constexpr (QJL) {
            // x~_u = Pi^T y^ (all four M tiles, K blocks outermost); then each
            // tile gives the residual r = x_u - x~_u of its two K blocks
            // (original domain), whose S r MFMAs run at once for all four
            // output tiles (the K order of every z accumulator stays 0..7)
            f32x16 ax0[4], ax1[4];
            dense_pit_tiles<B>(P, sm.ctab, cw, l, ax0, ax1);
            f32x16 za[4][2];
#pragma unroll
            for (int mz = 0; mz < 4; ++mz) za[mz][0] = za[mz][1] = f32x16{};
            float gam2 = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float x0[16], x1[16];
                from_accumulators(ax0[mt], ax1[mt], x0, x1);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int kb = 2 * mt + kk;
                    uint32_t rh[8], rl[8];
#pragma unroll
                    for (int il = 16 * kk; il < 16 * kk + 16; ++il) {
                        const int b8 = il >> 3, w = il & 7, i = 32 * mt + il;
                        const float xt = (w < 4 ? x0[4 * b8 + w] : x1[4 * b8 + w - 4]) * kRotScale;
                        const float r = xget(i) * inv - xt;
                        gam2 = __builtin_fmaf(r, r, gam2);
                        uint32_t hi, lo;
                        split_h(r * kDenseResidualScale, &hi, &lo);
                        const int d = (il & 15) >> 1;
                        if (il & 1) {
                            rh[d] |= hi << 16;
                            rl[d] |= lo << 16;
                        } else {
                            rh[d] = hi;
                            rl[d] = lo;
                        }
                    }
                    u32x4 h0, h1, l0, l1;
                    to_operands(u32x4{rh[0], rh[1], rh[2], rh[3]}, u32x4{rh[4], rh[5], rh[6], rh[7]}, &h0, &h1);
                    to_operands(u32x4{rl[0], rl[1], rl[2], rl[3]}, u32x4{rl[4], rl[5], rl[6], rl[7]}, &l0, &l1);
#pragma unroll
                    for (int mz = 0; mz < 4; ++mz) {
                        const u32x4 a = gmat_frag(P.s_rows, 32 * mz + (l & 31), 2 * kb + (l >> 5));
                        za[mz][0] = mfma(a, h0, za[mz][0]);
                        za[mz][0] = mfma(a, l0, za[mz][0]);
                        za[mz][1] = mfma(a, h1, za[mz][1]);
                        za[mz][1] = mfma(a, l1, za[mz][1]);
                    }
                }
            }
            const float gam = __builtin_sqrtf(gam2);
            gh = f2h(gam);
            ghat = h2f(gh);
#pragma unroll
            for (int mz = 0; mz < 4; ++mz) {
                float z0[16], z1[16];
                from_accumulators(za[mz][0], za[mz][1], z0, z1);
                uint32_t word = 0u;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    word |= (z0[r] >= 0.0f ? 1u : 0u) << own_row(0, r);
                    word |= (z1[r] >= 0.0f ? 1u : 0u) << own_row(1, r);
                }
                sw[mz] = word;
            }
        }

        if (base + l < n) norms[base + l] = static_cast<uint16_t>(nh);
        words_store<W>(codes, base, n, cw, stage, l);
        if constexpr (QJL) {
            if (base + l < n) rnorms[base + l] = static_cast<uint16_t>(gh);
            words_store<4>(signs, base, n, sw, stage, l);
        }
        if constexpr (ROUNDTRIP) {
            VecOutT<OUT_F16> out;
            if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
            out.begin(tile, l);
            auto scol = [&](int row, int chunk) { return gmat_frag(P.s_cols, row, chunk); };
            auto done = [&](int mt) {
                if constexpr (OUT_F16) {
                    if (single) out.store_cols(y, ldy_bytes, base, n, 4 * mt);
                }
            };
            // the output is what tq_dequantize forms from the record (Pi^T y^
            // again: the residual step's accumulators are not kept).  The
            // codes and the Pi^T pointers pass through opaque copies so that
            // the compiler does not reuse the residual step's table addresses
            // and fragment loads (holding them live until here); nothing is
            // scheduled across either.
            __builtin_amdgcn_sched_barrier(0);
            DenseDev P2 = P;
            const int oz = opaque_zero();
            P2.pit_hi += oz;
            P2.pit_lo += oz;
            uint32_t cw2[W];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                cw2[k] = cw[k];
                pin(cw2[k]);
            }
            dense_dequant_vec<B, QJL>(P2, sm.ctab, cw2, nhat, ghat, sw, scol, out, l, done);
            if (!OUT_F16 || !single) out.store(y, ldy_bytes, base, n);
        }
    }
}

template <int B, bool QJL, bool OUT_F16>
__global__ __launch_bounds__(256) void tq_dequant_kernel(DenseDev P, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ norms,
                                                         const uint32_t* __restrict__ signs,
                                                         const uint16_t* __restrict__ rnorms, int64_t n,
                                                         char* __restrict__ y, int64_t ldy_bytes) {
    constexpr int W = (128 * B + 31) / 32;
    __shared__ u32x4 tiles[4][kTileBytes / 16];
    __shared__ uint32_t ctab[32];
    __shared__ float thr_unused[16];
    dense_tables_to_lds<B>(P, ctab, thr_unused);
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* tile = tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
    const bool single = ntiles <= kSimds;
    for (int64_t t = blockIdx.x * 4LL + wave; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        uint32_t cw[W];
        words_load<W>(codes, base, n, cw, stage, l);
        const bool live = base + l < n;
        const float nhat = live ? h2f(norms[base + l]) : 0.0f;
        uint32_t sw[4] = {0u, 0u, 0u, 0u};
        float ghat = 0.0f;
        if constexpr (QJL) {
            words_load<4>(signs, base, n, sw, stage, l);
            ghat = live ? h2f(rnorms[base + l]) : 0.0f;
        }
        VecOutT<OUT_F16> out;
        if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
        out.begin(tile, l);
        dense_dequant_vec<B, QJL>(
            P, ctab, cw, nhat, ghat, sw, [&](int row, int chunk) { return gmat_frag(P.s_cols, row, chunk); }, out, l,
            [&](int mt) {
                if constexpr (OUT_F16) {
                    if (single) out.store_cols(y, ldy_bytes, base, n, 4 * mt);
                }
            });
        if (!OUT_F16 || !single) out.store(y, ldy_bytes, base, n);
    }
}

template <int B, bool QJL>
hipError_t launch_tq_quant(const DenseDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                           uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                           int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    constexpr int WAVES = 4;
    const int64_t ntiles = (n + 63) / 64;
    const int64_t blocks = (ntiles + WAVES - 1) / WAVES;
    const int grid = static_cast<int>(blocks < 256 * 4 ? (blocks > 0 ? blocks : 1) : 256 * 4);
    const char* xc = static_cast<const char*>(x);
    char* yc = static_cast<char*>(y);
#define TQ_LAUNCH(IF, OF, RT)                                                                                  \
    hipLaunchKernelGGL((tq_quant_kernel<B, QJL, IF, OF, RT, WAVES>), dim3(grid), dim3(WAVES * 64), 0, s, P, xc, \
                       ldx_bytes, n, codes, norms, signs, rnorms, yc, ldy_bytes)
    if (!roundtrip) {
        if (in_f16) TQ_LAUNCH(true, true, false); else TQ_LAUNCH(false, true, false);
    } else if (in_f16) {
        if (out_f16) TQ_LAUNCH(true, true, true); else TQ_LAUNCH(true, false, true);
    } else {
        if (out_f16) TQ_LAUNCH(false, true, true); else TQ_LAUNCH(false, false, true);
    }
#undef TQ_LAUNCH
    return hipGetLastError();
}

template <int B, bool QJL>
hipError_t launch_tq_dequant(const DenseDev& P, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                             const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                             hipStream_t s) {
    const int64_t ntiles = (n + 63) / 64;
    const int64_t blocks = (ntiles + 3) / 4;
    const int grid = static_cast<int>(blocks < 256 * 8 ? (blocks > 0 ? blocks : 1) : 256 * 8);
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
