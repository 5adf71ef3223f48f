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
// 8 kb .. 8 kb + 7 of both halves.  Pi, Pi^T, T and S^T are permuted on the
// host so that accumulator element r of M tile mt in half h is slot
// 16 mt + r of that half, so operands and results never leave their lane.
// The record's 4 B code words split evenly too: half h packs its 64 codes
// into record words 2 B h .. 2 B h + 2 B - 1.
//
// QJL stage.  The sign sketch of the residual r = x_u - Pi^T y^ is formed in
// the rotated domain: S r = T (y - y^) with T = S Pi^T (host, float64), and
// gamma = |r| = |y - y^| (Pi orthogonal).  So the quantiser never forms
// Pi^T y^; only a reconstruction (roundtrip, dequantiser) does.
//
// Precision: 16 Pi = P_hi + 2^-11 P_lo and 16 v = v_hi + 2^-11 v_lo as exact
// half pairs, three products folded into one fp32 accumulator,
// P_hi (2^11 v_hi) + P_hi v_lo + P_lo v_hi = 2^19 (Pi v) + O(2^-22); codes
// from the rotor path's exact slot table with thresholds scaled by 2^19; T
// and 8 (y - y^) enter T (y - y^) as pairs the same way (T unscaled).
//
// Operands.  Pi sits in LDS (the quantiser); Pi^T, T and S^T are read from
// L2 in fragment order (one contiguous kilobyte per wave and fragment), the
// fragments of K block kb + 1 requested before the products of K block kb.
#pragma once

#include "rq_dense_dev.h"
#include "rq_rotor_dev.h"
#include "rq_tile2_dev.h"

namespace rqk {

constexpr int kDenseSlots = 64;

// The lane's 64 input slots.
// The lane's 64 input slots from the DMA-filled tile (rows of 256 / 512
// bytes, chunk c of row v at position c ^ (v & 15); lane half h reads chunks
// 8 h .. (fp16) or 16 h .. (fp32) of its row, 16 rows of a half-wave on 16
// distinct bank groups).
template <bool IN_F16>
struct DSlots;

template <>
struct DSlots<true> {
    uint32_t w[kDenseSlots / 2];
    __device__ void read(const char* tile, int vi, int h) {
        const char* row = tile + vi * 256;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(row + 16 * ((8 * h + k) ^ (vi & 15)));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = q[e];
                w[4 * k + e] = x;
            }
        }
    }
    __device__ float get(int j) const { return h2f((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu)); }
};

template <>
struct DSlots<false> {
    float v[kDenseSlots];
    __device__ void read(const char* tile, int vi, int h) {
        const char* row = tile + vi * 512;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(row + 16 * ((16 * h + k) ^ (vi & 15)));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = q[e];
                v[4 * k + e] = __builtin_bit_cast(float, x);
            }
        }
    }
    __device__ float get(int j) const { return v[j]; }
};

// mat_to_lds of 2^11 times a half matrix (exact: |2^11 P_hi| < 2^14).
template <int NT>
__device__ __forceinline__ void mat_to_lds_x2048(const uint16_t* __restrict__ g, u32x4* __restrict__ m) {
    static_assert(128 * 16 % NT == 0, "block size");
    const u32x4* src = reinterpret_cast<const u32x4*>(g);
    constexpr f16x2 k2048 = {static_cast<f16>(2048.0f), static_cast<f16>(2048.0f)};
    u32x4 v[128 * 16 / NT];
#pragma unroll
    for (int it = 0; it < 128 * 16 / NT; ++it) v[it] = src[it * NT + threadIdx.x];
#pragma unroll
    for (int it = 0; it < 128 * 16 / NT; ++it) {
        const int q = it * NT + threadIdx.x, row = q >> 4, c = q & 15;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = v[it][e];
            w[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, x) * k2048);
        }
        m[row * 16 + (c ^ (row & 15))] = w;
    }
}

// Operands of K block kb from the 8 split slots (half pairs): 2^11 hi, lo, hi.
struct Split8 {
    u32x4 h11, lo, hi;
};

// Splits of 8 values v into the three operands, pairs at a time: val16(e)
// gives a = 16 v; hi = half(a) (packed conversion), 2^11 hi by a packed half
// multiply (exact), lo = half(2^11 a - 2^11 hi) (the fma is exact, since
// a - hi is).  Bit for bit what split16 gives per value.
template <class Val16>
__device__ __forceinline__ Split8 split8(Val16 val16) {
    constexpr f16x2 k2048 = {static_cast<f16>(2048.0f), static_cast<f16>(2048.0f)};
    Split8 s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float a = val16(2 * q), b = val16(2 * q + 1);
        const uint32_t hi = cvt_pk(a, b);
        const f16x2 h11 = __builtin_bit_cast(f16x2, hi) * k2048;
        const float ha = static_cast<float>(h11[0]), hb = static_cast<float>(h11[1]);
        s.hi[q] = hi;
        s.h11[q] = __builtin_bit_cast(uint32_t, h11);
        s.lo[q] = cvt_pk(__builtin_fmaf(a, 2048.0f, -ha), __builtin_fmaf(b, 2048.0f, -hb));
    }
    return s;
}

// The three products of one K block for the four M tiles, M tiles innermost
// (four independent accumulators between dependent MFMAs); per accumulator
// the order is always 2^11 hi, lo, hi.
__device__ __forceinline__ void kblock3(f32x16 (&acc)[4], const Split8& s, const u32x4 (&fh)[4],
                                        const u32x4 (&fl)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(fh[mt], s.h11, acc[mt]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(fh[mt], s.lo, acc[mt]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(fl[mt], s.hi, acc[mt]);
}

// A fragment-ordered 128 x 128 half matrix in global memory.
constexpr int kFragMatBytes = 128 * 128 * 2;
__device__ __forceinline__ u32x4 gfrag(rsrc_t rs, uint32_t voff, int mt, int kb) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (mt * 8 + kb) * 1024, 0);
}

// The hi and lo fragments of one K block (all four M tiles) of a
// fragment-ordered pair, and the fragments of one K block of a single
// matrix.
struct Frag8 {
    u32x4 h[4], l[4];
};
struct Frag4 {
    u32x4 f[4];
};
struct GPair {
    rsrc_t hi, lo;
    uint32_t vo;
    __device__ GPair(const uint16_t* mh, const uint16_t* ml, int l)
        : hi(make_rsrc(mh, kFragMatBytes)), lo(make_rsrc(ml, kFragMatBytes)), vo(16u * static_cast<uint32_t>(l)) {}
    __device__ Frag8 load(int kb) const {
        Frag8 f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f.h[mt] = gfrag(hi, vo, mt, kb);
            f.l[mt] = gfrag(lo, vo, mt, kb);
        }
        return f;
    }
};
struct GOne {
    rsrc_t m;
    uint32_t vo;
    __device__ GOne(const uint16_t* p, int l) : m(make_rsrc(p, kFragMatBytes)), vo(16u * static_cast<uint32_t>(l)) {}
    __device__ Frag4 load(int kb) const {
        Frag4 f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) f.f[mt] = gfrag(m, vo, mt, kb);
        return f;
    }
};

// acc[mt] = sum over K blocks of (hi, lo matrix pair) x make(kb); `first`
// holds K block 0's fragments (requested by the caller as early as it can),
// later K blocks are requested one K block ahead.
template <class Make>
__device__ __forceinline__ void gprod3(f32x16 (&acc)[4], const GPair& g, const Frag8& first, Make make) {
    Frag8 f[2];
    f[0] = first;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int cur = kb & 1;
        if (kb < 7) f[cur ^ 1] = g.load(kb + 1);
        kblock3(acc, make(kb), f[cur].h, f[cur].l);
    }
}

// acc[mt] = sum over K blocks of (exact half matrix) x make(kb), likewise.
template <class Make>
__device__ __forceinline__ void gprod1(f32x16 (&acc)[4], const GOne& g, const Frag4& first, Make make) {
    Frag4 f[2];
    f[0] = first;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int cur = kb & 1;
        if (kb < 7) f[cur ^ 1] = g.load(kb + 1);
        const u32x4 b = make(kb);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(f[cur].f[mt], b, acc[mt]);
    }
}

// x~ = Pi^T y^ of the lane's 64 slots (accumulator scale 2^19), y^ the
// centroids of the lane's codes; the same sequence in the quantiser's
// roundtrip and in the dequantiser.
template <int B>
__device__ __forceinline__ void dense_pit2(const GPair& g, const Frag8& first, const uint2* __restrict__ ptab,
                                           const uint32_t (&cw)[2 * B], f32x16 (&ax)[4]) {
    constexpr f16x2 k2048 = {static_cast<f16>(2048.0f), static_cast<f16>(2048.0f)};
    // slots 8 kb + 2 q and 8 kb + 2 q + 1 are one 2B-bit code pair; the
    // table entries of K block kb + 1 are read while K block kb is formed
    uint2 ent[2][4];
    auto read = [&](int kb, uint2 (&d)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = ptab[get_code<2 * B, 2 * B>(cw, 4 * kb + q)];
    };
    read(0, ent[0]);
    gprod3(ax, g, first, [&](int kb) {
        const int cur = kb & 1;
        if (kb < 7) read(kb + 1, ent[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        Split8 s;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t hi = ent[cur][q].x, lo = ent[cur][q].y;
            s.hi[q] = hi;
            s.lo[q] = lo;
            s.h11[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) * k2048);   // exact
        }
        return s;
    });
}

// S^T sigma of the lane's slots from its two sign words (sign indices
// 64 h .. 64 h + 63; K block kb takes bits 8 kb .. 8 kb + 7); the same
// sequence in the roundtrip and the dequantiser.
__device__ __forceinline__ void dense_back2(const GOne& g, const Frag4& first, uint32_t sw0, uint32_t sw1,
                                            f32x16 (&acc)[4]) {
    gprod1(acc, g, first, [&](int kb) {
        const uint32_t w = kb < 4 ? sw0 : sw1;
        u32x4 d0, d1;
        sigma16((w >> (16 * ((kb >> 1) & 1))) & 0xFFFFu, d0, d1);
        return (kb & 1) ? d1 : d0;
    });
}

// Output slots of the lane, n^ x~ (MSE) or n^ (x~ + k (S^T sigma)) (QJL) with
// x~ = ax * kRotScale, as the 16-byte words the lane stores: its 64 slots are
// coordinates 64 h .. 64 h + 63 of row vi, 128 (fp16) or 256 (fp32)
// contiguous bytes.  fp16 output is the rounding of the materialised fp32
// value.
template <bool OUT_F16>
struct OutWords {
    u32x4 w[OUT_F16 ? 8 : 16];
};
template <bool QJL, bool OUT_F16>
__device__ __forceinline__ void dense_out_words(const f32x16 (&ax)[4], const f32x16 (&aq)[4], float k, float nhat,
                                                OutWords<OUT_F16>& out) {
    // n^ (ax 2^-19 + k aq) == (n^ 2^-19) (ax + (k 2^19) aq) bit for bit
    // (power-of-two scalings commute with rounding)
    const float k19 = k * (1.0f / kRotScale), n19 = nhat * kRotScale;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float o[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = ax[mt][r];
            if constexpr (QJL) {
                const float f = aq[mt][r];
                v = __builtin_fmaf(k19, f, v);
            }
            o[r] = n19 * v;
        }
        constexpr int NC = OUT_F16 ? 2 : 4;   // 16-byte words of this M tile
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (OUT_F16) {
                    float a = o[8 * c + 2 * q], b = o[8 * c + 2 * q + 1];
                    pin(a);
                    pin(b);
                    out.w[NC * mt + c][q] = cvt_pk(a, b);
                } else {
                    out.w[NC * mt + c][q] = __builtin_bit_cast(uint32_t, o[4 * c + q]);
                }
            }
    }
}
// Stores them for the tile at row `base`; rows at or beyond n are not
// written.  The stores are ordinary (cached) ones: L2 merges a lane's
// 16-byte pieces into whole lines, where non-temporal stores of partial
// lines cost several times more.
template <bool OUT_F16>
__device__ __forceinline__ void dense_out_put(const OutWords<OUT_F16>& out, char* __restrict__ y, int64_t ldy_bytes,
                                              int64_t base, int64_t n, int vi, int h) {
    const rsrc_t rs = make_rsrc(y + base * ldy_bytes, tile2_range(n - base, ldy_bytes));
    const uint32_t voff = static_cast<uint32_t>(vi) * static_cast<uint32_t>(ldy_bytes) +
                          static_cast<uint32_t>((OUT_F16 ? 128 : 256) * h);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < (OUT_F16 ? 8 : 16); ++c)
        __builtin_amdgcn_raw_buffer_store_b128(out.w[c], rs, voff, 16 * c, 0);
    store_data_fence();
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
    constexpr int TB = 32 * (IN_F16 ? 256 : 512);   // input tile (LDS DMA)
    constexpr int SW = 32 * W > 128 ? 32 * W : 128;
    // The input tiles come first: the copies address them below 64 KB.
    static_assert(WAVES * TB <= 65536, "input tiles must lie in the first 64 KB of LDS");
    struct Lds {
        u32x4 tiles[WAVES][TB / 16];
        u32x4 bins[kBinSlots];      // slot table, thresholds and centroids times 2^19
        u32x4 pih[128 * 16];       // P_hi, or 2^11 P_hi for fp16 input
        u32x4 pil[128 * 16];
        uint2 ptab[1 << (2 * B)];   // centroid pair table
        uint32_t stage[WAVES][SW];
    };
    __shared__ Lds lds;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (n + 31) / 32;
    const int64_t tstep = static_cast<int64_t>(gridDim.x) * WAVES;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * WAVES + wave;
    char* tile = reinterpret_cast<char*>(lds.tiles[wave]);
    if (t0 < ntiles) tile2_dma<IN_F16>(x, ldx_bytes, t0 * 32, n, tile, lane_id());
    dense_tables_to_lds<B>(P, lds.ptab);
    dense_bins_to_lds(P, lds.bins);
    if constexpr (IN_F16) mat_to_lds_x2048<NT>(P.pi2_hi, lds.pih);   // 2^11 P_hi
    else mat_to_lds<NT>(P.pi2_hi, lds.pih);
    mat_to_lds<NT>(P.pi2_lo, lds.pil);
    __syncthreads();
    const float ba = P.bin_a * kRotScale, bb = P.bin_b;
    const char* binc = reinterpret_cast<const char*>(lds.bins);
    uint32_t* stw = lds.stage[wave];

    // A roundtrip stores each tile's output after the next tile's input has
    // arrived (the wait for the input covers every earlier memory operation,
    // so stores issued just before it would be waited for at once).
    OutWords<OUT_F16> pend;
    int64_t pend_base = -1;

    for (int64_t t = t0; t < ntiles; t += tstep) {
        const int64_t base = t * 32;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int h = l >> 5, vi = l & 31;
        // this tile's input, then the next tile's copy into the same buffer
        DSlots<IN_F16> in;
        tile2_dma_wait();
        in.read(tile, vi, h);
        lds_reads_done();
        if (t + tstep < ntiles) tile2_dma<IN_F16>(x, ldx_bytes, (t + tstep) * 32, n, tile, l);
        if constexpr (ROUNDTRIP) {
            if (pend_base >= 0) dense_out_put<OUT_F16>(pend, y, ldy_bytes, pend_base, n, vi, h);
        }
        float ss = 0.0f;
        if constexpr (IN_F16) {
#pragma unroll
            for (int k = 0; k < kDenseSlots / 2; ++k) {
                const f16x2 v = __builtin_bit_cast(f16x2, in.w[k]);
                ss = __builtin_amdgcn_fdot2(v, v, ss, false);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kDenseSlots; ++j) {
                const float v = in.get(j);
                ss = __builtin_fmaf(v, v, ss);
            }
        }
        ss = ss + other_half(ss, h);
        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);

        const float inv16 = 16.0f * inv;   // (v inv) 16 == v (16 inv): power-of-two scaling

        // y = Pi x_u, Pi from LDS.  fp16 input enters the MFMAs as it is
        // (exact): (2^11 P_hi) x + P_lo x = 2^15 Pi x, then times 16 / |x|.
        // fp32 input is normalised first and split: accumulator 2^19 Pi x_u.
        // (K block kb + 1's fragments are read before K block kb's MFMAs
        // issue; the scheduling barrier keeps the compiler from moving each
        // read down next to its MFMA)
        f32x16 ay[4];
        u32x4 fh[2][4], fl[2][4];
        auto pi_frags = [&](int kb, u32x4 (&dh)[4], u32x4 (&dl)[4]) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = 32 * mt + (l & 31), chunk = 2 * kb + h;
                dh[mt] = mat_frag(lds.pih, row, chunk);
                dl[mt] = mat_frag(lds.pil, row, chunk);
            }
        };
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) ay[mt] = f32x16{};
        pi_frags(0, fh[0], fl[0]);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const int cur = kb & 1;
            if (kb < 7) pi_frags(kb + 1, fh[cur ^ 1], fl[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (IN_F16) {
                const u32x4 xb = {in.w[4 * kb], in.w[4 * kb + 1], in.w[4 * kb + 2], in.w[4 * kb + 3]};
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) ay[mt] = mfma(fh[cur][mt], xb, ay[mt]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) ay[mt] = mfma(fl[cur][mt], xb, ay[mt]);
            } else {
                kblock3(ay, split8([&](int e) { return in.get(8 * kb + e) * inv16; }), fh[cur], fl[cur]);
            }
        }
        const float ysc = IN_F16 ? inv16 : 1.0f;
        // phases stay in order: interleaving the rotation with the sketch
        // below only lengthens register lifetimes
        __builtin_amdgcn_sched_barrier(0);

        // QJL: the first fragments of T (y - y^) requested now
        const GPair tg(P.t2_hi, P.t2_lo, l);
        Frag8 tf0;
        if constexpr (QJL) tf0 = tg.load(0);

        // codes; with QJL the accumulators become 2^19 (y - y^) in place
        uint32_t cw[LW];
#pragma unroll
        for (int k = 0; k < LW; ++k) cw[k] = 0u;
        // (slot-table entries read CB at a time ahead of their use)
        constexpr int CB = QJL ? 8 : 16;
#pragma unroll
        for (int b0 = 0; b0 < 64; b0 += CB) {
            float e[CB];
            u32x4 ent[CB];
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                const int mt = (b0 + i) >> 4, r = (b0 + i) & 15;
                e[i] = IN_F16 ? ay[mt][r] * ysc : ay[mt][r];
                const char* pe = binc + dense_slot(e[i], ba, bb);
                if constexpr (QJL) {
                    ent[i] = *reinterpret_cast<const u32x4*>(pe);
                } else {
                    const uint2 v = *reinterpret_cast<const uint2*>(pe);
                    ent[i] = u32x4{v.x, v.y, 0u, 0u};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                const int mt = (b0 + i) >> 4, r = (b0 + i) & 15;
                float cv;
                put_code<B, LW>(cw, b0 + i, dense_decide(e[i], ent[i], &cv));
                if constexpr (QJL) ay[mt][r] = e[i] - cv;
            }
        }

        // QJL: gamma = |y - y^|, z = T (y - y^) (scale 2^14), sign words
        // 2 h, 2 h + 1: bit r of M tile 2 w + p at 16 p + r = [z >= 0]
        uint32_t sw0 = 0u, sw1 = 0u, gh = 0u;
        float ghat = 0.0f;
        if constexpr (QJL) {
            // (summed at the accumulator scale 2^19 and scaled once: bit for
            // bit the sum of the unscaled squares)
            float gam2 = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float d = ay[mt][r];
                    gam2 = __builtin_fmaf(d, d, gam2);
                }
            gam2 = (gam2 + other_half(gam2, h)) * (kRotScale * kRotScale);
            gh = f2h(__builtin_sqrtf(gam2));
            ghat = h2f(gh);
            f32x16 za[4];
            gprod3(za, tg, tf0, [&](int kb) {
                return split8([&](int e) { return ay[kb >> 1][8 * (kb & 1) + e] * (kRotScale * 8.0f); });
            });
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

        // the reconstruction's first Pi^T fragments requested before the
        // record is written
        const GPair pg(P.pit2_hi, P.pit2_lo, l);
        Frag8 pf0;
        if constexpr (ROUNDTRIP) pf0 = pg.load(0);

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
            f32x16 ax[4], aq[4];
            dense_pit2<B>(pg, pf0, lds.ptab, cw, ax);
            if constexpr (QJL) {
                const GOne sg(P.s_back, l);
                dense_back2(sg, sg.load(0), sw0, sw1, aq);
            }
            dense_out_words<QJL, OUT_F16>(ax, aq, P.qjl_scale * ghat, nhat, pend);
            pend_base = base;
        }
    }
    if constexpr (ROUNDTRIP) {
        if (pend_base >= 0) {
            const int l = lane_id();
            dense_out_put<OUT_F16>(pend, y, ldy_bytes, pend_base, n, l & 31, l >> 5);
        }
    }
}

template <int B, bool QJL, bool OUT_F16>
__global__ __launch_bounds__(256, 2) void tq_dequant_kernel(DenseDev P, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ norms,
                                                         const uint32_t* __restrict__ signs,
                                                         const uint16_t* __restrict__ rnorms, int64_t n,
                                                         char* __restrict__ y, int64_t ldy_bytes) {
    constexpr int LW = 2 * B;
    constexpr int W = 4 * B;
    constexpr int SW = 32 * W > 128 ? 32 * W : 128;
    struct Lds {
        uint2 ptab[1 << (2 * B)];   // centroid pair table
        uint32_t stage[4][SW];
    };
    __shared__ Lds lds;
    dense_tables_to_lds<B>(P, lds.ptab);
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t* stw = lds.stage[wave];
    const int64_t ntiles = (n + 31) / 32;
    // each tile's output is stored after the next tile's record has arrived
    OutWords<OUT_F16> pend;
    int64_t pend_base = -1;
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
        if (pend_base >= 0) dense_out_put<OUT_F16>(pend, y, ldy_bytes, pend_base, n, vi, h);
        f32x16 ax[4], aq[4];
        const GPair pg(P.pit2_hi, P.pit2_lo, l);
        dense_pit2<B>(pg, pg.load(0), lds.ptab, cw, ax);
        if constexpr (QJL) {
            const GOne sg(P.s_back, l);
            dense_back2(sg, sg.load(0), sw0, sw1, aq);
        }
        dense_out_words<QJL, OUT_F16>(ax, aq, P.qjl_scale * ghat, nhat, pend);
        pend_base = base;
    }
    if (pend_base >= 0) {
        const int l = lane_id();
        dense_out_put<OUT_F16>(pend, y, ldy_bytes, pend_base, n, l & 31, l >> 5);
    }
}

// ----------------------------------------------------------- launchers --
// fp16 input: eight-wave workgroups sharing one LDS copy of Pi (two waves
// per SIMD); fp32 input tiles need four waves' LDS.
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
        else TQ_LAUNCH(true, false, true, 8);
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
