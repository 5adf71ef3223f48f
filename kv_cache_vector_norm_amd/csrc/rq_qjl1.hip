// QJL-only codec (one bit per coordinate in total, no MSE stage): the
// residual of the QJL stage is the whole unit vector (blog's QJL demo with
// zero MSE bits: r = x, gamma = 1; README "CUDA Kernels" lists the 1-bit
// QJL quantiser and score kernels).  Record: fp16 norm, 128 sign bits of
// S x_u, fp16 gamma = ||x_u||.  Dequantisation: n^ sqrt(pi/2)/m gamma^ S^T sigma.
//
// Same machinery as the rotor QJL kernels (one lane per vector, S x_u on
// 32x32x16 fp16 MFMAs from exact hi/lo halves of x_u carried times 2^12,
// sign words from the accumulator sign bits, S^T sigma on MFMAs), without
// the group loop: every K block of the residual is ready after the norm.
//
// Outlier-channel separation (README "CUDA Kernels": the 1-bit QJL quantiser
// separates outliers): with OUTL, the k channels listed for a vector's head
// are read out of the LDS tile as exact halves, stored in the record's
// outlier array and cleared before the norm, so the sign sketch sees only
// the inlier part; dequantisation writes the stored values back over those
// channels after the reconstruction has left.
#include "rq_rotor_dev.h"

namespace rqk {

// Lane l's vector (row base + l) belongs to head (base + l) / head_rows;
// channel i of that head is chans[head * k + i] (masked to 0..127).
__device__ __forceinline__ uint32_t outlier_channel(const OutlierArgs& o, int64_t head, int i) {
    const rsrc_t rc = make_rsrc(o.chans, static_cast<uint32_t>(o.heads * o.k));
    return __builtin_amdgcn_raw_buffer_load_b8(rc, static_cast<uint32_t>(head * o.k + i), 0, 0) & 127u;
}

// fp16 tile in LDS: store this lane's outlier halves, then clear them.
__device__ __forceinline__ void outliers_take_f16(const OutlierArgs& o, int64_t base, int64_t n, u32x4* tile, int l) {
    const int64_t head = (base + l) / o.head_rows;
    const rsrc_t ro = make_rsrc(o.out + base * o.k, tile_range(n - base, 2 * o.k));
    char* t8 = reinterpret_cast<char*>(tile);
    for (int i = 0; i < o.k; ++i) {
        const uint32_t c = outlier_channel(o, head, i);
        uint16_t* p = reinterpret_cast<uint16_t*>(t8 + swz(l, static_cast<int>(c >> 3)) * 16 + (c & 7) * 2);
        const uint16_t v = *p;
        __builtin_amdgcn_raw_buffer_store_b16(v, ro, static_cast<uint32_t>(2 * (l * o.k + i)), 0, kNonTemporal);
        *p = 0;
    }
}

// fp32 input: half h of the row (coordinates 64 h .. 64 h + 63) is in LDS;
// its outlier values are stored as halves (round to nearest even), then cleared.
__device__ __forceinline__ void outliers_take_f32(const OutlierArgs& o, int64_t base, int64_t n, u32x4* tile, int l,
                                                  int h) {
    const int64_t head = (base + l) / o.head_rows;
    const rsrc_t ro = make_rsrc(o.out + base * o.k, tile_range(n - base, 2 * o.k));
    char* t8 = reinterpret_cast<char*>(tile);
    for (int i = 0; i < o.k; ++i) {
        const int c = static_cast<int>(outlier_channel(o, head, i)) - 64 * h;
        if (c < 0 || c >= 64) continue;
        float* p = reinterpret_cast<float*>(t8 + swz(l, c >> 2) * 16 + (c & 3) * 4);
        const float v = *p;
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(f2h(v)), ro, static_cast<uint32_t>(2 * (l * o.k + i)),
                                              0, kNonTemporal);
        *p = 0.0f;
    }
}

// After this wave's output rows have been stored: the stored outlier values
// over their channels (the wait orders them after the earlier stores).
template <bool OUT_F16>
__device__ __forceinline__ void outliers_put(const OutlierArgs& o, int64_t base, int64_t n, char* y, int64_t ldy_bytes,
                                             int l) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int64_t head = (base + l) / o.head_rows;
    const rsrc_t ri = make_rsrc(o.in + base * o.k, tile_range(n - base, 2 * o.k));
    const rsrc_t ry = make_rsrc(y + base * ldy_bytes, tile_range(n - base, ldy_bytes));
    for (int i = 0; i < o.k; ++i) {
        const uint32_t c = outlier_channel(o, head, i);
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(ri, static_cast<uint32_t>(2 * (l * o.k + i)), 0, 0);
        const uint32_t off = static_cast<uint32_t>(l * ldy_bytes);
        if constexpr (OUT_F16)
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v), ry, off + 2 * c, 0, kNonTemporal);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, h2f(v)), ry, off + 4 * c, 0,
                                                  kNonTemporal);
    }
}

template <bool IN_F16, bool OUT_F16, bool ROUNDTRIP, bool OUTL = false>
__global__ __launch_bounds__(256) void qjl1_quant_kernel(Qjl1Dev P, const char* __restrict__ x, int64_t ldx_bytes,
                                                         int64_t n, uint16_t* __restrict__ norms,
                                                         uint32_t* __restrict__ signs, uint16_t* __restrict__ rnorms,
                                                         char* __restrict__ y, int64_t ldy_bytes, OutlierArgs o) {
    static_assert(!(OUTL && ROUNDTRIP), "outlier sessions have no fused roundtrip");
    constexpr float D = kQjlDomain;
    struct Lds {
        u32x4 tiles[4][kTileBytes / 16];
        u32x4 s_fwd[128 * 16];
        u32x4 s_back[ROUNDTRIP ? 128 * 16 : 1];
    };
    __shared__ Lds lds;
    mat_to_lds(P.s_fwd, lds.s_fwd);
    if constexpr (ROUNDTRIP) mat_to_lds(P.s_back, lds.s_back);
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* tile = lds.tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
    const bool single = ntiles <= kSimds;   // at most one tile per SIMD: output leaves in quarters
    for (int64_t t = blockIdx.x * 4LL + wave; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 64;
        const int l = lane_id() + opaque_zero();
        VecIn<IN_F16> in;
        if constexpr (!OUTL) {
            in.load(x, ldx_bytes, base, n, tile, l);
        } else if constexpr (IN_F16) {
            tile_load(x, ldx_bytes, base, n, 0, tile, l);
            wave_lds_sync();
            outliers_take_f16(o, base, n, tile, l);
            in.own_row(tile, l);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                tile_load(x, ldx_bytes, base, n, 256 * h, tile, l);
                wave_lds_sync();
                outliers_take_f32(o, base, n, tile, l, h);
                wave_lds_sync();
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const u32x4 q = tile[swz(l, c)];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t w = q[e];
                        in.v[64 * h + 4 * c + e] = __builtin_bit_cast(float, w);
                    }
                }
            }
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
            const float v = in.get(i);
            ss = __builtin_fmaf(v, v, ss);
        }
        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);
        const float sc = inv * D;

        f32x16 za[4][2];
#pragma unroll
        for (int m = 0; m < 4; ++m) za[m][0] = za[m][1] = f32x16{};
        float g2 = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            uint32_t rh[8], rl[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int i = 16 * kb + 2 * d;
                const float a = __builtin_fmaf(in.get(i), sc, 0.0f);
                const float b = __builtin_fmaf(in.get(i + 1), sc, 0.0f);
                g2 = __builtin_fmaf(a, a, g2);
                g2 = __builtin_fmaf(b, b, g2);
                split_pair(a, b, &rh[d], &rl[d]);
            }
            u32x4 oh0, oh1, ol0, ol1;
            to_operands(u32x4{rh[0], rh[1], rh[2], rh[3]}, u32x4{rh[4], rh[5], rh[6], rh[7]}, &oh0, &oh1);
            to_operands(u32x4{rl[0], rl[1], rl[2], rl[3]}, u32x4{rl[4], rl[5], rl[6], rl[7]}, &ol0, &ol1);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) issue_fwd(lds.s_fwd, za[mt], kb, mt, oh0, oh1, ol0, ol1, l);
        }
        const float gam = __builtin_sqrtf(g2) * (1.0f / D);
        const uint32_t gh = f2h(gam);
        const float ghat = h2f(gh);
        uint32_t sw[4];
        u32x4 sig[ROUNDTRIP ? 2 : 1][8];
        sign_chain<ROUNDTRIP>(za, sw, sig, l);

        half_store(norms, base, n, nh, l);
        half_store(rnorms, base, n, gh, l);
        words_store<4>(signs, base, n, sw, stage, l);

        if constexpr (ROUNDTRIP) {
            const float zero[kD] = {};
            VecOutT<OUT_F16> out;
            if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
            out.begin(tile, l);
            back_out(lds.s_back, sig, (P.qjl_scale * ghat) * D, nhat * (1.0f / D), zero, out, l, [&](int mt) {
                if constexpr (OUT_F16) {
                    if (single) out.store_cols(y, ldy_bytes, base, n, 4 * mt);
                }
            });
            if (!OUT_F16 || !single) out.store(y, ldy_bytes, base, n);
        }
    }
}

template <bool OUT_F16, bool OUTL = false>
__global__ __launch_bounds__(256) void qjl1_dequant_kernel(Qjl1Dev P, const uint16_t* __restrict__ norms,
                                                           const uint32_t* __restrict__ signs,
                                                           const uint16_t* __restrict__ rnorms, int64_t n,
                                                           char* __restrict__ y, int64_t ldy_bytes, OutlierArgs o) {
    constexpr float D = kQjlDomain;
    struct Lds {
        u32x4 tiles[4][kTileBytes / 16];
        u32x4 s_back[128 * 16];
    };
    __shared__ Lds lds;
    mat_to_lds(P.s_back, lds.s_back);
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* tile = lds.tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
    const bool single = ntiles <= kSimds;   // at most one tile per SIMD: output leaves in quarters
    for (int64_t t = blockIdx.x * 4LL + wave; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 64;
        const int l = lane_id() + opaque_zero();
        u32x4 wv[2];
        load_sign_pairs(signs, base, n, wv, stage, l);
        const float nhat = h2f(half_load(norms, base, n, l));
        const float ghat = h2f(half_load(rnorms, base, n, l));
        u32x4 sig[2][8];
        sigma_from_words(wv, sig, l);
        const float zero[kD] = {};
        VecOutT<OUT_F16> out;
        if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
        out.begin(tile, l);
        back_out(lds.s_back, sig, (P.qjl_scale * ghat) * D, nhat * (1.0f / D), zero, out, l, [&](int mt) {
            if constexpr (OUT_F16) {
                if (single) out.store_cols(y, ldy_bytes, base, n, 4 * mt);
            }
        });
        if (!OUT_F16 || !single) out.store(y, ldy_bytes, base, n);
        if constexpr (OUTL) outliers_put<OUT_F16>(o, base, n, y, ldy_bytes, l);
    }
}

hipError_t qjl1_quantize(const Qjl1Dev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n, uint16_t* norms,
                         uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16, int64_t ldy_bytes, bool roundtrip,
                         hipStream_t s) {
    const int grid = grid_for(n, 1);
    const char* xc = static_cast<const char*>(x);
    char* yc = static_cast<char*>(y);
#define Q1_LAUNCH(IF, OF, RT)                                                                                  \
    hipLaunchKernelGGL((qjl1_quant_kernel<IF, OF, RT>), dim3(grid), dim3(256), 0, s, P, xc, ldx_bytes, n, norms, \
                       signs, rnorms, yc, ldy_bytes, OutlierArgs{})
    if (!roundtrip) {
        if (in_f16) Q1_LAUNCH(true, true, false); else Q1_LAUNCH(false, true, false);
    } else if (in_f16) {
        if (out_f16) Q1_LAUNCH(true, true, true); else Q1_LAUNCH(true, false, true);
    } else {
        if (out_f16) Q1_LAUNCH(false, true, true); else Q1_LAUNCH(false, false, true);
    }
#undef Q1_LAUNCH
    return hipGetLastError();
}

hipError_t qjl1_dequantize(const Qjl1Dev& P, const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms,
                           int64_t n, void* y, bool out_f16, int64_t ldy_bytes, hipStream_t s) {
    const int grid = grid_for(n, 1);
    char* yc = static_cast<char*>(y);
    if (out_f16)
        hipLaunchKernelGGL((qjl1_dequant_kernel<true>), dim3(grid), dim3(256), 0, s, P, norms, signs, rnorms, n, yc,
                           ldy_bytes, OutlierArgs{});
    else
        hipLaunchKernelGGL((qjl1_dequant_kernel<false>), dim3(grid), dim3(256), 0, s, P, norms, signs, rnorms, n, yc,
                           ldy_bytes, OutlierArgs{});
    return hipGetLastError();
}

hipError_t qjl1_quantize_outliers(const Qjl1Dev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                                  uint16_t* norms, uint32_t* signs, uint16_t* rnorms, const OutlierArgs& o,
                                  hipStream_t s) {
    const int grid = grid_for(n, 1);
    const char* xc = static_cast<const char*>(x);
    if (in_f16)
        hipLaunchKernelGGL((qjl1_quant_kernel<true, true, false, true>), dim3(grid), dim3(256), 0, s, P, xc, ldx_bytes,
                           n, norms, signs, rnorms, nullptr, 0, o);
    else
        hipLaunchKernelGGL((qjl1_quant_kernel<false, true, false, true>), dim3(grid), dim3(256), 0, s, P, xc,
                           ldx_bytes, n, norms, signs, rnorms, nullptr, 0, o);
    return hipGetLastError();
}

hipError_t qjl1_dequantize_outliers(const Qjl1Dev& P, const uint16_t* norms, const uint32_t* signs,
                                    const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                                    const OutlierArgs& o, hipStream_t s) {
    const int grid = grid_for(n, 1);
    char* yc = static_cast<char*>(y);
    if (out_f16)
        hipLaunchKernelGGL((qjl1_dequant_kernel<true, true>), dim3(grid), dim3(256), 0, s, P, norms, signs, rnorms, n,
                           yc, ldy_bytes, o);
    else
        hipLaunchKernelGGL((qjl1_dequant_kernel<false, true>), dim3(grid), dim3(256), 0, s, P, norms, signs, rnorms,
                           n, yc, ldy_bytes, o);
    return hipGetLastError();
}

}  // namespace rqk
