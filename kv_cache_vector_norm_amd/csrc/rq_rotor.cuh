// RotorQuant codec kernels for gfx950 (templates; instantiated per bit width
// and mode in rq_rotor_inst.hip): quantize, dequantize and the fused
// roundtrip, MSE-only or with the QJL residual stage.
//
// Per vector (RotorQuant README, "The Fused CUDA Kernel" and "RotorQuant
// Fused Kernels": normalize -> embed -> rotor sandwich -> quantize ->
// inverse sandwich -> extract -> rescale):
//   n = ||x||, x_u = x / n; groups v_g = (x_u[3g], x_u[3g+1], x_u[3g+2]) with
//   a zero pad; y_g = M_g v_g, M_g the 3x3 matrix of the sandwich (R v) R~
//   (README "Non-Commutative Algebra Bug Fix"); code = #{k : y > t_k};
//   dequant x~_g = M_g^T c[code] (the inverse sandwich (R~ v) R).
// QJL (README Stage 2; blog QJL section; hyper.ai Algorithm 2):
//   r = x_u - x~_u, gamma = ||r||, sign bits of S r; dequant adds
//   sqrt(pi/2)/m * gamma * S^T sigma.
// The rotor matrices and codebook are wave-uniform (scalar loads); S and S^T
// are half matrices in LDS feeding 32x32x16 MFMAs; the residual enters the
// MFMA as an exact hi + lo pair of halves (scaled by 2^12), S being exactly
// representable in half.
#pragma once

#include "rq_common.cuh"
#include "rq_rotor_decl.h"

namespace rqk {


// The 43 rotor matrices (387 wave-uniform floats, more than the SGPR file
// holds) are staged in LDS once per workgroup and read per group with
// broadcast DS reads; their address is offset by an opaque zero made inside
// each loop iteration, so they are not all hoisted into registers.
constexpr float kResidualScale = 4096.0f;   // 2^12: keeps the residual's lo half normal

template <int B>
constexpr int code_words(int coords) { return (coords * B + 31) / 32; }

// 8 sign bits -> eight halves +-1 (bit 1 -> +1), packed in pairs.
__device__ __forceinline__ u32x4 sigma8(uint32_t byte) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t b0 = (byte >> (2 * p)) & 1u, b1 = (byte >> (2 * p + 1)) & 1u;
        r[p] = 0xBC00BC00u ^ (b0 << 15) ^ (b1 << 31);
    }
    return r;
}

// -------------------------------------------------------------- inputs --
// The vector's coordinates are read once from the LDS tile into registers
// (fp16: 16 chunks of 8 halves; fp32: 128 floats in two 256-byte passes).
template <bool IN_F16>
struct VecIn;

template <>
struct VecIn<true> {
    u32x4 ch[16];
    __device__ float get(int i) const {
        const uint32_t w = ch[i >> 3][(i & 7) >> 1];
        return h2f((i & 1) ? (w >> 16) : (w & 0xFFFFu));
    }
    __device__ void load(const char* x, int64_t ld_bytes, int64_t base, int64_t n, u32x4* t, int l) {
        tile_load(x, ld_bytes, base, n, 0, t, l);
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < 16; ++c) ch[c] = t[swz(l, c)];
    }
    // Separates two passes over the coordinates: the second pass converts
    // again instead of keeping all 128 converted floats of the first alive.
    __device__ void fence() {
#pragma unroll
        for (int c = 0; c < 16; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) pin_lane(ch[c], e);
    }
};

template <>
struct VecIn<false> {
    float v[kD];
    __device__ float get(int i) const { return v[i]; }
    __device__ void fence() {}
    __device__ void load(const char* x, int64_t ld_bytes, int64_t base, int64_t n, u32x4* t, int l) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            tile_load(x, ld_bytes, base, n, 256 * h, t, l);
            wave_lds_sync();
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const u32x4 q = t[swz(l, c)];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t qe = q[e];
                    v[64 * h + 4 * c + e] = __builtin_bit_cast(float, qe);
                }
            }
        }
    }
};

// ----------------------------------------------------- shared stages --
// y_g = M_g v (forward sandwich as a matrix), x~_g = M_g^T yh (inverse).
__device__ __forceinline__ void rot_fwd(const float* __restrict__ m, const float v[3], float y[3]) {
#pragma unroll
    for (int r = 0; r < 3; ++r) y[r] = __builtin_fmaf(m[3 * r + 2], v[2], __builtin_fmaf(m[3 * r + 1], v[1], m[3 * r] * v[0]));
}
__device__ __forceinline__ void rot_inv(const float* __restrict__ m, const float yh[3], float x[3]) {
#pragma unroll
    for (int j = 0; j < 3; ++j) x[j] = __builtin_fmaf(m[6 + j], yh[2], __builtin_fmaf(m[3 + j], yh[1], m[j] * yh[0]));
}

// QJL term of dequantisation for one 32-coordinate M tile: q0/q1 receive
// (S^T sigma)_i of this lane's own vector for i = 32 mt + own_row(h, r).
template <int MT>
__device__ __forceinline__ void qjl_back_tile(const u32x4* __restrict__ st, const uint32_t (&sw)[4], float (&q0)[16],
                                              float (&q1)[16], int l) {
    f32x16 a0 = {}, a1 = {};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const uint32_t word = sw[kb >> 1] >> (16 * (kb & 1));
        u32x4 op0, op1;
        to_operands(sigma8(word & 0xFFu), sigma8((word >> 8) & 0xFFu), &op0, &op1);
        const u32x4 a = mat_frag(st, 32 * MT + (l & 31), 2 * kb + (l >> 5));
        a0 = mfma(a, op0, a0);
        a1 = mfma(a, op1, a1);
    }
    from_accumulators(a0, a1, q0, q1);
}

__device__ __forceinline__ float own_pick(const float (&q0)[16], const float (&q1)[16], int il) {
    // il in [0, 32): row 8b + w; w < 4 -> q0[4b + w], else q1[4b + w - 4]
    const int b = il >> 3, w = il & 7;
    return w < 4 ? q0[4 * b + w] : q1[4 * b + w - 4];
}

// Dequantise one vector from its record into `out` (unit-domain MSE part,
// plus the QJL term, times the stored norm).
template <int B, bool QJL, int W, class Out>
__device__ __forceinline__ void dequant_vec(const RotorDev& P, const float* __restrict__ lut,
                                            const u32x4* __restrict__ st, const uint32_t (&cw)[W], float nhat,
                                            float ghat, const uint32_t (&sw)[4], Out& out, int l) {
    if constexpr (!QJL) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            float yh[3], xt[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) yh[r] = lut[get_code<B, W>(cw, 3 * g + r)];
            rot_inv(P.rotmat + 9 * g, yh, xt);
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (3 * g + j < kD) out.set(3 * g + j, nhat * xt[j]);
        }
    } else {
        const float k = P.qjl_scale * ghat;
        auto tile = [&](auto mt_c) {
            constexpr int MT = decltype(mt_c)::value;
            float q0[16], q1[16];
            qjl_back_tile<MT>(st, sw, q0, q1, l);
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                if (3 * g + 2 < 32 * MT || 3 * g >= 32 * MT + 32) continue;
                __builtin_amdgcn_sched_barrier(0);
                float yh[3], xt[3];
#pragma unroll
                for (int r = 0; r < 3; ++r) yh[r] = lut[get_code<B, W>(cw, 3 * g + r)];
                rot_inv(P.rotmat + 9 * g, yh, xt);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int i = 3 * g + j;
                    if (i < kD && i >= 32 * MT && i < 32 * MT + 32)
                        out.set(i, nhat * __builtin_fmaf(k, own_pick(q0, q1, i - 32 * MT), xt[j]));
                }
            }
        };
        tile(std::integral_constant<int, 0>{});
        tile(std::integral_constant<int, 1>{});
        tile(std::integral_constant<int, 2>{});
        tile(std::integral_constant<int, 3>{});
    }
}

// ------------------------------------------------------------ kernels --
// LDS: one 16 KB transpose tile per wave, S (quantize side) and S^T
// (dequantize side) as needed, the centroid table.
template <int B, bool QJL, bool IN_F16, bool OUT_F16, bool ROUNDTRIP>
__global__ __launch_bounds__(256) void rq_quant_kernel(RotorDev P, const char* __restrict__ x, int64_t ldx_bytes,
                                                       int64_t n, uint32_t* __restrict__ codes,
                                                       uint16_t* __restrict__ norms, uint32_t* __restrict__ signs,
                                                       uint16_t* __restrict__ rnorms, char* __restrict__ y,
                                                       int64_t ldy_bytes) {
    constexpr int W = code_words<B>(kRotCoords);
    constexpr int L = 1 << B;
    __shared__ u32x4 tiles[4][kTileBytes / 16];
    __shared__ u32x4 s_rows[QJL ? 128 * 16 : 1];
    __shared__ u32x4 s_cols[(QJL && ROUNDTRIP) ? 128 * 16 : 1];
    __shared__ float lut[L];
    __shared__ float thr_lds[L];
    __shared__ float rot_lds[kGroups * 9];

    if (threadIdx.x < L) lut[threadIdx.x] = P.cent[threadIdx.x];
    if (threadIdx.x < L - 1) thr_lds[threadIdx.x] = P.thr[threadIdx.x];
    for (int i = threadIdx.x; i < kGroups * 9; i += blockDim.x) rot_lds[i] = P.rotmat[i];
    if constexpr (QJL) {
        mat_to_lds(P.s_rows, s_rows);
        if constexpr (ROUNDTRIP) mat_to_lds(P.s_cols, s_cols);
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    u32x4* tile = tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;

    for (int64_t t = blockIdx.x * 4LL + wave; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        RotorDev Q = P;
        Q.rotmat = rot_lds + z;
        float thr[L - 1];
#pragma unroll
        for (int k = 0; k < L - 1; ++k) thr[k] = uniform(thr_lds[k + z]);
        VecIn<IN_F16> in;
        in.load(x, ldx_bytes, base, n, tile, l);

        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
            const float v = in.get(i);
            ss = __builtin_fmaf(v, v, ss);
        }
        in.fence();
        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);

        uint32_t cw[W];
#pragma unroll
        for (int k = 0; k < W; ++k) cw[k] = 0u;
        uint32_t rh[QJL ? kD / 2 : 1], rl[QJL ? kD / 2 : 1];
        float gam2 = 0.0f;

#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            const float* m = Q.rotmat + 9 * g;
            float v[3], yv[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) v[j] = (3 * g + j < kD) ? in.get(3 * g + j) * inv : 0.0f;
            rot_fwd(m, v, yv);
            uint32_t code[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                code[r] = quant_code<B>(yv[r], thr);
                put_code<B, W>(cw, 3 * g + r, code[r]);
            }
            {
                const int w0 = (B * 3 * g) >> 5, w1 = (B * (3 * g + 2) + B - 1) >> 5;
#pragma unroll
                for (int k = 0; k < W; ++k)
                    if (k >= w0 && k <= w1) pin(cw[k]);
            }
            if constexpr (QJL) {
                float yh[3], xt[3];
#pragma unroll
                for (int r = 0; r < 3; ++r) yh[r] = lut[code[r]];
                rot_inv(m, yh, xt);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int i = 3 * g + j;
                    if (i >= kD) continue;
                    {
                        const float r = v[j] - xt[j];
                        gam2 = __builtin_fmaf(r, r, gam2);
                        uint32_t hi, lo;
                        split_h(r * kResidualScale, &hi, &lo);
                        if (i & 1) {
                            rh[i >> 1] |= hi << 16;
                            rl[i >> 1] |= lo << 16;
                            pin(rh[i >> 1]);
                            pin(rl[i >> 1]);
                            pin(gam2);
                        } else {
                            rh[i >> 1] = hi;
                            rl[i >> 1] = lo;
                        }
                    }
                }
            }
        }

        uint32_t sw[4] = {0u, 0u, 0u, 0u};
        float ghat = 0.0f;
        uint32_t gh = 0u;
        if constexpr (QJL) {
            const float gam = __builtin_sqrtf(gam2);
            gh = f2h(gam);
            ghat = h2f(gh);
            auto zt = [&](auto mt_c) {
                constexpr int MT = decltype(mt_c)::value;
                f32x16 a0 = {}, a1 = {};
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    const u32x4 a = mat_frag(s_rows, 32 * MT + (l & 31), 2 * kb + (l >> 5));
                    u32x4 h0, h1, l0, l1;
                    to_operands(u32x4{rh[8 * kb], rh[8 * kb + 1], rh[8 * kb + 2], rh[8 * kb + 3]},
                                u32x4{rh[8 * kb + 4], rh[8 * kb + 5], rh[8 * kb + 6], rh[8 * kb + 7]}, &h0, &h1);
                    to_operands(u32x4{rl[8 * kb], rl[8 * kb + 1], rl[8 * kb + 2], rl[8 * kb + 3]},
                                u32x4{rl[8 * kb + 4], rl[8 * kb + 5], rl[8 * kb + 6], rl[8 * kb + 7]}, &l0, &l1);
                    a0 = mfma(a, h0, a0);
                    a0 = mfma(a, l0, a0);
                    a1 = mfma(a, h1, a1);
                    a1 = mfma(a, l1, a1);
                }
                float z0[16], z1[16];
                from_accumulators(a0, a1, z0, z1);
                uint32_t word = 0u;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    word |= (z0[r] >= 0.0f ? 1u : 0u) << own_row(0, r);
                    word |= (z1[r] >= 0.0f ? 1u : 0u) << own_row(1, r);
                }
                sw[MT] = word;
            };
            zt(std::integral_constant<int, 0>{});
            zt(std::integral_constant<int, 1>{});
            zt(std::integral_constant<int, 2>{});
            zt(std::integral_constant<int, 3>{});
        }

        // record
        if (base + l < n) norms[base + l] = static_cast<uint16_t>(nh);
        words_store<W>(codes, base, n, cw, stage, l);
        if constexpr (QJL) {
            if (base + l < n) rnorms[base + l] = static_cast<uint16_t>(gh);
            words_store<4>(signs, base, n, sw, stage, l);
        }

        // The reconstruction is exactly what rq_dequant_kernel computes from
        // the record just written.
        if constexpr (ROUNDTRIP) {
            VecOutT<OUT_F16> out;
            if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
            out.begin(tile, l);
            dequant_vec<B, QJL, W>(Q, lut, s_cols, cw, nhat, ghat, sw, out, l);
            out.store(y, ldy_bytes, base, n);
        }
    }
}

template <int B, bool QJL, bool OUT_F16>
__global__ __launch_bounds__(256) void rq_dequant_kernel(RotorDev P, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ norms,
                                                         const uint32_t* __restrict__ signs,
                                                         const uint16_t* __restrict__ rnorms, int64_t n,
                                                         char* __restrict__ y, int64_t ldy_bytes) {
    constexpr int W = code_words<B>(kRotCoords);
    constexpr int L = 1 << B;
    __shared__ u32x4 tiles[4][kTileBytes / 16];
    __shared__ u32x4 s_cols[QJL ? 128 * 16 : 1];
    __shared__ float lut[L];
    __shared__ float rot_lds[kGroups * 9];
    if (threadIdx.x < L) lut[threadIdx.x] = P.cent[threadIdx.x];
    for (int i = threadIdx.x; i < kGroups * 9; i += blockDim.x) rot_lds[i] = P.rotmat[i];
    if constexpr (QJL) mat_to_lds(P.s_cols, s_cols);
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    u32x4* tile = tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
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
        RotorDev Q = P;
        Q.rotmat = rot_lds + z;
        dequant_vec<B, QJL, W>(Q, lut, s_cols, cw, nhat, ghat, sw, out, l);
        out.store(y, ldy_bytes, base, n);
    }
}

// ----------------------------------------------------------- launchers --
inline int grid_for(int64_t n, int per_cu) {
    const int64_t ntiles = (n + 63) / 64;
    const int64_t blocks = (ntiles + 3) / 4;
    const int64_t cap = 256LL * per_cu * 4;
    return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

template <int B, bool QJL>
hipError_t launch_quant_b(const RotorDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                                 uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y,
                                 bool out_f16, int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    const int grid = grid_for(n, QJL ? 1 : 2);
    const char* xc = static_cast<const char*>(x);
    char* yc = static_cast<char*>(y);
#define RQ_LAUNCH(IF, OF, RT)                                                                                     \
    hipLaunchKernelGGL((rq_quant_kernel<B, QJL, IF, OF, RT>), dim3(grid), dim3(256), 0, s, P, xc, ldx_bytes, n, \
                       codes, norms, signs, rnorms, yc, ldy_bytes)
    if (!roundtrip) {
        if (in_f16) RQ_LAUNCH(true, true, false); else RQ_LAUNCH(false, true, false);
    } else if (in_f16) {
        if (out_f16) RQ_LAUNCH(true, true, true); else RQ_LAUNCH(true, false, true);
    } else {
        if (out_f16) RQ_LAUNCH(false, true, true); else RQ_LAUNCH(false, false, true);
    }
#undef RQ_LAUNCH
    return hipGetLastError();
}

template <int B, bool QJL>
hipError_t launch_dequant_b(const RotorDev& P, const uint32_t* codes, const uint16_t* norms,
                                   const uint32_t* signs, const uint16_t* rnorms, int64_t n, void* y, bool out_f16,
                                   int64_t ldy_bytes, hipStream_t s) {
    const int grid = grid_for(n, QJL ? 1 : 2);
    char* yc = static_cast<char*>(y);
    if (out_f16)
        hipLaunchKernelGGL((rq_dequant_kernel<B, QJL, true>), dim3(grid), dim3(256), 0, s, P, codes, norms, signs,
                           rnorms, n, yc, ldy_bytes);
    else
        hipLaunchKernelGGL((rq_dequant_kernel<B, QJL, false>), dim3(grid), dim3(256), 0, s, P, codes, norms, signs,
                           rnorms, n, yc, ldy_bytes);
    return hipGetLastError();
}

}  // namespace rqk
