// Building blocks of the RotorQuant codec kernels (gfx950): the slot-table
// set-up, centroid pairs and rotor matrix products shared by the two-lanes-
// per-vector codec kernels (rq_rotor_codec_dev.h), and the one-lane-per-
// vector QJL helpers of the QJL-only kernels (rq_qjl1.hip).
//
// Per vector (RotorQuant README, "The Fused CUDA Kernel"): groups of three
// coordinates go through y_g = M_g v_g, M_g the 3x3 matrix of the sandwich
// (R v) R~, and back through x~_g = M_g^T c[code].  QJL (README Stage 2;
// blog QJL section; hyper.ai Algorithm 2): sign bits of S r and the
// back-projection sqrt(pi/2)/m * gamma * S^T sigma.
//
// One-lane-per-vector QJL layout: 64 vectors per wave, S r on 32x32x16
// MFMAs over the tile's two 32-vector halves, with the rows of S permuted
// on the host so that each lane's accumulators hold 16 consecutive sign
// indices of one vector; sign words are then a chain of v_alignbit on the
// accumulator sign bits.
#pragma once

#include "rq_common_dev.h"
#include "rq_rotor_decl.h"

namespace rqk {

// Working domain of the QJL kernels: every unit-domain quantity (normalised
// input, rotated coordinates, boundaries, centroids, reconstruction,
// residual) is carried times 2^12.  The scaling is exact, leaves every
// comparison and rounding unchanged, and keeps the residual's low half a
// normal half for the MFMA.  The MSE-only kernels work at scale 1.
constexpr float kQjlDomain = 4096.0f;

template <int B>
constexpr int code_words(int coords) { return (coords * B + 31) / 32; }


// -------------------------------------------------------------- set-up --
template <bool QJL, int NT = kBlock>
__device__ __forceinline__ void stage_bins(const u32x4_t* __restrict__ g, u32x4* __restrict__ s) {
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    const u32x4* src = reinterpret_cast<const u32x4*>(g);
    for (int i = threadIdx.x; i < kBinSlots; i += NT) {
        const u32x4 e = src[i];
        const uint32_t e0 = e[0], e1 = e[1], e2 = e[2], e3 = e[3];
        s[i] = u32x4{e0, __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, e1) * D),
                     __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, e2) * D),
                     __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, e3) * D)};
    }
}

// Centroid pairs indexed by two adjacent codes of the bit stream.
template <int B, bool QJL>
__device__ __forceinline__ void stage_pairs(const float* __restrict__ cent, f32x2* __restrict__ pairs) {
    constexpr int L = 1 << B;
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    for (int p = threadIdx.x; p < L * L; p += kBlock) pairs[p] = f32x2{cent[p & (L - 1)] * D, cent[p >> B] * D};
}

// ------------------------------------------------------------ per lane --
// Centroids of codes 2p and 2p + 1.
template <int B, int W>
__device__ __forceinline__ f32x2 pair_vals(const uint32_t (&cw)[W], int p, const f32x2* __restrict__ pairs) {
    constexpr uint32_t mask = (1u << (2 * B)) - 1u;
    const int bit = 2 * B * p, wi = bit >> 5, off = bit & 31;
    uint32_t f;
    if (off + 2 * B <= 32 || wi + 1 >= W) f = cw[wi] >> off;
    else f = __builtin_amdgcn_alignbit(cw[wi + 1], cw[wi], off);
    return pairs[f & mask];
}

template <bool IN_F16>
__device__ __forceinline__ void load_vec(const char* __restrict__ x, int64_t ld_bytes, int64_t base, int64_t n,
                                         u32x4* __restrict__ t, int l, float (&v)[kD]) {
    if constexpr (IN_F16) {
        tile_load(x, ld_bytes, base, n, 0, t, l);
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const u32x4 q = t[swz(l, c)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = q[e];
                v[8 * c + 2 * e] = h2f(w & 0xFFFFu);
                v[8 * c + 2 * e + 1] = h2f(w >> 16);
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            tile_load(x, ld_bytes, base, n, 256 * h, t, l);
            wave_lds_sync();
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const u32x4 q = t[swz(l, c)];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = q[e];
                    v[64 * h + 4 * c + e] = __builtin_bit_cast(float, w);
                }
            }
        }
    }
}

// y_g = M_g v (forward sandwich as a matrix), x~_g = M_g^T yh (inverse).
__device__ __forceinline__ void rot_fwd(const float* __restrict__ m, const float v[3], float y[3]) {
#pragma unroll
    for (int r = 0; r < 3; ++r) y[r] = __builtin_fmaf(m[3 * r + 2], v[2], __builtin_fmaf(m[3 * r + 1], v[1], m[3 * r] * v[0]));
}
__device__ __forceinline__ void rot_inv(const float* __restrict__ m, const float yh[3], float x[3]) {
#pragma unroll
    for (int j = 0; j < 3; ++j) x[j] = __builtin_fmaf(m[6 + j], yh[2], __builtin_fmaf(m[3 + j], yh[1], m[j] * yh[0]));
}

// ---------------------------------------------------------------- QJL --
// Four MFMAs of K block kb against 32-row M tile mt of the permuted S, for
// the tile's two 32-vector halves; hi then lo of the residual.
__device__ __forceinline__ void issue_fwd(const u32x4* __restrict__ sf, f32x16 (&acc)[2], int kb, int mt,
                                          const u32x4& h0, const u32x4& h1, const u32x4& l0, const u32x4& l1,
                                          int l) {
    const u32x4 a = mat_frag(sf, 32 * mt + (l & 31), 2 * kb + (l >> 5));
    acc[0] = mfma(a, h0, acc[0]);
    acc[0] = mfma(a, l0, acc[0]);
    acc[1] = mfma(a, h1, acc[1]);
    acc[1] = mfma(a, l1, acc[1]);
}

// +-1 halves (sign of z_a, sign of z_b): +1 for z >= 0.  An accumulator that
// starts at +0 never ends at -0, so the sign bit is exactly [z < 0].
__device__ __forceinline__ uint32_t sigma_pair(float za, float zb) {
    const uint32_t t = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, zb), __builtin_bit_cast(uint32_t, za),
                                             0x070C030Cu);
    return (t & 0x80008000u) | 0x3C003C00u;
}

// Sign words of the own vector from the S r accumulators (bit j = [z_j >= 0]),
// and with BACK the +-1 operands of S^T sigma for both vector halves.
template <bool BACK>
__device__ __forceinline__ void sign_chain(const f32x16 (&za)[4][2], uint32_t (&sw)[4],
                                           u32x4 (&sig)[BACK ? 2 : 1][8], int l) {
    const uint32_t sel = (l >> 5) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float z0[16], z1[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e0 = za[mt][0][r];
            const float e1 = za[mt][1][r];
            z0[r] = e0;
            z1[r] = e1;
        }
        // sign bits: z1 of M tile rows 15..0 into bits 31..16, z0 into 15..0
        uint32_t pb = 0u;
#pragma unroll
        for (int r = 15; r >= 0; --r) pb = __builtin_amdgcn_alignbit(pb, __builtin_bit_cast(uint32_t, z1[r]), 31);
#pragma unroll
        for (int r = 15; r >= 0; --r) pb = __builtin_amdgcn_alignbit(pb, __builtin_bit_cast(uint32_t, z0[r]), 31);
        const auto sp = __builtin_amdgcn_permlane32_swap(pb, pb, false, false);
        const uint32_t p0 = sp[0], p1 = sp[1];
        sw[mt] = ~__builtin_amdgcn_perm(p1, p0, sel);
        if constexpr (BACK) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sig[0][2 * mt + c][q] = sigma_pair(z0[8 * c + 2 * q], z0[8 * c + 2 * q + 1]);
                    sig[1][2 * mt + c][q] = sigma_pair(z1[8 * c + 2 * q], z1[8 * c + 2 * q + 1]);
                }
        }
    }
}

// 16 sign bits (bit e = [z_e >= 0]) -> eight dwords of +-1 half pairs,
// dword q = (sigma_2q, sigma_2q+1): the same values sigma_pair gives.
__device__ __forceinline__ void sigma16(uint32_t bits16, u32x4& d0, u32x4& d1) {
    const uint32_t nb = ~bits16;
    const uint32_t u = (nb & 0x5555u) | ((nb & 0xAAAAu) << 15);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        d0[q] = ((u << (15 - 2 * q)) & 0x80008000u) | 0x3C003C00u;
        d1[q] = ((u << (7 - 2 * q)) & 0x80008000u) | 0x3C003C00u;
    }
}

// sigma operands (B side of S^T sigma) of the tile's two vector halves, from
// the record's sign words of vectors l % 32 and 32 + l % 32.
__device__ __forceinline__ void sigma_from_words(const u32x4 (&wv)[2], u32x4 (&sig)[2][8], int l) {
    const int sh = 16 * (l >> 5);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint32_t w = wv[nt][mt];
            sigma16((w >> sh) & 0xFFFFu, sig[nt][2 * mt], sig[nt][2 * mt + 1]);
        }
}

// Reconstruction with the QJL term: out_j = n^ (x~_j + k (S^T sigma)_j),
// evaluated as (n^ / D) * fma(k D, u_j, D x~_j).  xt holds D x~ (own vector).
// done(mt) runs once the outputs of M tile mt (coordinates 32 mt ..) are set.
template <class Out, class Done>
__device__ __forceinline__ void back_out(const u32x4* __restrict__ sb, const u32x4 (&sig)[2][8], float kq, float ns,
                                         const float (&xt)[kD], Out& out, int l, Done done) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        f32x16 a0 = {}, a1 = {};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const u32x4 a = mat_frag(sb, 32 * mt + (l & 31), 2 * kb + (l >> 5));
            a0 = mfma(a, sig[0][kb], a0);
            a1 = mfma(a, sig[1][kb], a1);
        }
        float u0[16], u1[16];
        from_accumulators(a0, a1, u0, u1);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int j = 32 * mt + r;
            out.set2(j, ns * __builtin_fmaf(kq, u0[r], xt[j]), ns * __builtin_fmaf(kq, u0[r + 1], xt[j + 1]));
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int j = 32 * mt + 16 + r;
            out.set2(j, ns * __builtin_fmaf(kq, u1[r], xt[j]), ns * __builtin_fmaf(kq, u1[r + 1], xt[j + 1]));
        }
        done(mt);
    }
}
template <class Out>
__device__ __forceinline__ void back_out(const u32x4* __restrict__ sb, const u32x4 (&sig)[2][8], float kq, float ns,
                                         const float (&xt)[kD], Out& out, int l) {
    back_out(sb, sig, kq, ns, xt, out, l, [](int) {});
}

// Record sign words of vectors l % 32 and 32 + l % 32 (through LDS).
__device__ __forceinline__ void load_sign_pairs(const uint32_t* __restrict__ src, int64_t base, int64_t n,
                                                u32x4 (&wv)[2], uint32_t* __restrict__ stage, int l) {
    const rsrc_t rs = make_rsrc(src + base * 4, tile_range(n - base, 16));
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 4; ++it)
        stage[it * 64 + l] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    wave_lds_sync();
    const u32x4* s4 = reinterpret_cast<const u32x4*>(stage);
    wv[0] = s4[l & 31];
    wv[1] = s4[32 + (l & 31)];
    wave_lds_sync();
}

// ------------------------------------------------------------ kernels --
// Input vector in registers: fp16 kept as packed pairs (converted per use),
// fp32 as floats.
template <bool IN_F16>
struct VecIn;

template <>
struct VecIn<true> {
    uint32_t h[kD / 2];
    __device__ float get(int i) const { return h2f((i & 1) ? (h[i >> 1] >> 16) : (h[i >> 1] & 0xFFFFu)); }
    __device__ void load(const char* x, int64_t ld_bytes, int64_t base, int64_t n, u32x4* t, int l) {
        tile_load(x, ld_bytes, base, n, 0, t, l);
        own_row(t, l);
    }
    // own row of a tile already in LDS
    __device__ void own_row(const u32x4* t, int l) {
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const u32x4 q = t[swz(l, c)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = q[e];
                h[4 * c + e] = w;
            }
        }
    }
};

template <>
struct VecIn<false> {
    float v[kD];
    __device__ float get(int i) const { return v[i]; }
    __device__ void load(const char* x, int64_t ld_bytes, int64_t base, int64_t n, u32x4* t, int l) {
        load_vec<false>(x, ld_bytes, base, n, t, l, v);
    }
};

// ----------------------------------------------------------- launchers --
inline int grid_for(int64_t n, int per_cu) {
    const int64_t ntiles = (n + 63) / 64;
    const int64_t blocks = (ntiles + 3) / 4;
    const int64_t cap = 256LL * per_cu * 4;
    return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace rqk
