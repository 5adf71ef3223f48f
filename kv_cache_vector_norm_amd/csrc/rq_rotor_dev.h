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
//
// Mapping: one lane per vector, 64 vectors per wave.  The code of a
// coordinate and its centroid come from one 16-byte lookup (slot from one
// fma, then one compare against the boundary inside the slot).  S r runs on
// 32x32x16 MFMAs issued while the group loop goes on: each 16-coordinate K
// block of the residual (an exact hi + lo half pair) is multiplied as soon as
// it is complete.  The rows of S are permuted on the host so that each lane's
// accumulator holds 16 consecutive sign indices of one vector; sign words are
// then a chain of v_alignbit on the accumulator sign bits, and the +-1
// operands of S^T sigma come straight from the accumulators.
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

// Group in which coordinate 16 kb + 15 (the end of K block kb) is produced,
// and the K block whose MFMAs are issued during group g (one 32-row M tile
// per group, in the four groups after the block completes).
__host__ __device__ constexpr int kb_done(int kb) { return (16 * kb + 15) / 3; }
__host__ __device__ constexpr int pending_kb(int g) {
    for (int kb = 0; kb < 7; ++kb)
        if (g > kb_done(kb) && g <= kb_done(kb) + 4) return kb;
    return -1;
}
static_assert(kb_done(7) == kGroups - 1, "last K block ends in the last group");
static_assert(kb_done(1) - kb_done(0) > 4 && kb_done(4) - kb_done(3) > 4, "pending K blocks overlap");

// -------------------------------------------------------------- set-up --
template <bool QJL>
__device__ __forceinline__ void stage_bins(const u32x4_t* __restrict__ g, u32x4* __restrict__ s) {
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    const u32x4* src = reinterpret_cast<const u32x4*>(g);
    for (int i = threadIdx.x; i < kBinSlots; i += kBlock) {
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
// Code of y and its centroid (both in the working domain).
__device__ __forceinline__ uint32_t lut_quant(float y, float ba, float bb, const u32x4* __restrict__ bins,
                                              float* val) {
    const uint32_t off = __builtin_bit_cast(uint32_t, __builtin_fmaf(y, ba, bb)) & 0xFF0u;
    const u32x4 e = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(bins) + off);
    const uint32_t base = e[0], thr = e[1], lo = e[2], hi = e[3];
    const bool gt = y > __builtin_bit_cast(float, thr);
    *val = __builtin_bit_cast(float, gt ? hi : lo);
    return base + (gt ? 1u : 0u);
}

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

// S^T sigma of the own vector into u (coordinate order).
__device__ __forceinline__ void back_proj(const u32x4* __restrict__ sb, const u32x4 (&sig)[2][8], float (&u)[kD],
                                          int l) {
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
        for (int r = 0; r < 16; ++r) {
            u[32 * mt + r] = u0[r];
            u[32 * mt + 16 + r] = u1[r];
        }
    }
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

// Rotor matrices are read with scalar loads (constant address space) two
// groups ahead of use, from the padded table (one 64-byte line per group,
// so each group's nine floats come in two loads).  A scalar-cache miss costs an L2 round trip, far more
// than the two groups of lead, so every 64-byte line of the table is touched
// once per wave before the tile loop (the loads overlap the block's staging).
typedef __attribute__((address_space(4))) const float* cfloat_ptr;
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(4))) const f32x8* cf32x8_ptr;
// p: a group's 64-byte line of the padded table (32-byte aligned)
__device__ __forceinline__ void load_mat(cfloat_ptr p, float (&m)[9]) {
    const f32x8 v = *reinterpret_cast<cf32x8_ptr>(p);
#pragma unroll
    for (int k = 0; k < 8; ++k) m[k] = v[k];
    m[8] = p[8];
}
constexpr int kRotLines = kGroups;
struct RotWarm {
    uint32_t v[kRotLines];
};
// Issues one scalar load per line; finish() consumes them (one wait) later.
__device__ __forceinline__ void warm_rotor_table(cfloat_ptr p, RotWarm& w) {
#pragma unroll
    for (int i = 0; i < kRotLines; ++i) w.v[i] = __builtin_bit_cast(uint32_t, p[16 * i]);
}
__device__ __forceinline__ void warm_finish(const RotWarm& w) {
    uint32_t acc = 0u;
#pragma unroll
    for (int i = 0; i < kRotLines; ++i) acc ^= w.v[i];
    asm volatile("" ::"s"(acc));
}

// LDS: the slot table first (LDS address 0, so a slot's byte offset is its
// address), one 16 KB transpose tile per wave, and (QJL) the permuted S and
// S^T.  The group loop is software-pipelined: in group g's region the
// forward rotation and slot lookups of group g + 1 are issued before the
// compare / inverse / residual work of group g, so LDS latency hides behind
// a group of arithmetic; the rotor matrix of g + 2 is fetched there too.
template <int B, bool QJL, bool IN_F16, bool OUT_F16, bool ROUNDTRIP>
__global__ __launch_bounds__(256) void rq_quant_kernel(RotorDev P, const char* __restrict__ x, int64_t ldx_bytes,
                                                       int64_t n, uint32_t* __restrict__ codes,
                                                       uint16_t* __restrict__ norms, uint32_t* __restrict__ signs,
                                                       uint16_t* __restrict__ rnorms, char* __restrict__ y,
                                                       int64_t ldy_bytes) {
    constexpr int W = code_words<B>(kRotCoords);
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    constexpr bool BACK = QJL && ROUNDTRIP;
    // fp16 input of the next tile in flight during this one, where the
    // registers allow (not in the QJL roundtrip, which holds x~ as well)
    constexpr bool AHEAD = IN_F16 && !BACK;
    struct Lds {
        u32x4 bins[kBinSlots];
        u32x4 tiles[4][kTileBytes / 16];
        u32x4 s_fwd[QJL ? 128 * 16 : 1];
        u32x4 s_back[BACK ? 128 * 16 : 1];
    };
    __shared__ Lds lds;
    u32x4* bins = lds.bins;
    u32x4(*tiles)[kTileBytes / 16] = lds.tiles;
    u32x4* s_fwd = lds.s_fwd;
    u32x4* s_back = lds.s_back;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (n + 63) / 64;
    const int64_t t0 = blockIdx.x * 4LL + wave;
    // at most one tile per SIMD in the whole launch: no other wave can
    // overlap this one's stores, so the output leaves in quarters
    const bool single = ntiles <= kSimds;
    // the first tile's input is requested before the block's staging, so the
    // two latencies overlap
    TileRegs first;
    if constexpr (IN_F16) {
        if (t0 < ntiles) tile_fetch(x, ldx_bytes, t0 * 64, n, 0, first, lane_id());
    }
    // rotor table lines into the scalar cache, in flight with the staging
    RotWarm warm;
    warm_rotor_table(reinterpret_cast<cfloat_ptr>(reinterpret_cast<uintptr_t>(P.rotmat16)), warm);
    stage_bins<QJL>(P.bins, bins);
    if constexpr (QJL) mat_to_lds(P.s_fwd, s_fwd);
    if constexpr (BACK) mat_to_lds(P.s_back, s_back);
    __syncthreads();
    if constexpr (IN_F16) {
        if (t0 < ntiles) tile_put(first, tiles[wave], lane_id());
    }
    warm_finish(warm);

    const float ba = P.bin_a * (1.0f / D), bb = P.bin_b;
    u32x4* tile = tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const char* binc = reinterpret_cast<const char*>(bins);

    for (int64_t t = t0; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const cfloat_ptr rot = reinterpret_cast<cfloat_ptr>(reinterpret_cast<uintptr_t>(P.rotmat16)) + z;
        VecIn<IN_F16> in;
        if constexpr (AHEAD) {
            if (t != t0) tile_put(first, tile, l);
            in.own_row(tile, l);
            const int64_t tn = t + gridDim.x * 4LL;
            if (tn < ntiles) tile_fetch(x, ldx_bytes, tn * 64, n, 0, first, l);
        } else if constexpr (IN_F16) {
            if (t != t0) tile_load(x, ldx_bytes, base, n, 0, tile, l);
            in.own_row(tile, l);
        } else {
            in.load(x, ldx_bytes, base, n, tile, l);
        }
        // sum of squares: fp16 pairs through v_dot2_f32_f16 (exact products,
        // fp32 accumulation), fp32 input by fused multiply-adds
        float ss = 0.0f;
        if constexpr (IN_F16) {
#pragma unroll
            for (int i = 0; i < kD / 2; ++i) {
                const f16x2 h = __builtin_bit_cast(f16x2, in.h[i]);
                ss = __builtin_amdgcn_fdot2(h, h, ss, false);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                const float v = in.get(i);
                ss = __builtin_fmaf(v, v, ss);
            }
        }
        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);
        const float sc = inv * D;

        uint32_t cw[W];
#pragma unroll
        for (int k = 0; k < W; ++k) cw[k] = 0u;
        VecOutT<OUT_F16> out;
        if constexpr (ROUNDTRIP && !QJL) {
            if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
            out.begin(tile, l);
        }
        f32x16 za[QJL ? 4 : 1][2];
#pragma unroll
        for (int m = 0; m < (QJL ? 4 : 1); ++m) za[m][0] = za[m][1] = f32x16{};
        float xt[BACK ? kD : 1];
        float g2 = 0.0f, pend = 0.0f;
        uint32_t rh[8], rl[8];
        u32x4 oh0{}, oh1{}, ol0{}, ol1{}, frag{};

        // pipeline state: matrices of groups g, g+1, g+2 (ring of 3); the
        // inputs, rotated coordinates and table entries of groups g, g+1
        float mx[3][9];
        float va[2][3], ya[2][3];
        u32x4 ea[2][3];
        auto stage_a = [&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value;
            constexpr int s = g & 1;
            static_for<0, 3>([&](auto jc) __attribute__((always_inline)) {
                constexpr int i = 3 * g + decltype(jc)::value;
                // fma with +0 (one v_fma_mix on the fp16 input); differs from
                // x * sc only in the sign of a zero, which no step observes
                if constexpr (i < kD) va[s][i - 3 * g] = __builtin_fmaf(in.get(i), sc, 0.0f);
                else va[s][i - 3 * g] = 0.0f;
            });
            rot_fwd(mx[g % 3], va[s], ya[s]);
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const uint32_t off = __builtin_bit_cast(uint32_t, __builtin_fmaf(ya[s][r], ba, bb)) & 0xFF0u;
                ea[s][r] = *reinterpret_cast<const u32x4*>(binc + off);
            }
        };
        load_mat(rot, mx[0]);
        load_mat(rot + 16, mx[1]);
        stage_a(std::integral_constant<int, 0>{});

        static_for<0, kGroups>([&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value;
            constexpr int s = g & 1;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (QJL) {
                constexpr int kb = pending_kb(g);
                if constexpr (kb >= 0) {
                    constexpr int mt = g - kb_done(kb) - 1;
                    za[mt][0] = mfma(frag, oh0, za[mt][0]);
                    za[mt][0] = mfma(frag, ol0, za[mt][0]);
                    za[mt][1] = mfma(frag, oh1, za[mt][1]);
                    za[mt][1] = mfma(frag, ol1, za[mt][1]);
                }
            }
            if constexpr (g + 1 < kGroups) stage_a(std::integral_constant<int, g + 1>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (QJL) {
                constexpr int kb = pending_kb(g + 1);
                if constexpr (kb >= 0) {
                    constexpr int mt = g + 1 - kb_done(kb) - 1;
                    frag = mat_frag(s_fwd, 32 * mt + (l & 31), 2 * kb + (l >> 5));
                }
            }
            if constexpr (g + 2 < kGroups) load_mat(rot + 16 * (g + 2), mx[(g + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);

            // stage B of group g
            float yh[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const u32x4 e = ea[s][r];
                const uint32_t ebase = e[0], ethr = e[1], elo = e[2], ehi = e[3];
                const bool gt = ya[s][r] > __builtin_bit_cast(float, ethr);
                yh[r] = __builtin_bit_cast(float, gt ? ehi : elo);
                put_code<B, W>(cw, 3 * g + r, ebase + (gt ? 1u : 0u));
            }
            {
                constexpr int w0 = (B * 3 * g) >> 5, w1 = (B * (3 * g + 2) + B - 1) >> 5;
#pragma unroll
                for (int k = w0; k <= w1 && k < W; ++k) pin(cw[k]);
            }
            if constexpr (ROUNDTRIP || QJL) {
                float xo[3];
                rot_inv(mx[g % 3], yh, xo);
                static_for<0, 3>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    constexpr int i = 3 * g + j;
                    if constexpr (i < kD) {
                        if constexpr (!QJL) {
                            const float o = nhat * xo[j];
                            if constexpr (i & 1) out.set2(i - 1, pend, o);
                            else pend = o;
                        } else {
                            if constexpr (BACK) xt[i] = xo[j];
                            const float r = va[s][j] - xo[j];
                            g2 = __builtin_fmaf(r, r, g2);
                            if constexpr ((i & 1) == 0) {
                                pend = r;
                            } else {
                                constexpr int d = (i & 15) >> 1;
                                split_pair(pend, r, &rh[d], &rl[d]);
                                pin(rh[d]);
                                pin(rl[d]);
                                pin(g2);
                                if constexpr ((i & 15) == 15) {
                                    to_operands(u32x4{rh[0], rh[1], rh[2], rh[3]}, u32x4{rh[4], rh[5], rh[6], rh[7]},
                                                &oh0, &oh1);
                                    to_operands(u32x4{rl[0], rl[1], rl[2], rl[3]}, u32x4{rl[4], rl[5], rl[6], rl[7]},
                                                &ol0, &ol1);
                                }
                            }
                        }
                    }
                });
            }
            // When the launch has at most one tile per SIMD (small batches,
            // where nothing else overlaps the stores), fp16 output of the MSE roundtrip
            // leaves a quarter of each row at a time: coordinates 32 m ..
            // 32 m + 31 are complete after group (32 m + 31) / 3.  Larger
            // batches store whole rows, which HBM writes more efficiently.
            if constexpr (ROUNDTRIP && !QJL && OUT_F16) {
                if (single) {
                    if constexpr (g == 10) out.store_cols(y, ldy_bytes, base, n, 0);
                    if constexpr (g == 21) out.store_cols(y, ldy_bytes, base, n, 4);
                    if constexpr (g == 31) out.store_cols(y, ldy_bytes, base, n, 8);
                }
            }
        });

        if constexpr (ROUNDTRIP && !QJL) {      // frees the tile for the record
            if constexpr (OUT_F16) {
                if (single) out.store_cols(y, ldy_bytes, base, n, 12);
                else out.store(y, ldy_bytes, base, n);
            } else {
                out.store(y, ldy_bytes, base, n);
            }
        }

        uint32_t sw[4] = {0u, 0u, 0u, 0u};
        uint32_t gh = 0u;
        float ghat = 0.0f;
        u32x4 sig[BACK ? 2 : 1][8];
        if constexpr (QJL) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) issue_fwd(s_fwd, za[mt], 7, mt, oh0, oh1, ol0, ol1, l);
            const float gam = __builtin_sqrtf(g2) * (1.0f / D);
            gh = f2h(gam);
            ghat = h2f(gh);
            sign_chain<BACK>(za, sw, sig, l);
        }

        // record
        half_store(norms, base, n, nh, l);
        words_store<W>(codes, base, n, cw, stage, l);
        if constexpr (QJL) {
            half_store(rnorms, base, n, gh, l);
            words_store<4>(signs, base, n, sw, stage, l);
        }

        // The reconstruction is exactly what rq_dequant_kernel computes from
        // the record just written.
        if constexpr (BACK) {
            const float kq = (P.qjl_scale * ghat) * D;
            const float ns = nhat * (1.0f / D);
            VecOutT<OUT_F16> o2;
            if constexpr (!OUT_F16) o2.bind(y, ldy_bytes, base, n);
            o2.begin(tile, l);
            // with at most one tile per SIMD, fp16 rows leave a quarter at a
            // time, each while the next is computed; else whole rows
            back_out(s_back, sig, kq, ns, xt, o2, l, [&](int mt) {
                if constexpr (OUT_F16) {
                    if (single) o2.store_cols(y, ldy_bytes, base, n, 4 * mt);
                }
            });
            if (!OUT_F16 || !single) o2.store(y, ldy_bytes, base, n);
        }
    }
}

// Dequantisation: the centroid pairs of group g + 1 and its rotor matrix
// (both from LDS) are fetched in group g's region.
template <int B, bool QJL, bool OUT_F16>
__global__ __launch_bounds__(256) void rq_dequant_kernel(RotorDev P, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ norms,
                                                         const uint32_t* __restrict__ signs,
                                                         const uint16_t* __restrict__ rnorms, int64_t n,
                                                         char* __restrict__ y, int64_t ldy_bytes) {
    constexpr int W = code_words<B>(kRotCoords);
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    struct Lds {
        f32x2 pairs[1 << (2 * B)];
        float rot[kGroups * 9 + 1];
        u32x4 tiles[4][kTileBytes / 16];
        u32x4 s_back[QJL ? 128 * 16 : 1];
    };
    __shared__ Lds lds;
    f32x2* pairs = lds.pairs;
    float* rot_lds = lds.rot;
    u32x4(*tiles)[kTileBytes / 16] = lds.tiles;
    u32x4* s_back = lds.s_back;
    stage_pairs<B, QJL>(P.cent, pairs);
    for (int i = threadIdx.x; i < kGroups * 9; i += kBlock) rot_lds[i] = P.rotmat[i];
    if constexpr (QJL) mat_to_lds(P.s_back, s_back);
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* tile = tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
    for (int64_t t = blockIdx.x * 4LL + wave; t < ntiles; t += gridDim.x * 4LL) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const float* rot = rot_lds + z;
        uint32_t cw[W];
        words_load<W>(codes, base, n, cw, stage, l);
        const float nhat = h2f(half_load(norms, base, n, l));
        float u[QJL ? kD : 1];
        float kq = 0.0f, ns = nhat;
        if constexpr (QJL) {
            u32x4 wv[2];
            load_sign_pairs(signs, base, n, wv, stage, l);
            const float ghat = h2f(half_load(rnorms, base, n, l));
            u32x4 sig[2][8];
            sigma_from_words(wv, sig, l);
            back_proj(s_back, sig, u, l);
            kq = (P.qjl_scale * ghat) * D;
            ns = nhat * (1.0f / D);
        }
        VecOutT<OUT_F16> out;
        if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
        out.begin(tile, l);
        float pend = 0.0f;
        f32x2 pv[4];
        float mx[2][9];
        // pairs whose first code lies in group g
        auto fetch = [&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value;
            static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                constexpr int i = 3 * g + decltype(rc)::value;
                if constexpr ((i & 1) == 0) pv[(i >> 1) & 3] = pair_vals<B, W>(cw, i >> 1, pairs);
            });
#pragma unroll
            for (int k = 0; k < 9; ++k) mx[g & 1][k] = rot[9 * g + k];
        };
        fetch(std::integral_constant<int, 0>{});
        static_for<0, kGroups>([&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (g + 1 < kGroups) fetch(std::integral_constant<int, g + 1>{});
            __builtin_amdgcn_sched_barrier(0);
            float yh[3], xo[3];
            static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                constexpr int r = decltype(rc)::value;
                constexpr int i = 3 * g + r;
                const f32x2 q = pv[(i >> 1) & 3];
                const float a = q[0], b = q[1];
                yh[r] = (i & 1) ? b : a;
            });
            rot_inv(mx[g & 1], yh, xo);
            static_for<0, 3>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                constexpr int i = 3 * g + j;
                if constexpr (i < kD) {
                    float o;
                    if constexpr (QJL) o = ns * __builtin_fmaf(kq, u[i], xo[j]);
                    else o = nhat * xo[j];
                    if constexpr (i & 1) out.set2(i - 1, pend, o);
                    else pend = o;
                }
            });
        });
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
