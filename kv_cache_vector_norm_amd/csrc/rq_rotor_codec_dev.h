// RotorQuant codec kernels for gfx950, two lanes per vector (templates;
// instantiated per bit width and mode in rq_rotor_inst.hip): quantize,
// dequantize and the fused roundtrip, MSE-only or with the QJL residual stage.
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
// Mapping.  A wave owns a tile of 32 vectors; lanes v and v + 32 share
// vector v.  Lane half 0 runs groups 0..21 (coordinates 0..65) and half 1
// groups 22..42 (coordinates 66..127 and the pad slot 128) plus one idle
// step on a zero matrix, so both halves take the same 22 group steps with
// the same register indices: local slot j of half h is coordinate 66 h + j.
// Half the group chain per lane and 32-vector tiles let a wave take two or
// more tiles even at 65,536 vectors, and it overlaps the next tile's input
// fetch and the previous tile's stores with its arithmetic (with one tile
// per wave, every wave's load, arithmetic and store phases would run in
// lockstep across the chip).
//
// Data paths.  Tiles cross LDS in rows padded to 272 (fp16) or 528 (fp32)
// bytes: 16-byte chunks for the coalesced global transfers, and per-lane
// dword (fp16) or dword-pair (fp32) accesses from byte 132 h (264 h) of the
// row for the lane's slots.  Each half reads its own group's rotor matrix
// from LDS; the slot table is the one-lookup quantiser of the one-lane
// design.  Code words: each half packs its slots at local bit B j.  Half 1's
// stream starts at bit 66 B of the record, so its words are funnel-shifted
// by 66 B mod 32, and the record word both halves share is joined with one
// cross-half swap.
// QJL: S r runs on 32x32x16 MFMAs.  K block kb is slots 8 kb .. 8 kb + 7 of
// both halves (half 1's slots 62 and 63, which hold the pad and the idle
// step, carry half 0's slots 64 and 65), and S is permuted on the host so
// that half h's accumulators hold sign indices 64 h .. 64 h + 63 in order:
// sign words and the +-1 operands of S^T sigma come straight from them, and
// S^T sigma returns each half its own slots.
#pragma once

#include "rq_rotor_dev.h"
#include "rq_tile2_dev.h"

namespace rqk {

constexpr int kHalf1 = 66;                   // first coordinate of lane half 1
constexpr int kSteps = 22;                   // group steps per lane
constexpr int kSlots = 3 * kSteps;           // local slots per lane
constexpr int kRotStride = 12;               // floats per group in the LDS matrix table
constexpr int kRotGroups = kGroups + 1;      // + the idle step's zero matrix
// Per-wave record stage: the code words of a tile (with the slack the
// copies read past them), later the sign words in the same place.
template <int B>
constexpr int stage_words2() {
    return (32 * code_words<B>(kRotCoords) + 1 + 63) / 64 * 64;
}

template <bool F16>
constexpr int half_bytes2() { return F16 ? 2 * kHalf1 : 4 * kHalf1; }

template <int B>
struct CodeSplit {
    static constexpr int W = code_words<B>(kRotCoords);   // record words per vector
    static constexpr int L = (kSlots * B + 31) / 32;      // local words per lane
    static constexpr int J = kHalf1 * B / 32;             // record word shared by both halves
    static constexpr int S = kHalf1 * B % 32;             // bit of word J where half 1's stream starts
    static_assert(S != 0 && W == 2 * J + 1 && L == J + 1, "code word split");
    static_assert(stage_words2<B>() >= 128, "stage holds the sign words");
};

// Group step after which K block kb (slots 8 kb .. 8 kb + 7) is complete, and
// the MFMAs issued at step s: 2 kb + p for the M tiles 2 p and 2 p + 1 of K
// block kb, in the two steps after it completes; -1 for none.
__host__ __device__ constexpr int kb2_done(int kb) { return (8 * kb + 7) / 3; }
__host__ __device__ constexpr int mfma2_at(int s) {
    for (int kb = 0; kb < 7; ++kb) {
        if (s == kb2_done(kb) + 1) return 2 * kb;
        if (s == kb2_done(kb) + 2) return 2 * kb + 1;
    }
    return -1;
}
__host__ __device__ constexpr bool mfma2_schedule_ok() {
    for (int kb = 0; kb + 1 < 7; ++kb)
        if (kb2_done(kb + 1) - kb2_done(kb) < 2) return false;
    // operands of K block kb + 2 (same register set) start after kb's last use
    for (int kb = 0; kb + 2 < 8; ++kb)
        if ((8 * (kb + 2)) / 3 <= kb2_done(kb) + 2) return false;
    return kb2_done(7) == kSteps - 1;
}
static_assert(mfma2_schedule_ok(), "MFMA schedule of the group loop");

// The lane's 66 input slots (half 1's slots 62..65, the pad and the idle
// step, read as zero).
template <bool IN_F16>
struct Slots2;

template <>
struct Slots2<true> {
    uint32_t w[kSlots / 2];
    __device__ void read(const char* tile, int vi, int h) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(tile + vi * row_bytes2<true>() + half_bytes2<true>() * h);
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < kSlots / 2; ++k) w[k] = p[k];
        w[31] = h ? 0u : w[31];
        w[32] = h ? 0u : w[32];
        wave_lds_sync();
    }
    __device__ float get(int j) const { return h2f((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu)); }
    __device__ float sumsq() const {
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < kSlots / 2; ++k) {
            const f16x2 v = __builtin_bit_cast(f16x2, w[k]);
            ss = __builtin_amdgcn_fdot2(v, v, ss, false);
        }
        return ss;
    }
};

template <>
struct Slots2<false> {
    float v[kSlots];
    __device__ void read(const char* tile, int vi, int h) {
        const f32x2* p = reinterpret_cast<const f32x2*>(tile + vi * row_bytes2<false>() + half_bytes2<false>() * h);
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < kSlots / 2; ++k) {
            const f32x2 q = p[k];
            const float a = q[0], b = q[1];
            v[2 * k] = a;
            v[2 * k + 1] = b;
        }
#pragma unroll
        for (int j = 62; j < kSlots; ++j) v[j] = h ? 0.0f : v[j];
        wave_lds_sync();
    }
    __device__ float get(int j) const { return v[j]; }
    __device__ float sumsq() const {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) ss = __builtin_fmaf(v[j], v[j], ss);
        return ss;
    }
};

// Rotor matrices, 12 floats per group (the ninth to eleventh unused), and a
// zero matrix for half 1's idle step.
template <int NT>
__device__ __forceinline__ void stage_rot(const float* __restrict__ g, float* __restrict__ s) {
    for (int i = threadIdx.x; i < kRotGroups * kRotStride; i += NT) {
        const int grp = i / kRotStride, k = i - grp * kRotStride;
        s[i] = (grp < kGroups && k < 9) ? g[9 * grp + k] : 0.0f;
    }
}
__device__ __forceinline__ void load_mat2(const float* __restrict__ p, float (&m)[9]) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t ak = a[k];
        const uint32_t bk = b[k];
        m[k] = __builtin_bit_cast(float, ak);
        m[4 + k] = __builtin_bit_cast(float, bk);
    }
    m[8] = p[8];
}

// Record code words of the lane's vector from its local words (the half
// with the lower coordinates also stores the shared word J).
template <int B>
__device__ __forceinline__ void code_words_to_stage(const uint32_t (&cw)[CodeSplit<B>::L], uint32_t* __restrict__ st,
                                                    int vi, int h) {
    using C = CodeSplit<B>;
    const uint32_t from1 = other_half(cw[0] << C::S, h);
    uint32_t* row = st + vi * C::W + (h ? C::J + 1 : 0);
#pragma unroll
    for (int k = 0; k < C::J; ++k) {
        const uint32_t sh = __builtin_amdgcn_alignbit(cw[k + 1], cw[k], 32 - C::S);
        row[k] = h ? sh : cw[k];
    }
    if (h == 0) row[C::J] = cw[C::J] | from1;
}

// Local words of the lane's vector from the staged record words.
template <int B>
__device__ __forceinline__ void code_words_from_stage(const uint32_t* __restrict__ st, uint32_t (&cw)[CodeSplit<B>::L],
                                                      int vi, int h) {
    using C = CodeSplit<B>;
    const uint32_t* row = st + vi * C::W + (h ? C::J : 0);
    const uint32_t sh = h ? C::S : 0u;
#pragma unroll
    for (int k = 0; k < C::L; ++k) cw[k] = __builtin_amdgcn_alignbit(row[k + 1], row[k], sh);
}

// S^T sigma: four M tiles, K blocks in order (the quantiser's roundtrip and
// the dequantiser issue the same sequence).
__device__ __forceinline__ void back_proj2(const u32x4* __restrict__ sb, const u32x4 (&sig)[8], f32x16 (&acc)[4],
                                           int l, int h) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(mat_frag(sb, 32 * mt + (l & 31), 2 * kb + h), sig[kb], acc[mt]);
}

// out_j = ns * (x~_j + kq u_j) for the lane's 66 slots (u_j of slots 64, 65
// of half 0 from half 1's accumulators), written as pairs.
template <bool OUT_F16>
__device__ __forceinline__ void qjl_out2(const f32x16 (&acc)[4], const float (&xt)[kSlots], float kq, float ns,
                                         char* rowo, int h) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float u[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = acc[mt][r];
            u[r] = e;
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int j = 16 * mt + r;
            out_pair<OUT_F16>(rowo, j >> 1, ns * __builtin_fmaf(kq, u[r], xt[j]),
                              ns * __builtin_fmaf(kq, u[r + 1], xt[j + 1]));
        }
    }
    const float e14 = acc[3][14];
    const float e15 = acc[3][15];
    const float u64 = other_half(e14, h), u65 = other_half(e15, h);
    out_pair<OUT_F16>(rowo, 32, ns * __builtin_fmaf(kq, u64, xt[64]), ns * __builtin_fmaf(kq, u65, xt[65]));
}

// ------------------------------------------------------------ kernels --
// LDS: the slot table first (LDS address 0, so a slot's byte offset is its
// address), the rotor matrices, (QJL) the permuted S and S^T, one tile and
// one record stage per wave.  The group loop is software-pipelined: in step
// s's region the forward rotation and slot lookups of step s + 1 are issued
// before the compare / inverse / residual work of step s, and the matrix of
// step s + 2 is fetched there too.
template <int B, bool QJL, bool IN_F16, bool OUT_F16, bool ROUNDTRIP, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void rq_quant_kernel(RotorDev P, const char* __restrict__ x, int64_t ldx_bytes,
                                                       int64_t n, uint32_t* __restrict__ codes,
                                                       uint16_t* __restrict__ norms, uint32_t* __restrict__ signs,
                                                       uint16_t* __restrict__ rnorms, char* __restrict__ y,
                                                       int64_t ldy_bytes) {
    using C = CodeSplit<B>;
    constexpr int W = C::W, L = C::L;
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    constexpr bool BACK = QJL && ROUNDTRIP;
    constexpr int RBI = row_bytes2<IN_F16>(), RBO = row_bytes2<OUT_F16>();
    constexpr int TB = 32 * (RBI > RBO ? RBI : RBO);
    constexpr int NT = 64 * WAVES;
    struct Lds {
        u32x4 bins[kBinSlots];
        float rot[kRotGroups * kRotStride];
        u32x4 s_fwd[QJL ? 128 * 16 : 1];
        u32x4 s_back[BACK ? 128 * 16 : 1];
        u32x4 tiles[WAVES][TB / 16];
        uint32_t stage[WAVES][stage_words2<B>()];
    };
    __shared__ Lds lds;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (n + 31) / 32;
    const int64_t tstep = static_cast<int64_t>(gridDim.x) * WAVES;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * WAVES + wave;
    // fp16 input: each tile's fetch is issued one tile ahead (the first one
    // before the block's staging, so the two latencies overlap)
    Tile2Regs<true> nx;
    if constexpr (IN_F16) {
        if (t0 < ntiles) tile2_fetch<true>(x, ldx_bytes, t0 * 32, n, nx, lane_id());
    }
    stage_bins<QJL, NT>(P.bins, lds.bins);
    stage_rot<NT>(P.rotmat, lds.rot);
    if constexpr (QJL) mat_to_lds<NT>(P.s_fwd, lds.s_fwd);
    if constexpr (BACK) mat_to_lds<NT>(P.s_back, lds.s_back);
    __syncthreads();

    const float ba = P.bin_a * (1.0f / D), bb = P.bin_b;
    char* tile = reinterpret_cast<char*>(lds.tiles[wave]);
    uint32_t* stw = lds.stage[wave];
    const char* binc = reinterpret_cast<const char*>(lds.bins);

    for (int64_t t = t0; t < ntiles; t += tstep) {
        const int64_t base = t * 32;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int h = l >> 5, vi = l & 31;
        Slots2<IN_F16> in;
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
        // sum of squares of each half, then of the vector (the same sum, in
        // the same order, in both lanes)
        float ss = in.sumsq();
        ss = ss + other_half(ss, h);
        const float nrm = __builtin_sqrtf(ss);
        const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
        const uint32_t nh = f2h(nrm);
        const float nhat = h2f(nh);
        const float sc = inv * D;

        uint32_t cw[L];
#pragma unroll
        for (int k = 0; k < L; ++k) cw[k] = 0u;
        const float* rotp = lds.rot + kSteps * kRotStride * h + z;
        char* rowo = tile + vi * RBO + half_bytes2<OUT_F16>() * h;
        f32x16 za[QJL ? 4 : 1];
#pragma unroll
        for (int m = 0; m < (QJL ? 4 : 1); ++m) za[m] = f32x16{};
        float xt[BACK ? kSlots : 1];
        float g2 = 0.0f, pend = 0.0f;
        u32x4 oph[2] = {}, opl[2] = {}, fa[2] = {};
        uint32_t xh = 0u, xl = 0u;

        // pipeline state: matrices of steps s, s+1, s+2 (ring of 3); the
        // inputs, rotated coordinates and table entries of steps s, s+1
        float mx[3][9];
        float va[2][3], ya[2][3];
        u32x4 ea[2][3];
        auto stage_a = [&](auto sc_) __attribute__((always_inline)) {
            constexpr int s = decltype(sc_)::value;
            constexpr int p = s & 1;
#pragma unroll
            for (int r = 0; r < 3; ++r) va[p][r] = __builtin_fmaf(in.get(3 * s + r), sc, 0.0f);
            rot_fwd(mx[s % 3], va[p], ya[p]);
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const uint32_t off = __builtin_bit_cast(uint32_t, __builtin_fmaf(ya[p][r], ba, bb)) & 0xFF0u;
                ea[p][r] = *reinterpret_cast<const u32x4*>(binc + off);
            }
        };
        load_mat2(rotp, mx[0]);
        load_mat2(rotp + kRotStride, mx[1]);
        stage_a(std::integral_constant<int, 0>{});

        static_for<0, kSteps>([&](auto sc_) __attribute__((always_inline)) {
            constexpr int s = decltype(sc_)::value;
            constexpr int p = s & 1;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (QJL) {
                constexpr int q = mfma2_at(s);
                if constexpr (q >= 0) {
                    constexpr int kb = q >> 1, m0 = 2 * (q & 1);
                    za[m0] = mfma(fa[0], oph[kb & 1], za[m0]);
                    za[m0] = mfma(fa[0], opl[kb & 1], za[m0]);
                    za[m0 + 1] = mfma(fa[1], oph[kb & 1], za[m0 + 1]);
                    za[m0 + 1] = mfma(fa[1], opl[kb & 1], za[m0 + 1]);
                }
            }
            if constexpr (s + 1 < kSteps) stage_a(std::integral_constant<int, s + 1>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (QJL) {
                constexpr int q = mfma2_at(s + 1);
                if constexpr (q >= 0) {
                    constexpr int kb = q >> 1, m0 = 2 * (q & 1);
                    fa[0] = mat_frag(lds.s_fwd, 32 * m0 + (l & 31), 2 * kb + h);
                    fa[1] = mat_frag(lds.s_fwd, 32 * (m0 + 1) + (l & 31), 2 * kb + h);
                }
            }
            if constexpr (s + 2 < kSteps) load_mat2(rotp + (s + 2) * kRotStride, mx[(s + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);

            // stage B of step s
            float yh[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const u32x4 e = ea[p][r];
                const uint32_t ebase = e[0], ethr = e[1], elo = e[2], ehi = e[3];
                const bool gt = ya[p][r] > __builtin_bit_cast(float, ethr);
                yh[r] = __builtin_bit_cast(float, gt ? ehi : elo);
                uint32_t code = ebase + (gt ? 1u : 0u);
                if constexpr (s == kSteps - 1) code = h ? 0u : code;   // half 1's idle step
                put_code<B, L>(cw, 3 * s + r, code);
            }
            {
                constexpr int w0 = (B * 3 * s) >> 5, w1 = (B * (3 * s + 2) + B - 1) >> 5;
#pragma unroll
                for (int k = w0; k <= w1 && k < L; ++k) pin(cw[k]);
            }
            if constexpr (ROUNDTRIP || QJL) {
                float xo[3];
                rot_inv(mx[s % 3], yh, xo);
                static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                    constexpr int r = decltype(rc)::value;
                    constexpr int j = 3 * s + r;
                    if constexpr (!QJL) {
                        const float o = nhat * xo[r];
                        if constexpr (j & 1) out_pair<OUT_F16>(rowo, j >> 1, pend, o);
                        else pend = o;
                    } else {
                        if constexpr (BACK) xt[j] = xo[r];
                        float res = va[p][r] - xo[r];
                        if constexpr (j >= 62) res = h ? 0.0f : res;   // half 1: pad and idle slots
                        g2 = __builtin_fmaf(res, res, g2);
                        if constexpr ((j & 1) == 0) {
                            pend = res;
                        } else {
                            uint32_t hi, lo;
                            split_pair(pend, res, &hi, &lo);
                            pin(hi);
                            pin(lo);
                            pin(g2);
                            if constexpr (j < 64) {
                                constexpr int kb = j >> 3, dq = (j & 7) >> 1;
                                oph[kb & 1][dq] = hi;
                                opl[kb & 1][dq] = lo;
                            } else {
                                xh = hi;
                                xl = lo;
                            }
                        }
                    }
                });
            }
        });

        if constexpr (ROUNDTRIP && !QJL) tile2_store<OUT_F16>(y, ldy_bytes, base, n, tile, l);

        uint32_t sw0 = 0u, sw1 = 0u, gh = 0u;
        float ghat = 0.0f;
        u32x4 sig[BACK ? 8 : 1];
        if constexpr (QJL) {
            // K block 7: half 1's slots 62, 63 carry half 0's slots 64, 65
            const uint32_t oxh = other_half(xh, h), oxl = other_half(xl, h);
            const uint32_t h3 = oph[1][3], l3 = opl[1][3];
            oph[1][3] = h ? oxh : h3;
            opl[1][3] = h ? oxl : l3;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const u32x4 a = mat_frag(lds.s_fwd, 32 * mt + (l & 31), 14 + h);
                za[mt] = mfma(a, oph[1], za[mt]);
                za[mt] = mfma(a, opl[1], za[mt]);
            }
            const float g2t = g2 + other_half(g2, h);
            const float gam = __builtin_sqrtf(g2t) * (1.0f / D);
            gh = f2h(gam);
            ghat = h2f(gh);
            // sign words 2h, 2h+1: bit i of M tile pair (2w, 2w+1) = [z >= 0]
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
            if constexpr (BACK) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float a = za[mt][8 * c + 2 * q];
                            const float b = za[mt][8 * c + 2 * q + 1];
                            sig[2 * mt + c][q] = sigma_pair(a, b);
                        }
            }
        }

        // record
        half_store2(norms, base, n, nh, vi);
        wave_lds_sync();
        code_words_to_stage<B>(cw, stw, vi, h);
        words2_store<W>(codes, base, n, stw, l);
        if constexpr (QJL) {
            half_store2(rnorms, base, n, gh, vi);
            wave_lds_sync();   // the code words have left the stage
            stw[vi * 4 + 2 * h] = sw0;
            stw[vi * 4 + 2 * h + 1] = sw1;
            words2_store<4>(signs, base, n, stw, l);
        }

        // The reconstruction is exactly what rq_dequant_kernel computes from
        // the record just written.
        if constexpr (BACK) {
            const float kq = (P.qjl_scale * ghat) * D;
            const float ns = nhat * (1.0f / D);
            f32x16 acc[4];
            back_proj2(lds.s_back, sig, acc, l, h);
            wave_lds_sync();
            qjl_out2<OUT_F16>(acc, xt, kq, ns, rowo, h);
            tile2_store<OUT_F16>(y, ldy_bytes, base, n, tile, l);
        }
    }
}

// Dequantisation: the centroid pairs of step s + 1 and its matrix (both
// from LDS) are fetched in step s's region.
template <int B, bool QJL, bool OUT_F16>
__global__ __launch_bounds__(256) void rq_dequant_kernel(RotorDev P, const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ norms,
                                                         const uint32_t* __restrict__ signs,
                                                         const uint16_t* __restrict__ rnorms, int64_t n,
                                                         char* __restrict__ y, int64_t ldy_bytes) {
    using C = CodeSplit<B>;
    constexpr int W = C::W, L = C::L;
    constexpr float D = QJL ? kQjlDomain : 1.0f;
    constexpr int RBO = row_bytes2<OUT_F16>();
    struct Lds {
        f32x2 pairs[1 << (2 * B)];
        float rot[kRotGroups * kRotStride];
        u32x4 s_back[QJL ? 128 * 16 : 1];
        u32x4 tiles[4][32 * RBO / 16];
        uint32_t stage[4][stage_words2<B>()];
    };
    __shared__ Lds lds;
    stage_pairs<B, QJL>(P.cent, lds.pairs);
    stage_rot<kBlock>(P.rotmat, lds.rot);
    if constexpr (QJL) mat_to_lds(P.s_back, lds.s_back);
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
        const float* rotp = lds.rot + kSteps * kRotStride * h + z;
        words2_load<W>(codes, base, n, stw, l);
        uint32_t cw[L];
        code_words_from_stage<B>(stw, cw, vi, h);
        const float nhat = h2f(half_load2(norms, base, n, vi));
        float kq = 0.0f, ns = nhat;
        f32x16 acc[QJL ? 4 : 1];
        if constexpr (QJL) {
            words2_load<4>(signs, base, n, stw, l);   // the code words are in registers
            const uint32_t sw0 = stw[vi * 4 + 2 * h], sw1 = stw[vi * 4 + 2 * h + 1];
            const float ghat = h2f(half_load2(rnorms, base, n, vi));
            u32x4 sig[8];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint32_t w = mt < 2 ? sw0 : sw1;
                sigma16((w >> (16 * (mt & 1))) & 0xFFFFu, sig[2 * mt], sig[2 * mt + 1]);
            }
            back_proj2(lds.s_back, sig, acc, l, h);
            kq = (P.qjl_scale * ghat) * D;
            ns = nhat * (1.0f / D);
        }
        char* rowo = tile + vi * RBO + half_bytes2<OUT_F16>() * h;
        wave_lds_sync();
        float pend = 0.0f;
        f32x2 pv[4];
        float mx[2][9];
        // pairs whose first slot lies in step s
        auto fetch = [&](auto sc_) __attribute__((always_inline)) {
            constexpr int s = decltype(sc_)::value;
            static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                constexpr int j = 3 * s + decltype(rc)::value;
                if constexpr ((j & 1) == 0) pv[(j >> 1) & 3] = pair_vals<B, L>(cw, j >> 1, lds.pairs);
            });
            load_mat2(rotp + s * kRotStride, mx[s & 1]);
        };
        fetch(std::integral_constant<int, 0>{});
        static_for<0, kSteps>([&](auto sc_) __attribute__((always_inline)) {
            constexpr int s = decltype(sc_)::value;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (s + 1 < kSteps) fetch(std::integral_constant<int, s + 1>{});
            __builtin_amdgcn_sched_barrier(0);
            float yh[3], xo[3];
            static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                constexpr int r = decltype(rc)::value;
                constexpr int j = 3 * s + r;
                const f32x2 q = pv[(j >> 1) & 3];
                const float a = q[0], b = q[1];
                yh[r] = (j & 1) ? b : a;
            });
            rot_inv(mx[s & 1], yh, xo);
            static_for<0, 3>([&](auto rc) __attribute__((always_inline)) {
                constexpr int r = decltype(rc)::value;
                constexpr int j = 3 * s + r;
                float o;
                if constexpr (QJL) {
                    float u;
                    if constexpr (j < 64) {
                        const float e = acc[j >> 4][j & 15];
                        u = e;
                    } else {
                        const float e = acc[3][j - 50];   // slots 64, 65: half 1's elements 14, 15
                        u = other_half(e, h);
                    }
                    o = ns * __builtin_fmaf(kq, u, xo[r]);
                } else {
                    o = nhat * xo[r];
                }
                if constexpr (j & 1) out_pair<OUT_F16>(rowo, j >> 1, pend, o);
                else pend = o;
            });
        });
        tile2_store<OUT_F16>(y, ldy_bytes, base, n, tile, l);
    }
}

// ----------------------------------------------------------- launchers --
// Workgroups of `waves` waves, at most per_cu per compute unit in one round:
// every wave then loops over its tiles.
inline int grid2_for(int64_t n, int waves, int per_cu) {
    const int64_t ntiles = (n + 31) / 32;
    const int64_t blocks = (ntiles + waves - 1) / waves;
    const int64_t cap = 256LL * per_cu;
    return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

// Launch shapes: QJL kernels with fp16 input and output run eight waves per
// workgroup sharing one copy of S and S^T (two waves per SIMD); the other
// QJL shapes need four waves' LDS.  MSE-only kernels run four-wave groups,
// two per compute unit in a round.
#ifndef RQ_QJL_F16_WAVES
#define RQ_QJL_F16_WAVES 8
#endif
#ifndef RQ_MSE_PER_CU
#define RQ_MSE_PER_CU 2
#endif
template <int B, bool QJL>
hipError_t launch_quant_b(const RotorDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                          int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    const char* xc = static_cast<const char*>(x);
    char* yc = static_cast<char*>(y);
    constexpr int WF = QJL ? RQ_QJL_F16_WAVES : 4;   // fp16 in and out
    constexpr int PC = QJL ? 1 : RQ_MSE_PER_CU;
#define RQ_LAUNCH(IF, OF, RT, WV)                                                                               \
    hipLaunchKernelGGL((rq_quant_kernel<B, QJL, IF, OF, RT, WV>), dim3(grid2_for(n, WV, PC)), dim3(64 * WV), 0, s, \
                       P, xc, ldx_bytes, n, codes, norms, signs, rnorms, yc, ldy_bytes)
    if (!roundtrip) {
        if (in_f16) RQ_LAUNCH(true, true, false, WF);
        else RQ_LAUNCH(false, true, false, 4);
    } else if (in_f16) {
        if (out_f16) RQ_LAUNCH(true, true, true, WF);
        else RQ_LAUNCH(true, false, true, 4);
    } else {
        if (out_f16) RQ_LAUNCH(false, true, true, 4);
        else RQ_LAUNCH(false, false, true, 4);
    }
#undef RQ_LAUNCH
    return hipGetLastError();
}

template <int B, bool QJL>
hipError_t launch_dequant_b(const RotorDev& P, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                            const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                            hipStream_t s) {
    const int grid = grid2_for(n, 4, QJL ? 1 : RQ_MSE_PER_CU);
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
