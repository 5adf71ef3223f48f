// PolarQuant for gfx950 (PolarQuant article: "Полярное преобразование",
// "Алгоритм PolarQuant на практике", "Степень сжатия"): y = Pi x, then a
// recursive polar transform of y in four levels (pairs -> angle + radius,
// 128 -> 64 -> 32 -> 16 -> 8 radii), each angle coded against its level's
// Lloyd codebook (4 bits on [0, 2 pi), then 2 bits on [0, pi/2]), the 8 final
// radii stored as halves: 16 words per vector.
//
// One vector per lane, 64 per wave, as in the other codec kernels.  The
// rotation reuses the TurboQuant kernels' exact-enough MFMA scheme (Pi and the
// unit vector both as half pairs, three 32x32x16 products per K step).  The
// pairs of each level sit in one lane and, for every level, inside the same
// 32-coordinate M tile, so each tile's codes and radii are finished straight
// from its accumulators.
//
// Angle codes are taken without any arctangent: for a boundary t, the angle
// of (a, b) exceeds t exactly when b cos t - a sin t > 0 (the angle and t
// differ by less than pi).  The first level's codebook is uniform (t_k =
// k pi / 8), so its point is folded into the first octant by exact moves —
// a turn by pi (negation), a turn by -pi/2 (swap and negate), a reflection
// in the diagonal (swap) — each adding its share of the code, and one cross
// product against t_1 finishes it.
#include "rq_dense.cuh"

namespace rqk {

// float2 entries of PolarDev::tab
constexpr int kPqBnd0 = 0;    // level 1: (cos, sin) of t_1..t_7 (only t_1 is read)
constexpr int kPqBnd = 7;     // levels 2..4: 3 each, level L at kPqBnd + 3 (L - 2)
constexpr int kPqCen0 = 16;   // level 1: 16 centroids
constexpr int kPqCen = 32;    // levels 2..4: 4 each, level L at kPqCen + 4 (L - 2)
constexpr int kPqTab2 = 44;
static_assert(2 * kPqTab2 == kPolarTab, "table size");

__device__ __forceinline__ void pq_tab_to_lds(const float* __restrict__ g, float2* __restrict__ t) {
    if (threadIdx.x < kPqTab2) t[threadIdx.x] = reinterpret_cast<const float2*>(g)[threadIdx.x];
}

// #{k : angle(a, b) > t_k} on [0, 2 pi) with the 15 uniform boundaries
// t_k = k pi / 8 (see the header): lower half-plane (+8), second quadrant of
// what is left (+4), upper octant of that (+2, reflected), then the side of
// the ray at pi / 8 (c1, s1 = cos, sin of t_1).
__device__ __forceinline__ uint32_t pq_code_first(float a, float b, float c1, float s1) {
    const bool lower = b < 0.0f;
    const float u = lower ? -a : a, v = lower ? -b : b;
    const bool left = u < 0.0f;   // u = 0 stays: angle pi/2 is below t_4, and (0, 0) codes 0
    const float u1 = left ? v : u, v1 = left ? -u : v;
    const bool diag = v1 > u1;
    const float u2 = diag ? v1 : u1, v2 = diag ? u1 : v1;
    const float x = __builtin_fmaf(v2, c1, -(u2 * s1));
    const bool fine = diag ? (x < 0.0f) : (x > 0.0f);
    return (lower ? 8u : 0u) + (left ? 4u : 0u) + (diag ? 2u : 0u) + (fine ? 1u : 0u);
}

// #{k : angle(a, b) > t_k} on [0, pi/2] (a, b >= 0) with 3 boundaries.
__device__ __forceinline__ uint32_t pq_code_later(float a, float b, const float* c, const float* s) {
    uint32_t code = 0u;
#pragma unroll
    for (int k = 0; k < 3; ++k) code += (__builtin_fmaf(b, c[k], -(a * s[k])) > 0.0f) ? 1u : 0u;
    return code;
}

// Radii use the hardware square root (within an ulp): they feed the next
// level's decisions and the stored halves, far above that error.
__device__ __forceinline__ float pq_radius(float a, float b) {
    return __builtin_amdgcn_sqrtf(__builtin_fmaf(a, a, b * b));
}

// Boundary constants of one wave, held in SGPRs.
struct PqBounds {
    float c0, s0;
    float c[3][3], s[3][3];
    __device__ void load(const float2* __restrict__ tab, int z) {
        c0 = uniform(tab[kPqBnd0 + z].x);
        s0 = uniform(tab[kPqBnd0 + z].y);
#pragma unroll
        for (int L = 0; L < 3; ++L)
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                c[L][k] = uniform(tab[kPqBnd + 3 * L + k + z].x);
                s[L][k] = uniform(tab[kPqBnd + 3 * L + k + z].y);
            }
    }
};

// Codes and radii of M tile MT (unit-domain coordinates 32 MT .. 32 MT + 31,
// y0 / y1 as from_accumulators leaves them, still scaled by 2^19) into the
// record words w; its two final radii go to rad[2 MT], rad[2 MT + 1].
// Tile-local pair m covers coordinates 2m, 2m + 1 = rows 8 b + 4 h + 2 p and
// the next, b = m / 4, h = (m / 2) % 2, p = m % 2: registers 4 b + 2 p and
// 4 b + 2 p + 1 of own half h.
template <int MT>
__device__ __forceinline__ void pq_encode_tile(const float (&y0)[16], const float (&y1)[16], const PqBounds& B,
                                               uint32_t (&w)[kPolarWords], float (&rad)[8]) {
    float r1[16], r2[8], r3[4];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int b = m >> 2, h = (m >> 1) & 1, p = m & 1;
        const float a = (h ? y1[4 * b + 2 * p] : y0[4 * b + 2 * p]) * kRotScale;
        const float bb = (h ? y1[4 * b + 2 * p + 1] : y0[4 * b + 2 * p + 1]) * kRotScale;
        const int M = 16 * MT + m;                                   // level-1 pair, bits 4 M
        w[M >> 3] |= pq_code_first(a, bb, B.c0, B.s0) << (4 * (M & 7));
        r1[m] = pq_radius(a, bb);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int K = 8 * MT + k;                                    // level 2, bits 256 + 2 K
        w[8 + (K >> 4)] |= pq_code_later(r1[2 * k], r1[2 * k + 1], B.c[0], B.s[0]) << (2 * (K & 15));
        r2[k] = pq_radius(r1[2 * k], r1[2 * k + 1]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int J = 4 * MT + j;                                    // level 3, bits 320 + 2 J
        w[10] |= pq_code_later(r2[2 * j], r2[2 * j + 1], B.c[1], B.s[1]) << (2 * J);
        r3[j] = pq_radius(r2[2 * j], r2[2 * j + 1]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int I = 2 * MT + i;                                    // level 4, bits 352 + 2 I
        w[11] |= pq_code_later(r3[2 * i], r3[2 * i + 1], B.c[2], B.s[2]) << (2 * I);
        rad[I] = pq_radius(r3[2 * i], r3[2 * i + 1]);
    }
}

// y~ of one record, divided by the norm of its radii and split into the
// half pairs of the rotation (h11 = 2^11 hi, hi, lo of 16 y~_u); returns that
// norm.  The levels are walked back from the radii: r -> (r cos c, r sin c).
__device__ __forceinline__ float pq_decode_split(const float2* __restrict__ tab, const uint32_t (&w)[kPolarWords],
                                                 uint32_t (&yh11)[64], uint32_t (&yh)[64], uint32_t (&yl)[64]) {
    float R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) R[i] = h2f((w[12 + (i >> 1)] >> (16 * (i & 1))) & 0xFFFFu);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(R[i], R[i], ss);
    const float rn = __builtin_sqrtf(ss);
    const float inv16 = rn > 0.0f ? 16.0f / rn : 0.0f;
#pragma unroll
    for (int MT = 0; MT < 4; ++MT) {
        float r3[4], r2[8], r1[16];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int I = 2 * MT + i;
            const float2 cs = tab[kPqCen + 8 + ((w[11] >> (2 * I)) & 3u)];
            const float r = R[I] * inv16;
            r3[2 * i] = r * cs.x;
            r3[2 * i + 1] = r * cs.y;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int J = 4 * MT + j;
            const float2 cs = tab[kPqCen + 4 + ((w[10] >> (2 * J)) & 3u)];
            r2[2 * j] = r3[j] * cs.x;
            r2[2 * j + 1] = r3[j] * cs.y;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int K = 8 * MT + k;
            const float2 cs = tab[kPqCen + ((w[8 + (K >> 4)] >> (2 * (K & 15))) & 3u)];
            r1[2 * k] = r2[k] * cs.x;
            r1[2 * k + 1] = r2[k] * cs.y;
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int M = 16 * MT + m;
            const float2 cs = tab[kPqCen0 + ((w[M >> 3] >> (4 * (M & 7))) & 15u)];
            // 16 y~_u of coordinates 2M, 2M + 1 -> hi = half(v), lo = half((v - hi) 2^11)
            const float va = r1[m] * cs.x, vb = r1[m] * cs.y;
            const uint32_t hi = cvt_pk(va, vb);
            const float da = va - h2f(hi & 0xFFFFu), db = vb - h2f(hi >> 16);
            yh[M] = hi;
            yl[M] = cvt_pk(da * 2048.0f, db * 2048.0f);
            yh11[M] = pk_scale2048(hi);
        }
    }
    return rn;
}

// x~ = Pi^T y~ of one record into `out` (coordinates in increasing order);
// The scoring form of pq_decode_split followed by rot_mfma<0>: each 32
// coordinates are split and enter the rotation's two K blocks as soon as
// they are decoded, so only one chunk's half pairs are live (the same
// values and the same MFMA order as the two steps one after the other).
template <class FragHi, class FragLo>
__device__ __forceinline__ float pq_decode_rot(const float2* __restrict__ tab, const uint32_t (&w)[kPolarWords],
                                               FragHi fa_hi, FragLo fa_lo, int l, float (&own0)[16],
                                               float (&own1)[16]) {
    float R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) R[i] = h2f((w[12 + (i >> 1)] >> (16 * (i & 1))) & 0xFFFFu);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(R[i], R[i], ss);
    const float rn = __builtin_sqrtf(ss);
    const float inv16 = rn > 0.0f ? 16.0f / rn : 0.0f;
    f32x16 a0 = {}, a1 = {};
#pragma unroll
    for (int MT = 0; MT < 4; ++MT) {
        float r3[4], r2[8], r1[16];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int I = 2 * MT + i;
            const float2 cs = tab[kPqCen + 8 + ((w[11] >> (2 * I)) & 3u)];
            const float r = R[I] * inv16;
            r3[2 * i] = r * cs.x;
            r3[2 * i + 1] = r * cs.y;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int J = 4 * MT + j;
            const float2 cs = tab[kPqCen + 4 + ((w[10] >> (2 * J)) & 3u)];
            r2[2 * j] = r3[j] * cs.x;
            r2[2 * j + 1] = r3[j] * cs.y;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int K = 8 * MT + k;
            const float2 cs = tab[kPqCen + ((w[8 + (K >> 4)] >> (2 * (K & 15))) & 3u)];
            r1[2 * k] = r2[k] * cs.x;
            r1[2 * k + 1] = r2[k] * cs.y;
        }
        uint32_t yh11[16], yh[16], yl[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int M = 16 * MT + m;
            const float2 cs = tab[kPqCen0 + ((w[M >> 3] >> (4 * (M & 7))) & 15u)];
            const float va = r1[m] * cs.x, vb = r1[m] * cs.y;
            const uint32_t hi = cvt_pk(va, vb);
            const float da = va - h2f(hi & 0xFFFFu), db = vb - h2f(hi >> 16);
            yh[m] = hi;
            yl[m] = cvt_pk(da * 2048.0f, db * 2048.0f);
            yh11[m] = pk_scale2048(hi);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kb = 2 * MT + kk, o = 8 * kk;
            const int row = l & 31, chunk = 2 * kb + (l >> 5);
            const u32x4 ph = fa_hi(row, chunk);
            const u32x4 pl = fa_lo(row, chunk);
            u32x4 b11_0, b11_1, bh_0, bh_1, bl_0, bl_1;
            to_operands(u32x4{yh11[o], yh11[o + 1], yh11[o + 2], yh11[o + 3]},
                        u32x4{yh11[o + 4], yh11[o + 5], yh11[o + 6], yh11[o + 7]}, &b11_0, &b11_1);
            to_operands(u32x4{yh[o], yh[o + 1], yh[o + 2], yh[o + 3]},
                        u32x4{yh[o + 4], yh[o + 5], yh[o + 6], yh[o + 7]}, &bh_0, &bh_1);
            to_operands(u32x4{yl[o], yl[o + 1], yl[o + 2], yl[o + 3]},
                        u32x4{yl[o + 4], yl[o + 5], yl[o + 6], yl[o + 7]}, &bl_0, &bl_1);
            a0 = mfma(ph, b11_0, a0);
            a0 = mfma(ph, bl_0, a0);
            a0 = mfma(pl, bh_0, a0);
            a1 = mfma(ph, b11_1, a1);
            a1 = mfma(ph, bl_1, a1);
            a1 = mfma(pl, bh_1, a1);
        }
    }
    from_accumulators(a0, a1, own0, own1);
    return rn;
}

// done(mt) runs once coordinates 32 mt .. 32 mt + 31 are set.
template <class Out, class Done>
__device__ __forceinline__ void pq_dequant_vec(const PolarDev& P, const float2* __restrict__ tab,
                                               const uint32_t (&w)[kPolarWords], Out& out, int l, Done done) {
    uint32_t yh11[64], yh[64], yl[64];
    const float rn = pq_decode_split(tab, w, yh11, yh, yl) * kRotScale;
    auto tile = [&](auto mt_c) {
        constexpr int MT = decltype(mt_c)::value;
        float x0[16], x1[16];
        rot_mfma<MT>(
            yh11, yh, yl, [&](int row, int chunk) { return gmat_frag(P.pit_hi, row, chunk); },
            [&](int row, int chunk) { return gmat_frag(P.pit_lo, row, chunk); }, l, x0, x1);
#pragma unroll
        for (int il = 0; il < 32; ++il) {
            const int b8 = il >> 3, k = il & 7;
            const float xv = k < 4 ? x0[4 * b8 + k] : x1[4 * b8 + k - 4];
            out.set(32 * MT + il, rn * xv);
        }
        done(MT);
    };
    tile(std::integral_constant<int, 0>{});
    tile(std::integral_constant<int, 1>{});
    tile(std::integral_constant<int, 2>{});
    tile(std::integral_constant<int, 3>{});
}

// ------------------------------------------------------------ kernels --
constexpr int kPqWaves = 4;

struct PqQuantLds {
    u32x4 tiles[kPqWaves][kTileBytes / 16];
    u32x4 pih[128 * 16];
    u32x4 pil[128 * 16];
    float2 tab[kPqTab2];
};

template <bool IN_F16, bool OUT_F16, bool ROUNDTRIP>
__global__ __launch_bounds__(kPqWaves * 64) void pq_quant_kernel(PolarDev P, const char* __restrict__ x,
                                                                 int64_t ldx_bytes, int64_t n,
                                                                 uint32_t* __restrict__ words, char* __restrict__ y,
                                                                 int64_t ldy_bytes) {
    __shared__ PqQuantLds sm;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (n + 63) / 64;
    const bool single = ntiles <= kSimds;   // at most one tile per SIMD: output leaves in quarters
    const int64_t tstep = gridDim.x * (int64_t)kPqWaves;
    // fp16 input is fetched one tile ahead (the first one before the block's
    // staging), so each tile's load latency hides behind the previous tile
    TileRegs nxt;
    const int64_t t0 = blockIdx.x * (int64_t)kPqWaves + wave;
    if constexpr (IN_F16) {
        if (t0 < ntiles) tile_fetch(x, ldx_bytes, t0 * 64, n, 0, nxt, lane_id());
    }
    pq_tab_to_lds(P.tab, sm.tab);
    mat_to_lds<kPqWaves * 64>(P.pi_hi, sm.pih);
    mat_to_lds<kPqWaves * 64>(P.pi_lo, sm.pil);
    __syncthreads();

    u32x4* tile = sm.tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    for (int64_t t = t0; t < ntiles; t += tstep) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        PqBounds B;
        B.load(sm.tab, z);

        // load, norm (same arithmetic as the other codec kernels)
        uint32_t xin[IN_F16 ? 64 : 1];
        float xf32[IN_F16 ? 1 : 128];
        if constexpr (IN_F16) {
            tile_put(nxt, tile, l);
            if (t + tstep < ntiles) tile_fetch(x, ldx_bytes, (t + tstep) * 64, n, 0, nxt, l);
            wave_lds_sync();
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const u32x4 q = tile[swz(l, c)];
#pragma unroll
                for (int e = 0; e < 4; ++e) xin[4 * c + e] = q[e];
            }
        } else {
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
                const uint32_t v = xin[i >> 1];
                return h2f((i & 1) ? (v >> 16) : (v & 0xFFFFu));
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

        // y_u = Pi x_u tile by tile, each tile's codes and radii at once
        uint32_t w[kPolarWords];
#pragma unroll
        for (int k = 0; k < kPolarWords; ++k) w[k] = 0u;
        float rad[8];
        {
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
                pq_encode_tile<MT>(y0, y1, B, w, rad);
            };
            tile_q(std::integral_constant<int, 0>{});
            tile_q(std::integral_constant<int, 1>{});
            tile_q(std::integral_constant<int, 2>{});
            tile_q(std::integral_constant<int, 3>{});
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) w[12 + i] = f2h(rad[2 * i] * nrm) | (f2h(rad[2 * i + 1] * nrm) << 16);

        words_store<kPolarWords>(words, base, n, w, stage, l);
        if constexpr (ROUNDTRIP) {
            VecOutT<OUT_F16> out;
            if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
            out.begin(tile, l);
            pq_dequant_vec(P, sm.tab, w, out, l, [&](int mt) {
                if constexpr (OUT_F16) {
                    if (single) out.store_cols(y, ldy_bytes, base, n, 4 * mt);
                }
            });
            if (!OUT_F16 || !single) out.store(y, ldy_bytes, base, n);
        }
    }
}

template <bool OUT_F16>
__global__ __launch_bounds__(kPqWaves * 64) void pq_dequant_kernel(PolarDev P, const uint32_t* __restrict__ words,
                                                                   int64_t n, char* __restrict__ y,
                                                                   int64_t ldy_bytes) {
    __shared__ u32x4 tiles[kPqWaves][kTileBytes / 16];
    __shared__ float2 tab[kPqTab2];
    pq_tab_to_lds(P.tab, tab);
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    u32x4* tile = tiles[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);
    const int64_t ntiles = (n + 63) / 64;
    const bool single = ntiles <= kSimds;
    for (int64_t t = blockIdx.x * (int64_t)kPqWaves + wave; t < ntiles; t += gridDim.x * (int64_t)kPqWaves) {
        const int64_t base = t * 64;
        const int z = opaque_zero();
        const int l = lane_id() + z;
        uint32_t w[kPolarWords];
        words_load<kPolarWords>(words, base, n, w, stage, l);
        VecOutT<OUT_F16> out;
        if constexpr (!OUT_F16) out.bind(y, ldy_bytes, base, n);
        out.begin(tile, l);
        pq_dequant_vec(P, tab, w, out, l, [&](int mt) {
            if constexpr (OUT_F16) {
                if (single) out.store_cols(y, ldy_bytes, base, n, 4 * mt);
            }
        });
        if (!OUT_F16 || !single) out.store(y, ldy_bytes, base, n);
    }
}

// Scores of up to 32 query rows of one KV head against its keys.  Prologue:
// each wave rotates the chunk's query rows by one 32-row tile of Pi (lane r
// holds query row r, unit-normalised and split like the codec's vectors) and
// the rotated rows become the A operand, again as half pairs.  Main loop: a
// wave decodes 64 keys (one per lane) into split y~_u and one 32-row MFMA
// tile gives all rows' estimates for those keys.
struct PqScoreLds {
    float qhat[kPolarScoreRows][kD + 4];
    u32x4 ah[kPolarScoreRows * 16];
    u32x4 al[kPolarScoreRows * 16];
    float qn[kPolarScoreRows];
    float2 tab[kPqTab2];
    uint32_t stage[kPqWaves][64 * kPolarWords];
};

__global__ __launch_bounds__(kPqWaves * 64) void pq_score_kernel(PolarDev P, const float* __restrict__ q, int group,
                                                                 int chunks, const uint32_t* __restrict__ words,
                                                                 int64_t t, int64_t kv_stride,
                                                                 float* __restrict__ scores, int64_t ld) {
    __shared__ PqScoreLds sm;
    const int kvh = blockIdx.y / chunks;
    const int ch = blockIdx.y - kvh * chunks;
    const int64_t row0 = static_cast<int64_t>(kvh) * group + kPolarScoreRows * ch;
    const int nrows = min(kPolarScoreRows, group - kPolarScoreRows * ch);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id();
    pq_tab_to_lds(P.tab, sm.tab);
    {
        // lane l < nrows: query row row0 + l, unit-normalised, split; the
        // row is read twice (its norm, then 16 coordinates per K block) so
        // that only one block's half pairs are live
        const bool live = l < nrows;
        const float4* src = reinterpret_cast<const float4*>(q + (row0 + (live ? l : 0)) * kD);
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < kD / 4; ++c) {
            const float4 v = live ? src[c] : float4{0.0f, 0.0f, 0.0f, 0.0f};
            ss = __builtin_fmaf(v.x, v.x, ss);
            ss = __builtin_fmaf(v.y, v.y, ss);
            ss = __builtin_fmaf(v.z, v.z, ss);
            ss = __builtin_fmaf(v.w, v.w, ss);
        }
        const float nq = __builtin_sqrtf(ss);
        const float inv = nq > 0.0f ? 1.0f / nq : 0.0f;
        if (wave == 0 && l < kPolarScoreRows) sm.qn[l] = nq;
        auto rot = [&](auto mt_c) {
            constexpr int MT = decltype(mt_c)::value;
            f32x16 a0 = {}, a1 = {};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                uint32_t vh11[8], vh[8], vl[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 v = live ? src[4 * kb + c] : float4{0.0f, 0.0f, 0.0f, 0.0f};
                    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int k = 0; k < 4; k += 2) {
                        uint32_t a0h, b0h, c0h, a1h, b1h, c1h;
                        split16(e[k] * inv, &a0h, &b0h, &c0h);
                        split16(e[k + 1] * inv, &a1h, &b1h, &c1h);
                        const int i = 2 * c + (k >> 1);
                        vh11[i] = a0h | (a1h << 16);
                        vh[i] = b0h | (b1h << 16);
                        vl[i] = c0h | (c1h << 16);
                    }
                }
                const int row = 32 * MT + (l & 31), chunk = 2 * kb + (l >> 5);
                const u32x4 ph = gmat_frag(P.pi_hi, row, chunk);
                const u32x4 pl = gmat_frag(P.pi_lo, row, chunk);
                u32x4 b11_0, b11_1, bh_0, bh_1, bl_0, bl_1;
                to_operands(u32x4{vh11[0], vh11[1], vh11[2], vh11[3]}, u32x4{vh11[4], vh11[5], vh11[6], vh11[7]},
                            &b11_0, &b11_1);
                to_operands(u32x4{vh[0], vh[1], vh[2], vh[3]}, u32x4{vh[4], vh[5], vh[6], vh[7]}, &bh_0, &bh_1);
                to_operands(u32x4{vl[0], vl[1], vl[2], vl[3]}, u32x4{vl[4], vl[5], vl[6], vl[7]}, &bl_0, &bl_1);
                a0 = mfma(ph, b11_0, a0);
                a0 = mfma(ph, bl_0, a0);
                a0 = mfma(pl, bh_0, a0);
                a1 = mfma(ph, b11_1, a1);
                a1 = mfma(ph, bl_1, a1);
                a1 = mfma(pl, bh_1, a1);
            }
            float y0[16], y1[16];
            from_accumulators(a0, a1, y0, y1);
            if (l < kPolarScoreRows) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sm.qhat[l][32 * MT + own_row(0, r)] = y0[r] * kRotScale;
                    sm.qhat[l][32 * MT + own_row(1, r)] = y1[r] * kRotScale;
                }
            }
        };
        if (wave == 0) rot(std::integral_constant<int, 0>{});
        else if (wave == 1) rot(std::integral_constant<int, 1>{});
        else if (wave == 2) rot(std::integral_constant<int, 2>{});
        else rot(std::integral_constant<int, 3>{});
    }
    __syncthreads();
    // A operand: row r, chunk c (8 halves) of 16 Pi q_u, as hi and lo
    for (int e = threadIdx.x; e < kPolarScoreRows * 16; e += kPqWaves * 64) {
        const int r = e >> 4, c = e & 15;
        u32x4 hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a = sm.qhat[r][8 * c + 2 * k] * 16.0f, b = sm.qhat[r][8 * c + 2 * k + 1] * 16.0f;
            const uint32_t h = cvt_pk(a, b);
            hi[k] = h;
            lo[k] = cvt_pk((a - h2f(h & 0xFFFFu)) * 2048.0f, (b - h2f(h >> 16)) * 2048.0f);
        }
        sm.ah[r * 16 + (c ^ (r & 15))] = hi;
        sm.al[r * 16 + (c ^ (r & 15))] = lo;
    }
    __syncthreads();

    const uint32_t* kw = words + static_cast<int64_t>(kvh) * kv_stride * kPolarWords;
    float* out = scores + row0 * ld;
    uint32_t* stage = sm.stage[wave];
    const int64_t ntiles = (t + 63) / 64;
    for (int64_t tt = blockIdx.x * (int64_t)kPqWaves + wave; tt < ntiles; tt += gridDim.x * (int64_t)kPqWaves) {
        const int64_t base = tt * 64;
        const int z = opaque_zero();
        const int lz = lane_id() + z;
        uint32_t w[kPolarWords];
        words_load<kPolarWords>(kw, base, t, w, stage, lz);
        float s0[16], s1[16];
        const float rn = pq_decode_rot(
                             sm.tab, w, [&](int row, int chunk) { return mat_frag(sm.ah, row, chunk); },
                             [&](int row, int chunk) { return mat_frag(sm.al, row, chunk); }, lz, s0, s1) *
                         kRotScale;
        // rows past nrows are skipped (a uniform test) and fall outside the
        // range; keys past the end get an offset beyond it
        const rsrc_t rs = make_rsrc(out + base, static_cast<uint32_t>(((nrows - 1) * ld + (t - base)) * 4));
        const uint32_t voff = base + lz < t ? static_cast<uint32_t>(lz * 4) : 0x80000000u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = own_row(h, r);
                if (row < nrows) {
                    const float v = (h ? s1[r] : s0[r]) * rn * sm.qn[row];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff,
                                                          static_cast<int>(row * ld * 4), kNonTemporal);
                }
            }
        }
    }
}

// ------------------------------------------------- attention values --
// Decode attention with PolarQuant values (the weighted-sum pass of
// rq_attend).  Each wave walks 64-key tiles of its KV head.  Lane l decodes
// the record of key l into y~ / ||r|| (the levels walked back from the
// radii, as in the dequantiser; the radii norm ||r|| joins the key's
// weight), 32 coordinates at a time, into a [coordinate][key] block in LDS;
// lane (n, h) then takes coordinate 32 nt + n of keys 8h..8h+7 of each
// 16-key block as split halves (2^11 hi, lo11, hi) against the weights
// p ||r|| of query row n (hi, lo11) on 32x32x16 MFMAs.  The partial rows
// hold sum_t p_t y~_t in columns 0..127; the combine applies Pi^T (the
// dequantiser's x~ = Pi^T y~ is linear) and divides by the sum of weights.
constexpr int kPvPitch = 68;   // floats per coordinate row of the block (bank spread)
struct PqValueLds {
    float2 tab[kPqTab2];
    float yb[kPqWaves][32][kPvPitch];   // per wave; its first 4 KB also stage the records
    float rn[kPqWaves][64];
    float sum[32][kPartStride];
};
static_assert(32 * kPvPitch * 4 >= 64 * kPolarWords * 4, "record staging fits in the block");

__global__ __launch_bounds__(kPqWaves * 64) void pq_attend_values_kernel(PolarDev P, PolarValueArgs a) {
    __shared__ PqValueLds sm;
    const int qblocks = (a.group + 31) / 32;
    const int kvh = blockIdx.y / qblocks, qb = blockIdx.y % qblocks;
    const int row0 = kvh * a.group + qb * 32;
    const int nrows = min(32, a.group - qb * 32);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t rbase = static_cast<int64_t>(kvh) * a.kv_stride;
    const int64_t ntiles = (a.t + 63) / 64;
    pq_tab_to_lds(P.tab, sm.tab);
    __syncthreads();

    const int l = lane_id();
    const int n = l & 31, hh = l >> 5;
    const bool live = n < nrows;
    const float mrow = live ? a.stats[row0 + n].x : 0.0f;
    // estimates of this call's rows; rows past nrows lie outside the range and read as zero
    const rsrc_t rsc = make_rsrc(a.scores + static_cast<int64_t>(row0) * a.ld,
                                 static_cast<uint32_t>(nrows * a.ld * 4));
    const float2* tab = sm.tab;
    float(*yb)[kPvPitch] = sm.yb[wave];
    uint32_t* stage = reinterpret_cast<uint32_t*>(&sm.yb[wave][0][0]);
    float* rnw = sm.rn[wave];
    f32x16 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x16{};

    for (int64_t tile = blockIdx.x * (int64_t)kPqWaves + wave; tile < ntiles; tile += gridDim.x * (int64_t)kPqWaves) {
        const int64_t kbase = tile * 64;
        const int kleft = static_cast<int>(a.t - kbase < 64 ? a.t - kbase : 64);   // live keys of the tile
        const int z = opaque_zero();
        const int lz = l + z;
        // estimates of row n for keys 16 kb + 8 hh .. + 7
        u32x4 sv[4][2];
        const uint32_t soff = static_cast<uint32_t>((n * a.ld + kbase + 8 * hh) * 4);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                sv[kb][q] = __builtin_amdgcn_raw_buffer_load_b128(rsc, soff, 64 * kb + 16 * q, kNonTemporal);
        // key lz's record (zero past the end) and its radii norm
        uint32_t w[kPolarWords];
        words_load<kPolarWords>(a.words + rbase * kPolarWords, kbase, a.t, w, stage, lz);
        float R[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) R[i] = h2f((w[12 + (i >> 1)] >> (16 * (i & 1))) & 0xFFFFu);
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(R[i], R[i], ss);
        const float rn = __builtin_sqrtf(ss);
        const float inv = rn > 0.0f ? 1.0f / rn : 0.0f;
        rnw[lz] = rn;
        wave_lds_sync();
        // weights p ||r|| of keys 16 kb + 8 hh + k for row n, split
        u32x4 wh[4], wl[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int k0 = 16 * kb + 8 * hh;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float w2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 2 * q + e;
                    const uint32_t sbits = sv[kb][k >> 2][k & 3];
                    const float sc = __builtin_bit_cast(float, sbits);
                    const bool in = live && k0 + k < kleft;
                    const float ex = in ? __builtin_amdgcn_exp2f((sc * a.scale - mrow) * 1.44269504088896341f) : 0.0f;
                    w2[e] = ex * rnw[k0 + k];
                }
                const uint32_t h = cvt_pk(w2[0], w2[1]);
                wh[kb][q] = h;
                wl[kb][q] = cvt_pk((w2[0] - h2f(h & 0xFFFFu)) * 2048.0f, (w2[1] - h2f(h >> 16)) * 2048.0f);
            }
        }
        // y~ / ||r||, 32 coordinates (M tile MT of the dequantiser) at a time
#pragma unroll
        for (int MT = 0; MT < 4; ++MT) {
            float r3[4], r2[8], r1[16];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int I = 2 * MT + i;
                const float2 cs = tab[kPqCen + 8 + ((w[11] >> (2 * I)) & 3u)];
                const float r = R[I] * inv;
                r3[2 * i] = r * cs.x;
                r3[2 * i + 1] = r * cs.y;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int J = 4 * MT + j;
                const float2 cs = tab[kPqCen + 4 + ((w[10] >> (2 * J)) & 3u)];
                r2[2 * j] = r3[j] * cs.x;
                r2[2 * j + 1] = r3[j] * cs.y;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int K = 8 * MT + k;
                const float2 cs = tab[kPqCen + ((w[8 + (K >> 4)] >> (2 * (K & 15))) & 3u)];
                r1[2 * k] = r2[k] * cs.x;
                r1[2 * k + 1] = r2[k] * cs.y;
            }
            wave_lds_sync();   // the previous block's reads (or the record staging) are done
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int M = 16 * MT + m;
                const float2 cs = tab[kPqCen0 + ((w[M >> 3] >> (4 * (M & 7))) & 15u)];
                yb[2 * m][lz] = r1[m] * cs.x;
                yb[2 * m + 1][lz] = r1[m] * cs.y;
            }
            wave_lds_sync();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float4 y0 = *reinterpret_cast<const float4*>(&yb[n][16 * kb + 8 * hh]);
                const float4 y1 = *reinterpret_cast<const float4*>(&yb[n][16 * kb + 8 * hh + 4]);
                const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                u32x4 b11, blo, bhi;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t h = cvt_pk(y[2 * q], y[2 * q + 1]);
                    bhi[q] = h;
                    b11[q] = pk_scale2048(h);
                    blo[q] = cvt_pk((y[2 * q] - h2f(h & 0xFFFFu)) * 2048.0f, (y[2 * q + 1] - h2f(h >> 16)) * 2048.0f);
                }
                acc[MT] = mfma(wh[kb], b11, acc[MT]);
                acc[MT] = mfma(wh[kb], blo, acc[MT]);
                acc[MT] = mfma(wl[kb], bhi, acc[MT]);
            }
        }
        wave_lds_sync();   // this tile's block reads are done before the next staging
    }

    // the block's partial rows: the four waves' sums added in wave order
    // through LDS, then written as producer blockIdx.x
    const float uc = 1.0f / 2048.0f;
    for (int wv = 0; wv < kPqWaves; ++wv) {
        if (wave == wv) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = own_row(hh, r);
                if (m < nrows) {
                    float* dst = sm.sum[m];
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const float c = acc[nt][r] * uc;
                        dst[32 * nt + n] = wv == 0 ? c : dst[32 * nt + n] + c;
                    }
                }
            }
        }
        __syncthreads();
    }
    float* out = a.part + (static_cast<int64_t>(blockIdx.x) * a.rows + row0) * kPartStride;
    for (int i = threadIdx.x; i < nrows * kPartStride; i += kPqWaves * 64) {
        const int m = i / kPartStride, c = i % kPartStride;
        out[static_cast<int64_t>(m) * kPartStride + c] = c < kD ? sm.sum[m][c] : 0.0f;
    }
}

// ------------------------------------------------------------ launchers --
static int pq_grid(int64_t n, int64_t cap) {
    const int64_t ntiles = (n + 63) / 64;
    const int64_t blocks = (ntiles + kPqWaves - 1) / kPqWaves;
    return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

hipError_t polar_quantize(const PolarDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* words, void* y, bool out_f16, int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    const int grid = pq_grid(n, 256 * 4);
    const char* xc = static_cast<const char*>(x);
    char* yc = static_cast<char*>(y);
#define PQ_LAUNCH(IF, OF, RT)                                                                                     \
    hipLaunchKernelGGL((pq_quant_kernel<IF, OF, RT>), dim3(grid), dim3(kPqWaves * 64), 0, s, P, xc, ldx_bytes, n, \
                       words, yc, ldy_bytes)
    if (!roundtrip) {
        if (in_f16) PQ_LAUNCH(true, true, false); else PQ_LAUNCH(false, true, false);
    } else if (in_f16) {
        if (out_f16) PQ_LAUNCH(true, true, true); else PQ_LAUNCH(true, false, true);
    } else {
        if (out_f16) PQ_LAUNCH(false, true, true); else PQ_LAUNCH(false, false, true);
    }
#undef PQ_LAUNCH
    return hipGetLastError();
}

hipError_t polar_dequantize(const PolarDev& P, const uint32_t* words, int64_t n, void* y, bool out_f16,
                            int64_t ldy_bytes, hipStream_t s) {
    const int grid = pq_grid(n, 256 * 8);
    char* yc = static_cast<char*>(y);
    if (out_f16)
        hipLaunchKernelGGL((pq_dequant_kernel<true>), dim3(grid), dim3(kPqWaves * 64), 0, s, P, words, n, yc, ldy_bytes);
    else
        hipLaunchKernelGGL((pq_dequant_kernel<false>), dim3(grid), dim3(kPqWaves * 64), 0, s, P, words, n, yc, ldy_bytes);
    return hipGetLastError();
}

hipError_t polar_score(const PolarDev& P, const float* q, int hq, int group, const uint32_t* words, int64_t t,
                       int64_t kv_stride, float* scores, int64_t ld_scores, hipStream_t s) {
    const int chunks = (group + kPolarScoreRows - 1) / kPolarScoreRows;
    const int gy = (hq / group) * chunks;
    // about three blocks per CU in all (the kernel's occupancy), each walking
    // its key slice tile by tile
    const int64_t want = (768 + gy - 1) / gy;
    const int gx = pq_grid(t, want > 0 ? want : 1);
    hipLaunchKernelGGL(pq_score_kernel, dim3(gx, gy), dim3(kPqWaves * 64), 0, s, P, q, group, chunks, words, t,
                       kv_stride, scores, ld_scores);
    return hipGetLastError();
}

hipError_t polar_attend_values(const PolarDev& P, const PolarValueArgs& a, int producers, int kv_heads,
                               hipStream_t s) {
    const int qblocks = (a.group + 31) / 32;
    hipLaunchKernelGGL(pq_attend_values_kernel, dim3(producers, kv_heads * qblocks), dim3(kPqWaves * 64), 0, s, P, a);
    return hipGetLastError();
}

}  // namespace rqk
