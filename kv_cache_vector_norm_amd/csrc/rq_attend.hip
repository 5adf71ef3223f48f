// Decode attention read straight from a compressed KV cache: for query row h
// of KV head j = h / group,
//   out_h = sum_t softmax_t(scale * s_ht) * v~_t,
// s_ht the q.k estimate over key t's record (the estimator of rq_score) and
// v~_t the dequantisation of value t's record (PolarQuant article, KV-cache
// section: attention is softmax(Q K^T / sqrt(d)) V; README, note under
// "Triton Kernels": the scores are taken from the compressed keys).
//
// The values are never decoded to vectors.  Dequantisation is linear in the
// stored centroids and signs once the norms are folded into the weights:
//   v~_t = n^_t X^T c_t + kappa n^_t gamma^_t S^T sigma_t
// (X^T = the inverse rotor sandwich, or Pi^T; kappa = sqrt(pi/2)/m), so
//   sum_t p_t v~_t = X^T (sum_t p_t n^_t c_t) + kappa S^T (sum_t p_t n^_t gamma^_t sigma_t).
// The two sums are products of a weight matrix [rows x keys] with the
// centroid / sign matrices [keys x coordinates] and run on 32x32x16 fp16
// MFMAs; X^T and S^T are applied once per query row at the end.  PolarQuant
// values are the one kind decoded (to y~ = Pi x~, in rq_polar.hip's value
// pass): sum_t p_t v~_t = Pi^T (sum_t p_t y~_t), Pi^T once per row.  PolarQuant
// keys are scored by pq_score in pass 1.
//
// Passes (all on the caller's stream, workspace from the caller):
//   1. the estimates s (rq_score's kernel) into the workspace;
//   2. per row M = max scale*s and L = sum exp(scale*s - M) (one pass, the
//      running-maximum form);
//   3. per (KV head, <= 32 rows, key slice) wave: the two weighted sums over
//      its tiles in the rotated domain, written as partial rows;
//   4. per row: sum the partials in a fixed order, apply X^T and kappa S^T,
//      divide by L.
#include "rq_common.cuh"
#include "rq_kernels.h"

namespace rqk {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, l) pairs of a running maximum and a sum of exp(x - m): merge b into a.
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    const float a = m == -INFINITY ? 0.0f : l * exp2_hw((m - mn) * kLog2e);
    const float b = m2 == -INFINITY ? 0.0f : l2 * exp2_hw((m2 - mn) * kLog2e);
    l = a + b;
    m = mn;
}

// ------------------------------------------------------ pass 2: row stats --
__global__ __launch_bounds__(256) void attend_stats_kernel(const float* __restrict__ scores, int64_t ld, int64_t t,
                                                          float scale, float2* __restrict__ stats) {
    const int row = blockIdx.x;
    const float* s = scores + static_cast<int64_t>(row) * ld;
    float m = -INFINITY, l = 0.0f;
    auto add = [&](float x) {
        const float v = x * scale;
        if (v > m) {
            l = l * exp2_hw((m - v) * kLog2e) + 1.0f;
            m = v;
        } else {
            l += exp2_hw((v - m) * kLog2e);
        }
    };
    // rows are 16-byte aligned (the pitch is a multiple of 4 floats)
    const float4* s4 = reinterpret_cast<const float4*>(s);
    const int64_t t4 = t / 4;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < t4; i += 256) {
        const float4 v = s4[i];
        add(v.x);
        add(v.y);
        add(v.z);
        add(v.w);
    }
    for (int64_t i = 4 * t4 + threadIdx.x; i < t; i += 256) add(s[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const float l2 = __shfl_xor(l, off);
        ml_merge(m, l, m2, l2);
    }
    __shared__ float2 part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = make_float2(m, l);
    __syncthreads();
    if (threadIdx.x == 0) {
        float mm = part[0].x, ll = part[0].y;
        for (int w = 1; w < 4; ++w) ml_merge(mm, ll, part[w].x, part[w].y);
        stats[row] = make_float2(mm, ll);
    }
}

// ------------------------------------------------ pass 3: weighted sums --

struct AttendArgs {
    const float* scores;      // [rows][ld] raw estimates of this call's rows
    int64_t ld;
    const float2* stats;      // [rows] (M, L) of scale * estimate
    float scale;
    const uint32_t* codes;    // value records
    const uint16_t* norms;
    const uint32_t* signs;
    const uint16_t* rnorms;
    int64_t t, kv_stride;
    int group, rows;          // rows: query rows of the call
    const float* cent;        // value centroids
    float* part;              // [producers][rows][kPartStride]
    PageTable pt;             // value record rows (pages == nullptr: kvh * kv_stride + key)
};

// Exact split of a pair into fp16 hi and lo11 = half((x - hi) 2^11).
__device__ __forceinline__ void split_pair11(float a, float b, uint32_t* hi, uint32_t* lo11) {
    const uint32_t h = cvt_pk(a, b);
    *hi = h;
    *lo11 = cvt_pk((a - h2f(h & 0xFFFFu)) * 2048.0f, (b - h2f(h >> 16)) * 2048.0f);
}

// CODES: the centroid sums (codes and norms are read); QJL: the sign sums
// (signs, norms and residual norms).  A QJL value session runs two passes,
// one of each, writing disjoint columns of the partial rows: each pass
// holds half the accumulators, so two waves fit on a SIMD.
// Register budget: two waves per SIMD for the centroid pass (3- and 4-bit
// values included), three for the sign pass.
template <int B, bool QJL, bool PAD, bool CODES = true>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CODES ? 2 : 3))) void attend_values_kernel(
    AttendArgs a) {
    constexpr int L = 1 << B;
    constexpr int W = CODES ? (((PAD ? kRotCoords : kD) * B) + 31) / 32 : 1;
    struct alignas(16) Wave {
        uint32_t code[W + 1][64];   // [word][key]; one spare word row for the straddle read
        uint32_t sign[4][64];
        alignas(16) uint16_t nrm[64];
        alignas(16) uint16_t gam[64];
    };
    struct Lds {
        // codes (k, k+1) -> 2^11 C_hi, C_lo and C_hi half pairs at [p], [257 + p],
        // [514 + p]: 1,028 bytes apart, so no two-address LDS read fetches two of
        // them together and each lands in its own MFMA operand without moves
        uint32_t ptab[CODES ? 3 * 257 : 1];
        u32x4 sig[QJL ? 256 : 1][2];   // eight sign bits -> {+-1, +-2^11} half pairs (bit 2q + e: dword q, half e)
        Wave w[4];
        float sum[32][kPartStride];   // the block's partial rows, waves added in order
    };
    __shared__ Lds lds;

    const int qblocks = (a.group + 31) / 32;
    const int kvh = blockIdx.y / qblocks, qb = blockIdx.y % qblocks;
    const int row0 = kvh * a.group + qb * 32;
    const int nrows = min(32, a.group - qb * 32);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t rbase = static_cast<int64_t>(kvh) * a.kv_stride;
    const int64_t ntiles = (a.t + 63) / 64;

    float sc = 1.0f;
    if constexpr (CODES) {
        const float cmax = fmaxf(fabsf(a.cent[L - 1]), fabsf(a.cent[0]));
        int e;
        frexpf(cmax, &e);
        sc = cmax > 0.0f ? ldexpf(1.0f, 1 - e) : 1.0f;     // |sc c| in [1, 2) at most
        for (int p = threadIdx.x; p < L * L; p += kBlock) {
            uint32_t h0, l0, h1, l1;
            split_h11(a.cent[p & (L - 1)] * sc, &h0, &l0);
            split_h11(a.cent[p >> B] * sc, &h1, &l1);
            const uint32_t hp = h0 | (h1 << 16);
            lds.ptab[p] = pk_scale2048(hp);
            lds.ptab[257 + p] = l0 | (l1 << 16);
            lds.ptab[514 + p] = hp;
        }
        for (int i = threadIdx.x; i < 4 * 64; i += kBlock) lds.w[i >> 6].code[W][i & 63] = 0u;
    }
    if constexpr (QJL) {
        // sigma = 2 bit - 1 as half pairs; the sign bit is set where the stored bit is 0
        for (int p = threadIdx.x; p < 256; p += kBlock) {
            u32x4 s1, s11;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t b0 = (p >> (2 * q)) & 1u, b1 = (p >> (2 * q + 1)) & 1u;
                const uint32_t sgn = ((b0 ^ 1u) << 15) | ((b1 ^ 1u) << 31);
                s1[q] = 0x3C003C00u | sgn;     // +-1
                s11[q] = 0x68006800u | sgn;    // +-2^11
            }
            lds.sig[p][0] = s1;
            lds.sig[p][1] = s11;
        }
    }
    __syncthreads();

    Wave& wv = lds.w[wave];
    const int l = lane_id();
    const int n = l & 31, hh = l >> 5;
    const bool live = n < nrows;
    const float mrow = live ? a.stats[row0 + n].x : 0.0f;
    const rsrc_t rsc = make_rsrc(a.scores + static_cast<int64_t>(row0) * a.ld,
                                 static_cast<uint32_t>(nrows * a.ld * 4));

    f32x16 acc_c[4], acc_p, acc_s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        acc_c[nt] = f32x16{};
        acc_s[nt] = f32x16{};
    }
    acc_p = f32x16{};

    // One tile's inputs in registers: this lane's row of estimates (keys
    // 16 kb + 8 hh .. + 7 of each K block) and dword l of the tile's code,
    // sign and norm runs.  They are fetched one tile ahead of their use, so
    // each tile's load latency hides behind the previous tile's arithmetic.
    struct TileIn {
        u32x4 sv[4][2];
        uint32_t cw[W];
        uint32_t sw[4];
        uint32_t nb, gb;
    };
    auto fetch = [&](int64_t tile, TileIn& r) {
        const int64_t kbase = tile * 64;
        const uint32_t soff = static_cast<uint32_t>((n * a.ld + kbase + 8 * hh) * 4);
        // (rows past nrows lie outside rsc's range and read as zero)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                r.sv[kb][q] = __builtin_amdgcn_raw_buffer_load_b128(rsc, soff, 64 * kb + 16 * q, kNonTemporal);
        const int64_t left = a.t - kbase;
        int64_t row = rbase + kbase;
        if (a.pt.pages != nullptr) {
            const int64_t pg = a.pt.pages[kvh * a.pt.stride + (kbase >> a.pt.shift)];
            row = (pg << a.pt.shift) + (kbase & ((int64_t(1) << a.pt.shift) - 1));
        }
        if constexpr (CODES) {
            const rsrc_t rc = make_rsrc(a.codes + row * W, tile_range(left, 4 * W));
#pragma unroll
            for (int it = 0; it < W; ++it)
                r.cw[it] = __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<uint32_t>(4 * l), 256 * it,
                                                                kNonTemporal);
        }
        if constexpr (QJL) {
            const rsrc_t rs = make_rsrc(a.signs + row * 4, tile_range(left, 16));
#pragma unroll
            for (int it = 0; it < 4; ++it)
                r.sw[it] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
        }
        const rsrc_t rn = make_rsrc(a.norms + row, tile_range(left, 2));
        r.nb = __builtin_amdgcn_raw_buffer_load_b16(rn, static_cast<uint32_t>(2 * l), 0, kNonTemporal);
        r.gb = 0u;
        if constexpr (QJL) {
            const rsrc_t rg = make_rsrc(a.rnorms + row, tile_range(left, 2));
            r.gb = __builtin_amdgcn_raw_buffer_load_b16(rg, static_cast<uint32_t>(2 * l), 0, kNonTemporal);
        }
    };

    const int64_t tstep = gridDim.x * 4LL;
    TileIn nx;
    if (blockIdx.x * 4LL + wave < ntiles) fetch(blockIdx.x * 4LL + wave, nx);
    for (int64_t tile = blockIdx.x * 4LL + wave; tile < ntiles; tile += tstep) {
        const int64_t kbase = tile * 64;
        const int kleft = static_cast<int>(a.t - kbase < 64 ? a.t - kbase : 64);   // live keys of the tile
        u32x4 sv[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            sv[kb][0] = nx.sv[kb][0];
            sv[kb][1] = nx.sv[kb][1];
        }
        // the tile's value records into LDS, key-minor
        wave_lds_sync();
        if constexpr (CODES) {
#pragma unroll
            for (int it = 0; it < W; ++it) {
                const int d = it * 64 + l;
                wv.code[d % W][d / W] = nx.cw[it];
            }
        }
        if constexpr (QJL) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int d = it * 64 + l;
                wv.sign[d & 3][d >> 2] = nx.sw[it];
            }
            wv.gam[l] = static_cast<uint16_t>(nx.gb);
        }
        wv.nrm[l] = static_cast<uint16_t>(nx.nb);
        wave_lds_sync();
        if (tile + tstep < ntiles) fetch(tile + tstep, nx);

#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int k0 = 16 * kb + 8 * hh;
            // weights p n^ (and p n^ gamma^) of keys k0..k0+7 for row n, split
            const u32x4 nh = *reinterpret_cast<const u32x4*>(&wv.nrm[k0]);
            u32x4 gh{};
            if constexpr (QJL) gh = *reinterpret_cast<const u32x4*>(&wv.gam[k0]);
            u32x4 wh, wl, gwh, gwl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float w2[2], g2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 2 * q + e;
                    const uint32_t sbits = sv[kb][k >> 2][k & 3];
                    const float s = __builtin_bit_cast(float, sbits);
                    const bool in = live && k0 + k < kleft;
                    const float ex = in ? exp2_hw((s * a.scale - mrow) * kLog2e) : 0.0f;
                    const uint32_t nn = e ? (nh[q] >> 16) : (nh[q] & 0xFFFFu);
                    w2[e] = ex * h2f(nn);
                    if constexpr (QJL) {
                        const uint32_t gg = e ? (gh[q] >> 16) : (gh[q] & 0xFFFFu);
                        g2[e] = w2[e] * h2f(gg);
                    }
                }
                uint32_t h, lo;
                if constexpr (CODES) {
                    split_pair11(w2[0], w2[1], &h, &lo);
                    wh[q] = h;
                    wl[q] = lo;
                }
                if constexpr (QJL) {
                    split_pair11(g2[0], g2[1], &h, &lo);
                    gwh[q] = h;
                    gwl[q] = lo;
                }
            }
            // centroid operands: coordinate 32 nt + n (nt < 4), pad slot (nt = 4)
#pragma unroll
            for (int nt = 0; nt < (CODES ? (PAD ? 5 : 4) : 0); ++nt) {
                const int coord = nt < 4 ? 32 * nt + n : 128;
                const int bit = B * coord, wi = bit >> 5, off = bit & 31;
                const u32x4 w0a = *reinterpret_cast<const u32x4*>(&wv.code[wi][k0]);
                const u32x4 w0b = *reinterpret_cast<const u32x4*>(&wv.code[wi][k0 + 4]);
                u32x4 w1a{}, w1b{};
                if constexpr (32 % B != 0) {
                    w1a = *reinterpret_cast<const u32x4*>(&wv.code[wi + 1][k0]);
                    w1b = *reinterpret_cast<const u32x4*>(&wv.code[wi + 1][k0 + 4]);
                }
                u32x4 b11, blo, bhi;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t f[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int k = 2 * q + e;
                        const uint32_t x0 = k < 4 ? w0a[k] : w0b[k - 4];
                        if constexpr (32 % B != 0) {
                            const uint32_t x1 = k < 4 ? w1a[k] : w1b[k - 4];
                            f[e] = __builtin_amdgcn_alignbit(x1, x0, off) & (L - 1);
                        } else {
                            f[e] = (x0 >> off) & (L - 1);
                        }
                    }
                    const uint32_t ix = f[0] | (f[1] << B);
                    const bool keep = nt < 4 || n == 0;
                    b11[q] = keep ? lds.ptab[ix] : 0u;
                    blo[q] = keep ? lds.ptab[257 + ix] : 0u;
                    bhi[q] = keep ? lds.ptab[514 + ix] : 0u;
                }
                f32x16& acc = nt < 4 ? acc_c[nt] : acc_p;
                acc = mfma(wh, b11, acc);
                acc = mfma(wh, blo, acc);
                acc = mfma(wl, bhi, acc);
            }
            if constexpr (QJL) {
                // sign operands: index 32 nt + n, +-2^11 (hi) and +-1 (lo11)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const u32x4 sa = *reinterpret_cast<const u32x4*>(&wv.sign[nt][k0]);
                    const u32x4 sb = *reinterpret_cast<const u32x4*>(&wv.sign[nt][k0 + 4]);
                    uint32_t byte = 0u;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const uint32_t x = k < 4 ? sa[k] : sb[k - 4];
                        byte |= ((x >> n) & 1u) << k;
                    }
                    const u32x4 s1 = lds.sig[byte][0], s11 = lds.sig[byte][1];
                    acc_s[nt] = mfma(gwh, s11, acc_s[nt]);
                    acc_s[nt] = mfma(gwl, s1, acc_s[nt]);
                }
            }
        }
    }

    // the block's partial rows: the four waves' sums are added in wave order
    // through LDS, then written as producer blockIdx.x
    const float uc = 1.0f / (2048.0f * sc), us = 1.0f / 2048.0f;
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 8 * (r / 4) + (r % 4) + 4 * hh;
                if (m < nrows) {
                    float* dst = lds.sum[m];
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        if constexpr (CODES) {
                            const float c = acc_c[nt][r] * uc;
                            dst[32 * nt + n] = w == 0 ? c : dst[32 * nt + n] + c;
                        }
                        if constexpr (QJL) {
                            const float g = acc_s[nt][r] * us;
                            dst[kPartSigma + 32 * nt + n] = w == 0 ? g : dst[kPartSigma + 32 * nt + n] + g;
                        }
                    }
                    if (CODES && n == 0) {
                        const float pc = PAD ? acc_p[r] * uc : 0.0f;
                        dst[kPartPad] = w == 0 ? pc : dst[kPartPad] + pc;
                    }
                }
            }
        }
        __syncthreads();
    }
    float* out = a.part + (static_cast<int64_t>(blockIdx.x) * a.rows + row0) * kPartStride;
    // columns of this pass: the sign sums (QJL), or the centroid sums, the
    // pad slot and the spare columns (CODES)
    for (int i = threadIdx.x; i < nrows * kPartStride; i += kBlock) {
        const int m = i / kPartStride, c = i % kPartStride;
        const bool sig = c >= kPartSigma && c < kPartSigma + kD;
        if (sig ? QJL : CODES)
            out[static_cast<int64_t>(m) * kPartStride + c] = (sig || c < kPartSigma || c == kPartPad) ? lds.sum[m][c] : 0.0f;
    }
}

// ----------------------------------------------------- pass 4: combine --
struct CombineArgs {
    const float* part;
    int64_t producers;
    int rows;
    const float2* stats;
    bool rotor, qjl;
    const float* rotmat;      // rotor: [43][9], y = M v with M[r][c] = rotmat[9 g + 3 r + c]
    const uint16_t* pi_hi;    // dense: 16 Pi = hi + 2^-11 lo, row-major
    const uint16_t* pi_lo;
    const uint16_t* s_rows;   // QJL: S row-major halves
    float kappa;
    float* out;
    int64_t ld_out;
};

__global__ __launch_bounds__(320) void attend_combine_kernel(CombineArgs a) {
    const int row = blockIdx.x;
    __shared__ float oc[kRotCoords + 3];
    __shared__ float os[kD];
    const int j = threadIdx.x;
    // producers in a fixed order: eight interleaved running sums (loads in
    // flight together), added pairwise at the end
    const int col = j < kD ? j : (j < 2 * kD ? kPartSigma + (j - kD) : kPartPad);
    if (j < 2 * kD + 1 && (j < kD || j == 2 * kD || a.qjl)) {
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        const int64_t pstride = static_cast<int64_t>(a.rows) * kPartStride;
        const float* src = a.part + static_cast<int64_t>(row) * kPartStride + col;
        int64_t p = 0;
        for (; p + 8 <= a.producers; p += 8)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] += src[(p + u) * pstride];
        for (int u = 0; p < a.producers; ++p, ++u) acc[u] += src[p * pstride];
        const float v = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
        if (j < kD) oc[j] = v;
        else if (j == 2 * kD) oc[kD] = v;
        else os[j - kD] = v;
    } else if (j < 2 * kD) {
        os[j - kD] = 0.0f;
    }
    __syncthreads();
    if (j < kD) {
        float x = 0.0f;
        if (a.rotor) {
            const int g = j / 3, c = j % 3;
            const float* m = a.rotmat + 9 * g;
#pragma unroll
            for (int r = 0; r < 3; ++r) x = __builtin_fmaf(m[3 * r + c], oc[3 * g + r], x);
        } else {
            for (int i = 0; i < kD; ++i) {
                const float pij = (h2f(a.pi_hi[i * kD + j]) + h2f(a.pi_lo[i * kD + j]) * (1.0f / 2048.0f)) * 0.0625f;
                x = __builtin_fmaf(pij, oc[i], x);
            }
        }
        if (a.qjl) {
            float y = 0.0f;
            for (int k = 0; k < kD; ++k) y = __builtin_fmaf(h2f(a.s_rows[k * kD + j]), os[k], y);
            x = __builtin_fmaf(a.kappa, y, x);
        }
        a.out[row * a.ld_out + j] = x / a.stats[row].y;
    }
}

// ----------------------------------------------------------- launchers --
AttendPlan attend_plan(int hq, int group, int64_t t) {
    AttendPlan p;
    p.ld = (t + 3) & ~int64_t(3);
    const int kv_heads = hq / group;
    const int qblocks = (group + 31) / 32;
    const int64_t ntiles = (t + 63) / 64;
    const int64_t want = (ntiles + 3) / 4;
    const int64_t units = static_cast<int64_t>(kv_heads) * qblocks;
    int64_t gx = 512 / units;
    if (gx > 64) gx = 64;           // partial rows per query row stay few
    if (gx > want) gx = want;
    if (gx < 1) gx = 1;
    p.gx = static_cast<int>(gx);
    p.producers = gx;
    auto up = [](int64_t b) { return (b + 255) & ~int64_t(255); };
    p.off_scores = 0;
    p.off_stats = up(static_cast<int64_t>(hq) * p.ld * 4);
    p.off_part = p.off_stats + up(static_cast<int64_t>(hq) * 8);
    p.bytes = p.off_part + up(p.producers * hq * kPartStride * 4);
    return p;
}

// Centroid sums, then (QJL) sign sums: two passes over the tiles.
template <int B, bool QJL, bool PAD>
static void launch_values(const AttendArgs& a, const AttendPlan& p, int kv_heads, hipStream_t s) {
    const int qblocks = (a.group + 31) / 32;
    const dim3 grid(p.gx, kv_heads * qblocks);
    hipLaunchKernelGGL((attend_values_kernel<B, false, PAD, true>), grid, dim3(kBlock), 0, s, a);
    if constexpr (QJL) hipLaunchKernelGGL((attend_values_kernel<1, true, false, false>), grid, dim3(kBlock), 0, s, a);
}

template <bool QJL, bool PAD>
static hipError_t launch_values_b(int b, const AttendArgs& a, const AttendPlan& p, int kv_heads, hipStream_t s) {
    switch (b) {
        case 1: launch_values<1, QJL, PAD>(a, p, kv_heads, s); break;
        case 2: launch_values<2, QJL, PAD>(a, p, kv_heads, s); break;
        case 3: launch_values<3, QJL, PAD>(a, p, kv_heads, s); break;
        case 4: launch_values<4, QJL, PAD>(a, p, kv_heads, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

hipError_t attend(const ScoreTables& kt, const ScoreTables& vt, const float* q, int hq, int group,
                  const uint32_t* kcodes, const uint16_t* knorms, const uint32_t* ksigns, const uint16_t* krnorms,
                  const uint32_t* vcodes, const uint16_t* vnorms, const uint32_t* vsigns, const uint16_t* vrnorms,
                  int64_t t, int64_t kv_stride, float scale, void* workspace, float* out, int64_t ld_out,
                  hipStream_t s, const PageTable& kpt, const PageTable& vpt) {
    const AttendPlan p = attend_plan(hq, group, t);
    char* ws = static_cast<char*>(workspace);
    float* scores = reinterpret_cast<float*>(ws + p.off_scores);
    float2* stats = reinterpret_cast<float2*>(ws + p.off_stats);
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    const int kv_heads = hq / group;
    // 1. estimates, in chunks of whole KV heads (PolarQuant keys: one launch)
    if (kt.polar) {
        const hipError_t e = polar_score(kt.pol, q, hq, group, kcodes, t, kv_heads > 1 ? kv_stride : 0, scores, p.ld, s);
        if (e != hipSuccess) return e;
    }
    const int heads_per_chunk = group >= kScoreChunkRows ? 1 : kScoreChunkRows / group;
    for (int h0 = 0; h0 < (kt.polar ? 0 : kv_heads); h0 += heads_per_chunk) {
        const int nh = kv_heads - h0 < heads_per_chunk ? kv_heads - h0 : heads_per_chunk;
        const hipError_t e = score(kt, q + static_cast<int64_t>(h0) * group * kD, nh * group, group, kcodes, knorms,
                                   ksigns, krnorms, t, kv_stride, h0, scores + static_cast<int64_t>(h0) * group * p.ld,
                                   p.ld, s, kpt);
        if (e != hipSuccess) return e;
    }
    // 2. row statistics
    hipLaunchKernelGGL(attend_stats_kernel, dim3(hq), dim3(kBlock), 0, s, scores, p.ld, t, scale, stats);
    // 3. weighted sums in the rotated domain (PolarQuant values: of y~)
    if (vt.polar) {
        PolarValueArgs pa;
        pa.scores = scores;
        pa.ld = p.ld;
        pa.stats = stats;
        pa.scale = scale;
        pa.words = vcodes;
        pa.t = t;
        pa.kv_stride = kv_stride;
        pa.group = group;
        pa.rows = hq;
        pa.part = part;
        const hipError_t e = polar_attend_values(vt.pol, pa, static_cast<int>(p.producers), kv_heads, s);
        if (e != hipSuccess) return e;
    }
    AttendArgs a;
    a.scores = scores;
    a.ld = p.ld;
    a.stats = stats;
    a.scale = scale;
    a.codes = vcodes;
    a.norms = vnorms;
    a.signs = vsigns;
    a.rnorms = vrnorms;
    a.t = t;
    a.kv_stride = kv_stride;
    a.group = group;
    a.rows = hq;
    a.cent = vt.dense ? vt.den.cent : vt.rot.cent;
    a.part = part;
    a.pt = vpt;
    hipError_t e = hipSuccess;
    if (vt.polar) {
        // (done above)
    } else if (vt.dense)
        e = vt.qjl ? launch_values_b<true, false>(vt.mse_bits, a, p, kv_heads, s)
                   : launch_values_b<false, false>(vt.mse_bits, a, p, kv_heads, s);
    else
        e = vt.qjl ? launch_values_b<true, true>(vt.mse_bits, a, p, kv_heads, s)
                   : launch_values_b<false, true>(vt.mse_bits, a, p, kv_heads, s);
    if (e != hipSuccess) return e;
    // 4. combine
    CombineArgs c;
    c.part = part;
    c.producers = p.producers;
    c.rows = hq;
    c.stats = stats;
    c.rotor = !vt.dense && !vt.polar;
    c.qjl = vt.qjl;
    c.rotmat = vt.rot.rotmat;
    c.pi_hi = vt.polar ? vt.pol.pi_hi : vt.den.pi_hi;   // x~ = Pi^T (sums)
    c.pi_lo = vt.polar ? vt.pol.pi_lo : vt.den.pi_lo;
    c.s_rows = vt.dense ? vt.den.s_rows : vt.rot.s_rows;
    c.kappa = vt.qjl_scale;
    c.out = out;
    c.ld_out = ld_out;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(hq), dim3(320), 0, s, c);
    return hipGetLastError();
}

}  // namespace rqk
