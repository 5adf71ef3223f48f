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
// centroid / sign matrices [keys x coordinates] and run on MFMAs (32x32x16
// fp16 for groups of more than 16 query rows; 16x16x32, the signs in bf16,
// for smaller groups); X^T and S^T are applied once per query row at the end.  PolarQuant
// values are the one kind decoded (to y~ = Pi x~, in rq_polar.hip's value
// pass): sum_t p_t v~_t = Pi^T (sum_t p_t y~_t), Pi^T once per row.  PolarQuant
// keys are scored by pq_score in pass 1.
//
// Passes (all on the caller's stream, workspace from the caller):
//   1. the estimates s (rq_score's kernel) into the workspace;
//   2. per row M = max scale*s and L = sum exp(scale*s - M) (one pass, the
//      running-maximum form);
//   3. per (KV head, <= 32 rows, key slice) wave: the two weighted sums over
//      its tiles in the rotated domain, written as partial rows (one launch
//      for groups of at most 16 rows, else one per sum);
//   4. per row: sum the partials in a fixed order, apply X^T and kappa S^T,
//      divide by L.
#include "rq_common_dev.h"
#include "rq_kernels.h"

#include <mutex>

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
    // groups of at most 16 rows, row statistics taken here: the scoring
    // launch's per-workgroup maxima ([rm_n][rm_ld]) instead of stats; the
    // partial rows then carry their sums of weights and the row maximum
    const float* rowmax = nullptr;
    int64_t rm_ld = 0;
    int rm_n = 0;
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
//
// Per tile, the weights (p n^ for the centroid sums, p n^ gamma^ for the
// sign sums) are computed only for the block's live query rows: lane l takes
// key pair l % 32 of rows l / 32, l / 32 + 2, ..., and writes the split
// halves to a per-wave table that the MFMA A fragments read (rows past the
// live ones are zero operands).
template <int B, bool QJL, bool PAD, bool CODES = true>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CODES ? 2 : 3))) void attend_values_kernel(
    AttendArgs a) {
    static_assert(CODES != QJL, "one kind of sum per pass");
    constexpr int L = 1 << B;
    constexpr int W = CODES ? (((PAD ? kRotCoords : kD) * B) + 31) / 32 : 1;
    constexpr int WTS = 36;   // weight-table row pitch (dwords): conflict-free 16-byte reads
    struct alignas(16) Wave {
        uint32_t code[W + 1][68];   // [word][key] (rows 68 apart: lanes reading different words of
                                    // the same keys hit different banks); a spare row for straddles
        uint32_t sign[4][68];       // [word][key], rows padded like the code rows
        alignas(16) uint16_t nrm[64];
        alignas(16) uint16_t gam[64];
    };
    struct WaveW {
        uint32_t hi[32][WTS];       // [row][key pair]: fp16 hi of the weights of keys 2q, 2q+1
        uint32_t lo[32][WTS];       // lo11 = half((w - hi) 2^11)
    };
    struct Lds {
        // codes (k, k+1) -> C_lo and C_hi half pairs at [p] and [257 + p]: 1,028
        // bytes apart, so no two-address LDS read fetches both together and
        // each lands in its own MFMA operand without moves (2^11 C_hi is one
        // packed multiply of C_hi)
        uint32_t ptab[CODES ? 2 * 257 : 1];
        float centf[PAD ? L : 1];      // the centroids (rotor pad slot, summed on the VALU)
        // two keys' four sign bits (key a: bits 0..3, key b: bits 4..7) -> for
        // each of the four bit positions nt, the +-1 half pair (sigma_a, sigma_b)
        u32x4 sig[QJL ? 256 : 1];
        Wave w[4];
        union {
            WaveW wt[4];                  // tile loop: per-wave weight tables
            float sum[32][kPartStride];   // after it: the block's partial rows, waves added in order
        };
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
            lds.ptab[p] = l0 | (l1 << 16);
            lds.ptab[257 + p] = h0 | (h1 << 16);
        }
        for (int i = threadIdx.x; i < 4 * 64; i += kBlock) lds.w[i >> 6].code[W][i & 63] = 0u;
        if constexpr (PAD) {
            if (threadIdx.x < L) lds.centf[threadIdx.x] = a.cent[threadIdx.x];
        }
    }
    if constexpr (QJL) {
        // sigma = 2 bit - 1 as half pairs; the sign bit is set where the stored bit is 0
        for (int p = threadIdx.x; p < 256; p += kBlock) {
            u32x4 e;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const uint32_t ba = (p >> nt) & 1u, bb = (p >> (4 + nt)) & 1u;
                e[nt] = 0x3C003C00u | ((ba ^ 1u) << 15) | ((bb ^ 1u) << 31);
            }
            lds.sig[p] = e;
        }
    }
    __syncthreads();

    Wave& wv = lds.w[wave];
    WaveW& wt = lds.wt[wave];
    const int l = lane_id();
    const int n = l & 31, hh = l >> 5;
    const bool live = n < nrows;
    const rsrc_t rsc = make_rsrc(a.scores + static_cast<int64_t>(row0) * a.ld,
                                 static_cast<uint32_t>(nrows * a.ld * 4));
    // the weight rows of this lane: l / 32 + 2 i for i < ri, key pair l % 32
    const int ri = (nrows - hh + 1) >> 1;
    float mrow[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mrow[i] = i < ri ? a.stats[row0 + hh + 2 * i].x : 0.0f;

    f32x16 acc_c[4], acc_s[4];
    // rotor pad slot: sum of p n^ c[code of slot 128] of rows hh + 2 i over this lane's keys
    float padacc[PAD ? 16 : 1];
#pragma unroll
    for (int i = 0; i < (PAD ? 16 : 1); ++i) padacc[i] = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        acc_c[nt] = f32x16{};
        acc_s[nt] = f32x16{};
    }

    // One tile's inputs in registers: this lane's row of estimates (keys
    // 16 kb + 8 hh .. + 7 of each K block) and dword l of the tile's code,
    // sign and norm runs.  They are fetched one tile ahead of their use, so
    // each tile's load latency hides behind the previous tile's arithmetic.
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    struct TileIn {
        u32x2 sp[16];
        uint32_t cw[W];
        uint32_t sw[4];
        uint32_t nb, gb;
    };
    auto fetch = [&](int64_t tile, TileIn& r) {
        const int64_t kbase = tile * 64;
        // estimates of keys 2 n, 2 n + 1 of rows hh + 2 i (rows past nrows lie
        // outside rsc's range and read as zero)
        const uint32_t soff = static_cast<uint32_t>((hh * a.ld + kbase + 2 * n) * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i < ri) r.sp[i] = __builtin_amdgcn_raw_buffer_load_b64(rsc, soff, static_cast<int>(2 * i * a.ld * 4),
                                                                       kNonTemporal);
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
        u32x2 sp[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sp[i] = nx.sp[i];
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
        // weights of the live rows into the table
        {
            const uint32_t nn = *reinterpret_cast<const uint32_t*>(&wv.nrm[2 * n]);
            uint32_t gg = 0u;
            if constexpr (QJL) gg = *reinterpret_cast<const uint32_t*>(&wv.gam[2 * n]);
            const float n0 = h2f(nn & 0xFFFFu), n1 = h2f(nn >> 16);
            const float ga = h2f(gg & 0xFFFFu), gb = h2f(gg >> 16);
            const bool in0 = 2 * n < kleft, in1 = 2 * n + 1 < kleft;
            float cp0 = 0.0f, cp1 = 0.0f;   // centroids of the pad slot of keys 2 n, 2 n + 1
            if constexpr (PAD) {
                cp0 = lds.centf[wv.code[4 * B][2 * n] & (L - 1)];
                cp1 = lds.centf[wv.code[4 * B][2 * n + 1] & (L - 1)];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i < ri) {
                    const uint32_t b0 = sp[i][0];
                    const uint32_t b1 = sp[i][1];
                    const float s0 = __builtin_bit_cast(float, b0), s1 = __builtin_bit_cast(float, b1);
                    const float e0 = in0 ? exp2_hw((s0 * a.scale - mrow[i]) * kLog2e) : 0.0f;
                    const float e1 = in1 ? exp2_hw((s1 * a.scale - mrow[i]) * kLog2e) : 0.0f;
                    float w0 = e0 * n0, w1 = e1 * n1;   // p n^ (sign pass: p n^ gamma^)
                    if constexpr (QJL) {
                        w0 = w0 * ga;
                        w1 = w1 * gb;
                    }
                    if constexpr (PAD) padacc[i] = __builtin_fmaf(w1, cp1, __builtin_fmaf(w0, cp0, padacc[i]));
                    uint32_t h, lo;
                    split_pair11(w0, w1, &h, &lo);
                    wt.hi[hh + 2 * i][n] = h;
                    wt.lo[hh + 2 * i][n] = lo;
                }
            }
        }
        wave_lds_sync();
        if (tile + tstep < ntiles) fetch(tile + tstep, nx);

#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int k0 = 16 * kb + 8 * hh;
            // A operands: row n's weights of keys k0..k0+7 (zero past the live rows)
            u32x4 wh{}, wl{};
            if (live) {
                wh = *reinterpret_cast<const u32x4*>(&wt.hi[n][8 * kb + 4 * hh]);
                wl = *reinterpret_cast<const u32x4*>(&wt.lo[n][8 * kb + 4 * hh]);
            }
            const u32x4 gwh = wh, gwl = wl;
            // centroid operands: column n of N tile nt is coordinate 4 n + nt, so
            // the lane's four coordinates share one field of 4 B bits per key,
            // read once per K block
            if constexpr (CODES) {
                const int bit = 4 * B * n, wi = bit >> 5, off = bit & 31;
                const u32x4 w0a = *reinterpret_cast<const u32x4*>(&wv.code[wi][k0]);
                const u32x4 w0b = *reinterpret_cast<const u32x4*>(&wv.code[wi][k0 + 4]);
                u32x4 w1a{}, w1b{};
                if constexpr (32 % (4 * B) != 0) {
                    w1a = *reinterpret_cast<const u32x4*>(&wv.code[wi + 1][k0]);
                    w1b = *reinterpret_cast<const u32x4*>(&wv.code[wi + 1][k0 + 4]);
                }
                uint32_t fld[8];   // keys k0..k0+7: their codes of coordinates 4 n .. 4 n + 3 from bit 0
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t x0 = k < 4 ? w0a[k] : w0b[k - 4];
                    if constexpr (32 % (4 * B) != 0) {
                        const uint32_t x1 = k < 4 ? w1a[k] : w1b[k - 4];
                        fld[k] = __builtin_amdgcn_alignbit(x1, x0, off);
                    } else {
                        fld[k] = x0 >> off;
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    u32x4 b11, blo, bhi;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t f0 = (fld[2 * q] >> (B * nt)) & (L - 1);
                        const uint32_t f1 = (fld[2 * q + 1] >> (B * nt)) & (L - 1);
                        const uint32_t ix = f0 | (f1 << B);
                        const uint32_t hp = lds.ptab[257 + ix];
                        blo[q] = lds.ptab[ix];
                        bhi[q] = hp;
                        b11[q] = pk_scale2048(hp);
                    }
                    acc_c[nt] = mfma(wh, b11, acc_c[nt]);
                    acc_c[nt] = mfma(wh, blo, acc_c[nt]);
                    acc_c[nt] = mfma(wl, bhi, acc_c[nt]);
                }
            }
            if constexpr (QJL) {
                // sign operands: column n of N tile nt is sign index 4 n + nt, so
                // each key's four bits of the lane lie in one nibble of one word;
                // +-2^11 (hi) is a packed multiply of +-1 (lo11)
                const u32x4 sa = *reinterpret_cast<const u32x4*>(&wv.sign[n >> 3][k0]);
                const u32x4 sb = *reinterpret_cast<const u32x4*>(&wv.sign[n >> 3][k0 + 4]);
                const int sh = 4 * (n & 7);
                u32x4 s1[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t xa = q < 2 ? sa[2 * q] : sb[2 * q - 4];
                    const uint32_t xb = q < 2 ? sa[2 * q + 1] : sb[2 * q - 3];
                    const uint32_t pb = ((xa >> sh) & 0xFu) | (((xb >> sh) & 0xFu) << 4);
                    const u32x4 e = lds.sig[pb];
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const uint32_t en = e[nt];
                        s1[nt][q] = en;
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    u32x4 s11;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t v = s1[nt][q];
                        s11[q] = pk_scale2048(v);
                    }
                    acc_s[nt] = mfma(gwh, s11, acc_s[nt]);
                    acc_s[nt] = mfma(gwl, s1[nt], acc_s[nt]);
                }
            }
        }
    }

    // the block's partial rows: the four waves' sums are added in wave order
    // through LDS (over the weight tables, once every wave has left its tiles),
    // then written as producer blockIdx.x
    __syncthreads();
    // pad slot: this half-wave's 32 key pairs added in a fixed butterfly order
    if constexpr (PAD) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) padacc[i] += __shfl_xor(padacc[i], off);
    }
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
                            dst[4 * n + nt] = w == 0 ? c : dst[4 * n + nt] + c;
                        }
                        if constexpr (QJL) {
                            const float g = acc_s[nt][r] * us;
                            dst[kPartSigma + 4 * n + nt] = w == 0 ? g : dst[kPartSigma + 4 * n + nt] + g;
                        }
                    }
                }
            }
            if (CODES && n == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (i < ri) {
                        float* dst = lds.sum[hh + 2 * i];
                        float pc = 0.0f;
                        if constexpr (PAD) pc = padacc[i];
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

// Exact split of a pair into bf16 hi = bf16(x) and lo = bf16(x - hi) (both
// round to nearest even; x - hi is exact in fp32): x = hi + lo to 2^-18.
__device__ __forceinline__ void split_pair_bf16(float a, float b, uint32_t* hi, uint32_t* lo) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
    const float ha = __builtin_bit_cast(float, h << 16), hb = __builtin_bit_cast(float, h & 0xFFFF0000u);
    *hi = h;
    *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a - ha, b - hb}), bf16x2));
}
__device__ __forceinline__ f32x4 mfma16_bf(const u32x4& a, const u32x4& b, const f32x4& c) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

// 8x8 bit matrix held in (lo, hi), row k = byte k (bytes 0..3 in lo, 4..7 in
// hi), column j = bit j: transposed in place by three rounds of masked swaps
// (1x1, 2x2 and 4x4 blocks), so that afterwards byte j holds column j.
__device__ __forceinline__ void transpose8x8(uint32_t& lo, uint32_t& hi) {
    uint32_t t;
    t = (lo ^ (lo >> 7)) & 0x00AA00AAu;
    lo ^= t ^ (t << 7);
    t = (hi ^ (hi >> 7)) & 0x00AA00AAu;
    hi ^= t ^ (t << 7);
    t = (lo ^ (lo >> 14)) & 0x0000CCCCu;
    lo ^= t ^ (t << 14);
    t = (hi ^ (hi >> 14)) & 0x0000CCCCu;
    hi ^= t ^ (t << 14);
    t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
    lo ^= t;
    hi ^= t >> 4;
}

// 8x8 matrix of 2-bit elements in d[0..3], row r in bits 16 (r % 2) .. + 15
// of d[r / 2], element c of a row at bits 2 c, 2 c + 1: transposed in place
// (masked swaps of 1x1, 2x2 and 4x4 blocks).
__device__ __forceinline__ void transpose8x8_2b(uint32_t (&d)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = ((d[i] >> 14) ^ d[i]) & 0x0000CCCCu;
        d[i] ^= t ^ (t << 14);
    }
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        const uint32_t t = ((d[i] >> 4) ^ d[i + 1]) & 0x0F0F0F0Fu;
        d[i + 1] ^= t;
        d[i] ^= t << 4;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t t = ((d[i] >> 8) ^ d[i + 2]) & 0x00FF00FFu;
        d[i + 2] ^= t;
        d[i] ^= t << 8;
    }
}

// Groups of at most 16 query rows (GQA 4:1 and 8:1): both weighted sums in
// one pass over the tiles, on 16x16x32 MFMAs whose M dimension is the
// group's rows (a 32-row M tile would carry 4 or 8 live rows of 32).  Per
// 64-key tile each wave stages the records key-minor in LDS and writes the
// weights of the live rows (p n^, and with QJL p n^ gamma^) to its tables as
// the two-pass kernel does; then two K steps of 32 keys: lane (c, g) =
// (l % 16, l / 16) holds keys 32 ks + 8 g .. + 7 and, in N tile nt,
// coordinate (sign index) 8 c + nt, so the lane's eight coordinates share
// one field of 8 B code bits per key and one byte of its sign bits.  The
// sign sums run on bf16 MFMAs: +-1 is exact in bf16, so the exact split of
// the weight into bf16 hi + lo (2^-18 relative) multiplies one shared B
// operand, which is built on the VALU from the eight keys' sign bytes (a
// shift, a mask and byte permutes: LDS bandwidth bounds this loop, so no
// table).  The scores, norms and the staging are read once for both sums.
template <int B, bool QJL, bool PAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attend_values16_kernel(AttendArgs a) {
    constexpr int L = 1 << B;
    constexpr int W = (((PAD ? kRotCoords : kD) * B) + 31) / 32;
    constexpr int WTS = 36;               // weight-table row pitch (dwords)
    constexpr int NK = QJL ? 2 : 1;       // weight kinds: p n^, p n^ gamma^
    constexpr bool STR = 32 % (8 * B) != 0;   // 3-bit fields straddle code words
    // 1- and 2-bit codes: the lane's 8 x 8 block of codes (keys x coordinates)
    // is transposed, so that four keys' codes of one coordinate form the index
    // of a table entry holding their four C_lo (or C_hi) halves
    constexpr bool QV = B <= 2;
    constexpr int NQV = QV ? 1 << (4 * B) : 1;
    struct alignas(16) Wave {
        uint32_t code[W + 1][68];         // [word][key], as in the two-pass kernel
        uint32_t sign[QJL ? 4 : 1][68];
        alignas(16) uint16_t nrm[64];
        alignas(16) uint16_t gam[64];
    };
    struct WaveW {
        // [kind][row][key pair]: the weights of keys 2 q, 2 q + 1 split as fp16
        // hi and lo11 = half((w - hi) 2^11) (kind 0), bf16 hi and lo (kind 1)
        uint32_t hi[NK][16][WTS];
        uint32_t lo[NK][16][WTS];
    };
    struct Lds {
        // code pairs -> C_lo at [p], C_hi at [257 + p] (1,028 bytes apart: no
        // two-address read pairs them); 1- and 2-bit codes: four codes -> C_lo
        // halves at qtab[p], C_hi at qtab[257 + p] (2,056 bytes apart)
        uint32_t ptab[QV ? 1 : 2 * 257];
        uint2 qtab[QV ? 257 + NQV : 1];
        float centf[PAD ? L : 1];
        Wave w[4];
        union {
            WaveW wt[4];
            float sum[16][kPartStride];
        };
    };
    __shared__ Lds lds;

    const int kvh = blockIdx.y;            // one row block per KV head
    const int row0 = kvh * a.group;
    const int nrows = a.group;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t rbase = static_cast<int64_t>(kvh) * a.kv_stride;
    const int64_t ntiles = (a.t + 63) / 64;

    const float cmax = fmaxf(fabsf(a.cent[L - 1]), fabsf(a.cent[0]));
    int ce;
    frexpf(cmax, &ce);
    const float sc = cmax > 0.0f ? ldexpf(1.0f, 1 - ce) : 1.0f;   // |sc c| in [1, 2) at most
    if constexpr (QV) {
        for (int p = threadIdx.x; p < NQV; p += kBlock) {
            uint32_t h[4], o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) split_h11(a.cent[(p >> (B * k)) & (L - 1)] * sc, &h[k], &o[k]);
            lds.qtab[p] = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            lds.qtab[257 + p] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    } else {
        for (int p = threadIdx.x; p < L * L; p += kBlock) {
            uint32_t h0, l0, h1, l1;
            split_h11(a.cent[p & (L - 1)] * sc, &h0, &l0);
            split_h11(a.cent[p >> B] * sc, &h1, &l1);
            lds.ptab[p] = l0 | (l1 << 16);
            lds.ptab[257 + p] = h0 | (h1 << 16);
        }
    }
    for (int i = threadIdx.x; i < 4 * 64; i += kBlock) lds.w[i >> 6].code[W][i & 63] = 0u;
    if constexpr (PAD) {
        if (threadIdx.x < L) lds.centf[threadIdx.x] = a.cent[threadIdx.x];
    }
    __syncthreads();

    Wave& wv = lds.w[wave];
    WaveW& wt = lds.wt[wave];
    const int l = lane_id();
    const int n = l & 31, hh = l >> 5;    // weights: key pair n of rows hh + 2 i
    const int c = l & 15, g = l >> 4;     // MFMA operands
    // byte c % 4 of two sign words into bytes 0, 1 (selA) or 2, 3 (selB) of a dword
    const uint32_t sb4 = static_cast<uint32_t>(c & 3);
    const uint32_t selA = sb4 | ((4u + sb4) << 8) | 0x0C0C0000u;
    const uint32_t selB = 0x00000C0Cu | (sb4 << 16) | ((4u + sb4) << 24);
    const bool live = c < nrows;
    const rsrc_t rsc = make_rsrc(a.scores + static_cast<int64_t>(row0) * a.ld,
                                 static_cast<uint32_t>(nrows * a.ld * 4));
    const int ri = (nrows - hh + 1) >> 1;
    // row maxima: from the row statistics, or (rowmax) over the scoring
    // launch's workgroups, reduced through LDS before the tile loop
    const bool fused = a.rowmax != nullptr;
    if (fused) {
        const int r = threadIdx.x & 15, b0 = threadIdx.x >> 4;
        float m = -INFINITY;
        if (r < nrows)
            for (int b = b0; b < a.rm_n; b += kBlock / 16) m = fmaxf(m, a.rowmax[b * a.rm_ld + row0 + r]);
        lds.sum[r][b0] = m;
        __syncthreads();
        if (threadIdx.x < 16) {
            float mm = lds.sum[threadIdx.x][0];
            for (int b = 1; b < kBlock / 16; ++b) mm = fmaxf(mm, lds.sum[threadIdx.x][b]);
            lds.sum[threadIdx.x][kPartStride - 1] = mm;
        }
        __syncthreads();
    }
    float mrow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        mrow[i] = i < ri ? (fused ? lds.sum[hh + 2 * i][kPartStride - 1] : a.stats[row0 + hh + 2 * i].x) : 0.0f;
    // (fused) this lane's sum of exp(scale s - M) of rows hh + 2 i over its keys
    float lsum[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) lsum[i] = 0.0f;
    __syncthreads();   // the maxima are read before the weight tables take their place

    f32x4 acc_c[8], acc_s[QJL ? 8 : 1];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc_c[nt] = f32x4{};
#pragma unroll
    for (int nt = 0; nt < (QJL ? 8 : 1); ++nt) acc_s[nt] = f32x4{};
    float padacc[PAD ? 8 : 1];
#pragma unroll
    for (int i = 0; i < (PAD ? 8 : 1); ++i) padacc[i] = 0.0f;

    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    struct TileIn {
        u32x2 sp[8];
        uint32_t cw[W];
        uint32_t sw[4];
        uint32_t nb, gb;
    };
    auto fetch = [&](int64_t tile, TileIn& r) {
        const int64_t kbase = tile * 64;
        const uint32_t soff = static_cast<uint32_t>((hh * a.ld + kbase + 2 * n) * 4);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < ri) r.sp[i] = __builtin_amdgcn_raw_buffer_load_b64(rsc, soff, static_cast<int>(2 * i * a.ld * 4),
                                                                      kNonTemporal);
        const int64_t left = a.t - kbase;
        int64_t row = rbase + kbase;
        if (a.pt.pages != nullptr) {
            const int64_t pg = a.pt.pages[kvh * a.pt.stride + (kbase >> a.pt.shift)];
            row = (pg << a.pt.shift) + (kbase & ((int64_t(1) << a.pt.shift) - 1));
        }
        const rsrc_t rc = make_rsrc(a.codes + row * W, tile_range(left, 4 * W));
#pragma unroll
        for (int it = 0; it < W; ++it)
            r.cw[it] = __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
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
        const int kleft = static_cast<int>(a.t - kbase < 64 ? a.t - kbase : 64);
        u32x2 sp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sp[i] = nx.sp[i];
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < W; ++it) {
            const int d = it * 64 + l;
            wv.code[d % W][d / W] = nx.cw[it];
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
        {
            const uint32_t nn = *reinterpret_cast<const uint32_t*>(&wv.nrm[2 * n]);
            uint32_t gg = 0u;
            if constexpr (QJL) gg = *reinterpret_cast<const uint32_t*>(&wv.gam[2 * n]);
            const float n0 = h2f(nn & 0xFFFFu), n1 = h2f(nn >> 16);
            const float ga = h2f(gg & 0xFFFFu), gb = h2f(gg >> 16);
            const bool in0 = 2 * n < kleft, in1 = 2 * n + 1 < kleft;
            float cp0 = 0.0f, cp1 = 0.0f;   // centroids of the pad slot of keys 2 n, 2 n + 1
            if constexpr (PAD) {
                cp0 = lds.centf[wv.code[4 * B][2 * n] & (L - 1)];
                cp1 = lds.centf[wv.code[4 * B][2 * n + 1] & (L - 1)];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i < ri) {
                    const uint32_t b0 = sp[i][0];
                    const uint32_t b1 = sp[i][1];
                    const float s0 = __builtin_bit_cast(float, b0), s1 = __builtin_bit_cast(float, b1);
                    const float e0 = in0 ? exp2_hw((s0 * a.scale - mrow[i]) * kLog2e) : 0.0f;
                    const float e1 = in1 ? exp2_hw((s1 * a.scale - mrow[i]) * kLog2e) : 0.0f;
                    const float w0 = e0 * n0, w1 = e1 * n1;
                    lsum[i] += e0 + e1;
                    if constexpr (PAD) padacc[i] = __builtin_fmaf(w1, cp1, __builtin_fmaf(w0, cp0, padacc[i]));
                    uint32_t h, lo;
                    split_pair11(w0, w1, &h, &lo);
                    wt.hi[0][hh + 2 * i][n] = h;
                    wt.lo[0][hh + 2 * i][n] = lo;
                    if constexpr (QJL) {
                        split_pair_bf16(w0 * ga, w1 * gb, &h, &lo);
                        wt.hi[NK - 1][hh + 2 * i][n] = h;
                        wt.lo[NK - 1][hh + 2 * i][n] = lo;
                    }
                }
            }
        }
        wave_lds_sync();
        if (tile + tstep < ntiles) fetch(tile + tstep, nx);

#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k0 = 32 * ks + 8 * g;   // the lane's first key of this K step
            // A operands: row c's weights of keys k0 .. k0 + 7 (zero past the live rows)
            u32x4 wh{}, wl{};
            if (live) {
                wh = *reinterpret_cast<const u32x4*>(&wt.hi[0][c][16 * ks + 4 * g]);
                wl = *reinterpret_cast<const u32x4*>(&wt.lo[0][c][16 * ks + 4 * g]);
            }
            {
                const int bit = 8 * B * c, wi = bit >> 5, off = bit & 31;
                const u32x4 w0a = *reinterpret_cast<const u32x4*>(&wv.code[wi][k0]);
                const u32x4 w0b = *reinterpret_cast<const u32x4*>(&wv.code[wi][k0 + 4]);
                u32x4 w1a{}, w1b{};
                if constexpr (STR) {
                    w1a = *reinterpret_cast<const u32x4*>(&wv.code[wi + 1][k0]);
                    w1b = *reinterpret_cast<const u32x4*>(&wv.code[wi + 1][k0 + 4]);
                }
                uint32_t fld[8];   // keys k0 .. k0 + 7: codes of coordinates 8 c .. 8 c + 7 from bit 0
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t x0 = k < 4 ? w0a[k] : w0b[k - 4];
                    if constexpr (STR) {
                        const uint32_t x1 = k < 4 ? w1a[k] : w1b[k - 4];
                        fld[k] = __builtin_amdgcn_alignbit(x1, x0, off);
                    } else {
                        fld[k] = x0 >> off;
                    }
                }
                if constexpr (QV) {
                    // rows of the transposed block: the 8 keys' codes of
                    // coordinate 8 c + nt, key k at bit B k
                    uint32_t tr[4];
                    if constexpr (B == 2) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) tr[i] = __builtin_amdgcn_perm(fld[2 * i + 1], fld[2 * i], 0x05040100u);
                        transpose8x8_2b(tr);
                    } else {
                        tr[0] = __builtin_amdgcn_perm(fld[1], fld[0], 0x0C0C0400u) |
                                __builtin_amdgcn_perm(fld[3], fld[2], 0x04000C0Cu);
                        tr[1] = __builtin_amdgcn_perm(fld[5], fld[4], 0x0C0C0400u) |
                                __builtin_amdgcn_perm(fld[7], fld[6], 0x04000C0Cu);
                        transpose8x8(tr[0], tr[1]);
                    }
                    // table reads run one N tile ahead of their MFMAs
                    u32x4 blo[2], bhi[2];
                    auto qread = [&](int nt, u32x4& lo4, u32x4& hi4) __attribute__((always_inline)) {
                        const uint32_t v = B == 2 ? tr[nt >> 1] >> (16 * (nt & 1)) : tr[nt >> 2] >> (8 * (nt & 3));
                        const uint32_t i0 = v & (NQV - 1), i1 = (v >> (4 * B)) & (NQV - 1);
                        const uint2 l0 = lds.qtab[i0], l1 = lds.qtab[i1];
                        const uint2 h0 = lds.qtab[257 + i0], h1 = lds.qtab[257 + i1];
                        lo4 = u32x4{l0.x, l0.y, l1.x, l1.y};
                        hi4 = u32x4{h0.x, h0.y, h1.x, h1.y};
                    };
                    qread(0, blo[0], bhi[0]);
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (nt < 7) qread(nt + 1, blo[(nt + 1) & 1], bhi[(nt + 1) & 1]);
                        const u32x4 lo4 = blo[nt & 1], hi4 = bhi[nt & 1];
                        u32x4 b11;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t hq = hi4[q];
                            b11[q] = pk_scale2048(hq);
                        }
                        acc_c[nt] = mfma16(wh, b11, acc_c[nt]);
                        acc_c[nt] = mfma16(wh, lo4, acc_c[nt]);
                        acc_c[nt] = mfma16(wl, hi4, acc_c[nt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                } else {
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    u32x4 b11, blo, bhi;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t f0 = (fld[2 * q] >> (B * nt)) & (L - 1);
                        const uint32_t f1 = (fld[2 * q + 1] >> (B * nt)) & (L - 1);
                        const uint32_t ix = f0 | (f1 << B);
                        const uint32_t hp = lds.ptab[257 + ix];
                        blo[q] = lds.ptab[ix];
                        bhi[q] = hp;
                        b11[q] = pk_scale2048(hp);
                    }
                    acc_c[nt] = mfma16(wh, b11, acc_c[nt]);
                    acc_c[nt] = mfma16(wh, blo, acc_c[nt]);
                    acc_c[nt] = mfma16(wl, bhi, acc_c[nt]);
                }
                }
            }
            if constexpr (QJL) {
                u32x4 swh{}, swl{};
                if (live) {
                    swh = *reinterpret_cast<const u32x4*>(&wt.hi[NK - 1][c][16 * ks + 4 * g]);
                    swl = *reinterpret_cast<const u32x4*>(&wt.lo[NK - 1][c][16 * ks + 4 * g]);
                }
                // sign index 8 c + nt is bit nt of byte c % 4 of sign word c / 4:
                // the eight keys' bytes, transposed, give one table index per N tile
                const u32x4 sa = *reinterpret_cast<const u32x4*>(&wv.sign[c >> 2][k0]);
                const u32x4 sb = *reinterpret_cast<const u32x4*>(&wv.sign[c >> 2][k0 + 4]);
                uint32_t x[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t xa = sa[k], xb = sb[k];
                    x[k] = xa;
                    x[4 + k] = xb;
                }
                const uint32_t glo = __builtin_amdgcn_perm(x[1], x[0], selA) | __builtin_amdgcn_perm(x[3], x[2], selB);
                const uint32_t ghi = __builtin_amdgcn_perm(x[5], x[4], selA) | __builtin_amdgcn_perm(x[7], x[6], selB);
                // byte k of glo / ghi: key k's (k + 4's) byte.  Operand of N tile
                // nt: the high byte of key k's bf16 +-1 is 0x3F or 0xBF by bit nt
                // of that byte, the low byte 0x80; one byte permute per dword
                u32x4 s1[8];
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const uint32_t ylo = ((glo << (7 - nt)) & 0x80808080u) ^ 0xBFBFBFBFu;
                    const uint32_t yhi = ((ghi << (7 - nt)) & 0x80808080u) ^ 0xBFBFBFBFu;
                    s1[nt] = u32x4{__builtin_amdgcn_perm(ylo, 0x80808080u, 0x05000400u),
                                   __builtin_amdgcn_perm(ylo, 0x80808080u, 0x07000600u),
                                   __builtin_amdgcn_perm(yhi, 0x80808080u, 0x05000400u),
                                   __builtin_amdgcn_perm(yhi, 0x80808080u, 0x07000600u)};
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    acc_s[nt] = mfma16_bf(swh, s1[nt], acc_s[nt]);
                    acc_s[nt] = mfma16_bf(swl, s1[nt], acc_s[nt]);
                }
            }
        }
    }

    // the block's partial rows: the four waves' sums added in wave order
    // through LDS (over the weight tables, once every wave has left its
    // tiles), then written as producer blockIdx.x
    __syncthreads();
    if constexpr (PAD) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) padacc[i] += __shfl_xor(padacc[i], off);
    }
    if (fused) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) lsum[i] += __shfl_xor(lsum[i], off);
    }
    const float uc = 1.0f / (2048.0f * sc);
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * g + i;
                if (m < nrows) {
                    float* dst = lds.sum[m];
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) {
                        const int col = 8 * c + nt;
                        const float cv = acc_c[nt][i] * uc;
                        dst[col] = w == 0 ? cv : dst[col] + cv;
                        if constexpr (QJL) {
                            const float sv = acc_s[nt][i];
                            dst[kPartSigma + col] = w == 0 ? sv : dst[kPartSigma + col] + sv;
                        }
                    }
                }
            }
            if (n == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i < ri) {
                        float* dst = lds.sum[hh + 2 * i];
                        float pc = 0.0f;
                        if constexpr (PAD) pc = padacc[i];
                        dst[kPartPad] = w == 0 ? pc : dst[kPartPad] + pc;
                        dst[kPartPad + 1] = w == 0 ? lsum[i] : dst[kPartPad + 1] + lsum[i];
                        dst[kPartPad + 2] = mrow[i];
                    }
                }
            }
        }
        __syncthreads();
    }
    float* out = a.part + (static_cast<int64_t>(blockIdx.x) * a.rows + row0) * kPartStride;
    // columns: centroid sums, (QJL) sign sums, the pad slot, and (fused) the
    // sum of weights and the row maximum
    for (int i = threadIdx.x; i < nrows * kPartStride; i += kBlock) {
        const int m = i / kPartStride, col = i % kPartStride;
        const bool sig = col >= kPartSigma && col < kPartSigma + kD;
        const bool keep = sig || col < kPartSigma || col == kPartPad || (fused && col <= kPartPad + 2);
        if (!sig || QJL) out[static_cast<int64_t>(m) * kPartStride + col] = keep ? lds.sum[m][col] : 0.0f;
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
    // the partial rows carry the sums of weights (column kPartPad + 1) and the
    // row maximum (kPartPad + 2): their sum and that maximum are written to
    // stats_out, which takes the place of the row statistics pass
    float2* stats_out = nullptr;
};

__global__ __launch_bounds__(320) void attend_combine_kernel(CombineArgs a) {
    const int row = blockIdx.x;
    __shared__ float oc[kRotCoords + 3];
    __shared__ float os[kD];
    __shared__ float lsum;
    const int j = threadIdx.x;
    const bool fused = a.stats_out != nullptr;
    // producers in a fixed order: eight interleaved running sums (loads in
    // flight together), added pairwise at the end
    const int col = j < kD ? j : (j < 2 * kD ? kPartSigma + (j - kD) : kPartPad + (j - 2 * kD));
    if (fused && j == 2 * kD + 1) {
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        const int64_t pstride = static_cast<int64_t>(a.rows) * kPartStride;
        const float* src = a.part + static_cast<int64_t>(row) * kPartStride + col;
        int64_t p = 0;
        for (; p + 8 <= a.producers; p += 8)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] += src[(p + u) * pstride];
        for (int u = 0; p < a.producers; ++p, ++u) acc[u] += src[p * pstride];
        lsum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    } else if (j < 2 * kD + 1 && (j < kD || j == 2 * kD || a.qjl)) {
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
        a.out[row * a.ld_out + j] = x / (fused ? lsum : a.stats[row].y);
        if (fused && j == 0)
            a.stats_out[row] = make_float2(a.part[static_cast<int64_t>(row) * kPartStride + kPartPad + 2], lsum);
    }
}

// ----------------------------------------------------------- launchers --
AttendPlan attend_plan(int hq, int group, int64_t t, int plan_rows) {
    AttendPlan p;
    p.ld = (t + 3) & ~int64_t(3);
    const int kv_heads = (plan_rows > 0 ? plan_rows : hq) / group;
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
    p.off_rowmax = p.off_part + up(p.producers * hq * kPartStride * 4);
    // groups of at most 16 rows: the scoring launches' per-workgroup row maxima
    int64_t rm = 0;
    if (group <= 16) {
        const int all = hq / group, chunk = kScoreChunkRows / group;
        const int first = all < chunk ? all : chunk, last = all - (all - 1) / chunk * chunk;
        const int a = score_slices16(t, first), b = score_slices16(t, last);
        rm = static_cast<int64_t>(a > b ? a : b) * hq * 4;
    }
    p.bytes = p.off_rowmax + up(rm);
    return p;
}

// Groups of at most 16 rows: both sums in one pass.  Larger groups:
// centroid sums, then (QJL) sign sums, two passes over the tiles.
template <int B, bool QJL, bool PAD>
static void launch_values(const AttendArgs& a, const AttendPlan& p, int kv_heads, hipStream_t s) {
    if (a.group <= 16) {
        hipLaunchKernelGGL((attend_values16_kernel<B, QJL, PAD>), dim3(p.gx, kv_heads), dim3(kBlock), 0, s, a);
        return;
    }
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
                  hipStream_t s, const PageTable& kpt, const PageTable& vpt, int plan_rows) {
    const AttendPlan p = attend_plan(hq, group, t, plan_rows);
    char* ws = static_cast<char*>(workspace);
    float* scores = reinterpret_cast<float*>(ws + p.off_scores);
    float2* stats = reinterpret_cast<float2*>(ws + p.off_stats);
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    const int kv_heads = hq / group;
    const int heads_per_chunk = group >= kScoreChunkRows ? 1 : kScoreChunkRows / group;
    // Groups of at most 16 rows over rotor or dense keys and values: no row
    // statistics pass.  The scoring launches leave per-workgroup row maxima,
    // the value pass reduces them and sums its weights, and the combine adds
    // those sums (and writes the statistics for later use) -- when every
    // scoring chunk has the same number of workgroups.
    int rm_n = 0;
    bool fused = false;
    if (group <= 16 && !kt.polar && !vt.polar) {
        const int first = kv_heads < heads_per_chunk ? kv_heads : heads_per_chunk;
        const int last = kv_heads - (kv_heads - 1) / heads_per_chunk * heads_per_chunk;
        rm_n = score_slices16(t, first);
        fused = score_slices16(t, last) == rm_n;
    }
    float* rowmax = fused ? reinterpret_cast<float*>(ws + p.off_rowmax) : nullptr;
    // 1. estimates, in chunks of whole KV heads (PolarQuant keys: one launch)
    if (kt.polar) {
        const hipError_t e = polar_score(kt.pol, q, hq, group, kcodes, t, kv_heads > 1 ? kv_stride : 0, scores, p.ld, s);
        if (e != hipSuccess) return e;
    }
    for (int h0 = 0; h0 < (kt.polar ? 0 : kv_heads); h0 += heads_per_chunk) {
        const int nh = kv_heads - h0 < heads_per_chunk ? kv_heads - h0 : heads_per_chunk;
        RowMax rm;
        if (fused) {
            rm.ptr = rowmax + static_cast<int64_t>(h0) * group;
            rm.ld = hq;
            rm.scale = scale;
        }
        const hipError_t e = score(kt, q + static_cast<int64_t>(h0) * group * kD, nh * group, group, kcodes, knorms,
                                   ksigns, krnorms, t, kv_stride, h0, scores + static_cast<int64_t>(h0) * group * p.ld,
                                   p.ld, s, kpt, ScoreOutliers{}, rm);
        if (e != hipSuccess) return e;
    }
    // 2. row statistics
    if (!fused) hipLaunchKernelGGL(attend_stats_kernel, dim3(hq), dim3(kBlock), 0, s, scores, p.ld, t, scale, stats);
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
    a.rowmax = rowmax;
    a.rm_ld = hq;
    a.rm_n = rm_n;
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
    c.stats_out = fused ? stats : nullptr;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(hq), dim3(320), 0, s, c);
    return hipGetLastError();
}

// ------------------------------------------------ fixed scratch buffer --
// The workspace of rq_attend_noalloc: one array per GPU, part of the code
// object, so it exists on every device the library runs on until the
// process ends.  Host code never uses this name as an address (on the host
// it is only a stand-in); it uses the device address hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace rqk
