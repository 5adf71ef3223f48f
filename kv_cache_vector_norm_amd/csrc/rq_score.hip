// q.k estimator over compressed keys (README estimator formula:
//   <q,k> ~ <q,k_mse> + ||r|| sqrt(pi/2)/m <S q, sign(S r)>),
// for grouped-query attention (query row h reads KV head h / group).
//
// <q, x~_mse> is evaluated as <q^, y^> with q^ the forward-rotated query
// (blog section on the random rotation: rotate the query once instead of
// dequantising every key; for rotors M_g^T is the inverse sandwich, so
// <q, M^T y^> = <M q, y^>).  Per key the score is
//   n^ * ( <q^, c[code]> + gamma^ sqrt(pi/2)/m <S q, sigma> ).
//
// Prologue: one block per query row writes q^ and S q as exact half pairs
// with a power-of-two row scale.  Main kernel: each lane decodes one key's
// record once (centroids as exact half pairs, sign bits as +-1 halves), the
// tile's keys become the B operand of 32x32x16 MFMAs whose A operand is the
// staged query rows of one KV head (rows are the GQA group).
#include "rq_common.cuh"
#include "rq_kernels.h"

namespace rqk {

// ---------------------------------------------------------- staged rows --
// Per query row, in 16-byte chunks:
//   Q1 [18 chunks] = 2^11 * hi(s_q q^)   Q2 = hi(s_q q^)   Q3 = lo(s_q q^)
//   P1 [16 chunks] = 2^11 * hi(s_p S q)  P2 = lo(s_p S q)
// with hi(v) = half(v), lo(v) = half((v - hi) * 2^11) (split_h11); q^ has 144 slots
// (129 or 128 used, the rest zero).  Against centroid halves
// C_hi = half(s_c c), C_lo = half((s_c c - C_hi) 2^11):
//   Q1 C_hi + Q2 C_lo + Q3 C_hi = 2^11 s_q s_c <q^, c>  (to ~2^-22 relative),
//   P1 sigma + P2 sigma = 2^11 s_p <S q, sigma>.
constexpr int kQSlots = 144;
constexpr int kQChunks = kQSlots / 8;   // 18
constexpr int kPChunks = 16;
constexpr int kRowChunks = 3 * kQChunks + 2 * kPChunks;   // 86
constexpr int kRowStride = kRowChunks + 1;                 // LDS row pitch (bank spread)
constexpr int kOffQ1 = 0, kOffQ2 = kQChunks, kOffQ3 = 2 * kQChunks, kOffP1 = 3 * kQChunks,
              kOffP2 = 3 * kQChunks + kPChunks;
static_assert(kRowChunks * 16 + 8 <= kScoreQueryBytes, "workspace row too small");

struct ProArgs {
    const float* q;
    int hq;
    bool dense, qjl;
    const float* rotmat;     // rotor: [43][9]
    const uint16_t* pi_hi;   // dense: Pi = (hi + lo 2^-11) / 16, row-major
    const uint16_t* pi_lo;
    const uint16_t* s_rows;  // QJL: S, row-major halves
    u32x4* rows;             // [hq][kRowChunks]
    float* scales;           // [hq][2]: 1 / (2^11 s_q), 1 / (2^11 s_p)
};

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(red[0], red[1]);
    __syncthreads();
    return v;
}

// power-of-two scale putting the largest magnitude in [1, 2)
__device__ __forceinline__ float pow2_scale(float maxabs) {
    if (!(maxabs > 0.0f)) return 1.0f;
    int e;
    frexpf(maxabs, &e);
    return ldexpf(1.0f, 1 - e);
}

__global__ __launch_bounds__(128) void score_prologue(ProArgs a) {
    __shared__ float qs[kD];
    __shared__ float red[2];
    __shared__ uint16_t hv[5][kQSlots];
    const int h = blockIdx.x, i = threadIdx.x;
    qs[i] = a.q[static_cast<int64_t>(h) * kD + i];
    for (int k = i; k < kQSlots; k += 128)
        for (int v = 0; v < 5; ++v) hv[v][k] = 0;
    __syncthreads();
    // rotated query: rotor groups (129 slots) or y = Pi q (128)
    float qh = 0.0f, qh_pad = 0.0f;
    if (!a.dense) {
        const int g = i / 3, r = i % 3;
        const float* m = a.rotmat + 9 * g;
        const float v2 = (3 * g + 2 < kD) ? qs[3 * g + 2] : 0.0f;
        qh = __builtin_fmaf(m[3 * r + 2], v2, __builtin_fmaf(m[3 * r + 1], qs[3 * g + 1], m[3 * r] * qs[3 * g]));
        if (i == 0) {   // slot 128: last row of group 42 (pad input 0)
            const float* m42 = a.rotmat + 9 * 42;
            qh_pad = __builtin_fmaf(m42[8], 0.0f, __builtin_fmaf(m42[7], qs[127], m42[6] * qs[126]));
        }
    } else {
        float acc = 0.0f;
        for (int k = 0; k < kD; ++k) {
            const float p = (h2f(a.pi_hi[i * kD + k]) + h2f(a.pi_lo[i * kD + k]) * (1.0f / 2048.0f)) * 0.0625f;
            acc = __builtin_fmaf(p, qs[k], acc);
        }
        qh = acc;
    }
    float pj = 0.0f;
    if (a.qjl) {
        float acc = 0.0f;
        for (int k = 0; k < kD; ++k) acc = __builtin_fmaf(h2f(a.s_rows[i * kD + k]), qs[k], acc);
        pj = acc;
    }
    const float sq = pow2_scale(block_max(fmaxf(fabsf(qh), fabsf(qh_pad)), red));
    const float sp = pow2_scale(block_max(fabsf(pj), red));
    auto put = [&](int slot, float v) {
        uint32_t hi, lo;
        split_h11(v * sq, &hi, &lo);
        hv[0][slot] = static_cast<uint16_t>(f2h(h2f(hi) * 2048.0f));
        hv[1][slot] = static_cast<uint16_t>(hi);
        hv[2][slot] = static_cast<uint16_t>(lo);
    };
    put(i, qh);
    if (!a.dense && i == 0) put(128, qh_pad);
    if (a.qjl) {
        uint32_t hi, lo;
        split_h11(pj * sp, &hi, &lo);
        hv[3][i] = static_cast<uint16_t>(f2h(h2f(hi) * 2048.0f));
        hv[4][i] = static_cast<uint16_t>(lo);
    }
    __syncthreads();
    u32x4* row = a.rows + static_cast<int64_t>(h) * kRowChunks;
    const u32x4* src;
    for (int c = i; c < kRowChunks; c += 128) {
        int v, k;
        if (c < 3 * kQChunks) {
            v = c / kQChunks;
            k = c % kQChunks;
        } else {
            v = 3 + (c - 3 * kQChunks) / kPChunks;
            k = (c - 3 * kQChunks) % kPChunks;
        }
        src = reinterpret_cast<const u32x4*>(&hv[v][0]);
        row[c] = src[k];
    }
    if (i == 0) {
        a.scales[2 * h] = 1.0f / (2048.0f * sq);
        a.scales[2 * h + 1] = 1.0f / (2048.0f * sp);
    }
}

// -------------------------------------------------------------- main --
struct MainArgs {
    const uint32_t* codes;
    const uint16_t* norms;
    const uint32_t* signs;
    const uint16_t* rnorms;
    int64_t t, kv_stride;
    int kv_head0, group, rows_per_block;
    const u32x4* rows;
    const float* scales;
    const float* cent;
    float qjl_scale;
    float* scores;
    int64_t ld;
};

// Each 8-bit group of sign bits -> eight +-1 halves (bit 1 -> +1).
__device__ __forceinline__ u32x4 sigma_bits(uint32_t byte) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t b0 = (byte >> (2 * p)) & 1u, b1 = (byte >> (2 * p + 1)) & 1u;
        r[p] = 0xBC00BC00u ^ (b0 << 15) ^ (b1 << 31);
    }
    return r;
}

template <int B, bool QJL, int NC, int NMT>
__global__ __launch_bounds__(256) void score_kernel(MainArgs a) {
    constexpr int W = (NC * B + 31) / 32;
    constexpr int L = 1 << B;
    constexpr int KB1 = (NC + 15) / 16;   // K blocks of <q^, c>
    __shared__ u32x4 qrows[NMT * 32 * kRowStride];
    __shared__ float rscale[NMT * 32][2];
    __shared__ uint32_t ctab[L];          // C_hi | C_lo << 16 per code
    __shared__ uint32_t stage[4][64 * (W > 4 ? W : 4)];

    const int head = blockIdx.y;             // KV head within this call (query block folded below)
    const int qblocks = (a.group + a.rows_per_block - 1) / a.rows_per_block;
    const int kvh = head / qblocks, qb = head % qblocks;
    const int row0 = kvh * a.group + qb * a.rows_per_block;
    const int nrows = min(a.rows_per_block, a.group - qb * a.rows_per_block);

    // stage this block's query rows (rows >= nrows are zero)
    for (int q = threadIdx.x; q < NMT * 32 * kRowChunks; q += blockDim.x) {
        const int r = q / kRowChunks, c = q % kRowChunks;
        qrows[r * kRowStride + c] = r < nrows ? a.rows[static_cast<int64_t>(row0 + r) * kRowChunks + c]
                                              : u32x4{0u, 0u, 0u, 0u};
    }
    for (int r = threadIdx.x; r < NMT * 32; r += blockDim.x) {
        rscale[r][0] = r < nrows ? a.scales[2 * (row0 + r)] : 0.0f;
        rscale[r][1] = r < nrows ? a.scales[2 * (row0 + r) + 1] : 0.0f;
    }
    if (threadIdx.x < L) {
        const float cmax = fabsf(a.cent[L - 1]) > fabsf(a.cent[0]) ? fabsf(a.cent[L - 1]) : fabsf(a.cent[0]);
        const float sc = pow2_scale(cmax);
        uint32_t hi, lo;
        split_h11(a.cent[threadIdx.x] * sc, &hi, &lo);
        ctab[threadIdx.x] = hi | (lo << 16);
    }
    __syncthreads();
    float inv_sc;
    {
        const float cmax = fabsf(a.cent[L - 1]) > fabsf(a.cent[0]) ? fabsf(a.cent[L - 1]) : fabsf(a.cent[0]);
        inv_sc = 1.0f / pow2_scale(cmax);
    }

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t* st = stage[wave];
    const int64_t ntiles = (a.t + 63) / 64;
    const int64_t rbase = static_cast<int64_t>(a.kv_head0 + kvh) * a.kv_stride;

    for (int64_t tile = blockIdx.x * 4LL + wave; tile < ntiles; tile += gridDim.x * 4LL) {
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int64_t kbase = tile * 64;
        const int64_t nk = a.t;   // keys of this head
        // record of this lane's key
        uint32_t cw[W];
        words_load<W>(a.codes + rbase * W, kbase, nk, cw, st, l);
        uint32_t sw[4] = {0u, 0u, 0u, 0u};
        if constexpr (QJL) words_load<4>(a.signs + rbase * 4, kbase, nk, sw, st, l);
        const bool live = kbase + l < nk;
        const float nhat = live ? h2f(a.norms[rbase + kbase + l]) : 0.0f;
        const float ghat = (QJL && live) ? h2f(a.rnorms[rbase + kbase + l]) : 0.0f;

        f32x16 acc1[NMT][2], acc2[NMT][2];
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc1[m][nt] = f32x16{};
                acc2[m][nt] = f32x16{};
            }

#pragma unroll
        for (int kb = 0; kb < KB1; ++kb) {
            __builtin_amdgcn_sched_barrier(0);
            u32x4 h0, h1, lo0, lo1;   // own chunk 0 / 1 of C_hi and C_lo
            uint32_t hp[8], lp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t hh = 0u, ll = 0u;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int i = 16 * kb + 2 * e + s;
                    if (i < NC) {
                        const uint32_t v = ctab[get_code<B, W>(cw, i)];
                        hh |= (v & 0xFFFFu) << (16 * s);
                        ll |= (v >> 16) << (16 * s);
                    }
                }
                hp[e] = hh;
                lp[e] = ll;
            }
            u32x4 ch0{hp[0], hp[1], hp[2], hp[3]}, ch1{hp[4], hp[5], hp[6], hp[7]};
            u32x4 cl0{lp[0], lp[1], lp[2], lp[3]}, cl1{lp[4], lp[5], lp[6], lp[7]};
            to_operands(ch0, ch1, &h0, &h1);
            to_operands(cl0, cl1, &lo0, &lo1);
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                const int r = 32 * m + (l & 31);
                const int kc = 2 * kb + (l >> 5);
                const u32x4 q1 = qrows[r * kRowStride + kOffQ1 + kc];
                const u32x4 q2 = qrows[r * kRowStride + kOffQ2 + kc];
                const u32x4 q3 = qrows[r * kRowStride + kOffQ3 + kc];
                acc1[m][0] = mfma(q1, h0, acc1[m][0]);
                acc1[m][0] = mfma(q2, lo0, acc1[m][0]);
                acc1[m][0] = mfma(q3, h0, acc1[m][0]);
                acc1[m][1] = mfma(q1, h1, acc1[m][1]);
                acc1[m][1] = mfma(q2, lo1, acc1[m][1]);
                acc1[m][1] = mfma(q3, h1, acc1[m][1]);
            }
        }
        if constexpr (QJL) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t word = sw[kb >> 1] >> (16 * (kb & 1));
                u32x4 s0, s1;
                to_operands(sigma_bits(word & 0xFFu), sigma_bits((word >> 8) & 0xFFu), &s0, &s1);
#pragma unroll
                for (int m = 0; m < NMT; ++m) {
                    const int r = 32 * m + (l & 31);
                    const int kc = 2 * kb + (l >> 5);
                    const u32x4 p1 = qrows[r * kRowStride + kOffP1 + kc];
                    const u32x4 p2 = qrows[r * kRowStride + kOffP2 + kc];
                    acc2[m][0] = mfma(p1, s0, acc2[m][0]);
                    acc2[m][0] = mfma(p2, s0, acc2[m][0]);
                    acc2[m][1] = mfma(p1, s1, acc2[m][1]);
                    acc2[m][1] = mfma(p2, s1, acc2[m][1]);
                }
            }
        }
        // per-key factors for the two 32-key halves: lane l of half nt needs
        // key nt * 32 + l % 32
        float kn[2], kg[2];
        {
            const auto sn = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, nhat),
                                                             __builtin_bit_cast(uint32_t, nhat), false, false);
            const float gk = ghat * a.qjl_scale;
            const auto sg = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, gk),
                                                             __builtin_bit_cast(uint32_t, gk), false, false);
            const uint32_t n0 = sn[0], n1 = sn[1], g0 = sg[0], g1 = sg[1];
            kn[0] = __builtin_bit_cast(float, n0);
            kn[1] = __builtin_bit_cast(float, n1);
            kg[0] = __builtin_bit_cast(float, g0);
            kg[1] = __builtin_bit_cast(float, g1);
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t key = kbase + 32 * nt + (l & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * m + 8 * (r / 4) + 4 * (l >> 5) + (r % 4);
                    float v = acc1[m][nt][r] * (rscale[row][0] * inv_sc);
                    if constexpr (QJL) v = __builtin_fmaf(kg[nt], acc2[m][nt][r] * rscale[row][1], v);
                    v *= kn[nt];
                    if (row < nrows && key < nk) a.scores[static_cast<int64_t>(row0 + row) * a.ld + key] = v;
                }
            }
    }
}

template <int B, bool QJL, int NC, int NMT>
static void launch_main(const MainArgs& a, int kv_heads, int qblocks, hipStream_t s) {
    const int64_t ntiles = (a.t + 63) / 64;
    const int64_t want = (ntiles + 3) / 4;
    const int64_t per_head_cap = (4096 + kv_heads * qblocks - 1) / (kv_heads * qblocks);
    const int gx = static_cast<int>(want < per_head_cap ? want : (per_head_cap > 0 ? per_head_cap : 1));
    hipLaunchKernelGGL((score_kernel<B, QJL, NC, NMT>), dim3(gx, kv_heads * qblocks), dim3(256), 0, s, a);
}

template <int B, bool QJL>
static void launch_main_b(bool dense, int nmt, const MainArgs& a, int kv_heads, int qblocks, hipStream_t s) {
    if (dense) {
        if (nmt == 1) launch_main<B, QJL, 128, 1>(a, kv_heads, qblocks, s);
        else launch_main<B, QJL, 128, 2>(a, kv_heads, qblocks, s);
    } else {
        if (nmt == 1) launch_main<B, QJL, 129, 1>(a, kv_heads, qblocks, s);
        else launch_main<B, QJL, 129, 2>(a, kv_heads, qblocks, s);
    }
}

hipError_t score(const ScoreTables& t, const float* q, int hq, int group, const uint32_t* codes,
                 const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms, int64_t tkeys,
                 int64_t kv_stride, int kv_head0, void* ws, float* scores, int64_t ld_scores, hipStream_t s) {
    ProArgs pa;
    pa.q = q;
    pa.hq = hq;
    pa.dense = t.dense;
    pa.qjl = t.qjl;
    pa.rotmat = t.rot.rotmat;
    pa.pi_hi = t.den.pi_hi;
    pa.pi_lo = t.den.pi_lo;
    pa.s_rows = t.dense ? t.den.s_rows : t.rot.s_rows;
    pa.rows = static_cast<u32x4*>(ws);
    pa.scales = reinterpret_cast<float*>(static_cast<char*>(ws) + static_cast<size_t>(kScoreChunkRows) * kRowChunks * 16);
    hipLaunchKernelGGL(score_prologue, dim3(hq), dim3(128), 0, s, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    MainArgs a;
    a.codes = codes;
    a.norms = norms;
    a.signs = signs;
    a.rnorms = rnorms;
    a.t = tkeys;
    a.kv_stride = kv_stride;
    a.kv_head0 = kv_head0;
    a.group = group;
    a.rows_per_block = group < 64 ? group : 64;
    a.rows = pa.rows;
    a.scales = pa.scales;
    a.cent = t.dense ? t.den.cent : t.rot.cent;
    a.qjl_scale = t.qjl_scale;
    a.scores = scores;
    a.ld = ld_scores;
    const int kv_heads = hq / group;
    const int qblocks = (group + 63) / 64;
    const int nmt = a.rows_per_block > 32 ? 2 : 1;
    switch (t.mse_bits * 2 + (t.qjl ? 1 : 0)) {
        case 2: launch_main_b<1, false>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 3: launch_main_b<1, true>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 4: launch_main_b<2, false>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 5: launch_main_b<2, true>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 6: launch_main_b<3, false>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 7: launch_main_b<3, true>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 8: launch_main_b<4, false>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        case 9: launch_main_b<4, true>(t.dense, nmt, a, kv_heads, qblocks, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rqk
