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
// with a power-of-two row scale.  Main kernel: the staged query rows of one
// KV head are the A operand of 32x32x16 MFMAs; the B operand is decoded from
// the records straight into MFMA layout: lane (n, h) of a wave serves keys n
// and 32 + n of the 64-key tile and K slots 8h..8h+7 of each 16-wide block,
// turning two codes into packed centroid halves with one LDS lookup and sign
// bits into +-1 halves with shifts.  The rotor pad coordinate (slot 128) is
// added in fp32 in the epilogue.
#include "rq_common.cuh"
#include "rq_kernels.h"

namespace rqk {

// ---------------------------------------------------------- staged rows --
// Per query row, in 16-byte chunks:
//   Q1 [16 chunks] = 2^11 * hi(s_q q^)   Q2 = hi(s_q q^)   Q3 = lo(s_q q^)
//   P1 [16 chunks] = 2^11 * hi(s_p S q)  P2 = lo(s_p S q)
// with hi(v) = half(v), lo(v) = half((v - hi) * 2^11) (split_h11) over
// slots 0..127.  Against centroid halves C_hi = half(s_c c),
// C_lo = half((s_c c - C_hi) 2^11):
//   Q1 C_hi + Q2 C_lo + Q3 C_hi = 2^11 s_q s_c <q^, c>  (to ~2^-22 relative),
//   P1 sigma + P2 sigma = 2^11 s_p <S q, sigma>.
// Row scalars (after the rows): 1 / (2^11 s_q), 1 / (2^11 s_p), and the
// rotor pad slot q^_128 in fp32.
constexpr int kQChunks = 16;
constexpr int kRowChunks = 5 * kQChunks;     // 80
constexpr int kRowStride = kRowChunks + 1;   // LDS row pitch (bank spread)
constexpr int kOffQ1 = 0, kOffQ2 = kQChunks, kOffQ3 = 2 * kQChunks, kOffP1 = 3 * kQChunks, kOffP2 = 4 * kQChunks;
constexpr int kRowScalars = 3;
static_assert(kRowChunks * 16 + kRowScalars * 4 <= kScoreQueryBytes, "workspace row too small");

struct ProArgs {
    const float* q;
    int hq;
    bool dense, qjl;
    const float* rotmat;      // rotor: [43][9]
    const uint16_t* pit_hi;   // dense: Pi^T = (hi + lo 2^-11) / 16, row-major
    const uint16_t* pit_lo;
    const uint16_t* s_cols;   // QJL: S^T, row-major halves
    u32x4* rows;              // [hq][kRowChunks]
    float* scalars;           // [hq][kRowScalars]
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

// One block of 128 threads per query row; thread i owns slot i.  The
// transposed tables are read so that a warp's loads are contiguous.
__global__ __launch_bounds__(128) void score_prologue(ProArgs a) {
    __shared__ float qs[kD];
    __shared__ float red[2];
    __shared__ __align__(16) uint16_t hv[5][kD];
    const int h = blockIdx.x, i = threadIdx.x;
    qs[i] = a.q[static_cast<int64_t>(h) * kD + i];
    __syncthreads();
    float qh = 0.0f, qpad = 0.0f;
    if (!a.dense) {
        const int g = i / 3, r = i % 3;
        const float* m = a.rotmat + 9 * g;
        const float v2 = (3 * g + 2 < kD) ? qs[3 * g + 2] : 0.0f;
        qh = __builtin_fmaf(m[3 * r + 2], v2, __builtin_fmaf(m[3 * r + 1], qs[3 * g + 1], m[3 * r] * qs[3 * g]));
        // slot 128: last row of group 42 (pad input 0)
        const float* m42 = a.rotmat + 9 * 42;
        qpad = __builtin_fmaf(m42[8], 0.0f, __builtin_fmaf(m42[7], qs[127], m42[6] * qs[126]));
    } else {
        float acc = 0.0f;
#pragma unroll 16
        for (int k = 0; k < kD; ++k) {
            const float p =
                (h2f(a.pit_hi[k * kD + i]) + h2f(a.pit_lo[k * kD + i]) * (1.0f / 2048.0f)) * 0.0625f;
            acc = __builtin_fmaf(p, qs[k], acc);
        }
        qh = acc;
    }
    float pj = 0.0f;
    if (a.qjl) {
        float acc = 0.0f;
#pragma unroll 16
        for (int k = 0; k < kD; ++k) acc = __builtin_fmaf(h2f(a.s_cols[k * kD + i]), qs[k], acc);
        pj = acc;
    }
    const float sq = pow2_scale(block_max(fabsf(qh), red));
    const float sp = pow2_scale(block_max(fabsf(pj), red));
    {
        uint32_t hi, lo;
        split_h11(qh * sq, &hi, &lo);
        hv[0][i] = static_cast<uint16_t>(f2h(h2f(hi) * 2048.0f));
        hv[1][i] = static_cast<uint16_t>(hi);
        hv[2][i] = static_cast<uint16_t>(lo);
        split_h11(pj * sp, &hi, &lo);
        hv[3][i] = static_cast<uint16_t>(f2h(h2f(hi) * 2048.0f));
        hv[4][i] = static_cast<uint16_t>(lo);
    }
    __syncthreads();
    u32x4* row = a.rows + static_cast<int64_t>(h) * kRowChunks;
    for (int c = i; c < kRowChunks; c += 128) row[c] = reinterpret_cast<const u32x4*>(&hv[c / kQChunks][0])[c % kQChunks];
    if (i == 0) {
        float* s = a.scalars + static_cast<int64_t>(h) * kRowScalars;
        s[0] = 1.0f / (2048.0f * sq);
        s[1] = 1.0f / (2048.0f * sp);
        s[2] = qpad;
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
    const float* scalars;
    const float* cent;
    float qjl_scale;
    float* scores;
    int64_t ld;
};

// 8 sign bits (bit e = [z_e >= 0]) -> four dwords of +-1 half pairs.
__device__ __forceinline__ u32x4 sigma8(uint32_t byte) {
    const uint32_t nb = ~byte;
    const uint32_t u = (nb & 0x55u) | ((nb & 0xAAu) << 15);
    u32x4 d;
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = ((u << (15 - 2 * q)) & 0x80008000u) | 0x3C003C00u;
    return d;
}

// One 16-bit record entry of key `idx` (relative to the tile base), 0 past n.
__device__ __forceinline__ uint32_t half_at(const uint16_t* __restrict__ src, int64_t base, int64_t n, int idx) {
    const rsrc_t rs = make_rsrc(src + base, tile_range(n - base, 2));
    return __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<uint32_t>(2 * idx), 0, kNonTemporal);
}

template <int B, bool QJL, bool PAD, int NMT>
__global__ __launch_bounds__(256) void score_kernel(MainArgs a) {
    constexpr int NC = PAD ? kRotCoords : kD;
    constexpr int W = (NC * B + 31) / 32;
    constexpr int L = 1 << B;
    constexpr int SW = W > 4 ? W : 4;
    constexpr int ROWS = NMT * 32;
    struct Lds {
        uint32_t pairs[L * L][2];     // codes (a, b) -> {C_hi[a] | C_hi[b] << 16, C_lo[a] | C_lo[b] << 16}
        float rsc[ROWS][4];           // {1 / (2^11 s_q s_c), 1 / (2^11 s_p), q^_128, 0}
        float cent[L];
        uint32_t stage[4][64 * SW];
        u32x4 qrows[ROWS * kRowStride];
    };
    __shared__ Lds lds;

    const int head = blockIdx.y;   // KV head within this call (query block folded below)
    const int qblocks = (a.group + a.rows_per_block - 1) / a.rows_per_block;
    const int kvh = head / qblocks, qb = head % qblocks;
    const int row0 = kvh * a.group + qb * a.rows_per_block;
    const int nrows = min(a.rows_per_block, a.group - qb * a.rows_per_block);

    float inv_sc;
    {
        const float cmax = fabsf(a.cent[L - 1]) > fabsf(a.cent[0]) ? fabsf(a.cent[L - 1]) : fabsf(a.cent[0]);
        const float sc = pow2_scale(cmax);
        inv_sc = 1.0f / sc;
        for (int p = threadIdx.x; p < L * L; p += kBlock) {
            uint32_t h0, l0, h1, l1;
            split_h11(a.cent[p & (L - 1)] * sc, &h0, &l0);
            split_h11(a.cent[p >> B] * sc, &h1, &l1);
            lds.pairs[p][0] = h0 | (h1 << 16);
            lds.pairs[p][1] = l0 | (l1 << 16);
        }
        if (threadIdx.x < L) lds.cent[threadIdx.x] = a.cent[threadIdx.x];
    }
    // this block's query rows (rows >= nrows are zero), all loads in flight at once
    {
        constexpr int PER = ROWS * kRowChunks / kBlock;
        static_assert(ROWS * kRowChunks % kBlock == 0, "staging split");
        u32x4 v[PER];
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int q = it * kBlock + threadIdx.x, r = q / kRowChunks, c = q % kRowChunks;
            v[it] = r < nrows ? a.rows[static_cast<int64_t>(row0 + r) * kRowChunks + c] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int q = it * kBlock + threadIdx.x, r = q / kRowChunks, c = q % kRowChunks;
            lds.qrows[r * kRowStride + c] = v[it];
        }
    }
    for (int r = threadIdx.x; r < ROWS; r += kBlock) {
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
        if (r < nrows) {
            const float* s = a.scalars + static_cast<int64_t>(row0 + r) * kRowScalars;
            s0 = s[0] * inv_sc;
            s1 = s[1];
            s2 = s[2];
        }
        lds.rsc[r][0] = s0;
        lds.rsc[r][1] = s1;
        lds.rsc[r][2] = s2;
        lds.rsc[r][3] = 0.0f;
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t* st = lds.stage[wave];
    const int64_t nk = a.t;   // keys of this head
    const int64_t ntiles = (nk + 63) / 64;
    const int64_t rbase = static_cast<int64_t>(a.kv_head0 + kvh) * a.kv_stride;
    const char* pairc = reinterpret_cast<const char*>(lds.pairs);

    for (int64_t tile = blockIdx.x * 4LL + wave; tile < ntiles; tile += gridDim.x * 4LL) {
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int n = l & 31, hh = l >> 5;
        const int64_t kbase = tile * 64;

        // code words of keys n and 32 + n, shifted so this lane's K slots
        // start at bit 0 (slot 8 hh of each block is bit 8 B hh further)
        uint32_t cw[2][W];
        {
            const rsrc_t rs = make_rsrc(a.codes + (rbase + kbase) * W, tile_range(nk - kbase, 4 * W));
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < W; ++it)
                st[it * 64 + l] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(4 * l), 256 * it,
                                                                        kNonTemporal);
            wave_lds_sync();
#pragma unroll
            for (int k = 0; k < W; ++k) {
                cw[0][k] = st[n * W + k];
                cw[1][k] = st[(32 + n) * W + k];
            }
        }
        float cpad[2] = {0.0f, 0.0f};
        if constexpr (PAD) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) cpad[nt] = lds.cent[cw[nt][4 * B] & (L - 1)];
        }
        uint32_t cs[2][W];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const uint32_t nxt = k + 1 < W ? cw[nt][k + 1] : 0u;
                if constexpr (B == 4) cs[nt][k] = hh ? nxt : cw[nt][k];
                else cs[nt][k] = __builtin_amdgcn_alignbit(nxt, cw[nt][k], 8 * B * hh);
            }
        uint32_t sg[2][4];
        if constexpr (QJL) {
            const rsrc_t rs = make_rsrc(a.signs + (rbase + kbase) * 4, tile_range(nk - kbase, 16));
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < 4; ++it)
                st[it * 64 + l] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(4 * l), 256 * it,
                                                                        kNonTemporal);
            wave_lds_sync();
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sg[0][k] = st[n * 4 + k] >> (8 * hh);
                sg[1][k] = st[(32 + n) * 4 + k] >> (8 * hh);
            }
        }
        wave_lds_sync();
        float kn[2], kg[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            kn[nt] = h2f(half_at(a.norms + rbase, kbase, nk, 32 * nt + n));
            kg[nt] = QJL ? h2f(half_at(a.rnorms + rbase, kbase, nk, 32 * nt + n)) * a.qjl_scale : 0.0f;
        }

        f32x16 acc1[NMT][2], acc2[NMT][2];
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc1[m][nt] = f32x16{};
                acc2[m][nt] = f32x16{};
            }

#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            __builtin_amdgcn_sched_barrier(0);
            u32x4 ch[2], cl[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int bit = 16 * B * kb + 2 * B * q, wi = bit >> 5, off = bit & 31;
                    uint32_t f = cs[nt][wi] >> off;
                    if (off + 2 * B > 32) f = __builtin_amdgcn_alignbit(cs[nt][wi + 1], cs[nt][wi], off);
                    const uint32_t addr = (f & (L * L - 1)) * 8u;
                    const uint32_t hi = *reinterpret_cast<const uint32_t*>(pairc + addr);
                    const uint32_t lo = *reinterpret_cast<const uint32_t*>(pairc + addr + 4);
                    ch[nt][q] = hi;
                    cl[nt][q] = lo;
                }
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                const int r = (32 * m + n) * kRowStride + 2 * kb + hh;
                const u32x4 q1 = lds.qrows[r + kOffQ1];
                const u32x4 q2 = lds.qrows[r + kOffQ2];
                const u32x4 q3 = lds.qrows[r + kOffQ3];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc1[m][nt] = mfma(q1, ch[nt], acc1[m][nt]);
                    acc1[m][nt] = mfma(q2, cl[nt], acc1[m][nt]);
                    acc1[m][nt] = mfma(q3, ch[nt], acc1[m][nt]);
                }
            }
        }
        if constexpr (QJL) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                __builtin_amdgcn_sched_barrier(0);
                u32x4 s[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) s[nt] = sigma8((sg[nt][kb >> 1] >> (16 * (kb & 1))) & 0xFFu);
#pragma unroll
                for (int m = 0; m < NMT; ++m) {
                    const int r = (32 * m + n) * kRowStride + 2 * kb + hh;
                    const u32x4 p1 = lds.qrows[r + kOffP1];
                    const u32x4 p2 = lds.qrows[r + kOffP2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        acc2[m][nt] = mfma(p1, s[nt], acc2[m][nt]);
                        acc2[m][nt] = mfma(p2, s[nt], acc2[m][nt]);
                    }
                }
            }
        }

        // epilogue: rows past nrows fall outside the descriptor's range, keys
        // past the end get an offset beyond it
        const rsrc_t rs = make_rsrc(a.scores + static_cast<int64_t>(row0) * a.ld + kbase,
                                    static_cast<uint32_t>(((nrows - 1) * a.ld + (nk - kbase)) * 4));
        uint32_t voff[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int key = 32 * nt + n;
            voff[nt] = kbase + key < nk ? static_cast<uint32_t>((4 * hh * a.ld + key) * 4) : 0x80000000u;
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rowc = 32 * m + 8 * (r / 4) + (r % 4);   // row without the lane-half term 4 hh
                const float* rsv = lds.rsc[rowc + 4 * hh];
                const float s0 = rsv[0], s1 = rsv[1], s2 = rsv[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const float e1 = acc1[m][nt][r];
                    float v = e1 * s0;
                    if constexpr (PAD) v = __builtin_fmaf(s2, cpad[nt], v);
                    if constexpr (QJL) {
                        const float e2 = acc2[m][nt][r];
                        v = __builtin_fmaf(kg[nt], e2 * s1, v);
                    }
                    v *= kn[nt];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff[nt],
                                                          static_cast<int>(rowc * a.ld * 4), kNonTemporal);
                }
            }
    }
}

template <int B, bool QJL, bool PAD, int NMT>
static void launch_main(const MainArgs& a, int kv_heads, int qblocks, hipStream_t s) {
    const int64_t ntiles = (a.t + 63) / 64;
    const int64_t want = (ntiles + 3) / 4;
    const int64_t per_head_cap = (4096 + kv_heads * qblocks - 1) / (kv_heads * qblocks);
    const int gx = static_cast<int>(want < per_head_cap ? want : (per_head_cap > 0 ? per_head_cap : 1));
    hipLaunchKernelGGL((score_kernel<B, QJL, PAD, NMT>), dim3(gx, kv_heads * qblocks), dim3(kBlock), 0, s, a);
}

template <int B, bool QJL>
static void launch_main_b(bool dense, int nmt, const MainArgs& a, int kv_heads, int qblocks, hipStream_t s) {
    if (dense) {
        if (nmt == 1) launch_main<B, QJL, false, 1>(a, kv_heads, qblocks, s);
        else launch_main<B, QJL, false, 2>(a, kv_heads, qblocks, s);
    } else {
        if (nmt == 1) launch_main<B, QJL, true, 1>(a, kv_heads, qblocks, s);
        else launch_main<B, QJL, true, 2>(a, kv_heads, qblocks, s);
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
    pa.pit_hi = t.den.pit_hi;
    pa.pit_lo = t.den.pit_lo;
    pa.s_cols = t.dense ? t.den.s_cols : t.rot.s_cols;
    pa.rows = static_cast<u32x4*>(ws);
    pa.scalars =
        reinterpret_cast<float*>(static_cast<char*>(ws) + static_cast<size_t>(kScoreChunkRows) * kRowChunks * 16);
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
    a.scalars = pa.scalars;
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
