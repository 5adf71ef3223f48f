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
// Each block first builds, in LDS, the query side for its (KV head, <= 64
// query rows): q^ and S q as exact fp16 half pairs with power-of-two row
// scales, all on 32x32x16 MFMAs from an exact hi/lo split of the query
// (q^ = Pi q on the dense path; on the rotor path q^ = Phi q with Phi the
// 128 x 128 block-diagonal matrix of the rotor sandwiches, the pad slot
// q^_128 from the last rotor in fp32).  Those rows are then
// the A operand of the scoring MFMAs; the B operand is decoded from the
// records straight into MFMA layout: lane (n, h) of a wave serves keys n and
// 32 + n of the 64-key tile and K slots 8h..8h+7 of each 16-wide block
// (groups of at most 16 rows: 16x16x32 MFMAs, lane (c, g) serving keys
// 16 j + c and K slots 8g..8g+7 of each 32-wide step), turning four 1- or
// 2-bit codes (or two wider ones) into packed centroid halves with LDS
// table lookups and eight sign bits into +-1 halves with a table or shifts.
// The rotor pad coordinate (slot 128) is added in fp32 in the epilogue.
//
// QJL-only keys with separated outlier channels (OUTL; README "CUDA
// Kernels": the 1-bit quantiser separates outliers): the block's query rows
// are split into their values on the KV head's outlier channels (kept in
// fp32) and the rest q_in (those channels cleared) before S q_in is built;
// per key the score is n^ gamma^ sqrt(pi/2)/m <S q_in, sigma> +
// sum_i q_{c_i} o^_i over the key's stored outlier halves o^.
#include "rq_common_dev.h"
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
// Row scalars: 1 / (2^11 s_q s_c), 1 / (2^11 s_p), and the rotor pad slot
// q^_128 in fp32.
constexpr int kQChunks = 16;
constexpr int kRowChunks = 5 * kQChunks;     // 80
constexpr int kRowStride = kRowChunks + 1;   // LDS row pitch (bank spread)
constexpr int kOffQ1 = 0, kOffQ2 = kQChunks, kOffQ3 = 2 * kQChunks, kOffP1 = 3 * kQChunks, kOffP2 = 4 * kQChunks;

// power-of-two scale putting the largest magnitude in [1, 2)
__device__ __forceinline__ float pow2_scale(float maxabs) {
    if (!(maxabs > 0.0f)) return 1.0f;
    int e;
    frexpf(maxabs, &e);
    return ldexpf(1.0f, 1 - e);
}

// -------------------------------------------------------------- main --
struct MainArgs {
    const float* q;            // [rows of this call][128] fp32 queries
    const float* rotmat;       // rotor: [43][9]
    const uint16_t* x_hi;      // 16 Pi (dense) or 16 Phi (rotor) = hi + 2^-11 lo, row-major halves
    const uint16_t* x_lo;
    const uint16_t* s_rows;    // QJL: S, row-major halves
    const uint32_t* codes;
    const uint16_t* norms;
    const uint32_t* signs;
    const uint16_t* rnorms;
    int64_t t, kv_stride;
    int kv_head0, group, rows_per_block;
    const float* cent;
    float qjl_scale;
    float* scores;
    int64_t ld;
    PageTable pt;
    const uint8_t* ochans = nullptr;   // OUTL: outlier channels, [KV heads][ok]
    const uint16_t* outl = nullptr;    // OUTL: outlier halves of the keys, [record rows][ok]
    int ok = 0;                        // outlier channels per head (<= 16)
    RowMax rm;                         // groups of at most 16 rows: per-workgroup row maxima
};

// Record row of the first key of the 64-key tile at key kbase of KV head
// `head` (global index); pages never split a tile (page size >= 64 keys).
__device__ __forceinline__ int64_t tile_row(const PageTable& pt, int64_t rbase, int head, int64_t kbase) {
    if (pt.pages == nullptr) return rbase + kbase;
    const int64_t pg = pt.pages[head * pt.stride + (kbase >> pt.shift)];
    return (pg << pt.shift) + (kbase & ((int64_t(1) << pt.shift) - 1));
}

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

// One tile's record in registers: lane l holds dword it * 64 + l of the
// tile's code and sign runs, and the fp16 norm / residual norm of keys
// l % 32 + 32 j (KPL = 2) or l % 16 + 16 j (KPL = 4).  Fetched one tile ahead.
template <int W, int KPL, bool OUTL = false>
struct RecRegs {
    uint32_t c[W > 0 ? W : 1];
    uint32_t s[4];
    uint32_t kn[KPL], kg[KPL];
    uint32_t o[OUTL ? 16 : 1];  // half it * 64 + l of the tile's outlier halves
};
template <int W, bool QJL, int KPL, bool OUTL = false>
__device__ __forceinline__ void rec_fetch(const MainArgs& a, int64_t rbase, int head, int64_t kbase,
                                          RecRegs<W, KPL, OUTL>& r, int l) {
    const int64_t left = a.t - kbase;
    const int64_t row = tile_row(a.pt, rbase, head, kbase);
    const rsrc_t rc = make_rsrc(a.codes + row * W, tile_range(left, 4 * W));
#pragma unroll
    for (int it = 0; it < W; ++it)
        r.c[it] = __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    if constexpr (QJL) {
        const rsrc_t rsg = make_rsrc(a.signs + row * 4, tile_range(left, 16));
#pragma unroll
        for (int it = 0; it < 4; ++it)
            r.s[it] = __builtin_amdgcn_raw_buffer_load_b32(rsg, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    }
    constexpr int KS = 64 / KPL;   // key stride between a lane's keys
    const int n = l & (KS - 1);
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        r.kn[j] = half_at(a.norms + row, 0, left, KS * j + n);
        r.kg[j] = QJL ? half_at(a.rnorms + row, 0, left, KS * j + n) : 0u;
    }
    if constexpr (OUTL) {
        // the tile's keys hold 64 ok halves in one run (16-bit loads: the run
        // starts on any half boundary)
        const rsrc_t ro = make_rsrc(a.outl + row * a.ok, tile_range(left, 2 * a.ok));
#pragma unroll
        for (int it = 0; it < 16; ++it)
            r.o[it] = it < a.ok ? __builtin_amdgcn_raw_buffer_load_b16(ro, static_cast<uint32_t>(2 * l), 128 * it,
                                                                       kNonTemporal)
                                : 0u;
    }
}

// OUTL: the tile's outlier halves into the wave's LDS stage (key-major,
// ok halves per key).
template <int W, int KPL, bool OUTL>
__device__ __forceinline__ void stage_outliers(const MainArgs& a, const RecRegs<W, KPL, OUTL>& r,
                                               uint32_t* __restrict__ ost, int l) {
    if constexpr (OUTL) {
        uint16_t* o16 = reinterpret_cast<uint16_t*>(ost);
#pragma unroll
        for (int it = 0; it < 16; ++it)
            if (it < a.ok) o16[it * 64 + l] = static_cast<uint16_t>(r.o[it]);
    }
}

// ------------------------------------------------------- query side --
// Stores 4 consecutive fp16 values (packed in two dwords) at slots
// j..j+3 (j % 4 == 0) of array `off` of a staged row.
__device__ __forceinline__ void put4(u32x4* qrows, int row, int off, int j, uint32_t d0, uint32_t d1) {
    char* p = reinterpret_cast<char*>(qrows) + (static_cast<size_t>(row) * kRowStride + off + (j >> 3)) * 16 +
              (j & 7) * 2;
    *reinterpret_cast<uint2*>(p) = make_uint2(d0, d1);
}

// The block's query products for one 32-row M tile (wave w) and all its
// query rows: X q' with X = 16 Pi (dense) or 16 Phi (rotor: the block-diagonal
// matrix of the 43 rotor sandwiches, pad column dropped), split as
// X = hi + 2^-11 lo; and, with QJL, S q'.  q' = q * s0 (s0 a power of two)
// enters as 2^11 hi, lo11 = (q' - hi) 2^11 and hi, computed once per K block
// for both products.  Outputs (unscaled) hold rows 32 w + 8 (r / 4) +
// 4 h + r % 4 of query row 32 nt + l % 32.
// A-operand fragments of wave w's M tile of X (hi, lo) and S, all 8 K blocks.
template <bool QJL, bool X>
struct QueryFrags {
    u32x4 xh[X ? 8 : 1], xl[X ? 8 : 1], sa[QJL ? 8 : 1];
};
template <bool QJL, bool X>
__device__ __forceinline__ void query_frags(const MainArgs& a, int w, int l, QueryFrags<QJL, X>& f) {
    const int n = l & 31, hh = l >> 5;
    const u32x4* gxh = reinterpret_cast<const u32x4*>(a.x_hi);
    const u32x4* gxl = reinterpret_cast<const u32x4*>(a.x_lo);
    const u32x4* gs = reinterpret_cast<const u32x4*>(a.s_rows);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int i = (32 * w + n) * 16 + 2 * kb + hh;
        if constexpr (X) {
            f.xh[kb] = gxh[i];
            f.xl[kb] = gxl[i];
        }
        if constexpr (QJL) f.sa[kb] = gs[i];
    }
}

// Exact split of the block's query rows q' = q * s0 into the three B
// operands 2^11 hi, lo11 = (q' - hi) 2^11 and hi, for K blocks 2w, 2w + 1
// (wave w) of every N tile, written to LDS for all four waves.
template <int NMT, class Lds>
__device__ __forceinline__ void query_split(Lds& lds, u32x4* bop, int w, int l) {
    const int n = l & 31, hh = l >> 5;
#pragma unroll
    for (int nt = 0; nt < NMT; ++nt) {
        const int row = 32 * nt + n;
        const float s0 = lds.s0[row];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int kb = 2 * w + k2;
            const float* qv = &lds.qf[row][16 * kb + 8 * hh];
            u32x4 h11, l11, h;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float x0 = qv[2 * p] * s0, x1 = qv[2 * p + 1] * s0;
                const uint32_t hp = cvt_pk(x0, x1);
                const float f0 = h2f(hp & 0xFFFFu), f1 = h2f(hp >> 16);
                h[p] = hp;
                h11[p] = pk_scale2048(hp);
                l11[p] = cvt_pk((x0 - f0) * 2048.0f, (x1 - f1) * 2048.0f);
            }
            u32x4* b = bop + ((nt * 8 + kb) * 3) * 64 + l;
            b[0] = h11;
            b[64] = l11;
            b[128] = h;
        }
    }
}

template <bool QJL, bool X, int NMT>
__device__ __forceinline__ void query_products(const QueryFrags<QJL, X>& fr, const u32x4* bop,
                                               const float (&s0r)[NMT], int l, float (&ox)[NMT][16],
                                               float (&os)[NMT][16]) {
#pragma unroll
    for (int nt = 0; nt < NMT; ++nt) {
        f32x16 ax = {}, as = {};
        // the split operands of K block kb + 1 are read before K block kb's
        // MFMAs issue (the scheduling barrier keeps each read from moving
        // down next to its MFMA)
        u32x4 op[2][3];
        auto read = [&](int kb, u32x4 (&d)[3]) {
            const u32x4* b = bop + ((nt * 8 + kb) * 3) * 64 + l;
            d[0] = b[0];
            d[1] = b[64];
            d[2] = b[128];
        };
        read(0, op[0]);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const int cur = kb & 1;
            if (kb < 7) read(kb + 1, op[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 h11 = op[cur][0], l11 = op[cur][1], h = op[cur][2];
            if constexpr (X) {
                ax = mfma(fr.xh[kb], h11, ax);
                ax = mfma(fr.xh[kb], l11, ax);
                ax = mfma(fr.xl[kb], h, ax);
            }
            if constexpr (QJL) {
                as = mfma(fr.sa[kb], h11, as);
                as = mfma(fr.sa[kb], l11, as);
            }
        }
        const float ux = 1.0f / (2048.0f * 16.0f) / s0r[nt], us = 1.0f / 2048.0f / s0r[nt];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = ax[r];
            ox[nt][r] = e * ux;
            const float f = as[r];
            os[nt][r] = f * us;
        }
    }
}

// Row maxima of |out| over the 128 product rows: lane halves, then waves.
template <int NMT, class Lds>
__device__ __forceinline__ void product_row_max(const float (&out)[NMT][16], Lds& lds, int k, int w, int l) {
#pragma unroll
    for (int nt = 0; nt < NMT; ++nt) {
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(out[nt][r]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, m),
                                                         __builtin_bit_cast(uint32_t, m), false, false);
        const uint32_t a0 = sw[0], a1 = sw[1];
        m = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
        if ((l >> 5) == 0) lds.part[k][w][32 * nt + (l & 31)] = m;
    }
}

// Writes the split halves of out * s (s the row scale) into the staged rows:
// arrays offA = 2^11 hi, offB = lo11, and (if offC >= 0) offC = hi; stores
// 1 / (2^11 s) * mul in rsc[row][rsc_slot].
template <int NMT, class Lds>
__device__ __forceinline__ void product_store(const float (&out)[NMT][16], Lds& lds, int k, int w, int l, int offA,
                                              int offB, int offC, int rsc_slot, float mul) {
    const int n = l & 31, hh = l >> 5;
#pragma unroll
    for (int nt = 0; nt < NMT; ++nt) {
        const int row = 32 * nt + n;
        const float mx = fmaxf(fmaxf(lds.part[k][0][row], lds.part[k][1][row]),
                               fmaxf(lds.part[k][2][row], lds.part[k][3][row]));
        const float sc = pow2_scale(mx);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t A[2], Bv[2], C[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float x0 = out[nt][4 * b + 2 * q] * sc, x1 = out[nt][4 * b + 2 * q + 1] * sc;
                const uint32_t hp = cvt_pk(x0, x1);
                C[q] = hp;
                A[q] = pk_scale2048(hp);
                Bv[q] = cvt_pk((x0 - h2f(hp & 0xFFFFu)) * 2048.0f, (x1 - h2f(hp >> 16)) * 2048.0f);
            }
            const int j = 32 * w + 8 * b + 4 * hh;
            put4(lds.qrows, row, offA, j, A[0], A[1]);
            put4(lds.qrows, row, offB, j, Bv[0], Bv[1]);
            if (offC >= 0) put4(lds.qrows, row, offC, j, C[0], C[1]);
        }
        if (w == 0 && hh == 0) lds.rsc[row][rsc_slot] = mul / (2048.0f * sc);
    }
}

// Rotor path: q^ = Phi q on the VALU (each slot is one row of its group's
// 3x3 sandwich matrix; blog section on the random rotation: rotate the
// query once), written over the staged fp32 rows: job (row, group) reads and
// writes that group's three entries, the pad input being 0 (slot 128 lands
// in the row's padding).
template <int ROWS, class Lds>
__device__ __forceinline__ void rotor_qhat_in_place(Lds& lds) {
    // a thread's jobs in batches of four: the batch's LDS reads are all
    // issued before its writes (the compiler cannot tell jobs apart, so
    // one job at a time would serialise every read behind the last write)
    constexpr int JOBS = ROWS * kGroups, PER = (JOBS + kBlock - 1) / kBlock, BATCH = 4;
#pragma unroll
    for (int b0 = 0; b0 < PER; b0 += BATCH) {
        float v[BATCH][3], m[BATCH][9];
        float* qp[BATCH];
        bool ok[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int job = threadIdx.x + (b0 + i) * kBlock;
            ok[i] = b0 + i < PER && job < JOBS;
            const int jc = ok[i] ? job : 0;
            const int r = jc / kGroups, g = jc - r * kGroups;
            qp[i] = &lds.qf[r][3 * g];
            const u32x4 m0 = *reinterpret_cast<const u32x4*>(&lds.rot[12 * g]);
            const u32x4 m1 = *reinterpret_cast<const u32x4*>(&lds.rot[12 * g + 4]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t a0 = m0[k];
                const uint32_t a1 = m1[k];
                m[i][k] = __builtin_bit_cast(float, a0);
                m[i][4 + k] = __builtin_bit_cast(float, a1);
            }
            m[i][8] = lds.rot[12 * g + 8];
            v[i][0] = qp[i][0];
            v[i][1] = qp[i][1];
            v[i][2] = g == kGroups - 1 ? 0.0f : qp[i][2];
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if (!ok[i]) continue;
            float y[3];
#pragma unroll
            for (int rr = 0; rr < 3; ++rr)
                y[rr] = __builtin_fmaf(m[i][3 * rr + 2], v[i][2],
                                       __builtin_fmaf(m[i][3 * rr + 1], v[i][1], m[i][3 * rr] * v[i][0]));
            qp[i][0] = y[0];
            qp[i][1] = y[1];
            qp[i][2] = y[2];
        }
    }
}

// Q1 = 2^11 hi, Q2 = hi, Q3 = lo11 of sc q^ over slots 0..127 (sc a power of
// two putting the row's largest |q^| in [1, 2)), whole 16-byte chunks per
// thread, and the row scalar 1 / (2^11 sc) * inv_sc.
template <int ROWS, class Lds>
__device__ __forceinline__ void rotor_qhat_store(Lds& lds, float inv_sc) {
    constexpr int TPR = kBlock / ROWS, CPT = kD / TPR;
    const int t = threadIdx.x, r = t / TPR, part = t % TPR;
    const float* q = &lds.qf[r][CPT * part];
    float v[CPT];
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        v[k] = q[k];
        mx = fmaxf(mx, fabsf(v[k]));
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float sc = pow2_scale(mx);
#pragma unroll
    for (int c = 0; c < CPT / 8; ++c) {
        u32x4 A, Bv, C;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float x0 = v[8 * c + 2 * d] * sc, x1 = v[8 * c + 2 * d + 1] * sc;
            const uint32_t hp = cvt_pk(x0, x1);
            C[d] = hp;
            A[d] = pk_scale2048(hp);
            Bv[d] = cvt_pk((x0 - h2f(hp & 0xFFFFu)) * 2048.0f, (x1 - h2f(hp >> 16)) * 2048.0f);
        }
        const int chunk = (CPT * part) / 8 + c;
        u32x4* row = lds.qrows + r * kRowStride;
        row[kOffQ1 + chunk] = A;
        row[kOffQ3 + chunk] = Bv;
        row[kOffQ2 + chunk] = C;
    }
    if (part == 0) lds.rsc[r][0] = inv_sc / (2048.0f * sc);
}

// Builds the block's staged query rows (see "staged rows") and row scalars.
// The block's query rows as loaded at kernel start: thread t holds float4 t
// of each 256-float4 slice (rows >= nrows read as zero).
template <int NMT>
struct QueryRegs {
    float4 v[NMT * 32 * 32 / kBlock];
};
template <int NMT>
__device__ __forceinline__ void query_load(const MainArgs& a, int row0, int nrows, QueryRegs<NMT>& qr) {
    const int t = threadIdx.x;
#pragma unroll
    for (int it = 0; it < NMT * 32 * 32 / kBlock; ++it) {
        const int idx = it * kBlock + t, r = idx >> 5, c = idx & 31;
        qr.v[it] = r < nrows ? reinterpret_cast<const float4*>(a.q + static_cast<int64_t>(row0 + r) * kD)[c]
                             : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

template <bool PAD, bool QJL, int NMT, bool OUTL = false, class Lds>
__device__ __forceinline__ void build_query_rows(const MainArgs& a, const QueryRegs<NMT>& qr,
                                                 const QueryFrags<QJL, !PAD>& fr, float inv_sc, Lds& lds,
                                                 int ghead = 0) {
    constexpr int ROWS = NMT * 32;
    constexpr int TPR = kBlock / ROWS;   // threads per row
    constexpr int CPT = kD / TPR;        // coordinates per thread
    const int t = threadIdx.x;
    {
        constexpr int PER = ROWS * 32 / kBlock;
        const float4* v = qr.v;
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int idx = it * kBlock + t, r = idx >> 5, c = idx & 31;
            *reinterpret_cast<float4*>(&lds.qf[r][4 * c]) = v[it];
        }
    }
    __syncthreads();
    if constexpr (OUTL) {
        // the KV head's outlier channels: the query values there are kept for
        // the separate term, then cleared so that S q sees q_in only
        for (int idx = t; idx < ROWS * a.ok; idx += kBlock) {
            const int r = idx / a.ok, i = idx % a.ok;
            lds.qo[r][i] = lds.qf[r][a.ochans[static_cast<int64_t>(ghead) * a.ok + i] & 127];
        }
        __syncthreads();
        for (int idx = t; idx < ROWS * a.ok; idx += kBlock) {
            const int r = idx / a.ok, i = idx % a.ok;
            lds.qf[r][a.ochans[static_cast<int64_t>(ghead) * a.ok + i] & 127] = 0.0f;
        }
        __syncthreads();
    }
    {
        const int r = t / TPR, part = t % TPR;
        const float* q = lds.qf[r];
        float mq = 0.0f;
#pragma unroll
        for (int k = 0; k < CPT; ++k) mq = fmaxf(mq, fabsf(q[part * CPT + k]));
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) mq = fmaxf(mq, __shfl_xor(mq, o));
        if (part == 0) {
            lds.s0[r] = pow2_scale(mq);
            // rotor slot 128 (last row of group 42, pad input 0) in fp32
            float qpad = 0.0f;
            if constexpr (PAD) {
                const float* m42 = a.rotmat + 9 * 42;
                qpad = __builtin_fmaf(m42[8], 0.0f, __builtin_fmaf(m42[7], q[127], m42[6] * q[126]));
            }
            lds.rsc[r][1] = 0.0f;
            lds.rsc[r][2] = qpad;
            lds.rsc[r][3] = 0.0f;
        }
    }
    __syncthreads();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    // the split operands live where the staged rows go later
    static_assert(NMT * 8 * 3 * 64 <= ROWS * kRowStride, "split operands overlay the staged rows");
    u32x4* bop = lds.qrows;
    query_split<NMT>(lds, bop, w, l);
    float s0r[NMT];
#pragma unroll
    for (int nt = 0; nt < NMT; ++nt) s0r[nt] = lds.s0[32 * nt + (l & 31)];
    __syncthreads();
    // rotor: q^ on the VALU over the fp32 rows (S q' reads the split operands)
    if constexpr (PAD) rotor_qhat_in_place<ROWS>(lds);
    float ox[NMT][16], os[NMT][16];
    query_products<QJL, !PAD, NMT>(fr, bop, s0r, l, ox, os);
    if constexpr (!PAD) product_row_max<NMT>(ox, lds, 0, w, l);
    if constexpr (QJL) product_row_max<NMT>(os, lds, 1, w, l);
    __syncthreads();
    if constexpr (PAD) rotor_qhat_store<ROWS>(lds, inv_sc);
    else product_store<NMT>(ox, lds, 0, w, l, kOffQ1, kOffQ3, kOffQ2, 0, inv_sc);
    if constexpr (QJL) product_store<NMT>(os, lds, 1, w, l, kOffP1, kOffP2, -1, 1, 1.0f);
    __syncthreads();
}

// NMT = 1, 2: 32-row M tiles (32x32x16 MFMAs), NMT = 0: groups of at most 16
// query rows on 16x16x32 MFMAs (the query side is built as for one 32-row
// tile and rows 0..15 are read).
template <int B, bool QJL, bool PAD, int NMT, bool OUTL = false>
__global__ __launch_bounds__(256) void score_kernel(MainArgs a) {
    static_assert(!OUTL || (B == 0 && QJL && !PAD), "outlier channels are separated for QJL-only keys");
    constexpr int NB = NMT > 0 ? NMT : 1;   // 32-row tiles of the query build
    constexpr int KPL = NMT > 0 ? 2 : 4;    // keys per lane in a 64-key tile
    constexpr int NC = PAD ? kRotCoords : kD;
    constexpr int W = (NC * B + 31) / 32;
    constexpr int L = 1 << B;
    constexpr int WA = W > 0 ? W : 1;   // B = 0: QJL-only keys, no code words
    constexpr int SW = W > 4 ? W : 4;
    constexpr int ROWS = NB * 32;
    // 1- and 2-bit codes: four codes (one byte or nibble of the stream) select
    // two dwords of C_hi halves and two of C_lo halves, which land in the MFMA
    // operand as they are; wider codes go by pairs.  Sign bytes map to their
    // four +-1 dwords through a table while LDS stays within two blocks per CU.
    constexpr bool QUAD = B == 1 || B == 2;
    constexpr int NQ = QUAD ? 1 << (4 * B) : 1;
    // C_lo entries start 2056 bytes after the C_hi ones: no two-address LDS
    // read can fetch a C_hi and a C_lo entry together, so each 8-byte read
    // lands in its own half of an MFMA operand without register moves
    constexpr int QLO = QUAD ? 257 : 1;
    constexpr bool STAB = QJL && B <= 3;
    struct Lds {
        uint32_t pairs[L * L][2];     // codes (a, b) -> {C_hi[a] | C_hi[b] << 16, C_lo[a] | C_lo[b] << 16}
        uint2 quad[QLO + NQ];         // codes (a, b, c, d) -> C_hi halves at [p], C_lo halves at [QLO + p]
        u32x4 sigt[STAB ? 256 : 1];   // sign byte -> sigma8
        float rsc[ROWS][4];           // {1 / (2^11 s_q s_c), 1 / (2^11 s_p), q^_128, 0}
        float cent[L];
        float s0[ROWS];               // power of two putting max |q| of a row in [1, 2)
        float part[2][4][ROWS];       // per-wave partial maxima of the two products
        uint32_t stage[4][64 * SW + 4];   // (+4: the 3-bit reads of the 16-row loop run one word past)
        float qf[ROWS][kD + 4];
        u32x4 qrows[ROWS * kRowStride];
        float rot[PAD ? 12 * kGroups : 4];             // rotor matrices, 12 floats per group
        float qo[OUTL ? ROWS : 1][16];                 // query values on the outlier channels
        uint32_t ostage[OUTL ? 4 : 1][OUTL ? 512 : 1];  // per wave: the tile's outlier halves
    };
    __shared__ Lds lds;

    const int head = blockIdx.y;   // KV head within this call (query block folded below)
    const int qblocks = (a.group + a.rows_per_block - 1) / a.rows_per_block;
    const int kvh = head / qblocks, qb = head % qblocks;
    const int row0 = kvh * a.group + qb * a.rows_per_block;
    const int nrows = min(a.rows_per_block, a.group - qb * a.rows_per_block);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ntiles = (a.t + 63) / 64;
    const int64_t rbase = static_cast<int64_t>(a.kv_head0 + kvh) * a.kv_stride;
    const int64_t tstep = gridDim.x * 4LL;
    const int t = threadIdx.x;
    // Global loads in the order of use (loads complete in order): the
    // codebook and (rotor) the sandwich matrices, the query rows, the S
    // (and dense Pi) fragments of the query build, then the first tile's record.
    const float cv = t < L ? a.cent[t] : 0.0f;
    constexpr int RV = (12 * kGroups + kBlock - 1) / kBlock;
    float rv[RV] = {};
    if constexpr (PAD) {
#pragma unroll
        for (int k = 0; k < RV; ++k) {
            const int i = t + kBlock * k, g = i / 12, e = i - 12 * g;
            rv[k] = (g < kGroups && e < 9) ? a.rotmat[9 * g + e] : 0.0f;
        }
    }
    QueryRegs<NB> qr;
    query_load<NB>(a, row0, nrows, qr);
    QueryFrags<QJL, !PAD> fr;
    query_frags<QJL, !PAD>(a, wave, lane_id(), fr);
    RecRegs<W, KPL, OUTL> rec;
    int64_t tile = blockIdx.x * 4LL + wave;
    const int ghead = a.kv_head0 + kvh;
    if (tile < ntiles) rec_fetch<W, QJL, KPL, OUTL>(a, rbase, ghead, tile * 64, rec, lane_id());

    float inv_sc;
    {
        if (t < L) lds.cent[t] = cv;
        if constexpr (PAD) {
#pragma unroll
            for (int k = 0; k < RV; ++k)
                if (t + kBlock * k < 12 * kGroups) lds.rot[t + kBlock * k] = rv[k];
        }
        __syncthreads();
        const float cmax = fabsf(lds.cent[L - 1]) > fabsf(lds.cent[0]) ? fabsf(lds.cent[L - 1]) : fabsf(lds.cent[0]);
        const float sc = pow2_scale(cmax);
        inv_sc = 1.0f / sc;
        for (int p = t; p < L * L; p += kBlock) {
            uint32_t h0, l0, h1, l1;
            split_h11(lds.cent[p & (L - 1)] * sc, &h0, &l0);
            split_h11(lds.cent[p >> B] * sc, &h1, &l1);
            lds.pairs[p][0] = h0 | (h1 << 16);
            lds.pairs[p][1] = l0 | (l1 << 16);
        }
        if constexpr (QUAD) {
            for (int p = t; p < NQ; p += kBlock) {
                uint32_t h[4], o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) split_h11(lds.cent[(p >> (B * i)) & (L - 1)] * sc, &h[i], &o[i]);
                lds.quad[p] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                lds.quad[QLO + p] = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            }
        }
        if constexpr (STAB) {
            for (int p = t; p < 256; p += kBlock) lds.sigt[p] = sigma8(static_cast<uint32_t>(p));
        }
    }
    build_query_rows<PAD, QJL, NB, OUTL>(a, qr, fr, inv_sc, lds, ghead);
    uint32_t* ost = lds.ostage[wave];
    const uint16_t* oh = reinterpret_cast<const uint16_t*>(ost);

    uint32_t* st = lds.stage[wave];
    const int64_t nk = a.t;   // keys of this head
    const char* pairc = reinterpret_cast<const char*>(lds.pairs);

    // C_hi / C_lo operand halves of eight codes held in the low 8 B bits of f
    auto decode8 = [&](uint32_t f, u32x4& ch, u32x4& cl) {
        if constexpr (QUAD) {
            const uint32_t i0 = f & (NQ - 1), i1 = (f >> (4 * B)) & (NQ - 1);
            const uint2 h0 = lds.quad[i0], h1 = lds.quad[i1];
            const uint2 o0 = lds.quad[QLO + i0], o1 = lds.quad[QLO + i1];
            ch = u32x4{h0.x, h0.y, h1.x, h1.y};
            cl = u32x4{o0.x, o0.y, o1.x, o1.y};
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t addr = ((f >> (2 * B * q)) & (L * L - 1)) * 8u;
                ch[q] = *reinterpret_cast<const uint32_t*>(pairc + addr);
                cl[q] = *reinterpret_cast<const uint32_t*>(pairc + addr + 4);
            }
        }
    };

    if constexpr (NMT == 0) {
        // Lane (c, g) = (l % 16, l / 16) serves keys 16 j + c (j = 0..3) of the
        // 64-key tile and, in the 32-wide K step ks, slots 32 g + 8 ks .. + 7
        // (the order of the K slots is free; this one gives each lane 32
        // consecutive slots, so their code bits are B consecutive words of
        // the key's record and their sign bits one sign word, read once per
        // key); the A operand of step ks is chunk 4 g + ks of staged row c.
        // The block's query rows do not change, so the A operands are read from
        // LDS once for all of the wave's tiles (Q1 = 2^11 Q2 is rebuilt by an
        // exact packed multiply): LDS bandwidth bounds this loop.
        u32x4 aq2[4], aq3[4], ap1[4], ap2[4];
        {
            const int l = lane_id(), c = l & 15, g = l >> 4;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int r = c * kRowStride + 4 * g + ks;
                if constexpr (B > 0) {
                    aq2[ks] = lds.qrows[r + kOffQ2];
                    aq3[ks] = lds.qrows[r + kOffQ3];
                }
                if constexpr (QJL) {
                    ap1[ks] = lds.qrows[r + kOffP1];
                    ap2[ks] = lds.qrows[r + kOffP2];
                }
            }
        }
        // largest scale * estimate of rows 4 g .. 4 g + 3 over this lane's keys
        float rmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        for (; tile < ntiles; tile += tstep) {
            const int z = opaque_zero();
            const int l = lane_id() + z;
            const int c = l & 15, g = l >> 4;
            const int64_t kbase = tile * 64;
            uint32_t cs[4][4];          // [j][ks]: the lane's 8 B code bits, from bit 0
            float cpad[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (B > 0) {
                wave_lds_sync();
#pragma unroll
                for (int it = 0; it < W; ++it) st[it * 64 + l] = rec.c[it];
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t* kw = st + (16 * j + c) * W;
                    // slots 32 g .. 32 g + 31: words B g .. B g + B - 1 of the key's
                    // stream; step ks starts at bit 8 B ks of them (only 3-bit
                    // codes straddle words)
                    uint32_t lw[B];
#pragma unroll
                    for (int k = 0; k < B; ++k) lw[k] = kw[B * g + k];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int bit = 8 * B * ks, wi = bit >> 5, off = bit & 31;
                        if (off + 8 * B > 32)
                            cs[j][ks] = __builtin_amdgcn_alignbit(lw[wi + 1 < B ? wi + 1 : wi], lw[wi], off);
                        else cs[j][ks] = lw[wi] >> off;
                    }
                    if constexpr (PAD) cpad[j] = lds.cent[kw[4 * B] & (L - 1)];
                }
            }
            uint32_t sb[4][4];   // [j][ks]: the lane's sign byte
            if constexpr (QJL) {
                wave_lds_sync();
#pragma unroll
                for (int it = 0; it < 4; ++it) st[it * 64 + l] = rec.s[it];
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // sign indices 32 g .. 32 g + 31: sign word g, byte ks for step ks
                    const uint32_t sw = st[(16 * j + c) * 4 + g];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) sb[j][ks] = (sw >> (8 * ks)) & 0xFFu;
                }
            }
            wave_lds_sync();
            float kn[4], kg[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kn[j] = h2f(rec.kn[j]);
                kg[j] = QJL ? h2f(rec.kg[j]) * a.qjl_scale : 0.0f;
            }
            stage_outliers(a, rec, ost, l);
            if (tile + tstep < ntiles) rec_fetch<W, QJL, KPL, OUTL>(a, rbase, ghead, (tile + tstep) * 64, rec, l);

            f32x4 acc1[4], acc2[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc1[j] = f32x4{};
                acc2[j] = f32x4{};
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if constexpr (B > 0) {
                    const u32x4 q2 = aq2[ks], q3 = aq3[ks];
                    u32x4 q1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t v = q2[e];
                        q1[e] = pk_scale2048(v);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x4 ch, cl;
                        decode8(cs[j][ks], ch, cl);
                        acc1[j] = mfma16(q1, ch, acc1[j]);
                        acc1[j] = mfma16(q2, cl, acc1[j]);
                        acc1[j] = mfma16(q3, ch, acc1[j]);
                    }
                }
                if constexpr (QJL) {
                    const u32x4 p1 = ap1[ks], p2 = ap2[ks];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x4 sv;
                        if constexpr (STAB) sv = lds.sigt[sb[j][ks]];
                        else sv = sigma8(sb[j][ks]);
                        acc2[j] = mfma16(p1, sv, acc2[j]);
                        acc2[j] = mfma16(p2, sv, acc2[j]);
                    }
                }
            }

            // epilogue: lane (c, g) holds rows 4 g .. 4 g + 3 of key 16 j + c;
            // rows past nrows fall outside the descriptor's range, keys past
            // the end get an offset beyond it
            const rsrc_t rs = make_rsrc(a.scores + static_cast<int64_t>(row0) * a.ld + kbase,
                                        static_cast<uint32_t>(((nrows - 1) * a.ld + (nk - kbase)) * 4));
            // OUTL: sum_i q_{c_i} o^_i for rows 4 g + i of keys 16 j + c
            float ot[4][4] = {};
            if constexpr (OUTL) {
                wave_lds_sync();
                for (int i = 0; i < a.ok; ++i) {
                    float ov[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) ov[j] = h2f(oh[(16 * j + c) * a.ok + i]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float qv = lds.qo[4 * g + r][i];
#pragma unroll
                        for (int j = 0; j < 4; ++j) ot[r][j] = __builtin_fmaf(qv, ov[j], ot[r][j]);
                    }
                }
            }
            if (4 * g < nrows) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * g + i;
                    const float* rsv = lds.rsc[row];
                    const float s0 = rsv[0], s1 = rsv[1], s2 = rsv[2];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = 16 * j + c;
                        const float e1 = acc1[j][i];
                        float v = e1 * s0;
                        if constexpr (PAD) v = __builtin_fmaf(s2, cpad[j], v);
                        if constexpr (QJL) {
                            const float e2 = acc2[j][i];
                            v = __builtin_fmaf(kg[j], e2 * s1, v);
                        }
                        v *= kn[j];
                        if constexpr (OUTL) v += ot[i][j];
                        const bool in = kbase + key < nk;
                        const uint32_t voff = in ? static_cast<uint32_t>((row * a.ld + key) * 4) : 0x80000000u;
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff, 0,
                                                              kNonTemporal);
                        if (a.rm.ptr != nullptr && in) rmax[i] = fmaxf(rmax[i], v * a.rm.scale);
                    }
                }
            }
        }
        if (a.rm.ptr != nullptr) {
            // the 16 lanes of each row quad, then the four waves, through LDS
            const int l = lane_id(), c = l & 15, g = l >> 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) rmax[i] = fmaxf(rmax[i], __shfl_xor(rmax[i], o));
            __syncthreads();
            if (c == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) lds.part[0][wave][4 * g + i] = rmax[i];
            }
            __syncthreads();
            if (t < nrows) {
                const float m = fmaxf(fmaxf(lds.part[0][0][t], lds.part[0][1][t]),
                                      fmaxf(lds.part[0][2][t], lds.part[0][3][t]));
                a.rm.ptr[static_cast<int64_t>(blockIdx.x) * a.rm.ld + row0 + t] = m;
            }
        }
    } else {
    for (; tile < ntiles; tile += tstep) {
        const int z = opaque_zero();
        const int l = lane_id() + z;
        const int n = l & 31, hh = l >> 5;
        const int64_t kbase = tile * 64;

        // code words of keys n and 32 + n, shifted so this lane's K slots
        // start at bit 0 (slot 8 hh of each block is bit 8 B hh further)
        uint32_t cw[2][WA];
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < W; ++it) st[it * 64 + l] = rec.c[it];
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < W; ++k) {
            cw[0][k] = st[n * W + k];
            cw[1][k] = st[(32 + n) * W + k];
        }
        float cpad[2] = {0.0f, 0.0f};
        if constexpr (PAD && B > 0) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) cpad[nt] = lds.cent[cw[nt][4 * B] & (L - 1)];
        }
        uint32_t cs[2][WA];
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
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < 4; ++it) st[it * 64 + l] = rec.s[it];
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
            kn[nt] = h2f(rec.kn[nt]);
            kg[nt] = QJL ? h2f(rec.kg[nt]) * a.qjl_scale : 0.0f;
        }
        // next tile's record, in flight during this tile's MFMAs and stores
        stage_outliers(a, rec, ost, l);
        if (tile + tstep < ntiles) rec_fetch<W, QJL, KPL, OUTL>(a, rbase, ghead, (tile + tstep) * 64, rec, l);

        f32x16 acc1[NMT][2], acc2[NMT][2];
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc1[m][nt] = f32x16{};
                acc2[m][nt] = f32x16{};
            }

        if constexpr (B > 0) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                // (no scheduling barrier: lookups of the next block may move up)
                u32x4 ch[2], cl[2];
                if constexpr (QUAD) {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        // this lane's eight slots of block kb: 8 B bits (cs is pre-shifted by 8 B hh)
                        const int bit = 16 * B * kb;
                        const uint32_t f = cs[nt][bit >> 5] >> (bit & 31);
                        const uint32_t i0 = f & (NQ - 1), i1 = (f >> (4 * B)) & (NQ - 1);
                        const uint2 h0 = lds.quad[i0], h1 = lds.quad[i1];
                        const uint2 o0 = lds.quad[QLO + i0], o1 = lds.quad[QLO + i1];
                        ch[nt] = u32x4{h0.x, h0.y, h1.x, h1.y};
                        cl[nt] = u32x4{o0.x, o0.y, o1.x, o1.y};
                    }
                } else {
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
        }
        if constexpr (QJL) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                // (no scheduling barrier)
                u32x4 s[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const uint32_t byte = (sg[nt][kb >> 1] >> (16 * (kb & 1))) & 0xFFu;
                    if constexpr (STAB) s[nt] = lds.sigt[byte];
                    else s[nt] = sigma8(byte);
                }
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
        // OUTL: sum_i q_{c_i} o^_i for the lane's rows of keys n and 32 + n
        float ot[OUTL ? NMT : 1][OUTL ? 16 : 1][2] = {};
        if constexpr (OUTL) {
            wave_lds_sync();
            for (int i = 0; i < a.ok; ++i) {
                const float ov0 = h2f(oh[n * a.ok + i]), ov1 = h2f(oh[(32 + n) * a.ok + i]);
#pragma unroll
                for (int m = 0; m < NMT; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float qv = lds.qo[32 * m + 8 * (r / 4) + (r % 4) + 4 * hh][i];
                        ot[m][r][0] = __builtin_fmaf(qv, ov0, ot[m][r][0]);
                        ot[m][r][1] = __builtin_fmaf(qv, ov1, ot[m][r][1]);
                    }
            }
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rowc = 32 * m + 8 * (r / 4) + (r % 4);   // row without the lane-half term 4 hh
                if constexpr (NMT == 1) {
                    if (rowc >= nrows) continue;   // no lane holds a live row (small GQA groups)
                }
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
                    if constexpr (OUTL) v += ot[m][r][nt];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff[nt],
                                                          static_cast<int>(rowc * a.ld * 4), kNonTemporal);
                }
            }
    }
    }
}

// Grid: (key slices, KV heads x query-row blocks).  Every block pays for
// building its query rows once, so the slices per (head, row block) are only
// as many as fill the workgroup slots of the chip in one round (two per CU
// for the 32-row variant, one for the 64-row variant, whose LDS is larger);
// each wave then walks many 64-key tiles.  At least one tile per wave.
static int64_t score_slices(int64_t t, int64_t units, int nmt) {
    const int64_t ntiles = (t + 63) / 64;
    const int64_t want = (ntiles + 3) / 4;
    const int64_t slots = 256LL * (nmt < 2 ? 2 : 1);
    int64_t gx = slots / units;
    if (gx > want) gx = want;
    if (gx < 1) gx = 1;
    return gx;
}
int score_slices16(int64_t t, int kv_heads) { return static_cast<int>(score_slices(t, kv_heads, 0)); }

template <int B, bool QJL, bool PAD, int NMT, bool OUTL = false>
static void launch_main(const MainArgs& a, int kv_heads, int qblocks, hipStream_t s) {
    const int64_t gx = score_slices(a.t, static_cast<int64_t>(kv_heads) * qblocks, NMT);
    hipLaunchKernelGGL((score_kernel<B, QJL, PAD, NMT, OUTL>), dim3(static_cast<unsigned>(gx), kv_heads * qblocks),
                       dim3(kBlock), 0, s, a);
}

template <int B, bool QJL>
static void launch_main_b(bool dense, int nmt, const MainArgs& a, int kv_heads, int qblocks, hipStream_t s) {
    if (dense) {
        if (nmt == 0) launch_main<B, QJL, false, 0>(a, kv_heads, qblocks, s);
        else if (nmt == 1) launch_main<B, QJL, false, 1>(a, kv_heads, qblocks, s);
        else launch_main<B, QJL, false, 2>(a, kv_heads, qblocks, s);
    } else {
        if (nmt == 0) launch_main<B, QJL, true, 0>(a, kv_heads, qblocks, s);
        else if (nmt == 1) launch_main<B, QJL, true, 1>(a, kv_heads, qblocks, s);
        else launch_main<B, QJL, true, 2>(a, kv_heads, qblocks, s);
    }
}

hipError_t score(const ScoreTables& t, const float* q, int hq, int group, const uint32_t* codes,
                 const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms, int64_t tkeys,
                 int64_t kv_stride, int kv_head0, float* scores, int64_t ld_scores, hipStream_t s,
                 const PageTable& pt, const ScoreOutliers& so, const RowMax& rm) {
    MainArgs a;
    a.rm = rm;
    a.pt = pt;
    a.q = q;
    a.rotmat = t.rot.rotmat;
    a.x_hi = t.dense ? t.den.pi_hi : t.rot.phi_hi;
    a.x_lo = t.dense ? t.den.pi_lo : t.rot.phi_lo;
    a.s_rows = t.dense ? t.den.s_rows : t.rot.s_rows;
    a.codes = codes;
    a.norms = norms;
    a.signs = signs;
    a.rnorms = rnorms;
    a.t = tkeys;
    a.kv_stride = kv_stride;
    a.kv_head0 = kv_head0;
    a.group = group;
    a.rows_per_block = group < 64 ? group : 64;
    a.cent = t.dense ? t.den.cent : t.rot.cent;
    a.qjl_scale = t.qjl_scale;
    a.scores = scores;
    a.ld = ld_scores;
    const int kv_heads = hq / group;
    const int qblocks = (group + 63) / 64;
    const int nmt = a.rows_per_block > 32 ? 2 : a.rows_per_block > 16 ? 1 : 0;
    if (rm.ptr != nullptr && nmt != 0) return hipErrorInvalidValue;
    if (so.chans) {
        if (t.mse_bits != 0 || !t.qjl) return hipErrorInvalidValue;
        a.ochans = so.chans;
        a.outl = so.values;
        a.ok = so.k;
        if (nmt == 0) launch_main<0, true, false, 0, true>(a, kv_heads, qblocks, s);
        else if (nmt == 1) launch_main<0, true, false, 1, true>(a, kv_heads, qblocks, s);
        else launch_main<0, true, false, 2, true>(a, kv_heads, qblocks, s);
        return hipGetLastError();
    }
    switch (t.mse_bits * 2 + (t.qjl ? 1 : 0)) {
        case 1: launch_main_b<0, true>(t.dense, nmt, a, kv_heads, qblocks, s); break;
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
