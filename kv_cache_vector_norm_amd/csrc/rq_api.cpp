// C ABI of the codec (declared in include/rq.h): argument checks, session
// set-up, and dispatch to the HIP launchers.  No call here allocates after
// rq_init, and nothing is enqueued when an argument check fails.
#include "../../include/rq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "rq_host.h"
#include "rq_kernels.h"

static_assert(RQ_SCORE_CHUNK == rqk::kScoreChunkRows, "score chunk size");
static_assert(RQ_MAX_OUTLIERS == rqk::kMaxOutliers, "outlier channels per head");
static_assert(RQ_ATTEND_NOALLOC_BYTES == rqk::kNoAllocScratchBytes, "fixed attention scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(RQ_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Test hook: RQ_TEST_FAIL_ALLOC=k makes the k-th device allocation of an
// rq_init call fail (k >= 1), to exercise the clean-up path.
int g_alloc_countdown_init() {
    const char* v = std::getenv("RQ_TEST_FAIL_ALLOC");
    return v ? std::atoi(v) : 0;
}

struct DevAlloc {
    int countdown;
    std::vector<void*> owned;
    explicit DevAlloc(int k) : countdown(k) {}
    hipError_t alloc(void** p, size_t bytes) {
        if (countdown > 0 && --countdown == 0) return hipErrorOutOfMemory;
        const hipError_t e = hipMalloc(p, bytes);
        if (e == hipSuccess) owned.push_back(*p);
        return e;
    }
    void release() {
        for (void* p : owned) (void)hipFree(p);
        owned.clear();
    }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int dtype) { return dtype == RQ_F16 ? 2 : 4; }

}  // namespace

struct rq_ctx {
    rqh::Tables host;
    int device = -1;
    uint64_t seed = 0;
    std::vector<void*> dev;   // every device allocation of this session
    // rotor tables
    float* rotmat = nullptr;
    float* rotmat16 = nullptr;
    float* thr = nullptr;
    float* cent = nullptr;
    rqk::u32x4_t* bins = nullptr;
    // QJL
    uint16_t* s_rows = nullptr;
    uint16_t* s_cols = nullptr;
    uint16_t* s_fwd = nullptr;
    uint16_t* s_back = nullptr;
    uint16_t* phi_hi = nullptr;
    uint16_t* phi_lo = nullptr;
    // dense (TurboQuant): Pi split into exact half pairs, both layouts
    uint16_t* pi_hi = nullptr;
    uint16_t* pi_lo = nullptr;
    uint16_t* pit_hi = nullptr;
    uint16_t* pit_lo = nullptr;
    // dense codec kernels (two lanes per vector): Pi and Pi^T permuted
    uint16_t* pi2_hi = nullptr;
    uint16_t* pi2_lo = nullptr;
    uint16_t* pit2_hi = nullptr;
    uint16_t* pit2_lo = nullptr;
    uint16_t* t2_hi = nullptr;   // T = S Pi^T (sessions with QJL)
    uint16_t* t2_lo = nullptr;
    // PolarQuant: fp32 Pi and the (cos, sin) table of its angle codebooks
    float* pi32 = nullptr;
    float* pq_tab = nullptr;
};

extern "C" {

const char* rq_last_error(void) { return g_last_error.c_str(); }

const char* rq_version(void) { return "rq-mi355x 1.0 (gfx950)"; }

int rq_bench_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const char* fn = "rq_bench_copy";
    if (bytes < 0 || bytes % 16) return fail(RQ_EINVAL, std::string(fn) + ": bytes must be a non-negative multiple of 16");
    if (bytes == 0) return RQ_OK;
    if (!src || !dst) return fail(RQ_EINVAL, std::string(fn) + ": NULL pointer");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(RQ_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
    const char* s8 = static_cast<const char*>(src);
    const char* d8 = static_cast<const char*>(dst);
    if (s8 < d8 + bytes && d8 < s8 + bytes) return fail(RQ_EINVAL, std::string(fn) + ": src and dst overlap");
    const hipError_t e = rqk::copy_bytes(src, dst, bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RQ_OK : hip_fail(e, fn);
}

static void to_abi(const rqh::Layout& l, rq_layout_t* out) {
    out->d = l.d;
    out->bits = l.bits;
    out->mse_bits = l.mse_bits;
    out->mode = l.mode;
    out->n_coords = l.n_coords;
    out->n_groups = l.n_groups;
    out->levels = l.levels;
    out->code_words = l.code_words;
    out->sign_words = l.sign_words;
    out->record_bytes = l.record_bytes;
}

int rq_layout(int d, int bits, int mode, rq_layout_t* out) {
    if (!out) return fail(RQ_EINVAL, "rq_layout: out is NULL");
    rqh::Layout l;
    std::string err;
    const int rc = rqh::make_layout(d, bits, mode, &l, &err);
    if (rc) return fail(rc == 2 ? RQ_EUNSUPPORTED : RQ_EINVAL, "rq_layout: " + err);
    to_abi(l, out);
    return RQ_OK;
}

static void copy_params(const rqh::Tables& t, rq_params_host_t* out) {
    auto cp = [](void* dst, const void* src, size_t bytes) {
        if (dst && bytes) std::memcpy(dst, src, bytes);
    };
    cp(out->rotors, t.rotors.data(), t.rotors.size() * sizeof(float));
    cp(out->rotmats, t.rotmats.data(), t.rotmats.size() * sizeof(float));
    cp(out->centroids, t.centroids.data(), t.centroids.size() * sizeof(float));
    cp(out->boundaries, t.boundaries.data(), t.boundaries.size() * sizeof(float));
    cp(out->pi, t.pi.data(), t.pi.size() * sizeof(float));
    cp(out->s, t.s.data(), t.s.size() * sizeof(uint16_t));
}

int rq_host_params(int d, int bits, uint64_t seed, int mode, rq_params_host_t* out) {
    if (!out) return fail(RQ_EINVAL, "rq_host_params: out is NULL");
    rqh::Tables t;
    std::string err;
    const int rc = rqh::make_tables(d, bits, seed, mode, &t, &err);
    if (rc) return fail(rc == 2 ? RQ_EUNSUPPORTED : RQ_EINVAL, "rq_host_params: " + err);
    copy_params(t, out);
    return RQ_OK;
}

int rq_host_quantizer(int d, int bits, int mode, float* bias, uint32_t* table) {
    if (!bias || !table) return fail(RQ_EINVAL, "rq_host_quantizer: NULL argument");
    rqh::Tables t;
    std::string err;
    const int rc = rqh::make_tables(d, bits, 0, mode, &t, &err);
    if (rc) return fail(rc == 2 ? RQ_EUNSUPPORTED : RQ_EINVAL, "rq_host_quantizer: " + err);
    if (mode & RQ_POLAR) return fail(RQ_EINVAL, "rq_host_quantizer: RQ_POLAR sessions have no slot table");
    *bias = t.bin_b;
    std::memcpy(table, t.bins.data(), t.bins.size() * sizeof(rqh::BinEntry));
    return RQ_OK;
}

int rq_get_layout(const rq_ctx* ctx, rq_layout_t* out) {
    if (!ctx || !out) return fail(RQ_EINVAL, "rq_get_layout: NULL argument");
    to_abi(ctx->host.lay, out);
    return RQ_OK;
}

int rq_get_params(const rq_ctx* ctx, rq_params_host_t* out) {
    if (!ctx || !out) return fail(RQ_EINVAL, "rq_get_params: NULL argument");
    copy_params(ctx->host, out);
    return RQ_OK;
}

void rq_free(rq_ctx* ctx) {
    if (!ctx) return;
    int cur = -1;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != ctx->device && ctx->device >= 0;
    if (switch_dev) (void)hipSetDevice(ctx->device);
    for (void* p : ctx->dev) (void)hipFree(p);
    if (switch_dev) (void)hipSetDevice(cur);
    delete ctx;
}

int rq_init(int d, int bits, uint64_t seed, int mode, rq_ctx** out) {
    if (!out) return fail(RQ_EINVAL, "rq_init: out is NULL");
    *out = nullptr;
    rq_ctx* ctx = new (std::nothrow) rq_ctx;
    if (!ctx) return fail(RQ_ENOMEM, "rq_init: host allocation failed");
    std::string err;
    const int rc = rqh::make_tables(d, bits, seed, mode, &ctx->host, &err);
    if (rc) {
        delete ctx;
        return fail(rc == 2 ? RQ_EUNSUPPORTED : RQ_EINVAL, "rq_init: " + err);
    }
    ctx->seed = seed;
    hipError_t e = hipGetDevice(&ctx->device);
    if (e != hipSuccess) {
        delete ctx;
        return hip_fail(e, "rq_init: hipGetDevice");
    }
    const rqh::Tables& t = ctx->host;
    const int n = t.lay.d;
    DevAlloc da(g_alloc_countdown_init());
    auto upload = [&](void** dst, const void* src, size_t bytes) -> hipError_t {
        if (bytes == 0) {
            *dst = nullptr;
            return hipSuccess;
        }
        hipError_t r = da.alloc(dst, bytes);
        if (r != hipSuccess) return r;
        return hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice);
    };
    // derived half tables
    std::vector<uint16_t> s_cols, s_fwd, s_back, pi_hi, pi_lo, pit_hi, pit_lo, phi_hi, phi_lo;
    std::vector<uint16_t> pi2_hi, pi2_lo, pit2_hi, pit2_lo, t2_hi, t2_lo;
    std::vector<float> pq_tab;
    const bool polar = mode & RQ_POLAR;
    const bool rotor = !(mode & (RQ_DENSE | RQ_POLAR));
    auto half_value = [](uint16_t h) {
        const int ex = (h >> 10) & 0x1F, mant = h & 0x3FF;
        const double v = ex == 0 ? std::ldexp(static_cast<double>(mant), -24) : std::ldexp(1.0 + mant / 1024.0, ex - 15);
        return (h & 0x8000) ? -v : v;
    };
    // exact-enough half pair of s v: hi = half(s v), lo = half((s v - hi) * 2^11)
    auto split_scaled = [half_value](double v, double s, uint16_t* hi, uint16_t* lo) {
        const double x = v * s;
        const uint16_t h = rqh::double_to_half_rne(x);
        *hi = h;
        *lo = rqh::double_to_half_rne((x - half_value(h)) * 2048.0);
    };
    auto split16 = [split_scaled](double v, uint16_t* hi, uint16_t* lo) { split_scaled(v, 16.0, hi, lo); };
    // The dense codec kernels read the matrices they do not stage in LDS in
    // MFMA fragment order: the 16 bytes that lane l takes as the A operand of
    // M tile mt and K block kb (row 32 mt + l % 32, columns 16 kb + 8 (l / 32)
    // .. + 7 of the permuted matrix) sit at ((mt * 8 + kb) * 64 + l) * 16, so
    // one wave's fragment is one contiguous kilobyte.
    auto frag_order = [n](const std::vector<uint16_t>& m) {
        std::vector<uint16_t> f(m.size());
        for (int mt = 0; mt < n / 32; ++mt)
            for (int kb = 0; kb < n / 16; ++kb)
                for (int l = 0; l < 64; ++l)
                    for (int e = 0; e < 8; ++e)
                        f[((static_cast<size_t>(mt) * (n / 16) + kb) * 64 + l) * 8 + e] =
                            m[static_cast<size_t>(32 * mt + (l & 31)) * n + 16 * kb + 8 * (l >> 5) + e];
        return f;
    };
    std::vector<float> rotmat16;
    if (rotor) {
        // the rotor matrices padded to 16 floats (one 64-byte line) per group,
        // for the codec kernels' scalar loads
        rotmat16.assign(static_cast<size_t>(t.lay.n_groups) * 16, 0.0f);
        for (int g = 0; g < t.lay.n_groups; ++g)
            for (int k = 0; k < 9; ++k) rotmat16[16 * g + k] = t.rotmats[9 * g + k];
        // Phi[i][j]: slot i = 3 g + r reads coordinates 3 g .. 3 g + 2 through row r of M_g
        phi_hi.assign(static_cast<size_t>(n) * n, 0);
        phi_lo.assign(static_cast<size_t>(n) * n, 0);
        for (int i = 0; i < n; ++i) {
            const int g = i / 3, r = i % 3;
            for (int c = 0; c < 3; ++c) {
                const int j = 3 * g + c;
                if (j >= n) continue;
                split16(static_cast<double>(t.rotmats[9 * g + 3 * r + c]), &phi_hi[i * n + j], &phi_lo[i * n + j]);
            }
        }
    }
    if (mode & RQ_QJL) {
        s_cols.resize(t.s.size());
        for (int j = 0; j < n; ++j)
            for (int i = 0; i < n; ++i) s_cols[i * n + j] = t.s[j * n + i];
        s_fwd.resize(t.s.size());
        s_back.resize(t.s.size());
        if (t.lay.mse_bits == 0) {
            // QJL-only kernels (one lane per vector): accumulator row p of a
            // 32-row M tile (lane half h = bit 2 of p) holds sign index /
            // coordinate perm_row(p); K slot k of a 32-wide K pair feeds sign
            // index perm_k(k).
            auto perm_row = [](int p) { return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3); };
            auto perm_k = [](int k) { return (k & ~31) | (((k >> 3) & 1) << 4) | (((k >> 4) & 1) << 3) | (k & 7); };
            for (int p = 0; p < n; ++p)
                for (int k = 0; k < n; ++k) {
                    s_fwd[p * n + k] = t.s[perm_row(p) * n + k];
                    s_back[p * n + k] = t.s[perm_k(k) * n + perm_row(p)];
                }
        } else {
            // Codec kernels with two lanes per vector: local slot j of lane
            // half h is coordinate 66 h + j for rotor sessions, except that
            // half 1's slots 62 and 63 stand for coordinates 64 and 65.  Accumulator element r of
            // half h in M tile mt (row p = 8 (r / 4) + 4 h + r % 4) holds sign
            // index / coordinate slot 64 h + 16 mt + r / slot 16 mt + r; K
            // column 16 kb + 8 h + e takes slot 8 kb + e of half h (forward)
            // or sign index 64 h + 8 kb + e (back-projection).
            // (dense sessions: slot j of half h is coordinate 64 h + j)
            const bool dense_map = mode & RQ_DENSE;
            auto slot_coord = [dense_map](int h, int j) {
                return dense_map ? 64 * h + j : (h == 0 ? j : (j < 62 ? 66 + j : j + 2));
            };
            auto row_half = [](int r) { return ((r & 31) >> 2) & 1; };
            auto row_elem = [](int r) { return (r >> 5) * 16 + 4 * ((r & 31) >> 3) + (r & 3); };
            auto col_half = [](int c) { return (c >> 3) & 1; };
            auto col_slot = [](int c) { return 8 * (c >> 4) + (c & 7); };
            for (int r = 0; r < n; ++r)
                for (int c = 0; c < n; ++c) {
                    const int sign_row = 64 * row_half(r) + row_elem(r);
                    const int coord_col = slot_coord(col_half(c), col_slot(c));
                    const int coord_row = slot_coord(row_half(r), row_elem(r));
                    const int sign_col = 64 * col_half(c) + col_slot(c);
                    s_fwd[r * n + c] = t.s[sign_row * n + coord_col];
                    s_back[r * n + c] = t.s[sign_col * n + coord_row];
                }
            if (dense_map) {
                // The dense kernels form S r as T (y - y^) with T = S Pi^T
                // (r = Pi^T (y - y^) for orthogonal Pi), in the same permuted
                // order as s_fwd with y coordinates for x coordinates; T is
                // an exact-enough half pair T = hi + 2^-11 lo.  S^T is read
                // in fragment order; s_fwd itself is not needed.
                std::vector<double> tm(static_cast<size_t>(n) * n, 0.0);
                for (int i = 0; i < n; ++i)
                    for (int j = 0; j < n; ++j) {
                        double acc = 0.0;
                        for (int k = 0; k < n; ++k)
                            acc += half_value(t.s[i * n + k]) * static_cast<double>(t.pi[j * n + k]);
                        tm[static_cast<size_t>(i) * n + j] = acc;
                    }
                t2_hi.resize(t.s.size());
                t2_lo.resize(t.s.size());
                for (int r = 0; r < n; ++r)
                    for (int c = 0; c < n; ++c)
                        split_scaled(tm[static_cast<size_t>(64 * row_half(r) + row_elem(r)) * n +
                                        slot_coord(col_half(c), col_slot(c))],
                                     1.0, &t2_hi[r * n + c], &t2_lo[r * n + c]);
                t2_hi = frag_order(t2_hi);
                t2_lo = frag_order(t2_lo);
                s_back = frag_order(s_back);
                s_fwd.clear();
            }
        }
    }
    if (polar) {
        // (cos, sin) of the decision boundaries (level 1: t_1..t_7, of which
        // the kernels read t_1, folding the point into the first octant;
        // later levels: all three), then of every centroid, levels in order.
        std::vector<double> bnd, cen;
        for (int k = 0; k < 7; ++k) bnd.push_back(t.boundaries[k]);
        for (int k = 15; k < rqh::kPolarBoundaries; ++k) bnd.push_back(t.boundaries[k]);
        for (float c : t.centroids) cen.push_back(c);
        for (double a : bnd) {
            pq_tab.push_back(static_cast<float>(std::cos(a)));
            pq_tab.push_back(static_cast<float>(std::sin(a)));
        }
        for (double a : cen) {
            pq_tab.push_back(static_cast<float>(std::cos(a)));
            pq_tab.push_back(static_cast<float>(std::sin(a)));
        }
        if (pq_tab.size() != static_cast<size_t>(rqk::kPolarTab)) {
            delete ctx;
            return fail(RQ_EINVAL, "rq_init: PolarQuant table size");
        }
    }
    if (mode & (RQ_DENSE | RQ_POLAR)) {
        // Pi = hi + lo exactly enough: hi = half(Pi * 2^4), lo = half((Pi * 2^4 - hi) * 2^11);
        // the kernels undo the 2^4 and 2^11 scales in fp32.
        pi_hi.resize(t.pi.size());
        pi_lo.resize(t.pi.size());
        pit_hi.resize(t.pi.size());
        pit_lo.resize(t.pi.size());
        for (int r = 0; r < n; ++r)
            for (int c = 0; c < n; ++c) {
                uint16_t h, lo;
                split16(static_cast<double>(t.pi[r * n + c]), &h, &lo);
                pi_hi[r * n + c] = h;
                pi_lo[r * n + c] = lo;
                pit_hi[c * n + r] = h;
                pit_lo[c * n + r] = lo;
            }
    }
    if (mode & (RQ_DENSE | RQ_POLAR)) {
        // The dense and PolarQuant codec kernels' MFMA layouts (two lanes per vector, slot j
        // of half h = coordinate 64 h + j): accumulator row r of M tile mt
        // (lane half h = bit 2 of r % 32, element 4 (r % 32 / 8) + r % 4) is
        // coordinate 64 h + 16 mt + element; K column c is slot 8 (c / 16) +
        // c % 8 of half (c / 8) % 2.  pi2 = Pi, pit2 = Pi^T in that order (pit2 in
        // fragment order; pi2 is staged in LDS row by row).
        auto row_coord = [](int r) { return 64 * (((r & 31) >> 2) & 1) + 16 * (r >> 5) + 4 * ((r & 31) >> 3) + (r & 3); };
        auto col_coord = [](int c) { return 64 * ((c >> 3) & 1) + 8 * (c >> 4) + (c & 7); };
        pi2_hi.resize(t.pi.size());
        pi2_lo.resize(t.pi.size());
        pit2_hi.resize(t.pi.size());
        pit2_lo.resize(t.pi.size());
        for (int r = 0; r < n; ++r)
            for (int c = 0; c < n; ++c) {
                split16(static_cast<double>(t.pi[row_coord(r) * n + col_coord(c)]), &pi2_hi[r * n + c],
                        &pi2_lo[r * n + c]);
                split16(static_cast<double>(t.pi[col_coord(c) * n + row_coord(r)]), &pit2_hi[r * n + c],
                        &pit2_lo[r * n + c]);
            }
        pit2_hi = frag_order(pit2_hi);
        pit2_lo = frag_order(pit2_lo);
    }
    do {
        if (rotor) {
            if ((e = upload(reinterpret_cast<void**>(&ctx->rotmat), t.rotmats.data(), t.rotmats.size() * 4)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->rotmat16), rotmat16.data(), rotmat16.size() * 4)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->phi_hi), phi_hi.data(), phi_hi.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->phi_lo), phi_lo.data(), phi_lo.size() * 2)) != hipSuccess) break;
        }
        if ((e = upload(reinterpret_cast<void**>(&ctx->thr), t.boundaries.data(), t.boundaries.size() * 4)) != hipSuccess) break;
        if ((e = upload(reinterpret_cast<void**>(&ctx->cent), t.centroids.data(), t.centroids.size() * 4)) != hipSuccess) break;
        static_assert(sizeof(rqh::BinEntry) == sizeof(rqk::u32x4_t) && rqh::kBins == rqk::kBinSlots, "slot table");
        if ((e = upload(reinterpret_cast<void**>(&ctx->bins), t.bins.data(), t.bins.size() * sizeof(rqh::BinEntry))) != hipSuccess) break;
        if (mode & RQ_QJL) {
            if ((e = upload(reinterpret_cast<void**>(&ctx->s_rows), t.s.data(), t.s.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->s_cols), s_cols.data(), s_cols.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->s_fwd), s_fwd.data(), s_fwd.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->s_back), s_back.data(), s_back.size() * 2)) != hipSuccess) break;
        }
        if (polar) {
            if ((e = upload(reinterpret_cast<void**>(&ctx->pi32), t.pi.data(), t.pi.size() * 4)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pq_tab), pq_tab.data(), pq_tab.size() * 4)) != hipSuccess) break;
        }
        if (mode & (RQ_DENSE | RQ_POLAR)) {
            if ((e = upload(reinterpret_cast<void**>(&ctx->pi_hi), pi_hi.data(), pi_hi.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pi_lo), pi_lo.data(), pi_lo.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pit_hi), pit_hi.data(), pit_hi.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pit_lo), pit_lo.data(), pit_lo.size() * 2)) != hipSuccess) break;
        }
        if (mode & (RQ_DENSE | RQ_POLAR)) {
            if ((e = upload(reinterpret_cast<void**>(&ctx->pi2_hi), pi2_hi.data(), pi2_hi.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pi2_lo), pi2_lo.data(), pi2_lo.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pit2_hi), pit2_hi.data(), pit2_hi.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->pit2_lo), pit2_lo.data(), pit2_lo.size() * 2)) != hipSuccess) break;
        }
        if (mode & RQ_DENSE) {
            if ((e = upload(reinterpret_cast<void**>(&ctx->t2_hi), t2_hi.data(), t2_hi.size() * 2)) != hipSuccess) break;
            if ((e = upload(reinterpret_cast<void**>(&ctx->t2_lo), t2_lo.data(), t2_lo.size() * 2)) != hipSuccess) break;
        }
    } while (false);
    if (e != hipSuccess) {
        da.release();
        delete ctx;
        if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
            return fail(RQ_ENOMEM, std::string("rq_init: device allocation failed: ") + hipGetErrorString(e));
        return hip_fail(e, "rq_init");
    }
    ctx->dev = da.owned;
    *out = ctx;
    return RQ_OK;
}

// ------------------------------------------------------------ checks --
static int check_ctx(const rq_ctx* ctx, bool dense, const char* fn) {
    if (!ctx) return fail(RQ_EINVAL, std::string(fn) + ": ctx is NULL");
    if (ctx->host.lay.mode & RQ_POLAR)
        return fail(RQ_EINVAL, std::string(fn) + ": a PolarQuant session (use pq_*)");
    const bool is_dense = ctx->host.lay.mode & RQ_DENSE;
    if (dense != is_dense)
        return fail(RQ_EINVAL, std::string(fn) + (dense ? ": needs an RQ_DENSE session" : ": needs a rotor session (use tq_*)"));
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device)
        return fail(RQ_EINVAL, std::string(fn) + ": current HIP device is not the session's device");
    return RQ_OK;
}

static int check_vectors(const void* p, int dtype, int64_t ld, const char* what, const char* fn) {
    if (dtype != RQ_F16 && dtype != RQ_F32) return fail(RQ_EINVAL, std::string(fn) + ": bad dtype for " + what);
    if (!p) return fail(RQ_EINVAL, std::string(fn) + ": " + what + " is NULL");
    if (!aligned(p, 16)) return fail(RQ_EINVAL, std::string(fn) + ": " + what + " must be 16-byte aligned");
    if (ld < rqh::kDim) return fail(RQ_EINVAL, std::string(fn) + ": leading dimension of " + what + " < 128");
    if ((ld * static_cast<int64_t>(elem_size(dtype))) % 16 != 0)
        return fail(RQ_EINVAL, std::string(fn) + ": row pitch of " + what + " must be a multiple of 16 bytes");
    if (ld * static_cast<int64_t>(elem_size(dtype)) > (int64_t(1) << 26))
        return fail(RQ_EINVAL, std::string(fn) + ": row pitch of " + what + " exceeds 2^26 bytes");
    return RQ_OK;
}

static int check_record(const rq_ctx* ctx, const void* codes, const void* norms, const void* signs,
                        const void* rnorms, const char* fn) {
    const bool has_codes = ctx->host.lay.code_words > 0;
    if ((has_codes && !codes) || !norms) return fail(RQ_EINVAL, std::string(fn) + ": codes and norms are required");
    if ((has_codes && !aligned(codes, 4)) || !aligned(norms, 2))
        return fail(RQ_EINVAL, std::string(fn) + ": misaligned record array");
    const bool qjl = ctx->host.lay.mode & RQ_QJL;
    if (qjl != (signs != nullptr) || qjl != (rnorms != nullptr))
        return fail(RQ_EINVAL, std::string(fn) + ": signs/rnorms must be given exactly for RQ_QJL sessions");
    if (qjl && (!aligned(signs, 4) || !aligned(rnorms, 2)))
        return fail(RQ_EINVAL, std::string(fn) + ": misaligned record array");
    return RQ_OK;
}

static rqk::RotorTables rotor_tables(const rq_ctx* c) {
    rqk::RotorTables t;
    t.rotmat = c->rotmat;
    t.rotmat16 = c->rotmat16;
    t.thr = c->thr;
    t.cent = c->cent;
    t.bins = c->bins;
    t.bin_a = rqh::kBinA;
    t.bin_b = c->host.bin_b;
    t.s_rows = c->s_rows;
    t.s_cols = c->s_cols;
    t.s_fwd = c->s_fwd;
    t.s_back = c->s_back;
    t.phi_hi = c->phi_hi;
    t.phi_lo = c->phi_lo;
    t.qjl_scale = static_cast<float>(std::sqrt(M_PI / 2.0) / rqh::kQjlRows);
    t.mse_bits = c->host.lay.mse_bits;
    t.qjl = c->host.lay.mode & RQ_QJL;
    return t;
}

static rqk::DenseTables dense_tables(const rq_ctx* c) {
    rqk::DenseTables t;
    t.pi_hi = c->pi_hi;
    t.pi_lo = c->pi_lo;
    t.pit_hi = c->pit_hi;
    t.pit_lo = c->pit_lo;
    t.pi2_hi = c->pi2_hi;
    t.pi2_lo = c->pi2_lo;
    t.pit2_hi = c->pit2_hi;
    t.pit2_lo = c->pit2_lo;
    t.t2_hi = c->t2_hi;
    t.t2_lo = c->t2_lo;
    t.s_back = c->s_back;
    t.thr = c->thr;
    t.cent = c->cent;
    t.s_rows = c->s_rows;
    t.s_cols = c->s_cols;
    t.bins = c->bins;
    t.bin_a = rqh::kBinA;
    t.bin_b = c->host.bin_b;
    t.qjl_scale = static_cast<float>(std::sqrt(M_PI / 2.0) / rqh::kQjlRows);
    t.mse_bits = c->host.lay.mse_bits;
    t.qjl = c->host.lay.mode & RQ_QJL;
    return t;
}

static rqk::Qjl1Dev qjl1_tables(const rq_ctx* c) {
    rqk::Qjl1Dev t;
    t.s_fwd = c->s_fwd;
    t.s_back = c->s_back;
    t.qjl_scale = static_cast<float>(std::sqrt(M_PI / 2.0) / rqh::kQjlRows);
    return t;
}

static rqk::ScoreTables score_tables(const rq_ctx* ctx) {
    const bool dense = ctx->host.lay.mode & RQ_DENSE;
    rqk::ScoreTables st;
    st.dense = dense;
    st.rot = dense ? rqk::RotorTables{} : rotor_tables(ctx);
    st.den = dense ? dense_tables(ctx) : rqk::DenseTables{};
    st.mse_bits = ctx->host.lay.mse_bits;
    st.qjl = ctx->host.lay.mode & RQ_QJL;
    st.qjl_scale = static_cast<float>(std::sqrt(M_PI / 2.0) / rqh::kQjlRows);
    return st;
}

static int check_polar(const rq_ctx* ctx, const char* fn) {
    if (!ctx) return fail(RQ_EINVAL, std::string(fn) + ": ctx is NULL");
    if (!(ctx->host.lay.mode & RQ_POLAR)) return fail(RQ_EINVAL, std::string(fn) + ": needs an RQ_POLAR session");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device)
        return fail(RQ_EINVAL, std::string(fn) + ": current HIP device is not the session's device");
    return RQ_OK;
}

static rqk::PolarDev polar_tables(const rq_ctx* c) {
    rqk::PolarDev p;
    p.pi_hi = c->pi_hi;
    p.pi_lo = c->pi_lo;
    p.pit_hi = c->pit_hi;
    p.pit_lo = c->pit_lo;
    p.pi32 = c->pi32;
    p.tab = c->pq_tab;
    p.pi2_hi = c->pi2_hi;
    p.pi2_lo = c->pi2_lo;
    p.pit2_hi = c->pit2_hi;
    p.pit2_lo = c->pit2_lo;
    return p;
}

static int finish(hipError_t e, const char* fn) { return e == hipSuccess ? RQ_OK : hip_fail(e, fn); }

static int quantize_impl(rq_ctx* ctx, bool dense, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* codes,
                         uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, int y_dtype, int64_t ldy,
                         bool roundtrip, void* stream, const char* fn) {
    int rc;
    if ((rc = check_ctx(ctx, dense, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, std::string(fn) + ": n < 0");
    if ((rc = check_vectors(x, x_dtype, ldx, "x", fn))) return rc;
    if ((rc = check_record(ctx, codes, norms, signs, rnorms, fn))) return rc;
    if (roundtrip) {
        if ((rc = check_vectors(y, y_dtype, ldy, "y", fn))) return rc;
        const char* xb = static_cast<const char*>(x);
        const char* yb = static_cast<const char*>(y);
        const int64_t xs = (n > 0 ? (n - 1) * ldx + rqh::kDim : 0) * static_cast<int64_t>(elem_size(x_dtype));
        const int64_t ys = (n > 0 ? (n - 1) * ldy + rqh::kDim : 0) * static_cast<int64_t>(elem_size(y_dtype));
        if (n > 0 && xb < yb + ys && yb < xb + xs) return fail(RQ_EINVAL, std::string(fn) + ": x and y overlap");
    }
    if (n == 0) return RQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t ldx_b = ldx * static_cast<int64_t>(elem_size(x_dtype));
    const int64_t ldy_b = roundtrip ? ldy * static_cast<int64_t>(elem_size(y_dtype)) : 0;
    hipError_t e;
    if (ctx->host.lay.mse_bits == 0)
        e = rqk::qjl1_quantize(qjl1_tables(ctx), x, x_dtype == RQ_F16, ldx_b, n, norms, signs, rnorms, y,
                               y_dtype == RQ_F16, ldy_b, roundtrip, s);
    else if (!dense)
        e = rqk::rotor_quantize(rotor_tables(ctx), x, x_dtype == RQ_F16, ldx_b, n, codes, norms, signs, rnorms, y,
                                y_dtype == RQ_F16, ldy_b, roundtrip, s);
    else
        e = rqk::dense_quantize(dense_tables(ctx), x, x_dtype == RQ_F16, ldx_b, n, codes, norms, signs, rnorms, y,
                                y_dtype == RQ_F16, ldy_b, roundtrip, s);
    return finish(e, fn);
}

static int dequantize_impl(rq_ctx* ctx, bool dense, const uint32_t* codes, const uint16_t* norms,
                           const uint32_t* signs, const uint16_t* rnorms, int64_t n, void* y, int y_dtype,
                           int64_t ldy, void* stream, const char* fn) {
    int rc;
    if ((rc = check_ctx(ctx, dense, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, std::string(fn) + ": n < 0");
    if ((rc = check_record(ctx, codes, norms, signs, rnorms, fn))) return rc;
    if ((rc = check_vectors(y, y_dtype, ldy, "y", fn))) return rc;
    if (n == 0) return RQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t ldy_b = ldy * static_cast<int64_t>(elem_size(y_dtype));
    hipError_t e;
    if (ctx->host.lay.mse_bits == 0)
        e = rqk::qjl1_dequantize(qjl1_tables(ctx), norms, signs, rnorms, n, y, y_dtype == RQ_F16, ldy_b, s);
    else if (!dense)
        e = rqk::rotor_dequantize(rotor_tables(ctx), codes, norms, signs, rnorms, n, y, y_dtype == RQ_F16, ldy_b, s);
    else
        e = rqk::dense_dequantize(dense_tables(ctx), codes, norms, signs, rnorms, n, y, y_dtype == RQ_F16, ldy_b, s);
    return finish(e, fn);
}

int rq_quantize(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* codes, uint16_t* norms,
                uint32_t* signs, uint16_t* rnorms, void* stream) {
    return quantize_impl(ctx, false, x, x_dtype, n, ldx, codes, norms, signs, rnorms, nullptr, RQ_F16, 0, false,
                         stream, "rq_quantize");
}

int rq_dequantize(rq_ctx* ctx, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                  const uint16_t* rnorms, int64_t n, void* y, int y_dtype, int64_t ldy, void* stream) {
    return dequantize_impl(ctx, false, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream, "rq_dequantize");
}

int rq_roundtrip(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* codes, uint16_t* norms,
                 uint32_t* signs, uint16_t* rnorms, void* y, int y_dtype, int64_t ldy, void* stream) {
    return quantize_impl(ctx, false, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, true, stream,
                         "rq_roundtrip");
}

int tq_quantize(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* codes, uint16_t* norms,
                uint32_t* signs, uint16_t* rnorms, void* stream) {
    return quantize_impl(ctx, true, x, x_dtype, n, ldx, codes, norms, signs, rnorms, nullptr, RQ_F16, 0, false,
                         stream, "tq_quantize");
}

int tq_dequantize(rq_ctx* ctx, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                  const uint16_t* rnorms, int64_t n, void* y, int y_dtype, int64_t ldy, void* stream) {
    return dequantize_impl(ctx, true, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream, "tq_dequantize");
}

int tq_roundtrip(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* codes, uint16_t* norms,
                 uint32_t* signs, uint16_t* rnorms, void* y, int y_dtype, int64_t ldy, void* stream) {
    return quantize_impl(ctx, true, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, true, stream,
                         "tq_roundtrip");
}

int rq_score(rq_ctx* ctx, const float* q, int hq, int group, const uint32_t* codes, const uint16_t* norms,
             const uint32_t* signs, const uint16_t* rnorms, int64_t t, int64_t kv_stride, float* scores,
             int64_t ld_scores, void* stream) {
    const char* fn = "rq_score";
    if (!ctx) return fail(RQ_EINVAL, "rq_score: ctx is NULL");
    int rc;
    if ((rc = check_ctx(ctx, ctx->host.lay.mode & RQ_DENSE, fn))) return rc;
    if (!q || !aligned(q, 16)) return fail(RQ_EINVAL, "rq_score: q must be a 16-byte aligned device pointer");
    if (hq < 1 || group < 1 || hq % group) return fail(RQ_EINVAL, "rq_score: need hq >= 1, group >= 1, hq % group == 0");
    if (t < 0) return fail(RQ_EINVAL, "rq_score: t < 0");
    if ((rc = check_record(ctx, codes, norms, signs, rnorms, fn))) return rc;
    const int kv_heads = hq / group;
    if (kv_heads > 1 && kv_stride < t) return fail(RQ_EINVAL, "rq_score: kv_stride < t");
    if (!scores || !aligned(scores, 4)) return fail(RQ_EINVAL, "rq_score: scores must be a 4-byte aligned device pointer");
    if (ld_scores < t) return fail(RQ_EINVAL, "rq_score: ld_scores < t");
    if (ld_scores > (int64_t(1) << 23)) return fail(RQ_EINVAL, "rq_score: ld_scores > 2^23");
    if (group > RQ_SCORE_CHUNK) return fail(RQ_EINVAL, "rq_score: group > RQ_SCORE_CHUNK");
    if (t == 0) return RQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const rqk::ScoreTables st = score_tables(ctx);
    // query rows in chunks that keep whole KV heads together
    const int heads_per_chunk = std::max(1, RQ_SCORE_CHUNK / group);
    for (int h0 = 0; h0 < kv_heads; h0 += heads_per_chunk) {
        const int nh = std::min(heads_per_chunk, kv_heads - h0);
        const hipError_t e = rqk::score(st, q + static_cast<int64_t>(h0) * group * rqh::kDim, nh * group, group,
                                        codes, norms, signs, rnorms, t, kv_stride, h0,
                                        scores + static_cast<int64_t>(h0) * group * ld_scores, ld_scores, s);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return RQ_OK;
}

int64_t rq_attend_workspace(int hq, int group, int64_t t) {
    if (hq < 1 || group < 1 || hq % group || t < 1 || t > RQ_ATTEND_MAX_KEYS) return -1;
    return rqk::attend_plan(hq, group, t).bytes;
}

static int attend_impl(const rq_ctx* kctx, const rq_ctx* vctx, const float* q, int hq, int group,
                       const uint32_t* kcodes, const uint16_t* knorms, const uint32_t* ksigns, const uint16_t* krnorms,
                       const uint32_t* vcodes, const uint16_t* vnorms, const uint32_t* vsigns,
                       const uint16_t* vrnorms, int64_t t, int64_t kv_stride, float scale, void* workspace,
                       int64_t workspace_bytes, float* out, int64_t ld_out, void* stream, bool noalloc) {
    const char* fn = noalloc ? "rq_attend_noalloc" : "rq_attend";
    if (!kctx || !vctx) return fail(RQ_EINVAL, std::string(fn) + ": key and value sessions are required");
    int rc;
    const bool kpolar = kctx->host.lay.mode & RQ_POLAR;
    const bool vpolar = vctx->host.lay.mode & RQ_POLAR;
    if ((rc = kpolar ? check_polar(kctx, fn) : check_ctx(kctx, kctx->host.lay.mode & RQ_DENSE, fn))) return rc;
    if ((rc = vpolar ? check_polar(vctx, fn) : check_ctx(vctx, vctx->host.lay.mode & RQ_DENSE, fn))) return rc;
    if (!q || !aligned(q, 16)) return fail(RQ_EINVAL, std::string(fn) + ": q must be a 16-byte aligned device pointer");
    if (hq < 1 || group < 1 || hq % group) return fail(RQ_EINVAL, std::string(fn) + ": need hq >= 1, group >= 1, hq % group == 0");
    if (hq > RQ_ATTEND_MAX_ROWS) return fail(RQ_EINVAL, std::string(fn) + ": hq > RQ_ATTEND_MAX_ROWS");
    if (group > RQ_SCORE_CHUNK) return fail(RQ_EINVAL, std::string(fn) + ": group > RQ_SCORE_CHUNK");
    if (t < 1) return fail(RQ_EINVAL, std::string(fn) + ": softmax over no keys (t < 1)");
    if (t > RQ_ATTEND_MAX_KEYS) return fail(RQ_EINVAL, std::string(fn) + ": t > RQ_ATTEND_MAX_KEYS");
    if (hq / group > 1 && kv_stride < t) return fail(RQ_EINVAL, std::string(fn) + ": kv_stride < t");
    if (kpolar) {
        if (!kcodes || !aligned(kcodes, 4) || knorms || ksigns || krnorms)
            return fail(RQ_EINVAL, std::string(fn) + ": PolarQuant keys come as 16-word records in kcodes (knorms, ksigns, krnorms NULL)");
    } else if ((rc = check_record(kctx, kcodes, knorms, ksigns, krnorms, fn))) {
        return rc;
    }
    if (vpolar) {
        if (!vcodes || !aligned(vcodes, 4) || vnorms || vsigns || vrnorms)
            return fail(RQ_EINVAL, std::string(fn) + ": PolarQuant values come as 16-word records in vcodes (vnorms, vsigns, vrnorms NULL)");
    } else if ((rc = check_record(vctx, vcodes, vnorms, vsigns, vrnorms, fn))) {
        return rc;
    }
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return fail(RQ_EINVAL, std::string(fn) + ": scale is not finite");
    const rqk::AttendPlan plan = rqk::attend_plan(hq, group, t);
    if (noalloc) {
        if (plan.bytes > rqk::kNoAllocScratchBytes)
            return fail(RQ_EINVAL, "rq_attend_noalloc: rq_attend_workspace(hq, group, t) = " + std::to_string(plan.bytes) +
                                       " bytes exceeds the fixed scratch of RQ_ATTEND_NOALLOC_BYTES = " +
                                       std::to_string(rqk::kNoAllocScratchBytes));
    } else {
        if (!workspace || !aligned(workspace, 256)) return fail(RQ_EINVAL, std::string(fn) + ": workspace must be a 256-byte aligned device pointer");
        if (workspace_bytes < plan.bytes) return fail(RQ_EINVAL, std::string(fn) + ": workspace smaller than rq_attend_workspace()");
    }
    if (!out || !aligned(out, 4)) return fail(RQ_EINVAL, std::string(fn) + ": out must be a 4-byte aligned device pointer");
    if (ld_out < rqh::kDim) return fail(RQ_EINVAL, std::string(fn) + ": ld_out < 128");
    if (!vpolar && vctx->host.lay.mse_bits == 0)
        return fail(RQ_EUNSUPPORTED, std::string(fn) + ": value sessions need at least one MSE bit");
    rqk::ScoreTables kt;
    if (kpolar) {
        kt.dense = false;
        kt.polar = true;
        kt.pol = polar_tables(kctx);
        kt.mse_bits = 0;
        kt.qjl = false;
        kt.qjl_scale = 0.0f;
    } else {
        kt = score_tables(kctx);
    }
    rqk::ScoreTables vt;
    if (vpolar) {
        vt.dense = false;
        vt.polar = true;
        vt.pol = polar_tables(vctx);
        vt.mse_bits = 0;
        vt.qjl = false;
        vt.qjl_scale = 0.0f;
    } else {
        vt = score_tables(vctx);
    }
    if (noalloc) {
        const hipError_t e = rqk::noalloc_scratch(&workspace);
        if (e != hipSuccess) return hip_fail(e, "rq_attend_noalloc: address of the fixed scratch");
    }
    return finish(rqk::attend(kt, vt, q, hq, group, kcodes, knorms, ksigns, krnorms, vcodes, vnorms, vsigns, vrnorms, t,
                              kv_stride, scale, workspace, out, ld_out, static_cast<hipStream_t>(stream)),
                  fn);
}

int rq_attend(const rq_ctx* kctx, const rq_ctx* vctx, const float* q, int hq, int group, const uint32_t* kcodes,
              const uint16_t* knorms, const uint32_t* ksigns, const uint16_t* krnorms, const uint32_t* vcodes,
              const uint16_t* vnorms, const uint32_t* vsigns, const uint16_t* vrnorms, int64_t t, int64_t kv_stride,
              float scale, void* workspace, int64_t workspace_bytes, float* out, int64_t ld_out, void* stream) {
    return attend_impl(kctx, vctx, q, hq, group, kcodes, knorms, ksigns, krnorms, vcodes, vnorms, vsigns, vrnorms, t,
                       kv_stride, scale, workspace, workspace_bytes, out, ld_out, stream, false);
}

int rq_attend_noalloc(const rq_ctx* kctx, const rq_ctx* vctx, const float* q, int hq, int group,
                      const uint32_t* kcodes, const uint16_t* knorms, const uint32_t* ksigns, const uint16_t* krnorms,
                      const uint32_t* vcodes, const uint16_t* vnorms, const uint32_t* vsigns, const uint16_t* vrnorms,
                      int64_t t, int64_t kv_stride, float scale, float* out, int64_t ld_out, void* stream) {
    return attend_impl(kctx, vctx, q, hq, group, kcodes, knorms, ksigns, krnorms, vcodes, vnorms, vsigns, vrnorms, t,
                       kv_stride, scale, nullptr, 0, out, ld_out, stream, true);
}

// ---------------------------------------------- outlier-channel separation --
static int check_outlier_ctx(const rq_ctx* ctx, const char* fn) {
    if (!ctx) return fail(RQ_EINVAL, std::string(fn) + ": ctx is NULL");
    int rc;
    if ((rc = check_ctx(ctx, ctx->host.lay.mode & RQ_DENSE, fn))) return rc;
    if (!(ctx->host.lay.mode & RQ_QJL) || ctx->host.lay.mse_bits != 0)
        return fail(RQ_EINVAL, std::string(fn) + ": needs a QJL-only session (bits = 1 with RQ_QJL)");
    return RQ_OK;
}

static int check_outlier_arrays(int k, const uint8_t* chans, const uint16_t* outliers, const char* fn) {
    if (k < 0 || k > RQ_MAX_OUTLIERS) return fail(RQ_EINVAL, std::string(fn) + ": k outside 0..RQ_MAX_OUTLIERS");
    if (k > 0 && (!chans || !outliers)) return fail(RQ_EINVAL, std::string(fn) + ": chans and outliers are required for k > 0");
    if (outliers && !aligned(outliers, 2)) return fail(RQ_EINVAL, std::string(fn) + ": outliers must be 2-byte aligned");
    return RQ_OK;
}

int rq_outlier_channels(const void* x, int x_dtype, int64_t heads, int64_t head_rows, int64_t ldx, int k,
                        uint8_t* chans, void* stream) {
    const char* fn = "rq_outlier_channels";
    int rc;
    if (heads < 0 || head_rows < 1) return fail(RQ_EINVAL, "rq_outlier_channels: need heads >= 0, head_rows >= 1");
    if (heads > 65535) return fail(RQ_EINVAL, "rq_outlier_channels: heads > 65535");
    if (k < 0 || k > RQ_MAX_OUTLIERS) return fail(RQ_EINVAL, "rq_outlier_channels: k outside 0..RQ_MAX_OUTLIERS");
    if (heads == 0 || k == 0) return RQ_OK;
    if ((rc = check_vectors(x, x_dtype, ldx, "x", fn))) return rc;
    if (!chans) return fail(RQ_EINVAL, "rq_outlier_channels: chans is NULL");
    const hipError_t e = rqk::outlier_select(x, x_dtype == RQ_F16, heads, head_rows,
                                             ldx * static_cast<int64_t>(elem_size(x_dtype)), k, chans,
                                             static_cast<hipStream_t>(stream));
    return finish(e, fn);
}

static rqk::OutlierArgs outlier_args(int64_t n, int64_t head_rows, int k, const uint8_t* chans) {
    rqk::OutlierArgs o;
    o.chans = chans;
    o.heads = k > 0 ? (n + head_rows - 1) / head_rows : 0;
    o.head_rows = head_rows;
    o.k = k;
    return o;
}

int rq_quantize_outliers(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, int64_t head_rows, int k,
                         const uint8_t* chans, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, uint16_t* outliers,
                         void* stream) {
    const char* fn = "rq_quantize_outliers";
    int rc;
    if ((rc = check_outlier_ctx(ctx, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, "rq_quantize_outliers: n < 0");
    if (head_rows < 1) return fail(RQ_EINVAL, "rq_quantize_outliers: head_rows < 1");
    if ((rc = check_vectors(x, x_dtype, ldx, "x", fn))) return rc;
    if ((rc = check_record(ctx, nullptr, norms, signs, rnorms, fn))) return rc;
    if ((rc = check_outlier_arrays(k, chans, outliers, fn))) return rc;
    if (n == 0) return RQ_OK;
    rqk::OutlierArgs o = outlier_args(n, head_rows, k, chans);
    o.out = outliers;
    const hipError_t e = rqk::qjl1_quantize_outliers(qjl1_tables(ctx), x, x_dtype == RQ_F16,
                                                     ldx * static_cast<int64_t>(elem_size(x_dtype)), n, norms, signs,
                                                     rnorms, o, static_cast<hipStream_t>(stream));
    return finish(e, fn);
}

int rq_dequantize_outliers(rq_ctx* ctx, const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms,
                           const uint16_t* outliers, int64_t n, int64_t head_rows, int k, const uint8_t* chans,
                           void* y, int y_dtype, int64_t ldy, void* stream) {
    const char* fn = "rq_dequantize_outliers";
    int rc;
    if ((rc = check_outlier_ctx(ctx, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, "rq_dequantize_outliers: n < 0");
    if (head_rows < 1) return fail(RQ_EINVAL, "rq_dequantize_outliers: head_rows < 1");
    if ((rc = check_record(ctx, nullptr, norms, signs, rnorms, fn))) return rc;
    if ((rc = check_outlier_arrays(k, chans, outliers, fn))) return rc;
    if ((rc = check_vectors(y, y_dtype, ldy, "y", fn))) return rc;
    if (n == 0) return RQ_OK;
    rqk::OutlierArgs o = outlier_args(n, head_rows, k, chans);
    o.in = outliers;
    const hipError_t e = rqk::qjl1_dequantize_outliers(qjl1_tables(ctx), norms, signs, rnorms, n, y, y_dtype == RQ_F16,
                                                       ldy * static_cast<int64_t>(elem_size(y_dtype)), o,
                                                       static_cast<hipStream_t>(stream));
    return finish(e, fn);
}

int rq_score_outliers(rq_ctx* ctx, const float* q, int hq, int group, const uint16_t* norms, const uint32_t* signs,
                      const uint16_t* rnorms, const uint16_t* outliers, int k, const uint8_t* chans, int64_t t,
                      int64_t kv_stride, float* scores, int64_t ld_scores, void* stream) {
    const char* fn = "rq_score_outliers";
    int rc;
    if ((rc = check_outlier_ctx(ctx, fn))) return rc;
    if ((rc = check_outlier_arrays(k, chans, outliers, fn))) return rc;
    if (k == 0) return rq_score(ctx, q, hq, group, nullptr, norms, signs, rnorms, t, kv_stride, scores, ld_scores, stream);
    if (!q || !aligned(q, 16)) return fail(RQ_EINVAL, "rq_score_outliers: q must be a 16-byte aligned device pointer");
    if (hq < 1 || group < 1 || hq % group) return fail(RQ_EINVAL, "rq_score_outliers: need hq >= 1, group >= 1, hq % group == 0");
    if (t < 0) return fail(RQ_EINVAL, "rq_score_outliers: t < 0");
    if ((rc = check_record(ctx, nullptr, norms, signs, rnorms, fn))) return rc;
    const int kv_heads = hq / group;
    if (kv_heads > 1 && kv_stride < t) return fail(RQ_EINVAL, "rq_score_outliers: kv_stride < t");
    if (!scores || !aligned(scores, 4)) return fail(RQ_EINVAL, "rq_score_outliers: scores must be a 4-byte aligned device pointer");
    if (ld_scores < t) return fail(RQ_EINVAL, "rq_score_outliers: ld_scores < t");
    if (ld_scores > (int64_t(1) << 23)) return fail(RQ_EINVAL, "rq_score_outliers: ld_scores > 2^23");
    if (group > RQ_SCORE_CHUNK) return fail(RQ_EINVAL, "rq_score_outliers: group > RQ_SCORE_CHUNK");
    if (t == 0) return RQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const rqk::ScoreTables st = score_tables(ctx);
    rqk::ScoreOutliers so;
    so.chans = chans;
    so.values = outliers;
    so.k = k;
    const int heads_per_chunk = std::max(1, RQ_SCORE_CHUNK / group);
    for (int h0 = 0; h0 < kv_heads; h0 += heads_per_chunk) {
        const int nh = std::min(heads_per_chunk, kv_heads - h0);
        const hipError_t e = rqk::score(st, q + static_cast<int64_t>(h0) * group * rqh::kDim, nh * group, group,
                                        nullptr, norms, signs, rnorms, t, kv_stride, h0,
                                        scores + static_cast<int64_t>(h0) * group * ld_scores, ld_scores, s,
                                        rqk::PageTable{}, so);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return RQ_OK;
}

// ------------------------------------------------------ paged KV cache --
// A pool of fixed-size pages of compressed K and V record rows shared by
// sequences; a sequence reserves its pages when it is opened (so its page
// table is fixed and uploaded once) and returns them when closed.
struct rq_cache {
    struct Pool {
        uint32_t* codes = nullptr;
        uint16_t* norms = nullptr;
        uint32_t* signs = nullptr;
        uint16_t* rnorms = nullptr;
    };
    struct Seq {
        bool open = false;
        int64_t cap = 0, pph = 0;          // tokens per (layer, head); pages per (layer, head)
        std::vector<int64_t> len;          // tokens cached, per layer
        std::vector<int32_t> pages;        // [layer][head][pph]
        int32_t* table = nullptr;          // device copy of `pages`
    };
    const rq_ctx* k = nullptr;
    const rq_ctx* v = nullptr;
    int layers = 0, kv_heads = 0, shift = 0, device = -1;
    int64_t page = 0, max_pages = 0, stage = 0;
    Pool kp, vp, ks, vs;
    std::vector<int32_t> free_pages;
    std::vector<Seq> seqs;
    std::vector<void*> dev;
};

static hipError_t pool_alloc(DevAlloc& da, const rq_ctx* c, int64_t rows, rq_cache::Pool* p) {
    const rqh::Layout& l = c->host.lay;
    hipError_t e;
    if (l.code_words > 0 && (e = da.alloc(reinterpret_cast<void**>(&p->codes), rows * l.code_words * 4)) != hipSuccess)
        return e;
    if ((e = da.alloc(reinterpret_cast<void**>(&p->norms), rows * 2)) != hipSuccess) return e;
    if (l.mode & RQ_QJL) {
        if ((e = da.alloc(reinterpret_cast<void**>(&p->signs), rows * 16)) != hipSuccess) return e;
        if ((e = da.alloc(reinterpret_cast<void**>(&p->rnorms), rows * 2)) != hipSuccess) return e;
    }
    return hipSuccess;
}

static rqk::PageTable page_table(const rq_cache* c, const rq_cache::Seq& q, int layer) {
    rqk::PageTable pt;
    pt.pages = q.table + static_cast<int64_t>(layer) * c->kv_heads * q.pph;
    pt.shift = c->shift;
    pt.stride = q.pph;
    return pt;
}

static int check_seq(const rq_cache* c, int seq, int layer, const char* fn) {
    if (!c) return fail(RQ_EINVAL, std::string(fn) + ": cache is NULL");
    if (seq < 0 || seq >= static_cast<int>(c->seqs.size()) || !c->seqs[seq].open)
        return fail(RQ_EINVAL, std::string(fn) + ": no such open sequence");
    if (layer < 0 || layer >= c->layers) return fail(RQ_EINVAL, std::string(fn) + ": layer out of range");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != c->device)
        return fail(RQ_EINVAL, std::string(fn) + ": current HIP device is not the cache's device");
    return RQ_OK;
}

int rq_cache_create(const rq_ctx* kctx, const rq_ctx* vctx, int layers, int kv_heads, int page_tokens,
                    int64_t max_pages, int64_t stage_tokens, rq_cache** out) {
    const char* fn = "rq_cache_create";
    if (!out) return fail(RQ_EINVAL, "rq_cache_create: out is NULL");
    *out = nullptr;
    if (!kctx || !vctx) return fail(RQ_EINVAL, "rq_cache_create: key and value sessions are required");
    int rc;
    if ((rc = check_ctx(kctx, kctx->host.lay.mode & RQ_DENSE, fn))) return rc;
    if ((rc = check_ctx(vctx, vctx->host.lay.mode & RQ_DENSE, fn))) return rc;
    if (vctx->host.lay.mse_bits == 0) return fail(RQ_EUNSUPPORTED, "rq_cache_create: value sessions need an MSE stage");
    if (layers < 1 || kv_heads < 1) return fail(RQ_EINVAL, "rq_cache_create: layers and kv_heads must be >= 1");
    if (page_tokens < 64 || page_tokens > (1 << 20) || (page_tokens & (page_tokens - 1)))
        return fail(RQ_EINVAL, "rq_cache_create: page_tokens must be a power of two in [64, 2^20]");
    if (max_pages < 1 || max_pages > (int64_t(1) << 31) - 1) return fail(RQ_EINVAL, "rq_cache_create: max_pages out of range");
    if (stage_tokens < 1) return fail(RQ_EINVAL, "rq_cache_create: stage_tokens must be >= 1");
    rq_cache* c = new (std::nothrow) rq_cache;
    if (!c) return fail(RQ_ENOMEM, "rq_cache_create: host allocation failed");
    c->k = kctx;
    c->v = vctx;
    c->layers = layers;
    c->kv_heads = kv_heads;
    c->page = page_tokens;
    while ((int64_t(1) << c->shift) < page_tokens) ++c->shift;
    c->max_pages = max_pages;
    c->stage = stage_tokens;
    c->device = kctx->device;
    DevAlloc da(0);
    const int64_t rows = max_pages * page_tokens, srows = stage_tokens * kv_heads;
    hipError_t e;
    if ((e = pool_alloc(da, kctx, rows, &c->kp)) != hipSuccess || (e = pool_alloc(da, vctx, rows, &c->vp)) != hipSuccess ||
        (e = pool_alloc(da, kctx, srows, &c->ks)) != hipSuccess || (e = pool_alloc(da, vctx, srows, &c->vs)) != hipSuccess) {
        da.release();
        delete c;
        return fail(RQ_ENOMEM, std::string("rq_cache_create: device allocation failed: ") + hipGetErrorString(e));
    }
    c->dev = da.owned;
    c->free_pages.resize(static_cast<size_t>(max_pages));
    for (int64_t i = 0; i < max_pages; ++i) c->free_pages[static_cast<size_t>(i)] = static_cast<int32_t>(max_pages - 1 - i);
    *out = c;
    return RQ_OK;
}

void rq_cache_free(rq_cache* c) {
    if (!c) return;
    (void)hipDeviceSynchronize();
    for (auto& q : c->seqs)
        if (q.table) (void)hipFree(q.table);
    for (void* p : c->dev) (void)hipFree(p);
    delete c;
}

int rq_cache_open(rq_cache* c, int64_t max_tokens, int* seq) {
    if (!c || !seq) return fail(RQ_EINVAL, "rq_cache_open: cache and seq are required");
    if (max_tokens < 1) return fail(RQ_EINVAL, "rq_cache_open: max_tokens must be >= 1");
    const int64_t pph = (max_tokens + c->page - 1) / c->page;
    const int64_t need = pph * c->layers * c->kv_heads;
    if (need > static_cast<int64_t>(c->free_pages.size()))
        return fail(RQ_ENOMEM, "rq_cache_open: not enough free pages in the pool");
    rq_cache::Seq q;
    q.open = true;
    q.cap = pph * c->page;
    q.pph = pph;
    q.len.assign(static_cast<size_t>(c->layers), 0);
    q.pages.resize(static_cast<size_t>(need));
    for (int64_t i = 0; i < need; ++i) {
        q.pages[static_cast<size_t>(i)] = c->free_pages.back();
        c->free_pages.pop_back();
    }
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&q.table), static_cast<size_t>(need) * 4);
    if (e == hipSuccess) e = hipMemcpy(q.table, q.pages.data(), static_cast<size_t>(need) * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        for (int32_t pg : q.pages) c->free_pages.push_back(pg);
        if (q.table) (void)hipFree(q.table);
        return hip_fail(e, "rq_cache_open");
    }
    int id = -1;
    for (size_t i = 0; i < c->seqs.size(); ++i)
        if (!c->seqs[i].open) {
            id = static_cast<int>(i);
            break;
        }
    if (id < 0) {
        id = static_cast<int>(c->seqs.size());
        c->seqs.emplace_back();
    }
    c->seqs[static_cast<size_t>(id)] = std::move(q);
    *seq = id;
    return RQ_OK;
}

int rq_cache_close(rq_cache* c, int seq) {
    int rc;
    if ((rc = check_seq(c, seq, 0, "rq_cache_close"))) return rc;
    rq_cache::Seq& q = c->seqs[static_cast<size_t>(seq)];
    (void)hipDeviceSynchronize();   // no launch may still read the pages or the table
    for (int32_t pg : q.pages) c->free_pages.push_back(pg);
    (void)hipFree(q.table);
    q = rq_cache::Seq{};
    return RQ_OK;
}

int64_t rq_cache_length(const rq_cache* c, int seq, int layer) {
    if (!c || seq < 0 || seq >= static_cast<int>(c->seqs.size()) || !c->seqs[seq].open || layer < 0 || layer >= c->layers)
        return -1;
    return c->seqs[static_cast<size_t>(seq)].len[static_cast<size_t>(layer)];
}

int64_t rq_cache_free_pages(const rq_cache* c) { return c ? static_cast<int64_t>(c->free_pages.size()) : -1; }

// Quantises n new rows of each of `heads` (layer, KV head) blocks of x
// ([heads][n][ld]) and scatters them to key positions t0.. of those blocks'
// pages; block j's page list starts at pt.pages + j * pt.stride (the page
// tables of consecutive layers follow each other).
static int cache_quantize_into_pages(rq_cache* c, const rq_ctx* ctx, const rq_cache::Pool& stage,
                                     const rq_cache::Pool& pool, const rqk::PageTable& pt, const void* x, int dtype,
                                     int64_t n, int64_t ld, int64_t t0, hipStream_t s, const char* fn, int heads = 0) {
    if (heads <= 0) heads = c->kv_heads;
    const rqh::Layout& l = ctx->host.lay;
    const bool dense = l.mode & RQ_DENSE;
    const bool qjl = l.mode & RQ_QJL;
    const char* xb = static_cast<const char*>(x);
    const int64_t es = static_cast<int64_t>(elem_size(dtype));
    int rc;
    if (n * heads <= c->stage * c->kv_heads) {
        // every block's n rows in one launch: rows j * n + i, pitch ld
        if ((rc = quantize_impl(const_cast<rq_ctx*>(ctx), dense, x, dtype, n * heads, ld, stage.codes, stage.norms,
                                stage.signs, stage.rnorms, nullptr, RQ_F32, 0, false, s, fn)))
            return rc;
        return finish(rqk::scatter_rows(stage.codes, stage.norms, stage.signs, stage.rnorms, pool.codes, pool.norms,
                                        pool.signs, pool.rnorms, l.code_words, qjl, n, t0, heads, pt, false, s),
                      fn);
    }
    for (int j = 0; j < heads; ++j) {
        rqk::PageTable hp = pt;
        hp.pages = pt.pages + static_cast<int64_t>(j) * pt.stride;
        for (int64_t c0 = 0; c0 < n; c0 += c->stage) {
            const int64_t m = std::min(c->stage, n - c0);
            if ((rc = quantize_impl(const_cast<rq_ctx*>(ctx), dense, xb + (j * n + c0) * ld * es, dtype, m, ld, stage.codes,
                                    stage.norms, stage.signs, stage.rnorms, nullptr, RQ_F32, 0, false, s, fn)))
                return rc;
            const hipError_t e = rqk::scatter_rows(stage.codes, stage.norms, stage.signs, stage.rnorms, pool.codes,
                                                   pool.norms, pool.signs, pool.rnorms, l.code_words, qjl, m, t0 + c0, 1,
                                                   hp, false, s);
            if (e != hipSuccess) return hip_fail(e, fn);
        }
    }
    return RQ_OK;
}

int rq_cache_append(rq_cache* c, int seq, int layer, const void* k, const void* v, int dtype, int64_t n, int64_t ld,
                    void* stream) {
    const char* fn = "rq_cache_append";
    int rc;
    if ((rc = check_seq(c, seq, layer, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, "rq_cache_append: n < 0");
    if ((rc = check_vectors(k, dtype, ld, "k", fn))) return rc;
    if ((rc = check_vectors(v, dtype, ld, "v", fn))) return rc;
    rq_cache::Seq& q = c->seqs[static_cast<size_t>(seq)];
    int64_t& len = q.len[static_cast<size_t>(layer)];
    if (len + n > q.cap) return fail(RQ_EINVAL, "rq_cache_append: the sequence's reserved tokens are exhausted");
    if (n == 0) return RQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const rqk::PageTable pt = page_table(c, q, layer);
    if ((rc = cache_quantize_into_pages(c, c->k, c->ks, c->kp, pt, k, dtype, n, ld, len, s, fn))) return rc;
    if ((rc = cache_quantize_into_pages(c, c->v, c->vs, c->vp, pt, v, dtype, n, ld, len, s, fn))) return rc;
    len += n;
    return RQ_OK;
}

int rq_cache_read(const rq_cache* c, int seq, int layer, int which, uint32_t* codes, uint16_t* norms, uint32_t* signs,
                  uint16_t* rnorms, void* stream) {
    const char* fn = "rq_cache_read";
    int rc;
    if ((rc = check_seq(c, seq, layer, fn))) return rc;
    if (which != 0 && which != 1) return fail(RQ_EINVAL, "rq_cache_read: which must be 0 (keys) or 1 (values)");
    const rq_ctx* ctx = which ? c->v : c->k;
    if ((rc = check_record(ctx, codes, norms, signs, rnorms, fn))) return rc;
    const rq_cache::Seq& q = c->seqs[static_cast<size_t>(seq)];
    const int64_t n = q.len[static_cast<size_t>(layer)];
    const rq_cache::Pool& pool = which ? c->vp : c->kp;
    const rqh::Layout& l = ctx->host.lay;
    return finish(rqk::scatter_rows(pool.codes, pool.norms, pool.signs, pool.rnorms, codes, norms, signs, rnorms,
                                    l.code_words, l.mode & RQ_QJL, n, 0, c->kv_heads, page_table(c, q, layer), true,
                                    static_cast<hipStream_t>(stream)),
                  fn);
}

int64_t rq_cache_attend_workspace(const rq_cache* c, int hq, int64_t t) {
    if (!c || hq < 1 || hq % c->kv_heads || t < 0 || t > RQ_ATTEND_MAX_KEYS) return -1;
    return t == 0 ? 0 : rqk::attend_plan(hq, hq / c->kv_heads, t).bytes;
}

int rq_cache_attend(rq_cache* c, int seq, int layer, const float* q, int hq, float scale, const float* k_cur,
                    const float* v_cur, void* workspace, int64_t workspace_bytes, float* out, int64_t ld_out,
                    void* stream) {
    const char* fn = "rq_cache_attend";
    int rc;
    if ((rc = check_seq(c, seq, layer, fn))) return rc;
    if (!q || !aligned(q, 16)) return fail(RQ_EINVAL, "rq_cache_attend: q must be a 16-byte aligned device pointer");
    if (hq < 1 || hq % c->kv_heads || hq > RQ_ATTEND_MAX_ROWS)
        return fail(RQ_EINVAL, "rq_cache_attend: hq must be a positive multiple of kv_heads, <= RQ_ATTEND_MAX_ROWS");
    if ((k_cur == nullptr) != (v_cur == nullptr)) return fail(RQ_EINVAL, "rq_cache_attend: give both or neither of k_cur, v_cur");
    if (k_cur && (!aligned(k_cur, 4) || !aligned(v_cur, 4))) return fail(RQ_EINVAL, "rq_cache_attend: misaligned k_cur / v_cur");
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return fail(RQ_EINVAL, "rq_cache_attend: scale is not finite");
    if (!out || !aligned(out, 4) || ld_out < rqh::kDim) return fail(RQ_EINVAL, "rq_cache_attend: bad out / ld_out");
    const rq_cache::Seq& sq = c->seqs[static_cast<size_t>(seq)];
    const int64_t t = sq.len[static_cast<size_t>(layer)];
    const int group = hq / c->kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (t == 0) {
        if (!k_cur) return fail(RQ_EINVAL, "rq_cache_attend: no cached tokens and no current token");
        return finish(rqk::merge_current(q, hq, group, k_cur, v_cur, nullptr, scale, out, ld_out, s), fn);
    }
    const rqk::AttendPlan plan = rqk::attend_plan(hq, group, t);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < plan.bytes)
        return fail(RQ_EINVAL, "rq_cache_attend: workspace missing, misaligned or smaller than rq_cache_attend_workspace()");
    const rqk::PageTable pt = page_table(c, sq, layer);
    const rqk::ScoreTables kt = score_tables(c->k), vt = score_tables(c->v);
    hipError_t e = rqk::attend(kt, vt, q, hq, group, c->kp.codes, c->kp.norms, c->kp.signs, c->kp.rnorms, c->vp.codes,
                               c->vp.norms, c->vp.signs, c->vp.rnorms, t, 0, scale, workspace, out, ld_out, s, pt, pt);
    if (e == hipSuccess && k_cur)
        e = rqk::merge_current(q, hq, group, k_cur, v_cur,
                               reinterpret_cast<const float2*>(static_cast<char*>(workspace) + plan.off_stats), scale,
                               out, ld_out, s);
    return finish(e, fn);
}

// ------------------------------------------- all layers of a decode step --
static int check_layers(const rq_cache* c, int seq, int layer0, int nlayers, int64_t* len, const char* fn) {
    int rc;
    if ((rc = check_seq(c, seq, 0, fn))) return rc;
    if (nlayers < 1 || layer0 < 0 || layer0 + nlayers > c->layers)
        return fail(RQ_EINVAL, std::string(fn) + ": layers [layer0, layer0 + nlayers) out of range");
    const rq_cache::Seq& q = c->seqs[static_cast<size_t>(seq)];
    const int64_t t = q.len[static_cast<size_t>(layer0)];
    for (int l = layer0 + 1; l < layer0 + nlayers; ++l)
        if (q.len[static_cast<size_t>(l)] != t)
            return fail(RQ_EINVAL, std::string(fn) + ": the layers hold different numbers of cached tokens");
    *len = t;
    return RQ_OK;
}

int rq_cache_append_layers(rq_cache* c, int seq, int layer0, int nlayers, const void* k, const void* v, int dtype,
                           int64_t n, int64_t ld, void* stream) {
    const char* fn = "rq_cache_append_layers";
    int rc;
    int64_t t0 = 0;
    if ((rc = check_layers(c, seq, layer0, nlayers, &t0, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, "rq_cache_append_layers: n < 0");
    if ((rc = check_vectors(k, dtype, ld, "k", fn))) return rc;
    if ((rc = check_vectors(v, dtype, ld, "v", fn))) return rc;
    rq_cache::Seq& q = c->seqs[static_cast<size_t>(seq)];
    if (t0 + n > q.cap) return fail(RQ_EINVAL, "rq_cache_append_layers: the sequence's reserved tokens are exhausted");
    if (n == 0) return RQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const rqk::PageTable pt = page_table(c, q, layer0);
    const int heads = nlayers * c->kv_heads;
    if ((rc = cache_quantize_into_pages(c, c->k, c->ks, c->kp, pt, k, dtype, n, ld, t0, s, fn, heads))) return rc;
    if ((rc = cache_quantize_into_pages(c, c->v, c->vs, c->vp, pt, v, dtype, n, ld, t0, s, fn, heads))) return rc;
    for (int l = layer0; l < layer0 + nlayers; ++l) q.len[static_cast<size_t>(l)] += n;
    return RQ_OK;
}

int64_t rq_cache_attend_layers_workspace(const rq_cache* c, int nlayers, int hq, int64_t t) {
    if (!c || nlayers < 1 || hq < 1 || hq % c->kv_heads || t < 0 || t > RQ_ATTEND_MAX_KEYS) return -1;
    if (static_cast<int64_t>(nlayers) * hq > RQ_ATTEND_MAX_ROWS) return -1;
    return t == 0 ? 0 : rqk::attend_plan(nlayers * hq, hq / c->kv_heads, t, hq).bytes;
}

int rq_cache_attend_layers(rq_cache* c, int seq, int layer0, int nlayers, const float* q, int hq, float scale,
                           const float* k_cur, const float* v_cur, void* workspace, int64_t workspace_bytes,
                           float* out, int64_t ld_out, void* stream) {
    const char* fn = "rq_cache_attend_layers";
    int rc;
    int64_t t = 0;
    if ((rc = check_layers(c, seq, layer0, nlayers, &t, fn))) return rc;
    if (!q || !aligned(q, 16)) return fail(RQ_EINVAL, "rq_cache_attend_layers: q must be a 16-byte aligned device pointer");
    if (hq < 1 || hq % c->kv_heads || static_cast<int64_t>(nlayers) * hq > RQ_ATTEND_MAX_ROWS)
        return fail(RQ_EINVAL, "rq_cache_attend_layers: hq must be a positive multiple of kv_heads and nlayers * hq <= RQ_ATTEND_MAX_ROWS");
    if ((k_cur == nullptr) != (v_cur == nullptr)) return fail(RQ_EINVAL, "rq_cache_attend_layers: give both or neither of k_cur, v_cur");
    if (k_cur && (!aligned(k_cur, 4) || !aligned(v_cur, 4))) return fail(RQ_EINVAL, "rq_cache_attend_layers: misaligned k_cur / v_cur");
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return fail(RQ_EINVAL, "rq_cache_attend_layers: scale is not finite");
    if (!out || !aligned(out, 4) || ld_out < rqh::kDim) return fail(RQ_EINVAL, "rq_cache_attend_layers: bad out / ld_out");
    const rq_cache::Seq& sq = c->seqs[static_cast<size_t>(seq)];
    const int group = hq / c->kv_heads;
    const int rows = nlayers * hq;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (t == 0) {
        if (!k_cur) return fail(RQ_EINVAL, "rq_cache_attend_layers: no cached tokens and no current token");
        return finish(rqk::merge_current(q, rows, group, k_cur, v_cur, nullptr, scale, out, ld_out, s), fn);
    }
    const rqk::AttendPlan plan = rqk::attend_plan(rows, group, t, hq);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < plan.bytes)
        return fail(RQ_EINVAL, "rq_cache_attend_layers: workspace missing, misaligned or smaller than rq_cache_attend_layers_workspace()");
    // the layers' page tables follow each other: query row l * hq + h reads
    // KV head l * kv_heads + h / group, whose pages start at that head's row
    const rqk::PageTable pt = page_table(c, sq, layer0);
    const rqk::ScoreTables kt = score_tables(c->k), vt = score_tables(c->v);
    hipError_t e = rqk::attend(kt, vt, q, rows, group, c->kp.codes, c->kp.norms, c->kp.signs, c->kp.rnorms, c->vp.codes,
                               c->vp.norms, c->vp.signs, c->vp.rnorms, t, 0, scale, workspace, out, ld_out, s, pt, pt,
                               hq);
    if (e == hipSuccess && k_cur)
        e = rqk::merge_current(q, rows, group, k_cur, v_cur,
                               reinterpret_cast<const float2*>(static_cast<char*>(workspace) + plan.off_stats), scale,
                               out, ld_out, s);
    return finish(e, fn);
}

// ---------------------------------------------------------- PolarQuant --
static int pq_quantize_impl(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* words,
                            void* y, int y_dtype, int64_t ldy, bool roundtrip, void* stream, const char* fn) {
    int rc;
    if ((rc = check_polar(ctx, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, std::string(fn) + ": n < 0");
    if ((rc = check_vectors(x, x_dtype, ldx, "x", fn))) return rc;
    if (!words || !aligned(words, 4)) return fail(RQ_EINVAL, std::string(fn) + ": words must be a 4-byte aligned device pointer");
    if (roundtrip) {
        if ((rc = check_vectors(y, y_dtype, ldy, "y", fn))) return rc;
        const char* xb = static_cast<const char*>(x);
        const char* yb = static_cast<const char*>(y);
        const int64_t xs = (n > 0 ? (n - 1) * ldx + rqh::kDim : 0) * static_cast<int64_t>(elem_size(x_dtype));
        const int64_t ys = (n > 0 ? (n - 1) * ldy + rqh::kDim : 0) * static_cast<int64_t>(elem_size(y_dtype));
        if (n > 0 && xb < yb + ys && yb < xb + xs) return fail(RQ_EINVAL, std::string(fn) + ": x and y overlap");
    }
    if (n == 0) return RQ_OK;
    const int64_t ldx_b = ldx * static_cast<int64_t>(elem_size(x_dtype));
    const int64_t ldy_b = roundtrip ? ldy * static_cast<int64_t>(elem_size(y_dtype)) : 0;
    return finish(rqk::polar_quantize(polar_tables(ctx), x, x_dtype == RQ_F16, ldx_b, n, words, y, y_dtype == RQ_F16,
                                      ldy_b, roundtrip, static_cast<hipStream_t>(stream)),
                  fn);
}

int pq_quantize(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* words, void* stream) {
    return pq_quantize_impl(ctx, x, x_dtype, n, ldx, words, nullptr, RQ_F16, 0, false, stream, "pq_quantize");
}

int pq_roundtrip(rq_ctx* ctx, const void* x, int x_dtype, int64_t n, int64_t ldx, uint32_t* words, void* y,
                 int y_dtype, int64_t ldy, void* stream) {
    return pq_quantize_impl(ctx, x, x_dtype, n, ldx, words, y, y_dtype, ldy, true, stream, "pq_roundtrip");
}

int pq_dequantize(rq_ctx* ctx, const uint32_t* words, int64_t n, void* y, int y_dtype, int64_t ldy, void* stream) {
    const char* fn = "pq_dequantize";
    int rc;
    if ((rc = check_polar(ctx, fn))) return rc;
    if (n < 0) return fail(RQ_EINVAL, "pq_dequantize: n < 0");
    if (!words || !aligned(words, 4)) return fail(RQ_EINVAL, "pq_dequantize: words must be a 4-byte aligned device pointer");
    if ((rc = check_vectors(y, y_dtype, ldy, "y", fn))) return rc;
    if (n == 0) return RQ_OK;
    return finish(rqk::polar_dequantize(polar_tables(ctx), words, n, y, y_dtype == RQ_F16,
                                        ldy * static_cast<int64_t>(elem_size(y_dtype)), static_cast<hipStream_t>(stream)),
                  fn);
}

int pq_score(rq_ctx* ctx, const float* q, int hq, int group, const uint32_t* words, int64_t t, int64_t kv_stride,
             float* scores, int64_t ld_scores, void* stream) {
    const char* fn = "pq_score";
    int rc;
    if ((rc = check_polar(ctx, fn))) return rc;
    if (!q || !aligned(q, 16)) return fail(RQ_EINVAL, "pq_score: q must be a 16-byte aligned device pointer");
    if (hq < 1 || group < 1 || hq % group) return fail(RQ_EINVAL, "pq_score: need hq >= 1, group >= 1, hq % group == 0");
    if (hq > RQ_ATTEND_MAX_ROWS) return fail(RQ_EINVAL, "pq_score: hq > 65535");
    if (t < 0) return fail(RQ_EINVAL, "pq_score: t < 0");
    if (!words || !aligned(words, 4)) return fail(RQ_EINVAL, "pq_score: words must be a 4-byte aligned device pointer");
    if (hq / group > 1 && kv_stride < t) return fail(RQ_EINVAL, "pq_score: kv_stride < t");
    if (!scores || !aligned(scores, 4)) return fail(RQ_EINVAL, "pq_score: scores must be a 4-byte aligned device pointer");
    if (ld_scores < t) return fail(RQ_EINVAL, "pq_score: ld_scores < t");
    if (ld_scores > (int64_t(1) << 23)) return fail(RQ_EINVAL, "pq_score: ld_scores > 2^23");
    if (t == 0) return RQ_OK;
    return finish(rqk::polar_score(polar_tables(ctx), q, hq, group, words, t, hq / group > 1 ? kv_stride : 0, scores,
                                   ld_scores, static_cast<hipStream_t>(stream)),
                  fn);
}

}  // extern "C"


