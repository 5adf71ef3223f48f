// Host core: parameter tables of a codec session and record layout.
//
// Everything here is float64 and is rounded once to the stored precision.
// Build without -ffast-math and with -ffp-contract=off: the normals must be
// the exact libm values of the published Box-Muller formula.
#include "rq_host.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <utility>

namespace rqh {

namespace {

constexpr uint64_t kGoldenGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kStreamMul = 0xD1B54A32D192ED03ull;
constexpr uint64_t kTagRotors = 1, kTagPi = 2, kTagS = 3;
constexpr double kPi = 3.141592653589793;
constexpr double kTwoPi = 2.0 * kPi;

float to_f32(double x) { return static_cast<float>(x); }

}  // namespace

// ----------------------------------------------------------------- layout --
int make_layout(int d, int bits, int mode, Layout* out, std::string* err) {
    if (mode & ~(kModeQjl | kModeDense | kModePolar)) {
        if (err) *err = "unknown mode bits";
        return 1;
    }
    if (mode & kModePolar) {
        if (mode != kModePolar) {
            if (err) *err = "RQ_POLAR takes no other mode bits";
            return 1;
        }
        if (bits != kPolarBits[0]) {
            if (err) *err = "RQ_POLAR sessions have bits = 4 (4-bit first level, 2-bit later levels)";
            return 1;
        }
        if (d <= 0) {
            if (err) *err = "d must be positive";
            return 1;
        }
        if (d != kDim) {
            if (err) *err = "only d = 128 is implemented";
            return 2;
        }
        Layout l;
        l.d = d;
        l.bits = bits;
        l.mse_bits = bits;
        l.mode = mode;
        l.n_coords = d;
        l.n_groups = 0;
        l.levels = 1 << bits;
        l.code_words = kPolarWords;
        l.sign_words = 0;
        l.record_bytes = 4 * kPolarWords;
        *out = l;
        return 0;
    }
    const bool qjl = mode & kModeQjl;
    const int mse_bits = qjl ? bits - 1 : bits;
    if (mse_bits < (qjl ? 0 : 1) || mse_bits > kMaxMseBits) {
        if (err) *err = qjl ? "bits must be 1..5 with RQ_QJL" : "bits must be 1..4";
        return 1;
    }
    if (d <= 0) {
        if (err) *err = "d must be positive";
        return 1;
    }
    if (d != kDim) {
        if (err) *err = "only d = 128 is implemented";
        return 2;
    }
    Layout l;
    l.d = d;
    l.bits = bits;
    l.mse_bits = mse_bits;
    l.mode = mode;
    l.n_groups = (mode & kModeDense) ? 0 : (d + 2) / 3;
    l.n_coords = (mode & kModeDense) ? d : 3 * l.n_groups;
    l.levels = 1 << mse_bits;
    l.code_words = (l.n_coords * mse_bits + 31) / 32;
    l.sign_words = qjl ? kQjlRows / 32 : 0;
    l.record_bytes = 4 * l.code_words + 2 + (qjl ? 4 * l.sign_words + 2 : 0);
    *out = l;
    return 0;
}

// ------------------------------------------------------------ SplitMix64 --
// Steele, Lea and Flood (2014): advance by the golden gamma, then mix.
uint64_t splitmix64_next(uint64_t* state) {
    *state += kGoldenGamma;
    uint64_t z = *state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double next_uniform(uint64_t* state) {
    const uint64_t w = splitmix64_next(state);
    return (static_cast<double>(w >> 11) + 0.5) * 0x1p-53;
}

// Box-Muller: two uniforms give sqrt(-2 ln u1) cos(2 pi u2), then the sine.
std::vector<double> normals(uint64_t seed, uint64_t tag, size_t count) {
    uint64_t state = seed ^ (tag * kStreamMul);
    std::vector<double> out;
    out.reserve(count + 1);
    while (out.size() < count) {
        const double u1 = next_uniform(&state);
        const double u2 = next_uniform(&state);
        const double rad = std::sqrt(-2.0 * std::log(u1));
        const double ang = kTwoPi * u2;
        out.push_back(rad * std::cos(ang));
        out.push_back(rad * std::sin(ang));
    }
    out.resize(count);
    return out;
}

// ------------------------------------------------------------------ rotors --
// Rotor R = s + b12 e12 + b13 e13 + b23 e23 acting on v = v1 e1 + v2 e2 + v3 e3.
// The left product R v has grade-1 part t and trivector part t123; the right
// product with R~ = s - b12 e12 - b13 e13 - b23 e23 keeps grade 1.  These are
// the sparse products written out from e_i e_i = 1, e_i e_j = -e_j e_i.
static void sandwich3(const double r[4], const double v[3], double y[3]) {
    const double s = r[0], b12 = r[1], b13 = r[2], b23 = r[3];
    const double t1 = s * v[0] + b12 * v[1] + b13 * v[2];
    const double t2 = s * v[1] - b12 * v[0] + b23 * v[2];
    const double t3 = s * v[2] - b13 * v[0] - b23 * v[1];
    const double t123 = b12 * v[2] - b13 * v[1] + b23 * v[0];
    y[0] = s * t1 + b12 * t2 + b13 * t3 + b23 * t123;
    y[1] = -b12 * t1 + s * t2 + b23 * t3 - b13 * t123;
    y[2] = -b13 * t1 - b23 * t2 + s * t3 + b12 * t123;
}

float rotor_matrix_entry_check(const float rf[4], double m[9]) {
    const double r[4] = {rf[0], rf[1], rf[2], rf[3]};
    for (int j = 0; j < 3; ++j) {
        double e[3] = {0.0, 0.0, 0.0}, y[3];
        e[j] = 1.0;
        sandwich3(r, e, y);
        for (int i = 0; i < 3; ++i) m[3 * i + j] = y[i];
    }
    return static_cast<float>(m[0] * (m[4] * m[8] - m[5] * m[7]) - m[1] * (m[3] * m[8] - m[5] * m[6]) +
                              m[2] * (m[3] * m[7] - m[4] * m[6]));
}

static void make_rotors(int d, uint64_t seed, std::vector<float>* rotors, std::vector<float>* mats) {
    const int g = (d + 2) / 3;
    const std::vector<double> z = normals(seed, kTagRotors, 3 * static_cast<size_t>(g));
    rotors->assign(4 * g, 0.0f);
    mats->assign(9 * g, 0.0f);
    for (int i = 0; i < g; ++i) {
        const double b12 = z[3 * i], b13 = z[3 * i + 1], b23 = z[3 * i + 2];
        // exp(B) = cos|b| + sin|b|/|b| B, then divide by sqrt(<R R~>_0)
        const double th = std::sqrt(b12 * b12 + b13 * b13 + b23 * b23);
        const double k = th > 0.0 ? std::sin(th) / th : 1.0;
        double r[4] = {std::cos(th), k * b12, k * b13, k * b23};
        const double n2 = r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
        const double inv = std::sqrt(n2);
        float rf[4];
        for (int c = 0; c < 4; ++c) {
            rf[c] = to_f32(r[c] / inv);
            (*rotors)[4 * i + c] = rf[c];
        }
        double m[9];
        rotor_matrix_entry_check(rf, m);
        for (int c = 0; c < 9; ++c) (*mats)[9 * i + c] = to_f32(m[c]);
    }
}

// ----------------------------------------------------------------- Lloyd-Max --
// Coordinate law of a uniform unit vector in R^d:
//   f(x) = C (1 - x^2)^k on [-1, 1],  k = (d - 3)/2,
//   C = Gamma(d/2) / (sqrt(pi) Gamma((d - 1)/2)).
// Cell mass by composite Gauss-Legendre; first moment in closed form:
//   int_a^b x (1-x^2)^k dx = ((1-a^2)^(k+1) - (1-b^2)^(k+1)) / (2 (k+1)).
namespace {

struct GaussLegendre {
    std::vector<double> x, w;
    explicit GaussLegendre(int n) : x(n), w(n) {
        // Newton iteration on P_n from the Chebyshev-like first guess; the
        // weight is 2 / ((1 - z^2) P_n'(z)^2) at the converged node.
        auto legendre = [n](double z, double* dp) {
            double p0 = 1.0, p1 = z;
            for (int k = 2; k <= n; ++k) {
                const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                p0 = p1;
                p1 = p2;
            }
            *dp = n * (z * p1 - p0) / (z * z - 1.0);
            return p1;
        };
        for (int i = 0; i < n; ++i) {
            double z = std::cos(kPi * (i + 0.75) / (n + 0.5));
            for (int it = 0; it < 100; ++it) {
                double dp;
                const double dz = legendre(z, &dp) / dp;
                z -= dz;
                if (std::fabs(dz) <= 1e-15) break;
            }
            double dp;
            legendre(z, &dp);
            x[i] = z;
            w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
        }
    }
};

struct SphereLaw {
    int d;
    double k, logc;
    GaussLegendre gl{24};
    explicit SphereLaw(int dim) : d(dim), k((dim - 3) / 2.0) {
        logc = std::lgamma(dim / 2.0) - 0.5 * std::log(kPi) - std::lgamma((dim - 1) / 2.0);
    }
    double mass(double a, double b) const {
        if (b <= a) return 0.0;
        const int panels = std::max(1, static_cast<int>(std::ceil((b - a) / 0.005)));
        const double h = (b - a) / panels;
        double sum = 0.0;
        for (int p = 0; p < panels; ++p) {
            const double mid = a + (p + 0.5) * h;
            double ps = 0.0;
            for (size_t i = 0; i < gl.x.size(); ++i) {
                const double x = mid + 0.5 * h * gl.x[i];
                const double u = 1.0 - x * x;
                ps += gl.w[i] * (u > 0.0 ? std::pow(u, k) : 0.0);
            }
            sum += 0.5 * h * ps;
        }
        return std::exp(logc) * sum;
    }
    double first_moment(double a, double b) const {
        const double kp1 = k + 1.0;
        const double ua = std::max(0.0, 1.0 - a * a), ub = std::max(0.0, 1.0 - b * b);
        return std::exp(logc) * (std::pow(ua, kp1) - std::pow(ub, kp1)) / (2.0 * kp1);
    }
};

}  // namespace

void lloyd_max_unit_sphere(int d, int bits, std::vector<double>* centroids, std::vector<double>* boundaries) {
    static std::mutex mu;
    static std::map<std::pair<int, int>, std::pair<std::vector<double>, std::vector<double>>> cache;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find({d, bits});
        if (it != cache.end()) {
            *centroids = it->second.first;
            *boundaries = it->second.second;
            return;
        }
    }
    const int levels = 1 << bits;
    const SphereLaw law(d);
    const double sigma = 1.0 / std::sqrt(static_cast<double>(d));
    std::vector<double> c(levels), t(levels - 1), nc(levels);
    for (int i = 0; i < levels; ++i) c[i] = sigma * (-2.0 + 4.0 * (i + 0.5) / levels);
    for (int iter = 0; iter < 200000; ++iter) {
        for (int i = 0; i + 1 < levels; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
        for (int i = 0; i < levels; ++i) {
            const double lo = i == 0 ? -1.0 : t[i - 1];
            const double hi = i == levels - 1 ? 1.0 : t[i];
            nc[i] = law.first_moment(lo, hi) / law.mass(lo, hi);
        }
        // the density is symmetric: keep the iterate exactly antisymmetric
        double delta = 0.0;
        std::vector<double> sym(levels);
        for (int i = 0; i < levels; ++i) {
            sym[i] = 0.5 * (nc[i] - nc[levels - 1 - i]);
            delta = std::max(delta, std::fabs(sym[i] - c[i]));
        }
        c.swap(sym);
        if (delta < 1e-15) break;
    }
    for (int i = 0; i + 1 < levels; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
    *centroids = c;
    *boundaries = t;
    std::lock_guard<std::mutex> lock(mu);
    cache[{d, bits}] = {c, t};
}

// ------------------------------------------------------- PolarQuant angles --
// Cell masses and first moments of the angle density by composite
// Gauss-Legendre (panels of at most 0.005 rad, 24 nodes: the integrands are
// smooth, so every integral is exact to rounding).
namespace {

struct AngleLaw {
    int level;
    double lo, hi, logc;
    int power;   // k - 1
    GaussLegendre gl{24};
    explicit AngleLaw(int l) : level(l) {
        lo = 0.0;
        hi = l == 0 ? kTwoPi : 0.5 * kPi;
        const double k = std::ldexp(1.0, l);
        power = static_cast<int>(k) - 1;
        logc = l == 0 ? -std::log(kTwoPi)
                      : std::lgamma(k) - (k - 2.0) * std::log(2.0) - 2.0 * std::lgamma(0.5 * k);
    }
    double density(double th) const {
        if (level == 0) return std::exp(logc);
        const double s = std::sin(2.0 * th);
        return std::exp(logc) * std::pow(s, power);
    }
    double moment(double a, double b, int p) const {
        if (b <= a) return 0.0;
        const int panels = std::max(1, static_cast<int>(std::ceil((b - a) / 0.005)));
        const double h = (b - a) / panels;
        double sum = 0.0;
        for (int q = 0; q < panels; ++q) {
            const double mid = a + (q + 0.5) * h;
            double ps = 0.0;
            for (size_t i = 0; i < gl.x.size(); ++i) {
                const double th = mid + 0.5 * h * gl.x[i];
                ps += gl.w[i] * (p ? th : 1.0) * density(th);
            }
            sum += 0.5 * h * ps;
        }
        return sum;
    }
};

}  // namespace

// Lloyd's algorithm from a uniform start: boundaries at the midpoints of the
// centroids, each centroid moved to the conditional mean of its cell, until
// no centroid moves by 1e-14 (the iterate of that last step is kept).
void lloyd_polar(int level, std::vector<double>* centroids, std::vector<double>* boundaries) {
    static std::mutex mu;
    static std::map<int, std::pair<std::vector<double>, std::vector<double>>> cache;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(level);
        if (it != cache.end()) {
            *centroids = it->second.first;
            *boundaries = it->second.second;
            return;
        }
    }
    const AngleLaw law(level);
    const int levels = 1 << kPolarBits[level];
    std::vector<double> c(levels), t(levels + 1), nc(levels);
    for (int i = 0; i < levels; ++i) c[i] = law.lo + (i + 0.5) * (law.hi - law.lo) / levels;
    for (int iter = 0; iter < 10000; ++iter) {
        t[0] = law.lo;
        t[levels] = law.hi;
        for (int i = 1; i < levels; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
        double delta = 0.0;
        for (int i = 0; i < levels; ++i) {
            const double mass = law.moment(t[i], t[i + 1], 0);
            nc[i] = mass > 0.0 ? law.moment(t[i], t[i + 1], 1) / mass : 0.5 * (t[i] + t[i + 1]);
            delta = std::max(delta, std::fabs(nc[i] - c[i]));
        }
        c.swap(nc);
        if (delta < 1e-14) break;
    }
    std::vector<double> b(levels - 1);
    for (int i = 0; i + 1 < levels; ++i) b[i] = 0.5 * (c[i] + c[i + 1]);
    *centroids = c;
    *boundaries = b;
    std::lock_guard<std::mutex> lock(mu);
    cache[level] = {c, b};
}

// ------------------------------------------------------------ Householder --
// G (n x n, row-major) = Q R with Householder reflections; then column j of
// Q is negated where R_jj < 0, so that diag(R) > 0 and Q is unique.
void householder_q(const std::vector<double>& g, int n, std::vector<double>* qout) {
    std::vector<double> a(g);
    std::vector<std::vector<double>> vs(n);
    std::vector<double> rdiag(n);
    for (int j = 0; j < n; ++j) {
        double norm2 = 0.0;
        for (int i = j; i < n; ++i) norm2 += a[i * n + j] * a[i * n + j];
        const double norm = std::sqrt(norm2);
        const double x0 = a[j * n + j];
        const double alpha = x0 >= 0.0 ? -norm : norm;
        std::vector<double> v(n - j);
        for (int i = j; i < n; ++i) v[i - j] = a[i * n + j];
        v[0] -= alpha;
        double vn2 = 0.0;
        for (double e : v) vn2 += e * e;
        if (vn2 > 0.0) {
            const double vinv = 1.0 / std::sqrt(vn2);
            for (double& e : v) e *= vinv;
            for (int c = j; c < n; ++c) {
                double dot = 0.0;
                for (int i = j; i < n; ++i) dot += v[i - j] * a[i * n + c];
                for (int i = j; i < n; ++i) a[i * n + c] -= 2.0 * v[i - j] * dot;
            }
        }
        rdiag[j] = a[j * n + j];
        vs[j] = std::move(v);
    }
    // Q = H_0 H_1 ... H_{n-1}: apply to the identity from the last reflector.
    std::vector<double> q(static_cast<size_t>(n) * n, 0.0);
    for (int i = 0; i < n; ++i) q[i * n + i] = 1.0;
    for (int j = n - 1; j >= 0; --j) {
        const std::vector<double>& v = vs[j];
        for (int c = 0; c < n; ++c) {
            double dot = 0.0;
            for (int i = j; i < n; ++i) dot += v[i - j] * q[i * n + c];
            for (int i = j; i < n; ++i) q[i * n + c] -= 2.0 * v[i - j] * dot;
        }
    }
    for (int j = 0; j < n; ++j)
        if (rdiag[j] < 0.0)
            for (int i = 0; i < n; ++i) q[i * n + j] = -q[i * n + j];
    *qout = std::move(q);
}

// --------------------------------------------------------------- half RNE --
uint16_t double_to_half_rne(double x) {
    uint64_t bits;
    std::memcpy(&bits, &x, sizeof bits);
    const uint16_t sign = static_cast<uint16_t>((bits >> 63) << 15);
    const double a = std::fabs(x);
    if (std::isnan(x)) return sign | 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;                 // rounds to infinity
    if (a < 0x1p-14) {                                      // subnormal range
        const double q = std::nearbyint(a * 0x1p24);        // exact scaling, RNE
        return sign | static_cast<uint16_t>(q);             // q == 1024 is the smallest normal
    }
    int e2;
    std::frexp(a, &e2);                                     // a = f 2^e2, f in [0.5, 1)
    int e = e2 - 1;                                         // a in [2^e, 2^(e+1))
    double m = std::nearbyint(std::ldexp(a, 10 - e));       // [1024, 2048]
    if (m >= 2048.0) {
        m = 1024.0;
        ++e;
    }
    if (e > 15) return sign | 0x7C00;
    return sign | static_cast<uint16_t>(((e + 15) << 10) | (static_cast<int>(m) - 1024));
}

// ------------------------------------------------------------------- bins --
int bin_slot(float y, float bin_b) {
    const float t = std::fmaf(y, kBinA, bin_b);
    uint32_t u;
    std::memcpy(&u, &t, 4);
    return static_cast<int>((u & 0xFF0u) >> 4);
}

bool make_bins(Tables* t) {
    const std::vector<float>& c = t->centroids;
    const std::vector<float>& b = t->boundaries;
    const int nb = static_cast<int>(b.size());
    const float magic = 12582912.0f;   // 1.5 * 2^23: fp32 sums in [2^23, 2^24) are integers
    // bias 16 * o with o = 128 + k / 16: slot(y) ~ floor(127 y + o)
    for (int k : {0, 1, -1, 2, -2, 3, -3, 4, -4, 5, -5, 6, -6, 7, -7}) {
        const float bias = magic + 16.0f * 128.0f + static_cast<float>(k);
        // no wrap-around for |y| <= 1.001: the integer part stays in [0, 4096)
        const float lo_t = std::fmaf(-1.001f, kBinA, bias) - magic;
        const float hi_t = std::fmaf(1.001f, kBinA, bias) - magic;
        if (lo_t < 0.0f || hi_t > 4095.0f) continue;
        std::vector<int> owner(kBins, -1);
        bool ok = true;
        int prev = -1;
        for (int i = 0; i < nb && ok; ++i) {
            const int s = bin_slot(b[i], bias);
            if (s <= prev || owner[s] >= 0) ok = false;
            else owner[s] = i;
            prev = s;
        }
        if (!ok) continue;
        t->bin_b = bias;
        t->bins.assign(kBins, BinEntry{});
        uint32_t base = 0;
        for (int s = 0; s < kBins; ++s) {
            BinEntry e;
            e.base = base;
            e.c_lo = c[base];
            if (owner[s] >= 0) {
                e.thr = b[owner[s]];
                e.c_hi = c[base + 1];
                ++base;
            } else {
                e.thr = std::numeric_limits<float>::infinity();
                e.c_hi = c[base];
            }
            t->bins[s] = e;
        }
        return true;
    }
    return false;
}

// ----------------------------------------------------------------- tables --
int make_tables(int d, int bits, uint64_t seed, int mode, Tables* out, std::string* err) {
    Layout lay;
    const int rc = make_layout(d, bits, mode, &lay, err);
    if (rc) return rc;
    Tables t;
    t.lay = lay;
    if (mode & kModePolar) {
        // the four codebooks concatenated, then Pi as in the dense sessions
        for (int level = 0; level < kPolarLevels; ++level) {
            std::vector<double> c, b;
            lloyd_polar(level, &c, &b);
            for (double v : c) t.centroids.push_back(to_f32(v));
            for (double v : b) t.boundaries.push_back(to_f32(v));
        }
        const std::vector<double> g = normals(seed, kTagPi, static_cast<size_t>(d) * d);
        std::vector<double> q;
        householder_q(g, d, &q);
        t.pi.resize(q.size());
        for (size_t i = 0; i < q.size(); ++i) t.pi[i] = to_f32(q[i]);
        *out = std::move(t);
        return 0;
    }
    std::vector<double> c, b;
    if (lay.mse_bits == 0) {
        c.assign(1, 0.0);   // QJL only: one level of value 0, no boundaries
    } else {
        lloyd_max_unit_sphere(d, lay.mse_bits, &c, &b);
    }
    t.centroids.resize(c.size());
    t.boundaries.resize(b.size());
    for (size_t i = 0; i < c.size(); ++i) t.centroids[i] = to_f32(c[i]);
    for (size_t i = 0; i < b.size(); ++i) t.boundaries[i] = to_f32(b[i]);
    if (!make_bins(&t)) {
        if (err) *err = "no bin grid separates the codebook boundaries";
        return 2;
    }
    if (mode & kModeDense) {
        const std::vector<double> g = normals(seed, kTagPi, static_cast<size_t>(d) * d);
        std::vector<double> q;
        householder_q(g, d, &q);
        t.pi.resize(q.size());
        for (size_t i = 0; i < q.size(); ++i) t.pi[i] = to_f32(q[i]);
    } else {
        make_rotors(d, seed, &t.rotors, &t.rotmats);
    }
    if (mode & kModeQjl) {
        const std::vector<double> z = normals(seed, kTagS, static_cast<size_t>(kQjlRows) * d);
        t.s.resize(z.size());
        for (size_t i = 0; i < z.size(); ++i) t.s[i] = double_to_half_rne(z[i]);
    }
    *out = std::move(t);
    return 0;
}

}  // namespace rqh
