// Host core of the codec: parameter generation and record-layout arithmetic.
// Plain C++17, no HIP: it builds and runs on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace rqh {

constexpr int kDim = 128;          // the only d the device kernels support
constexpr int kQjlRows = 128;      // m, rows of S
constexpr int kMaxMseBits = 4;

enum : int { kModeQjl = 1, kModeDense = 2, kModePolar = 4 };

// PolarQuant (recursive polar transform of y = Pi x): four levels of angle
// codes, 4 bits on [0, 2 pi) for the 64 first-level pairs, 2 bits on
// [0, pi/2] for the 32 / 16 / 8 pairs of later levels, and 8 final radii as
// halves; a record of 16 u32 words (codes in words 0..11, radii in 12..15).
constexpr int kPolarLevels = 4;
constexpr int kPolarBits[kPolarLevels] = {4, 2, 2, 2};
constexpr int kPolarWords = 16;
constexpr int kPolarCentroids = 16 + 4 + 4 + 4;   // codebooks of the four levels, concatenated
constexpr int kPolarBoundaries = 15 + 3 + 3 + 3;

struct Layout {
    int d = 0, bits = 0, mse_bits = 0, mode = 0;
    int n_coords = 0, n_groups = 0, levels = 0;
    int code_words = 0, sign_words = 0, record_bytes = 0;
};

// Returns 0, 1 (invalid) or 2 (unsupported); fills *out on success.
int make_layout(int d, int bits, int mode, Layout* out, std::string* err);

// Exact nearest-centroid lookup through a 256-entry table.  The device maps a
// unit-domain coordinate y to a table slot with one fp32 fused multiply-add
// whose result, biased by 1.5 * 2^23, is an integer held in the low mantissa
// bits:  t = fma(y, kBinA, bin_b),  slot = (bits(t) & 0xFF0) / 16.
// The map is monotone in y, so with every Lloyd-Max boundary assigned (by the
// same fp32 fma, evaluated here) to its own slot,
//   #{k : y > t_k} = base[slot] + (y > thr[slot]),
// exactly for every y; value = y > thr[slot] ? c_hi : c_lo is c[code].
// Slots are 1/127 wide in y; make_bins picks the bias so no two boundaries
// share a slot and |y| <= 1.001 never wraps.
constexpr int kBins = 256;
constexpr float kBinA = 2032.0f;   // 16 * 127
struct BinEntry {
    uint32_t base;
    float thr, c_lo, c_hi;
};
// Slot of y under bias bin_b (the device computation, bit for bit).
int bin_slot(float y, float bin_b);

struct Tables {
    Layout lay;
    std::vector<BinEntry> bins;     // [kBins]
    float bin_b = 0.0f;
    std::vector<float> rotors;      // [G][4] s, b12, b13, b23
    std::vector<float> rotmats;     // [G][9] row-major M, y = M v
    std::vector<float> centroids;   // [L]
    std::vector<float> boundaries;  // [L-1]
    std::vector<float> pi;          // [d][d] row-major (dense)
    std::vector<uint16_t> s;        // [m][d] half bits, row-major (QJL)
};

// Lloyd's algorithm for the angle law of PolarQuant level `level` (0-based):
// level 0 uniform on [0, 2 pi), level l >= 1 the density
// Gamma(k) / (2^(k-2) Gamma(k/2)^2) sin^(k-1)(2 theta) on [0, pi/2], k = 2^l.
void lloyd_polar(int level, std::vector<double>* centroids, std::vector<double>* boundaries);

// Builds every table of (d, bits, seed, mode); returns 0/1/2 as make_layout.
int make_tables(int d, int bits, uint64_t seed, int mode, Tables* out, std::string* err);

// Fills t->bins and t->bin_b from t->centroids / t->boundaries; returns
// false if no bias separates the boundaries (not the case for d = 128).
bool make_bins(Tables* t);

// --- pieces exposed for host tests --------------------------------------
uint64_t splitmix64_next(uint64_t* state);
std::vector<double> normals(uint64_t seed, uint64_t tag, size_t count);
void lloyd_max_unit_sphere(int d, int bits, std::vector<double>* centroids,
                           std::vector<double>* boundaries);
void householder_q(const std::vector<double>& g, int n, std::vector<double>* q);
uint16_t double_to_half_rne(double x);
float rotor_matrix_entry_check(const float r[4], double m[9]);  // fills m, returns det

}  // namespace rqh
