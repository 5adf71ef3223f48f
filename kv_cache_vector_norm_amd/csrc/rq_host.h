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

enum : int { kModeQjl = 1, kModeDense = 2 };

struct Layout {
    int d = 0, bits = 0, mse_bits = 0, mode = 0;
    int n_coords = 0, n_groups = 0, levels = 0;
    int code_words = 0, sign_words = 0, record_bytes = 0;
};

// Returns 0, 1 (invalid) or 2 (unsupported); fills *out on success.
int make_layout(int d, int bits, int mode, Layout* out, std::string* err);

struct Tables {
    Layout lay;
    std::vector<float> rotors;      // [G][4] s, b12, b13, b23
    std::vector<float> rotmats;     // [G][9] row-major M, y = M v
    std::vector<float> centroids;   // [L]
    std::vector<float> boundaries;  // [L-1]
    std::vector<float> pi;          // [d][d] row-major (dense)
    std::vector<uint16_t> s;        // [m][d] half bits, row-major (QJL)
};

// Builds every table of (d, bits, seed, mode); returns 0/1/2 as make_layout.
int make_tables(int d, int bits, uint64_t seed, int mode, Tables* out, std::string* err);

// --- pieces exposed for host tests --------------------------------------
uint64_t splitmix64_next(uint64_t* state);
std::vector<double> normals(uint64_t seed, uint64_t tag, size_t count);
void lloyd_max_unit_sphere(int d, int bits, std::vector<double>* centroids,
                           std::vector<double>* boundaries);
void householder_q(const std::vector<double>& g, int n, std::vector<double>* q);
uint16_t double_to_half_rne(double x);
float rotor_matrix_entry_check(const float r[4], double m[9]);  // fills m, returns det

}  // namespace rqh
