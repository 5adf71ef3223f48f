// Launchers of the device kernels (called by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rqk {

// 16-byte table entry as seen by host code
struct u32x4_t {
    uint32_t v[4];
};

// Slots of the quantiser lookup table: entry = {base code, boundary inside
// the slot (+inf if none), c[base], c[base + 1]}; a unit-domain coordinate y
// falls in slot (bits(fma(y, bin_a, bin_b)) & 0xFF0) / 16.
constexpr int kBinSlots = 256;

// Device-resident tables of a rotor session.
struct RotorTables {
    const float* rotmat;     // [43][9]
    const float* rotmat16;   // [43][16]: the same matrices, one 64-byte line per group
    const float* thr;        // [L-1]
    const float* cent;       // [L]
    const u32x4_t* bins;     // [kBinSlots]
    float bin_a, bin_b;
    const uint16_t* s_rows;  // [128][128] halves (QJL)
    const uint16_t* s_cols;  // [128][128] halves, S^T (QJL)
    const uint16_t* s_fwd;   // S, rows and columns permuted for the codec kernels' MFMA layout
    const uint16_t* s_back;  // S^T, rows and columns permuted for the back-projection
    const uint16_t* phi_hi;  // 16 Phi = hi + 2^-11 lo: the rotor transform of the first 128
    const uint16_t* phi_lo;  //   slots as a block-diagonal 128 x 128 matrix (scoring)
    float qjl_scale;
    int mse_bits;
    bool qjl;
};

// Device-resident tables of a dense (TurboQuant) session.  Pi is stored as
// two half matrices, Pi = (hi + lo * 2^-11) / 16, in both layouts.
struct DenseTables {
    const uint16_t* pi_hi;   // [128][128] row-major
    const uint16_t* pi_lo;
    const uint16_t* pit_hi;  // transposed
    const uint16_t* pit_lo;
    const uint16_t* pi2_hi;  // Pi permuted for the codec kernels' MFMA layout, row-major
    const uint16_t* pi2_lo;
    const uint16_t* pit2_hi; // Pi^T permuted likewise, in MFMA fragment order
    const uint16_t* pit2_lo;
    const uint16_t* t2_hi;   // T = S Pi^T permuted likewise, fragment order (QJL)
    const uint16_t* t2_lo;
    const uint16_t* s_back;  // S^T permuted likewise, fragment order (QJL)
    const float* thr;
    const float* cent;
    const uint16_t* s_rows;
    const uint16_t* s_cols;
    const u32x4_t* bins;     // the slot table of the rotor sessions (same codebook)
    float bin_a, bin_b;
    float qjl_scale;
    int mse_bits;
    bool qjl;
};

// PolarQuant sessions (rq_polar.hip): y = Pi x, four levels of polar angle
// codes and eight half radii in a 16-word record per vector.
constexpr int kPolarTab = 2 * (7 + 3 + 3 + 3) + 2 * (16 + 4 + 4 + 4);   // floats
constexpr int kPolarWords = 16;       // u32 words per record
struct PolarDev {
    const uint16_t* pi_hi;    // 16 Pi = hi + 2^-11 lo, row-major (y = Pi x)
    const uint16_t* pi_lo;
    const uint16_t* pit_hi;   // the same pair transposed (x = Pi^T y)
    const uint16_t* pit_lo;
    const float* pi32;        // Pi in fp32, row-major
    const float* tab;         // kPolarTab floats: (cos, sin) of boundaries, then of centroids
    // codec kernels (two lanes per vector): the pair permuted as for the dense
    // codec, Pi row by row (staged in LDS), Pi^T in MFMA fragment order
    const uint16_t* pi2_hi;
    const uint16_t* pi2_lo;
    const uint16_t* pit2_hi;
    const uint16_t* pit2_lo;
};
struct ScoreTables {
    bool dense;
    RotorTables rot;
    DenseTables den;
    bool polar = false;      // PolarQuant keys (rq_attend only): records are 16-word rows
    PolarDev pol{};
    int mse_bits;
    bool qjl;
    float qjl_scale;
};

// Query rows per scoring launch (RQ_SCORE_CHUNK of rq.h).
constexpr int kScoreChunkRows = 4096;

hipError_t rotor_quantize(const RotorTables& t, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                          int64_t ldy_bytes, bool roundtrip, hipStream_t s);

hipError_t rotor_dequantize(const RotorTables& t, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                            const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                            hipStream_t s);

hipError_t dense_quantize(const DenseTables& t, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                          int64_t ldy_bytes, bool roundtrip, hipStream_t s);

hipError_t dense_dequantize(const DenseTables& t, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                            const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                            hipStream_t s);

// Outlier channels of QJL-only keys: record row r belongs to head
// r / head_rows, whose k channels are chans[head * k .. + k) (increasing,
// < 128); the record's outlier array holds k halves per row.
constexpr int kMaxOutliers = 16;
struct OutlierArgs {
    const uint8_t* chans = nullptr;
    int64_t heads = 0;            // rows of chans
    int64_t head_rows = 1;
    int k = 0;
    uint16_t* out = nullptr;      // quantise: written [n][k]
    const uint16_t* in = nullptr; // dequantise: read [n][k]
};
// Scoring QJL-only keys with separated outliers: channel sets per KV head
// (global head index) and the keys' outlier halves, record-row major.
struct ScoreOutliers {
    const uint8_t* chans = nullptr;
    const uint16_t* values = nullptr;
    int k = 0;
};

// Optional page table of record rows: key t of (global) KV head j lives in
// record row pages[j * stride + (t >> shift)] * 2^shift + (t & (2^shift - 1)).
// With pages == nullptr, KV head j's keys are rows j * kv_stride + t.
struct PageTable {
    const int32_t* pages = nullptr;
    int shift = 0;          // log2 of the page size in keys, >= 6
    int64_t stride = 0;     // table entries per KV head
};

// Optional output of the scoring kernel for groups of at most 16 rows (the
// attention path): for each workgroup x of the launch and query row r of the
// call, the largest scale * estimate over the workgroup's keys, at
// ptr[x * ld + r] (-inf where it has none).
struct RowMax {
    float* ptr = nullptr;
    int64_t ld = 0;
    float scale = 0.0f;
};

// Workgroups along the keys of one scoring launch for groups of at most 16
// rows over kv_heads KV heads of t keys (the launch's grid.x).
int score_slices16(int64_t t, int kv_heads);

// Scores hq query rows (group rows per KV head) against t keys per KV head;
// KV head j (0-based within this call) reads record rows
// (kv_head0 + j) * kv_stride + [0, t).
hipError_t score(const ScoreTables& t, const float* q, int hq, int group, const uint32_t* codes,
                 const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms, int64_t tkeys,
                 int64_t kv_stride, int kv_head0, float* scores, int64_t ld_scores, hipStream_t s,
                 const PageTable& pt = PageTable{}, const ScoreOutliers& so = ScoreOutliers{},
                 const RowMax& rm = RowMax{});


// A partial row of the attention value pass: centroid sums for coordinates
// 0..127 (PolarQuant values: the sums of y~), sign sums 0..127, the rotor
// pad coordinate, padding.
constexpr int kPartStride = 260;
constexpr int kPartSigma = 128;
constexpr int kPartPad = 256;

// The PolarQuant value pass of rq_attend: partial rows [producers][rows]
// [kPartStride] of sum_t p_t y~_t for the estimates `scores` (row stride ld)
// and the row statistics `stats` (max, sum of exp) of scale * estimate.
struct PolarValueArgs {
    const float* scores;
    int64_t ld;
    const float2* stats;
    float scale;
    const uint32_t* words;    // value records, 16 words per key; KV head j at row j * kv_stride
    int64_t t, kv_stride;
    int group, rows;
    float* part;
};
hipError_t polar_attend_values(const PolarDev& P, const PolarValueArgs& a, int producers, int kv_heads,
                               hipStream_t s);

// Decode attention over compressed keys and values (rq_attend): workspace
// layout for hq query rows over t keys, and the launcher.
struct AttendPlan {
    int64_t ld;                      // row pitch of the estimates (floats)
    int gx;                          // key slices per (KV head, 32-row block)
    int64_t producers;               // partial rows per query row (one per key-slice block)
    int64_t off_scores, off_stats, off_part, off_rowmax, bytes;
};
// plan_rows: the query rows whose KV heads size the key slices (default
// hq).  A call over several layers of a paged cache passes one layer's rows,
// so that every (KV head, row block) is cut into the same slices, and summed
// in the same order, as in a one-layer call.
AttendPlan attend_plan(int hq, int group, int64_t t, int plan_rows = 0);

hipError_t attend(const ScoreTables& kt, const ScoreTables& vt, const float* q, int hq, int group,
                  const uint32_t* kcodes, const uint16_t* knorms, const uint32_t* ksigns, const uint16_t* krnorms,
                  const uint32_t* vcodes, const uint16_t* vnorms, const uint32_t* vsigns, const uint16_t* vrnorms,
                  int64_t t, int64_t kv_stride, float scale, void* workspace, float* out, int64_t ld_out,
                  hipStream_t s, const PageTable& kpt = PageTable{}, const PageTable& vpt = PageTable{},
                  int plan_rows = 0);

// rq_attend_noalloc: a fixed device array per GPU (rq_attend.hip) serves as
// the workspace.  noalloc_scratch resolves its address on the current device
// (once per device, then cached); it allocates nothing.
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// QJL-only sessions (one bit in total, no MSE stage; rotor or dense alike):
// the record is norm, signs of S x_u and gamma, with no code words.
struct Qjl1Dev {
    const uint16_t* s_fwd;   // S with rows permuted for the quantiser's MFMA layout
    const uint16_t* s_back;  // S^T permuted for the dequantiser
    float qjl_scale;
};
hipError_t qjl1_quantize(const Qjl1Dev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n, uint16_t* norms,
                         uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16, int64_t ldy_bytes, bool roundtrip,
                         hipStream_t s);
hipError_t qjl1_dequantize(const Qjl1Dev& P, const uint16_t* norms, const uint32_t* signs, const uint16_t* rnorms,
                           int64_t n, void* y, bool out_f16, int64_t ldy_bytes, hipStream_t s);
hipError_t qjl1_quantize_outliers(const Qjl1Dev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                                  uint16_t* norms, uint32_t* signs, uint16_t* rnorms, const OutlierArgs& o,
                                  hipStream_t s);
hipError_t qjl1_dequantize_outliers(const Qjl1Dev& P, const uint16_t* norms, const uint32_t* signs,
                                    const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                                    const OutlierArgs& o, hipStream_t s);
// Per head of head_rows consecutive rows: the k channels of largest mean |x|
// (rq_outlier.hip).
hipError_t outlier_select(const void* x, bool in_f16, int64_t heads, int64_t head_rows, int64_t ldx_bytes, int k,
                          uint8_t* chans, hipStream_t s);

constexpr int kPolarScoreRows = 32;   // query rows per scoring workgroup
hipError_t polar_quantize(const PolarDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* words, void* y, bool out_f16, int64_t ldy_bytes, bool roundtrip, hipStream_t s);
hipError_t polar_dequantize(const PolarDev& P, const uint32_t* words, int64_t n, void* y, bool out_f16,
                            int64_t ldy_bytes, hipStream_t s);
hipError_t polar_score(const PolarDev& P, const float* q, int hq, int group, const uint32_t* words, int64_t t,
                       int64_t kv_stride, float* scores, int64_t ld_scores, hipStream_t s);

// Reference copy of `bytes` (a multiple of 16, 16-byte aligned) with the
// codec kernels' 16-byte buffer load/store pattern (rq_copy.hip).
hipError_t copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t s);

// Paged cache helpers (rq_cache.hip).
hipError_t scatter_rows(const uint32_t* src_codes, const uint16_t* src_norms, const uint32_t* src_signs,
                        const uint16_t* src_rnorms, uint32_t* dst_codes, uint16_t* dst_norms, uint32_t* dst_signs,
                        uint16_t* dst_rnorms, int words, bool qjl, int64_t n, int64_t t0, int heads,
                        const PageTable& pt, bool gather, hipStream_t s);
hipError_t merge_current(const float* q, int hq, int group, const float* kcur, const float* vcur,
                         const float2* stats, float scale, float* out, int64_t ld_out, hipStream_t s);

}  // namespace rqk
