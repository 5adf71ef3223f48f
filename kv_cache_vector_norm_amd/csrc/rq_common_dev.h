// Device-side building blocks shared by the codec kernels (gfx950 only).
//
// Thread mapping used throughout: a wave of 64 lanes owns a tile of 64
// vectors, lane l owning vector (tile base + l).  Global memory is read and
// written in fully coalesced 16-byte chunks and transposed through a per-wave
// LDS tile; every per-vector step then runs in registers with compile-time
// coordinate indices.  MFMA contractions over the tile use
// v_permlane32_swap to move between "lane = vector" and the 32x32x16 operand
// layout (lanes l and l+32 hold the two 8-element K halves of row l % 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rqk {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;        // vector dimension
constexpr int kGroups = 43;    // ceil(128 / 3) rotor groups
constexpr int kRotCoords = 129;
constexpr int kWave = 64;
constexpr int kTileBytes = 64 * 256;   // one wave's LDS transpose tile
constexpr int kSimds = 256 * 4;         // MI355X: 256 compute units of 4 SIMDs

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N).  The
// per-group loops use it instead of #pragma unroll, whose size limit a long
// body exceeds, so that every register-array index is a constant.
template <int I, int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// ------------------------------------------------------------------ LDS --
// 64 rows x 16 chunks of 16 B.  Chunk c of row r lives in slot
// r * 16 + (c ^ (r & 15)): row-wise (one lane per row) and chunk-wise (16
// lanes per row) accesses are then both free of bank conflicts.
__device__ __forceinline__ int swz(int r, int c) { return r * 16 + (c ^ (r & 15)); }

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (DS instructions of one wave complete in order; this stops the
// compiler from moving accesses across the point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// An SGPR zero the compiler cannot see through.  Kernels with a grid-stride
// tile loop derive the lane index from it inside each iteration: otherwise
// loop-invariant code motion hoists every per-lane address of the tile
// transposes out of the loop and keeps them live (hundreds of VGPRs).
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// Pins a value at this program point.  The per-vector loops are fully
// unrolled into one large basic block; without pins the instruction selector
// sinks each group's arithmetic down to the final use, keeping every loaded
// input live at once.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
template <class V>
__device__ __forceinline__ void pin_lane(V& vec, int e) {
    uint32_t x = vec[e];
    asm volatile("" : "+v"(x));
    vec[e] = x;
}
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// A wave-uniform float forced into an SGPR.
__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// --------------------------------------------------------- conversions --
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(f16, static_cast<uint16_t>(bits16)));
}
__device__ __forceinline__ uint32_t f2h(float x) {   // round to nearest even
    return __builtin_bit_cast(uint16_t, static_cast<f16>(x));
}
__device__ __forceinline__ uint32_t pack2h(float a, float b) { return f2h(a) | (f2h(b) << 16); }

// Two floats -> two halves (round to nearest even) in one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}

// Two halves times 2^11 (v_pk_mul_f16; exact for |x| < 32).
__device__ __forceinline__ uint32_t pk_scale2048(uint32_t h2) {
    const f16x2 v = __builtin_bit_cast(f16x2, h2) * f16x2{static_cast<f16>(2048.0f), static_cast<f16>(2048.0f)};
    return __builtin_bit_cast(uint32_t, v);
}

// Exact split of a float pair: (a, b) ~= hi + lo, hi = half(a, b) and lo the
// halves of the fp32 residuals a - hi (exact) rounded to nearest even.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t* hi, uint32_t* lo) {
    const uint32_t h = cvt_pk(a, b);
    *hi = h;
    *lo = cvt_pk(a - h2f(h & 0xFFFFu), b - h2f(h >> 16));
}

// Exact split of a float into two halves: x ~= hi + lo with the residual of
// hi's rounding kept in lo (both round to nearest even).
__device__ __forceinline__ void split_h(float x, uint32_t* hi, uint32_t* lo) {
    const f16 h = static_cast<f16>(x);
    const f16 l = static_cast<f16>(x - static_cast<float>(h));
    *hi = __builtin_bit_cast(uint16_t, h);
    *lo = __builtin_bit_cast(uint16_t, l);
}

// Split with the low half scaled: x = hi + 2^-11 lo11 to ~2^-22 relative,
// hi = half(x), lo11 = half((x - hi) * 2^11).  x - hi is exact in fp32 and
// the scaling is exact, so only the final rounding of lo11 is lost.
__device__ __forceinline__ void split_h11(float x, uint32_t* hi, uint32_t* lo11) {
    const uint32_t h = f2h(x);
    *hi = h;
    *lo11 = f2h((x - h2f(h)) * 2048.0f);
}

// -------------------------------------------------------------- tiles --
// Global traffic goes through raw buffer instructions: a per-tile descriptor
// (base address in SGPRs, byte range = the rows that exist), a per-lane
// 32-bit offset fixed for the kernel and a uniform per-instruction offset.
// Accesses beyond the range read 0 and drop stores, which handles the
// ragged last tile without per-row branches.  Row pitches are at most 2^26
// bytes, so every offset of a 64-row tile fits in 32 bits.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 buffer descriptor dword 3
constexpr int kNonTemporal = 2;          // aux bits: nt

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             kRsrcWord3);
}
// Byte range of `rows_left` rows of `row_bytes` (all of 32-bit space for a full tile).
__device__ __forceinline__ uint32_t tile_range(int64_t rows_left, int64_t row_bytes) {
    return rows_left >= 64 ? 0xFFFFFFFFu : static_cast<uint32_t>(rows_left * row_bytes);
}

// A tile's 64 rows of 256 bytes (from byte `col_off` of each row) in
// registers: lane l holds chunk l % 16 of rows 4 it + l / 16; rows at or
// beyond n read as zero.  tile_put then writes them into the LDS tile.
struct TileRegs {
    u32x4 v[16];
};
__device__ __forceinline__ void tile_fetch(const char* __restrict__ src, int64_t ld_bytes, int64_t base, int64_t n,
                                           int col_off, TileRegs& r, int l) {
    const int rr = l >> 4, c = l & 15;
    const uint32_t voff = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld_bytes) + static_cast<uint32_t>(c * 16);
    const rsrc_t rs = make_rsrc(src + base * ld_bytes + col_off, tile_range(n - base, ld_bytes));
    const int step = static_cast<int>(4 * ld_bytes);
#pragma unroll
    for (int it = 0; it < 16; ++it) r.v[it] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, it * step, kNonTemporal);
}
__device__ __forceinline__ void tile_put(const TileRegs& r, u32x4* __restrict__ tile, int l) {
    const int rr = l >> 4, c = l & 15;
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const u32x4 v = r.v[it];
        tile[swz(4 * it + rr, c)] = v;
    }
}

// Reads 64 rows of 256 bytes (starting at byte offset `col_off` of each row)
// into the wave's LDS tile; rows at or beyond n are zero.  Lane l moves
// chunk l % 16 of rows 4 it + l / 16.
__device__ __forceinline__ void tile_load(const char* __restrict__ src, int64_t ld_bytes, int64_t base,
                                          int64_t n, int col_off, u32x4* __restrict__ tile, int l) {
    wave_lds_sync();
    const int rr = l >> 4, c = l & 15;
    const uint32_t voff = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld_bytes) + static_cast<uint32_t>(c * 16);
    const rsrc_t rs = make_rsrc(src + base * ld_bytes + col_off, tile_range(n - base, ld_bytes));
    const int step = static_cast<int>(4 * ld_bytes);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, it * step, kNonTemporal);
        tile[swz(4 * it + rr, c)] = v;
    }
}

// A buffer store of more than 64 bits reads its data registers after it has
// issued, so an instruction in the next cycles must not overwrite them (the
// vector-memory store-data hazard; 128-bit stores whose first data register
// was rewritten by the very next VALU instruction stored that new value when
// two workgroups shared a CU).  The compiler does not separate them here, so
// every 128-bit store group is closed by this fence: nothing is scheduled
// across it and it adds two wait states.
__device__ __forceinline__ void store_data_fence() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");
    __builtin_amdgcn_sched_barrier(0);
}

// Writes the LDS tile to 64 rows of 256 bytes (from byte `col_off` of each
// row).  Rows 4 it + l / 16 for it = b, b + 4, b + 8, b + 12 share one LDS
// swizzle, so each group of four is read with one address and immediate
// offsets, then stored with no other instruction in between.
__device__ __forceinline__ void tile_store(char* __restrict__ dst, int64_t ld_bytes, int64_t base, int64_t n,
                                           int col_off, const u32x4* __restrict__ tile, int l) {
    const int rr = l >> 4, c = l & 15;
    const uint32_t voff = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld_bytes) + static_cast<uint32_t>(c * 16);
    const rsrc_t rs = make_rsrc(dst + base * ld_bytes + col_off, tile_range(n - base, ld_bytes));
    const int step = static_cast<int>(4 * ld_bytes);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = tile[swz(4 * (b + 4 * k) + rr, c)];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rs, voff, (b + 4 * k) * step, kNonTemporal);
        store_data_fence();
    }
}

// Writes chunks c0 .. c0 + 3 (64 bytes) of the LDS tile's 64 rows: lane l
// moves chunk c0 + l % 4 of rows l / 4 + 16 k.  Lets a kernel store each
// finished quarter of fp16 output rows while it computes the next.
__device__ __forceinline__ void tile_store_cols(char* __restrict__ dst, int64_t ld_bytes, int64_t base, int64_t n,
                                                const u32x4* __restrict__ tile, int l, int c0) {
    const int rr = l >> 2, c = c0 + (l & 3);
    const uint32_t voff = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld_bytes) + static_cast<uint32_t>(c * 16);
    const rsrc_t rs = make_rsrc(dst + base * ld_bytes, tile_range(n - base, ld_bytes));
    const int step = static_cast<int>(16 * ld_bytes);
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = tile[swz(rr + 16 * k, c)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_amdgcn_raw_buffer_store_b128(v[k], rs, voff, k * step, kNonTemporal);
    store_data_fence();
}

// Record rows of `words` u32 per vector are contiguous, so a tile's rows form
// one run of 64 * words dwords: stage through LDS (row-major, stride `words`,
// odd or small strides are conflict-free for dword access) and copy the run.
template <int WORDS>
__device__ __forceinline__ void words_store(uint32_t* __restrict__ dst, int64_t base, int64_t n,
                                            const uint32_t (&w)[WORDS], uint32_t* __restrict__ stage, int l) {
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < WORDS; ++k) stage[l * WORDS + k] = w[k];
    wave_lds_sync();
    const rsrc_t rs = make_rsrc(dst + base * WORDS, tile_range(n - base, 4 * WORDS));
#pragma unroll
    for (int it = 0; it < WORDS; ++it) {
        const uint32_t v = stage[it * 64 + l];
        __builtin_amdgcn_raw_buffer_store_b32(v, rs, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    }
    wave_lds_sync();
}

template <int WORDS>
__device__ __forceinline__ void words_load(const uint32_t* __restrict__ src, int64_t base, int64_t n,
                                           uint32_t (&w)[WORDS], uint32_t* __restrict__ stage, int l) {
    const rsrc_t rs = make_rsrc(src + base * WORDS, tile_range(n - base, 4 * WORDS));
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < WORDS; ++it)
        stage[it * 64 + l] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < WORDS; ++k) w[k] = stage[l * WORDS + k];
    wave_lds_sync();
}

// One 16-bit value per lane (norms): lanes beyond n are dropped / read 0.
__device__ __forceinline__ void half_store(uint16_t* __restrict__ dst, int64_t base, int64_t n, uint32_t v, int l) {
    const rsrc_t rs = make_rsrc(dst + base, tile_range(n - base, 2));
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v), rs, static_cast<uint32_t>(2 * l), 0, kNonTemporal);
}
__device__ __forceinline__ uint32_t half_load(const uint16_t* __restrict__ src, int64_t base, int64_t n, int l) {
    const rsrc_t rs = make_rsrc(src + base, tile_range(n - base, 2));
    return __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<uint32_t>(2 * l), 0, kNonTemporal);
}

// ------------------------------------------------------------- codes --
// Dense little-endian bit stream: code i at bits [B*i, B*i + B).
template <int B, int W>
__device__ __forceinline__ void put_code(uint32_t (&w)[W], int i, uint32_t code) {
    const int bit = B * i, wi = bit >> 5, off = bit & 31;
    w[wi] |= code << off;
    if (off + B > 32) w[wi + 1] |= code >> (32 - off);
}

template <int B, int W>
__device__ __forceinline__ uint32_t get_code(const uint32_t (&w)[W], int i) {
    const int bit = B * i, wi = bit >> 5, off = bit & 31;
    uint32_t c = w[wi] >> off;
    if (off + B > 32) c |= w[wi + 1] << (32 - off);
    return c & ((1u << B) - 1u);
}

// code = #{k : y > t_k}: nearest centroid with midpoint boundaries, a tie
// going to the lower index.
template <int B>
__device__ __forceinline__ uint32_t quant_code(float y, const float (&thr)[(1 << B) - 1]) {
    uint32_t code = 0;
#pragma unroll
    for (int k = 0; k < (1 << B) - 1; ++k) code += (y > thr[k]) ? 1u : 0u;
    return code;
}

// ------------------------------------------------------------- MFMA --
__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}
// 16x16x32: lane l holds row (A) or column (B) l % 16, K elements
// 8 (l / 16) .. + 7; the result holds column l % 16, rows 4 (l / 16) .. + 3.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}

// Lane l holds X = its own vector's K-chunk 0 and Y = chunk 1 (8 halves each).
// Returns the B (or A) operands for the tile's two 32-vector halves:
// op0 = vectors 0..31, op1 = vectors 32..63.
__device__ __forceinline__ void to_operands(const u32x4& x, const u32x4& y, u32x4* op0, u32x4* op1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t xk = x[k];
        const uint32_t yk = y[k];
        const auto r = __builtin_amdgcn_permlane32_swap(xk, yk, false, false);
        const uint32_t r0 = r[0];
        const uint32_t r1 = r[1];
        (*op0)[k] = r0;
        (*op1)[k] = r1;
    }
}

// Accumulators of the two vector halves -> this lane's own vector values:
// own0[r] = row 8(r/4) + r%4, own1[r] = row 8(r/4) + 4 + r%4 of the 32-row
// M tile.
__device__ __forceinline__ void from_accumulators(const f32x16& a0, const f32x16& a1, float (&own0)[16],
                                                  float (&own1)[16]) {
    // Elements are copied to scalars first: a bit cast applied directly to an
    // element of a vector reached through a reference was observed to read
    // element 0 for every index.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float e0 = a0[r];
        const float e1 = a1[r];
        const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, e0),
                                                        __builtin_bit_cast(uint32_t, e1), false, false);
        const uint32_t o0 = s[0];
        const uint32_t o1 = s[1];
        own0[r] = __builtin_bit_cast(float, o0);
        own1[r] = __builtin_bit_cast(float, o1);
    }
}

// Row index (within a 32-row M tile) of own0/own1 register r.
__host__ __device__ constexpr int own_row(int half, int r) { return 8 * (r / 4) + 4 * half + (r % 4); }

// Matrix slab in LDS: 128 rows x 128 halves, 16-byte chunks swizzled per row.
__device__ __forceinline__ u32x4 mat_frag(const u32x4* __restrict__ m, int row, int chunk) {
    return m[row * 16 + (chunk ^ (row & 15))];
}

// Copies a 128 x 128 half matrix (row-major, 32 KB) into swizzled LDS.
// Threads per block of the codec kernels (the TurboQuant QJL kernels use
// 128).  The copy is unrolled so all of a thread's loads are in flight
// before the first LDS store waits on one.
constexpr int kBlock = 256;
template <int NT = kBlock>
__device__ __forceinline__ void mat_to_lds(const uint16_t* __restrict__ g, u32x4* __restrict__ m) {
    static_assert(128 * 16 % NT == 0, "block size");
    const u32x4* src = reinterpret_cast<const u32x4*>(g);
    u32x4 v[128 * 16 / NT];
#pragma unroll
    for (int it = 0; it < 128 * 16 / NT; ++it) v[it] = src[it * NT + threadIdx.x];
#pragma unroll
    for (int it = 0; it < 128 * 16 / NT; ++it) {
        const int q = it * NT + threadIdx.x, row = q >> 4, c = q & 15;
        m[row * 16 + (c ^ (row & 15))] = v[it];
    }
}

// ------------------------------------------------------------- outputs --
// Coordinates must be set in increasing order.  Each completed 16-byte chunk
// goes straight into this lane's row of the LDS tile; fp32 output flushes the
// first 256-byte half to memory when coordinate 64 begins.
template <bool OUT_F16>
struct VecOutT;

template <>
struct VecOutT<true> {
    u32x4 cur;
    u32x4* t;
    int l;
    __device__ void begin(u32x4* tile, int lane) {
        t = tile;
        l = lane;
        wave_lds_sync();
    }
    __device__ void set(int i, float v) {
        // the fp32 value is materialised first: half output is the round-
        // to-nearest-even of the fp32 output (no fused single rounding)
        pin(v);
        const uint32_t h = f2h(v);
        const int w = (i & 7) >> 1;
        if (i & 1) cur[w] |= h << 16; else cur[w] = h;
        if ((i & 7) == 7) {
            t[swz(l, i >> 3)] = cur;
        }
    }
    // coordinates i (even) and i + 1
    __device__ void set2(int i, float v0, float v1) {
        pin(v0);
        pin(v1);
        cur[(i & 7) >> 1] = cvt_pk(v0, v1);
        if ((i & 7) == 6) t[swz(l, i >> 3)] = cur;
    }
    __device__ void store(char* y, int64_t ld_bytes, int64_t base, int64_t n) {
        wave_lds_sync();
        tile_store(y, ld_bytes, base, n, 0, t, l);
    }
    // coordinates 8 c0 .. 8 c0 + 31 of every row, once all lanes have set them
    __device__ void store_cols(char* y, int64_t ld_bytes, int64_t base, int64_t n, int c0) {
        wave_lds_sync();
        tile_store_cols(y, ld_bytes, base, n, t, l, c0);
    }
};

template <>
struct VecOutT<false> {
    u32x4 cur;
    u32x4* t;
    int l;
    char* y;
    int64_t ld_bytes, base, n;
    __device__ void begin(u32x4* tile, int lane) {
        t = tile;
        l = lane;
        wave_lds_sync();
    }
    __device__ void bind(char* yy, int64_t ldb, int64_t b, int64_t nn) {
        y = yy;
        ld_bytes = ldb;
        base = b;
        n = nn;
    }
    __device__ void set(int i, float v) {
        cur[i & 3] = __builtin_bit_cast(uint32_t, v);
        if ((i & 3) == 3) t[swz(l, (i >> 2) & 15)] = cur;
        if (i == 63) {
            wave_lds_sync();
            tile_store(y, ld_bytes, base, n, 0, t, l);
            wave_lds_sync();
        }
    }
    __device__ void set2(int i, float v0, float v1) {
        set(i, v0);
        set(i + 1, v1);
    }
    __device__ void store(char* yy, int64_t ldb, int64_t b, int64_t nn) {
        wave_lds_sync();
        tile_store(yy, ldb, b, nn, 256, t, l);
    }
};

}  // namespace rqk
