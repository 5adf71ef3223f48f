// Two-lanes-per-vector tile helpers shared by the rotor and dense codec
// kernels (gfx950): a wave owns a tile of 32 vectors, lanes v and v + 32
// sharing vector v.  Tiles cross LDS in rows padded to 272 (fp16) or 528
// (fp32) bytes, so that 16-byte chunks serve the coalesced global transfers
// and each lane's reads of its own part of a row spread over the banks.
#pragma once

#include "rq_common_dev.h"

namespace rqk {

template <bool F16>
constexpr int row_bytes2() { return F16 ? 272 : 528; }

// ------------------------------------------------------------ helpers --
// v as held by the other lane of this lane's vector (lane l +- 32).
__device__ __forceinline__ uint32_t other_half(uint32_t v, int h) {
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const uint32_t a = s[0];
    const uint32_t b = s[1];
    return h ? a : b;
}
__device__ __forceinline__ float other_half(float v, int h) {
    return __builtin_bit_cast(float, other_half(__builtin_bit_cast(uint32_t, v), h));
}

// Byte range of a 32-row tile's rows (all of 32-bit space for a full tile).
__device__ __forceinline__ uint32_t tile2_range(int64_t rows_left, int64_t row_bytes) {
    return rows_left >= 32 ? 0xFFFFFFFFu : static_cast<uint32_t>(rows_left * row_bytes);
}

// 32 rows of 256 (fp16) or 512 (fp32) bytes: lane l moves chunk l % CH of
// rows RPI it + l / CH.
template <bool F16>
struct Tile2Regs {
    u32x4 v[F16 ? 8 : 16];
};
template <bool F16>
struct Tile2Shape {
    static constexpr int CH = F16 ? 16 : 32;   // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;         // rows per instruction
    static constexpr int IT = 32 / RPI;         // instructions per tile
    static constexpr int RB = row_bytes2<F16>();
};

template <bool F16>
__device__ __forceinline__ void tile2_fetch(const char* __restrict__ src, int64_t ld_bytes, int64_t base, int64_t n,
                                            Tile2Regs<F16>& r, int l) {
    using T = Tile2Shape<F16>;
    const int rr = l / T::CH, c = l % T::CH;
    const uint32_t voff = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld_bytes) + static_cast<uint32_t>(16 * c);
    const rsrc_t rs = make_rsrc(src + base * ld_bytes, tile2_range(n - base, ld_bytes));
    const int step = static_cast<int>(T::RPI * ld_bytes);
#pragma unroll
    for (int it = 0; it < T::IT; ++it) r.v[it] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, it * step, kNonTemporal);
}

template <bool F16>
__device__ __forceinline__ void tile2_put(const Tile2Regs<F16>& r, char* __restrict__ tile, int l) {
    using T = Tile2Shape<F16>;
    const int rr = l / T::CH, c = l % T::CH;
    char* p = tile + rr * T::RB + 16 * c;
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
        const u32x4 v = r.v[it];
        *reinterpret_cast<u32x4*>(p + it * T::RPI * T::RB) = v;
    }
}

// A tile's 32 rows of 256 (fp16) or 512 (fp32) bytes copied into LDS by the
// gfx950 direct-to-LDS buffer load (16 bytes per lane), without registers:
// rows unpadded, 16-byte chunk c of row v at position c ^ (v & 15).
// Instruction it fills the kilobyte at 1024 it (rows RPI it ..): lane l
// writes position l % CH of row RPI it + l / CH and reads the chunk that
// belongs there.  Rows at or beyond n read as zero.  The copy is
// asynchronous: tile2_dma_wait() before the tile is read.
typedef __attribute__((address_space(3))) void lds_void_t;
template <bool F16>
__device__ __forceinline__ void tile2_dma(const char* __restrict__ src, int64_t ld_bytes, int64_t base, int64_t n,
                                          char* tile, int l) {
    using T = Tile2Shape<F16>;
    const rsrc_t rs = make_rsrc(src + base * ld_bytes, tile2_range(n - base, ld_bytes));
    const int rr = l / T::CH, p = l % T::CH;
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
        const int row = T::RPI * it + rr;
        const uint32_t voff = static_cast<uint32_t>(row) * static_cast<uint32_t>(ld_bytes) +
                              static_cast<uint32_t>(16 * (p ^ (row & 15)));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + 1024 * it), 16, voff, 0, 0, kNonTemporal);
    }
}
// Waits until this wave's LDS reads have returned (before a copy overwrites
// what they read).
__device__ __forceinline__ void lds_reads_done() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
}
// Waits for this wave's outstanding vector-memory operations, the tile copy
// among them.
__device__ __forceinline__ void tile2_dma_wait() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    wave_lds_sync();
}

// Writes the tile's 32 rows from LDS; each group of four 16-byte reads is
// followed by its four stores with nothing in between.
template <bool F16>
__device__ __forceinline__ void tile2_store(char* __restrict__ dst, int64_t ld_bytes, int64_t base, int64_t n,
                                            const char* __restrict__ tile, int l) {
    using T = Tile2Shape<F16>;
    const int rr = l / T::CH, c = l % T::CH;
    const uint32_t voff = static_cast<uint32_t>(rr) * static_cast<uint32_t>(ld_bytes) + static_cast<uint32_t>(16 * c);
    const rsrc_t rs = make_rsrc(dst + base * ld_bytes, tile2_range(n - base, ld_bytes));
    const int step = static_cast<int>(T::RPI * ld_bytes);
    const char* p = tile + rr * T::RB + 16 * c;
    wave_lds_sync();
#pragma unroll
    for (int b = 0; b < T::IT; b += 4) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const u32x4*>(p + (b + k) * T::RPI * T::RB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rs, voff, (b + k) * step, kNonTemporal);
        store_data_fence();
    }
}

// Record rows of WORDS dwords per vector, a tile's 32 rows contiguous:
// copied through the stage (row-major, WORDS dwords per vector).  The range
// is exact, so the last partial instruction of an odd WORDS stays inside
// the tile.
template <int WORDS>
__device__ __forceinline__ void words2_store(uint32_t* __restrict__ dst, int64_t base, int64_t n,
                                             const uint32_t* __restrict__ stage, int l) {
    const int64_t rows = n - base < 32 ? n - base : 32;
    const rsrc_t rs = make_rsrc(dst + base * WORDS, static_cast<uint32_t>(rows * 4 * WORDS));
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < (32 * WORDS + 63) / 64; ++it) {
        const uint32_t v = stage[it * 64 + l];
        __builtin_amdgcn_raw_buffer_store_b32(v, rs, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    }
}
template <int WORDS>
__device__ __forceinline__ void words2_load(const uint32_t* __restrict__ src, int64_t base, int64_t n,
                                            uint32_t* __restrict__ stage, int l) {
    const int64_t rows = n - base < 32 ? n - base : 32;
    const rsrc_t rs = make_rsrc(src + base * WORDS, static_cast<uint32_t>(rows * 4 * WORDS));
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < (32 * WORDS + 63) / 64; ++it)
        stage[it * 64 + l] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<uint32_t>(4 * l), 256 * it, kNonTemporal);
    wave_lds_sync();
}

// One 16-bit value per vector; both lanes of a vector store the same value.
__device__ __forceinline__ void half_store2(uint16_t* __restrict__ dst, int64_t base, int64_t n, uint32_t v, int vi) {
    const rsrc_t rs = make_rsrc(dst + base, tile2_range(n - base, 2));
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v), rs, static_cast<uint32_t>(2 * vi), 0, kNonTemporal);
}
__device__ __forceinline__ uint32_t half_load2(const uint16_t* __restrict__ src, int64_t base, int64_t n, int vi) {
    const rsrc_t rs = make_rsrc(src + base, tile2_range(n - base, 2));
    return __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<uint32_t>(2 * vi), 0, kNonTemporal);
}

// Output slots 2 k and 2 k + 1 (pair k of the lane's part of its LDS row,
// rowo).  fp16 output is the rounding of the materialised fp32 value.
template <bool F16>
__device__ __forceinline__ void out_pair(char* rowo, int k, float a, float b) {
    if constexpr (F16) {
        pin(a);
        pin(b);
        *reinterpret_cast<uint32_t*>(rowo + 4 * k) = cvt_pk(a, b);
    } else {
        *reinterpret_cast<f32x2*>(rowo + 8 * k) = f32x2{a, b};
    }
}

}  // namespace rqk
