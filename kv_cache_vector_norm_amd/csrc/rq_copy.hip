// Reference copy: the practical HBM ceiling the codec kernels are measured
// against.  It moves bytes with exactly the codec's global access pattern:
// each wave reads a 16 KB block as 16 coalesced 16-byte non-temporal raw
// buffer loads (64 lanes x 16 B each), then writes it back with 16 such
// stores; the descriptor's range drops the ragged tail.
#include "rq_common_dev.h"
#include "rq_kernels.h"

namespace rqk {

constexpr int kCopyBlock = 16384;   // bytes per wave per iteration

__global__ __launch_bounds__(256) void copy_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                   int64_t bytes) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nblocks = (bytes + kCopyBlock - 1) / kCopyBlock;
    for (int64_t c = blockIdx.x * 4LL + wave; c < nblocks; c += gridDim.x * 4LL) {
        const int l = lane_id() + opaque_zero();
        const int64_t base = c * kCopyBlock;
        const int64_t left = bytes - base;
        const uint32_t range = left >= kCopyBlock ? static_cast<uint32_t>(kCopyBlock) : static_cast<uint32_t>(left);
        const rsrc_t rs = make_rsrc(src + base, range);
        const rsrc_t rd = make_rsrc(dst + base, range);
        const uint32_t voff = static_cast<uint32_t>(16 * l);
        u32x4 v[16];
#pragma unroll
        for (int it = 0; it < 16; ++it) v[it] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 1024 * it, kNonTemporal);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < 16; ++it) __builtin_amdgcn_raw_buffer_store_b128(v[it], rd, voff, 1024 * it, kNonTemporal);
        store_data_fence();
    }
}

hipError_t copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    const int64_t nblocks = (bytes + kCopyBlock - 1) / kCopyBlock;
    const int64_t want = (nblocks + 3) / 4;
    // one round of up to eight workgroups per compute unit, then grid-stride
    const int grid = static_cast<int>(want < 256 * 8 ? want : 256 * 8);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, s, static_cast<const char*>(src),
                       static_cast<char*>(dst), bytes);
    return hipGetLastError();
}

}  // namespace rqk
