// Choice of the outlier channels of QJL-only keys (rq_outlier_channels): per
// head, the k channels with the largest mean |x_j| over the head's keys, a
// tie going to the lower channel, listed in increasing order (README "CUDA
// Kernels": the 1-bit QJL quantiser separates outliers; the blog's Lemma-1
// section and the podcast page: LLM vectors carry very large outliers).
//
// One workgroup per head.  Thread t reads the 16-byte chunk t % 16 (eight
// channels) of rows t / 16, t / 16 + 16, ... and keeps eight fp32 sums of
// |x| in a fixed order; the sixteen row-phase partials of each channel are
// then added in a fixed order in LDS, so the sums (and the choice) are
// deterministic.  Each channel finds its rank among the 128 sums and its
// position among the chosen channels by counting.
#include "rq_common_dev.h"
#include "rq_kernels.h"

namespace rqk {

template <bool IN_F16>
__global__ __launch_bounds__(256) void outlier_select_kernel(const char* __restrict__ x, int64_t head_rows,
                                                             int64_t ldx_bytes, int k, uint8_t* __restrict__ chans) {
    __shared__ float part[16][kD + 4];
    __shared__ float sum[kD];
    __shared__ int chosen[kD];
    const int t = threadIdx.x;
    const int c8 = t & 15, r0 = t >> 4;
    const char* base = x + static_cast<int64_t>(blockIdx.x) * head_rows * ldx_bytes;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (IN_F16) {
        for (int64_t r = r0; r < head_rows; r += 16) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(base + r * ldx_bytes + 16 * c8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = v[e];
                acc[2 * e] += fabsf(h2f(w & 0xFFFFu));
                acc[2 * e + 1] += fabsf(h2f(w >> 16));
            }
        }
    } else {
        for (int64_t r = r0; r < head_rows; r += 16) {
            const float* row = reinterpret_cast<const float*>(base + r * ldx_bytes) + 8 * c8;
            const float4 a = *reinterpret_cast<const float4*>(row);
            const float4 b = *reinterpret_cast<const float4*>(row + 4);
            acc[0] += fabsf(a.x);
            acc[1] += fabsf(a.y);
            acc[2] += fabsf(a.z);
            acc[3] += fabsf(a.w);
            acc[4] += fabsf(b.x);
            acc[5] += fabsf(b.y);
            acc[6] += fabsf(b.z);
            acc[7] += fabsf(b.w);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][8 * c8 + e] = acc[e];
    __syncthreads();
    if (t < kD) {
        float s = 0.0f;
        for (int p = 0; p < 16; ++p) s += part[p][t];
        sum[t] = s;
    }
    __syncthreads();
    if (t < kD) {
        const float me = sum[t];
        int rank = 0;
        for (int j = 0; j < kD; ++j) {
            const float o = sum[j];
            rank += (o > me || (o == me && j < t)) ? 1 : 0;
        }
        chosen[t] = rank < k ? 1 : 0;
    }
    __syncthreads();
    if (t < kD && chosen[t]) {
        int pos = 0;
        for (int j = 0; j < t; ++j) pos += chosen[j];
        chans[static_cast<int64_t>(blockIdx.x) * k + pos] = static_cast<uint8_t>(t);
    }
}

hipError_t outlier_select(const void* x, bool in_f16, int64_t heads, int64_t head_rows, int64_t ldx_bytes, int k,
                          uint8_t* chans, hipStream_t s) {
    if (heads == 0 || k == 0) return hipSuccess;
    const char* xc = static_cast<const char*>(x);
    if (in_f16)
        hipLaunchKernelGGL((outlier_select_kernel<true>), dim3(static_cast<unsigned>(heads)), dim3(256), 0, s, xc,
                           head_rows, ldx_bytes, k, chans);
    else
        hipLaunchKernelGGL((outlier_select_kernel<false>), dim3(static_cast<unsigned>(heads)), dim3(256), 0, s, xc,
                           head_rows, ldx_bytes, k, chans);
    return hipGetLastError();
}

}  // namespace rqk
