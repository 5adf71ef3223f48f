// Kernels of the paged compressed KV cache (rq_cache_* in rq.h): moving
// freshly quantised record rows into their pages, and folding the current
// token's exact key and value into an attention result over the cache.
#include "rq_common_dev.h"
#include "rq_kernels.h"

namespace rqk {

// Row i of head j's block of `n` dense rows <-> key position t0 + i of head
// j in its page pages[j * stride + (t0 + i) >> shift], slot (t0 + i) & mask;
// dense -> pages (append) or pages -> dense (read back).
struct ScatterArgs {
    const uint32_t* src_codes;
    const uint16_t* src_norms;
    const uint32_t* src_signs;
    const uint16_t* src_rnorms;
    uint32_t* dst_codes;
    uint16_t* dst_norms;
    uint32_t* dst_signs;
    uint16_t* dst_rnorms;
    int words;                // code words per row (0 for QJL-only records)
    bool qjl;
    int64_t n, t0;
    int heads;
    const int32_t* pages;
    int shift;
    int64_t stride;
    bool gather;              // pages -> dense rows instead
};

__global__ __launch_bounds__(256) void scatter_rows_kernel(ScatterArgs a) {
    const int64_t idx = blockIdx.x * 256LL + threadIdx.x;
    if (idx >= a.n * a.heads) return;
    const int j = static_cast<int>(idx / a.n);
    const int64_t i = idx - j * a.n;
    const int64_t key = a.t0 + i;
    const int64_t pg = a.pages[j * a.stride + (key >> a.shift)];
    const int64_t prow = (pg << a.shift) + (key & ((int64_t(1) << a.shift) - 1));
    const int64_t src = a.gather ? prow : idx;
    const int64_t dst = a.gather ? idx : prow;
    for (int w = 0; w < a.words; ++w) a.dst_codes[dst * a.words + w] = a.src_codes[src * a.words + w];
    a.dst_norms[dst] = a.src_norms[src];
    if (a.qjl) {
        for (int w = 0; w < 4; ++w) a.dst_signs[dst * 4 + w] = a.src_signs[src * 4 + w];
        a.dst_rnorms[dst] = a.src_rnorms[src];
    }
}

hipError_t scatter_rows(const uint32_t* src_codes, const uint16_t* src_norms, const uint32_t* src_signs,
                        const uint16_t* src_rnorms, uint32_t* dst_codes, uint16_t* dst_norms, uint32_t* dst_signs,
                        uint16_t* dst_rnorms, int words, bool qjl, int64_t n, int64_t t0, int heads,
                        const PageTable& pt, bool gather, hipStream_t s) {
    ScatterArgs a{src_codes, src_norms, src_signs, src_rnorms, dst_codes, dst_norms, dst_signs, dst_rnorms,
                  words,     qjl,       n,         t0,         heads,     pt.pages,  pt.shift,  pt.stride, gather};
    const int64_t total = n * heads;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// out_h over the cached keys (normalised, with row statistics (M, L) of
// scale * estimate) merged with the exact current key k and value v of KV
// head h / group: s = scale <q_h, k>,
//   out_h <- (L e^(M - M') out_h + e^(s - M') v) / (L e^(M - M') + e^(s - M')),
// M' = max(M, s).  With no cached keys (stats == nullptr) out_h = v.
struct MergeArgs {
    const float* q;
    const float* kcur;        // [kv_heads][128] fp32
    const float* vcur;
    const float2* stats;      // [hq] or nullptr
    float scale;
    int group;
    float* out;
    int64_t ld_out;
};

__global__ __launch_bounds__(128) void merge_current_kernel(MergeArgs a) {
    const int h = blockIdx.x;
    const int j = h / a.group;
    const int i = threadIdx.x;
    __shared__ float part[2];
    float d = a.q[static_cast<int64_t>(h) * kD + i] * a.kcur[static_cast<int64_t>(j) * kD + i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
    if ((i & 63) == 0) part[i >> 6] = d;
    __syncthreads();
    const float s = (part[0] + part[1]) * a.scale;
    const float v = a.vcur[static_cast<int64_t>(j) * kD + i];
    float* o = a.out + static_cast<int64_t>(h) * a.ld_out + i;
    if (a.stats == nullptr) {
        *o = v;
        return;
    }
    const float2 ml = a.stats[h];
    const float mn = fmaxf(ml.x, s);
    const float wo = ml.y * __builtin_amdgcn_exp2f((ml.x - mn) * 1.4426950408889634f);
    const float wc = __builtin_amdgcn_exp2f((s - mn) * 1.4426950408889634f);
    *o = (wo * *o + wc * v) / (wo + wc);
}

hipError_t merge_current(const float* q, int hq, int group, const float* kcur, const float* vcur,
                         const float2* stats, float scale, float* out, int64_t ld_out, hipStream_t s) {
    MergeArgs a{q, kcur, vcur, stats, scale, group, out, ld_out};
    hipLaunchKernelGGL(merge_current_kernel, dim3(hq), dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace rqk
