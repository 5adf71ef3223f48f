// Declarations of the rotor kernel variants instantiated in rq_rotor_inst.hip.
#pragma once

#include "rq_kernels.h"

namespace rqk {

struct RotorDev {
    const float* __restrict__ rotmat;
    const float* __restrict__ rotmat16;
    const float* __restrict__ cent;
    const u32x4_t* __restrict__ bins;
    const uint16_t* __restrict__ s_fwd;
    const uint16_t* __restrict__ s_back;
    float bin_a, bin_b;
    float qjl_scale;
};

template <int B, bool QJL>
hipError_t launch_quant_b(const RotorDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n, uint32_t* codes,
                          uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16, int64_t ldy_bytes,
                          bool roundtrip, hipStream_t s);
template <int B, bool QJL>
hipError_t launch_dequant_b(const RotorDev& P, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                            const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes, hipStream_t s);

}  // namespace rqk
