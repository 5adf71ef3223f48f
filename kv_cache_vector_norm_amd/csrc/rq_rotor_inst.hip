// One (bits, QJL) variant of the rotor kernels per translation unit, so the
// variants build in parallel.  RQ_B and RQ_QJL are set by the build.
#include "rq_rotor_codec_dev.h"

namespace rqk {
template hipError_t launch_quant_b<RQ_B, RQ_QJL>(const RotorDev&, const void*, bool, int64_t, int64_t, uint32_t*,
                                                 uint16_t*, uint32_t*, uint16_t*, void*, bool, int64_t, bool,
                                                 hipStream_t);
template hipError_t launch_dequant_b<RQ_B, RQ_QJL>(const RotorDev&, const uint32_t*, const uint16_t*,
                                                   const uint32_t*, const uint16_t*, int64_t, void*, bool, int64_t,
                                                   hipStream_t);
}  // namespace rqk
