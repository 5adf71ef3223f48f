// One (bits, QJL) variant of the dense kernels per translation unit.
#include "rq_dense_codec_dev.h"

namespace rqk {
template hipError_t launch_tq_quant<RQ_B, RQ_QJL>(const DenseDev&, const void*, bool, int64_t, int64_t, uint32_t*,
                                                  uint16_t*, uint32_t*, uint16_t*, void*, bool, int64_t, bool,
                                                  hipStream_t);
template hipError_t launch_tq_dequant<RQ_B, RQ_QJL>(const DenseDev&, const uint32_t*, const uint16_t*,
                                                    const uint32_t*, const uint16_t*, int64_t, void*, bool, int64_t,
                                                    hipStream_t);
}  // namespace rqk
