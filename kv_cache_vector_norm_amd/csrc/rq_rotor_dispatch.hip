// Dispatch of rotor-session calls to the (bits, QJL) kernel variants.
#include "rq_rotor_decl.h"

namespace rqk {

static RotorDev make_dev(const RotorTables& t) {
    RotorDev P;
    P.rotmat = t.rotmat;
    P.rotmat16 = t.rotmat16;
    P.cent = t.cent;
    P.bins = t.bins;
    P.bin_a = t.bin_a;
    P.bin_b = t.bin_b;
    P.s_fwd = t.s_fwd;
    P.s_back = t.s_back;
    P.qjl_scale = t.qjl_scale;
    return P;
}

hipError_t rotor_quantize(const RotorTables& t, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                          int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    const RotorDev P = make_dev(t);
#define RQ_CASE(BB, Q)                                                                                              \
    return launch_quant_b<BB, Q>(P, x, in_f16, ldx_bytes, n, codes, norms, signs, rnorms, y, out_f16, ldy_bytes, \
                                 roundtrip, s)
    if (t.qjl) {
        switch (t.mse_bits) {
            case 1: RQ_CASE(1, true);
            case 2: RQ_CASE(2, true);
            case 3: RQ_CASE(3, true);
            case 4: RQ_CASE(4, true);
        }
    } else {
        switch (t.mse_bits) {
            case 1: RQ_CASE(1, false);
            case 2: RQ_CASE(2, false);
            case 3: RQ_CASE(3, false);
            case 4: RQ_CASE(4, false);
        }
    }
#undef RQ_CASE
    return hipErrorInvalidValue;
}

hipError_t rotor_dequantize(const RotorTables& t, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                            const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                            hipStream_t s) {
    const RotorDev P = make_dev(t);
#define RQ_CASE(BB, Q) return launch_dequant_b<BB, Q>(P, codes, norms, signs, rnorms, n, y, out_f16, ldy_bytes, s)
    if (t.qjl) {
        switch (t.mse_bits) {
            case 1: RQ_CASE(1, true);
            case 2: RQ_CASE(2, true);
            case 3: RQ_CASE(3, true);
            case 4: RQ_CASE(4, true);
        }
    } else {
        switch (t.mse_bits) {
            case 1: RQ_CASE(1, false);
            case 2: RQ_CASE(2, false);
            case 3: RQ_CASE(3, false);
            case 4: RQ_CASE(4, false);
        }
    }
#undef RQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace rqk
