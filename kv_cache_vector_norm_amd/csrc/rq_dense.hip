// Dispatch of dense-session (TurboQuant) calls to the (bits, QJL) variants.
#include "rq_dense_dev.h"

namespace rqk {

template <int B, bool QJL>
hipError_t launch_tq_quant(const DenseDev& P, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                           uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                           int64_t ldy_bytes, bool roundtrip, hipStream_t s);
template <int B, bool QJL>
hipError_t launch_tq_dequant(const DenseDev& P, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                             const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                             hipStream_t s);

static DenseDev make_dense(const DenseTables& t) {
    DenseDev P;
    P.pi_hi = t.pi_hi;
    P.pi_lo = t.pi_lo;
    P.pit_hi = t.pit_hi;
    P.pit_lo = t.pit_lo;
    P.pi2_hi = t.pi2_hi;
    P.pi2_lo = t.pi2_lo;
    P.pit2_hi = t.pit2_hi;
    P.pit2_lo = t.pit2_lo;
    P.t2_hi = t.t2_hi;
    P.t2_lo = t.t2_lo;
    P.s_back = t.s_back;
    P.thr = t.thr;
    P.cent = t.cent;
    P.s_rows = t.s_rows;
    P.s_cols = t.s_cols;
    P.bins = t.bins;
    P.bin_a = t.bin_a;
    P.bin_b = t.bin_b;
    P.qjl_scale = t.qjl_scale;
    return P;
}

hipError_t dense_quantize(const DenseTables& t, const void* x, bool in_f16, int64_t ldx_bytes, int64_t n,
                          uint32_t* codes, uint16_t* norms, uint32_t* signs, uint16_t* rnorms, void* y, bool out_f16,
                          int64_t ldy_bytes, bool roundtrip, hipStream_t s) {
    const DenseDev P = make_dense(t);
#define TQ_CASE(BB, Q)                                                                                              \
    return launch_tq_quant<BB, Q>(P, x, in_f16, ldx_bytes, n, codes, norms, signs, rnorms, y, out_f16, ldy_bytes, \
                                  roundtrip, s)
    if (t.qjl) {
        switch (t.mse_bits) {
            case 1: TQ_CASE(1, true);
            case 2: TQ_CASE(2, true);
            case 3: TQ_CASE(3, true);
            case 4: TQ_CASE(4, true);
        }
    } else {
        switch (t.mse_bits) {
            case 1: TQ_CASE(1, false);
            case 2: TQ_CASE(2, false);
            case 3: TQ_CASE(3, false);
            case 4: TQ_CASE(4, false);
        }
    }
#undef TQ_CASE
    return hipErrorInvalidValue;
}

hipError_t dense_dequantize(const DenseTables& t, const uint32_t* codes, const uint16_t* norms, const uint32_t* signs,
                            const uint16_t* rnorms, int64_t n, void* y, bool out_f16, int64_t ldy_bytes,
                            hipStream_t s) {
    const DenseDev P = make_dense(t);
#define TQ_CASE(BB, Q) return launch_tq_dequant<BB, Q>(P, codes, norms, signs, rnorms, n, y, out_f16, ldy_bytes, s)
    if (t.qjl) {
        switch (t.mse_bits) {
            case 1: TQ_CASE(1, true);
            case 2: TQ_CASE(2, true);
            case 3: TQ_CASE(3, true);
            case 4: TQ_CASE(4, true);
        }
    } else {
        switch (t.mse_bits) {
            case 1: TQ_CASE(1, false);
            case 2: TQ_CASE(2, false);
            case 3: TQ_CASE(3, false);
            case 4: TQ_CASE(4, false);
        }
    }
#undef TQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace rqk
