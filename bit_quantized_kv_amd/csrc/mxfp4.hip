// MX-FP4 quantize and decode kernels for gfx950 (filled in below).
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

hipError_t launch_mxfp4_quantize(const QuantizeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mxfp4_decode(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace tq
