// Stand-ins for libtq's kernel launchers, linked only into the host-code
// sanitizer build (AddressSanitizer and UndefinedBehaviorSanitizer on
// abi.cpp and codebook.cpp, built with the host compiler).  Each reports
// "no device", so a call that passes every argument check returns TQ_ERR_HIP
// and nothing else of the library runs; the checks, the descriptor and
// parameter handling, the split choices and the codebook builder run as in
// the real library.  Test infrastructure: the product library never links
// this file.
#include "tq_common.h"

namespace tq {

hipError_t launch_quantize_append(const QuantizeParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quantize_mfma(const QuantizeParams &, hipStream_t) { return hipErrorNoDevice; }
float quantize_lut_scale(const float *, int) { return 0.0f; }
hipError_t launch_dequantize(const DequantParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_read_probe(const void *, size_t, unsigned *, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_zero_fill(void *, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t scratch_workspace(hipStream_t, void **) { return hipErrorNoDevice; }
hipError_t launch_decode_ref(const DecodeParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_mfma(const DecodeParams &, hipStream_t) { return hipErrorNoDevice; }

}  // namespace tq
