// fp8 (OCP e4m3) softmax branch: placeholder until the e4m3 kernels land.
#include "kernels_bf16.h"

namespace hyb {

hipError_t launch_quant_fp8(const Dims&, const Bf16Args&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_softmax_fp8(const Dims&, const Bf16Args&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace hyb
