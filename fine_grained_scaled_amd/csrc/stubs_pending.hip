// Launchers whose kernels are not written yet: they report "unsupported".
#include "fgs_internal.h"
namespace fgs {
hipError_t launch_gemm_nvfp4(const GemmArgs&, hipStream_t) { return hipErrorNotSupported; }
}
