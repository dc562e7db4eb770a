#include "common.hpp"
#include "fa_kernels.hpp"
namespace fa355 {
hipError_t launch_backward(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}
