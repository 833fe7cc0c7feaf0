// placeholder: replaced by the decode kernels
#include "kernels.h"
namespace mxattn {
hipError_t launch_decode(const DecodeArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}
