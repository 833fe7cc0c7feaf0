// placeholder: replaced by the selection kernels
#include "kernels.h"
namespace mxattn {
hipError_t launch_select(const SelectArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}
