// Launchers replaced for the host-only sanitizer build of the C ABI: every call that
// passes validation ends here, so it returns a HIP error the driver expects to see
// (KDA_ERR_HIP) instead of touching a device.
#include "kda_launch.h"

namespace kda {

hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_spec(const SpecArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_table(const TableArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_combine(const CombineArgs&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_backward(const BackwardArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t scratch_address(void** p) {
    *p = nullptr;
    return hipErrorNotSupported;
}

}  // namespace kda
