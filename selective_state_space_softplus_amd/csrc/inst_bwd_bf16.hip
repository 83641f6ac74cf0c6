// The scan_bwd launchers for bf16 inputs, one per launch shape.
#include "launch_bwd.h"

namespace ss_host {
template int launch_bwd<uint16_t, 1, 2>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<uint16_t, 4, 2>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<uint16_t, 8, 2>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<uint16_t, 8, 4>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<uint16_t, 8, 8>(ss::BwdParams, bool, bool, hipStream_t, int*);
}  // namespace ss_host
