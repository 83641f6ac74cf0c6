// The scan_bwd launchers for f32 inputs, one per launch shape.
#include "launch_bwd.h"

namespace ss_host {
template int launch_bwd<float, 1, 2>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<float, 4, 2>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<float, 8, 2>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<float, 8, 4>(ss::BwdParams, bool, bool, hipStream_t, int*);
template int launch_bwd<float, 8, 8>(ss::BwdParams, bool, bool, hipStream_t, int*);
}  // namespace ss_host
