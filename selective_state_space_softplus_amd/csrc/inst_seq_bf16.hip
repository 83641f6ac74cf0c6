// The scan_seq launchers for bf16 inputs, one per launch shape.
#include "launch_seq.h"

namespace ss_host {
template int launch_seq<uint16_t, 1, 2>(ss::ScanParams, SeqMode, void*, size_t, hipStream_t);
template int launch_seq<uint16_t, 4, 2>(ss::ScanParams, SeqMode, void*, size_t, hipStream_t);
template int launch_seq<uint16_t, 4, 4>(ss::ScanParams, SeqMode, void*, size_t, hipStream_t);
template int launch_seq<uint16_t, 8, 2>(ss::ScanParams, SeqMode, void*, size_t, hipStream_t);
template int launch_seq<uint16_t, 8, 4>(ss::ScanParams, SeqMode, void*, size_t, hipStream_t);
template int launch_seq<uint16_t, 8, 8>(ss::ScanParams, SeqMode, void*, size_t, hipStream_t);
}  // namespace ss_host
