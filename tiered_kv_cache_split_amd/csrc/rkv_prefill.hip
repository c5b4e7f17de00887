// placeholder until the MFMA prefill kernel lands
#include "rkv_internal.h"
namespace rkv {
int prefill_rows_per_block() { return 128; }
int prefill_keys_per_iter() { return 64; }
hipError_t launch_prefill_segment(const SegParams &, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace rkv
