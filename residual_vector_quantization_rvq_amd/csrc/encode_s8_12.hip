// encode_s8_12.hip -- encoder instantiations for stage counts 8, 12 (one unit per group so they compile in parallel).
#include "encode_impl.h"

namespace rvq {
template hipError_t launch_stage_count<8>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
template hipError_t launch_stage_count<12>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
}  // namespace rvq
