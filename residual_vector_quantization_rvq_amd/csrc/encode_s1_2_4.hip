// encode_s1_2_4.hip -- encoder instantiations for stage counts 1, 2, 4 (one unit per group so they compile in parallel).
#include "encode_impl.h"

namespace rvq {
template hipError_t launch_stage_count<1>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
template hipError_t launch_stage_count<2>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
template hipError_t launch_stage_count<4>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
}  // namespace rvq
