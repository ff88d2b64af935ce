// encode_s18.hip -- encoder instantiations for stage counts 18 (one unit per group so they compile in parallel).
#include "encode_impl.h"

namespace rvq {
template hipError_t launch_stage_count<18>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
}  // namespace rvq
