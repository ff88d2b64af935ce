// encode_s20.hip -- encoder instantiations for stage counts 20 (one unit per group so they compile in parallel).
#include "encode_impl.h"

namespace rvq {
template hipError_t launch_stage_count<20>(const EncodePlan &, const EncodeArgs &, hipEvent_t *,
                                            hipStream_t);
}  // namespace rvq
