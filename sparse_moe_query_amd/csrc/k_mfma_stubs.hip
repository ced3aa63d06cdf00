// Placeholder launchers until the matrix-core kernels are in place.
#include "gqe_common.h"
#include "gqe_internal.h"

hipError_t launch_proj_mfma(const GqeDims&, const WorkPlan&, const void*, const void*, const PackedLayout&, char*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_combine_mfma(const GqeDims&, const WorkPlan&, const void*, const PackedLayout&, void*, char*, hipStream_t) {
    return hipErrorNotSupported;
}
