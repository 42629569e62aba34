// kernels_q2.hip -- instantiates the 2-bit layer (one token and grouped), expert and
// matvec kernels.
#include "grouped_kernels.h"

namespace fmoe {
namespace dev {
template hipError_t qmatvec_b<2>(const uint8_t *, int, int, const float *, float *, hipStream_t);
template hipError_t gateup_b<2>(const uint8_t *, int, int, const float *, float *, hipStream_t);
template hipError_t layer_b<2>(const LayerArgs &, hipStream_t, int);
template hipError_t layer_ptr_b<2>(const LayerArgs &, hipStream_t, int);
template hipError_t group_b<2>(const GroupArgs &, hipStream_t, int);
template hipError_t group_route_b<2>(const GroupArgs &, hipStream_t);
template hipError_t group_experts_b<2>(const GroupArgs &, hipStream_t);
}  // namespace dev
}  // namespace fmoe
