// kernels_q4.hip -- instantiates the 4-bit layer (one token and grouped), expert and
// matvec kernels.
#include "grouped_kernels.h"

namespace fmoe {
namespace dev {
template hipError_t qmatvec_b<4>(const uint8_t *, int, int, const float *, float *, hipStream_t);
template hipError_t gateup_b<4>(const uint8_t *, int, int, const float *, float *, hipStream_t);
template hipError_t layer_b<4>(const LayerArgs &, hipStream_t, int);
template hipError_t layer_ptr_b<4>(const LayerArgs &, hipStream_t, int);
template hipError_t route1_b<4>(const float *, int, int, int32_t *, float *, hipStream_t);
template hipError_t group_b<4>(const GroupArgs &, hipStream_t, int);
template hipError_t group_route_b<4>(const GroupArgs &, hipStream_t);
template hipError_t group_experts_b<4>(const GroupArgs &, hipStream_t);
}  // namespace dev
}  // namespace fmoe
