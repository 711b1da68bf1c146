// moe_mxfp8.hip -- MXFP8 instances of the expert-indexed MoE GEMV (moe_impl.hpp).
#include "moe_impl.hpp"

namespace mxq {

bool launch_moe_mxfp8(const MoeArgs& a, hipStream_t st) {
    return launch_moe_cb<kMXFP8, 16>(a, st);
}

}  // namespace mxq
