// moe_mxfp4.hip -- MXFP4 instances of the expert-indexed MoE GEMV (moe_impl.hpp).
#include "moe_impl.hpp"

namespace mxq {

bool launch_moe_mxfp4(const MoeArgs& a, hipStream_t st) {
    return launch_moe_cb<kMXFP4, 16>(a, st);
}

}  // namespace mxq
