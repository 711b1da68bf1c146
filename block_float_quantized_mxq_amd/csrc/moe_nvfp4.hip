// moe_nvfp4.hip -- NVFP4 instances of the expert-indexed MoE GEMV (moe_impl.hpp).
#include "moe_impl.hpp"

namespace mxq {

bool launch_moe_nvfp4(const MoeArgs& a, hipStream_t st) {
    return (code_bytes_per_row(kNVFP4, a.k) % 16) == 0 ? launch_moe_cb<kNVFP4, 16>(a, st)
                                                        : launch_moe_cb<kNVFP4, 8>(a, st);
}

}  // namespace mxq
