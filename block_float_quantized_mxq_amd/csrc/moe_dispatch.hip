// moe_dispatch.hip -- routes an MoE GEMV to its format's instances.
#include "kernels.hpp"

namespace mxq {

bool launch_moe_mxfp4(const MoeArgs& a, hipStream_t st);
bool launch_moe_mxfp8(const MoeArgs& a, hipStream_t st);
bool launch_moe_nvfp4(const MoeArgs& a, hipStream_t st);

bool launch_moe(const MoeArgs& a, hipStream_t st) {
    switch (a.fmt) {
        case kMXFP4: return launch_moe_mxfp4(a, st);
        case kMXFP8: return launch_moe_mxfp8(a, st);
        case kNVFP4: return launch_moe_nvfp4(a, st);
    }
    return false;
}

}  // namespace mxq
