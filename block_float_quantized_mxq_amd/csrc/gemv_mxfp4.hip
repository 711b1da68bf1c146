// gemv_mxfp4.hip -- MXFP4 instances of the dense GEMV (gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace mxq {

bool launch_gemv_mxfp4(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    return launch_gemv_cb<kMXFP4, 16>(a, cfg, st);
}

}  // namespace mxq
