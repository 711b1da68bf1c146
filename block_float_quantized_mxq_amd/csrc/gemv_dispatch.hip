// gemv_dispatch.hip -- routes a dense GEMV to its format's instances.
#include <cstdlib>

#include "kernels.hpp"

namespace mxq {

bool launch_gemv_mxfp4(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st);
bool launch_gemv_mxfp8(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st);
bool launch_gemv_nvfp4(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st);

bool launch_gemv(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    switch (a.fmt) {
        case kMXFP4: return launch_gemv_mxfp4(a, cfg, st);
        case kMXFP8: return launch_gemv_mxfp8(a, cfg, st);
        case kNVFP4: return launch_gemv_nvfp4(a, cfg, st);
    }
    return false;
}

}  // namespace mxq
