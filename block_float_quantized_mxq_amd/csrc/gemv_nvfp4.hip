// gemv_nvfp4.hip -- NVFP4 instances of the dense GEMV (gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace mxq {

bool launch_gemv_nvfp4(const GemvArgs& a, const GemvConfig& cfg, hipStream_t st) {
    if (code_bytes_per_row(kNVFP4, a.k) % 16 == 0) return launch_gemv_cb<kNVFP4, 16>(a, cfg, st);
    return launch_gemv_cb<kNVFP4, 8>(a, cfg, st);  // rows of 8 * odd bytes
}

}  // namespace mxq
