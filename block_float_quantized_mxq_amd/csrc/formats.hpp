// formats.hpp -- format tags and row geometry shared by host and device code.
#pragma once

#include <stdint.h>

namespace mxq {

// Values match mxq_format_t in include/mxq.h.
enum : int { kMXFP4 = 1, kMXFP8 = 2, kNVFP4 = 3 };

// Bytes of packed codes in one weight row of k elements.
__host__ __device__ constexpr int64_t code_bytes_per_row(int fmt, int64_t k) { return fmt == kMXFP8 ? k : k / 2; }
// Elements sharing one block scale.
__host__ __device__ constexpr int block_elems(int fmt) { return fmt == kNVFP4 ? 16 : 32; }

}  // namespace mxq
