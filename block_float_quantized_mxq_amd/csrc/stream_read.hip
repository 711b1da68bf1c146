// stream_read.hip -- the achievable-bandwidth reference for the GEMV kernels:
// a plain streaming read of a byte range, 16 bytes per lane per load with the
// nontemporal hint (as the GEMV reads its codes), on a persistent grid of 8
// workgroups per compute unit.  Two layouts: lanes interleaved over the whole
// range with 4 loads in flight per lane (best for ranges of tens of MB), or one
// contiguous range per workgroup with 16 loads in flight per lane (best from
// about a hundred MB; on MI355X 6.7-6.8 TB/s over 1 GiB).  The loaded words are
// XOR-folded and one word per workgroup is stored, so the loads cannot be
// dropped.  Decode time is bounded by how fast weights stream from memory
// ("The memory wall" section of the "MLxcel 0.8 release" post, slide 15 of the
// talk); this kernel measures that bound for a given byte count.
#include "kernels.hpp"
#include "rows_core.hpp"

namespace mxq {

template <bool CONTIGUOUS>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
    constexpr int U = CONTIGUOUS ? 16 : 4;
    uint32_t acc = 0;
    int64_t i, end, stride;
    if constexpr (CONTIGUOUS) {
        const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
        const int64_t b0 = (int64_t)blockIdx.x * per;
        i = b0 + threadIdx.x;
        end = b0 + per < n16 ? b0 + per : n16;
        stride = 256;
    } else {
        i = (int64_t)blockIdx.x * 256 + threadIdx.x;
        end = n16;
        stride = (int64_t)gridDim.x * 256;
    }
    for (; i + (U - 1) * stride < end; i += U * stride) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < end; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // one word per workgroup: the fold of its lanes (order does not matter for XOR)
    __shared__ uint32_t part[4];
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

bool launch_stream_read(const void* p, int64_t bytes, uint32_t* sink, int64_t workgroups, int contiguous,
                        hipStream_t st) {
    const auto kernel = contiguous ? stream_read_kernel<true> : stream_read_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)workgroups), dim3(256), 0, st, reinterpret_cast<const u32x4_t*>(p),
                       bytes / 16, sink);
    return true;
}

}  // namespace mxq
