// Shard selection: a strided 2-D byte copy (narrow along dim 0 or dim 1).
//
// Load-time work, bit-exact.  Each workgroup copies whole rows; within a row
// the 64-lane wavefronts move the widest unit (16, 8, 4, 2 or 1 bytes) that
// divides the row length, both leading dimensions and both base addresses,
// so a row of bf16 weights is read and written with 16-byte vector accesses.
#include "common.hpp"

namespace tpk {

template <typename U>
__global__ __launch_bounds__(256) void copy2d_kernel(const uint8_t* __restrict__ src,
                                                     int64_t src_ld, uint8_t* __restrict__ dst,
                                                     int64_t dst_ld, int64_t rows,
                                                     int64_t row_units) {
    // grid: x over units within a row (blockDim-wide strips), y over rows
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const U* s = reinterpret_cast<const U*>(src + r * src_ld);
        U* d = reinterpret_cast<U*>(dst + r * dst_ld);
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < row_units;
             i += (int64_t)gridDim.x * blockDim.x)
            d[i] = s[i];
    }
}

template <typename U>
static hipError_t launch_unit(const void* src, int64_t src_ld, void* dst, int64_t dst_ld,
                              int64_t rows, int64_t row_bytes, hipStream_t s) {
    int64_t units = row_bytes / (int64_t)sizeof(U);
    int64_t gx = ceil_div(units, 256);
    if (gx > 1024) gx = 1024;
    int64_t gy = rows < 65535 ? rows : 65535;
    // keep the total number of workgroups bounded but >= a few per CU
    while (gx * gy > (int64_t)1 << 20 && gy > 1) gy = (gy + 1) / 2;
    hipLaunchKernelGGL(copy2d_kernel<U>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s,
                       static_cast<const uint8_t*>(src), src_ld, static_cast<uint8_t*>(dst),
                       dst_ld, rows, units);
    return hipGetLastError();
}

hipError_t launch_copy2d(const void* src, int64_t src_ld, void* dst, int64_t dst_ld,
                         int64_t rows, int64_t row_bytes, hipStream_t s) {
    if (rows <= 0 || row_bytes <= 0) return hipSuccess;
    uint64_t g = (uint64_t)(uintptr_t)src | (uint64_t)(uintptr_t)dst | (uint64_t)src_ld |
                 (uint64_t)dst_ld | (uint64_t)row_bytes;
    if ((g & 15u) == 0) return launch_unit<uint4>(src, src_ld, dst, dst_ld, rows, row_bytes, s);
    if ((g & 7u) == 0) return launch_unit<uint2>(src, src_ld, dst, dst_ld, rows, row_bytes, s);
    if ((g & 3u) == 0) return launch_unit<uint32_t>(src, src_ld, dst, dst_ld, rows, row_bytes, s);
    if ((g & 1u) == 0) return launch_unit<uint16_t>(src, src_ld, dst, dst_ld, rows, row_bytes, s);
    return launch_unit<uint8_t>(src, src_ld, dst, dst_ld, rows, row_bytes, s);
}

}  // namespace tpk
