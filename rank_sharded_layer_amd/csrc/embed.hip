// Vocab-parallel masked embedding gather for one rank.
//
// out[i, :] = table_shard[ids[i] - start, :] when start <= ids[i] < end and
// +0.0 otherwise (vLLM source analysis 13, §2.4.1; "Tensor parallelism:
// implemented from scratch", VocabParallelEmbedding.forward).
//
// One 64-lane wavefront per token row.  The id is loaded once per wave (a
// uniform scalar load) and the in-shard test is therefore wave-uniform: a
// masked row is written with zero stores and the table is never touched.
// Rows move as 16-byte vectors when the row length and both base addresses
// allow it, else element by element.  Bit-exact.
#include "common.hpp"

namespace tpk {

template <typename U>
__global__ __launch_bounds__(256) void vocab_embed_kernel(const int64_t* __restrict__ ids,
                                                          int64_t n,
                                                          const uint8_t* __restrict__ table,
                                                          int64_t start, int64_t end,
                                                          int64_t row_units,
                                                          uint8_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    // the wave index is uniform across the wave: make that explicit so the id
    // load and the in-shard branch are scalar
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t i = wave; i < n; i += nwaves) {
        const int64_t id = ids[i];
        U* dst = reinterpret_cast<U*>(out) + i * row_units;
        if (id >= start && id < end) {
            const U* src = reinterpret_cast<const U*>(table) + (id - start) * row_units;
            for (int64_t j = lane; j < row_units; j += 64) dst[j] = src[j];
        } else {
            U z;
            __builtin_memset(&z, 0, sizeof(U));
            for (int64_t j = lane; j < row_units; j += 64) dst[j] = z;
        }
    }
}

template <typename U>
static hipError_t launch_unit(const int64_t* ids, int64_t n, const void* table, int64_t start,
                              int64_t end, int64_t row_bytes, void* out, hipStream_t s) {
    const int64_t units = row_bytes / (int64_t)sizeof(U);
    int64_t blocks = ceil_div(n, 4);
    if (blocks > 65535) blocks = 65535;
    hipLaunchKernelGGL(vocab_embed_kernel<U>, dim3((unsigned)blocks), dim3(256), 0, s, ids, n,
                       static_cast<const uint8_t*>(table), start, end, units,
                       static_cast<uint8_t*>(out));
    return hipGetLastError();
}

hipError_t launch_vocab_embed(const int64_t* ids, int64_t n, const void* table, int64_t start,
                              int64_t end, int64_t h, int esize, void* out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t row_bytes = h * esize;
    uint64_t g = (uint64_t)(uintptr_t)table | (uint64_t)(uintptr_t)out | (uint64_t)row_bytes;
    if ((g & 15u) == 0) return launch_unit<uint4>(ids, n, table, start, end, row_bytes, out, s);
    if ((g & 3u) == 0) return launch_unit<uint32_t>(ids, n, table, start, end, row_bytes, out, s);
    return launch_unit<uint16_t>(ids, n, table, start, end, row_bytes, out, s);
}

}  // namespace tpk
