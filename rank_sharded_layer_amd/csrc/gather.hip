// Full logits of the vocab-parallel LM head and the greedy next token, one
// device.
//
// Rank r's logits cover vocabulary columns [start_r, end_r) (per =
// ceil(V/t), start_r = r per, end_r = min((r+1) per, V)).  The all-gather
// concatenates them along the vocabulary and truncates to V ("Tensor
// parallelism: implemented from scratch", TPTransformer.forward; "vLLM
// source analysis 13" §2.4.2: Y = gather([Y_1, Y_2])).  The unpadded shards
// concatenate to exactly that.  The generation loop of the same page takes
// argmax of the logits: the first column holding the maximum, a NaN counting
// as larger than every number (the rule of the torch.argmax it calls).
//
// One workgroup of 1024 threads per token row.  Thread k scans 16-byte
// vectors k, k + 1024, ... of each shard in column order (4 loads in flight;
// element-wise where the shard width or the buffers do not allow vectors),
// copies them to the full row when asked, and keeps the first best
// (value, column) it sees; the 1024 candidates then meet in a fixed tree
// whose combine rule (NaN first, then the larger value, ties to the smaller
// column) is associative and commutative, so the result is the row's first
// maximum whatever the tree.  Deterministic.
#include "common.hpp"

namespace tpk {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

struct ShardPtrs {
    const float* p[TP_MAX_RANKS];
};

struct Best {
    float v;
    int64_t i;       // column, -1 = none yet
};

// a before b in the argmax order: NaN beats numbers, larger beats smaller,
// and among equals (or two NaNs) the smaller column wins
__device__ __forceinline__ bool better(const Best& a, const Best& b) {
    if (b.i < 0) return a.i >= 0;
    if (a.i < 0) return false;
    const bool an = a.v != a.v, bn = b.v != b.v;
    if (an != bn) return an;
    if (!an && a.v != b.v) return a.v > b.v;
    return a.i < b.i;
}

__device__ __forceinline__ void offer(Best& b, float v, int64_t col) {
    // columns arrive in increasing order per thread: strictly better only
    const bool vn = v != v;
    if (b.i < 0) {
        b.v = v;
        b.i = col;
    } else if (b.v == b.v && (vn || v > b.v)) {
        b.v = v;
        b.i = col;
    }
}

constexpr int GB = 1024;     // threads per row
constexpr int GU = 4;        // 16-byte loads per thread in flight

template <bool VEC>
__global__ __launch_bounds__(GB) void logits_gather_argmax_kernel(ShardPtrs shards, int t, int64_t vocab,
                                                                 int64_t per, float* __restrict__ full,
                                                                 int64_t* __restrict__ argmax) {
    __shared__ float sv[GB];
    __shared__ int64_t si[GB];
    const int64_t row = blockIdx.x;
    Best b{0.0f, -1};
    for (int r = 0; r < t; ++r) {
        const int64_t start = (int64_t)r * per;
        int64_t end = start + per;
        if (end > vocab) end = vocab;
        if (end <= start) break;                       // trailing empty shards
        const int64_t w = end - start;
        const float* src = shards.p[r] + row * w;
        float* dst = full ? full + row * vocab + start : nullptr;
        if (VEC) {
            // GU independent vectors per thread per pass (columns still
            // increase per thread, so offer() keeps the first maximum)
            const f32x4v* s4 = reinterpret_cast<const f32x4v*>(src);
            f32x4v* d4 = reinterpret_cast<f32x4v*>(dst);
            const int64_t nv = w / 4;
            int64_t v = threadIdx.x;
            for (; v + (GU - 1) * GB < nv; v += GU * GB) {
                f32x4v x[GU];
#pragma unroll
                for (int u = 0; u < GU; ++u) x[u] = __builtin_nontemporal_load(s4 + v + u * GB);
#pragma unroll
                for (int u = 0; u < GU; ++u) {
                    if (dst) __builtin_nontemporal_store(x[u], d4 + v + u * GB);
                    const int64_t c = start + (v + u * GB) * 4;
                    offer(b, x[u].x, c);
                    offer(b, x[u].y, c + 1);
                    offer(b, x[u].z, c + 2);
                    offer(b, x[u].w, c + 3);
                }
            }
            for (; v < nv; v += GB) {
                const f32x4v x = __builtin_nontemporal_load(s4 + v);
                if (dst) __builtin_nontemporal_store(x, d4 + v);
                const int64_t c = start + v * 4;
                offer(b, x.x, c);
                offer(b, x.y, c + 1);
                offer(b, x.z, c + 2);
                offer(b, x.w, c + 3);
            }
        } else {
            for (int64_t j = threadIdx.x; j < w; j += GB) {
                const float x = src[j];
                if (dst) dst[j] = x;
                offer(b, x, start + j);
            }
        }
    }
    sv[threadIdx.x] = b.v;
    si[threadIdx.x] = b.i;
    __syncthreads();
    for (int s = GB / 2; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s) {
            const Best o{sv[threadIdx.x + s], si[threadIdx.x + s]};
            const Best m{sv[threadIdx.x], si[threadIdx.x]};
            if (better(o, m)) {
                sv[threadIdx.x] = o.v;
                si[threadIdx.x] = o.i;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0 && argmax) argmax[row] = si[0];
}

}  // namespace

hipError_t launch_logits_gather_argmax(const void* const* shards, int t, int64_t n, int64_t vocab, void* full,
                                       int64_t* argmax, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    ShardPtrs sp = {};
    const int64_t per = (vocab + t - 1) / t;
    uint64_t g = (uint64_t)(uintptr_t)full;
    bool vec = true;
    for (int r = 0; r < t; ++r) {
        sp.p[r] = static_cast<const float*>(shards[r]);
        g |= (uint64_t)(uintptr_t)shards[r];
        const int64_t start = (int64_t)r * per;
        int64_t end = start + per;
        if (end > vocab) end = vocab;
        // whole float4 rows in the shard and at its place in the full row
        if (end > start && (((end - start) % 4) != 0 || (start % 4) != 0)) vec = false;
    }
    if ((g & 15u) != 0 || (full && vocab % 4 != 0)) vec = false;
    float* f = static_cast<float*>(full);
    if (vec)
        hipLaunchKernelGGL((logits_gather_argmax_kernel<true>), dim3((unsigned)n), dim3(GB), 0, s, sp, t, vocab, per,
                           f, argmax);
    else
        hipLaunchKernelGGL((logits_gather_argmax_kernel<false>), dim3((unsigned)n), dim3(GB), 0, s, sp, t, vocab,
                           per, f, argmax);
    return hipGetLastError();
}

}  // namespace tpk
