// Sequence-parallel epilogue of a row-parallel layer, one rank, one device.
//
// The all-reduce of the t partials is split into a reduce-scatter and an
// all-gather, and the per-token work between them (residual add, RMSNorm)
// runs only on the tokens a rank holds ("Tensor parallelism: implemented from
// scratch", Exercises, item 1).  With the ring of "vLLM source analysis 13"
// §1.1.1, rank r ends the reduce-scatter holding chunk c = (r + 1) mod t,
// summed ((P_c + P_{c+1}) + ...) + P_{c+t-1} in fp32.  Chunks are token rows
// [floor(c n / t), floor((c+1) n / t)).  For each owned row this kernel
//   1. adds the t partial rows in that order (fp32),
//   2. adds the residual row (one fp32 add) and rounds once to the storage
//      type: the new residual stream, written to residual_out,
//   3. normalises the stored row: y = v / sqrt(mean(v^2) + eps) * w.
// Transfers are not performed (one device); the arithmetic and the HBM
// traffic of the rank's share are.
//
// Layout: one workgroup of 1024 threads per row; a thread owns 16-byte
// vectors tid, tid + 1024, ... of the row.  For t = 2, 4, 8, 16 every partial
// load of a vector is issued before the first add.  The first KEEP vectors
// of each thread stay in registers for step 3; further ones (rows longer than
// 1024 x KEEP vectors) are read back from residual_out, which the same thread
// wrote.  The mean square is reduced in a fixed tree (wave shuffles, then the
// wave sums in order): deterministic.  Both outputs are written with
// non-temporal stores (nothing reads them back soon).  Measured at the 70B
// prefill shard (8 x 1024 rows of 8192): 256-thread workgroups, 36.9 us
// (one round of blocks: every block loads, then stores, at the same time);
// 1024 threads, 34.3 us; plus non-temporal stores, 31.1 us = 74% of HBM.
#include "common.hpp"

namespace tpk {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SpParts {
    const void* p[TP_MAX_RANKS];
};

template <typename T> struct SpVec;
template <> struct SpVec<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void widen(const u32x4& r, float* f) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    // rounds to the storage type; f holds the rounded values afterwards
    static __device__ __forceinline__ u32x4 narrow(float* f) {
        u32x4 o;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
        o.x = w[0];
        o.y = w[1];
        o.z = w[2];
        o.w = w[3];
        return o;
    }
};
template <> struct SpVec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void widen(const u32x4& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    static __device__ __forceinline__ u32x4 narrow(float* f) {
        u32x4 o;
        o.x = __float_as_uint(f[0]);
        o.y = __float_as_uint(f[1]);
        o.z = __float_as_uint(f[2]);
        o.w = __float_as_uint(f[3]);
        return o;
    }
};

// sum over the BS threads in a fixed order; every thread gets the result
template <int BS>
__device__ __forceinline__ float block_sum(float v, float* ldsw) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) ldsw[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = ldsw[0];
#pragma unroll
    for (int w = 1; w < BS / 64; ++w) s = s + ldsw[w];
    return s;
}

// T = t fixed at compile time (all loads of a vector in flight), or 0 for a
// runtime t
template <typename InT, int T, int KEEP, int BS>
__global__ __launch_bounds__(BS) void rs_add_rmsnorm_kernel(SpParts parts, int t, int c, int64_t row0,
                                                            int64_t h, const InT* residual,
                                                            const InT* __restrict__ weight, float eps,
                                                            InT* residual_out, InT* __restrict__ out) {
    using V = SpVec<InT>;
    constexpr int N = V::N;
    __shared__ float ldsw[BS / 64];
    const int tt = T > 0 ? T : t;
    const int64_t r = blockIdx.x;                        // row within the chunk
    const int64_t grow = row0 + r;                       // row within [n, h]
    const int64_t nvec = h / N;
    const u32x4* res = reinterpret_cast<const u32x4*>(residual + r * h);
    u32x4* rout = reinterpret_cast<u32x4*>(residual_out + r * h);

    // one vector: ring-order sum of the partials, + residual, rounded
    auto reduce_vec = [&](int64_t v, float* f) {
        float acc[N], g[N];
        if constexpr (T > 0) {
            u32x4 raw[T];
#pragma unroll
            for (int j = 0; j < T; ++j) {
                const int src = c + j < T ? c + j : c + j - T;
                raw[j] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(static_cast<const InT*>(parts.p[src]) + grow * h) + v);
            }
            V::widen(raw[0], acc);
#pragma unroll
            for (int j = 1; j < T; ++j) {
                V::widen(raw[j], g);
#pragma unroll
                for (int q = 0; q < N; ++q) acc[q] = acc[q] + g[q];
            }
        } else {
            V::widen(__builtin_nontemporal_load(
                         reinterpret_cast<const u32x4*>(static_cast<const InT*>(parts.p[c]) + grow * h) + v),
                     acc);
            for (int j = 1; j < tt; ++j) {
                const int src = c + j < tt ? c + j : c + j - tt;
                V::widen(__builtin_nontemporal_load(
                             reinterpret_cast<const u32x4*>(static_cast<const InT*>(parts.p[src]) + grow * h) + v),
                         g);
#pragma unroll
                for (int q = 0; q < N; ++q) acc[q] = acc[q] + g[q];
            }
        }
        V::widen(res[v], g);
#pragma unroll
        for (int q = 0; q < N; ++q) f[q] = acc[q] + g[q];
        __builtin_nontemporal_store(V::narrow(f), rout + v);
    };

    float keep[KEEP][N];
    float ss = 0.0f;
    const int64_t v0 = threadIdx.x;
#pragma unroll
    for (int k = 0; k < KEEP; ++k) {
        const int64_t v = v0 + (int64_t)k * BS;
        if (v < nvec) {
            reduce_vec(v, keep[k]);
#pragma unroll
            for (int q = 0; q < N; ++q) ss = ss + keep[k][q] * keep[k][q];
        }
    }
    for (int64_t v = v0 + (int64_t)KEEP * BS; v < nvec; v += BS) {
        float f[N];
        reduce_vec(v, f);
#pragma unroll
        for (int q = 0; q < N; ++q) ss = ss + f[q] * f[q];
    }
    const float total = block_sum<BS>(ss, ldsw);
    const float inv = 1.0f / __fsqrt_rn(total / (float)h + eps);

    const u32x4* wv = reinterpret_cast<const u32x4*>(weight);
    u32x4* ov = reinterpret_cast<u32x4*>(out + r * h);
    auto norm_vec = [&](int64_t v, float* f) {
        float w[N];
        V::widen(wv[v], w);
#pragma unroll
        for (int q = 0; q < N; ++q) f[q] = f[q] * inv * w[q];
        __builtin_nontemporal_store(V::narrow(f), ov + v);
    };
#pragma unroll
    for (int k = 0; k < KEEP; ++k) {
        const int64_t v = v0 + (int64_t)k * BS;
        if (v < nvec) norm_vec(v, keep[k]);
    }
    for (int64_t v = v0 + (int64_t)KEEP * BS; v < nvec; v += BS) {
        float f[N];
        V::widen(rout[v], f);
        norm_vec(v, f);
    }
}

// Element-wise form for rows that are not whole 16-byte vectors or buffers
// that are not 16-byte aligned: same order and roundings.
template <typename InT>
__global__ __launch_bounds__(256) void rs_add_rmsnorm_scalar_kernel(SpParts parts, int t, int c, int64_t row0,
                                                                   int64_t h, const InT* residual,
                                                                   const InT* weight, float eps,
                                                                   InT* residual_out, InT* out) {
    __shared__ float lds4[4];
    const int64_t r = blockIdx.x;
    const int64_t grow = row0 + r;
    float ss = 0.0f;
    for (int64_t j = threadIdx.x; j < h; j += 256) {
        float acc = Elem<InT>::load(static_cast<const InT*>(parts.p[c]) + grow * h + j);
        for (int k = 1; k < t; ++k) {
            const int src = c + k < t ? c + k : c + k - t;
            acc = acc + Elem<InT>::load(static_cast<const InT*>(parts.p[src]) + grow * h + j);
        }
        const float v = acc + Elem<InT>::load(residual + r * h + j);
        Elem<InT>::store(residual_out + r * h + j, v);
        const float s = Elem<InT>::load(residual_out + r * h + j);     // the stored value
        ss = ss + s * s;
    }
    const float total = block_sum<256>(ss, lds4);
    const float inv = 1.0f / __fsqrt_rn(total / (float)h + eps);
    for (int64_t j = threadIdx.x; j < h; j += 256) {
        const float s = Elem<InT>::load(residual_out + r * h + j);
        Elem<InT>::store(out + r * h + j, s * inv * Elem<InT>::load(weight + j));
    }
}

template <typename InT, int KEEP, int BS>
hipError_t launch_vec(const SpParts& pp, int t, int c, int64_t row0, int64_t rows, int64_t h, const void* residual,
                      const void* weight, float eps, void* residual_out, void* out, hipStream_t s) {
    const dim3 grid((unsigned)rows);
    const InT* res = static_cast<const InT*>(residual);
    const InT* w = static_cast<const InT*>(weight);
    InT* ro = static_cast<InT*>(residual_out);
    InT* o = static_cast<InT*>(out);
    switch (t) {
        case 2: hipLaunchKernelGGL((rs_add_rmsnorm_kernel<InT, 2, KEEP, BS>), grid, dim3(BS), 0, s, pp, t, c, row0, h, res, w, eps, ro, o); break;
        case 4: hipLaunchKernelGGL((rs_add_rmsnorm_kernel<InT, 4, KEEP, BS>), grid, dim3(BS), 0, s, pp, t, c, row0, h, res, w, eps, ro, o); break;
        case 8: hipLaunchKernelGGL((rs_add_rmsnorm_kernel<InT, 8, KEEP, BS>), grid, dim3(BS), 0, s, pp, t, c, row0, h, res, w, eps, ro, o); break;
        case 16: hipLaunchKernelGGL((rs_add_rmsnorm_kernel<InT, 16, KEEP, BS>), grid, dim3(BS), 0, s, pp, t, c, row0, h, res, w, eps, ro, o); break;
        default: hipLaunchKernelGGL((rs_add_rmsnorm_kernel<InT, 0, KEEP, BS>), grid, dim3(BS), 0, s, pp, t, c, row0, h, res, w, eps, ro, o); break;
    }
    return hipGetLastError();
}

template <typename InT>
hipError_t launch_typed(const void* const* partials, int t, int c, int64_t row0, int64_t rows, int64_t h,
                        const void* residual, const void* weight, float eps, void* residual_out, void* out,
                        hipStream_t s) {
    SpParts pp = {};
    uint64_t g = (uint64_t)(uintptr_t)residual | (uint64_t)(uintptr_t)weight | (uint64_t)(uintptr_t)residual_out |
                 (uint64_t)(uintptr_t)out;
    for (int r = 0; r < t; ++r) {
        pp.p[r] = partials[r];
        g |= (uint64_t)(uintptr_t)partials[r];
    }
    constexpr int N = SpVec<InT>::N;
    if ((g & 15u) == 0 && h % N == 0) {
        // keep up to 4 vectors per thread (8192 bf16 / 4096 fp32 elements per
        // row) in registers
        // 1024 threads, one vector each in registers (8192 bf16 / 4096 fp32
        // elements per row; longer rows read the rest back).  A second one
        // would take the t = 8 kernel past 64 VGPRs and leave one workgroup
        // per CU instead of two (measured 35.7 us against 31.1 us).
        return launch_vec<InT, 1, 1024>(pp, t, c, row0, rows, h, residual, weight, eps, residual_out, out, s);
    }
    hipLaunchKernelGGL((rs_add_rmsnorm_scalar_kernel<InT>), dim3((unsigned)rows), dim3(256), 0, s, pp, t, c, row0, h,
                       static_cast<const InT*>(residual), static_cast<const InT*>(weight), eps,
                       static_cast<InT*>(residual_out), static_cast<InT*>(out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rs_add_rmsnorm(const void* const* partials, int t, int tp_rank, int64_t n, int64_t h, tp_dtype dt,
                                 const void* residual, const void* weight, float eps, void* residual_out, void* out,
                                 hipStream_t s) {
    const int c = (tp_rank + 1) % t;
    const int64_t lo = (int64_t)(((__int128)c * n) / t), hi = (int64_t)(((__int128)(c + 1) * n) / t);
    if (hi <= lo) return hipSuccess;
    if (dt == TP_BF16)
        return launch_typed<uint16_t>(partials, t, c, lo, hi - lo, h, residual, weight, eps, residual_out, out, s);
    return launch_typed<float>(partials, t, c, lo, hi - lo, h, residual, weight, eps, residual_out, out, s);
}

}  // namespace tpk
