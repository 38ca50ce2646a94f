// Sum of the t rank partials in ring reduce-scatter chunk order, one device.
//
// The K elements are cut into t contiguous chunks [floor(cK/t), floor((c+1)K/t)).
// A ring reduce-scatter (vLLM source analysis 13, §1.1.1) adds chunk c into
// the running sum as it travels c -> c+1 -> ... so its value is
// ((P_c + P_{c+1}) + P_{c+2}) + ... + P_{c+t-1}; every rank then receives that
// chunk unchanged in the all-gather (§1.1.2).  This kernel performs exactly
// that arithmetic (fp32 adds, one rounding at the end) without the transfers.
//
// TP_ORDER_RANK is the one-shot form instead (the low-latency all-reduce of
// "vLLM source analysis 13" §1.2 and the custom all-reduce of "AIInfraGuide
// 6.2" §6.3: every rank reads all buffers and adds them into a zero
// accumulator): ((0 + P_0) + P_1) + ... + P_{t-1} for every element, on the
// same kernels with the rotation off and a +0 start.
//
// HBM-streaming design: grid.y is the chunk, so the rotation of the partial
// order is uniform per workgroup and the per-element index math is a single
// add.  Each lane moves 16-byte vectors (8 bf16 or 4 fp32).  For t = 2, 4,
// 8, 16 a kernel with t fixed at compile time issues all t loads of a vector
// before the first add and gives each lane one vector (a large grid of short
// workgroups); other t use a generic kernel that keeps UNROLL vectors per
// partial in flight.  The unaligned head and tail of a chunk
// (when its bounds are not multiples of the vector width) are done element
// by element by the chunk's first workgroup.  No atomics: bit-reproducible.
#include "common.hpp"

namespace tpk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PartPtrs {
    const void* p[TP_MAX_RANKS];
};

template <typename InT> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    using raw = u32x4;
    static __device__ __forceinline__ void widen(const raw& r, float* f) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    using raw = u32x4;
    static __device__ __forceinline__ void widen(const raw& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
};

template <typename OutT, int N> struct VecStore;
template <> struct VecStore<uint16_t, 8> {
    static __device__ __forceinline__ void store(uint16_t* p, const float* f) {
        uint4 o;
        o.x = pack_bf16x2(f[0], f[1]);
        o.y = pack_bf16x2(f[2], f[3]);
        o.z = pack_bf16x2(f[4], f[5]);
        o.w = pack_bf16x2(f[6], f[7]);
        *reinterpret_cast<uint4*>(p) = o;
    }
};
template <> struct VecStore<float, 8> {
    static __device__ __forceinline__ void store(float* p, const float* f) {
        reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
};
template <> struct VecStore<float, 4> {
    static __device__ __forceinline__ void store(float* p, const float* f) {
        *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    }
};

__device__ __forceinline__ int64_t chunk_lo(int64_t K, int t, int c) {
    // floor(c*K/t) without overflow for K < 2^56 and t <= 64
    return (int64_t)(((unsigned __int128)c * (unsigned __int128)K) / (unsigned)t);
}

// The chunk's unaligned head [lo, min(vlo, hi)) and tail [max(vhi, lo), hi),
// element by element, in the same rotated order as the vector body.
template <typename InT, typename OutT>
__device__ __forceinline__ void reduce_edges(const PartPtrs& parts, int t, int c, int rank_order, int64_t lo,
                                             int64_t hi, int64_t vlo, int64_t vhi,
                                             OutT* __restrict__ out) {
    const int c0 = rank_order ? 0 : c;
    auto src = [&](int j) -> const InT* {
        int r = c0 + j;
        if (r >= t) r -= t;
        return static_cast<const InT*>(parts.p[r]);
    };
    const float z = rank_order ? 0.0f : -0.0f;      // -0 + x == x for every x
    const int64_t head_end = vlo < hi ? vlo : hi;
    const int64_t tail_beg = vhi > head_end ? vhi : head_end;
    for (int64_t i = lo + threadIdx.x; i < head_end; i += blockDim.x) {
        float acc = z + Elem<InT>::load(src(0) + i);
        for (int j = 1; j < t; ++j) acc = acc + Elem<InT>::load(src(j) + i);
        Elem<OutT>::store(out + i, acc);
    }
    for (int64_t i = tail_beg + threadIdx.x; i < hi; i += blockDim.x) {
        float acc = z + Elem<InT>::load(src(0) + i);
        for (int j = 1; j < t; ++j) acc = acc + Elem<InT>::load(src(j) + i);
        Elem<OutT>::store(out + i, acc);
    }
}

// Same arithmetic with t fixed at compile time.  Each lane owns one 16-byte
// vector per pass and issues all T loads of it before its first add, so
// T x 16 bytes per lane are in flight (256 B at T = 16).  The adds then run
// in the ring order with one rounding at the store: bit-identical to the
// generic kernel.  The launcher gives every lane a single vector, so the grid
// is large and each workgroup is short; the stride loop only runs when the
// grid limit caps the workgroups per chunk.
template <typename InT, typename OutT, int T>
__global__ __launch_bounds__(256) void ring_reduce_fixed_kernel(PartPtrs parts, int64_t K,
                                                                OutT* __restrict__ out,
                                                                int blocks_per_chunk, int rank_order) {
    using V = Vec<InT>;
    constexpr int N = V::N;
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(K, T, c);
    const int64_t hi = chunk_lo(K, T, c + 1);
    int64_t vlo = (lo + N - 1) / N * N;
    int64_t vhi = hi / N * N;
    if (vhi < vlo) vhi = vlo;
    if (blockIdx.x == 0) reduce_edges<InT, OutT>(parts, T, c, rank_order, lo, hi, vlo, vhi, out);

    // position j of the ring order reads rank (c + j) mod T (rank order:
    // rank j); wave-uniform
    const int c0 = rank_order ? 0 : c;
    const float z = rank_order ? 0.0f : -0.0f;      // the one-shot sum starts at +0
    const typename V::raw* s[T];
#pragma unroll
    for (int j = 0; j < T; ++j) {
        const int r = c0 + j < T ? c0 + j : c0 + j - T;
        s[j] = reinterpret_cast<const typename V::raw*>(static_cast<const InT*>(parts.p[r]) + vlo);
    }
    OutT* o = out + vlo;
    const int64_t nvec = (vhi - vlo) / N;
    const int64_t stride = (int64_t)blocks_per_chunk * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        typename V::raw raw[T];
#pragma unroll
        for (int j = 0; j < T; ++j) raw[j] = __builtin_nontemporal_load(s[j] + v);
        float acc[N], f[N];
        V::widen(raw[0], acc);
#pragma unroll
        for (int q = 0; q < N; ++q) acc[q] = z + acc[q];
#pragma unroll
        for (int j = 1; j < T; ++j) {
            V::widen(raw[j], f);
#pragma unroll
            for (int q = 0; q < N; ++q) acc[q] = acc[q] + f[q];
        }
        VecStore<OutT, N>::store(o + v * N, acc);
    }
}

template <typename InT, typename OutT, int UNROLL>
__global__ __launch_bounds__(256) void ring_reduce_kernel(PartPtrs parts, int t, int64_t K,
                                                          OutT* __restrict__ out,
                                                          int blocks_per_chunk, int rank_order) {
    using V = Vec<InT>;
    constexpr int N = V::N;
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(K, t, c);
    const int64_t hi = chunk_lo(K, t, c + 1);
    // vector-aligned body [vlo, vhi)
    int64_t vlo = (lo + N - 1) / N * N;
    int64_t vhi = hi / N * N;
    if (vhi < vlo) vhi = vlo;

    // the rotated order for this chunk: position j reads rank (c + j) mod t
    // (rank order: rank j).  The index is wave-uniform, so the pointer comes
    // straight from the kernel-argument segment with a scalar load.
    const int c0 = rank_order ? 0 : c;
    const float z = rank_order ? 0.0f : -0.0f;      // the one-shot sum starts at +0
    auto src = [&](int j) -> const InT* {
        int r = c0 + j;
        if (r >= t) r -= t;
        return static_cast<const InT*>(parts.p[r]);
    };

    if (blockIdx.x == 0) reduce_edges<InT, OutT>(parts, t, c, rank_order, lo, hi, vlo, vhi, out);

    const int64_t nvec = (vhi - vlo) / N;
    const int64_t stride = (int64_t)blocks_per_chunk * blockDim.x;
    int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; v + (UNROLL - 1) * stride < nvec; v += UNROLL * stride) {
        float acc[UNROLL][N];
        typename V::raw raw[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t e = vlo + (v + u * stride) * N;
            raw[u] = __builtin_nontemporal_load(reinterpret_cast<const typename V::raw*>(src(0) + e));
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            V::widen(raw[u], acc[u]);
#pragma unroll
            for (int q = 0; q < N; ++q) acc[u][q] = z + acc[u][q];
        }
        for (int j = 1; j < t; ++j) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t e = vlo + (v + u * stride) * N;
                raw[u] = __builtin_nontemporal_load(reinterpret_cast<const typename V::raw*>(src(j) + e));
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float f[N];
                V::widen(raw[u], f);
#pragma unroll
                for (int q = 0; q < N; ++q) acc[u][q] = acc[u][q] + f[q];
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t e = vlo + (v + u * stride) * N;
            VecStore<OutT, N>::store(out + e, acc[u]);
        }
    }
    for (; v < nvec; v += stride) {
        const int64_t e = vlo + v * N;
        float acc[N];
        V::widen(*reinterpret_cast<const typename V::raw*>(src(0) + e), acc);
#pragma unroll
        for (int q = 0; q < N; ++q) acc[q] = z + acc[q];
        for (int j = 1; j < t; ++j) {
            float f[N];
            V::widen(*reinterpret_cast<const typename V::raw*>(src(j) + e), f);
#pragma unroll
            for (int q = 0; q < N; ++q) acc[q] = acc[q] + f[q];
        }
        VecStore<OutT, N>::store(out + e, acc);
    }
}

// Element-wise fallback for buffers that are not 16-byte aligned.
template <typename InT, typename OutT>
__global__ __launch_bounds__(256) void ring_reduce_scalar_kernel(PartPtrs parts, int t, int64_t K,
                                                                 OutT* __restrict__ out,
                                                                 int blocks_per_chunk, int rank_order) {
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(K, t, c);
    const int64_t hi = chunk_lo(K, t, c + 1);
    const float z = rank_order ? 0.0f : -0.0f;      // the one-shot sum starts at +0
    for (int64_t i = lo + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi;
         i += (int64_t)blocks_per_chunk * blockDim.x) {
        int r = rank_order ? 0 : c;
        float acc = z + Elem<InT>::load(static_cast<const InT*>(parts.p[r]) + i);
        for (int j = 1; j < t; ++j) {
            r = r + 1 == t ? 0 : r + 1;
            acc = acc + Elem<InT>::load(static_cast<const InT*>(parts.p[r]) + i);
        }
        Elem<OutT>::store(out + i, acc);
    }
}

template <typename InT, typename OutT>
static hipError_t launch_typed(const void* const* p, int t, int64_t K, void* out, int ro, hipStream_t s) {
    PartPtrs pp = {};
    uint64_t g = (uint64_t)(uintptr_t)out;
    for (int r = 0; r < t; ++r) {
        pp.p[r] = p[r];
        g |= (uint64_t)(uintptr_t)p[r];
    }
    const int64_t chunk = ceil_div(K, t);
    const bool fixed = (g & 15u) == 0 && (t == 2 || t == 4 || t == 8 || t == 16);
    // fixed-t kernel: one 16-byte vector per lane (measured best: many short
    // workgroups); generic kernel: ~8 vectors per lane per workgroup pass.
    // At least one workgroup per chunk either way.
    const int64_t per_block = 256LL * (fixed ? 1 : 8) * (16 / (int64_t)sizeof(InT));
    int64_t bpc = ceil_div(chunk, per_block);
    if (bpc < 1) bpc = 1;
    if (bpc > 65535) bpc = 65535;
    dim3 grid((unsigned)bpc, (unsigned)t);
    if (fixed) {
        OutT* o = static_cast<OutT*>(out);
        const int b = (int)bpc;
        switch (t) {
        case 2: hipLaunchKernelGGL((ring_reduce_fixed_kernel<InT, OutT, 2>), grid, dim3(256), 0, s, pp, K, o, b, ro); break;
        case 4: hipLaunchKernelGGL((ring_reduce_fixed_kernel<InT, OutT, 4>), grid, dim3(256), 0, s, pp, K, o, b, ro); break;
        case 8: hipLaunchKernelGGL((ring_reduce_fixed_kernel<InT, OutT, 8>), grid, dim3(256), 0, s, pp, K, o, b, ro); break;
        default: hipLaunchKernelGGL((ring_reduce_fixed_kernel<InT, OutT, 16>), grid, dim3(256), 0, s, pp, K, o, b, ro); break;
        }
    } else if ((g & 15u) == 0) {
        constexpr int UNROLL = sizeof(InT) == 2 ? 2 : 4;
        hipLaunchKernelGGL((ring_reduce_kernel<InT, OutT, UNROLL>), grid, dim3(256), 0, s, pp, t, K,
                           static_cast<OutT*>(out), (int)bpc, ro);
    } else {
        hipLaunchKernelGGL((ring_reduce_scalar_kernel<InT, OutT>), grid, dim3(256), 0, s, pp, t, K,
                           static_cast<OutT*>(out), (int)bpc, ro);
    }
    return hipGetLastError();
}

hipError_t launch_ring_reduce(const void* const* parts, int t, int64_t K, tp_dtype in_dt,
                              void* out, tp_dtype out_dt, tp_order order, hipStream_t s) {
    if (K <= 0) return hipSuccess;
    const int ro = order == TP_ORDER_RANK ? 1 : 0;
    if (in_dt == TP_BF16 && out_dt == TP_BF16) return launch_typed<uint16_t, uint16_t>(parts, t, K, out, ro, s);
    if (in_dt == TP_BF16 && out_dt == TP_F32) return launch_typed<uint16_t, float>(parts, t, K, out, ro, s);
    return launch_typed<float, float>(parts, t, K, out, ro, s);
}

}  // namespace tpk
