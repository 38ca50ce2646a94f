// Internal helpers shared by the libtpshard kernels and host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpshard.h"

namespace tpk {

// ---- bf16 helpers (device) ----------------------------------------------

// bf16 -> fp32 is exact: the 16 bits are the top half of the fp32 encoding.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32): round to
// nearest, ties to even; NaN stays NaN.
typedef float cvt_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 cvt_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// pack two fp32 into two bf16 (lo in the low half), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((cvt_f32x2){lo, hi}, cvt_bf16x2));
}

// ---- element load/store by dtype ----------------------------------------

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// SiLU(g) * u in fp32: g * sigmoid(g) * u, the quotient g / (1 + e^-g) taken
// as g times the hardware reciprocal (1 ulp) of 1 + e^-g.  For g -> -inf,
// e^-g -> inf, whose reciprocal is 0, and the product goes to -0; for
// g -> +inf it goes to g.  (1 + e^-g rounds to 1 for g > 17, whose
// reciprocal is exactly 1.)
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t dtype_size(tp_dtype dt) { return dt == TP_F32 ? 4 : 2; }

}  // namespace tpk

// ---- host-side launchers implemented in the kernel translation units ------

namespace tpk {

hipError_t launch_copy2d(const void* src, int64_t src_ld_bytes, void* dst, int64_t dst_ld_bytes,
                         int64_t rows, int64_t row_bytes, hipStream_t s);

hipError_t launch_load_block(const void* src_host, tp_dtype src_dt, int64_t src_ld, int64_t r0, int64_t c0,
                             int64_t rows, int64_t cols, void* dst, tp_dtype dst_dt, int64_t dst_ld, int64_t dr0,
                             int64_t dc0, void* staging, hipStream_t s);
hipError_t launch_ring_reduce(const void* const* parts, int t, int64_t K, tp_dtype in_dt,
                              void* out, tp_dtype out_dt, tp_order order, hipStream_t s);

hipError_t launch_rs_add_rmsnorm(const void* const* partials, int t, int tp_rank, int64_t n, int64_t h, tp_dtype dt,
                                 const void* residual, const void* weight, float eps, void* residual_out, void* out,
                                 hipStream_t s);

hipError_t launch_logits_gather_argmax(const void* const* shards, int t, int64_t n, int64_t vocab, void* full,
                                       int64_t* argmax, hipStream_t s);

size_t attention_ws_bytes(int64_t n, int nq, int nkv, int causal);
hipError_t launch_attention(const void* qkv, int64_t n, int nq, int nkv, int head_dim, int causal, void* out,
                            void* ws, hipStream_t s);

hipError_t launch_vocab_embed(const int64_t* ids, int64_t n, const void* table, int64_t start,
                              int64_t end, int64_t h, int esize, void* out, hipStream_t s);

// GEMM planning and launch.  C[M, N] = A[M, K] . B[Nb, K]^T (+bias), or for a
// gated call act[M, N] = SiLU(A . B[0:N]^T) * (A . B[N:2N]^T) with Nb = 2N.
struct GemmPlan {
    int kernel;       // which tile configuration
    int splits;       // split-K factor (1 = none)
    int64_t k_split;  // K elements per split (multiple of the tile K) when splits > 1
    size_t ws_bytes;  // fp32 workspace for split-K partial sums (or the tail pieces)
    // balanced last round: the first full_tiles tiles run whole; each of the
    // remaining tiles is cut into tail_split K pieces of tail_k elements
    int full_tiles;
    int tail_split;   // 0 = no tail split
    int64_t tail_k;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool gated, tp_dtype dt);

hipError_t launch_gemm(const GemmPlan& plan, const void* A, const void* B, const void* bias,
                       void* C, int64_t M, int64_t N, int64_t K, bool gated, tp_dtype dt,
                       tp_dtype out_dt, void* ws, hipStream_t s);

// the fp32 products (gemm_f32.hip), no workspace
hipError_t launch_gemm_f32(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                           int64_t K, bool gated, hipStream_t s);

}  // namespace tpk
