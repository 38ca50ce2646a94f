// Head-parallel attention core of one rank ("vLLM source analysis 13"
// §2.3.3: each rank runs self-attention on its own heads; "Tensor
// parallelism: implemented from scratch", TPAttention.forward: the rank's
// query heads share its KV heads by repeat_interleave, under a causal mask):
//   out[i, h] = softmax_s(q_i,h . k_s,g / sqrt(d) [s <= i if causal]) . v_s,g,
//   g = h / (nq / nkv), d = 128.
// The input is the rank's packed QKV projection output [n, (nq + 2 nkv) d]
// (q heads, then k heads, then v heads); the output [n, nq d] is the
// row-parallel o_proj's input.  bf16 in and out, fp32 softmax and
// accumulation, probabilities rounded to bf16 for the P.V product.
//
// Design (flash-attention order, one pass over the keys):
//   * workgroup = 4 waves = up to 4 query heads of one KV group on the same
//     32 queries; the 64-key K and V blocks are staged once in LDS and read
//     by all four;
//   * scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
//     keys as rows, queries as columns), so a lane owns one query and 32 of
//     the block's 64 scores: the running max and sum need one exchange with
//     the partner lane (l ^ 32) per block;
//   * O^T = V^T P^T: the probabilities are the B operand straight from the
//     score accumulators -- the 16 keys of a K step are taken in the order
//     the accumulator holds them (keys 4h..4h+3 and 8+4h..8+4h+3 of each 16
//     for lane half h), and V^T is read in the same order;
//   * K in LDS is row-major with 16-byte chunk c of key r at c ^ (r & 15)
//     (conflict-free fragment reads); V is stored transposed [d][key] with
//     136-byte rows (conflict-free 8-byte fragment reads);
//   * the next block's K and V are loaded into registers while the current
//     one is multiplied;
//   * causal: a tile stops at its last query's block, the diagonal block is
//     masked, and tiles are dispatched heaviest first;
//   * a tile's keys are cut into chunks of at most 32 blocks, one workgroup
//     each, so that long (causal: late) tiles do not set the kernel's
//     length; a tile with more than one chunk writes fp32 partials (O, the
//     running max and sum) to the workspace, and a second kernel merges its
//     chunks in order.
#include "common.hpp"

namespace tpk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats to packed bf16 with the hardware conversion (round to nearest
// even; the values here are finite)
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

constexpr int AD = 128;          // head_dim
constexpr int AQ = 32;           // queries per tile
constexpr int AK = 64;           // keys per block
constexpr int VT_LD = AK + 4;    // V^T row: 64 keys + 4 pad (136 bytes)
constexpr int ACH = 32;          // key blocks per chunk (a workgroup's share of a long tile)
constexpr int APART = AQ * AD + 2 * AQ;   // floats of one wave's partial: O, m, l

struct AttnArgs {
    const uint16_t* qkv;
    uint16_t* out;
    int64_t n;
    int64_t ld;                  // qkv row length (elements)
    int nq, nkv, rep, causal;
    int ntiles;
    int cmax;                    // chunks of the longest tile
    float scale_log2;            // log2(e) / sqrt(d)
    float* part;                 // [ntiles][cmax][heads/4 quads][4 waves][APART] fp32
};

// key blocks of query tile `tile`
__host__ __device__ __forceinline__ int tile_blocks(int tile, int64_t n, int causal) {
    if (!causal) return (int)((n + AK - 1) / AK);
    int64_t last = (int64_t)tile * AQ + AQ - 1;
    if (last > n - 1) last = n - 1;
    return (int)(last / AK) + 1;
}

__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[AK * AD];
    __shared__ __attribute__((aligned(16))) uint16_t vt[AD * VT_LD];
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int tid = threadIdx.x;
    // unit = (tile, chunk of at most ACH key blocks); heaviest tiles first
    const int ut = (int)blockIdx.x / a.cmax, uc = (int)blockIdx.x - ut * a.cmax;
    const int tile = a.causal ? a.ntiles - 1 - ut : ut;
    const int g = blockIdx.y;
    const int hsub = blockIdx.z * 4 + wid;            // head within the group
    const bool active = hsub < a.rep;
    const int head = g * a.rep + (active ? hsub : 0);
    const int64_t q0 = (int64_t)tile * AQ;
    const int r = lane & 31, hh = lane >> 5;
    const int64_t qi = q0 + r;                        // this lane's query

    // every load is a buffer load over [n, ld]: rows past n read as zero
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.qkv, (short)0, (int)(a.n * a.ld * 2), 0x00020000);
    auto ld16 = [&](int64_t row, int col) -> u32x4 {
        return __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((row * a.ld + col) * 2), 0, 0);
    };
    // Q fragments (B operand): query qi, d = 16 s + 8 hh .. + 8
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld16(qi, head * AD + 16 * s + 8 * hh));

    // key range of this unit: blocks [b0, b1) of the tile's nbt
    const int nbt = tile_blocks(tile, a.n, a.causal);
    const int b0 = uc * ACH;
    if (b0 >= nbt) return;                            // no such chunk (uniform)
    const int b1 = b0 + ACH < nbt ? b0 + ACH : nbt;
    const bool split = nbt > ACH;
    const int kcol = (a.nq + g) * AD, vcol = (a.nq + a.nkv + g) * AD;

    // staging: K items (key, chunk) = tid + 256 i; V items (key pair, chunk) = tid + 256 i
    u32x4 kreg[4], vreg[2][2];
    auto load_block = [&](int kb) {
        const int64_t k0 = (int64_t)kb * AK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, key = idx >> 4, c = idx & 15;
            kreg[i] = ld16(k0 + key, kcol + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, kp = idx & 31, c = idx >> 5;
#pragma unroll
            for (int e = 0; e < 2; ++e) vreg[i][e] = ld16(k0 + 2 * kp + e, vcol + 8 * c);
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, key = idx >> 4, c = idx & 15;
            *reinterpret_cast<u32x4*>(ks + key * AD + ((c ^ (key & 15)) * 8)) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, kp = idx & 31, c = idx >> 5;
            const uint32_t w0[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
            const uint32_t w1[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // d = 8 c + e: (V[2kp][d], V[2kp+1][d]) as one 32-bit word
                const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
                const uint32_t hi = (e & 1) ? (w1[e >> 1] & 0xffff0000u) : (w1[e >> 1] << 16);
                *reinterpret_cast<uint32_t*>(vt + (8 * c + e) * VT_LD + 2 * kp) = lo | hi;
            }
        }
    };

    f32x16 oacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) oacc[t][q] = 0.0f;
    float m = -INFINITY, lsum = 0.0f;

    load_block(b0);
    for (int kb = b0; kb < b1; ++kb) {
        store_block();
        __syncthreads();
        if (kb + 1 < b1) load_block(kb + 1);
        if (active) {
            // S^T = K Q^T for the block's two 32-key tiles
            f32x16 sacc[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int q = 0; q < 16; ++q) sacc[tt][q] = 0.0f;
                const int key = 32 * tt + r;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + key * AD + (((2 * s + hh) ^ (key & 15)) * 8));
                    sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[tt], 0, 0, 0);
                }
            }
            // scale (base-2 units), mask, running max and sum for query qi;
            // lane half hh holds keys 8 j + 4 hh + i of each tile
            const int kbase_i = kb * AK;
            const int qi32 = (int)qi, n32 = (int)a.n;
            const bool diag = a.causal ? (kbase_i + AK - 1 > (int)q0) : (kbase_i + AK > n32);
            float mloc = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    float v = sacc[tt][q] * a.scale_log2;
                    if (diag) {
                        const int key = kbase_i + 32 * tt + 8 * (q >> 2) + 4 * hh + (q & 3);
                        if ((a.causal && key > qi32) || key >= n32) v = -INFINITY;
                    }
                    sacc[tt][q] = v;
                    mloc = fmaxf(mloc, v);
                }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            const float mnew = fmaxf(m, mloc);
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // 0 on the first block (m = -inf)
            float psum = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const float p = __builtin_amdgcn_exp2f(sacc[tt][q] - mnew);
                    sacc[tt][q] = p;
                    psum += p;
                }
            psum += __shfl_xor(psum, 32, 64);
            lsum = lsum * alpha + psum;
            m = mnew;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int q = 0; q < 16; ++q) oacc[t][q] *= alpha;
            // P^T fragments: K step (tt, q2) = accumulator values 8 q2 .. 8 q2 + 7
            bf16x8 pf[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = cvt_bf16x2(sacc[tt][8 * q2 + 2 * e], sacc[tt][8 * q2 + 2 * e + 1]);
                    pf[tt][q2] = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
                }
            // O^T += V^T P^T: lane (d row, hh) reads keys 16 q2 + 4 hh + 0..3
            // and 16 q2 + 8 + 4 hh + 0..3 of tile tt
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const uint16_t* vrow = vt + (32 * dt + r) * VT_LD;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        const int kk = 32 * tt + 16 * q2 + 4 * hh;
                        const u32x2 x0 = *reinterpret_cast<const u32x2*>(vrow + kk);
                        const u32x2 x1 = *reinterpret_cast<const u32x2*>(vrow + kk + 8);
                        const bf16x8 vf = __builtin_bit_cast(bf16x8, (u32x4){x0.x, x0.y, x1.x, x1.y});
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[tt][q2], oacc[dt], 0, 0, 0);
                    }
            }
        }
        __syncthreads();
    }

    if (split) {
        // this chunk's unnormalised O, running max and sum for the combine
        float* pp = a.part + (((((int64_t)ut * a.cmax + uc) * gridDim.y + g) * gridDim.z + blockIdx.z) * 4 + wid) * APART;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 32 * dt + 8 * j + 4 * hh;
                *reinterpret_cast<float4*>(pp + r * AD + d) =
                    make_float4(oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]);
            }
        if (hh == 0) {
            pp[AQ * AD + r] = m;
            pp[AQ * AD + AQ + r] = lsum;
        }
        return;
    }
    // out[qi, head, d]: lane holds d = 32 dt + 8 j + 4 hh + i
    if (active && qi < a.n) {
        const float inv = 1.0f / lsum;
        uint16_t* o = a.out + qi * (int64_t)a.nq * AD + (int64_t)head * AD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 32 * dt + 8 * j + 4 * hh;
                const float v0 = oacc[dt][4 * j], v1 = oacc[dt][4 * j + 1];
                const float v2 = oacc[dt][4 * j + 2], v3 = oacc[dt][4 * j + 3];
                *reinterpret_cast<u32x2*>(o + d) =
                    (u32x2){cvt_bf16x2(v0 * inv, v1 * inv), cvt_bf16x2(v2 * inv, v3 * inv)};
            }
    }
}

// Merges the chunks of the split tiles: for query i of head h,
// m* = max_c m_c, out = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c,
// chunks in order.  Block (tile, KV group, quad x 4 + wave): 256 threads,
// thread = (query tid / 8, 16 consecutive d).
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a, int nz) {
    const int ut = blockIdx.x;
    const int tile = a.causal ? a.ntiles - 1 - ut : ut;
    const int nbt = tile_blocks(tile, a.n, a.causal);
    if (nbt <= ACH) return;                              // written directly
    const int nch = (nbt + ACH - 1) / ACH;
    const int g = blockIdx.y;
    const int z = blockIdx.z >> 2, wv = blockIdx.z & 3;
    const int hsub = z * 4 + wv;
    if (hsub >= a.rep) return;
    const int head = g * a.rep + hsub;
    const int qq = threadIdx.x >> 3, d0 = (threadIdx.x & 7) * 16;
    const int64_t qi = (int64_t)tile * AQ + qq;
    if (qi >= a.n) return;
    auto chunk = [&](int c) -> const float* {
        return a.part + (((((int64_t)ut * a.cmax + c) * gridDim.y + g) * nz + z) * 4 + wv) * APART;
    };
    float mx = -INFINITY;
    for (int c = 0; c < nch; ++c) mx = fmaxf(mx, chunk(c)[AQ * AD + qq]);
    float acc[16], den = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    for (int c = 0; c < nch; ++c) {
        const float* pp = chunk(c);
        const float w = __builtin_amdgcn_exp2f(pp[AQ * AD + qq] - mx);
        den = den + w * pp[AQ * AD + AQ + qq];
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            const float4 o = *reinterpret_cast<const float4*>(pp + qq * AD + d0 + e);
            acc[e] = acc[e] + w * o.x;
            acc[e + 1] = acc[e + 1] + w * o.y;
            acc[e + 2] = acc[e + 2] + w * o.z;
            acc[e + 3] = acc[e + 3] + w * o.w;
        }
    }
    const float inv = 1.0f / den;
    uint16_t* o = a.out + qi * (int64_t)a.nq * AD + (int64_t)head * AD + d0;
    u32x4 w0, w1;
    w0.x = cvt_bf16x2(acc[0] * inv, acc[1] * inv);
    w0.y = cvt_bf16x2(acc[2] * inv, acc[3] * inv);
    w0.z = cvt_bf16x2(acc[4] * inv, acc[5] * inv);
    w0.w = cvt_bf16x2(acc[6] * inv, acc[7] * inv);
    w1.x = cvt_bf16x2(acc[8] * inv, acc[9] * inv);
    w1.y = cvt_bf16x2(acc[10] * inv, acc[11] * inv);
    w1.z = cvt_bf16x2(acc[12] * inv, acc[13] * inv);
    w1.w = cvt_bf16x2(acc[14] * inv, acc[15] * inv);
    reinterpret_cast<u32x4*>(o)[0] = w0;
    reinterpret_cast<u32x4*>(o)[1] = w1;
}

AttnArgs attn_args(int64_t n, int nq, int nkv, int causal) {
    AttnArgs a{};
    a.n = n;
    a.ld = (int64_t)(nq + 2 * nkv) * AD;
    a.nq = nq;
    a.nkv = nkv;
    a.rep = nq / nkv;
    a.causal = causal ? 1 : 0;
    a.ntiles = (int)((n + AQ - 1) / AQ);
    const int nbmax = tile_blocks(a.ntiles - 1, n, a.causal);
    a.cmax = (nbmax + ACH - 1) / ACH;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)AD);
    return a;
}

}  // namespace

size_t attention_ws_bytes(int64_t n, int nq, int nkv, int causal) {
    if (n <= 0) return 0;
    const AttnArgs a = attn_args(n, nq, nkv, causal);
    if (a.cmax <= 1) return 0;
    const int nz = (a.rep + 3) / 4;
    return (size_t)a.ntiles * a.cmax * nkv * nz * 4 * APART * sizeof(float);
}

hipError_t launch_attention(const void* qkv, int64_t n, int nq, int nkv, int head_dim, int causal, void* out,
                            void* ws, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (head_dim != AD) return hipErrorInvalidValue;
    AttnArgs a = attn_args(n, nq, nkv, causal);
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.out = static_cast<uint16_t*>(out);
    a.part = static_cast<float*>(ws);
    if (a.cmax > 1 && !ws) return hipErrorInvalidValue;
    const int nz = (a.rep + 3) / 4;
    hipLaunchKernelGGL(attention_kernel, dim3((unsigned)(a.ntiles * a.cmax), (unsigned)nkv, (unsigned)nz), dim3(256),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.cmax <= 1) return e;
    hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)a.ntiles, (unsigned)nkv, (unsigned)(nz * 4)),
                       dim3(256), 0, s, a, nz);
    return hipGetLastError();
}

}  // namespace tpk
