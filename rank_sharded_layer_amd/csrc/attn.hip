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
//   * workgroup = 8 waves = two 32-query halves of a 64-query tile x up to
//     4 query heads of one KV group, one workgroup per CU; each 64-key
//     block of K and V goes from global memory straight into LDS
//     (buffer_load ... lds, double-buffered, one barrier per block) and is
//     read by all eight.  With 64 = the key block size, both halves of a
//     tile have the same key blocks (causal or ragged), so sharing a block
//     between two query halves halves the K/V traffic per query against
//     32-query workgroups of 4 waves at two per CU;
//   * scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
//     keys as rows, queries as columns), so a lane owns one query and 32 of
//     the block's 64 scores: the running max and sum need one exchange with
//     the partner lane (l ^ 32) per block;
//   * O^T = V^T P^T: the probabilities are the B operand straight from the
//     score accumulators -- the 16 keys of a K step are taken in the order
//     the accumulator holds them (keys 4h..4h+3 and 8+4h..8+4h+3 of each 16
//     for lane half h) -- and the V^T fragments come from row-major V in LDS
//     through the transposing read ds_read_b64_tr_b16;
//   * a block's probabilities are first taken against the running max; only
//     when one of them would exceed 2^13 (and on the first block) is the
//     block's maximum computed, the max moved and the accumulators rescaled,
//     so most blocks need neither the maximum nor the 64 rescales;
//   * causal work balance: query tiles are paired heavy with light (tile p
//     with tile nt-1-p, a near-constant number of key blocks per pair), each
//     pair's concatenated key blocks are cut into k equal chunks, and one
//     workgroup takes one chunk, so every workgroup has the same work.  A
//     tile that spans several chunks writes fp32 partials (unnormalised O,
//     running max and sum) per chunk to the workspace, and a second kernel
//     merges them in key order.
#include "common.hpp"

#include <type_traits>

namespace tpk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ void wg_barrier() {
    // s_barrier alone: the waits it needs are issued explicitly before it
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int AD = 128;          // head_dim
constexpr int AQ = 32;           // queries per wave
constexpr int AQW = 64;          // queries per tile: two 32-query halves of a workgroup
constexpr int AK = 64;           // keys per block
constexpr int AW = 8;            // waves: (query half, head of a quad)
constexpr int APART = AQ * AD + 2 * AQ;   // floats of one wave's partial: O, m, l
constexpr int AUNITS = 256;      // target workgroups: one per CU
constexpr int AMINCH = 8;        // fewest key blocks per chunk
constexpr float ATAU_SUM = 8192.0f;   // largest accepted sum of a lane's 32 probabilities

struct AttnArgs {
    const uint16_t* qkv;
    uint16_t* out;
    int64_t n;
    int64_t ld;                  // qkv row length (elements)
    int nq, nkv, rep, causal;
    int ntiles;                  // query tiles of AQW
    int npairs;                  // (ntiles + 1) / 2
    int kch;                     // chunks per pair
    float scale_log2;            // log2(e) / sqrt(d)
    float* part;                 // [npairs][kch][2][nkv][quads][AW waves][APART] fp32
};

// key blocks of query tile `tile`
__host__ __device__ __forceinline__ int tile_blocks(int tile, int64_t n, int causal) {
    if (!causal) return (int)((n + AK - 1) / AK);
    int64_t last = (int64_t)tile * AQW + AQW - 1;
    if (last > n - 1) last = n - 1;
    return (int)(last / AK) + 1;
}

// Pair p = (tile p, tile ntiles-1-p; one tile when they coincide).  Its key
// blocks in order: tile p's, then the other tile's; chunk c of the pair is
// [c T / k, (c+1) T / k) of that list, T its length.
struct PairPlan {
    int ta, tb;                  // tiles (tb = -1: none)
    int na, total;               // blocks of ta, of the pair
};

__host__ __device__ __forceinline__ PairPlan pair_plan(int p, const AttnArgs& a) {
    PairPlan pp;
    pp.ta = p;
    pp.tb = a.ntiles - 1 - p;
    pp.na = tile_blocks(pp.ta, a.n, a.causal);
    if (pp.tb == pp.ta) pp.tb = -1;
    pp.total = pp.na + (pp.tb >= 0 ? tile_blocks(pp.tb, a.n, a.causal) : 0);
    return pp;
}

__host__ __device__ __forceinline__ int chunk_lo(int c, int total, int k) {
    return (int)(((int64_t)c * total) / k);
}

__global__ __launch_bounds__(AW * 64, 1) void attention_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint16_t ks0[AK * AD];
    __shared__ __attribute__((aligned(1024))) uint16_t ks1[AK * AD];
    __shared__ __attribute__((aligned(1024))) uint16_t vs0[AK * AD];
    __shared__ __attribute__((aligned(1024))) uint16_t vs1[AK * AD];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = (int)blockIdx.x / a.kch, c = (int)blockIdx.x - p * a.kch;
    const int g = blockIdx.y;
    const int half = wid >> 2;                        // query half of the tile
    const int hsub = blockIdx.z * 4 + (wid & 3);      // head within the group
    const bool active = hsub < a.rep;
    const int head = g * a.rep + (active ? hsub : 0);
    const int r = lane & 31, hh = lane >> 5;
    const int kcol = (a.nq + g) * AD, vcol = (a.nq + a.nkv + g) * AD;

    // every load is a buffer load over [n, ld]: rows past n, and blocks past
    // the segment (base offset 2^31), read as zero
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.qkv, (short)0, (int)(a.n * a.ld * 2), 0x00020000);
    const uint32_t row_b = (uint32_t)(a.ld * 2);

    // K and V blocks go from global memory straight into LDS (a wave
    // instruction fills 64 consecutive 16-byte slots, lane l slot l, so each
    // lane fetches the chunk that belongs in its slot).  LDS layouts, chosen
    // so that every fragment read is conflict-free and its address is one
    // per-lane base plus immediate offsets:
    //   K: the 32-byte piece d = 16 s .. 16 s + 15 of key k at byte
    //      2048 s + 32 k, its two 16-byte halves swapped when bit 3 of k is
    //      set (16 consecutive keys of one half then cover all 16 bank
    //      groups);
    //   V: the 64-byte piece d = 32 t .. 32 t + 31 of key k at byte
    //      4096 t + 64 k (4 consecutive keys of one piece = 256 contiguous
    //      bytes, what a half-wave transposing read takes).
    // A block is 16 instructions of K and 16 of V; this wave's instruction
    // q fills slots 64 J .. + 63, J = 2 wid + q:
    //   K: s = J >> 1, key 32 (J & 1) + (lane >> 1), half
    //      (lane & 1) ^ ((lane >> 4) & 1);
    //   V: t = J >> 2, key 16 (J & 3) + (lane >> 2), chunk (lane & 3) of
    //      the piece.
    constexpr int PQ = 16 / AW;                       // instructions per wave and operand
    uint32_t koff[PQ], voff[PQ];
#pragma unroll
    for (int q = 0; q < PQ; ++q) {
        const int J = PQ * wid + q;
        const int kk = 32 * (J & 1) + (lane >> 1);
        const int kc = 2 * (J >> 1) + ((lane & 1) ^ ((lane >> 4) & 1));
        koff[q] = (uint32_t)kk * row_b + (uint32_t)(kcol + 8 * kc) * 2;
        const int vk = 16 * (J & 3) + (lane >> 2);
        voff[q] = (uint32_t)vk * row_b + (uint32_t)(vcol + 32 * (J >> 2) + 8 * (lane & 3)) * 2;
    }
    auto issue = [&](uint32_t base, uint16_t* buf, const uint32_t (&off)[PQ]) {
#pragma unroll
        for (int q = 0; q < PQ; ++q) {
            auto* dst = (__attribute__((address_space(3))) void*)(reinterpret_cast<uint8_t*>(buf) + (PQ * wid + q) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, base + off[q], 0, 0, 0);
        }
    };
    // K fragment (A operand) of key 32 tt + r, d = 16 s + 8 hh .. + 8
    const int kfrag_b = r * 32 + 16 * (hh ^ ((r >> 3) & 1));
    auto kfrag = [&](const uint16_t* kbuf, int s, int tt) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(kbuf) + kfrag_b + 2048 * s + 1024 * tt);
    };
    // V^T fragment (A operand, rows d = 32 dt + (lane & 31)) for keys
    // kb0 + 4 hh + 0..3 and kb0 + 8 + 4 hh + 0..3 (kb0 = 32 tt + 16 q2):
    // ds_read_b64_tr_b16 gives lane i of a 16-lane group element i & 3 of
    // lanes 4 k + (i >> 2), k = 0..3, so lane j of the group addresses key
    // row (j >> 2) at columns 4 (j & 3) .. + 3 of the group's 16 columns
    const int vfrag_b = (4 * hh + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
    auto vfrag = [&](const uint16_t* vbuf, int kb0, int dt) -> bf16x8 {
        const uint8_t* pv = reinterpret_cast<const uint8_t*>(vbuf) + vfrag_b + 4096 * dt + 64 * kb0;
        const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(pv));
        const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(pv + 512));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    const PairPlan pp = pair_plan(p, a);
    const int lo = chunk_lo(c, pp.total, a.kch), hi = chunk_lo(c + 1, pp.total, a.kch);
    // at most two segments: a piece of tile ta, then a piece of tile tb
#pragma unroll 1
    for (int sg = 0; sg < 2; ++sg) {
        int tile, b0, b1;
        if (sg == 0) {
            tile = pp.ta;
            b0 = lo;
            b1 = hi < pp.na ? hi : pp.na;
        } else {
            tile = pp.tb;
            b0 = (lo > pp.na ? lo : pp.na) - pp.na;
            b1 = hi - pp.na;
        }
        if (tile < 0 || b0 >= b1) continue;          // uniform
        if (sg == 1) wg_barrier();                    // the first segment's buffers are free
        const int nbt = tile_blocks(tile, a.n, a.causal);
        const bool whole = b0 == 0 && b1 == nbt;
        const int64_t q0 = (int64_t)tile * AQW + AQ * half;
        const int64_t qi = q0 + r;                    // this lane's query
        const int qi32 = (int)qi, n32 = (int)a.n;
        // the tile's last block holds its diagonal (causal) or the end of
        // the keys (ragged n): masked
        const bool mask_end = b1 == nbt && (a.causal || (int64_t)nbt * AK > a.n);
        auto blk_base = [&](int kb) -> uint32_t {
            return kb < b1 ? (uint32_t)kb * (uint32_t)AK * row_b : 0x80000000u;
        };

        f32x16 oacc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 16; ++q) oacc[t][q] = 0.0f;
        float m = -INFINITY, lsum = 0.0f;            // running max (base-2 units) and this lane's sum

        issue(blk_base(b0), ks0, koff);
        issue(blk_base(b0), vs0, voff);
        if (active) {
            // Q fragments (B operand): query qi, d = 16 s + 8 hh .. + 8
            bf16x8 qf[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rs, (uint32_t)(qi * row_b + (head * AD + 16 * s + 8 * hh) * 2), 0, 0));
            // S^T = K Q^T for a block's two 32-key tiles; all 16 fragment
            // reads are issued before the first MFMA
            auto scores = [&](const uint16_t* kbuf, f32x16 (&sc)[2]) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int q = 0; q < 16; ++q) sc[tt][q] = 0.0f;
                bf16x8 kf[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) kf[i] = kfrag(kbuf, i >> 1, i & 1);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i >> 1], sc[i & 1], 0, 0, 0);
            };
            // softmax of block kb's scores sc, then O += V^T P^T from vbuf
            auto softmax_pv = [&](int kb, f32x16 (&sc)[2], const uint16_t* vbuf) {
                // lane half hh holds keys 8 j + 4 hh + i of each 32-key tile
                if (mask_end && kb == b1 - 1) {
                    // keys past min(qi, n - 1) (causal) or past n - 1: key
                    // kb AK + off with off = 32 tt + 8 (q >> 2) + 4 hh + (q & 3)
                    int lim = (a.causal && qi32 < n32 ? qi32 : n32 - 1) - kb * AK - 4 * hh;
                    asm volatile("" : "+v"(lim));          // computed here, not hoisted
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int q = 0; q < 16; ++q)
                            if (32 * tt + 8 * (q >> 2) + (q & 3) > lim) sc[tt][q] = -INFINITY;
                }
                // probabilities against the running max m, packed to bf16 as
                // the P^T fragments (K step (tt, q2) = accumulator values
                // 8 q2 .. 8 q2 + 7) and summed as packed (one bf16 dot
                // product with (1, 1) per pair: the sum of exactly the
                // weights the P.V product uses).  Kept while the sum over the
                // lane's 32 keys (which bounds each) stays within ATAU_SUM;
                // otherwise -- and on the first block, m = -inf -- m moves to
                // the block's maximum and the block is redone.
                bf16x8 pf[2][2];
                auto probs = [&](float nmx) -> float {
                    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int q2 = 0; q2 < 2; ++q2) {
                            uint32_t w[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[tt][8 * q2 + 2 * e], a.scale_log2, nmx));
                                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[tt][8 * q2 + 2 * e + 1], a.scale_log2, nmx));
                                w[e] = cvt_bf16x2(p0, p1);
                                ps[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), one2, ps[e], false);
                            }
                            pf[tt][q2] = __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
                        }
                    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
                };
                float psum = probs(-m);
                if (__any(!(psum <= ATAU_SUM))) {           // also catches inf and NaN (m = -inf)
                    float mloc = -INFINITY;
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int q = 0; q < 16; ++q) mloc = fmaxf(mloc, sc[tt][q]);
                    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
                    const float mn = fmaxf(m, mloc * a.scale_log2);
                    const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first block
                    psum = probs(-mn);
                    lsum = lsum * alpha;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int q = 0; q < 16; ++q) oacc[t][q] *= alpha;
                    m = mn;
                }
                lsum += psum;                               // this lane's 32 keys; halves meet at the end
                // O^T += V^T P^T: the A fragment of (tt, q2) holds keys
                // 32 tt + 16 q2 + {4 hh + 0..3, 8 + 4 hh + 0..3}, the order in
                // which the score accumulators hold them
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
                            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(vbuf, 32 * tt + 16 * q2, dt),
                                                                              pf[tt][q2], oacc[dt], 0, 0, 0);
            };
            // one key block kb; buffers alternate with its parity
            auto step = [&](int kb, auto P) {
                constexpr bool odd = decltype(P)::value != 0;
                // K(kb), V(kb) landed (own DMA), then everyone's; all waves
                // are done with block kb-1, whose buffers take block kb+1
                __builtin_amdgcn_s_waitcnt(0x0f70);        // vmcnt(0)
                wg_barrier();
                issue(blk_base(kb + 1), odd ? ks0 : ks1, koff);
                issue(blk_base(kb + 1), odd ? vs0 : vs1, voff);
                f32x16 sc[2];
                scores(odd ? ks1 : ks0, sc);
                softmax_pv(kb, sc, odd ? vs1 : vs0);
            };
            for (int kb = b0; kb < b1; kb += 2) {
                step(kb, std::integral_constant<int, 0>());
                if (kb + 1 < b1) step(kb + 1, std::integral_constant<int, 1>());
            }
        } else {
            // a wave without a head still moves its share of every block
            for (int kb = b0; kb < b1; ++kb) {
                __builtin_amdgcn_s_waitcnt(0x0f70);
                wg_barrier();
                const bool odd = ((kb - b0) & 1) != 0;
                issue(blk_base(kb + 1), odd ? ks0 : ks1, koff);
                issue(blk_base(kb + 1), odd ? vs0 : vs1, voff);
            }
        }
        // the last step issued only zero-fill loads past the segment
        __builtin_amdgcn_s_waitcnt(0x0f70);

        if (!active) continue;
        lsum += __shfl_xor(lsum, 32, 64);
        if (!whole) {
            // this segment's unnormalised O, running max and sum for the combine
            const int64_t slot = ((int64_t)p * a.kch + c) * 2 + sg;
            float* pw = a.part + (((slot * gridDim.y + g) * gridDim.z + blockIdx.z) * AW + wid) * APART;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = 32 * dt + 8 * j + 4 * hh;
                    *reinterpret_cast<float4*>(pw + r * AD + d) =
                        make_float4(oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]);
                }
            if (hh == 0) {
                pw[AQ * AD + r] = m;
                pw[AQ * AD + AQ + r] = lsum;
            }
        } else if (qi < a.n) {
            // out[qi, head, d]: lane holds d = 32 dt + 8 j + 4 hh + i
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
}

// Merges the pieces of a split tile: for query i of head h,
// m* = max_c m_c, out = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c,
// pieces in key order, four at a time with the maximum carried over.
// Block (tile, KV group, quad x AW + wave of the producing workgroup): 256
// threads, thread = (query of the wave's 32: tid / 8, 16 consecutive d).
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a, int nz) {
    const int tile = blockIdx.x;
    const int p = tile < a.ntiles - 1 - tile ? tile : a.ntiles - 1 - tile;
    const int sg = tile == p ? 0 : 1;
    const PairPlan pp = pair_plan(p, a);
    const int s0 = sg == 0 ? 0 : pp.na;
    const int s1 = sg == 0 ? pp.na : pp.total;
    // the pieces: chunks of the pair whose block range meets [s0, s1)
    auto meets = [&](int cc) {
        const int l = chunk_lo(cc, pp.total, a.kch), h = chunk_lo(cc + 1, pp.total, a.kch);
        return (l > s0 ? l : s0) < (h < s1 ? h : s1);
    };
    int npc = 0;
    for (int cc = 0; cc < a.kch; ++cc) npc += meets(cc) ? 1 : 0;
    if (npc <= 1) return;                                // one piece: written directly
    const int g = blockIdx.y;
    const int z = blockIdx.z / AW, wv = blockIdx.z % AW;
    const int hsub = z * 4 + (wv & 3);
    if (hsub >= a.rep) return;
    const int head = g * a.rep + hsub;
    const int qq = threadIdx.x >> 3, d0 = (threadIdx.x & 7) * 16;
    const int64_t qi = (int64_t)tile * AQW + AQ * (wv >> 2) + qq;
    if (qi >= a.n) return;
    auto piece = [&](int cc) -> const float* {
        const int64_t slot = ((int64_t)p * a.kch + cc) * 2 + sg;
        return a.part + (((slot * gridDim.y + g) * nz + z) * AW + wv) * APART;
    };
    // pieces in groups of 4, all of a group's loads in flight together;
    // the running max and sum carry across groups (online, in key order)
    int cf = 0;
    while (!meets(cf)) ++cf;
    int cl = a.kch - 1;
    while (!meets(cl)) --cl;
    float mx = -INFINITY, den = 0.0f, acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    for (int g0 = cf; g0 <= cl; g0 += 4) {
        float mg[4], lg[4];
        float4 og[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = g0 + i;
            if (cc <= cl && meets(cc)) {
                const float* pw = piece(cc);
                mg[i] = pw[AQ * AD + qq];
                lg[i] = pw[AQ * AD + AQ + qq];
#pragma unroll
                for (int e = 0; e < 4; ++e) og[i][e] = *reinterpret_cast<const float4*>(pw + qq * AD + d0 + 4 * e);
            } else {
                mg[i] = -INFINITY;
                lg[i] = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) og[i][e] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
        const float gm = fmaxf(fmaxf(mx, fmaxf(mg[0], mg[1])), fmaxf(mg[2], mg[3]));
        const float f = __builtin_amdgcn_exp2f(mx - gm);           // 0 before the first piece
        den = den * f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = acc[e] * f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float w = __builtin_amdgcn_exp2f(mg[i] - gm);      // 0 for a missing piece
            den = den + w * lg[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[4 * e] = acc[4 * e] + w * og[i][e].x;
                acc[4 * e + 1] = acc[4 * e + 1] + w * og[i][e].y;
                acc[4 * e + 2] = acc[4 * e + 2] + w * og[i][e].z;
                acc[4 * e + 3] = acc[4 * e + 3] + w * og[i][e].w;
            }
        }
        mx = gm;
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
    a.ntiles = (int)((n + AQW - 1) / AQW);
    a.npairs = (a.ntiles + 1) / 2;
    // chunks per pair: about AUNITS workgroups in all, chunks of at least
    // AMINCH blocks
    const int nz = (a.rep + 3) / 4;
    const int64_t per = (int64_t)a.npairs * nkv * nz;
    const int k = (int)((AUNITS + per - 1) / per);
    const int t0 = pair_plan(0, a).total;             // the longest pair (causal: all about equal)
    const int kmax = t0 / AMINCH > 1 ? t0 / AMINCH : 1;
    a.kch = k < kmax ? k : kmax;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)AD);
    return a;
}

}  // namespace

size_t attention_ws_bytes(int64_t n, int nq, int nkv, int causal) {
    if (n <= 0) return 0;
    const AttnArgs a = attn_args(n, nq, nkv, causal);
    if (a.kch <= 1) return 0;                        // every pair in one workgroup: no split tiles
    const int nz = (a.rep + 3) / 4;
    return (size_t)a.npairs * a.kch * 2 * nkv * nz * AW * APART * sizeof(float);
}

hipError_t launch_attention(const void* qkv, int64_t n, int nq, int nkv, int head_dim, int causal, void* out,
                            void* ws, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (head_dim != AD) return hipErrorInvalidValue;
    AttnArgs a = attn_args(n, nq, nkv, causal);
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.out = static_cast<uint16_t*>(out);
    a.part = static_cast<float*>(ws);
    if (a.kch > 1 && !ws) return hipErrorInvalidValue;
    const int nz = (a.rep + 3) / 4;
    hipLaunchKernelGGL(attention_kernel, dim3((unsigned)(a.npairs * a.kch), (unsigned)nkv, (unsigned)nz),
                       dim3(AW * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.kch <= 1) return e;
    hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)a.ntiles, (unsigned)nkv, (unsigned)(nz * AW)),
                       dim3(256), 0, s, a, nz);
    return hipGetLastError();
}

}  // namespace tpk
