// GEMMs of the rank shard: C[M, N] = A[M, K] . B[N, K]^T, both operands
// contiguous along K (weights stored [out, in], x . W^T), and the fused
// column-parallel gate_up form act = SiLU(A . G^T) * (A . U^T) with
// B = [G ; U] (gate rows first).  bf16 operands, fp32 accumulation on MFMAs.
//
// Kernels, and the shapes plan_gemm gives them:
//   * gemm_bf16_pipe_kernel: direct-to-LDS tiles on v_mfma_f32_16x16x32_bf16
//     with a deep LDS pipeline -- 256 x 256 tiles for large products (paired
//     K = 64 stages; a part-filled last round of tiles is cut into K pieces
//     that tail_fixup_kernel adds), 256 x 192 tiles with K split in two and
//     128 x 192 tiles for products with few output tiles, 64 x 128 tiles for
//     the split-K tiles of small products.
//   * gemm_bf16_dl_kernel: direct-to-LDS 128 x 128 tiles on 32x32x16 MFMAs,
//     two workgroups per CU, for mid-sized products.
//   * gemm_bf16_kernel: register-staged tiles with element-wise loads, for
//     operands the 16-byte buffer loads cannot serve (unaligned, or K not a
//     multiple of 8).
//   * gemm_bf16_rs_kernel + rs_finalize_kernel: decode products (M <= 64)
//     with the weights streamed from HBM straight into MFMA fragments, K
//     cut into slices whose fp32 partial tiles the finish pass adds.
//   * gemm_bf16_stream_kernel + stream_finalize_kernel: decode products too
//     small in 16-row blocks for the register-streaming grid, streamed
//     through an LDS ring.
//   * splitk_finalize_kernel: adds split-K partials in split order and
//     applies the epilogue.
// Common to all of them:
//   * gated epilogue: a tile loads BN/2 gate rows and the SAME BN/2 up rows,
//     so a lane holds gate and up accumulators of the same (row, column) and
//     applies SiLU(g) * u in registers; gate/up products never reach memory;
//   * every partial sum (split-K, K pieces, K slices) is added in a fixed
//     order by a finish pass: deterministic, no atomics;
//   * tile order: workgroups are dispatched round-robin over the 8 XCDs; the
//     linear block id is remapped so that each XCD receives a contiguous run
//     of tiles, grouped GROUP_M tiles tall so that the operand panels a run
//     shares stay in that XCD's L2.
//
// The fp32 kernels are in gemm_f32.hip.
#include <stdlib.h>

#include <type_traits>
#include <utility>

#include "common.hpp"

namespace tpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_STORE_BF16 = 0, EPI_STORE_F32 = 1, EPI_GATED_BF16 = 2, EPI_SPLIT = 3 };

struct GemmArgs {
    const uint16_t* A;      // [M, K]
    const uint16_t* B;      // [Nb, K]
    const uint16_t* bias;   // [N] or null (store epilogues only)
    void* C;                // output [M, N], or fp32 workspace [splits][M][Nb]
    int64_t M, N, K, Nb;    // N = output columns (act columns when gated)
    int64_t k_split;        // K elements per split
    int tiles_m, tiles_n;
    int vec_out;            // 1: output row length and base allow 8/16-byte stores
    // balanced last round (direct-to-LDS kernel): blocks >= full_tiles are
    // K pieces of the remaining tiles, tail_split pieces of tail_k each,
    // written as fp32 [BM][BN] partial tiles to tail_ws
    int full_tiles, tail_split;
    int64_t tail_k;
    float* tail_ws;
};

constexpr int GROUP_M = 8;

// Workgroup barrier without a memory fence: memory operations in flight
// (the next tiles' DMA, fragment reads) are not waited for; the kernels
// wait for what they need with explicit counters.  The compiler-only fences
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// logical tile id -> (tile row, tile column), grouped GROUP_M tile rows tall
__host__ __device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int per_group = GROUP_M * tiles_n;
    const int group = b / per_group;
    const int first_m = group * GROUP_M;
    int gsize = tiles_m - first_m;
    if (gsize > GROUP_M) gsize = GROUP_M;
    const int in_group = b - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
    const int nb = tiles_m * tiles_n;
    int b = blockIdx.x;
    // XCD-aware remap: block b executes on XCD (b mod 8); give each XCD a
    // contiguous range of logical tile ids.
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    const int per_group = GROUP_M * tiles_n;
    const int group = b / per_group;
    const int first_m = group * GROUP_M;
    int gsize = tiles_m - first_m;
    if (gsize > GROUP_M) gsize = GROUP_M;
    const int in_group = b - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

// B-tile row base of MFMA tile i of wave column wn (output-column side).
// Gated tiles: the first TN/2 tiles are gate rows, the rest the same up rows.
template <int BN, int WN, bool GATED, int RB = 32>
__device__ __forceinline__ int b_tile_row_of(int i, int wn) {
    constexpr int WTN = BN / WN, TN = WTN / RB;
    if (GATED) {
        constexpr int HALF_W = WTN / 2;
        return i < TN / 2 ? wn * HALF_W + i * RB : BN / 2 + wn * HALF_W + (i - TN / 2) * RB;
    }
    return wn * WTN + i * RB;
}

// Stores 4 consecutive output columns gn .. gn+3 of output row gm: fp32
// split-K partials (row length Nb), or C (+bias) in bf16/fp32, or the gated
// activation (v already holds SiLU(g)*u).  Columns past the end are skipped.
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs& p, int64_t gm, int64_t gn, float (&v)[4]) {
    if (EPI == EPI_SPLIT) {
        float* dst = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.M * p.Nb + gm * p.Nb + gn;
        if (p.vec_out && gn + 3 < p.Nb) {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (gn + q < p.Nb) dst[q] = v[q];
        }
        return;
    }
    if (EPI != EPI_GATED_BF16 && p.bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (gn + q < p.N) v[q] = v[q] + bf16_to_f32(p.bias[gn + q]);
    }
    if (EPI == EPI_STORE_F32) {
        float* dst = static_cast<float*>(p.C) + gm * p.N + gn;
        if (p.vec_out && gn + 3 < p.N) {
            // a final fp32 output (the LM head's logits) is not read back
            // here: non-temporal stores (135 -> 116 us at the Qwen3 vocab
            // shard; the same hint on 8-byte bf16 stores made o_proj 2.5x
            // slower)
            typedef float f32x4v __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store((f32x4v){v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4v*>(dst));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (gn + q < p.N) dst[q] = v[q];
        }
    } else {
        uint16_t* dst = static_cast<uint16_t*>(p.C) + gm * p.N + gn;
        if (p.vec_out && gn + 3 < p.N) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (gn + q < p.N) dst[q] = f32_to_bf16(v[q]);
        }
    }
}

// Writes one workgroup's accumulators: split-K partials (fp32), the gated
// SiLU(g)*u activation (bf16), or C (+bias) in bf16/fp32.  Lane l holds
// output row (l & 31) and columns 8g + 4(l >> 5) + q of each 32x32 tile.
template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p, f32x16 (&acc)[BN / WN / 32][BM / WM / 32],
                                              int64_t m0, int64_t n0, int wm, int wn, int lane) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    auto b_tile_row = [&](int i) { return b_tile_row_of<BN, WN, GATED>(i, wn); };
    const int mrow = lane & 31;
    const int ncol = 4 * (lane >> 5);
    if (EPI == EPI_SPLIT) {
        float* ws = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.M * p.Nb;
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int64_t gm = m0 + wm * WTM + j * 32 + mrow;
            if (gm >= p.M) continue;
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t gn = n0 + b_tile_row(i) + 8 * g + ncol;
                    float* dst = ws + gm * p.Nb + gn;
                    if (p.vec_out && gn + 3 < p.Nb) {
                        *reinterpret_cast<float4*>(dst) =
                            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (gn + q < p.Nb) dst[q] = acc[i][j][4 * g + q];
                    }
                }
        }
    } else if (GATED) {
        uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int64_t gm = m0 + wm * WTM + j * 32 + mrow;
            if (gm >= p.M) continue;
#pragma unroll
            for (int i = 0; i < TN / 2; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t gn = n0 + wn * (WTN / 2) + i * 32 + 8 * g + ncol;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = silu_mul(acc[i][j][4 * g + q], acc[i + TN / 2][j][4 * g + q]);
                    uint16_t* dst = C + gm * p.N + gn;
                    if (p.vec_out && gn + 3 < p.N) {
                        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (gn + q < p.N) dst[q] = f32_to_bf16(v[q]);
                    }
                }
        }
    } else {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int64_t gm = m0 + wm * WTM + j * 32 + mrow;
            if (gm >= p.M) continue;
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t gn = n0 + b_tile_row(i) + 8 * g + ncol;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[q] = acc[i][j][4 * g + q];
                        if (p.bias && gn + q < p.N) v[q] = v[q] + bf16_to_f32(p.bias[gn + q]);
                    }
                    if (EPI == EPI_STORE_F32) {
                        float* dst = static_cast<float*>(p.C) + gm * p.N + gn;
                        if (p.vec_out && gn + 3 < p.N) {
                            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (gn + q < p.N) dst[q] = v[q];
                        }
                    } else {
                        uint16_t* dst = static_cast<uint16_t*>(p.C) + gm * p.N + gn;
                        if (p.vec_out && gn + 3 < p.N) {
                            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (gn + q < p.N) dst[q] = f32_to_bf16(v[q]);
                        }
                    }
                }
        }
    }
}

// Register-staged tiles (v_mfma_f32_32x32x16_bf16): element-wise global
// loads staged through registers into double-buffered LDS (the next K tile
// is fetched while the MFMAs run on the current one; one barrier per K
// step).  Each tile row is BK = 64 bf16 = 8 16-byte chunks, chunk c of row r
// stored at position swz(r, c), which keeps the row-wise 16-byte stores and
// the fragment loads (32 rows, one chunk) free of bank conflicts.
// Output tile of one workgroup: BM rows of A (tokens) x BN rows of B
// (weight rows = output columns; gated: BN/2 gate rows + the same BN/2 up
// rows).  The weight fragment is the MFMA's A operand and the token fragment
// its B operand, so in each 32x32 result lane l holds token row (l & 31) and
// output columns 8g + 4(l >> 5) + q, q = 0..3: four consecutive columns per
// group g, written with one 8-byte (bf16) or 16-byte (fp32) store.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmArgs p) {
    constexpr int BK = 64;
    constexpr int NT = WM * WN * 64;
    constexpr int KC = BK / 8;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    constexpr int A_LD = BM * KC / NT;
    constexpr int B_LD = BN * KC / NT;
    static_assert(KC == 8, "swizzle assumes 8 chunks per row");
    static_assert(BM * KC % NT == 0 && BN * KC % NT == 0, "tile/threads mismatch");
    static_assert(!GATED || TN % 2 == 0, "gated tiles pair gate and up MFMA tiles");
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;

    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;

    int tile_m, tile_n;
    tile_coords(p.tiles_m, p.tiles_n, tile_m, tile_n);
    const int64_t m0 = (int64_t)tile_m * BM;
    const int64_t n0 = GATED ? (int64_t)tile_n * (BN / 2) : (int64_t)tile_n * BN;
    const int64_t k_begin = (int64_t)blockIdx.y * p.k_split;
    int64_t k_end = k_begin + p.k_split;
    if (k_end > p.K) k_end = p.K;

    const uint16_t* __restrict__ A = p.A;
    const uint16_t* __restrict__ B = p.B;

    // global row of B for local tile row lr (gated: gate rows then the same up rows)
    auto b_row = [&](int lr, bool& ok) -> int64_t {
        if (GATED) {
            const int half = BN / 2;
            const int64_t c = n0 + (lr < half ? lr : lr - half);
            ok = c < p.N;
            return lr < half ? c : p.N + c;
        }
        const int64_t r = n0 + lr;
        ok = r < p.Nb;
        return r;
    };

    // ---- global -> register staging ------------------------------------
    // Element-wise loads: this kernel serves operands the 16-byte buffer
    // loads of the other kernels cannot (K not a multiple of 8, or operands
    // not 16-byte aligned).  Rows outside the matrix and K past the end of
    // the range read as zero.
    u32x4 ra[A_LD], rb[B_LD];

    auto load_tile = [&](int64_t k0) {
        // element-wise path (K not a multiple of 8 or unaligned operands)
        auto load_chunk = [&](const uint16_t* src, int64_t row, bool ok, int64_t k) -> u32x4 {
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t lo = 0, hi = 0;
                if (ok && k + 2 * q < k_end) lo = src[row * p.K + k + 2 * q];
                if (ok && k + 2 * q + 1 < k_end) hi = src[row * p.K + k + 2 * q + 1];
                w[q] = lo | (hi << 16);
            }
            return u32x4{w[0], w[1], w[2], w[3]};
        };
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int v = tid + i * NT;
            const int row = v / KC, kc = v % KC;
            ra[i] = load_chunk(A, m0 + row, m0 + row < p.M, k0 + kc * 8);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int v = tid + i * NT;
            const int row = v / KC, kc = v % KC;
            bool ok;
            const int64_t gb = b_row(row, ok);
            rb[i] = load_chunk(B, gb, ok, k0 + kc * 8);
        }
    };

    auto store_tile = [&](int buf) {
        uint16_t* As = smem + buf * (A_ELEMS + B_ELEMS);
        uint16_t* Bs = As + A_ELEMS;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int v = tid + i * NT;
            const int row = v / KC, kc = v % KC;
            *reinterpret_cast<u32x4*>(As + row * BK + swz(row, kc) * 8) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int v = tid + i * NT;
            const int row = v / KC, kc = v % KC;
            *reinterpret_cast<u32x4*>(Bs + row * BK + swz(row, kc) * 8) = rb[i];
        }
    };

    // B-tile row base of the wave's MFMA tile i (output-column side)
    auto b_tile_row = [&](int i) -> int {
        if (GATED) {
            constexpr int HALF_W = WTN / 2;     // gate (or up) rows per wave
            return i < TN / 2 ? wn * HALF_W + i * 32 : BN / 2 + wn * HALF_W + (i - TN / 2) * 32;
        }
        return wn * WTN + i * 32;
    };

    // fragments, double-buffered in registers: sub-step kk+1 is read from LDS
    // while the MFMAs of sub-step kk run
    bf16x8 wf[2][TN], xf[2][TM];
    auto read_frags = [&](int buf, int kk, int slot) {
        const uint16_t* As = smem + buf * (A_ELEMS + B_ELEMS);
        const uint16_t* Bs = As + A_ELEMS;
        const int c = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const int row = b_tile_row(i) + (lane & 31);
            wf[slot][i] = *reinterpret_cast<const bf16x8*>(Bs + row * BK + swz(row, c) * 8);
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int row = wm * WTM + j * 32 + (lane & 31);
            xf[slot][j] = *reinterpret_cast<const bf16x8*>(As + row * BK + swz(row, c) * 8);
        }
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- main loop -------------------------------------------------------
    // LDS buffer (kt & 1) holds K tile kt.  One K step = 4 sub-steps of 16;
    // while the MFMAs of sub-step kk run, the fragments of kk+1 are read
    // (register double buffer).  Tile kt+1 (staged in registers) is written
    // to the other LDS buffer during sub-step 0, tile kt+2 is fetched into
    // the registers during sub-step 1, and the barrier sits before sub-step
    // 3, whose MFMAs cover the reads of the next tile's first fragments.
    // The last two K steps are peeled so the steady-state body has no
    // branches and the interleave hints apply to one scheduling region.
    constexpr int MF = TN * TM;          // MFMAs per sub-step
    constexpr int NR = TN + TM;          // fragment reads per sub-step
    constexpr int NW = A_LD + B_LD;      // 16-byte LDS writes (and global loads) per K step

    auto mfma_step = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[slot][i], xf[slot][j], acc[i][j], 0, 0, 0);
    };

    auto k_step = [&](int kt, auto store_c, auto load_c, auto next_c) {
        constexpr bool STORE = decltype(store_c)::value;   // tile kt+1 -> other LDS buffer
        constexpr bool LOAD = decltype(load_c)::value;     // fetch tile kt+2
        constexpr bool NEXT = decltype(next_c)::value;     // read tile kt+1's first fragments
        const int cur = kt & 1;
        // sub-step 0
        read_frags(cur, 1, 1);
        if (STORE) store_tile(cur ^ 1);
        mfma_step(0);
#pragma unroll
        for (int q = 0; q < MF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (STORE && q < NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        // sub-step 1
        read_frags(cur, 2, 0);
        if (LOAD) load_tile(k_begin + (int64_t)(kt + 2) * BK);
        mfma_step(1);
#pragma unroll
        for (int q = 0; q < MF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (LOAD && q < NW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        // sub-step 2
        read_frags(cur, 3, 1);
        mfma_step(0);
#pragma unroll
        for (int q = 0; q < MF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __syncthreads();
        // sub-step 3
        if (NEXT) read_frags(cur ^ 1, 0, 0);
        mfma_step(1);
#pragma unroll
        for (int q = 0; q < MF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (NEXT && q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    const int nk = (int)ceil_div(k_end - k_begin, BK);
    if (nk > 0) {
        load_tile(k_begin);
        store_tile(0);
        if (nk > 1) load_tile(k_begin + BK);
        __syncthreads();
        read_frags(0, 0, 0);
        int kt = 0;
        for (; kt + 2 < nk; ++kt) k_step(kt, T_{}, T_{}, T_{});
        if (kt + 1 < nk) {
            k_step(kt, T_{}, F_{}, T_{});
            ++kt;
        }
        k_step(kt, F_{}, F_{}, F_{});
    }

    gemm_epilogue<BM, BN, WM, WN, EPI>(p, acc, m0, n0, wm, wn, lane);
}

// Which output tile and K range a workgroup of the tiled kernels owns.
// Whole tiles come first, remapped so that each XCD (block b runs on XCD
// b mod 8) gets a contiguous range of logical tile ids; with a balanced last
// round the remaining tiles follow as tail_split K pieces each.
struct Unit {
    int tile_m, tile_n;
    int64_t k_begin, k_end;
    bool tail;
};
__device__ __forceinline__ Unit unit_of(const GemmArgs& p) {
    Unit u;
    const int bid = blockIdx.x;
    u.tail = p.tail_split > 1 && bid >= p.full_tiles;
    if (!u.tail) {
        int b = bid;
        const int nb = p.tail_split > 1 ? p.full_tiles : p.tiles_m * p.tiles_n;
        if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
        tile_of(b, p.tiles_m, p.tiles_n, u.tile_m, u.tile_n);
        u.k_begin = (int64_t)blockIdx.y * p.k_split;
        u.k_end = u.k_begin + p.k_split;
    } else {
        const int v = bid - p.full_tiles;
        tile_of(p.full_tiles + v / p.tail_split, p.tiles_m, p.tiles_n, u.tile_m, u.tile_n);
        u.k_begin = (int64_t)(v % p.tail_split) * p.tail_k;
        u.k_end = u.k_begin + p.tail_k;
    }
    if (u.k_end > p.K) u.k_end = p.K;
    return u;
}

// A K piece of a balanced-last-round tile: the fp32 partial tile [BM][BN]
// in B-row order (gated: gate rows, then up rows) goes to the workspace.
template <int BM, int BN, int WM, int WN, bool GATED>
__device__ __forceinline__ void store_tail_piece(const GemmArgs& p, f32x16 (&acc)[BN / WN / 32][BM / WM / 32],
                                                 int wm, int wn, int lane) {
    constexpr int WTM = BM / WM, TM = WTM / 32, TN = BN / WN / 32;
    float* t = p.tail_ws + (int64_t)(blockIdx.x - p.full_tiles) * BM * BN;
    const int mrow = lane & 31, ncol = 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int lm = wm * WTM + j * 32 + mrow;
                const int ln = b_tile_row_of<BN, WN, GATED>(i, wn) + 8 * g + ncol;
                *reinterpret_cast<float4*>(t + lm * BN + ln) =
                    make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            }
}

// Direct-to-LDS variant (16-byte-aligned operands, K a multiple of 8).
// Tiles move from global memory straight into LDS with buffer_load ... lds:
// one wave instruction fills 64 consecutive 16-byte LDS slots, lane l writing
// slot l.  LDS layout: each tile row is its BK = 64 bf16 (8 slots) followed by
// one pad slot, a row stride of 144 bytes.  Fragment reads (32 rows, one
// 16-byte chunk) then hit 32 distinct banks groups for 32- and 64-bank LDS,
// and the chunk of sub-step kk is at a constant offset (32 kk bytes) from a
// per-fragment base, so reads use immediate offsets.  Lanes that land on a
// pad slot fetch with an out-of-range offset and write zeros.  No VGPR
// staging and no LDS stores: tile kt+1 streams into the other LDS buffer
// while tile kt is multiplied; one wait + barrier per K step.  The two LDS
// buffers are distinct objects so that the compiler's wait insertion can
// tell the in-flight next tile from the one being read.
template <int BM, int BN, int WM, int WN, int EPI, bool KTAIL, int NST>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_dl_kernel(GemmArgs p) {
    constexpr int BK = 64;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    constexpr int RS = 9;                        // 16-byte slots per LDS row (8 data + 1 pad)
    constexpr int ROWB = RS * 16;                // row stride in bytes
    constexpr int A_SLOTS = BM * RS, B_SLOTS = BN * RS;
    static_assert(A_SLOTS % 64 == 0 && B_SLOTS % 64 == 0, "tiles must fill whole 64-slot blocks");
    constexpr int A_INSTR = A_SLOTS / 64, N_INSTR = (A_SLOTS + B_SLOTS) / 64;
    constexpr int PER_WAVE = (N_INSTR + NW - 1) / NW;
    static_assert(!GATED || TN % 2 == 0, "gated tiles pair gate and up MFMA tiles");
    constexpr int BUF_BYTES = (A_SLOTS + B_SLOTS) * 16;
    constexpr uint32_t SENT = 0x80000000u;

    static_assert(NST >= 2, "at least double buffering");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;

    int tile_m, tile_n;
    int64_t k_begin, k_end;
    const int bid = blockIdx.x;
    const bool tail_unit = p.tail_split > 1 && bid >= p.full_tiles;
    if (!tail_unit) {
        int b = bid;
        const int nb = p.tail_split > 1 ? p.full_tiles : p.tiles_m * p.tiles_n;
        // XCD-aware remap: block b executes on XCD (b mod 8); give each XCD
        // a contiguous range of logical tile ids
        if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
        tile_of(b, p.tiles_m, p.tiles_n, tile_m, tile_n);
        k_begin = (int64_t)blockIdx.y * p.k_split;
        k_end = k_begin + p.k_split;
    } else {
        const int u = bid - p.full_tiles;
        tile_of(p.full_tiles + u / p.tail_split, p.tiles_m, p.tiles_n, tile_m, tile_n);
        k_begin = (int64_t)(u % p.tail_split) * p.tail_k;
        k_end = k_begin + p.tail_k;
    }
    if (k_end > p.K) k_end = p.K;
    const int64_t m0 = (int64_t)tile_m * BM;
    const int64_t n0 = GATED ? (int64_t)tile_n * (BN / 2) : (int64_t)tile_n * BN;

    auto b_row = [&](int lr, bool& ok) -> int64_t {
        if (GATED) {
            const int half = BN / 2;
            const int64_t c = n0 + (lr < half ? lr : lr - half);
            ok = c < p.N;
            return lr < half ? c : p.N + c;
        }
        const int64_t r = n0 + lr;
        ok = r < p.Nb;
        return r;
    };

    // per (instruction, lane): byte offset of the chunk within the tile's
    // K window (SENT for pads and rows outside the matrix), and its chunk
    // index (for the partial last K tile)
    uint32_t off[PER_WAVE];
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
        const int j = wid * PER_WAVE + q;
        const int slot = j * 64 + lane;
        off[q] = SENT;
        if (j < N_INSTR) {
            if (slot < A_SLOTS) {
                const int r = slot / RS, c = slot % RS;
                if (c < 8 && m0 + r < p.M) off[q] = (uint32_t)(((int64_t)r * p.K + c * 8) * 2);
            } else {
                const int sb = slot - A_SLOTS;
                const int r = sb / RS, c = sb % RS;
                bool ok;
                const int64_t gb = b_row(r, ok);
                if (c < 8 && ok) off[q] = (uint32_t)(((gb - n0) * p.K + c * 8) * 2);
            }
        }
    }
    const uint16_t* a_tile = p.A + m0 * p.K;
    const uint16_t* b_tile = p.B + n0 * p.K;

    // KTAIL: the K range may end inside a tile (K or the split length not a
    // multiple of BK); chunks at or past k_end are then fetched as zeros.
    auto issue_tile = [&](int64_t k0, uint8_t* buf) {
        __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(a_tile + k0), (short)0, 0x7fffffff, 0x00020000);
        __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)(b_tile + k0), (short)0, 0x7fffffff, 0x00020000);
        const bool tail = KTAIL && k0 + BK > k_end;
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int j = wid * PER_WAVE + q;
            if (PER_WAVE * NW != N_INSTR && j >= N_INSTR) break;
            uint32_t o = off[q];
            if (KTAIL && tail) {
                // chunk index of this lane's slot (pads count as chunk 8)
                const int slot = j * 64 + lane;
                const int c = (slot < A_SLOTS ? slot : slot - A_SLOTS) % RS;
                if (k0 + c * 8 >= k_end) o = SENT;
            }
            auto* dst = (__attribute__((address_space(3))) void*)(buf + j * 1024);
            if (j < A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, o, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, o, 0, 0, 0);
        }
    };

    // fragment bases (bytes within a buffer); sub-step kk adds 32 kk
    int fb_w[TN], fb_x[TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
        fb_w[i] = A_SLOTS * 16 + (b_tile_row_of<BN, WN, GATED>(i, wn) + (lane & 31)) * ROWB + (lane >> 5) * 16;
#pragma unroll
    for (int j = 0; j < TM; ++j) fb_x[j] = (wm * WTM + j * 32 + (lane & 31)) * ROWB + (lane >> 5) * 16;

    bf16x8 wf[2][TN], xf[2][TM];
    auto read_frags = [&](const uint8_t* buf, int kk, int slot) {
#pragma unroll
        for (int i = 0; i < TN; ++i) wf[slot][i] = *reinterpret_cast<const bf16x8*>(buf + fb_w[i] + kk * 32);
#pragma unroll
        for (int j = 0; j < TM; ++j) xf[slot][j] = *reinterpret_cast<const bf16x8*>(buf + fb_x[j] + kk * 32);
    };

    f32x16 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    constexpr int MF = TN * TM;          // MFMAs per 16-wide sub-step
    constexpr int NR = TN + TM;          // fragment reads per sub-step
    auto mfma_step = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int j = 0; j < TM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[slot][i], xf[slot][j], acc[i][j], 0, 0, 0);
    };
    // one MFMA, one fragment read, ... so reads overlap the matrix pipe
    auto interleave = [&](bool reads) {
#pragma unroll
        for (int q = 0; q < MF; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (reads && q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    // LDS ring of NST stages: stage (kt mod NST) holds K tile kt; tiles
    // kt+1 .. kt+NST-1 are in flight while tile kt is multiplied.
    // One K step: issue tile kt+NST-1 (into the stage tile kt-1 used, free
    // since the previous barrier), sub-steps 0..2 read the next sub-step's
    // fragments under the current MFMAs, then wait until tile kt+1 has
    // landed (this wave's DMA, then the barrier for everyone's), and
    // sub-step 3 reads tile kt+1's first fragments under its MFMAs.
    constexpr int PW_MIN = N_INSTR / NW;             // DMA instructions per tile, any wave
    constexpr int VM_AHEAD = (NST - 2) * PW_MIN < 63 ? (NST - 2) * PW_MIN : 63;
    auto stage = [&](int s) { return lds + s * BUF_BYTES; };
    const int nk = (int)ceil_div(k_end - k_begin, BK);
    auto kof = [&](int t) { return k_begin + (int64_t)t * BK; };
    if (nk > 0) {
#pragma unroll
        for (int t = 0; t < NST - 1; ++t)
            if (t < nk) issue_tile(kof(t), stage(t));
        if (nk >= NST - 1)
            __builtin_amdgcn_s_waitcnt(0x0f70 | (VM_AHEAD & 15) | ((VM_AHEAD >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        read_frags(stage(0), 0, 0);
        int rs = 0;                                  // stage of tile kt
        auto k_step = [&](int kt, auto more_c) {
            constexpr bool MORE = decltype(more_c)::value;   // a tile kt+1 follows
            const uint8_t* cur = stage(rs);
            const int rn = rs + 1 == NST ? 0 : rs + 1;
            const bool issue = MORE && kt + NST - 1 < nk;
            if (issue) issue_tile(kof(kt + NST - 1), stage(rs == 0 ? NST - 1 : rs - 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) {
                read_frags(cur, kk + 1, (kk + 1) & 1);
                mfma_step(kk & 1);
                interleave(true);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (MORE) {
                if (issue)
                    __builtin_amdgcn_s_waitcnt(0x0f70 | (VM_AHEAD & 15) | ((VM_AHEAD >> 4) << 14));
                else
                    __builtin_amdgcn_s_waitcnt(0x0f70);
                __syncthreads();
                read_frags(stage(rn), 0, 0);
            }
            mfma_step(1);
            interleave(MORE);
            __builtin_amdgcn_sched_barrier(0);
            rs = rn;
        };
        for (int kt = 0; kt + 1 < nk; ++kt) k_step(kt, std::true_type{});
        k_step(nk - 1, std::false_type{});
    }
    if (tail_unit) {
        // fp32 partial tile [BM][BN] in B-row order (gated: gate then up columns)
        float* t = p.tail_ws + (int64_t)(bid - p.full_tiles) * BM * BN;
        const int mrow = lane & 31, ncol = 4 * (lane >> 5);
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int lm = wm * WTM + j * 32 + mrow;
                    const int ln = b_tile_row_of<BN, WN, GATED>(i, wn) + 8 * g + ncol;
                    *reinterpret_cast<float4*>(t + lm * BN + ln) =
                        make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                }
        return;
    }
    gemm_epilogue<BM, BN, WM, WN, EPI>(p, acc, m0, n0, wm, wn, lane);
}

// fp32 plain-store epilogue of the 16x16x32 kernels through LDS (the LM
// head's logits): the results are written to LDS in the MFMA's lane layout
// (4 consecutive output columns of one token) and read back as whole 1 KiB
// output rows, so each wave store is 1 KiB of contiguous output instead of
// 16 rows x 64 bytes; they go out with non-temporal stores (the logits are
// not read back here).  Two passes of 128 token rows (the waves with wm = 0,
// then wm = 1); the 16-byte slot s of token row t sits at s ^ (t & 15), so
// writes and reads are conflict-free.  Same-box A/B at the Qwen3 vocab
// shard: 105 vs 118 us on one machine, equal (118 us) on another; the same
// staging for bf16 outputs (o_proj, down) measured no gain, so they store
// directly.  The caller's LDS ring is free: no DMA is in
// flight after the last K step, and a barrier waits for the last fragment
// reads.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void staged_store_f32(const GemmArgs& p, f32x4 (&acc)[BN / WN / 16][BM / WM / 16],
                                                 uint8_t* lds, int64_t m0, int64_t n0, int wm, int wn, int lane) {
    constexpr int WTM = BM / WM;
    constexpr int TM = WTM / 16, TN = BN / WN / 16;
    constexpr int NT = WM * WN * 64;
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int tl = lane & 15, cl = 4 * (lane >> 4);
    float* C = static_cast<float*>(p.C);
    __builtin_amdgcn_s_waitcnt(0x0070);                 // vmcnt(0) lgkmcnt(0)
    bare_barrier();
#pragma unroll
    for (int h = 0; h < WM; ++h) {
        if (h > 0) {
            __builtin_amdgcn_s_waitcnt(0xc07f);         // lgkmcnt(0): last pass's reads done
            bare_barrier();
        }
        if (wm == h) {
#pragma unroll
            for (int j = 0; j < TM; ++j)
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int t = j * 16 + tl;
                    const int col = b_tile_row_of<BN, WN, false, 16>(i, wn) + cl;
                    float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                    if (p.bias) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (n0 + col + q < p.N) v[q] = v[q] + bf16_to_f32(p.bias[n0 + col + q]);
                    }
                    const int slot = (col >> 2) ^ (t & 15);
                    *reinterpret_cast<f32x4v*>(lds + t * (BN * 4) + slot * 16) = (f32x4v){v[0], v[1], v[2], v[3]};
                }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0): this pass's writes done
        bare_barrier();
        constexpr int PIECES = WTM * BN / 4;                // 16-byte pieces of the pass
#pragma unroll 4
        for (int pc = threadIdx.x; pc < PIECES; pc += NT) {
            const int t = pc / (BN / 4), k = pc % (BN / 4);
            const int64_t gm = m0 + h * WTM + t, gn = n0 + 4 * k;
            if (gm >= p.M || gn >= p.N) continue;
            const f32x4v x = *reinterpret_cast<const f32x4v*>(lds + t * (BN * 4) + 16 * (k ^ (t & 15)));
            float* dst = C + gm * p.N + gn;
            if (gn + 3 < p.N) {
                __builtin_nontemporal_store(x, reinterpret_cast<f32x4v*>(dst));
            } else {
                for (int e = 0; gn + e < p.N; ++e) dst[e] = x[e];
            }
        }
    }
}

// Direct-to-LDS loads of paired stages (K = 64, tile rows of 128 bytes):
// one wave instruction fetches 8 tile rows x 128 contiguous bytes, whole
// 128-byte lines.  Chunk c of tile row r sits at position c ^ ((r >> 1) & 7),
// so the 16 rows of one fragment read fall in 16 distinct 16-byte bank
// groups (rows alternate between the two 128-byte halves of the 256 bytes
// the 64 banks cover); lane l of an instruction fills slot l and fetches
// the chunk that belongs there.  A stage holds BM A rows, then BN B rows
// (gated: BN/2 gate rows, then the same BN/2 up rows).  Rows past the end
// of the operand get an offset past the buffer's range, which loads zeros.
template <int BM, int BN, int NW, bool GATED>
struct PairDma {
    static constexpr int ROW2 = 128;                          // bytes per tile row
    static constexpr int STAGE2 = (BM + BN) * ROW2;
    static constexpr int N2 = STAGE2 / 1024, A2 = BM * ROW2 / 1024;
    static_assert(N2 % NW == 0, "each wave issues the same number of DMA instructions");
    static constexpr int PW2 = N2 / NW;                       // instructions per wave and stage
    static constexpr uint32_t SENT = 0x80000000u;
    uint32_t off[PW2];
    const uint16_t* a_tile;
    const uint16_t* b_tile;
    int wid;

    __device__ __forceinline__ PairDma(const GemmArgs& p, int64_t m0, int64_t n0, int wid_, int lane)
        : a_tile(p.A + m0 * p.K), b_tile(p.B + n0 * p.K), wid(wid_) {
#pragma unroll
        for (int q = 0; q < PW2; ++q) {
            const int j = wid * PW2 + q;
            const int r = j * 8 + (lane >> 3);                // tile row; (r >> 1) & 7 = (4 (j & 1) + (lane >> 4)) & 7
            const int c = (lane & 7) ^ ((4 * (j & 1) + (lane >> 4)) & 7);
            off[q] = SENT;
            if (j < A2) {
                if (m0 + r < p.M) off[q] = (uint32_t)(((int64_t)r * p.K + c * 8) * 2);
            } else {
                const int lr = r - BM;
                int64_t gb;
                bool ok;
                if (GATED) {
                    const int half = BN / 2;
                    const int64_t cc = n0 + (lr < half ? lr : lr - half);
                    ok = cc < p.N;
                    gb = lr < half ? cc : p.N + cc;
                } else {
                    gb = n0 + lr;
                    ok = gb < p.Nb;
                }
                if (ok) off[q] = (uint32_t)(((gb - n0) * p.K + c * 8) * 2);
            }
        }
    }

    // stage K = k0 .. k0 + 63 into the STAGE2 bytes at buf
    __device__ __forceinline__ void issue(int64_t k0, uint8_t* buf) const {
        __amdgpu_buffer_rsrc_t rsa =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a_tile + k0), (short)0, 0x7fffffff, 0x00020000);
        __amdgpu_buffer_rsrc_t rsb =
            __builtin_amdgcn_make_buffer_rsrc((void*)(b_tile + k0), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int q = 0; q < PW2; ++q) {
            const int j = wid * PW2 + q;
            const uint32_t o = off[q];
            auto* dst = (__attribute__((address_space(3))) void*)(buf + j * 1024);
            if (j < A2)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, o, 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, o, 0, 0, 0);
        }
    }
};

// s_waitcnt immediate for vmcnt(n) with lgkmcnt and expcnt left alone
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// Epilogue of the direct-to-LDS kernels (16x16 blocks, acc[i][j]: weight
// block i, token block j; lane l holds rows (output columns)
// b_row(i) + 4 (l >> 4) + q of column (token) wm WTM + 16 j + (l & 15)).
// A balanced-last-round K piece goes to the fp32 tail workspace in B-row
// order; otherwise the tile goes through the epilogue (fp32 rows staged
// through LDS when the output allows 16-byte stores).
template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void pipe_epilogue(const GemmArgs& p, bool tail, f32x4 (&acc)[BN / WN / 16][BM / WM / 16],
                                              uint8_t* lds, int64_t m0, int64_t n0, int wm, int wn, int lane) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    const int mrow = lane & 15, ncol = 4 * (lane >> 4);
    if (tail) {
        float* t = p.tail_ws + (int64_t)(blockIdx.x - p.full_tiles) * BM * BN;
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int lm = wm * WTM + j * 16 + mrow;
                const int ln = b_tile_row_of<BN, WN, GATED, 16>(i, wn) + ncol;
                *reinterpret_cast<float4*>(t + lm * BN + ln) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        return;
    }
    // (the staged store's slot swizzle needs BN / 4 a power of two)
    if constexpr (EPI == EPI_STORE_F32 && (BN & (BN - 1)) == 0) {
        if (p.vec_out) {
            staged_store_f32<BM, BN, WM, WN>(p, acc, lds, m0, n0, wm, wn, lane);
            return;
        }
    }
    // bf16 tile wholly inside the output (no bias): 8-byte stores without
    // per-element checks, one row address per token block and the column
    // offsets as immediates
    if constexpr (EPI == EPI_STORE_BF16 || EPI == EPI_GATED_BF16) {
        constexpr int COLS = GATED ? BN / 2 : BN;
        if (p.vec_out && !(EPI == EPI_STORE_BF16 && p.bias) && m0 + BM <= p.M && n0 + COLS <= p.N) {
            uint16_t* const C = static_cast<uint16_t*>(p.C);
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                uint16_t* row = C + (m0 + wm * WTM + j * 16 + mrow) * p.N + n0 + ncol;
#pragma unroll
                for (int i = 0; i < (GATED ? TN / 2 : TN); ++i) {
                    float v[4];
                    int col;
                    if (GATED) {
                        col = wn * (WTN / 2) + i * 16;
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = silu_mul(acc[i][j][q], acc[i + TN / 2][j][q]);
                    } else {
                        col = b_tile_row_of<BN, WN, false, 16>(i, wn);
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q];
                    }
                    *reinterpret_cast<uint2*>(row + col) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const int64_t gm = m0 + wm * WTM + j * 16 + mrow;
        if (gm >= p.M) continue;
        if (GATED) {
#pragma unroll
            for (int i = 0; i < TN / 2; ++i) {
                const int64_t gn = n0 + wn * (WTN / 2) + i * 16 + ncol;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = silu_mul(acc[i][j][q], acc[i + TN / 2][j][q]);
                store4<EPI>(p, gm, gn, v);
            }
        } else {
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int64_t gn = n0 + b_tile_row_of<BN, WN, GATED, 16>(i, wn) + ncol;
                float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                store4<EPI>(p, gm, gn, v);
            }
        }
    }
}

// Deep-pipelined direct-to-LDS kernel with 16x16x32 MFMAs (16-byte-aligned
// operands, K a multiple of 8): the 256 x 256, 256 x 192, 128 x 192 and
// 64 x 128 tiles.  PAIR (every K range a multiple of 64; the only form the
// 192-wide tiles take) replaces the four single stages below by two stages
// of K = 64, so that each DMA request is a whole 128-byte line (see the PAIR
// branch); the rest of this comment describes single stages.
//   * MFMA shape: v_mfma_f32_16x16x32_bf16 moves half the accumulator data
//     per flop of the 32x32x16 form; on this power-limited part that buys
//     clock (measured ~15% more MFMA throughput on random operands).  Lane
//     l holds operand row l & 15, K chunk l >> 4 (8 values), and result
//     rows 4 (l >> 4) .. +3 (weight rows = output columns) of column l & 15
//     (a token).
//   * LDS ring of 4 stages of K = 32 (tile rows of 64 bytes, no padding):
//     the stage of K step s+3 is filled by DMA while step s is multiplied;
//     a step's data is certified (own DMA waited, then a barrier) two
//     steps before it is multiplied.
//   * each K step is 32 MFMAs per wave; the fragments of step s+1 are read
//     into the other of two register slots under them.
//   * the barrier is a bare s_barrier after a vmcnt wait: it does not wait
//     for the fragment reads in flight.
// Bank spreading: a ds_read_b128 serves 16 lanes (16 rows of one chunk
// column) per LDS cycle across 64 banks = 16 groups of 16 bytes; a 64-byte
// row covers 4 groups, so the 16-byte chunk c of tile row r sits at position
// c ^ ((r >> 2) & 3) of its row and 16 consecutive rows hit 16 distinct
// groups.  The DMA applies the permutation on the global side (lane l of an
// instruction fills slot l and fetches the chunk that belongs there).
template <int BM, int BN, int WM, int WN, int EPI, bool KTAIL, bool PAIR>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_pipe_kernel(GemmArgs p) {
    constexpr int BK = 32;
    constexpr int NST = 4;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;          // 16-row MFMA blocks per wave
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    constexpr int ROWB = BK * 2;                         // 64 bytes per tile row
    constexpr int A_BYTES = BM * ROWB;
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int N_INSTR = STAGE / 1024;                // one wave instruction fills 1 KiB
    constexpr int A_INSTR = A_BYTES / 1024;
    static_assert(PAIR || N_INSTR % NW == 0, "each wave issues the same number of DMA instructions");
    constexpr int PW = N_INSTR / NW;
    static_assert(!GATED || TN % 2 == 0, "gated tiles pair gate and up MFMA blocks");
    constexpr uint32_t SENT = 0x80000000u;
    // 128 x 192 tiles keep one workgroup per CU (their tile count is sized
    // to the CU count): the ring is padded past half of the CU's 160 KiB
    constexpr int LDS_BYTES = (BM == 128 && BN == 192) ? 96 * 1024 : NST * STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wid / WN, wn = wid % WN;

    const Unit u = unit_of(p);
    const int64_t m0 = (int64_t)u.tile_m * BM;
    const int64_t n0 = GATED ? (int64_t)u.tile_n * (BN / 2) : (int64_t)u.tile_n * BN;
    const int64_t k_begin = u.k_begin, k_end = u.k_end;

    f32x4 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    if constexpr (PAIR) {
        // Paired stages: two LDS buffers of K = 64 (tile rows of 128 bytes),
        // each multiplied as two K steps of 32 (h = 0, 1).  A DMA instruction
        // then fetches 8 rows x 128 contiguous bytes: whole 128-byte lines,
        // half the L1 -> L2 requests of the 64-byte rows of single stages.
        //   * the chunk layout and the DMA are those of PairDma;
        //   * pair q + 1 is DMA'd into the other buffer from the middle of
        //     step 2q - 1 (once every wave holds pair q - 1's last
        //     fragments) and certified in the middle of step 2q + 1, two K
        //     steps later; one barrier per pair;
        //   * fragments of step s + 1 are read under the MFMAs of step s.
        using Dma = PairDma<BM, BN, NW, GATED>;
        constexpr int ROW2 = Dma::ROW2;                      // 128 bytes
        constexpr int STAGE2 = Dma::STAGE2;
        static_assert(2 * STAGE2 <= NST * STAGE, "two pair buffers fit the ring");
        constexpr int PW2 = Dma::PW2;
        const Dma dma(p, m0, n0, wid, lane);
        auto issue_pair = [&](int64_t k0, int buf) { dma.issue(k0, lds + buf * STAGE2); };
        // fragment reads: lane l reads row l & 15 of a 16-row block, chunk
        // 4 h + (l >> 4), at its swizzled position
        const int lrow = lane & 15;
        const int lo0 = lrow * ROW2 + ((((lane >> 4)) ^ (lrow >> 1)) * 16);
        const int lo1 = lrow * ROW2 + (((4 + (lane >> 4)) ^ (lrow >> 1)) * 16);
        bf16x8 wf[2][TN], xf[2][TM];
        auto read_one = [&](int buf, int lo, auto slot_c, int r) {
            constexpr int SL = decltype(slot_c)::value;
            const uint8_t* b = lds + buf * STAGE2 + lo;
            if (r < TN)
                wf[SL][r] = *reinterpret_cast<const bf16x8*>(b + (BM + b_tile_row_of<BN, WN, GATED, 16>(r, wn)) * ROW2);
            else
                xf[SL][r - TN] = *reinterpret_cast<const bf16x8*>(b + (wm * WTM + (r - TN) * 16) * ROW2);
        };
        auto mfma_block = [&](auto slot_c, int i) {
            constexpr int SL = decltype(slot_c)::value;
#pragma unroll
            for (int j = 0; j < TM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[SL][i], xf[SL][j], acc[i][j], 0, 0, 0);
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        constexpr int NR = TN + TM;
        constexpr int MF = TN * TM;
        const int np = (int)((k_end - k_begin) / 64);
        if (np > 0) {
            issue_pair(k_begin, 0);
            if (np > 1) issue_pair(k_begin + 64, 1);
            if (np > 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(PW2));
            else
                __builtin_amdgcn_s_waitcnt(0x0f70);
            bare_barrier();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < NR; ++r) read_one(0, lo0, S0{}, r);
            // pair q, buffer q & 1.  Step 2q (h = 0): read step 2q + 1's
            // fragments (same buffer, h = 1) under its MFMAs.  Step 2q + 1
            // (h = 1): half its MFMAs; certify pair q + 1 (DMA landed, every
            // wave's reads done); refill buffer q & 1 with pair q + 2; read
            // step 2q + 2's fragments (pair q + 1, h = 0) under the other half.
            auto pair_steps = [&](int q, auto full_c) {
                constexpr bool FULL = decltype(full_c)::value;
                const int buf = q & 1;
                const bool next = FULL || q + 1 < np;
                const bool dma = FULL || q + 2 < np;
#pragma unroll
                for (int r = 0; r < NR; ++r) read_one(buf, lo1, S1{}, r);
#pragma unroll
                for (int i = 0; i < TN; ++i) mfma_block(S0{}, i);
#pragma unroll
                for (int qq = 0; qq < MF; ++qq) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if ((qq % (MF / 4)) < NR / 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TN / 2; ++i) mfma_block(S1{}, i);
                __builtin_amdgcn_sched_barrier(0);
                if (next) {
                    __builtin_amdgcn_s_waitcnt(0x0070);          // vmcnt(0) lgkmcnt(0)
                    bare_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                    if (dma) issue_pair(k_begin + (int64_t)(q + 2) * 64, buf);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < NR; ++r) read_one(buf ^ 1, lo0, S0{}, r);
                }
#pragma unroll
                for (int i = TN / 2; i < TN; ++i) mfma_block(S1{}, i);
                if (FULL) {
#pragma unroll
                    for (int qq = 0; qq < MF / 2; ++qq) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (qq < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            int q = 0;
            for (; q + 2 < np; ++q) pair_steps(q, std::true_type{});
            for (; q < np; ++q) pair_steps(q, std::false_type{});
        }
    } else {
        // DMA: instruction j of a stage fills slots 64 j .. 64 j + 63, i.e. tile
        // rows 16 j + (lane >> 2), position lane & 3, which holds chunk cl
        const int cl = (lane & 3) ^ ((lane >> 4) & 3);
        uint32_t off[PW];
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            const int j = wid * PW + q;
            const int r = j * 16 + (lane >> 2);
            off[q] = SENT;
            if (j < A_INSTR) {
                if (m0 + r < p.M) off[q] = (uint32_t)(((int64_t)r * p.K + cl * 8) * 2);
            } else {
                const int lr = r - BM;
                int64_t gb;
                bool ok;
                if (GATED) {
                    const int half = BN / 2;
                    const int64_t c = n0 + (lr < half ? lr : lr - half);
                    ok = c < p.N;
                    gb = lr < half ? c : p.N + c;
                } else {
                    gb = n0 + lr;
                    ok = gb < p.Nb;
                }
                if (ok) off[q] = (uint32_t)(((gb - n0) * p.K + cl * 8) * 2);
            }
        }
        const uint16_t* a_tile = p.A + m0 * p.K;
        const uint16_t* b_tile = p.B + n0 * p.K;
        auto issue_stage = [&](int64_t k0, int st) {
            __amdgpu_buffer_rsrc_t rsa =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a_tile + k0), (short)0, 0x7fffffff, 0x00020000);
            __amdgpu_buffer_rsrc_t rsb =
                __builtin_amdgcn_make_buffer_rsrc((void*)(b_tile + k0), (short)0, 0x7fffffff, 0x00020000);
            const bool tail = KTAIL && k0 + BK > k_end;
#pragma unroll
            for (int q = 0; q < PW; ++q) {
                const int j = wid * PW + q;
                uint32_t o = off[q];
                if (KTAIL && tail && k0 + cl * 8 >= k_end) o = SENT;
                auto* dst = (__attribute__((address_space(3))) void*)(lds + st * STAGE + j * 1024);
                if (j < A_INSTR)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 16, o, 0, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, o, 0, 0, 0);
            }
        };

        // fragment reads: lane l reads row l & 15 of a 16-row block, chunk
        // l >> 4, at its swizzled position
        const int lo = (lane & 15) * ROWB + (((lane >> 4) ^ (((lane & 15) >> 2) & 3)) * 16);
        const int xbase = wm * WTM * ROWB + lo;
        const int wbase = A_BYTES + lo;

        bf16x8 wf[2][TN], xf[2][TM];
        auto read_frags = [&](int st, auto slot_c) {
            constexpr int SL = decltype(slot_c)::value;
            const uint8_t* b = lds + st * STAGE;
#pragma unroll
            for (int i = 0; i < TN; ++i)
                wf[SL][i] = *reinterpret_cast<const bf16x8*>(b + wbase + b_tile_row_of<BN, WN, GATED, 16>(i, wn) * ROWB);
#pragma unroll
            for (int j = 0; j < TM; ++j)
                xf[SL][j] = *reinterpret_cast<const bf16x8*>(b + xbase + j * 16 * ROWB);
        };

        constexpr int MF = TN * TM;
        constexpr int NR = TN + TM;
        auto mfma_slot = [&](auto slot_c) {
            constexpr int SL = decltype(slot_c)::value;
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[SL][i], xf[SL][j], acc[i][j], 0, 0, 0);
        };

        const int nk = (int)ceil_div(k_end - k_begin, BK);
        auto kof = [&](int s) { return k_begin + (int64_t)s * BK; };
        auto vm_wait = [&](bool one_stage_in_flight) {
            // this wave's DMA of older stages has landed; the newest (PW
            // instructions) may still be in flight
            if (one_stage_in_flight)
                __builtin_amdgcn_s_waitcnt(0x0f70 | (PW & 15) | ((PW >> 4) << 14));
            else
                __builtin_amdgcn_s_waitcnt(0x0f70);
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;

        if (nk > 0) {
            for (int s = 0; s < 3; ++s)
                if (s < nk) issue_stage(kof(s), s);
            vm_wait(nk > 2);
            bare_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_frags(0, S0{});
            // K step s multiplies slot s mod 2 and reads step s + 1 into the
            // other slot.  It first refills the stage of step s - 1 with step
            // s + 3, and ends by certifying step s + 2.  FULL: all of this is
            // known to apply (steady state, no branches between the MFMAs and
            // the reads they hide); otherwise each part is checked.
            auto step = [&](int s, auto sa, auto sb, auto full_c) {
                constexpr bool FULL = decltype(full_c)::value;
                const bool dma = FULL || s + 3 < nk;
                const bool more = FULL || s + 1 < nk;
                const bool bar = FULL || s + 2 < nk;
                if (dma) issue_stage(kof(s + 3), (s + 3) & 3);
                __builtin_amdgcn_sched_barrier(0);
                if (more) read_frags((s + 1) & 3, sb);
                mfma_slot(sa);
#pragma unroll
                for (int q = 0; q < MF; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (FULL && (q % (MF / 4)) < NR / 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (bar) {
                    vm_wait(dma);
                    bare_barrier();
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            using T_ = std::true_type;
            using F_ = std::false_type;
            int s = 0;
            for (; s + 4 < nk; s += 2) {
                step(s, S0{}, S1{}, T_{});
                step(s + 1, S1{}, S0{}, T_{});
            }
            // at most 4 steps remain (s is even here): unrolled, so that the
            // register slots stay compile-time
            if (s < nk) step(s, S0{}, S1{}, F_{});
            if (s + 1 < nk) step(s + 1, S1{}, S0{}, F_{});
            if (s + 2 < nk) step(s + 2, S0{}, S1{}, F_{});
            if (s + 3 < nk) step(s + 3, S1{}, S0{}, F_{});
        }

    }  // single stages

    pipe_epilogue<BM, BN, WM, WN, EPI>(p, u.tail, acc, lds, m0, n0, wm, wn, lane);
}

// Adds the split-K partial sums in split order and applies the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const float* __restrict__ ws, int splits,
                                                              int64_t M, int64_t N, int64_t Nb,
                                                              const uint16_t* __restrict__ bias,
                                                              void* __restrict__ out) {
    const int64_t total = M * N;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = idx / N, col = idx - row * N;
        if (EPI == EPI_GATED_BF16) {
            float g = ws[row * Nb + col], u = ws[row * Nb + N + col];
            for (int s = 1; s < splits; ++s) {
                g = g + ws[(int64_t)s * M * Nb + row * Nb + col];
                u = u + ws[(int64_t)s * M * Nb + row * Nb + N + col];
            }
            static_cast<uint16_t*>(out)[idx] = f32_to_bf16(silu_mul(g, u));
        } else {
            float v = ws[row * Nb + col];
            for (int s = 1; s < splits; ++s) v = v + ws[(int64_t)s * M * Nb + row * Nb + col];
            if (bias) v = v + bf16_to_f32(bias[col]);
            if (EPI == EPI_STORE_F32)
                static_cast<float*>(out)[idx] = v;
            else
                static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
        }
    }
}

// ---- weight-streaming decode GEMM (M <= 64) --------------------------------
//
// Decode multiplies a few token rows by a large weight matrix: HBM-bound on
// the weights, which must stream in long contiguous runs (a 64-byte piece per
// row, as a 32-wide K stage reads, runs at about two thirds of the bandwidth
// that 256-byte and longer runs reach) with many bytes in flight.  Design:
//   * persistent grid, one workgroup per CU; the work is a list of units
//     (output tile of 128 weight rows, K chunk of 128), tile-major, cut into
//     gridDim.x equal contiguous ranges, so every CU streams the same number
//     of weight bytes and its DMA never stops between tiles;
//   * LDS holds weights only: a unit stage is 128 weight rows x 256
//     contiguous bytes, fetched 4 rows x 256 B per wave instruction straight
//     into LDS; a ring of 4 stages keeps three units (96 KiB) in flight;
//   * 4 waves, each 16 tokens x all 128 weight rows (16x16x32 MFMAs); a wave
//     loads its tokens' fragments from global memory (the token rows are
//     small and stay in L2) into registers two units ahead;
//   * when a workgroup leaves a tile it writes its fp32 partial tile; a
//     finalize pass adds a tile's partials in K order (deterministic) and
//     applies the epilogue.
// LDS rows are 256 bytes (16 chunks); chunk c of row r sits at position
// c ^ (r & 15), so the 16 rows of a fragment read hit 16 distinct bank groups.
constexpr int STR_BM = 64, STR_BN = 128, STR_BK = 128, STR_NST = 4;
constexpr int STR_ROWB = STR_BK * 2;
constexpr int STR_STAGE = STR_BN * STR_ROWB;                    // 32 KiB of weight rows
constexpr int STR_LDS = STR_NST * STR_STAGE;                    // 128 KiB
constexpr int STR_NW = 4;
constexpr int STR_PW = STR_STAGE / 1024 / STR_NW;               // DMA instructions per wave and unit
constexpr int STR_TL = STR_BK / 32;                             // token loads per lane and unit (one per sub-step)

__host__ __device__ __forceinline__ int64_t str_unit_begin(int w, int64_t units, int P) {
    return ((int64_t)w * units) / P;
}

// One streamed product: C-partials of A[M, K] . B[Nb, K]^T, tiles of 128 B
// rows (gated: 64 gate rows and the same 64 up rows), units of 128 K.
struct StreamOp {
    const uint16_t* A;
    const uint16_t* B;
    int64_t M, N, K, Nb;
    int64_t units;
    int kc, maxseg;
    float* part;            // [P][maxseg][BM][BN] fp32 partial tiles
};

__host__ __device__ __forceinline__ StreamOp make_stream_op(const uint16_t* A, const uint16_t* B, int64_t M,
                                                            int64_t N, int64_t K, bool gated, float* part,
                                                            int P) {
    StreamOp o;
    o.A = A;
    o.B = B;
    o.M = M;
    o.N = N;
    o.K = K;
    o.Nb = gated ? 2 * N : N;
    const int64_t cols = gated ? STR_BN / 2 : STR_BN;
    const int64_t tiles = (N + cols - 1) / cols;
    o.kc = (int)((K + STR_BK - 1) / STR_BK);
    o.units = tiles * o.kc;
    const int64_t per_wg = (o.units + P - 1) / P;
    o.maxseg = (int)((per_wg + o.kc - 1) / o.kc + 1);
    o.part = part;
    return o;
}

// (tile, K chunk) of a unit, advanced one unit at a time (no divisions in
// the loop)
struct UnitPos {
    int t, kc;
    __device__ __forceinline__ void next(int kcs) {
        if (++kc == kcs) {
            kc = 0;
            ++t;
        }
    }
};

// Runs workgroup w's range of units of o.
template <bool GATED, bool KTAIL>
__device__ __forceinline__ void stream_units(const StreamOp& o, uint8_t* lds, int w, int P) {
    constexpr int BM = STR_BM, BN = STR_BN, ROWB = STR_ROWB, NST = STR_NST, PW = STR_PW;
    constexpr int TB = BN / 16;                              // 16-row weight blocks (8)
    constexpr int cols = GATED ? BN / 2 : BN;
    constexpr uint32_t SENT = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t u0 = str_unit_begin(w, o.units, P), u1 = str_unit_begin(w + 1, o.units, P);
    const int n = (int)(u1 - u0);
    if (n <= 0) return;

    // weight DMA, per lane and instruction: instruction q fills tile rows
    // 4 j + (lane >> 4), j = wid PW + q, position lane & 15, i.e. chunk
    // (lane & 15) ^ (row & 15); byte offset relative to the tile's first row
    // and the unit's K start (both in the uniform buffer base)
    uint32_t boff[PW];
    int bcol[PW], kch[PW];
#pragma unroll
    for (int q = 0; q < PW; ++q) {
        const int r = (wid * PW + q) * 4 + (lane >> 4);
        kch[q] = ((lane & 15) ^ (r & 15)) * 8;
        int64_t g;
        if (GATED) {
            g = r < BN / 2 ? r : o.N + (r - BN / 2);
            bcol[q] = r < BN / 2 ? r : r - BN / 2;
        } else {
            g = r;
            bcol[q] = r;
        }
        boff[q] = (uint32_t)((g * o.K + kch[q]) * 2);
    }
    auto issue_w = [&](const UnitPos& up, int st) {
        const int64_t k0 = (int64_t)up.kc * STR_BK;
        const int64_t n0 = (int64_t)up.t * cols;
        const int ncols = (int)((o.N - n0) < cols ? (o.N - n0) : cols);
        const int kleft = (int)((o.K - k0) < STR_BK ? (o.K - k0) : STR_BK);
        __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)(o.B + n0 * o.K + k0), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            bool ok = bcol[q] < ncols;
            if (KTAIL) ok = ok && kch[q] < kleft;
            auto* dst = (__attribute__((address_space(3))) void*)(lds + st * STR_STAGE + (wid * PW + q) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, dst, 16, ok ? boff[q] : SENT, 0, 0, 0);
        }
    };
    // token fragments: lane l holds token 16 wid + (l & 15), K chunk
    // 4 kk + (l >> 4) of sub-step kk
    const int tok = wid * 16 + (lane & 15);
    uint32_t toff[STR_TL];
#pragma unroll
    for (int kk = 0; kk < STR_TL; ++kk)
        toff[kk] = tok < o.M ? (uint32_t)(((int64_t)tok * o.K + (4 * kk + (lane >> 4)) * 8) * 2) : SENT;
    bf16x8 tf[3][STR_TL];
    auto load_t = [&](const UnitPos& up, auto slot_c) {
        constexpr int SL = decltype(slot_c)::value;
        const int64_t k0 = (int64_t)up.kc * STR_BK;
        const int kleft = (int)((o.K - k0) < STR_BK ? (o.K - k0) : STR_BK);
        __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(o.A + k0), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int kk = 0; kk < STR_TL; ++kk) {
            uint32_t off = toff[kk];
            if (KTAIL && (4 * kk + (lane >> 4)) * 8 >= kleft) off = SENT;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsa, off, 0, 0);
            tf[SL][kk] = __builtin_bit_cast(bf16x8, v);
        }
    };

    int lo[STR_TL];
#pragma unroll
    for (int kk = 0; kk < STR_TL; ++kk) lo[kk] = (lane & 15) * ROWB + ((((4 * kk + (lane >> 4)) ^ (lane & 15))) * 16);

    f32x4 acc[TB];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < TB; ++i) acc[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    };
    zero_acc();

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    constexpr int AHEAD = NST - 1;                   // weight units in flight beyond the one multiplied
    // issue order, as if steps -3..-1 had run: each step issues the tokens
    // of unit +2, then the weights of unit +3
    UnitPos pw, pt, pc;                              // next weight issue, next token load, current unit
    pc.t = (int)(u0 / o.kc);
    pc.kc = (int)(u0 - (int64_t)pc.t * o.kc);
    pw = pc;
    pt = pc;
    issue_w(pw, 0);
    pw.next(o.kc);
    load_t(pt, S0{});
    pt.next(o.kc);
    if (n > 1) {
        issue_w(pw, 1);
        pw.next(o.kc);
        load_t(pt, S1{});
        pt.next(o.kc);
    }
    if (n > 2) {
        issue_w(pw, 2);
        pw.next(o.kc);
    }

    int seg = 0;
    bool full_wait = false;
    // unit i: its weights (DMA, slot i mod 4) and tokens (registers, slot
    // i mod 3) have landed; it first issues the weights of unit i+3 and the
    // tokens of unit i+2
    auto step = [&](int i, auto slot_c, auto next2_c) {
        // vector-memory operations issued after this unit's tokens (which
        // follow its weights) may stay in flight: unit i+1's weights (issued
        // with this unit's tokens), unit i+1's tokens and unit i+2's weights
        constexpr int N2 = PW + STR_TL + PW, N1 = PW + STR_TL;
        if (full_wait || i + 1 >= n) __builtin_amdgcn_s_waitcnt(0x0f70);
        else if (i + 2 < n) __builtin_amdgcn_s_waitcnt(0x0f70 | (N2 & 15) | ((N2 >> 4) << 14));
        else __builtin_amdgcn_s_waitcnt(0x0f70 | (N1 & 15) | ((N1 >> 4) << 14));
        full_wait = false;
        bare_barrier();
        if (i + 2 < n) {
            load_t(pt, next2_c);
            pt.next(o.kc);
        }
        if (i + AHEAD < n) {
            issue_w(pw, (i + AHEAD) % NST);
            pw.next(o.kc);
        }
        constexpr int SL = decltype(slot_c)::value;
        const uint8_t* b = lds + (i % NST) * STR_STAGE;
        bf16x8 wf[STR_TL][TB];
#pragma unroll
        for (int kk = 0; kk < STR_TL; ++kk)
#pragma unroll
            for (int ib = 0; ib < TB; ++ib) wf[kk][ib] = *reinterpret_cast<const bf16x8*>(b + lo[kk] + ib * 16 * ROWB);
#pragma unroll
        for (int kk = 0; kk < STR_TL; ++kk)
#pragma unroll
            for (int ib = 0; ib < TB; ++ib)
                acc[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[kk][ib], tf[SL][kk], acc[ib], 0, 0, 0);
        const bool last_of_tile = pc.kc + 1 == o.kc;
        pc.next(o.kc);
        if (i + 1 == n || last_of_tile) {
            // leaving tile t: fp32 partial tile [BM tokens][BN B rows]
            float* out = o.part + ((int64_t)w * o.maxseg + seg) * BM * BN;
#pragma unroll
            for (int ib = 0; ib < TB; ++ib) {
                const int ln = ib * 16 + 4 * (lane >> 4);
                *reinterpret_cast<float4*>(out + tok * BN + ln) =
                    make_float4(acc[ib][0], acc[ib][1], acc[ib][2], acc[ib][3]);
            }
            zero_acc();
            ++seg;
            full_wait = true;                   // stores in flight: the next wait counts them too
        }
    };
    int i = 0;
    for (; i + 3 <= n; i += 3) {
        step(i, S0{}, S2{});
        step(i + 1, S1{}, S0{});
        step(i + 2, S2{}, S1{});
    }
    if (i < n) step(i, S0{}, S2{});
    if (i + 1 < n) step(i + 1, S1{}, S0{});
}

// Adds tile t's partials (from the workgroups whose unit ranges cover it, in
// workgroup = K order) for token rows m and 4 consecutive columns from g4,
// and stores them through the epilogue of `out`.
template <int EPI>
__device__ __forceinline__ void stream_finish4(const StreamOp& o, const GemmArgs& out, int P, int64_t t, int w0,
                                               int m, int g4) {
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    constexpr int BM = STR_BM, BN = STR_BN;
    constexpr int cols = GATED ? BN / 2 : BN;
    const int64_t first = t * o.kc, last = first + o.kc - 1;
    float v0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, v1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    bool any = false;
    for (int w = w0; w < P; ++w) {
        const int64_t b = str_unit_begin(w, o.units, P), e = str_unit_begin(w + 1, o.units, P);
        if (b > last) break;
        if (e <= first || e <= b) continue;        // before the tile, or an empty range
        const int seg = (int)(t - b / o.kc);
        const float* part = o.part + ((int64_t)w * o.maxseg + seg) * BM * BN + (int64_t)m * BN;
        const float4 a = *reinterpret_cast<const float4*>(part + g4);
        float4 c = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (GATED) c = *reinterpret_cast<const float4*>(part + BN / 2 + g4);
        if (!any) {
            v0[0] = a.x; v0[1] = a.y; v0[2] = a.z; v0[3] = a.w;
            v1[0] = c.x; v1[1] = c.y; v1[2] = c.z; v1[3] = c.w;
            any = true;
        } else {
            v0[0] = v0[0] + a.x; v0[1] = v0[1] + a.y; v0[2] = v0[2] + a.z; v0[3] = v0[3] + a.w;
            v1[0] = v1[0] + c.x; v1[1] = v1[1] + c.y; v1[2] = v1[2] + c.z; v1[3] = v1[3] + c.w;
        }
    }
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = GATED ? silu_mul(v0[q], v1[q]) : v0[q];
    store4<EPI>(out, m, t * cols + g4, v);
}

// first workgroup whose unit range meets tile t
__device__ __forceinline__ int stream_first_wg(const StreamOp& o, int P, int64_t t) {
    const int64_t first = t * o.kc;
    int w0 = (int)((first * P) / o.units);
    while (w0 + 1 < P && str_unit_begin(w0 + 1, o.units, P) <= first) ++w0;
    while (w0 > 0 && str_unit_begin(w0, o.units, P) > first) --w0;
    return w0;
}

template <bool GATED, bool KTAIL>
__global__ __launch_bounds__(256) void gemm_bf16_stream_kernel(StreamOp o) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[STR_LDS];
    stream_units<GATED, KTAIL>(o, lds, blockIdx.x, gridDim.x);
}

// Block (t, y) finishes tile t; each thread 4 consecutive columns of one
// token row.
template <int EPI>
__global__ __launch_bounds__(256) void stream_finalize_kernel(StreamOp o, GemmArgs out, int P) {
    constexpr int cols = EPI == EPI_GATED_BF16 ? STR_BN / 2 : STR_BN;
    const int64_t t = blockIdx.x;
    const int idx = blockIdx.y * blockDim.x + threadIdx.x;
    const int m = idx / (cols / 4), g4 = (idx % (cols / 4)) * 4;
    if (m >= o.M) return;
    stream_finish4<EPI>(o, out, P, t, stream_first_wg(o, P, t), m, g4);
}

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}

// ---- register-streaming decode GEMM (M <= 64) -----------------------------
//
// The decode product reads a large weight matrix once for at most 64 token
// rows, so its time is the weight stream from HBM.  This kernel keeps LDS
// out of that stream:
//   * one workgroup of 4 waves per CU (one per SIMD).  Workgroup (q, g) owns
//     K slice q (4 R elements, R = 256 for K a multiple of 1024) and the
//     16-row weight blocks g, g + G, ..., so at any time the G workgroups of
//     a slice read G adjacent blocks; wave w owns the R-element K range w of
//     the slice.  Four waves per CU stream faster than eight: a probe reading
//     a 235 MB matrix in this pattern took 41 us with 4 waves of 256 K and
//     46.5 us with 8 (same box);
//   * a wave loads the fragments of all 64 tokens over its K range once and
//     keeps them in registers (R/2 VGPRs);
//   * weights go straight from HBM into MFMA A-fragments: for K step i of a
//     block, lane l reads the 16 bytes of block row l & 15 at K chunk
//     4 i + (l >> 4), so one instruction reads 16 rows x 64 contiguous bytes
//     and the R/32 instructions of a block walk along each row (the 4 waves
//     together read 8 R contiguous bytes of every row);
//   * two register slots of R/32 fragments: two blocks of loads per wave
//     are in flight (16 KiB at R = 256);
//   * after each block the waves' fp32 partials [64 tokens][16 rows] meet in
//     LDS, are added in wave (= K) order and stored as the workgroup's
//     partial tile; a finalize pass adds the S slices' tiles in slice order
//     and applies the epilogue.  No atomics: the result is deterministic.
constexpr int RS_WAVES = 4;
constexpr int RS_SLICE = 1024;      // K per workgroup: RS_WAVES waves of 256
constexpr int RS_HOLD = 28;         // partial tiles a workgroup keeps in LDS (112 KiB)

struct RsOp {
    const uint16_t* A;      // tokens [M, K]
    const uint16_t* B;      // weights [Nb, K]
    float* part;            // [S][rbn][64 tokens][16 rows] fp32 partial tiles
    int64_t M, K, Nb;
    int S, G, R, rbn;       // K slices, workgroups per slice, K per wave, 16-row blocks
};

// S = ceil(K / RS_SLICE) slices, R = K per wave rounded up to the 32 of a K step
// (at most 256: the tokens' fragments take R/2 VGPRs), up to 256 / S
// workgroups per slice.
__host__ __device__ inline RsOp make_rs_op(const uint16_t* A, const uint16_t* B, float* part, int64_t M,
                                           int64_t K, int64_t Nb) {
    RsOp o;
    o.A = A;
    o.B = B;
    o.part = part;
    o.M = M;
    o.K = K;
    o.Nb = Nb;
    o.S = (int)((K + RS_SLICE - 1) / RS_SLICE);
    const int64_t per_slice = (K + o.S - 1) / o.S;
    o.R = (int)(((per_slice + RS_WAVES - 1) / RS_WAVES + 31) / 32 * 32);
    o.rbn = (int)((Nb + 15) / 16);
    o.G = 256 / o.S < o.rbn ? 256 / o.S : o.rbn;
    return o;
}

template <int NKS, bool EDGE>
__global__ __launch_bounds__(RS_WAVES * 64) void gemm_bf16_rs_kernel(RsOp o) {
    __shared__ __attribute__((aligned(16))) float red[2][RS_WAVES][1024];
    // the workgroup's partial tiles, written to memory in one burst after
    // the weight stream when they fit (stores interleaved with the stream
    // slowed it: a 235 MB probe in this pattern took 52.0 us with per-block
    // stores and 49.4 us with the burst, same box)
    __shared__ __attribute__((aligned(16))) float hold[RS_HOLD][1024];
    constexpr uint32_t SENT = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = blockIdx.x / o.G, g = blockIdx.x - q * o.G;
    const int nb = (o.rbn - g + o.G - 1) / o.G;                  // blocks g + j G, j < nb
    const int64_t kw = ((int64_t)q * RS_WAVES + wid) * o.R;      // the wave's first K
    const int r16 = lane & 15, ch = lane >> 4;

    // tokens: fragment (i, tb) of lane l is token 16 tb + (l & 15), K chunk
    // kw + 32 i + 8 (l >> 4); absent tokens and K past the end read as zero
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)o.A, (short)0, 0x7fffffff, 0x00020000);
    bf16x8 tk[NKS][4];
#pragma unroll
    for (int i = 0; i < NKS; ++i)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int64_t m = tb * 16 + r16, k = kw + i * 32 + ch * 8;
            const uint32_t off = (m < o.M && k < o.K) ? (uint32_t)((m * o.K + k) * 2) : SENT;
            tk[i][tb] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsa, off, 0, 0));
        }

    // weights: K steps of this lane that lie inside K (all of them unless EDGE)
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)o.B, (short)0, 0x7fffffff, 0x00020000);
    uint32_t kok = 0;
#pragma unroll
    for (int i = 0; i < NKS; ++i)
        if (kw + i * 32 + ch * 8 < o.K) kok |= 1u << i;
    const uint32_t lane_off = (uint32_t)(((int64_t)r16 * o.K + kw + ch * 8) * 2);
    const uint32_t blk_bytes = (uint32_t)(16 * o.K * 2);

    bf16x8 wt[2][NKS];
    // block j of the workgroup (weight block g + j G): byte offset for this
    // lane, or the sentinel past the range
    auto block_off = [&](int j) -> uint32_t {
        const int b = g + j * o.G;
        bool ok = j < nb;
        if (EDGE) ok = ok && (int64_t)b * 16 + r16 < o.Nb;
        return ok ? (uint32_t)b * blk_bytes + lane_off : SENT;
    };
    // load K step i of the block at `base` into slot SL
    auto issue = [&](uint32_t base, auto slot_c, auto step_c) {
        constexpr int SL = decltype(slot_c)::value, I = decltype(step_c)::value;
        uint32_t off = base + (uint32_t)(I * 64);
        if (EDGE && (base == SENT || !((kok >> I) & 1u))) off = SENT;
        wt[SL][I] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsb, off, 0, 0));
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // prologue: blocks 0 and 1, in step order: the compiler's wait counts
    // merge this order with the loop's, and a different one would make
    // every fragment of a slot wait for the slot's last load
    {
        const uint32_t p0 = block_off(0), p1 = block_off(1);
        static_for(std::make_integer_sequence<int, NKS>{}, [&](auto i) {
            issue(p0, S0{}, i);
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for(std::make_integer_sequence<int, NKS>{}, [&](auto i) {
            issue(p1, S1{}, i);
            __builtin_amdgcn_sched_barrier(0);
        });
    }

    f32x4 acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    float* part = o.part + (int64_t)q * o.rbn * 1024;
    const bool hold_all = nb <= RS_HOLD;

    auto block = [&](int j, auto slot_c) {
        constexpr int SL = decltype(slot_c)::value;
        const uint32_t nxt = block_off(j + 2);
        static_for(std::make_integer_sequence<int, NKS>{}, [&](auto step_c) {
            constexpr int I = decltype(step_c)::value;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wt[SL][I], tk[I][tb], acc[tb], 0, 0, 0);
            // refill the fragment just multiplied (block j + 2): the loads in
            // flight stay spread evenly over the block
            issue(nxt, slot_c, step_c);
            __builtin_amdgcn_sched_barrier(0);
        });
        // lane l holds rows 4 (l >> 4) + 0..3 of token 16 tb + (l & 15)
        float* mine = &red[j & 1][wid][0];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            *reinterpret_cast<f32x4*>(mine + (tb * 16 + r16) * 16 + 4 * ch) = acc[tb];
            acc[tb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);                 // lgkmcnt(0): the LDS writes are done
        bare_barrier();
        const int e = threadIdx.x * 4;
        f32x4 v = *reinterpret_cast<const f32x4*>(&red[j & 1][0][e]);
#pragma unroll
        for (int w = 1; w < RS_WAVES; ++w) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(&red[j & 1][w][e]);
            v = v + t;
        }
        if (hold_all)
            *reinterpret_cast<f32x4*>(&hold[j][e]) = v;
        else
            *reinterpret_cast<f32x4*>(part + (int64_t)(g + j * o.G) * 1024 + e) = v;
        // the next block's accumulators start after this barrier: without the
        // opaque definition the compiler hoists their MFMAs above it (they
        // start from zero), which forces a wait for every load in flight
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) asm volatile("" : "+v"(acc[tb]));
    };
    int j = 0;
    for (; j + 1 < nb; j += 2) {
        block(j, S0{});
        block(j + 1, S1{});
    }
    if (j < nb) block(j, S0{});
    if (hold_all) {
        __syncthreads();
        const int e = threadIdx.x * 4;
        for (int jj = 0; jj < nb; ++jj)
            *reinterpret_cast<f32x4*>(part + (int64_t)(g + jj * o.G) * 1024 + e) =
                *reinterpret_cast<const f32x4*>(&hold[jj][e]);
    }
}

// Thread (token m, columns j .. j+3): adds the S slices' partials in slice
// order and stores through the epilogue of `out`.  A workgroup covers 16
// columns of all 64 tokens; a wave reads 16 tokens x 64 contiguous bytes.
template <int EPI>
__global__ __launch_bounds__(256) void rs_finalize_kernel(RsOp o, GemmArgs out) {
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    const int t = threadIdx.x;
    const int64_t m = (t & 15) + 16 * (t >> 6);
    const int64_t j = (int64_t)blockIdx.x * 16 + ((t >> 4) & 3) * 4;
    if (m >= o.M || j >= out.N) return;
    auto at = [&](int q, int64_t row) -> int64_t {
        return (((int64_t)q * o.rbn + (row >> 4)) * 64 + m) * 16 + (row & 15);
    };
    float v0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, v1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((out.N & 3) == 0) {
        for (int q = 0; q < o.S; ++q) {
            const float4 a = *reinterpret_cast<const float4*>(o.part + at(q, j));
            v0[0] = v0[0] + a.x; v0[1] = v0[1] + a.y; v0[2] = v0[2] + a.z; v0[3] = v0[3] + a.w;
            if (GATED) {
                const float4 c = *reinterpret_cast<const float4*>(o.part + at(q, out.N + j));
                v1[0] = v1[0] + c.x; v1[1] = v1[1] + c.y; v1[2] = v1[2] + c.z; v1[3] = v1[3] + c.w;
            }
        }
    } else {
        for (int q = 0; q < o.S; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < out.N) {
                    v0[e] = v0[e] + o.part[at(q, j + e)];
                    if (GATED) v1[e] = v1[e] + o.part[at(q, out.N + j + e)];
                }
    }
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = GATED ? silu_mul(v0[e], v1[e]) : v0[e];
    store4<EPI>(out, m, j, v);
}

// Finishes the tiles of a balanced last round: adds each tile's K pieces in
// piece order and applies the epilogue (gated SiLU(g)*u, or store + bias).
// One thread per 4 consecutive output columns of a tile row (float4 reads).
template <int EPI>
__global__ __launch_bounds__(256) void tail_fixup_kernel(GemmArgs p, int BM, int BN) {
    constexpr bool GATED = EPI == EPI_GATED_BF16;
    const int ntail = p.tiles_m * p.tiles_n - p.full_tiles;
    const int cols = GATED ? BN / 2 : BN;
    const int q4 = cols / 4;
    const int64_t per_tile = (int64_t)BM * q4;
    const int64_t total = (int64_t)ntail * per_tile;
    const int64_t piece = (int64_t)BM * BN;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx / per_tile);
        const int64_t rem = idx - (int64_t)t * per_tile;
        const int lm = (int)(rem / q4), lc = (int)(rem % q4) * 4;
        int tm, tn;
        tile_of(p.full_tiles + t, p.tiles_m, p.tiles_n, tm, tn);
        const int64_t m = (int64_t)tm * BM + lm;
        const int64_t n = (int64_t)tn * cols + lc;
        if (m >= p.M || n >= p.N) continue;
        const float* base = p.tail_ws + (int64_t)t * p.tail_split * piece + (int64_t)lm * BN + lc;
        float4 g = *reinterpret_cast<const float4*>(base);
        float4 u = GATED ? *reinterpret_cast<const float4*>(base + BN / 2) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int s = 1; s < p.tail_split; ++s) {
            const float4 a = *reinterpret_cast<const float4*>(base + s * piece);
            g.x = g.x + a.x; g.y = g.y + a.y; g.z = g.z + a.z; g.w = g.w + a.w;
            if (GATED) {
                const float4 b = *reinterpret_cast<const float4*>(base + s * piece + BN / 2);
                u.x = u.x + b.x; u.y = u.y + b.y; u.z = u.z + b.z; u.w = u.w + b.w;
            }
        }
        float v[4];
        if (GATED) {
            v[0] = silu_mul(g.x, u.x); v[1] = silu_mul(g.y, u.y); v[2] = silu_mul(g.z, u.z); v[3] = silu_mul(g.w, u.w);
        } else {
            v[0] = g.x; v[1] = g.y; v[2] = g.z; v[3] = g.w;
        }
        store4<EPI>(p, m, n, v);
    }
}

// ---- planning -------------------------------------------------------------

enum Kern { K_F32 = 0, K_BF16_LARGE = 1, K_BF16_SMALL = 2, K_BF16_HUGE8 = 4, K_BF16_DEC4 = 6,
            K_BF16_STREAM = 7, K_BF16_RS = 8, K_BF16_MID = 9, K_BF16_W192 = 10 };

// Tile configurations (BM tokens x BN weight rows):
//   HUGE8 256x256, 2x4 waves of 128x64 (prefill-sized problems; deep-pipelined
//         16x16x32 kernel when the operands allow direct-to-LDS loads)
//   LARGE 128x128, 2x2 waves of 64x64
//   SMALL  64x128, 1x2 waves of 64x64 (decode, M <= 64)
//   DEC4   64x128, 1x4 waves of 64x32, deep-pipelined 16x16x32 kernel (decode,
//          M <= 64; same tiling as SMALL, which serves it when the operands
//          do not allow direct-to-LDS loads)
//   W192  256x192, 2x4 waves of 128x48, paired stages, K split in two
//          (few output columns with long K: the QKV projection at TP=16)
//   STREAM 64x128 weight-streaming persistent kernel (decode, M <= 64, large
//          weights): one workgroup per CU over equal ranges of (tile, K chunk)
struct TileCfg { int bm, bn, wm, wn; };
static TileCfg tile_cfg(int k) {
    switch (k) {
        case K_BF16_HUGE8: return TileCfg{256, 256, 2, 4};
        case K_BF16_SMALL: return TileCfg{64, 128, 1, 2};
        case K_BF16_DEC4: return TileCfg{64, 128, 1, 4};
        case K_BF16_MID: return TileCfg{128, 192, 2, 4};
        case K_BF16_W192: return TileCfg{256, 192, 2, 4};
        default: return TileCfg{128, 128, 2, 2};
    }
}

// Workgroups of the direct-to-LDS kernel resident on one CU: its LDS ring
// (2 buffers of BM + BN rows of 144 bytes) against the CU's 160 KiB.
static int64_t wgs_per_cu(int k) {
    TileCfg c = tile_cfg(k);
    const int64_t ring = (int64_t)2 * (c.bm + c.bn) * 144;
    const int64_t w = (int64_t)160 * 1024 / ring;
    return w < 1 ? 1 : w;
}

static void tiles_for(int kern, int64_t M, int64_t N, bool gated, int& tm, int& tn) {
    if (kern == K_F32) {
        tm = (int)ceil_div(M, 64);
        tn = (int)(gated ? ceil_div(N, 32) : ceil_div(N, 64));
        return;
    }
    TileCfg c = tile_cfg(kern);
    tm = (int)ceil_div(M, c.bm);
    tn = (int)(gated ? ceil_div(N, c.bn / 2) : ceil_div(N, c.bn));
}

// CUs of an MI355X: the weight-streaming kernel runs one workgroup on each
constexpr int kStreamWGs = 256;

// fp32 partial-tile workspace of the weight-streaming kernel
static size_t stream_ws_bytes(int64_t M, int64_t N, int64_t K, bool gated) {
    const StreamOp o = make_stream_op(nullptr, nullptr, M, N, K, gated, nullptr, kStreamWGs);
    return (size_t)kStreamWGs * o.maxseg * STR_BM * STR_BN * sizeof(float);
}
static int64_t stream_units_of(int64_t N, int64_t K, bool gated) {
    return make_stream_op(nullptr, nullptr, 1, N, K, gated, nullptr, kStreamWGs).units;
}

static size_t rs_ws_bytes(int64_t M, int64_t K, int64_t Nb) {
    const RsOp o = make_rs_op(nullptr, nullptr, nullptr, M, K, Nb);
    return (size_t)o.S * (size_t)o.rbn * 1024 * sizeof(float);
}

// Split-K target: about this many workgroups for shapes with fewer output
// tiles than CUs.
constexpr int64_t kSplitTarget = 1024;
// DEC4 (48 KiB of LDS ring, three workgroups per CU) aims at one full round
// of 768 workgroups without exceeding it.
constexpr int64_t kSplitTargetDec4 = 768;

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool gated, tp_dtype dt) {
    GemmPlan pl{};
    pl.splits = 1;
    pl.k_split = K;
    pl.ws_bytes = 0;
    pl.full_tiles = 0;
    pl.tail_split = 0;
    pl.tail_k = K;
    if (dt == TP_F32) {
        pl.kernel = K_F32;
        return pl;
    }
    int tm, tn;
    const int64_t Nb0 = gated ? 2 * N : N;
    // register-streaming kernel: enough 16-row blocks for two per workgroup
    if (M <= 64 && K % 8 == 0 && K >= 1024 && Nb0 * K * 2 < ((int64_t)1 << 31) && M * K * 2 < ((int64_t)1 << 31)) {
        const RsOp o = make_rs_op(nullptr, nullptr, nullptr, M, K, Nb0);
        if (o.rbn >= 2 * (256 / o.S)) {
            pl.kernel = K_BF16_RS;
            pl.ws_bytes = rs_ws_bytes(M, K, Nb0);
            return pl;
        }
    }
    if (M <= 64 && K % 8 == 0 && Nb0 * K * 2 < ((int64_t)1 << 31)) {
        if (stream_units_of(N, K, gated) >= 2 * kStreamWGs) {
            pl.kernel = K_BF16_STREAM;
            pl.ws_bytes = stream_ws_bytes(M, N, K, gated);
            return pl;
        }
    }
    if (M > 64) {
        tiles_for(K_BF16_HUGE8, M, N, gated, tm, tn);
        pl.kernel = (int64_t)tm * tn >= 512 ? K_BF16_HUGE8 : K_BF16_LARGE;
        // Fewer 256 x 256 tiles than two rounds.  For long K first: 256 x 192
        // tiles with K split in two when the two halves make one round that
        // fills at least three quarters of the CUs (the QKV projection at
        // TP=16: 8192 x 8192 -> 768 is 128 tiles x 2 halves).  Per flop they
        // move 0.70x the operand bytes of 128 x 192 tiles from L2 to LDS, and
        // these launches run at the L2 -> LDS rate (~10 TB/s over all CUs);
        // the two fp32 halves are added in order by the split finish pass.
        //
        // Otherwise 128 x 192 tiles on the paired-stage kernel when they fill
        // at least three quarters of the CUs in every round (e.g. 8192 x 2048
        // -> 768: 256 tiles, one per CU, where 128 x 128 tiles left a quarter
        // of a round empty).
        if (pl.kernel == K_BF16_LARGE && !gated && K % 128 == 0 && K >= 4096) {
            int wm, wn;
            tiles_for(K_BF16_W192, M, N, gated, wm, wn);
            const int64_t wt = (int64_t)wm * wn;
            if (2 * wt <= 256 && 2 * wt >= 192) {
                pl.kernel = K_BF16_W192;
                pl.splits = 2;
                pl.k_split = K / 2;
                pl.ws_bytes = (size_t)2 * (size_t)M * (size_t)N * sizeof(float);
                return pl;
            }
        }
        if (pl.kernel == K_BF16_LARGE && !gated && K % 64 == 0) {
            int mm, mn;
            tiles_for(K_BF16_MID, M, N, gated, mm, mn);
            const int64_t mt = (int64_t)mm * mn;
            if (mt >= 192 && (mt % 256 == 0 || mt % 256 >= 192)) pl.kernel = K_BF16_MID;
        }
    } else {
        pl.kernel = K_BF16_DEC4;
    }
    tiles_for(pl.kernel, M, N, gated, tm, tn);
    const int64_t tiles = (int64_t)tm * tn;
    const int64_t Nb = gated ? 2 * N : N;
    // fewer tiles than CUs: split K so that the launch fills the machine
    if (tiles < 256 && K >= 1024 && pl.kernel != K_BF16_MID) {
        int64_t want = pl.kernel == K_BF16_DEC4 ? kSplitTargetDec4 / tiles : ceil_div(kSplitTarget, tiles);
        int64_t maxs = pl.kernel == K_BF16_DEC4 ? K / 256 : K / 512;
        int64_t s = want < maxs ? want : maxs;
        if (s > 1) {
            int64_t ks = ceil_div(ceil_div(K, s), 64) * 64;
            s = ceil_div(K, ks);
            if (s > 1) {
                pl.splits = (int)s;
                pl.k_split = ks;
                pl.ws_bytes = (size_t)s * (size_t)M * (size_t)Nb * sizeof(float);
            }
        }
    }
    // Balanced last round: with tiles = q * slots + rem (0 < rem <= slots/2,
    // slots = CUs x resident workgroups per CU), the last round would run
    // half empty or worse; instead cut each of the last rem tiles into
    // s = slots / rem K pieces so that round holds about one piece per slot,
    // and add the pieces afterwards (tail_fixup_kernel, fixed order).  Only
    // for long K: each piece costs a 4-byte-per-element partial tile written
    // and read back, which pieces shorter than 1024 do not pay for.
    const int64_t slots = 256 * wgs_per_cu(pl.kernel);
    if (pl.splits == 1 && K % 8 == 0 && tiles > slots && tiles % slots != 0 && pl.kernel != K_BF16_MID) {
        const int64_t rem = tiles % slots;
        int64_t sp = slots / rem;
        if (sp >= 2) {
            const int64_t tk = ceil_div(ceil_div(K, sp), 64) * 64;
            sp = ceil_div(K, tk);
            if (sp >= 2 && tk >= 1024) {
                TileCfg c = tile_cfg(pl.kernel);
                pl.full_tiles = (int)(tiles - rem);
                pl.tail_split = (int)sp;
                pl.tail_k = tk;
                pl.ws_bytes = (size_t)rem * (size_t)sp * (size_t)c.bm * (size_t)c.bn * sizeof(float);
            }
        }
    }
    return pl;
}

// adds the K pieces of a balanced last round (no-op without one)
template <int BM, int BN, int EPI>
static void launch_tail_fixup(const GemmArgs& a, int ntiles, hipStream_t s) {
    if (a.tail_split > 1 && EPI != EPI_SPLIT) {
        const int cols = EPI == EPI_GATED_BF16 ? BN / 2 : BN;
        int64_t blocks = ceil_div((int64_t)(ntiles - a.full_tiles) * BM * (cols / 4), 256);
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL((tail_fixup_kernel<EPI>), dim3((unsigned)blocks), dim3(256), 0, s, a, BM, BN);
    }
}

// direct-to-LDS kernel with 32x32x16 MFMAs (128 x 128 tiles)
template <int BM, int BN, int WM, int WN, int EPI>
static void launch_dl_one(const GemmArgs& a, int splits, hipStream_t s) {
    const int ntiles = a.tiles_m * a.tiles_n;
    const int units = a.tail_split > 1 ? a.full_tiles + (ntiles - a.full_tiles) * a.tail_split : ntiles;
    dim3 grid((unsigned)units, (unsigned)splits);
    const bool ktail = (a.K % 64) != 0 || (a.k_split % 64) != 0;
    // LDS ring depth 2: deeper rings measured slower here because they
    // cost a second resident workgroup per CU (occupancy beats depth)
    constexpr int NST = 2;
    if (ktail)
        hipLaunchKernelGGL((gemm_bf16_dl_kernel<BM, BN, WM, WN, EPI, true, NST>), grid, dim3(WM * WN * 64), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_bf16_dl_kernel<BM, BN, WM, WN, EPI, false, NST>), grid, dim3(WM * WN * 64), 0, s, a);
    launch_tail_fixup<BM, BN, EPI>(a, ntiles, s);
}

// register-staged kernel with element-wise loads (operands the 16-byte
// buffer loads cannot serve); whole tiles only
template <int BM, int BN, int WM, int WN, int EPI>
static void launch_reg_one(const GemmArgs& a, int splits, hipStream_t s) {
    const size_t lds = (size_t)2 * (BM + BN) * 64 * sizeof(uint16_t);
    auto kern = gemm_bf16_kernel<BM, BN, WM, WN, EPI>;
    if (lds > 65536) {
        // opt in to more than 64 KiB of LDS once per instantiation (a
        // function-local static: initialised once, thread-safe)
        static const bool opted_in = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         (int)lds) == hipSuccess;
        (void)opted_in;
    }
    dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)splits);
    hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), lds, s, a);
}

// deep-pipelined kernel (K steps of 32; direct-to-LDS operands only)
template <int BM, int BN, int WM, int WN, int EPI>
static void launch_pipe_one(const GemmArgs& a, int splits, hipStream_t s) {
    const int ntiles = a.tiles_m * a.tiles_n;
    const int units = a.tail_split > 1 ? a.full_tiles + (ntiles - a.full_tiles) * a.tail_split : ntiles;
    dim3 grid((unsigned)units, (unsigned)splits);
    const bool kt32 = (a.K % 32) != 0 || (a.k_split % 32) != 0;
    if constexpr (BN == 192) {
        // paired stages only (the planner takes these tiles for K ranges
        // that are multiples of 64, without tail pieces)
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, false, true>), grid, dim3(WM * WN * 64), 0, s, a);
        return;
    } else {
    // paired K = 64 stages: every K range a multiple of 64
    const bool pair = BM == 256 && a.K % 64 == 0 && a.k_split % 64 == 0 &&
                      (a.tail_split <= 1 || a.tail_k % 64 == 0);
    if constexpr (BM == 256) {
        if (pair) {
            hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, false, true>), grid, dim3(WM * WN * 64), 0, s, a);
            launch_tail_fixup<BM, BN, EPI>(a, ntiles, s);
            return;
        }
    }
    if (kt32)
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, true, false>), grid, dim3(WM * WN * 64), 0, s, a);
    else
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, EPI, false, false>), grid, dim3(WM * WN * 64), 0, s, a);
    launch_tail_fixup<BM, BN, EPI>(a, ntiles, s);
    }
}

enum Launcher { L_PIPE = 0, L_DL = 1, L_REG = 2 };

template <int L, int BM, int BN, int WM, int WN, int EPI>
static void launch_one(const GemmArgs& a, int splits, hipStream_t s) {
    if constexpr (L == L_PIPE) launch_pipe_one<BM, BN, WM, WN, EPI>(a, splits, s);
    else if constexpr (L == L_DL) launch_dl_one<BM, BN, WM, WN, EPI>(a, splits, s);
    else launch_reg_one<BM, BN, WM, WN, EPI>(a, splits, s);
}

template <int L, int BM, int BN, int WM, int WN>
static void launch_epi(int epi, const GemmArgs& a, int splits, hipStream_t s) {
    switch (epi) {
        case EPI_STORE_BF16: launch_one<L, BM, BN, WM, WN, EPI_STORE_BF16>(a, splits, s); break;
        case EPI_STORE_F32: launch_one<L, BM, BN, WM, WN, EPI_STORE_F32>(a, splits, s); break;
        case EPI_GATED_BF16:
            // 192-column tiles hold an odd number of 16-row blocks per wave:
            // the planner never gives them gated products
            if constexpr (BN != 192) launch_one<L, BM, BN, WM, WN, EPI_GATED_BF16>(a, splits, s);
            break;
        default: launch_one<L, BM, BN, WM, WN, EPI_SPLIT>(a, splits, s); break;
    }
}

// kern is the tile configuration (HUGE8 only for 16-byte-loadable operands)
static void launch_bf16_kern(int kern, int epi, const GemmArgs& a, int splits, bool vec, hipStream_t s) {
    if (!vec) {
        if (kern == K_BF16_DEC4 || kern == K_BF16_SMALL) launch_epi<L_REG, 64, 128, 1, 2>(epi, a, splits, s);
        else launch_epi<L_REG, 128, 128, 2, 2>(epi, a, splits, s);
        return;
    }
    switch (kern) {
        case K_BF16_HUGE8: launch_epi<L_PIPE, 256, 256, 2, 4>(epi, a, splits, s); break;
        case K_BF16_MID: launch_epi<L_PIPE, 128, 192, 2, 4>(epi, a, splits, s); break;
        case K_BF16_W192: launch_epi<L_PIPE, 256, 192, 2, 4>(epi, a, splits, s); break;
        case K_BF16_DEC4:
        case K_BF16_SMALL: launch_epi<L_PIPE, 64, 128, 1, 4>(epi, a, splits, s); break;
        default: launch_epi<L_DL, 128, 128, 2, 2>(epi, a, splits, s); break;
    }
}

hipError_t launch_gemm(const GemmPlan& pl, const void* A, const void* B, const void* bias, void* C,
                       int64_t M, int64_t N, int64_t K, bool gated, tp_dtype dt, tp_dtype out_dt,
                       void* ws, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t Nb = gated ? 2 * N : N;
    if (pl.kernel == K_F32) return launch_gemm_f32(A, B, bias, C, M, N, K, gated, s);
    const bool vec = (K % 8) == 0 && (((uintptr_t)A | (uintptr_t)B) & 15u) == 0;
    if (pl.kernel == K_BF16_RS) {
        if (!vec || !ws || (((uintptr_t)ws) & 15u) != 0) {
            // operands the 16-byte buffer loads cannot serve: the tiled kernel, whole K
            GemmPlan alt = pl;
            alt.kernel = K_BF16_SMALL;
            alt.splits = 1;
            alt.k_split = K;
            alt.ws_bytes = 0;
            return launch_gemm(alt, A, B, bias, C, M, N, K, gated, dt, out_dt, ws, s);
        }
        const RsOp o = make_rs_op(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B),
                                  static_cast<float*>(ws), M, K, Nb);
        const bool edge = (int64_t)o.S * RS_WAVES * o.R != K || (Nb % 16) != 0;
        const dim3 grid((unsigned)(o.S * o.G));
        switch (o.R / 32) {
#define RS_LAUNCH(NKS)                                                                         \
    case NKS:                                                                                  \
        if (edge) hipLaunchKernelGGL((gemm_bf16_rs_kernel<NKS, true>), grid, dim3(RS_WAVES * 64), 0, s, o);  \
        else hipLaunchKernelGGL((gemm_bf16_rs_kernel<NKS, false>), grid, dim3(RS_WAVES * 64), 0, s, o);      \
        break;
            RS_LAUNCH(4)
            RS_LAUNCH(5)
            RS_LAUNCH(6)
            RS_LAUNCH(7)
            RS_LAUNCH(8)
#undef RS_LAUNCH
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        GemmArgs a{};
        a.bias = static_cast<const uint16_t*>(bias);
        a.C = C;
        a.M = M;
        a.N = N;
        a.Nb = Nb;
        a.vec_out = (N % 4) == 0 && (((uintptr_t)C) & 15u) == 0;
        const dim3 fgrid((unsigned)ceil_div(N, 16));
        const int epi = gated ? EPI_GATED_BF16 : (out_dt == TP_F32 ? EPI_STORE_F32 : EPI_STORE_BF16);
        if (epi == EPI_GATED_BF16)
            hipLaunchKernelGGL(rs_finalize_kernel<EPI_GATED_BF16>, fgrid, dim3(256), 0, s, o, a);
        else if (epi == EPI_STORE_F32)
            hipLaunchKernelGGL(rs_finalize_kernel<EPI_STORE_F32>, fgrid, dim3(256), 0, s, o, a);
        else
            hipLaunchKernelGGL(rs_finalize_kernel<EPI_STORE_BF16>, fgrid, dim3(256), 0, s, o, a);
        return hipGetLastError();
    }
    if (pl.kernel == K_BF16_STREAM) {
        if (!vec || !ws || (((uintptr_t)ws) & 15u) != 0) {
            // operands DMA cannot load: the element-wise tiled kernel, whole K
            GemmPlan alt = pl;
            alt.kernel = K_BF16_SMALL;
            alt.splits = 1;
            alt.k_split = K;
            alt.ws_bytes = 0;
            return launch_gemm(alt, A, B, bias, C, M, N, K, gated, dt, out_dt, ws, s);
        }
        const StreamOp o = make_stream_op(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), M, N, K,
                                          gated, static_cast<float*>(ws), kStreamWGs);
        const bool ktail = (K % STR_BK) != 0;
        if (gated) {
            if (ktail) hipLaunchKernelGGL((gemm_bf16_stream_kernel<true, true>), dim3(kStreamWGs), dim3(256), 0, s, o);
            else hipLaunchKernelGGL((gemm_bf16_stream_kernel<true, false>), dim3(kStreamWGs), dim3(256), 0, s, o);
        } else {
            if (ktail) hipLaunchKernelGGL((gemm_bf16_stream_kernel<false, true>), dim3(kStreamWGs), dim3(256), 0, s, o);
            else hipLaunchKernelGGL((gemm_bf16_stream_kernel<false, false>), dim3(kStreamWGs), dim3(256), 0, s, o);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // finalize: block (tile, y), thread = (token row, 4 columns)
        GemmArgs a{};
        a.bias = static_cast<const uint16_t*>(bias);
        a.C = C;
        a.M = M;
        a.N = N;
        a.Nb = Nb;
        a.vec_out = (N % 4) == 0 && (((uintptr_t)C) & 15u) == 0;
        const int cols = gated ? STR_BN / 2 : STR_BN;
        const dim3 fgrid((unsigned)ceil_div(N, cols), (unsigned)ceil_div(M * (cols / 4), 256));
        const int epi = gated ? EPI_GATED_BF16 : (out_dt == TP_F32 ? EPI_STORE_F32 : EPI_STORE_BF16);
        if (epi == EPI_GATED_BF16)
            hipLaunchKernelGGL(stream_finalize_kernel<EPI_GATED_BF16>, fgrid, dim3(256), 0, s, o, a, kStreamWGs);
        else if (epi == EPI_STORE_F32)
            hipLaunchKernelGGL(stream_finalize_kernel<EPI_STORE_F32>, fgrid, dim3(256), 0, s, o, a, kStreamWGs);
        else
            hipLaunchKernelGGL(stream_finalize_kernel<EPI_STORE_BF16>, fgrid, dim3(256), 0, s, o, a, kStreamWGs);
        return hipGetLastError();
    }
    GemmArgs a{};
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.bias = static_cast<const uint16_t*>(bias);
    a.M = M;
    a.N = N;
    a.K = K;
    a.Nb = Nb;
    a.k_split = pl.splits > 1 ? pl.k_split : K;
    // operands the 16-byte loads cannot serve take the element-wise kernel,
    // 128 x 128 tiles in place of the direct-to-LDS ones
    const bool dma_tiles = pl.kernel == K_BF16_HUGE8 || pl.kernel == K_BF16_MID || pl.kernel == K_BF16_W192;
    const int kern = (!vec && dma_tiles) ? K_BF16_LARGE : pl.kernel;
    if (pl.splits > 1) {
        // split partials are kept in B-row coordinates over all Nb rows
        TileCfg c = tile_cfg(kern);
        a.tiles_m = (int)ceil_div(M, c.bm);
        a.tiles_n = (int)ceil_div(Nb, c.bn);
        a.N = Nb;
        a.C = ws;
        a.vec_out = (Nb % 4) == 0 && (((uintptr_t)ws) & 15u) == 0;
        launch_bf16_kern(kern, EPI_SPLIT, a, pl.splits, vec, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        int64_t blocks = ceil_div(M * N, 256);
        if (blocks > 8192) blocks = 8192;
        const int epi = gated ? EPI_GATED_BF16 : (out_dt == TP_F32 ? EPI_STORE_F32 : EPI_STORE_BF16);
        const float* wsf = static_cast<const float*>(ws);
        const uint16_t* bb = static_cast<const uint16_t*>(bias);
        if (epi == EPI_GATED_BF16)
            hipLaunchKernelGGL(splitk_finalize_kernel<EPI_GATED_BF16>, dim3((unsigned)blocks), dim3(256), 0, s,
                               wsf, pl.splits, M, N, Nb, bb, C);
        else if (epi == EPI_STORE_F32)
            hipLaunchKernelGGL(splitk_finalize_kernel<EPI_STORE_F32>, dim3((unsigned)blocks), dim3(256), 0, s,
                               wsf, pl.splits, M, N, Nb, bb, C);
        else
            hipLaunchKernelGGL(splitk_finalize_kernel<EPI_STORE_BF16>, dim3((unsigned)blocks), dim3(256), 0, s,
                               wsf, pl.splits, M, N, Nb, bb, C);
        return hipGetLastError();
    }
    int tm, tn;
    tiles_for(kern, M, N, gated, tm, tn);
    a.tiles_m = tm;
    a.tiles_n = tn;
    a.C = C;
    if (pl.tail_split > 1 && vec && ws && (((uintptr_t)ws) & 15u) == 0) {
        a.full_tiles = pl.full_tiles;
        a.tail_split = pl.tail_split;
        a.tail_k = pl.tail_k;
        a.tail_ws = static_cast<float*>(ws);
    }
    a.vec_out = (N % 4) == 0 && (((uintptr_t)C) & 15u) == 0;
    const int epi = gated ? EPI_GATED_BF16 : (out_dt == TP_F32 ? EPI_STORE_F32 : EPI_STORE_BF16);
    launch_bf16_kern(kern, epi, a, 1, vec, s);
    return hipGetLastError();
}

}  // namespace tpk
