// GEMMs of the rank shard: C[M, N] = A[M, K] . B[N, K]^T, both operands
// contiguous along K (weights stored [out, in], x . W^T), and the fused
// column-parallel gate_up form act = SiLU(A . G^T) * (A . U^T) with
// B = [G ; U] (gate rows first).
//
// bf16 path: MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulators.
//   * Workgroup tile BM x BN x BK, WM x WN wavefronts, each wave owning a
//     (BM/WM) x (BN/WN) block of 32x32 MFMA tiles.
//   * Global -> LDS: 16-byte loads, double-buffered LDS so the next K tile is
//     fetched while MFMAs run on the current one; one barrier per K step.
//   * LDS layout: each tile row is BK bf16 = BK/8 16-byte chunks; chunk c of
//     row r is stored at position c ^ ((r ^ (r >> 3)) & 7), which keeps both
//     the row-wise 16-byte stores and the MFMA fragment loads (32 rows, one
//     chunk) free of bank conflicts for 32- and 64-bank LDS.
//   * Gated epilogue: a tile loads BN/2 gate rows and the SAME BN/2 up rows;
//     each wave's MFMA N-tiles are split half gate, half up, so a lane holds
//     gate and up accumulators of the same (row, column) and applies
//     SiLU(g) * u in registers.  Gate/up products never reach memory.
//   * Split-K (small M): blockIdx.y picks a K range; fp32 partial sums go to
//     a workspace and a finalize kernel adds the splits in order 0..S-1 and
//     applies the epilogue (deterministic, no atomics).
//   * Tile order: workgroups are dispatched round-robin over the 8 XCDs; the
//     linear block id is remapped so that each XCD receives a contiguous run
//     of tiles, grouped GROUP_M tiles tall so that the weight tile and the
//     activation tiles a run shares stay in that XCD's L2.
//
// fp32 path: VALU FMA tiles (no reduced-precision fp32 modes).
#include "common.hpp"

namespace tpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_STORE_BF16 = 0, EPI_STORE_F32 = 1, EPI_GATED_BF16 = 2, EPI_SPLIT = 3,
           EPI_GATED_F32 = 4 };

struct GemmArgs {
    const uint16_t* A;      // [M, K]
    const uint16_t* B;      // [Nb, K]
    const uint16_t* bias;   // [N] or null (store epilogues only)
    void* C;                // output [M, N], or fp32 workspace [splits][M][Nb]
    int64_t M, N, K, Nb;    // N = output columns (act columns when gated)
    int64_t k_split;        // K elements per split
    int tiles_m, tiles_n;
};

constexpr int GROUP_M = 8;

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

template <int BM, int BN, int BK, int WM, int WN, int EPI, bool VEC>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmArgs p) {
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

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (A_ELEMS + B_ELEMS)];

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

    // ---- global -> register staging ------------------------------------
    u32x4 ra[A_LD], rb[B_LD];

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

    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int v = tid + i * NT;
            const int row = v / KC, kc = v % KC;
            const int64_t gm = m0 + row;
            const int64_t k = k0 + kc * 8;
            if (VEC) {
                if (gm < p.M && k < k_end)
                    ra[i] = *reinterpret_cast<const u32x4*>(A + gm * p.K + k);
                else
                    ra[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t lo = 0, hi = 0;
                    if (gm < p.M && k + 2 * q < k_end) lo = A[gm * p.K + k + 2 * q];
                    if (gm < p.M && k + 2 * q + 1 < k_end) hi = A[gm * p.K + k + 2 * q + 1];
                    w[q] = lo | (hi << 16);
                }
                ra[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int v = tid + i * NT;
            const int row = v / KC, kc = v % KC;
            bool ok;
            const int64_t gb = b_row(row, ok);
            const int64_t k = k0 + kc * 8;
            if (VEC) {
                if (ok && k < k_end)
                    rb[i] = *reinterpret_cast<const u32x4*>(B + gb * p.K + k);
                else
                    rb[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t lo = 0, hi = 0;
                    if (ok && k + 2 * q < k_end) lo = B[gb * p.K + k + 2 * q];
                    if (ok && k + 2 * q + 1 < k_end) hi = B[gb * p.K + k + 2 * q + 1];
                    w[q] = lo | (hi << 16);
                }
                rb[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
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

    // wave's B-tile row base for MFMA N-tile tn
    auto b_tile_row = [&](int tn) -> int {
        if (GATED) {
            constexpr int HALF_W = WTN / 2;     // gate (or up) rows per wave
            return tn < TN / 2 ? wn * HALF_W + tn * 32 : BN / 2 + wn * HALF_W + (tn - TN / 2) * 32;
        }
        return wn * WTN + tn * 32;
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (int)ceil_div(k_end - k_begin, BK);
    if (nk > 0) {
        load_tile(k_begin);
        store_tile(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tile(k_begin + (int64_t)(kt + 1) * BK);
        const uint16_t* As = smem + cur * (A_ELEMS + B_ELEMS);
        const uint16_t* Bs = As + A_ELEMS;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WTM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8*>(As + row * BK + swz(row, c) * 8);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = b_tile_row(j) + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + row * BK + swz(row, c) * 8);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue --------------------------------------------------------
    // 32x32 MFMA result layout: lane l holds column (l & 31) of the tile and,
    // in accumulator r, row 8*(r/4) + 4*(l/32) + (r%4).
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
    if (EPI == EPI_SPLIT) {
        float* ws = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.M * p.Nb;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t gc = n0 + b_tile_row(j) + col_l;
                if (gc >= p.Nb) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t gr = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                    if (gr < p.M) ws[gr * p.Nb + gc] = acc[i][j][r];
                }
            }
    } else if (GATED) {
        uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN / 2; ++j) {
                const int64_t gc = n0 + wn * (WTN / 2) + j * 32 + col_l;
                if (gc >= p.N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t gr = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                    if (gr < p.M) C[gr * p.N + gc] = f32_to_bf16(silu_mul(acc[i][j][r], acc[i][j + TN / 2][r]));
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t gc = n0 + b_tile_row(j) + col_l;
                if (gc >= p.N) continue;
                const float bv = p.bias ? bf16_to_f32(p.bias[gc]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t gr = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                    if (gr >= p.M) continue;
                    const float v = acc[i][j][r] + bv;
                    if (EPI == EPI_STORE_F32)
                        static_cast<float*>(p.C)[gr * p.N + gc] = v;
                    else
                        static_cast<uint16_t*>(p.C)[gr * p.N + gc] = f32_to_bf16(v);
                }
            }
    }
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

// ---- fp32 VALU GEMM -----------------------------------------------------

struct F32Args {
    const float* A;
    const float* B;
    const float* bias;
    float* C;
    int64_t M, N, K, Nb;
    int tiles_m, tiles_n;
};

// 64 x 64 B-row tile (gated: 32 gate + the same 32 up rows), BK = 16, 256
// threads each computing 4 rows x 4 B-columns; a thread's columns are
// {2tx, 2tx+1, 32+2tx, 33+2tx} so that, gated, its gate and up values meet.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Args p) {
    constexpr int TMT = 64, TNT = 64, BK = 16;
    constexpr bool GATED = EPI == EPI_GATED_F32;
    __shared__ float As[BK][TMT + 4];
    __shared__ float Bs[BK][TNT + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int tile_m = blockIdx.x / p.tiles_n, tile_n = blockIdx.x % p.tiles_n;
    const int64_t m0 = (int64_t)tile_m * TMT;
    const int64_t n0 = GATED ? (int64_t)tile_n * (TNT / 2) : (int64_t)tile_n * TNT;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + i * 256;
            const int row = v / BK, kk = v % BK;
            const int64_t gm = m0 + row, k = k0 + kk;
            As[kk][row] = (gm < p.M && k < p.K) ? p.A[gm * p.K + k] : 0.0f;
            int64_t gb;
            bool ok;
            if (GATED) {
                const int64_t c = n0 + (row < 32 ? row : row - 32);
                ok = c < p.N;
                gb = row < 32 ? c : p.N + c;
            } else {
                gb = n0 + row;
                ok = gb < p.Nb;
            }
            Bs[kk][row] = (ok && k < p.K) ? p.B[gb * p.K + k] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][(j >> 1) * 32 + tx * 2 + (j & 1)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gr = m0 + ty * 4 + i;
        if (gr >= p.M) continue;
        if (GATED) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t gc = n0 + tx * 2 + j;
                if (gc < p.N) p.C[gr * p.N + gc] = silu_mul(acc[i][j], acc[i][j + 2]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t gc = n0 + (j >> 1) * 32 + tx * 2 + (j & 1);
                if (gc < p.N) p.C[gr * p.N + gc] = acc[i][j] + (p.bias ? p.bias[gc] : 0.0f);
            }
        }
    }
}

// ---- planning -------------------------------------------------------------

enum Kern { K_F32 = 0, K_BF16_LARGE = 1, K_BF16_SMALL = 2 };

// Tile configurations: LARGE 128x128x64 with 2x2 waves; SMALL (M <= 64)
// 64x128x64 with 1x2 waves.
struct TileCfg { int bm, bn; };
static TileCfg tile_cfg(int k) { return k == K_BF16_SMALL ? TileCfg{64, 128} : TileCfg{128, 128}; }

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

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool gated, tp_dtype dt) {
    GemmPlan pl{};
    pl.splits = 1;
    pl.k_split = K;
    pl.ws_bytes = 0;
    if (dt == TP_F32) {
        pl.kernel = K_F32;
        return pl;
    }
    pl.kernel = M <= 64 ? K_BF16_SMALL : K_BF16_LARGE;
    int tm, tn;
    tiles_for(pl.kernel, M, N, gated, tm, tn);
    const int64_t tiles = (int64_t)tm * tn;
    const int64_t Nb = gated ? 2 * N : N;
    // fewer tiles than CUs: split K so that the launch fills the machine
    if (tiles < 256 && K >= 1024) {
        int64_t want = ceil_div(1024, tiles);
        int64_t maxs = K / 512;
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
    return pl;
}

template <int BM, int BN, int WM, int WN, int EPI>
static void launch_bf16_cfg(const GemmArgs& a, int splits, bool vec, hipStream_t s) {
    dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)splits);
    dim3 block(WM * WN * 64);
    if (vec)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 64, WM, WN, EPI, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 64, WM, WN, EPI, false>), grid, block, 0, s, a);
}

template <int BM, int BN, int WM, int WN>
static void launch_bf16_epi(int epi, const GemmArgs& a, int splits, bool vec, hipStream_t s) {
    switch (epi) {
        case EPI_STORE_BF16: launch_bf16_cfg<BM, BN, WM, WN, EPI_STORE_BF16>(a, splits, vec, s); break;
        case EPI_STORE_F32: launch_bf16_cfg<BM, BN, WM, WN, EPI_STORE_F32>(a, splits, vec, s); break;
        case EPI_GATED_BF16: launch_bf16_cfg<BM, BN, WM, WN, EPI_GATED_BF16>(a, splits, vec, s); break;
        default: launch_bf16_cfg<BM, BN, WM, WN, EPI_SPLIT>(a, splits, vec, s); break;
    }
}

hipError_t launch_gemm(const GemmPlan& pl, const void* A, const void* B, const void* bias, void* C,
                       int64_t M, int64_t N, int64_t K, bool gated, tp_dtype dt, tp_dtype out_dt,
                       void* ws, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t Nb = gated ? 2 * N : N;
    int tm, tn;
    tiles_for(pl.kernel, M, N, gated && pl.splits == 1, tm, tn);
    if (pl.kernel == K_F32) {
        F32Args a{static_cast<const float*>(A), static_cast<const float*>(B),
                  static_cast<const float*>(bias), static_cast<float*>(C), M, N, K, Nb, tm, tn};
        dim3 grid((unsigned)(tm * tn));
        if (gated)
            hipLaunchKernelGGL(gemm_f32_kernel<EPI_GATED_F32>, grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE_F32>, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const bool vec = (K % 8) == 0 && (((uintptr_t)A | (uintptr_t)B) & 15u) == 0;
    GemmArgs a{};
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.bias = static_cast<const uint16_t*>(bias);
    a.M = M;
    a.N = N;
    a.K = K;
    a.Nb = Nb;
    a.k_split = pl.splits > 1 ? pl.k_split : K;
    if (pl.splits > 1) {
        // split partials are kept in B-row coordinates over all Nb rows
        TileCfg c = tile_cfg(pl.kernel);
        a.tiles_m = (int)ceil_div(M, c.bm);
        a.tiles_n = (int)ceil_div(Nb, c.bn);
        a.N = Nb;
        a.C = ws;
        if (pl.kernel == K_BF16_SMALL)
            launch_bf16_epi<64, 128, 1, 2>(EPI_SPLIT, a, pl.splits, vec, s);
        else
            launch_bf16_epi<128, 128, 2, 2>(EPI_SPLIT, a, pl.splits, vec, s);
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
    a.tiles_m = tm;
    a.tiles_n = tn;
    a.C = C;
    const int epi = gated ? EPI_GATED_BF16 : (out_dt == TP_F32 ? EPI_STORE_F32 : EPI_STORE_BF16);
    if (pl.kernel == K_BF16_SMALL)
        launch_bf16_epi<64, 128, 1, 2>(epi, a, 1, vec, s);
    else
        launch_bf16_epi<128, 128, 2, 2>(epi, a, 1, vec, s);
    return hipGetLastError();
}

}  // namespace tpk
