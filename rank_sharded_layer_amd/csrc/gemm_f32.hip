// fp32 GEMMs of the rank shard (the same contract as the bf16 path in
// gemm.hip: C[M, N] = A[M, K] . B[N, K]^T (+bias), or the gated form
// act = SiLU(A . G^T) * (A . U^T) with B = [G ; U]): fp32 products and sums
// throughout, no reduced-precision fp32 modes.
//   * few tokens (M <= 32), 16-byte rows, K <= 2048: gemm_f32_mfma_kernel on
//     v_mfma_f32_16x16x4_f32;
//   * few tokens otherwise: gemm_f32_small_kernel (VALU, 4 B rows per wave);
//   * larger M: gemm_f32_kernel (VALU FMA tiles).
#include "common.hpp"

namespace tpk {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// epilogues of gemm_f32_kernel: C (+bias), or the gated activation
enum F32Epi { F32_STORE = 0, F32_GATED = 1 };

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
    constexpr bool GATED = EPI == F32_GATED;
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

// fp32, few tokens (M <= 32): each wave owns RW weight rows (gated: RW/2
// gate rows and the same up rows) for all M tokens; lane l takes k = l,
// l+64, ... and keeps M x RW fp32 partial dot products (sequential FMAs);
// the 64 lanes' partials are then added in lane order through LDS
// (deterministic).  Launch-latency-sized problems get ~N/RW waves.
template <bool GATED, int MT>
__global__ __launch_bounds__(256) void gemm_f32_small_kernel(F32Args p) {
    constexpr int RW = 4;                       // B rows per wave
    constexpr int NW = 4;                       // waves per workgroup
    __shared__ float red[NW][MT * RW][65];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // this wave's B rows
    const int64_t unit = (int64_t)blockIdx.x * NW + w;     // RW/2 act columns (gated) or RW rows
    int64_t brow[RW];
    bool bok[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        if (GATED) {
            const int64_t c = unit * (RW / 2) + (r % (RW / 2));
            bok[r] = c < p.N;
            brow[r] = r < RW / 2 ? c : p.N + c;
        } else {
            brow[r] = unit * RW + r;
            bok[r] = brow[r] < p.Nb;
        }
    }
    float acc[MT][RW];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[m][r] = 0.0f;
    for (int64_t k = lane; k < p.K; k += 64) {
        float wv[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) wv[r] = bok[r] ? p.B[brow[r] * p.K + k] : 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float xv = m < p.M ? p.A[(int64_t)m * p.K + k] : 0.0f;
#pragma unroll
            for (int r = 0; r < RW; ++r) acc[m][r] = fmaf(xv, wv[r], acc[m][r]);
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < RW; ++r) red[w][m * RW + r][lane] = acc[m][r];
    __syncthreads();
    // lane e of wave w finishes value e (m = e / RW, r = e % RW) of this wave
    for (int e = lane; e < MT * RW; e += 64) {
        float v = 0.0f;
        for (int l = 0; l < 64; ++l) v = v + red[w][e][l];
        red[w][e][64] = v;
    }
    __syncthreads();
    for (int e = lane; e < MT * RW; e += 64) {
        const int m = e / RW, r = e % RW;
        if (m >= p.M) continue;
        if (GATED) {
            if (r >= RW / 2) continue;
            const int64_t c = unit * (RW / 2) + r;
            if (c < p.N) p.C[(int64_t)m * p.N + c] = silu_mul(red[w][e][64], red[w][m * RW + r + RW / 2][64]);
        } else {
            const int64_t c = unit * RW + r;
            if (c < p.N) p.C[(int64_t)m * p.N + c] = red[w][e][64] + (p.bias ? p.bias[c] : 0.0f);
        }
    }
}

// fp32, few tokens (M <= 32, K <= 2048, 16-byte rows): one workgroup of 16
// waves per COLS output columns, the waves splitting K into 16 ranges of
// STEPS x 16.  The weight rows of a workgroup fill one 16-row MFMA block
// (COLS = 16, gated: a block of 16 gate rows and one of the same 16 up rows;
// COLS <= 8 gated: gate rows in block rows 0..7, the same up rows in 8..15;
// COLS < 16 plain: block rows past COLS are zero and not loaded), so that
// narrow products still spread over every CU.  Per 16 K values a lane loads
// 16 bytes of its weight row (row l & 15, K values 4 (l >> 4) .. +3) and 16
// bytes of its token row, and the four K values go in order to four
// v_mfma_f32_16x16x4_f32 (fp32 products and sums, no reduced-precision
// inputs).  Every load of a wave is issued before its first MFMA: the whole
// product is one round trip to memory per wave.  The 16 waves' sums meet in
// LDS and are added in wave (= K) order, so the result is deterministic.
constexpr int F32W = 16;

template <bool GATED, int TB, int STEPS, int COLS>
__global__ __launch_bounds__(F32W * 64) void gemm_f32_mfma_kernel(F32Args p) {
    static_assert(COLS == 16 || COLS == 8 || COLS == 4, "column blocks of 16, 8 or 4");
    constexpr bool PAIRED = GATED && COLS <= 8;          // gate and up rows share one block
    constexpr int RB = (GATED && !PAIRED) ? 2 : 1;
    typedef float f4v __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) f32x4 red[F32W][RB][TB][64];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kq = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * COLS;
    const int64_t kbeg = (int64_t)wid * STEPS * 16 + kq * 4;
    const float* wrow[RB];
    bool wok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row;
        if (PAIRED) {
            const int c = r16 & 7;
            wok[rb] = c < COLS && n0 + c < p.N;
            row = (r16 < 8 ? 0 : p.N) + n0 + c;
        } else if (GATED) {
            wok[rb] = n0 + r16 < p.N;
            row = (rb == 0 ? 0 : p.N) + n0 + r16;
        } else {
            wok[rb] = r16 < COLS && n0 + r16 < p.N;
            row = n0 + r16;
        }
        wrow[rb] = p.B + (wok[rb] ? row : 0) * p.K;
    }
    const float* xrow[TB];
    bool xok[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        xok[tb] = tb * 16 + r16 < p.M;
        xrow[tb] = p.A + (int64_t)(tb * 16 + r16) * p.K;
    }
    f4v w[STEPS][RB], x[STEPS][TB];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t k = kbeg + s * 16;
        const bool kin = k < p.K;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            w[s][rb] = (kin && wok[rb]) ? *reinterpret_cast<const f4v*>(wrow[rb] + k) : (f4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            x[s][tb] = (kin && xok[tb]) ? *reinterpret_cast<const f4v*>(xrow[tb] + k) : (f4v){0.0f, 0.0f, 0.0f, 0.0f};
    }
    f32x4 acc[RB][TB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rb][tb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    acc[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x4f32(w[s][rb][e], x[s][tb][e], acc[rb][tb], 0, 0, 0);
    // lane l of block (rb, tb) holds block rows 4 (l >> 4) .. +3 for token
    // 16 tb + (l & 15)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) red[wid][rb][tb][lane] = acc[rb][tb];
    __syncthreads();
    const int t = threadIdx.x;
    if (t >= TB * 64) return;
    const int tb = t >> 6, l = t & 63;
    // this thread's columns n0 + 4 (l >> 4) .. +3 (paired: block rows of the
    // gate half only, the up rows sit 8 rows = two lane groups further)
    const int c4 = 4 * (l >> 4);
    if (c4 >= COLS) return;
    f32x4 v0 = red[0][0][tb][l];
#pragma unroll
    for (int wv = 1; wv < F32W; ++wv) v0 = v0 + red[wv][0][tb][l];
    float v[4];
    if constexpr (GATED) {
        const int ub = PAIRED ? 0 : RB - 1, ul = PAIRED ? l + 32 : l;
        f32x4 v1 = red[0][ub][tb][ul];
#pragma unroll
        for (int wv = 1; wv < F32W; ++wv) v1 = v1 + red[wv][ub][tb][ul];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu_mul(v0[e], v1[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = v0[e];
    }
    const int64_t m = tb * 16 + (l & 15);
    const int64_t c0 = n0 + c4;
    if (m >= p.M || c0 >= p.N) return;
    float* dst = p.C + m * p.N + c0;
    if (!GATED && p.bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < p.N) v[e] = v[e] + p.bias[c0 + e];
    }
    if (c0 + 3 < p.N && ((p.N & 3) == 0) && ((((uintptr_t)p.C) & 15u) == 0)) {
        *reinterpret_cast<f4v*>(dst) = (f4v){v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < p.N) dst[e] = v[e];
    }
}

// Output columns per workgroup of gemm_f32_mfma_kernel: gated, 8 (a full
// 16-row block of 8 gate and 8 up rows) unless 16 still give every CU a
// workgroup; plain, the widest of 16, 8, 4 that gives every CU one, else 4.
// (Qwen3-0.6B rank at TP=2, 16 tokens: gate_up 1536 act columns, 16 -> 8:
// 9.8 -> 7.4 us; down 1024 columns, 16 -> 4: 9.0 -> 8.0 us.)
static int f32_cols_of(int64_t N, bool gated) {
    constexpr int64_t kWGs = 256;
    if (gated) return N >= 16 * kWGs ? 16 : 8;
    return N >= 16 * kWGs ? 16 : N >= 8 * kWGs ? 8 : 4;
}

hipError_t launch_gemm_f32(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                           int64_t K, bool gated, hipStream_t s) {
    const int64_t Nb = gated ? 2 * N : N;
    const int tm = (int)ceil_div(M, 64);
    const int tn = (int)(gated ? ceil_div(N, 32) : ceil_div(N, 64));
    F32Args a{static_cast<const float*>(A), static_cast<const float*>(B),
              static_cast<const float*>(bias), static_cast<float*>(C), M, N, K, Nb, tm, tn};
    const bool f32_vec = (K % 4) == 0 && (((uintptr_t)A | (uintptr_t)B) & 15u) == 0;
    if (M <= 32 && f32_vec && K <= 16 * 16 * 8) {
        // one 16-wave workgroup per COLS output columns, STEPS x 16 K per
        // wave; COLS as wide as still gives a workgroup to every CU
        const int steps = (int)ceil_div(K, 16 * F32W);
        const int cols = f32_cols_of(N, gated);
        const dim3 g((unsigned)ceil_div(N, cols));
#define F32M_STEPS(G_, TB_, C_)                                                                              \
    switch (steps) {                                                                                         \
        case 1: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 1, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        case 2: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 2, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        case 3: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 3, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        case 4: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 4, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        case 5: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 5, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        case 6: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 6, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        case 7: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 7, C_>), g, dim3(F32W * 64), 0, s, a); break; \
        default: hipLaunchKernelGGL((gemm_f32_mfma_kernel<G_, TB_, 8, C_>), g, dim3(F32W * 64), 0, s, a); break; \
    }
#define F32M_LAUNCH(G_, TB_)                                   \
    switch (cols) {                                            \
        case 16: F32M_STEPS(G_, TB_, 16) break;                \
        case 8: F32M_STEPS(G_, TB_, 8) break;                  \
        default: F32M_STEPS(G_, TB_, 4) break;                 \
    }
        if (gated) {
            if (M <= 16) { F32M_LAUNCH(true, 1) } else { F32M_LAUNCH(true, 2) }
        } else {
            if (M <= 16) { F32M_LAUNCH(false, 1) } else { F32M_LAUNCH(false, 2) }
        }
#undef F32M_LAUNCH
#undef F32M_STEPS
        return hipGetLastError();
    }
    if (M <= 32) {
        // 4 waves per workgroup, 4 B rows (gated: 2 act columns) per wave
        const int64_t units = gated ? ceil_div(N, 2) : ceil_div(N, 4);
        dim3 g((unsigned)ceil_div(units, 4));
        if (gated) {
            if (M <= 16) hipLaunchKernelGGL((gemm_f32_small_kernel<true, 16>), g, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((gemm_f32_small_kernel<true, 32>), g, dim3(256), 0, s, a);
        } else {
            if (M <= 16) hipLaunchKernelGGL((gemm_f32_small_kernel<false, 16>), g, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((gemm_f32_small_kernel<false, 32>), g, dim3(256), 0, s, a);
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)(tm * tn));
    if (gated)
        hipLaunchKernelGGL(gemm_f32_kernel<F32_GATED>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(gemm_f32_kernel<F32_STORE>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace tpk
