/*
 * tp_oracle.c -- fp64 CPU oracle for one tensor-parallel rank's share of a
 * Transformer layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the HIP library
 * is checked against.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Style: plain loops in the order the pages state the method; fp64 for every
 * floating-point value unless a function says otherwise; OpenMP only splits
 * independent output rows (it never changes a sum's order).  Built with
 * -O2 -ffp-contract=off and without -ffast-math so every sum is the plain
 * left-to-right sequence written here.
 *
 * Pages cited (titles as the pages give them, shortened):
 *   [VLLM13]  "vLLM source analysis 13 -- vLLM distributed inference: tensor
 *             parallelism in detail"
 *   [NANO22]  "Nano-vLLM source walkthrough no. 22 -- tensor parallelism (2):
 *             code"
 *   [SCRATCH] "Tensor parallelism: implemented from scratch" (AI-infra
 *             handbook, distributed serving)
 *   [GUIDE62] "AIInfraGuide 6.2 -- tensor-parallel inference"
 *
 * Weight storage follows [NANO22] §2: a linear layer's weight is stored
 * [out, in] and the layer computes y = x . W^T, so a column split is a cut of
 * dim 0 (whole rows) and a row split is a cut of dim 1 (columns).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Scalar pieces                                                            */
/* ------------------------------------------------------------------------ */

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}).  [SCRATCH] "Implementation",
 * class TPMLP: the MLP applies F.silu to the gate projection and multiplies
 * the result by the up projection. */
ORC_API double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Round an fp32 value to bfloat16 with round-to-nearest-even, returning the
 * 16 stored bits.  bfloat16 keeps the top 16 bits of the IEEE-754 binary32
 * encoding (1 sign, 8 exponent, 7 mantissa bits).  The discarded low half is
 * compared with the halfway point 0x8000; ties go to the candidate whose last
 * kept bit is 0.  NaN stays NaN (quiet bit forced).  Overflow past the largest
 * finite bf16 rounds to infinity, as RNE prescribes. */
ORC_API uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xffffu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
    return (uint16_t)hi;
}

ORC_API float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

ORC_API void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

ORC_API void orc_bf16_to_f64_array(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (double)orc_bf16_to_f32(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Linear layers                                                            */
/* ------------------------------------------------------------------------ */

/* y[i, o] = sum_k x[i, k] * w[o, k]  (+ bias[o] if bias != NULL).
 * F.linear semantics, weight stored [out, in]: [NANO22] §2 and §4.  The sum
 * runs k = 0, 1, ..., K-1 and the bias is added last. */
ORC_API void orc_linear(const double* x, int64_t n, int64_t k,
                        const double* w, int64_t m, const double* bias,
                        double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const double* xi = x + i * k;
        for (int64_t o = 0; o < m; ++o) {
            const double* wo = w + o * k;
            double s = 0.0;
            for (int64_t j = 0; j < k; ++j) s += xi[j] * wo[j];
            if (bias) s += bias[o];
            y[i * m + o] = s;
        }
    }
}

/* Unsharded MLP: y = (SiLU(x . gate^T) * (x . up^T)) . down^T.
 *   x [n, h], gate/up [f, h], down [h, f], y [n, h].
 * [SCRATCH] "Implementation", class TPMLP (down(silu(gate(x)) * up(x)));
 * [GUIDE62] §1, FFN written as Y = act(XA) B.
 * Row-at-a-time: the [f] intermediate of one token is built, then projected. */
ORC_API void orc_mlp(const double* x, int64_t n, int64_t h,
                     const double* gate, const double* up, int64_t f,
                     const double* down, double* y) {
#pragma omp parallel
    {
        double* act = (double*)malloc(sizeof(double) * (size_t)(f > 0 ? f : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const double* xi = x + i * h;
            for (int64_t j = 0; j < f; ++j) {
                double g = 0.0, u = 0.0;
                for (int64_t k = 0; k < h; ++k) {
                    g += xi[k] * gate[j * h + k];
                    u += xi[k] * up[j * h + k];
                }
                act[j] = orc_silu(g) * u;
            }
            for (int64_t o = 0; o < h; ++o) {
                double s = 0.0;
                for (int64_t j = 0; j < f; ++j) s += act[j] * down[o * f + j];
                y[i * h + o] = s;
            }
        }
        free(act);
    }
}

/* Rank r's partial of the tensor-parallel MLP, computed from the FULL
 * weights by index arithmetic (no shard copies):
 *   P_r = SiLU(x . G_r^T) * (x . U_r^T) . D_r^T
 * with G_r = gate rows [r*f/t, (r+1)*f/t), U_r the same rows of up and
 * D_r = down columns [r*f/t, (r+1)*f/t).
 * [GUIDE62] §1: the first matrix is cut by columns (A = [A_1..A_t]), the
 * activation acts element-wise on each rank's own columns, the second matrix
 * is cut along f into B_1..B_t, and rank i obtains the full-shape n x h
 * partial act(X A_i) B_i.  In [out, in] storage the column cut of gate/up
 * is a row range and the row cut of down is a column range ([NANO22] §2).
 * The caller guarantees t divides f. */
ORC_API void orc_mlp_rank(const double* x, int64_t n, int64_t h,
                          const double* gate, const double* up, int64_t f,
                          const double* down, int tp_rank, int tp_size,
                          double* partial) {
    int64_t fl = f / tp_size;
    int64_t f0 = (int64_t)tp_rank * fl;
#pragma omp parallel
    {
        double* act = (double*)malloc(sizeof(double) * (size_t)(fl > 0 ? fl : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const double* xi = x + i * h;
            for (int64_t j = 0; j < fl; ++j) {
                const double* gr = gate + (f0 + j) * h;
                const double* ur = up + (f0 + j) * h;
                double g = 0.0, u = 0.0;
                for (int64_t k = 0; k < h; ++k) {
                    g += xi[k] * gr[k];
                    u += xi[k] * ur[k];
                }
                act[j] = orc_silu(g) * u;
            }
            for (int64_t o = 0; o < h; ++o) {
                const double* dr = down + o * f + f0;
                double s = 0.0;
                for (int64_t j = 0; j < fl; ++j) s += act[j] * dr[j];
                partial[i * h + o] = s;
            }
        }
        free(act);
    }
}

/* Element-wise SiLU(g) * u on the local [n, f_l] activations (the step that
 * stays on each rank because it is element-wise: [GUIDE62] §1). */
ORC_API void orc_silu_mul(const double* g, const double* u, int64_t count,
                          double* act) {
    for (int64_t i = 0; i < count; ++i) act[i] = orc_silu(g[i]) * u[i];
}

/* ------------------------------------------------------------------------ */
/* Shard selection (element-size generic, bit-exact copies)                 */
/* ------------------------------------------------------------------------ */

/* out = full.narrow(dim, start, len) made contiguous.  full is [rows, cols]
 * row-major with `esize`-byte elements. */
ORC_API int orc_narrow(const void* full, int64_t rows, int64_t cols, int esize,
                       int dim, int64_t start, int64_t len, void* out) {
    const unsigned char* src = (const unsigned char*)full;
    unsigned char* dst = (unsigned char*)out;
    if (dim == 0) {
        if (start < 0 || start + len > rows) return 1;
        for (int64_t i = 0; i < len; ++i)
            for (int64_t j = 0; j < cols; ++j)
                memcpy(dst + (i * cols + j) * esize,
                       src + ((start + i) * cols + j) * esize, (size_t)esize);
    } else if (dim == 1) {
        if (start < 0 || start + len > cols) return 1;
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < len; ++j)
                memcpy(dst + (i * len + j) * esize,
                       src + (i * cols + start + j) * esize, (size_t)esize);
    } else {
        return 1;
    }
    return 0;
}

/* Column-/row-parallel weight loader: shard_size = size(dim)/t,
 * start = tp_rank * shard_size, narrow(dim, start, shard_size).
 * [NANO22] §3 (ColumnParallelLinear.weight_loader, dim 0) and §4
 * (RowParallelLinear.weight_loader, dim 1); divisibility is asserted there
 * (divide()), so a non-divisible size is an error here too. */
ORC_API int orc_shard(const void* full, int64_t rows, int64_t cols, int esize,
                      int dim, int tp_rank, int tp_size, void* out) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size) return 1;
    int64_t s = dim == 0 ? rows : cols;
    if (s % tp_size != 0) return 2;
    int64_t sh = s / tp_size;
    return orc_narrow(full, rows, cols, esize, dim, (int64_t)tp_rank * sh, sh, out);
}

/* Merged column-parallel table (gate_up): [NANO22] §5, "double cut".
 * For each projection id in order (0 = gate, 1 = up):
 *   cut 1 (which projection): segment offset = sum(sizes[:id]) / t,
 *                             segment length = sizes[id] / t  (rows of the
 *                             rank's merged table);
 *   cut 2 (which rank): the full projection weight is chunked into t equal
 *                       pieces along dim 0 and piece tp_rank is copied in.
 * gate and up are [f, h]; out is [2*f/t, h]. */
ORC_API int orc_shard_gate_up(const void* gate, const void* up, int64_t f,
                              int64_t h, int esize, int tp_rank, int tp_size,
                              void* out) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size) return 1;
    if (f % tp_size != 0) return 2;
    const void* parts[2] = {gate, up};
    int64_t sizes[2] = {f, f};
    for (int id = 0; id < 2; ++id) {
        int64_t before = 0;
        for (int p = 0; p < id; ++p) before += sizes[p];
        int64_t seg_off = before / tp_size;
        int64_t seg_len = sizes[id] / tp_size;
        int64_t chunk = sizes[id] / tp_size;
        unsigned char* dst = (unsigned char*)out + seg_off * h * esize;
        int rc = orc_narrow(parts[id], sizes[id], h, esize, 0,
                            (int64_t)tp_rank * chunk, seg_len, dst);
        if (rc) return rc;
    }
    return 0;
}

/* Which KV heads rank r holds, for n_kv KV heads at TP degree t.
 * t <= n_kv: heads [r*n_kv/t, (r+1)*n_kv/t) ([NANO22] §5: the KV heads are
 *            chunked over ranks like the Q heads).
 * t >  n_kv: one head per rank, each head replicated on t/n_kv ranks and t
 *            divisible by n_kv ([GUIDE62] §2.2).  Rank r takes head
 *            r / (t/n_kv), the head its own Q heads are grouped with: rank r
 *            holds Q heads [r*nq/t, (r+1)*nq/t) and Q head j reads KV head
 *            j / (nq/n_kv), which is r / (t/n_kv) for all of them. */
ORC_API int orc_kv_heads_for_rank(int64_t n_kv, int tp_rank, int tp_size,
                                  int64_t* first, int64_t* count) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size || n_kv < 1) return 1;
    if (tp_size <= n_kv) {
        if (n_kv % tp_size) return 2;
        *count = n_kv / tp_size;
        *first = (int64_t)tp_rank * (*count);
    } else {
        if (tp_size % n_kv) return 2;
        *count = 1;
        *first = (int64_t)tp_rank / (tp_size / n_kv);
    }
    return 0;
}

/* Merged QKV table for rank r: rows [q heads_r ; k heads_r ; v heads_r],
 * each head head_dim rows of h columns.  [NANO22] §5 (QKVParallelLinear:
 * q segment at offset 0, k after q, v after q and k; each segment filled from
 * the rank's chunk of the full projection) with the replication rule of
 * [GUIDE62] §2.2 when t exceeds the KV head count.
 * wq [nq*hd, h], wk/wv [n_kv*hd, h]; out [(nq/t + 2*kvc)*hd, h]. */
ORC_API int orc_shard_qkv(const void* wq, const void* wk, const void* wv,
                          int64_t nq, int64_t n_kv, int64_t hd, int64_t h,
                          int esize, int tp_rank, int tp_size, void* out) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size) return 1;
    if (nq % tp_size) return 2;
    int64_t kv0 = 0, kvc = 0;
    int rc = orc_kv_heads_for_rank(n_kv, tp_rank, tp_size, &kv0, &kvc);
    if (rc) return rc;
    int64_t qc = nq / tp_size;
    unsigned char* dst = (unsigned char*)out;
    rc = orc_narrow(wq, nq * hd, h, esize, 0, (int64_t)tp_rank * qc * hd, qc * hd, dst);
    if (rc) return rc;
    dst += qc * hd * h * esize;
    rc = orc_narrow(wk, n_kv * hd, h, esize, 0, kv0 * hd, kvc * hd, dst);
    if (rc) return rc;
    dst += kvc * hd * h * esize;
    return orc_narrow(wv, n_kv * hd, h, esize, 0, kv0 * hd, kvc * hd, dst);
}

/* ------------------------------------------------------------------------ */
/* Checkpoint-style loaders                                                 */
/* ------------------------------------------------------------------------ */

/* The loaders of [NANO22] §3-§5 applied to a full checkpoint tensor, in the
 * order [MINISGL] §8 (weight loading and sharding) gives: select the rank's
 * shard, convert it to the parameter's dtype, copy it into the parameter.
 * Element types: 0 = fp32, 1 = bf16 (raw 16-bit patterns).  Copying into a
 * parameter of the other type is torch's copy_: fp32 -> bf16 rounds to
 * nearest even (orc_f32_to_bf16), bf16 -> fp32 is exact (the 16 bits become
 * the top half of the fp32 encoding), equal types copy the bits. */
static void convert_one(const void* src, int src_dt, int64_t si, void* dst, int dst_dt, int64_t di) {
    if (src_dt == 0 && dst_dt == 0) {
        ((float*)dst)[di] = ((const float*)src)[si];
    } else if (src_dt == 0) {
        ((uint16_t*)dst)[di] = orc_f32_to_bf16(((const float*)src)[si]);
    } else if (dst_dt == 1) {
        ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
    } else {
        uint32_t u = (uint32_t)((const uint16_t*)src)[si] << 16;
        memcpy((float*)dst + di, &u, 4);
    }
}

/* Rows [r0, r0 + nrows) x columns [c0, c0 + ncols) of src ([*, src_cols] in
 * src_dt) converted into dst rows [d0, d0 + nrows) ([*, ncols] in dst_dt). */
static void copy_convert(const void* src, int src_dt, int64_t src_cols, int64_t r0, int64_t c0,
                         int64_t nrows, int64_t ncols, void* dst, int dst_dt, int64_t d0) {
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t j = 0; j < ncols; ++j)
            convert_one(src, src_dt, (r0 + i) * src_cols + c0 + j, dst, dst_dt, (d0 + i) * ncols + j);
}

static int valid_load_dt(int a, int b) { return (a == 0 || a == 1) && (b == 0 || b == 1); }

/* Column (dim 0, [NANO22] §3) or row (dim 1, §4) parallel loader: the
 * rank's narrow(dim, r S/t, S/t) of src [rows, cols], converted into dst
 * ([rows/t, cols] or [rows, cols/t]).  Returns 2 when t does not divide S. */
ORC_API int orc_load_shard(const void* src, int src_dt, int64_t rows, int64_t cols, int dim, int tp_rank,
                           int tp_size, void* dst, int dst_dt) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size || (dim != 0 && dim != 1)) return 1;
    if (!valid_load_dt(src_dt, dst_dt)) return 1;
    int64_t s = dim == 0 ? rows : cols;
    if (s % tp_size) return 2;
    int64_t sh = s / tp_size;
    if (dim == 0)
        copy_convert(src, src_dt, cols, (int64_t)tp_rank * sh, 0, sh, cols, dst, dst_dt, 0);
    else
        copy_convert(src, src_dt, cols, 0, (int64_t)tp_rank * sh, rows, sh, dst, dst_dt, 0);
    return 0;
}

/* [NANO22] §5, the merged column-parallel loader, one projection per call
 * (shard_id 0 = gate, 1 = up), in place on the rank's [2 f/t, h] table:
 *   cut 1: output_sizes = [f, f]; the projection's segment starts at
 *          sum(output_sizes[:shard_id]) / t and is output_sizes[shard_id] / t
 *          rows long;
 *   cut 2: src [f, h] is chunked into t pieces along dim 0 and piece
 *          tp_rank fills the segment, converted to the table's type.
 * Rows outside the segment are not touched. */
ORC_API int orc_load_gate_up(void* table, int table_dt, const void* src, int src_dt, int shard_id, int64_t f,
                             int64_t h, int tp_rank, int tp_size) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size || shard_id < 0 || shard_id > 1) return 1;
    if (!valid_load_dt(src_dt, table_dt)) return 1;
    if (f % tp_size) return 2;
    int64_t output_sizes[2] = {f, f};
    int64_t before = 0;
    for (int p = 0; p < shard_id; ++p) before += output_sizes[p];
    int64_t seg_off = before / tp_size;
    int64_t seg_len = output_sizes[shard_id] / tp_size;
    int64_t chunk = output_sizes[shard_id] / tp_size;
    copy_convert(src, src_dt, h, (int64_t)tp_rank * chunk, 0, seg_len, h, table, table_dt, seg_off);
    return 0;
}

/* [NANO22] §5, the QKV loader, one projection per call, in place on the
 * rank's [(nq/t + 2 kvc) hd, h] table (segments q, k, v in that order):
 *   shard_id 0 (q): src [nq hd, h]; the segment at row 0 takes the rank's
 *                   chunk of the heads, heads [r nq/t, (r+1) nq/t);
 *   shard_id 1 (k), 2 (v): src [n_kv hd, h]; the segment after q (k) or
 *                   after q and k (v) takes the rank's KV heads from
 *                   orc_kv_heads_for_rank (its chunk when t <= n_kv, the
 *                   replicated head r / (t/n_kv) otherwise, [GUIDE62] §2.2).
 * Rows outside the segment are not touched. */
ORC_API int orc_load_qkv(void* table, int table_dt, const void* src, int src_dt, int shard_id, int64_t nq,
                         int64_t n_kv, int64_t hd, int64_t h, int tp_rank, int tp_size) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size || shard_id < 0 || shard_id > 2) return 1;
    if (!valid_load_dt(src_dt, table_dt)) return 1;
    if (nq % tp_size) return 2;
    int64_t kv0 = 0, kvc = 0;
    int rc = orc_kv_heads_for_rank(n_kv, tp_rank, tp_size, &kv0, &kvc);
    if (rc) return rc;
    int64_t qc = nq / tp_size;
    if (shard_id == 0)
        copy_convert(src, src_dt, h, (int64_t)tp_rank * qc * hd, 0, qc * hd, h, table, table_dt, 0);
    else if (shard_id == 1)
        copy_convert(src, src_dt, h, kv0 * hd, 0, kvc * hd, h, table, table_dt, qc * hd);
    else
        copy_convert(src, src_dt, h, kv0 * hd, 0, kvc * hd, h, table, table_dt, (qc + kvc) * hd);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Vocab-parallel embedding and LM head                                     */
/* ------------------------------------------------------------------------ */

/* Rank r's contiguous vocab range: per = ceil(V/t), start = r*per,
 * end = min((r+1)*per, V).  [SCRATCH] "Implementation", class
 * VocabParallelEmbedding.  (When t divides V this is the even split of
 * [VLLM13] §2.4.1.)  A trailing rank may get an empty range (start >= V);
 * then start is clamped so that end - start is 0. */
ORC_API int orc_vocab_range(int64_t vocab, int tp_rank, int tp_size,
                            int64_t* start, int64_t* end) {
    if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size || vocab < 0) return 1;
    int64_t per = (vocab + tp_size - 1) / tp_size;
    int64_t s = (int64_t)tp_rank * per;
    int64_t e = (int64_t)(tp_rank + 1) * per;
    if (e > vocab) e = vocab;
    if (s > e) s = e;
    *start = s;
    *end = e;
    return 0;
}

/* Full (unsharded) lookup: out[i] = table[ids[i]] for 0 <= ids[i] < V, and a
 * zero row otherwise (the sum of the rank outputs for an id no rank owns).
 * Element-size generic: rows are copied bit for bit. */
ORC_API void orc_embed_full(const int64_t* ids, int64_t n, const void* table,
                            int64_t vocab, int64_t h, int esize, void* out) {
    for (int64_t i = 0; i < n; ++i) {
        unsigned char* dst = (unsigned char*)out + i * h * esize;
        if (ids[i] >= 0 && ids[i] < vocab)
            memcpy(dst, (const unsigned char*)table + ids[i] * h * esize,
                   (size_t)(h * esize));
        else
            memset(dst, 0, (size_t)(h * esize));
    }
}

/* Rank r's masked lookup.  mask = (id < start) | (id >= end); the looked-up
 * row is table_shard[id - start] where the mask is false, and the output row
 * is filled with +0.0 (all-zero bits) where it is true.  [SCRATCH]
 * "Implementation", VocabParallelEmbedding.forward (masked_fill of the ids,
 * lookup, masked_fill of the rows); [VLLM13] §2.4.1 (ids outside the rank's
 * range give zero rows).  The table row is never read for a masked id. */
ORC_API int orc_embed_rank(const int64_t* ids, int64_t n, const void* table_shard,
                           int64_t vocab, int64_t h, int esize, int tp_rank,
                           int tp_size, void* out) {
    int64_t start, end;
    int rc = orc_vocab_range(vocab, tp_rank, tp_size, &start, &end);
    if (rc) return rc;
    for (int64_t i = 0; i < n; ++i) {
        unsigned char* dst = (unsigned char*)out + i * h * esize;
        int masked = (ids[i] < start) || (ids[i] >= end);
        if (masked)
            memset(dst, 0, (size_t)(h * esize));
        else
            memcpy(dst, (const unsigned char*)table_shard + (ids[i] - start) * h * esize,
                   (size_t)(h * esize));
    }
    return 0;
}

/* Rank r's LM-head logits: logits_r = x . E_r^T with E_r the rank's
 * [V_r, h] rows of the (tied) table.  [VLLM13] §2.4.2 (Y_i = X E_i^T, the
 * full logits being the concatenation along vocab).  The table passed is
 * the FULL [V, h] table; the rank's rows are selected by orc_vocab_range. */
ORC_API int orc_lm_head_rank(const double* x, int64_t n, int64_t h,
                             const double* table, int64_t vocab, int tp_rank,
                             int tp_size, double* logits) {
    int64_t start, end;
    int rc = orc_vocab_range(vocab, tp_rank, tp_size, &start, &end);
    if (rc) return rc;
    orc_linear(x, n, h, table + start * h, end - start, NULL, logits);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Ring all-reduce: schedule and simulation                                 */
/* ------------------------------------------------------------------------ */

/* Chunk c of K elements split over t ranks: [floor(c*K/t), floor((c+1)*K/t)).
 * [VLLM13] §1.1.1 cuts the data into N chunks of about K/N elements; the exact
 * boundary for K not divisible by N is not given there, and this floor rule
 * is the reading used. */
ORC_API void orc_chunk_bounds(int64_t K, int t, int c, int64_t* lo, int64_t* hi) {
    *lo = (int64_t)(((__int128)c * K) / t);
    *hi = (int64_t)(((__int128)(c + 1) * K) / t);
}

typedef struct {
    int phase;   /* 0 = reduce-scatter (receiver adds), 1 = all-gather (receiver copies) */
    int step;    /* round within the phase, 0 .. t-2 */
    int src;     /* sending rank */
    int dst;     /* receiving rank, (src + 1) mod t */
    int chunk;   /* chunk index moved in this transfer */
    int64_t offset, len;  /* element range of that chunk */
} orc_ring_step;

/* The ring schedule of [VLLM13] §1.1.1-1.1.2: t ranks on a logical ring,
 * each sending to its right neighbour.  Reduce-scatter round s (s = 0..t-2):
 * rank r sends chunk (r - s) mod t and the receiver adds it into its own
 * copy of that chunk; after t-1 rounds rank r holds the fully reduced chunk
 * (r + 1) mod t.  All-gather round s: rank r sends chunk (r + 1 - s) mod t and
 * the receiver overwrites its copy.  Which rank starts with which chunk is
 * drawn in figures the text does not carry; the rotation above is the reading
 * used (every rank sends a different chunk in every round, as the text
 * requires).  Returns the number of steps written, 2*t*(t-1), or -1 if
 * max_steps is too small. */
ORC_API int orc_ring_schedule(int t, int64_t K, orc_ring_step* steps, int max_steps) {
    int need = 2 * t * (t - 1);
    if (need > max_steps) return -1;
    int k = 0;
    for (int phase = 0; phase < 2; ++phase) {
        for (int s = 0; s < t - 1; ++s) {
            for (int r = 0; r < t; ++r) {
                int c = phase == 0 ? ((r - s) % t + t) % t : ((r + 1 - s) % t + t) % t;
                orc_ring_step* st = &steps[k++];
                st->phase = phase;
                st->step = s;
                st->src = r;
                st->dst = (r + 1) % t;
                st->chunk = c;
                int64_t lo, hi;
                orc_chunk_bounds(K, t, c, &lo, &hi);
                st->offset = lo;
                st->len = hi - lo;
            }
        }
    }
    return k;
}

/* Simulate the ring all-reduce in fp32 on t separate rank buffers, following
 * the schedule above step by step.  Within a round all sends happen "at
 * once": each round first snapshots the chunks being sent, then applies them.
 * Only the element window [lo, hi) is simulated (every element evolves on its
 * own, so a window is exact); parts[r] points at rank r's full K-element
 * fp32 buffer.  After the all-gather every rank must hold the same values;
 * the function returns 0 and writes rank 0's window to out (hi-lo values) if
 * so, and 3 if any rank differs.  Memory: t * (hi - lo) floats. */
ORC_API int orc_ring_allreduce_f32(const float* const* parts, int t, int64_t K,
                                   int64_t lo, int64_t hi, float* out) {
    if (t < 1 || lo < 0 || hi > K || lo > hi) return 1;
    int64_t w = hi - lo;
    float* buf = (float*)malloc(sizeof(float) * (size_t)(w > 0 ? w : 1) * (size_t)t);
    float* snd = (float*)malloc(sizeof(float) * (size_t)(w > 0 ? w : 1) * (size_t)t);
    if (!buf || !snd) { free(buf); free(snd); return 4; }
    for (int r = 0; r < t; ++r) memcpy(buf + (int64_t)r * w, parts[r] + lo, sizeof(float) * (size_t)w);
    for (int phase = 0; phase < 2; ++phase) {
        for (int s = 0; s < t - 1; ++s) {
            /* every rank posts its send for this round */
            for (int r = 0; r < t; ++r) {
                int c = phase == 0 ? ((r - s) % t + t) % t : ((r + 1 - s) % t + t) % t;
                int64_t clo, chi;
                orc_chunk_bounds(K, t, c, &clo, &chi);
                for (int64_t i = lo; i < hi; ++i) {
                    if (i < clo || i >= chi) continue;
                    snd[(int64_t)r * w + (i - lo)] = buf[(int64_t)r * w + (i - lo)];
                }
            }
            /* every receiver applies what its left neighbour sent */
            for (int r = 0; r < t; ++r) {
                int c = phase == 0 ? ((r - s) % t + t) % t : ((r + 1 - s) % t + t) % t;
                int d = (r + 1) % t;
                int64_t clo, chi;
                orc_chunk_bounds(K, t, c, &clo, &chi);
                for (int64_t i = lo; i < hi; ++i) {
                    if (i < clo || i >= chi) continue;
                    float v = snd[(int64_t)r * w + (i - lo)];
                    float* dv = &buf[(int64_t)d * w + (i - lo)];
                    if (phase == 0)
                        *dv = *dv + v;   /* reduce-scatter: add into own copy */
                    else
                        *dv = v;         /* all-gather: overwrite */
                }
            }
        }
    }
    int rc = 0;
    for (int r = 1; r < t && !rc; ++r)
        if (memcmp(buf, buf + (int64_t)r * w, sizeof(float) * (size_t)w) != 0) rc = 3;
    memcpy(out, buf, sizeof(float) * (size_t)w);
    free(buf);
    free(snd);
    return rc;
}

/* Exact-as-possible reference sum of the t partials in fp64. */
ORC_API void orc_reduce_sum_f64(const double* const* parts, int t, int64_t K, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K; ++i) {
        double s = 0.0;
        for (int r = 0; r < t; ++r) s += parts[r][i];
        out[i] = s;
    }
}

/* Head-parallel attention core of one rank ([VLLM13] §2.3.3: each rank runs
 * self-attention on its own heads, scores = q k^T / sqrt(head_dim), a
 * max-subtracted softmax along the keys, then probs . v; [SCRATCH]
 * TPAttention.forward: the rank's nq query heads share its nkv KV heads by
 * repeat_interleave, so query head j reads KV head j / (nq / nkv), under the
 * causal mask tril(ones(T, S)) when causal).  RoPE and the q/k norms come
 * before this step and are not part of it.
 *   qkv: [n, (nq + 2 nkv) d] fp64, the rank's QKV projection output (q heads,
 *   then k heads, then v heads, d columns each); rows: the query rows to
 *   compute (every step is independent per query row); out: [n_rows, nq d].
 * Returns 0, or 1 for bad arguments, 4 if out of memory. */
ORC_API int orc_attention_rank(const double* qkv, int64_t n, int nq, int nkv, int d, int causal,
                               const int64_t* rows, int64_t n_rows, double* out) {
    if (n < 1 || nq < 1 || nkv < 1 || nq % nkv != 0 || d < 1) return 1;
    const int64_t ld = (int64_t)(nq + 2 * nkv) * d;
    const int rep = nq / nkv;
    const double scale = 1.0 / sqrt((double)d);
    int rc = 0;
#pragma omp parallel
    {
        double* sc = (double*)malloc(sizeof(double) * (size_t)n);
        if (!sc) {
#pragma omp atomic write
            rc = 4;
        } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
            for (int64_t ri = 0; ri < n_rows; ++ri) {
                for (int h = 0; h < nq; ++h) {
                    const int64_t i = rows[ri];
                    const int g = h / rep;
                    const double* q = qkv + i * ld + (int64_t)h * d;
                    const int64_t S = causal ? i + 1 : n;     /* keys 0 .. S-1 */
                    double mx = -INFINITY;
                    for (int64_t s = 0; s < S; ++s) {
                        const double* k = qkv + s * ld + (int64_t)(nq + g) * d;
                        double dot = 0.0;
                        for (int e = 0; e < d; ++e) dot += q[e] * k[e];
                        sc[s] = dot * scale;
                        if (sc[s] > mx) mx = sc[s];
                    }
                    double sum = 0.0;
                    for (int64_t s = 0; s < S; ++s) {
                        sc[s] = exp(sc[s] - mx);
                        sum += sc[s];
                    }
                    double* o = out + ri * (int64_t)nq * d + (int64_t)h * d;
                    for (int e = 0; e < d; ++e) o[e] = 0.0;
                    for (int64_t s = 0; s < S; ++s) {
                        const double* v = qkv + s * ld + (int64_t)(nq + nkv + g) * d;
                        const double p = sc[s] / sum;
                        for (int e = 0; e < d; ++e) o[e] += p * v[e];
                    }
                }
            }
            free(sc);
        }
    }
    return rc;
}

/* One-shot all-reduce: every rank reads all ranks' buffers and adds them,
 * in rank order, into an accumulator that starts at zero ([VLLM13] §1.2,
 * the low-latency all-reduce pseudocode: out = zeros_like(x), then
 * out += load_from(buf) for each peer buffer; [GUIDE62] §6.3: each GPU
 * reads the others' buffers and sums).  fp32 adds:
 * out[i] = ((0 + P_0[i]) + P_1[i]) + ... + P_{t-1}[i].  Every rank computes
 * the same sum, so one result stands for all of them. */
ORC_API void orc_reduce_rank_f32(const float* const* parts, int t, int64_t K, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K; ++i) {
        float acc = 0.0f;
        for (int r = 0; r < t; ++r) acc = acc + parts[r][i];
        out[i] = acc;
    }
}

/* Full logits from the vocab-parallel LM head and the greedy next token.
 * [SCRATCH] TPTransformer.forward all-gathers every rank's logits,
 * concatenates them along the vocabulary and truncates to the vocabulary
 * size; its generation loop then takes argmax of the logits ([VLLM13] §2.4.2:
 * Y = gather([Y_1, Y_2])).  Shard r holds columns [start_r, end_r) of
 * orc_vocab_range without padding, so concatenating the shards gives the
 * truncated result directly.  argmax: the first index of the maximum, a NaN
 * counting as larger than every number (the rule of the torch.argmax the
 * demo calls).  shards[r]: n x (end_r - start_r) values; full (may be NULL):
 * n x vocab; argmax: n.  Returns 0, or 1 for bad arguments. */
ORC_API int orc_logits_gather_argmax(const double* const* shards, int t, int64_t n, int64_t vocab,
                                     double* full, int64_t* argmax) {
    if (t < 1 || n < 0 || vocab < 1) return 1;
    for (int64_t i = 0; i < n; ++i) {
        double best = 0.0;
        int64_t bi = -1;
        int nan_seen = 0;
        for (int r = 0; r < t; ++r) {
            int64_t start, end;
            if (orc_vocab_range(vocab, r, t, &start, &end)) return 1;
            const int64_t w = end - start;
            for (int64_t j = 0; j < w; ++j) {
                const double v = shards[r][i * w + j];
                const int64_t col = start + j;
                if (full) full[i * vocab + col] = v;
                if (nan_seen) continue;
                if (v != v) {
                    nan_seen = 1;
                    bi = col;
                } else if (bi < 0 || v > best) {
                    best = v;
                    bi = col;
                }
            }
        }
        argmax[i] = bi;
    }
    return 0;
}

/* Token-row chunk c of the sequence-parallel split: rows [floor(c n/t),
 * floor((c+1) n/t)).  [SCRATCH] Exercises, item 1 (sequence parallelism):
 * after the reduce-scatter every rank holds the complete result for 1/t of
 * the tokens.  The split is along tokens (whole rows); the floor rule for n
 * not divisible by t is the same reading as orc_chunk_bounds. */
ORC_API void orc_sp_rows(int64_t n, int t, int c, int64_t* lo, int64_t* hi) {
    *lo = (int64_t)(((__int128)c * n) / t);
    *hi = (int64_t)(((__int128)(c + 1) * n) / t);
}

/* Sequence-parallel epilogue of a row-parallel layer for rank `rank`
 * ([SCRATCH] Exercises, item 1: split the all-reduce into a reduce-scatter
 * and an all-gather; each rank does the residual add and RMSNorm only on
 * the tokens it holds).  Steps, in that order:
 *   1. the reduce-scatter half of the ring of [VLLM13] §1.1.1 (the same
 *      rounds as orc_ring_schedule's phase 0), simulated in fp32 on t
 *      separate rank buffers, with the chunks being token-row ranges
 *      (orc_sp_rows).  Afterwards rank r holds the complete chunk
 *      c = (r + 1) mod t; only that chunk's rows are simulated (rows evolve
 *      independently, so this is exact);
 *   2. the residual add, one fp32 add per element: v = s + residual, then
 *      one rounding to bf16 (RNE) if round_bf16 -- the new residual stream,
 *      written to residual_out (fp32 values);
 *   3. RMSNorm of each row of the rounded values, in fp64:
 *      y_j = v_j / sqrt(mean_k v_k^2 + eps) * w_j.  The pages use RMSNorm
 *      (fused with the all-reduce in serving engines, [SCRATCH] conclusions
 *      list) but do not write it out; this is its usual definition, with eps
 *      an argument.
 * parts[r]: rank r's partial, n*h fp32 values; residual and residual_out:
 * the chunk's rows, (hi-lo)*h; weight: h; out: (hi-lo)*h fp64.
 * Returns 0, or 1 for bad arguments, 4 if out of memory. */
ORC_API int orc_rs_add_rmsnorm(const float* const* parts, int t, int rank, int64_t n, int64_t h,
                               const float* residual, const double* weight, double eps,
                               int round_bf16, float* residual_out, double* out) {
    if (t < 1 || rank < 0 || rank >= t || n < 0 || h < 1) return 1;
    const int c = (rank + 1) % t;
    int64_t lo, hi;
    orc_sp_rows(n, t, c, &lo, &hi);
    const int64_t w = (hi - lo) * h;            /* elements of the owned chunk */
    float* buf = (float*)malloc(sizeof(float) * (size_t)(w > 0 ? w : 1) * (size_t)t);
    float* snd = (float*)malloc(sizeof(float) * (size_t)(w > 0 ? w : 1) * (size_t)t);
    if (!buf || !snd) { free(buf); free(snd); return 4; }
    for (int r = 0; r < t; ++r) memcpy(buf + (int64_t)r * w, parts[r] + lo * h, sizeof(float) * (size_t)w);
    /* reduce-scatter rounds s = 0..t-2: rank q sends chunk (q - s) mod t to
     * q + 1, which adds it to its own copy; only transfers of chunk c touch
     * the simulated rows */
    for (int s = 0; s < t - 1; ++s) {
        for (int q = 0; q < t; ++q)
            if (((q - s) % t + t) % t == c) memcpy(snd + (int64_t)q * w, buf + (int64_t)q * w, sizeof(float) * (size_t)w);
        for (int q = 0; q < t; ++q) {
            if (((q - s) % t + t) % t != c) continue;
            const int d = (q + 1) % t;
            for (int64_t i = 0; i < w; ++i) buf[(int64_t)d * w + i] = buf[(int64_t)d * w + i] + snd[(int64_t)q * w + i];
        }
    }
    const float* red = buf + (int64_t)rank * w;   /* what rank `rank` holds now */
    for (int64_t i = 0; i < w; ++i) {
        float v = red[i] + residual[i];
        if (round_bf16) v = orc_bf16_to_f32(orc_f32_to_bf16(v));
        residual_out[i] = v;
    }
    for (int64_t r = 0; r < hi - lo; ++r) {
        const float* v = residual_out + r * h;
        double ss = 0.0;
        for (int64_t j = 0; j < h; ++j) ss += (double)v[j] * (double)v[j];
        const double rms = sqrt(ss / (double)h + eps);
        for (int64_t j = 0; j < h; ++j) out[r * h + j] = (double)v[j] / rms * weight[j];
    }
    free(buf);
    free(snd);
    return 0;
}

/* Per-rank traffic of the ring all-reduce: every rank sends (and receives)
 * one chunk per round for t-1 reduce-scatter and t-1 all-gather rounds, so
 * 2(t-1) rounds and, for t dividing K, 2(t-1)*K/t elements.  [VLLM13] §1.2.
 * Computed here by walking the schedule, not from the closed form. */
ORC_API int orc_ring_traffic(int t, int64_t K, int64_t* sent_per_rank,
                             int64_t* recv_per_rank, int* rounds) {
    int max = 2 * t * (t - 1) + 1;
    orc_ring_step* st = (orc_ring_step*)malloc(sizeof(orc_ring_step) * (size_t)max);
    if (!st) return 4;
    int ns = orc_ring_schedule(t, K, st, max);
    if (ns < 0) { free(st); return 1; }
    for (int r = 0; r < t; ++r) { sent_per_rank[r] = 0; recv_per_rank[r] = 0; }
    int maxround = -1;
    for (int k = 0; k < ns; ++k) {
        sent_per_rank[st[k].src] += st[k].len;
        recv_per_rank[st[k].dst] += st[k].len;
        int rr = st[k].phase * (t - 1) + st[k].step;
        if (rr > maxround) maxround = rr;
    }
    *rounds = maxround + 1;
    free(st);
    return 0;
}
