/*
 * tpshard.h -- C ABI of libtpshard: one tensor-parallel (TP) rank's share of a
 * Transformer layer on one AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles shortened):
 *   [VLLM13]  "vLLM source analysis 13 -- vLLM distributed inference: tensor
 *             parallelism in detail"
 *   [NANO22]  "Nano-vLLM source walkthrough no. 22 -- tensor parallelism (2):
 *             code"
 *   [SCRATCH] "Tensor parallelism: implemented from scratch" (AI-infra
 *             handbook)
 *   [GUIDE62] "AIInfraGuide 6.2 -- tensor-parallel inference"
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless the comment says HOST.  The caller
 *     owns every buffer; the library keeps no pointer after a call returns and
 *     allocates no device memory (scratch space comes in through `workspace`;
 *     tp_mlp_rank_forward_noalloc uses a fixed array in the library image
 *     instead, TP_NOALLOC_SCRATCH_BYTES per GPU).
 *   - Compute calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream).  They never synchronize the device.
 *   - Tensors are dense and row-major.  A linear layer's weight is stored
 *     [out, in] and the layer computes y = x . W^T ([NANO22] §2), so both GEMM
 *     operands are contiguous along the reduction dimension.
 *   - Element types: TP_BF16 (bfloat16 bits) and TP_F32.  Supported
 *     (input, output) pairs: F32 -> F32, BF16 -> BF16, BF16 -> F32.  Products
 *     accumulate in fp32; an output is rounded once (round-to-nearest-even).
 *   - Errors: every argument is validated on the host before anything is
 *     launched.  A failing call returns a non-zero tp_status, launches
 *     nothing (TP_EHIP excepted: the launch itself failed), and leaves a
 *     message in tp_last_error() (per thread).  Nothing aborts or prints.
 *     Divisibility is an error, as the pages' divide() assertion makes it.
 *   - Alignment: 16-byte aligned pointers and reduction sizes that are a
 *     multiple of 8 (bf16) take the vector path; anything else takes a
 *     slower element-wise path with identical results.  Workspaces and
 *     staging buffers must be aligned as each entry point states
 *     (TP_EALIGN otherwise).
 *   - bf16 GEMM sizes: the kernels address operand tiles with 32-bit byte
 *     offsets, so the reduction size K must satisfy 256 K 2 < 2^31
 *     (K < 4194304), and a fused gate_up table must have its up rows within
 *     2 GiB of its gate rows: (f_local + 256) K 2 < 2^31.  Larger shapes
 *     return TP_ESHAPE.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef TP_API
#define TP_API __attribute__((visibility("default")))
#endif

#define TP_ABI_VERSION 1
#define TP_MAX_RANKS 64
/* Device scratch of tp_mlp_rank_forward_noalloc, held by each GPU the
 * library runs on until the process ends. */
#define TP_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum {
    TP_OK = 0,
    TP_EINVAL = 1,      /* bad argument: null pointer, rank outside [0, t), t outside [1, 64], n <= 0 ... */
    TP_ESHAPE = 2,      /* sizes that do not divide, or buffers whose sizes do not match */
    TP_EDTYPE = 3,      /* unsupported element type or (input, output) pair */
    TP_EALIGN = 4,      /* a buffer that must be aligned is not: workspaces (16 bytes; 256 for
                           tp_mlp_rank_forward), loader staging, attention qkv/out (16 bytes) */
    TP_EHIP = 5,        /* the HIP runtime reported an error on launch */
    TP_EWORKSPACE = 6   /* workspace missing or smaller than the matching *_workspace_bytes query */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Summation order of tp_partial_reduce. */
typedef enum {
    TP_ORDER_RING = 0,  /* ring reduce-scatter chunk order (see tp_partial_reduce) */
    TP_ORDER_RANK = 1   /* one-shot order: ((0 + P_0) + P_1) + ... for every element */
} tp_order;

/* One transfer of the ring all-reduce schedule (tp_ring_schedule). */
typedef struct {
    int phase;          /* 0 = reduce-scatter (receiver adds), 1 = all-gather (receiver overwrites) */
    int step;           /* round within the phase, 0 .. t-2 */
    int src;            /* sending rank */
    int dst;            /* receiving rank = (src + 1) mod t */
    int chunk;          /* chunk moved */
    int64_t offset;     /* first element of the chunk */
    int64_t len;        /* elements in the chunk */
} tp_ring_step;

/* ---- library ------------------------------------------------------------ */

TP_API int tp_abi_version(void);                 /* TP_ABI_VERSION */
TP_API const char* tp_last_error(void);          /* last error of this thread; "" after success; static storage */
TP_API const char* tp_status_string(int status); /* "TP_OK", "TP_EINVAL", ... */

/* ---- shard selection (load time) --------------------------------------- */

/* out = full.narrow(dim, tp_rank * S/t, S/t) as a contiguous tensor, S =
 * full.size(dim).  [NANO22] §3 (ColumnParallelLinear weight loader: dim 0,
 * whole output rows) and §4 (RowParallelLinear: dim 1, input columns).
 *   full [rows, cols]; out [rows/t, cols] (dim 0) or [rows, cols/t] (dim 1).
 * TP_ESHAPE if t does not divide S; bit-exact copy. */
TP_API tp_status tp_shard_weights(const void* full, int64_t rows, int64_t cols, tp_dtype dt,
                           int dim, int tp_rank, int tp_size, void* out, void* stream);

/* Fused gate_up table of rank r: rows [0, f/t) = gate rows [r f/t, (r+1) f/t),
 * rows [f/t, 2f/t) = the same rows of up.  [NANO22] §5 (merged column-parallel
 * "double cut": the projection picks the segment, the rank picks its chunk
 * of that projection).  gate, up [f, h]; out [2 f/t, h].  TP_ESHAPE if t does
 * not divide f. */
TP_API tp_status tp_shard_gate_up(const void* gate, const void* up, int64_t f, int64_t h,
                           tp_dtype dt, int tp_rank, int tp_size, void* out, void* stream);

/* HOST-only.  KV heads held by rank r: for t <= n_kv, heads
 * [r n_kv/t, (r+1) n_kv/t); for t > n_kv one head, r / (t/n_kv), each head
 * being replicated on t/n_kv ranks ([GUIDE62] §2.2).  TP_ESHAPE if neither
 * count divides the other. */
TP_API tp_status tp_kv_heads_for_rank(int64_t n_kv, int tp_rank, int tp_size,
                               int64_t* first /*HOST*/, int64_t* count /*HOST*/);

/* Merged QKV table of rank r: [q heads ; k heads ; v heads], head_dim rows per
 * head.  [NANO22] §5 (QKVParallelLinear segments q, k, v) with the GQA
 * replication of tp_kv_heads_for_rank.  wq [n_q*hd, h], wk/wv [n_kv*hd, h];
 * out [(n_q/t + 2*kv_count)*hd, h].  TP_ESHAPE if t does not divide n_q. */
TP_API tp_status tp_shard_qkv(const void* wq, const void* wk, const void* wv,
                       int64_t n_q, int64_t n_kv, int64_t head_dim, int64_t h,
                       tp_dtype dt, int tp_rank, int tp_size, void* out, void* stream);

/* ---- checkpoint-style loaders (load time) -------------------------------- */

/* The weight loaders of [NANO22] §3-§5 straight from a checkpoint tensor in
 * HOST memory, in the order [MINISGL] §8 (weight loading and sharding) gives
 * to keep device memory at the shard's size: select the rank's shard, convert
 * the dtype, copy it into the local parameter.  Only the shard crosses the
 * host link (one strided 2-D copy on `stream`); the conversion runs on the
 * GPU: fp32 -> bf16 rounds to nearest even (a NaN stays a NaN), bf16 -> fp32
 * is exact, equal dtypes copy the bits.
 *   src: HOST pointer (pageable or pinned) to the full tensor, row-major,
 *        in src_dt; it must stay valid and unchanged until the stream has
 *        passed the call (pageable sources are copied before the call
 *        returns; a dim-1 cut (row-parallel: a segment of every row) of
 *        pageable memory is gathered on the host in 16 MiB blocks and
 *        synchronises the stream).
 *   dst: DEVICE table in dst_dt; staging: DEVICE buffer, 16-byte aligned, of
 *        at least tp_load_staging_bytes(chunk rows, chunk cols, src_dt,
 *        dst_dt) bytes (0 bytes, NULL allowed, when the dtypes match); it
 *        must not be reused until the stream has passed the call.
 *   src_dt, dst_dt: TP_F32 or TP_BF16.
 * Errors as for the shard selection above; TP_EWORKSPACE for a short
 * staging buffer.  Bit-exact to the rule above. */
TP_API tp_status tp_load_staging_bytes(int64_t rows, int64_t cols, tp_dtype src_dt, tp_dtype dst_dt,
                                       size_t* bytes /*HOST*/);

/* Column (dim 0) or row (dim 1) parallel loader ([NANO22] §3, §4):
 * dst = src.narrow(dim, tp_rank S/t, S/t) in dst_dt.  src [rows, cols];
 * dst [rows/t, cols] (dim 0) or [rows, cols/t] (dim 1); chunk = dst's shape. */
TP_API tp_status tp_load_shard(const void* src /*HOST*/, tp_dtype src_dt, int64_t rows, int64_t cols, int dim,
                               int tp_rank, int tp_size, void* dst, tp_dtype dst_dt, void* staging,
                               size_t staging_bytes, void* stream);

/* One projection of the fused gate_up table ([NANO22] §5, the merged
 * column-parallel loader): shard_id 0 = gate, 1 = up.  The projection's
 * segment of the rank's table is rows [shard_id f/t, (shard_id+1) f/t) (the
 * first cut) and it receives rows [tp_rank f/t, (tp_rank+1) f/t) of src
 * (the second cut, chunk(t)[tp_rank]).  src [f, h]; dst the rank's
 * [2 f/t, h] table (other rows untouched); chunk [f/t, h].  Loading both
 * projections gives tp_shard_gate_up's table. */
TP_API tp_status tp_load_gate_up(const void* src /*HOST*/, tp_dtype src_dt, int shard_id, int64_t f, int64_t h,
                                 int tp_rank, int tp_size, void* dst, tp_dtype dst_dt, void* staging,
                                 size_t staging_bytes, void* stream);

/* One projection of the merged QKV table ([NANO22] §5, the QKV loader, with
 * the GQA replication of tp_kv_heads_for_rank): shard_id 0 = q (src
 * [n_q hd, h]; segment rows [0, n_q/t hd) <- heads [r n_q/t, (r+1) n_q/t)),
 * 1 = k and 2 = v (src [n_kv hd, h]; segments after q, then after k, each
 * kv_count hd rows <- the rank's KV heads).  dst the rank's
 * [(n_q/t + 2 kv_count) hd, h] table (other rows untouched); chunk = the
 * segment.  Loading q, k and v gives tp_shard_qkv's table. */
TP_API tp_status tp_load_qkv(const void* src /*HOST*/, tp_dtype src_dt, int shard_id, int64_t n_q, int64_t n_kv,
                             int64_t head_dim, int64_t h, int tp_rank, int tp_size, void* dst, tp_dtype dst_dt,
                             void* staging, size_t staging_bytes, void* stream);

/* ---- column-parallel gate_up with the local SiLU(gate)*up ---------------- */

/* act = SiLU(x . G^T) * (x . U^T), G = w_gate_up rows [0, f_local),
 * U = rows [f_local, 2 f_local).  [SCRATCH] "Implementation" (class TPMLP:
 * gate/up column-parallel, SiLU(gate)*up local); [GUIDE62] §1 (the activation
 * is element-wise, so it needs no communication).  Fused: gate and up
 * products are never written; act is rounded once to dt.
 *   x [n, h] dt; w_gate_up [2 f_local, h] dt; act [n, f_local] dt.
 * workspace: at least tp_gate_up_workspace_bytes(...) bytes, 16-byte
 * aligned (NULL allowed when the query returns 0). */
TP_API tp_status tp_gate_up_workspace_bytes(int64_t n, int64_t h, int64_t f_local, tp_dtype dt,
                                     size_t* bytes /*HOST*/);
TP_API tp_status tp_gate_up_act_rank(const void* x, int64_t n, int64_t h, const void* w_gate_up,
                              int64_t f_local, tp_dtype dt, void* act,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- generic rank linear (row-parallel down / o_proj, column-parallel QKV) */

/* y = x . w^T (+ bias).  Row-parallel layers pass the bias on rank 0 only, so
 * that the sum over ranks adds it once ([NANO22] §4).
 *   x [n, k] dt; w [m, k] dt; bias [m] dt or NULL; y [n, m] out_dt.
 * workspace: at least tp_linear_workspace_bytes(...) bytes, 16-byte
 * aligned (NULL allowed when the query returns 0). */
TP_API tp_status tp_linear_workspace_bytes(int64_t n, int64_t k, int64_t m, tp_dtype dt,
                                    size_t* bytes /*HOST*/);
TP_API tp_status tp_linear_rank_forward(const void* x, int64_t n, int64_t k, const void* w,
                                 int64_t m, const void* bias, tp_dtype dt, void* y,
                                 tp_dtype out_dt, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---- the rank's MLP share ------------------------------------------------ */

/* partial = (SiLU(x . G_r^T) * (x . U_r^T)) . D_r^T, the full-shape [n, h]
 * partial sum of rank r ([GUIDE62] §1: Y = sum_i act(X A_i) B_i; [SCRATCH]
 * TPMLP.forward).  Two launches: tp_gate_up_act_rank into the workspace,
 * then tp_linear_rank_forward with the down shard.  No bias.
 *   x [n, h] dt; w_gate_up [2 f_local, h] dt (gate rows first, as made by
 *   tp_shard_gate_up); w_down [h, f_local] dt (tp_shard_weights dim 1);
 *   partial [n, h] out_dt.  The activation is held in dt (bf16 for bf16).
 * workspace: at least tp_mlp_workspace_bytes(...) bytes, 256-byte aligned. */
TP_API tp_status tp_mlp_workspace_bytes(int64_t n, int64_t h, int64_t f_local, tp_dtype dt,
                                 size_t* bytes /*HOST*/);
TP_API tp_status tp_mlp_rank_forward(const void* x, int64_t n, int64_t h, const void* w_gate_up,
                              const void* w_down, int64_t f_local, tp_dtype dt,
                              void* partial, tp_dtype out_dt,
                              void* workspace, size_t workspace_bytes, void* stream);

/* tp_mlp_rank_forward for callers that cannot allocate device memory: code
 * under HIP stream capture, serving loops and harnesses that forbid
 * allocation.  Same arguments, kernels and results as tp_mlp_rank_forward,
 * without the workspace: the activation and split-K partials live in a
 * library-owned device array of TP_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU,
 * so the call allocates nothing.
 *   Limit: shapes whose tp_mlp_workspace_bytes exceeds 64 MiB return
 *   TP_EWORKSPACE (for example the Llama-3.1-70B decode share, 64 tokens at
 *   TP=4, needs about 16 MB; its 8192-token prefill share at TP=8 needs
 *   about 123 MB and must use tp_mlp_rank_forward).
 *   Every call on one GPU uses that GPU's single array: calls that overlap
 *   in time on one GPU (other streams, other host threads) race and must be
 *   serialised by the caller.  Nothing in the array needs clearing between
 *   calls: each call writes every byte it reads.
 *   The stream must belong to the current device. */
TP_API tp_status tp_mlp_rank_forward_noalloc(const void* x, int64_t n, int64_t h, const void* w_gate_up,
                                             const void* w_down, int64_t f_local, tp_dtype dt,
                                             void* partial, tp_dtype out_dt, void* stream);

/* ---- sum of the t partials (the all-reduce's arithmetic, one device) ----- */

/* out = sum_r partials[r], element-wise over K elements, in fp32, rounded
 * once to out_dt.  Deterministic and bit-reproducible; no atomics.
 *   order TP_ORDER_RING: the order a ring reduce-scatter adds them
 *     ([VLLM13] §1.1.1): the K elements are cut into t chunks
 *     [floor(c K/t), floor((c+1) K/t)); chunk c is accumulated as
 *     ((P_c + P_{c+1}) + P_{c+2}) + ... + P_{c+t-1} (indices mod t).
 *   order TP_ORDER_RANK: the one-shot all-reduce, where every rank reads all
 *     buffers and adds them into a zero accumulator ([VLLM13] §1.2, the
 *     low-latency all-reduce; [GUIDE62] §6.3): ((0 + P_0) + P_1) + ... +
 *     P_{t-1} for every element (a sum of negative zeros is +0).
 *   partials: HOST array of t device pointers, each [K] in_dt; out [K] out_dt
 *   (may alias partials[c] only if t == 1).  1 <= t <= TP_MAX_RANKS. */
TP_API tp_status tp_partial_reduce(const void* const* partials /*HOST array*/, int t, int64_t K,
                            tp_dtype in_dt, void* out, tp_dtype out_dt, tp_order order,
                            void* stream);

/* HOST-only.  The ring all-reduce schedule that order follows: reduce-scatter
 * round s, rank r sends chunk (r - s) mod t to (r+1) mod t, which adds it;
 * all-gather round s, rank r sends chunk (r + 1 - s) mod t, which the
 * receiver copies.  2 t (t-1) steps; each rank sends 2(t-1) K/t elements in
 * 2(t-1) rounds ([VLLM13] §1.2).  steps: HOST array of max_steps entries. */
TP_API tp_status tp_ring_schedule(int t, int64_t K, tp_ring_step* steps /*HOST*/, int max_steps,
                           int* n_steps /*HOST*/);

/* The full logits and the greedy next token from the t vocab-parallel LM-head
 * shards (the gather that follows tp_lm_head_rank).  [SCRATCH]
 * TPTransformer.forward all-gathers the ranks' logits, concatenates them
 * along the vocabulary and truncates to `vocab`; its generation loop takes
 * argmax ([VLLM13] §2.4.2: Y = gather([Y_1, Y_2])).  Shard r holds columns
 * [start_r, end_r) of tp_vocab_range without padding, so
 *   full[i, start_r + j] = shards[r][i, j]                 (bit-exact copy)
 *   argmax[i] = first column of the maximum of full[i, :], a NaN counting
 *               as larger than every number (torch.argmax's rule).
 *   shards: HOST array of t device pointers, shard r [n, end_r - start_r]
 *   fp32 (an empty trailing shard may be null); full [n, vocab] fp32 or
 *   NULL; argmax [n] int64 (device) or NULL; at least one of the two.
 *   dt must be TP_F32.  Deterministic. */
TP_API tp_status tp_logits_gather_argmax(const void* const* shards /*HOST array*/, int t, int64_t n, int64_t vocab,
                                         tp_dtype dt, void* full, int64_t* argmax, void* stream);

/* ---- sequence-parallel epilogue (reduce-scatter + residual add + RMSNorm) */

/* HOST-only.  Token rows [lo, hi) that rank tp_rank holds after the ring
 * reduce-scatter: chunk c = (tp_rank + 1) mod t, lo = floor(c n / t),
 * hi = floor((c + 1) n / t).  [SCRATCH] Exercises, item 1 (sequence
 * parallelism: the reduce-scatter leaves each rank the complete rows of 1/t
 * of the tokens); the ring and its final owner as in tp_ring_schedule. */
TP_API tp_status tp_sp_rows(int64_t n, int tp_rank, int tp_size, int64_t* lo /*HOST*/, int64_t* hi /*HOST*/);

/* Rank tp_rank's share of the row-parallel layer's epilogue in sequence-
 * parallel form ([SCRATCH] Exercises, item 1: reduce-scatter, then the
 * residual add and RMSNorm on the rank's own tokens only; all-gather comes
 * after).  For each row i in [lo, hi) of tp_sp_rows:
 *   s   = ((P_c[i] + P_{c+1}[i]) + ...) + P_{c+t-1}[i]      fp32, ring order
 *   v   = round(s + residual[i - lo])                       one fp32 add, one
 *                                                           rounding to dt
 *   out = round(v / sqrt(mean_j v_j^2 + eps) * weight)      fp32
 * The pages name RMSNorm without writing it out; this is its usual form, and
 * eps is the caller's (1e-5 in the Llama configurations).
 *   partials: HOST array of t device pointers, each [n, h] dt (the ranks'
 *             row-parallel partials); residual, residual_out, out:
 *             [hi - lo, h] dt (the rank's rows only); weight: [h] dt.
 *   residual_out may be residual (in-place update); out must not alias
 *   the partials or residual.  dt: TP_BF16 or TP_F32.  1 <= t <= TP_MAX_RANKS,
 *   0 <= tp_rank < t, n >= 0, h >= 1, eps >= 0.  A rank with no rows
 *   (n < t) launches nothing, and its row buffers may then be null.
 *   Deterministic (fixed reduction order). */
TP_API tp_status tp_rs_add_rmsnorm(const void* const* partials /*HOST array*/, int t, int tp_rank, int64_t n,
                                   int64_t h, tp_dtype dt, const void* residual, const void* weight, float eps,
                                   void* residual_out, void* out, void* stream);

/* ---- head-parallel attention core ----------------------------------------- */

/* The rank's share of self-attention, between its QKV projection and its
 * o_proj ([VLLM13] §2.3.3: each rank runs attention on its own heads with no
 * communication; [SCRATCH] TPAttention.forward: the rank's query heads share
 * its KV heads by repeat_interleave, under a causal mask):
 *   out[i, h] = sum_s softmax_s(q[i,h] . k[s,g] / sqrt(d)) v[s,g],
 *   g = h / (nq / nkv), keys s <= i when causal, all n keys otherwise.
 * RoPE and the q/k norms come before this step.  fp32 softmax and
 * accumulation; the probabilities are rounded to bf16 for the product with
 * v; out is rounded once to bf16.
 *   qkv [n, (nq + 2 nkv) head_dim] bf16: the QKV projection output of the
 *   rank (q heads, then k heads, then v heads), 16-byte aligned;
 *   out [n, nq head_dim] bf16, 16-byte aligned, must not overlap qkv.
 *   head_dim must be 128; nkv divides nq; dt must be TP_BF16; qkv under
 *   2 GiB.
 * workspace: at least tp_attention_workspace_bytes(...) bytes, 16-byte
 *   aligned.  The work is cut into about 256 equal pieces (pairs of a
 *   light and a heavy 64-query tile, each pair's key blocks in equal
 *   chunks); a tile spread over several pieces leaves fp32 partial results
 *   there, merged by a second launch.  Zero bytes (NULL allowed) for short
 *   sequences, where every piece holds whole tiles. */
TP_API tp_status tp_attention_workspace_bytes(int64_t n, int nq, int nkv, int head_dim, tp_dtype dt, int causal,
                                              size_t* bytes /*HOST*/);
TP_API tp_status tp_attention_rank(const void* qkv, int64_t n, int nq, int nkv, int head_dim, tp_dtype dt,
                                   int causal, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---- vocab-parallel embedding and LM head -------------------------------- */

/* HOST-only.  Rank r's vocab range: per = ceil(V/t), start = r per,
 * end = min((r+1) per, V) ([SCRATCH] class VocabParallelEmbedding); a
 * trailing rank may get an empty range. */
TP_API tp_status tp_vocab_range(int64_t vocab, int tp_rank, int tp_size,
                         int64_t* start /*HOST*/, int64_t* end /*HOST*/);

/* out[i, :] = table_shard[ids[i] - start, :] if start <= ids[i] < end, else
 * +0.0 (the table is not read for such rows).  [VLLM13] §2.4.1; [SCRATCH]
 * VocabParallelEmbedding.forward.  Summing the t ranks' outputs (for example
 * with tp_partial_reduce) gives the full lookup.  Ids outside [0, V) are not
 * an error: every rank writes a zero row for them.
 *   ids [n] int64; table_shard [end - start, h] dt; out [n, h] dt. */
TP_API tp_status tp_vocab_embed_rank(const int64_t* ids, int64_t n, const void* table_shard,
                              int64_t vocab, int64_t h, int tp_rank, int tp_size,
                              tp_dtype dt, void* out, void* stream);

/* logits_r = x . T_r^T, the rank's slice of the logits along vocab
 * ([VLLM13] §2.4.2: Y_i = X E_i^T; the full logits are the concatenation).
 *   x [n, h] dt; table_shard [v_local, h] dt; logits [n, v_local] out_dt.
 * workspace: at least tp_linear_workspace_bytes(n, h, v_local, dt) bytes,
 * 16-byte aligned (NULL allowed when that is 0). */
TP_API tp_status tp_lm_head_rank(const void* x, int64_t n, int64_t h, const void* table_shard,
                          int64_t v_local, tp_dtype dt, void* logits, tp_dtype out_dt,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
