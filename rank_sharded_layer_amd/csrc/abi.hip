// C entry points of libtpshard: argument validation, workspace layout and
// kernel launches.  Every check happens on the host before anything is
// launched; a failing check returns a status and leaves a message in a
// per-thread buffer.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.hpp"

// Scratch of tp_mlp_rank_forward_noalloc: device memory the library owns, so
// that callers which cannot allocate (code under stream capture, serving
// loops that forbid allocation) can run the MLP share.  Each GPU the library
// runs on holds its own copy of this array until the process ends.  In host
// code this name is only a stand-in for the device symbol: kernels get the
// address hipGetSymbolAddress returns for the current device.
static __device__ __attribute__((aligned(256))) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

tp_status fail(tp_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

tp_status ok() {
    g_err[0] = '\0';
    return TP_OK;
}

tp_status hip_status(hipError_t e, const char* where) {
    if (e != hipSuccess) return fail(TP_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
    return ok();
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

bool valid_dt(tp_dtype dt) { return dt == TP_F32 || dt == TP_BF16; }

bool valid_pair(tp_dtype in, tp_dtype out) {
    return (in == TP_F32 && out == TP_F32) || (in == TP_BF16 && (out == TP_BF16 || out == TP_F32));
}

constexpr int64_t kMaxElems = (int64_t)1 << 48;

tp_status check_rank(int tp_rank, int tp_size) {
    if (tp_size < 1 || tp_size > TP_MAX_RANKS)
        return fail(TP_EINVAL, "tp_size %d outside [1, %d]", tp_size, TP_MAX_RANKS);
    if (tp_rank < 0 || tp_rank >= tp_size)
        return fail(TP_EINVAL, "tp_rank %d outside [0, %d)", tp_rank, tp_size);
    return TP_OK;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// workspace of the two MLP launches: act [n, f_local] then the split-K area
struct MlpLayout {
    tpk::GemmPlan gu, down;
    size_t act_bytes, total;
};

MlpLayout mlp_layout(int64_t n, int64_t h, int64_t f_local, tp_dtype dt) {
    MlpLayout L;
    L.gu = tpk::plan_gemm(n, f_local, h, true, dt);
    L.down = tpk::plan_gemm(n, h, f_local, false, dt);
    L.act_bytes = align256((size_t)n * (size_t)f_local * tpk::dtype_size(dt));
    size_t split = L.gu.ws_bytes > L.down.ws_bytes ? L.gu.ws_bytes : L.down.ws_bytes;
    L.total = L.act_bytes + align256(split);
    return L;
}

tp_status check_gemm_dims(int64_t n, int64_t k, int64_t m, const char* fn) {
    if (n <= 0 || k <= 0 || m <= 0) return fail(TP_EINVAL, "%s: sizes must be positive (n=%lld k=%lld m=%lld)", fn,
                                                (long long)n, (long long)k, (long long)m);
    if (n > INT32_MAX / 2 || m > INT32_MAX / 2 || k > INT32_MAX / 2 || n * k > kMaxElems || m * k > kMaxElems ||
        n * m > kMaxElems)
        return fail(TP_ESHAPE, "%s: sizes too large", fn);
    return TP_OK;
}

// The bf16 GEMM kernels address a tile's operand rows through 32-bit byte
// offsets from the tile's first row (buffer loads).  A tile spans at most
// 256 rows of either operand, and a gated tile's up rows sit f_local rows
// after its gate rows in the fused table, so both spans must stay under
// 2 GiB: 256 k 2 < 2^31 (k < 2^22) and, gated, (f_local + 256) k 2 < 2^31
// (the fused table of the rank under about 2 GiB).
tp_status check_bf16_offsets(int64_t k, int64_t f_local, bool gated, tp_dtype dt, const char* fn) {
    if (dt != TP_BF16) return TP_OK;
    const int64_t lim = (int64_t)1 << 31;
    if (256 * k * 2 >= lim)
        return fail(TP_ESHAPE, "%s: reduction size %lld too large (bf16 tiles need 256 rows x K under 2 GiB)", fn,
                    (long long)k);
    if (gated && (f_local + 256) * k * 2 >= lim)
        return fail(TP_ESHAPE, "%s: fused gate_up table of %lld x %lld too large (the up rows must lie within 2 GiB "
                    "of the gate rows)", fn, (long long)(2 * f_local), (long long)k);
    return TP_OK;
}

// a caller workspace that is needed must be 16-byte aligned (vector stores
// of the fp32 partial tiles)
tp_status check_ws(size_t need, void* workspace, size_t workspace_bytes, size_t align, const char* fn) {
    if (need == 0) return TP_OK;
    if (!workspace || workspace_bytes < need)
        return fail(TP_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) & (align - 1))
        return fail(TP_EALIGN, "%s: workspace not %zu-byte aligned", fn, align);
    return TP_OK;
}

// The two launches of the MLP share on workspace ws (act, then the split-K
// area), laid out as L says.
hipError_t mlp_launch(const MlpLayout& L, const void* x, int64_t n, int64_t h, const void* w_gate_up,
                      const void* w_down, int64_t f_local, tp_dtype dt, void* partial, tp_dtype out_dt, void* ws,
                      hipStream_t s) {
    char* base = static_cast<char*>(ws);
    void* act = base;
    void* split = base + L.act_bytes;
    hipError_t e = tpk::launch_gemm(L.gu, x, w_gate_up, nullptr, act, n, f_local, h, true, dt, dt, split, s);
    if (e == hipSuccess) e = tpk::launch_gemm(L.down, act, w_down, nullptr, partial, n, h, f_local, false, dt, out_dt, split, s);
    return e;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

tp_status scratch_of_current_device(void** out, const char* fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TP_EHIP, "%s: hipGetDevice: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(TP_EINVAL, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TP_EHIP, "%s: hipGetSymbolAddress(scratch): HIP error %d (%s)", fn, (int)e,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TP_OK;
}

}  // namespace

extern "C" {

int tp_abi_version(void) { return TP_ABI_VERSION; }

const char* tp_last_error(void) { return g_err; }

const char* tp_status_string(int st) {
    switch (st) {
        case TP_OK: return "TP_OK";
        case TP_EINVAL: return "TP_EINVAL";
        case TP_ESHAPE: return "TP_ESHAPE";
        case TP_EDTYPE: return "TP_EDTYPE";
        case TP_EALIGN: return "TP_EALIGN";
        case TP_EHIP: return "TP_EHIP";
        case TP_EWORKSPACE: return "TP_EWORKSPACE";
        default: return "TP_UNKNOWN";
    }
}

// ---- shard selection -------------------------------------------------------

tp_status tp_shard_weights(const void* full, int64_t rows, int64_t cols, tp_dtype dt, int dim, int tp_rank,
                           int tp_size, void* out, void* stream) {
    if (!full || !out) return fail(TP_EINVAL, "tp_shard_weights: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_shard_weights: bad dtype %d", (int)dt);
    if (dim != 0 && dim != 1) return fail(TP_EINVAL, "tp_shard_weights: dim %d not 0 or 1", dim);
    if (tp_status st = check_rank(tp_rank, tp_size)) return st;
    if (rows <= 0 || cols <= 0 || rows * cols > kMaxElems)
        return fail(TP_EINVAL, "tp_shard_weights: bad shape [%lld, %lld]", (long long)rows, (long long)cols);
    const int64_t S = dim == 0 ? rows : cols;
    if (S % tp_size) return fail(TP_ESHAPE, "tp_shard_weights: size %lld of dim %d not divisible by tp_size %d",
                                 (long long)S, dim, tp_size);
    const int64_t es = (int64_t)tpk::dtype_size(dt);
    const int64_t sh = S / tp_size;
    hipError_t e;
    if (dim == 0) {
        // whole rows: one contiguous block
        const char* src = static_cast<const char*>(full) + (int64_t)tp_rank * sh * cols * es;
        e = tpk::launch_copy2d(src, sh * cols * es, out, sh * cols * es, 1, sh * cols * es, as_stream(stream));
    } else {
        const char* src = static_cast<const char*>(full) + (int64_t)tp_rank * sh * es;
        e = tpk::launch_copy2d(src, cols * es, out, sh * es, rows, sh * es, as_stream(stream));
    }
    return hip_status(e, "tp_shard_weights");
}

tp_status tp_shard_gate_up(const void* gate, const void* up, int64_t f, int64_t h, tp_dtype dt, int tp_rank,
                           int tp_size, void* out, void* stream) {
    if (!gate || !up || !out) return fail(TP_EINVAL, "tp_shard_gate_up: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_shard_gate_up: bad dtype %d", (int)dt);
    if (tp_status st = check_rank(tp_rank, tp_size)) return st;
    if (f <= 0 || h <= 0 || f * h > kMaxElems) return fail(TP_EINVAL, "tp_shard_gate_up: bad shape");
    if (f % tp_size) return fail(TP_ESHAPE, "tp_shard_gate_up: f %lld not divisible by tp_size %d", (long long)f,
                                 tp_size);
    const int64_t es = (int64_t)tpk::dtype_size(dt);
    const int64_t fl = f / tp_size;
    const int64_t seg = fl * h * es;  // bytes of one projection's rank chunk
    // segment 0 (gate) then segment 1 (up); each is the rank's chunk of the projection
    hipError_t e = tpk::launch_copy2d(static_cast<const char*>(gate) + tp_rank * seg, seg, out, seg, 1, seg,
                                      as_stream(stream));
    if (e == hipSuccess)
        e = tpk::launch_copy2d(static_cast<const char*>(up) + tp_rank * seg, seg, static_cast<char*>(out) + seg, seg,
                               1, seg, as_stream(stream));
    return hip_status(e, "tp_shard_gate_up");
}

tp_status tp_kv_heads_for_rank(int64_t n_kv, int tp_rank, int tp_size, int64_t* first, int64_t* count) {
    if (!first || !count) return fail(TP_EINVAL, "tp_kv_heads_for_rank: null pointer");
    if (tp_status st = check_rank(tp_rank, tp_size)) return st;
    if (n_kv < 1) return fail(TP_EINVAL, "tp_kv_heads_for_rank: n_kv %lld < 1", (long long)n_kv);
    if (tp_size <= n_kv) {
        if (n_kv % tp_size)
            return fail(TP_ESHAPE, "tp_kv_heads_for_rank: n_kv %lld not divisible by tp_size %d", (long long)n_kv,
                        tp_size);
        *count = n_kv / tp_size;
        *first = tp_rank * (*count);
    } else {
        if (tp_size % n_kv)
            return fail(TP_ESHAPE, "tp_kv_heads_for_rank: tp_size %d not divisible by n_kv %lld", tp_size,
                        (long long)n_kv);
        *count = 1;
        *first = tp_rank / (tp_size / n_kv);
    }
    return ok();
}

tp_status tp_shard_qkv(const void* wq, const void* wk, const void* wv, int64_t n_q, int64_t n_kv, int64_t head_dim,
                       int64_t h, tp_dtype dt, int tp_rank, int tp_size, void* out, void* stream) {
    if (!wq || !wk || !wv || !out) return fail(TP_EINVAL, "tp_shard_qkv: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_shard_qkv: bad dtype %d", (int)dt);
    if (tp_status st = check_rank(tp_rank, tp_size)) return st;
    if (n_q < 1 || n_kv < 1 || head_dim < 1 || h < 1 || n_q * head_dim * h > kMaxElems)
        return fail(TP_EINVAL, "tp_shard_qkv: bad shape");
    if (n_q % tp_size)
        return fail(TP_ESHAPE, "tp_shard_qkv: n_q %lld not divisible by tp_size %d", (long long)n_q, tp_size);
    int64_t kv0, kvc;
    if (tp_status st = tp_kv_heads_for_rank(n_kv, tp_rank, tp_size, &kv0, &kvc)) return st;
    const int64_t es = (int64_t)tpk::dtype_size(dt);
    const int64_t head_bytes = head_dim * h * es;
    const int64_t qc = n_q / tp_size;
    char* o = static_cast<char*>(out);
    hipStream_t s = as_stream(stream);
    hipError_t e = tpk::launch_copy2d(static_cast<const char*>(wq) + tp_rank * qc * head_bytes, qc * head_bytes, o,
                                      qc * head_bytes, 1, qc * head_bytes, s);
    o += qc * head_bytes;
    if (e == hipSuccess)
        e = tpk::launch_copy2d(static_cast<const char*>(wk) + kv0 * head_bytes, kvc * head_bytes, o,
                               kvc * head_bytes, 1, kvc * head_bytes, s);
    o += kvc * head_bytes;
    if (e == hipSuccess)
        e = tpk::launch_copy2d(static_cast<const char*>(wv) + kv0 * head_bytes, kvc * head_bytes, o,
                               kvc * head_bytes, 1, kvc * head_bytes, s);
    return hip_status(e, "tp_shard_qkv");
}

// ---- checkpoint-style loaders -----------------------------------------------

namespace {

size_t load_staging(int64_t rows, int64_t cols, tp_dtype src_dt, tp_dtype dst_dt) {
    if (src_dt == dst_dt) return 0;
    return align256((size_t)rows * (size_t)cols * tpk::dtype_size(src_dt));
}

// common checks, then block [r0, r0 + rows) x [c0, c0 + cols) of the host
// tensor (row length src_ld) into the table at (dr0, dc0), row length dst_ld
tp_status load_block(const char* fn, const void* src, tp_dtype src_dt, int64_t src_ld, int64_t r0, int64_t c0,
                     int64_t rows, int64_t cols, void* dst, tp_dtype dst_dt, int64_t dst_ld, int64_t dr0,
                     int64_t dc0, void* staging, size_t staging_bytes, void* stream) {
    const size_t need = load_staging(rows, cols, src_dt, dst_dt);
    if (need > 0) {
        if (!staging || staging_bytes < need)
            return fail(TP_EWORKSPACE, "%s: staging buffer of %zu bytes needed, %zu given", fn, need,
                        staging ? staging_bytes : (size_t)0);
        if (((uintptr_t)staging & 15u) != 0) return fail(TP_EALIGN, "%s: staging must be 16-byte aligned", fn);
    }
    hipError_t e = tpk::launch_load_block(src, src_dt, src_ld, r0, c0, rows, cols, dst, dst_dt, dst_ld, dr0, dc0,
                                          staging, as_stream(stream));
    return hip_status(e, fn);
}

tp_status load_common(const char* fn, const void* src, tp_dtype src_dt, void* dst, tp_dtype dst_dt, int tp_rank,
                      int tp_size) {
    if (!src || !dst) return fail(TP_EINVAL, "%s: null pointer", fn);
    if (!valid_dt(src_dt) || !valid_dt(dst_dt))
        return fail(TP_EDTYPE, "%s: bad dtype pair %d -> %d", fn, (int)src_dt, (int)dst_dt);
    return check_rank(tp_rank, tp_size);
}

}  // namespace

tp_status tp_load_staging_bytes(int64_t rows, int64_t cols, tp_dtype src_dt, tp_dtype dst_dt, size_t* bytes) {
    if (!bytes) return fail(TP_EINVAL, "tp_load_staging_bytes: null pointer");
    if (!valid_dt(src_dt) || !valid_dt(dst_dt)) return fail(TP_EDTYPE, "tp_load_staging_bytes: bad dtype");
    if (rows < 0 || cols < 0 || (cols > 0 && rows > kMaxElems / cols))
        return fail(TP_EINVAL, "tp_load_staging_bytes: bad shape");
    *bytes = load_staging(rows, cols, src_dt, dst_dt);
    return ok();
}

tp_status tp_load_shard(const void* src, tp_dtype src_dt, int64_t rows, int64_t cols, int dim, int tp_rank,
                        int tp_size, void* dst, tp_dtype dst_dt, void* staging, size_t staging_bytes, void* stream) {
    if (tp_status st = load_common("tp_load_shard", src, src_dt, dst, dst_dt, tp_rank, tp_size)) return st;
    if (dim != 0 && dim != 1) return fail(TP_EINVAL, "tp_load_shard: dim %d not 0 or 1", dim);
    if (rows < 1 || cols < 1 || rows > kMaxElems / cols)
        return fail(TP_EINVAL, "tp_load_shard: bad shape [%lld, %lld]", (long long)rows, (long long)cols);
    const int64_t S = dim == 0 ? rows : cols;
    if (S % tp_size)
        return fail(TP_ESHAPE, "tp_load_shard: size %lld of dim %d not divisible by tp_size %d", (long long)S, dim,
                    tp_size);
    const int64_t sh = S / tp_size;
    if (dim == 0)
        return load_block("tp_load_shard", src, src_dt, cols, tp_rank * sh, 0, sh, cols, dst, dst_dt, cols, 0, 0,
                          staging, staging_bytes, stream);
    return load_block("tp_load_shard", src, src_dt, cols, 0, tp_rank * sh, rows, sh, dst, dst_dt, sh, 0, 0, staging,
                      staging_bytes, stream);
}

tp_status tp_load_gate_up(const void* src, tp_dtype src_dt, int shard_id, int64_t f, int64_t h, int tp_rank,
                          int tp_size, void* dst, tp_dtype dst_dt, void* staging, size_t staging_bytes, void* stream) {
    if (tp_status st = load_common("tp_load_gate_up", src, src_dt, dst, dst_dt, tp_rank, tp_size)) return st;
    if (shard_id != 0 && shard_id != 1) return fail(TP_EINVAL, "tp_load_gate_up: shard_id %d not 0 (gate) or 1 (up)", shard_id);
    if (f < 1 || h < 1 || f > kMaxElems / h) return fail(TP_EINVAL, "tp_load_gate_up: bad shape");
    if (f % tp_size)
        return fail(TP_ESHAPE, "tp_load_gate_up: f %lld not divisible by tp_size %d", (long long)f, tp_size);
    const int64_t fc = f / tp_size;
    return load_block("tp_load_gate_up", src, src_dt, h, tp_rank * fc, 0, fc, h, dst, dst_dt, h, shard_id * fc, 0,
                      staging, staging_bytes, stream);
}

tp_status tp_load_qkv(const void* src, tp_dtype src_dt, int shard_id, int64_t n_q, int64_t n_kv, int64_t head_dim,
                      int64_t h, int tp_rank, int tp_size, void* dst, tp_dtype dst_dt, void* staging,
                      size_t staging_bytes, void* stream) {
    if (tp_status st = load_common("tp_load_qkv", src, src_dt, dst, dst_dt, tp_rank, tp_size)) return st;
    if (shard_id < 0 || shard_id > 2) return fail(TP_EINVAL, "tp_load_qkv: shard_id %d not 0 (q), 1 (k) or 2 (v)", shard_id);
    if (n_q < 1 || n_kv < 1 || head_dim < 1 || h < 1 || n_q * head_dim > kMaxElems / h)
        return fail(TP_EINVAL, "tp_load_qkv: bad shape");
    if (n_q % tp_size)
        return fail(TP_ESHAPE, "tp_load_qkv: n_q %lld not divisible by tp_size %d", (long long)n_q, tp_size);
    int64_t kv0, kvc;
    if (tp_status st = tp_kv_heads_for_rank(n_kv, tp_rank, tp_size, &kv0, &kvc)) return st;
    const int64_t qc = n_q / tp_size;
    // segment of the projection in the rank's table, and the rows of the
    // full projection it takes (whole heads of head_dim rows)
    int64_t seg, first, count;
    if (shard_id == 0) {
        seg = 0;
        first = tp_rank * qc;
        count = qc;
    } else {
        seg = shard_id == 1 ? qc : qc + kvc;
        first = kv0;
        count = kvc;
    }
    return load_block("tp_load_qkv", src, src_dt, h, first * head_dim, 0, count * head_dim, h, dst, dst_dt, h,
                      seg * head_dim, 0, staging, staging_bytes, stream);
}

// ---- GEMMs --------------------------------------------------------------------

tp_status tp_gate_up_workspace_bytes(int64_t n, int64_t h, int64_t f_local, tp_dtype dt, size_t* bytes) {
    if (!bytes) return fail(TP_EINVAL, "tp_gate_up_workspace_bytes: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_gate_up_workspace_bytes: bad dtype %d", (int)dt);
    if (tp_status st = check_gemm_dims(n, h, 2 * f_local, "tp_gate_up_workspace_bytes")) return st;
    if (tp_status st = check_bf16_offsets(h, f_local, true, dt, "tp_gate_up_workspace_bytes")) return st;
    *bytes = tpk::plan_gemm(n, f_local, h, true, dt).ws_bytes;
    return ok();
}

tp_status tp_gate_up_act_rank(const void* x, int64_t n, int64_t h, const void* w_gate_up, int64_t f_local,
                              tp_dtype dt, void* act, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !w_gate_up || !act) return fail(TP_EINVAL, "tp_gate_up_act_rank: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_gate_up_act_rank: bad dtype %d", (int)dt);
    if (tp_status st = check_gemm_dims(n, h, 2 * f_local, "tp_gate_up_act_rank")) return st;
    if (tp_status st = check_bf16_offsets(h, f_local, true, dt, "tp_gate_up_act_rank")) return st;
    tpk::GemmPlan pl = tpk::plan_gemm(n, f_local, h, true, dt);
    if (tp_status st = check_ws(pl.ws_bytes, workspace, workspace_bytes, 16, "tp_gate_up_act_rank")) return st;
    return hip_status(tpk::launch_gemm(pl, x, w_gate_up, nullptr, act, n, f_local, h, true, dt, dt, workspace,
                                       as_stream(stream)),
                      "tp_gate_up_act_rank");
}

tp_status tp_linear_workspace_bytes(int64_t n, int64_t k, int64_t m, tp_dtype dt, size_t* bytes) {
    if (!bytes) return fail(TP_EINVAL, "tp_linear_workspace_bytes: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_linear_workspace_bytes: bad dtype %d", (int)dt);
    if (tp_status st = check_gemm_dims(n, k, m, "tp_linear_workspace_bytes")) return st;
    if (tp_status st = check_bf16_offsets(k, 0, false, dt, "tp_linear_workspace_bytes")) return st;
    *bytes = tpk::plan_gemm(n, m, k, false, dt).ws_bytes;
    return ok();
}

tp_status tp_linear_rank_forward(const void* x, int64_t n, int64_t k, const void* w, int64_t m, const void* bias,
                                 tp_dtype dt, void* y, tp_dtype out_dt, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    if (!x || !w || !y) return fail(TP_EINVAL, "tp_linear_rank_forward: null pointer");
    if (!valid_dt(dt) || !valid_dt(out_dt) || !valid_pair(dt, out_dt))
        return fail(TP_EDTYPE, "tp_linear_rank_forward: unsupported dtype pair (%d -> %d)", (int)dt, (int)out_dt);
    if (tp_status st = check_gemm_dims(n, k, m, "tp_linear_rank_forward")) return st;
    if (tp_status st = check_bf16_offsets(k, 0, false, dt, "tp_linear_rank_forward")) return st;
    tpk::GemmPlan pl = tpk::plan_gemm(n, m, k, false, dt);
    if (tp_status st = check_ws(pl.ws_bytes, workspace, workspace_bytes, 16, "tp_linear_rank_forward")) return st;
    return hip_status(tpk::launch_gemm(pl, x, w, bias, y, n, m, k, false, dt, out_dt, workspace, as_stream(stream)),
                      "tp_linear_rank_forward");
}

tp_status tp_mlp_workspace_bytes(int64_t n, int64_t h, int64_t f_local, tp_dtype dt, size_t* bytes) {
    if (!bytes) return fail(TP_EINVAL, "tp_mlp_workspace_bytes: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_mlp_workspace_bytes: bad dtype %d", (int)dt);
    if (tp_status st = check_gemm_dims(n, h, 2 * f_local, "tp_mlp_workspace_bytes")) return st;
    if (tp_status st = check_bf16_offsets(h, f_local, true, dt, "tp_mlp_workspace_bytes")) return st;
    if (tp_status st = check_bf16_offsets(f_local, 0, false, dt, "tp_mlp_workspace_bytes")) return st;
    *bytes = mlp_layout(n, h, f_local, dt).total;
    return ok();
}

tp_status tp_mlp_rank_forward(const void* x, int64_t n, int64_t h, const void* w_gate_up, const void* w_down,
                              int64_t f_local, tp_dtype dt, void* partial, tp_dtype out_dt, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (!x || !w_gate_up || !w_down || !partial) return fail(TP_EINVAL, "tp_mlp_rank_forward: null pointer");
    if (!valid_dt(dt) || !valid_dt(out_dt) || !valid_pair(dt, out_dt))
        return fail(TP_EDTYPE, "tp_mlp_rank_forward: unsupported dtype pair (%d -> %d)", (int)dt, (int)out_dt);
    if (tp_status st = check_gemm_dims(n, h, 2 * f_local, "tp_mlp_rank_forward")) return st;
    if (tp_status st = check_bf16_offsets(h, f_local, true, dt, "tp_mlp_rank_forward")) return st;
    if (tp_status st = check_bf16_offsets(f_local, 0, false, dt, "tp_mlp_rank_forward")) return st;
    MlpLayout L = mlp_layout(n, h, f_local, dt);
    if (tp_status st = check_ws(L.total, workspace, workspace_bytes, 256, "tp_mlp_rank_forward")) return st;
    return hip_status(mlp_launch(L, x, n, h, w_gate_up, w_down, f_local, dt, partial, out_dt, workspace,
                                 as_stream(stream)),
                      "tp_mlp_rank_forward");
}

tp_status tp_mlp_rank_forward_noalloc(const void* x, int64_t n, int64_t h, const void* w_gate_up,
                                      const void* w_down, int64_t f_local, tp_dtype dt, void* partial,
                                      tp_dtype out_dt, void* stream) {
    const char* fn = "tp_mlp_rank_forward_noalloc";
    if (!x || !w_gate_up || !w_down || !partial) return fail(TP_EINVAL, "%s: null pointer", fn);
    if (!valid_dt(dt) || !valid_dt(out_dt) || !valid_pair(dt, out_dt))
        return fail(TP_EDTYPE, "%s: unsupported dtype pair (%d -> %d)", fn, (int)dt, (int)out_dt);
    if (tp_status st = check_gemm_dims(n, h, 2 * f_local, fn)) return st;
    if (tp_status st = check_bf16_offsets(h, f_local, true, dt, fn)) return st;
    if (tp_status st = check_bf16_offsets(f_local, 0, false, dt, fn)) return st;
    MlpLayout L = mlp_layout(n, h, f_local, dt);
    if (L.total > (size_t)TP_NOALLOC_SCRATCH_BYTES)
        return fail(TP_EWORKSPACE, "%s: this shape needs %zu bytes of scratch, more than the library's %zu "
                    "(use tp_mlp_rank_forward with a caller workspace)", fn, L.total,
                    (size_t)TP_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (tp_status st = scratch_of_current_device(&ws, fn)) return st;
    return hip_status(mlp_launch(L, x, n, h, w_gate_up, w_down, f_local, dt, partial, out_dt, ws, as_stream(stream)),
                      fn);
}

// ---- reduce -------------------------------------------------------------------

tp_status tp_partial_reduce(const void* const* partials, int t, int64_t K, tp_dtype in_dt, void* out, tp_dtype out_dt,
                            tp_order order, void* stream) {
    if (!partials || !out) return fail(TP_EINVAL, "tp_partial_reduce: null pointer");
    if (t < 1 || t > TP_MAX_RANKS) return fail(TP_EINVAL, "tp_partial_reduce: t %d outside [1, %d]", t, TP_MAX_RANKS);
    for (int r = 0; r < t; ++r)
        if (!partials[r]) return fail(TP_EINVAL, "tp_partial_reduce: partials[%d] is null", r);
    if (K < 0 || K > kMaxElems) return fail(TP_EINVAL, "tp_partial_reduce: K %lld out of range", (long long)K);
    if (!valid_dt(in_dt) || !valid_dt(out_dt) || !valid_pair(in_dt, out_dt))
        return fail(TP_EDTYPE, "tp_partial_reduce: unsupported dtype pair (%d -> %d)", (int)in_dt, (int)out_dt);
    if (order != TP_ORDER_RING && order != TP_ORDER_RANK)
        return fail(TP_EINVAL, "tp_partial_reduce: unknown order %d", (int)order);
    return hip_status(tpk::launch_ring_reduce(partials, t, K, in_dt, out, out_dt, order, as_stream(stream)),
                      "tp_partial_reduce");
}

static tp_status check_attention(int64_t n, int nq, int nkv, int head_dim, tp_dtype dt, const char* fn) {
    if (dt != TP_BF16) return fail(TP_EDTYPE, "%s: bf16 only", fn);
    if (head_dim != 128) return fail(TP_EINVAL, "%s: head_dim %d (128 supported)", fn, head_dim);
    if (nq < 1 || nkv < 1 || nq > 4096 || nkv > 4096) return fail(TP_EINVAL, "%s: bad head counts", fn);
    if (nq % nkv != 0) return fail(TP_ESHAPE, "%s: nkv %d does not divide nq %d", fn, nkv, nq);
    if (n < 0 || n * (int64_t)(nq + 2 * nkv) * head_dim * 2 >= ((int64_t)1 << 31))
        return fail(TP_EINVAL, "%s: qkv must be under 2 GiB", fn);
    return TP_OK;
}

tp_status tp_attention_workspace_bytes(int64_t n, int nq, int nkv, int head_dim, tp_dtype dt, int causal,
                                       size_t* bytes) {
    if (!bytes) return fail(TP_EINVAL, "tp_attention_workspace_bytes: null pointer");
    if (tp_status st = check_attention(n, nq, nkv, head_dim, dt, "tp_attention_workspace_bytes")) return st;
    *bytes = tpk::attention_ws_bytes(n, nq, nkv, causal);
    return ok();
}

tp_status tp_attention_rank(const void* qkv, int64_t n, int nq, int nkv, int head_dim, tp_dtype dt, int causal,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
    if (!qkv || !out) return fail(TP_EINVAL, "tp_attention_rank: null pointer");
    if (tp_status st = check_attention(n, nq, nkv, head_dim, dt, "tp_attention_rank")) return st;
    const size_t need = tpk::attention_ws_bytes(n, nq, nkv, causal);
    if (tp_status st = check_ws(need, workspace, workspace_bytes, 16, "tp_attention_rank")) return st;
    if ((((uintptr_t)qkv) | ((uintptr_t)out)) & 15u)
        return fail(TP_EALIGN, "tp_attention_rank: qkv and out must be 16-byte aligned");
    const uintptr_t q0 = (uintptr_t)qkv, q1 = q0 + (uintptr_t)(n * (int64_t)(nq + 2 * nkv) * head_dim * 2);
    const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (uintptr_t)(n * (int64_t)nq * head_dim * 2);
    if (n > 0 && o0 < q1 && q0 < o1) return fail(TP_EINVAL, "tp_attention_rank: out overlaps qkv");
    return hip_status(tpk::launch_attention(qkv, n, nq, nkv, head_dim, causal, out, workspace, as_stream(stream)),
                      "tp_attention_rank");
}

tp_status tp_logits_gather_argmax(const void* const* shards, int t, int64_t n, int64_t vocab, tp_dtype dt, void* full,
                                  int64_t* argmax, void* stream) {
    if (!shards || (!full && !argmax)) return fail(TP_EINVAL, "tp_logits_gather_argmax: null pointer");
    if (t < 1 || t > TP_MAX_RANKS)
        return fail(TP_EINVAL, "tp_logits_gather_argmax: t %d outside [1, %d]", t, TP_MAX_RANKS);
    if (dt != TP_F32) return fail(TP_EDTYPE, "tp_logits_gather_argmax: logits must be fp32");
    if (n < 0 || n > INT32_MAX || vocab < 1 || vocab > kMaxElems || n * vocab > kMaxElems)
        return fail(TP_EINVAL, "tp_logits_gather_argmax: bad shape n %lld vocab %lld", (long long)n, (long long)vocab);
    for (int r = 0; r < t; ++r) {
        int64_t s, e;
        if (tp_status st = tp_vocab_range(vocab, r, t, &s, &e)) return st;
        if (e > s && !shards[r]) return fail(TP_EINVAL, "tp_logits_gather_argmax: shards[%d] is null", r);
        if (full && shards[r] == full) return fail(TP_EINVAL, "tp_logits_gather_argmax: full aliases shards[%d]", r);
    }
    ok();
    return hip_status(tpk::launch_logits_gather_argmax(shards, t, n, vocab, full, argmax, as_stream(stream)),
                      "tp_logits_gather_argmax");
}

tp_status tp_sp_rows(int64_t n, int tp_rank, int tp_size, int64_t* lo, int64_t* hi) {
    if (!lo || !hi) return fail(TP_EINVAL, "tp_sp_rows: null pointer");
    if (tp_size < 1 || tp_size > TP_MAX_RANKS || tp_rank < 0 || tp_rank >= tp_size)
        return fail(TP_EINVAL, "tp_sp_rows: rank %d of %d", tp_rank, tp_size);
    if (n < 0 || n > kMaxElems) return fail(TP_EINVAL, "tp_sp_rows: n out of range");
    const int c = (tp_rank + 1) % tp_size;
    *lo = (int64_t)(((__int128)c * n) / tp_size);
    *hi = (int64_t)(((__int128)(c + 1) * n) / tp_size);
    return ok();
}

tp_status tp_rs_add_rmsnorm(const void* const* partials, int t, int tp_rank, int64_t n, int64_t h, tp_dtype dt,
                            const void* residual, const void* weight, float eps, void* residual_out, void* out,
                            void* stream) {
    if (!partials || !weight) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: null pointer");
    if (t < 1 || t > TP_MAX_RANKS) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: t %d outside [1, %d]", t, TP_MAX_RANKS);
    if (tp_rank < 0 || tp_rank >= t) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: rank %d of %d", tp_rank, t);
    if (n < 0 || n > kMaxElems) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: n out of range");
    const int c = (tp_rank + 1) % t;
    const bool rows = ((__int128)(c + 1) * n) / t > ((__int128)c * n) / t;
    // the row buffers may be null when the rank holds no rows
    if (rows && (!residual || !residual_out || !out)) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: null pointer");
    for (int r = 0; r < t; ++r) {
        if (!partials[r]) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: partials[%d] is null", r);
        if (rows && (partials[r] == out || partials[r] == residual_out))
            return fail(TP_EINVAL, "tp_rs_add_rmsnorm: an output aliases partials[%d]", r);
    }
    if (n < 0 || h < 1 || n > INT32_MAX || h > INT32_MAX || n * h > kMaxElems)
        return fail(TP_EINVAL, "tp_rs_add_rmsnorm: bad shape n %lld h %lld", (long long)n, (long long)h);
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_rs_add_rmsnorm: bad dtype %d", (int)dt);
    if (!(eps >= 0.0f) || eps == INFINITY) return fail(TP_EINVAL, "tp_rs_add_rmsnorm: eps must be finite and >= 0");
    if (rows && (out == residual || out == residual_out))
        return fail(TP_EINVAL, "tp_rs_add_rmsnorm: out aliases the residual");
    return hip_status(tpk::launch_rs_add_rmsnorm(partials, t, tp_rank, n, h, dt, residual, weight, eps, residual_out, out,
                                                 as_stream(stream)),
                      "tp_rs_add_rmsnorm");
}

tp_status tp_ring_schedule(int t, int64_t K, tp_ring_step* steps, int max_steps, int* n_steps) {
    if (!steps || !n_steps) return fail(TP_EINVAL, "tp_ring_schedule: null pointer");
    if (t < 1 || t > TP_MAX_RANKS) return fail(TP_EINVAL, "tp_ring_schedule: t %d outside [1, %d]", t, TP_MAX_RANKS);
    if (K < 0 || K > kMaxElems) return fail(TP_EINVAL, "tp_ring_schedule: K out of range");
    const int need = 2 * t * (t - 1);
    if (max_steps < need) return fail(TP_ESHAPE, "tp_ring_schedule: %d steps needed, room for %d", need, max_steps);
    int k = 0;
    for (int phase = 0; phase < 2; ++phase)
        for (int s = 0; s < t - 1; ++s)
            for (int r = 0; r < t; ++r) {
                // reduce-scatter: rank r forwards the partially reduced chunk it
                // received last round (its own chunk at s = 0); all-gather: it
                // forwards the finished chunk it owns / just received.
                const int c = phase == 0 ? (((r - s) % t) + t) % t : (((r + 1 - s) % t) + t) % t;
                tp_ring_step& st = steps[k++];
                st.phase = phase;
                st.step = s;
                st.src = r;
                st.dst = (r + 1) % t;
                st.chunk = c;
                const int64_t lo = (int64_t)(((__int128)c * K) / t);
                const int64_t hi = (int64_t)(((__int128)(c + 1) * K) / t);
                st.offset = lo;
                st.len = hi - lo;
            }
    *n_steps = k;
    return ok();
}

// ---- vocab parallel ---------------------------------------------------------

tp_status tp_vocab_range(int64_t vocab, int tp_rank, int tp_size, int64_t* start, int64_t* end) {
    if (!start || !end) return fail(TP_EINVAL, "tp_vocab_range: null pointer");
    if (tp_status st = check_rank(tp_rank, tp_size)) return st;
    if (vocab < 1 || vocab > kMaxElems) return fail(TP_EINVAL, "tp_vocab_range: vocab %lld out of range", (long long)vocab);
    const int64_t per = (vocab + tp_size - 1) / tp_size;
    int64_t s = tp_rank * per, e = (tp_rank + 1) * per;
    if (e > vocab) e = vocab;
    if (s > e) s = e;
    *start = s;
    *end = e;
    return ok();
}

tp_status tp_vocab_embed_rank(const int64_t* ids, int64_t n, const void* table_shard, int64_t vocab, int64_t h,
                              int tp_rank, int tp_size, tp_dtype dt, void* out, void* stream) {
    if (!ids || !out) return fail(TP_EINVAL, "tp_vocab_embed_rank: null pointer");
    if (!valid_dt(dt)) return fail(TP_EDTYPE, "tp_vocab_embed_rank: bad dtype %d", (int)dt);
    if (n <= 0 || h <= 0 || n * h > kMaxElems) return fail(TP_EINVAL, "tp_vocab_embed_rank: bad shape");
    int64_t s, e;
    if (tp_status st = tp_vocab_range(vocab, tp_rank, tp_size, &s, &e)) return st;
    if (e > s && !table_shard) return fail(TP_EINVAL, "tp_vocab_embed_rank: null table for a non-empty shard");
    return hip_status(tpk::launch_vocab_embed(ids, n, table_shard, s, e, h, (int)tpk::dtype_size(dt), out,
                                              as_stream(stream)),
                      "tp_vocab_embed_rank");
}

tp_status tp_lm_head_rank(const void* x, int64_t n, int64_t h, const void* table_shard, int64_t v_local, tp_dtype dt,
                          void* logits, tp_dtype out_dt, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !table_shard || !logits) return fail(TP_EINVAL, "tp_lm_head_rank: null pointer");
    if (!valid_dt(dt) || !valid_dt(out_dt) || !valid_pair(dt, out_dt))
        return fail(TP_EDTYPE, "tp_lm_head_rank: unsupported dtype pair (%d -> %d)", (int)dt, (int)out_dt);
    if (tp_status st = check_gemm_dims(n, h, v_local, "tp_lm_head_rank")) return st;
    if (tp_status st = check_bf16_offsets(h, 0, false, dt, "tp_lm_head_rank")) return st;
    tpk::GemmPlan pl = tpk::plan_gemm(n, v_local, h, false, dt);
    if (tp_status st = check_ws(pl.ws_bytes, workspace, workspace_bytes, 16, "tp_lm_head_rank")) return st;
    return hip_status(tpk::launch_gemm(pl, x, table_shard, nullptr, logits, n, v_local, h, false, dt, out_dt,
                                       workspace, as_stream(stream)),
                      "tp_lm_head_rank");
}

}  // extern "C"
