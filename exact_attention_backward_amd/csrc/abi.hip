// C ABI of the library: argument validation, workspace layout and dispatch.
// Every entry point validates before any HIP call, so the error paths run
// (and are tested) on machines without a GPU.
#include <stdint.h>
#include <stddef.h>

#include "launch.h"

using namespace attn;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kErrBytes = 256;   // status words of the deterministic mode

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the caller's strides, or those of the contiguous layouts
attn_strides_t strides_of(const attn_shape_t* s) {
    if (s->strides != nullptr) return *s->strides;
    const long long d = s->head_dim;
    const attn_tensor_strides_t qs{(long long)s->seqlen_q * s->num_heads_q * d, (long long)s->num_heads_q * d, d};
    const attn_tensor_strides_t ks{(long long)s->seqlen_k * s->num_heads_kv * d, (long long)s->num_heads_kv * d, d};
    return attn_strides_t{qs, ks, ks, qs, qs, qs, ks, ks};
}

int validate_shape(const attn_shape_t* s) {
    if (s == nullptr) return ATTN_ERR_NULL_ARG;
    if (s->dtype != ATTN_DTYPE_F32 && s->dtype != ATTN_DTYPE_BF16 && s->dtype != ATTN_DTYPE_F16)
        return ATTN_ERR_UNSUPPORTED;
    if (s->head_dim < 8 || s->head_dim > 128 || s->head_dim % 8 != 0) return ATTN_ERR_UNSUPPORTED;
    if (s->batch <= 0 || s->num_heads_q <= 0 || s->num_heads_kv <= 0 || s->seqlen_q <= 0 || s->seqlen_k <= 0)
        return ATTN_ERR_BAD_SHAPE;
    if (s->num_heads_q % s->num_heads_kv != 0) return ATTN_ERR_BAD_SHAPE;
    if ((s->cu_seqlens_q == nullptr) != (s->cu_seqlens_k == nullptr)) return ATTN_ERR_BAD_SHAPE;
    if (s->cu_seqlens_q != nullptr) {
        if (s->total_q <= 0 || s->total_k <= 0) return ATTN_ERR_BAD_SHAPE;
        if ((reinterpret_cast<uintptr_t>(s->cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(s->cu_seqlens_k) & 3u))
            return ATTN_ERR_MISALIGNED;
    } else if (s->seqused_q != nullptr || s->seqused_k != nullptr) {
        return ATTN_ERR_BAD_SHAPE;   // used lengths are a varlen feature
    }
    if ((reinterpret_cast<uintptr_t>(s->seqused_q) & 3u) || (reinterpret_cast<uintptr_t>(s->seqused_k) & 3u) ||
        (reinterpret_cast<uintptr_t>(s->alibi_slopes) & 3u))
        return ATTN_ERR_MISALIGNED;
    if (!(s->softmax_scale == s->softmax_scale)) return ATTN_ERR_BAD_SHAPE;   // NaN scale
    if (s->causal != 0 && s->causal != 1) return ATTN_ERR_BAD_SHAPE;
    if (s->local != 0 && s->local != 1) return ATTN_ERR_BAD_SHAPE;
    if (s->local && (s->window_left < -1 || s->window_right < -1)) return ATTN_ERR_BAD_SHAPE;
    if (s->deterministic != 0 && s->deterministic != 1) return ATTN_ERR_BAD_SHAPE;
    if (s->dq_algo != ATTN_DQ_SEPARATE && s->dq_algo != ATTN_DQ_ATOMIC && s->dq_algo != ATTN_DQ_STORED_DS)
        return ATTN_ERR_UNSUPPORTED;
    if (s->dq_algo == ATTN_DQ_STORED_DS && s->dtype == ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
    // element counts must stay addressable with 64-bit offsets and 32-bit row counts
    const long long rows_q = s->cu_seqlens_q ? s->total_q : (long long)s->batch * s->seqlen_q;
    const long long rows_k = s->cu_seqlens_k ? s->total_k : (long long)s->batch * s->seqlen_k;
    if (rows_q > 0x7fffffffLL || rows_k > 0x7fffffffLL) return ATTN_ERR_BAD_SHAPE;
    // one-dimensional grids of the streaming kernels: (row, head) pairs times
    // lanes per pair must stay below 2^32 threads
    if (rows_q * s->num_heads_q > (1LL << 27) || rows_k * s->num_heads_kv > (1LL << 27)) return ATTN_ERR_BAD_SHAPE;
    // strides: non-negative and 16-byte multiples (rows and heads start on
    // 16-byte boundaries); a tile's byte offset within one sequence's rows
    // travels in a 32-bit offset, and all buffer ranges stay below kOobOff
    const long long esz = s->dtype == ATTN_DTYPE_F32 ? 4 : 2;
    const attn_strides_t d = strides_of(s);
    const attn_tensor_strides_t* all[] = {&d.q, &d.k, &d.v, &d.o, &d.dout, &d.dq, &d.dk, &d.dv};
    for (int t = 0; t < 8; ++t) {
        const attn_tensor_strides_t* x = all[t];
        if (x->batch < 0 || x->row < 0 || x->head < 0) return ATTN_ERR_BAD_SHAPE;
        if ((x->batch * esz) % 16 || (x->row * esz) % 16 || (x->head * esz) % 16) return ATTN_ERR_MISALIGNED;
        // rows of q, k, v, o, dout, dq, dk, dv in one sequence
        const long long len = (t == 1 || t == 2 || t >= 6) ? s->seqlen_k : s->seqlen_q;
        if ((len + 1) * x->row * esz >= kOobOff - (1LL << 20)) return ATTN_ERR_BAD_SHAPE;
        if (x->head * esz >= (1LL << 31)) return ATTN_ERR_BAD_SHAPE;   // 32-bit head steps
    }
    const attn_tensor_strides_t* bs[] = {&s->bias_strides, &s->dbias_strides};
    const void* bp[] = {s->bias, s->dbias};
    for (int t = 0; t < 2; ++t) {
        if (bp[t] == nullptr) continue;
        if (bs[t]->batch < 0 || bs[t]->row < 0 || bs[t]->head < 0) return ATTN_ERR_BAD_SHAPE;
        if (reinterpret_cast<uintptr_t>(bp[t]) % esz) return ATTN_ERR_MISALIGNED;
    }
    return ATTN_OK;
}

// the backward entry points: an elementwise bias or its gradient needs the
// atomic dQ mode (the forward takes a bias whatever dq_algo says)
int validate_bwd(const attn_shape_t* s) {
    const int st = validate_shape(s);
    if (st) return st;
    if ((s->bias != nullptr || s->dbias != nullptr) && s->dq_algo != ATTN_DQ_ATOMIC) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

bool varlen(const attn_shape_t* s) { return s->cu_seqlens_q != nullptr; }

// the head dim the kernels tile with: head_dim rounded up to 64 or 128
int padded_hd(const attn_shape_t* s) { return s->head_dim <= 64 ? 64 : 128; }

Strides to_kernel(const attn_tensor_strides_t& t) { return Strides{t.batch, t.row, t.head}; }

// Window bounds of the kernels: key j visible to query i iff
// i + off - lo <= j <= i + off + hi (kNoWindow: unbounded side).  Sequences
// hold fewer than 2^27 rows, so a window of kNoWindow or more already spans
// every key and is clamped there (keeping i + off + hi inside 32 bits).
int win_lo(const attn_shape_t* s) {
    return s->local && s->window_left >= 0 ? (s->window_left < kNoWindow ? s->window_left : kNoWindow) : kNoWindow;
}
int win_hi(const attn_shape_t* s) {
    if (s->causal) return 0;   // the causal bound is the tighter one (window_right >= 0)
    return s->local && s->window_right >= 0 ? (s->window_right < kNoWindow ? s->window_right : kNoWindow)
                                            : kNoWindow;
}
// whether any bound applies (the kernels' masked instantiation)
bool masked(const attn_shape_t* s) { return win_lo(s) < kNoWindow || win_hi(s) < kNoWindow; }
long long rows_q(const attn_shape_t* s) { return varlen(s) ? s->total_q : (long long)s->batch * s->seqlen_q; }

size_t elem_bytes(const attn_shape_t* s) { return s->dtype == ATTN_DTYPE_F32 ? 4 : 2; }

// workspace = [dQ accumulator fp32][ordering counters int32][status words]
size_t accum_bytes(const attn_shape_t* s) {
    return align_up((size_t)rows_q(s) * s->num_heads_q * padded_hd(s) * sizeof(float));
}
int nblk_m(const attn_shape_t* s) {
    const int bm = bwd_block_m(s->dtype, padded_hd(s));
    return (s->seqlen_q + bm - 1) / bm;
}
size_t sem_bytes(const attn_shape_t* s) {
    return align_up((size_t)s->batch * s->num_heads_q * nblk_m(s) * sizeof(int32_t));
}
// stored-dS mode: [first query block of each sequence, int32][dS blocks]
long long ds_qb(const attn_shape_t* s) {
    if (varlen(s)) return (long long)(s->total_q + kDsRows - 1) / kDsRows + s->batch;
    return (long long)s->batch * ((s->seqlen_q + kDsRows - 1) / kDsRows);
}
int ds_nn(const attn_shape_t* s) { return (s->seqlen_k + kDsKeys - 1) / kDsKeys; }
size_t ds_table_bytes(const attn_shape_t* s) {
    return s->dq_algo == ATTN_DQ_STORED_DS ? align_up((size_t)(s->batch + 1) * sizeof(int32_t)) : 0;
}
size_t ds_bytes(const attn_shape_t* s) {
    if (s->dq_algo != ATTN_DQ_STORED_DS) return 0;
    return (size_t)s->num_heads_q * (size_t)ds_qb(s) * (size_t)ds_nn(s) * kDsBlockBytes;
}
size_t workspace_bytes(const attn_shape_t* s) {
    return accum_bytes(s) + sem_bytes(s) + kErrBytes + ds_table_bytes(s) + ds_bytes(s);
}

int check_launch() {
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL_ARG: return "null argument";
        case ATTN_ERR_BAD_SHAPE: return "bad shape";
        case ATTN_ERR_UNSUPPORTED: return "unsupported dtype, head_dim or dq_algo";
        case ATTN_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

size_t attn_bwd_workspace_bytes(const attn_shape_t* shape) {
    if (validate_bwd(shape) != ATTN_OK) return 0;
    return workspace_bytes(shape);
}

int attn_fwd(const attn_shape_t* s, const void* q, const void* k, const void* v, void* o, float* lse,
             void* stream) {
    int st = validate_shape(s);
    if (st) return st;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_MISALIGNED;
    FwdArgs a{q, k, v, o, lse, s->cu_seqlens_q, s->cu_seqlens_k, s->seqused_q, s->seqused_k, s->batch,
              s->num_heads_q, s->num_heads_kv,
              s->seqlen_q, s->seqlen_k, s->total_q, s->total_k, s->softmax_scale};
    (void)hipGetLastError();   // clear a stale error so the check below is ours
    a.win_lo = win_lo(s);
    a.win_hi = win_hi(s);
    a.alibi = s->alibi_slopes;
    const attn_strides_t d = strides_of(s);
    a.d = s->head_dim;
    a.sq = to_kernel(d.q);
    a.sk = to_kernel(d.k);
    a.sv = to_kernel(d.v);
    a.so = to_kernel(d.o);
    a.bias = s->bias;
    a.sbias = to_kernel(s->bias_strides);
    // the MFMA forward for the 16-bit types; fp32 and the elementwise bias
    // take the plain one
    if (s->dtype != ATTN_DTYPE_F32 && s->bias == nullptr)
        launch_fwd_mfma(a, s->dtype, padded_hd(s), masked(s), reinterpret_cast<hipStream_t>(stream));
    else
        launch_fwd(a, s->dtype, padded_hd(s), masked(s), reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

}  // extern "C"

namespace {

// The enqueue steps behind the entry points; arguments already validated.
void enqueue_preprocess(const attn_shape_t* s, const void* o, const void* dout, float* delta, void* workspace,
                        hipStream_t hs) {
    // the preprocess kernel also clears the counters and status words, and
    // the accumulator where it is added into (atomic modes); the dS blocks
    // are written before they are read
    const bool atomic = s->dq_algo == ATTN_DQ_ATOMIC;
    char* zero = reinterpret_cast<char*>(workspace) + (atomic ? 0 : accum_bytes(s));
    const size_t zero_bytes = (atomic ? accum_bytes(s) : 0) + sem_bytes(s) + kErrBytes;
    const attn_strides_t d = strides_of(s);
    PreArgs a{o, dout, delta, rows_q(s) * s->num_heads_q, s->num_heads_q, s->seqlen_q, s->total_q, varlen(s),
              s->head_dim, to_kernel(d.o), to_kernel(d.dout), reinterpret_cast<u32x4*>(zero),
              (long long)(zero_bytes / 16)};
    launch_preprocess(a, s->dtype, padded_hd(s), hs);
    if (s->dq_algo == ATTN_DQ_STORED_DS && varlen(s))
        launch_ds_table(s->cu_seqlens_q, s->batch, s->seqlen_q, s->total_q,
                        reinterpret_cast<int*>(reinterpret_cast<char*>(workspace) + accum_bytes(s) + sem_bytes(s) +
                                               kErrBytes),
                        hs);
}

// dq_out: the separate and stored-dS modes write dQ = T(dq_scale * sum)
// there instead of to the accumulator (null: the accumulator)
void enqueue_bwd(const attn_shape_t* s, const void* q, const void* k, const void* v, const void* dout,
                 const float* lse, const float* delta, void* workspace, void* dk, void* dv, void* dq_out,
                 float dq_scale, hipStream_t hs) {
    char* ws = reinterpret_cast<char*>(workspace);
    BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq_acc = reinterpret_cast<float*>(ws);
    a.sem = reinterpret_cast<int*>(ws + accum_bytes(s));
    a.err = reinterpret_cast<int*>(ws + accum_bytes(s) + sem_bytes(s));
    a.dk = dk;
    a.dv = dv;
    a.cu_q = s->cu_seqlens_q;
    a.cu_k = s->cu_seqlens_k;
    a.used_q = s->seqused_q;
    a.used_k = s->seqused_k;
    a.batch = s->batch;
    a.hq = s->num_heads_q;
    a.hkv = s->num_heads_kv;
    a.seqlen_q = s->seqlen_q;
    a.seqlen_k = s->seqlen_k;
    a.total_q = s->total_q;
    a.total_k = s->total_k;
    a.nblk_n = (s->seqlen_k + kBwdBlockN - 1) / kBwdBlockN;
    a.nblk_m = nblk_m(s);
    a.scale = s->softmax_scale;
    a.deterministic = s->deterministic;
    a.win_lo = win_lo(s);
    a.win_hi = win_hi(s);
    a.alibi = s->alibi_slopes;
    a.dq_out = s->dq_algo == ATTN_DQ_ATOMIC ? nullptr : dq_out;
    a.dq_scale = dq_scale;
    const attn_strides_t d = strides_of(s);
    a.d = s->head_dim;
    a.sq = to_kernel(d.q);
    a.sk = to_kernel(d.k);
    a.sv = to_kernel(d.v);
    a.sdo = to_kernel(d.dout);
    a.sdq = to_kernel(d.dq);
    a.sdk = to_kernel(d.dk);
    a.sdv = to_kernel(d.dv);
    a.bias = s->bias;
    a.dbias = s->dbias;
    a.sbias = to_kernel(s->bias_strides);
    a.sdbias = to_kernel(s->dbias_strides);
    if (s->dq_algo == ATTN_DQ_STORED_DS) {
        char* tab = ws + accum_bytes(s) + sem_bytes(s) + kErrBytes;
        a.ds_qb_base = varlen(s) ? reinterpret_cast<const int*>(tab) : nullptr;
        a.ds = tab + ds_table_bytes(s);
        a.ds_qb = ds_qb(s);
        a.ds_nn = ds_nn(s);
    }
    // dBias blocks the kernel does not visit (masked tiles) must read zero
    if (s->dbias != nullptr) launch_zero_blocks(s->dbias, a.sdbias, s->dtype, a, hs);
    launch_bwd(a, s->dtype, padded_hd(s), masked(s), s->dq_algo, hs);
    if (s->dq_algo == ATTN_DQ_SEPARATE) {
        BwdArgs e = a;
        e.nblk_m = (s->seqlen_q + bwd_dq_block_m() - 1) / bwd_dq_block_m();
        launch_bwd_dq(e, s->dtype, padded_hd(s), masked(s), hs);
    } else if (s->dq_algo == ATTN_DQ_STORED_DS) {
        launch_bwd_dq_gemm(a, s->dtype, padded_hd(s), masked(s), hs);
    }
}

void enqueue_postprocess(const attn_shape_t* s, const void* workspace, void* dq, float scale, hipStream_t hs) {
    PostArgs a{reinterpret_cast<const float*>(workspace), dq, rows_q(s) * s->num_heads_q, s->num_heads_q,
               s->seqlen_q, s->total_q, varlen(s), scale, s->cu_seqlens_q, s->seqused_q, s->batch,
               s->head_dim, to_kernel(strides_of(s).dq)};
    launch_postprocess(a, s->dtype, padded_hd(s), hs);
}

}  // namespace

extern "C" {

int attn_bwd_preprocess(const attn_shape_t* s, const void* o, const void* dout, float* delta, void* workspace,
                        size_t workspace_size, void* stream) {
    int st = validate_shape(s);
    if (st) return st;
    if (!o || !dout || !delta || !workspace) return ATTN_ERR_NULL_ARG;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(delta) || !aligned16(workspace)) return ATTN_ERR_MISALIGNED;
    if (workspace_size < workspace_bytes(s)) return ATTN_ERR_BAD_SHAPE;
    (void)hipGetLastError();   // clear a stale error so the check below is ours
    enqueue_preprocess(s, o, dout, delta, workspace, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

int attn_bwd(const attn_shape_t* s, const void* q, const void* k, const void* v, const void* dout, const float* lse,
             const float* delta, void* workspace, size_t workspace_size, void* dk, void* dv, void* stream) {
    int st = validate_bwd(s);
    if (st) return st;
    if (!q || !k || !v || !dout || !lse || !delta || !workspace || !dk || !dv) return ATTN_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
        !aligned16(delta) || !aligned16(workspace) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_MISALIGNED;
    if (workspace_size < workspace_bytes(s)) return ATTN_ERR_BAD_SHAPE;
    (void)hipGetLastError();   // clear a stale error so the check below is ours
    enqueue_bwd(s, q, k, v, dout, lse, delta, workspace, dk, dv, nullptr, 0.f, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

int attn_bwd_dq_postprocess(const attn_shape_t* s, const void* workspace, size_t workspace_size, void* dq,
                            float scale, void* stream) {
    int st = validate_shape(s);
    if (st) return st;
    if (!workspace || !dq) return ATTN_ERR_NULL_ARG;
    if (!aligned16(workspace) || !aligned16(dq)) return ATTN_ERR_MISALIGNED;
    if (workspace_size < workspace_bytes(s)) return ATTN_ERR_BAD_SHAPE;
    (void)hipGetLastError();   // clear a stale error so the check below is ours
    enqueue_postprocess(s, workspace, dq, scale, reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

int attn_bwd_full(const attn_shape_t* s, const void* q, const void* k, const void* v, const void* dout,
                  const float* lse, const float* delta, void* workspace, size_t workspace_size, void* dq, void* dk,
                  void* dv, void* stream) {
    int st = validate_bwd(s);
    if (st) return st;
    if (!q || !k || !v || !dout || !lse || !delta || !workspace || !dq || !dk || !dv) return ATTN_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
        !aligned16(delta) || !aligned16(workspace) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_MISALIGNED;
    if (workspace_size < workspace_bytes(s)) return ATTN_ERR_BAD_SHAPE;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // clear a stale error so the check below is ours
    enqueue_bwd(s, q, k, v, dout, lse, delta, workspace, dk, dv, dq, s->softmax_scale, hs);
    if (s->dq_algo == ATTN_DQ_ATOMIC) enqueue_postprocess(s, workspace, dq, s->softmax_scale, hs);
    return check_launch();
}

}  // extern "C"
