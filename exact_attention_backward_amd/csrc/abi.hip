// C ABI of the library: argument validation, workspace layout and dispatch.
// Every entry point validates before any HIP call, so the error paths run
// (and are tested) on machines without a GPU.
#include <stdint.h>
#include <stddef.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "launch.h"

using namespace attn;

// Scratch memory of the no-allocation entry point (see scratch_base below).
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

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
    if (s->head_dim < 8 || s->head_dim > 256 || s->head_dim % 8 != 0) return ATTN_ERR_UNSUPPORTED;
    if (s->head_dim > 128 && s->dtype == ATTN_DTYPE_F32) return ATTN_ERR_UNSUPPORTED;
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
    if (s->max_workspace_bytes < 0) return ATTN_ERR_BAD_SHAPE;
    if (!(s->dropout_p >= 0.f && s->dropout_p < 1.f)) return ATTN_ERR_BAD_SHAPE;   // NaN included
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

// The dQ mode the kernels run: above head dim 128 the atomic mode runs as
// the separate one (the key-stationary kernel that adds dQ with atomics keeps
// a K/V tile per wave in registers, which does not fit at 256).
int algo_of(const attn_shape_t* s) {
    return s->dq_algo == ATTN_DQ_ATOMIC && s->head_dim > 128 ? ATTN_DQ_SEPARATE : s->dq_algo;
}

// the backward entry points: outside the atomic dQ mode the kernels copy
// the bias in 16-byte chunks (rows, batch and head steps and the base
// 16-byte aligned) and address a tile of up to 64 bias or dBias rows with
// 32-bit offsets
int validate_bwd(const attn_shape_t* s) {
    const int st = validate_shape(s);
    if (st) return st;
    if (algo_of(s) != ATTN_DQ_ATOMIC) {
        const long long esz = s->dtype == ATTN_DTYPE_F32 ? 4 : 2;
        if (s->bias != nullptr) {
            const attn_tensor_strides_t& b = s->bias_strides;
            if (reinterpret_cast<uintptr_t>(s->bias) % 16 || (b.batch * esz) % 16 || (b.head * esz) % 16 ||
                (b.row * esz) % 16)
                return ATTN_ERR_MISALIGNED;
        }
        const attn_tensor_strides_t* bs[] = {&s->bias_strides, &s->dbias_strides};
        const void* bp[] = {s->bias, s->dbias};
        for (int t = 0; t < 2; ++t)
            if (bp[t] != nullptr && (65 * bs[t]->row + s->seqlen_k + 8) * esz >= kOobOff - (1LL << 20))
                return ATTN_ERR_BAD_SHAPE;
    }
    return ATTN_OK;
}

bool varlen(const attn_shape_t* s) { return s->cu_seqlens_q != nullptr; }

// The kernels' dropout parameters: keep iff the random byte >= round(256 p)
// (at most 255), kept values scaled by 1 / (1 - p).
Dropout dropout_args(const attn_shape_t* s) {
    Dropout d{};
    if (s->dropout_p > 0.f) {
        const double p = s->dropout_p;
        d.on = 1;
        d.thr = (unsigned)std::min(255.0, std::floor(256.0 * p + 0.5));
        d.k0 = (unsigned)(s->dropout_seed & 0xffffffffu);
        d.k1 = (unsigned)(s->dropout_seed >> 32);
        d.off = s->dropout_offset;
        d.rp = (float)(1.0 / (1.0 - p));
    }
    return d;
}

// the head dim the kernels tile with: head_dim rounded up to 64, 128 or 256
int padded_hd(const attn_shape_t* s) { return s->head_dim <= 64 ? 64 : s->head_dim <= 128 ? 128 : 256; }

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
// ---- stored-dS mode: [block table][dS blocks]
// Query rows per tile of the dK/dV kernel (its dS blocks come per tile).
int ds_bm(const attn_shape_t* s) { return kv_block_m(padded_hd(s)); }
// Entries of the per-query-tile table: every sequence's tiles.
long long ds_tiles(const attn_shape_t* s) {
    const int bm = ds_bm(s);
    if (varlen(s)) return (long long)s->total_q / bm + s->batch;
    return (long long)s->batch * ((s->seqlen_q + bm - 1) / bm);
}
// dS blocks of one sequence: the blocks of each query tile's visiting key tiles
long long ds_seq_blocks(const attn_shape_t* s, int len_q, int len_k) {
    const int bm = ds_bm(s);
    long long n = 0;
    for (int m = 0; m * bm < len_q; ++m) n += ds_tile_blocks(m, bm, len_q, len_k, win_lo(s), win_hi(s), masked(s));
    return n;
}
// dS blocks per q-head: exact for dense problems and for varlen ones whose
// offsets the caller also gave in host memory (without used lengths); else
// the bound of every sequence's full rectangle of 32-row and 128-key blocks,
// sum_b (len_b / 32 + blocks per tile) * ceil(seqlen_k / 128)
long long ds_head_blocks(const attn_shape_t* s) {
    if (!varlen(s)) return (long long)s->batch * ds_seq_blocks(s, s->seqlen_q, s->seqlen_k);
    if (s->cu_seqlens_q_host != nullptr && s->cu_seqlens_k_host != nullptr && s->seqused_q == nullptr &&
        s->seqused_k == nullptr) {
        long long n = 0;
        for (int b = 0; b < s->batch; ++b) {
            // clamped as the kernels clamp the device offsets
            const int* cq = s->cu_seqlens_q_host;
            const int* ck = s->cu_seqlens_k_host;
            int q0 = std::min(std::max(cq[b], 0), s->total_q), q1 = std::min(std::max(cq[b + 1], q0), s->total_q);
            int k0 = std::min(std::max(ck[b], 0), s->total_k), k1 = std::min(std::max(ck[b + 1], k0), s->total_k);
            n += ds_seq_blocks(s, std::min(q1 - q0, s->seqlen_q), std::min(k1 - k0, s->seqlen_k));
        }
        return n;
    }
    const long long per_tile = ds_bm(s) / kDsRows;
    return ((long long)s->total_q / kDsRows + per_tile * s->batch) * ((s->seqlen_k + kDsKeys - 1) / kDsKeys);
}

// How attn_bwd runs for a shape: the dQ mode after the workspace cap
// (max_workspace_bytes) and, for the stored-dS mode, the kv-heads per
// launch (their q-heads' dS fits the workspace at once).
struct Plan {
    int algo;
    int chunk;            // kv-heads per launch (stored dS), else all
    long long head_blocks;   // stored dS: blocks per q-head
};
size_t base_bytes(const attn_shape_t* s, int algo, bool with_accum);
Plan plan(const attn_shape_t* s) {
    Plan p{algo_of(s), s->num_heads_kv, 0};
    if (p.algo != ATTN_DQ_STORED_DS) return p;
    p.head_blocks = ds_head_blocks(s);
    // block indices are int32 in the table (a q-head's dS past 2^31 blocks,
    // 16 TiB, could not be allocated anyway): the separate mode instead
    if (p.head_blocks > 0x7fffffffLL) return Plan{ATTN_DQ_SEPARATE, s->num_heads_kv, 0};
    const int G = s->num_heads_q / s->num_heads_kv;
    const double per_kv = (double)G * (double)p.head_blocks * kDsBlockBytes;   // bytes of one kv-head group
    if (s->max_workspace_bytes > 0) {
        const double avail = (double)s->max_workspace_bytes - (double)base_bytes(s, ATTN_DQ_STORED_DS, true);
        const double fit = avail > 0 ? std::floor(avail / std::max(per_kv, 1.0)) : 0.0;
        p.chunk = (int)std::min<double>(s->num_heads_kv, fit);
        if (p.chunk < 1) p = Plan{ATTN_DQ_SEPARATE, s->num_heads_kv, 0};   // not even one group fits
    }
    return p;
}
size_t ds_table_bytes(const attn_shape_t* s, int algo) {
    return algo == ATTN_DQ_STORED_DS ? align_up((size_t)(s->batch + 1 + ds_tiles(s)) * sizeof(int32_t)) : 0;
}
size_t ds_bytes(const attn_shape_t* s, const Plan& p) {
    if (p.algo != ATTN_DQ_STORED_DS) return 0;
    const int G = s->num_heads_q / s->num_heads_kv;
    return (size_t)p.chunk * G * (size_t)p.head_blocks * kDsBlockBytes;
}
// everything but the dS blocks
size_t base_bytes(const attn_shape_t* s, int algo, bool with_accum) {
    return (with_accum ? accum_bytes(s) : 0) + sem_bytes(s) + kErrBytes + ds_table_bytes(s, algo);
}
size_t workspace_bytes(const attn_shape_t* s) {
    const Plan p = plan(s);
    return base_bytes(s, p.algo, true) + ds_bytes(s, p);
}

// Byte offsets of the workspace parts from the workspace base.  The entry
// points that take a workspace use the full layout; the no-allocation entry
// point (attn_bwd_full only) leaves the accumulator out unless dQ is added
// atomically, since the other dQ passes write dQ straight to the output.
struct Layout {
    Plan p;
    size_t accum, sem, err, tab, ds, total;
};
Layout layout(const attn_shape_t* s, bool with_accum) {
    Layout l;
    l.p = plan(s);
    l.accum = 0;
    l.sem = with_accum ? accum_bytes(s) : 0;
    l.err = l.sem + sem_bytes(s);
    l.tab = l.err + kErrBytes;
    l.ds = l.tab + ds_table_bytes(s, l.p.algo);
    l.total = l.ds + ds_bytes(s, l.p);
    return l;
}

int check_launch() {
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// ---- scratch memory of attn_bwd_full_noalloc: a static device array, one
// copy per GPU, held from the library's load on that GPU to the process end.
// In host code the array's name is not a device address; its address on
// each device is looked up once, with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};

int scratch_base(char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
        g_scratch[dev] = reinterpret_cast<char*>(p);
    }
    *out = g_scratch[dev];
    return ATTN_OK;
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
        case ATTN_ERR_SCRATCH: return "problem needs more than the no-allocation entry point's scratch memory";
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
    a.drop = dropout_args(s);
    // the MFMA forward for the 16-bit types; fp32 takes the plain one
    if (s->dtype != ATTN_DTYPE_F32)
        launch_fwd_mfma(a, s->dtype, padded_hd(s), masked(s), reinterpret_cast<hipStream_t>(stream));
    else
        launch_fwd(a, s->dtype, padded_hd(s), masked(s), reinterpret_cast<hipStream_t>(stream));
    return check_launch();
}

}  // extern "C"

namespace {

// The enqueue steps behind the entry points; arguments already validated.

// Kernel arguments shared by the backward kernels and the dS table kernel:
// problem, workspace parts and, for the stored-dS mode, its table and blocks.
BwdArgs bwd_args(const attn_shape_t* s, const Layout& l, void* workspace) {
    char* ws = reinterpret_cast<char*>(workspace);
    BwdArgs a{};
    a.dq_acc = reinterpret_cast<float*>(ws + l.accum);
    a.sem = reinterpret_cast<int*>(ws + l.sem);
    a.err = reinterpret_cast<int*>(ws + l.err);
    a.cu_q = s->cu_seqlens_q;
    a.cu_k = s->cu_seqlens_k;
    a.used_q = s->seqused_q;
    a.used_k = s->seqused_k;
    a.batch = s->batch;
    a.hq = s->num_heads_q;
    a.hkv = s->num_heads_kv;
    a.hkv0 = 0;
    a.hkv_n = s->num_heads_kv;
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
    a.drop = dropout_args(s);
    if (l.p.algo == ATTN_DQ_STORED_DS) {
        a.ds_tile_base = reinterpret_cast<const int*>(ws + l.tab);
        a.ds_prefix = a.ds_tile_base + s->batch + 1;
        a.ds_ntiles = (int)ds_tiles(s);
        a.ds_head_blocks = l.p.head_blocks;
        a.ds = ws + l.ds;
    }
    return a;
}

void enqueue_preprocess(const attn_shape_t* s, const Layout& l, const void* o, const void* dout, float* delta,
                        void* workspace, hipStream_t hs) {
    // the preprocess kernel also clears the counters and status words, and
    // the accumulator where it is added into (atomic modes); the dS blocks
    // are written before they are read
    const bool atomic = l.p.algo == ATTN_DQ_ATOMIC;
    char* zero = reinterpret_cast<char*>(workspace) + (atomic ? l.accum : l.sem);
    const size_t zero_bytes = l.tab - (atomic ? l.accum : l.sem);
    const attn_strides_t d = strides_of(s);
    PreArgs a{o, dout, delta, rows_q(s) * s->num_heads_q, s->num_heads_q, s->seqlen_q, s->total_q, varlen(s),
              s->head_dim, to_kernel(d.o), to_kernel(d.dout), reinterpret_cast<u32x4*>(zero),
              (long long)(zero_bytes / 16)};
    if (l.p.algo == ATTN_DQ_STORED_DS) {
        const BwdArgs t = bwd_args(s, l, workspace);
        launch_preprocess(a, s->dtype, padded_hd(s), &t, ds_bm(s), masked(s), hs);
    } else {
        launch_preprocess(a, s->dtype, padded_hd(s), nullptr, 0, false, hs);
    }
}

// ---- a second stream per device for the separate mode's dQ kernel, which
// needs neither the dK/dV kernel nor its outputs: on small problems, where
// neither kernel fills the GPU alone, the two run side by side (8% on B=2
// H=8 S=1024 D=64; on the full-size shapes 0.5-1.5% slower, so they keep
// one stream: side_worth).  (The masked-dBias clear stays on the caller's
// stream, ahead of the kernels: beside them it gained 1%, but a masked
// element inside a visited tile then got the clear's +0 or the kernel's
// -0 (P = 0 times a negative dP - D) depending on timing.)  The side stream is
// forked from the caller's stream after the work enqueued so far and joined
// back before the call returns, so to the caller everything stays ordered on
// its own stream.  Created once per device (default priority, non-blocking),
// held until the process ends; the fork/join pairs of concurrent callers are
// serialised so that each wait sees its own record.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// whether the dK/dV kernel leaves most of the GPU idle: at most one key
// tile (of 128 keys) per compute unit over all (sequence, kv-head) groups
// (its workgroups take two tiles each under a causal mask)
bool side_worth(const attn_shape_t* s) {
    constexpr long long kComputeUnits = 256;
    const long long tiles = (long long)((s->seqlen_k + 127) / 128) * s->num_heads_kv * s->batch;
    return tiles <= kComputeUnits;
}

// under g_side_mu.  Not created while `hs` is being captured into a graph
// (the call then runs on the caller's stream alone).
int side_stream(hipStream_t hs, SideStream** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
    SideStream& ss = g_side[dev];
    if (ss.s == nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(hs, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return ATTN_ERR_HIP;
        hipStream_t st = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return ATTN_ERR_HIP;
        if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
            if (f) (void)hipEventDestroy(f);
            (void)hipStreamDestroy(st);
            return ATTN_ERR_HIP;
        }
        ss.s = st;
        ss.fork = f;
        ss.join = j;
    }
    *out = &ss;
    return ATTN_OK;
}

// dq_out: the separate and stored-dS modes write dQ = T(dq_scale * sum)
// there instead of to the accumulator (null: the accumulator).  side: the
// separate mode may use the side stream (not for the no-allocation entry
// point, which creates nothing)
void enqueue_bwd(const attn_shape_t* s, const Layout& l, const void* q, const void* k, const void* v,
                 const void* dout, const float* lse, const float* delta, void* workspace, void* dk, void* dv,
                 void* dq_out, float dq_scale, hipStream_t hs, bool side) {
    BwdArgs a = bwd_args(s, l, workspace);
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dk = dk;
    a.dv = dv;
    a.dq_out = l.p.algo == ATTN_DQ_ATOMIC ? nullptr : dq_out;
    a.dq_scale = dq_scale;
    // masked dBias elements read zero (the kernels write the visible ones,
    // and the masked ones of the tiles they visit, after this)
    if (s->dbias != nullptr && masked(s)) launch_zero_masked(s->dbias, a.sdbias, s->dtype, a, hs);
    // on small problems the separate mode's dQ kernel runs on the side
    // stream (when there is one to take)
    const bool sep_side = l.p.algo == ATTN_DQ_SEPARATE && side_worth(s);
    std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
    SideStream* ss = nullptr;
    if (side && sep_side) {
        lock.lock();
        if (side_stream(hs, &ss) != ATTN_OK || hipEventRecord(ss->fork, hs) != hipSuccess ||
            hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
            ss = nullptr;   // one after the other on the caller's stream
    }
    const hipStream_t aux = ss != nullptr ? ss->s : hs;
    if (l.p.algo == ATTN_DQ_STORED_DS) {
        // kv-head groups in chunks whose dS fits the workspace: the dK/dV
        // kernel stores the chunk's dS, the dQ pass consumes it
        for (int h0 = 0; h0 < s->num_heads_kv; h0 += l.p.chunk) {
            a.hkv0 = h0;
            a.hkv_n = std::min(l.p.chunk, s->num_heads_kv - h0);
            launch_bwd(a, s->dtype, padded_hd(s), masked(s), ATTN_DQ_STORED_DS, hs);
            launch_bwd_dq_gemm(a, s->dtype, padded_hd(s), masked(s), hs);
        }
    } else if (l.p.algo == ATTN_DQ_SEPARATE) {
        BwdArgs e = a;
        e.nblk_m = (s->seqlen_q + bwd_dq_block_m() - 1) / bwd_dq_block_m();
        if (sep_side && ss != nullptr) {
            launch_bwd_dq(e, s->dtype, padded_hd(s), masked(s), aux);
            launch_bwd(a, s->dtype, padded_hd(s), masked(s), l.p.algo, hs);
        } else {
            launch_bwd(a, s->dtype, padded_hd(s), masked(s), l.p.algo, hs);
            launch_bwd_dq(e, s->dtype, padded_hd(s), masked(s), hs);
        }
    } else {
        launch_bwd(a, s->dtype, padded_hd(s), masked(s), l.p.algo, hs);
    }
    if (ss != nullptr) {
        (void)hipEventRecord(ss->join, ss->s);   // a failure here is left for check_launch
        (void)hipStreamWaitEvent(hs, ss->join, 0);
    }
}

void enqueue_postprocess(const attn_shape_t* s, const Layout& l, const void* workspace, void* dq, float scale,
                         hipStream_t hs) {
    PostArgs a{reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) + l.accum), dq, rows_q(s) * s->num_heads_q, s->num_heads_q,
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
    enqueue_preprocess(s, layout(s, true), o, dout, delta, workspace, reinterpret_cast<hipStream_t>(stream));
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
    enqueue_bwd(s, layout(s, true), q, k, v, dout, lse, delta, workspace, dk, dv, nullptr, 0.f,
                reinterpret_cast<hipStream_t>(stream), true);
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
    enqueue_postprocess(s, layout(s, true), workspace, dq, scale, reinterpret_cast<hipStream_t>(stream));
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
    const Layout l = layout(s, true);
    enqueue_bwd(s, l, q, k, v, dout, lse, delta, workspace, dk, dv, dq, s->softmax_scale, hs, true);
    if (l.p.algo == ATTN_DQ_ATOMIC) enqueue_postprocess(s, l, workspace, dq, s->softmax_scale, hs);
    return check_launch();
}

int attn_bwd_full_noalloc(const attn_shape_t* s, const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv, void* stream) {
    int st = validate_bwd(s);
    if (st) return st;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(lse) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_MISALIGNED;
    // scratch = [D, fp32 in the LSE layout][workspace without the accumulator
    // unless dQ is added atomically]
    const size_t d_bytes = align_up((size_t)rows_q(s) * s->num_heads_q * sizeof(float));
    const Layout l = layout(s, plan(s).algo == ATTN_DQ_ATOMIC);
    if (d_bytes + l.total > kScratchBytes) return ATTN_ERR_SCRATCH;
    char* base = nullptr;
    st = scratch_base(&base);
    if (st) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // clear a stale error so the check below is ours
    float* delta = reinterpret_cast<float*>(base);
    void* ws = base + d_bytes;
    enqueue_preprocess(s, l, o, dout, delta, ws, hs);
    enqueue_bwd(s, l, q, k, v, dout, lse, delta, ws, dk, dv, dq, s->softmax_scale, hs, false);
    if (l.p.algo == ATTN_DQ_ATOMIC) enqueue_postprocess(s, l, ws, dq, s->softmax_scale, hs);
    return check_launch();
}

}  // extern "C"
