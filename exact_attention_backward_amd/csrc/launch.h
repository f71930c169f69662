// Kernel argument blocks, element load/store helpers and launcher prototypes
// shared by the kernel sources and the C ABI layer.
#pragma once

#include "common.h"

#include <type_traits>

namespace attn {

// Element strides of one tensor: between batch entries (dense layouts only),
// rows (tokens) and heads; the head dimension is contiguous.
struct Strides {
    long long b, r, h;
};

// Offset of a sequence's first row: its batch entry (dense) or its packed
// first row q0 (varlen).
__host__ __device__ __forceinline__ long long seq_off(const Strides& s, bool varlen, int b, int q0) {
    return varlen ? (long long)q0 * s.r : (long long)b * s.b;
}
// Offset of flattened row r (b * S + i dense, the packed row varlen).
__host__ __device__ __forceinline__ long long flat_row_off(const Strides& s, bool varlen, long long r, int S) {
    if (varlen) return r * s.r;
    const long long b = r / S;
    return b * s.b + (r - b * S) * s.r;
}

// Dropout of P (drop iff the element's random byte < thr; kept values are
// scaled by rp = 1 / (1 - p)): the Philox4x32-10 key (k0, k1), the fourth
// counter word, and on = 0 when there is no dropout.  See drop_block.
struct Dropout {
    int on;
    unsigned thr, k0, k1, off;
    float rp;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* used_q;   // varlen: per-sequence used lengths, or null
    const int32_t* used_k;
    int batch, hq, hkv, seqlen_q, seqlen_k, total_q, total_k;
    float scale;
    int win_lo, win_hi;      // visibility: i + off - win_lo <= j <= i + off + win_hi
    const float* alibi;      // per q-head ALiBi slopes, or null
    int d;                   // head dim (the kernels' HD is this rounded up to 64 or 128)
    Strides sq, sk, sv, so;
    const void* bias;        // elementwise bias [b, h, i, j] (I/O type), or null
    Strides sbias;           // its batch, row and head strides (columns contiguous)
    Dropout drop;
};

struct PreArgs {
    const void* o;
    const void* dout;
    float* delta;
    long long rows;      // flattened rows of O times heads
    int h, s;            // heads, dense sequence length
    long long total;     // varlen total rows
    bool varlen;
    int d;               // head dim
    Strides so, sdo;
    u32x4* zero;         // workspace words the kernel also clears (16-byte units), n16 of them
    long long n16;
};

struct PostArgs {
    const float* acc;
    void* dq;
    long long rows;
    int h, s;
    long long total;
    bool varlen;
    float scale;
    // varlen with used lengths: rows past a sequence's used length are skipped
    const int32_t* cu_q;
    const int32_t* used_q;
    int batch;
    int d;               // head dim
    Strides sdq;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* delta;
    float* dq_acc;       // fp32 [B, Hq, Sq, D] or [Hq, total_q, D]
    int* sem;            // deterministic mode: one counter per (sequence, q-head, query tile)
    int* err;            // deterministic mode: set when an ordered wait gave up
    void* dk;
    void* dv;
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* used_q;   // varlen: per-sequence used lengths, or null
    const int32_t* used_k;
    int batch, hq, hkv, seqlen_q, seqlen_k, total_q, total_k;
    // visibility of key j to query i (off = len_k - len_q, bottom-right
    // aligned): i + off - win_lo <= j <= i + off + win_hi; kNoWindow on an
    // unbounded side.  Kernels instantiated with MASKED = false (no bound at
    // all) ignore them.
    int win_lo, win_hi;
    // ALiBi: logit - slope[q-head] |i + off - j| (natural-log units), or null
    const float* alibi;
    // dQ passes that own whole rows (separate, stored dS): when set, dQ goes
    // straight to this [rows, Hq, D] tensor of the I/O type as
    // T(dq_scale * sum), the product rounded to fp32 first, instead of to
    // the fp32 accumulator
    void* dq_out;
    float dq_scale;
    int d;               // head dim (the kernels' HD is this rounded up to 64 or 128;
                         // columns from d on are zero in every tile)
    Strides sq, sk, sv, sdo, sdq, sdk, sdv;
    // elementwise bias [b, h, i, j] added to the logits and its gradient dS,
    // or null; batch, row and head strides
    const void* bias;
    void* dbias;
    Strides sbias, sdbias;
    Dropout drop;
    int nblk_n;          // key tiles per sequence (of the longest sequence)
    int nblk_m;          // query tiles per sequence (of the longest sequence)
    float scale;
    int deterministic;
    // stored-dS mode: the dS blocks (32 x 128 of the 16-bit I/O type each) of
    // the q-heads of this launch's kv-head chunk, ds_head_blocks blocks per
    // q-head; within a q-head, query tile m of sequence b holds its
    // (BM / 32) x cnt(m) blocks (see ds_key_range) from block
    // ds_prefix[ds_tile_base[b] + m] on (-1: none stored), 32-row block r
    // and key tile n at + r * cnt(m) + n - N0(m)
    void* ds;
    const int* ds_tile_base;   // [batch + 1]: each sequence's first entry of ds_prefix
    const int* ds_prefix;      // [ds_ntiles]
    int ds_ntiles;
    long long ds_head_blocks;
    // kv-heads hkv0 .. hkv0 + hkv_n - 1 only (a chunk of the problem's
    // kv-heads: the launch's grid covers these groups; the stored-dS region
    // starts at q-head hkv0 * Hq / Hkv)
    int hkv0, hkv_n;
    // masked launches of the dK/dV and dQ kernels: 1 = a workgroup takes two
    // tiles of complementary cost (p and last - p), 0 = one tile each (set
    // by each launcher: pairs only when single tiles would outnumber the
    // compute units, since on a small grid a pair doubles the longest
    // workgroup's work)
    int pair_tiles;
};

constexpr int kComputeUnits = 256;   // of an MI355X

// dS blocks of the stored-dS mode: 32 query rows x 128 keys of bf16 or fp16 (8 KiB),
// in the register order of the key-stationary kernel's MFMA operands: 16-byte
// chunk (g, l) for g = 2 p + c (keys 32p .. 32p + 31, rows 16c .. 16c + 15)
// holds key 32 p + l % 32, rows 16c + 4 (l / 32) + 0..3 and
// 16c + 8 + 4 (l / 32) + 0..3.  The chunk of lane l sits at slot ds_chunk(g, l)
// (lanes 32..63 are moved by four chunks, so that the dQ pass's transposing
// reads of keys k and k + 32 lanes apart hit different LDS banks).
constexpr int kDsRows = 32;
constexpr int kDsKeys = 128;
constexpr int kDsBlockBytes = kDsRows * kDsKeys * 2;
__host__ __device__ constexpr int ds_chunk(int g, int l) { return g * 64 + (l ^ ((l >> 5) << 2)); }

// Query rows per tile of the stored-dS dK/dV kernel (kDsRows-row blocks each).
__host__ __device__ constexpr int kv_block_m(int hd) { return hd >= 128 ? 32 : 64; }

// The key tiles (kDsKeys keys each) whose dS the key-stationary kernel stores
// for query tile m (bm rows) of a sequence with len_q query and len_k key
// rows: exactly those that visit the tile, a contiguous run n0 .. n1 (n1 <
// n0: none).  Visibility: key j to row i iff i + off - lo <= j <= i + off +
// hi, off = len_k - len_q (masked); every key when !masked.  Shared by the
// host's workspace sizing, the table kernel and both dS kernels.
struct KeyRange {
    int n0, n1;
};
// 32-bit arithmetic: the ABI keeps every sequence below 2^27 rows and clamps
// window sizes to 2^29, so |x| and |y| below stay under 2^30.
__host__ __device__ inline KeyRange ds_key_range(int m, int bm, int len_q, int len_k, int lo, int hi, bool masked) {
    const int nblk = (len_k + kDsKeys - 1) / kDsKeys;
    if (!masked) return KeyRange{0, nblk - 1};
    const int off = len_k - len_q;
    // first: the smallest n whose last visible row reaches the tile's first row
    const int x = m * bm + off - lo + 1;   // need min((n + 1) kDsKeys, len_k) >= x
    if (x > len_k) return KeyRange{0, -1};
    const int n0 = x <= kDsKeys ? 0 : (x + kDsKeys - 1) / kDsKeys - 1;
    // last: the largest n whose first visible row is in or before the tile
    const int y = (m + 1) * bm - 1 + off + hi;   // need n kDsKeys <= y
    if (y < 0) return KeyRange{0, -1};
    return KeyRange{n0, y / kDsKeys < nblk - 1 ? y / kDsKeys : nblk - 1};
}
// dS blocks of query tile m: 32-row blocks per tile times the tile's key tiles
__host__ __device__ inline long long ds_tile_blocks(int m, int bm, int len_q, int len_k, int lo, int hi, bool masked) {
    const KeyRange r = ds_key_range(m, bm, len_q, len_k, lo, hi, masked);
    return r.n1 >= r.n0 ? (long long)(bm / kDsRows) * (r.n1 - r.n0 + 1) : 0;
}

// x * s rounded to fp32 and held in a register, so that a following
// conversion to fp16 rounds that fp32 value: the empty asm keeps the
// compiler from fusing the multiply into a mixed-precision
// multiply-and-convert (one rounding of the exact product instead of two).
__device__ __forceinline__ float mul_f32(float x, float s) {
    float y = x * s;
    asm volatile("" : "+v"(y));
    return y;
}

// An unbounded side of the visibility window (far beyond any sequence length).
constexpr int kNoWindow = 1 << 29;

// Query rows per tile of the main kernel (keys per tile are fixed at 128).
int bwd_block_m(int dtype, int head_dim);
constexpr int kBwdBlockN = 128;

void launch_fwd(const FwdArgs& a, int dtype, int hd, bool masked, hipStream_t st);
// the MFMA forward (bf16 and fp16, no elementwise bias)
void launch_fwd_mfma(const FwdArgs& a, int dtype, int hd, bool masked, hipStream_t st);
// zero every sequence's [Hq, len_q, len_k] block of a [b, h, i, j] tensor with strides s
void launch_zero_masked(void* p, const Strides& s, int dtype, const BwdArgs& a, hipStream_t st);
// table (stored-dS mode, else null): also build its block table (for query
// tiles of bm rows) in an extra workgroup
void launch_preprocess(const PreArgs& a, int dtype, int hd, const BwdArgs* table, int bm, bool masked,
                       hipStream_t st);
void launch_postprocess(const PostArgs& a, int dtype, int hd, hipStream_t st);
void launch_bwd(const BwdArgs& a, int dtype, int hd, bool masked, int dq_algo, hipStream_t st);
// dK/dV kernel for head dims above 128 (16-bit types, separate or stored-dS dQ)
void launch_bwd_kv_wide(const BwdArgs& a, int dtype, bool masked, bool store_ds, hipStream_t st);
// stored-dS mode: dQ = dS K from the stored blocks (16-bit types), and the
// per-sequence block table of varlen problems
void launch_bwd_dq_gemm(const BwdArgs& a, int dtype, int hd, bool masked, hipStream_t st);
// query-stationary dQ pass; a.nblk_m must count its query tiles (bwd_dq_block_m() rows each)
void launch_bwd_dq(const BwdArgs& a, int dtype, int hd, bool masked, hipStream_t st);
int bwd_dq_block_m();

// ---------------------------------------------------------------------------
// element access for the three I/O types
// ---------------------------------------------------------------------------
__device__ __forceinline__ float load_elem(const f16_t* p, long long i) { return (float)p[i]; }
__device__ __forceinline__ void store_elem(f16_t* p, long long i, float x) { p[i] = (f16_t)x; }
__device__ __forceinline__ void load8(const f16_t* p, float* x) {
    const f16x8 h = *reinterpret_cast<const f16x8*>(p);
    const f32x8 f = __builtin_convertvector(h, f32x8);
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = f[t];
}
__device__ __forceinline__ void store8(f16_t* p, const float* x) {
    const f32x8 f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    *reinterpret_cast<f16x8*>(p) = __builtin_convertvector(f, f16x8);
}
__device__ __forceinline__ float load_elem(const bf16_t* p, long long i) {
    return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}
__device__ __forceinline__ float load_elem(const float* p, long long i) { return p[i]; }
__device__ __forceinline__ void store_elem(bf16_t* p, long long i, float x) {
    p[i] = (bf16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}
__device__ __forceinline__ void store_elem(float* p, long long i, float x) { p[i] = x; }

__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        x[2 * t] = bf16_lo(w[t]);
        x[2 * t + 1] = bf16_hi(w[t]);
    }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        x[t] = u[t];
        x[4 + t] = v[t];
    }
}
// load8 with the non-temporal hint (data read once)
template <class T>
__device__ __forceinline__ void load8_nt(const T* p, float* x) {
    if constexpr (sizeof(T) == 2) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        if constexpr (std::is_same<T, f16_t>::value) {
            const f32x8 f = __builtin_convertvector(__builtin_bit_cast(f16x8, w), f32x8);
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = f[t];
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[2 * t] = bf16_lo(w[t]);
                x[2 * t + 1] = bf16_hi(w[t]);
            }
        }
    } else {
        const f32x4 u = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[t] = u[t];
            x[4 + t] = v[t];
        }
    }
}
__device__ __forceinline__ void store8(bf16_t* p, const float* x) {
    const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    *reinterpret_cast<u32x4*>(p) = w;
}
__device__ __forceinline__ void store8(float* p, const float* x) {
    const f32x4 u = {x[0], x[1], x[2], x[3]};
    const f32x4 v = {x[4], x[5], x[6], x[7]};
    *reinterpret_cast<f32x4*>(p) = u;
    *reinterpret_cast<f32x4*>(p + 4) = v;
}

}  // namespace attn
