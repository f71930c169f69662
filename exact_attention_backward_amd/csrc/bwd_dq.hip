// Query-stationary dQ pass of the attention backward for gfx950.
//
// One workgroup (4 waves) owns 128 query rows of one (sequence, q-head) and
// loops over 64-key tiles of K and V, recomputing for each tile
//   S^T  = K Q^T           (MFMA; K rows from LDS, Q rows of the wave in registers)
//   dP^T = V dO^T          (MFMA; V rows from LDS, dO rows in registers)
//   P    = exp2(S s log2e - LSE log2e),  dS = P (dP - D)
//   dQ  += dS K            (MFMA; dS straight from the S^T registers, K^T via
//                           transposing LDS reads)
// and writes its dQ rows once, with plain stores, into the fp32 accumulator
// (scaled and converted by the dQ postprocess).  This is the dQ half of the
// per-tile work of the Composable Kernel pipeline page
// "block_fmha_bwd_dq_dk_dv_pipeline_trload_kr_ktr_vr.hpp Source File" (stages
// 1, 2, 4, 5, 7), scheduled over keys instead of over queries so that no two
// workgroups add into the same dQ row: on MI355X fp32 atomics to device
// memory are executed memory-side, at about 1.3 TB/s, which bounds the
// key-stationary schedule's dQ accumulation far below the MFMA rate.
//
// Computing S^T (keys as rows) makes the lane of an accumulator own one query
// row and hold 8 keys per 16-key slice, which is exactly the layout of the dQ
// product's A operand (rows = queries, contraction over keys), so P and dS
// never leave the registers.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;

template <class T, int HD>
struct DqCfg {
    static constexpr int BQ = 32 * kWaves;   // query rows per workgroup
    static constexpr int BN = 32;            // keys per K/V tile
    // K/V tiles in the LDS ring (the copies of NS - 2 later tiles stay in
    // flight while one is consumed; at head dim 256 a tile's copies are
    // twice as many and the ring is three deep)
    static constexpr int NS = sizeof(T) == 2 ? (HD <= 128 ? 4 : 3) : 2;
    static constexpr int ROWB = HD * (int)sizeof(T);
    static constexpr int TILE = BN * ROWB;
    static constexpr int BUF_K = 0, BUF_V = TILE;
    static constexpr int BUF_BYTES = 2 * TILE;
    static constexpr int LDS_BYTES = NS * BUF_BYTES;
    // workgroups per CU: two for the 16-bit types up to head dim 128, else one
    static constexpr int WG_PER_CU = sizeof(T) == 2 && HD <= 128 ? 2 : 1;
    // elementwise bias: each wave's [32 rows][BN keys] block, two buffers
    // (tile parity), copied one tile ahead
    static constexpr int BIAS_W = 32 * BN * (int)sizeof(T);
    static constexpr int BIAS_ROWB = BN * (int)sizeof(T);
    static constexpr int BOPS = BIAS_W / 1024;       // copies per wave and tile
    static constexpr int OFF_BIAS = LDS_BYTES;
    static constexpr int LDS_BYTES_BIAS = OFF_BIAS + 2 * kWaves * BIAS_W;
    static_assert(LDS_BYTES_BIAS <= 160 * 1024 / WG_PER_CU, "LDS budget");
    static constexpr int NC = HD / 16;       // 16-wide chunks of the head dim
    static constexpr int NDB = HD / 32;      // 32-column blocks of the head dim
    static constexpr int NJB = BN / 32;      // 32-key blocks of a K tile
    static constexpr int NJC = BN / 16;      // 16-key chunks of a K tile
};

template <class T, int HD>
using DqOp = typename Elem<T>::op_t;

// Row-major operand: lane gets M[row][col .. col+7].
template <class T, int ROWB>
__device__ __forceinline__ DqOp<T, 0> dq_read_row(const char* lds, int row, int col) {
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(typename Elem<T>::op_t, lds_read16(lds, swz<ROWB>(row, col * 2)));
    } else {
        const f32x4 a = __builtin_bit_cast(f32x4, lds_read16(lds, swz<ROWB>(row, col * 4)));
        const f32x4 b = __builtin_bit_cast(f32x4, lds_read16(lds, swz<ROWB>(row, col * 4 + 16)));
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
}

// Column operand: lane (l32) gets M[r1 + t][c0 + l32] and M[r2 + t][c0 + l32], t = 0..3.
template <class T, int ROWB>
__device__ __forceinline__ DqOp<T, 0> dq_read_col(const char* lds, int r1, int r2, int c0, int lane) {
    if constexpr (sizeof(T) == 2) {
        const int s = lane & 15;
        const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
        const u32x2 x = lds_read_tr(lds, swz<ROWB>(r1 + (s >> 2), col * 2));
        const u32x2 y = lds_read_tr(lds, swz<ROWB>(r2 + (s >> 2), col * 2));
        const u32x4 w = {x[0], x[1], y[0], y[1]};
        return __builtin_bit_cast(typename Elem<T>::op_t, w);
    } else {
        const int col = c0 + (lane & 31);
        f32x8 r;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            r[t] = *reinterpret_cast<const float*>(lds + swz<ROWB>(r1 + t, col * 4));
            r[4 + t] = *reinterpret_cast<const float*>(lds + swz<ROWB>(r2 + t, col * 4));
        }
        return r;
    }
}

template <class T>
__device__ __forceinline__ DqOp<T, 0> dq_load_global(const T* p, bool ok) {
    if constexpr (sizeof(T) == 2) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok) w = *reinterpret_cast<const u32x4*>(p);
        return __builtin_bit_cast(typename Elem<T>::op_t, w);
    } else {
        f32x8 r = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (ok) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(p);
            const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
            r = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        }
        return r;
    }
}

// Per-lane plan of a K or V tile copy into its swizzled LDS image (see the
// key-stationary kernel): each wave fills 1 KiB segments with buffer loads
// whose lanes fetch the global chunk the swizzle puts in their slot.
template <int ROWB, int NROWS>
struct DqTileCopy {
    static constexpr int CPR = ROWB / 16;
    static constexpr int N = NROWS * CPR / 64 / kWaves;
    static_assert(NROWS * CPR % (64 * kWaves) == 0, "segment split");
    int voff[N];
    // stride_bytes: between rows in memory; valid: 16-byte chunks of a row
    // inside the head dim (the others read zeros)
    __device__ __forceinline__ void init(int w, int lane, int stride_bytes, int valid) {
#pragma unroll
        for (int t = 0; t < N; ++t) {
            const int slot = (w + t * kWaves) * 64 + lane;
            const int r = slot / CPR;
            const int c = (slot % CPR) ^ swz_key<ROWB>(r);
            voff[t] = c < valid ? r * stride_bytes + c * 16 : kOobOff;
        }
    }
    __device__ __forceinline__ void issue(i32x4 src, const char* lds, int w) const {
#pragma unroll
        for (int t = 0; t < N; ++t) dma_to_lds16(src, lds_addr(lds + (w + t * kWaves) * 1024), voff[t]);
    }
};

__device__ __forceinline__ void dq_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(n) for a run-time n in [0, 16): all but the n most
// recently issued VMEM operations are complete (gfx9 field layout).
__device__ __forceinline__ void dq_wait_vmem_but(int n) {
    switch (n) {
#define ATTN_VMCNT_CASE(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | 0x0F70); break;
        ATTN_VMCNT_CASE(0) ATTN_VMCNT_CASE(1) ATTN_VMCNT_CASE(2) ATTN_VMCNT_CASE(3)
        ATTN_VMCNT_CASE(4) ATTN_VMCNT_CASE(5) ATTN_VMCNT_CASE(6) ATTN_VMCNT_CASE(7)
        ATTN_VMCNT_CASE(8) ATTN_VMCNT_CASE(9) ATTN_VMCNT_CASE(10) ATTN_VMCNT_CASE(11)
        ATTN_VMCNT_CASE(12) ATTN_VMCNT_CASE(13) ATTN_VMCNT_CASE(14) ATTN_VMCNT_CASE(15)
#undef ATTN_VMCNT_CASE
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

}  // namespace

// dQ rows of query tile m (128 rows) of q-head hq in sequence b.  BIAS: an
// elementwise bias (and ALiBi too when slopes are given); DROP (with BIAS):
// dropout of P as well (dS = P (dP / (1 - p) - D) on kept, -P D on dropped
// elements).
template <class T, int HD, bool MASKED, bool ALIBI, bool BIAS, bool DROP>
__device__ __forceinline__ void dq_tile(int m, const BwdArgs& a, int b, int hq, int hkv, const SeqInfo& si,
                                        char* smem) {
    using C = DqCfg<T, HD>;
    using op_t = typename Elem<T>::op_t;
    constexpr int BQ = C::BQ, BN = C::BN;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int i0 = m * BQ;
    if (i0 >= si.len_q) return;
    const bool varlen = a.cu_q != nullptr;
    const int off = si.len_k - si.len_q;   // bottom-right alignment of the mask

    // key tiles any row of this tile can see: kt_b .. kt_b + n_kt - 1
    int key_end = si.len_k, kt_b = 0;
    if (MASKED) {
        key_end = min(key_end, min(i0 + BQ, si.len_q) - 1 + off + a.win_hi + 1);
        const int key_beg = i0 + off - a.win_lo;   // the first row's lower bound
        kt_b = key_beg > 0 ? key_beg / BN : 0;
    }
    const int n_kt = key_end > 0 ? max((key_end + BN - 1) / BN - kt_b, 0) : 0;

    const T* kg = reinterpret_cast<const T*>(a.k) + seq_off(a.sk, varlen, b, si.k0) + (long long)hkv * a.sk.h;
    const T* vg = reinterpret_cast<const T*>(a.v) + seq_off(a.sv, varlen, b, si.k0) + (long long)hkv * a.sv.h;

    const int valid = a.d * (int)sizeof(T) / 16;   // 16-byte chunks of a row inside the head dim
    DqTileCopy<C::ROWB, BN> kcopy, vcopy;
    kcopy.init(w, lane, (int)(a.sk.r * (long long)sizeof(T)), valid);
    vcopy.init(w, lane, (int)(a.sv.r * (long long)sizeof(T)), valid);
    constexpr int kOpsPerTile = 2 * DqTileCopy<C::ROWB, BN>::N;   // copies one wave issues per tile
    static_assert(kOpsPerTile * (C::NS - 2) < 16, "vmcnt range");
    // the u-th tile of the run (key tile kt_b + u) goes to ring buffer u % NS
    auto buf_of = [&](int u) { return smem + (u % C::NS) * C::BUF_BYTES; };
    auto issue_tile = [&](int u) {
        const int kt = kt_b + u;
        const int rows = min(si.len_k - kt * BN, BN);
        char* buf = buf_of(u);
        kcopy.issue(rsrc_words(kg + (long long)kt * BN * a.sk.r, (unsigned)(rows * a.sk.r * (long long)sizeof(T))),
                    buf + C::BUF_K, w);
        vcopy.issue(rsrc_words(vg + (long long)kt * BN * a.sv.r, (unsigned)(rows * a.sv.r * (long long)sizeof(T))),
                    buf + C::BUF_V, w);
    };

    // ---- this lane's query row: Q and dO rows as MFMA B operands, LSE and D
    const int i = i0 + 32 * w + l32;
    const bool row_ok = i < si.len_q;
    op_t qreg[C::NC], doreg[C::NC];
    {
        const T* qg = reinterpret_cast<const T*>(a.q) + seq_off(a.sq, varlen, b, si.q0) + (long long)hq * a.sq.h +
                      (long long)i * a.sq.r;
        const T* dog = reinterpret_cast<const T*>(a.dout) + seq_off(a.sdo, varlen, b, si.q0) +
                       (long long)hq * a.sdo.h + (long long)i * a.sdo.r;
#pragma unroll
        for (int c = 0; c < C::NC; ++c) {
            const bool ok = row_ok && 16 * c + 8 * h < a.d;
            qreg[c] = dq_load_global<T>(qg + 16 * c + 8 * h, ok);
            doreg[c] = dq_load_global<T>(dog + 16 * c + 8 * h, ok);
        }
    }
    const long long row0 = varlen ? (long long)hq * a.total_q + si.q0 : ((long long)b * a.hq + hq) * a.seqlen_q;
    float l2 = 0.f, dl = 0.f;
    if (row_ok) {
        const float lse = a.lse[row0 + i];
        l2 = lse == -INFINITY ? 0.f : lse * kLog2e;
        dl = a.delta[row0 + i];
    }
    const float scale2 = a.scale * kLog2e;
    // ALiBi slope of this q-head, negated, in log2 units
    const float nsl2 = ALIBI || (BIAS && a.alibi != nullptr) ? -a.alibi[hq] * kLog2e : 0.f;
    // key j is visible to this lane's row iff lim_lo <= j < lim
    const int lim = row_ok ? (MASKED ? min(si.len_k, i + off + a.win_hi + 1) : si.len_k) : 0;
    const int lim_lo = MASKED ? i + off - a.win_lo : 0;
    // elementwise bias: each wave copies the [32 rows][BN keys] block of its
    // rows for tile u + 1 during step u (LDS, two buffers), ahead of that
    // step's tile copies, so the wait at the top of step u + 1 covers it.
    // Lane L of copy k takes row (16-byte chunks per row CPB) k * 64 / CPB +
    // L / CPB, chunk L % CPB.  The range ends with the last valid row, at its
    // valid keys rounded up to 16 bytes (inside the row: bias rows are
    // 16-byte aligned); later rows read zeros.
    using bchunk_t = std::conditional_t<sizeof(T) == 2, u32x2, u32x4>;
    constexpr int CPB = C::BIAS_ROWB / 16;
    const long long sbr_b = a.sbias.r * (long long)sizeof(T);
    const int bias_voff = BIAS ? (int)((lane / CPB) * sbr_b) + (lane % CPB) * 16 : 0;
    const unsigned bias_lds = lds_addr(smem) + C::OFF_BIAS + w * C::BIAS_W;
    const int rows_w = si.len_q - (i0 + 32 * w);   // this wave's valid rows (may be <= 0)
    auto issue_bias = [&](int u) {
        const int jt = (kt_b + u) * BN;
        const char* base = reinterpret_cast<const char*>(a.bias) +
                           ((long long)b * a.sbias.b + (long long)hq * a.sbias.h +
                            (long long)(i0 + 32 * w) * a.sbias.r + jt) * (long long)sizeof(T);
        const unsigned bytes = a.bias == nullptr || rows_w <= 0
                                   ? 0u
                                   : (unsigned)((min(rows_w, 32) - 1) * sbr_b) +
                                         (unsigned)(((si.len_k - jt) * (int)sizeof(T) + 15) & ~15);
        const i32x4 rb = rsrc_words(base, bytes);
        const unsigned dst = bias_lds + (u & 1) * kWaves * C::BIAS_W;
#pragma unroll
        for (int k = 0; k < C::BOPS; ++k)
            dma_to_lds16_so(rb, dst + k * 1024, bias_voff, (int)(k * (64 / CPB) * sbr_b));
    };

    f32x16 dq[C::NDB];
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) dq[d][v] = 0.f;
    }

    // prologue: the first NS - 1 tiles in flight (after the first bias block)
    if (BIAS && n_kt > 0) issue_bias(0);
    for (int u = 0; u < C::NS - 1 && u < n_kt; ++u) issue_tile(u);
    for (int u = 0; u < n_kt; ++u) {
        const char* buf = buf_of(u);
        // tile u has landed once only the tiles issued after it may be in
        // flight; with a bias only the tile copied in the last step may (the
        // bias of tile u went out just before it), and none when that tile
        // is u itself (a ring of two)
        if constexpr (BIAS)
            dq_wait_vmem_but(C::NS >= 3 && u + C::NS - 2 < n_kt ? kOpsPerTile : 0);
        else
            dq_wait_vmem_but(kOpsPerTile * (min(u + C::NS - 2, n_kt - 1) - u));
        __syncthreads();   // tile u is visible to all waves; tile u-1's buffer is free
        const int j0 = (kt_b + u) * BN;
        // this tile's bias: this lane's row, keys 32 jb + 8 q4 + 4h .. + 3
        bchunk_t bia[BIAS ? C::NJB * 4 : 1];
        if constexpr (BIAS) {
            const char* bl = smem + C::OFF_BIAS + (u & 1) * kWaves * C::BIAS_W + w * C::BIAS_W + l32 * C::BIAS_ROWB;
#pragma unroll
            for (int q = 0; q < C::NJB * 4; ++q)   // 32 jb + 8 q4 = 8 q
                bia[q] = *reinterpret_cast<const bchunk_t*>(bl + (8 * q + 4 * h) * (int)sizeof(T));
            if (u + 1 < n_kt) issue_bias(u + 1);
        }
        if (u + C::NS - 1 < n_kt) issue_tile(u + C::NS - 1);
        const char* lk = buf + C::BUF_K;
        const char* lv = buf + C::BUF_V;
        const bool edge = !((j0 + BN <= si.len_k) && (i0 + BQ <= si.len_q) &&
                            (!MASKED || (j0 + BN - 1 <= i0 + off + a.win_hi && j0 >= i0 + BQ - 1 + off - a.win_lo)));

        // ---- S^T = K Q^T and dP^T = V dO^T (rows = keys, columns = this wave's queries)
        f32x16 st[C::NJB], dpt[C::NJB];
#pragma unroll
        for (int jb = 0; jb < C::NJB; ++jb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                st[jb][v] = 0.f;
                dpt[jb][v] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < C::NC; ++c) {
                const op_t ak = dq_read_row<T, C::ROWB>(lk, 32 * jb + l32, 16 * c + 8 * h);
                const op_t av = dq_read_row<T, C::ROWB>(lv, 32 * jb + l32, 16 * c + 8 * h);
                mma16(st[jb], ak, qreg[c]);
                mma16(dpt[jb], av, doreg[c]);
            }
        }
        if constexpr (sizeof(T) == 2) {
            // all operand reads first, so the MFMA chains do not wait on LDS latency
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NJB * C::NC, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::NJB * C::NC, 0);
        }

        // ---- P = exp2(S s log2e - LSE log2e), dS = P (dP - D); edge tiles test visibility
        // ALiBi distance of key j0 + 32 jb + acc_row(v, h) from this lane's
        // diagonal key i + off: fdist + 32 jb + 8 (v / 4) + v % 4
        const float fdist = (float)(j0 + 4 * h - i - off);
        // dropout: this lane's row i of the 4 x 4 blocks (keys j0 + 8 q + 4h ..
        // + 3, q = 4 jb + q4): word i % 4, byte (key % 4).  The four lanes of
        // a group of four rows (lanes 4k .. 4k + 3, i % 4 = lane % 4) need the
        // same blocks: lane c draws block 4 jb + c and the group trades words.
        unsigned dword_[DROP ? C::NJB * 4 : 1];
        if constexpr (DROP) {
            const int c = lane & 3;
#pragma unroll
            for (int jb = 0; jb < C::NJB; ++jb) {
                const int q = 4 * jb + c;
                const u32x4 w = quad_word_transpose(
                    drop_block((unsigned)((j0 + 8 * q + 4 * h) >> 2), (unsigned)(i >> 2), (unsigned)(b * a.hq + hq),
                               a.drop.off, a.drop.k0, a.drop.k1),
                    c);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) dword_[4 * jb + q4] = w[q4];
            }
        }
        auto softmax_grad = [&](auto masked) {
#pragma unroll
            for (int jb = 0; jb < C::NJB; ++jb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float x = st[jb][v] * scale2 - l2;
                    if constexpr (ALIBI || BIAS)
                        x = fmaf(nsl2, fabsf(fdist + (float)(32 * jb + 8 * (v >> 2) + (v & 3))), x);
                    if constexpr (BIAS) {
                        const bchunk_t bq = bia[4 * jb + (v >> 2)];
                        float bv;
                        if constexpr (sizeof(T) == 2) bv = b16_elem<T>(bq, v & 3);
                        else bv = __builtin_bit_cast(f32x4, bq)[v & 3];   // whole vector: a cast of one element reads element 0
                        x = fmaf(bv, kLog2e, x);
                    }
                    float p = __builtin_amdgcn_exp2f(x);
                    if constexpr (decltype(masked)::value) {
                        const int j = j0 + 32 * jb + acc_row(v, h);
                        p = (j < lim && j >= lim_lo) ? p : 0.f;
                    }
                    if constexpr (DROP) {
                        const bool keep = drop_keep(dword_[4 * jb + (v >> 2)], v & 3, a.drop.thr);
                        dpt[jb][v] = p * ((keep ? a.drop.rp * dpt[jb][v] : 0.f) - dl);
                    } else {
                        dpt[jb][v] = p * (dpt[jb][v] - dl);
                    }
                }
            }
        };
        if (edge)
            softmax_grad(std::true_type{});
        else
            softmax_grad(std::false_type{});

        // ---- dQ += dS K: A = dS (this lane's row, 8 keys per slice), B = K^T via transposing reads
#pragma unroll
        for (int c = 0; c < C::NJC; ++c) {
            const int jb = c >> 1, vb = 8 * (c & 1);
            op_t ads;
            float td[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) td[u] = dpt[jb][vb + u];
            to_op(ads, td);
            const int r1 = 16 * c + 4 * h, r2 = 16 * c + 8 + 4 * h;
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
                const op_t bk = dq_read_col<T, C::ROWB>(lk, r1, r2, 32 * d, lane);
                mma16(dq[d], ads, bk);
            }
        }
        if constexpr (sizeof(T) == 2) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NJC * C::NDB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, C::NJC * C::NDB, 0);
        }
    }

    // ---- write this tile's dQ rows once: scaled and converted into dq, or
    // unscaled into the accumulator (the postprocess applies s)
    if (a.dq_out != nullptr) {
        const long long ostride = a.sdq.r;
        T* o = reinterpret_cast<T*>(a.dq_out) + seq_off(a.sdq, varlen, b, si.q0) + (long long)hq * a.sdq.h +
               (long long)(i0 + 32 * w) * ostride;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = acc_row(v, h);
                const float y = mul_f32(dq[d][v], a.dq_scale);   // rounded to fp32, then to T
                if (i0 + 32 * w + r < si.len_q && 32 * d + l32 < a.d)
                    store_elem(o, (long long)r * ostride + 32 * d + l32, y);
            }
        }
        return;
    }
    float* dqa = a.dq_acc + (row0 + i0 + 32 * w) * HD;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = acc_row(v, h);
            if (i0 + 32 * w + r < si.len_q) dqa[(long long)r * HD + 32 * d + l32] = dq[d][v];
        }
    }
}


template <class T, int HD, bool MASKED, bool ALIBI, bool BIAS, bool DROP>
__global__ __launch_bounds__(kThreads, (DqCfg<T, HD>::WG_PER_CU)) void bwd_dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[BIAS ? DqCfg<T, HD>::LDS_BYTES_BIAS : DqCfg<T, HD>::LDS_BYTES];
    // ---- which query tiles: all query tiles of all q-heads of one (sequence,
    // kv-head) run on one XCD, so their K/V reads share an L2.  Under a causal
    // mask the keys a query tile sees grow linearly with its index, so
    // workgroup p takes the tiles p and (last - p) (also under a window), on
    // grids larger than the GPU (pair_tiles); else each takes one tile.
    const int G = a.hq / a.hkv;
    const bool pair = MASKED && a.pair_tiles;
    const int n_pair = pair ? (a.nblk_m + 1) / 2 : a.nblk_m;
    const int per_group = n_pair * G;          // workgroups of one (sequence, kv-head)
    int grp, slot;
    {
        const int groups = a.hkv * a.batch;
        if (groups % kXcds == 0) {
            const int xcd = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
            grp = (s / per_group) * kXcds + xcd;
            slot = s % per_group;
        } else {
            grp = blockIdx.x / per_group;
            slot = blockIdx.x % per_group;
        }
    }
    const int hkv = grp % a.hkv;
    const int b = grp / a.hkv;
    const int hq = hkv * G + slot / n_pair;
    const int p = slot % n_pair;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    if (MASKED) {
        const int nq = (si.len_q + DqCfg<T, HD>::BQ - 1) / DqCfg<T, HD>::BQ;   // this sequence's query tiles
        const int m2 = pair ? nq - 1 - p : p;   // unpaired: tile p alone
        if (m2 > p) {
            dq_tile<T, HD, MASKED, ALIBI, BIAS, DROP>(m2, a, b, hq, hkv, si, smem);   // the longer tile first
            __syncthreads();   // its LDS ring is free again
        }
        if (p < nq && p <= m2) dq_tile<T, HD, MASKED, ALIBI, BIAS, DROP>(p, a, b, hq, hkv, si, smem);
    } else {
        dq_tile<T, HD, MASKED, ALIBI, BIAS, DROP>(p, a, b, hq, hkv, si, smem);
    }
}

template <class T, int HD>
static void launch_dq_t(const BwdArgs& a0, bool masked, hipStream_t st) {
    BwdArgs a = a0;   // pairs of query tiles on grids larger than the GPU
    a.pair_tiles = masked && (long long)a.nblk_m * a.hq * a.batch > kComputeUnits;
    const unsigned grid = (unsigned)((a.pair_tiles ? (a.nblk_m + 1) / 2 : a.nblk_m) * a.hq * a.batch);
    // variants: plain, ALiBi, bias (+ ALiBi), dropout (+ bias, ALiBi)
    const bool alibi = a.alibi != nullptr, bias = a.bias != nullptr, drop = a.drop.on;
    if (masked) {
        if (drop) bwd_dq_kernel<T, HD, true, false, true, true><<<grid, kThreads, 0, st>>>(a);
        else if (bias) bwd_dq_kernel<T, HD, true, false, true, false><<<grid, kThreads, 0, st>>>(a);
        else if (alibi) bwd_dq_kernel<T, HD, true, true, false, false><<<grid, kThreads, 0, st>>>(a);
        else bwd_dq_kernel<T, HD, true, false, false, false><<<grid, kThreads, 0, st>>>(a);
    } else {
        if (drop) bwd_dq_kernel<T, HD, false, false, true, true><<<grid, kThreads, 0, st>>>(a);
        else if (bias) bwd_dq_kernel<T, HD, false, false, true, false><<<grid, kThreads, 0, st>>>(a);
        else if (alibi) bwd_dq_kernel<T, HD, false, true, false, false><<<grid, kThreads, 0, st>>>(a);
        else bwd_dq_kernel<T, HD, false, false, false, false><<<grid, kThreads, 0, st>>>(a);
    }
}

int bwd_dq_block_m() { return 32 * kWaves; }

// ---------------------------------------------------------------------------
// MFMA forward (bf16 / fp16): the same query-stationary schedule.  Per key
// tile, S^T = K Q^T (this lane's query in its accumulator column), an online
// softmax in base 2 (a running row maximum shared with the partner lane that
// holds the tile's other keys, and a running partial row sum), and
// O^T += V^T P^T: V^T through the transposing reads the dQ pass uses for K,
// P (rounded to the operand type) straight from the S^T registers.  The O^T
// accumulator's column is again this lane's query, so the rescale by the
// change of the row maximum is one scalar per lane.  Not part of the
// backward; it produces O and LSE for it.  BIAS: an elementwise bias added to
// the scaled logits (and ALiBi too when slopes are given); DROP (with BIAS):
// dropout of P with the backward's Philox stream, so O sums the kept
// probabilities times 1 / (1 - p) while the row sum and LSE take every
// visible key.
// ---------------------------------------------------------------------------
template <class T, int HD, bool MASKED, bool ALIBI, bool BIAS, bool DROP>
__device__ __forceinline__ void fwd_tile(int m, const FwdArgs& a, int b, int hq, int hkv, const SeqInfo& si,
                                         char* smem) {
    using C = DqCfg<T, HD>;
    using op_t = typename Elem<T>::op_t;
    constexpr int BQ = C::BQ, BN = C::BN;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int i0 = m * BQ;
    if (i0 >= si.len_q) return;
    const bool varlen = a.cu_q != nullptr;
    const int off = si.len_k - si.len_q;

    int key_end = si.len_k, kt_b = 0;
    if (MASKED) {
        key_end = min(key_end, min(i0 + BQ, si.len_q) - 1 + off + a.win_hi + 1);
        const int key_beg = i0 + off - a.win_lo;
        kt_b = key_beg > 0 ? key_beg / BN : 0;
    }
    const int n_kt = key_end > 0 ? max((key_end + BN - 1) / BN - kt_b, 0) : 0;

    const T* kg = reinterpret_cast<const T*>(a.k) + seq_off(a.sk, varlen, b, si.k0) + (long long)hkv * a.sk.h;
    const T* vg = reinterpret_cast<const T*>(a.v) + seq_off(a.sv, varlen, b, si.k0) + (long long)hkv * a.sv.h;
    const int valid = a.d * (int)sizeof(T) / 16;
    DqTileCopy<C::ROWB, BN> kcopy, vcopy;
    kcopy.init(w, lane, (int)(a.sk.r * (long long)sizeof(T)), valid);
    vcopy.init(w, lane, (int)(a.sv.r * (long long)sizeof(T)), valid);
    constexpr int kOpsPerTile = 2 * DqTileCopy<C::ROWB, BN>::N;
    auto buf_of = [&](int u) { return smem + (u % C::NS) * C::BUF_BYTES; };
    auto issue_tile = [&](int u) {
        const int kt = kt_b + u;
        const int rows = min(si.len_k - kt * BN, BN);
        char* buf = buf_of(u);
        kcopy.issue(rsrc_words(kg + (long long)kt * BN * a.sk.r, (unsigned)(rows * a.sk.r * (long long)sizeof(T))),
                    buf + C::BUF_K, w);
        vcopy.issue(rsrc_words(vg + (long long)kt * BN * a.sv.r, (unsigned)(rows * a.sv.r * (long long)sizeof(T))),
                    buf + C::BUF_V, w);
    };

    // ---- this lane's query row as the B operand of S^T = K Q^T
    const int i = i0 + 32 * w + l32;
    const bool row_ok = i < si.len_q;
    op_t qreg[C::NC];
    {
        const T* qg = reinterpret_cast<const T*>(a.q) + seq_off(a.sq, varlen, b, si.q0) + (long long)hq * a.sq.h +
                      (long long)i * a.sq.r;
#pragma unroll
        for (int c = 0; c < C::NC; ++c) qreg[c] = dq_load_global<T>(qg + 16 * c + 8 * h, row_ok && 16 * c + 8 * h < a.d);
    }
    const float scale2 = a.scale * kLog2e;
    const float nsl2 = ALIBI || (BIAS && a.alibi != nullptr) ? -a.alibi[hq] * kLog2e : 0.f;
    const int lim = row_ok ? (MASKED ? min(si.len_k, i + off + a.win_hi + 1) : si.len_k) : 0;
    const int lim_lo = MASKED ? i + off - a.win_lo : 0;
    // elementwise bias: this lane's row, or null (no bias, or a row past the
    // sequence).  Each element is used once, by one lane, so it is read
    // straight from memory: 4 keys per load where the row's 4-key groups are
    // 8-byte aligned, else one element at a time; keys past the sequence read
    // as zero.
    const uint16_t* brow = nullptr;
    bool bvec = false;
    if constexpr (BIAS) {
        if (a.bias != nullptr && row_ok) {
            brow = reinterpret_cast<const uint16_t*>(a.bias) + (long long)b * a.sbias.b + (long long)hq * a.sbias.h +
                   (long long)i * a.sbias.r;
            bvec = (reinterpret_cast<uintptr_t>(a.bias) & 7) == 0 && (a.sbias.b & 3) == 0 && (a.sbias.h & 3) == 0 &&
                   (a.sbias.r & 3) == 0;
        }
    }

    f32x16 o[C::NDB];   // O^T: rows = head-dim columns, column = this lane's query
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) o[d][v] = 0.f;
    }
    float mrow = -INFINITY, lsum = 0.f;   // running maximum (log2 units) and this lane's partial sum

    for (int u = 0; u < C::NS - 1 && u < n_kt; ++u) issue_tile(u);
    for (int u = 0; u < n_kt; ++u) {
        const char* buf = buf_of(u);
        dq_wait_vmem_but(kOpsPerTile * (min(u + C::NS - 2, n_kt - 1) - u));
        __syncthreads();
        if (u + C::NS - 1 < n_kt) issue_tile(u + C::NS - 1);
        const char* lk = buf + C::BUF_K;
        const char* lv = buf + C::BUF_V;
        const int j0 = (kt_b + u) * BN;
        const bool edge = !((j0 + BN <= si.len_k) && (i0 + BQ <= si.len_q) &&
                            (!MASKED || (j0 + BN - 1 <= i0 + off + a.win_hi && j0 >= i0 + BQ - 1 + off - a.win_lo)));

        // this tile's bias: keys 32 jb + 8 q4 + 4h .. + 3 of this lane's row (q = 4 jb + q4)
        u32x2 bia[BIAS ? C::NJB * 4 : 1];
        if constexpr (BIAS) {
#pragma unroll
            for (int q = 0; q < C::NJB * 4; ++q) {
                const int jc = j0 + 8 * q + 4 * h;
                u32x2 wv = {0u, 0u};
                if (brow != nullptr) {
                    if (bvec && jc + 4 <= si.len_k) {
                        wv = *reinterpret_cast<const u32x2*>(brow + jc);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (jc + e < si.len_k) wv[e >> 1] |= (unsigned)brow[jc + e] << (16 * (e & 1));
                    }
                }
                bia[q] = wv;
            }
        }
        // dropout: lane c of each group of four rows draws block 4 jb + c of
        // the tile (keys j0 + 8 q + 4h .. + 3) and the group trades words so
        // that each lane holds its own row's word of every block
        unsigned dword_[DROP ? C::NJB * 4 : 1];
        if constexpr (DROP) {
            const int c = lane & 3;
#pragma unroll
            for (int jb = 0; jb < C::NJB; ++jb) {
                const int q = 4 * jb + c;
                const u32x4 wd = quad_word_transpose(
                    drop_block((unsigned)((j0 + 8 * q + 4 * h) >> 2), (unsigned)(i >> 2), (unsigned)(b * a.hq + hq),
                               a.drop.off, a.drop.k0, a.drop.k1),
                    c);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) dword_[4 * jb + q4] = wd[q4];
            }
        }

        f32x16 st[C::NJB];
#pragma unroll
        for (int jb = 0; jb < C::NJB; ++jb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) st[jb][v] = 0.f;
#pragma unroll
            for (int c = 0; c < C::NC; ++c)
                mma16(st[jb], dq_read_row<T, C::ROWB>(lk, 32 * jb + l32, 16 * c + 8 * h), qreg[c]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, C::NJB * C::NC, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, C::NJB * C::NC, 0);

        // ---- logits in log2 units; keys this row does not see are -inf
        const float fdist = (float)(j0 + 4 * h - i - off);
        auto logits = [&](auto masked) {
#pragma unroll
            for (int jb = 0; jb < C::NJB; ++jb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float x = st[jb][v] * scale2;
                    if constexpr (ALIBI || BIAS)
                        x = fmaf(nsl2, fabsf(fdist + (float)(32 * jb + 8 * (v >> 2) + (v & 3))), x);
                    if constexpr (BIAS) x = fmaf(b16_elem<T>(bia[4 * jb + (v >> 2)], v & 3), kLog2e, x);
                    if constexpr (decltype(masked)::value) {
                        const int j = j0 + 32 * jb + acc_row(v, h);
                        x = (j < lim && j >= lim_lo) ? x : -INFINITY;
                    }
                    st[jb][v] = x;
                }
            }
        };
        if (edge)
            logits(std::true_type{});
        else
            logits(std::false_type{});

        // ---- online softmax: the tile's maximum over both lanes of the row
        float tmax = -INFINITY;
#pragma unroll
        for (int jb = 0; jb < C::NJB; ++jb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, st[jb][v]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(mrow, tmax);
        const float mref = mnew == -INFINITY ? 0.f : mnew;   // a row with no key yet keeps P = 0
        const float corr = __builtin_amdgcn_exp2f(mrow - mref);
        lsum *= corr;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
            for (int v = 0; v < 16; ++v) o[d][v] *= corr;
        }
#pragma unroll
        for (int jb = 0; jb < C::NJB; ++jb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(st[jb][v] - mref);
                lsum += p;   // the row sum (and LSE) over every visible key
                if constexpr (DROP)
                    st[jb][v] = drop_keep(dword_[4 * jb + (v >> 2)], v & 3, a.drop.thr) ? p : 0.f;
                else
                    st[jb][v] = p;
            }
        }
        mrow = mnew;

        // ---- O^T += V^T P^T: A = V^T via transposing reads, B = P (this lane's query, 8 keys per slice)
#pragma unroll
        for (int c = 0; c < C::NJC; ++c) {
            const int jb = c >> 1, vb = 8 * (c & 1);
            op_t pb;
            float tp[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) tp[t] = st[jb][vb + t];
            to_op(pb, tp);
            const int r1 = 16 * c + 4 * h, r2 = 16 * c + 8 + 4 * h;
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) mma16(o[d], dq_read_col<T, C::ROWB>(lv, r1, r2, 32 * d, lane), pb);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NJC * C::NDB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, C::NJC * C::NDB, 0);
    }

    // ---- epilogue: O = O^T / l (this lane's query row), LSE = (m + log2 l) ln 2
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!row_ok) return;
    const float inv = ltot > 0.f ? (DROP ? a.drop.rp : 1.f) / ltot : 0.f;
    T* orow = reinterpret_cast<T*>(a.o) + seq_off(a.so, varlen, b, si.q0) + (long long)hq * a.so.h +
              (long long)i * a.so.r;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int col = 32 * d + acc_row(v, h);
            if (col < a.d) store_elem(orow, col, o[d][v] * inv);
        }
    }
    if (h == 0) {
        const long long li = varlen ? (long long)hq * a.total_q + si.q0 + i : ((long long)b * a.hq + hq) * a.seqlen_q + i;
        a.lse[li] = ltot > 0.f ? (mrow + log2f(ltot)) * kLn2 : -INFINITY;
    }
}

template <class T, int HD, bool MASKED, bool ALIBI, bool BIAS, bool DROP>
__global__ __launch_bounds__(kThreads, (DqCfg<T, HD>::WG_PER_CU)) void fwd_mfma_kernel(FwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[DqCfg<T, HD>::LDS_BYTES];
    // all query tiles of all q-heads of one (sequence, kv-head) on one XCD;
    // masked: workgroup p takes the tiles p and (last - p)
    constexpr int BQ = DqCfg<T, HD>::BQ;
    const int G = a.hq / a.hkv;
    const int nblk_m = (a.seqlen_q + BQ - 1) / BQ;
    const int n_pair = MASKED ? (nblk_m + 1) / 2 : nblk_m;
    const int per_group = n_pair * G;
    int grp, slot;
    {
        const int groups = a.hkv * a.batch;
        if (groups % kXcds == 0) {
            const int xcd = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
            grp = (s / per_group) * kXcds + xcd;
            slot = s % per_group;
        } else {
            grp = blockIdx.x / per_group;
            slot = blockIdx.x % per_group;
        }
    }
    const int hkv = grp % a.hkv;
    const int b = grp / a.hkv;
    const int hq = hkv * G + slot / n_pair;
    const int p = slot % n_pair;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    if (MASKED) {
        const int nq = (si.len_q + BQ - 1) / BQ;
        const int m2 = nq - 1 - p;
        if (m2 > p) {
            fwd_tile<T, HD, MASKED, ALIBI, BIAS, DROP>(m2, a, b, hq, hkv, si, smem);
            __syncthreads();
        }
        if (p < nq && p <= m2) fwd_tile<T, HD, MASKED, ALIBI, BIAS, DROP>(p, a, b, hq, hkv, si, smem);
    } else {
        fwd_tile<T, HD, MASKED, ALIBI, BIAS, DROP>(p, a, b, hq, hkv, si, smem);
    }
}

template <class T, int HD>
static void launch_fwd_mfma_t(const FwdArgs& a, bool masked, hipStream_t st) {
    constexpr int BQ = DqCfg<T, HD>::BQ;
    const int nblk_m = (a.seqlen_q + BQ - 1) / BQ;
    const unsigned grid = (unsigned)((masked ? (nblk_m + 1) / 2 : nblk_m) * a.hq * a.batch);
    // variants: plain, ALiBi, bias (+ ALiBi), dropout (+ bias, ALiBi)
    const bool alibi = a.alibi != nullptr, bias = a.bias != nullptr, drop = a.drop.on;
    if (masked) {
        if (drop) fwd_mfma_kernel<T, HD, true, false, true, true><<<grid, kThreads, 0, st>>>(a);
        else if (bias) fwd_mfma_kernel<T, HD, true, false, true, false><<<grid, kThreads, 0, st>>>(a);
        else if (alibi) fwd_mfma_kernel<T, HD, true, true, false, false><<<grid, kThreads, 0, st>>>(a);
        else fwd_mfma_kernel<T, HD, true, false, false, false><<<grid, kThreads, 0, st>>>(a);
    } else {
        if (drop) fwd_mfma_kernel<T, HD, false, false, true, true><<<grid, kThreads, 0, st>>>(a);
        else if (bias) fwd_mfma_kernel<T, HD, false, false, true, false><<<grid, kThreads, 0, st>>>(a);
        else if (alibi) fwd_mfma_kernel<T, HD, false, true, false, false><<<grid, kThreads, 0, st>>>(a);
        else fwd_mfma_kernel<T, HD, false, false, false, false><<<grid, kThreads, 0, st>>>(a);
    }
}

void launch_fwd_mfma(const FwdArgs& a, int dtype, int hd, bool masked, hipStream_t st) {
    if (dtype == ATTN_DTYPE_BF16) {
        if (hd == 64) launch_fwd_mfma_t<bf16_t, 64>(a, masked, st);
        else if (hd == 128) launch_fwd_mfma_t<bf16_t, 128>(a, masked, st);
        else launch_fwd_mfma_t<bf16_t, 256>(a, masked, st);
    } else {
        if (hd == 64) launch_fwd_mfma_t<f16_t, 64>(a, masked, st);
        else if (hd == 128) launch_fwd_mfma_t<f16_t, 128>(a, masked, st);
        else launch_fwd_mfma_t<f16_t, 256>(a, masked, st);
    }
}

void launch_bwd_dq(const BwdArgs& a, int dtype, int hd, bool masked, hipStream_t st) {
    if (dtype == ATTN_DTYPE_BF16) {
        if (hd == 64) launch_dq_t<bf16_t, 64>(a, masked, st);
        else if (hd == 128) launch_dq_t<bf16_t, 128>(a, masked, st);
        else launch_dq_t<bf16_t, 256>(a, masked, st);
    } else if (dtype == ATTN_DTYPE_F16) {
        if (hd == 64) launch_dq_t<f16_t, 64>(a, masked, st);
        else if (hd == 128) launch_dq_t<f16_t, 128>(a, masked, st);
        else launch_dq_t<f16_t, 256>(a, masked, st);
    } else {   // fp32: head dims up to 128
        if (hd == 64) launch_dq_t<float, 64>(a, masked, st);
        else launch_dq_t<float, 128>(a, masked, st);
    }
}

}  // namespace attn
