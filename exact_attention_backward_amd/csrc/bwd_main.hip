// Main backward kernel of exact attention for gfx950.
//
// One workgroup (4 waves) owns a tile of 128 keys of one (sequence, kv-head)
// and loops over the query tiles that can see it, for every q-head of the
// kv-head's GQA group.  This is the key-stationary schedule of the
// Composable Kernel page "block_fmha_bwd_dq_dk_dv_pipeline_trload_kr_ktr_vr.hpp
// Source File" (one K/V tile per block, loop over Q tiles, five GEMMs):
//
//   stage 1  S  = Q K^T                 (MFMA, K from registers)
//   stage 2  P  = exp2(S s log2e - LSE log2e), masked on edge tiles only
//   stage 4  dP = dO V^T                (MFMA, V from registers)
//   stage 3  dV += P^T dO               (MFMA, P^T straight from the S registers)
//   stage 5  dS = P (dP - D)
//   stage 6  dK += dS^T Q               (MFMA, dS^T straight from the registers)
//   stage 7  dQ_tile = dS K             (MFMA, dS via LDS, K^T from registers)
//            dQaccum += dQ_tile         (fp32 atomics, or ordered adds)
//
// Wave w owns keys 32w..32w+31 of the tile: it keeps those rows of K and V in
// registers as MFMA B operands, accumulates their dK and dV rows in fp32 for
// the whole loop, and, for the dQ product, holds a 32-column slice of K^T.
// All transposed operands (dO and Q for stages 3 and 6, dS for stage 7, K^T)
// come from LDS through the transposing read ds_read_b64_tr_b16, so every
// tile is stored once, row-major and swizzled.
#include "bwd_shared.h"
#include "kv_kernel.h"

#include <type_traits>

namespace attn {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = kBwdBlockN;

template <class T, int HD, bool DQ_ATOMIC = true>
struct BwdCfg {
    static constexpr int BM = HD == 128 ? 32 : 64;   // query rows per tile
    static constexpr int ROWB = HD * (int)sizeof(T);                       // LDS bytes per Q/dO/K row
    static constexpr int DSROWB = BM * (int)sizeof(T);                     // LDS bytes per dS^T row
    static constexpr int TILE = BM * ROWB;
    // LDS map: [resident K tile] | buffers of (Q, dO, LSE, D) | [dS^T]; the
    // K tile and dS^T are only needed when dQ is accumulated here
    static constexpr int K_BYTES = DQ_ATOMIC ? kBN * ROWB : 0;
    static constexpr int DS_BYTES = DQ_ATOMIC ? kBN * DSROWB : 0;
    static constexpr int OFF_K = 0;
    static constexpr int BUF_Q = 0, BUF_DO = TILE, BUF_LSE = 2 * TILE, BUF_DL = 2 * TILE + BM * 4;
    static constexpr int BUF_BYTES = 2 * TILE + 2 * BM * 4;
    static constexpr int OFF_BUF = K_BYTES;
    static constexpr int OFF_DS = OFF_BUF + 2 * BUF_BYTES;
    static constexpr int LDS_BYTES = OFF_DS + (DS_BYTES > 0 ? DS_BYTES : 16);
    static constexpr int NC = HD / 16;     // 16-wide chunks of the head dim
    static constexpr int NMB = BM / 32;    // 32-row blocks of a query tile
    static constexpr int NDB = HD / 32;    // 32-column blocks of the head dim
    static constexpr int NIC = BM / 16;    // 16-wide chunks of the query rows
    static constexpr int NJC = kBN / 16;   // 16-wide chunks of the keys
    static constexpr int DQB = NMB * NDB / kWaves;   // dQ 32x32 blocks per wave
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(NMB * NDB % kWaves == 0 && kWaves % NDB == 0, "dQ block split");
    static_assert(BM <= 64, "one load instruction per LSE/D tile");
};

// --------------------------------------------------------------------------
// operand loads
// --------------------------------------------------------------------------

// Row-major operand: lane gets M[row][col .. col+7] (col = 16c + 8h).
template <class T, int ROWB>
__device__ __forceinline__ typename Elem<T>::op_t read_op_row(const char* lds, int row, int col) {
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(typename Elem<T>::op_t, lds_read16(lds, swz<ROWB>(row, col * 2)));
    } else {
        // whole-vector casts: a bit cast of a subscripted vector element is
        // miscompiled (it reads element 0), so elements are never cast singly
        const f32x4 a = __builtin_bit_cast(f32x4, lds_read16(lds, swz<ROWB>(row, col * 4)));
        const f32x4 b = __builtin_bit_cast(f32x4, lds_read16(lds, swz<ROWB>(row, col * 4 + 16)));
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
}

// Column operand: lane (l32 = lane % 32) gets M[r1 + t][c0 + l32] for t = 0..3
// and M[r2 + t][c0 + l32] for t = 0..3, rows r1/r2 chosen per lane half.
template <class T, int ROWB>
__device__ __forceinline__ typename Elem<T>::op_t read_op_col(const char* lds, int r1, int r2, int c0, int lane) {
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

// Stage NROWS rows (row0 ..) of a global [rows, stride] tensor into a swizzled
// LDS tile; rows at or past `valid` (>= 1) are written as zeros.  The loads
// are unconditional (the row index is clamped into range) so that all of them
// issue back to back and their latencies overlap.
template <class T, int ROWB, int NROWS>
__device__ __forceinline__ void stage_rows(char* lds, const T* g, long long stride, int row0, int valid) {
    constexpr int CPR = ROWB / 16;
    constexpr int N = NROWS * CPR / kThreads;
    static_assert(NROWS * CPR % kThreads == 0, "tile split");
    u32x4 v[N];
#pragma unroll
    for (int t = 0; t < N; ++t) {
        const int c = threadIdx.x + t * kThreads;
        const int r = c / CPR, ch = c % CPR;
        const int rr = min(row0 + r, valid - 1);
        v[t] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(g + (long long)rr * stride) + ch * 16);
    }
#pragma unroll
    for (int t = 0; t < N; ++t) {
        const int c = threadIdx.x + t * kThreads;
        const int r = c / CPR, ch = c % CPR;
        const u32x4 z = {0u, 0u, 0u, 0u};
        lds_write(lds, swz<ROWB>(r, ch * 16), row0 + r < valid ? v[t] : z);
    }
}

__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-lane plan for copying a tile of NROWS rows (row length ROWB bytes in
// LDS, rows stride_bytes apart in HBM) into its swizzled LDS image with
// buffer_load ... lds, by a workgroup of WAVES waves: instruction t of wave w
// fills the 1 KiB LDS segment w + t * WAVES, lane l writing 16-byte slot l of
// it; the lane fetches whichever global chunk the swizzle puts in that slot.
// The per-lane byte offsets are computed once; a tile copy is then one
// descriptor (built with scalar instructions) and N buffer loads per wave.
// Rows outside the descriptor's range arrive as zeros.
template <int ROWB, int NROWS, int WAVES = kWaves>
struct TileCopy {
    static constexpr int CPR = ROWB / 16;
    static constexpr int N = NROWS * CPR / 64 / WAVES;
    static_assert(NROWS * CPR % (64 * WAVES) == 0, "segment split");
    int voff[N];
    // stride_bytes: between rows in memory; valid: 16-byte chunks of a row
    // inside the head dim (the others read zeros)
    __device__ __forceinline__ void init(int w, int lane, int stride_bytes, int valid) {
#pragma unroll
        for (int t = 0; t < N; ++t) {
            const int slot = (w + t * WAVES) * 64 + lane;
            const int r = slot / CPR;
            const int c = (slot % CPR) ^ swz_key<ROWB>(r);
            voff[t] = c < valid ? r * stride_bytes + c * 16 : kOobOff;
        }
    }
    __device__ __forceinline__ void issue(rsrc_t src, char* lds, int w) const {
#pragma unroll
        for (int t = 0; t < N; ++t) buffer_to_lds16(src, lds + (w + t * WAVES) * 1024, voff[t]);
    }
    // untracked copies (see dma_to_lds16)
    __device__ __forceinline__ void issue_untracked(i32x4 src, const char* lds, int w) const {
#pragma unroll
        for (int t = 0; t < N; ++t) dma_to_lds16(src, lds_addr(lds + (w + t * WAVES) * 1024), voff[t]);
    }
};

// --------------------------------------------------------------------------
// the kernel
// --------------------------------------------------------------------------
template <class T, int HD, bool MASKED, bool DQ_ATOMIC>
__global__ __launch_bounds__(kThreads, 1) void bwd_kernel(BwdArgs a) {
    using C = BwdCfg<T, HD, DQ_ATOMIC>;
    using op_t = typename Elem<T>::op_t;
    constexpr int BM = C::BM;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    // ---- which key tile: deterministic masked runs dispatch the highest key
    // tile of a (sequence, kv-head) first, since it reaches every query tile
    // first and so is first in the fixed summation order.
    // Workgroups are dispatched round-robin over the 8 XCDs (each with its
    // own L2).  All key tiles of one (sequence, kv-head) are put on the same
    // XCD, in consecutive dispatch slots, so the dQ tiles they all add into
    // and the Q/dO tiles they all read stay in one L2.  Within a group the
    // dispatch order still follows the key-tile order.
    int grp, nb_lin;
    {
        const int groups = a.hkv * a.batch;
        if (groups % kXcds == 0) {
            const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
            grp = (slot / a.nblk_n) * kXcds + xcd;
            nb_lin = slot % a.nblk_n;
        } else {
            grp = blockIdx.x / a.nblk_n;
            nb_lin = blockIdx.x % a.nblk_n;
        }
    }
    const int hkv = grp % a.hkv;
    const int b = grp / a.hkv;
    const int n = (MASKED && a.deterministic) ? a.nblk_n - 1 - nb_lin : nb_lin;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    if (n * kBN >= si.len_k) return;
    const bool varlen = a.cu_q != nullptr;
    const int G = a.hq / a.hkv;
    const int off = si.len_k - si.len_q;   // bottom-right alignment of the mask
    int m_begin = 0, m_end = (si.len_q + BM - 1) / BM;
    if (MASKED) {
        // query rows that see some key of the tile: from the first row whose
        // upper bound reaches key n*kBN to the last row whose lower bound
        // still admits the tile's last key
        const int first_row = n * kBN - off - a.win_hi;
        const int last_row = min(n * kBN + kBN, si.len_k) - 1 - off + a.win_lo;
        m_begin = first_row > 0 ? first_row / BM : 0;
        m_end = last_row < 0 ? 0 : min(last_row, si.len_q - 1) / BM + 1;
    }
    const int n_m = max(m_end - m_begin, 0);
    const int n_tiles = G * n_m;            // (q-head, query tile) pairs, q-head major
    const int nblk_k = (si.len_k + kBN - 1) / kBN;

    const T* kg = reinterpret_cast<const T*>(a.k) + seq_off(a.sk, varlen, b, si.k0) + (long long)hkv * a.sk.h;
    const T* vg = reinterpret_cast<const T*>(a.v) + seq_off(a.sv, varlen, b, si.k0) + (long long)hkv * a.sv.h;
    const int valid = a.d * (int)sizeof(T) / 16;   // 16-byte chunks of a row inside the head dim
    char* lk = smem + C::OFF_K;
    char* lds_ds = smem + C::OFF_DS;

    // query-side tile t (q-head hkv*G + t / n_m, query tile m_begin + t % n_m)
    auto tile_head = [&](int t) { return hkv * G + t / n_m; };
    auto tile_row0 = [&](int t) { return (m_begin + t % n_m) * BM; };
    auto lse_base = [&](int hq) -> long long {
        return varlen ? (long long)hq * a.total_q + si.q0 : ((long long)b * a.hq + hq) * a.seqlen_q;
    };
    TileCopy<C::ROWB, BM> qcopy, docopy;
    qcopy.init(w, lane, (int)(a.sq.r * (long long)sizeof(T)), valid);
    docopy.init(w, lane, (int)(a.sdo.r * (long long)sizeof(T)), valid);
    const long long q_seq = seq_off(a.sq, varlen, b, si.q0), do_seq = seq_off(a.sdo, varlen, b, si.q0);
    auto issue_tile = [&](int t, char* buf) {
        const int hq = tile_head(t), i0 = tile_row0(t);
        const int rows = min(si.len_q - i0, BM);
        const long long q_elem = q_seq + (long long)hq * a.sq.h + (long long)i0 * a.sq.r;
        const long long do_elem = do_seq + (long long)hq * a.sdo.h + (long long)i0 * a.sdo.r;
        qcopy.issue_untracked(rsrc_words(reinterpret_cast<const T*>(a.q) + q_elem,
                                         (unsigned)(rows * a.sq.r * (long long)sizeof(T))), buf + C::BUF_Q, w);
        docopy.issue_untracked(rsrc_words(reinterpret_cast<const T*>(a.dout) + do_elem,
                                          (unsigned)(rows * a.sdo.r * (long long)sizeof(T))), buf + C::BUF_DO, w);
        const long long lb = lse_base(hq) + i0;
        if (w == 0 && lane < BM) dma_to_lds4(rsrc_words(a.lse + lb, rows * 4), lds_addr(buf + C::BUF_LSE), lane * 4);
        if (w == 1 && lane < BM) dma_to_lds4(rsrc_words(a.delta + lb, rows * 4), lds_addr(buf + C::BUF_DL), lane * 4);
    };

    // ---- prologue: first query tile, the resident K tile, K/V rows of this wave
    if (n_tiles > 0) issue_tile(0, smem + C::OFF_BUF);
    if constexpr (DQ_ATOMIC) {
        TileCopy<C::ROWB, kBN> kcopy;
        kcopy.init(w, lane, (int)(a.sk.r * (long long)sizeof(T)), valid);
        const int rows = min(si.len_k - n * kBN, kBN);
        kcopy.issue(make_rsrc(kg + (long long)n * kBN * a.sk.r, (unsigned)(rows * a.sk.r * (long long)sizeof(T))), lk,
                    w);
    }
    op_t kreg[C::NC], vreg[C::NC];
    {
        const int j = n * kBN + 32 * w + l32;
        const bool ok = j < si.len_k;
#pragma unroll
        for (int c = 0; c < C::NC; ++c) {
            const int col = 16 * c + 8 * h;   // first of this lane's 8 columns of chunk c
            kreg[c] = load_op_global<T>(kg + (long long)j * a.sk.r + col, ok && col < a.d);
            vreg[c] = load_op_global<T>(vg + (long long)j * a.sv.r + col, ok && col < a.d);
        }
    }
    wait_vmem();
    __syncthreads();
    // dQ blocks of this wave: column block db_w, row blocks mb_w0 + x * (kWaves / NDB)
    const int db_w = w % C::NDB;
    const int mb_w0 = w / C::NDB;

    f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            dk[d][v] = 0.f;
            dv[d][v] = 0.f;
        }
    }

    const float scale2 = a.scale * kLog2e;
    const int j = n * kBN + 32 * w + l32;   // this lane's key (column of S)

    for (int t = 0; t < n_tiles; ++t) {
        char* buf = smem + C::OFF_BUF + (t & 1) * C::BUF_BYTES;
        char* nbuf = smem + C::OFF_BUF + ((t + 1) & 1) * C::BUF_BYTES;
        const int hq = tile_head(t);
        const int i0 = tile_row0(t);
        const int m = i0 / BM;
        // all waves are done with the other buffer and with dS^T of tile t-1;
        // this tile's data has landed (each wave waited for its own copies)
        __syncthreads();
        if (t + 1 < n_tiles) issue_tile(t + 1, nbuf);
        const char* lq = buf + C::BUF_Q;
        const char* ldo = buf + C::BUF_DO;
        const float* llse = reinterpret_cast<const float*>(buf + C::BUF_LSE);
        const float* ldl = reinterpret_cast<const float*>(buf + C::BUF_DL);

        // per-row key limits: key j is visible to row i iff lo(i) <= j < lim(i)
        const bool edge = !((i0 + BM <= si.len_q) && (n * kBN + kBN <= si.len_k) &&
                            (!MASKED || (n * kBN + kBN - 1 <= i0 + off + a.win_hi &&
                                         n * kBN >= i0 + BM - 1 + off - a.win_lo)));

        // ---- stages 1 and 4: S = Q K^T and dP = dO V^T for this wave's keys
        f32x16 s[C::NMB], dp[C::NMB];
#pragma unroll
        for (int mb = 0; mb < C::NMB; ++mb) {
            op_t aq[C::NC], ado[C::NC];
#pragma unroll
            for (int c = 0; c < C::NC; ++c) {
                aq[c] = read_op_row<T, C::ROWB>(lq, 32 * mb + l32, 16 * c + 8 * h);
                ado[c] = read_op_row<T, C::ROWB>(ldo, 32 * mb + l32, 16 * c + 8 * h);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[mb][v] = 0.f;
                dp[mb][v] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < C::NC; ++c) {
                mma16(s[mb], aq[c], kreg[c]);
                mma16(dp[mb], ado[c], vreg[c]);
            }
        }

        // ---- stages 2 and 5: P = exp2(S s log2e - LSE log2e); dS = P (dP - D).
        // Only edge tiles test visibility (key j is visible to row i iff
        // lo(i) <= j < lim(i)); the branch is uniform.
        // ALiBi slope of this tile's q-head, negated, in log2 units
        const float nsl2 = a.alibi != nullptr ? -a.alibi[hq] * kLog2e : 0.f;
        // this (sequence, q-head)'s elementwise bias and dBias, or null
        const T* bias_h = a.bias != nullptr ? reinterpret_cast<const T*>(a.bias) + (long long)b * a.sbias.b +
                                                  (long long)hq * a.sbias.h
                                            : nullptr;
        T* dbias_h = a.dbias != nullptr ? reinterpret_cast<T*>(a.dbias) + (long long)b * a.sdbias.b +
                                              (long long)hq * a.sdbias.h
                                        : nullptr;
        // extra: ALiBi, the bias and dropout (each present or not); rows and
        // keys past the sequence read no bias.  Dropout: the rows r..r+3 of
        // key j form one column of a 4 x 4 block; dropped elements leave dV
        // (P zeroed) and enter dS as -P D
        auto softmax_grad = [&](auto masked, auto extra) {
#pragma unroll
            for (int mb = 0; mb < C::NMB; ++mb) {
                // dropout: bit 4 q4 + e of keep is element (row 32 mb + 8 q4 + 4h
                // + e, key j).  The four lanes of a group of four keys (lanes
                // 4k .. 4k + 3, j % 4 = lane % 4) need the same blocks: lane c
                // draws block q4 = c and the group trades the decisions.
                unsigned keep_m = 0xffffffffu;
                if constexpr (decltype(extra)::value) {
                    if (a.drop.on) {
                        const int c = lane & 3;
                        const unsigned m = drop_mask16(
                            drop_block((unsigned)(j >> 2), (unsigned)((i0 + 32 * mb + 8 * c + 4 * h) >> 2),
                                       (unsigned)(b * a.hq + hq), a.drop.off, a.drop.k0, a.drop.k1),
                            a.drop.thr);
                        const unsigned sh = 4u * (unsigned)c;
                        keep_m = ((quad_bcast<0>(m) >> sh) & 0xfu) | (((quad_bcast<1>(m) >> sh) & 0xfu) << 4) |
                                 (((quad_bcast<2>(m) >> sh) & 0xfu) << 8) | (((quad_bcast<3>(m) >> sh) & 0xfu) << 12);
                    }
                }
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int r = 32 * mb + 8 * q4 + 4 * h;
                    const f32x4 lse = *reinterpret_cast<const f32x4*>(llse + r);
                    const f32x4 dl = *reinterpret_cast<const f32x4*>(ldl + r);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 4 * q4 + e;
                        const float l2 = lse[e] == -INFINITY ? 0.f : lse[e] * kLog2e;
                        float x = s[mb][v] * scale2 - l2;
                        if constexpr (decltype(extra)::value) {
                            const int ib = i0 + r + e;
                            x = fmaf(nsl2, fabsf((float)(j - ib - off)), x);
                            if (bias_h != nullptr && ib < si.len_q && j < si.len_k)
                                x = fmaf(load_elem(bias_h, (long long)ib * a.sbias.r + j), kLog2e, x);
                        }
                        float p = __builtin_amdgcn_exp2f(x);
                        if constexpr (decltype(masked)::value) {
                            const int i = i0 + r + e;
                            const int lim =
                                i < si.len_q ? (MASKED ? min(si.len_k, i + off + a.win_hi + 1) : si.len_k) : 0;
                            const int lo = MASKED ? i + off - a.win_lo : 0;
                            p = (j < lim && j >= lo) ? p : 0.f;
                        }
                        if constexpr (decltype(extra)::value) {
                            if (a.drop.on) {
                                const bool keep = (keep_m >> (4 * q4 + e)) & 1u;
                                s[mb][v] = keep ? p : 0.f;
                                dp[mb][v] = p * ((keep ? a.drop.rp * dp[mb][v] : 0.f) - dl[e]);
                                continue;
                            }
                        }
                        s[mb][v] = p;
                        dp[mb][v] = p * (dp[mb][v] - dl[e]);
                    }
                }
            }
        };
        if (a.alibi != nullptr || a.bias != nullptr || a.drop.on) {
            if (edge)
                softmax_grad(std::true_type{}, std::true_type{});
            else
                softmax_grad(std::false_type{}, std::true_type{});
        } else {
            if (edge)
                softmax_grad(std::true_type{}, std::false_type{});
            else
                softmax_grad(std::false_type{}, std::false_type{});
        }

        // ---- stages 3 and 6: dV += P^T dO, dK += dS^T Q
#pragma unroll
        for (int c = 0; c < C::NIC; ++c) {
            const int mb = c >> 1, vb = 8 * (c & 1);
            op_t pa, dsa;
            float tp[8], td[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                tp[u] = s[mb][vb + u];
                td[u] = dp[mb][vb + u];
            }
            to_op(pa, tp);
            to_op(dsa, td);
            const int r1 = 16 * c + 4 * h, r2 = 16 * c + 8 + 4 * h;
            op_t bdo[C::NDB], bq[C::NDB];
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
                bdo[d] = read_op_col<T, C::ROWB>(ldo, r1, r2, 32 * d, lane);
                bq[d] = read_op_col<T, C::ROWB>(lq, r1, r2, 32 * d, lane);
            }
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
                mma16(dv[d], pa, bdo[d]);
                mma16(dk[d], dsa, bq[d]);
            }
        }

        if constexpr (!DQ_ATOMIC) {
            // dBias = dS, straight from the registers (dQ comes from another
            // pass; each step ends with a full wait for memory operations)
            if (dbias_h != nullptr) {
#pragma unroll
                for (int mb = 0; mb < C::NMB; ++mb) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int ib = i0 + 32 * mb + acc_row(v, h);
                        if (ib < si.len_q && j < si.len_k)
                            store_elem(dbias_h, (long long)ib * a.sdbias.r + j, dp[mb][v]);
                    }
                }
            }
        }
        if constexpr (DQ_ATOMIC) {
        // ---- dS^T to LDS (row = key, column = query row)
        {
            const int jr = 32 * w + l32;
#pragma unroll
            for (int mb = 0; mb < C::NMB; ++mb) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int col = 32 * mb + 8 * q4 + 4 * h;
                    if constexpr (sizeof(T) == 2) {
                        const u32x2 wv = {pack2<T>(dp[mb][4 * q4], dp[mb][4 * q4 + 1]),
                                          pack2<T>(dp[mb][4 * q4 + 2], dp[mb][4 * q4 + 3])};
                        lds_write(lds_ds, swz<C::DSROWB>(jr, col * 2), wv);
                    } else {
                        const f32x4 wv = {dp[mb][4 * q4], dp[mb][4 * q4 + 1], dp[mb][4 * q4 + 2],
                                          dp[mb][4 * q4 + 3]};
                        lds_write(lds_ds, swz<C::DSROWB>(jr, col * 4), wv);
                    }
                }
            }
        }
        __syncthreads();
        if (dbias_h != nullptr) {
            // dBias = dS of this tile (rows and keys inside the sequence),
            // copied from its LDS image (already in the I/O type); consecutive
            // threads take consecutive keys of a row
            for (int e = threadIdx.x; e < BM * kBN; e += kThreads) {
                const int ii = e / kBN, jj = e % kBN;
                const int ib = i0 + ii, jb = n * kBN + jj;
                if (ib < si.len_q && jb < si.len_k)
                    dbias_h[(long long)ib * a.sdbias.r + jb] =
                        *reinterpret_cast<const T*>(lds_ds + swz<C::DSROWB>(jj, ii * (int)sizeof(T)));
            }
        }

        // ---- stage 7: dQ tile = dS K for this wave's blocks
        f32x16 dq[C::DQB];
#pragma unroll
        for (int x = 0; x < C::DQB; ++x) {
#pragma unroll
            for (int v = 0; v < 16; ++v) dq[x][v] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < C::NJC; ++c) {
            op_t ads[C::DQB];
#pragma unroll
            for (int x = 0; x < C::DQB; ++x) {
                const int mb = mb_w0 + x * (kWaves / C::NDB);
                ads[x] = read_op_col<T, C::DSROWB>(lds_ds, 16 * c + 8 * h, 16 * c + 8 * h + 4, 32 * mb, lane);
            }
            const op_t kt = read_op_col<T, C::ROWB>(lk, 16 * c + 8 * h, 16 * c + 8 * h + 4, 32 * db_w, lane);
#pragma unroll
            for (int x = 0; x < C::DQB; ++x) mma16(dq[x], ads[x], kt);
        }

        // ---- dQ accumulation: fp32 atomics, or in a fixed order per tile
        const long long row0 = lse_base(hq);
        float* dqa = a.dq_acc + row0 * HD;
        int* sem = a.sem + ((long long)b * a.hq + hq) * a.nblk_m + m;
        if (a.deterministic) {
            int rank;
            if (MASKED) {
                // the key tiles that visit query tile m are a contiguous run
                // ending at the last one whose first key some row of the tile
                // sees; they come in descending order
                const int x = (m + 1) * BM + off + a.win_hi;
                const int last = min(nblk_k - 1, (x + kBN - 1) / kBN - 1);
                rank = last - n;
            } else {
                rank = n;
            }
            // The counter and the dQ adds are device-scope atomics, which the
            // memory side performs (they bypass the per-XCD L2s), and the
            // tile's adds only write: observing the count with a coherent
            // relaxed load, then issuing the adds, orders them after the
            // previous contributor's.  No acquire fence: on this chip one
            // invalidates the XCD's whole L2, for every step of every
            // workgroup (measured ten times slower overall).
            if (threadIdx.x == 0) {
                int spins = 0;
                while (__hip_atomic_load(sem, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != rank) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > (1 << 24)) {
                        __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
            __syncthreads();
        }
        {
            float* dq_tile = dqa + (long long)i0 * HD;   // uniform base of this query tile
            auto add_dq = [&](auto ragged) {
#pragma unroll
                for (int x = 0; x < C::DQB; ++x) {
                    const int mb = mb_w0 + x * (kWaves / C::NDB);
                    const int col = 32 * db_w + l32;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = 32 * mb + acc_row(v, h);
                        const unsigned o = (unsigned)(r * HD + col);
                        if (!decltype(ragged)::value || i0 + r < si.len_q) atomic_add_f32(dq_tile + o, dq[x][v]);
                    }
                }
            };
            if (i0 + BM <= si.len_q)
                add_dq(std::false_type{});
            else
                add_dq(std::true_type{});
        }
        if (a.deterministic) {
            // every wave's adds have been performed (vmcnt counts atomics
            // until the memory side acknowledges them) before the next
            // contributor is let in; a release fence would also write back
            // the whole L2, which holds nothing the next contributor reads
            wait_vmem();
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_fetch_add(sem, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        }
        // the next tile's copies are complete; on full tiles of the atomic
        // mode this tile's 16 * DQB atomics, issued after them, may still fly
        if (DQ_ATOMIC && !a.deterministic && i0 + BM <= si.len_q)
            wait_vmem_but<16 * C::DQB>();
        else
            wait_vmem();
    }

    // ---- epilogue: dK = s * sum dS^T Q, dV (times 1 / (1 - p) under dropout);
    // rows past the sequence are not written
    const float dv_scale = a.drop.on ? a.drop.rp : 1.f;
    T* dkg = reinterpret_cast<T*>(a.dk) + seq_off(a.sdk, varlen, b, si.k0) + (long long)hkv * a.sdk.h;
    T* dvg = reinterpret_cast<T*>(a.dv) + seq_off(a.sdv, varlen, b, si.k0) + (long long)hkv * a.sdv.h;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int jj = n * kBN + 32 * w + acc_row(v, h);
            if (jj < si.len_k && 32 * d + l32 < a.d) {
                store_elem(dkg, (long long)jj * a.sdk.r + 32 * d + l32, dk[d][v] * a.scale);
                store_elem(dvg, (long long)jj * a.sdv.r + 32 * d + l32, dv[d][v] * dv_scale);
            }
        }
    }
}

int bwd_block_m(int dtype, int head_dim) {
    if (head_dim > 128) return kv_block_m(head_dim);   // no fused kernel at these widths
    if (head_dim == 128) return dtype == ATTN_DTYPE_F32 ? BwdCfg<float, 128>::BM : BwdCfg<bf16_t, 128>::BM;
    static_assert(BwdCfg<bf16_t, 128, true>::BM == BwdCfg<bf16_t, 128, false>::BM, "one query tiling");
    return dtype == ATTN_DTYPE_F32 ? BwdCfg<float, 64>::BM : BwdCfg<bf16_t, 64>::BM;
}

template <class T, int HD>
static void launch_bwd_t(const BwdArgs& a, bool masked, int dq_algo, hipStream_t st) {
    const unsigned grid = (unsigned)(a.nblk_n * a.hkv * a.batch);
    if constexpr (sizeof(T) == 2) {
        // masked: one workgroup per pair of key tiles on grids larger than the
        // GPU; the launch's kv-heads only
        BwdArgs b = a;
        b.pair_tiles = masked && (long long)a.nblk_n * a.hkv_n * a.batch > kComputeUnits;
        const unsigned kv_grid = (unsigned)((b.pair_tiles ? (a.nblk_n + 1) / 2 : a.nblk_n) * a.hkv_n * a.batch);
        static_assert(KvCfg<HD>::BM == BwdCfg<T, HD, false>::BM, "one query tiling");
        static_assert(KvCfg<HD>::BM % kDsRows == 0, "query tiles hold whole dS blocks");
        if (dq_algo == ATTN_DQ_SEPARATE || dq_algo == ATTN_DQ_STORED_DS) {
            launch_kv<T, HD>(b, masked, dq_algo == ATTN_DQ_STORED_DS, a.alibi != nullptr, kv_grid, st);
            return;
        }
    }
    const bool dq_atomic = dq_algo == ATTN_DQ_ATOMIC;
    if (masked) {
        if (dq_atomic) bwd_kernel<T, HD, true, true><<<grid, kThreads, 0, st>>>(a);
        else bwd_kernel<T, HD, true, false><<<grid, kThreads, 0, st>>>(a);
    } else {
        if (dq_atomic) bwd_kernel<T, HD, false, true><<<grid, kThreads, 0, st>>>(a);
        else bwd_kernel<T, HD, false, false><<<grid, kThreads, 0, st>>>(a);
    }
}

void launch_bwd(const BwdArgs& a, int dtype, int hd, bool masked, int dq_algo, hipStream_t st) {
    if (hd == 256) {   // 16-bit types, separate or stored-dS dQ (the ABI maps the atomic mode there)
        launch_bwd_kv_wide(a, dtype, masked, dq_algo == ATTN_DQ_STORED_DS, st);
        return;
    }
    if (dtype == ATTN_DTYPE_BF16) {
        if (hd == 64) launch_bwd_t<bf16_t, 64>(a, masked, dq_algo, st);
        else launch_bwd_t<bf16_t, 128>(a, masked, dq_algo, st);
    } else if (dtype == ATTN_DTYPE_F16) {
        if (hd == 64) launch_bwd_t<f16_t, 64>(a, masked, dq_algo, st);
        else launch_bwd_t<f16_t, 128>(a, masked, dq_algo, st);
    } else {
        if (hd == 64) launch_bwd_t<float, 64>(a, masked, dq_algo, st);
        else launch_bwd_t<float, 128>(a, masked, dq_algo, st);
    }
}

}  // namespace attn
