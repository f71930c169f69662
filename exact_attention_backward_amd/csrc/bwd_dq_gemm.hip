// dQ from stored dS (bf16 or fp16): dQ / s = dS K, the fifth product of the
// Composable Kernel page "block_fmha_bwd_dq_dk_dv_pipeline_trload_kr_ktr_vr.hpp
// Source File" (stage 7), as a pass of its own over the dS blocks the dK/dV
// kernel stored, so that no partial dQ is ever added with atomics.
//
// One workgroup (4 waves) owns 256 query rows of one (sequence, q-head); wave
// w owns the two 32-row dS blocks 8m + 2w and 8m + 2w + 1.  Per 32-key stage
// the workgroup copies the K rows into LDS and each wave its part of its two
// dS blocks (both with buffer_load ... lds, two stages in flight in a ring of
// three; 72 KiB of LDS, so two workgroups share a CU), then each wave adds the
// 64 x 32 product dS K into its fp32 dQ rows:
// the A operands come from the stored operand-register order through two
// transposing LDS reads per 16-key slice and block, the B operand K^T through
// the transposing LDS read too, each B read feeding both blocks' MFMAs.  LDS traffic
// per MFMA, not the matrix cores, bounds this pass besides HBM.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kGWaves = 4;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGXcds = 8;
template <int HD>
struct DqgCfg {
    // 32-row dS blocks per wave: two (their fp32 dQ rows are 2 x HD / 2
    // registers per lane) up to head dim 128, one at 256
    static constexpr int RB = HD <= 128 ? 2 : 1;
    static constexpr int BQ = kGWaves * RB * kDsRows;   // query rows per workgroup
    static constexpr int BN = kDsKeys;              // keys per dS block
    static constexpr int BS = 32;                   // keys per pipeline stage
    static constexpr int SPB = BN / BS;             // stages per dS block
    static constexpr int ROWB = HD * 2;
    static constexpr int K_BYTES = BS * ROWB;
    static constexpr int DS_PART = kDsBlockBytes / SPB;   // one block's part per stage
    static constexpr int STAGE = K_BYTES + kGWaves * RB * DS_PART;
    static constexpr int NS = 3;                    // ring of stages
    static constexpr int PD = NS - 1;               // stages in flight ahead
    static constexpr int LDS_BYTES = NS * STAGE;
    static constexpr int NDB = HD / 32;
    static constexpr int KOPS = BS * (ROWB / 16) / 64 / kGWaves;   // K copy instructions per wave and stage
    static constexpr int OPS = KOPS + RB * DS_PART / 1024;          // copy instructions per wave and stage
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(BS * (ROWB / 16) % (64 * kGWaves) == 0, "K tile split");
    static_assert(OPS * (PD - 1) < 64, "vmcnt range");
};

// Transposing read of a row-major 16-bit tile (see lds_read_tr): lane gets
// M[r1 + t][c0 + lane % 32] and M[r2 + t][c0 + lane % 32], t = 0..3.
template <class T, int ROWB>
__device__ __forceinline__ typename Elem<T>::op_t g_read_col(const char* lds, int r1, int r2, int c0, int lane) {
    const int s = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const u32x2 x = lds_read_tr(lds, swz<ROWB>(r1 + (s >> 2), col * 2));
    const u32x2 y = lds_read_tr(lds, swz<ROWB>(r2 + (s >> 2), col * 2));
    const u32x4 w = {x[0], x[1], y[0], y[1]};
    return __builtin_bit_cast(typename Elem<T>::op_t, w);
}

// s_waitcnt vmcnt(N) alone (lgkmcnt and expcnt left at their maxima): all but
// the N most recently issued VMEM operations are complete.
template <int N>
__device__ __forceinline__ void g_wait_vmem_but() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace

// dQ rows of query tile m (256 rows) of q-head hq in sequence b.
template <class T, int HD, bool MASKED>
__device__ __forceinline__ void gemm_tile(int m, const BwdArgs& a, int b, int hq, int hkv, const SeqInfo& si,
                                          char* smem) {
    using C = DqgCfg<HD>;
    constexpr int BQ = C::BQ, BN = C::BN;
    constexpr int kGRB = C::RB;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int i0 = m * BQ;
    if (i0 >= si.len_q) return;
    const bool varlen = a.cu_q != nullptr;
    const int off = si.len_k - si.len_q;   // bottom-right alignment of the mask
    const int nblk_k = (si.len_k + BN - 1) / BN;
    // the dK/dV kernel's query tiles: KBM rows, KR 32-row blocks each
    constexpr int KBM = kv_block_m(HD), KR = KBM / kDsRows;
    const int G = a.hq / a.hkv;
    // first stored block of query tile mm of this sequence (-1: none stored)
    auto tile_first = [&](int mm) {
        const int idx = a.ds_tile_base[b] + mm;
        return idx < a.ds_tile_base[b + 1] && idx < a.ds_ntiles ? a.ds_prefix[idx] : -1;
    };

    // key blocks a 32-row block can see: first_block .. last_block (last < 0:
    // none, also for a block with no stored dS, which only malformed
    // cu_seqlens produce).  The dK/dV kernel has stored exactly the blocks of
    // each query tile that some row of it sees, a superset of these.
    auto last_block = [&](int lq) {
        if (lq * kDsRows >= si.len_q || tile_first(lq / KR) < 0) return -1;
        if (!MASKED) return nblk_k - 1;
        // the last key the block's last row sees
        const int x = min((lq + 1) * kDsRows, si.len_q) - 1 + off + a.win_hi;
        if (x < 0) return -1;
        const int y = lq * kDsRows + off - a.win_lo;   // the first key its first row sees
        if (y > si.len_k - 1) return -1;
        return min(nblk_k - 1, x / BN);
    };
    auto first_block = [&](int lq) {
        if (!MASKED) return 0;
        const int y = lq * kDsRows + off - a.win_lo;
        return y > 0 ? y / BN : 0;
    };
    const int lq0 = m * (BQ / kDsRows) + kGRB * w;   // this wave's first 32-row block within the sequence
    int n_first_b[kGRB], n_last_b[kGRB];
#pragma unroll
    for (int r = 0; r < kGRB; ++r) {
        n_last_b[r] = last_block(lq0 + r);
        n_first_b[r] = n_last_b[r] < 0 ? nblk_k : first_block(lq0 + r);
    }
    int n_first_w = n_first_b[0], n_last_w = n_last_b[0];
#pragma unroll
    for (int r = 1; r < kGRB; ++r) {
        n_first_w = min(n_first_w, n_first_b[r]);
        n_last_w = max(n_last_w, n_last_b[r]);
    }
    // the workgroup's key blocks: n_first .. n_last over its blocks with rows
    int n_first = nblk_k, n_last = -1;
    for (int lq = m * (BQ / kDsRows); lq < (m + 1) * (BQ / kDsRows); ++lq) {
        const int l = last_block(lq);
        if (l < 0) continue;
        n_last = max(n_last, l);
        n_first = min(n_first, first_block(lq));
    }

    const long long kstride = a.sk.r;   // elements between K rows
    const char* kbytes = reinterpret_cast<const char*>(a.k) +
                         (seq_off(a.sk, varlen, b, si.k0) + (long long)hkv * a.sk.h) * 2;
    // this wave's dS blocks: block r's key block n sits at dsr[r] + n blocks
    // (the tile's first block, + its 32-row block times the tile's key
    // blocks, - the tile's first key block)
    const char* dsr[kGRB];
#pragma unroll
    for (int r = 0; r < kGRB; ++r) {
        const int lq = lq0 + r, mm = lq / KR;
        const KeyRange kr = ds_key_range(mm, KBM, si.len_q, si.len_k, a.win_lo, a.win_hi, MASKED);
        const long long first = n_last_b[r] < 0 ? 0 : tile_first(mm);
        dsr[r] = reinterpret_cast<const char*>(a.ds) +
                 ((long long)(hq - a.hkv0 * G) * a.ds_head_blocks + first + (long long)(lq % KR) * (kr.n1 - kr.n0 + 1) -
                  kr.n0) * kDsBlockBytes;
    }

    const unsigned lds0 = lds_addr(smem);
    // K copy plan: instruction t of wave w fills LDS segment w + 4t of a
    // stage; chunks past the head dim read zeros
    int kvoff[C::KOPS];
#pragma unroll
    for (int t = 0; t < C::KOPS; ++t) {
        constexpr int CPR = C::ROWB / 16;
        const int sl = (w + t * kGWaves) * 64 + lane;
        const int r = sl / CPR;
        const int c = (sl % CPR) ^ swz_key<C::ROWB>(r);
        kvoff[t] = c * 8 < a.d ? r * (int)(kstride * 2) + c * 16 : kOobOff;
    }
    // stage u holds keys BS u .. BS u + BS - 1 (part hf = u % SPB of key block
    // u / SPB) and the matching parts of every wave's dS blocks (zeros for a
    // block whose rows see none of these keys); the stages run from u_beg
    // (the first key block's) to u_end, the v-th of them in ring buffer
    // v % NS.  Every wave issues OPS copies per stage, empty ones past the
    // last stage, so that one wait count serves the whole loop
    const int u_beg = C::SPB * n_first;
    const int u_end = C::SPB * (n_last + 1);
    const int n_stage = max(u_end - u_beg, 0);
    auto issue = [&](int v) {
        const unsigned base = lds0 + (v % C::NS) * C::STAGE;
        const int u = u_beg + v;
        const int n = u / C::SPB, hf = u % C::SPB;
        const bool live = v < n_stage;
        const int rows = live ? max(min(si.len_k - u * C::BS, C::BS), 0) : 0;
        const i32x4 kr = rsrc_words(kbytes + (long long)u * C::BS * kstride * 2, (unsigned)(rows * kstride * 2));
#pragma unroll
        for (int t = 0; t < C::KOPS; ++t) dma_to_lds16(kr, base + (w + t * kGWaves) * 1024, kvoff[t]);
#pragma unroll
        for (int r = 0; r < kGRB; ++r) {
            const bool mine = live && n >= n_first_b[r] && n <= n_last_b[r];
            const i32x4 dr = rsrc_words(dsr[r] + (long long)(mine ? n : 0) * kDsBlockBytes + hf * C::DS_PART,
                                        mine ? C::DS_PART : 0);
#pragma unroll
            for (int t = 0; t < C::DS_PART / 1024; ++t)
                dma_to_lds16_nt(dr, base + C::K_BYTES + (kGRB * w + r) * C::DS_PART + t * 1024, t * 1024 + lane * 16);
        }
    };

    // A operand of a 16-key slice from the stored chunks (see ds_chunk): two
    // transposing reads; in each group of 16 lanes, source lane s points at
    // rows 16c + 4 (s % 4) .. + 3 of key k0 + s / 4 (those rows sit in chunk
    // lane 32 ((s % 4) & 1) + key, bytes 8 ((s % 4) >> 1) ..), so output lane
    // u receives row 16c + u of keys k0 .. k0 + 3 (c = (lane / 16) % 2,
    // k0 = 8 (lane / 32) for the first read, + 4 for the second)
    const int ts = lane & 15, te = ts >> 2, tq = ts & 3;
    const int abase = (((lane >> 4) & 1) * 64 + 32 * (tq & 1) + 8 * (lane >> 5) + te) * 16 + 8 * (tq >> 1);
    const int aoff0 = abase + 64 * (tq & 1), aoff1 = abase + 64 * ((tq & 1) ^ 1);

    f32x16 acc[kGRB][C::NDB];
#pragma unroll
    for (int r = 0; r < kGRB; ++r) {
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[r][d][v] = 0.f;
        }
    }

#pragma unroll
    for (int v = 0; v < C::PD; ++v) issue(v);
    for (int v = 0; v < n_stage; ++v) {
        // stage v has landed for this wave (the PD - 1 later ones may still
        // fly); after the barrier for all, and every wave is done with stage
        // v - 1, whose buffer receives stage v + PD
        g_wait_vmem_but<C::OPS * (C::PD - 1)>();
        __syncthreads();
        issue(v + C::PD);
        const int kb = (u_beg + v) / C::SPB;   // key block of the stage
        if (kb >= n_first_w && kb <= n_last_w) {
            const char* stage = smem + (v % C::NS) * C::STAGE;
            const char* ds = stage + C::K_BYTES + kGRB * w * C::DS_PART;
#pragma unroll
            for (int sl = 0; sl < C::BS / 16; ++sl) {
                // keys 16 sl .. 16 sl + 15 of the stage: pair sl / 2 of its part (one pair
                // when a stage holds 32 keys), keys 16 (sl % 2) ..
                const int so = (2 * (sl >> 1) * 64 + 16 * (sl & 1)) * 16;
                typename Elem<T>::op_t av[kGRB];
#pragma unroll
                for (int r = 0; r < kGRB; ++r) {
                    const u32x2 x = lds_read_tr(ds, r * C::DS_PART + aoff0 + so);
                    const u32x2 y = lds_read_tr(ds, r * C::DS_PART + aoff1 + so);
                    const u32x4 wv = {x[0], x[1], y[0], y[1]};
                    av[r] = __builtin_bit_cast(typename Elem<T>::op_t, wv);
                }
#pragma unroll
                for (int d = 0; d < C::NDB; ++d) {
                    const typename Elem<T>::op_t bk = g_read_col<T, C::ROWB>(stage, 16 * sl + 8 * h, 16 * sl + 8 * h + 4, 32 * d, lane);
#pragma unroll
                    for (int r = 0; r < kGRB; ++r) mma16(acc[r][d], av[r], bk);
                }
            }
        }
    }
    g_wait_vmem_but<0>();   // the empty copies past the end have retired before the waves exit

    // ---- this wave's dQ rows, written once: scaled and converted into dq,
    // or unscaled into the accumulator (the postprocess applies s)
    if (a.dq_out != nullptr) {
        const long long ostride = a.sdq.r;
#pragma unroll
        for (int r = 0; r < kGRB; ++r) {
            const int r0 = (lq0 + r) * kDsRows;
            T* o = reinterpret_cast<T*>(a.dq_out) + seq_off(a.sdq, varlen, b, si.q0) + (long long)hq * a.sdq.h +
                   (long long)r0 * ostride;
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rr = acc_row(v, h);
                    const float y = mul_f32(acc[r][d][v], a.dq_scale);   // rounded to fp32, then to T
                    if (r0 + rr < si.len_q && 32 * d + l32 < a.d)
                        store_elem(o, (long long)rr * ostride + 32 * d + l32, y);
                }
            }
        }
        return;
    }
    const long long row0 = varlen ? (long long)hq * a.total_q + si.q0 : ((long long)b * a.hq + hq) * a.seqlen_q;
#pragma unroll
    for (int r = 0; r < kGRB; ++r) {
        const int r0 = (lq0 + r) * kDsRows;
        float* dqa = a.dq_acc + (row0 + r0) * HD;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rr = acc_row(v, h);
                if (r0 + rr < si.len_q) dqa[(long long)rr * HD + 32 * d + l32] = acc[r][d][v];
            }
        }
    }
}

template <class T, int HD, bool MASKED>
__global__ __launch_bounds__(kGThreads, 1) void bwd_dq_gemm_kernel(BwdArgs a) {
    using C = DqgCfg<HD>;
    constexpr int BQ = C::BQ;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    // ---- which query tiles: all tiles of all q-heads of one (sequence,
    // kv-head) on one XCD, so their K reads share an L2
    const int G = a.hq / a.hkv;
    const int nblk_q = (a.seqlen_q + BQ - 1) / BQ;
    // masked, on grids larger than the GPU (pair_tiles): workgroup p takes
    // query tiles p and nblk_q - 1 - p, whose key ranges add up to the same
    // length for every p (balanced work); else one tile each
    const bool pair = MASKED && a.pair_tiles;
    const int n_pair = pair ? (nblk_q + 1) / 2 : nblk_q;
    const int per_group = n_pair * G;
    int grp, slot;
    {
        const int groups = a.hkv_n * a.batch;
        if (groups % kGXcds == 0) {
            const int xcd = blockIdx.x % kGXcds, s = blockIdx.x / kGXcds;
            grp = (s / per_group) * kGXcds + xcd;
            slot = s % per_group;
        } else {
            grp = blockIdx.x / per_group;
            slot = blockIdx.x % per_group;
        }
    }
    const int hkv = a.hkv0 + grp % a.hkv_n;
    const int b = grp / a.hkv_n;
    const int hq = hkv * G + slot / n_pair;
    const int p = slot % n_pair;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    const int nblk_q_seq = (si.len_q + BQ - 1) / BQ;   // this sequence's query tiles
    if (MASKED) {
        // the longer tile first, then its partner (once the first tile's LDS
        // stages are no longer read); unpaired: tile p alone
        const int m2 = pair ? nblk_q_seq - 1 - p : p;
        if (m2 > p) {
            gemm_tile<T, HD, MASKED>(m2, a, b, hq, hkv, si, smem);
            __syncthreads();
        }
        if (p < nblk_q_seq && p <= m2) gemm_tile<T, HD, MASKED>(p, a, b, hq, hkv, si, smem);
    } else {
        gemm_tile<T, HD, MASKED>(p, a, b, hq, hkv, si, smem);
    }
}

template <class T, int HD>
static void launch_dq_gemm_hd(const BwdArgs& a0, bool masked, hipStream_t st) {
    BwdArgs a = a0;
    const int nblk_q = (a.seqlen_q + DqgCfg<HD>::BQ - 1) / DqgCfg<HD>::BQ;
    // pairs of query tiles on grids larger than the GPU
    a.pair_tiles = masked && (long long)nblk_q * (a.hq / a.hkv) * a.hkv_n * a.batch > kComputeUnits;
    const int n_pair = a.pair_tiles ? (nblk_q + 1) / 2 : nblk_q;   // workgroups per (sequence, q-head)
    const unsigned grid = (unsigned)(n_pair * (a.hq / a.hkv) * a.hkv_n * a.batch);
    if (masked) bwd_dq_gemm_kernel<T, HD, true><<<grid, kGThreads, 0, st>>>(a);
    else bwd_dq_gemm_kernel<T, HD, false><<<grid, kGThreads, 0, st>>>(a);
}
template <class T>
static void launch_dq_gemm_t(const BwdArgs& a, int hd, bool masked, hipStream_t st) {
    if (hd == 64) launch_dq_gemm_hd<T, 64>(a, masked, st);
    else if (hd == 128) launch_dq_gemm_hd<T, 128>(a, masked, st);
    else launch_dq_gemm_hd<T, 256>(a, masked, st);
}

void launch_bwd_dq_gemm(const BwdArgs& a, int dtype, int hd, bool masked, hipStream_t st) {
    if (dtype == ATTN_DTYPE_F16) launch_dq_gemm_t<f16_t>(a, hd, masked, st);
    else launch_dq_gemm_t<bf16_t>(a, hd, masked, st);
}

}  // namespace attn
