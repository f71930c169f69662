// The dK/dV kernel with split wave roles (bwd_kv_kernel) of the stored-dS and
// separate dQ modes, as a template header: bwd_main.hip instantiates it for
// head dims up to 128 and bwd_kv_wide.hip for up to 256 (compiled with its
// own register-allocation flags).
#pragma once

#include <type_traits>

#include "bwd_shared.h"

namespace attn {

// --------------------------------------------------------------------------
// dK/dV kernel with split wave roles (16-bit types, dQ left to another
// pass).  Same key tiling and dispatch as bwd_kernel, but eight waves per
// workgroup, two per SIMD: the 32 keys of pair p (keys 32p..32p+31) are
// shared by a "P wave" (waves 0-3) and a "dS wave" (waves 4-7).  Per query
// tile t:
//
//   P wave : X = Q K^T (stage 1), P = exp2(X s log2e - LSE log2e) (stage 2),
//            P to LDS for its partner, dV += P^T dO (stage 3)
//   dS wave: X = dO V^T (stage 4) for tile t; for tile t-1, with the P its
//            partner left in LDS: dS = P (dP - D) (stage 5), dK += dS^T Q (stage 6)
//
// Each wave holds one K or V slice (its B operand) and one accumulator, so
// both fit in the register budget of two waves per SIMD, and the two waves
// of a SIMD overlap each other's MFMA, exponential and LDS work.  The dS wave
// runs one tile behind so that a single barrier per tile publishes P.
// Query-side tiles (Q, dO, LSE, D) are prefetched two tiles ahead into a
// ring of four LDS buffers (the dS wave still reads tile t-1).
//
// The loop body is kept lean: the loops are unrolled by the ring length, so
// every LDS address is a per-lane constant plus an immediate (the swizzle
// only permutes address bits the ring offsets leave zero), tile coordinates
// advance incrementally, and every wave issues the same three copies per
// tile (past the last tile with a scalar offset beyond every range), so each
// wait count is a constant.
//
// Masking: a padded query row (past the sequence) has Q = dO = 0 and
// LSE = D = 0 in LDS, so its P is finite and its P dO and dS terms are zero;
// a padded key only affects its own dK/dV rows, which are not stored.  Only
// the tiles a causal or window bound crosses need a mask.
// --------------------------------------------------------------------------
// Head dims up to 128: eight waves (two per SIMD, four key pairs, 128 keys
// per workgroup).  Up to 256: four waves (one per SIMD, whose registers then
// hold the twice as wide operand and accumulator), two pairs, 64 keys.
template <int HD>
struct KvCfg {
    static constexpr int NW = HD <= 128 ? 8 : 4;     // waves per workgroup
    static constexpr int NP = NW / 2;                // key pairs: a P wave and a dS wave each
    static constexpr int KBN = 32 * NP;              // keys per workgroup (a key tile)
    static constexpr int KPB = kDsKeys / KBN;        // key tiles per 128-key dS block
    static constexpr int BM = kv_block_m(HD);        // query rows per tile
    static constexpr int ROWB = HD * 2;
    static constexpr int TILE = BM * ROWB;
    static constexpr int NBUF = 4;                   // ring of query-side tile buffers
    static constexpr int PD = NBUF - 2;              // prefetch distance in tiles
    static constexpr int BUF_Q = 0, BUF_DO = TILE, BUF_LSE = 2 * TILE, BUF_DL = 2 * TILE + 256;
    static constexpr int BUF_DUMP = 2 * TILE + 512;   // target of the empty statistic copies
    static constexpr int BUF_BYTES = 2 * TILE + 768;
    static constexpr int NMB = BM / 32;              // 32-row blocks of a query tile
    static constexpr int NIC = BM / 16;              // 16-wide chunks of the query rows
    static constexpr int PSLOT = NIC * 16 * 64;      // P of one pair: its NIC operand chunks per lane
    static constexpr int OFF_P = NBUF * BUF_BYTES;   // [pair][tile parity] P slots
    static constexpr int OFF_CONST = OFF_P + NP * 2 * PSLOT;   // 16 bytes per wave, see kv_tile
    static constexpr int LDS_BYTES = OFF_CONST + NW * 16;
    // elementwise bias: per P wave a [BM rows][32 keys] image (64-byte rows)
    // in each of two buffers (tile parity), copied one tile ahead
    static constexpr int BIAS_PAIR = BM * 64;
    static constexpr int OFF_BIAS = (LDS_BYTES + 1023) / 1024 * 1024;
    // dBias (dS wave): the tile's dS, key-major (one key's BM rows, padded
    // by 8 bytes against bank conflicts), read back row-major for 16-byte stores
    static constexpr int DBIMG_ROWB = 2 * BM + 8;
    static constexpr int DBIMG = 32 * DBIMG_ROWB;
    static constexpr int OFF_DBIMG = OFF_BIAS + 2 * NP * BIAS_PAIR;
    static constexpr int LDS_BYTES_BIAS = OFF_DBIMG + NP * DBIMG;
    static constexpr int BOPS = BM / 16;             // bias copies per tile and P wave (16 rows each)
    static constexpr int NDBW = BM / 16;             // dBias stores per tile and dS wave (16 bytes each)
    static constexpr int NDBS = BM / 2;              // the same one element each (unaligned dBias, ragged keys)
    static constexpr int NC = HD / 16;               // 16-wide chunks of the head dim
    static constexpr int NDB = HD / 32;              // 32-column blocks of the head dim
    static constexpr int SEG = TILE / 1024 / NW;     // 1 KiB segments of a Q or dO tile per wave
    static constexpr int OPS = 2 * SEG + 1;          // copy instructions per tile and wave
    static_assert(TILE % (1024 * NW) == 0, "whole segments per wave");
    static_assert(KBN * KPB == kDsKeys, "key tiles tile a dS block");
    static_assert(LDS_BYTES_BIAS <= 160 * 1024, "LDS budget");
    static_assert(BUF_BYTES % 256 == 0 && TILE % 256 == 0, "XOR addressing needs 256-byte aligned tiles");
    static_assert(BM * 4 <= 256, "LSE/D tile in one 256-byte slot");
};

// All work of one key tile n of sequence b, kv-head hkv (the body of
// bwd_kv_kernel).  ALIBI: ALiBi slopes; BIAS: an elementwise bias (and ALiBi
// too when slopes are given) and, when dbias is set, its gradient dS; DROP
// (with BIAS): dropout of P as well.  Under dropout the P wave passes P to
// its partner with the sign bit set on dropped elements (P >= 0 otherwise),
// feeds the kept P to dV, and the dS wave forms P (dP / (1 - p) - D) on kept
// and -P D on dropped elements.
template <class T, int HD, bool MASKED, bool STORE_DS, bool ALIBI, bool BIAS, bool DROP>
__device__ __forceinline__ void kv_tile(const BwdArgs& a, int b, int hkv, int n, const SeqInfo& si, char* smem) {
    static_assert(sizeof(T) == 2, "16-bit operand types");
    using C = KvCfg<HD>;
    using op_t = typename Elem<T>::op_t;
    constexpr int BM = C::BM, NMB = C::NMB, ROWB = C::ROWB;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = w / C::NP;   // 0: P wave (S, P, dV), 1: dS wave (dP, dS, dK)
    const int pair = w % C::NP;   // keys 32 * pair .. + 31 of the tile
    constexpr int KBN = C::KBN;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    // keys whose query range the tile takes: its own, or with the stored dS
    // and tiles smaller than a dS block (KPB > 1) the whole block's, since
    // the tile writes its part of the block for every query tile that
    // stores the block (the query tiles outside its own keys' range are
    // fully masked and store zeros), also when the part lies past the keys
    constexpr bool BLOCK_RANGE = STORE_DS && C::KPB > 1;
    const int kr0 = BLOCK_RANGE ? n / C::KPB * kDsKeys : n * KBN;
    const int kr1 = BLOCK_RANGE ? kr0 + kDsKeys : n * KBN + KBN;
    if (kr0 >= si.len_k) return;
    const bool varlen = a.cu_q != nullptr;
    const int G = a.hq / a.hkv;
    const int off = si.len_k - si.len_q;   // bottom-right alignment of the mask
    int m_begin = 0, m_end = (si.len_q + BM - 1) / BM;
    if (MASKED) {
        // query rows that see some key of the range: from the first row whose
        // upper bound reaches its first key to the last row whose lower bound
        // still admits its last key
        const int first_row = kr0 - off - a.win_hi;
        const int last_row = min(kr1, si.len_k) - 1 - off + a.win_lo;
        m_begin = first_row > 0 ? first_row / BM : 0;
        m_end = last_row < 0 ? 0 : min(last_row, si.len_q - 1) / BM + 1;
    }
    const int n_m = max(m_end - m_begin, 0);
    const int n_tiles = G * n_m;            // (q-head, query tile) pairs, q-head major

    // this wave's K (P wave) or V (dS wave) rows, and the dV (P wave) or dK
    // (dS wave) rows it writes: element offsets of the kv-head's first row
    // and the row strides
    const Strides& s_in = role == 0 ? a.sk : a.sv;
    const long long in_base = seq_off(s_in, varlen, b, si.k0) + (long long)hkv * s_in.h;
    const Strides& s_out = role == 0 ? a.sdv : a.sdk;
    const long long out_base = seq_off(s_out, varlen, b, si.k0) + (long long)hkv * s_out.h;

    // ---- per-lane LDS offsets, fixed for the whole kernel
    const unsigned lds0 = lds_addr(smem);
    // row operand of the first product: row 32 mb + l32, chunk 2c + h at (rbase ^ 32c) + mb * 32 ROWB
    const int rbase = swz<ROWB>(l32, 16 * h);
    // column operand of the second product: rows 16c + 8e + 4h + (lane % 16) / 4,
    // columns 32d + 16 ((lane / 16) % 2) + 4 (lane % 4), at (tbase[e] ^ 64d) + c * 16 ROWB
    const int s16 = lane & 15;
    const int tcol = 2 * (16 * ((lane >> 4) & 1) + 4 * (s16 & 3));
    const int tbase0 = swz<ROWB>(4 * h + (s16 >> 2), tcol);
    const int tbase1 = swz<ROWB>(8 + 4 * h + (s16 >> 2), tcol);
    const int tile_off = role == 0 ? C::BUF_Q : C::BUF_DO;    // row operand of the first product
    const int col_off = role == 0 ? C::BUF_DO : C::BUF_Q;     // column operand of the second
    const int pslots = C::OFF_P + pair * 2 * C::PSLOT;

    // ---- copies: this wave's 1 KiB segments w + s NW (s < SEG) of the Q and
    // dO tiles, then LSE (wave 0), D (wave 1) or an empty copy (the others).
    // Row strides in bytes; chunks past the head dim read zeros.
    const int qrow_b = (int)(a.sq.r * (long long)sizeof(T)), dorow_b = (int)(a.sdo.r * (long long)sizeof(T));
    int seg_voff_q[C::SEG], seg_voff_do[C::SEG];
#pragma unroll
    for (int sg = 0; sg < C::SEG; ++sg) {
        constexpr int CPR = ROWB / 16;
        const int slot = (w + sg * C::NW) * 64 + lane;
        const int r = slot / CPR;
        const int c = (slot % CPR) ^ swz_key<ROWB>(r);
        const bool ok = c * 16 < a.d * (int)sizeof(T);
        seg_voff_q[sg] = ok ? r * qrow_b + c * 16 : kOobOff;
        seg_voff_do[sg] = ok ? r * dorow_b + c * 16 : kOobOff;
    }
    // bytes between q-heads (the ABI keeps head strides below 2 GiB), needed
    // once per n_m tiles: each wave parks them in its own LDS slot and reads
    // them back at a head change, so they do not occupy scalar registers
    // across the loops
    char* wconst = smem + C::OFF_CONST + w * 16;
    if (lane == 0) {
        const u32x4 hb = {(unsigned)(a.sq.h * (long long)sizeof(T)), (unsigned)(a.sdo.h * (long long)sizeof(T)),
                          (unsigned)(varlen ? a.total_q : a.seqlen_q) * 4u, 0u};
        *reinterpret_cast<u32x4*>(wconst) = hb;
    }
    // the group's first q-head, first query tile in Q, dO and LSE/D (this
    // wave's statistic); the descriptors step from there one head at a time
    const char* q_head = reinterpret_cast<const char*>(a.q) +
                         (seq_off(a.sq, varlen, b, si.q0) + (long long)m_begin * BM * a.sq.r +
                          (long long)hkv * G * a.sq.h) * (long long)sizeof(T);
    const char* do_head = reinterpret_cast<const char*>(a.dout) +
                          (seq_off(a.sdo, varlen, b, si.q0) + (long long)m_begin * BM * a.sdo.r +
                           (long long)hkv * G * a.sdo.h) * (long long)sizeof(T);
    const char* l_head =
        (w == 0 ? reinterpret_cast<const char*>(a.lse) : reinterpret_cast<const char*>(a.delta)) +
        ((varlen ? (long long)hkv * G * a.total_q + si.q0 : ((long long)b * a.hq + (long long)hkv * G) * a.seqlen_q) +
         m_begin * BM) * 4;
    // issue cursor: the next tile to copy.  The descriptors point at the
    // current q-head's first tile; a tile's offset from there goes into the
    // scalar offset.  The range word (which the scalar offset counts against)
    // ends at the sequence's last row, the same for every head, so rows past
    // the sequence read zeros; the empty copies past the last tile take a
    // scalar offset past every range.
    int is_t = 0, is_m = m_begin;
    const int full_q = BM * qrow_b, full_do = BM * dorow_b;   // bytes between query tiles
    const int rows_left = max(si.len_q - m_begin * BM, 0);   // rows from the first tile to the sequence end
    i32x4 rq = rsrc_words(q_head, (unsigned)(rows_left * qrow_b));
    i32x4 rdo = rsrc_words(do_head, (unsigned)(rows_left * dorow_b));
    i32x4 rs = rsrc_words(l_head, w < 2 ? (unsigned)rows_left * 4u : 0u);
    // LDS bases of this wave's copies: its 1 KiB segment of the Q tile (dO
    // follows at a constant distance) and its statistic slot (LSE, D, or the
    // dump slot of the other waves); a buffer's ring offset is an immediate
    const unsigned seg_base = lds0 + C::BUF_Q + w * 1024;
    const unsigned stat_base = lds0 + (w == 0 ? C::BUF_LSE : w == 1 ? C::BUF_DL : C::BUF_DUMP);
    auto issue_next = [&](auto iss_c) {   // iss_c: ring offset of the tile's buffer (a constant)
        constexpr unsigned ISB = decltype(iss_c)::value;
        const bool live = is_t < n_tiles;
        const int rel = is_m - m_begin;   // the tile's offset from the head's first tile, in tiles
        const int so_q = live ? rel * full_q : kOobOff, so_do = live ? rel * full_do : kOobOff;
        if constexpr (C::SEG == 1) {
            dma_to_lds16_at<ISB>(rq, seg_base, seg_voff_q[0], so_q);
            dma_to_lds16_at<ISB + C::BUF_DO - C::BUF_Q>(rdo, seg_base, seg_voff_do[0], so_do);
        } else {
            static_assert(C::SEG == 4, "segment counts of the configurations");
            dma_to_lds16_at<ISB>(rq, seg_base, seg_voff_q[0], so_q);
            dma_to_lds16_at<ISB + C::NW * 1024>(rq, seg_base, seg_voff_q[1], so_q);
            dma_to_lds16_at<ISB + 2 * C::NW * 1024>(rq, seg_base, seg_voff_q[2], so_q);
            dma_to_lds16_at<ISB + 3 * C::NW * 1024>(rq, seg_base, seg_voff_q[3], so_q);
            constexpr unsigned D0 = ISB + C::BUF_DO - C::BUF_Q;
            dma_to_lds16_at<D0>(rdo, seg_base, seg_voff_do[0], so_do);
            dma_to_lds16_at<D0 + C::NW * 1024>(rdo, seg_base, seg_voff_do[1], so_do);
            dma_to_lds16_at<D0 + 2 * C::NW * 1024>(rdo, seg_base, seg_voff_do[2], so_do);
            dma_to_lds16_at<D0 + 3 * C::NW * 1024>(rdo, seg_base, seg_voff_do[3], so_do);
        }
        dma_to_lds4_at<ISB>(rs, stat_base, lane * 4, live ? rel * (BM * 4) : kOobOff);
        ++is_t;
        if (++is_m == m_end) {
            is_m = m_begin;
            // the next q-head (once per n_m tiles)
            const u32x4 hb = *reinterpret_cast<const u32x4*>(wconst);
            rsrc_advance(rq, __builtin_amdgcn_readfirstlane(hb[0]));
            rsrc_advance(rdo, __builtin_amdgcn_readfirstlane(hb[1]));
            rsrc_advance(rs, __builtin_amdgcn_readfirstlane(hb[2]));
        }
    };

    // ---- prologue: the first query-side tiles, then this wave's K (P wave)
    // or V (dS wave) rows as B operands.  The wait for all of them here tells
    // the compiler that the K/V registers are ready; otherwise it would wait
    // for them (vmcnt(0), the prefetches included) inside the loop.
    static_assert(C::PD == 2, "the prologue issues two tiles");
    issue_next(std::integral_constant<unsigned, 0>{});
    issue_next(std::integral_constant<unsigned, C::BUF_BYTES>{});
    op_t wreg[C::NC];
    {
        const T* src = reinterpret_cast<const T*>(role == 0 ? a.k : a.v) + in_base;
        const int j = n * KBN + 32 * pair + l32;
        const bool ok = j < si.len_k;
#pragma unroll
        for (int c = 0; c < C::NC; ++c)
            wreg[c] = load_op_global<T>(src + (long long)j * s_in.r + 16 * c + 8 * h, ok && 16 * c + 8 * h < a.d);
    }
    // ALiBi: lane g holds the slope of the group's q-head g (groups of up to
    // 64 q-heads; larger ones read the slope per tile)
    float slope_v = 0.f;
    if ((ALIBI || (BIAS && a.alibi != nullptr)) && lane < G) slope_v = a.alibi[hkv * G + lane];

    // ---- elementwise bias (P wave): the [BM rows][32 keys] block of tile
    // t + 1 is copied during step t into the bias buffer of t + 1's parity,
    // before the tile copies of that step, so the wait at the top of step
    // t + 1 covers it.  Lane L copies row L / 4 (+ 16 per copy), keys
    // 8 (L % 4) .. + 7 of the pair.  The range ends with the tile's last
    // valid row, at its valid keys rounded up to a 16-byte chunk (inside the
    // row: bias rows are 16-byte aligned); later rows read zeros.
    const long long sbr_b = a.sbias.r * (long long)sizeof(T);
    const int bias_voff = BIAS ? (int)((lane >> 2) * sbr_b) + pair * 64 + (lane & 3) * 16 : 0;
    const unsigned bias_lds = lds0 + C::OFF_BIAS + pair * C::BIAS_PAIR;
    auto issue_bias = [&](auto buf_c, int m, int g) {
        constexpr unsigned BB = decltype(buf_c)::value * C::NP * C::BIAS_PAIR;
        const char* base = reinterpret_cast<const char*>(a.bias) +
                           ((long long)b * a.sbias.b + (long long)(hkv * G + g) * a.sbias.h +
                            (long long)m * BM * a.sbias.r + (long long)n * KBN) * (long long)sizeof(T);
        const int rows = min(BM, si.len_q - m * BM);
        const unsigned bytes = a.bias == nullptr ? 0u   // dBias without a bias: zeros
                                                 : (unsigned)((rows - 1) * sbr_b) +
                                                       (unsigned)((max(si.len_k - n * KBN, 0) * (int)sizeof(T) + 15) & ~15);
        const i32x4 rb = rsrc_words(base, bytes);
#pragma unroll
        for (int k = 0; k < C::BOPS; ++k)
            dma_to_lds16_so(rb, bias_lds + BB + k * 1024, bias_voff, (int)(k * 16 * sbr_b));
    };
    if (BIAS && role == 0 && n_tiles > 0) issue_bias(std::integral_constant<unsigned, 0>{}, m_begin, 0);
    wait_vmem();

    f32x16 acc[C::NDB];   // dV rows (P wave) or unscaled dK rows (dS wave) of this pair's keys
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;
    }
    const float scale2 = a.scale * kLog2e;
    const int j = n * KBN + 32 * pair + l32;   // this lane's key (column of S)
    // a query tile starting at row i0 needs the mask iff i0 < diag_hi (some
    // key past a row's upper bound) or i0 > diag_lo (some key before a
    // row's lower bound)
    const int diag_hi = n * KBN + KBN - 1 - off - a.win_hi;
    const int diag_lo = n * KBN - off + a.win_lo - BM + 1;
    int cur_m = m_begin;                       // query tile of tile t
    int cur_g = 0;                             // q-head (within the group) of tile t
    // stored-dS mode: whether the key tile reaches past the sequence (its dS
    // columns are then zeroed), and the dS blocks of tile t and of tile t-1:
    // block (32-row block r, this key tile) of a tile at ptr + r * stride, or
    // none (ptr null: the table stores nothing for the tile, which only
    // malformed cu_seqlens produce; its stores get an empty range).  A tile's
    // first block (the same in every q-head's region) comes from the table
    // for the range's first tile only and then advances by each tile's
    // blocks: a table read inside the loop would wait for every copy in
    // flight (vmcnt counts both)
    const bool ragged_k = n * KBN + KBN > si.len_k;
    const int ds_t0 = STORE_DS ? a.ds_tile_base[b] : 0;
    const int ds_t1 = STORE_DS ? min(a.ds_tile_base[b + 1], a.ds_ntiles) : 0;
    // A tile's first block is the same in every q-head's region.  The table
    // gives the range's first tile's; the others follow by adding each
    // tile's blocks (a table read inside the loop would wait for every copy
    // in flight: vmcnt counts both).  The table's entries only grow along a
    // sequence, and a tile whose blocks would overflow the region is -1
    // (only malformed cu_seqlens make one), so checking the range's first and
    // last tiles once covers every tile; a key tile that fails stores nothing.
    const int ds_first0 = STORE_DS && n_m > 0 && ds_t0 + m_end <= ds_t1 && a.ds_prefix[ds_t0 + m_end - 1] >= 0
                              ? a.ds_prefix[ds_t0 + m_begin]
                              : -1;
    const char* ds_head0 = STORE_DS ? reinterpret_cast<const char*>(a.ds) +
                                          (long long)(hkv - a.hkv0) * G * a.ds_head_blocks * kDsBlockBytes
                                    : nullptr;
    // Cursor over the query tiles of one q-head: the key range n0 .. n1 of
    // tile m (ds_key_range's, here never empty: every tile visited sees key
    // tile n; from one tile to the next both bounds' arguments x, y grow by
    // BM) and blk, the index of block (0, key tile n) in the q-head's region
    struct DsCursor {
        int x, y, n0, cnt, blk;
    };
    const int ds_nblk = (si.len_k + kDsKeys - 1) / kDsKeys;
    auto ds_range = [&](DsCursor& c) {
        int n1 = ds_nblk - 1;
        c.n0 = 0;
        if (MASKED) {
            c.n0 = c.x <= kDsKeys ? 0 : (c.x + kDsKeys - 1) / kDsKeys - 1;
            n1 = min(ds_nblk - 1, c.y / kDsKeys);
        }
        c.cnt = n1 - c.n0 + 1;
    };
    auto ds_start = [&](DsCursor& c) {   // the q-head's first tile
        c.x = m_begin * BM + off - a.win_lo + 1;
        c.y = (m_begin + 1) * BM - 1 + off + a.win_hi;
        ds_range(c);
        c.blk = ds_first0 + n / C::KPB - c.n0;
    };
    DsCursor ds_cur{};   // tile t
    if (STORE_DS) ds_start(ds_cur);
    const char* ds_head = ds_first0 >= 0 ? ds_head0 : nullptr;   // region of tile t's q-head (null: no stores)
    struct DsBlocks {
        const char* head;
        int blk, cnt;
    };
    DsBlocks ds_last{ds_head, ds_cur.blk, ds_cur.cnt};   // tile t-1: what its stores need
    constexpr int NST = STORE_DS ? 2 * NMB : 0;   // dS stores per dS-wave step
    // dBias stores per dS-wave step: NDBW 16-byte stores, or NDBS element
    // stores where dBias rows are not 16-byte aligned or the key tile is
    // ragged.  The wait counts assume the smaller number: more stores issued
    // after a tile's copies only make a wait stricter.
    constexpr int NDB = BIAS ? C::NDBW : 0;
    constexpr int NSTW = NST + NDB;
    // dBias (dS wave): element (row r of tile t-1, this lane's key j) goes to
    // the tile's first row + r * row stride + j, one 16-bit store each.  Keys
    // past the sequence take an offset past every range; rows past it fall
    // outside the range (it ends at the last valid row's last key).
    const long long sdbr_b = a.sdbias.r * (long long)sizeof(T);
    // (not with dropout, whose kernel has no registers to spare for it)
    const bool db_wide = BIAS && !DROP && a.dbias != nullptr && n * KBN + KBN <= si.len_k &&
                         ((reinterpret_cast<unsigned long long>(a.dbias) |
                           (unsigned long long)(a.sdbias.b * (long long)sizeof(T)) |
                           (unsigned long long)(a.sdbias.h * (long long)sizeof(T)) | (unsigned long long)sdbr_b) &
                          15) == 0;
    const int db_voff = j < si.len_k ? (int)(4 * h * sdbr_b) + (32 * pair + l32) * (int)sizeof(T) : kOobOff;
    int db_m = m_begin, db_g = 0;   // dS wave: query tile and q-head of tile t-1
    // P wave's transposing reads of its bias image: lane (l32, h) gets key
    // l32 of rows r0 + 4h + 0..3 (see lds_read_tr; source lane s of each
    // 16-lane group points at row r0 + 4h + s / 4, keys 16 * (lane / 16 % 2) + 4 (s % 4))
    const int bias_rd = C::OFF_BIAS + pair * C::BIAS_PAIR + (((lane & 15) >> 2) + 4 * h) * 64 +
                        2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    // one step: tile t for the P wave, tiles t (first product) and t-1 for the dS wave
    auto step = [&](auto role_c, auto first_c, auto k_c, int t, f32x16* xc, f32x16* xp) {
        constexpr int R = decltype(role_c)::value;   // this wave's role, a constant per loop
        constexpr bool FIRST = decltype(first_c)::value;   // the dS wave's first step (no tile t-1)
        // ring buffers of tiles t, t-1 and t+PD (t = K mod NBUF), compile-time
        // constants: LDS addresses are per-lane constants plus immediate offsets
        constexpr int K = decltype(k_c)::value;
        constexpr unsigned CUR = K * C::BUF_BYTES;
        constexpr unsigned PREV = ((K + C::NBUF - 1) % C::NBUF) * C::BUF_BYTES;
        constexpr unsigned ISS = ((K + C::PD) % C::NBUF) * C::BUF_BYTES;
        // this wave's copies of tile t have landed (those of the PD - 1 later
        // tiles may still fly); after the barrier all waves' have, P of tile
        // t-1 is in LDS, and every wave is done with tile t-2, whose buffer
        // receives tile t+3
        // in the stored-dS and bias variants each dS-wave step also issues
        // NSTW stores (dS, dBias), before its copies, so the copies of tile t
        // are counted past the stores of the PD - 1 later steps (the first
        // step has no dS; it stores an empty range instead, to keep the count)
        if (NSTW > 0 && R == 1)
            wait_vmem_but<C::OPS * (C::PD - 1) + NSTW * (C::PD - 1)>();
        else
            wait_vmem_but<C::OPS * (C::PD - 1)>();
        __syncthreads();
        const int i0 = cur_m * BM;
        const int g_t = cur_g;   // tile t's q-head within the group
        // ALiBi slope of tile t's q-head, negated, in log2 units
        float nsl2 = 0.f;
        if constexpr ((ALIBI || BIAS) && R == 0) {
            const float sl = G <= 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                     __builtin_bit_cast(int, slope_v), cur_g))
                                     : (a.alibi != nullptr ? load_uniform_f32(a.alibi, hkv * G + cur_g) : 0.f);
            nsl2 = -sl * kLog2e;
        }
        // row statistics of the tile whose second product comes in this step,
        // read now so their latency hides behind the first product: LSE of
        // tile t (P wave), or D and the partner's P of tile t-1 (dS wave)
        const float* lst = reinterpret_cast<const float*>(
            smem + (R == 0 ? CUR + C::BUF_LSE : PREV + C::BUF_DL) + 16 * h);
        f32x4 stat[NMB * 4];
        u32x4 pin[C::NIC];
#pragma unroll
        for (int q = 0; q < NMB * 4; ++q) stat[q] = *reinterpret_cast<const f32x4*>(lst + 8 * q);
        // the bias of tile t (P wave): rows 32 mb + 8 q4 + 4h + 0..3 of this lane's key
        u32x2 bia[BIAS && R == 0 ? NMB * 4 : 1];
        if constexpr (BIAS && R == 0) {
#pragma unroll
            for (int q = 0; q < NMB * 4; ++q)
                bia[q] = lds_read_tr(smem, bias_rd + (K & 1) * C::NP * C::BIAS_PAIR + q * 8 * 64);
        }
        if constexpr (R == 1) {
            const int psr = pslots + ((K + 1) & 1) * C::PSLOT + lane * 16;   // slot of tile t-1
#pragma unroll
            for (int c = 0; c < C::NIC; ++c) pin[c] = *reinterpret_cast<const u32x4*>(smem + psr + c * 1024);
        }

        // ---- X = Q K^T (P wave) or dO V^T (dS wave) for tile t, then the
        // copies of tile t + PD.  Steps start with it, except the dS wave's
        // in the stored-dS variant, which end with it: there the dS, dK and
        // dS-store work for tile t-1 goes first, while the P wave of the same
        // SIMD computes the exponentials of tile t (measured 1.8% faster with
        // the stores, 0.8% slower without them)
        constexpr bool DS_LATE = R == 1 && NSTW > 0;
        auto first_product = [&]() {
        if (t < n_tiles) {
            // the swizzle XOR touches only address bits 5-7, which are zero
            // in the ring offset, so the offset is an immediate
            const int rb = tile_off + rbase;
            op_t ra[C::NC];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
                for (int c = 0; c < C::NC; ++c)
                    ra[c] = __builtin_bit_cast(op_t, lds_read16(smem, (rb ^ (32 * c)) + (int)CUR + mb * 32 * ROWB));
#pragma unroll
                for (int v = 0; v < 16; ++v) xc[mb][v] = 0.f;
#pragma unroll
                for (int c = 0; c < C::NC; ++c) mma16(xc[mb], ra[c], wreg[c]);
            }
            // all operand reads first, so the MFMA chain does not wait on LDS latency
            __builtin_amdgcn_sched_group_barrier(0x100, NMB * C::NC, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NMB * C::NC, 0);
        }
        if constexpr (BIAS && R == 0) {
            // the bias of tile t + 1 (the q-head's next query tile, or the next
            // q-head's first)
            if (t + 1 < n_tiles) {
                const bool wrap = cur_m + 1 == m_end;
                issue_bias(std::integral_constant<unsigned, (K + 1) & 1>{}, wrap ? m_begin : cur_m + 1,
                           wrap ? cur_g + 1 : cur_g);
            }
        }
        issue_next(std::integral_constant<unsigned, ISS>{});
        };
        if constexpr (!DS_LATE) first_product();
        const DsBlocks ds_prev = ds_last;           // dS blocks of tile t-1
        if (STORE_DS) ds_last = DsBlocks{ds_head, ds_cur.blk, ds_cur.cnt};
        const int dbm = db_m, dbg = db_g;            // query tile and q-head of tile t-1
        if (BIAS && R == 1) {
            db_m = cur_m;
            db_g = cur_g;
        }
        bool new_head = false;
        if (++cur_m == m_end) {
            cur_m = m_begin;
            ++cur_g;
            new_head = true;
        }
        // the dS blocks of tile t+1, worked out at the end of the step, while
        // its last MFMAs run (here, after the barrier, they delayed the step)
        auto advance_ds = [&]() {
            if (STORE_DS && R == 1) {
                if (new_head) {
                    if (ds_head) ds_head += (long long)a.ds_head_blocks * kDsBlockBytes;
                    ds_start(ds_cur);
                } else {
                    const int n0 = ds_cur.n0, blocks = (BM / kDsRows) * ds_cur.cnt;
                    ds_cur.x += BM;
                    ds_cur.y += BM;
                    ds_range(ds_cur);
                    ds_cur.blk += blocks + n0 - ds_cur.n0;
                }
            }
        };
        // the tile whose second product this wave computes now
        const int tt = R == 0 ? t : t - 1;   // the dS wave's later steps always have a tile t-1
        if (FIRST || (R == 0 && tt >= n_tiles)) {
            if (NSTW > 0 && FIRST) {   // the dS wave's first step: empty stores
                const rsrc_t none = make_rsrc(STORE_DS ? a.ds : a.dbias, 0);
                const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < NSTW; ++k) __builtin_amdgcn_raw_buffer_store_b128(z, none, lane * 16, 0, 2);
            }
            if constexpr (DS_LATE) first_product();
            advance_ds();
            return;
        }
        constexpr unsigned buf = R == 0 ? CUR : PREV;
        const int ps = pslots + ((R == 0 ? K : K + 1) & 1) * C::PSLOT + lane * 16;   // slot of tile tt
        op_t opa[C::NIC];
        if constexpr (R == 0) {
            // ---- P = exp2(S s log2e - LSE log2e), masked on the tiles the mask crosses
            const int dj = j - (i0 + off + 4 * h);   // key column relative to this lane's first row
            const int dj_hi = dj - a.win_hi, dj_lo = dj + a.win_lo;
            const float fdj = (float)dj;   // ALiBi distance of row r + e: |fdj - (r + e)|
            // rows past the sequence (Q = dO = 0, LSE = D = 0): zero P with
            // ALiBi, whose term a negative slope makes grow with the distance
            // (an infinite P would turn 0 * P into NaN for real keys)
            const int row_lim = si.len_q - i0 - 4 * h;
            auto softmax = [&](auto masked) {
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int r = 32 * mb + 8 * q4;   // + 4h + e
                        const f32x4 lse = stat[mb * 4 + q4];
                        constexpr bool XA = ALIBI || BIAS;   // an ALiBi term (slope 0 when absent)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int v = 4 * q4 + e;
                            float p;
                            if constexpr (decltype(masked)::value) {
                                const float l2 = lse[e] == -INFINITY ? 0.f : lse[e] * kLog2e;
                                float x = xc[mb][v] * scale2 - l2;
                                if constexpr (XA) x = fmaf(nsl2, fabsf(fdj - (float)(r + e)), x);
                                if constexpr (BIAS) x = fmaf(b16_elem<T>(bia[mb * 4 + q4], e), kLog2e, x);
                                p = __builtin_amdgcn_exp2f(x);
                                // i + off - lo <= j <= i + off + hi, i = i0 + r + 4h + e
                                bool vis = dj_hi <= r + e && dj_lo >= r + e;
                                if constexpr (XA) vis = vis && r + e < row_lim;
                                p = vis ? p : 0.f;
                            } else {
                                float x = fmaf(xc[mb][v], scale2, -lse[e] * kLog2e);
                                if constexpr (XA) x = fmaf(nsl2, fabsf(fdj - (float)(r + e)), x);
                                if constexpr (BIAS) x = fmaf(b16_elem<T>(bia[mb * 4 + q4], e), kLog2e, x);
                                p = __builtin_amdgcn_exp2f(x);
                            }
                            xc[mb][v] = p;
                        }
                    }
                }
            };
            if ((MASKED && (i0 < diag_hi || i0 > diag_lo)) || ((ALIBI || BIAS) && i0 + BM > si.len_q))
                softmax(std::true_type{});
            else
                softmax(std::false_type{});
            // dropout: bit 4 q + e of keep is element (rows r + e of 4 x 4 block
            // q = 4 mb + q4, this lane's key j): byte j % 4 of word e
            unsigned keep = 0xffffffffu;
            if constexpr (DROP) {
                // the four lanes of a group of four keys (lanes 4k .. 4k + 3,
                // key j % 4 = lane % 4, the same rows) need the same generator
                // blocks: lane c draws block 4 qq + c and the group trades the
                // decisions, lane c taking key c's nibble of each block
                keep = 0u;
                const int c = lane & 3;
                const unsigned sh = 4u * (unsigned)c;
#pragma unroll
                for (int qq = 0; qq < NMB; ++qq) {
                    const int q = 4 * qq + c;
                    const u32x4 dw = drop_block((unsigned)(j >> 2), (unsigned)((i0 + 8 * q + 4 * h) >> 2),
                                                (unsigned)(b * a.hq + hkv * G + g_t), a.drop.off, a.drop.k0,
                                                a.drop.k1);
                    const unsigned m = drop_mask16(dw, a.drop.thr);
                    keep |= ((quad_bcast<0>(m) >> sh) & 0xfu) << (16 * qq);
                    keep |= ((quad_bcast<1>(m) >> sh) & 0xfu) << (16 * qq + 4);
                    keep |= ((quad_bcast<2>(m) >> sh) & 0xfu) << (16 * qq + 8);
                    keep |= ((quad_bcast<3>(m) >> sh) & 0xfu) << (16 * qq + 12);
                }
            }
#pragma unroll
            for (int c = 0; c < C::NIC; ++c) {
                float tp[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) tp[u] = xc[c >> 1][8 * (c & 1) + u];
                if constexpr (DROP) {
                    // element u of slice c: block q = 2c + u / 4, row e = u % 4
                    float te[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const bool k = (keep >> (8 * c + u)) & 1u;
                        te[u] = k ? tp[u] : -tp[u];
                        tp[u] = k ? tp[u] : 0.f;
                    }
                    op_t enc;
                    to_op(enc, te);
                    to_op(opa[c], tp);
                    lds_write(smem, ps + c * 1024, __builtin_bit_cast(u32x4, enc));
                } else {
                    to_op(opa[c], tp);
                    // P goes to the partner in the operand type it already has
                    // for P^T dO (half the LDS bytes of fp32)
                    lds_write(smem, ps + c * 1024, __builtin_bit_cast(u32x4, opa[c]));
                }
            }
        } else {
            // ---- dS = P (dP - D) with P from the partner wave (the value
            // its dV product used, rounded to the operand type)
            float pf[C::NIC][8];
#pragma unroll
            for (int c = 0; c < C::NIC; ++c) from_op(__builtin_bit_cast(op_t, pin[c]), pf[c]);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 dl = stat[mb * 4 + q4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 4 * q4 + e;
                        const float pv = pf[2 * mb + (v >> 3)][v & 7];
                        if constexpr (DROP) {
                            // sign bit set: dropped (P = -0 included)
                            const bool kept = !__builtin_signbit(pv);
                            xp[mb][v] = fabsf(pv) * ((kept ? a.drop.rp * xp[mb][v] : 0.f) - dl[e]);
                        } else {
                            xp[mb][v] = pv * (xp[mb][v] - dl[e]);
                        }
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < C::NIC; ++c) {
                float td[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) td[u] = xp[c >> 1][8 * (c & 1) + u];
                to_op(opa[c], td);
            }
            if (STORE_DS && ragged_k) {
                // a key past the sequence meets zero K rows in dQ = dS K; its
                // stored dS is zero so that a non-finite value cannot reach them
                // (its dK row is not stored either)
                const bool kill = j >= si.len_k;
#pragma unroll
                for (int c = 0; c < C::NIC; ++c) {
                    u32x4 wv = __builtin_bit_cast(u32x4, opa[c]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) wv[q] = kill ? 0u : wv[q];
                    opa[c] = __builtin_bit_cast(op_t, wv);
                }
            }
        }
        // ---- dV += P^T dO (P wave) or dK += dS^T Q (dS wave)
        // the XOR touches address bits 6-7 only, zero in the ring offset
        const int t0 = col_off + tbase0, t1 = col_off + tbase1;
        // every transposing read is issued before the first MFMA.  With the
        // dS stores in the block, the compiler sinks the reads to their uses
        // (exposing the LDS latency once per MFMA) unless a scheduling
        // barrier separates them; without the stores the grouping hints below
        // give a better interleaving.
        u32x4 bop[C::NIC][C::NDB];
#pragma unroll
        for (int c = 0; c < C::NIC; ++c) {
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
                const u32x2 x = lds_read_tr(smem, (t0 ^ (64 * d)) + (int)buf + c * 16 * ROWB);
                const u32x2 y = lds_read_tr(smem, (t1 ^ (64 * d)) + (int)buf + c * 16 * ROWB);
                bop[c][d] = u32x4{x[0], x[1], y[0], y[1]};
            }
        }
#pragma unroll
        for (int c = 0; c < C::NIC; ++c) {
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) mma16(acc[d], opa[c], __builtin_bit_cast(op_t, bop[c][d]));
        }
        if constexpr (!STORE_DS) {
            // every read first
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NIC * C::NDB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, C::NIC * C::NDB, 0);
        } else {
            // one slice ahead (fewer registers held by the dS wave, which
            // also keeps its store offsets): the reads of slice c + 1 go
            // between the MFMAs of slice c
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::NDB, 0);
#pragma unroll
            for (int c = 1; c < C::NIC; ++c) {
#pragma unroll
                for (int d = 0; d < C::NDB; ++d) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x008, C::NDB, 0);
        }
        if (STORE_DS && R == 1) {
            // dS (16-bit) of this pair's 32 keys straight from the MFMA operand
            // registers to the dS block: chunk (pair, c, lane) holds, for key
            // 32 pair + lane % 32, the rows 16c + 4 (lane / 32) + 0..3 and
            // 16c + 8 + 4 (lane / 32) + 0..3 (the dQ pass reads it back with
            // transposing reads).  Issued after the dK MFMAs, which run meanwhile.
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const rsrc_t dst = make_rsrc(
                    ds_prev.head + (long long)(ds_prev.blk + mb * ds_prev.cnt) * kDsBlockBytes,
                    ds_prev.head ? kDsBlockBytes : 0);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    // non-temporal: read once, by the dQ pass
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, opa[2 * mb + c]), dst,
                                                           ds_chunk(2 * (pair + n % C::KPB * C::NP) + c, lane) * 16,
                                                           0, 2);
                }
            }
        }
        if (BIAS && R == 1) {
            // dBias = dS of tile t-1 (16-bit, the value dK's product used),
            // element (row 32 mb + 8 q4 + 4h + e, key j) of operand slice c =
            // 2 mb + q4 / 2, element 4 (q4 % 2) + e; an empty range without dBias
            const char* dbase = reinterpret_cast<const char*>(a.dbias) +
                                ((long long)b * a.sdbias.b + (long long)(hkv * G + dbg) * a.sdbias.h +
                                 (long long)dbm * BM * a.sdbias.r + (long long)n * KBN) * (long long)sizeof(T);
            const int rows = min(BM, si.len_q - dbm * BM);
            const unsigned bytes = a.dbias != nullptr ? (unsigned)((rows - 1) * sdbr_b) +
                                                            (unsigned)(max(si.len_k - n * KBN, 0) * (int)sizeof(T))
                                                      : 0u;
            const rsrc_t dst = make_rsrc(dbase, bytes);
            if (!DROP && db_wide) {
                // through this wave's LDS image: lane (l32, h) leaves its key's
                // rows 32 (c / 2) + 16 (c % 2) + 4h + 0..3 and + 8 .. 11, then
                // transposing reads give lane u of 16-lane group g keys
                // 8 kc .. + 7 of row 16 rb + u, (rb, kc) = (x / 4, x % 4) for
                // x = 4 p + g: one 16-byte store each
                const int img = C::OFF_DBIMG + pair * C::DBIMG;
#pragma unroll
                for (int c = 0; c < C::NIC; ++c) {
                    const u32x4 wv = __builtin_bit_cast(u32x4, opa[c]);
                    const int r0 = 32 * (c >> 1) + 16 * (c & 1) + 4 * h;
                    *reinterpret_cast<u32x2*>(smem + img + l32 * C::DBIMG_ROWB + 2 * r0) = u32x2{wv[0], wv[1]};
                    *reinterpret_cast<u32x2*>(smem + img + l32 * C::DBIMG_ROWB + 2 * (r0 + 8)) = u32x2{wv[2], wv[3]};
                }
                const int u16 = lane & 15, g = lane >> 4;
#pragma unroll
                for (int p = 0; p < C::NDBW; ++p) {
                    const int x = 4 * p + g, rb = x >> 2, kc = x & 3;
                    // source lane u16 points at key 8 kc + u16 / 4, rows 16 rb + 4 (u16 % 4) .. + 3
                    const int src = img + (8 * kc + (u16 >> 2)) * C::DBIMG_ROWB + 2 * (16 * rb + 4 * (u16 & 3));
                    const u32x2 k0 = lds_read_tr(smem, src);
                    const u32x2 k4 = lds_read_tr(smem, src + 4 * C::DBIMG_ROWB);
                    const int row = 16 * rb + u16;
                    const int voff = row < rows ? (int)(row * sdbr_b) + (32 * pair + 8 * kc) * (int)sizeof(T) : kOobOff;
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{k0[0], k0[1], k4[0], k4[1]}, dst, voff, 0, 2);
                }
            } else {
#pragma unroll
                for (int c = 0; c < C::NIC; ++c) {
                    const u32x4 wv = __builtin_bit_cast(u32x4, opa[c]);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int r = 32 * (c >> 1) + 8 * (2 * (c & 1) + (u >> 2)) + (u & 3);   // + 4h
                        const unsigned short x =
                            (unsigned short)((u & 1) ? (wv[u >> 1] >> 16) : (wv[u >> 1] & 0xffffu));
                        __builtin_amdgcn_raw_buffer_store_b16(x, dst, db_voff, (int)(r * sdbr_b), 2);
                    }
                }
            }
        }
        if constexpr (DS_LATE) {
            __builtin_amdgcn_sched_barrier(0);
            first_product();
        }
        advance_ds();
    };

    // the dS wave keeps X of tile t until step t+1: two register sets, unrolled
    // by two.  Each role runs its own copy of the loop (the same number of
    // steps and barriers), compiled for that role alone.
    f32x16 xA[NMB], xB[NMB];
    // The dS wave's first step (no tile t-1 yet) is peeled off its loop.
    // The loops are unrolled by the ring length, so each step's buffers are
    // constants (NBUF is even, which also fixes the tile parity per step).
    static_assert(C::NBUF == 4, "the unrolled loops below assume a ring of four");
    const std::false_type later;
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    if (role == 0) {
        const std::integral_constant<int, 0> r0;
        for (int t = 0; t <= n_tiles; t += 4) {
            step(r0, later, K0{}, t, xA, xB);
            if (t + 1 > n_tiles) break;
            step(r0, later, K1{}, t + 1, xB, xA);
            if (t + 2 > n_tiles) break;
            step(r0, later, K2{}, t + 2, xA, xB);
            if (t + 3 > n_tiles) break;
            step(r0, later, K3{}, t + 3, xB, xA);
        }
    } else {
        const std::integral_constant<int, 1> r1;
        step(r1, std::true_type{}, K0{}, 0, xA, xB);
        for (int t = 1; t <= n_tiles; t += 4) {
            step(r1, later, K1{}, t, xB, xA);
            if (t + 1 > n_tiles) break;
            step(r1, later, K2{}, t + 1, xA, xB);
            if (t + 2 > n_tiles) break;
            step(r1, later, K3{}, t + 2, xB, xA);
            if (t + 3 > n_tiles) break;
            step(r1, later, K0{}, t + 3, xA, xB);
        }
    }

    // ---- epilogue: dV (P wave) or dK = s * sum dS^T Q (dS wave); rows past
    // the sequence are not written
    T* dst = reinterpret_cast<T*>(role == 0 ? a.dv : a.dk) + out_base;
    const float f = role == 0 ? (DROP ? a.drop.rp : 1.f) : a.scale;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int jj = n * KBN + 32 * pair + acc_row(v, h);
            if (jj < si.len_k && 32 * d + l32 < a.d) store_elem(dst, (long long)jj * s_out.r + 32 * d + l32, acc[d][v] * f);
        }
    }
}


template <class T, int HD, bool MASKED, bool STORE_DS, bool ALIBI, bool BIAS, bool DROP>
__global__ __launch_bounds__(KvCfg<HD>::NW * 64, 1) void bwd_kv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[BIAS ? KvCfg<HD>::LDS_BYTES_BIAS : KvCfg<HD>::LDS_BYTES];
    constexpr int KBN = KvCfg<HD>::KBN;
    // key tiles per sequence: with the stored dS every tile of a dS block
    // that starts inside the keys (see kv_tile)
    constexpr int KROUND = STORE_DS ? KvCfg<HD>::KPB : 1;
    // ---- key tiles: all those of one (sequence, kv-head) on one XCD.  Under
    // a causal mask key tile n is seen by a number of query tiles that falls
    // linearly with n, so on grids larger than the GPU (pair_tiles)
    // workgroup p takes the tiles p and (last - p), which together always
    // cost about the same (under a window alone the pairs cost about the
    // same anyway); on smaller ones each workgroup takes one tile.
    const bool pair = MASKED && a.pair_tiles;
    const int per_group = pair ? (a.nblk_n + 1) / 2 : a.nblk_n;
    int grp, p;
    {
        const int groups = a.hkv_n * a.batch;
        if (groups % kXcds == 0) {
            const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
            grp = (slot / per_group) * kXcds + xcd;
            p = slot % per_group;
        } else {
            grp = blockIdx.x / per_group;
            p = blockIdx.x % per_group;
        }
    }
    const int hkv = a.hkv0 + grp % a.hkv_n;
    const int b = grp / a.hkv_n;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    if (MASKED) {
        const int nk = (si.len_k + KROUND * KBN - 1) / (KROUND * KBN) * KROUND;   // this sequence's key tiles
        const int n2 = pair ? nk - 1 - p : p;
        // one call site in a loop: a single copy of the (large) tile body
        const int cnt = pair ? (p <= n2) + (n2 > p) : (p < nk ? 1 : 0);
        for (int k = 0; k < cnt; ++k) {
            if (k) __syncthreads();   // the first tile's LDS ring and P slots are free again
            kv_tile<T, HD, MASKED, STORE_DS, ALIBI, BIAS, DROP>(a, b, hkv, k == 0 && p <= n2 ? p : n2, si, smem);
        }
    } else {
        kv_tile<T, HD, MASKED, STORE_DS, ALIBI, BIAS, DROP>(a, b, hkv, p, si, smem);
    }
}

// the dK/dV kernel's instantiation for (mask, stored dS, ALiBi, bias,
// dropout): the bias variant also applies ALiBi slopes when given, the
// dropout variant a bias and ALiBi slopes when given
template <class T, int HD, bool M, bool S, bool A, bool B, bool D>
static void launch_kv3(const BwdArgs& a, unsigned grid, hipStream_t st) {
    bwd_kv_kernel<T, HD, M, S, A, B, D><<<grid, KvCfg<HD>::NW * 64, 0, st>>>(a);
}
template <class T, int HD, bool M, bool S>
static void launch_kv2(const BwdArgs& a, bool alibi, unsigned grid, hipStream_t st) {
    if (a.drop.on) launch_kv3<T, HD, M, S, false, true, true>(a, grid, st);
    else if (a.bias != nullptr || a.dbias != nullptr) launch_kv3<T, HD, M, S, false, true, false>(a, grid, st);
    else if (alibi) launch_kv3<T, HD, M, S, true, false, false>(a, grid, st);
    else launch_kv3<T, HD, M, S, false, false, false>(a, grid, st);
}
template <class T, int HD, bool M>
static void launch_kv1(const BwdArgs& a, bool store_ds, bool alibi, unsigned grid, hipStream_t st) {
    if (store_ds) launch_kv2<T, HD, M, true>(a, alibi, grid, st);
    else launch_kv2<T, HD, M, false>(a, alibi, grid, st);
}
template <class T, int HD>
static void launch_kv(const BwdArgs& a, bool masked, bool store_ds, bool alibi, unsigned grid, hipStream_t st) {
    if (masked) launch_kv1<T, HD, true>(a, store_ds, alibi, grid, st);
    else launch_kv1<T, HD, false>(a, store_ds, alibi, grid, st);
}


}  // namespace attn
