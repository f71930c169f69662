// Plain forward (input generator), backward preprocess (D = rowsum(dO * O),
// workspace clear) and dQ postprocess (fp32 accumulator -> I/O type).
//
// The preprocess and postprocess are HBM-streaming kernels: every thread
// moves 16-byte vectors, rows are read contiguously, and the only arithmetic
// is a fused multiply-add chain (preprocess) or a scale + convert
// (postprocess).
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace attn {

// Index of (sequence row r, head h) in the [B, H, S] / [H, total] layouts of
// LSE, D and the dQ accumulator.  r is the flattened row of Q (b * Sq + i for
// dense, the packed row for varlen).
__device__ __forceinline__ long long lse_index(bool varlen, long long r, int h, int H, int S, long long total) {
    if (varlen) return (long long)h * total + r;
    long long b = r / S, i = r - b * S;
    return (b * H + h) * S + i;
}

// ---------------------------------------------------------------------------
// forward: one thread per query row (two above head dim 128, each holding
// half the row's columns and adding the other's dot-product half by a
// shuffle), K/V tiles of 32 keys staged in LDS, online softmax in base 2.
// Not performance-tracked.
// ---------------------------------------------------------------------------
template <int HD>
constexpr int fwd_threads_per_row() { return HD > 128 ? 2 : 1; }

template <class T, int HD, bool MASKED>
__global__ __launch_bounds__(128 * fwd_threads_per_row<HD>()) void fwd_kernel(FwdArgs a) {
    constexpr int BQ = 128, BK = 32;
    constexpr int TPR = fwd_threads_per_row<HD>(), HDT = HD / TPR;   // threads per row, columns per thread
    __shared__ float ks[BK][HD];
    __shared__ float vs[BK][HD];
    const int qb = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    if (qb * BQ >= si.len_q) return;
    const int hkv = hq / (a.hq / a.hkv);
    const int part = (int)threadIdx.x % TPR, c0 = part * HDT;   // this thread's columns c0 .. c0 + HDT - 1
    const int i = qb * BQ + (int)threadIdx.x / TPR;
    const bool row_ok = i < si.len_q;
    const int off = si.len_k - si.len_q;
    const bool varlen = a.cu_q != nullptr;
    const T* qp = reinterpret_cast<const T*>(a.q);
    const T* kp = reinterpret_cast<const T*>(a.k);
    const T* vp = reinterpret_cast<const T*>(a.v);
    const long long qrow = seq_off(a.sq, varlen, b, si.q0) + (long long)hq * a.sq.h + (long long)i * a.sq.r;
    const long long kbase = seq_off(a.sk, varlen, b, si.k0) + (long long)hkv * a.sk.h;
    const long long vbase = seq_off(a.sv, varlen, b, si.k0) + (long long)hkv * a.sv.h;

    // columns from a.d on are zero (the head dim padded to HD)
    float q[HDT], o[HDT];
    const float qs = a.scale * kLog2e;
#pragma unroll
    for (int d = 0; d < HDT; ++d) {
        q[d] = row_ok && c0 + d < a.d ? (float)load_elem(qp, qrow + c0 + d) * qs : 0.f;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    // ALiBi slope in the log2 units of the scaled logits (0: no bias)
    const float sl2 = a.alibi != nullptr ? a.alibi[hq] * kLog2e : 0.f;
    // this row of the elementwise bias (log2 units at use), or null
    const T* brow = a.bias != nullptr && row_ok
                        ? reinterpret_cast<const T*>(a.bias) + (long long)b * a.sbias.b + (long long)hq * a.sbias.h +
                              (long long)i * a.sbias.r
                        : nullptr;
    // keys any row of the block can see: with a mask, from the first row's
    // lower bound (aligned down to a tile) to the last row's upper bound
    const int whi = a.win_hi, wlo = a.win_lo;
    int kbeg = 0, kend = si.len_k;
    if (MASKED) {
        kend = min(kend, min(qb * BQ + BQ, si.len_q) - 1 + off + a.win_hi + 1);
        const int first = qb * BQ + off - a.win_lo;
        kbeg = first > 0 ? first / BK * BK : 0;
    }
    for (int kt = kbeg; kt < kend; kt += BK) {
        __syncthreads();
        for (int e = threadIdx.x; e < BK * HD; e += blockDim.x) {
            const int jj = e / HD, d = e % HD, j = kt + jj;
            const bool ok = j < si.len_k && d < a.d;
            ks[jj][d] = ok ? (float)load_elem(kp, kbase + (long long)j * a.sk.r + d) : 0.f;
            vs[jj][d] = ok ? (float)load_elem(vp, vbase + (long long)j * a.sv.r + d) : 0.f;
        }
        __syncthreads();
        float s[BK];
        float tmax = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < BK; ++jj) {
            const int j = kt + jj;
            const int dj = j - i - off;   // i + off - lo <= j <= i + off + hi
            const bool vis = row_ok && j < si.len_k && (!MASKED || (dj <= whi && dj >= -wlo));
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < HDT; ++d) acc = fmaf(q[d], ks[jj][c0 + d], acc);
            if constexpr (TPR == 2) acc += __shfl_xor(acc, 1);   // the row's other half
            float x = acc - sl2 * fabsf((float)dj);
            if (brow != nullptr && vis) x = fmaf((float)load_elem(brow, j), kLog2e, x);
            s[jj] = vis ? x : -INFINITY;
            tmax = fmaxf(tmax, s[jj]);
        }
        if (tmax > -INFINITY) {
            const float mn = fmaxf(m, tmax);
            const float corr = exp2f(m - mn);
            l *= corr;
#pragma unroll
            for (int d = 0; d < HDT; ++d) o[d] *= corr;
            // dropout: this row's random word of each 4 x 4 block of the tile
            unsigned dw[BK / 4];
            if (a.drop.on) {
#pragma unroll
                for (int t = 0; t < BK / 4; ++t)
                    dw[t] = word_at(drop_block((unsigned)(kt / 4 + t), (unsigned)(i >> 2), (unsigned)(b * a.hq + hq),
                                               a.drop.off, a.drop.k0, a.drop.k1),
                                    i & 3);
            }
#pragma unroll
            for (int jj = 0; jj < BK; ++jj) {
                float p = exp2f(s[jj] - mn);
                l += p;   // the sum (and LSE) over every visible key
                if (a.drop.on && !drop_keep(dw[jj >> 2], jj & 3, a.drop.thr)) p = 0.f;
#pragma unroll
                for (int d = 0; d < HDT; ++d) o[d] = fmaf(p, vs[jj][c0 + d], o[d]);
            }
            m = mn;
        }
    }
    if (!row_ok) return;
    const float inv = l > 0.f ? (a.drop.on ? a.drop.rp : 1.f) / l : 0.f;
    T* op = reinterpret_cast<T*>(a.o);
    const long long ob = seq_off(a.so, varlen, b, si.q0) + (long long)hq * a.so.h + (long long)i * a.so.r;
#pragma unroll
    for (int d = 0; d < HDT; ++d) {
        if (c0 + d < a.d) store_elem(op, ob + c0 + d, o[d] * inv);
    }
    const long long li = varlen ? (long long)hq * a.total_q + si.q0 + i
                                : ((long long)b * a.hq + hq) * a.seqlen_q + i;
    if (part == 0) a.lse[li] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// preprocess: D = rowsum(dO * O).  One workgroup takes one head and 64
// consecutive token rows: HD / 8 lanes per row read 16 bytes each of O and dO
// (a contiguous head row), reduce by shuffles, and the 64 sums leave through
// LDS as one contiguous 256-byte run of D, so no D line is shared between
// workgroups (they would sit in different L2s and be written back partially).
// ---------------------------------------------------------------------------
// The stored-dS block table, built by one extra workgroup of the preprocess: first the exclusive prefix sum
// of each sequence's query tiles (tile_base, batch + 1 entries), then that of
// the dS blocks of every query tile over all sequences (prefix, one entry
// per tile): the tile's first block within a q-head's region.  A tile whose
// blocks would end past ds_head_blocks (only with malformed cu_seqlens,
// whose clamped lengths can add up to more rows than total_q) gets -1: no dS
// is stored or read for it.  Lengths are clamped as the kernels clamp them.
__device__ __forceinline__ void ds_table_body(const BwdArgs& a, int bm, bool masked) {
    __shared__ long long part[256];
    int* tile_base = const_cast<int*>(a.ds_tile_base);
    int* prefix = const_cast<int*>(a.ds_prefix);
    auto scan = [&](long long v) {   // inclusive scan of v over the workgroup
        part[threadIdx.x] = v;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const long long x = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
            __syncthreads();
            part[threadIdx.x] += x;
            __syncthreads();
        }
        const long long r = part[threadIdx.x];
        const long long total = part[255];
        __syncthreads();
        return make_longlong2(r, total);
    };
    long long carry = 0;
    for (int c0 = 0; c0 < a.batch; c0 += 256) {
        const int b = c0 + (int)threadIdx.x;
        long long v = 0;
        if (b < a.batch) {
            const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q,
                                        a.used_k);
            v = (si.len_q + bm - 1) / bm;
        }
        const longlong2 r = scan(v);
        if (b < a.batch) tile_base[b] = (int)min(carry + r.x - v, (long long)a.ds_ntiles);
        carry += r.y;
    }
    if (threadIdx.x == 0) tile_base[a.batch] = (int)min(carry, (long long)a.ds_ntiles);
    __syncthreads();
    const int ntiles = (int)min(carry, (long long)a.ds_ntiles);
    long long blocks = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 256) {
        const int t = t0 + (int)threadIdx.x;
        long long v = 0;
        if (t < ntiles) {
            // the sequence of tile t: the last b with tile_base[b] <= t
            int lo = 0, hi = a.batch - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tile_base[mid] <= t) lo = mid;
                else hi = mid - 1;
            }
            const SeqInfo si = seq_info(lo, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q,
                                        a.used_k);
            v = ds_tile_blocks(t - tile_base[lo], bm, si.len_q, si.len_k, a.win_lo, a.win_hi, masked);
        }
        const longlong2 r = scan(v);
        if (t < ntiles) {
            const long long first = blocks + r.x - v;
            prefix[t] = first + v <= a.ds_head_blocks ? (int)first : -1;
        }
        blocks += r.y;
    }
}

// Tokens per preprocess workgroup: two passes of its 256 lanes over rows of
// HD / 8 lanes each (measured on the B=4 H=16 S=4096 bf16 shapes: 6.3 TB/s
// at head dim 128 against 5.9 with four passes and 5.5 with one)
template <int HD>
constexpr int pre_tokens() { return 2 * 256 / (HD / 8); }

// TABLE: the grid's first workgroup builds the stored-dS block table instead
// (it runs beside the D workgroups, so the table costs no launch of its own;
// first, so that it does not run on alone at the end)
template <class T, int HD, bool TABLE>
__global__ __launch_bounds__(256) void preprocess_kernel(PreArgs a, BwdArgs t, int bm, bool masked) {
    constexpr int LPR = HD / 8;
    constexpr int RPP = 256 / LPR;                 // rows per pass
    constexpr int kPreTokens = pre_tokens<HD>();
    constexpr int PASSES = kPreTokens / RPP;
    static_assert(PASSES * RPP == kPreTokens && kPreTokens <= 256, "whole passes, one D word per lane");
    __shared__ float dsum[kPreTokens];
    {
        // the workspace words attn_bwd accumulates into (grid-stride)
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < a.n16;
             i += (long long)gridDim.x * blockDim.x)
            a.zero[i] = z;
    }
    if (TABLE && blockIdx.x == 0) {
        ds_table_body(t, bm, masked);
        return;
    }
    const unsigned bid = blockIdx.x - (TABLE ? 1u : 0u);
    const long long tokens = a.rows / a.h;
    const int h = (int)(bid % (unsigned)a.h);
    const long long r0 = (long long)(bid / (unsigned)a.h) * kPreTokens;
    const int part = threadIdx.x % LPR, slot = threadIdx.x / LPR;
    const bool live = part * 8 < a.d;   // this lane's 8 columns lie within the head dim
    float x[PASSES][8], y[PASSES][8];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const long long r = min(r0 + p * RPP + slot, tokens - 1);
        if (live) {
            // O and dO are read once here: non-temporal loads
            load8_nt(reinterpret_cast<const T*>(a.o) + flat_row_off(a.so, a.varlen, r, a.s) + (long long)h * a.so.h +
                         part * 8, x[p]);
            load8_nt(reinterpret_cast<const T*>(a.dout) + flat_row_off(a.sdo, a.varlen, r, a.s) +
                         (long long)h * a.sdo.h + part * 8, y[p]);
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) x[p][t] = y[p][t] = 0.f;
        }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = fmaf(x[p][t], y[p][t], acc);
#pragma unroll
        for (int w = LPR / 2; w > 0; w >>= 1) acc += __shfl_xor(acc, w, LPR);
        if (part == 0) dsum[p * RPP + slot] = acc;
    }
    __syncthreads();
    const long long r = r0 + threadIdx.x;
    if (threadIdx.x < kPreTokens && r < tokens)
        a.delta[lse_index(a.varlen, r, h, a.h, a.s, a.total)] = dsum[threadIdx.x];
}

// Zero the masked elements of a [b, h, i, j] tensor (dBias): in row i of
// (sequence b, q-head h), the keys j < len_k outside i + off - lo <= j <=
// i + off + hi.  The backward kernels write every visible element of the
// rows i < len_q, so nothing else needs clearing.  kZeroRows rows per
// workgroup, 64 lanes each; 16-byte stores where the row is 16-byte aligned.
constexpr int kZeroRows = 4;
template <class T>
__global__ __launch_bounds__(256) void zero_masked_kernel(T* p, Strides s, BwdArgs a) {
    const int i = blockIdx.x * kZeroRows + (int)(threadIdx.x >> 6), h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x & 63;
    const SeqInfo si = seq_info(b, a.seqlen_q, a.seqlen_k, a.total_q, a.total_k, a.cu_q, a.cu_k, a.used_q, a.used_k);
    if (i >= si.len_q) return;
    T* row = p + (long long)b * s.b + (long long)h * s.h + (long long)i * s.r;
    const int off = si.len_k - si.len_q;
    const int lo = min(max(i + off - a.win_lo, 0), si.len_k);        // keys [0, lo) lie before the window
    const int hi = min(max(i + off + a.win_hi + 1, 0), si.len_k);    // keys [hi, len_k) lie after it
    constexpr int E = 16 / (int)sizeof(T);
    const bool al = (reinterpret_cast<unsigned long long>(row) & 15) == 0;
    auto zero_range = [&](int x0, int x1) {   // keys [x0, x1)
        if (x0 >= x1) return;
        const int a0 = al ? min((x0 + E - 1) / E * E, x1) : x1;   // first key of the 16-byte part
        const int a1 = al ? max(x1 / E * E, a0) : x1;             // its end
        for (int j = x0 + t; j < a0; j += 64) store_elem(row, j, 0.f);
        for (int j = a1 + t; j < x1; j += 64) store_elem(row, j, 0.f);
        for (int c = a0 / E + t; c < a1 / E; c += 64) reinterpret_cast<u32x4*>(row)[c] = u32x4{0u, 0u, 0u, 0u};
    };
    zero_range(0, lo);
    zero_range(max(hi, lo), si.len_k);
}

// ---------------------------------------------------------------------------
// postprocess: dQ[row, h, :] = T(scale * acc[h, row, :])
// ---------------------------------------------------------------------------
template <class T, int HD>
__global__ __launch_bounds__(256) void postprocess_kernel(PostArgs a) {
    constexpr int LPR = HD / 8;
    const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gt / LPR;
    if (row >= a.rows) return;
    const int part = (int)(gt % LPR);
    const long long r = row / a.h;
    const int h = (int)(row - r * a.h);
    if (a.used_q != nullptr) {
        // the sequence holding token r (the last b with cu[b] <= r); tokens
        // past its used length, or past every sequence, keep their dQ
        int lo = 0, hi = a.batch;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_q[mid] <= r) lo = mid;
            else hi = mid - 1;
        }
        if (lo >= a.batch) return;
        const int len = min(a.cu_q[lo + 1] - a.cu_q[lo], max(a.used_q[lo], 0));
        if (r >= (long long)a.cu_q[lo] + len) return;
    }
    if (part * 8 >= a.d) return;   // padding columns of the accumulator
    const float* src = a.acc + lse_index(a.varlen, r, h, a.h, a.s, a.total) * HD + part * 8;
    const f32x4 u = *reinterpret_cast<const f32x4*>(src);
    const f32x4 w = *reinterpret_cast<const f32x4*>(src + 4);
    float x[8] = {u[0], u[1], u[2], u[3], w[0], w[1], w[2], w[3]};
    // the product is rounded to fp32 before the conversion to T
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = mul_f32(x[t], a.scale);
    store8(reinterpret_cast<T*>(a.dq) + flat_row_off(a.sdq, a.varlen, r, a.s) + (long long)h * a.sdq.h + part * 8, x);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class T, int HD>
static void launch_fwd_t(const FwdArgs& a, bool masked, hipStream_t st) {
    dim3 grid((a.seqlen_q + 127) / 128, a.hq, a.batch);
    constexpr int threads = 128 * fwd_threads_per_row<HD>();
    if (masked)
        fwd_kernel<T, HD, true><<<grid, threads, 0, st>>>(a);
    else
        fwd_kernel<T, HD, false><<<grid, threads, 0, st>>>(a);
}

void launch_fwd(const FwdArgs& a, int dtype, int hd, bool masked, hipStream_t st) {
    if (dtype == ATTN_DTYPE_BF16) {
        if (hd == 64) launch_fwd_t<bf16_t, 64>(a, masked, st);
        else if (hd == 128) launch_fwd_t<bf16_t, 128>(a, masked, st);
        else launch_fwd_t<bf16_t, 256>(a, masked, st);
    } else if (dtype == ATTN_DTYPE_F16) {
        if (hd == 64) launch_fwd_t<f16_t, 64>(a, masked, st);
        else if (hd == 128) launch_fwd_t<f16_t, 128>(a, masked, st);
        else launch_fwd_t<f16_t, 256>(a, masked, st);
    } else {   // fp32: head dims up to 128
        if (hd == 64) launch_fwd_t<float, 64>(a, masked, st);
        else launch_fwd_t<float, 128>(a, masked, st);
    }
}

void launch_zero_masked(void* p, const Strides& s, int dtype, const BwdArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.seqlen_q + kZeroRows - 1) / kZeroRows), (unsigned)a.hq, (unsigned)a.batch);
    if (dtype == ATTN_DTYPE_BF16) zero_masked_kernel<bf16_t><<<grid, 256, 0, st>>>(reinterpret_cast<bf16_t*>(p), s, a);
    else if (dtype == ATTN_DTYPE_F16) zero_masked_kernel<f16_t><<<grid, 256, 0, st>>>(reinterpret_cast<f16_t*>(p), s, a);
    else zero_masked_kernel<float><<<grid, 256, 0, st>>>(reinterpret_cast<float*>(p), s, a);
}

void launch_preprocess(const PreArgs& a, int dtype, int hd, const BwdArgs* table, int bm, bool masked,
                       hipStream_t st) {
    const long long tokens = a.rows / a.h;
    const BwdArgs t = table ? *table : BwdArgs{};
    auto go = [&](auto tc, auto hc, auto table_c) {
        using T = decltype(tc);
        constexpr int HD = decltype(hc)::value;
        constexpr int kPreTokens = pre_tokens<HD>();
        const unsigned blocks = (unsigned)((tokens + kPreTokens - 1) / kPreTokens * a.h) + (table ? 1u : 0u);
        preprocess_kernel<T, HD, decltype(table_c)::value><<<blocks, 256, 0, st>>>(a, t, bm, masked);
    };
    auto by_hd = [&](auto tc, auto table_c) {
        if (hd == 64) go(tc, std::integral_constant<int, 64>{}, table_c);
        else if (hd == 128 || sizeof(decltype(tc)) == 4) go(tc, std::integral_constant<int, 128>{}, table_c);
        else go(tc, std::integral_constant<int, 256>{}, table_c);
    };
    auto by_table = [&](auto tc) {
        if (table) by_hd(tc, std::true_type{});
        else by_hd(tc, std::false_type{});
    };
    if (dtype == ATTN_DTYPE_BF16) by_table(bf16_t{});
    else if (dtype == ATTN_DTYPE_F16) by_table(f16_t{});
    else by_hd(float{}, std::false_type{});   // no stored dS in fp32
}

void launch_postprocess(const PostArgs& a, int dtype, int hd, hipStream_t st) {
    const long long threads = a.rows * (hd / 8);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (dtype == ATTN_DTYPE_BF16) {
        if (hd == 64) postprocess_kernel<bf16_t, 64><<<blocks, 256, 0, st>>>(a);
        else if (hd == 128) postprocess_kernel<bf16_t, 128><<<blocks, 256, 0, st>>>(a);
        else postprocess_kernel<bf16_t, 256><<<blocks, 256, 0, st>>>(a);
    } else if (dtype == ATTN_DTYPE_F16) {
        if (hd == 64) postprocess_kernel<f16_t, 64><<<blocks, 256, 0, st>>>(a);
        else if (hd == 128) postprocess_kernel<f16_t, 128><<<blocks, 256, 0, st>>>(a);
        else postprocess_kernel<f16_t, 256><<<blocks, 256, 0, st>>>(a);
    } else {
        if (hd == 64) postprocess_kernel<float, 64><<<blocks, 256, 0, st>>>(a);
        else postprocess_kernel<float, 128><<<blocks, 256, 0, st>>>(a);
    }
}

}  // namespace attn
