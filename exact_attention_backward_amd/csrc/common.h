// Shared device-side helpers of the gfx950 attention kernels: vector types,
// MFMA wrappers, bf16/fp16 packing, the XOR-swizzled LDS tile addressing and the
// transposing LDS read.  Written for CDNA4 (wave64, 160 KiB LDS per CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_bwd.h"

namespace attn {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// A bf16 value stored as its 16-bit pattern.  All bf16 vectors are moved as
// integer words; the compiler's element access on __bf16 vectors is avoided,
// and so is __builtin_bit_cast of a subscripted vector element (v[i]), which
// this compiler lowers as a read of element 0: vectors are bit cast whole, or
// the element is first copied into a scalar.
typedef uint16_t bf16_t;
// IEEE binary16, stored and converted natively (v_cvt_f16_f32 rounds to nearest even).
typedef _Float16 f16_t;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// element type traits: bf16 and fp16 (MFMA 32x32x16 of that type) and fp32
// (MFMA 32x32x2 f32)
// ---------------------------------------------------------------------------
template <class T> struct Elem;

template <> struct Elem<bf16_t> {
    // 8 consecutive-k operand values of one lane: 16 bytes
    typedef bf16x8 op_t;
    static constexpr int kBytes = 2;
    static constexpr attn_dtype_t kDtype = ATTN_DTYPE_BF16;
};
template <> struct Elem<f16_t> {
    typedef f16x8 op_t;
    static constexpr int kBytes = 2;
    static constexpr attn_dtype_t kDtype = ATTN_DTYPE_F16;
};
template <> struct Elem<float> {
    typedef f32x8 op_t;
    static constexpr int kBytes = 4;
    static constexpr attn_dtype_t kDtype = ATTN_DTYPE_F32;
};

// c += a * b over one 16-long slice of the contraction index.
// Lane l holds a[i = l % 32][k = 8 * (l / 32) + t] and b[k = 8 * (l / 32) + t][j = l % 32]
// for t = 0..7; c is the 32x32 fp32 accumulator in the MFMA output layout
// (lane l, value v -> row 8 * (v / 4) + 4 * (l / 32) + v % 4, column l % 32).
__device__ __forceinline__ void mma16(f32x16& c, const bf16x8& a, const bf16x8& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& c, const f16x8& a, const f16x8& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& c, const f32x8& a, const f32x8& b) {
    // step t pairs k = t (lanes 0-31) with k = 8 + t (lanes 32-63)
#pragma unroll
    for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], c, 0, 0, 0);
}

// Row of the MFMA 32x32 output held by value v of lane half h (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// ---------------------------------------------------------------------------
// bf16 conversion (round to nearest even, the hardware v_cvt_pk_bf16_f32)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two fp32 values -> one word of two 16-bit values of type T (low = first).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
template <class T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) { return pack_bf16x2(lo, hi); }
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) { return pack_f16x2(lo, hi); }

// Eight fp32 values -> MFMA operand of type T.
__device__ __forceinline__ void to_op(bf16x8& o, const float* x) {
    u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
               pack_bf16x2(x[6], x[7])};
    o = __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ void to_op(f16x8& o, const float* x) {
    u32x4 w = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]),
               pack_f16x2(x[6], x[7])};
    o = __builtin_bit_cast(f16x8, w);
}
__device__ __forceinline__ void to_op(f32x8& o, const float* x) {
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = x[t];
}

// Element e (0..3) of four 16-bit values of type T packed two per word, low
// half first, in fp32 (exact).
template <class T> __device__ __forceinline__ float b16_elem(u32x2 w, int e);
template <> __device__ __forceinline__ float b16_elem<bf16_t>(u32x2 w, int e) {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
}
template <> __device__ __forceinline__ float b16_elem<f16_t>(u32x2 w, int e) {
    const unsigned short u = (unsigned short)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
    return (float)__builtin_bit_cast(f16_t, u);
}

// MFMA operand of a 16-bit type -> its eight values in fp32 (exact).
__device__ __forceinline__ void from_op(const bf16x8& o, float* x) {
    const u32x4 w = __builtin_bit_cast(u32x4, o);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        x[2 * t] = bf16_lo(w[t]);
        x[2 * t + 1] = bf16_hi(w[t]);
    }
}
__device__ __forceinline__ void from_op(const f16x8& o, float* x) {
    const f32x8 f = __builtin_convertvector(o, f32x8);
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = f[t];
}

// ---------------------------------------------------------------------------
// LDS tiles: row-major, 16-byte chunks XOR-swizzled by a function of the row.
// LDS serves 256 bytes per cycle from 64 four-byte banks, so a 16-byte chunk
// slot is (row * ROW_BYTES / 16 + chunk) mod 16.  The swizzle keeps both
// access patterns of the kernels conflict-free:
//  - 16-byte reads of one logical chunk by 16 consecutive rows;
//  - transposing reads of 4 consecutive rows (starting at a multiple of 4)
//    by 4 consecutive chunks (a 64-byte column group).
// A plain XOR with the low row bits only permutes chunks inside a 64-byte
// group and leaves the second pattern 4-way conflicted.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__device__ __forceinline__ int swz_key(int row) {
    constexpr int kChunks = ROW_BYTES / 16;
    if constexpr (kChunks >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (kChunks == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else return (row >> 2) & (kChunks - 1);
}
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row, int byte) {
    return row * ROW_BYTES + (((byte >> 4) ^ swz_key<ROW_BYTES>(row)) << 4) + (byte & 15);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// source lane s supplies the address of 4 consecutive 16-bit elements; output
// lane u receives element (u % 4) of source lanes 4e + u / 4, e = 0..3.  Used
// on a row-major tile, where lane s points at row r0 + s / 4, columns
// c0 + 4 (s % 4) .. +3, output lane u gets the column c0 + u of rows r0..r0+3.
__device__ __forceinline__ u32x2 lds_read_tr(const char* lds_base, int byte_off) {
    bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_base + byte_off));
    return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read16(const char* lds_base, int byte_off) {
    return *reinterpret_cast<const u32x4*>(lds_base + byte_off);
}

template <class V>
__device__ __forceinline__ void lds_write(char* lds_base, int byte_off, const V& v) {
    *reinterpret_cast<V*>(lds_base + byte_off) = v;
}

// ---------------------------------------------------------------------------
// buffer resources: base address, byte range and the gfx9 raw-buffer format
// word.  Loads past the range return zeros and stores/atomics past it are
// dropped.  The check is on the sum of the per-lane, instruction and scalar
// offsets (measured: a scalar offset past the range reads zeros), so a range
// that should end at a tile's last valid byte includes the scalar offset.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A per-lane buffer offset past every range the kernels build (the ranges,
// scalar offsets included, stay below it): the lane's load returns zeros.
// It fills the tile columns past the head dim.
constexpr int kOobOff = 0x7FFFFFF0;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void buffer_to_lds16(rsrc_t r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
// 4 bytes per lane from buffer offset voff into LDS at lds + 4 * lane.
__device__ __forceinline__ void buffer_to_lds4(rsrc_t r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_atomic_add(float v, rsrc_t r, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, voff, 0, 0);
}

// The same copies issued from inline assembly, for the main loop's prefetch.
// The compiler's wait-count pass cannot tell which LDS bytes an LDS-DMA copy
// writes, so after a tracked copy it waits for it before the next LDS read,
// even one of a different buffer; that serialises the prefetch with the
// compute it should overlap.  These copies are invisible to that pass: the
// caller waits for them explicitly (vmcnt) before the barrier that publishes
// the buffer.  Extra untracked VMEM operations only make the compiler's own
// in-order vmcnt waits more conservative.  The descriptor words are
// {base[31:0], base[47:32] (stride 0), byte range, raw-buffer format}.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base, unsigned bytes) {
    const unsigned long long b = reinterpret_cast<unsigned long long>(base);
    i32x4 r = {__builtin_amdgcn_readfirstlane((int)(unsigned)b),
               __builtin_amdgcn_readfirstlane((int)((unsigned)(b >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
    return r;
}
// Move a descriptor's base address by `bytes` (the 48-bit address of words
// 0-1; the stride field above it is zero and an address never carries into it).
__device__ __forceinline__ void rsrc_advance(i32x4& r, unsigned bytes) {
    const unsigned long long base =
        (((unsigned long long)(unsigned)r[1] << 32) | (unsigned)r[0]) + (unsigned long long)bytes;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)base);
    r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(base >> 32));
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((unsigned)(size_t)((__attribute__((address_space(3))) const char*)p));
}
// M0 (the LDS base of the copy) is an input operand bound to that register,
// so the compiler sets it, knows it changed, and never sees it clobbered.
// The compiler does not insert hazard wait states around inline assembly,
// so the s_nop provides them: one after an M0 write, and five after a VALU
// instruction writes an SGPR that a vector memory instruction then reads
// (the descriptor and scalar offset may come straight from v_readfirstlane
// or from a v_readlane of a spilled SGPR).
__device__ __forceinline__ void dma_to_lds16(i32x4 r, unsigned lds, int voff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" :: "{m0}"(lds), "v"(voff), "s"(r) : "memory");
}
// The same with the non-temporal hint, for data read once (streams that
// should not displace reused tiles from the L2).
__device__ __forceinline__ void dma_to_lds16_nt(i32x4 r, unsigned lds, int voff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" :: "{m0}"(lds), "v"(voff), "s"(r) : "memory");
}
// The same with a scalar offset added to the address; the range check
// applies to the scalar plus the per-lane offset.
__device__ __forceinline__ void dma_to_lds16_so(i32x4 r, unsigned lds, int voff, int soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" :: "{m0}"(lds), "v"(voff), "s"(r), "s"(soff)
                 : "memory");
}
__device__ __forceinline__ void dma_to_lds4_so(i32x4 r, unsigned lds, int voff, int soff) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, %3 offen lds" :: "{m0}"(lds), "v"(voff), "s"(r), "s"(soff)
                 : "memory");
}
// The scalar-offset copies to an LDS address given as an SGPR base plus a
// constant.  The base passes through an empty asm at every call, so the
// compiler cannot precompute base + OFF for each ring buffer of an unrolled
// loop and keep all those addresses live; the add itself stays visible to
// it (it writes SCC).
template <unsigned OFF>
__device__ __forceinline__ void dma_to_lds16_at(i32x4 r, unsigned base, int voff, int soff) {
    asm volatile("" : "+s"(base));
    dma_to_lds16_so(r, base + OFF, voff, soff);
}
template <unsigned OFF>
__device__ __forceinline__ void dma_to_lds4_at(i32x4 r, unsigned base, int voff, int soff) {
    asm volatile("" : "+s"(base));
    dma_to_lds4_so(r, base + OFF, voff, soff);
}
__device__ __forceinline__ void dma_to_lds4(i32x4 r, unsigned lds, int voff) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds" :: "{m0}"(lds), "v"(voff), "s"(r) : "memory");
}

// A read-only fp32 value at a wave-uniform index, loaded through the scalar
// data cache (the constant address space): a scalar load counts against
// lgkmcnt, not vmcnt, so waiting for it does not wait for the copies in flight.
__device__ __forceinline__ float load_uniform_f32(const float* p, int i) {
    typedef const __attribute__((address_space(4))) float cfloat;
    return ((cfloat*)p)[__builtin_amdgcn_readfirstlane(i)];
}

// ---------------------------------------------------------------------------
// dropout: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011).  Ten rounds on a 128-bit counter
// under a 64-bit key; a round multiplies words 0 and 2 by two odd constants
// into 64-bit products and mixes the halves with words 1 and 3 and the key,
// which grows by two Weyl constants between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, unsigned k0, unsigned k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const unsigned long long p0 = (unsigned long long)0xD2511F53u * c[0];
        const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * c[2];
        const u32x4 n = {(unsigned)(p1 >> 32) ^ c[1] ^ k0, (unsigned)p1, (unsigned)(p0 >> 32) ^ c[3] ^ k1,
                         (unsigned)p0};
        c = n;
    }
    return c;
}

// The random bytes of the 4 x 4 (row, key) block (4 i4 + r, 4 j4 + c) of the
// (sequence, q-head) with index bh: byte c (least significant first) of word
// r.  An element is kept iff its byte >= the threshold round(256 p).
__device__ __forceinline__ u32x4 drop_block(unsigned j4, unsigned i4, unsigned bh, unsigned off, unsigned k0,
                                            unsigned k1) {
    const u32x4 c = {j4, i4, bh, off};
    return philox4x32_10(c, k0, k1);
}
__device__ __forceinline__ bool drop_keep(unsigned word, int byte, unsigned thr) {
    return ((word >> (8 * byte)) & 0xffu) >= thr;
}
// The keep decisions of one generator output (a block of 4 rows x 4 keys):
// bit 4 c + e is byte c of word e against the threshold, element (row e, key c).
__device__ __forceinline__ unsigned drop_mask16(u32x4 w, unsigned thr) {
    unsigned m = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int c = 0; c < 4; ++c) m |= (((w[e] >> (8 * c)) & 0xffu) >= thr ? 1u : 0u) << (4 * c + e);
    }
    return m;
}
// v of lane Q of this lane's group of four consecutive lanes (a DPP quad broadcast)
template <int Q>
__device__ __forceinline__ unsigned quad_bcast(unsigned v) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, Q * 0x55, 0xf, 0xf, false);
}
// Word r (a run-time 0..3) of a generator output.
__device__ __forceinline__ unsigned word_at(u32x4 w, int r) {
    return r == 0 ? w[0] : r == 1 ? w[1] : r == 2 ? w[2] : w[3];
}
// A 4 x 4 transpose of words in a group of four consecutive lanes: lane s
// holds the output w of block s; lane c (= its lane % 4) gets word c of the
// block of lane q as element q.  Round r reads lane (c + r) % 4 (a DPP quad
// rotation), which sends its word (s - r) % 4, that is c.
__device__ __forceinline__ u32x4 quad_word_transpose(u32x4 w, int c) {
    const unsigned g0 = word_at(w, c);
    const unsigned g1 = (unsigned)__builtin_amdgcn_mov_dpp((int)word_at(w, (c + 3) & 3), 0x39, 0xf, 0xf, false);
    const unsigned g2 = (unsigned)__builtin_amdgcn_mov_dpp((int)word_at(w, (c + 2) & 3), 0x4e, 0xf, 0xf, false);
    const unsigned g3 = (unsigned)__builtin_amdgcn_mov_dpp((int)word_at(w, (c + 1) & 3), 0x93, 0xf, 0xf, false);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = (q - c) & 3;   // g_r is word c of block (c + r) % 4
        out[q] = r == 0 ? g0 : r == 1 ? g1 : r == 2 ? g2 : g3;
    }
    return out;
}

// ---------------------------------------------------------------------------
// problem geometry on the device
// ---------------------------------------------------------------------------
struct SeqInfo {
    int q0, len_q;   // first row of the sequence in Q (flattened [rows, H, D]) and its length
    int k0, len_k;
};

// used_q / used_k (varlen only, may be null): per-sequence used lengths that
// replace the offset difference; the sequence still starts at cu[b].
__device__ __forceinline__ SeqInfo seq_info(int b, int seqlen_q, int seqlen_k, int total_q, int total_k,
                                            const int32_t* cu_q, const int32_t* cu_k,
                                            const int32_t* used_q = nullptr, const int32_t* used_k = nullptr) {
    SeqInfo s;
    if (cu_q == nullptr) {
        s.q0 = b * seqlen_q;
        s.len_q = seqlen_q;
        s.k0 = b * seqlen_k;
        s.len_k = seqlen_k;
    } else {
        // offsets clamped into the buffers and lengths to the declared maxima,
        // so malformed offsets cannot address outside the tensors
        int a = min(max(cu_q[b], 0), total_q), e = min(max(cu_q[b + 1], a), total_q);
        s.q0 = a;
        s.len_q = min(e - a, seqlen_q);
        a = min(max(cu_k[b], 0), total_k);
        e = min(max(cu_k[b + 1], a), total_k);
        s.k0 = a;
        s.len_k = min(e - a, seqlen_k);
        if (used_q != nullptr) s.len_q = min(s.len_q, max(used_q[b], 0));
        if (used_k != nullptr) s.len_k = min(s.len_k, max(used_k[b], 0));
    }
    return s;
}

}  // namespace attn
