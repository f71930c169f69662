/*
 * attn_bwd.h -- C ABI of the MI355X (gfx950) exact-attention backward library.
 *
 * The library computes the gradient of exact softmax attention,
 *     O = dropout(softmax(s * Q K^T [+ ALiBi] [+ bias] [+ causal / local mask])) V,
 * i.e. dQ, dK and dV from Q, K, V, O, dO and the per-row log-sum-exp LSE,
 * as a fused, tiled pass that recomputes the probabilities from LSE instead
 * of storing them.  The operation and its stages are those of the
 * Composable Kernel page "block_fmha_bwd_dq_dk_dv_pipeline_trload_kr_ktr_vr.hpp
 * Source File" (BlockFmhaBwdDQDKDVPipelineTrLoadKRKTRVR, stages 1-7); the dK/dV
 * epilogue and GQA reduction follow CollectiveEpilogueBwd /
 * CollectiveEpilogueBwdGQA on "flash-attention/hopper/epilogue_bwd.hpp"; the dQ
 * conversion follows FlashAttentionBackwardPostprocess on
 * "flash_bwd_postprocess.py".
 *
 * One backward step is three calls on one stream, in this order:
 *     attn_bwd_preprocess      D = rowsum(dO * O); clears the workspace
 *     attn_bwd                 dK, dV; dQ accumulated in fp32 in the workspace
 *     attn_bwd_dq_postprocess  dQ = scale * dQaccum, converted to the I/O type
 * or two: attn_bwd_preprocess, then attn_bwd_full (dK, dV and dQ, the latter
 * written in the I/O type by the dQ pass itself where that pass owns whole
 * rows).
 * attn_fwd is a forward (O and LSE) that produces the backward's inputs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, 16-byte aligned, head
 *    dimension innermost and contiguous; rows, heads and batch entries are
 *    contiguous too unless shape->strides gives their strides.  The caller allocates and frees every buffer,
 *    the workspace included; the library never allocates device memory,
 *    frees or synchronises.  Every call only enqueues work on `stream` (a
 *    hipStream_t, NULL = the default stream) and returns.  attn_bwd and
 *    attn_bwd_full may run part of that work (the separate dQ mode's dQ
 *    kernel on problems whose dK/dV grid cannot fill the GPU) on a stream of
 *    the library's own, one per device,
 *    created at first use (not while `stream` is being captured into a
 *    graph) and held until the process ends: it is forked from `stream` by an
 *    event after the work enqueued before the call and joined back by another
 *    before the call returns, so all of it stays ordered on `stream` and the
 *    call can be captured.  attn_bwd_full_noalloc never uses it.
 *  - Layouts (element type = shape->dtype for Q K V O dO dQ dK dV; fp32 for
 *    LSE and D):
 *        dense : Q, O, dO, dQ [B, Sq, Hq, D];  K, V, dK, dV [B, Sk, Hkv, D]
 *                LSE, D [B, Hq, Sq]
 *        varlen: Q, O, dO, dQ [total_q, Hq, D]; K, V, dK, dV [total_k, Hkv, D]
 *                LSE, D [Hq, total_q]
 *    (index order; with shape->strides, element (b, i, h, d) of a dense
 *    tensor sits at b * batch + i * row + h * head + d, and row r of a
 *    varlen one at r * row + h * head + d).
 *    Varlen is selected by non-NULL cu_seqlens_q/cu_seqlens_k (device int32
 *    arrays of batch+1 nondecreasing offsets starting at 0 and ending at
 *    total_q/total_k); sequence b occupies rows [cu[b], cu[b+1]) and no
 *    sequence may be longer than seqlen_q/seqlen_k.
 *  - Used lengths (varlen only; the `seqused` arrays of the FlashAttention-3
 *    backward epilogue page): when seqused_q (seqused_k) is non-NULL,
 *    sequence b has min(seqused[b], cu[b+1] - cu[b]) query (key) rows
 *    starting at cu[b]; the rows after them take no part and their outputs
 *    (O, LSE of attn_fwd; dQ, dK, dV) are left untouched.  Given without
 *    cu_seqlens they are rejected (ATTN_ERR_BAD_SHAPE).
 *  - Causal masking is aligned to the bottom-right corner of each
 *    (sequence, head) block: key j is visible to query i iff
 *    j <= i + (len_k - len_q).  A query row that sees no key has LSE = -inf,
 *    O = 0, and gets dQ = 0.
 *  - Local (sliding-window) masks, with local = 1, use the same diagonal:
 *    key j is visible to query i iff
 *        i + off - window_left <= j <= i + off + window_right,
 *    off = len_k - len_q, a side of -1 being unbounded, intersected with the
 *    causal bound when causal = 1.  (The composable-kernel pipeline page
 *    leaves the mask's rule to its mask object; this is the reading taken.)
 *    local = 0 (a zero-initialised shape) means no window.
 *  - ALiBi: when alibi_slopes is non-NULL (device, fp32 [num_heads_q],
 *    4-byte aligned, read only), the logit of query i and key j under q-head
 *    h becomes s * q_i . k_j - alibi_slopes[h] * |i + off - j| (natural-log
 *    units, the masks' diagonal).  The composable-kernel pipeline page adds a
 *    position encoding per (row, column) after the scale without its formula;
 *    this linear bias is the reading taken.  attn_fwd's LSE includes it and
 *    attn_bwd must get the same slopes.
 *  - Elementwise bias (every dQ mode): with bias non-NULL the logit of
 *    query i, key j under q-head h of sequence b gets + bias[b * batch + h *
 *    head + i * row + j] (bias_strides, in elements; 0 broadcasts; keys
 *    contiguous), in natural-log units, in attn_fwd and attn_bwd alike.
 *    Outside ATTN_DQ_ATOMIC the kernels copy the bias in 16-byte chunks: its
 *    base and batch, head and row steps must be 16-byte aligned
 *    (ATTN_ERR_MISALIGNED otherwise).  With dbias non-NULL, attn_bwd /
 *    attn_bwd_full write dBias = dS (the gradient of the logit, rounded to
 *    the I/O type, as the composable-kernel pipeline's dBias tile) at the
 *    same positions with dbias_strides: every (i, j) of each sequence's
 *    len_q x len_k block of every q-head, zero where masked.  dbias must not
 *    overlap other tensors or itself.
 *  - Dropout (dropout_p > 0): the composable-kernel pipeline page drops
 *    elements of P after the softmax and rescales the kept ones by
 *    rp_undrop = 1 / (1 - p) ("Dropout" in its stage 2; dV, dK, dQ and dBias
 *    scaled by rp_undrop).  P and the LSE are those without dropout; O =
 *    (Z P / (1 - p)) V, and the backward gives dV = (Z P)^T dO / (1 - p),
 *    dS = P (Z dO V^T / (1 - p) - D), D = rowsum(dO * O).  The pages name no
 *    generator; Z comes from Philox4x32-10 (Salmon et al., SC 2011): one
 *    call per 4 x 4 block of (row, key) positions of a (sequence, q-head),
 *    counter = (key / 4, row / 4, sequence * Hq + q-head, dropout_offset),
 *    key = (low, high 32 bits of dropout_seed); element (row, key) takes
 *    byte key % 4 (least significant first) of output word row % 4 and is
 *    kept iff that byte >= round(256 p) (so p acts rounded to a multiple of
 *    1/256; the rescale uses p as given).  Rows and keys are positions
 *    within the sequence.  attn_fwd and attn_bwd must get the same p, seed
 *    and offset; callers advance dropout_offset (or the seed) per step.
 *  - GQA: Hq must be a multiple of Hkv; q-head h uses kv-head h / (Hq / Hkv)
 *    (contiguous groups).  dK and dV of a kv-head are the sums over its
 *    q-heads.
 *  - Errors: every call validates its arguments before touching the GPU and
 *    returns a status (attn_status_t); on error nothing is enqueued.  A launch
 *    failure reported by the HIP runtime returns ATTN_ERR_HIP.  No C++
 *    exception crosses this interface.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_ARG = 1,     /* a required pointer is NULL (the workspace included) */
    ATTN_ERR_BAD_SHAPE = 2,    /* non-positive size, Hq % Hkv != 0, causal/local not 0 or 1,
                                  window sizes below -1, varlen without both
                                  cu_seqlens, workspace too small, more than 2^27
                                  (row, head) pairs in Q or K, a negative stride,
                                  about 2 GiB or more of one sequence's rows of a
                                  tensor (seqlen x row stride), dropout_p outside
                                  [0, 1), ... */
    ATTN_ERR_UNSUPPORTED = 3,  /* dtype not F32/BF16/F16, head_dim not a multiple of 8 in
                                  [8, 256] ([8, 128] for F32), unknown dq_algo,
                                  ATTN_DQ_STORED_DS with F32 */
    ATTN_ERR_MISALIGNED = 4,   /* a tensor pointer or stride is not 16-byte aligned
                                  (cu_seqlens, seqused and alibi_slopes: 4-byte) */
    ATTN_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
    ATTN_ERR_SCRATCH = 6       /* attn_bwd_full_noalloc: the problem needs more than the
                                  library's fixed scratch memory */
} attn_status_t;

typedef enum attn_dtype {
    ATTN_DTYPE_F32 = 0,        /* fp32 I/O, fp32 MFMA contractions */
    ATTN_DTYPE_BF16 = 1,       /* bf16 I/O, bf16 MFMA operands, fp32 accumulation */
    ATTN_DTYPE_F16 = 2         /* IEEE binary16 I/O, fp16 MFMA operands, fp32
                                  accumulation (the kernels' fp16/bf16 element-type
                                  choice on the composable-kernel backward page);
                                  P and dS are rounded to fp16 like they are to bf16 */
} attn_dtype_t;

/* How attn_bwd produces dQ (the modes agree up to fp32 summation order and
 * one rounding point: for bf16/fp16, the dK/dV kernel of the separate and
 * stored-dS modes forms dS = P (dP - D) from P after its rounding to the I/O
 * type, the operand its dV product uses, where the atomic kernel and the
 * separate dQ pass use P in fp32; see attn_bwd).
 *  ATTN_DQ_SEPARATE: a query-stationary second pass recomputes S and dP per
 *    (query tile, key tile) and writes each dQ row once: no atomics, bitwise
 *    reproducible; seven contractions per tile pair instead of five.
 *  ATTN_DQ_ATOMIC: the key-stationary kernel adds dS K for each tile pair
 *    into the fp32 accumulator with global atomics (with deterministic = 1,
 *    in a fixed order per dQ tile); head dims up to 128 (wider heads run as
 *    ATTN_DQ_SEPARATE).
 *  ATTN_DQ_STORED_DS (bf16 and fp16): the key-stationary kernel stores dS
 *    in the 16-bit I/O type (the operand type the pages' dQ = dS K product
 *    uses) in the workspace; a second pass forms dQ = dS K from it and writes every
 *    accumulator row once: five contractions per tile pair, no atomics,
 *    bitwise reproducible, at the cost of a workspace that grows with
 *    Sq x Sk (2 bytes per query row and key, per q-head). */
typedef enum attn_dq_algo {
    ATTN_DQ_SEPARATE = 0,
    ATTN_DQ_ATOMIC = 1,
    ATTN_DQ_STORED_DS = 2
} attn_dq_algo_t;

/* Element strides of one tensor (FA3's (row, d, head, batch) tensor strides
 * with d contiguous): between batch entries (dense layouts; ignored for
 * varlen, whose rows are packed), between rows (tokens) and between heads.
 * All non-negative and 16-byte multiples (8 elements for bf16/fp16, 4 for
 * fp32). */
typedef struct attn_tensor_strides {
    int64_t batch;
    int64_t row;
    int64_t head;
} attn_tensor_strides_t;

/* Strides of every tensor the calls read or write (LSE and D are always
 * contiguous).  Outputs must not overlap one another or the inputs. */
typedef struct attn_strides {
    attn_tensor_strides_t q, k, v, o, dout, dq, dk, dv;
} attn_strides_t;

/* Problem description, passed by pointer and only read.  Plain old data. */
typedef struct attn_shape {
    int32_t batch;           /* dense batch B, or number of sequences when varlen */
    int32_t num_heads_q;     /* Hq */
    int32_t num_heads_kv;    /* Hkv, divides Hq */
    int32_t seqlen_q;        /* dense Sq, or the longest query sequence when varlen */
    int32_t seqlen_k;        /* dense Sk, or the longest key sequence when varlen */
    int32_t head_dim;        /* D: a multiple of 8, 8..256 (F32: ..128); the kernels pad it
                                with zeros to 64, 128 or 256 and compute at that size.
                                Above 128 ATTN_DQ_ATOMIC runs as ATTN_DQ_SEPARATE (the
                                atomic kernel keeps a K/V tile per wave in registers,
                                which does not fit at 256) */
    int32_t total_q;         /* varlen only: rows of Q (= cu_seqlens_q[batch]) */
    int32_t total_k;         /* varlen only: rows of K (= cu_seqlens_k[batch]) */
    const int32_t* cu_seqlens_q;  /* device, [batch+1], or NULL for dense */
    const int32_t* cu_seqlens_k;  /* device, [batch+1], or NULL for dense */
    float softmax_scale;     /* s in softmax(s * Q K^T); always explicit */
    int32_t causal;          /* 0 or 1 */
    int32_t deterministic;   /* 1: dQ summed in a fixed order, bitwise reproducible */
    int32_t dtype;           /* attn_dtype_t */
    int32_t dq_algo;         /* attn_dq_algo_t: how attn_bwd accumulates dQ */
    const int32_t* seqused_q;     /* varlen only: device [batch] used query lengths, or NULL */
    const int32_t* seqused_k;     /* varlen only: device [batch] used key lengths, or NULL */
    int32_t local;           /* 1: local (sliding-window) mask, see window_left/right */
    int32_t window_left;     /* local: keys at most this many before the diagonal, -1 = any */
    int32_t window_right;    /* local: keys at most this many after the diagonal, -1 = any */
    const float* alibi_slopes;    /* device [num_heads_q] fp32 ALiBi slopes, or NULL for none */
    const attn_strides_t* strides; /* HOST pointer, read during each call; NULL = the
                                      contiguous layouts above */
    const void* bias;        /* device elementwise bias (dtype), or NULL: see below */
    attn_tensor_strides_t bias_strides;
    void* dbias;             /* device output dBias (dtype), or NULL: see below */
    attn_tensor_strides_t dbias_strides;
    int64_t max_workspace_bytes;  /* 0 = no cap.  Else ATTN_DQ_STORED_DS keeps its workspace
                                     within this many bytes where it can: it runs the
                                     kv-head groups in chunks whose dS blocks fit, and,
                                     when not even one group's fit, behaves as
                                     ATTN_DQ_SEPARATE (attn_bwd_workspace_bytes reports
                                     the size of the mode taken).  Other modes ignore it */
    const int32_t* cu_seqlens_q_host;  /* varlen, optional: HOST copies of cu_seqlens_q/_k, read */
    const int32_t* cu_seqlens_k_host;  /* during each call; with both (and no seqused) the
                                          stored-dS workspace is sized exactly from them */
    uint64_t dropout_seed;   /* dropout: the generator key (see the conventions above) */
    float dropout_p;         /* drop probability in [0, 1); 0 = no dropout */
    uint32_t dropout_offset; /* dropout: the generator's fourth counter word */
} attn_shape_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_string(int status);

/* Bytes of device workspace attn_bwd_preprocess/attn_bwd/attn_bwd_dq_postprocess
 * need for this shape: the fp32 dQ accumulator ([B, Hq, Sq, D] dense,
 * [Hq, total_q, D] varlen) followed by the int32 ordering counters of the
 * deterministic mode and, for ATTN_DQ_STORED_DS, a table of per-query-tile
 * offsets and the dS blocks: 32 query rows x 128 keys of 16-bit dS each, for
 * every q-head, only for the (query tile, key tile) pairs the causal or
 * window mask leaves visible (the tiles hold 32 query rows for head dims
 * above 64, else 64).  Dense problems and varlen ones with host copies of
 * cu_seqlens are sized exactly; other varlen problems by the bound
 * (total_q / 32 + 2 batch) x ceil(seqlen_k / 128) blocks per q-head.  With
 * max_workspace_bytes the dS blocks are those of one chunk of kv-head groups
 * (or none, see attn_shape_t).  Each part is 256-byte aligned.  Returns 0 if
 * the shape is invalid. */
size_t attn_bwd_workspace_bytes(const attn_shape_t* shape);

/* Plain forward: O = softmax(s Q K^T) V and LSE (natural log) per row.
 * Not performance-tracked; used to make O/LSE inputs for the backward.
 * q, k, v: inputs; o, lse: outputs (fully overwritten). */
int attn_fwd(const attn_shape_t* shape, const void* q, const void* k, const void* v,
             void* o, float* lse, void* stream);

/* Backward preprocess: D[b, h, i] = sum_d dO[b, i, h, d] * O[b, i, h, d],
 * accumulated in fp32 (D is consumed, never shown, by the pipeline page's
 * stage 5).  Also clears the workspace parts attn_bwd accumulates into (the
 * zero-initialised accumulator contract of CollectiveEpilogueBwdGQA::store_zero):
 * the ordering counters and status words always, the dQ accumulator for
 * ATTN_DQ_ATOMIC (the other modes overwrite it).  For ATTN_DQ_STORED_DS with
 * varlen it also writes the table of each sequence's first 32-row query
 * block.
 * o, dout: inputs; delta: output [LSE layout]; workspace: output, at least
 * attn_bwd_workspace_bytes(shape) bytes (workspace_bytes says how many). */
int attn_bwd_preprocess(const attn_shape_t* shape, const void* o, const void* dout,
                        float* delta, void* workspace, size_t workspace_bytes, void* stream);

/* Main backward.  Per K/V tile (key-stationary kernel): recompute
 * P = exp(s Q K^T - LSE), dP = dO V^T, dS = P (dP - D); dV = P^T dO and
 * dK = s dS^T Q are written to dk/dv (fully overwritten, GQA groups summed,
 * zero rows for keys no query sees).  dQ / s = dS K goes to the workspace's
 * fp32 accumulator:
 *  - shape->dq_algo == ATTN_DQ_SEPARATE: a second, query-stationary kernel
 *    writes every accumulator row once (no atomics; bitwise reproducible
 *    whatever shape->deterministic says);
 *  - shape->dq_algo == ATTN_DQ_STORED_DS: the key-stationary kernel stores
 *    dS (bf16 or fp16) in the workspace and a second kernel writes every
 *    accumulator row once as the sum of dS K over the key blocks the row can
 *    see;
 *  - shape->dq_algo == ATTN_DQ_ATOMIC: the partials are added with fp32
 *    atomics, or, when shape->deterministic, in a fixed order per dQ tile so
 *    that repeated runs are bitwise identical.  The accumulator must then
 *    have been cleared by attn_bwd_preprocess for this shape since the last
 *    attn_bwd (running attn_bwd twice without it adds dQ twice).  This is
 *    the mode of the elementwise bias: it also writes dBias when asked.
 * q, k, v, dout, lse, delta: inputs; dk, dv (and shape->dbias): outputs;
 * workspace: in/out. */
int attn_bwd(const attn_shape_t* shape, const void* q, const void* k, const void* v,
             const void* dout, const float* lse, const float* delta,
             void* workspace, size_t workspace_bytes, void* dk, void* dv, void* stream);

/* dQ postprocess: dq = dtype(scale * dQaccum), the product in fp32, bf16 and
 * fp16 rounded to nearest even (FlashAttentionBackwardPostprocess).  Pass
 * scale = shape->softmax_scale.  workspace: input; dq: output. */
int attn_bwd_dq_postprocess(const attn_shape_t* shape, const void* workspace,
                            size_t workspace_bytes, void* dq, float scale, void* stream);

/* attn_bwd and the dQ conversion in one call (after attn_bwd_preprocess, in
 * place of attn_bwd + attn_bwd_dq_postprocess), with scale =
 * shape->softmax_scale and the same results bit for bit (the non-
 * deterministic atomic mode: up to the order of its atomic additions, as
 * between any two runs).  The separate and stored-dS modes, whose dQ pass
 * owns whole rows, write dq = dtype(scale * dS K) straight from that pass
 * (the product rounded to fp32, then to nearest even, as the postprocess
 * does), skipping the fp32 accumulator and the conversion pass; the atomic
 * mode runs the postprocess.  Only rows of the sequences are written (with
 * seqused, rows past the used lengths keep their contents).  Same layouts,
 * workspace and errors as attn_bwd; the accumulator's contents afterwards
 * are unspecified.
 * q, k, v, dout, lse, delta: inputs; dq, dk, dv: outputs; workspace: in/out. */
int attn_bwd_full(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                  const void* dout, const float* lse, const float* delta,
                  void* workspace, size_t workspace_bytes, void* dq, void* dk, void* dv,
                  void* stream);

/* attn_bwd_preprocess + attn_bwd_full in one call that allocates nothing and
 * takes no workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  D and the workspace live in a scratch array of
 * ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * (from its first use there to the end of the process); the call uses the
 * copy of the current device, so `stream` must belong to that device.  The
 * scratch must hold D (4 bytes per query row and q-head, rounded up to 256)
 * plus the workspace of shape->dq_algo without the fp32 dQ accumulator, which
 * only ATTN_DQ_ATOMIC needs (it then takes 4 * head_dim bytes per query row
 * and q-head); ATTN_DQ_STORED_DS also needs its dS blocks (see
 * attn_bwd_workspace_bytes).  Larger problems return ATTN_ERR_SCRATCH and
 * enqueue nothing.  Results equal those of attn_bwd_preprocess followed by
 * attn_bwd_full with the same shape, bit for bit in the separate, stored-dS
 * and deterministic atomic modes.  Every call on a GPU uses that GPU's one
 * scratch array: calls that may overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller; each call clears what
 * it needs cleared itself.
 * q, k, v, o, dout, lse: inputs; dq, dk, dv: outputs (as attn_bwd_full). */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_bwd_full_noalloc(const attn_shape_t* shape, const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse,
                          void* dq, void* dk, void* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
