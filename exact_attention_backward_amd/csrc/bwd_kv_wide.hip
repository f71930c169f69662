// The dK/dV kernel (kv_kernel.h) for head dims above 128, up to 256: four
// waves, one per SIMD, 64 keys per workgroup.  A wave's K or V slice (64
// VGPRs) and its accumulator (128) fill the VGPRs; the compiler keeps the
// overflow in the AGPRs a single wave per SIMD leaves free (no scratch).
// Its own translation unit, compiled in parallel with the narrower ones.
#include "kv_kernel.h"

namespace attn {

void launch_bwd_kv_wide(const BwdArgs& a0, int dtype, bool masked, bool store_ds, hipStream_t st) {
    using C = KvCfg<256>;
    BwdArgs a = a0;
    // key tiles of the longest sequence (with the stored dS, whole dS blocks of them)
    const int round = store_ds ? C::KPB : 1;
    a.nblk_n = (a.seqlen_k + round * C::KBN - 1) / (round * C::KBN) * round;
    a.pair_tiles = masked && (long long)a.nblk_n * a.hkv_n * a.batch > kComputeUnits;
    const unsigned grid = (unsigned)((a.pair_tiles ? (a.nblk_n + 1) / 2 : a.nblk_n) * a.hkv_n * a.batch);
    if (dtype == ATTN_DTYPE_BF16)
        launch_kv<bf16_t, 256>(a, masked, store_ds, a.alibi != nullptr, grid, st);
    else
        launch_kv<f16_t, 256>(a, masked, store_ds, a.alibi != nullptr, grid, st);
}

}  // namespace attn
