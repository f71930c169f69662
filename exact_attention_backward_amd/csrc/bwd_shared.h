// Helpers shared by the key-stationary backward kernels (bwd_main.hip and
// the dK/dV kernel of kv_kernel.h).
#pragma once

#include "common.h"
#include "launch.h"

namespace attn {

constexpr int kXcds = 8;   // accelerator complex dies of an MI355X

// 8 consecutive elements of a global row as an MFMA operand (zero if !ok).
template <class T>
__device__ __forceinline__ typename Elem<T>::op_t load_op_global(const T* p, bool ok) {
    if constexpr (sizeof(T) == 2) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok) w = *reinterpret_cast<const u32x4*>(p);
        return __builtin_bit_cast(typename Elem<T>::op_t, w);
    } else {
        f32x8 r = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (ok) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(p);
            const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                r[t] = a[t];
                r[4 + t] = b[t];
            }
        }
        return r;
    }
}

// s_waitcnt vmcnt(0) alone (lgkmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recently issued VMEM operations are
// complete (the counter retires in issue order).  gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}


}  // namespace attn
