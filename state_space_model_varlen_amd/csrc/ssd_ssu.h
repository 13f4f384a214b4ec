// Helpers shared by the decode kernels (selective state update, ReplaySSM):
// 16-byte runs of state or input kept as loaded, DPP row sums, streaming stores.
#pragma once

#include <type_traits>

#include "ssd_device.h"

namespace ssd {

// Non-temporal store of 8 state values (16 bytes of bf16, 32 bytes of float).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store8_nt(bf16 *p, const float *v) {
    bf16x8 q;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = static_cast<bf16>(v[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, q), reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8_nt(f16 *p, const float *v) {
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    f16x8 q;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = static_cast<f16>(v[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, q), reinterpret_cast<u32x4 *>(p));
}
// 8 fp16 values with stochastic rounding (elements e .. e + 7 of stream kind)
__device__ __forceinline__ void store8_sr_nt(f16 *p, const float *v, const SrKey &k, uint64_t e,
                                             uint32_t kind) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sr8_f16(v, k, e, kind)),
                                reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8_nt(float *p, const float *v) {
    const f32x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(lo, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(hi, reinterpret_cast<f32x4 *>(p) + 1);
}

// 8 consecutive elements kept as loaded (16 bytes of bf16, 32 bytes of float)
// and widened to float only where they are used.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    uint4 w;
    __device__ __forceinline__ void load(const bf16 *p) { w = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void mask(uint32_t m) { w.x &= m; w.y &= m; w.z &= m; w.w &= m; }
    __device__ __forceinline__ void store(bf16 *p) const { *reinterpret_cast<uint4 *>(p) = w; }
    __device__ __forceinline__ void widen(float *f) const {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw8<f16> {
    uint4 w;
    __device__ __forceinline__ void load(const f16 *p) { w = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void mask(uint32_t m) { w.x &= m; w.y &= m; w.z &= m; w.w &= m; }
    __device__ __forceinline__ void store(f16 *p) const { *reinterpret_cast<uint4 *>(p) = w; }
    __device__ __forceinline__ void widen(float *f) const {
        typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
        const f16x8 q = __builtin_bit_cast(f16x8, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(q[i]);
    }
};
template <> struct Raw8<float> {
    uint4 lo, hi;
    __device__ __forceinline__ void load(const float *p) {
        lo = *reinterpret_cast<const uint4 *>(p);
        hi = *reinterpret_cast<const uint4 *>(p + 4);
    }
    __device__ __forceinline__ void mask(uint32_t m) {
        lo.x &= m; lo.y &= m; lo.z &= m; lo.w &= m; hi.x &= m; hi.y &= m; hi.z &= m; hi.w &= m;
    }
    __device__ __forceinline__ void store(float *p) const {
        reinterpret_cast<uint4 *>(p)[0] = lo;
        reinterpret_cast<uint4 *>(p)[1] = hi;
    }
    __device__ __forceinline__ void widen(float *f) const {
        f[0] = __uint_as_float(lo.x); f[1] = __uint_as_float(lo.y);
        f[2] = __uint_as_float(lo.z); f[3] = __uint_as_float(lo.w);
        f[4] = __uint_as_float(hi.x); f[5] = __uint_as_float(hi.y);
        f[6] = __uint_as_float(hi.z); f[7] = __uint_as_float(hi.w);
    }
};

// Sum over each aligned group of W lanes (W = N / 8: 16 or 2), every lane of
// the group ending with the total, with DPP lane moves (no LDS traffic): four
// rotations of a 16-lane row, or the swap of neighbouring lanes.
template <int W> __device__ __forceinline__ float row_sum(float v) {
    static_assert(W == 16 || W == 2, "group width");
    auto mv = [](float a, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                      decltype(ctrl)::value, 0xf,
                                                                      0xf, false));
    };
    if constexpr (W == 16) {
        v += mv(v, std::integral_constant<int, 0x128>());   // row_ror:8
        v += mv(v, std::integral_constant<int, 0x124>());   // row_ror:4
        v += mv(v, std::integral_constant<int, 0x122>());   // row_ror:2
        v += mv(v, std::integral_constant<int, 0x121>());   // row_ror:1
    } else {
        v += mv(v, std::integral_constant<int, 0xb1>());    // quad_perm:[1,0,3,2]
    }
    return v;
}

}  // namespace ssd
