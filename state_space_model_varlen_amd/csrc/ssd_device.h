// Device-side building blocks shared by the SSD prefill and decode kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Scalar conversions. bf16 <- f32 rounds to nearest even (IEEE conversion).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// ---------------------------------------------------------------------------
// 16-byte vector loads / stores of 8 bf16 or 4 float.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void load(const bf16 *p, float *out) {
        uint4 raw = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void store(bf16 *p, const float *in) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(in[i]);
        *reinterpret_cast<bf16x8 *>(p) = v;
    }
};
template <> struct Vec16<float> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void load(const float *p, float *out) {
        float4 v = *reinterpret_cast<const float4 *>(p);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
    __device__ __forceinline__ static void store(float *p, const float *in) {
        *reinterpret_cast<float4 *>(p) = make_float4(in[0], in[1], in[2], in[3]);
    }
};

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles with float32 accumulation.
//
// Operand layout used by every kernel (lane l of a wave64, KPL values per lane):
//   A (16 x K):  lane l holds A[l % 16][(l / 16) * KPL + v],  v = 0 .. KPL-1
//   B (K x 16):  lane l holds B[(l / 16) * KPL + v][l % 16]
//   D (16 x 16): lane l holds D[(l / 16) * 4 + v][l % 16],    v = 0 .. 3
// The K index of a (lane group, v) pair only has to be the same for A and B:
// the contraction sums over every K either way.
//   bf16: v_mfma_f32_16x16x32_bf16, KPL = 8, K = 32 per instruction
//   f32 : v_mfma_f32_16x16x4_f32,   KPL = 1, K = 4 per instruction
template <typename T> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int KPL = 8;
    static constexpr int K = 32;
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static void set(frag &f, int v, float x) { f[v] = static_cast<bf16>(x); }
    __device__ __forceinline__ static frag zero() {
        frag f;
#pragma unroll
        for (int v = 0; v < 8; ++v) f[v] = static_cast<bf16>(0.0f);
        return f;
    }
    // KPL consecutive storage elements starting at p (16-byte aligned).
    __device__ __forceinline__ static frag load(const bf16 *p) {
        return *reinterpret_cast<const bf16x8 *>(p);
    }
};
template <> struct Mma<float> {
    static constexpr int KPL = 1;
    static constexpr int K = 4;
    typedef float frag;
    __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static void set(frag &f, int, float x) { f = x; }
    __device__ __forceinline__ static frag zero() { return 0.0f; }
    __device__ __forceinline__ static frag load(const float *p) { return *p; }
};

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    return z;
}

// ---------------------------------------------------------------------------
// Wave-level inclusive prefix sum (wave64).
__device__ __forceinline__ float wave_inclusive_sum(float v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        float o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// Chunk metadata as written by the cumsum kernel (int32):
//   meta[0 .. S]               chunk_cu
//   meta[S + 1 + 3c + {0,1,2}] sequence, first token, token count of chunk c
struct ChunkInfo {
    int seq, start, len;
};
__device__ __forceinline__ ChunkInfo chunk_info(const int32_t *meta, int S, int c) {
    const int32_t *m = meta + (S + 1) + 3 * c;
    ChunkInfo ci;
    ci.seq = m[0];
    ci.start = m[1];
    ci.len = m[2];
    return ci;
}

}  // namespace ssd
