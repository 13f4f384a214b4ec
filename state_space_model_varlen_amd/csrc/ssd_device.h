// Device-side building blocks shared by the SSD prefill and decode kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include "ssd_launch.h"

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef _Float16 f16;
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
__device__ __forceinline__ float to_f32(f16 v) { return static_cast<float>(v); }
template <> __device__ __forceinline__ f16 from_f32<f16>(float v) { return static_cast<f16>(v); }

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
template <> struct Vec16<f16> {
    static constexpr int kElems = 8;
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    __device__ __forceinline__ static void load(const f16 *p, float *out) {
        const f16x8 v = *reinterpret_cast<const f16x8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = static_cast<float>(v[i]);
    }
    __device__ __forceinline__ static void store(f16 *p, const float *in) {
        f16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<f16>(in[i]);
        *reinterpret_cast<f16x8 *>(p) = v;
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

// Step-size preprocessing (see DtTf): softplus(v) = log(1 + exp(v)), v itself
// above 20, then the clamp; `bias` is bias[h], read once by the caller. Callers
// test tf.on once per group of already-loaded values (a branch right after a
// load would make the compiler wait on that load there).
__device__ __forceinline__ float dt_transform(const DtTf &tf, float raw, float bias) {
    const float v = raw + bias;
    const float sp = v > 20.0f ? v : log1pf(__expf(v));
    return fminf(fmaxf(sp, tf.lo), tf.hi);
}

// LDS writes of a wave made visible to the same wave's later reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
// 4-element loads / stores (16 bytes of float, 8 bytes of bf16) widened to float.
template <typename T> __device__ __forceinline__ void load4(const T *p, float *v);
template <> __device__ __forceinline__ void load4<float>(const float *p, float *v) {
    const float4 q = *reinterpret_cast<const float4 *>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <> __device__ __forceinline__ void load4<bf16>(const bf16 *p, float *v) {
    const uint2 q = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
}
template <> __device__ __forceinline__ void load4<f16>(const f16 *p, float *v) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 q = *reinterpret_cast<const f16x4 *>(p);
    v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
}
template <typename T> __device__ __forceinline__ void store4(T *p, const float *v);
template <> __device__ __forceinline__ void store4<float>(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, const float *v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 q;
    q[0] = static_cast<bf16>(v[0]);
    q[1] = static_cast<bf16>(v[1]);
    q[2] = static_cast<bf16>(v[2]);
    q[3] = static_cast<bf16>(v[3]);
    *reinterpret_cast<bf16x4 *>(p) = q;
}

template <> __device__ __forceinline__ void store4<f16>(f16 *p, const float *v) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 q;
    q[0] = static_cast<f16>(v[0]);
    q[1] = static_cast<f16>(v[1]);
    q[2] = static_cast<f16>(v[2]);
    q[3] = static_cast<f16>(v[3]);
    *reinterpret_cast<f16x4 *>(p) = q;
}

// ---------------------------------------------------------------------------
// Stochastic rounding of fp16 state stores.
//
// Philox4x32 with R rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): per round two 32 x 32 -> 64-bit
// products of counter words with fixed multipliers, the high halves mixed with
// the other counter words and the key, the key bumped by two Weyl constants
// between rounds. Element e of a destination array of kind k takes the 16-bit
// half e % 2 (low half first) of word (e / 2) % 4 of
// Philox(counter = (e / 8 low, e / 8 high, k, 0), key = seed): one call draws
// for 8 consecutive elements.
__device__ __forceinline__ uint4 philox4x32(uint4 c, uint32_t k0, uint32_t k1, int rounds)
{
    for (int r = 0; r < rounds; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // (one 32 x 32 -> 64-bit product each: both halves from one multiply)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// x rounded to one of the two fp16 values bracketing it: the one away from zero
// with probability (|x| - |lo|) / (|hi| - |lo|), taken when d / 2^16 < probability
// for a 16-bit draw d (d < 2^16). The probability has at most 13 fractional bits
// for normal fp16 spacings and at most 16 for |x| >= 2^-17, so there the draw is
// exactly unbiased. Non-finite values and |x| > 65504 round to nearest even.
//
// Without branches or fp16 conversions on the stochastic side:
// - fp16 normal range (|x| >= 2^-14): the probability is L / 2^13 for the 13
//   float32 mantissa bits L that fp16 drops, and d / 2^16 < L / 2^13 exactly
//   when (d >> 3) < L, i.e. when adding 8191 - (d >> 3) to |x|'s bits carries
//   into the kept bits; truncating then gives hi (the carry may step the
//   exponent, as it should) or lo. The fp16 bits are the float32 bits shifted
//   by 13 with the exponent rebased by 127 - 15 = 112.
// - below 2^-14 (fp16 subnormals, spacing 2^-24): t = |x| 2^24 is exact, lo is
//   floor(t) units of 2^-24 and the probability is t - floor(t), both exact.
__device__ __forceinline__ f16 sr_f16(float x, uint32_t d)
{
    const uint32_t xb = __builtin_bit_cast(uint32_t, x);
    const uint32_t ab = xb & 0x7FFFFFFFu;
    const float a = __builtin_bit_cast(float, ab);
    const uint32_t nb = ((ab + (8191u - (d >> 3))) >> 13) - (112u << 10);
    const float t = fminf(a, 0x1p-14f) * 0x1p24f;     // (clamped: used below 2^-14 only)
    const float fl = floorf(t);
    const uint32_t sb = (uint32_t)fl + (static_cast<float>(d) * 0x1p-16f < t - fl ? 1u : 0u);
    const uint32_t mag = a < 0x1p-14f ? sb : nb;
    const uint16_t res = (uint16_t)(mag | ((xb >> 16) & 0x8000u));
    return a <= 65504.0f ? __builtin_bit_cast(f16, res) : static_cast<f16>(x);
}

// M values (M even) rounded as by sr_f16, packed two fp16 values per word
// (value 2 j in the low half of out[j]); value 2 j draws the low 16 bits of
// w[j], value 2 j + 1 the high 16 bits. In the fp16 normal range
// (2^-14 <= |x| <= 65504) only the carry step runs, and gfx950 has it as one
// instruction: v_cvt_sr_f16_f32 adds the top 13 bits of its 32-bit random
// operand to the 13 float32 mantissa bits that fp16 drops, truncates, and
// writes the fp16 result with its sign into the half of the destination that
// its word-select operand names (the other half kept). The carry step adds
// 8191 - (d >> 3), which for d = the low 16 bits of w is the top 13 bits of
// ~w << 16, and for d = the high 16 bits the top 13 bits of ~w itself. (The
// instruction's use of its operand was checked on the device value by value
// against this carry rule over the whole normal range; below 2^-14 it still
// adds 13 bits at the normal-range position, which is not the rule there.
// The bit-exact tests compare every store with the oracle's rounding.)
// Value slot i of the M is redone with the general rule, behind a
// wave-uniform branch, when some lane holds a value outside the normal range
// in that slot: state values near zero are common, and deciding per slot
// rather than once for all M keeps most slots on the one-instruction path.
// Inside the branch the lanes in the normal range keep the convert's result.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <int M>
__device__ __forceinline__ void sr_f16_pairs(const float *v, const uint32_t *w, uint32_t *out)
{
    static_assert(M % 2 == 0, "pairs");
#pragma unroll
    for (int j = 0; j < M / 2; ++j) {
        const uint32_t nw = ~w[j];
        f16x2 q = {};
        q = __builtin_amdgcn_cvt_sr_f16_f32(q, v[2 * j], nw << 16, false);
        q = __builtin_amdgcn_cvt_sr_f16_f32(q, v[2 * j + 1], nw, true);
        uint32_t r = __builtin_bit_cast(uint32_t, q);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // 2 (|x| bits - bits(2^-14)), modulo 2^32: above 2 (bits(65504) - bits(2^-14))
            // for |x| < 2^-14, |x| > 65504, infinities and NaNs
            const uint32_t off = (__builtin_bit_cast(uint32_t, v[2 * j + h]) << 1) -
                                 (0x38800000u << 1);
            if (__builtin_amdgcn_ballot_w64(off > ((0x477FE000u - 0x38800000u) << 1)) != 0) {
                // sr_f16's rule where the convert's result does not apply: below
                // 2^-14, floor(t) units of 2^-24 plus one when d / 2^16 < t - floor(t)
                // (t = |x| 2^24, every step exact; the truncating conversion is the
                // floor of t >= 0); above 65504 and for non-finite values, nearest
                const float xv = v[2 * j + h];
                const float a = fabsf(xv);
                const float t = fminf(a, 0x1p-14f) * 0x1p24f;   // (at most 2^10)
                const uint32_t d = h ? w[j] >> 16 : w[j] & 0xFFFFu;
                const uint32_t sb =
                    (uint32_t)t + ((float)d < __builtin_amdgcn_fractf(t) * 65536.0f ? 1u : 0u);
                uint32_t g = h ? r >> 16 : r & 0xFFFFu;
                g = a < 0x1p-14f ? sb | ((__builtin_bit_cast(uint32_t, xv) >> 16) & 0x8000u) : g;
                g = a <= 65504.0f ? g : (uint32_t)__builtin_bit_cast(uint16_t, static_cast<f16>(xv));
                r = h ? (r & 0xFFFFu) | (g << 16) : (r & 0xFFFF0000u) | g;
            }
        }
        out[j] = r;
    }
}

// Philox streams of the state arrays a kernel writes
constexpr uint32_t kSrFinal = 0, kSrCkpt = 1, kSrStates = 2, kSrReplay = 3;

// The key of one kernel's stores (seed read once); rounds = 0: nearest even.
struct SrKey {
    uint32_t k0 = 0, k1 = 0;
    int rounds = 0;
};
// `standin`: any 8 readable bytes, loaded instead of the seed when there is none
// (so no branch separates the load from its use)
__device__ __forceinline__ SrKey sr_key(const SrCtx &c, const void *standin)
{
    const uint64_t s = *(c.seed ? c.seed : reinterpret_cast<const uint64_t *>(standin));
    SrKey k;
    k.k0 = (uint32_t)s;
    k.k1 = (uint32_t)(s >> 32);
    k.rounds = c.seed ? c.rounds : 0;
    return k;
}
// The same without a stand-in (the seed is read only when there is one), for
// kernels with no array known to hold 8 bytes.
__device__ __forceinline__ SrKey sr_key_checked(const SrCtx &c)
{
    SrKey k;
    if (c.seed) {
        const uint64_t s = *c.seed;
        k.k0 = (uint32_t)s;
        k.k1 = (uint32_t)(s >> 32);
        k.rounds = c.rounds;
    }
    return k;
}

// The four words that draw for elements 8 (e / 8) .. 8 (e / 8) + 7 of stream kind.
__device__ __forceinline__ uint4 sr_words(const SrKey &k, uint64_t e, uint32_t kind) {
    const uint64_t blk = e >> 3;
    return philox4x32(make_uint4((uint32_t)blk, (uint32_t)(blk >> 32), kind, 0u), k.k0, k.k1,
                      k.rounds);
}
__device__ __forceinline__ uint32_t sr_lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t sr_hi16(uint32_t w) { return w >> 16; }

// 4 consecutive state values to storage; e = flat index of the first one in the
// destination array (a multiple of 4), kind = its stream. Only fp16 stores round
// stochastically.
template <typename T>
__device__ __forceinline__ void put4(T *p, const float *v, const SrKey &, uint64_t, uint32_t) {
    store4<T>(p, v);
}
template <>
__device__ __forceinline__ void put4<f16>(f16 *p, const float *v, const SrKey &k, uint64_t e,
                                          uint32_t kind) {
    if (k.rounds == 0) {
        store4<f16>(p, v);
        return;
    }
    const uint4 w = sr_words(k, e, kind);
    // elements 8 (e / 8) .. + 3 take words 0 and 1, the next four words 2 and 3
    const bool upper = (e >> 2) & 1;
    const uint32_t ws[2] = {upper ? w.z : w.x, upper ? w.w : w.y};
    uint32_t q[2];
    sr_f16_pairs<4>(v, ws, q);
    *reinterpret_cast<uint2 *>(p) = make_uint2(q[0], q[1]);
}
// 8 consecutive state values (elements e .. e + 7 of stream kind, e a multiple
// of 8) stochastically rounded to fp16 with one Philox call, as 16 bytes;
// k.rounds > 0.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 sr8_f16(const float *v, const SrKey &k, uint64_t e,
                                         uint32_t kind) {
    const uint4 w = sr_words(k, e, kind);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t q[4];
    sr_f16_pairs<8>(v, ws, q);
    return __builtin_bit_cast(f16x8, make_uint4(q[0], q[1], q[2], q[3]));
}
// The same stored at p (16-byte aligned)
__device__ __forceinline__ void put8_sr(f16 *p, const float *v, const SrKey &k, uint64_t e,
                                        uint32_t kind) {
    *reinterpret_cast<f16x8 *>(p) = sr8_f16(v, k, e, kind);
}

// ---------------------------------------------------------------------------
// LDS transpose read (gfx950 ds_read_b64_tr_b16). Each lane names an 8-byte
// word (4 bf16); inside every group of 16 lanes, lane i receives element
// (i % 4) of the words named by lanes 4 v + i / 4, v = 0 .. 3.
//
// mfma_frag_tr() builds the 16x16x32 operand fragment (8 K-values for one
// M/N index per lane, K = 8 (lane / 16) + v) from a row-major LDS tile whose
// rows are the K index and whose 16 columns starting at `col0` are the M/N
// index: lane j of a group names row k0 + 8 kg + j / 4, columns col0 + 4 (j % 4),
// so lane i gets rows k0 + 8 kg + v of column col0 + i. Two reads give v = 0..7.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i16 lds_read_tr16(const bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(p));
}
__device__ __forceinline__ bf16x8 mfma_frag_tr(const bf16 *tile, int ld, int k0, int col0,
                                               int lane) {
    const int kg = lane >> 4, j = lane & 15;
    const bf16 *p = tile + (k0 + 8 * kg + (j >> 2)) * ld + col0 + 4 * (j & 3);
    const v4i16 lo = lds_read_tr16(p);
    const v4i16 hi = lds_read_tr16(p + 4 * ld);
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

// Same fragment with the "split" K order: lane group kg holds K = 4 kg + v for
// v < 4 and K = 16 + 4 kg + (v - 4) for v >= 4. Each read then covers 16
// consecutive tile rows across the wave, so with a row pitch of 40 dwords
// the 8 rows one 32-lane half reads start in 8 distinct 8-bank groups (no
// bank conflicts), and with 36 dwords they overlap in 4 banks only. Both
// operands of an MFMA must use the same K order.
__device__ __forceinline__ bf16x8 mfma_frag_tr_split(const bf16 *tile, int ld, int k0, int col0,
                                                     int lane) {
    const int kg = lane >> 4, j = lane & 15;
    const bf16 *p = tile + (k0 + 4 * kg + (j >> 2)) * ld + col0 + 4 * (j & 3);
    const v4i16 lo = lds_read_tr16(p);
    const v4i16 hi = lds_read_tr16(p + 16 * ld);
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

// ---------------------------------------------------------------------------
// M consecutive elements (M a multiple of 8 for bf16, of 4 for float) as
// 16-byte vector loads / stores, widened to / narrowed from float.
template <typename T, int M> __device__ __forceinline__ void load_run(const T *p, float *v) {
    constexpr int E = Vec16<T>::kElems;
    static_assert(M % E == 0, "whole 16-byte vectors only");
#pragma unroll
    for (int i = 0; i < M / E; ++i) Vec16<T>::load(p + E * i, v + E * i);
}
template <typename T, int M> __device__ __forceinline__ void store_run(T *p, const float *v) {
    constexpr int E = Vec16<T>::kElems;
    static_assert(M % E == 0, "whole 16-byte vectors only");
#pragma unroll
    for (int i = 0; i < M / E; ++i) Vec16<T>::store(p + E * i, v + E * i);
}
// M consecutive state values (M a multiple of 8, e a multiple of 8, p 16-byte
// aligned for fp16)
template <typename T, int M>
__device__ __forceinline__ void put_run(T *p, const float *v, const SrKey &k, uint64_t e,
                                        uint32_t kind) {
    if constexpr (std::is_same<T, f16>::value) {
        static_assert(M % 8 == 0, "runs of 8");
        if (k.rounds == 0) {
            store_run<f16, M>(p, v);
            return;
        }
#pragma unroll
        for (int i = 0; i < M / 8; ++i) put8_sr(p + 8 * i, v + 8 * i, k, e + 8 * i, kind);
    } else {
        store_run<T, M>(p, v);
    }
}

// ---------------------------------------------------------------------------
// Raw buffer loads (gfx9 buffer resource: base address, no stride, a size in
// bytes, dword 3 = 0x00020000). A load at a byte offset at or past the size
// returns zeros and touches no memory: the prefill kernels give each chunk's
// tile a resource ending at the chunk's last row, so rows past the end come
// back as zeros with no branch and no clamped address.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float buf_ldf(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
// 8-byte store; one at or past the resource's size is dropped
__device__ __forceinline__ void buf_st8(rsrc_t r, uint32_t off, uint2 v) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i, v), r, (int)off, 0, 0);
}
// 4 consecutive state values of type T at byte offset `off` as floats; zeros at
// or past the resource's size (an empty resource reads nothing)
template <typename T> __device__ __forceinline__ void buf_load4(rsrc_t r, uint32_t off, float *v);
template <> __device__ __forceinline__ void buf_load4<float>(rsrc_t r, uint32_t off, float *v) {
    const uint4 w = buf_ld16(r, off);
    v[0] = __uint_as_float(w.x);
    v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z);
    v[3] = __uint_as_float(w.w);
}
template <> __device__ __forceinline__ void buf_load4<bf16>(rsrc_t r, uint32_t off, float *v) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    v[0] = __uint_as_float((uint32_t)w[0] << 16);
    v[1] = __uint_as_float((uint32_t)w[0] & 0xffff0000u);
    v[2] = __uint_as_float((uint32_t)w[1] << 16);
    v[3] = __uint_as_float((uint32_t)w[1] & 0xffff0000u);
}
template <> __device__ __forceinline__ void buf_load4<f16>(rsrc_t r, uint32_t off, float *v) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 q = __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    v[0] = static_cast<float>(q[0]);
    v[1] = static_cast<float>(q[1]);
    v[2] = static_cast<float>(q[2]);
    v[3] = static_cast<float>(q[3]);
}
// four floats as bf16 (round to nearest even), in one 8-byte word
__device__ __forceinline__ uint2 pack_bf16x4(const float *v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 q;
    q[0] = static_cast<bf16>(v[0]);
    q[1] = static_cast<bf16>(v[1]);
    q[2] = static_cast<bf16>(v[2]);
    q[3] = static_cast<bf16>(v[3]);
    return __builtin_bit_cast(uint2, q);
}

// ---------------------------------------------------------------------------
// CB in MFMA fragment order (bf16 inputs). For row tile rt = i / 16 and K block
// ks = j / 32 of a chunk, the 16 x 32 A fragment of the intra-chunk product is
// stored as 64 lanes x 8 bf16 (one contiguous 1 KiB wave load): lane
// i % 16 + 16 kg, element v, in the split K order j % 32 = 4 kg + v % 4 + 16 (v / 4).
__host__ __device__ __forceinline__ int64_t cb_frag_offset(int Q, int i, int j) {
    const int rt = i >> 4, ks = j >> 5, jl = j & 31;
    const int kg = (jl & 15) >> 2, v = (jl & 3) + ((jl >> 4) << 2);
    const int lane = (i & 15) + 16 * kg;
    return (((int64_t)rt * (Q >> 5) + ks) * 64 + lane) * 8 + v;
}

// ---------------------------------------------------------------------------
// XCD-aware block order. Workgroups are dispatched round-robin over the 8 XCDs
// (each with its own L2); this maps the hardware block id to a logical id so
// that each XCD works on one contiguous range of logical ids, which keeps
// blocks that share data (the same chunk's B, C and CB) on one L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical_block(int pid, int nblocks) {
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    const int xcd = pid % kXcds, slot = pid / kXcds;
    const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + slot;
}

// ---------------------------------------------------------------------------
// Chunk metadata as written by the cumsum kernel (int32):
//   meta[0 .. S]               chunk_cu
//   meta[S + 1 + 3c + {0,1,2}] sequence, first token, token count of chunk c
//   meta[S + 1 + 3 mc + s]     cu_seqlens[s] clamped to [0, T], s = 0..S
//                              (mc = max_chunks): sequence s spans tokens
//                              [meta[..s], max(meta[..s], meta[..s + 1]))
//   meta[2 (S + 1) + 3 mc + s] tokens in the first chunk of sequence s (Q, or
//                              fewer in align mode), s = 0..S-1
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
