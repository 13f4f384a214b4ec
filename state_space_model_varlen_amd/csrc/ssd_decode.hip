// Decode / MTP verify selective state update and the rollback commit on
// MI355X (gfx950). One target token plus draft tokens per request, inputs laid
// out (batch, tokens, ...) (vLLM PR #52928 "[Mamba] Add FlashInfer ReplaySSM
// support for MTP", sections "Summary" and "Design"). The state after every
// token is kept so the next step can roll back to the accepted count.
//
// Bandwidth-bound: per (request, head) the [P x N] state streams in once and
// out once per kept token; the float32 state lives in registers across tokens.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// Non-temporal store of 8 state values (16 bytes of bf16, 32 bytes of float).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store8_nt(bf16 *p, const float *v) {
    bf16x8 q;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = static_cast<bf16>(v[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, q), reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8_nt(float *p, const float *v) {
    const f32x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(lo, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(hi, reinterpret_cast<f32x4 *>(p) + 1);
}

// Block (h, r), 256 threads. The state is cut into 16-byte chunks of 8
// elements; chunk q = tid + 256 k covers row p = q / (N / 8), columns
// 8 (q % (N / 8)) .. +7, so every vector access of the block is contiguous and
// the N / 8 lanes sharing a row sit next to each other in one wave (their
// partial dot products with C are summed with lane shuffles).
template <typename TIn, typename TS, int P, int N>
__global__ __launch_bounds__(256) void state_update_kernel(
    int T, int H, int G, int num_slots, TS *cache, const int32_t *__restrict__ idx,
    const TIn *__restrict__ x, const TIn *__restrict__ dt, const float *__restrict__ A,
    const TIn *__restrict__ B, const TIn *__restrict__ C, const float *__restrict__ D,
    TIn *__restrict__ y, TS *__restrict__ inter)
{
    constexpr int CPR = N / 8;                       // chunks per state row
    constexpr int NCH = P * N / 8;                   // chunks per (request, head)
    constexpr int KC = (NCH + 255) / 256;            // chunks per thread
    const int h = blockIdx.x, r = blockIdx.y;
    const int tid = threadIdx.x;
    const int g = h / (H / G);
    const int n0 = (tid % CPR) * 8;

    const int slot = idx[r];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const int64_t PN = (int64_t)P * N;
    TS *cs = cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN;

    float st[KC][8];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int q = tid + 256 * k;
        if (q < NCH && slot_ok) {
            const int p = q / CPR;
            if constexpr (sizeof(TS) == 2) {
                Vec16<TS>::load(cs + (int64_t)p * N + n0, st[k]);
            } else {
                Vec16<TS>::load(cs + (int64_t)p * N + n0, st[k]);
                Vec16<TS>::load(cs + (int64_t)p * N + n0 + 4, st[k] + 4);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 8; ++v) st[k][v] = 0.0f;
        }
    }

    const float Ah = A[h];
    const float Dh = D ? D[h] : 0.0f;
    for (int t = 0; t < T; ++t) {
        const int64_t rt = (int64_t)r * T + t;
        const float dtv = to_f32(dt[rt * H + h]);
        const float decay = __expf(dtv * Ah);
        float b8[8], c8[8];
        const TIn *bp = B + (rt * G + g) * N + n0;
        const TIn *cp = C + (rt * G + g) * N + n0;
        if constexpr (sizeof(TIn) == 2) {
            Vec16<TIn>::load(bp, b8);
            Vec16<TIn>::load(cp, c8);
        } else {
            Vec16<TIn>::load(bp, b8);
            Vec16<TIn>::load(bp + 4, b8 + 4);
            Vec16<TIn>::load(cp, c8);
            Vec16<TIn>::load(cp + 4, c8 + 4);
        }
        const TIn *xr = x + (rt * H + h) * P;
        TIn *yr = y + (rt * H + h) * P;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            const int q = tid + 256 * k;
            if (q < NCH) {
                const int p = q / CPR;
                const float xv = to_f32(xr[p]);
                const float u = dtv * xv;
                float part = 0.0f;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    st[k][v] = decay * st[k][v] + u * b8[v];
                    part += c8[v] * st[k][v];
                }
                part = group_sum(part, CPR);
                if ((tid % CPR) == 0) yr[p] = from_f32<TIn>(part + Dh * xv);
                if (inter) {
                    // written once and read only by a later rollback: stream past the caches
                    TS *ip = inter + (rt * H + h) * PN + (int64_t)p * N + n0;
                    store8_nt(ip, st[k]);
                }
            }
        }
    }
    if (!inter && slot_ok) {
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            const int q = tid + 256 * k;
            if (q < NCH) {
                const int p = q / CPR;
                if constexpr (sizeof(TS) == 2) {
                    Vec16<TS>::store(cs + (int64_t)p * N + n0, st[k]);
                } else {
                    Vec16<TS>::store(cs + (int64_t)p * N + n0, st[k]);
                    Vec16<TS>::store(cs + (int64_t)p * N + n0 + 4, st[k] + 4);
                }
            }
        }
    }
}

// Rollback commit: cache[idx[r]] = inter[r, accepted[r]], 16 bytes per thread.
template <typename TS>
__global__ __launch_bounds__(256) void state_commit_kernel(int T, int64_t HPN, int num_slots,
                                                           TS *cache, const int32_t *__restrict__ idx,
                                                           const TS *__restrict__ inter,
                                                           const int32_t *__restrict__ accepted)
{
    constexpr int VE = 16 / sizeof(TS);
    const int r = blockIdx.y;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VE;
    const int a = accepted[r];
    const int slot = idx[r];
    if (e >= HPN || a < 0 || a >= T || slot < 0 || slot >= num_slots) return;
    const uint4 v = *reinterpret_cast<const uint4 *>(inter + ((int64_t)r * T + a) * HPN + e);
    *reinterpret_cast<uint4 *>(cache + (int64_t)slot * HPN + e) = v;
}

template <typename TIn, typename TS, int P, int N>
static void launch_ssu_t(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *inter, hipStream_t st)
{
    dim3 grid(d.H, d.R);
    hipLaunchKernelGGL((state_update_kernel<TIn, TS, P, N>), grid, dim3(256), 0, st, d.T, d.H, d.G,
                       d.num_slots, static_cast<TS *>(cache), idx, static_cast<const TIn *>(x),
                       static_cast<const TIn *>(dt), A, static_cast<const TIn *>(B),
                       static_cast<const TIn *>(C), D, static_cast<TIn *>(y),
                       static_cast<TS *>(inter));
}

template <typename TIn, typename TS>
static void launch_ssu_pn(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                          const void *dt, const float *A, const void *B, const void *C,
                          const float *D, void *y, void *inter, hipStream_t st)
{
    if (d.P == 64 && d.N == 128) launch_ssu_t<TIn, TS, 64, 128>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
    else if (d.P == 64 && d.N == 16) launch_ssu_t<TIn, TS, 64, 16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
    else if (d.P == 16 && d.N == 128) launch_ssu_t<TIn, TS, 16, 128>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
    else launch_ssu_t<TIn, TS, 16, 16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
}

void launch_state_update(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *inter, void *stream)
{
    if (d.R <= 0 || d.T <= 0) return;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (d.in_bf16) {
        if (d.state_bf16) launch_ssu_pn<bf16, bf16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
        else launch_ssu_pn<bf16, float>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
    } else {
        if (d.state_bf16) launch_ssu_pn<float, bf16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
        else launch_ssu_pn<float, float>(d, cache, idx, x, dt, A, B, C, D, y, inter, st);
    }
}

void launch_state_commit(const DecodeDims &d, void *cache, const int32_t *idx, const void *inter,
                         const int32_t *accepted, void *stream)
{
    if (d.R <= 0 || d.T <= 0) return;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t HPN = (int64_t)d.H * d.P * d.N;
    const int VE = d.state_bf16 ? 8 : 4;
    dim3 grid((unsigned)((HPN / VE + 255) / 256), d.R);
    if (d.state_bf16)
        hipLaunchKernelGGL(state_commit_kernel<bf16>, grid, dim3(256), 0, st, d.T, HPN, d.num_slots,
                           static_cast<bf16 *>(cache), idx, static_cast<const bf16 *>(inter),
                           accepted);
    else
        hipLaunchKernelGGL(state_commit_kernel<float>, grid, dim3(256), 0, st, d.T, HPN, d.num_slots,
                           static_cast<float *>(cache), idx, static_cast<const float *>(inter),
                           accepted);
}

}  // namespace ssd
