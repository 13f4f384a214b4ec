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
#include "ssd_ssu.h"

namespace ssd {

// Block (h, r), 256 threads. The state is cut into 16-byte chunks of 8
// elements; chunk q = tid + 256 k covers row p = q / (N / 8), columns
// 8 (q % (N / 8)) .. +7, so every vector access of the block is contiguous and
// the N / 8 lanes sharing a row sit next to each other in one wave (their
// partial dot products with C are summed across the lanes).
//
// Tokens are handled TM at a time: every load of a group (the state, and dt,
// x, B, C of its TM tokens) is issued before any arithmetic, with no branch
// between a load and its use (token indices past T are clamped, the state of an
// invalid slot is loaded from slot 0 and zeroed), so the block waits on memory
// once per group instead of once per load.
template <typename TIn, typename TS, int P, int N, int TM>
__global__ __launch_bounds__(256) void state_update_kernel(
    int T, int H, int G, int num_slots, TS *cache, const int32_t *__restrict__ idx,
    const TIn *__restrict__ x, const TIn *__restrict__ dt, const float *__restrict__ A,
    const TIn *__restrict__ B, const TIn *__restrict__ C, const float *__restrict__ D,
    TIn *__restrict__ y, TS *__restrict__ inter, const int32_t *__restrict__ cu, int Ttot,
    DtTf tf, SrCtx sr)
{
    constexpr int CPR = N / 8;                       // chunks per state row
    constexpr int NCH = P * N / 8;                   // chunks per (request, head)
    constexpr int KC = (NCH + 255) / 256;            // chunks per thread
    static_assert(NCH % 256 == 0 || KC == 1, "chunk split");
    const int h = blockIdx.x, r = blockIdx.y;
    const int tid = threadIdx.x;
    const int g = h / (H / G);
    const int n0 = (tid % CPR) * 8;

    // tokens of request r: tb .. tb + Tr - 1 of the packed rows
    int tb = r * T, Tr = T;
    if (cu) {
        int a = cu[r], b = cu[r + 1];
        a = a < 0 ? 0 : (a > Ttot ? Ttot : a);
        b = b < 0 ? 0 : (b > Ttot ? Ttot : b);
        tb = a;
        Tr = b > a ? b - a : 0;
    }
    if (Tr == 0) return;   // no token: nothing changes
    const int slot = idx[r];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const int64_t PN = (int64_t)P * N;
    TS *cs = cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN;

    int qk[KC], pk[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int q = tid + 256 * k;
        qk[k] = q < NCH ? q : NCH - 1;       // (only when NCH < 256: duplicates, not stored)
        pk[k] = qk[k] / CPR;
    }
    const float Ah = A[h];
    const float Dh = D ? D[h] : 0.0f;
    const float bh = tf.bias ? tf.bias[h] : 0.0f;
    const SrKey srk = sr_key(sr, cache);
    float dtv[TM], xv[TM][KC];
    Raw8<TIn> braw[TM], craw[TM];
    // requests dt, x, B, C of tokens t0 .. t0 + TM - 1 (clamped to Tr - 1)
    auto load_group = [&](int t0) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int t = t0 + j < Tr ? t0 + j : Tr - 1;
            const int64_t rt = (int64_t)tb + t;
            dtv[j] = to_f32(dt[rt * H + h]);
            braw[j].load(B + (rt * G + g) * N + n0);
            craw[j].load(C + (rt * G + g) * N + n0);
#pragma unroll
            for (int k = 0; k < KC; ++k) xv[j][k] = to_f32(x[(rt * H + h) * P + pk[k]]);
        }
    };

    // the state and the first token group are requested together; the state of an
    // invalid slot is loaded from slot 0 and cleared bit-wise (no branch)
    const uint32_t keep = slot_ok ? 0xffffffffu : 0u;
    float st[KC][8];
    {
        Raw8<TS> sr[KC];
        load_group(0);
#pragma unroll
        for (int k = 0; k < KC; ++k) sr[k].load(cs + (int64_t)pk[k] * N + n0);
        __builtin_amdgcn_sched_barrier(0);   // keep every request of the group ahead of the waits
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            sr[k].mask(keep);
            sr[k].widen(st[k]);
        }
    }

    // (Tr >= 1, so the first group always runs and its loads are not sunk past a
    // loop-entry test)
    int t0 = 0;
    do {
        if (t0 > 0) load_group(t0);
        if (tf.on) {
#pragma unroll
            for (int j = 0; j < TM; ++j) dtv[j] = dt_transform(tf, dtv[j], bh);
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            if (t0 + j >= Tr) break;
            const int64_t rt = (int64_t)tb + t0 + j;
            const float decay = __expf(dtv[j] * Ah);
            float b8[8], c8[8];
            braw[j].widen(b8);
            craw[j].widen(c8);
            TIn *yr = y + (rt * H + h) * P;
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                const float u = dtv[j] * xv[j][k];
                float part = 0.0f;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    st[k][v] = decay * st[k][v] + u * b8[v];
                    part += c8[v] * st[k][v];
                }
                part = row_sum<CPR>(part);
                if ((tid % CPR) == 0 && tid + 256 * k < NCH)
                    yr[pk[k]] = from_f32<TIn>(part + Dh * xv[j][k]);
                if (inter && tid + 256 * k < NCH) {
                    // written once and read only by a later rollback: stream past the caches
                    const int64_t io = (rt * H + h) * PN + (int64_t)pk[k] * N + n0;
                    if constexpr (std::is_same<TS, f16>::value) {
                        if (srk.rounds > 0)
                            store8_sr_nt(inter + io, st[k], srk, (uint64_t)io, kSrStates);
                        else
                            store8_nt(inter + io, st[k]);
                    } else
                        store8_nt(inter + io, st[k]);
                }
            }
        }
        t0 += TM;
    } while (t0 < Tr);
    if (!inter && slot_ok) {
        const int64_t so = (int64_t)slot * H * PN + (int64_t)h * PN;
#pragma unroll
        for (int k = 0; k < KC; ++k)
            if (tid + 256 * k < NCH)
                put_run<TS, 8>(cs + (int64_t)pk[k] * N + n0, st[k], srk,
                               (uint64_t)(so + (int64_t)pk[k] * N + n0), kSrFinal);
    }
}

// Rollback commit: cache[idx[r]] = inter[token a of request r], 16 bytes per
// thread (request r's tokens: r T .., or cu[r] .. cu[r+1]-1 when packed).
template <typename TS>
__global__ __launch_bounds__(256) void state_commit_kernel(int T, int64_t HPN, int num_slots,
                                                           TS *cache, const int32_t *__restrict__ idx,
                                                           const TS *__restrict__ inter,
                                                           const int32_t *__restrict__ accepted,
                                                           const int32_t *__restrict__ cu, int Ttot)
{
    constexpr int VE = 16 / sizeof(TS);
    const int r = blockIdx.y;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VE;
    int tb = r * T, Tr = T;
    if (cu) {
        int a0 = cu[r], b0 = cu[r + 1];
        a0 = a0 < 0 ? 0 : (a0 > Ttot ? Ttot : a0);
        b0 = b0 < 0 ? 0 : (b0 > Ttot ? Ttot : b0);
        tb = a0;
        Tr = b0 > a0 ? b0 - a0 : 0;
    }
    const int a = accepted[r];
    const int slot = idx[r];
    if (e >= HPN || a < 0 || a >= Tr || slot < 0 || slot >= num_slots) return;
    const uint4 v = *reinterpret_cast<const uint4 *>(inter + ((int64_t)tb + a) * HPN + e);
    *reinterpret_cast<uint4 *>(cache + (int64_t)slot * HPN + e) = v;
}

template <typename TIn, typename TS, int P, int N>
static void launch_ssu_t(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *inter, hipStream_t st, const int32_t *cu,
                         int Ttot, const DtTf &tf)
{
    dim3 grid(d.H, d.R);
#define SSD_SSU_LAUNCH(TM)                                                                        \
    hipLaunchKernelGGL((state_update_kernel<TIn, TS, P, N, TM>), grid, dim3(256), 0, st, d.T,     \
                       d.H, d.G, d.num_slots, static_cast<TS *>(cache), idx,                      \
                       static_cast<const TIn *>(x), static_cast<const TIn *>(dt), A,              \
                       static_cast<const TIn *>(B), static_cast<const TIn *>(C), D,               \
                       static_cast<TIn *>(y), static_cast<TS *>(inter), cu, Ttot, tf, d.sr)
    // tokens per load group: the whole request when it has up to 4 tokens
    if (d.T <= 1) SSD_SSU_LAUNCH(1);
    else if (d.T <= 2) SSD_SSU_LAUNCH(2);
    else if (d.T <= 3) SSD_SSU_LAUNCH(3);
    else SSD_SSU_LAUNCH(4);
#undef SSD_SSU_LAUNCH
}

template <typename TIn, typename TS>
static void launch_ssu_pn(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                          const void *dt, const float *A, const void *B, const void *C,
                          const float *D, void *y, void *inter, hipStream_t st, const int32_t *cu,
                          int Ttot, const DtTf &tf)
{
    if (d.P == 64 && d.N == 128) launch_ssu_t<TIn, TS, 64, 128>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
    else if (d.P == 64 && d.N == 16) launch_ssu_t<TIn, TS, 64, 16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
    else if (d.P == 16 && d.N == 128) launch_ssu_t<TIn, TS, 16, 128>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
    else launch_ssu_t<TIn, TS, 16, 16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
}

void launch_state_update(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *inter, void *stream, const int32_t *cu,
                         int Ttot, const DtTf &tf)
{
    if (d.R <= 0 || d.T <= 0) return;
    if (!cu) Ttot = d.R * d.T;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (d.in_bf16) {
        if (d.state_f16) launch_ssu_pn<bf16, f16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
        else if (d.state_bf16) launch_ssu_pn<bf16, bf16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
        else launch_ssu_pn<bf16, float>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
    } else {
        if (d.state_f16) launch_ssu_pn<float, f16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
        else if (d.state_bf16) launch_ssu_pn<float, bf16>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
        else launch_ssu_pn<float, float>(d, cache, idx, x, dt, A, B, C, D, y, inter, st, cu, Ttot, tf);
    }
}

void launch_state_commit(const DecodeDims &d, void *cache, const int32_t *idx, const void *inter,
                         const int32_t *accepted, void *stream, const int32_t *cu, int Ttot)
{
    if (d.R <= 0 || d.T <= 0) return;
    if (!cu) Ttot = d.R * d.T;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t HPN = (int64_t)d.H * d.P * d.N;
    // (a copy: fp16 moves as the 2-byte bf16 instantiation does)
    const bool two = d.state_bf16 || d.state_f16;
    const int VE = two ? 8 : 4;
    dim3 grid((unsigned)((HPN / VE + 255) / 256), d.R);
    if (two)
        hipLaunchKernelGGL(state_commit_kernel<bf16>, grid, dim3(256), 0, st, d.T, HPN, d.num_slots,
                           static_cast<bf16 *>(cache), idx, static_cast<const bf16 *>(inter),
                           accepted, cu, Ttot);
    else
        hipLaunchKernelGGL(state_commit_kernel<float>, grid, dim3(256), 0, st, d.T, HPN, d.num_slots,
                           static_cast<float *>(cache), idx, static_cast<const float *>(inter),
                           accepted, cu, Ttot);
}

// fp32 -> fp16 of n values with the state stores' rounding (element e of
// stream `kind`), 8 values (one Philox call) per thread.
__global__ __launch_bounds__(256) void round_f16_kernel(const float *__restrict__ in,
                                                        f16 *__restrict__ out, int64_t n, SrCtx sr,
                                                        int kind)
{
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (e0 >= n) return;
    const SrKey srk = sr_key_checked(sr);   // (in may hold fewer than 8 bytes)
    if (e0 + 8 <= n && (reinterpret_cast<uintptr_t>(out + e0) & 15u) == 0) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = in[e0 + j];
        put_run<f16, 8>(out + e0, v, srk, (uint64_t)e0, (uint32_t)kind);
        return;
    }
    const uint4 w = sr_words(srk, (uint64_t)e0, (uint32_t)kind);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    for (int j = 0; j < 8 && e0 + j < n; ++j) {
        const uint32_t d = (j & 1) ? sr_hi16(ws[j >> 1]) : sr_lo16(ws[j >> 1]);
        out[e0 + j] = srk.rounds > 0 ? sr_f16(in[e0 + j], d) : static_cast<f16>(in[e0 + j]);
    }
}

void launch_round_f16(const float *in, void *out, int64_t n, const SrCtx &sr, int kind,
                      void *stream)
{
    if (n <= 0) return;
    const int64_t groups = (n + 7) / 8;
    hipLaunchKernelGGL(round_f16_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), in, static_cast<f16 *>(out), n, sr,
                       kind);
}

}  // namespace ssd
