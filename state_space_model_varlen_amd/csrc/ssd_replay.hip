// ReplaySSM MTP decode on MI355X (gfx950): a checkpoint state and a ring of
// the inputs per slot instead of a stored state per draft token (vLLM PR
// #52928 "[Mamba] Add FlashInfer ReplaySSM support for MTP", sections
// "Summary" and "Design"; vLLM PR #55688, "Summary": materialisation of the
// pending history into the checkpoint).
//
// Per slot the ring holds x, dt and B of the n accepted tokens since the
// checkpoint at positions (start + i) mod W. A verify step rebuilds the
// current state from the checkpoint and those tokens, runs the T new tokens
// (writing y), and appends their inputs after the history; it rewrites the
// checkpoint only when the next window might not fit (n + T > W - T). The
// window's positions never overlap the history it reads, so the B ring, which
// the heads of a group share, has no write-after-read race between blocks.
//
// The history is folded without per-token state updates: with S_i the sum of
// dt over the history tokens after token i,
//     state = exp(A S_0') ckpt + sum_i exp(A S_i) dt_i x_i (x) B_i,
// (S_0' the sum over all of them), taken in reverse token order with a
// running suffix sum: one fused multiply-add per state element per token.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_ssu.h"

namespace ssd {

namespace {

__device__ __forceinline__ int clamp_int(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Block (h, r) thread layout shared with the selective state update: chunk
// q = tid + 256 k of 8 state elements covers row q / (N / 8), columns
// 8 (q % (N / 8)) .. + 7.
template <int P, int N> struct ChunkMap {
    static constexpr int CPR = N / 8;            // chunks per state row
    static constexpr int NCH = P * N / 8;        // chunks per (slot, head)
    static constexpr int KC = (NCH + 255) / 256; // chunks per thread
    static_assert(NCH % 256 == 0 || KC == 1, "chunk split");
};

// Folds history tokens n-1 .. 0 of a slot into acc (sum_i exp(A S_i) dt_i
// x_i (x) B_i) and returns S = sum_i dt_i. Tokens are taken TM at a time,
// every load of a group issued before its arithmetic; indices below 0 are
// clamped to a real position and their dt forced to zero (no contribution,
// no branch between a load and its use).
template <typename TIn, int P, int N, int TM>
__device__ __forceinline__ float fold_history(int n, int start, int W, int H, int G, int h, int g,
                                              int64_t cs, float Ah, const TIn *ring_x,
                                              const TIn *ring_dt, const TIn *ring_B,
                                              const int (&pk)[ChunkMap<P, N>::KC], int n0,
                                              float (&acc)[ChunkMap<P, N>::KC][8])
{
    constexpr int KC = ChunkMap<P, N>::KC;
    float S = 0.0f;
    for (int i1 = n - 1; i1 >= 0; i1 -= TM) {
        float dtv[TM], xv[TM][KC];
        Raw8<TIn> braw[TM];
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int i = i1 - j;
            int pos = start + (i > 0 ? i : 0);
            pos = pos < W ? pos : pos - W;
            const int64_t e = cs * W + pos;
            const float d = to_f32(ring_dt[e * H + h]);
            dtv[j] = i >= 0 ? d : 0.0f;
            braw[j].load(ring_B + (e * G + g) * N + n0);
#pragma unroll
            for (int k = 0; k < KC; ++k) xv[j][k] = to_f32(ring_x[(e * H + h) * P + pk[k]]);
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const float w = __expf(Ah * S) * dtv[j];
            S += dtv[j];
            float b8[8];
            braw[j].widen(b8);
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                const float u = w * xv[j][k];
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[k][v] += u * b8[v];
            }
        }
    }
    return S;
}

// Verify step. Block (h, r), 256 threads.
template <typename TIn, typename TS, int P, int N, int TM>
__global__ __launch_bounds__(256) void replay_update_kernel(
    int T, int H, int G, int num_slots, int W, TS *ckpt, TIn *ring_x, TIn *ring_dt, TIn *ring_B,
    const int32_t *__restrict__ cursor, const int32_t *__restrict__ idx, const TIn *__restrict__ x,
    const TIn *__restrict__ dt, const float *__restrict__ A, const TIn *__restrict__ B,
    const TIn *__restrict__ C, const float *__restrict__ D, TIn *__restrict__ y, SrCtx sr)
{
    typedef ChunkMap<P, N> M;
    constexpr int CPR = M::CPR, NCH = M::NCH, KC = M::KC;
    const int h = blockIdx.x, r = blockIdx.y;
    const int tid = threadIdx.x;
    const int g = h / (H / G);
    const int n0 = (tid % CPR) * 8;
    const int L = W - T;                      // history capacity

    const int slot = idx[r];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const int64_t cs = slot_ok ? slot : 0;
    const int start = clamp_int(cursor[2 * cs], 0, W - 1);
    const int n = slot_ok ? clamp_int(cursor[2 * cs + 1], 0, L) : 0;
    const int64_t PN = (int64_t)P * N;
    TS *ck = ckpt + (cs * H + h) * PN;

    int pk[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int q = tid + 256 * k;
        pk[k] = (q < NCH ? q : NCH - 1) / CPR;   // (only when NCH < 256: duplicates, not stored)
    }
    const float Ah = A[h];
    const float Dh = D ? D[h] : 0.0f;
    const SrKey srk = sr_key(sr, ckpt);

    // checkpoint (an invalid slot reads slot 0 and is cleared bit-wise), then the history
    const uint32_t keep = slot_ok ? 0xffffffffu : 0u;
    Raw8<TS> cr[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) cr[k].load(ck + (int64_t)pk[k] * N + n0);
    float st[KC][8];
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
        for (int v = 0; v < 8; ++v) st[k][v] = 0.0f;
    const float S = fold_history<TIn, P, N, 4>(n, start, W, H, G, h, g, cs, Ah, ring_x, ring_dt,
                                               ring_B, pk, n0, st);
    const float a0 = __expf(Ah * S);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        cr[k].mask(keep);
        float s8[8];
        cr[k].widen(s8);
#pragma unroll
        for (int v = 0; v < 8; ++v) st[k][v] += a0 * s8[v];
    }
    // the next window might not fit after this one: the rebuilt state becomes the checkpoint
    if (slot_ok && n + T > L) {
#pragma unroll
        for (int k = 0; k < KC; ++k)
            if (tid + 256 * k < NCH)
                put_run<TS, 8>(ck + (int64_t)pk[k] * N + n0, st[k], srk,
                               (uint64_t)((cs * H + h) * PN + (int64_t)pk[k] * N + n0), kSrReplay);
    }

    // the window: T tokens, TM at a time, y for each; inputs appended to the ring
    const int first_head = (h % (H / G)) == 0;   // one head per group writes the B ring
    float dtv[TM], xv[TM][KC];
    Raw8<TIn> braw[TM], craw[TM], xraw[TM];
    TIn dtraw[TM];
    const int xo = 8 * (tid < P / 8 ? tid : P / 8 - 1);
    auto load_group = [&](int t0) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int t = t0 + j < T ? t0 + j : T - 1;
            const int64_t rt = (int64_t)r * T + t;
            dtraw[j] = dt[rt * H + h];
            dtv[j] = to_f32(dtraw[j]);
            braw[j].load(B + (rt * G + g) * N + n0);
            craw[j].load(C + (rt * G + g) * N + n0);
            xraw[j].load(x + (rt * H + h) * P + xo);
#pragma unroll
            for (int k = 0; k < KC; ++k) xv[j][k] = to_f32(x[(rt * H + h) * P + pk[k]]);
        }
    };
    int t0 = 0;
    do {   // (T >= 1: the launcher enqueues nothing for T = 0)
        load_group(t0);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            if (t0 + j >= T) break;
            const int t = t0 + j;
            const int64_t rt = (int64_t)r * T + t;
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
            }
            if (slot_ok) {
                int pos = start + n + t;
                pos = pos < W ? pos : pos - W;
                const int64_t e = cs * W + pos;
                if (tid < P / 8) xraw[j].store(ring_x + (e * H + h) * P + xo);
                if (tid == 0) ring_dt[e * H + h] = dtraw[j];
                if (first_head && tid < CPR) braw[j].store(ring_B + (e * G + g) * N + n0);
            }
        }
        t0 += TM;
    } while (t0 < T);
}

// Verify step for bf16 inputs and checkpoints, P = 64, N = 128, T <= 4 and
// W <= 16 KT. Taking the history and the window as one run of tokens
// k = 0 .. n + T - 1 (history first) with lambda_k = A sum_{k' <= k} dt_k',
// every output is the dual (quadratic) form of the recurrence over that run:
//   y_t = exp(lambda_{n+t}) (C_t . ckpt) + D x_t
//         + sum_{k <= n+t} exp(lambda_{n+t} - lambda_k) dt_k (C_t . B_k) x_k.
// C . ckpt and C . B are MFMA products (the checkpoint rows are read straight
// from memory as operand fragments); the decay weights and the sums over at
// most 16 KT tokens are a few scalars per lane. No state is built per token:
// the state after the history is formed only when it becomes the checkpoint.
//
// One wave per (head, request), four independent waves per block (heads
// 4 b .. 4 b + 3 of one request). Each wave holds all 64 checkpoint rows as
// MFMA operand fragments (16 KB of loads in flight per wave), and the
// (token, token) work - C_t . B_k, lambda, the decay weights - is done once
// per head. Lane p then forms y_t[p] from coalesced loads of x_k[p] and the
// weights, broadcast from LDS. Only wave-level synchronisation: a wave past
// the last head leaves at once.
template <int KT>
__global__ __launch_bounds__(256) void replay_update_wave_kernel(
    int T, int H, int G, int num_slots, int W, bf16 *ckpt, bf16 *ring_x, bf16 *ring_dt,
    bf16 *ring_B, const int32_t *__restrict__ cursor, const int32_t *__restrict__ idx,
    const bf16 *__restrict__ x, const bf16 *__restrict__ dt, const float *__restrict__ A,
    const bf16 *__restrict__ B, const bf16 *__restrict__ C, const float *__restrict__ D,
    bf16 *__restrict__ y)
{
    constexpr int P = 64, N = 128, NK = 16 * KT;   // token slots: history + window
    __shared__ float s_g[4][4][NK];                // per wave: weights G[t][k]
    __shared__ float s_ys[4][4][P];                // C_t . ckpt, [t][p]
    __shared__ float s_w[4][NK];                   // checkpoint rewrite: token weights
    __shared__ bf16 s_x[4][NK][P];                 // x_k[p]
    __shared__ __attribute__((aligned(16))) bf16 s_b[4][NK][N];   // B_k
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = 4 * blockIdx.x + w, r = blockIdx.y;
    if (h >= H) return;
    const int r16 = lane & 15, kg = lane >> 4;
    const int g = h / (H / G);
    const int L = W - T;

    // ---- loads in two phases (no branch between a load and its use). First the
    // window's C (A fragments, row t = r16; rows past T read as zero), the
    // checkpoint and the cursor, and C_t . ckpt on MFMA straight into LDS; then
    // the token slots' B, dt and x (L2-resident rows). The checkpoint fragments
    // (64 VGPRs) are then never live together with the token rows, which keeps
    // the kernel at four waves per SIMD: 16 KB of checkpoint in flight per wave.
    const rsrc_t rc = make_rsrc(C + ((int64_t)r * T * G + g) * N, (uint32_t)((T - 1) * G * N + N) * 2);
    uint4 cf[4], kf[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) cf[ks] = buf_ld16(rc, (uint32_t)(r16 * G * N + 32 * ks + 8 * kg) * 2);
    const int slot = idx[r];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const int64_t cs = slot_ok ? slot : 0;
    // (an invalid slot reads slot 0's cursor and checkpoint, both discarded)
    const int cur0 = cursor[2 * cs], cur1 = cursor[2 * cs + 1];
    const bf16 *ckh = ckpt + (cs * H + h) * P * N;
#pragma unroll
    for (int pg = 0; pg < 4; ++pg)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            kf[pg][ks] = *reinterpret_cast<const uint4 *>(ckh + (16 * pg + r16) * N + 32 * ks + 8 * kg);
    const float Ah = A[h];
    const float Dh = D ? D[h] : 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    float *sg = &s_g[w][0][0], *sy = &s_ys[w][0][0];
    {
        const uint32_t kslot = slot_ok ? 0xffffffffu : 0u;
#pragma unroll
        for (int pg = 0; pg < 4; ++pg) {
            f32x4 ys = zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint4 kv = kf[pg][ks];
                kv.x &= kslot; kv.y &= kslot; kv.z &= kslot; kv.w &= kslot;
                ys = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cf[ks]),
                                                             __builtin_bit_cast(bf16x8, kv), ys, 0, 0, 0);
            }
            if (kg == 0) {
#pragma unroll
                for (int v = 0; v < 4; ++v) sy[v * P + 16 * pg + r16] = ys[v];
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int start = clamp_int(cur0, 0, W - 1);
    const int n = slot_ok ? clamp_int(cur1, 0, L) : 0;
    const bool ck = slot_ok && n + T > L;
    auto ring_pos = [&](int k) {
        const int q = start + k;
        return q < W ? q : q - W;
    };
    // B and dt of token slot k = 16 kt + r16: ring for k < n, window token k - n
    uint4 bfr[KT][4];
    bf16 dtraw[KT];
    float dtk[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const int k = 16 * kt + r16;
        const bool hist = k < n;
        const int tw = clamp_int(k - n, 0, T - 1);
        const int64_t e = cs * W + ring_pos(hist ? k : 0);
        const bf16 *bsrc = hist ? ring_B + (e * G + g) * N : B + (((int64_t)r * T + tw) * G + g) * N;
        const bf16 *dsrc = hist ? ring_dt + e * H + h : dt + ((int64_t)r * T + tw) * H + h;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            bfr[kt][ks] = *reinterpret_cast<const uint4 *>(bsrc + 32 * ks + 8 * kg);
        dtraw[kt] = *dsrc;
    }
    // x_k[p] for every token slot, lane p (one 128-byte row per slot), and x_t[p]
    // of the window tokens
    bf16 xkr[NK], xtr[4];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const bool hist = k < n;
        const int tw = clamp_int(k - n, 0, T - 1);
        const bf16 *src = hist ? ring_x + ((cs * W + ring_pos(k)) * H + h) * P
                               : x + (((int64_t)r * T + tw) * H + h) * P;
        xkr[k] = src[lane];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int tl = t < T ? t : T - 1;
        xtr[t] = x[(((int64_t)r * T + tl) * H + h) * P + lane];
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- masks, then the MFMA products (C_t . B_k)[t][k]
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const int k = 16 * kt + r16;
        const uint32_t live = k < n + T ? 0xffffffffu : 0u;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bfr[kt][ks].x &= live; bfr[kt][ks].y &= live; bfr[kt][ks].z &= live; bfr[kt][ks].w &= live;
        }
        dtk[kt] = k < n + T ? to_f32(dtraw[kt]) : 0.0f;
    }
    f32x4 cb[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        cb[kt] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            cb[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cf[ks]),
                                                             __builtin_bit_cast(bf16x8, bfr[kt][ks]),
                                                             cb[kt], 0, 0, 0);
    }

    // ---- lambda_k = A sum_{k' <= k} dt_k', summed in token order; lane r16
    // keeps lambda of slot 16 kt + r16 (dt of slot 16 kt + j sits in lane j)
    float lk[KT];
    {
        float run = 0.0f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            float mine = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                run += Ah * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dtk[kt]), j));
                mine = r16 == j ? run : mine;
            }
            lk[kt] = mine;
        }
    }
    // lambda of token slot m (m uniform, m < NK)
    auto lam_at = [&](int m) {
        const float v = KT > 1 && (m >> 4) ? lk[KT > 1 ? 1 : 0] : lk[0];
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), m & 15));
    };
    float lt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) lt[t] = lam_at(n + (t < T ? t : T - 1));

    // ---- weights G[t][k] = [k <= n + t] exp(lambda_{n+t} - lambda_k) dt_k CB[t][k]
    // (lanes of row 0 hold rows t = v of CB) and C_t . ckpt to LDS as [t][p]
    if (kg == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int k = 16 * kt + r16;
                const float gv = __expf(lt[v] - lk[kt]) * dtk[kt] * cb[kt][v];
                sg[v * NK + k] = (v < T && k <= n + v) ? gv : 0.0f;
            }
        }
    }
    wave_lds_sync();

    // ---- y_t[p], lane p
    float xk[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) xk[k] = k < n + T ? to_f32(xkr[k]) : 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (t >= T) break;
        float acc = __expf(lt[t]) * sy[t * P + lane];
#pragma unroll
        for (int k = 0; k < NK; ++k) acc += sg[t * NK + k] * xk[k];
        acc += Dh * to_f32(xtr[t]);
        y[(((int64_t)r * T + t) * H + h) * P + lane] = from_f32<bf16>(acc);
    }

    // ---- the window's inputs join the ring (B by the group's first head)
    if (slot_ok) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < T) ring_x[((cs * W + ring_pos(n + t)) * H + h) * P + lane] = xtr[t];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const int k = 16 * kt + r16;
            if (k >= n && k < n + T) {
                const int64_t e = cs * W + ring_pos(k);
                if (kg == 0) ring_dt[e * H + h] = dtraw[kt];
                if (h % (H / G) == 0) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        *reinterpret_cast<uint4 *>(ring_B + (e * G + g) * N + 32 * ks + 8 * kg) =
                            bfr[kt][ks];
                }
            }
        }
    }

    // ---- checkpoint rewrite: the state after the history,
    //   exp(lambda_{n-1}) ckpt + sum_{i<n} exp(lambda_{n-1} - lambda_i) dt_i x_i (x) B_i,
    // one 16-row group at a time (lane (r16, kg): row 16 pg + r16, columns
    // 32 ks + 8 kg .. + 7, the layout the checkpoint was loaded in). The rows
    // are read again here (this wave's own, still in L2) rather than kept in
    // registers from the MFMA phase: that frees 64 VGPRs for all the other
    // steps, three waves per SIMD instead of two.
    if (ck) {
        const float lh = n > 0 ? lam_at(n - 1) : 0.0f;
        bf16 (*sb)[N] = s_b[w];
        bf16 (*sx)[P] = s_x[w];
        float *sw = s_w[w];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const int k = 16 * kt + r16;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                *reinterpret_cast<uint4 *>(&sb[k][32 * ks + 8 * kg]) = bfr[kt][ks];
            if (kg == 0) sw[k] = k < n ? __expf(lh - lk[kt]) * dtk[kt] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < NK; ++k) sx[k][lane] = xkr[k];
        wave_lds_sync();
        const float a0 = __expf(lh);
        bf16 *ckw = ckpt + (cs * H + h) * P * N;
#pragma unroll
        for (int pg = 0; pg < 4; ++pg) {
            const int p = 16 * pg + r16;
            float st[4][8];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Raw8<bf16> kr;
                kr.w = *reinterpret_cast<const uint4 *>(ckw + p * N + 32 * ks + 8 * kg);
                kr.widen(st[ks]);
#pragma unroll
                for (int v = 0; v < 8; ++v) st[ks][v] *= a0;
            }
            for (int i = 0; i < n; ++i) {
                const float u = sw[i] * to_f32(sx[i][p]);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    Raw8<bf16> br;
                    br.w = *reinterpret_cast<const uint4 *>(&sb[i][32 * ks + 8 * kg]);
                    float b8[8];
                    br.widen(b8);
#pragma unroll
                    for (int v = 0; v < 8; ++v) st[ks][v] += u * b8[v];
                }
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) store_run<bf16, 8>(ckw + p * N + 32 * ks + 8 * kg, st[ks]);
        }
    }
}

// Materialise: ckpt[s] = checkpoint followed by the history. Block (h, r).
template <typename TIn, typename TS, int P, int N>
__global__ __launch_bounds__(256) void replay_materialize_kernel(
    int L, int H, int G, int num_slots, int W, TS *ckpt, const TIn *__restrict__ ring_x,
    const TIn *__restrict__ ring_dt, const TIn *__restrict__ ring_B,
    const int32_t *__restrict__ cursor, const int32_t *__restrict__ idx,
    const float *__restrict__ A, SrCtx sr)
{
    typedef ChunkMap<P, N> M;
    constexpr int CPR = M::CPR, NCH = M::NCH, KC = M::KC;
    const int h = blockIdx.x, r = blockIdx.y;
    const int tid = threadIdx.x;
    const int slot = idx[r];
    if (slot < 0 || slot >= num_slots) return;
    const int g = h / (H / G);
    const int n0 = (tid % CPR) * 8;
    const int64_t cs = slot;
    const int start = clamp_int(cursor[2 * cs], 0, W - 1);
    const int n = clamp_int(cursor[2 * cs + 1], 0, L);
    const int64_t PN = (int64_t)P * N;
    TS *ck = ckpt + (cs * H + h) * PN;
    int pk[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int q = tid + 256 * k;
        pk[k] = (q < NCH ? q : NCH - 1) / CPR;
    }
    const float Ah = A[h];
    const SrKey srk = sr_key(sr, ckpt);
    Raw8<TS> cr[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) cr[k].load(ck + (int64_t)pk[k] * N + n0);
    float st[KC][8];
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
        for (int v = 0; v < 8; ++v) st[k][v] = 0.0f;
    const float S = fold_history<TIn, P, N, 4>(n, start, W, H, G, h, g, cs, Ah, ring_x, ring_dt,
                                               ring_B, pk, n0, st);
    const float a0 = __expf(Ah * S);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        float s8[8];
        cr[k].widen(s8);
#pragma unroll
        for (int v = 0; v < 8; ++v) st[k][v] += a0 * s8[v];
        if (tid + 256 * k < NCH)
            put_run<TS, 8>(ck + (int64_t)pk[k] * N + n0, st[k], srk,
                           (uint64_t)((cs * H + h) * PN + (int64_t)pk[k] * N + n0), kSrReplay);
    }
}

// Cursor moves, one thread per request. mode 0: advance after a verify step
// with window T and accepted[r] drafts; mode 1: history folded (materialised).
__global__ __launch_bounds__(256) void replay_cursor_kernel(int R, int T, int W, int num_slots,
                                                            int mode, int32_t *cursor,
                                                            const int32_t *__restrict__ idx,
                                                            const int32_t *__restrict__ accepted)
{
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= R) return;
    const int slot = idx[r];
    if (slot < 0 || slot >= num_slots) return;
    const int L = W - T;
    int start = clamp_int(cursor[2 * slot], 0, W - 1);
    int n = clamp_int(cursor[2 * slot + 1], 0, L);
    if (mode == 0) {
        const int a = clamp_int(accepted[r], 0, T - 1);
        if (n + T > L) {           // that verify step rewrote the checkpoint
            start = (start + n) % W;
            n = 1 + a;
        } else {
            n += 1 + a;
        }
    } else {
        start = (start + n) % W;
        n = 0;
    }
    cursor[2 * slot] = start;
    cursor[2 * slot + 1] = n;
}

template <typename TIn, typename TS, int P, int N>
void launch_update_t(const DecodeDims &d, int W, void *ckpt, void *rx, void *rdt, void *rB,
                     const int32_t *cursor, const int32_t *idx, const void *x, const void *dt,
                     const float *A, const void *B, const void *C, const float *D, void *y,
                     hipStream_t st)
{
    dim3 grid(d.H, d.R);
#define SSD_REPLAY_LAUNCH(TM)                                                                     \
    hipLaunchKernelGGL((replay_update_kernel<TIn, TS, P, N, TM>), grid, dim3(256), 0, st, d.T,    \
                       d.H, d.G, d.num_slots, W, static_cast<TS *>(ckpt), static_cast<TIn *>(rx), \
                       static_cast<TIn *>(rdt), static_cast<TIn *>(rB), cursor, idx,              \
                       static_cast<const TIn *>(x), static_cast<const TIn *>(dt), A,              \
                       static_cast<const TIn *>(B), static_cast<const TIn *>(C), D,               \
                       static_cast<TIn *>(y), d.sr)
    if (d.T <= 1) SSD_REPLAY_LAUNCH(1);
    else if (d.T <= 2) SSD_REPLAY_LAUNCH(2);
    else if (d.T <= 3) SSD_REPLAY_LAUNCH(3);
    else SSD_REPLAY_LAUNCH(4);
#undef SSD_REPLAY_LAUNCH
}

template <typename TIn, typename TS, int P, int N>
void launch_materialize_t(const DecodeDims &d, int W, void *ckpt, const void *rx, const void *rdt,
                          const void *rB, const int32_t *cursor, const int32_t *idx,
                          const float *A, hipStream_t st)
{
    hipLaunchKernelGGL((replay_materialize_kernel<TIn, TS, P, N>), dim3(d.H, d.R), dim3(256), 0,
                       st, W - d.T, d.H, d.G, d.num_slots, W, static_cast<TS *>(ckpt),
                       static_cast<const TIn *>(rx), static_cast<const TIn *>(rdt),
                       static_cast<const TIn *>(rB), cursor, idx, A, d.sr);
}

// dispatch on (in dtype, state dtype, P, N) for the shapes the GPU path supports
template <template <typename, typename, int, int> class Op, typename... Args>
void dispatch(const DecodeDims &d, Args &&...args)
{
    auto pn = [&](auto tin, auto ts) {
        typedef decltype(tin) TIn;
        typedef decltype(ts) TS;
        if (d.P == 64 && d.N == 128) Op<TIn, TS, 64, 128>::run(d, args...);
        else if (d.P == 64 && d.N == 16) Op<TIn, TS, 64, 16>::run(d, args...);
        else if (d.P == 16 && d.N == 128) Op<TIn, TS, 16, 128>::run(d, args...);
        else Op<TIn, TS, 16, 16>::run(d, args...);
    };
    if (d.in_bf16) {
        if (d.state_f16) pn(bf16(), f16());
        else if (d.state_bf16) pn(bf16(), bf16());
        else pn(bf16(), float());
    } else {
        if (d.state_f16) pn(float(), f16());
        else if (d.state_bf16) pn(float(), bf16());
        else pn(float(), float());
    }
}

template <typename TIn, typename TS, int P, int N> struct UpdateOp {
    template <typename... A> static void run(const DecodeDims &d, A... a) { launch_update_t<TIn, TS, P, N>(d, a...); }
};
template <typename TIn, typename TS, int P, int N> struct MaterializeOp {
    template <typename... A> static void run(const DecodeDims &d, A... a) { launch_materialize_t<TIn, TS, P, N>(d, a...); }
};

}  // namespace

void launch_replay_update(const DecodeDims &d, int W, void *ckpt, void *rx, void *rdt, void *rB,
                          const int32_t *cursor, const int32_t *idx, const void *x, const void *dt,
                          const float *A, const void *B, const void *C, const float *D, void *y,
                          void *stream)
{
    if (d.R <= 0 || d.T <= 0) return;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (d.in_bf16 && d.state_bf16 && d.P == 64 && d.N == 128 && d.T <= 4 && W <= 32) {
#define SSD_REPLAY_FAST(KT)                                                                       \
    hipLaunchKernelGGL((replay_update_wave_kernel<KT>), dim3((d.H + 3) / 4, d.R), dim3(256), 0, st, \
                       d.T,                                                                       \
                       d.H, d.G, d.num_slots, W, static_cast<bf16 *>(ckpt), static_cast<bf16 *>(rx), \
                       static_cast<bf16 *>(rdt), static_cast<bf16 *>(rB), cursor, idx,            \
                       static_cast<const bf16 *>(x), static_cast<const bf16 *>(dt), A,            \
                       static_cast<const bf16 *>(B), static_cast<const bf16 *>(C), D,             \
                       static_cast<bf16 *>(y))
        if (W <= 16) SSD_REPLAY_FAST(1);
        else SSD_REPLAY_FAST(2);
#undef SSD_REPLAY_FAST
        return;
    }
    dispatch<UpdateOp>(d, W, ckpt, rx, rdt, rB, cursor, idx, x, dt, A, B, C, D, y, st);
}

void launch_replay_advance(const DecodeDims &d, int W, int32_t *cursor, const int32_t *idx,
                           const int32_t *accepted, void *stream)
{
    if (d.R <= 0 || d.T <= 0) return;
    hipLaunchKernelGGL(replay_cursor_kernel, dim3((d.R + 255) / 256), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), d.R, d.T, W, d.num_slots, 0, cursor,
                       idx, accepted);
}

void launch_replay_materialize(const DecodeDims &d, int W, void *ckpt, const void *rx,
                               const void *rdt, const void *rB, int32_t *cursor,
                               const int32_t *idx, const float *A, void *stream)
{
    if (d.R <= 0) return;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    dispatch<MaterializeOp>(d, W, ckpt, rx, rdt, rB, static_cast<const int32_t *>(cursor), idx, A,
                            st);
    hipLaunchKernelGGL(replay_cursor_kernel, dim3((d.R + 255) / 256), dim3(256), 0, st, d.R, d.T,
                       W, d.num_slots, 1, cursor, idx, static_cast<const int32_t *>(nullptr));
}

}  // namespace ssd
