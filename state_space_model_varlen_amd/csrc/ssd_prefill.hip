// Mamba2 SSD chunked varlen prefill on MI355X (gfx950): the five steps of the
// chunked scan - chunk cumsum, chunk state, state passing, bmm, chunk scan -
// as split in vLLM PR #61501 (section "Details"), with the initial state read
// from the cache slot inside state passing and each chunk's entering state
// kept in the workspace for chunk scan (vLLM PR #62922, section "Details").
//
// Notation: chunk c = (seq, start, len) from the metadata, head h, group
// g = h / (H / G), local token index i in [0, len), cum = inclusive cumsum of
// dt * A_h inside the chunk.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ===========================================================================
// Step 1: chunk metadata + chunk cumsum.
// Grid (max_chunks, ceil(H / kCumsumHeads)), 256 threads. Every block finds
// its own chunk from cu_seqlens with a block-wide scan of per-sequence chunk
// counts (no host sync, no extra launch); blocks with blockIdx.y == 0 publish
// the metadata. Each wave then runs a wavefront prefix sum of dt * A over the
// chunk for its heads.
constexpr int kCumsumHeads = 16;

__device__ __forceinline__ int wave_inclusive_sum_int(int v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <typename TIn>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(
    int T, int S, int H, int Q, int max_chunks, const TIn *__restrict__ dt,
    const float *__restrict__ A, const int32_t *__restrict__ cu, int32_t *__restrict__ meta,
    float *__restrict__ cum_out, float *__restrict__ dt_out)
{
    __shared__ int s_wave_tot[4];
    __shared__ int s_found[2];
    __shared__ float s_dt[256][kCumsumHeads + 1];

    const int c = blockIdx.x;
    const int hb = blockIdx.y * kCumsumHeads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool publish = blockIdx.y == 0;
    const bool publish_cu = publish && blockIdx.x == 0;

    if (tid == 0) {
        s_found[0] = -1;
        s_found[1] = 0;
    }
    int running = 0;
    for (int base = 0; base < S; base += 256) {
        __syncthreads();
        const int s = base + tid;
        int cnt = 0;
        if (s < S) {
            const int a = clampi(cu[s], 0, T), b = clampi(cu[s + 1], 0, T);
            const int L = b > a ? b - a : 0;
            cnt = (L + Q - 1) / Q;
        }
        int incl = wave_inclusive_sum_int(cnt, lane);
        if (lane == 63) s_wave_tot[wave] = incl;
        __syncthreads();
        int wave_off = 0, tile_tot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wave_off += (w < wave) ? s_wave_tot[w] : 0;
            tile_tot += s_wave_tot[w];
        }
        const int first = running + wave_off + incl - cnt;  // chunk_cu[s]
        if (s < S) {
            if (publish_cu) meta[s] = first < max_chunks ? first : max_chunks;
            if (cnt > 0 && c >= first && c < first + cnt) {
                s_found[0] = s;
                s_found[1] = c - first;
            }
        }
        running += tile_tot;
    }
    if (publish_cu && tid == 0) meta[S] = running < max_chunks ? running : max_chunks;
    __syncthreads();

    const int seq = s_found[0];
    int start = 0, len = 0;
    if (seq >= 0) {
        const int a = clampi(cu[seq], 0, T), b = clampi(cu[seq + 1], 0, T);
        start = a + s_found[1] * Q;
        len = b - start < Q ? b - start : Q;
    }
    if (publish && tid == 0) {
        int32_t *m = meta + (S + 1) + 3 * c;
        m[0] = seq;
        m[1] = start;
        m[2] = len;
    }
    if (len <= 0) return;

    const int nh = H - hb < kCumsumHeads ? H - hb : kCumsumHeads;
    for (int idx = tid; idx < Q * kCumsumHeads; idx += 256) {
        const int i = idx / kCumsumHeads, hh = idx % kCumsumHeads;
        float v = 0.0f;
        if (i < len && hh < nh) v = to_f32(dt[(int64_t)(start + i) * H + hb + hh]);
        s_dt[i][hh] = v;
    }
    __syncthreads();

    const int E = (Q + kWave - 1) / kWave;  // positions per lane (<= 4)
    for (int hh = wave; hh < nh; hh += 4) {
        const int h = hb + hh;
        const float Ah = A[h];
        float vals[4], loc[4], run = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = lane * E + e;
            const float d = (e < E && i < Q) ? s_dt[i][hh] : 0.0f;
            vals[e] = d;
            run += d * Ah;
            loc[e] = run;
        }
        const float incl = wave_inclusive_sum(run, lane);
        const float off = incl - run;
        const int64_t row = ((int64_t)h * max_chunks + c) * Q;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = lane * E + e;
            if (e < E && i < Q) {
                cum_out[row + i] = off + loc[e];
                dt_out[row + i] = vals[e];
            }
        }
    }
}

// ===========================================================================
// Transposed LDS staging: copy rows [0, nvalid) of a row-major [rows x W]
// source tile (row stride ld_src elements) into LDS as dst[w][t] (row length
// ldt), scaling source row t by wt[t] when SCALE, zero-filling rows
// [nvalid, rows). Each thread moves VE x VE blocks (VE = elements per 16-byte
// vector): VE vector loads, a register transpose, VE vector LDS stores - so
// both sides move 16 bytes per lane and MFMA operand reads along t are
// contiguous.
template <typename TIn, int W, bool SCALE>
__device__ __forceinline__ void stage_transposed(TIn *dst, int ldt, const TIn *src, int64_t ld_src,
                                                 int nvalid, int rows, const float *wt, int tid,
                                                 int nthreads)
{
    constexpr int VE = Vec16<TIn>::kElems;
    constexpr int CB = W / VE;
    const int units = (rows / VE) * CB;
    for (int u = tid; u < units; u += nthreads) {
        const int tb = u / CB, cb = u % CB;
        float v[VE][VE];
#pragma unroll
        for (int r = 0; r < VE; ++r) {
            const int t = tb * VE + r;
            if (t < nvalid) {
                Vec16<TIn>::load(src + (int64_t)t * ld_src + cb * VE, v[r]);
                if (SCALE) {
                    const float s = wt[t];
#pragma unroll
                    for (int e = 0; e < VE; ++e) v[r][e] *= s;
                }
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) v[r][e] = 0.0f;
            }
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            float col[VE];
#pragma unroll
            for (int r = 0; r < VE; ++r) col[r] = v[r][e];
            Vec16<TIn>::store(dst + (cb * VE + e) * ldt + tb * VE, col);
        }
    }
}

// Padded LDS row length (elements) for a row of `len` elements: keeps rows
// 16-byte aligned and pads each by 16 bytes so that the 16 rows an MFMA
// operand read touches start in different LDS banks.
template <typename TIn> __host__ __device__ constexpr int padded(int len) {
    return len + 16 / (int)sizeof(TIn);
}

// ===========================================================================
// Step 2: chunk state. Grid (H, max_chunks), 256 threads (4 waves).
// S_c = (w * x)^T [P x len] . B [len x N] on MFMA, w_t = exp(cum_last - cum_t) dt_t,
// with x and B staged transposed through LDS in slabs of 64 tokens.
constexpr int kStateSlab = 64;

template <typename TIn, int P, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(
    int S, int H, int G, int Q, int max_chunks, const TIn *__restrict__ x,
    const TIn *__restrict__ B, const int32_t *__restrict__ meta, const float *__restrict__ cum,
    const float *__restrict__ dtc, float *__restrict__ states)
{
    typedef Mma<TIn> M;
    constexpr int LD = padded<TIn>(kStateSlab);
    constexpr int RT = P / 16, CT = N / 16;
    constexpr int RPW = (RT + 3) / 4;  // row tiles per wave
    __shared__ __attribute__((aligned(16))) TIn xs[P * LD];
    __shared__ __attribute__((aligned(16))) TIn bs[N * LD];
    __shared__ float ws[kStateSlab];

    const int h = blockIdx.x, c = blockIdx.y;
    const ChunkInfo ci = chunk_info(meta, S, c);
    if (ci.len <= 0) return;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;

    const float *cumrow = cum + ((int64_t)h * max_chunks + c) * Q;
    const float *dtrow = dtc + ((int64_t)h * max_chunks + c) * Q;
    const float cum_last = cumrow[ci.len - 1];
    const TIn *xsrc = x + ((int64_t)ci.start * H + h) * P;
    const TIn *bsrc = B + ((int64_t)ci.start * G + g) * N;

    f32x4 acc[RPW][CT];
#pragma unroll
    for (int a = 0; a < RPW; ++a)
#pragma unroll
        for (int b = 0; b < CT; ++b) acc[a][b] = zero4();

    for (int t0 = 0; t0 < ci.len; t0 += kStateSlab) {
        const int nvalid = ci.len - t0 < kStateSlab ? ci.len - t0 : kStateSlab;
        __syncthreads();
        if (tid < kStateSlab)
            ws[tid] = tid < nvalid ? __expf(cum_last - cumrow[t0 + tid]) * dtrow[t0 + tid] : 0.0f;
        __syncthreads();
        stage_transposed<TIn, P, true>(xs, LD, xsrc + (int64_t)t0 * H * P, (int64_t)H * P, nvalid,
                                       kStateSlab, ws, tid, 256);
        stage_transposed<TIn, N, false>(bs, LD, bsrc + (int64_t)t0 * G * N, (int64_t)G * N, nvalid,
                                        kStateSlab, nullptr, tid, 256);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kStateSlab / M::K; ++kk) {
            const int k = kk * M::K + kg * M::KPL;
#pragma unroll
            for (int a = 0; a < RPW; ++a) {
                const int rt = wave + 4 * a;
                if (rt < RT) {
                    const typename M::frag af = M::load(&xs[(rt * 16 + r16) * LD + k]);
#pragma unroll
                    for (int b = 0; b < CT; ++b) {
                        const typename M::frag bf = M::load(&bs[(b * 16 + r16) * LD + k]);
                        acc[a][b] = M::run(af, bf, acc[a][b]);
                    }
                }
            }
        }
    }

    float *out = states + ((int64_t)c * H + h) * P * N;
#pragma unroll
    for (int a = 0; a < RPW; ++a) {
        const int rt = wave + 4 * a;
        if (rt < RT) {
#pragma unroll
            for (int b = 0; b < CT; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    out[(rt * 16 + kg * 4 + v) * N + b * 16 + r16] = acc[a][b][v];
        }
    }
}

// ===========================================================================
// Step 3: state passing. Grid (S * H * EB), 256 threads, 4 consecutive state
// elements per thread (EB = ceil(P*N / 1024) blocks per (sequence, head)).
// Sequential over the sequence's chunks; bandwidth-bound.
template <typename TS>
__device__ __forceinline__ void load4(const TS *p, float *v);
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
template <typename TS>
__device__ __forceinline__ void store4(TS *p, const float *v);
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

template <typename TS>
__global__ __launch_bounds__(256) void state_passing_kernel(
    int S, int H, int PN, int Q, int max_chunks, int num_slots, const float *states,
    const float *__restrict__ cum, const int32_t *__restrict__ meta, TS *cache,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ has_init, float *entering,
    TS *__restrict__ ckpt)
{
    const int EB = (PN + 1023) / 1024;
    const int b = blockIdx.x;
    const int eb = b % EB;
    const int h = (b / EB) % H;
    const int s = b / (EB * H);
    const int e = (eb * 256 + threadIdx.x) * 4;
    if (s >= S || e >= PN) return;

    const int slot = idx[s];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const bool read_init = slot_ok && (has_init != nullptr && has_init[s] != 0);
    TS *cslot = cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN + e;

    float hs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (read_init) load4<TS>(cslot, hs);

    int c0 = meta[s], c1 = meta[s + 1];
    c0 = c0 < max_chunks ? c0 : max_chunks;
    c1 = c1 < max_chunks ? c1 : max_chunks;
    for (int c = c0; c < c1; ++c) {
        const int len = meta[(S + 1) + 3 * c + 2];
        const float decay = len > 0 ? __expf(cum[((int64_t)h * max_chunks + c) * Q + len - 1]) : 1.0f;
        const int64_t off = ((int64_t)c * H + h) * PN + e;
        float sc[4];
        load4<float>(states + off, sc);
        float nh[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) nh[k] = decay * hs[k] + sc[k];
        // the chunk state at `off` is consumed above before the entering state
        // (possibly the same buffer) overwrites it
        store4<float>(entering + off, hs);
        if (ckpt) store4<TS>(ckpt + off, nh);
#pragma unroll
        for (int k = 0; k < 4; ++k) hs[k] = nh[k];
    }
    if (slot_ok) store4<TS>(cslot, hs);
}

// ===========================================================================
// Step 4: bmm. Grid (max_chunks, G, ceil(Q / 64)), 256 threads. Wave w computes
// CB rows [64 z + 16 w, +16) against every 16-column tile at or left of the
// diagonal: C rows (A operand) and B rows (B operand) load straight from HBM
// because d_state is the contiguous index of both.
template <typename TIn, int N>
__global__ __launch_bounds__(256) void bmm_kernel(int S, int G, int Q, int max_chunks,
                                                  const TIn *__restrict__ B,
                                                  const TIn *__restrict__ C,
                                                  const int32_t *__restrict__ meta,
                                                  float *__restrict__ CB)
{
    typedef Mma<TIn> M;
    constexpr int NK = (N + M::K - 1) / M::K;
    const int c = blockIdx.x, g = blockIdx.y;
    const ChunkInfo ci = chunk_info(meta, S, c);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int i0 = blockIdx.z * 64 + wave * 16;
    if (ci.len <= 0 || i0 >= ci.len) return;

    typename M::frag af[NK];
    const int i = i0 + r16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n = kk * M::K + kg * M::KPL;
        af[kk] = (i < ci.len && n < N) ? M::load(C + ((int64_t)(ci.start + i) * G + g) * N + n)
                                       : M::zero();
    }
    float *out = CB + ((int64_t)c * G + g) * Q * Q;
    for (int jt = 0; jt <= i0 / 16; ++jt) {
        const int j = jt * 16 + r16;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n = kk * M::K + kg * M::KPL;
            const typename M::frag bf = (j < ci.len && n < N)
                ? M::load(B + ((int64_t)(ci.start + j) * G + g) * N + n) : M::zero();
            acc = M::run(af[kk], bf, acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) out[(int64_t)(i0 + kg * 4 + v) * Q + jt * 16 + r16] = acc[v];
    }
}

// ===========================================================================
// Step 5: chunk scan. Grid (H, max_chunks), 256 threads (4 waves). x of the
// whole chunk is staged transposed in LDS (MFMA B operand for the intra-chunk
// product), the entering state as bf16/f32 [P][N] in LDS (B operand of the
// state term). Wave w handles the 16-row tiles r with r mod 8 in {w, 7 - w}
// so that the causal work is balanced. Per row tile:
//   acc  = sum_j (CB[i,j] exp(cum_i - cum_j) dt_j [j <= i]) x_j      (MFMA)
//   acc += (exp(cum_i) C_i) . H_in^T                                  (MFMA)
//   y_i  = acc + D_h x_i
template <typename TIn, int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    int S, int H, int G, int Q, int max_chunks, const TIn *__restrict__ x,
    const TIn *__restrict__ C, const float *__restrict__ D, const int32_t *__restrict__ meta,
    const float *__restrict__ cum, const float *__restrict__ dtc, const float *__restrict__ CB,
    const float *__restrict__ entering, TIn *__restrict__ y)
{
    typedef Mma<TIn> M;
    constexpr int KPL = M::KPL, KS = M::K;
    constexpr int PT = P / 16;
    constexpr int LDH = padded<TIn>(N);
    constexpr int NK = (N + KS - 1) / KS;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int LDX = padded<TIn>(Q);
    TIn *xs = reinterpret_cast<TIn *>(smem);                  // [P][LDX]
    TIn *hsm = xs + P * LDX;                                   // [P][LDH]
    float *scum = reinterpret_cast<float *>(hsm + P * LDH);    // [Q]
    float *sdt = scum + Q;                                     // [Q]

    const int h = blockIdx.x, c = blockIdx.y;
    const ChunkInfo ci = chunk_info(meta, S, c);
    if (ci.len <= 0) return;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int len = ci.len;

    const float *cumrow = cum + ((int64_t)h * max_chunks + c) * Q;
    const float *dtrow = dtc + ((int64_t)h * max_chunks + c) * Q;
    for (int i = tid; i < Q; i += 256) {
        scum[i] = cumrow[i];
        sdt[i] = dtrow[i];
    }
    stage_transposed<TIn, P, false>(xs, LDX, x + ((int64_t)ci.start * H + h) * P, (int64_t)H * P,
                                    len, (Q + 7) / 8 * 8, nullptr, tid, 256);
    {
        const float *hin = entering + ((int64_t)c * H + h) * P * N;
        for (int e = tid * 4; e < P * N; e += 256 * 4) {
            float v[4];
            load4<float>(hin + e, v);
            const int p = e / N, n = e % N;
#pragma unroll
            for (int k = 0; k < 4; ++k) hsm[p * LDH + n + k] = from_f32<TIn>(v[k]);
        }
    }
    __syncthreads();

    const float Dh = D ? D[h] : 0.0f;
    const TIn *Cbase = C + ((int64_t)ci.start * G + g) * N;
    const float *CBc = CB + ((int64_t)c * G + g) * Q * Q;
    const int ntiles = (len + 15) / 16;

    for (int rr = 0; rr < (Q / 16 + 7) / 8 * 2; ++rr) {
        // wave w: tiles 8q + w and 8q + 7 - w for q = 0, 1, ...
        const int q8 = rr >> 1;
        const int rt = 8 * q8 + ((rr & 1) ? 7 - wave : wave);
        if (rt >= ntiles) continue;
        const int i0 = rt * 16;
        const int i = i0 + r16;              // A-operand row of this lane
        const float cum_i = scum[i < Q ? i : Q - 1];

        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = zero4();

        // intra-chunk: K over j = 0 .. i0 + 15
        for (int j0 = 0; j0 <= i0 + 15; j0 += KS) {
            const int jb = j0 + kg * KPL;
            typename M::frag af;
            float cbv[KPL];
            if constexpr (KPL == 8) {
                const float4 q0 = *reinterpret_cast<const float4 *>(CBc + (int64_t)i * Q + jb);
                const float4 q1 = *reinterpret_cast<const float4 *>(CBc + (int64_t)i * Q + jb + 4);
                cbv[0] = q0.x; cbv[1] = q0.y; cbv[2] = q0.z; cbv[3] = q0.w;
                cbv[4] = q1.x; cbv[5] = q1.y; cbv[6] = q1.z; cbv[7] = q1.w;
            } else {
#pragma unroll
                for (int v = 0; v < KPL; ++v) cbv[v] = CBc[(int64_t)i * Q + jb + v];
            }
#pragma unroll
            for (int v = 0; v < KPL; ++v) {
                const int j = jb + v;
                const float m = (j <= i) ? cbv[v] * __expf(cum_i - scum[j]) * sdt[j] : 0.0f;
                M::set(af, v, m);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const typename M::frag bf = M::load(&xs[(pt * 16 + r16) * LDX + jb]);
                acc[pt] = M::run(af, bf, acc[pt]);
            }
        }
        // state term: (exp(cum_i) C_i) . H_in^T
        {
            const float ei = __expf(cum_i);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n = kk * KS + kg * KPL;
                typename M::frag af = M::zero();
                if (i < len && n < N) {
                    float cv[Vec16<TIn>::kElems > KPL ? Vec16<TIn>::kElems : KPL];
                    if constexpr (KPL == 8) {
                        Vec16<TIn>::load(Cbase + (int64_t)i * G * N + n, cv);
                    } else {
#pragma unroll
                        for (int v = 0; v < KPL; ++v) cv[v] = to_f32(Cbase[(int64_t)i * G * N + n + v]);
                    }
#pragma unroll
                    for (int v = 0; v < KPL; ++v) M::set(af, v, ei * cv[v]);
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const typename M::frag bf = (n < N) ? M::load(&hsm[(pt * 16 + r16) * LDH + n])
                                                        : M::zero();
                    acc[pt] = M::run(af, bf, acc[pt]);
                }
            }
        }
        // epilogue: + D x, store
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int p = pt * 16 + r16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int io = i0 + kg * 4 + v;
                if (io < len) {
                    const float xv = to_f32(xs[p * LDX + io]);
                    y[((int64_t)(ci.start + io) * H + h) * P + p] = from_f32<TIn>(acc[pt][v] + Dh * xv);
                }
            }
        }
    }
}

// ===========================================================================
// Launchers.
static inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

template <typename TIn>
static void launch_cumsum_t(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                            int32_t *meta, float *cum, float *dto, hipStream_t st)
{
    dim3 grid(d.max_chunks, (d.H + kCumsumHeads - 1) / kCumsumHeads);
    hipLaunchKernelGGL(chunk_cumsum_kernel<TIn>, grid, dim3(256), 0, st, d.T, d.S, d.H, d.Q,
                       d.max_chunks, static_cast<const TIn *>(dt), A, cu, meta, cum, dto);
}

void launch_chunk_cumsum(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                         int32_t *meta, float *cum, float *dto, void *stream)
{
    if (d.max_chunks <= 0) return;
    if (d.in_bf16) launch_cumsum_t<bf16>(d, dt, A, cu, meta, cum, dto, as_stream(stream));
    else launch_cumsum_t<float>(d, dt, A, cu, meta, cum, dto, as_stream(stream));
}

template <typename TIn, int P, int N>
static void launch_state_t(const PrefillDims &d, const void *x, const void *B, const int32_t *meta,
                           const float *cum, const float *dtc, float *states, hipStream_t st)
{
    dim3 grid(d.H, d.max_chunks);
    hipLaunchKernelGGL((chunk_state_kernel<TIn, P, N>), grid, dim3(256), 0, st, d.S, d.H, d.G, d.Q,
                       d.max_chunks, static_cast<const TIn *>(x), static_cast<const TIn *>(B),
                       meta, cum, dtc, states);
}

template <typename TIn, int N>
static void launch_bmm_t(const PrefillDims &d, const void *B, const void *C, const int32_t *meta,
                         float *CB, hipStream_t st)
{
    dim3 grid(d.max_chunks, d.G, (d.Q + 63) / 64);
    hipLaunchKernelGGL((bmm_kernel<TIn, N>), grid, dim3(256), 0, st, d.S, d.G, d.Q, d.max_chunks,
                       static_cast<const TIn *>(B), static_cast<const TIn *>(C), meta, CB);
}

template <typename TIn, int P, int N>
static size_t scan_smem(int Q)
{
    return sizeof(TIn) * ((size_t)P * padded<TIn>(Q) + (size_t)P * padded<TIn>(N)) +
           sizeof(float) * 2 * (size_t)Q;
}

template <typename TIn, int P, int N>
static void launch_scan_t(const PrefillDims &d, const void *x, const void *C, const float *D,
                          const int32_t *meta, const float *cum, const float *dtc, const float *CB,
                          const float *entering, void *y, hipStream_t st)
{
    dim3 grid(d.H, d.max_chunks);
    const size_t smem = scan_smem<TIn, P, N>(d.Q);
    if (smem > 65536) {
        // raise the dynamic LDS limit of this instantiation once (idempotent)
        static bool raised = false;
        if (!raised) {
            hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_scan_kernel<TIn, P, N>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            raised = true;
        }
    }
    hipLaunchKernelGGL((chunk_scan_kernel<TIn, P, N>), grid, dim3(256), smem, st, d.S, d.H, d.G,
                       d.Q, d.max_chunks, static_cast<const TIn *>(x), static_cast<const TIn *>(C),
                       D, meta, cum, dtc, CB, entering, static_cast<TIn *>(y));
}

#define SSD_DISPATCH_PN(d, FN, TIN, ...)                                 \
    do {                                                                 \
        if ((d).P == 64 && (d).N == 128) FN<TIN, 64, 128>(__VA_ARGS__);  \
        else if ((d).P == 64 && (d).N == 16) FN<TIN, 64, 16>(__VA_ARGS__); \
        else if ((d).P == 16 && (d).N == 128) FN<TIN, 16, 128>(__VA_ARGS__); \
        else FN<TIN, 16, 16>(__VA_ARGS__);                               \
    } while (0)

void launch_chunk_state(const PrefillDims &d, const void *x, const void *B, const int32_t *meta,
                        const float *cum, const float *dtc, float *states, void *stream)
{
    if (d.max_chunks <= 0) return;
    hipStream_t st = as_stream(stream);
    if (d.in_bf16) SSD_DISPATCH_PN(d, launch_state_t, bf16, d, x, B, meta, cum, dtc, states, st);
    else SSD_DISPATCH_PN(d, launch_state_t, float, d, x, B, meta, cum, dtc, states, st);
}

void launch_bmm(const PrefillDims &d, const void *B, const void *C, const int32_t *meta, float *CB,
                void *stream)
{
    if (d.max_chunks <= 0) return;
    hipStream_t st = as_stream(stream);
    if (d.in_bf16) {
        if (d.N == 128) launch_bmm_t<bf16, 128>(d, B, C, meta, CB, st);
        else launch_bmm_t<bf16, 16>(d, B, C, meta, CB, st);
    } else {
        if (d.N == 128) launch_bmm_t<float, 128>(d, B, C, meta, CB, st);
        else launch_bmm_t<float, 16>(d, B, C, meta, CB, st);
    }
}

void launch_state_passing(const PrefillDims &d, const float *states, const float *cum,
                          const int32_t *meta, void *cache, const int32_t *idx,
                          const uint8_t *has_init, float *entering, void *ckpt, void *stream)
{
    if (d.S <= 0) return;
    const int PN = d.P * d.N;
    const int EB = (PN + 1023) / 1024;
    dim3 grid((unsigned)((int64_t)d.S * d.H * EB));
    hipStream_t st = as_stream(stream);
    if (d.state_bf16)
        hipLaunchKernelGGL(state_passing_kernel<bf16>, grid, dim3(256), 0, st, d.S, d.H, PN, d.Q,
                           d.max_chunks, d.num_slots, states, cum, meta,
                           static_cast<bf16 *>(cache), idx, has_init, entering,
                           static_cast<bf16 *>(ckpt));
    else
        hipLaunchKernelGGL(state_passing_kernel<float>, grid, dim3(256), 0, st, d.S, d.H, PN, d.Q,
                           d.max_chunks, d.num_slots, states, cum, meta,
                           static_cast<float *>(cache), idx, has_init, entering,
                           static_cast<float *>(ckpt));
}

void launch_chunk_scan(const PrefillDims &d, const void *x, const void *C, const float *D,
                       const int32_t *meta, const float *cum, const float *dtc, const float *CB,
                       const float *entering, void *y, void *stream)
{
    if (d.max_chunks <= 0) return;
    hipStream_t st = as_stream(stream);
    if (d.in_bf16)
        SSD_DISPATCH_PN(d, launch_scan_t, bf16, d, x, C, D, meta, cum, dtc, CB, entering, y, st);
    else
        SSD_DISPATCH_PN(d, launch_scan_t, float, d, x, C, D, meta, cum, dtc, CB, entering, y, st);
}

size_t chunk_scan_smem_bytes(const PrefillDims &d)
{
    size_t s;
    if (d.in_bf16) {
        if (d.P == 64) s = d.N == 128 ? scan_smem<bf16, 64, 128>(d.Q) : scan_smem<bf16, 64, 16>(d.Q);
        else s = d.N == 128 ? scan_smem<bf16, 16, 128>(d.Q) : scan_smem<bf16, 16, 16>(d.Q);
    } else {
        if (d.P == 64) s = d.N == 128 ? scan_smem<float, 64, 128>(d.Q) : scan_smem<float, 64, 16>(d.Q);
        else s = d.N == 128 ? scan_smem<float, 16, 128>(d.Q) : scan_smem<float, 16, 16>(d.Q);
    }
    return s;
}

}  // namespace ssd
