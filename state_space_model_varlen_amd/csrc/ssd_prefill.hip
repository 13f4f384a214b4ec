// Mamba2 SSD chunked varlen prefill on MI355X (gfx950): the five steps of the
// chunked scan - chunk cumsum, chunk state, state passing, bmm, chunk scan -
// as split in vLLM PR #61501 (section "Details"), with the initial state read
// from the cache slot inside state passing and each chunk's entering state
// kept in the workspace for chunk scan (vLLM PR #62922, section "Details").
//
// Notation: chunk c = (seq, start, len) from the metadata, head h, group
// g = h / (H / G), local token index i in [0, len), cum = inclusive cumsum of
// dt * A_h inside the chunk.
#include <type_traits>

#include <hip/hip_ext.h>

#include "ssd_device.h"
#include "ssd_launch.h"

// A kernel launch of the prefill; under a launch trace, hipExtLaunchKernelGGL
// records the kernel's own start and end on the trace's two events for it.
#define SSD_LAUNCH(d, name, kernel, grid, block, smem, st, ...)                                \
    do {                                                                                       \
        void *ev0_ = nullptr, *ev1_ = nullptr;                                                 \
        if (ssd::trace_events((d).trace, (name), &ev0_, &ev1_))                                \
            hipExtLaunchKernelGGL(kernel, grid, block, smem, st, static_cast<hipEvent_t>(ev0_), \
                                  static_cast<hipEvent_t>(ev1_), 0u, __VA_ARGS__);             \
        else                                                                                   \
            hipLaunchKernelGGL(kernel, grid, block, smem, st, __VA_ARGS__);                    \
    } while (0)

namespace ssd {

// ===========================================================================
// Step 1: chunk metadata + chunk cumsum.
// Grid (max_chunks, ceil(H / 4)), 256 threads: one wave per head. Every block
// finds its own chunk from cu_seqlens with a block-wide scan of per-sequence
// chunk counts (no host sync, no extra launch); blocks with blockIdx.y == 0
// publish the metadata. Each wave then runs a wavefront prefix sum of dt * A
// over the chunk (Q / 64 consecutive positions per lane).
constexpr int kCumsumHeadsPerBlock = 4;

__device__ __forceinline__ int wave_inclusive_sum_int(int v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Length of a sequence's first chunk: Q, or with `prefix` (align mode) the
// distance from the sequence's first token to the next absolute multiple of Q
// when prefix[s] tokens precede it.
__device__ __forceinline__ int first_chunk_len(int Q, const int32_t *__restrict__ prefix, int s)
{
    const int pl = prefix ? prefix[s] : 0;
    const int o = pl > 0 ? pl % Q : 0;
    return o > 0 ? Q - o : Q;
}

// Block-wide: locate chunk c among the sequences of cu_seqlens. Writes
// chunk_cu to meta[0..S], the clamped cu_seqlens after the chunk triples and
// the first-chunk lengths after those when `publish_cu`. Returns (seq, k, f,
// a, b) through shared memory: chunk c is chunk k of sequence seq, whose first
// chunk has f tokens and whose clamped token range is [a, b); seq = -1 when
// c >= nc.
__device__ void find_chunk(int T, int S, int Q, int max_chunks, const int32_t *__restrict__ cu,
                           const int32_t *__restrict__ prefix, int c, bool publish_cu,
                           int32_t *__restrict__ meta, int *s_found, int *s_wave_tot)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        s_found[0] = -1;
        s_found[1] = 0;
        s_found[2] = Q;
    }
    int running = 0;
    for (int base = 0; base < S; base += 256) {
        __syncthreads();
        const int s = base + tid;
        int cnt = 0, f = Q, a = 0, b = 0;
        if (s < S) {
            a = clampi(cu[s], 0, T);
            b = clampi(cu[s + 1], 0, T);
            const int L = b > a ? b - a : 0;
            f = first_chunk_len(Q, prefix, s);
            cnt = L == 0 ? 0 : (L <= f ? 1 : 1 + (L - f + Q - 1) / Q);
        }
        const int incl = wave_inclusive_sum_int(cnt, lane);
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
            if (publish_cu) {
                meta[s] = first < max_chunks ? first : max_chunks;
                meta[(S + 1) + 3 * max_chunks + s] = clampi(cu[s], 0, T);
                meta[2 * (S + 1) + 3 * max_chunks + s] = f;
            }
            if (cnt > 0 && c >= first && c < first + cnt) {
                s_found[0] = s;
                s_found[1] = c - first;
                s_found[2] = f;
                s_found[3] = a;     // the sequence's clamped token range, so that
                s_found[4] = b;     // found_chunk need not load it again
            }
        }
        running += tile_tot;
    }
    if (publish_cu && tid == 0) {
        meta[S] = running < max_chunks ? running : max_chunks;
        meta[(S + 1) + 3 * max_chunks + S] = clampi(cu[S], 0, T);
    }
    __syncthreads();
}

// Chunk (seq, start, len) of chunk c after find_chunk (from what it kept of cu_seqlens).
__device__ __forceinline__ ChunkInfo found_chunk(int Q, const int *s_found)
{
    ChunkInfo ci;
    ci.seq = s_found[0];
    ci.start = 0;
    ci.len = 0;
    if (ci.seq >= 0) {
        const int a = s_found[3], b = s_found[4];
        const int k = s_found[1], f = s_found[2];
        ci.start = a + (k == 0 ? 0 : f + (k - 1) * Q);
        const int cap = k == 0 ? f : Q;
        ci.len = b - ci.start < cap ? b - ci.start : cap;
    }
    return ci;
}

// Wavefront prefix sum of dt * A_h over chunk c for head h (one wave). The
// chunk is taken in blocks of 64 positions, position 64 j + lane in block j:
// a wave prefix sum per block, the blocks chained in order,
//   cum = (((tot_0 + tot_1) + ...) + tot_{j-1}) + incl_j,
// which is also the order in which the combined call's state launch, with one
// wave per block, forms it (the two give the same values bit for bit).
template <typename TIn>
__device__ __forceinline__ void cumsum_wave(int H, int Q, int max_chunks, int c, int h,
                                            const ChunkInfo &ci, int lane,
                                            const TIn *__restrict__ dt, const float *__restrict__ A,
                                            float *__restrict__ cum_out, float *__restrict__ dt_out,
                                            const DtTf &tf)
{
    constexpr int J = 4;                    // blocks of 64 positions (Q <= 256)
    const float Ah = A[h];
    const float bh = tf.bias ? tf.bias[h] : 0.0f;
    float vals[J];
    // (loads at clamped positions, zeroed after: no branch between a load and its use)
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = kWave * j + lane;
        const int ic = i < ci.len ? i : ci.len - 1;
        vals[j] = to_f32(dt[(int64_t)(ci.start + ic) * H + h]);
    }
    if (tf.on) {
#pragma unroll
        for (int j = 0; j < J; ++j) vals[j] = dt_transform(tf, vals[j], bh);
    }
    const int64_t row = ((int64_t)h * max_chunks + c) * Q;
    float off = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int i = kWave * j + lane;
        if (kWave * j >= Q) break;
        const float v = i < ci.len ? vals[j] : 0.0f;
        const float incl = wave_inclusive_sum(v * Ah, lane);
        if (i < Q) {
            cum_out[row + i] = j == 0 ? incl : off + incl;
            dt_out[row + i] = v;
        }
        const float tot = __shfl(incl, kWave - 1);
        off = j == 0 ? tot : off + tot;
    }
}

__device__ __forceinline__ void publish_chunk(int S, int c, const ChunkInfo &ci,
                                              int32_t *__restrict__ meta)
{
    int32_t *m = meta + (S + 1) + 3 * c;
    m[0] = ci.seq;
    m[1] = ci.start;
    m[2] = ci.len;
}

// The same chunk counts for one wave alone, for kernels that run before any
// metadata exists (the combined call's state launch): sequences are taken 64 at
// a time, so the cost grows with S (callers keep S small). Results are the same
// in every lane and are returned through readfirstlane, so that the compiler
// keeps them in scalar registers: a buffer resource built from a value it takes
// for a per-lane one makes every load through it a loop over lanes.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Sequence base + lane: chunk count, clamped token range [a, b), first-chunk length.
struct LaneSeq {
    int cnt, a, b, f;
};
__device__ __forceinline__ LaneSeq lane_seq(int T, int S, int Q, const int32_t *__restrict__ cu,
                                            const int32_t *__restrict__ prefix, int base, int lane)
{
    LaneSeq r{0, 0, 0, Q};
    const int s = base + lane;
    if (s < S) {
        r.a = clampi(cu[s], 0, T);
        r.b = clampi(cu[s + 1], 0, T);
        const int L = r.b > r.a ? r.b - r.a : 0;
        r.f = first_chunk_len(Q, prefix, s);
        r.cnt = L == 0 ? 0 : (L <= r.f ? 1 : 1 + (L - r.f + Q - 1) / Q);
    }
    return r;
}

// Sequence s: its first chunk index (not clamped), chunk count, clamped token
// range and first-chunk length; also the batch's total chunk count.
struct SeqSpan {
    int c0, cnt, a, b, f, total;
};
__device__ __forceinline__ SeqSpan wave_seq_span(int T, int S, int Q, const int32_t *__restrict__ cu,
                                                 const int32_t *__restrict__ prefix, int s, int lane)
{
    SeqSpan r{0, 0, 0, 0, Q, 0};
    int running = 0;
    for (int base = 0; base < S; base += kWave) {
        const LaneSeq ls = lane_seq(T, S, Q, cu, prefix, base, lane);
        const int incl = wave_inclusive_sum_int(ls.cnt, lane);
        if (s >= base && s < base + kWave) {   // (uniform: s is the same in every lane)
            const int src = s - base;
            r.c0 = running + __shfl(incl - ls.cnt, src);
            r.cnt = __shfl(ls.cnt, src);
            r.a = __shfl(ls.a, src);
            r.b = __shfl(ls.b, src);
            r.f = __shfl(ls.f, src);
        }
        running += __shfl(incl, kWave - 1);
    }
    r.total = uniform(running);
    r.c0 = uniform(r.c0);
    r.cnt = uniform(r.cnt);
    r.a = uniform(r.a);
    r.b = uniform(r.b);
    r.f = uniform(r.f);
    return r;
}

// Chunk c: (sequence, first token, token count), sequence -1 past the last chunk.
__device__ __forceinline__ ChunkInfo wave_find_chunk(int T, int S, int Q,
                                                     const int32_t *__restrict__ cu,
                                                     const int32_t *__restrict__ prefix, int c,
                                                     int lane)
{
    ChunkInfo ci;
    ci.seq = -1;
    ci.start = 0;
    ci.len = 0;
    int running = 0;
    for (int base = 0; base < S; base += kWave) {
        const LaneSeq ls = lane_seq(T, S, Q, cu, prefix, base, lane);
        const int incl = wave_inclusive_sum_int(ls.cnt, lane);
        const int first = running + incl - ls.cnt;
        const unsigned long long hit = __ballot(ls.cnt > 0 && c >= first && c < first + ls.cnt);
        if (hit) {
            const int src = __builtin_ctzll(hit);
            const int k = c - __shfl(first, src), f = __shfl(ls.f, src);
            const int a = __shfl(ls.a, src), b = __shfl(ls.b, src);
            ci.seq = base + src;
            ci.start = a + (k == 0 ? 0 : f + (k - 1) * Q);
            const int cap = k == 0 ? f : Q;
            ci.len = b - ci.start < cap ? b - ci.start : cap;
        }
        running += __shfl(incl, kWave - 1);
    }
    ci.seq = uniform(ci.seq);
    ci.start = uniform(ci.start);
    ci.len = uniform(ci.len);
    return ci;
}

template <typename TIn>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(
    int T, int S, int H, int Q, int max_chunks, const TIn *__restrict__ dt,
    const float *__restrict__ A, const int32_t *__restrict__ cu, int32_t *__restrict__ meta,
    float *__restrict__ cum_out, float *__restrict__ dt_out, DtTf tf,
    const int32_t *__restrict__ prefix)
{
    __shared__ int s_wave_tot[4];
    __shared__ int s_found[5];
    const int c = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool publish = blockIdx.y == 0;
    find_chunk(T, S, Q, max_chunks, cu, prefix, c, publish && blockIdx.x == 0, meta, s_found,
               s_wave_tot);
    const ChunkInfo ci = found_chunk(Q, s_found);
    if (publish && threadIdx.x == 0) publish_chunk(S, c, ci, meta);
    const int h = blockIdx.y * kCumsumHeadsPerBlock + wave;
    if (ci.len <= 0 || h >= H) return;
    cumsum_wave<TIn>(H, Q, max_chunks, c, h, ci, lane, dt, A, cum_out, dt_out, tf);
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
// Step 2: chunk state (generic path). Grid (H, max_chunks), 256 threads (4 waves).
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
// Sequential over the sequence's chunks in float32 registers; bandwidth-bound.
// The entering states are stored in the dtype chunk scan feeds its MFMA
// (TE = input dtype), the checkpoints and the final state in the cache dtype.
template <typename TS, typename TE, int EG>
__global__ __launch_bounds__(256) void state_passing_kernel(
    int S, int H, int PN, int Q, int max_chunks, int num_slots, const float *states,
    const float *__restrict__ cum, const int32_t *__restrict__ meta, TS *cache,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ has_init, TE *entering,
    TS *__restrict__ ckpt, SrCtx sr)
{
    // a block covers 1024 EG consecutive state elements of one (sequence, head):
    // group g of a thread is elements e0 + 1024 g .. + 3 (PN is a multiple of
    // 1024 EG whenever EG > 1)
    const int EB = (PN + 1024 * EG - 1) / (1024 * EG);
    const int b = blockIdx.x;
    const int eb = b % EB;
    const int h = (b / EB) % H;
    const int s = b / (EB * H);
    const int e0 = eb * 1024 * EG + threadIdx.x * 4;
    if (s >= S || e0 >= PN) return;

    const int slot = idx[s];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const bool read_init = slot_ok && (has_init != nullptr && has_init[s] != 0);
    TS *cslot = cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN + e0;

    // every load below is unconditional (a branch between a load and its use makes
    // the compiler wait on the load right there): the initial state is loaded from
    // slot 0 when there is none and cleared bit-wise; batch entries past the
    // sequence's last chunk reload that chunk and are not used
    float hs[EG][4];
#pragma unroll
    for (int g = 0; g < EG; ++g) load4<TS>(cslot + 1024 * g, hs[g]);
    const uint32_t keep = read_init ? 0xffffffffu : 0u;
    const SrKey srk = sr_key(sr, meta);

    int c0 = meta[s], c1 = meta[s + 1];
    c0 = c0 < max_chunks ? c0 : max_chunks;
    c1 = c1 < max_chunks ? c1 : max_chunks;
    // chunks in batches (16, 4 and 1 with one element group per thread; 4 and 1
    // with four): every chunk state of a batch is requested before the sequential
    // recurrence over it runs, and a batch never reaches past the sequence's last
    // chunk (so its loads need no guard)
    bool masked = false;
    auto batch = [&](int cb, auto kb) {
        constexpr int K = decltype(kb)::value;
        float sc[K][EG][4], dec[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = cb + k;
#pragma unroll
            for (int g = 0; g < EG; ++g)
                load4<float>(states + ((int64_t)c * H + h) * PN + e0 + 1024 * g, sc[k][g]);
            const int len = meta[(S + 1) + 3 * c + 2];
            const float cl = cum[((int64_t)h * max_chunks + c) * Q + (len > 0 ? len - 1 : 0)];
            dec[k] = len > 0 ? __expf(cl) : 1.0f;
        }
        if (!masked) {     // the initial state is used only now, after the batch was requested
#pragma unroll
            for (int g = 0; g < EG; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) hs[g][q] = __uint_as_float(__float_as_uint(hs[g][q]) & keep);
            masked = true;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
            for (int g = 0; g < EG; ++g) {
                const int64_t off = ((int64_t)(cb + k) * H + h) * PN + e0 + 1024 * g;
                // the chunk state at `off` was loaded above, before the entering
                // state (which may share its memory) is stored
                store4<TE>(entering + off, hs[g]);
#pragma unroll
                for (int q = 0; q < 4; ++q) hs[g][q] = dec[k] * hs[g][q] + sc[k][g][q];
                if (ckpt) put4<TS>(ckpt + off, hs[g], srk, (uint64_t)off, kSrCkpt);
            }
        }
    };
    int cb = c0;
    if constexpr (EG == 1)
        for (; cb + 16 <= c1; cb += 16) batch(cb, std::integral_constant<int, 16>());
    for (; cb + 4 <= c1; cb += 4) batch(cb, std::integral_constant<int, 4>());
    for (; cb < c1; ++cb) batch(cb, std::integral_constant<int, 1>());
    if (!masked) {
#pragma unroll
        for (int g = 0; g < EG; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) hs[g][q] = __uint_as_float(__float_as_uint(hs[g][q]) & keep);
    }
    if (slot_ok) {
#pragma unroll
        for (int g = 0; g < EG; ++g)
            put4<TS>(cslot + 1024 * g, hs[g], srk,
                     (uint64_t)(((int64_t)slot * H + h) * PN + e0 + 1024 * g), kSrFinal);
    }
}

// ===========================================================================
// Step 4: bmm. Grid (max_chunks, G, Q / 16), 256 threads. Block z owns CB rows
// [16 z, 16 z + 16); its 4 waves share the 16-column tiles at or left of the
// diagonal (wave w: tiles w, w + 4, ...). Each tile is computed transposed,
// CB^T = B . C^T (A operand: B rows, B operand: C rows - both load straight
// from HBM because d_state is their contiguous index), so that each lane ends
// up holding 4 consecutive columns of one CB row and stores them at once.
// CB is stored in the input dtype (chunk scan rounds its masked product to
// that dtype for the MFMA in any case): row-major for float32 inputs, MFMA
// fragment order (cb_frag_offset) for bf16 inputs.
// Row tile z of CB for chunk c, group g (one block of 256 threads).
template <typename TIn, int N>
__device__ __forceinline__ void bmm_rows(int G, int Q, int c, int g, int z, const ChunkInfo &ci,
                                         const TIn *__restrict__ B, const TIn *__restrict__ C,
                                         TIn *__restrict__ CB)
{
    typedef Mma<TIn> M;
    constexpr int NK = (N + M::K - 1) / M::K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int i0 = z * 16;
    if (ci.len <= 0 || i0 >= ci.len) return;

    // rows past the chunk's end are loaded at the last row and zeroed after the
    // load (no branch between a load and its use)
    typename M::frag cf[NK];       // C rows i0 .. i0 + 15 (B operand)
    const int i = i0 + r16;
    const int ic = i < ci.len ? i : ci.len - 1;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n = kk * M::K + kg * M::KPL;
        const int nc = n < N ? n : 0;
        const typename M::frag f = M::load(C + ((int64_t)(ci.start + ic) * G + g) * N + nc);
        cf[kk] = (i < ci.len && n < N) ? f : M::zero();
    }
    TIn *cbc = CB + ((int64_t)c * G + g) * Q * Q;
    // bf16 (fragment order): the 16 x 32 blocks holding the diagonal are written
    // whole, zero above the diagonal, so that chunk scan needs no causal mask
    const int jd = i0 / 16;
    const int jmax = sizeof(TIn) == 2 && (jd & 1) == 0 ? jd + 1 : jd;
    for (int jt = wave; jt <= jmax; jt += 4) {
        const int jc = jt * 16 + 4 * kg;
        if (jt > jd) {
            const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            store4<TIn>(cbc + cb_frag_offset(Q, i, jc), z);
            continue;
        }
        const int j = jt * 16 + r16;
        const int jcl = j < ci.len ? j : ci.len - 1;
        typename M::frag bfr[NK];  // B rows j (A operand)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n = kk * M::K + kg * M::KPL;
            const int nc = n < N ? n : 0;
            const typename M::frag f = M::load(B + ((int64_t)(ci.start + jcl) * G + g) * N + nc);
            bfr[kk] = (j < ci.len && n < N) ? f : M::zero();
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc = M::run(bfr[kk], cf[kk], acc);
        // lane holds CB^T[16 jt + 4 kg + v][i] = CB[i][16 jt + 4 kg + v], v = 0..3:
        // 4 consecutive elements in either layout (row-major for float32 inputs,
        // MFMA fragment order for bf16 inputs)
        float v4[4] = {acc[0], acc[1], acc[2], acc[3]};
        if (jt == jd) {
#pragma unroll
            for (int v = 0; v < 4; ++v) v4[v] = jc + v <= i ? v4[v] : 0.0f;
        }
        if constexpr (sizeof(TIn) == 2) store4<TIn>(cbc + cb_frag_offset(Q, i, jc), v4);
        else store4<TIn>(cbc + (int64_t)i * Q + jc, v4);
    }
}

template <typename TIn, int N>
__global__ __launch_bounds__(256) void bmm_kernel(int S, int G, int Q, int max_chunks,
                                                  const TIn *__restrict__ B,
                                                  const TIn *__restrict__ C,
                                                  const int32_t *__restrict__ meta,
                                                  TIn *__restrict__ CB)
{
    const int c = blockIdx.x;
    bmm_rows<TIn, N>(G, Q, c, blockIdx.y, blockIdx.z, chunk_info(meta, S, c), B, C, CB);
}

// CB for one (chunk, group) pair per block (bf16, d_state 128), for batches
// with enough pairs to fill the chip. The chunk's B rows are staged in LDS once
// and every row tile of the pair reads its A operands there, where the row-tile
// blocks of bmm_kernel each fetch them again from L2 (at Q = 256 that is 136
// column tiles of 4 KiB per pair instead of 64 KiB). Same products, layout and
// zeros as bmm_rows. Block of 2 Q threads (Q / 32 waves); wave w takes row
// tiles w and Q / 16 - 1 - w, so the causal work is balanced.
constexpr int kCbLDB = 136;       // B row pitch in LDS (bf16): 68 dwords, conflict-free b128 reads
constexpr int kCbPairMin = 128;   // pairs from which the per-pair kernel is used

// The pair body for a block of NT >= 2 Q threads (waves past Q / 32 only take
// part in the barrier); bs: Q x kCbLDB bf16 of LDS.
template <int Q, int NT>
__device__ __forceinline__ void cb_pair(int G, int c, int g, const ChunkInfo &ci,
                                        const bf16 *__restrict__ B, const bf16 *__restrict__ C,
                                        bf16 *__restrict__ CB, bf16 *bs)
{
    constexpr int N = 128, KV = Q * (N / 8) / NT > 0 ? Q * (N / 8) / NT : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int len = ci.len;
    // B and C rows through buffer resources ending at the chunk's last row
    // (rows past it read as zero, with no branch around the loads)
    const uint32_t brow = (uint32_t)G * N * 2;
    const rsrc_t rb = make_rsrc(B + ((int64_t)ci.start * G + g) * N, (uint32_t)(len - 1) * brow + N * 2);
    const rsrc_t rc = make_rsrc(C + ((int64_t)ci.start * G + g) * N, (uint32_t)(len - 1) * brow + N * 2);
    uint4 bv[KV];
#pragma unroll
    for (int k = 0; k < KV; ++k) {
        const int u = tid + NT * k;
        bv[k] = buf_ld16(rb, (uint32_t)(u >> 4) * brow + 16 * (u & 15));
    }
    // C rows i = 16 rt + r16 of the wave's two row tiles: B operand fragments
    const int rt[2] = {Q / 16 - 1 - wave, wave};
    uint4 cf[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            cf[a][kk] = buf_ld16(rc, (uint32_t)(16 * rt[a] + r16) * brow + 64 * kk + 16 * kg);
#pragma unroll
    for (int k = 0; k < KV; ++k) {
        const int u = tid + NT * k;
        *reinterpret_cast<uint4 *>(bs + (u >> 4) * kCbLDB + 8 * (u & 15)) = bv[k];
    }
    __syncthreads();
    if (wave >= Q / 32) return;   // (no row tiles: the C loads above read nothing)
    bf16 *cbc = CB + ((int64_t)c * G + g) * Q * Q;
    const int ntiles = (len + 15) / 16;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int z = rt[a];
        if (z >= ntiles) continue;
        const int i = 16 * z + r16;
        // the 16 x 32 blocks holding the diagonal are written whole, zero above it
        const int jmax = (z & 1) == 0 ? z + 1 : z;
        for (int jt = 0; jt <= jmax; ++jt) {
            const int jc = jt * 16 + 4 * kg;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 af =
                    *reinterpret_cast<const bf16x8 *>(bs + (16 * jt + r16) * kCbLDB + 32 * kk + 8 * kg);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, cf[a][kk]),
                                                              acc, 0, 0, 0);
            }
            // lane holds CB[i][16 jt + 4 kg + v], v = 0..3
            float v4[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
            for (int v = 0; v < 4; ++v) v4[v] = jt <= z && jc + v <= i ? v4[v] : 0.0f;
            store4<bf16>(cbc + cb_frag_offset(Q, i, jc), v4);
        }
    }
}

template <int Q>
__global__ __launch_bounds__(2 * Q) void bmm_pair_kernel(int S, int G,
                                                         const bf16 *__restrict__ B,
                                                         const bf16 *__restrict__ C,
                                                         const int32_t *__restrict__ meta,
                                                         bf16 *__restrict__ CB)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int c = blockIdx.x / G, g = blockIdx.x - c * G;
    const ChunkInfo ci = chunk_info(meta, S, c);
    if (ci.len <= 0) return;
    cb_pair<Q, 2 * Q>(G, c, g, ci, B, C, CB, reinterpret_cast<bf16 *>(smem));
}

bool cb_by_pair(const PrefillDims &d)
{
    return d.in_bf16 && d.N == 128 && (int64_t)d.max_chunks * d.G >= kCbPairMin;
}

// Steps 1 and 4 in one launch (the combined call): grid (max_chunks, HB + G Q / 16),
// HB = ceil(H / 4). Blocks with blockIdx.y < HB are cumsum blocks (four heads,
// metadata published by blockIdx.y == 0), the others compute one CB row tile.
// Every block finds its chunk from cu_seqlens itself, so the two halves do not
// wait for each other.
template <typename TIn, int N>
__global__ __launch_bounds__(256) void chunk_prep_kernel(
    int T, int S, int H, int G, int Q, int max_chunks, const TIn *__restrict__ dt,
    const float *__restrict__ A, const int32_t *__restrict__ cu, int32_t *__restrict__ meta,
    float *__restrict__ cum_out, float *__restrict__ dt_out, const TIn *__restrict__ B,
    const TIn *__restrict__ C, TIn *__restrict__ CB, DtTf tf, const int32_t *__restrict__ prefix)
{
    __shared__ int s_wave_tot[4];
    __shared__ int s_found[5];
    const int c = blockIdx.x;
    const int HB = (H + kCumsumHeadsPerBlock - 1) / kCumsumHeadsPerBlock;
    const bool publish = blockIdx.y == 0;
    find_chunk(T, S, Q, max_chunks, cu, prefix, c, publish && blockIdx.x == 0, meta, s_found,
               s_wave_tot);
    const ChunkInfo ci = found_chunk(Q, s_found);
    if ((int)blockIdx.y < HB) {
        if (publish && threadIdx.x == 0) publish_chunk(S, c, ci, meta);
        const int h = blockIdx.y * kCumsumHeadsPerBlock + (threadIdx.x >> 6);
        if (ci.len <= 0 || h >= H) return;
        cumsum_wave<TIn>(H, Q, max_chunks, c, h, ci, threadIdx.x & 63, dt, A, cum_out, dt_out,
                         tf);
    } else {
        const int y = blockIdx.y - HB, tiles = Q / 16;
        bmm_rows<TIn, N>(G, Q, c, y / tiles, y % tiles, ci, B, C, CB);
    }
}

// ===========================================================================
// Step 5: chunk scan (generic path: float32, and the bf16 shapes without a
// fast kernel). Grid (H, max_chunks), 256 threads (4 waves). x of the whole
// chunk is staged transposed in LDS (MFMA B operand for the intra-chunk
// product), the entering state [P][N] in LDS (B operand of the state term). Wave w handles the 16-row tiles r with r mod 8 in {w, 7 - w}
// so that the causal work is balanced. Per row tile:
//   acc  = sum_j (CB[i,j] exp(cum_i - cum_j) dt_j [j <= i]) x_j      (MFMA)
//   acc += (exp(cum_i) C_i) . H_in^T                                  (MFMA)
//   y_i  = acc + D_h x_i
template <typename TIn, int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    int S, int H, int G, int Q, int max_chunks, const TIn *__restrict__ x,
    const TIn *__restrict__ C, const float *__restrict__ D, const int32_t *__restrict__ meta,
    const float *__restrict__ cum, const float *__restrict__ dtc, const TIn *__restrict__ CB,
    const TIn *__restrict__ entering, TIn *__restrict__ y)
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
        const TIn *hin = entering + ((int64_t)c * H + h) * P * N;
        for (int e = tid * 4; e < P * N; e += 256 * 4) {
            const int p = e / N, n = e % N;
#pragma unroll
            for (int k = 0; k < 4; ++k) hsm[p * LDH + n + k] = hin[e + k];
        }
    }
    __syncthreads();

    const float Dh = D ? D[h] : 0.0f;
    const TIn *Cbase = C + ((int64_t)ci.start * G + g) * N;
    const TIn *CBc = CB + ((int64_t)c * G + g) * Q * Q;
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
            float cbv[Vec16<TIn>::kElems > KPL ? Vec16<TIn>::kElems : KPL];
            if constexpr (KPL == 8) {
                // fragment order: the 8 values are j = j0 + 4 kg + v % 4 + 16 (v / 4)
                Vec16<TIn>::load(CBc + cb_frag_offset(Q, i, j0 + 4 * kg), cbv);
            } else {
#pragma unroll
                for (int v = 0; v < KPL; ++v) cbv[v] = to_f32(CBc[(int64_t)i * Q + jb + v]);
            }
#pragma unroll
            for (int v = 0; v < KPL; ++v) {
                const int j = KPL == 8 ? j0 + 4 * kg + (v & 3) + ((v >> 2) << 4) : jb + v;
                const float m = (j <= i) ? cbv[v] * __expf(cum_i - scum[j]) * sdt[j] : 0.0f;
                M::set(af, v, m);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                typename M::frag bf;
                if constexpr (KPL == 8) {     // split K order, as the CB fragment
                    const TIn *xp = &xs[(pt * 16 + r16) * LDX + j0 + 4 * kg];
                    typedef short v4s __attribute__((ext_vector_type(4)));
                    const v4s lo = *reinterpret_cast<const v4s *>(xp);
                    const v4s hi = *reinterpret_cast<const v4s *>(xp + 16);
                    typedef short v8s __attribute__((ext_vector_type(8)));
                    const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    bf = __builtin_bit_cast(typename M::frag, both);
                } else {
                    bf = M::load(&xs[(pt * 16 + r16) * LDX + jb]);
                }
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
// Fast bf16 kernels for headdim 64, d_state 128 (gfx950).
//
// Tiles are staged in LDS row-major - token rows, 16-byte copies straight
// from HBM - and MFMA operands that need the token index contiguous per lane
// are read with the LDS transpose read (mfma_frag_tr). Rows are padded: 72
// elements (36 dwords) in chunk_state, which puts the four rows one 16-lane
// group reads in disjoint bank ranges; 80 elements (40 dwords) in the fused
// state kernel and the chunk scan, with no overlap at all. Blocks are put in
// XCD-aware order so the heads sharing a chunk's B, C and CB run on one L2.
constexpr int kFastLD = 72;   // row pitch of token-major tiles (64 bf16 + 8 pad)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint4 ld16(const bf16 *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(bf16 *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

// Chunk state, bf16, P = 64, N = 128 split in two 64-column halves.
// Grid: max_chunks * 2 * H blocks of 256 threads, logical order (chunk, half, head).
// Wave w computes rows p in [16 w, 16 w + 16) of the [64 x 64] half-state:
//   S[p][n] = sum_t (w_t x_t[p]) B_t[n],  w_t = exp(cum_last - cum_t) dt_t.
template <int Q>
__global__ __launch_bounds__(256) void chunk_state_fast_kernel(
    int S, int H, int G, int max_chunks, const bf16 *__restrict__ x,
    const bf16 *__restrict__ B, const int32_t *__restrict__ meta, const float *__restrict__ cum,
    const float *__restrict__ dtc, float *__restrict__ states)
{
    constexpr int P = 64, N = 128, NH = 64, LD = kFastLD;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *xs = reinterpret_cast<bf16 *>(smem);   // [Q][LD]  w_t * x_t
    bf16 *bs = xs + Q * LD;                      // [Q][LD]  B_t, one column half
    float *ws = reinterpret_cast<float *>(bs + Q * LD);

    const int nblk = max_chunks * 2 * H;
    const int lb = xcd_logical_block(blockIdx.x, nblk);
    const int h = lb % H, nh = (lb / H) & 1, c = lb / (2 * H);
    const ChunkInfo ci = chunk_info(meta, S, c);
    if (ci.len <= 0) return;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int len = ci.len;

    // issue every global load of the chunk first: x rows and B half-rows, 8 vectors of
    // 8 bf16 per row, Q rows each -> Q / 32 vectors of each per thread (<= 8)
    // (buffer resources ending at the chunk's last row: rows past it read as zeros,
    // with no branch between a load and its use)
    constexpr int kVec = Q / 32;          // vectors of each tile per thread
    uint4 xr[kVec], br[kVec];
    const uint32_t xrow = (uint32_t)H * P * 2, brow = (uint32_t)G * N * 2;
    const rsrc_t rx = make_rsrc(x + ((int64_t)ci.start * H + h) * P, (uint32_t)(len - 1) * xrow + P * 2);
    const rsrc_t rb = make_rsrc(B + ((int64_t)ci.start * G + g) * N + nh * NH,
                                (uint32_t)(len - 1) * brow + NH * 2);
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        const int u = tid + 256 * k;
        const uint32_t t = u >> 3, c8 = u & 7;
        xr[k] = buf_ld16(rx, t * xrow + 16 * c8);
        br[k] = buf_ld16(rb, t * brow + 16 * c8);
    }
    const float *cumrow = cum + ((int64_t)h * max_chunks + c) * Q;
    const float *dtrow = dtc + ((int64_t)h * max_chunks + c) * Q;
    const float cum_last = cumrow[len - 1];
    for (int t = tid; t < Q; t += 256)
        ws[t] = t < len ? __expf(cum_last - cumrow[t]) * dtrow[t] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        const int u = tid + 256 * k;
        {
            const int t = u >> 3, c8 = u & 7;
            float v[8];
            const uint32_t w4[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
            const float wt = ws[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w4[i] << 16) * wt;
                v[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u) * wt;
            }
            Vec16<bf16>::store(xs + t * LD + 8 * c8, v);
            st16(bs + t * LD + 8 * c8, br[k]);
        }
    }
    __syncthreads();

    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = zero4();
    const int nk = (len + 31) / 32;
    for (int ks = 0; ks < nk; ++ks) {
        const int t0 = 32 * ks;
        const bf16x8 af = mfma_frag_tr_split(xs, LD, t0, 16 * wave, lane);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const bf16x8 bf = mfma_frag_tr_split(bs, LD, t0, 16 * ct, lane);
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[ct], 0, 0, 0);
        }
    }
    // direct stores: for each (ct, v) 16 lanes write 64 contiguous bytes. (Staging
    // this tile through LDS for 16-byte stores was tried; the compiler merged the
    // LDS writes into ds_write2_b32 with wrong offsets, so it is not done.)
    float *out = states + ((int64_t)c * H + h) * P * N + nh * NH;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[(16 * wave + 4 * kg + v) * N + 16 * ct + r16] = acc[ct][v];
}

// Chunk state and state passing in one pass, bf16, P = 64, N = 128 (used by
// the combined call). One block of 512 threads per (sequence, head, half of
// the state columns), walking the sequence's chunks in order; the running
// state H lives in the MFMA accumulators (wave w owns rows 16 (w % 4) .. + 15
// and columns 32 (w / 4) .. + 31 of the half, as two 16 x 16 tiles):
//   entering[c] = H;   H <- exp(cum_last) H + sum_t x_t (w_t B_t)^T,
//   w_t = exp(cum_last - cum_t) dt_t,
// and checkpoints / the final state are written from the same registers, so
// chunk states never go to memory. The tiles of chunk c + 1 are in flight to
// registers (buffer loads that return zeros past the chunk's end) while chunk
// c is contracted; x is staged as loaded, B scaled by w_t.
constexpr int kScanLDX = 80;   // x row pitch in LDS (bf16): conflict-free transpose reads
constexpr int kScanNSL = 64;   // state columns per block
constexpr int kScanLDB = kScanNSL + 16;

template <int Q> struct StateScanRegs {
    static constexpr int kXV = (Q * 8 + 511) / 512;    // x vectors (8 bf16) per thread
    static constexpr int kBV = (Q * 8 + 511) / 512;    // B vectors per thread (8 per row)
    static constexpr int kJ = (Q + kWave - 1) / kWave; // 64-position blocks of a chunk
    uint4 x[kXV], b[kBV];
    float cm[kBV], dt[kBV];                            // cum and dt of the B rows
    float cl;                                          // cum at the chunk's last token
    uint32_t dr;                                       // raw bf16 dt (OWN: waves < kJ)
};

// With OWN (the combined call, few sequences) the same launch also does step 1
// and, unsegmented, step 4, so that neither needs a launch of its own:
//   - every state block finds its sequence's chunks from cu_seqlens and scans
//     dt * A_h over each chunk itself, one chunk ahead: wave w < Q / 64 takes
//     positions 64 w .. + 63 (a wave prefix sum, kept with dt in the unused pad
//     columns of the LDS x rows, and the block's total), and the staging of the
//     next step chains the blocks in order - the cumsum kernel's order, so the
//     values are the same bit for bit;
//   - the blocks of column slice 0 publish what the later launches read: the
//     cumsum and dt rows of their head, and (head 0) the chunk metadata;
//   - own.CB set: max_chunks G more blocks compute CB, one (chunk, group) pair
//     each, in the CUs the short chains leave free: after the state blocks, or
//     in longest-chain-first order right after the first round of them (ahead
//     of the shorter chains, which are each mostly start-up latency), their
//     count then padded to a multiple of 8 so that the state blocks behind them
//     keep their XCD.
constexpr int kStateRound = 512;   // state blocks in flight at once: two per CU
template <int Q, bool CKPT, bool SEG, bool OWN, typename TS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void state_scan_fast_kernel(
    int S, int H, int G, int max_chunks, int num_slots, const bf16 *__restrict__ x,
    const bf16 *__restrict__ B, const int32_t *__restrict__ meta, const float *__restrict__ cum,
    const float *__restrict__ dtc, TS *cache, const int32_t *__restrict__ idx,
    const uint8_t *__restrict__ has_init, bf16 *__restrict__ entering, TS *__restrict__ ckpt,
    SrCtx sr, int nseg, float *__restrict__ seg_fin, float *__restrict__ seg_L,
    float *__restrict__ seg_F, int32_t *__restrict__ seg_I, int lpt, OwnPrep own, int T,
    const int32_t *__restrict__ prefix)
{
    constexpr int P = 64, N = 128, NSL = kScanNSL, NS = N / NSL;
    constexpr int LDX = kScanLDX, LDB = kScanLDB;
    constexpr int J = StateScanRegs<Q>::kJ;
    static_assert(LDX >= P + 4, "the cum / dt / block-total pad of an x row");
    typedef StateScanRegs<Q> Regs;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *xs = reinterpret_cast<bf16 *>(smem);   // [Q][LDX]  x_t (OWN: pad floats at column P:
                                                 //  block prefix sum, dt; row j < J: block j's total)
    bf16 *bs = xs + Q * LDX;                     // [Q][LDB]  w_t B_t (slice columns)

    // logical order (head, segment of sequence, column slice): each XCD takes a
    // contiguous range of heads with every sequence of the batch, so a batch of
    // long and short sequences gives every XCD the same chain lengths, and the
    // heads that share a B group sit side by side on one XCD
    const int nsg = SEG ? nseg : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    int bid = (int)blockIdx.x;   // the state block's index (past the CB blocks)
    if constexpr (OWN) {
        const int nstate = S * nsg * H * NS;
        int cb_at = nstate, cb_n = max_chunks * G;
        if (!SEG && lpt) {
            const int per_rank = H * NS;
            const int r1 = (kStateRound + per_rank - 1) / per_rank * per_rank;
            cb_at = r1 < nstate ? r1 : nstate;
            cb_n = own.CB != nullptr ? (cb_n + kXcds - 1) / kXcds * kXcds : 0;
        }
        if (!SEG && lpt ? bid >= cb_at && bid < cb_at + cb_n : bid >= nstate) {
            // CB of one (chunk, group) pair, through this kernel's LDS
            const int pr = bid - cb_at, c = pr / G, g = pr - c * G;
            if (!SEG && lpt && c >= max_chunks) return;   // (padding)
            const ChunkInfo ci = wave_find_chunk(T, S, Q, own.cu, prefix, c, lane);
            if (ci.len > 0)   // (the same in every wave)
                cb_pair<Q, 512>(G, c, g, ci, B, static_cast<const bf16 *>(own.C),
                                static_cast<bf16 *>(own.CB), xs);
            return;
        }
        if (!SEG && lpt && bid >= cb_at) bid -= cb_n;
    }
    int q, h, s, b, sb;
    // longest chain first with OWN: the sequence's span, cache slot and
    // has-initial flag come from the same per-lane loads as the ranking (one
    // memory latency; with no flag array a byte of idx stands in and the flag
    // is ignored)
    SeqSpan lsp{0, 0, 0, 0, Q, 0};
    int lslot = 0, lflag = 0;
    if (!SEG && lpt) {
        // Longest chain first (few sequences, heads a multiple of 8): XCD x owns
        // heads [x H / 8, (x + 1) H / 8) of every sequence, and its blocks go out
        // in order of the sequences' chunk counts, longest first, so that the
        // long chains start in the first round on every XCD. Every wave ranks the
        // sequences itself (count descending, then index): rank r -> sequence s.
        const int xcd = bid % kXcds, slot = bid / kXcds;
        const int hx = H / kXcds;
        const int r = slot / (hx * NS), rem = slot - r * (hx * NS);
        h = xcd * hx + rem / NS;
        q = rem - (rem / NS) * NS;
        auto pick = [&](int cnt) {
            int rank = 0;
            for (int t = 0; t < S; ++t) {
                const int ct = __shfl(cnt, t);
                rank += (ct > cnt || (ct == cnt && t < lane)) ? 1 : 0;
            }
            const unsigned long long hit = __ballot(lane < S && rank == r);
            return hit ? (int)__builtin_ctzll(hit) : 0;
        };
        if constexpr (OWN) {
            // lane = sequence (S <= 64 here): its slot and flag, then its span
            // (requested before the span's loads wait)
            const int sl = lane < S ? lane : 0;
            const int il = idx[sl];
            const int fl = (has_init != nullptr ? has_init : reinterpret_cast<const uint8_t *>(idx))[sl];
            const LaneSeq ls = lane_seq(T, S, Q, own.cu, prefix, 0, lane);
            const int incl = wave_inclusive_sum_int(ls.cnt, lane), excl = incl - ls.cnt;
            // ranked by the clamped counts the metadata would hold
            s = pick((incl < max_chunks ? incl : max_chunks) - (excl < max_chunks ? excl : max_chunks));
            lsp.c0 = uniform(__shfl(excl, s));
            lsp.cnt = uniform(__shfl(ls.cnt, s));
            lsp.a = uniform(__shfl(ls.a, s));
            lsp.b = uniform(__shfl(ls.b, s));
            lsp.f = uniform(__shfl(ls.f, s));
            lsp.total = uniform(__shfl(incl, kWave - 1));
            lslot = uniform(__shfl(il, s));
            lflag = uniform(__shfl(fl, s));
        } else {
            const int sl = lane < S ? lane : S - 1;
            s = pick(meta[sl + 1] - meta[sl]);
        }
        b = 0;
        sb = s;
    } else {
        const int nblk = S * nsg * H * NS;
        const int lb = xcd_logical_block(bid, nblk);
        q = lb % NS;
        sb = (lb / NS) % (S * nsg);
        h = lb / (NS * S * nsg);
        s = sb / nsg;
        b = sb - s * nsg;
    }
    const int g = h / (H / G);
    const int r16 = lane & 15, kg = lane >> 4;
    const int pw = wave & 3, nh = wave >> 2;
    const int n0 = q * NSL;
    const int PN = P * N;
    // this lane's state elements: row 16 pw + r16, columns n0 + 32 nh + 16 j + 4 kg + 0..3
    const int64_t run = (int64_t)(16 * pw + r16) * N + n0 + 32 * nh + 4 * kg;

    // every per-sequence value is requested before any is used (one memory
    // latency): chunk range, token range, slot, has-initial flag
    const int tokoff = (S + 1) + 3 * max_chunks;
    int c0, c1, first, end, fcl, total = 0;   // fcl: first chunk's length (Q unless aligned)
    SrKey srk;
    float Ah = 0.0f, bh = 0.0f;
    if constexpr (OWN) {
        const SeqSpan sp = !SEG && lpt ? lsp : wave_seq_span(T, S, Q, own.cu, prefix, s, lane);
        c0 = sp.c0;
        c1 = sp.c0 + sp.cnt;
        first = sp.a;
        end = sp.b;
        fcl = sp.f;
        total = sp.total;
        srk = sr_key_checked(sr);
        Ah = own.A[h];
        bh = own.tf.bias ? own.tf.bias[h] : 0.0f;
    } else {
        c0 = meta[s];
        c1 = meta[s + 1];
        first = meta[tokoff + s];
        end = meta[tokoff + s + 1];
        fcl = meta[tokoff + (S + 1) + s];
        srk = sr_key(sr, meta);
    }
    const bool early = OWN && !SEG && lpt;
    const int slot = early ? lslot : idx[s];
    // (with no flag array, a byte of idx stands in and the flag is ignored)
    const uint8_t hflag = early ? (uint8_t)lflag
                                : (has_init != nullptr ? has_init : reinterpret_cast<const uint8_t *>(idx))[s];
    __builtin_amdgcn_sched_barrier(0);
    c0 = c0 < max_chunks ? c0 : max_chunks;
    c1 = c1 < max_chunks ? c1 : max_chunks;
    c1 = c1 > c0 ? c1 : c0;
    end = end > first ? end : first;
    fcl = fcl < 1 ? 1 : (fcl > Q ? Q : fcl);
    // this block's chunks lo .. hi - 1: all of the sequence's, or segment b of
    // min(nseg, chunks) near-equal segments (a sequence with no chunk has one)
    int lo = c0, hi = c1;
    if constexpr (SEG) {
        const int n = c1 - c0;
        const int ns = n < nsg ? (n > 1 ? n : 1) : nsg;
        if (b >= ns) return;   // (uniform over the block, before any barrier)
        lo = c0 + b * n / ns;
        hi = c0 + (b + 1) * n / ns;
    }
    // chunk c of the sequence: tokens first + off(c) .., at most cap(c) of them
    auto chunk_off = [&](int c) { return c == c0 ? 0 : fcl + (c - c0 - 1) * Q; };
    auto chunk_cap = [&](int c) { return c == c0 ? fcl : Q; };
    if constexpr (OWN) {
        // the per-sequence metadata (chunk_cu, clamped cu_seqlens, first-chunk
        // lengths), and after the last sequence the chunk slots no chunk fills
        if (h == 0 && q == 0 && b == 0) {
            if (tid == 0) {
                own.meta[s] = c0;
                own.meta[tokoff + s] = first;
                own.meta[tokoff + (S + 1) + s] = fcl;
                if (s == S - 1) {
                    own.meta[S] = total < max_chunks ? total : max_chunks;
                    own.meta[tokoff + S] = end;
                }
            }
            if (s == S - 1) {
                for (int cc = (total < max_chunks ? total : max_chunks) + tid; cc < max_chunks;
                     cc += 512) {
                    int32_t *m = own.meta + (S + 1) + 3 * cc;
                    m[0] = -1;
                    m[1] = 0;
                    m[2] = 0;
                }
            }
        }
    }
    const bool slot_ok = slot >= 0 && slot < num_slots;
    TS *cslot = cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN + run;

    // the initial state, through a resource that is empty when the block does
    // not start from it (no cached state, a bad slot, a later segment): zeros
    // then, and no memory read
    const bool want_init = slot_ok && has_init != nullptr && hflag != 0 && b == 0;
    const rsrc_t rinit = make_rsrc(cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN,
                                   want_init ? (uint32_t)(PN * sizeof(TS)) : 0u);
    float iv[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) buf_load4<TS>(rinit, (uint32_t)((run + 16 * j) * sizeof(TS)), iv[j]);
    f32x4 acc[2];

    // byte offsets inside a chunk's tiles (the same for every chunk)
    const uint32_t xrow = (uint32_t)H * P * 2, brow = (uint32_t)G * N * 2;
    uint32_t xo[Regs::kXV], bo[Regs::kBV], to[Regs::kBV];
#pragma unroll
    for (int k = 0; k < Regs::kXV; ++k) {
        const int u = tid + 512 * k;
        xo[k] = u < Q * 8 ? (uint32_t)(u >> 3) * xrow + 16 * (u & 7) : 0xfffffff0u;
    }
#pragma unroll
    for (int k = 0; k < Regs::kBV; ++k) {
        const int u = tid + 512 * k;
        bo[k] = u < Q * 8 ? (uint32_t)(u >> 3) * brow + 16 * (u & 7) : 0xfffffff0u;
        to[k] = u < Q * 8 ? (uint32_t)(u >> 3) * 4 : 0xfffffff0u;
    }

    // chunk c clamped to the block's range: its first token, and its token
    // count (0 past the block's last chunk)
    auto chunk_at = [&](int c, int &st) {
        const bool any = c < hi;
        c = c < hi ? c : hi - 1;
        c = c > lo ? c : lo;
        st = first + chunk_off(c);
        const int len = end - st < chunk_cap(c) ? end - st : chunk_cap(c);
        return any ? len : 0;
    };
    // Loads of chunk c's tiles through buffer resources that end at the chunk's
    // last row: rows past it read as zero. Past the last chunk (and for a
    // sequence with no chunk) every resource is empty and nothing is read.
    auto fetch_xv = [&](uint4 *xr, int c) {
        const bool any = c < hi;
        int st;
        const int len = chunk_at(c, st);
        const rsrc_t rx = make_rsrc(x + ((int64_t)st * H + h) * P,
                                    any ? (uint32_t)(len - 1) * xrow + P * 2 : 0u);
#pragma unroll
        for (int k = 0; k < Regs::kXV; ++k) xr[k] = buf_ld16(rx, xo[k]);
    };
    auto fetch_dt = [&](Regs &R, int c) {
        const bool any = c < hi;
        int st;
        const int len = chunk_at(c, st);
        c = c < hi ? c : hi - 1;
        c = c > lo ? c : lo;
        if constexpr (OWN) {
            // raw dt of position 64 w + lane for waves w < J first (their scan
            // runs before the x and B tiles are needed); the others read nothing
            const rsrc_t rt = make_rsrc(static_cast<const bf16 *>(own.dt) + (int64_t)st * H + h,
                                        any && wave < J ? (uint32_t)(len - 1) * H * 2 + 2 : 0u);
            R.dr = __builtin_amdgcn_raw_buffer_load_b16(rt, (uint32_t)(kWave * wave + lane) * H * 2,
                                                        0, 0);
        } else {
            const int64_t row = ((int64_t)h * max_chunks + c) * Q;
            const rsrc_t rc = make_rsrc(cum + row, any ? (uint32_t)len * 4 : 0u);
            // (the cumsum at the chunk's last token first: a vector load, since a
            // scalar one would share its wait counter with the LDS reads of the
            // MFMA phase and stall them on global latency)
            R.cl = buf_ldf(rc, (uint32_t)(len - 1) * 4);
        }
    };
    auto fetch_b = [&](Regs &R, int c) {
        const bool any = c < hi;
        int st;
        const int len = chunk_at(c, st);
        c = c < hi ? c : hi - 1;
        c = c > lo ? c : lo;
        const rsrc_t rb = make_rsrc(B + ((int64_t)st * G + g) * N + n0,
                                    any ? (uint32_t)(len - 1) * brow + NSL * 2 : 0u);
#pragma unroll
        for (int k = 0; k < Regs::kBV; ++k) {
            R.b[k] = buf_ld16(rb, bo[k]);
            if constexpr (!OWN) {
                const int64_t row = ((int64_t)h * max_chunks + c) * Q;
                const rsrc_t rc = make_rsrc(cum + row, any ? (uint32_t)len * 4 : 0u);
                const rsrc_t rd = make_rsrc(dtc + row, any ? (uint32_t)len * 4 : 0u);
                R.cm[k] = buf_ldf(rc, to[k]);
                R.dt[k] = buf_ldf(rd, to[k]);
            }
        }
    };

    // OWN: wave w < J scans dt * A_h over positions 64 w .. + 63 of chunk c
    // (fetched into R) into the pads of those x rows (prefix sum within the
    // 64-position block, dt; positions past the chunk's end add nothing and
    // hold dt 0) and the block's total into the pad of row w; the staging of
    // the step that folds chunk c chains the blocks (cum_at).
    auto scan_chunk = [&](const Regs &R, int c) {
        if (wave >= J) return;
        int st;
        const int len = chunk_at(c, st);
        const int i = kWave * wave + lane;
        float v = __uint_as_float(R.dr << 16);
        if (own.tf.on) v = dt_transform(own.tf, v, bh);
        v = i < len ? v : 0.0f;
        const float incl = wave_inclusive_sum(v * Ah, lane);
        if (i < Q) {
            float2 cd;
            cd.x = incl;
            cd.y = v;
            *reinterpret_cast<float2 *>(xs + i * LDX + P) = cd;
        }
        if (lane == kWave - 1) reinterpret_cast<float *>(xs + wave * LDX + P)[2] = incl;
    };
    // cum at position t of the chunk staged in xs (after the barrier that
    // follows scan_chunk): the totals of the blocks before t's, then its own
    // prefix sum; also its dt. The running sums of the block totals are read
    // from the pads once per step (read_boff), in the order the cumsum kernel
    // adds them.
    float boff[J];   // the totals of the blocks before block j
    auto read_boff = [&]() {
        boff[0] = 0.0f;
#pragma unroll
        for (int j = 1; j < J; ++j) {
            const float tj = reinterpret_cast<const float *>(xs + (j - 1) * LDX + P)[2];
            boff[j] = j == 1 ? tj : boff[j - 1] + tj;
        }
    };
    auto cum_at = [&](int t, float &dtv) {
        const float2 cd = *reinterpret_cast<const float2 *>(xs + t * LDX + P);
        dtv = cd.y;
        const int jb = t >> 6;
        float off = 0.0f;
#pragma unroll
        for (int j = 1; j < J; ++j) off = jb == j ? boff[j] : off;
        return jb == 0 ? cd.x : off + cd.x;
    };

    // one iteration: the step's stores, then stage chunk c into LDS - x from the
    // register set xcur, refilled with chunk c + 2 (the two sets alternate), B
    // from R.b, refilled with chunk c + 1, dt one chunk ahead too - then fold
    // chunk c into the running state. An empty sequence makes one pass over zero
    // tiles (it changes nothing) with its stores switched off.
    float F = 0.0f;   // log decay from the block's first chunk to chunk c
    auto step = [&](Regs &R, uint4 *xcur, int c) {
        const bool live = c < hi;
        const int st = first + chunk_off(c);
        const int len = end - st < chunk_cap(c) ? end - st : chunk_cap(c);
        __syncthreads();   // the previous chunk's MFMA reads of xs / bs are done
        // (OWN: the cumsum at the chunk's last token from the pads; an empty
        // chunk's pads hold zeros)
        float cl = R.cl;
        if constexpr (OWN) {
            read_boff();
            float unused;
            cl = cum_at(len > 0 ? len - 1 : 0, unused);
        }
        // Every store of the step is issued here, before the next chunk's loads:
        // the memory operations issued after those loads are then only loads,
        // which the compiler counts exactly, and its waits for them never wait
        // for a store (stores that depend on the block or the chunk would make
        // it count conservatively). acc still holds the state entering chunk c,
        // which is also the checkpoint of chunk c - 1.
        if (live) {
            const int64_t off = ((int64_t)c * H + h) * PN + run;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
                store4<bf16>(entering + off + 16 * j, v);
            }
            if constexpr (CKPT) {
                if (c > lo) {
                    const int64_t pk = off - (int64_t)H * PN;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
                        put4<TS>(ckpt + pk + 16 * j, v, srk, (uint64_t)(pk + 16 * j), kSrCkpt);
                    }
                }
            }
            if constexpr (OWN) {
                // slice 0 publishes the chunk's cumsum and dt rows (thread t < Q:
                // position t), head 0 its (sequence, start, length)
                if (q == 0) {
                    if (tid < Q) {
                        float dtt;
                        const float cmt = cum_at(tid, dtt);
                        const int64_t row = ((int64_t)h * max_chunks + c) * Q;
                        own.cum[row + tid] = cmt;
                        own.dtc[row + tid] = dtt;
                    }
                    if (h == 0 && tid == 0) {
                        int32_t *m = own.meta + (S + 1) + 3 * c;
                        m[0] = s;
                        m[1] = st;
                        m[2] = len;
                    }
                }
            }
        }
        if constexpr (SEG) {
            if (live && q == 0 && tid == 0) {
                seg_F[(int64_t)h * max_chunks + c] = F;
                if (h == 0) seg_I[c] = b > 0 ? sb : -1;
            }
            F += cl;
        }
        // Staging (u < Q * 8 holds for every thread where 512 (k + 1) <= Q * 8; said
        // so at compile time, so that no path skips a staging and leaves its
        // registers counted as loads in flight)
        fetch_dt(R, c + 1);
#pragma unroll
        for (int k = 0; k < Regs::kXV; ++k) {
            const int u = tid + 512 * k;
            if (512 * (k + 1) <= Q * 8 || u < Q * 8) st16(xs + (u >> 3) * LDX + 8 * (u & 7), xcur[k]);
        }
        fetch_xv(xcur, c + 2);   // (x two chunks ahead, in the set just staged)
#pragma unroll
        for (int k = 0; k < Regs::kBV; ++k) {
            const int u = tid + 512 * k;
            if (512 * (k + 1) <= Q * 8 || u < Q * 8) {
                const int t = u >> 3;
                float cmt, dtt;
                if constexpr (OWN) {
                    cmt = cum_at(t, dtt);
                } else {
                    cmt = R.cm[k];
                    dtt = R.dt[k];
                }
                const float w = t < len ? __expf(cl - cmt) * dtt : 0.0f;
                const uint32_t w4[4] = {R.b[k].x, R.b[k].y, R.b[k].z, R.b[k].w};
                float f[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f[2 * i] = __uint_as_float(w4[i] << 16) * w;
                    f[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u) * w;
                }
                Vec16<bf16>::store(bs + t * LDB + 8 * (u & 7), f);
            }
        }
        const float decay = __expf(cl);

        fetch_b(R, c + 1);
        __syncthreads();

#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] *= decay;
        // K steps of 32 tokens, software-pipelined: the fragments of step ks + 1
        // are requested before the MFMAs of step ks
        const int nk = (len + 31) >> 5;
        bf16x8 xf = mfma_frag_tr_split(xs, LDX, 0, 16 * pw, lane);
        bf16x8 bf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = mfma_frag_tr_split(bs, LDB, 0, 32 * nh + 16 * j, lane);
        for (int ks = 1; ks < nk; ++ks) {
            const bf16x8 xn = mfma_frag_tr_split(xs, LDX, 32 * ks, 16 * pw, lane);
            bf16x8 bn[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bn[j] = mfma_frag_tr_split(bs, LDB, 32 * ks, 32 * nh + 16 * j, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], xf, acc[j], 0, 0, 0);
            xf = xn;
            bf[0] = bn[0];
            bf[1] = bn[1];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], xf, acc[j], 0, 0, 0);
        if constexpr (OWN) scan_chunk(R, c + 1);   // (read after the next step's first barrier)
    };

    // The first chunk's tiles are requested together with the initial state; the
    // loop body runs at least once, so no branch separates these loads from their
    // use and the compiler's wait counts stay exact.
    Regs R;
    uint4 x2[Regs::kXV];
    fetch_dt(R, lo);
    fetch_xv(R.x, lo);
    fetch_b(R, lo);
    fetch_xv(x2, lo + 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (OWN) scan_chunk(R, lo);
    const bool read_init = slot_ok && has_init != nullptr && hflag != 0 && b == 0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = read_init ? iv[j][e] : 0.0f;
    int c = lo;
    do {
        step(R, R.x, c);
        if (++c >= hi) break;
        step(R, x2, c);
    } while (++c < hi);
    if constexpr (CKPT) {
        // the last chunk's checkpoint (the others were written one step later,
        // as the state entering the next chunk)
        if (hi > lo) {
            const int64_t pk = ((int64_t)(hi - 1) * H + h) * PN + run;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
                put4<TS>(ckpt + pk + 16 * j, v, srk, (uint64_t)(pk + 16 * j), kSrCkpt);
            }
        }
    }

    if constexpr (SEG) {
        // the segment's local final state and total decay, for the carry step
        if (q == 0 && tid == 0) seg_L[(int64_t)sb * H + h] = F;
        float *fin = seg_fin + ((int64_t)sb * H + h) * PN + run;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
            store4<float>(fin + 16 * j, v);
        }
    } else if (slot_ok) {
        const int64_t fo = ((int64_t)slot * H + h) * PN + run;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
            put4<TS>(cslot + 16 * j, v, srk, (uint64_t)(fo + 16 * j), kSrFinal);
        }
    }
}

// The fused state kernel for batches of short sequences (no segments):
// persistent blocks, each walking several (sequence, head, slice) items in the
// same head-major order, with the one-chunk-ahead prefetch crossing item
// boundaries. While an item's last chunk is folded in, the next item's initial
// state and first tiles are in flight, and its metadata was requested one item
// earlier, through vector loads (a scalar load in the loop would share its wait
// counter with the MFMA phase's LDS reads). What the single-item kernel pays
// per block - metadata, then the state and tiles, then the stores - is paid
// once per block instead of once per item. Same arithmetic, same outputs.
template <int Q, bool CKPT, typename TS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void state_scan_multi_kernel(
    int S, int H, int G, int max_chunks, int num_slots, const bf16 *__restrict__ x,
    const bf16 *__restrict__ B, const int32_t *__restrict__ meta, const float *__restrict__ cum,
    const float *__restrict__ dtc, TS *cache, const int32_t *__restrict__ idx,
    const uint8_t *__restrict__ has_init, bf16 *__restrict__ entering, TS *__restrict__ ckpt,
    SrCtx sr)
{
    constexpr int P = 64, N = 128, NSL = kScanNSL, NS = N / NSL;
    constexpr int LDX = kScanLDX, LDB = kScanLDB;
    typedef StateScanRegs<Q> Regs;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *xs = reinterpret_cast<bf16 *>(smem);   // [Q][LDX]  x_t
    bf16 *bs = xs + Q * LDX;                     // [Q][LDB]  w_t B_t (slice columns)

    // items in logical order (h S + s) NS + q; XCD x owns one contiguous range of
    // them and its blocks walk that range with a stride of their count
    const int nitems = S * H * NS;
    const int xcd = blockIdx.x % kXcds, bslot = blockIdx.x / kXcds;
    const int nbx = ((int)gridDim.x - xcd + kXcds - 1) / kXcds;
    const int qx = nitems / kXcds, rx_ = nitems % kXcds;
    const int ibase = xcd < rx_ ? xcd * (qx + 1) : rx_ * (qx + 1) + (xcd - rx_) * qx;
    const int icnt = qx + (xcd < rx_ ? 1 : 0);
    const int nmine = bslot < icnt ? (icnt - bslot + nbx - 1) / nbx : 0;
    if (nmine == 0) return;   // (uniform over the block, before any barrier)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int pw = wave & 3, nh = wave >> 2;
    const int PN = P * N;
    // this lane's state elements: row 16 pw + r16, columns n0 + 32 nh + 16 j + 4 kg + 0..3
    const int64_t run0 = (int64_t)(16 * pw + r16) * N + 32 * nh + 4 * kg;
    const int tokoff = (S + 1) + 3 * max_chunks;
    const SrKey srk = sr_key(sr, meta);

    // an item's metadata as raw vector loads (clamped to the block's last item)
    const rsrc_t rmeta = make_rsrc(meta, (uint32_t)(2 * (S + 1) + 3 * max_chunks + S) * 4u);
    const rsrc_t ridx = make_rsrc(idx, (uint32_t)S * 4u);
    const rsrc_t rflag = make_rsrc(has_init, has_init != nullptr ? (uint32_t)S : 0u);
    struct MetaRaw {
        float c0, c1, first, end, fcl, slot;
        uint32_t flag;
    };
    auto item_id = [&](int k) { return ibase + bslot + (k < nmine ? k : nmine - 1) * nbx; };
    auto meta_load = [&](MetaRaw &m, int k) {
        const int s = (item_id(k) / NS) % S;
        m.c0 = buf_ldf(rmeta, (uint32_t)s * 4);
        m.c1 = buf_ldf(rmeta, (uint32_t)(s + 1) * 4);
        m.first = buf_ldf(rmeta, (uint32_t)(tokoff + s) * 4);
        m.end = buf_ldf(rmeta, (uint32_t)(tokoff + s + 1) * 4);
        m.fcl = buf_ldf(rmeta, (uint32_t)(tokoff + S + 1 + s) * 4);
        m.slot = buf_ldf(ridx, (uint32_t)s * 4);
        m.flag = __builtin_amdgcn_raw_buffer_load_b8(rflag, (int)s, 0, 0);
    };
    struct Item {
        int h, g, n0, lo, hi, first, end, fcl;
        int64_t run;
        bool slot_ok, read_init;
        int slot;
    };
    auto rfl = [](float v) { return __builtin_amdgcn_readfirstlane(__float_as_int(v)); };
    auto make_item = [&](const MetaRaw &m, int k) {
        Item it;
        const int lb = item_id(k);
        it.h = lb / (NS * S);
        it.g = it.h / (H / G);
        it.n0 = (lb % NS) * NSL;
        it.run = run0 + it.n0;
        int c0 = rfl(m.c0), c1 = rfl(m.c1);
        c0 = c0 < max_chunks ? c0 : max_chunks;
        c1 = c1 < max_chunks ? c1 : max_chunks;
        it.lo = c0;
        it.hi = c1 > c0 ? c1 : c0;
        it.first = rfl(m.first);
        const int end = rfl(m.end);
        it.end = end > it.first ? end : it.first;
        const int fcl = rfl(m.fcl);
        it.fcl = fcl < 1 ? 1 : (fcl > Q ? Q : fcl);
        it.slot = rfl(m.slot);
        it.slot_ok = it.slot >= 0 && it.slot < num_slots;
        it.read_init = it.slot_ok && has_init != nullptr &&
                       __builtin_amdgcn_readfirstlane((int)m.flag) != 0;
        return it;
    };
    auto chunk_off = [](const Item &it, int c) { return c == it.lo ? 0 : it.fcl + (c - it.lo - 1) * Q; };
    auto chunk_cap = [](const Item &it, int c) { return c == it.lo ? it.fcl : Q; };
    auto chunk_len = [&](const Item &it, int c) {
        const int st = it.first + chunk_off(it, c);
        const int cap = chunk_cap(it, c);
        return it.end - st < cap ? it.end - st : cap;
    };

    // byte offsets inside a chunk's tiles (the same for every chunk)
    const uint32_t xrow = (uint32_t)H * P * 2, brow = (uint32_t)G * N * 2;
    uint32_t xo[Regs::kXV], bo[Regs::kBV], to[Regs::kBV];
#pragma unroll
    for (int k = 0; k < Regs::kXV; ++k) {
        const int u = tid + 512 * k;
        xo[k] = u < Q * 8 ? (uint32_t)(u >> 3) * xrow + 16 * (u & 7) : 0xfffffff0u;
    }
#pragma unroll
    for (int k = 0; k < Regs::kBV; ++k) {
        const int u = tid + 512 * k;
        bo[k] = u < Q * 8 ? (uint32_t)(u >> 3) * brow + 16 * (u & 7) : 0xfffffff0u;
        to[k] = u < Q * 8 ? (uint32_t)(u >> 3) * 4 : 0xfffffff0u;
    }
    // chunk c of item `it` through buffer resources ending at the chunk's last row
    // (rows past it read as zero); c outside the item's chunks reads nothing
    auto fetch = [&](Regs &R, const Item &it, int c) {
        const bool any = c < it.hi;
        c = c < it.hi ? c : it.hi - 1;
        c = c > it.lo ? c : it.lo;
        const int st = it.first + chunk_off(it, c);
        int len = chunk_len(it, c);
        len = any ? len : 0;
        const rsrc_t rx = make_rsrc(x + ((int64_t)st * H + it.h) * P,
                                    any ? (uint32_t)(len - 1) * xrow + P * 2 : 0u);
        const rsrc_t rb = make_rsrc(B + ((int64_t)st * G + it.g) * N + it.n0,
                                    any ? (uint32_t)(len - 1) * brow + NSL * 2 : 0u);
        const int64_t row = ((int64_t)it.h * max_chunks + c) * Q;
        const rsrc_t rc = make_rsrc(cum + row, any ? (uint32_t)len * 4 : 0u);
        const rsrc_t rd = make_rsrc(dtc + row, any ? (uint32_t)len * 4 : 0u);
        R.cl = buf_ldf(rc, (uint32_t)(len - 1) * 4);
#pragma unroll
        for (int k = 0; k < Regs::kXV; ++k) R.x[k] = buf_ld16(rx, xo[k]);
#pragma unroll
        for (int k = 0; k < Regs::kBV; ++k) {
            R.b[k] = buf_ld16(rb, bo[k]);
            R.cm[k] = buf_ldf(rc, to[k]);
            R.dt[k] = buf_ldf(rd, to[k]);
        }
    };
    // an item's initial state (slot 0 stands in for a bad slot; selected later)
    auto init_load = [&](float (&iv)[2][4], const Item &it) {
        const TS *cs = cache + ((int64_t)(it.slot_ok ? it.slot : 0) * H + it.h) * PN + it.run;
#pragma unroll
        for (int j = 0; j < 2; ++j) load4<TS>(cs + 16 * j, iv[j]);
    };

    MetaRaw mnext, mnext2;
    meta_load(mnext, 0);
    Item cur = make_item(mnext, 0);
    meta_load(mnext, 1);
    float iv[2][4];
    init_load(iv, cur);
    Regs R;
    fetch(R, cur, cur.lo);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = cur.read_init ? iv[j][e] : 0.0f;

    for (int k = 0; k < nmine; ++k) {
        const bool have_next = k + 1 < nmine;
        const Item nxt = make_item(mnext, k + 1);   // (the last item again when there is none)
        // the metadata of the item after the next (requested before this item's
        // tile loads, so it has arrived when those are waited for)
        meta_load(mnext2, k + 2);
        // an empty sequence makes one pass over zero tiles with its stores off
        const int cend = cur.hi > cur.lo ? cur.hi : cur.lo + 1;
        for (int c = cur.lo; c < cend; ++c) {
            const bool live = c < cur.hi;
            const int len = chunk_len(cur, c);
            // rows the MFMA phase reads: whole 32-token K steps, at least one (it
            // always runs the first, also for an empty item); rows past them are
            // left as they are (items here are mostly short)
            const int rows = len > 32 ? ((len + 31) >> 5) << 5 : 32;
            __syncthreads();   // the previous chunk's MFMA reads of xs / bs are done
#pragma unroll
            for (int kx = 0; kx < Regs::kXV; ++kx) {
                const int u = tid + 512 * kx;
                if (u < Q * 8 && (u >> 3) < rows) st16(xs + (u >> 3) * LDX + 8 * (u & 7), R.x[kx]);
            }
#pragma unroll
            for (int kb = 0; kb < Regs::kBV; ++kb) {
                const int u = tid + 512 * kb;
                if (u < Q * 8 && (u >> 3) < rows) {
                    const int t = u >> 3;
                    const float w = t < len ? __expf(R.cl - R.cm[kb]) * R.dt[kb] : 0.0f;
                    const uint32_t w4[4] = {R.b[kb].x, R.b[kb].y, R.b[kb].z, R.b[kb].w};
                    float f[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        f[2 * i] = __uint_as_float(w4[i] << 16) * w;
                        f[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u) * w;
                    }
                    Vec16<bf16>::store(bs + t * LDB + 8 * (u & 7), f);
                }
            }
            const float decay = __expf(R.cl);
            // the next chunk: this item's, or after its last the next item's first,
            // together with that item's initial state (one code path, no branch
            // around the loads)
            const bool last = c + 1 >= cend;
            const Item &tgt = last ? nxt : cur;
            float ivn[2][4];
            init_load(ivn, tgt);
            fetch(R, tgt, last ? nxt.lo : c + 1);
            __syncthreads();

            const int64_t off = ((int64_t)c * H + cur.h) * PN + cur.run;
            if (live) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
                    store4<bf16>(entering + off + 16 * j, v);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][e] *= decay;
            const int nk = (len + 31) >> 5;
            bf16x8 xf = mfma_frag_tr_split(xs, LDX, 0, 16 * pw, lane);
            bf16x8 bf[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[j] = mfma_frag_tr_split(bs, LDB, 0, 32 * nh + 16 * j, lane);
            for (int ks = 1; ks < nk; ++ks) {
                const bf16x8 xn = mfma_frag_tr_split(xs, LDX, 32 * ks, 16 * pw, lane);
                bf16x8 bn[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bn[j] = mfma_frag_tr_split(bs, LDB, 32 * ks, 32 * nh + 16 * j, lane);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], xf, acc[j], 0, 0, 0);
                xf = xn;
                bf[0] = bn[0];
                bf[1] = bn[1];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], xf, acc[j], 0, 0, 0);
            if constexpr (CKPT) {
                if (live) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float w[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
                        put4<TS>(ckpt + off + 16 * j, w, srk, (uint64_t)(off + 16 * j), kSrCkpt);
                    }
                }
            }
            if (last) {
                // the item's final state, then the next item's initial state
                if (cur.slot_ok) {
                    const int64_t fo = ((int64_t)cur.slot * H + cur.h) * PN + cur.run;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
                        put4<TS>(cache + fo + 16 * j, v, srk, (uint64_t)(fo + 16 * j), kSrFinal);
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[j][e] = nxt.read_init ? ivn[j][e] : 0.0f;
            }
        }
        if (!have_next) break;
        cur = nxt;
        mnext = mnext2;
    }
}

// Carry step of segmented state passing. A segment's chunk chain is linear in
// its starting state, so with h_b the true state entering segment b, fin_b the
// segment's final state from a zero start (the first segment's from the cached
// one) and L_b its total log decay:
//     h_1 = fin_0,   h_{b+1} = exp(L_b) h_b + fin_b,   final = h_ns.
// Grid: S * H * (P N / 1024) blocks of 256 threads, 4 consecutive state
// elements per thread; h_b (b >= 1) is kept in bf16 for the chunk scan, the
// final state goes to the cache slot as the unsegmented path writes it.
constexpr int kMaxSeg = 8;

template <typename TS>
__global__ __launch_bounds__(256) void state_carry_kernel(
    int S, int H, int PN, int nseg, int max_chunks, int num_slots,
    const int32_t *__restrict__ meta, const float *__restrict__ seg_fin,
    const float *__restrict__ seg_L, bf16 *__restrict__ carry, TS *cache,
    const int32_t *__restrict__ idx, SrCtx sr)
{
    const int bx = blockIdx.x;
    const int per = PN / 1024;
    const int e0 = (bx % per) * 1024 + 4 * threadIdx.x;
    const int h = (bx / per) % H, s = bx / (per * H);
    int c0 = meta[s], c1 = meta[s + 1];
    const int slot = idx[s];
    const SrKey srk = sr_key(sr, meta);
    c0 = c0 < max_chunks ? c0 : max_chunks;
    c1 = c1 < max_chunks ? c1 : max_chunks;
    const int n = c1 > c0 ? c1 - c0 : 0;
    const int ns = n < nseg ? (n > 1 ? n : 1) : nseg;
    // Every segment's values are requested before the chain starts, through
    // buffer resources that end at the sequence's last segment: entries past it
    // read as zero (no decay, nothing added) and stores there are dropped, so the
    // chain has no branch and one wait covers all the loads.
    const int64_t sq = (int64_t)s * nseg * H;
    const rsrc_t rf = make_rsrc(seg_fin + sq * PN, (uint32_t)((int64_t)ns * H * PN * 4));
    const rsrc_t rl = make_rsrc(seg_L + sq, (uint32_t)(ns * H * 4));
    const rsrc_t rc = make_rsrc(carry + sq * PN, (uint32_t)((int64_t)ns * H * PN * 2));
    float fin[kMaxSeg][4], L[kMaxSeg];
#pragma unroll
    for (int b = 0; b < kMaxSeg; ++b) {
        const uint32_t eo = (uint32_t)((b * H + h) * PN + e0);
        const uint4 w = buf_ld16(rf, eo * 4);
        fin[b][0] = __uint_as_float(w.x);
        fin[b][1] = __uint_as_float(w.y);
        fin[b][2] = __uint_as_float(w.z);
        fin[b][3] = __uint_as_float(w.w);
        L[b] = buf_ldf(rl, (uint32_t)(b * H + h) * 4);
    }
    float v[4] = {fin[0][0], fin[0][1], fin[0][2], fin[0][3]};
#pragma unroll
    for (int b = 1; b < kMaxSeg; ++b) {
        buf_st8(rc, (uint32_t)((b * H + h) * PN + e0) * 2, pack_bf16x4(v));
        const float d = __expf(L[b]);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = d * v[i] + fin[b][i];
    }
    // (the chain completes here, not inside the branch below, which would put
    // the last segment's loads after it)
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
    if (slot >= 0 && slot < num_slots) {
        const int64_t fo = ((int64_t)slot * H + h) * PN + e0;
        put4<TS>(cache + fo, v, srk, (uint64_t)fo, kSrFinal);
    }
}

// Chunk scan, bf16, P = 64, N = 128. Grid: max_chunks * H blocks of 2 Q threads
// (Q / 32 waves), logical order (chunk, head). Wave w owns the 16-row tiles w and
// Q / 16 - 1 - w, which balances the causal work.
//
// The segment decay exp(cum_i - cum_j) is split at R_k, the cumsum at the last
// position of the 32-token K block k that holds j:
//     exp(cum_i - cum_j) dt_j = exp(cum_i - R_k) * [exp(R_k - cum_j) dt_j]
// The bracket depends on j only; it scales x once per block while the x tile is
// staged (B operand x'_j). What remains per A element is the CB value times
// one per-(row, K block) factor: one exponential per lane per K step instead
// of eight. Within a block both factors stay in [exp(-span), exp(span)], span
// = |cum| change over the block; a block whose span exceeds kMaxSpan (where
// float32/bf16 range could be lost) is computed with the exact per-element
// exponentials on unscaled x instead. When the whole chunk's span fits, one
// reference serves every block (R = cum at the chunk's end): x' carries
// exp(R - cum_j) dt_j, A is CB exactly as stored (no arithmetic per K step),
// and each output row is scaled once by exp(cum_i - R) after the loop.
//   acc  = sum_j A_ij x'_j,   A_ij = CB[i,j] exp(cum_i - R_k) [j <= i]    (MFMA)
//   acc += (exp(cum_i) C_i) . H_in^T                                        (MFMA)
//   y_i  = acc + D_h x_i
// CB fragments (one contiguous 1 KiB wave load per K step) are requested
// before the staging barrier; y leaves through a per-wave LDS tile
// as 16-byte row stores.
constexpr float kMaxSpan = 60.0f;    // natural-log units
constexpr int kScanLDR = 20;         // p-major y tile pitch (bf16) of the epilogue
constexpr int kScanXLD = 80;         // x' row pitch (bf16): 40 dwords, conflict-free transpose reads

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// CB fragments of one row tile (MFMA fragment order, cb_frag_offset): K steps
// 0 .. nk-1, one contiguous 1 KiB wave load each.
template <int K>
__device__ __forceinline__ void load_cb_frags(const bf16 *CBc, int Q, int rt, int lane, int nk,
                                              uint4 *f)
{
    const bf16 *base = CBc + ((int64_t)rt * (Q >> 5) * 64 + lane) * 8;
    // steps past nk load step nk - 1 again (never used): no branch around a load
    const int last = nk > 0 ? nk - 1 : 0;
#pragma unroll
    for (int ks = 0; ks < K; ++ks) f[ks] = ld16(base + (int64_t)(ks < last ? ks : last) * 512);
}

// One 16-row tile of the chunk scan (rows i0 .. i0 + 15) for one wave; see the
// kernel comment. When `prefetch_next`, the CB fragments of the next tile
// (row tile nrt, nnk steps) are requested after this tile's intra-chunk loop.
template <int Q, int K, int KN>
__device__ __forceinline__ void scan_row_tile(
    int i0, int nk, const uint4 *cbf, bool exact, bool single, float rs, int len, int lane,
    rsrc_t rc, uint32_t crow, const float *scum, const float *sdt, const bf16 *xs, const bf16 *hs,
    bf16 *yw, rsrc_t rx, uint32_t xrow, int H, float Dh, bf16 *yout, const bf16 *CBc, int nrt,
    int nnk, uint4 *ncf, bool prefetch_next, const uint4 *xe_pre)
{
    constexpr int P = 64, N = 128, LDX = kScanXLD, LDH = N + 8;
    if (nk == 0) {
        if (prefetch_next) load_cb_frags<KN>(CBc, Q, nrt, lane, nnk, ncf);
        return;
    }
    const int r16 = lane & 15, kg = lane >> 4;
    const int i = i0 + r16;
    const float ci2 = scum[i];

    uint4 cr[N / 32];                    // C rows of the state term (raw bf16 A operand)
#pragma unroll
    for (int kk = 0; kk < N / 32; ++kk)
        cr[kk] = buf_ld16(rc, (uint32_t)i * crow + 64 * kk + 16 * kg);   // zeros past len
    // x of the D x term: row r16, p = 32 k + 8 kg + 0..7 (requested in the prologue)
    const uint4 xe[2] = {xe_pre[0], xe_pre[1]};

    f32x4 acc[P / 16];
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) acc[pt] = zero4();

#pragma unroll
    for (int ks = 0; ks < K; ++ks) {
        if (ks < nk) {
            const int j0 = 32 * ks;
            const float cbv[8] = {bf16_lo(cbf[ks].x), bf16_hi(cbf[ks].x), bf16_lo(cbf[ks].y),
                                  bf16_hi(cbf[ks].y), bf16_lo(cbf[ks].z), bf16_hi(cbf[ks].z),
                                  bf16_lo(cbf[ks].w), bf16_hi(cbf[ks].w)};
            bf16x8 af;
            if (single) {
                // whole-chunk reference: x' carries exp(R - cum_j) dt_j, the row factor
                // exp(cum_i - R) comes after the loop, so A is CB as stored
                af = __builtin_bit_cast(bf16x8, cbf[ks]);
            } else if (!exact) {
                // CB is zero above the diagonal (see bmm), and e is finite (at most
                // exp(kMaxSpan): the cumsum does not increase in this mode): no mask
                const float e = __builtin_amdgcn_exp2f(ci2 - scum[j0 + 31 < Q ? j0 + 31 : Q - 1]);
#pragma unroll
                for (int v = 0; v < 8; ++v) af[v] = static_cast<bf16>(cbv[v] * e);
            } else {
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const int j = j0 + 4 * kg + (v & 3) + ((v >> 2) << 4);
                    const float m = cbv[v] * __builtin_amdgcn_exp2f(ci2 - scum[j]) * sdt[j];
                    af[v] = static_cast<bf16>(j <= i ? m : 0.0f);
                }
            }
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                const bf16x8 bf = mfma_frag_tr_split(xs, LDX, j0, 16 * pt, lane);
                acc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[pt], 0, 0, 0);
            }
        }
    }
    if (prefetch_next) load_cb_frags<KN>(CBc, Q, nrt, lane, nnk, ncf);

    // state term: acc2 = C . H_in^T on raw C, then each output row i gets
    // exp(cum_i) * acc2 (the lane's rows are i0 + 4 kg + v)
    f32x4 acc2[P / 16];
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) acc2[pt] = zero4();
#pragma unroll
    for (int kk = 0; kk < N / 32; ++kk) {
        const int n = 32 * kk + 8 * kg;
        const bf16x8 af = __builtin_bit_cast(bf16x8, cr[kk]);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const bf16x8 bf = *reinterpret_cast<const bf16x8 *>(hs + (16 * pt + r16) * LDH + n);
            acc2[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc2[pt], 0, 0, 0);
        }
    }
    float erow[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) erow[v] = __builtin_amdgcn_exp2f(scum[i0 + 4 * kg + v]);
    if (single) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float f = __builtin_amdgcn_exp2f(scum[i0 + 4 * kg + v] - rs);
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) acc[pt][v] *= f;
        }
    }
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[pt][v] += erow[v] * acc2[pt][v];

    // epilogue: the SSM part goes through the wave's LDS tile, stored p-major
    // (yw[p][r], r = row in the tile) with one 8-byte write of 4 rows per p tile,
    // and comes back with transpose reads as 8 consecutive p of one row (r16),
    // where D x is added from 16-byte x loads before the 16-byte store
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) {
        const float v4[4] = {acc[pt][0], acc[pt][1], acc[pt][2], acc[pt][3]};
        store4<bf16>(yw + (16 * pt + r16) * kScanLDR + 4 * kg, v4);
    }
    wave_lds_sync();
    // (the transpose reads run with every lane active: each lane's result is
    // gathered from words named by other lanes)
    bf16x8 sv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) sv[k] = mfma_frag_tr(yw, kScanLDR, 32 * k, 0, lane);
    if (i < len) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint4 su = __builtin_bit_cast(uint4, sv[k]), xv = xe[k];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, sw[4] = {su.x, su.y, su.z, su.w};
            float o[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[2 * q] = bf16_lo(sw[q]) + Dh * bf16_lo(xw[q]);
                o[2 * q + 1] = bf16_hi(sw[q]) + Dh * bf16_hi(xw[q]);
            }
            Vec16<bf16>::store(yout + (int64_t)i * H * P + 32 * k + 8 * kg, o);
        }
    }
    wave_lds_sync();
}

template <int Q, bool SEG, bool BYC>
__global__ __launch_bounds__(2 * Q) __attribute__((amdgpu_waves_per_eu(4)))
void chunk_scan_fast_kernel(
    int S, int H, int G, int max_chunks, const bf16 *__restrict__ x,
    const bf16 *__restrict__ C, const float *__restrict__ D, const int32_t *__restrict__ meta,
    const float *__restrict__ cum, const float *__restrict__ dtc, const bf16 *__restrict__ CB,
    const bf16 *__restrict__ entering, bf16 *__restrict__ y, const int32_t *__restrict__ seg_I,
    const float *__restrict__ seg_F, const bf16 *__restrict__ carry)
{
    constexpr int P = 64, N = 128, LDX = kScanXLD, LDH = N + 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16 *xs = reinterpret_cast<bf16 *>(smem);                // [Q][LDX]  x' (or x)
    bf16 *hs = xs + Q * LDX;                                   // [P][LDH]  entering state
    bf16 *ys = hs + P * LDH;                                   // [Q / 32][P][kScanLDR]
    float *scum = reinterpret_cast<float *>(ys + (Q / 32) * P * kScanLDR);  // [Q] cum * log2(e)
    float *sdt = scum + Q;                                     // [Q]
    // Chunks of 128 or more tokens (few state registers per thread): everything
    // that depends on the unit alone is requested before anything is waited on -
    // the chunk's metadata, its segment and decay, its cumsum and dt rows and the
    // entering state - so the start pays one memory latency instead of a chain of
    // them; what depends on the chunk's tokens or segment (x, C, CB, the carried
    // state) follows once the metadata is in. (No branch comes before those
    // requests, so the kernel's arguments are read in one batch.) Smaller chunks
    // keep the loads in the order of use: their many state registers per thread
    // would stay live across the start.
    constexpr bool kEarly = Q >= 128;
    // (the arguments read through vector loads or written, in registers before
    // the first scheduling barrier below: one batch of argument loads; the
    // metadata and segment arrays stay out of this, so that the compiler still
    // reads them through scalar loads)
    if constexpr (kEarly)
        asm volatile("" ::"s"(x), "s"(C), "s"(cum), "s"(dtc), "s"(CB), "s"(entering), "s"(y),
                     "s"(carry), "s"(S), "s"(H), "s"(G), "s"(max_chunks));

    // Unit (chunk c, head h). With BYC, the (chunk, group) pairs u = c G + g
    // are dealt to the XCDs as u mod 8, each with all heads of its group: every
    // XCD gets the same share of real chunks, whatever the padding of max_chunks
    // and however the chunk lengths vary along the batch (the grid is padded to
    // whole rounds of 8 pairs; the padding blocks leave at once, with kEarly
    // after requests that read nothing). Otherwise each XCD takes one contiguous range of
    // units in order c H + h. Either way the heads that read one (chunk,
    // group)'s C and CB share an L2.
    int h, c;
    bool pad = false;
    if constexpr (BYC) {
        const int hpg = H / G;
        const int slot = blockIdx.x / kXcds, m = slot / hpg;
        const int u = (int)(blockIdx.x % kXcds) + kXcds * m;
        c = u / G;
        h = (u - c * G) * hpg + (slot - m * hpg);
        pad = c >= max_chunks;
        c = pad ? max_chunks - 1 : c;
    } else {
        const int lb = xcd_logical_block(blockIdx.x, max_chunks * H);
        h = lb % H;
        c = lb / H;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int nthr = 2 * Q;
    constexpr int kHVec = P * N / 8 / nthr > 0 ? P * N / 8 / nthr : 1;
    const ChunkInfo ci = chunk_info(meta, S, c);
    // segmented state passing: the entering state is the stored local one plus
    // exp(F) times the segment's starting state (none in a first segment)
    int sid = -1;
    float sF = 0.0f;
    if constexpr (SEG) {
        sid = seg_I[c];
        sF = seg_F[(int64_t)h * max_chunks + c];
    }
    const float *cumrow = cum + ((int64_t)h * max_chunks + c) * Q;
    const float *dtrow = dtc + ((int64_t)h * max_chunks + c) * Q;
    const int iq = tid < Q ? tid : Q - 1;          // 2 Q threads: one position each
    const bf16 *hin = entering + ((int64_t)c * H + h) * P * N;
    float cmv, dtv;
    uint4 hr[kHVec];
    auto load_rows = [&]() {
        // (through resources that are empty for a padding block: nothing read)
        const rsrc_t rcm = make_rsrc(cumrow, pad ? 0u : (uint32_t)Q * 4);
        const rsrc_t rdt = make_rsrc(dtrow, pad ? 0u : (uint32_t)Q * 4);
        const rsrc_t rh = make_rsrc(hin, pad ? 0u : (uint32_t)(P * N * 2));
        cmv = buf_ldf(rcm, (uint32_t)iq * 4);
        dtv = buf_ldf(rdt, (uint32_t)iq * 4);
        __builtin_amdgcn_sched_barrier(0);   // (the scheduler would otherwise move them last)
#pragma unroll
        for (int k = 0; k < kHVec; ++k) {
            const int u = tid + nthr * k;
            hr[k] = buf_ld16(rh, (uint32_t)((u >> 4) * N + 8 * (u & 15)) * 2);
        }
    };
    if constexpr (kEarly) {
        load_rows();
        __builtin_amdgcn_sched_barrier(0);
        if (pad || ci.len <= 0) {
            // (consumed on this path too, so that the compiler keeps the requests
            // ahead of the branch instead of moving them into the other path)
#pragma unroll
            for (int k = 0; k < kHVec; ++k) asm volatile("" ::"v"(hr[k].x));
            asm volatile("" ::"v"(cmv), "v"(dtv), "v"(sF), "v"(sid));
            return;
        }
    } else {
        if (pad || ci.len <= 0) return;
        load_rows();
    }
    const int g = h / (H / G);
    constexpr int kStepsB = Q / 32;                   // K steps of row tile B (at most)
    constexpr int kStepsA = Q / 64 > 0 ? Q / 64 : 1;  // K steps of row tile A (at most)
    const int len = ci.len;

    const int ntiles = (len + 15) / 16;
    const int rtA = wave, rtB = Q / 16 - 1 - wave;
    const int nkA = rtA < ntiles ? (16 * rtA + 15) / 32 + 1 : 0;
    const int nkB = rtB < ntiles ? (16 * rtB + 15) / 32 + 1 : 0;

    // stage cum, dt, the entering state and x' (or x in exact mode). x and C come
    // through buffer resources ending at the chunk's last row: rows past it read as
    // zeros, with no branch around the loads (a branch would make the compiler wait
    // on each load where the branches join)
    const uint32_t xrow = (uint32_t)H * P * 2, crow = (uint32_t)G * N * 2;
    const rsrc_t rx = make_rsrc(x + ((int64_t)ci.start * H + h) * P, (uint32_t)(len - 1) * xrow + P * 2);
    const rsrc_t rc = make_rsrc(C + ((int64_t)ci.start * G + g) * N, (uint32_t)(len - 1) * crow + N * 2);
    // requests in the order they are needed (the wait counter is in order), after
    // cum, dt and the entering state: the carried state, x, then the CB fragments
    // of the larger row tile B (tile A's follow later)
    uint4 hc[kHVec];
    if constexpr (SEG) {
        const bool has = sid >= 0;
        const rsrc_t rh = make_rsrc(carry + ((int64_t)(has ? sid : 0) * H + h) * P * N,
                                    has ? (uint32_t)(P * N * 2) : 0u);
#pragma unroll
        for (int k = 0; k < kHVec; ++k) {
            const int u = tid + nthr * k;
            hc[k] = buf_ld16(rh, (uint32_t)((u >> 4) * N + 8 * (u & 15)) * 2);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 xr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {        // Q rows x 8 vectors over 2 Q threads
        const int u = tid + nthr * k;
        xr[k] = buf_ld16(rx, (uint32_t)(u >> 3) * xrow + 16 * (u & 7));
    }
    const bf16 *CBc = CB + ((int64_t)c * G + g) * Q * Q;
    uint4 cbf[kStepsB];
    load_cb_frags<kStepsB>(CBc, Q, rtB, lane, nkB, cbf);
    // the x rows of both row tiles for the epilogue's D x term (row 16 rt + lane % 16,
    // p = 32 k + 8 (lane / 16) + 0..7), requested with the staging loads of the same
    // rows, while those lines are in flight or in L2 (zeros past len)
    uint4 xeB[2], xeA[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        xeB[k] = buf_ld16(rx, (uint32_t)(16 * rtB + (lane & 15)) * xrow + 64 * k + 16 * (lane >> 4));
        xeA[k] = buf_ld16(rx, (uint32_t)(16 * rtA + (lane & 15)) * xrow + 64 * k + 16 * (lane >> 4));
    }
    if constexpr (kEarly) __builtin_amdgcn_sched_barrier(0);   // (every request out first)
    scum[iq] = cmv * kLog2e;          // (threads past Q rewrite position Q - 1 with the
    sdt[iq] = dtv;                     //  same values: no branch, so the loads stay first)
#pragma unroll
    for (int k = 0; k < kHVec; ++k) {
        const int u = tid + nthr * k;
        bf16 *dst = hs + (u >> 4) * LDH + 8 * (u & 15);
        if constexpr (SEG) {
            const float ef = sid >= 0 ? __expf(sF) : 0.0f;
            const uint32_t a4[4] = {hr[k].x, hr[k].y, hr[k].z, hr[k].w};
            const uint32_t c4[4] = {hc[k].x, hc[k].y, hc[k].z, hc[k].w};
            float f[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[2 * i] = bf16_lo(a4[i]) + ef * bf16_lo(c4[i]);
                f[2 * i + 1] = bf16_hi(a4[i]) + ef * bf16_hi(c4[i]);
            }
            Vec16<bf16>::store(dst, f);
        } else {
            st16(dst, hr[k]);
        }
    }
    __syncthreads();
    // scaling factors of x: G_j = exp(R_k - cum_j) dt_j. The factored modes need a
    // cumsum that never increases (A_h dt_j <= 0, the decaying case) and block
    // spans of at most kMaxSpan: a factor exp(cum_i - R_k) with i past block k is
    // then at most 1, and at most exp(kMaxSpan) inside it. A chunk with a larger
    // span, or with any step where A_h dt_j > 0, takes the exact mode.
    bool big = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int t = (tid + nthr * k) >> 3;
        const float rk = scum[(t | 31) < Q ? (t | 31) : Q - 1];
        const float prev = t > 0 ? scum[t - 1] : 0.0f;
        big |= fabsf(rk - scum[t]) > kMaxSpan * kLog2e || scum[t] > prev;
    }
    const bool exact = __syncthreads_or(big) != 0;
    // whole-chunk reference when the chunk's decay span fits (the cumsum does not
    // increase here, so every factor is in [exp(-span), exp(span)]): R = cum at the
    // chunk's end (positions past it hold it)
    const float rs = scum[Q - 1];
    const bool single = !exact && scum[0] - rs <= kMaxSpan * kLog2e;
    // only the rows the intra-chunk MFMAs read (whole 32-token K steps up to the
    // chunk's last row); rows past them are left as they are
    const int xrows = ((len + 31) >> 5) << 5;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int u = tid + nthr * k;
        const int t = u >> 3, c8 = u & 7;
        uint4 v = xr[k];
        if (t >= xrows) continue;
        if (!exact) {
            const float rk = single ? rs : scum[(t | 31) < Q ? (t | 31) : Q - 1];
            const float gt = __builtin_amdgcn_exp2f(rk - scum[t]) *
                             sdt[t];
            float f[8];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = bf16_lo(w4[q]) * gt;
                f[2 * q + 1] = bf16_hi(w4[q]) * gt;
            }
            Vec16<bf16>::store(xs + t * LDX + 8 * c8, f);
        } else {
            st16(xs + t * LDX + 8 * c8, v);
        }
    }
    __syncthreads();

    const float Dh = D ? D[h] : 0.0f;
    bf16 *yw = ys + wave * P * kScanLDR;

    // tile B first (larger); tile A's CB fragments are requested once B's are consumed
    uint4 caf[kStepsA];
    scan_row_tile<Q, kStepsB, kStepsA>(16 * rtB, nkB, cbf, exact, single, rs, len, lane, rc, crow,
                                       scum, sdt,
                                       xs, hs, yw, rx, xrow, H, Dh,
                                       y + ((int64_t)ci.start * H + h) * P, CBc, rtA, nkA, caf,
                                       true, xeB);
    scan_row_tile<Q, kStepsA, kStepsA>(16 * rtA, nkA, caf, exact, single, rs, len, lane, rc, crow,
                                       scum, sdt,
                                       xs, hs, yw, rx, xrow, H, Dh,
                                       y + ((int64_t)ci.start * H + h) * P, CBc, 0, 0, caf, false,
                                       xeA);
}

// ===========================================================================
// Batches of short sequences in one launch. One block of four waves per
// (sequence, head) walks its sequence in sub-chunks of SUB (32 or 64) tokens, cut
// so that none crosses a chunk boundary (every checkpoint is then a sub-chunk's
// exit state), and does both halves of the scan for each sub-chunk: y from the
// intra-sub-chunk product, the state the sub-chunk enters with and D x; then
// the state it passes on. The initial state is read from the cache slot once
// and the final state written back to it: no cumsum, CB, entering or chunk
// state goes through HBM. Chunking is exact algebra, so the sub-chunk size
// changes results only by rounding.
//
// Per sub-chunk (len tokens, local cum = inclusive cumsum of dt A_h), wave w
// (rows past the sub-chunk leave a wave idle in (a)-(c)):
//   (a) CB^T tiles (j x i) for its row tile i in [16 w, 16 w + 16): B rows
//       times C rows over N; each output tile is half of a split-K A fragment
//       of (b), taken element by element as CB[i][j] exp(cum_i - cum_j) dt_j
//       for j <= i (exact exponentials, no decay factoring);
//   (b) y_i += sum_j A_ij x_j over its row tile, all 64 p;
//   (c) y_i += exp(cum_i) C_i . H_in^T (H_in in bf16 from LDS), + D_h x_i;
//   (d) its 16 state columns p in [16 w, 16 w + 16), all 128 n, in MFMA
//       accumulators across sub-chunks: H <- exp(cum_last) H
//       + sum_t (exp(cum_last - cum_t) dt_t B_t) x_t^T.
constexpr int kShortLDX = 72;    // x tile pitch (bf16)
constexpr int kShortLDB = 136;   // B tile and state tile pitch (bf16): 68 dwords, conflict-free
constexpr int kShortLDY = 72;    // y staging tile pitch (bf16)

template <int SUB, typename TS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void short_scan_kernel(
    int T, int S, int H, int G, int Q, int num_slots, const bf16 *__restrict__ x,
    const bf16 *__restrict__ dt, const float *__restrict__ A, const bf16 *__restrict__ B,
    const bf16 *__restrict__ C, const float *__restrict__ D, const int32_t *__restrict__ cu,
    TS *cache, const int32_t *__restrict__ idx, const uint8_t *__restrict__ has_init,
    bf16 *__restrict__ y, TS *__restrict__ ckpt, SrCtx sr, DtTf tf,
    const int32_t *__restrict__ prefix)
{
    constexpr int P = 64, N = 128, LDX = kShortLDX, LDB = kShortLDB, LDY = kShortLDY;
    static_assert(SUB == 32 || SUB == 64, "sub-chunks of 32 or 64 tokens");
    constexpr int KS = SUB / 32;           // 32-token K steps per sub-chunk
    __shared__ __attribute__((aligned(16))) bf16 xs[SUB * LDX];   // x_t (raw)
    __shared__ __attribute__((aligned(16))) bf16 bs[SUB * LDB];   // B_t (raw)
    // the entering state H_in[p][n] (bf16); after (c) the waves' y staging tiles
    __shared__ __attribute__((aligned(16))) bf16 hs[P * LDB];
    __shared__ int s_acc[4];

    // (sequence, head) in logical order (s G + g) (H / G) + h % (H / G): each XCD
    // takes a contiguous range, so the heads sharing a sequence's B and C rows sit
    // on one L2
    const int lb = xcd_logical_block(blockIdx.x, S * H);
    const int s = lb / H, h = lb - s * H;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int PN = P * N;

    int a = cu[s], b = cu[s + 1];
    a = clampi(a, 0, T);
    b = clampi(b, 0, T);
    b = b > a ? b : a;
    const int L = b - a;
    const int f = first_chunk_len(Q, prefix, s);     // tokens of the first chunk
    const int slot = idx[s];
    const bool slot_ok = slot >= 0 && slot < num_slots;
    const bool read_init = slot_ok && has_init != nullptr && has_init[s] != 0;
    const SrKey srk = sr_key_checked(sr);
    const float Ah = A[h];
    const float bias = tf.bias ? tf.bias[h] : 0.0f;
    const float Dh = D ? D[h] : 0.0f;

    // chunk_cu[s]: the first checkpoint row of this sequence (checkpoints only)
    int crow = 0;
    if (ckpt != nullptr) {
        int part = 0;
        for (int t = tid; t < s; t += 256) {
            const int ta = clampi(cu[t], 0, T), tb = clampi(cu[t + 1], 0, T);
            const int tl = tb > ta ? tb - ta : 0;
            const int tf_ = first_chunk_len(Q, prefix, t);
            part += tl == 0 ? 0 : (tl <= tf_ ? 1 : 1 + (tl - tf_ + Q - 1) / Q);
        }
        part = (int)group_sum((float)part, kWave);   // (exact: counts stay far below 2^24)
        if (lane == 0) s_acc[w] = part;
        __syncthreads();
        crow = s_acc[0] + s_acc[1] + s_acc[2] + s_acc[3];
    }

    // this lane's state elements (d): p = 16 w + r16, n = 16 nt + 4 kg + 0..3
    const int pcol = 16 * w + r16;
    TS *cslot = cache + ((int64_t)(slot_ok ? slot : 0) * H + h) * PN + (int64_t)pcol * N + 4 * kg;
    f32x4 hst[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        float v[4];
        load4<TS>(cslot + 16 * nt, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) hst[nt][e] = read_init ? v[e] : 0.0f;
    }

    const uint32_t xrow = (uint32_t)H * P * 2, nrow = (uint32_t)G * N * 2;
    // sub-chunks: never past a chunk boundary (the first chunk has f tokens, the
    // others Q), at most SUB tokens
    int pos = 0, chunk_end = f < L ? f : L, k = 0;
    while (pos < L) {
        const int len = chunk_end - pos < SUB ? chunk_end - pos : SUB;
        const int st = a + pos;
        // ---- loads: dt (one token per lane), x and B tiles, this wave's C rows
        const int tq = lane < len ? lane : len - 1;
        float dtv = to_f32(dt[(int64_t)(st + tq) * H + h]);
        const rsrc_t rx = make_rsrc(x + ((int64_t)st * H + h) * P, (uint32_t)(len - 1) * xrow + P * 2);
        const rsrc_t rb = make_rsrc(B + ((int64_t)st * G + g) * N, (uint32_t)(len - 1) * nrow + N * 2);
        const rsrc_t rc = make_rsrc(C + ((int64_t)st * G + g) * N, (uint32_t)(len - 1) * nrow + N * 2);
        uint4 xr[SUB / 32], br[SUB / 16], cfr[4];
#pragma unroll
        for (int q = 0; q < SUB / 32; ++q) {   // SUB rows x 8 vectors over 256 threads
            const int u = tid + 256 * q;
            xr[q] = buf_ld16(rx, (uint32_t)(u >> 3) * xrow + 16 * (u & 7));
        }
#pragma unroll
        for (int q = 0; q < SUB / 16; ++q) {   // SUB rows x 16 vectors
            const int u = tid + 256 * q;
            br[q] = buf_ld16(rb, (uint32_t)(u >> 4) * nrow + 16 * (u & 15));
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)         // C row 16 w + r16, n = 32 kk + 8 kg .. + 7
            cfr[kk] = buf_ld16(rc, (uint32_t)(16 * w + r16) * nrow + 64 * kk + 16 * kg);
        __builtin_amdgcn_sched_barrier(0);
        if (tf.on) dtv = dt_transform(tf, dtv, bias);
        dtv = lane < len ? dtv : 0.0f;        // (lanes past SUB: len <= SUB)
        const float cum = wave_inclusive_sum(dtv * Ah, lane);
        const float cl = __shfl(cum, len - 1);
        const float wt = __expf(cl - cum) * dtv;     // weight of token `lane` in the state

        __syncthreads();   // the previous sub-chunk's reads of xs, bs, hs are done
#pragma unroll
        for (int q = 0; q < SUB / 32; ++q) {
            const int u = tid + 256 * q;
            *reinterpret_cast<uint4 *>(xs + (u >> 3) * LDX + 8 * (u & 7)) = xr[q];
        }
#pragma unroll
        for (int q = 0; q < SUB / 16; ++q) {
            const int u = tid + 256 * q;
            *reinterpret_cast<uint4 *>(bs + (u >> 4) * LDB + 8 * (u & 15)) = br[q];
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const float v4[4] = {hst[nt][0], hst[nt][1], hst[nt][2], hst[nt][3]};
            store4<bf16>(hs + pcol * LDB + 16 * nt + 4 * kg, v4);
        }
        __syncthreads();

        // ---- (a) + (b): intra-sub-chunk product for row tile w
        const int i0 = 16 * w;
        f32x4 yacc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) yacc[pt] = zero4();
        if (i0 < len) {
            const int ii = i0 + r16;                 // this lane's row in the A fragments
            const float cum_i = __shfl(cum, ii);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (32 * ks > i0 + 15) break;        // (uniform over the wave)
                // CB^T tiles j in [32 ks, 32 ks + 16) and [32 ks + 16, 32 ks + 32)
                f32x4 cbt[2];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    cbt[half] = zero4();
                    const int j0 = 32 * ks + 16 * half;
                    if (j0 <= i0 + 15) {
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            const bf16x8 bfr = *reinterpret_cast<const bf16x8 *>(
                                bs + (j0 + r16) * LDB + 32 * kk + 8 * kg);
                            cbt[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                bfr, __builtin_bit_cast(bf16x8, cfr[kk]), cbt[half], 0, 0, 0);
                        }
                    }
                }
                // A fragment, split K order: v < 4 -> j = 32 ks + 4 kg + v,
                // v >= 4 -> j = 32 ks + 16 + 4 kg + v - 4
                bf16x8 af;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const int j = 32 * ks + 4 * kg + (v & 3) + ((v >> 2) << 4);
                    const float cj = __shfl(cum, j), dj = __shfl(dtv, j);
                    const float m = cbt[v >> 2][v & 3] * __expf(cum_i - cj) * dj;
                    af[v] = static_cast<bf16>(j <= ii ? m : 0.0f);
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x8 xf = mfma_frag_tr_split(xs, LDX, 32 * ks, 16 * pt, lane);
                    yacc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xf, yacc[pt], 0, 0, 0);
                }
            }
            // ---- (c): exp(cum_i) C_i . H_in^T, then D x (rows i0 + 4 kg + v, p = 16 pt + r16)
            f32x4 sacc[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) sacc[pt] = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x8 hf = *reinterpret_cast<const bf16x8 *>(
                        hs + (16 * pt + r16) * LDB + 32 * kk + 8 * kg);
                    sacc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, cfr[kk]), hf, sacc[pt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = i0 + 4 * kg + v;
                const float ei = __expf(__shfl(cum, i));
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const float xv = static_cast<float>(xs[i * LDX + 16 * pt + r16]);
                    yacc[pt][v] += ei * sacc[pt][v] + Dh * xv;
                }
            }
        }
        __syncthreads();   // every wave is done reading hs: it becomes the y staging area

        // ---- y: through this wave's staging tile as 16-byte row stores
        if (i0 < len) {
            bf16 *yw = hs + w * 16 * LDY;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    yw[(4 * kg + v) * LDY + 16 * pt + r16] = static_cast<bf16>(yacc[pt][v]);
            wave_lds_sync();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int r = (lane >> 3) + 8 * q, c8 = lane & 7;
                const uint4 v = *reinterpret_cast<const uint4 *>(yw + r * LDY + 8 * c8);
                if (i0 + r < len)
                    *reinterpret_cast<uint4 *>(y + ((int64_t)(st + i0 + r) * H + h) * P + 8 * c8) = v;
            }
        }

        // ---- (d): the state passed on, this wave's 16 columns p
        const float decay = __expf(cl);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) hst[nt][e] *= decay;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (32 * ks >= len) break;               // (uniform)
            float wv[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) wv[v] = __shfl(wt, 32 * ks + 4 * kg + (v & 3) + ((v >> 2) << 4));
            const bf16x8 xf = mfma_frag_tr_split(xs, LDX, 32 * ks, 16 * w, lane);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const bf16x8 braw = mfma_frag_tr_split(bs, LDB, 32 * ks, 16 * nt, lane);
                bf16x8 bw;
#pragma unroll
                for (int v = 0; v < 8; ++v) bw[v] = static_cast<bf16>(static_cast<float>(braw[v]) * wv[v]);
                hst[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw, xf, hst[nt], 0, 0, 0);
            }
        }
        pos += len;
        if (pos == chunk_end) {
            // the exit state of chunk k: its checkpoint
            if (ckpt != nullptr) {
                const int64_t off = ((int64_t)(crow + k) * H + h) * PN + (int64_t)pcol * N + 4 * kg;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const float v4[4] = {hst[nt][0], hst[nt][1], hst[nt][2], hst[nt][3]};
                    put4<TS>(ckpt + off + 16 * nt, v4, srk, (uint64_t)(off + 16 * nt), kSrCkpt);
                }
            }
            ++k;
            chunk_end = chunk_end + Q < L ? chunk_end + Q : L;
        }
    }
    if (slot_ok) {
        const int64_t fo = ((int64_t)slot * H + h) * PN + (int64_t)pcol * N + 4 * kg;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const float v4[4] = {hst[nt][0], hst[nt][1], hst[nt][2], hst[nt][3]};
            put4<TS>(cslot + 16 * nt, v4, srk, (uint64_t)(fo + 16 * nt), kSrFinal);
        }
    }
}

// ===========================================================================
// Launchers.
static inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

static inline bool use_fast(const PrefillDims &d) { return d.in_bf16 && d.P == 64 && d.N == 128; }

// Raise a kernel's dynamic LDS limit to what a launch needs (only needed above
// 64 KiB; the limit must leave room for the kernel's static LDS).
static void allow_lds(const void *fn, size_t bytes, size_t &raised_to)
{
    if (bytes > 65536 && bytes > raised_to) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
            hipSuccess)
            raised_to = bytes;
    }
}

template <typename TIn>
static void launch_cumsum_t(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                            int32_t *meta, float *cum, float *dto, hipStream_t st, const DtTf &tf)
{
    dim3 grid(d.max_chunks, (d.H + kCumsumHeadsPerBlock - 1) / kCumsumHeadsPerBlock);
    SSD_LAUNCH(d, "chunk_cumsum", chunk_cumsum_kernel<TIn>, grid, dim3(256), 0, st, d.T, d.S, d.H, d.Q,
                       d.max_chunks, static_cast<const TIn *>(dt), A, cu, meta, cum, dto, tf,
                       d.prefix);
}

template <typename TIn, int N>
static void launch_prep_t(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                          int32_t *meta, float *cum, float *dto, const void *B, const void *C,
                          void *CB, hipStream_t st, const DtTf &tf)
{
    const int HB = (d.H + kCumsumHeadsPerBlock - 1) / kCumsumHeadsPerBlock;
    dim3 grid(d.max_chunks, HB + d.G * (d.Q / 16));
    SSD_LAUNCH(d, "chunk_prep", (chunk_prep_kernel<TIn, N>), grid, dim3(256), 0, st, d.T, d.S, d.H, d.G, d.Q,
                       d.max_chunks, static_cast<const TIn *>(dt), A, cu, meta, cum, dto,
                       static_cast<const TIn *>(B), static_cast<const TIn *>(C),
                       static_cast<TIn *>(CB), tf, d.prefix);
}

void launch_chunk_prep(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                       int32_t *meta, float *cum, float *dto, const void *B, const void *C,
                       void *CB, void *stream, const DtTf &tf)
{
    if (d.max_chunks <= 0) return;
    hipStream_t st = as_stream(stream);
    if (d.in_bf16) {
        if (d.N == 128) launch_prep_t<bf16, 128>(d, dt, A, cu, meta, cum, dto, B, C, CB, st, tf);
        else launch_prep_t<bf16, 16>(d, dt, A, cu, meta, cum, dto, B, C, CB, st, tf);
    } else {
        if (d.N == 128) launch_prep_t<float, 128>(d, dt, A, cu, meta, cum, dto, B, C, CB, st, tf);
        else launch_prep_t<float, 16>(d, dt, A, cu, meta, cum, dto, B, C, CB, st, tf);
    }
}

void launch_chunk_cumsum(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                         int32_t *meta, float *cum, float *dto, void *stream, const DtTf &tf)
{
    if (d.max_chunks <= 0) return;
    if (d.in_bf16) launch_cumsum_t<bf16>(d, dt, A, cu, meta, cum, dto, as_stream(stream), tf);
    else launch_cumsum_t<float>(d, dt, A, cu, meta, cum, dto, as_stream(stream), tf);
}

template <typename TIn, int P, int N>
static void launch_state_t(const PrefillDims &d, const void *x, const void *B, const int32_t *meta,
                           const float *cum, const float *dtc, float *states, hipStream_t st)
{
    dim3 grid(d.H, d.max_chunks);
    SSD_LAUNCH(d, "chunk_state", (chunk_state_kernel<TIn, P, N>), grid, dim3(256), 0, st, d.S, d.H, d.G, d.Q,
                       d.max_chunks, static_cast<const TIn *>(x), static_cast<const TIn *>(B),
                       meta, cum, dtc, states);
}

template <typename TIn, int N>
static void launch_bmm_t(const PrefillDims &d, const void *B, const void *C, const int32_t *meta,
                         void *CB, hipStream_t st)
{
    dim3 grid(d.max_chunks, d.G, d.Q / 16);
    SSD_LAUNCH(d, "bmm_chunk", (bmm_kernel<TIn, N>), grid, dim3(256), 0, st, d.S, d.G, d.Q, d.max_chunks,
                       static_cast<const TIn *>(B), static_cast<const TIn *>(C), meta,
                       static_cast<TIn *>(CB));
}

template <typename TIn, int P, int N>
static size_t scan_smem(int Q)
{
    return sizeof(TIn) * ((size_t)P * padded<TIn>(Q) + (size_t)P * padded<TIn>(N)) +
           sizeof(float) * 2 * (size_t)Q;
}

template <typename TIn, int P, int N>
static void launch_scan_t(const PrefillDims &d, const void *x, const void *C, const float *D,
                          const int32_t *meta, const float *cum, const float *dtc, const void *CB,
                          const void *entering, void *y, hipStream_t st)
{
    dim3 grid(d.H, d.max_chunks);
    const size_t smem = scan_smem<TIn, P, N>(d.Q);
    static size_t raised = 0;
    allow_lds(reinterpret_cast<const void *>(&chunk_scan_kernel<TIn, P, N>), smem, raised);
    SSD_LAUNCH(d, "chunk_scan", (chunk_scan_kernel<TIn, P, N>), grid, dim3(256), smem, st, d.S, d.H, d.G,
                       d.Q, d.max_chunks, static_cast<const TIn *>(x), static_cast<const TIn *>(C),
                       D, meta, cum, dtc, static_cast<const TIn *>(CB),
                       static_cast<const TIn *>(entering), static_cast<TIn *>(y));
}

template <int Q>
static void launch_state_fast(const PrefillDims &d, const void *x, const void *B,
                              const int32_t *meta, const float *cum, const float *dtc,
                              float *states, hipStream_t st)
{
    const size_t smem = (size_t)Q * (2 * kFastLD * sizeof(bf16) + sizeof(float));
    static size_t raised = 0;
    allow_lds(reinterpret_cast<const void *>(&chunk_state_fast_kernel<Q>), smem, raised);
    const unsigned nblk = (unsigned)((int64_t)d.max_chunks * 2 * d.H);
    SSD_LAUNCH(d, "chunk_state", chunk_state_fast_kernel<Q>, dim3(nblk), dim3(256), smem, st, d.S, d.H, d.G,
                       d.max_chunks, static_cast<const bf16 *>(x), static_cast<const bf16 *>(B),
                       meta, cum, dtc, states);
}

template <int Q, bool SEG, bool BYC>
static void launch_scan_fast_b(const PrefillDims &d, const void *x, const void *C, const float *D,
                               const int32_t *meta, const float *cum, const float *dtc,
                               const void *CB, const void *entering, void *y, const SegBufs &seg,
                               unsigned nblk, hipStream_t st)
{
    const size_t smem = (size_t)Q * (kScanXLD * sizeof(bf16) + 2 * sizeof(float)) +
                        (size_t)64 * (128 + 8) * sizeof(bf16) +
                        (size_t)(Q / 32) * 64 * kScanLDR * sizeof(bf16);
    static size_t raised = 0;
    allow_lds(reinterpret_cast<const void *>(&chunk_scan_fast_kernel<Q, SEG, BYC>), smem, raised);
    SSD_LAUNCH(d, SEG ? "chunk_scan_segmented" : "chunk_scan", (chunk_scan_fast_kernel<Q, SEG, BYC>), dim3(nblk), dim3(2 * Q), smem, st, d.S,
                       d.H, d.G, d.max_chunks, static_cast<const bf16 *>(x),
                       static_cast<const bf16 *>(C), D, meta, cum, dtc,
                       static_cast<const bf16 *>(CB), static_cast<const bf16 *>(entering),
                       static_cast<bf16 *>(y), seg.I, seg.F, static_cast<const bf16 *>(seg.carry));
}

template <int Q, bool SEG>
static void launch_scan_fast_s(const PrefillDims &d, const void *x, const void *C, const float *D,
                               const int32_t *meta, const float *cum, const float *dtc,
                               const void *CB, const void *entering, void *y, const SegBufs &seg,
                               hipStream_t st)
{
    // (chunk, group)-interleaved XCD order once there are at least two pairs per XCD
    const int64_t pairs = (int64_t)d.max_chunks * d.G;
    const bool by_chunk = pairs >= 2 * kXcds;
    const int64_t rounds = (pairs + kXcds - 1) / kXcds;
    const unsigned nblk = (unsigned)(by_chunk ? rounds * kXcds * (d.H / d.G)
                                              : (int64_t)d.max_chunks * d.H);
    if (by_chunk)
        launch_scan_fast_b<Q, SEG, true>(d, x, C, D, meta, cum, dtc, CB, entering, y, seg, nblk, st);
    else
        launch_scan_fast_b<Q, SEG, false>(d, x, C, D, meta, cum, dtc, CB, entering, y, seg, nblk, st);
}

template <int Q>
static void launch_scan_fast(const PrefillDims &d, const void *x, const void *C, const float *D,
                             const int32_t *meta, const float *cum, const float *dtc,
                             const void *CB, const void *entering, void *y, const SegBufs *seg,
                             hipStream_t st)
{
    if (seg && seg->nseg > 1)
        launch_scan_fast_s<Q, true>(d, x, C, D, meta, cum, dtc, CB, entering, y, *seg, st);
    else
        launch_scan_fast_s<Q, false>(d, x, C, D, meta, cum, dtc, CB, entering, y, SegBufs(), st);
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
    if (use_fast(d)) {
        switch (d.Q) {
        case 32: launch_state_fast<32>(d, x, B, meta, cum, dtc, states, st); break;
        case 64: launch_state_fast<64>(d, x, B, meta, cum, dtc, states, st); break;
        case 128: launch_state_fast<128>(d, x, B, meta, cum, dtc, states, st); break;
        default: launch_state_fast<256>(d, x, B, meta, cum, dtc, states, st); break;
        }
        return;
    }
    if (d.in_bf16) SSD_DISPATCH_PN(d, launch_state_t, bf16, d, x, B, meta, cum, dtc, states, st);
    else SSD_DISPATCH_PN(d, launch_state_t, float, d, x, B, meta, cum, dtc, states, st);
}

template <int Q>
static void launch_bmm_pair(const PrefillDims &d, const void *B, const void *C, const int32_t *meta,
                            void *CB, hipStream_t st)
{
    const size_t smem = (size_t)Q * kCbLDB * sizeof(bf16);
    static size_t raised = 0;
    allow_lds(reinterpret_cast<const void *>(&bmm_pair_kernel<Q>), smem, raised);
    SSD_LAUNCH(d, "bmm_chunk_pairs", bmm_pair_kernel<Q>, dim3((unsigned)((int64_t)d.max_chunks * d.G)),
                       dim3(2 * Q), smem, st, d.S, d.G, static_cast<const bf16 *>(B),
                       static_cast<const bf16 *>(C), meta, static_cast<bf16 *>(CB));
}

void launch_bmm(const PrefillDims &d, const void *B, const void *C, const int32_t *meta, void *CB,
                void *stream)
{
    if (d.max_chunks <= 0) return;
    hipStream_t st = as_stream(stream);
    if (cb_by_pair(d)) {
        switch (d.Q) {
            case 32: launch_bmm_pair<32>(d, B, C, meta, CB, st); break;
            case 64: launch_bmm_pair<64>(d, B, C, meta, CB, st); break;
            case 128: launch_bmm_pair<128>(d, B, C, meta, CB, st); break;
            default: launch_bmm_pair<256>(d, B, C, meta, CB, st); break;
        }
        return;
    }
    if (d.in_bf16) {
        if (d.N == 128) launch_bmm_t<bf16, 128>(d, B, C, meta, CB, st);
        else launch_bmm_t<bf16, 16>(d, B, C, meta, CB, st);
    } else {
        if (d.N == 128) launch_bmm_t<float, 128>(d, B, C, meta, CB, st);
        else launch_bmm_t<float, 16>(d, B, C, meta, CB, st);
    }
}

constexpr int64_t kSpMinBlocks = 1024;   // four blocks per CU

template <typename TS, typename TE>
static void launch_sp_t(const PrefillDims &d, const float *states, const float *cum,
                        const int32_t *meta, void *cache, const int32_t *idx,
                        const uint8_t *has_init, void *entering, void *ckpt, hipStream_t st)
{
    const int PN = d.P * d.N;
    // four element groups per thread (more bytes in flight per sequence-chain
    // latency) when the state splits evenly and there are still enough blocks
    const int64_t blocks4 = (int64_t)d.S * d.H * (PN / 4096);
    if (PN % 4096 == 0 && blocks4 >= kSpMinBlocks) {
        SSD_LAUNCH(d, "state_passing", (state_passing_kernel<TS, TE, 4>), dim3((unsigned)blocks4), dim3(256), 0,
                           st, d.S, d.H, PN, d.Q, d.max_chunks, d.num_slots, states, cum, meta,
                           static_cast<TS *>(cache), idx, has_init, static_cast<TE *>(entering),
                           static_cast<TS *>(ckpt), d.sr);
        return;
    }
    const int EB = (PN + 1023) / 1024;
    dim3 grid((unsigned)((int64_t)d.S * d.H * EB));
    SSD_LAUNCH(d, "state_passing", (state_passing_kernel<TS, TE, 1>), grid, dim3(256), 0, st, d.S, d.H, PN,
                       d.Q, d.max_chunks, d.num_slots, states, cum, meta, static_cast<TS *>(cache),
                       idx, has_init, static_cast<TE *>(entering), static_cast<TS *>(ckpt), d.sr);
}

void launch_state_passing(const PrefillDims &d, const float *states, const float *cum,
                          const int32_t *meta, void *cache, const int32_t *idx,
                          const uint8_t *has_init, void *entering, void *ckpt, void *stream)
{
    if (d.S <= 0) return;
    hipStream_t st = as_stream(stream);
    if (d.state_f16) {
        if (d.in_bf16) launch_sp_t<f16, bf16>(d, states, cum, meta, cache, idx, has_init, entering, ckpt, st);
        else launch_sp_t<f16, float>(d, states, cum, meta, cache, idx, has_init, entering, ckpt, st);
    } else if (d.state_bf16) {
        if (d.in_bf16) launch_sp_t<bf16, bf16>(d, states, cum, meta, cache, idx, has_init, entering, ckpt, st);
        else launch_sp_t<bf16, float>(d, states, cum, meta, cache, idx, has_init, entering, ckpt, st);
    } else {
        if (d.in_bf16) launch_sp_t<float, bf16>(d, states, cum, meta, cache, idx, has_init, entering, ckpt, st);
        else launch_sp_t<float, float>(d, states, cum, meta, cache, idx, has_init, entering, ckpt, st);
    }
}

constexpr int64_t kMultiMinItems = 1024;   // items from which the multi-item kernel runs
constexpr int64_t kMultiBlocks = 512;      // its blocks: two per CU

template <int Q, bool CKPT, bool SEG, bool OWN, typename TS>
static void launch_state_scan_k(const PrefillDims &d, const void *x, const void *B,
                                const int32_t *meta, const float *cum, const float *dtc,
                                void *cache, const int32_t *idx, const uint8_t *has_init,
                                void *entering, void *ckpt, const SegBufs &seg,
                                const OwnPrep &own, hipStream_t st)
{
    const size_t smem = (size_t)Q * (kScanLDX + kScanLDB) * sizeof(bf16);
    if constexpr (!SEG && !OWN) {
        // batches of short sequences (on average at most half a chunk each) with
        // many items: persistent blocks, two per CU, several items each
        const int64_t items = (int64_t)d.S * d.H * (128 / kScanNSL);
        if ((int64_t)d.T * 2 <= (int64_t)d.S * d.Q && items >= kMultiMinItems) {
            static size_t raised_m = 0;
            allow_lds(reinterpret_cast<const void *>(&state_scan_multi_kernel<Q, CKPT, TS>), smem,
                      raised_m);
            const unsigned nblk = (unsigned)(items < kMultiBlocks ? items : kMultiBlocks);
            SSD_LAUNCH(d, "chunk_state_passing_multi", (state_scan_multi_kernel<Q, CKPT, TS>), dim3(nblk), dim3(512), smem,
                               st, d.S, d.H, d.G, d.max_chunks, d.num_slots,
                               static_cast<const bf16 *>(x), static_cast<const bf16 *>(B), meta,
                               cum, dtc, static_cast<TS *>(cache), idx, has_init,
                               static_cast<bf16 *>(entering), static_cast<TS *>(ckpt), d.sr);
            return;
        }
    }
    static size_t raised = 0;
    allow_lds(reinterpret_cast<const void *>(&state_scan_fast_kernel<Q, CKPT, SEG, OWN, TS>), smem,
              raised);
    const int nseg = SEG ? seg.nseg : 1;
    const int64_t nstate = (int64_t)d.S * nseg * d.H * (128 / kScanNSL);
    // longest chain first: few sequences (one wave ranks them), heads a multiple of 8
    const int lpt = !SEG && d.S > 1 && d.S <= 64 && d.H % kXcds == 0;
    // OWN: the CB blocks, one per (chunk, group) pair (padded to a multiple of 8
    // in longest-chain-first order, where they go out among the state blocks)
    int64_t ncb = OWN && own.CB ? (int64_t)d.max_chunks * d.G : 0;
    if (lpt) ncb = (ncb + kXcds - 1) / kXcds * kXcds;
    const char *name = OWN ? (SEG ? "chunk_state_passing_segmented_prep" : "chunk_state_passing_prep_bmm")
                           : (SEG ? "chunk_state_passing_segmented" : "chunk_state_passing");
    SSD_LAUNCH(d, name, (state_scan_fast_kernel<Q, CKPT, SEG, OWN, TS>), dim3((unsigned)(nstate + ncb)), dim3(512), smem,
                       st, d.S, d.H, d.G, d.max_chunks, d.num_slots, static_cast<const bf16 *>(x),
                       static_cast<const bf16 *>(B), meta, cum, dtc, static_cast<TS *>(cache), idx,
                       has_init, static_cast<bf16 *>(entering), static_cast<TS *>(ckpt), d.sr,
                       nseg, seg.fin, seg.L, seg.F, seg.I, lpt, own, d.T, d.prefix);
    if constexpr (SEG) {
        const int PN = 64 * 128;
        const int ncar = d.S * d.H * (PN / 1024);
        SSD_LAUNCH(d, "state_carry", state_carry_kernel<TS>, dim3((unsigned)ncar), dim3(256), 0, st,
                           d.S, d.H, PN, nseg, d.max_chunks, d.num_slots, meta, seg.fin, seg.L,
                           static_cast<bf16 *>(seg.carry), static_cast<TS *>(cache), idx, d.sr);
    }
}

template <int Q, bool OWN, typename TS>
static void launch_state_scan_o(const PrefillDims &d, const void *x, const void *B,
                                const int32_t *meta, const float *cum, const float *dtc,
                                void *cache, const int32_t *idx, const uint8_t *has_init,
                                void *entering, void *ckpt, const SegBufs *seg,
                                const OwnPrep &own, hipStream_t st)
{
    if (ckpt)
        launch_state_scan_k<Q, true, false, OWN, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init,
                                                     entering, ckpt, SegBufs(), own, st);
    else if (OWN && seg && seg->nseg > 1) {
        // (segments come only with the own-prep path: state_segments() needs few
        // (sequence, head) pairs, so few sequences)
        if constexpr (OWN)
            launch_state_scan_k<Q, false, true, true, TS>(d, x, B, meta, cum, dtc, cache, idx,
                                                          has_init, entering, ckpt, *seg, own, st);
    } else
        launch_state_scan_k<Q, false, false, OWN, TS>(d, x, B, meta, cum, dtc, cache, idx,
                                                      has_init, entering, ckpt, SegBufs(), own, st);
}

template <int Q, typename TS>
static void launch_state_scan_q(const PrefillDims &d, const void *x, const void *B,
                                const int32_t *meta, const float *cum, const float *dtc,
                                void *cache, const int32_t *idx, const uint8_t *has_init,
                                void *entering, void *ckpt, const SegBufs *seg,
                                const OwnPrep *own, hipStream_t st)
{
    if (own)
        launch_state_scan_o<Q, true, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering,
                                         ckpt, seg, *own, st);
    else
        launch_state_scan_o<Q, false, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering,
                                          ckpt, seg, OwnPrep(), st);
}

template <typename TS>
static void launch_state_scan_t(const PrefillDims &d, const void *x, const void *B,
                                const int32_t *meta, const float *cum, const float *dtc,
                                void *cache, const int32_t *idx, const uint8_t *has_init,
                                void *entering, void *ckpt, const SegBufs *seg,
                                const OwnPrep *own, hipStream_t st)
{
    switch (d.Q) {
    case 32: launch_state_scan_q<32, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st); break;
    case 64: launch_state_scan_q<64, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st); break;
    case 128: launch_state_scan_q<128, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st); break;
    default: launch_state_scan_q<256, TS>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st); break;
    }
}

bool fused_state_path(const PrefillDims &d) { return use_fast(d); }

// Segments per sequence: enough (state scan) blocks to give every CU about two,
// at most kMaxSeg, never more than the chunks there can be.
constexpr int64_t kSegBlocks = 512;

int state_segments(const PrefillDims &d)
{
    if (!use_fast(d) || d.S <= 0 || d.max_chunks < 2) return 1;
    const int64_t base = (int64_t)d.S * d.H * (128 / kScanNSL);
    int64_t n = kSegBlocks / base;
    n = n < kMaxSeg ? n : kMaxSeg;
    n = n < d.max_chunks ? n : d.max_chunks;
    return n > 1 ? (int)n : 1;
}

bool own_prep_path(const PrefillDims &d)
{
    return use_fast(d) && d.S > 0 && d.S <= kOwnPrepMaxSeqs;
}

void launch_state_scan(const PrefillDims &d, const void *x, const void *B, const int32_t *meta,
                       const float *cum, const float *dtc, void *cache, const int32_t *idx,
                       const uint8_t *has_init, void *entering, void *ckpt, void *stream,
                       const SegBufs *seg, const OwnPrep *own)
{
    if (d.S <= 0) return;
    hipStream_t st = as_stream(stream);
    if (d.state_f16)
        launch_state_scan_t<f16>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st);
    else if (d.state_bf16)
        launch_state_scan_t<bf16>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st);
    else
        launch_state_scan_t<float>(d, x, B, meta, cum, dtc, cache, idx, has_init, entering, ckpt, seg, own, st);
}

constexpr int kShortSub = 32;   // tokens per sub-chunk of the short-sequence kernel (32 measured
                                // faster than 64 on 32 x 32-token continuations)

bool short_scan_path(const PrefillDims &d)
{
    return use_fast(d) && d.S > 0 && 2 * (int64_t)d.T <= (int64_t)d.S * d.Q;
}

template <typename TS>
static void launch_short_t(const PrefillDims &d, const void *x, const void *dt, const float *A,
                           const void *B, const void *C, const float *D, const int32_t *cu,
                           void *cache, const int32_t *idx, const uint8_t *has_init, void *y,
                           void *ckpt, hipStream_t st, const DtTf &tf)
{
    const unsigned nblk = (unsigned)((int64_t)d.S * d.H);
    SSD_LAUNCH(d, "short_scan", (short_scan_kernel<kShortSub, TS>), dim3(nblk), dim3(256), 0, st, d.T, d.S,
               d.H, d.G, d.Q, d.num_slots, static_cast<const bf16 *>(x),
               static_cast<const bf16 *>(dt), A, static_cast<const bf16 *>(B),
               static_cast<const bf16 *>(C), D, cu, static_cast<TS *>(cache), idx, has_init,
               static_cast<bf16 *>(y), static_cast<TS *>(ckpt), d.sr, tf, d.prefix);
}

void launch_short_scan(const PrefillDims &d, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const int32_t *cu,
                       void *cache, const int32_t *idx, const uint8_t *has_init, void *y,
                       void *ckpt, void *stream, const DtTf &tf)
{
    hipStream_t st = as_stream(stream);
    if (d.state_f16)
        launch_short_t<f16>(d, x, dt, A, B, C, D, cu, cache, idx, has_init, y, ckpt, st, tf);
    else if (d.state_bf16)
        launch_short_t<bf16>(d, x, dt, A, B, C, D, cu, cache, idx, has_init, y, ckpt, st, tf);
    else
        launch_short_t<float>(d, x, dt, A, B, C, D, cu, cache, idx, has_init, y, ckpt, st, tf);
}

void launch_chunk_scan(const PrefillDims &d, const void *x, const void *C, const float *D,
                       const int32_t *meta, const float *cum, const float *dtc, const void *CB,
                       const void *entering, void *y, void *stream, const SegBufs *seg)
{
    if (d.max_chunks <= 0) return;
    hipStream_t st = as_stream(stream);
    if (use_fast(d)) {
        switch (d.Q) {
        case 32: launch_scan_fast<32>(d, x, C, D, meta, cum, dtc, CB, entering, y, seg, st); break;
        case 64: launch_scan_fast<64>(d, x, C, D, meta, cum, dtc, CB, entering, y, seg, st); break;
        case 128: launch_scan_fast<128>(d, x, C, D, meta, cum, dtc, CB, entering, y, seg, st); break;
        default: launch_scan_fast<256>(d, x, C, D, meta, cum, dtc, CB, entering, y, seg, st); break;
        }
        return;
    }
    if (d.in_bf16)
        SSD_DISPATCH_PN(d, launch_scan_t, bf16, d, x, C, D, meta, cum, dtc, CB, entering, y, st);
    else
        SSD_DISPATCH_PN(d, launch_scan_t, float, d, x, C, D, meta, cum, dtc, CB, entering, y, st);
}

}  // namespace ssd
