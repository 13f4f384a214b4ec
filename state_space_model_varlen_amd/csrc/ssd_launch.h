// Internal launcher interface between the C ABI (ssd_api.cpp) and the kernels.
// Every launcher only enqueues on the given stream; arguments are validated
// by the caller.
#pragma once

#include <stddef.h>
#include <stdint.h>

struct ssd_launch_trace;   // include/ssd_mi355x.h

namespace ssd {

// Per-launch timing of a combined call: every launch names itself; with a
// trace whose event array has room, it gets the two events (start, end) that
// its launch must record and true, else false.
bool trace_events(ssd_launch_trace *t, const char *name, void **start, void **stop);

// The layer's step-size preprocessing, applied where dt is read:
// dt = min(max(softplus(dt_raw + bias[h]), lo), hi) when `on`.
struct DtTf {
    const float *bias = nullptr;
    float lo = 0.0f, hi = 0.0f;
    int on = 0;
};

// Stochastic rounding of fp16 state stores: the seed is read on the device
// (one word per step), `rounds` Philox rounds; no seed: round to nearest even.
struct SrCtx {
    const uint64_t *seed = nullptr;
    int rounds = 0;
};

struct PrefillDims {
    int T, S, H, P, N, G, Q;
    int max_chunks;
    int num_slots;
    bool in_bf16;
    bool state_bf16;
    bool state_f16 = false;   // fp16 state cache and checkpoints
    SrCtx sr;
    // align mode: prefix[s] tokens precede sequence s, chunk boundaries fall on
    // absolute multiples of Q (nullptr: chunks start at each sequence's start)
    const int32_t *prefix = nullptr;
    ssd_launch_trace *trace = nullptr;   // per-launch timing (nullptr: none)
};

struct DecodeDims {
    int R, T, H, P, N, G;
    int num_slots;
    bool in_bf16;
    bool state_bf16;
    bool state_f16 = false;   // fp16 state cache and per-token states
    SrCtx sr;
};

// fp32 -> fp16 with the library's stochastic rounding (kind: Philox stream of
// the destination array), or round to nearest even without a seed.
void launch_round_f16(const float *in, void *out, int64_t n, const SrCtx &sr, int kind,
                      void *stream);

void launch_chunk_cumsum(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                         int32_t *meta, float *cum, float *dto, void *stream,
                         const DtTf &tf = DtTf());
// Steps 1 and 4 (cumsum with chunk metadata, and CB) in one launch.
void launch_chunk_prep(const PrefillDims &d, const void *dt, const float *A, const int32_t *cu,
                       int32_t *meta, float *cum, float *dto, const void *B, const void *C,
                       void *CB, void *stream, const DtTf &tf = DtTf());
void launch_chunk_state(const PrefillDims &d, const void *x, const void *B, const int32_t *meta,
                        const float *cum, const float *dtc, float *states, void *stream);
void launch_state_passing(const PrefillDims &d, const float *states, const float *cum,
                          const int32_t *meta, void *cache, const int32_t *idx,
                          const uint8_t *has_init, void *entering, void *ckpt, void *stream);
// Chunk state and state passing in one launch (bf16 inputs, headdim 64,
// d_state 128 only: fused_state_path()); writes what state passing writes and
// needs no chunk-state buffer.
bool fused_state_path(const PrefillDims &d);

// Segmented state passing (fused path, no checkpoints): each sequence's chunk
// chain is cut into up to `nseg` segments that run in parallel, each from a zero
// state (the first from the cached one). A segment leaves its local final state
// (fin, float32 [S nseg][H][P][N]) and total log decay (L, [S nseg][H]); for
// every chunk, the log decay from its segment's start (F, [H][max_chunks]) and
// the segment's global index s nseg + b (I, [max_chunks], -1 in a first
// segment). The carry step then chains the segments into each one's true
// starting state (carry, bf16 [S nseg][H][P][N]) and writes the final states;
// the chunk scan adds exp(F) carry to the local entering states. Segments are
// used only together with OwnPrep (below).
struct SegBufs {
    int nseg = 1;
    float *fin = nullptr, *L = nullptr, *F = nullptr;
    int32_t *I = nullptr;
    void *carry = nullptr;
};
// Segments the combined call uses for these dimensions (1: unsegmented).
int state_segments(const PrefillDims &d);

// The combined call's state launch doing steps 1 and 4 as well (own_prep_path:
// the fused state path with at most kOwnPrepMaxSeqs sequences): its state
// blocks find their chunks from cu_seqlens and scan dt themselves, and publish
// the metadata, cumsum and dt rows (meta, cum, dtc) that the later launches
// read; with CB set, one block per (chunk, group) pair after the state blocks
// computes CB. No cumsum, prep or bmm launch then runs.
struct OwnPrep {
    const void *dt = nullptr;
    const float *A = nullptr;
    const int32_t *cu = nullptr;
    DtTf tf;
    int32_t *meta = nullptr;
    float *cum = nullptr, *dtc = nullptr;
    const void *C = nullptr;
    void *CB = nullptr;
};
constexpr int kOwnPrepMaxSeqs = 256;
bool own_prep_path(const PrefillDims &d);

void launch_state_scan(const PrefillDims &d, const void *x, const void *B, const int32_t *meta,
                       const float *cum, const float *dtc, void *cache, const int32_t *idx,
                       const uint8_t *has_init, void *entering, void *ckpt, void *stream,
                       const SegBufs *seg = nullptr, const OwnPrep *own = nullptr);
void launch_bmm(const PrefillDims &d, const void *B, const void *C, const int32_t *meta, void *CB,
                void *stream);
// Whether launch_bmm computes CB with one block per (chunk, group) pair (bf16,
// d_state 128, enough pairs to fill the chip); the combined call then runs step
// 1 alone and launch_bmm after it, instead of launch_chunk_prep.
bool cb_by_pair(const PrefillDims &d);
void launch_chunk_scan(const PrefillDims &d, const void *x, const void *C, const float *D,
                       const int32_t *meta, const float *cum, const float *dtc, const void *CB,
                       const void *entering, void *y, void *stream,
                       const SegBufs *seg = nullptr);

// Batches of short sequences (bf16, headdim 64, d_state 128, on average at most
// half a chunk per sequence: 2 T <= S Q): the whole prefill in one launch, one
// block per (sequence, head) walking its sequence in sub-chunks, with the
// initial state read from and the final state written to the cache slot, and
// no workspace.
bool short_scan_path(const PrefillDims &d);
void launch_short_scan(const PrefillDims &d, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const int32_t *cu,
                       void *cache, const int32_t *idx, const uint8_t *has_init, void *y,
                       void *ckpt, void *stream, const DtTf &tf);

// cu (optional): packed-varlen requests, request r owning tokens cu[r] .. cu[r+1]-1
// of Ttot packed rows; without it request r owns tokens r T .. r T + T - 1.
void launch_state_update(const DecodeDims &d, void *cache, const int32_t *idx, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *inter, void *stream,
                         const int32_t *cu = nullptr, int Ttot = 0, const DtTf &tf = DtTf());
void launch_state_commit(const DecodeDims &d, void *cache, const int32_t *idx, const void *inter,
                         const int32_t *accepted, void *stream, const int32_t *cu = nullptr,
                         int Ttot = 0);

// ReplaySSM decode: verify step, cursor move after sampling, materialisation.
void launch_replay_update(const DecodeDims &d, int W, void *ckpt, void *rx, void *rdt, void *rB,
                          const int32_t *cursor, const int32_t *idx, const void *x, const void *dt,
                          const float *A, const void *B, const void *C, const float *D, void *y,
                          void *stream);
void launch_replay_advance(const DecodeDims &d, int W, int32_t *cursor, const int32_t *idx,
                           const int32_t *accepted, void *stream);
void launch_replay_materialize(const DecodeDims &d, int W, void *ckpt, const void *rx,
                               const void *rdt, const void *rB, int32_t *cursor,
                               const int32_t *idx, const float *A, void *stream);

}  // namespace ssd
