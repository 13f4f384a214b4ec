/*
 * ssd_mi355x.h - C ABI of the MI355X (gfx950) Mamba2 SSD varlen scan and the
 * decode / MTP selective state update.
 *
 * What the operations compute (per head h, group g = h / (H / G), state h_t
 * of shape [P x N]):
 *
 *     h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t
 *     y_t = h_t . C_t + D_h * x_t                         (contraction over N)
 *
 * the selective state-space recurrence whose recurrent state the pages cache
 * and roll back (vLLM PR #52928 "[Mamba] Add FlashInfer ReplaySSM support
 * for MTP", section "Summary") and whose FP32 recurrence they keep (vLLM PR
 * #62922, section "Details"). Prefill evaluates it with the chunked SSD scan
 * in the pages' five steps - chunk cumsum, chunk state, state passing, bmm,
 * chunk scan (vLLM PR #61501, section "Details") - over packed varlen batches
 * given by cu_seqlens, with initial states read from a slot-indexed state
 * cache inside state passing and every chunk's entering state kept in the
 * workspace for chunk scan (vLLM PR #62922, sections "Overview", "Details").
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers are device pointers unless the argument says "host". Problem
 *   descriptors (ssd_problem, ssu_problem) are host structs read during the
 *   call only.
 * - Layouts are row-major and contiguous, last index fastest:
 *     x, y [T,H,P]; dt [T,H]; A, D [H] float32; B, C [T,G,N];
 *     cu_seqlens [S+1] int32 with cu_seqlens[0] = 0, non-decreasing,
 *       cu_seqlens[S] = T; state_indices [S] int32; has_initial_state [S] uint8;
 *     state cache [num_slots,H,P,N]; checkpoints [max_chunks,H,P,N].
 *   Every array pointer must be 16-byte aligned.
 * - Chunks: sequence s is split into ceil(L_s / Q) chunks of Q tokens starting
 *   at its first token, the last one possibly partial; no chunk spans two
 *   sequences. chunk_cu[s] = sum over s' < s of ceil(L_s' / Q) numbers them;
 *   nc = chunk_cu[S] <= max_chunks = T / Q + S (ssd_max_chunks).
 * - Ownership: the caller allocates every buffer, workspace included. The
 *   library allocates nothing, keeps no pointer after returning and holds no
 *   mutable global state, so concurrent calls on different buffers are safe.
 * - Asynchrony: every call only enqueues work on `stream` (a hipStream_t;
 *   NULL = the default stream) and never synchronises the host.
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   a failed check returns its status and writes nothing. SSD_ERR_HIP reports
 *   a launch failure. Device-resident values (cu_seqlens, state_indices,
 *   num_accepted) are not read by the host: kernels clamp token ranges to
 *   [0, T) and chunk numbers to max_chunks, skip a slot index outside
 *   [0, num_slots) (its initial state counts as zero and nothing is written
 *   there) and skip an accepted count outside [0, tokens_per_req), so bad
 *   device data gives wrong numbers, never an out-of-bounds access.
 *   Duplicate slot indices within one call are a caller error (the writes
 *   race).
 * - Precision: all recurrence arithmetic in float32; results are rounded to
 *   their storage dtype (round to nearest even) when stored. With bf16 inputs
 *   the dense contractions run on bf16 MFMA with float32 accumulation, so their
 *   operands are bf16: x, B, C as given, and rounded to bf16 first: CB, the
 *   decay-scaled B (exp(cum_last - cum_t) dt_t B_t) and x (exp(R - cum_j) dt_j
 *   x_j), and each chunk's entering state (stored in bf16 between the launches).
 *   Two partial results are rounded to bf16 before the last step: y's SSM part
 *   before D_h x is added (y is then rounded again when stored), and in a
 *   segmented call the entering state local + exp(F) carry (each term bf16).
 *   With A_h dt <= 0 (a decaying state, as in Mamba2) these roundings stay far
 *   inside the tolerances the tests apply (2e-2 absolute + 1e-2 relative per
 *   element); with A_h dt > 0 the state grows, and the rounding of the state
 *   term scales with the state's size rather than with y's.
 * - Supported on the GPU: headdim P in {16, 64}, d_state N in {16, 128},
 *   chunk_size Q in {32, 64, 128, 256}, dtypes float32 and bfloat16. Other
 *   shapes return SSD_ERR_UNSUPPORTED.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 3

enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a size is negative / zero where it must not be, or H % G != 0 */
    SSD_ERR_DTYPE = 3,       /* unknown dtype code */
    SSD_ERR_UNSUPPORTED = 4, /* valid but not built for the GPU (P, N, Q outside the sets above) */
    SSD_ERR_WORKSPACE = 5,   /* workspace smaller than ssd_workspace_bytes() */
    SSD_ERR_HIP = 6,         /* a kernel launch failed */
    SSD_ERR_ALIGN = 7,       /* an array pointer is not 16-byte aligned */
    SSD_ERR_SCRATCH = 8      /* the problem needs more workspace than the static scratch
                                array of ssd_combined_varlen_noalloc holds */
};

/* SSD_F16 is a state dtype only (state caches, checkpoints, per-token and
 * ReplaySSM states); inputs are SSD_F32 or SSD_BF16. */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_F16 = 2 } ssd_dtype;

/* One packed varlen prefill (host struct). */
typedef struct {
    int32_t total_tokens; /* T: tokens of all sequences together */
    int32_t num_seqs;     /* S */
    int32_t nheads;       /* H */
    int32_t headdim;      /* P */
    int32_t d_state;      /* N */
    int32_t ngroups;      /* G: heads h share B, C group h / (H / G) */
    int32_t chunk_size;   /* Q */
    int32_t num_slots;    /* rows of the state cache */
    int32_t in_dtype;     /* ssd_dtype of x, dt, B, C, y */
    int32_t state_dtype;  /* ssd_dtype of the state cache and the checkpoints */
} ssd_problem;

/* One decode / MTP verify batch (host struct). */
typedef struct {
    int32_t num_reqs;       /* R */
    int32_t tokens_per_req; /* T: 1 for plain decode, 1 + drafts for MTP verify */
    int32_t nheads;         /* H */
    int32_t headdim;        /* P */
    int32_t d_state;        /* N */
    int32_t ngroups;        /* G */
    int32_t num_slots;      /* rows of the state cache */
    int32_t in_dtype;       /* ssd_dtype of x, dt, B, C, y */
    int32_t state_dtype;    /* ssd_dtype of the state cache and the intermediate states */
} ssu_problem;

/*
 * The layer's step-size preprocessing, fused into the kernels that read dt:
 *   dt = min(max(softplus(dt_raw + dt_bias[h]), dt_min), dt_max)
 * in float32, softplus(v) = log(1 + exp(v)) (v itself above 20). The step
 * size is defined this way in the workload of vLLM PR #52928 ("Summary": the
 * same kernels with the model's input conventions) and the pages' test
 * inputs; dt_raw is then the pre-activation value in in_dtype.
 */
typedef struct {
    const float *dt_bias; /* [H] float32 on the device, or NULL (no bias) */
    float dt_min;         /* lower clamp (0 for none) */
    float dt_max;         /* upper clamp (a huge value for none); dt_min <= dt_max */
} ssd_dt_transform;

/*
 * Options of the _ex entry points (every field may be NULL / 0):
 *   dt_transform  the step-size preprocessing above
 *   prefix_lens   [S] int32 on the device: align mode (see
 *                 ssd_combined_varlen_aligned); prefill only
 *   sr_seed       stochastic rounding of fp16 state stores (vLLM PR #61501,
 *                 "Serve and client commands": a float16 SSM cache with
 *                 stochastic rounding and a configurable number of Philox
 *                 rounds; "Details", its list of changes: one seed per step
 *                 read from a device buffer). Points to one
 *                 uint64 on the device, read by the kernels, so a caller can
 *                 refresh it per step without host synchronisation. Requires
 *                 state_dtype SSD_F16. NULL: round to nearest even.
 *   sr_rounds     Philox4x32 rounds, 1..16 (e.g. 5 or 10)
 *   trace         per-launch timing events (ssd_launch_trace below)
 * Rounding: x becomes the fp16 value above or below it in magnitude, the
 * farther one with probability (|x| - |lo|) / (|hi| - |lo|), drawn as
 * d / 2^16 from a 16-bit draw d (non-finite values and |x| > 65504 round to
 * nearest even). Element e of a destination array of kind k takes the 16-bit
 * half e mod 2 (low half first) of word (e/2) mod 4 of
 * Philox4x32-R(counter = (e/8 low, e/8 high, k, 0), key = seed); kinds:
 * 0 final states, 1 checkpoints, 2 per-token states, 3 ReplaySSM checkpoints.
 * e is the flat element index in that array.
 */
/*
 * Per-launch timing of a prefill call (ssd_options.trace; profiling only): the
 * call's k-th kernel launch records its own start on events[2k] and its end on
 * events[2k + 1] (hipExtLaunchKernelGGL: the kernel's execution, as a kernel
 * trace times it), so hipEventElapsedTime(events[2k], events[2k + 1]) is its
 * duration. The events are hipEvent_t handles the caller created with timing
 * enabled; launches whose pair lies at or past `capacity` events run without.
 */
#define SSD_TRACE_MAX_LAUNCHES 16
typedef struct ssd_launch_trace {
    void *const *events;    /* [capacity] hipEvent_t (2 per launch), or NULL (names only) */
    int32_t capacity;
    int32_t count;          /* out: kernel launches of the call */
    const char *names[SSD_TRACE_MAX_LAUNCHES];   /* out: static name of launch k */
} ssd_launch_trace;

typedef struct {
    const ssd_dt_transform *dt_transform;
    const int32_t *prefix_lens;
    const uint64_t *sr_seed;
    int32_t sr_rounds;
    ssd_launch_trace *trace;   /* host struct, or NULL; ssd_combined_varlen_ex only */
} ssd_options;

/* SSD_ABI_VERSION of the built library. */
int ssd_abi_version(void);

/* Static text for a status code (never NULL). */
const char *ssd_status_string(int status);

/* Host-side sizing helpers; they validate `p` and return 0 when it is invalid. */
int64_t ssd_max_chunks(const ssd_problem *p);      /* T / Q + S */
int64_t ssd_chunk_meta_count(const ssd_problem *p); /* int32 entries of chunk_meta */
size_t ssd_workspace_bytes(const ssd_problem *p);  /* for ssd_combined_varlen */

/*
 * Step 1 - chunk metadata and chunk cumsum (vLLM PR #61501, section
 * "Details": the first of the five steps; chunk metadata derived on the device
 * from cu_seqlens, so no host synchronisation is needed).
 *   dt          [T,H] in_dtype, post-activation step sizes
 *   A           [H] float32
 *   cu_seqlens  [S+1] int32
 *   chunk_meta  out, int32 [ssd_chunk_meta_count]:
 *                 [0..S]            chunk_cu
 *                 [S+1+3c+0,1,2]    sequence, first token, token count of chunk c
 *                                   (-1, 0, 0 for c >= nc)
 *                 [S+1+3mc+s]       cu_seqlens[s] clamped to [0, T], s = 0..S
 *                                   (mc = ssd_max_chunks)
 *                 [2S+2+3mc+s]      tokens in sequence s's first chunk, s < S
 *   dA_cumsum   out, float32 [H, max_chunks, Q]: inclusive cumsum of dt*A_h over
 *               the chunk's tokens; positions past the chunk's end hold the chunk's
 *               total again (summed in another order: equal to the last position's
 *               value within float32 rounding)
 *   dt_chunk    out, float32 [H, max_chunks, Q]: dt per chunk position, 0 past the end
 * Rows c >= nc of dA_cumsum / dt_chunk are left unwritten.
 */
int ssd_chunk_cumsum(const ssd_problem *p, const void *dt, const float *A,
                     const int32_t *cu_seqlens, int32_t *chunk_meta, float *dA_cumsum,
                     float *dt_chunk, void *stream);

/*
 * Step 2 - chunk state (vLLM PR #61501, section "Details"): the state each
 * chunk produces from a zero entering state,
 *   S_c[h,p,n] = sum_t exp(cum_last - cum_t) * dt_t * x_t[h,p] * B_t[g,n].
 *   x [T,H,P], B [T,G,N] in_dtype; chunk_meta, dA_cumsum, dt_chunk from step 1
 *   chunk_states out, float32 [max_chunks,H,P,N] (rows c >= nc unwritten)
 */
int ssd_chunk_state(const ssd_problem *p, const void *x, const void *B,
                    const int32_t *chunk_meta, const float *dA_cumsum, const float *dt_chunk,
                    float *chunk_states, void *stream);

/*
 * Step 3 - state passing, reading initial states from the cache by slot and
 * writing final states back in place (vLLM PR #62922, sections "Overview" and
 * "Details"; vLLM PR #61501, section "Details": gather only where a sequence
 * has an initial state, scatter final states into their slots in the cache
 * dtype; checkpoints for prefills that store every chunk state). Per sequence
 * s and head h, sequentially over its chunks:
 *   H_0 = has_initial_state[s] ? cache[state_indices[s], h] : 0
 *   entering_states[c] = H_c;  H_{c+1} = exp(cum_last(c)) * H_c + S_c
 *   checkpoints[c] = round(H_{c+1})       (exit state of chunk c)
 *   cache[state_indices[s], h] = round(H_last)   (after all reads of that slot)
 *   state_cache       in/out [num_slots,H,P,N] state_dtype; slots not named in
 *                     state_indices are not touched
 *   state_indices     [S] int32
 *   has_initial_state [S] uint8, or NULL: no sequence reads its slot
 *   entering_states   out [max_chunks,H,P,N] in in_dtype (the precision chunk scan
 *                     multiplies it in); must not overlap chunk_states
 *   checkpoints       out [max_chunks,H,P,N] state_dtype, or NULL to skip
 * A zero-length sequence writes its initial state (or zeros) back to its slot.
 */
int ssd_state_passing(const ssd_problem *p, const float *chunk_states, const float *dA_cumsum,
                      const int32_t *chunk_meta, void *state_cache,
                      const int32_t *state_indices, const uint8_t *has_initial_state,
                      void *entering_states, void *checkpoints, void *stream);

/*
 * Steps 2 and 3 in one launch (same pages and sections as steps 2 and 3):
 * the chunk states are folded into the running state as they are produced
 * and never stored, so no chunk_states buffer exists. Outputs and cache
 * semantics are exactly those of ssd_state_passing (entering_states in
 * in_dtype, checkpoints and the final state in state_dtype, zero-length
 * sequences write their initial state or zeros back). Only bf16 inputs with
 * headdim 64 and d_state 128 are supported (SSD_ERR_UNSUPPORTED otherwise);
 * ssd_combined_varlen uses it for exactly those shapes.
 *   x [T,H,P], B [T,G,N] bf16; chunk_meta, dA_cumsum, dt_chunk from step 1;
 *   state_cache, state_indices, has_initial_state, entering_states,
 *   checkpoints as for ssd_state_passing.
 */
int ssd_chunk_state_passing(const ssd_problem *p, const void *x, const void *B,
                            const int32_t *chunk_meta, const float *dA_cumsum,
                            const float *dt_chunk, void *state_cache,
                            const int32_t *state_indices, const uint8_t *has_initial_state,
                            void *entering_states, void *checkpoints, void *stream);

/*
 * Step 4 - bmm (vLLM PR #61501, section "Details"): CB[c,g,i,j] = C_i . B_j
 * inside each chunk, float32 accumulation. B, C [T,G,N] in_dtype; CB out:
 * Q*Q elements per (chunk, group) at offset (c*G + g)*Q*Q, in in_dtype (chunk
 * scan multiplies in that precision). Layout inside a (chunk, group) block:
 *   float32 inputs: row-major, element (i, j) at i*Q + j;
 *   bf16 inputs: MFMA fragment order - element (i, j) at
 *     ((i/16 * Q/32 + j/32) * 64 + lane) * 8 + v, lane = i%16 + 16*kg,
 *     where j%32 = 4*kg + v%4 + 16*(v/4) (one contiguous 1 KiB block per
 *     16-row x 32-column operand tile).
 * Defined for j <= i < chunk length (the causal part chunk scan reads); for
 * bf16 inputs also for every (i, j) with i < chunk length in the 16-row x
 * 32-column blocks that hold the diagonal, as zero where j > i (chunk scan
 * then needs no causal mask). Other entries are unspecified.
 */
int ssd_bmm_chunk(const ssd_problem *p, const void *B, const void *C,
                  const int32_t *chunk_meta, void *CB, void *stream);

/*
 * Step 5 - chunk scan (vLLM PR #61501, section "Details"; entering states from
 * the workspace, vLLM PR #62922, section "Details"):
 *   y_i = sum_{j<=i} CB[i,j] * exp(cum_i - cum_j) * dt_j * x_j
 *         + exp(cum_i) * (H_in . C_i) + D_h * x_i
 *   x [T,H,P], C [T,G,N] in_dtype; D [H] float32 or NULL (= 0); CB from step 4;
 *   entering_states from step 3 (in_dtype); y out [T,H,P] in_dtype.
 */
int ssd_chunk_scan(const ssd_problem *p, const void *x, const void *C, const float *D,
                   const int32_t *chunk_meta, const float *dA_cumsum, const float *dt_chunk,
                   const void *CB, const void *entering_states, void *y, void *stream);

/*
 * The whole prefill: steps 1-5 enqueued on one stream with no host
 * synchronisation (one to four launches; how the steps are grouped depends
 * on the shapes), intermediates in the caller's workspace (vLLM PR #61501,
 * sections "Details" and "Claims"; vLLM PR #62922, section "Details").
 * Semantics are those of the five steps composed: every initial state is
 * read as it was before the call even though the call overwrites the slot.
 * For bf16 inputs with headdim 64 and d_state 128:
 *   - steps 2 and 3 run as ssd_chunk_state_passing (and the workspace holds
 *     no chunk states);
 *   - with at most 256 sequences, steps 1 and 4 run inside that launch (its
 *     blocks find their chunks from cu_seqlens and scan dt themselves, and
 *     leave in the workspace the metadata, cumsum, dt and CB the steps would
 *     write, bit for bit): the call is two launches, state and chunk scan,
 *     and its results equal those of ssd_chunk_cumsum, ssd_bmm_chunk,
 *     ssd_chunk_state_passing and ssd_chunk_scan called one by one, bit for
 *     bit;
 *   - with no checkpoints and few (sequence, head) pairs, each sequence's
 *     chunk chain is cut into segments that run in parallel and are chained
 *     afterwards by one more launch, which also computes CB (the recurrence
 *     is linear in its starting state); the workspace then also holds the
 *     segments' states. Results agree with the unsegmented path within
 *     rounding, not bit for bit;
 *   - batches of short sequences (on average at most half a chunk each) run
 *     as one launch that uses no workspace.
 *   workspace        device buffer of at least ssd_workspace_bytes(p) bytes,
 *                    256-byte aligned; its contents on entry do not matter
 *   checkpoints      [max_chunks,H,P,N] state_dtype or NULL
 * Sizes with num_seqs = 0 or total_tokens = 0 enqueue nothing beyond
 * zero-length write-backs.
 */
int ssd_combined_varlen(const ssd_problem *p, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D, const int32_t *cu_seqlens,
                        void *state_cache, const int32_t *state_indices,
                        const uint8_t *has_initial_state, void *y, void *checkpoints,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode / MTP verify state update (vLLM PR #52928, sections "Summary" and
 * "Design": one target token plus draft tokens per request, (batch, tokens, ...)
 * inputs; vLLM PR #55688, review of the SSU dispatch: the plain
 * selective_state_update next to the ReplaySSM kernels). Per request r and head h, starting from
 * state_cache[state_indices[r], h], the recurrence runs over the request's T
 * tokens in float32; y_t is written for every token. With
 * intermediate_states non-NULL the state after token t is stored (rounded)
 * at intermediate_states[r, t] - what a rollback to t accepted drafts reads -
 * and the cache is not written; with NULL the state after the last token is
 * rounded and written back to the slot.
 *   x, y [R,T,H,P]; dt [R,T,H]; B, C [R,T,G,N] in_dtype; A, D [H] float32 (D may be NULL)
 *   state_cache [num_slots,H,P,N] state_dtype; state_indices [R] int32
 *   intermediate_states [R,T,H,P,N] state_dtype or NULL
 */
int selective_state_update(const ssu_problem *p, void *state_cache, const int32_t *state_indices,
                           const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, void *y, void *intermediate_states,
                           void *stream);

/*
 * Rollback / commit to the accepted count (vLLM PR #52928, section "Summary":
 * the accepted length decides the next state): for every request r with
 * 0 <= num_accepted[r] < T, copy intermediate_states[r, num_accepted[r]] into
 * state_cache[state_indices[r]]. num_accepted [R] int32 counts accepted draft
 * tokens (the target token is always accepted).
 */
int ssd_state_commit(const ssu_problem *p, void *state_cache, const int32_t *state_indices,
                     const void *intermediate_states, const int32_t *num_accepted, void *stream);

/*
 * Step 1 with the dt preprocessing: as ssd_chunk_cumsum with dt_raw in place
 * of dt; dt_chunk receives the preprocessed float32 step sizes, so steps 2-5
 * are unchanged. dt_transform must not be NULL.
 */
int ssd_chunk_cumsum_dt(const ssd_problem *p, const ssd_dt_transform *dt_transform,
                        const void *dt_raw, const float *A, const int32_t *cu_seqlens,
                        int32_t *chunk_meta, float *dA_cumsum, float *dt_chunk, void *stream);

/*
 * ssd_combined_varlen with the dt preprocessing applied in step 1.
 */
int ssd_combined_varlen_dt(const ssd_problem *p, const ssd_dt_transform *dt_transform,
                           const void *x, const void *dt_raw, const float *A, const void *B,
                           const void *C, const float *D, const int32_t *cu_seqlens,
                           void *state_cache, const int32_t *state_indices,
                           const uint8_t *has_initial_state, void *y, void *checkpoints,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Align-mode prefill (vLLM PR #55688, "Summary": prefix caching in the align
 * cache mode; checkpoints serve prefix reuse, vLLM PR #61501 "Details"): sequence s
 * continues after prefix_lens[s] cached tokens, and chunk boundaries fall on
 * absolute token positions that are multiples of Q, so its first chunk holds
 * Q - (prefix_lens[s] mod Q) tokens (Q when that is 0) and every checkpoint
 * is the state at an absolute multiple of Q (or the sequence's end). Results
 * are those of ssd_combined_varlen otherwise; y and the final states do not
 * depend on where chunks are cut.
 *   prefix_lens   [S] int32 on the device (negative values count as 0)
 *   checkpoints   [ssd_max_chunks_aligned(p),H,P,N] state_dtype or NULL; row
 *                 chunk_cu[s] + k holds the exit state of sequence s's chunk k
 *   workspace     at least ssd_workspace_bytes_aligned(p) bytes
 */
int64_t ssd_max_chunks_aligned(const ssd_problem *p);   /* T/Q + 2 S */
size_t ssd_workspace_bytes_aligned(const ssd_problem *p);
int ssd_combined_varlen_aligned(const ssd_problem *p, const int32_t *prefix_lens, const void *x,
                                const void *dt, const float *A, const void *B, const void *C,
                                const float *D, const int32_t *cu_seqlens, void *state_cache,
                                const int32_t *state_indices, const uint8_t *has_initial_state,
                                void *y, void *checkpoints, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Packed-varlen MTP verify (vLLM PR #52928, section "Summary": variable-length
 * batches use the packed cu_seqlens interface) with optional dt preprocessing.
 * Request r owns tokens cu_seqlens[r] .. cu_seqlens[r+1]-1 of the packed
 * arrays (any count, 0 included: a request with no token changes nothing);
 * otherwise as selective_state_update, with intermediate_states indexed by
 * packed token.
 *   total_tokens     rows of the packed arrays (T_tot)
 *   cu_seqlens       [R+1] int32 on the device, non-decreasing (values are
 *                    clamped to [0, T_tot] on the device)
 *   x, y [T_tot,H,P]; dt [T_tot,H]; B, C [T_tot,G,N] in_dtype
 *   intermediate_states [T_tot,H,P,N] state_dtype or NULL
 *   dt_transform     NULL: dt as given; else dt is dt_raw, preprocessed
 * p->tokens_per_req is a hint only (the most tokens of a request; >= 1).
 */
int selective_state_update_varlen(const ssu_problem *p, int32_t total_tokens,
                                  const int32_t *cu_seqlens,
                                  const ssd_dt_transform *dt_transform, void *state_cache,
                                  const int32_t *state_indices, const void *x, const void *dt,
                                  const float *A, const void *B, const void *C, const float *D,
                                  void *y, void *intermediate_states, void *stream);

/*
 * Rollback after a packed-varlen verify: for every request r with
 * 0 <= num_accepted[r] < (its token count), copy
 * intermediate_states[cu_seqlens[r] + num_accepted[r]] into its slot.
 */
int ssd_state_commit_varlen(const ssu_problem *p, int32_t total_tokens,
                            const int32_t *cu_seqlens, void *state_cache,
                            const int32_t *state_indices, const void *intermediate_states,
                            const int32_t *num_accepted, void *stream);

/*
 * ssd_combined_varlen with options (dt preprocessing, align mode, stochastic
 * rounding of fp16 final states and checkpoints); the workspace must hold
 * ssd_workspace_bytes_aligned(p) bytes when prefix_lens is set.
 */
int ssd_combined_varlen_ex(const ssd_problem *p, const ssd_options *opt, const void *x,
                           const void *dt, const float *A, const void *B, const void *C,
                           const float *D, const int32_t *cu_seqlens, void *state_cache,
                           const int32_t *state_indices, const uint8_t *has_initial_state,
                           void *y, void *checkpoints, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * selective_state_update with options (dt preprocessing, stochastic rounding
 * of fp16 stores); with cu_seqlens non-NULL it is the packed-varlen form over
 * total_tokens rows (see selective_state_update_varlen), else the uniform form
 * (total_tokens unused). opt->prefix_lens is ignored.
 */
int selective_state_update_ex(const ssu_problem *p, const ssd_options *opt, int32_t total_tokens,
                              const int32_t *cu_seqlens, void *state_cache,
                              const int32_t *state_indices, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              void *y, void *intermediate_states, void *stream);

/*
 * fp32 -> fp16 of n values with the rounding of the state stores (stream
 * `kind`, element e = index in the array; sr_seed NULL: nearest even). For
 * converting states between caches, and for checking the rounding itself.
 */
int ssd_round_f16(const float *in, void *out, int64_t n, const uint64_t *sr_seed,
                  int32_t sr_rounds, int32_t kind, void *stream);

/*
 * ReplaySSM MTP decode (vLLM PR #52928, sections "Summary" and "Design": each
 * layer keeps a checkpoint state and a ring of the inputs per slot, the
 * accepted length moves a shared cursor before the next forward, and the
 * checkpoint is rewritten only when the next verify window would not fit;
 * vLLM PR #55688, "Summary": pending history is materialised into the
 * checkpoint before a state is published). No state per draft token is
 * written: a rollback is a cursor move.
 *
 * Storage per slot s (caller-owned, ring_len = W entries, W >= 2 T):
 *   ckpt     [num_slots,H,P,N] state_dtype   checkpoint state (the state cache)
 *   ring_x   [num_slots,W,H,P] in_dtype      inputs of the tokens since the
 *   ring_dt  [num_slots,W,H]   in_dtype      checkpoint, ring order
 *   ring_B   [num_slots,W,G,N] in_dtype
 *   cursor   [num_slots,2]     int32         (start, n): the n accepted tokens
 *            not yet in the checkpoint sit at ring positions (start + i) mod W,
 *            i = 0..n-1. A slot whose checkpoint was just written by a prefill
 *            needs cursor (any start, 0). Values out of range are clamped
 *            (start to [0, W), n to [0, W - T]).
 * The current state of slot s is the checkpoint followed by those n tokens.
 * Requests of one call must use distinct slots.
 */

/*
 * Verify step: per request r (slot s = state_indices[r]) and head h, rebuild
 * the current state from ckpt[s] and the n history tokens, then run the T new
 * tokens in float32, writing y_t for each and appending their x, dt, B to the
 * ring at positions (start + n + t) mod W. When n + T > W - T (the window
 * after this one might not fit) the rebuilt state is first rounded into
 * ckpt[s]. The cursor is only read.
 *   x, y [R,T,H,P]; dt [R,T,H]; B, C [R,T,G,N] in_dtype; A, D [H] float32
 *   (D may be NULL)
 */
int ssd_replay_update(const ssu_problem *p, int32_t ring_len, void *ckpt, void *ring_x,
                      void *ring_dt, void *ring_B, const int32_t *cursor,
                      const int32_t *state_indices, const void *x, const void *dt,
                      const float *A, const void *B, const void *C, const float *D, void *y,
                      void *stream);

/*
 * Cursor move after sampling: num_accepted[r] in [0, T) accepted draft tokens
 * (the target token is always kept), so 1 + num_accepted[r] tokens of the
 * last window join the history. With (start, n) the cursor the verify step
 * read: if that step rewrote the checkpoint (n + T > W - T) the cursor becomes
 * ((start + n) mod W, 1 + a), else (start, n + 1 + a). T is the window of that
 * verify step (p->tokens_per_req). Out-of-range counts are clamped.
 */
/* ssd_replay_update / ssd_replay_materialize with stochastic rounding of fp16
 * checkpoints (opt->sr_seed; dt_transform and prefix_lens are not supported). */
int ssd_replay_update_ex(const ssu_problem *p, const ssd_options *opt, int32_t ring_len,
                         void *ckpt, void *ring_x, void *ring_dt, void *ring_B,
                         const int32_t *cursor, const int32_t *state_indices, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *stream);
int ssd_replay_materialize_ex(const ssu_problem *p, const ssd_options *opt, int32_t ring_len,
                              void *ckpt, const void *ring_x, const void *ring_dt,
                              const void *ring_B, int32_t *cursor, const int32_t *state_indices,
                              const float *A, void *stream);

int ssd_replay_advance(const ssu_problem *p, int32_t ring_len, int32_t *cursor,
                       const int32_t *state_indices, const int32_t *num_accepted, void *stream);

/*
 * Materialise: for every request r, fold the history of slot state_indices[r]
 * into its checkpoint (ckpt[s] = rounded current state) and set its cursor to
 * ((start + n) mod W, 0). Two launches on the stream (the cursor is reset
 * after every head has read it). p->tokens_per_req only bounds n (W - T).
 */
int ssd_replay_materialize(const ssu_problem *p, int32_t ring_len, void *ckpt,
                           const void *ring_x, const void *ring_dt, const void *ring_B,
                           int32_t *cursor, const int32_t *state_indices, const float *A,
                           void *stream);

/*
 * ssd_combined_varlen that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Arguments, semantics
 * and results are those of ssd_combined_varlen (the same launches, bit for
 * bit); the workspace is a static device array of the library,
 * SSD_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held on every GPU the library
 * runs on until the process ends. Its device address is looked up on the
 * first call on each device (that device current: the device of `stream`).
 * A problem whose ssd_workspace_bytes exceeds it returns SSD_ERR_SCRATCH and
 * enqueues nothing. All calls on one GPU share that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race on it; calls queued
 * on one stream are safe. The call allocates nothing (no hipMalloc, no
 * library allocation) and needs no clearing of the array.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
size_t ssd_noalloc_scratch_bytes(void);   /* SSD_NOALLOC_SCRATCH_BYTES */
int ssd_combined_varlen_noalloc(const ssd_problem *p, const void *x, const void *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const int32_t *cu_seqlens, void *state_cache,
                                const int32_t *state_indices, const uint8_t *has_initial_state,
                                void *y, void *checkpoints, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
