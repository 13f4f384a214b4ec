// C ABI of the MI355X SSD library: host-side validation, workspace layout and
// dispatch to the kernel launchers. Nothing here reads device memory or
// synchronises; every check runs before the first launch of a call.
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "ssd_launch.h"
#include "../../include/ssd_mi355x.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int32_t d) { return d == SSD_F32 || d == SSD_BF16; }
// states may also be fp16
bool state_dtype_ok(int32_t d) { return dtype_ok(d) || d == SSD_F16; }

bool gpu_shape_ok(int P, int N) { return (P == 16 || P == 64) && (N == 16 || N == 128); }

bool chunk_ok(int Q) { return Q == 32 || Q == 64 || Q == 128 || Q == 256; }

// Shape / dtype checks of a prefill descriptor (no pointers); `aligned`: the
// chunk bound of align mode (T / Q + 2 S), which sizes the grids of that mode.
int check_problem(const ssd_problem *p, bool aligned = false)
{
    if (!p) return SSD_ERR_NULL;
    if (p->total_tokens < 0 || p->num_seqs < 0 || p->nheads <= 0 || p->headdim <= 0 ||
        p->d_state <= 0 || p->ngroups <= 0 || p->chunk_size <= 0 || p->num_slots < 0)
        return SSD_ERR_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_SHAPE;
    if (p->num_seqs > 0 && p->num_slots <= 0) return SSD_ERR_SHAPE;
    if (!dtype_ok(p->in_dtype) || !state_dtype_ok(p->state_dtype)) return SSD_ERR_DTYPE;
    if (!gpu_shape_ok(p->headdim, p->d_state) || !chunk_ok(p->chunk_size)) return SSD_ERR_UNSUPPORTED;
    // grid limits: chunks and heads index grid dimensions
    const int64_t mc = (int64_t)p->total_tokens / p->chunk_size +
                       (aligned ? 2 : 1) * (int64_t)p->num_seqs;
    if (mc > 65535 || p->nheads > 65535) return SSD_ERR_UNSUPPORTED;
    if (mc * p->nheads * 2 > 0x7fffffffLL) return SSD_ERR_UNSUPPORTED;
    if ((int64_t)p->num_seqs * p->nheads * ((p->headdim * p->d_state + 1023) / 1024) > 0x7fffffffLL)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

int check_ssu(const ssu_problem *p)
{
    if (!p) return SSD_ERR_NULL;
    if (p->num_reqs < 0 || p->tokens_per_req < 0 || p->nheads <= 0 || p->headdim <= 0 ||
        p->d_state <= 0 || p->ngroups <= 0 || p->num_slots < 0)
        return SSD_ERR_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_SHAPE;
    if (p->num_reqs > 0 && p->num_slots <= 0) return SSD_ERR_SHAPE;
    if (!dtype_ok(p->in_dtype) || !state_dtype_ok(p->state_dtype)) return SSD_ERR_DTYPE;
    if (!gpu_shape_ok(p->headdim, p->d_state)) return SSD_ERR_UNSUPPORTED;
    if (p->nheads > 0x7fffffff / 2 || p->num_reqs > 65535) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Upper bound on the chunks of a batch: T / Q + S (each sequence adds at most
// one partial chunk), T / Q + 2 S in align mode (a partial chunk at each end).
int64_t max_chunks_of(const ssd_problem *p, bool aligned)
{
    return (int64_t)p->total_tokens / p->chunk_size + (aligned ? 2 : 1) * (int64_t)p->num_seqs;
}

ssd::PrefillDims dims_of(const ssd_problem *p, bool aligned = false)
{
    ssd::PrefillDims d;
    d.T = p->total_tokens;
    d.S = p->num_seqs;
    d.H = p->nheads;
    d.P = p->headdim;
    d.N = p->d_state;
    d.G = p->ngroups;
    d.Q = p->chunk_size;
    d.max_chunks = (int)max_chunks_of(p, aligned);
    d.num_slots = p->num_slots;
    d.in_bf16 = p->in_dtype == SSD_BF16;
    d.state_bf16 = p->state_dtype == SSD_BF16;
    d.state_f16 = p->state_dtype == SSD_F16;
    return d;
}

ssd::DecodeDims dims_of(const ssu_problem *p)
{
    ssd::DecodeDims d;
    d.R = p->num_reqs;
    d.T = p->tokens_per_req;
    d.H = p->nheads;
    d.P = p->headdim;
    d.N = p->d_state;
    d.G = p->ngroups;
    d.num_slots = p->num_slots;
    d.in_bf16 = p->in_dtype == SSD_BF16;
    d.state_bf16 = p->state_dtype == SSD_BF16;
    d.state_f16 = p->state_dtype == SSD_F16;
    return d;
}

// Host copy of the dt preprocessing parameters (NULL transform: rejected).
int dt_tf_of(const ssd_dt_transform *t, ssd::DtTf *out)
{
    if (!t) return SSD_ERR_NULL;
    if (!(t->dt_min <= t->dt_max)) return SSD_ERR_SHAPE;   // (NaN bounds fail too)
    out->bias = t->dt_bias;
    out->lo = t->dt_min;
    out->hi = t->dt_max;
    out->on = 1;
    return SSD_OK;
}

int launch_status()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of ssd_combined_varlen, 256-byte aligned pieces in this order.
struct Workspace {
    size_t meta, cum, dt, cb, states, entering, total;
    // segmented state passing (nseg > 1): per-segment final states, starting
    // states, decays, and per-chunk decay / segment index
    int nseg;
    size_t seg_fin, seg_carry, seg_L, seg_F, seg_I;
};

Workspace workspace_layout(const ssd_problem *p, bool aligned = false)
{
    const size_t mc = (size_t)max_chunks_of(p, aligned);
    const size_t H = p->nheads, P = p->headdim, N = p->d_state, G = p->ngroups, Q = p->chunk_size;
    Workspace w;
    w.meta = 0;
    w.cum = w.meta + round_up(sizeof(int32_t) * (3 * (size_t)p->num_seqs + 2 + 3 * mc));
    w.dt = w.cum + round_up(sizeof(float) * H * mc * Q);
    w.cb = w.dt + round_up(sizeof(float) * H * mc * Q);
    const size_t ein = p->in_dtype == SSD_BF16 ? 2 : 4;
    w.states = w.cb + round_up(ein * mc * G * Q * Q);
    // the fused state kernel keeps chunk states in registers: no buffer for them
    const size_t nstates = ssd::fused_state_path(dims_of(p)) ? 0 : mc * H * P * N;
    w.entering = w.states + round_up(sizeof(float) * nstates);
    w.seg_fin = w.entering + round_up(ein * mc * H * P * N);
    w.nseg = ssd::state_segments(dims_of(p, aligned));
    const size_t nsb = w.nseg > 1 ? (size_t)p->num_seqs * w.nseg : 0;
    const size_t nsc = w.nseg > 1 ? mc : 0;
    w.seg_carry = w.seg_fin + round_up(sizeof(float) * nsb * H * P * N);
    w.seg_L = w.seg_carry + round_up(2 * nsb * H * P * N);
    w.seg_F = w.seg_L + round_up(sizeof(float) * nsb * H);
    w.seg_I = w.seg_F + round_up(sizeof(float) * nsc * H);
    w.total = w.seg_I + round_up(sizeof(int32_t) * nsc);
    return w;
}

}  // namespace

namespace ssd {

bool trace_events(ssd_launch_trace *t, const char *name, void **start, void **stop)
{
    if (!t) return false;
    const int k = t->count++;
    if (k < SSD_TRACE_MAX_LAUNCHES) t->names[k] = name;
    if (!t->events || 2 * (int64_t)k + 1 >= t->capacity) return false;
    *start = t->events[2 * k];
    *stop = t->events[2 * k + 1];
    return true;
}

}  // namespace ssd

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char *ssd_status_string(int status)
{
    switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid sizes";
    case SSD_ERR_DTYPE: return "unknown dtype";
    case SSD_ERR_UNSUPPORTED: return "shape not supported by the GPU kernels";
    case SSD_ERR_WORKSPACE: return "workspace too small";
    case SSD_ERR_HIP: return "HIP launch failure";
    case SSD_ERR_ALIGN: return "array pointer not 16-byte aligned";
    case SSD_ERR_SCRATCH: return "problem needs more workspace than the no-alloc scratch array holds";
    default: return "unknown status";
    }
}

int64_t ssd_max_chunks(const ssd_problem *p)
{
    if (check_problem(p) != SSD_OK) return 0;
    return (int64_t)p->total_tokens / p->chunk_size + p->num_seqs;
}

int64_t ssd_chunk_meta_count(const ssd_problem *p)
{
    if (check_problem(p) != SSD_OK) return 0;
    return 3 * (int64_t)p->num_seqs + 2 + 3 * ssd_max_chunks(p);
}

size_t ssd_workspace_bytes(const ssd_problem *p)
{
    if (check_problem(p) != SSD_OK) return 0;
    return workspace_layout(p).total;
}

int ssd_chunk_cumsum(const ssd_problem *p, const void *dt, const float *A,
                     const int32_t *cu_seqlens, int32_t *chunk_meta, float *dA_cumsum,
                     float *dt_chunk, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!dt || !A || !cu_seqlens || !chunk_meta || !dA_cumsum || !dt_chunk) return SSD_ERR_NULL;
    if (!aligned16(dA_cumsum) || !aligned16(dt_chunk)) return SSD_ERR_ALIGN;
    ssd::launch_chunk_cumsum(dims_of(p), dt, A, cu_seqlens, chunk_meta, dA_cumsum, dt_chunk, stream);
    return launch_status();
}

int ssd_chunk_cumsum_dt(const ssd_problem *p, const ssd_dt_transform *dt_transform,
                        const void *dt_raw, const float *A, const int32_t *cu_seqlens,
                        int32_t *chunk_meta, float *dA_cumsum, float *dt_chunk, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    ssd::DtTf tf;
    rc = dt_tf_of(dt_transform, &tf);
    if (rc) return rc;
    if (!dt_raw || !A || !cu_seqlens || !chunk_meta || !dA_cumsum || !dt_chunk) return SSD_ERR_NULL;
    if (!aligned16(dA_cumsum) || !aligned16(dt_chunk)) return SSD_ERR_ALIGN;
    ssd::launch_chunk_cumsum(dims_of(p), dt_raw, A, cu_seqlens, chunk_meta, dA_cumsum, dt_chunk,
                             stream, tf);
    return launch_status();
}

int ssd_chunk_state(const ssd_problem *p, const void *x, const void *B,
                    const int32_t *chunk_meta, const float *dA_cumsum, const float *dt_chunk,
                    float *chunk_states, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!x || !B || !chunk_meta || !dA_cumsum || !dt_chunk || !chunk_states) return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(B) || !aligned16(chunk_states)) return SSD_ERR_ALIGN;
    ssd::launch_chunk_state(dims_of(p), x, B, chunk_meta, dA_cumsum, dt_chunk, chunk_states, stream);
    return launch_status();
}

int ssd_state_passing(const ssd_problem *p, const float *chunk_states, const float *dA_cumsum,
                      const int32_t *chunk_meta, void *state_cache,
                      const int32_t *state_indices, const uint8_t *has_initial_state,
                      void *entering_states, void *checkpoints, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!chunk_states || !dA_cumsum || !chunk_meta || !state_cache || !state_indices ||
        !entering_states)
        return SSD_ERR_NULL;
    if (!aligned16(chunk_states) || !aligned16(state_cache) || !aligned16(entering_states) ||
        !aligned16(checkpoints))
        return SSD_ERR_ALIGN;
    ssd::launch_state_passing(dims_of(p), chunk_states, dA_cumsum, chunk_meta, state_cache,
                              state_indices, has_initial_state, entering_states, checkpoints,
                              stream);
    return launch_status();
}

int ssd_chunk_state_passing(const ssd_problem *p, const void *x, const void *B,
                            const int32_t *chunk_meta, const float *dA_cumsum,
                            const float *dt_chunk, void *state_cache,
                            const int32_t *state_indices, const uint8_t *has_initial_state,
                            void *entering_states, void *checkpoints, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    const ssd::PrefillDims d = dims_of(p);
    if (!ssd::fused_state_path(d)) return SSD_ERR_UNSUPPORTED;
    if (!x || !B || !chunk_meta || !dA_cumsum || !dt_chunk || !state_cache || !state_indices ||
        !entering_states)
        return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(B) || !aligned16(state_cache) ||
        !aligned16(entering_states) || !aligned16(checkpoints))
        return SSD_ERR_ALIGN;
    ssd::launch_state_scan(d, x, B, chunk_meta, dA_cumsum, dt_chunk, state_cache, state_indices,
                           has_initial_state, entering_states, checkpoints, stream);
    return launch_status();
}

int ssd_bmm_chunk(const ssd_problem *p, const void *B, const void *C,
                  const int32_t *chunk_meta, void *CB, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!B || !C || !chunk_meta || !CB) return SSD_ERR_NULL;
    if (!aligned16(B) || !aligned16(C) || !aligned16(CB)) return SSD_ERR_ALIGN;
    ssd::launch_bmm(dims_of(p), B, C, chunk_meta, CB, stream);
    return launch_status();
}

int ssd_chunk_scan(const ssd_problem *p, const void *x, const void *C, const float *D,
                   const int32_t *chunk_meta, const float *dA_cumsum, const float *dt_chunk,
                   const void *CB, const void *entering_states, void *y, void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!x || !C || !chunk_meta || !dA_cumsum || !dt_chunk || !CB || !entering_states || !y)
        return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(C) || !aligned16(CB) || !aligned16(entering_states) ||
        !aligned16(y))
        return SSD_ERR_ALIGN;
    ssd::launch_chunk_scan(dims_of(p), x, C, D, chunk_meta, dA_cumsum, dt_chunk, CB,
                           entering_states, y, stream);
    return launch_status();
}

static int combined(const ssd_problem *p, const ssd::DtTf &tf, const void *x, const void *dt,
                    const float *A, const void *B, const void *C, const float *D,
                    const int32_t *cu_seqlens, void *state_cache, const int32_t *state_indices,
                    const uint8_t *has_initial_state, void *y, void *checkpoints, void *workspace,
                    size_t workspace_bytes, void *stream, const int32_t *prefix = nullptr,
                    const ssd::SrCtx &sr = ssd::SrCtx(), ssd_launch_trace *trace = nullptr)
{
    const bool aligned = prefix != nullptr;
    int rc = check_problem(p, aligned);
    if (rc) return rc;
    if (!x || !dt || !A || !B || !C || !cu_seqlens || !state_cache || !state_indices || !y ||
        !workspace)
        return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
        !aligned16(state_cache) || !aligned16(checkpoints) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return SSD_ERR_ALIGN;
    const Workspace w = workspace_layout(p, aligned);
    if (workspace_bytes < w.total) return SSD_ERR_WORKSPACE;

    ssd::PrefillDims d = dims_of(p, aligned);
    d.prefix = prefix;
    d.sr = sr;
    d.trace = trace;
    if (trace) trace->count = 0;
    // short sequences: one launch, no workspace
    if (ssd::short_scan_path(d)) {
        ssd::launch_short_scan(d, x, dt, A, B, C, D, cu_seqlens, state_cache, state_indices,
                               has_initial_state, y, checkpoints, stream, tf);
        return launch_status();
    }
    char *base = static_cast<char *>(workspace);
    int32_t *meta = reinterpret_cast<int32_t *>(base + w.meta);
    float *cum = reinterpret_cast<float *>(base + w.cum);
    float *dtc = reinterpret_cast<float *>(base + w.dt);
    void *cb = base + w.cb;
    float *states = reinterpret_cast<float *>(base + w.states);
    void *entering = base + w.entering;

    // segmented state passing when the state kernel alone would leave CUs idle
    // (not with checkpoints, which need every chunk's true state in that kernel)
    ssd::SegBufs seg;
    if (w.nseg > 1 && !checkpoints) {
        seg.nseg = w.nseg;
        seg.fin = reinterpret_cast<float *>(base + w.seg_fin);
        seg.carry = base + w.seg_carry;
        seg.L = reinterpret_cast<float *>(base + w.seg_L);
        seg.F = reinterpret_cast<float *>(base + w.seg_F);
        seg.I = reinterpret_cast<int32_t *>(base + w.seg_I);
    }
    // few sequences: steps 1 and 4 inside the state launch, so the call is two
    // launches, or three with the carry step of a segmented state pass
    if (ssd::own_prep_path(d)) {
        ssd::OwnPrep own;
        own.dt = dt;
        own.A = A;
        own.cu = cu_seqlens;
        own.tf = tf;
        own.meta = meta;
        own.cum = cum;
        own.dtc = dtc;
        own.C = C;
        own.CB = cb;
        ssd::launch_state_scan(d, x, B, meta, cum, dtc, state_cache, state_indices,
                               has_initial_state, entering, checkpoints, stream, &seg, &own);
        ssd::launch_chunk_scan(d, x, C, D, meta, cum, dtc, cb, entering, y, stream, &seg);
        return launch_status();
    }
    // (more sequences: never segmented, see state_segments) steps 1 and 4 in one
    // launch, or, with many (chunk, group) pairs, step 4 one pair per block after
    // step 1
    if (ssd::cb_by_pair(d)) {
        ssd::launch_chunk_cumsum(d, dt, A, cu_seqlens, meta, cum, dtc, stream, tf);
        ssd::launch_bmm(d, B, C, meta, cb, stream);
    } else {
        ssd::launch_chunk_prep(d, dt, A, cu_seqlens, meta, cum, dtc, B, C, cb, stream, tf);
    }
    if (ssd::fused_state_path(d)) {
        ssd::launch_state_scan(d, x, B, meta, cum, dtc, state_cache, state_indices,
                               has_initial_state, entering, checkpoints, stream);
    } else {
        ssd::launch_chunk_state(d, x, B, meta, cum, dtc, states, stream);
        ssd::launch_state_passing(d, states, cum, meta, state_cache, state_indices,
                                  has_initial_state, entering, checkpoints, stream);
    }
    ssd::launch_chunk_scan(d, x, C, D, meta, cum, dtc, cb, entering, y, stream);
    return launch_status();
}

int ssd_combined_varlen(const ssd_problem *p, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D, const int32_t *cu_seqlens,
                        void *state_cache, const int32_t *state_indices,
                        const uint8_t *has_initial_state, void *y, void *checkpoints,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    return combined(p, ssd::DtTf(), x, dt, A, B, C, D, cu_seqlens, state_cache, state_indices,
                    has_initial_state, y, checkpoints, workspace, workspace_bytes, stream);
}

// Stochastic rounding parameters of an options struct (fp16 states only).
static int sr_of(const ssd_options *o, int32_t state_dtype, ssd::SrCtx *sr)
{
    if (!o || !o->sr_seed) return SSD_OK;
    if (state_dtype != SSD_F16) return SSD_ERR_UNSUPPORTED;
    if (o->sr_rounds < 1 || o->sr_rounds > 16) return SSD_ERR_SHAPE;
    sr->seed = o->sr_seed;
    sr->rounds = o->sr_rounds;
    return SSD_OK;
}

int ssd_combined_varlen_ex(const ssd_problem *p, const ssd_options *opt, const void *x,
                           const void *dt, const float *A, const void *B, const void *C,
                           const float *D, const int32_t *cu_seqlens, void *state_cache,
                           const int32_t *state_indices, const uint8_t *has_initial_state,
                           void *y, void *checkpoints, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    int rc = check_problem(p);
    if (rc) return rc;
    ssd::DtTf tf;
    ssd::SrCtx sr;
    if (opt && opt->dt_transform) {
        rc = dt_tf_of(opt->dt_transform, &tf);
        if (rc) return rc;
    }
    rc = sr_of(opt, p->state_dtype, &sr);
    if (rc) return rc;
    return combined(p, tf, x, dt, A, B, C, D, cu_seqlens, state_cache, state_indices,
                    has_initial_state, y, checkpoints, workspace, workspace_bytes, stream,
                    opt ? opt->prefix_lens : nullptr, sr, opt ? opt->trace : nullptr);
}

int64_t ssd_max_chunks_aligned(const ssd_problem *p)
{
    if (check_problem(p, true) != SSD_OK) return 0;
    return max_chunks_of(p, true);
}

size_t ssd_workspace_bytes_aligned(const ssd_problem *p)
{
    if (check_problem(p, true) != SSD_OK) return 0;
    return workspace_layout(p, true).total;
}

int ssd_combined_varlen_aligned(const ssd_problem *p, const int32_t *prefix_lens, const void *x,
                                const void *dt, const float *A, const void *B, const void *C,
                                const float *D, const int32_t *cu_seqlens, void *state_cache,
                                const int32_t *state_indices, const uint8_t *has_initial_state,
                                void *y, void *checkpoints, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    if (!prefix_lens) return SSD_ERR_NULL;
    return combined(p, ssd::DtTf(), x, dt, A, B, C, D, cu_seqlens, state_cache, state_indices,
                    has_initial_state, y, checkpoints, workspace, workspace_bytes, stream,
                    prefix_lens);
}

int ssd_combined_varlen_dt(const ssd_problem *p, const ssd_dt_transform *dt_transform,
                           const void *x, const void *dt_raw, const float *A, const void *B,
                           const void *C, const float *D, const int32_t *cu_seqlens,
                           void *state_cache, const int32_t *state_indices,
                           const uint8_t *has_initial_state, void *y, void *checkpoints,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    ssd::DtTf tf;
    const int rc = dt_tf_of(dt_transform, &tf);
    if (rc) return rc;
    return combined(p, tf, x, dt_raw, A, B, C, D, cu_seqlens, state_cache, state_indices,
                    has_initial_state, y, checkpoints, workspace, workspace_bytes, stream);
}

int selective_state_update(const ssu_problem *p, void *state_cache, const int32_t *state_indices,
                           const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, void *y, void *intermediate_states,
                           void *stream)
{
    int rc = check_ssu(p);
    if (rc) return rc;
    if (!state_cache || !state_indices || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    if (!aligned16(state_cache) || !aligned16(B) || !aligned16(C) ||
        !aligned16(intermediate_states))
        return SSD_ERR_ALIGN;
    ssd::launch_state_update(dims_of(p), state_cache, state_indices, x, dt, A, B, C, D, y,
                             intermediate_states, stream);
    return launch_status();
}

int ssd_state_commit(const ssu_problem *p, void *state_cache, const int32_t *state_indices,
                     const void *intermediate_states, const int32_t *num_accepted, void *stream)
{
    int rc = check_ssu(p);
    if (rc) return rc;
    if (!state_cache || !state_indices || !intermediate_states || !num_accepted) return SSD_ERR_NULL;
    if (!aligned16(state_cache) || !aligned16(intermediate_states)) return SSD_ERR_ALIGN;
    ssd::launch_state_commit(dims_of(p), state_cache, state_indices, intermediate_states,
                             num_accepted, stream);
    return launch_status();
}

int selective_state_update_varlen(const ssu_problem *p, int32_t total_tokens,
                                  const int32_t *cu_seqlens,
                                  const ssd_dt_transform *dt_transform, void *state_cache,
                                  const int32_t *state_indices, const void *x, const void *dt,
                                  const float *A, const void *B, const void *C, const float *D,
                                  void *y, void *intermediate_states, void *stream)
{
    int rc = check_ssu(p);
    if (rc) return rc;
    if (p->tokens_per_req < 1 || total_tokens < 0) return SSD_ERR_SHAPE;
    ssd::DtTf tf;
    if (dt_transform) {
        rc = dt_tf_of(dt_transform, &tf);
        if (rc) return rc;
    }
    if (!cu_seqlens || !state_cache || !state_indices || !x || !dt || !A || !B || !C || !y)
        return SSD_ERR_NULL;
    if (!aligned16(state_cache) || !aligned16(B) || !aligned16(C) ||
        !aligned16(intermediate_states))
        return SSD_ERR_ALIGN;
    if (total_tokens == 0) return SSD_OK;
    ssd::launch_state_update(dims_of(p), state_cache, state_indices, x, dt, A, B, C, D, y,
                             intermediate_states, stream, cu_seqlens, total_tokens, tf);
    return launch_status();
}

int selective_state_update_ex(const ssu_problem *p, const ssd_options *opt, int32_t total_tokens,
                              const int32_t *cu_seqlens, void *state_cache,
                              const int32_t *state_indices, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              void *y, void *intermediate_states, void *stream)
{
    int rc = check_ssu(p);
    if (rc) return rc;
    if (p->tokens_per_req < 1 && cu_seqlens) return SSD_ERR_SHAPE;
    if (total_tokens < 0) return SSD_ERR_SHAPE;
    ssd::DtTf tf;
    ssd::SrCtx sr;
    if (opt && opt->dt_transform) {
        rc = dt_tf_of(opt->dt_transform, &tf);
        if (rc) return rc;
    }
    rc = sr_of(opt, p->state_dtype, &sr);
    if (rc) return rc;
    if (!state_cache || !state_indices || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
    if (!aligned16(state_cache) || !aligned16(B) || !aligned16(C) ||
        !aligned16(intermediate_states))
        return SSD_ERR_ALIGN;
    ssd::DecodeDims d = dims_of(p);
    d.sr = sr;
    if (cu_seqlens) {
        if (total_tokens == 0) return SSD_OK;
        ssd::launch_state_update(d, state_cache, state_indices, x, dt, A, B, C, D, y,
                                 intermediate_states, stream, cu_seqlens, total_tokens, tf);
    } else {
        ssd::launch_state_update(d, state_cache, state_indices, x, dt, A, B, C, D, y,
                                 intermediate_states, stream, nullptr, 0, tf);
    }
    return launch_status();
}

int ssd_round_f16(const float *in, void *out, int64_t n, const uint64_t *sr_seed,
                  int32_t sr_rounds, int32_t kind, void *stream)
{
    if (n < 0) return SSD_ERR_SHAPE;
    if (n == 0) return SSD_OK;
    if (!in || !out) return SSD_ERR_NULL;
    if (sr_seed && (sr_rounds < 1 || sr_rounds > 16)) return SSD_ERR_SHAPE;
    ssd::SrCtx sr;
    sr.seed = sr_seed;
    sr.rounds = sr_seed ? sr_rounds : 0;
    ssd::launch_round_f16(in, out, n, sr, kind, stream);
    return launch_status();
}

int ssd_state_commit_varlen(const ssu_problem *p, int32_t total_tokens,
                            const int32_t *cu_seqlens, void *state_cache,
                            const int32_t *state_indices, const void *intermediate_states,
                            const int32_t *num_accepted, void *stream)
{
    int rc = check_ssu(p);
    if (rc) return rc;
    if (p->tokens_per_req < 1 || total_tokens < 0) return SSD_ERR_SHAPE;
    if (!cu_seqlens || !state_cache || !state_indices || !intermediate_states || !num_accepted)
        return SSD_ERR_NULL;
    if (!aligned16(state_cache) || !aligned16(intermediate_states)) return SSD_ERR_ALIGN;
    if (total_tokens == 0) return SSD_OK;
    ssd::launch_state_commit(dims_of(p), state_cache, state_indices, intermediate_states,
                             num_accepted, stream, cu_seqlens, total_tokens);
    return launch_status();
}

static int check_replay(const ssu_problem *p, int32_t ring_len)
{
    int rc = check_ssu(p);
    if (rc) return rc;
    // the history (W - T entries) must hold a whole window: W >= 2 T
    if (ring_len <= 0 || (int64_t)ring_len < 2 * (int64_t)p->tokens_per_req) return SSD_ERR_SHAPE;
    return SSD_OK;
}

int ssd_replay_update(const ssu_problem *p, int32_t ring_len, void *ckpt, void *ring_x,
                      void *ring_dt, void *ring_B, const int32_t *cursor,
                      const int32_t *state_indices, const void *x, const void *dt,
                      const float *A, const void *B, const void *C, const float *D, void *y,
                      void *stream)
{
    int rc = check_replay(p, ring_len);
    if (rc) return rc;
    if (!ckpt || !ring_x || !ring_dt || !ring_B || !cursor || !state_indices || !x || !dt || !A ||
        !B || !C || !y)
        return SSD_ERR_NULL;
    if (!aligned16(ckpt) || !aligned16(ring_x) || !aligned16(ring_B) || !aligned16(x) ||
        !aligned16(B) || !aligned16(C))
        return SSD_ERR_ALIGN;
    ssd::launch_replay_update(dims_of(p), ring_len, ckpt, ring_x, ring_dt, ring_B, cursor,
                              state_indices, x, dt, A, B, C, D, y, stream);
    return launch_status();
}

int ssd_replay_update_ex(const ssu_problem *p, const ssd_options *opt, int32_t ring_len,
                         void *ckpt, void *ring_x, void *ring_dt, void *ring_B,
                         const int32_t *cursor, const int32_t *state_indices, const void *x,
                         const void *dt, const float *A, const void *B, const void *C,
                         const float *D, void *y, void *stream)
{
    int rc = check_replay(p, ring_len);
    if (rc) return rc;
    if (opt && (opt->dt_transform || opt->prefix_lens)) return SSD_ERR_UNSUPPORTED;
    ssd::SrCtx sr;
    rc = sr_of(opt, p->state_dtype, &sr);
    if (rc) return rc;
    if (!ckpt || !ring_x || !ring_dt || !ring_B || !cursor || !state_indices || !x || !dt || !A ||
        !B || !C || !y)
        return SSD_ERR_NULL;
    if (!aligned16(ckpt) || !aligned16(ring_x) || !aligned16(ring_B) || !aligned16(x) ||
        !aligned16(B) || !aligned16(C))
        return SSD_ERR_ALIGN;
    ssd::DecodeDims d = dims_of(p);
    d.sr = sr;
    ssd::launch_replay_update(d, ring_len, ckpt, ring_x, ring_dt, ring_B, cursor, state_indices,
                              x, dt, A, B, C, D, y, stream);
    return launch_status();
}

int ssd_replay_materialize_ex(const ssu_problem *p, const ssd_options *opt, int32_t ring_len,
                              void *ckpt, const void *ring_x, const void *ring_dt,
                              const void *ring_B, int32_t *cursor, const int32_t *state_indices,
                              const float *A, void *stream)
{
    int rc = check_replay(p, ring_len);
    if (rc) return rc;
    if (opt && (opt->dt_transform || opt->prefix_lens)) return SSD_ERR_UNSUPPORTED;
    ssd::SrCtx sr;
    rc = sr_of(opt, p->state_dtype, &sr);
    if (rc) return rc;
    if (!ckpt || !ring_x || !ring_dt || !ring_B || !cursor || !state_indices || !A)
        return SSD_ERR_NULL;
    if (!aligned16(ckpt) || !aligned16(ring_x) || !aligned16(ring_B)) return SSD_ERR_ALIGN;
    ssd::DecodeDims d = dims_of(p);
    d.sr = sr;
    ssd::launch_replay_materialize(d, ring_len, ckpt, ring_x, ring_dt, ring_B, cursor,
                                   state_indices, A, stream);
    return launch_status();
}

int ssd_replay_advance(const ssu_problem *p, int32_t ring_len, int32_t *cursor,
                       const int32_t *state_indices, const int32_t *num_accepted, void *stream)
{
    int rc = check_replay(p, ring_len);
    if (rc) return rc;
    if (!cursor || !state_indices || !num_accepted) return SSD_ERR_NULL;
    ssd::launch_replay_advance(dims_of(p), ring_len, cursor, state_indices, num_accepted, stream);
    return launch_status();
}

int ssd_replay_materialize(const ssu_problem *p, int32_t ring_len, void *ckpt,
                           const void *ring_x, const void *ring_dt, const void *ring_B,
                           int32_t *cursor, const int32_t *state_indices, const float *A,
                           void *stream)
{
    int rc = check_replay(p, ring_len);
    if (rc) return rc;
    if (!ckpt || !ring_x || !ring_dt || !ring_B || !cursor || !state_indices || !A)
        return SSD_ERR_NULL;
    if (!aligned16(ckpt) || !aligned16(ring_x) || !aligned16(ring_B)) return SSD_ERR_ALIGN;
    ssd::launch_replay_materialize(dims_of(p), ring_len, ckpt, ring_x, ring_dt, ring_B, cursor,
                                   state_indices, A, stream);
    return launch_status();
}

}  // extern "C"
