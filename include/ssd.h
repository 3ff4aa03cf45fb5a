/*
 * ssd.h -- C ABI of libssd, the MI355X (gfx950) Mamba-2 SSD chunked forward pass.
 *
 * The method (source: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核"):
 * the recurrence of section "Mamba-2 架构",
 *     h_t = exp(A dt_t) h_{t-1} + dt_t x_t (outer) B_t,   y_t = h_t . C_t + D x_t,
 * is evaluated chunk by chunk in three stages (end of section "Mamba-2 架构"):
 *   1. ssd_chunk_cumsum  -- section "Kernel 1": chunk-local cumsum of A*dt, times log2(e);
 *   2. ssd_state_pass    -- section "Kernel 2: fwd_pass_state": the state at every chunk
 *                           start, by the jump h_next = exp(G_last) h + (exp(G_last - G) dt B)^T X;
 *   3. ssd_chunk_out     -- section "Kernel 3：compute_out": per chunk
 *                           Y = exp(G) C h^T + (exp(G_i - G_j) (C B^T) causal-mask) (dt X) + D X.
 * ssd_forward runs the three in order on one stream.  ssd_step advances the
 * recurrence by one token per sequence (decode), continuing from the final state.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes use b = batch, L = seqlen, H = nheads, G = ngroups, P = headdim, N = dstate,
 * Q = chunk, nc = ceil(L / Q), Lp = nc * Q.  All arrays are dense, row-major and
 * contiguous, in *device* memory owned by the caller:
 *     x, y    [b, L, H, P]      element type `dtype`
 *     dt      [b, L, H]         element type `dtype`
 *     B, C    [b, L, G, N]      element type `dtype`; head h reads group h / (H / G)
 *     A, D    [H]               float32 (per-head decay rate and skip weight)
 *     h0, hT  [b, H, P, N]      float32 (initial and final state)
 *     G2, dtT [b, H, Lp]        float32 (stage-1 outputs, token-contiguous per head)
 *     S       [b, H, nc, P, N]  bfloat16 when dtype is SSD_BF16, float32 when SSD_F32
 * `problem` is a host pointer.  `stream` is a hipStream_t (NULL = the null stream).
 *
 * Alignment: x, y, B, C, S, G2, dtT, h0, hT, h and the workspace are read or
 * written with 8- and 16-byte vector accesses and must start on a 16-byte boundary
 * (hipMalloc and torch allocations do); dt, A and D need only their element
 * alignment.  A misaligned pointer returns SSD_ERR_MISALIGNED.
 *
 * Every call validates its arguments on the host before any launch and returns a
 * status; nothing is launched when it is not SSD_OK.  The library never allocates
 * device memory (and no host memory either, except ssd_plan_candidates, a host-only
 * query that builds its list on the host heap), never synchronises and keeps no
 * global mutable state apart from the
 * thread-local HIP error code and the static scratch of ssd_forward_noalloc (a
 * device array that the code object holds on each GPU, plus its per-device address).  Work is asynchronous on `stream`; buffers must stay
 * valid until it completes.  Inputs and outputs must not overlap, except that
 * h0 and hT may be the same buffer.  Since a call issues only kernel launches (no
 * allocation, memset, copy or synchronisation), ssd_forward, the three stages and
 * ssd_step may be recorded into a HIP graph on a capturing stream and replayed.
 *
 * Supported set: dtype SSD_F32 or SSD_BF16; headdim 64; dstate a multiple of 64
 * up to 512; chunk 64, 128 or 256; batch * nheads <= 65535; seqlen * nheads * headdim
 * and seqlen * ngroups * dstate below 2^30; chunk * nheads * headdim and chunk *
 * ngroups * dstate below 2^31; ceil(seqlen / chunk) * batch * nheads below 2^31 / chunk
 * (the one-head output kernel's grid of 2 * chunk threads per workgroup, counted in 32
 * bits); any seqlen >= 1 (a partial last chunk is
 * zero-padded, which is exact: a token with dt = 0 and x = B = C = 0 changes
 * nothing).  Other shapes return SSD_ERR_UNSUPPORTED.
 *
 * Numerics: for SSD_BF16 the matrix products take bf16 operands with fp32
 * accumulation, the running state is fp32, the chunk-start states S are stored in
 * bf16 (the output stage reads them in the input precision) and y is rounded to
 * bf16 (round to nearest even).  For SSD_F32 everything stays fp32.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,     /* a required pointer is NULL                          */
    SSD_ERR_BAD_SHAPE = 2,    /* a dimension <= 0, or nheads not divisible by ngroups */
    SSD_ERR_UNSUPPORTED = 3,  /* outside the supported dtype / headdim / dstate / chunk set */
    SSD_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than ssd_workspace_bytes() */
    SSD_ERR_HIP = 5,          /* a HIP launch failed; see ssd_last_hip_error()        */
    SSD_ERR_MISALIGNED = 6,   /* a vector-accessed array does not start on 16 bytes  */
    SSD_ERR_SCRATCH = 7,      /* ssd_forward_noalloc: the problem needs more than
                                 SSD_SCRATCH_BYTES of workspace                         */
    SSD_ERR_PLAN = 8          /* a launch plan the kernels cannot run for the problem   */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
    int64_t batch, seqlen, nheads, ngroups, headdim, dstate, chunk;
    int32_t dtype;            /* an ssd_dtype value */
} ssd_problem;

/* Host-only checks of `problem` (dimensions, divisibility, supported set).  No GPU. */
ssd_status ssd_validate(const ssd_problem *problem);

/* Bytes of device workspace ssd_forward needs (G2, dtT, S and the state pass's group
 * state, each 256-byte aligned); 0 if `problem` is not valid.  Host-only. */
size_t ssd_workspace_bytes(const ssd_problem *problem);

/* Stage 1 (section "Kernel 1：计算累积和"): for each (b, h) and token t of chunk c,
 *     G2[b,h,t]  = log2(e) * sum_{k = cQ .. t} A[h] * dt[b,k,h]     (fp32 sum, then scaled)
 *     dtT[b,h,t] = float(dt[b,t,h])
 * For padded positions t >= L: dtT = 0 and G2 repeats the chunk's last valid value (so
 * G2 at a chunk's last position is the cumsum at its last valid token).
 * Reads dt, A; writes G2 and dtT ([b, H, Lp]). */
ssd_status ssd_chunk_cumsum(const ssd_problem *problem, const void *dt, const float *A,
                            float *G2, float *dtT, void *stream);

/* Stage 2 (section "Kernel 2: fwd_pass_state", the decayed chunk jump): serially over
 * chunks c, S[b,h,c] = h (the state at the chunk start, h = h0 or 0 for c = 0), then
 *     h <- exp2(G2_last) h + Xw_c^T B_c,   Xw_c[t,p] = round(w_t x[t,p]),
 *     w_t = dtT_t exp2(G2_last - G2_t)   (token t's dt times its decay to the chunk's end)
 * with G2_last = G2 at the chunk's last position.  The weight w_t multiplies the
 * 64-wide x row (rounded to the input type) instead of the N-wide B row; the product
 * is the same sum of w_t x[t,p] B[t,n].
 * After the last chunk hT = h (skipped when hT is NULL).  h0 may be NULL (zero
 * initial state).  Reads x, B, G2, dtT, h0; writes S, hT. */
ssd_status ssd_state_pass(const ssd_problem *problem, const void *x, const void *B,
                          const float *G2, const float *dtT, const float *h0, void *S,
                          float *hT, void *stream);

/* Stage 3 (section "Kernel 3：compute_out", the decayed chunk output): for each chunk,
 *     y_i = exp2(G2_i) C_i . S_c^T
 *         + sum_{j <= i in the chunk} exp2(G2_i - G2_j) (C_i . B_j) dt_j x_j
 *         + D[h] x_i
 * with the causal mask applied by selection (masked exponents never reach the sum).
 * C B^T, the decay matrix and C S^T live only in registers and LDS.  Reads x, B, C,
 * G2, dtT, S, D; writes y. */
ssd_status ssd_chunk_out(const ssd_problem *problem, const void *x, const void *B,
                         const void *C, const float *G2, const float *dtT, const void *S,
                         const float *D, void *y, void *stream);

/* The whole forward pass: stage 1, 2 and 3 on `stream`, no host synchronisation.
 * `workspace` (device, >= ssd_workspace_bytes(problem) bytes) holds the intermediates.
 * On return G2 and dtT hold the stage-1 outputs.  The state pass may split each
 * (batch, head) chain of chunks into groups that run in parallel from a zero state (the
 * jump is linear), combine the group-final states with a short scan and let stage 3 add
 * the carried-in state; S then holds chunk-start states relative to their group (the
 * first chunk of every group after the first, whose state is zero, is not written), and
 * its contents are otherwise unspecified.  Short fp32 problems (see ssd_launch_plan.fused)
 * run as one launch that writes G2, dtT, y and hT and leaves S unwritten (with h0 and hT the
 * same buffer they run the four-launch plan of one serial chain instead).  h0 may be NULL;
 * hT may be NULL (final state not wanted).  Writes y and hT. */
ssd_status ssd_forward(const ssd_problem *problem, const void *x, const void *dt,
                       const float *A, const void *B, const void *C, const float *D,
                       const float *h0, void *y, float *hT, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ssd_forward with timing marks, for profiling the forward pass as it runs.
 * `events` holds SSD_FORWARD_EVENTS (5) hipEvent_t handles created by the caller;
 * they are recorded on `stream` right before stage 1, after stage 1, after the
 * state pass, after the group scan (recorded straight after the previous mark when
 * the state pass runs as one serial chain and no scan is launched) and after stage
 * 3, so each pair of consecutive marks brackets exactly one kernel launch (or
 * none; under the one-launch plan the first four marks follow one another and the last
 * pair brackets the one kernel).  events == NULL behaves exactly like ssd_forward. */
#define SSD_FORWARD_EVENTS 5

/* One of the four launches of ssd_forward, alone: stage 0 the chunk cumsum, 1 the state
 * pass, 2 the group scan (no launch when the state pass runs as one serial chain), 3 the
 * chunk output; ssd_forward issues stages 0, 1, 2, 3 in this order on one workspace.
 * For timing one kernel by itself: a stage reads the inputs and what the earlier stages
 * left in `workspace` (filled by a previous ssd_forward or by the earlier stages of the
 * same problem and inputs) and recomputes its own results, so stages 0, 1 and 3 may be
 * repeated back to back (stage 1 writes hT when it runs as one chain: h0 and hT must not
 * be the same buffer then).  Stage 2 rewrites part of the workspace in place and belongs
 * once after each stage 1; after a repeated stage 1, run stage 2 before stage 3.  A stage
 * outside 0..3 returns SSD_ERR_UNSUPPORTED.  Under the one-launch plan stages 0, 1 and 2
 * launch nothing and stage 3 is the whole forward.  Other arguments and errors as for
 * ssd_forward. */
ssd_status ssd_forward_stage(const ssd_problem *problem, const void *x, const void *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const float *h0, void *y, float *hT, void *workspace,
                             size_t workspace_bytes, int stage, void *stream);
ssd_status ssd_forward_timed(const ssd_problem *problem, const void *x, const void *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const float *h0, void *y, float *hT, void *workspace,
                             size_t workspace_bytes, void *stream, void *const *events);

/* ssd_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels
 * and results as ssd_forward, with the workspace taken from a static device array of
 * SSD_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends.  It calls no allocating routine; the caller still provides every input and
 * output.  The array is the one of the stream's device (the current device for the
 * NULL stream); its address is looked up on the first call for that device.
 * Problems with ssd_workspace_bytes() > SSD_SCRATCH_BYTES return SSD_ERR_SCRATCH before
 * any launch (128 MiB covers, e.g., b1 L16384 H32 P64 N256 Q256, which needs about
 * 99 MB).  Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs clearing: the forward writes every intermediate before
 * reading it): calls that overlap on one GPU -- on two streams, or from two threads
 * without ordering -- race and must not be issued.  Other arguments and errors as for
 * ssd_forward. */
#define SSD_SCRATCH_BYTES (128u << 20)
ssd_status ssd_forward_noalloc(const ssd_problem *problem, const void *x, const void *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               const float *h0, void *y, float *hT, void *stream);

/* One decode step (the recurrence of section "Mamba-2 架构" applied to a single token
 * per sequence; section "Kernel 2: fwd_pass_state" notes that at inference the final
 * state is handed to the next call as its initial state).  For every (b, h), with
 * g = h / (H / G):
 *     h[b,h,p,n] <- exp(A[h] dt[b,h]) h[b,h,p,n] + dt[b,h] x[b,h,p] B[b,g,n]
 *     y[b,h,p]    = sum_n h[b,h,p,n] C[b,g,n] + D[h] x[b,h,p]      (the updated h)
 * Shapes: x, y [b, H, P] and dt [b, H] and B, C [b, G, N] in element type `dtype`;
 * A, D [H] float32; h [b, H, P, N] float32, read and overwritten in place (the hT
 * layout of ssd_forward, so a forward's final state continues directly).
 * problem->seqlen must be 1 and problem->chunk is ignored; any headdim >= 1 and
 * dstate a multiple of 64 up to 512, with batch * nheads * ceil(headdim / 4) at most
 * 2^26 - 4 (one 64-lane wave per 4 state rows; the dispatch grid counts work-items in
 * 32 bits), else SSD_ERR_UNSUPPORTED before any launch.  The exponential is exp2 of A dt log2(e) in
 * fp32, the update and the dot product are fp32, y is rounded to `dtype`.  All
 * pointers are required. */
ssd_status ssd_step(const ssd_problem *problem, const void *x, const void *dt, const float *A,
                    const void *B, const void *C, const float *D, float *h, void *y,
                    void *stream);

/* How ssd_forward launches `problem` on this GPU: the per-shape choices of the state pass
 * (kernel, chunks per group, groups, state columns per workgroup) and of the chunk output (the
 * head-blocked kernel or the one-head kernel, heads per workgroup, column halves split over
 * wave pairs), with the workgroup counts.  Host-only; for reports and tuning. */
typedef struct {
    int32_t sp_group_chunks;    /* chunks per state-pass group (K) */
    int32_t sp_groups;          /* state-pass groups per (batch, head) chain (ng) */
    int32_t sp_columns;         /* state columns per state-pass workgroup */
    int32_t sp_workgroups;      /* state-pass workgroups */
    int32_t scan;               /* 1 when the group scan runs (sp_groups > 1) */
    int32_t co_head_blocked;    /* 1: full chunks on the head-blocked kernel */
    int32_t co_heads_per_block; /* heads per chunk-output workgroup (1: one-head kernel) */
    int32_t co_column_split;    /* 2: state columns split over wave pairs (N = 512) */
    int32_t co_workgroups;      /* chunk-output workgroups (ragged last chunk included) */
    int32_t co_threads;         /* threads per head-blocked (else one-head) workgroup */
    int32_t sp_register_transposed; /* 1: the state pass transposes B in registers (256
                                       columns per workgroup), 0: through LDS */
    int32_t sp_threads;         /* threads per state-pass workgroup */
    int32_t fused;              /* 1: the whole forward as one launch (fp32, chunk 64, headdim
                                   64, dstate 64, at most 8 chunks per sequence): per (batch,
                                   head) and half of the headdim rows, one workgroup of 256
                                   threads per chunk walks the jump over the earlier chunks
                                   and computes its chunk's output, one more the final state
                                   (co_workgroups = 2 batch nheads (nchunks + 1)); the
                                   state-pass and scan fields then describe no launch.
                                   A call with h0 and hT the same buffer runs the
                                   four-launch plan of one serial chain instead (its final
                                   state would overwrite h0 while other workgroups read
                                   it) */
} ssd_launch_plan;

ssd_status ssd_plan(const ssd_problem *problem, ssd_launch_plan *plan);

/* The search space of the forward's launch configuration for `problem` (the optimisations
 * are chosen per shape together with block size and occupancy, by measuring every
 * candidate: dbyun.net, section "Mamba-2 性能优化"; thetimeai.ru, section "Почему раскладка
 * памяти важна не меньше формул").  A candidate combines
 *   - a state-pass kernel: 256, 128 or 64 state columns per workgroup (those dividing
 *     dstate; bf16 only, fp32 always 64), for 256 columns B transposed through LDS or in
 *     registers (sp_register_transposed);
 *   - a split of every chain of chunks into groups: the cost model's count for that
 *     kernel, then 1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96 and 128 groups as far as the
 *     chain has chunks (sp_group_chunks = ceil(nc / groups), sp_groups = ceil(nc /
 *     sp_group_chunks));
 *   - a chunk-output kernel: head-blocked with each divisor of nheads / ngroups up to 64
 *     as heads per workgroup (bf16, chunk 128 or 256 with dstate 64, 128 or 256, and chunk
 *     128 with dstate 512), or one head per workgroup;
 * with the derived fields filled in, duplicates and configurations whose grids do not fit
 * 32-bit work-item counts left out.  plans[0] is ssd_plan's choice.  Writes the first
 * min(capacity, count) candidates to `plans` (NULL allowed when capacity is 0) and their
 * number to *count.  Host-only; SSD_ERR_NULL_ARG for a NULL count, a negative capacity or
 * NULL plans with capacity > 0. */
ssd_status ssd_plan_candidates(const ssd_problem *problem, ssd_launch_plan *plans,
                               int32_t capacity, int32_t *count);

/* Workspace bytes of the forward under `plan` (NULL: ssd_plan's choice, the same as
 * ssd_workspace_bytes); 0 if `problem` or `plan` is not valid.  Host-only. */
size_t ssd_workspace_bytes_planned(const ssd_problem *problem, const ssd_launch_plan *plan);

/* Launches first_stage .. last_stage (0 chunk cumsum, 1 state pass, 2 group scan, 3 chunk
 * output; 0 .. 3 is the whole forward pass) under launch plan `plan` (NULL: ssd_plan's
 * choice; ssd_forward, ssd_forward_timed and ssd_forward_stage are this call with a NULL
 * plan), the results of any valid plan being the method's, with the rounding of its own
 * grouping.  A plan is valid when its choices are among those ssd_plan_candidates
 * describes, with any chunks per group from 1 to nc, and each derived field matches what
 * these choices give (ssd_plan_candidates' output always is); else SSD_ERR_PLAN before any
 * launch.  `workspace` must hold ssd_workspace_bytes_planned(problem, plan) bytes and is
 * laid out per plan: stages of one forward run with the same plan.  `events` (NULL: no
 * marks) has SSD_FORWARD_EVENTS entries indexed by stage: events[i] is recorded right
 * before stage i and events[last_stage + 1] after the last, for first_stage <= i <=
 * last_stage.  Stages outside 0 .. 3 or first_stage > last_stage: SSD_ERR_UNSUPPORTED.
 * Stage repetition rules, other arguments and errors as for ssd_forward_stage. */
ssd_status ssd_forward_planned(const ssd_problem *problem, const ssd_launch_plan *plan,
                               const void *x, const void *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *h0, void *y, float *hT,
                               void *workspace, size_t workspace_bytes, int32_t first_stage,
                               int32_t last_stage, void *const *events, void *stream);

/* Offsets (bytes) of G2, dtT and S inside an ssd_forward workspace.  Host-only. */
ssd_status ssd_workspace_layout(const ssd_problem *problem, size_t *off_G2, size_t *off_dtT,
                                size_t *off_S);

/* Static text for a status code. */
const char *ssd_status_string(ssd_status status);

/* hipError_t of the last SSD_ERR_HIP returned on this thread (0 if none). */
int ssd_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
