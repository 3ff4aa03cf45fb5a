// ssd_api.cpp -- the C ABI declared in include/ssd.h: host-side validation,
// workspace layout and the three-stage forward on one stream.
#include "../../include/ssd.h"

#include <hip/hip_runtime.h>

#include <initializer_list>
#include <vector>

#include "ssd_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Arrays the kernels touch with 8- and 16-byte vector accesses must start on 16
// bytes; NULL (an absent optional array) passes.
bool aligned16(std::initializer_list<const void *> ptrs)
{
    for (const void *p : ptrs)
        if ((reinterpret_cast<uintptr_t>(p) & 15) != 0) return false;
    return true;
}

ssd_status check_shape(const ssd_problem *p)
{
    if (p == nullptr) return SSD_ERR_NULL_ARG;
    if (p->batch <= 0 || p->seqlen <= 0 || p->nheads <= 0 || p->ngroups <= 0 || p->headdim <= 0 ||
        p->dstate <= 0 || p->chunk <= 0)
        return SSD_ERR_BAD_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (p->dtype != SSD_F32 && p->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (p->headdim != 64) return SSD_ERR_UNSUPPORTED;
    if (p->dstate % 64 != 0 || p->dstate > 512) return SSD_ERR_UNSUPPORTED;
    if (p->chunk != 64 && p->chunk != 128 && p->chunk != 256) return SSD_ERR_UNSUPPORTED;
    // 32-bit grid and index limits of the kernels (each factor bounded before a product)
    if (p->batch > 65535 || p->nheads > 65535) return SSD_ERR_UNSUPPORTED;
    if (p->batch * p->nheads > 65535) return SSD_ERR_UNSUPPORTED;
    if (p->seqlen > (int64_t(1) << 30)) return SSD_ERR_UNSUPPORTED;
    // one-head chunk output: one workgroup of 2 * chunk threads per (chunk, batch, head) in
    // a 1-D grid, whose work-item count the dispatch packet holds in 32 bits
    if ((p->seqlen + p->chunk - 1) / p->chunk * p->batch * p->nheads >= (int64_t(1) << 31) / p->chunk)
        return SSD_ERR_UNSUPPORTED;
    // in-chunk element offsets are 32-bit, and so are byte offsets within one batch
    // of x and of B / C
    if (p->chunk * p->nheads * p->headdim >= (int64_t(1) << 31)) return SSD_ERR_UNSUPPORTED;
    if (p->chunk * p->ngroups * p->dstate >= (int64_t(1) << 31)) return SSD_ERR_UNSUPPORTED;
    if (p->seqlen * p->nheads * p->headdim >= (int64_t(1) << 30)) return SSD_ERR_UNSUPPORTED;
    if (p->seqlen * p->ngroups * p->dstate >= (int64_t(1) << 30)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// The decode step's own set: one token per sequence, no chunking.
ssd_status check_step_shape(const ssd_problem *p)
{
    if (p == nullptr) return SSD_ERR_NULL_ARG;
    if (p->batch <= 0 || p->seqlen <= 0 || p->nheads <= 0 || p->ngroups <= 0 || p->headdim <= 0 ||
        p->dstate <= 0)
        return SSD_ERR_BAD_SHAPE;
    if (p->seqlen != 1 || p->nheads % p->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (p->dtype != SSD_F32 && p->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (p->dstate % 64 != 0 || p->dstate > 512) return SSD_ERR_UNSUPPORTED;
    // 32-bit head and row indices
    if (p->batch > (int64_t(1) << 31) || p->nheads > (int64_t(1) << 30) ||
        p->headdim > (int64_t(1) << 30))
        return SSD_ERR_UNSUPPORTED;
    if (p->batch * p->nheads > (int64_t(1) << 31) / p->headdim) return SSD_ERR_UNSUPPORTED;
    // the dispatch grid counts work-items in 32 bits: one wave of 64 per ceil(P/4) rows of
    // each (batch, head), in workgroups of 4 waves, so at most 2^24 - 1 workgroups
    const int64_t waves = p->batch * p->nheads * ((p->headdim + 3) / 4);
    if ((waves + 3) / 4 > (int64_t(1) << 24) - 1) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd::Shape make_shape(const ssd_problem *p)
{
    ssd::Shape s;
    s.b = p->batch; s.L = p->seqlen; s.H = p->nheads; s.G = p->ngroups;
    s.P = p->headdim; s.N = p->dstate; s.Q = p->chunk;
    s.nc = (s.L + s.Q - 1) / s.Q;
    s.Lp = s.nc * s.Q;
    s.bf16 = p->dtype == SSD_BF16;
    return s;
}

struct Layout {
    size_t g2, dtt, wt, S, ug, gam, beta, hb, total;
};

// Workspace of the forward pass under launch plan lp: the stage-1 outputs, the
// chunk-start states and, when the state pass is split into groups, the group states,
// group decays and per-chunk decays since the group start.
Layout layout_of(const ssd::Shape &s, const ssd::LaunchPlan &lp)
{
    const size_t bh = size_t(s.b) * s.H;
    const size_t cum = bh * s.Lp * sizeof(float);
    const size_t snap = bh * s.nc * s.P * s.N * (s.bf16 ? 2 : 4);
    const size_t ng = size_t(lp.sp_groups);
    const bool grouped = ng > 1;
    Layout l;
    l.g2 = 0;
    l.dtt = align_up(cum);
    l.wt = l.dtt + align_up(cum);
    l.S = l.wt + align_up(cum);
    l.ug = l.S + align_up(snap);
    l.gam = l.ug + (grouped ? align_up(bh * ng * s.P * s.N * sizeof(float)) : 0);
    l.beta = l.gam + (grouped ? align_up(bh * ng * sizeof(float)) : 0);
    l.hb = l.beta + (grouped ? align_up(bh * s.nc * sizeof(float)) : 0);
    l.total = l.hb + ((grouped && s.bf16) ? align_up(bh * ng * s.P * s.N * 2) : 0);
    return l;
}

ssd::LaunchPlan to_internal(const ssd_launch_plan &p)
{
    ssd::LaunchPlan lp;
    lp.sp_group_chunks = p.sp_group_chunks;
    lp.sp_groups = p.sp_groups;
    lp.sp_columns = p.sp_columns;
    lp.sp_workgroups = p.sp_workgroups;
    lp.scan = p.scan;
    lp.co_head_blocked = p.co_head_blocked;
    lp.co_heads_per_block = p.co_heads_per_block;
    lp.co_column_split = p.co_column_split;
    lp.co_workgroups = p.co_workgroups;
    lp.co_threads = p.co_threads;
    lp.sp_register_transposed = p.sp_register_transposed;
    lp.sp_threads = p.sp_threads;
    lp.fused = p.fused;
    return lp;
}

ssd_launch_plan to_public(const ssd::LaunchPlan &lp)
{
    ssd_launch_plan p;
    p.sp_group_chunks = lp.sp_group_chunks;
    p.sp_groups = lp.sp_groups;
    p.sp_columns = lp.sp_columns;
    p.sp_workgroups = lp.sp_workgroups;
    p.scan = lp.scan;
    p.co_head_blocked = lp.co_head_blocked;
    p.co_heads_per_block = lp.co_heads_per_block;
    p.co_column_split = lp.co_column_split;
    p.co_workgroups = lp.co_workgroups;
    p.co_threads = lp.co_threads;
    p.sp_register_transposed = lp.sp_register_transposed;
    p.sp_threads = lp.sp_threads;
    p.fused = lp.fused;
    return p;
}

// The plan a forward call runs: the cost model's when `plan` is NULL, else the caller's
// after checking that the kernels can run it.
ssd_status resolve_plan(const ssd::Shape &s, const ssd_launch_plan *plan, ssd::LaunchPlan &lp)
{
    if (plan == nullptr) {
        lp = ssd::plan_of(s);
        return SSD_OK;
    }
    lp = to_internal(*plan);
    return ssd::plan_valid(s, lp) ? SSD_OK : SSD_ERR_PLAN;
}

ssd_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return SSD_OK;
    g_last_hip_error = int(e);
    return SSD_ERR_HIP;
}

}  // namespace

int ssd::hip_status(hipError_t e) { return ::hip_status(e); }

extern "C" {

ssd_status ssd_validate(const ssd_problem *problem) { return check_shape(problem); }

size_t ssd_workspace_bytes(const ssd_problem *problem)
{
    if (check_shape(problem) != SSD_OK) return 0;
    const ssd::Shape s = make_shape(problem);
    return layout_of(s, ssd::plan_of(s)).total;
}

size_t ssd_workspace_bytes_planned(const ssd_problem *problem, const ssd_launch_plan *plan)
{
    if (check_shape(problem) != SSD_OK) return 0;
    const ssd::Shape s = make_shape(problem);
    ssd::LaunchPlan lp;
    if (resolve_plan(s, plan, lp) != SSD_OK) return 0;
    return layout_of(s, lp).total;
}

ssd_status ssd_workspace_layout(const ssd_problem *problem, size_t *off_G2, size_t *off_dtT,
                                size_t *off_S)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (!off_G2 || !off_dtT || !off_S) return SSD_ERR_NULL_ARG;
    const ssd::Shape s = make_shape(problem);
    const Layout l = layout_of(s, ssd::plan_of(s));
    *off_G2 = l.g2;
    *off_dtT = l.dtt;
    *off_S = l.S;
    return SSD_OK;
}

ssd_status ssd_plan(const ssd_problem *problem, ssd_launch_plan *plan)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (plan == nullptr) return SSD_ERR_NULL_ARG;
    *plan = to_public(ssd::plan_of(make_shape(problem)));
    return SSD_OK;
}

ssd_status ssd_plan_candidates(const ssd_problem *problem, ssd_launch_plan *plans,
                               int32_t capacity, int32_t *count)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (count == nullptr || capacity < 0 || (capacity > 0 && plans == nullptr))
        return SSD_ERR_NULL_ARG;
    const ssd::Shape s = make_shape(problem);
    const int n = ssd::plan_candidates(s, nullptr, 0);
    std::vector<ssd::LaunchPlan> all((size_t)n);
    ssd::plan_candidates(s, all.data(), n);
    for (int i = 0; i < n && i < capacity; ++i) plans[i] = to_public(all[(size_t)i]);
    *count = n;
    return SSD_OK;
}

ssd_status ssd_chunk_cumsum(const ssd_problem *problem, const void *dt, const float *A, float *G2,
                            float *dtT, void *stream)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (!dt || !A || !G2 || !dtT) return SSD_ERR_NULL_ARG;
    if (!aligned16({G2, dtT})) return SSD_ERR_MISALIGNED;
    return hip_status(ssd::launch_chunk_cumsum(make_shape(problem), dt, A, G2, dtT, nullptr,
                                               (hipStream_t)stream));
}

ssd_status ssd_state_pass(const ssd_problem *problem, const void *x, const void *B,
                          const float *G2, const float *dtT, const float *h0, void *S, float *hT,
                          void *stream)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (!x || !B || !G2 || !dtT || !S) return SSD_ERR_NULL_ARG;
    if (!aligned16({x, B, G2, dtT, h0, S, hT})) return SSD_ERR_MISALIGNED;
    return hip_status(ssd::launch_state_pass(make_shape(problem), x, B, G2, dtT, h0, S, hT,
                                             (hipStream_t)stream));
}

ssd_status ssd_chunk_out(const ssd_problem *problem, const void *x, const void *B, const void *C,
                         const float *G2, const float *dtT, const void *S, const float *D, void *y,
                         void *stream)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (!x || !B || !C || !G2 || !dtT || !S || !D || !y) return SSD_ERR_NULL_ARG;
    if (!aligned16({x, B, C, G2, dtT, S, y})) return SSD_ERR_MISALIGNED;
    return hip_status(ssd::launch_chunk_out(make_shape(problem), x, B, C, G2, dtT, S, D, y,
                                            (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Launches first..last (0 chunk cumsum, 1 state pass, 2 group scan, 3 chunk output) of
// the forward under `plan` (NULL: the cost model's) on `stream`, with events[i] recorded
// right before launch i and events[last + 1] after the last (events NULL: no marks).
ssd_status forward_launches(const ssd_problem *problem, const ssd_launch_plan *plan,
                            const void *x, const void *dt, const float *A, const void *B,
                            const void *C, const float *D, const float *h0, void *y, float *hT,
                            void *workspace, size_t workspace_bytes, void *stream,
                            void *const *events, int first, int last)
{
    const ssd_status st = check_shape(problem);
    if (st != SSD_OK) return st;
    if (first < 0 || last > SSD_FORWARD_EVENTS - 2 || first > last) return SSD_ERR_UNSUPPORTED;
    if (!x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_NULL_ARG;
    if (events != nullptr)
        for (int i = first; i <= last + 1; ++i)
            if (!events[i]) return SSD_ERR_NULL_ARG;
    const ssd::Shape s = make_shape(problem);
    ssd::LaunchPlan lp;
    const ssd_status pst = resolve_plan(s, plan, lp);
    if (pst != SSD_OK) return pst;
    // The one-launch kernel's final-state workgroups write hT while other workgroups of the
    // same (batch, head) may still be reading h0: with h0 and hT the same buffer the call
    // runs the four-launch plan of one serial chain instead, on the same workspace layout.
    if (lp.fused && h0 != nullptr && static_cast<const void *>(h0) == static_cast<const void *>(hT))
        lp = ssd::plan_one_chain(s);
    const Layout l = layout_of(s, lp);
    if (workspace == nullptr || workspace_bytes < l.total) return SSD_ERR_WORKSPACE;
    if (!aligned16({x, B, C, h0, y, hT, workspace})) return SSD_ERR_MISALIGNED;
    char *ws = static_cast<char *>(workspace);
    float *G2 = reinterpret_cast<float *>(ws + l.g2);
    float *dtT = reinterpret_cast<float *>(ws + l.dtt);
    float *wT = reinterpret_cast<float *>(ws + l.wt);
    void *S = ws + l.S;
    float *Ug = reinterpret_cast<float *>(ws + l.ug);
    float *gam = reinterpret_cast<float *>(ws + l.gam);
    float *beta = reinterpret_cast<float *>(ws + l.beta);
    void *Hb = ws + l.hb;
    hipStream_t hs = (hipStream_t)stream;
    auto mark = [&](int i) -> ssd_status {
        return events ? hip_status(hipEventRecord((hipEvent_t)events[i], hs)) : SSD_OK;
    };
    auto launch = [&](int i) -> hipError_t {
        if (lp.fused)   // the whole forward is the last stage's one launch
            return i == 3 ? ssd::launch_forward_small(s, x, dt, A, B, C, D, h0, y, hT, G2, dtT, hs)
                          : hipSuccess;
        switch (i) {
        case 0: return ssd::launch_chunk_cumsum(s, dt, A, G2, dtT, wT, hs);
        case 1:
            return ssd::launch_state_pass_grouped(s, lp, x, B, G2, wT, h0, S, hT, Ug, gam, beta,
                                                  hs);
        case 2: return ssd::launch_group_scan(s, lp, hT, Ug, Hb, gam, hs);
        default:
            return ssd::launch_chunk_out_corrected(s, lp, x, B, C, G2, dtT, S, D, y, Ug, Hb,
                                                   beta, hs);
        }
    };
    ssd_status r = SSD_OK;
    for (int i = first; i <= last && r == SSD_OK; ++i) {
        r = mark(i);
        if (r == SSD_OK) r = hip_status(launch(i));
    }
    if (r == SSD_OK) r = mark(last + 1);
    return r;
}

}  // namespace

extern "C" {

ssd_status ssd_forward_timed(const ssd_problem *problem, const void *x, const void *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const float *h0, void *y, float *hT, void *workspace,
                             size_t workspace_bytes, void *stream, void *const *events)
{
    return forward_launches(problem, nullptr, x, dt, A, B, C, D, h0, y, hT, workspace,
                            workspace_bytes, stream, events, 0, SSD_FORWARD_EVENTS - 2);
}

ssd_status ssd_forward(const ssd_problem *problem, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const float *h0, void *y,
                       float *hT, void *workspace, size_t workspace_bytes, void *stream)
{
    return forward_launches(problem, nullptr, x, dt, A, B, C, D, h0, y, hT, workspace,
                            workspace_bytes, stream, nullptr, 0, SSD_FORWARD_EVENTS - 2);
}

ssd_status ssd_forward_stage(const ssd_problem *problem, const void *x, const void *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const float *h0, void *y, float *hT, void *workspace,
                             size_t workspace_bytes, int stage, void *stream)
{
    return forward_launches(problem, nullptr, x, dt, A, B, C, D, h0, y, hT, workspace,
                            workspace_bytes, stream, nullptr, stage, stage);
}

ssd_status ssd_forward_planned(const ssd_problem *problem, const ssd_launch_plan *plan,
                               const void *x, const void *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *h0, void *y, float *hT,
                               void *workspace, size_t workspace_bytes, int32_t first_stage,
                               int32_t last_stage, void *const *events, void *stream)
{
    return forward_launches(problem, plan, x, dt, A, B, C, D, h0, y, hT, workspace,
                            workspace_bytes, stream, events, first_stage, last_stage);
}

ssd_status ssd_step(const ssd_problem *problem, const void *x, const void *dt, const float *A,
                    const void *B, const void *C, const float *D, float *h, void *y, void *stream)
{
    const ssd_status st = check_step_shape(problem);
    if (st != SSD_OK) return st;
    if (!x || !dt || !A || !B || !C || !D || !h || !y) return SSD_ERR_NULL_ARG;
    if (!aligned16({x, B, C, h, y})) return SSD_ERR_MISALIGNED;
    ssd::Shape s;
    s.b = problem->batch; s.L = 1; s.H = problem->nheads; s.G = problem->ngroups;
    s.P = problem->headdim; s.N = problem->dstate; s.Q = 1; s.nc = 1; s.Lp = 1;
    s.bf16 = problem->dtype == SSD_BF16;
    return hip_status(ssd::launch_decode_step(s, x, dt, A, B, C, D, h, y, (hipStream_t)stream));
}

const char *ssd_status_string(ssd_status status)
{
    switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL_ARG: return "a required pointer is NULL";
    case SSD_ERR_BAD_SHAPE: return "bad shape (dimension <= 0 or nheads not divisible by ngroups)";
    case SSD_ERR_UNSUPPORTED: return "unsupported dtype/headdim/dstate/chunk";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP launch failed";
    case SSD_ERR_MISALIGNED: return "a vector-accessed array does not start on a 16-byte boundary";
    case SSD_ERR_SCRATCH:
        return "the problem needs more workspace than the static scratch of ssd_forward_noalloc "
               "holds (SSD_SCRATCH_BYTES); use ssd_forward with a workspace";
    case SSD_ERR_PLAN: return "the launch plan is not one the kernels can run for this problem";
    }
    return "unknown status";
}

int ssd_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
