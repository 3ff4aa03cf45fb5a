// ssd_launch.h -- internal interface between the C ABI (ssd_api.cpp) and the
// kernel launchers (ssd_kernels.hip).  Shapes are already validated here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// SSD_OK for hipSuccess; otherwise SSD_ERR_HIP, with the code kept for
// ssd_last_hip_error() on this thread (ssd_api.cpp).
int hip_status(hipError_t e);

struct Shape {
    int64_t b, L, H, G, P, N, Q, nc, Lp;
    bool bf16;
};

// wT may be NULL (not written): the forward's state-pass weights, see below
hipError_t launch_chunk_cumsum(const Shape &s, const void *dt, const float *A, float *G2,
                               float *dtT, float *wT, hipStream_t st);

hipError_t launch_state_pass(const Shape &s, const void *x, const void *B, const float *G2,
                             const float *dtT, const float *h0, void *S, float *hT,
                             hipStream_t st);

hipError_t launch_chunk_out(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, hipStream_t st);

// The launch configuration of the forward pass (host only): the state pass's kernel
// (state columns per workgroup, B transposed in registers or through LDS), the split of
// each serial chain of chunks into sp_groups groups of sp_group_chunks chunks (1 group:
// one chain), and the chunk output's kernel (head-blocked with co_heads_per_block heads
// per workgroup, or one head per workgroup); the other fields follow from these.
// fused = 1: the whole forward as one launch (forward_small below); the state-pass and
// group-scan fields then describe no launch.
struct LaunchPlan {
    int sp_group_chunks, sp_groups, sp_columns, sp_workgroups, scan;
    int co_head_blocked, co_heads_per_block, co_column_split, co_workgroups, co_threads;
    int sp_register_transposed, sp_threads, fused;
};
// The cost model's choice for shape s.
LaunchPlan plan_of(const Shape &s);
// The four-launch plan with one serial state-pass chain per (batch, head) and column block
// (no groups, no scan): the same workspace layout as the one-launch plan.
LaunchPlan plan_one_chain(const Shape &s);
// Every configuration of the search space for shape s, plan_of(s) first; writes at most
// cap of them and returns how many there are.
int plan_candidates(const Shape &s, LaunchPlan *out, int cap);
// True when lp is a configuration the kernels can run for s: its choices are among the
// kernels' supported ones (any chunks per group from 1 to nc) and its derived fields are
// the ones these choices give.
bool plan_valid(const Shape &s, const LaunchPlan &lp);

// Grouped state pass as used by the forward pass: with lp.sp_groups > 1, S receives
// chunk-start states relative to their group, Ug the final local state of each
// group, gam each group's decay and beta the per-chunk decay since the group
// start; with one group it is the plain state pass (true states, hT written).
// launch_group_scan then (more than one group only) turns Ug into the true group-start
// states H_g and writes hT.  Scratch: Ug [b*H, ng, P, N], gam [b*H, ng], beta [b*H, nc],
// all fp32, and for bf16 problems Hb [b*H, ng, P, N] bf16 (H_g rounded, zeros for
// group 0).
// The forward's state passes read the weights w_t = dtT_t exp2(G2_last - G2_t) that its
// stage 1 wrote to the workspace (wT [b, H, Lp]); the public stage-2 entry point
// (launch_state_pass) forms them from dtT and G2 instead.
// fp32 state pass over ng groups of K chunks (ssd_kernels.hip): local chunk-start
// states into S, final local states into Ug, decays into gam and beta; with one group
// (Ug NULL) true states and hT.
hipError_t launch_state_pass_f32_grouped(const Shape &s, const void *x, const void *B,
                                         const float *G2, const float *wT, const float *h0,
                                         void *S, float *hT, float *Ug, float *gam, float *beta,
                                         int K, int ng, hipStream_t st);
hipError_t launch_state_pass_grouped(const Shape &s, const LaunchPlan &lp, const void *x,
                                     const void *B, const float *G2, const float *wT,
                                     const float *h0, void *S, float *hT, float *Ug, float *gam,
                                     float *beta, hipStream_t st);
hipError_t launch_group_scan(const Shape &s, const LaunchPlan &lp, float *hT, float *Ug, void *Hb,
                             const float *gam, hipStream_t st);

// Chunk output that adds beta_c H_g to the handed-over chunk-start states
// (one group: S already holds true states).  Hg is fp32, Hb its bf16 copy.
hipError_t launch_chunk_out_corrected(const Shape &s, const LaunchPlan &lp, const void *x,
                                      const void *B, const void *C, const float *G2,
                                      const float *dtT, const void *S, const float *D, void *y,
                                      const float *Hg, const void *Hb, const float *beta,
                                      hipStream_t st);

// Threads per fp32 chunk-output workgroup: two waves with one 32-token row tile each for
// 64-token chunks when the grid has fewer than 1024 workgroups (the chunk's tiles side by
// side), else Q (Q/64 waves with two row tiles each).
int chunk_out_f32_threads(const Shape &s);

// The whole forward in one launch for fp32 problems of at most kSmallMaxChunks chunks of 64
// tokens, headdim 64, dstate 64 (ssd_small.hip): one workgroup per (batch, head, chunk,
// half of the headdim rows) walks the jump over the earlier chunks and computes its
// chunk's output, one more per (batch, head, half) the final state; writes y, hT (may be
// NULL) and the chunk cumsum and dt into G2 and dtT.
constexpr int kSmallMaxChunks = 8;
bool forward_small_eligible(const Shape &s);
int64_t forward_small_workgroups(const Shape &s);
hipError_t launch_forward_small(const Shape &s, const void *x, const void *dt, const float *A,
                                const void *B, const void *C, const float *D, const float *h0,
                                void *y, float *hT, float *G2, float *dtT, hipStream_t st);

// One decode step per (batch, head), h updated in place (ssd_step.hip).
hipError_t launch_decode_step(const Shape &s, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D, float *h, void *y,
                              hipStream_t st);

// bf16 kernels (ssd_bf16.hip)
hipError_t launch_state_pass_bf16(const Shape &s, const void *x, const void *B, const float *G2,
                                  const float *dtT, const float *h0, void *S, float *hT,
                                  hipStream_t st);
// hb: heads per head-blocked workgroup for the full chunks (0: every chunk on the
// one-head kernel)
hipError_t launch_chunk_out_bf16(const Shape &s, const void *x, const void *B, const void *C,
                                 const float *G2, const float *dtT, const void *S, const float *D,
                                 void *y, const float *Hg, const void *Hb, const float *beta, int K,
                                 int ng, int hb, hipStream_t st);

}  // namespace ssd
