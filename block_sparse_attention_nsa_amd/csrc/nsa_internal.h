// nsa_internal.h -- host-side glue between the C ABI (nsa_api.hip) and the
// kernel files: the backward workspace layout and the kernel launchers.
#pragma once

#include <algorithm>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nsa_device.h"

namespace nsa {

// Host description of a validated problem (plus the device Problem).
struct HostProblem {
    Problem dev;
    int dtype;      // 0 f32, 1 bf16
    int ZH;         // Z * Hkv
    int CT;         // tokens per inversion chunk
    int C;          // inversion chunks per (z, hkv): ceil(Tmax / CT)
    int CR;         // query rows per dK/dV work item
    int64_t rows;   // query rows in lse/delta: B*Hq*T (dense) or Hq*T (packed)
    int64_t cap;    // token-list capacity: Smin * rows of block_idx
    int64_t items_ub;  // upper bound on dK/dV work items
    int64_t pslots;    // fp32 partial slots reserved for split lists
    // dK/dV may run on pairs of blocks (2 block_size keys per workgroup, one
    // row list) when every row selects its whole causal prefix; decided on
    // the device, possible only without partial slots, for block_size <= 64,
    // bf16, and S * block_size >= the longest sequence.
    bool pair_possible;
    // dS hand-off: the dK/dV kernel stores dS and the dQ kernel forms dq =
    // scale dS K from it (bf16, G a multiple of 16, no window, selections
    // that cannot cover whole causal prefixes: S * block_size < longest
    // sequence).  The backward then runs dK/dV before dQ.
    bool ds_handoff;
    // Scheduling policy of the hand-off dQ (nsa_sel_problem.sched_policy):
    // 0 one workgroup per item in a static longest-first order, 1 a
    // persistent grid taking the same order from a device counter.
    int sched;
    // The caller's strides of q, k, v, o, dO, dq, dk, dv when the problem is
    // strided (the device copies hold 32-bit head / token strides).
    int64_t given[8][3];
};

// Backward workspace carve (all offsets 256-byte aligned).
struct BwdWorkspace {
    float* delta;        // [rows]
    int* chunk_pos;      // [ZH][C][NBmax]: per-chunk counts, then list cursors
    int* offsets;        // [ZH][NBmax + 1]: CSR offsets inside each region
    int* tokens;         // [cap]: inverted lists
    int* item_pre;       // [ZH][NBmax + 1]: exclusive prefix of work items per list
    int* pslot_pre;      // [ZH][NBmax + 1]: exclusive prefix of partial slots per list
    int* zh_base;        // [2][ZH + 1]: global prefixes of items and partial slots,
                         // then [2][ZH]: per-(z, hkv) totals of both, [ZH]: per-(z,
                         // hkv) whole-prefix flags, [1]: all of them set
    int* ticket;         // [3]: scan workgroups done (the last one plans), then the
                         // persistent hand-off dQ's item counter and leaver count
                         // (all three zeroed by the inversion's count kernel)
    int* iota;           // [Tmax] (pair_possible): iota[t] = t, the lists of a
                         // whole-prefix selection
    float* partials;     // [pslots][bs][D][2]
    int* posmap;         // (ds_handoff) [block_idx rows][S]: list position of each slot, or -1
    uint16_t* ds;        // (ds_handoff) [cap][bs][G] bf16: dS of every listed (token, block)
    size_t bytes;
};

BwdWorkspace carve_bwd_workspace(const HostProblem& hp, void* base);

// ---- launchers (return the launch status) ---------------------------------
hipError_t launch_delta(const HostProblem& hp, const void* o, const void* dO, float* delta,
                        hipStream_t st);
hipError_t launch_invert(const HostProblem& hp, const int* block_idx, const BwdWorkspace& ws,
                         hipStream_t st);
// dsink[h] = -sum over head h's rows of exp(sink[h] - lse) * Delta (fixed
// order: one workgroup per head).
hipError_t launch_dsink(const HostProblem& hp, const float* lse, const float* delta,
                        const float* sink, float* dsink, hipStream_t st);
// Counts of padding / out-of-range / future / repeated block_idx entries
// (counts[4], zeroed first on the stream).
hipError_t launch_check_idx(const HostProblem& hp, const int* block_idx, unsigned long long* counts,
                            hipStream_t st);
// Delta, the inversion and the dK/dV work plan, as the backward's prepare
// stage runs them (for bf16 the Delta rows and the inversion counts share one
// launch; the last scan workgroup writes the plan).
hipError_t launch_prepare_lists(const HostProblem& hp, const int* block_idx, const BwdWorkspace& ws,
                                hipStream_t st);
hipError_t launch_prepare(const HostProblem& hp, const void* o, const void* dO, const int* block_idx,
                          const BwdWorkspace& ws, hipStream_t st);

hipError_t launch_fwd_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                           const int* block_idx, void* o, float* lse, hipStream_t st);
hipError_t launch_dq_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const float* delta,
                          const int* block_idx, void* dq, hipStream_t st);
// parts: kDkdvBlocks (the per-block kernel: whole lists straight to dk/dv,
// split lists as fp32 partials), kDkdvReduce (partials summed, unattended
// blocks zeroed), or both.
constexpr int kDkdvBlocks = 1, kDkdvReduce = 2, kDkdvAll = 3;
hipError_t launch_dkdv_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                            const void* dO, const float* lse, const float* delta,
                            const BwdWorkspace& ws, void* dk, void* dv, hipStream_t st,
                            int parts = kDkdvAll);

// dQ from the handed-off dS (ds_handoff); runs after the dK/dV block kernel.
size_t dq_ds_lds_bytes(const HostProblem& hp);
hipError_t launch_dq_handoff(const HostProblem& hp, const void* k, const int* block_idx,
                             const BwdWorkspace& ws, void* dq, hipStream_t st);

hipError_t launch_fwd_f32(const HostProblem& hp, const float* q, const float* k, const float* v,
                          const int* block_idx, float* o, float* lse, hipStream_t st);
hipError_t launch_dq_f32(const HostProblem& hp, const float* q, const float* k, const float* v,
                         const float* dO, const float* lse, const float* delta,
                         const int* block_idx, float* dq, hipStream_t st);
hipError_t launch_dkdv_f32(const HostProblem& hp, const float* q, const float* k, const float* v,
                           const float* dO, const float* lse, const float* delta,
                           const BwdWorkspace& ws, float* dk, float* dv, hipStream_t st);

// Give-ups of the bounded in-kernel waits of the query and dK/dV kernels on
// the current device (synchronous reads of each file's counter).
hipError_t read_wait_timeouts_query(unsigned* out);
hipError_t read_wait_timeouts_dkdv(unsigned* out);

// Dynamic LDS the bf16 forward / dQ kernels need (0 if unsupported).
size_t query_lds_bytes(const HostProblem& hp);
// LDS of the largest inversion kernel (block counts, chunk-table scan, fill).
size_t invert_lds_bytes(const HostProblem& hp);

}  // namespace nsa
