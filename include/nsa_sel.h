/*
 * nsa_sel.h -- C ABI of the MI355X (gfx950) NSA selection-attention library
 * (libnsa_sel.so).
 *
 * What it computes.  Page 1 of the reference text, "test_kernel_backward.py
 * -- GRADCHECK GATE for the NSA selection BACKWARD kernel" (docstring and
 * run_one), defines the call: q, k, v and a per-token list of selected key
 * blocks (block_idx, block_size) give o; o.backward(dO) gives dQ, dK, dV; G =
 * Hq/Hkv query heads share one KV head and its block list.  Page 3, the
 * cudnn-frontend SM80 backward pull request (walkthrough and review of
 * sdpa_bwd_wrapper_sm80), shows the backward consuming o, dO and the forward's
 * lse, and packed (THD) batches described by cumulative sequence lengths.
 *
 * For query row (z, h, t) -- z a batch entry or packed sequence, h a query
 * head, t a sequence-local token -- with hkv = h / G and NB = ceil(len/bs):
 *   Sel = { u : u listed in block_idx[z, hkv, t, :], 0 <= u < NB }   (a set)
 *   A   = { j : j / bs in Sel, j < len, j <= t }
 *   lse = log sum_{j in A} exp(scale <q, k_j>),  o = sum_{j in A} P_j v_j
 * (with a sliding window W = window > 0, A also keeps only j > t - W; the
 * page 3 backward lists sliding-window masks among its flavours)
 * and the backward is the exact gradient of o.  An empty A gives o = 0,
 * lse = -inf, dq = 0.  Negative or >= NB entries are padding.  Repeated
 * entries count once.  Keys listed by no row get dk = dv = 0.
 *
 * Layouts (row-major, last dimension D contiguous):
 *   dense  (layout NSA_DENSE, cu_seqlens == NULL): q, o, dO, dq [B][Hq][T][D];
 *          k, v, dk, dv [B][Hkv][T][D]; block_idx [B][Hkv][T][S] int32;
 *          lse, delta [B][Hq][T] float.
 *   packed (layout NSA_PACKED, cu_seqlens != NULL, B == 1, T = total tokens):
 *          q, o, dO, dq [T][Hq][D]; k, v, dk, dv [T][Hkv][D];
 *          block_idx [Hkv][T][S] with sequence-local block numbers;
 *          lse, delta [Hq][T]; cu_seqlens [n_seqs + 1] int32 on the device,
 *          cu_seqlens[0] = 0, non-decreasing, cu_seqlens[n_seqs] = T, and
 *          max_seqlen >= every sequence length (host value).
 *   q, k, v, o, dO, dq, dk and dv are contiguous in these layouts when the
 *   problem's `strided` is 0; with strided = 1 each of them has its own
 *   element strides for its (batch entry, head, token) dimensions (page 3's
 *   backward honours the output strides its caller declares), so e.g. a
 *   [B][T][H][D] buffer is passed as the dense layout with strides
 *   (T*H*D, D, H*D).  block_idx, lse, delta and cu_seqlens stay contiguous.
 * Element type: dtype NSA_F32 (float) or NSA_BF16 (bfloat16) for q, k, v, o,
 * dO, dq, dk, dv; lse/delta are float; block_idx/cu_seqlens are int32.
 *
 * Ownership and errors.  Every pointer is device memory owned by the caller;
 * the library allocates nothing.  Inputs are read-only; outputs are fully
 * overwritten and must not alias inputs.  All work is queued on `stream` only
 * and is asynchronous: device faults surface at the caller's next
 * synchronisation.  Each call checks its arguments on the host before any
 * HIP call and returns a non-zero nsa_status without touching any buffer when
 * a check fails; nsa_last_error() then names the failed check (thread-local
 * text).  There is no fallback path: an unsupported shape is an error.
 * The library keeps no state besides that text and is reentrant.
 *
 * Supported (else NSA_ERR_UNSUPPORTED): dtype f32 with D in {16, 32, 64,
 * 128} and any block_size >= 1 (vector-ALU kernels); dtype bf16 with D in
 * {32, 64, 128} and block_size in {16, 32, 64, 128} (matrix-core kernels),
 * and 12 * JK * D + 10 * NBmax + 32 <= 163840 bytes of forward/dQ LDS (JK =
 * 64 for block_size >= 64, else 32; NBmax = ceil(max length / block_size);
 * e.g. NBmax <= 6550 at D = 128, block_size 64).  For both: S <= 4096,
 * NBmax <= 8192, (B or n_seqs) * Hkv <= 8192, max length * G <= 2^30,
 * Hq * T * D < 2^31, max length * min(S, NBmax) < 2^31 (inverted-list
 * entries of one (batch entry, KV head)); for each of the eight q-like and
 * k-like tensors a token stride < 2^23 elements and, per batch entry,
 * (H - 1) * head stride + (T - 1) * token stride + D <= 2^31 - 128 elements.
 */
#ifndef NSA_SEL_H
#define NSA_SEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nsa_status {
    NSA_OK = 0,
    NSA_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, inconsistent sizes */
    NSA_ERR_UNSUPPORTED = 2,   /* valid but outside the supported set above */
    NSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    NSA_ERR_HIP = 4            /* a HIP runtime call failed (launch error) */
} nsa_status;

typedef enum nsa_dtype { NSA_F32 = 0, NSA_BF16 = 1 } nsa_dtype;

typedef enum nsa_layout {
    NSA_DENSE = 0,   /* [B][H][T][D], cu_seqlens must be NULL */
    NSA_PACKED = 1   /* [T][H][D] sequences back to back, cu_seqlens required */
} nsa_layout;

/* Problem description (host memory, read only during the call). */
typedef struct nsa_sel_problem {
    int32_t layout;      /* nsa_layout */
    int32_t B;           /* batch entries (dense); 1 for packed */
    int32_t T;           /* tokens per entry (dense) or total tokens (packed) */
    int32_t Hq;          /* query heads */
    int32_t Hkv;         /* key/value heads; G = Hq / Hkv */
    int32_t D;           /* head dimension */
    int32_t S;           /* slots per block_idx row */
    int32_t block_size;  /* keys per block */
    int32_t n_seqs;      /* packed: number of sequences; dense: ignored */
    int32_t max_seqlen;  /* packed: bound on every sequence length; dense: ignored */
    int32_t dtype;       /* nsa_dtype */
    float scale;         /* softmax scale applied to <q, k> (e.g. 1/sqrt(D)) */
    int32_t window;      /* sliding window: keys t - window < j <= t only; 0 = none */
    /* Memory layout of the eight q-like / k-like tensors.  strided = 0: the
     * contiguous layouts above (the arrays below are not read).  strided = 1:
     * stride_x = element strides of tensor x's batch-entry, head and token
     * dimensions (packed problems do not read stride_x[0]); the D elements of
     * a row are contiguous.  Only the strides of tensors a call takes are
     * read.  Each stride must be >= 0 (0 repeats an input along that
     * dimension), a multiple of 8 for bf16 (16-byte aligned rows), and the
     * rows of an output must not overlap one another (checked:
     * NSA_ERR_INVALID_ARG). */
    int32_t strided;
    int64_t stride_q[3], stride_k[3], stride_v[3], stride_o[3];
    int64_t stride_do[3], stride_dq[3], stride_dk[3], stride_dv[3];
    /* Dense only: keys per (batch entry, KV head), >= T; 0 means T.  With
     * Tk > T the T queries are the last T positions of the key range
     * (bottom-right causal alignment, a backward flavour page 3 of the
     * reference text lists): query t sees keys j <= t + Tk - T, block
     * numbers in block_idx count blocks of the Tk keys, and k, v, dk, dv are
     * [B, Hkv, Tk, D] (default strides from Tk).  Packed problems need 0 or
     * T (queries and keys share the cumulative lengths). */
    int32_t Tk;
    /* Work scheduling of the dQ stage when it takes the dS that dK/dV hands
     * over (nsa_sel_bwd_ds_handoff() != 0; ignored otherwise).  Page 3 of the
     * reference text (the pull request porting the SM80 SDPA backward; the
     * review comment on bwd_params_for_flavor) passes a scheduling policy to
     * its backward: natural order, with longest-processing-time first named
     * as a pending tweak for packed inputs.  0: one workgroup per (token
     * window, KV head) item, launched longest first (the latest token
     * windows, which list the most blocks), dealt out by the hardware
     * dispatcher.  1: a persistent grid of one workgroup per compute unit
     * that takes the items in that same order from a counter in the
     * workspace.  Each item is one workgroup's alone either way, so results
     * are bitwise the same.  Other values: NSA_ERR_INVALID_ARG. */
    int32_t sched_policy;
} nsa_sel_problem;

typedef struct hipStream_t_opaque* nsa_stream_t; /* a hipStream_t; NULL = null stream */

/* Forward: o and lse from q, k, v and block_idx (the online softmax over the
 * gathered blocks).  cu_seqlens is NULL for dense inputs.  Needs no
 * workspace. */
nsa_status nsa_sel_fwd(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* block_idx, const int32_t* cu_seqlens, void* o,
                       float* lse, nsa_stream_t stream);

/* Bytes of device workspace nsa_sel_bwd needs for this problem (0 when the
 * problem is invalid; check nsa_last_error()).  The workspace must be
 * 256-byte aligned; its contents need not be initialised. */
size_t nsa_sel_bwd_workspace_bytes(const nsa_sel_problem* p);

/* Backward: dq, dk, dv from q, k, v, the forward's o and lse, dO and
 * block_idx.  Runs, in order on `stream`: Delta = rowsum(dO * o); the
 * block -> query inversion; the dK/dV kernel (per key block and row chunk,
 * no atomics) and its fixed-order reduction; the dQ kernel (no atomics).
 * When the dK/dV kernel hands its dS over to dQ -- bf16, G = 4, 8 or a
 * multiple of 16, block_size >= 32, S <= 64, no window and S * block_size
 * below the longest key range, so selections that cannot cover whole causal
 * prefixes -- dQ is
 * dq = scale dS K from that dS (2 D flops per pair) instead of a
 * recomputation of S and dP per query tile (6 D); the workspace then also
 * holds dS (bf16, block_size * G per listed (token, block) pair).  Results
 * are deterministic (bitwise repeatable). */
nsa_status nsa_sel_bwd(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dO,
                       const int32_t* block_idx, const int32_t* cu_seqlens, void* dq, void* dk,
                       void* dv, void* workspace, size_t workspace_bytes,
                       nsa_stream_t stream);

/* nsa_sel_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from a 64 MiB
 * device array built into the library instead of a caller buffer.  Nothing
 * is allocated (no hipMalloc, hipFree or allocating library call); each GPU
 * the library runs on holds its own copy of the array until the process
 * ends, its address looked up once per device.  When the dS hand-off (see
 * nsa_sel_bwd) would not fit in the array, dQ recomputes dS instead (results
 * then agree with nsa_sel_bwd's within the bf16 tolerance, not bitwise).  A
 * problem that needs more workspace even so is refused with
 * NSA_ERR_WORKSPACE before any HIP call.  The array keeps the last
 * call's contents; nothing in it needs to start at zero.  All calls on one
 * GPU share that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and corrupt each other's results -- order
 * them on one stream or serialise them. */
nsa_status nsa_sel_bwd_noalloc(const nsa_sel_problem* p, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* dO,
                               const int32_t* block_idx, const int32_t* cu_seqlens, void* dq,
                               void* dk, void* dv, nsa_stream_t stream);

/* The backward in three stages on one workspace; nsa_sel_bwd is exactly
 * prepare, dkdv, dq in this order.  prepare computes Delta and the block ->
 * query inversion (and the dK/dV work plan) into the workspace; dkdv and dq
 * read them, so they need a workspace prepared for the same problem,
 * block_idx, o and dO (a caller that reuses one block_idx with several
 * q/k/v/dO may also keep the inversion: dkdv uses Delta, so o/dO must match).
 * dkdv writes fp32 partials into the workspace, and, for problems whose dQ
 * takes over the dK/dV kernel's dS (see nsa_sel_bwd), that dS: dq must then
 * run after dkdv (after nsa_sel_bwd_dkdv_blocks) on the same workspace; for
 * the other problems dq and dkdv are independent.  dq and
 * nsa_sel_bwd_dkdv_reduce are always independent of each other (they read
 * and write disjoint data), so after _blocks they may run concurrently. */
nsa_status nsa_sel_bwd_prepare(const nsa_sel_problem* p, const void* o, const void* dO,
                               const int32_t* block_idx, const int32_t* cu_seqlens,
                               void* workspace, size_t workspace_bytes, nsa_stream_t stream);

/* nsa_sel_bwd_prepare in its two independent parts, same workspace:
 * _lists computes the block -> query inversion and the dK/dV work plan from
 * block_idx alone (so it may run before or during the forward), _delta
 * computes Delta from o and dO.  They write disjoint parts of the
 * workspace: calling both, in either order or concurrently on two streams,
 * equals nsa_sel_bwd_prepare (bitwise). */
nsa_status nsa_sel_bwd_prepare_lists(const nsa_sel_problem* p, const int32_t* block_idx,
                                     const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, nsa_stream_t stream);
nsa_status nsa_sel_bwd_prepare_delta(const nsa_sel_problem* p, const void* o, const void* dO,
                                     const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, nsa_stream_t stream);
nsa_status nsa_sel_bwd_dq(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const int32_t* block_idx,
                          const int32_t* cu_seqlens, void* dq, void* workspace,
                          size_t workspace_bytes, nsa_stream_t stream);
nsa_status nsa_sel_bwd_dkdv(const nsa_sel_problem* p, const void* q, const void* k,
                            const void* v, const void* dO, const float* lse,
                            const int32_t* cu_seqlens, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, nsa_stream_t stream);

/* nsa_sel_bwd_dkdv in its two kernels, same arguments and workspace:
 * _blocks runs the per-key-block kernel (a list handled by one work item
 * goes straight to dk/dv, a longer list to fp32 partials in the workspace),
 * then _reduce sums the partials in a fixed order and writes zeros for
 * blocks no row attends to.  Calling both in this order equals
 * nsa_sel_bwd_dkdv (for dtype f32 all work is in _blocks and _reduce does
 * nothing).  _reduce takes no q/k/v/dO/lse. */
nsa_status nsa_sel_bwd_dkdv_blocks(const nsa_sel_problem* p, const void* q, const void* k,
                                   const void* v, const void* dO, const float* lse,
                                   const int32_t* cu_seqlens, void* dk, void* dv, void* workspace,
                                   size_t workspace_bytes, nsa_stream_t stream);
nsa_status nsa_sel_bwd_dkdv_reduce(const nsa_sel_problem* p, const int32_t* cu_seqlens, void* dk,
                                   void* dv, void* workspace, size_t workspace_bytes,
                                   nsa_stream_t stream);

/* Delta preprocess alone: delta[row] = sum_d dO[row, d] * o[row, d] (float
 * accumulation), layout of lse.  The backward's first stage (page 3 names it
 * the do_dot step of its kernel chain). */
nsa_status nsa_sel_delta(const nsa_sel_problem* p, const void* o, const void* dO,
                         const int32_t* cu_seqlens, float* delta, nsa_stream_t stream);

/* Block -> query inversion alone.  For every (z, hkv, u) it lists, in
 * ascending order, the tokens t >= u * block_size whose row lists block u
 * (once each; with a sliding window, only those whose window reaches the
 * block: (u + 1) * block_size > t - window + 1).  Z = B (dense) or n_seqs (packed); NBmax = ceil(T /
 * block_size) (dense) or ceil(max_seqlen / block_size) (packed); Smin =
 * min(S, NBmax).  Outputs: offsets [Z][Hkv][NBmax + 1] int32, offsets of
 * each list inside the (z, hkv) region of `tokens` (offsets[..][0] = 0, the
 * last one is the region's entry count; blocks past a packed sequence's end
 * have empty lists); tokens: the region of (z, hkv) starts at entry
 * Smin * r0, where r0 is the block_idx row of token 0 of (z, hkv):
 * (z * Hkv + hkv) * T dense, hkv * T + cu_seqlens[z] packed.  Capacity of
 * tokens: nsa_sel_invert_tokens_capacity() entries.  Uses the backward's
 * workspace (its size from nsa_sel_bwd_workspace_bytes()). */
nsa_status nsa_sel_invert(const nsa_sel_problem* p, const int32_t* block_idx,
                          const int32_t* cu_seqlens, int32_t* offsets, int32_t* tokens,
                          void* workspace, size_t workspace_bytes, nsa_stream_t stream);

/* Attention sink (page 3's backward chain has a dSink step; the reading
 * taken): sink [Hq] float (device) holds one logit per query head, in natural
 * log units with no scale applied, that joins every row's softmax
 * denominator and carries no value:
 *   lse = log(sum_{j in A} exp(scale <q, k_j>) + exp(sink[h])),
 *   o   = sum_{j in A} exp(scale <q, k_j> - lse) v_j
 * (an empty A gives o = 0, lse = sink[h]).  nsa_sel_fwd_sink is nsa_sel_fwd
 * with the sink (sink == NULL: no sink).  The backward needs nothing new for
 * dq, dk, dv: nsa_sel_bwd (or its stages) given this lse computes them.
 * nsa_sel_bwd_dsink, called after the backward's prepare stage on the same
 * workspace (it reads Delta there), writes dsink [Hq] float:
 *   dsink[h] = -sum over the rows of head h of exp(sink[h] - lse) * Delta
 * in a fixed order (deterministic).  sink must not be NULL there. */
nsa_status nsa_sel_fwd_sink(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* block_idx, const int32_t* cu_seqlens, const float* sink,
                            void* o, float* lse, nsa_stream_t stream);
nsa_status nsa_sel_bwd_dsink(const nsa_sel_problem* p, const float* lse, const float* sink,
                             const int32_t* cu_seqlens, float* dsink, void* workspace,
                             size_t workspace_bytes, nsa_stream_t stream);

/* Validation of a block_idx (optional; the other calls accept any entry).
 * Writes four counts over all rows of the problem into counts[4] (device
 * memory, uint64, overwritten): [0] padding entries (negative), [1] entries
 * out of range (>= NB of the row's sequence), [2] future entries (in range
 * but starting after the row's token: they add no key), [3] repeats (each
 * further occurrence of an in-range block the row already lists; the
 * computation attends such a block once).  These are the readings of page 1's
 * block lists (padding where S exceeds a row's valid block count) that the
 * kernels apply; nothing here changes how they treat an entry.  Needs no
 * workspace; queued on `stream`. */
nsa_status nsa_sel_check_block_idx(const nsa_sel_problem* p, const int32_t* block_idx,
                                   const int32_t* cu_seqlens, uint64_t* counts,
                                   nsa_stream_t stream);

/* Entries the tokens array of nsa_sel_invert must hold: Smin * B * Hkv * T
 * (dense) or Smin * Hkv * T (packed). */
size_t nsa_sel_invert_tokens_capacity(const nsa_sel_problem* p);

/* Health check of the kernels' internal synchronisation.  The waves of a
 * forward, dQ or dK/dV workgroup order their use of shared LDS stages with
 * counters, and every wait on a counter is bounded (about 2^18 polls) so that
 * a kernel always finishes.  *count receives the number of such waits that
 * gave up on the current device since the library was loaded; each one means
 * a launch may have computed from an incomplete stage (a library defect,
 * never expected: 0 is the only healthy value).  Synchronises the current
 * device (a blocking device-to-host copy of the counters). */
nsa_status nsa_sel_wait_timeouts(uint64_t* count);

/* Whether nsa_sel_bwd hands dS from the dK/dV kernel over to dQ for this
 * problem (the conditions stated at nsa_sel_bwd): 1 yes, 0 no, -1 the
 * problem is invalid (see nsa_last_error()).  Host only, no HIP call. */
int32_t nsa_sel_bwd_ds_handoff(const nsa_sel_problem* p);

/* The git commit the library was built from ("unknown" outside a git
 * checkout; "+dirty" when its sources had uncommitted changes). */
const char* nsa_build_git(void);

/* Text of a status code, and the detail of the calling thread's last
 * error (empty string if none). */
const char* nsa_status_string(nsa_status s);
const char* nsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_SEL_H */
