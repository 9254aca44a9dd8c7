// nsa_common.hip -- kernels shared by the bf16 and f32 paths:
//   * delta_*:    Delta[row] = sum_d dO[row, d] * o[row, d]   (backward preprocess;
//                 page 3's kernel chain names this step do_dot)
//   * inv_count / inv_scan / inv_fill: the block -> query inversion.  For every
//                 (z, hkv, block u), the ascending tokens t >= u*bs listing u,
//                 as CSR lists, so that dK/dV of block u can be accumulated by one
//                 owner without global atomics.  Integer work, bit-exact: counts
//                 use LDS atomics (order-free), the fill is a stable pass.
//   * plan:       global prefix of dK/dV work items and fp32 partial slots
//                 (written by the scan's last workgroup).
#include <algorithm>

#include "nsa_internal.h"

namespace nsa {

// ---- Delta ----------------------------------------------------------------

// Row r of lse / delta ([B][Hq][T] dense, [Hq][T] packed) -> element
// offsets of its rows in o and dO.  r0 is a row of the same workgroup at or
// before r (wave-uniform), so the one 64-bit division per workgroup is
// scalar; a batch entry holds Hq * T < 2^31 rows (checked on the host), so
// the rest is 32-bit.
__device__ __forceinline__ void delta_row_offsets(const Problem& p, int64_t r0, int64_t r,
                                                  int64_t& oo, int64_t& od) {
    const uint32_t per = (uint32_t)p.Hq * (uint32_t)p.T;
    uint32_t b = (uint32_t)(r0 / per);
    uint32_t rr = (uint32_t)(r - (int64_t)b * per);
    while (rr >= per) {  // a workgroup's rows span few entries
        rr -= per;
        ++b;
    }
    const uint32_t h = rr / (uint32_t)p.T, t = rr - h * (uint32_t)p.T;
    oo = (int64_t)b * p.lo.sb + (int32_t)(h * p.lo.sh + t * p.lo.st);
    od = (int64_t)b * p.ldo.sb + (int32_t)(h * p.ldo.sh + t * p.ldo.st);
}

// bf16 rows: D/8 lanes per row, 16-byte loads, fp32 products and sums.
// A lane's eight products, summed in element order:
__device__ __forceinline__ float delta_dot8(uint4 a, uint4 b) {
    const uint32_t av[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc += bf16_to_f32(av[i] & 0xffff) * bf16_to_f32(bv[i] & 0xffff);
        acc += bf16_to_f32(av[i] >> 16) * bf16_to_f32(bv[i] >> 16);
    }
    return acc;
}
// ... then over the row's TPR lanes by a butterfly.
template <int TPR>
__device__ __forceinline__ float delta_lanes_sum(float acc) {
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
    return acc;
}

// One 256-thread block covers rows [blk * 256 / (D/8), ...) in lse order.
template <int D>
__device__ __forceinline__ void delta_rows_bf16(const Problem& p, const uint16_t* __restrict__ o,
                                                const uint16_t* __restrict__ dO,
                                                float* __restrict__ delta, int64_t nrows, int64_t blk) {
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    int64_t r = blk * RPB + threadIdx.x / TPR;
    int part = threadIdx.x % TPR;
    float acc = 0.f;
    if (r < nrows) {
        int64_t oo, od;
        delta_row_offsets(p, blk * RPB, r, oo, od);
        acc = delta_dot8(ldg16(o + oo + part * 8), ldg16(dO + od + part * 8));
    }
    acc = delta_lanes_sum<TPR>(acc);
    if (r < nrows && part == 0) delta[r] = acc;
}

template <int D>
constexpr int delta_rows_per_block() { return 256 / (D / 8); }

// The stand-alone Delta launch: NR groups of 256 / (D/8) rows per block, each
// thread issuing the loads of all its NR rows before the first product, so
// that a quarter as many, longer-lived blocks keep four times the bytes in
// flight.  Each row's arithmetic is the one above (same lanes, same order),
// so Delta is bitwise the same as from count_delta_kernel.
template <int D, int NR>
__global__ __launch_bounds__(256) void delta_bf16_kernel(Problem p, const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dO,
                                                         float* __restrict__ delta, int64_t nrows) {
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    const int64_t r0 = (int64_t)blockIdx.x * (RPB * NR);
    const int part = threadIdx.x % TPR;
    uint4 a[NR], b[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t r = r0 + i * RPB + threadIdx.x / TPR;
        a[i] = make_uint4(0, 0, 0, 0);
        b[i] = a[i];
        if (r < nrows) {
            int64_t oo, od;
            delta_row_offsets(p, r0, r, oo, od);
            a[i] = ldg16(o + oo + part * 8);
            b[i] = ldg16(dO + od + part * 8);
        }
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int64_t r = r0 + i * RPB + threadIdx.x / TPR;
        const float acc = delta_lanes_sum<TPR>(r < nrows ? delta_dot8(a[i], b[i]) : 0.f);
        if (r < nrows && part == 0) delta[r] = acc;
    }
}

__global__ __launch_bounds__(256) void delta_f32_kernel(Problem p, const float* __restrict__ o,
                                                        const float* __restrict__ dO,
                                                        float* __restrict__ delta, int64_t nrows) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= nrows) return;
    int64_t oo, od;
    delta_row_offsets(p, (int64_t)blockIdx.x * blockDim.x, r, oo, od);
    float acc = 0.f;
    for (int d = 0; d < p.D; ++d) acc += o[oo + d] * dO[od + d];
    delta[r] = acc;
}

// Row groups per block of the stand-alone bf16 Delta launch.
constexpr int kDeltaGroups = 4;

hipError_t launch_delta(const HostProblem& hp, const void* o, const void* dO, float* delta,
                        hipStream_t st) {
    const Problem& p = hp.dev;
    int64_t nrows = hp.rows;
    if (nrows == 0) return hipSuccess;
    if (hp.dtype == 1) {
        constexpr int NR = kDeltaGroups;
        const int rpb = 256 / (p.D / 8) * NR;
        dim3 grid((unsigned)((nrows + rpb - 1) / rpb));
        switch (p.D) {
            case 32:
                hipLaunchKernelGGL((delta_bf16_kernel<32, NR>), grid, dim3(256), 0, st, p,
                                   (const uint16_t*)o, (const uint16_t*)dO, delta, nrows);
                break;
            case 64:
                hipLaunchKernelGGL((delta_bf16_kernel<64, NR>), grid, dim3(256), 0, st, p,
                                   (const uint16_t*)o, (const uint16_t*)dO, delta, nrows);
                break;
            case 128:
                hipLaunchKernelGGL((delta_bf16_kernel<128, NR>), grid, dim3(256), 0, st, p,
                                   (const uint16_t*)o, (const uint16_t*)dO, delta, nrows);
                break;
            default:
                return hipErrorInvalidValue;
        }
    } else {
        dim3 grid((unsigned)((nrows + 255) / 256));
        hipLaunchKernelGGL(delta_f32_kernel, grid, dim3(256), 0, st, p, (const float*)o,
                           (const float*)dO, delta, nrows);
    }
    return hipGetLastError();
}

// ---- inversion ----------------------------------------------------------------
//
// Per (z, hkv) the tokens are cut into C chunks of CT tokens.  count: per
// chunk, how many of its tokens list each block (LDS histogram), stored
// block-major [zh][u][c].  scan: one flat exclusive prefix over that
// block-major array gives, for chunk c, where its first entry of block u goes
// (all earlier blocks, then earlier chunks of u); its last workgroup also
// writes the dK/dV work plan.  fill: the waves of a chunk's workgroup take
// consecutive runs of its tokens, split each block's cursor by their counts,
// and append their tokens in ascending order, so every list is ascending (a
// stable counting sort; bit-exact).
//
// A row's entry u counts when 0 <= u < NBz and u*bs <= t (and, with a
// sliding window W, the block reaches into the window: (u+1)*bs > t - W + 1;
// a listing whose keys all lie below the window adds nothing), once however
// often the row repeats it.  Each wave keeps a 16-bit array `last` over the blocks:
// every valid entry of the row first writes its position in the row to
// last[u] (lanes of one write that hit the same u leave exactly one of their
// positions), then the entry whose position survived stands for u.  Every u
// of the row is written before it is read, so `last` needs no clearing
// between rows; plain LDS writes and reads replace atomics, and distinct
// blocks never contend for one word.
// (tp: the row's key position, token + qoff)
__device__ __forceinline__ bool entry_ok(int u, int NBz, int bs, int tp, int W) {
    return u >= 0 && u < NBz && u * bs <= tp && (W <= 0 || (u + 1) * bs > tp - W + 1);
}

// Calls f(u, si) once per distinct valid entry u of row (S entries, key
// position tp), from the lane holding the representative entry si (lane si
// % 64).
// Rows of up to 65535 entries (positions fit 16 bits).
template <typename F>
__device__ __forceinline__ void for_each_distinct(const int* row, int S, int NBz, int bs, int tp,
                                                  int W, int lane, volatile uint16_t* last, F&& f) {
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int si = s0 + lane;
        const int u = si < S ? row[si] : -1;
        if (entry_ok(u, NBz, bs, tp, W)) last[u] = (uint16_t)si;
    }
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int si = s0 + lane;
        const int u = si < S ? row[si] : -1;
        if (entry_ok(u, NBz, bs, tp, W) && last[u] == (uint16_t)si) f(u, si);
    }
}

constexpr int kInvWaves = 4;
constexpr int kRowStage = 4096;  // ints of block_idx staged in LDS at a time

// Rows of tokens [t0, t1) of (z, hkv) are contiguous in block_idx: copy
// them to LDS with coalesced loads (t1 - t0 <= kRowStage / S).
__device__ __forceinline__ void stage_rows(const Problem& p, const Seq& s, const int* idx, int hkv,
                                           int t0, int t1, int* buf) {
    const int* src = idx_row(p, s, idx, hkv, t0);
    const int n = (t1 - t0) * p.S;
    // Unrolled so that several loads of each thread are in flight at once.
#pragma unroll 8
    for (int i = threadIdx.x; i < n; i += blockDim.x) buf[i] = src[i];
}

// Block-idx entries per block for chunk c of (z, hkv) zh: 4 waves take the
// chunk's tokens round-robin and count each row's distinct valid entries in
// an LDS histogram (integer atomics: the counts do not depend on order).
__device__ __forceinline__ void count_chunk(const Problem& p, int CT, int C, const int* __restrict__ idx,
                                            int* __restrict__ chunk_pos, int c, int zh,
                                            int* __restrict__ ticket) {
    // The scan that follows counts its finished workgroups from zero, and the
    // persistent hand-off dQ its items and leavers.
    if (c == 0 && zh == 0 && threadIdx.x < 3) ticket[threadIdx.x] = 0;
    extern __shared__ int sm[];
    int* hist = sm;                                          // [NBmax]
    const int NBH = (p.NBmax + 1) / 2;                       // ints per 16-bit array
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    volatile uint16_t* last = reinterpret_cast<volatile uint16_t*>(sm + p.NBmax + w * NBH);
    int* rows = sm + p.NBmax + kInvWaves * NBH;              // [kRowStage]
    const int z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    const int NBz = (s.klen + p.bs - 1) / p.bs;
    for (int u = threadIdx.x; u < p.NBmax; u += blockDim.x) hist[u] = 0;
    const int t_end = min(c * CT + CT, s.len);
    const int per = max(1, kRowStage / p.S);
    for (int tb = c * CT; tb < t_end; tb += per) {
        const int te = min(tb + per, t_end);
        __syncthreads();
        stage_rows(p, s, idx, hkv, tb, te, rows);
        __syncthreads();
        for (int t = tb + w; t < te; t += kInvWaves)
            for_each_distinct(rows + (t - tb) * p.S, p.S, NBz, p.bs, t + s.qoff, p.window, lane, last,
                              [&](int u, int) { atomicAdd(&hist[u], 1); });
    }
    __syncthreads();
    int* out = chunk_pos + (int64_t)zh * p.NBmax * C;
    for (int u = threadIdx.x; u < p.NBmax; u += blockDim.x) out[(int64_t)u * C + c] = hist[u];
}

__global__ __launch_bounds__(64 * kInvWaves) void inv_count_kernel(Problem p, int CT, int C,
                                                                   const int* __restrict__ idx,
                                                                   int* __restrict__ chunk_pos,
                                                                   int* __restrict__ ticket) {
    count_chunk(p, CT, C, idx, chunk_pos, blockIdx.x, blockIdx.y, ticket);
}

// The backward's first launch for bf16: the count blocks (C per (z, hkv),
// first in the grid, latency-bound) and the Delta blocks (bandwidth-bound)
// run side by side instead of one kernel after the other.
template <int D>
__global__ __launch_bounds__(256) void count_delta_kernel(Problem p, int CT, int C, int ZH,
                                                          const int* __restrict__ idx,
                                                          int* __restrict__ chunk_pos,
                                                          int* __restrict__ ticket,
                                                          const uint16_t* __restrict__ o,
                                                          const uint16_t* __restrict__ dO,
                                                          float* __restrict__ delta, int64_t nrows) {
    static_assert(64 * kInvWaves == 256, "count and Delta blocks share one block size");
    const int64_t n_count = (int64_t)C * ZH;
    if ((int64_t)blockIdx.x < n_count)
        count_chunk(p, CT, C, idx, chunk_pos, blockIdx.x % C, blockIdx.x / C, ticket);
    else
        delta_rows_bf16<D>(p, o, dO, delta, nrows, (int64_t)blockIdx.x - n_count);
}

// Exclusive prefix of one int per thread over a 256-thread block (x of
// thread i lands in thread i + 1's result); *total gets the sum.  Shuffle
// scan inside each wave, then the four wave sums through scratch[0..4).
// Ends with a barrier, so scratch may be reused at once.
__device__ __forceinline__ int block_scan256(int x, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    if (lane == 63) scratch[w] = v;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sw = scratch[i];
        base += i < w ? sw : 0;
        tot += sw;
    }
    *total = tot;
    __syncthreads();
    return base + v - x;
}

// Exclusive prefix sum of vals[0..n) (LDS) by one 256-thread block into
// out[0..n] (out[n] = total).  scratch: 4 ints of LDS.
__device__ void block_excl_scan(const int* vals, int n, int* out, int* scratch) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    const int a = min(tid * per, n), b = min(a + per, n);
    int sum = 0;
    for (int i = a; i < b; ++i) sum += vals[i];
    int total;
    int run = block_scan256(sum, scratch, &total);
    if (tid == 0) out[n] = total;
    for (int i = a; i < b; ++i) {
        int x = vals[i];
        out[i] = run;
        run += x;
    }
    __syncthreads();
}

// In-place exclusive prefix sum of a global array of n ints by one
// 256-thread block, through LDS: coalesced copy in (entry i at i + i / 64,
// so the 64-entry segment of each thread starts on its own bank), each
// thread sums its segment, one scan of the 256 segment sums, each thread
// rewrites its segment, coalesced copy out.  Returns the total to every
// thread.  buf: n + n / 64 + 1 ints of LDS; scratch: 4 ints.
__device__ int block_excl_scan_global(int* a, int n, int* buf, int* scratch) {
    const int tid = threadIdx.x, nt = blockDim.x;  // nt == 256
#pragma unroll 16
    for (int i = tid; i < n; i += nt) buf[i + (i >> 6)] = a[i];
    __syncthreads();
    const int nseg = (n + 63) >> 6;  // 64-entry segments, 256 per pass
    int carry = 0;
    for (int s0 = 0; s0 < nseg; s0 += nt) {
        const int seg = s0 + tid;
        const int lo = seg * 64, hi = min(lo + 64, n);
        int* sb = buf + seg * 65;
        int sum = 0;
        for (int i = lo; i < hi; ++i) sum += sb[i - lo];
        int pass_total;
        int run = carry + block_scan256(sum, scratch, &pass_total);
        for (int i = lo; i < hi; ++i) {
            const int x = sb[i - lo];
            sb[i - lo] = run;
            run += x;
        }
        carry += pass_total;
    }
    __syncthreads();
#pragma unroll 16
    for (int i = tid; i < n; i += nt) a[i] = buf[i + (i >> 6)];
    __syncthreads();
    return carry;
}

// Per (z, hkv): list cursors for every (block, chunk), CSR offsets, and the
// number of dK/dV work items (ceil(rows / CR), rows = tokens * G; at least
// one for a block inside the sequence when min1, so that its workgroup
// writes the zeros of an empty list) and fp32 partial slots (the items, when
// a list needs more than one) per list.
__global__ __launch_bounds__(256) void inv_scan_kernel(Problem p, int C, int CR, int min1,
                                                       int* __restrict__ chunk_pos,
                                                       int* __restrict__ offsets,
                                                       int* __restrict__ item_pre,
                                                       int* __restrict__ pslot_pre,
                                                       int* __restrict__ zh_base,
                                                       int* __restrict__ ticket) {
    int* zh_tot = zh_base + 2 * (gridDim.x + 1);
    extern __shared__ int sm[];
    const int NB = p.NBmax;
    const int VN = max(NB, (int)gridDim.x);
    int* vals = sm;             // [max(NB, ZH)]
    int* scratch = sm + VN;     // [257]
    int* sbuf = sm + VN + 257;  // [NB C + NB C / 64 + 1]
    const int zh = blockIdx.x;
    int* cp = chunk_pos + (int64_t)zh * NB * C;
    int* off = offsets + (int64_t)zh * (NB + 1);
    const int total = block_excl_scan_global(cp, NB * C, sbuf, scratch);
    for (int u = threadIdx.x; u < NB; u += blockDim.x) {
        const int i = u * C;  // the scanned table is still in sbuf
        vals[u] = sbuf[i + (i >> 6)];
    }
    __syncthreads();
    for (int u = threadIdx.x; u <= NB; u += blockDim.x) off[u] = u < NB ? vals[u] : total;
    __syncthreads();
    const Seq sq = seq_of(p, zh / p.Hkv);
    const int len = sq.klen;  // keys: every block inside them gets an item below
    // Whole causal prefixes: a row's listed blocks can only be blocks at or
    // before its own, so every row lists all of them exactly when every block
    // u of the keys is listed by every token whose key position t + qoff
    // reaches it: len - u bs tokens from u bs on when queries and keys align.
    int short_list = 0;
    for (int u = threadIdx.x; u < NB; u += blockDim.x)
        if (u * p.bs < len && off[u + 1] - off[u] != sq.len - max(0, u * p.bs - sq.qoff)) short_list = 1;
    const int zh_full = !__syncthreads_or(short_list);
    for (int u = threadIdx.x; u < NB; u += blockDim.x) {
        const int rows = (off[u + 1] - off[u]) * p.G;
        const int items = (rows + CR - 1) / CR;
        vals[u] = min1 && u * p.bs < len ? max(items, 1) : items;
    }
    __syncthreads();
    int* ipre = item_pre + (int64_t)zh * (NB + 1);
    block_excl_scan(vals, NB, ipre, scratch);
    for (int u = threadIdx.x; u < NB; u += blockDim.x) vals[u] = vals[u] > 1 ? vals[u] : 0;
    __syncthreads();
    int* ppre = pslot_pre + (int64_t)zh * (NB + 1);
    block_excl_scan(vals, NB, ppre, scratch);
    // The last workgroup to finish also writes the global prefixes over
    // (z, hkv) of items and partial slots (the dK/dV work plan): each
    // workgroup publishes its totals, then takes a ticket; the one holding
    // the last ticket reads every total back from L2.
    __shared__ int last;
    if (threadIdx.x == 0) {
        zh_tot[zh] = ipre[NB];
        zh_tot[gridDim.x + zh] = ppre[NB];
        zh_tot[2 * gridDim.x + zh] = zh_full;
        __threadfence();
        last = atomicAdd(ticket, 1) == (int)gridDim.x - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    const int ZH = gridDim.x;
    for (int i = threadIdx.x; i < ZH; i += blockDim.x)
        vals[i] = __hip_atomic_load(&zh_tot[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    block_excl_scan(vals, ZH, zh_base, scratch);
    for (int i = threadIdx.x; i < ZH; i += blockDim.x)
        vals[i] = __hip_atomic_load(&zh_tot[ZH + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    block_excl_scan(vals, ZH, zh_base + ZH + 1, scratch);
    // Every (z, hkv) selects whole causal prefixes: the flag the dK/dV
    // launches read (zh_base[2 (ZH + 1) + 3 ZH]).
    int part = 0;
    for (int i = threadIdx.x; i < ZH; i += blockDim.x)
        if (!__hip_atomic_load(&zh_tot[2 * ZH + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) part = 1;
    const int any_short = __syncthreads_or(part);
    if (threadIdx.x == 0) zh_tot[3 * ZH] = !any_short;
}

// Stable fill of chunk c of (z, hkv) zh by NW waves.  The chunk's rows are
// staged in LDS a batch of tokens at a time; the batch's tokens are cut into
// NW consecutive runs, one per wave.  Each wave counts the distinct valid
// entries of its run per block (hist[w][u], plain LDS increments: a row's
// lanes hold distinct blocks and a wave takes its rows one after another),
// the block cursors are then split over the waves in wave order (hist[w][u]
// becomes the first position of wave w's entries of block u), and each wave
// appends its tokens, ascending, at those positions.  So every list is
// ascending in t, exactly as one wave walking the whole chunk would write it.
// whole: the whole-prefix flag the scan wrote (null when the lists are
// always wanted).  When it is set the backward needs no lists (every list of
// block u is the tokens u bs .. len - 1, read from iota[u bs ..] instead):
// the workgroups of (z, hkv) 0 write iota[t] = t for their chunk and return.
// posmap (optional, laid out like block_idx): for every row and slot, the
// position of the row's token in the list of the slot's block, -1 for slots
// that are no entry (padding, out of range, future, outside the window, or
// a repeat of a block the row lists in another slot).
__global__ __launch_bounds__(512) void inv_fill_kernel(Problem p, int CT, int C,
                                                       const int* __restrict__ idx,
                                                       const int* __restrict__ chunk_pos,
                                                       int* __restrict__ tokens,
                                                       const int* __restrict__ whole,
                                                       int* __restrict__ iota,
                                                       int* __restrict__ posmap) {
    if (whole && *whole) {
        if (blockIdx.y == 0)
            for (int t = blockIdx.x * CT + (int)threadIdx.x; t < min(p.Tmax, (int)(blockIdx.x + 1) * CT);
                 t += blockDim.x)
                iota[t] = t;
        return;
    }
    extern __shared__ int sm[];
    const int NB = p.NBmax, NBH = (NB + 1) / 2, NW = (int)blockDim.x >> 6;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int* cursor = sm;                                     // [NB]
    int* hist = sm + NB;                                  // [NW][NB]
    volatile uint16_t* last =
        reinterpret_cast<volatile uint16_t*>(sm + NB + NW * NB + w * NBH);  // [NW][NB] u16
    int* rows = sm + NB + NW * NB + NW * NBH;             // [kRowStage]
    int* hw = hist + w * NB;
    const int c = blockIdx.x, zh = blockIdx.y, z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    if (c * CT >= s.len) return;  // chunk past a short sequence's end
    const int NBz = (s.klen + p.bs - 1) / p.bs;
    const int* cp = chunk_pos + (int64_t)zh * NB * C;
    for (int u = threadIdx.x; u < NB; u += blockDim.x) cursor[u] = cp[(int64_t)u * C + c];
    int* out = tokens + region_base(p, s, hkv);
    const int t_end = min(c * CT + CT, s.len);
    const int per = max(1, kRowStage / p.S);
    for (int tb = c * CT; tb < t_end; tb += per) {
        const int te = min(tb + per, t_end);
        for (int u = lane; u < NB; u += 64) hw[u] = 0;
        __syncthreads();
        stage_rows(p, s, idx, hkv, tb, te, rows);
        __syncthreads();
        // This wave's run of the batch.
        const int n = te - tb, q = n / NW, rm = n % NW;
        const int r0 = tb + w * q + min(w, rm), r1 = r0 + q + (w < rm ? 1 : 0);
        for (int t = r0; t < r1; ++t)
            for_each_distinct(rows + (t - tb) * p.S, p.S, NBz, p.bs, t + s.qoff, p.window, lane, last,
                              [&](int u, int) { hw[u] += 1; });
        __syncthreads();
        for (int u = threadIdx.x; u < NB; u += blockDim.x) {
            int run = cursor[u];
            for (int v = 0; v < NW; ++v) {
                const int x = hist[v * NB + u];
                hist[v * NB + u] = run;
                run += x;
            }
            cursor[u] = run;
        }
        __syncthreads();
        for (int t = r0; t < r1; ++t) {
            // posmap: every slot of the row gets -1, then the slot standing
            // for block u its position in u's list (the same lane writes
            // both, in this order).
            int* pm = posmap ? posmap + (s.i_base + (int64_t)hkv * p.T + t) * p.S : nullptr;
            if (pm)
                for (int si = lane; si < p.S; si += 64) pm[si] = -1;
            for_each_distinct(rows + (t - tb) * p.S, p.S, NBz, p.bs, t + s.qoff, p.window, lane, last,
                              [&](int u, int si) {
                                  const int pos = hw[u];
                                  hw[u] = pos + 1;
                                  out[pos] = t;
                                  if (pm) pm[si] = pos;
                              });
        }
        __syncthreads();
    }
}

// Waves of the fill: as many as LDS allows (at most 8), at least four tokens
// each (measured: with 16-token chunks, 4 waves beat 2 and 8).
int fill_waves(const HostProblem& hp) {
    const int64_t NB = hp.dev.NBmax, NBH = (NB + 1) / 2;
    int nw = 8;
    while (nw > 1 && 4 * (NB + nw * (NB + NBH) + kRowStage) > 163840) --nw;
    return std::max(1, std::min(nw, hp.CT / 4));
}

size_t fill_lds_bytes(const HostProblem& hp, int nw) {
    const int64_t NB = hp.dev.NBmax, NBH = (NB + 1) / 2;
    return sizeof(int) * (size_t)(NB + nw * (NB + NBH) + kRowStage);
}

size_t invert_lds_bytes(const HostProblem& hp) {
    const int64_t NB = hp.dev.NBmax, NBH = (NB + 1) / 2, n_cp = NB * hp.C;
    const int64_t count = NB + kInvWaves * NBH + kRowStage;
    const int64_t scan = std::max<int64_t>(NB, hp.ZH) + 257 + n_cp + n_cp / 64 + 1;
    const int64_t fill = NB + (NB + NBH) + kRowStage;  // one wave: the least the fill needs
    return sizeof(int) * (size_t)std::max(count, std::max(scan, fill));
}

namespace {
size_t count_lds_bytes(const Problem& p) {
    return sizeof(int) * (p.NBmax + kInvWaves * ((p.NBmax + 1) / 2) + kRowStage);
}

// Scan and stable fill (after the counts are in chunk_pos).
hipError_t launch_scan_fill(const HostProblem& hp, const int* block_idx, const BwdWorkspace& ws,
                            hipStream_t st, bool lists_optional) {
    const Problem& p = hp.dev;
    const int64_t n_cp = (int64_t)p.NBmax * hp.C;  // <= 2^14 + NBmax by the choice of CT
    size_t lds_scan = sizeof(int) * (std::max(p.NBmax, hp.ZH) + 257 + n_cp + n_cp / 64 + 1);
    // Without partial slots no list is split and the dK/dV kernel itself
    // writes the zeros of empty lists (one item each), so no reduce runs.
    hipLaunchKernelGGL(inv_scan_kernel, dim3(hp.ZH), dim3(256), lds_scan, st, p, hp.C, hp.CR,
                       hp.pslots == 0 ? 1 : 0, ws.chunk_pos, ws.offsets, ws.item_pre, ws.pslot_pre,
                       ws.zh_base, ws.ticket);
    const int nw = fill_waves(hp);
    const bool skip = lists_optional && hp.pair_possible;
    hipLaunchKernelGGL(inv_fill_kernel, dim3(hp.C, hp.ZH), dim3(64 * nw), fill_lds_bytes(hp, nw), st,
                       p, hp.CT, hp.C, block_idx, ws.chunk_pos, ws.tokens,
                       skip ? ws.zh_base + 2 * (hp.ZH + 1) + 3 * hp.ZH : nullptr, ws.iota,
                       lists_optional && hp.ds_handoff ? ws.posmap : nullptr);
    return hipGetLastError();
}
}  // namespace

// ---- attention-sink gradient -------------------------------------------------
//
// The sink logit of head h joins every row's softmax denominator with no
// value, so o moves by -P_sink o as it grows and its gradient is
// dsink[h] = -sum over the rows of head h of exp(sink[h] - lse) Delta
// (the reading of page 3's dSink chain step).  One 1024-thread workgroup
// per head walks the head's rows (dense: B runs of T, packed: one run of T)
// in a fixed order, four independent loads in flight per thread, and reduces
// its per-thread sums through LDS in a fixed tree, so the result is
// deterministic.
constexpr int kDsinkThreads = 1024;
__global__ __launch_bounds__(kDsinkThreads) void dsink_kernel(Problem p, const float* __restrict__ lse,
                                                              const float* __restrict__ delta,
                                                              const float* __restrict__ sink,
                                                              float* __restrict__ dsink) {
    __shared__ float red[kDsinkThreads];
    const int h = blockIdx.x;
    const float sk = sink[h];
    float acc = 0.f;
    for (int b = 0; b < p.B; ++b) {
        const int64_t base = ((int64_t)b * p.Hq + h) * p.T;  // packed: B = 1, [Hq][T]
#pragma unroll 4
        for (int t = threadIdx.x; t < p.T; t += kDsinkThreads) {
            const float x = lse[base + t];
            acc += x == -__builtin_huge_valf() ? 0.f : __expf(sk - x) * delta[base + t];
        }
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kDsinkThreads / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) dsink[h] = -red[0];
}

hipError_t launch_dsink(const HostProblem& hp, const float* lse, const float* delta,
                        const float* sink, float* dsink, hipStream_t st) {
    if (hp.dev.Hq == 0) return hipSuccess;
    hipLaunchKernelGGL(dsink_kernel, dim3(hp.dev.Hq), dim3(kDsinkThreads), 0, st, hp.dev, lse, delta,
                       sink, dsink);
    return hipGetLastError();
}

// ---- block_idx validation -------------------------------------------------
//
// counts[0..4) (added to zeros): padding entries (negative), out-of-range
// entries (>= NB of the row's sequence), future entries (in range, u * bs >
// t: they add no key), and repeats (each further occurrence of an in-range
// block the row already lists).  One wave per row, four per workgroup; a
// row's distinct in-range blocks are counted with the same 16-bit
// last-writer array as the inversion; per-lane counts, one 64-bit atomic add
// per wave and counter (integer, so the totals are exact).
constexpr int kChkWaves = 4, kChkRows = 64;

__global__ __launch_bounds__(64) void zero_counts_kernel(unsigned long long* __restrict__ counts) {
    if (threadIdx.x < 4) counts[threadIdx.x] = 0ull;
}

__global__ __launch_bounds__(64 * kChkWaves) void check_idx_kernel(Problem p, const int* __restrict__ idx,
                                                                   unsigned long long* __restrict__ counts) {
    extern __shared__ uint16_t lastbuf[];  // [kChkWaves][NBmax]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    volatile uint16_t* last = lastbuf + w * p.NBmax;
    const int zh = blockIdx.y, z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    const int NBz = (s.klen + p.bs - 1) / p.bs;
    unsigned long long c[4] = {0ull, 0ull, 0ull, 0ull};
    const int t0 = blockIdx.x * kChkRows, t1 = min(s.len, t0 + kChkRows);
    for (int t = t0 + w; t < t1; t += kChkWaves) {
        const int* row = idx_row(p, s, idx, hkv, t);
        int inr = 0, dist = 0;
        for (int s0 = 0; s0 < p.S; s0 += 64) {
            const int si = s0 + lane;
            if (si >= p.S) continue;
            const int u = row[si];
            if (u < 0) {
                ++c[0];
            } else if (u >= NBz) {
                ++c[1];
            } else {
                ++inr;
                if ((int64_t)u * p.bs > t + s.qoff) ++c[2];
                last[u] = (uint16_t)si;
            }
        }
        for (int s0 = 0; s0 < p.S; s0 += 64) {
            const int si = s0 + lane;
            if (si >= p.S) continue;
            const int u = row[si];
            if (u >= 0 && u < NBz && last[u] == (uint16_t)si) ++dist;
        }
        c[3] += (unsigned long long)(inr - dist);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned long long x = c[i];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
        if (lane == 0 && x) atomicAdd(&counts[i], x);
    }
}

hipError_t launch_check_idx(const HostProblem& hp, const int* block_idx, unsigned long long* counts,
                            hipStream_t st) {
    const Problem& p = hp.dev;
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, st, counts);
    if (hp.ZH == 0 || p.Tmax == 0 || p.S == 0) return hipGetLastError();
    const dim3 grid((unsigned)((p.Tmax + kChkRows - 1) / kChkRows), (unsigned)hp.ZH);
    hipLaunchKernelGGL(check_idx_kernel, grid, dim3(64 * kChkWaves),
                       sizeof(uint16_t) * kChkWaves * (size_t)p.NBmax, st, p, block_idx, counts);
    return hipGetLastError();
}

hipError_t launch_invert(const HostProblem& hp, const int* block_idx, const BwdWorkspace& ws,
                         hipStream_t st) {
    const Problem& p = hp.dev;
    if (hp.ZH == 0 || hp.C == 0) return hipSuccess;
    hipLaunchKernelGGL(inv_count_kernel, dim3(hp.C, hp.ZH), dim3(64 * kInvWaves), count_lds_bytes(p),
                       st, p, hp.CT, hp.C, block_idx, ws.chunk_pos, ws.ticket);
    return launch_scan_fill(hp, block_idx, ws, st, false);
}

// The prepare stage without Delta: the inversion and the dK/dV plan (as the
// backward needs them, lists optional for whole-prefix selections).
hipError_t launch_prepare_lists(const HostProblem& hp, const int* block_idx, const BwdWorkspace& ws,
                                hipStream_t st) {
    const Problem& p = hp.dev;
    if (hp.ZH == 0 || hp.C == 0) return hipSuccess;
    hipLaunchKernelGGL(inv_count_kernel, dim3(hp.C, hp.ZH), dim3(64 * kInvWaves), count_lds_bytes(p),
                       st, p, hp.CT, hp.C, block_idx, ws.chunk_pos, ws.ticket);
    return launch_scan_fill(hp, block_idx, ws, st, true);
}

hipError_t launch_prepare(const HostProblem& hp, const void* o, const void* dO, const int* block_idx,
                          const BwdWorkspace& ws, hipStream_t st) {
    const Problem& p = hp.dev;
    if (hp.dtype != 1 || hp.ZH == 0 || hp.C == 0 || hp.rows == 0) {
        const hipError_t e = launch_delta(hp, o, dO, ws.delta, st);
        if (e != hipSuccess) return e;
        return launch_invert(hp, block_idx, ws, st);
    }
    const int64_t n_count = (int64_t)hp.C * hp.ZH;
    auto go = [&](auto kernel, int rpb) {
        const int64_t n_delta = (hp.rows + rpb - 1) / rpb;
        hipLaunchKernelGGL(kernel, dim3((unsigned)(n_count + n_delta)), dim3(256), count_lds_bytes(p), st,
                           p, hp.CT, hp.C, hp.ZH, block_idx, ws.chunk_pos, ws.ticket, (const uint16_t*)o,
                           (const uint16_t*)dO, ws.delta, hp.rows);
    };
    switch (p.D) {
        case 32: go(count_delta_kernel<32>, delta_rows_per_block<32>()); break;
        case 64: go(count_delta_kernel<64>, delta_rows_per_block<64>()); break;
        case 128: go(count_delta_kernel<128>, delta_rows_per_block<128>()); break;
        default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // The backward reads lists only through the dK/dV launches, which take
    // them from iota when the selection is a whole prefix everywhere.
    return launch_scan_fill(hp, block_idx, ws, st, true);
}


}  // namespace nsa
