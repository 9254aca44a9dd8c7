// nsa_common.hip -- kernels shared by the bf16 and f32 paths:
//   * delta_*:    Delta[row] = sum_d dO[row, d] * o[row, d]   (backward preprocess;
//                 page 3's kernel chain names this step do_dot)
//   * inv_count / inv_scan / inv_fill: the block -> query inversion.  For every
//                 (z, hkv, block u), the ascending tokens t >= u*bs listing u,
//                 as CSR lists, so that dK/dV of block u can be accumulated by one
//                 owner without global atomics.  Integer work, bit-exact: counts
//                 use LDS atomics (order-free), the fill is a stable sequential pass.
//   * plan:       global prefix of dK/dV work items and fp32 partial slots.
#include "nsa_internal.h"

namespace nsa {

// ---- Delta ----------------------------------------------------------------

// bf16 rows: D/8 lanes per row, 16-byte loads, fp32 products and sums.
template <int D>
__global__ __launch_bounds__(256) void delta_bf16_kernel(Problem p, const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dO,
                                                         float* __restrict__ delta, int64_t nrows) {
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    int part = threadIdx.x % TPR;
    float acc = 0.f;
    if (r < nrows) {
        uint4 a = ldg16(o + r * D + part * 8);
        uint4 b = ldg16(dO + r * D + part * 8);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc += bf16_to_f32(av[i] & 0xffff) * bf16_to_f32(bv[i] & 0xffff);
            acc += bf16_to_f32(av[i] >> 16) * bf16_to_f32(bv[i] >> 16);
        }
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
    if (r < nrows && part == 0) {
        int64_t out = r;
        if (p.packed) {  // q rows are (token, h); delta is [Hq][T]
            int64_t tok = r / p.Hq, h = r % p.Hq;
            out = h * p.T + tok;
        }
        delta[out] = acc;
    }
}

__global__ __launch_bounds__(256) void delta_f32_kernel(Problem p, const float* __restrict__ o,
                                                        const float* __restrict__ dO,
                                                        float* __restrict__ delta, int64_t nrows) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= nrows) return;
    float acc = 0.f;
    for (int d = 0; d < p.D; ++d) acc += o[r * p.D + d] * dO[r * p.D + d];
    int64_t out = r;
    if (p.packed) {
        int64_t tok = r / p.Hq, h = r % p.Hq;
        out = h * p.T + tok;
    }
    delta[out] = acc;
}

hipError_t launch_delta(const HostProblem& hp, const void* o, const void* dO, float* delta,
                        hipStream_t st) {
    const Problem& p = hp.dev;
    int64_t nrows = hp.rows;
    if (nrows == 0) return hipSuccess;
    if (hp.dtype == 1) {
        int rpb = 256 / (p.D / 8);
        dim3 grid((unsigned)((nrows + rpb - 1) / rpb));
        switch (p.D) {
            case 32:
                hipLaunchKernelGGL(delta_bf16_kernel<32>, grid, dim3(256), 0, st, p,
                                   (const uint16_t*)o, (const uint16_t*)dO, delta, nrows);
                break;
            case 64:
                hipLaunchKernelGGL(delta_bf16_kernel<64>, grid, dim3(256), 0, st, p,
                                   (const uint16_t*)o, (const uint16_t*)dO, delta, nrows);
                break;
            case 128:
                hipLaunchKernelGGL(delta_bf16_kernel<128>, grid, dim3(256), 0, st, p,
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

// ---- inversion --------------------------------------------------------------

// Does slot si of this row contribute an entry for token t?  A block number
// in [0, NBz) whose first key is <= t, and the first slot holding that block.
__device__ __forceinline__ bool entry_valid(const int* row, int si, int u, int NBz, int bs, int t) {
    if (u < 0 || u >= NBz || u * bs > t) return false;
    for (int s2 = 0; s2 < si; ++s2)
        if (row[s2] == u) return false;
    return true;
}

__global__ __launch_bounds__(256) void inv_count_kernel(Problem p, int CT, int C,
                                                        const int* __restrict__ idx,
                                                        int* __restrict__ chunk_pos) {
    extern __shared__ int hist[];
    const int c = blockIdx.x, zh = blockIdx.y, z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    const int NBz = (s.len + p.bs - 1) / p.bs;
    for (int u = threadIdx.x; u < p.NBmax; u += blockDim.x) hist[u] = 0;
    __syncthreads();
    const int t_end = min(c * CT + CT, s.len);
    for (int t = c * CT + threadIdx.x; t < t_end; t += blockDim.x) {
        const int* row = idx_row(p, s, idx, hkv, t);
        for (int si = 0; si < p.S; ++si) {
            int u = row[si];
            if (entry_valid(row, si, u, NBz, p.bs, t)) atomicAdd(&hist[u], 1);
        }
    }
    __syncthreads();
    int* out = chunk_pos + ((int64_t)zh * C + c) * p.NBmax;
    for (int u = threadIdx.x; u < p.NBmax; u += blockDim.x) out[u] = hist[u];
}

// Exclusive prefix sum of vals[0..n) (LDS) by one 256-thread block into
// out[0..n] (out[n] = total).  scratch: 256 ints of LDS.
__device__ void block_excl_scan(const int* vals, int n, int* out, int* scratch) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    const int a = min(tid * per, n), b = min(a + per, n);
    int sum = 0;
    for (int i = a; i < b; ++i) sum += vals[i];
    scratch[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < nt; ++i) {
            int x = scratch[i];
            scratch[i] = run;
            run += x;
        }
        out[n] = run;
    }
    __syncthreads();
    int run = scratch[tid];
    for (int i = a; i < b; ++i) {
        int x = vals[i];
        out[i] = run;
        run += x;
    }
    __syncthreads();
}

// Per (z, hkv): list sizes, CSR offsets, per-chunk fill cursors, and the
// number of dK/dV work items (ceil(rows / CR), rows = tokens * G) and fp32
// partial slots (items, when a list needs more than one) per list.
__global__ __launch_bounds__(256) void inv_scan_kernel(Problem p, int C, int CR,
                                                       int* __restrict__ chunk_pos,
                                                       int* __restrict__ offsets,
                                                       int* __restrict__ item_pre,
                                                       int* __restrict__ pslot_pre,
                                                       int* __restrict__ zh_tot) {
    extern __shared__ int sm[];
    const int NB = p.NBmax;
    int* vals = sm;             // [NB]
    int* scratch = sm + NB;     // [256]
    const int zh = blockIdx.x;
    int* cp = chunk_pos + (int64_t)zh * C * NB;
    int* off = offsets + (int64_t)zh * (NB + 1);
    for (int u = threadIdx.x; u < NB; u += blockDim.x) {
        int run = 0;
        for (int c = 0; c < C; ++c) {
            int x = cp[(int64_t)c * NB + u];
            cp[(int64_t)c * NB + u] = run;
            run += x;
        }
        vals[u] = run;
    }
    __syncthreads();
    block_excl_scan(vals, NB, off, scratch);
    for (int u = threadIdx.x; u < NB; u += blockDim.x) {
        int o0 = off[u];
        for (int c = 0; c < C; ++c) cp[(int64_t)c * NB + u] += o0;
        int rows = vals[u] * p.G;
        vals[u] = (rows + CR - 1) / CR;
    }
    __syncthreads();
    int* ipre = item_pre + (int64_t)zh * (NB + 1);
    block_excl_scan(vals, NB, ipre, scratch);
    for (int u = threadIdx.x; u < NB; u += blockDim.x) vals[u] = vals[u] > 1 ? vals[u] : 0;
    __syncthreads();
    int* ppre = pslot_pre + (int64_t)zh * (NB + 1);
    block_excl_scan(vals, NB, ppre, scratch);
    if (threadIdx.x == 0) {
        zh_tot[zh] = ipre[NB];
        zh_tot[gridDim.x + zh] = ppre[NB];
    }
}

// Stable fill: one wave walks its chunk's tokens in ascending order and
// appends each to the lists of the blocks it validly lists.
__global__ __launch_bounds__(64) void inv_fill_kernel(Problem p, int CT, int C,
                                                      const int* __restrict__ idx,
                                                      const int* __restrict__ chunk_pos,
                                                      int* __restrict__ tokens) {
    extern __shared__ int sm[];
    int* cursor = sm;              // [NBmax]
    int* rowbuf = sm + p.NBmax;    // [S]
    const int c = blockIdx.x, zh = blockIdx.y, z = zh / p.Hkv, hkv = zh % p.Hkv;
    const int lane = threadIdx.x;
    const Seq s = seq_of(p, z);
    const int NBz = (s.len + p.bs - 1) / p.bs;
    const int* cp = chunk_pos + ((int64_t)zh * C + c) * p.NBmax;
    for (int u = lane; u < p.NBmax; u += 64) cursor[u] = cp[u];
    int* out = tokens + region_base(p, s, hkv);
    const int t_end = min(c * CT + CT, s.len);
    __syncthreads();
    for (int t = c * CT; t < t_end; ++t) {
        const int* row = idx_row(p, s, idx, hkv, t);
        for (int si = lane; si < p.S; si += 64) rowbuf[si] = row[si];
        __syncthreads();
        for (int s0 = 0; s0 < p.S; s0 += 64) {
            int si = s0 + lane;
            if (si < p.S) {
                int u = rowbuf[si];
                if (entry_valid(rowbuf, si, u, NBz, p.bs, t)) {
                    int pos = cursor[u];
                    cursor[u] = pos + 1;
                    out[pos] = t;
                }
            }
            __syncthreads();
        }
    }
}

// Global exclusive prefixes over (z, hkv) of work items and partial slots.
__global__ __launch_bounds__(256) void plan_kernel(int ZH, const int* __restrict__ zh_tot,
                                                   int* __restrict__ zh_base) {
    extern __shared__ int sm[];
    int* vals = sm;
    int* scratch = sm + ZH;
    for (int i = threadIdx.x; i < ZH; i += blockDim.x) vals[i] = zh_tot[i];
    __syncthreads();
    block_excl_scan(vals, ZH, zh_base, scratch);
    for (int i = threadIdx.x; i < ZH; i += blockDim.x) vals[i] = zh_tot[ZH + i];
    __syncthreads();
    block_excl_scan(vals, ZH, zh_base + ZH + 1, scratch);
}

hipError_t launch_invert(const HostProblem& hp, const int* block_idx, const BwdWorkspace& ws,
                         hipStream_t st) {
    const Problem& p = hp.dev;
    if (hp.ZH == 0) return hipSuccess;
    dim3 grid(hp.C, hp.ZH);
    size_t lds_count = sizeof(int) * p.NBmax;
    hipLaunchKernelGGL(inv_count_kernel, grid, dim3(256), lds_count, st, p, hp.CT, hp.C,
                       block_idx, ws.chunk_pos);
    size_t lds_scan = sizeof(int) * (p.NBmax + 256);
    hipLaunchKernelGGL(inv_scan_kernel, dim3(hp.ZH), dim3(256), lds_scan, st, p, hp.C, hp.CR,
                       ws.chunk_pos, ws.offsets, ws.item_pre, ws.pslot_pre,
                       ws.zh_base + 2 * (hp.ZH + 1));
    size_t lds_fill = sizeof(int) * (p.NBmax + p.S);
    hipLaunchKernelGGL(inv_fill_kernel, grid, dim3(64), lds_fill, st, p, hp.CT, hp.C, block_idx,
                       ws.chunk_pos, ws.tokens);
    return hipGetLastError();
}

hipError_t launch_plan(const HostProblem& hp, const BwdWorkspace& ws, hipStream_t st) {
    if (hp.ZH == 0) return hipSuccess;
    size_t lds = sizeof(int) * (hp.ZH + 256);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), lds, st, hp.ZH,
                       ws.zh_base + 2 * (hp.ZH + 1), ws.zh_base);
    return hipGetLastError();
}

}  // namespace nsa
