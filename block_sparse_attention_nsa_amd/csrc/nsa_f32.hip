// nsa_f32.hip -- float32 kernels on the vector ALU (no fp32 rounding of the
// inputs): one thread per query row for the forward and dQ, one thread per
// key for dK/dV (walking that key's block list from the inversion).  These
// serve float32 problems, whose tolerance (2e-3 max-abs on page 1's gate)
// bf16 matrix-core arithmetic could not meet.
#include "nsa_internal.h"

namespace nsa {

// Packed layouts: the sequence holding global token `tok` (cu ascending).
__device__ __forceinline__ int seq_of_token(const Problem& p, int tok) {
    int lo = 0, hi = p.Z;  // cu[lo] <= tok < cu[hi] for valid cu
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (p.cu[mid] <= tok) lo = mid; else hi = mid;
    }
    return lo;
}

// Row r of the q-like tensor -> (z, h, t).  Dense rows are (b, h, t); packed
// rows are (token, h).
// Flat row r of a [B, H, T, ..] (dense; T = Tn) or [Ttot, H, ..] (packed)
// tensor -> (entry, head, token).
__device__ __forceinline__ void decode_qrow(const Problem& p, int64_t r, int H, int& z, int& h,
                                            int& t, int Tn) {
    if (p.packed) {
        int tok = (int)(r / H);
        h = (int)(r % H);
        z = seq_of_token(p, tok);
        t = tok - min(max(p.cu[z], 0), p.T);
    } else {
        t = (int)(r % Tn);
        h = (int)((r / Tn) % H);
        z = (int)(r / ((int64_t)Tn * H));
    }
}

// (tp: the query's key position)
__device__ __forceinline__ bool slot_valid(const int* row, int si, int u, int NBz, int bs, int tp) {
    if (u < 0 || u >= NBz || u * bs > tp) return false;
    for (int s2 = 0; s2 < si; ++s2)
        if (row[s2] == u) return false;
    return true;
}

template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(Problem p, const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const int* __restrict__ idx,
                                                      float* __restrict__ o,
                                                      float* __restrict__ lse, int64_t nrows) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= nrows) return;
    int z, h, t;
    decode_qrow(p, r, p.Hq, z, h, t, p.T);
    const Seq s = seq_of(p, z);
    if (t < 0 || t >= s.len) return;
    const int hkv = h / p.G, NBz = (s.klen + p.bs - 1) / p.bs, tp = t + s.qoff;
    const int* row = idx_row(p, s, idx, hkv, t);
    float qv[D], acc[D];
    const float* qr = q + row_off(p.lq, s, h, t);
    for (int d = 0; d < D; ++d) {
        qv[d] = qr[d] * p.scale_log2;
        acc[d] = 0.f;
    }
    float m = -__builtin_huge_valf(), l = 0.f;
    for (int si = 0; si < p.S; ++si) {
        const int u = row[si];
        if (!slot_valid(row, si, u, NBz, p.bs, tp)) continue;
        const int j1 = min((u + 1) * p.bs, tp + 1);
        // Sliding window: keys tp - window < j only.
        const int j0 = p.window > 0 ? max(u * p.bs, tp - p.window + 1) : u * p.bs;
        for (int j = j0; j < j1; ++j) {
            const float* kr = k + row_off(p.lk, s, hkv, j);
            const float* vr = v + row_off(p.lv, s, hkv, j);
            float x = 0.f;
            for (int d = 0; d < D; ++d) x += qv[d] * kr[d];
            const float mn = fmaxf(m, x);
            const float alpha = exp2f(m - mn);
            const float pj = exp2f(x - mn);
            l = l * alpha + pj;
            for (int d = 0; d < D; ++d) acc[d] = acc[d] * alpha + pj * vr[d];
            m = mn;
        }
    }
    float* orow = o + row_off(p.lo, s, h, t);
    float inv, lse_r;
    if (p.sink) {
        finish_row_sink(p.sink[h], m, l, inv, lse_r);
    } else {
        inv = l > 0.f ? 1.f / l : 0.f;
        lse_r = l > 0.f ? (m + log2f(l)) * kLn2 : -__builtin_huge_valf();
    }
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    lse[l_off(p, s, h, t)] = lse_r;
}

template <int D>
__global__ __launch_bounds__(128) void dq_f32_kernel(Problem p, const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     const float* __restrict__ dO,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ delta,
                                                     const int* __restrict__ idx,
                                                     float* __restrict__ dq, int64_t nrows) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= nrows) return;
    int z, h, t;
    decode_qrow(p, r, p.Hq, z, h, t, p.T);
    const Seq s = seq_of(p, z);
    if (t < 0 || t >= s.len) return;
    const int hkv = h / p.G, NBz = (s.klen + p.bs - 1) / p.bs, tp = t + s.qoff;
    const int* row = idx_row(p, s, idx, hkv, t);
    const int64_t lo = l_off(p, s, h, t);
    const float* qr = q + row_off(p.lq, s, h, t);
    const float* dr = dO + row_off(p.ldo, s, h, t);
    float qv[D], dov[D], acc[D];
    for (int d = 0; d < D; ++d) {
        qv[d] = qr[d] * p.scale_log2;
        dov[d] = dr[d];
        acc[d] = 0.f;
    }
    const float lse2 = lse[lo] * kLog2e, dl = delta[lo];
    for (int si = 0; si < p.S; ++si) {
        const int u = row[si];
        if (!slot_valid(row, si, u, NBz, p.bs, tp)) continue;
        const int j1 = min((u + 1) * p.bs, tp + 1);
        // Sliding window: keys tp - window < j only.
        const int j0 = p.window > 0 ? max(u * p.bs, tp - p.window + 1) : u * p.bs;
        for (int j = j0; j < j1; ++j) {
            const float* kr = k + row_off(p.lk, s, hkv, j);
            const float* vr = v + row_off(p.lv, s, hkv, j);
            float x = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
                x += qv[d] * kr[d];
                dp += dov[d] * vr[d];
            }
            const float ds = exp2f(x - lse2) * (dp - dl);
            for (int d = 0; d < D; ++d) acc[d] += ds * kr[d];
        }
    }
    float* dqr = dq + row_off(p.ldq, s, h, t);
    for (int d = 0; d < D; ++d) dqr[d] = acc[d] * p.scale;
}

// One thread per key (z, hkv, j): its block's inverted list gives the rows.
template <int D>
__global__ __launch_bounds__(128) void dkdv_f32_kernel(
    Problem p, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ offsets,
    const int* __restrict__ tokens, float* __restrict__ dk, float* __restrict__ dv,
    int64_t nkeys) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= nkeys) return;
    int z, hkv, j;
    decode_qrow(p, r, p.Hkv, z, hkv, j, p.Tk);
    const Seq s = seq_of(p, z);
    if (j < 0 || j >= s.klen) return;
    const int u = j / p.bs;
    const int zh = z * p.Hkv + hkv;
    const int* off = offsets + (int64_t)zh * (p.NBmax + 1);
    const int* list = tokens + region_base(p, s, hkv) + off[u];
    const int cnt = off[u + 1] - off[u];
    const float* kr = k + row_off(p.lk, s, hkv, j);
    const float* vr = v + row_off(p.lv, s, hkv, j);
    float kv[D], vv[D], ak[D], av[D];
    for (int d = 0; d < D; ++d) {
        kv[d] = kr[d] * p.scale_log2;
        vv[d] = vr[d];
        ak[d] = 0.f;
        av[d] = 0.f;
    }
    for (int e = 0; e < cnt; ++e) {
        const int t = list[e], tp = t + s.qoff;
        if (j > tp || (p.window > 0 && tp - p.window >= j)) continue;
        for (int gg = 0; gg < p.G; ++gg) {
            const int h = hkv * p.G + gg;
            const int64_t lo = l_off(p, s, h, t);
            const float* qr = q + row_off(p.lq, s, h, t);
            const float* dr = dO + row_off(p.ldo, s, h, t);
            float x = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
                x += qr[d] * kv[d];
                dp += dr[d] * vv[d];
            }
            const float P = exp2f(x - lse[lo] * kLog2e);
            const float ds = P * (dp - delta[lo]);
            for (int d = 0; d < D; ++d) {
                ak[d] += ds * qr[d];
                av[d] += P * dr[d];
            }
        }
    }
    float* dkr = dk + row_off(p.ldk, s, hkv, j);
    float* dvr = dv + row_off(p.ldv, s, hkv, j);
    for (int d = 0; d < D; ++d) {
        dkr[d] = ak[d] * p.scale;
        dvr[d] = av[d];
    }
}

#define NSA_DISPATCH_D_F32(D_, CALL)                          \
    do {                                                      \
        switch (D_) {                                         \
            case 16: { constexpr int D = 16; CALL; break; }   \
            case 32: { constexpr int D = 32; CALL; break; }   \
            case 64: { constexpr int D = 64; CALL; break; }   \
            case 128: { constexpr int D = 128; CALL; break; } \
            default: return hipErrorInvalidValue;             \
        }                                                     \
    } while (0)

hipError_t launch_fwd_f32(const HostProblem& hp, const float* q, const float* k, const float* v,
                          const int* block_idx, float* o, float* lse, hipStream_t st) {
    const int64_t n = hp.rows;
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)((n + 127) / 128));
    NSA_DISPATCH_D_F32(hp.dev.D, hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, dim3(128), 0, st,
                                                    hp.dev, q, k, v, block_idx, o, lse, n));
    return hipGetLastError();
}

hipError_t launch_dq_f32(const HostProblem& hp, const float* q, const float* k, const float* v,
                         const float* dO, const float* lse, const float* delta,
                         const int* block_idx, float* dq, hipStream_t st) {
    const int64_t n = hp.rows;
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)((n + 127) / 128));
    NSA_DISPATCH_D_F32(hp.dev.D, hipLaunchKernelGGL((dq_f32_kernel<D>), grid, dim3(128), 0, st,
                                                    hp.dev, q, k, v, dO, lse, delta, block_idx,
                                                    dq, n));
    return hipGetLastError();
}

hipError_t launch_dkdv_f32(const HostProblem& hp, const float* q, const float* k, const float* v,
                           const float* dO, const float* lse, const float* delta,
                           const BwdWorkspace& ws, float* dk, float* dv, hipStream_t st) {
    // keys: [B, Hkv, Tk] (dense) or [Ttot, Hkv] (packed, Tk = T)
    const int64_t n = (int64_t)hp.dev.B * hp.dev.Hkv * hp.dev.Tk;
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)((n + 127) / 128));
    NSA_DISPATCH_D_F32(hp.dev.D, hipLaunchKernelGGL((dkdv_f32_kernel<D>), grid, dim3(128), 0, st,
                                                    hp.dev, q, k, v, dO, lse, delta, ws.offsets,
                                                    ws.tokens, dk, dv, n));
    return hipGetLastError();
}

}  // namespace nsa
