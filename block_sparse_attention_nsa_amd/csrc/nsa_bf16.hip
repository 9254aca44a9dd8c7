// nsa_bf16.hip -- key-major bf16 matrix-core (MFMA 16x16x32) kernels for
// gfx950 (the query-major forward and dQ kernels are in nsa_query.hip):
//
//   dkdv  one workgroup = one key block u (BS/16 waves x 16 keys) and one chunk
//         of its inverted query-row list; rows (token, head) are staged 32 at a
//         time in LDS and shared by the waves: S = Q K^T, dP = dO V^T,
//         dV += P^T dO, dK += dS^T Q.  A list longer than one chunk writes fp32
//         partials that dkdv_reduce sums in chunk order (deterministic).
//
// Method: page 1 of the reference text (NSA selection gradcheck gate) defines
// the call and its gradients; the forward/backward formulas are the plain
// masked softmax and its exact gradient, as stated in include/nsa_sel.h.
#include "nsa_internal.h"

namespace nsa {

#ifndef NSA_DKDV_WAVES_PER_EU
#define NSA_DKDV_WAVES_PER_EU 2
#endif
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ bf16x8 pack_operand(const float (&lo)[4], const float (&hi)[4]) {
    return as_bf16x8(make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
struct ItemRef {
    int zh, u, kitem, nitems;
};

// Work item b -> (z*Hkv + hkv, block u, chunk k) by binary search over the
// prefixes the planner wrote.  Returns false past the last item.
__device__ __forceinline__ bool find_item(int b, int ZH, int NB, const int* __restrict__ zh_base,
                                          const int* __restrict__ item_pre, ItemRef& it) {
    if (b >= zh_base[ZH]) return false;
    int lo = 0, hi = ZH;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (zh_base[mid] <= b) lo = mid; else hi = mid;
    }
    it.zh = lo;
    const int local = b - zh_base[lo];
    const int* ip = item_pre + (int64_t)lo * (NB + 1);
    lo = 0;
    hi = NB;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (ip[mid] <= local) lo = mid; else hi = mid;
    }
    it.u = lo;
    it.kitem = local - ip[lo];
    it.nitems = ip[lo + 1] - ip[lo];
    return true;
}

// Rows of one 32-row step: staged Q and dO (row-major, padded rows) plus the
// per-row token, lse*log2(e) and Delta (16-byte aligned for vector reads).
template <int D>
struct RowTile {
    static constexpr int kStride = D + 8;
    uint16_t q[32 * kStride];
    uint16_t dO[32 * kStride];
    __attribute__((aligned(16))) int t[32];
    __attribute__((aligned(16))) float nlse2[32];
    __attribute__((aligned(16))) float dl[32];
};

// Position in the flattened (entry, head) row list, advanced 32 rows at a
// time without dividing: row f = e * G + h.
struct RowPos {
    int e, h;
};
__device__ __forceinline__ void advance32(RowPos& rp, int G, int q32, int r32) {
    rp.h += r32;
    rp.e += q32;
    if (rp.h >= G) {
        rp.h -= G;
        ++rp.e;
    }
}

// This thread's share of one step: CH 16-byte chunks of Q and dO (chunk
// c = i*NT + tid is row c / QCH, columns 8 * (c % QCH)), and for threads < 32
// the metadata of row tid.
template <int D, int NT>
struct StepShare {
    static constexpr int QCH = D / 8;
    static constexpr int CH = (32 * QCH + NT - 1) / NT;
};

template <int D, int NT>
struct TokRegs {
    int t[StepShare<D, NT>::CH], h[StepShare<D, NT>::CH];
    int tm, hm;
};

template <int D, int NT>
struct RowRegs {
    uint4 q[StepShare<D, NT>::CH], d[StepShare<D, NT>::CH];
    int t;
    float nlse2, dl;
};

template <int D, int BS>
__global__ __launch_bounds__(BS / 16 * 64) __attribute__((amdgpu_waves_per_eu(NSA_DKDV_WAVES_PER_EU, 8)))
void dkdv_bf16_kernel(
    Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ offsets,
    const int* __restrict__ tokens, const int* __restrict__ item_pre,
    const int* __restrict__ pslot_pre, const int* __restrict__ zh_base, int CR,
    float* __restrict__ partials, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int NW = BS / 16, NT = NW * 64, KD = D / 32, ND = D / 16;
    constexpr int QST = RowTile<D>::kStride, QCH = StepShare<D, NT>::QCH, CH = StepShare<D, NT>::CH;
    __shared__ RowTile<D> tiles[2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r = lane & 15;
    const int ZH = p.Z * p.Hkv, NB = p.NBmax, G = p.G;
    ItemRef it;
    if (!find_item(blockIdx.x, ZH, NB, zh_base, item_pre, it)) return;
    const int z = it.zh / p.Hkv, hkv = it.zh % p.Hkv, u = it.u;
    const Seq s = seq_of(p, z);
    const int* off = offsets + (int64_t)it.zh * (NB + 1);
    const int* list = tokens + region_base(p, s, hkv) + off[u];
    const int R = (off[u + 1] - off[u]) * G;
    const int f_begin = it.kitem * CR, f_end = min(R, f_begin + CR);
    const int q32 = 32 / G, r32 = 32 % G;

    // Row bases: q/dO of this (z, group) and lse/Delta; 32-bit offsets below.
    const int qsh = (int)s.q_sh, qst = (int)s.q_st;
    const uint16_t* qb = q + s.q_base + (int64_t)(hkv * G) * s.q_sh;
    const uint16_t* db = dO + s.q_base + (int64_t)(hkv * G) * s.q_sh;
    const float* lb = lse + s.l_base + (int64_t)(hkv * G) * p.T;
    const float* deb = delta + s.l_base + (int64_t)(hkv * G) * p.T;

    // Fetch cursors of this thread's chunk rows and of its metadata row.
    RowPos fp[CH], fm;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int f = f_begin + (i * NT + tid) / QCH;
        fp[i].e = f / G;
        fp[i].h = f % G;
    }
    fm.e = (f_begin + tid) / G;
    fm.h = (f_begin + tid) % G;

    // Token ids of the step at f0 (the cursors point at it; advanced after).
    auto fetch = [&](int f0, TokRegs<D, NT>& tk) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = i * NT + tid;
            const bool ok = c < 32 * QCH && f0 + c / QCH < f_end;
            tk.t[i] = ok ? list[fp[i].e] : -1;
            tk.h[i] = fp[i].h;
            advance32(fp[i], G, q32, r32);
        }
        tk.tm = (tid < 32 && f0 + tid < f_end) ? list[fm.e] : -1;
        tk.hm = fm.h;
        advance32(fm, G, q32, r32);
    };
    auto load = [&](const TokRegs<D, NT>& tk, RowRegs<D, NT>& rr) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int o_ = tk.h[i] * qsh + tk.t[i] * qst + 8 * ((i * NT + tid) % QCH);
            rr.q[i] = make_uint4(0, 0, 0, 0);
            rr.d[i] = make_uint4(0, 0, 0, 0);
            if (tk.t[i] >= 0) {
                rr.q[i] = ldg16(qb + o_);
                rr.d[i] = ldg16(db + o_);
            }
        }
        rr.t = tk.tm;
        rr.nlse2 = 0.f;
        rr.dl = 0.f;
        if (tk.tm >= 0) {
            const int lo_ = tk.hm * p.T + tk.tm;
            rr.nlse2 = -lb[lo_] * kLog2e;
            rr.dl = deb[lo_];
        }
    };
    auto store = [&](const RowRegs<D, NT>& rr, RowTile<D>& tile) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = i * NT + tid;
            if (c < 32 * QCH) {
                const int row = c / QCH, dc = c % QCH;
                *reinterpret_cast<uint4*>(tile.q + row * QST + 8 * dc) = rr.q[i];
                *reinterpret_cast<uint4*>(tile.dO + row * QST + 8 * dc) = rr.d[i];
            }
        }
        if (tid < 32) {
            tile.t[tid] = rr.t;
            tile.nlse2[tid] = rr.nlse2;
            tile.dl[tid] = rr.dl;
        }
    };

    // Pipeline: token ids three steps ahead, rows two steps ahead (two
    // alternating register sets), LDS double-buffered.
    TokRegs<D, NT> tk;
    RowRegs<D, NT> ra, rb;
    fetch(f_begin, tk);
    load(tk, ra);
    fetch(f_begin + 32, tk);
    load(tk, rb);
    fetch(f_begin + 64, tk);

    const int kw0 = u * BS + 16 * w;  // this wave's 16 keys
    const int jk = kw0 + r;
    bf16x8 kf[KD], vf[KD];
    {
        const bool in = jk < s.len;
        const int64_t ko = k_off(s, hkv, in ? jk : 0);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            kf[kk] = in ? as_bf16x8(ldg16(k + ko + 32 * kk + 8 * g)) : zero_bf16x8();
            vf[kk] = in ? as_bf16x8(ldg16(v + ko + 32 * kk + 8 * g)) : zero_bf16x8();
        }
    }
    f32x4 dka[ND], dva[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
        dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    store(ra, tiles[0]);
    __syncthreads();
    const float c2 = p.scale_log2;

    // One 32-row step: issue the loads two steps ahead into `next2`, compute
    // from LDS buffer `buf`, then move `next1` (loaded a step earlier) into
    // the other buffer.
    auto step = [&](int f0, RowTile<D>& tl, RowTile<D>& tn, RowRegs<D, NT>& next2,
                    RowRegs<D, NT>& next1) {
        if (f0 + 64 < f_end) load(tk, next2);
        if (f0 + 96 < f_end) fetch(f0 + 96, tk);
        f32x4 sc[2], dp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            sc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                const bf16x8 qa = as_bf16x8(*reinterpret_cast<const uint4*>(tl.q + (16 * rt + r) * QST + 32 * kk + 8 * g));
                const bf16x8 da = as_bf16x8(*reinterpret_cast<const uint4*>(tl.dO + (16 * rt + r) * QST + 32 * kk + 8 * g));
                sc[rt] = mfma(qa, kf[kk], sc[rt]);
                dp[rt] = mfma(da, vf[kk], dp[rt]);
            }
        }
        float pv[2][4], dsv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int4 tt = *reinterpret_cast<const int4*>(tl.t + 16 * rt + 4 * g);
            const float4 nl = *reinterpret_cast<const float4*>(tl.nlse2 + 16 * rt + 4 * g);
            const float4 dd = *reinterpret_cast<const float4*>(tl.dl + 16 * rt + 4 * g);
            const int tv[4] = {tt.x, tt.y, tt.z, tt.w};
            const float nv[4] = {nl.x, nl.y, nl.z, nl.w};
            const float dv_[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float P = jk <= tv[i] ? fast_exp2(fmaf(sc[rt][i], c2, nv[i])) : 0.f;
                pv[rt][i] = P;
                dsv[rt][i] = P * (dp[rt][i] - dv_[i]);
            }
        }
        const bf16x8 pa = pack_operand(pv[0], pv[1]);
        const bf16x8 dsa = pack_operand(dsv[0], dsv[1]);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const bf16x8 dob = lds_col_operand(tl.dO, QST, 0, 16, 16 * dt, lane);
            dva[dt] = mfma(pa, dob, dva[dt]);
            const bf16x8 qb_ = lds_col_operand(tl.q, QST, 0, 16, 16 * dt, lane);
            dka[dt] = mfma(dsa, qb_, dka[dt]);
        }
        if (f0 + 32 < f_end) store(next1, tn);
        __syncthreads();
    };
    for (int f0 = f_begin; f0 < f_end; f0 += 64) {
        step(f0, tiles[0], tiles[1], ra, rb);
        if (f0 + 32 < f_end) step(f0 + 32, tiles[1], tiles[0], rb, ra);
    }
    // dK/dV lanes: key kw0 + 4g + i, column 16dt + r.
    if (it.nitems == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kw0 + 4 * g + i;
            if (key >= s.len) continue;
            const int64_t ko = k_off(s, hkv, key);
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                dk[ko + 16 * dt + r] = f32_to_bf16(dka[dt][i] * p.scale);
                dv[ko + 16 * dt + r] = f32_to_bf16(dva[dt][i]);
            }
        }
    } else {
        const int slot = zh_base[ZH + 1 + it.zh] + pslot_pre[(int64_t)it.zh * (NB + 1) + u] + it.kitem;
        float* pk = partials + (int64_t)slot * 2 * BS * D;
        float* pvv = pk + BS * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kl = 16 * w + 4 * g + i;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                pk[kl * D + 16 * dt + r] = dka[dt][i];
                pvv[kl * D + 16 * dt + r] = dva[dt][i];
            }
        }
    }
}

// Sums the fp32 partials of split lists in chunk order and writes zeros for
// blocks no row attends to.  Blocks handled whole by one item are skipped.
// Each thread owns 4 consecutive outputs; the chunk loads are issued four at
// a time but added strictly in chunk order (deterministic).
template <int D, int BS>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(
    Problem p, const int* __restrict__ item_pre, const int* __restrict__ pslot_pre,
    const int* __restrict__ zh_base, const float* __restrict__ partials,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int E4 = BS * D / 4;  // float4 per plane (dk or dv) of one block
    const int NB = p.NBmax, ZH = p.Z * p.Hkv;
    const int zh = blockIdx.x / NB, u = blockIdx.x % NB;
    const int z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    if (u * BS >= s.len) return;
    const int* ip = item_pre + (int64_t)zh * (NB + 1);
    const int n = ip[u + 1] - ip[u];
    if (n == 1) return;
    const int slot0 = n > 1 ? zh_base[ZH + 1 + zh] + pslot_pre[(int64_t)zh * (NB + 1) + u] : 0;
    const float4* part = reinterpret_cast<const float4*>(partials) + (int64_t)slot0 * 2 * E4;
    for (int e4 = threadIdx.x; e4 < 2 * E4; e4 += blockDim.x) {
        const int plane = e4 / E4, el = (e4 % E4) * 4;
        const int kl = el / D, d = el % D, key = u * BS + kl;
        if (key >= s.len) continue;
        const float4* src = part + e4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int kk = 0;
        for (; kk + 4 <= n; kk += 4) {
            const float4 x0 = src[(int64_t)(kk + 0) * 2 * E4];
            const float4 x1 = src[(int64_t)(kk + 1) * 2 * E4];
            const float4 x2 = src[(int64_t)(kk + 2) * 2 * E4];
            const float4 x3 = src[(int64_t)(kk + 3) * 2 * E4];
            acc.x += x0.x; acc.y += x0.y; acc.z += x0.z; acc.w += x0.w;
            acc.x += x1.x; acc.y += x1.y; acc.z += x1.z; acc.w += x1.w;
            acc.x += x2.x; acc.y += x2.y; acc.z += x2.z; acc.w += x2.w;
            acc.x += x3.x; acc.y += x3.y; acc.z += x3.z; acc.w += x3.w;
        }
        for (; kk < n; ++kk) {
            const float4 x = src[(int64_t)kk * 2 * E4];
            acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
        }
        const float m = plane == 0 ? p.scale : 1.f;
        const uint2 pk = make_uint2(pack_bf16x2(acc.x * m, acc.y * m), pack_bf16x2(acc.z * m, acc.w * m));
        uint16_t* dst = (plane == 0 ? dk : dv) + k_off(s, hkv, key) + d;
        *reinterpret_cast<uint2*>(dst) = pk;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define NSA_DISPATCH_D_BS(D_, BS_, CALL)                                                   \
    do {                                                                                  \
        if ((D_) == 32 && (BS_) == 32) { constexpr int D = 32, BS = 32; CALL; }           \
        else if ((D_) == 32 && (BS_) == 64) { constexpr int D = 32, BS = 64; CALL; }      \
        else if ((D_) == 32 && (BS_) == 128) { constexpr int D = 32, BS = 128; CALL; }    \
        else if ((D_) == 64 && (BS_) == 32) { constexpr int D = 64, BS = 32; CALL; }      \
        else if ((D_) == 64 && (BS_) == 64) { constexpr int D = 64, BS = 64; CALL; }      \
        else if ((D_) == 64 && (BS_) == 128) { constexpr int D = 64, BS = 128; CALL; }    \
        else if ((D_) == 128 && (BS_) == 32) { constexpr int D = 128, BS = 32; CALL; }    \
        else if ((D_) == 128 && (BS_) == 64) { constexpr int D = 128, BS = 64; CALL; }    \
        else if ((D_) == 128 && (BS_) == 128) { constexpr int D = 128, BS = 128; CALL; }  \
        else return hipErrorInvalidValue;                                                 \
    } while (0)

hipError_t launch_dkdv_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                            const void* dO, const float* lse, const float* delta,
                            const BwdWorkspace& ws, void* dk, void* dv, hipStream_t st) {
    if (hp.ZH == 0) return hipSuccess;
    const unsigned items = (unsigned)hp.items_ub;
    const unsigned nred = (unsigned)((int64_t)hp.ZH * hp.dev.NBmax);
    if (items) {
        NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                          hipLaunchKernelGGL((dkdv_bf16_kernel<D, BS>), dim3(items), dim3(BS / 16 * 64),
                                             0, st, hp.dev, (const uint16_t*)q, (const uint16_t*)k,
                                             (const uint16_t*)v, (const uint16_t*)dO, lse, delta,
                                             ws.offsets, ws.tokens, ws.item_pre, ws.pslot_pre,
                                             ws.zh_base, hp.CR, ws.partials, (uint16_t*)dk,
                                             (uint16_t*)dv));
    }
    if (nred) {
        NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                          hipLaunchKernelGGL((dkdv_reduce_kernel<D, BS>), dim3(nred), dim3(256), 0,
                                             st, hp.dev, ws.item_pre, ws.pslot_pre, ws.zh_base,
                                             ws.partials, (uint16_t*)dk, (uint16_t*)dv));
    }
    return hipGetLastError();
}

}  // namespace nsa
