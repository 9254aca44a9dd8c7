// nsa_dkdv.hip -- key-major dK / dV for bf16 on gfx950 matrix cores
// (v_mfma_f32_16x16x32_bf16).
//
// One workgroup = one key block u (BS keys, KPW of them per wave) and one
// chunk of the block's inverted list of query rows (token, head).  The
// rows are taken 32 at a time, newest token first, and copied from HBM
// straight into a three-stage LDS ring by buffer loads that write LDS (no
// register staging), two steps ahead of their use.  Every wave reads the
// shared tile:
//     S = Q K^T,  dP = dO V^T              (K, V of the wave's keys in VGPRs)
//     P = exp(S*scale - lse) (causal),  dS = P (dP - Delta)
//     dV^T += dO^T P,  dK^T += Q^T dS      (accumulated transposed)
// A list longer than one chunk writes fp32 partials that dkdv_reduce sums in
// chunk order, so the result does not depend on scheduling.
//
// Scheduling: work items are dealt out so that consecutive items (the blocks
// of one (batch, kv-head) group) run on one XCD; as all of them walk their
// row lists from the newest token down, the groups that share rows read them
// at about the same time and mostly from that XCD's L2.
//
// Method: page 1 of the reference text (NSA selection gradcheck gate) defines
// the call and its gradients; the backward formulas are the exact gradient of
// the masked softmax attention, as stated in include/nsa_sel.h.
#include "nsa_internal.h"

namespace nsa {

namespace {

// One stage of the row ring: the Q and dO tiles of 32 rows (RowTile layout)
// and their per-row token, lse and Delta.
template <int D>
struct alignas(16) Stage {
    uint16_t q[32 * D];
    uint16_t dO[32 * D];
    int t[32];
    float lse[32];
    float dl[32];
};

struct ItemRef {
    int zh, u, kitem, nitems;
};

// Work item b -> (z*Hkv + hkv, block u, chunk k) by binary search over the
// prefixes the planner wrote.
__device__ __forceinline__ void find_item(int b, int ZH, int NB, const int* __restrict__ zh_base,
                                          const int* __restrict__ item_pre, ItemRef& it) {
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
}

// Cursor over the flattened row list (row f = e * G + h), walked downwards 32
// rows at a time without dividing.  hoff = h * (byte stride of a head).
struct Cursor {
    int f, e, h;
    uint32_t hoff;
};

__device__ __forceinline__ Cursor cursor_at(int f, int G, uint32_t hstride) {
    Cursor c;
    c.f = f;
    const int ff = max(f, 0);
    c.e = ff / G;
    c.h = ff - c.e * G;
    c.hoff = (uint32_t)c.h * hstride;
    return c;
}

// Moves the cursor 32 rows down: q32 = 32 / G, r32 = 32 % G.
__device__ __forceinline__ void retreat32(Cursor& c, int G, int q32, int r32, uint32_t r32_stride,
                                          uint32_t G_stride) {
    c.f -= 32;
    c.h -= r32;
    c.e -= q32;
    c.hoff -= r32_stride;
    if (c.h < 0) {
        c.h += G;
        c.e -= 1;
        c.hoff += G_stride;
    }
}

__device__ __forceinline__ bf16x8 pack8(const float (&lo)[4], const float (&hi)[4]) {
    return as_bf16x8(make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
}

}  // namespace

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// Keys per wave: 16 keeps a wave within 256 registers (two or more waves per
// SIMD hide each other's LDS and load latency) at twice the LDS operand reads
// per matrix op of 32 keys per wave (one wave per SIMD).
#ifndef NSA_DKDV_KPW
#define NSA_DKDV_KPW 16
#endif
constexpr int kDkdvKpw = NSA_DKDV_KPW;
static_assert(kDkdvKpw == 16 || kDkdvKpw == 32, "keys per wave");

template <int D, int BS, int KPW>
__global__ __launch_bounds__(BS / KPW * 64)
__attribute__((amdgpu_waves_per_eu(KPW == 16 ? 2 : 1, KPW == 16 ? 8 : 1)))
void dkdv_kernel(Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
                 const float* __restrict__ lse, const float* __restrict__ delta,
                 const int* __restrict__ offsets, const int* __restrict__ tokens,
                 const int* __restrict__ item_pre, const int* __restrict__ pslot_pre,
                 const int* __restrict__ zh_base, int CR, float* __restrict__ partials,
                 uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    using L = RowTile<D>;
    constexpr int NW = BS / KPW, NT = KPW / 16, KD = D / 32, ND = D / 16, QCH = L::QCH, NI = L::NI;
    constexpr int NJ = (NI + NW - 1) / NW;  // 1 KB row loads per tile for each wave (at most)
    __shared__ Stage<D> st0, st1, st2;
    __shared__ __attribute__((aligned(16))) int tk0[32], tk1[32], tk2[32];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r = lane & 15;
    const int ZH = p.Z * p.Hkv, NB = p.NBmax, G = p.G;
    const int n_items = zh_base[ZH];
    if ((int)blockIdx.x >= n_items) return;
    ItemRef it;
    find_item(xcd_remap(blockIdx.x, n_items), ZH, NB, zh_base, item_pre, it);
    const int z = it.zh / p.Hkv, hkv = it.zh % p.Hkv, u = it.u;
    const Seq s = seq_of(p, z);
    const int* off = offsets + (int64_t)it.zh * (NB + 1);
    const int* list = tokens + region_base(p, s, hkv) + off[u];
    const int R = (off[u + 1] - off[u]) * G;
    const int f_begin = it.kitem * CR, f_end = min(R, f_begin + CR);
    const int nsteps = (f_end - f_begin + 31) / 32;

    // Buffers of this (z, kv group): rows (h, t) of q / dO and lse / Delta.
    // Every valid row lies below the sizes; invalid rows use an offset past
    // them and load zeros.
    const uint16_t* qb = q + s.q_base + (int64_t)(hkv * G) * s.q_sh;
    const uint16_t* db = dO + s.q_base + (int64_t)(hkv * G) * s.q_sh;
    const int64_t q_elems = (int64_t)(G - 1) * s.q_sh + (int64_t)(s.len - 1) * s.q_st + D;
    const buf_rsrc rq = make_rsrc(qb, (uint32_t)(2 * q_elems));
    const buf_rsrc rd = make_rsrc(db, (uint32_t)(2 * q_elems));
    const int64_t l_first = s.l_base + (int64_t)(hkv * G) * p.T;
    const uint32_t l_bytes = (uint32_t)(4 * ((int64_t)(G - 1) * p.T + s.len));
    const buf_rsrc rl = make_rsrc(lse + l_first, l_bytes);
    const buf_rsrc rdl = make_rsrc(delta + l_first, l_bytes);
    constexpr uint32_t kOob = 0xFFFFFFF0u;
    const uint32_t qsh_b = (uint32_t)(2 * s.q_sh), qst_b = (uint32_t)(2 * s.q_st);
    const uint32_t lsh_b = (uint32_t)(4 * p.T);
    const int q32 = 32 / G, r32 = 32 % G;
    const uint32_t q_r32 = (uint32_t)r32 * qsh_b, q_G = (uint32_t)G * qsh_b;
    const uint32_t l_r32 = (uint32_t)r32 * lsh_b, l_G = (uint32_t)G * lsh_b;

    // Rows this lane loads: 1 KB load jj = w + NW * j of a tile covers the
    // 16-byte positions 64 jj + lane, i.e. row (64 jj + lane) / QCH at some
    // LDS slot, which holds data chunk chunk(row, slot) of that row.
    Cursor cq[NJ];
    int qrow[NJ];
    uint32_t cofs[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int jj = min(w + NW * j, NI - 1);
        const int pos = 64 * jj + lane;
        qrow[j] = pos / QCH;
        cofs[j] = 16u * (uint32_t)L::chunk(qrow[j], pos % QCH);
        cq[j] = cursor_at(f_end - 32 + qrow[j], G, qsh_b);
    }
    // Wave 0, lanes < 32: row `lane` of each step, once for the token list
    // (one step ahead of the rows) and once for lse / Delta.
    const int mrow = lane & 31;
    const bool meta = w == 0 && lane < 32;
    Cursor ct = cursor_at(f_end - 32 + mrow, G, 0u);
    Cursor cm = cursor_at(f_end - 32 + mrow, G, lsh_b);
    const buf_rsrc rt = make_rsrc(list, (uint32_t)(4 * (R / G)));

    // (A) token ids of a step into its ring slot: list[e] of every row.
    auto tok_dma = [&](int* slot_t) {
        if (meta) dma4(rt, slot_t, ct.f >= f_begin ? 4u * (uint32_t)ct.e : kOob);
        retreat32(ct, G, q32, r32, 0u, 0u);
    };
    // (B) the rows of a step into stage `sg`, with token ids from `slot_t`
    // (written by an earlier tok_dma that has completed): Q and dO rows,
    // then the row token (-1 for rows past the chunk), lse and Delta.
    auto row_dma = [&](const int* slot_t, Stage<D>& sg) {
        int tj[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) tj[j] = slot_t[qrow[j]];
        const int tm = slot_t[mrow];
        if (meta) sg.t[lane] = cm.f >= f_begin ? tm : -1;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int jj = w + NW * j;
            if (jj < NI) {
                const uint32_t vo = cq[j].f >= f_begin
                                        ? cq[j].hoff + (uint32_t)tj[j] * qst_b + cofs[j] : kOob;
                dma16(rq, reinterpret_cast<uint8_t*>(sg.q) + 1024 * jj, vo);
                dma16(rd, reinterpret_cast<uint8_t*>(sg.dO) + 1024 * jj, vo);
            }
            retreat32(cq[j], G, q32, r32, q_r32, q_G);
        }
        if (meta) {
            const uint32_t lo = cm.f >= f_begin ? cm.hoff + 4u * (uint32_t)tm : kOob;
            dma4(rl, sg.lse, lo);
            dma4(rdl, sg.dl, lo);
        }
        retreat32(cm, G, q32, r32, l_r32, l_G);
    };

    // K and V of this wave's KPW keys as MFMA B operands: kf[kt][kk] holds
    // K[key 16kt + r][32kk + 8g .. + 7].
    const int kbase = u * BS + KPW * w;
    bf16x8 kf[NT][KD], vf[NT][KD];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
        const int key = kbase + 16 * kt + r;
        const bool in = key < s.len;
        const int64_t ko = k_off(s, hkv, in ? key : 0);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            kf[kt][kk] = in ? as_bf16x8(ldg16(k + ko + 32 * kk + 8 * g)) : as_bf16x8(make_uint4(0, 0, 0, 0));
            vf[kt][kk] = in ? as_bf16x8(ldg16(v + ko + 32 * kk + 8 * g)) : as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }

    // LDS byte offsets inside a tile of this lane's operand reads (rows 16..
    // of a tile sit 16 RB bytes further).
    uint32_t a_off[KD], t_off[ND];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) a_off[kk] = L::a_off(lane, kk);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) t_off[dt] = L::t_off(lane, dt);

    f32x4 dkt[NT][ND], dvt[NT][ND];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            dkt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dvt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    const float c2 = p.scale_log2;

    // One step on a staged tile, in phases the compiler may not interleave
    // (so every operand read gets a register of its own and is in flight
    // well before its use): (1) all reads of S / dP operands and of the row
    // metadata, (2) S and dP, (3) all transposed reads of Q and dO, (4) P and
    // dS, (5) dV^T and dK^T.
    auto compute = [&](const Stage<D>& sg) {
        const uint8_t* tq = reinterpret_cast<const uint8_t*>(sg.q);
        const uint8_t* td = reinterpret_cast<const uint8_t*>(sg.dO);
        bf16x8 qa[KD][2], da[KD][2];
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                qa[kk][rt] = *reinterpret_cast<const bf16x8*>(tq + a_off[kk] + rt * 16 * L::RB);
                da[kk][rt] = *reinterpret_cast<const bf16x8*>(td + a_off[kk] + rt * 16 * L::RB);
            }
        int4 tt[2];
        float4 ll[2], dd[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            tt[rt] = *reinterpret_cast<const int4*>(sg.t + 16 * rt + 4 * g);
            ll[rt] = *reinterpret_cast<const float4*>(sg.lse + 16 * rt + 4 * g);
            dd[rt] = *reinterpret_cast<const float4*>(sg.dl + 16 * rt + 4 * g);
        }
        __builtin_amdgcn_sched_barrier(0);

        f32x4 sc[2][NT], dp[2][NT];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                sc[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                dp[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int kt = 0; kt < NT; ++kt) {
                    sc[rt][kt] = mfma(qa[kk][rt], kf[kt][kk], sc[rt][kt]);
                    dp[rt][kt] = mfma(da[kk][rt], vf[kt][kk], dp[rt][kt]);
                }
        __builtin_amdgcn_sched_barrier(0);

        // Transposed operands: the contraction rows are 4g + e and 16 + 4g +
        // e, the rows the C layout of S gave this lane.
        bf16x8 dcol[ND], qcol[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint2 d0 = lds_read_tr(reinterpret_cast<const uint16_t*>(td + t_off[dt]));
            const uint2 d1 = lds_read_tr(reinterpret_cast<const uint16_t*>(td + t_off[dt] + 16 * L::RB));
            const uint2 q0 = lds_read_tr(reinterpret_cast<const uint16_t*>(tq + t_off[dt]));
            const uint2 q1 = lds_read_tr(reinterpret_cast<const uint16_t*>(tq + t_off[dt] + 16 * L::RB));
            dcol[dt] = __builtin_bit_cast(bf16x8, make_uint4(d0.x, d0.y, d1.x, d1.y));
            qcol[dt] = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
        }
        __builtin_amdgcn_sched_barrier(0);

        // P and dS for rows 16rt + 4g + i, keys kbase + 16kt + r.  The
        // exponential is taken for every entry and masked by a select.
        float pv[NT][2][4], dsv[NT][2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int tv[4] = {tt[rt].x, tt[rt].y, tt[rt].z, tt[rt].w};
            const float nl[4] = {-ll[rt].x * kLog2e, -ll[rt].y * kLog2e, -ll[rt].z * kLog2e,
                                 -ll[rt].w * kLog2e};
            const float de[4] = {dd[rt].x, dd[rt].y, dd[rt].z, dd[rt].w};
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                const int key = kbase + 16 * kt + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = fast_exp2(fmaf(sc[rt][kt][i], c2, nl[i]));
                    const float P = key <= tv[i] ? e : 0.f;
                    pv[kt][rt][i] = P;
                    dsv[kt][rt][i] = P * (dp[rt][kt][i] - de[i]);
                }
            }
        }
        bf16x8 pb[NT], dsb[NT];
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            pb[kt] = pack8(pv[kt][0], pv[kt][1]);
            dsb[kt] = pack8(dsv[kt][0], dsv[kt][1]);
        }
        __builtin_amdgcn_sched_barrier(0);

        // dV^T[d][key] += sum_rows dO[row][d] P[row][key]; dK^T likewise with
        // Q and dS.
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                dvt[kt][dt] = mfma(dcol[dt], pb[kt], dvt[kt][dt]);
                dkt[kt][dt] = mfma(qcol[dt], dsb[kt], dkt[kt][dt]);
            }
    };

    // Loads a wave issues per step in (B): 2 per row load group (Q, dO), and
    // lse / Delta on wave 0.  The end-of-step wait lets these newest loads
    // stay in flight; everything older (the rows of the next step, the token
    // ids of the step after) is then complete.  A wave without a full share
    // of row loads waits for all of them.
    constexpr int kInFlight = 2 * NJ;
    const bool full_share = w + NW * (NJ - 1) < NI;
    auto end_wait = [&](bool ahead) {
        if (full_share && ahead) {
            if (w == 0) wait_vm_barrier<kInFlight + 2>(); else wait_vm_barrier<kInFlight>();
        } else {
            wait_vm_barrier<0>();
        }
    };

    // Prologue: token ids of steps 0..2, then the rows of steps 0 and 1.
    tok_dma(tk0);
    tok_dma(tk1);
    tok_dma(tk2);
    wait_vm_barrier<0>();
    row_dma(tk0, st0);
    row_dma(tk1, st1);
    end_wait(true);

    // Step i: (A) token ids of step i + 3 into slot (i + 3) % 3 (last read in
    // step i - 2), (B) rows of step i + 2 into stage (i + 2) % 3 (last read in
    // step i - 1), compute stage i % 3, wait, barrier.
    auto step = [&](int i, const Stage<D>& cur, Stage<D>& nxt2, int* tk_fill, const int* tk_next2) {
        if (i + 3 < nsteps) tok_dma(tk_fill);
        if (i + 2 < nsteps) row_dma(tk_next2, nxt2);
        compute(cur);
        end_wait(i + 2 < nsteps);
    };
    for (int i = 0; i < nsteps; i += 3) {
        step(i, st0, st2, tk0, tk2);
        if (i + 1 < nsteps) step(i + 1, st1, st0, tk1, tk0);
        if (i + 2 < nsteps) step(i + 2, st2, st1, tk2, tk1);
    }

    // Output: dvt[kt][dt][i] = dV[key kbase + 16kt + r][16dt + 4g + i].
    if (it.nitems == 1) {
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            const int key = kbase + 16 * kt + r;
            if (key >= s.len) continue;
            const int64_t ko = k_off(s, hkv, key);
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const f32x4 a = dkt[kt][dt], b = dvt[kt][dt];
                *reinterpret_cast<uint2*>(dk + ko + 16 * dt + 4 * g) =
                    make_uint2(pack_bf16x2(a[0] * p.scale, a[1] * p.scale),
                               pack_bf16x2(a[2] * p.scale, a[3] * p.scale));
                *reinterpret_cast<uint2*>(dv + ko + 16 * dt + 4 * g) =
                    make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
            }
        }
    } else {
        // Partial slot layout: [dk, dv][16-key tile of the block][dt][lane] x
        // 4 floats; this wave's tiles are NT w + kt.
        const int slot = zh_base[ZH + 1 + it.zh] + pslot_pre[(int64_t)it.zh * (NB + 1) + u] + it.kitem;
        f32x4* pk = reinterpret_cast<f32x4*>(partials + (int64_t)slot * 2 * BS * D);
        f32x4* pv_ = pk + BS * D / 4;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const int e = ((w * NT + kt) * ND + dt) * 64 + lane;
                pk[e] = dkt[kt][dt];
                pv_[e] = dvt[kt][dt];
            }
    }
}

// Sums the fp32 partials of split lists in chunk order and writes zeros for
// blocks no row attends to (blocks handled whole by one item are skipped).
// Thread e4 owns one float4 of the slot layout [plane][tile][dt][lane], i.e.
// dK or dV of key 16 tile + (lane & 15), columns 16 dt + 4
// (lane >> 4) .. + 3.  Chunk loads are issued four at a time but added
// strictly in chunk order.
template <int D, int BS>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(
    Problem p, const int* __restrict__ item_pre, const int* __restrict__ pslot_pre,
    const int* __restrict__ zh_base, const float* __restrict__ partials,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int ND = D / 16, E4 = BS * D / 4;  // float4 per plane of one block
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
        const int plane = e4 / E4, x = e4 % E4;
        const int ln = x % 64, dt = (x / 64) % ND, tile = x / (64 * ND);
        const int key = u * BS + 16 * tile + (ln & 15), d = 16 * dt + 4 * (ln >> 4);
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
            const float4 y = src[(int64_t)kk * 2 * E4];
            acc.x += y.x; acc.y += y.y; acc.z += y.z; acc.w += y.w;
        }
        const float m = plane == 0 ? p.scale : 1.f;
        const uint2 pk = make_uint2(pack_bf16x2(acc.x * m, acc.y * m), pack_bf16x2(acc.z * m, acc.w * m));
        uint16_t* dst = (plane == 0 ? dk : dv) + k_off(s, hkv, key) + d;
        *reinterpret_cast<uint2*>(dst) = pk;
    }
}

// ---------------------------------------------------------------------------
// launcher
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
                            const BwdWorkspace& ws, void* dk, void* dv, hipStream_t st,
                            int parts) {
    if (hp.ZH == 0) return hipSuccess;
    const unsigned items = (parts & kDkdvBlocks) ? (unsigned)hp.items_ub : 0u;
    const unsigned nred = (parts & kDkdvReduce) ? (unsigned)((int64_t)hp.ZH * hp.dev.NBmax) : 0u;
    if (items) {
        NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                          hipLaunchKernelGGL((dkdv_kernel<D, BS, kDkdvKpw>), dim3(items),
                                             dim3(BS / kDkdvKpw * 64), 0,
                                             st, hp.dev, (const uint16_t*)q, (const uint16_t*)k,
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
