// nsa_dkdv.hip -- key-major dK / dV for bf16 on gfx950 matrix cores
// (v_mfma_f32_16x16x32_bf16).
//
// One workgroup = one key block u (BS keys, BS / 16 waves) and one chunk of
// the block's inverted list of query rows (token, head).  The rows are taken
// 32 at a time, newest token first, and copied from HBM straight into a
// four-stage LDS ring by buffer loads that write LDS (no register staging),
// two steps ahead of their use.  Per step and 32 keys:
//     S = Q K^T,  dP = dO V^T              (K, V of the keys in VGPRs)
//     P = exp(S*scale - lse) (causal),  dS = P (dP - Delta)
//     dV^T += dO^T P,  dK^T += Q^T dS      (accumulated transposed)
// the first two lines on one wave, the last on another (see dkdv_kernel).
// A list longer than one chunk writes fp32 partials that dkdv_reduce sums in
// chunk order, so the result does not depend on scheduling.
//
// Scheduling: with a multiple of 8 (batch, kv-head) groups of equal length,
// work items are dealt out so that consecutive items (the blocks of one
// group) run on one XCD; as all of them walk their row lists from the newest
// token down, the blocks that share rows read them at about the same time
// and mostly from that XCD's L2.  Otherwise (packed sequences, or fewer
// groups than XCDs, where contiguous ranges would give some XCDs all the
// long early-block lists) items are dealt round-robin over the XCDs.
//
// Method: page 1 of the reference text (NSA selection gradcheck gate) defines
// the call and its gradients; the backward formulas are the exact gradient of
// the masked softmax attention, as stated in include/nsa_sel.h.
#include <algorithm>
#include <type_traits>

#include "nsa_internal.h"

namespace nsa {

namespace {

// One stage of the row ring: the Q and dO tiles of 32 rows (RowTile layout)
// and their lse and Delta, one copy per accumulator wave (entries 32.. take
// the zeros of unused lanes).
template <int D, int NP>
struct alignas(16) Stage {
    uint16_t q[32 * D];
    uint16_t dO[32 * D];
    float lse[NP][64];
    float dl[NP][64];
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
// rows at a time without dividing.  hoff / hoff2 = h * (byte stride of a head)
// in two tensors.
struct Cursor {
    int f, e, h;
    uint32_t hoff, hoff2;
};

__device__ __forceinline__ Cursor cursor_at(int f, int G, uint32_t hstride, uint32_t hstride2 = 0) {
    Cursor c;
    c.f = f;
    const int ff = max(f, 0);
    c.e = ff / G;
    c.h = ff - c.e * G;
    c.hoff = (uint32_t)c.h * hstride;
    c.hoff2 = (uint32_t)c.h * hstride2;
    return c;
}

// Moves the cursor 32 rows down: q32 = 32 / G, r32 = 32 % G; the strides
// are r32 and G times the heads' byte strides.
__device__ __forceinline__ void retreat32(Cursor& c, int G, int q32, int r32, uint32_t r32_stride,
                                          uint32_t G_stride, uint32_t r32_stride2 = 0,
                                          uint32_t G_stride2 = 0) {
    c.f -= 32;
    c.h -= r32;
    c.e -= q32;
    c.hoff -= r32_stride;
    c.hoff2 -= r32_stride2;
    if (c.h < 0) {
        c.h += G;
        c.e -= 1;
        c.hoff += G_stride;
        c.hoff2 += G_stride2;
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
// Waves come in pairs; pair a owns keys u BS + 32 a .. + 31 of the block.
//   S wave (w = a):        S = Q K^T, dP = dO V^T with its keys' K and V in
//                          VGPRs; P and dS (bf16) go to its pair's LDS slot.
//   accumulator (w = NP + a): one step behind, dV^T += dO^T P and
//                          dK^T += Q^T dS from that slot and the staged rows
//                          (read transposed); it also issues the row loads.
// Splitting the two halves of the work keeps 32 keys per wave (each staged
// tile is read by two waves of a pair per operand layout, not by four waves
// of 16 keys) while neither wave needs more than 256 VGPRs, so two
// workgroups share a CU and their waves hide each other's latency.
// The slot is reused every step: the accumulator counts in `freed` when it
// has read it, and the S wave waits for that count before writing again.
// PAIRED: a launch over pairs of the problem's blocks (BS = 2 block_size
// keys per workgroup) that runs only when the planner found whole causal
// prefixes everywhere (then the list of block 2U holds every row that sees a
// key of block 2U + 1 and the rows it adds see none of them: the causal mask
// removes those).  pair_on: this is the per-block launch of a problem that
// also has the paired one, so it runs only when the paired one does not.
// WIN: the problem has a sliding window (keys t - window < j only); the
// paired launch never has one.  BK: keys of one block (BS, except 16-key
// blocks, which run on a 32-key tile whose upper 16 keys -- the next
// block's -- are masked out and never written).  DS != 0: the S waves also
// store dS (bf16) for the dQ kernel that takes it over, dsout[entry][key in
// the block][head], entry = region_base + the row's position in the block's
// list; DS = 1 for G a multiple of 16 (a 16-row half of a step is 16 heads of
// one token), DS = 2 for G = 4 or 8 (the four rows a lane holds are four
// heads of one token).
template <int D, int BS, bool PAIRED, bool WIN, int BK = BS, int DS = 0>
__global__ __launch_bounds__(BS / 16 * 64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void dkdv_kernel(Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
                 const float* __restrict__ lse, const float* __restrict__ delta,
                 const int* __restrict__ offsets, const int* __restrict__ tokens,
                 const int* __restrict__ item_pre, const int* __restrict__ pslot_pre,
                 const int* __restrict__ zh_base, const int* __restrict__ iota, int CR, int pair_on,
                 float* __restrict__ partials, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                 uint16_t* __restrict__ dsout) {
    using L = RowTile<D>;
    constexpr int NP = BS / 32, KD = D / 32, ND = D / 16, QCH = L::QCH, NI = L::NI;
    constexpr int NJ = (NI + NP - 1) / NP;  // 1 KB row loads per tile for each accumulator (at most)
    constexpr bool kEven = NP * NJ == NI;   // every accumulator has exactly NJ
    __shared__ Stage<D, NP> st0, st1, st2, st3;
    // Token ids of the rows of step x in tkr[a][x % 4], one copy per
    // accumulator wave a (entries 32.. unused).
    __shared__ __attribute__((aligned(16))) int tkr[NP][4][64];
    __shared__ uint4 pbuf[NP][2][2][64];  // [pair][P, dS][key tile][lane]
    __shared__ int freed[NP];
    __shared__ int wait_fail;  // an S wave's wait gave up (see spin_ge)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r = lane & 15;
    const bool s_wave = w < NP;
    const int a = s_wave ? w : w - NP;
    const int ZH = p.Z * p.Hkv, NB = p.NBmax, G = p.G;
    const int whole_prefix = pair_on ? zh_base[2 * (ZH + 1) + 3 * ZH] : 0;
    if (PAIRED ? !whole_prefix : whole_prefix) return;
    // Paired: NU pairs of blocks per (z, hkv), one item each.
    const int NU = PAIRED ? (NB + 1) / 2 : NB;
    const int n_items = PAIRED ? ZH * NU : zh_base[ZH];
    if ((int)blockIdx.x >= n_items) return;
    ItemRef it;
    int li = (!p.packed && ZH % 8 == 0) ? xcd_remap(blockIdx.x, n_items) : (int)blockIdx.x;
    if (!p.packed && ZH % 8 == 0 && n_items == ZH * NU) {
        // One item per block (every list fits one chunk): the XCD's ZH / 8
        // groups are interleaved block-major, so its launch order runs from
        // the longest lists to the shortest once, not once per group.  (A
        // bijection on the items either way.)
        const int gx = ZH / 8, per = n_items / 8;
        const int x = li / per, k = li % per;
        li = (x * gx + k % gx) * NU + k / gx;
    }
    if constexpr (PAIRED) {
        it.zh = li / NU;
        it.u = li - it.zh * NU;
        it.kitem = 0;
        it.nitems = 1;
    } else {
        find_item(li, ZH, NB, zh_base, item_pre, it);
    }
    const int z = it.zh / p.Hkv, hkv = it.zh % p.Hkv, u = it.u;
    const Seq s = seq_of(p, z);
    if (PAIRED && u * BS >= s.klen) return;  // pair past a short sequence's end
    const int lu = PAIRED ? 2 * u : u;      // the list walked: block lu's
    const int* off = offsets + (int64_t)it.zh * (NB + 1);
    // Paired (whole prefixes): block lu's list is the tokens lu bs .. len - 1.
    const int* list = PAIRED ? iota + lu * p.bs : tokens + region_base(p, s, hkv) + off[lu];
    const int R = (off[lu + 1] - off[lu]) * G;
    const int64_t ds_entry0 = DS ? region_base(p, s, hkv) + off[lu] : 0;
    const int gsh = G == 4 ? 2 : 3;
    const int f_begin = it.kitem * CR, f_end = min(R, f_begin + CR);
    const int nsteps = (f_end - f_begin + 31) / 32;
    static_assert(BK == BS || (BK == 16 && BS == 32 && !PAIRED), "a 16-key block on a 32-key tile");
    const int kbase = u * BK + 32 * a;
    if (tid < NP) freed[tid] = 0;
    if (tid == 0) wait_fail = 0;

    f32x4 dkt[2][ND], dvt[2][ND];  // accumulators: dK^T / dV^T of keys kbase + 16 kt + r

    if (s_wave) {
        // K and V of the pair's 32 keys as MFMA B operands: kf[kt][kk] holds
        // K[key 16kt + r][32kk + 8g .. + 7].
        bf16x8 kf[2][KD], vf[2][KD];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int key = kbase + 16 * kt + r;
            const bool in = 16 * kt < BK && key < s.klen;
            const uint16_t* kr = k + row_off(p.lk, s, hkv, in ? key : 0) + 8 * g;
            const uint16_t* vr = v + row_off(p.lv, s, hkv, in ? key : 0) + 8 * g;
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                kf[kt][kk] = in ? as_bf16x8(ldg16(kr + 32 * kk)) : as_bf16x8(make_uint4(0, 0, 0, 0));
                vf[kt][kk] = in ? as_bf16x8(ldg16(vr + 32 * kk)) : as_bf16x8(make_uint4(0, 0, 0, 0));
            }
        }
        uint32_t a_off[KD];
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) a_off[kk] = L::a_off(lane, kk);
        const float c2 = p.scale_log2;

        // One step in phases the compiler may not interleave (every operand
        // read gets its own register and is in flight before its use): all
        // reads of the tile and its row metadata, S and dP, then P and dS.
        auto s_step = [&](int i, const Stage<D, NP>& sg) {
            if (i < nsteps) {
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
                    tt[rt] = *reinterpret_cast<const int4*>(&tkr[a][i & 3][16 * rt + 4 * g]);
                    ll[rt] = *reinterpret_cast<const float4*>(&sg.lse[a][16 * rt + 4 * g]);
                    dd[rt] = *reinterpret_cast<const float4*>(&sg.dl[a][16 * rt + 4 * g]);
                }
                __builtin_amdgcn_sched_barrier(0);

                f32x4 sc[2][2], dp[2][2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        sc[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        dp[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                // S, and dP.  Per-block items issue the dP products inside p_ds below,
                // between P's exponentials (P needs S alone, so the wave's own
                // softmax fills the matrix pipe's shadow: dK/dV 1-3 % faster on
                // sparse lists); paired items keep the two sets together (the
                // split measured 2-3 % slower there).
                constexpr bool kLateDp = !PAIRED;
#pragma unroll
                for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt) {
                            sc[rt][kt] = mfma(qa[kk][rt], kf[kt][kk], sc[rt][kt]);
                            if constexpr (!kLateDp) dp[rt][kt] = mfma(da[kk][rt], vf[kt][kk], dp[rt][kt]);
                        }
                if constexpr (!kLateDp) __builtin_amdgcn_sched_barrier(0);

                // P and dS for rows 16rt + 4g + i, keys kbase + 16kt + r; the
                // exponential is taken for every entry and masked by a select.
                // Row x of the step is list row f_end - 32 (i + 1) + x; rows
                // below the chunk take token -1 (no key passes the mask).
                const int f0 = f_end - 32 * (i + 1) - f_begin;
                int tv[2][4];  // key positions of the rows' tokens; -1: no row
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int x0 = f0 + 16 * rt + 4 * g;
                    tv[rt][0] = x0 >= 0 ? tt[rt].x + s.qoff : -1;
                    tv[rt][1] = x0 + 1 >= 0 ? tt[rt].y + s.qoff : -1;
                    tv[rt][2] = x0 + 2 >= 0 ? tt[rt].z + s.qoff : -1;
                    tv[rt][3] = x0 + 3 >= 0 ? tt[rt].w + s.qoff : -1;
                }
                float pv[2][2][4], dsv[2][2][4];
                auto p_ds = [&](auto masked) __attribute__((always_inline)) {
                    if constexpr (kLateDp) {
#pragma unroll
                        for (int kk = 0; kk < KD; ++kk)
#pragma unroll
                            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                                for (int kt = 0; kt < 2; ++kt)
                                    dp[rt][kt] = mfma(da[kk][rt], vf[kt][kk], dp[rt][kt]);
                    }
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) {
                        const float nl[4] = {-ll[rt].x * kLog2e, -ll[rt].y * kLog2e, -ll[rt].z * kLog2e,
                                             -ll[rt].w * kLog2e};
                        const float de[4] = {dd[rt].x, dd[rt].y, dd[rt].z, dd[rt].w};
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt) {
                            const int key = kbase + 16 * kt + r;
#pragma unroll
                            for (int i4 = 0; i4 < 4; ++i4) {
                                const float e = fast_exp2(fmaf(sc[rt][kt][i4], c2, nl[i4]));
                                float P = e;
                                if constexpr (decltype(masked)::value) {
                                    const bool vis = 16 * kt < BK &&
                                                     (WIN ? key <= tv[rt][i4] && key + p.window > tv[rt][i4]
                                                          : key <= tv[rt][i4]);
                                    P = vis ? e : 0.f;
                                }
                                pv[kt][rt][i4] = P;
                                if constexpr (!kLateDp) dsv[kt][rt][i4] = P * (dp[rt][kt][i4] - de[i4]);
                            }
                        }
                    }
                    if constexpr (kLateDp) {
                        // One dP product, then three of P's instructions.
#pragma unroll
                        for (int x = 0; x < 4 * KD; ++x) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                            __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);  // VALU, transcendental
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int rt = 0; rt < 2; ++rt) {
                            const float de[4] = {dd[rt].x, dd[rt].y, dd[rt].z, dd[rt].w};
#pragma unroll
                            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                                for (int i4 = 0; i4 < 4; ++i4)
                                    dsv[kt][rt][i4] = pv[kt][rt][i4] * (dp[rt][kt][i4] - de[i4]);
                        }
                    }
                };
                // Every row of the step exists and sees all of the pair's keys
                // (away from the diagonal and the list's end): no selects.
                int tmin = min(min(min(tv[0][0], tv[0][1]), min(tv[0][2], tv[0][3])),
                               min(min(tv[1][0], tv[1][1]), min(tv[1][2], tv[1][3])));
                bool open = BK >= 32 && tmin >= kbase + 31;
                if constexpr (WIN) {
                    const int tmax = max(max(max(tv[0][0], tv[0][1]), max(tv[0][2], tv[0][3])),
                                         max(max(tv[1][0], tv[1][1]), max(tv[1][2], tv[1][3])));
                    open = open && kbase + p.window > tmax;
                }
                if (wave_all(open)) p_ds(std::false_type{});
                else p_ds(std::true_type{});
                uint4 pk[2][2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    pk[0][kt] = __builtin_bit_cast(uint4, pack8(pv[kt][0], pv[kt][1]));
                    pk[1][kt] = __builtin_bit_cast(uint4, pack8(dsv[kt][0], dsv[kt][1]));
                }
                if constexpr (DS) {
                    // dS of the step's rows: lane (g, r) holds list rows
                    // fl .. fl + 3 (fl = the step's first row + 16 rt + 4 g)
                    // of key 32 a + 16 kt + r -- with G a multiple of 4, four
                    // heads of one entry, 8 contiguous bytes.
                    const int fr0 = __builtin_amdgcn_readfirstlane(f_end - 32 * (i + 1));
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) {
                        const int fr = fr0 + 16 * rt, fl = fr + 4 * g;
                        uint16_t* dst;
                        if constexpr (DS == 1) {
                            // G a multiple of 16: a 16-row half is one entry
                            // (wave-uniform).
                            if (fr < f_begin) continue;  // rows of another item
                            const int e = fr / G;
                            dst = dsout + ((ds_entry0 + e) * BS + 32 * a) * G + (fr - e * G) + 4 * g;
                        } else {
                            // G = 4 or 8: entries differ across the lanes.
                            if (fl < f_begin) continue;
                            const int e = fl >> gsh;
                            dst = dsout + ((ds_entry0 + e) * BS + 32 * a) * G + (fl - e * G);
                        }
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt) {
                            const uint4 x = pk[1][kt];
                            // Non-temporal: dS is read once, by the dQ kernel
                            // after the reduce, and would otherwise push the
                            // fp32 partials and the q / dO rows out of the
                            // caches.
                            const u32x2 v = rt == 0 ? u32x2{x.x, x.y} : u32x2{x.z, x.w};
                            __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(dst + (int64_t)(16 * kt + r) * G));
                        }
                    }
                }
                // The accumulator has read the previous step's P / dS.
                if (i > 0) spin_ge(&freed[a], i, &wait_fail);
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) pbuf[a][x][kt][lane] = pk[x][kt];
            }
            // (An S wave issues no loads; with DS its stores may stay in flight.)
            if constexpr (DS) wait_vm_barrier<60>();
            else wait_vm_barrier<0>();
        };
        // The accumulators' prologue has two barriers.
        wait_vm_barrier<0>();
        wait_vm_barrier<0>();
        for (int i = 0; i <= nsteps; i += 4) {
            s_step(i, st0);
            if (i + 1 <= nsteps) s_step(i + 1, st1);
            if (i + 2 <= nsteps) s_step(i + 2, st2);
            if (i + 3 <= nsteps) s_step(i + 3, st3);
        }
        report_wait_timeouts(&wait_fail);
        return;
    }

    // ---- accumulator wave -------------------------------------------------
    // Buffers of this (z, kv group): rows (h, t) of q / dO and lse / Delta.
    // Every valid row lies below the sizes; invalid rows use an offset past
    // them and load zeros.
    const uint16_t* qb = q + head_base(p.lq, s, hkv * G);
    const uint16_t* db = dO + head_base(p.ldo, s, hkv * G);
    const int64_t q_elems = (int64_t)(G - 1) * p.lq.sh + (int64_t)(s.len - 1) * p.lq.st + D;
    const int64_t d_elems = (int64_t)(G - 1) * p.ldo.sh + (int64_t)(s.len - 1) * p.ldo.st + D;
    const buf_rsrc rq = make_rsrc(qb, (uint32_t)(2 * q_elems));
    const buf_rsrc rd = make_rsrc(db, (uint32_t)(2 * d_elems));
    const int64_t l_first = s.l_base + (int64_t)(hkv * G) * p.T;
    const uint32_t l_bytes = (uint32_t)(4 * ((int64_t)(G - 1) * p.T + s.len));
    const buf_rsrc rl = make_rsrc(lse + l_first, l_bytes);
    const buf_rsrc rdl = make_rsrc(delta + l_first, l_bytes);
    constexpr uint32_t kOob = 0xFFFFFFF0u;
    // Byte strides of a head and of a token in q and in dO.
    const uint32_t qsh_b = (uint32_t)(2 * p.lq.sh), qst_b = (uint32_t)(2 * p.lq.st);
    const uint32_t dsh_b = (uint32_t)(2 * p.ldo.sh), dst_b = (uint32_t)(2 * p.ldo.st);
    const uint32_t lsh_b = (uint32_t)(4 * p.T);
    const int q32 = 32 / G, r32 = 32 % G;
    const bool same_qd = qsh_b == dsh_b && qst_b == dst_b;
    const uint32_t q_r32 = (uint32_t)r32 * qsh_b, q_G = (uint32_t)G * qsh_b;
    const uint32_t d_r32 = (uint32_t)r32 * dsh_b, d_G = (uint32_t)G * dsh_b;
    const uint32_t l_r32 = (uint32_t)r32 * lsh_b, l_G = (uint32_t)G * lsh_b;

    // Rows this lane loads: 1 KB load jj = a + NP * j of a tile covers the
    // 16-byte positions 64 jj + lane, i.e. row (64 jj + lane) / QCH at some
    // LDS slot, which holds data chunk chunk(row, slot) of that row.
    Cursor cq[NJ];
    int qrow[NJ];
    uint32_t cofs[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int jj = min(a + NP * j, NI - 1);
        const int pos = 64 * jj + lane;
        qrow[j] = pos / QCH;
        cofs[j] = 16u * (uint32_t)L::chunk(qrow[j], pos % QCH);
        cq[j] = cursor_at(f_end - 32 + qrow[j], G, qsh_b, dsh_b);
    }
    // Lanes < 32: row `lane` of each step, once for the token list (one step
    // ahead of the rows) and once for lse / Delta, into this accumulator's
    // own copies (lanes 32.. load zeros into unused entries).
    const int mrow = lane & 31;
    const bool meta = lane < 32;
    Cursor ct = cursor_at(f_end - 32 + mrow, G, 0u);
    Cursor cm = cursor_at(f_end - 32 + mrow, G, lsh_b);
    const buf_rsrc rt = make_rsrc(list, (uint32_t)(4 * (R / G)));

    // (A) token ids of step x into tkr[a][x % 4]: list[e] of every row.
    auto tok_dma = [&](int x) {
        dma4(rt, &tkr[a][x & 3][0], meta && ct.f >= f_begin ? 4u * (uint32_t)ct.e : kOob);
        retreat32(ct, G, q32, r32, 0u, 0u);
    };
    // (B) the rows of step x into stage `sg` with token ids from
    // tkr[a][x % 4] (written by an earlier tok_dma that has completed): Q and
    // dO rows, then lse and Delta.  `pre` runs once the token ids are read.
    auto row_dma = [&](int x, Stage<D, NP>& sg, auto&& pre) {
        const int* slot_t = &tkr[a][x & 3][0];
        int tj[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) tj[j] = slot_t[qrow[j]];
        const int tm = slot_t[mrow];
        pre();
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int jj = a + NP * j;
            if (kEven || jj < NI) {
                // Token ids are < 2^20 and byte token strides < 2^24 (both
                // checked on the host): 24-bit multiplies, full rate.  When
                // q and dO share a layout (uniform) one offset serves both.
                const bool in = cq[j].f >= f_begin;
                const uint32_t vq = in ? cq[j].hoff + __umul24((uint32_t)tj[j], qst_b) + cofs[j] : kOob;
                const uint32_t vd = same_qd ? vq
                                  : in ? cq[j].hoff2 + __umul24((uint32_t)tj[j], dst_b) + cofs[j] : kOob;
                dma16(rq, reinterpret_cast<uint8_t*>(sg.q) + 1024 * jj, vq);
                dma16(rd, reinterpret_cast<uint8_t*>(sg.dO) + 1024 * jj, vd);
            }
            retreat32(cq[j], G, q32, r32, q_r32, q_G, d_r32, d_G);
        }
        {
            const uint32_t lo = meta && cm.f >= f_begin ? cm.hoff + 4u * (uint32_t)tm : kOob;
            dma4(rl, &sg.lse[a][0], lo);
            dma4(rdl, &sg.dl[a][0], lo);
        }
        retreat32(cm, G, q32, r32, l_r32, l_G);
    };

    uint32_t t_off[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) t_off[dt] = L::t_off(lane, dt);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            dkt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dvt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // The products of one step on a staged tile and the pair's P / dS:
    // dV^T[d][key] += sum_rows dO[row][d] P[row][key]; dK^T likewise with Q
    // and dS.  The transposed operand's contraction rows are 4g + e and
    // 16 + 4g + e, the rows the C layout of S gave the S wave's lane.
    auto acc_step = [&](const Stage<D, NP>& sg) {
        uint4 pk[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) pk[x][kt] = pbuf[a][x][kt][lane];
        signal(&freed[a], lane);
        const uint8_t* tq = reinterpret_cast<const uint8_t*>(sg.q);
        const uint8_t* td = reinterpret_cast<const uint8_t*>(sg.dO);
        bf16x8 dcol[ND], qcol[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint2 d0 = lds_read_tr(reinterpret_cast<const uint16_t*>(td + t_off[dt]));
            const uint2 d1 = lds_read_tr(reinterpret_cast<const uint16_t*>(td + t_off[dt] + 16 * L::RB));
            dcol[dt] = __builtin_bit_cast(bf16x8, make_uint4(d0.x, d0.y, d1.x, d1.y));
        }
        __builtin_amdgcn_sched_barrier(0);
        // The dO^T operands are all in flight; the Q^T reads go out while the
        // dV^T products run.
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                dvt[kt][dt] = mfma(dcol[dt], __builtin_bit_cast(bf16x8, pk[0][kt]), dvt[kt][dt]);
            const uint2 q0 = lds_read_tr(reinterpret_cast<const uint16_t*>(tq + t_off[dt]));
            const uint2 q1 = lds_read_tr(reinterpret_cast<const uint16_t*>(tq + t_off[dt] + 16 * L::RB));
            qcol[dt] = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                dkt[kt][dt] = mfma(qcol[dt], __builtin_bit_cast(bf16x8, pk[1][kt]), dkt[kt][dt]);
    };

    // Loads an accumulator issues per step: the token ids (A), 2 per row
    // load group (Q, dO) and lse / Delta (B), every step, also past the end
    // of the list (they then load zeros into stages and slots nobody reads
    // any more).  The end-of-step wait lets the newest (B) loads stay in
    // flight; everything older (the rows of the next step, the token ids of
    // the step after) is then complete.  An accumulator without a full
    // share of row loads waits for all of them.
    constexpr int kInFlight = 2 * NJ + 2;
    const bool full_share = kEven || a + NP * (NJ - 1) < NI;
    auto end_wait = [&]() {
        if (kEven || full_share) wait_vm_barrier<kInFlight>(); else wait_vm_barrier<0>();
    };

    // Prologue: token ids of steps 0..2, then the rows of steps 0 and 1.
    tok_dma(0);
    tok_dma(1);
    tok_dma(2);
    wait_vm_barrier<0>();
    row_dma(0, st0, [] {});
    row_dma(1, st1, [] {});
    end_wait();

    // Step i (0 <= i <= nsteps): read the token ids of step i + 2, then
    // issue (A) those of step i + 3 into slot (i + 3) % 4 (last read in step
    // i - 1) and (B) the rows of step i + 2 into stage (i + 2) % 4 (last read
    // by the accumulators in step i - 1); the products of step i - 1 (stage
    // (i - 1) % 4); wait, barrier.  The S waves work on step i (stage i % 4,
    // token slot i % 4) meanwhile.
    auto step = [&](int i, const Stage<D, NP>& prev, Stage<D, NP>& nxt2) {
        row_dma(i + 2, nxt2, [&] { tok_dma(i + 3); });
        if (i > 0) acc_step(prev);
        end_wait();
    };
    for (int i = 0; i <= nsteps; i += 4) {
        step(i, st3, st2);
        if (i + 1 <= nsteps) step(i + 1, st0, st3);
        if (i + 2 <= nsteps) step(i + 2, st1, st0);
        if (i + 3 <= nsteps) step(i + 3, st2, st1);
    }

    // Output: dvt[kt][dt][i] = dV[key kbase + 16kt + r][16dt + 4g + i].
    if (it.nitems == 1) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int key = kbase + 16 * kt + r;
            if (16 * kt >= BK || key >= s.klen) continue;
            uint16_t* dkr = dk + row_off(p.ldk, s, hkv, key) + 4 * g;
            uint16_t* dvr = dv + row_off(p.ldv, s, hkv, key) + 4 * g;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const f32x4 x = dkt[kt][dt], y = dvt[kt][dt];
                *reinterpret_cast<uint2*>(dkr + 16 * dt) =
                    make_uint2(pack_bf16x2(x[0] * p.scale, x[1] * p.scale),
                               pack_bf16x2(x[2] * p.scale, x[3] * p.scale));
                *reinterpret_cast<uint2*>(dvr + 16 * dt) =
                    make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
    } else {
        // Partial slot layout: [dk, dv][16-key tile of the block][dt][lane] x
        // 4 floats; this pair's tiles are 2 a + kt.
        const int slot = zh_base[ZH + 1 + it.zh] + pslot_pre[(int64_t)it.zh * (NB + 1) + u] + it.kitem;
        f32x4* pk = reinterpret_cast<f32x4*>(partials + (int64_t)slot * 2 * BS * D);
        f32x4* pv_ = pk + BS * D / 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const int e = ((a * 2 + kt) * ND + dt) * 64 + lane;
                pk[e] = dkt[kt][dt];
                pv_[e] = dvt[kt][dt];
            }
    }
}

// Sums the fp32 partials of split lists in chunk order and writes zeros for
// blocks no row attends to (blocks handled whole by one item are skipped).
// Thread e4 owns one float4 of the slot layout [plane][tile][dt][lane], i.e.
// dK or dV of key 16 tile + (lane & 15), columns 16 dt + 4
// (lane >> 4) .. + 3.  Chunk loads are issued eight at a time but added
// strictly in chunk order.  rs workgroups share one block, each a contiguous
// share of its float4s (the launch picks rs so that there are about 4096
// workgroups, at least enough for 4 float4s per thread: with few blocks, up
// to 16 per block, so a block listed by many rows does not hold back the
// others; with many, fewer, since most blocks need no reduction and their
// workgroups only exit).
template <int D, int BS, int BK = BS>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(
    Problem p, const int* __restrict__ item_pre, const int* __restrict__ pslot_pre,
    const int* __restrict__ zh_base, const float* __restrict__ partials, int rs,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int ND = D / 16, E4 = BS * D / 4;  // float4 per plane of one block
    const int NB = p.NBmax, ZH = p.Z * p.Hkv;
    const int bu = blockIdx.x / rs, sp = blockIdx.x % rs;
    const int zh = bu / NB, u = bu % NB;
    const int z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    if (u * BK >= s.klen) return;
    const int* ip = item_pre + (int64_t)zh * (NB + 1);
    const int n = ip[u + 1] - ip[u];
    if (n == 1) return;
    const int slot0 = n > 1 ? zh_base[ZH + 1 + zh] + pslot_pre[(int64_t)zh * (NB + 1) + u] : 0;
    const float4* part = reinterpret_cast<const float4*>(partials) + (int64_t)slot0 * 2 * E4;
    // This workgroup's float4s: e0 + threadIdx.x + 256 q for q < kP (rs is
    // at least 2 E4 / (256 kP)); each thread loads its kP of them for four
    // chunks at a time and adds them in chunk order.
    constexpr int kP = 4;
    const int per = (2 * E4 + rs - 1) / rs;
    const int e0 = sp * per, e_end = min(2 * E4, e0 + per);
    int pos[kP], key[kP];
    bool on[kP];
#pragma unroll
    for (int q = 0; q < kP; ++q) {
        pos[q] = e0 + (int)threadIdx.x + 256 * q;
        const int x = pos[q] % E4;
        const int ln = x % 64, tile = x / (64 * ND);
        key[q] = u * BK + 16 * tile + (ln & 15);
        on[q] = pos[q] < e_end && 16 * tile < BK && key[q] < s.klen;
    }
    float4 acc[kP];
#pragma unroll
    for (int q = 0; q < kP; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int kk = 0; kk < n; kk += 4) {
        float4 x[kP][4];
#pragma unroll
        for (int q = 0; q < kP; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[q][j] = on[q] && kk + j < n ? part[pos[q] + (int64_t)(kk + j) * 2 * E4]
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (kk + j >= n) break;
#pragma unroll
            for (int q = 0; q < kP; ++q) {
                acc[q].x += x[q][j].x; acc[q].y += x[q][j].y; acc[q].z += x[q][j].z; acc[q].w += x[q][j].w;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kP; ++q) {
        if (!on[q]) continue;
        const int plane = pos[q] / E4, x = pos[q] % E4;
        const int dt = (x / 64) % ND, d = 16 * dt + 4 * ((x % 64) >> 4);
        const float m = plane == 0 ? p.scale : 1.f;
        const uint2 pk = make_uint2(pack_bf16x2(acc[q].x * m, acc[q].y * m), pack_bf16x2(acc[q].z * m, acc[q].w * m));
        uint16_t* dst = plane == 0 ? dk + row_off(p.ldk, s, hkv, key[q]) + d
                                   : dv + row_off(p.ldv, s, hkv, key[q]) + d;
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
    const int64_t n_blocks = (int64_t)hp.ZH * hp.dev.NBmax;
    const int tile = std::max(32, hp.dev.bs);  // keys per partial slot
    const int64_t rs_min = ((int64_t)tile * hp.dev.D / 2 + 1023) / 1024;  // 2 E4 / (256 * 4)
    const int rs = (int)std::max<int64_t>(rs_min, std::min<int64_t>(16, 4096 / std::max<int64_t>(1, n_blocks)));
    // Without partial slots every list (empty ones included) is written whole
    // by the block kernel: nothing to reduce.
    const unsigned nred = (parts & kDkdvReduce) && hp.pslots > 0 ? (unsigned)(n_blocks * rs) : 0u;
    if (items) {
        const int pair_on = hp.pair_possible ? 1 : 0;
        auto go = [&](auto kernel, unsigned grid, int threads) {
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, st, hp.dev, (const uint16_t*)q,
                               (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dO, lse,
                               delta, ws.offsets, ws.tokens, ws.item_pre, ws.pslot_pre, ws.zh_base,
                               ws.iota, hp.CR, pair_on, ws.partials, (uint16_t*)dk, (uint16_t*)dv,
                               ws.ds);
        };
        if (pair_on) {
            // The paired launch first (it does the work for whole-prefix
            // selections); the per-block launch then exits at once.
            const unsigned pairs = (unsigned)((int64_t)hp.ZH * ((hp.dev.NBmax + 1) / 2));
            NSA_DISPATCH_D_BS(hp.dev.D, 2 * hp.dev.bs,
                              go(dkdv_kernel<D, BS, true, false>, pairs, BS / 16 * 64));
        }
        if (hp.dev.bs == 16) {
            // 16-key blocks on the 32-key tile (two waves).
            if (hp.dev.window > 0)
                NSA_DISPATCH_D_BS(hp.dev.D, 32, go(dkdv_kernel<D, 32, false, true, 16>, items, 128));
            else
                NSA_DISPATCH_D_BS(hp.dev.D, 32, go(dkdv_kernel<D, 32, false, false, 16>, items, 128));
        } else if (hp.dev.window > 0) {
            NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs, go(dkdv_kernel<D, BS, false, true>, items, BS / 16 * 64));
        } else if (hp.ds_handoff) {
            // Also stores dS for the dQ kernel that takes it over.
            NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                              if (hp.dev.G % 16 == 0) go(dkdv_kernel<D, BS, false, false, BS, 1>, items, BS / 16 * 64);
                              else go(dkdv_kernel<D, BS, false, false, BS, 2>, items, BS / 16 * 64));
        } else {
            NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs, go(dkdv_kernel<D, BS, false, false>, items, BS / 16 * 64));
        }
    }
    if (nred && hp.dev.bs == 16) {
        NSA_DISPATCH_D_BS(hp.dev.D, 32,
                          hipLaunchKernelGGL((dkdv_reduce_kernel<D, 32, 16>), dim3(nred), dim3(256), 0,
                                             st, hp.dev, ws.item_pre, ws.pslot_pre, ws.zh_base,
                                             ws.partials, rs, (uint16_t*)dk, (uint16_t*)dv));
    } else if (nred) {
        NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                          hipLaunchKernelGGL((dkdv_reduce_kernel<D, BS>), dim3(nred), dim3(256), 0,
                                             st, hp.dev, ws.item_pre, ws.pslot_pre, ws.zh_base,
                                             ws.partials, rs, (uint16_t*)dk, (uint16_t*)dv));
    }
    return hipGetLastError();
}

// Bounded waits of this file's kernels that gave up (see spin_ge).
hipError_t read_wait_timeouts_dkdv(unsigned* out) {
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(g_wait_timeouts), sizeof(unsigned), 0,
                               hipMemcpyDeviceToHost);
}

}  // namespace nsa
