// nsa_bf16.hip -- bf16 matrix-core (MFMA 16x16x32) kernels for gfx950:
//
//   fwd   one wave = one 16-row query tile: the G heads of 16/G consecutive
//         tokens (G < 16) or 16 heads of one token (G >= 16), i.e. the heads
//         of a GQA group stacked as the MFMA rows.  The wave walks the union
//         of its tokens' listed blocks in ascending order, 32 keys at a time:
//         S^T = K Q^T (K straight from HBM as the A operand), mask, online
//         softmax in the base-2 domain, O^T += V^T P^T (V staged row-major in
//         LDS, read transposed by ds_read_b64_tr_b16).  Emits o and lse.
//   dq    same tiling; recomputes P from lse, dP^T = V dO^T, dS = P (dP - Delta),
//         dQ^T += K^T dS^T.  One owner per output row: no atomics.
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

constexpr int kWaves = 4;  // waves per workgroup in fwd / dq
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ bf16x8 pack_operand(const float (&lo)[4], const float (&hi)[4]) {
    return as_bf16x8(make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
}

// Per-wave LDS region of the fwd / dq kernels: a 32-key x D bf16 tile, the
// per-block token masks and the compacted union list.
template <int D>
struct WaveLds {
    static constexpr int kStride = D + 8;                         // tile row stride (elements)
    static constexpr int kTileBytes = 32 * kStride * 2;
    static __host__ __device__ size_t bytes(int NBmax) {
        size_t b = kTileBytes + (size_t)NBmax * 4 + (size_t)NBmax * 2;
        return (b + 15) & ~(size_t)15;
    }
};

// Union of the blocks listed by the wave's n_tok tokens t0.. (all < len):
// ascending block numbers in ulist, and in umask[u] bit a set when token
// t0 + a lists u.  Only blocks whose first key is <= the token count.
__device__ int build_union(const Problem& p, const Seq& s, const int* __restrict__ idx, int hkv,
                           int t0, int n_tok, int NBz, uint32_t* umask, uint16_t* ulist,
                           int lane) {
    for (int u = lane; u < NBz; u += 64) umask[u] = 0u;
    wave_lds_fence();
    const int* rows = idx_row(p, s, idx, hkv, t0);
    const int n_ent = n_tok * p.S;
    for (int e = lane; e < n_ent; e += 64) {
        int a = e / p.S;
        int u = rows[e];
        if (u >= 0 && u < NBz && u * p.bs <= t0 + a) atomicOr(&umask[u], 1u << a);
    }
    wave_lds_fence();
    int n = 0;
    for (int base = 0; base < NBz; base += 64) {
        int u = base + lane;
        uint32_t m = u < NBz ? umask[u] : 0u;
        uint64_t bal = __ballot(m != 0u);
        if (m) ulist[n + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)u;
        n += __popcll(bal);
    }
    wave_lds_fence();
    return n;
}

// The query row a lane stands for inside its wave's 16-row tile.
struct LaneRow {
    int tok;     // token offset inside the wave (bit in the union masks)
    int h, t;    // query head and token (safe values when !valid)
    bool valid;
};

__device__ __forceinline__ LaneRow lane_row(const Problem& p, int hkv, int ht, int t0, int n_tok,
                                            int tpw, int r) {
    LaneRow x;
    if (p.G >= 16) {
        int hg = ht * 16 + r;
        x.tok = 0;
        x.valid = hg < p.G;
        x.h = hkv * p.G + (x.valid ? hg : 0);
    } else {
        x.tok = r / p.G;
        x.valid = (r < tpw * p.G) && (x.tok < n_tok);
        x.h = hkv * p.G + r % p.G;
    }
    if (!x.valid) x.tok = 0;
    x.t = t0 + x.tok;
    return x;
}

// Decode the workgroup of a fwd / dq launch: grid = (Z*Hkv*n_ht) heads x
// wg_per_head token groups, XCD-aware, latest (heaviest) token groups first.
struct TileCoord {
    int z, hkv, ht, wgi;
};
__device__ __forceinline__ TileCoord tile_coord(const Problem& p, int n_ht, int wg_per_head) {
    int L = xcd_remap(blockIdx.x, gridDim.x);
    int head = L / wg_per_head;
    TileCoord c;
    c.wgi = wg_per_head - 1 - (L % wg_per_head);
    int zh = head / n_ht;
    c.ht = head % n_ht;
    c.z = zh / p.Hkv;
    c.hkv = zh % p.Hkv;
    return c;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(Problem p, const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const int* __restrict__ idx,
                                                       uint16_t* __restrict__ o,
                                                       float* __restrict__ lse, int tpw, int n_ht,
                                                       int wg_per_head) {
    constexpr int KD = D / 32, ND = D / 16, VST = WaveLds<D>::kStride, VCH = D / 8;
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const TileCoord tc = tile_coord(p, n_ht, wg_per_head);
    const Seq s = seq_of(p, tc.z);
    const int t0 = (tc.wgi * kWaves + w) * tpw;
    if (t0 >= s.len) return;
    const int n_tok = min(tpw, s.len - t0);
    const int NBz = (s.len + BS - 1) / BS;
    const int t_last = t0 + n_tok - 1;

    unsigned char* my = smem + (size_t)w * WaveLds<D>::bytes(p.NBmax);
    uint16_t* vt = reinterpret_cast<uint16_t*>(my);
    uint32_t* umask = reinterpret_cast<uint32_t*>(my + WaveLds<D>::kTileBytes);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);

    const LaneRow lr = lane_row(p, tc.hkv, tc.ht, t0, n_tok, tpw, r);
    bf16x8 qf[KD];
    {
        const uint16_t* qrow = q + q_off(s, lr.h, lr.t);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
            qf[kk] = lr.valid ? as_bf16x8(ldg16(qrow + 32 * kk + 8 * g)) : zero_bf16x8();
    }
    const int nU = build_union(p, s, idx, tc.hkv, t0, n_tok, NBz, umask, ulist, lane);

    f32x4 acc[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    for (int iu = 0; iu < nU; ++iu) {
        const int u = __builtin_amdgcn_readfirstlane(ulist[iu]);
        const uint32_t tm = umask[u];
        const bool sel = lr.valid && ((tm >> lr.tok) & 1u);
#pragma unroll
        for (int sb = 0; sb < BS / 32; ++sb) {
            const int j0 = u * BS + sb * 32;
            if (j0 > t_last) break;
            // V rows of this 32-key slice (row-major into LDS after the scores).
            uint4 vreg[32 * VCH / 64];
#pragma unroll
            for (int c = 0; c < 32 * VCH / 64; ++c) {
                int cid = c * 64 + lane, key = cid / VCH, dc = cid % VCH, j = j0 + key;
                vreg[c] = j < s.len ? ldg16(v + k_off(s, tc.hkv, j) + 8 * dc) : make_uint4(0, 0, 0, 0);
            }
            f32x4 sc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int j = j0 + 16 * kt + r;
                const uint16_t* krow = k + k_off(s, tc.hkv, j);
                sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    bf16x8 kf = j < s.len ? as_bf16x8(ldg16(krow + 32 * kk + 8 * g)) : zero_bf16x8();
                    sc[kt] = mfma(kf, qf[kk], sc[kt]);
                }
            }
#pragma unroll
            for (int c = 0; c < 32 * VCH / 64; ++c) {
                int cid = c * 64 + lane, key = cid / VCH, dc = cid % VCH;
                *reinterpret_cast<uint4*>(vt + key * VST + 8 * dc) = vreg[c];
            }
            // Mask + online softmax.  Lane: row r, keys j0 + 16kt + 4g + i.
            float x[2][4];
            float mloc = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int j = j0 + 16 * kt + 4 * g + i;
                    bool ok = sel && j <= lr.t;
                    x[kt][i] = ok ? sc[kt][i] * p.scale_log2 : kNegInf;
                    mloc = fmaxf(mloc, x[kt][i]);
                }
            const float m_new = fmaxf(m_run, col_max4(mloc));
            const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
            float pv[2][4];
            float psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[kt][i] = x[kt][i] == kNegInf ? 0.f : fast_exp2(x[kt][i] - m_new);
                    psum += pv[kt][i];
                }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            const bf16x8 pb = pack_operand(pv[0], pv[1]);
            wave_lds_fence();
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                acc[dt] *= alpha;
                bf16x8 va = lds_col_operand(vt, VST, 0, 16, 16 * dt, lane);
                acc[dt] = mfma(va, pb, acc[dt]);
            }
            wave_lds_fence();
        }
    }
    const float l_tot = col_sum4(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (lr.valid) {
        uint16_t* orow = o + q_off(s, lr.h, lr.t);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            uint2 pk = make_uint2(pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                                  pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv));
            *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = pk;
        }
        if (g == 0)
            lse[l_off(p, s, lr.h, lr.t)] =
                l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void dq_bf16_kernel(
    Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ idx, uint16_t* __restrict__ dq,
    int tpw, int n_ht, int wg_per_head) {
    constexpr int KD = D / 32, ND = D / 16, KST = WaveLds<D>::kStride;
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const TileCoord tc = tile_coord(p, n_ht, wg_per_head);
    const Seq s = seq_of(p, tc.z);
    const int t0 = (tc.wgi * kWaves + w) * tpw;
    if (t0 >= s.len) return;
    const int n_tok = min(tpw, s.len - t0);
    const int NBz = (s.len + BS - 1) / BS;
    const int t_last = t0 + n_tok - 1;

    unsigned char* my = smem + (size_t)w * WaveLds<D>::bytes(p.NBmax);
    uint16_t* kt_lds = reinterpret_cast<uint16_t*>(my);
    uint32_t* umask = reinterpret_cast<uint32_t*>(my + WaveLds<D>::kTileBytes);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);

    const LaneRow lr = lane_row(p, tc.hkv, tc.ht, t0, n_tok, tpw, r);
    bf16x8 qf[KD], df[KD];
    {
        const int64_t ro = q_off(s, lr.h, lr.t);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            qf[kk] = lr.valid ? as_bf16x8(ldg16(q + ro + 32 * kk + 8 * g)) : zero_bf16x8();
            df[kk] = lr.valid ? as_bf16x8(ldg16(dO + ro + 32 * kk + 8 * g)) : zero_bf16x8();
        }
    }
    const int64_t lo_ = l_off(p, s, lr.h, lr.t);
    const float lse2 = lr.valid ? lse[lo_] * kLog2e : 0.f;
    const float dl = lr.valid ? delta[lo_] : 0.f;
    const int nU = build_union(p, s, idx, tc.hkv, t0, n_tok, NBz, umask, ulist, lane);

    f32x4 acc[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int iu = 0; iu < nU; ++iu) {
        const int u = __builtin_amdgcn_readfirstlane(ulist[iu]);
        const uint32_t tm = umask[u];
        const bool sel = lr.valid && ((tm >> lr.tok) & 1u);
#pragma unroll
        for (int sb = 0; sb < BS / 32; ++sb) {
            const int j0 = u * BS + sb * 32;
            if (j0 > t_last) break;
            f32x4 sc[2], dp[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int j = j0 + 16 * kt + r;
                const bool in = j < s.len;
                const int64_t ko = k_off(s, tc.hkv, j);
                sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    uint4 kraw = in ? ldg16(k + ko + 32 * kk + 8 * g) : make_uint4(0, 0, 0, 0);
                    uint4 vraw = in ? ldg16(v + ko + 32 * kk + 8 * g) : make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4*>(kt_lds + (16 * kt + r) * KST + 32 * kk + 8 * g) = kraw;
                    sc[kt] = mfma(as_bf16x8(kraw), qf[kk], sc[kt]);
                    dp[kt] = mfma(as_bf16x8(vraw), df[kk], dp[kt]);
                }
            }
            float ds[2][4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int j = j0 + 16 * kt + 4 * g + i;
                    bool ok = sel && j <= lr.t;
                    float P = ok ? fast_exp2(sc[kt][i] * p.scale_log2 - lse2) : 0.f;
                    ds[kt][i] = P * (dp[kt][i] - dl);
                }
            const bf16x8 dsb = pack_operand(ds[0], ds[1]);
            wave_lds_fence();
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                bf16x8 ka = lds_col_operand(kt_lds, KST, 0, 16, 16 * dt, lane);
                acc[dt] = mfma(ka, dsb, acc[dt]);
            }
            wave_lds_fence();
        }
    }
    if (lr.valid) {
        uint16_t* drow = dq + q_off(s, lr.h, lr.t);
        const float sc_ = p.scale;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            uint2 pk = make_uint2(pack_bf16x2(acc[dt][0] * sc_, acc[dt][1] * sc_),
                                  pack_bf16x2(acc[dt][2] * sc_, acc[dt][3] * sc_));
            *reinterpret_cast<uint2*>(drow + 16 * dt + 4 * g) = pk;
        }
    }
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

template <int D, int BS>
__global__ __launch_bounds__(BS / 16 * 64) void dkdv_bf16_kernel(
    Problem p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ offsets,
    const int* __restrict__ tokens, const int* __restrict__ item_pre,
    const int* __restrict__ pslot_pre, const int* __restrict__ zh_base, int CR,
    float* __restrict__ partials, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int NW = BS / 16, NT = NW * 64, KD = D / 32, ND = D / 16, QST = D + 8, QCH = D / 8;
    __shared__ __align__(16) uint16_t qs[32 * QST];
    __shared__ __align__(16) uint16_t ds_[32 * QST];
    __shared__ int row_t[32];
    __shared__ float row_lse2[32], row_dl[32];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r = lane & 15;
    const int ZH = p.Z * p.Hkv, NB = p.NBmax;
    ItemRef it;
    if (!find_item(blockIdx.x, ZH, NB, zh_base, item_pre, it)) return;
    const int z = it.zh / p.Hkv, hkv = it.zh % p.Hkv, u = it.u;
    const Seq s = seq_of(p, z);
    const int* off = offsets + (int64_t)it.zh * (NB + 1);
    const int* list = tokens + region_base(p, s, hkv) + off[u];
    const int R = (off[u + 1] - off[u]) * p.G;
    const int f_begin = it.kitem * CR, f_end = min(R, f_begin + CR);

    const int kw0 = u * BS + 16 * w;  // this wave's 16 keys
    const int jk = kw0 + r;
    bf16x8 kf[KD], vf[KD];
    {
        const bool in = jk < s.len;
        const int64_t ko = k_off(s, hkv, jk);
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

    for (int f0 = f_begin; f0 < f_end; f0 += 32) {
        __syncthreads();
        for (int c = tid; c < 32 * QCH; c += NT) {
            const int row = c / QCH, dc = c % QCH, f = f0 + row;
            uint4 qv = make_uint4(0, 0, 0, 0), dv4 = make_uint4(0, 0, 0, 0);
            if (f < f_end) {
                const int t = list[f / p.G], h = hkv * p.G + f % p.G;
                const int64_t o_ = q_off(s, h, t) + 8 * dc;
                qv = ldg16(q + o_);
                dv4 = ldg16(dO + o_);
            }
            *reinterpret_cast<uint4*>(qs + row * QST + 8 * dc) = qv;
            *reinterpret_cast<uint4*>(ds_ + row * QST + 8 * dc) = dv4;
        }
        if (tid < 32) {
            const int f = f0 + tid;
            if (f < f_end) {
                const int t = list[f / p.G], h = hkv * p.G + f % p.G;
                const int64_t lo_ = l_off(p, s, h, t);
                row_t[tid] = t;
                row_lse2[tid] = lse[lo_] * kLog2e;
                row_dl[tid] = delta[lo_];
            } else {
                row_t[tid] = -1;
                row_lse2[tid] = 0.f;
                row_dl[tid] = 0.f;
            }
        }
        __syncthreads();
        // S = Q K^T and dP = dO V^T for rows 16rt + 4g + i, key jk.
        f32x4 sc[2], dp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            sc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) {
                bf16x8 qa = as_bf16x8(*reinterpret_cast<const uint4*>(qs + (16 * rt + r) * QST + 32 * kk + 8 * g));
                bf16x8 da = as_bf16x8(*reinterpret_cast<const uint4*>(ds_ + (16 * rt + r) * QST + 32 * kk + 8 * g));
                sc[rt] = mfma(qa, kf[kk], sc[rt]);
                dp[rt] = mfma(da, vf[kk], dp[rt]);
            }
        }
        float pv[2][4], dsv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rt + 4 * g + i;
                const int t = row_t[row];
                const bool ok = t >= 0 && jk <= t;
                const float P = ok ? fast_exp2(sc[rt][i] * p.scale_log2 - row_lse2[row]) : 0.f;
                pv[rt][i] = P;
                dsv[rt][i] = P * (dp[rt][i] - row_dl[row]);
            }
        const bf16x8 pa = pack_operand(pv[0], pv[1]);
        const bf16x8 dsa = pack_operand(dsv[0], dsv[1]);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            bf16x8 dob = lds_col_operand(ds_, QST, 0, 16, 16 * dt, lane);
            dva[dt] = mfma(pa, dob, dva[dt]);
            bf16x8 qb = lds_col_operand(qs, QST, 0, 16, 16 * dt, lane);
            dka[dt] = mfma(dsa, qb, dka[dt]);
        }
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
template <int D, int BS>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(
    Problem p, const int* __restrict__ item_pre, const int* __restrict__ pslot_pre,
    const int* __restrict__ zh_base, const float* __restrict__ partials,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    const int NB = p.NBmax, ZH = p.Z * p.Hkv;
    const int zh = blockIdx.x / NB, u = blockIdx.x % NB;
    const int z = zh / p.Hkv, hkv = zh % p.Hkv;
    const Seq s = seq_of(p, z);
    if (u * BS >= s.len) return;
    const int* ip = item_pre + (int64_t)zh * (NB + 1);
    const int n = ip[u + 1] - ip[u];
    if (n == 1) return;
    const int slot0 = n > 1 ? zh_base[ZH + 1 + zh] + pslot_pre[(int64_t)zh * (NB + 1) + u] : 0;
    for (int e = threadIdx.x; e < BS * D; e += blockDim.x) {
        const int kl = e / D, d = e % D, key = u * BS + kl;
        if (key >= s.len) continue;
        float a = 0.f, b = 0.f;
        for (int kk = 0; kk < n; ++kk) {
            const float* pk = partials + (int64_t)(slot0 + kk) * 2 * BS * D;
            a += pk[e];
            b += pk[BS * D + e];
        }
        const int64_t ko = k_off(s, hkv, key) + d;
        dk[ko] = f32_to_bf16(a * p.scale);
        dv[ko] = f32_to_bf16(b);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
size_t fwd_bf16_lds_bytes(const HostProblem& hp) {
    const int D = hp.dev.D;
    size_t per = 0;
    if (D == 32) per = WaveLds<32>::bytes(hp.dev.NBmax);
    else if (D == 64) per = WaveLds<64>::bytes(hp.dev.NBmax);
    else if (D == 128) per = WaveLds<128>::bytes(hp.dev.NBmax);
    return per * kWaves;
}

namespace {
struct QTiling {
    int tpw, n_ht, wg_per_head;
    unsigned grid;
};
QTiling q_tiling(const HostProblem& hp) {
    const Problem& p = hp.dev;
    QTiling t;
    t.tpw = p.G >= 16 ? 1 : 16 / p.G;
    t.n_ht = p.G >= 16 ? (p.G + 15) / 16 : 1;
    int wave_tiles = (p.Tmax + t.tpw - 1) / t.tpw;
    t.wg_per_head = (wave_tiles + kWaves - 1) / kWaves;
    t.grid = (unsigned)((int64_t)hp.ZH * t.n_ht * t.wg_per_head);
    return t;
}
}  // namespace

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

hipError_t launch_fwd_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                           const int* block_idx, void* o, float* lse, hipStream_t st) {
    const QTiling t = q_tiling(hp);
    if (t.grid == 0) return hipSuccess;
    const size_t lds = fwd_bf16_lds_bytes(hp);
    NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                      hipLaunchKernelGGL((fwd_bf16_kernel<D, BS>), dim3(t.grid), dim3(256), lds, st,
                                         hp.dev, (const uint16_t*)q, (const uint16_t*)k,
                                         (const uint16_t*)v, block_idx, (uint16_t*)o, lse, t.tpw,
                                         t.n_ht, t.wg_per_head));
    return hipGetLastError();
}

hipError_t launch_dq_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const float* delta,
                          const int* block_idx, void* dq, hipStream_t st) {
    const QTiling t = q_tiling(hp);
    if (t.grid == 0) return hipSuccess;
    const size_t lds = fwd_bf16_lds_bytes(hp);
    NSA_DISPATCH_D_BS(hp.dev.D, hp.dev.bs,
                      hipLaunchKernelGGL((dq_bf16_kernel<D, BS>), dim3(t.grid), dim3(256), lds, st,
                                         hp.dev, (const uint16_t*)q, (const uint16_t*)k,
                                         (const uint16_t*)v, (const uint16_t*)dO, lse, delta,
                                         block_idx, (uint16_t*)dq, t.tpw, t.n_ht, t.wg_per_head));
    return hipGetLastError();
}

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
