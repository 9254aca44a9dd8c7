// nsa_query.hip -- query-major bf16 kernels (forward and dQ) for gfx950.
//
// A workgroup owns up to 64 consecutive tokens of one (batch entry or packed
// sequence, KV head) and all their query heads, cut into 16-row tiles: the G
// heads of 16/G tokens (G < 16) or 16 heads of one token (G >= 16) -- the heads
// of a GQA group share one block list and are stacked as the MFMA rows.  Each
// wave holds RT tiles.  The workgroup walks the union of its tokens' listed
// blocks in ascending order, 32 keys at a time ("jobs"); every K/V slice is
// loaded from HBM once per workgroup (buffer loads, two jobs ahead) into a
// double-buffered LDS stage and read by the waves whose tiles list that
// block.  Per tile:
//   forward  S^T = K Q^T, mask, online softmax (base 2, lazy rescale),
//            O^T += V^T P^T  (V read transposed from LDS: ds_read_b64_tr_b16)
//   dQ       S^T = K Q^T, dP^T = V dO^T, dS = P (dP - Delta), dQ^T += K^T dS^T
// Every output row has one owner: no atomics.
//
// Method: page 1 of the reference text (NSA selection gradcheck gate) defines
// the call and its gradients; the formulas are the plain masked softmax and
// its exact gradient, as stated in include/nsa_sel.h.
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr float kNegInfQ = -__builtin_huge_valf();
constexpr float kLazyQ = 8.f;  // rescale only when a row max grows by > 2^8

__device__ __forceinline__ bf16x8 zero8() { return as_bf16x8(make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ bf16x8 pack8(const float (&lo)[4], const float (&hi)[4]) {
    return as_bf16x8(make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
}

// LDS of one workgroup: two stages of K and V slices (32 keys x D, padded
// rows), then per-block token masks (bit a = token T0 + a lists the block)
// and the compacted union.
template <int D>
struct QLds {
    static constexpr int kStride = D + 16;
    static constexpr int kTile = 32 * kStride;                 // elements per slice
    static constexpr int kStageBytes = 2 * 2 * kTile * 2;      // 2 stages x (K, V)
    static __host__ __device__ size_t bytes(int NBmax) {
        return (size_t)kStageBytes + (size_t)NBmax * 8 + (((size_t)NBmax * 2 + 15) & ~(size_t)15) + 16;
    }
};

// Host-chosen tiling of the query rows.
struct QGeo {
    int tpt;        // tokens per tile (G < 16), else 1
    int n_ht;       // tiles per token (G >= 16), else 1
    int TW;         // tokens per workgroup (<= 64)
    int wg_per_zh;  // workgroups per (z, hkv)
};

// Rows of one tile as seen by lane row r.
struct TileRow {
    int tok;      // token index inside the workgroup (bit of the block masks)
    int h, t;     // query head and token (safe values when !valid)
    bool valid;
};

__device__ __forceinline__ TileRow tile_row(const Problem& p, const QGeo& qg, int hkv, int T0,
                                            int len, int tau, int r) {
    TileRow x;
    if (p.G >= 16) {
        const int hg = 16 * (tau % qg.n_ht) + r;
        x.tok = tau / qg.n_ht;
        x.valid = hg < p.G && x.tok < qg.TW && T0 + x.tok < len;
        x.h = hkv * p.G + (hg < p.G ? hg : 0);
    } else {
        x.tok = tau * qg.tpt + r / p.G;
        x.valid = r < qg.tpt * p.G && x.tok < qg.TW && T0 + x.tok < len;
        x.h = hkv * p.G + r % p.G;
    }
    if (!x.valid) x.tok = 0;
    x.t = T0 + x.tok;
    return x;
}

// Mask of the workgroup tokens of tile tau.
__device__ __forceinline__ uint64_t tile_tokens(const Problem& p, const QGeo& qg, int tau) {
    if (p.G >= 16) {
        const int a = tau / qg.n_ht;
        return a < qg.TW ? 1ull << a : 0ull;
    }
    const int a = tau * qg.tpt;
    if (a >= qg.TW) return 0ull;  // tile past the workgroup's tokens: idle
    return ((1ull << qg.tpt) - 1ull) << a;
}

struct WgCoord {
    int z, hkv, T0;
};
__device__ __forceinline__ WgCoord wg_coord(const Problem& p, const QGeo& qg) {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    WgCoord c;
    const int zh = L / qg.wg_per_zh;
    c.z = zh / p.Hkv;
    c.hkv = zh % p.Hkv;
    c.T0 = (qg.wg_per_zh - 1 - (L % qg.wg_per_zh)) * qg.TW;  // heaviest (latest) first
    return c;
}

// Union of the blocks listed by tokens T0 .. T0+n_tok-1: umask[u] holds the
// tokens listing block u (0 <= u < NBz, u*bs <= t); ulist the ascending
// blocks with a non-empty mask.  Returns their count (same for all threads).
__device__ int wg_union(const Problem& p, const Seq& s, const int* __restrict__ idx, int hkv,
                        int T0, int n_tok, int NBz, unsigned long long* umask, uint16_t* ulist,
                        int* n_out) {
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int u = tid; u < NBz; u += nt) umask[u] = 0ull;
    __syncthreads();
    const int* rows = idx_row(p, s, idx, hkv, T0);
    const int n_ent = n_tok * p.S;
    for (int e = tid; e < n_ent; e += nt) {
        const int a = e / p.S, u = rows[e];
        if (u >= 0 && u < NBz && u * p.bs <= T0 + a) atomicOr(&umask[u], 1ull << a);
    }
    __syncthreads();
    if (tid < 64) {
        int n = 0;
        for (int base = 0; base < NBz; base += 64) {
            const int u = base + tid;
            const bool nz = u < NBz && umask[u] != 0ull;
            const uint64_t bal = __ballot(nz);
            if (nz) ulist[n + __popcll(bal & ((1ull << tid) - 1ull))] = (uint16_t)u;
            n += __popcll(bal);
        }
        if (tid == 0) *n_out = n;
    }
    __syncthreads();
    return *n_out;
}

// The workgroup's walk: 32-key jobs (block ulist[iu], slice sb), slices that
// start after the last token skipped.  All values wave-uniform.
struct Job {
    int iu, sb, u, j0;
    bool ok;
};
template <int BS>
__device__ __forceinline__ Job first_job(const uint16_t* ulist, int nU) {
    Job j;
    j.iu = 0;
    j.sb = 0;
    j.ok = nU > 0;
    j.u = j.ok ? __builtin_amdgcn_readfirstlane(ulist[0]) : 0;
    j.j0 = j.u * BS;
    return j;
}
template <int BS>
__device__ __forceinline__ Job next_job_q(Job c, const uint16_t* ulist, int nU, int t_last) {
    if (!c.ok) return c;
    if (c.sb + 1 < BS / 32 && c.j0 + 32 <= t_last) {
        ++c.sb;
        c.j0 += 32;
        return c;
    }
    if (c.iu + 1 >= nU) {
        c.ok = false;
        return c;
    }
    ++c.iu;
    c.sb = 0;
    c.u = __builtin_amdgcn_readfirstlane(ulist[c.iu]);
    c.j0 = c.u * BS;
    return c;
}

// This thread's share of one job's K and V slices (CH 16-byte chunks each).
template <int D, int NT>
struct SliceShare {
    static constexpr int VCH = D / 8;                      // chunks per key row
    static constexpr int CH = (32 * VCH + NT - 1) / NT;   // chunks per thread per tensor
};
template <int D, int NT>
struct SliceRegs {
    uint4 k[SliceShare<D, NT>::CH], v[SliceShare<D, NT>::CH];
};

template <int D, int NT>
__device__ __forceinline__ void slice_load(const uint16_t* kb, const uint16_t* vb, int kst2, int j0,
                                           int len, SliceRegs<D, NT>& sr) {
    constexpr int VCH = SliceShare<D, NT>::VCH;
    const char* kbase = reinterpret_cast<const char*>(kb) + (int64_t)j0 * kst2;
    const char* vbase = reinterpret_cast<const char*>(vb) + (int64_t)j0 * kst2;
    const uint32_t bytes = (uint32_t)((len - 1 - j0) * kst2 + 2 * D);
    const buf_rsrc rk = make_rsrc(kbase, bytes), rv = make_rsrc(vbase, bytes);
#pragma unroll
    for (int i = 0; i < SliceShare<D, NT>::CH; ++i) {
        const int c = i * NT + (int)threadIdx.x;
        const int off = (c / VCH) * kst2 + 16 * (c % VCH);
        // Chunks past the slice (c >= 32 * VCH) read past the descriptor and
        // come back as zero; they are not stored.
        const int voff = c < 32 * VCH ? off : 0x7fffffff;
        sr.k[i] = buf_load16(rk, voff, 0);
        sr.v[i] = buf_load16(rv, voff, 0);
    }
}

template <int D, int NT>
__device__ __forceinline__ void slice_store(const SliceRegs<D, NT>& sr, uint16_t* ks, uint16_t* vs) {
    constexpr int VCH = SliceShare<D, NT>::VCH, ST = QLds<D>::kStride;
#pragma unroll
    for (int i = 0; i < SliceShare<D, NT>::CH; ++i) {
        const int c = i * NT + (int)threadIdx.x;
        if (c < 32 * VCH) {
            const int o_ = (c / VCH) * ST + 8 * (c % VCH);
            *reinterpret_cast<uint4*>(ks + o_) = sr.k[i];
            *reinterpret_cast<uint4*>(vs + o_) = sr.v[i];
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, int BS, int RT, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_q_kernel(Problem p, QGeo qg,
                                                        const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const int* __restrict__ idx,
                                                        uint16_t* __restrict__ o,
                                                        float* __restrict__ lse) {
    constexpr int NT = NW * 64, KD = D / 32, ND = D / 16, ST = QLds<D>::kStride;
    constexpr int TILE = QLds<D>::kTile;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* stage = reinterpret_cast<uint16_t*>(smem);  // [2][K,V][TILE]
    unsigned long long* umask = reinterpret_cast<unsigned long long*>(smem + QLds<D>::kStageBytes);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);
    int* n_u = reinterpret_cast<int*>(smem + QLds<D>::bytes(p.NBmax) - 16);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const WgCoord wc = wg_coord(p, qg);
    const Seq s = seq_of(p, wc.z);
    if (wc.T0 >= s.len) return;
    const int n_tok = min(qg.TW, s.len - wc.T0);
    const int t_last = wc.T0 + n_tok - 1;
    const int NBz = (s.len + BS - 1) / BS;
    const int kst2 = (int)s.k_st * 2;
    const uint16_t* kb = k + s.k_base + wc.hkv * s.k_sh;
    const uint16_t* vb = v + s.k_base + wc.hkv * s.k_sh;

    // Per-tile state of this lane's row.
    TileRow tr[RT];
    uint64_t tmask[RT];
    bf16x8 qf[RT][KD];
    f32x4 acc[RT][ND];
    float m_run[RT], l_run[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int tau = w * RT + i;
        tr[i] = tile_row(p, qg, wc.hkv, wc.T0, s.len, tau, r);
        tmask[i] = tile_tokens(p, qg, tau);
        const uint16_t* qrow = q + s.q_base + (int)(tr[i].h * s.q_sh + tr[i].t * s.q_st) + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
            qf[i][kk] = tr[i].valid ? as_bf16x8(ldg16(qrow + 32 * kk)) : zero8();
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[i] = kNegInfQ;
        l_run[i] = 0.f;
    }
    const int nU = wg_union(p, s, idx, wc.hkv, wc.T0, n_tok, NBz, umask, ulist, n_u);
    const float c2 = p.scale_log2;

    // Pipeline: slices loaded two jobs ahead (registers A/B), LDS stages 0/1.
    Job j0 = first_job<BS>(ulist, nU);
    Job j1 = next_job_q<BS>(j0, ulist, nU, t_last);
    Job j2 = next_job_q<BS>(j1, ulist, nU, t_last);
    SliceRegs<D, NT> ra, rb;
    if (j0.ok) slice_load<D, NT>(kb, vb, kst2, j0.j0, s.len, ra);
    if (j1.ok) slice_load<D, NT>(kb, vb, kst2, j1.j0, s.len, rb);
    if (j0.ok) slice_store<D, NT>(ra, stage, stage + TILE);
    __syncthreads();

    auto do_job = [&](const Job& cur, int buf, SliceRegs<D, NT>& next2, const Job& jn2,
                      SliceRegs<D, NT>& next1, const Job& jn1) {
        if (jn2.ok) slice_load<D, NT>(kb, vb, kst2, jn2.j0, s.len, next2);
        const uint16_t* ks = stage + buf * 2 * TILE;
        const uint16_t* vs = ks + TILE;
        const uint64_t bm = umask[cur.u];
        bool any = false;
#pragma unroll
        for (int i = 0; i < RT; ++i) any |= (bm & tmask[i]) != 0ull;
        if (any) {
            bf16x8 ka[2][KD];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int kk = 0; kk < KD; ++kk)
                    ka[kt][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(ks + (16 * kt + r) * ST + 32 * kk + 8 * g));
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                if ((bm & tmask[i]) == 0ull) continue;
                f32x4 sc[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) sc[kt] = mfma(ka[kt][kk], qf[i][kk], sc[kt]);
                }
                // No mask when every token of the tile lists the block, the
                // slice ends before the tile's first token, and all rows exist.
                const bool full = ((bm & tmask[i]) == tmask[i]) && (cur.j0 + 31 <= tr[i].t - (tr[i].tok - (int)__builtin_ctzll(tmask[i]))) && tr[i].valid;
                float mloc = kNegInfQ;
                if (__builtin_amdgcn_readfirstlane((int)__all(full))) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) mloc = fmaxf(mloc, sc[kt][e]);
                } else {
                    const bool sel = tr[i].valid && ((bm >> tr[i].tok) & 1ull);
                    const int lim = sel ? tr[i].t - cur.j0 : -1;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (16 * kt + 4 * g + e > lim) sc[kt][e] = kNegInfQ;
                            mloc = fmaxf(mloc, sc[kt][e]);
                        }
                }
                const float mblk = col_max4(mloc);
                const bool grow = mblk * c2 > m_run[i] * c2 + kLazyQ;
                if (__builtin_amdgcn_readfirstlane((int)__any(grow))) {
                    const float m_new = grow ? mblk : m_run[i];
                    const float alpha = grow ? fast_exp2((m_run[i] - m_new) * c2) : 1.f;
#pragma unroll
                    for (int dt = 0; dt < ND; ++dt) acc[i][dt] *= alpha;
                    l_run[i] *= alpha;
                    m_run[i] = m_new;
                }
                const float mc = m_run[i] == kNegInfQ ? 0.f : m_run[i] * c2;
                float pv[2][4];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pv[kt][e] = fast_exp2(fmaf(sc[kt][e], c2, -mc));
                        l_run[i] += pv[kt][e];
                    }
                const bf16x8 pb = pack8(pv[0], pv[1]);
#pragma unroll
                for (int dt = 0; dt < ND; ++dt) {
                    const bf16x8 va = lds_col_operand(vs, ST, 0, 16, 16 * dt, lane);
                    acc[i][dt] = mfma(va, pb, acc[i][dt]);
                }
            }
        }
        if (jn1.ok) slice_store<D, NT>(next1, stage + (buf ^ 1) * 2 * TILE, stage + (buf ^ 1) * 2 * TILE + TILE);
        __syncthreads();
    };

    while (j0.ok) {
        Job j3 = next_job_q<BS>(j2, ulist, nU, t_last);
        do_job(j0, 0, ra, j2, rb, j1);
        if (!j1.ok) break;
        Job j4 = next_job_q<BS>(j3, ulist, nU, t_last);
        do_job(j1, 1, rb, j3, ra, j2);
        j0 = j2;
        j1 = j3;
        j2 = j4;
    }

#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const float l_tot = col_sum4(l_run[i]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (tr[i].valid) {
            uint16_t* orow = o + s.q_base + (int)(tr[i].h * s.q_sh + tr[i].t * s.q_st) + 4 * g;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const uint2 pk = make_uint2(pack_bf16x2(acc[i][dt][0] * inv, acc[i][dt][1] * inv),
                                            pack_bf16x2(acc[i][dt][2] * inv, acc[i][dt][3] * inv));
                *reinterpret_cast<uint2*>(orow + 16 * dt) = pk;
            }
            if (g == 0)
                lse[l_off(p, s, tr[i].h, tr[i].t)] =
                    l_tot > 0.f ? (m_run[i] * c2 + fast_log2(l_tot)) * kLn2 : kNegInfQ;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int BS, int RT, int NW>
__global__ __launch_bounds__(NW * 64) void dq_q_kernel(
    Problem p, QGeo qg, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ idx, uint16_t* __restrict__ dq) {
    constexpr int NT = NW * 64, KD = D / 32, ND = D / 16, ST = QLds<D>::kStride;
    constexpr int TILE = QLds<D>::kTile;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
    unsigned long long* umask = reinterpret_cast<unsigned long long*>(smem + QLds<D>::kStageBytes);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);
    int* n_u = reinterpret_cast<int*>(smem + QLds<D>::bytes(p.NBmax) - 16);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
    const WgCoord wc = wg_coord(p, qg);
    const Seq s = seq_of(p, wc.z);
    if (wc.T0 >= s.len) return;
    const int n_tok = min(qg.TW, s.len - wc.T0);
    const int t_last = wc.T0 + n_tok - 1;
    const int NBz = (s.len + BS - 1) / BS;
    const int kst2 = (int)s.k_st * 2;
    const uint16_t* kb = k + s.k_base + wc.hkv * s.k_sh;
    const uint16_t* vb = v + s.k_base + wc.hkv * s.k_sh;

    TileRow tr[RT];
    uint64_t tmask[RT];
    bf16x8 qf[RT][KD], df[RT][KD];
    f32x4 acc[RT][ND];
    float nlse2[RT], dl[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int tau = w * RT + i;
        tr[i] = tile_row(p, qg, wc.hkv, wc.T0, s.len, tau, r);
        tmask[i] = tile_tokens(p, qg, tau);
        const int ro = (int)(tr[i].h * s.q_sh + tr[i].t * s.q_st) + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            qf[i][kk] = tr[i].valid ? as_bf16x8(ldg16(q + s.q_base + ro + 32 * kk)) : zero8();
            df[i][kk] = tr[i].valid ? as_bf16x8(ldg16(dO + s.q_base + ro + 32 * kk)) : zero8();
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t lo_ = l_off(p, s, tr[i].h, tr[i].t);
        // A row with no key has lse = -inf and every score masked to -inf:
        // 0 keeps exp2(-inf + 0) = 0 instead of -inf + inf = NaN.
        const float lse_r = tr[i].valid ? lse[lo_] : 0.f;
        nlse2[i] = lse_r == kNegInfQ ? 0.f : -lse_r * kLog2e;
        dl[i] = tr[i].valid ? delta[lo_] : 0.f;
    }
    const int nU = wg_union(p, s, idx, wc.hkv, wc.T0, n_tok, NBz, umask, ulist, n_u);
    const float c2 = p.scale_log2;

    Job j0 = first_job<BS>(ulist, nU);
    Job j1 = next_job_q<BS>(j0, ulist, nU, t_last);
    Job j2 = next_job_q<BS>(j1, ulist, nU, t_last);
    SliceRegs<D, NT> ra, rb;
    if (j0.ok) slice_load<D, NT>(kb, vb, kst2, j0.j0, s.len, ra);
    if (j1.ok) slice_load<D, NT>(kb, vb, kst2, j1.j0, s.len, rb);
    if (j0.ok) slice_store<D, NT>(ra, stage, stage + TILE);
    __syncthreads();

    auto do_job = [&](const Job& cur, int buf, SliceRegs<D, NT>& next2, const Job& jn2,
                      SliceRegs<D, NT>& next1, const Job& jn1) {
        if (jn2.ok) slice_load<D, NT>(kb, vb, kst2, jn2.j0, s.len, next2);
        const uint16_t* ks = stage + buf * 2 * TILE;
        const uint16_t* vs = ks + TILE;
        const uint64_t bm = umask[cur.u];
        bool any = false;
#pragma unroll
        for (int i = 0; i < RT; ++i) any |= (bm & tmask[i]) != 0ull;
        if (any) {
            bf16x8 ka[2][KD], va[2][KD];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    const int o_ = (16 * kt + r) * ST + 32 * kk + 8 * g;
                    ka[kt][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(ks + o_));
                    va[kt][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(vs + o_));
                }
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                if ((bm & tmask[i]) == 0ull) continue;
                f32x4 sc[2], dp[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) {
                        sc[kt] = mfma(ka[kt][kk], qf[i][kk], sc[kt]);
                        dp[kt] = mfma(va[kt][kk], df[i][kk], dp[kt]);
                    }
                }
                const bool full = ((bm & tmask[i]) == tmask[i]) && (cur.j0 + 31 <= tr[i].t - (tr[i].tok - (int)__builtin_ctzll(tmask[i]))) && tr[i].valid;
                if (!__builtin_amdgcn_readfirstlane((int)__all(full))) {
                    const bool sel = tr[i].valid && ((bm >> tr[i].tok) & 1ull);
                    const int lim = sel ? tr[i].t - cur.j0 : -1;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (16 * kt + 4 * g + e > lim) sc[kt][e] = kNegInfQ;
                }
                float ds[2][4];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float P = fast_exp2(fmaf(sc[kt][e], c2, nlse2[i]));
                        ds[kt][e] = P * (dp[kt][e] - dl[i]);
                    }
                const bf16x8 dsb = pack8(ds[0], ds[1]);
#pragma unroll
                for (int dt = 0; dt < ND; ++dt) {
                    const bf16x8 kta = lds_col_operand(ks, ST, 0, 16, 16 * dt, lane);
                    acc[i][dt] = mfma(kta, dsb, acc[i][dt]);
                }
            }
        }
        if (jn1.ok) slice_store<D, NT>(next1, stage + (buf ^ 1) * 2 * TILE, stage + (buf ^ 1) * 2 * TILE + TILE);
        __syncthreads();
    };

    while (j0.ok) {
        Job j3 = next_job_q<BS>(j2, ulist, nU, t_last);
        do_job(j0, 0, ra, j2, rb, j1);
        if (!j1.ok) break;
        Job j4 = next_job_q<BS>(j3, ulist, nU, t_last);
        do_job(j1, 1, rb, j3, ra, j2);
        j0 = j2;
        j1 = j3;
        j2 = j4;
    }

#pragma unroll
    for (int i = 0; i < RT; ++i) {
        if (!tr[i].valid) continue;
        uint16_t* drow = dq + s.q_base + (int)(tr[i].h * s.q_sh + tr[i].t * s.q_st) + 4 * g;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint2 pk = make_uint2(pack_bf16x2(acc[i][dt][0] * p.scale, acc[i][dt][1] * p.scale),
                                        pack_bf16x2(acc[i][dt][2] * p.scale, acc[i][dt][3] * p.scale));
            *reinterpret_cast<uint2*>(drow + 16 * dt) = pk;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {
constexpr int kRT = 2;  // row tiles per wave
constexpr int kNW = 8;  // waves per workgroup

QGeo q_geo(const HostProblem& hp) {
    const Problem& p = hp.dev;
    QGeo qg;
    const int tiles = kNW * kRT;
    if (p.G >= 16) {
        qg.tpt = 1;
        qg.n_ht = (p.G + 15) / 16;
        qg.TW = std::max(1, tiles / qg.n_ht);
    } else {
        qg.tpt = 16 / p.G;
        qg.n_ht = 1;
        qg.TW = std::min(64, tiles * qg.tpt);
    }
    qg.wg_per_zh = (p.Tmax + qg.TW - 1) / qg.TW;
    return qg;
}
}  // namespace

size_t query_lds_bytes(const HostProblem& hp) {
    switch (hp.dev.D) {
        case 32: return QLds<32>::bytes(hp.dev.NBmax);
        case 64: return QLds<64>::bytes(hp.dev.NBmax);
        case 128: return QLds<128>::bytes(hp.dev.NBmax);
    }
    return 0;
}

// Waves actually holding tiles (tiles beyond TW*tiles-per-token are idle but
// still take part in staging).
#define NSA_Q_DISPATCH(D_, BS_, CALL)                                                      \
    do {                                                                                   \
        if ((D_) == 32 && (BS_) == 32) { constexpr int D = 32, BS = 32; CALL; }            \
        else if ((D_) == 32 && (BS_) == 64) { constexpr int D = 32, BS = 64; CALL; }       \
        else if ((D_) == 32 && (BS_) == 128) { constexpr int D = 32, BS = 128; CALL; }     \
        else if ((D_) == 64 && (BS_) == 32) { constexpr int D = 64, BS = 32; CALL; }       \
        else if ((D_) == 64 && (BS_) == 64) { constexpr int D = 64, BS = 64; CALL; }       \
        else if ((D_) == 64 && (BS_) == 128) { constexpr int D = 64, BS = 128; CALL; }     \
        else if ((D_) == 128 && (BS_) == 32) { constexpr int D = 128, BS = 32; CALL; }     \
        else if ((D_) == 128 && (BS_) == 64) { constexpr int D = 128, BS = 64; CALL; }     \
        else if ((D_) == 128 && (BS_) == 128) { constexpr int D = 128, BS = 128; CALL; }   \
        else return hipErrorInvalidValue;                                                  \
    } while (0)

hipError_t launch_fwd_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                           const int* block_idx, void* o, float* lse, hipStream_t st) {
    const QGeo qg = q_geo(hp);
    const unsigned grid = (unsigned)((int64_t)hp.ZH * qg.wg_per_zh);
    if (grid == 0) return hipSuccess;
    const size_t lds = query_lds_bytes(hp);
    NSA_Q_DISPATCH(hp.dev.D, hp.dev.bs,
                   hipLaunchKernelGGL((fwd_q_kernel<D, BS, kRT, kNW>), dim3(grid), dim3(kNW * 64), lds,
                                      st, hp.dev, qg, (const uint16_t*)q, (const uint16_t*)k,
                                      (const uint16_t*)v, block_idx, (uint16_t*)o, lse));
    return hipGetLastError();
}

hipError_t launch_dq_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const float* delta,
                          const int* block_idx, void* dq, hipStream_t st) {
    const QGeo qg = q_geo(hp);
    const unsigned grid = (unsigned)((int64_t)hp.ZH * qg.wg_per_zh);
    if (grid == 0) return hipSuccess;
    const size_t lds = query_lds_bytes(hp);
    NSA_Q_DISPATCH(hp.dev.D, hp.dev.bs,
                   hipLaunchKernelGGL((dq_q_kernel<D, BS, kRT, kNW>), dim3(grid), dim3(kNW * 64), lds,
                                      st, hp.dev, qg, (const uint16_t*)q, (const uint16_t*)k,
                                      (const uint16_t*)v, (const uint16_t*)dO, lse, delta, block_idx,
                                      (uint16_t*)dq));
    return hipGetLastError();
}

}  // namespace nsa
