// nsa_query.hip -- query-major bf16 kernels (forward and dQ) for gfx950.
//
// A workgroup owns up to 64 consecutive tokens of one (batch entry or packed
// sequence, KV head) and all their query heads, cut into 16-row tiles: the G
// heads of 16/G tokens (G < 16) or 16 heads of one token (G >= 16) -- the heads
// of a GQA group share one block list and are stacked as the MFMA rows.  Each
// wave holds RT tiles.  The workgroup walks the union of its tokens' listed
// blocks in ascending order, one job at a time (a 64-key block, half of a
// 128-key one, or a 32-key block); every K/V slice is copied from HBM once
// per workgroup, straight into a four-stage LDS ring by buffer loads that
// write LDS (two jobs ahead, no register staging), and read by the waves
// whose tiles list that block.  Per tile:
//   forward  S^T = K Q^T, mask, online softmax (base 2, lazy rescale),
//            O^T += V^T P^T  (V read transposed from LDS: ds_read_b64_tr_b16)
//   dQ       S^T = K Q^T, dP^T = V dO^T, dS = P (dP - Delta), dQ^T += K^T dS^T
//   dQ from the dS the dK/dV kernel hands off: dQ^T += K^T dS^T (K alone in
//            the ring, dS tiles staged per wave)
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

// Keys per job: whole 64-key blocks (half blocks of 128), 32 for 32-key
// blocks.  A 16-key block is walked as a 32-key job (the matrix-core step
// contracts 32 keys) whose second 16 keys -- the next block's -- are masked
// out: KT keys of the job belong to its block.
template <int BS>
struct JobKeys {
    static constexpr int JK = BS >= 64 ? 64 : 32;
    static constexpr int KT = BS < JK ? BS : JK;
};

// One stage of the K/V ring: JK-key slices of K and V, rows in the RowTile
// layout (rows 32.. repeat the slots of rows 0..).
template <int D, int JK>
struct alignas(16) KVStage {
    uint16_t k[JK * D];
    uint16_t v[JK * D];
};
// A stage holding K alone (dQ from a handed-off dS needs no V).
template <int D, int JK>
struct alignas(16) KStage {
    uint16_t k[JK * D];
};
constexpr int kQStages = 4;  // ring depth
constexpr int kQAhead = 2;   // jobs between issuing a stage's loads and computing it

// LDS of one workgroup: the ring (static, separate variables) and, in
// dynamic LDS, per-block token masks (bit a = token T0 + a lists the block)
// and the compacted union.
template <int D, int JK>
struct QLds {
    static constexpr size_t kStatic = (size_t)kQStages * sizeof(KVStage<D, JK>) + 64;
    static __host__ __device__ size_t dynamic_bytes(int NBmax) {
        return (size_t)NBmax * 8 + (((size_t)NBmax * 2 + 15) & ~(size_t)15) + 16;
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

// Mask of the workgroup tokens of tile tau (wave-uniform: stated with
// readfirstlane so the mask lives in scalar registers; as a vector-register
// pair it was spilled and reloaded inside the job loop, and a reload waits
// for every load in flight, ring stages included).
__device__ __forceinline__ uint64_t tile_tokens(const Problem& p, const QGeo& qg, int tau) {
    uint64_t m;
    if (p.G >= 16) {
        const int a = tau / qg.n_ht;
        m = a < qg.TW ? 1ull << a : 0ull;
    } else {
        const int a = tau * qg.tpt;
        m = a >= qg.TW ? 0ull : ((1ull << qg.tpt) - 1ull) << a;  // past the tokens: idle
    }
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)m);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(m >> 32));
    return ((uint64_t)hi << 32) | lo;
}

struct WgCoord {
    int z, hkv, T0;
};
// Packed inputs with at most 64 sequences: workgroup b takes kv head
// b % Hkv and the (b / Hkv)-th non-empty (window level, sequence) pair,
// levels from the latest window down (level lw holds token windows starting
// at (L - 1 - lw) TW), sequences in index order within a level; workgroups
// past the last pair are empty and come last.  (Empty workgroups spread
// through the launch order, one per window past a short sequence's end, were
// measured to hold back the dispatch of the real ones: forward on 8 packed
// sequences of 128-4096 tokens, 32/8 heads, D 128, 0.618 -> 0.460 ms.)  Each wave computes this alone: lane z holds sequence
// z's first level s_z = L - ceil(len_z / TW), so P(lw) = sum_z max(0, lw -
// s_z) pairs precede level lw and #{z : s_z <= lw} lie on it; 64 candidate
// levels are tested per pass, one per lane.  Returns false when b is past
// the last pair.
__device__ bool packed_pair(const Problem& p, const QGeo& qg, int b, int& zh, int& w) {
    const int lane = threadIdx.x & 63, L = qg.wg_per_zh;
    int s_z = L;
    if (lane < p.Z) {
        const int len = min(max(p.cu[lane + 1] - p.cu[lane], 0), p.Tmax);
        s_z = L - (len + qg.TW - 1) / qg.TW;
    }
    const int hkv = b % p.Hkv, n = b / p.Hkv;
    for (int c = 0; c < L; c += 64) {
        const int lw = c + lane;
        int before = 0, on = 0;
        for (int z = 0; z < p.Z; ++z) {
            const int sz = __builtin_amdgcn_readlane(s_z, z);
            before += max(0, lw - sz);
            on += sz <= lw ? 1 : 0;
        }
        const uint64_t hit = __ballot(lw < L && before <= n && n < before + on);
        if (hit) {
            const int src = __builtin_ctzll(hit), lev = c + src;
            const int r = n - __builtin_amdgcn_readlane(before, src);
            const uint64_t live = __ballot(lane < p.Z && s_z <= lev);
            const int rank = __popcll(live & ((1ull << lane) - 1ull));
            const uint64_t pick = __ballot(((live >> lane) & 1ull) && rank == r);
            zh = __builtin_ctzll(pick) * p.Hkv + hkv;
            w = lev;
            return true;
        }
    }
    return false;
}

// With a multiple of 8 (z, hkv) groups of equal length (dense inputs) the
// workgroups of one group run on one XCD (consecutive logical indices) and
// share its K/V in that L2, and every XCD gets the same work.  With fewer
// groups than XCDs, one group's token windows would be cut across XCDs by
// position and the XCDs holding the latest tokens would get most of the
// work; then, and for packed inputs, workgroups are dealt round-robin over
// the XCDs, latest token first (packed: as above, or, with more than 64
// sequences, every (window, group) in turn, empty ones included).  K/V then
// come from HBM or the memory-side cache more often.  b: the workgroup's
// place in that order (its block index, or the item a persistent workgroup
// took), of nb in all.
__device__ __forceinline__ WgCoord wg_coord(const Problem& p, const QGeo& qg, int b, int nb) {
    WgCoord c;
    int zh, w;
    const int ZH = p.Z * p.Hkv;
    if (p.packed && p.Z <= 64) {
        if (!packed_pair(p, qg, b, zh, w)) {
            zh = 0;
            w = -1;  // past the last pair: T0 lies past every sequence
        }
    } else if (p.packed || ZH % 8 != 0) {
        zh = b % ZH;
        w = b / ZH;
    } else {
        const int L = xcd_remap(b, nb);
        zh = L / qg.wg_per_zh;
        w = L % qg.wg_per_zh;
    }
    c.z = zh / p.Hkv;
    c.hkv = zh % p.Hkv;
    c.T0 = (qg.wg_per_zh - 1 - w) * qg.TW;
    return c;
}
__device__ __forceinline__ WgCoord wg_coord(const Problem& p, const QGeo& qg) {
    return wg_coord(p, qg, (int)blockIdx.x, (int)gridDim.x);
}

// Union of the blocks listed by tokens T0 .. T0+n_tok-1: umask[u] holds the
// tokens listing block u (0 <= u < NBz, u*bs <= t, and inside the token's
// sliding window if there is one); ulist the ascending
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
        // (With a sliding window, only blocks reaching into token T0 + a's
        // window: the others are masked entirely, so they are not walked.)
        const int tp = T0 + a + s.qoff;  // the token's key position
        if (u >= 0 && u < NBz && u * p.bs <= tp &&
            (p.window <= 0 || (u + 1) * p.bs > tp - p.window + 1))
            atomicOr(&umask[u], 1ull << a);
    }
    __syncthreads();
    // The listed blocks in ascending order, and their token masks moved to
    // the same positions (umask[i] = the mask of block ulist[i]), so a walk
    // reads a job's block and mask from one position.  In place: a
    // position never exceeds its block, and each 64-block chunk's masks are
    // read before any lane writes.
    if (tid < 64) {
        int n = 0;
        for (int base = 0; base < NBz; base += 64) {
            const int u = base + tid;
            const uint64_t m = u < NBz ? umask[u] : 0ull;
            const bool nz = m != 0ull;
            const uint64_t bal = __ballot(nz);
            if (nz) {
                const int pos = n + __popcll(bal & ((1ull << tid) - 1ull));
                ulist[pos] = (uint16_t)u;
                umask[pos] = m;
            }
            n += __popcll(bal);
        }
        if (tid == 0) *n_out = n;
    }
    __syncthreads();
    return *n_out;
}

// The workgroup's walk: JK-key jobs (block ulist[iu], slice sb), slices that
// start after the last token skipped.  All values wave-uniform.  bm: the
// tokens of the workgroup that list the block (umask[iu]), read with the
// block for the jobs a wave computes (MASK), so the job's first operand
// reads need no LDS round trip of their own.
struct Job {
    int iu, sb, u, j0;
    bool ok;
    uint64_t bm;
};
struct UnionList {
    const uint16_t* ulist;
    const unsigned long long* umask;
    int nU;
};
template <int BS, bool MASK = false>
__device__ __forceinline__ Job first_job(const UnionList& ul) {
    Job j;
    j.iu = 0;
    j.sb = 0;
    j.ok = ul.nU > 0;
    j.u = j.ok ? __builtin_amdgcn_readfirstlane(ul.ulist[0]) : 0;
    j.bm = MASK && j.ok ? uniform64(ul.umask[0]) : 0ull;
    j.j0 = j.u * BS;
    return j;
}
template <int BS, bool MASK = false>
__device__ __forceinline__ Job next_job_q(Job c, const UnionList& ul, int t_last) {
    constexpr int JK = JobKeys<BS>::JK;
    if (!c.ok) return c;
    if (c.sb + 1 < BS / JK && c.j0 + JK <= t_last) {
        ++c.sb;
        c.j0 += JK;
        return c;
    }
    if (c.iu + 1 >= ul.nU) {
        c.ok = false;
        return c;
    }
    ++c.iu;
    c.sb = 0;
    c.u = __builtin_amdgcn_readfirstlane(ul.ulist[c.iu]);
    if constexpr (MASK) c.bm = uniform64(ul.umask[c.iu]);
    c.j0 = c.u * BS;
    return c;
}

// Buffer-to-LDS loads of one job's K and V slices (JK keys from key j0):
// 1 KB load jj (< 2 NI; K for jj < NI, V after) is issued by wave jj % NW,
// lane l writing RowTile position 64 (jj % NI) + l.  The K and V buffer
// descriptors cover the (sequence, KV head) and are built once; a job adds
// its first key's offset to each lane's 32-bit offset, and a lane whose key
// lies past the sequence (or a job slot past the last job) gets an offset
// past every descriptor, which loads zeros.
template <int D, int NW, int JK, bool KONLY = false>
struct KVLoad {
    using L = RowTile<D>;
    static constexpr int NI = JK * 2 * D / 1024;      // 1 KB loads per tensor
    static constexpr int NL = KONLY ? NI : 2 * NI;     // loads per job
    static constexpr int NJ = (NL + NW - 1) / NW;      // loads per wave (at most)
    static constexpr int RPL = 64 / L::QCH;            // key rows per 1 KB load
    static constexpr uint32_t kOob = 0xFFFFFFF0u;      // past every descriptor's size
    buf_rsrc rk, rv;     // K and V of the (sequence, KV head)
    uint32_t voff[NJ];   // byte offset of this lane's 16 bytes in a slice from key 0
    int jj[NJ];          // load index (>= 2 NI: none)
    int lrow;            // this lane's key row inside its load
    int kst2, vst2, len;
    // w must be wave-uniform (it selects the descriptor of each load).
    // kst2 / vst2: byte strides between the keys of K / V; len >= 1 keys.
    __device__ void init(int w, int lane, const uint16_t* kb, const uint16_t* vb, int kst2_,
                         int vst2_, int len_) {
        w = __builtin_amdgcn_readfirstlane(w);
        kst2 = kst2_;
        vst2 = vst2_;
        len = len_;
        rk = make_rsrc(kb, (uint32_t)((int64_t)(len - 1) * kst2 + 2 * D));
        rv = make_rsrc(vb, (uint32_t)((int64_t)(len - 1) * vst2 + 2 * D));
        lrow = lane / L::QCH;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            jj[j] = w + NW * j;
            const int pos = 64 * (jj[j] % NI) + lane, row = pos / L::QCH;
            voff[j] = (uint32_t)row * (uint32_t)(jj[j] < NI ? kst2 : vst2) +
                      16u * (uint32_t)L::chunk(row, pos % L::QCH);
        }
    }
    // Loads this wave issues per job when it has its full share; kEven: all
    // waves have it.
    static constexpr int kPerWave = NJ;
    static constexpr bool kEven = NL % NW == 0;
    __device__ bool full_share() const { return jj[NJ - 1] < NL; }
    // Issued for every job slot, also past the last job (ok == false): those
    // loads all fall out of range and write zeros into a free stage, so a
    // wave always has the same number of loads in flight.
    template <class Stage>
    __device__ void issue(int j0, bool ok, Stage& st) const {
        const uint32_t ko = (uint32_t)j0 * (uint32_t)kst2, vo = (uint32_t)j0 * (uint32_t)vst2;
        const int lim = ok ? len - j0 : 0;  // rows r < lim of the job exist
        const bool whole = lim >= JK;       // wave-uniform: no row past the sequence
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const bool isk = jj[j] < NI;
            const uint32_t on = voff[j] + (isk ? ko : vo);
            const uint32_t o = whole || lrow < lim - RPL * (jj[j] % NI) ? on : kOob;
            if constexpr (KONLY) {
                if (kEven || jj[j] < NI) dma16(rk, reinterpret_cast<uint8_t*>(st.k) + 1024 * jj[j], o);
            } else if constexpr (kEven) {
                // Every wave has NJ loads: pick K or V without branching, so
                // the count of loads in flight is the same on every path.
                uint8_t* dst = isk ? reinterpret_cast<uint8_t*>(st.k) + 1024 * jj[j]
                                   : reinterpret_cast<uint8_t*>(st.v) + 1024 * (jj[j] - NI);
                dma16(isk ? rk : rv, dst, o);
            } else {
                if (jj[j] < NI) dma16(rk, reinterpret_cast<uint8_t*>(st.k) + 1024 * jj[j], o);
                else if (jj[j] < 2 * NI) dma16(rv, reinterpret_cast<uint8_t*>(st.v) + 1024 * (jj[j] - NI), o);
            }
        }
    }
};

// vmcnt(N) alone (no barrier).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// LDS address of a __shared__ int (for the counter instructions below).
// The workgroup's walk over its jobs with a ring of kQStages K/V stages and
// no workgroup barrier per job: waves advance at their own pace, at most one
// job apart (slack kQAhead - 1), synchronised by two counters per stage.
//   landed[s]: waves whose share of the stage's job has arrived in LDS;
//   done[s]:   waves that finished computing the stage's job.
// Job j lives in stage j % kQStages.  In its step j a wave
//   1. waits until every wave finished job j + A - NS (the last user of the
//      stage job j + A goes to), then issues its share of job j + A;
//   2. waits for its own share of job j + 1 (vmcnt) and counts it in landed;
//   3. waits until all shares of job j landed, computes job j, counts done.
// The slowest wave can always proceed (everything it waits for was counted
// by waves at or ahead of it), so the walk ends.  Counts are cumulative: the
// u-th use of a stage is complete at NW * (u + 1).
template <int D, int BS, int NW, class Compute>
__device__ __forceinline__ void q_ring(const KVLoad<D, NW, JobKeys<BS>::JK>& ld, const UnionList& ul,
                                       int t_last, int lane, Compute&& compute) {
    constexpr int JK = JobKeys<BS>::JK, NS = kQStages, A = kQAhead;
    using LD = KVLoad<D, NW, JK>;
    static_assert(NS == 4 && A == 2, "the unrolled walk below is written for 4 stages, 2 ahead");
    __shared__ KVStage<D, JK> s0, s1, s2, s3;
    __shared__ int landed[NS], done[NS], wait_fail;
    if (threadIdx.x < NS) {
        landed[threadIdx.x] = 0;
        done[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) wait_fail = 0;
    __syncthreads();
    const bool full = ld.full_share();
    auto own_landed = [&]() {
        if constexpr (LD::kEven) {
            wait_vm<(A - 1) * LD::kPerWave>();
        } else {
            if (full) wait_vm<(A - 1) * LD::kPerWave>(); else wait_vm<0>();
        }
    };
    int j = 0;
    auto step = [&](const Job& cur, const Job& iss, const KVStage<D, JK>& cs, KVStage<D, JK>& is,
                    int* land_c, int* land_n, int* done_c, int* done_i) {
        const int jf = j + A - NS;
        if (jf >= 0) spin_ge(done_i, NW * (jf / NS + 1), &wait_fail);
        ld.issue(iss.j0, iss.ok, is);
        own_landed();
        signal(land_n, lane);
        spin_ge(land_c, NW * (j / NS + 1), &wait_fail);
        compute(cur, cs);
        signal(done_c, lane);
        ++j;
    };
    Job jc = first_job<BS, true>(ul);
    Job ji = jc;
    ld.issue(ji.j0, ji.ok, s0);
    ji = next_job_q<BS>(ji, ul, t_last);
    ld.issue(ji.j0, ji.ok, s1);
    ji = next_job_q<BS>(ji, ul, t_last);
    own_landed();
    signal(&landed[0], lane);
    while (jc.ok) {
        step(jc, ji, s0, s2, &landed[0], &landed[1], &done[0], &done[2]);
        jc = next_job_q<BS, true>(jc, ul, t_last);
        ji = next_job_q<BS>(ji, ul, t_last);
        if (!jc.ok) break;
        step(jc, ji, s1, s3, &landed[1], &landed[2], &done[1], &done[3]);
        jc = next_job_q<BS, true>(jc, ul, t_last);
        ji = next_job_q<BS>(ji, ul, t_last);
        if (!jc.ok) break;
        step(jc, ji, s2, s0, &landed[2], &landed[3], &done[2], &done[0]);
        jc = next_job_q<BS, true>(jc, ul, t_last);
        ji = next_job_q<BS>(ji, ul, t_last);
        if (!jc.ok) break;
        step(jc, ji, s3, s1, &landed[3], &landed[0], &done[3], &done[1]);
        jc = next_job_q<BS, true>(jc, ul, t_last);
        ji = next_job_q<BS>(ji, ul, t_last);
    }
    // Loads of job slots past the end finish before the wave leaves.
    wait_vm<0>();
    report_wait_timeouts(&wait_fail);
}

// The same walk with a workgroup barrier after every job, for the cases
// where most tiles work on most jobs, so the counters above only add
// waiting: selections that can cover whole causal prefixes (forward and
// dQ), and forward tiles of 4 or more tokens (G <= 4): job j is computed from stage j % 4 while
// the loads of job j + 3 go to stage (j + 3) % 4, last read by job j - 1
// (freed by the barrier that ended it); the end-of-job wait leaves the
// loads of jobs j + 2 and j + 3 in flight.
template <int D, int BS, int NW, class Compute>
__device__ __forceinline__ void q_ring_sync(const KVLoad<D, NW, JobKeys<BS>::JK>& ld,
                                            const UnionList& ul, int t_last, Compute&& compute) {
    constexpr int JK = JobKeys<BS>::JK;
    using LD = KVLoad<D, NW, JK>;
    static_assert(kQStages == 4, "the unrolled walk below is written for 4 stages");
    __shared__ KVStage<D, JK> s0, s1, s2, s3;
    const bool full = ld.full_share();
    auto ring_wait = [&]() {
        if constexpr (LD::kEven) {
            wait_vm_barrier<2 * LD::kPerWave>();
        } else {
            if (full) wait_vm_barrier<2 * LD::kPerWave>(); else wait_vm_barrier<0>();
        }
    };
    Job jc = first_job<BS, true>(ul);
    Job j1 = next_job_q<BS, true>(jc, ul, t_last);
    Job j2 = next_job_q<BS, true>(j1, ul, t_last);
    Job j3 = next_job_q<BS, true>(j2, ul, t_last);
    ld.issue(jc.j0, jc.ok, s0);
    ld.issue(j1.j0, j1.ok, s1);
    ld.issue(j2.j0, j2.ok, s2);
    if constexpr (LD::kEven) {
        wait_vm_barrier<2 * LD::kPerWave>();
    } else {
        if (full) wait_vm_barrier<2 * LD::kPerWave>(); else wait_vm_barrier<0>();
    }
    auto step = [&](const KVStage<D, JK>& cs, KVStage<D, JK>& is) {
        ld.issue(j3.j0, j3.ok, is);
        compute(jc, cs);
        ring_wait();
        jc = j1;
        j1 = j2;
        j2 = j3;
        j3 = next_job_q<BS, true>(j3, ul, t_last);
    };
    while (jc.ok) {
        step(s0, s3);
        if (!jc.ok) break;
        step(s1, s0);
        if (!jc.ok) break;
        step(s2, s1);
        if (!jc.ok) break;
        step(s3, s2);
    }
    // Loads of job slots past the end finish before the wave leaves.
    wait_vm_barrier<0>();
}

// Per-wave dS tiles of one job (JK keys x 16 heads, rows of 32 bytes), one
// per tile of the wave; two of these alternate between consecutive jobs.
template <int JK, int NW, int RT>
struct alignas(16) DsBuf {
    uint16_t v[NW][RT][JK * 16];
};

// The walk of q_ring for dQ from a handed-off dS: the ring holds K alone,
// and each wave also stages the dS tiles its tiles need, one job ahead, in
// two buffers of its own (job j in buffer j % 2).  In its step j a wave
//   1. issues the dS tiles of job j + 1 (buffer (j + 1) % 2, last read by its
//      own job j - 1);
//   2. waits until every wave finished job j + A - NS, then issues its share
//      of job j + A;
//   3. waits for its share of job j + 1 and its dS tiles of job j (issued in
//      step j - 1, before that share), counts landed;
//   4. waits until all shares of job j landed, computes job j, counts done.
// issue_ds returns the count of loads it issued (0, NDMA or 2 NDMA), which
// the wait in 3 leaves in flight with the ring's job j + A.
template <int D, int BS, int NW, int RT, class IssueDs, class Compute>
__device__ __forceinline__ void q_ring_ds(const KVLoad<D, NW, JobKeys<BS>::JK, true>& ld,
                                          const UnionList& ul, int t_last, int lane,
                                          IssueDs&& issue_ds, Compute&& compute) {
    constexpr int JK = JobKeys<BS>::JK, NS = kQStages, A = kQAhead, NDMA = JK / 32;
    using LD = KVLoad<D, NW, JK, true>;
    using DB = DsBuf<JK, NW, RT>;
    static_assert(NS == 4 && A == 2 && RT == 2, "the walk below is written for 4 stages, 2 ahead, 2 tiles");
    __shared__ KStage<D, JK> s0, s1, s2, s3;
    __shared__ DB d0, d1;
    __shared__ int landed[NS], done[NS], wait_fail;
    if (threadIdx.x < NS) {
        landed[threadIdx.x] = 0;
        done[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) wait_fail = 0;
    __syncthreads();
    const bool full = ld.full_share();
    // Everything but the ring's newest job and the newest dS tiles landed.
    auto own_landed = [&](int nds) {
        if (LD::kEven && full) {
            if (nds == 0) wait_vm<LD::kPerWave>();
            else if (nds == NDMA) wait_vm<LD::kPerWave + NDMA>();
            else wait_vm<LD::kPerWave + 2 * NDMA>();
        } else {
            wait_vm<0>();
        }
    };
    int j = 0;
    auto step = [&](const Job& cur, const Job& nxt, const Job& iss, const KStage<D, JK>& cs,
                    KStage<D, JK>& is, const DB& dc, DB& dn, int* land_c, int* land_n,
                    int* done_c, int* done_i) {
        const int nds = issue_ds(nxt, dn);
        const int jf = j + A - NS;
        if (jf >= 0) spin_ge(done_i, NW * (jf / NS + 1), &wait_fail);
        ld.issue(iss.j0, iss.ok, is);
        own_landed(nds);
        signal(land_n, lane);
        spin_ge(land_c, NW * (j / NS + 1), &wait_fail);
        compute(cur, cs, dc);
        signal(done_c, lane);
        ++j;
    };
    Job jc = first_job<BS>(ul);
    Job jn = next_job_q<BS>(jc, ul, t_last);
    Job ji = next_job_q<BS>(jn, ul, t_last);
    issue_ds(jc, d0);
    ld.issue(jc.j0, jc.ok, s0);
    ld.issue(jn.j0, jn.ok, s1);
    if (LD::kEven && full) wait_vm<LD::kPerWave>(); else wait_vm<0>();
    signal(&landed[0], lane);
    auto advance = [&]() {
        jc = jn;
        jn = ji;
        ji = next_job_q<BS>(ji, ul, t_last);
    };
    while (jc.ok) {
        step(jc, jn, ji, s0, s2, d0, d1, &landed[0], &landed[1], &done[0], &done[2]);
        advance();
        if (!jc.ok) break;
        step(jc, jn, ji, s1, s3, d1, d0, &landed[1], &landed[2], &done[1], &done[3]);
        advance();
        if (!jc.ok) break;
        step(jc, jn, ji, s2, s0, d0, d1, &landed[2], &landed[3], &done[2], &done[0]);
        advance();
        if (!jc.ok) break;
        step(jc, jn, ji, s3, s1, d1, d0, &landed[3], &landed[0], &done[3], &done[1]);
        advance();
    }
    // Loads of job slots past the end finish before the wave leaves.
    wait_vm<0>();
    report_wait_timeouts(&wait_fail);
}

}  // namespace

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, int BS, int RT, int NW, bool SYNC, bool WIN>
__global__ __launch_bounds__(NW * 64) void fwd_q_kernel(Problem p, QGeo qg,
                                                        const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const int* __restrict__ idx,
                                                        uint16_t* __restrict__ o,
                                                        float* __restrict__ lse) {
    using L = RowTile<D>;
    constexpr int KD = D / 32, ND = D / 16, JK = JobKeys<BS>::JK, NKT = JK / 16, NKS = JK / 32;
    constexpr int KT = JobKeys<BS>::KT;  // keys of the job inside its block
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned long long* umask = reinterpret_cast<unsigned long long*>(smem);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);
    int* n_u = reinterpret_cast<int*>(smem + QLds<D, JK>::dynamic_bytes(p.NBmax) - 16);

    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6),
              g = lane >> 4, r = lane & 15;
    const WgCoord wc = wg_coord(p, qg);
    const Seq s = seq_of(p, wc.z);
    if (wc.T0 >= s.len) return;
    const int n_tok = min(qg.TW, s.len - wc.T0);
    const int t_last = wc.T0 + n_tok - 1 + s.qoff;  // key position of the last query
    const int NBz = (s.klen + BS - 1) / BS;
    const int qoff = s.qoff;
    using LD = KVLoad<D, NW, JK>;
    LD ld;
    ld.init(w, lane, k + head_base(p.lk, s, wc.hkv), v + head_base(p.lv, s, wc.hkv),
            2 * p.lk.st, 2 * p.lv.st, s.klen);
    uint32_t a_off[KD], t_off[ND];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) a_off[kk] = L::a_off(lane, kk);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) t_off[dt] = L::t_off(lane, dt);

    // Per-tile state of this lane's row.
    TileRow tr[RT];
    uint64_t tmask[RT];
    bf16x8 qf[RT][KD];
    f32x4 acc[RT][ND];
    // Running max and sum per row; mc = the max in base-2 units, or 0 while
    // the row has seen no key (the exponent's offset, updated with m_run).
    float m_run[RT], l_run[RT], mc[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int tau = w * RT + i;
        tr[i] = tile_row(p, qg, wc.hkv, wc.T0, s.len, tau, r);
        tmask[i] = uniform64(tile_tokens(p, qg, tau));
        const uint16_t* qrow = q + row_off(p.lq, s, tr[i].h, tr[i].t) + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
            qf[i][kk] = tr[i].valid ? as_bf16x8(ldg16(qrow + 32 * kk)) : zero8();
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[i] = kNegInfQ;
        l_run[i] = 0.f;
        mc[i] = 0.f;
    }
    const int nU = wg_union(p, s, idx, wc.hkv, wc.T0, n_tok, NBz, umask, ulist, n_u);
    const float c2 = p.scale_log2;

    // Pieces of one tile's job.  K operands: all 16-key x 32-d slices of the
    // job, each lane's 16 bytes (A layout).
    using KOps = bf16x8[NKT][KD];
    auto read_k = [&](const uint8_t* ks, KOps& ka) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int kk = 0; kk < KD; ++kk)
                ka[kt][kk] = *reinterpret_cast<const bf16x8*>(ks + a_off[kk] + kt * 16 * L::RB);
    };
    // Transposed V operand of keys 32 ks_ .. 32 ks_ + 31 (the C layout of S
    // gave this lane keys 32ks + 4g + e and 32ks + 16 + 4g + e).
    auto read_v = [&](const uint8_t* vs, int ks_, bf16x8 (&vop)[ND]) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint8_t* vb0 = vs + t_off[dt] + 32 * ks_ * L::RB;
            const uint2 v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(vb0));
            const uint2 v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(vb0 + 16 * L::RB));
            vop[dt] = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        }
    };
    // Mask, online softmax (lazy rescale of tile i's O and l), P in bf16.
    auto softmax = [&](int i, f32x4 (&sc)[NKT], const Job& cur, uint64_t bm,
                       bf16x8 (&pb)[NKS]) __attribute__((always_inline)) {
        // No mask when every token of the tile lists the block, the slice
        // ends before the tile's first token, and all rows exist.
        const bool full = KT == JK && ((bm & tmask[i]) == tmask[i]) &&
                          (cur.j0 + JK - 1 <= tr[i].t + qoff - (tr[i].tok - (int)__builtin_ctzll(tmask[i]))) &&
                          tr[i].valid && (!WIN || cur.j0 > tr[i].t + qoff - p.window);
        // The mask overwrites masked scores in place (the no-mask path then
        // needs no copies of the scores where the two paths meet).
        if (!wave_all(full)) {
            const bool sel = tr[i].valid && ((bm >> tr[i].tok) & 1ull);
            // Key 16 kt + 4 g + e is masked past lim; compared as
            // 16 kt + e > lim - 4 g so the left side is a constant.
            const int lim = (sel ? tr[i].t + qoff - cur.j0 : -1) - 4 * g;
            // Sliding window: keys below t - window + 1 too (same form).
            const int lo = WIN ? tr[i].t + qoff - p.window + 1 - cur.j0 - 4 * g : 0;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * kt >= KT || 16 * kt + e > lim || (WIN && 16 * kt + e < lo))
                        sc[kt][e] = kNegInfQ;
        }
        // Row max of the lane's 4 NKT scores: a v_max3 chain.
        float mloc = vmax3(sc[0][0], sc[0][1], sc[0][2]);
#pragma unroll
        for (int x = 3; x + 1 < 4 * NKT; x += 2) mloc = vmax3(mloc, sc[x / 4][x % 4], sc[(x + 1) / 4][(x + 1) % 4]);
        if constexpr ((4 * NKT) % 2 == 0) mloc = vmax(mloc, sc[NKT - 1][3]);
        const float mblk = col_max4(mloc);
        const bool grow = mblk * c2 > m_run[i] * c2 + kLazyQ;
        if (wave_any(grow)) {
            const float m_new = grow ? mblk : m_run[i];
            const float alpha = grow ? fast_exp2((m_run[i] - m_new) * c2) : 1.f;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) acc[i][dt] *= alpha;
            l_run[i] *= alpha;
            m_run[i] = m_new;
            mc[i] = m_new == kNegInfQ ? 0.f : m_new * c2;
        }
        float lsum[4];
#pragma unroll
        for (int ks_ = 0; ks_ < NKS; ++ks_) {
            float p0[4], p1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p0[e] = fast_exp2(fmaf(sc[2 * ks_][e], c2, -mc[i]));
                p1[e] = fast_exp2(fmaf(sc[2 * ks_ + 1][e], c2, -mc[i]));
                lsum[e] = ks_ == 0 ? p0[e] + p1[e] : lsum[e] + (p0[e] + p1[e]);
            }
            pb[ks_] = pack8(p0, p1);
        }
        l_run[i] += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };

    // One job: for each tile whose tokens list the block, S^T = K Q^T (all
    // K operand reads in flight at once), the softmax, then O^T += V^T P^T
    // with the transposed V reads of each 32-key step issued together.  The
    // K operands die before the O step, which leaves the registers for that.
    auto compute = [&](const Job& cur, const KVStage<D, JK>& sg) {
        const uint8_t* ks = reinterpret_cast<const uint8_t*>(sg.k);
        const uint8_t* vs = reinterpret_cast<const uint8_t*>(sg.v);
        const uint64_t bm = cur.bm;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            if ((bm & tmask[i]) == 0ull) continue;
            f32x4 sc[NKT];
            {
                KOps ka;
                read_k(ks, ka);
                // All K reads are issued before the products (each into its
                // own registers), not one read per product.
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KD; ++kk) sc[kt] = mfma(ka[kt][kk], qf[i][kk], sc[kt]);
                }
            }
            // The transposed V reads of the first 32 keys go out while the
            // products run (they do not depend on the softmax).
            bf16x8 vop0[ND];
            read_v(vs, 0, vop0);
            bf16x8 pb[NKS];
            softmax(i, sc, cur, bm, pb);
#pragma unroll
            for (int ks_ = 0; ks_ < NKS; ++ks_) {
                bf16x8 vop[ND];
                if (ks_ == 0) {
#pragma unroll
                    for (int dt = 0; dt < ND; ++dt) vop[dt] = vop0[dt];
                } else {
                    read_v(vs, ks_, vop);
                }
#pragma unroll
                for (int dt = 0; dt < ND; ++dt) acc[i][dt] = mfma(vop[dt], pb[ks_], acc[i][dt]);
            }
        }
    };

    // The same job for both tiles of the wave at once (whole-prefix
    // selections, where every tile works on nearly every job): each K and V
    // operand read from LDS feeds both tiles' products, which halves the
    // LDS reads, and one tile's softmax overlaps the other's products.  A
    // tile none of whose tokens lists the block is masked out entirely.
    auto compute_pair = [&](const Job& cur, const KVStage<D, JK>& sg) {
        static_assert(RT == 2, "two tiles per wave");
        const uint8_t* ks = reinterpret_cast<const uint8_t*>(sg.k);
        const uint8_t* vs = reinterpret_cast<const uint8_t*>(sg.v);
        const uint64_t bm = cur.bm;
        // Neither tile's tokens list the block (or both tiles are idle: past
        // the workgroup's tokens when G < 4): nothing to compute.  Loads and
        // barriers happen outside, so leaving early is safe.
        if ((bm & (tmask[0] | tmask[1])) == 0ull) return;
        f32x4 sc0[NKT], sc1[NKT];
        {
            KOps ka;
            read_k(ks, ka);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                sc0[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                sc1[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    sc0[kt] = mfma(ka[kt][kk], qf[0][kk], sc0[kt]);
                    sc1[kt] = mfma(ka[kt][kk], qf[1][kk], sc1[kt]);
                }
            }
        }
        bf16x8 vop0[ND];
        read_v(vs, 0, vop0);
        bf16x8 pb0[NKS], pb1[NKS];
        softmax(0, sc0, cur, bm, pb0);
        softmax(1, sc1, cur, bm, pb1);
#pragma unroll
        for (int ks_ = 0; ks_ < NKS; ++ks_) {
            bf16x8 vop[ND];
            if (ks_ == 0) {
#pragma unroll
                for (int dt = 0; dt < ND; ++dt) vop[dt] = vop0[dt];
            } else {
                read_v(vs, ks_, vop);
            }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                acc[0][dt] = mfma(vop[dt], pb0[ks_], acc[0][dt]);
                acc[1][dt] = mfma(vop[dt], pb1[ks_], acc[1][dt]);
            }
        }
    };

    if constexpr (SYNC) {
        q_ring_sync<D, BS, NW>(ld, UnionList{ulist, umask, nU}, t_last, compute_pair);
    } else {
        q_ring<D, BS, NW>(ld, UnionList{ulist, umask, nU}, t_last, lane, compute);
    }

#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const float l_tot = col_sum4(l_run[i]);
        float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float lse_r = l_tot > 0.f ? (m_run[i] * c2 + fast_log2(l_tot)) * kLn2 : kNegInfQ;
        if (p.sink) finish_row_sink(p.sink[tr[i].h], m_run[i] * c2, l_tot, inv, lse_r);
        if (tr[i].valid) {
            uint16_t* orow = o + row_off(p.lo, s, tr[i].h, tr[i].t) + 4 * g;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const uint2 pk = make_uint2(pack_bf16x2(acc[i][dt][0] * inv, acc[i][dt][1] * inv),
                                            pack_bf16x2(acc[i][dt][2] * inv, acc[i][dt][3] * inv));
                *reinterpret_cast<uint2*>(orow + 16 * dt) = pk;
            }
            if (g == 0) lse[l_off(p, s, tr[i].h, tr[i].t)] = lse_r;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int BS, int RT, int NW, bool SYNC, bool WIN>
__global__ __launch_bounds__(NW * 64) void dq_q_kernel(
    Problem p, QGeo qg, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, const int* __restrict__ idx, uint16_t* __restrict__ dq) {
    using L = RowTile<D>;
    constexpr int KD = D / 32, ND = D / 16, JK = JobKeys<BS>::JK, NKT = JK / 16, NKS = JK / 32;
    constexpr int KT = JobKeys<BS>::KT;  // keys of the job inside its block
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned long long* umask = reinterpret_cast<unsigned long long*>(smem);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);
    int* n_u = reinterpret_cast<int*>(smem + QLds<D, JK>::dynamic_bytes(p.NBmax) - 16);

    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), g = lane >> 4, r = lane & 15;
    const WgCoord wc = wg_coord(p, qg);
    const Seq s = seq_of(p, wc.z);
    if (wc.T0 >= s.len) return;
    const int n_tok = min(qg.TW, s.len - wc.T0);
    const int t_last = wc.T0 + n_tok - 1 + s.qoff;  // key position of the last query
    const int NBz = (s.klen + BS - 1) / BS;
    const int qoff = s.qoff;
    using LD = KVLoad<D, NW, JK>;
    LD ld;
    ld.init(w, lane, k + head_base(p.lk, s, wc.hkv), v + head_base(p.lv, s, wc.hkv),
            2 * p.lk.st, 2 * p.lv.st, s.klen);
    uint32_t a_off[KD], t_off[ND];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) a_off[kk] = L::a_off(lane, kk);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) t_off[dt] = L::t_off(lane, dt);

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
        const uint16_t* qrow = q + row_off(p.lq, s, tr[i].h, tr[i].t) + 8 * g;
        const uint16_t* drow = dO + row_off(p.ldo, s, tr[i].h, tr[i].t) + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
            qf[i][kk] = tr[i].valid ? as_bf16x8(ldg16(qrow + 32 * kk)) : zero8();
            df[i][kk] = tr[i].valid ? as_bf16x8(ldg16(drow + 32 * kk)) : zero8();
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

    // Pieces of one tile's job.  Mask of S^T (-inf outside the tile's
    // selection and causal range), then dS = P (dP - Delta) in bf16.
    auto dscore = [&](int i, f32x4 (&sc)[NKT], const f32x4 (&dp)[NKT], const Job& cur, uint64_t bm,
                      bf16x8 (&dsb)[NKS]) __attribute__((always_inline)) {
        const bool full = KT == JK && ((bm & tmask[i]) == tmask[i]) &&
                          (cur.j0 + JK - 1 <= tr[i].t + qoff - (tr[i].tok - (int)__builtin_ctzll(tmask[i]))) &&
                          tr[i].valid && (!WIN || cur.j0 > tr[i].t + qoff - p.window);
        if (!__builtin_amdgcn_readfirstlane((int)__all(full))) {
            const bool sel = tr[i].valid && ((bm >> tr[i].tok) & 1ull);
            // Key 16 kt + 4 g + e is masked past lim (constant left side).
            const int lim = (sel ? tr[i].t + qoff - cur.j0 : -1) - 4 * g;
            const int lo = WIN ? tr[i].t + qoff - p.window + 1 - cur.j0 - 4 * g : 0;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * kt >= KT || 16 * kt + e > lim || (WIN && 16 * kt + e < lo))
                        sc[kt][e] = kNegInfQ;
        }
#pragma unroll
        for (int ks_ = 0; ks_ < NKS; ++ks_) {
            float d0[4], d1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d0[e] = fast_exp2(fmaf(sc[2 * ks_][e], c2, nlse2[i])) * (dp[2 * ks_][e] - dl[i]);
                d1[e] = fast_exp2(fmaf(sc[2 * ks_ + 1][e], c2, nlse2[i])) * (dp[2 * ks_ + 1][e] - dl[i]);
            }
            dsb[ks_] = pack8(d0, d1);
        }
    };
    // Transposed K operand of keys 32 ks_ .. 32 ks_ + 31 for dQ^T += K^T dS^T.
    auto read_kt = [&](const uint8_t* ks, int ks_, bf16x8 (&kop)[ND]) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint8_t* kb0 = ks + t_off[dt] + 32 * ks_ * L::RB;
            const uint2 k0 = lds_read_tr(reinterpret_cast<const uint16_t*>(kb0));
            const uint2 k1 = lds_read_tr(reinterpret_cast<const uint16_t*>(kb0 + 16 * L::RB));
            kop[dt] = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
        }
    };

    // One job: for each tile whose tokens list the block, S^T = K Q^T and
    // dP^T = V dO^T (all K and V operand reads in flight at once), dS, then
    // dQ^T += K^T dS^T with the transposed K reads of each 32-key step issued
    // together.
    auto compute = [&](const Job& cur, const KVStage<D, JK>& sg) {
        const uint8_t* ks = reinterpret_cast<const uint8_t*>(sg.k);
        const uint8_t* vs = reinterpret_cast<const uint8_t*>(sg.v);
        const uint64_t bm = cur.bm;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            if (!__builtin_amdgcn_readfirstlane((int)((bm & tmask[i]) != 0ull))) continue;
            f32x4 sc[NKT], dp[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                bf16x8 ka[KD], va[KD];
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    ka[kk] = *reinterpret_cast<const bf16x8*>(ks + a_off[kk] + kt * 16 * L::RB);
                    va[kk] = *reinterpret_cast<const bf16x8*>(vs + a_off[kk] + kt * 16 * L::RB);
                }
                // The step's K and V reads are all issued before its products.
                __builtin_amdgcn_sched_barrier(0);
                sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KD; ++kk) {
                    sc[kt] = mfma(ka[kk], qf[i][kk], sc[kt]);
                    dp[kt] = mfma(va[kk], df[i][kk], dp[kt]);
                }
            }
            bf16x8 dsb[NKS];
            dscore(i, sc, dp, cur, bm, dsb);
            // dQ^T += K^T dS^T, 32 keys per step.
#pragma unroll
            for (int ks_ = 0; ks_ < NKS; ++ks_) {
                bf16x8 kop[ND];
                read_kt(ks, ks_, kop);
#pragma unroll
                for (int dt = 0; dt < ND; ++dt) acc[i][dt] = mfma(kop[dt], dsb[ks_], acc[i][dt]);
            }
        }
    };

    if constexpr (SYNC) {
        q_ring_sync<D, BS, NW>(ld, UnionList{ulist, umask, nU}, t_last, compute);
    } else {
        q_ring<D, BS, NW>(ld, UnionList{ulist, umask, nU}, t_last, lane, compute);
    }

#pragma unroll
    for (int i = 0; i < RT; ++i) {
        if (!tr[i].valid) continue;
        uint16_t* drow = dq + row_off(p.ldq, s, tr[i].h, tr[i].t) + 4 * g;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint2 pk = make_uint2(pack_bf16x2(acc[i][dt][0] * p.scale, acc[i][dt][1] * p.scale),
                                        pack_bf16x2(acc[i][dt][2] * p.scale, acc[i][dt][3] * p.scale));
            *reinterpret_cast<uint2*>(drow + 16 * dt) = pk;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ from the dS that the dK/dV kernel hands off
// ---------------------------------------------------------------------------
// The dK/dV kernel forms dS = P (dP - Delta) for every listed (row, key) pair
// and, for these problems, also stores it (bf16):
//   ds [entry][key in block][head of the group], entry = region_base of the
//       (z, hkv) + the (token, block) listing's position in the block's list;
//   posmap [block_idx row][slot] = that entry for the slot standing for a
//       listed block (its first occurrence in the row), else -1.
// Then dQ needs no second pass over S and dP: dq = scale sum over the row's
// listed blocks of dS K, one product (2 D flops per pair instead of 6 D) and
// no q, dO, lse or Delta reads.  The walk is the dQ kernel's (16-row tiles,
// the union of the workgroup's listed blocks in ascending order, K shared
// through an LDS ring); per job, each tile one of whose tokens lists the
// block takes its dS tile (staged by buffer-to-LDS loads, zeros for the
// tile's tokens that do not list it, read transposed as the B operand) and
// adds K^T dS^T.  TPT = tokens per tile: 1 (16 heads of one token, G a
// multiple of 16), 2 (G = 8) or 4 (G = 4).  dS tile in LDS, 32 bytes per
// key: [key][16 tile rows] for TPT <= 2; for TPT = 4 [key pair][token]
// [key of the pair][4 heads], so that one 16-byte load holds two keys of
// one token (8 contiguous bytes per key in ds).  block_size >= 32, S <= 64,
// no sliding window, and a (z, hkv) region of ds spans < 2^31 bytes.
// Byte of (key, heads 4 col4 .. + 3) in a TPT = 4 dS tile.
__device__ __forceinline__ uint32_t ds_tile_byte(int key, int col4) {
    return (uint32_t)((((key >> 1) * 4 + col4) * 16) + (key & 1) * 8);
}

// The dQ of one (window, group) work item b of nb (its place in the launch
// order of wg_coord).
template <int D, int BS, int RT, int NW, int TPT>
__device__ __forceinline__ void dq_ds_item(const Problem& p, const QGeo& qg,
                                           const uint16_t* __restrict__ k,
                                           const int* __restrict__ idx,
                                           const int* __restrict__ posmap,
                                           const uint16_t* __restrict__ ds,
                                           uint16_t* __restrict__ dq, int b, int nb) {
    using L = RowTile<D>;
    constexpr int ND = D / 16, JK = JobKeys<BS>::JK, NKS = JK / 32, NDMA = JK / 32;
    static_assert(BS >= 32 && JobKeys<BS>::KT == JK, "whole 32-key steps of one block");
    static_assert(TPT == 1 || TPT == 2 || TPT == 4, "tokens per tile");
    using DB = DsBuf<JK, NW, RT>;
    constexpr uint32_t kOob = 0xFFFFFFF0u;  // past the region descriptor (2^31 bytes): loads zeros
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned long long* umask = reinterpret_cast<unsigned long long*>(smem);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(umask + p.NBmax);
    int* n_u = reinterpret_cast<int*>(smem + QLds<D, JK>::dynamic_bytes(p.NBmax) - 16);

    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6),
              g = lane >> 4, r = lane & 15;
    const WgCoord wc = wg_coord(p, qg, b, nb);
    const Seq s = seq_of(p, wc.z);
    if (wc.T0 >= s.len) return;
    const int n_tok = min(qg.TW, s.len - wc.T0);
    const int t_last = wc.T0 + n_tok - 1 + s.qoff;  // key position of the last query
    const int NBz = (s.klen + BS - 1) / BS;
    using LD = KVLoad<D, NW, JK, true>;
    LD ld;
    const uint16_t* kb = k + head_base(p.lk, s, wc.hkv);
    ld.init(w, lane, kb, kb, 2 * p.lk.st, 2 * p.lk.st, s.klen);
    uint32_t t_off[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) t_off[dt] = L::t_off(lane, dt);

    // Per tile and token: the token's block list and list positions (lane x
    // holds slot x); per tile its first head inside the group and its
    // accumulators.
    const int* rows = idx_row(p, s, idx, wc.hkv, wc.T0);
    const int* prows = posmap + (rows - idx);
    int u_l[RT][TPT], pos_l[RT][TPT], h0[RT];
    f32x4 acc[RT][ND];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int tau = w * RT + i;
        h0[i] = TPT == 1 ? 16 * (tau % qg.n_ht) : 0;
#pragma unroll
        for (int a = 0; a < TPT; ++a) {
            const int tok = TPT == 1 ? tau / qg.n_ht : tau * TPT + a;
            const bool have = tok < qg.TW && wc.T0 + tok < s.len && lane < p.S;
            u_l[i][a] = have ? rows[tok * p.S + lane] : -1;
            pos_l[i][a] = have ? prows[tok * p.S + lane] : -1;
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int nU = wg_union(p, s, idx, wc.hkv, wc.T0, n_tok, NBz, umask, ulist, n_u);

    // One descriptor over the (z, hkv) region of ds; a lane's offset selects
    // its token's entry.  Lane l of 1 KB load jd fills tile bytes 1024 jd +
    // 16 l: key 32 jd + l / 2, heads h0 + 8 (l % 2) (TPT 1); key 32 jd + l / 2
    // of token l % 2 (TPT 2); keys 32 jd + 2 (l / 4) + {0, 1} of token l % 4
    // (TPT 4).
    const buf_rsrc rs = make_rsrc(ds + region_base(p, s, wc.hkv) * BS * p.G, 0x80000000u);
    const int my_tok = TPT == 1 ? 0 : (lane & (TPT - 1));
    const int my_key = TPT == 4 ? 2 * (lane >> 2) : (lane >> 1);
    const int my_head = TPT == 1 ? 8 * (lane & 1) : 0;
    // Entry of tile i's token a for block u (-1: it does not list u); all
    // wave-uniform.
    auto listing = [&](int i, int a, int u) __attribute__((always_inline)) -> uint64_t {
        return __ballot(u_l[i][a] == u && pos_l[i][a] >= 0);
    };
    auto entry = [&](int i, int a, int u) __attribute__((always_inline)) -> int {
        const uint64_t m = listing(i, a, u);
        return m ? __builtin_amdgcn_readlane(pos_l[i][a], (int)__builtin_ctzll(m)) : -1;
    };
    // One token per tile: a descriptor per dS tile, fixed lane offsets.
    const int64_t ds_base = region_base(p, s, wc.hkv);
    const uint32_t lane_off = (uint32_t)((my_key * p.G + my_head) * 2);
    auto issue_ds = [&](const Job& jb, DB& buf) __attribute__((always_inline)) -> int {
        if (!jb.ok) return 0;
        const int kofs = jb.j0 - jb.u * BS;
        int n = 0;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            if constexpr (TPT == 1) {
                const uint64_t m = listing(i, 0, jb.u);
                if (!m) continue;
                const int e0 = __builtin_amdgcn_readlane(pos_l[i][0], (int)__builtin_ctzll(m));
                const buf_rsrc rt = make_rsrc(ds + ((ds_base + e0) * BS + kofs) * p.G + h0[i],
                                              (uint32_t)((JK - 1) * p.G * 2 + 32));
#pragma unroll
                for (int jd = 0; jd < NDMA; ++jd)
                    dma16(rt, reinterpret_cast<uint8_t*>(buf.v[w][i]) + 1024 * jd,
                          lane_off + (uint32_t)(32 * jd * p.G * 2));
                n += NDMA;
                continue;
            }
            int e[TPT];
            bool any = false;
#pragma unroll
            for (int a = 0; a < TPT; ++a) {
                e[a] = entry(i, a, jb.u);
                any = any || e[a] >= 0;
            }
            if (!any) continue;
            int mine = e[0];
#pragma unroll
            for (int a = 1; a < TPT; ++a) mine = my_tok == a ? e[a] : mine;
#pragma unroll
            for (int jd = 0; jd < NDMA; ++jd) {
                const uint32_t off =
                    mine < 0 ? kOob
                             : (uint32_t)(((mine * BS + kofs + 32 * jd + my_key) * p.G + h0[i] + my_head) * 2);
                dma16(rs, reinterpret_cast<uint8_t*>(buf.v[w][i]) + 1024 * jd, off);
            }
            n += NDMA;
        }
        return n;
    };
    // dQ^T += K^T dS^T for the tiles one of whose tokens lists the job's
    // block: the transposed K operand of each 32-key step is read once for
    // both tiles.
    const int q4 = r >> 2, c4 = r & 3;  // (TPT = 4 tile reads)
    auto compute = [&](const Job& cur, const KStage<D, JK>& sg, const DB& buf) {
        bool act[RT];
        bool any = false;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            act[i] = false;
#pragma unroll
            for (int a = 0; a < TPT; ++a) act[i] = act[i] || listing(i, a, cur.u) != 0ull;
            any = any || act[i];
        }
        if (!any) return;
        const uint8_t* ks = reinterpret_cast<const uint8_t*>(sg.k);
        auto read_kop = [&](int ks_, bf16x8 (&kop)[ND]) __attribute__((always_inline)) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const uint8_t* kb0 = ks + t_off[dt] + 32 * ks_ * L::RB;
                const uint2 k0 = lds_read_tr(reinterpret_cast<const uint16_t*>(kb0));
                const uint2 k1 = lds_read_tr(reinterpret_cast<const uint16_t*>(kb0 + 16 * L::RB));
                kop[dt] = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
            }
        };
        // B operand dS^T[keys 32 ks_ + 4 g + e, 32 ks_ + 16 + 4 g + e][row r]
        // of tile i: the key order of the transposed K reads.
        auto read_bop = [&](int ks_, int i) __attribute__((always_inline)) -> bf16x8 {
            if constexpr (TPT == 4) {
                const uint8_t* tb = reinterpret_cast<const uint8_t*>(buf.v[w][i]);
                const int klo = 32 * ks_ + 4 * g + q4;
                const uint2 lo = lds_read_tr(reinterpret_cast<const uint16_t*>(tb + ds_tile_byte(klo, c4)));
                const uint2 hi = lds_read_tr(reinterpret_cast<const uint16_t*>(tb + ds_tile_byte(klo + 16, c4)));
                return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
            } else {
                return lds_col_operand(buf.v[w][i], 16, 32 * ks_, 32 * ks_ + 16, 0, lane);
            }
        };
        if constexpr (TPT == 1) {
            // All of the job's operand reads in flight at once, then the
            // products (each accumulator still takes the 32-key steps in
            // order).  Measured 5 % faster here; with 4 tokens per tile the
            // extra registers slowed the dK/dV reduce that runs beside it.
            bf16x8 kop[NKS][ND], bop[NKS][RT];
#pragma unroll
            for (int ks_ = 0; ks_ < NKS; ++ks_) {
                read_kop(ks_, kop[ks_]);
#pragma unroll
                for (int i = 0; i < RT; ++i) bop[ks_][i] = read_bop(ks_, i);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                if (!act[i]) continue;
#pragma unroll
                for (int ks_ = 0; ks_ < NKS; ++ks_)
#pragma unroll
                    for (int dt = 0; dt < ND; ++dt) acc[i][dt] = mfma(kop[ks_][dt], bop[ks_][i], acc[i][dt]);
            }
        } else {
#pragma unroll
            for (int ks_ = 0; ks_ < NKS; ++ks_) {
                bf16x8 kop[ND];
                read_kop(ks_, kop);
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    if (!act[i]) continue;
                    const bf16x8 bop = read_bop(ks_, i);
#pragma unroll
                    for (int dt = 0; dt < ND; ++dt) acc[i][dt] = mfma(kop[dt], bop, acc[i][dt]);
                }
            }
        }
    };

    q_ring_ds<D, BS, NW, RT>(ld, UnionList{ulist, umask, nU}, t_last, lane, issue_ds, compute);

#pragma unroll
    for (int i = 0; i < RT; ++i) {
        int h, t;
        if constexpr (TPT == 1) {
            // 16 heads of one token (the tile's head range lies inside G)
            const int tok = (w * RT + i) / qg.n_ht;
            if (tok >= qg.TW || wc.T0 + tok >= s.len) continue;
            h = wc.hkv * p.G + h0[i] + r;
            t = wc.T0 + tok;
        } else {
            const TileRow trw = tile_row(p, qg, wc.hkv, wc.T0, s.len, w * RT + i, r);
            if (!trw.valid) continue;
            h = trw.h;
            t = trw.t;
        }
        uint16_t* drow = dq + row_off(p.ldq, s, h, t) + 4 * g;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint2 pk = make_uint2(pack_bf16x2(acc[i][dt][0] * p.scale, acc[i][dt][1] * p.scale),
                                        pack_bf16x2(acc[i][dt][2] * p.scale, acc[i][dt][3] * p.scale));
            *reinterpret_cast<uint2*>(drow + 16 * dt) = pk;
        }
    }
}

// One workgroup per work item, in the launch order of wg_coord (latest
// token windows first); the hardware dispatcher deals them out greedily.
template <int D, int BS, int RT, int NW, int TPT>
__global__ __launch_bounds__(NW * 64) void dq_ds_kernel(Problem p, QGeo qg,
                                                        const uint16_t* __restrict__ k,
                                                        const int* __restrict__ idx,
                                                        const int* __restrict__ posmap,
                                                        const uint16_t* __restrict__ ds,
                                                        uint16_t* __restrict__ dq) {
    dq_ds_item<D, BS, RT, NW, TPT>(p, qg, k, idx, posmap, ds, dq, (int)blockIdx.x, (int)gridDim.x);
}

// Persistent form (scheduling policy 1): a grid of at most one workgroup per
// CU, each taking the next item of the same longest-first order from the
// counter sched[0] until none is left; every item is still one workgroup's
// alone, so the result is the same bit for bit.  The prepare stage zeroes
// sched[0..1]; the last workgroup to leave zeroes them again, so that a dQ
// stage run twice after one prepare also starts from zero.  Every
// workgroup leaves once the counter has passed n_items.
template <int D, int BS, int RT, int NW, int TPT>
__global__ __launch_bounds__(NW * 64) void dq_ds_persistent(Problem p, QGeo qg,
                                                            const uint16_t* __restrict__ k,
                                                            const int* __restrict__ idx,
                                                            const int* __restrict__ posmap,
                                                            const uint16_t* __restrict__ ds,
                                                            uint16_t* __restrict__ dq,
                                                            int* __restrict__ sched, int n_items) {
    __shared__ int item_s;
    for (;;) {
        if (threadIdx.x == 0) item_s = atomicAdd(&sched[0], 1);
        __syncthreads();
        const int item = item_s;
        __syncthreads();
        if (item >= n_items) break;
        dq_ds_item<D, BS, RT, NW, TPT>(p, qg, k, idx, posmap, ds, dq, item, n_items);
        // The next item rebuilds the union and reuses the ring's LDS.
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        __threadfence();
        if (atomicAdd(&sched[1], 1) == (int)gridDim.x - 1) {
            atomicExch(&sched[0], 0);
            atomicExch(&sched[1], 0);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {
// Tiles per wave and waves per workgroup (16 tiles per workgroup).
constexpr int kRT_F = 2, kNW_F = 8;
constexpr int kRT_Q = 2, kNW_Q = 8;

QGeo q_geo(const HostProblem& hp, int kRT, int kNW) {
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
        case 32: return (hp.dev.bs >= 64 ? QLds<32, 64>::kStatic : QLds<32, 32>::kStatic) + QLds<32, 32>::dynamic_bytes(hp.dev.NBmax);
        case 64: return (hp.dev.bs >= 64 ? QLds<64, 64>::kStatic : QLds<64, 32>::kStatic) + QLds<64, 32>::dynamic_bytes(hp.dev.NBmax);
        case 128: return (hp.dev.bs >= 64 ? QLds<128, 64>::kStatic : QLds<128, 32>::kStatic) + QLds<128, 32>::dynamic_bytes(hp.dev.NBmax);
    }
    return 0;
}

namespace {
size_t query_dynamic_lds(const HostProblem& hp) {
    switch (hp.dev.D) {
        case 32: return QLds<32, 32>::dynamic_bytes(hp.dev.NBmax);
        case 64: return QLds<64, 32>::dynamic_bytes(hp.dev.NBmax);
        case 128: return QLds<128, 32>::dynamic_bytes(hp.dev.NBmax);
    }
    return 0;
}
}  // namespace

// Waves actually holding tiles (tiles beyond TW*tiles-per-token are idle but
// still take part in staging).
#define NSA_Q_DISPATCH(D_, BS_, CALL)                                                      \
    do {                                                                                   \
        if ((D_) == 32 && (BS_) == 16) { constexpr int D = 32, BS = 16; CALL; }            \
        else if ((D_) == 64 && (BS_) == 16) { constexpr int D = 64, BS = 16; CALL; }       \
        else if ((D_) == 128 && (BS_) == 16) { constexpr int D = 128, BS = 16; CALL; }     \
        else if ((D_) == 32 && (BS_) == 32) { constexpr int D = 32, BS = 32; CALL; }       \
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

// The barrier-per-job walk when the selection can cover a token's whole
// causal prefix (S block_size >= max length): then every tile works on
// nearly every job.
static bool q_sync(const HostProblem& hp) {
    return (int64_t)hp.dev.S * hp.dev.bs >= (int64_t)hp.dev.Tmax;
}

// The forward also takes the barrier walk when a tile holds 4 or more tokens
// (G <= 4): a tile then needs most of its workgroup's jobs even on sparse
// lists, and a barrier per job costs less than the counters (8 packed
// sequences, 32 / 8 heads, 16 blocks per row: forward 0.364 -> 0.345 ms; with
// 16 heads per tile, one token, the barrier walk took 0.346 -> 0.641 ms).
// dQ measured the same either way and keeps the counters.
static bool fwd_sync(const HostProblem& hp) {
    return q_sync(hp) || hp.dev.G <= 4;
}

hipError_t launch_fwd_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                           const int* block_idx, void* o, float* lse, hipStream_t st) {
    const QGeo qg = q_geo(hp, kRT_F, kNW_F);
    const unsigned grid = (unsigned)((int64_t)hp.ZH * qg.wg_per_zh);
    if (grid == 0) return hipSuccess;
    const size_t lds = query_dynamic_lds(hp);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kNW_F * 64), lds, st, hp.dev, qg,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, block_idx,
                           (uint16_t*)o, lse);
    };
    const bool win = hp.dev.window > 0;
    NSA_Q_DISPATCH(hp.dev.D, hp.dev.bs,
                   if (fwd_sync(hp)) {
                       if (win) go(fwd_q_kernel<D, BS, kRT_F, kNW_F, true, true>);
                       else go(fwd_q_kernel<D, BS, kRT_F, kNW_F, true, false>);
                   } else {
                       if (win) go(fwd_q_kernel<D, BS, kRT_F, kNW_F, false, true>);
                       else go(fwd_q_kernel<D, BS, kRT_F, kNW_F, false, false>);
                   });
    return hipGetLastError();
}

hipError_t launch_dq_bf16(const HostProblem& hp, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const float* delta,
                          const int* block_idx, void* dq, hipStream_t st) {
    const QGeo qg = q_geo(hp, kRT_Q, kNW_Q);
    const unsigned grid = (unsigned)((int64_t)hp.ZH * qg.wg_per_zh);
    if (grid == 0) return hipSuccess;
    const size_t lds = query_dynamic_lds(hp);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kNW_Q * 64), lds, st, hp.dev, qg,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           (const uint16_t*)dO, lse, delta, block_idx, (uint16_t*)dq);
    };
    const bool win = hp.dev.window > 0;
    NSA_Q_DISPATCH(hp.dev.D, hp.dev.bs,
                   if (q_sync(hp)) {
                       if (win) go(dq_q_kernel<D, BS, kRT_Q, kNW_Q, true, true>);
                       else go(dq_q_kernel<D, BS, kRT_Q, kNW_Q, true, false>);
                   } else {
                       if (win) go(dq_q_kernel<D, BS, kRT_Q, kNW_Q, false, true>);
                       else go(dq_q_kernel<D, BS, kRT_Q, kNW_Q, false, false>);
                   });
    return hipGetLastError();
}

// LDS of the hand-off dQ kernel: the K ring, the dS buffers, the counters
// and the union.
size_t dq_ds_lds_bytes(const HostProblem& hp) {
    const size_t JK = hp.dev.bs >= 64 ? 64 : 32;
    return 4 * JK * hp.dev.D * 2 + 2 * (size_t)kNW_Q * kRT_Q * JK * 32 + 64 + query_dynamic_lds(hp);
}

hipError_t launch_dq_handoff(const HostProblem& hp, const void* k, const int* block_idx,
                             const BwdWorkspace& ws, void* dq, hipStream_t st) {
    const QGeo qg = q_geo(hp, kRT_Q, kNW_Q);
    const int64_t n_items = (int64_t)hp.ZH * qg.wg_per_zh;
    if (n_items == 0) return hipSuccess;
    const size_t lds = query_dynamic_lds(hp);
    unsigned pgrid = 0;  // persistent grid: one workgroup per CU (LDS allows no more)
    if (hp.sched == 1) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        pgrid = (unsigned)std::min<int64_t>(n_items, std::max(cus, 1));
    }
    auto go = [&](auto kernel, auto persistent) {
        if (pgrid)
            hipLaunchKernelGGL(persistent, dim3(pgrid), dim3(kNW_Q * 64), lds, st, hp.dev, qg,
                               (const uint16_t*)k, block_idx, (const int*)ws.posmap,
                               (const uint16_t*)ws.ds, (uint16_t*)dq, ws.ticket + 1, (int)n_items);
        else
            hipLaunchKernelGGL(kernel, dim3((unsigned)n_items), dim3(kNW_Q * 64), lds, st, hp.dev, qg,
                               (const uint16_t*)k, block_idx, (const int*)ws.posmap,
                               (const uint16_t*)ws.ds, (uint16_t*)dq);
    };
    const int D = hp.dev.D, BS = hp.dev.bs, G = hp.dev.G;
    const int tpt = G % 16 == 0 ? 1 : G == 8 ? 2 : G == 4 ? 4 : 0;
#define NSA_DQ_DS(D_, BS_)                                                                      \
    else if (D == D_ && BS == BS_) {                                                            \
        if (tpt == 1) go(dq_ds_kernel<D_, BS_, kRT_Q, kNW_Q, 1>,                                \
                         dq_ds_persistent<D_, BS_, kRT_Q, kNW_Q, 1>);                           \
        else if (tpt == 2) go(dq_ds_kernel<D_, BS_, kRT_Q, kNW_Q, 2>,                           \
                              dq_ds_persistent<D_, BS_, kRT_Q, kNW_Q, 2>);                      \
        else if (tpt == 4) go(dq_ds_kernel<D_, BS_, kRT_Q, kNW_Q, 4>,                           \
                              dq_ds_persistent<D_, BS_, kRT_Q, kNW_Q, 4>);                      \
        else return hipErrorInvalidValue;                                                       \
    }
    if (false) {}
    NSA_DQ_DS(32, 32) NSA_DQ_DS(32, 64) NSA_DQ_DS(32, 128)
    NSA_DQ_DS(64, 32) NSA_DQ_DS(64, 64) NSA_DQ_DS(64, 128)
    NSA_DQ_DS(128, 32) NSA_DQ_DS(128, 64) NSA_DQ_DS(128, 128)
    else return hipErrorInvalidValue;
#undef NSA_DQ_DS
    return hipGetLastError();
}

// Bounded waits of this file's kernels that gave up (see spin_ge).
hipError_t read_wait_timeouts_query(unsigned* out) {
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(g_wait_timeouts), sizeof(unsigned), 0,
                               hipMemcpyDeviceToHost);
}

}  // namespace nsa
