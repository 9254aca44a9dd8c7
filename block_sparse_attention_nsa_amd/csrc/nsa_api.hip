// nsa_api.hip -- the C ABI declared in include/nsa_sel.h: argument checks
// (all on the host, before any HIP call), workspace carving and the ordered
// launch of the kernels on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "nsa_internal.h"
#include "nsa_sel.h"

namespace {

thread_local std::string g_last_error;

nsa_status fail(nsa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

nsa_status hip_fail(hipError_t e, const char* what) {
    return fail(NSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool misaligned(const void* ptr, size_t a) { return ((uintptr_t)ptr) % a != 0; }

// Validates the problem and fills the host/device descriptions.
nsa_status make_problem(const nsa_sel_problem* p, nsa::HostProblem& hp) {
    if (!p) return fail(NSA_ERR_INVALID_ARG, "problem pointer is NULL");
    if (p->layout != NSA_DENSE && p->layout != NSA_PACKED)
        return fail(NSA_ERR_INVALID_ARG, "layout %d is not NSA_DENSE or NSA_PACKED", p->layout);
    const bool packed = p->layout == NSA_PACKED;
    if (p->dtype != NSA_F32 && p->dtype != NSA_BF16)
        return fail(NSA_ERR_INVALID_ARG, "dtype %d is not NSA_F32 or NSA_BF16", p->dtype);
    if (p->B < 0 || p->T < 0) return fail(NSA_ERR_INVALID_ARG, "B=%d and T=%d must be >= 0", p->B, p->T);
    if (p->Hq < 1 || p->Hkv < 1) return fail(NSA_ERR_INVALID_ARG, "Hq=%d and Hkv=%d must be >= 1", p->Hq, p->Hkv);
    if (p->Hq % p->Hkv) return fail(NSA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
    if (p->D < 1) return fail(NSA_ERR_INVALID_ARG, "D=%d must be >= 1", p->D);
    if (p->S < 1) return fail(NSA_ERR_INVALID_ARG, "S=%d must be >= 1", p->S);
    if (p->block_size < 1) return fail(NSA_ERR_INVALID_ARG, "block_size=%d must be >= 1", p->block_size);
    if (!isfinite(p->scale)) return fail(NSA_ERR_INVALID_ARG, "scale is not finite");
    if (p->window < 0) return fail(NSA_ERR_INVALID_ARG, "window=%d is negative (0: none)", p->window);
    int Tmax = p->T, Z = p->B;
    // Keys per (z, hkv): dense problems may have more keys than queries.
    if (p->Tk < 0) return fail(NSA_ERR_INVALID_ARG, "Tk=%d must be >= 0 (0: T)", p->Tk);
    if (p->sched_policy != 0 && p->sched_policy != 1)
        return fail(NSA_ERR_INVALID_ARG, "sched_policy=%d is not 0 (static) or 1 (persistent)",
                    p->sched_policy);
    if (packed && p->Tk != 0 && p->Tk != p->T)
        return fail(NSA_ERR_INVALID_ARG, "packed inputs need Tk = 0 or T (got %d)", p->Tk);
    const int Tk = p->Tk == 0 ? p->T : p->Tk;
    if (!packed && Tk < p->T) return fail(NSA_ERR_INVALID_ARG, "Tk=%d is below T=%d", Tk, p->T);
    if (packed) {
        if (p->B != 1) return fail(NSA_ERR_INVALID_ARG, "packed inputs need B == 1 (got %d)", p->B);
        if (p->n_seqs < 0) return fail(NSA_ERR_INVALID_ARG, "n_seqs=%d must be >= 0", p->n_seqs);
        if (p->T > 0 && p->n_seqs < 1) return fail(NSA_ERR_INVALID_ARG, "T=%d tokens but n_seqs=%d", p->T, p->n_seqs);
        if (p->max_seqlen < 0 || p->max_seqlen > p->T)
            return fail(NSA_ERR_INVALID_ARG, "max_seqlen=%d must lie in [0, T=%d]", p->max_seqlen, p->T);
        if (p->T > 0 && p->max_seqlen < 1) return fail(NSA_ERR_INVALID_ARG, "max_seqlen must be >= 1 when T > 0");
        Tmax = p->max_seqlen;
        Z = p->n_seqs;
    }
    if (p->S > 4096) return fail(NSA_ERR_UNSUPPORTED, "S=%d exceeds 4096 slots", p->S);
    if (p->dtype == NSA_BF16) {
        if (p->D != 32 && p->D != 64 && p->D != 128)
            return fail(NSA_ERR_UNSUPPORTED, "bf16 needs D in {32, 64, 128} (got %d)", p->D);
        if (p->block_size != 16 && p->block_size != 32 && p->block_size != 64 && p->block_size != 128)
            return fail(NSA_ERR_UNSUPPORTED, "bf16 needs block_size in {16, 32, 64, 128} (got %d)", p->block_size);
    } else {
        if (p->D != 16 && p->D != 32 && p->D != 64 && p->D != 128)
            return fail(NSA_ERR_UNSUPPORTED, "f32 needs D in {16, 32, 64, 128} (got %d)", p->D);
    }
    // Blocks of the keys (the queries' positions end where the keys end).
    const int64_t Kmax = packed ? Tmax : Tk;
    const int64_t NBmax = (Kmax + p->block_size - 1) / p->block_size;
    if (NBmax > 8192) return fail(NSA_ERR_UNSUPPORTED, "ceil(max length / block_size) = %lld exceeds 8192", (long long)NBmax);
    const int G = p->Hq / p->Hkv;
    if ((int64_t)Tmax * G > (1ll << 30)) return fail(NSA_ERR_UNSUPPORTED, "max length * G exceeds 2^30 rows");
    if ((int64_t)p->Hq * p->T * p->D >= (1ll << 31))
        return fail(NSA_ERR_UNSUPPORTED, "Hq * T * D = %lld elements per batch entry exceeds 2^31 - 1",
                    (long long)p->Hq * p->T * p->D);
    if ((int64_t)p->Hkv * Tk * p->D >= (1ll << 31))
        return fail(NSA_ERR_UNSUPPORTED, "Hkv * Tk * D = %lld elements per batch entry exceeds 2^31 - 1",
                    (long long)p->Hkv * Tk * p->D);
    const int64_t ZH = (int64_t)Z * p->Hkv;
    if (ZH > 8192) return fail(NSA_ERR_UNSUPPORTED, "(batch or sequences) * Hkv = %lld exceeds 8192", (long long)ZH);
    const int64_t idx_rows = (int64_t)p->B * p->Hkv * p->T;
    const int64_t Smin = std::min<int64_t>(p->S, std::max<int64_t>(NBmax, 1));
    // The inverted lists of one (z, hkv) hold up to Tmax * Smin entries,
    // addressed with 32-bit offsets (scans, cursors, the fill's positions).
    if ((int64_t)Tmax * Smin >= (1ll << 31))
        return fail(NSA_ERR_UNSUPPORTED, "max length * min(S, NBmax) = %lld list entries per (batch, KV head) "
                    "exceeds 2^31 - 1", (long long)Tmax * Smin);
    if (p->strided != 0 && p->strided != 1)
        return fail(NSA_ERR_INVALID_ARG, "strided=%d is not 0 or 1", p->strided);

    nsa::Problem& d = hp.dev;
    d.B = p->B; d.T = p->T; d.Tk = Tk; d.Hq = p->Hq; d.Hkv = p->Hkv; d.G = G; d.D = p->D; d.S = p->S;
    d.bs = p->block_size; d.Z = Z; d.packed = packed ? 1 : 0; d.Tmax = Tmax; d.NBmax = (int)NBmax;
    d.Smin = (int)Smin; d.scale = p->scale; d.scale_log2 = p->scale * nsa::kLog2e; d.cu = nullptr;
    d.sink = nullptr;
    d.window = p->window;
    // Element strides (batch entry, head, token) of the eight tensors.
    {
        const int64_t D = p->D;
        auto dflt = [&](int64_t H, int64_t T) {
            // (32-bit head / token strides: check_qk bounds them before any use)
            return packed ? nsa::TLayout{0, (int32_t)D, (int32_t)(H * D)}
                          : nsa::TLayout{H * T * D, (int32_t)(T * D), (int32_t)D};
        };
        auto given = [&](const int64_t* x) {
            auto c32 = [](int64_t v) { return (int32_t)std::max<int64_t>(-1, std::min<int64_t>(v, INT32_MAX)); };
            return nsa::TLayout{packed ? 0 : x[0], c32(x[1]), c32(x[2])};
        };
        const bool st = p->strided == 1;
        d.strided = st ? 1 : 0;
        const int64_t* src[8] = {p->stride_q, p->stride_k, p->stride_v, p->stride_o,
                                 p->stride_do, p->stride_dq, p->stride_dk, p->stride_dv};
        for (int i = 0; i < 8; ++i)
            for (int j = 0; j < 3; ++j) hp.given[i][j] = st ? src[i][j] : 0;
        d.lq = st ? given(p->stride_q) : dflt(p->Hq, p->T);
        d.lo = st ? given(p->stride_o) : dflt(p->Hq, p->T);
        d.ldo = st ? given(p->stride_do) : dflt(p->Hq, p->T);
        d.ldq = st ? given(p->stride_dq) : dflt(p->Hq, p->T);
        d.lk = st ? given(p->stride_k) : dflt(p->Hkv, Tk);
        d.lv = st ? given(p->stride_v) : dflt(p->Hkv, Tk);
        d.ldk = st ? given(p->stride_dk) : dflt(p->Hkv, Tk);
        d.ldv = st ? given(p->stride_dv) : dflt(p->Hkv, Tk);
    }
    hp.dtype = p->dtype;
    hp.ZH = (int)ZH;
    // Inversion chunks of CT tokens: at least 64 (smaller chunks multiply the
    // count and fill workgroups, whose launch then costs more than their
    // work: with 16-token chunks the prepare stage took 0.108 / 0.092 ms on 8
    // packed sequences / a dense causal 4 x 4096 problem, 0.091 / 0.080 with
    // 64), growing in steps of 16 so that the per-(z, hkv) chunk x block
    // table stays within 2^14 entries.
    {
        const int64_t work = (int64_t)Tmax * NBmax;
        hp.CT = 16 * (int)std::max<int64_t>(4, (work + (16ll << 14) - 1) / (16ll << 14));
    }
    hp.C = (Tmax + hp.CT - 1) / hp.CT;
    hp.rows = (int64_t)p->B * p->Hq * p->T;
    hp.cap = Smin * idx_rows;
    const int64_t rows_ub = hp.cap * G;
    // Rows per dK/dV work item: about 1/2048 of the row bound (several items
    // per workgroup slot, so the last round is short), within [1024, 16384].
    int64_t cr = (rows_ub / 2048 + 31) / 32 * 32;
    hp.CR = (int)std::min<int64_t>(16384, std::max<int64_t>(1024, cr));
    hp.items_ub = ZH * NBmax + (rows_ub + hp.CR - 1) / hp.CR;
    if (hp.items_ub > (1ll << 31) - 1) return fail(NSA_ERR_UNSUPPORTED, "too many dK/dV work items");
    hp.pslots = (p->dtype == NSA_BF16 && (int64_t)Tmax * G > hp.CR) ? hp.items_ub : 0;
    // (Block pairs assume a block's list starts at its own first token:
    // queries and keys aligned, Tk = T.)
    hp.pair_possible = p->dtype == NSA_BF16 && hp.pslots == 0 && p->block_size <= 64 && p->window == 0 &&
                       (int64_t)p->S * p->block_size >= Tmax && ZH > 0 && NBmax > 0 && Tk == p->T;
    // dS hand-off: the dQ kernel's tiles hold 16 heads of one token, or all
    // heads of 2 or 4 tokens; one 32-bit offset spans a (z, hkv) region of dS.
    // (Lists that can cover whole key prefixes recompute dS: measured faster
    // on a dense causal problem than moving their dS through memory.)
    hp.ds_handoff = p->dtype == NSA_BF16 && (G % 16 == 0 || G == 8 || G == 4) && p->window == 0 &&
                    p->block_size >= 32 && p->S <= 64 && (int64_t)p->S * p->block_size < Kmax &&
                    (int64_t)Tmax * Smin * p->block_size * G * 2 < (1ll << 31);
    if (hp.ds_handoff && nsa::dq_ds_lds_bytes(hp) > 163840) hp.ds_handoff = false;
    hp.sched = p->sched_policy;
    if (nsa::invert_lds_bytes(hp) > 163840)
        return fail(NSA_ERR_UNSUPPORTED, "the block inversion needs %zu bytes of LDS for %lld blocks (max 163840)",
                    nsa::invert_lds_bytes(hp), (long long)NBmax);
    if (p->dtype == NSA_BF16 && nsa::query_lds_bytes(hp) > 163840)
        return fail(NSA_ERR_UNSUPPORTED, "bf16 forward/dQ need %zu bytes of LDS for %lld blocks (max 163840)",
                    nsa::query_lds_bytes(hp), (long long)NBmax);
    return NSA_OK;
}

nsa::BwdWorkspace carve(const nsa::HostProblem& hp, void* base) {
    nsa::BwdWorkspace w{};
    size_t off = 0;
    char* b = static_cast<char*>(base);
    auto take = [&](size_t bytes) -> char* {
        char* ptr = b ? b + off : nullptr;
        off += align256(bytes);
        return ptr;
    };
    const int64_t ZH = hp.ZH, NB = hp.dev.NBmax;
    w.delta = (float*)take(sizeof(float) * hp.rows);
    w.chunk_pos = (int*)take(sizeof(int) * ZH * hp.C * NB);
    w.offsets = (int*)take(sizeof(int) * ZH * (NB + 1));
    w.tokens = (int*)take(sizeof(int) * hp.cap);
    w.item_pre = (int*)take(sizeof(int) * ZH * (NB + 1));
    w.pslot_pre = (int*)take(sizeof(int) * ZH * (NB + 1));
    w.zh_base = (int*)take(sizeof(int) * (2 * (ZH + 1) + 3 * ZH + 1));
    w.ticket = (int*)take(3 * sizeof(int));
    w.iota = (int*)take(hp.pair_possible ? sizeof(int) * hp.dev.Tmax : 0);
    // (16-key blocks use the 32-key tile's slot layout)
    w.partials = (float*)take(sizeof(float) * hp.pslots * 2 * std::max(32, hp.dev.bs) * hp.dev.D);
    const bool ho = hp.ds_handoff;
    w.posmap = (int*)take(ho ? sizeof(int) * (size_t)hp.dev.B * hp.dev.Hkv * hp.dev.T * hp.dev.S : 0);
    w.ds = (uint16_t*)take(ho ? sizeof(uint16_t) * (size_t)hp.cap * hp.dev.bs * hp.dev.G : 0);
    w.bytes = off;
    return w;
}

// cu_seqlens must be given exactly for packed problems that hold tokens.
nsa_status check_cu(const nsa::HostProblem& hp, const int32_t* cu) {
    if (!hp.dev.packed && cu) return fail(NSA_ERR_INVALID_ARG, "cu_seqlens given for a dense problem");
    if (hp.dev.packed && hp.dev.T > 0 && !cu) return fail(NSA_ERR_INVALID_ARG, "cu_seqlens is NULL for a packed problem");
    if (cu && misaligned(cu, 4)) return fail(NSA_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
    return NSA_OK;
}

nsa_status check_tensor(const void* ptr, int64_t elems, size_t align, const char* name) {
    if (elems > 0 && !ptr) return fail(NSA_ERR_INVALID_ARG, "%s is NULL", name);
    if (ptr && misaligned(ptr, align))
        return fail(NSA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    return NSA_OK;
}

// The eight tensors with a (batch entry, head, token, D) layout.
enum Which { kQ, kK, kV, kO, kDO, kDQ, kDK, kDV };
const char* const kWhichName[] = {"q", "k", "v", "o", "dO", "dq", "dk", "dv"};

const nsa::TLayout& layout_of(const nsa::Problem& d, Which w) {
    switch (w) {
        case kQ: return d.lq;
        case kK: return d.lk;
        case kV: return d.lv;
        case kO: return d.lo;
        case kDO: return d.ldo;
        case kDQ: return d.ldq;
        case kDK: return d.ldk;
        default: return d.ldv;
    }
}

// Pointer, alignment and strides of one of the eight tensors.  Strides are
// >= 0, multiples of 8 elements for bf16 (every row 16-byte aligned), the
// token stride below 2^23 elements (the kernels form byte offsets of tokens
// with 24-bit multiplies), and one batch entry spans less than 2^31 - 128
// elements (offsets inside an entry are 32-bit, and one past every such
// offset marks a load out of range).  Outputs
// must map distinct (entry, head, token, d) to distinct elements: with the
// dimensions sorted by stride, each stride reaches past everything the
// smaller ones span.
nsa_status check_qk(const nsa::HostProblem& hp, Which w, const void* ptr) {
    const nsa::Problem& d = hp.dev;
    const char* name = kWhichName[w];
    const bool qlike = w == kQ || w == kO || w == kDO || w == kDQ;
    const int64_t nb = d.packed ? 1 : d.B, nh = qlike ? d.Hq : d.Hkv, nt = qlike ? d.T : d.Tk, D = d.D;
    if (nb * nh * nt == 0) return NSA_OK;
    if (!ptr) return fail(NSA_ERR_INVALID_ARG, "%s is NULL", name);
    const bool bf16 = hp.dtype == NSA_BF16;
    if (misaligned(ptr, bf16 ? 16 : 4))
        return fail(NSA_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, bf16 ? 16 : 4);
    const nsa::TLayout& L = layout_of(d, w);
    const int64_t* x = d.strided ? hp.given[w] : nullptr;
    const int64_t sb = x ? (d.packed ? 0 : x[0]) : L.sb, sh0 = x ? x[1] : L.sh, st0 = x ? x[2] : L.st;
    if (sb < 0 || sh0 < 0 || st0 < 0)
        return fail(NSA_ERR_INVALID_ARG, "%s strides (%lld, %lld, %lld) must be >= 0", name,
                    (long long)sb, (long long)sh0, (long long)st0);
    if (bf16 && (sb % 8 || sh0 % 8 || st0 % 8))
        return fail(NSA_ERR_INVALID_ARG, "%s strides (%lld, %lld, %lld) are not multiples of 8 "
                    "(bf16 rows must be 16-byte aligned)", name, (long long)sb, (long long)sh0,
                    (long long)st0);
    // (The 32-bit device strides were clamped; read the caller's values.)
    const int64_t sh = d.strided ? hp.given[w][1] : L.sh, stt = d.strided ? hp.given[w][2] : L.st;
    if (stt >= (1ll << 23))
        return fail(NSA_ERR_UNSUPPORTED, "%s token stride %lld is not below 2^23 elements", name, (long long)stt);
    const int64_t entry = (nh - 1) * sh + (nt - 1) * stt + D;
    if (entry > (1ll << 31) - 128)
        return fail(NSA_ERR_UNSUPPORTED, "%s spans %lld elements per batch entry (limit 2^31 - 128)",
                    name, (long long)entry);
    if (w == kO || w == kDQ || w == kDK || w == kDV) {
        struct Dim { int64_t n, s; } dims[4] = {{D, 1}, {nb, sb}, {nh, sh}, {nt, stt}};
        std::sort(dims, dims + 4, [](const Dim& a, const Dim& b) { return a.s < b.s; });
        int64_t span = 0;  // elements spanned by the dimensions taken so far, minus 1
        for (const Dim& x : dims) {
            if (x.n <= 1) continue;
            if (x.s <= span)
                return fail(NSA_ERR_INVALID_ARG, "output %s has overlapping rows (stride %lld within "
                            "a span of %lld elements)", name, (long long)x.s, (long long)span + 1);
            span += (x.n - 1) * x.s;
        }
    }
    return NSA_OK;
}

struct Sizes {
    int64_t q, kv, idx, lse;
};
Sizes sizes_of(const nsa::HostProblem& hp) {
    const nsa::Problem& d = hp.dev;
    return {(int64_t)d.B * d.Hq * d.T * d.D, (int64_t)d.B * d.Hkv * d.Tk * d.D,
            (int64_t)d.B * d.Hkv * d.T * d.S, (int64_t)d.B * d.Hq * d.T};
}

#define NSA_TRY(x)                       \
    do {                                 \
        nsa_status st_ = (x);            \
        if (st_ != NSA_OK) return st_;   \
    } while (0)

#define NSA_HIP(x, what)                           \
    do {                                           \
        hipError_t e_ = (x);                       \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

// Marks a tensor an entry point does not take (distinct from NULL, which is
// an error for a non-empty tensor).
const char g_absent_tag = 0;
const void* const kAbsent = &g_absent_tag;

// Shared checks of the backward entry points: problem, tensors (those given),
// workspace size and alignment.
struct BwdArgs {
    const void *q, *k, *v, *o, *dO, *dq, *dk, *dv;
    const float* lse;
    const int32_t *idx, *cu;
    void* ws;
    size_t ws_bytes;
};

// check_ws = false: the workspace is the built-in scratch (its size is
// checked by the caller), so only the problem and tensors are checked.
nsa_status check_bwd(const nsa_sel_problem* p, const BwdArgs& a, nsa::HostProblem& hp,
                     bool check_ws = true) {
    NSA_TRY(make_problem(p, hp));
    NSA_TRY(check_cu(hp, a.cu));
    const Sizes sz = sizes_of(hp);
    const struct {
        const void* ptr;
        Which w;
    } ts[] = {{a.q, kQ}, {a.k, kK}, {a.v, kV}, {a.o, kO}, {a.dO, kDO}, {a.dq, kDQ}, {a.dk, kDK},
              {a.dv, kDV}};
    for (const auto& t : ts)
        if (t.ptr != kAbsent) NSA_TRY(check_qk(hp, t.w, t.ptr));
    if (a.lse != kAbsent) NSA_TRY(check_tensor(a.lse, sz.lse, 4, "lse"));
    if (a.idx != kAbsent) NSA_TRY(check_tensor(a.idx, sz.idx, 4, "block_idx"));
    if (check_ws) {
        const nsa::BwdWorkspace need = carve(hp, nullptr);
        if (need.bytes && (!a.ws || a.ws_bytes < need.bytes))
            return fail(NSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", a.ws_bytes, need.bytes);
        if (a.ws && misaligned(a.ws, 256)) return fail(NSA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    }
    hp.dev.cu = a.cu;
    return NSA_OK;
}

nsa_status run_prepare(const nsa::HostProblem& hp, const BwdArgs& a, hipStream_t st) {
    const nsa::BwdWorkspace ws = carve(hp, a.ws);
    NSA_HIP(nsa::launch_prepare(hp, a.o, a.dO, a.idx, ws, st), "Delta / inversion launch");
    return NSA_OK;
}

nsa_status run_dq(const nsa::HostProblem& hp, const BwdArgs& a, hipStream_t st) {
    const nsa::BwdWorkspace ws = carve(hp, a.ws);
    if (hp.dtype == NSA_BF16 && hp.ds_handoff) {
        NSA_HIP(nsa::launch_dq_handoff(hp, a.k, a.idx, ws, (void*)a.dq, st), "dQ (dS hand-off) launch");
    } else if (hp.dtype == NSA_BF16) {
        NSA_HIP(nsa::launch_dq_bf16(hp, a.q, a.k, a.v, a.dO, a.lse, ws.delta, a.idx, (void*)a.dq, st), "dQ launch");
    } else {
        NSA_HIP(nsa::launch_dq_f32(hp, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                                   (const float*)a.dO, a.lse, ws.delta, a.idx, (float*)a.dq, st),
                "dQ launch");
    }
    return NSA_OK;
}

nsa_status run_dkdv(const nsa::HostProblem& hp, const BwdArgs& a, hipStream_t st,
                    int parts = nsa::kDkdvAll) {
    const nsa::BwdWorkspace ws = carve(hp, a.ws);
    if (hp.dtype == NSA_BF16) {
        NSA_HIP(nsa::launch_dkdv_bf16(hp, a.q, a.k, a.v, a.dO, a.lse, ws.delta, ws, (void*)a.dk,
                                      (void*)a.dv, st, parts),
                "dK/dV launch");
    } else {
        // One vector-ALU kernel does all of it; the reduce part is empty.
        if (!(parts & nsa::kDkdvBlocks)) return NSA_OK;
        NSA_HIP(nsa::launch_dkdv_f32(hp, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                                     (const float*)a.dO, a.lse, ws.delta, ws, (float*)a.dk,
                                     (float*)a.dv, st),
                "dK/dV launch");
    }
    return NSA_OK;
}

}  // namespace

namespace nsa {
BwdWorkspace carve_bwd_workspace(const HostProblem& hp, void* base) { return carve(hp, base); }
}  // namespace nsa

// ---- backward without allocation -----------------------------------------
// A fixed device array stands in for the backward's workspace in
// nsa_sel_bwd_noalloc.  Each device the library runs on holds its own copy
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address, looked up once per device.
nsa_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(NSA_ERR_UNSUPPORTED, "device %d is beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(NSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NSA_OK;
}
}  // namespace

extern "C" {

const char* nsa_status_string(nsa_status s) {
    switch (s) {
        case NSA_OK: return "ok";
        case NSA_ERR_INVALID_ARG: return "invalid argument";
        case NSA_ERR_UNSUPPORTED: return "unsupported problem";
        case NSA_ERR_WORKSPACE: return "workspace missing or too small";
        case NSA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* nsa_last_error(void) { return g_last_error.c_str(); }

// Set by the build (the commit of the sources compiled).
#ifndef NSA_BUILD_GIT
#define NSA_BUILD_GIT "unknown"
#endif
const char* nsa_build_git(void) { return NSA_BUILD_GIT; }

int32_t nsa_sel_bwd_ds_handoff(const nsa_sel_problem* p) {
    g_last_error.clear();
    nsa::HostProblem hp;
    if (!p) {
        fail(NSA_ERR_INVALID_ARG, "problem pointer is NULL");
        return -1;
    }
    if (make_problem(p, hp) != NSA_OK) return -1;
    return hp.ds_handoff ? 1 : 0;
}

nsa_status nsa_sel_wait_timeouts(uint64_t* count) {
    g_last_error.clear();
    if (!count) return fail(NSA_ERR_INVALID_ARG, "count is NULL");
    unsigned a = 0, b = 0;
    NSA_HIP(nsa::read_wait_timeouts_query(&a), "reading the query kernels' wait counter");
    NSA_HIP(nsa::read_wait_timeouts_dkdv(&b), "reading the dK/dV kernel's wait counter");
    *count = (uint64_t)a + b;
    return NSA_OK;
}

nsa_status nsa_sel_fwd(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* block_idx, const int32_t* cu_seqlens, void* o, float* lse,
                       nsa_stream_t stream) {
    return nsa_sel_fwd_sink(p, q, k, v, block_idx, cu_seqlens, nullptr, o, lse, stream);
}

nsa_status nsa_sel_fwd_sink(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* block_idx, const int32_t* cu_seqlens, const float* sink,
                            void* o, float* lse, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    NSA_TRY(make_problem(p, hp));
    NSA_TRY(check_cu(hp, cu_seqlens));
    if (sink) NSA_TRY(check_tensor(sink, hp.dev.Hq, 4, "sink"));
    hp.dev.sink = sink;
    const Sizes sz = sizes_of(hp);
    NSA_TRY(check_qk(hp, kQ, q));
    NSA_TRY(check_qk(hp, kK, k));
    NSA_TRY(check_qk(hp, kV, v));
    NSA_TRY(check_qk(hp, kO, o));
    NSA_TRY(check_tensor(block_idx, sz.idx, 4, "block_idx"));
    NSA_TRY(check_tensor(lse, sz.lse, 4, "lse"));
    if (sz.q == 0) return NSA_OK;
    hp.dev.cu = cu_seqlens;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (hp.dtype == NSA_BF16) {
        NSA_HIP(nsa::launch_fwd_bf16(hp, q, k, v, block_idx, o, lse, st), "forward launch");
    } else {
        NSA_HIP(nsa::launch_fwd_f32(hp, (const float*)q, (const float*)k, (const float*)v,
                                    block_idx, (float*)o, lse, st),
                "forward launch");
    }
    return NSA_OK;
}

size_t nsa_sel_bwd_workspace_bytes(const nsa_sel_problem* p) {
    g_last_error.clear();
    nsa::HostProblem hp;
    if (!p) {
        fail(NSA_ERR_INVALID_ARG, "problem pointer is NULL");
        return 0;
    }
    if (make_problem(p, hp) != NSA_OK) return 0;
    return carve(hp, nullptr).bytes;
}

size_t nsa_sel_invert_tokens_capacity(const nsa_sel_problem* p) {
    g_last_error.clear();
    nsa::HostProblem hp;
    if (!p) {
        fail(NSA_ERR_INVALID_ARG, "problem pointer is NULL");
        return 0;
    }
    if (make_problem(p, hp) != NSA_OK) return 0;
    return (size_t)hp.cap;
}

nsa_status nsa_sel_delta(const nsa_sel_problem* p, const void* o, const void* dO,
                         const int32_t* cu_seqlens, float* delta, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    NSA_TRY(make_problem(p, hp));
    NSA_TRY(check_cu(hp, cu_seqlens));
    const Sizes sz = sizes_of(hp);
    NSA_TRY(check_qk(hp, kO, o));
    NSA_TRY(check_qk(hp, kDO, dO));
    NSA_TRY(check_tensor(delta, sz.lse, 4, "delta"));
    if (sz.q == 0) return NSA_OK;
    hp.dev.cu = cu_seqlens;
    NSA_HIP(nsa::launch_delta(hp, o, dO, delta, reinterpret_cast<hipStream_t>(stream)), "delta launch");
    return NSA_OK;
}

nsa_status nsa_sel_invert(const nsa_sel_problem* p, const int32_t* block_idx,
                          const int32_t* cu_seqlens, int32_t* offsets, int32_t* tokens,
                          void* workspace, size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    NSA_TRY(make_problem(p, hp));
    NSA_TRY(check_cu(hp, cu_seqlens));
    const Sizes sz = sizes_of(hp);
    NSA_TRY(check_tensor(block_idx, sz.idx, 4, "block_idx"));
    const int64_t n_off = (int64_t)hp.ZH * (hp.dev.NBmax + 1);
    NSA_TRY(check_tensor(offsets, n_off, 4, "offsets"));
    NSA_TRY(check_tensor(tokens, hp.cap, 4, "tokens"));
    const nsa::BwdWorkspace need = carve(hp, nullptr);
    if (need.bytes && (!workspace || workspace_bytes < need.bytes))
        return fail(NSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need.bytes);
    if (workspace && misaligned(workspace, 256)) return fail(NSA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (hp.ZH == 0 || hp.dev.NBmax == 0) {
        if (n_off) NSA_HIP(hipMemsetAsync(offsets, 0, sizeof(int) * n_off, reinterpret_cast<hipStream_t>(stream)), "offsets clear");
        return NSA_OK;
    }
    hp.dev.cu = cu_seqlens;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const nsa::BwdWorkspace ws = carve(hp, workspace);
    NSA_HIP(nsa::launch_invert(hp, block_idx, ws, st), "inversion launch");
    NSA_HIP(hipMemcpyAsync(offsets, ws.offsets, sizeof(int) * n_off, hipMemcpyDeviceToDevice, st), "offsets copy");
    if (hp.cap)
        NSA_HIP(hipMemcpyAsync(tokens, ws.tokens, sizeof(int) * hp.cap, hipMemcpyDeviceToDevice, st), "tokens copy");
    return NSA_OK;
}

nsa_status nsa_sel_bwd_dsink(const nsa_sel_problem* p, const float* lse, const float* sink,
                             const int32_t* cu_seqlens, float* dsink, void* workspace,
                             size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    NSA_TRY(make_problem(p, hp));
    NSA_TRY(check_cu(hp, cu_seqlens));
    NSA_TRY(check_tensor(lse, sizes_of(hp).lse, 4, "lse"));
    if (!sink) return fail(NSA_ERR_INVALID_ARG, "sink is NULL");
    NSA_TRY(check_tensor(sink, hp.dev.Hq, 4, "sink"));
    NSA_TRY(check_tensor(dsink, hp.dev.Hq, 4, "dsink"));
    const nsa::BwdWorkspace need = carve(hp, nullptr);
    if (need.bytes && (!workspace || workspace_bytes < need.bytes))
        return fail(NSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need.bytes);
    if (workspace && misaligned(workspace, 256)) return fail(NSA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    hp.dev.cu = cu_seqlens;
    const nsa::BwdWorkspace ws = carve(hp, workspace);
    NSA_HIP(nsa::launch_dsink(hp, lse, ws.delta, sink, dsink, reinterpret_cast<hipStream_t>(stream)),
            "dsink launch");
    return NSA_OK;
}

nsa_status nsa_sel_check_block_idx(const nsa_sel_problem* p, const int32_t* block_idx,
                                   const int32_t* cu_seqlens, uint64_t* counts,
                                   nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    NSA_TRY(make_problem(p, hp));
    NSA_TRY(check_cu(hp, cu_seqlens));
    NSA_TRY(check_tensor(block_idx, sizes_of(hp).idx, 4, "block_idx"));
    NSA_TRY(check_tensor(counts, 4, 8, "counts"));
    hp.dev.cu = cu_seqlens;
    NSA_HIP(nsa::launch_check_idx(hp, block_idx, reinterpret_cast<unsigned long long*>(counts),
                                  reinterpret_cast<hipStream_t>(stream)),
            "block_idx check launch");
    return NSA_OK;
}

nsa_status nsa_sel_bwd(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dO,
                       const int32_t* block_idx, const int32_t* cu_seqlens, void* dq, void* dk,
                       void* dv, void* workspace, size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{q, k, v, o, dO, dq, dk, dv, lse, block_idx, cu_seqlens, workspace, workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    NSA_TRY(run_prepare(hp, a, st));
    NSA_TRY(run_dkdv(hp, a, st));
    return run_dq(hp, a, st);
}

nsa_status nsa_sel_bwd_noalloc(const nsa_sel_problem* p, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* dO,
                               const int32_t* block_idx, const int32_t* cu_seqlens, void* dq,
                               void* dk, void* dv, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    BwdArgs a{q, k, v, o, dO, dq, dk, dv, lse, block_idx, cu_seqlens, nullptr, kScratchBytes};
    NSA_TRY(check_bwd(p, a, hp, false));
    size_t need = carve(hp, nullptr).bytes;
    // Without room for the dS hand-off, dQ recomputes dS (the same results
    // within the stated tolerance; the hand-off buffers dominate its need).
    if (need > kScratchBytes && hp.ds_handoff) {
        hp.ds_handoff = false;
        need = carve(hp, nullptr).bytes;
    }
    if (need > kScratchBytes)
        return fail(NSA_ERR_WORKSPACE, "this backward needs %zu bytes of workspace; the built-in scratch of "
                    "nsa_sel_bwd_noalloc holds %zu (use nsa_sel_bwd with a caller workspace)",
                    need, kScratchBytes);
    if (sizes_of(hp).q == 0) return NSA_OK;
    NSA_TRY(scratch_address(&a.ws));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    NSA_TRY(run_prepare(hp, a, st));
    NSA_TRY(run_dkdv(hp, a, st));
    return run_dq(hp, a, st);
}

nsa_status nsa_sel_bwd_prepare(const nsa_sel_problem* p, const void* o, const void* dO,
                               const int32_t* block_idx, const int32_t* cu_seqlens,
                               void* workspace, size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{kAbsent, kAbsent, kAbsent, o,       dO,      kAbsent, kAbsent,
                    kAbsent, (const float*)kAbsent, block_idx, cu_seqlens, workspace, workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    return run_prepare(hp, a, reinterpret_cast<hipStream_t>(stream));
}

nsa_status nsa_sel_bwd_prepare_lists(const nsa_sel_problem* p, const int32_t* block_idx,
                                     const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{kAbsent, kAbsent, kAbsent, kAbsent, kAbsent, kAbsent, kAbsent,
                    kAbsent, (const float*)kAbsent, block_idx, cu_seqlens, workspace, workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    const nsa::BwdWorkspace ws = carve(hp, workspace);
    NSA_HIP(nsa::launch_prepare_lists(hp, block_idx, ws, reinterpret_cast<hipStream_t>(stream)),
            "inversion launch");
    return NSA_OK;
}

nsa_status nsa_sel_bwd_prepare_delta(const nsa_sel_problem* p, const void* o, const void* dO,
                                     const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{kAbsent, kAbsent, kAbsent, o,       dO,      kAbsent, kAbsent,
                    kAbsent, (const float*)kAbsent, (const int32_t*)kAbsent, cu_seqlens, workspace,
                    workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    const nsa::BwdWorkspace ws = carve(hp, workspace);
    NSA_HIP(nsa::launch_delta(hp, o, dO, ws.delta, reinterpret_cast<hipStream_t>(stream)), "delta launch");
    return NSA_OK;
}

nsa_status nsa_sel_bwd_dq(const nsa_sel_problem* p, const void* q, const void* k, const void* v,
                          const void* dO, const float* lse, const int32_t* block_idx,
                          const int32_t* cu_seqlens, void* dq, void* workspace,
                          size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{q, k, v, kAbsent, dO, dq, kAbsent, kAbsent, lse, block_idx, cu_seqlens,
                    workspace, workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    return run_dq(hp, a, reinterpret_cast<hipStream_t>(stream));
}

nsa_status nsa_sel_bwd_dkdv(const nsa_sel_problem* p, const void* q, const void* k,
                            const void* v, const void* dO, const float* lse,
                            const int32_t* cu_seqlens, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{q, k, v, kAbsent, dO, kAbsent, dk, dv, lse, (const int32_t*)kAbsent,
                    cu_seqlens, workspace, workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    return run_dkdv(hp, a, reinterpret_cast<hipStream_t>(stream));
}

nsa_status nsa_sel_bwd_dkdv_blocks(const nsa_sel_problem* p, const void* q, const void* k,
                                   const void* v, const void* dO, const float* lse,
                                   const int32_t* cu_seqlens, void* dk, void* dv, void* workspace,
                                   size_t workspace_bytes, nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{q, k, v, kAbsent, dO, kAbsent, dk, dv, lse, (const int32_t*)kAbsent,
                    cu_seqlens, workspace, workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    return run_dkdv(hp, a, reinterpret_cast<hipStream_t>(stream), nsa::kDkdvBlocks);
}

nsa_status nsa_sel_bwd_dkdv_reduce(const nsa_sel_problem* p, const int32_t* cu_seqlens, void* dk,
                                   void* dv, void* workspace, size_t workspace_bytes,
                                   nsa_stream_t stream) {
    g_last_error.clear();
    nsa::HostProblem hp;
    const BwdArgs a{kAbsent, kAbsent, kAbsent, kAbsent, kAbsent, kAbsent, dk, dv,
                    (const float*)kAbsent, (const int32_t*)kAbsent, cu_seqlens, workspace,
                    workspace_bytes};
    NSA_TRY(check_bwd(p, a, hp));
    if (sizes_of(hp).q == 0) return NSA_OK;
    return run_dkdv(hp, a, reinterpret_cast<hipStream_t>(stream), nsa::kDkdvReduce);
}

}  // extern "C"
