/*
 * nsa_oracle.c -- plain float64 CPU oracle for NSA selection attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library; it is written from the definition of the method.
 *
 * Source of the method: page 1 of the reference text, "test_kernel_backward.py
 * -- GRADCHECK GATE for the NSA selection BACKWARD kernel" (module docstring
 * and run_one): each query token attends, per KV head, only to the key/value
 * blocks listed for it in block_idx; G = Hq/Hkv query heads share one KV head
 * and its list; the backward is the exact gradient of that forward.  The page
 * does not print the forward body, so this file writes out the plain masked
 * softmax definition:
 *
 *   Sel(b,h,t) = { u : u = block_idx[b,hkv,t,s] for some s, 0 <= u < NB }
 *   A(b,h,t)   = { j : floor(j/bs) in Sel, j < T, j <= t }      (set semantics)
 *   s_j = scale * <q[b,h,t], k[b,hkv,j]>,  lse = log sum_{j in A} exp(s_j)
 *   P_j = exp(s_j - lse),                   o = sum_{j in A} P_j v[b,hkv,j]
 *   dP_j = <dO[b,h,t], v_j>, Delta = sum_j P_j dP_j, dS_j = P_j (dP_j - Delta)
 *   dq = scale sum_j dS_j k_j
 *   dk_j = scale sum_{rows r with j in A(r)} dS_{r,j} q_r
 *   dv_j =       sum_{rows r with j in A(r)} P_{r,j} dO_r
 * with hkv = floor(h / G) and an empty A giving o = 0, lse = -inf, dq = 0.
 *
 * Optional attention sink (page 3 names a dSink step of the backward chain
 * without defining it; the reading taken): a per-head logit sink[h], no
 * scale applied, that joins every row's softmax denominator with no value
 * vector, lse = log(sum_{j in A} exp(s_j) + exp(sink[h])).  P_j, o, Delta,
 * dS and the dq/dk/dv sums keep the formulas above with this lse (an empty
 * A then gives lse = sink[h]); the sink's own gradient, summed over the
 * rows of head h, is -sum_rows exp(sink[h] - lse) Delta (computed in
 * oracle/__init__.py).  sink == NULL means no sink.
 *
 * Bottom-right causal alignment (the pages list it among the backward's
 * flavours, nothing more; the reading taken): a dense problem may have Tk >=
 * T keys per (batch entry, KV head); the T queries are then the last T
 * positions of the key range, query t at key position t + (Tk - T), so
 * causality reads j <= t + (Tk - T) and the key set is capped at j < Tk
 * (Tk = T: the usual causal mask).  Below, "t" in a key comparison means
 * that position.
 *
 * Optional sliding window (the pages list sliding-window masks among the
 * backward's flavours; the reading taken): window W >= 1 further limits A to
 * the keys j with t - W < j <= t (W = 0: no limit).  It is a mask on the
 * keys only: block lists, and so the block -> query inversion, are
 * unchanged.
 *
 * Layout (dense, contiguous, row-major): q, o, dO, dq [B][Hq][T][D];
 * k, v, dk, dv [B][Hkv][Tk][D]; block_idx [B][Hkv][T][S] int32; lse, delta
 * [B][Hq][T].  Packed variable-length batches are handled by the Python side
 * as one dense B=1 call per sequence (no key crosses a sequence boundary).
 *
 * Parity pinned by tests/test_oracle_pins.py (finite differences, dense
 * masked autograd, causal SDPA equivalence, GQA head sum, closed forms,
 * invariants, brute-force inversion).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int B, Hq, Hkv, T, D, S, bs;
    double scale;
    const double* sink; /* [Hq] or NULL */
    int window;         /* 0: none */
    int Tk;             /* keys per (batch entry, KV head), >= T */
} shape_t;

/* Key position of query t (bottom-right alignment). */
static int kpos(const shape_t* sh, int t) { return t + (sh->Tk - sh->T); }

static int n_blocks(const shape_t* sh) { return (sh->Tk + sh->bs - 1) / sh->bs; }

static const int32_t* idx_row(const shape_t* sh, const int32_t* idx, int b, int hkv, int t) {
    return idx + (((int64_t)b * sh->Hkv + hkv) * sh->T + t) * sh->S;
}

static const double* qrow(const shape_t* sh, const double* x, int b, int h, int t) {
    return x + (((int64_t)b * sh->Hq + h) * sh->T + t) * sh->D;
}

static const double* krow(const shape_t* sh, const double* x, int b, int hkv, int j) {
    return x + (((int64_t)b * sh->Hkv + hkv) * sh->Tk + j) * sh->D;
}

static double dot(const double* a, const double* b, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += a[d] * b[d];
    return s;
}

/* Is block u listed in this row?  Negative and out-of-range entries never
 * match, and several copies of u count as one listing (set semantics). */
static int row_lists_block(const int32_t* row, int S, int u) {
    for (int s = 0; s < S; ++s)
        if (row[s] == u) return 1;
    return 0;
}

/* Ascending list of the keys in A(b,h,t); returns its size. */
static int selected_keys(const shape_t* sh, const int32_t* row, int t, int* keys) {
    int NB = n_blocks(sh), n = 0, tp = kpos(sh, t);
    for (int u = 0; u < NB; ++u) {
        if (!row_lists_block(row, sh->S, u)) continue;
        for (int j = u * sh->bs; j < (u + 1) * sh->bs && j < sh->Tk && j <= tp; ++j)
            if (sh->window <= 0 || j > tp - sh->window) keys[n++] = j;
    }
    return n;
}

/* Softmax of one row of head h over its selected keys (and the head's sink
 * logit, if any).  Writes P (n values) and returns lse (-inf when the row
 * has no key and there is no sink). */
static double row_softmax(const shape_t* sh, int h, const double* q_r, const double* K,
                          const int* keys, int n, double* P) {
    const double sk = sh->sink ? sh->sink[h] : -INFINITY;
    if (n == 0) return sk;
    double m = sk;
    for (int a = 0; a < n; ++a) {
        P[a] = sh->scale * dot(q_r, K + (int64_t)keys[a] * sh->D, sh->D);
        if (P[a] > m) m = P[a];
    }
    double sum = sh->sink ? exp(sk - m) : 0.0;
    for (int a = 0; a < n; ++a) sum += exp(P[a] - m);
    double lse = m + log(sum);
    for (int a = 0; a < n; ++a) P[a] = exp(P[a] - lse);
    return lse;
}

/* Forward of one row (b,h,t): o_out[D], *lse_out. */
static void fwd_row(const shape_t* sh, const double* q, const double* k, const double* v,
                    const int32_t* idx, int b, int h, int t, double* o_out, double* lse_out,
                    int* keys, double* P) {
    int G = sh->Hq / sh->Hkv, hkv = h / G, D = sh->D;
    const double* K = krow(sh, k, b, hkv, 0);
    const double* V = krow(sh, v, b, hkv, 0);
    int n = selected_keys(sh, idx_row(sh, idx, b, hkv, t), t, keys);
    double lse = row_softmax(sh, h, qrow(sh, q, b, h, t), K, keys, n, P);
    for (int d = 0; d < D; ++d) o_out[d] = 0.0;
    for (int a = 0; a < n; ++a) {
        const double* vj = V + (int64_t)keys[a] * D;
        for (int d = 0; d < D; ++d) o_out[d] += P[a] * vj[d];
    }
    *lse_out = lse;
}

/* lse and Delta = sum_j P_j dP_j of one row, plus dq if dq_out != NULL. */
static void bwd_row(const shape_t* sh, const double* q, const double* k, const double* v,
                    const double* dO, const int32_t* idx, int b, int h, int t, double* lse_out,
                    double* delta_out, double* dq_out, int* keys, double* P, double* dP) {
    int G = sh->Hq / sh->Hkv, hkv = h / G, D = sh->D;
    const double* K = krow(sh, k, b, hkv, 0);
    const double* V = krow(sh, v, b, hkv, 0);
    const double* do_r = qrow(sh, dO, b, h, t);
    int n = selected_keys(sh, idx_row(sh, idx, b, hkv, t), t, keys);
    double lse = row_softmax(sh, h, qrow(sh, q, b, h, t), K, keys, n, P);
    double delta = 0.0;
    for (int a = 0; a < n; ++a) {
        dP[a] = dot(do_r, V + (int64_t)keys[a] * D, D);
        delta += P[a] * dP[a];
    }
    if (dq_out) {
        for (int d = 0; d < D; ++d) dq_out[d] = 0.0;
        for (int a = 0; a < n; ++a) {
            double dS = P[a] * (dP[a] - delta);
            const double* kj = K + (int64_t)keys[a] * D;
            for (int d = 0; d < D; ++d) dq_out[d] += sh->scale * dS * kj[d];
        }
    }
    *lse_out = lse;
    *delta_out = delta;
}

/* dk_j and dv_j of one key (b, hkv, j) straight from their defining sums over
 * the rows that attend to j; row_lse / row_delta are [B][Hq][T]. */
static void dkdv_key(const shape_t* sh, const double* q, const double* k, const double* v,
                     const double* dO, const int32_t* idx, const double* row_lse,
                     const double* row_delta, int b, int hkv, int j, double* dk_out,
                     double* dv_out) {
    int G = sh->Hq / sh->Hkv, D = sh->D, u = j / sh->bs;
    const double* kj = krow(sh, k, b, hkv, j);
    const double* vj = krow(sh, v, b, hkv, j);
    for (int d = 0; d < D; ++d) dk_out[d] = dv_out[d] = 0.0;
    int t0 = j - (sh->Tk - sh->T);  /* the first query whose position reaches j */
    for (int t = t0 < 0 ? 0 : t0; t < sh->T; ++t) {
        if (sh->window > 0 && kpos(sh, t) >= j + sh->window) break;  /* key j left row t's window */
        if (!row_lists_block(idx_row(sh, idx, b, hkv, t), sh->S, u)) continue;
        for (int g = 0; g < G; ++g) {
            int h = hkv * G + g;
            int64_t r = ((int64_t)b * sh->Hq + h) * sh->T + t;
            const double* q_r = q + r * D;
            const double* do_r = dO + r * D;
            double Pj = exp(sh->scale * dot(q_r, kj, D) - row_lse[r]);
            double dS = Pj * (dot(do_r, vj, D) - row_delta[r]);
            for (int d = 0; d < D; ++d) {
                dk_out[d] += sh->scale * dS * q_r[d];
                dv_out[d] += Pj * do_r[d];
            }
        }
    }
}

static int shape_ok(const shape_t* sh) {
    if (sh->B < 0 || sh->T < 0 || sh->D <= 0 || sh->S <= 0 || sh->bs <= 0) return 0;
    if (sh->Tk < sh->T) return 0;
    if (sh->Hkv <= 0 || sh->Hq <= 0 || sh->Hq % sh->Hkv) return 0;
    return 1;
}

#define SHAPE_ARGS                                                                            \
    int B, int Hq, int Hkv, int T, int D, int S, int bs, double scale, const double* sink, \
        int window, int Tk
#define MAKE_SHAPE shape_t sh = {B, Hq, Hkv, T, D, S, bs, scale, sink, window, Tk}

int nsa_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Forward of the rows listed in rows[] (flat (b*Hq + h)*T + t); rows == NULL
 * means every row in order.  o_out is [n_rows][D], lse_out [n_rows]. */
int nsa_oracle_fwd_rows(SHAPE_ARGS, const double* q, const double* k, const double* v,
                        const int32_t* idx, int64_t n_rows, const int64_t* rows, double* o_out,
                        double* lse_out) {
    MAKE_SHAPE;
    if (!shape_ok(&sh)) return 1;
    int64_t cap = (int64_t)S * bs;
    int err = 0;
#pragma omp parallel
    {
        int* keys = (int*)malloc(sizeof(int) * (size_t)cap);
        double* P = (double*)malloc(sizeof(double) * (size_t)cap);
        if (!keys || !P) err = 2;
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!keys || !P) continue;
            int64_t r = rows ? rows[i] : i;
            int t = (int)(r % T), h = (int)((r / T) % Hq), b = (int)(r / ((int64_t)T * Hq));
            fwd_row(&sh, q, k, v, idx, b, h, t, o_out + i * D, lse_out + i, keys, P);
        }
        free(keys);
        free(P);
    }
    return err;
}

/* lse, Delta and (optionally) dq of the listed rows. */
int nsa_oracle_bwd_rows(SHAPE_ARGS, const double* q, const double* k, const double* v,
                        const double* dO, const int32_t* idx, int64_t n_rows,
                        const int64_t* rows, double* lse_out, double* delta_out,
                        double* dq_out) {
    MAKE_SHAPE;
    if (!shape_ok(&sh)) return 1;
    int64_t cap = (int64_t)S * bs;
    int err = 0;
#pragma omp parallel
    {
        int* keys = (int*)malloc(sizeof(int) * (size_t)cap);
        double* P = (double*)malloc(sizeof(double) * (size_t)cap);
        double* dP = (double*)malloc(sizeof(double) * (size_t)cap);
        if (!keys || !P || !dP) err = 2;
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!keys || !P || !dP) continue;
            int64_t r = rows ? rows[i] : i;
            int t = (int)(r % T), h = (int)((r / T) % Hq), b = (int)(r / ((int64_t)T * Hq));
            bwd_row(&sh, q, k, v, dO, idx, b, h, t, lse_out + i, delta_out + i,
                    dq_out ? dq_out + i * D : NULL, keys, P, dP);
        }
        free(keys);
        free(P);
        free(dP);
    }
    return err;
}

/* dk, dv of the listed keys (flat (b*Hkv + hkv)*Tk + j); keys == NULL means
 * every key.  row_lse / row_delta must hold every row [B][Hq][T] (from
 * nsa_oracle_bwd_rows over all rows).  Outputs are [n_keys][D]. */
int nsa_oracle_dkdv_keys(SHAPE_ARGS, const double* q, const double* k, const double* v,
                         const double* dO, const int32_t* idx, const double* row_lse,
                         const double* row_delta, int64_t n_keys, const int64_t* keys,
                         double* dk_out, double* dv_out) {
    MAKE_SHAPE;
    if (!shape_ok(&sh)) return 1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_keys; ++i) {
        int64_t r = keys ? keys[i] : i;
        int j = (int)(r % Tk), hkv = (int)((r / Tk) % Hkv), b = (int)(r / ((int64_t)Tk * Hkv));
        dkdv_key(&sh, q, k, v, dO, idx, row_lse, row_delta, b, hkv, j, dk_out + i * D,
                 dv_out + i * D);
    }
    return 0;
}

/* Full forward: o [B][Hq][T][D], lse [B][Hq][T]. */
int nsa_oracle_fwd(SHAPE_ARGS, const double* q, const double* k, const double* v,
                   const int32_t* idx, double* o, double* lse) {
    return nsa_oracle_fwd_rows(B, Hq, Hkv, T, D, S, bs, scale, sink, window, Tk, q, k, v, idx,
                               (int64_t)B * Hq * T, NULL, o, lse);
}

/* Full backward: dq like q, dk/dv like k; lse/delta [B][Hq][T] are outputs
 * too (delta = sum_j P_j dP_j). */
int nsa_oracle_bwd(SHAPE_ARGS, const double* q, const double* k, const double* v,
                   const double* dO, const int32_t* idx, double* dq, double* dk, double* dv,
                   double* lse, double* delta) {
    int rc = nsa_oracle_bwd_rows(B, Hq, Hkv, T, D, S, bs, scale, sink, window, Tk, q, k, v, dO,
                                 idx, (int64_t)B * Hq * T, NULL, lse, delta, dq);
    if (rc) return rc;
    return nsa_oracle_dkdv_keys(B, Hq, Hkv, T, D, S, bs, scale, sink, window, Tk, q, k, v, dO, idx,
                                lse, delta, (int64_t)B * Hkv * Tk, NULL, dk, dv);
}

/* Block -> query inversion, brute force.  For every (b, hkv, u) in order, the
 * ascending tokens t whose key set A meets block u: t lists u and its key
 * position t + Tk - T >= u*bs (a listed block that starts after it adds no
 * key, so it is not an entry);
 * each token appears once however often it lists u.  counts is
 * [B][Hkv][NB]; tokens receives the lists back to back in that order (its
 * capacity is cap entries).  Returns the total entry count, or -1 if cap is
 * too small. */
int64_t nsa_oracle_invert(int B, int Hkv, int T, int Tk, int S, int bs, int window,
                          const int32_t* idx, int32_t* counts, int32_t* tokens, int64_t cap) {
    shape_t sh = {B, Hkv, Hkv, T, 1, S, bs, 1.0, NULL, window, Tk};
    int NB = n_blocks(&sh);
    int64_t n = 0;
    for (int b = 0; b < B; ++b)
        for (int hkv = 0; hkv < Hkv; ++hkv)
            for (int u = 0; u < NB; ++u) {
                int32_t c = 0;
                for (int t = 0; t < T; ++t) {
                    if (kpos(&sh, t) < u * bs) continue;
                    if (!row_lists_block(idx_row(&sh, idx, b, hkv, t), S, u)) continue;
                    /* with a window: only rows whose window reaches a key of u */
                    if (window > 0 && (u + 1) * bs - 1 <= kpos(&sh, t) - window) continue;
                    if (n >= cap) return -1;
                    tokens[n++] = t;
                    ++c;
                }
                counts[((int64_t)b * Hkv + hkv) * NB + u] = c;
            }
    return n;
}

/* Number of useful (query-head row, key) pairs: sum over rows of |A|. */
int64_t nsa_oracle_count_pairs(int B, int Hq, int Hkv, int T, int Tk, int S, int bs,
                               const int32_t* idx) {
    shape_t sh = {B, Hq, Hkv, T, 1, S, bs, 1.0, NULL, 0, Tk};
    if (!shape_ok(&sh)) return -1;
    int G = Hq / Hkv;
    int* keys = (int*)malloc(sizeof(int) * (size_t)S * bs);
    if (!keys) return -1;
    int64_t n = 0;
    for (int b = 0; b < B; ++b)
        for (int hkv = 0; hkv < Hkv; ++hkv)
            for (int t = 0; t < T; ++t)
                n += (int64_t)G * selected_keys(&sh, idx_row(&sh, idx, b, hkv, t), t, keys);
    free(keys);
    return n;
}
