/*
 * Exact-attention oracle: plain, slow, fp64, CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or helper
 * with the GPU library.
 *
 * Sources (pofe.ai, "FlashAttention for inference: tiled prefill and split-KV
 * decoding", cited below as [pofe]):
 *   - the plain definition S = Q K^T / sqrt(d), P = softmax(S), O = P V
 *     ([pofe] section "The bottleneck it attacks");
 *   - the online-softmax update with running max m, running sum l and
 *     unnormalised output o~, initial state (-inf, 0, 0), final o = o~ / l
 *     ([pofe] section "The online softmax, with every symbol defined");
 *   - the combine rule for independent partials: a softmax over the chunks'
 *     log-sum-exps lambda_k = m_k + log l_k ([pofe] same section, and the
 *     `merge` helper in section "Minimal implementation");
 *   - the query-tile / key-tile loop with causal tile skipping and a masked
 *     diagonal tile ([pofe] section "Prefill: tiles, loop order and the
 *     tensor cores", pseudocode);
 *   - split-KV decoding over a paged cache read through a block table
 *     ([pofe] sections "Decode: a different bottleneck" and "Minimal
 *     implementation": cache (num_blocks, block_size, kv_heads, head_dim),
 *     block_table (batch, max_blocks) int32).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - query head h uses KV head h / (Hq / Hkv) (contiguous groups);
 *   - the log-sum-exp is the natural log over *scaled* scores;
 *   - causal prefill is square: row i sees keys 0..i;
 *   - a row with no visible key has O = 0 and LSE = -inf (an empty sum);
 *   - a block with no visible key for a row leaves that row's state unchanged
 *     (the -inf - (-inf) case is guarded).
 *
 * Every function works in double precision.  Layouts (row-major, contiguous):
 *   prefill  q, o: [B][Hq][N][d]   k, v: [B][Hkv][N][d]   lse: [B][Hq][N]
 *   decode   q, o: [B][Hq][d]      lse: [B][Hq]
 *            contiguous cache k, v: [B][S][Hkv][d]   (block_table == NULL)
 *            paged cache      k, v: [num_blocks][P][Hkv][d]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads of every parallel loop below: 0 = the OpenMP runtime's default.  The   */
/* count is passed to each parallel region explicitly (num_threads clause), so a */
/* request holds even where the process carries more than one OpenMP runtime     */
/* (the calling thread's settings would then live in the other one).  Results do */
/* not depend on it: every row or sequence is computed by one thread.            */
static int g_threads = 0;

static int oracle_threads(void)
{
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* The plain definition for one query row (two passes, no rescaling) over    */
/* the keys j0 .. n-1.  Keys/values are rows of d doubles, `stride` doubles  */
/* apart; `s` is caller scratch of at least n doubles.  With softcap > 0     */
/* each score becomes softcap * tanh(s / softcap) before the softmax; a      */
/* window is a j0 above 0.  (Sliding windows and logit soft-capping are      */
/* variants the pofe.ai page lists in section "Interaction with              */
/* post-trained models"; their definitions are the readings in the notes.)   */
/* ------------------------------------------------------------------------ */
static void plain_row_ext(const double *q, const double *k, const double *v,
                          size_t stride, int64_t j0, int64_t n, int d, double scale,
                          double softcap, double *s, double *o, double *lse)
{
    if (j0 < 0) j0 = 0;
    if (n <= j0) {
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    /* scores s_j = scale * <q, k_j>, soft-capped if asked */
    for (int64_t j = j0; j < n; ++j) {
        const double *kj = k + (size_t)j * stride;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += q[c] * kj[c];
        s[j] = scale * acc;
        if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);
    }
    /* m = max_j s_j */
    double m = s[j0];
    for (int64_t j = j0 + 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    /* Z = sum_j exp(s_j - m);  O = (1/Z) sum_j exp(s_j - m) v_j */
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    double z = 0.0;
    for (int64_t j = j0; j < n; ++j) {
        const double w = exp(s[j] - m);
        const double *vj = v + (size_t)j * stride;
        z += w;
        for (int c = 0; c < d; ++c) o[c] += w * vj[c];
    }
    for (int c = 0; c < d; ++c) o[c] /= z;
    *lse = m + log(z);
}

/* ------------------------------------------------------------------------ */
/* Prefill by the plain definition.                                          */
/* Computes rows i with i % row_step == 0 (row_step = 1: every row); other   */
/* rows of o and lse are left untouched.  causal != 0: row i sees keys 0..i; */
/* otherwise all N keys.  Returns 0, or -1 on bad arguments / no memory.    */
/* ------------------------------------------------------------------------ */
int oracle_prefill_ext(const double *q, const double *k, const double *v,
                       double *o, double *lse, int B, int Hq, int Hkv, int N, int d,
                       int causal, double scale, int window, double softcap, int row_step)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || N < 0 || d <= 0 || Hq % Hkv != 0 || row_step < 1 ||
        softcap < 0.0)
        return -1;
    const int g = Hq / Hkv;
    const int64_t rows = (int64_t)B * Hq * N;
    int err = 0;
#pragma omp parallel num_threads(oracle_threads())
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int i = (int)(r % N);
                if (i % row_step) continue;
                const int64_t bh = r / N;          /* b * Hq + h */
                const int b = (int)(bh / Hq), h = (int)(bh % Hq);
                const int hk = h / g;
                const double *kb = k + ((size_t)b * Hkv + hk) * (size_t)N * d;
                const double *vb = v + ((size_t)b * Hkv + hk) * (size_t)N * d;
                /* visible keys: j <= i when causal; j >= i - window when window >= 0 */
                const int64_t n = causal ? (int64_t)i + 1 : (int64_t)N;
                const int64_t j0 = window >= 0 ? (int64_t)i - window : 0;
                plain_row_ext(q + (size_t)r * d, kb, vb, (size_t)d, j0, n, d, scale, softcap, s,
                              o + (size_t)r * d, lse + r);
            }
            free(s);
        }
    }
    return err ? -1 : 0;
}

int oracle_prefill(const double *q, const double *k, const double *v,
                   double *o, double *lse, int B, int Hq, int Hkv, int N, int d,
                   int causal, double scale, int row_step)
{
    return oracle_prefill_ext(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, -1, 0.0, row_step);
}

/* ------------------------------------------------------------------------ */
/* Gather one sequence's keys/values for one KV head into contiguous rows.   */
/* Token t of sequence b lives in physical page block_table[b][t / P],       */
/* slot t % P; with block_table == NULL the cache is [B][S][Hkv][d] with     */
/* S = max_blocks * P.                                                       */
/* ------------------------------------------------------------------------ */
static int gather_seq(const double *cache, const int32_t *block_table,
                      int b, int hk, int64_t len, int Hkv, int d, int P,
                      int max_blocks, double *dst)
{
    const size_t row = (size_t)Hkv * d;
    for (int64_t t = 0; t < len; ++t) {
        const double *src;
        if (block_table) {
            const int32_t page = block_table[(size_t)b * max_blocks + t / P];
            if (page < 0) return -1;
            src = cache + ((size_t)page * P + (size_t)(t % P)) * row + (size_t)hk * d;
        } else {
            src = cache + ((size_t)b * max_blocks * P + (size_t)t) * row + (size_t)hk * d;
        }
        memcpy(dst + (size_t)t * d, src, sizeof(double) * (size_t)d);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode (one query token per sequence) by the plain definition, keys       */
/* 0..seq_lens[b]-1 gathered through the block table (or contiguous).       */
/* ------------------------------------------------------------------------ */
int oracle_decode_ext(const double *q, const double *k_cache, const double *v_cache,
                      const int32_t *block_table, const int32_t *seq_lens,
                      double *o, double *lse, int B, int Hq, int Hkv, int d,
                      int page_size, int max_blocks, double scale, int window, double softcap)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0 || page_size <= 0 ||
        max_blocks < 0 || softcap < 0.0)
        return -1;
    const int g = Hq / Hkv;
    const int64_t cap = (int64_t)max_blocks * page_size;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > cap) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads())
    for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk) {
        const int b = (int)(bk / Hkv), hk = (int)(bk % Hkv);
        const int64_t len = seq_lens[b];
        double *kk = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1) * d);
        double *vv = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1) * d);
        double *s = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
        if (!kk || !vv || !s ||
            gather_seq(k_cache, block_table, b, hk, len, Hkv, d, page_size, max_blocks, kk) ||
            gather_seq(v_cache, block_table, b, hk, len, Hkv, d, page_size, max_blocks, vv)) {
#pragma omp atomic write
            err = 1;
        } else {
            /* the query is token len - 1: with a window it sees keys len-1-window .. len-1 */
            const int64_t j0 = window >= 0 ? len - 1 - window : 0;
            for (int j = 0; j < g; ++j) {
                const int h = hk * g + j;
                const size_t r = (size_t)b * Hq + h;
                plain_row_ext(q + r * d, kk, vv, (size_t)d, j0, len, d, scale, softcap, s, o + r * d,
                              lse + r);
            }
        }
        free(kk);
        free(vv);
        free(s);
    }
    return err ? -1 : 0;
}

int oracle_decode(const double *q, const double *k_cache, const double *v_cache,
                  const int32_t *block_table, const int32_t *seq_lens,
                  double *o, double *lse, int B, int Hq, int Hkv, int d,
                  int page_size, int max_blocks, double scale)
{
    return oracle_decode_ext(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d,
                             page_size, max_blocks, scale, -1, 0.0);
}

/* ------------------------------------------------------------------------ */
/* The pages' online-softmax update, one row.                                 */
/*   m_new = max(m, max_t s_t);  c = exp(m - m_new)  (0 when m = -inf);      */
/*   l = c*l + sum_t exp(s_t - m_new);  o~ = c*o~ + sum_t exp(s_t - m_new) v_t */
/* Masked scores are -inf.  A block whose scores are all -inf (and a state    */
/* still at m = -inf) leaves the state unchanged.                            */
/* ------------------------------------------------------------------------ */
typedef struct {
    double m, l, c; /* running max, running sum, last correction factor */
} row_state;

static void online_update(row_state *st, double *ot, const double *s,
                          const double *const *vrows, int nb, int d)
{
    double bmax = -INFINITY;
    for (int t = 0; t < nb; ++t)
        if (s[t] > bmax) bmax = s[t];
    const double m_new = st->m > bmax ? st->m : bmax;
    if (m_new == -INFINITY) { /* nothing visible yet: state unchanged */
        st->c = 1.0;
        return;
    }
    const double c = (st->m == -INFINITY) ? 0.0 : exp(st->m - m_new);
    double lsum = 0.0;
    for (int x = 0; x < d; ++x) ot[x] *= c;
    for (int t = 0; t < nb; ++t) {
        if (s[t] == -INFINITY) continue;
        const double p = exp(s[t] - m_new);
        lsum += p;
        for (int x = 0; x < d; ++x) ot[x] += p * vrows[t][x];
    }
    st->l = c * st->l + lsum;
    st->m = m_new;
    st->c = c;
}

/* final o = o~ / l and lambda = m + log l; an empty row gives 0 and -inf */
static void online_finish(const row_state *st, const double *ot, int d, double *o, double *lse)
{
    if (st->m == -INFINITY || st->l == 0.0) {
        for (int x = 0; x < d; ++x) o[x] = 0.0;
        *lse = -INFINITY;
        return;
    }
    for (int x = 0; x < d; ++x) o[x] = ot[x] / st->l;
    *lse = st->m + log(st->l);
}

/* ------------------------------------------------------------------------ */
/* Worked-example trace: one row with given scores s[0..n) and scalar        */
/* values v[0..n), blocks of `block` keys.  After block j (0-based) writes   */
/* m_out[j], l_out[j], o_out[j] (= o~), c_out[j].  Returns the number of     */
/* blocks, final output in *o and log-sum-exp in *lse.                       */
/* ------------------------------------------------------------------------ */
int oracle_online_trace(const double *s, const double *v, int n, int block,
                        double *m_out, double *l_out, double *o_out, double *c_out,
                        double *o, double *lse)
{
    if (n < 0 || block <= 0) return -1;
    row_state st = {-INFINITY, 0.0, 1.0};
    double ot = 0.0;
    int nblk = 0;
    for (int j0 = 0; j0 < n; j0 += block, ++nblk) {
        const int nb = (n - j0 < block) ? n - j0 : block;
        const double *vr[nb > 0 ? nb : 1];
        for (int t = 0; t < nb; ++t) vr[t] = v + j0 + t;
        online_update(&st, &ot, s + j0, vr, nb, 1);
        m_out[nblk] = st.m;
        l_out[nblk] = st.l;
        o_out[nblk] = ot;
        c_out[nblk] = st.c;
    }
    online_finish(&st, &ot, 1, o, lse);
    return nblk;
}

/* ------------------------------------------------------------------------ */
/* Prefill by the pages' tiled algorithm: for each (sequence, head, query    */
/* tile of Br rows), walk key tiles of Bc columns up to the tile's causal    */
/* limit, computing the Br x Bc score tile (diagonal tiles masked) and       */
/* applying the online update row by row.  Same layouts as oracle_prefill.   */
/* ------------------------------------------------------------------------ */
int oracle_prefill_tiled(const double *q, const double *k, const double *v,
                         double *o, double *lse, int B, int Hq, int Hkv, int N, int d,
                         int causal, double scale, int Br, int Bc)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || N < 0 || d <= 0 || Hq % Hkv != 0 || Br <= 0 || Bc <= 0)
        return -1;
    const int g = Hq / Hkv;
    const int ntiles = (N + Br - 1) / Br;
    const int64_t work = (int64_t)B * Hq * ntiles;
    int err = 0;
#pragma omp parallel num_threads(oracle_threads())
    {
        row_state *st = (row_state *)malloc(sizeof(row_state) * (size_t)Br);
        double *ot = (double *)malloc(sizeof(double) * (size_t)Br * d);
        double *S = (double *)malloc(sizeof(double) * (size_t)Br * Bc);
        const double **vr = (const double **)malloc(sizeof(double *) * (size_t)Bc);
        if (!st || !ot || !S || !vr) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t w = 0; w < work; ++w) {
                const int ti = (int)(w % ntiles);
                const int64_t bh = w / ntiles;
                const int b = (int)(bh / Hq), h = (int)(bh % Hq), hk = h / g;
                const double *qb = q + (size_t)bh * N * d;
                const double *kb = k + ((size_t)b * Hkv + hk) * (size_t)N * d;
                const double *vb = v + ((size_t)b * Hkv + hk) * (size_t)N * d;
                const int r0 = ti * Br;
                const int nr = (N - r0 < Br) ? N - r0 : Br;
                for (int r = 0; r < nr; ++r) {
                    st[r].m = -INFINITY; st[r].l = 0.0; st[r].c = 1.0;
                    for (int x = 0; x < d; ++x) ot[(size_t)r * d + x] = 0.0;
                }
                /* last key any row of this tile may see */
                const int kmax = causal ? r0 + nr - 1 : N - 1;
                for (int j0 = 0; j0 <= kmax; j0 += Bc) { /* tiles above the diagonal skipped */
                    const int nc = (N - j0 < Bc) ? N - j0 : Bc;
                    for (int r = 0; r < nr; ++r) {
                        const int i = r0 + r;
                        const double *qi = qb + (size_t)i * d;
                        for (int t = 0; t < nc; ++t) {
                            const int j = j0 + t;
                            if (causal && j > i) { S[(size_t)r * Bc + t] = -INFINITY; continue; }
                            const double *kj = kb + (size_t)j * d;
                            double acc = 0.0;
                            for (int x = 0; x < d; ++x) acc += qi[x] * kj[x];
                            S[(size_t)r * Bc + t] = scale * acc;
                        }
                    }
                    for (int t = 0; t < nc; ++t) vr[t] = vb + (size_t)(j0 + t) * d;
                    for (int r = 0; r < nr; ++r)
                        online_update(&st[r], ot + (size_t)r * d, S + (size_t)r * Bc, vr, nc, d);
                }
                for (int r = 0; r < nr; ++r) {
                    const size_t row = (size_t)bh * N + (size_t)(r0 + r);
                    online_finish(&st[r], ot + (size_t)r * d, d, o + row * d, lse + row);
                }
            }
        }
        free(st); free(ot); free(S); free(vr);
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Combine rule for independent partials (one row at a time):                */
/*   Lambda = log sum_k exp(lambda_k)  (evaluated as max + log sum exp(. - max)) */
/*   o = sum_k exp(lambda_k - Lambda) o_k                                    */
/* o_parts: [rows][max_splits][d], lse_parts: [rows][max_splits];             */
/* n_splits (may be NULL = max_splits for every row) gives how many leading   */
/* partials of each row are used.  Zero partials (or all -inf) give o = 0,    */
/* Lambda = -inf.                                                            */
/* ------------------------------------------------------------------------ */
int oracle_lse_combine(const double *o_parts, const double *lse_parts, const int32_t *n_splits,
                       int rows, int max_splits, int d, double *o, double *lse)
{
    if (rows < 0 || max_splits < 0 || d <= 0) return -1;
    for (int r = 0; r < rows; ++r) {
        const int ns = n_splits ? n_splits[r] : max_splits;
        if (ns < 0 || ns > max_splits) return -1;
        const double *lam = lse_parts + (size_t)r * max_splits;
        const double *op = o_parts + (size_t)r * max_splits * d;
        double mx = -INFINITY;
        for (int kx = 0; kx < ns; ++kx)
            if (lam[kx] > mx) mx = lam[kx];
        double *orow = o + (size_t)r * d;
        for (int x = 0; x < d; ++x) orow[x] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int kx = 0; kx < ns; ++kx) z += exp(lam[kx] - mx);
        const double Lam = mx + log(z);
        for (int kx = 0; kx < ns; ++kx) {
            const double w = exp(lam[kx] - Lam);
            for (int x = 0; x < d; ++x) orow[x] += w * op[(size_t)kx * d + x];
        }
        lse[r] = Lam;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Split-KV decode by the pages' scheme: each sequence's keys are cut into   */
/* chunks of `chunk` tokens; each chunk runs the online update over blocks   */
/* of `block` tokens and yields (o_k, lambda_k); the partials are merged by  */
/* the combine rule.  Same layouts as oracle_decode.  If o_parts/lse_parts   */
/* are non-NULL they receive the partials ([B*Hq][max_chunks][d] and         */
/* [B*Hq][max_chunks], max_chunks = ceil(max_blocks*P / chunk)); chunks past */
/* a sequence's length are written as (0, -inf).                             */
/* ------------------------------------------------------------------------ */
int oracle_split_decode(const double *q, const double *k_cache, const double *v_cache,
                        const int32_t *block_table, const int32_t *seq_lens,
                        double *o, double *lse, int B, int Hq, int Hkv, int d,
                        int page_size, int max_blocks, double scale, int chunk, int block,
                        double *o_parts, double *lse_parts)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0 || page_size <= 0 ||
        max_blocks < 0 || chunk <= 0 || block <= 0)
        return -1;
    const int g = Hq / Hkv;
    const int64_t cap = (int64_t)max_blocks * page_size;
    const int max_chunks = (int)((cap + chunk - 1) / chunk);
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > cap) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(oracle_threads())
    for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk) {
        const int b = (int)(bk / Hkv), hk = (int)(bk % Hkv);
        const int64_t len = seq_lens[b];
        const size_t alloc_rows = (size_t)(len > 0 ? len : 1);
        double *kk = (double *)malloc(sizeof(double) * alloc_rows * d);
        double *vv = (double *)malloc(sizeof(double) * alloc_rows * d);
        double *s = (double *)malloc(sizeof(double) * (size_t)block);
        const double **vr = (const double **)malloc(sizeof(double *) * (size_t)block);
        double *ot = (double *)malloc(sizeof(double) * (size_t)d);
        double *po = (double *)malloc(sizeof(double) * (size_t)(max_chunks > 0 ? max_chunks : 1) * d);
        double *pl = (double *)malloc(sizeof(double) * (size_t)(max_chunks > 0 ? max_chunks : 1));
        if (!kk || !vv || !s || !vr || !ot || !po || !pl ||
            gather_seq(k_cache, block_table, b, hk, len, Hkv, d, page_size, max_blocks, kk) ||
            gather_seq(v_cache, block_table, b, hk, len, Hkv, d, page_size, max_blocks, vv)) {
#pragma omp atomic write
            err = 1;
        } else {
            for (int j = 0; j < g; ++j) {
                const int h = hk * g + j;
                const size_t r = (size_t)b * Hq + h;
                const double *qr = q + r * d;
                for (int c = 0; c < max_chunks; ++c) {
                    const int64_t t0 = (int64_t)c * chunk;
                    int64_t t1 = t0 + chunk;
                    if (t1 > len) t1 = len;
                    row_state st = {-INFINITY, 0.0, 1.0};
                    for (int x = 0; x < d; ++x) ot[x] = 0.0;
                    for (int64_t u0 = t0; u0 < t1; u0 += block) {
                        const int nb = (int)((t1 - u0 < block) ? t1 - u0 : block);
                        for (int t = 0; t < nb; ++t) {
                            const double *kt = kk + (size_t)(u0 + t) * d;
                            double acc = 0.0;
                            for (int x = 0; x < d; ++x) acc += qr[x] * kt[x];
                            s[t] = scale * acc;
                            vr[t] = vv + (size_t)(u0 + t) * d;
                        }
                        online_update(&st, ot, s, vr, nb, d);
                    }
                    online_finish(&st, ot, d, po + (size_t)c * d, pl + c);
                }
                const int32_t nsp = (int32_t)max_chunks;
                oracle_lse_combine(po, pl, &nsp, 1, max_chunks, d, o + r * d, lse + r);
                if (o_parts && lse_parts) {
                    memcpy(o_parts + r * (size_t)max_chunks * d, po,
                           sizeof(double) * (size_t)max_chunks * d);
                    memcpy(lse_parts + r * (size_t)max_chunks, pl, sizeof(double) * (size_t)max_chunks);
                }
            }
        }
        free(kk); free(vv); free(s); free(vr); free(ot); free(po); free(pl);
    }
    return err ? -1 : 0;
}

/* number of OpenMP threads the oracle will use */
/* ------------------------------------------------------------------------ */
/* FP8 inputs.  One byte in the OCP 8-bit floating-point format E4M3 (the    */
/* "FN" variant: finite values only): bit 7 sign, bits 6..3 exponent with    */
/* bias 7, bits 2..0 mantissa.  Exponent field 0 holds subnormals            */
/* (mantissa / 8 * 2^-6); the code with every exponent and mantissa bit set  */
/* (0x7f, 0xff) is NaN; there is no infinity, so the largest value is        */
/* 1.75 * 2^8 = 448.  Written from that definition; the pages name FP8       */
/* attention ([pofe] "The bottleneck it attacks", the FlashAttention-3 line) */
/* but not its format, which is the one the gfx950 matrix cores take.        */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_value(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

int oracle_e4m3_decode(const uint8_t *in, double *out, int64_t n)
{
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(in[i]);
    return 0;
}

/* Set the number of OpenMP threads the oracle's parallel loops use (n > 0), e.g. one
 * for a single-core timing; returns the count now in effect. */
int oracle_set_num_threads(int n)
{
    if (n > 0) g_threads = n;
    return oracle_threads();
}

int oracle_num_threads(void)
{
    return oracle_threads();
}

/* Threads a parallel region of the oracle actually runs with (the runtime may */
/* grant fewer than requested). */
int oracle_threads_used(void)
{
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(oracle_threads())
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#endif
    return used;
}
