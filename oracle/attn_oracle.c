/*
 * attn_oracle.c -- plain fp64 CPU reference for paged prefix-shared attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (prefix_shared_paged_amd/) never links, imports or calls it, and shares no
 * code with it.
 *
 * What it computes is the plain definition of attention that the pages state:
 *   - the score of a query against a key is their dot product scaled by
 *     1/sqrt(head_dim) (the PagedDecode kernel of "SGLang 深度拆解"
 *     (chenxutan.com), section 3.2, divides the score by sqrtf(head_dim));
 *   - the output is the softmax-weighted sum of the values over the visible
 *     keys (same section: max pass, then exp-sum and weighted sum, then
 *     divide);
 *   - a new token attends to the cached prefix plus the new tokens up to and
 *     including itself (section 2.3 / the PagedPrefill kernel of section 3.2
 *     walks the whole context; the causal cut-off j <= t is the plain reading
 *     of "prefix + new tokens" generation order);
 *   - query head h reads KV head h / (Hq / Hkv) (grouped-query attention,
 *     contiguous groups).
 *
 * It works on the LOGICAL per-request sequences (K, V of positions 0..L-1),
 * never through a slot pool or a req_to_token table.  All arithmetic is in
 * double; inputs are float32 arrays whose values are widened exactly.
 *
 * Two orders of evaluation are provided so that each pins the other:
 *   method 0: two passes -- maximum first, then exp-sum and weighted sum
 *             (the order of the PagedDecode kernel, section 3.2);
 *   method 1: one pass with a running maximum that rescales the running sum
 *             and accumulator whenever the maximum grows (the online-softmax
 *             update of the PagedPrefill kernel, section 3.2).
 *
 * A quantised KV cache (FP8 codes, "SGLang 深度拆解" section 4.3) is given as
 * the decoded code values in K / V plus one factor per KV head for K and one
 * for V: the key used is K * kscale[kv] and the value V * vscale[kv], each
 * product formed in double (exact for float32 operands) before it is used.
 *
 * Plus the merge of two partial softmax states (m, l, o) over disjoint key
 * sets.  The pages do not print this merge; it is the online-softmax update
 * of section 3.2 applied to a whole block instead of a single key.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n_rows;           /* query rows */
    const int64_t *row_req;   /* request of each query row */
    const int64_t *row_pos;   /* absolute position t of each query row */
    const int64_t *kv_off;    /* [n_req+1] first logical K/V row of each request */
    const float *K, *V, *Q;
    int32_t Hq, Hkv, D;
    int32_t Dv;               /* value width (V rows [Hkv, Dv], O rows Dv) */
    double scale;
    const double *kscale, *vscale; /* per KV head dequantisation factors, NULL -> 1 */
    const int32_t *heads;     /* q heads to evaluate */
    int32_t n_heads;
    const int64_t *key_lo, *key_hi; /* per query row key range, NULL -> [0, t] */
    int32_t method;
    int32_t n_threads;
    double *O, *M, *L, *LSE;  /* outputs, indexed [row][head slot] */
    int64_t next;             /* work counter */
    pthread_mutex_t mu;
} job_t;

/* Evaluate one (query row, head) pair. */
static void eval_one(job_t *jb, int64_t row, int32_t hs, double *sbuf) {
    const int32_t D = jb->D, Dv = jb->Dv, Hq = jb->Hq, Hkv = jb->Hkv;
    const int32_t h = jb->heads ? jb->heads[hs] : hs;
    const int32_t group = Hq / Hkv;
    const int32_t kvh = h / group;
    const double ks = jb->kscale ? jb->kscale[kvh] : 1.0;
    const double vs = jb->vscale ? jb->vscale[kvh] : 1.0;
    const int64_t r = jb->row_req[row];
    const int64_t t = jb->row_pos[row];
    const int64_t base = jb->kv_off[r];
    int64_t lo = jb->key_lo ? jb->key_lo[row] : 0;
    int64_t hi = jb->key_hi ? jb->key_hi[row] : t + 1;
    if (hi > t + 1) hi = t + 1;              /* causal: keys j <= t only */
    const float *q = jb->Q + (row * (int64_t)Hq + h) * D;
    const int64_t ho = (int64_t)jb->n_heads * row + hs;
    double *o = jb->O + ho * Dv;
    for (int32_t d = 0; d < Dv; d++) o[d] = 0.0;

    if (hi <= lo) { /* empty key set: l = 0, m = -inf, o = 0 */
        jb->M[ho] = -INFINITY;
        jb->L[ho] = 0.0;
        jb->LSE[ho] = -INFINITY;
        return;
    }
    double m = -INFINITY, l = 0.0;
    if (jb->method == 0) {
        /* pass 1: scores and their maximum */
        for (int64_t j = lo; j < hi; j++) {
            const float *k = jb->K + ((base + j) * Hkv + kvh) * D;
            double s = 0.0;
            for (int32_t d = 0; d < D; d++) s += (double)q[d] * ((double)k[d] * ks);
            s *= jb->scale;
            sbuf[j - lo] = s;
            if (s > m) m = s;
        }
        /* pass 2: exp-sum and weighted sum of values */
        for (int64_t j = lo; j < hi; j++) {
            const float *v = jb->V + ((base + j) * Hkv + kvh) * Dv;
            double w = exp(sbuf[j - lo] - m);
            l += w;
            for (int32_t d = 0; d < Dv; d++) o[d] += w * ((double)v[d] * vs);
        }
    } else {
        /* one pass, running maximum */
        for (int64_t j = lo; j < hi; j++) {
            const float *k = jb->K + ((base + j) * Hkv + kvh) * D;
            const float *v = jb->V + ((base + j) * Hkv + kvh) * Dv;
            double s = 0.0;
            for (int32_t d = 0; d < D; d++) s += (double)q[d] * ((double)k[d] * ks);
            s *= jb->scale;
            double m_new = s > m ? s : m;
            double c = exp(m - m_new);      /* rescale of what came before */
            double w = exp(s - m_new);
            l = l * c + w;
            for (int32_t d = 0; d < Dv; d++) o[d] = o[d] * c + w * ((double)v[d] * vs);
            m = m_new;
        }
    }
    for (int32_t d = 0; d < Dv; d++) o[d] /= l;
    jb->M[ho] = m;
    jb->L[ho] = l;
    jb->LSE[ho] = m + log(l);
}

static void *worker(void *arg) {
    job_t *jb = (job_t *)arg;
    const int64_t total = jb->n_rows * jb->n_heads;
    /* scratch for the scores of one query row (two-pass method) */
    int64_t maxlen = 1;
    for (int64_t i = 0; i < jb->n_rows; i++) {
        int64_t len = jb->row_pos[i] + 1;
        if (len > maxlen) maxlen = len;
    }
    double *sbuf = (double *)malloc(sizeof(double) * (size_t)maxlen);
    if (!sbuf) return (void *)1;
    /* work units per grab: small calls still spread over all threads */
    int64_t chunk = total / ((int64_t)jb->n_threads * 8);
    if (chunk < 1) chunk = 1;
    if (chunk > 16) chunk = 16;
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int64_t start = jb->next;
        jb->next += chunk;
        pthread_mutex_unlock(&jb->mu);
        if (start >= total) break;
        int64_t end = start + chunk < total ? start + chunk : total;
        for (int64_t w = start; w < end; w++)
            eval_one(jb, w / jb->n_heads, (int32_t)(w % jb->n_heads), sbuf);
    }
    free(sbuf);
    return NULL;
}

/*
 * oracle_attention, oracle_attention_kv_scaled, oracle_attention_dv --
 * softmax(q k^T * scale, causal) v for a set of query rows.
 *
 *   n_req, kv_off[n_req+1]: logical K/V rows of request r are
 *       K[kv_off[r] .. kv_off[r+1]) (layout [rows, Hkv, D], float32).
 *   n_rows, row_req[n_rows], row_pos[n_rows]: query row i belongs to request
 *       row_req[i] and sits at absolute position row_pos[i] of that request.
 *   Q: [n_rows, Hq, D] float32.
 *   heads[n_heads]: q heads to evaluate (NULL -> all Hq heads, n_heads = Hq).
 *   key_lo/key_hi[n_rows]: optional key range [lo, hi) intersected with the
 *       causal range [0, t]; NULL -> the causal range.
 *   O: [n_rows, n_heads, D] double;  M, Lsum, LSE: [n_rows, n_heads] double.
 *       M is the maximum score, Lsum = sum_j exp(s_j - M), LSE = M + ln Lsum.
 *       An empty key range gives O = 0, Lsum = 0, M = LSE = -inf.
 *   method: 0 two-pass, 1 online.  n_threads >= 1.
 *   kscale, vscale [Hkv] (oracle_attention_kv_scaled / _dv, NULL -> 1): the
 *       keys and values used are K * kscale[kv] and V * vscale[kv].
 *   Dv (oracle_attention_dv; the others use Dv = D): the width of a value row,
 *       V [rows, Hkv, Dv] and O [n_rows, n_heads, Dv] -- for attention in a
 *       latent space where scores use D dims and values Dv of them.
 * Returns 0, or -1 on invalid arguments / allocation failure.
 */
int oracle_attention_dv(int64_t n_req, const int64_t *kv_off, const float *K, const float *V,
                        const double *kscale, const double *vscale,
                        int64_t n_rows, const int64_t *row_req, const int64_t *row_pos,
                        const float *Q, int32_t Hq, int32_t Hkv, int32_t D, int32_t Dv, double scale,
                               const int32_t *heads, int32_t n_heads,
                               const int64_t *key_lo, const int64_t *key_hi,
                               double *O, double *M, double *Lsum, double *LSE,
                               int32_t method, int32_t n_threads) {
    if (Hq <= 0 || Hkv <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv != 0 || n_threads < 1) return -1;
    if (!heads) n_heads = Hq;
    for (int64_t i = 0; i < n_rows; i++) {
        int64_t r = row_req[i];
        if (r < 0 || r >= n_req) return -1;
        if (row_pos[i] < 0 || row_pos[i] >= kv_off[r + 1] - kv_off[r]) return -1;
    }
    for (int32_t i = 0; heads && i < n_heads; i++)
        if (heads[i] < 0 || heads[i] >= Hq) return -1;
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.n_rows = n_rows; jb.row_req = row_req; jb.row_pos = row_pos; jb.kv_off = kv_off;
    jb.K = K; jb.V = V; jb.kscale = kscale; jb.vscale = vscale; jb.Q = Q; jb.Hq = Hq; jb.Hkv = Hkv; jb.D = D; jb.Dv = Dv; jb.scale = scale;
    jb.heads = heads; jb.n_heads = n_heads; jb.key_lo = key_lo; jb.key_hi = key_hi;
    jb.method = method; jb.n_threads = n_threads; jb.O = O; jb.M = M; jb.L = Lsum; jb.LSE = LSE; jb.next = 0;
    pthread_mutex_init(&jb.mu, NULL);
    int rc = 0;
    if (n_threads == 1) {
        if (worker(&jb) != NULL) rc = -1;
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
        if (!th) { pthread_mutex_destroy(&jb.mu); return -1; }
        int started = 0;
        for (int i = 0; i < n_threads; i++) {
            if (pthread_create(&th[i], NULL, worker, &jb) != 0) { rc = -1; break; }
            started++;
        }
        for (int i = 0; i < started; i++) {
            void *ret = NULL;
            pthread_join(th[i], &ret);
            if (ret != NULL) rc = -1;
        }
        free(th);
    }
    pthread_mutex_destroy(&jb.mu);
    return rc;
}

int oracle_attention(int64_t n_req, const int64_t *kv_off, const float *K, const float *V,
                     int64_t n_rows, const int64_t *row_req, const int64_t *row_pos,
                     const float *Q, int32_t Hq, int32_t Hkv, int32_t D, double scale,
                     const int32_t *heads, int32_t n_heads,
                     const int64_t *key_lo, const int64_t *key_hi,
                     double *O, double *M, double *Lsum, double *LSE,
                     int32_t method, int32_t n_threads) {
    return oracle_attention_dv(n_req, kv_off, K, V, NULL, NULL, n_rows, row_req, row_pos, Q, Hq, Hkv, D, D,
                               scale, heads, n_heads, key_lo, key_hi, O, M, Lsum, LSE, method, n_threads);
}

int oracle_attention_kv_scaled(int64_t n_req, const int64_t *kv_off, const float *K, const float *V,
                               const double *kscale, const double *vscale,
                               int64_t n_rows, const int64_t *row_req, const int64_t *row_pos,
                               const float *Q, int32_t Hq, int32_t Hkv, int32_t D, double scale,
                               const int32_t *heads, int32_t n_heads,
                               const int64_t *key_lo, const int64_t *key_hi,
                               double *O, double *M, double *Lsum, double *LSE,
                               int32_t method, int32_t n_threads) {
    return oracle_attention_dv(n_req, kv_off, K, V, kscale, vscale, n_rows, row_req, row_pos, Q, Hq, Hkv, D,
                               D, scale, heads, n_heads, key_lo, key_hi, O, M, Lsum, LSE, method, n_threads);
}

/*
 * oracle_attention_probs -- the explicit attention-probability matrix of one
 * request and one q head (small inputs only).
 *   K: [L, Hkv, D], Q: [n_q, Hq, D] with positions pos[n_q] (each < L).
 *   P: [n_q, L] double, P[i][j] = exp(s_ij - max_i) / sum_i for j <= pos[i],
 *   0 for the keys a query must not see.
 */
int oracle_attention_probs(int64_t L, const float *K, int64_t n_q, const int64_t *pos,
                           const float *Q, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t h, double scale, double *P) {
    if (Hq % Hkv != 0 || h < 0 || h >= Hq) return -1;
    const int32_t kvh = h / (Hq / Hkv);
    for (int64_t i = 0; i < n_q; i++) {
        if (pos[i] < 0 || pos[i] >= L) return -1;
        const float *q = Q + (i * Hq + h) * D;
        double *p = P + i * L;
        double m = -INFINITY;
        for (int64_t j = 0; j < L; j++) {
            p[j] = 0.0;
            if (j > pos[i]) continue;
            const float *k = K + (j * Hkv + kvh) * D;
            double s = 0.0;
            for (int32_t d = 0; d < D; d++) s += (double)q[d] * (double)k[d];
            p[j] = s * scale;
            if (p[j] > m) m = p[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j <= pos[i]; j++) { p[j] = exp(p[j] - m); l += p[j]; }
        for (int64_t j = 0; j <= pos[i]; j++) p[j] /= l;
    }
    return 0;
}

/*
 * oracle_merge_states -- combine partial softmax states over two disjoint key
 * sets A and B:  m = max(mA, mB);  l = lA e^(mA-m) + lB e^(mB-m);
 * o = (lA e^(mA-m) oA + lB e^(mB-m) oB) / l.  A state with l = 0 (empty set,
 * m = -inf) is the identity.  n states of dimension D each; outputs may alias
 * the A inputs.
 */
void oracle_merge_states(int64_t n, int32_t D,
                         const double *mA, const double *lA, const double *oA,
                         const double *mB, const double *lB, const double *oB,
                         double *mO, double *lO, double *oO) {
    for (int64_t i = 0; i < n; i++) {
        double ma = mA[i], mb = mB[i], la = lA[i], lb = lB[i];
        const double *oa = oA + i * D, *ob = oB + i * D;
        double *oo = oO + i * D;
        if (lb == 0.0) {
            for (int32_t d = 0; d < D; d++) oo[d] = oa[d];
            mO[i] = ma; lO[i] = la;
            continue;
        }
        if (la == 0.0) {
            for (int32_t d = 0; d < D; d++) oo[d] = ob[d];
            mO[i] = mb; lO[i] = lb;
            continue;
        }
        double m = ma > mb ? ma : mb;
        double wa = la * exp(ma - m), wb = lb * exp(mb - m);
        double l = wa + wb;
        for (int32_t d = 0; d < D; d++) oo[d] = (wa * oa[d] + wb * ob[d]) / l;
        mO[i] = m; lO[i] = l;
    }
}
