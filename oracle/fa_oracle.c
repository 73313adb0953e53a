/*
 * fa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow fp64 CPU reference ("the oracle") for the attention forward
 * pass.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code, header or constant with the HIP
 * library: it decodes the 16-bit inputs itself, evaluates the defining formula
 * row by row in double precision, and writes fp64 results.
 *
 * What it computes, and where the pages define it:
 *   - orc_attention: Attention(Q,K,V) = softmax(scale * Q K^T) V for each query
 *     row, the defining formula of the FlashAttn operator guide (function
 *     description) and of the aclnnIncreFlashAttention guide (section 1.2).
 *     lse = log(sum_j exp(s_j - m)) + m with m the row maximum (FlashAttn
 *     developer guide, 1.6 LSE).  A row with no valid key gives out = 0 and
 *     lse = +inf (developer guide, 1.7 RowInvalid).
 *       valid keys: j < L_b, where L_b is the batch's actual KV length clamped
 *       to [0, KV_S] (developer guide 1.4, "the shorter takes effect"; IFA
 *       guide 1.1 padded cache), minus the masked ones: causal masks j > i
 *       (developer guide 1.5, lower triangle kept), a boolean mask excludes
 *       the nonzero entries (IFA guide 8.1, true positions are masked).
 *       GQA: query head n1 reads KV head n1 / g (developer guide 1.1: g
 *       consecutive query heads share one KV head).
 *   - orc_split_partials: the split-KV stage-1 quantities per KV chunk c,
 *     m_c = max s_j, l_c = sum exp(s_j - m_c), O_c = sum exp(s_j - m_c) v_j,
 *     with O_c left unnormalised (FlashDecoding tutorial, 3.2 Stage 1; FlashAttn
 *     developer guide 10, FD block).  An empty chunk gives m = -inf, l = 0, O = 0.
 *   - orc_merge: the FD reduction m = max_c m_c, l = sum_c l_c exp(m_c - m),
 *     o = sum_c O_c exp(m_c - m) / l, lse = log l + m (FlashAttn developer
 *     guide 10, FD block formula; FlashDecoding tutorial section 2).
 *   - Window mask (developer guide 1.5, mask mode 4): query row i keeps the
 *     band of keys i - win_left <= j <= i + win_right; a negative bound is
 *     unbounded on that side (the guide sets both to -1 when no window is used).
 *   - Packed variable-length layout TND (developer guide 1.3 and 1.4): q is
 *     (Q_T, Q_N, D) and k, v (KV_T, KV_N, D), the sequences laid end to end;
 *     sequence b holds q rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and kv
 *     rows cu_seqlens_kv[b] .. cu_seqlens_kv[b+1] - 1.  The per-batch lengths,
 *     when given, truncate (the shorter takes effect): seqused_q for the query
 *     rows, the actual KV lengths for the keys.  Indices i, j of masks are
 *     positions inside the sequence.  A query row past its sequence's used
 *     length is not computed and keeps the initial output (0 and lse = +inf,
 *     the output initialisation the developer guide describes).  Rows are
 *     numbered t * Q_N + n1, the (Q_T, Q_N) order of the TND lse.
 *   - seqused_q with the padded layouts BNSD / BSND (developer guide 1.4: the
 *     per-batch used lengths apply to every layout; only cu_seqlens is
 *     TND-only): query rows i >= seqused_q[b] of batch b are not computed and
 *     keep the initial output, 0 and lse = +inf, as in TND.
 *   - Paged KV caches (FlashAttn developer guide 1.2): token j of batch b is
 *     row j % block_size of physical block block_table[b][j / block_size];
 *     PA_BBND blocks are [block_size][KV_N][D], PA_BNBD blocks [KV_N][block_size][D].
 *
 * Two passes per row (scores and max first, then exponentials), natural exp
 * and log, no blocking or reordering beyond that.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, QN, KVN, QS, KVS, D;
    int32_t layout;             /* 0 = BNSD, 1 = BSND, 2 = TND (q, k, v, out alike) */
    int32_t dtype;              /* 0 = fp16, 1 = bf16 storage */
    double scale;
    const int64_t *lens;        /* [B] actual KV lengths, or NULL (= KV_S) */
    int32_t mask_mode;          /* 0 none, 1 causal (j > i excluded), 2 boolean tensor, 3 window */
    const uint8_t *mask;        /* mode 2: nonzero = excluded */
    int64_t mask_stride[4];     /* element strides for (b, n1, i, j); 0 broadcasts */
    int32_t kv_layout;          /* 0 = as layout, 1 = paged BBND, 2 = paged BNBD */
    const int32_t *block_table; /* [B][max_blocks] physical block ids */
    int64_t block_size, max_blocks;
    int64_t win_left, win_right; /* mode 3: keys i - win_left .. i + win_right; < 0 unbounded */
    const int32_t *cu_q, *cu_kv; /* TND: [B + 1] sequence starts (QS = Q_T, KVS = KV_T) */
    const int32_t *used_q;      /* [B] used query rows (any layout), or NULL */
} orc_problem;

static double dec16(int32_t dtype, uint16_t h)
{
    if (dtype == 1) { /* bfloat16: the top half of an IEEE single */
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    /* IEEE binary16 */
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return s ? -v : v;
}

static int64_t q_index(const orc_problem *p, int64_t b, int64_t n, int64_t i)
{
    if (p->layout == 2) return ((p->cu_q[b] + i) * p->QN + n) * p->D;
    return p->layout == 0 ? ((b * p->QN + n) * p->QS + i) * p->D
                          : ((b * p->QS + i) * p->QN + n) * p->D;
}

static int64_t kv_index(const orc_problem *p, int64_t b, int64_t n, int64_t j)
{
    if (p->kv_layout != 0) {
        const int64_t blk = p->block_table[b * p->max_blocks + j / p->block_size];
        const int64_t r = j % p->block_size;
        return p->kv_layout == 1 ? ((blk * p->block_size + r) * p->KVN + n) * p->D
                                 : ((blk * p->KVN + n) * p->block_size + r) * p->D;
    }
    if (p->layout == 2) return ((p->cu_kv[b] + j) * p->KVN + n) * p->D;
    return p->layout == 0 ? ((b * p->KVN + n) * p->KVS + j) * p->D
                          : ((b * p->KVS + j) * p->KVN + n) * p->D;
}

/* Keys of batch b: the cache length (the sequence's own length in TND),
 * truncated by the actual length when one is given. */
static int64_t row_length(const orc_problem *p, int64_t b)
{
    const int64_t cap = p->layout == 2 ? (int64_t)p->cu_kv[b + 1] - p->cu_kv[b] : p->KVS;
    int64_t L = p->lens ? p->lens[b] : cap;
    if (L < 0) L = 0;
    if (L > cap) L = cap;
    return L;
}

static int key_valid(const orc_problem *p, int64_t b, int64_t n1, int64_t i, int64_t j)
{
    if (p->mask_mode == 1 && j > i) return 0;
    if (p->mask_mode == 3) {
        if (p->win_left >= 0 && j < i - p->win_left) return 0;
        if (p->win_right >= 0 && j > i + p->win_right) return 0;
    }
    if (p->mask_mode == 2) {
        const int64_t *st = p->mask_stride;
        if (p->mask[b * st[0] + n1 * st[1] + i * st[2] + j * st[3]] != 0) return 0;
    }
    return 1;
}

/* s_j = scale * sum_d q_d k_{j,d} for the valid keys in [j0, j1); returns the
 * maximum (-inf when none is valid).  Invalid entries of s are left untouched
 * and flagged in ok[]. */
static double scores(const orc_problem *p, const uint16_t *k, const double *qd,
                     int64_t b, int64_t n1, int64_t i, int64_t j0, int64_t j1,
                     double *s, unsigned char *ok)
{
    const int64_t n2 = n1 / (p->QN / p->KVN);
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        ok[j] = (unsigned char)key_valid(p, b, n1, i, j);
        if (!ok[j]) continue;
        const uint16_t *kr = k + kv_index(p, b, n2, j);
        double acc = 0.0;
        for (int64_t d = 0; d < p->D; ++d) acc += qd[d] * dec16(p->dtype, kr[d]);
        s[j] = p->scale * acc;
        if (s[j] > m) m = s[j];
    }
    return m;
}

/* sum_j exp(s_j - m) and sum_j exp(s_j - m) v_j over the valid keys of [j0, j1). */
static double weighted_values(const orc_problem *p, const uint16_t *v, int64_t b, int64_t n1,
                              int64_t j0, int64_t j1, const double *s, const unsigned char *ok,
                              double m, double *o)
{
    const int64_t n2 = n1 / (p->QN / p->KVN);
    double l = 0.0;
    for (int64_t d = 0; d < p->D; ++d) o[d] = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        if (!ok[j]) continue;
        const double w = exp(s[j] - m);
        const uint16_t *vr = v + kv_index(p, b, n2, j);
        l += w;
        for (int64_t d = 0; d < p->D; ++d) o[d] += w * dec16(p->dtype, vr[d]);
    }
    return l;
}

typedef struct {
    const orc_problem *p;
    const uint16_t *q, *k, *v;
    int64_t nrows;
    const int64_t *rows;        /* flat row ids (b*QN + n1)*QS + i (TND: t*QN + n1), or NULL for all */
    int64_t splits, chunk;      /* split mode when splits > 0 */
    double *out, *lse;          /* attention mode: [nrows][D], [nrows] */
    double *o_part, *m_part, *l_part; /* split mode: [nrows][splits][D], [nrows][splits] */
    int nthreads, tid;
} job;

static void *worker(void *arg)
{
    job *jb = (job *)arg;
    const orc_problem *p = jb->p;
    double *s = (double *)malloc(sizeof(double) * (size_t)(p->KVS > 0 ? p->KVS : 1));
    unsigned char *ok = (unsigned char *)malloc((size_t)(p->KVS > 0 ? p->KVS : 1));
    double *qd = (double *)malloc(sizeof(double) * (size_t)p->D);
    if (!s || !ok || !qd) { free(s); free(ok); free(qd); return (void *)1; }
    for (int64_t r = jb->tid; r < jb->nrows; r += jb->nthreads) {
        const int64_t row = jb->rows ? jb->rows[r] : r;
        int64_t i, n1, b;
        int computed = 1;
        if (p->layout == 2) { /* row = t * Q_N + n1; t lies in sequence b */
            const int64_t t = row / p->QN;
            n1 = row % p->QN;
            b = 0;
            while (b < p->B && p->cu_q[b + 1] <= t) ++b;
            i = b < p->B ? t - p->cu_q[b] : 0;
            if (b == p->B || (p->used_q && i >= p->used_q[b])) computed = 0;
        } else {
            i = row % p->QS;
            n1 = (row / p->QS) % p->QN;
            b = row / (p->QS * p->QN);
            if (p->used_q && i >= p->used_q[b]) computed = 0; /* past the used rows */
        }
        if (!computed) { /* outside every sequence's used rows: initial output */
            if (jb->splits == 0) {
                for (int64_t d = 0; d < p->D; ++d) jb->out[r * p->D + d] = 0.0;
                jb->lse[r] = INFINITY;
            } else {
                for (int64_t c = 0; c < jb->splits; ++c) {
                    for (int64_t d = 0; d < p->D; ++d) jb->o_part[(r * jb->splits + c) * p->D + d] = 0.0;
                    jb->m_part[r * jb->splits + c] = -INFINITY;
                    jb->l_part[r * jb->splits + c] = 0.0;
                }
            }
            continue;
        }
        const int64_t L = row_length(p, b);
        const uint16_t *qr = jb->q + q_index(p, b, n1, i);
        for (int64_t d = 0; d < p->D; ++d) qd[d] = dec16(p->dtype, qr[d]);
        if (jb->splits == 0) {
            double *o = jb->out + r * p->D;
            const double m = scores(p, jb->k, qd, b, n1, i, 0, L, s, ok);
            if (m == -INFINITY) { /* no valid key: RowInvalid defaults */
                for (int64_t d = 0; d < p->D; ++d) o[d] = 0.0;
                jb->lse[r] = INFINITY;
                continue;
            }
            const double l = weighted_values(p, jb->v, b, n1, 0, L, s, ok, m, o);
            for (int64_t d = 0; d < p->D; ++d) o[d] /= l;
            jb->lse[r] = log(l) + m;
        } else {
            for (int64_t c = 0; c < jb->splits; ++c) {
                int64_t j0 = c * jb->chunk, j1 = j0 + jb->chunk;
                if (j0 > L) j0 = L;
                if (j1 > L) j1 = L;
                double *o = jb->o_part + (r * jb->splits + c) * p->D;
                const double m = scores(p, jb->k, qd, b, n1, i, j0, j1, s, ok);
                jb->m_part[r * jb->splits + c] = m;
                if (m == -INFINITY) {
                    for (int64_t d = 0; d < p->D; ++d) o[d] = 0.0;
                    jb->l_part[r * jb->splits + c] = 0.0;
                    continue;
                }
                jb->l_part[r * jb->splits + c] = weighted_values(p, jb->v, b, n1, j0, j1, s, ok, m, o);
            }
        }
    }
    free(s); free(ok); free(qd);
    return NULL;
}

static int check(const orc_problem *p)
{
    if (!p || p->B < 0 || p->QN <= 0 || p->KVN <= 0 || p->QS < 0 || p->KVS < 0 || p->D <= 0) return -1;
    if (p->QN % p->KVN != 0) return -2;
    if (p->mask_mode == 2 && !p->mask) return -3;
    if (p->kv_layout != 0 && (!p->block_table || p->block_size <= 0 || p->max_blocks <= 0 ||
                              p->KVS > p->max_blocks * p->block_size)) return -5;
    if (p->layout == 2) { /* well-formed cumulative lengths within the packed tensors */
        if (!p->cu_q || !p->cu_kv || p->kv_layout != 0) return -6;
        if (p->cu_q[0] != 0 || p->cu_kv[0] != 0) return -6;
        for (int64_t b = 0; b < p->B; ++b)
            if (p->cu_q[b + 1] < p->cu_q[b] || p->cu_kv[b + 1] < p->cu_kv[b]) return -6;
        if (p->cu_q[p->B] > p->QS || p->cu_kv[p->B] > p->KVS) return -6;
    }
    return 0;
}

static int run(job *proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    job jobs[256];
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].nthreads = nthreads;
        jobs[t].tid = t;
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) { rc = -10; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -11;
    }
    return rc;
}

/* Attention output and lse for nrows query rows (rows == NULL: all B*QN*QS rows
 * in flat order).  out is [nrows][D], lse [nrows]; both fp64. */
int orc_attention(const orc_problem *p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  int64_t nrows, const int64_t *rows, double *out, double *lse, int nthreads)
{
    int rc = check(p);
    if (rc) return rc;
    job jb;
    memset(&jb, 0, sizeof jb);
    jb.p = p; jb.q = q; jb.k = k; jb.v = v;
    jb.nrows = nrows; jb.rows = rows; jb.out = out; jb.lse = lse;
    return run(&jb, nthreads);
}

/* Per-chunk partials for chunk c covering keys [c*chunk, (c+1)*chunk) cut at L_b. */
int orc_split_partials(const orc_problem *p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       int64_t splits, int64_t chunk, int64_t nrows, const int64_t *rows,
                       double *o_part, double *m_part, double *l_part, int nthreads)
{
    int rc = check(p);
    if (rc) return rc;
    if (splits <= 0 || chunk <= 0) return -4;
    job jb;
    memset(&jb, 0, sizeof jb);
    jb.p = p; jb.q = q; jb.k = k; jb.v = v;
    jb.nrows = nrows; jb.rows = rows; jb.splits = splits; jb.chunk = chunk;
    jb.o_part = o_part; jb.m_part = m_part; jb.l_part = l_part;
    return run(&jb, nthreads);
}

/* Merge per-chunk partials row by row (FD reduction). */
int orc_merge(int64_t nrows, int64_t splits, int64_t D, const double *o_part, const double *m_part,
              const double *l_part, double *out, double *lse)
{
    if (nrows < 0 || splits <= 0 || D <= 0) return -4;
    for (int64_t r = 0; r < nrows; ++r) {
        const double *m = m_part + r * splits;
        const double *l = l_part + r * splits;
        double mg = -INFINITY;
        for (int64_t c = 0; c < splits; ++c)
            if (m[c] > mg) mg = m[c];
        double *o = out + r * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (mg == -INFINITY) { lse[r] = INFINITY; continue; }
        double lg = 0.0;
        for (int64_t c = 0; c < splits; ++c) {
            if (m[c] == -INFINITY) continue;
            const double w = exp(m[c] - mg);
            lg += l[c] * w;
            const double *oc = o_part + (r * splits + c) * D;
            for (int64_t d = 0; d < D; ++d) o[d] += oc[d] * w;
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= lg;
        lse[r] = log(lg) + mg;
    }
    return 0;
}
