/*
 * pa_oracle.c -- plain fp64 CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (the "Paged Attention" section of "[TIL] Optimizing paged
 * attention" defines attention as a softmax over the context of the query-key
 * products times a scale, used to weight the value vectors; the "Baseline"
 * section's kernel fixes the indexing and that the score is multiplied, not
 * divided, by the scale):
 *
 *   for every sequence b and query head h, with g = h / (query_heads / kv_heads),
 *     s[t]      = scale * sum_d q[b][h][d] * K[t][g][d]            t = 0 .. ctx[b]-1
 *     out[b][h] = sum_t exp(s[t] - max s) * V[t][g] / sum_t exp(s[t] - max s)
 *
 * where K[t][g] / V[t][g] are fetched through the block table: token t of
 * sequence b lives in logical page t / page_size, slot t % page_size, and the
 * physical page is block_tables[b][t / page_size]; the element offset of
 * (physical page p, slot s, kv head g, dim d) in each cache is
 * ((p * page_size + s) * kv_heads + g) * head_dim + d  (the "Data Layout" section
 * and the Baseline kernel of the same page).
 *
 * Precision: the fp16 inputs are widened exactly to double by this file's own
 * binary16 decoder; every sum is accumulated serially in double; exp is libm's.
 * The softmax is evaluated in two passes (max, then exponentials), which is the
 * definition with the usual shift by the maximum; it is not the streaming
 * recurrence the GPU uses.
 *
 * ctx[b] == 0 (no token) is defined as an all-zero output row; the pages leave
 * that case open.
 *
 * pa_oracle_attend_partitioned() evaluates the same result through the
 * split-context route: per partition of partition_size tokens it forms the
 * partition's maximum m_p, its exponential sum l_p and its unnormalised weighted
 * value sum acc_p, then combines them as
 *   M = max_p m_p,  out = sum_p exp(m_p - M) acc_p / sum_p exp(m_p - M) l_p
 * skipping partitions that hold no token (the "V4 (Context-axis parallelism)"
 * merge kernel of the first page; the phase-2 log-sum-exp reduction of the
 * "paged_attention_v2_pytorch.py" commit page is the same combination written
 * with normalised partials).  It exists to pin that combination to the direct
 * definition, in double precision.
 *
 * pa_oracle_append() is the step before attention in a decode loop: it stores the
 * new token's key and value rows in the cache (see its own comment).
 *
 * pa_oracle_attend_zero_pages() is the same definition with one more reading: a block
 * table entry outside the pool [0, num_pages) that the context would dereference
 * reads as a page of zero keys and values (each such token scores 0 and adds a zero
 * value row).  The first page shows unused table slots as placeholders ("Baseline"
 * section) and never describes an entry that names no page; this reading is the
 * engine's debug-bounds mode.  pa_oracle_bad_entries() lists those entries as a
 * bitmap over the table.
 *
 * Error handling: return 0 on success; 1 for a bad argument (sizes, null
 * pointers, query_heads % kv_heads != 0); 2 when a context length or (outside the
 * zero-page reading) a block table entry that would be dereferenced lies outside
 * the pool.  Nothing is read outside the arrays the arguments describe.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE-754 binary16 -> double: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double pa_oracle_half_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1F;
    int frac = bits & 0x3FF;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);                   /* subnormal: frac * 2^-14 * 2^-10 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);    /* (1 + frac/1024) * 2^(expo-15) */
    }
    return sign ? -mag : mag;
}

typedef struct {
    int batch, query_heads, kv_heads, head_dim, page_size, max_pages, num_pages;
    const uint16_t *q, *k, *v;
    const int32_t *block_tables, *ctx;
    double scale;
    int zero_pages;   /* entries outside the pool read as zero pages (else an error) */
} problem_t;

static int check_problem(const problem_t *p)
{
    if (p->batch < 0 || p->query_heads <= 0 || p->kv_heads <= 0 || p->head_dim <= 0 ||
        p->page_size <= 0 || p->max_pages <= 0 || p->num_pages < 0)
        return 1;
    if (p->query_heads % p->kv_heads) return 1;
    if (p->batch > 0 && (!p->q || !p->block_tables || !p->ctx)) return 1;
    for (int b = 0; b < p->batch; ++b) {
        long long L = p->ctx[b];
        if (L < 0 || L > (long long)p->max_pages * p->page_size) return 2;
        long long pages = (L + p->page_size - 1) / p->page_size;
        if (pages > 0 && (!p->k || !p->v)) return 1;
        for (long long lp = 0; lp < pages && !p->zero_pages; ++lp) {
            int32_t phys = p->block_tables[(size_t)b * p->max_pages + lp];
            if (phys < 0 || phys >= p->num_pages) return 2;
        }
    }
    return 0;
}

/* Whether token t of sequence b sits in a page of the pool (always, outside the
 * zero-page reading: check_problem() has rejected every other table). */
static int in_pool(const problem_t *p, int b, long long t)
{
    int32_t phys = p->block_tables[(size_t)b * p->max_pages + t / p->page_size];
    return phys >= 0 && phys < p->num_pages;
}

/* Offset of element (token t of sequence b, kv head g, dim 0) in the K / V pool. */
static size_t kv_offset(const problem_t *p, int b, long long t, int g)
{
    long long lp = t / p->page_size;
    long long slot = t % p->page_size;
    long long phys = p->block_tables[(size_t)b * p->max_pages + lp];
    return (size_t)(((phys * p->page_size + slot) * p->kv_heads + g) * (long long)p->head_dim);
}

/* Score of token t for (b, h): scale * sum_d q * k, summed over d in order. */
static double score(const problem_t *p, int b, int h, int g, long long t)
{
    const uint16_t *qrow = p->q + ((size_t)b * p->query_heads + h) * p->head_dim;
    if (!in_pool(p, b, t)) return 0.0;                    /* a zero key row scores 0 */
    const uint16_t *krow = p->k + kv_offset(p, b, t, g);
    double dot = 0.0;
    for (int d = 0; d < p->head_dim; ++d)
        dot += pa_oracle_half_to_double(qrow[d]) * pa_oracle_half_to_double(krow[d]);
    return p->scale * dot;
}

/* Direct definition for one (b, h); writes head_dim doubles to o. */
static void attend_one(const problem_t *p, int b, int h, double *o, double *s)
{
    int group = p->query_heads / p->kv_heads;
    int g = h / group;
    long long L = p->ctx[b];
    for (int d = 0; d < p->head_dim; ++d) o[d] = 0.0;
    if (L == 0) return;

    double m = -INFINITY;
    for (long long t = 0; t < L; ++t) {
        s[t] = score(p, b, h, g, t);
        if (s[t] > m) m = s[t];
    }
    double z = 0.0;
    for (long long t = 0; t < L; ++t) {
        double w = exp(s[t] - m);
        z += w;
        if (!in_pool(p, b, t)) continue;                  /* a zero value row adds nothing */
        const uint16_t *vrow = p->v + kv_offset(p, b, t, g);
        for (int d = 0; d < p->head_dim; ++d) o[d] += w * pa_oracle_half_to_double(vrow[d]);
    }
    for (int d = 0; d < p->head_dim; ++d) o[d] /= z;
}

/* Split-context route for one (b, h): per-partition (m, l, acc), then the combination. */
static void attend_one_partitioned(const problem_t *p, int b, int h, long long part,
                                   double *o, double *acc)
{
    int group = p->query_heads / p->kv_heads;
    int g = h / group;
    long long L = p->ctx[b];
    for (int d = 0; d < p->head_dim; ++d) o[d] = 0.0;
    if (L == 0) return;
    long long nparts = (L + part - 1) / part;

    /* pass 1: the global maximum over the partition maxima */
    double M = -INFINITY;
    for (long long pi = 0; pi < nparts; ++pi) {
        long long t0 = pi * part, t1 = t0 + part < L ? t0 + part : L;
        double m_p = -INFINITY;
        for (long long t = t0; t < t1; ++t) {
            double st = score(p, b, h, g, t);
            if (st > m_p) m_p = st;
        }
        if (m_p > M) M = m_p;
    }
    /* pass 2: each partition's (m_p, l_p, acc_p), rescaled by exp(m_p - M) */
    double Lsum = 0.0;
    for (long long pi = 0; pi < nparts; ++pi) {
        long long t0 = pi * part, t1 = t0 + part < L ? t0 + part : L;
        double m_p = -INFINITY;
        for (long long t = t0; t < t1; ++t) {
            double st = score(p, b, h, g, t);
            if (st > m_p) m_p = st;
        }
        double l_p = 0.0;
        for (int d = 0; d < p->head_dim; ++d) acc[d] = 0.0;
        for (long long t = t0; t < t1; ++t) {
            double w = exp(score(p, b, h, g, t) - m_p);
            l_p += w;
            if (!in_pool(p, b, t)) continue;
            const uint16_t *vrow = p->v + kv_offset(p, b, t, g);
            for (int d = 0; d < p->head_dim; ++d) acc[d] += w * pa_oracle_half_to_double(vrow[d]);
        }
        if (l_p == 0.0) continue;                         /* a partition with no token */
        double beta = exp(m_p - M);
        Lsum += beta * l_p;
        for (int d = 0; d < p->head_dim; ++d) o[d] += beta * acc[d];
    }
    for (int d = 0; d < p->head_dim; ++d) o[d] /= Lsum;
}

static int run(const problem_t *p, const int32_t *rows, int n_rows, long long part,
               int nthreads, double *out)
{
    int rc = check_problem(p);
    if (rc) return rc;
    if (!out) return 1;
    long long total = rows ? n_rows : (long long)p->batch * p->query_heads;
    for (long long i = 0; rows && i < total; ++i)
        if (rows[i] < 0 || rows[i] >= p->batch * p->query_heads) return 1;
    long long max_ctx = 0;
    for (int b = 0; b < p->batch; ++b) if (p->ctx[b] > max_ctx) max_ctx = p->ctx[b];
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(max_ctx + p->head_dim + 1));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long long i = 0; i < total; ++i) {
            if (!scratch) continue;
            long long flat = rows ? rows[i] : i;
            int b = (int)(flat / p->query_heads), h = (int)(flat % p->query_heads);
            double *o = out + (size_t)i * p->head_dim;
            if (part > 0) attend_one_partitioned(p, b, h, part, o, scratch);
            else attend_one(p, b, h, o, scratch);
        }
        free(scratch);
    }
    return failed ? 3 : 0;
}

/*
 * out: double [n_rows][head_dim] when rows != NULL (rows lists flat indices b*query_heads+h),
 *      else double [batch][query_heads][head_dim].
 * q: fp16 bits [batch][query_heads][head_dim]; k, v: fp16 bits
 * [num_pages][page_size][kv_heads][head_dim]; block_tables: int32 [batch][max_pages];
 * ctx: int32 [batch].  nthreads: OpenMP threads over output rows (each row is summed
 * serially, so results do not depend on it).
 */
int pa_oracle_attend(int batch, int query_heads, int kv_heads, int head_dim, int page_size,
                     int max_pages, int num_pages, const uint16_t *q, const uint16_t *k,
                     const uint16_t *v, const int32_t *block_tables, const int32_t *ctx,
                     double scale, const int32_t *rows, int n_rows, int nthreads, double *out)
{
    problem_t p = {batch, query_heads, kv_heads, head_dim, page_size, max_pages, num_pages,
                   q, k, v, block_tables, ctx, scale, 0};
    return run(&p, rows, n_rows, 0, nthreads, out);
}

/* pa_oracle_attend() under the zero-page reading (same arguments). */
int pa_oracle_attend_zero_pages(int batch, int query_heads, int kv_heads, int head_dim,
                                int page_size, int max_pages, int num_pages, const uint16_t *q,
                                const uint16_t *k, const uint16_t *v,
                                const int32_t *block_tables, const int32_t *ctx, double scale,
                                const int32_t *rows, int n_rows, int nthreads, double *out)
{
    problem_t p = {batch, query_heads, kv_heads, head_dim, page_size, max_pages, num_pages,
                   q, k, v, block_tables, ctx, scale, 1};
    return run(&p, rows, n_rows, 0, nthreads, out);
}

/*
 * The table entries a decode step dereferences (logical pages lp < ceil(ctx[b] /
 * page_size) of each sequence) that lie outside the pool [0, num_pages): bit
 * (b * max_pages + lp) % 32 of word (b * max_pages + lp) / 32 of `bitmap`, which holds
 * ceil(batch * max_pages / 32) words and is cleared first.  Returns the number of
 * such entries, or -1 for a bad argument.
 */
long long pa_oracle_bad_entries(int batch, int page_size, int max_pages, int num_pages,
                                const int32_t *block_tables, const int32_t *ctx,
                                uint32_t *bitmap)
{
    if (batch < 0 || page_size <= 0 || max_pages <= 0 || num_pages < 0) return -1;
    if (batch > 0 && (!block_tables || !ctx || !bitmap)) return -1;
    long long nbits = (long long)batch * max_pages;
    memset(bitmap, 0, sizeof(uint32_t) * (size_t)((nbits + 31) / 32));
    long long count = 0;
    for (int b = 0; b < batch; ++b) {
        long long L = ctx[b];
        if (L < 0 || L > (long long)max_pages * page_size) return -1;
        long long pages = (L + page_size - 1) / page_size;
        for (long long lp = 0; lp < pages; ++lp) {
            int32_t phys = block_tables[(size_t)b * max_pages + lp];
            if (phys >= 0 && phys < num_pages) continue;
            long long bit = (long long)b * max_pages + lp;
            bitmap[bit / 32] |= 1u << (bit % 32);
            ++count;
        }
    }
    return count;
}

int pa_oracle_attend_partitioned(int batch, int query_heads, int kv_heads, int head_dim,
                                 int page_size, int max_pages, int num_pages, const uint16_t *q,
                                 const uint16_t *k, const uint16_t *v,
                                 const int32_t *block_tables, const int32_t *ctx, double scale,
                                 int partition_size, const int32_t *rows, int n_rows,
                                 int nthreads, double *out)
{
    if (partition_size <= 0) return 1;
    problem_t p = {batch, query_heads, kv_heads, head_dim, page_size, max_pages, num_pages,
                   q, k, v, block_tables, ctx, scale, 0};
    return run(&p, rows, n_rows, partition_size, nthreads, out);
}

/*
 * The step before attention: storing the new token's key and value rows.
 *
 * The cache exists so that the keys and values of a sequence's earlier tokens are reused
 * rather than recomputed (the "Paged Attention" section of "[TIL] Optimizing paged
 * attention"); a decode step therefore first stores its own token's rows.  Under the
 * layout of that page's "Data Layout" section, the token at position pos of sequence b
 * belongs in slot pos % page_size of physical page block_tables[b][pos / page_size], so
 * for every KV head g:
 *
 *   K[page][slot][g][:] = new_k[b][g][:]      V[page][slot][g][:] = new_v[b][g][:]
 *
 * A negative positions[b] means that sequence stores nothing in this step.  A position
 * at or past the end of the table row (max_pages * page_size) or a table entry outside
 * the pool names no slot: that sequence is skipped as well and the cache keeps its old
 * bytes.  The pages do not describe this step; both rules are this oracle's reading.
 *
 * new_k, new_v: fp16 bits [batch][kv_heads][head_dim]; k, v: the caches, modified in
 * place.  *n_written (may be NULL) receives the number of sequences stored.
 * Returns 0, or 1 for a bad argument.
 */
int pa_oracle_append(int batch, int kv_heads, int head_dim, int page_size, int max_pages,
                     int num_pages, const uint16_t *new_k, const uint16_t *new_v,
                     const int32_t *block_tables, const int32_t *positions, uint16_t *k,
                     uint16_t *v, int *n_written)
{
    if (batch < 0 || kv_heads <= 0 || head_dim <= 0 || page_size <= 0 || max_pages <= 0 ||
        num_pages < 0)
        return 1;
    if (batch > 0 && (!new_k || !new_v || !block_tables || !positions || !k || !v)) return 1;
    int written = 0;
    for (int b = 0; b < batch; ++b) {
        long long pos = positions[b];
        if (pos < 0 || pos >= (long long)max_pages * page_size) continue;
        long long phys = block_tables[(size_t)b * max_pages + pos / page_size];
        if (phys < 0 || phys >= num_pages) continue;
        long long slot = pos % page_size;
        for (int g = 0; g < kv_heads; ++g) {
            size_t dst = (size_t)(((phys * page_size + slot) * kv_heads + g) * (long long)head_dim);
            size_t src = ((size_t)b * kv_heads + g) * (size_t)head_dim;
            for (int d = 0; d < head_dim; ++d) {
                k[dst + d] = new_k[src + d];
                v[dst + d] = new_v[src + d];
            }
        }
        ++written;
    }
    if (n_written) *n_written = written;
    return 0;
}

/* Threads an OpenMP region would use by default on this machine (1 without OpenMP). */
int pa_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
