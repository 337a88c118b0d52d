/*
 * Oracle for sliding-window grouped-query attention over a rolling-buffer
 * KV cache.  TEST INFRASTRUCTURE ONLY: nothing in the product library links,
 * loads or calls this file.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.
 *
 * Plain, slow and meant to be read against the paper:
 *   Mistral 7B (Chinese translation), section 2 "Architectural details":
 *     - paragraph "Sliding Window Attention" and the Figure 1 caption: the
 *       hidden state at position i attends to at most W earlier states of the
 *       layer below, ending at i itself;
 *     - paragraph "Rolling Buffer Cache" and the Figure 2 caption: a cache of
 *       fixed size W; the keys and values of time step i go to slot i mod W and
 *       overwrite older entries;
 *     - paragraph "Pre-fill and Chunking" and the Figure 3 caption: a chunk
 *       attends causally to itself and, through the window, to the cache.
 *   Section 1 "Introduction" names grouped-query attention (GQA): query heads
 *   share key/value heads.
 *
 * Readings taken where the pages leave a step open (listed in full in the
 * design notes of the repository):
 *   - window: W keys, positions j with i-W < j <= i (the caption bounds the
 *     window by W tokens; a W-slot ring holds exactly these after writing
 *     position i);
 *   - GQA grouping: query head h uses key/value head floor(h / G), G = Hq/Hkv;
 *   - softmax scale: passed in by the caller (1/sqrt(head_dim) by default);
 *   - positions are 0-based, so the first overwrite happens at i = W.
 *
 * Arithmetic: every input is an exact float32 value (bf16 inputs are exactly
 * representable in float32); all arithmetic is IEEE double.  No blocking, no
 * online softmax, no reordering: scores, max, exp, sum, weighted sum, divide.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGUMENT (-1)
#define ORACLE_MISSING_KEY (-2)
#define ORACLE_NO_MEMORY (-3)

/*
 * Attention of a set of queries of ONE sequence over that sequence's keys and
 * values, given on absolute positions (never through the ring).
 *
 *   q      [n_q][n_q_heads][head_dim]       query rows, q_pos[r] = absolute position
 *   k, v   [n_kv][n_kv_heads][head_dim]     k[t], v[t] belong to position kv_pos0 + t
 *   out    [n_q][n_q_heads][head_dim]       double
 *
 * For query position i and head h (g = h / G):
 *   J(i)  = { j : max(0, i-W+1) <= j <= i }
 *   s_j   = scale * sum_d q[i,h,d] k[j,g,d]
 *   o     = sum_j exp(s_j - max s) v[j,g,:] / sum_j exp(s_j - max s)
 * Returns ORACLE_MISSING_KEY if some j in J(i) is not covered by k/v.
 */
int swa_oracle_attend(int n_q, int n_q_heads, int n_kv_heads, int head_dim,
                      int window, double scale,
                      const float *q, const int64_t *q_pos,
                      int n_kv, int64_t kv_pos0,
                      const float *k, const float *v, double *out)
{
    if (n_q < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
        window <= 0 || n_kv < 0 || n_q_heads % n_kv_heads != 0)
        return ORACLE_BAD_ARGUMENT;
    const int group = n_q_heads / n_kv_heads;

    /* Check coverage first so that nothing is computed on a bad request. */
    for (int r = 0; r < n_q; r++) {
        int64_t i = q_pos[r];
        int64_t lo = i - window + 1;
        if (lo < 0) lo = 0;
        if (i < 0 || lo < kv_pos0 || i >= kv_pos0 + n_kv)
            return ORACLE_MISSING_KEY;
    }

    int status = ORACLE_OK;
    const int64_t total = (int64_t)n_q * n_q_heads;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)window);
        double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!scores || !acc) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t task = 0; task < total; task++) {
                const int r = (int)(task / n_q_heads);
                const int h = (int)(task % n_q_heads);
                const int g = h / group;
                const int64_t i = q_pos[r];
                int64_t lo = i - window + 1;
                if (lo < 0) lo = 0;
                const int n = (int)(i - lo + 1);
                const float *qrow = q + ((size_t)r * n_q_heads + h) * head_dim;

                /* scores over the band, and their maximum */
                double m = -INFINITY;
                for (int t = 0; t < n; t++) {
                    const float *krow = k + ((size_t)(lo + t - kv_pos0) * n_kv_heads + g) * head_dim;
                    double dot = 0.0;
                    for (int d = 0; d < head_dim; d++)
                        dot += (double)qrow[d] * (double)krow[d];
                    scores[t] = scale * dot;
                    if (scores[t] > m) m = scores[t];
                }
                /* softmax weights and the weighted sum of values */
                double l = 0.0;
                for (int d = 0; d < head_dim; d++) acc[d] = 0.0;
                for (int t = 0; t < n; t++) {
                    const double p = exp(scores[t] - m);
                    const float *vrow = v + ((size_t)(lo + t - kv_pos0) * n_kv_heads + g) * head_dim;
                    l += p;
                    for (int d = 0; d < head_dim; d++)
                        acc[d] += p * (double)vrow[d];
                }
                double *orow = out + ((size_t)r * n_q_heads + h) * head_dim;
                for (int d = 0; d < head_dim; d++) orow[d] = acc[d] / l;
            }
        }
        free(scores);
        free(acc);
    }
    return status;
}

/*
 * Rolling buffer: apply the writes of a batch of sequences in position order.
 *
 *   ring     [n_cache][n_kv_heads][window][row_bytes]   bytes, updated in place
 *   rows     [total_tokens][n_kv_heads][row_bytes]     new keys (or values)
 *   cu_seqlens[num_seqs+1], start_pos[num_seqs], cache_idx[num_seqs]
 *
 * Token t of sequence b has absolute position start_pos[b] + t and is stored
 * at slot (position mod W) of cache row cache_idx[b] (paragraph "Rolling
 * Buffer Cache").  Every write is applied, in increasing position, so a later
 * position overwrites an earlier one that maps to the same slot.  Slots never
 * written keep their bytes.  The copy is bytewise: the oracle of a cache write
 * is exact for every dtype.
 */
int swa_oracle_ring_write(unsigned char *ring, int n_cache, int n_kv_heads,
                          int window, int row_bytes,
                          const unsigned char *rows, int num_seqs,
                          const int32_t *cu_seqlens, const int32_t *start_pos,
                          const int32_t *cache_idx)
{
    if (n_cache <= 0 || n_kv_heads <= 0 || window <= 0 || row_bytes <= 0 || num_seqs < 0)
        return ORACLE_BAD_ARGUMENT;
    for (int b = 0; b < num_seqs; b++) {
        const int row = cache_idx ? cache_idx[b] : b;
        if (row < 0 || row >= n_cache || start_pos[b] < 0 || cu_seqlens[b + 1] < cu_seqlens[b])
            return ORACLE_BAD_ARGUMENT;
        for (int32_t tok = cu_seqlens[b]; tok < cu_seqlens[b + 1]; tok++) {
            const int64_t pos = (int64_t)start_pos[b] + (tok - cu_seqlens[b]);
            const int64_t slot = pos % window;
            for (int g = 0; g < n_kv_heads; g++) {
                unsigned char *dst = ring + ((((size_t)row * n_kv_heads + g) * window + slot) * row_bytes);
                const unsigned char *src = rows + (((size_t)tok * n_kv_heads + g) * row_bytes);
                memcpy(dst, src, (size_t)row_bytes);
            }
        }
    }
    return ORACLE_OK;
}

/* Threads for the following oracle calls (CPU timings at a stated thread count). */
void swa_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of threads the OpenMP runtime will use (reported with CPU timings). */
int swa_oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
