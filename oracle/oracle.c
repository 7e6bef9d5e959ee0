/*
 * Reference oracle for the paged-KV attention step.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library.  It shares no code with the HIP path.
 *
 * Plain, slow and obviously correct: every floating-point step is done in
 * double precision, in the order the definition states, with no blocking,
 * fusion or reordering.  Inputs are read in their storage type (fp32, or bf16
 * as raw 16-bit words) and widened exactly to double on every read.
 *
 * What is computed (sources: "mini-sglang from Scratch, Engine and sampler",
 * sections on initialisation order and on the hand-driven engine; "Stage 4
 * milestone", table "What each chapter adds"; the Mini-SGLang Engine article's
 * per-layer pipeline, where the KV write precedes attention):
 *
 *   store_kv   pool[out_loc[t]] = new[t] for every new token t, K and V alike.
 *              The pool row of a slot is [kv_heads, head_dim] contiguous.
 *
 *   attention  For request b (page-table row table_idx[b], device_len
 *              L = seq_lens[b]) the query tokens are the request's new tokens;
 *              with n of them, query i sits at position p = L - n + i (so
 *              p = cached_len + i, and a one-token decode sits at L - 1).
 *              For every q head h, with kv head kv = h / (q_heads / kv_heads):
 *                K_j = Kpool[page_table[row, j], kv, :],  V_j likewise, j <= p
 *                s_j = scale * sum_c q[c] K_j[c]
 *                m   = max_j s_j,  e_j = exp(s_j - m),  l = sum_j e_j
 *                out = sum_j e_j V_j / l,   lse = m + log(l)
 *              scale defaults to 1/sqrt(head_dim) in the Python wrapper.
 *              Sums run in increasing j (and c) order.
 *
 *   rope       Rotary position embedding of the new tokens' q and k, the step
 *              the Mini-SGLang Engine article's per-layer pipeline runs between
 *              the QKV projection and the KV write.  The pages give no formula;
 *              this is the published rotary embedding (Su et al., "RoFormer",
 *              section 3.2, the general form) with the pairing of the GPT-NeoX and
 *              Qwen families: element i of a head is paired with element
 *              i + d/2, and for a token at position p the pair turns by
 *              a_i = p * base^(-2i/d), i = 0 .. d/2 - 1:
 *                y[i]       = x[i] cos a_i - x[i + d/2] sin a_i
 *                y[i + d/2] = x[i + d/2] cos a_i + x[i] sin a_i
 *              Every head of the token (q heads and kv heads alike) turns by
 *              the same angles.
 *
 *   vocab_embed  Vocabulary indexing, the small custom kernel the Stage 4
 *              milestone's table pairs with the KV write: the embedding rows
 *              of the step's token ids.  Under tensor parallelism each rank
 *              holds the rows [vocab_start, vocab_start + rows) of the table
 *              (the table "What each chapter adds": several cards read the
 *              weights together); a token id outside that range gives a zero
 *              row, so the ranks' outputs sum to the full table's rows:
 *                out[t] = weight[ids[t] - vocab_start]  if the id is in range
 *                out[t] = 0                             otherwise.
 *              A row is copied bit for bit.
 *
 * Error behaviour: none; arguments are assumed valid (the Python wrapper
 * checks shapes before calling).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* exact widening of one stored element */
static double orc_load(const void *base, int64_t i, int dtype)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

void oracle_store_kv(uint8_t *k_pool, uint8_t *v_pool, int64_t row_bytes,
                     const uint8_t *k_new, const uint8_t *v_new,
                     const int32_t *out_loc, int64_t num_tokens)
{
    for (int64_t t = 0; t < num_tokens; ++t) {
        memcpy(k_pool + (int64_t)out_loc[t] * row_bytes, k_new + t * row_bytes, (size_t)row_bytes);
        memcpy(v_pool + (int64_t)out_loc[t] * row_bytes, v_new + t * row_bytes, (size_t)row_bytes);
    }
}

/* One (query token, q head) pair.  s is caller scratch of length >= p + 1. */
static void orc_one(int dtype, const void *q, int64_t q_off,
                    const void *k_pool, const void *v_pool,
                    const int32_t *pt_row, int64_t p, int64_t kv_heads,
                    int64_t kv, int64_t head_dim, double scale,
                    double *s, double *out, double *lse)
{
    int64_t row_elems = kv_heads * head_dim;
    /* scores */
    for (int64_t j = 0; j <= p; ++j) {
        int64_t base = (int64_t)pt_row[j] * row_elems + kv * head_dim;
        double dot = 0.0;
        for (int64_t c = 0; c < head_dim; ++c)
            dot += orc_load(q, q_off + c, dtype) * orc_load(k_pool, base + c, dtype);
        s[j] = scale * dot;
    }
    /* softmax statistics */
    double m = -INFINITY;
    for (int64_t j = 0; j <= p; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j <= p; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* weighted sum of V */
    for (int64_t c = 0; c < head_dim; ++c)
        out[c] = 0.0;
    for (int64_t j = 0; j <= p; ++j) {
        int64_t base = (int64_t)pt_row[j] * row_elems + kv * head_dim;
        for (int64_t c = 0; c < head_dim; ++c)
            out[c] += s[j] * orc_load(v_pool, base + c, dtype);
    }
    for (int64_t c = 0; c < head_dim; ++c)
        out[c] /= l;
    *lse = m + log(l);
}

/*
 * q        [T, q_heads, head_dim]   (T = q_start[n_req])
 * k_pool   [slots, kv_heads, head_dim], v_pool likewise
 * out      [T, q_heads, head_dim] double,  lse [T, q_heads] double
 * q_start  [n_req + 1]: request b's query tokens are rows q_start[b] .. q_start[b+1]-1
 */
void oracle_attention(int dtype, int64_t n_req, const int32_t *table_idx,
                      const int32_t *seq_lens, const int32_t *q_start,
                      const int32_t *page_table, int64_t row_stride,
                      const void *q, const void *k_pool, const void *v_pool,
                      int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                      double scale, double *out, double *lse)
{
    int64_t group = q_heads / kv_heads;
    int64_t T = q_start[n_req];
    int64_t max_len = 1;
    for (int64_t b = 0; b < n_req; ++b)
        if (seq_lens[b] > max_len)
            max_len = seq_lens[b];
    /* request of every query row */
    int64_t *req_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    for (int64_t b = 0; b < n_req; ++b)
        for (int64_t t = q_start[b]; t < q_start[b + 1]; ++t)
            req_of[t] = b;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)max_len);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < T * q_heads; ++w) {
            int64_t t = w / q_heads;
            int64_t h = w % q_heads;
            int64_t b = req_of[t];
            int64_t n = q_start[b + 1] - q_start[b];
            int64_t p = (int64_t)seq_lens[b] - n + (t - q_start[b]);
            const int32_t *pt_row = page_table + (int64_t)table_idx[b] * row_stride;
            orc_one(dtype, q, (t * q_heads + h) * head_dim, k_pool, v_pool, pt_row, p,
                    kv_heads, h / group, head_dim, scale, s,
                    out + (t * q_heads + h) * head_dim, lse + t * q_heads + h);
        }
        free(s);
    }
    free(req_of);
}

/*
 * x   [T, heads, head_dim] in storage type dtype; positions [T];
 * out [T, heads, head_dim] double.  head_dim is even.
 */
void oracle_rope(int dtype, const void *x, int64_t num_tokens, int64_t heads,
                 int64_t head_dim, const int32_t *positions, double base, double *out)
{
    int64_t half = head_dim / 2;
    for (int64_t t = 0; t < num_tokens; ++t) {
        double p = (double)positions[t];
        for (int64_t h = 0; h < heads; ++h) {
            int64_t row = (t * heads + h) * head_dim;
            for (int64_t i = 0; i < half; ++i) {
                double a = p * pow(base, -2.0 * (double)i / (double)head_dim);
                double x1 = orc_load(x, row + i, dtype);
                double x2 = orc_load(x, row + i + half, dtype);
                out[row + i] = x1 * cos(a) - x2 * sin(a);
                out[row + i + half] = x2 * cos(a) + x1 * sin(a);
            }
        }
    }
}

/*
 * weight [rows, row_bytes] (any storage type, copied as bytes); ids [T];
 * out [T, row_bytes].
 */
void oracle_vocab_embed(const uint8_t *weight, int64_t rows, int64_t row_bytes,
                        int64_t vocab_start, const int32_t *ids, int64_t num_tokens,
                        uint8_t *out)
{
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t r = (int64_t)ids[t] - vocab_start;
        if (r >= 0 && r < rows)
            memcpy(out + t * row_bytes, weight + r * row_bytes, (size_t)row_bytes);
        else
            memset(out + t * row_bytes, 0, (size_t)row_bytes);
    }
}

/* thread control for timing; n <= 0 leaves the OpenMP default */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
