/*
 * Oracle for one decode step of attention over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the GPU path.
 *
 * What it computes is the plain definition, in double precision:
 *
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V
 *
 * as written in the "softmax problem" section of the dothoosh.com article on
 * StreamingLLM and attention sinks, applied to one block of new query rows
 * against the cached keys and values ("KV cache" item of the nextadmin.net
 * lesson "KV cache and Flash Attention": a new token's attention is one query
 * against the cached keys).  Every score is formed, the full softmax is taken
 * with an explicit mask, and the weighted sum of V is accumulated: no tiling,
 * no running max, no split.
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *  - scale is 1/sqrt(d) unless the caller passes another one (the formula in
 *    the StreamingLLM article has it; the lesson's tiled-softmax snippet omits it).
 *  - query head h reads KV head h / (Hq/Hkv) (grouped-query attention shares
 *    one K/V head among consecutive query heads; lesson, "KV cache math").
 *  - seq_lens[b] = T counts every cached position including the q_len new
 *    ones; new row i sits at position P = T - q_len + i and sees positions
 *    <= P (verification pass of the speculative-decoding article: each draft
 *    position sees every earlier position).
 *  - sink/window mask: row at P sees p <= P with p < n_sink or p >= P-window+1
 *    (StreamingLLM: first 4 tokens plus the 4,092 most recent = 4,096 kept).
 *  - ring slot of position p: p if p < n_sink, else
 *    n_sink + (p - n_sink) mod (capacity - n_sink) (sinks are never evicted,
 *    the window rolls over the remaining slots).
 *  - paged slot: block_table[b][p / block_size] * block_size + p % block_size
 *    (lesson, "PagedAttention": 16-token blocks, a page table from logical
 *    positions to physical blocks).
 *  - tree mask (token-tree verification: SpecInfer verifies a tree of draft
 *    tokens with a custom attention mask, speculative-decoding article; EAGLE-2
 *    grows such trees, aioapex.com article): the q_len new positions
 *    P0 .. P0 + q_len - 1 (P0 = T - q_len) are the tree's tokens; row i sees every
 *    earlier cached position p < P0 and the new position P0 + j exactly when bit j
 *    of its mask word is set (its ancestors and itself).
 *
 * Storage formats are decoded from their bit definitions (IEEE binary16,
 * bfloat16 = the top half of binary32, OCP 8-bit E4M3), exactly, into double.
 *
 * An 8-bit KV cache (the FP8 KV-cache option the lesson lists among its serving
 * flags, and KV quantisation in the StreamingLLM article's outlook) stores
 * E4M3 codes; the pages fix no scaling, so the reading taken is the plainest
 * one: one fp32 scale per KV head for K and one for V, the real value being
 * code * scale.  The oracle dequantises (in double) and then runs unchanged.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8_E4M3 = 3 };
enum { OR_CONTIGUOUS = 0, OR_PAGED = 1, OR_RING = 2 };
enum { OR_CAUSAL = 0, OR_SINK_WINDOW = 1, OR_TREE = 2 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_to_f64(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-14 * 2^-10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the high 16 bits of an IEEE binary32. */
static double bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit E4M3 (the "FN" variant): 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); no infinities, the codes
 * S.1111.111 are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_to_f64(uint8_t c) {
    int sign = c >> 7;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);                  /* m/8 * 2^(1-7) */
    else
        v = ldexp((double)(m + 8), e - 10);        /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return f16_to_f64(((const uint16_t*)base)[idx]);
    case OR_FP8_E4M3: return e4m3_to_f64(((const uint8_t*)base)[idx]);
    default: return bf16_to_f64(((const uint16_t*)base)[idx]);
    }
}

double oracle_decode_elem(const void* base, int dtype, int64_t idx) {
    return load_elem(base, dtype, idx);
}

/* Does the new row at position P attend position p?  (explicit mask) */
int oracle_attends(int mask_mode, int64_t P, int64_t p, int n_sink, int window) {
    if (p < 0 || p > P) return 0;                  /* causal: only earlier or same positions */
    if (mask_mode == OR_CAUSAL) return 1;
    return (p < n_sink) || (p >= P - window + 1);  /* sinks, or inside the trailing window */
}

/* Tree mask: does a new row with mask word `bits` attend position p of a sequence
 * whose new block starts at P0 and holds q_len positions? */
int oracle_attends_tree(int64_t P0, int q_len, uint64_t bits, int64_t p) {
    if (p < 0) return 0;
    if (p < P0) return 1;                          /* the cached prefix */
    if (p >= P0 + q_len) return 0;
    return (int)((bits >> (p - P0)) & 1u);         /* an ancestor in the tree, or itself */
}

/* Flat slot (row of the [slots, Hkv, d] view of the cache) holding position p
 * of sequence b.  Returns -1 when the position has no slot. */
int64_t oracle_slot(int cache_mode, int b, int64_t p, int capacity, int block_size,
                    const int32_t* block_table, int blocks_per_seq, int n_sink) {
    if (p < 0) return -1;
    if (cache_mode == OR_CONTIGUOUS) {
        if (p >= capacity) return -1;
        return (int64_t)b * capacity + p;
    }
    if (cache_mode == OR_PAGED) {
        if (p >= capacity) return -1;
        int64_t page = p / block_size;
        int64_t phys = block_table[(int64_t)b * blocks_per_seq + page];
        return phys * block_size + p % block_size;
    }
    /* ring: sinks pinned at the front, the rest rolls over capacity - n_sink slots */
    if (p < n_sink) return (int64_t)b * capacity + p;
    return (int64_t)b * capacity + n_sink + (p - n_sink) % (capacity - n_sink);
}

/* Enumerate, in increasing position order, what the row (b, i) attends.
 * Writes up to `max_out` positions and slots (either pointer may be NULL);
 * returns the total count. */
int64_t oracle_attended(int cache_mode, int mask_mode, int b, int i, int q_len, int64_t T,
                        int n_sink, int window, int capacity, int block_size,
                        const int32_t* block_table, int blocks_per_seq, uint64_t tree_bits,
                        int64_t* pos_out, int64_t* slot_out, int64_t max_out) {
    int64_t P = T - q_len + i;
    int64_t n = 0;
    for (int64_t p = 0; p < T; ++p) {
        const int att = mask_mode == OR_TREE ? oracle_attends_tree(T - q_len, q_len, tree_bits, p)
                                             : oracle_attends(mask_mode, P, p, n_sink, window);
        if (!att) continue;
        if (n < max_out) {
            if (pos_out) pos_out[n] = p;
            if (slot_out)
                slot_out[n] = oracle_slot(cache_mode, b, p, capacity, block_size, block_table,
                                          blocks_per_seq, n_sink);
        }
        ++n;
    }
    return n;
}

typedef struct {
    int dtype, batch, num_q_heads, num_kv_heads, head_dim, q_len;
    int cache_mode, capacity, block_size, blocks_per_seq;
    int mask_mode, n_sink, window;
    double scale;                 /* 0 => 1/sqrt(head_dim) */
    int kv_dtype;                 /* element type of the caches; dtype when equal */
    const float* k_scale;         /* [num_kv_heads] dequantisation scales, or NULL (1) */
    const float* v_scale;
    const uint64_t* tree_mask;    /* OR_TREE: [batch, q_len] mask words, else unused */
} oracle_problem;

/* One output row: out[d] for (b, i, h).  Returns the number of attended
 * positions (0 => the row is all zeros by convention). */
static int64_t decode_one_row(const oracle_problem* pr, const void* q, const void* kc,
                              const void* vc, const int32_t* block_table, int64_t T,
                              int b, int i, int h, double* out, int64_t* slots, double* w) {
    const int D = pr->head_dim;
    const int g = pr->num_q_heads / pr->num_kv_heads;
    const int kvh = h / g;
    const double scale = pr->scale != 0.0 ? pr->scale : 1.0 / sqrt((double)D);
    const uint64_t bits =
        pr->mask_mode == OR_TREE ? pr->tree_mask[(int64_t)b * pr->q_len + i] : 0;
    const int64_t n = oracle_attended(pr->cache_mode, pr->mask_mode, b, i, pr->q_len, T,
                                      pr->n_sink, pr->window, pr->capacity, pr->block_size,
                                      block_table, pr->blocks_per_seq, bits, NULL, slots,
                                      INT64_MAX);
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (n == 0) return 0;
    const int64_t qbase = (((int64_t)b * pr->q_len + i) * pr->num_q_heads + h) * D;
    const int kvt = pr->kv_dtype;
    const double ks = pr->k_scale ? (double)pr->k_scale[kvh] : 1.0;
    const double vs = pr->v_scale ? (double)pr->v_scale[kvh] : 1.0;
    /* scores s_p = q . k_p * scale, k_p dequantised */
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        const int64_t kbase = (slots[j] * pr->num_kv_heads + kvh) * D;
        double s = 0.0;
        for (int d = 0; d < D; ++d)
            s += load_elem(q, pr->dtype, qbase + d) * (load_elem(kc, kvt, kbase + d) * ks);
        w[j] = s * scale;
        if (w[j] > m) m = w[j];
    }
    /* softmax weights */
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        w[j] = exp(w[j] - m);
        sum += w[j];
    }
    /* weighted sum of V */
    for (int64_t j = 0; j < n; ++j) {
        const double wj = w[j] / sum;
        const int64_t vbase = (slots[j] * pr->num_kv_heads + kvh) * D;
        for (int d = 0; d < D; ++d) out[d] += wj * (load_elem(vc, kvt, vbase + d) * vs);
    }
    return n;
}

/* Longest attended list over the batch (sizes the per-thread scratch). */
static int64_t max_attended(const oracle_problem* pr, const int32_t* seq_lens) {
    int64_t mx = 0;
    for (int b = 0; b < pr->batch; ++b)
        if (seq_lens[b] > mx) mx = seq_lens[b];
    return mx;
}

/*
 * Compute the listed rows.  rows[3*r .. 3*r+2] = (b, i, h); out[r*D .. r*D+D).
 * n_threads <= 0 => OpenMP default.  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int oracle_decode_rows(const oracle_problem* pr, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* rows, int64_t n_rows, double* out, int n_threads) {
    if (!pr || pr->num_kv_heads <= 0 || pr->num_q_heads % pr->num_kv_heads) return -1;
    if (pr->mask_mode == OR_TREE && (pr->cache_mode == OR_RING || !pr->tree_mask || pr->q_len > 64))
        return -1;
    if (pr->cache_mode == OR_RING) {
        /* every position a row can attend must still be live in the ring */
        if (pr->mask_mode != OR_SINK_WINDOW || pr->window < 1 ||
            (int64_t)pr->n_sink + pr->window + pr->q_len - 1 > pr->capacity)
            return -1;
    } else {
        for (int b = 0; b < pr->batch; ++b)
            if (seq_lens[b] > pr->capacity) return -1;
    }
    const int64_t cap = max_attended(pr, seq_lens) + 1;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel
    {
        int64_t* slots = (int64_t*)malloc(sizeof(int64_t) * cap);
        double* w = (double*)malloc(sizeof(double) * cap);
        if (!slots || !w) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n_rows; ++r) {
                const int b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
                decode_one_row(pr, q, k_cache, v_cache, block_table, seq_lens[b], b, i, h,
                               out + r * pr->head_dim, slots, w);
            }
        }
        free(slots);
        free(w);
    }
    return err ? -1 : 0;
}

/* Every row, out laid out [batch, q_len, num_q_heads, head_dim]. */
int oracle_decode(const oracle_problem* pr, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                  double* out, int n_threads) {
    const int64_t n_rows = (int64_t)pr->batch * pr->q_len * pr->num_q_heads;
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * 3 * (n_rows ? n_rows : 1));
    if (!rows) return -1;
    int64_t r = 0;
    for (int b = 0; b < pr->batch; ++b)
        for (int i = 0; i < pr->q_len; ++i)
            for (int h = 0; h < pr->num_q_heads; ++h, ++r) {
                rows[3 * r] = b;
                rows[3 * r + 1] = i;
                rows[3 * r + 2] = h;
            }
    int rc = oracle_decode_rows(pr, q, k_cache, v_cache, block_table, seq_lens, rows, n_rows,
                                out, n_threads);
    free(rows);
    return rc;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
