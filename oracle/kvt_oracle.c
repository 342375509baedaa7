/*
 * kvt_oracle.c -- plain, slow, obviously correct CPU oracle for the tiered KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file:
 * only the tests, the smoke check and the bench's CPU-baseline leg use it.  It shares no
 * code, header, table or constant with the HIP library; the two are compared, never mixed.
 *
 * Every floating-point result is computed in fp64 from the exact values the stored bytes
 * encode (IEEE fp16 / bf16 / q8_0 decoded here from their definitions).  Copies are plain
 * memcpy loops.  Top-k is a full sort.  OpenMP only splits independent output rows.
 *
 * Sources (the pages this follows):
 *   [vLLM-CPU] "vllm/v1/kv_offload/cpu/gpu_worker.py" (a vLLM fork's CPU offloading worker):
 *              compute_sub_block_ptrs, _fill_direct_ops, transfer_async.
 *   [QSA-KVO]  "QSA KV cache host-RAM offload for ExLlamaV3" (qsa-kv-offload.patch):
 *              CacheLayer_qsa_offload docstring, QSAIndexer.sparse_attend,
 *              qsa_sparse_attend_rows_staged, the online-softmax fold.
 *   [llama-T]  "llama/cuda: tiered KV cache (--kv-vram-cells)", llama.cpp PR #319:
 *              the commit text on the VRAM head / host tail and tail staging.
 *
 * Status codes: 0 ok, -1 invalid argument, -2 out of range, -4 overlap.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ERANGE (-2)
#define ORC_EOVERLAP (-4)

/* element formats, numbered independently of the library (same meaning) */
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_Q8_0 3

/* ------------------------------------------------------------------------------------------ */
/* scalar decoders, written from the IEEE 754 binary16 and bfloat16 definitions               */
/* ------------------------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 value. */
double orc_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return (double)x;
}

static double elem_to_f64(const uint8_t *p, int fmt)
{
    uint16_t u;
    memcpy(&u, p, 2);
    return fmt == ORC_BF16 ? orc_bf16_to_f64(u) : orc_f16_to_f64(u);
}

/* q8_0 block: 2-byte little-endian fp16 scale d, then 32 signed bytes q; value = d * q.
 * A K or V row of `kvh` heads x `hd` dims is kvh * hd/32 consecutive blocks, head-major. */
static double q8_0_value(const uint8_t *row, int kvh_index, int hd, int dim)
{
    const uint8_t *blk = row + (size_t)(kvh_index * (hd / 32) + dim / 32) * 34;
    uint16_t d;
    memcpy(&d, blk, 2);
    int8_t q = (int8_t)blk[2 + dim % 32];
    return orc_f16_to_f64(d) * (double)q;
}

/* ------------------------------------------------------------------------------------------ */
/* O1  sub-block pointer tables            [vLLM-CPU] compute_sub_block_ptrs                  */
/* ------------------------------------------------------------------------------------------ */
/* Block b of the tensor holds `bpc` sub-blocks (pages) of `page_bytes` each; sub-block j of b
 * starts at base + b*row_stride + j*page_bytes.  The pointers of all listed blocks are laid
 * out block-major and the run [skip, skip + n_out) of that list is the output. */
int orc_sub_block_ptrs(uint64_t base, uint64_t row_stride, uint64_t page_bytes,
                       const int64_t *block_ids, int64_t n_ids, int32_t bpc, int32_t skip,
                       uint64_t *out, int64_t n_out)
{
    if (bpc < 1 || skip < 0 || skip >= bpc || n_ids < 0 || n_out < 0)
        return ORC_EINVAL;
    if (n_out > n_ids * (int64_t)bpc - skip)
        return ORC_ERANGE;
    for (int64_t o = 0; o < n_out; o++) {
        int64_t flat = o + skip;      /* position in the block-major list */
        int64_t i = flat / bpc;       /* which listed block */
        int64_t j = flat % bpc;       /* which sub-block inside it */
        if (block_ids[i] < 0)
            return ORC_ERANGE;
        out[o] = base + (uint64_t)block_ids[i] * row_stride + (uint64_t)j * page_bytes;
    }
    return ORC_OK;
}

/* Number of chunk-side blocks a transfer of n sub-blocks starting `skip` into its first block
 * consumes: ceil((n + skip) / bpc)   [vLLM-CPU] transfer_async. */
int64_t orc_chunks_consumed(int64_t n, int32_t skip, int32_t bpc)
{
    return (n + skip + bpc - 1) / bpc;
}

/* ------------------------------------------------------------------------------------------ */
/* O2  batched swap                        [vLLM-CPU] transfer_async -> swap_blocks_batch     */
/* ------------------------------------------------------------------------------------------ */
/* Destination ranges must not overlap each other or any source range (the copy order is then
 * irrelevant).  Checked by brute force, O(n^2) -- keep n moderate. */
int orc_check_disjoint(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, int64_t n)
{
    for (int64_t i = 0; i < n; i++) {
        if (!sizes[i])
            continue;
        for (int64_t j = 0; j < n; j++) {
            if (!sizes[j])
                continue;
            if (j != i && dst[i] < dst[j] + sizes[j] && dst[j] < dst[i] + sizes[i])
                return ORC_EOVERLAP;
            if (dst[i] < src[j] + sizes[j] && src[j] < dst[i] + sizes[i])
                return ORC_EOVERLAP;
        }
    }
    return ORC_OK;
}

/* copy sizes[i] bytes from address src[i] to address dst[i], for every i; size 0 is a no-op */
int orc_swap(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, int64_t n,
             int nthreads)
{
    if (n < 0)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t i = 0; i < n; i++)
        if (sizes[i])
            memcpy((void *)(uintptr_t)dst[i], (const void *)(uintptr_t)src[i], (size_t)sizes[i]);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O3  index scoring and top-k             [QSA-KVO] CacheLayer_qsa_offload docstring:        */
/*     the pooled plane is scored in full on every step; a top-k selection picks the blocks   */
/* ------------------------------------------------------------------------------------------ */
/* s[h][b] = sum over d = 0 .. dim-1 (in that order) of q[h][d] * pooled[b][d], in fp64.
 * Inputs are fp16; each product is exact in fp64. */
int orc_index_scores(const uint16_t *pooled, int64_t n_blocks, int32_t dim, const uint16_t *q,
                     int32_t n_sel, double *scores, int nthreads)
{
    if (n_blocks < 0 || dim < 1 || n_sel < 1)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t b = 0; b < n_blocks; b++) {
        for (int32_t h = 0; h < n_sel; h++) {
            double s = 0.0;
            for (int32_t d = 0; d < dim; d++)
                s += orc_f16_to_f64(q[(size_t)h * dim + d]) *
                     orc_f16_to_f64(pooled[(size_t)b * dim + d]);
            scores[(size_t)h * n_blocks + b] = s;
        }
    }
    return ORC_OK;
}

typedef struct {
    double s;
    int64_t id;
} orc_cand;

/* rank order: larger score first; equal scores -> lower block id first; NaN after all numbers */
static int cand_cmp(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn)
        return an ? 1 : -1;
    if (!an && a->s != b->s)
        return a->s > b->s ? -1 : 1;
    return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);
}

static int id_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* Per selection head: sort all blocks by rank order, keep the first k, emit their ids in
 * ascending order; when k exceeds n_blocks the remaining slots hold -1. */
int orc_topk(const double *scores, int32_t n_sel, int64_t n_blocks, int32_t k, int32_t *ids)
{
    if (n_sel < 1 || n_blocks < 0 || k < 1)
        return ORC_EINVAL;
    orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(n_blocks ? n_blocks : 1));
    if (!c)
        return ORC_EINVAL;
    for (int32_t h = 0; h < n_sel; h++) {
        for (int64_t b = 0; b < n_blocks; b++) {
            c[b].s = scores[(size_t)h * n_blocks + b];
            c[b].id = b;
        }
        qsort(c, (size_t)n_blocks, sizeof(orc_cand), cand_cmp);
        int32_t *row = ids + (size_t)h * k;
        int32_t take = (int32_t)(n_blocks < k ? n_blocks : k);
        for (int32_t i = 0; i < take; i++)
            row[i] = (int32_t)c[i].id;
        qsort(row, (size_t)take, sizeof(int32_t), id_cmp);
        for (int32_t i = take; i < k; i++)
            row[i] = -1;
    }
    free(c);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O4  top-k gather                        [QSA-KVO] sparse_attend / CacheLayer_qsa_offload   */
/* ------------------------------------------------------------------------------------------ */
/* A plane is addressed through byte strides ("a base pointer plus computed offsets"): token r
 * of physical block p, head h starts at  plane + p*block_stride + h*head_stride + r*token_stride
 * and holds hd elements of elem_bytes.  The pages' token-major layout [token][head][dim] is
 * block_stride = bt*kvh*hd*eb, head_stride = hd*eb, token_stride = kvh*hd*eb.
 * Logical block b lives in physical block table[b] (identity when the table is NULL).
 * For head h and selection slot i with id b >= 0:
 *   out[h][i*bt + r][:] = the hd elements of token r of block phys(b), head h,  r < bt.
 * Slots with id < 0 are left untouched; a block outside [0, n_blocks) is an error. */
int orc_gather(const uint8_t *k_plane, const uint8_t *v_plane, int64_t n_blocks, int32_t kvh,
               int32_t hd, int32_t elem_bytes, int64_t block_stride, int64_t head_stride,
               int64_t token_stride, const int32_t *block_table, int32_t bt, const int32_t *ids,
               int32_t k, uint8_t *k_out, uint8_t *v_out)
{
    if (kvh < 1 || hd < 1 || elem_bytes < 1 || bt < 1 || k < 1 || n_blocks < 0)
        return ORC_EINVAL;
    size_t slice = (size_t)hd * elem_bytes;
    for (int32_t h = 0; h < kvh; h++) {
        for (int32_t i = 0; i < k; i++) {
            int32_t b = ids[(size_t)h * k + i];
            if (b < 0)
                continue;
            int64_t pb = block_table ? block_table[b] : b;
            if (pb < 0 || pb >= n_blocks)
                return ORC_ERANGE;
            for (int32_t r = 0; r < bt; r++) {
                size_t src_off = (size_t)(pb * block_stride + (int64_t)h * head_stride +
                                          (int64_t)r * token_stride);
                size_t dst_off = ((size_t)h * k * bt + (size_t)i * bt + r) * slice;
                memcpy(k_out + dst_off, k_plane + src_off, slice);
                memcpy(v_out + dst_off, v_plane + src_off, slice);
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O5  tail staging                        [llama-T] commit text: used host rows -> VRAM      */
/* ------------------------------------------------------------------------------------------ */
/* staging[r - row_begin] = plane[r] for r in [row_begin, row_end), bytes */
int orc_stage_tail(const uint8_t *plane, int64_t row_bytes, int64_t row_begin, int64_t row_end,
                   uint8_t *staging)
{
    if (row_bytes < 1 || row_begin < 0 || row_end < row_begin)
        return ORC_EINVAL;
    for (int64_t r = row_begin; r < row_end; r++)
        memcpy(staging + (size_t)(r - row_begin) * row_bytes, plane + (size_t)r * row_bytes,
               (size_t)row_bytes);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O6  decode attention over gathered K/V  [QSA-KVO] staged path: GQA map, softmax, fold      */
/* ------------------------------------------------------------------------------------------ */
/* q: [n_qh][hd], K/V: [kvh][n_kv][hd], all of format fmt (F16 or BF16).  Query head i reads
 * kv head i / (n_qh / kvh).  Keys j < n_valid[kv] take part (all n_kv when n_valid is NULL):
 *   l_j = scale * q_i . K[kv][j],  o_i = sum_j exp(l_j - max l) V[kv][j] / sum_j exp(l_j - max l)
 * No valid key gives o_i = 0. */
int orc_attn_decode(const uint8_t *q, int32_t n_qh, int32_t kvh, int32_t hd, int32_t fmt,
                    const uint8_t *k, const uint8_t *v, int64_t n_kv, const int32_t *n_valid,
                    double scale, double *out, int nthreads)
{
    if (n_qh < 1 || kvh < 1 || n_qh % kvh || hd < 1 || n_kv < 0 ||
        (fmt != ORC_F16 && fmt != ORC_BF16))
        return ORC_EINVAL;
    int32_t group = n_qh / kvh;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (int32_t i = 0; i < n_qh; i++) {
        int32_t kv = i / group;
        int64_t nv = n_valid ? n_valid[kv] : n_kv;
        if (nv > n_kv)
            nv = n_kv;
        double *o = out + (size_t)i * hd;
        for (int32_t d = 0; d < hd; d++)
            o[d] = 0.0;
        if (nv <= 0)
            continue;
        double *l = (double *)malloc(sizeof(double) * (size_t)nv);
        double m = -INFINITY;
        for (int64_t j = 0; j < nv; j++) {
            double s = 0.0;
            for (int32_t d = 0; d < hd; d++)
                s += elem_to_f64(q + ((size_t)i * hd + d) * 2, fmt) *
                     elem_to_f64(k + (((size_t)kv * n_kv + j) * hd + d) * 2, fmt);
            l[j] = scale * s;
            if (l[j] > m)
                m = l[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < nv; j++) {
            double w = exp(l[j] - m);
            den += w;
            for (int32_t d = 0; d < hd; d++)
                o[d] += w * elem_to_f64(v + (((size_t)kv * n_kv + j) * hd + d) * 2, fmt);
        }
        for (int32_t d = 0; d < hd; d++)
            o[d] /= den;
        free(l);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* O7  tiered prefill attention            [llama-T] VRAM head + host tail, output identical  */
/*     to an all-device cache; [QSA-KVO] GQA map                                              */
/* ------------------------------------------------------------------------------------------ */
/* The cache holds n_kv logical rows; row r lives at head + r*row_bytes when r < n_head and at
 * tail + (r - n_head)*row_bytes otherwise.  A row holds kvh heads x hd dims in format fmt
 * (F16, BF16: hd*2 bytes per head; Q8_0: hd/32 blocks of 34 bytes per head).
 * q: [n_q][n_qh][hd] fp16; query row t sits at position q_pos0 + t.  With causal set it sees
 * keys j <= q_pos0 + t (and j < n_kv); otherwise all n_kv keys.  Only query rows
 * [t_begin, t_end) are computed; out holds [t_end - t_begin][n_qh][hd] doubles. */
static double kv_value(const uint8_t *row, int32_t fmt, int32_t hd, int32_t h, int32_t d)
{
    if (fmt == ORC_Q8_0)
        return q8_0_value(row, h, hd, d);
    return elem_to_f64(row + ((size_t)h * hd + d) * 2, fmt);
}

int orc_attn_prefill(const uint16_t *q, int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh,
                     int32_t hd, const uint8_t *k_head, const uint8_t *v_head, int64_t n_head,
                     const uint8_t *k_tail, const uint8_t *v_tail, int64_t n_kv, int32_t fmt,
                     int32_t causal, double scale, int64_t t_begin, int64_t t_end, double *out,
                     int nthreads)
{
    if (n_q < 0 || n_qh < 1 || kvh < 1 || n_qh % kvh || hd < 1 || n_kv < 0 || n_head < 0 ||
        n_head > n_kv || t_begin < 0 || t_end > n_q || t_end < t_begin)
        return ORC_EINVAL;
    if (fmt != ORC_F16 && fmt != ORC_BF16 && fmt != ORC_Q8_0)
        return ORC_EINVAL;
    if (fmt == ORC_Q8_0 && hd % 32)
        return ORC_EINVAL;
    int64_t row_bytes = fmt == ORC_Q8_0 ? (int64_t)kvh * (hd / 32) * 34 : (int64_t)kvh * hd * 2;
    int32_t group = n_qh / kvh;
    int64_t n_rows = (t_end - t_begin) * n_qh;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t x = 0; x < n_rows; x++) {
        int64_t t = t_begin + x / n_qh;
        int32_t i = (int32_t)(x % n_qh);
        int32_t kv = i / group;
        int64_t last = causal ? q_pos0 + t : n_kv - 1;
        if (last > n_kv - 1)
            last = n_kv - 1;
        double *o = out + (size_t)x * hd;
        for (int32_t d = 0; d < hd; d++)
            o[d] = 0.0;
        if (last < 0)
            continue;
        const uint16_t *qi = q + ((size_t)t * n_qh + i) * hd;
        double *qd = (double *)malloc(sizeof(double) * (size_t)hd);
        for (int32_t d = 0; d < hd; d++)
            qd[d] = orc_f16_to_f64(qi[d]);
        double *l = (double *)malloc(sizeof(double) * (size_t)(last + 1));
        double m = -INFINITY;
        for (int64_t j = 0; j <= last; j++) {
            const uint8_t *kr = j < n_head ? k_head + (size_t)j * row_bytes
                                           : k_tail + (size_t)(j - n_head) * row_bytes;
            double s = 0.0;
            for (int32_t d = 0; d < hd; d++)
                s += qd[d] * kv_value(kr, fmt, hd, kv, d);
            l[j] = scale * s;
            if (l[j] > m)
                m = l[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j <= last; j++) {
            const uint8_t *vr = j < n_head ? v_head + (size_t)j * row_bytes
                                           : v_tail + (size_t)(j - n_head) * row_bytes;
            double w = exp(l[j] - m);
            den += w;
            for (int32_t d = 0; d < hd; d++)
                o[d] += w * kv_value(vr, fmt, hd, kv, d);
        }
        for (int32_t d = 0; d < hd; d++)
            o[d] /= den;
        free(l);
        free(qd);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Pool rebuild at the write head          [QSA-KVO] CacheLayer_qsa_offload docstring          */
/* ------------------------------------------------------------------------------------------ */
/* fp64 -> fp16, rounding to nearest with ties to even, from the definition: for a normal
 * result the value is scaled so that its 11 significant bits are the integer part, for a
 * subnormal one it is counted in units of 2^-24; the remainder decides the rounding.  Values
 * at or beyond 65520 (halfway between 65504 and 65536) round to infinity.  NaN gives 0x7E00. */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7E00;
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7C00);
    int e;
    (void)frexp(a, &e);                  /* a = f * 2^e, f in [0.5, 1) */
    int unbiased = e - 1;                /* a in [2^unbiased, 2^(unbiased+1)) */
    double units;                        /* a in units of the result's last place */
    int32_t bits_exp;
    if (a == 0.0 || unbiased < -14) {    /* subnormal (or zero) */
        units = ldexp(a, 24);
        bits_exp = 0;
    } else {
        units = ldexp(a, 10 - unbiased); /* in [1024, 2048) */
        bits_exp = unbiased + 15;
    }
    double whole = floor(units);
    double rem = units - whole;          /* exact: both are in a range where doubles are exact */
    uint32_t q = (uint32_t)whole;
    if (rem > 0.5 || (rem == 0.5 && (q & 1u)))
        q++;
    /* normal: q in [1024, 2048]; the implicit bit goes into the exponent field by addition,
     * which also carries q == 2048 into the next binade (and 65504 + ulp into infinity) */
    uint32_t bits = bits_exp == 0 ? q : ((uint32_t)(bits_exp - 1) << 10) + q;
    return (uint16_t)(sign | bits);
}

/* After an append of seq tokens to sequence b at positions [len, len + seq), len =
 * cache_seqlens[b] (len < 0: no such sequence), every pooled block those positions fall in,
 * j = len/cr ... (len + seq - 1)/cr, is rebuilt from the raw key rows the block holds: rows
 * [j*cr, min(j*cr + cr, len + seq)).  The pooled key is the mean of those rows, per element:
 * their sum in fp64 (exact for up to 512 fp16 values), divided by the count, rounded once to
 * fp16.  A block's rows sit in page block_table[b][(j*cr) / page_size] (cr divides
 * page_size), rows (j*cr) % page_size.., and its pooled row is row ((j*cr) % page_size) / cr
 * of the same page in the pooled plane.  Blocks whose table slot or page is out of range are
 * skipped.  raw: [n_pages][page_size][dim] fp16 bits; pooled: [n_pages][page_size/cr][dim]. */
int orc_pool_rebuild(const uint16_t *raw, uint16_t *pooled, int32_t dim, int32_t bsz, int32_t seq,
                     const int32_t *cache_seqlens, const int32_t *block_table,
                     int32_t pages_per_seq, int32_t page_size, int32_t cr, int64_t n_pages)
{
    if (dim < 1 || bsz < 0 || seq < 0 || pages_per_seq < 1 || page_size < 1 || cr < 1 ||
        cr > 512 || page_size % cr || n_pages < 0)
        return ORC_EINVAL;
    const int32_t per_page = page_size / cr;
    for (int32_t b = 0; b < bsz; b++) {
        const int64_t len = cache_seqlens[b];
        if (len < 0 || seq == 0)
            continue;
        const int64_t end = len + seq;
        for (int64_t j = len / cr; j <= (end - 1) / cr; j++) {
            const int64_t first = j * cr;
            const int64_t slot = first / page_size;
            if (slot >= pages_per_seq)
                continue;
            const int64_t page = block_table[(int64_t)b * pages_per_seq + slot];
            if (page < 0 || page >= n_pages)
                continue;
            const int64_t rows = (end - first) < cr ? (end - first) : cr;
            const int64_t row0 = first % page_size;
            for (int32_t d = 0; d < dim; d++) {
                double s = 0.0;
                for (int64_t r = 0; r < rows; r++)
                    s += orc_f16_to_f64(raw[((size_t)page * page_size + row0 + r) * dim + d]);
                pooled[((size_t)page * per_page + row0 / cr) * dim + d] =
                    orc_f64_to_f16(s / (double)rows);
            }
        }
    }
    return ORC_OK;
}
