/*
 * CPU oracle for token-wise INT4 KV-cache quantization with a block-diagonal
 * Hadamard rotation, and for paged decode attention over that cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * path (the HIP library) never links, imports or calls it, and it shares no
 * source, header, table or helper with the HIP kernels.
 *
 * It is deliberately plain and slow: scalar loops in the order the method is
 * described, no blocking, no fusion, no reordering.  The quantization path is
 * fp32 (that is the arithmetic whose result must be reproduced bit for bit);
 * attention is fp64.  Build with `gcc -O2 -ffp-contract=off` so that no
 * multiply-add is fused behind our back, and never with -ffast-math.
 *
 * Sources (cited by page title and section):
 *   [EXPL]  "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化"
 *           (youngju.dev blog explainer of the SAW-INT4 preprint).
 *           Sections used: "KVキャッシュこそが本当のボトルネックである理由"
 *           (the KV cache as bottleneck; paged layout, fused attention),
 *           "素朴なINT4はなぜ崩れるのか" (naive INT4; token-wise scales),
 *           "回転のトリック — ブロック対角アダマール" (block-diagonal Hadamard),
 *           "システムこそが設計である — 融合カーネル" and its figure
 *           (fused rotate + quantize + append into paged KV blocks).
 *   [SUMM]  "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World
 *           LLM Serving" (gist.science AI-generated summary), sections on the
 *           problem, the solution and the results.
 *   [BDFP4] "BitDecoding-FP4:FP4 KVキャッシュのネイティブ復号" (sns.style),
 *           opening summary and section 深掘り分析: the quantizer variants at
 *           the end of this file (scales per group chosen by search, 4-bit
 *           microscaling formats).
 * Where the pages leave a step open, the reading taken is stated at the step.
 * Every such reading is one the HIP path must reproduce exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD (-1)

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, written from the format definitions.          */
/* ------------------------------------------------------------------------ */

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary16 -> binary32.  Every half value is exactly representable. */
float kvq_oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t expo = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t frac = (uint32_t)h & 0x3FFu;
    float mag;
    if (expo == 0x1Fu) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        /* subnormal: frac * 2^-24, exact in binary32 */
        mag = ldexpf((float)frac, -24);
    } else {
        mag = ldexpf((float)(frac | 0x400u), (int)expo - 25);
    }
    return sign ? -mag : mag;
}

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t kvq_oracle_f32_to_f16(float f)
{
    uint32_t u = bits_of(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t expo = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;

    if (expo == 0xFFu) {                        /* Inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (frac ? 0x200u : 0u));
    }
    /* Work with the exact value  m * 2^(e) where m is a 24-bit integer. */
    if (expo == 0 && frac == 0) return sign;   /* signed zero */
    uint32_t m;
    int e;
    if (expo == 0) { m = frac; e = -149; }     /* binary32 subnormal */
    else { m = frac | 0x800000u; e = (int)expo - 150; }

    /* Target: half normal values are M * 2^(E-25) with M in [1024, 2047],
     * E in [1, 30]; subnormals are M * 2^-24 with M in [0, 1023].
     * Find the exponent q of the unit in the last place of the result. */
    /* value = m * 2^e; position of the leading bit: */
    int lead = 31 - __builtin_clz(m) + e;      /* value in [2^lead, 2^(lead+1)) */
    int q = lead - 10;                          /* ulp exponent for a normal half */
    if (q < -24) q = -24;                       /* subnormal range: fixed ulp 2^-24 */
    /* round m * 2^e to a multiple of 2^q, ties to even */
    int shift = q - e;                          /* number of bits to drop */
    uint64_t M;
    if (shift <= 0) {
        M = (uint64_t)m << (-shift);
    } else if (shift > 40) {
        M = 0;                                  /* far below half an ulp */
    } else {
        uint64_t mm = m;
        uint64_t kept = mm >> shift;
        uint64_t rem = mm & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (kept & 1ull))) kept += 1;
        M = kept;
    }
    /* Rounding may have carried into a new binade. */
    if (M >= 2048) { M >>= 1; q += 1; }
    if (q < -24) return sign;                   /* cannot happen, kept for clarity */
    if (M < 1024) {
        /* subnormal (q == -24) or zero */
        return (uint16_t)(sign | (uint16_t)M);
    }
    int E = q + 25;                             /* biased half exponent */
    if (E >= 31) return (uint16_t)(sign | 0x7C00u);   /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)(M - 1024));
}

/* ------------------------------------------------------------------------ */
/* Block-diagonal Hadamard rotation  ([EXPL] "回転のトリック").               */
/* ------------------------------------------------------------------------ */

/* Reading: the Hadamard matrix is Sylvester's, in natural order
 * (H_2n = [[H, H], [H, -H]]); the rotation is R = H / sqrt(Bh), so it is
 * orthogonal and its own inverse, as the section requires.  The fp32 factor
 * is the round-to-nearest binary32 value of 1/sqrt(Bh).  For the block sizes
 * the cache supports these are 0x3E3504F3 (Bh=32), 0x3E000000 (Bh=64) and
 * 0x3DB504F3 (Bh=128); a test pins them against a 50-digit computation. */
float kvq_oracle_hadamard_scale(int bh)
{
    if (bh <= 0) return 1.0f;
    return (float)(1.0 / sqrt((double)bh));
}

/* Unnormalised FWHT applied independently to each contiguous block of Bh
 * entries (the rotation never crosses a block, which is what keeps it
 * compatible with the paged layout).  Stages run with the butterfly span h
 * ascending 1, 2, 4, ..., Bh/2; each butterfly replaces (u, v) by
 * (u + v, u - v), one binary32 operation each. */
void kvq_oracle_fwht_f32(float *y, int n, int bh)
{
    if (bh <= 1) return;
    for (int b0 = 0; b0 + bh <= n; b0 += bh) {
        for (int h = 1; h < bh; h <<= 1) {
            for (int i = 0; i < bh; i++) {
                if (i & h) continue;
                float u = y[b0 + i];
                float v = y[b0 + i + h];
                y[b0 + i] = u + v;
                y[b0 + i + h] = u - v;
            }
        }
    }
}

/* fp64 rotation R.x = H.x / sqrt(Bh) per block (used for the query and the
 * inverse rotation of the attention output; R is its own inverse). */
void kvq_oracle_rotate_f64(double *x, int n, int bh)
{
    if (bh <= 0) return;
    double c = 1.0 / sqrt((double)bh);
    for (int b0 = 0; b0 + bh <= n; b0 += bh) {
        for (int h = 1; h < bh; h <<= 1) {
            for (int i = 0; i < bh; i++) {
                if (i & h) continue;
                double u = x[b0 + i];
                double v = x[b0 + i + h];
                x[b0 + i] = u + v;
                x[b0 + i + h] = u - v;
            }
        }
        for (int i = 0; i < bh; i++) x[b0 + i] *= c;
    }
}

/* ------------------------------------------------------------------------ */
/* Token-wise INT4 quantization of one vector ([EXPL] "素朴なINT4は..." for    */
/* the one-scale-per-token choice, "回転のトリック" for rotating first, and   */
/* the fused-kernel figure for the order rotate -> quantize -> append).       */
/* ------------------------------------------------------------------------ */

#define ORACLE_MAX_D 1024

/* x: D fp16 values of one (token, KV head, K-or-V).  Writes D/2 packed bytes
 * and one fp16 scale.  Steps:
 *   1. widen to fp32 (exact);
 *   2. if Bh > 0: block FWHT (above), then multiply by the fp32 1/sqrt(Bh);
 *   3. m = max |y|;
 *   4. scale s32 = m / 7 (IEEE division), stored as s16 = fp16(s32) (RNE).
 *      Reading: symmetric absmax scale, no zero point, stored in fp16, and
 *      the codes are computed against the stored s16 so that decode sees
 *      exactly the scale the codes were made with;
 *   5. if s16 == 0 every code is 0; else code = clamp(rint(y / s16), -8, 7)
 *      with IEEE division and rounding half to even;
 *   6. two's-complement nibbles, element 2j in the low nibble of byte j. */
int kvq_oracle_quantize_vector(const uint16_t *x, int d, int bh,
                               uint8_t *codes, uint16_t *scale_out)
{
    if (d <= 0 || d > ORACLE_MAX_D || (d & 1)) return ORACLE_BAD;
    if (bh < 0 || (bh > 0 && (bh > d || (bh & (bh - 1)) || d % bh))) return ORACLE_BAD;
    float y[ORACLE_MAX_D];
    for (int i = 0; i < d; i++) y[i] = kvq_oracle_f16_to_f32(x[i]);
    if (bh > 1) {
        kvq_oracle_fwht_f32(y, d, bh);
        float c = kvq_oracle_hadamard_scale(bh);
        for (int i = 0; i < d; i++) y[i] = y[i] * c;
    }
    float m = 0.0f;
    for (int i = 0; i < d; i++) {
        float a = fabsf(y[i]);
        if (a > m) m = a;
    }
    float s32 = m / 7.0f;
    uint16_t s16 = kvq_oracle_f32_to_f16(s32);
    float s = kvq_oracle_f16_to_f32(s16);
    for (int j = 0; j < d / 2; j++) {
        int c[2];
        for (int t = 0; t < 2; t++) {
            int code = 0;
            if (s != 0.0f) {
                float qv = y[2 * j + t] / s;
                code = (int)rintf(qv);
                if (code < -8) code = -8;
                if (code > 7) code = 7;
            }
            c[t] = code;
        }
        codes[j] = (uint8_t)((c[0] & 0xF) | ((c[1] & 0xF) << 4));
    }
    *scale_out = s16;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Paged layout ([EXPL] "KVキャッシュこそが..." names the paged layout; the  */
/* fused-kernel figure appends each token into a paged block).               */
/* Reading (the pages fix no byte layout): one physical page of a pool holds */
/* the code rows of KV heads 0..Hkv-1 ([P][D/2] bytes each), then the scales */
/* of heads 0..Hkv-1 ([P] little-endian fp16 each): Hkv * tile bytes, with   */
/* tile = P*D/2 + 2P the share of one (page, head); separate pools for K    */
/* and V.                                                                    */
/* The page table is int32 [batch][max_pages_per_seq], logical page ->       */
/* physical page; token position pos of sequence b lives in logical page     */
/* pos / P at slot pos % P.                                                  */
/* ------------------------------------------------------------------------ */

static int64_t tile_bytes(int d, int p) { return (int64_t)p * (d / 2) + 2 * (int64_t)p; }

/* Offsets inside one page of an INT4 pool: the code row and the scale of
 * (KV head h, slot). */
static int64_t code_offset(int d, int p, int h, int slot) { return ((int64_t)h * p + slot) * (d / 2); }
static int64_t scale_offset(int hkv, int d, int p, int h, int slot)
{
    return (int64_t)hkv * p * (d / 2) + ((int64_t)h * p + slot) * 2;
}

int64_t kvq_oracle_tile_bytes(int d, int p) { return tile_bytes(d, p); }

/* Locate (physical page, slot) of token position pos of sequence seq.
 * Returns -1 on any out-of-range index. */
static int64_t locate(const int32_t *page_table, int max_pages, int64_t num_pages,
                      int seq, int pos, int p, int *slot)
{
    if (pos < 0 || seq < 0) return -1;
    int lp = pos / p;
    if (lp >= max_pages) return -1;
    int64_t page = page_table[(int64_t)seq * max_pages + lp];
    if (page < 0 || page >= num_pages) return -1;
    *slot = pos % p;
    return page;
}

/* Quantize every new token's K and V and write them into their slots; no
 * other byte of either pool changes (past tokens are never revisited). */
int kvq_oracle_kv_quant_append(const uint16_t *k_new, const uint16_t *v_new,
                               const int32_t *token_seq, const int32_t *token_pos,
                               int32_t num_tokens, const int32_t *page_table,
                               int32_t max_pages_per_seq, uint8_t *k_pool,
                               uint8_t *v_pool, int64_t num_pages,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t had_block)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0) return ORACLE_BAD;
    int64_t tb = tile_bytes(head_dim, page_size);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int32_t t = 0; t < num_tokens; t++) {
        int slot = 0;
        int64_t page = locate(page_table, max_pages_per_seq, num_pages,
                              token_seq[t], token_pos[t], page_size, &slot);
        if (page < 0) { bad = 1; continue; }
        for (int h = 0; h < num_kv_heads; h++) {
            for (int which = 0; which < 2; which++) {
                const uint16_t *src = (which == 0 ? k_new : v_new) +
                                      ((int64_t)t * num_kv_heads + h) * head_dim;
                uint8_t *pg = (which == 0 ? k_pool : v_pool) + page * num_kv_heads * tb;
                uint16_t s16;
                if (kvq_oracle_quantize_vector(src, head_dim, had_block,
                                               pg + code_offset(head_dim, page_size, h, slot),
                                               &s16) != ORACLE_OK) {
                    bad = 1;
                    continue;
                }
                uint8_t *sp = pg + scale_offset(num_kv_heads, head_dim, page_size, h, slot);
                sp[0] = (uint8_t)(s16 & 0xFF);
                sp[1] = (uint8_t)(s16 >> 8);
            }
        }
    }
    return bad ? ORACLE_BAD : ORACLE_OK;
}

/* fp16 baseline append: copy each token's fp16 K/V into fp16 pools laid out
 * [page][head][slot][D]. */
int kvq_oracle_kv_append_fp16(const uint16_t *k_new, const uint16_t *v_new,
                              const int32_t *token_seq, const int32_t *token_pos,
                              int32_t num_tokens, const int32_t *page_table,
                              int32_t max_pages_per_seq, uint16_t *k_pool,
                              uint16_t *v_pool, int64_t num_pages,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size)
{
    int bad = 0;
    for (int32_t t = 0; t < num_tokens; t++) {
        int slot = 0;
        int64_t page = locate(page_table, max_pages_per_seq, num_pages,
                              token_seq[t], token_pos[t], page_size, &slot);
        if (page < 0) { bad = 1; continue; }
        for (int h = 0; h < num_kv_heads; h++) {
            int64_t src = ((int64_t)t * num_kv_heads + h) * head_dim;
            int64_t dst = ((page * num_kv_heads + h) * page_size + slot) * (int64_t)head_dim;
            memcpy(k_pool + dst, k_new + src, (size_t)head_dim * 2);
            memcpy(v_pool + dst, v_new + src, (size_t)head_dim * 2);
        }
    }
    return bad ? ORACLE_BAD : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the paged cache, fp64.                              */
/* Reading: query heads qh map to KV head qh / (Hq / Hkv); the caller's       */
/* softmax_scale multiplies the dot product; because R is orthogonal,         */
/* (R q).(R k) = q.k, so the query is rotated instead of un-rotating keys,    */
/* and the weighted sum of rotated values is rotated back at the end.        */
/* A context length <= 0 gives a zero output row.                             */
/* ------------------------------------------------------------------------ */

/* Element i of (KV head h, slot) of one page pg of an INT4 pool. */
static double dequant(const uint8_t *pg, int hkv, int h, int d, int p, int slot, int i)
{
    uint8_t byte = pg[code_offset(d, p, h, slot) + i / 2];
    int nib = (i & 1) ? (byte >> 4) : (byte & 0xF);
    int code = (nib & 8) ? nib - 16 : nib;
    const uint8_t *sp = pg + scale_offset(hkv, d, p, h, slot);
    uint16_t s16 = (uint16_t)(sp[0] | (sp[1] << 8));
    return (double)code * (double)kvq_oracle_f16_to_f32(s16);
}

/* Generic softmax attention for one (sequence, query head) over L keys
 * provided by a callback-free loop: k_at/v_at fill a D-vector for key j. */
static void attend_one(const double *qrot, int L, int d, double scale,
                       void (*fetch)(const void *ctx, int j, int which, double *out),
                       const void *ctx, double *out)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double kv[ORACLE_MAX_D];
    double M = -INFINITY;
    for (int j = 0; j < L; j++) {
        fetch(ctx, j, 0, kv);
        double dot = 0.0;
        for (int i = 0; i < d; i++) dot += qrot[i] * kv[i];
        z[j] = scale * dot;
        if (z[j] > M) M = z[j];
    }
    double wsum = 0.0;
    for (int i = 0; i < d; i++) out[i] = 0.0;
    for (int j = 0; j < L; j++) {
        double w = exp(z[j] - M);
        wsum += w;
        fetch(ctx, j, 1, kv);
        for (int i = 0; i < d; i++) out[i] += w * kv[i];
    }
    for (int i = 0; i < d; i++) out[i] = (L > 0) ? out[i] / wsum : 0.0;
    free(z);
}

typedef struct {
    const uint8_t *k_pool, *v_pool;
    const int32_t *page_table;
    int max_pages;
    int64_t num_pages;
    int seq, kvh, hkv, d, p;
    int fp16;               /* 1: fp16 pools, 0: INT4 pools */
} paged_ctx;

static void fetch_paged(const void *vctx, int j, int which, double *out)
{
    const paged_ctx *c = (const paged_ctx *)vctx;
    int slot = 0;
    int64_t page = locate(c->page_table, c->max_pages, c->num_pages, c->seq, j, c->p, &slot);
    if (c->fp16) {
        const uint16_t *pool = (const uint16_t *)(which == 0 ? c->k_pool : c->v_pool);
        const uint16_t *row = pool + ((page * c->hkv + c->kvh) * c->p + slot) * (int64_t)c->d;
        for (int i = 0; i < c->d; i++) out[i] = (double)kvq_oracle_f16_to_f32(row[i]);
    } else {
        const uint8_t *pool = which == 0 ? c->k_pool : c->v_pool;
        const uint8_t *pg = pool + page * c->hkv * tile_bytes(c->d, c->p);
        for (int i = 0; i < c->d; i++) out[i] = dequant(pg, c->hkv, c->kvh, c->d, c->p, slot, i);
    }
}

static int decode_common(const uint16_t *q, const void *k_pool, const void *v_pool,
                         int64_t num_pages, const int32_t *page_table,
                         int32_t max_pages_per_seq, const int32_t *context_lens,
                         int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t page_size, int32_t had_block,
                         float softmax_scale, float *out, int fp16)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        head_dim > ORACLE_MAX_D || page_size <= 0 || num_q_heads % num_kv_heads)
        return ORACLE_BAD;
    for (int b = 0; b < batch; b++) {
        int L = context_lens[b];
        if (L > (int64_t)max_pages_per_seq * page_size) return ORACLE_BAD;
        for (int lp = 0; lp < (L + page_size - 1) / page_size; lp++) {
            int32_t pg = page_table[(int64_t)b * max_pages_per_seq + lp];
            if (pg < 0 || pg >= num_pages) return ORACLE_BAD;
        }
    }
    int group = num_q_heads / num_kv_heads;
    int64_t units = (int64_t)batch * num_q_heads;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < units; u++) {
        int b = (int)(u / num_q_heads), qh = (int)(u % num_q_heads);
        double qrot[ORACLE_MAX_D], o[ORACLE_MAX_D];
        const uint16_t *qrow = q + ((int64_t)b * num_q_heads + qh) * head_dim;
        for (int i = 0; i < head_dim; i++) qrot[i] = (double)kvq_oracle_f16_to_f32(qrow[i]);
        if (!fp16) kvq_oracle_rotate_f64(qrot, head_dim, had_block);
        paged_ctx c = { (const uint8_t *)k_pool, (const uint8_t *)v_pool, page_table,
                        max_pages_per_seq, num_pages, b, qh / group, num_kv_heads,
                        head_dim, page_size, fp16 };
        int L = context_lens[b];
        attend_one(qrot, L, head_dim, (double)softmax_scale, fetch_paged, &c, o);
        if (!fp16 && L > 0) kvq_oracle_rotate_f64(o, head_dim, had_block);
        float *orow = out + ((int64_t)b * num_q_heads + qh) * head_dim;
        for (int i = 0; i < head_dim; i++) orow[i] = (float)o[i];
    }
    return ORACLE_OK;
}

int kvq_oracle_paged_decode_attn_int4(const uint16_t *q, const uint8_t *k_pool,
                                      const uint8_t *v_pool, int64_t num_pages,
                                      const int32_t *page_table, int32_t max_pages_per_seq,
                                      const int32_t *context_lens, int32_t batch,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size,
                                      int32_t had_block, float softmax_scale, float *out)
{
    return decode_common(q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq,
                         context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                         page_size, had_block, softmax_scale, out, 0);
}

int kvq_oracle_paged_decode_attn_fp16(const uint16_t *q, const uint16_t *k_pool,
                                      const uint16_t *v_pool, int64_t num_pages,
                                      const int32_t *page_table, int32_t max_pages_per_seq,
                                      const int32_t *context_lens, int32_t batch,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size,
                                      float softmax_scale, float *out)
{
    return decode_common(q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq,
                         context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                         page_size, 0, softmax_scale, out, 1);
}

/* Dense reference: softmax(q . K^T * scale) . V for one sequence, fp64, with
 * no paging, no rotation and no quantization.  q [Hq][D], K and V [L][Hkv][D]. */
typedef struct { const double *k, *v; int hkv, kvh, d; } dense_ctx;

static void fetch_dense(const void *vctx, int j, int which, double *out)
{
    const dense_ctx *c = (const dense_ctx *)vctx;
    const double *src = (which == 0 ? c->k : c->v) + ((int64_t)j * c->hkv + c->kvh) * c->d;
    for (int i = 0; i < c->d; i++) out[i] = src[i];
}

int kvq_oracle_dense_decode_f64(const double *q, const double *k, const double *v,
                                int32_t L, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, double softmax_scale, double *out)
{
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        head_dim <= 0 || head_dim > ORACLE_MAX_D)
        return ORACLE_BAD;
    int group = num_q_heads / num_kv_heads;
    for (int qh = 0; qh < num_q_heads; qh++) {
        dense_ctx c = { k, v, num_kv_heads, qh / group, head_dim };
        attend_one(q + (int64_t)qh * head_dim, L, head_dim, softmax_scale, fetch_dense, &c,
                   out + (int64_t)qh * head_dim);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Quantizer variants on the same paged cache and the same attention.       */
/*                                                                           */
/* Sources: "BitDecoding-FP4:FP4 KVキャッシュのネイティブ復号", section      */
/* 深掘り分析 (Outlier-Aware Key Quantization: with one scale per token, a   */
/* single outlier widens the range of the whole token; smoothing and a      */
/* Hadamard rotation spread outliers, and a scale search picks a suitable    */
/* scale per group) and its opening summary (4-bit microscaling KV formats,  */
/* NVFP4 and MXFP4); "KVキャッシュを4ビットへ — SAW-INT4...", section         */
/* 回転のトリック (block-diagonal Hadamard, in the QuaRot / SpinQuant line of */
/* rotations, whose randomized form multiplies by a random +-1 diagonal      */
/* first).                                                                   */
/*                                                                           */
/* Readings (the pages fix no arithmetic for these):                        */
/*  - scale groups: contiguous groups of scale_group channels of the         */
/*    (rotated) head vector, one scale each; scale_group = had_block gives   */
/*    one scale per Hadamard block; 128 is the method's token-wise scale;    */
/*  - scale search (INT4): candidate scales s_k = fp16(fp32(m a_k) / 7)      */
/*    for the clipping ratios a_k = (16 - k) / 16, k = 0..7, m the group's  */
/*    absmax; each candidate's codes are those of the plain quantizer with  */
/*    s_k, its error is the sum over the group of D_i^2, where D_i is the    */
/*    residual y_i - s_k c_i (exact in fp32 for these ratios) in units of   */
/*    2^(E-12), E the exponent with m < 2^E, rounded to an integer (ties to  */
/*    even): an exact integer, so the choice does not depend on the order of */
/*    the sum; the smallest error wins, ties to the larger ratio;            */
/*  - randomized Hadamard: x -> R (S x) with S = diag(+-1) given as a        */
/*    128-bit mask (bit i set: channel i negated); keys and values are       */
/*    written with R S, the query is rotated with R S as well, and the       */
/*    output is brought back with S R (the inverse of R S);                  */
/*  - MXFP4: groups of 32, OCP microscaling layout: E2M1 elements            */
/*    {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit, and one E8M0 shared      */
/*    scale 2^X per group with X = floor(log2 m) - 2 (m = the group's        */
/*    absmax; 2 is the exponent of E2M1's largest normal value); an element */
/*    becomes the E2M1 value nearest y / 2^X (ties to the code whose         */
/*    mantissa bit is 0; beyond 6 it saturates to 6); the sign bit is set   */
/*    iff y < 0, so a zero (of either sign) is stored as +0 and the stored   */
/*    byte does not depend on how a zero was reached; a group of zeros gets  */
/*    X = -127 (byte 0) and zero codes.                                      */
/* Scales of a page follow its code rows: for (KV head h, slot, group g) at  */
/* Hkv * P * D/2 + ((h * P + slot) * (D / G) + g) * scale_bytes, with       */
/* scale_bytes 2 (fp16) for INT4 and 1 (E8M0) for MXFP4.                     */
/* ------------------------------------------------------------------------ */

#define ORACLE_FMT_INT4 0
#define ORACLE_FMT_MXFP4 1

typedef struct {
    int32_t format;
    int32_t had_block;
    int32_t scale_group;
    int32_t scale_search;
    uint32_t sign_mask[4];
} kvq_oracle_qcfg;

static int cfg_ok(const kvq_oracle_qcfg *c, int d)
{
    if (!c || d <= 0 || d > ORACLE_MAX_D || (d & 1) || d > 128) return 0;
    int bh = c->had_block;
    if (bh < 0 || (bh > 0 && (bh > d || (bh & (bh - 1)) || d % bh))) return 0;
    int g = c->scale_group;
    if (g <= 0 || d % g) return 0;
    if (c->format == ORACLE_FMT_INT4) return c->scale_search == 0 || c->scale_search == 1;
    if (c->format == ORACLE_FMT_MXFP4) return g == 32 && c->scale_search == 0;
    return 0;
}

static int scale_bytes_of(const kvq_oracle_qcfg *c) { return c->format == ORACLE_FMT_MXFP4 ? 1 : 2; }

static int sign_of(const kvq_oracle_qcfg *c, int i) { return (c->sign_mask[i >> 5] >> (i & 31)) & 1u; }

int64_t kvq_oracle_tile_bytes_cfg(int d, int p, const kvq_oracle_qcfg *c)
{
    if (!cfg_ok(c, d) || p <= 0) return -1;
    return (int64_t)p * (d / 2) + (int64_t)p * (d / c->scale_group) * scale_bytes_of(c);
}

/* y = R (S x) in fp32: widen, negate the masked channels (exact), then the
 * block FWHT and the 1/sqrt(Bh) factor exactly as the plain quantizer does. */
static void rotate_fwd_cfg_f32(const uint16_t *x, int d, const kvq_oracle_qcfg *c, float *y)
{
    for (int i = 0; i < d; i++) {
        y[i] = kvq_oracle_f16_to_f32(x[i]);
        if (sign_of(c, i)) y[i] = -y[i];
    }
    if (c->had_block > 1) {
        kvq_oracle_fwht_f32(y, d, c->had_block);
        float cb = kvq_oracle_hadamard_scale(c->had_block);
        for (int i = 0; i < d; i++) y[i] = y[i] * cb;
    }
}

/* INT4 codes of one group for a given fp16 scale (as the plain quantizer). */
static void int4_codes(const float *y, int n, float s, int *codes)
{
    for (int i = 0; i < n; i++) {
        int code = 0;
        if (s != 0.0f) {
            code = (int)rintf(y[i] / s);
            if (code < -8) code = -8;
            if (code > 7) code = 7;
        }
        codes[i] = code;
    }
}

/* One INT4 group: codes and the fp16 scale bits. */
static void int4_group(const float *y, int n, int search, int *codes, uint16_t *s16_out)
{
    float m = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(y[i]);
        if (a > m) m = a;
    }
    if (!search) {
        uint16_t s16 = kvq_oracle_f32_to_f16(m / 7.0f);
        int4_codes(y, n, kvq_oracle_f16_to_f32(s16), codes);
        *s16_out = s16;
        return;
    }
    int E = 0;
    if (m > 0.0f) (void)frexpf(m, &E);           /* m = f 2^E, f in [0.5, 1): m < 2^E */
    int64_t best_err = -1;
    int cand[ORACLE_MAX_D];
    for (int k = 0; k < 8; k++) {
        float a = (float)(16 - k) / 16.0f;
        uint16_t s16 = kvq_oracle_f32_to_f16((m * a) / 7.0f);
        float s = kvq_oracle_f16_to_f32(s16);
        int4_codes(y, n, s, cand);
        int64_t err = 0;
        for (int i = 0; i < n; i++) {
            float r = y[i] - s * (float)cand[i];
            double D = rint(ldexp((double)r, 12 - E));
            err += (int64_t)D * (int64_t)D;
        }
        if (best_err < 0 || err < best_err) {
            best_err = err;
            *s16_out = s16;
            for (int i = 0; i < n; i++) codes[i] = cand[i];
        }
    }
}

/* E2M1 magnitudes by code 0..7, and the nearest code to a >= 0 (ties to the
 * even code, whose mantissa bit is 0; saturates at 6). */
static const float e2m1_grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static int e2m1_nearest(float a)
{
    int best = 0;
    float bd = fabsf(a - e2m1_grid[0]);
    for (int k = 1; k < 8; k++) {
        float dk = fabsf(a - e2m1_grid[k]);
        if (dk < bd || (dk == bd && (k & 1) == 0)) { best = k; bd = dk; }
    }
    return best;
}

float kvq_oracle_e2m1_value(int code)
{
    float v = e2m1_grid[code & 7];
    return (code & 8) ? -v : v;
}

/* One MXFP4 group: 4-bit codes (sign in bit 3) and the E8M0 byte. */
static void mxfp4_group(const float *y, int n, int *codes, uint8_t *e8m0_out)
{
    float m = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(y[i]);
        if (a > m) m = a;
    }
    if (m == 0.0f) {
        for (int i = 0; i < n; i++) codes[i] = 0;
        *e8m0_out = 0;
        return;
    }
    int E = 0;
    (void)frexpf(m, &E);          /* floor(log2 m) = E - 1 */
    int X = E - 1 - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    for (int i = 0; i < n; i++) {
        float v = ldexpf(y[i], -X);
        codes[i] = (y[i] < 0.0f ? 8 : 0) | e2m1_nearest(fabsf(v));
    }
    *e8m0_out = (uint8_t)(X + 127);
}

/* One (token, KV head, K-or-V) vector under a variant: D/2 packed code bytes
 * and D / scale_group scales (fp16 little-endian or E8M0 bytes). */
int kvq_oracle_quantize_vector_cfg(const uint16_t *x, int d, const kvq_oracle_qcfg *c,
                                   uint8_t *codes_out, uint8_t *scales_out)
{
    if (!cfg_ok(c, d)) return ORACLE_BAD;
    float y[ORACLE_MAX_D];
    int codes[ORACLE_MAX_D];
    rotate_fwd_cfg_f32(x, d, c, y);
    int G = c->scale_group;
    for (int g = 0; g < d / G; g++) {
        if (c->format == ORACLE_FMT_INT4) {
            uint16_t s16 = 0;
            int4_group(y + g * G, G, c->scale_search, codes + g * G, &s16);
            scales_out[2 * g] = (uint8_t)(s16 & 0xFF);
            scales_out[2 * g + 1] = (uint8_t)(s16 >> 8);
        } else {
            mxfp4_group(y + g * G, G, codes + g * G, scales_out + g);
        }
    }
    for (int j = 0; j < d / 2; j++)
        codes_out[j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
    return ORACLE_OK;
}

/* Element i of a stored vector (still in the rotated basis). */
static double dequant_cfg(const uint8_t *codes, const uint8_t *scales, int d, const kvq_oracle_qcfg *c, int i)
{
    uint8_t byte = codes[i / 2];
    int nib = (i & 1) ? (byte >> 4) : (byte & 0xF);
    int g = i / c->scale_group;
    if (c->format == ORACLE_FMT_INT4) {
        int code = (nib & 8) ? nib - 16 : nib;
        uint16_t s16 = (uint16_t)(scales[2 * g] | (scales[2 * g + 1] << 8));
        return (double)code * (double)kvq_oracle_f16_to_f32(s16);
    }
    (void)d;
    return (double)kvq_oracle_e2m1_value(nib) * ldexp(1.0, (int)scales[g] - 127);
}

/* Reconstruction of x in the original basis (S R applied to the dequantized
 * vector, fp64): for accuracy reports. */
int kvq_oracle_reconstruct_cfg(const uint16_t *x, int d, const kvq_oracle_qcfg *c, double *out)
{
    uint8_t codes[ORACLE_MAX_D / 2], scales[ORACLE_MAX_D * 2];
    if (kvq_oracle_quantize_vector_cfg(x, d, c, codes, scales) != ORACLE_OK) return ORACLE_BAD;
    for (int i = 0; i < d; i++) out[i] = dequant_cfg(codes, scales, d, c, i);
    kvq_oracle_rotate_f64(out, d, c->had_block);
    for (int i = 0; i < d; i++)
        if (sign_of(c, i)) out[i] = -out[i];
    return ORACLE_OK;
}

static int64_t scale_offset_cfg(int hkv, int d, int p, int h, int slot, const kvq_oracle_qcfg *c)
{
    int ng = d / c->scale_group;
    return (int64_t)hkv * p * (d / 2) + ((int64_t)h * p + slot) * ng * scale_bytes_of(c);
}

int kvq_oracle_kv_quant_append_cfg(const uint16_t *k_new, const uint16_t *v_new,
                                   const int32_t *token_seq, const int32_t *token_pos,
                                   int32_t num_tokens, const int32_t *page_table,
                                   int32_t max_pages_per_seq, uint8_t *k_pool,
                                   uint8_t *v_pool, int64_t num_pages,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t page_size, const kvq_oracle_qcfg *c)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || page_size <= 0 || !cfg_ok(c, head_dim)) return ORACLE_BAD;
    int64_t tb = kvq_oracle_tile_bytes_cfg(head_dim, page_size, c);
    int sbytes = scale_bytes_of(c) * (head_dim / c->scale_group);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int32_t t = 0; t < num_tokens; t++) {
        int slot = 0;
        int64_t page = locate(page_table, max_pages_per_seq, num_pages,
                              token_seq[t], token_pos[t], page_size, &slot);
        if (page < 0) { bad = 1; continue; }
        for (int h = 0; h < num_kv_heads; h++) {
            for (int which = 0; which < 2; which++) {
                const uint16_t *src = (which == 0 ? k_new : v_new) +
                                      ((int64_t)t * num_kv_heads + h) * head_dim;
                uint8_t *pg = (which == 0 ? k_pool : v_pool) + page * num_kv_heads * tb;
                uint8_t sc[ORACLE_MAX_D * 2];
                if (kvq_oracle_quantize_vector_cfg(src, head_dim, c,
                                                   pg + code_offset(head_dim, page_size, h, slot),
                                                   sc) != ORACLE_OK) {
                    bad = 1;
                    continue;
                }
                memcpy(pg + scale_offset_cfg(num_kv_heads, head_dim, page_size, h, slot, c), sc,
                       (size_t)sbytes);
            }
        }
    }
    return bad ? ORACLE_BAD : ORACLE_OK;
}

typedef struct {
    const uint8_t *k_pool, *v_pool;
    const int32_t *page_table;
    int max_pages;
    int64_t num_pages;
    int seq, kvh, hkv, d, p;
    const kvq_oracle_qcfg *c;
} paged_cfg_ctx;

static void fetch_paged_cfg(const void *vctx, int j, int which, double *out)
{
    const paged_cfg_ctx *x = (const paged_cfg_ctx *)vctx;
    int slot = 0;
    int64_t page = locate(x->page_table, x->max_pages, x->num_pages, x->seq, j, x->p, &slot);
    const uint8_t *pool = which == 0 ? x->k_pool : x->v_pool;
    const uint8_t *pg = pool + page * x->hkv * kvq_oracle_tile_bytes_cfg(x->d, x->p, x->c);
    const uint8_t *codes = pg + code_offset(x->d, x->p, x->kvh, slot);
    const uint8_t *scales = pg + scale_offset_cfg(x->hkv, x->d, x->p, x->kvh, slot, x->c);
    for (int i = 0; i < x->d; i++) out[i] = dequant_cfg(codes, scales, x->d, x->c, i);
}

/* Decode attention over a variant's cache, fp64: q' = R (S q); softmax over
 * the dequantized (rotated) keys; o = S R (sum w v').  L <= 0: zero row. */
int kvq_oracle_paged_decode_attn_cfg(const uint16_t *q, const uint8_t *k_pool,
                                     const uint8_t *v_pool, int64_t num_pages,
                                     const int32_t *page_table, int32_t max_pages_per_seq,
                                     const int32_t *context_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size,
                                     const kvq_oracle_qcfg *c, float softmax_scale, float *out)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || page_size <= 0 ||
        num_q_heads % num_kv_heads || !cfg_ok(c, head_dim))
        return ORACLE_BAD;
    for (int b = 0; b < batch; b++) {
        int L = context_lens[b];
        if (L > (int64_t)max_pages_per_seq * page_size) return ORACLE_BAD;
        for (int lp = 0; lp < (L + page_size - 1) / page_size; lp++) {
            int32_t pg = page_table[(int64_t)b * max_pages_per_seq + lp];
            if (pg < 0 || pg >= num_pages) return ORACLE_BAD;
        }
    }
    int group = num_q_heads / num_kv_heads;
    int64_t units = (int64_t)batch * num_q_heads;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < units; u++) {
        int b = (int)(u / num_q_heads), qh = (int)(u % num_q_heads);
        double qrot[ORACLE_MAX_D], o[ORACLE_MAX_D];
        const uint16_t *qrow = q + ((int64_t)b * num_q_heads + qh) * head_dim;
        for (int i = 0; i < head_dim; i++) {
            qrot[i] = (double)kvq_oracle_f16_to_f32(qrow[i]);
            if (sign_of(c, i)) qrot[i] = -qrot[i];
        }
        kvq_oracle_rotate_f64(qrot, head_dim, c->had_block);
        paged_cfg_ctx x = { k_pool, v_pool, page_table, max_pages_per_seq, num_pages, b, qh / group,
                            num_kv_heads, head_dim, page_size, c };
        int L = context_lens[b];
        attend_one(qrot, L, head_dim, (double)softmax_scale, fetch_paged_cfg, &x, o);
        if (L > 0) {
            kvq_oracle_rotate_f64(o, head_dim, c->had_block);
            for (int i = 0; i < head_dim; i++)
                if (sign_of(c, i)) o[i] = -o[i];
        }
        float *orow = out + ((int64_t)b * num_q_heads + qh) * head_dim;
        for (int i = 0; i < head_dim; i++) orow[i] = (float)o[i];
    }
    return ORACLE_OK;
}

int kvq_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the next parallel regions (timing only: every unit is computed
 * sequentially, so results do not depend on it). */
void kvq_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
