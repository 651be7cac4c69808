/*
 * pkv_oracle.c - plain, slow CPU oracle for the paged int8 ("C8") KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library; the two agree only because both
 * implement the same definitions, stated below.
 *
 * Sources (web pages; sections named as printed on them):
 *  [P1] "Mojo Opset" README (XPU-Forces/mojo_opset), "Op List" table:
 *       MojoStorePagedKVCache, MojoPagedDecodeGQA, MojoDequant, MojoDynamicQuant.
 *  [P2] PR #379 "feat: [MLU] add mlu experimental ops; fix post norm bug",
 *       its code-review summary and the four review passes (Must fix /
 *       Suggestions / Notes) on MojoStorePagedKVCacheC8 and
 *       MojoDequantFromPagedKVCache.
 *
 * Definitions implemented (each function repeats the one it follows):
 *  - store, per-token mode: dynamic symmetric int8 quantization (the
 *    MojoDynamicQuant row of [P1]) with scale = absmax/127 per token and KV
 *    head, q = clamp(round_half_even(x/scale), -128, 127) ([P2] pass 2 and
 *    pass 3 Notes give round(x/scale).clamp(-128,127); torch.round rounds half
 *    to even), the division done in fp32 ([P2] pass 4, Must fix: cast to
 *    float32 before dividing).
 *  - store, per-block mode: one fp32 scale per (block, KV head) ([P2] passes
 *    1 and 2 name a per-block scale layout for quant_mode != 0).
 *  - store, per-channel mode: static fp32 scales, one per (KV head, channel),
 *    given by the caller and broadcast over the tokens ([P2] pass 1 Notes: the
 *    dequant forward handles the per-channel layout scale[..., None, :]; pass 2
 *    Nits: the store's docstring names a per-channel quantization).  The store
 *    only writes codes, q = clamp(round_half_even(fl32(x / s_c)), -128, 127),
 *    which saturates where |x| exceeds the calibrated range.
 *  - dequant: fp32 product of the int8 code and its scale, then bf16 ([P2]
 *    pass 1 and 4 Must fix: the multiply must run in fp32); rows written at a
 *    per-sequence offset that defaults to the exclusive prefix sum of the
 *    context lengths ([P2] pass 1 Must fix on context_seq_offset).
 *  - decode: grouped-query attention of one new query per sequence over the
 *    paged cache ([P1] MojoPagedDecodeGQA), generalised to a causal chunk of
 *    q_len new queries, accumulated in fp64 over the dequantized values.
 *  - paged MLA store and decode ([P1] MojoStorePagedMLAKVCache,
 *    MojoPagedDecodeMLA): latent attention over a per-token int8 latent row
 *    and rotary-key row shared by all heads (the reading is stated at the MLA
 *    section below).
 *
 * Cache layout (the boundary contract; element (block, head, slot, channel)):
 *   K  [NB][Hkv][BS][D]   int8, or bf16 in mode 2
 *   V  [NB][Hkv][BS/16][D][16]   int8, or bf16 in mode 2 (the page in 16-slot tiles, each
 *                                 channel-major: 16 consecutive slots of one channel adjacent;
 *                                 a block size that is not a multiple of 16 makes one tile of
 *                                 BS slots, [NB][Hkv][D][BS])
 *   scales mode 0: [NB][Hkv][BS] fp32;  mode 1: [NB][Hkv] fp32;  mode 2: none;
 *          mode 3: [Hkv][D] fp32 (inputs, never written)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MODE_PER_TOKEN 0
#define MODE_PER_BLOCK 1
#define MODE_BF16 2
#define MODE_PER_CHANNEL 3

/* ------------------------------------------------------------------------- */
/* bf16 <-> floating point                                                    */
/* ------------------------------------------------------------------------- */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the upper half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest bf16 to x, ties to the even significand.  Written from the
 * definition: find the bf16 grid spacing at x, take the two neighbours on the
 * grid and keep the nearer one.  Every step is exact in double. */
uint16_t oracle_bf16_round(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);              /* a in [2^(e-1), 2^e) */
    int E = e - 1;             /* unbiased exponent of a */
    if (E < -126)
        E = -126;              /* subnormals share the smallest normal spacing */
    double spacing = ldexp(1.0, E - 7); /* 8 significant bits */
    double n = a / spacing;    /* exact: power-of-two division */
    double lo = floor(n);
    double rem = n - lo;
    double k = lo;
    if (rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) != 0.0))
        k = lo + 1.0;
    double r = k * spacing;
    const double max_bf16 = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
    if (r > max_bf16)
        return sign | 0x7f80;   /* rounds beyond the largest finite: infinity */
    float rf = (float)r;        /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------- */
/* layout helpers                                                             */
/* ------------------------------------------------------------------------- */

typedef struct {
    int mode, nb, hkv, bs, d;
    void *k, *v;
    float *ks, *vs;
} cache_t;

static int64_t k_index(const cache_t *c, int64_t blk, int h, int slot, int ch)
{
    return ((blk * c->hkv + h) * c->bs + slot) * (int64_t)c->d + ch;
}

static int64_t v_index(const cache_t *c, int64_t blk, int h, int slot, int ch)
{
    int64_t page = (blk * c->hkv + h) * (int64_t)c->bs * c->d;
    int t = c->bs % 16 == 0 ? 16 : c->bs; /* slots per tile */
    return page + ((int64_t)(slot / t) * c->d + ch) * t + slot % t;
}

static int64_t tok_scale_index(const cache_t *c, int64_t blk, int h, int slot)
{
    return (blk * c->hkv + h) * c->bs + slot;
}

static int64_t blk_scale_index(const cache_t *c, int64_t blk, int h)
{
    return blk * c->hkv + h;
}

static int64_t ch_scale_index(const cache_t *c, int h, int ch)
{
    return (int64_t)h * c->d + ch;
}

/* the scale of cache element (blk, h, slot, ch) in the int8 modes */
static float scale_of(const cache_t *c, int is_v, int64_t blk, int h, int slot, int ch)
{
    const float *sc = is_v ? c->vs : c->ks;
    if (c->mode == MODE_PER_TOKEN)
        return sc[tok_scale_index(c, blk, h, slot)];
    if (c->mode == MODE_PER_BLOCK)
        return sc[blk_scale_index(c, blk, h)];
    return sc[ch_scale_index(c, h, ch)];
}

/* ------------------------------------------------------------------------- */
/* quantization primitives                                                    */
/* ------------------------------------------------------------------------- */

/* q = clamp(round_half_even(fl32(x / s)), -128, 127); q = 0 when s == 0. */
static int8_t quant_one(float x, float s)
{
    if (s == 0.0f)
        return 0;
    float r = nearbyintf(x / s); /* default rounding mode: to nearest, ties even */
    if (r > 127.0f)
        r = 127.0f;
    if (r < -128.0f)
        r = -128.0f;
    return (int8_t)r;
}

/* fl32(absmax / 127) */
static float absmax_scale(float absmax)
{
    return absmax / 127.0f;
}

/* ------------------------------------------------------------------------- */
/* store                                                                      */
/* ------------------------------------------------------------------------- */

/* Per-token (mode 0), bf16 (mode 2) and per-channel (mode 3) store of one
 * token of one KV head into (blk, slot). x points at D bf16 values. */
static void store_token(cache_t *c, int is_v, int64_t blk, int h, int slot, const uint16_t *x)
{
    if (c->mode == MODE_BF16) {
        uint16_t *dst = (uint16_t *)(is_v ? c->v : c->k);
        for (int ch = 0; ch < c->d; ch++)
            dst[is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch)] = x[ch];
        return;
    }
    if (c->mode == MODE_PER_CHANNEL) {
        const float *sc = is_v ? c->vs : c->ks;
        int8_t *dst = (int8_t *)(is_v ? c->v : c->k);
        for (int ch = 0; ch < c->d; ch++)
            dst[is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch)] =
                quant_one(bf16_to_float(x[ch]), sc[ch_scale_index(c, h, ch)]);
        return;
    }
    float absmax = 0.0f;
    for (int ch = 0; ch < c->d; ch++) {
        float a = fabsf(bf16_to_float(x[ch]));
        if (a > absmax)
            absmax = a;
    }
    float s = absmax_scale(absmax);
    int8_t *dst = (int8_t *)(is_v ? c->v : c->k);
    for (int ch = 0; ch < c->d; ch++)
        dst[is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch)] =
            quant_one(bf16_to_float(x[ch]), s);
    (is_v ? c->vs : c->ks)[tok_scale_index(c, blk, h, slot)] = s;
}

/* Per-block (mode 1) store of the new tokens of sequence b that fall in its
 * logical block j, for KV head h.  Positions [lo, hi) are new; positions
 * [j*BS, lo) already hold codes under the block's current scale s_old.
 *   s = max(s_old, fl32(absmax_new / 127))
 *   if s > s_old: every old code is re-quantized, q <- quant(fl32(q * s_old), s)
 *   new codes:    q = quant(x, s)
 * x_first points at the bf16 row [Hkv][D] of the token at position lo. */
static void store_block(cache_t *c, int is_v, int64_t blk, int h, int j, int lo, int hi,
                        const uint16_t *x_first, int64_t row_stride)
{
    int8_t *dst = (int8_t *)(is_v ? c->v : c->k);
    float *sc = is_v ? c->vs : c->ks;
    int n_old = lo - j * c->bs;
    float s_old = n_old > 0 ? sc[blk_scale_index(c, blk, h)] : 0.0f;
    float absmax = 0.0f;
    for (int p = lo; p < hi; p++) {
        const uint16_t *x = x_first + (int64_t)(p - lo) * row_stride + (int64_t)h * c->d;
        for (int ch = 0; ch < c->d; ch++) {
            float a = fabsf(bf16_to_float(x[ch]));
            if (a > absmax)
                absmax = a;
        }
    }
    float s_new = absmax_scale(absmax);
    float s = s_new > s_old ? s_new : s_old;
    if (n_old > 0 && s > s_old) {
        for (int slot = 0; slot < n_old; slot++)
            for (int ch = 0; ch < c->d; ch++) {
                int64_t i = is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch);
                float old_value = (float)dst[i] * s_old; /* fl32 */
                dst[i] = quant_one(old_value, s);
            }
    }
    for (int p = lo; p < hi; p++) {
        int slot = p - j * c->bs;
        const uint16_t *x = x_first + (int64_t)(p - lo) * row_stride + (int64_t)h * c->d;
        for (int ch = 0; ch < c->d; ch++) {
            int64_t i = is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch);
            dst[i] = quant_one(bf16_to_float(x[ch]), s);
        }
    }
    sc[blk_scale_index(c, blk, h)] = s;
}

/*
 * Store T new tokens (k_new, v_new: bf16 [T][Hkv][D]).
 *
 * Slot of token t:
 *  - slot_mapping != NULL: slot = slot_mapping[t]; block = slot / BS,
 *    offset = slot % BS; a negative slot means "skip" (padding token).
 *  - otherwise token i of sequence b is t = cu_q_lens[b] + i (cu_q_lens NULL:
 *    one token per sequence, t = b); its position is
 *    p = context_lengths[b] - q_len_b + i, its block
 *    block_table[b][p / BS] and its offset p % BS.
 * Mode 1 requires the block-table form.
 * Returns 0, or -1 on an argument it cannot serve.
 */
int oracle_store(int mode, int nb, int hkv, int bs, int d, void *k_cache, void *v_cache,
                 float *k_scale, float *v_scale, const uint16_t *k_new, const uint16_t *v_new,
                 int num_tokens, const int64_t *slot_mapping, const int32_t *cu_q_lens,
                 const int32_t *context_lengths, const int32_t *block_table, int batch, int mbs)
{
    cache_t c = {mode, nb, hkv, bs, d, k_cache, v_cache, k_scale, v_scale};
    const int64_t row = (int64_t)hkv * d;
    if (mode < 0 || mode > 3 || bs <= 0 || d <= 0 || hkv <= 0)
        return -1;
    if (slot_mapping) {
        if (mode == MODE_PER_BLOCK)
            return -1;
        for (int t = 0; t < num_tokens; t++) {
            int64_t slot = slot_mapping[t];
            if (slot < 0)
                continue;
            if (slot / bs >= nb)
                return -1;
            for (int h = 0; h < hkv; h++) {
                store_token(&c, 0, slot / bs, h, (int)(slot % bs), k_new + t * row + (int64_t)h * d);
                store_token(&c, 1, slot / bs, h, (int)(slot % bs), v_new + t * row + (int64_t)h * d);
            }
        }
        return 0;
    }
    if (!context_lengths || !block_table)
        return -1;
    for (int b = 0; b < batch; b++) {
        int qlen = cu_q_lens ? cu_q_lens[b + 1] - cu_q_lens[b] : 1;
        int t0 = cu_q_lens ? cu_q_lens[b] : b;
        int ctx = context_lengths[b];
        int prior = ctx - qlen;
        if (qlen <= 0)
            continue;
        if (mode != MODE_PER_BLOCK) {
            for (int i = 0; i < qlen; i++) {
                int p = prior + i;
                if (p < 0)
                    continue; /* inactive decode slot (context length 0): nothing to store */
                if (p / bs >= mbs)
                    return -1;
                int64_t blk = block_table[(int64_t)b * mbs + p / bs];
                if (blk < 0 || blk >= nb)
                    return -1;
                for (int h = 0; h < hkv; h++) {
                    store_token(&c, 0, blk, h, p % bs, k_new + (int64_t)(t0 + i) * row + (int64_t)h * d);
                    store_token(&c, 1, blk, h, p % bs, v_new + (int64_t)(t0 + i) * row + (int64_t)h * d);
                }
            }
        } else {
            if (prior < 0)
                continue; /* inactive decode slot */
            for (int j = prior / bs; j * bs < ctx; j++) {
                int lo = prior > j * bs ? prior : j * bs;
                int hi = ctx < (j + 1) * bs ? ctx : (j + 1) * bs;
                if (j >= mbs)
                    return -1;
                int64_t blk = block_table[(int64_t)b * mbs + j];
                if (blk < 0 || blk >= nb)
                    return -1;
                int64_t t_lo = t0 + (lo - prior);
                for (int h = 0; h < hkv; h++) {
                    store_block(&c, 0, blk, h, j, lo, hi, k_new + t_lo * row, row);
                    store_block(&c, 1, blk, h, j, lo, hi, v_new + t_lo * row, row);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* dequant                                                                    */
/* ------------------------------------------------------------------------- */

/* Dequantized value of cache element (blk, h, slot, ch) as an fp32:
 * fl32(float(q) * s); mode 2 returns the stored bf16 value. */
static float deq_f32(const cache_t *c, int is_v, int64_t blk, int h, int slot, int ch)
{
    int64_t i = is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch);
    if (c->mode == MODE_BF16)
        return bf16_to_float(((const uint16_t *)(is_v ? c->v : c->k))[i]);
    float s = scale_of(c, is_v, blk, h, slot, ch);
    return (float)((const int8_t *)(is_v ? c->v : c->k))[i] * s;
}

/* Exact dequantized value in fp64: double(q) * double(s) (no rounding). */
static double deq_f64(const cache_t *c, int is_v, int64_t blk, int h, int slot, int ch)
{
    int64_t i = is_v ? v_index(c, blk, h, slot, ch) : k_index(c, blk, h, slot, ch);
    if (c->mode == MODE_BF16)
        return (double)bf16_to_float(((const uint16_t *)(is_v ? c->v : c->k))[i]);
    float s = scale_of(c, is_v, blk, h, slot, ch);
    return (double)((const int8_t *)(is_v ? c->v : c->k))[i] * (double)s;
}

/*
 * Gather every sequence's cache back to bf16.
 * out[(off_b + p) * token_stride + h * head_stride + ch] = bf16(fl32(q * s))
 * for p < context_lengths[b]; off_b = seq_offsets[b], or the exclusive prefix
 * sum of context_lengths when seq_offsets is NULL.  Other rows untouched.
 */
int oracle_dequant(int mode, int nb, int hkv, int bs, int d, const void *k_cache,
                   const void *v_cache, const float *k_scale, const float *v_scale,
                   const int32_t *block_table, int mbs, const int32_t *context_lengths,
                   const int64_t *seq_offsets, int batch, uint16_t *k_out, uint16_t *v_out,
                   int64_t token_stride, int64_t head_stride)
{
    cache_t c = {mode, nb, hkv, bs, d, (void *)k_cache, (void *)v_cache, (float *)k_scale,
                 (float *)v_scale};
    int64_t off = 0;
    for (int b = 0; b < batch; b++) {
        int64_t base = seq_offsets ? seq_offsets[b] : off;
        if (context_lengths[b] > mbs * bs)
            return -1;
        for (int p = 0; p < context_lengths[b]; p++) {
            int64_t blk = block_table[(int64_t)b * mbs + p / bs];
            if (blk < 0 || blk >= nb)
                return -1;
            for (int h = 0; h < hkv; h++)
                for (int ch = 0; ch < d; ch++) {
                    int64_t o = (base + p) * token_stride + h * head_stride + ch;
                    if (k_out)
                        k_out[o] = oracle_bf16_round(deq_f32(&c, 0, blk, h, p % bs, ch));
                    if (v_out)
                        v_out[o] = oracle_bf16_round(deq_f32(&c, 1, blk, h, p % bs, ch));
                }
        }
        off += context_lengths[b];
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* decode attention                                                           */
/* ------------------------------------------------------------------------- */

typedef struct {
    cache_t c;
    const uint16_t *q;
    int hq;
    const int32_t *block_table;
    int mbs;
    const int32_t *context_lengths;
    const int32_t *cu_q_lens;
    int batch;
    double scale;
    int window; /* > 0: a query sees only its last `window` keys (itself included) */
    uint16_t *out;
    double *out_f64;
    double *lse;
    int next_item; /* shared work counter, guarded by mu */
    pthread_mutex_t mu;
} decode_job;

/*
 * One (sequence b, KV head h) item.  For each new query i < q_len_b of the
 * sequence and each of the G = Hq/Hkv query heads hq = h*G + g:
 *   keys t = t0 .. prior_b + i (causal; prior_b = ctx_b - q_len_b), t0 = 0, or
 *   with a sliding window of W keys t0 = max(0, prior_b + i - W + 1) (the
 *   sliding-window paged decode of [P1]'s op list: each query attends to its
 *   last W positions)
 *   l_t = scale * sum_ch Q[ch] * K^[t][ch]            (fp64)
 *   m = max_t l_t,  w_t = exp(l_t - m),  L = sum_t w_t
 *   out[ch] = (sum_t w_t * V^[t][ch]) / L,  lse = m + ln L
 * with K^, V^ the exact fp64 dequantized values.  No keys: out = 0, lse = -inf.
 */
static void decode_item(decode_job *J, int b, int h, double *l)
{
    const cache_t *c = &J->c;
    int g_count = J->hq / c->hkv;
    int d = c->d;
    int qlen = J->cu_q_lens ? J->cu_q_lens[b + 1] - J->cu_q_lens[b] : 1;
    int row0 = J->cu_q_lens ? J->cu_q_lens[b] : b;
    int ctx = J->context_lengths[b];
    int prior = ctx - qlen;
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < qlen; i++) {
        int nkeys = prior + i + 1; /* keys 0 .. prior + i */
        if (nkeys < 0)
            nkeys = 0;
        int t0 = J->window > 0 && nkeys > J->window ? nkeys - J->window : 0;
        for (int g = 0; g < g_count; g++) {
            int hq = h * g_count + g;
            int64_t o = ((int64_t)(row0 + i) * J->hq + hq) * d;
            const uint16_t *qv = J->q + o;
            for (int ch = 0; ch < d; ch++)
                acc[ch] = 0.0;
            if (nkeys == 0) {
                for (int ch = 0; ch < d; ch++) {
                    J->out[o + ch] = oracle_bf16_round(0.0);
                    if (J->out_f64)
                        J->out_f64[o + ch] = 0.0;
                }
                if (J->lse)
                    J->lse[(int64_t)(row0 + i) * J->hq + hq] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int t = t0; t < nkeys; t++) {
                int64_t blk = J->block_table[(int64_t)b * J->mbs + t / c->bs];
                double dot = 0.0;
                for (int ch = 0; ch < d; ch++)
                    dot += (double)bf16_to_float(qv[ch]) * deq_f64(c, 0, blk, h, t % c->bs, ch);
                l[t] = J->scale * dot;
                if (l[t] > m)
                    m = l[t];
            }
            double sum = 0.0;
            for (int t = t0; t < nkeys; t++) {
                int64_t blk = J->block_table[(int64_t)b * J->mbs + t / c->bs];
                double w = exp(l[t] - m);
                sum += w;
                for (int ch = 0; ch < d; ch++)
                    acc[ch] += w * deq_f64(c, 1, blk, h, t % c->bs, ch);
            }
            for (int ch = 0; ch < d; ch++) {
                double y = acc[ch] / sum;
                J->out[o + ch] = oracle_bf16_round(y);
                if (J->out_f64)
                    J->out_f64[o + ch] = y;
            }
            if (J->lse)
                J->lse[(int64_t)(row0 + i) * J->hq + hq] = m + log(sum);
        }
    }
    free(acc);
}

static void *decode_worker(void *arg)
{
    decode_job *J = (decode_job *)arg;
    int max_ctx = 1;
    for (int b = 0; b < J->batch; b++)
        if (J->context_lengths[b] > max_ctx)
            max_ctx = J->context_lengths[b];
    double *l = (double *)malloc(sizeof(double) * (size_t)max_ctx);
    int items = J->batch * J->c.hkv;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int it = J->next_item++;
        pthread_mutex_unlock(&J->mu);
        if (it >= items)
            break;
        decode_item(J, it / J->c.hkv, it % J->c.hkv, l);
    }
    free(l);
    return NULL;
}

/*
 * Attention of every new query over the paged cache.
 * q: bf16 [Tq][Hq][D] with Tq = cu_q_lens[batch] (or batch when cu_q_lens is
 * NULL, one query per sequence).  Writes out (bf16 [Tq][Hq][D], the fp64
 * result rounded once), and when non-NULL out_f64 (the fp64 result) and lse
 * (natural-log sum of exponentials, fp64 [Tq][Hq]).  Work items are spread
 * over nthreads threads; the arithmetic of each item does not depend on it.
 */
int oracle_decode(int mode, int nb, int hkv, int bs, int d, const void *k_cache,
                  const void *v_cache, const float *k_scale, const float *v_scale,
                  const uint16_t *q, int hq, const int32_t *block_table, int mbs,
                  const int32_t *context_lengths, const int32_t *cu_q_lens, int batch,
                  double scale, uint16_t *out, double *out_f64, double *lse, int nthreads,
                  int window)
{
    if (hkv <= 0 || hq % hkv != 0 || !out || window < 0)
        return -1;
    for (int b = 0; b < batch; b++) {
        if (context_lengths[b] > mbs * bs)
            return -1;
        for (int j = 0; j * bs < context_lengths[b]; j++)
            if (block_table[(int64_t)b * mbs + j] < 0 || block_table[(int64_t)b * mbs + j] >= nb)
                return -1;
    }
    decode_job J;
    memset(&J, 0, sizeof J);
    J.c = (cache_t){mode, nb, hkv, bs, d, (void *)k_cache, (void *)v_cache, (float *)k_scale,
                    (float *)v_scale};
    J.q = q;
    J.hq = hq;
    J.block_table = block_table;
    J.mbs = mbs;
    J.context_lengths = context_lengths;
    J.cu_q_lens = cu_q_lens;
    J.batch = batch;
    J.scale = scale;
    J.window = window;
    J.out = out;
    J.out_f64 = out_f64;
    J.lse = lse;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads == 1) {
        decode_worker(&J);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
        for (int i = 0; i < nthreads; i++)
            pthread_create(&th[i], NULL, decode_worker, &J);
        for (int i = 0; i < nthreads; i++)
            pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* paged MLA (latent) cache                                                   */
/* ------------------------------------------------------------------------- */
/*
 * [P1] lists MojoStorePagedMLAKVCache (KVCache rows) and MojoPagedDecodeMLA
 * (Attention rows) next to the GQA ops and says nothing more about them.  The
 * reading taken here is multi-head latent attention in its absorbed decode
 * form: every token keeps one compressed latent row c (Dc channels) and one
 * decoupled rotary key row r (Dr channels), shared by all query heads; a head
 * scores key t as scale * (q_c . c_t + q_r . r_t) and returns the weighted sum
 * of the latent rows (Dc channels; the value up-projection that follows is a
 * separate matrix product).  C8 storage: each of the two rows of a token is
 * quantized like a per-token row of the GQA cache (its own scale
 * fl32(absmax / 127), codes round-half-even, clamped), so a token carries two
 * fp32 scales.
 *
 * Layout:
 *   latent [NB][BS][Dc] int8    rope [NB][BS][Dr] int8
 *   latent_scale [NB][BS] fp32  rope_scale [NB][BS] fp32
 */

/* quantize one row of n bf16 values with its own absmax scale */
static void quant_row(const uint16_t *x, int n, int8_t *codes, float *scale)
{
    float absmax = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(bf16_to_float(x[i]));
        if (a > absmax)
            absmax = a;
    }
    float s = absmax_scale(absmax);
    for (int i = 0; i < n; i++)
        codes[i] = quant_one(bf16_to_float(x[i]), s);
    *scale = s;
}

/*
 * Store T new tokens: latent_new bf16 [T][Dc], rope_new bf16 [T][Dr].  Slots
 * are resolved as in oracle_store (slot_mapping, or cu_q_lens + context
 * lengths + block table).  Returns 0, or -1 on an argument it cannot serve.
 */
int oracle_mla_store(int nb, int bs, int dc, int dr, int8_t *latent, int8_t *rope,
                     float *latent_scale, float *rope_scale, const uint16_t *latent_new,
                     const uint16_t *rope_new, int num_tokens, const int64_t *slot_mapping,
                     const int32_t *cu_q_lens, const int32_t *context_lengths,
                     const int32_t *block_table, int batch, int mbs)
{
    if (bs <= 0 || dc <= 0 || dr <= 0)
        return -1;
    if (slot_mapping) {
        for (int t = 0; t < num_tokens; t++) {
            int64_t slot = slot_mapping[t];
            if (slot < 0)
                continue; /* padding token */
            if (slot / bs >= nb)
                return -1;
            quant_row(latent_new + (int64_t)t * dc, dc, latent + slot * dc, &latent_scale[slot]);
            quant_row(rope_new + (int64_t)t * dr, dr, rope + slot * dr, &rope_scale[slot]);
        }
        return 0;
    }
    if (!context_lengths || !block_table)
        return -1;
    for (int b = 0; b < batch; b++) {
        int qlen = cu_q_lens ? cu_q_lens[b + 1] - cu_q_lens[b] : 1;
        int t0 = cu_q_lens ? cu_q_lens[b] : b;
        int prior = context_lengths[b] - qlen;
        for (int i = 0; i < qlen; i++) {
            int p = prior + i;
            if (p < 0)
                continue; /* inactive decode slot (context length 0): nothing to store */
            if (p / bs >= mbs)
                return -1;
            int64_t blk = block_table[(int64_t)b * mbs + p / bs];
            if (blk < 0 || blk >= nb)
                return -1;
            int64_t slot = blk * bs + p % bs; /* row of the token in the page arrays */
            quant_row(latent_new + (int64_t)(t0 + i) * dc, dc, latent + slot * dc, &latent_scale[slot]);
            quant_row(rope_new + (int64_t)(t0 + i) * dr, dr, rope + slot * dr, &rope_scale[slot]);
        }
    }
    return 0;
}

typedef struct {
    int nb, bs, dc, dr;
    const int8_t *latent, *rope;
    const float *latent_scale, *rope_scale;
    const uint16_t *q_latent, *q_rope;
    int heads;
    const int32_t *block_table;
    int mbs;
    const int32_t *context_lengths;
    int batch;
    double scale;
    uint16_t *out;
    double *out_f64;
    double *lse;
    int next_item;
    pthread_mutex_t mu;
} mla_job;

/*
 * Sequence b, head h (one new query per sequence, at the last position; keys
 * t = 0 .. ctx_b - 1, the new token included):
 *   c^_t = double(code) * double(latent_scale)   r^_t likewise (exact in fp64)
 *   l_t = scale * (sum_i q_c[i] c^_t[i] + sum_j q_r[j] r^_t[j])
 *   m = max_t l_t,  w_t = exp(l_t - m),  L = sum_t w_t
 *   out[i] = (sum_t w_t c^_t[i]) / L,  lse = m + ln L
 * No keys: out = 0, lse = -inf.
 */
static void mla_item(mla_job *J, int b, int h, double *l, double *acc)
{
    int64_t o = ((int64_t)b * J->heads + h);
    const uint16_t *qc = J->q_latent + o * J->dc;
    const uint16_t *qr = J->q_rope + o * J->dr;
    int ctx = J->context_lengths[b];
    if (ctx <= 0) {
        for (int i = 0; i < J->dc; i++) {
            J->out[o * J->dc + i] = oracle_bf16_round(0.0);
            if (J->out_f64)
                J->out_f64[o * J->dc + i] = 0.0;
        }
        if (J->lse)
            J->lse[o] = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int t = 0; t < ctx; t++) {
        int64_t row = (int64_t)J->block_table[(int64_t)b * J->mbs + t / J->bs] * J->bs + t % J->bs;
        double sc = (double)J->latent_scale[row], sr = (double)J->rope_scale[row];
        double dot = 0.0;
        for (int i = 0; i < J->dc; i++)
            dot += (double)bf16_to_float(qc[i]) * ((double)J->latent[row * J->dc + i] * sc);
        for (int j = 0; j < J->dr; j++)
            dot += (double)bf16_to_float(qr[j]) * ((double)J->rope[row * J->dr + j] * sr);
        l[t] = J->scale * dot;
        if (l[t] > m)
            m = l[t];
    }
    for (int i = 0; i < J->dc; i++)
        acc[i] = 0.0;
    double sum = 0.0;
    for (int t = 0; t < ctx; t++) {
        int64_t row = (int64_t)J->block_table[(int64_t)b * J->mbs + t / J->bs] * J->bs + t % J->bs;
        double sc = (double)J->latent_scale[row];
        double w = exp(l[t] - m);
        sum += w;
        for (int i = 0; i < J->dc; i++)
            acc[i] += w * ((double)J->latent[row * J->dc + i] * sc);
    }
    for (int i = 0; i < J->dc; i++) {
        double y = acc[i] / sum;
        J->out[o * J->dc + i] = oracle_bf16_round(y);
        if (J->out_f64)
            J->out_f64[o * J->dc + i] = y;
    }
    if (J->lse)
        J->lse[o] = m + log(sum);
}

static void *mla_worker(void *arg)
{
    mla_job *J = (mla_job *)arg;
    int max_ctx = 1;
    for (int b = 0; b < J->batch; b++)
        if (J->context_lengths[b] > max_ctx)
            max_ctx = J->context_lengths[b];
    double *l = (double *)malloc(sizeof(double) * (size_t)max_ctx);
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->dc);
    int items = J->batch * J->heads;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int it = J->next_item++;
        pthread_mutex_unlock(&J->mu);
        if (it >= items)
            break;
        mla_item(J, it / J->heads, it % J->heads, l, acc);
    }
    free(acc);
    free(l);
    return NULL;
}

/*
 * Latent attention of one new query per sequence.  q_latent bf16 [B][H][Dc],
 * q_rope bf16 [B][H][Dr]; out bf16 [B][H][Dc] (the fp64 result rounded once),
 * out_f64 (optional) fp64 [B][H][Dc], lse (optional) fp64 [B][H].
 */
int oracle_mla_decode(int nb, int bs, int dc, int dr, const int8_t *latent, const int8_t *rope,
                      const float *latent_scale, const float *rope_scale, const uint16_t *q_latent,
                      const uint16_t *q_rope, int heads, const int32_t *block_table, int mbs,
                      const int32_t *context_lengths, int batch, double scale, uint16_t *out,
                      double *out_f64, double *lse, int nthreads)
{
    if (bs <= 0 || dc <= 0 || dr <= 0 || heads <= 0 || !out)
        return -1;
    for (int b = 0; b < batch; b++) {
        if (context_lengths[b] > mbs * bs)
            return -1;
        for (int j = 0; j * bs < context_lengths[b]; j++)
            if (block_table[(int64_t)b * mbs + j] < 0 || block_table[(int64_t)b * mbs + j] >= nb)
                return -1;
    }
    mla_job J;
    memset(&J, 0, sizeof J);
    J.nb = nb;
    J.bs = bs;
    J.dc = dc;
    J.dr = dr;
    J.latent = latent;
    J.rope = rope;
    J.latent_scale = latent_scale;
    J.rope_scale = rope_scale;
    J.q_latent = q_latent;
    J.q_rope = q_rope;
    J.heads = heads;
    J.block_table = block_table;
    J.mbs = mbs;
    J.context_lengths = context_lengths;
    J.batch = batch;
    J.scale = scale;
    J.out = out;
    J.out_f64 = out_f64;
    J.lse = lse;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads == 1) {
        mla_worker(&J);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
        for (int i = 0; i < nthreads; i++)
            pthread_create(&th[i], NULL, mla_worker, &J);
        for (int i = 0; i < nthreads; i++)
            pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return 0;
}
