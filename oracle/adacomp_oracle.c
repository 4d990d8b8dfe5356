/*
 * AdaComp CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded implementation of the AdaComp compressor and
 * of the matching decode-accumulate, used only to check the GPU library.  Only
 * the tests, the smoke entry point and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the HIP library.
 *
 * Source of the method: "AdaComp (Adaptive Residual Gradient Compression)",
 * AIMech curated page --
 *   [Def]  the one-sentence definition paragraph at the top of the page;
 *   [M1]   Claims, Mechanism "local-bin soft-threshold and mean-g_max
 *          quantization" (Algorithm 2 of the paper);
 *   [App]  Claims, Application "conv 40x and FC/LSTM 200x compression"
 *          (Table 2): L_T = 50 for conv, 500 for FC/LSTM, 8-bit sparse index
 *          words when L_T < 64, 16-bit words otherwise;
 *   [Lim]  Claims, Limitation "minibatch size, activity and variable message
 *          length" and "Curated Limitations & Negative Results": the number
 *          of transmitted elements varies, so the message has variable length.
 *   [Opt]  the arXiv abstract of the same paper: AdaComp is shown with SGD
 *          with momentum and Adam as the optimizers of the training runs.
 *   [LS]   Claims, Mechanism "self-adjusting sparsity prevents residual
 *          explosion" (Figures 4-6): the hard Local Selection (LS) baseline
 *          that AdaComp is contrasted with, which has no soft threshold and
 *          transmits only a fixed number of bin maxima.
 *
 * Per layer (segment) the pages define, in this order:
 *   G = residue + dW;  H = G + dW;  bins of length L_T over G;
 *   g_max(i) = max |G| over bin i;  transmit every index with |H| >= g_max(i);
 *   s = (1/B) * sum_i g_max(i);  G_q = sign(G) * s for transmitted indices;
 *   residue <- G - G_q for transmitted indices, residue <- G otherwise.
 *
 * Readings where the pages are silent:
 *   - fp32 arithmetic, round-to-nearest-even, no contraction: H is
 *     fl(fl(residue + dW) + dW), never residue + 2*dW rounded once.
 *   - bins are consecutive runs of L_T elements of the flattened (C-order)
 *     layer; the last bin may be shorter and still counts in B.
 *   - ">=" is inclusive, so every tie with the bin maximum is transmitted.
 *   - sign(0) = 0: an element with G = 0 quantizes to 0, so it is not sent
 *     (a sign bit cannot encode it) and its residue stays G either way.
 *   - s: the bin maxima are summed left to right in double precision, the
 *     sum is divided by B in double precision, and the quotient is rounded
 *     once to float.
 *   - the message layout below is this project's own definition; the pages
 *     give only the index word widths.
 *   - decode + SGD step: the summed messages are the gradient of one step
 *     of SGD with momentum in its usual form (no dampening, no Nesterov):
 *     g = scale * sum (+ weight_decay * w when weight_decay != 0),
 *     m = momentum * m + g, w = w - lr * m, each operation rounded to float.
 *   - decode + Adam step: Adam with bias-corrected moments in its textbook
 *     form, each operation rounded to float: g as above, m = b1*m + (1-b1)*g,
 *     v = b2*v + (1-b2)*(g*g), w = w - lr * ((m/c1) / (sqrt(v/c2) + eps))
 *     with c1 = 1 - b1^t, c2 = 1 - b2^t for step t >= 1 (each computed in
 *     double and rounded once to float; 1-b1, 1-b2 are float operations).
 *   - LS (segment flag 1): per bin exactly one element is transmitted, the
 *     first (lowest index) whose |G| equals the bin maximum, and none when
 *     the maximum is 0; it is quantized with the same layer-wide s and the
 *     residue is updated as above.  The page says only "a fixed number of
 *     bin maxima"; one per bin is the plainest reading.
 *
 * Message layout (all fields little-endian, every region 16-byte aligned,
 * padding bytes zero):
 *   header, 32 bytes: u32 magic 0x43414441, u16 version 1, u16 0, u32 nseg,
 *     u32 plan_hash (FNV-1a 32 over the segment table), u64 total_bytes,
 *     u64 total_survivors;
 *   directory at byte 32: nseg x {f32 s, u32 nsurv, u64 entries_offset};
 *   count regions, one per segment in table order: B words of w bits, the
 *     number of transmitted elements of each bin;
 *   entry regions, one per segment in table order, packed after the count
 *     regions: nsurv words of w bits, bin-major with ascending in-bin index,
 *     word = sign << (w-1) | in_bin_index, sign = 1 iff G < 0.
 *   w = 8 if L_T < 64 else 16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    uint64_t offset;  /* first element of the layer in the flat buffers */
    uint64_t numel;   /* number of elements of the layer */
    uint32_t bin_len; /* L_T */
    uint32_t flags;   /* 0: AdaComp; ORACLE_FLAG_LS: hard local selection */
} oracle_segment;

#define ORACLE_FLAG_LS 1u

enum {
    ORACLE_OK = 0,
    ORACLE_BAD_ARG = -1,
    ORACLE_NO_ROOM = -2,
    ORACLE_BAD_MESSAGE = -3,
};

#define ORACLE_MAGIC 0x43414441u
#define ORACLE_VERSION 1u

static uint64_t round_up16(uint64_t x) { return (x + 15u) & ~(uint64_t)15u; }

/* Index word width from [App] / [Lim]: 8 bits below L_T = 64, else 16. */
static uint32_t word_bytes(uint32_t bin_len) { return bin_len < 64u ? 1u : 2u; }

static uint64_t num_bins(const oracle_segment *sg) {
    return (sg->numel + sg->bin_len - 1u) / sg->bin_len;
}

static void put_u16(uint8_t *p, uint32_t v) {
    p[0] = (uint8_t)(v & 0xffu);
    p[1] = (uint8_t)((v >> 8) & 0xffu);
}
static void put_u32(uint8_t *p, uint32_t v) {
    for (int i = 0; i < 4; ++i) p[i] = (uint8_t)((v >> (8 * i)) & 0xffu);
}
static void put_u64(uint8_t *p, uint64_t v) {
    for (int i = 0; i < 8; ++i) p[i] = (uint8_t)((v >> (8 * i)) & 0xffu);
}
static uint32_t get_u16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get_u32(const uint8_t *p) {
    uint32_t v = 0;
    for (int i = 3; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static uint64_t get_u64(const uint8_t *p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static void put_word(uint8_t *p, uint32_t wb, uint32_t v) {
    if (wb == 1u) p[0] = (uint8_t)v; else put_u16(p, v);
}
static uint32_t get_word(const uint8_t *p, uint32_t wb) {
    return wb == 1u ? (uint32_t)p[0] : get_u16(p);
}

/* FNV-1a, 32 bit (offset basis 2166136261, prime 16777619), over each
 * segment's offset (8 bytes), numel (8), bin_len (4) and flags (4), all
 * little-endian, in table order. */
uint32_t oracle_plan_hash(const oracle_segment *segs, uint32_t nseg) {
    uint32_t h = 2166136261u;
    uint8_t buf[24];
    for (uint32_t i = 0; i < nseg; ++i) {
        put_u64(buf, segs[i].offset);
        put_u64(buf + 8, segs[i].numel);
        put_u32(buf + 16, segs[i].bin_len);
        put_u32(buf + 20, segs[i].flags);
        for (int k = 0; k < 24; ++k) {
            h ^= buf[k];
            h *= 16777619u;
        }
    }
    return h;
}

static int check_segments(const oracle_segment *segs, uint32_t nseg) {
    if (segs == NULL || nseg == 0u) return ORACLE_BAD_ARG;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (segs[i].numel == 0u || segs[i].numel >= ((uint64_t)1 << 32)) return ORACLE_BAD_ARG;
        if (segs[i].bin_len == 0u || segs[i].bin_len > 32768u) return ORACLE_BAD_ARG;
        if (segs[i].flags != 0u && segs[i].flags != ORACLE_FLAG_LS) return ORACLE_BAD_ARG;
    }
    return ORACLE_OK;
}

/* Byte offset of the first count region. */
static uint64_t counts_begin(uint32_t nseg) { return round_up16(32u + 16u * (uint64_t)nseg); }

/* Byte offset where the entry regions begin (after every count region). */
static uint64_t entries_begin(const oracle_segment *segs, uint32_t nseg) {
    uint64_t at = counts_begin(nseg);
    for (uint32_t i = 0; i < nseg; ++i)
        at = round_up16(at + num_bins(&segs[i]) * word_bytes(segs[i].bin_len));
    return at;
}

/* Largest message the segment table can produce: every element transmitted. */
int oracle_message_capacity(const oracle_segment *segs, uint32_t nseg, uint64_t *cap) {
    int st = check_segments(segs, nseg);
    if (st != ORACLE_OK) return st;
    uint64_t at = entries_begin(segs, nseg);
    for (uint32_t i = 0; i < nseg; ++i)
        at = round_up16(at + segs[i].numel * word_bytes(segs[i].bin_len));
    *cap = at;
    return ORACLE_OK;
}

/*
 * One compression step over every segment, in table order.  residue is
 * updated in place; dW is read.  The message is written to msg (msg_cap
 * bytes); its length goes to *msg_bytes.  gmax_out (nullable) receives every
 * bin maximum, segments in table order, bins in order.
 */
int oracle_compress(const oracle_segment *segs, uint32_t nseg, float *residue,
                    const float *dW, uint8_t *msg, uint64_t msg_cap,
                    float *gmax_out, uint64_t *msg_bytes) {
    int st = check_segments(segs, nseg);
    if (st != ORACLE_OK) return st;
    uint64_t cap = 0;
    oracle_message_capacity(segs, nseg, &cap);
    if (msg_cap < cap) return ORACLE_NO_ROOM;
    memset(msg, 0, cap);

    uint64_t count_at = counts_begin(nseg);
    uint64_t entry_at = entries_begin(segs, nseg);
    uint64_t total_surv = 0;
    uint64_t gmax_at = 0;

    for (uint32_t l = 0; l < nseg; ++l) {
        const oracle_segment *sg = &segs[l];
        const uint64_t N = sg->numel;
        const uint32_t LT = sg->bin_len;
        const uint32_t wb = word_bytes(LT);
        const uint64_t B = num_bins(sg);
        float *r = residue + sg->offset;
        const float *dw = dW + sg->offset;

        float *G = (float *)malloc(N * sizeof(float));
        float *H = (float *)malloc(N * sizeof(float));
        float *gmax = (float *)malloc(B * sizeof(float));
        if (!G || !H || !gmax) {
            free(G); free(H); free(gmax);
            return ORACLE_BAD_ARG;
        }

        /* [Def], [M1]: accumulated residual gradient and the probe H. */
        for (uint64_t j = 0; j < N; ++j) {
            G[j] = r[j] + dw[j];
            H[j] = G[j] + dw[j];
        }

        /* [Def], [M1]: uniform bins of length L_T, local maximum of |G|. */
        for (uint64_t b = 0; b < B; ++b) {
            uint64_t lo = b * LT, hi = lo + LT < N ? lo + LT : N;
            float m = 0.0f;
            for (uint64_t j = lo; j < hi; ++j)
                if (fabsf(G[j]) > m) m = fabsf(G[j]);
            gmax[b] = m;
        }

        /* [Def], [M1]: one layer-wide scale, the mean of the bin maxima. */
        double acc = 0.0;
        for (uint64_t b = 0; b < B; ++b) acc += (double)gmax[b];
        const float s = (float)(acc / (double)B);

        /* [Def], [M1]: soft-threshold selection, ternary quantization and the
         * residue update; [App]: the sparse-indexed ternarized words.
         * [LS]: instead of the soft threshold, only the bin's first maximum. */
        const int ls = (sg->flags & ORACLE_FLAG_LS) != 0u;
        uint64_t nsurv = 0;
        for (uint64_t b = 0; b < B; ++b) {
            uint64_t lo = b * LT, hi = lo + LT < N ? lo + LT : N;
            uint64_t first_max = hi;
            if (ls && gmax[b] > 0.0f)
                for (uint64_t j = lo; j < hi && first_max == hi; ++j)
                    if (fabsf(G[j]) == gmax[b]) first_max = j;
            uint32_t cnt = 0;
            for (uint64_t j = lo; j < hi; ++j) {
                int sent = ls ? j == first_max : fabsf(H[j]) >= gmax[b] && G[j] != 0.0f;
                if (sent) {
                    float gq = G[j] > 0.0f ? s : -s;
                    r[j] = G[j] - gq;
                    uint32_t sign = G[j] < 0.0f ? 1u : 0u;
                    uint32_t word = (sign << (8u * wb - 1u)) | (uint32_t)(j - lo);
                    put_word(msg + entry_at + (nsurv + cnt) * wb, wb, word);
                    ++cnt;
                } else {
                    r[j] = G[j];
                }
            }
            put_word(msg + count_at + b * wb, wb, cnt);
            nsurv += cnt;
        }

        uint8_t *dir = msg + 32u + 16u * (uint64_t)l;
        uint32_t sbits;
        memcpy(&sbits, &s, 4);
        put_u32(dir, sbits);
        put_u32(dir + 4, (uint32_t)nsurv);
        put_u64(dir + 8, entry_at);

        if (gmax_out) memcpy(gmax_out + gmax_at, gmax, B * sizeof(float));
        gmax_at += B;
        count_at = round_up16(count_at + B * wb);
        entry_at = round_up16(entry_at + nsurv * wb);
        total_surv += nsurv;
        free(G); free(H); free(gmax);
    }

    put_u32(msg, ORACLE_MAGIC);
    put_u16(msg + 4, ORACLE_VERSION);
    put_u16(msg + 6, 0u);
    put_u32(msg + 8, nseg);
    put_u32(msg + 12, oracle_plan_hash(segs, nseg));
    put_u64(msg + 16, entry_at);
    put_u64(msg + 24, total_surv);
    if (msg_bytes) *msg_bytes = entry_at;
    return ORACLE_OK;
}

/*
 * Sum K messages into out: for every message in order k = 0..K-1 and every
 * transmitted index j of it, out[j] = fl32(out[j] + sign * s).  An element no
 * message transmits gets no addition at all.  accumulate = 0 first sets every
 * element of every segment to +0; accumulate = 1 starts from out as given.
 * Elements outside every segment are left untouched.  The pages say only that
 * the quantized elements are transmitted; summing them is the data-parallel
 * aggregation they feed.
 */
int oracle_decode_accumulate(const oracle_segment *segs, uint32_t nseg,
                             const uint8_t *const *msgs, uint32_t K, float *out,
                             int accumulate) {
    int st = check_segments(segs, nseg);
    if (st != ORACLE_OK) return st;
    if (!accumulate)
        for (uint32_t l = 0; l < nseg; ++l)
            for (uint64_t j = 0; j < segs[l].numel; ++j) out[segs[l].offset + j] = 0.0f;
    const uint32_t hash = oracle_plan_hash(segs, nseg);
    for (uint32_t k = 0; k < K; ++k) {
        const uint8_t *m = msgs[k];
        if (get_u32(m) != ORACLE_MAGIC || get_u16(m + 4) != ORACLE_VERSION ||
            get_u32(m + 8) != nseg || get_u32(m + 12) != hash)
            return ORACLE_BAD_MESSAGE;
        uint64_t count_at = counts_begin(nseg);
        for (uint32_t l = 0; l < nseg; ++l) {
            const oracle_segment *sg = &segs[l];
            const uint32_t wb = word_bytes(sg->bin_len);
            const uint64_t B = num_bins(sg);
            const uint8_t *dir = m + 32u + 16u * (uint64_t)l;
            uint32_t sbits = get_u32(dir);
            float s;
            memcpy(&s, &sbits, 4);
            uint64_t e = get_u64(dir + 8);
            uint64_t seen = 0;
            for (uint64_t b = 0; b < B; ++b) {
                uint32_t cnt = get_word(m + count_at + b * wb, wb);
                for (uint32_t c = 0; c < cnt; ++c) {
                    uint32_t word = get_word(m + e, wb);
                    e += wb;
                    uint32_t sign = word >> (8u * wb - 1u);
                    uint32_t idx = word & ((1u << (8u * wb - 1u)) - 1u);
                    uint64_t j = b * sg->bin_len + idx;
                    if (j >= sg->numel) return ORACLE_BAD_MESSAGE;
                    float q = sign ? -s : s;
                    out[sg->offset + j] = out[sg->offset + j] + q;
                }
                seen += cnt;
            }
            if (seen != get_u32(dir + 4)) return ORACLE_BAD_MESSAGE;
            count_at = round_up16(count_at + B * wb);
        }
    }
    return ORACLE_OK;
}

/*
 * Sum K messages (as oracle_decode_accumulate with accumulate = 0) and apply
 * one step of SGD with momentum to every element of every segment, [Opt]:
 *   g = scale * sum;  if weight_decay != 0: g = g + weight_decay * w;
 *   m = momentum * m + g;  w = w - lr * m.
 * Every operation is one float operation rounded to nearest (no contraction).
 * Elements outside every segment are left untouched.
 */
int oracle_decode_sgd(const oracle_segment *segs, uint32_t nseg, const uint8_t *const *msgs,
                      uint32_t K, float *w, float *m, float lr, float momentum,
                      float weight_decay, float scale) {
    int st = check_segments(segs, nseg);
    if (st != ORACLE_OK) return st;
    uint64_t span = 0;
    for (uint32_t l = 0; l < nseg; ++l)
        if (segs[l].offset + segs[l].numel > span) span = segs[l].offset + segs[l].numel;
    float *sum = (float *)malloc((span ? span : 1) * sizeof(float));
    if (!sum) return ORACLE_BAD_ARG;
    st = oracle_decode_accumulate(segs, nseg, msgs, K, sum, 0);
    if (st == ORACLE_OK) {
        for (uint32_t l = 0; l < nseg; ++l) {
            for (uint64_t j = segs[l].offset; j < segs[l].offset + segs[l].numel; ++j) {
                float g = scale * sum[j];
                if (weight_decay != 0.0f) g = g + weight_decay * w[j];
                m[j] = momentum * m[j] + g;
                w[j] = w[j] - lr * m[j];
            }
        }
    }
    free(sum);
    return st;
}

/*
 * Sum K messages and apply one Adam step (step number t >= 1) to every
 * element of every segment, [Opt]:
 *   g = scale * sum;  if weight_decay != 0: g = g + weight_decay * w;
 *   m = b1 * m + (1 - b1) * g;  v = b2 * v + (1 - b2) * (g * g);
 *   w = w - lr * ((m / c1) / (sqrt(v / c2) + eps)),
 *   c1 = 1 - b1^t, c2 = 1 - b2^t (double, rounded once to float).
 */
int oracle_decode_adam(const oracle_segment *segs, uint32_t nseg, const uint8_t *const *msgs,
                       uint32_t K, float *w, float *m, float *v, float lr, float b1, float b2,
                       float eps, float weight_decay, float scale, uint32_t t) {
    int st = check_segments(segs, nseg);
    if (st != ORACLE_OK) return st;
    if (t == 0u) return ORACLE_BAD_ARG;
    uint64_t span = 0;
    for (uint32_t l = 0; l < nseg; ++l)
        if (segs[l].offset + segs[l].numel > span) span = segs[l].offset + segs[l].numel;
    float *sum = (float *)malloc((span ? span : 1) * sizeof(float));
    if (!sum) return ORACLE_BAD_ARG;
    st = oracle_decode_accumulate(segs, nseg, msgs, K, sum, 0);
    if (st == ORACLE_OK) {
        const float c1 = (float)(1.0 - pow((double)b1, (double)t));
        const float c2 = (float)(1.0 - pow((double)b2, (double)t));
        const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
        for (uint32_t l = 0; l < nseg; ++l) {
            for (uint64_t j = segs[l].offset; j < segs[l].offset + segs[l].numel; ++j) {
                float g = scale * sum[j];
                if (weight_decay != 0.0f) g = g + weight_decay * w[j];
                m[j] = b1 * m[j] + omb1 * g;
                v[j] = b2 * v[j] + omb2 * (g * g);
                const float mh = m[j] / c1;
                const float vh = v[j] / c2;
                w[j] = w[j] - lr * (mh / (sqrtf(vh) + eps));
            }
        }
    }
    free(sum);
    return st;
}
