/*
 * Command-line driver of the CPU oracle (oracle/adacomp_oracle.c), built
 * together with it by the CPU tests twice: plainly, and with the address and
 * undefined-behaviour sanitizers.  It runs every entry point of the oracle on
 * the cases of an input file and prints every result as hexadecimal words, so
 * the two builds can be compared text for text.
 *
 * Input, whitespace separated, floats as the hexadecimal of their bits:
 *   ncases
 *   per case:
 *     nseg K T span
 *     nseg lines: offset numel bin_len flags
 *     K learners, each: span words (starting residue), then T x span words
 *       (dW of each step)
 *     span words each of w, m, v
 *     lr momentum weight_decay scale beta1 beta2 eps (float bits), step
 * Output per case: the status and the results of each call, one tagged line
 * per array.  Exit status 0 when the input was read whole.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    uint64_t offset, numel;
    uint32_t bin_len, flags;
} seg_t;

uint32_t oracle_plan_hash(const seg_t *segs, uint32_t nseg);
int oracle_message_capacity(const seg_t *segs, uint32_t nseg, uint64_t *cap);
int oracle_compress(const seg_t *segs, uint32_t nseg, float *residue, const float *dW,
                    uint8_t *msg, uint64_t msg_cap, float *gmax_out, uint64_t *msg_bytes);
int oracle_decode_accumulate(const seg_t *segs, uint32_t nseg, const uint8_t *const *msgs,
                             uint32_t K, float *out, int accumulate);
int oracle_decode_sgd(const seg_t *segs, uint32_t nseg, const uint8_t *const *msgs, uint32_t K,
                      float *w, float *m, float lr, float momentum, float weight_decay,
                      float scale);
int oracle_decode_adam(const seg_t *segs, uint32_t nseg, const uint8_t *const *msgs, uint32_t K,
                       float *w, float *m, float *v, float lr, float b1, float b2, float eps,
                       float weight_decay, float scale, uint32_t t);

static FILE *in;

static int read_u64(uint64_t *v) {
    unsigned long long x;
    if (fscanf(in, "%llu", &x) != 1) return 0;
    *v = x;
    return 1;
}

static int read_floats(float *a, uint64_t n) {
    for (uint64_t i = 0; i < n; ++i) {
        unsigned x;
        if (fscanf(in, "%x", &x) != 1) return 0;
        memcpy(&a[i], &x, 4);
    }
    return 1;
}

static void print_floats(const char *tag, const float *a, uint64_t n) {
    printf("%s", tag);
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t x;
        memcpy(&x, &a[i], 4);
        printf(" %08x", x);
    }
    printf("\n");
}

static void print_bytes(const char *tag, const uint8_t *a, uint64_t n) {
    printf("%s %llu ", tag, (unsigned long long)n);
    for (uint64_t i = 0; i < n; ++i) printf("%02x", a[i]);
    printf("\n");
}

static uint64_t total_bins(const seg_t *s, uint32_t n) {
    uint64_t b = 0;
    for (uint32_t i = 0; i < n; ++i) b += (s[i].numel + s[i].bin_len - 1) / s[i].bin_len;
    return b;
}

static int run_case(int c) {
    uint64_t nseg, K, T, span;
    if (!read_u64(&nseg) || !read_u64(&K) || !read_u64(&T) || !read_u64(&span)) return 0;
    seg_t *segs = calloc(nseg ? nseg : 1, sizeof(seg_t));
    for (uint64_t i = 0; i < nseg; ++i) {
        uint64_t lt, fl;
        if (!read_u64(&segs[i].offset) || !read_u64(&segs[i].numel) || !read_u64(&lt) ||
            !read_u64(&fl))
            return 0;
        segs[i].bin_len = (uint32_t)lt;
        segs[i].flags = (uint32_t)fl;
    }
    printf("case %d hash %08x\n", c, oracle_plan_hash(segs, (uint32_t)nseg));
    uint64_t cap = 0;
    const int st = oracle_message_capacity(segs, (uint32_t)nseg, &cap);
    printf("capacity %d %llu\n", st, (unsigned long long)cap);

    float *r = malloc(span * sizeof(float));
    float *d = malloc(span * sizeof(float));
    uint8_t **msgs = calloc(K ? K : 1, sizeof(uint8_t *));
    const uint64_t nb = st == 0 ? total_bins(segs, (uint32_t)nseg) : 0;
    float *gmax = malloc((nb ? nb : 1) * sizeof(float));
    for (uint64_t k = 0; k < K; ++k) {
        msgs[k] = malloc(cap ? cap : 1);
        if (!read_floats(r, span)) return 0;
        for (uint64_t t = 0; t < T; ++t) {
            if (!read_floats(d, span)) return 0;
            uint64_t bytes = 0;
            const int cs = oracle_compress(segs, (uint32_t)nseg, r, d, msgs[k], cap, gmax, &bytes);
            printf("compress %llu %llu %d\n", (unsigned long long)k, (unsigned long long)t, cs);
            if (cs != 0) continue;
            print_floats("residue", r, span);
            print_floats("gmax", gmax, nb);
            print_bytes("message", msgs[k], bytes);
        }
    }
    float *w = malloc(span * sizeof(float));
    float *m = malloc(span * sizeof(float));
    float *v = malloc(span * sizeof(float));
    float p[7];
    uint64_t step;
    if (!read_floats(w, span) || !read_floats(m, span) || !read_floats(v, span) ||
        !read_floats(p, 7) || !read_u64(&step))
        return 0;
    if (st == 0 && K > 0 && T > 0) {
        const uint8_t *const *mm = (const uint8_t *const *)msgs;
        float *out = malloc(span * sizeof(float));
        memcpy(out, w, span * sizeof(float));
        printf("decode %d\n", oracle_decode_accumulate(segs, (uint32_t)nseg, mm, (uint32_t)K, out, 0));
        print_floats("sum", out, span);
        memcpy(out, w, span * sizeof(float));
        printf("decode_acc %d\n", oracle_decode_accumulate(segs, (uint32_t)nseg, mm, (uint32_t)K, out, 1));
        print_floats("acc", out, span);
        float *w1 = malloc(span * sizeof(float)), *m1 = malloc(span * sizeof(float));
        float *v1 = malloc(span * sizeof(float));
        memcpy(w1, w, span * sizeof(float));
        memcpy(m1, m, span * sizeof(float));
        printf("sgd %d\n", oracle_decode_sgd(segs, (uint32_t)nseg, mm, (uint32_t)K, w1, m1, p[0],
                                             p[1], p[2], p[3]));
        print_floats("sgd_w", w1, span);
        print_floats("sgd_m", m1, span);
        memcpy(w1, w, span * sizeof(float));
        memcpy(m1, m, span * sizeof(float));
        memcpy(v1, v, span * sizeof(float));
        printf("adam %d\n", oracle_decode_adam(segs, (uint32_t)nseg, mm, (uint32_t)K, w1, m1, v1,
                                               p[0], p[4], p[5], p[6], p[2], p[3], (uint32_t)step));
        print_floats("adam_w", w1, span);
        print_floats("adam_m", m1, span);
        print_floats("adam_v", v1, span);
        /* a message whose directory survivor count disagrees is refused */
        uint64_t bytes = 0;
        memcpy(r, w, span * sizeof(float));
        oracle_compress(segs, (uint32_t)nseg, r, m, msgs[0], cap, gmax, &bytes);
        msgs[0][36] ^= 1u;
        printf("corrupt %d\n", oracle_decode_accumulate(segs, (uint32_t)nseg, mm, 1, out, 0));
        free(out); free(w1); free(m1); free(v1);
    }
    for (uint64_t k = 0; k < K; ++k) free(msgs[k]);
    free(msgs); free(segs); free(r); free(d); free(gmax); free(w); free(m); free(v);
    return 1;
}

int main(int argc, char **argv) {
    if (argc < 2) return 2;
    in = fopen(argv[1], "r");
    if (!in) return 2;
    int n = 0;
    if (fscanf(in, "%d", &n) != 1) return 2;
    for (int c = 0; c < n; ++c)
        if (!run_case(c)) {
            fprintf(stderr, "input ends inside case %d\n", c);
            return 2;
        }
    fclose(in);
    return 0;
}
