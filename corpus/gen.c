/*
 * Seeded synthetic corpora for BPE training.
 *
 * This module only produces bytes. It holds none of the training method's
 * arithmetic (no character classes, no pair counting, no merging), so the
 * oracle and the GPU path can both read its output without sharing any step
 * of the method.
 *
 * Random numbers: xoshiro256** (Blackman & Vigna, "Scrambled linear
 * pseudorandom number generators", 2018), seeded by expanding a 64-bit seed
 * with SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", 2014), both written here from their published definitions.
 *
 * Two families of corpora:
 *   corpus_words  - space-separated words drawn Zipf(s) from a fixed random
 *                   vocabulary, with digit tokens, attached punctuation and a
 *                   newline in place of the space once a line reaches 80 B.
 *   corpus_runs   - alternating segments of single-byte runs and uniform
 *                   random bytes, with geometric lengths.
 * Both fill exactly n bytes (the token stream is cut at n).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct { uint64_t s[4]; } rng_t;

static uint64_t splitmix64_next(uint64_t *x) {
    uint64_t z = (*x += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static void rng_seed(rng_t *r, uint64_t seed) {
    uint64_t x = seed;
    for (int i = 0; i < 4; i++) r->s[i] = splitmix64_next(&x);
}

static inline uint64_t rotl64(uint64_t v, int k) { return (v << k) | (v >> (64 - k)); }

static inline uint64_t rng_next(rng_t *r) {
    uint64_t *s = r->s;
    uint64_t out = rotl64(s[1] * 5, 7) * 9;
    uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl64(s[3], 45);
    return out;
}

/* uniform double in [0, 1) with 53 random bits */
static inline double rng_u01(rng_t *r) { return (double)(rng_next(r) >> 11) * 0x1.0p-53; }

/* uniform integer in [0, m), m >= 1, by rejection of the biased top range */
static inline uint64_t rng_below(rng_t *r, uint64_t m) {
    uint64_t lim = (UINT64_MAX / m) * m;
    uint64_t v;
    do { v = rng_next(r); } while (v >= lim);
    return v % m;
}

/* geometric on {1, 2, ...} with success probability p (mean 1/p), by inversion */
static inline uint64_t rng_geom(rng_t *r, double p) {
    double u = 1.0 - rng_u01(r); /* (0, 1] */
    double g = floor(log(u) / log1p(-p));
    return 1 + (uint64_t)g;
}

/* ------------------------------------------------------------------------ */
/* alphabets: each letter is a UTF-8 byte string of length 1..3              */

typedef struct { uint8_t b[4]; uint8_t len; } letter_t;

static size_t utf8_encode(uint32_t cp, uint8_t *o) {
    if (cp < 0x80) { o[0] = (uint8_t)cp; return 1; }
    if (cp < 0x800) { o[0] = 0xC0 | (cp >> 6); o[1] = 0x80 | (cp & 0x3F); return 2; }
    o[0] = 0xE0 | (cp >> 12); o[1] = 0x80 | ((cp >> 6) & 0x3F); o[2] = 0x80 | (cp & 0x3F);
    return 3;
}

static letter_t mk_letter(uint32_t cp) {
    letter_t l; memset(&l, 0, sizeof l);
    l.len = (uint8_t)utf8_encode(cp, l.b);
    return l;
}

enum { ALPHA_ASCII = 0, ALPHA_TURKISH = 1, ALPHA_MIXED = 2 };

typedef struct {
    letter_t ascii[26];
    letter_t turkish[29];
    letter_t two[64]; int n_two;
    letter_t three[32];
} alphabets_t;

static void build_alphabets(alphabets_t *a) {
    for (int i = 0; i < 26; i++) a->ascii[i] = mk_letter('a' + i);
    /* Turkish lowercase alphabet (29 letters); c-cedilla, g-breve, dotless i,
       o-umlaut, s-cedilla and u-umlaut are two-byte UTF-8 */
    static const uint32_t tr[29] = {'a', 'b', 'c', 0xE7, 'd', 'e', 'f', 'g', 0x11F, 'h',
                                    0x131, 'i', 'j', 'k', 'l', 'm', 'n', 'o', 0xF6, 'p',
                                    'r', 's', 0x15F, 't', 'u', 0xFC, 'v', 'y', 'z'};
    for (int i = 0; i < 29; i++) a->turkish[i] = mk_letter(tr[i]);
    /* two-byte letters: Latin-1 U+00E0..U+00FF without the division sign,
       plus the three Turkish letters outside that block */
    a->n_two = 0;
    for (uint32_t cp = 0xE0; cp <= 0xFF; cp++)
        if (cp != 0xF7) a->two[a->n_two++] = mk_letter(cp);
    a->two[a->n_two++] = mk_letter(0x11F);
    a->two[a->n_two++] = mk_letter(0x131);
    a->two[a->n_two++] = mk_letter(0x15F);
    /* three-byte letters: 32 fixed code points U+0905..U+0924 */
    for (int i = 0; i < 32; i++) a->three[i] = mk_letter(0x905 + i);
}

static letter_t draw_letter(rng_t *r, const alphabets_t *a, int kind) {
    if (kind == ALPHA_ASCII) return a->ascii[rng_below(r, 26)];
    if (kind == ALPHA_TURKISH) return a->turkish[rng_below(r, 29)];
    /* mixed: 70% ASCII, 20% two-byte, 10% three-byte */
    uint64_t u = rng_below(r, 10);
    if (u < 7) return a->ascii[rng_below(r, 26)];
    if (u < 9) return a->two[rng_below(r, (uint64_t)a->n_two)];
    return a->three[rng_below(r, 32)];
}

static const char PUNCT[33] = "!\"#$%&'()*+,-./:;<=>?@[\\]^_`{|}~";

/* binary search: smallest i with cdf[i] > u */
static uint32_t cdf_search(const double *cdf, uint32_t n, double u) {
    uint32_t lo = 0, hi = n - 1;
    while (lo < hi) {
        uint32_t mid = lo + (hi - lo) / 2;
        if (cdf[mid] > u) hi = mid; else lo = mid + 1;
    }
    return lo;
}

/*
 * Word corpus. Returns 0 on success, -1 on bad arguments or allocation failure.
 *   n_words      vocabulary size V (rank r = the r-th word generated)
 *   zipf_s       Zipf exponent: P(rank r) proportional to r^-s
 *   min_len/max_len  word length in letters, uniform
 *   alphabet     0 = a..z, 1 = 29-letter Turkish, 2 = mixed 1/2/3-byte letters
 *   digit_p      probability that a token is a digit run of 1..max_digits digits
 *   punct_p      probability that a token is one punctuation byte (attached)
 */
int corpus_words(uint8_t *out, uint64_t n, uint64_t seed, uint32_t n_words, double zipf_s,
                 uint32_t min_len, uint32_t max_len, int alphabet, double digit_p,
                 double punct_p, uint32_t max_digits) {
    if (!out || n_words == 0 || min_len == 0 || max_len < min_len || max_len > 64 ||
        max_digits == 0 || alphabet < 0 || alphabet > 2)
        return -1;
    rng_t r;
    rng_seed(&r, seed);
    alphabets_t A;
    build_alphabets(&A);

    /* vocabulary: word w occupies wbytes[woff[w] .. woff[w+1]) */
    uint64_t *woff = (uint64_t *)malloc(sizeof(uint64_t) * ((size_t)n_words + 1));
    uint8_t *wbytes = (uint8_t *)malloc((size_t)n_words * max_len * 3);
    double *cdf = (double *)malloc(sizeof(double) * n_words);
    if (!woff || !wbytes || !cdf) { free(woff); free(wbytes); free(cdf); return -1; }
    uint64_t pos = 0;
    for (uint32_t w = 0; w < n_words; w++) {
        woff[w] = pos;
        uint32_t len = min_len + (uint32_t)rng_below(&r, max_len - min_len + 1);
        for (uint32_t j = 0; j < len; j++) {
            letter_t l = draw_letter(&r, &A, alphabet);
            memcpy(wbytes + pos, l.b, l.len);
            pos += l.len;
        }
    }
    woff[n_words] = pos;
    double acc = 0.0;
    for (uint32_t w = 0; w < n_words; w++) { acc += pow((double)(w + 1), -zipf_s); cdf[w] = acc; }
    for (uint32_t w = 0; w < n_words; w++) cdf[w] /= acc;
    cdf[n_words - 1] = 1.0;

    uint64_t o = 0, line = 0;
    int first = 1;
    while (o < n) {
        double u = rng_u01(&r);
        if (u < punct_p && !first) {
            /* punctuation byte attached to the previous token, no separator */
            out[o++] = (uint8_t)PUNCT[rng_below(&r, 32)];
            line++;
            continue;
        }
        if (!first) {
            uint8_t sep = line >= 80 ? '\n' : ' ';
            out[o++] = sep;
            line = (sep == '\n') ? 0 : line + 1;
            if (o >= n) break;
        }
        first = 0;
        if (u < punct_p + digit_p) {
            uint32_t nd = 1 + (uint32_t)rng_below(&r, max_digits);
            for (uint32_t j = 0; j < nd && o < n; j++) { out[o++] = (uint8_t)('0' + rng_below(&r, 10)); line++; }
        } else {
            uint32_t w = cdf_search(cdf, n_words, rng_u01(&r));
            uint64_t len = woff[w + 1] - woff[w];
            if (len > n - o) len = n - o;
            memcpy(out + o, wbytes + woff[w], len);
            o += len;
            line += len;
        }
    }
    free(woff); free(wbytes); free(cdf);
    return 0;
}

/*
 * Run corpus: alternating segments, starting with a run segment.
 *   run segment:    one byte uniform in 0..255 repeated Geom(1/run_mean) times
 *   random segment: Geom(1/rand_mean) bytes uniform in 0..255
 */
int corpus_runs(uint8_t *out, uint64_t n, uint64_t seed, double run_mean, double rand_mean) {
    if (!out || run_mean < 1.0 || rand_mean < 1.0) return -1;
    rng_t r;
    rng_seed(&r, seed);
    uint64_t o = 0;
    int run = 1;
    while (o < n) {
        if (run) {
            uint8_t b = (uint8_t)rng_below(&r, 256);
            uint64_t len = rng_geom(&r, 1.0 / run_mean);
            if (len > n - o) len = n - o;
            memset(out + o, b, len);
            o += len;
        } else {
            uint64_t len = rng_geom(&r, 1.0 / rand_mean);
            if (len > n - o) len = n - o;
            for (uint64_t j = 0; j < len; j++) out[o + j] = (uint8_t)rng_below(&r, 256);
            o += len;
        }
        run = !run;
    }
    return 0;
}

/* Raw generator output, for pinning the generator itself against its
   published reference values. */
void corpus_rng_raw(uint64_t seed, uint64_t *out, uint64_t count) {
    rng_t r;
    rng_seed(&r, seed);
    for (uint64_t i = 0; i < count; i++) out[i] = rng_next(&r);
}

uint64_t corpus_splitmix_raw(uint64_t seed, uint64_t *out, uint64_t count) {
    uint64_t x = seed;
    for (uint64_t i = 0; i < count; i++) out[i] = splitmix64_next(&x);
    return x;
}

/* Raw xoshiro256** output from an explicit state (for the published vector). */
void corpus_rng_raw_state(const uint64_t *state, uint64_t *out, uint64_t count) {
    rng_t r;
    for (int i = 0; i < 4; i++) r.s[i] = state[i];
    for (uint64_t i = 0; i < count; i++) out[i] = rng_next(&r);
}
