/*
 * Sanitizer run of the C oracle and the corpus generator (host code only).
 *
 * TEST INFRASTRUCTURE ONLY: built with gcc -fsanitize=address,undefined by
 * oracle.build_sanitize_check() and run as a child process by the CPU tests,
 * so that the oracle's hand-managed memory (growing arrays, hash maps,
 * heaps, tries) and the generator's buffers are exercised under
 * AddressSanitizer and UndefinedBehaviorSanitizer. It repeats brute-force
 * pins the Python tests also check, through the same C entry points:
 *   1. the literal oracle equals the chunk-multiset oracle (merges, tokens,
 *      lengths) on every string of length <= 6 over {a, b, 1, space, 0xC3};
 *   2. on small corpora of every generator recipe: literal == chunks, the
 *      encoder applied to the training text with the learned list gives the
 *      training tokens, and the longest-match tokens spell the text back;
 *   3. the empty corpus and a corpus that runs out of pairs.
 * Prints "ok" and exits 0, or prints the first failure and exits 1; a
 * sanitizer report aborts with a nonzero status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_train_literal(const uint8_t *b, uint64_t n, uint32_t n_merges, uint32_t *merges, uint32_t *n_done,
                         uint32_t *tokens, uint64_t *n_tokens, uint64_t *lengths);
int oracle_train_chunks(const uint8_t *b, uint64_t n, uint32_t n_merges, uint32_t *merges, uint32_t *n_done,
                        uint32_t *tokens, uint64_t *n_tokens, uint64_t *lengths);
int oracle_encode(const uint8_t *b, uint64_t n, const uint32_t *pairs, uint32_t n_merges, uint32_t *counts,
                  uint32_t *tokens, uint64_t *n_tokens);
int oracle_trie_encode(const uint8_t *b, uint64_t n, const uint32_t *pairs, uint32_t n_merges, uint32_t *tokens,
                       uint64_t *n_tokens);
int corpus_words(uint8_t *out, uint64_t n, uint64_t seed, uint32_t n_words, double zipf_s, uint32_t min_len,
                 uint32_t max_len, int alphabet, double digit_p, double punct_p, uint32_t max_digits);
int corpus_runs(uint8_t *out, uint64_t n, uint64_t seed, double run_mean, double rand_mean);

typedef struct {
    uint32_t *merges, n_done, *tokens;
    uint64_t n_tokens, *lengths;
} result_t;

static int train(int literal, const uint8_t *b, uint64_t n, uint32_t m, result_t *r) {
    r->merges = malloc(sizeof(uint32_t) * 3 * (m ? m : 1));
    r->tokens = malloc(sizeof(uint32_t) * (n ? n : 1));
    r->lengths = malloc(sizeof(uint64_t) * (m + 1));
    if (!r->merges || !r->tokens || !r->lengths) return -2;
    return (literal ? oracle_train_literal : oracle_train_chunks)(b, n, m, r->merges, &r->n_done, r->tokens,
                                                                  &r->n_tokens, r->lengths);
}

static void release(result_t *r) {
    free(r->merges);
    free(r->tokens);
    free(r->lengths);
}

static int same(const result_t *a, const result_t *b) {
    return a->n_done == b->n_done && a->n_tokens == b->n_tokens &&
           !memcmp(a->merges, b->merges, sizeof(uint32_t) * 3 * a->n_done) &&
           !memcmp(a->tokens, b->tokens, sizeof(uint32_t) * a->n_tokens) &&
           !memcmp(a->lengths, b->lengths, sizeof(uint64_t) * (a->n_done + 1));
}

static int fail(const char *what, uint64_t n) {
    printf("FAIL: %s (n = %llu)\n", what, (unsigned long long)n);
    return 1;
}

/* literal == chunks; encoder(training text) == training tokens; the
   longest-match tokens' strings concatenate to the text */
static int check_corpus(const uint8_t *b, uint64_t n, uint32_t m, int with_literal) {
    result_t lit = {0}, chk = {0};
    if (train(0, b, n, m, &chk) != 0) return fail("chunk oracle failed", n);
    if (with_literal) {
        if (train(1, b, n, m, &lit) != 0) return fail("literal oracle failed", n);
        if (!same(&lit, &chk)) return fail("literal and chunk oracles differ", n);
        release(&lit);
    }
    uint32_t k = chk.n_done;
    uint32_t *pairs = malloc(sizeof(uint32_t) * 2 * (k ? k : 1));
    uint32_t *counts = malloc(sizeof(uint32_t) * (k ? k : 1));
    uint32_t *enc = malloc(sizeof(uint32_t) * (n ? n : 1));
    uint32_t *ids = malloc(sizeof(uint32_t) * (n ? n : 1));
    uint64_t *len = malloc(sizeof(uint64_t) * (256 + k));
    if (!pairs || !counts || !enc || !ids || !len) return fail("allocation", n);
    for (uint32_t i = 0; i < k; i++) {
        pairs[2 * i] = chk.merges[3 * i];
        pairs[2 * i + 1] = chk.merges[3 * i + 1];
    }
    uint64_t ne = 0, nt = 0;
    if (oracle_encode(b, n, pairs, k, counts, enc, &ne) != 0) return fail("encoder failed", n);
    if (ne != chk.n_tokens || memcmp(enc, chk.tokens, sizeof(uint32_t) * ne))
        return fail("encoding the training text differs from training", n);
    for (uint32_t i = 0; i < k; i++)
        if (counts[i] != chk.merges[3 * i + 2]) return fail("encoder counts differ from training counts", n);
    if (oracle_trie_encode(b, n, pairs, k, ids, &nt) != 0) return fail("longest match failed", n);
    for (uint32_t i = 0; i < 256 + k; i++)
        len[i] = i < 256 ? 1 : len[pairs[2 * (i - 256)]] + len[pairs[2 * (i - 256) + 1]];
    uint64_t total = 0;
    for (uint64_t i = 0; i < nt; i++) total += len[ids[i]];
    if (total != n) return fail("longest-match tokens do not cover the text", n);
    free(pairs);
    free(counts);
    free(enc);
    free(ids);
    free(len);
    release(&chk);
    return 0;
}

int main(void) {
    static const uint8_t alpha[5] = {0x61, 0x62, 0x31, 0x20, 0xC3};
    uint8_t s[8];
    unsigned strings = 0;
    for (int L = 0; L <= 6; L++) {
        uint32_t total = 1;
        for (int i = 0; i < L; i++) total *= 5;
        for (uint32_t v = 0; v < total; v++) {
            uint32_t x = v;
            for (int i = 0; i < L; i++) {
                s[i] = alpha[x % 5];
                x /= 5;
            }
            result_t a = {0}, c = {0};
            if (train(1, s, (uint64_t)L, 8, &a) != 0 || train(0, s, (uint64_t)L, 8, &c) != 0)
                return fail("oracle failed on a short string", (uint64_t)L);
            if (!same(&a, &c)) return fail("literal and chunk oracles differ on a short string", (uint64_t)L);
            release(&a);
            release(&c);
            strings++;
        }
    }
    /* corpora of the five recipes (word lists, Turkish letters, mixed UTF-8,
       runs plus random bytes) at small sizes */
    static const uint64_t sizes[3] = {4093, 16384, 65537};
    uint8_t *buf = malloc(65537);
    if (!buf) return fail("allocation", 0);
    unsigned corpora = 0;
    for (int z = 0; z < 3; z++) {
        uint64_t n = sizes[z];
        for (int recipe = 0; recipe < 4; recipe++) {
            int rc;
            if (recipe < 3)
                rc = corpus_words(buf, n, 100 + 10 * z + recipe, 300, 1.1, 2, recipe == 1 ? 14 : 8, recipe, 0.03,
                                  0.02, 4);
            else
                rc = corpus_runs(buf, n, 200 + z, 64.0, 256.0);
            if (rc != 0) return fail("generator failed", n);
            if (check_corpus(buf, n, 120, n <= 16384)) return 1;
            corpora++;
        }
    }
    /* degenerate inputs: empty, one byte, a corpus with no countable pair */
    if (check_corpus(buf, 0, 5, 1) || check_corpus((const uint8_t *)"x", 1, 5, 1) ||
        check_corpus((const uint8_t *)"a1b2c3 ", 7, 5, 1))
        return 1;
    free(buf);
    printf("ok: %u short strings, %u corpora\n", strings, corpora);
    return 0;
}
