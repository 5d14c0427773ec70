/*
 * CPU oracles for BPE training (plain C, single-threaded).
 *
 * TEST INFRASTRUCTURE ONLY. The GPU library never links or calls this file;
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load it. It shares no code, header, table or constant with the GPU path.
 *
 * What is computed (page "bpe - GPU BPE Tokenizer Pipeline", llm.istanbul):
 *   - "Nedir bu ya?": repeat { find the most frequent adjacent pair, give it
 *     one new symbol }.
 *   - "Ne Yapar? 1": each byte gets a character class; a class change tags
 *     that symbol with WORD_START_BIT (0x10000); pairs are not counted
 *     across the bit.
 *   - "Satir Satir Analiz 1)": the class function.
 *   - page head, training pipeline: clear the table and count everything
 *     again each iteration, then a deterministic maximum.
 *   - "Ne Yapar? 3": the merged symbol carries WORD_START_BIT.
 * Open points are read as in oracle/reference.py (bit at position 0 and on
 * the right-hand symbol of a change, overlapping counts, ties to the
 * smallest (left, right), new id 256 + k, left-to-right non-overlapping
 * merge that never crosses the bit, left bit kept, tag once, stop when no
 * pair is left).
 *
 * Two oracles with one signature:
 *   oracle_train_literal - the definition as written: a full recount of the
 *                          whole sequence every iteration. O(n * merges).
 *   oracle_train_chunks  - the same result computed on the multiset of
 *                          distinct chunks (maximal runs between word-start
 *                          bits never interact), with pair counts kept up to
 *                          date by touching only chunks that contain the
 *                          merged pair, and a lazy max-heap for the argmax.
 *                          Pinned to the literal oracle by tests.
 *
 * And the encoder of the same method (text encoded with a learned merge
 * list, "Nedir bu ya?"):
 *   oracle_encode        - tag, then apply merge k = pairs[2k], pairs[2k+1]
 *                          (new id 256 + k) over the whole sequence, k in
 *                          order, each exactly as a training iteration
 *                          applies its pair; counts[k] = occurrences of the
 *                          pair just before merge k. O(n * merges).
 *
 * And inference ("Nedir bu ya?", inference paragraph; "Ne Yapar? 4"):
 *   oracle_trie_encode   - greedy longest match: from the current position,
 *                          emit the id of the longest vocabulary string the
 *                          text continues with there, move past it. The
 *                          vocabulary is the merge list's: id b < 256 is the
 *                          byte b, id 256 + k the string of pairs[2k]
 *                          followed by that of pairs[2k+1]; a string several
 *                          ids spell maps to the smallest. A plain pointer
 *                          trie (first child / next sibling lists).
 *
 * Outputs of both trainers:
 *   merges[3k+0..2] = left, right, count of merge k (new id 256 + k)
 *   tokens[0..*n_tokens) = final symbols, id | 0x10000 on chunk starts
 *   lengths[k] = sequence length before merge k, lengths[*n_done] = final
 * Return 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define O_WS 0x10000u
#define O_ID 0xFFFFu
#define O_BASE 256u
#define O_MAX_MERGES (0x10000u - O_BASE)

/* The page's byte classes ("Satir Satir Analiz 1)") as a table filled from
   the class members: ASCII letters and every byte >= 0x80 (UTF-8 letters stay
   letters) 0, ASCII digits 1, space 2, newline 4, all other bytes 3. */
static uint8_t class_of[256];
static int classes_ready;

static void fill_classes(void) {
    for (int b = 0; b < 256; b++) class_of[b] = 3;
    for (int b = 0; b < 26; b++) class_of['A' + b] = class_of['a' + b] = 0;
    for (int b = 0x80; b < 256; b++) class_of[b] = 0;
    for (int b = 0; b < 10; b++) class_of['0' + b] = 1;
    class_of[' '] = 2;
    class_of['\n'] = 4;
    classes_ready = 1;
}

uint32_t oracle_char_class(uint32_t x) {
    if (!classes_ready) fill_classes();
    return x < 256 ? class_of[x] : 0;
}

void oracle_tag(const uint8_t *b, uint64_t n, uint32_t *s) {
    for (uint64_t i = 0; i < n; i++) {
        int start = (i == 0) || oracle_char_class(b[i]) != oracle_char_class(b[i - 1]);
        s[i] = (uint32_t)b[i] | (start ? O_WS : 0u);
    }
}

static inline uint32_t pair_key(uint32_t l, uint32_t r) { return (l << 16) | r; }

static uint64_t next_pow2(uint64_t v) {
    uint64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

static inline uint64_t mix64(uint64_t x) {
    x ^= x >> 33; x *= 0xff51afd7ed558ccdULL;
    x ^= x >> 33; x *= 0xc4ceb9fe1a85ec53ULL;
    x ^= x >> 33;
    return x;
}

/* ======================================================================== */
/* literal oracle                                                            */

int oracle_train_literal(const uint8_t *b, uint64_t n, uint32_t n_merges, uint32_t *merges,
                         uint32_t *n_done, uint32_t *tokens, uint64_t *n_tokens, uint64_t *lengths) {
    if ((!b && n) || !merges || !n_done || !n_tokens || n_merges > O_MAX_MERGES) return -1;
    uint32_t *s = (uint32_t *)malloc(sizeof(uint32_t) * (n ? n : 1));
    uint32_t *t = (uint32_t *)malloc(sizeof(uint32_t) * (n ? n : 1));
    uint64_t cap = next_pow2(2 * n + 16);
    uint64_t *mkey = (uint64_t *)malloc(sizeof(uint64_t) * cap); /* UINT64_MAX = empty */
    uint64_t *mcnt = (uint64_t *)malloc(sizeof(uint64_t) * cap);
    if (!s || !t || !mkey || !mcnt) { free(s); free(t); free(mkey); free(mcnt); return -2; }
    oracle_tag(b, n, s);
    uint64_t len = n;
    uint32_t k = 0;
    for (; k < n_merges; k++) {
        if (lengths) lengths[k] = len;
        /* clear the table and count every adjacent pair again */
        memset(mkey, 0xFF, sizeof(uint64_t) * cap);
        uint64_t used = 0;
        for (uint64_t i = 1; i < len; i++) {
            if (s[i] & O_WS) continue;
            uint32_t key = pair_key(s[i - 1] & O_ID, s[i] & O_ID);
            uint64_t h = mix64(key) & (cap - 1);
            while (mkey[h] != UINT64_MAX && mkey[h] != key) h = (h + 1) & (cap - 1);
            if (mkey[h] == UINT64_MAX) { mkey[h] = key; mcnt[h] = 0; used++; }
            mcnt[h]++;
        }
        if (used == 0) break;
        /* deterministic maximum: highest count, then smallest key */
        uint64_t best_cnt = 0; uint32_t best_key = 0;
        for (uint64_t h = 0; h < cap; h++) {
            if (mkey[h] == UINT64_MAX) continue;
            uint32_t key = (uint32_t)mkey[h];
            if (mcnt[h] > best_cnt || (mcnt[h] == best_cnt && key < best_key)) {
                best_cnt = mcnt[h]; best_key = key;
            }
        }
        uint32_t L = best_key >> 16, R = best_key & O_ID, X = O_BASE + k;
        merges[3 * k + 0] = L; merges[3 * k + 1] = R; merges[3 * k + 2] = (uint32_t)best_cnt;
        /* left-to-right, non-overlapping, never across a word start */
        uint64_t o = 0;
        for (uint64_t i = 0; i < len;) {
            if (i + 1 < len && !(s[i + 1] & O_WS) && (s[i] & O_ID) == L && (s[i + 1] & O_ID) == R) {
                t[o++] = X | (s[i] & O_WS);
                i += 2;
            } else {
                t[o++] = s[i];
                i += 1;
            }
        }
        uint32_t *tmp = s; s = t; t = tmp;
        len = o;
    }
    if (lengths) lengths[k] = len;
    *n_done = k;
    *n_tokens = len;
    if (tokens) memcpy(tokens, s, sizeof(uint32_t) * len);
    free(s); free(t); free(mkey); free(mcnt);
    return 0;
}

/* ======================================================================== */
/* chunk-multiset oracle                                                     */

typedef struct {
    uint32_t *sym;   /* current ids of this distinct chunk (no flag bits) */
    uint32_t len;
    uint32_t stamp;  /* last iteration that touched it, plus one */
    uint64_t freq;   /* occurrences in the corpus */
} ochunk_t;

typedef struct {
    int64_t count;
    uint32_t *list;  /* chunks that (may) contain this pair; may hold duplicates */
    uint32_t nlist, caplist;
    uint32_t dirty;  /* iteration stamp, plus one */
} opair_t;

typedef struct {
    uint64_t *keys;  /* UINT64_MAX = empty; else pair key */
    uint32_t *ids;   /* index into pairs[] */
    uint64_t cap, used;
    opair_t *pairs;
    uint32_t npairs, cappairs;
} opairmap_t;

static int pm_init(opairmap_t *m, uint64_t cap) {
    m->cap = next_pow2(cap < 1024 ? 1024 : cap);
    m->used = 0;
    m->keys = (uint64_t *)malloc(sizeof(uint64_t) * m->cap);
    m->ids = (uint32_t *)malloc(sizeof(uint32_t) * m->cap);
    m->cappairs = 1024; m->npairs = 0;
    m->pairs = (opair_t *)malloc(sizeof(opair_t) * m->cappairs);
    if (!m->keys || !m->ids || !m->pairs) return -2;
    memset(m->keys, 0xFF, sizeof(uint64_t) * m->cap);
    return 0;
}

static void pm_free(opairmap_t *m) {
    for (uint32_t i = 0; i < m->npairs; i++) free(m->pairs[i].list);
    free(m->keys); free(m->ids); free(m->pairs);
}

static int pm_grow(opairmap_t *m) {
    uint64_t ncap = m->cap * 2;
    uint64_t *nk = (uint64_t *)malloc(sizeof(uint64_t) * ncap);
    uint32_t *ni = (uint32_t *)malloc(sizeof(uint32_t) * ncap);
    if (!nk || !ni) { free(nk); free(ni); return -2; }
    memset(nk, 0xFF, sizeof(uint64_t) * ncap);
    for (uint64_t h = 0; h < m->cap; h++) {
        if (m->keys[h] == UINT64_MAX) continue;
        uint64_t g = mix64(m->keys[h]) & (ncap - 1);
        while (nk[g] != UINT64_MAX) g = (g + 1) & (ncap - 1);
        nk[g] = m->keys[h]; ni[g] = m->ids[h];
    }
    free(m->keys); free(m->ids);
    m->keys = nk; m->ids = ni; m->cap = ncap;
    return 0;
}

/* pair record for key, created (count 0) if absent; NULL on allocation failure */
static opair_t *pm_get(opairmap_t *m, uint32_t key) {
    uint64_t h = mix64(key) & (m->cap - 1);
    while (m->keys[h] != UINT64_MAX) {
        if (m->keys[h] == key) return &m->pairs[m->ids[h]];
        h = (h + 1) & (m->cap - 1);
    }
    if (2 * (m->used + 1) > m->cap) {
        if (pm_grow(m)) return NULL;
        return pm_get(m, key);
    }
    if (m->npairs == m->cappairs) {
        uint32_t nc = m->cappairs * 2;
        opair_t *np = (opair_t *)realloc(m->pairs, sizeof(opair_t) * nc);
        if (!np) return NULL;
        m->pairs = np; m->cappairs = nc;
    }
    opair_t *p = &m->pairs[m->npairs];
    memset(p, 0, sizeof *p);
    m->keys[h] = key; m->ids[h] = m->npairs++; m->used++;
    return p;
}

static int pair_list_add(opair_t *p, uint32_t c) {
    if (p->nlist == p->caplist) {
        uint32_t nc = p->caplist ? p->caplist * 2 : 4;
        uint32_t *nl = (uint32_t *)realloc(p->list, sizeof(uint32_t) * nc);
        if (!nl) return -2;
        p->list = nl; p->caplist = nc;
    }
    p->list[p->nlist++] = c;
    return 0;
}

/* max-heap on (count desc, key asc); entries may be stale */
typedef struct { int64_t count; uint32_t key; } oheap_e;
typedef struct { oheap_e *a; uint64_t n, cap; } oheap_t;

static inline int heap_before(oheap_e x, oheap_e y) {
    return x.count > y.count || (x.count == y.count && x.key < y.key);
}

static int heap_push(oheap_t *h, int64_t count, uint32_t key) {
    if (h->n == h->cap) {
        uint64_t nc = h->cap ? h->cap * 2 : 1024;
        oheap_e *na = (oheap_e *)realloc(h->a, sizeof(oheap_e) * nc);
        if (!na) return -2;
        h->a = na; h->cap = nc;
    }
    uint64_t i = h->n++;
    oheap_e e = {count, key};
    while (i > 0) {
        uint64_t p = (i - 1) / 2;
        if (!heap_before(e, h->a[p])) break;
        h->a[i] = h->a[p];
        i = p;
    }
    h->a[i] = e;
    return 0;
}

static oheap_e heap_pop(oheap_t *h) {
    oheap_e top = h->a[0];
    oheap_e e = h->a[--h->n];
    uint64_t i = 0;
    for (;;) {
        uint64_t l = 2 * i + 1, r = l + 1, b = i;
        oheap_e be = e;
        if (l < h->n && heap_before(h->a[l], be)) { b = l; be = h->a[l]; }
        if (r < h->n && heap_before(h->a[r], be)) { b = r; be = h->a[r]; }
        if (b == i) break;
        h->a[i] = h->a[b];
        i = b;
    }
    if (h->n) h->a[i] = e;
    return top;
}

/* distinct-chunk dictionary keyed by the chunk's bytes */
typedef struct {
    uint64_t *hash;  /* 0 = empty (hashes are forced non-zero) */
    uint32_t *idx;
    uint64_t cap;
} odict_t;

static int dict_grow(odict_t *d) {
    uint64_t ncap = d->cap * 2;
    uint64_t *nh = (uint64_t *)calloc(ncap, sizeof(uint64_t));
    uint32_t *ni = (uint32_t *)malloc(sizeof(uint32_t) * ncap);
    if (!nh || !ni) { free(nh); free(ni); return -2; }
    for (uint64_t h = 0; h < d->cap; h++) {
        if (!d->hash[h]) continue;
        uint64_t g = d->hash[h] & (ncap - 1);
        while (nh[g]) g = (g + 1) & (ncap - 1);
        nh[g] = d->hash[h]; ni[g] = d->idx[h];
    }
    free(d->hash); free(d->idx);
    d->hash = nh; d->idx = ni; d->cap = ncap;
    return 0;
}

static uint64_t bytes_hash(const uint8_t *p, uint32_t len) {
    uint64_t h = 0xcbf29ce484222325ULL; /* FNV-1a 64 */
    for (uint32_t i = 0; i < len; i++) { h ^= p[i]; h *= 0x100000001b3ULL; }
    h = mix64(h ^ len);
    return h ? h : 1;
}

int oracle_train_chunks(const uint8_t *b, uint64_t n, uint32_t n_merges, uint32_t *merges,
                        uint32_t *n_done, uint32_t *tokens, uint64_t *n_tokens, uint64_t *lengths) {
    if ((!b && n) || !merges || !n_done || !n_tokens || n_merges > O_MAX_MERGES) return -1;
    int rc = -2;
    /* 1. chunk boundaries: a chunk starts where the word-start bit would be set */
    uint64_t nocc = 0;
    for (uint64_t i = 0; i < n; i++)
        if (i == 0 || oracle_char_class(b[i]) != oracle_char_class(b[i - 1])) nocc++;
    uint32_t *seq = (uint32_t *)malloc(sizeof(uint32_t) * (nocc ? nocc : 1));
    uint64_t *first = NULL;  /* byte offset of each distinct chunk's first occurrence */
    uint32_t *blen = NULL;   /* byte length of each distinct chunk */
    ochunk_t *ch = NULL;
    uint32_t nch = 0, capch = 0;
    odict_t d = {0};
    opairmap_t pm = {0};
    oheap_t heap = {0};
    uint32_t *work = NULL;
    if (!seq) goto out;
    d.cap = 1ULL << 16;
    d.hash = (uint64_t *)calloc(d.cap, sizeof(uint64_t));
    d.idx = (uint32_t *)malloc(sizeof(uint32_t) * d.cap);
    if (!d.hash || !d.idx) goto out;

    /* 2. deduplicate chunks by their bytes and count their frequencies */
    uint64_t occ = 0;
    for (uint64_t i = 0; i < n;) {
        uint64_t j = i + 1;
        while (j < n && oracle_char_class(b[j]) == oracle_char_class(b[i])) j++;
        uint32_t len = (uint32_t)(j - i);
        uint64_t hv = bytes_hash(b + i, len);
        uint64_t h = hv & (d.cap - 1);
        uint32_t id = UINT32_MAX;
        while (d.hash[h]) {
            if (d.hash[h] == hv) {
                uint32_t c = d.idx[h];
                if (blen[c] == len && memcmp(b + first[c], b + i, len) == 0) { id = c; break; }
            }
            h = (h + 1) & (d.cap - 1);
        }
        if (id == UINT32_MAX && 2 * ((uint64_t)nch + 1) > d.cap) {
            if (dict_grow(&d)) goto out;
            h = hv & (d.cap - 1);
            while (d.hash[h]) h = (h + 1) & (d.cap - 1);
        }
        if (id == UINT32_MAX) {
            if (nch == capch) {
                uint32_t nc = capch ? capch * 2 : 4096;
                ochunk_t *nchp = (ochunk_t *)realloc(ch, sizeof(ochunk_t) * nc);
                if (!nchp) goto out;
                ch = nchp;
                uint64_t *nf = (uint64_t *)realloc(first, sizeof(uint64_t) * nc);
                if (!nf) goto out;
                first = nf;
                uint32_t *nb = (uint32_t *)realloc(blen, sizeof(uint32_t) * nc);
                if (!nb) goto out;
                blen = nb;
                capch = nc;
            }
            id = nch++;
            first[id] = i; blen[id] = len;
            ch[id].len = len; ch[id].freq = 0; ch[id].stamp = 0;
            ch[id].sym = (uint32_t *)malloc(sizeof(uint32_t) * len);
            if (!ch[id].sym) goto out;
            for (uint32_t q = 0; q < len; q++) ch[id].sym[q] = b[i + q];
            d.hash[h] = hv; d.idx[h] = id;
        }
        ch[id].freq++;
        seq[occ++] = id;
        i = j;
    }
    free(d.hash); d.hash = NULL;
    free(d.idx); d.idx = NULL;

    /* 3. exact pair counts over the multiset, and pair -> chunk lists */
    if (pm_init(&pm, 4096)) goto out;
    for (uint32_t c = 0; c < nch; c++) {
        for (uint32_t q = 1; q < ch[c].len; q++) {
            opair_t *p = pm_get(&pm, pair_key(ch[c].sym[q - 1], ch[c].sym[q]));
            if (!p) goto out;
            p->count += (int64_t)ch[c].freq;
            if (p->nlist == 0 || p->list[p->nlist - 1] != c)
                if (pair_list_add(p, c)) goto out;
        }
    }
    for (uint64_t h = 0; h < pm.cap; h++) {
        if (pm.keys[h] == UINT64_MAX) continue;
        opair_t *p = &pm.pairs[pm.ids[h]];
        if (p->count > 0 && heap_push(&heap, p->count, (uint32_t)pm.keys[h])) goto out;
    }

    /* 4. merge loop */
    uint64_t total = n;
    uint32_t *dirty = NULL; uint32_t ndirty = 0, capdirty = 0;
    uint32_t maxlen = 1;
    for (uint32_t c = 0; c < nch; c++) if (ch[c].len > maxlen) maxlen = ch[c].len;
    work = (uint32_t *)malloc(sizeof(uint32_t) * maxlen);
    if (!work) goto out;
    uint32_t k = 0;
    for (; k < n_merges; k++) {
        if (lengths) lengths[k] = total;
        /* argmax: pop until an entry matches the current count */
        uint32_t best = 0; int64_t bcount = 0; int found = 0;
        while (heap.n) {
            oheap_e e = heap_pop(&heap);
            opair_t *p = pm_get(&pm, e.key);
            if (!p) goto out_dirty;
            if (p->count > 0 && p->count == e.count) { best = e.key; bcount = e.count; found = 1; break; }
        }
        if (!found) break;
        uint32_t L = best >> 16, R = best & O_ID, X = O_BASE + k;
        merges[3 * k + 0] = L; merges[3 * k + 1] = R; merges[3 * k + 2] = (uint32_t)bcount;
        ndirty = 0;
        opair_t *bp = pm_get(&pm, best);
        uint32_t nl = bp->nlist;
        uint32_t *lst = bp->list;
        bp->list = NULL; bp->nlist = 0; bp->caplist = 0;
        for (uint32_t li = 0; li < nl; li++) {
            uint32_t c = lst[li];
            ochunk_t *C = &ch[c];
            if (C->stamp == k + 1) continue;
            C->stamp = k + 1;
            int has = 0;
            for (uint32_t q = 1; q < C->len; q++)
                if (C->sym[q - 1] == L && C->sym[q] == R) { has = 1; break; }
            if (!has) continue;
            /* remove this chunk's pairs, merge, add its new pairs back */
            for (uint32_t q = 1; q < C->len; q++) {
                uint32_t key = pair_key(C->sym[q - 1], C->sym[q]);
                opair_t *p = pm_get(&pm, key);
                if (!p) { free(lst); goto out_dirty; }
                p->count -= (int64_t)C->freq;
                if (p->dirty != k + 1) {
                    p->dirty = k + 1;
                    if (ndirty == capdirty) {
                        capdirty = capdirty ? capdirty * 2 : 1024;
                        uint32_t *nd = (uint32_t *)realloc(dirty, sizeof(uint32_t) * capdirty);
                        if (!nd) { free(lst); goto out_dirty; }
                        dirty = nd;
                    }
                    dirty[ndirty++] = key;
                }
            }
            uint32_t o = 0;
            for (uint32_t q = 0; q < C->len;) {
                if (q + 1 < C->len && C->sym[q] == L && C->sym[q + 1] == R) { work[o++] = X; q += 2; }
                else { work[o++] = C->sym[q]; q += 1; }
            }
            total -= (uint64_t)(C->len - o) * C->freq;
            memcpy(C->sym, work, sizeof(uint32_t) * o);
            C->len = o;
            for (uint32_t q = 1; q < C->len; q++) {
                uint32_t key = pair_key(C->sym[q - 1], C->sym[q]);
                opair_t *p = pm_get(&pm, key);
                if (!p) { free(lst); goto out_dirty; }
                p->count += (int64_t)C->freq;
                if (p->dirty != k + 1) {
                    p->dirty = k + 1;
                    if (ndirty == capdirty) {
                        capdirty = capdirty ? capdirty * 2 : 1024;
                        uint32_t *nd = (uint32_t *)realloc(dirty, sizeof(uint32_t) * capdirty);
                        if (!nd) { free(lst); goto out_dirty; }
                        dirty = nd;
                    }
                    dirty[ndirty++] = key;
                }
                /* only pairs with the new id are new to this chunk */
                if ((C->sym[q - 1] == X || C->sym[q] == X) && (p->nlist == 0 || p->list[p->nlist - 1] != c))
                    if (pair_list_add(p, c)) { free(lst); goto out_dirty; }
            }
        }
        free(lst);
        for (uint32_t q = 0; q < ndirty; q++) {
            opair_t *p = pm_get(&pm, dirty[q]);
            if (!p) goto out_dirty;
            if (p->count > 0 && heap_push(&heap, p->count, dirty[q])) goto out_dirty;
        }
    }
    if (lengths) lengths[k] = total;
    *n_done = k;

    /* 5. expand the chunk sequence back to the token sequence */
    {
        uint64_t o = 0;
        for (uint64_t i = 0; i < occ; i++) {
            const ochunk_t *C = &ch[seq[i]];
            if (tokens) {
                tokens[o] = C->sym[0] | O_WS;
                for (uint32_t q = 1; q < C->len; q++) tokens[o + q] = C->sym[q];
            }
            o += C->len;
        }
        *n_tokens = o;
    }
    rc = 0;
out_dirty:
    free(dirty);
out:
    free(work);
    free(heap.a);
    if (pm.keys) pm_free(&pm);
    free(d.hash); free(d.idx);
    if (ch) for (uint32_t c = 0; c < nch; c++) free(ch[c].sym);
    free(ch); free(first); free(blen); free(seq);
    return rc;
}

/* ======================================================================== */
/* encoder                                                                   */

int oracle_encode(const uint8_t *b, uint64_t n, const uint32_t *pairs, uint32_t n_merges, uint32_t *counts,
                  uint32_t *tokens, uint64_t *n_tokens) {
    if ((!b && n) || (!pairs && n_merges) || !n_tokens || n_merges > O_MAX_MERGES) return -1;
    for (uint32_t k = 0; k < n_merges; k++)
        if (pairs[2 * k] >= O_BASE + k || pairs[2 * k + 1] >= O_BASE + k) return -1;
    uint32_t *s = (uint32_t *)malloc(sizeof(uint32_t) * (n ? n : 1));
    uint32_t *t = (uint32_t *)malloc(sizeof(uint32_t) * (n ? n : 1));
    if (!s || !t) { free(s); free(t); return -2; }
    oracle_tag(b, n, s);
    uint64_t len = n;
    for (uint32_t k = 0; k < n_merges; k++) {
        const uint32_t L = pairs[2 * k], R = pairs[2 * k + 1], X = O_BASE + k;
        uint32_t c = 0;
        for (uint64_t i = 1; i < len; i++)
            if (!(s[i] & O_WS) && (s[i - 1] & O_ID) == L && (s[i] & O_ID) == R) c++;
        if (counts) counts[k] = c;
        uint64_t o = 0;
        for (uint64_t i = 0; i < len;) {
            if (i + 1 < len && !(s[i + 1] & O_WS) && (s[i] & O_ID) == L && (s[i + 1] & O_ID) == R) {
                t[o++] = X | (s[i] & O_WS);
                i += 2;
            } else {
                t[o++] = s[i];
                i += 1;
            }
        }
        uint32_t *tmp = s; s = t; t = tmp;
        len = o;
    }
    *n_tokens = len;
    if (tokens) memcpy(tokens, s, sizeof(uint32_t) * len);
    free(s); free(t);
    return 0;
}

/* ======================================================================== */
/* greedy longest-match inference                                            */

typedef struct {
    int32_t first;    /* first child, -1 if none          */
    int32_t next;     /* next sibling, -1 if none         */
    int32_t tok;      /* id spelled by the path, -1 if none */
    uint8_t byte;     /* edge label from the parent        */
} tnode_t;

typedef struct {
    tnode_t *v;
    uint64_t n, cap;
} ttrie_t;

static int64_t tt_child(const ttrie_t *t, int64_t node, uint8_t c) {
    for (int32_t k = t->v[node].first; k >= 0; k = t->v[k].next)
        if (t->v[k].byte == c) return k;
    return -1;
}

static int64_t tt_add(ttrie_t *t, int64_t node, uint8_t c) {
    int64_t k = tt_child(t, node, c);
    if (k >= 0) return k;
    if (t->n == t->cap) {
        uint64_t cap = t->cap ? 2 * t->cap : 1024;
        tnode_t *v = (tnode_t *)realloc(t->v, sizeof(tnode_t) * cap);
        if (!v) return -2;
        t->v = v;
        t->cap = cap;
    }
    k = (int64_t)t->n++;
    t->v[k].first = -1;
    t->v[k].tok = -1;
    t->v[k].byte = c;
    t->v[k].next = t->v[node].first;
    t->v[node].first = (int32_t)k;
    return k;
}

/* Returns 0, -1 on bad arguments (an id that does not exist yet), -2 on
   allocation failure or a vocabulary too large for 32-bit node indexes. */
int oracle_trie_encode(const uint8_t *b, uint64_t n, const uint32_t *pairs, uint32_t n_merges, uint32_t *tokens,
                       uint64_t *n_tokens) {
    if ((!b && n) || (!pairs && n_merges) || !n_tokens || n_merges > O_MAX_MERGES) return -1;
    const uint32_t nv = O_BASE + n_merges;
    uint64_t *off = (uint64_t *)malloc(sizeof(uint64_t) * nv);
    uint64_t *len = (uint64_t *)malloc(sizeof(uint64_t) * nv);
    if (!off || !len) { free(off); free(len); return -2; }
    uint64_t total = 0;
    for (uint32_t i = 0; i < nv; i++) {
        if (i < O_BASE) {
            len[i] = 1;
        } else {
            const uint32_t k = i - O_BASE, l = pairs[2 * k], r = pairs[2 * k + 1];
            if (l >= i || r >= i) { free(off); free(len); return -1; }
            len[i] = len[l] + len[r];
        }
        off[i] = total;
        total += len[i];
        if (total > ((uint64_t)1 << 31)) { free(off); free(len); return -2; }
    }
    uint8_t *pool = (uint8_t *)malloc(total ? total : 1);
    if (!pool) { free(off); free(len); return -2; }
    for (uint32_t i = 0; i < nv; i++) {
        if (i < O_BASE) {
            pool[off[i]] = (uint8_t)i;
        } else {
            const uint32_t k = i - O_BASE, l = pairs[2 * k], r = pairs[2 * k + 1];
            memcpy(pool + off[i], pool + off[l], len[l]);
            memcpy(pool + off[i] + len[l], pool + off[r], len[r]);
        }
    }
    ttrie_t t = {(tnode_t *)malloc(sizeof(tnode_t) * 1024), 0, 1024};
    int rc = t.v ? 0 : -2;
    if (!rc) {  /* node 0 is the root */
        t.n = 1;
        t.v[0].first = -1; t.v[0].next = -1; t.v[0].tok = -1; t.v[0].byte = 0;
    }
    for (uint32_t i = 0; i < nv && !rc; i++) {
        int64_t node = 0;
        for (uint64_t j = 0; j < len[i]; j++) {
            node = tt_add(&t, node, pool[off[i] + j]);
            if (node < 0 || t.n > 0x7FFFFFFFu) { rc = -2; break; }
        }
        if (!rc && t.v[node].tok < 0) t.v[node].tok = (int32_t)i;   /* smallest id keeps the string */
    }
    uint64_t o = 0;
    for (uint64_t i = 0; i < n && !rc;) {
        int64_t node = 0, best = -1;
        uint64_t best_len = 0;
        for (uint64_t j = i; j < n; j++) {
            node = tt_child(&t, node, b[j]);
            if (node < 0) break;
            if (t.v[node].tok >= 0) { best = t.v[node].tok; best_len = j - i + 1; }
        }
        /* every byte is a token, so best_len >= 1 */
        if (tokens) tokens[o] = (uint32_t)best;
        o++;
        i += best_len;
    }
    *n_tokens = o;
    free(t.v); free(pool); free(off); free(len);
    return rc;
}
