/*
 * bpe.h - C ABI of an MI355X (gfx950) library for byte-level BPE training.
 *
 * The operation is the training loop of the page "bpe - GPU BPE Tokenizer
 * Pipeline (Egitim + Cikarim)" (llm.istanbul/learn/tr/13_bpe):
 *   - "Nedir bu ya?": repeatedly find the most frequent adjacent pair of
 *     symbols and give it one new symbol;
 *   - "Ne Yapar? 1": each byte gets a character class (Letter, Digit,
 *     Space, Punct, Newline; "Satir Satir Analiz 1)" prints the function);
 *     at a class change the symbol is tagged with WORD_START_BIT 0x10000
 *     and pairs are never counted across the tag;
 *   - page head, training pipeline: every iteration clears the pair table,
 *     counts all pairs again, takes a deterministic maximum, merges, and
 *     compacts the symbol array with a prefix scan ("Ne Yapar? 3");
 *   - "Ne Yapar? 3": the merged symbol carries WORD_START_BIT.
 * Readings of points the page leaves open:
 *   - the first symbol carries the tag, and the tag sits on the right-hand
 *     symbol of a class change;
 *   - every adjacent position counts, overlapping ones included
 *     ("aaa" counts (a,a) twice);
 *   - the maximum breaks ties to the smallest (left, right);
 *   - merge k creates id 256 + k;
 *   - merging is left to right and non-overlapping, so a run of identical
 *     pairs merges its 1st, 3rd, 5th ... occurrence;
 *   - the merged symbol keeps the left symbol's tag;
 *   - tagging happens once, before the first iteration;
 *   - training stops early when no countable pair is left.
 * The counts are those of a full recount, but they are not recounted: the
 * library counts once (after tagging) into a global table and then, at
 * every merge, subtracts the old pairs that touch a changed position and
 * adds the new pairs that touch the new symbol. Every other adjacency is
 * the same before and after the merge, so the table stays exact.
 *
 * Tokens are uint32: bits 0-15 hold the id, bit 16 the word-start tag,
 * bits 17-31 are zero. Ids fit in 16 bits, hence BPE_MAX_MERGES. Between
 * iterations the device holds 16-bit ids alone: a word is a maximal run of
 * one byte class and every token lies inside one word, so a token's tag is
 * a change of class from the token before it (or position 0), which the
 * library derives from a per-id class table when tokens are read out.
 *
 * Pointers: arguments named "bytes", "merges", "tokens" and "lengths" may be
 * host or device pointers (device memory of the state's GPU); the library
 * tells them apart with hipPointerGetAttributes. Output arrays are owned by
 * the caller. A state and its workspace are owned by the library unless the
 * caller passes a workspace in bpe_config, which must then outlive the state.
 * No call throws, aborts or exits; each returns a bpe_status, and
 * bpe_last_error() gives a thread-local message for the last failure.
 * One state must not be used from two threads at once; separate states may.
 */
#ifndef BPE_H
#define BPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BPE_OK = 0,         /* success                                                  */
    BPE_DONE = 1,       /* bpe_step: no countable pair is left, nothing merged      */
    BPE_EINVAL = -1,    /* bad argument (null pointer, size out of range, ...)      */
    BPE_ETABLE = -2,    /* the global pair table overflowed; use a larger table     */
    BPE_EIDSPACE = -3,  /* more than BPE_MAX_MERGES merges requested                */
    BPE_ENOMEM = -4,    /* device or host allocation failed                         */
    BPE_EHIP = -5,      /* a HIP runtime call failed (detail in bpe_last_error)     */
    BPE_ESTATE = -6     /* the state holds a device-side error from an earlier call */
} bpe_status;

#define BPE_WORD_START 0x10000u
#define BPE_ID_MASK 0xFFFFu
#define BPE_BASE_VOCAB 256u
#define BPE_MAX_MERGES 65280u            /* 0x10000 - 256: ids stay within 16 bits */
#define BPE_MAX_BYTES 0x7FFFFFFFull      /* corpus size limit (2^31 - 1 bytes)     */

/* One learned merge: (left, right) became id 256 + its index; count is the
   number of adjacent (left, right) positions counted when it was chosen. */
typedef struct {
    uint32_t left, right, count;
} bpe_merge;

typedef struct {
    uint32_t table_log2;     /* global pair table of 2^table_log2 slots (8 B each);
                                otherwise 10..30; 0 = automatic: room under the 7/8
                                limit for min(3n, 65536 + 512 * merges) keys, where
                                merges is bpe_train's n_merges (BPE_MAX_MERGES for
                                bpe_init and bpe_workspace_bytes). Claimed keys never
                                exceed 3n; an overflow is BPE_ETABLE, never a dropped
                                count.                                                 */
    uint32_t flags;          /* 0, or BPE_FLAG_OVERSUBSCRIBE (a testing aid)           */
    void *stream;            /* hipStream_t all work is ordered on; NULL = the state
                                creates and owns a blocking stream (ordered after the
                                legacy default stream)                                 */
    void *workspace;         /* device memory of at least bpe_workspace_bytes();
                                NULL = the state allocates its own                     */
    size_t workspace_bytes;  /* size of workspace (ignored when workspace is NULL)     */
} bpe_config;

/* Testing aid for bpe_config.flags: launch each merge pass with four times
   as many workgroups as the device can hold at once, so that most of them
   start only after earlier ones have finished. Results do not change: no
   workgroup of a pass ever waits for one that has not started (see
   bpe_run). Slower; for tests only. */
#define BPE_FLAG_OVERSUBSCRIBE 1u

/* For bpe_train_chunked (other calls ignore it): always train over the
   distinct words, whatever memory their records take (testing aid). */
#define BPE_FLAG_ALWAYS_CHUNKS 2u

typedef struct bpe_state bpe_state;

/* Device workspace needed for a corpus of n bytes with this config (cfg may be
   NULL for defaults; an automatic table is sized for up to BPE_MAX_MERGES
   merges, so the result also suffices for bpe_train with any n_merges).
   Host arithmetic only; 0 if n or the config is invalid. */
size_t bpe_workspace_bytes(size_t n, const bpe_config *cfg);

/*
 * Train up to n_merges merges on bytes[0..n) and return the result: the loop
 * of "Nedir bu ya?" (most frequent adjacent pair -> one new symbol) run
 * n_merges times over the symbols tagged as in "Ne Yapar? 1", each
 * iteration the training pipeline of the page head (count, deterministic
 * maximum, merge, prefix-scan compaction of "Ne Yapar? 3").
 *   merges    out, n_merges entries (host or device); merge i creates id 256 + i
 *   n_done    out (host): merges produced; < n_merges if no pair was left
 *   tokens    out (host or device) or NULL: final symbols, id | tag
 *   tokens_cap  capacity of tokens in elements (n always suffices)
 *   n_tokens  out (host) or NULL: number of final symbols
 * Blocks until the result is available. Equivalent to bpe_init + bpe_run +
 * bpe_sync + bpe_merges + bpe_tokens + bpe_free. n == 0 is valid (no merges,
 * no tokens). Errors: BPE_EINVAL, BPE_EIDSPACE (n_merges > BPE_MAX_MERGES),
 * BPE_ETABLE (table overflow; nothing partial is returned), BPE_ENOMEM, BPE_EHIP.
 */
bpe_status bpe_train(const uint8_t *bytes, size_t n, uint32_t n_merges, const bpe_config *cfg,
                     bpe_merge *merges, uint32_t *n_done, uint32_t *tokens, size_t tokens_cap,
                     size_t *n_tokens);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): bpe_train
   on a workspace that lives in the library itself, a file-scope device
   array of BPE_STATIC_SCRATCH_BYTES that every device the library runs on
   holds until the process ends. Nothing is allocated on the device or the
   host (no stream is created: stream is the caller's hipStream_t, NULL for
   the null stream; the workspace is cleared by kernels at the start of
   each call). Limits: n <= BPE_STATIC_MAX_BYTES and a pair table of at most
   2^BPE_STATIC_MAX_TABLE_LOG2 slots (table_log2 0 = automatic, capped
   there); beyond them BPE_EINVAL with a message. All calls on one device
   share the array, which keeps the last call's contents: calls that
   overlap on one device (from two threads, or on two streams) race and
   must not be made. Pointers and results as bpe_train; blocks until done.
   Errors as bpe_train. */
#define BPE_STATIC_SCRATCH_BYTES (32u << 20)
#define BPE_STATIC_MAX_BYTES (2u << 20)
#define BPE_STATIC_MAX_TABLE_LOG2 20u
bpe_status bpe_train_static(const uint8_t *bytes, size_t n, uint32_t n_merges, uint32_t table_log2, void *stream,
                            bpe_merge *merges, uint32_t *n_done, uint32_t *tokens, size_t tokens_cap,
                            size_t *n_tokens);

/*
 * bpe_train's results computed from the corpus's distinct words. Pairs are
 * counted within words and merges never cross a word start (page "bpe - GPU
 * BPE Tokenizer Pipeline", "Ne Yapar? 1" and "Nedir bu ya?"), so all
 * occurrences of a word are rewritten alike and a pair's count is the sum,
 * over the distinct words holding it, of the word's frequency times the
 * pair's occurrences in it. Training runs on each distinct word of 2..32
 * bytes once, with that weight (a word the word table cannot hold, longer
 * ones included, is kept once per occurrence): the same counts, so the same
 * merges, ties and counts included. The tokens are the learned list applied
 * to the same bytes by the encoder (bpe_encoder_encode), which gives the
 * training tokens. Arguments and results as bpe_train: merges (host or
 * device), n_done (host), tokens (host or device, or NULL), tokens_cap,
 * n_tokens (host, or NULL); cfg->table_log2 sizes the pair table as for
 * bpe_train (a corpus of at most 1,024 distinct words, none longer than 32
 * bytes, is trained in one workgroup's LDS, without it), cfg->stream
 * orders the work (NULL: a stream of its own), cfg->flags may hold
 * BPE_FLAG_ALWAYS_CHUNKS (other bits as for bpe_train), and cfg->workspace
 * must be NULL: the call allocates its own device memory (the word table,
 * 76 bytes per distinct word of at most 32 bytes, 2 bytes per symbol of a
 * longer word, the pair table with 24 more bytes per slot for the pairs'
 * chunk lists, and up to 256 bytes per distinct word for the lists
 * themselves) and frees it before returning. Where the distinct words'
 * records would take more than 8 bytes per input byte (text with few
 * repeated words, where the full array is faster), it runs bpe_train
 * instead.
 * Blocks until done. Errors as bpe_train, and as bpe_encoder_encode for the
 * tokens.
 */
bpe_status bpe_train_chunked(const uint8_t *bytes, size_t n, uint32_t n_merges, const bpe_config *cfg,
                             bpe_merge *merges, uint32_t *n_done, uint32_t *tokens, size_t tokens_cap,
                             size_t *n_tokens);

/* Create a training state: tag bytes[0..n) (n >= 1) into symbols with the
   character classes of "Ne Yapar? 1" ("Satir Satir Analiz 1)") and count the
   pairs of iteration 0 into the global pair table ("Ne Yapar? 2").
   Asynchronous on the state's stream; bytes must stay valid until the next
   synchronising call (bpe_sync, bpe_step, ...). */
bpe_status bpe_init(const uint8_t *bytes, size_t n, const bpe_config *cfg, bpe_state **out);

/* Enqueue up to n_merges more iterations of "Nedir bu ya?" without waiting
   and without any host round trip between iterations: one plain kernel
   launch per iteration, each reading the merge the previous one prepared
   on the device. Iterations after the last countable pair do nothing.
   Shared devices: a pass never needs its whole grid resident at once.
   Its workgroups wait for one another only for work a running workgroup
   has already taken on (the scan's look-back waits for lower tiles, which
   are handed out in order; a table sweep waits for chunks already
   claimed), so any subset of resident workgroups completes the pass, and
   other kernels on the device only slow it down. Each wait is bounded all
   the same; one that gives up marks the state BPE_ESTATE (device error
   bit 2), which only a fault can cause. BPE_EIDSPACE if the total would
   exceed BPE_MAX_MERGES. */
bpe_status bpe_run(bpe_state *s, uint32_t n_merges);

/* Wait for the enqueued work; *n_done (may be NULL) = merges produced so far.
   Returns BPE_ETABLE / BPE_ESTATE if the device reported an error. */
bpe_status bpe_sync(bpe_state *s, uint32_t *n_done);

/* One iteration of "Nedir bu ya?", synchronously: *out = the merge made.
   BPE_DONE (and *out untouched) when no countable pair is left;
   BPE_EIDSPACE once all BPE_MAX_MERGES ids are used. */
bpe_status bpe_step(bpe_state *s, bpe_merge *out);

/* Copy the merges produced so far (up to cap) to out; *n_out = how many exist. */
bpe_status bpe_merges(bpe_state *s, bpe_merge *out, uint32_t cap, uint32_t *n_out);

/* Copy the current symbol sequence to out; *n_out = its length. After the
   last merge these are the training corpus's tokens: the sequence the
   merges of "Nedir bu ya?" have rewritten, each symbol id | 0x10000 where
   a word starts ("Ne Yapar? 1"; a merged symbol keeps its left part's bit,
   "Ne Yapar? 3"). With out NULL or cap 0 only the length is returned; cap
   below the length is BPE_EINVAL. */
bpe_status bpe_tokens(bpe_state *s, uint32_t *out, size_t cap, size_t *n_out);

/* Sequence length before each merge so far, then the current length:
   out[0] = n, out[i] = length after merge i - 1; *n_out = merges + 1. */
bpe_status bpe_lengths(bpe_state *s, uint32_t *out, uint32_t cap, uint32_t *n_out);

/* The pair counts the next iteration will choose from (the counts of the
   current sequence, "Ne Yapar? 2"): keys[i] = left << 16 | right, counts[i]
   its number of adjacent positions (pairs whose count fell to zero are left
   out), in table order; *n_out = number of distinct pairs. Both arrays are host or device, cap entries each; with cap
   0 only the number is returned, with cap below it BPE_EINVAL. */
bpe_status bpe_pair_counts(bpe_state *s, uint32_t *keys, uint32_t *counts, size_t cap, size_t *n_out);

/* The global pair table's size and use: *slots = 2^table_log2, *claimed =
   slots holding a key (a key keeps its slot for the life of the state, so
   this only grows, with the distinct pairs the corpus and its merges have
   produced), *limit = the claims at which the table counts as full
   (BPE_ETABLE). Any pointer may be NULL. Waits for the enqueued work. */
bpe_status bpe_table_usage(bpe_state *s, uint32_t *slots, uint32_t *claimed, uint32_t *limit);

/* Apply a given merge list as the state's next k iterations, in order
   (page "bpe - GPU BPE Tokenizer Pipeline", "Nedir bu ya?": a learned merge
   list is the tokenizer; its merges are applied in the order they were
   learned). Iteration m = (merges made so far) + i merges the pair
   (merges[i].left, merges[i].right) into the new id 256 + m exactly as a
   training iteration merges its chosen pair (left to right, non-
   overlapping, never across the word-start bit), and keeps the pair counts
   up to date, so training can go on afterwards (bpe_run / bpe_step): this
   is resume by replaying a saved merge list. The count recorded for each
   replayed merge is the pair's count just before it (0 if it does not
   occur; the merge then changes nothing but still uses up its id).
   merges: k entries, host or device, caller-owned; only left and right are
   read. Blocks until the k iterations are done.
   Errors: BPE_EINVAL (NULL pointers, or a pair naming an id >= 256 + m,
   which does not exist yet; nothing is applied), BPE_EIDSPACE (the ids run
   out), BPE_ESTATE (training on this state has stopped, or a device
   error), BPE_ETABLE, BPE_EHIP. */
bpe_status bpe_replay(bpe_state *s, const bpe_merge *merges, uint32_t k);

/* ---------------------------------------------------------------- encoding
   Encoding text with a learned merge list (page "bpe - GPU BPE Tokenizer
   Pipeline", "Nedir bu ya?": the list is applied in the order it was
   learned; "Ne Yapar? 1": no merge crosses a word start). The result equals
   applying merge k, k = 0, 1, ..., to every non-overlapping occurrence left
   to right over the whole tagged text, and is computed word by word, the
   lowest-rank pair first. Tokens are in the training format: id | 0x10000 on
   the first token of each word. A pair listed twice acts at its first rank
   (it never occurs again after that merge). */
typedef struct bpe_encoder bpe_encoder;

/* Build the rank table of merges[0..n_merges) (host or device; counts are
   not read) on the current device and create the encoder's stream.
   Errors: BPE_EINVAL (NULL out, an id that does not exist before its
   merge), BPE_EIDSPACE (above 65,280 merges), BPE_ENOMEM, BPE_EHIP. */
bpe_status bpe_encoder_build(const bpe_merge *merges, uint32_t n_merges, bpe_encoder **out);

/* Encode bytes[0..n) (host or device) on stream (a hipStream_t, or NULL for
   the encoder's own). tokens (host or device, capacity tokens_cap >= n, or
   NULL for the count only) receive the tokens, *n_tokens their count.
   With the word cache (bpe_encoder_cache; on by default from 1 MiB) three
   kernels first collect the distinct words of 2..32 bytes of every second
   4 KiB tile and encode each once; then three kernels (the walk over 1 KiB
   tiles, a scan of the token counts of groups of 64 tiles, the copy of
   each tile's tokens to its place), a wait for the total and a sized copy
   for host tokens. Device buffers are pooled in the encoder (about 5 bytes
   per input byte, the cache's 76 bytes per slot, plus scratch of 12 bytes
   per position for words that do not fit a tile's LDS, at most 2^24
   positions per call), so calls on one encoder must not overlap. Errors:
   BPE_EINVAL (NULL encoder or n_tokens, NULL bytes with n > 0, n >
   BPE_MAX_BYTES, tokens_cap < n), BPE_ENOMEM (also: words past a tile's
   LDS longer than the scratch in total), BPE_EHIP. */
bpe_status bpe_encoder_encode(bpe_encoder *e, const uint8_t *bytes, size_t n, void *stream, uint32_t *tokens,
                              size_t tokens_cap, size_t *n_tokens);

/* Time the encoder's kernels: bpe_encoder_encode of device bytes once, then
   reps runs back to back on the encoder's stream with HIP events between
   the stages; ms (4 * reps entries, or NULL): the word cache's three
   kernels (with the small init kernel), walk, scan and copy times of each
   run. */
bpe_status bpe_encoder_profile(bpe_encoder *e, const uint8_t *bytes, size_t n, uint32_t reps, float *ms,
                               size_t *n_tokens);

/* Size of the encoder's word cache for later calls. Words are encoded each
   on its own (page "bpe - GPU BPE Tokenizer Pipeline", "Nedir bu ya?" and
   "Ne Yapar? 1": merges never cross a word start), so every occurrence of a
   word encodes alike and each distinct word of 2..32 bytes found in every
   second 4 KiB tile is encoded once per call into a hash table (linear
   probing over 2^log2_slots slots, at most 8 probes); its occurrences copy
   the result after comparing their bytes with the cached word's. log2_slots:
   BPE_CACHE_AUTO (none below 1 MiB of input, else one slot per 256 input
   bytes, 2^18..2^22), 0 (no cache) or 8..24.
   key_bits (at most BPE_CACHE_KEY_BITS): hash bits in a slot's key; fewer
   bits make distinct words share keys, which only sends more words down
   the uncached path (a testing aid). Tokens never depend on either
   setting. A new encoder has the automatic size; a call that cannot
   allocate the cache's memory runs without it. Errors: BPE_EINVAL. */
#define BPE_CACHE_AUTO 0xFFFFFFFFu
#define BPE_CACHE_KEY_BITS 32u
bpe_status bpe_encoder_cache(bpe_encoder *e, uint32_t log2_slots, uint32_t key_bits);

/* Release the encoder and its buffers. NULL is a no-op. */
void bpe_encoder_free(bpe_encoder *e);

/* One-shot encoding: bpe_encoder_build, bpe_encoder_encode on cfg's stream
   (cfg may be NULL; its table size and workspace are not used),
   bpe_encoder_free. Errors as those calls, and BPE_EINVAL for a bad cfg. */
bpe_status bpe_encode(const uint8_t *bytes, size_t n, const bpe_merge *merges, uint32_t n_merges,
                      const bpe_config *cfg, uint32_t *tokens, size_t tokens_cap, size_t *n_tokens);

/* ---------------------------------------------------------------- inference
   Greedy longest-match tokenization with a learned vocabulary (page "bpe -
   GPU BPE Tokenizer Pipeline": the inference paragraph of "Nedir bu ya?",
   "Ne Yapar? 4", "Host Mimarisi 1-4"): at each position the token is the
   longest vocabulary string the text continues with there. The vocabulary
   is a merge list's: id b < 256 is the byte b, id 256 + k the string of
   merge k's left id followed by its right id's. A string that several ids
   spell maps to the smallest id. */
typedef struct bpe_trie bpe_trie;

/* Build the prefix tree of the vocabulary of merges[0..n_merges) (host or
   device; counts are not read) on the current device, as a double array in
   device memory, and create the trie's own stream. Errors: BPE_EINVAL for a
   NULL out, an id that does not exist before its merge, a merge joining
   strings of different byte classes (no trained merge does; such a string
   could match across a word start, which the kernel's per-word
   decomposition excludes), or a vocabulary past 2^21 - 1 trie slots or
   2^27 string bytes; BPE_EIDSPACE above 65,280 merges; BPE_ENOMEM,
   BPE_EHIP. */
bpe_status bpe_trie_build(const bpe_merge *merges, uint32_t n_merges, bpe_trie **out);

/* Size of the trie's double array in 8-byte slots, and the longest
   vocabulary string in bytes (either pointer may be NULL). */
bpe_status bpe_trie_info(const bpe_trie *t, uint32_t *slots, uint32_t *max_len);

/* Tokenize bytes[0..n) (host or device). stream: a hipStream_t, or NULL for
   the trie's own stream; device input is read on it. tokens (host or
   device, capacity tokens_cap >= n, or NULL to get only the count) receive
   plain token ids; *n_tokens the count. Three kernels (walk, scan of the
   per-tile counts, copy), then a wait for the 4-byte total and a sized
   copy when tokens is host memory. The trie keeps pooled device buffers
   between calls (grown by half when a call needs more; about 3 bytes per
   input byte), so calls on one trie must not overlap. Errors: BPE_EINVAL
   (NULL trie or n_tokens, NULL bytes with n > 0, n > BPE_MAX_BYTES,
   tokens_cap < n), BPE_ENOMEM, BPE_EHIP. */
bpe_status bpe_trie_encode(bpe_trie *t, const uint8_t *bytes, size_t n, void *stream, uint32_t *tokens,
                           size_t tokens_cap, size_t *n_tokens);

/* Time the inference kernels: bpe_trie_encode of device bytes[0..n) once
   (tokens to the trie's pooled buffer), then reps runs back to back on the
   trie's own stream with a HIP event after each kernel, one host wait at
   the end. ms (host, 3 * reps entries, or NULL) receives the device time of
   each run's walk, scan and copy kernels in that order; *n_tokens the token
   count. Errors: BPE_EINVAL (NULL arguments, n = 0, reps = 0, host bytes),
   BPE_ESTATE (runs disagree), BPE_ENOMEM, BPE_EHIP. */
bpe_status bpe_trie_profile(bpe_trie *t, const uint8_t *bytes, size_t n, uint32_t reps, float *ms,
                            size_t *n_tokens);

/* Release the trie and its buffers. NULL is a no-op. */
void bpe_trie_free(bpe_trie *t);

/* Device time of the iterations run by bpe_profile. */
typedef struct {
    double merge_ms;         /* total time of the iteration launches (selection, merge,
                                compaction and count update: one launch each)        */
    uint32_t launches;       /* number of iterations timed                            */
    uint32_t merges_done;    /* merges produced by the state after the run            */
    uint32_t sweeps;         /* iterations among them that swept the whole pair table
                                (the others took the merge from the candidate list)   */
    uint32_t reserved;       /* 0 */
} bpe_profile_result;

/* Like bpe_run followed by bpe_sync, but with a HIP event recorded on the
   state's stream after each iteration's launch, to time it. merge_ms (host,
   n_merges entries, or NULL) receives the per-iteration times; iterations
   after training stopped take ~0 ms. One host wait at the end, as in
   bpe_run + bpe_sync. The events are created once per device and kept until
   the process ends. */
bpe_status bpe_profile(bpe_state *s, uint32_t n_merges, bpe_profile_result *out, float *merge_ms);

/* Release the state and everything it owns (not a caller workspace). NULL is a no-op. */
void bpe_free(bpe_state *s);

/* Static description of a status code. */
const char *bpe_strerror(bpe_status st);

/* Thread-local detail of the most recent failure in this thread ("" if none). */
const char *bpe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BPE_H */
