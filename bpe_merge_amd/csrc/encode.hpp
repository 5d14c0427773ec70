// Encoding new text with a learned merge list, word by word (page "bpe -
// GPU BPE Tokenizer Pipeline", "Nedir bu ya?": a learned list is applied to
// text in the order its merges were learned; "Ne Yapar? 1": merges never
// cross a word start).
//
// Applying merge k over the whole text, k = 0, 1, ..., equals merging,
// inside each word (maximal run of one byte class), the pair of lowest rank
// again and again, each time at all its non-overlapping occurrences left to
// right: a pair containing id 256 + k has rank > k, so a merge never
// creates a pair of lower rank than its own, and words never interact. One
// pass over the text then replaces one pass per merge. The decomposition
// is the inference kernels' (trie.hpp): a workgroup takes a tile and owns
// the words starting in it, one-byte words are final at once. Since a word's
// tokens depend on its bytes alone, the distinct words are encoded once,
// into a word cache (below), and the walk copies their tokens; the words
// the cache does not hold are taken by the lanes of a wave from a queue. A
// lane runs one iteration of its word per round: find the lowest-rank pair
// on the word's live list, merge it everywhere in the word, look up the
// ranks of the pairs the merges made. Ranks come from a hash table of the
// list (pair -> first rank of that pair; a repeated pair never occurs again
// after its first merge, so later copies are dead). The output is the
// training format: id | 0x10000 on the first token of each word.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "trie.hpp"

namespace bpek {

constexpr uint32_t RK_NONE = 0xFFFFu;   // no such pair in the list
constexpr uint32_t RK_STALE = 0xFFFEu;  // a pair a merge made, rank not yet looked up
constexpr uint32_t NIL = 0xFFFFFFFFu;

// Rank table: 64-bit slots key << 32 | rank, empty = all ones (the key
// 0xFFFFFFFF = (65535, 65535) never appears in a list: an entry's ids are
// below 256 + its index <= 65534). Linear probing, at most probes slots.
struct RankTable {
    const unsigned long long* slot;
    uint32_t mask;
    uint32_t probes;
    const uint16_t* bytes;  // rank of every byte pair, 256 x 256 (RK_NONE if absent)
};

__host__ __device__ __forceinline__ uint32_t rank_of(const RankTable& rt, uint32_t key) {
    uint32_t h = mix32(key) & rt.mask;
    for (uint32_t p = 0; p < rt.probes; ++p) {
        const unsigned long long v = rt.slot[h];
        const uint32_t k = (uint32_t)(v >> 32);
        if (k == key) return (uint32_t)(v & 0xFFFFull);
        if (k == 0xFFFFFFFFu) break;
        h = (h + 1u) & rt.mask;
    }
    return RK_NONE;
}

// A word's live list: sym, next live position and rank of the pair
// starting at each position, in LDS (16-bit, positions relative to the
// tile) or in global scratch (positions relative to the word).
struct LdsWord {
    uint16_t* sym;
    uint16_t* nx;
    uint16_t* rk;
    __host__ __device__ uint32_t s(uint32_t i) const { return sym[i]; }
    __host__ __device__ uint32_t n(uint32_t i) const { return nx[i]; }
    __host__ __device__ uint32_t r(uint32_t i) const { return rk[i]; }
    __host__ __device__ void set_s(uint32_t i, uint32_t v) const { sym[i] = (uint16_t)v; }
    __host__ __device__ void set_n(uint32_t i, uint32_t v) const { nx[i] = (uint16_t)v; }
    __host__ __device__ void set_r(uint32_t i, uint32_t v) const { rk[i] = (uint16_t)v; }
};
struct GlobalWord {
    uint16_t* sym;
    uint32_t* nx;
    uint16_t* rk;
    __host__ __device__ uint32_t s(uint32_t i) const { return sym[i]; }
    __host__ __device__ uint32_t n(uint32_t i) const { return nx[i]; }
    __host__ __device__ uint32_t r(uint32_t i) const { return rk[i]; }
    __host__ __device__ void set_s(uint32_t i, uint32_t v) const { sym[i] = (uint16_t)v; }
    __host__ __device__ void set_n(uint32_t i, uint32_t v) const { nx[i] = v; }
    __host__ __device__ void set_r(uint32_t i, uint32_t v) const { rk[i] = (uint16_t)v; }
};

// One iteration on the live list of a word [q, wend): the lowest-rank pair
// (its first occurrence, from the left); if there is none the word is
// final and this returns true. Otherwise its occurrences are merged left to
// right (the left symbol becomes 256 + rank, the right one leaves the list;
// after a merge the scan goes on past the new symbol, so a run of one
// symbol is paired from its left end), and the pairs the merges made get
// their ranks.
template <class W>
__host__ __device__ __forceinline__ bool merge_iteration(const W& a, uint32_t q, uint32_t wend, const RankTable& rt) {
    uint32_t best = RK_NONE, bi = q, bprev = NIL;
    for (uint32_t i = q, prev = NIL;;) {
        const uint32_t j = a.n(i);
        if (j >= wend) break;
        const uint32_t r = a.r(i);
        if (r < best) {
            best = r;
            bi = i;
            bprev = prev;
        }
        prev = i;
        i = j;
    }
    if (best == RK_NONE) return true;
    const uint32_t X = BASE + best;
    for (uint32_t i = bi, pv = bprev;;) {
        const uint32_t j = a.n(i);
        if (j >= wend) break;
        if (a.r(i) == best) {
            const uint32_t k = a.n(j);
            a.set_s(i, X);
            a.set_n(i, k);
            a.set_r(i, RK_STALE);
            if (pv != NIL) a.set_r(pv, RK_STALE);
            pv = i;
            i = k;
            if (i >= wend) break;
        } else {
            pv = i;
            i = j;
        }
    }
    for (uint32_t i = bprev != NIL ? bprev : bi;;) {
        const uint32_t j = a.n(i);
        if (j >= wend) break;
        if (a.r(i) == RK_STALE) a.set_r(i, rank_of(rt, (a.s(i) << 16) | a.s(j)));
        i = j;
    }
    return false;
}

// A word from global scratch, by one thread: the bytes text[w0, w0 + len)
// (relative positions 0 .. len) are encoded in the scratch arrays at base;
// its tokens (id | WS on the first) are written to tok. Returns the token
// count.
__device__ __attribute__((noinline)) uint32_t encode_word_global(const uint8_t* __restrict__ text, size_t w0,
                                                                 uint32_t len, uint16_t* sym, uint32_t* nx,
                                                                 uint16_t* rk, RankTable rt, uint32_t* tok) {
    const GlobalWord a{sym, nx, rk};
    for (uint32_t i = 0; i < len; ++i) {
        sym[i] = text[w0 + i];
        nx[i] = i + 1u;
    }
    for (uint32_t i = 0; i + 1u < len; ++i) rk[i] = rt.bytes[((uint32_t)sym[i] << 8) | sym[i + 1u]];
    while (!merge_iteration(a, 0u, len, rt)) {
    }
    uint32_t c = 0;
    for (uint32_t i = 0; i < len; i = nx[i]) tok[c++] = sym[i] | (i == 0u ? WS : 0u);
    return c;
}

// ---------------------------------------------------------------- word cache
// A word's encoding depends on its bytes alone, and a text repeats few
// distinct words many times, so each distinct word can be encoded once: the
// insert pass puts the words of 2 .. WC_MAXLEN bytes of a sample of the
// tiles into a hash table, the fill pass encodes the word of every used
// slot into the slot's record, and the walk takes a word's tokens from a
// record holding the same bytes.
//
// A slot is claimed by a CAS on its key and the claimer stores a text
// position of its word. Nothing else is shared: device-scope atomics on one
// address serialise at memory (about 10 ns each), so a claim counter or a
// list of claimed slots, touched by every new word, would cost more than
// the rest of the pass; the fill pass scans all slots instead. A record is
// built from the bytes it encodes (those at the slot's position, over the
// key's length) and stores them, and the walk uses a record only when those
// bytes and that length equal the word's own; a word that finds no such
// record (probes used up, a different word under its key) is encoded by the
// walk itself.
// The walk reads records only, never keys: one cache line per probe. A
// record holds a word and its tokens under the encoder's merge list, so it
// stays right for every later call and records are never cleared; the
// record memory starts zeroed, and a record whose token-start word is 0
// was never filled and ends a probe run, as a free slot ends the insert's.
// A record is 16 u32 in two halves of 32 bytes; the first serves words of
// up to WC_SHORT bytes with up to WC_TOK_SHORT tokens alone: bytes 0-15
// [0, 4), length [4] (0: not cached: the slot's position did not hold that
// many bytes, or the word has more than WC_TOK tokens), token starts [5]
// (bit k: a token starts at offset k), token ids 0-3 [6, 8) (two per u32);
// the second holds bytes 16-31 [8, 12) and token ids 4-11 [12, 16). A
// short record keeps the records of a text's frequent words within the
// caches: a walk lookup reads 32 bytes.
constexpr uint32_t WC_MAXLEN = 32;    // longest cached word
constexpr uint32_t WC_SHORT = 16;     // longest word served by the first half
constexpr uint32_t WC_TOK = 12;       // most tokens a record holds
constexpr uint32_t WC_TOK_SHORT = 4;  // tokens in the first half
constexpr uint32_t WC_REC = 16;       // u32 per record (64 bytes)
constexpr uint32_t WC_HALF = 8;
constexpr uint32_t WC_LENW = 4, WC_MASKW = 5, WC_T0 = 6, WC_B1 = 8, WC_T1 = 12;
constexpr uint32_t WC_PROBES = 8;
constexpr uint32_t WC_BATCH = 3;     // words a thread of the insert pass or the walk handles with their loads in flight together

struct WordCache {
    unsigned long long* key;   // per slot: 0 = free, else hash bits << 6 | length
    uint32_t* pos;             // per slot: a text position of a word with that key
    uint32_t* rec;             // WC_REC words per slot
    uint32_t mask;             // slots - 1
    uint32_t kmask;            // hash bits kept in a key (fewer bits, more words sharing a key)
};

// Bytes s[a, a + len), len <= 4 NW, little-endian in w[0, NW), zero past
// len. s is 4-byte aligned; reads at most 4 NW + 4 bytes from s + (a & ~3).
template <int NW>
__device__ __forceinline__ void wc_pack_lds(const uint8_t* s, uint32_t a, uint32_t len, uint32_t (&w)[NW]) {
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(s);
    const uint32_t b = a >> 2, r = a & 3u;
    uint32_t lo = s32[b];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        uint32_t v = 0u;
        if (4u * (uint32_t)k < len) {
            const uint32_t hi = s32[b + (uint32_t)k + 1u];
            v = __builtin_amdgcn_alignbyte(hi, lo, r);
            lo = hi;
            const uint32_t rem = len - 4u * (uint32_t)k;
            if (rem < 4u) v &= (1u << (8u * rem)) - 1u;
        }
        w[k] = v;
    }
}

// 32-bit hash of a packed word (len <= 4 NW; the same value for any such
// NW): per 4 bytes an xor, a multiply and an xorshift, then the Murmur3
// finaliser. A key only has to tell apart the words that meet in one probe
// run (a record is used only after comparing bytes), so 32 bits suffice,
// and 32-bit multiplies keep the hash cheap: it runs once per word in the
// insert pass and again in the walk.
template <int NW>
__device__ __forceinline__ uint32_t wc_hash(const uint32_t (&w)[NW], uint32_t len) {
    uint32_t h = 0x9E3779B9u ^ len;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if (4u * (uint32_t)k < len) {
            h ^= w[k];
            h *= 0x85EBCA6Bu;
            h ^= h >> 13;
        }
    }
    return mix32(h);
}

__device__ __forceinline__ unsigned long long wc_key(const WordCache& wc, uint32_t h, uint32_t len) {
    return ((unsigned long long)(h & wc.kmask) << 6) | len;  // len >= 2: never 0
}
__device__ __forceinline__ uint32_t wc_slot(const WordCache& wc, uint32_t h) { return h & wc.mask; }

// Linear probing from slot: stop at the key, or claim the first free slot
// (CAS; the claimer records its position); give up after WC_PROBES slots.
// A plain load that still shows a slot free only costs the CAS.
__device__ __forceinline__ void wc_insert(const WordCache& wc, unsigned long long key, uint32_t slot, uint32_t pos) {
    for (uint32_t p = 0; p < WC_PROBES; ++p) {
        unsigned long long v = wc.key[slot];
        if (v == 0ull) {
            v = atomicCAS(wc.key + slot, 0ull, key);
            if (v == 0ull) {
                wc.pos[slot] = pos;
                return;
            }
        }
        if (v == key) return;
        slot = (slot + 1u) & wc.mask;
    }
}

// One probe: the first NW words of the slot's record into r.
template <uint32_t NW>
__device__ __forceinline__ void wc_probe(const WordCache& wc, uint32_t slot, uint32_t (&r)[NW]) {
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    const uint32_t* rp = wc.rec + (size_t)slot * WC_REC;
#pragma unroll
    for (int k = 0; k < (int)NW / 4; ++k) {
        const v4 x = *reinterpret_cast<const v4*>(rp + 4 * k);
        r[4 * k] = x.x;
        r[4 * k + 1] = x.y;
        r[4 * k + 2] = x.z;
        r[4 * k + 3] = x.w;
    }
}

// Whether a probed record r (its first half, or all of it) holds the
// packed word w of length len; with the first half only, len <= WC_SHORT
// and w has 4 words.
template <uint32_t NW, int NB>
__device__ __forceinline__ bool wc_match(const uint32_t (&w)[NB], uint32_t len, const uint32_t (&r)[NW]) {
    static_assert(NB == (NW == WC_REC ? 8 : 4), "packed bytes match the record part");
    uint32_t d = r[WC_LENW] ^ len;
#pragma unroll
    for (int k = 0; k < 4; ++k) d |= w[k] ^ r[k];
#pragma unroll
    for (int k = 4; k < NB; ++k) d |= w[k] ^ r[WC_B1 + (k - 4)];
    return d == 0u;
}

// The record holding the packed word w of length len (probing from slot),
// into r; false if none before a never-filled record, within WC_PROBES
// slots.
__device__ __forceinline__ bool wc_lookup(const WordCache& wc, uint32_t slot, const uint32_t (&w)[8], uint32_t len,
                                          uint32_t (&r)[WC_REC]) {
    for (uint32_t p = 0; p < WC_PROBES; ++p) {
        wc_probe<WC_REC>(wc, slot, r);
        if (wc_match(w, len, r)) return true;
        if (r[WC_MASKW] == 0u) return false;
        slot = (slot + 1u) & wc.mask;
    }
    return false;
}

// Free every slot (before the insert pass).
__global__ void k_wc_clear(WordCache wc, uint32_t slots) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < slots; i += gridDim.x * blockDim.x) wc.key[i] = 0ull;
}

// Fill pass: every used slot's word, its key's length of bytes from its
// position (n bytes of text), encoded in a thread's LDS range of WC_MAXLEN
// positions. A workgroup takes chunks of FILL_CHUNK slots, lists the used
// ones in LDS (a block scan: a used slot is one in five or so, and a wave
// waits for its slowest lane's word) and encodes them one per thread. The
// record gets those bytes (zero past the length), the token ids, the
// offsets where tokens start and the length; a range past the text's end
// gets length 0, which no lookup accepts.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_wc_fill(const uint8_t* __restrict__ text, uint32_t n, WordCache wc,
                                                 RankTable rt, uint32_t slots) {
    constexpr uint32_t PER = 4;
    constexpr uint32_t FILL_CHUNK = TPB * PER;
    static_assert(FILL_CHUNK <= 65536, "chunk offsets fit 16 bits");
    __shared__ uint16_t s_sym[TPB * WC_MAXLEN], s_nx[TPB * WC_MAXLEN], s_rk[TPB * WC_MAXLEN];
    __shared__ uint16_t s_used[FILL_CHUNK];
    __shared__ uint32_t s_w[TPB / 64];
    const LdsWord lw{s_sym, s_nx, s_rk};
    const uint32_t tid = threadIdx.x;
    const uint32_t b = tid * WC_MAXLEN;
    for (uint32_t c0 = blockIdx.x * FILL_CHUNK; c0 < slots; c0 += gridDim.x * FILL_CHUNK) {
        uint32_t used = 0u;
#pragma unroll
        for (uint32_t k = 0; k < PER; ++k) {
            const uint32_t slot = c0 + tid * PER + k;
            used |= (slot < slots && wc.key[slot] != 0ull) ? 1u << k : 0u;
        }
        uint32_t nused;
        uint32_t off = block_exclusive_sum<TPB>(__popc(used), s_w, &nused);
        for (uint32_t m = used; m; m &= m - 1u) s_used[off++] = (uint16_t)(tid * PER + (__ffs(m) - 1));
        lds_barrier();
        for (uint32_t i = tid; i < nused; i += TPB) {
            const uint32_t slot = c0 + s_used[i];
            const uint32_t len = (uint32_t)(wc.key[slot] & 63ull);
            const uint32_t at = wc.pos[slot];
            uint32_t* rp = wc.rec + (size_t)slot * WC_REC;
            if (len > WC_MAXLEN || at > n || n - at < len) {
                rp[WC_LENW] = 0u;
                rp[WC_MASKW] = 1u;  // filled, matching no word
                continue;
            }
            const uint8_t* src = text + at;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t v = 0u;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t j = 4u * (uint32_t)k + (uint32_t)u;
                    if (j < len) v |= (uint32_t)src[j] << (8 * u);
                }
                rp[k < 4 ? k : WC_B1 + (k - 4)] = v;
            }
            for (uint32_t j = 0; j < len; ++j) {
                s_sym[b + j] = src[j];
                s_nx[b + j] = (uint16_t)(b + j + 1u);
            }
            for (uint32_t j = 0; j + 1u < len; ++j)
                s_rk[b + j] = rt.bytes[((uint32_t)s_sym[b + j] << 8) | s_sym[b + j + 1u]];
            while (!merge_iteration(lw, b, b + len, rt)) {
            }
            uint16_t* t0 = reinterpret_cast<uint16_t*>(rp + WC_T0);
            uint16_t* t1 = reinterpret_cast<uint16_t*>(rp + WC_T1);
            uint32_t m = 0u, c = 0u;
            for (uint32_t x = b; x < b + len; x = s_nx[x], ++c) {
                m |= 1u << (x - b);
                if (c < WC_TOK_SHORT)
                    t0[c] = s_sym[x];
                else if (c < WC_TOK)
                    t1[c - WC_TOK_SHORT] = s_sym[x];
            }
            rp[WC_MASKW] = m;
            rp[WC_LENW] = c <= WC_TOK ? len : 0u;  // more tokens than a record holds: not cached
        }
        lds_barrier();
    }
}

// A tile's text copy, [t0 - 16, t0 + 16 NCH - 16) in 16-byte chunks (zero
// outside the text), held in registers from its load to its store into
// LDS: a workgroup loads the next tile's text as it starts a tile, so the
// load's latency passes while the tile is worked on.
template <int TPB, uint32_t NCH>
struct TileText {
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    static constexpr uint32_t R = (NCH + TPB - 1) / TPB;
    v4 v[R];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t t0) {
#pragma unroll
        for (uint32_t j = 0; j < R; ++j) {
            const uint32_t k = threadIdx.x + j * TPB;
            if (k < NCH) v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, t0 - 16u + 16u * k, 0, 0);
        }
    }
    // s_txt[16 k + i] = byte i of chunk k
    __device__ __forceinline__ void store(uint8_t* s_txt) const {
#pragma unroll
        for (uint32_t j = 0; j < R; ++j) {
            const uint32_t k = threadIdx.x + j * TPB;
            if (k < NCH) *reinterpret_cast<v4*>(s_txt + 16u * k) = v[j];
        }
    }
};

// The byte_class value of each byte of x, four at a time. Range tests are
// subtractions on bytes that first get bit 7, so no borrow crosses a byte;
// a byte of 0x80 or more is a letter whatever its low bits say.
__device__ __forceinline__ uint32_t byte_class4(uint32_t x) {
    const uint32_t H = 0x80808080u;
    const uint32_t hi = x & H, lo = x & 0x7F7F7F7Fu;
    const uint32_t t = lo | 0x20202020u | H, l = lo | H;  // t: ASCII letters in lower case
    const uint32_t letter = hi | ((t - 0x61616161u) & ~(t - 0x7B7B7B7Bu) & H);
    const uint32_t digit = (l - 0x30303030u) & ~(l - 0x3A3A3A3Au) & ~hi & H;
    const uint32_t space = ~(((lo ^ 0x20202020u) | H) - 0x01010101u) & ~hi & H;
    const uint32_t nl = ~(((lo ^ 0x0A0A0A0Au) | H) - 0x01010101u) & ~hi & H;
    const uint32_t other = H & ~(letter | digit | space | nl);
    return (digit >> 7) | (space >> 6) | (nl >> 5) | ((other >> 7) * 3u);
}

// With the text of tile t stored in LDS (s_txt[p + 16 + mis] = text[t0 +
// p], TILE bytes and the halo), the word starts inside the tile in s_sb,
// and *s_after, the first class change in the halo (CAP if none). Returns
// this thread's starts (bit k: position 16 tid + k) of words of two bytes
// or more and, in *single, those of one-byte words. The caller clears
// *s_after to CAP before; this clears s_sb and ends with the starts
// recorded.
template <int TPB, uint32_t TILE, uint32_t CAP>
__device__ __forceinline__ uint32_t tile_words(uint32_t t0, uint32_t nrel, uint32_t sh, const uint8_t* s_txt,
                                               uint32_t* s_sb, uint32_t* s_after, uint32_t* single) {
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < TILE / 32u; i += TPB) s_sb[i] = 0u;
    __syncthreads();
    uint32_t multi;
    {
        // bit k of ch (k = 0..16): a class change between positions p0 + k - 1
        // and p0 + k (or the text's first byte), from the classes of
        // positions p0 .. p0 + 15 four at a time (aligned LDS words, shifted
        // into place) and of the bytes on either side
        const uint32_t p0 = 16u * tid;
        const uint32_t a = p0 + sh;  // LDS offset of position p0
        const uint32_t* w = reinterpret_cast<const uint32_t*>(s_txt) + (a >> 2);
        uint32_t prev = byte_class(s_txt[a - 1u]), ch = 0u, lo = w[0];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t hi = w[j + 1];
            const uint32_t code = byte_class4(__builtin_amdgcn_alignbyte(hi, lo, a & 3u));
            lo = hi;
            const uint32_t d = code ^ ((code << 8) | prev);            // bytes 0..7
            const uint32_t nz = (d + 0x7F7F7F7Fu) & 0x80808080u;       // bit 7: byte nonzero
            ch |= ((((nz >> 7) * 0x204081u) >> 21) & 0xFu) << (4 * j);  // the four bit 7s, packed
            prev = code >> 24;
        }
        ch |= (byte_class(s_txt[a + 16u]) != prev ? 1u : 0u) << 16;
        if (t0 + p0 == 0u) ch |= 1u;
        const uint32_t lim = nrel > p0 ? min(nrel - p0, 17u) : 0u;
        const uint32_t inside = (1u << lim) - 1u;  // positions before the text's end
        const uint32_t starts = inside & ch & 0xFFFFu;
        const uint32_t bnd = (~inside | ch) & 0x1FFFEu;  // bit k: position p0 + k starts a word or is past the end
        *single = starts & (bnd >> 1);
        multi = starts & ~*single;
        if (starts) atomicOr(&s_sb[p0 >> 5], starts << (p0 & 31u));
    }
    {
        uint32_t after = CAP;
        const uint32_t p0 = TILE + TRIE_HALO_PER_THREAD * tid;
        uint32_t pc = byte_class(s_txt[p0 - 1u + sh]);
#pragma unroll
        for (int k = 0; k < (int)TRIE_HALO_PER_THREAD; ++k) {
            const uint32_t c = byte_class(s_txt[p0 + k + sh]);
            if (p0 + k < nrel && c != pc && after == CAP) after = p0 + k;
            pc = c;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) after = min(after, (uint32_t)__shfl_xor(after, o));
        if ((tid & 63u) == 0u) atomicMin(s_after, after);
    }
    return multi;
}

// End of the word starting at q (< TILE): the next start in the tile, else
// last_end.
template <uint32_t TILE>
__device__ __forceinline__ uint32_t word_end(const uint32_t* s_sb, uint32_t q, uint32_t last_end) {
    for (uint32_t x = q + 1u; x < TILE;) {
        const uint32_t m = s_sb[x >> 5] & (0xFFFFFFFFu << (x & 31u));
        if (m) return (x & ~31u) + (__ffs(m) - 1);
        x = (x & ~31u) + 32u;
    }
    return last_end;
}

// Insert pass: every stride-th tile of the walk's (tiles 0, stride, ...),
// every word of 2 .. WC_MAXLEN bytes starting in it put into the cache.
// (six waves per SIMD and three words per thread with their loads in
// flight: the pass waits on its loads and claims; 256 MiB corpus, 0.35 ms
// per pass with the compiler's register budget and one word at a time,
// 0.27-0.29 ms with both)
template <int TPB>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(6))) void k_wc_insert(const uint8_t* __restrict__ text, uint32_t n, uint32_t ntiles,
                                                   uint32_t stride, WordCache wc) {
    constexpr uint32_t TILE = TPB * 16u;
    constexpr uint32_t HALO = TPB * TRIE_HALO_PER_THREAD;
    constexpr uint32_t CAP = TILE + HALO;
    constexpr uint32_t NCH = (CAP + 32u) / 16u;
    static_assert(HALO > WC_MAXLEN, "a cached word ends inside the copy");
    __shared__ __align__(16) uint8_t s_txt[NCH * 16u];
    __shared__ uint32_t s_sb[TILE / 32u];
    __shared__ uint16_t s_list[TILE];
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_after;

    const uint32_t tid = threadIdx.x;
    const uint32_t mis = (uint32_t)((uintptr_t)text & 15u);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(text - mis), 0, (int)((n + mis + 15u) & ~15u), 0x00020000);
    const uint32_t sh = 16u + mis;
    const uint32_t nsamp = (ntiles + stride - 1u) / stride;
    for (uint32_t tt = blockIdx.x; tt < nsamp; tt += gridDim.x) {
        const uint32_t t = tt * stride;
        if (tid == 0) s_after = CAP;
        const uint32_t t0 = t * TILE;
        const uint32_t nrel = n - t0;
        {
            // the previous tile's reads of s_txt ended before its last barrier
            TileText<TPB, NCH> tx;
            tx.load(rs, t0);
            tx.store(s_txt);
        }
        uint32_t single;
        const uint32_t multi = tile_words<TPB, TILE, CAP>(t0, nrel, sh, s_txt, s_sb, &s_after, &single);
        uint32_t nwords;
        uint32_t woff = block_exclusive_sum<TPB>(__popc(multi), s_w, &nwords);
        for (uint32_t m = multi; m; m &= m - 1u) s_list[woff++] = (uint16_t)(16u * tid + (__ffs(m) - 1));
        lds_barrier();
        const uint32_t lim = nrel < CAP ? nrel : CAP;
        const uint32_t last_end = s_after < lim ? s_after : lim;
        // WC_BATCH words per thread with their home slots' keys loaded
        // together; a word already in its home slot (most occurrences of
        // frequent words) needs nothing more
        for (uint32_t i0 = tid; i0 < nwords; i0 += WC_BATCH * TPB) {
            uint32_t q[WC_BATCH], slot[WC_BATCH];
            unsigned long long key[WC_BATCH], v[WC_BATCH];
#pragma unroll
            for (int u = 0; u < (int)WC_BATCH; ++u) {
                const uint32_t i = i0 + (uint32_t)u * TPB;
                key[u] = 0ull;
                if (i < nwords) {
                    q[u] = s_list[i];
                    const uint32_t len = word_end<TILE>(s_sb, q[u], last_end) - q[u];
                    // a longer word (also one running past the copy: its
                    // length here is at least HALO) is not cached
                    if (len <= WC_MAXLEN) {
                        uint32_t w[8];
                        wc_pack_lds(s_txt, q[u] + sh, len, w);
                        const uint32_t h = wc_hash(w, len);
                        key[u] = wc_key(wc, h, len);
                        slot[u] = wc_slot(wc, h);
                        v[u] = wc.key[slot[u]];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < (int)WC_BATCH; ++u)
                if (key[u] && v[u] != key[u]) wc_insert(wc, key[u], slot[u], t0 + q[u]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- the walk
// Error flag of a call (status[1]): long words need more scratch than the
// call has.
constexpr uint32_t ENC_ERR_SCRATCH = 1u;
constexpr uint32_t ENC_GROUP = 64;  // tiles per group sum

// Tiles of TILE = 16 TPB bytes, t = blockIdx.x, blockIdx.x + gridDim.x,
// ... A tile's tokens are those of the words starting in it: the words
// ending within CAP bytes of its start are encoded in LDS, a last word
// running further in scratch reserved from status[2] (capacity scratch_cap
// positions; past it ENC_ERR_SCRATCH is set in status[1] and the word is
// skipped; sym_g, nx_g, rk_g: the scratch arrays). Outputs for tile t, in
// its region of CAP words at tok32 + t * CAP: the 16-bit ids of the cnt[t]
// tokens encoded in LDS, and from word CAP / 2 on the bits marking word
// starts among them; the long last word's tokens at ovf + ovf_pos[t]
// (ovf_n[t] of them; NO_OVF / 0 otherwise). The tile's token count is
// added to gsum[t / ENC_GROUP].
template <int TPB>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(3))) void k_enc_walk(
    const uint8_t* __restrict__ text, uint32_t n, RankTable rt, uint32_t* __restrict__ tok32,
    uint32_t* __restrict__ cnt, uint32_t* __restrict__ ovf_pos, uint32_t* __restrict__ ovf_n,
    uint32_t* __restrict__ gsum, uint32_t ntiles, uint16_t* sym_g, uint32_t* nx_g, uint16_t* rk_g, uint32_t* ovf,
    uint32_t* status, uint32_t scratch_cap, WordCache wc) {
    constexpr uint32_t TILE = TPB * 16u;
    constexpr uint32_t HALO = TPB * TRIE_HALO_PER_THREAD;
    constexpr uint32_t CAP = TILE + HALO;
    constexpr uint32_t PER = CAP / TPB;
    constexpr uint32_t NCH = (CAP + 32u) / 16u;
    static_assert(CAP % TPB == 0 && PER <= 32, "compaction covers CAP positions, at most 32 per thread");

    __shared__ __align__(16) uint8_t s_txt[NCH * 16u];  // s_txt[p + 16 + mis] = text[t0 + p]
    __shared__ uint32_t s_flag[CAP / 32u];             // token starts
    __shared__ uint32_t s_sb[TILE / 32u];              // word starts in the tile
    __shared__ uint16_t s_sym[CAP], s_nx[CAP], s_rk[CAP];
    __shared__ __align__(4) uint16_t s_aux[CAP];       // word list, then staged output ids
    __shared__ uint32_t s_ws[CAP / 32u];               // staged output: word-start bits
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_ovf_pos, s_ovf_n, s_after, s_nq;
    static_assert(CAP % 2u == 0, "ids are stored two at a time");
    constexpr uint32_t DLIST = TILE / 2;  // with the cache: the queue's words at s_aux[DLIST..)
    // flags on a queued position: look the word up from its home slot (a
    // word of more than WC_SHORT bytes or WC_TOK_SHORT tokens), or from the
    // second slot after it (its home slot and the next hold other words)
    constexpr uint32_t RETRY = 0x8000u, RETRY_NEXT = 0x4000u;
    static_assert(CAP < RETRY_NEXT, "positions leave the flag bits free");
    static_assert(DLIST + TILE / 2 <= CAP, "word list and queue fit s_aux");

    const uint32_t tid = threadIdx.x;
    const uint32_t mis = (uint32_t)((uintptr_t)text & 15u);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(text - mis), 0, (int)((n + mis + 15u) & ~15u), 0x00020000);
    const LdsWord lw{s_sym, s_nx, s_rk};
    const uint32_t sh = 16u + mis;
    uint32_t* const err = status + 1;
    uint32_t* const scratch_used = status + 2;

    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        if (tid == 0) {
            s_ovf_pos = NO_OVF;
            s_ovf_n = 0u;
            s_after = CAP;
            s_nq = 0u;
        }
        for (uint32_t i = tid; i < CAP / 32u; i += TPB) s_flag[i] = 0u;
        const uint32_t t0 = t * TILE;
        const uint32_t nrel = n - t0;
        auto lbyte = [&](uint32_t q) -> uint32_t { return s_txt[q + sh]; };  // q < CAP
        {
            // the previous tile's reads of s_txt ended before its compaction
            TileText<TPB, NCH> tx;
            tx.load(rs, t0);
            tx.store(s_txt);
        }

        // word starts: one-byte words are final here, the others listed
        uint32_t single;
        const uint32_t multi = tile_words<TPB, TILE, CAP>(t0, nrel, sh, s_txt, s_sb, &s_after, &single);
        // s_ws is read by the previous tile's last loop: cleared only past
        // the barrier in tile_words
        for (uint32_t i = tid; i < CAP / 32u; i += TPB) s_ws[i] = 0u;
        if (single) {
            const uint32_t p0 = 16u * tid;
            atomicOr(&s_flag[p0 >> 5], single << (p0 & 31u));
            for (uint32_t m = single; m; m &= m - 1u) {
                const uint32_t k = __ffs(m) - 1;
                s_sym[p0 + k] = (uint16_t)lbyte(p0 + k);
            }
        }
        uint32_t nwords;
        uint32_t woff = block_exclusive_sum<TPB>(__popc(multi), s_w, &nwords);
        for (uint32_t m = multi; m; m &= m - 1u) s_aux[woff++] = (uint16_t)(16u * tid + (__ffs(m) - 1));
        __syncthreads();

        const uint32_t lim = nrel < CAP ? nrel : CAP;
        const uint32_t last_end = s_after < lim ? s_after : lim;
        const bool last_open = s_after >= CAP && lim < nrel;

        // live list of the word [q, wend) from its bytes, with the ranks of
        // its byte pairs (eight loads in flight, then the stores)
        auto init_word = [&](uint32_t q, uint32_t wend) {
            for (uint32_t i = q; i < wend; ++i) {
                s_sym[i] = (uint16_t)lbyte(i);
                s_nx[i] = (uint16_t)(i + 1u);
            }
            for (uint32_t i = q; i + 1u < wend; i += 8u) {
                uint32_t r[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t p = i + (uint32_t)u;
                    r[u] = p + 1u < wend ? rt.bytes[(lbyte(p) << 8) | lbyte(p + 1u)] : 0u;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (i + (uint32_t)u + 1u < wend) s_rk[i + u] = (uint16_t)r[u];
            }
        };
        auto flag_tokens = [&](uint32_t q, uint32_t wend) {
            for (uint32_t i = q; i < wend; i = s_nx[i]) atomicOr(&s_flag[i >> 5], 1u << (i & 31u));
        };
        // a cached word at q: the token starts and ids of its record r (the
        // first half for a word of up to WC_SHORT bytes and WC_TOK_SHORT tokens)
        auto put_tokens = [&](uint32_t q, const auto& r) {
            constexpr uint32_t NT = sizeof(r) / sizeof(r[0]) == WC_REC ? WC_TOK : WC_TOK_SHORT;
            uint32_t m = r[WC_MASKW];
            const uint32_t o = q & 31u;
            atomicOr(&s_flag[q >> 5], m << o);
            if (o && (m >> (32u - o))) atomicOr(&s_flag[(q >> 5) + 1u], m >> (32u - o));
#pragma unroll
            for (int k = 0; k < (int)NT; ++k) {
                if (m) {
                    const uint32_t two = k < (int)WC_TOK_SHORT ? r[WC_T0 + k / 2]
                                                               : r[WC_T1 + (k - (int)WC_TOK_SHORT) / 2];
                    s_sym[q + __ffs(m) - 1] = (uint16_t)(two >> (16 * (k & 1)));
                    m &= m - 1u;
                }
            }
        };

        // with the cache: every word of 2 .. WC_SHORT bytes takes its tokens
        // from the first half of the record in its home slot or the slot
        // after it (where most words that lost their home slot to another
        // went), WC_BATCH words per thread with their loads in flight
        // together; the other words are listed for the queue, flagged when
        // the queue should look them up (longer cached words, and short ones
        // whose first two slots hold other words)
        const uint16_t* ql = s_aux;
        uint32_t nq = nwords;
        if (wc.key) {
            for (uint32_t i0 = tid; i0 < nwords; i0 += WC_BATCH * TPB) {
                uint32_t q[WC_BATCH], len[WC_BATCH], w[WC_BATCH][4], r[WC_BATCH][WC_HALF], r1[WC_BATCH][WC_HALF];
                bool cand[WC_BATCH];
#pragma unroll
                for (int u = 0; u < (int)WC_BATCH; ++u) {
                    const uint32_t i = i0 + (uint32_t)u * TPB;
                    cand[u] = false;
                    if (i < nwords) {
                        q[u] = s_aux[i];
                        len[u] = word_end<TILE>(s_sb, q[u], last_end) - q[u];
                        cand[u] = len[u] <= WC_SHORT;
                    }
                    if (cand[u]) {
                        wc_pack_lds(s_txt, q[u] + sh, len[u], w[u]);
                        const uint32_t home = wc_slot(wc, wc_hash(w[u], len[u]));
                        wc_probe<WC_HALF>(wc, home, r[u]);
                        wc_probe<WC_HALF>(wc, (home + 1u) & wc.mask, r1[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < (int)WC_BATCH; ++u) {
                    const uint32_t i = i0 + (uint32_t)u * TPB;
                    if (i >= nwords) continue;
                    const bool hit = cand[u] && wc_match(w[u], len[u], r[u]);
                    const bool hit1 = cand[u] && !hit && r[u][WC_MASKW] && wc_match(w[u], len[u], r1[u]);
                    if (hit && __popc(r[u][WC_MASKW]) <= WC_TOK_SHORT)
                        put_tokens(q[u], r[u]);
                    else if (hit1 && __popc(r1[u][WC_MASKW]) <= WC_TOK_SHORT)
                        put_tokens(q[u], r1[u]);
                    else if (hit || hit1)  // more tokens than the first half holds: the whole record
                        s_aux[DLIST + atomicAdd(&s_nq, 1u)] = (uint16_t)(q[u] | RETRY);
                    else if (cand[u])  // a never-filled record ends the probe run
                        s_aux[DLIST + atomicAdd(&s_nq, 1u)] =
                            (uint16_t)(q[u] | (r[u][WC_MASKW] && r1[u][WC_MASKW] ? RETRY | RETRY_NEXT : 0u));
                    else
                        s_aux[DLIST + atomicAdd(&s_nq, 1u)] = (uint16_t)(q[u] | (len[u] <= WC_MAXLEN ? RETRY : 0u));
                }
            }
            lds_barrier();
            ql = s_aux + DLIST;
            nq = s_nq;
        }

        // the listed words: a wave queue, one iteration of a lane's word per
        // round
        {
            constexpr uint32_t NWAVE = TPB / 64u;
            const uint32_t wave = tid >> 6;
            const uint32_t share = (nq + NWAVE - 1u) / NWAVE;
            const uint32_t w_hi = min(nq, (wave + 1u) * share);
            uint32_t next = min(nq, wave * share);
            uint32_t q = 0, wend = 0, gq = NO_OVF;
            bool act = false;
            for (;;) {
                const unsigned long long need = __ballot(!act);
                if (need) {
                    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(need >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)need, 0u));
                    const uint32_t wi = next + below;
                    if (!act && wi < w_hi) {
                        q = ql[wi];
                        bool cached = false;
                        if (q & RETRY) {
                            const uint32_t from = (q & RETRY_NEXT) ? 2u : 0u;
                            q &= ~(RETRY | RETRY_NEXT);
                            wend = word_end<TILE>(s_sb, q, last_end);
                            const uint32_t len = wend - q;
                            uint32_t w[8], r[WC_REC];
                            wc_pack_lds(s_txt, q + sh, len, w);
                            const uint32_t h = wc_hash(w, len);
                            if (wc_lookup(wc, (wc_slot(wc, h) + from) & wc.mask, w, len, r)) {
                                put_tokens(q, r);
                                cached = true;
                            }
                        }
                        wend = word_end<TILE>(s_sb, q, last_end);
                        if (cached) {
                        } else if (last_open && wend == last_end) {
                            gq = q;  // runs past the copy: encoded from global memory below
                        } else {
                            init_word(q, wend);
                            act = true;
                        }
                    }
                    next += (uint32_t)__popcll(need);
                }
                if (__ballot(act) == 0ull && next >= w_hi) break;
                if (act && merge_iteration(lw, q, wend, rt)) {
                    flag_tokens(q, wend);
                    act = false;
                }
            }
            const unsigned long long gm = __ballot(gq != NO_OVF);
            uint32_t e = 0u;
            if (gm) {
                // the open word's end: the first position past the copy with
                // another class, or the text's end, searched by the wave 1 KiB
                // at a time; the search stops once the word is longer than
                // any call's scratch
                const uint32_t g = (uint32_t)__shfl((int)gq, (int)(__ffsll((long long)gm) - 1));
                const uint32_t cls = byte_class(lbyte(g));
                const uint32_t lane = tid & 63u;
                const uint32_t a0 = t0 + mis + lim;  // offset of position lim from text - mis
                for (uint32_t c = a0 >> 4;; c += 64u) {
                    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
                    const uint32_t ac = (c + lane) << 4;
                    const v4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, ac, 0, 0);
                    uint32_t stop = 0xFFFFFFFFu;
#pragma unroll
                    for (int k = 15; k >= 0; --k) {
                        const uint32_t a = ac + (uint32_t)k;
                        const uint32_t b = (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
                        if (a >= a0 && (a - mis - t0 >= nrel || byte_class(b) != cls)) stop = a - mis - t0;
                    }
                    const unsigned long long sm = __ballot(stop != 0xFFFFFFFFu);
                    if (sm) {
                        e = (uint32_t)__shfl((int)stop, (int)(__ffsll((long long)sm) - 1));
                        break;
                    }
                    const uint32_t past = ((c + 64u) << 4) - mis - t0;  // every position below is in the word
                    if (past - g > scratch_cap) {
                        e = past;
                        break;
                    }
                }
            }
            if (gq != NO_OVF) {
                const uint32_t len = e - gq;
                const uint32_t at = atomicAdd(scratch_used, len);
                if (at + len > scratch_cap || at + len < at) {
                    atomicOr(err, ENC_ERR_SCRATCH);
                } else {
                    s_ovf_pos = at;
                    s_ovf_n = encode_word_global(text, (size_t)t0 + gq, len, sym_g + at, nx_g + at, rk_g + at, rt,
                                                 ovf + at);
                }
            }
        }

        __syncthreads();

        // compaction: final symbols at the recorded starts, WS on word starts
        uint32_t bits;
        {
            const uint32_t lo = PER * tid, wi = lo >> 5, sb = lo & 31u;
            const uint32_t w0 = s_flag[wi];
            const uint32_t w1 = (wi + 1u < CAP / 32u) ? s_flag[wi + 1u] : 0u;
            const unsigned long long both = ((unsigned long long)w1 << 32) | w0;
            bits = (uint32_t)(both >> sb) & (uint32_t)((1ull << PER) - 1ull);
        }
        uint32_t nlds;
        const uint32_t off = block_exclusive_sum<TPB>(__popc(bits), s_w, &nlds);
        {
            // the word starts among this thread's positions (none past the tile)
            const uint32_t lo = PER * tid, wi = lo >> 5, sb = lo & 31u;
            uint32_t wsp = 0u;
            if (lo < TILE) {
                const uint32_t w0 = s_sb[wi];
                const uint32_t w1 = (wi + 1u < TILE / 32u) ? s_sb[wi + 1u] : 0u;
                wsp = (uint32_t)((((unsigned long long)w1 << 32) | w0) >> sb);
            }
            // bit k of ws: this thread's k-th token starts a word
            uint32_t ws = 0u, k = 0u;
            for (uint32_t m = bits; m; m &= m - 1u, ++k) {
                const uint32_t b = __ffs(m) - 1;
                ws |= ((wsp >> b) & 1u) << k;
                s_aux[off + k] = s_sym[PER * tid + b];
            }
            if (ws) {
                const uint32_t o = off & 31u;
                atomicOr(&s_ws[off >> 5], ws << o);
                if (o && (ws >> (32u - o))) atomicOr(&s_ws[(off >> 5) + 1u], ws >> (32u - o));
            }
        }
        __syncthreads();
        // the tile's region of CAP words: 16-bit ids from its start, the
        // word-start bits from word CAP / 2
        // (two ids per 4-byte store; the one past an odd count lies inside
        // the ids' part)
        uint32_t* d16 = tok32 + (size_t)t * CAP;
        uint32_t* dws = tok32 + (size_t)t * CAP + CAP / 2u;
        for (uint32_t i = tid; 2u * i < nlds; i += TPB) d16[i] = reinterpret_cast<const uint32_t*>(s_aux)[i];
        for (uint32_t i = tid; i < (nlds + 31u) / 32u; i += TPB) dws[i] = s_ws[i];
        if (tid == 0) {
            cnt[t] = nlds;
            ovf_pos[t] = s_ovf_pos;
            ovf_n[t] = s_ovf_n;
            atomicAdd(gsum + t / ENC_GROUP, nlds + s_ovf_n);
        }
    }
}

// status[0..3] (total, error flags, scratch used, spare) and the group sums
// gsum[0, ngroups) cleared.
__global__ void k_enc_init(uint32_t* status, uint32_t* gsum, uint32_t ngroups) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 4u) status[i] = 0u;
    for (uint32_t g = i; g < ngroups; g += gridDim.x * blockDim.x) gsum[g] = 0u;
}

// Exclusive scan of the group sums in place (one workgroup, each thread a
// contiguous run of them); the total into *total.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_enc_gscan(uint32_t* __restrict__ gsum, uint32_t ngroups, uint32_t* total) {
    __shared__ uint32_t s_w[TPB / 64];
    const uint32_t per = (ngroups + TPB - 1u) / TPB;
    const uint32_t lo = min(ngroups, threadIdx.x * per), hi = min(ngroups, lo + per);
    uint32_t sum = 0u;
    for (uint32_t g = lo; g < hi; ++g) sum += gsum[g];
    uint32_t all;
    uint32_t run = block_exclusive_sum<TPB>(sum, s_w, &all);
    for (uint32_t g = lo; g < hi; ++g) {
        const uint32_t x = gsum[g];
        gsum[g] = run;
        run += x;
    }
    if (threadIdx.x == 0) *total = all;
}

// Tile slices (16-bit ids and word-start bits, as the walk leaves them) to
// their places in out as 32-bit tokens, each tile's long last word's
// tokens after its own from the overflow area. A workgroup takes a group
// of ENC_GROUP tiles at a time: the tiles' counts and offsets within the
// group into LDS, then every (tile, 8 of its first CPT tokens) pair of the
// group, U pairs per thread with their loads in flight (consecutive
// threads on consecutive pairs of a tile: 16-byte id loads); tokens past
// CPT in a tile and the overflow tokens after.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_enc_copy(const uint32_t* __restrict__ tok32,
                                                  const uint32_t* __restrict__ cnt,
                                                  const uint32_t* __restrict__ ovf_pos,
                                                  const uint32_t* __restrict__ ovf_n,
                                                  const uint32_t* __restrict__ gpfx, const uint32_t* __restrict__ ovf,
                                                  uint32_t* __restrict__ out, uint32_t ntiles, uint32_t cap) {
    static_assert(ENC_GROUP == 64 && TPB >= 64, "a group's counts are scanned by one wave");
    constexpr uint32_t CPT = 512, PPT = CPT / 8u;  // tokens and pairs per tile in the main pass
    constexpr uint32_t U = 4;
    static_assert((ENC_GROUP * PPT) % (TPB * U) == 0, "pairs split evenly");
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    typedef uint32_t v4u __attribute__((ext_vector_type(4), aligned(4)));  // output: 4-byte aligned only
    __shared__ uint32_t s_off[ENC_GROUP], s_c[ENC_GROUP], s_no[ENC_GROUP], s_op[ENC_GROUP];
    const uint32_t tid = threadIdx.x;
    const uint32_t ngroups = (ntiles + ENC_GROUP - 1u) / ENC_GROUP;
    for (uint32_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const uint32_t t0 = g * ENC_GROUP;
        if (tid < 64u) {
            const uint32_t t = t0 + tid;
            const uint32_t c = t < ntiles ? cnt[t] : 0u, no = t < ntiles ? ovf_n[t] : 0u;
            uint32_t x = c + no;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = (uint32_t)__shfl_up((int)x, o);
                if (tid >= (uint32_t)o) x += y;
            }
            s_off[tid] = x - c - no;
            s_c[tid] = c;
            s_no[tid] = no;
            s_op[tid] = no ? ovf_pos[t] : 0u;
        }
        __syncthreads();
        uint32_t* o = out + gpfx[g];
        for (uint32_t p0 = tid; p0 < ENC_GROUP * PPT; p0 += TPB * U) {
            v4 ids[U];
            uint32_t ws[U];
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                const uint32_t p = p0 + TPB * u, j = p / PPT, k = 8u * (p % PPT);
                if (k < s_c[j]) {
                    const uint32_t* r = tok32 + (size_t)(t0 + j) * cap;
                    ids[u] = *reinterpret_cast<const v4*>(r + k / 2u);
                    ws[u] = r[cap / 2u + k / 32u] >> (k & 31u);
                }
            }
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                const uint32_t p = p0 + TPB * u, j = p / PPT, k = 8u * (p % PPT);
                const uint32_t c = s_c[j];
                if (k < c) {
                    uint32_t tk[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        tk[q] = ((ids[u][q >> 1] >> (16 * (q & 1))) & 0xFFFFu) | (((ws[u] >> q) & 1u) << 16);
                    uint32_t* d = o + s_off[j] + k;
                    if (k + 8u <= c) {
                        *reinterpret_cast<v4u*>(d) = v4u{tk[0], tk[1], tk[2], tk[3]};
                        *reinterpret_cast<v4u*>(d + 4) = v4u{tk[4], tk[5], tk[6], tk[7]};
                    } else {
#pragma unroll
                        for (int q = 0; q < 8; ++q)
                            if (k + (uint32_t)q < c) d[q] = tk[q];
                    }
                }
            }
        }
        // tokens past CPT (rare: a tile of mostly one-byte words), then the
        // long words' tokens: one wave per tile
        for (uint32_t j = tid >> 6; j < ENC_GROUP; j += TPB / 64u) {
            const uint32_t c = s_c[j], no = s_no[j];
            if (c <= CPT && !no) continue;
            const uint16_t* s16 = reinterpret_cast<const uint16_t*>(tok32 + (size_t)(t0 + j) * cap);
            const uint32_t* sws = tok32 + (size_t)(t0 + j) * cap + cap / 2u;
            uint32_t* d = o + s_off[j];
            for (uint32_t i = CPT + (tid & 63u); i < c; i += 64u)
                d[i] = (uint32_t)s16[i] | (((sws[i >> 5] >> (i & 31u)) & 1u) << 16);
            const uint32_t* ov = ovf + s_op[j];
            for (uint32_t i = tid & 63u; i < no; i += 64u) d[c + i] = ov[i];
        }
        __syncthreads();
    }
}

}  // namespace bpek
