// Training over the distinct words of a corpus (gfx950, wave64).
//
// Pairs are counted within words only and merges never cross a word start
// (page "bpe - GPU BPE Tokenizer Pipeline", "Ne Yapar? 1" and "Nedir bu
// ya?"), so every occurrence of a word is rewritten alike by every merge,
// and a pair's count is the sum over the distinct words containing it of
// (occurrences of the word) x (occurrences of the pair in it). Training can
// therefore run on each distinct word once, with its pair counts weighted
// by the word's frequency: the same counts, so the same merges, ties
// included. A corpus is turned into such chunks by
//   k_wc_insert (encode.hpp) over every tile: each word of 2..CK_MAXW bytes
//     claims a slot of a hash table keyed by its hash and length;
//   k_ck_record: each claimed slot gets its word's bytes;
//   k_ck_count: each word finds the slot holding exactly its bytes and
//     counts there (summed per workgroup in LDS first); a word without one
//     (longer, or lost to the probe limit) goes to a list of its own, one
//     chunk per occurrence;
//   k_ck_size, k_ck_build: the chunks with their symbols and weights. A
//     chunk of at most CK_MAXW symbols (the table's words, weighted by
//     their counts, and the short listed words) is a 64-byte record of
//     16-bit symbols, zero past its length, which one thread reads with
//     four 16-byte loads; a longer one (weight 1) lies in an array of its
//     own.
// The iterations take one of three routes: k_ck_small (at most 1,024
// record chunks, no long ones: every iteration in one workgroup, the pair
// counts in LDS); k_ck_solo (chunks_solo.hpp: no long chunks; every
// iteration in one workgroup, touching only the chunks on the merged
// pair's occurrence list); or k_ck_pairs, which counts the chunks' pairs
// into the global pair table, and k_ck_merge per iteration: the selection
// of merge.hpp (ticket 0 of a counter selects from the candidate list or
// calls a sweep, and publishes; the other workgroups load their first
// records meanwhile), then every chunk containing the pair is rewritten in
// place (left to right, without overlap) and its count changes are summed
// in LDS and added to the table.
// The tokens of the whole corpus come from the encoder afterwards: a
// learned list applied to its own training text gives the training tokens.
#pragma once

#include "encode.hpp"
#include "merge.hpp"

namespace bpek {

constexpr uint32_t CK_MAXW = WC_MAXLEN;  // longest word kept in the table
constexpr int CK_PF = 3;                 // records a thread of the merge pass loads during the selection
constexpr int CK_NB = 16;                // symbol filters a thread of the merge pass reads at once

// The listed words (one chunk per occurrence): text positions and lengths,
// n[0] of them (entries past cap are counted but not stored); n[1] of them
// are longer than CK_MAXW, with n[2] bytes in all.
struct CkList {
    uint32_t* pos;
    uint32_t* len;
    uint32_t* n;
    uint32_t cap;
};

// The chunks. Record chunks c < nr: symbols in rec[4c .. 4c + 4) (two per
// 32-bit word, the first in the low half; zero past the length when
// built), length rlen[c], weight rw[c], and a filter of the symbols it
// holds, rbloom[c] (bit ck_bit(s) set for each symbol s). Long chunks
// c < nl: symbols at lsym[loff[c] .. loff[c] + llen[c]), weight 1. A chunk
// only shrinks, in place.
struct Chunks {
    uint4* rec;
    uint32_t* rlen;
    uint32_t* rw;
    unsigned long long* rbloom;
    uint32_t nr;
    uint16_t* lsym;
    uint32_t* loff;
    uint32_t* llen;
    uint32_t nl;
};

// Maximum of a 64-bit value over the wave (every lane gets it): DPP row
// shifts, then the row broadcasts, on the two halves; no LDS round trip.
__device__ __forceinline__ unsigned long long wave_max64(unsigned long long v) {
    auto step = [&](uint32_t lo, uint32_t hi) {
        const unsigned long long o = ((unsigned long long)hi << 32) | lo;
        v = o > v ? o : v;
    };
    step(dpp<DPP_ROW_SHR1>(0u, (uint32_t)v), dpp<DPP_ROW_SHR1>(0u, (uint32_t)(v >> 32)));
    step(dpp<DPP_ROW_SHR2>(0u, (uint32_t)v), dpp<DPP_ROW_SHR2>(0u, (uint32_t)(v >> 32)));
    step(dpp<DPP_ROW_SHR4>(0u, (uint32_t)v), dpp<DPP_ROW_SHR4>(0u, (uint32_t)(v >> 32)));
    step(dpp<DPP_ROW_SHR8>(0u, (uint32_t)v), dpp<DPP_ROW_SHR8>(0u, (uint32_t)(v >> 32)));
    step(dpp<DPP_ROW_BCAST15, 0xA>(0u, (uint32_t)v), dpp<DPP_ROW_BCAST15, 0xA>(0u, (uint32_t)(v >> 32)));
    step(dpp<DPP_ROW_BCAST31, 0xC>(0u, (uint32_t)v), dpp<DPP_ROW_BCAST31, 0xC>(0u, (uint32_t)(v >> 32)));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

// ... and over the workgroup (NW waves; s_best holds NW values; two barriers).
template <int NW>
__device__ __forceinline__ unsigned long long block_max64(unsigned long long v, unsigned long long* s_best,
                                                          uint32_t lane, uint32_t w) {
    v = wave_max64(v);
    if (lane == 0) s_best[w] = v;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NW; ++i) v = s_best[i] > v ? s_best[i] : v;
    lds_barrier();
    return v;
}

// A symbol's bit in a chunk's filter (Fibonacci hashing to 6 bits).
__device__ __forceinline__ unsigned long long ck_bit(uint32_t s) { return 1ull << ((s * 0x9E3779B1u) >> 26); }

// The filter of the first len symbols of a record's 16 words.
__device__ __forceinline__ unsigned long long ck_filter(const uint32_t (&wds)[16], uint32_t len) {
    unsigned long long f = 0ull;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        if ((uint32_t)i < len) f |= ck_bit((wds[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu);
    return f;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
    return v;
}

// Appends the lanes' entries with take set, one counter atomic per wave
// (and two more when long words are among them). Called by all active
// lanes of the wave.
__device__ __forceinline__ void ck_list_append(const CkList& l, bool take, uint32_t pos, uint32_t len) {
    const unsigned long long m = __ballot(take);
    if (!m) return;
    const int lead = __ffsll((long long)m) - 1;
    const uint32_t below =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    uint32_t base = 0u;
    if ((int)(threadIdx.x & 63u) == lead) base = atomicAdd(l.n, (uint32_t)__popcll(m));
    base = (uint32_t)__shfl((int)base, lead);
    if (take && base + below < l.cap) {
        l.pos[base + below] = pos;
        l.len[base + below] = len;
    }
    const bool lg = take && len > CK_MAXW;
    const unsigned long long ml = __ballot(lg);
    if (ml) {
        const uint32_t bytes = wave_sum(lg ? len : 0u);
        if ((int)(threadIdx.x & 63u) == lead) {
            atomicAdd(l.n + 1, (uint32_t)__popcll(ml));
            atomicAdd(l.n + 2, bytes);
        }
    }
}

// Every claimed slot's record gets the bytes of its word (the claimer's
// text position, the key's length), zero past the length; a slot whose
// range is not inside the text gets no bytes and matches nothing.
__global__ void k_ck_record(const uint8_t* __restrict__ text, uint32_t n, WordCache wc, uint32_t slots) {
    for (uint32_t s = blockIdx.x * blockDim.x + threadIdx.x; s < slots; s += gridDim.x * blockDim.x) {
        const unsigned long long k = wc.key[s];
        if (!k) continue;
        const uint32_t len = (uint32_t)(k & 63ull), at = wc.pos[s];
        uint32_t* rp = wc.rec + (size_t)s * 8u;
        if (len > CK_MAXW || at > n || n - at < len) {
            // (a claimer's word always lies inside the text) bytes that no
            // packed word shorter than 32 bytes has; the 32-byte word of
            // these bytes would match, and its chunk be these bytes: right
            for (int j = 0; j < 8; ++j) rp[j] = 0xFFFFFFFFu;
            continue;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t v = 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = 4u * (uint32_t)j + (uint32_t)u;
                if (i < len) v |= (uint32_t)text[at + i] << (8 * u);
            }
            rp[j] = v;
        }
    }
}

// The slot whose key and record hold exactly the packed word w of length
// len (probing from its home slot up to WC_PROBES slots, stopping at a free
// slot); NO_SLOT if none.
__device__ __forceinline__ uint32_t ck_find(const WordCache& wc, unsigned long long key, uint32_t slot,
                                            const uint32_t (&w)[8]) {
    for (uint32_t p = 0; p < WC_PROBES; ++p) {
        const unsigned long long v = wc.key[slot];
        if (v == 0ull) return NO_SLOT;
        if (v == key) {
            const uint32_t* rp = wc.rec + (size_t)slot * 8u;
            uint32_t d = 0u;
#pragma unroll
            for (int j = 0; j < 8; ++j) d |= rp[j] ^ w[j];
            if (d == 0u) return slot;
        }
        slot = (slot + 1u) & wc.mask;
    }
    return NO_SLOT;
}

// Occurrences of every word of two bytes or more: 256-thread workgroups on
// the walk's tiles (TILE = 16 TPB bytes and the halo in LDS). A word found
// in the table adds one to its slot's count (summed per workgroup in an LDS
// table keyed by the slot, added to cnt when the tile is done); any other
// word goes to the list. One-byte words have no pairs and are left out.
template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_ck_count(const uint8_t* __restrict__ text, uint32_t n, uint32_t ntiles,
                                                  WordCache wc, uint32_t* __restrict__ cnt, CkList list) {
    constexpr uint32_t TILE = TPB * 16u;
    constexpr uint32_t HALO = TPB * TRIE_HALO_PER_THREAD;
    constexpr uint32_t CAP = TILE + HALO;
    constexpr uint32_t NCH = (CAP + 32u) / 16u;
    static_assert(HALO > CK_MAXW, "a tabled word ends inside the copy");
    __shared__ __align__(16) uint8_t s_txt[NCH * 16u];
    __shared__ uint32_t s_sb[TILE / 32u];
    __shared__ uint16_t s_list[TILE];
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_after;
    __shared__ LdsTable<LT> tab;

    const uint32_t tid = threadIdx.x;
    const uint32_t mis = (uint32_t)((uintptr_t)text & 15u);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(text - mis), 0, (int)((n + mis + 15u) & ~15u), 0x00020000);
    const uint32_t sh = 16u + mis;
    tab.clear(TPB);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
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
        __syncthreads();
        const uint32_t lim = nrel < CAP ? nrel : CAP;
        const uint32_t last_end = s_after < lim ? s_after : lim;
        const bool last_open = s_after >= CAP && lim < nrel;
        for (uint32_t i0 = 0; i0 < nwords; i0 += TPB) {  // uniform trip count: the list append is wave-wide
            const uint32_t i = i0 + tid;
            bool to_list = false;
            uint32_t q = 0u, len = 0u;
            if (i < nwords) {
                q = s_list[i];
                const uint32_t wend = word_end<TILE>(s_sb, q, last_end);
                len = wend - q;
                if (last_open && wend == last_end) {
                    // runs past the copy: its length from global memory
                    const uint32_t cls = byte_class(s_txt[q + sh]);
                    uint32_t e = lim;
                    while (e < nrel && byte_class(text[(size_t)t0 + e]) == cls) ++e;
                    len = e - q;
                }
                uint32_t slot = NO_SLOT;
                if (len <= CK_MAXW) {
                    uint32_t w[8];
                    wc_pack_lds(s_txt, q + sh, len, w);
                    const uint32_t h = wc_hash(w, len);
                    slot = ck_find(wc, wc_key(wc, h, len), wc_slot(wc, h), w);
                }
                if (slot != NO_SLOT) {
                    if (!tab.insert(slot, 1u)) atomicAdd(cnt + slot, 1u);
                } else {
                    to_list = true;
                }
            }
            ck_list_append(list, to_list, t0 + q, len);
        }
        __syncthreads();  // the tile's counts are in LDS
        if (tab.used > LT / 2 || t + gridDim.x >= ntiles) {  // uniform
            for (uint32_t s = tid; s < (uint32_t)LT; s += TPB) {
                const uint32_t k = tab.keys[s], c = tab.cnts[s];
                if (k != EMPTY && c) atomicAdd(cnt + k, c);
                tab.keys[s] = EMPTY;
                tab.cnts[s] = 0u;
            }
            if (tid == 0) tab.used = 0u;
        }
        __syncthreads();
    }
}

// sizes[0] += the slots with a count (the table's chunks); one atomic per
// workgroup.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_ck_size(const uint32_t* __restrict__ cnt, uint32_t slots, uint32_t* sizes) {
    __shared__ uint32_t s_w[TPB / 64];
    uint32_t c = 0u;
    for (uint32_t i = blockIdx.x * TPB + threadIdx.x; i < slots; i += gridDim.x * TPB) c += cnt[i] ? 1u : 0u;
    c = wave_sum(c);
    if ((threadIdx.x & 63u) == 0u) s_w[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0u;
#pragma unroll
        for (int k = 0; k < TPB / 64; ++k) t += s_w[k];
        if (t) atomicAdd(sizes, t);
    }
}

// Four bytes (little-endian in x) as four 16-bit symbols in two words.
__device__ __forceinline__ uint2 ck_widen(uint32_t x) {
    return make_uint2((x & 0xFFu) | ((x & 0xFF00u) << 8), ((x >> 16) & 0xFFu) | ((x >> 8) & 0xFF0000u));
}

// The chunks, in any order (the counts and the merges do not depend on
// it). Each workgroup takes a contiguous range of the slots and one of the
// nlist listed words, counts the chunks of each kind its range makes, and
// takes their places with one atomic per counter: ctr[0] record chunks,
// ctr[1] long chunks, ctr[2] long chunks' symbols (all zero before).
template <int TPB>
__global__ __launch_bounds__(TPB) void k_ck_build(const uint8_t* __restrict__ text, WordCache wc,
                                                  const uint32_t* __restrict__ cnt, uint32_t slots, CkList list,
                                                  uint32_t nlist, Chunks ck, uint32_t* ctr) {
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_base[3];
    const uint32_t tid = threadIdx.x;
    {  // the table's words: the record's bytes widened, weight = count
        const uint32_t per = (slots + gridDim.x - 1u) / gridDim.x;
        const uint32_t lo = min(slots, blockIdx.x * per), hi = min(slots, lo + per);
        uint32_t mine = 0u;
        for (uint32_t i = lo + tid; i < hi; i += TPB) mine += cnt[i] ? 1u : 0u;
        uint32_t all;
        const uint32_t off = block_exclusive_sum<TPB>(mine, s_w, &all);
        if (tid == 0) s_base[0] = all ? atomicAdd(ctr, all) : 0u;
        __syncthreads();
        uint32_t c = s_base[0] + off;
        for (uint32_t i = lo + tid; i < hi; i += TPB) {
            const uint32_t k = cnt[i];
            if (!k) continue;
            const uint4* src = reinterpret_cast<const uint4*>(wc.rec + (size_t)i * 8u);
            const uint4 a = src[0], b = src[1];
            const uint32_t bytes[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t wds[16];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint2 x = ck_widen(bytes[j]);
                wds[2 * j] = x.x;
                wds[2 * j + 1] = x.y;
            }
            uint4* dst = ck.rec + 4u * (size_t)c;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = make_uint4(wds[4 * j], wds[4 * j + 1], wds[4 * j + 2], wds[4 * j + 3]);
            const uint32_t len = (uint32_t)(wc.key[i] & 63ull);
            ck.rlen[c] = len;
            ck.rw[c] = k;
            ck.rbloom[c] = ck_filter(wds, len);
            ++c;
        }
        __syncthreads();  // s_base is reused below
    }
    {  // the listed words, weight 1: short ones as records, long ones as they are
        const uint32_t per = (nlist + gridDim.x - 1u) / gridDim.x;
        const uint32_t lo = min(nlist, blockIdx.x * per), hi = min(nlist, lo + per);
        uint32_t ns = 0u, nl = 0u, nb = 0u;
        for (uint32_t i = lo + tid; i < hi; i += TPB) {
            const uint32_t len = list.len[i];
            if (len > CK_MAXW) {
                ++nl;
                nb += len;
            } else {
                ++ns;
            }
        }
        uint32_t as, al, ab;
        uint32_t os = block_exclusive_sum<TPB>(ns, s_w, &as);
        uint32_t ol = block_exclusive_sum<TPB>(nl, s_w, &al);
        uint32_t ob = block_exclusive_sum<TPB>(nb, s_w, &ab);
        if (tid == 0) {
            s_base[0] = as ? atomicAdd(ctr + 0, as) : 0u;
            s_base[1] = al ? atomicAdd(ctr + 1, al) : 0u;
            s_base[2] = ab ? atomicAdd(ctr + 2, ab) : 0u;
        }
        __syncthreads();
        os += s_base[0];
        ol += s_base[1];
        ob += s_base[2];
        for (uint32_t i = lo + tid; i < hi; i += TPB) {
            const uint32_t at = list.pos[i], len = list.len[i];
            if (len > CK_MAXW) {
                for (uint32_t j = 0; j < len; ++j) ck.lsym[ob + j] = text[at + j];
                ck.loff[ol] = ob;
                ck.llen[ol] = len;
                ++ol;
                ob += len;
            } else {
                uint32_t wds[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t q = 2u * (uint32_t)j;
                    wds[j] = (q < len ? (uint32_t)text[at + q] : 0u) |
                             (q + 1u < len ? (uint32_t)text[at + q + 1u] << 16 : 0u);
                }
                uint4* dst = ck.rec + 4u * (size_t)os;
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[j] = make_uint4(wds[4 * j], wds[4 * j + 1], wds[4 * j + 2], wds[4 * j + 3]);
                ck.rlen[os] = len;
                ck.rw[os] = 1u;
                ck.rbloom[os] = ck_filter(wds, len);
                ++os;
            }
        }
    }
}

// A record's 32 symbols, in 16 words.
struct CkRec {
    uint32_t v[16];
    __device__ __forceinline__ void load(const Chunks& ck, uint32_t c) {
        const uint4* rp = ck.rec + 4u * (size_t)c;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 q = rp[j];
            v[4 * j] = q.x;
            v[4 * j + 1] = q.y;
            v[4 * j + 2] = q.z;
            v[4 * j + 3] = q.w;
        }
    }
    // symbol i (i a constant after unrolling)
    __device__ __forceinline__ uint32_t sym(int i) const { return (v[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu; }
};

// Symbol i of a record row in LDS, and its replacement. The row is only
// ever accessed as 32-bit words, so that no access through another type
// can be reordered around the row's stores.
__device__ __forceinline__ uint32_t row_sym(const uint32_t* row, uint32_t i) {
    return (row[i >> 1] >> ((i & 1u) * 16u)) & 0xFFFFu;
}
__device__ __forceinline__ void row_set(uint32_t* row, uint32_t i, uint32_t v) {
    const uint32_t sh = (i & 1u) * 16u;
    row[i >> 1] = (row[i >> 1] & ~(0xFFFFu << sh)) | (v << sh);
}

// Bits 1 .. len - 1: the pairs (i - 1, i) of a chunk of len symbols.
__device__ __forceinline__ uint32_t ck_pair_mask(uint32_t len) {
    return len >= 32u ? 0xFFFFFFFEu : (len >= 2u ? (1u << len) - 2u : 0u);
}

// Every adjacent pair of every chunk, weighted by the chunk's count, into
// the global table (summed per workgroup in LDS first).
template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_ck_pairs(Chunks ck, GTable gt, Ctl* ctl) {
    __shared__ LdsTable<LT> tab;
    tab.clear(TPB);
    lds_barrier();
    const uint32_t stride = gridDim.x * TPB;
    for (uint32_t c = blockIdx.x * TPB + threadIdx.x; c < ck.nr; c += stride) {
        CkRec r;
        r.load(ck, c);
        const uint32_t pm = ck_pair_mask(ck.rlen[c]), w = ck.rw[c];
#pragma unroll
        for (int i = 1; i < 32; ++i)
            if ((pm >> i) & 1u) {
                const uint32_t key = (r.sym(i - 1) << 16) | r.sym(i);
                if (!tab.insert(key, w)) gt_add(gt, key, w, ctl);
            }
    }
    for (uint32_t c = blockIdx.x * TPB + threadIdx.x; c < ck.nl; c += stride) {
        const uint16_t* s = ck.lsym + ck.loff[c];
        const uint32_t len = ck.llen[c];
        uint32_t prev = s[0];
        for (uint32_t j = 1; j < len; ++j) {
            const uint32_t x = s[j];
            const uint32_t key = (prev << 16) | x;
            if (!tab.insert(key, 1u)) gt_add(gt, key, 1u, ctl);
            prev = x;
        }
    }
    lds_barrier();
    for (int i = threadIdx.x; i < LT; i += TPB) {
        const uint32_t key = tab.keys[i], c = tab.cnts[i];
        if (key != EMPTY && c) gt_add(gt, key, c, ctl);
    }
}

// Bit k: chunk c0 + k stride (below ck->nr) may hold both symbols of need
// (two filter bits; both set is necessary, not sufficient). With ck, the
// CK_NB filters are read into bl first (all loads in flight together);
// without it, bl already holds them.
__device__ __forceinline__ uint32_t ck_hits(unsigned long long (&bl)[CK_NB], unsigned long long need,
                                            const Chunks* ck, uint32_t c0, uint32_t stride) {
    if (ck) {
#pragma unroll
        for (int k = 0; k < CK_NB; ++k) {
            const uint32_t ci = c0 + (uint32_t)k * stride;
            bl[k] = ci < ck->nr ? ck->rbloom[ci] : 0ull;
        }
    }
    uint32_t hits = 0u;
#pragma unroll
    for (int k = 0; k < CK_NB; ++k) hits |= (bl[k] & need) == need ? 1u << k : 0u;
    return hits;
}

// One training iteration over the chunks (launch it; a launch after
// training has stopped does nothing). The selection is merge.hpp's: the
// workgroup that draws ticket 0 of the iteration's counter selects and
// publishes, every workgroup reads the publication (and joins a sweep when
// it says so); a thread's first record is loaded before that wait. Then
// each thread rewrites its chunks that contain the merged pair: in place,
// left to right without overlap, each occurrence of (L, R) becoming X.
// With the chunk's weight, every old pair with a side inside a merged
// occurrence is taken out and every new pair with a side X is put in; the
// other pairs map one to one onto each other (X is a new id), so this is
// the chunk's exact recount. The keys taken out all hold L or R and those
// put in all hold X, so a key only falls or only rises in a launch, as the
// candidate list requires. The changes are summed in LDS and go to the
// table once the workgroup is done.
template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_ck_merge(uint32_t it, Ctl* ctl, Chunks ck, GTable gt, Sweep* sw,
                                                  uint32_t* merges) {
    __shared__ LdsTable<LT> tab;
    __shared__ uint32_t s_rec[TPB * 17];  // a thread's record being rewritten (rows padded: no bank conflicts)
    __shared__ uint32_t s_tile[2], s_u32, s_w[TPB / 64];
    __shared__ unsigned long long s_best[TPB / 64];
    if (ctl->done) return;
    const uint32_t p = it & 1u;
    const uint32_t X = BASE + it;
    const bool do_count = X != IDM;  // X = 65535 is the last id: nothing reads counts after it
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* tick = &ctl->tile_ctr[p];
    uint32_t* const my_rec = s_rec + 17u * tid;
    if (blockIdx.x == 0 && tid == 0) {
        // the counters of the next iteration (the previous one's are done with)
        __hip_atomic_store(&ctl->tile_ctr[p ^ 1u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st_agent(&sw->c1[p ^ 1u], 0u);
        st_agent(&sw->c1done[p ^ 1u], 0u);
        st_agent(&sw->c2[p ^ 1u], 0u);
        st_agent(&sw->smax[p ^ 1u], 0ull);
    }
    tab.clear(TPB);
    if (tid == 0) s_tile[0] = atomicAdd(tick, 1u);
    uint32_t theta = sw->theta;
    lds_barrier();
    if (s_tile[0] == 0u) select_and_publish<TPB>(gt, sw, p, it, theta, s_best, lane, w);  // uniform
    const uint32_t stride = gridDim.x * TPB;
    uint32_t c = blockIdx.x * TPB + tid;
    // A thread's record chunks are c, c + stride, ..., taken in batches of
    // CK_NB whose filters are read together; a record is read only when its
    // filter holds both L and R. The first batch's filters and its first
    // CK_PF records are in flight during the wait for the publication.
    unsigned long long bl[CK_NB];
#pragma unroll
    for (int k = 0; k < CK_NB; ++k) {
        const uint32_t ci = c + (uint32_t)k * stride;
        bl[k] = ci < ck.nr ? ck.rbloom[ci] : 0ull;
    }
    CkRec r[CK_PF];
    uint32_t rl[CK_PF], rw[CK_PF];
#pragma unroll
    for (int k = 0; k < CK_PF; ++k) {
        const uint32_t ci = c + (uint32_t)k * stride;
        rl[k] = 0u;
        rw[k] = 0u;
        if (ci < ck.nr) {
            r[k].load(ck, ci);
            rl[k] = ck.rlen[ci];
            rw[k] = ck.rw[ci];
        }
    }
    unsigned long long best = read_publication(sw, ctl, p, it, s_best);
    if (best == SEL_SWEEP) best = sweep_select<TPB>(gt, sw, ctl, p, it, s_best, &s_u32, lane, w, theta);
    if (best == 0ull) {  // uniform: no countable pair is left
        if (blockIdx.x == 0 && tid == 0) st_agent(&ctl->done, 1u);
        return;
    }
    const uint32_t key = __builtin_amdgcn_readfirstlane(~(uint32_t)best);
    const uint32_t L = key >> 16, R = key & IDM;
    if (blockIdx.x == 0 && tid == 0) {
        merges[3 * it + 0] = L;
        merges[3 * it + 1] = R;
        merges[3 * it + 2] = (uint32_t)(best >> 32);
        ctl->L = L;
        ctl->R = R;
        ctl->X = X;
        ctl->k = it + 1;
        ctl->m = it + 1;
    }
    auto add = [&](uint32_t a, uint32_t b, uint32_t d) {
        const uint32_t k = (a << 16) | b;
        if (!tab.insert(k, d)) gt_add_sel(gt, k, d, ctl, sw, theta);
    };
    const unsigned long long need = ck_bit(L) | ck_bit(R);
    for (uint32_t b0 = 0u; c + b0 * stride < ck.nr; b0 += (uint32_t)CK_NB)
    for (uint32_t hits = ck_hits(bl, need, b0 ? &ck : nullptr, c + b0 * stride, stride); hits; hits &= hits - 1u) {
        const uint32_t k = (uint32_t)__ffs(hits) - 1u;
        const uint32_t cc = c + (b0 + k) * stride;
        CkRec cur;
        uint32_t len = 0u, wt = 0u;
        bool got = false;
#pragma unroll
        for (int j = 0; j < CK_PF; ++j)
            if (b0 == 0u && k == (uint32_t)j) {
                cur = r[j];
                len = rl[j];
                wt = rw[j];
                got = true;
            }
        if (!got) {
            cur.load(ck, cc);
            len = ck.rlen[cc];
            wt = ck.rw[cc];
        }
        const uint32_t pm = ck_pair_mask(len);
        uint32_t occ = 0u;  // bit i: the pair (i - 1, i) is (L, R)
#pragma unroll
        for (int i = 1; i < 32; ++i) occ |= (cur.sym(i - 1) == L && cur.sym(i) == R) ? 1u << i : 0u;
        occ &= pm;
        if (occ) {
            // bit i of sel: (i - 1, i) is merged (left to right without
            // overlap: in a run of occurrences of (L, L), every other one)
            uint32_t sel = occ;
            if (L == R) {
                sel = 0u;
                uint32_t prev = 0u;
#pragma unroll
                for (int i = 1; i < 32; ++i) {
                    const uint32_t b = (occ >> i) & 1u & (prev ^ 1u);
                    sel |= b << i;
                    prev = b;
                }
            }
            const uint32_t site = sel | (sel >> 1);              // positions in a merged occurrence
            const uint32_t changed = (site | (site << 1)) & pm;  // old pairs with a side in one
            const uint32_t minus = (uint32_t)(-(int)wt);
            // the old symbols, read at variable positions below
#pragma unroll
            for (int j = 0; j < 16; ++j) my_rec[j] = cur.v[j];
            if (do_count)
                for (uint32_t m = changed; m; m &= m - 1u) {
                    const uint32_t i = (uint32_t)__ffs(m) - 1u;
                    add(row_sym(my_rec, i - 1u), row_sym(my_rec, i), minus);
                }
            uint16_t* dst = reinterpret_cast<uint16_t*>(ck.rec + 4u * (size_t)cc);
            uint32_t o = 0u, pv = 0u;
            unsigned long long f = 0ull;
#pragma unroll 1
            for (uint32_t i = 0; i < len; ++i) {
                if ((sel >> i) & 1u) continue;  // the right half of a merged occurrence
                const bool mx = i < 31u && ((sel >> (i + 1u)) & 1u);
                const uint32_t cur = mx ? X : row_sym(my_rec, i);
                dst[o] = (uint16_t)cur;
                f |= ck_bit(cur);
                if (do_count && o && (pv == X || cur == X)) add(pv, cur, wt);
                pv = cur;
                ++o;
            }
            ck.rlen[cc] = o;
            ck.rbloom[cc] = f;
        }
    }
    for (uint32_t cl = blockIdx.x * TPB + tid; cl < ck.nl; cl += stride) {
        const uint32_t n = ck.llen[cl];
        uint16_t* s = ck.lsym + ck.loff[cl];
        // a quick look first: most chunks do not hold the pair
        bool has = false;
        for (uint32_t j = 1; j < n && !has; ++j) has = s[j - 1] == L && s[j] == R;
        if (!has) continue;
        const uint32_t minus = 0xFFFFFFFFu;  // weight 1
        // old pair (j-1, j) is looked at when j is reached; prev is the old
        // symbol at j-1 (the output may have overwritten it), in_site says
        // whether j-1 was inside a merged occurrence
        uint32_t o = 0, prev = 0u;
        bool in_site = false;
        for (uint32_t j = 0; j < n;) {
            const uint32_t a = s[j];
            if (a == L && j + 1u < n && s[j + 1u] == R) {
                if (do_count) {
                    if (j) add(prev, L, minus);
                    add(L, R, minus);
                }
                prev = R;
                in_site = true;
                s[o++] = (uint16_t)X;
                j += 2u;
            } else {
                if (do_count && in_site) add(prev, a, minus);
                prev = a;
                in_site = false;
                s[o++] = (uint16_t)a;
                j += 1u;
            }
        }
        ck.llen[cl] = o;
        if (do_count)
            for (uint32_t j = 1; j < o; ++j)
                if (s[j - 1] == X || s[j] == X) add(s[j - 1], s[j], 1u);
    }
    // the summed changes, one per thread at a time: the non-empty entries
    // first gathered (in the record rows, free now), so that no thread adds
    // several of them one after another while others idle
    lds_barrier();
    uint32_t mine = 0u;
    for (uint32_t i = tid; i < (uint32_t)LT; i += TPB) mine += (tab.keys[i] != EMPTY && tab.cnts[i] != 0u) ? 1u : 0u;
    uint32_t total;
    uint32_t at = block_exclusive_sum<TPB>(mine, s_w, &total);
    static_assert(2 * LT <= 17 * TPB, "the gathered entries fit the record rows");
    for (uint32_t i = tid; i < (uint32_t)LT; i += TPB)
        if (tab.keys[i] != EMPTY && tab.cnts[i] != 0u) {
            s_rec[2u * at] = tab.keys[i];
            s_rec[2u * at + 1u] = tab.cnts[i];
            ++at;
        }
    lds_barrier();
    for (uint32_t i = tid; i < total; i += TPB) gt_add_sel(gt, s_rec[2u * i], s_rec[2u * i + 1u], ctl, sw, theta);
}

// ---------------------------------------------------------------- one workgroup, every iteration
// Training over at most TPB record chunks (no long ones) in one workgroup
// and one launch: each thread holds one chunk's record in registers for the
// whole run, the weighted pair counts live in an LDS hash table of LT
// slots (linear probing; a claimed slot keeps its key), and an iteration is
// a maximum over that table, the rewrite of the chunks that hold the pair
// with their count changes (the same exact recount as k_ck_merge), and a
// barrier. The maximum is the same packed value as the multi-workgroup
// path's (count << 32 | ~key over the nonzero counts), so the merges are
// the same. If the LDS table fills, ERR_LDS_FULL is set and nothing of the
// run is used: the caller trains with the multi-workgroup path instead.
constexpr uint32_t ERR_LDS_FULL = 4u;

template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_ck_small(Chunks ck, uint32_t n_merges, uint32_t* merges, Ctl* ctl) {
    static_assert((LT & (LT - 1)) == 0 && LT % TPB == 0, "LT: a power of two, a multiple of TPB");
    __shared__ uint32_t t_key[LT], t_cnt[LT];
    __shared__ uint32_t s_rec[TPB * 17];  // a thread's record being rewritten (rows padded: no bank conflicts)
    __shared__ unsigned long long s_best[TPB / 64];
    __shared__ uint32_t s_full;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
    for (uint32_t i = tid; i < (uint32_t)LT; i += TPB) {
        t_key[i] = EMPTY;
        t_cnt[i] = 0u;
    }
    if (tid == 0) s_full = 0u;
    const bool mine = tid < ck.nr;
    CkRec r;
    uint32_t len = 0u, wt = 0u;
    if (mine) {
        r.load(ck, tid);
        len = ck.rlen[tid];
        wt = ck.rw[tid];
    }
    uint32_t* const my_rec = s_rec + 17u * tid;
    auto add = [&](uint32_t a, uint32_t b, uint32_t d) {
        const uint32_t key = (a << 16) | b;
        uint32_t h = mix32(key) & (uint32_t)(LT - 1);
        for (uint32_t p = 0; p < (uint32_t)LT; ++p, h = (h + 1u) & (uint32_t)(LT - 1)) {
            uint32_t cur = __hip_atomic_load(&t_key[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (cur == EMPTY) {
                cur = atomicCAS(&t_key[h], EMPTY, key);
                if (cur == EMPTY) cur = key;
            }
            if (cur == key) {
                atomicAdd(&t_cnt[h], d);
                return;
            }
        }
        s_full = 1u;
    };
    __syncthreads();
    if (mine) {
        const uint32_t pm = ck_pair_mask(len);
#pragma unroll
        for (int i = 1; i < 32; ++i)
            if ((pm >> i) & 1u) add(r.sym(i - 1), r.sym(i), wt);
    }
    __syncthreads();
    uint32_t it = 0;
    for (; it < n_merges && !s_full; ++it) {  // s_full: read after a barrier, uniform
        unsigned long long best = 0ull;
        for (uint32_t i = tid; i < (uint32_t)LT; i += TPB) {
            const uint32_t c = t_cnt[i];
            const unsigned long long v = c ? ((unsigned long long)c << 32) | (uint32_t)~t_key[i] : 0ull;
            best = v > best ? v : best;
        }
        best = block_max64<TPB / 64>(best, s_best, lane, w);
        if (best == 0ull) break;  // uniform: no pair is left
        const uint32_t key = ~(uint32_t)best;
        const uint32_t L = key >> 16, R = key & IDM, X = BASE + it;
        const bool do_count = X != IDM;
        if (tid == 0) {
            merges[3 * it + 0] = L;
            merges[3 * it + 1] = R;
            merges[3 * it + 2] = (uint32_t)(best >> 32);
        }
        const uint32_t pm = ck_pair_mask(len);
        uint32_t occ = 0u;
#pragma unroll
        for (int i = 1; i < 32; ++i) occ |= (r.sym(i - 1) == L && r.sym(i) == R) ? 1u << i : 0u;
        occ &= pm;
        if (occ) {
            uint32_t sel = occ;
            if (L == R) {
                sel = 0u;
                uint32_t prev = 0u;
#pragma unroll
                for (int i = 1; i < 32; ++i) {
                    const uint32_t b = (occ >> i) & 1u & (prev ^ 1u);
                    sel |= b << i;
                    prev = b;
                }
            }
            const uint32_t site = sel | (sel >> 1);
            const uint32_t changed = (site | (site << 1)) & pm;
            const uint32_t minus = (uint32_t)(-(int)wt);
#pragma unroll
            for (int j = 0; j < 16; ++j) my_rec[j] = r.v[j];
            if (do_count)
                for (uint32_t m = changed; m; m &= m - 1u) {
                    const uint32_t i = (uint32_t)__ffs(m) - 1u;
                    add(row_sym(my_rec, i - 1u), row_sym(my_rec, i), minus);
                }
            // in place in the row: position o <= i is written after i is read
            uint32_t o = 0u, pv = 0u;
#pragma unroll 1
            for (uint32_t i = 0; i < len; ++i) {
                if ((sel >> i) & 1u) continue;
                const bool mx = i < 31u && ((sel >> (i + 1u)) & 1u);
                const uint32_t cur = mx ? X : row_sym(my_rec, i);
                row_set(my_rec, o, cur);
                if (do_count && o && (pv == X || cur == X)) add(pv, cur, wt);
                pv = cur;
                ++o;
            }
            len = o;
#pragma unroll
            for (int j = 0; j < 16; ++j) r.v[j] = my_rec[j];
        }
        __syncthreads();  // every count change is in before the next maximum
    }
    if (tid == 0) {
        ctl->k = it;
        ctl->m = it;
        ctl->done = 1u;
        if (s_full) ctl->err |= ERR_LDS_FULL;
    }
}

}  // namespace bpek
