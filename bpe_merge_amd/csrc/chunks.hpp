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
//   k_ck_size, k_ck_build: the chunks (slots with a count, then the listed
//     words) with their symbols, lengths and weights.
// k_ck_pairs counts the chunks' pairs into the global pair table, and
// k_ck_merge runs one iteration: the selection of merge.hpp (ticket 0 of a
// counter selects from the candidate list or calls a sweep, and publishes),
// then every chunk containing the pair is rewritten in place (left to
// right, without overlap) and its count changes are summed in LDS and
// added to the table. The tokens of the whole corpus come from the
// encoder afterwards: a learned list applied to its own training text
// gives the training tokens.
#pragma once

#include "encode.hpp"
#include "merge.hpp"

namespace bpek {

constexpr uint32_t CK_MAXW = WC_MAXLEN;  // longest word kept in the table

// The listed words (one chunk per occurrence): text positions and lengths,
// *n of them (entries past cap are counted but not stored).
struct CkList {
    uint32_t* pos;
    uint32_t* len;
    uint32_t* n;
    uint32_t cap;
};

// The chunks: symbols of chunk c at sym[off[c] .. off[c] + len[c]) (16-bit
// ids; a chunk only shrinks, in place), weight w[c] = its occurrences.
struct Chunks {
    uint16_t* sym;
    uint32_t* off;
    uint32_t* len;
    uint32_t* w;
    uint32_t n;
};

// Appends the lanes' entries with take set, one counter atomic per wave.
// Called by all active lanes of the wave.
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

// sizes[0] += chunks of the table (slots with a count), sizes[1] += their
// symbols; one atomic pair per wave.
__global__ void k_ck_size(WordCache wc, const uint32_t* __restrict__ cnt, uint32_t slots, uint32_t* sizes) {
    uint32_t c = 0u, s = 0u;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < slots; i += gridDim.x * blockDim.x)
        if (cnt[i]) {
            ++c;
            s += (uint32_t)(wc.key[i] & 63ull);
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        c += (uint32_t)__shfl_xor((int)c, o);
        s += (uint32_t)__shfl_xor((int)s, o);
    }
    if ((threadIdx.x & 63u) == 0u && (c | s)) {
        atomicAdd(sizes + 0, c);
        atomicAdd(sizes + 1, s);
    }
}

// The chunks, in any order (the counts and the merges do not depend on it):
// table chunks take their index and symbol range from two counters ctr[0],
// ctr[1] (zero before; one atomic pair per wave); the listed words follow
// as chunks n_table.., their symbols at list_base + list_off[k] (list_off:
// exclusive sums of the listed lengths).
__global__ void k_ck_build(const uint8_t* __restrict__ text, WordCache wc, const uint32_t* __restrict__ cnt,
                           uint32_t slots, CkList list, const uint32_t* __restrict__ list_off, uint32_t n_table,
                           uint32_t list_base, Chunks ck, uint32_t* ctr) {
    const uint32_t lane = threadIdx.x & 63u;
    for (uint32_t i0 = blockIdx.x * blockDim.x; i0 < slots; i0 += gridDim.x * blockDim.x) {
        const uint32_t i = i0 + threadIdx.x;
        const uint32_t c = i < slots ? cnt[i] : 0u;
        const uint32_t len = c ? (uint32_t)(wc.key[i] & 63ull) : 0u;
        // wave-wide exclusive sums of the chunk flags and lengths
        uint32_t ci = c ? 1u : 0u, li = len;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t a = (uint32_t)__shfl_up((int)ci, o), b = (uint32_t)__shfl_up((int)li, o);
            if (lane >= (uint32_t)o) {
                ci += a;
                li += b;
            }
        }
        const uint32_t tc = (uint32_t)__shfl((int)ci, 63), tl = (uint32_t)__shfl((int)li, 63);
        uint32_t bc = 0u, bl = 0u;
        if (lane == 63u && tc) {
            bc = atomicAdd(ctr + 0, tc);
            bl = atomicAdd(ctr + 1, tl);
        }
        bc = (uint32_t)__shfl((int)bc, 63) + ci - (c ? 1u : 0u);
        bl = (uint32_t)__shfl((int)bl, 63) + li - len;
        if (c) {
            const uint32_t* rp = wc.rec + (size_t)i * 8u;
            for (uint32_t j = 0; j < len; ++j) ck.sym[bl + j] = (uint16_t)((rp[j >> 2] >> (8u * (j & 3u))) & 0xFFu);
            ck.off[bc] = bl;
            ck.len[bc] = len;
            ck.w[bc] = c;
        }
    }
    const uint32_t nl = min(*list.n, list.cap);
    for (uint32_t k = blockIdx.x * blockDim.x + threadIdx.x; k < nl; k += gridDim.x * blockDim.x) {
        const uint32_t c = n_table + k, at = list.pos[k], len = list.len[k], o = list_base + list_off[k];
        for (uint32_t j = 0; j < len; ++j) ck.sym[o + j] = text[at + j];
        ck.off[c] = o;
        ck.len[c] = len;
        ck.w[c] = 1u;
    }
}

// Every adjacent pair of every chunk, weighted by the chunk's count, into
// the global table (summed per workgroup in LDS first).
template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_ck_pairs(Chunks ck, GTable gt, Ctl* ctl) {
    __shared__ LdsTable<LT> tab;
    tab.clear(TPB);
    lds_barrier();
    for (uint32_t c = blockIdx.x * TPB + threadIdx.x; c < ck.n; c += gridDim.x * TPB) {
        const uint32_t o = ck.off[c], len = ck.len[c], w = ck.w[c];
        if (len < 2u) continue;
        uint32_t prev = ck.sym[o];
        for (uint32_t j = 1; j < len; ++j) {
            const uint32_t s = ck.sym[o + j];
            const uint32_t key = (prev << 16) | s;
            if (!tab.insert(key, w)) gt_add(gt, key, w, ctl);
            prev = s;
        }
    }
    lds_barrier();
    for (int i = threadIdx.x; i < LT; i += TPB) {
        const uint32_t key = tab.keys[i], c = tab.cnts[i];
        if (key != EMPTY && c) gt_add(gt, key, c, ctl);
    }
}

// One training iteration over the chunks (launch it; a launch after
// training has stopped does nothing). The selection is merge.hpp's: the
// workgroup that draws ticket 0 of the iteration's counter selects and
// publishes, every workgroup reads the publication (and joins a sweep when
// it says so). Then each thread rewrites its chunks that contain the merged
// pair: in place, left to right without overlap, each occurrence of (L, R)
// becoming X. With the chunk's weight, every old pair with a side inside a
// merged occurrence is taken out and every new pair with a side X is put
// in; the other pairs map one to one onto each other (X is a new id), so
// this is the chunk's exact recount. The keys taken out all hold L or R and
// those put in all hold X, so a key only falls or only rises in a launch,
// as the candidate list requires. The changes are summed in LDS and go to
// the table once the workgroup is done.
template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_ck_merge(uint32_t it, Ctl* ctl, Chunks ck, GTable gt, Sweep* sw,
                                                  uint32_t* merges) {
    __shared__ LdsTable<LT> tab;
    __shared__ uint32_t s_tile[2], s_u32;
    __shared__ unsigned long long s_best[TPB / 64];
    if (ctl->done) return;
    const uint32_t p = it & 1u;
    const uint32_t X = BASE + it;
    const bool do_count = X != IDM;  // X = 65535 is the last id: nothing reads counts after it
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* tick = &ctl->tile_ctr[p];
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
    for (uint32_t c = blockIdx.x * TPB + tid; c < ck.n; c += gridDim.x * TPB) {
        const uint32_t len = ck.len[c];
        if (len < 2u) continue;
        uint16_t* s = ck.sym + ck.off[c];
        // a quick look first: most chunks do not hold the pair
        bool has = false;
        for (uint32_t j = 1; j < len && !has; ++j) has = s[j - 1] == L && s[j] == R;
        if (!has) continue;
        const uint32_t wt = ck.w[c], minus = (uint32_t)(-(int)wt);
        auto add = [&](uint32_t a, uint32_t b, uint32_t d) {
            const uint32_t k = (a << 16) | b;
            if (!tab.insert(k, d)) gt_add_sel(gt, k, d, ctl, sw, theta);
        };
        // old pair (j-1, j) is looked at when j is reached; prev is the old
        // symbol at j-1 (the output may have overwritten it), in_site says
        // whether j-1 was inside a merged occurrence
        uint32_t o = 0, prev = 0u;
        bool in_site = false;
        for (uint32_t j = 0; j < len;) {
            const uint32_t a = s[j];
            if (a == L && j + 1u < len && s[j + 1u] == R) {
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
        ck.len[c] = o;
        if (do_count)
            for (uint32_t j = 1; j < o; ++j)
                if (s[j - 1] == X || s[j] == X) add(s[j - 1], s[j], wt);
    }
    finish_counts<TPB, LT>(tab, gt, ctl, sw, theta);
}

}  // namespace bpek
