// Greedy longest-match inference over a double-array trie of a learned
// vocabulary (page "bpe - GPU BPE Tokenizer Pipeline", "Nedir bu ya?"
// inference paragraph, "Ne Yapar? 4", "Satir Satir Analiz 3)", "Host
// Mimarisi 1-4").
//
// The page walks a BFS-ordered trie with sorted children, searching the
// children of each node (binary search), with the root's 256 children and
// the depth-1 nodes cached in shared memory. Here the trie is a double
// array: the child of slot s by byte c is slot base(s) + c, valid when that
// slot's check field names s. One 8-byte load per byte walked, no search.
// The root's 256 children are cached in LDS, as on the page.
//
// Parallel decomposition: no vocabulary string crosses a byte-class change
// (a merge joins two symbols of one word, and a word is a run of one class),
// so a longest match never crosses one either, and every word (maximal
// same-class run) can be matched on its own. A workgroup takes a tile of
// TILE bytes and owns the words that start in it; one thread walks one
// word's chain of longest matches to the word's end, which may lie past the
// tile. Three passes, as the page's three dispatches (chunked walk, prefix
// sum, compaction): the walk writes each tile's tokens compacted into a
// per-tile slice with a count, one workgroup scans the counts, and a copy
// pass moves every slice to its place. The walk time of a tile varies with
// its words, so no tile ever waits for another.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace bpek {

// ---------------------------------------------------------------- node entries
// slot entry: bits 0-20 check (parent slot + 1; 0 = free slot), bits 21-41
// base (0 = no children), bits 42-58 token id + 1 (0 = no token ends here).
constexpr uint32_t TR_FIELD = 21;
constexpr unsigned long long TR_MASK = (1ull << TR_FIELD) - 1ull;
constexpr uint32_t TR_MAX_SLOTS = (1u << TR_FIELD) - 1u;  // so that check = slot + 1 fits

__host__ __device__ __forceinline__ uint32_t tr_check(unsigned long long e) { return (uint32_t)(e & TR_MASK); }
__host__ __device__ __forceinline__ uint32_t tr_base(unsigned long long e) {
    return (uint32_t)((e >> TR_FIELD) & TR_MASK);
}
__host__ __device__ __forceinline__ uint32_t tr_tok1(unsigned long long e) {
    return (uint32_t)((e >> (2 * TR_FIELD)) & 0x1FFFFull);
}
__host__ __device__ __forceinline__ unsigned long long tr_pack(uint32_t check, uint32_t base, uint32_t tok1) {
    return (unsigned long long)check | ((unsigned long long)base << TR_FIELD) |
           ((unsigned long long)tok1 << (2 * TR_FIELD));
}

// ---------------------------------------------------------------- helpers

// Exclusive prefix sum over the workgroup (TPB threads); the total goes to
// *total. Uses s_w (TPB / 64 words); ends with a barrier.
template <int TPB>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* s_w, uint32_t* total) {
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= (uint32_t)o) x += y;
    }
    if (lane == 63u) s_w[w] = x;
    lds_barrier();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < TPB / 64; ++i) {
        const uint32_t t = s_w[i];
        before += (i < (int)w) ? t : 0u;
        all += t;
    }
    *total = all;
    lds_barrier();
    return before + x - v;
}

// One longest match at relative position p (byte b0, word class cls),
// reading text bytes with byte_at(q) for q < lim: the token id and its
// length in bytes. *cut is set when the walk stopped only because it
// reached lim with more of the word and of the trie left (the caller then
// matches again with a reader that goes further).
template <typename ByteAt>
__device__ __forceinline__ void longest_match(const unsigned long long* __restrict__ da,
                                              const unsigned long long* s_root, uint32_t root_base, uint32_t p,
                                              uint32_t lim, uint32_t b0, uint32_t cls, ByteAt byte_at,
                                              uint32_t* tok, uint32_t* len, bool* cut) {
    unsigned long long e = s_root[b0];
    uint32_t slot = root_base + b0;
    uint32_t best = tr_tok1(e) - 1u, blen = 1u;  // every byte is a token
    bool c_ut = false;
    for (uint32_t j = 1;; ++j) {
        const uint32_t base = tr_base(e);
        if (base == 0u) break;
        if (p + j >= lim) {
            c_ut = true;
            break;
        }
        const uint32_t c = byte_at(p + j);
        if (byte_class(c) != cls) break;  // the word ends; no string crosses it
        const unsigned long long e2 = da[base + c];
        if (tr_check(e2) != slot + 1u) break;
        slot = base + c;
        e = e2;
        const uint32_t t1 = tr_tok1(e);
        if (t1) {
            best = t1 - 1u;
            blen = j + 1u;
        }
    }
    *tok = best;
    *len = blen;
    *cut = c_ut;
}

// The rest of a word from relative position p (a token start, p < nrel)
// with bytes read from global memory: a match that ran past the LDS copy,
// and every token past it. Tokens at positions below cap are recorded in
// LDS (s_flag, s_tok); the others are counted into *ovf_n, the first of
// them noted in *ovf_pos. Returns nothing else; runs for at most one word
// per tile (the last one), so it is kept out of line.
__device__ __attribute__((noinline)) void finish_word_global(
    const uint8_t* __restrict__ text, uint32_t t0, uint32_t nrel, uint32_t p, uint32_t cls,
    const unsigned long long* __restrict__ da, const unsigned long long* s_root, uint32_t root_base, uint32_t cap,
    uint32_t* s_flag, uint16_t* s_tok, uint32_t* ovf_pos, uint32_t* ovf_n) {
    auto gbyte = [&](uint32_t q) -> uint32_t { return text[t0 + q]; };
    for (;;) {
        uint32_t tok, len;
        bool cut;
        longest_match(da, s_root, root_base, p, nrel, gbyte(p), cls, gbyte, &tok, &len, &cut);
        if (p < cap) {
            atomicOr(&s_flag[p >> 5], 1u << (p & 31u));
            s_tok[p] = (uint16_t)tok;
        } else {
            if (*ovf_pos == 0xFFFFFFFFu) *ovf_pos = p;
            *ovf_n += 1u;
        }
        p += len;
        if (p >= nrel || byte_class(gbyte(p)) != cls) break;
    }
}

// ---------------------------------------------------------------- pass 1: walk
constexpr uint32_t TRIE_HALO_PER_THREAD = 4;  // LDS bytes past the tile, per thread
constexpr uint32_t NO_OVF = 0xFFFFFFFFu;

// Tiles of TILE = 16 TPB bytes, t = blockIdx.x, blockIdx.x + gridDim.x, ...
// Outputs for tile t: tok16[t * CAP + i], i < cnt[t], the ids of the tokens
// of the words starting in the tile, in order, as far as CAP bytes from the
// tile start; for a last word running further, ovf_pos[t] is the relative
// position of its first token at or past CAP and ovf_n[t] the number of its
// tokens from there (NO_OVF and 0 otherwise). text: n bytes, any alignment;
// da: the double array (every base + 255 inside it).
template <int TPB>
__global__ __launch_bounds__(TPB) void k_trie_walk(const uint8_t* __restrict__ text, uint32_t n,
                                                   const unsigned long long* __restrict__ da, uint32_t root_base,
                                                   uint16_t* __restrict__ tok16, uint32_t* __restrict__ cnt,
                                                   uint32_t* __restrict__ ovf_pos, uint32_t* __restrict__ ovf_n,
                                                   uint32_t ntiles) {
    constexpr uint32_t TILE = TPB * 16u;          // words starting here are this tile's
    constexpr uint32_t HALO = TPB * TRIE_HALO_PER_THREAD;
    constexpr uint32_t CAP = TILE + HALO;         // token starts recorded in LDS
    constexpr uint32_t PER = CAP / TPB;           // positions per thread in the compaction
    constexpr uint32_t NCH = (CAP + 32u) / 16u;   // 16-byte chunks loaded per tile
    static_assert(CAP % TPB == 0 && PER <= 32, "compaction covers CAP positions, at most 32 per thread");

    __shared__ __align__(16) uint8_t s_txt[NCH * 16u];  // s_txt[p + 16 + mis] = text[t0 + p]
    __shared__ uint32_t s_flag[CAP / 32u];             // token starts
    __shared__ uint32_t s_sb[TILE / 32u];              // word starts in the tile
    __shared__ uint16_t s_tok[CAP];                    // token id at each start
    __shared__ uint16_t s_aux[CAP];                    // word list, then staged output
    __shared__ unsigned long long s_root[256];
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_ovf_pos, s_ovf_n, s_after;

    const uint32_t tid = threadIdx.x;
    // the text through a 16-byte aligned base; the range is rounded up to
    // whole 16-byte blocks (bytes past n in the last block are loaded but
    // never used, and lie in the same block, so on the same page)
    const uint32_t mis = (uint32_t)((uintptr_t)text & 15u);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(text - mis), 0, (int)((n + mis + 15u) & ~15u), 0x00020000);

    for (uint32_t i = tid; i < 256u; i += TPB) s_root[i] = da[root_base + i];

    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        if (tid == 0) {
            s_ovf_pos = NO_OVF;
            s_ovf_n = 0u;
            s_after = CAP;
        }
        for (uint32_t i = tid; i < CAP / 32u; i += TPB) s_flag[i] = 0u;
        for (uint32_t i = tid; i < TILE / 32u; i += TPB) s_sb[i] = 0u;
        const uint32_t t0 = t * TILE;
        const uint32_t nrel = n - t0;

        // text [t0 - 16, t0 + CAP + 16) into LDS, 16-byte aligned chunks
        for (uint32_t k = tid; k < NCH; k += TPB) {
            typedef uint32_t v4 __attribute__((ext_vector_type(4)));
            const v4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, t0 - 16u + 16u * k, 0, 0);
            *reinterpret_cast<v4*>(s_txt + 16u * k) = v;
        }
        __syncthreads();  // also orders the previous tile's LDS reads before these writes
        const uint32_t sh = 16u + mis;
        auto lbyte = [&](uint32_t q) -> uint32_t { return s_txt[q + sh]; };  // q < CAP

        // Word starts in [t0, t0 + TILE), 16 positions per thread: into the
        // LDS bitmap s_sb. A one-byte word is its own token (every byte is
        // one) and is recorded here; longer words go to the list s_aux.
        // The first word start in [t0 + TILE, t0 + CAP) ends the tile's last
        // word (if there is none, that word may run past the copy).
        uint32_t multi;
        {
            const uint32_t p0 = 16u * tid;
            uint32_t pc = byte_class(s_txt[p0 - 1u + sh]);
            uint32_t starts = 0, bnd = 0;  // bnd bit k: a word boundary at p0 + k (k = 1..16)
#pragma unroll
            for (int k = 0; k <= 16; ++k) {
                const uint32_t c = byte_class(s_txt[p0 + k + sh]);
                const bool inside = p0 + k < nrel;
                const bool change = c != pc || t0 + p0 + k == 0u;
                if (k < 16) starts |= ((inside && change) ? 1u : 0u) << k;
                if (k >= 1) bnd |= ((!inside || change) ? 1u : 0u) << k;
                pc = c;
            }
            const uint32_t single = starts & (bnd >> 1);
            multi = starts & ~single;
            const uint32_t sb = p0 & 31u;  // the 16 positions share one 32-bit word
            if (starts) atomicOr(&s_sb[p0 >> 5], starts << sb);
            if (single) {
                atomicOr(&s_flag[p0 >> 5], single << sb);
                for (uint32_t m = single; m; m &= m - 1u) {
                    const uint32_t k = __ffs(m) - 1;
                    s_tok[p0 + k] = (uint16_t)lbyte(p0 + k);
                }
            }
        }
        uint32_t after = CAP;
        {
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
            if ((tid & 63u) == 0u) atomicMin(&s_after, after);
        }
        uint32_t nwords;
        uint32_t woff = block_exclusive_sum<TPB>(__popc(multi), s_w, &nwords);
        for (uint32_t m = multi; m; m &= m - 1u) s_aux[woff++] = (uint16_t)(16u * tid + (__ffs(m) - 1));
        __syncthreads();

        // The walk over the words of two bytes or more. Each wave takes a
        // contiguous share of them; a lane without a word takes the wave's
        // next one (ballot + mbcnt), so lanes stay busy until the share is
        // done. A lane follows its word's chain of longest matches, one
        // trie step per round: the byte from the LDS copy, one 8-byte load
        // of the slot it leads to. A word ends at the next start in s_sb;
        // the tile's last word ends at the first start past the tile, or is
        // open (it may run past the copy, and is then finished from global
        // memory after the loop).
        {
            const uint32_t lim = nrel < CAP ? nrel : CAP;
            const uint32_t last_end = s_after < lim ? s_after : lim;
            const bool last_open = s_after >= CAP && lim < nrel;
            constexpr uint32_t NWAVE = TPB / 64u;
            const uint32_t wave = tid >> 6;
            const uint32_t share = (nwords + NWAVE - 1u) / NWAVE;
            const uint32_t w_hi = min(nwords, (wave + 1u) * share);
            uint32_t next = min(nwords, wave * share);  // the wave's next word (uniform)
            uint32_t p = 0, j = 0, slot = 0, best = 0, blen = 0, wend = 0, gp = NO_OVF;
            unsigned long long e = 0ull;
            bool act = false;
            auto begin_match = [&](uint32_t q) {
                const uint32_t b = lbyte(q);
                e = s_root[b];
                slot = root_base + b;
                best = tr_tok1(e) - 1u;  // every byte is a token
                blen = 1u;
                j = 1u;
                p = q;
            };
            for (;;) {
                const unsigned long long need = __ballot(!act);
                if (need) {
                    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(need >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)need, 0u));
                    if (!act && next + below < w_hi) {
                        const uint32_t q = s_aux[next + below];
                        // the word's end: the next start after q
                        wend = last_end;
                        for (uint32_t x = q + 1u; x < TILE;) {
                            const uint32_t m = s_sb[x >> 5] & (0xFFFFFFFFu << (x & 31u));
                            if (m) {
                                wend = (x & ~31u) + (__ffs(m) - 1);
                                break;
                            }
                            x = (x & ~31u) + 32u;
                        }
                        begin_match(q);
                        act = true;
                    }
                    next += (uint32_t)__popcll(need);
                }
                if (__ballot(act) == 0ull) break;
                if (act) {
                    const uint32_t base = tr_base(e);
                    const uint32_t q = p + j;
                    const bool go = base != 0u && q < wend;
                    const uint32_t addr = go ? base + lbyte(q) : 0u;
                    const unsigned long long e2 = da[addr];
                    // a step down the trie, as selects (fewer register copies
                    // than branches: the walk is bound by vector issue)
                    const bool adv = go && tr_check(e2) == slot + 1u;
                    const uint32_t t1 = adv ? tr_tok1(e2) : 0u;
                    best = t1 ? t1 - 1u : best;
                    blen = t1 ? j + 1u : blen;
                    slot = adv ? addr : slot;
                    e = adv ? e2 : e;
                    j += adv ? 1u : 0u;
                    if (!adv) {
                        const bool open = last_open && wend == last_end;
                        if (open && base != 0u && q >= lim) {
                            gp = p;  // the match may go on past the LDS copy
                            act = false;
                        } else {
                            atomicOr(&s_flag[p >> 5], 1u << (p & 31u));
                            s_tok[p] = (uint16_t)best;
                            const uint32_t np = p + blen;
                            if (np < wend) {
                                begin_match(np);
                            } else {
                                if (open && np < nrel && byte_class(text[t0 + np]) == byte_class(lbyte(p))) gp = np;
                                act = false;
                            }
                        }
                    }
                }
            }
            if (gp != NO_OVF) {
                const uint32_t cls = byte_class(gp < lim ? lbyte(gp) : (uint32_t)text[t0 + gp]);
                finish_word_global(text, t0, nrel, gp, cls, da, s_root, root_base, CAP, s_flag, s_tok, &s_ovf_pos,
                                   &s_ovf_n);
            }
        }
        __syncthreads();

        // compaction of the recorded starts: PER positions per thread
        uint32_t bits;
        {
            const uint32_t lo = PER * tid, wi = lo >> 5, sb = lo & 31u;
            const uint32_t w0 = s_flag[wi];
            const uint32_t w1 = (wi + 1u < CAP / 32u) ? s_flag[wi + 1u] : 0u;
            const unsigned long long both = ((unsigned long long)w1 << 32) | w0;
            bits = (uint32_t)(both >> sb) & (uint32_t)((1ull << PER) - 1ull);
        }
        uint32_t nlds;
        uint32_t off = block_exclusive_sum<TPB>(__popc(bits), s_w, &nlds);
        for (uint32_t m = bits; m; m &= m - 1u) s_aux[off++] = s_tok[PER * tid + (__ffs(m) - 1)];
        __syncthreads();
        uint16_t* dst = tok16 + (size_t)t * CAP;
        for (uint32_t i = tid; i < nlds; i += TPB) dst[i] = s_aux[i];
        if (tid == 0) {
            cnt[t] = nlds;
            ovf_pos[t] = s_ovf_pos;
            ovf_n[t] = s_ovf_n;
        }
    }
}

// ---------------------------------------------------------------- pass 2: scan
// One workgroup: pfx[t] = tokens of all tiles below t (cnt + ovf_n), and
// *total = all of them. The arrays hold npad entries (a multiple of 4 TPB;
// entries past ntiles are ignored). Wave w owns a contiguous segment; its
// lanes read consecutive groups of four entries (16-byte loads, coalesced
// across the wave): a first pass sums the segment, a second writes the
// prefixes, each group's offset from a wave scan of the group sums.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_trie_scan(const uint32_t* __restrict__ cnt,
                                                   const uint32_t* __restrict__ ovf_n, uint32_t* __restrict__ pfx,
                                                   uint32_t ntiles, uint32_t npad, uint32_t* total) {
    constexpr uint32_t NWAVE = TPB / 64u;
    __shared__ uint32_t s_w[NWAVE];
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint32_t seg = npad / NWAVE;  // a multiple of 256
    const uint32_t lo = w * seg;
    auto group = [&](uint32_t i, uint32_t (&g)[4]) {
        const uint4 c = *reinterpret_cast<const uint4*>(cnt + i);
        const uint4 o = *reinterpret_cast<const uint4*>(ovf_n + i);
        g[0] = i < ntiles ? c.x + o.x : 0u;
        g[1] = i + 1u < ntiles ? c.y + o.y : 0u;
        g[2] = i + 2u < ntiles ? c.z + o.z : 0u;
        g[3] = i + 3u < ntiles ? c.w + o.w : 0u;
    };
    uint32_t sum = 0;
#pragma unroll 4
    for (uint32_t v = 0; v < seg; v += 256u) {
        uint32_t g[4];
        group(lo + v + 4u * lane, g);
        sum += g[0] + g[1] + g[2] + g[3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0u) s_w[w] = sum;
    __syncthreads();
    uint32_t run = 0, all = 0;
#pragma unroll
    for (uint32_t k = 0; k < NWAVE; ++k) {
        const uint32_t x = s_w[k];
        run += k < w ? x : 0u;
        all += x;
    }
    for (uint32_t v = 0; v < seg; v += 256u) {
        const uint32_t i = lo + v + 4u * lane;
        uint32_t g[4];
        group(i, g);
        const uint32_t gs = g[0] + g[1] + g[2] + g[3];
        uint32_t incl = gs;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o);
            if (lane >= (uint32_t)o) incl += y;
        }
        uint4 r;
        r.x = run + incl - gs;
        r.y = r.x + g[0];
        r.z = r.y + g[1];
        r.w = r.z + g[2];
        *reinterpret_cast<uint4*>(pfx + i) = r;
        run += __shfl(incl, 63);
    }
    if (threadIdx.x == 0) *total = all;
}

// ---------------------------------------------------------------- pass 3: copy
// Tokens tok(0) .. tok(c - 1) of one tile to out[base ..]: a scalar head up
// to a 16-byte boundary of out, then four tokens per thread and 16-byte
// store (two groups in flight), then a scalar tail.
template <int TPB, typename Tok>
__device__ __forceinline__ void copy_tokens(uint32_t* __restrict__ out, uint32_t base, uint32_t c, Tok tok) {
    const uint32_t mis = (uint32_t)(((uintptr_t)(out + base) >> 2) & 3u);  // out is 4-byte aligned
    const uint32_t head = min(c, (4u - mis) & 3u);
    if (threadIdx.x < head) out[base + threadIdx.x] = tok(threadIdx.x);
    const uint32_t ng = (c - head) / 4u;
    uint4* o4 = reinterpret_cast<uint4*>(out + base + head);
    uint32_t g = threadIdx.x;
    for (; g + TPB < ng; g += 2u * TPB) {
        const uint32_t i = head + 4u * g, k = i + 4u * TPB;
        const uint4 a = make_uint4(tok(i), tok(i + 1u), tok(i + 2u), tok(i + 3u));
        const uint4 b = make_uint4(tok(k), tok(k + 1u), tok(k + 2u), tok(k + 3u));
        o4[g] = a;
        o4[g + TPB] = b;
    }
    for (; g < ng; g += TPB) {
        const uint32_t i = head + 4u * g;
        o4[g] = make_uint4(tok(i), tok(i + 1u), tok(i + 2u), tok(i + 3u));
    }
    const uint32_t done = head + 4u * ng;
    if (threadIdx.x < c - done) out[base + done + threadIdx.x] = tok(done + threadIdx.x);
}

// Tile slices to their places in out (16-bit ids widened to 32 bits); the
// tokens of a tile's last word past its recorded range are walked again,
// from global memory, by one thread.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_trie_copy(const uint8_t* __restrict__ text, uint32_t n,
                                                   const unsigned long long* __restrict__ da, uint32_t root_base,
                                                   const uint16_t* __restrict__ tok16,
                                                   const uint32_t* __restrict__ cnt,
                                                   const uint32_t* __restrict__ ovf_pos,
                                                   const uint32_t* __restrict__ ovf_n,
                                                   const uint32_t* __restrict__ pfx, uint32_t* __restrict__ out,
                                                   uint32_t ntiles, uint32_t tile, uint32_t cap) {
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint32_t c = cnt[t], base = pfx[t];
        const uint16_t* src = tok16 + (size_t)t * cap;
        copy_tokens<TPB>(out, base, c, [&](uint32_t i) -> uint32_t { return src[i]; });
        const uint32_t no = ovf_n[t];
        if (threadIdx.x == 0 && no) {
            const uint32_t t0 = t * tile, nrel = n - t0;
            uint32_t p = ovf_pos[t];
            const uint32_t cls = byte_class(text[t0 + p]);
            auto gbyte = [&](uint32_t q) -> uint32_t { return text[t0 + q]; };
            uint32_t o = base + c;
            for (uint32_t k = 0; k < no && p < nrel; ++k) {
                uint32_t tok, len;
                bool cut;
                longest_match(da, da + root_base, root_base, p, nrel, gbyte(p), cls, gbyte, &tok, &len, &cut);
                out[o++] = tok;
                p += len;
            }
        }
    }
}

}  // namespace bpek
