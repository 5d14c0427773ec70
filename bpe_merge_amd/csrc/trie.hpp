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

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

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
    __shared__ uint16_t s_tok[CAP];                    // token id at each start
    __shared__ uint16_t s_aux[CAP];                    // word list, then staged output
    __shared__ unsigned long long s_root[256];
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_ovf_pos, s_ovf_n;

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
        }
        for (uint32_t i = tid; i < CAP / 32u; i += TPB) s_flag[i] = 0u;
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

        // word starts in [t0, t0 + TILE)
        uint32_t starts = 0;
        {
            const uint32_t p0 = 16u * tid;
            uint32_t pc = byte_class(s_txt[p0 - 1u + sh]);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t c = byte_class(s_txt[p0 + j + sh]);
                const bool st = (p0 + j < nrel) && (t0 + p0 + j == 0u || c != pc);
                starts |= (st ? 1u : 0u) << j;
                pc = c;
            }
        }
        uint32_t nwords;
        uint32_t woff = block_exclusive_sum<TPB>(__popc(starts), s_w, &nwords);
        for (uint32_t m = starts; m; m &= m - 1u) s_aux[woff++] = (uint16_t)(16u * tid + (__ffs(m) - 1));
        __syncthreads();

        // one thread per word: its chain of longest matches to the word's
        // end, from the LDS copy; a word that runs past it (only the tile's
        // last word can) is finished from global memory
        const uint32_t lim = nrel < CAP ? nrel : CAP;
        for (uint32_t w = tid; w < nwords; w += TPB) {
            uint32_t p = s_aux[w];
            uint32_t b = lbyte(p);
            const uint32_t cls = byte_class(b);
            for (;;) {
                uint32_t tok, len;
                bool cut;
                longest_match(da, s_root, root_base, p, lim, b, cls, lbyte, &tok, &len, &cut);
                if (cut) {
                    finish_word_global(text, t0, nrel, p, cls, da, s_root, root_base, CAP, s_flag, s_tok,
                                       &s_ovf_pos, &s_ovf_n);
                    break;
                }
                atomicOr(&s_flag[p >> 5], 1u << (p & 31u));
                s_tok[p] = (uint16_t)tok;
                p += len;
                if (p >= lim) {
                    if (p < nrel && byte_class(text[t0 + p]) == cls)
                        finish_word_global(text, t0, nrel, p, cls, da, s_root, root_base, CAP, s_flag, s_tok,
                                           &s_ovf_pos, &s_ovf_n);
                    break;
                }
                b = lbyte(p);
                if (byte_class(b) != cls) break;
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
// *total = all of them.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_trie_scan(const uint32_t* __restrict__ cnt,
                                                   const uint32_t* __restrict__ ovf_n, uint32_t* __restrict__ pfx,
                                                   uint32_t ntiles, uint32_t* total) {
    __shared__ uint32_t s_w[TPB / 64];
    const uint32_t per = (ntiles + TPB - 1u) / TPB;
    const uint32_t lo = threadIdx.x * per, hi = lo + per < ntiles ? lo + per : ntiles;
    uint32_t sum = 0;
    for (uint32_t t = lo; t < hi; ++t) sum += cnt[t] + ovf_n[t];
    uint32_t all;
    uint32_t run = block_exclusive_sum<TPB>(sum, s_w, &all);
    for (uint32_t t = lo; t < hi; ++t) {
        pfx[t] = run;
        run += cnt[t] + ovf_n[t];
    }
    if (threadIdx.x == 0) *total = all;
}

// ---------------------------------------------------------------- pass 3: copy
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
        for (uint32_t i = threadIdx.x; i < c; i += TPB) out[base + i] = src[i];
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
