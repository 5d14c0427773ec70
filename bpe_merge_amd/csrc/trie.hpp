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
// tile. Token starts are marked in LDS, compacted, and written at an offset
// found by a decoupled look-back over tile token counts.
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

// Control words of one trie: a monotonic tile counter (each launch starts
// at the count the host expects, so nothing is reset between launches), the
// total token count, and the epoch of the last launch that hit the wait
// bound (0 if none).
struct alignas(64) TrieCtl {
    uint32_t tile_ctr;
    uint32_t total;
    uint32_t err_epoch;
};

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

// Look-back over tile token counts (one wave): the number of tokens in
// tiles below t. Status words as in the merge pass (flag, epoch, payload =
// the tile's count for an aggregate, the inclusive count for a prefix).
// The wait is bounded by wall-clock time: past `limit` ticks it reports
// failure and returns 0, so the kernel always finishes.
__device__ __forceinline__ uint32_t count_lookback(const unsigned long long* status, uint32_t t, uint32_t epoch,
                                                   uint32_t lane, unsigned long long limit, bool* failed) {
    constexpr unsigned long long AGG = 1ull << 62, PRE = 2ull << 62;
    uint32_t acc = 0;
    long long top = (long long)t - 1;
    const unsigned long long t_start = wall_clock64();
    for (;;) {
        const long long idx = top - (long long)lane;
        unsigned long long s = (idx >= 0) ? __hip_atomic_load(status + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                          : (PRE | ((unsigned long long)epoch << 32));
        for (;;) {
            const bool v = (s >> 62) != 0ull && (uint32_t)((s >> 32) & 0x3FFFFFFFull) == epoch;
            const unsigned long long pm = __ballot(v && (s >> 62) == 2ull);
            const uint32_t plane = pm ? (uint32_t)(__ffsll((long long)pm) - 1) : 64u;
            const bool ok = (lane <= plane) ? v : true;
            if (__ballot(!ok) == 0ull) {
                acc += wave_sum_u32((lane <= plane) ? (uint32_t)s : 0u);
                if (plane < 64u) return acc;
                break;
            }
            if (wall_clock64() - t_start > limit) {
                *failed = true;
                return 0u;
            }
            __builtin_amdgcn_s_sleep(2);
            if (idx >= 0 && !v) s = __hip_atomic_load(status + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        top -= 64;
    }
    (void)AGG;
}

// One longest match from relative position p (byte b0 = byte(p), class
// cls): the token id and its length in bytes. byte(q) fetches text bytes;
// nrel is the text length relative to the tile start.
template <typename ByteAt>
__device__ __forceinline__ void longest_match(const unsigned long long* __restrict__ da,
                                              const unsigned long long* s_root, uint32_t root_base, uint32_t p,
                                              uint32_t nrel, uint32_t b0, uint32_t cls, ByteAt byte_at,
                                              uint32_t* tok, uint32_t* len) {
    unsigned long long e = s_root[b0];
    uint32_t slot = root_base + b0;
    uint32_t best = tr_tok1(e) - 1u, blen = 1u;  // every byte is a token
    for (uint32_t j = 1;; ++j) {
        const uint32_t base = tr_base(e);
        if (base == 0u || p + j >= nrel) break;
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
}

// ---------------------------------------------------------------- the kernel
// text: n bytes (any alignment); da: the double array (every base + 255 is
// inside it); out: room for n tokens. Tiles are handed out in order by the
// monotonic counter ctl->tile_ctr (minus tile_base), so every tile a
// workgroup waits on is held by a running workgroup.
template <int TPB>
__global__ __launch_bounds__(TPB) void k_trie_encode(const uint8_t* __restrict__ text, uint32_t n,
                                                     const unsigned long long* __restrict__ da, uint32_t root_base,
                                                     uint32_t* __restrict__ out, TrieCtl* ctl,
                                                     unsigned long long* status, uint32_t epoch, uint32_t ntiles,
                                                     uint32_t tile_base, unsigned long long wait_limit) {
    constexpr uint32_t TILE = TPB * 16u;          // words starting here are this tile's
    constexpr uint32_t HALO = 2048u;              // bytes past the tile kept in LDS
    constexpr uint32_t CAP = TILE + HALO;         // token starts recorded in LDS
    constexpr uint32_t PER = CAP / TPB;           // positions per thread in the compaction
    constexpr uint32_t NCH = (CAP + 32u) / 16u;   // 16-byte chunks loaded per tile
    static_assert(CAP % TPB == 0 && PER <= 32, "compaction covers CAP positions, at most 32 per thread");
    constexpr unsigned long long AGG = 1ull << 62, PRE = 2ull << 62;

    __shared__ __align__(16) uint8_t s_txt[NCH * 16u];  // s_txt[p + 16 + mis] = text[t0 + p]
    __shared__ uint32_t s_flag[CAP / 32u];             // token starts
    __shared__ uint16_t s_tok[CAP];                    // token id at each start
    __shared__ uint16_t s_aux[CAP];                    // word list, then staged output
    __shared__ unsigned long long s_root[256];
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_tile, s_prefix, s_ovf_pos, s_ovf_n, s_fail;

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    // the text through a 16-byte aligned base; the range is rounded up to
    // whole 16-byte blocks (bytes past n in the last block are loaded but
    // never used, and lie in the same block, so on the same page)
    const uint32_t mis = (uint32_t)((uintptr_t)text & 15u);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(text - mis), 0, (int)((n + mis + 15u) & ~15u), 0x00020000);

    for (uint32_t i = tid; i < 256u; i += TPB) s_root[i] = da[root_base + i];

    for (;;) {
        if (tid == 0) {
            s_tile = atomicAdd(&ctl->tile_ctr, 1u) - tile_base;
            s_ovf_pos = 0xFFFFFFFFu;
            s_ovf_n = 0u;
            s_fail = 0u;
        }
        for (uint32_t i = tid; i < CAP / 32u; i += TPB) s_flag[i] = 0u;
        __syncthreads();  // also orders the previous tile's LDS reads before the new writes
        const uint32_t t = s_tile;
        if (t >= ntiles) break;
        const uint32_t t0 = t * TILE;
        const uint32_t nrel = n - t0;

        // text [t0 - 16, t0 + CAP + 16) into LDS, 16-byte aligned chunks
        for (uint32_t k = tid; k < NCH; k += TPB) {
            typedef uint32_t v4 __attribute__((ext_vector_type(4)));
            const v4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, t0 - 16u + 16u * k, 0, 0);
            *reinterpret_cast<v4*>(s_txt + 16u * k) = v;
        }
        __syncthreads();
        const uint32_t sh = 16u + mis;
        auto byte_at = [&](uint32_t q) -> uint32_t {
            return (q < CAP) ? (uint32_t)s_txt[q + sh] : (uint32_t)text[t0 + q];
        };

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

        // one thread per word: its chain of longest matches to the word's end
        for (uint32_t w = tid; w < nwords; w += TPB) {
            uint32_t p = s_aux[w];
            uint32_t b = s_txt[p + sh];
            const uint32_t cls = byte_class(b);
            for (;;) {
                uint32_t tok, len;
                longest_match(da, s_root, root_base, p, nrel, b, cls, byte_at, &tok, &len);
                if (p < CAP) {
                    atomicOr(&s_flag[p >> 5], 1u << (p & 31u));
                    s_tok[p] = (uint16_t)tok;
                } else {
                    // only the tile's last word runs this far; its later
                    // tokens are counted now and written after the look-back
                    if (s_ovf_pos == 0xFFFFFFFFu) s_ovf_pos = p;
                    s_ovf_n += 1u;
                }
                p += len;
                if (p >= nrel) break;
                b = byte_at(p);
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
        const uint32_t novf = s_ovf_n;
        const uint32_t count = nlds + novf;

        if (tid < 64u) {
            uint32_t prefix = 0;
            if (t == 0u) {
                if (lane == 0u)
                    __hip_atomic_store(status, PRE | ((unsigned long long)epoch << 32) | count, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            } else {
                if (lane == 0u)
                    __hip_atomic_store(status + t, AGG | ((unsigned long long)epoch << 32) | count, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                bool failed = false;
                prefix = count_lookback(status, t, epoch, lane, wait_limit, &failed);
                if (lane == 0u) {
                    __hip_atomic_store(status + t, PRE | ((unsigned long long)epoch << 32) | (prefix + count),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (failed) {
                        s_fail = 1u;
                        atomicExch(&ctl->err_epoch, epoch);
                    }
                }
            }
            if (lane == 0u) s_prefix = prefix;
        }
        // stage this thread's tokens in order (s_aux is free again)
        for (uint32_t m = bits; m; m &= m - 1u) s_aux[off++] = s_tok[PER * tid + (__ffs(m) - 1)];
        __syncthreads();

        const uint32_t prefix = s_prefix;
        if (s_fail == 0u) {
            for (uint32_t i = tid; i < nlds; i += TPB) out[prefix + i] = s_aux[i];
            if (tid == 0u && novf) {
                // the rest of the last word, walked again from its first
                // token past the recorded range
                uint32_t p = s_ovf_pos;
                uint32_t b = text[t0 + p];
                const uint32_t cls = byte_class(b);
                uint32_t o = prefix + nlds;
                for (uint32_t k = 0; k < novf; ++k) {
                    uint32_t tok, len;
                    longest_match(da, s_root, root_base, p, nrel, b, cls, byte_at, &tok, &len);
                    out[o++] = tok;
                    p += len;
                    if (p >= nrel) break;
                    b = byte_at(p);
                }
            }
        }
        if (tid == 0u && t == ntiles - 1u) ctl->total = prefix + count;
    }
}

}  // namespace bpek
