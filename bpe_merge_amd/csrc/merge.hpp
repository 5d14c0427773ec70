// Merge + compaction + count update: one pass over the symbols per
// training iteration (gfx950, wave64).
//
// For the merge (L, R) -> X chosen by k_find_max, the pass
//   1. applies the merge left to right without overlap (page "bpe - GPU BPE
//      Tokenizer Pipeline", "Nedir bu ya?"; chains of identical pairs
//      resolved by run-length parity),
//   2. compacts the symbol array with an exclusive prefix scan of the kept
//      flags ("Ne Yapar? 3"), carrying WORD_START_BIT on merged symbols,
//   3. brings the global pair table ("Ne Yapar? 2") to the counts of the new
//      sequence: every old pair that touches a changed position loses one,
//      every new pair that touches a new symbol X gains one. A workgroup
//      sums these changes in an LDS table and adds the sums to the global
//      table at the end.
// The page runs these as separate dispatches with a three-pass scan; here
// the scan is a single-pass decoupled look-back over 8192-symbol tiles, so
// the symbols are read once and written once per iteration.
#pragma once

#include "kernels.hpp"

namespace bpek {

// Selection recurrence. An occurrence at position i (right symbol of the
// pair) is occ_i = (no tag on s_i) and id(s_{i-1}) == L and id(s_i) == R;
// the left-to-right scan merges it iff sel_i = occ_i and not sel_{i-1}.
// A segment's effect on this recurrence and on the number of symbols it
// keeps is a 4-tuple, composed associatively across lanes, waves and tiles:
//   c0      symbols kept when the segment is entered with sel = 0
//   d       extra symbol kept when entered with sel = 1 (0 or 1: only the
//           segment's leading chain of occurrences depends on the entry)
//   o0, o1  sel of the segment's last position for entry sel = 0 / 1
// Packed into 32 bits: c0 in bits 0-23, d bit 24, o0 bit 25, o1 bit 26.

__device__ __forceinline__ uint32_t tup_make(uint32_t c0, uint32_t d, uint32_t o0, uint32_t o1) {
    return c0 | (d << 24) | (o0 << 25) | (o1 << 26);
}
constexpr uint32_t TUP_ID = 1u << 26;  // empty segment: keeps nothing, passes sel through

__device__ __forceinline__ uint32_t tup_c0(uint32_t a) { return a & 0xFFFFFFu; }
__device__ __forceinline__ uint32_t tup_d(uint32_t a) { return (a >> 24) & 1u; }
__device__ __forceinline__ uint32_t tup_o(uint32_t a, uint32_t s) { return (a >> (25 + s)) & 1u; }

// segment a followed by segment b
__device__ __forceinline__ uint32_t tup_then(uint32_t a, uint32_t b) {
    const uint32_t ao0 = tup_o(a, 0), ao1 = tup_o(a, 1), bd = tup_d(b);
    const uint32_t c0 = tup_c0(a) + tup_c0(b) + (ao0 & bd);
    const uint32_t c1 = tup_c0(a) + tup_d(a) + tup_c0(b) + (ao1 & bd);
    return tup_make(c0, c1 - c0, tup_o(b, ao0), tup_o(b, ao1));
}

// The same tuple unpacked, for spans whose kept count can exceed 24 bits.
struct Span {
    uint32_t c0, d, o0, o1;
};

// packed segment a followed by span b
__device__ __forceinline__ Span span_after(uint32_t a, Span b) {
    const uint32_t ao0 = tup_o(a, 0), ao1 = tup_o(a, 1);
    const uint32_t c0 = tup_c0(a) + b.c0 + (ao0 & b.d);
    const uint32_t c1 = tup_c0(a) + tup_d(a) + b.c0 + (ao1 & b.d);
    return Span{c0, c1 - c0, ao0 ? b.o1 : b.o0, ao1 ? b.o1 : b.o0};
}

// Tile status words for the look-back: flag (bits 62-63: 1 aggregate,
// 2 inclusive prefix), epoch = iteration + 1 (bits 32-61), payload (bits
// 0-31: the tile's tuple for an aggregate; kept count before the next tile
// | sel << 31 for a prefix). Words of earlier iterations carry another
// epoch, so nothing is reset between iterations.
constexpr unsigned long long ST_AGG = 1ull << 62;
constexpr unsigned long long ST_PRE = 2ull << 62;

__device__ __forceinline__ unsigned long long st_pack(unsigned long long flag, uint32_t epoch, uint32_t payload) {
    return flag | ((unsigned long long)epoch << 32) | payload;
}
__device__ __forceinline__ void st_store(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long st_load(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool st_valid(unsigned long long s, uint32_t epoch) {
    return (s >> 62) != 0ull && (uint32_t)((s >> 32) & 0x3FFFFFFFull) == epoch;
}

// Decoupled look-back, run by one wave: the exclusive prefix of tile t (kept
// symbols before it, sel of the position before it). Each round reads the
// status words of the 64 * PL tiles below the current window top at once
// (lane l holds tiles top - PL*l - q, q = 0..PL-1), waits until every word
// up to the nearest prefix is published, and folds the aggregates in
// between. The wait is bounded: past SPIN_LIMIT polls it records ERR_SPIN
// and returns a zero prefix, so the kernel always finishes.
template <int PL>
__device__ __forceinline__ void lookback(const unsigned long long* status, uint32_t t, uint32_t epoch,
                                         uint32_t lane, Ctl* ctl, uint32_t& off, uint32_t& sel) {
    Span acc{0u, 0u, 0u, 1u};
    long long top = (long long)t - 1;
    uint32_t spins = 0;
    for (;;) {
        unsigned long long st[PL];
#pragma unroll
        for (int q = 0; q < PL; ++q) {
            const long long idx = top - (long long)(PL * lane + q);
            st[q] = (idx >= 0) ? st_load(status + idx) : st_pack(ST_PRE, epoch, 0u);
        }
        int fq;          // this lane's first q holding a prefix (PL if none)
        uint32_t plane;  // first lane holding a prefix (64 if none)
        for (;;) {
            fq = PL;
            bool all_valid = true, valid_below_fq = true;
#pragma unroll
            for (int q = PL - 1; q >= 0; --q) {
                const bool v = st_valid(st[q], epoch);
                if (v && (st[q] >> 62) == 2ull) fq = q;
                all_valid = all_valid && v;
            }
#pragma unroll
            for (int q = 0; q < PL; ++q)
                if (q < fq) valid_below_fq = valid_below_fq && st_valid(st[q], epoch);
            const unsigned long long pm = __ballot(fq < PL);
            plane = pm ? (uint32_t)(__ffsll((long long)pm) - 1) : 64u;
            const bool ok = (lane < plane) ? all_valid : (lane == plane ? valid_below_fq : true);
            if (__ballot(!ok) == 0ull) break;
            if (++spins > SPIN_LIMIT) {
                if (lane == 0) {
                    atomicOr(&ctl->err, ERR_SPIN);
                    atomicExch(&ctl->done, 1u);
                }
                off = 0;
                sel = 0;
                return;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int q = 0; q < PL; ++q) {
                const long long idx = top - (long long)(PL * lane + q);
                if (idx >= 0 && !st_valid(st[q], epoch)) st[q] = st_load(status + idx);
            }
        }
        // fold this lane's aggregates, lowest tile first
        uint32_t a = TUP_ID;
        uint32_t pay = 0;
#pragma unroll
        for (int q = PL - 1; q >= 0; --q) {
            const bool inc = (lane < plane) || (lane == plane && q < fq);
            if (inc) a = tup_then(a, (uint32_t)(st[q] & 0xFFFFFFFFull));
            if (q == fq) pay = (uint32_t)(st[q] & 0xFFFFFFFFull);
        }
        // fold across lanes: higher lanes hold lower tiles and come first
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t other = __shfl_down(a, o);
            if (lane + o < 64) a = tup_then(other, a);
        }
        a = __shfl(a, 0);
        acc = span_after(a, acc);
        if (plane < 64) {
            const uint32_t p = __shfl(pay, (int)plane);
            const uint32_t base = p & 0x7FFFFFFFu, bsel = p >> 31;
            off = base + acc.c0 + (bsel ? acc.d : 0u);
            sel = bsel ? acc.o1 : acc.o0;
            return;
        }
        top -= 64 * PL;
    }
}

// LDS index skew for staged output (thread-contiguous runs spread over banks)
__device__ __forceinline__ uint32_t skew(uint32_t i) { return i + (i >> 5); }

// Count changes of one thread's positions (bit j: position g0 + j).
// sel holds sel for positions g0 .. g0 + V (bit V: the next thread's first),
// sel_in the sel of position g0 - 1; x the old symbols, left the old symbol
// at g0 - 1. Position i changes if it is dropped (sel_i) or becomes X
// (sel_{i+1}). An old pair (i - 1, i), counted when i carries no word-start
// tag, is gone if i - 1 or i changes. A kept position i with no tag forms
// the new pair (left neighbour, value) and it is new if either side is an X:
// the left neighbour is X when i - 1 was dropped (sel_{i-1}), otherwise the
// unchanged old symbol i - 1; the value is X when sel_{i+1}.
template <int V>
struct Changes {
    uint32_t gone, born;  // position masks
    __device__ __forceinline__ Changes(const uint32_t (&x)[V], uint32_t sel, uint32_t sel_in) {
        constexpr uint32_t VM = (1u << V) - 1u;
        uint32_t untagged = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) untagged |= (uint32_t)!(x[j] & WS) << j;  // positions past n carry WS
        const uint32_t sm1 = ((sel << 1) | sel_in) & VM, s0 = sel & VM, sp1 = (sel >> 1) & VM;
        gone = (sm1 | s0 | sp1) & untagged;
        born = ~s0 & (sm1 | sp1) & untagged & VM;
    }
};

template <int TPB, int LT>
// two workgroups per CU = 4 waves per SIMD: at most 128 VGPRs
__global__ __launch_bounds__(TPB, 4) void k_merge(Ctl* ctl, uint32_t* __restrict__ buf0,
                                               uint32_t* __restrict__ buf1, GTable gt,
                                               unsigned long long* status,
                                               uint32_t* lengths) {
    constexpr int V = 16;  // symbols per thread: four 16-byte loads
    constexpr int TILE = TPB * V;
    constexpr int NW = TPB / 64;
    __shared__ LdsTable<LT> tab;  // count changes of this workgroup
    __shared__ uint32_t s_stage[TILE + TILE / 32];
    __shared__ uint32_t s_wagg[NW];
    __shared__ uint32_t s_tile, s_off, s_sel;

    const uint32_t k = ld_relaxed(&ctl->k);
    const uint32_t it = ld_relaxed(&ctl->m);
    if (it >= k) return;  // no merge pending (uniform)
    const uint32_t L = ctl->L, R = ctl->R, X = ctl->X;
    const uint32_t n = ctl->n[it & 1u];
    const uint32_t* __restrict__ in = (it & 1u) ? buf1 : buf0;
    uint32_t* __restrict__ out = (it & 1u) ? buf0 : buf1;
    const uint32_t ntiles = (n + TILE - 1) / TILE;
    const uint32_t epoch = it + 1;
    // X == 65535 is the last possible id: no later iteration reads counts,
    // and the pair (X, X) would collide with the empty key
    const bool do_count = X != IDM;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;

    tab.clear(TPB);
    for (;;) {
        if (tid == 0) s_tile = atomicAdd(&ctl->tile_ctr, 1u);
        __syncthreads();
        const uint32_t t = s_tile;
        if (t >= ntiles) break;
        const uint32_t g0 = t * TILE + tid * V;

        // ---- 16 symbols, then one neighbour on each side
        uint32_t x[V];
        if (t * TILE + TILE <= n) {
            const uint4* p4 = reinterpret_cast<const uint4*>(in + g0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = p4[q];
                x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) x[j] = (g0 + j < n) ? in[g0 + j] : WS;
        }
        uint32_t a1 = __shfl_up(x[V - 1], 1), b1 = __shfl_down(x[0], 1);
        if (lane == 0) a1 = (g0 >= 1 && g0 - 1 < n) ? in[g0 - 1] : WS;
        if (lane == 63) b1 = (g0 + V < n) ? in[g0 + V] : WS;

        // ---- occurrences (bit j: position g0 + j; bit V: position g0 + V)
        uint32_t occ = 0, valid = 0;
        {
            uint32_t prev = a1;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const bool v = g0 + j < n;
                const bool o = v && (g0 + j >= 1) && !(x[j] & WS) && (prev & IDM) == L && (x[j] & IDM) == R;
                occ |= (uint32_t)o << j;
                valid |= (uint32_t)v << j;
                prev = x[j];
            }
            const bool oV = (g0 + V < n) && !(b1 & WS) && (x[V - 1] & IDM) == L && (b1 & IDM) == R;
            occ |= (uint32_t)oV << V;
        }

        // ---- this thread's tuple, then inclusive scans over the wave and the waves
        uint32_t tup;
        {
            uint32_t s0 = 0, s1 = 1, c0 = 0, c1 = 0;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const uint32_t o = (occ >> j) & 1u, v = (valid >> j) & 1u;
                s0 = o & ~s0 & 1u;
                s1 = o & ~s1 & 1u;
                c0 += v & ~s0 & 1u;
                c1 += v & ~s1 & 1u;
            }
            tup = tup_make(c0, c1 - c0, s0, s1);
        }
        uint32_t incl = tup;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t u = __shfl_up(incl, o);
            if (lane >= (uint32_t)o) incl = tup_then(u, incl);
        }
        uint32_t lane_excl = __shfl_up(incl, 1);
        if (lane == 0) lane_excl = TUP_ID;
        if (lane == 63) s_wagg[w] = incl;
        __syncthreads();
        uint32_t wave_excl = TUP_ID, tile_agg = TUP_ID;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            if (i == (int)w) wave_excl = tile_agg;
            tile_agg = tup_then(tile_agg, s_wagg[i]);
        }

        // ---- decoupled look-back (wave 0)
        if (w == 0) {
            uint32_t off = 0, sel = 0;
            if (t != 0) {
                if (lane == 0) st_store(status + t, st_pack(ST_AGG, epoch, tile_agg));
                lookback<4>(status, t, epoch, lane, ctl, off, sel);
            }
            if (lane == 0) {
                const uint32_t kept = tup_c0(tile_agg) + (sel ? tup_d(tile_agg) : 0u);
                st_store(status + t, st_pack(ST_PRE, epoch, (off + kept) | (tup_o(tile_agg, sel) << 31)));
                s_off = off;
                s_sel = sel;
            }
        }
        __syncthreads();
        const uint32_t tile_off = s_off, tile_sel = s_sel;
        const uint32_t texcl = tup_then(wave_excl, lane_excl);
        const uint32_t my_local = tup_c0(texcl) + (tile_sel ? tup_d(texcl) : 0u);
        const uint32_t sel_in = tup_o(texcl, tile_sel);
        const uint32_t tile_kept = tup_c0(tile_agg) + (tile_sel ? tup_d(tile_agg) : 0u);

        // ---- resolve sel and stage the kept symbols in LDS
        uint32_t selbits = 0;
        {
            uint32_t s = sel_in;
#pragma unroll
            for (int j = 0; j <= V; ++j) {
                s = (occ >> j) & ~s & 1u;
                selbits |= s << j;
            }
        }
        {
            uint32_t o = my_local;
#pragma unroll
            for (int j = 0; j < V; ++j) {
                if (((valid >> j) & 1u) && !((selbits >> j) & 1u)) {
                    s_stage[skew(o)] = ((selbits >> (j + 1)) & 1u) ? (X | (x[j] & WS)) : x[j];
                    ++o;
                }
            }
        }
        __syncthreads();

        // ---- the tile's kept symbols, 16-byte stores where aligned
        {
            const uint32_t head = min(tile_kept, (4u - (tile_off & 3u)) & 3u);
            if (tid < head) out[tile_off + tid] = s_stage[skew(tid)];
            const uint32_t body = (tile_kept - head) >> 2;
            uint4* o4 = reinterpret_cast<uint4*>(out + tile_off + head);
            for (uint32_t i = tid; i < body; i += TPB) {
                const uint32_t b = head + 4 * i;
                o4[i] = make_uint4(s_stage[skew(b)], s_stage[skew(b + 1)], s_stage[skew(b + 2)],
                                   s_stage[skew(b + 3)]);
            }
            const uint32_t rest = head + 4 * body;
            if (tid < tile_kept - rest) out[tile_off + rest + tid] = s_stage[skew(rest + tid)];
        }
        if (t == ntiles - 1 && tid == 0) {
            const uint32_t total = tile_off + tile_kept;
            ctl->n[(it + 1) & 1u] = total;
            lengths[it + 1] = total;
            __threadfence();
            atomicExch(&ctl->m, it + 1);
        }

        // ---- count changes at this thread's merge sites (none for most threads)
        if (do_count && (occ | sel_in)) {
            const Changes<V> ch(x, selbits, sel_in);
            if (ch.gone | ch.born) {
                uint32_t prev = a1;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    if ((ch.gone >> j) & 1u) {
                        const uint32_t key = pair_key(prev, x[j]);
                        if (!tab.insert(key, 0xFFFFFFFFu)) gt_add(gt, key, 0xFFFFFFFFu, ctl);
                    }
                    if ((ch.born >> j) & 1u) {
                        const uint32_t l = (j == 0 ? sel_in : (selbits >> (j - 1)) & 1u) ? X : prev;
                        const uint32_t r = ((selbits >> (j + 1)) & 1u) ? X : x[j];
                        const uint32_t key = pair_key(l, r);
                        if (!tab.insert(key, 1u)) gt_add(gt, key, 1u, ctl);
                    }
                    prev = x[j];
                }
            }
        }
    }
    __syncthreads();
    if (tab.used) flush_table(tab, TPB, gt, ctl);  // uniform: read after the barrier
}

}  // namespace bpek
