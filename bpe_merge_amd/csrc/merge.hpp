// Merge + compaction + count update: one pass over the symbols per
// training iteration (gfx950, wave64).
//
// For the merge (L, R) -> X (the table's maximum, selected at the start of
// the pass from a candidate list or by a sweep of the table), the pass
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
// the scan is a single-pass decoupled look-back over tiles of 32768 symbols
// (1024-thread workgroups, two halves of 16 symbols per thread), 16384
// (512 threads, two halves) or 8192 (512 threads, one half: the smallest
// corpora), so the symbols are read once and written once per iteration.
//
// The symbol array holds 16-bit ids and no word-start bit. The page tags
// the first symbol of each word ("Ne Yapar? 1"); here that tag is implied:
// a word is a maximal run of one byte class, every token lies inside one
// word, so a token has its first byte's class, and two neighbouring words
// always differ in class. A pair of neighbours therefore straddles a word
// start exactly when their classes differ, and the merge (L, R), a counted
// pair, has both ids in one class: any neighbouring L, R lie in one word.
// The class of every id is kept in a byte table (the class of X is that of
// L), and per class a bit mask of the ids in it; a pass copies the mask of
// its merge's class into LDS for the few pairs whose counts change.
#pragma once

#include "kernels.hpp"

namespace bpek {

// Selection recurrence. An occurrence at position i (right symbol of the
// pair) is occ_i = (s_{i-1} == L and s_i == R; no word start lies between
// them, as L and R share a class); the left-to-right scan merges it iff
// sel_i = occ_i and not sel_{i-1}.
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

// Cross-lane moves by DPP (data-parallel primitives of the GCN/CDNA vector
// ALU): v from another lane per CTRL, ident where that lane is outside the
// row or wave, or the row is masked off (row_mask RM). No LDS round trip.
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_WAVE_SHL1 = 0x130, DPP_WAVE_SHR1 = 0x138, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t ident, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, RM, 0xF, false);
}
// Inclusive scan over the 64 lanes of a wave with an associative op(a, b)
// (a then b; ident its identity): shifts of 1, 2, 4, 8 within rows of 16,
// then row 0's last lane into row 1 and row 2's into row 3, then lane 31
// into rows 2 and 3.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t ident, Op op) {
    v = op(dpp<DPP_ROW_SHR1>(ident, v), v);
    v = op(dpp<DPP_ROW_SHR2>(ident, v), v);
    v = op(dpp<DPP_ROW_SHR4>(ident, v), v);
    v = op(dpp<DPP_ROW_SHR8>(ident, v), v);
    v = op(dpp<DPP_ROW_BCAST15, 0xA>(ident, v), v);
    v = op(dpp<DPP_ROW_BCAST31, 0xC>(ident, v), v);
    return v;
}

// Decoupled look-back, run by one wave: the exclusive prefix of tile t (kept
// symbols before it, sel of the position before it). Each round reads the
// status words of the 64 * PL tiles below the current window top at once
// (lane l holds tiles top - PL*l - q, q = 0..PL-1), waits until every word
// up to the nearest prefix is published, and folds the aggregates in
// between. The wait is bounded: past SPIN_LIMIT polls it records ERR_SPIN
// and returns a zero prefix, so the kernel always finishes.
// The status words of one window (tiles top - PL*lane - q); below tile 0 a
// zero prefix. Every lane issues its PL loads (tile 0's word stands in for
// indexes below 0), so that the number of loads is fixed.
template <int PL>
__device__ __forceinline__ void lookback_window(const unsigned long long* status, int top, uint32_t epoch,
                                                uint32_t lane, unsigned long long (&st)[PL]) {
#pragma unroll
    for (int q = 0; q < PL; ++q) {
        const int idx = top - (int)(PL * lane + q);
        const unsigned long long v = st_load(status + (idx >= 0 ? idx : 0));
        st[q] = (idx >= 0) ? v : st_pack(ST_PRE, epoch, 0u);
    }
}

// first: the first window (tiles below t), already loaded by the caller
// (from global memory with lookback_window(status, t - 1, ...), or from
// lwin), so that its loads can be issued ahead of other memory traffic.
// lwin, if given, is an earlier copy of status words [lbase, lbase + nwin)
// in LDS; later windows that lie inside it are read from there. A stale
// copy is fine: a word only ever moves from invalid to aggregate to prefix
// within an epoch, and invalid words are read again from global memory.
template <int PL, bool SUM>
__device__ __forceinline__ void lookback(const unsigned long long* status, uint32_t t, uint32_t epoch,
                                         uint32_t lane, Ctl* ctl, const unsigned long long (&first)[PL],
                                         uint32_t& off, uint32_t& sel, const unsigned long long* lwin = nullptr,
                                         int lbase = 0, int nwin = 0) {
    Span acc{0u, 0u, 0u, 1u};  // SUM: acc.c0 alone
    int top = (int)t - 1;
    uint32_t spins = 0;
    for (bool at_first = true;; at_first = false) {
        unsigned long long st[PL];
        if (at_first) {
#pragma unroll
            for (int q = 0; q < PL; ++q) st[q] = first[q];
        } else if (lwin && top - (64 * PL - 1) >= lbase && top < lbase + nwin) {
#pragma unroll
            for (int q = 0; q < PL; ++q) st[q] = lwin[top - (int)(PL * lane + q) - lbase];
        } else {
            lookback_window<PL>(status, top, epoch, lane, st);
        }
        int fq;          // this lane's first q holding a prefix (PL if none)
        uint32_t plane;  // first lane holding a prefix (64 if none); uniform
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
                const int idx = top - (int)(PL * lane + q);
                if (idx >= 0 && !st_valid(st[q], epoch)) st[q] = st_load(status + idx);
            }
        }
        // fold this lane's aggregates, lowest tile (highest q) first, then
        // across the lanes, highest lane (lowest tiles) first: an upward
        // scan with the operands swapped, read at lane 63. For L != R every
        // aggregate is a plain kept count and the fold is a sum.
        uint32_t a = SUM ? 0u : TUP_ID;
        uint32_t pay = 0;
#pragma unroll
        for (int q = PL - 1; q >= 0; --q) {
            const bool inc = (lane < plane) || (lane == plane && q < fq);
            const uint32_t v = (uint32_t)(st[q] & 0xFFFFFFFFull);
            if (SUM) {
                a += inc ? v : 0u;
            } else if (inc) {
                a = tup_then(a, v);
            }
            if (q == fq) pay = v;
        }
        if (SUM) {
            a = wave_scan(a, 0u, [](uint32_t x, uint32_t y) { return x + y; });
            acc.c0 += (uint32_t)__builtin_amdgcn_readlane((int)a, 63);
        } else {
            a = wave_scan(a, TUP_ID, [](uint32_t x, uint32_t y) { return tup_then(y, x); });
            acc = span_after((uint32_t)__builtin_amdgcn_readlane((int)a, 63), acc);
        }
        if (plane < 64) {
            const uint32_t p = (uint32_t)__builtin_amdgcn_readlane((int)pay, (int)plane);
            const uint32_t base = p & 0x7FFFFFFFu, bsel = p >> 31;
            if (SUM) {
                off = base + acc.c0;
                sel = 0u;
            } else {
                off = base + acc.c0 + (bsel ? acc.d : 0u);
                sel = bsel ? acc.o1 : acc.o0;
            }
            return;
        }
        top -= 64 * PL;
    }
}

// LDS index skew for staged output in 16-bit slots: one bank (two slots)
// further every 128 symbols, so that the runs of consecutive threads, and
// the store groups, start on different banks
__host__ __device__ constexpr uint32_t skew(uint32_t i) { return i + 2u * (i >> 7); }
// The staging buffer is written and read both in 16-bit slots and in 4-byte
// words (pairs of slots from an even index: the skew keeps them whole);
// these types tell the compiler that the two views alias.
typedef uint16_t __attribute__((may_alias)) lds16_t;
typedef uint32_t __attribute__((may_alias)) lds32_t;



// Count changes of one thread's positions (bit j: position g0 + j).
// sel holds sel for positions g0 .. g0 + V (bit V: the next thread's first),
// sel_in the sel of position g0 - 1, valid the positions below n. Position
// i changes if it is dropped (sel_i) or becomes X (sel_{i+1}). An old pair
// (i - 1, i) is gone if i - 1 or i changes. A kept position i forms the new
// pair (left neighbour, value) and it is new if either side is an X: the
// left neighbour is X when i - 1 was dropped (sel_{i-1}), otherwise the
// unchanged old symbol i - 1; the value is X when sel_{i+1}. Both masks
// hold candidates: a pair counts only if its ids share a class (no word
// start between them), which count_changes tests. For L != R the pair
// (i - 1, i) of a dropped position i is (L, R) itself, and no other
// changed position holds it: its count after the pass is 0, set once for
// the whole pass (zero_count) instead of one decrement per site, so those
// positions are left out (merged_pair_set).
template <int V>
struct Changes {
    uint32_t gone, born;  // position masks
    __device__ __forceinline__ Changes(uint32_t sel, uint32_t sel_in, uint32_t valid, bool merged_pair_set) {
        constexpr uint32_t VM = (1u << V) - 1u;
        const uint32_t sm1 = ((sel << 1) | sel_in) & VM, s0 = sel & VM, sp1 = (sel >> 1) & VM;
        gone = (sm1 | (merged_pair_set ? 0u : s0) | sp1) & valid;
        born = ~s0 & (sm1 | sp1) & valid & VM;
    }
};

// The count of key in the global table set to 0 (no-op when the key has
// no slot). Used for the merged pair (L, R) with L != R, which occurs
// nowhere after its pass; no other change of the pass touches its slot.
__device__ __forceinline__ void zero_count(const GTable& gt, uint32_t key) {
    uint32_t h = mix32(key) & gt.mask;
    for (uint32_t p = 0; p < GT_PROBES; ++p) {
        const unsigned long long v = __hip_atomic_load(gt.slot + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t cur = (uint32_t)v;
        if (cur == key) {
            __hip_atomic_store(gt.slot + h, (unsigned long long)key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (cur == EMPTY) return;
        h = (h + 1) & gt.mask;
    }
}

// The arguments of count_changes, held from a tile's staging until after
// the next tile's loads are issued (gone = born = 0: nothing to count).
struct CountArgs {
    uint32_t gone, born, sel, sel_in, left;
    const uint16_t* st;
    uint32_t o, kept;
};

// Apply one thread's count changes (masks from Changes) to the workgroup's
// LDS table (the global table when LDS has no room), one changed pair per
// loop turn, so that the insert code exists once. The old symbol at a
// position j of the thread is needed without indexing registers: a dropped
// position held R, one that becomes X held L, and any other position is
// kept unchanged and already staged in LDS (st, at the thread's offset o
// plus the number of kept positions before j). left: old symbol at g0 - 1
// (NOSYM before the first position). cm: the bit mask of the ids below X
// in the merge's class, in LDS; X is in that class, NOSYM in none.
template <int LT>
__device__ __forceinline__ void count_changes(LdsTable<LT>& tab, const GTable& gt, Ctl* ctl, Sweep* sw,
                                              uint32_t theta, uint32_t gone, uint32_t born, uint32_t sel,
                                              uint32_t sel_in, uint32_t left, const uint16_t* st, uint32_t o,
                                              uint32_t kept, uint32_t L, uint32_t R, uint32_t X, const uint32_t* cm) {
    auto old_id = [&](uint32_t j) -> uint32_t {
        if ((sel >> j) & 1u) return R;
        if ((sel >> (j + 1)) & 1u) return L;
        return (uint32_t)reinterpret_cast<const lds16_t*>(st)[skew(o + __popc(kept & ((1u << j) - 1u)))];
    };
    auto in_class = [&](uint32_t v) -> bool {
        return v == X || v == L || v == R || (v < X && ((cm[v >> 5] >> (v & 31u)) & 1u));
    };
    const uint32_t sm1 = (sel << 1) | sel_in;  // bit j: sel of position j - 1
    // one position per loop turn: its old pair (gone) and its new pair
    // (born) share the two old ids and their class tests
    for (uint32_t both = gone | born; both; both &= both - 1u) {
        const uint32_t j = __ffs(both) - 1;
        const uint32_t xl = j ? old_id(j - 1) : left, xj = old_id(j);
        // one id of each pair is L, R or X: the pair lies in one word iff
        // the other id has the merge's class too
        const bool cl = in_class(xl), cj = in_class(xj);
        const bool l_is_x = (sm1 >> j) & 1u, j_is_x = (sel >> (j + 1)) & 1u;
        const bool g = ((gone >> j) & 1u) && cl && cj;
        const bool b = ((born >> j) & 1u) && (l_is_x || cl) && (j_is_x || cj);
        const uint32_t kg = pair_key(xl, xj), kb = pair_key(l_is_x ? X : xl, j_is_x ? X : xj);
#pragma unroll 1
        for (uint32_t e = 0; e < 2u; ++e) {
            if (!(e ? b : g)) continue;
            const uint32_t key = e ? kb : kg, delta = e ? 1u : 0xFFFFFFFFu;
            if (!tab.insert(key, delta)) {
                gt_add_sel(gt, key, delta, ctl, sw, theta);  // the LDS table is full
                // (rare) drain this path's memory operations here: otherwise
                // the compiler assumes they may still be pending where the
                // paths join, and waits for every access, the next tile's
                // loads included, before the look-back
                __builtin_amdgcn_s_waitcnt(0);
            }
        }
    }
}

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
constexpr int BUF_RSRC_FLAGS = 0x00020000;  // raw buffer, gfx9 (dword 3 of the resource)
constexpr uint32_t BUF_OOB = 0x80000000u;   // an offset past any buffer: the store is dropped
// cache policy of the output stores: non-temporal (the next iteration reads
// them back long after this pass has streamed the rest of the array)
constexpr int BUF_NT = 2;

// A position past the array or before its start, in registers: no id
// equals it and it belongs to no class.
constexpr uint32_t NOSYM = 0x10000u;

// A tile is HALVES (two, or one for the smallest corpora) halves of
// TPB * 16 symbols; a thread holds 16 consecutive symbols of each, at
// g0 = tile * TILE + tid * 16 and g0 + TILE / 2. Issue the loads of each
// (two 16-byte loads) and, on the wave's edge lanes,
// of the neighbours the shuffles cannot supply: hw = sym[g0 - 2] |
// sym[g0 - 1] << 16 on lane 0, hr (low half: sym[g0 + 16]) on lane 63.
// Buffer loads through a resource covering the tile, the two symbols before
// it and the one after it (within n, in whole 4-byte words: the padded
// array holds the 16-bit word past n): every lane issues the same four
// loads per half, a lane with nothing to load uses an offset past the resource (the
// hardware returns 0 without a memory access), and a tile past the end gets
// an empty resource. With no branch and a fixed count, the compiler can
// wait for these loads alone, later. The words stay packed until fix_tile,
// so that nothing reads them in the round that issues them. Values outside
// [0, n) are undefined here; fix_tile replaces them by NOSYM.
struct TileRegs {
    uint32_t xr[2][8];  // per half: 16 ids, two per word
    uint32_t hw[2], hr[2];
};
template <int TILE, int HALVES>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ in, uint32_t n, uint32_t tile,
                                          uint32_t ntiles, uint32_t tid, uint32_t lane, TileRegs& r) {
    tile = __builtin_amdgcn_readfirstlane(tile);  // uniform: the resource lives in SGPRs
    const uint32_t ts = tile * TILE, hb = ts >= 2u ? ts - 2u : 0u;  // even: 4-byte aligned
    const uint32_t end = tile < ntiles ? min(n, ts + TILE + 1u) : hb;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(in) + hb, 0, (int)((2u * (end - hb) + 2u) & ~3u), BUF_RSRC_FLAGS);
    // the edge values first: the compiler can then wait for them without
    // waiting for the 16-byte loads (one in-order counter)
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        const uint32_t g0 = ts + (uint32_t)h * (TILE / HALVES) + tid * 16u, o = 2u * (g0 - hb);
        r.hw[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, (lane == 0 && g0 >= 2u) ? o - 4u : BUF_OOB, 0, 0);
        r.hr[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane == 63 ? o + 32u : BUF_OOB, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        const uint32_t o = 2u * (ts + (uint32_t)h * (TILE / HALVES) + tid * 16u - hb);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 16u * q, 0, 0);
            r.xr[h][4 * q] = v.x; r.xr[h][4 * q + 1] = v.y; r.xr[h][4 * q + 2] = v.z; r.xr[h][4 * q + 3] = v.w;
        }
    }
}

// The 16 ids of one half, unpacked.
__device__ __forceinline__ void unpack(uint32_t (&x)[16], const uint32_t (&xr)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[2 * j] = xr[j] & 0xFFFFu;
        x[2 * j + 1] = xr[j] >> 16;
    }
}

// After load_tile, for one half: its 16 ids, NOSYM in place of every
// value outside [0, n), then the neighbours a1 = sym[g0 - 1],
// a2 = sym[g0 - 2], b1 = sym[g0 + 16] (NOSYM outside [0, n)).
__device__ __forceinline__ void fix_tile(uint32_t (&x)[16], const uint32_t (&xr)[8], uint32_t hw, uint32_t hr,
                                         uint32_t g0, uint32_t n, uint32_t lane, bool full, uint32_t& a1,
                                         uint32_t& a2, uint32_t& b1) {
    unpack(x, xr);
    if (!full) {  // uniform: the last tile
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = (g0 + j < n) ? x[j] : NOSYM;
    }
    // selects, not conditional stores: the outputs stay in registers
    const uint32_t d1 = dpp<DPP_WAVE_SHR1>(NOSYM, x[15]);  // from lane - 1
    const uint32_t d2 = dpp<DPP_WAVE_SHR1>(NOSYM, x[14]);
    const uint32_t d3 = dpp<DPP_WAVE_SHL1>(NOSYM, x[0]);  // from lane + 1
    const uint32_t e1 = (g0 >= 1u && g0 - 1u < n) ? hw >> 16 : NOSYM;
    const uint32_t e2 = (g0 >= 2u && g0 - 2u < n) ? hw & 0xFFFFu : NOSYM;
    const uint32_t e3 = (g0 + 16u < n) ? hr & 0xFFFFu : NOSYM;
    a1 = lane == 0 ? e1 : d1;
    a2 = lane == 0 ? e2 : d2;
    b1 = lane == 63 ? e3 : d3;
}

// Occurrence bits of a thread (bit j: position g0 + j, bit V: position
// g0 + V) and its valid positions; a1 = sym[g0 - 1], b1 = sym[g0 + V].
template <int V>
__device__ __forceinline__ void occurrences(const uint32_t (&x)[V], uint32_t a1, uint32_t b1, uint32_t g0,
                                            uint32_t n, uint32_t L, uint32_t R, uint32_t& occ,
                                            uint32_t& valid) {
    // bitwise, not short-circuit: no branch per position. A position
    // outside [0, n) holds NOSYM, which equals neither L nor R.
    occ = 0;
    uint32_t prev = a1;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const uint32_t o = (uint32_t)(prev == L) & (uint32_t)(x[j] == R);
        occ |= o << j;
        prev = x[j];
    }
    occ |= ((uint32_t)(x[V - 1] == L) & (uint32_t)(b1 == R)) << V;
    valid = (g0 >= n) ? 0u : (n - g0 >= (uint32_t)V ? (1u << V) - 1u : (1u << (n - g0)) - 1u);
}

// Write the kept symbols of a tile from LDS (st, 16-bit slots) to
// out[tile_off .. tile_off + tile_kept) as 16-bit ids: up to 7 single
// symbols to reach 16-byte alignment, whole groups of 8 (one 16-byte store
// each), up to 7 single symbols at the end. Each thread issues the same
// fixed sequence of buffer stores (one 2-byte, TILE/8/TPB 16-byte, one
// 2-byte); a store with nothing to write gets an offset past the buffer,
// which the hardware drops. With no branch and a fixed count, the compiler
// can wait for loads issued before these stores without waiting for the
// stores themselves. out is 16-byte aligned.
template <int TPB, int TILE>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ out, const uint16_t* st, uint32_t tile_off,
                                           uint32_t tile_kept) {
    const uint32_t tid = threadIdx.x;
    tile_off = __builtin_amdgcn_readfirstlane(tile_off);  // uniform: the resource lives in SGPRs
    tile_kept = __builtin_amdgcn_readfirstlane(tile_kept);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(out + tile_off, 0, (int)(2u * tile_kept), BUF_RSRC_FLAGS);
    const uint32_t head = min(tile_kept, (8u - (tile_off & 7u)) & 7u);
    const uint32_t body = (tile_kept - head) >> 3;
    const uint32_t rest = head + 8 * body;
    const lds16_t* s16 = reinterpret_cast<const lds16_t*>(st);
    const lds32_t* s32 = reinterpret_cast<const lds32_t*>(st);
    {
        const bool on = tid < head;
        const uint32_t i = on ? tid : 0u;
        __builtin_amdgcn_raw_buffer_store_b16(s16[skew(i)], rs, on ? 2u * i : BUF_OOB, 0, 0);
    }
    // Group q of the thread holds symbols b + 8 * TPB * q .. + 7 with
    // b = head + 8 * tid, read as the five 4-byte words of slots b0 .. b0 + 9
    // (b0 = b rounded down to even; the skew moves by whole words); when b
    // is odd (head odd: uniform) the pairs are shifted by one slot with a
    // funnel shift. A step of 8 * TPB symbols (a multiple of 128) moves
    // every skewed index by the same amount. A group past the body still
    // reads inside the (padded) staging buffer; its store is dropped.
    constexpr uint32_t QSTEP = skew(8 * TPB) / 2;  // in words
    static_assert((8 * TPB) % 128 == 0, "groups keep their offset within 128 symbols");
    const uint32_t b = head + 8u * tid;
    const uint32_t b0 = b & ~1u;
    const bool odd = (head & 1u) != 0u;
    uint32_t a[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) a[k] = skew(b0 + 2u * (uint32_t)k) >> 1;
#pragma unroll
    for (int q = 0; q < TILE / 8 / TPB; ++q) {
        const bool on = tid + q * TPB < body;
        uint32_t u[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) u[k] = s32[a[k] + q * QSTEP];
        v4u32 v;
        if (odd) {
            v = v4u32{__builtin_amdgcn_alignbit(u[1], u[0], 16), __builtin_amdgcn_alignbit(u[2], u[1], 16),
                      __builtin_amdgcn_alignbit(u[3], u[2], 16), __builtin_amdgcn_alignbit(u[4], u[3], 16)};
        } else {
            v = v4u32{u[0], u[1], u[2], u[3]};
        }
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, on ? 2u * (b + 8u * TPB * q) : BUF_OOB, 0, BUF_NT);
    }
    {
        const bool on = tid < tile_kept - rest;
        const uint32_t i = on ? rest + tid : 0u;
        __builtin_amdgcn_raw_buffer_store_b16(s16[skew(i)], rs, on ? 2u * i : BUF_OOB, 0, 0);
    }
}

// Stage the kept symbols of a thread at tile-local offset o; a symbol whose
// right neighbour merges into it becomes X.
// xr: the thread's 16 symbols as loaded (two per word); x: the same
// unpacked (read only when something changes).
template <int V>
__device__ __forceinline__ void stage(uint16_t* st, uint32_t o, const uint32_t (&xr)[V / 2], const uint32_t (&x)[V],
                                      uint32_t valid, uint32_t sel, uint32_t X) {
    constexpr uint32_t VM = (1u << V) - 1u;
    lds16_t* s16 = reinterpret_cast<lds16_t*>(st);
    if (valid == VM && (sel & ((VM << 1) | 1u)) == 0u) {
        // nothing dropped or replaced (most threads): the loaded words go
        // to LDS as they are, from the first even slot at or after o
        // (o + 1 when o is odd: then the pairs are shifted by one symbol);
        // the first symbol and the last two go alone, so that the same ten
        // stores serve both cases
        lds32_t* s32 = reinterpret_cast<lds32_t*>(st);
        const bool odd = (o & 1u) != 0u;
        const uint32_t e = o + (odd ? 1u : 0u);
        s16[skew(o)] = (uint16_t)(xr[0] & 0xFFFFu);
#pragma unroll
        for (int k = 0; k < V / 2 - 1; ++k)
            s32[skew(e + 2u * (uint32_t)k) >> 1] = odd ? __builtin_amdgcn_alignbit(xr[k + 1], xr[k], 16) : xr[k];
        s16[skew(o + V - 2)] = (uint16_t)(xr[V / 2 - 1] & 0xFFFFu);
        s16[skew(o + V - 1)] = (uint16_t)(xr[V / 2 - 1] >> 16);
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if (((valid >> j) & 1u) && !((sel >> j) & 1u)) {
                s16[skew(o)] = (uint16_t)(((sel >> (j + 1)) & 1u) ? X : x[j]);
                ++o;
            }
        }
    }
}

// The last tile publishes the new length and advances the iteration.
// Nothing in this launch reads these; the next launch and the host read
// them after the kernel boundary.
__device__ __forceinline__ void finish_iteration(Ctl* ctl, uint32_t* lengths, uint32_t it, uint32_t total) {
    ctl->n[(it + 1) & 1u] = total;
    lengths[it + 1] = total;
    ctl->k = it + 1;
    ctl->m = it + 1;
}

// Look-back of the pipelined path: windows of 64 * LB_PL status words; the
// LB_WIN words below the tile (two windows) are copied to LDS by
// global_load_lds.
constexpr int LB_PL = 4;
constexpr int LB_WIN = 2 * 64 * LB_PL;
// s_waitcnt immediate (gfx9 encoding): vmcnt <= n (n < 16), expcnt and
// lgkmcnt untouched
constexpr int wait_vm(int n) { return 0x0F70 | n; }
static_assert(LB_WIN % 128 == 0, "whole 16-byte copies per lane");

// Prefixes over the workgroup's NW <= 16 wave totals tot[] in LDS, for the
// calling wave w (uniform): the combination of the totals of waves 0 .. w-1
// (ident for wave 0) and of all NW. Lane i of each 16-lane row takes total
// i, a row scan by DPP row shifts combines them (lanes shifted in from
// outside the row take ident), and two single lanes are read: a handful of
// instructions in place of a select per wave. op(a, b) is a then b.
template <int NW, typename Op>
__device__ __forceinline__ void waves_prefix(const uint32_t* tot, uint32_t w, uint32_t lane, uint32_t ident, Op op,
                                             uint32_t& before, uint32_t& all) {
    static_assert(NW >= 1 && NW <= 16, "one row of 16 lanes");
    const uint32_t i = lane & 15u;
    uint32_t v = i < (uint32_t)NW ? tot[i] : ident;
    // DPP row_shr:1, 2, 4, 8 (row and bank masks all on; no bound control)
    v = op((uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x111, 0xF, 0xF, false), v);
    v = op((uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x112, 0xF, 0xF, false), v);
    v = op((uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x114, 0xF, 0xF, false), v);
    v = op((uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x118, 0xF, 0xF, false), v);
    all = (uint32_t)__builtin_amdgcn_readlane((int)v, NW - 1);
    before = w ? (uint32_t)__builtin_amdgcn_readlane((int)v, (int)w - 1) : ident;
}

// Copy 16 bytes per lane from global memory straight into LDS at
// lds + 16 * lane, with cache policy sc1 (agent-coherent, like st_load).
// Inline assembly, so that the compiler does not track the copy: it would
// otherwise drain every vector memory operation at each later barrier and
// before each later LDS access it cannot tell apart from the destination.
// The caller waits for the copy (vmcnt) before reading the destination,
// and nothing else accesses that LDS range.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else in these kernels uses it
__device__ __forceinline__ void lds_copy16(const unsigned long long* src, const void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Values loaded by load_tile that a round does not consume: an empty use,
// so that the compiler waits for their loads in that round and not when
// the registers are next loaded.
template <int HALVES>
__device__ __forceinline__ void retire(const TileRegs& r) {
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
        asm volatile("" ::"v"(r.xr[h][0]), "v"(r.xr[h][1]), "v"(r.xr[h][2]), "v"(r.xr[h][3]), "v"(r.xr[h][4]),
                     "v"(r.xr[h][5]), "v"(r.xr[h][6]), "v"(r.xr[h][7]), "v"(r.hw[h]), "v"(r.hr[h]));
}

// ---------------------------------------------------------------- selection
constexpr int SWEEP_UNROLL = 8;  // table loads in flight per thread

// Maximum of v over the workgroup (every thread gets it). s_best: NW slots.
template <int NW>
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, unsigned long long* s_best,
                                                             uint32_t lane, uint32_t w) {
    v = wave_max_u64(v);
    if (lane == 0) s_best[w] = v;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NW; ++i) v = s_best[i] > v ? s_best[i] : v;
    lds_barrier();  // s_best free again
    return v;
}

// A chunk counter claimed by the workgroup: thread 0 takes the next chunk,
// every thread gets its number.
__device__ __forceinline__ uint32_t claim_chunk(uint32_t* ctr, uint32_t* s_u32) {
    if (threadIdx.x == 0) *s_u32 = atomicAdd(ctr, 1u);
    lds_barrier();
    const uint32_t c = *s_u32;
    lds_barrier();  // s_u32 free again
    return c;
}

// The largest packed candidate (COLLECT false) of this thread's slots of
// chunk c, or (COLLECT true) the chunk's slots whose count is theta or more
// appended to the candidate list. Agent-coherent loads: other workgroups'
// table adds reach memory, not this XCD's L2.
// (Table sizes are powers of two of at least 1024 slots, so a wave's lanes
// run the same rounds.)
template <int TPB, bool COLLECT>
__device__ __forceinline__ unsigned long long sweep_chunk(const GTable& gt, Sweep* sw, uint32_t c, uint32_t theta) {
    static_assert(SWEEP_CHUNK % (64 * SWEEP_UNROLL) == 0, "whole waves per round");
    const uint32_t slots = gt.mask + 1u;
    const uint32_t end = min(slots, (c + 1u) * SWEEP_CHUNK);
    unsigned long long best = 0ull;
    for (uint32_t s0 = c * SWEEP_CHUNK + threadIdx.x; s0 < end; s0 += SWEEP_UNROLL * TPB) {
        unsigned long long v[SWEEP_UNROLL];
#pragma unroll
        for (int k = 0; k < SWEEP_UNROLL; ++k) {
            const uint32_t i = s0 + k * TPB;
            v[k] = i < end ? ld_agent(gt.slot + i) : 0ull;
        }
        if (COLLECT) {
            uint32_t take = 0u;  // slots past the end hold 0, below theta
#pragma unroll
            for (int k = 0; k < SWEEP_UNROLL; ++k) take |= ((uint32_t)(v[k] >> 32) >= theta ? 1u : 0u) << k;
            cand_append_wave<SWEEP_UNROLL>(sw, s0, TPB, take);
        } else {
#pragma unroll
            for (int k = 0; k < SWEEP_UNROLL; ++k) {
                const unsigned long long cv = candidate(v[k]);
                best = cv > best ? cv : best;
            }
        }
    }
    return best;
}

// An iteration that sweeps the table. Running workgroups claim chunks of
// the table and fold each chunk's maximum into smax; the workgroup whose
// chunks complete the count of finished chunks has every chunk's maximum in
// smax: it empties the candidate list, stores the new threshold and
// publishes the maximum. Every workgroup waits for the publication (it
// comes from a workgroup that is running), then all claim chunks again to
// collect the slots at or above the threshold (no one waits for that: the
// merge pass's own adds append what they lift across theta, and counts of
// existing pairs only fall). A workgroup that starts after the chunks are
// gone only reads the publication.
template <int TPB>
__device__ __forceinline__ unsigned long long sweep_select(const GTable& gt, Sweep* sw, Ctl* ctl, uint32_t p,
                                                            uint32_t it, unsigned long long* s_best,
                                                            uint32_t* s_u32, uint32_t lane, uint32_t w,
                                                            uint32_t& theta) {
    constexpr int NW = TPB / 64;
    const uint32_t nch = (gt.mask + SWEEP_CHUNK) / SWEEP_CHUNK;
    uint32_t mine = 0;
    unsigned long long part = 0ull;
    for (uint32_t c; (c = claim_chunk(&sw->c1[p], s_u32)) < nch; ++mine) {
        const unsigned long long m = sweep_chunk<TPB, false>(gt, sw, c, 0u);
        part = m > part ? m : part;
    }
    const unsigned long long wbest = block_max_u64<NW>(part, s_best, lane, w);
    const uint32_t shift_now = ld_agent(&sw->shift);
    const uint32_t shift = shift_now ? shift_now : SHIFT_DEFAULT;
    if (threadIdx.x == 0) {
        if (mine) {
            // the maximum is in smax before the chunks count as finished
            const unsigned long long o = atomicMax(&sw->smax[p], wbest);
            asm volatile("" ::"v"(o));
            if (atomicAdd(&sw->c1done[p], mine) + mine == nch) {
                const unsigned long long m = ld_agent(&sw->smax[p]);
                const uint32_t mc = (uint32_t)(m >> 32);
                st_agent(&sw->cand_n, 0u);
                st_agent(&sw->theta, mc - (mc >> shift));
                st_agent(&sw->shift, shift);
                st_agent(&sw->cand_ok, 1u);
                st_agent(&sw->sweeps, ld_agent(&sw->sweeps) + 1u);
                st_agent(&sw->spub[p], m);
                __builtin_amdgcn_s_waitcnt(0);  // the stores above are complete before the epoch
                st_agent(&sw->spub_epoch[p], it + 1u);
            }
        }
        uint32_t spins = 0;
        while (ld_agent(&sw->spub_epoch[p]) != it + 1u) {
            if (++spins > SPIN_LIMIT) {
                atomicOr(&ctl->err, ERR_SPIN);
                atomicExch(&ctl->done, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        s_best[0] = ld_agent(&sw->spub[p]);
    }
    lds_barrier();
    const unsigned long long best = s_best[0];
    lds_barrier();  // s_best free again
    const uint32_t mc = (uint32_t)(best >> 32);
    theta = mc - (mc >> shift);
    if (best != 0ull)
        for (uint32_t c; (c = claim_chunk(&sw->c2[p], s_u32)) < nch;) sweep_chunk<TPB, true>(gt, sw, c, theta);
    return best;
}

// The largest packed candidate among the list's first n entries whose
// count is theta or more (0 if none). Plain loads: the list and the table
// are as the previous launch left them, and nothing changes them before
// the selection is published.
template <int TPB>
__device__ __forceinline__ unsigned long long list_max(const GTable& gt, const Sweep* sw, uint32_t n, uint32_t theta,
                                                        unsigned long long* s_best, uint32_t lane, uint32_t w) {
    unsigned long long best = 0ull;
    for (uint32_t i = threadIdx.x; i < n; i += TPB) {
        const unsigned long long v = gt.slot[sw->cand[i] & gt.mask];
        const unsigned long long c = (uint32_t)(v >> 32) >= theta ? candidate(v) : 0ull;
        best = c > best ? c : best;
    }
    return block_max_u64<TPB / 64>(best, s_best, lane, w);
}

// The per-workgroup flush of count changes (flush_table) with the merge
// pass's table adds.
template <int LT>
__device__ __forceinline__ void flush_table_sel(LdsTable<LT>& tab, int tpb, const GTable& gt, Ctl* ctl, Sweep* sw,
                                                uint32_t theta) {
    for (int i = threadIdx.x; i < LT; i += tpb) {
        const uint32_t key = tab.keys[i], c = tab.cnts[i];
        if (key != EMPTY && c != 0u) gt_add_sel(gt, key, c, ctl, sw, theta);
        tab.keys[i] = EMPTY;
        tab.cnts[i] = 0u;
    }
    if (threadIdx.x == 0) {
        tab.used = 0u;
        tab.qn = 0u;
    }
}

// The merge of iteration it, selected by the workgroup that drew ticket 0
// (every thread of it calls this): the replayed pair if k_force listed one, else
// the maximum over the candidate list if the list vouches for it, else
// SEL_SWEEP (with the shift for that sweep steered by the list's size: a
// list longer than the target narrows the next window, a small one widens
// it). Then published: each of the first PUB_COPIES threads writes its
// copy's value and, once that store is complete, its epoch.
template <int TPB>
__device__ __forceinline__ void select_and_publish(const GTable& gt, Sweep* sw, uint32_t p, uint32_t it,
                                                   uint32_t theta, unsigned long long* s_best, uint32_t lane,
                                                   uint32_t w) {
    unsigned long long sel;
    if (sw->force_epoch == it + 1u) {
        sel = sw->force_val;
    } else {
        const uint32_t nc = sw->cand_n;
        const bool ok = sw->cand_ok != 0u;
        unsigned long long best = 0ull;
        if (ok && nc <= CAND_MAX) best = list_max<TPB>(gt, sw, nc, theta, s_best, lane, w);
        sel = best ? best : SEL_SWEEP;
        if (!best && threadIdx.x == 0) {
            uint32_t shift = sw->shift ? sw->shift : SHIFT_DEFAULT;
            if (ok && nc > CAND_TARGET) shift = min(shift + 1u, SHIFT_MAX);
            else if (ok && nc < CAND_TARGET / 16u && shift > 1u) shift = shift - 1u;
            st_agent(&sw->shift, shift);  // read by the sweep, after the publication
        }
    }
    static_assert(PUB_COPIES % TPB == 0 || TPB % PUB_COPIES == 0, "whole rounds of copies");
    __syncthreads();  // the shift above is complete before any copy is published
    for (uint32_t c = threadIdx.x; c < PUB_COPIES; c += TPB) {
        st_agent(&sw->pub[p][c], sel);
        __builtin_amdgcn_s_waitcnt(0);  // the value is visible before its epoch
        st_agent(&sw->pub_epoch[p][c], it + 1u);
    }
}

// The published merge of iteration it, from this workgroup's copy (a
// bounded wait for the workgroup that drew ticket 0, which is running). Every thread of the workgroup calls this.
__device__ __forceinline__ unsigned long long read_publication(Sweep* sw, Ctl* ctl, uint32_t p, uint32_t it,
                                                               unsigned long long* s_best) {
    if (threadIdx.x == 0) {
        const uint32_t c = blockIdx.x % PUB_COPIES;
        uint32_t spins = 0;
        while (ld_agent(&sw->pub_epoch[p][c]) != it + 1u) {
            if (++spins > SPIN_LIMIT) {
                atomicOr(&ctl->err, ERR_SPIN);
                atomicExch(&ctl->done, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        s_best[0] = ld_agent(&sw->pub[p][c]);
    }
    lds_barrier();
    const unsigned long long v = s_best[0];
    lds_barrier();  // s_best free again
    return v;
}

// Once this workgroup has written its last tile: add its summed count
// changes to the global table (it has read the publication, so every read
// of the selection is done). Every thread of the workgroup calls this once
// per pass.
template <int TPB, int LT>
__device__ __forceinline__ void finish_counts(LdsTable<LT>& tab, const GTable& gt, Ctl* ctl, Sweep* sw,
                                              uint32_t theta) {
    lds_barrier();  // every count change of the workgroup is in LDS
    if (tab.used) flush_table_sel(tab, TPB, gt, ctl, sw, theta);  // uniform: read after the barrier
}

// Symbols of a merge pass's tile: HALVES halves of 16 symbols per thread.
__host__ __device__ constexpr int merge_tile(int tpb, int halves) { return tpb * 16 * halves; }

// Dynamic LDS of the pass of iteration it: the class mask of ids up to
// X = 256 + it.
__host__ __device__ constexpr uint32_t cmask_lds_bytes(uint32_t it) { return 4u * (((BASE + it) >> 5) + 1u); }

// One launch per iteration it (the host passes it; a launch after training
// has stopped does nothing). The workgroup that draws ticket 0 selects the
// merge and publishes it; the others read the publication while their
// first tile's loads are in flight. Then a persistent pass: workgroups take
// tiles from a counter, in order, so every tile a look-back waits for is
// held by a running workgroup that has already published or is about to
// publish its aggregate.
//
// L != R (nearly every merge): occurrences cannot overlap, so every
// occurrence is merged and sel_i = occ_i. A tile's kept symbols, its staged
// output and its count changes are then known from the tile and the two
// symbols before each half; the look-back only supplies the tile's output
// offset. The workgroup publishes the tile's aggregate, stages it, takes
// the next tile and issues its loads, applies the count changes, and only
// then waits for the look-back and writes: the next tile's loads are in
// flight while it waits.
//
// L == R: the selection carries along runs (sel_i = occ_i and not
// sel_{i-1}) and a tile's selection can depend on every tile before it, so
// staging waits for the look-back's sel as well.
template <int TPB, int LT, int HALVES>
// 4 waves per SIMD: at most 128 VGPRs
__global__ __launch_bounds__(TPB, 4) void k_merge(uint32_t it, Ctl* ctl, uint16_t* __restrict__ buf0,
                                               uint16_t* __restrict__ buf1, GTable gt,
                                               unsigned long long* status,
                                               uint32_t* lengths, Sweep* sw, uint32_t* merges,
                                               uint8_t* __restrict__ cls, uint32_t* __restrict__ cmask) {
    constexpr int V = 16;  // symbols per thread and half: two 16-byte loads
    constexpr int HALF = TPB * V;
    constexpr int TILE = HALVES * HALF;
    constexpr bool TWO = HALVES == 2;
    static_assert(HALVES == 1 || HALVES == 2, "one or two halves");
    static_assert(TILE == merge_tile(TPB, HALVES), "the host sizes grids by this tile");
    constexpr int NW = TPB / 64;
    constexpr uint32_t VM = (1u << V) - 1u;
    constexpr uint32_t SST = TILE + TILE / 64;  // one staging buffer (skewed)
    __shared__ LdsTable<LT> tab;  // count changes of this workgroup
    __shared__ uint16_t s_stage[2 * SST + 8];  // + 8: reads of dropped store groups stay inside
    // ids up to X in the merge's class: (X >> 5) + 1 words of dynamic LDS
    // (cmask_lds_bytes), so that early passes of small corpora keep two
    // workgroups per CU
    extern __shared__ uint32_t s_cmask[];
    __shared__ uint32_t s_wagg[NW], s_waggb[NW];
    __shared__ uint32_t s_tile[2], s_off[2], s_sel, s_dep, s_off_now, s_u32;
    __shared__ unsigned long long s_best[NW];
    __shared__ __align__(16) unsigned long long s_win[LB_WIN];

    // state the previous launch left (plain, uniform loads: scalar, cached)
    if (ctl->done) return;  // training has stopped
    const uint32_t p = it & 1u;  // parity of the per-iteration counters
    const uint32_t n = ctl->n[it & 1u];
    const uint16_t* __restrict__ in = (it & 1u) ? buf1 : buf0;
    uint16_t* __restrict__ out = (it & 1u) ? buf0 : buf1;
    const uint32_t ntiles = (n + TILE - 1) / TILE;
    const uint32_t epoch = it + 1;
    const uint32_t X = BASE + it;
    // X == 65535 is the last possible id: no later iteration reads counts,
    // and the pair (X, X) would collide with the empty key
    const bool do_count = X != IDM;
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: in a scalar register
    uint32_t* tile_ctr = &ctl->tile_ctr[p];
    // ticket 0 of the tile counter is the selection of the merge, not a
    // tile: ticket k > 0 is tile k - 1
    constexpr uint32_t tile_base = 1u;
    if (blockIdx.x == 0 && tid == 0) {
        // the counters of the next iteration (the previous one's are done with)
        __hip_atomic_store(&ctl->tile_ctr[p ^ 1u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st_agent(&sw->c1[p ^ 1u], 0u);
        st_agent(&sw->c1done[p ^ 1u], 0u);
        st_agent(&sw->c2[p ^ 1u], 0u);
        st_agent(&sw->smax[p ^ 1u], 0ull);
    }

    tab.clear(TPB);
    if (tid == 0) s_tile[0] = atomicAdd(tile_ctr, 1u);
    uint32_t theta = sw->theta;  // the list's threshold, as the previous launch left it
    lds_barrier();
    // ---- the merge: selected by the workgroup that drew ticket 0 (it is
    // running), before it issues any tile load, and published to all
    if (s_tile[0] == 0u) {  // uniform
        select_and_publish<TPB>(gt, sw, p, it, theta, s_best, lane, w);
        if (tid == 0) s_tile[1] = atomicAdd(tile_ctr, 1u);
        lds_barrier();
        if (tid == 0) s_tile[0] = s_tile[1];
        lds_barrier();
    }
    uint32_t t = s_tile[0] - tile_base;
    TileRegs tr;
    static_assert(V == 16, "load_tile and fix_tile take 16 symbols per thread and half");
    load_tile<TILE, HALVES>(in, n, t, ntiles, tid, lane, tr);
    unsigned long long best = read_publication(sw, ctl, p, it, s_best);
    if (best == SEL_SWEEP) best = sweep_select<TPB>(gt, sw, ctl, p, it, s_best, &s_u32, lane, w, theta);  // uniform
    if (best == 0ull) {  // uniform: no countable pair is left
        if (blockIdx.x == 0 && tid == 0) st_agent(&ctl->done, 1u);
        return;
    }
    // uniform: keep the merge in scalar registers
    const uint32_t key = __builtin_amdgcn_readfirstlane(~(uint32_t)best);
    const uint32_t L = key >> 16;
    // the class of the merge (L < X: set by the start or an earlier pass);
    // a replayed pair of two classes never occurs: its R matches no symbol
    const uint32_t c = __builtin_amdgcn_readfirstlane((uint32_t)cls[L]);
    if (c >= N_CLASSES) {  // uniform over the grid: the same L everywhere
        if (blockIdx.x == 0 && tid == 0) {
            atomicOr(&ctl->err, ERR_CLASS);
            st_agent(&ctl->done, 1u);
        }
        return;
    }
    const uint32_t R = (uint32_t)cls[key & IDM] == c ? key & IDM : NOSYM + 1u;
    if (blockIdx.x == 0 && tid == 0) {
        merges[3 * it + 0] = L;
        merges[3 * it + 1] = key & IDM;
        merges[3 * it + 2] = __builtin_amdgcn_readfirstlane((uint32_t)(best >> 32));
        ctl->L = L;
        ctl->R = key & IDM;
        ctl->X = X;
        // X has L's class; passes of this launch read only bits below X
        cls[X] = (uint8_t)c;
        atomicOr(&cmask[c * CLASS_WORDS + (X >> 5)], 1u << (X & 31u));
        // every (L, R) with L != R is merged: its count becomes 0 (Changes)
        if (do_count && L != R && R == (key & IDM)) zero_count(gt, key);
    }
    // the mask of the merge's class, for the ids up to X
    for (uint32_t i = tid; i <= (X >> 5) && i < CLASS_WORDS; i += TPB) s_cmask[i] = cmask[c * CLASS_WORDS + i];

    if (L != R) {
        // tp: the tile staged in the previous round, waiting for its offset
        // (ntiles: none); kp its kept count; cur the staging buffer of the
        // current tile (the pending one is in the other)
        uint32_t tp = ntiles, kp = 0, cur = 0;
        // The tile after t, taken one round ahead: waiting for a returning
        // atomic waits for every older access of the wave (one counter), so
        // it is issued after the stores of a round and consumed in the next.
        uint32_t grab = 0;
        if (tid == 0) grab = atomicAdd(tile_ctr, 1u);
        // the loop-top waits count on the stores each round issues after its
        // loads; the first loads get the same six stores (nothing written)
        store_tile<TPB, TILE>(out, s_stage, 0u, 0u);
        for (uint32_t round = 1; t < ntiles || tp < ntiles; ++round) {
            uint32_t tn = ntiles, tile_kept = 0;
            CountArgs cca{}, ccb{};
            // the previous tile's first look-back window (the 512 status
            // words below it), copied straight into LDS before anything else
            // of the round, so that it has arrived by the time wave 0
            // examines it and occupies no registers meanwhile
            const int lb_top = (int)tp - 1;
            const int lb_base = lb_top >= LB_WIN - 1 ? lb_top - (LB_WIN - 1) : 0;
            if (w == 0 && tp < ntiles && tp != 0) {
#pragma unroll
                for (int q = 0; q < LB_WIN / 128; ++q)
                    lds_copy16(status + lb_base + 2 * (lane + 64 * q), s_win + 128 * q);
            }
            if (t < ntiles) {  // uniform
                const uint32_t g0 = t * TILE + tid * V;  // half A; half B at g0 + HALF
                const bool full = t * TILE + TILE <= n;
                uint32_t x[V], a1, a2, b1, occa, valida, occb = 0, validb = 0, sel_inb = 0, leftb = NOSYM;
                fix_tile(x, tr.xr[0], tr.hw[0], tr.hr[0], g0, n, lane, full, a1, a2, b1);
                occurrences<V>(x, a1, b1, g0, n, L, R, occa, valida);
                // sel = occ; the position before g0 is merged iff it is an occurrence
                const uint32_t sel_ina = (a2 == L && a1 == R) ? 1u : 0u;  // NOSYM before the start
                const uint32_t lefta = a1;
                if constexpr (TWO) {
                    fix_tile(x, tr.xr[1], tr.hw[1], tr.hr[1], g0 + HALF, n, lane, full, a1, a2, b1);
                    occurrences<V>(x, a1, b1, g0 + HALF, n, L, R, occb, validb);
                    sel_inb = (a2 == L && a1 == R) ? 1u : 0u;
                    leftb = a1;
                }

                // ---- kept counts of both halves in one word (at most HALF
                // each): wave scan, then across the waves
                const uint32_t kept = __popc(valida & ~occa & VM) | (__popc(validb & ~occb & VM) << 16);
                const uint32_t incl = wave_scan(kept, 0u, [](uint32_t a, uint32_t b) { return a + b; });
                if (lane == 63) s_wagg[w] = incl;
                if (tid == 0) s_tile[round & 1u] = grab - tile_base;
                lds_barrier();
                uint32_t before, all;
                waves_prefix<NW>(s_wagg, w, lane, 0u, [](uint32_t a, uint32_t b) { return a + b; }, before, all);
                const uint32_t kept_a = all & 0xFFFFu;
                tile_kept = kept_a + (all >> 16);
                const uint32_t ex = incl - kept + before;
                // the tile's aggregate goes out before anything else is done
                if (tid == 0 && t != 0)
                    st_store(status + t, st_pack(ST_AGG, epoch, tup_make(tile_kept, 0u, 0u, 0u)));

                uint16_t* st = s_stage + cur * SST;
                // half B first (its ids are unpacked), then half A again from its words
                if constexpr (TWO) {
                    stage<V>(st, kept_a + (ex >> 16), tr.xr[1], x, validb, occb, X);
                    if (do_count && (occb | sel_inb)) {
                        const Changes<V> ch(occb, sel_inb, validb, true);
                        ccb = CountArgs{ch.gone, ch.born, occb, sel_inb, leftb, st, kept_a + (ex >> 16), validb & ~occb};
                    }
                    unpack(x, tr.xr[0]);
                }
                stage<V>(st, ex & 0xFFFFu, tr.xr[0], x, valida, occa, X);
                if (do_count && (occa | sel_ina)) {
                    const Changes<V> ch(occa, sel_ina, valida, true);
                    cca = CountArgs{ch.gone, ch.born, occa, sel_ina, lefta, st, ex & 0xFFFFu, valida & ~occa};
                }
                tn = s_tile[round & 1u];
            } else {
                retire<HALVES>(tr);
            }
            // ---- the next tile's loads (an empty resource when there is none), then this
            // tile's count changes (they need the old symbols only as masks and staged values)
            load_tile<TILE, HALVES>(in, n, tn, ntiles, tid, lane, tr);
            if (cca.gone | cca.born)
                count_changes<LT>(tab, gt, ctl, sw, theta, cca.gone, cca.born, cca.sel, cca.sel_in, cca.left, cca.st,
                                  cca.o, cca.kept, L, R, X, s_cmask);
            if (ccb.gone | ccb.born)
                count_changes<LT>(tab, gt, ctl, sw, theta, ccb.gone, ccb.born, ccb.sel, ccb.sel_in, ccb.left, ccb.st,
                                  ccb.o, ccb.kept, L, R, X, s_cmask);
            // ---- the previous tile: its predecessors have had a round to publish
            if (tp < ntiles && w == 0) {
                uint32_t off = 0, sel = 0;
                if (tp != 0) {
                    // the window's copies are older than the four loads per
                    // half of load_tile above: all but that many accesses done
                    __builtin_amdgcn_s_waitcnt(wait_vm(4 * HALVES));
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    unsigned long long lbw[LB_PL];
#pragma unroll
                    for (int q = 0; q < LB_PL; ++q) {
                        const int idx = lb_top - (int)(LB_PL * lane + q);
                        lbw[q] = idx >= 0 ? s_win[idx - lb_base] : st_pack(ST_PRE, epoch, 0u);
                    }
                    lookback<LB_PL, true>(status, tp, epoch, lane, ctl, lbw, off, sel, s_win, lb_base, LB_WIN);
                }
                if (lane == 0) {
                    st_store(status + tp, st_pack(ST_PRE, epoch, off + kp));
                    s_off[round & 1u] = off;
                }
            }
            lds_barrier();
            // the grab goes before the stores so that waiting for it later
            // does not wait for them; the stores are issued in every round
            // (all dropped when no tile is pending) to keep their count fixed
            if (tid == 0 && tn < ntiles) grab = atomicAdd(tile_ctr, 1u);
            const uint32_t tile_off = tp < ntiles ? s_off[round & 1u] : 0u;
            store_tile<TPB, TILE>(out, s_stage + (cur ^ 1u) * SST, tile_off, tp < ntiles ? kp : 0u);
            if (tp == ntiles - 1 && tid == 0) finish_iteration(ctl, lengths, it, tile_off + kp);
            if (t < ntiles) {
                tp = t;
                kp = tile_kept;
                cur ^= 1u;
            } else {
                tp = ntiles;
            }
            t = tn;
        }
    } else {
        // L == R: the selection of a position depends on the one before it
        // (run-length parity), so a tile's selection depends on the state it
        // is entered with, but only through its leading chain of
        // occurrences: the first position that is not an occurrence resets
        // it. When neither the tile's first position nor the one before it
        // (whose selection decides the pair across the boundary for the
        // counts) is an occurrence, the entry state is known to be "not
        // selected": the tile is staged at once and pipelined like the
        // L != R path (its look-back, a round later, only supplies the
        // output offset). Otherwise the tile runs its look-back at once, as
        // its staging needs the entry state, and is stored in the next round
        // with no second look-back. Tile 0 (entered with nothing selected)
        // publishes its inclusive prefix as soon as it is staged: a
        // workgroup's immediate look-back never waits for its own pending
        // tile, whose aggregate is out, but would wait for tile 0's prefix.
        // Aggregates are the selection tuples.
        uint32_t tp = ntiles, kp = 0, cur = 0, agg_p = TUP_ID, off_p = 0;
        bool done_p = false;  // the pending tile's prefix is out (offset off_p)
        uint32_t grab = 0;
        if (tid == 0) grab = atomicAdd(tile_ctr, 1u);
        store_tile<TPB, TILE>(out, s_stage, 0u, 0u);
        for (uint32_t round = 1; t < ntiles || tp < ntiles; ++round) {
            uint32_t tn = ntiles, tile_kept = 0, tile_agg = TUP_ID, off_t = 0;
            CountArgs cca{}, ccb{};
            bool dep = false;
            const int lb_top = (int)tp - 1;
            const int lb_base = lb_top >= LB_WIN - 1 ? lb_top - (LB_WIN - 1) : 0;
            const bool lb_pending = tp < ntiles && !done_p;  // tile 0 is always done
            if (w == 0 && lb_pending) {
#pragma unroll
                for (int q = 0; q < LB_WIN / 128; ++q)
                    lds_copy16(status + lb_base + 2 * (lane + 64 * q), s_win + 128 * q);
            }
            if (t < ntiles) {  // uniform
                const uint32_t g0 = t * TILE + tid * V;  // half A; half B at g0 + HALF
                const bool full = t * TILE + TILE <= n;
                uint32_t x[V], a1, a2, b1, occa, valida, occb = 0, validb = 0, leftb = NOSYM;
                fix_tile(x, tr.xr[0], tr.hw[0], tr.hr[0], g0, n, lane, full, a1, a2, b1);
                occurrences<V>(x, a1, b1, g0, n, L, R, occa, valida);
                const uint32_t lefta = a1;
                const uint32_t dep0 = (occa & 1u) | (uint32_t)(a2 == L && a1 == L);  // used by thread 0
                if constexpr (TWO) {
                    fix_tile(x, tr.xr[1], tr.hw[1], tr.hr[1], g0 + HALF, n, lane, full, a1, a2, b1);
                    occurrences<V>(x, a1, b1, g0 + HALF, n, L, R, occb, validb);
                    leftb = a1;
                }

                // ---- each half's tuple per thread, then inclusive scans over
                // the wave and the waves, half by half
                auto thread_tuple = [](uint32_t occ, uint32_t valid) -> uint32_t {
                    uint32_t s0 = 0, s1 = 1, c0 = 0, c1 = 0;
#pragma unroll
                    for (int j = 0; j < V; ++j) {
                        const uint32_t o = (occ >> j) & 1u, v = (valid >> j) & 1u;
                        s0 = o & ~s0 & 1u;
                        s1 = o & ~s1 & 1u;
                        c0 += v & ~s0 & 1u;
                        c1 += v & ~s1 & 1u;
                    }
                    return tup_make(c0, c1 - c0, s0, s1);
                };
                auto then = [](uint32_t a, uint32_t b) { return tup_then(a, b); };
                const uint32_t incla = wave_scan(thread_tuple(occa, valida), TUP_ID, then);
                const uint32_t inclb = TWO ? wave_scan(thread_tuple(occb, validb), TUP_ID, then) : TUP_ID;
                const uint32_t lane_excla = dpp<DPP_WAVE_SHR1>(TUP_ID, incla);
                const uint32_t lane_exclb = dpp<DPP_WAVE_SHR1>(TUP_ID, inclb);
                if (lane == 63) {
                    s_wagg[w] = incla;
                    if constexpr (TWO) s_waggb[w] = inclb;
                }
                if (tid == 0) {
                    s_tile[round & 1u] = grab - tile_base;
                    s_dep = dep0;
                }
                lds_barrier();
                uint32_t wave_excla, agg_a, wave_exclb = TUP_ID, agg_b = TUP_ID;
                waves_prefix<NW>(s_wagg, w, lane, TUP_ID, then, wave_excla, agg_a);
                if constexpr (TWO) waves_prefix<NW>(s_waggb, w, lane, TUP_ID, then, wave_exclb, agg_b);
                tile_agg = tup_then(agg_a, agg_b);
                dep = s_dep != 0u;  // uniform
                // the tile's aggregate (tile 0: prefix) goes out before anything else is done
                if (tid == 0)
                    st_store(status + t, t != 0 ? st_pack(ST_AGG, epoch, tile_agg)
                                                : st_pack(ST_PRE, epoch, tup_c0(tile_agg) | (tup_o(tile_agg, 0u) << 31)));
                uint32_t tile_sel = 0;
                if (dep) {  // uniform: the entry state is needed now
                    if (w == 0) {
                        uint32_t off = 0, sel = 0;
                        unsigned long long lbw[4];
                        lookback_window<4>(status, (int)t - 1, epoch, lane, lbw);
                        lookback<4, false>(status, t, epoch, lane, ctl, lbw, off, sel);
                        if (lane == 0) {
                            const uint32_t kept = tup_c0(tile_agg) + (sel ? tup_d(tile_agg) : 0u);
                            st_store(status + t,
                                     st_pack(ST_PRE, epoch, (off + kept) | (tup_o(tile_agg, sel) << 31)));
                            s_off_now = off;
                            s_sel = sel;
                        }
                    }
                    lds_barrier();
                    tile_sel = s_sel;
                    off_t = s_off_now;
                }
                const uint32_t texcla = tup_then(wave_excla, lane_excla);
                const uint32_t texclb = tup_then(agg_a, tup_then(wave_exclb, lane_exclb));
                tile_kept = tup_c0(tile_agg) + (tile_sel ? tup_d(tile_agg) : 0u);

                // ---- resolve sel, stage, count changes (each half's ids
                // unpacked again from its words: fewer registers held over
                // the scans and the look-back)
                auto resolve = [](uint32_t occ, uint32_t sel_in) -> uint32_t {
                    uint32_t selbits = 0, sv = sel_in;
#pragma unroll
                    for (int j = 0; j <= V; ++j) {
                        sv = (occ >> j) & ~sv & 1u;
                        selbits |= sv << j;
                    }
                    return selbits;
                };
                uint16_t* st = s_stage + cur * SST;
                if constexpr (TWO) {
                    unpack(x, tr.xr[1]);
                    const uint32_t loc = tup_c0(texclb) + (tile_sel ? tup_d(texclb) : 0u);
                    const uint32_t sel_in = tup_o(texclb, tile_sel);
                    const uint32_t selbits = resolve(occb, sel_in);
                    stage<V>(st, loc, tr.xr[1], x, validb, selbits, X);
                    if (do_count && (occb | sel_in)) {
                        const Changes<V> ch(selbits, sel_in, validb, false);
                        ccb = CountArgs{ch.gone, ch.born, selbits, sel_in, leftb, st, loc, validb & ~selbits};
                    }
                }
                unpack(x, tr.xr[0]);
                {
                    const uint32_t loc = tup_c0(texcla) + (tile_sel ? tup_d(texcla) : 0u);
                    const uint32_t sel_in = tup_o(texcla, tile_sel);
                    const uint32_t selbits = resolve(occa, sel_in);
                    stage<V>(st, loc, tr.xr[0], x, valida, selbits, X);
                    if (do_count && (occa | sel_in)) {
                        const Changes<V> ch(selbits, sel_in, valida, false);
                        cca = CountArgs{ch.gone, ch.born, selbits, sel_in, lefta, st, loc, valida & ~selbits};
                    }
                }
                tn = s_tile[round & 1u];
            } else {
                retire<HALVES>(tr);
            }
            // ---- the next tile's loads (an empty resource when there is none), then this
            // tile's count changes (they need the old symbols only as masks and staged values)
            load_tile<TILE, HALVES>(in, n, tn, ntiles, tid, lane, tr);
            if (cca.gone | cca.born)
                count_changes<LT>(tab, gt, ctl, sw, theta, cca.gone, cca.born, cca.sel, cca.sel_in, cca.left, cca.st,
                                  cca.o, cca.kept, L, R, X, s_cmask);
            if (ccb.gone | ccb.born)
                count_changes<LT>(tab, gt, ctl, sw, theta, ccb.gone, ccb.born, ccb.sel, ccb.sel_in, ccb.left, ccb.st,
                                  ccb.o, ccb.kept, L, R, X, s_cmask);
            // ---- the previous tile: its offset (unless its look-back is done)
            if (tp < ntiles && w == 0) {
                uint32_t off = off_p, sel = 0;
                if (!done_p) {  // tp != 0
                    __builtin_amdgcn_s_waitcnt(wait_vm(4 * HALVES));
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    unsigned long long lbw[LB_PL];
#pragma unroll
                    for (int q = 0; q < LB_PL; ++q) {
                        const int idx = lb_top - (int)(LB_PL * lane + q);
                        lbw[q] = idx >= 0 ? s_win[idx - lb_base] : st_pack(ST_PRE, epoch, 0u);
                    }
                    lookback<LB_PL, false>(status, tp, epoch, lane, ctl, lbw, off, sel, s_win, lb_base, LB_WIN);
                    if (lane == 0)
                        st_store(status + tp, st_pack(ST_PRE, epoch, (off + kp) | (tup_o(agg_p, sel) << 31)));
                }
                if (lane == 0) s_off[round & 1u] = off;
            }
            lds_barrier();
            if (tid == 0 && tn < ntiles) grab = atomicAdd(tile_ctr, 1u);
            const uint32_t tile_off = tp < ntiles ? s_off[round & 1u] : 0u;
            store_tile<TPB, TILE>(out, s_stage + (cur ^ 1u) * SST, tile_off, tp < ntiles ? kp : 0u);
            if (tp == ntiles - 1 && tid == 0) finish_iteration(ctl, lengths, it, tile_off + kp);
            if (t < ntiles) {
                tp = t;
                kp = tile_kept;
                agg_p = tile_agg;
                done_p = dep || t == 0;
                off_p = off_t;
                cur ^= 1u;
            } else {
                tp = ntiles;
            }
            t = tn;
        }
    }
    finish_counts<TPB, LT>(tab, gt, ctl, sw, theta);
}

}  // namespace bpek
