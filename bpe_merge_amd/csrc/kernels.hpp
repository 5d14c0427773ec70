// Device code of the BPE training iteration for gfx950 (CDNA4, wave64).
//
// Steps of one training iteration, after the page "bpe - GPU BPE Tokenizer
// Pipeline (Egitim + Cikarim)" (llm.istanbul/learn/tr/13_bpe): word-boundary
// tagging ("Ne Yapar? 1", once), pair counting in two levels, first in a
// workgroup-local table and then in one global table ("Ne Yapar? 2"), a
// deterministic maximum (pipeline list at the head of the page), then merge
// + prefix-scan compaction of the symbol array ("Ne Yapar? 3").
//
// How the work is laid out here (not the page's WGSL dispatch plan):
//   k_tag_count  bytes -> 16-bit symbols (the word starts decide which
//                pairs count; they are not stored: a word start is a change
//                of class between neighbours), and the pair counts of
//                iteration 0 in the global table (LDS aggregation first).
//   k_merge      (merge.hpp) one persistent pass per iteration that selects
//                the merge (from a candidate list, or by a sweep of the
//                global table when the list cannot vouch for the maximum),
//                applies it, compacts with a single-pass decoupled look-back
//                scan, and updates the global table by the pairs the merge
//                destroyed and created: the symbols are read once and
//                written once per iteration, with no host round trip.
// The global table always holds the exact pair counts of the current
// sequence, as a full recount would give them. A merge changes only the
// pairs at its own sites: every other adjacency of the new sequence is an
// adjacency of the old one, and the other way round. So the recount the
// page does every iteration is replaced by subtracting the old pairs that
// touch a changed position and adding the new pairs that touch a new
// symbol, which costs work in proportion to the merge's occurrences rather
// than to the sequence length.
// All arithmetic is integer; results do not depend on scheduling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpek {

constexpr uint32_t WS = 0x10000u;        // word-start bit of a token at the boundary
constexpr uint32_t IDM = 0xFFFFu;        // id field of a token
constexpr uint32_t N_CLASSES = 5;        // byte classes (byte_class)
constexpr uint32_t CLASS_WORDS = 2048;   // words of a class's bit mask: one bit per 16-bit id
constexpr uint32_t EMPTY = 0xFFFFFFFFu;  // empty key (the pair 65535,65535 is never counted)
constexpr uint32_t BASE = 256u;

constexpr uint32_t ERR_TABLE = 1u;  // the global pair table is full
// A bounded wait of the merge pass exceeded its bound: the look-back of the
// scan (for a lower tile's status) or a table sweep (for the maximum of all
// chunks). Both wait only for work a workgroup that is already running has
// taken on, so only a fault can make them fail.
constexpr uint32_t ERR_SPIN = 2u;
constexpr uint32_t ERR_CLASS = 16u;  // a merge names an id with no class (ids below X always have one)

constexpr uint32_t LDS_PROBES = 16;        // buckets probed before giving up on an LDS table
constexpr uint32_t GT_PROBES = 4096;       // slots probed before giving up on the global table
constexpr uint32_t SPIN_LIMIT = 1u << 22;  // polls of one wait before giving up

// Device-resident control block; one per training state.
struct alignas(64) Ctl {
    uint32_t k;           // merges chosen so far
    uint32_t m;           // merges applied so far (m == k between iterations)
    uint32_t done;        // 1 once no pair is left (or after a device error)
    uint32_t err;         // ERR_* bits
    uint32_t n[2];        // symbol counts; n[m & 1] is the current one
    uint32_t L, R, X;     // merge being applied: (L, R) -> X
    uint32_t tile_ctr[2];  // tiles handed out by k_merge, per iteration parity (cleared one iteration ahead)
    uint32_t used;        // claimed slots of the global table
};

// Selection state, carried from one iteration's merge pass to the next.
//
// The merge of an iteration is the maximum over the global table of the
// packed value count << 32 | ~key (highest count, ties to the smallest
// (left, right), whatever the order of evaluation). A candidate list holds
// every slot whose count is at least a threshold theta; whenever the
// largest count on the list reaches theta, no slot off the list can beat
// it and the maximum is taken over the list alone. The list stays complete
// because the count of an existing pair only falls (every new adjacency
// involves the newest id), and a new pair whose count the merge pass lifts
// across theta is appended by the add that does it. When the list's
// maximum falls below theta (or the list overflowed), the iteration sweeps
// the whole table and rebuilds the list with theta = max - (max >> shift),
// the shift adapted to the list sizes seen.
//
// The workgroup that draws the pass's first ticket from the tile counter
// (so it is running; ticket 0 is this job, not a tile) selects the merge:
// the maximum over the list, or a mark that the pass sweeps, or the pair a
// replay lists, before it issues any load of its own tile, while the other
// workgroups load theirs. It publishes the result to PUB_COPIES copies
// (value, then epoch = iteration + 1), one read by each group of
// workgroups, so that their polls do not pile up on one address. No workgroup changes the
// table before it has read the publication, which follows every read of the
// selection, and a workgroup that starts late reads only the publication:
// no wait in the pass is on a workgroup that has not started, so the pass
// needs no co-residency of its grid. A sweep is split into chunks of the
// table that running workgroups claim from a counter; the workgroup that
// finishes the last chunk of the maximum publishes it (spub), and the
// candidates are collected from chunks claimed the same way. Counters are
// kept per iteration parity and cleared one iteration ahead.
constexpr uint32_t CAND_MAX = 16384;
constexpr uint32_t CAND_TARGET = 2048;  // list size the shift steers towards
constexpr uint32_t SHIFT_DEFAULT = 3;   // theta = 7/8 of the maximum
constexpr uint32_t SHIFT_MAX = 16;
constexpr uint32_t SWEEP_CHUNK = 16384;           // table slots per sweep chunk
constexpr unsigned long long SEL_SWEEP = ~0ull;  // the pass sweeps (never a packed maximum)
constexpr uint32_t PUB_COPIES = 256;              // copies of a published merge
struct Sweep {
    unsigned long long pub[2][PUB_COPIES];  // per parity: the pass's merge (packed maximum,
                                            // or SEL_SWEEP), published by tile 0's workgroup
    uint32_t pub_epoch[2][PUB_COPIES];      // per parity: 1 + the iteration pub holds
    unsigned long long force_val;  // a replayed iteration's merge, packed
    uint32_t force_epoch;          // 1 + the iteration force_val is for (0: none)
    uint32_t pad0;
    unsigned long long smax[2];  // per parity: maximum over the sweep's finished chunks
    unsigned long long spub[2];  // per parity: the sweep's maximum, published
    uint32_t spub_epoch[2];      // per parity: 1 + the iteration whose maximum spub holds
    uint32_t c1[2];              // per parity: chunks claimed for the maximum
    uint32_t c1done[2];          // per parity: chunks whose maximum is in smax
    uint32_t c2[2];              // per parity: chunks claimed for the candidates
    uint32_t theta;              // the list's threshold
    uint32_t shift;              // for the next sweep (0: none yet)
    uint32_t cand_n;             // entries appended (above CAND_MAX: overflowed)
    uint32_t cand_ok;            // the list holds every slot with count >= theta
    uint32_t sweeps;             // iterations that swept the table
    uint32_t cand[CAND_MAX];     // slot indexes
};

// Global pair table: open addressing with linear probing over 64-bit slots
// holding count << 32 | key. An empty slot holds key EMPTY with count 0; a
// claimed slot keeps its key for good (a pair whose count falls to zero
// never occurs again: every new adjacency involves the newest id), so probe
// chains are never broken.
struct GTable {
    unsigned long long* slot;
    uint32_t mask;   // slots - 1 (a power of two)
    uint32_t limit;  // claims allowed before the table counts as full
};
constexpr unsigned long long GT_EMPTY = 0xFFFFFFFFull;

// Workgroup barrier that orders LDS only. __syncthreads() also orders the
// workgroup's global memory accesses, which on gfx9 means waiting for every
// outstanding global load and store of the wave (one vmcnt counter for
// both) at every barrier. Waves of these kernels share data only through
// LDS, so their global loads and stores stay in flight across barriers.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Agent-coherent load and store (relaxed atomics at agent scope: sc1 on
// gfx950), for state that workgroups on other XCDs change during a pass:
// an sc1 store is visible on every XCD once it has completed, and an sc1
// load never returns a stale line of this XCD's L2.
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Murmur3 32-bit finalizer: spreads packed pair keys; the low bits pick an
// LDS bucket, the top 8 bits the partition.
__host__ __device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// Character class: 4 newline, 2 space, 1 ASCII digit, 0 letter (ASCII
// letters and every byte >= 0x80, so UTF-8 letters stay letters), 3 other.
__device__ __forceinline__ uint32_t byte_class(uint32_t b) {
    uint32_t c = 3u;
    c = ((b | 0x20u) - 0x61u < 26u) ? 0u : c;
    c = (b >= 0x80u) ? 0u : c;
    c = (b - 0x30u < 10u) ? 1u : c;
    c = (b == 0x20u) ? 2u : c;
    c = (b == 0x0Au) ? 4u : c;
    return c;
}

__device__ __forceinline__ uint32_t pair_key(uint32_t left_sym, uint32_t right_sym) {
    return ((left_sym & IDM) << 16) | (right_sym & IDM);
}

__device__ __forceinline__ void fail_table(Ctl* ctl) {
    atomicOr(&ctl->err, ERR_TABLE);
    atomicExch(&ctl->done, 1u);
}

// The slot of key in the global table, claimed if the key is new; NO_SLOT
// (and ERR_TABLE) if the table is full.
constexpr uint32_t NO_SLOT = 0xFFFFFFFFu;
__device__ __forceinline__ uint32_t gt_slot(const GTable& gt, uint32_t key, Ctl* ctl) {
    uint32_t h = mix32(key) & gt.mask;
    for (uint32_t p = 0; p < GT_PROBES; ++p) {
        unsigned long long* slot = gt.slot + h;
        uint32_t cur = (uint32_t)__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cur == EMPTY) {
            const unsigned long long old = atomicCAS(slot, GT_EMPTY, (unsigned long long)key);
            if (old == GT_EMPTY) {
                if (atomicAdd(&ctl->used, 1u) >= gt.limit) fail_table(ctl);
                cur = key;
            } else {
                cur = (uint32_t)old;
            }
        }
        if (cur == key) return h;
        h = (h + 1) & gt.mask;
    }
    fail_table(ctl);
    return NO_SLOT;
}

// Add delta (two's complement, so negative deltas work) to the count of key
// in the global table, claiming a slot for a new key. Within one launch a
// key only ever receives deltas of one sign, so no count goes below zero.
__device__ __forceinline__ void gt_add(const GTable& gt, uint32_t key, uint32_t delta, Ctl* ctl) {
    const uint32_t h = gt_slot(gt, key, ctl);
    if (h != NO_SLOT) atomicAdd(gt.slot + h, (unsigned long long)(long long)(int)delta << 32);
}

// Append a slot to the candidate list (its entry is dropped past CAND_MAX;
// the overflow shows in cand_n).
__device__ __forceinline__ void cand_append(Sweep* sw, uint32_t slot) {
    const uint32_t i = atomicAdd(&sw->cand_n, 1u);
    if (i < CAND_MAX) __hip_atomic_store(&sw->cand[i], slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// cand_append for the slots slot0 + k * stride (k < N) whose bit k of take
// is set, for every lane of a wave at once, with one counter atomic per
// wave (a sweep over a table of many equal small counts appends tens of
// thousands of slots, and the list's counter is one address). Called by
// all 64 lanes of the wave.
template <int N>
__device__ __forceinline__ void cand_append_wave(Sweep* sw, uint32_t slot0, uint32_t stride, uint32_t take) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t mine = (uint32_t)__popc(take);
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
        if (lane >= (uint32_t)o) incl += y;
    }
    const uint32_t total = (uint32_t)__shfl((int)incl, 63);
    if (total == 0u) return;
    uint32_t base = 0u;
    if (lane == 63u) base = atomicAdd(&sw->cand_n, total);
    base = (uint32_t)__shfl((int)base, 63) + incl - mine;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        if ((take >> k) & 1u) {
            if (base < CAND_MAX)
                __hip_atomic_store(&sw->cand[base], slot0 + (uint32_t)k * stride, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            ++base;
        }
    }
}

// gt_add for the merge pass: an increase that lifts the count from below
// theta to theta or more appends the slot to the candidate list.
__device__ __forceinline__ void gt_add_sel(const GTable& gt, uint32_t key, uint32_t delta, Ctl* ctl, Sweep* sw,
                                           uint32_t theta) {
    const uint32_t h = gt_slot(gt, key, ctl);
    if (h == NO_SLOT) return;
    const unsigned long long d = (unsigned long long)(long long)(int)delta << 32;
    if ((int)delta > 0) {
        const uint32_t old = (uint32_t)(atomicAdd(gt.slot + h, d) >> 32);
        if (old < theta && old + delta >= theta) cand_append(sw, h);
    } else {
        atomicAdd(gt.slot + h, d);
    }
}

// ---------------------------------------------------------------- LDS table
// LT slots in buckets of 4, read with one 16-byte LDS load, so a key sits at
// its first probe unless its whole home bucket was taken first. Plain data
// (no constructor) so that it can live in __shared__.
template <int LT>
struct LdsTable {
    static_assert(LT % 4 == 0 && (LT & (LT - 1)) == 0, "LT: power of two, buckets of 4");
    static constexpr uint32_t NB = LT / 4;
    alignas(16) uint32_t keys[LT];
    uint32_t cnts[LT];
    uint32_t used;  // claimed slots
    uint32_t qn;    // queued keys

    // every thread of the block; a barrier must follow before use
    __device__ __forceinline__ void clear(int tpb) {
        for (int i = threadIdx.x; i < LT; i += tpb) {
            keys[i] = EMPTY;
            cnts[i] = 0u;
        }
        if (threadIdx.x == 0) {
            used = 0u;
            qn = 0u;
        }
    }

    // every thread of the block: clear the first nslots slots only
    __device__ __forceinline__ void clear_first(uint32_t nslots, int tpb) {
        for (uint32_t i = threadIdx.x; i < nslots; i += tpb) {
            keys[i] = EMPTY;
            cnts[i] = 0u;
        }
        if (threadIdx.x == 0) {
            used = 0u;
            qn = 0u;
        }
    }

    // full insert: home bucket, then further buckets; false if none has room
    // (nbmask + 1 buckets in use, at most NB)
    __device__ __forceinline__ bool insert(uint32_t key, uint32_t c, uint32_t nbmask = NB - 1) {
        uint32_t b = mix32(key) & nbmask;
        for (uint32_t p = 1; p <= LDS_PROBES; ++p) {
            for (uint32_t s = 0; s < 4; ++s) {
                uint32_t* slot = keys + 4 * b + s;
                uint32_t cur = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (cur == EMPTY) {
                    cur = atomicCAS(slot, EMPTY, key);
                    if (cur == EMPTY) {
                        atomicAdd(&used, 1u);
                        cur = key;
                    }
                }
                if (cur == key) {
                    atomicAdd(cnts + 4 * b + s, c);
                    return true;
                }
            }
            b = (b + p) & nbmask;
        }
        return false;
    }

    // Count one per non-EMPTY key k[j], in two phases per 8 keys per thread:
    //   1. each lane reads the home buckets of its keys (4 at a time, all
    //      loads issued before any is examined) and adds to keys it finds;
    //   2. keys not found are queued in LDS and, after a barrier, inserted by
    //      the whole block, one queued key per lane.
    // A set bit j of fold means key j equals the next non-EMPTY key, whose
    // add carries it (a run of one key costs one add). qk/qc: LDS scratch of
    // qcap >= 8 * tpb entries each. Every thread of the block calls this.
    template <int V>
    __device__ __forceinline__ void count(const uint32_t (&k)[V], uint32_t fold, uint32_t* qk, uint32_t* qc,
                                          uint32_t qcap, int tpb, const GTable& gt, Ctl* ctl) {
        constexpr int G = 4;
        static_assert(V % (2 * G) == 0, "keys come in groups of 8");
        uint32_t carry = 0;
#pragma unroll
        for (int g = 0; g < V; g += G) {
            uint32_t bk[G];
            uint4 kv[G];
#pragma unroll
            for (int j = 0; j < G; ++j) bk[j] = mix32(k[g + j]) & (NB - 1);
#pragma unroll
            for (int j = 0; j < G; ++j) kv[j] = reinterpret_cast<const uint4*>(keys)[bk[j]];
            uint32_t miss = 0, cnt[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                cnt[j] = 0;
                const uint32_t key = k[g + j];
                if (key != EMPTY) {
                    if ((fold >> (g + j)) & 1u) {
                        ++carry;
                    } else {
                        cnt[j] = carry + 1;
                        carry = 0;
                        const uint32_t s = kv[j].x == key ? 0u : kv[j].y == key ? 1u : kv[j].z == key ? 2u
                                         : kv[j].w == key ? 3u : 4u;
                        if (s < 4u) atomicAdd(cnts + 4 * bk[j] + s, cnt[j]);
                        else miss |= 1u << j;
                    }
                }
            }
            if (miss) {
                uint32_t q = atomicAdd(&qn, (uint32_t)__popc(miss));
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    if ((miss >> j) & 1u) {
                        if (q < qcap) {
                            qk[q] = k[g + j];
                            qc[q] = cnt[j];
                        } else {
                            gt_add(gt, k[g + j], cnt[j], ctl);
                        }
                        ++q;
                    }
                }
            }
            if ((g / G) % 2 == 0) continue;  // drain after every 8 keys per thread
            lds_barrier();
            const uint32_t nq = min(qn, qcap);
            if (nq) {  // uniform: read after the barrier
                for (uint32_t i = threadIdx.x; i < nq; i += tpb)
                    if (!insert(qk[i], qc[i])) gt_add(gt, qk[i], qc[i], ctl);
                lds_barrier();
                if (threadIdx.x == 0) qn = 0u;
                lds_barrier();
            }
        }
    }
};

// Add every nonzero LDS count to the global table and clear the LDS table.
// Every thread of the block, after a barrier that follows the last change
// to tab; a barrier must follow before tab is used again.
template <int LT>
__device__ __forceinline__ void flush_table(LdsTable<LT>& tab, int tpb, const GTable& gt, Ctl* ctl) {
    for (int i = threadIdx.x; i < LT; i += tpb) {
        const uint32_t key = tab.keys[i], c = tab.cnts[i];
        if (key != EMPTY && c != 0u) gt_add(gt, key, c, ctl);
        tab.keys[i] = EMPTY;
        tab.cnts[i] = 0u;
    }
    if (threadIdx.x == 0) {
        tab.used = 0u;
        tab.qn = 0u;
    }
}

// ---------------------------------------------------------------- small kernels

__global__ void k_init_ctl(Ctl* ctl, uint32_t n, uint32_t* lengths) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        ctl->k = 0; ctl->m = 0; ctl->done = 0; ctl->err = 0;
        ctl->n[0] = n; ctl->n[1] = 0;
        ctl->L = 0; ctl->R = 0; ctl->X = 0;
        ctl->tile_ctr[0] = 0; ctl->tile_ctr[1] = 0; ctl->used = 0;
        lengths[0] = n;
    }
}

// The class of every id (a byte: its byte class; a merged id: written by
// the pass that creates it) and, per class, the bit mask of its ids.
// Launched over at least 65,536 threads.
__global__ void k_init_classes(uint8_t* __restrict__ cls, uint32_t* __restrict__ cmask) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 65536u) cls[i] = i < BASE ? (uint8_t)byte_class(i) : (uint8_t)0xFFu;
    if (i < N_CLASSES * CLASS_WORDS) {
        const uint32_t c = i / CLASS_WORDS, wd = i % CLASS_WORDS;
        uint32_t m = 0;
        if (wd < BASE / 32u)
            for (uint32_t b = 0; b < 32u; ++b) m |= (byte_class(32u * wd + b) == c ? 1u : 0u) << b;
        cmask[i] = m;
    }
}

// Tokens in the boundary's format from the 16-bit ids sym[begin ..
// begin + count): id | WS on the first token of each word, that is at
// position 0 and wherever the class changes from the token before (words
// are maximal runs of one class, and every token lies inside one).
__global__ void k_expand(const uint16_t* __restrict__ sym, uint32_t begin, uint32_t count,
                         const uint8_t* __restrict__ cls, uint32_t* __restrict__ out) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x) {
        const uint32_t p = begin + i, v = sym[p];
        const bool start = p == 0u || cls[v] != cls[sym[p - 1u]];
        out[i] = v | (start ? WS : 0u);
    }
}

// fill a buffer of 64-bit words with one value (status words, table slots)
__global__ void k_fill64(unsigned long long* p, size_t count, unsigned long long v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ---------------------------------------------------------------- tag + count (iteration 0)
// Blocks take chunks of TPB * 16 bytes in turn; a thread covers 16
// consecutive bytes (one 16-byte load when the input is aligned, two
// 16-byte stores of 16-bit symbols). The word starts decide which pairs
// are counted; the symbol array holds the ids alone (a word start is a
// change of class between neighbours). The chunk loop is uniform over the block so
// that the LDS table can be flushed between chunks.

template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_tag_count(const uint8_t* __restrict__ bytes, uint32_t n,
                                                   uint16_t* __restrict__ sym, GTable gt, Ctl* ctl) {
    constexpr uint32_t CH = TPB * 16;
    constexpr uint32_t QCAP = TPB * 8;
    __shared__ LdsTable<LT> tab;
    __shared__ uint32_t s_qk[QCAP], s_qc[QCAP];
    tab.clear(TPB);
    lds_barrier();
    const bool aligned = ((uintptr_t)bytes & 15u) == 0;
    const uint32_t nchunks = (n + CH - 1) / CH;
    for (uint32_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
        const size_t base = (size_t)ch * CH + threadIdx.x * 16;
        uint32_t b[16];
        if (aligned && base + 16 <= n) {
            uint4 v = *reinterpret_cast<const uint4*>(bytes + base);
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 16; ++j) b[j] = (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) b[j] = (base + j < n) ? bytes[base + j] : 0u;
        }
        const uint32_t prev = (base && base - 1 < n) ? bytes[base - 1] : 0u;
        uint32_t pcls = byte_class(prev);
        uint32_t s[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t c = byte_class(b[j]);
            bool start = (base + j == 0) || (c != pcls);
            s[j] = b[j] | (start ? WS : 0u);
            pcls = c;
        }
        if (base + 16 <= n) {
            uint4* o = reinterpret_cast<uint4*>(sym + base);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                o[q] = make_uint4(b[8 * q] | (b[8 * q + 1] << 16), b[8 * q + 2] | (b[8 * q + 3] << 16),
                                  b[8 * q + 4] | (b[8 * q + 5] << 16), b[8 * q + 6] | (b[8 * q + 7] << 16));
        } else {
            for (int j = 0; j < 16; ++j)
                if (base + j < n) sym[base + j] = (uint16_t)b[j];
        }
        // pairs whose right symbol starts no word; equal keys folded into one add
        uint32_t keys[16];
        uint32_t fold = 0, lastkey = EMPTY, prevj = 0, left = prev;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            keys[j] = EMPTY;
            if (base + j < n && !(s[j] & WS)) {
                const uint32_t key = pair_key(left, b[j]);
                if (key == lastkey) fold |= 1u << prevj;
                lastkey = key;
                keys[j] = key;
                prevj = j;
            }
            left = b[j];
        }
        tab.template count<16>(keys, fold, s_qk, s_qc, QCAP, TPB, gt, ctl);
        if (2u * tab.used > (uint32_t)LT) {  // uniform: read after the barrier that ends count
            flush_table(tab, TPB, gt, ctl);
            lds_barrier();
        }
    }
    lds_barrier();
    flush_table(tab, TPB, gt, ctl);
}

// ---------------------------------------------------------------- maximum
// Packed candidates (count << 32 | ~key) of table slots, compared as
// unsigned 64-bit values: highest count, ties to the smallest key.

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        unsigned lo = __shfl_xor((unsigned)(v & 0xFFFFFFFFull), off);
        unsigned hi = __shfl_xor((unsigned)(v >> 32), off);
        unsigned long long o = ((unsigned long long)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// slot value -> packed candidate (0 for an empty or zero-count slot)
__device__ __forceinline__ unsigned long long candidate(unsigned long long v) {
    return (v >> 32) ? (v ^ 0xFFFFFFFFull) : 0ull;
}

// ---------------------------------------------------------------- replay
// A replayed iteration m merges the listed pair pairs[2m], pairs[2m+1] (a
// learned merge list applied in order, "Nedir bu ya?"), not the table's
// maximum; its count is looked up in the table. A pair that does not occur
// still counts as a merge: count 0, nothing changes, id 256 + m is used up.
// The packed value is never 0 or SEL_SWEEP (~key != 0 for 16-bit ids), and
// the candidate list stays valid through the iteration.

__device__ __forceinline__ uint32_t gt_count(const GTable& gt, uint32_t key) {
    uint32_t h = mix32(key) & gt.mask;
    for (uint32_t p = 0; p < GT_PROBES; ++p) {
        const unsigned long long v =
            __hip_atomic_load(gt.slot + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t cur = (uint32_t)v;
        if (cur == key) return (uint32_t)(v >> 32);
        if (cur == EMPTY) return 0u;
        h = (h + 1) & gt.mask;
    }
    return 0u;
}

// Launched before the merge pass of a replayed iteration: its merge is the
// listed pair, not the table's maximum.
__global__ void k_force(Ctl* ctl, GTable gt, Sweep* sw, const uint32_t* __restrict__ pairs) {
    if (blockIdx.x != 0 || threadIdx.x != 0 || ctl->done) return;
    const uint32_t m = ctl->m;
    const uint32_t key = (pairs[2 * m] << 16) | pairs[2 * m + 1];
    sw->force_val = ((unsigned long long)gt_count(gt, key) << 32) | (uint32_t)~key;
    sw->force_epoch = m + 1u;
}

}  // namespace bpek
