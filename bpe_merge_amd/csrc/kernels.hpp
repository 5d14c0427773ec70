// Device code of the BPE training iteration for gfx950 (CDNA4, wave64).
//
// Steps of one training iteration, after the page "bpe - GPU BPE Tokenizer
// Pipeline (Egitim + Cikarim)" (llm.istanbul/learn/tr/13_bpe): word-boundary
// tagging ("Ne Yapar? 1", once), pair counting through a workgroup-local
// table flushed into a global table ("Ne Yapar? 2"), a deterministic maximum
// (pipeline list at the head of the page), then merge + prefix-scan
// compaction of the symbol array ("Ne Yapar? 3").
//
// How the work is laid out here (not the page's WGSL dispatch plan):
//   k_tag_count  bytes -> tagged uint32 symbols, and the pair counts of
//                iteration 0 (LDS hash, flushed once per workgroup).
//   k_find_max   one sweep of the global table: packed (count, ~key) u64
//                maximum, slot reset, and, in the last workgroup to finish,
//                the choice of the merge (device-resident, no host sync).
//   k_merge      one persistent pass over the symbols that applies the merge
//                (run-length parity for runs of identical pairs), compacts
//                with a single-pass decoupled look-back scan, and counts the
//                pairs of the *new* sequence for the next iteration, so the
//                symbols are read once and written once per iteration.
// All arithmetic is integer; results do not depend on scheduling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpek {

constexpr uint32_t WS = 0x10000u;     // word-start bit of a symbol
constexpr uint32_t IDM = 0xFFFFu;     // id field of a symbol
constexpr uint32_t EMPTY = 0xFFFFFFFFu;  // empty slot key (pair 65535,65535 is never counted)
constexpr uint32_t BASE = 256u;

constexpr uint32_t ERR_TABLE = 1u;    // a key found no slot within the probe limit
constexpr uint32_t ERR_SPIN = 2u;     // a look-back wait exceeded its bound

constexpr uint32_t GLOBAL_PROBES = 512;
constexpr uint32_t LDS_PROBES = 16;
constexpr uint32_t SPIN_LIMIT = 1u << 22;

// Device-resident control block; one per training state.
struct alignas(64) Ctl {
    uint32_t k;           // merges chosen so far
    uint32_t m;           // merges applied so far (m == k between iterations)
    uint32_t limit;       // iterations allowed in total
    uint32_t done;        // 1 once no pair is left (or after a device error)
    uint32_t err;         // ERR_* bits
    uint32_t n[2];        // symbol counts; n[m & 1] is the current one
    uint32_t L, R, X;     // merge being applied: (L, R) -> X
    uint32_t tile_ctr;    // dynamic tile counter of k_merge
    uint32_t sweep_done;  // k_find_max workgroups finished
    uint32_t pad[3];
    unsigned long long best;  // packed argmax of the current sweep
};

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Murmur3 32-bit finalizer: spreads packed pair keys over table slots.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
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

// ---------------------------------------------------------------- tables
// Global table: T slots of {uint32 key, uint32 count}, open addressing with
// triangular probing (visits every slot of a power-of-two table).

__device__ __forceinline__ void global_add(uint32_t* table, uint32_t mask, uint32_t key, uint32_t c,
                                           Ctl* ctl) {
    uint32_t h = mix32(key) & mask;
    for (uint32_t p = 1; p <= GLOBAL_PROBES; ++p) {
        uint32_t* slot = table + 2u * h;
        uint32_t cur = ld_relaxed(slot);
        if (cur == EMPTY) {
            cur = atomicCAS(slot, EMPTY, key);
            if (cur == EMPTY) cur = key;
        }
        if (cur == key) {
            atomicAdd(slot + 1, c);
            return;
        }
        h = (h + p) & mask;
    }
    atomicOr(&ctl->err, ERR_TABLE);
    atomicExch(&ctl->done, 1u);
}

// Workgroup table in LDS: LT slots; a key that finds no slot within
// LDS_PROBES goes straight to the global table.
template <int LT>
__device__ __forceinline__ void lds_add(uint32_t* keys, uint32_t* cnts, uint32_t key, uint32_t c,
                                        uint32_t* table, uint32_t mask, Ctl* ctl) {
    uint32_t h = mix32(key) & (LT - 1);
    for (uint32_t p = 1; p <= LDS_PROBES; ++p) {
        uint32_t cur = __hip_atomic_load(keys + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (cur == EMPTY) {
            cur = atomicCAS(keys + h, EMPTY, key);
            if (cur == EMPTY) cur = key;
        }
        if (cur == key) {
            atomicAdd(cnts + h, c);
            return;
        }
        h = (h + p) & (LT - 1);
    }
    global_add(table, mask, key, c, ctl);
}

template <int TPB, int LT>
__device__ __forceinline__ void lds_table_clear(uint32_t* keys, uint32_t* cnts) {
    for (int i = threadIdx.x; i < LT; i += TPB) {
        keys[i] = EMPTY;
        cnts[i] = 0u;
    }
}

template <int TPB, int LT>
__device__ __forceinline__ void lds_table_flush(const uint32_t* keys, const uint32_t* cnts,
                                                uint32_t* table, uint32_t mask, Ctl* ctl) {
    for (int i = threadIdx.x; i < LT; i += TPB) {
        uint32_t k = keys[i];
        if (k != EMPTY) global_add(table, mask, k, cnts[i], ctl);
    }
}

// Run-length pre-aggregation of one thread's counted pairs before the LDS
// table: consecutive equal keys (long runs of one byte) become one add.
template <int LT>
struct PairCounter {
    uint32_t key = EMPTY;
    uint32_t cnt = 0;
    __device__ __forceinline__ void add(uint32_t k, uint32_t* keys, uint32_t* cnts, uint32_t* table,
                                        uint32_t mask, Ctl* ctl) {
        if (k == key) {
            ++cnt;
        } else {
            if (cnt) lds_add<LT>(keys, cnts, key, cnt, table, mask, ctl);
            key = k;
            cnt = 1;
        }
    }
    __device__ __forceinline__ void finish(uint32_t* keys, uint32_t* cnts, uint32_t* table,
                                           uint32_t mask, Ctl* ctl) {
        if (cnt) lds_add<LT>(keys, cnts, key, cnt, table, mask, ctl);
        cnt = 0;
        key = EMPTY;
    }
};

// ---------------------------------------------------------------- small kernels

__global__ void k_init_ctl(Ctl* ctl, uint32_t n, uint32_t* lengths) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        ctl->k = 0; ctl->m = 0; ctl->limit = 0; ctl->done = 0; ctl->err = 0;
        ctl->n[0] = n; ctl->n[1] = 0;
        ctl->L = 0; ctl->R = 0; ctl->X = 0;
        ctl->tile_ctr = 0; ctl->sweep_done = 0;
        ctl->best = 0ull;
        lengths[0] = n;
    }
}

__global__ void k_set_limit(Ctl* ctl, uint32_t limit) {
    if (threadIdx.x == 0 && blockIdx.x == 0) ctl->limit = limit;
}

// fill a buffer of 64-bit words with one value (table reset, status reset)
__global__ void k_fill64(unsigned long long* p, size_t count, unsigned long long v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ---------------------------------------------------------------- tag + count (iteration 0)
// Each thread step covers 16 consecutive bytes: one 16-byte load when the
// input is aligned, four 16-byte stores of symbols.

template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_tag_count(const uint8_t* __restrict__ bytes, uint32_t n,
                                                   uint32_t* __restrict__ sym, uint32_t* table,
                                                   uint32_t mask, Ctl* ctl) {
    __shared__ uint32_t s_keys[LT];
    __shared__ uint32_t s_cnts[LT];
    lds_table_clear<TPB, LT>(s_keys, s_cnts);
    __syncthreads();
    PairCounter<LT> pc;
    const bool aligned = ((uintptr_t)bytes & 15u) == 0;
    const size_t stride = (size_t)gridDim.x * TPB * 16;
    for (size_t base = ((size_t)blockIdx.x * TPB + threadIdx.x) * 16; base < n; base += stride) {
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
        uint32_t prev = base ? bytes[base - 1] : 0u;
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
            for (int q = 0; q < 4; ++q) o[q] = make_uint4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
        } else {
            for (int j = 0; j < 16; ++j)
                if (base + j < n) sym[base + j] = s[j];
        }
        uint32_t left = prev;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (base + j < n && !(s[j] & WS)) pc.add(pair_key(left, b[j]), s_keys, s_cnts, table, mask, ctl);
            left = b[j];
        }
    }
    pc.finish(s_keys, s_cnts, table, mask, ctl);
    __syncthreads();
    lds_table_flush<TPB, LT>(s_keys, s_cnts, table, mask, ctl);
}

// ---------------------------------------------------------------- find max
// Packed value: count in the high word, ~key in the low word, so the u64
// maximum is the highest count with ties to the smallest (left, right).

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

template <int TPB>
__global__ __launch_bounds__(TPB) void k_find_max(Ctl* ctl, uint32_t* table, uint32_t n_slots,
                                                  uint32_t* merges) {
    __shared__ unsigned long long s_best[TPB / 64];
    __shared__ uint32_t s_last;
    const uint32_t done = ld_relaxed(&ctl->done);
    const uint32_t k = ld_relaxed(&ctl->k);
    const uint32_t m = ld_relaxed(&ctl->m);
    const uint32_t limit = ld_relaxed(&ctl->limit);
    if (done || k != m || k >= limit) return;  // uniform over the grid

    unsigned long long best = 0ull;
    uint4* t4 = reinterpret_cast<uint4*>(table);
    const uint32_t n4 = n_slots / 2;
    for (uint32_t i = blockIdx.x * TPB + threadIdx.x; i < n4; i += gridDim.x * TPB) {
        uint4 v = t4[i];
        if (v.x != EMPTY) {
            unsigned long long p = ((unsigned long long)v.y << 32) | (uint32_t)~v.x;
            best = p > best ? p : best;
        }
        if (v.z != EMPTY) {
            unsigned long long p = ((unsigned long long)v.w << 32) | (uint32_t)~v.z;
            best = p > best ? p : best;
        }
        if (v.x != EMPTY || v.z != EMPTY) t4[i] = make_uint4(EMPTY, 0u, EMPTY, 0u);
    }
    best = wave_max_u64(best);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) s_best[w] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long b = 0ull;
        for (int i = 0; i < TPB / 64; ++i) b = s_best[i] > b ? s_best[i] : b;
        if (b) atomicMax(&ctl->best, b);
        __threadfence();
        uint32_t prev = atomicAdd(&ctl->sweep_done, 1u);
        s_last = (prev == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last && threadIdx.x == 0) {
        __threadfence();
        unsigned long long b = __hip_atomic_load(&ctl->best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (b == 0ull) {
            ctl->done = 1u;  // no countable pair is left
        } else {
            uint32_t key = ~(uint32_t)(b & 0xFFFFFFFFull);
            uint32_t cnt = (uint32_t)(b >> 32);
            merges[3 * k + 0] = key >> 16;
            merges[3 * k + 1] = key & IDM;
            merges[3 * k + 2] = cnt;
            ctl->L = key >> 16;
            ctl->R = key & IDM;
            ctl->X = BASE + k;
            ctl->tile_ctr = 0u;
            ctl->k = k + 1;
        }
        ctl->best = 0ull;
        ctl->sweep_done = 0u;
    }
}

// ---------------------------------------------------------------- merge + compact + count
//
// Selection: an occurrence at position i (right symbol of the pair) is
//   occ_i = no tag on s_i, id(s_{i-1}) == L, id(s_i) == R
// and the left-to-right scan merges it iff sel_i = occ_i and not sel_{i-1}.
// A segment's effect on this recurrence and on the number of symbols it
// keeps is the 4-tuple below, composed associatively across lanes, waves
// and tiles:
//   c0  symbols kept when the segment is entered with sel = 0
//   d   extra symbol kept when entered with sel = 1 (0 or 1: only the
//       leading chain of occurrences depends on the entry state)
//   o0, o1  sel of the segment's last position for entry sel = 0 / 1
// Packed into 32 bits: c0 in bits 0-23, d bit 24, o0 bit 25, o1 bit 26.

__device__ __forceinline__ uint32_t tup_make(uint32_t c0, uint32_t d, uint32_t o0, uint32_t o1) {
    return c0 | (d << 24) | (o0 << 25) | (o1 << 26);
}
constexpr uint32_t TUP_ID = 1u << 26;  // empty segment: keeps nothing, passes sel through

// segment a followed by segment b
__device__ __forceinline__ uint32_t tup_then(uint32_t a, uint32_t b) {
    const uint32_t ac0 = a & 0xFFFFFFu, ad = (a >> 24) & 1u, ao0 = (a >> 25) & 1u, ao1 = (a >> 26) & 1u;
    const uint32_t bc0 = b & 0xFFFFFFu, bd = (b >> 24) & 1u, bo0 = (b >> 25) & 1u, bo1 = (b >> 26) & 1u;
    const uint32_t c0 = ac0 + bc0 + (ao0 & bd);
    const uint32_t c1 = ac0 + ad + bc0 + (ao1 & bd);
    const uint32_t o0 = ao0 ? bo1 : bo0;
    const uint32_t o1 = ao1 ? bo1 : bo0;
    return tup_make(c0, c1 - c0, o0, o1);
}

// Tile status words for the look-back: flag (bits 62-63: 1 aggregate,
// 2 inclusive prefix), epoch = iteration + 1 (bits 32-61), payload (bits 0-31:
// a tuple for an aggregate; kept-count | sel << 31 for a prefix). Stale words
// of earlier iterations carry another epoch, so nothing is reset in between.
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

// Wave 0 of a tile's workgroup: find the exclusive prefix (kept symbols
// before the tile, sel of the position before it) from the predecessors'
// status words, 64 tiles per round.
__device__ __forceinline__ void lookback(const unsigned long long* status, uint32_t t, uint32_t epoch,
                                         uint32_t lane, Ctl* ctl, uint32_t& off, uint32_t& sel) {
    // tiles already passed (those closest to t), unpacked: the kept count can
    // exceed the 24 bits of a packed tuple when the prefix lies far back
    uint32_t acc_c0 = 0, acc_d = 0, acc_o0 = 0, acc_o1 = 1;
    long long j = (long long)t - 1;
    uint32_t spins = 0;
    for (;;) {
        const long long idx = j - (long long)lane;
        unsigned long long st = (idx >= 0) ? st_load(status + idx) : st_pack(ST_PRE, epoch, 0u);
        int p;
        for (;;) {
            const bool valid = (st >> 62) != 0ull && (uint32_t)((st >> 32) & 0x3FFFFFFFull) == epoch;
            const unsigned long long pm = __ballot(valid && (st >> 62) == 2ull);
            const unsigned long long vm = __ballot(valid);
            p = pm ? (__ffsll((long long)pm) - 1) : 64;
            const unsigned long long need = (p >= 63) ? ~0ull : ((2ull << p) - 1ull);
            if ((vm & need) == need) break;
            if (++spins > SPIN_LIMIT) {  // bounded wait: report and carry on
                if (lane == 0) {
                    atomicOr(&ctl->err, ERR_SPIN);
                    atomicExch(&ctl->done, 1u);
                }
                off = 0;
                sel = 0;
                return;
            }
            if (!valid && idx >= 0) st = st_load(status + idx);
        }
        // compose the aggregates of lanes [0, p): lane 63 holds the lowest tile
        uint32_t a = (lane < (uint32_t)p) ? (uint32_t)(st & 0xFFFFFFFFull) : TUP_ID;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t other = __shfl_down(a, o);
            if (lane + o < 64) a = tup_then(other, a);
        }
        a = __shfl(a, 0);
        {   // acc = (window a, then acc)
            const uint32_t ac0 = a & 0xFFFFFFu, ad = (a >> 24) & 1u, ao0 = (a >> 25) & 1u, ao1 = (a >> 26) & 1u;
            const uint32_t c0 = ac0 + acc_c0 + (ao0 & acc_d);
            const uint32_t c1 = ac0 + ad + acc_c0 + (ao1 & acc_d);
            const uint32_t o0 = ao0 ? acc_o1 : acc_o0;
            const uint32_t o1 = ao1 ? acc_o1 : acc_o0;
            acc_c0 = c0; acc_d = c1 - c0; acc_o0 = o0; acc_o1 = o1;
        }
        if (p < 64) {
            const uint32_t pay = __shfl((uint32_t)(st & 0xFFFFFFFFull), p);
            const uint32_t base = pay & 0x7FFFFFFFu, bsel = pay >> 31;
            off = base + acc_c0 + (bsel ? acc_d : 0u);
            sel = bsel ? acc_o1 : acc_o0;
            return;
        }
        j -= 64;
    }
}

// LDS index skew for the staged output (spreads thread-contiguous runs over banks)
__device__ __forceinline__ uint32_t skew(uint32_t i) { return i + (i >> 5); }

template <int TPB, int V, int LT>
__global__ __launch_bounds__(TPB) void k_merge(Ctl* ctl, uint32_t* __restrict__ buf0,
                                               uint32_t* __restrict__ buf1, uint32_t* table,
                                               uint32_t mask, unsigned long long* status,
                                               uint32_t* lengths) {
    constexpr int TILE = TPB * V;
    constexpr int NW = TPB / 64;
    static_assert(V == 16, "a thread owns 16 symbols (four 16-byte loads)");
    __shared__ uint32_t s_keys[LT];
    __shared__ uint32_t s_cnts[LT];
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
    const bool do_count = X != IDM;  // the last possible id: nothing can follow
    const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;

    lds_table_clear<TPB, LT>(s_keys, s_cnts);
    PairCounter<LT> pc;

    for (;;) {
        if (tid == 0) s_tile = atomicAdd(&ctl->tile_ctr, 1u);
        __syncthreads();
        const uint32_t t = s_tile;
        if (t >= ntiles) break;
        const uint32_t g0 = t * TILE + tid * V;

        // ---- load 16 symbols plus two on the left and one on the right
        uint32_t x[V];
        if (g0 + V <= n) {
            const uint4* p4 = reinterpret_cast<const uint4*>(in + g0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint4 v = p4[q];
                x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) x[j] = (g0 + j < n) ? in[g0 + j] : WS;
        }
        const uint32_t a1 = (g0 >= 1 && g0 - 1 < n) ? in[g0 - 1] : WS;
        const uint32_t a2 = (g0 >= 2 && g0 - 2 < n) ? in[g0 - 2] : WS;
        const uint32_t b1 = (g0 + V < n) ? in[g0 + V] : WS;

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

        // ---- this thread's tuple
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

        // ---- inclusive scan over the wave, then over waves
        uint32_t incl = tup;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint32_t u = __shfl_up(incl, o);
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
            if (t == 0) {
                // nothing before tile 0
            } else {
                if (lane == 0) st_store(status + t, st_pack(ST_AGG, epoch, tile_agg));
                lookback(status, t, epoch, lane, ctl, off, sel);
            }
            if (lane == 0) {
                const uint32_t kept = (tile_agg & 0xFFFFFFu) + (sel ? ((tile_agg >> 24) & 1u) : 0u);
                const uint32_t osel = sel ? ((tile_agg >> 26) & 1u) : ((tile_agg >> 25) & 1u);
                st_store(status + t, st_pack(ST_PRE, epoch, (off + kept) | (osel << 31)));
                s_off = off;
                s_sel = sel;
            }
        }
        __syncthreads();
        const uint32_t tile_off = s_off, tile_sel = s_sel;
        const uint32_t texcl = tup_then(wave_excl, lane_excl);
        const uint32_t my_local = (texcl & 0xFFFFFFu) + (tile_sel ? ((texcl >> 24) & 1u) : 0u);
        const uint32_t sel_in = tile_sel ? ((texcl >> 26) & 1u) : ((texcl >> 25) & 1u);
        const uint32_t tile_kept = (tile_agg & 0xFFFFFFu) + (tile_sel ? ((tile_agg >> 24) & 1u) : 0u);

        // ---- resolve sel for real, emit kept symbols to LDS, count new pairs
        uint32_t selbits = 0;
        {
            uint32_t s = sel_in;
#pragma unroll
            for (int j = 0; j <= V; ++j) {
                s = (occ >> j) & ~s & 1u;
                selbits |= s << j;
            }
        }
        uint32_t prevval;
        if (sel_in) prevval = X | (a2 & WS);              // g0-1 merged into g0-2
        else prevval = (selbits & 1u) ? (X | (a1 & WS)) : a1;
        uint32_t o = my_local;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if (((valid >> j) & 1u) && !((selbits >> j) & 1u)) {
                const uint32_t v = ((selbits >> (j + 1)) & 1u) ? (X | (x[j] & WS)) : x[j];
                s_stage[skew(o)] = v;
                ++o;
                if (do_count && !(v & WS)) pc.add(pair_key(prevval, v), s_keys, s_cnts, table, mask, ctl);
                prevval = v;
            }
        }
        pc.finish(s_keys, s_cnts, table, mask, ctl);
        __syncthreads();

        // ---- coalesced write of the tile's kept symbols
        for (uint32_t i = tid; i < tile_kept; i += TPB) out[tile_off + i] = s_stage[skew(i)];
        if (t == ntiles - 1 && tid == 0) {
            const uint32_t total = tile_off + tile_kept;
            ctl->n[(it + 1) & 1u] = total;
            lengths[it + 1] = total;
            __threadfence();
            atomicExch(&ctl->m, it + 1);
        }
        __syncthreads();
    }
    __syncthreads();
    lds_table_flush<TPB, LT>(s_keys, s_cnts, table, mask, ctl);
}

}  // namespace bpek
