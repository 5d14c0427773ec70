// Device code of the BPE training iteration for gfx950 (CDNA4, wave64).
//
// Steps of one training iteration, after the page "bpe - GPU BPE Tokenizer
// Pipeline (Egitim + Cikarim)" (llm.istanbul/learn/tr/13_bpe): word-boundary
// tagging ("Ne Yapar? 1", once), pair counting in two levels, first in a
// workgroup-local table and then across workgroups ("Ne Yapar? 2"), a
// deterministic maximum (pipeline list at the head of the page), then merge
// + prefix-scan compaction of the symbol array ("Ne Yapar? 3").
//
// How the work is laid out here (not the page's WGSL dispatch plan):
//   k_tag_count  bytes -> tagged uint32 symbols, and the pair counts of
//                iteration 0.
//   k_merge      (merge.hpp) one persistent pass over the symbols that
//                applies the merge, compacts with a single-pass decoupled
//                look-back scan, and counts the pairs of the new sequence for
//                the next iteration: the symbols are read once and written
//                once per iteration.
//   k_select     the second counting level plus the maximum: one workgroup
//                per key partition sums that partition's partial counts in
//                LDS, takes its maximum, and the last workgroup to finish
//                records the merge (device-resident, no host round trip).
// Counting: a workgroup aggregates its pairs in an LDS hash table; when the
// table is half full (and at the end) it is flushed as (key, count) records
// into NPART hash partitions of a record pool, grouped by partition in LDS
// and written with one atomic reservation per partition and 64-record chunk.
// Global memory sees no per-pair atomics: MI355X performs device-scope
// atomics at a few tens of G/s, far below the symbol rate, and most pairs of
// a tile are distinct once training is past its first iterations.
// All arithmetic is integer; results do not depend on scheduling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpek {

constexpr uint32_t WS = 0x10000u;        // word-start bit of a symbol
constexpr uint32_t IDM = 0xFFFFu;        // id field of a symbol
constexpr uint32_t EMPTY = 0xFFFFFFFFu;  // empty key (the pair 65535,65535 is never counted)
constexpr uint32_t BASE = 256u;

constexpr uint32_t ERR_TABLE = 1u;  // counting capacity exceeded (record pool or select table)
constexpr uint32_t ERR_SPIN = 2u;   // a look-back wait exceeded its bound

constexpr uint32_t LDS_PROBES = 16;       // buckets probed before giving up on an LDS table
constexpr uint32_t SPIN_LIMIT = 1u << 22;  // polls of one look-back before giving up

constexpr uint32_t NPART = 256;  // key partitions of the record pool
constexpr uint32_t CHUNK = 64;   // records reserved at a time per partition and workgroup

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
    uint32_t sweep_done;  // k_select workgroups finished
    uint32_t pad[3];
    unsigned long long best;  // packed argmax of the current selection
};

// Record pool: partition p owns records [p * pcap, (p + 1) * pcap); part_n[p]
// of them are reserved (filled, or padded with EMPTY keys).
struct Pool {
    uint2* rec;        // {key, count}
    uint32_t* part_n;  // NPART reservation counters
    uint32_t pcap;     // records per partition
};

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Murmur3 32-bit finalizer: spreads packed pair keys; the low bits pick an
// LDS bucket, the top 8 bits the partition.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

__device__ __forceinline__ uint32_t part_of(uint32_t key) { return mix32(key) >> 24; }

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

// One record written on its own (rare: an LDS table with no free bucket).
__device__ __forceinline__ void emit_one(const Pool& pool, uint32_t key, uint32_t c, Ctl* ctl) {
    const uint32_t p = part_of(key);
    const uint32_t pos = atomicAdd(pool.part_n + p, 1u);
    if (pos < pool.pcap) {
        pool.rec[(size_t)p * pool.pcap + pos] = make_uint2(key, c);
    } else {
        atomicOr(&ctl->err, ERR_TABLE);
        atomicExch(&ctl->done, 1u);
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
                                          uint32_t qcap, int tpb, const Pool& pool, Ctl* ctl) {
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
                            emit_one(pool, k[g + j], cnt[j], ctl);
                        }
                        ++q;
                    }
                }
            }
            if ((g / G) % 2 == 0) continue;  // drain after every 8 keys per thread
            __syncthreads();
            const uint32_t nq = min(qn, qcap);
            if (nq) {  // uniform: read after the barrier
                for (uint32_t i = threadIdx.x; i < nq; i += tpb)
                    if (!insert(qk[i], qc[i])) emit_one(pool, qk[i], qc[i], ctl);
                __syncthreads();
                if (threadIdx.x == 0) qn = 0u;
                __syncthreads();
            }
        }
    }
};

// ---------------------------------------------------------------- record emission
// Per-workgroup state for writing LDS table contents to the record pool.
// For each partition the workgroup holds a reserved chunk (cur_base, with
// cur_left records unused). A flush counts its entries per partition,
// reserves fresh contiguous chunks where the current one is too small (one
// global atomic per partition that needs space), ranks entries within their
// partition with LDS atomics and writes them.
struct Emitter {
    uint32_t cur_base[NPART];
    uint32_t cur_left[NPART];
    uint32_t hist[NPART];
    uint32_t rank[NPART];
    uint32_t avail[NPART];
    uint32_t obase[NPART];
    uint32_t nbase[NPART];

    // every thread; a barrier must follow before use
    __device__ __forceinline__ void init(int tpb) {
        for (int p = threadIdx.x; p < (int)NPART; p += tpb) {
            cur_left[p] = 0u;
            cur_base[p] = 0u;
            hist[p] = 0u;
        }
    }

    // Write every occupied slot of tab as a record. Every thread of the
    // block, after a barrier that follows the last change to tab.
    template <int LT>
    __device__ __forceinline__ void flush(const LdsTable<LT>& tab, int tpb, const Pool& pool, Ctl* ctl) {
        for (int i = threadIdx.x; i < LT; i += tpb) {
            const uint32_t key = tab.keys[i];
            if (key != EMPTY) atomicAdd(hist + part_of(key), 1u);
        }
        __syncthreads();
        for (int p = threadIdx.x; p < (int)NPART; p += tpb) {
            const uint32_t need = hist[p], left = cur_left[p];
            avail[p] = min(need, left);
            obase[p] = cur_base[p];
            rank[p] = 0u;
            if (need > left) {
                const uint32_t rest = need - left;
                const uint32_t nch = (rest + CHUNK - 1) / CHUNK;
                const uint32_t b = atomicAdd(pool.part_n + p, nch * CHUNK);
                nbase[p] = b;
                cur_base[p] = b + rest;
                cur_left[p] = nch * CHUNK - rest;
            } else {
                cur_base[p] += need;
                cur_left[p] = left - need;
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < LT; i += tpb) {
            const uint32_t key = tab.keys[i];
            if (key == EMPTY) continue;
            const uint32_t p = part_of(key);
            const uint32_t r = atomicAdd(rank + p, 1u);
            const uint32_t pos = (r < avail[p]) ? obase[p] + r : nbase[p] + (r - avail[p]);
            if (pos < pool.pcap) {
                pool.rec[(size_t)p * pool.pcap + pos] = make_uint2(key, tab.cnts[i]);
            } else {
                atomicOr(&ctl->err, ERR_TABLE);
                atomicExch(&ctl->done, 1u);
            }
        }
        __syncthreads();
        for (int p = threadIdx.x; p < (int)NPART; p += tpb) hist[p] = 0u;
    }

    // Fill the unused rest of every reserved chunk with EMPTY records (end
    // of the kernel; every thread of the block).
    __device__ __forceinline__ void pad(int tpb, const Pool& pool) {
        for (int p = threadIdx.x; p < (int)NPART; p += tpb) {
            const uint32_t b = cur_base[p], e = min(cur_base[p] + cur_left[p], pool.pcap);
            for (uint32_t i = b; i < e; ++i) pool.rec[(size_t)p * pool.pcap + i] = make_uint2(EMPTY, 0u);
        }
    }
};

// every thread of the block, after a barrier that follows the last count
template <int LT>
__device__ __forceinline__ void flush_if_half_full(LdsTable<LT>& tab, Emitter& em, int tpb, const Pool& pool,
                                                   Ctl* ctl) {
    if (2u * tab.used > (uint32_t)LT) {
        em.flush(tab, tpb, pool, ctl);
        __syncthreads();
        tab.clear(tpb);
        __syncthreads();
    }
}

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

// fill a buffer of 64-bit words with one value (status reset)
__global__ void k_fill64(unsigned long long* p, size_t count, unsigned long long v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// fill a buffer of 32-bit words with one value (reservation counters)
__global__ void k_fill32(uint32_t* p, size_t count, uint32_t v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ---------------------------------------------------------------- tag + count (iteration 0)
// Blocks take chunks of TPB * 16 bytes in turn; a thread covers 16
// consecutive bytes (one 16-byte load when the input is aligned, four
// 16-byte stores of symbols). The chunk loop is uniform over the block so
// that the LDS table can be flushed between chunks.

template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_tag_count(const uint8_t* __restrict__ bytes, uint32_t n,
                                                   uint32_t* __restrict__ sym, Pool pool, Ctl* ctl) {
    constexpr uint32_t CH = TPB * 16;
    constexpr uint32_t QCAP = TPB * 8;
    __shared__ LdsTable<LT> tab;
    __shared__ Emitter em;
    __shared__ uint32_t s_qk[QCAP], s_qc[QCAP];
    tab.clear(TPB);
    em.init(TPB);
    __syncthreads();
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
            for (int q = 0; q < 4; ++q) o[q] = make_uint4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
        } else {
            for (int j = 0; j < 16; ++j)
                if (base + j < n) sym[base + j] = s[j];
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
        tab.template count<16>(keys, fold, s_qk, s_qc, QCAP, TPB, pool, ctl);
        flush_if_half_full(tab, em, TPB, pool, ctl);
    }
    __syncthreads();
    em.flush(tab, TPB, pool, ctl);
    __syncthreads();
    em.pad(TPB, pool);
}

// ---------------------------------------------------------------- select
// One workgroup per partition: sum the partition's records in an LDS table
// of `slots` slots, take the maximum of the packed value (count << 32 |
// ~key) (highest count, ties to the smallest (left, right), independent of
// order), fold it into ctl->best with atomicMax, and reset the partition.
// A partition with more distinct pairs than the table holds is summed in S
// passes over its records, pass s taking the keys whose hash bits 12.. are
// s modulo S (S doubles until every pass fits). The last workgroup to
// finish records the merge and sets up the merge pass.

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

template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_select(Ctl* ctl, Pool pool, uint32_t slots, uint32_t* merges) {
    __shared__ LdsTable<LT> tab;
    __shared__ unsigned long long s_best[TPB / 64];
    __shared__ uint32_t s_last, s_nrec, s_fail;
    const uint32_t done = ld_relaxed(&ctl->done);
    const uint32_t k = ld_relaxed(&ctl->k);
    const uint32_t m = ld_relaxed(&ctl->m);
    const uint32_t limit = ld_relaxed(&ctl->limit);
    if (done || k != m || k >= limit) return;  // uniform over the grid

    const uint32_t p = blockIdx.x;
    slots = min(max(slots, 64u), (uint32_t)LT);
    const uint32_t nbmask = slots / 4 - 1;
    if (threadIdx.x == 0) s_nrec = min(pool.part_n[p], pool.pcap);
    __syncthreads();
    const uint32_t nrec = s_nrec;
    const uint4* r4 = reinterpret_cast<const uint4*>(pool.rec + (size_t)p * pool.pcap);
    unsigned long long best = 0ull;
    for (uint32_t S = 1;; S *= 2) {
        bool failed = false;
        best = 0ull;
        for (uint32_t pass = 0; pass < S; ++pass) {
            tab.clear_first(slots, TPB);
            if (threadIdx.x == 0) s_fail = 0u;
            __syncthreads();
            for (uint32_t i = threadIdx.x; 2 * i < nrec; i += TPB) {
                const uint4 v = r4[i];
                if (v.x != EMPTY && ((mix32(v.x) >> 12) & (S - 1)) == pass && !tab.insert(v.x, v.y, nbmask))
                    s_fail = 1u;
                if (2 * i + 1 < nrec && v.z != EMPTY && ((mix32(v.z) >> 12) & (S - 1)) == pass &&
                    !tab.insert(v.z, v.w, nbmask))
                    s_fail = 1u;
            }
            __syncthreads();
            if (s_fail) {  // uniform: read after the barrier
                failed = true;
                break;
            }
            for (uint32_t i = threadIdx.x; i < slots; i += TPB) {
                const uint32_t key = tab.keys[i];
                if (key != EMPTY) {
                    const unsigned long long v = ((unsigned long long)tab.cnts[i] << 32) | (uint32_t)~key;
                    best = v > best ? v : best;
                }
            }
            __syncthreads();
        }
        if (!failed) break;
        if (S >= 4096) {  // cannot happen below 2^12 * slots distinct pairs
            if (threadIdx.x == 0) {
                atomicOr(&ctl->err, ERR_TABLE);
                atomicExch(&ctl->done, 1u);
            }
            break;
        }
        __syncthreads();
    }
    best = wave_max_u64(best);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) s_best[w] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long b = 0ull;
        for (int i = 0; i < TPB / 64; ++i) b = s_best[i] > b ? s_best[i] : b;
        if (b) atomicMax(&ctl->best, b);
        pool.part_n[p] = 0u;  // consumed
        __threadfence();
        const uint32_t prev = atomicAdd(&ctl->sweep_done, 1u);
        s_last = (prev == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last && threadIdx.x == 0) {
        __threadfence();
        const unsigned long long b = __hip_atomic_load(&ctl->best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (b == 0ull) {
            ctl->done = 1u;  // no countable pair is left
        } else {
            const uint32_t key = ~(uint32_t)(b & 0xFFFFFFFFull);
            const uint32_t cnt = (uint32_t)(b >> 32);
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

}  // namespace bpek
