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

// Workgroup pair table in LDS: LT slots in buckets of 4, read with one
// 16-byte LDS load, so a key sits at its first probe unless its whole home
// bucket was taken first. Counting a batch of keys is two phases per group
// of 8 keys per thread:
//   1. every lane reads the home buckets of its keys and adds the counts of
//      keys it finds (no divergent probe loops);
//   2. keys not found are queued in LDS and, after a barrier, the whole
//      block inserts them, one queued key per lane (claiming slots with CAS,
//      probing further buckets, or going to the global table).
// The table is flushed into the global table and cleared once it is half
// full, and at the end of a kernel. Plain data (no constructor) so that it
// can live in __shared__.
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

    // full insert: home bucket, then further buckets, then the global table
    __device__ __forceinline__ void insert(uint32_t key, uint32_t c, uint32_t* table, uint32_t mask, Ctl* ctl) {
        uint32_t b = mix32(key) & (NB - 1);
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
                    return;
                }
            }
            b = (b + p) & (NB - 1);
        }
        global_add(table, mask, key, c, ctl);
    }

    // Count one per non-EMPTY key k[j]. A set bit j of fold means key j
    // equals the next non-EMPTY key, whose add carries it (a run of one key
    // costs one add). qk/qc: LDS scratch of qcap >= 8 * tpb entries each.
    // Every thread of the block calls this (it contains barriers).
    template <int V>
    __device__ __forceinline__ void count(const uint32_t (&k)[V], uint32_t fold, uint32_t* qk, uint32_t* qc,
                                          uint32_t qcap, int tpb, uint32_t* table, uint32_t mask, Ctl* ctl) {
        constexpr int G = 4;  // keys probed together (one 16-byte LDS load each)
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
                            global_add(table, mask, k[g + j], cnt[j], ctl);
                        }
                        ++q;
                    }
                }
            }
            if ((g / G) % 2 == 0) continue;  // drain after every 8 keys per thread
            __syncthreads();
            const uint32_t nq = min(qn, qcap);
            if (nq) {  // uniform: read after the barrier
                for (uint32_t i = threadIdx.x; i < nq; i += tpb) insert(qk[i], qc[i], table, mask, ctl);
                __syncthreads();
                if (threadIdx.x == 0) qn = 0u;
                __syncthreads();
            }
        }
    }

    // every thread of the block
    __device__ __forceinline__ void flush(int tpb, uint32_t* table, uint32_t mask, Ctl* ctl) {
        for (int i = threadIdx.x; i < LT; i += tpb) {
            const uint32_t key = keys[i];
            if (key != EMPTY) global_add(table, mask, key, cnts[i], ctl);
        }
    }

    // every thread of the block, after a barrier that follows the last count
    __device__ __forceinline__ void flush_if_half_full(int tpb, uint32_t* table, uint32_t mask, Ctl* ctl) {
        if (2u * used > (uint32_t)LT) {
            flush(tpb, table, mask, ctl);
            __syncthreads();
            clear(tpb);
            __syncthreads();
        }
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
// Blocks take chunks of TPB * 16 bytes in turn; a thread covers 16
// consecutive bytes (one 16-byte load when the input is aligned, four
// 16-byte stores of symbols). The chunk loop is uniform over the block so
// that the LDS table can be flushed between chunks.

template <int TPB, int LT>
__global__ __launch_bounds__(TPB) void k_tag_count(const uint8_t* __restrict__ bytes, uint32_t n,
                                                   uint32_t* __restrict__ sym, uint32_t* table,
                                                   uint32_t mask, Ctl* ctl) {
    constexpr uint32_t CHUNK = TPB * 16;
    constexpr uint32_t QCAP = TPB * 8;
    __shared__ LdsTable<LT> tab;
    __shared__ uint32_t s_qk[QCAP], s_qc[QCAP];
    tab.clear(TPB);
    __syncthreads();
    const bool aligned = ((uintptr_t)bytes & 15u) == 0;
    const uint32_t nchunks = (n + CHUNK - 1) / CHUNK;
    for (uint32_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
        const size_t base = (size_t)ch * CHUNK + threadIdx.x * 16;
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
        tab.template count<16>(keys, fold, s_qk, s_qc, QCAP, TPB, table, mask, ctl);
        tab.flush_if_half_full(TPB, table, mask, ctl);
    }
    __syncthreads();
    tab.flush(TPB, table, mask, ctl);
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

    // four 16-byte loads (eight slots) in flight per thread per round
    unsigned long long best = 0ull;
    uint4* t4 = reinterpret_cast<uint4*>(table);
    const uint32_t n4 = n_slots / 2;
    constexpr uint32_t U = 4;
    for (uint32_t i0 = blockIdx.x * TPB * U + threadIdx.x; i0 < n4; i0 += gridDim.x * TPB * U) {
        uint4 v[U];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t i = i0 + u * TPB;
            v[u] = (i < n4) ? t4[i] : make_uint4(EMPTY, 0u, EMPTY, 0u);
        }
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            if (v[u].x != EMPTY) {
                const unsigned long long p = ((unsigned long long)v[u].y << 32) | (uint32_t)~v[u].x;
                best = p > best ? p : best;
            }
            if (v[u].z != EMPTY) {
                const unsigned long long p = ((unsigned long long)v[u].w << 32) | (uint32_t)~v[u].z;
                best = p > best ? p : best;
            }
            if (v[u].x != EMPTY || v[u].z != EMPTY) t4[i0 + u * TPB] = make_uint4(EMPTY, 0u, EMPTY, 0u);
        }
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

}  // namespace bpek
