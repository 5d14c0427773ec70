// Training over the distinct words in one workgroup with occurrence lists
// (gfx950, wave64).
//
// Each pair of the pair table has a list of the record chunks that hold it.
// A pair appears in a chunk only once in a run: a new adjacency always
// involves the newest id (page "bpe - GPU BPE Tokenizer Pipeline", "Nedir
// bu ya?": each merge makes one new symbol), so a chunk never gains an
// existing pair, and a pair's list is complete when the pair first appears:
// the initial pairs' lists are built once (k_occ_scan to count, k_occ_place
// to place, k_occ_scan again to fill), and the lists of the pairs an iteration creates (all hold its
// new id X) are the chunks it rewrote that hold them. An iteration then
// touches only the chunks on the merged pair's list (a listed chunk that no
// longer holds the pair is skipped), so one workgroup runs every iteration
// in one launch (k_ck_solo): the selection from a candidate table in LDS,
// the rewrite of the listed chunks, the count changes, the new lists. No
// other workgroup exists, so nothing waits on another.
#pragma once

#include "chunks.hpp"

namespace bpek {

// Occurrence lists: list of table slot s at pool[off[s] - len[s] .. off[s]).
struct OccLists {
    uint32_t* off;
    uint32_t* len;
    uint32_t* pool;
    uint32_t cap;  // pool entries
};

// The table's pairs by pair id (claim order): slot[id] the table slot,
// key[id], cnt[id] its count (kept equal to the slot's), and id_of[slot].
// A sweep reads cnt[] front to back instead of gathering table slots.
struct PairIds {
    uint32_t* slot;
    uint32_t* key;
    uint32_t* cnt;
    uint32_t* id_of;
};

constexpr uint32_t ERR_SOLO = 8u;  // an LDS table, the pool or the scratch filled: the run is not used

// The slot of a key that is in the table (NO_SLOT if it is not).
__device__ __forceinline__ uint32_t gt_find(const GTable& gt, uint32_t key) {
    uint32_t h = mix32(key) & gt.mask;
    for (uint32_t p = 0; p < GT_PROBES; ++p, h = (h + 1u) & gt.mask) {
        const uint32_t k = (uint32_t)gt.slot[h];
        if (k == key) return h;
        if (k == EMPTY) return NO_SLOT;
    }
    return NO_SLOT;
}

// Bit i (1 <= i < 32, within pm): pair (i - 1, i) of the record is the first
// of its key in the record.
__device__ __forceinline__ uint32_t ck_first_pairs(const CkRec& r, uint32_t pm) {
    uint32_t k[32];
#pragma unroll
    for (int i = 1; i < 32; ++i) k[i] = (r.sym(i - 1) << 16) | r.sym(i);
    uint32_t first = 0u;
#pragma unroll
    for (int i = 1; i < 32; ++i) {
        bool dup = false;
#pragma unroll
        for (int j = 1; j < i; ++j) dup |= ((pm >> j) & 1u) && k[j] == k[i];
        first |= dup ? 0u : 1u << i;
    }
    return first & pm;
}

// PLACE false: len[s] += the record chunks holding the key of slot s (each
// once). PLACE true: each such chunk's index written to its list (off[s]
// moves from the list's start to its end).
template <int TPB, bool PLACE>
__global__ __launch_bounds__(TPB) void k_occ_scan(Chunks ck, GTable gt, OccLists ol) {
    for (uint32_t c = blockIdx.x * TPB + threadIdx.x; c < ck.nr; c += gridDim.x * TPB) {
        CkRec r;
        r.load(ck, c);
        const uint32_t first = ck_first_pairs(r, ck_pair_mask(ck.rlen[c]));
        for (uint32_t m = first; m; m &= m - 1u) {
            const uint32_t i = (uint32_t)__ffs(m) - 1u;
            uint32_t key = 0u;
#pragma unroll
            for (int j = 1; j < 32; ++j)
                if ((uint32_t)j == i) key = (r.sym(j - 1) << 16) | r.sym(j);
            const uint32_t s = gt_find(gt, key);
            if (s == NO_SLOT) continue;  // not reached: k_ck_pairs put every pair in
            if (PLACE)
                ol.pool[atomicAdd(ol.off + s, 1u)] = c;
            else
                atomicAdd(ol.len + s, 1u);
        }
    }
}

// Each workgroup takes a contiguous range of the slots: the lists' starts
// (off), the range's total taken from *ctr with one atomic; and the claimed
// slots (key not EMPTY) given pair ids, counted in ctr[1].
template <int TPB>
__global__ __launch_bounds__(TPB) void k_occ_place(GTable gt, OccLists ol, PairIds pid, uint32_t* ctr) {
    __shared__ uint32_t s_w[TPB / 64];
    __shared__ uint32_t s_base[2];
    const uint32_t slots = gt.mask + 1u, tid = threadIdx.x;
    const uint32_t per = (slots + gridDim.x - 1u) / gridDim.x;
    const uint32_t lo = min(slots, blockIdx.x * per), hi = min(slots, lo + per);
    uint32_t n = 0u, nc = 0u;
    for (uint32_t s = lo + tid; s < hi; s += TPB) {
        n += ol.len[s];
        nc += (uint32_t)gt.slot[s] != EMPTY ? 1u : 0u;
    }
    uint32_t all, allc;
    uint32_t at = block_exclusive_sum<TPB>(n, s_w, &all);
    uint32_t atc = block_exclusive_sum<TPB>(nc, s_w, &allc);
    if (tid == 0) {
        s_base[0] = all ? atomicAdd(ctr, all) : 0u;
        s_base[1] = allc ? atomicAdd(ctr + 1, allc) : 0u;
    }
    __syncthreads();
    at += s_base[0];
    atc += s_base[1];
    for (uint32_t s = lo + tid; s < hi; s += TPB) {
        ol.off[s] = at;
        at += ol.len[s];
        const unsigned long long v = gt.slot[s];
        if ((uint32_t)v != EMPTY) {
            pid.slot[atc] = s;
            pid.key[atc] = (uint32_t)v;
            pid.cnt[atc] = (uint32_t)(v >> 32);
            pid.id_of[s] = atc;
            ++atc;
        }
    }
}

// Every iteration of the run in one workgroup of TPB threads. State kept in
// LDS for the whole run: the candidate table (CT slots keyed by table
// slot, with the pair, its count and its list's place: every slot whose
// count is at least theta, and others); per iteration, the change table (KT slots keyed by
// pair: the summed count change, and for a new pair the number of chunks
// listing it and its list's place). An iteration:
//   1. the merge: the maximum of count << 32 | ~key over the candidates;
//      when it is below theta (or the candidates are not complete), over
//      every claimed slot of the pair table (a sweep), which also refills
//      the candidates (theta = max - (max >> shift));
//   2. each chunk on the pair's list, one per thread: the occurrences, the
//      merged ones left to right without overlap, the old pairs with a side
//      in one taken out and the new pairs put in with the chunk's weight,
//      the record rewritten (in an LDS row, then stored), and for each new
//      pair's first occurrence in the chunk an entry (change-table index,
//      chunk) in scratch;
//   3. the changes into the table, one per thread: a falling pair's count
//      (its candidate's too), a new pair's slot claimed with its count (a
//      candidate if it reaches theta) and its list placed in the pool;
//   4. scratch's entries into their lists.
// Pool, scratch or change table full: ERR_SOLO, and the caller trains
// with the multi-workgroup passes instead. Pair table full: ERR_TABLE.
template <int TPB, int CT, int KT>
__global__ __launch_bounds__(TPB) void k_ck_solo(Chunks ck, GTable gt, OccLists ol, const uint32_t* pool_used0,
                                                 PairIds pid, const uint32_t* n_claimed0, uint2* scratch,
                                                 uint32_t scratch_cap, uint32_t n_merges, uint32_t* merges,
                                                 Ctl* ctl) {
    static_assert((CT & (CT - 1)) == 0 && (KT & (KT - 1)) == 0, "table sizes: powers of two");
    if (ctl->done) return;  // the counting before found the pair table full
    __shared__ uint32_t c_slot[CT], c_key[CT], c_cnt[CT], c_off[CT], c_len[CT];
    __shared__ uint32_t k_key[KT], k_d[KT], k_n[KT], k_base[KT];
    __shared__ uint32_t s_rec[TPB * 17];
    __shared__ unsigned long long s_best[TPB / 64];
    __shared__ uint32_t s_bidx[TPB / 64], s_nge[TPB / 64];
    // scalars: 0 theta, 1 shift, 2 candidates held, 3 candidates complete,
    // 4 pool used, 5 claimed slots, 6 scratch entries, 7 error bits,
    // 8 the merged pair's slot, 9 pair-table claims, 10 collected,
    // 11 and 12 the merged pair's list (end, length)
    __shared__ uint32_t s_v[16];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
    for (uint32_t i = tid; i < (uint32_t)CT; i += TPB) c_slot[i] = EMPTY;
    for (uint32_t i = tid; i < (uint32_t)KT; i += TPB) {
        k_key[i] = EMPTY;
        k_d[i] = 0u;
        k_n[i] = 0u;
    }
    if (tid == 0) {
        s_v[0] = 0u;
        s_v[1] = SHIFT_DEFAULT;
        s_v[2] = 0u;
        s_v[3] = 0u;
        s_v[4] = *pool_used0;
        s_v[5] = *n_claimed0;
        s_v[6] = 0u;
        s_v[7] = 0u;
        s_v[9] = ctl->used;
    }
    uint32_t* const my_rec = s_rec + 17u * tid;
    __syncthreads();

    // a slot into the candidate table (count updated if it is there); false
    // if the table is more than half full (not probed then) or no free slot
    // is found
    auto cand_put = [&](uint32_t slot, uint32_t key, uint32_t cnt, uint32_t off, uint32_t len) -> bool {
        if (s_v[2] > (uint32_t)CT / 2u) return false;
        uint32_t h = mix32(slot) & (uint32_t)(CT - 1);
        for (uint32_t p = 0; p < (uint32_t)CT / 4u; ++p, h = (h + 1u) & (uint32_t)(CT - 1)) {
            uint32_t cur = __hip_atomic_load(&c_slot[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (cur == EMPTY) {
                cur = atomicCAS(&c_slot[h], EMPTY, slot);
                if (cur == EMPTY) {
                    atomicAdd(&s_v[2], 1u);
                    cur = slot;
                }
            }
            if (cur == slot) {
                c_key[h] = key;
                c_cnt[h] = cnt;
                c_off[h] = off;
                c_len[h] = len;
                return true;
            }
        }
        return false;
    };
    // the candidate's count, if the slot is a candidate
    auto cand_set = [&](uint32_t slot, uint32_t cnt) {
        uint32_t h = mix32(slot) & (uint32_t)(CT - 1);
        for (uint32_t p = 0; p < (uint32_t)CT / 4u; ++p, h = (h + 1u) & (uint32_t)(CT - 1)) {
            const uint32_t cur = c_slot[h];
            if (cur == slot) {
                c_cnt[h] = cnt;
                return;
            }
            if (cur == EMPTY) return;
        }
    };
    // the change table's index of a key (claimed if new); KT if full
    auto chg = [&](uint32_t key) -> uint32_t {
        uint32_t h = mix32(key) & (uint32_t)(KT - 1);
        for (uint32_t p = 0; p < (uint32_t)KT; ++p, h = (h + 1u) & (uint32_t)(KT - 1)) {
            uint32_t cur = __hip_atomic_load(&k_key[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (cur == EMPTY) {
                cur = atomicCAS(&k_key[h], EMPTY, key);  // the fields of a free entry are zero
                if (cur == EMPTY) cur = key;
            }
            if (cur == key) return h;
        }
        atomicOr(&s_v[7], ERR_SOLO);
        return (uint32_t)KT;
    };

    uint32_t it = 0;
    for (; it < n_merges; ++it) {
        // ---- 1. the merge
        unsigned long long best = 0ull;
        if (s_v[3]) {
            unsigned long long b = 0ull;
            uint32_t bi = 0u;
            for (uint32_t i = tid; i < (uint32_t)CT; i += TPB) {
                const uint32_t c = c_cnt[i];
                const unsigned long long v =
                    c_slot[i] != EMPTY && c ? ((unsigned long long)c << 32) | (uint32_t)~c_key[i] : 0ull;
                if (v > b) {
                    b = v;
                    bi = i;
                }
            }
            const unsigned long long wb = wave_max64(b);
            const unsigned long long m = __ballot(b == wb);
            if (lane == (uint32_t)(__ffsll((long long)m) - 1)) {
                s_best[w] = wb;
                s_bidx[w] = bi;
            }
            lds_barrier();
            uint32_t at = 0u;
#pragma unroll
            for (int i = 0; i < TPB / 64; ++i)
                if (s_best[i] > best) {
                    best = s_best[i];
                    at = s_bidx[i];
                }
            if (best && (uint32_t)(best >> 32) >= s_v[0]) {
                if (tid == 0) {
                    s_v[8] = c_slot[at];
                    s_v[11] = c_off[at];
                    s_v[12] = c_len[at];
                }
            } else {
                best = 0ull;
            }
        }
        if (best == 0ull) {
            // a sweep over the pairs' counts by id (eight loads in flight
            // per thread): the top count and how many pairs hold at least
            // the current theta; then the maximum (the top count's pair of
            // the smallest key) and where it is, from a second pass that
            // refills the candidates (theta = top - (top >> shift)), or, when
            // theta already equals the top count and more pairs hold it than
            // the table may, from one over the pairs of the top count only
            // (every merge then sweeps until that changes)
            const uint32_t nc = s_v[5], theta0 = s_v[0];
            uint32_t top = 0u, nge = 0u;
            for (uint32_t i0 = tid; i0 < nc; i0 += 8u * TPB) {
                uint32_t c[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) c[u] = i0 + (uint32_t)u * TPB < nc ? pid.cnt[i0 + (uint32_t)u * TPB] : 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    top = max(top, c[u]);
                    nge += c[u] && c[u] >= theta0 ? 1u : 0u;
                }
            }
            top = (uint32_t)wave_max64(top);
            nge = wave_sum(nge);
            if (lane == 0) {
                s_best[w] = top;
                s_nge[w] = nge;
            }
            lds_barrier();
            top = 0u;
            nge = 0u;
#pragma unroll
            for (int i = 0; i < TPB / 64; ++i) {
                top = max(top, (uint32_t)s_best[i]);
                nge += s_nge[i];
            }
            lds_barrier();
            if (top == 0u) break;  // uniform: no pair is left
            const bool flat = theta0 == top && nge > (uint32_t)CT / 2u;
            for (uint32_t shift = s_v[1];; ++shift) {
                const uint32_t theta = flat || shift >= 31u ? top : top - (top >> shift);
                if (!flat) {
                    for (uint32_t i = tid; i < (uint32_t)CT; i += TPB) c_slot[i] = EMPTY;
                    if (tid == 0) {
                        s_v[2] = 0u;
                        s_v[10] = 0u;
                    }
                    lds_barrier();
                }
                uint32_t bid = 0u;
                best = 0ull;
                for (uint32_t i0 = tid; i0 < nc; i0 += 8u * TPB) {
                    uint32_t c[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        c[u] = i0 + (uint32_t)u * TPB < nc ? pid.cnt[i0 + (uint32_t)u * TPB] : 0u;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (c[u] >= theta && c[u]) {
                            const uint32_t id = i0 + (uint32_t)u * TPB, kk = pid.key[id];
                            if (!flat) {
                                const uint32_t sl = pid.slot[id];
                                if (!cand_put(sl, kk, c[u], ol.off[sl], ol.len[sl])) atomicOr(&s_v[10], 1u);
                            }
                            const unsigned long long v = ((unsigned long long)c[u] << 32) | (uint32_t)~kk;
                            if (v > best) {
                                best = v;
                                bid = id;
                            }
                        }
                }
                const unsigned long long wb = wave_max64(best);
                const unsigned long long m = __ballot(best == wb);
                if (lane == (uint32_t)(__ffsll((long long)m) - 1)) {
                    s_best[w] = wb;
                    s_bidx[w] = bid;
                }
                lds_barrier();
                best = 0ull;
#pragma unroll
                for (int i = 0; i < TPB / 64; ++i)
                    if (s_best[i] > best) {
                        best = s_best[i];
                        bid = s_bidx[i];
                    }
                // at most half full, so that the pairs this run adds find room
                const bool ok = !flat && !s_v[10] && s_v[2] <= (uint32_t)CT / 2u;
                const uint32_t held = s_v[2];
                lds_barrier();  // every thread has read the counts before they change
                if (flat || ok || theta == top) {  // uniform
                    if (tid == 0) {
                        const uint32_t sl = pid.slot[bid];
                        s_v[8] = sl;
                        s_v[11] = ol.off[sl];
                        s_v[12] = ol.len[sl];
                        s_v[3] = ok ? 1u : 0u;
                        if (!flat) {
                            s_v[0] = theta;
                            // steer the next window towards a quarter of the table
                            s_v[1] = held > (uint32_t)CT / 4u ? min(shift + 1u, SHIFT_MAX)
                                                              : (shift > 1u ? shift - 1u : 1u);
                        }
                    }
                    break;
                }
            }
        }
        lds_barrier();
        const uint32_t key = ~(uint32_t)best;
        const uint32_t L = key >> 16, R = key & IDM, X = BASE + it;
        const bool do_count = X != IDM;  // X = 65535 is the last id: nothing reads counts after it
        if (tid == 0) {
            merges[3 * it + 0] = L;
            merges[3 * it + 1] = R;
            merges[3 * it + 2] = (uint32_t)(best >> 32);
        }
        // ---- 2. the chunks on the pair's list
        const uint32_t n = s_v[12], start = s_v[11] - n;
        for (uint32_t e = tid; e < n; e += TPB) {
            const uint32_t c = ol.pool[start + e];
            CkRec r;
            r.load(ck, c);
            const uint32_t len = ck.rlen[c], wt = ck.rw[c];
            const uint32_t pm = ck_pair_mask(len);
            uint32_t occ = 0u;
#pragma unroll
            for (int i = 1; i < 32; ++i) occ |= (r.sym(i - 1) == L && r.sym(i) == R) ? 1u << i : 0u;
            occ &= pm;
            if (!occ) continue;  // a chunk that lost the pair to an earlier merge
            uint32_t sel = occ;
            if (L == R) {
                sel = 0u;
                uint32_t prev = 0u;
#pragma unroll
                for (int i = 1; i < 32; ++i) {
                    const uint32_t b = (occ >> i) & 1u & (prev ^ 1u);
                    sel |= b << i;
                    prev = b;
                }
            }
            const uint32_t site = sel | (sel >> 1);
            const uint32_t changed = (site | (site << 1)) & pm;
            const uint32_t minus = (uint32_t)(-(int)wt);
#pragma unroll
            for (int j = 0; j < 16; ++j) my_rec[j] = r.v[j];
            if (do_count)
                for (uint32_t m = changed; m; m &= m - 1u) {
                    const uint32_t i = (uint32_t)__ffs(m) - 1u;
                    const uint32_t h = chg((row_sym(my_rec, i - 1u) << 16) | row_sym(my_rec, i));
                    if (h < (uint32_t)KT) atomicAdd(&k_d[h], minus);
                }
            // in place in the row: position o <= i is written after i is read
            uint32_t o = 0u, pv = 0u;
#pragma unroll 1
            for (uint32_t i = 0; i < len; ++i) {
                if ((sel >> i) & 1u) continue;
                const bool mx = i < 31u && ((sel >> (i + 1u)) & 1u);
                const uint32_t cur = mx ? X : row_sym(my_rec, i);
                row_set(my_rec, o, cur);
                if (do_count && o && (pv == X || cur == X)) {
                    const uint32_t h = chg((pv << 16) | cur);
                    if (h < (uint32_t)KT) {
                        atomicAdd(&k_d[h], wt);
                        // the chunk is listed once per pair: at its first occurrence
                        bool seen = false;
                        for (uint32_t j = 1; j < o && !seen; ++j)
                            seen = row_sym(my_rec, j - 1u) == pv && row_sym(my_rec, j) == cur;
                        if (!seen) {
                            atomicAdd(&k_n[h], 1u);
                            const uint32_t q = atomicAdd(&s_v[6], 1u);
                            if (q < scratch_cap)
                                scratch[q] = make_uint2(h, c);
                            else
                                atomicOr(&s_v[7], ERR_SOLO);
                        }
                    }
                }
                pv = cur;
                ++o;
            }
            uint4* dst = ck.rec + 4u * (size_t)c;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dst[j] = make_uint4(my_rec[4 * j], my_rec[4 * j + 1], my_rec[4 * j + 2], my_rec[4 * j + 3]);
            ck.rlen[c] = o;
        }
        __syncthreads();  // and scratch and the records are visible to the whole workgroup
        if (s_v[7]) break;  // uniform
        // ---- 3. the changes into the pair table, one entry per thread
        for (uint32_t i = tid; i < (uint32_t)KT; i += TPB) {
            const uint32_t kk = k_key[i];
            if (kk == EMPTY) continue;
            const uint32_t d = k_d[i];
            if ((int)d < 0) {
                // a falling pair: it is in the table
                uint32_t h = mix32(kk) & gt.mask;
                for (uint32_t p = 0; p < GT_PROBES; ++p, h = (h + 1u) & gt.mask) {
                    const unsigned long long v = gt.slot[h];
                    const uint32_t id = pid.id_of[h];  // loaded with the slot: used if the key matches
                    if ((uint32_t)v == kk) {
                        const uint32_t c = (uint32_t)(v >> 32) + d;
                        gt.slot[h] = ((unsigned long long)c << 32) | kk;
                        pid.cnt[id] = c;
                        cand_set(h, c);
                        break;
                    }
                }
            } else if (d) {
                // a new pair (it holds X): claim a slot with its count
                uint32_t h = mix32(kk) & gt.mask, p = 0;
                for (; p < GT_PROBES; ++p, h = (h + 1u) & gt.mask)
                    if (atomicCAS(gt.slot + h, GT_EMPTY, ((unsigned long long)d << 32) | kk) == GT_EMPTY) break;
                if (p == GT_PROBES || atomicAdd(&s_v[9], 1u) >= gt.limit) {
                    atomicOr(&s_v[7], ERR_TABLE);
                    continue;
                }
                const uint32_t id = atomicAdd(&s_v[5], 1u);
                pid.slot[id] = h;
                pid.key[id] = kk;
                pid.cnt[id] = d;
                pid.id_of[h] = id;
                const uint32_t cnt = k_n[i];
                const uint32_t base = atomicAdd(&s_v[4], cnt);
                if (base + cnt > ol.cap) {
                    atomicOr(&s_v[7], ERR_SOLO);
                    continue;
                }
                if (d >= s_v[0] && !cand_put(h, kk, d, base + cnt, cnt)) s_v[3] = 0u;  // no room: the next merge sweeps
                ol.len[h] = cnt;
                ol.off[h] = base + cnt;
                k_base[i] = base;
                k_n[i] = 0u;  // now the fill count
            }
        }
        lds_barrier();
        if (s_v[7]) break;  // uniform
        // ---- 4. the new lists
        const uint32_t nscr = s_v[6];
        for (uint32_t j = tid; j < nscr; j += TPB) {
            const uint2 en = scratch[j];
            ol.pool[k_base[en.x] + atomicAdd(&k_n[en.x], 1u)] = en.y;
        }
        lds_barrier();
        for (uint32_t i = tid; i < (uint32_t)KT; i += TPB) {
            k_key[i] = EMPTY;
            k_d[i] = 0u;
            k_n[i] = 0u;
        }
        if (tid == 0) s_v[6] = 0u;
        __syncthreads();  // every store of the iteration is visible to the next
    }
    if (tid == 0) {
        ctl->k = it;
        ctl->m = it;
        ctl->done = 1u;
        ctl->used = s_v[9];
        ctl->err |= s_v[7];
    }
}

}  // namespace bpek
