// Host driver and C ABI of the BPE training library (include/bpe.h).
//
// The whole merge loop is enqueued on one stream with no host round trip
// between iterations: each iteration is one launch of the fused selection /
// merge / compaction / count-update pass (k_merge), which reads the
// iteration number, the merge and the sequence length from device state
// prepared by the launch before it, and does nothing once training has
// stopped. The host reads back a few bytes
// of status at the end, then copies only the merges and tokens that exist,
// in the spirit of the page's single submit with a sized readback ("Host
// Mimarisi 4", page "bpe - GPU BPE Tokenizer Pipeline").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/bpe.h"
#include "kernels.hpp"
#include "merge.hpp"
#include "trie.hpp"
#include "encode.hpp"
#include "chunks.hpp"
#include "chunks_solo.hpp"

using bpek::Ctl;

namespace {

// launch shapes
// The merge pass runs 1024-thread workgroups on 32768-symbol tiles (one per
// CU; two halves of 16 symbols per thread: fewer look-backs, status words
// and tile-counter atomics per symbol), or, when a corpus has fewer than two
// such tiles per CU, 512-thread workgroups on 16384-symbol tiles (two per
// CU), or, below one of those per CU, 512-thread workgroups on 8192-symbol
// tiles (one half), so that more of the chip takes part.
enum MergeKind { MERGE_BIG, MERGE_SMALL, MERGE_TINY };
constexpr int MERGE_TPB_BIG = 1024;
constexpr int MERGE_TPB_SMALL = 512;
constexpr int MERGE_LT = 1024;             // LDS slots for count changes, per workgroup
constexpr int TILE = bpek::merge_tile(MERGE_TPB_BIG, 2);  // the larger tile: symbol buffers are padded to it
constexpr int TILE_SMALL = bpek::merge_tile(MERGE_TPB_SMALL, 2);
constexpr int TILE_TINY = bpek::merge_tile(MERGE_TPB_SMALL, 1);  // the smallest tile
constexpr int TAG_TPB = 256;
constexpr int TAG_LT = 4096;

thread_local std::string g_err;

void set_err(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

#define HIP_TRY(expr)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess) {                                                              \
            set_err("%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, __LINE__); \
            return BPE_EHIP;                                                                 \
        }                                                                                    \
    } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

uint32_t ceil_log2(size_t v) {
    uint32_t r = 0;
    while ((size_t(1) << r) < v) ++r;
    return r;
}

// The automatic table size for n bytes and up to n_merges merges. Claimed
// slots (one per distinct pair the sequence ever holds) stay below 3n:
// n - 1 pairs at the start, and at most two new ones per merge site, of
// which there are at most n - 1 in all. Measured growth is far smaller:
// 10-25 new keys per merge on word corpora, about 350 on runs of random
// bytes; 512 per merge plus the 65,536 byte pairs bounds both. The table
// is sized so that the smaller estimate stays under its 7/8 limit.
uint32_t table_log2_for(size_t n, const bpe_config* cfg, uint32_t n_merges = BPE_MAX_MERGES) {
    if (cfg && cfg->table_log2) return cfg->table_log2;
    const uint64_t est = std::min<uint64_t>(3ull * (n ? n : 1), 65536ull + 512ull * n_merges);
    const uint32_t l = ceil_log2(size_t(est + est / 7 + 1));
    return std::min<uint32_t>(30, std::max<uint32_t>(12, l));
}

// Workgroups of the tag pass: enough to fill the chip, never more than
// there are chunks to hand out.
size_t tag_grid_bound(size_t n) { return (n + TAG_TPB * 16 - 1) / (TAG_TPB * 16) + 1; }

// The global table counts as full at 7/8 load (linear probing stays short).
uint32_t table_limit(uint32_t tlog2) { return uint32_t((1ull << tlog2) - (1ull << tlog2) / 8); }

struct Layout {
    size_t ctl, sweep, sym0, sym1, table, status, merges, lengths, fpairs, cls, cmask, total;
    uint32_t max_tiles;
};

Layout layout_for(size_t n, uint32_t tlog2) {
    Layout L{};
    size_t a = 0;
    L.ctl = a;
    a += 256;
    L.sweep = a;
    a = align_up(a + sizeof(bpek::Sweep), 256);
    const size_t sym_elems = align_up(n ? n : 1, TILE) + 64;
    L.sym0 = a;  // 16-bit ids
    a = align_up(a + 2 * sym_elems, 256);
    L.sym1 = a;
    a = align_up(a + 2 * sym_elems, 256);
    L.table = a;
    a = align_up(a + 8 * (size_t(1) << tlog2), 256);
    // at least 512 words: the look-back copies a 512-word window from index 0
    L.max_tiles = std::max<uint32_t>(uint32_t((n + TILE_TINY - 1) / TILE_TINY) + 1, 512);
    L.status = a;
    a = align_up(a + 8 * size_t(L.max_tiles), 256);
    L.merges = a;
    a = align_up(a + 12 * size_t(BPE_MAX_MERGES), 256);
    L.lengths = a;
    a = align_up(a + 4 * (size_t(BPE_MAX_MERGES) + 1), 256);
    L.fpairs = a;  // pairs of replayed iterations, indexed by iteration
    a = align_up(a + 8 * size_t(BPE_MAX_MERGES), 256);
    L.cls = a;  // class of every id
    a = align_up(a + 65536, 256);
    L.cmask = a;  // per class, the bit mask of its ids
    a = align_up(a + 4 * size_t(bpek::N_CLASSES) * bpek::CLASS_WORDS, 256);
    L.total = a;
    return L;
}

bool config_ok(size_t n, const bpe_config* cfg) {
    if (n > BPE_MAX_BYTES) {
        set_err("n = %zu exceeds the limit of %llu bytes", n, (unsigned long long)BPE_MAX_BYTES);
        return false;
    }
    if (cfg) {
        if (cfg->flags & ~uint32_t(BPE_FLAG_OVERSUBSCRIBE | BPE_FLAG_ALWAYS_CHUNKS)) {
            set_err("bpe_config.flags holds an unknown bit (0x%x)", cfg->flags);
            return false;
        }
        if (cfg->table_log2 && (cfg->table_log2 < 10 || cfg->table_log2 > 30)) {
            set_err("table_log2 = %u is outside 10..30", cfg->table_log2);
            return false;
        }
    }
    return true;
}

bool is_device_pointer(const void* p) {
    hipPointerAttribute_t a;
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged;
}

}  // namespace

struct bpe_state {
    int device = 0;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    bool null_stream = false;  // work goes to the null stream (a caller's NULL, without allocation)
    void* ws = nullptr;
    bool own_ws = false;
    size_t n = 0;
    uint32_t tlog2 = 0;
    Layout lay{};
    Ctl* ctl = nullptr;
    bpek::Sweep* sweep = nullptr;
    uint16_t* sym0 = nullptr;
    uint16_t* sym1 = nullptr;
    uint8_t* cls = nullptr;
    uint32_t* cmask = nullptr;
    unsigned long long* table = nullptr;
    unsigned long long* status = nullptr;
    uint32_t* merges = nullptr;
    uint32_t* lengths = nullptr;
    uint32_t* fpairs = nullptr;
    uint32_t requested = 0;  // iterations enqueued so far
    int merge_grid = 0, tag_grid = 0, fill_grid = 0;
    int merge_kind = MERGE_BIG;
    bool poisoned = false;   // a device error was seen

    uint32_t slots() const { return 1u << tlog2; }
    bpek::GTable gtable() const { return bpek::GTable{table, slots() - 1u, table_limit(tlog2)}; }
};

namespace {

// The merge pass of iteration it (one launch per iteration; a pass after
// training has stopped does nothing). Plain launches: no workgroup of the
// pass waits for one that has not started, so the grid need not be
// resident all at once.
template <int TPB, int HALVES>
void launch_merge_kind(bpe_state* s, uint32_t it) {
    hipLaunchKernelGGL((bpek::k_merge<TPB, MERGE_LT, HALVES>), dim3(s->merge_grid), dim3(TPB),
                       bpek::cmask_lds_bytes(it), s->stream, it, s->ctl, s->sym0, s->sym1, s->gtable(), s->status,
                       s->lengths, s->sweep, s->merges, s->cls, s->cmask);
}

void launch_merge(bpe_state* s, uint32_t it) {
    if (s->merge_kind == MERGE_BIG)
        launch_merge_kind<MERGE_TPB_BIG, 2>(s, it);
    else if (s->merge_kind == MERGE_SMALL)
        launch_merge_kind<MERGE_TPB_SMALL, 2>(s, it);
    else
        launch_merge_kind<MERGE_TPB_SMALL, 1>(s, it);
}

void launch_force(bpe_state* s) {
    hipLaunchKernelGGL(bpek::k_force, dim3(1), dim3(64), 0, s->stream, s->ctl, s->gtable(), s->sweep, s->fpairs);
}


bpe_status read_ctl(bpe_state* s, Ctl* h) {
    HIP_TRY(hipStreamSynchronize(s->stream));
    HIP_TRY(hipMemcpy(h, s->ctl, sizeof(Ctl), hipMemcpyDeviceToHost));
    if (h->err) {
        s->poisoned = true;
        if (h->err & bpek::ERR_TABLE) {
            set_err("the global pair table is full (%u of %u slots claimed; give a larger table_log2)",
                    table_limit(s->tlog2), s->slots());
            return BPE_ETABLE;
        }
        set_err("device error bits 0x%x", h->err);
        return BPE_ESTATE;
    }
    return BPE_OK;
}

// Timing events, kept per device for the life of the process so that a
// profiled run does not pay for creating them.
std::mutex g_ev_mu;
std::vector<hipEvent_t> g_ev[64];

bpe_status event_pool(int device, size_t count, std::vector<hipEvent_t>** out) {
    if (device < 0 || device >= 64) {
        set_err("device index %d out of range", device);
        return BPE_EINVAL;
    }
    std::lock_guard<std::mutex> lk(g_ev_mu);
    std::vector<hipEvent_t>& v = g_ev[device];
    while (v.size() < count) {
        hipEvent_t e;
        HIP_TRY(hipEventCreate(&e));
        v.push_back(e);
    }
    *out = &v;
    return BPE_OK;
}

// Iterations requested .. requested + n_merges - 1, which the passes are
// told; once training stops (no pair left) the later passes do nothing.
bpe_status state_setup(bpe_state* s, const uint8_t* bytes, size_t n, const bpe_config* cfg, uint32_t tlog2,
                       const Layout& lay, bool may_allocate);
void state_release(bpe_state* s);
bpe_status init_state(const uint8_t* bytes, size_t n, const bpe_config* cfg, uint32_t n_merges, bpe_state** out);

bpe_status enqueue_run(bpe_state* s, uint32_t n_merges, uint32_t* first) {
    if (size_t(s->requested) + n_merges > BPE_MAX_MERGES) {
        set_err("%u + %u merges exceed the id space (%u merges)", s->requested, n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    *first = s->requested;
    s->requested += n_merges;
    return BPE_OK;
}

}  // namespace

extern "C" {

size_t bpe_workspace_bytes(size_t n, const bpe_config* cfg) {
    if (!config_ok(n, cfg)) return 0;
    return layout_for(n, table_log2_for(n, cfg)).total;
}

const char* bpe_strerror(bpe_status st) {
    switch (st) {
        case BPE_OK: return "ok";
        case BPE_DONE: return "no countable pair is left";
        case BPE_EINVAL: return "invalid argument";
        case BPE_ETABLE: return "the global pair table is full";
        case BPE_EIDSPACE: return "merge count exceeds the 16-bit id space";
        case BPE_ENOMEM: return "out of memory";
        case BPE_EHIP: return "HIP runtime error";
        case BPE_ESTATE: return "state holds a device error";
    }
    return "unknown status";
}

const char* bpe_last_error(void) { return g_err.c_str(); }

bpe_status bpe_init(const uint8_t* bytes, size_t n, const bpe_config* cfg, bpe_state** out) {
    g_err.clear();
    return init_state(bytes, n, cfg, BPE_MAX_MERGES, out);
}

}  // extern "C"

namespace {

// bpe_init with the number of merges the caller will ask for (it sizes an
// automatic table; BPE_MAX_MERGES if unknown).
bpe_status init_state(const uint8_t* bytes, size_t n, const bpe_config* cfg, uint32_t n_merges, bpe_state** out) {
    if (!out) {
        set_err("out is NULL");
        return BPE_EINVAL;
    }
    *out = nullptr;
    if (!bytes || n == 0) {
        set_err("bytes must be non-NULL and n >= 1");
        return BPE_EINVAL;
    }
    if (!config_ok(n, cfg)) return BPE_EINVAL;
    const uint32_t tlog2 = table_log2_for(n, cfg, n_merges);
    const Layout lay = layout_for(n, tlog2);
    if (cfg && cfg->workspace && cfg->workspace_bytes < lay.total) {
        set_err("workspace of %zu bytes is smaller than the %zu bytes needed", cfg->workspace_bytes, lay.total);
        return BPE_EINVAL;
    }
    if (cfg && cfg->workspace && (reinterpret_cast<uintptr_t>(cfg->workspace) & 255u)) {
        set_err("workspace must be 256-byte aligned");
        return BPE_EINVAL;
    }

    bpe_state* s = new (std::nothrow) bpe_state();
    if (!s) {
        set_err("host allocation failed");
        return BPE_ENOMEM;
    }
    const bpe_status st = state_setup(s, bytes, n, cfg, tlog2, lay, true);
    if (st != BPE_OK) {
        bpe_free(s);
        return st;
    }
    *out = s;
    return BPE_OK;
}

// Fill a default-constructed state for bytes[0..n) (validated by the
// caller) and enqueue tagging and the first count. With may_allocate, a
// missing stream or workspace is created and owned by the state; without,
// the state uses the caller's stream (NULL: the null stream) and workspace
// and creates nothing. On failure the caller releases the state.
bpe_status state_setup(bpe_state* s, const uint8_t* bytes, size_t n, const bpe_config* cfg, uint32_t tlog2,
                       const Layout& lay, bool may_allocate) {
    auto fail = [](bpe_status st) { return st; };
    hipError_t e = hipGetDevice(&s->device);
    if (e != hipSuccess) {
        set_err("hipGetDevice failed: %s", hipGetErrorString(e));
        return fail(BPE_EHIP);
    }
    s->n = n;
    s->tlog2 = tlog2;
    s->lay = lay;
    if ((cfg && cfg->stream) || !may_allocate) {
        s->stream = static_cast<hipStream_t>(cfg ? cfg->stream : nullptr);
        s->null_stream = s->stream == nullptr;
    } else {
        // a blocking stream: it still orders after work on the legacy
        // default stream that produced the input
        e = hipStreamCreate(&s->stream);
        if (e != hipSuccess) {
            set_err("hipStreamCreate failed: %s", hipGetErrorString(e));
            return fail(BPE_EHIP);
        }
        s->own_stream = true;
    }
    if (cfg && cfg->workspace) {
        s->ws = cfg->workspace;
    } else if (!may_allocate) {
        set_err("no workspace given");
        return BPE_EINVAL;
    } else {
        e = hipMalloc(&s->ws, lay.total);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            set_err("hipMalloc of %zu bytes failed: %s", lay.total, hipGetErrorString(e));
            return fail(BPE_ENOMEM);
        }
        s->own_ws = true;
    }
    char* base = static_cast<char*>(s->ws);
    s->ctl = reinterpret_cast<Ctl*>(base + lay.ctl);
    s->sweep = reinterpret_cast<bpek::Sweep*>(base + lay.sweep);
    s->sym0 = reinterpret_cast<uint16_t*>(base + lay.sym0);
    s->sym1 = reinterpret_cast<uint16_t*>(base + lay.sym1);
    s->cls = reinterpret_cast<uint8_t*>(base + lay.cls);
    s->cmask = reinterpret_cast<uint32_t*>(base + lay.cmask);
    s->table = reinterpret_cast<unsigned long long*>(base + lay.table);
    s->status = reinterpret_cast<unsigned long long*>(base + lay.status);
    s->merges = reinterpret_cast<uint32_t*>(base + lay.merges);
    s->lengths = reinterpret_cast<uint32_t*>(base + lay.lengths);
    s->fpairs = reinterpret_cast<uint32_t*>(base + lay.fpairs);

    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, s->device);
    if (e != hipSuccess || cus <= 0) {
        set_err("cannot query the compute-unit count: %s", hipGetErrorString(e));
        return fail(BPE_EHIP);
    }
    int per_cu = 0;
    // the largest tile that still gives every CU work
    const size_t tiles_small = (n + TILE_SMALL - 1) / TILE_SMALL;
    s->merge_kind = (n + TILE - 1) / TILE >= 2 * size_t(cus) ? MERGE_BIG
                    : tiles_small >= size_t(cus)             ? MERGE_SMALL
                                                             : MERGE_TINY;
    size_t merge_tile = TILE;
    if (s->merge_kind == MERGE_BIG) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bpek::k_merge<MERGE_TPB_BIG, MERGE_LT, 2>,
                                                         MERGE_TPB_BIG, 0);
    } else if (s->merge_kind == MERGE_SMALL) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bpek::k_merge<MERGE_TPB_SMALL, MERGE_LT, 2>,
                                                         MERGE_TPB_SMALL, 0);
        merge_tile = TILE_SMALL;
    } else {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bpek::k_merge<MERGE_TPB_SMALL, MERGE_LT, 1>,
                                                         MERGE_TPB_SMALL, 0);
        merge_tile = TILE_TINY;
    }
    if (e != hipSuccess || per_cu <= 0) per_cu = 1;
    s->merge_grid = int(std::min<size_t>(size_t(cus) * per_cu, (n + merge_tile - 1) / merge_tile + 1));
    s->tag_grid = int(std::min<size_t>(size_t(cus) * 2, tag_grid_bound(n)));
    s->fill_grid = cus * 4;
    // testing aid: four times the workgroups that can be resident at once,
    // so that most of them start only when earlier ones have finished
    if (cfg && (cfg->flags & BPE_FLAG_OVERSUBSCRIBE)) s->merge_grid = int(size_t(cus) * per_cu * 4);

    // input bytes: device memory is read in place, host memory is uploaded
    // into the second symbol buffer first (2n bytes hold n bytes)
    const uint8_t* src = bytes;
    if (!is_device_pointer(bytes)) {
        e = hipMemcpyAsync(s->sym1, bytes, n, hipMemcpyHostToDevice, s->stream);
        if (e != hipSuccess) {
            set_err("upload of the corpus failed: %s", hipGetErrorString(e));
            return fail(BPE_EHIP);
        }
        src = reinterpret_cast<const uint8_t*>(s->sym1);
    }
    hipLaunchKernelGGL(bpek::k_fill64, dim3(4), dim3(256), 0, s->stream,
                       reinterpret_cast<unsigned long long*>(s->sweep), sizeof(bpek::Sweep) / 8, 0ull);
    hipLaunchKernelGGL(bpek::k_init_ctl, dim3(1), dim3(64), 0, s->stream, s->ctl, uint32_t(n), s->lengths);
    hipLaunchKernelGGL(bpek::k_init_classes, dim3(256), dim3(256), 0, s->stream, s->cls, s->cmask);
    hipLaunchKernelGGL(bpek::k_fill64, dim3(s->fill_grid), dim3(256), 0, s->stream, s->table, size_t(s->slots()),
                       bpek::GT_EMPTY);
    hipLaunchKernelGGL(bpek::k_fill64, dim3(s->fill_grid), dim3(256), 0, s->stream, s->status,
                       size_t(lay.max_tiles), 0ull);
    hipLaunchKernelGGL((bpek::k_tag_count<TAG_TPB, TAG_LT>), dim3(s->tag_grid), dim3(TAG_TPB), 0, s->stream,
                       src, uint32_t(n), s->sym0, s->gtable(), s->ctl);
    e = hipGetLastError();
    if (e != hipSuccess) {
        set_err("kernel launch failed: %s", hipGetErrorString(e));
        return fail(BPE_EHIP);
    }
    return BPE_OK;
}

// Wait for the state's work and release what it owns (not the state).
void state_release(bpe_state* s) {
    (void)hipSetDevice(s->device);
    if (s->stream || s->null_stream) (void)hipStreamSynchronize(s->stream);
    if (s->own_ws && s->ws) (void)hipFree(s->ws);
    if (s->own_stream && s->stream) (void)hipStreamDestroy(s->stream);
    s->ws = nullptr;
    s->stream = nullptr;
    s->own_ws = s->own_stream = false;
}

}  // namespace

extern "C" {

bpe_status bpe_run(bpe_state* s, uint32_t n_merges) {
    g_err.clear();
    if (!s) {
        set_err("state is NULL");
        return BPE_EINVAL;
    }
    if (s->poisoned) {
        set_err("the state holds a device error from an earlier call");
        return BPE_ESTATE;
    }
    HIP_TRY(hipSetDevice(s->device));
    uint32_t it0 = 0;
    bpe_status st = enqueue_run(s, n_merges, &it0);
    if (st != BPE_OK) return st;
    for (uint32_t i = 0; i < n_merges; ++i) launch_merge(s, it0 + i);
    HIP_TRY(hipGetLastError());
    return BPE_OK;
}

bpe_status bpe_sync(bpe_state* s, uint32_t* n_done) {
    g_err.clear();
    if (!s) {
        set_err("state is NULL");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    bpe_status st = read_ctl(s, &h);
    if (n_done) *n_done = h.k;
    return st;
}

bpe_status bpe_step(bpe_state* s, bpe_merge* out) {
    g_err.clear();
    if (!s || !out) {
        set_err("state and out must be non-NULL");
        return BPE_EINVAL;
    }
    if (s->poisoned) {
        set_err("the state holds a device error from an earlier call");
        return BPE_ESTATE;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl before;
    bpe_status st = read_ctl(s, &before);
    if (st != BPE_OK) return st;
    if (before.done) return BPE_DONE;
    // the limit follows the merges actually made, so a step after an early
    // stop or after bpe_run always allows exactly one more iteration
    if (before.k + 1 > BPE_MAX_MERGES) {
        set_err("the id space of %u merges is used up", BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    s->requested = before.k + 1;
    launch_merge(s, before.k);
    HIP_TRY(hipGetLastError());
    Ctl after;
    st = read_ctl(s, &after);
    if (st != BPE_OK) return st;
    if (after.k == before.k) return BPE_DONE;
    uint32_t m3[3];
    HIP_TRY(hipMemcpy(m3, s->merges + 3 * size_t(after.k - 1), sizeof m3, hipMemcpyDeviceToHost));
    out->left = m3[0];
    out->right = m3[1];
    out->count = m3[2];
    return BPE_OK;
}

bpe_status bpe_merges(bpe_state* s, bpe_merge* out, uint32_t cap, uint32_t* n_out) {
    g_err.clear();
    if (!s || (!out && cap)) {
        set_err("state must be non-NULL, and out non-NULL when cap > 0");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    bpe_status st = read_ctl(s, &h);
    if (st != BPE_OK) return st;
    if (n_out) *n_out = h.k;
    const uint32_t c = std::min(cap, h.k);
    if (c) HIP_TRY(hipMemcpy(out, s->merges, sizeof(bpe_merge) * size_t(c), hipMemcpyDefault));
    return BPE_OK;
}

bpe_status bpe_tokens(bpe_state* s, uint32_t* out, size_t cap, size_t* n_out) {
    g_err.clear();
    if (!s) {
        set_err("state is NULL");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    bpe_status st = read_ctl(s, &h);
    if (st != BPE_OK) return st;
    const size_t len = h.n[h.m & 1u];
    if (n_out) *n_out = len;
    if (!out || cap == 0) return BPE_OK;
    if (cap < len) {
        set_err("tokens capacity %zu is below the %zu symbols", cap, len);
        return BPE_EINVAL;
    }
    // the ids with their word starts (k_expand), written straight into
    // device memory; for host memory through the free symbol buffer (2
    // bytes per symbol: the tokens in two halves), which the next pass
    // overwrites anyway
    const uint16_t* src = (h.m & 1u) ? s->sym1 : s->sym0;
    uint16_t* freebuf = (h.m & 1u) ? s->sym0 : s->sym1;
    const bool dev = is_device_pointer(out);
    const size_t part = dev ? len : (len + 1) / 2;
    for (size_t b = 0; b < len; b += part) {
        const size_t cnt = std::min(part, len - b);
        uint32_t* dst = dev ? out + b : reinterpret_cast<uint32_t*>(freebuf);
        const unsigned grid = unsigned(std::min<size_t>((cnt + 255) / 256, 4096));
        hipLaunchKernelGGL(bpek::k_expand, dim3(grid), dim3(256), 0, s->stream, src, uint32_t(b), uint32_t(cnt),
                           s->cls, dst);
        HIP_TRY(hipGetLastError());
        if (!dev) {
            HIP_TRY(hipMemcpyAsync(out + b, dst, 4 * cnt, hipMemcpyDeviceToHost, s->stream));
            HIP_TRY(hipStreamSynchronize(s->stream));
        }
    }
    if (dev) HIP_TRY(hipStreamSynchronize(s->stream));
    return BPE_OK;
}

bpe_status bpe_lengths(bpe_state* s, uint32_t* out, uint32_t cap, uint32_t* n_out) {
    g_err.clear();
    if (!s || (!out && cap)) {
        set_err("state must be non-NULL, and out non-NULL when cap > 0");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    bpe_status st = read_ctl(s, &h);
    if (st != BPE_OK) return st;
    if (n_out) *n_out = h.m + 1;
    const uint32_t c = std::min(cap, h.m + 1);
    if (c) HIP_TRY(hipMemcpy(out, s->lengths, 4 * size_t(c), hipMemcpyDefault));
    return BPE_OK;
}

bpe_status bpe_table_usage(bpe_state* s, uint32_t* slots, uint32_t* claimed, uint32_t* limit) {
    g_err.clear();
    if (!s) {
        set_err("state is NULL");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    const bpe_status st = read_ctl(s, &h);
    if (slots) *slots = s->slots();
    if (claimed) *claimed = h.used;
    if (limit) *limit = table_limit(s->tlog2);
    return st;
}

bpe_status bpe_pair_counts(bpe_state* s, uint32_t* keys, uint32_t* counts, size_t cap, size_t* n_out) {
    g_err.clear();
    if (!s || (cap && (!keys || !counts))) {
        set_err("state must be non-NULL, and keys/counts non-NULL when cap > 0");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    bpe_status st = read_ctl(s, &h);
    if (st != BPE_OK) return st;
    // the global table holds the counts of the current sequence
    std::vector<unsigned long long> tab(s->slots());
    HIP_TRY(hipMemcpy(tab.data(), s->table, 8 * tab.size(), hipMemcpyDeviceToHost));
    std::vector<std::pair<uint32_t, uint32_t>> sum;
    for (unsigned long long v : tab)
        if (v >> 32) sum.emplace_back(uint32_t(v), uint32_t(v >> 32));
    std::vector<uint32_t> k, c;
    for (const auto& kv : sum) {
        k.push_back(kv.first);
        c.push_back(uint32_t(kv.second));
    }
    if (n_out) *n_out = k.size();
    if (cap == 0) return BPE_OK;
    if (cap < k.size()) {
        set_err("capacity %zu is below the %zu distinct pairs", cap, k.size());
        return BPE_EINVAL;
    }
    if (!k.empty()) {
        HIP_TRY(hipMemcpy(keys, k.data(), 4 * k.size(), hipMemcpyDefault));
        HIP_TRY(hipMemcpy(counts, c.data(), 4 * c.size(), hipMemcpyDefault));
    }
    return BPE_OK;
}

bpe_status bpe_profile(bpe_state* s, uint32_t n_merges, bpe_profile_result* res, float* merge_ms) {
    g_err.clear();
    if (!s || !res) {
        set_err("state and out must be non-NULL");
        return BPE_EINVAL;
    }
    if (s->poisoned) {
        set_err("the state holds a device error from an earlier call");
        return BPE_ESTATE;
    }
    HIP_TRY(hipSetDevice(s->device));
    std::memset(res, 0, sizeof *res);
    std::vector<hipEvent_t>* ev = nullptr;
    bpe_status st = event_pool(s->device, size_t(n_merges) + 1, &ev);
    if (st != BPE_OK) return st;
    uint32_t sweeps0 = 0, sweeps1 = 0;
    HIP_TRY(hipStreamSynchronize(s->stream));
    HIP_TRY(hipMemcpy(&sweeps0, &s->sweep->sweeps, 4, hipMemcpyDeviceToHost));
    uint32_t it0 = 0;
    st = enqueue_run(s, n_merges, &it0);
    if (st != BPE_OK) return st;
    std::vector<hipEvent_t>& e = *ev;
    HIP_TRY(hipEventRecord(e[0], s->stream));
    for (uint32_t i = 0; i < n_merges; ++i) {
        launch_merge(s, it0 + i);
        HIP_TRY(hipEventRecord(e[size_t(i) + 1], s->stream));
    }
    HIP_TRY(hipGetLastError());
    HIP_TRY(hipEventSynchronize(e[size_t(n_merges)]));
    for (uint32_t i = 0; i < n_merges; ++i) {
        float c = 0.f;
        HIP_TRY(hipEventElapsedTime(&c, e[size_t(i)], e[size_t(i) + 1]));
        res->merge_ms += c;
        if (merge_ms) merge_ms[i] = c;
    }
    res->launches = n_merges;
    Ctl h;
    st = read_ctl(s, &h);
    res->merges_done = h.k;
    HIP_TRY(hipMemcpy(&sweeps1, &s->sweep->sweeps, 4, hipMemcpyDeviceToHost));
    res->sweeps = sweeps1 - sweeps0;
    return st;
}

bpe_status bpe_replay(bpe_state* s, const bpe_merge* merges, uint32_t k) {
    g_err.clear();
    if (!s || (!merges && k)) {
        set_err("state must be non-NULL, and merges non-NULL when k > 0");
        return BPE_EINVAL;
    }
    if (s->poisoned) {
        set_err("the state holds a device error from an earlier call");
        return BPE_ESTATE;
    }
    HIP_TRY(hipSetDevice(s->device));
    Ctl h;
    bpe_status st = read_ctl(s, &h);
    if (st != BPE_OK) return st;
    if (k == 0) return BPE_OK;
    if (h.done) {
        set_err("training on this state has stopped; nothing can be replayed");
        return BPE_ESTATE;
    }
    const uint32_t m0 = h.k;
    if (size_t(m0) + k > BPE_MAX_MERGES) {
        set_err("%u + %u merges exceed the id space (%u merges)", m0, k, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    std::vector<bpe_merge> hm(k);
    HIP_TRY(hipMemcpy(hm.data(), merges, sizeof(bpe_merge) * size_t(k), hipMemcpyDefault));
    std::vector<uint32_t> pairs(2 * size_t(k));
    for (uint32_t i = 0; i < k; ++i) {
        const uint32_t lim = bpek::BASE + m0 + i;  // ids that exist before merge m0 + i
        if (hm[i].left >= lim || hm[i].right >= lim) {
            set_err("merge %u (%u, %u) names an id that does not exist before it (ids < %u)", m0 + i,
                    hm[i].left, hm[i].right, lim);
            return BPE_EINVAL;
        }
        pairs[2 * i] = hm[i].left;
        pairs[2 * i + 1] = hm[i].right;
    }
    HIP_TRY(hipMemcpyAsync(s->fpairs + 2 * size_t(m0), pairs.data(), 4 * pairs.size(), hipMemcpyHostToDevice,
                           s->stream));
    s->requested = m0 + k;
    for (uint32_t i = 0; i < k; ++i) {
        launch_force(s);
        launch_merge(s, m0 + i);
    }
    HIP_TRY(hipGetLastError());
    st = read_ctl(s, &h);  // also keeps pairs alive until the copy has run
    if (st != BPE_OK) return st;
    if (h.k != m0 + k) {
        set_err("replay stopped after %u of %u merges", h.k - m0, k);
        return BPE_ESTATE;
    }
    return BPE_OK;
}

void bpe_free(bpe_state* s) {
    if (!s) return;
    state_release(s);
    delete s;
}

bpe_status bpe_train(const uint8_t* bytes, size_t n, uint32_t n_merges, const bpe_config* cfg, bpe_merge* merges,
                     uint32_t* n_done, uint32_t* tokens, size_t tokens_cap, size_t* n_tokens) {
    g_err.clear();
    if (!n_done || (!merges && n_merges) || (n && !bytes)) {
        set_err("bytes (when n > 0), merges (when n_merges > 0) and n_done must be non-NULL");
        return BPE_EINVAL;
    }
    if (n_merges > BPE_MAX_MERGES) {
        set_err("%u merges exceed the id space (%u merges)", n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    if (!config_ok(n, cfg)) return BPE_EINVAL;
    if (tokens && tokens_cap < n) {
        // the final length is only known at the end; n always suffices
        set_err("tokens_cap %zu is below n = %zu", tokens_cap, n);
        return BPE_EINVAL;
    }
    *n_done = 0;
    if (n_tokens) *n_tokens = 0;
    if (n == 0) return BPE_OK;
    bpe_state* s = nullptr;
    bpe_status st = init_state(bytes, n, cfg, n_merges, &s);
    if (st != BPE_OK) return st;
    st = bpe_run(s, n_merges);
    uint32_t done = 0;
    if (st == BPE_OK) st = bpe_sync(s, &done);
    if (st == BPE_OK && done) st = bpe_merges(s, merges, done, nullptr);
    if (st == BPE_OK && (tokens || n_tokens)) st = bpe_tokens(s, tokens, tokens ? tokens_cap : 0, n_tokens);
    if (st == BPE_OK) *n_done = done;
    bpe_free(s);
    return st;
}

}  // extern "C"

// ======================================================================== training without allocation
// bpe_train_static: bpe_train on a workspace in the library's own device
// memory, for callers that cannot allocate. The workspace is a file-scope
// device array; host code uses the address hipGetSymbolAddress returns for
// the current device (each device holds its own copy), never the array's
// name, which in host code is only a stand-in.

namespace {

static __device__ __align__(256) unsigned char scratch[BPE_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The address of this device's copy of scratch, looked up once per device
// (with that device current, as it is on every call).
bpe_status static_scratch(int device, void** out) {
    if (device < 0 || device >= 64) {
        set_err("device index %d out of range", device);
        return BPE_EINVAL;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            set_err("hipGetSymbolAddress of the static workspace failed: %s", hipGetErrorString(e));
            return BPE_EHIP;
        }
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return BPE_OK;
}

}  // namespace

extern "C" {

bpe_status bpe_train_static(const uint8_t* bytes, size_t n, uint32_t n_merges, uint32_t table_log2, void* stream,
                            bpe_merge* merges, uint32_t* n_done, uint32_t* tokens, size_t tokens_cap,
                            size_t* n_tokens) {
    g_err.clear();
    if (!n_done || (!merges && n_merges) || (n && !bytes)) {
        set_err("bytes (when n > 0), merges (when n_merges > 0) and n_done must be non-NULL");
        return BPE_EINVAL;
    }
    if (n_merges > BPE_MAX_MERGES) {
        set_err("%u merges exceed the id space (%u merges)", n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    if (n > BPE_STATIC_MAX_BYTES) {
        set_err("n = %zu exceeds the %u bytes the static workspace takes", n, BPE_STATIC_MAX_BYTES);
        return BPE_EINVAL;
    }
    if (table_log2 && (table_log2 < 10 || table_log2 > BPE_STATIC_MAX_TABLE_LOG2)) {
        set_err("table_log2 = %u is outside 10..%u for the static workspace", table_log2,
                BPE_STATIC_MAX_TABLE_LOG2);
        return BPE_EINVAL;
    }
    if (tokens && tokens_cap < n) {
        set_err("tokens_cap %zu is below n = %zu", tokens_cap, n);
        return BPE_EINVAL;
    }
    *n_done = 0;
    if (n_tokens) *n_tokens = 0;
    if (n == 0) return BPE_OK;
    const uint32_t tlog2 =
        table_log2 ? table_log2
                   : std::min<uint32_t>(BPE_STATIC_MAX_TABLE_LOG2, table_log2_for(n, nullptr, n_merges));
    const Layout lay = layout_for(n, tlog2);
    if (lay.total > BPE_STATIC_SCRATCH_BYTES) {
        set_err("%zu bytes of workspace needed, the static workspace holds %u", lay.total, BPE_STATIC_SCRATCH_BYTES);
        return BPE_EINVAL;
    }
    int device = 0;
    HIP_TRY(hipGetDevice(&device));
    void* ws = nullptr;
    bpe_status st = static_scratch(device, &ws);
    if (st != BPE_OK) return st;
    bpe_config cfg{};
    cfg.table_log2 = tlog2;
    cfg.stream = stream;
    cfg.workspace = ws;
    cfg.workspace_bytes = BPE_STATIC_SCRATCH_BYTES;
    bpe_state s;  // on the stack: nothing is allocated, on the host or the device
    st = state_setup(&s, bytes, n, &cfg, tlog2, lay, false);
    if (st == BPE_OK) st = bpe_run(&s, n_merges);
    uint32_t done = 0;
    if (st == BPE_OK) st = bpe_sync(&s, &done);
    if (st == BPE_OK && done) st = bpe_merges(&s, merges, done, nullptr);
    if (st == BPE_OK && (tokens || n_tokens)) st = bpe_tokens(&s, tokens, tokens ? tokens_cap : 0, n_tokens);
    if (st == BPE_OK) *n_done = done;
    state_release(&s);
    return st;
}

}  // extern "C"

// ======================================================================== inference
// Greedy longest-match tokenization over a double-array trie of a merge
// list's vocabulary (page "bpe - GPU BPE Tokenizer Pipeline", "Nedir bu
// ya?" inference paragraph, "Ne Yapar? 4", "Host Mimarisi 1-4").

struct bpe_trie {
    int device = 0;
    hipStream_t stream = nullptr;               // used when the caller passes none
    unsigned long long* da = nullptr;           // the double array
    size_t da_slots = 0;
    uint32_t root_base = 0;
    uint32_t max_len = 0;
    uint32_t* total = nullptr;                  // device: token count of the last call
    // pooled buffers, grown by half again when a call needs more ("Host
    // Mimarisi 2"); kept until bpe_trie_free
    uint16_t* slices = nullptr;                 // per-tile token slices (walk -> copy)
    size_t slices_cap = 0;
    uint32_t* tiles = nullptr;                  // cnt, ovf_pos, ovf_n, pfx: 4 x ntiles
    size_t tiles_cap = 0;
    uint8_t* text_buf = nullptr;
    size_t text_cap = 0;
    uint32_t* tok_buf = nullptr;
    size_t tok_cap = 0;
    int walk_grid = 0, copy_grid = 0;
};

namespace {

constexpr int TRIE_TPB = 512;
constexpr uint32_t TRIE_TILE = TRIE_TPB * 16;
constexpr uint32_t TRIE_CAP = TRIE_TILE + TRIE_TPB * bpek::TRIE_HALO_PER_THREAD;
constexpr int TRIE_SCAN_TPB = 1024;
constexpr int TRIE_COPY_TPB = 256;
constexpr uint64_t TRIE_MAX_STRING_BYTES = uint64_t(1) << 27;  // total vocabulary string bytes accepted

// The page's char_class, on the host.
uint32_t host_byte_class(uint32_t b) {
    if (b == 0x0Au) return 4u;
    if (b == 0x20u) return 2u;
    if (b >= 0x30u && b <= 0x39u) return 1u;
    if (b >= 0x80u || (b >= 0x61u && b <= 0x7Au) || (b >= 0x41u && b <= 0x5Au)) return 0u;
    return 3u;
}

// Vocabulary of a merge list -> prefix tree -> double array. Trie nodes are
// placed in BFS order (children of a node sorted by byte, "Host Mimarisi 1");
// a node's base is the lowest value >= 1 that puts all of its children on
// free slots (first fit, with a next-free-slot union-find).
bpe_status build_double_array(const std::vector<bpe_merge>& hm, std::vector<unsigned long long>* da,
                              uint32_t* root_base, uint32_t* max_len) {
    const uint32_t k = uint32_t(hm.size()), nv = bpek::BASE + k;
    std::vector<uint64_t> len(nv), off(nv);
    std::vector<uint32_t> cls(nv);
    uint64_t total = 0;
    for (uint32_t i = 0; i < nv; ++i) {
        if (i < bpek::BASE) {
            len[i] = 1;
            cls[i] = host_byte_class(i);
        } else {
            const uint32_t l = hm[i - bpek::BASE].left, r = hm[i - bpek::BASE].right;
            if (l >= i || r >= i) {
                set_err("merge %u (%u, %u) names an id that does not exist before it (ids < %u)", i - bpek::BASE, l,
                        r, i);
                return BPE_EINVAL;
            }
            if (cls[l] != cls[r]) {
                set_err("merge %u (%u, %u) joins strings of different byte classes; no trained merge does, and "
                        "such a string could match across a word start", i - bpek::BASE, l, r);
                return BPE_EINVAL;
            }
            len[i] = len[l] + len[r];
            cls[i] = cls[l];
        }
        off[i] = total;
        total += len[i];
        if (total > TRIE_MAX_STRING_BYTES) {
            set_err("the vocabulary's strings exceed %llu bytes", (unsigned long long)TRIE_MAX_STRING_BYTES);
            return BPE_EINVAL;
        }
    }
    std::vector<uint8_t> pool(total);
    for (uint32_t i = 0; i < nv; ++i) {
        if (i < bpek::BASE) {
            pool[off[i]] = uint8_t(i);
        } else {
            const uint32_t l = hm[i - bpek::BASE].left, r = hm[i - bpek::BASE].right;
            std::memcpy(&pool[off[i]], &pool[off[l]], len[l]);
            std::memcpy(&pool[off[i] + len[l]], &pool[off[r]], len[r]);
        }
        *max_len = uint32_t(std::max<uint64_t>(*max_len, len[i]));
    }

    // prefix tree: node 0 is the root; id i's node is reached from the node
    // of its left part by the bytes of its right part
    std::unordered_map<uint64_t, uint32_t> child;
    child.reserve(size_t(nv) * 2);
    std::vector<int32_t> tok(1, -1);
    std::vector<std::vector<uint8_t>> kids(1);
    std::vector<uint32_t> node_of(nv);
    for (uint32_t i = 0; i < nv; ++i) {
        uint32_t node = 0;
        uint64_t from = off[i], to = off[i] + len[i];
        if (i >= bpek::BASE) {
            const uint32_t l = hm[i - bpek::BASE].left;
            node = node_of[l];
            from = off[i] + len[l];
        }
        for (uint64_t j = from; j < to; ++j) {
            const uint64_t key = (uint64_t(node) << 8) | pool[j];
            auto it = child.find(key);
            if (it == child.end()) {
                const uint32_t nn = uint32_t(tok.size());
                if (nn >= bpek::TR_MAX_SLOTS) {
                    set_err("the vocabulary needs more than %u trie nodes", bpek::TR_MAX_SLOTS);
                    return BPE_EINVAL;
                }
                child.emplace(key, nn);
                tok.push_back(-1);
                kids.emplace_back();
                kids[node].push_back(pool[j]);
                node = nn;
            } else {
                node = it->second;
            }
        }
        node_of[i] = node;
        if (tok[node] < 0) tok[node] = int32_t(i);  // the smallest id keeps a string
    }

    // double array
    const uint32_t lim = bpek::TR_MAX_SLOTS + 256u;
    std::vector<uint32_t> nf(size_t(lim) + 1);  // next free slot at or after i
    for (uint32_t i = 0; i <= lim; ++i) nf[i] = i;
    auto find = [&](uint32_t i) {
        while (nf[i] != i) {
            nf[i] = nf[nf[i]];
            i = nf[i];
        }
        return i;
    };
    auto take = [&](uint32_t i) { nf[i] = i + 1; };
    std::vector<uint32_t> slot_of(tok.size()), base_of(tok.size(), 0), parent_slot(tok.size(), 0);
    std::vector<uint32_t> order;
    order.reserve(tok.size());
    order.push_back(0);
    slot_of[0] = 0;
    take(0);
    uint32_t top = 1;
    for (size_t qi = 0; qi < order.size(); ++qi) {
        const uint32_t node = order[qi];
        std::vector<uint8_t>& ks = kids[node];
        if (ks.empty()) continue;
        std::sort(ks.begin(), ks.end());
        uint32_t b = std::max<uint32_t>(1u, find(1u) > ks[0] ? find(1u) - ks[0] : 1u);
        for (;;) {
            if (b + 255u >= lim) {
                set_err("the vocabulary needs more than %u trie slots", bpek::TR_MAX_SLOTS);
                return BPE_EINVAL;
            }
            const uint32_t f = find(b + ks[0]);
            b = f - ks[0];
            bool ok = true;
            for (size_t j = 1; j < ks.size() && ok; ++j) ok = find(b + ks[j]) == b + ks[j];
            if (ok) break;
            ++b;
        }
        if (b + 255u >= lim) {
            set_err("the vocabulary needs more than %u trie slots", bpek::TR_MAX_SLOTS);
            return BPE_EINVAL;
        }
        base_of[node] = b;
        for (uint8_t c : ks) {
            const uint32_t kn = child.at((uint64_t(node) << 8) | c);
            slot_of[kn] = b + c;
            parent_slot[kn] = slot_of[node];
            take(b + c);
            order.push_back(kn);
        }
        top = std::max(top, b + 256u);
    }
    da->assign(top, 0ull);
    for (uint32_t node : order) {
        const uint32_t check = node == 0 ? 0u : parent_slot[node] + 1u;
        const uint32_t t1 = tok[node] < 0 ? 0u : uint32_t(tok[node]) + 1u;
        (*da)[slot_of[node]] = bpek::tr_pack(check, base_of[node], t1);
    }
    *root_base = base_of[0];
    return BPE_OK;
}

// A merge list from host or device memory into host memory: host lists are
// copied without touching the device, so a bad list is rejected before any
// device call.
bpe_status copy_merges(const bpe_merge* merges, uint32_t n_merges, bpe_merge* out) {
    if (!n_merges) return BPE_OK;
    if (is_device_pointer(merges))
        HIP_TRY(hipMemcpy(out, merges, sizeof(bpe_merge) * n_merges, hipMemcpyDeviceToHost));
    else
        std::memcpy(out, merges, sizeof(bpe_merge) * n_merges);
    return BPE_OK;
}

template <typename T>
bpe_status pool_grow(T** p, size_t* cap, size_t need, bool zero) {
    if (*cap >= need) return BPE_OK;
    const size_t ncap = std::max(need, *cap + *cap / 2);
    if (*p) HIP_TRY(hipFree(*p));
    *p = nullptr;
    *cap = 0;
    if (hipMalloc(reinterpret_cast<void**>(p), ncap * sizeof(T)) != hipSuccess) {
        (void)hipGetLastError();
        set_err("hipMalloc of %zu bytes failed", ncap * sizeof(T));
        return BPE_ENOMEM;
    }
    if (zero) HIP_TRY(hipMemset(*p, 0, ncap * sizeof(T)));
    *cap = ncap;
    return BPE_OK;
}

}  // namespace

extern "C" {

bpe_status bpe_trie_build(const bpe_merge* merges, uint32_t n_merges, bpe_trie** out) {
    g_err.clear();
    if (!out || (!merges && n_merges)) {
        set_err("out must be non-NULL, and merges non-NULL when n_merges > 0");
        return BPE_EINVAL;
    }
    *out = nullptr;
    if (n_merges > BPE_MAX_MERGES) {
        set_err("%u merges exceed the id space (%u merges)", n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    std::vector<bpe_merge> hm(n_merges);
    bpe_status st = copy_merges(merges, n_merges, hm.data());
    if (st != BPE_OK) return st;
    std::vector<unsigned long long> da;
    uint32_t root_base = 0, max_len = 0;
    st = build_double_array(hm, &da, &root_base, &max_len);
    if (st != BPE_OK) return st;

    bpe_trie* t = new (std::nothrow) bpe_trie();
    if (!t) {
        set_err("out of host memory");
        return BPE_ENOMEM;
    }
    auto fail = [&](bpe_status s) {
        bpe_trie_free(t);
        return s;
    };
    if (hipGetDevice(&t->device) != hipSuccess) return fail(BPE_EHIP);
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, t->device) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bpek::k_trie_walk<TRIE_TPB>, TRIE_TPB, 0) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        set_err("cannot query the device");
        return fail(BPE_EHIP);
    }
    t->walk_grid = cus * per_cu;
    t->copy_grid = cus * 8;
    // a blocking stream: a call with no stream of its own is then ordered
    // after work on the legacy default stream (the producer of its input,
    // the last user of its output)
    if (hipStreamCreate(&t->stream) != hipSuccess) {
        (void)hipGetLastError();
        set_err("hipStreamCreate failed");
        return fail(BPE_EHIP);
    }
    t->da_slots = da.size();
    t->root_base = root_base;
    t->max_len = max_len;
    if (hipMalloc(reinterpret_cast<void**>(&t->da), da.size() * sizeof(unsigned long long)) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&t->total), sizeof(uint32_t)) != hipSuccess) {
        (void)hipGetLastError();
        set_err("hipMalloc failed");
        return fail(BPE_ENOMEM);
    }
    if (hipMemcpy(t->da, da.data(), da.size() * sizeof(unsigned long long), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        set_err("uploading the trie failed");
        return fail(BPE_EHIP);
    }
    *out = t;
    return BPE_OK;
}

bpe_status bpe_trie_info(const bpe_trie* t, uint32_t* slots, uint32_t* max_len) {
    g_err.clear();
    if (!t) {
        set_err("trie must be non-NULL");
        return BPE_EINVAL;
    }
    if (slots) *slots = uint32_t(t->da_slots);
    if (max_len) *max_len = t->max_len;
    return BPE_OK;
}

}  // extern "C"

namespace {

// Per-tile arrays are padded to a multiple of 4 scan threads' worth, so the
// scan reads them with 16-byte loads.
uint32_t trie_npad(uint32_t ntiles) {
    const uint32_t q = 4u * TRIE_SCAN_TPB;
    return (ntiles + q - 1u) / q * q;
}

// The three passes on stream s: walk, scan, copy. ev, if given, gets an
// event recorded after each pass (3 events).
bpe_status trie_enqueue(bpe_trie* t, const uint8_t* src, uint32_t n, uint32_t* dst, hipStream_t s,
                        hipEvent_t* ev) {
    const uint32_t ntiles = (n + TRIE_TILE - 1) / TRIE_TILE;
    const uint32_t npad = trie_npad(ntiles);
    uint32_t* cnt = t->tiles;
    uint32_t* ovf_pos = cnt + npad;
    uint32_t* ovf_n = ovf_pos + npad;
    uint32_t* pfx = ovf_n + npad;
    hipLaunchKernelGGL(bpek::k_trie_walk<TRIE_TPB>, dim3(std::min<uint32_t>(ntiles, t->walk_grid)), dim3(TRIE_TPB),
                       0, s, src, n, t->da, t->root_base, t->slices, cnt, ovf_pos, ovf_n, ntiles);
    if (ev) HIP_TRY(hipEventRecord(ev[0], s));
    hipLaunchKernelGGL(bpek::k_trie_scan<TRIE_SCAN_TPB>, dim3(1), dim3(TRIE_SCAN_TPB), 0, s, cnt, ovf_n, pfx,
                       ntiles, npad, t->total);
    if (ev) HIP_TRY(hipEventRecord(ev[1], s));
    hipLaunchKernelGGL(bpek::k_trie_copy<TRIE_COPY_TPB>, dim3(std::min<uint32_t>(ntiles, t->copy_grid)),
                       dim3(TRIE_COPY_TPB), 0, s, src, n, t->da, t->root_base, t->slices, cnt, ovf_pos, ovf_n,
                       pfx, dst, ntiles, TRIE_TILE, TRIE_CAP);
    if (ev) HIP_TRY(hipEventRecord(ev[2], s));
    HIP_TRY(hipGetLastError());
    return BPE_OK;
}

bpe_status trie_pools(bpe_trie* t, size_t n) {
    const size_t ntiles = (n + TRIE_TILE - 1) / TRIE_TILE;
    bpe_status st = pool_grow(&t->slices, &t->slices_cap, ntiles * TRIE_CAP, false);
    if (st == BPE_OK) st = pool_grow(&t->tiles, &t->tiles_cap, 4 * size_t(trie_npad(uint32_t(ntiles))), false);
    return st;
}

}  // namespace

extern "C" {

bpe_status bpe_trie_encode(bpe_trie* t, const uint8_t* bytes, size_t n, void* stream, uint32_t* tokens,
                           size_t tokens_cap, size_t* n_tokens) {
    g_err.clear();
    if (!t || !n_tokens || (n && !bytes)) {
        set_err("trie and n_tokens must be non-NULL, and bytes non-NULL when n > 0");
        return BPE_EINVAL;
    }
    if (n > BPE_MAX_BYTES) {
        set_err("n = %zu exceeds the limit of %llu bytes", n, (unsigned long long)BPE_MAX_BYTES);
        return BPE_EINVAL;
    }
    if (tokens && tokens_cap < n) {
        set_err("tokens_cap %zu is below n = %zu", tokens_cap, n);
        return BPE_EINVAL;
    }
    *n_tokens = 0;
    if (n == 0) return BPE_OK;
    HIP_TRY(hipSetDevice(t->device));
    hipStream_t s = stream ? reinterpret_cast<hipStream_t>(stream) : t->stream;
    bpe_status st = trie_pools(t, n);
    if (st != BPE_OK) return st;
    const uint8_t* src = bytes;
    if (!is_device_pointer(bytes)) {
        st = pool_grow(&t->text_buf, &t->text_cap, n, false);
        if (st != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(t->text_buf, bytes, n, hipMemcpyHostToDevice, s));
        src = t->text_buf;
    }
    uint32_t* dst = tokens;
    if (!tokens || !is_device_pointer(tokens)) {
        st = pool_grow(&t->tok_buf, &t->tok_cap, n, false);
        if (st != BPE_OK) return st;
        dst = t->tok_buf;
    }
    st = trie_enqueue(t, src, uint32_t(n), dst, s, nullptr);
    if (st != BPE_OK) return st;
    uint32_t total = 0;
    HIP_TRY(hipMemcpyAsync(&total, t->total, sizeof total, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    if (total > n) {
        set_err("device reported %u tokens for %zu bytes", total, n);
        return BPE_ESTATE;
    }
    *n_tokens = total;
    if (tokens && dst != tokens) HIP_TRY(hipMemcpy(tokens, dst, sizeof(uint32_t) * size_t(total), hipMemcpyDefault));
    return BPE_OK;
}

bpe_status bpe_trie_profile(bpe_trie* t, const uint8_t* bytes, size_t n, uint32_t reps, float* ms,
                            size_t* n_tokens) {
    g_err.clear();
    if (!t || !n_tokens || !bytes || n == 0 || reps == 0 || n > BPE_MAX_BYTES) {
        set_err("trie, bytes and n_tokens must be non-NULL, 0 < n <= BPE_MAX_BYTES and reps > 0");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(t->device));
    if (!is_device_pointer(bytes)) {
        set_err("bpe_trie_profile reads device bytes only");
        return BPE_EINVAL;
    }
    size_t first = 0;
    bpe_status st = bpe_trie_encode(t, bytes, n, nullptr, nullptr, 0, &first);  // sizes the pools
    if (st != BPE_OK) return st;
    std::vector<hipEvent_t>* ev = nullptr;
    st = event_pool(t->device, 3 * size_t(reps) + 1, &ev);
    if (st != BPE_OK) return st;
    std::vector<hipEvent_t>& e = *ev;
    HIP_TRY(hipEventRecord(e[0], t->stream));
    for (uint32_t r = 0; r < reps; ++r) {
        st = trie_enqueue(t, bytes, uint32_t(n), t->tok_buf, t->stream, &e[3 * size_t(r) + 1]);
        if (st != BPE_OK) return st;
    }
    uint32_t total = 0;
    HIP_TRY(hipMemcpyAsync(&total, t->total, sizeof total, hipMemcpyDeviceToHost, t->stream));
    HIP_TRY(hipStreamSynchronize(t->stream));
    if (total != first) {
        set_err("repeated runs disagree on the token count (%u vs %zu)", total, first);
        return BPE_ESTATE;
    }
    for (size_t i = 0; i < 3 * size_t(reps); ++i) {
        float a = 0.f;
        HIP_TRY(hipEventElapsedTime(&a, e[i], e[i + 1]));
        if (ms) ms[i] = a;
    }
    *n_tokens = first;
    return BPE_OK;
}

void bpe_trie_free(bpe_trie* t) {
    if (!t) return;
    (void)hipSetDevice(t->device);
    if (t->stream) (void)hipStreamSynchronize(t->stream);
    if (t->da) (void)hipFree(t->da);
    if (t->total) (void)hipFree(t->total);
    if (t->slices) (void)hipFree(t->slices);
    if (t->tiles) (void)hipFree(t->tiles);
    if (t->text_buf) (void)hipFree(t->text_buf);
    if (t->tok_buf) (void)hipFree(t->tok_buf);
    if (t->stream) (void)hipStreamDestroy(t->stream);
    delete t;
}

}  // extern "C"

// ======================================================================== encoding
// A merge list applied to new text word by word, lowest rank first (equal
// to applying its merges in learned order over the whole text; page "bpe -
// GPU BPE Tokenizer Pipeline", "Nedir bu ya?").

struct bpe_encoder {
    int device = 0;
    hipStream_t stream = nullptr;
    unsigned long long* rt = nullptr;   // rank table
    uint16_t* rt_bytes = nullptr;       // rank of every byte pair
    uint32_t rt_mask = 0, rt_probes = 0;
    uint32_t* status = nullptr;         // total, error flags, scratch used
    uint32_t* slices = nullptr;         // per-tile token slices
    size_t slices_cap = 0;
    uint32_t* tiles = nullptr;          // cnt, ovf_pos, ovf_n, group sums
    size_t tiles_cap = 0;
    uint16_t* sym_g = nullptr;          // scratch of words too long for a tile's LDS
    size_t sym_cap = 0;
    uint32_t* nx_g = nullptr;
    size_t nx_cap = 0;
    uint16_t* rk_g = nullptr;
    size_t rk_cap = 0;
    uint32_t* ovf = nullptr;
    size_t ovf_cap = 0;
    uint8_t* text_buf = nullptr;
    size_t text_cap = 0;
    uint32_t* tok_buf = nullptr;
    size_t tok_cap = 0;
    // word cache: key, position and record per slot
    unsigned long long* wc_key = nullptr;
    size_t wc_key_cap = 0;
    uint32_t* wc_pos = nullptr;
    size_t wc_pos_cap = 0;
    uint32_t* wc_rec = nullptr;
    size_t wc_rec_cap = 0;
    uint32_t wc_log2 = BPE_CACHE_AUTO, wc_key_bits = BPE_CACHE_KEY_BITS;
    uint32_t wc_call_log2 = 0;  // the size the current call runs with (0: none)
    int walk_grid = 0, copy_grid = 0, insert_grid = 0, fill_grid = 0, clear_grid = 0;
};

namespace {

// The walk runs one wave per workgroup on 1 KiB tiles: its phases are
// chained by barriers, and with one wave a barrier waits for nothing else
// (256 MiB corpus: 256 threads on 4 KiB tiles 1.00 ms per walk, 128 on 2
// KiB 0.92, 64 on 1 KiB 0.85). The insert pass keeps 256 threads on 4 KiB
// tiles (faster there: 0.30 ms against 0.35 with 64).
constexpr int ENC_TPB = 64;
constexpr int INS_TPB = 256;
constexpr int ENC_SCAN_TPB = 1024;
constexpr int ENC_COPY_TPB = 256;
constexpr int WC_FILL_TPB = 256;
// The insert pass takes every WC_SAMPLE-th of its tiles: frequent words
// occur in most tiles, a word missed falls back to the walk's own encoding,
// and on the 256 MiB corpus 2 measured best (1: 2.35 ms per run, 2: 2.11,
// 3: 2.16, 4: 2.25; wider strides miss more words than they save in
// inserts).
constexpr uint32_t WC_SAMPLE = 2;
constexpr uint32_t WC_AUTO_MAX_LOG2 = 22;  // automatic size: 2^22 slots at most (256 MiB of records)
constexpr uint32_t ENC_TILE = ENC_TPB * 16;
constexpr uint32_t INS_TILE = INS_TPB * 16;
constexpr uint32_t ENC_CAP = ENC_TILE + ENC_TPB * bpek::TRIE_HALO_PER_THREAD;
constexpr size_t ENC_SCRATCH_MAX = size_t(1) << 24;  // positions of long words per call

size_t enc_scratch_cap(size_t n) { return std::min(n, ENC_SCRATCH_MAX); }

// Slots of the word cache for n bytes (0: no cache). Automatic: none below
// 1 MiB (the walk is bound by launches there, and the cache's three kernels
// cost more than they save: 64 KiB, 0.094 ms without, 0.124 with); above,
// one slot per 256 input bytes, a power of two in [2^18, 2^22] (a table
// too small for a text's distinct words fills up: 16 MiB of Turkish-like
// text, 2^16 slots 0.86 ms, 2^18 0.61 ms; 256 MiB, 2^20 1.91 ms, 2^22 1.95).
uint32_t enc_wc_log2(const bpe_encoder* e, size_t n) {
    if (e->wc_log2 != BPE_CACHE_AUTO) return e->wc_log2;
    if (n < (size_t(1) << 20)) return 0;
    uint32_t l = 18;
    while (l < WC_AUTO_MAX_LOG2 && (size_t(1) << l) < n / 256) ++l;
    return l;
}

bpe_status enc_pools(bpe_encoder* e, size_t n) {
    const size_t ntiles = (n + ENC_TILE - 1) / ENC_TILE;
    const size_t sc = enc_scratch_cap(n);
    const size_t ngroups = (ntiles + bpek::ENC_GROUP - 1) / bpek::ENC_GROUP;
    bpe_status st = pool_grow(&e->slices, &e->slices_cap, ntiles * ENC_CAP, false);
    if (st == BPE_OK) st = pool_grow(&e->tiles, &e->tiles_cap, 3 * ntiles + ngroups, false);
    if (st == BPE_OK) st = pool_grow(&e->sym_g, &e->sym_cap, sc, false);
    if (st == BPE_OK) st = pool_grow(&e->nx_g, &e->nx_cap, sc, false);
    if (st == BPE_OK) st = pool_grow(&e->rk_g, &e->rk_cap, sc, false);
    if (st == BPE_OK) st = pool_grow(&e->ovf, &e->ovf_cap, sc, false);
    // the cache never decides a token: without memory for it, the call
    // runs without it
    uint32_t l = enc_wc_log2(e, n);
    if (st == BPE_OK && l) {
        const size_t slots = size_t(1) << l;
        bpe_status cs = pool_grow(&e->wc_key, &e->wc_key_cap, slots, false);
        if (cs == BPE_OK) cs = pool_grow(&e->wc_pos, &e->wc_pos_cap, slots, false);
        // records start zeroed (never filled) and are never cleared
        if (cs == BPE_OK) cs = pool_grow(&e->wc_rec, &e->wc_rec_cap, slots * bpek::WC_REC, true);
        if (cs != BPE_OK) {
            g_err.clear();
            l = 0;
        }
    }
    e->wc_call_log2 = l;
    return st;
}

// The passes of one call on stream s: status init, the word cache's clear,
// insert and fill (with a cache), the walk, the scan of the group sums and
// the copy of the tokens to dst (their total to status[0]). ev, if given,
// gets an event after the cache passes, the walk, the scan and the copy.
bpe_status enc_enqueue(bpe_encoder* e, const uint8_t* src, uint32_t n, uint32_t* dst, hipStream_t s,
                       hipEvent_t* ev) {
    const uint32_t ntiles = (n + ENC_TILE - 1) / ENC_TILE;
    const uint32_t ngroups = (ntiles + bpek::ENC_GROUP - 1) / bpek::ENC_GROUP;
    uint32_t* cnt = e->tiles;
    uint32_t* ovf_pos = cnt + ntiles;
    uint32_t* ovf_n = ovf_pos + ntiles;
    uint32_t* gsum = ovf_n + ntiles;
    const bpek::RankTable rt{e->rt, e->rt_mask, e->rt_probes, e->rt_bytes};
    const uint32_t l = e->wc_call_log2;  // set by enc_pools for this n
    bpek::WordCache wc{};
    hipLaunchKernelGGL(bpek::k_enc_init, dim3(std::min<uint32_t>((ngroups + 255) / 256, e->clear_grid)), dim3(256),
                       0, s, e->status, gsum, ngroups);
    if (l) {
        const uint32_t slots = 1u << l;
        wc = bpek::WordCache{e->wc_key, e->wc_pos, e->wc_rec, slots - 1,
                             e->wc_key_bits ? ~0u << (32 - e->wc_key_bits) : 0u};
        hipLaunchKernelGGL(bpek::k_wc_clear, dim3(std::min<uint32_t>((slots + 255) / 256, e->clear_grid)), dim3(256),
                           0, s, wc, slots);
        const uint32_t itiles = (n + INS_TILE - 1) / INS_TILE, stride = WC_SAMPLE;
        hipLaunchKernelGGL(bpek::k_wc_insert<INS_TPB>,
                           dim3(std::min<uint32_t>((itiles + stride - 1) / stride, e->insert_grid)), dim3(INS_TPB),
                           0, s, src, n, itiles, stride, wc);
        hipLaunchKernelGGL(bpek::k_wc_fill<WC_FILL_TPB>,
                           dim3(std::min<uint32_t>((slots + 4 * WC_FILL_TPB - 1) / (4 * WC_FILL_TPB), e->fill_grid)),
                           dim3(WC_FILL_TPB), 0, s, src, n, wc, rt, slots);
    }
    if (ev) HIP_TRY(hipEventRecord(ev[0], s));
    hipLaunchKernelGGL(bpek::k_enc_walk<ENC_TPB>, dim3(std::min<uint32_t>(ntiles, e->walk_grid)), dim3(ENC_TPB), 0,
                       s, src, n, rt, e->slices, cnt, ovf_pos, ovf_n, gsum, ntiles, e->sym_g, e->nx_g, e->rk_g,
                       e->ovf, e->status, uint32_t(enc_scratch_cap(n)), wc);
    if (ev) HIP_TRY(hipEventRecord(ev[1], s));
    hipLaunchKernelGGL(bpek::k_enc_gscan<ENC_SCAN_TPB>, dim3(1), dim3(ENC_SCAN_TPB), 0, s, gsum, ngroups, e->status);
    if (ev) HIP_TRY(hipEventRecord(ev[2], s));
    hipLaunchKernelGGL(bpek::k_enc_copy<ENC_COPY_TPB>, dim3(std::min<uint32_t>(ngroups, e->copy_grid)),
                       dim3(ENC_COPY_TPB), 0, s, e->slices, cnt, ovf_pos, ovf_n, gsum, e->ovf, dst, ntiles, ENC_CAP);
    if (ev) HIP_TRY(hipEventRecord(ev[3], s));
    HIP_TRY(hipGetLastError());
    return BPE_OK;
}

}  // namespace

extern "C" {

bpe_status bpe_encoder_build(const bpe_merge* merges, uint32_t n_merges, bpe_encoder** out) {
    g_err.clear();
    if (!out || (!merges && n_merges)) {
        set_err("out must be non-NULL, and merges non-NULL when n_merges > 0");
        return BPE_EINVAL;
    }
    *out = nullptr;
    if (n_merges > BPE_MAX_MERGES) {
        set_err("%u merges exceed the id space (%u merges)", n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    std::vector<bpe_merge> hm(n_merges);
    const bpe_status cst = copy_merges(merges, n_merges, hm.data());
    if (cst != BPE_OK) return cst;
    // rank table: pair -> first rank; open addressing at most half full
    size_t slots = 1024;
    while (slots < 2 * size_t(n_merges)) slots *= 2;
    std::vector<unsigned long long> table(slots, ~0ull);
    std::vector<uint16_t> byte_ranks(65536, uint16_t(bpek::RK_NONE));
    uint32_t probes = 1;
    for (uint32_t r = 0; r < n_merges; ++r) {
        const uint32_t l = hm[r].left, rr = hm[r].right, lim = bpek::BASE + r;
        if (l >= lim || rr >= lim) {
            set_err("merge %u (%u, %u) names an id that does not exist before it (ids < %u)", r, l, rr, lim);
            return BPE_EINVAL;
        }
        const uint32_t key = (l << 16) | rr;
        uint32_t h = bpek::mix32(key) & uint32_t(slots - 1), p = 0;
        bool dup = false;
        while (table[h] != ~0ull) {
            if (uint32_t(table[h] >> 32) == key) {
                dup = true;  // a repeat never occurs again after the first merge of the pair
                break;
            }
            h = (h + 1) & uint32_t(slots - 1);
            ++p;
        }
        if (dup) continue;
        table[h] = (static_cast<unsigned long long>(key) << 32) | r;
        probes = std::max(probes, p + 1);
        if (l < bpek::BASE && rr < bpek::BASE) byte_ranks[(l << 8) | rr] = uint16_t(r);
    }
    bpe_encoder* e = new (std::nothrow) bpe_encoder();
    if (!e) {
        set_err("out of host memory");
        return BPE_ENOMEM;
    }
    auto fail = [&](bpe_status st) {
        bpe_encoder_free(e);
        return st;
    };
    int cus = 0, per_cu = 0, per_cu_ins = 0, per_cu_fill = 0;
    if (hipGetDevice(&e->device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, e->device) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bpek::k_enc_walk<ENC_TPB>, ENC_TPB, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_ins, bpek::k_wc_insert<INS_TPB>, INS_TPB, 0) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_fill, bpek::k_wc_fill<WC_FILL_TPB>, WC_FILL_TPB, 0) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0 || per_cu_ins <= 0 || per_cu_fill <= 0) {
        (void)hipGetLastError();
        set_err("cannot query the device");
        return fail(BPE_EHIP);
    }
    e->walk_grid = cus * per_cu;
    e->insert_grid = cus * per_cu_ins;
    e->fill_grid = cus * per_cu_fill;
    e->clear_grid = cus * 8;
    e->copy_grid = cus * 16;
    e->rt_mask = uint32_t(slots - 1);
    e->rt_probes = probes;
    // blocking, as the trie's: ordered after the legacy default stream
    if (hipStreamCreate(&e->stream) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&e->rt), slots * sizeof(unsigned long long)) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&e->status), 4 * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&e->rt_bytes), 65536 * sizeof(uint16_t)) != hipSuccess ||
        hipMemcpy(e->rt, table.data(), slots * sizeof(unsigned long long), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(e->rt_bytes, byte_ranks.data(), 65536 * sizeof(uint16_t), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        set_err("allocating or uploading the rank table failed");
        return fail(BPE_ENOMEM);
    }
    *out = e;
    return BPE_OK;
}

bpe_status bpe_encoder_encode(bpe_encoder* e, const uint8_t* bytes, size_t n, void* stream, uint32_t* tokens,
                              size_t tokens_cap, size_t* n_tokens) {
    g_err.clear();
    if (!e || !n_tokens || (n && !bytes)) {
        set_err("encoder and n_tokens must be non-NULL, and bytes non-NULL when n > 0");
        return BPE_EINVAL;
    }
    if (n > BPE_MAX_BYTES) {
        set_err("n = %zu exceeds the limit of %llu bytes", n, (unsigned long long)BPE_MAX_BYTES);
        return BPE_EINVAL;
    }
    if (tokens && tokens_cap < n) {
        set_err("tokens_cap %zu is below n = %zu", tokens_cap, n);
        return BPE_EINVAL;
    }
    *n_tokens = 0;
    if (n == 0) return BPE_OK;
    HIP_TRY(hipSetDevice(e->device));
    hipStream_t s = stream ? reinterpret_cast<hipStream_t>(stream) : e->stream;
    bpe_status st = enc_pools(e, n);
    if (st != BPE_OK) return st;
    const uint8_t* src = bytes;
    if (!is_device_pointer(bytes)) {
        st = pool_grow(&e->text_buf, &e->text_cap, n, false);
        if (st != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(e->text_buf, bytes, n, hipMemcpyHostToDevice, s));
        src = e->text_buf;
    }
    uint32_t* dst = tokens;
    if (!tokens || !is_device_pointer(tokens)) {
        st = pool_grow(&e->tok_buf, &e->tok_cap, n, false);
        if (st != BPE_OK) return st;
        dst = e->tok_buf;
    }
    st = enc_enqueue(e, src, uint32_t(n), dst, s, nullptr);
    if (st != BPE_OK) return st;
    uint32_t h[4] = {0, 0, 0, 0};
    HIP_TRY(hipMemcpyAsync(h, e->status, sizeof h, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    if (h[1]) {
        set_err("words too long for the encoder's scratch (%zu positions per call)", enc_scratch_cap(n));
        return BPE_ENOMEM;
    }
    if (h[0] > n) {
        set_err("device reported %u tokens for %zu bytes", h[0], n);
        return BPE_ESTATE;
    }
    *n_tokens = h[0];
    if (tokens && dst != tokens) HIP_TRY(hipMemcpy(tokens, dst, sizeof(uint32_t) * size_t(h[0]), hipMemcpyDefault));
    return BPE_OK;
}

bpe_status bpe_encoder_profile(bpe_encoder* e, const uint8_t* bytes, size_t n, uint32_t reps, float* ms,
                               size_t* n_tokens) {
    g_err.clear();
    if (!e || !n_tokens || !bytes || n == 0 || reps == 0 || n > BPE_MAX_BYTES) {
        set_err("encoder, bytes and n_tokens must be non-NULL, 0 < n <= BPE_MAX_BYTES and reps > 0");
        return BPE_EINVAL;
    }
    HIP_TRY(hipSetDevice(e->device));
    if (!is_device_pointer(bytes)) {
        set_err("bpe_encoder_profile reads device bytes only");
        return BPE_EINVAL;
    }
    size_t first = 0;
    bpe_status st = bpe_encoder_encode(e, bytes, n, nullptr, nullptr, 0, &first);
    if (st != BPE_OK) return st;
    std::vector<hipEvent_t>* ev = nullptr;
    st = event_pool(e->device, 4 * size_t(reps) + 1, &ev);
    if (st != BPE_OK) return st;
    std::vector<hipEvent_t>& evs = *ev;
    HIP_TRY(hipEventRecord(evs[0], e->stream));
    for (uint32_t r = 0; r < reps; ++r) {
        st = enc_enqueue(e, bytes, uint32_t(n), e->tok_buf, e->stream, &evs[4 * size_t(r) + 1]);
        if (st != BPE_OK) return st;
    }
    uint32_t h[4] = {0, 0, 0, 0};
    HIP_TRY(hipMemcpyAsync(h, e->status, sizeof h, hipMemcpyDeviceToHost, e->stream));
    HIP_TRY(hipStreamSynchronize(e->stream));
    if (h[1] || h[0] != first) {
        set_err("repeated runs disagree (%u tokens vs %zu, error flags %u)", h[0], first, h[1]);
        return BPE_ESTATE;
    }
    for (size_t i = 0; i < 4 * size_t(reps); ++i) {
        float a = 0.f;
        HIP_TRY(hipEventElapsedTime(&a, evs[i], evs[i + 1]));
        if (ms) ms[i] = a;
    }
    *n_tokens = first;
    return BPE_OK;
}

bpe_status bpe_encoder_cache(bpe_encoder* e, uint32_t log2_slots, uint32_t key_bits) {
    g_err.clear();
    if (!e || !(log2_slots == BPE_CACHE_AUTO || log2_slots == 0 || (log2_slots >= 8 && log2_slots <= 24)) ||
        key_bits > BPE_CACHE_KEY_BITS) {
        set_err("encoder must be non-NULL, log2_slots BPE_CACHE_AUTO, 0 or 8..24, key_bits at most %u",
                BPE_CACHE_KEY_BITS);
        return BPE_EINVAL;
    }
    e->wc_log2 = log2_slots;
    e->wc_key_bits = key_bits;
    return BPE_OK;
}

void bpe_encoder_free(bpe_encoder* e) {
    if (!e) return;
    (void)hipSetDevice(e->device);
    if (e->stream) (void)hipStreamSynchronize(e->stream);
    for (void* p : {(void*)e->rt, (void*)e->rt_bytes, (void*)e->status, (void*)e->slices, (void*)e->tiles, (void*)e->sym_g,
                    (void*)e->nx_g, (void*)e->rk_g, (void*)e->ovf, (void*)e->text_buf, (void*)e->tok_buf,
                    (void*)e->wc_key, (void*)e->wc_pos, (void*)e->wc_rec})
        if (p) (void)hipFree(p);
    if (e->stream) (void)hipStreamDestroy(e->stream);
    delete e;
}

bpe_status bpe_encode(const uint8_t* bytes, size_t n, const bpe_merge* merges, uint32_t n_merges,
                      const bpe_config* cfg, uint32_t* tokens, size_t tokens_cap, size_t* n_tokens) {
    g_err.clear();
    if (!n_tokens || (!merges && n_merges) || (n && !bytes)) {
        set_err("bytes (when n > 0), merges (when n_merges > 0) and n_tokens must be non-NULL");
        return BPE_EINVAL;
    }
    if (n_merges > BPE_MAX_MERGES) {
        set_err("%u merges exceed the id space (%u merges)", n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    if (!config_ok(n, cfg)) return BPE_EINVAL;
    if (tokens && tokens_cap < n) {
        set_err("tokens_cap %zu is below n = %zu", tokens_cap, n);
        return BPE_EINVAL;
    }
    *n_tokens = 0;
    if (n == 0) return BPE_OK;
    bpe_encoder* e = nullptr;
    bpe_status st = bpe_encoder_build(merges, n_merges, &e);
    if (st != BPE_OK) return st;
    st = bpe_encoder_encode(e, bytes, n, cfg ? cfg->stream : nullptr, tokens, tokens_cap, n_tokens);
    bpe_encoder_free(e);
    return st;
}

}  // extern "C"

// ======================================================================== training over distinct words
// bpe_train_chunked: bpe_train's results from the corpus's distinct words,
// each once with its frequency (chunks.hpp). One call: the word passes, a
// host wait for the chunk sizes, the chunks, the weighted pair counts, one
// launch per iteration, and the tokens from the encoder. Where the chunks'
// records would take more than 16 bytes per input byte (bytes with almost
// no repeated word), bpe_train runs instead, unless BPE_FLAG_ALWAYS_CHUNKS
// is set.

namespace {

// Device buffers of one call, freed together.
struct DevBufs {
    std::vector<void*> p;
    template <typename T>
    bpe_status get(T** out, size_t count) {
        *out = nullptr;
        if (!count) count = 1;
        if (hipMalloc(reinterpret_cast<void**>(out), count * sizeof(T)) != hipSuccess) {
            (void)hipGetLastError();
            set_err("hipMalloc of %zu bytes failed", count * sizeof(T));
            return BPE_ENOMEM;
        }
        p.push_back(*out);
        return BPE_OK;
    }
    ~DevBufs() {
        for (void* q : p) (void)hipFree(q);
    }
};

constexpr int CK_TPB = 256;
constexpr int CK_LT = 2048;  // LDS sums per workgroup (slots, or pairs)
constexpr int CK_MERGE_TPB = 256;
constexpr uint32_t CK_TILE = CK_TPB * 16;  // k_ck_count's tile
constexpr int CK_SMALL_TPB = 1024;          // k_ck_small: at most this many record chunks, no long ones
constexpr int CK_SMALL_LT = 8192;           // its LDS pair table
constexpr int CK_SOLO_TPB = 1024;           // k_ck_solo: one workgroup, every iteration
constexpr int CK_SOLO_CT = 2048;            // its candidate table
constexpr int CK_SOLO_KT = 2048;            // its per-iteration change table

// Word-table slots for n bytes: one per 128 bytes, a power of two in
// [2^16, 2^24] (a word that finds no slot within the probe limit is kept
// as a chunk of its own, so the size only moves work, never a result).
uint32_t ck_table_log2(size_t n) {
    uint32_t l = 16;
    while (l < 24 && (size_t(1) << l) < n / 128) ++l;
    return l;
}

// The work of bpe_train_chunked on the device; *full set (and nothing
// else done) when the full-array path is to run instead.
bpe_status train_chunked(const uint8_t* bytes, size_t n, uint32_t n_merges, const bpe_config* cfg,
                         bpe_merge* merges, uint32_t* n_done, uint32_t* tokens, size_t tokens_cap,
                         size_t* n_tokens, bool* full) {
    int dev = 0, cus = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    DevBufs mem;  // released last, after the stream has drained
    hipStream_t s = cfg && cfg->stream ? reinterpret_cast<hipStream_t>(cfg->stream) : nullptr;
    hipStream_t own = nullptr;
    if (!s) {
        HIP_TRY(hipStreamCreate(&own));  // blocking: ordered after the legacy default stream
        s = own;
    }
    struct StreamGuard {
        hipStream_t s, own;
        ~StreamGuard() {
            (void)hipStreamSynchronize(s);
            if (own) (void)hipStreamDestroy(own);
        }
    } guard{s, own};
    bpe_status st = BPE_OK;
    auto launch_ok = [&]() -> bpe_status {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            set_err("kernel launch failed: %s", hipGetErrorString(e));
            return BPE_EHIP;
        }
        return BPE_OK;
    };
    const bool always = cfg && (cfg->flags & BPE_FLAG_ALWAYS_CHUNKS);

    // the corpus on the device
    const uint8_t* text = bytes;
    if (!is_device_pointer(bytes)) {
        uint8_t* t = nullptr;
        if ((st = mem.get(&t, n)) != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(t, bytes, n, hipMemcpyHostToDevice, s));
        text = t;
    }

    // ---- the distinct words and their counts
    const uint32_t wl = ck_table_log2(n), slots = 1u << wl;
    unsigned long long* wkey = nullptr;
    uint32_t *wpos = nullptr, *wrec = nullptr, *wcnt = nullptr, *lpos = nullptr, *llen = nullptr, *small = nullptr;
    size_t lcap = n / 64 + 1024;  // listed words kept; the count runs again with room for all when more
    if ((st = mem.get(&wkey, slots)) != BPE_OK || (st = mem.get(&wpos, slots)) != BPE_OK ||
        (st = mem.get(&wrec, size_t(slots) * 8)) != BPE_OK || (st = mem.get(&wcnt, slots)) != BPE_OK ||
        (st = mem.get(&lpos, lcap)) != BPE_OK || (st = mem.get(&llen, lcap)) != BPE_OK ||
        (st = mem.get(&small, 16)) != BPE_OK)
        return st;
    const bpek::WordCache wc{wkey, wpos, wrec, slots - 1u, ~0u};  // 8 u32 of bytes per record here
    const uint32_t ins_tiles = uint32_t((n + INS_TILE - 1) / INS_TILE);
    const uint32_t ck_tiles = uint32_t((n + CK_TILE - 1) / CK_TILE);
    const uint32_t sgrid = std::min<uint32_t>((slots + 255) / 256, cus * 8);
    hipLaunchKernelGGL(bpek::k_wc_clear, dim3(sgrid), dim3(256), 0, s, wc, slots);
    hipLaunchKernelGGL(bpek::k_wc_insert<INS_TPB>, dim3(std::min<uint32_t>(ins_tiles, cus * 8)), dim3(INS_TPB), 0, s,
                       text, uint32_t(n), ins_tiles, 1u, wc);
    hipLaunchKernelGGL(bpek::k_ck_record, dim3(sgrid), dim3(256), 0, s, text, uint32_t(n), wc, slots);
    // small: [0] the table's chunks, [2..4] listed words (all, long ones,
    // their bytes), [8..10] the build's counters
    uint32_t h[5] = {0, 0, 0, 0, 0};
    for (;;) {
        const bpek::CkList list{lpos, llen, small + 2, uint32_t(lcap)};
        hipLaunchKernelGGL(bpek::k_fill64, dim3(sgrid), dim3(256), 0, s, reinterpret_cast<unsigned long long*>(wcnt),
                           size_t(slots / 2), 0ull);
        hipLaunchKernelGGL(bpek::k_fill64, dim3(1), dim3(64), 0, s, reinterpret_cast<unsigned long long*>(small),
                           size_t(8), 0ull);
        hipLaunchKernelGGL((bpek::k_ck_count<CK_TPB, CK_LT>), dim3(std::min<uint32_t>(ck_tiles, cus * 4)),
                           dim3(CK_TPB), 0, s, text, uint32_t(n), ck_tiles, wc, wcnt, list);
        hipLaunchKernelGGL(bpek::k_ck_size<256>, dim3(sgrid), dim3(256), 0, s, wcnt, slots, small);
        if ((st = launch_ok()) != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(h, small, sizeof h, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        // records of 64 bytes, long chunks' 16-bit symbols: a bound on their
        // memory against the corpus (an iteration reads 8 bytes of filter
        // per record and the records that hold the merged pair, the full
        // array's pass 4 bytes per symbol: the chunks win where the records
        // are fewer than about one per 8 bytes)
        const size_t n_rec = size_t(h[0]) + (h[2] - h[3]);
        if (!always && 64 * n_rec + 2 * size_t(h[4]) > 8 * n) {
            *full = true;
            return BPE_OK;
        }
        if (h[2] <= lcap) break;
        lcap = h[2];  // the same words again: the count is exact
        if ((st = mem.get(&lpos, lcap)) != BPE_OK || (st = mem.get(&llen, lcap)) != BPE_OK) return st;
    }
    const bpek::CkList list{lpos, llen, small + 2, uint32_t(lcap)};
    const uint32_t n_list = h[2];
    bpek::Chunks ck{};
    ck.nr = h[0] + (h[2] - h[3]);
    ck.nl = h[3];
    if ((st = mem.get(&ck.rec, 4 * size_t(ck.nr))) != BPE_OK || (st = mem.get(&ck.rlen, ck.nr)) != BPE_OK ||
        (st = mem.get(&ck.rw, ck.nr)) != BPE_OK || (st = mem.get(&ck.rbloom, ck.nr)) != BPE_OK || (st = mem.get(&ck.lsym, h[4])) != BPE_OK ||
        (st = mem.get(&ck.loff, ck.nl)) != BPE_OK || (st = mem.get(&ck.llen, ck.nl)) != BPE_OK)
        return st;
    hipLaunchKernelGGL(bpek::k_fill64, dim3(1), dim3(64), 0, s, reinterpret_cast<unsigned long long*>(small + 8),
                       size_t(2), 0ull);
    hipLaunchKernelGGL(bpek::k_ck_build<256>, dim3(sgrid), dim3(256), 0, s, text, wc, wcnt, slots, list, n_list, ck,
                       small + 8);
    if ((st = launch_ok()) != BPE_OK) return st;

    // ---- training state: control block, selection state, pair table, merges
    const uint32_t tlog2 = table_log2_for(n, cfg, n_merges);
    const size_t tslots = size_t(1) << tlog2;
    Ctl* ctl = nullptr;
    bpek::Sweep* sw = nullptr;
    unsigned long long* table = nullptr;
    uint32_t *dmerges = nullptr, *lengths = nullptr;
    if ((st = mem.get(&ctl, 1)) != BPE_OK || (st = mem.get(&sw, 1)) != BPE_OK ||
        (st = mem.get(&table, tslots)) != BPE_OK || (st = mem.get(&dmerges, 3 * size_t(BPE_MAX_MERGES))) != BPE_OK ||
        (st = mem.get(&lengths, 2)) != BPE_OK)
        return st;
    const bpek::GTable gt{table, uint32_t(tslots - 1), table_limit(tlog2)};
    Ctl hc;
    bool small_done = false;
    if (ck.nr <= uint32_t(CK_SMALL_TPB) && ck.nl == 0 && n_merges > 0) {
        // every iteration in one workgroup and one launch; its LDS table
        // may fill, and then the workgroups below train instead
        hipLaunchKernelGGL(bpek::k_init_ctl, dim3(1), dim3(64), 0, s, ctl, uint32_t(n), lengths);
        hipLaunchKernelGGL((bpek::k_ck_small<CK_SMALL_TPB, CK_SMALL_LT>), dim3(1), dim3(CK_SMALL_TPB), 0, s, ck,
                           n_merges, dmerges, ctl);
        if ((st = launch_ok()) != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(&hc, ctl, sizeof hc, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        small_done = !(hc.err & bpek::ERR_LDS_FULL);
    }
    if (!small_done && ck.nl == 0 && n_merges > 0) {
        // one workgroup, every iteration, with occurrence lists: the
        // weighted counts into the pair table, each pair's list of chunks
        const bpek::OccLists ol0{};
        bpek::OccLists ol = ol0;
        bpek::PairIds pid{};
        uint2* scratch = nullptr;
        ol.cap = uint32_t(std::min<size_t>(64 * size_t(ck.nr) + 4096, 0xFFFFFFF0u));
        const uint32_t scratch_cap = uint32_t(std::min<size_t>(2 * size_t(ck.nr) + 65536, 0xFFFFFFF0u));
        if ((st = mem.get(&ol.off, tslots)) != BPE_OK || (st = mem.get(&ol.len, tslots)) != BPE_OK ||
            (st = mem.get(&ol.pool, ol.cap)) != BPE_OK || (st = mem.get(&pid.slot, tslots)) != BPE_OK ||
            (st = mem.get(&pid.key, tslots)) != BPE_OK || (st = mem.get(&pid.cnt, tslots)) != BPE_OK ||
            (st = mem.get(&pid.id_of, tslots)) != BPE_OK || (st = mem.get(&scratch, scratch_cap)) != BPE_OK)
            return st;
        hipLaunchKernelGGL(bpek::k_init_ctl, dim3(1), dim3(64), 0, s, ctl, uint32_t(n), lengths);
        hipLaunchKernelGGL(bpek::k_fill64, dim3(cus * 4), dim3(256), 0, s, table, tslots, bpek::GT_EMPTY);
        hipLaunchKernelGGL(bpek::k_fill64, dim3(cus * 4), dim3(256), 0, s, reinterpret_cast<unsigned long long*>(ol.len),
                           tslots / 2, 0ull);
        hipLaunchKernelGGL(bpek::k_fill64, dim3(1), dim3(64), 0, s, reinterpret_cast<unsigned long long*>(small + 12),
                           size_t(1), 0ull);
        const uint32_t pgrid = std::max<uint32_t>(1, std::min<uint32_t>((ck.nr + 255) / 256, cus * 4));
        hipLaunchKernelGGL((bpek::k_ck_pairs<CK_MERGE_TPB, CK_LT>), dim3(pgrid), dim3(CK_MERGE_TPB), 0, s, ck, gt, ctl);
        hipLaunchKernelGGL((bpek::k_occ_scan<256, false>), dim3(pgrid), dim3(256), 0, s, ck, gt, ol);
        hipLaunchKernelGGL(bpek::k_occ_place<256>, dim3(std::min<uint32_t>(uint32_t((tslots + 255) / 256), cus * 8)),
                           dim3(256), 0, s, gt, ol, pid, small + 12);
        hipLaunchKernelGGL((bpek::k_occ_scan<256, true>), dim3(pgrid), dim3(256), 0, s, ck, gt, ol);
        hipLaunchKernelGGL((bpek::k_ck_solo<CK_SOLO_TPB, CK_SOLO_CT, CK_SOLO_KT>), dim3(1), dim3(CK_SOLO_TPB), 0, s,
                           ck, gt, ol, small + 12, pid, small + 13, scratch, scratch_cap, n_merges, dmerges, ctl);
        if ((st = launch_ok()) != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(&hc, ctl, sizeof hc, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        small_done = !(hc.err & bpek::ERR_SOLO);
        if (!small_done) {
            // the records were rewritten: built again for the passes below
            hipLaunchKernelGGL(bpek::k_fill64, dim3(1), dim3(64), 0, s,
                               reinterpret_cast<unsigned long long*>(small + 8), size_t(2), 0ull);
            hipLaunchKernelGGL(bpek::k_ck_build<256>, dim3(sgrid), dim3(256), 0, s, text, wc, wcnt, slots, list,
                               n_list, ck, small + 8);
            if ((st = launch_ok()) != BPE_OK) return st;
        }
    }
    if (!small_done) {
        hipLaunchKernelGGL(bpek::k_fill64, dim3(4), dim3(256), 0, s, reinterpret_cast<unsigned long long*>(sw),
                           sizeof(bpek::Sweep) / 8, 0ull);
        hipLaunchKernelGGL(bpek::k_init_ctl, dim3(1), dim3(64), 0, s, ctl, uint32_t(n), lengths);
        hipLaunchKernelGGL(bpek::k_fill64, dim3(cus * 4), dim3(256), 0, s, table, tslots, bpek::GT_EMPTY);
        // one workgroup per CU: more only add to the selection's wait and the
        // publication's polls (each thread has CK_PF records in flight anyway)
        const uint32_t nmax = std::max(ck.nr, ck.nl);
        const uint32_t grid = std::max<uint32_t>(1, std::min<uint32_t>((nmax + CK_MERGE_TPB - 1) / CK_MERGE_TPB, cus));
        hipLaunchKernelGGL((bpek::k_ck_pairs<CK_MERGE_TPB, CK_LT>), dim3(grid), dim3(CK_MERGE_TPB), 0, s, ck, gt, ctl);
        for (uint32_t it = 0; it < n_merges; ++it)
            hipLaunchKernelGGL((bpek::k_ck_merge<CK_MERGE_TPB, CK_LT>), dim3(grid), dim3(CK_MERGE_TPB), 0, s, it, ctl,
                               ck, gt, sw, dmerges);
        if ((st = launch_ok()) != BPE_OK) return st;
        HIP_TRY(hipMemcpyAsync(&hc, ctl, sizeof hc, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
    }
    if (hc.err) {
        if (hc.err & bpek::ERR_TABLE) {
            set_err("the global pair table is full (%u of %zu slots claimed; give a larger table_log2)",
                    table_limit(tlog2), tslots);
            return BPE_ETABLE;
        }
        set_err("device error bits 0x%x", hc.err);
        return BPE_ESTATE;
    }
    const uint32_t done = hc.k;
    if (done) HIP_TRY(hipMemcpy(merges, dmerges, sizeof(bpe_merge) * done, hipMemcpyDefault));
    *n_done = done;
    // ---- the tokens: the learned list applied to its own training text
    if (tokens || n_tokens) {
        size_t nt = 0;
        bpe_encoder* e = nullptr;
        std::vector<bpe_merge> hm(done);
        if (done) HIP_TRY(hipMemcpy(hm.data(), dmerges, sizeof(bpe_merge) * done, hipMemcpyDeviceToHost));
        st = bpe_encoder_build(hm.data(), done, &e);
        if (st != BPE_OK) return st;
        st = bpe_encoder_encode(e, text, n, s, tokens, tokens ? tokens_cap : 0, &nt);
        bpe_encoder_free(e);
        if (st != BPE_OK) return st;
        if (n_tokens) *n_tokens = nt;
    }
    return BPE_OK;
}

}  // namespace

extern "C" {

bpe_status bpe_train_chunked(const uint8_t* bytes, size_t n, uint32_t n_merges, const bpe_config* cfg,
                             bpe_merge* merges, uint32_t* n_done, uint32_t* tokens, size_t tokens_cap,
                             size_t* n_tokens) {
    g_err.clear();
    if (!n_done || (!merges && n_merges) || (n && !bytes)) {
        set_err("bytes (when n > 0), merges (when n_merges > 0) and n_done must be non-NULL");
        return BPE_EINVAL;
    }
    if (n_merges > BPE_MAX_MERGES) {
        set_err("%u merges exceed the id space (%u merges)", n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    if (!config_ok(n, cfg)) return BPE_EINVAL;
    if (cfg && cfg->workspace) {
        set_err("bpe_train_chunked allocates its own memory (bpe_config.workspace must be NULL)");
        return BPE_EINVAL;
    }
    if (tokens && tokens_cap < n) {
        set_err("tokens_cap %zu is below n = %zu", tokens_cap, n);
        return BPE_EINVAL;
    }
    *n_done = 0;
    if (n_tokens) *n_tokens = 0;
    if (n == 0) return BPE_OK;
    bool full = false;
    const bpe_status st = train_chunked(bytes, n, n_merges, cfg, merges, n_done, tokens, tokens_cap, n_tokens, &full);
    if (st != BPE_OK || !full) return st;
    // the chunk buffers are freed: the full-array path, same results
    return bpe_train(bytes, n, n_merges, cfg, merges, n_done, tokens, tokens_cap, n_tokens);
}

}  // extern "C"
