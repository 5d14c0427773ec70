// Host driver and C ABI of the BPE training library (include/bpe.h).
//
// The whole merge loop is enqueued on one stream with no host round trip
// between iterations: each iteration is a sweep of the global pair table
// for the maximum (k_find_max) followed by the fused merge / compaction /
// count-update pass (k_merge); both read the iteration
// number, the merge and the sequence length from the device control block,
// and do nothing once training has stopped. The host reads back a few bytes
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
#include <utility>
#include <vector>

#include "../../include/bpe.h"
#include "kernels.hpp"
#include "merge.hpp"

using bpek::Ctl;

namespace {

// launch shapes
constexpr int MERGE_TPB = 512;
constexpr int MERGE_LT = 1024;             // LDS slots for count changes, per workgroup
constexpr int TILE = MERGE_TPB * 16;       // symbols per scan tile (16 per thread)
constexpr int TAG_TPB = 256;
constexpr int TAG_LT = 4096;
constexpr int FIND_TPB = 256;
constexpr int FIND_U = 8;                  // 16-byte loads in flight per sweep thread

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

uint32_t table_log2_for(size_t n, const bpe_config* cfg) {
    if (cfg && cfg->table_log2) return cfg->table_log2;
    uint32_t l = ceil_log2(n ? n : 1) + 1;
    return std::min<uint32_t>(22, std::max<uint32_t>(12, l));
}

// Workgroups of the merge and tag passes: enough to fill the chip, never
// more than there are tiles to hand out.
size_t grid_bound(size_t n) { return (n + TILE - 1) / TILE + 1; }

// The global table counts as full at 7/8 load (linear probing stays short).
uint32_t table_limit(uint32_t tlog2) { return uint32_t((1ull << tlog2) - (1ull << tlog2) / 8); }

struct Layout {
    size_t ctl, sweep, sym0, sym1, table, status, merges, lengths, fpairs, total;
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
    L.sym0 = a;
    a = align_up(a + 4 * sym_elems, 256);
    L.sym1 = a;
    a = align_up(a + 4 * sym_elems, 256);
    L.table = a;
    a = align_up(a + 8 * (size_t(1) << tlog2), 256);
    // at least 512 words: the look-back copies a 512-word window from index 0
    L.max_tiles = std::max<uint32_t>(uint32_t((n + TILE - 1) / TILE) + 1, 512);
    L.status = a;
    a = align_up(a + 8 * size_t(L.max_tiles), 256);
    L.merges = a;
    a = align_up(a + 12 * size_t(BPE_MAX_MERGES), 256);
    L.lengths = a;
    a = align_up(a + 4 * (size_t(BPE_MAX_MERGES) + 1), 256);
    L.fpairs = a;  // pairs of replayed iterations, indexed by iteration
    a = align_up(a + 8 * size_t(BPE_MAX_MERGES), 256);
    L.total = a;
    return L;
}

bool config_ok(size_t n, const bpe_config* cfg) {
    if (n > BPE_MAX_BYTES) {
        set_err("n = %zu exceeds the limit of %llu bytes", n, (unsigned long long)BPE_MAX_BYTES);
        return false;
    }
    if (cfg) {
        if (cfg->flags != 0) {
            set_err("bpe_config.flags must be 0");
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
    void* ws = nullptr;
    bool own_ws = false;
    size_t n = 0;
    uint32_t tlog2 = 0;
    Layout lay{};
    Ctl* ctl = nullptr;
    bpek::Sweep* sweep = nullptr;
    uint32_t* sym0 = nullptr;
    uint32_t* sym1 = nullptr;
    unsigned long long* table = nullptr;
    unsigned long long* status = nullptr;
    uint32_t* merges = nullptr;
    uint32_t* lengths = nullptr;
    uint32_t* fpairs = nullptr;
    uint32_t requested = 0;  // iterations enqueued so far
    int merge_grid = 0, tag_grid = 0, fill_grid = 0, find_grid = 0;
    bool poisoned = false;   // a device error was seen

    uint32_t slots() const { return 1u << tlog2; }
    bpek::GTable gtable() const { return bpek::GTable{table, slots() - 1u, table_limit(tlog2)}; }
};

namespace {

void launch_find_max(bpe_state* s) {
    hipLaunchKernelGGL((bpek::k_find_max<FIND_TPB, FIND_U>), dim3(s->find_grid), dim3(FIND_TPB), 0, s->stream,
                       s->ctl, s->table, s->slots(), s->sweep);
}

void launch_merge(bpe_state* s) {
    hipLaunchKernelGGL((bpek::k_merge<MERGE_TPB, MERGE_LT>), dim3(s->merge_grid), dim3(MERGE_TPB), 0, s->stream,
                       s->ctl, s->sym0, s->sym1, s->gtable(), s->status, s->lengths, s->sweep,
                       uint32_t(s->find_grid), s->merges);
}

void launch_force(bpe_state* s) {
    hipLaunchKernelGGL(bpek::k_force, dim3(1), dim3(bpek::FORCE_TPB), 0, s->stream, s->ctl, s->gtable(), s->sweep, s->fpairs,
                       uint32_t(s->find_grid));
}

bpe_status launch_iteration(bpe_state* s) {
    launch_find_max(s);
    launch_merge(s);
    return BPE_OK;
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

bpe_status enqueue_run(bpe_state* s, uint32_t n_merges) {
    if (size_t(s->requested) + n_merges > BPE_MAX_MERGES) {
        set_err("%u + %u merges exceed the id space (%u merges)", s->requested, n_merges, BPE_MAX_MERGES);
        return BPE_EIDSPACE;
    }
    s->requested += n_merges;
    hipLaunchKernelGGL(bpek::k_set_limit, dim3(1), dim3(64), 0, s->stream, s->ctl, s->requested);
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
    const uint32_t tlog2 = table_log2_for(n, cfg);
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
    auto fail = [&](bpe_status st) {
        bpe_free(s);
        return st;
    };
    hipError_t e = hipGetDevice(&s->device);
    if (e != hipSuccess) {
        set_err("hipGetDevice failed: %s", hipGetErrorString(e));
        return fail(BPE_EHIP);
    }
    s->n = n;
    s->tlog2 = tlog2;
    s->lay = lay;
    if (cfg && cfg->stream) {
        s->stream = static_cast<hipStream_t>(cfg->stream);
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
    s->sym0 = reinterpret_cast<uint32_t*>(base + lay.sym0);
    s->sym1 = reinterpret_cast<uint32_t*>(base + lay.sym1);
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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bpek::k_merge<MERGE_TPB, MERGE_LT>,
                                                     MERGE_TPB, 0);
    if (e != hipSuccess || per_cu <= 0) per_cu = 1;
    s->merge_grid = int(std::min<size_t>(size_t(cus) * per_cu, grid_bound(n)));
    s->tag_grid = int(std::min<size_t>(size_t(cus) * 2, grid_bound(n)));
    s->fill_grid = cus * 4;
    // four sweep workgroups per CU (one round of loads each on the largest
    // default table), fewer for small tables; each merge workgroup reads
    // every sweep workgroup's maximum
    s->find_grid = int(std::min<size_t>(std::min<size_t>(size_t(cus) * 4, bpek::SWEEP_MAX_BLOCKS),
                                        std::max<size_t>(1, s->slots() / 2 / (FIND_TPB * FIND_U))));

    // input bytes: device memory is read in place, host memory is uploaded
    // into the second symbol buffer first (4n bytes hold n bytes)
    const uint8_t* src = bytes;
    if (!is_device_pointer(bytes)) {
        e = hipMemcpyAsync(s->sym1, bytes, n, hipMemcpyHostToDevice, s->stream);
        if (e != hipSuccess) {
            set_err("upload of the corpus failed: %s", hipGetErrorString(e));
            return fail(BPE_EHIP);
        }
        src = reinterpret_cast<const uint8_t*>(s->sym1);
    }
    hipLaunchKernelGGL(bpek::k_init_ctl, dim3(1), dim3(64), 0, s->stream, s->ctl, uint32_t(n), s->lengths);
    hipLaunchKernelGGL(bpek::k_fill64, dim3(4), dim3(256), 0, s->stream,
                       reinterpret_cast<unsigned long long*>(s->sweep), sizeof(bpek::Sweep) / 8, 0ull);
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
    *out = s;
    return BPE_OK;
}

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
    bpe_status st = enqueue_run(s, n_merges);
    if (st != BPE_OK) return st;
    for (uint32_t i = 0; i < n_merges; ++i) launch_iteration(s);
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
    hipLaunchKernelGGL(bpek::k_set_limit, dim3(1), dim3(64), 0, s->stream, s->ctl, s->requested);
    launch_iteration(s);
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
    const uint32_t* src = (h.m & 1u) ? s->sym1 : s->sym0;
    if (len) HIP_TRY(hipMemcpy(out, src, 4 * len, hipMemcpyDefault));
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

bpe_status bpe_profile(bpe_state* s, uint32_t n_merges, bpe_profile_result* res, float* find_ms,
                       float* merge_ms) {
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
    bpe_status st = event_pool(s->device, 2 * size_t(n_merges) + 1, &ev);
    if (st != BPE_OK) return st;
    st = enqueue_run(s, n_merges);
    if (st != BPE_OK) return st;
    std::vector<hipEvent_t>& e = *ev;
    HIP_TRY(hipEventRecord(e[0], s->stream));
    for (uint32_t i = 0; i < n_merges; ++i) {
        launch_find_max(s);
        HIP_TRY(hipEventRecord(e[2 * size_t(i) + 1], s->stream));
        launch_merge(s);
        HIP_TRY(hipEventRecord(e[2 * size_t(i) + 2], s->stream));
    }
    HIP_TRY(hipGetLastError());
    HIP_TRY(hipEventSynchronize(e[2 * size_t(n_merges)]));
    for (uint32_t i = 0; i < n_merges; ++i) {
        float a = 0.f, c = 0.f;
        HIP_TRY(hipEventElapsedTime(&a, e[2 * size_t(i)], e[2 * size_t(i) + 1]));
        HIP_TRY(hipEventElapsedTime(&c, e[2 * size_t(i) + 1], e[2 * size_t(i) + 2]));
        res->find_max_ms += a;
        res->merge_ms += c;
        if (find_ms) find_ms[i] = a;
        if (merge_ms) merge_ms[i] = c;
    }
    res->launches = n_merges;
    Ctl h;
    st = read_ctl(s, &h);
    res->merges_done = h.k;
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
    hipLaunchKernelGGL(bpek::k_set_limit, dim3(1), dim3(64), 0, s->stream, s->ctl, s->requested);
    for (uint32_t i = 0; i < k; ++i) {
        launch_force(s);
        launch_merge(s);
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
    (void)hipSetDevice(s->device);
    if (s->stream) (void)hipStreamSynchronize(s->stream);
    if (s->own_ws && s->ws) (void)hipFree(s->ws);
    if (s->own_stream && s->stream) (void)hipStreamDestroy(s->stream);
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
    bpe_status st = bpe_init(bytes, n, cfg, &s);
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
    bpe_state* s = nullptr;
    bpe_status st = bpe_init(bytes, n, cfg, &s);
    if (st != BPE_OK) return st;
    st = bpe_replay(s, merges, n_merges);
    if (st == BPE_OK) st = bpe_tokens(s, tokens, tokens ? tokens_cap : 0, n_tokens);
    bpe_free(s);
    return st;
}

}  // extern "C"
