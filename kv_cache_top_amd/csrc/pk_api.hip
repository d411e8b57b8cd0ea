// Host side of the C ABI: validation, ownership, the window mirror and launch
// sequencing.  Every step of the decode path runs in the HIP kernels; this
// file only decides sizes and launches them in stream order.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "pariskv.h"
#include "pk_device.hpp"
#include "pk_launch.hpp"

using pk::CodeTables;

struct pk_ctx {
    pk_config cfg;
    int batch = 0, n_kv = 0, n_q = 0, G = 0, units = 0;
    int64_t cap = 0;
    pk_dtype dt = PK_BF16;
    void* K = nullptr;
    void* V = nullptr;
    pk_mem mem = PK_MEM_DEVICE;
    int device = 0;
    float* scratch = nullptr;     // this device's address of the no-allocation scratch array
    CodeTables tab{};
    // window mirror (identical for every unit)
    bool prefilled = false;
    int64_t n = 0, sink_end = 0, r_end = 0, buf = 0;
    // sizes
    int nbins = 0, hstride = 0, max_chunks = 0, max_splits = 0;
    int64_t cmax = 0, sstride = 0;
    // device buffers
    uint8_t* ids = nullptr;       // [units][cap][16]   bucket ids
    uint8_t* rec = nullptr;       // [units][cap][128]  nibbles + w
    uint8_t* lut = nullptr;       // [units][16][256]   vote table
    float* ysum = nullptr;        // [units][128]       sum of rotated queries
    uint8_t* scores = nullptr;    // [units][sstride] + pad   min(coarse score, 255) (retrieval offset)
    uint16_t* hist = nullptr;     // [units][max_chunks][hstride] per-chunk #{score >= s}
    uint32_t* tot = nullptr;      // [units][nbins rounded up to even]  unit score histograms:
                                  // the scan adds into it, the rerank reads it, and the
                                  // fine selection zeroes it for the next step
    int32_t* meta = nullptr;      // [units][4]          {T, ties taken, C, k_eff}
    int32_t* cand_pos = nullptr;  // [units][cmax]
    float* cand_est = nullptr;    // [units][cmax]
    float* part = nullptr;        // [units][max_splits][G][130]
    float* dense_part = nullptr;  // partials of pk_dense_attend, allocated on its first use
    size_t dense_bytes = 0;
    float* cents = nullptr;       // [units][16][256][8] learned centroids (pk_fit_centroids), else
                                  // null: the analytic sign-pattern centroids
    long long* km_sums = nullptr; // [units][16][256][8] fixed-point sums of the fit
    pk::HotRing ring;             // device rows of the hot zone (host-memory stores only)
    // optional per-stage timing
    bool profiling = false;
    struct Mark {
        int stage;
        hipEvent_t a, b;
    };
    std::vector<Mark> marks;
    std::vector<hipEvent_t> event_pool;
};

// Scratch of pk_dense_attend_noalloc: the split partials of the dense
// attention, in a file-scope device array instead of memory allocated per
// call.  Every GPU the library runs on holds its own copy until the process
// ends; calls on one GPU share it.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace pk {
LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}
}  // namespace pk

namespace {

bool g_verbose = std::getenv("PK_VERBOSE") != nullptr;

// Device address of `scratch` on each device, looked up once per device with
// that device current (the host-side name of the array is not a device
// address).  nullptr until looked up.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int dev, float** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// A failed runtime call also sets the calling thread's last-error state; it is
// reported through the returned status and then cleared, so that the
// caller's next error check of its own work does not pick it up.
pk_status hip_fail(hipError_t e, const char* what) {
    if (g_verbose) std::fprintf(stderr, "pariskv: %s: %s\n", what, hipGetErrorString(e));
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? PK_ERR_OOM : PK_ERR_HIP;
}

pk_status alloc_fail() {
    (void)hipGetLastError();
    return PK_ERR_OOM;
}

pk_status runtime_fail(pk_status s = PK_ERR_HIP) {
    (void)hipGetLastError();
    return s;
}

#define PK_HIP(call)                                      \
    do {                                                  \
        hipError_t e_ = (call);                           \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// every device pointer an entry point receives must be 16-byte aligned (the
// kernels read and write them with 16-byte vector accesses)
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

hipEvent_t take_event(pk_ctx* c) {
    if (!c->event_pool.empty()) {
        hipEvent_t e = c->event_pool.back();
        c->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Times the next launch when profiling is on: the event pair is recorded by
// the kernel dispatch itself (begin and end of the kernel), so the duration
// excludes launch overheads between kernels.
struct StageTimer {
    pk_ctx* c;
    int stage;
    hipEvent_t a = nullptr, b = nullptr;
    StageTimer(pk_ctx* c_, int stage_, hipStream_t) : c(c_), stage(stage_) {
        if (!c->profiling) return;
        a = take_event(c);
        b = a ? take_event(c) : nullptr;
        if (!b) {
            if (a) c->event_pool.push_back(a);
            a = nullptr;
            return;
        }
        pk::launch_timing() = {a, b};
    }
    ~StageTimer() {
        if (!a) return;
        if (pk::launch_timing().start == a) {  // nothing was launched
            pk::launch_timing() = {};
            c->event_pool.push_back(a);
            c->event_pool.push_back(b);
            return;
        }
        c->marks.push_back({stage, a, b});
    }
};

int64_t coarse_count(int64_t n_r, int permille, int top_k) {
    const int64_t frac = ceil_div((int64_t)permille * n_r, 1000);
    int64_t c = frac > top_k ? frac : top_k;
    return c < n_r ? c : n_r;
}

// Chunk of retrieval-zone keys per scan/rerank block: the smallest power of
// two in [256, 8192] that keeps the grid at <= 2048 blocks.
int choose_chunk(int units, int64_t n_r) {
    int chunk = 256;
    while (chunk < 8192 && (int64_t)units * ceil_div(n_r, chunk) > 2048) chunk *= 2;
    return chunk;
}

size_t dtype_size(pk_dtype d) { return d == PK_F32 ? 4 : 2; }

void release_events(pk_ctx* c) {
    for (auto& m : c->marks) {
        c->event_pool.push_back(m.a);
        c->event_pool.push_back(m.b);
    }
    c->marks.clear();
}

void free_all(pk_ctx* c) {
    release_events(c);
    for (hipEvent_t e : c->event_pool) (void)hipEventDestroy(e);
    c->event_pool.clear();
    void* bufs[] = {c->ids,  c->rec,      c->lut,      c->ysum, c->scores, c->hist,   c->tot,
                    c->meta, c->cand_pos, c->cand_est, c->part, c->ring.k, c->ring.v,
                    c->dense_part, c->cents, c->km_sums};
    for (void* p : bufs)
        if (p) (void)hipFree(p);
}

// attention splits: the hot tokens (at most sink + local + buffer) and the
// selection are split separately
size_t rec_bytes(int sub_dim) {
    return sub_dim == 4    ? (size_t)pk::rec_bytes<4>()
           : sub_dim == 16 ? (size_t)pk::rec_bytes<16>()
                           : (size_t)pk::rec_bytes<8>();
}

// vote table bytes per unit: byte rows (m = 4, 8) or hash tables (m = 16)
size_t lut_bytes(int sub_dim) {
    return sub_dim == 16 ? (size_t)pk::lut_bytes<16>() : (size_t)pk::lut_bytes<8>();
}

int64_t max_attend_splits(const pk_config& cfg) {
    const int64_t hot = (int64_t)cfg.n_sink + cfg.n_local + cfg.buf_tokens;
    return ceil_div(hot, pk::attend_split_keys()) + ceil_div(cfg.top_k, pk::attend_split_keys());
}

pk_status validate_config(const pk_config* cfg, int n_kv, int n_q, int64_t capacity, int* G_out,
                          int* nbins_out) {
    if (!cfg || n_kv < 1 || n_q < 1 || capacity < 1) return PK_ERR_INVALID;
    if (cfg->head_dim != 128) return PK_ERR_UNSUPPORTED;
    if (cfg->n_sub * cfg->sub_dim != cfg->head_dim) return PK_ERR_INVALID;
    if (cfg->sub_dim != 8 && cfg->sub_dim != 4 && cfg->sub_dim != 16) return PK_ERR_UNSUPPORTED;
    if (cfg->rho < 1 || cfg->rho > pk::kRhoMax) return PK_ERR_INVALID;
    if (cfg->coarse_permille < 1 || cfg->coarse_permille > 1000) return PK_ERR_INVALID;
    if (cfg->codebook != 0 && cfg->codebook != 1) return PK_ERR_INVALID;
    if (cfg->top_k < 1 || cfg->n_sink < 0 || cfg->n_local < 0 || cfg->buf_tokens < 0)
        return PK_ERR_INVALID;
    if (cfg->buf_tokens > 0 && cfg->buf_tokens > cfg->n_local) return PK_ERR_INVALID;
    if (n_q % n_kv != 0) return PK_ERR_INVALID;
    const int G = n_q / n_kv;
    if (G < 1 || G > 16) return PK_ERR_INVALID;
    if (G != 1 && G != 2 && G != 4 && G != 8) return PK_ERR_UNSUPPORTED;
    int wmax = 0;
    for (int r = 0; r < cfg->rho; ++r) {
        if (cfg->vote_weight[r] < 1) return PK_ERR_INVALID;
        if (cfg->vote_weight[r] > wmax) wmax = cfg->vote_weight[r];
    }
    // a vote-table byte holds the votes of one subspace (m = 8) or of two (m = 4);
    // an m = 16 table entry holds one centroid's votes in 8 bits
    if (G * wmax * (cfg->sub_dim == 4 ? 2 : 1) > 255) return PK_ERR_INVALID;
    const int nbins = cfg->n_sub * G * wmax + 1;
    if (nbins > pk::kMaxBins) return PK_ERR_UNSUPPORTED;
    if (capacity > (int64_t)1 << 24) return PK_ERR_UNSUPPORTED;
    if (max_attend_splits(*cfg) > pk::attend_max_splits()) return PK_ERR_UNSUPPORTED;
    *G_out = G;
    *nbins_out = nbins;
    return PK_OK;
}

// Oldest local tokens to move into the retrieval zone before the next append
// (zero unless the previous step filled the update buffer).
int64_t pending_eviction(const pk_ctx* c) {
    if (c->cfg.buf_tokens == 0 || c->buf < c->cfg.buf_tokens) return 0;
    const int64_t local = c->n - c->buf - c->r_end;
    return std::max<int64_t>(0, local + c->buf - c->cfg.n_local);
}

// Encodes the evicted tokens and updates the mirror.  Call only when the
// buffer is full.
pk_status evict(pk_ctx* c, hipStream_t st) {
    const int64_t move = pending_eviction(c);
    if (move > 0) {
        StageTimer tm(c, PK_STAGE_ENCODE, st);
        PK_HIP(pk::launch_encode(c->dt == PK_BF16, c->K, c->cap, c->units, c->r_end, move, c->ids,
                                 c->rec, c->cfg.sign_bits, c->tab, st));
        if (c->cents)
            PK_HIP(pk::launch_km_ids(c->dt == PK_BF16, c->K, c->cap, c->units, c->r_end, move,
                                     c->cfg.sign_bits, c->cents, c->ids, st));
    }
    c->r_end += move;
    c->buf = 0;
    return PK_OK;
}

// splits of this step's attention: n_hot_splits over the hot tokens, then
// the selection
void split_plan(const pk_ctx* c, int* n_splits, int* n_hot_splits) {
    const int64_t hot = c->sink_end + (c->n - c->r_end);
    *n_hot_splits = (int)ceil_div(hot, pk::attend_split_keys());
    *n_splits = *n_hot_splits + (int)ceil_div(c->cfg.top_k, pk::attend_split_keys());
}

// qprep (optionally carrying the step's append), scan, rerank, fine select.
// With fuse_hot the fine launch also computes the hot-zone attention splits
// when it can (*hot_done tells whether it did).
pk_status run_retrieve(pk_ctx* c, const void* q, int32_t* sel, int32_t* sel_n, const void* k_new,
                       const void* v_new, hipStream_t st, bool fuse_hot = false,
                       bool* hot_done = nullptr) {
    if (hot_done) *hot_done = false;
    const bool bf16 = c->dt == PK_BF16;
    const int64_t row = (int64_t)pk::kD * dtype_size(c->dt);
    {
        StageTimer tm(c, PK_STAGE_QPREP, st);
        PK_HIP(pk::launch_qprep(bf16, q, c->units, c->G, c->cfg.sign_bits, c->cfg.rho,
                                c->cfg.vote_weight, c->cents, c->lut, c->ysum, c->cfg.sub_dim, k_new,
                                v_new, c->K, c->V,
                                row, c->cap, c->n - 1, pk::ring_slot(c->ring, c->sink_end, c->n - 1),
                                c->ring, st));
    }
    const int64_t n_r = c->r_end - c->sink_end;
    if (n_r <= 0) {
        PK_HIP(pk::launch_empty_select(c->units, sel_n, c->meta, st));
        return PK_OK;
    }
    const int64_t C = coarse_count(n_r, c->cfg.coarse_permille, c->cfg.top_k);
    const int chunk = choose_chunk(c->units, n_r);
    const int n_chunks = (int)ceil_div(n_r, chunk);
    const int tstride = (c->nbins + 1) & ~1;
    {
        StageTimer tm(c, PK_STAGE_SCAN, st);
        PK_HIP(pk::launch_scan(c->ids, c->cap, c->units, c->sink_end, n_r, chunk, n_chunks,
                               c->max_chunks, c->lut, c->scores, c->sstride, c->hist, c->hstride,
                               c->tot, c->nbins, c->cfg.sub_dim, st));
    }
    {
        StageTimer tm(c, PK_STAGE_RERANK, st);
        PK_HIP(pk::launch_rerank(chunk, c->scores, c->sstride, c->rec, c->ids, c->lut, c->cap,
                                 c->units, c->sink_end, n_r, n_chunks, c->max_chunks, c->hist,
                                 c->hstride, c->tot, c->nbins, C, c->cfg.top_k,
                                 c->ysum, c->tab, c->cand_pos, c->cand_est, c->cmax, c->meta,
                                 st));
    }
    StageTimer tm(c, PK_STAGE_FINE, st);
    int n_splits = 0, n_hs = 0;
    split_plan(c, &n_splits, &n_hs);
    if (fuse_hot && n_hs > 0 && n_splits <= c->max_splits &&
        pk::fine_hot_supported(bf16, c->G, c->ring.k != nullptr, (int)C, c->cmax)) {
        PK_HIP(pk::launch_fine_hot(c->cand_pos, c->cand_est, c->cmax, c->units, (int)C,
                                   c->cfg.top_k, sel, sel_n, c->G, c->K, c->V, c->cap, q,
                                   c->sink_end, c->r_end, c->n, n_splits, n_hs, c->part, c->tot,
                                   tstride, st));
        if (hot_done) *hot_done = true;
        return PK_OK;
    }
    PK_HIP(pk::launch_fine(c->cand_pos, c->cand_est, c->cmax, c->units, (int)C, c->cfg.top_k, sel,
                           sel_n, c->tot, tstride, st));
    return PK_OK;
}

// attention splits (those after the hot ones when hot_done), then the merge
pk_status run_attend(pk_ctx* c, const void* q, const int32_t* sel, const int32_t* sel_n,
                     float* out, hipStream_t st, bool hot_done = false) {
    int n_splits = 0, n_hs = 0;
    split_plan(c, &n_splits, &n_hs);
    if (n_splits > c->max_splits) return PK_ERR_INVALID;
    {
        StageTimer tm(c, PK_STAGE_ATTEND, st);
        PK_HIP(pk::launch_attend(c->dt == PK_BF16, c->G, c->K, c->V, c->cap, c->units, q,
                                 c->sink_end, c->r_end, c->n, sel, sel_n, c->cfg.top_k, n_splits,
                                 n_hs, hot_done ? n_hs : 0, c->part, c->ring, st));
    }
    StageTimer tm(c, PK_STAGE_COMBINE, st);
    PK_HIP(pk::launch_combine(c->part, c->units, c->G, n_splits, out, st));
    return PK_OK;
}

// Runs `launch_fn` (one kernel launch); with `kernel_us`, times that launch by
// events attached to the dispatch itself (the same timing as the per-stage
// profile), waits for it and stores its duration in microseconds.
template <typename F>
pk_status reference_launch(float* kernel_us, hipStream_t st, F&& launch_fn) {
    if (kernel_us == nullptr) {
        PK_HIP(launch_fn(st));
        return PK_OK;
    }
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return runtime_fail();
    if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return runtime_fail();
    }
    pk::launch_timing() = {a, b};
    hipError_t e = launch_fn(st);
    pk::launch_timing() = {};
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (e != hipSuccess) return hip_fail(e, "reference kernel");
    *kernel_us = 1000.0f * ms;
    return PK_OK;
}

}  // namespace

extern "C" {

const char* pk_status_string(pk_status s) {
    switch (s) {
        case PK_OK: return "ok";
        case PK_ERR_INVALID: return "invalid argument";
        case PK_ERR_NO_DEVICE: return "no gfx950 device";
        case PK_ERR_OOM: return "device out of memory";
        case PK_ERR_CAPACITY: return "capacity exceeded";
        case PK_ERR_HIP: return "HIP runtime error";
        case PK_ERR_UNSUPPORTED: return "unsupported configuration";
    }
    return "unknown status";
}

pk_status pk_create(const pk_config* cfg, int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                    int64_t capacity, pk_dtype kv_dtype, void* k_store, void* v_store,
                    pk_mem store_mem, pk_ctx** out) {
    if (!out) return PK_ERR_INVALID;
    *out = nullptr;
    if (batch < 1 || !k_store || !v_store) return PK_ERR_INVALID;
    // units index the grid's y dimension of most kernels (at most 65535)
    if ((int64_t)batch * n_kv_heads > 65535) return PK_ERR_UNSUPPORTED;
    if (kv_dtype != PK_F32 && kv_dtype != PK_BF16) return PK_ERR_INVALID;
    if (store_mem != PK_MEM_DEVICE && store_mem != PK_MEM_HOST_MAPPED) return PK_ERR_INVALID;
    int G = 0, nbins = 0;
    pk_status st = validate_config(cfg, n_kv_heads, n_q_heads, capacity, &G, &nbins);
    if (st != PK_OK) return st;
    if ((reinterpret_cast<uintptr_t>(k_store) | reinterpret_cast<uintptr_t>(v_store)) & 15)
        return PK_ERR_INVALID;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return PK_ERR_NO_DEVICE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PK_ERR_NO_DEVICE;
    // the kernels are built for gfx950 only: the current device must be able to load them
    if (pk::probe_kernel_image() != hipSuccess) return runtime_fail(PK_ERR_NO_DEVICE);
    float* scratch_ptr = nullptr;
    {
        const hipError_t e = scratch_address(dev, &scratch_ptr);
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    }

    pk_ctx* c = new (std::nothrow) pk_ctx();
    if (!c) return PK_ERR_OOM;
    c->cfg = *cfg;
    c->batch = batch;
    c->n_kv = n_kv_heads;
    c->n_q = n_q_heads;
    c->G = G;
    c->units = batch * n_kv_heads;
    c->cap = capacity;
    c->dt = kv_dtype;
    c->K = k_store;
    c->V = v_store;
    c->mem = store_mem;
    c->device = dev;
    c->scratch = scratch_ptr;
    c->nbins = nbins;
    c->hstride = (nbins + 7) / 8 * 8;
    c->sstride = (capacity + 7) / 8 * 8;
    if ((cfg->codebook == 0 ? pk_codebook : pk_codebook_quantile)(cfg->sub_dim, 8, c->tab.levels,
                                                                    c->tab.sq_thr) != PK_OK) {
        delete c;
        return PK_ERR_INVALID;
    }
    c->tab.sub_dim = cfg->sub_dim;
    c->max_chunks = (int)std::min<int64_t>(pk::kMaxChunks, ceil_div(capacity, 256));
    // candidate rows hold a multiple of 64 entries: the fine selection reads a
    // thread's (up to 64) candidates in 16-byte vectors
    c->cmax = (std::max<int64_t>(1, coarse_count(capacity, cfg->coarse_permille, cfg->top_k)) + 63) /
              64 * 64;
    c->max_splits = (int)max_attend_splits(*cfg);

    const int64_t U = c->units;
    struct Alloc {
        void** p;
        size_t bytes;
    } allocs[] = {
        {(void**)&c->ids, (size_t)(U * capacity * pk::kSub)},
        {(void**)&c->rec, (size_t)(U * capacity * rec_bytes(cfg->sub_dim))},
        {(void**)&c->lut, (size_t)U * lut_bytes(cfg->sub_dim)},
        {(void**)&c->ysum, (size_t)(U * pk::kD * 4)},
        // score rows padded to 16 B; the tail pad covers vector reads past the last row
        {(void**)&c->scores, (size_t)(U * c->sstride + 8192)},   // last chunk read whole
        {(void**)&c->hist, (size_t)(U * c->max_chunks * (int64_t)c->hstride * 2)},
        {(void**)&c->tot, (size_t)(U * ((c->nbins + 1) & ~1) * 4)},
        {(void**)&c->meta, (size_t)(U * 4 * 4)},
        {(void**)&c->cand_pos, (size_t)(U * c->cmax * 4)},
        {(void**)&c->cand_est, (size_t)(U * c->cmax * 4)},
        {(void**)&c->part, (size_t)(U * c->max_splits * (int64_t)G * (pk::kD + 2) * 4)},
    };
    for (auto& a : allocs) {
        if (hipMalloc(a.p, a.bytes) != hipSuccess) {
            free_all(c);
            delete c;
            return alloc_fail();
        }
    }
    c->ring.n_sink = cfg->n_sink;
    c->ring.span = std::max<int64_t>(1, (int64_t)cfg->n_local + cfg->buf_tokens);
    c->ring.rows = c->ring.n_sink + c->ring.span;
    if (store_mem == PK_MEM_HOST_MAPPED) {
        const size_t rb = (size_t)(U * c->ring.rows * pk::kD * dtype_size(kv_dtype));
        if (hipMalloc(&c->ring.k, rb) != hipSuccess || hipMalloc(&c->ring.v, rb) != hipSuccess) {
            free_all(c);
            delete c;
            return alloc_fail();
        }
    }
    if (hipMemset(c->meta, 0, U * 16) != hipSuccess ||
        hipMemset(c->tot, 0, U * ((c->nbins + 1) & ~1) * 4) != hipSuccess ||
        hipMemset(c->scores, 0, U * c->sstride + 8192) != hipSuccess ||
        hipMemset(c->lut, 0, (size_t)U * lut_bytes(cfg->sub_dim)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        free_all(c);
        delete c;
        return runtime_fail();
    }
    *out = c;
    return PK_OK;
}

void pk_destroy(pk_ctx* ctx) {
    if (!ctx) return;
    (void)hipDeviceSynchronize();
    free_all(ctx);
    delete ctx;
}

pk_status pk_stream_read(const void* src, size_t bytes, uint32_t* sink, float* kernel_us,
                         void* stream) {
    if (!src || !sink || bytes == 0 || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(src) & 15) || bytes > ((size_t)1 << 44))
        return PK_ERR_INVALID;
    return reference_launch(kernel_us, (hipStream_t)stream, [&](hipStream_t st) {
        return pk::launch_stream_read(src, (int64_t)(bytes / 16), sink, st);
    });
}

pk_status pk_gather_read(const void* src, int64_t n_rows, int32_t rec_bytes, const int32_t* idx,
                         int64_t count, uint32_t* sink, float* kernel_us, void* stream) {
    if (!src || !idx || !sink || n_rows < 1 || count < 1 || rec_bytes < 16 || rec_bytes > 1024 ||
        (rec_bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
        n_rows > (int64_t)1 << 40 || count > ((int64_t)1 << 40) / rec_bytes)
        return PK_ERR_INVALID;
    return reference_launch(kernel_us, (hipStream_t)stream, [&](hipStream_t st) {
        return pk::launch_gather_read(src, n_rows, rec_bytes, idx, count, sink, st);
    });
}

pk_status pk_get_window(const pk_ctx* c, int64_t* n_tokens, int64_t* sink_end, int64_t* r_end,
                        int64_t* buf) {
    if (!c) return PK_ERR_INVALID;
    if (n_tokens) *n_tokens = c->n;
    if (sink_end) *sink_end = c->sink_end;
    if (r_end) *r_end = c->r_end;
    if (buf) *buf = c->buf;
    return PK_OK;
}

pk_status pk_encode_keys(pk_ctx* c, int64_t n_tokens, void* stream) {
    if (!c || n_tokens < 1) return PK_ERR_INVALID;
    if (n_tokens > c->cap) return PK_ERR_CAPACITY;
    const int64_t sink_end = std::min<int64_t>(c->cfg.n_sink, n_tokens);
    const int64_t r_end = std::max<int64_t>(sink_end, n_tokens - c->cfg.n_local);
    StageTimer tm(c, PK_STAGE_ENCODE, (hipStream_t)stream);
    PK_HIP(pk::launch_encode(c->dt == PK_BF16, c->K, c->cap, c->units, sink_end, r_end - sink_end,
                             c->ids, c->rec, c->cfg.sign_bits, c->tab, (hipStream_t)stream));
    if (c->cents)
        PK_HIP(pk::launch_km_ids(c->dt == PK_BF16, c->K, c->cap, c->units, sink_end,
                                 r_end - sink_end, c->cfg.sign_bits, c->cents, c->ids,
                                 (hipStream_t)stream));
    PK_HIP(pk::launch_ring_fill(c->K, c->V, (int64_t)pk::kD * dtype_size(c->dt), c->cap, c->units,
                                sink_end, r_end, n_tokens, c->ring, (hipStream_t)stream));
    c->n = n_tokens;
    c->sink_end = sink_end;
    c->r_end = r_end;
    c->buf = 0;
    c->prefilled = true;
    return PK_OK;
}

pk_status pk_fit_centroids(pk_ctx* c, int64_t n_tokens, const int32_t* init_pos, int32_t iters,
                           void* stream) {
    if (!c || !init_pos || iters < 0 || iters > 1000) return PK_ERR_INVALID;
    if (c->prefilled) return PK_ERR_INVALID;          // ids of encoded keys would be stale
    if (c->cfg.sub_dim != 8) return PK_ERR_UNSUPPORTED;   // 256 fitted centroids of 8 coordinates
    if (n_tokens < 256) return PK_ERR_INVALID;
    if (n_tokens > c->cap) return PK_ERR_CAPACITY;
    const hipStream_t st = (hipStream_t)stream;
    // the initial positions index the store: checked on the host before any launch
    std::vector<int32_t> pos((size_t)c->units * 256);
    PK_HIP(hipMemcpyAsync(pos.data(), init_pos, pos.size() * sizeof(int32_t),
                          hipMemcpyDeviceToHost, st));
    PK_HIP(hipStreamSynchronize(st));
    for (int32_t p : pos)
        if (p < 0 || p >= n_tokens) return PK_ERR_INVALID;
    const size_t n = (size_t)c->units * pk::kSub * 256 * 8;
    if (!c->cents) {
        float* ct = nullptr;
        long long* sm = nullptr;
        if (hipMalloc((void**)&ct, n * sizeof(float)) != hipSuccess) return alloc_fail();
        if (hipMalloc((void**)&sm, n * sizeof(long long)) != hipSuccess) {
            (void)hipFree(ct);
            return alloc_fail();
        }
        c->cents = ct;
        c->km_sums = sm;
    }
    PK_HIP(hipMemsetAsync(c->cents, 0, n * sizeof(float), st));
    StageTimer tm(c, PK_STAGE_ENCODE, st);
    PK_HIP(pk::launch_km_fit(c->dt == PK_BF16, c->K, c->cap, c->units, n_tokens, init_pos, iters,
                             c->cfg.sign_bits, c->cents, c->km_sums, st));
    return PK_OK;
}

pk_status pk_append_decode_keys(pk_ctx* c, const void* k_new, const void* v_new, void* stream) {
    if (!c || !k_new || !v_new) return PK_ERR_INVALID;
    if (!aligned16(k_new) || !aligned16(v_new)) return PK_ERR_INVALID;
    if (!c->prefilled || c->cfg.buf_tokens == 0) return PK_ERR_INVALID;
    if (c->n + 1 > c->cap) return PK_ERR_CAPACITY;
    const hipStream_t st = (hipStream_t)stream;
    if (c->buf >= c->cfg.buf_tokens) {
        pk_status s = evict(c, st);
        if (s != PK_OK) return s;
    }
    const int64_t row = (int64_t)pk::kD * dtype_size(c->dt);
    {
        StageTimer tm(c, PK_STAGE_APPEND, st);
        PK_HIP(pk::launch_append(k_new, v_new, c->K, c->V, row, c->cap, c->n,
                                 pk::ring_slot(c->ring, c->sink_end, c->n), c->units, c->ring, st));
    }
    c->n += 1;
    c->buf += 1;
    return PK_OK;
}

pk_status pk_retrieve(pk_ctx* c, const void* q, int32_t* sel, int32_t* sel_n, void* stream) {
    if (!c || !q || !sel || !sel_n) return PK_ERR_INVALID;
    if (!aligned16(q) || !aligned16(sel) || !aligned16(sel_n)) return PK_ERR_INVALID;
    if (!c->prefilled) return PK_ERR_INVALID;
    return run_retrieve(c, q, sel, sel_n, nullptr, nullptr, (hipStream_t)stream);
}

pk_status pk_sparse_attend(pk_ctx* c, const void* q, const int32_t* sel, const int32_t* sel_n,
                           float* out, void* stream) {
    if (!c || !q || !sel || !sel_n || !out) return PK_ERR_INVALID;
    if (!aligned16(q) || !aligned16(sel) || !aligned16(sel_n) || !aligned16(out))
        return PK_ERR_INVALID;
    if (!c->prefilled) return PK_ERR_INVALID;
    return run_attend(c, q, sel, sel_n, out, (hipStream_t)stream);
}

pk_status pk_dense_attend(pk_ctx* c, const void* q, float* out, void* stream) {
    if (!c || !q || !out) return PK_ERR_INVALID;
    if (!aligned16(q) || !aligned16(out)) return PK_ERR_INVALID;
    if (!c->prefilled || c->n < 1) return PK_ERR_INVALID;
    if (c->ring.k != nullptr) return PK_ERR_UNSUPPORTED;
    const int64_t n_splits = ceil_div(c->n, pk::attend_split_keys());
    if (n_splits > pk::attend_max_splits()) return PK_ERR_UNSUPPORTED;
    const size_t need = (size_t)c->units * n_splits * c->G * (pk::kD + 2) * sizeof(float);
    if (need > c->dense_bytes) {
        if (c->dense_part) (void)hipFree(c->dense_part);
        c->dense_part = nullptr;
        c->dense_bytes = 0;
        if (hipMalloc((void**)&c->dense_part, need) != hipSuccess) return alloc_fail();
        c->dense_bytes = need;
    }
    const hipStream_t st = (hipStream_t)stream;
    // every token as one zone read straight from the store: sink_end = r_end = n
    PK_HIP(pk::launch_attend(c->dt == PK_BF16, c->G, c->K, c->V, c->cap, c->units, q, c->n, c->n,
                             c->n, nullptr, nullptr, c->cfg.top_k, (int)n_splits, (int)n_splits,
                             0, c->dense_part, pk::HotRing{}, st));
    PK_HIP(pk::launch_combine(c->dense_part, c->units, c->G, (int)n_splits, out, st));
    return PK_OK;
}

pk_status pk_dense_attend_noalloc(pk_ctx* c, const void* q, float* out, void* stream) {
    if (!c || !q || !out) return PK_ERR_INVALID;
    if (!aligned16(q) || !aligned16(out)) return PK_ERR_INVALID;
    if (!c->prefilled || c->n < 1) return PK_ERR_INVALID;
    if (c->ring.k != nullptr) return PK_ERR_UNSUPPORTED;
    const int64_t n_splits = ceil_div(c->n, pk::attend_split_keys());
    if (n_splits > pk::attend_max_splits()) return PK_ERR_UNSUPPORTED;
    const size_t need = (size_t)c->units * n_splits * c->G * (pk::kD + 2) * sizeof(float);
    if (need > kNoAllocScratchBytes) return PK_ERR_CAPACITY;
    // every (unit, split, head) partial the merge reads is written by the
    // attention launch before it: nothing of the scratch has to start at zero
    const hipStream_t st = (hipStream_t)stream;
    PK_HIP(pk::launch_attend(c->dt == PK_BF16, c->G, c->K, c->V, c->cap, c->units, q, c->n, c->n,
                             c->n, nullptr, nullptr, c->cfg.top_k, (int)n_splits, (int)n_splits,
                             0, c->scratch, pk::HotRing{}, st));
    PK_HIP(pk::launch_combine(c->scratch, c->units, c->G, (int)n_splits, out, st));
    return PK_OK;
}

size_t pk_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

pk_status pk_decode_step(pk_ctx* c, const void* k_new, const void* v_new, const void* q,
                         int32_t* sel, int32_t* sel_n, float* out, void* stream) {
    if (!c || !k_new || !v_new || !q || !sel || !sel_n || !out) return PK_ERR_INVALID;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(sel) ||
        !aligned16(sel_n) || !aligned16(out))
        return PK_ERR_INVALID;
    if (!c->prefilled || c->cfg.buf_tokens == 0) return PK_ERR_INVALID;
    if (c->n + 1 > c->cap) return PK_ERR_CAPACITY;
    const hipStream_t st = (hipStream_t)stream;
    if (c->buf >= c->cfg.buf_tokens) {
        pk_status s = evict(c, st);
        if (s != PK_OK) return s;
    }
    // the query-prep kernel copies the new token to position n (the old count)
    c->n += 1;
    c->buf += 1;
    bool hot_done = false;
    pk_status s = run_retrieve(c, q, sel, sel_n, k_new, v_new, st, true, &hot_done);
    if (s != PK_OK) return s;
    return run_attend(c, q, sel, sel_n, out, st, hot_done);
}

pk_status pk_profile_enable(pk_ctx* c, int32_t on) {
    if (!c) return PK_ERR_INVALID;
    if (hipDeviceSynchronize() != hipSuccess) return runtime_fail();
    release_events(c);
    c->profiling = on != 0;
    return PK_OK;
}

pk_status pk_profile_read(pk_ctx* c, double* ms, int64_t* launches) {
    if (!c || !ms || !launches) return PK_ERR_INVALID;
    for (int i = 0; i < PK_STAGE_COUNT; ++i) {
        ms[i] = 0.0;
        launches[i] = 0;
    }
    for (auto& m : c->marks) {
        PK_HIP(hipEventSynchronize(m.b));
        float t = 0.0f;
        PK_HIP(hipEventElapsedTime(&t, m.a, m.b));
        ms[m.stage] += t;
        launches[m.stage] += 1;
    }
    return PK_OK;
}

size_t pk_debug_size(const pk_ctx* c, int32_t what) {
    if (!c) return 0;
    const size_t U = (size_t)c->units, cap = (size_t)c->cap;
    switch (what) {
        case PK_DBG_IDS: return U * cap * pk::kSub;
        case PK_DBG_REC: return U * cap * rec_bytes(c->cfg.sub_dim);
        case PK_DBG_LUT: return U * lut_bytes(c->cfg.sub_dim);
        case PK_DBG_SCORES: return U * cap;
        case PK_DBG_CAND: return U * (size_t)c->cmax * 4;
        case PK_DBG_EST: return U * (size_t)c->cmax * 4;
        case PK_DBG_NCAND: return U * 16;
        case PK_DBG_CENTROIDS: return c->cents ? U * pk::kSub * 256 * 8 * sizeof(float) : 0;
    }
    return 0;
}

pk_status pk_debug_copy(pk_ctx* c, int32_t what, void* host_dst, size_t bytes, void* stream) {
    if (!c || !host_dst) return PK_ERR_INVALID;
    const size_t need = pk_debug_size(c, what);
    if (need == 0 || bytes != need) return PK_ERR_INVALID;
    const void* src = nullptr;
    switch (what) {
        case PK_DBG_IDS: src = c->ids; break;
        case PK_DBG_REC: src = c->rec; break;
        case PK_DBG_LUT: src = c->lut; break;
        case PK_DBG_SCORES: src = c->scores; break;
        case PK_DBG_CAND: src = c->cand_pos; break;
        case PK_DBG_EST: src = c->cand_est; break;
        case PK_DBG_NCAND: src = c->meta; break;
        case PK_DBG_CENTROIDS: src = c->cents; break;
    }
    const hipStream_t st = (hipStream_t)stream;
    if (what == PK_DBG_SCORES) {
        PK_HIP(hipMemcpy2DAsync(host_dst, c->cap, src, c->sstride, c->cap, c->units,
                                hipMemcpyDeviceToHost, st));
    } else {
        PK_HIP(hipMemcpyAsync(host_dst, src, bytes, hipMemcpyDeviceToHost, st));
    }
    PK_HIP(hipStreamSynchronize(st));
    return PK_OK;
}

}  // extern "C"
