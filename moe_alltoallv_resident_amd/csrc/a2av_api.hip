// C ABI of the dispatch/combine library (declared in include/a2av.h): argument
// checks, the handle's workspace, and the launch sequence on the caller's stream.
// Nothing here reads device data back, synchronises or allocates after a2av_create.
#include "../../include/a2av.h"
#include "a2av_internal.h"

#include <mutex>
#include <new>
#include <vector>

using a2av::Shape;
using a2av::Tables;

// One timed kernel launch: stage id and the events recorded around it.
struct TimedLaunch {
    int stage;
    hipEvent_t a, b;
};

struct a2av_context {
    a2av_config_t cfg;
    Shape sh;
    int device;
    bool direct;          // A2AV_PATH_DIRECT: no send buffer, rows go straight to receivers
    void* send_buf;       // [R][T*k][row]: send segments, then the return buffer (staged)
    void* meta;           // tables
    size_t meta_bytes;
    Tables tb;
    bool routed;          // latest planning came from a2av_dispatch (combine allowed)
    std::vector<TimedLaunch> timed;  // stage timing slots
    size_t timed_used;
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int nbits_for(int32_t E) {
    int b = 0;
    while ((1ll << b) < E) ++b;
    return b;
}

bool make_shape(const a2av_config_t* c, Shape* sh) {
    if (!c) return false;
    if (c->num_ranks < 1 || c->num_ranks > a2av::kMaxRanks) return false;
    if (c->tokens_per_rank < 0 || c->hidden < 1) return false;
    if (c->dtype != A2AV_F32 && c->dtype != A2AV_BF16) return false;
    if (c->experts_per_rank < 1) return false;
    const int64_t E = (int64_t)c->num_ranks * c->experts_per_rank;
    if (E > a2av::kMaxExperts) return false;
    if (c->top_k < 1 || c->top_k > a2av::kMaxTopK || c->top_k > E) return false;
    const int64_t TK = (int64_t)c->tokens_per_rank * c->top_k;
    if ((int64_t)c->num_ranks * TK > INT32_MAX) return false;          // rows are int32
    if ((int64_t)c->num_ranks * c->tokens_per_rank > INT32_MAX) return false;
    if (c->recv_capacity_rows < 0) return false;
    int64_t cap = c->recv_capacity_rows;
    if (cap == 0) cap = (int64_t)c->num_ranks * c->tokens_per_rank * std::min<int64_t>(c->top_k, c->experts_per_rank);
    if (cap > INT32_MAX) return false;
    if (c->path != A2AV_PATH_STAGED && c->path != A2AV_PATH_DIRECT) return false;
    if (c->recv_layout != A2AV_LAYOUT_SOURCE_MAJOR && c->recv_layout != A2AV_LAYOUT_EXPERT_MAJOR) return false;
    sh->R = c->num_ranks;
    sh->T = c->tokens_per_rank;
    sh->k = c->top_k;
    sh->E = (int32_t)E;
    sh->epr = c->experts_per_rank;
    sh->H = c->hidden;
    sh->dtype = c->dtype;
    sh->nbits = nbits_for((int32_t)E);
    sh->TK = TK;
    sh->cap = cap;
    sh->row_bytes = (int64_t)c->hidden * (c->dtype == A2AV_BF16 ? 2 : 4);
    sh->num_cu = 256;
    sh->layout = c->recv_layout;
    return true;
}

struct MetaLayout {
    size_t pos, cnt, send_off, recv_counts, recv_off, eoff, xbase, recv_eoff, dest, inv, total;
};

MetaLayout meta_layout(const Shape& sh) {
    MetaLayout m{};
    size_t o = 0;
    m.pos = o;         o += align_up(sizeof(int32_t) * (size_t)sh.R * (size_t)std::max<int64_t>(sh.TK, 1));
    m.cnt = o;         o += align_up(sizeof(int32_t) * (size_t)sh.R * sh.E);
    m.send_off = o;    o += align_up(sizeof(int32_t) * (size_t)sh.R * (sh.R + 1));
    m.recv_counts = o; o += align_up(sizeof(int32_t) * (size_t)sh.R * sh.R);
    m.recv_off = o;    o += align_up(sizeof(int32_t) * (size_t)sh.R * (sh.R + 1));
    m.eoff = o;        o += align_up(sizeof(int32_t) * (size_t)sh.R * (sh.E + 1));
    m.xbase = o;       o += align_up(sizeof(int32_t) * (size_t)sh.R * sh.E);
    m.recv_eoff = o;   o += align_up(sizeof(int32_t) * (size_t)sh.R * (sh.epr + 1));
    m.dest = o;        o += align_up(sizeof(int64_t) * (size_t)sh.R * (size_t)std::max<int64_t>(sh.TK, 1));
    m.inv = o;         o += align_up(sizeof(int32_t) * (size_t)sh.R * (size_t)std::max<int64_t>(sh.TK, 1));
    m.total = o;
    return m;
}

size_t send_bytes(const a2av_config_t* c, const Shape& sh) {
    if (c->path == A2AV_PATH_DIRECT) return 0;
    return (size_t)sh.R * (size_t)sh.TK * (size_t)sh.row_bytes;
}

bool on_device(const a2av_context* h) {
    int dev = -1;
    return hipGetDevice(&dev) == hipSuccess && dev == h->device;
}

int min_vec(const Shape& sh) { return sh.dtype == A2AV_F32 ? 4 : 2; }

// Row arrays are empty when there are no tokens; their pointers may then be null.
bool has_tokens(const Shape& sh) { return sh.T > 0; }

// Launch one kernel, with timing events around it while timing slots remain (never on a
// stream that is being captured into a graph: the events belong to eager timing only).
template <typename F>
int launch_timed(a2av_context* h, int stage, hipStream_t st, F&& launch) {
    TimedLaunch* t = nullptr;
    if (h->timed_used < h->timed.size()) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) return A2AV_ERR_HIP;
        if (cs == hipStreamCaptureStatusNone) t = &h->timed[h->timed_used++];
    }
    if (t) {
        t->stage = stage;
        if (hipEventRecord(t->a, st) != hipSuccess) return A2AV_ERR_HIP;
    }
    if (launch() != hipSuccess) return A2AV_ERR_HIP;
    if (t && hipEventRecord(t->b, st) != hipSuccess) return A2AV_ERR_HIP;
    return A2AV_OK;
}

void drop_timing(a2av_context* h) {
    for (TimedLaunch& t : h->timed) {
        (void)hipEventDestroy(t.a);
        (void)hipEventDestroy(t.b);
    }
    h->timed.clear();
    h->timed_used = 0;
}

enum { kStagePlan = 0, kStagePack = 1, kStageExchange = 2, kStageReturn = 3, kStageCombine = 4 };

// ---- the allocation-free bare collective -------------------------------------------
// Its three tables (send offsets, receive counts, receive offsets) live in `scratch`, a
// fixed device array each GPU holds for the life of the process.  Host code never uses
// the array's name as an address (on the host it names a stand-in object): the device
// address is looked up once per device with hipGetSymbolAddress and kept here.
constexpr int kMaxDevices = 64;

struct NoAllocLayout {
    size_t send_off, recv_counts, recv_off, total;
};

NoAllocLayout noalloc_layout(int64_t R) {
    NoAllocLayout m{};
    size_t o = 0;
    m.send_off = o;    o += align_up(sizeof(int32_t) * (size_t)R * (size_t)(R + 1));
    m.recv_counts = o; o += align_up(sizeof(int32_t) * (size_t)R * (size_t)R);
    m.recv_off = o;    o += align_up(sizeof(int32_t) * (size_t)R * (size_t)(R + 1));
    m.total = o;
    return m;
}

struct DeviceScratch {
    void* ptr;    // device address of `scratch` on this device, null until looked up
    int num_cu;
};

std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[A2AV_NOALLOC_SCRATCH_BYTES];

static_assert(A2AV_NOALLOC_MAX_RANKS <= a2av::kMaxRanks, "no-alloc rank limit");
static_assert(A2AV_ST_BOUNDS == a2av::kStBounds, "debug status bit");

namespace {

// This device's scratch address and CU count, looked up on its first call (with the
// device current) and kept for every later call.
int device_scratch(int dev, DeviceScratch* out) {
    if (dev < 0 || dev >= kMaxDevices) return A2AV_ERR_INVALID;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    DeviceScratch& ds = g_scratch[dev];
    if (!ds.ptr) {
        void* p = nullptr;
        int cus = 0;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            return A2AV_ERR_HIP;
        }
        ds.num_cu = cus;
        ds.ptr = p;
    }
    *out = ds;
    return A2AV_OK;
}

}  // namespace

extern "C" {

const char* a2av_error_string(int code) {
    switch (code) {
        case A2AV_OK: return "ok";
        case A2AV_ERR_INVALID: return "invalid argument or configuration";
        case A2AV_ERR_NOMEM: return "allocation failed";
        case A2AV_ERR_HIP: return "HIP runtime error";
        case A2AV_ERR_SCRATCH: return "shape exceeds the no-alloc scratch array";
        default: return "unknown error code";
    }
}

int64_t a2av_workspace_bytes(const a2av_config_t* cfg) {
    Shape sh;
    if (!make_shape(cfg, &sh)) return -1;
    return (int64_t)(align_up(send_bytes(cfg, sh)) + meta_layout(sh).total);
}

int a2av_create(const a2av_config_t* cfg, a2av_handle_t* out) {
    if (!out) return A2AV_ERR_INVALID;
    *out = nullptr;
    Shape sh;
    if (!make_shape(cfg, &sh)) return A2AV_ERR_INVALID;
    a2av_context* h = new (std::nothrow) a2av_context();
    if (!h) return A2AV_ERR_NOMEM;
    h->cfg = *cfg;
    h->sh = sh;
    h->direct = cfg->path == A2AV_PATH_DIRECT;
    if (hipGetDevice(&h->device) != hipSuccess ||
        hipDeviceGetAttribute(&h->sh.num_cu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess) {
        delete h;
        return A2AV_ERR_HIP;
    }
    const MetaLayout m = meta_layout(sh);
    const size_t sb = std::max<size_t>(send_bytes(cfg, sh), kAlign);
    if (hipMalloc(&h->send_buf, sb) != hipSuccess) { (void)hipGetLastError(); delete h; return A2AV_ERR_NOMEM; }
    if (hipMalloc(&h->meta, m.total) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(h->send_buf);
        delete h;
        return A2AV_ERR_NOMEM;
    }
    h->meta_bytes = m.total;
    char* b = static_cast<char*>(h->meta);
    h->tb.pos = reinterpret_cast<int32_t*>(b + m.pos);
    h->tb.cnt = reinterpret_cast<int32_t*>(b + m.cnt);
    h->tb.send_off = reinterpret_cast<int32_t*>(b + m.send_off);
    h->tb.recv_counts = reinterpret_cast<int32_t*>(b + m.recv_counts);
    h->tb.recv_off = reinterpret_cast<int32_t*>(b + m.recv_off);
    h->tb.eoff = reinterpret_cast<int32_t*>(b + m.eoff);
    h->tb.xbase = reinterpret_cast<int32_t*>(b + m.xbase);
    h->tb.recv_eoff = reinterpret_cast<int32_t*>(b + m.recv_eoff);
    h->tb.dest = reinterpret_cast<int64_t*>(b + m.dest);
    h->tb.inv = reinterpret_cast<int32_t*>(b + m.inv);
    // tables start at zero
    if (hipMemset(h->meta, 0, m.total) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(h->meta);
        (void)hipFree(h->send_buf);
        delete h;
        return A2AV_ERR_HIP;
    }
    h->routed = false;
    h->timed_used = 0;
    *out = h;
    return A2AV_OK;
}

int a2av_destroy(a2av_handle_t h) {
    if (!h) return A2AV_OK;
    int rc = A2AV_OK;
    drop_timing(h);
    if (hipFree(h->meta) != hipSuccess) rc = A2AV_ERR_HIP;
    if (hipFree(h->send_buf) != hipSuccess) rc = A2AV_ERR_HIP;
    delete h;
    return rc;
}

// The status word is updated with device atomics, which need a 4-byte aligned address.
static bool status_ok(const uint32_t* status) { return status && ((uintptr_t)status % 4) == 0; }

int a2av_dispatch(a2av_handle_t h, const void* x, const int32_t* topk_ids, void* recv, int32_t* split,
                  int32_t* recv_counts, int32_t* recv_offsets, uint32_t* status, void* stream) {
    if (!h || !status_ok(status) || !on_device(h)) return A2AV_ERR_INVALID;
    const Shape& sh = h->sh;
    if (has_tokens(sh) && (!x || !topk_ids || (sh.cap > 0 && !recv))) return A2AV_ERR_INVALID;
    const void* ptrs[] = {x, recv, h->send_buf};
    const int vec = a2av::pick_vec_bytes(sh.row_bytes, ptrs, 3);
    if (vec < min_vec(sh)) return A2AV_ERR_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const a2av::Outputs out{split, recv_counts, recv_offsets};
    const a2av::Tables& tb = h->tb;
    void* dst = h->direct ? recv : h->send_buf;
    int rc;
    if (a2av::small_dispatch(sh, h->direct)) {
        rc = launch_timed(h, kStagePack, st, [&] {
            return a2av::launch_dispatch_small(sh, tb, topk_ids, out, status, x, dst, h->direct, vec, st);
        });
        if (rc != A2AV_OK) return rc;
    } else {
        rc = launch_timed(h, kStagePlan, st, [&] { return a2av::launch_plan(sh, tb, topk_ids, out, status, st); });
        if (rc != A2AV_OK) return rc;
        rc = launch_timed(h, kStagePack, st,
                          [&] { return a2av::launch_pack(sh, tb, out, status, x, dst, h->direct, vec, st); });
        if (rc != A2AV_OK) return rc;
    }
    if (!h->direct && sh.TK > 0) {
        rc = launch_timed(h, kStageExchange, st, [&] {
            return a2av::launch_exchange(sh, tb, out, status, h->send_buf, recv, false, false, vec, st);
        });
        if (rc != A2AV_OK) return rc;
    }
    h->routed = true;
    return A2AV_OK;
}

int a2av_combine(a2av_handle_t h, const void* expert_out, const float* gates, void* y, uint32_t* status,
                 void* stream) {
    if (!h || !status_ok(status) || !on_device(h) || !h->routed) return A2AV_ERR_INVALID;
    const Shape& sh = h->sh;
    if (has_tokens(sh) && (!gates || !y || (sh.cap > 0 && !expert_out))) return A2AV_ERR_INVALID;
    const void* ptrs[] = {expert_out, y, h->send_buf};
    const int vec = a2av::pick_vec_bytes(sh.row_bytes, ptrs, 3);
    if (vec < min_vec(sh) || ((uintptr_t)gates % 4) != 0) return A2AV_ERR_INVALID;
    if (!has_tokens(sh)) return A2AV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const a2av::Tables& tb = h->tb;
    const a2av::Outputs none{nullptr, nullptr, nullptr};
    if (!h->direct) {
        int rc = launch_timed(h, kStageReturn, st, [&] {
            return a2av::launch_exchange(sh, tb, none, status, expert_out, h->send_buf, true, false, vec, st);
        });
        if (rc != A2AV_OK) return rc;
    }
    const void* rows = h->direct ? expert_out : h->send_buf;
    return launch_timed(h, kStageCombine, st,
                        [&] { return a2av::launch_combine(sh, tb, rows, gates, y, status, h->direct, vec, st); });
}

int a2av_alltoallv(a2av_handle_t h, const void* send, const int32_t* send_counts, void* recv, int32_t* recv_counts,
                   int32_t* recv_offsets, uint32_t* status, void* stream) {
    if (!h || !send_counts || !status_ok(status) || !on_device(h)) return A2AV_ERR_INVALID;
    const Shape& sh = h->sh;
    if (has_tokens(sh) && (!send || (sh.cap > 0 && !recv))) return A2AV_ERR_INVALID;
    const void* ptrs[] = {send, recv};
    const int vec = a2av::pick_vec_bytes(sh.row_bytes, ptrs, 2);
    if (vec < min_vec(sh)) return A2AV_ERR_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    h->routed = false;
    const a2av::Outputs out{nullptr, recv_counts, recv_offsets};
    if (a2av::launch_plan_from_counts(sh, h->tb, send_counts, status, st) != hipSuccess) return A2AV_ERR_HIP;
    if (a2av::launch_exchange(sh, h->tb, out, status, send, recv, false, true, vec, st) != hipSuccess)
        return A2AV_ERR_HIP;
    return A2AV_OK;
}

int a2av_alltoallv_noalloc(const a2av_config_t* cfg, const void* send, const int32_t* send_counts, void* recv,
                           int32_t* recv_counts, int32_t* recv_offsets, uint32_t* status, void* stream) {
    if (!cfg) return A2AV_ERR_INVALID;
    a2av_config_t c = *cfg;
    c.path = A2AV_PATH_STAGED;                 // not used by the bare collective
    c.recv_layout = A2AV_LAYOUT_SOURCE_MAJOR;
    Shape sh;
    if (!make_shape(&c, &sh) || !send_counts || !status_ok(status)) return A2AV_ERR_INVALID;
    if (sh.R > A2AV_NOALLOC_MAX_RANKS) return A2AV_ERR_SCRATCH;
    const NoAllocLayout m = noalloc_layout(sh.R);
    if (m.total > sizeof(scratch)) return A2AV_ERR_SCRATCH;
    if (has_tokens(sh) && (!send || (sh.cap > 0 && !recv))) return A2AV_ERR_INVALID;
    const void* ptrs[] = {send, recv};
    const int vec = a2av::pick_vec_bytes(sh.row_bytes, ptrs, 2);
    if (vec < min_vec(sh)) return A2AV_ERR_INVALID;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return A2AV_ERR_HIP;
    DeviceScratch ds{};
    const int rc = device_scratch(dev, &ds);
    if (rc != A2AV_OK) return rc;
    sh.num_cu = ds.num_cu;
    char* base = static_cast<char*>(ds.ptr);
    Tables tb{};                               // the collective touches only these three
    tb.send_off = reinterpret_cast<int32_t*>(base + m.send_off);
    tb.recv_counts = reinterpret_cast<int32_t*>(base + m.recv_counts);
    tb.recv_off = reinterpret_cast<int32_t*>(base + m.recv_off);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const a2av::Outputs out{nullptr, recv_counts, recv_offsets};
    if (a2av::launch_plan_from_counts(sh, tb, send_counts, status, st) != hipSuccess) return A2AV_ERR_HIP;
    if (a2av::launch_exchange(sh, tb, out, status, send, recv, false, true, vec, st) != hipSuccess)
        return A2AV_ERR_HIP;
    return A2AV_OK;
}

int a2av_copy_positions(a2av_handle_t h, int32_t* pos, void* stream) {
    if (!h || !on_device(h)) return A2AV_ERR_INVALID;
    const size_t n = sizeof(int32_t) * (size_t)h->sh.R * (size_t)h->sh.TK;
    if (n == 0) return A2AV_OK;
    if (!pos) return A2AV_ERR_INVALID;
    return hipMemcpyAsync(pos, h->tb.pos, n, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)) == hipSuccess
               ? A2AV_OK : A2AV_ERR_HIP;
}

int a2av_copy_recv_expert_offsets(a2av_handle_t h, int32_t* recv_expert_offsets, void* stream) {
    if (!h || !recv_expert_offsets || !on_device(h)) return A2AV_ERR_INVALID;
    if (h->sh.layout != A2AV_LAYOUT_EXPERT_MAJOR) return A2AV_ERR_INVALID;
    const size_t n = sizeof(int32_t) * (size_t)h->sh.R * (h->sh.epr + 1);
    return hipMemcpyAsync(recv_expert_offsets, h->tb.recv_eoff, n, hipMemcpyDeviceToDevice,
                          static_cast<hipStream_t>(stream)) == hipSuccess ? A2AV_OK : A2AV_ERR_HIP;
}

int a2av_copy_send_offsets(a2av_handle_t h, int32_t* send_offsets, void* stream) {
    if (!h || !send_offsets || !on_device(h)) return A2AV_ERR_INVALID;
    const size_t n = sizeof(int32_t) * (size_t)h->sh.R * (h->sh.R + 1);
    return hipMemcpyAsync(send_offsets, h->tb.send_off, n, hipMemcpyDeviceToDevice,
                          static_cast<hipStream_t>(stream)) == hipSuccess ? A2AV_OK : A2AV_ERR_HIP;
}

int a2av_expert_apply(a2av_handle_t h, const void* in, void* out, int32_t mode, void* stream) {
    if (!h || !on_device(h) || !h->routed) return A2AV_ERR_INVALID;
    if (mode != A2AV_EXPERT_IDENTITY && mode != A2AV_EXPERT_SCALE) return A2AV_ERR_INVALID;
    const Shape& sh = h->sh;
    if (has_tokens(sh) && sh.cap > 0 && (!in || !out)) return A2AV_ERR_INVALID;
    const void* ptrs[] = {in, out};
    const int vec = a2av::pick_vec_bytes(sh.row_bytes, ptrs, 2);
    if (vec < min_vec(sh)) return A2AV_ERR_INVALID;
    return a2av::launch_expert(sh, h->tb, in, out, mode, vec, static_cast<hipStream_t>(stream)) == hipSuccess
               ? A2AV_OK : A2AV_ERR_HIP;
}

int a2av_route_step(const int32_t* ids_table, const float* gates_table, int32_t steps, int64_t n, int32_t* counter,
                    int32_t* ids, float* gates, void* stream) {
    if (!ids_table || !gates_table || !counter || !ids || !gates || steps < 1 || n < 0) return A2AV_ERR_INVALID;
    return a2av::launch_route_step(ids_table, gates_table, steps, n, counter, ids, gates,
                                   static_cast<hipStream_t>(stream)) == hipSuccess ? A2AV_OK : A2AV_ERR_HIP;
}

int a2av_copy_reference(const void* src, void* dst, int64_t rows, int64_t row_bytes, void* stream) {
    if (rows < 0 || row_bytes < 16 || row_bytes % 16 != 0) return A2AV_ERR_INVALID;
    if (rows > 0 && (!src || !dst || ((uintptr_t)src % 16) != 0 || ((uintptr_t)dst % 16) != 0)) return A2AV_ERR_INVALID;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return A2AV_ERR_HIP;
    return a2av::launch_reference_copy(src, dst, rows, row_bytes, cus, static_cast<hipStream_t>(stream)) == hipSuccess
               ? A2AV_OK : A2AV_ERR_HIP;
}

int a2av_timing_begin(a2av_handle_t h, int32_t max_calls) {
    if (!h || max_calls < 1 || max_calls > A2AV_TIMING_MAX_CALLS) return A2AV_ERR_INVALID;
    drop_timing(h);
    try {
        h->timed.resize((size_t)max_calls * A2AV_STAGES);
    } catch (const std::bad_alloc&) {
        return A2AV_ERR_NOMEM;
    }
    for (TimedLaunch& t : h->timed) {
        t.a = t.b = nullptr;
        if (hipEventCreate(&t.a) != hipSuccess || hipEventCreate(&t.b) != hipSuccess) {
            drop_timing(h);
            return A2AV_ERR_HIP;
        }
    }
    h->timed_used = 0;
    return A2AV_OK;
}

int a2av_timing_end(a2av_handle_t h, double* ms_sum, int32_t* launches) {
    if (!h || !ms_sum || !launches) return A2AV_ERR_INVALID;
    for (int i = 0; i < A2AV_STAGES; ++i) { ms_sum[i] = 0.0; launches[i] = 0; }
    int rc = A2AV_OK;
    for (size_t i = 0; i < h->timed_used; ++i) {
        const TimedLaunch& t = h->timed[i];
        float ms = 0.0f;
        if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&ms, t.a, t.b) != hipSuccess) {
            rc = A2AV_ERR_HIP;
            continue;
        }
        ms_sum[t.stage] += ms;
        launches[t.stage] += 1;
    }
    drop_timing(h);
    return rc;
}

}  // extern "C"
