// api.hip -- the C ABI of libmoe.so (declared in include/moe.h): host-side argument checks,
// the gfx950 device check, workspace carving and the graph-cached whole-step forward
// ([FMF8] Phase 2: launches without host synchronisation, the serving path captured once as
// a graph and replayed with a single launch; the output memset fused away).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstring>
#include <mutex>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

struct DevState {
    int checked = 0;   // 0 unknown, 1 gfx950, -1 not usable
    DeviceInfo info{0};
    hipStream_t capture = nullptr;
    void* scratch = nullptr;   // this device's copy of `scratch` (moe_forward_noalloc)
};
DevState g_dev[kMaxDevices];
std::mutex g_mu;
thread_local int t_dev = 0;

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MOE_E_DEVICE;
    }
    t_dev = dev;
    DevState& d = g_dev[dev];
    if (d.checked == 0) {
        std::lock_guard<std::mutex> lk(g_mu);
        if (d.checked == 0) {
            hipDeviceProp_t p;
            if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
                (void)hipGetLastError();
                d.checked = -1;
            } else {
                d.info.cu_count = p.multiProcessorCount;
                d.checked = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
            }
        }
    }
    return d.checked == 1 ? MOE_OK : MOE_E_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

bool route_dims_ok(int M, int E, int k) {
    return M >= 0 && E >= 1 && E <= kMaxE && k >= 1 && k <= E && k <= kMaxK &&
           (long long)M * k <= INT_MAX && (long long)M * E <= (long long)INT_MAX * 16;
}

long long max_tasks_ll(int M, int k, int E, int n_blocks, int chunk_rows) {
    const long long R = (long long)M * k;
    const long long nonempty = R < E ? R : E;
    return (R / chunk_rows + nonempty) * n_blocks;
}

// ---- workspace of moe_forward ----------------------------------------------------------
constexpr int kWsParts = 15;
struct WsLayout {
    size_t off[kWsParts];
    size_t total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int M, int E, int k, int K, int N) {
    const size_t R = (size_t)M * k;
    const int Nb = N / 128;
    const size_t tasks = (size_t)max_tasks_ll(M, k, E, Nb, 1);  // any chunk_rows fits
    const size_t sz[kWsParts] = {
        R * 4,                      // 0 topk_ids
        R * 4,                      // 1 topk_weights
        (size_t)E * 4,              // 2 counts
        (size_t)(E + 1) * 4,        // 3 offsets
        (size_t)E * 4,              // 4 cursors
        tasks * sizeof(moe_task),   // 5 tasks
        4,                          // 6 ntasks
        MOE_QUEUE_WORDS * 4,        // 7 task counters
        R * 4,                      // 8 sorted_route_ids
        R * (size_t)K,              // 9 a_q
        (size_t)(K / 128) * R * 4,  // 10 a_scales
        R * (size_t)N * 4,          // 11 GEMM rows, sorted order
        R * 4,                      // 12 route_slots
        (size_t)M * K,              // 13 x_q (token-major codes)
        (size_t)(K / 128) * M * 4,  // 14 x_scales
    };
    WsLayout L;
    size_t p = 0;
    for (int i = 0; i < kWsParts; ++i) {
        L.off[i] = p;
        p = align256(p + sz[i]);
    }
    L.total = p;
    return L;
}

bool forward_dims_ok(int M, int E, int k, int K, int N) {
    return M >= 1 && route_dims_ok(M, E, k) && K >= 128 && K % 128 == 0 && N >= 128 &&
           N % 128 == 0 && (long long)M * k * (long long)K < (1LL << 40);
}

// Task chunk of the forward's grouped GEMM: 16 routed rows (the streaming forms) while experts
// average at most 16 rows, else 128 (the LDS-tiled form; K <= 8192) or 64 (the general form).
int default_chunk(int M, int k, int E, int K) {
    const long long avg = ((long long)M * k + E - 1) / E;
    if (avg <= 16) return 16;
    return K <= 8192 ? 128 : 64;
}

// ---- the enqueued step -----------------------------------------------------------------
struct FwdArgs {
    const float* logits;
    const uint16_t* x;
    const uint8_t* w_q;
    const float* w_scales;
    int M, E, k, K, N;
    float softcap;
    uint16_t* out;
    void* ws;
    int chunk, flags;
};

constexpr int kFwdFlagBits = MOE_FWD_GRAPH | MOE_FWD_STATIC_GRID | MOE_FWD_STAGED |
                             MOE_FWD_SCHED_MASK | MOE_FWD_ATOMIC_COMBINE |
                             MOE_FWD_ROUTE_KERNEL | MOE_FWD_ROUTE_SELF;

// Whether the step runs as two kernels: the small-batch GEMM with the route inside, then the
// combine (the default wherever that GEMM can route).
bool fwd_route_fused(int M, int E, int k, int K, int N, int chunk, int flags) {
    return !(flags & (MOE_FWD_ROUTE_KERNEL | MOE_FWD_STAGED)) &&
           forward_fused_applies(M, k, E, K, N, chunk) && fused_route_applies(M, k, E);
}
bool fwd_flags_ok(int flags) {
    return !(flags & ~kFwdFlagBits) && ((flags & MOE_FWD_SCHED_MASK) >> 3) <= 4;
}

// Task schedule of the forward's tiled gathering GEMM: the one the flags name, else the
// default for the chunk size (the persistent forms exist for chunks of at most 128 rows).
int fwd_sched(int flags, int chunk) {
    const int s = ((flags & MOE_FWD_SCHED_MASK) >> 3) - 1;
    if (s >= 0) return s;
    (void)chunk;
    return MOE_SCHED_DISPATCH;
}

hipError_t enqueue_forward(const FwdArgs& a, hipStream_t s) {
    const WsLayout L = ws_layout(a.M, a.E, a.k, a.K, a.N);
    char* base = static_cast<char*>(a.ws);
    auto at = [&](int i) { return base + L.off[i]; };
    int32_t* ids = reinterpret_cast<int32_t*>(at(0));
    float* wts = reinterpret_cast<float*>(at(1));
    int32_t* counts = reinterpret_cast<int32_t*>(at(2));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(3));
    int32_t* cursors = reinterpret_cast<int32_t*>(at(4));
    moe_task* tasks = reinterpret_cast<moe_task*>(at(5));
    int32_t* ntasks = reinterpret_cast<int32_t*>(at(6));
    uint32_t* queue = reinterpret_cast<uint32_t*>(at(7));
    int32_t* sorted = reinterpret_cast<int32_t*>(at(8));
    uint8_t* a_q = reinterpret_cast<uint8_t*>(at(9));
    float* a_s = reinterpret_cast<float*>(at(10));
    float* rows = reinterpret_cast<float*>(at(11));
    int32_t* slots = reinterpret_cast<int32_t*>(at(12));
    const int Nb = a.N / 128;
    const int max_tasks = (int)max_tasks_ll(a.M, a.k, a.E, Nb, a.chunk);
    hipError_t e;
    if (!(a.flags & MOE_FWD_STAGED) && gemm_fp8_tile_applies(a.K, a.chunk)) {
        // larger batch: each token quantised once while it is routed; the layout sorts the
        // routes; the tiled GEMM gathers each routed row from the token-major codes
        uint8_t* x_q = reinterpret_cast<uint8_t*>(at(13));
        float* x_s = reinterpret_cast<float*>(at(14));
        // the scatter-add form accumulates into fp32 token rows [M][N] (in the rows' space),
        // zeroed by the route kernel
        const bool atomic = a.flags & MOE_FWD_ATOMIC_COMBINE;
        if ((e = launch_route_quantize(a.logits, a.x, a.M, a.E, a.k, a.K, a.softcap, ids, wts,
                                       x_q, x_s, s, atomic ? rows : nullptr, a.N)) !=
            hipSuccess)
            return e;
        if ((e = launch_layout_sorted_wide(ids, a.M, a.k, a.E, Nb, a.chunk, counts, offsets,
                                           cursors, tasks, ntasks, queue, sorted, s)) !=
            hipSuccess)
            return e;
        if (atomic) {
            if ((e = launch_gemm_fp8_tile_gather_atomic(x_q, x_s, a.M, a.k, a.K, a.w_q,
                                                        a.w_scales, a.N, tasks, ntasks,
                                                        max_tasks, a.chunk, sorted, wts, rows,
                                                        s)) != hipSuccess)
                return e;
            return launch_acc_to_bf16(rows, a.M, a.N, a.out, s);
        }
        if ((e = launch_gemm_fp8_tile_gather(x_q, x_s, a.M, a.k, a.K, a.w_q, a.w_scales, a.N,
                                             tasks, ntasks, max_tasks, a.chunk, sorted, rows,
                                             fwd_sched(a.flags, a.chunk), queue, s)) !=
            hipSuccess)
            return e;
        return launch_scatter(rows, nullptr, wts, ids, a.M, a.k, a.E, a.N, a.out, s);
    }
    if (fwd_route_fused(a.M, a.E, a.k, a.K, a.N, a.chunk, a.flags)) {
        // two kernels: the route runs inside the GEMM, handing the routes over through tagged
        // words in the otherwise unused route_slots part; the combine clears them again
        uint32_t* handoff = reinterpret_cast<uint32_t*>(slots);
        if ((e = launch_gemm_fp8_fused_route(a.logits, a.x, a.M, a.k, a.E, a.K, a.softcap, a.w_q,
                                             a.w_scales, a.N, ids, wts, handoff,
                                             queue + MOE_QUEUE_HANDOFF_STATUS, rows,
                                             (a.flags & MOE_FWD_ROUTE_SELF) != 0, s)) !=
            hipSuccess)
            return e;
        return launch_scatter(rows, nullptr, wts, ids, a.M, a.k, a.E, a.N, a.out, s, handoff,
                              a.M * a.k);
    }
    if ((e = launch_route(a.logits, a.M, a.E, a.k, a.softcap, ids, wts, s)) != hipSuccess) return e;
    if (!(a.flags & MOE_FWD_STAGED) && forward_fused_applies(a.M, a.k, a.E, a.K, a.N, a.chunk)) {
        // small batch: layout, sort/gather and quantisation run inside the GEMM, whose fp32
        // rows land at their route ids
        if ((e = launch_gemm_fp8_fused(a.x, ids, a.M, a.k, a.E, a.K, a.w_q, a.w_scales, a.N, rows,
                                       s)) != hipSuccess)
            return e;
        return launch_scatter(rows, nullptr, wts, ids, a.M, a.k, a.E, a.N, a.out, s);
    }
    if ((e = launch_layout(ids, a.M, a.k, a.E, Nb, a.chunk, counts, offsets, cursors, tasks,
                           max_tasks, ntasks, queue, nullptr, nullptr, s)) != hipSuccess)
        return e;
    if ((e = launch_qsg(a.x, a.M, a.K, ids, a.k, a.E, cursors, sorted, slots, a_q, a_s, s)) !=
        hipSuccess)
        return e;
    uint32_t* q = (a.flags & MOE_FWD_STATIC_GRID) ? nullptr : queue;
    // fp32 rows at their route ids: the combine reads a token's k rows without a slot table
    if ((e = launch_gemm_fp8(a_q, a_s, a.M * a.k, a.K, a.w_q, a.w_scales, a.E, a.N, tasks,
                             ntasks, max_tasks, a.chunk, q, MOE_EPI_ROUTE_F32, sorted, rows,
                             s)) != hipSuccess)
        return e;
    return launch_scatter(rows, nullptr, wts, ids, a.M, a.k, a.E, a.N, a.out, s);
}

// graph cache: one executable graph per (device, arguments)
struct GraphEntry {
    int dev;
    FwdArgs args;
    hipGraphExec_t exec;
};
std::vector<GraphEntry> g_graphs;
constexpr size_t kMaxGraphs = 64;

bool same_args(const FwdArgs& a, const FwdArgs& b) {
    return a.logits == b.logits && a.x == b.x && a.w_q == b.w_q && a.w_scales == b.w_scales &&
           a.M == b.M && a.E == b.E && a.k == b.k && a.K == b.K && a.N == b.N &&
           std::memcmp(&a.softcap, &b.softcap, sizeof(float)) == 0 && a.out == b.out &&
           a.ws == b.ws && a.chunk == b.chunk && a.flags == b.flags;
}

int forward_graph(const FwdArgs& a, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_mu);
    const int dev = t_dev;
    for (auto& g : g_graphs)
        if (g.dev == dev && same_args(g.args, a)) return hip_status(hipGraphLaunch(g.exec, s));
    DevState& d = g_dev[dev];
    if (!d.capture) {
        if (hipStreamCreateWithFlags(&d.capture, hipStreamNonBlocking) != hipSuccess) {
            d.capture = nullptr;
            return MOE_E_HIP;
        }
    }
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(d.capture, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return MOE_E_HIP;
    const hipError_t le = enqueue_forward(a, d.capture);
    const hipError_t ce = hipStreamEndCapture(d.capture, &graph);
    if (le != hipSuccess || ce != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        (void)hipGetLastError();
        return MOE_E_HIP;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ie != hipSuccess) return MOE_E_HIP;
    if (g_graphs.size() >= kMaxGraphs) {
        (void)hipGraphExecDestroy(g_graphs.front().exec);
        g_graphs.erase(g_graphs.begin());
    }
    g_graphs.push_back(GraphEntry{dev, a, exec});
    return hip_status(hipGraphLaunch(exec, s));
}

// ---- scratch of the no-allocation forward ------------------------------------------------
// moe_forward_noalloc's workspace: a file-scope device array, one copy per GPU the library
// runs on, held until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is a stand-in, not a device address): the address of the current device's
// copy is looked up once per device and kept in DevState::scratch.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The current device's scratch address (check_device() has set t_dev to that device).
int noalloc_scratch(void** out) {
    DevState& d = g_dev[t_dev];
    if (!d.scratch) {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!d.scratch) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return MOE_E_HIP;
            }
            d.scratch = p;
        }
    }
    *out = d.scratch;
    return MOE_OK;
}

}  // namespace

const DeviceInfo& device_info() { return g_dev[t_dev].info; }

// ---- Mixtral-like expert FFN layer (BF16) ---------------------------------------------
constexpr int kFfnParts = 13;
struct FfnLayout {
    size_t off[kFfnParts];
    size_t total;
};
bool ffn_dims_ok(int M, int E, int k, int H, int F) {
    return M >= 1 && route_dims_ok(M, E, k) && H >= 256 && H % 256 == 0 && F >= 128 &&
           F % 128 == 0 && (long long)M * k * (long long)(H > F ? H : F) < (1LL << 40);
}
FfnLayout ffn_layout(int M, int E, int k, int H, int F) {
    const size_t R = (size_t)M * k;
    const size_t tu = (size_t)max_tasks_ll(M, k, E, 2 * F / 256, 1);
    const size_t td = (size_t)max_tasks_ll(M, k, E, H / 256, 1);
    const size_t sz[kFfnParts] = {
        R * 4,                     // 0 topk_ids
        R * 4,                     // 1 topk_weights
        (size_t)E * 4,             // 2 counts
        (size_t)(E + 1) * 4,       // 3 offsets
        (size_t)E * 4,             // 4 cursors
        tu * sizeof(moe_task),     // 5 tasks of the gated-up GEMM
        td * sizeof(moe_task),     // 6 tasks of the down GEMM
        16,                        // 7 ntasks (up, down)
        R * 4,                     // 8 sorted_route_ids
        R * 4,                     // 9 route_slots
        R * (size_t)F * 2,         // 10 act = silu(gate) * up, bf16 [R][F]
        R * (size_t)H * 4,         // 11 down-projection rows, f32 [R][H]
        2 * MOE_QUEUE_WORDS * 4,   // 12 task counters of the two GEMMs
    };
    FfnLayout L;
    size_t p = 0;
    for (int i = 0; i < kFfnParts; ++i) {
        L.off[i] = p;
        p = align256(p + sz[i]);
    }
    L.total = p;
    return L;
}

// ---- FP8 expert MLP layer ---------------------------------------------------------------
constexpr int kMlpParts = 16;
struct MlpLayout {
    size_t off[kMlpParts];
    size_t total;
};
bool mlp_dims_ok(int M, int E, int k, int H, int I) {
    return M >= 1 && route_dims_ok(M, E, k) && H >= 128 && H % 128 == 0 && I >= 128 &&
           I % 128 == 0 && (long long)M * k * (long long)(H > 2 * I ? H : 2 * I) < (1LL << 40);
}
MlpLayout mlp_layout(int M, int E, int k, int H, int I) {
    const size_t R = (size_t)M * k;
    const size_t tu = (size_t)max_tasks_ll(M, k, E, 2 * I / 128, 1);  // any chunk_rows fits
    const size_t td = (size_t)max_tasks_ll(M, k, E, H / 128, 1);
    const size_t sz[kMlpParts] = {
        R * 4,                        // 0 topk_ids
        R * 4,                        // 1 topk_weights
        (size_t)E * 4,                // 2 counts
        (size_t)(E + 1) * 4,          // 3 offsets
        (size_t)E * 4,                // 4 cursors
        tu * sizeof(moe_task),        // 5 gate+up tasks
        td * sizeof(moe_task),        // 6 down tasks
        64 + 2 * MOE_QUEUE_WORDS * 4, // 7 ntasks (2) at +0, task counters (2 x 16) at +64
        R * 4,                        // 8 sorted_route_ids
        R * 4,                        // 9 route_slots
        R * (size_t)H,                // 10 x codes, sorted
        (size_t)(H / 128) * R * 4,    // 11 x scales [H/128][R]
        R * (size_t)(2 * I) * 4,      // 12 gate+up rows f32, sorted
        R * (size_t)I,                // 13 act codes, sorted
        (size_t)(I / 128) * R * 4,    // 14 act scales [I/128][R]
        R * (size_t)H * 4,            // 15 down rows f32 at route ids
    };
    MlpLayout L;
    size_t p = 0;
    for (int i = 0; i < kMlpParts; ++i) {
        L.off[i] = p;
        p = align256(p + sz[i]);
    }
    L.total = p;
    return L;
}
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_E_INVAL: return "MOE_E_INVAL: invalid argument";
        case MOE_E_NOSPC: return "MOE_E_NOSPC: buffer too small";
        case MOE_E_HIP: return "MOE_E_HIP: HIP launch or runtime error";
        case MOE_E_DEVICE: return "MOE_E_DEVICE: no gfx950 device";
        default: return "unknown status";
    }
}

int moe_device_check(void) { return check_device(); }

int moe_route(const float* logits, int M, int E, int k, float softcap, int32_t* topk_ids,
              float* topk_weights, moe_stream_t stream) {
    if (!route_dims_ok(M, E, k)) return MOE_E_INVAL;
    if (M > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_E_INVAL;
    if (softcap != softcap) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_route(logits, M, E, k, softcap, topk_ids, topk_weights,
                                   (hipStream_t)stream));
}

int moe_router_logits(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                      float* logits, moe_stream_t stream) {
    if (M < 0 || H < 64 || H % 64 || E < 1 || E > kMaxE || (long long)M * H >= (1LL << 40))
        return MOE_E_INVAL;
    if ((long long)((M + 15) / 16) * ((E + 15) / 16) > 0x7FFFFFFFLL) return MOE_E_INVAL;
    if (M > 0 && (!x || !w_gate || !logits)) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_router_logits(x, M, H, w_gate, E, logits, (hipStream_t)stream));
}

int moe_route_quantize(const float* logits, const uint16_t* x, int M, int E, int k, int K,
                       float softcap, int32_t* topk_ids, float* topk_weights, uint8_t* x_q,
                       float* x_scales, moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || K < 128 || K % 128 || (long long)M * K >= (1LL << 40))
        return MOE_E_INVAL;
    if (M > 0 && (!logits || !x || !topk_ids || !topk_weights || !x_q || !x_scales))
        return MOE_E_INVAL;
    if (softcap != softcap) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_route_quantize(logits, x, M, E, k, K, softcap, topk_ids,
                                            topk_weights, x_q, x_scales, (hipStream_t)stream));
}

int moe_max_tasks(int M, int k, int E, int n_blocks, int chunk_rows) {
    if (!route_dims_ok(M, E, k) || n_blocks < 1 || chunk_rows < 1 || chunk_rows > 1024)
        return -1;
    const long long v = max_tasks_ll(M, k, E, n_blocks, chunk_rows);
    return v > INT_MAX ? -1 : (int)v;
}

int moe_build_layout(const int32_t* topk_ids, int M, int k, int E, int n_blocks,
                     int chunk_rows, int32_t* counts, int32_t* offsets, int32_t* cursors,
                     moe_task* tasks, int max_tasks, int32_t* ntasks, uint32_t* queue,
                     int32_t* sorted_route_ids, int32_t* route_slots, moe_stream_t stream) {
    const int need = moe_max_tasks(M, k, E, n_blocks, chunk_rows);
    if (need < 0) return MOE_E_INVAL;
    if ((M > 0 && !topk_ids) || !counts || !offsets || !cursors || !ntasks || !queue)
        return MOE_E_INVAL;
    if (route_slots && !sorted_route_ids) return MOE_E_INVAL;
    if (need > 0 && !tasks) return MOE_E_INVAL;
    if (max_tasks < need) return MOE_E_NOSPC;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_layout(topk_ids, M, k, E, n_blocks, chunk_rows, counts, offsets,
                                    cursors, tasks, max_tasks, ntasks, queue,
                                    M > 0 ? sorted_route_ids : nullptr, route_slots,
                                    (hipStream_t)stream));
}

int moe_quant_sort_gather(const uint16_t* x, int M, int K, const int32_t* topk_ids, int k,
                          int E, int32_t* cursors, int32_t* sorted_route_ids,
                          int32_t* route_slots, uint8_t* a_q, float* a_scales,
                          moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || K < 128 || K % 128) return MOE_E_INVAL;
    if (M > 0 && (!x || !topk_ids || !cursors || !sorted_route_ids || !a_q || !a_scales))
        return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_qsg(x, M, K, topk_ids, k, E, cursors, sorted_route_ids,
                                 route_slots, a_q, a_scales, (hipStream_t)stream));
}

int moe_sort_gather_bf16(const uint16_t* x, int M, int K, const int32_t* topk_ids, int k,
                         int E, int32_t* cursors, int32_t* sorted_route_ids,
                         int32_t* route_slots, uint16_t* a, moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || K < 8 || K % 8) return MOE_E_INVAL;
    if (M > 0 && (!x || !topk_ids || !cursors || !sorted_route_ids || !a)) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_gather_bf16(x, M, K, topk_ids, k, E, cursors, sorted_route_ids,
                                         route_slots, a, (hipStream_t)stream));
}

int moe_quantize_weights(const float* w, int E, int N, int K, uint8_t* w_q, float* w_scales,
                         moe_stream_t stream) {
    if (E < 1 || N < 128 || K < 128 || N % 128 || K % 128 || !w || !w_q || !w_scales)
        return MOE_E_INVAL;
    if ((long long)E * (N / 128) * (K / 128) > INT_MAX) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_quantize_weights(w, E, N, K, w_q, w_scales, (hipStream_t)stream));
}

int moe_gemm_n_tile(int mode) {
    return mode == MOE_GEMM_FP8_B128 ? 128 : mode == MOE_GEMM_BF16 ? 256 : -1;
}

int moe_grouped_gemm(int mode, const void* a, const float* a_scales, int rows, int K,
                     const void* w, const float* w_scales, int E, int N,
                     const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                     int chunk_rows, uint32_t* queue, int epilogue,
                     const int32_t* sorted_route_ids, void* out, int sched,
                     moe_stream_t stream) {
    if (sched < MOE_SCHED_AUTO || sched > MOE_SCHED_QUEUE_XCD) return MOE_E_INVAL;
    if (mode == MOE_GEMM_BF16) {
        if ((sched == MOE_SCHED_QUEUE || sched == MOE_SCHED_QUEUE_XCD) && !queue)
            return MOE_E_INVAL;
        if (rows < 0 || E < 1 || K < 64 || K % 64 || N < 256 || N % 256 || max_tasks < 0)
            return MOE_E_INVAL;
        if (chunk_rows < 1 || chunk_rows > 256) return MOE_E_INVAL;
        if (epilogue != MOE_EPI_STORE_F32 && epilogue != MOE_EPI_STORE_BF16 &&
            epilogue != MOE_EPI_SWIGLU_BF16)
            return MOE_E_INVAL;
        if (!w || !ntasks || !out || (max_tasks > 0 && !tasks)) return MOE_E_INVAL;
        if (rows > 0 && !a) return MOE_E_INVAL;
        if ((long long)E * N * K > (1ll << 40)) return MOE_E_INVAL;
        int rc = check_device();
        if (rc) return rc;
        return hip_status(launch_gemm_bf16(static_cast<const uint16_t*>(a), K,
                                           static_cast<const uint16_t*>(w), N, tasks, ntasks,
                                           max_tasks, epilogue, out, (hipStream_t)stream,
                                           nullptr, 1, sched, queue));
    }
    if (mode != MOE_GEMM_FP8_B128) return MOE_E_INVAL;
    if (sched != MOE_SCHED_AUTO) return MOE_E_INVAL;   // FP8: the task walk follows `queue`
    if (rows < 0 || E < 1 || K < 128 || K % 128 || N < 128 || N % 128 || max_tasks < 0)
        return MOE_E_INVAL;
    if (chunk_rows < 1 || chunk_rows > 256 || (chunk_rows > 64 && K > 8192)) return MOE_E_INVAL;
    if (epilogue != MOE_EPI_STORE_F32 && epilogue != MOE_EPI_STORE_BF16 &&
        epilogue != MOE_EPI_ROUTE_F32)
        return MOE_E_INVAL;
    if (!w || !w_scales || !ntasks || !out || (max_tasks > 0 && !tasks)) return MOE_E_INVAL;
    if (rows > 0 && (!a || !a_scales)) return MOE_E_INVAL;
    if (epilogue == MOE_EPI_ROUTE_F32 && !sorted_route_ids) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_gemm_fp8(static_cast<const uint8_t*>(a), a_scales, rows, K,
                                      static_cast<const uint8_t*>(w), w_scales, E, N, tasks,
                                      ntasks, max_tasks, chunk_rows, queue, epilogue,
                                      sorted_route_ids, out, (hipStream_t)stream));
}

int moe_grouped_gemm_routed(const uint16_t* x, const int32_t* topk_ids, int M, int k, int E,
                            int K, const uint8_t* w_q, const float* w_scales, int N,
                            float* rows, int32_t* counts, int32_t* offsets,
                            moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || M < 1 || N < 128 || N % 128) return MOE_E_INVAL;
    if (!x || !topk_ids || !w_q || !w_scales || !rows || (!counts != !offsets))
        return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    if (!forward_fused_applies(M, k, E, K, N, 16)) return MOE_E_INVAL;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_gemm_fp8_fused(x, topk_ids, M, k, E, K, w_q, w_scales, N, rows, s);
    if (e == hipSuccess && counts) e = launch_counts(topk_ids, M, k, E, counts, offsets, s);
    return hip_status(e);
}

int moe_route_grouped_gemm(const float* logits, const uint16_t* x, int M, int E, int k, int K,
                           float softcap, const uint8_t* w_q, const float* w_scales, int N,
                           int32_t* topk_ids, float* topk_weights, uint32_t* route_words,
                           uint32_t* status, float* rows, moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || M < 1 || N < 128 || N % 128 || softcap != softcap)
        return MOE_E_INVAL;
    if (!logits || !x || !w_q || !w_scales || !topk_ids || !topk_weights || !route_words ||
        !status || !rows)
        return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    if (!forward_fused_applies(M, k, E, K, N, 16) || !fused_route_applies(M, k, E))
        return MOE_E_INVAL;
    return hip_status(launch_gemm_fp8_fused_route(logits, x, M, k, E, K, softcap, w_q, w_scales,
                                                  N, topk_ids, topk_weights, route_words,
                                                  status, rows, false, (hipStream_t)stream));
}

int moe_grouped_gemm_gather(const uint8_t* x_q, const float* x_scales, int M, int k, int K,
                            const uint8_t* w, const float* w_scales, int E, int N,
                            const moe_task* tasks, const int32_t* ntasks, int max_tasks,
                            int chunk_rows, const int32_t* sorted_route_ids, float* rows,
                            uint32_t* queue, int sched, moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || K < 128 || K % 128 || N < 128 || N % 128 || max_tasks < 0)
        return MOE_E_INVAL;
    if (!gemm_fp8_tile_applies(K, chunk_rows)) return MOE_E_INVAL;
    if (!w || !w_scales || !ntasks || !rows || (max_tasks > 0 && !tasks)) return MOE_E_INVAL;
    if (M > 0 && (!x_q || !x_scales || !sorted_route_ids)) return MOE_E_INVAL;
    if (sched < MOE_SCHED_AUTO || sched > MOE_SCHED_QUEUE_XCD) return MOE_E_INVAL;
    if (sched == MOE_SCHED_AUTO) sched = fwd_sched(0, chunk_rows);
    if (sched != MOE_SCHED_DISPATCH && chunk_rows > 128) return MOE_E_INVAL;
    if ((sched == MOE_SCHED_QUEUE || sched == MOE_SCHED_QUEUE_XCD) && !queue) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_gemm_fp8_tile_gather(x_q, x_scales, M, k, K, w, w_scales, N, tasks,
                                                  ntasks, max_tasks, chunk_rows,
                                                  sorted_route_ids, rows, sched, queue,
                                                  (hipStream_t)stream));
}

int moe_scatter(const float* rows, const int32_t* route_slots, const float* topk_weights,
                const int32_t* topk_ids, int M, int k, int E, int N, uint16_t* out,
                moe_stream_t stream) {
    if (!route_dims_ok(M, E, k) || N < 4 || N % 4) return MOE_E_INVAL;
    if (M > 0 && (!rows || !topk_weights || !topk_ids || !out)) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_scatter(rows, route_slots, topk_weights, topk_ids, M, k, E, N, out,
                                     (hipStream_t)stream));
}

size_t moe_forward_workspace_bytes(int M, int E, int k, int K, int N) {
    if (!forward_dims_ok(M, E, k, K, N)) return 0;
    return ws_layout(M, E, k, K, N).total;
}

int64_t moe_forward_workspace_offset(int M, int E, int k, int K, int N, int which) {
    if (!forward_dims_ok(M, E, k, K, N) || which < 0 || which >= kWsParts) return -1;
    return (int64_t)ws_layout(M, E, k, K, N).off[which];
}

int moe_forward_ex(const float* logits, const uint16_t* x, const uint8_t* w_q,
                   const float* w_scales, int M, int E, int k, int K, int N, float softcap,
                   uint16_t* out, void* workspace, size_t workspace_bytes, int chunk_rows,
                   int flags, moe_stream_t stream) {
    if (!forward_dims_ok(M, E, k, K, N)) return MOE_E_INVAL;
    if (!logits || !x || !w_q || !w_scales || !out || !workspace) return MOE_E_INVAL;
    if (softcap != softcap) return MOE_E_INVAL;
    if (chunk_rows < 0 || chunk_rows > 256 || (chunk_rows > 64 && K > 8192)) return MOE_E_INVAL;
    if (!fwd_flags_ok(flags)) return MOE_E_INVAL;
    if (workspace_bytes < ws_layout(M, E, k, K, N).total) return MOE_E_NOSPC;
    const int chunk = chunk_rows ? chunk_rows : default_chunk(M, k, E, K);
    const int sched = ((flags & MOE_FWD_SCHED_MASK) >> 3) - 1;
    if (sched > MOE_SCHED_DISPATCH && chunk > 128) return MOE_E_INVAL;
    // the scatter-add form exists for the gathering tiled path under hardware dispatch
    if ((flags & MOE_FWD_ATOMIC_COMBINE) &&
        ((flags & MOE_FWD_STAGED) || !gemm_fp8_tile_applies(K, chunk) || sched > 0))
        return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    FwdArgs a{logits, x, w_q, w_scales, M, E, k, K, N, softcap, out, workspace, chunk, flags};
    hipStream_t s = (hipStream_t)stream;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_E_HIP;
    }
    if (!(flags & MOE_FWD_GRAPH) || cs != hipStreamCaptureStatusNone)
        return hip_status(enqueue_forward(a, s));
    return forward_graph(a, s);
}

int moe_forward_kernels(int M, int E, int k, int K, int N, int chunk_rows, int flags) {
    if (!forward_dims_ok(M, E, k, K, N)) return MOE_E_INVAL;
    if (chunk_rows < 0 || chunk_rows > 256 || (chunk_rows > 64 && K > 8192)) return MOE_E_INVAL;
    if (!fwd_flags_ok(flags)) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    const int chunk = chunk_rows ? chunk_rows : default_chunk(M, k, E, K);
    if (flags & MOE_FWD_STAGED) return 5;
    if (gemm_fp8_tile_applies(K, chunk)) return 4;
    if (fwd_route_fused(M, E, k, K, N, chunk, flags)) return 2;
    return forward_fused_applies(M, k, E, K, N, chunk) ? 3 : 5;
}

int moe_forward(const float* logits, const uint16_t* x, const uint8_t* w_q,
                const float* w_scales, int M, int E, int k, int K, int N, float softcap,
                uint16_t* out, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
    return moe_forward_ex(logits, x, w_q, w_scales, M, E, k, K, N, softcap, out, workspace,
                          workspace_bytes, 0, 0, stream);
}

int moe_forward_noalloc(const float* logits, const uint16_t* x, const uint8_t* w_q,
                        const float* w_scales, int M, int E, int k, int K, int N, float softcap,
                        uint16_t* out, moe_stream_t stream) {
    if (!forward_dims_ok(M, E, k, K, N)) return MOE_E_INVAL;
    if (!logits || !x || !w_q || !w_scales || !out) return MOE_E_INVAL;
    if (softcap != softcap) return MOE_E_INVAL;
    if (ws_layout(M, E, k, K, N).total > kNoAllocScratchBytes) return MOE_E_NOSPC;
    int rc = check_device();
    if (rc) return rc;
    void* ws = nullptr;
    if ((rc = noalloc_scratch(&ws)) != MOE_OK) return rc;
    // the same kernels as moe_forward, plain launches; each path clears what it accumulates
    // into (the route kernel zeroes the layout's counters, the layout resets the queue), so
    // whatever the last call left in the scratch does not matter
    FwdArgs a{logits, x, w_q, w_scales, M, E, k, K, N, softcap, out, ws,
              default_chunk(M, k, E, K), 0};
    return hip_status(enqueue_forward(a, (hipStream_t)stream));
}

// ---- Mixtral-like expert FFN layer (BF16) ---------------------------------------------
size_t moe_ffn_workspace_bytes(int M, int E, int k, int H, int F) {
    if (!ffn_dims_ok(M, E, k, H, F)) return 0;
    return ffn_layout(M, E, k, H, F).total;
}

int64_t moe_ffn_workspace_offset(int M, int E, int k, int H, int F, int which) {
    if (!ffn_dims_ok(M, E, k, H, F) || which < 0 || which >= kFfnParts) return -1;
    return (int64_t)ffn_layout(M, E, k, H, F).off[which];
}

int moe_ffn_forward(const float* logits, const uint16_t* x, const uint16_t* w_up,
                    const uint16_t* w_down, int M, int E, int k, int H, int F, float softcap,
                    uint16_t* out, void* workspace, size_t workspace_bytes, int chunk_rows,
                    int flags, moe_stream_t stream) {
    if (!ffn_dims_ok(M, E, k, H, F)) return MOE_E_INVAL;
    if (!logits || !x || !w_up || !w_down || !out || !workspace) return MOE_E_INVAL;
    if (softcap != softcap) return MOE_E_INVAL;
    if (chunk_rows < 0 || chunk_rows > 256) return MOE_E_INVAL;
    if ((flags & ~MOE_FWD_SCHED_MASK) || ((flags & MOE_FWD_SCHED_MASK) >> 3) > 4)
        return MOE_E_INVAL;
    const int sched = ((flags & MOE_FWD_SCHED_MASK) >> 3) - 1;   // -1: the default
    const FfnLayout L = ffn_layout(M, E, k, H, F);
    if (workspace_bytes < L.total) return MOE_E_NOSPC;
    int rc = check_device();
    if (rc) return rc;
    const int chunk = chunk_rows ? chunk_rows : 256;
    char* base = static_cast<char*>(workspace);
    auto at = [&](int i) { return base + L.off[i]; };
    int32_t* ids = reinterpret_cast<int32_t*>(at(0));
    float* wts = reinterpret_cast<float*>(at(1));
    int32_t* counts = reinterpret_cast<int32_t*>(at(2));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(3));
    int32_t* cursors = reinterpret_cast<int32_t*>(at(4));
    moe_task* tu = reinterpret_cast<moe_task*>(at(5));
    moe_task* td = reinterpret_cast<moe_task*>(at(6));
    int32_t* nt = reinterpret_cast<int32_t*>(at(7));
    int32_t* sorted = reinterpret_cast<int32_t*>(at(8));
    int32_t* slots = reinterpret_cast<int32_t*>(at(9));
    uint16_t* act = reinterpret_cast<uint16_t*>(at(10));
    float* down = reinterpret_cast<float*>(at(11));
    uint32_t* queue = reinterpret_cast<uint32_t*>(at(12));
    const int nbu = 2 * F / 256, nbd = H / 256;
    const int mtu = (int)max_tasks_ll(M, k, E, nbu, chunk);
    const int mtd = (int)max_tasks_ll(M, k, E, nbd, chunk);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // route; the layout over many workgroups in one launch (sorted route ids, route -> slot,
    // both task lists); gated-up GEMM gathering its rows from x on load with the SwiGLU
    // epilogue; down GEMM; combine through the slot table
    if ((e = launch_route(logits, M, E, k, softcap, ids, wts, s)) !=
            hipSuccess ||
        (e = launch_layout_sorted_wide(ids, M, k, E, nbu, chunk, counts, offsets, cursors, tu,
                                       nt, queue, sorted, s, slots, nbd, td, nt + 1,
                                       queue + MOE_QUEUE_WORDS)) != hipSuccess ||
        (e = launch_gemm_bf16(x, H, w_up, 2 * F, tu, nt, mtu, MOE_EPI_SWIGLU_BF16, act, s,
                              sorted, k, sched, queue)) != hipSuccess ||
        (e = launch_gemm_bf16(act, F, w_down, H, td, nt + 1, mtd, MOE_EPI_STORE_F32, down, s,
                              nullptr, 1, sched, queue + MOE_QUEUE_WORDS)) != hipSuccess ||
        (e = launch_scatter(down, slots, wts, ids, M, k, E, H, out, s)) != hipSuccess)
        return hip_status(e);
    return MOE_OK;
}

// ---- FP8 expert MLP layer ---------------------------------------------------------------
int moe_swiglu_quant(const float* h, int rows, int I, uint8_t* a_q, float* a_scales,
                     moe_stream_t stream) {
    if (rows < 0 || I < 128 || I % 128 || (long long)rows * 2 * I >= (1LL << 40))
        return MOE_E_INVAL;
    if (rows > 0 && (!h || !a_q || !a_scales)) return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    return hip_status(launch_swiglu_quant(h, rows, I, a_q, a_scales, (hipStream_t)stream));
}

size_t moe_mlp_workspace_bytes(int M, int E, int k, int H, int I) {
    if (!mlp_dims_ok(M, E, k, H, I)) return 0;
    return mlp_layout(M, E, k, H, I).total;
}

int64_t moe_mlp_workspace_offset(int M, int E, int k, int H, int I, int which) {
    if (!mlp_dims_ok(M, E, k, H, I) || which < 0 || which >= kMlpParts) return -1;
    return (int64_t)mlp_layout(M, E, k, H, I).off[which];
}

}  // extern "C"

namespace {
// Both projections of the FP8 MLP fit the small-batch GEMM: gate+up [M*k] x [2I, H] and down
// [M*k] x [H, I] with its activation step in the tile build.
bool mlp_small_batch(int M, int k, int E, int H, int I, int chunk) {
    return forward_fused_applies(M, k, E, H, 2 * I, chunk) &&
           forward_fused_applies(M, k, E, I, H, chunk);
}
}  // namespace

extern "C" {

int moe_mlp_forward_kernels(int M, int E, int k, int H, int I, int chunk_rows) {
    if (!mlp_dims_ok(M, E, k, H, I)) return MOE_E_INVAL;
    const int Kmax = H > I ? H : I;
    if (chunk_rows < 0 || chunk_rows > 256 || (chunk_rows > 64 && Kmax > 8192))
        return MOE_E_INVAL;
    int rc = check_device();
    if (rc) return rc;
    int chunk = chunk_rows ? chunk_rows : default_chunk(M, k, E, H);
    if (!chunk_rows && chunk > 64 && Kmax > 8192) chunk = 64;
    if (!mlp_small_batch(M, k, E, H, I, chunk)) return 7;
    return fused_route_applies(M, k, E) ? 3 : 4;
}

int moe_mlp_forward(const float* logits, const uint16_t* x, const uint8_t* w1_q,
                    const float* w1_scales, const uint8_t* w2_q, const float* w2_scales, int M,
                    int E, int k, int H, int I, float softcap, uint16_t* out, void* workspace,
                    size_t workspace_bytes, int chunk_rows, moe_stream_t stream) {
    if (!mlp_dims_ok(M, E, k, H, I)) return MOE_E_INVAL;
    if (!logits || !x || !w1_q || !w1_scales || !w2_q || !w2_scales || !out || !workspace)
        return MOE_E_INVAL;
    if (softcap != softcap) return MOE_E_INVAL;
    const int Kmax = H > I ? H : I;
    if (chunk_rows < 0 || chunk_rows > 256 || (chunk_rows > 64 && Kmax > 8192))
        return MOE_E_INVAL;
    const MlpLayout L = mlp_layout(M, E, k, H, I);
    if (workspace_bytes < L.total) return MOE_E_NOSPC;
    int rc = check_device();
    if (rc) return rc;
    int chunk = chunk_rows ? chunk_rows : default_chunk(M, k, E, H);
    if (!chunk_rows && chunk > 64 && Kmax > 8192) chunk = 64;
    char* base = static_cast<char*>(workspace);
    auto at = [&](int i) { return base + L.off[i]; };
    int32_t* ids = reinterpret_cast<int32_t*>(at(0));
    float* wts = reinterpret_cast<float*>(at(1));
    int32_t* counts = reinterpret_cast<int32_t*>(at(2));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(3));
    int32_t* cursors = reinterpret_cast<int32_t*>(at(4));
    moe_task* tu = reinterpret_cast<moe_task*>(at(5));
    moe_task* td = reinterpret_cast<moe_task*>(at(6));
    int32_t* nt = reinterpret_cast<int32_t*>(at(7));
    uint32_t* queue = reinterpret_cast<uint32_t*>(at(7) + 64);
    uint32_t* queue2 = queue + MOE_QUEUE_WORDS;
    int32_t* sorted = reinterpret_cast<int32_t*>(at(8));
    int32_t* slots = reinterpret_cast<int32_t*>(at(9));
    uint8_t* xq = reinterpret_cast<uint8_t*>(at(10));
    float* xs = reinterpret_cast<float*>(at(11));
    float* h1 = reinterpret_cast<float*>(at(12));
    uint8_t* aq = reinterpret_cast<uint8_t*>(at(13));
    float* as = reinterpret_cast<float*>(at(14));
    float* h2 = reinterpret_cast<float*>(at(15));
    const int R = M * k;
    const int nbu = 2 * I / 128, nbd = H / 128;
    const int mtu = (int)max_tasks_ll(M, k, E, nbu, chunk);
    const int mtd = (int)max_tasks_ll(M, k, E, nbd, chunk);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (mlp_small_batch(M, k, E, H, I, chunk)) {
        // small batch: the gate+up GEMM straight from the routed ids (layout, gather and
        // quantisation of x inside; the route too where it can, handing the routes over
        // through tagged words in the unused route_slots part) with rows at route ids; the
        // down GEMM the same way from the same ids, forming and requantising the activations
        // of its rows in its tile build (their codes and scales also land in parts 13-14, in
        // route order)
        uint32_t* handoff = nullptr;
        if (fused_route_applies(M, k, E)) {
            handoff = reinterpret_cast<uint32_t*>(slots);
            e = launch_gemm_fp8_fused_route(logits, x, M, k, E, H, softcap, w1_q, w1_scales, 2 * I,
                                            ids, wts, handoff, queue + MOE_QUEUE_HANDOFF_STATUS,
                                            h1, false, s);
        } else if ((e = launch_route(logits, M, E, k, softcap, ids, wts, s)) == hipSuccess) {
            e = launch_gemm_fp8_fused(x, ids, M, k, E, H, w1_q, w1_scales, 2 * I, h1, s);
        }
        if (e != hipSuccess ||
            (e = launch_gemm_fp8_fused_act(h1, ids, M, k, E, I, w2_q, w2_scales, H, h2, aq, as,
                                           s)) != hipSuccess ||
            (e = launch_scatter(h2, nullptr, wts, ids, M, k, E, H, out, s, handoff,
                                handoff ? R : 0)) != hipSuccess)
            return hip_status(e);
        return MOE_OK;
    }
    if ((e = launch_route(logits, M, E, k, softcap, ids, wts, s)) != hipSuccess ||
        (e = launch_layout2(ids, M, k, E, chunk, counts, offsets, cursors, nbu, tu, nt, queue,
                            nbd, td, nt + 1, queue2, s)) != hipSuccess ||
        (e = launch_qsg(x, M, H, ids, k, E, cursors, sorted, slots, xq, xs, s)) != hipSuccess ||
        (e = launch_gemm_fp8(xq, xs, R, H, w1_q, w1_scales, E, 2 * I, tu, nt, mtu, chunk, queue,
                             MOE_EPI_STORE_F32, sorted, h1, s)) != hipSuccess ||
        (e = launch_swiglu_quant(h1, R, I, aq, as, s)) != hipSuccess ||
        (e = launch_gemm_fp8(aq, as, R, I, w2_q, w2_scales, E, H, td, nt + 1, mtd, chunk,
                             queue2, MOE_EPI_ROUTE_F32, sorted, h2, s)) != hipSuccess ||
        (e = launch_scatter(h2, nullptr, wts, ids, M, k, E, H, out, s)) != hipSuccess)
        return hip_status(e);
    return MOE_OK;
}

}  // extern "C"
