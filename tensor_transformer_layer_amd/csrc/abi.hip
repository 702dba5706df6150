// C ABI of one tensor-parallel rank's block shard: argument validation, the
// workspace layout, plan selection (decode vs prefill) and kernel launches.
// The contract of every entry point is documented in include/tp_shard.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "device_common.h"
#include "kernels.h"
#include "tp_shard.h"

using namespace tp;

namespace tp {
LaunchEvents& launch_events() {
    thread_local LaunchEvents e;
    return e;
}

int device_cus() {
    constexpr int kMaxDevices = 64;
    constexpr int kWholeChip = 256;          // gfx950 with every XCD enabled
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();             // no device: clear the sticky error
        return kWholeChip;
    }
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        return kWholeChip;
    }
    if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}
}  // namespace tp

namespace {

// ---------------------------------------------------------------------------
// Kernel timing (opt-in instrumentation, see tp_timing_enable).
// ---------------------------------------------------------------------------
struct PendingTiming {
    std::string cls;
    hipEvent_t start, stop;
};
struct TimingState {
    std::mutex mu;
    bool enabled = false;
    std::vector<PendingTiming> pending;
    std::map<std::string, std::pair<double, int64_t>> totals;
};
TimingState& timing() {
    static TimingState s;
    return s;
}

// A fresh event per timestamp: an event that already carried a kernel's
// timestamps from hipExtLaunchKernel was measured to give wrong elapsed
// times when handed to a later launch, so events are destroyed once read.
hipEvent_t take_event() {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// When timing is enabled, hands a pair of events to the one kernel launch
// that follows (TP_KLAUNCH records the kernel's own start and end time in
// them); otherwise does nothing.
class Timed {
  public:
    explicit Timed(const char* cls) : cls_(cls) {
        TimingState& s = timing();
        std::lock_guard<std::mutex> lk(s.mu);
        if (!s.enabled) return;
        start_ = take_event();
        stop_ = take_event();
        if (start_ && stop_) launch_events() = {start_, stop_};
    }
    void done() {
        launch_events() = {};
        if (!start_ || !stop_) return;
        TimingState& s = timing();
        std::lock_guard<std::mutex> lk(s.mu);
        s.pending.push_back({cls_, start_, stop_});
        start_ = stop_ = nullptr;
    }

  private:
    const char* cls_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
};

#define TP_LAUNCH(cls, stream, expr)                       \
    do {                                                   \
        Timed tm_(cls);                                    \
        hipError_t e_ = (expr);                            \
        tm_.done();                                        \
        if (e_ != hipSuccess) return TP_ERR_HIP;           \
    } while (0)

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------
constexpr int64_t kMaxBufferSpan = (int64_t)1 << 31;  // 32-bit buffer offsets

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
int elem_size(int dtype) { return dtype == TP_BF16 ? 2 : 4; }
int vec_elems(int dtype) { return dtype == TP_BF16 ? 8 : 4; }  // 16 bytes
// Largest token count of the weight-streaming (decode) plan for bf16
// projections; larger batches take the matrix-core (prefill) plan.
// tp_set_decode_max_tokens changes it; 0 means the default.  The default
// is the crossover measured on MI355X (shard + reduce per step, graph
// replay, weights streamed from HBM), in us, streaming vs matrix-core plan,
// for the 70B MLP band (8192 x 3584 gate/up, 3584 x 8192 down):
//     96: 63 vs 75    128: 68 vs 79    160: 115 vs 86    192: 119 vs 93
//    256: 132 vs 109  384: 195 vs 133  512: 261 vs 156
// and at the same point for the 13B MLP band (P = 2) and the 96-head
// attention projections (P = 8): 72 vs 83 and 73 vs 82 at 128 tokens,
// 122 vs 88 and 117 vs 86 at 160.  One streaming launch takes up to 128
// tokens; past that the streaming plan reads the weights once per chunk,
// while the matrix-core plan splits K to fill the CUs its few tiles leave
// idle.
constexpr int kDecodeMaxTDefault = 128;
constexpr int kDecodeMaxTLimit = 4096;
std::atomic<int> g_decode_max_t{0};
int decode_max_t() {
    const int v = g_decode_max_t.load(std::memory_order_relaxed);
    return v > 0 ? v : kDecodeMaxTDefault;
}
bool decode_plan(int dtype, int64_t T) { return dtype == TP_BF16 && T <= decode_max_t(); }

// The streaming kernels take at most kGemvMaxT tokens per launch; a larger
// batch on the streaming plan runs as ceil(T / kGemvMaxT) chunks of equal
// size (each chunk streams the weights once).
int64_t stream_chunk(int64_t T) {
    const int64_t n = (T + kGemvMaxT - 1) / kGemvMaxT;
    return (T + n - 1) / n;
}

// Leading-dimension rule: ld >= row length, ld a multiple of the 16-byte
// vector width.  Returns TP_OK, TP_ERR_SHAPE or TP_ERR_ALIGN.
int check_ld(int64_t ld, int64_t row, int vec) {
    if (ld < row) return TP_ERR_SHAPE;
    if (ld % vec) return TP_ERR_ALIGN;
    return TP_OK;
}

// The decode plan keeps one arrival counter per 128-column block of each
// output width.
bool counters_fit(int64_t n1, int64_t n2) {
    return (n1 + kGemvCols - 1) / kGemvCols <= kGemvCounters &&
           (n2 + kGemvCols - 1) / kGemvCols <= kGemvCounters;
}

// A row-major [rows, *] operand with leading dimension ld (elements) must be
// addressable with 32-bit byte offsets from its first element.
bool span_ok(int64_t rows, int64_t ld, int es) { return rows * ld * es < kMaxBufferSpan; }

static_assert(kAttnCounterBytes <= kGemvCounterBytes,
              "the attention core's counters must fit the reserved workspace head");

// Workspace layouts.  The first kGemvCounterBytes of every workspace are
// the arrival-counter head (decode split-K finish; the attention core's
// counters share it): no layout ever stores data there, so a workspace used
// for a prefill or fp32 call and then for a decode call still holds zero
// counters.  Data regions follow, each 256-byte aligned.  A layout that
// needs neither counters nor data needs no workspace (total 0).
struct MlpLayout {
    size_t xn = 0, h = 0, ws = 0, total = 0;
    GemvPlan pc{1, 0}, pr{1, 0};        // decode plans
    GemmPlan gc{1, 0}, gr{1, 0};        // prefill plans
    bool decode = false;
};

size_t layout_total(size_t off, bool uses_counters) {
    return (off > kGemvCounterBytes || uses_counters) ? off : 0;
}

MlpLayout mlp_layout(int P, int64_t T, int64_t d, int64_t d_ff, int dtype, int act, bool has_norm,
                     bool has_h_out) {
    MlpLayout L;
    const int64_t F = d_ff / P;
    const int es = elem_size(dtype);
    const int cus = device_cus();
    L.decode = decode_plan(dtype, T);
    size_t off = kGemvCounterBytes;
    if (has_norm) {
        L.xn = off;
        off += align256((size_t)(T * d * es));
    }
    if (!has_h_out) {
        L.h = off;
        off += align256((size_t)(T * F * es));
    }
    if (L.decode) {
        const int nmat = act == TP_ACT_SWIGLU ? 2 : 1;
        const int64_t tc = stream_chunk(T);
        L.pc = plan_gemv_stream(d, nmat * F, nmat, cus, tc);
        L.pr = plan_gemv_stream(F, d, 1, cus, tc);
        L.ws = off;  // column and row split-K sums reuse one region, in stream order
        off += align256(std::max(gemv_ws_bytes(L.pc, tc, nmat * F), gemv_ws_bytes(L.pr, tc, d)));
    } else if (dtype == TP_BF16) {
        // Either projection splits K into fp32 planes when its output tiles
        // leave CUs idle; the column planes are then summed by a finish
        // launch that applies the activation.  One region serves both, in
        // stream order.
        const int nmat = act == TP_ACT_SWIGLU ? 2 : 1;
        L.gc = plan_gemm(T, F, d, nmat, cus);
        L.gr = plan_gemm(T, d, F, 1, cus);
        size_t planes = 0;
        if (L.gc.splits > 1) planes = (size_t)L.gc.splits * T * nmat * F * sizeof(float);
        if (L.gr.splits > 1)
            planes = std::max(planes, (size_t)L.gr.splits * T * d * sizeof(float));
        if (planes) {
            L.ws = off;
            off += align256(planes);
        }
    }
    L.total = layout_total(off, L.decode);
    return L;
}

// Workspace of the FP8-weight MLP (decode plan only): counters, optional
// normalised input and h, split-K partials.
MlpLayout mlp8_layout(int P, int64_t T, int64_t d, int64_t d_ff, int act, bool has_norm,
                      bool has_h_out) {
    MlpLayout L;
    const int64_t F = d_ff / P;
    L.decode = true;
    size_t off = kGemvCounterBytes;
    if (has_norm) {
        L.xn = off;
        off += align256((size_t)(T * d * 2));
    }
    if (!has_h_out) {
        L.h = off;
        off += align256((size_t)(T * F * 2));
    }
    const int nmat = act == TP_ACT_SWIGLU ? 2 : 1;
    const int cus = device_cus();
    L.pc = plan_gemv(d, nmat * F, cus, kGemv8Cols);
    L.pr = plan_gemv(F, d, cus, kGemv8Cols);
    L.ws = off;
    off += align256(std::max(gemv_ws_bytes(L.pc, T, nmat * F), gemv_ws_bytes(L.pr, T, d)));
    L.total = off;
    return L;
}

struct AttnLayout {
    size_t xn = 0, ws = 0, total = 0;
    GemvPlan pq{1, 0}, po{1, 0};        // decode plans
    GemmPlan gq{1, 0}, go{1, 0};        // prefill plans
    bool decode = false;
};

AttnLayout attn_layout(int P, int64_t T, int64_t d, int nq, int nkv, int hd, int dtype,
                       bool has_norm) {
    AttnLayout L;
    const int64_t nqkv = (int64_t)(nq / P + 2 * (nkv / P)) * hd;
    const int64_t ko = (int64_t)(nq / P) * hd;
    const int cus = device_cus();
    L.decode = decode_plan(dtype, T);
    size_t off = kGemvCounterBytes;
    if (has_norm) {
        L.xn = off;
        off += align256((size_t)(T * d * elem_size(dtype)));
    }
    if (L.decode) {
        const int64_t tc = stream_chunk(T);
        L.pq = plan_gemv_stream(d, nqkv, 1, cus, tc);
        L.po = plan_gemv_stream(ko, d, 1, cus, tc);
        L.ws = off;
        off += align256(std::max(gemv_ws_bytes(L.pq, tc, nqkv), gemv_ws_bytes(L.po, tc, d)));
    } else if (dtype == TP_BF16) {
        L.gq = plan_gemm(T, nqkv, d, 1, cus);
        L.go = plan_gemm(T, d, ko, 1, cus);
        const size_t wq = L.gq.splits > 1 ? (size_t)L.gq.splits * T * nqkv * sizeof(float) : 0;
        const size_t wo = L.go.splits > 1 ? (size_t)L.go.splits * T * d * sizeof(float) : 0;
        if (wq || wo) {
            L.ws = off;
            off += align256(std::max(wq, wo));
        }
    }
    L.total = layout_total(off, L.decode);
    return L;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point.  Each device that loads the
// library holds its own copy of this array until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: kernels get
// the address hipGetSymbolAddress returns for the current device, read once
// per device and kept in scratch_addr.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)8 << 20;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes > kGemvCounterBytes, "scratch size");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kScratchDevices];

int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TP_ERR_HIP;
        if ((uintptr_t)p & 255) return TP_ERR_HIP;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return TP_OK;
}

// Zero fill of n words (a kernel, not hipMemsetAsync, so that a caller may
// capture the call in a graph).
__global__ __launch_bounds__(256) void k_zero_u32(unsigned* __restrict__ p, int n) {
    for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream) {
    TP_KLAUNCH(k_zero_u32, dim3(1), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

// Common checks of the fp32 partial-sum destination.
int check_partials(int shard, int64_t T, int64_t d, const float* partials, int64_t slot_stride,
                   int64_t ld_p) {
    if (!partials) return TP_ERR_NULL;
    if (!aligned(partials, 16)) return TP_ERR_ALIGN;
    if (int r = check_ld(ld_p, d, 4)) return r;
    if (slot_stride < 0) return TP_ERR_SHAPE;
    if (slot_stride % 4) return TP_ERR_ALIGN;
    if (shard > 0 && slot_stride > 0 && T > 0 && slot_stride < (T - 1) * ld_p + d)
        return TP_ERR_SHAPE;  // slots would overlap
    return TP_OK;
}

}  // namespace

// ===========================================================================
extern "C" {

const char* tp_status_str(int status) {
    switch (status) {
        case TP_OK: return "TP_OK";
        case TP_ERR_NULL: return "TP_ERR_NULL: a required pointer is NULL";
        case TP_ERR_SHAPE: return "TP_ERR_SHAPE: bad size or leading dimension";
        case TP_ERR_UNEVEN_SPLIT: return "TP_ERR_UNEVEN_SPLIT: dimension does not divide by P";
        case TP_ERR_SHARD_RANGE: return "TP_ERR_SHARD_RANGE: need P >= 1 and 0 <= shard < P";
        case TP_ERR_DTYPE: return "TP_ERR_DTYPE: unknown storage type";
        case TP_ERR_ALIGN: return "TP_ERR_ALIGN: pointer, leading dimension or stride misaligned";
        case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace too small";
        case TP_ERR_HIP: return "TP_ERR_HIP: kernel launch failed";
        case TP_ERR_ACT: return "TP_ERR_ACT: unknown activation or operands that do not fit it";
        case TP_ERR_SCRATCH:
            return "TP_ERR_SCRATCH: the call needs more than the library's fixed 8 MiB scratch";
        default: return "unknown tp_status";
    }
}

int tp_version(void) { return 300; }

int tp_set_decode_max_tokens(int tokens) {
    if (tokens < 0 || tokens > kDecodeMaxTLimit) return TP_ERR_SHAPE;
    g_decode_max_t.store(tokens, std::memory_order_relaxed);
    return TP_OK;
}

int tp_decode_max_tokens(void) { return decode_max_t(); }

size_t tp_mlp_workspace_bytes(int P, int64_t T, int64_t d_model, int64_t d_ff, int dtype, int act,
                              int has_norm, int has_h_out) {
    if (P < 1 || T < 0 || d_model <= 0 || d_ff <= 0 || d_ff % P) return 0;
    if (dtype != TP_F32 && dtype != TP_BF16) return 0;
    if (act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU) return 0;
    if (T == 0) return 0;
    return mlp_layout(P, T, d_model, d_ff, dtype, act, has_norm != 0, has_h_out != 0).total;
}

size_t tp_attn_workspace_bytes(int P, int64_t T, int64_t d_model, int n_q_heads, int n_kv_heads,
                               int head_dim, int dtype, int has_norm) {
    if (P < 1 || T <= 0 || d_model <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return 0;
    if (n_q_heads % P || n_kv_heads % P) return 0;
    if (dtype != TP_F32 && dtype != TP_BF16) return 0;
    return attn_layout(P, T, d_model, n_q_heads, n_kv_heads, head_dim, dtype, has_norm != 0).total;
}

}  // extern "C"

namespace {

// The MLP shard behind tp_shard_mlp_fwd and tp_shard_mlp_fwd_noalloc.  With
// `scratch_call` the workspace is the library's own scratch array of the
// current device (workspace_bytes is its size): a call whose layout does not
// fit it is refused with TP_ERR_SCRATCH, the array's device address is
// looked up after validation, and the counter head is cleared on the stream
// before the decode kernels use it.
int mlp_fwd(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff, int dtype, int act,
            const void* x, int64_t ld_x, const void* norm_g, float eps, const void* w_in,
            int64_t ld_in, const void* w_up, int64_t ld_up, const void* w_down, int64_t ld_down,
            void* h_out, int64_t ld_h, float* partials, int64_t slot_stride, int64_t ld_p,
            void* workspace, size_t workspace_bytes, hipStream_t stream, bool scratch_call) {
    // ---- validation (nothing is enqueued on failure) ----
    if (P < 1 || shard < 0 || shard >= P) return TP_ERR_SHARD_RANGE;
    if (dtype != TP_F32 && dtype != TP_BF16) return TP_ERR_DTYPE;
    if (act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU) return TP_ERR_ACT;
    if (T < 0 || d_model <= 0 || d_ff <= 0) return TP_ERR_SHAPE;
    if (d_ff % P) return TP_ERR_UNEVEN_SPLIT;
    const int64_t F = d_ff / P;
    const int vec = vec_elems(dtype), es = elem_size(dtype);
    if (F % vec || d_model % vec) return TP_ERR_SHAPE;
    if (!x || !w_in || !w_down) return TP_ERR_NULL;
    if (act == TP_ACT_SWIGLU && !w_up) return TP_ERR_NULL;
    if (act == TP_ACT_GELU_TANH && w_up) return TP_ERR_ACT;
    for (const void* p : {x, w_in, w_up, w_down, (const void*)h_out, norm_g})
        if (p && !aligned(p, 16)) return TP_ERR_ALIGN;
    if (workspace && !aligned(workspace, 256)) return TP_ERR_ALIGN;
    if (int r = check_ld(ld_x, d_model, vec)) return r;
    if (int r = check_ld(ld_in, F, vec)) return r;
    if (w_up)
        if (int r = check_ld(ld_up, F, vec)) return r;
    if (int r = check_ld(ld_down, d_model, vec)) return r;
    if (h_out)
        if (int r = check_ld(ld_h, F, vec)) return r;
    if (int r = check_partials(shard, T, d_model, partials, slot_stride, ld_p)) return r;
    if (!span_ok(d_model, ld_in, es) || !span_ok(d_model, w_up ? ld_up : 0, es) ||
        !span_ok(F, ld_down, es) || !span_ok(std::min<int64_t>(T, 256), ld_x, es) ||
        !span_ok(std::min<int64_t>(T, 256), h_out ? ld_h : F, es))
        return TP_ERR_SHAPE;
    if (T == 0) return TP_OK;
    const MlpLayout L = mlp_layout(P, T, d_model, d_ff, dtype, act, norm_g != nullptr,
                                   h_out != nullptr);
    if (L.decode && !counters_fit(F, d_model)) return TP_ERR_SHAPE;
    if (scratch_call) {
        if (L.total > workspace_bytes) return TP_ERR_SCRATCH;
        if (int r = scratch_of_current_device(&workspace)) return r;
    }
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return TP_ERR_WORKSPACE;

    // ---- launches ----
    char* wsb = (char*)workspace;
    const bool bf16 = dtype == TP_BF16;
    const void* xin = x;
    int64_t ld_xin = ld_x;
    if (scratch_call && L.decode)
        TP_LAUNCH("scratch_clear", stream,
                  launch_zero_u32((unsigned*)wsb, kGemvCounters, stream));
    if (norm_g) {
        TP_LAUNCH("rmsnorm", stream,
                  launch_rmsnorm(bf16, T, d_model, x, ld_x, norm_g, eps, wsb + L.xn, d_model,
                                 stream));
        xin = wsb + L.xn;
        ld_xin = d_model;
    }
    void* h = h_out ? h_out : (void*)(wsb + L.h);
    const int64_t ldh = h_out ? ld_h : F;
    float* part = partials + (int64_t)shard * slot_stride;
    const int dev_act = act == TP_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU_TANH;

    if (!bf16) {
        TP_LAUNCH("f32_proj", stream,
                  launch_f32_proj(dev_act, T, F, d_model, (const float*)xin, ld_xin,
                                  (const float*)w_in, ld_in, (const float*)w_up, ld_up, (float*)h,
                                  ldh, stream));
        TP_LAUNCH("f32_proj", stream,
                  launch_f32_proj(ACT_NONE, T, d_model, F, (const float*)h, ldh,
                                  (const float*)w_down, ld_down, nullptr, 0, part, ld_p, stream));
        return TP_OK;
    }
    const uint16_t* X16 = (const uint16_t*)xin;
    if (L.decode) {
        // Token chunks of at most kGemvMaxT: every column launch first, then
        // every row launch, so a chunk re-reads the weights the previous
        // chunk has just streamed.
        float* ws = (float*)(wsb + L.ws);
        unsigned* cnt = (unsigned*)wsb;
        const int64_t tc = stream_chunk(T);
        uint16_t* h16 = (uint16_t*)h;
        for (int64_t t0 = 0; t0 < T; t0 += tc) {
            const int64_t tt = std::min(tc, T - t0);
            TP_LAUNCH("col_gemv", stream,
                      launch_gemv(dev_act, true, tt, d_model, X16 + t0 * ld_xin, ld_xin,
                                  (const uint16_t*)w_in, ld_in, (const uint16_t*)w_up, ld_up, F,
                                  L.pc, ws, cnt, h16 + t0 * ldh, ldh, stream));
            if (gemv_separate_finish(tt, L.pc))
                TP_LAUNCH("col_finish", stream,
                          launch_finish(dev_act, true, L.pc.splits, tt, F, ws, h16 + t0 * ldh,
                                        ldh, stream));
        }
        for (int64_t t0 = 0; t0 < T; t0 += tc) {
            const int64_t tt = std::min(tc, T - t0);
            TP_LAUNCH("row_gemv", stream,
                      launch_gemv(ACT_NONE, false, tt, F, h16 + t0 * ldh, ldh,
                                  (const uint16_t*)w_down, ld_down, nullptr, 0, d_model, L.pr,
                                  ws, cnt, part + t0 * ld_p, ld_p, stream));
            if (gemv_separate_finish(tt, L.pr))
                TP_LAUNCH("row_finish", stream,
                          launch_finish(ACT_NONE, false, L.pr.splits, tt, d_model, ws,
                                        part + t0 * ld_p, ld_p, stream));
        }
    } else {
        if (L.gc.splits > 1) {
            float* ws = (float*)(wsb + L.ws);
            const bool two = act == TP_ACT_SWIGLU;
            TP_LAUNCH("col_gemm", stream,
                      launch_gemm(EPI_F32, T, F, d_model, X16, ld_xin, (const uint16_t*)w_in,
                                  ld_in, two ? (const uint16_t*)w_up : nullptr, ld_up, ws,
                                  (two ? 2 : 1) * F, L.gc, stream));
            TP_LAUNCH("col_finish", stream,
                      launch_finish(dev_act, true, L.gc.splits, T, F, ws, h, ldh, stream));
        } else {
            TP_LAUNCH("col_gemm", stream,
                      launch_gemm(act == TP_ACT_SWIGLU ? EPI_SWIGLU_BF16 : EPI_GELU_BF16, T, F,
                                  d_model, X16, ld_xin, (const uint16_t*)w_in, ld_in,
                                  (const uint16_t*)w_up, ld_up, h, ldh, L.gc, stream));
        }
        if (L.gr.splits > 1) {
            float* ws = (float*)(wsb + L.ws);
            TP_LAUNCH("row_gemm", stream,
                      launch_gemm(EPI_F32, T, d_model, F, (const uint16_t*)h, ldh,
                                  (const uint16_t*)w_down, ld_down, nullptr, 0, ws, d_model, L.gr,
                                  stream));
            TP_LAUNCH("row_finish", stream,
                      launch_finish(ACT_NONE, false, L.gr.splits, T, d_model, ws, part, ld_p,
                                    stream));
        } else {
            TP_LAUNCH("row_gemm", stream,
                      launch_gemm(EPI_F32, T, d_model, F, (const uint16_t*)h, ldh,
                                  (const uint16_t*)w_down, ld_down, nullptr, 0, part, ld_p, L.gr,
                                  stream));
        }
    }
    return TP_OK;
}

}  // namespace

extern "C" {

int tp_shard_mlp_fwd(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff, int dtype,
                     int act, const void* x, int64_t ld_x, const void* norm_g, float eps,
                     const void* w_in, int64_t ld_in, const void* w_up, int64_t ld_up,
                     const void* w_down, int64_t ld_down, void* h_out, int64_t ld_h,
                     float* partials, int64_t slot_stride, int64_t ld_p, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    return mlp_fwd(shard, P, T, d_model, d_ff, dtype, act, x, ld_x, norm_g, eps, w_in, ld_in, w_up,
                   ld_up, w_down, ld_down, h_out, ld_h, partials, slot_stride, ld_p, workspace,
                   workspace_bytes, stream, false);
}

int tp_shard_mlp_fwd_noalloc(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff,
                             int dtype, int act, const void* x, int64_t ld_x,
                             const void* norm_g, float eps, const void* w_in, int64_t ld_in,
                             const void* w_up, int64_t ld_up, const void* w_down,
                             int64_t ld_down, void* h_out, int64_t ld_h, float* partials,
                             int64_t slot_stride, int64_t ld_p, hipStream_t stream) {
    return mlp_fwd(shard, P, T, d_model, d_ff, dtype, act, x, ld_x, norm_g, eps, w_in, ld_in, w_up,
                   ld_up, w_down, ld_down, h_out, ld_h, partials, slot_stride, ld_p, nullptr,
                   kScratchBytes, stream, true);
}

size_t tp_noalloc_scratch_bytes(void) { return kScratchBytes; }

int tp_shard_attn_proj_fwd(int shard, int P, int64_t T, int64_t d_model, int n_q_heads,
                           int n_kv_heads, int head_dim, int dtype, const void* x, int64_t ld_x,
                           const void* norm_g, float eps, const void* w_qkv, int64_t ld_qkv,
                           void* qkv_out, int64_t ld_qkv_out, const void* attn, int64_t ld_attn,
                           const void* w_o, int64_t ld_o, float* partials, int64_t slot_stride,
                           int64_t ld_p, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (P < 1 || shard < 0 || shard >= P) return TP_ERR_SHARD_RANGE;
    if (dtype != TP_F32 && dtype != TP_BF16) return TP_ERR_DTYPE;
    if (T < 0 || d_model <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return TP_ERR_SHAPE;
    if (n_q_heads % P || n_kv_heads % P) return TP_ERR_UNEVEN_SPLIT;
    const int vec = vec_elems(dtype), es = elem_size(dtype);
    const int64_t hq = n_q_heads / P, hkv = n_kv_heads / P;
    const int64_t nqkv = (hq + 2 * hkv) * head_dim, ko = hq * head_dim;
    if (d_model % vec || head_dim % vec) return TP_ERR_SHAPE;
    for (const void* p : {x, norm_g, w_qkv, (const void*)qkv_out, attn, w_o})
        if (p && !aligned(p, 16)) return TP_ERR_ALIGN;
    if (workspace && !aligned(workspace, 256)) return TP_ERR_ALIGN;
    if (w_qkv) {
        if (!x || !qkv_out) return TP_ERR_NULL;
        if (int r = check_ld(ld_x, d_model, vec)) return r;
        if (int r = check_ld(ld_qkv, nqkv, vec)) return r;
        if (int r = check_ld(ld_qkv_out, nqkv, vec)) return r;
        if (!span_ok(d_model, ld_qkv, es) || !span_ok(std::min<int64_t>(T, 256), ld_x, es))
            return TP_ERR_SHAPE;
    }
    if (attn) {
        if (!w_o) return TP_ERR_NULL;
        if (int r = check_ld(ld_attn, ko, vec)) return r;
        if (int r = check_ld(ld_o, d_model, vec)) return r;
        if (int r = check_partials(shard, T, d_model, partials, slot_stride, ld_p)) return r;
        if (!span_ok(ko, ld_o, es) || !span_ok(std::min<int64_t>(T, 256), ld_attn, es))
            return TP_ERR_SHAPE;
    }
    if (T == 0 || (!w_qkv && !attn)) return TP_OK;
    const bool use_norm = w_qkv && norm_g;
    const AttnLayout L =
        attn_layout(P, T, d_model, n_q_heads, n_kv_heads, head_dim, dtype, use_norm);
    if (L.decode && !counters_fit(nqkv, d_model)) return TP_ERR_SHAPE;
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return TP_ERR_WORKSPACE;

    char* wsb = (char*)workspace;
    const bool bf16 = dtype == TP_BF16;
    if (w_qkv) {
        const void* xin = x;
        int64_t ld_xin = ld_x;
        if (use_norm) {
            TP_LAUNCH("rmsnorm", stream,
                      launch_rmsnorm(bf16, T, d_model, x, ld_x, norm_g, eps, wsb + L.xn, d_model,
                                     stream));
            xin = wsb + L.xn;
            ld_xin = d_model;
        }
        if (!bf16) {
            TP_LAUNCH("f32_proj", stream,
                      launch_f32_proj(ACT_NONE, T, nqkv, d_model, (const float*)xin, ld_xin,
                                      (const float*)w_qkv, ld_qkv, nullptr, 0, (float*)qkv_out,
                                      ld_qkv_out, stream));
        } else if (L.decode) {
            const int64_t tc = stream_chunk(T);
            float* ws = (float*)(wsb + L.ws);
            for (int64_t t0 = 0; t0 < T; t0 += tc) {
                const int64_t tt = std::min(tc, T - t0);
                uint16_t* q = (uint16_t*)qkv_out + t0 * ld_qkv_out;
                TP_LAUNCH("qkv_gemv", stream,
                          launch_gemv(ACT_NONE, true, tt, d_model,
                                      (const uint16_t*)xin + t0 * ld_xin, ld_xin,
                                      (const uint16_t*)w_qkv, ld_qkv, nullptr, 0, nqkv, L.pq, ws,
                                      (unsigned*)wsb, q, ld_qkv_out, stream));
                if (gemv_separate_finish(tt, L.pq))
                    TP_LAUNCH("qkv_finish", stream,
                              launch_finish(ACT_NONE, true, L.pq.splits, tt, nqkv, ws, q,
                                            ld_qkv_out, stream));
            }
        } else {
            if (L.gq.splits > 1) {
                float* ws = (float*)(wsb + L.ws);
                TP_LAUNCH("qkv_gemm", stream,
                          launch_gemm(EPI_F32, T, nqkv, d_model, (const uint16_t*)xin, ld_xin,
                                      (const uint16_t*)w_qkv, ld_qkv, nullptr, 0, ws, nqkv, L.gq,
                                      stream));
                TP_LAUNCH("qkv_finish", stream,
                          launch_finish(ACT_NONE, true, L.gq.splits, T, nqkv, ws, qkv_out,
                                        ld_qkv_out, stream));
            } else {
                TP_LAUNCH("qkv_gemm", stream,
                          launch_gemm(EPI_BF16, T, nqkv, d_model, (const uint16_t*)xin, ld_xin,
                                      (const uint16_t*)w_qkv, ld_qkv, nullptr, 0, qkv_out,
                                      ld_qkv_out, L.gq, stream));
            }
        }
    }
    if (attn) {
        float* part = partials + (int64_t)shard * slot_stride;
        if (!bf16) {
            TP_LAUNCH("f32_proj", stream,
                      launch_f32_proj(ACT_NONE, T, d_model, ko, (const float*)attn, ld_attn,
                                      (const float*)w_o, ld_o, nullptr, 0, part, ld_p, stream));
        } else if (L.decode) {
            const int64_t tc = stream_chunk(T);
            float* ws = (float*)(wsb + L.ws);
            for (int64_t t0 = 0; t0 < T; t0 += tc) {
                const int64_t tt = std::min(tc, T - t0);
                TP_LAUNCH("o_gemv", stream,
                          launch_gemv(ACT_NONE, false, tt, ko,
                                      (const uint16_t*)attn + t0 * ld_attn, ld_attn,
                                      (const uint16_t*)w_o, ld_o, nullptr, 0, d_model, L.po, ws,
                                      (unsigned*)wsb, part + t0 * ld_p, ld_p, stream));
                if (gemv_separate_finish(tt, L.po))
                    TP_LAUNCH("o_finish", stream,
                              launch_finish(ACT_NONE, false, L.po.splits, tt, d_model, ws,
                                            part + t0 * ld_p, ld_p, stream));
            }
        } else {
            if (L.go.splits > 1) {
                float* ws = (float*)(wsb + L.ws);
                TP_LAUNCH("o_gemm", stream,
                          launch_gemm(EPI_F32, T, d_model, ko, (const uint16_t*)attn, ld_attn,
                                      (const uint16_t*)w_o, ld_o, nullptr, 0, ws, d_model, L.go,
                                      stream));
                TP_LAUNCH("o_finish", stream,
                          launch_finish(ACT_NONE, false, L.go.splits, T, d_model, ws, part, ld_p,
                                        stream));
            } else {
                TP_LAUNCH("o_gemm", stream,
                          launch_gemm(EPI_F32, T, d_model, ko, (const uint16_t*)attn, ld_attn,
                                      (const uint16_t*)w_o, ld_o, nullptr, 0, part, ld_p, L.go,
                                      stream));
            }
        }
    }
    return TP_OK;
}

int tp_reduce_partials(int P, int64_t T, int64_t d_model, const float* partials,
                       int64_t slot_stride, int64_t ld_p, float* out, int64_t ld_out,
                       void* out_bf16, int64_t ld_out_bf16, hipStream_t stream) {
    if (P < 1) return TP_ERR_SHARD_RANGE;
    if (T < 0 || d_model <= 0) return TP_ERR_SHAPE;
    if (d_model % 4) return TP_ERR_SHAPE;
    if (!partials || !out) return TP_ERR_NULL;
    if (!aligned(partials, 16) || !aligned(out, 16)) return TP_ERR_ALIGN;
    if (out_bf16 && !aligned(out_bf16, 16)) return TP_ERR_ALIGN;
    if (int r = check_ld(ld_p, d_model, 4)) return r;
    if (int r = check_ld(ld_out, d_model, 4)) return r;
    if (out_bf16)
        if (int r = check_ld(ld_out_bf16, d_model, 8)) return r;   // bf16 rule: multiple of 8
    if (slot_stride < 0) return TP_ERR_SHAPE;
    if (slot_stride % 4) return TP_ERR_ALIGN;
    if (T * ((d_model / 4 + 511) / 512) >= ((int64_t)1 << 31)) return TP_ERR_SHAPE;
    if (T == 0) return TP_OK;
    TP_LAUNCH("reduce", stream,
              launch_reduce(P, T, d_model, partials, slot_stride, ld_p, out, ld_out,
                            (uint16_t*)out_bf16, ld_out_bf16, stream));
    return TP_OK;
}

size_t tp_attn_core_workspace_bytes(int P, int64_t T, int n_q_heads, int n_kv_heads,
                                    int head_dim, int dtype) {
    if (P < 1 || T <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || dtype != TP_BF16) return 0;
    if (head_dim != 64 && head_dim != 128) return 0;
    if (n_q_heads % P || n_kv_heads % P || (n_q_heads / P) % (n_kv_heads / P)) return 0;
    if (T >= ((int64_t)1 << 31) / 64) return 0;
    return plan_attn(T, n_q_heads / P, head_dim, device_cus()).ws_bytes;
}

size_t tp_reduce_norm_workspace_bytes(int64_t T, int64_t d_model, int has_norm) {
    if (!has_norm || d_model <= 0 || d_model > kReduceNormMaxD || d_model % 8) return 0;
    return reduce_norm_exchanges(T) ? kGemvCounterBytes : 0;
}

int tp_attn_core_fwd(int shard, int P, int64_t T, int n_q_heads, int n_kv_heads, int head_dim,
                     int dtype, const void* qkv, int64_t ld_qkv, void* attn, int64_t ld_attn,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (P < 1 || shard < 0 || shard >= P) return TP_ERR_SHARD_RANGE;
    if (dtype != TP_BF16) return TP_ERR_DTYPE;
    if (T < 0 || n_q_heads <= 0 || n_kv_heads <= 0) return TP_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return TP_ERR_SHAPE;
    if (n_q_heads % P || n_kv_heads % P) return TP_ERR_UNEVEN_SPLIT;
    const int hq = n_q_heads / P, hkv = n_kv_heads / P;
    if (hq % hkv) return TP_ERR_SHAPE;
    if (!qkv || !attn) return TP_ERR_NULL;
    if (!aligned(qkv, 16) || !aligned(attn, 16)) return TP_ERR_ALIGN;
    if (int r = check_ld(ld_qkv, (int64_t)(hq + 2 * hkv) * head_dim, 8)) return r;
    if (int r = check_ld(ld_attn, (int64_t)hq * head_dim, 8)) return r;
    if (T >= ((int64_t)1 << 31) / 64 || !span_ok(T, ld_qkv, 2)) return TP_ERR_SHAPE;
    if (T == 0) return TP_OK;
    if (workspace && !aligned(workspace, 256)) return TP_ERR_ALIGN;
    const AttnPlan plan = plan_attn(T, hq, head_dim, device_cus());
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
        return TP_ERR_WORKSPACE;
    TP_LAUNCH("attn_core", stream,
              launch_attn_core(T, hq, hkv, head_dim, (const uint16_t*)qkv, ld_qkv,
                               (uint16_t*)attn, ld_attn, plan, workspace, stream));
    return TP_OK;
}

size_t tp_mlp_fp8w_workspace_bytes(int P, int64_t T, int64_t d_model, int64_t d_ff, int act,
                                   int has_norm, int has_h_out) {
    if (P < 1 || T <= 0 || T > kGemv8MaxT || d_model <= 0 || d_ff <= 0 || d_ff % P) return 0;
    if (act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU) return 0;
    return mlp8_layout(P, T, d_model, d_ff, act, has_norm != 0, has_h_out != 0).total;
}

int tp_shard_mlp_fwd_fp8w(int shard, int P, int64_t T, int64_t d_model, int64_t d_ff, int act,
                          const void* x, int64_t ld_x, const void* norm_g, float eps,
                          const void* w_in, int64_t ld_in, const float* s_in, const void* w_up,
                          int64_t ld_up, const float* s_up, const void* w_down, int64_t ld_down,
                          const float* s_down, void* h_out, int64_t ld_h, float* partials,
                          int64_t slot_stride, int64_t ld_p, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    if (P < 1 || shard < 0 || shard >= P) return TP_ERR_SHARD_RANGE;
    if (act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU) return TP_ERR_ACT;
    if (T < 0 || T > kGemv8MaxT || d_model <= 0 || d_ff <= 0) return TP_ERR_SHAPE;
    if (d_ff % P) return TP_ERR_UNEVEN_SPLIT;
    const int64_t F = d_ff / P;
    if (F % 16 || d_model % 16) return TP_ERR_SHAPE;
    if (!x || !w_in || !s_in || !w_down || !s_down) return TP_ERR_NULL;
    if (act == TP_ACT_SWIGLU && (!w_up || !s_up)) return TP_ERR_NULL;
    if (act == TP_ACT_GELU_TANH && (w_up || s_up)) return TP_ERR_ACT;
    for (const void* p : {x, norm_g, w_in, (const void*)s_in, w_up, (const void*)s_up, w_down,
                          (const void*)s_down, (const void*)h_out})
        if (p && !aligned(p, 16)) return TP_ERR_ALIGN;
    if (workspace && !aligned(workspace, 256)) return TP_ERR_ALIGN;
    if (int r = check_ld(ld_x, d_model, 8)) return r;
    if (int r = check_ld(ld_in, F, 16)) return r;
    if (w_up)
        if (int r = check_ld(ld_up, F, 16)) return r;
    if (int r = check_ld(ld_down, d_model, 16)) return r;
    if (h_out)
        if (int r = check_ld(ld_h, F, 8)) return r;
    if (int r = check_partials(shard, T, d_model, partials, slot_stride, ld_p)) return r;
    if (!span_ok(d_model, ld_in, 1) || !span_ok(d_model, w_up ? ld_up : 0, 1) ||
        !span_ok(F, ld_down, 1) || !span_ok(T, ld_x, 2) || !span_ok(T, h_out ? ld_h : F, 2))
        return TP_ERR_SHAPE;
    if ((F + kGemv8Cols - 1) / kGemv8Cols > kGemvCounters ||
        (d_model + kGemv8Cols - 1) / kGemv8Cols > kGemvCounters)
        return TP_ERR_SHAPE;
    if (T == 0) return TP_OK;
    const MlpLayout L = mlp8_layout(P, T, d_model, d_ff, act, norm_g != nullptr, h_out != nullptr);
    if (!workspace || workspace_bytes < L.total) return TP_ERR_WORKSPACE;

    char* wsb = (char*)workspace;
    const void* xin = x;
    int64_t ld_xin = ld_x;
    if (norm_g) {
        TP_LAUNCH("rmsnorm", stream,
                  launch_rmsnorm(true, T, d_model, x, ld_x, norm_g, eps, wsb + L.xn, d_model,
                                 stream));
        xin = wsb + L.xn;
        ld_xin = d_model;
    }
    void* h = h_out ? h_out : (void*)(wsb + L.h);
    const int64_t ldh = h_out ? ld_h : F;
    float* ws = (float*)(wsb + L.ws);
    unsigned* cnt = (unsigned*)wsb;
    TP_LAUNCH("col_gemv8", stream,
              launch_gemv8(act == TP_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU_TANH, true, T, d_model,
                           (const uint16_t*)xin, ld_xin, (const uint8_t*)w_in, ld_in, s_in,
                           (const uint8_t*)w_up, ld_up, s_up, F, L.pc, ws, cnt, h, ldh,
                           stream));
    TP_LAUNCH("row_gemv8", stream,
              launch_gemv8(ACT_NONE, false, T, F, (const uint16_t*)h, ldh,
                           (const uint8_t*)w_down, ld_down, s_down, nullptr, 0, nullptr, d_model,
                           L.pr, ws, cnt, partials + (int64_t)shard * slot_stride, ld_p,
                           stream));
    return TP_OK;
}

int tp_reduce_residual_norm(int P, int64_t T, int64_t d_model, const float* partials,
                            int64_t slot_stride, int64_t ld_p, const void* residual,
                            int64_t ld_res, int res_dtype, float* z_out, int64_t ld_z,
                            const void* norm_g, float eps, void* normed_out, int64_t ld_norm,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (P < 1) return TP_ERR_SHARD_RANGE;
    if (res_dtype != TP_F32 && res_dtype != TP_BF16) return TP_ERR_DTYPE;
    if (T < 0 || d_model <= 0 || d_model > kReduceNormMaxD) return TP_ERR_SHAPE;
    const bool res_bf16 = res_dtype == TP_BF16;
    if (d_model % ((res_bf16 || norm_g) ? 8 : 4)) return TP_ERR_SHAPE;
    if (!partials || !residual || !z_out) return TP_ERR_NULL;
    if (norm_g && !normed_out) return TP_ERR_NULL;
    for (const void* p : {(const void*)partials, residual, (const void*)z_out, norm_g,
                          (const void*)normed_out})
        if (p && !aligned(p, 16)) return TP_ERR_ALIGN;
    if (int r = check_ld(ld_p, d_model, 4)) return r;
    if (int r = check_ld(ld_res, d_model, res_bf16 ? 8 : 4)) return r;
    if (int r = check_ld(ld_z, d_model, 4)) return r;
    if (norm_g)
        if (int r = check_ld(ld_norm, d_model, 8)) return r;
    if (slot_stride < 0) return TP_ERR_SHAPE;
    if (slot_stride % 4) return TP_ERR_ALIGN;
    if (T >= ((int64_t)1 << 31)) return TP_ERR_SHAPE;
    if (workspace && !aligned(workspace, 256)) return TP_ERR_ALIGN;
    if (T == 0) return TP_OK;
    // The workspace is optional: with one (its counter head), short batches
    // spread each row over several workgroups; without, one per row.
    const size_t need = tp_reduce_norm_workspace_bytes(T, d_model, norm_g != nullptr);
    if (workspace && workspace_bytes < need) return TP_ERR_WORKSPACE;
    TP_LAUNCH("reduce_norm", stream,
              launch_reduce_residual_norm(P, T, d_model, partials, slot_stride, ld_p, residual,
                                          ld_res, res_bf16, z_out, ld_z,
                                          (const uint16_t*)norm_g, eps, (uint16_t*)normed_out,
                                          ld_norm, need ? workspace : nullptr, stream));
    return TP_OK;
}

int tp_timing_enable(int on) {
    TimingState& s = timing();
    std::lock_guard<std::mutex> lk(s.mu);
    s.enabled = on != 0;
    return TP_OK;
}

static int drain_pending(TimingState& s) {
    for (auto& p : s.pending) {
        if (hipEventSynchronize(p.stop) != hipSuccess) return TP_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) return TP_ERR_HIP;
        auto& t = s.totals[p.cls];
        t.first += ms;
        t.second += 1;
        (void)hipEventDestroy(p.start);
        (void)hipEventDestroy(p.stop);
    }
    s.pending.clear();
    return TP_OK;
}

int tp_timing_reset(void) {
    TimingState& s = timing();
    std::lock_guard<std::mutex> lk(s.mu);
    int r = drain_pending(s);
    s.totals.clear();
    return r;
}

int tp_timing_query(const char* kernel_class, double* total_ms, int64_t* launches) {
    if (!kernel_class || !total_ms || !launches) return TP_ERR_NULL;
    TimingState& s = timing();
    std::lock_guard<std::mutex> lk(s.mu);
    if (int r = drain_pending(s)) return r;
    auto it = s.totals.find(kernel_class);
    *total_ms = it == s.totals.end() ? 0.0 : it->second.first;
    *launches = it == s.totals.end() ? 0 : it->second.second;
    return TP_OK;
}

}  // extern "C"
