// C ABI of libmlora: argument checks, workspace layout and kernel dispatch.
// Declarations and the contract of every entry point are in include/mlora.h.
#include "mlora.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "kernels.h"

using namespace mlora;

namespace {

constexpr int64_t DECODE_MAX_T = 512;         // tokens per decode launch (8 chunks of 64)
constexpr int64_t PREFILL_MAX_T = 4096 * 256; // token chunk of the tiled kernels

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Checks an mlora_slots and fills the kernels' geometry (slice table normalised).
mlora_status check_slots(const mlora_slots *s, int64_t n_out, bool need_data, SlotGeom *g)
{
    if (s == nullptr)
        return MLORA_ERR_ARG;
    if (s->S < 1 || s->S > MLORA_MAX_SLOTS)
        return MLORA_ERR_UNSUPPORTED;
    if (s->R < 8 || s->R > MLORA_MAX_RANK || !is_pow2(s->R))
        return MLORA_ERR_UNSUPPORTED;
    if (s->n_slices < 1 || s->n_slices > MLORA_MAX_SLICES)
        return MLORA_ERR_UNSUPPORTED;
    std::memset(g, 0, sizeof *g);
    g->S = s->S;
    g->R = s->R;
    g->n_slices = s->n_slices;
    bool all_zero = true;
    for (int i = 0; i <= s->n_slices; ++i)
        all_zero &= s->slice_start[i] == 0;
    if (s->n_slices == 1 && all_zero) {
        g->slice_start[0] = 0;
        g->slice_start[1] = (int32_t)n_out;
    } else {
        if (s->slice_start[0] != 0 || s->slice_start[s->n_slices] != n_out)
            return MLORA_ERR_SHAPE;
        for (int i = 0; i < s->n_slices; ++i)
            if (s->slice_start[i + 1] <= s->slice_start[i])
                return MLORA_ERR_SHAPE;
        for (int i = 0; i <= s->n_slices; ++i)
            g->slice_start[i] = s->slice_start[i];
    }
    for (int i = s->n_slices + 1; i < 5; ++i)
        g->slice_start[i] = g->slice_start[s->n_slices];
    if (need_data) {
        if (s->A == nullptr || s->B == nullptr || s->factor == nullptr)
            return MLORA_ERR_ARG;
        if (!aligned16(s->A) || !aligned16(s->B))
            return MLORA_ERR_ARG;
    }
    g->A = (const uint16_t *)s->A;
    g->B = (const uint16_t *)s->B;
    g->factor = s->factor;
    g->rank = s->rank;
    return MLORA_OK;
}

// Workspace layout of one call; every region 256-byte aligned.  No region carries state from
// one call to the next.
struct Layout {
    size_t sort_cnt = 0;   // counting-sort scratch (plan)
    size_t v = 0;          // fp32 per 64-token chunk [sk][K][64][n_slices*R] shrink partials
    size_t part = 0;       // fp32 partial sums of the decode GEMM
    size_t pre = 0;        // prefill path: tile lists and V blocks
    size_t total = 0;
    size_t off_sort = 0, off_v = 0, off_part = 0, off_pre = 0;
};

// Regions for both paths, so one workspace size serves any flags.
Layout make_layout(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                   int32_t n_slices)
{
    Layout L;
    const int32_t wd = n_slices * R;
    L.sort_cnt = align_up(sort_workspace_bytes(T * K, S));
    if (T > 0)
        L.pre = align_up(prefill_workspace_bytes(
            prefill_config(std::min<int64_t>(T, PREFILL_MAX_T), K, n_in, n_out, S, R, n_slices)));
    const int64_t Tc = std::min<int64_t>(T, DECODE_MAX_T);
    L.v = 0;
    L.part = 0;
    if (Tc > 0) {
        const int64_t sk = decode_config(Tc, n_in, n_out).sk;
        const int64_t chunks = (Tc + 63) / 64, per = chunks > 1 ? 64 : Tc;
        L.v = align_up((size_t)chunks * sk * K * per * wd * sizeof(float));
        L.part = align_up(decode_partial_bytes(Tc, n_in, n_out));
    }
    L.off_sort = 0;
    L.off_v = L.off_sort + L.sort_cnt;
    L.off_part = L.off_v + L.v;
    L.off_pre = L.off_part + L.part;
    L.total = L.off_pre + L.pre;
    return L;
}

thread_local char g_last_error[256] = "";

mlora_status hip_status(hipError_t e, const char *where = "launch")
{
    if (e == hipSuccess)
        return MLORA_OK;
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e),
                  (int)e);
    return MLORA_ERR_HIP;
}

// Profiling hook: event pairs around the main product kernel of each mlora_linear call.
struct Trace {
    std::mutex mu;
    std::vector<hipEvent_t> begin, end;
    int32_t count = 0;
    bool active = false;
} g_trace;

void trace_release()
{
    for (hipEvent_t e : g_trace.begin)
        (void)hipEventDestroy(e);
    for (hipEvent_t e : g_trace.end)
        (void)hipEventDestroy(e);
    g_trace.begin.clear();
    g_trace.end.clear();
    g_trace.count = 0;
    g_trace.active = false;
}

}  // namespace

namespace mlora {

void trace_mark(hipStream_t stream, bool begin)
{
    if (!g_trace.active)
        return;
    std::lock_guard<std::mutex> lock(g_trace.mu);
    if (!g_trace.active || g_trace.count >= (int32_t)g_trace.begin.size())
        return;
    if (begin) {
        (void)hipEventRecord(g_trace.begin[g_trace.count], stream);
    } else {
        (void)hipEventRecord(g_trace.end[g_trace.count], stream);
        ++g_trace.count;
    }
}

}  // namespace mlora

extern "C" {

mlora_status mlora_trace_start(int32_t capacity)
{
    if (capacity < 1 || capacity > (1 << 20))
        return MLORA_ERR_ARG;
    std::lock_guard<std::mutex> lock(g_trace.mu);
    trace_release();
    g_trace.begin.resize(capacity);
    g_trace.end.resize(capacity);
    for (int32_t i = 0; i < capacity; ++i) {
        // no system-scope fence at the record: the pair then costs far less than a fenced one
        hipError_t e = hipEventCreateWithFlags(&g_trace.begin[i], hipEventDisableSystemFence);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&g_trace.end[i], hipEventDisableSystemFence);
        if (e != hipSuccess) {
            g_trace.begin.resize(i + 1);
            g_trace.end.resize(i + 1);
            trace_release();
            return hip_status(e, "trace event");
        }
    }
    g_trace.active = true;
    return MLORA_OK;
}

int32_t mlora_trace_stop(float *ms, int32_t capacity)
{
    std::lock_guard<std::mutex> lock(g_trace.mu);
    const int32_t n = std::min(g_trace.count, std::max<int32_t>(capacity, 0));
    int32_t out = n;
    for (int32_t i = 0; i < n && ms != nullptr; ++i) {
        hipError_t e = hipEventSynchronize(g_trace.end[i]);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms[i], g_trace.begin[i], g_trace.end[i]);
        if (e != hipSuccess) {
            (void)hip_status(e, "trace read");
            out = -1;
            break;
        }
    }
    trace_release();
    return out;
}


const char *mlora_last_error(void) { return g_last_error; }

const char *mlora_status_string(mlora_status status)
{
    switch (status) {
    case MLORA_OK: return "ok";
    case MLORA_ERR_ARG: return "invalid argument (null, negative or misaligned)";
    case MLORA_ERR_SHAPE: return "inconsistent shapes";
    case MLORA_ERR_RANK: return "adapter rank outside [1, R]";
    case MLORA_ERR_INDEX: return "slot index outside [-1, S)";
    case MLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLORA_ERR_HIP: return "HIP error";
    case MLORA_ERR_UNSUPPORTED: return "outside the supported limits";
    }
    return "unknown status";
}

float mlora_factor(float alpha, int32_t r, int32_t use_rslora)
{
    if (r < 1)
        return NAN;
    const double a = (double)alpha;
    return (float)(use_rslora ? a / std::sqrt((double)r) : a / (double)r);
}

int64_t mlora_slot_bytes(int32_t S, int32_t R, int64_t n_in, int64_t n_out, int32_t n_slices)
{
    if (S < 0 || R < 0 || n_in < 0 || n_out < 0 || n_slices < 0)
        return -1;
    return (int64_t)S * ((int64_t)n_slices * R * n_in + n_out * (int64_t)R) * 2;
}

size_t mlora_workspace_size(int64_t T, int32_t K, int64_t n_in, int64_t n_out,
                            const mlora_slots *slots)
{
    if (T < 0 || K < 1 || K > MLORA_MAX_K || n_in <= 0 || n_out <= 0 || slots == nullptr)
        return 0;
    SlotGeom g;
    if (check_slots(slots, n_out, false, &g) != MLORA_OK)
        return 0;
    return make_layout(T, K, n_in, n_out, g.S, g.R, g.n_slices).total + 256;
}

int64_t mlora_packed_weight_bytes(int64_t n_out, int64_t n_in)
{
    if (n_out < 1 || n_in < 1)
        return 0;
    return packed_weight_elems(n_out, n_in) * 2;
}

mlora_status mlora_pack_weight(const void *W, int64_t n_out, int64_t n_in, void *Wp,
                               hipStream_t stream)
{
    if (W == nullptr || Wp == nullptr || n_out < 1 || n_in < 1 || !aligned16(W) ||
        !aligned16(Wp))
        return MLORA_ERR_ARG;
    if (n_in % 8 != 0)
        return MLORA_ERR_SHAPE;
    return hip_status(launch_pack_weight((const uint16_t *)W, n_out, n_in, (uint16_t *)Wp, stream),
                      "pack weight");
}

mlora_status mlora_slot_load(void *A, void *B, float *factor, int32_t S, int32_t R,
                             int32_t n_slices, int64_t n_in, int64_t n_out, int32_t slot,
                             const void *A_src, const void *B_src, int32_t r, float f,
                             hipStream_t stream)
{
    if (A == nullptr || B == nullptr || factor == nullptr || A_src == nullptr ||
        B_src == nullptr || n_in < 1 || n_out < 1 || S < 1 || slot < 0 || slot >= S)
        return MLORA_ERR_ARG;
    if (S > MLORA_MAX_SLOTS || R < 8 || R > MLORA_MAX_RANK || !is_pow2(R) || n_slices < 1 ||
        n_slices > MLORA_MAX_SLICES)
        return MLORA_ERR_UNSUPPORTED;
    if (r < 1 || r > R)
        return MLORA_ERR_RANK;
    uint16_t *a_slot = (uint16_t *)A + (int64_t)slot * n_slices * R * n_in;
    uint16_t *b_slot = (uint16_t *)B + (int64_t)slot * n_out * R;
    const uint16_t *a_src = (const uint16_t *)A_src;
    for (int32_t s = 0; s < n_slices; ++s)
        if (hipError_t e = hipMemcpyAsync(a_slot + (int64_t)s * R * n_in,
                                          a_src + (int64_t)s * r * n_in, (size_t)r * n_in * 2,
                                          hipMemcpyDefault, stream);
            e != hipSuccess)
            return hip_status(e, "copy of A rows");
    if (hipError_t e = hipMemcpy2DAsync(b_slot, (size_t)R * 2, B_src, (size_t)r * 2, (size_t)r * 2,
                                        (size_t)n_out, hipMemcpyDefault, stream);
        e != hipSuccess)
        return hip_status(e, "copy of B columns");
    return hip_status(launch_slot_pad(a_slot, b_slot, factor + slot, R, r, n_slices, n_in, n_out,
                                      f, stream),
                      "slot padding");
}

mlora_status mlora_validate(const int32_t *idx, int64_t T, int32_t K, const mlora_slots *slots,
                            const int32_t *rank, int64_t *bad_value, hipStream_t stream)
{
    if (T < 0 || K < 1 || K > MLORA_MAX_K || slots == nullptr || (T > 0 && idx == nullptr))
        return MLORA_ERR_ARG;
    if (rank != nullptr)
        for (int32_t a = 0; a < slots->S; ++a)
            if (rank[a] < 1 || rank[a] > slots->R) {
                if (bad_value)
                    *bad_value = rank[a];
                return MLORA_ERR_RANK;
            }
    if (T == 0)
        return MLORA_OK;
    std::vector<int32_t> h((size_t)(T * K));
    if (hipMemcpyAsync(h.data(), idx, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream) != hipSuccess)
        return hip_status(hipGetLastError(), "copy of idx");
    if (hipError_t e = hipStreamSynchronize(stream); e != hipSuccess)
        return hip_status(e, "stream synchronize");
    for (int32_t v : h)
        if (v < -1 || v >= slots->S) {
            if (bad_value)
                *bad_value = v;
            return MLORA_ERR_INDEX;
        }
    return MLORA_OK;
}

mlora_status mlora_plan(const int32_t *idx, int64_t T, int32_t K, int32_t S, int32_t *perm,
                        int32_t *seg_slot, int32_t *seg_start, int32_t *seg_len,
                        int32_t *counts, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (T < 0 || K < 1 || K > MLORA_MAX_K || S < 1 || S > MLORA_MAX_SLOTS)
        return T < 0 || K < 1 ? MLORA_ERR_ARG : MLORA_ERR_UNSUPPORTED;
    if (counts == nullptr || seg_slot == nullptr || seg_start == nullptr || seg_len == nullptr)
        return MLORA_ERR_ARG;
    if (T > 0 && (idx == nullptr || perm == nullptr))
        return MLORA_ERR_ARG;
    if ((int64_t)T * K > INT32_MAX)
        return MLORA_ERR_UNSUPPORTED;
    const size_t need = sort_workspace_bytes(T * K, S);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return MLORA_ERR_WORKSPACE;
    trace_mark(stream, true);
    const hipError_t e = launch_stable_sort(idx, T * K, S, perm, seg_slot, seg_start, seg_len,
                                            counts, (int32_t *)ws, stream);
    trace_mark(stream, false);
    return hip_status(e);
}

mlora_status mlora_shrink(const void *x, int64_t T, int64_t n_in, const mlora_slots *slots,
                          const int32_t *idx, int32_t K, const float *scale, float *v, void *ws,
                          size_t ws_bytes, hipStream_t stream)
{
    (void)ws;
    (void)ws_bytes;
    if (T < 0 || n_in <= 0 || K < 1 || K > MLORA_MAX_K)
        return MLORA_ERR_ARG;
    if (n_in % 8 != 0)
        return MLORA_ERR_SHAPE;
    if (slots == nullptr)
        return MLORA_ERR_ARG;
    SlotGeom g;
    // the slice table is irrelevant to shrink: take a view with one output row per slice
    mlora_slots s1 = *slots;
    std::memset(s1.slice_start, 0, sizeof s1.slice_start);
    for (int i = 1; i <= s1.n_slices && i <= MLORA_MAX_SLICES; ++i)
        s1.slice_start[i] = i;
    mlora_status st = check_slots(&s1, s1.n_slices, true, &g);
    if (st != MLORA_OK)
        return st;
    if (T == 0)
        return MLORA_OK;
    if (x == nullptr || idx == nullptr || v == nullptr || !aligned16(x) || !aligned16(v))
        return MLORA_ERR_ARG;
    trace_mark(stream, true);
    const hipError_t e = launch_shrink_pairs((const uint16_t *)x, T, n_in, g, idx, K, scale, v,
                                             stream);
    trace_mark(stream, false);
    return hip_status(e);
}

mlora_status mlora_expand(const float *v, int64_t T, int64_t n_out, const mlora_slots *slots,
                          const int32_t *idx, int32_t K, void *y, hipStream_t stream)
{
    if (T < 0 || n_out <= 0 || K < 1 || K > MLORA_MAX_K)
        return MLORA_ERR_ARG;
    SlotGeom g;
    mlora_status st = check_slots(slots, n_out, true, &g);
    if (st != MLORA_OK)
        return st;
    if (T == 0)
        return MLORA_OK;
    if (v == nullptr || idx == nullptr || y == nullptr || !aligned16(v) || !aligned16(y))
        return MLORA_ERR_ARG;
    trace_mark(stream, true);
    const hipError_t e = launch_expand_tokens(v, T, n_out, g, idx, K, (uint16_t *)y, stream);
    trace_mark(stream, false);
    return hip_status(e);
}

}  // extern "C"

namespace {

// A second stream per device for the grouped decode's LoRA kernels (tile plan and group shrink),
// which do not depend on the base product: forked from the caller's stream and joined back
// before the expand with events, so the group shrink runs beside the decode GEMM.  Both are
// created once per device, at the device's first grouped call, with the default priority.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;                 // guards g_side and each fork / join sequence
std::map<int, SideStream> g_side;

// *out: the device's side stream, or nullptr when it does not exist yet and may not be created
// now (the caller's stream is being captured into a graph: creating a stream then could
// invalidate the capture; that call runs on the caller's stream alone).
hipError_t side_stream(hipStream_t caller, SideStream **out)
{
    *out = nullptr;
    int dev = -1;
    hipError_t e = caller != nullptr ? hipStreamGetDevice(caller, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    SideStream &ss = g_side[dev];
    if (ss.s == nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(caller, &cs)) != hipSuccess)
            return e;
        if (cs != hipStreamCaptureStatusNone)
            return hipSuccess;
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        SideStream n;
        e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        if (e != hipSuccess)
            return e;
        ss = n;
    }
    *out = &ss;
    return hipSuccess;
}

// The kernels mlora_linear runs for these sizes and flags (a host-side choice from the shapes):
// MLORA_PATH_TILED when forced or when the batch fills the GPU with 256 x 256 output tiles;
// else MLORA_PATH_GROUPED when forced or when the per-pair adapter reads of the decode kernels
// would exceed four times W's bytes (and the grouped expand keeps a launch's fp32 sums);
// else MLORA_PATH_DECODE.  MLORA_ERR_UNSUPPORTED: grouped forced where it does not fit.
mlora_status choose_path(int64_t T, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                         int32_t n_slices, int32_t K, uint32_t flags, bool lora, uint32_t *path)
{
    const bool force_decode = (flags & MLORA_PATH_DECODE) != 0;
    const bool force_tiled = (flags & MLORA_PATH_TILED) != 0;
    const bool force_grouped = (flags & MLORA_PATH_GROUPED) != 0;
    if (force_tiled || (!force_decode && !force_grouped &&
                        prefill_worth_it(T, n_in, n_out, K, lora ? n_slices * R : 0))) {
        *path = MLORA_PATH_TILED;
        return MLORA_OK;
    }
    *path = MLORA_PATH_DECODE;
    if (!lora || force_decode)
        return MLORA_OK;
    const int64_t Tc = std::min<int64_t>(std::max<int64_t>(T, 1), DECODE_MAX_T);
    const bool fits = grouped_decode_fits(grouped_config(Tc, K, n_in, n_out, S, R, n_slices));
    if (force_grouped && !fits) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "MLORA_PATH_GROUPED: the fp32 sums of %lld tokens x %lld outputs exceed "
                      "what the grouped expand keeps",
                      (long long)Tc, (long long)n_out);
        return MLORA_ERR_UNSUPPORTED;
    }
    if (fits && (force_grouped ||
                 grouped_decode_worth_it(Tc, K, n_in, n_out, n_slices * R, R)))
        *path = MLORA_PATH_GROUPED;
    return MLORA_OK;
}

// mlora_linear and mlora_linear_noalloc: checks, scratch regions and kernel dispatch.  With
// noalloc the scratch is the library's fixed per-device array (ws and ws_bytes unused) and holds
// only the regions of the path the call takes, from offset 0; otherwise it is the caller's
// workspace laid out as mlora_workspace_size() counts it (either path).
mlora_status linear_common(const void *x, const void *W, int64_t T, int64_t n_in, int64_t n_out,
                           const mlora_slots *slots, const int32_t *idx, int32_t K,
                           const float *scale, void *y, uint32_t flags, void *ws, size_t ws_bytes,
                           bool noalloc, hipStream_t stream)
{
    if (T < 0 || n_in <= 0 || n_out <= 0 || K < 1 || K > MLORA_MAX_K)
        return MLORA_ERR_ARG;
    {
        const uint32_t path = flags & (MLORA_PATH_DECODE | MLORA_PATH_TILED | MLORA_PATH_GROUPED);
        if (path & (path - 1))
            return MLORA_ERR_ARG;   // more than one path forced
    }
    if (n_in % 8 != 0)
        return MLORA_ERR_SHAPE;
    if (n_in > INT32_MAX / 2 || n_out > INT32_MAX / 2)
        return MLORA_ERR_UNSUPPORTED;
    const bool lora = (flags & MLORA_NO_ADAPTERS) == 0;
    SlotGeom g;
    std::memset(&g, 0, sizeof g);
    int32_t S = 1, R = 8, n_slices = 1;
    if (lora || slots != nullptr) {
        mlora_status st = check_slots(slots, n_out, lora, &g);
        if (st != MLORA_OK)
            return st;
        S = g.S;
        R = g.R;
        n_slices = g.n_slices;
    }
    if (T == 0)
        return MLORA_OK;
    if (x == nullptr || W == nullptr || y == nullptr || !aligned16(x) || !aligned16(W) ||
        !aligned16(y))
        return MLORA_ERR_ARG;
    if (lora && idx == nullptr)
        return MLORA_ERR_ARG;
    const bool packed = (flags & MLORA_W_PACKED) != 0;
    uint32_t path = 0;
    if (mlora_status st = choose_path(T, n_in, n_out, S, R, n_slices, K, flags, lora, &path);
        st != MLORA_OK)
        return st;
    const bool tiled = path == MLORA_PATH_TILED;
    // grouped decode: the decode kernels' base product, the LoRA terms per adapter group
    const bool grouped = path == MLORA_PATH_GROUPED;
    size_t off_v, off_part, off_pre, need;
    if (!noalloc) {
        const Layout L = make_layout(T, K, n_in, n_out, S, R, n_slices);
        off_v = L.off_v;
        off_part = L.off_part;
        off_pre = L.off_pre;
        need = L.total;
    } else if (tiled) {
        off_v = off_part = off_pre = 0;
        need = prefill_workspace_bytes(
            prefill_config(std::min<int64_t>(T, PREFILL_MAX_T), K, n_in, n_out, S, R, n_slices));
    } else if (grouped) {
        const int64_t Tc = std::min<int64_t>(T, DECODE_MAX_T);
        off_v = off_part = 0;
        off_pre = align_up(decode_partial_bytes(Tc, n_in, n_out));
        need = off_pre + prefill_workspace_bytes(grouped_config(Tc, K, n_in, n_out, S, R, n_slices));
    } else {
        const int64_t Tc = std::min<int64_t>(T, DECODE_MAX_T);
        const int64_t sk = decode_config(Tc, n_in, n_out).sk;
        const int64_t chunks = (Tc + 63) / 64, per = chunks > 1 ? 64 : Tc;
        off_v = off_pre = 0;
        off_part = align_up((size_t)chunks * sk * K * per * n_slices * R * sizeof(float));
        need = off_part + decode_partial_bytes(Tc, n_in, n_out);
    }
    uint8_t *wsb;
    if (noalloc) {
        if (need > MLORA_NOALLOC_SCRATCH_BYTES) {
            std::snprintf(g_last_error, sizeof g_last_error,
                          "mlora_linear_noalloc: this call needs %zu bytes of scratch, above the "
                          "fixed %zu",
                          need, (size_t)MLORA_NOALLOC_SCRATCH_BYTES);
            return MLORA_ERR_WORKSPACE;
        }
        void *p = nullptr;
        if (hipError_t e = noalloc_scratch(stream, &p); e != hipSuccess)
            return hip_status(e, "scratch address");
        wsb = (uint8_t *)p;
    } else {
        if (ws == nullptr || ws_bytes < need)
            return MLORA_ERR_WORKSPACE;
        wsb = (uint8_t *)ws;
        if (!aligned16(wsb))
            return MLORA_ERR_ARG;
    }
    float *upart = (float *)(wsb + off_v);
    float *part = (float *)(wsb + off_part);
    const uint16_t *xb = (const uint16_t *)x;
    uint16_t *yb = (uint16_t *)y;
    if (tiled) {
        // chunks of at most PREFILL_MAX_T tokens (the shrink's tile table lives in LDS)
        for (int64_t t0 = 0; t0 < T; t0 += PREFILL_MAX_T) {
            const int64_t Tc = std::min<int64_t>(PREFILL_MAX_T, T - t0);
            const PrefillCfg pc = prefill_config(Tc, K, n_in, n_out, S, R, n_slices);
            mlora_status st = hip_status(
                launch_prefill(xb + t0 * n_in, (const uint16_t *)W, packed, Tc, n_in, n_out,
                               lora ? &g : nullptr, lora ? idx + t0 * K : nullptr, K,
                               (lora && scale) ? scale + t0 * K : nullptr, yb + t0 * n_out, pc,
                               wsb + off_pre, stream),
                "prefill launch");
            if (st != MLORA_OK)
                return st;
        }
        return MLORA_OK;
    }
    // Launches of at most DECODE_MAX_T tokens (chunks of 64 inside): base GEMM + shrink pieces,
    // then the finish kernel.  Grouped: the group shrink first, the GEMM and the finish on the
    // base alone (the finish also keeps the fp32 sums), then the grouped expand.
    for (int64_t t0 = 0; t0 < T; t0 += DECODE_MAX_T) {
        const int64_t Tc = std::min<int64_t>(DECODE_MAX_T, T - t0);
        const DecodeCfg cfg = decode_config(Tc, n_in, n_out);
        const int32_t *idx_c = lora ? idx + t0 * K : nullptr;
        const float *scale_c = (lora && scale) ? scale + t0 * K : nullptr;
        if (grouped) {
            const PrefillCfg pc = grouped_config(Tc, K, n_in, n_out, S, R, n_slices);
            void *wpre = wsb + off_pre;
            // the tile plan and the group shrink on the side stream, forked before the GEMM is
            // enqueued and joined before the expand; the GEMM's launch goes in first so that
            // its workgroups are dispatched from the start.  When the GEMM takes the persistent
            // grid (every CU until it ends, nothing to run beside it) all of it goes on the
            // caller's stream in order, as in the no-allocation variant, which creates nothing
            std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
            SideStream *ss = nullptr;
            hipError_t e = hipSuccess;
            if (!noalloc && !decode_gemm_persistent(Tc, n_in, n_out)) {
                lk.lock();
                e = side_stream(stream, &ss);
                if (e == hipSuccess && ss != nullptr)
                    e = hipEventRecord(ss->fork, stream);
                if (e != hipSuccess)
                    return hip_status(e, "side stream fork");
            }
            if (ss == nullptr) {
                e = launch_grouped_shrink(xb + t0 * n_in, Tc, n_in, n_out, g, idx_c, K, scale_c,
                                          pc, wpre, stream);
                if (e != hipSuccess)
                    return hip_status(e, "grouped shrink launch");
            }
            trace_mark(stream, true);
            e = launch_decode_gemm(xb + t0 * n_in, (const uint16_t *)W, packed, Tc, n_in, n_out,
                                   part, cfg, nullptr, nullptr, K, nullptr, stream);
            trace_mark(stream, false);
            if (e != hipSuccess)
                return hip_status(e, "decode gemm launch");
            if (ss != nullptr) {
                e = hipStreamWaitEvent(ss->s, ss->fork, 0);
                if (e == hipSuccess)
                    e = launch_grouped_shrink(xb + t0 * n_in, Tc, n_in, n_out, g, idx_c, K,
                                              scale_c, pc, wpre, ss->s);
                if (e == hipSuccess)
                    e = hipEventRecord(ss->join, ss->s);
                if (e != hipSuccess)
                    return hip_status(e, "grouped shrink launch");
            }
            e = launch_decode_finish(part, cfg.sk, cfg.n_tiles, nullptr, 0, nullptr, Tc, n_out,
                                     nullptr, nullptr, 1, yb + t0 * n_out,
                                     grouped_base_sums(pc, wpre), stream);
            if (e != hipSuccess)
                return hip_status(e, "decode finish launch");
            if (ss != nullptr) {
                if ((e = hipStreamWaitEvent(stream, ss->join, 0)) != hipSuccess)
                    return hip_status(e, "side stream join");
                lk.unlock();
            }
            e = launch_grouped_expand(Tc, n_out, g, idx_c, K, yb + t0 * n_out, pc, wpre, stream);
            if (e != hipSuccess)
                return hip_status(e, "grouped expand launch");
            continue;
        }
        // the shrink inside the GEMM (pieces per split), or apart before a GEMM of the base
        // alone when the GEMM's workgroups would each chain several pieces
        const bool apart = lora && decode_shrink_apart(Tc, K, n_out, g.n_slices * g.R);
        hipError_t e = hipSuccess;
        if (apart) {
            e = launch_shrink_pairs(xb + t0 * n_in, Tc, n_in, g, idx_c, K, nullptr, upart, stream,
                                    true);
            if (e != hipSuccess)
                return hip_status(e, "shrink launch");
        }
        const bool fused = lora && !apart;
        trace_mark(stream, true);
        e = launch_decode_gemm(xb + t0 * n_in, (const uint16_t *)W, packed, Tc, n_in, n_out, part,
                               cfg, fused ? &g : nullptr, fused ? idx_c : nullptr, K,
                               fused ? upart : nullptr, stream);
        trace_mark(stream, false);
        if (e != hipSuccess)
            return hip_status(e, "decode gemm launch");
        e = launch_decode_finish(part, cfg.sk, cfg.n_tiles, lora ? upart : nullptr,
                                 apart ? 1 : cfg.sk, scale_c, Tc, n_out, lora ? &g : nullptr,
                                 idx_c, K, yb + t0 * n_out, nullptr, stream);
        if (e != hipSuccess)
            return hip_status(e, "decode finish launch");
    }
    return MLORA_OK;
}

}  // namespace

extern "C" {

mlora_status mlora_linear(const void *x, const void *W, int64_t T, int64_t n_in, int64_t n_out,
                          const mlora_slots *slots, const int32_t *idx, int32_t K,
                          const float *scale, void *y, uint32_t flags, void *ws, size_t ws_bytes,
                          hipStream_t stream)
{
    return linear_common(x, W, T, n_in, n_out, slots, idx, K, scale, y, flags, ws, ws_bytes,
                         false, stream);
}

uint32_t mlora_linear_path(int64_t T, int64_t n_in, int64_t n_out, const mlora_slots *slots,
                           int32_t K, uint32_t flags)
{
    if (T < 0 || n_in <= 0 || n_out <= 0 || K < 1 || K > MLORA_MAX_K)
        return 0;
    {
        const uint32_t p = flags & (MLORA_PATH_DECODE | MLORA_PATH_TILED | MLORA_PATH_GROUPED);
        if (p & (p - 1))
            return 0;
    }
    const bool lora = (flags & MLORA_NO_ADAPTERS) == 0;
    SlotGeom g;
    int32_t S = 1, R = 8, n_slices = 1;
    if (lora || slots != nullptr) {
        if (check_slots(slots, n_out, false, &g) != MLORA_OK)
            return 0;
        S = g.S;
        R = g.R;
        n_slices = g.n_slices;
    }
    uint32_t path = 0;
    return choose_path(T, n_in, n_out, S, R, n_slices, K, flags, lora, &path) == MLORA_OK ? path
                                                                                         : 0;
}

mlora_status mlora_linear_noalloc(const void *x, const void *W, int64_t T, int64_t n_in,
                                  int64_t n_out, const mlora_slots *slots, const int32_t *idx,
                                  int32_t K, const float *scale, void *y, uint32_t flags,
                                  hipStream_t stream)
{
    return linear_common(x, W, T, n_in, n_out, slots, idx, K, scale, y, flags, nullptr, 0, true,
                         stream);
}

}  // extern "C"
