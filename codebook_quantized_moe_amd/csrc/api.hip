// libmoeq C ABI: argument checks and dispatch. Every check runs before any launch, so a
// failing call leaves the stream untouched. Declarations and the contract of each call are in
// include/moeq.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "moeq.h"
#include "moeq_kernels.h"

using namespace moeq;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return MOEQ_OK;
}

// Reset this thread's sticky HIP error state, so that check_launch reports only our launch.
void clear_hip_error() { (void)hipGetLastError(); }

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOEQ_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Compute units of the current device (cached per device; MI355X has 256). Read from the
// device properties rather than an attribute enum, whose numbering is not stable across HIP
// runtime releases; any failure falls back to 256 and leaves no error state behind.
int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        clear_hip_error();
        return 256;
    }
    if (cache[dev] == 0) {
        hipDeviceProp_t prop;
        int n = 256;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0 &&
            prop.multiProcessorCount <= 4096)
            n = prop.multiProcessorCount;
        clear_hip_error();
        cache[dev] = n;
    }
    return cache[dev];
}

int check_sizes(const char* what, int T, int k, int E) {
    if (T < 0) return fail(MOEQ_EINVAL, "%s: T = %d must be >= 0", what, T);
    if (E < 1 || E > MOEQ_MAX_EXPERTS)
        return fail(MOEQ_EINVAL, "%s: E = %d must be in [1, %d]", what, E, MOEQ_MAX_EXPERTS);
    if (k < 1 || k > E) return fail(MOEQ_EINVAL, "%s: k = %d must be in [1, E = %d]", what, k, E);
    if ((long long)T * k >= (1LL << 31)) return fail(MOEQ_EINVAL, "%s: T*k too large", what);
    return MOEQ_OK;
}

int check_tables(const char* what, const float* tables, int n_tables, TableArgs* ta) {
    if (!tables) return fail(MOEQ_EINVAL, "%s: tables is NULL", what);
    if (n_tables < 1 || n_tables > MOEQ_MAX_TABLES)
        return fail(MOEQ_EINVAL, "%s: n_tables = %d must be in [1, %d]", what, n_tables, MOEQ_MAX_TABLES);
    memset(ta, 0, sizeof(*ta));
    ta->n = n_tables;
    for (int t = 0; t < n_tables; ++t)
        for (int m = 0; m < 8; ++m) {
            const float v = tables[t * 8 + m];
            if (!isfinite(v) || signbit(v))
                return fail(MOEQ_EINVAL,
                            "%s: tables[%d][%d] = %g: entries must be finite magnitudes with a clear sign bit",
                            what, t, m, (double)v);
            ta->v[t][m] = v;
        }
    return MOEQ_OK;
}

int check_hk(const char* what, int H, int I) {
    if (H <= 0 || I <= 0) return fail(MOEQ_EINVAL, "%s: H = %d and I = %d must be positive", what, H, I);
    if (H % 64 || I % 64)
        return fail(MOEQ_EUNSUPPORTED, "%s: H = %d and I = %d must be multiples of 64", what, H, I);
    return MOEQ_OK;
}

// Workgroups of a persistent launch: enough to hold every item once, at most as many as are
// resident at once (2 workgroups of 8 wavefronts per CU: 4 wavefronts per SIMD).
// Which projection kernels run: the prefill kernels (128-row MFMA tiles, weights decoded into
// LDS once per tile) when experts get many rows on average, the decode kernels (4-row tiles,
// weights decoded in registers, one pass over the weights) otherwise. MOEQ_FORCE_PATH=decode
// or prefill overrides the choice (both are exact; used to test each on the same inputs).
// The few-rows kernels keep one 4-byte entry per sorted row in LDS: they serve up to 4096
// rows (every call with T * k < 16 E, as E <= 256); larger calls always take the other path.
constexpr long long kDecodeMaxRows = 4096;

bool use_prefill_path(int T, int k, int E) {
    if ((long long)T * k > kDecodeMaxRows) return true;
    const char* f = getenv("MOEQ_FORCE_PATH");
    if (f && strcmp(f, "decode") == 0) return false;
    if (f && strcmp(f, "prefill") == 0) return true;
    return (long long)T * k >= 16LL * E;     // >= 16 rows per expert on average
}



}  // namespace

extern "C" {

const char* moeq_last_error(void) { return g_err; }

size_t moeq_workspace_bytes(int T, int k, int E, int H, int I) {
    (void)k; (void)E; (void)I;
    // the prefill kernels' work-queue counters, then x in pair-split order (gate|up)
    if (T <= 0 || H <= 0) return 0;
    return prefill_queue_bytes() + prefill_split_bytes(T, H);
}

int moeq_router_logits(const uint16_t* x, int T, int H, const uint16_t* router_w, int E,
                       float* logits, void* stream) {
    const char* w = "moeq_router_logits";
    if (T < 0 || H <= 0 || E < 1 || E > MOEQ_MAX_EXPERTS)
        return fail(MOEQ_EINVAL, "%s: bad sizes T=%d H=%d E=%d", w, T, H, E);
    if (H % 64 != 0) return fail(MOEQ_EUNSUPPORTED, "%s: H=%d must be a multiple of 64", w, H);
    if ((long long)T * H * 2 >= (1LL << 31) || (long long)E * H * 2 >= (1LL << 31))
        return fail(MOEQ_EUNSUPPORTED, "%s: x and router_w must be under 2 GiB (T=%d, H=%d)", w, T, H);
    if (T == 0) return ok();
    if (!x || !router_w || !logits) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(logits, 4))
        return fail(MOEQ_EUNSUPPORTED, "%s: x and router_w must be 16-byte aligned, logits 4-byte aligned", w);
    clear_hip_error();
    launch_router_logits(x, T, H, router_w, E, logits, (hipStream_t)stream);
    return check_launch(w);
}

int moeq_route_topk(const float* logits, int T, int E, int k, int gating, int32_t* topk_ids,
                    float* topk_w, void* stream) {
    const char* w = "moeq_route_topk";
    if (int r = check_sizes(w, T, k, E)) return r;
    if (gating != MOEQ_GATING_SOFTMAX_TOPK && gating != MOEQ_GATING_SIGMOID_TOPK)
        return fail(MOEQ_EINVAL, "%s: unknown gating %d", w, gating);
    if (T == 0) return ok();
    if (!logits || !topk_ids || !topk_w) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    clear_hip_error();
    launch_route_topk(logits, T, E, k, gating == MOEQ_GATING_SIGMOID_TOPK, topk_ids, topk_w,
                      (hipStream_t)stream);
    return check_launch(w);
}

int moeq_permute_by_expert(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                           int32_t* sorted_pair, int32_t* pair_pos, void* stream) {
    const char* w = "moeq_permute_by_expert";
    if (int r = check_sizes(w, T, k, E)) return r;
    if (!expert_offsets) return fail(MOEQ_EINVAL, "%s: expert_offsets is NULL", w);
    if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos)) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    clear_hip_error();
    launch_permute(topk_ids, T * k, E, expert_offsets, sorted_pair, pair_pos, (hipStream_t)stream);
    return check_launch(w);
}

// tokens up to which moeq_route_permute runs as one workgroup (beyond: the two kernels)
constexpr int kRoutePermuteOneGroup = 64;

int moeq_route_permute(const float* logits, int T, int E, int k, int gating, int32_t* topk_ids,
                       float* topk_w, int32_t* expert_offsets, int32_t* sorted_pair,
                       int32_t* pair_pos, void* stream) {
    const char* w = "moeq_route_permute";
    if (int r = check_sizes(w, T, k, E)) return r;
    if (gating != MOEQ_GATING_SOFTMAX_TOPK && gating != MOEQ_GATING_SIGMOID_TOPK)
        return fail(MOEQ_EINVAL, "%s: unknown gating %d", w, gating);
    if (!expert_offsets) return fail(MOEQ_EINVAL, "%s: expert_offsets is NULL", w);
    if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_pair || !pair_pos))
        return fail(MOEQ_EINVAL, "%s: null pointer", w);
    const bool sig = gating == MOEQ_GATING_SIGMOID_TOPK;
    clear_hip_error();
    if (T <= kRoutePermuteOneGroup) {
        launch_route_permute(logits, T, E, k, sig, topk_ids, topk_w, expert_offsets, sorted_pair,
                             pair_pos, (hipStream_t)stream);
    } else {
        launch_route_topk(logits, T, E, k, sig, topk_ids, topk_w, (hipStream_t)stream);
        launch_permute(topk_ids, T * k, E, expert_offsets, sorted_pair, pair_pos,
                       (hipStream_t)stream);
    }
    return check_launch(w);
}

static int projection(const char* w, bool gateup, const uint16_t* act, int T, int H, int I, int E,
                      int k, const int32_t* offsets, const int32_t* sorted_pair, const float* topk_w,
                      const uint8_t* codes0, const uint8_t* scales0, const uint8_t* codes1,
                      const uint8_t* scales1, const float* tables, int n_tables,
                      const uint8_t* table_id, void* out, void* ws, size_t ws_bytes,
                      hipStream_t stream, bool launch = true) {
    if (int r = check_sizes(w, T, k, E)) return r;
    if (int r = check_hk(w, H, I)) return r;
    SkinnyArgs a;
    memset(&a, 0, sizeof(a));
    if (int r = check_tables(w, tables, n_tables, &a.tables)) return r;
    // no tokens: nothing is read or written, so the arrays may be NULL (an empty tensor's
    // address), as for routing, permutation and combine
    if (T == 0 && launch) return ok();
    if (!act || !offsets || !sorted_pair || !codes0 || !scales0 || !table_id || !out ||
        (gateup && (!codes1 || !scales1)) || (!gateup && !topk_w))
        return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(act, 16) || !aligned(codes0, 16) || !aligned(out, 16) || !aligned(scales0, 4) ||
        (gateup && (!aligned(codes1, 16) || !aligned(scales1, 4))))
        return fail(MOEQ_EUNSUPPORTED, "%s: codes, activations and outputs must be 16-byte aligned, scales 4-byte aligned", w);
    const size_t need = moeq_workspace_bytes(T, k, E, H, I);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(MOEQ_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", w, need, ws_bytes);
    if (need > 0 && !aligned(ws, 16))
        return fail(MOEQ_EUNSUPPORTED, "%s: the workspace must be 16-byte aligned", w);
    const long long act_bytes = gateup ? (long long)T * H * 2 : (long long)T * k * I * 2;
    const long long mat_bytes = gateup ? (long long)I * H / 2 : (long long)H * I / 2;
    if (act_bytes >= (1LL << 31) || mat_bytes >= (1LL << 31))
        return fail(MOEQ_EUNSUPPORTED, "%s: activations and each expert matrix must stay below 2 GiB", w);
    if (T == 0 || !launch) return ok();
    a.act = act;
    a.act_bytes = (uint32_t)act_bytes;
    a.offsets = offsets;
    a.sorted_pair = sorted_pair;
    a.topk_w = topk_w;
    a.codes0 = codes0;
    a.scales0 = scales0;
    a.codes1 = codes1;
    a.scales1 = scales1;
    a.table_id = table_id;
    a.out = out;
    a.T = T;
    a.k = k;
    a.E = E;
    a.N = gateup ? I : H;
    a.K = gateup ? H : I;
    a.out_ld = gateup ? I : H;

    a.queue = static_cast<int32_t*>(ws);
    const long touched = (long)(E < T * k ? E : T * k);
    clear_hip_error();
    const bool prefill = use_prefill_path(T, k, E);
    if (gateup && prefill) {
        // the many-rows kernels read x in the decoder's pair-split K order
        uint16_t* xs = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + prefill_queue_bytes());
        launch_pair_split_rows(static_cast<const uint16_t*>(act), T, H, xs, cu_count(), stream);
        a.act = xs;
    } else if (gateup) {
        // the few-rows kernels reorder the x rows they stage, in LDS
        a.act_natural = 1;
    }
    if (prefill) {
        // upper bound of the 128-row tiles the device will find
        const long tiles = touched + (long)T * k / prefill_tile_rows();
        const char* groups_env = getenv("MOEQ_PREFILL_WORKGROUPS");   // testing only
        launch_prefill(a, gateup, tiles, cu_count(), groups_env ? atoi(groups_env) : 0, stream);
    } else {
        // upper bound of the 4-row tiles the device will find
        const long tiles = touched + (long)T * k / decode_tile_rows();
        const char* shape_env = getenv("MOEQ_DECODE_SHAPE");   // tuning only (0..4)
        launch_decode(a, gateup, tiles, cu_count(), shape_env ? atoi(shape_env) : 0, stream);
    }
    return check_launch(w);
}

int moeq_gateup_swiglu(const uint16_t* x, int T, int H, int I, int E, int k,
                       const int32_t* expert_offsets, const int32_t* sorted_pair,
                       const uint8_t* gate_codes, const uint8_t* gate_scales,
                       const uint8_t* up_codes, const uint8_t* up_scales, const float* tables,
                       int n_tables, const uint8_t* table_id, uint16_t* inter, void* ws,
                       size_t ws_bytes, void* stream) {
    return projection("moeq_gateup_swiglu", true, x, T, H, I, E, k, expert_offsets, sorted_pair,
                      nullptr, gate_codes, gate_scales, up_codes, up_scales, tables, n_tables,
                      table_id, inter, ws, ws_bytes, (hipStream_t)stream);
}

// The static scratch of moeq_gateup_swiglu_static. In host code `scratch` is only a stand-in
// for the symbol: its device address on the current device comes from hipGetSymbolAddress
// (each device holds its own copy), kept per device in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[MOEQ_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call there.
int static_scratch(const char* w, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        clear_hip_error();
        return fail(MOEQ_ELAUNCH, "%s: no current device (or device id %d >= %d)", w, dev,
                    kMaxDevices);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            clear_hip_error();
            return fail(MOEQ_ELAUNCH, "%s: the static scratch has no address on device %d: %s",
                        w, dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOEQ_OK;
}
}  // namespace

int moeq_gateup_swiglu_static(const uint16_t* x, int T, int H, int I, int E, int k,
                              const int32_t* expert_offsets, const int32_t* sorted_pair,
                              const uint8_t* gate_codes, const uint8_t* gate_scales,
                              const uint8_t* up_codes, const uint8_t* up_scales,
                              const float* tables, int n_tables, const uint8_t* table_id,
                              uint16_t* inter, void* stream) {
    const char* w = "moeq_gateup_swiglu_static";
    if (T > 0 && H > 0) {
        const size_t need = moeq_workspace_bytes(T, k, E, H, I);
        if (need > MOEQ_STATIC_SCRATCH_BYTES)
            return fail(MOEQ_EWORKSPACE,
                        "%s: T = %d, H = %d need %zu bytes of scratch, above the static %zu "
                        "(use moeq_gateup_swiglu with a workspace)",
                        w, T, H, need, (size_t)MOEQ_STATIC_SCRATCH_BYTES);
    }
    void* ws = nullptr;
    if (T > 0)
        if (int r = static_scratch(w, &ws)) return r;
    return projection(w, true, x, T, H, I, E, k, expert_offsets, sorted_pair, nullptr,
                      gate_codes, gate_scales, up_codes, up_scales, tables, n_tables, table_id,
                      inter, ws, MOEQ_STATIC_SCRATCH_BYTES, (hipStream_t)stream);
}

int moeq_down(const uint16_t* inter, int T, int H, int I, int E, int k,
              const int32_t* expert_offsets, const int32_t* sorted_pair, const float* topk_w,
              const uint8_t* down_codes, const uint8_t* down_scales, const float* tables,
              int n_tables, const uint8_t* table_id, float* yp, void* ws, size_t ws_bytes,
              void* stream) {
    return projection("moeq_down", false, inter, T, H, I, E, k, expert_offsets, sorted_pair, topk_w,
                      down_codes, down_scales, nullptr, nullptr, tables, n_tables, table_id, yp, ws,
                      ws_bytes, (hipStream_t)stream);
}

static int combine(const char* w, const float* yp, const int32_t* pair_pos,
                   const int32_t* expert_offsets, int T, int k, int E, int H,
                   const float* shared_z, const uint16_t* residual, uint16_t* y,
                   hipStream_t stream) {
    if (int r = check_sizes(w, T, k, E)) return r;
    if (H <= 0 || H % 4) return fail(MOEQ_EUNSUPPORTED, "%s: H = %d must be a positive multiple of 4", w, H);
    if (T == 0) return ok();
    if (!yp || !pair_pos || !expert_offsets || !y) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(yp, 16) || !aligned(y, 8) || (residual && !aligned(residual, 8)) ||
        (shared_z && !aligned(shared_z, 16)))
        return fail(MOEQ_EUNSUPPORTED, "%s: yp and shared_z must be 16-byte aligned, y and residual 8-byte aligned", w);
    clear_hip_error();
    launch_combine(yp, pair_pos, expert_offsets, T, k, E, H, shared_z, residual, y, stream);
    return check_launch(w);
}

int moeq_unpermute_combine(const float* yp, const int32_t* pair_pos, const int32_t* expert_offsets,
                           int T, int k, int E, int H, const uint16_t* residual, uint16_t* y,
                           void* stream) {
    return combine("moeq_unpermute_combine", yp, pair_pos, expert_offsets, T, k, E, H, nullptr,
                   residual, y, (hipStream_t)stream);
}

int moeq_unpermute_combine_shared(const float* yp, const int32_t* pair_pos,
                                  const int32_t* expert_offsets, int T, int k, int E, int H,
                                  const float* shared_z, const uint16_t* residual, uint16_t* y,
                                  void* stream) {
    return combine("moeq_unpermute_combine_shared", yp, pair_pos, expert_offsets, T, k, E, H,
                   shared_z, residual, y, (hipStream_t)stream);
}

size_t moeq_shared_workspace_bytes(int T, int H, int I) {
    if (T <= 0 || H <= 0) return 0;
    return shared_routing_bytes(T) + moeq_workspace_bytes(T, 1, 1, H, I);
}

int moeq_shared_expert(const uint16_t* x, int T, int H, int I, const uint8_t* gate_codes,
                       const uint8_t* gate_scales, const uint8_t* up_codes,
                       const uint8_t* up_scales, const uint8_t* down_codes,
                       const uint8_t* down_scales, const float* tables, int n_tables,
                       const uint8_t* table_id, uint16_t* inter, float* z, void* ws,
                       size_t ws_bytes, void* stream) {
    const char* w = "moeq_shared_expert";
    if (T < 0 || H <= 0) return fail(MOEQ_EINVAL, "%s: bad sizes T=%d H=%d", w, T, H);
    if (T == 0) return ok();
    const size_t need = moeq_shared_workspace_bytes(T, H, I);
    if (!ws || ws_bytes < need)
        return fail(MOEQ_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", w, need, ws_bytes);
    if (!aligned(ws, 256))
        return fail(MOEQ_EUNSUPPORTED, "%s: the workspace must be 256-byte aligned", w);
    // workspace: identity routing (offsets {0, T}, sorted_pair = 0..T-1, gate weights 1), then
    // the projections' own workspace
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base);
    int32_t* sorted_pair = reinterpret_cast<int32_t*>(base + 256);
    float* ones = reinterpret_cast<float*>(base + 256 + shared_rows_bytes(T));
    void* pws = base + shared_routing_bytes(T);
    const size_t pws_bytes = need - shared_routing_bytes(T);
    // validate both projections before launching anything
    if (int r = projection(w, true, x, T, H, I, 1, 1, offsets, sorted_pair, nullptr, gate_codes,
                           gate_scales, up_codes, up_scales, tables, n_tables, table_id, inter,
                           pws, pws_bytes, (hipStream_t)stream, false))
        return r;
    if (int r = projection(w, false, inter, T, H, I, 1, 1, offsets, sorted_pair, ones, down_codes,
                           down_scales, nullptr, nullptr, tables, n_tables, table_id, z, pws,
                           pws_bytes, (hipStream_t)stream, false))
        return r;
    clear_hip_error();
    launch_identity_routing(T, offsets, sorted_pair, ones, (hipStream_t)stream);
    if (int r = check_launch(w)) return r;
    if (int r = projection(w, true, x, T, H, I, 1, 1, offsets, sorted_pair, nullptr, gate_codes,
                           gate_scales, up_codes, up_scales, tables, n_tables, table_id, inter,
                           pws, pws_bytes, (hipStream_t)stream))
        return r;
    return projection(w, false, inter, T, H, I, 1, 1, offsets, sorted_pair, ones, down_codes,
                      down_scales, nullptr, nullptr, tables, n_tables, table_id, z, pws, pws_bytes,
                      (hipStream_t)stream);
}

// Workspace of moeq_moe_decode, in 256-byte aligned regions.
struct DecodeWs {
    size_t bar, ids, w, offsets, sorted_pair, pair_pos, inter, yp, total;
};

static size_t up256(size_t n) { return (n + 255) / 256 * 256; }

static DecodeWs decode_ws(int T, int k, int E, int H, int I) {
    DecodeWs d;
    const size_t P = (size_t)T * k;
    size_t o = 0;
    d.bar = o;          o += 256;
    d.ids = o;          o += up256(P * 4);
    d.w = o;            o += up256(P * 4);
    d.offsets = o;      o += up256((size_t)(E + 1) * 4);
    d.sorted_pair = o;  o += up256(P * 4);
    d.pair_pos = o;     o += up256(P * 4);
    d.inter = o;        o += up256(P * I * 2);
    d.yp = o;           o += up256(P * H * 4);
    d.total = o;
    return d;
}

static int check_ascending(const char* w, const float* table, int t) {
    for (int m = 1; m < 8; ++m)
        if (!(table[m] >= table[m - 1]))
            return fail(MOEQ_EINVAL, "%s: table %d must be non-decreasing (entry %d < entry %d)", w,
                        t, m, m - 1);
    if (!(table[7] > 0.0f))
        return fail(MOEQ_EINVAL, "%s: table %d has no positive magnitude", w, t);
    return MOEQ_OK;
}

int moeq_quantize(const uint16_t* wts, int E, int N, int K, const float* tables, int n_tables,
                  const uint8_t* table_id, uint8_t* codes, uint8_t* scales, double* row_err,
                  void* stream) {
    const char* w = "moeq_quantize";
    if (E < 1 || N < 1 || K < 32) return fail(MOEQ_EINVAL, "%s: bad sizes E=%d N=%d K=%d", w, E, N, K);
    if (K % 32) return fail(MOEQ_EUNSUPPORTED, "%s: K = %d must be a multiple of 32", w, K);
    TableArgs ta;
    if (int r = check_tables(w, tables, n_tables, &ta)) return r;
    for (int t = 0; t < n_tables; ++t)
        if (int r = check_ascending(w, tables + 8 * t, t)) return r;
    if (!wts || !table_id) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(wts, 16) || (codes && !aligned(codes, 16)) || (row_err && !aligned(row_err, 8)))
        return fail(MOEQ_EUNSUPPORTED, "%s: w and codes must be 16-byte aligned, row_err 8-byte aligned", w);
    if ((long long)E * N >= (1LL << 33)) return fail(MOEQ_EUNSUPPORTED, "%s: too many rows", w);
    clear_hip_error();
    launch_quantize(wts, (long long)E * N, K, N, ta, table_id, codes, scales, row_err,
                    (hipStream_t)stream);
    return check_launch(w);
}

size_t moeq_lloyd_workspace_bytes(int E, int N) {
    if (E < 1 || N < 1) return 0;
    return lloyd_workspace_bytes((long long)E * N);
}

int moeq_lloyd_stats(const uint16_t* wts, int E, int N, int K, const float* table, float gmax,
                     int accumulate, double* stats, void* ws, size_t ws_bytes, void* stream) {
    const char* w = "moeq_lloyd_stats";
    if (E < 1 || N < 1 || K < 32) return fail(MOEQ_EINVAL, "%s: bad sizes E=%d N=%d K=%d", w, E, N, K);
    if (K % 32) return fail(MOEQ_EUNSUPPORTED, "%s: K = %d must be a multiple of 32", w, K);
    TableArgs ta;
    if (int r = check_tables(w, table, 1, &ta)) return r;
    if (int r = check_ascending(w, table, 0)) return r;
    if (!(gmax > 0.0f) || !isfinite(gmax)) return fail(MOEQ_EINVAL, "%s: gmax = %g must be positive and finite", w, (double)gmax);
    if (!wts || !stats) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    const size_t need = moeq_lloyd_workspace_bytes(E, N);
    if (!ws || ws_bytes < need)
        return fail(MOEQ_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", w, need, ws_bytes);
    if (!aligned(wts, 16) || !aligned(stats, 8) || !aligned(ws, 8))
        return fail(MOEQ_EUNSUPPORTED, "%s: w must be 16-byte aligned, stats and ws 8-byte aligned", w);
    if ((long long)E * N >= (1LL << 33)) return fail(MOEQ_EUNSUPPORTED, "%s: too many rows", w);
    Table8 tab;
    for (int m = 0; m < 8; ++m) tab.v[m] = table[m];
    clear_hip_error();
    launch_lloyd_stats(wts, (long long)E * N, K, tab, gmax, static_cast<double*>(ws),
                       accumulate ? 1 : 0, stats, (hipStream_t)stream);
    return check_launch(w);
}

int moeq_lloyd_update(const double* stats, const float* table, float* next, double* sq_error) {
    const char* w = "moeq_lloyd_update";
    if (!stats || !table || !next) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    float out[8];
    double err = 0.0;
    for (int m = 0; m < 8; ++m) {
        out[m] = stats[8 + m] > 0.0 ? (float)(stats[m] / stats[8 + m]) : table[m];
        err += stats[16 + m];
    }
    for (int m = 0; m < 8; ++m) next[m] = out[m];
    if (sq_error) *sq_error = err;
    return ok();
}

int moeq_select_arms(const double* err_a, const double* err_b, int E, int N, int accumulate,
                     uint8_t* table_id, double* expert_err, void* stream) {
    const char* w = "moeq_select_arms";
    if (E < 1 || N < 1) return fail(MOEQ_EINVAL, "%s: bad sizes E=%d N=%d", w, E, N);
    if (!err_a || !err_b || !table_id || (accumulate && !expert_err))
        return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(err_a, 8) || !aligned(err_b, 8) || (expert_err && !aligned(expert_err, 8)))
        return fail(MOEQ_EUNSUPPORTED, "%s: error arrays must be 8-byte aligned", w);
    clear_hip_error();
    launch_select_arms(err_a, err_b, E, N, accumulate ? 1 : 0, table_id, expert_err,
                       (hipStream_t)stream);
    return check_launch(w);
}

size_t moeq_moe_decode_workspace_bytes(int T, int k, int E, int H, int I) {
    if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
    return decode_ws(T, k, E, H, I).total;
}

int moeq_moe_decode(const uint16_t* x, const float* logits, int T, int H, int I, int E, int k,
                    int gating, const uint8_t* gate_codes, const uint8_t* gate_scales,
                    const uint8_t* up_codes, const uint8_t* up_scales, const uint8_t* down_codes,
                    const uint8_t* down_scales, const float* tables, int n_tables,
                    const uint8_t* table_id, const uint16_t* residual, uint16_t* y, void* ws,
                    size_t ws_bytes, void* stream) {
    const char* w = "moeq_moe_decode";
    if (int r = check_sizes(w, T, k, E)) return r;
    if (gating != MOEQ_GATING_SOFTMAX_TOPK && gating != MOEQ_GATING_SIGMOID_TOPK)
        return fail(MOEQ_EINVAL, "%s: unknown gating %d", w, gating);
    if (T == 0) return ok();
    if ((long long)T * k > kDecodeMaxRows)
        return fail(MOEQ_EUNSUPPORTED, "%s: T * k = %lld above %lld rows (use the per-step calls)",
                    w, (long long)T * k, kDecodeMaxRows);
    if (!x || !logits || !y) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(y, 8) || (residual && !aligned(residual, 8)))
        return fail(MOEQ_EUNSUPPORTED, "%s: y and residual must be 8-byte aligned", w);
    const DecodeWs d = decode_ws(T, k, E, H, I);
    if (!ws || ws_bytes < d.total)
        return fail(MOEQ_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", w, d.total, ws_bytes);
    if (!aligned(ws, 256)) return fail(MOEQ_EUNSUPPORTED, "%s: the workspace must be 256-byte aligned", w);
    uint8_t* b = static_cast<uint8_t*>(ws);
    DecodeLayerArgs L;
    memset(&L, 0, sizeof(L));
    L.barrier = reinterpret_cast<int*>(b + d.bar);
    L.ids = reinterpret_cast<int32_t*>(b + d.ids);
    L.w = reinterpret_cast<float*>(b + d.w);
    L.offsets = reinterpret_cast<int32_t*>(b + d.offsets);
    L.sorted_pair = reinterpret_cast<int32_t*>(b + d.sorted_pair);
    L.pair_pos = reinterpret_cast<int32_t*>(b + d.pair_pos);
    uint16_t* inter = reinterpret_cast<uint16_t*>(b + d.inter);
    float* yp = reinterpret_cast<float*>(b + d.yp);
    // both projections validated as the per-step calls would (their workspace is unused here)
    const size_t pws = moeq_workspace_bytes(T, k, E, H, I);
    if (int r = projection(w, true, x, T, H, I, E, k, L.offsets, L.sorted_pair, nullptr,
                           gate_codes, gate_scales, up_codes, up_scales, tables, n_tables, table_id,
                           inter, ws, pws, (hipStream_t)stream, false))
        return r;
    if (int r = projection(w, false, inter, T, H, I, E, k, L.offsets, L.sorted_pair, L.w,
                           down_codes, down_scales, nullptr, nullptr, tables, n_tables, table_id,
                           yp, ws, pws, (hipStream_t)stream, false))
        return r;
    auto fill = [&](SkinnyArgs& a, bool gateup) {
        if (int r = check_tables(w, tables, n_tables, &a.tables)) return r;
        a.offsets = L.offsets;
        a.sorted_pair = L.sorted_pair;
        a.table_id = table_id;
        a.T = T;
        a.k = k;
        a.E = E;
        if (gateup) {
            a.act = x;                    // natural order, split in LDS
            a.act_natural = 1;
            a.act_bytes = (uint32_t)((long long)T * H * 2);
            a.codes0 = gate_codes; a.scales0 = gate_scales;
            a.codes1 = up_codes; a.scales1 = up_scales;
            a.out = inter;
            a.N = I; a.K = H; a.out_ld = I;
        } else {
            a.act = inter;
            a.act_bytes = (uint32_t)((long long)T * k * I * 2);
            a.topk_w = L.w;
            a.codes0 = down_codes; a.scales0 = down_scales;
            a.out = yp;
            a.N = H; a.K = I; a.out_ld = H;
        }
        return (int)MOEQ_OK;
    };
    if (int r = fill(L.gu, true)) return r;
    if (int r = fill(L.dn, false)) return r;
    L.logits = logits;
    L.sigmoid = gating == MOEQ_GATING_SIGMOID_TOPK ? 1 : 0;
    L.yp = yp;
    L.residual = residual;
    L.y = y;
    L.T = T; L.k = k; L.E = E; L.H = H;
    clear_hip_error();
    const int g = launch_decode_layer(L, cu_count(), (hipStream_t)stream);
    if (g < 0) return fail(MOEQ_ELAUNCH, "%s: the cooperative launch was refused (%d)", w, g);
    return check_launch(w);
}

int moeq_moe_decode_check(const void* ws, void* stream) {
    const char* w = "moeq_moe_decode_check";
    if (!ws) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    int flag = 0;
    clear_hip_error();
    if (hipMemcpyAsync(&flag, static_cast<const uint8_t*>(ws) + 4, sizeof(int),
                       hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
        hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return fail(MOEQ_ELAUNCH, "%s: reading the barrier word failed", w);
    if (flag) return fail(MOEQ_ELAUNCH, "%s: a grid barrier of the last call gave up waiting", w);
    return ok();
}

int moeq_debug_dequant(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                       const float* tables, int n_tables, const uint8_t* table_id, uint16_t* out,
                       void* stream) {
    const char* w = "moeq_debug_dequant";
    if (E < 1 || N < 1 || K < 1) return fail(MOEQ_EINVAL, "%s: sizes must be positive", w);
    if (K % 64) return fail(MOEQ_EUNSUPPORTED, "%s: K = %d must be a multiple of 64", w, K);
    TableArgs ta;
    if (int r = check_tables(w, tables, n_tables, &ta)) return r;
    if (!codes || !scales || !table_id || !out) return fail(MOEQ_EINVAL, "%s: null pointer", w);
    if (!aligned(codes, 4) || !aligned(out, 16))
        return fail(MOEQ_EUNSUPPORTED, "%s: codes must be 4-byte aligned, out 16-byte aligned", w);
    const size_t total = (size_t)E * N * (K / 8);
    size_t blocks = (total + 255) / 256;
    if (blocks > (size_t)cu_count() * 16) blocks = (size_t)cu_count() * 16;
    clear_hip_error();
    launch_dequant(codes, scales, E, N, K, table_id, ta, out, (int)blocks, (hipStream_t)stream);
    return check_launch(w);
}

}  // extern "C"
