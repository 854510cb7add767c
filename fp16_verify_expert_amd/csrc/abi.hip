// C ABI of libsmoe.so: host-side argument checks, device check, dispatch.
// Every check runs before anything is enqueued; no call allocates memory.
#include <atomic>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_err;

smoe_status fail(smoe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

smoe_status ok() {
    g_err.clear();
    return SMOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

smoe_status hip_result(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(SMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// gfx950 check, once per device.
smoe_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SMOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    static std::mutex mu;
    static int state[256];  // 0 unknown, 1 gfx950, 2 other
    static char names[256][64];
    if (dev < 0 || dev >= 256) return fail(SMOE_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(SMOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        snprintf(names[dev], sizeof(names[dev]), "%s", prop.gcnArchName);
        state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (state[dev] != 1)
        return fail(SMOE_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                    names[dev]);
    return SMOE_OK;
}

#define REQUIRE(cond, st, ...)                     \
    do {                                           \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

#define CHECK_DEVICE()                         \
    do {                                       \
        smoe_status _s = check_device();       \
        if (_s != SMOE_OK) return _s;          \
    } while (0)

smoe_status check_hek(int H, int E, int k) {
    REQUIRE(H > 0 && H % 128 == 0, SMOE_ERR_SHAPE, "H=%d must be a positive multiple of 128", H);
    REQUIRE(E >= 1 && E <= 256, SMOE_ERR_SHAPE, "E=%d must be in [1, 256]", E);
    REQUIRE(k >= 1 && k <= E, SMOE_ERR_SHAPE, "k=%d must be in [1, E=%d]", k, E);
    return SMOE_OK;
}

constexpr long long kMaxPairs = 1 << 20;

// Host checks shared by the grouped draft-FFN entry points (everything but
// the workspace); `name` prefixes the error message.
smoe_status check_wq(const char* name, const uint16_t* x, const int32_t* sorted_token,
                     const int32_t* expert_offsets, const int32_t* active,
                     const int32_t* n_active, const smoe_w4_expert* experts, int T, int k, int H,
                     int I, int E, int bits, int group_size, const uint16_t* y_sorted) {
    REQUIRE(x && sorted_token && expert_offsets && active && n_active && experts && y_sorted,
            SMOE_ERR_NULL, "%s: a required pointer is NULL", name);
    REQUIRE(T >= 0, SMOE_ERR_SHAPE, "%s: T=%d < 0", name, T);
    REQUIRE(bits == 2 || bits == 4 || bits == 8, SMOE_ERR_UNSUPPORTED, "%s: bits=%d (2, 4 or 8)",
            name, bits);
    smoe_status st = check_hek(H, E, k);
    if (st != SMOE_OK) return st;
    REQUIRE(I > 0 && I % 128 == 0, SMOE_ERR_SHAPE, "%s: I=%d must be a positive multiple of 128",
            name, I);
    REQUIRE(group_size == 128, SMOE_ERR_UNSUPPORTED,
            "%s: group_size=%d (only 128 is supported)", name, group_size);
    REQUIRE((long long)T * k <= kMaxPairs, SMOE_ERR_SHAPE, "%s: T*k exceeds 2^20", name);
    REQUIRE(smoe::w4a16_shape_supported(H, I), SMOE_ERR_SHAPE,
            "%s: H=%d, I=%d (each must be <= 16384)", name, H, I);
    REQUIRE(aligned(x, 16), SMOE_ERR_SHAPE, "%s: x must be 16-byte aligned", name);
    return SMOE_OK;
}

// Rewrites the thread's error message so it names `to` instead of `from`
// (entry points that forward to another one report under their own name).
void rename_error(const char* from, const char* to) {
    const size_t n = strlen(from);
    if (g_err.compare(0, n, from) == 0) g_err = std::string(to) + g_err.substr(n);
}

// Scratch memory of w4a16_grouped_ffn_noalloc: a file-scope device array, so
// the call needs no allocation.  Each GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol); it passes the device address looked up once per device below.
constexpr size_t kNoAllocScratch = SMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

// Device address of `scratch` on the current device, looked up with
// hipGetSymbolAddress on the first call made with that device current.
smoe_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SMOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 256) return fail(SMOE_ERR_UNSUPPORTED, "device index %d", dev);
    static std::mutex mu;
    static void* addr[256];
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SMOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return SMOE_OK;
}

// one-row matrix-vector reductions of a shared expert: 16 chunks of 16 bytes
// per lane and row
constexpr int kSharedMaxK = 8192;

}  // namespace

namespace smoe {
// CUs of the current device (cached per device); 0 if it cannot be queried.
int device_cu_count() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (!n) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace smoe

extern "C" {

int smoe_abi_version(void) { return SMOE_ABI_VERSION; }

const char* smoe_last_error(void) { return g_err.c_str(); }

smoe_status smoe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                             void* stream) {
    REQUIRE(src && sink, SMOE_ERR_NULL, "smoe_stream_read: src and sink are required");
    REQUIRE(bytes % 16 == 0 && aligned(src, 16), SMOE_ERR_SHAPE,
            "smoe_stream_read: bytes=%zu must be a multiple of 16 and src 16-byte aligned", bytes);
    REQUIRE(blocks >= 1 && blocks <= 65535, SMOE_ERR_SHAPE,
            "smoe_stream_read: blocks=%d must be in [1, 65535]", blocks);
    if (bytes == 0) return ok();
    CHECK_DEVICE();
    return hip_result(smoe::launch_stream_read(src, bytes, sink, blocks,
                                               static_cast<hipStream_t>(stream)),
                      "smoe_stream_read launch");
}

size_t smoe_workspace_bytes(int which, int T, int k, int H, int I, int E) {
    if (T < 0 || k < 1 || E < 1 || E > 256 || H <= 0 || I <= 0 || H % 128 || I % 128) return 0;
    if ((long long)T * k > kMaxPairs) return 0;
    if (which == 0) return smoe::w4a16_workspace_bytes(T, k, H, I, E);
    if (which == 1) return smoe::verify_workspace_bytes(T, T * k, H, I, E);
    if (which == 2) return T == 1 ? smoe::draft_layer_workspace_bytes(k, I, E) : 0;
    return 0;
}

smoe_status moe_route_topk(const uint16_t* x, const uint16_t* w_router,
                           const uint16_t* w_shared_gate, int T, int H, int E, int k,
                           int renormalize, int32_t* topk_ids, float* topk_w,
                           float* shared_gate, void* stream) {
    REQUIRE(x && w_router && topk_ids && topk_w, SMOE_ERR_NULL,
            "moe_route_topk: x, w_router, topk_ids and topk_w are required");
    REQUIRE(!w_shared_gate || shared_gate, SMOE_ERR_NULL,
            "moe_route_topk: shared_gate output is required with w_shared_gate");
    REQUIRE(T >= 0, SMOE_ERR_SHAPE, "moe_route_topk: T=%d < 0", T);
    smoe_status st = check_hek(H, E, k);
    if (st != SMOE_OK) return st;
    REQUIRE(aligned(x, 16) && aligned(w_router, 16) && aligned(w_shared_gate, 16),
            SMOE_ERR_SHAPE, "moe_route_topk: x, w_router, w_shared_gate must be 16-byte aligned");
    if (T == 0) return ok();
    CHECK_DEVICE();
    return hip_result(smoe::launch_route_topk(x, w_router, w_shared_gate, T, H, E, k,
                                              renormalize ? 1 : 0, topk_ids, topk_w, shared_gate,
                                              static_cast<hipStream_t>(stream)),
                      "moe_route_topk launch");
}

smoe_status elb_count(const int32_t* topk_ids, int T, int k, int E, int layer, int L,
                      int32_t* counters, int32_t* err_word, void* stream) {
    REQUIRE(topk_ids && counters, SMOE_ERR_NULL, "elb_count: topk_ids and counters are required");
    REQUIRE(T >= 0, SMOE_ERR_SHAPE, "elb_count: T=%d < 0", T);
    REQUIRE(E >= 1 && E <= 256 && k >= 1 && k <= E, SMOE_ERR_SHAPE,
            "elb_count: need 1 <= k=%d <= E=%d <= 256", k, E);
    REQUIRE(L >= 1 && layer >= 0 && layer < L, SMOE_ERR_SHAPE,
            "elb_count: layer=%d must be in [0, L=%d)", layer, L);
    REQUIRE((long long)T * k <= kMaxPairs, SMOE_ERR_SHAPE, "elb_count: T*k exceeds 2^20");
    if (T == 0) return ok();
    CHECK_DEVICE();
    return hip_result(smoe::launch_elb_count(topk_ids, T * k, E, layer, counters, err_word,
                                             static_cast<hipStream_t>(stream)),
                      "elb_count launch");
}

smoe_status moe_gather(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                       int32_t* sorted_token, int32_t* sorted_pair, int32_t* pair_pos,
                       int32_t* active, int32_t* n_active, int32_t* err_word, void* stream) {
    REQUIRE(expert_offsets && active && n_active, SMOE_ERR_NULL,
            "moe_gather: expert_offsets, active and n_active are required");
    REQUIRE(T == 0 || (topk_ids && sorted_token && sorted_pair && pair_pos), SMOE_ERR_NULL,
            "moe_gather: topk_ids, sorted_token, sorted_pair and pair_pos are required");
    REQUIRE(T >= 0, SMOE_ERR_SHAPE, "moe_gather: T=%d < 0", T);
    REQUIRE(E >= 1 && E <= 256 && k >= 1 && k <= E, SMOE_ERR_SHAPE,
            "moe_gather: need 1 <= k=%d <= E=%d <= 256", k, E);
    REQUIRE((long long)T * k <= kMaxPairs, SMOE_ERR_SHAPE, "moe_gather: T*k exceeds 2^20");
    CHECK_DEVICE();
    // T == 0 still writes empty maps (zero offsets, no active experts).
    return hip_result(smoe::launch_gather(topk_ids, T * k, k, E, expert_offsets, sorted_token,
                                          sorted_pair, pair_pos, active, n_active, err_word,
                                          static_cast<hipStream_t>(stream)),
                      "moe_gather launch");
}

smoe_status moe_route_plan(const uint16_t* x, const uint16_t* w_router,
                           const uint16_t* w_shared_gate, int T, int H, int E, int k,
                           int renormalize, int layer, int L, int32_t* counters,
                           int32_t* topk_ids, float* topk_w, float* shared_gate,
                           int32_t* expert_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                           int32_t* pair_pos, int32_t* active, int32_t* n_active,
                           void* workspace, size_t workspace_bytes, int32_t* err_word,
                           void* stream) {
    REQUIRE(expert_offsets && active && n_active, SMOE_ERR_NULL,
            "moe_route_plan: expert_offsets, active and n_active are required");
    REQUIRE(T == 0 || (x && w_router && topk_ids && topk_w && sorted_token && sorted_pair &&
                       pair_pos),
            SMOE_ERR_NULL,
            "moe_route_plan: x, w_router, topk_ids, topk_w and the sorted maps are required");
    REQUIRE(!w_shared_gate || shared_gate, SMOE_ERR_NULL,
            "moe_route_plan: shared_gate output is required with w_shared_gate");
    REQUIRE(T >= 0, SMOE_ERR_SHAPE, "moe_route_plan: T=%d < 0", T);
    smoe_status st = check_hek(H, E, k);
    if (st != SMOE_OK) return st;
    REQUIRE((long long)T * k <= smoe::kPlanMaxPairs, SMOE_ERR_SHAPE,
            "moe_route_plan: T*k=%lld exceeds %d (use the separate calls)", (long long)T * k,
            smoe::kPlanMaxPairs);
    REQUIRE((long long)T * (E + 1) <= smoe::kPlanMaxLogits, SMOE_ERR_SHAPE,
            "moe_route_plan: T*(E+1)=%lld exceeds %d (use the separate calls)",
            (long long)T * (E + 1), smoe::kPlanMaxLogits);
    REQUIRE(!counters || (L >= 1 && layer >= 0 && layer < L), SMOE_ERR_SHAPE,
            "moe_route_plan: layer=%d must be in [0, L=%d)", layer, L);
    REQUIRE(aligned(x, 16) && aligned(w_router, 16) && aligned(w_shared_gate, 16),
            SMOE_ERR_SHAPE, "moe_route_plan: x, w_router, w_shared_gate must be 16-byte aligned");
    const size_t lg_bytes = (size_t)T * (E + (w_shared_gate ? 1 : 0)) * sizeof(float);
    REQUIRE(!workspace || (workspace_bytes >= lg_bytes && aligned(workspace, 16)),
            SMOE_ERR_WORKSPACE,
            "moe_route_plan: workspace of %zu bytes, %zu needed (T*(E+1) fp32 logits, "
            "16-byte aligned)", workspace_bytes, lg_bytes);
    CHECK_DEVICE();
    // T == 0 still writes empty maps (zero offsets, no active experts).
    return hip_result(smoe::launch_route_plan(x, w_router, w_shared_gate, T, H, E, k,
                                              renormalize ? 1 : 0, layer, counters, topk_ids,
                                              topk_w, shared_gate, expert_offsets, sorted_token,
                                              sorted_pair, pair_pos, active, n_active, err_word,
                                              static_cast<float*>(workspace),
                                              static_cast<hipStream_t>(stream)),
                      "moe_route_plan launch");
}

smoe_status wq_grouped_ffn(const uint16_t* x, const int32_t* sorted_token,
                           const int32_t* expert_offsets, const int32_t* active,
                           const int32_t* n_active, const smoe_w4_expert* experts, int T, int k,
                           int H, int I, int E, int bits, int group_size, uint16_t* y_sorted,
                           void* workspace, size_t workspace_bytes, int32_t* err_word,
                           void* stream) {
    smoe_status st = check_wq("wq_grouped_ffn", x, sorted_token, expert_offsets, active,
                              n_active, experts, T, k, H, I, E, bits, group_size, y_sorted);
    if (st != SMOE_OK) return st;
    if (T == 0) return ok();
    const size_t need = smoe::w4a16_workspace_bytes(T, k, H, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "wq_grouped_ffn: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
            workspace_bytes);
    CHECK_DEVICE();
    return hip_result(smoe::launch_w4a16_ffn(x, sorted_token, expert_offsets, active, n_active,
                                             experts, T, k, H, I, E, bits, y_sorted, workspace,
                                             err_word, static_cast<hipStream_t>(stream)),
                      "wq_grouped_ffn launch");
}

smoe_status w4a16_grouped_ffn(const uint16_t* x, const int32_t* sorted_token,
                              const int32_t* expert_offsets, const int32_t* active,
                              const int32_t* n_active, const smoe_w4_expert* experts, int T,
                              int k, int H, int I, int E, int group_size, uint16_t* y_sorted,
                              void* workspace, size_t workspace_bytes, int32_t* err_word,
                              void* stream) {
    const smoe_status st = wq_grouped_ffn(x, sorted_token, expert_offsets, active, n_active,
                                          experts, T, k, H, I, E, 4, group_size, y_sorted,
                                          workspace, workspace_bytes, err_word, stream);
    if (st != SMOE_OK) rename_error("wq_grouped_ffn", "w4a16_grouped_ffn");
    return st;
}

smoe_status awq_grouped_ffn(const uint16_t* x, const int32_t* sorted_token,
                            const int32_t* expert_offsets, const int32_t* active,
                            const int32_t* n_active, const smoe_w4_expert* experts,
                            const uint16_t* const* act_scales, int T, int k, int H, int I, int E,
                            int group_size, uint16_t* y_sorted, void* workspace,
                            size_t workspace_bytes, int32_t* err_word, void* stream) {
    const char* name = "awq_grouped_ffn";
    REQUIRE(act_scales, SMOE_ERR_NULL, "%s: act_scales is required", name);
    smoe_status st = check_wq(name, x, sorted_token, expert_offsets, active, n_active, experts, T,
                              k, H, I, E, 4, group_size, y_sorted);
    if (st != SMOE_OK) return st;
    if (T == 0) return ok();
    const size_t need = smoe::w4a16_workspace_bytes(T, k, H, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", name, need,
            workspace_bytes);
    CHECK_DEVICE();
    return hip_result(smoe::launch_w4a16_ffn(x, sorted_token, expert_offsets, active, n_active,
                                             experts, T, k, H, I, E, 4, y_sorted, workspace,
                                             err_word, static_cast<hipStream_t>(stream),
                                             act_scales),
                      "awq_grouped_ffn launch");
}

smoe_status w4a16_grouped_ffn_noalloc(const uint16_t* x, const int32_t* sorted_token,
                                      const int32_t* expert_offsets, const int32_t* active,
                                      const int32_t* n_active, const smoe_w4_expert* experts,
                                      int T, int k, int H, int I, int E, int group_size,
                                      uint16_t* y_sorted, int32_t* err_word, void* stream) {
    const char* name = "w4a16_grouped_ffn_noalloc";
    smoe_status st = check_wq(name, x, sorted_token, expert_offsets, active, n_active, experts,
                              T, k, H, I, E, 4, group_size, y_sorted);
    if (st != SMOE_OK) return st;
    if (T == 0) return ok();
    const size_t need = smoe::w4a16_workspace_bytes(T, k, H, I, E);
    REQUIRE(need <= kNoAllocScratch, SMOE_ERR_SHAPE,
            "%s: T=%d, k=%d, I=%d needs %zu bytes of scratch; the library holds %zu (use "
            "w4a16_grouped_ffn with a workspace)", name, T, k, I, need, kNoAllocScratch);
    CHECK_DEVICE();
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != SMOE_OK) return st;
    return hip_result(smoe::launch_w4a16_ffn(x, sorted_token, expert_offsets, active, n_active,
                                             experts, T, k, H, I, E, 4, y_sorted, ws, err_word,
                                             static_cast<hipStream_t>(stream)),
                      "w4a16_grouped_ffn_noalloc launch");
}

smoe_status w4a16_grouped_ffn_shared(const uint16_t* x, const int32_t* sorted_token,
                                     const int32_t* expert_offsets, const int32_t* active,
                                     const int32_t* n_active, const smoe_w4_expert* experts,
                                     int T, int k, int H, int I, int E, int group_size,
                                     uint16_t* y_sorted, const uint16_t* shared_w13,
                                     const uint16_t* shared_w2, int shared_I,
                                     uint16_t* shared_h, uint16_t* shared_out, void* workspace,
                                     size_t workspace_bytes, int32_t* err_word, void* stream) {
    const char* name = "w4a16_grouped_ffn_shared";
    smoe_status st = check_wq(name, x, sorted_token, expert_offsets, active, n_active, experts,
                              T, k, H, I, E, 4, group_size, y_sorted);
    if (st != SMOE_OK) return st;
    REQUIRE(shared_w13 && shared_w2 && shared_h && shared_out, SMOE_ERR_NULL,
            "%s: shared_w13, shared_w2, shared_h and shared_out are required", name);
    REQUIRE(shared_I > 0 && shared_I % 128 == 0, SMOE_ERR_SHAPE,
            "%s: shared_I=%d must be a positive multiple of 128", name, shared_I);
    REQUIRE(aligned(shared_w13, 16) && aligned(shared_w2, 16) && aligned(shared_h, 16) &&
                aligned(shared_out, 16),
            SMOE_ERR_SHAPE, "%s: the shared expert's fp16 tensors must be 16-byte aligned", name);
    if (T == 0) return ok();
    const size_t need = smoe::w4a16_workspace_bytes(T, k, H, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", name, need,
            workspace_bytes);
    CHECK_DEVICE();
    return hip_result(smoe::launch_w4a16_ffn_shared(
                          x, sorted_token, expert_offsets, active, n_active, experts, T, k, H, I,
                          E, y_sorted, workspace, shared_w13, shared_w2, shared_I, shared_h,
                          shared_out, err_word, static_cast<hipStream_t>(stream)),
                      "w4a16_grouped_ffn_shared launch");
}

smoe_status moe_draft_route_ffn(const uint16_t* x, const uint16_t* w_router,
                                const uint16_t* w_shared_gate, int H, int I, int E, int k,
                                int renormalize, int layer, int L, int32_t* counters,
                                const smoe_w4_expert* experts, int group_size,
                                int32_t* topk_ids, float* topk_w, float* shared_gate,
                                int32_t* expert_offsets, int32_t* sorted_token,
                                int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                                int32_t* n_active, uint16_t* y_sorted,
                                const uint16_t* shared_w13, const uint16_t* shared_w2,
                                int shared_I, uint16_t* shared_h, uint16_t* shared_out,
                                const float* logits, void* workspace, size_t workspace_bytes,
                                int32_t* err_word, void* stream) {
    REQUIRE(x && w_router && experts && topk_ids && topk_w && expert_offsets && sorted_token &&
                sorted_pair && pair_pos && active && n_active && y_sorted,
            SMOE_ERR_NULL, "moe_draft_route_ffn: a required pointer is NULL");
    REQUIRE(!shared_w13 || (shared_w2 && shared_h && shared_out), SMOE_ERR_NULL,
            "moe_draft_route_ffn: shared_w2, shared_h and shared_out are required with shared_w13");
    REQUIRE(!shared_w13 || (shared_I > 0 && shared_I % 128 == 0 &&
                            shared_I <= kSharedMaxK && H <= kSharedMaxK),
            SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: shared_I=%d must be a positive multiple of 128, and shared_I "
            "and H at most %d", shared_I, kSharedMaxK);
    REQUIRE(!shared_w13 || (aligned(shared_w13, 16) && aligned(shared_w2, 16) &&
                            aligned(shared_h, 16)),
            SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: shared_w13, shared_w2 and shared_h must be 16-byte aligned");
    REQUIRE(!w_shared_gate || shared_gate, SMOE_ERR_NULL,
            "moe_draft_route_ffn: shared_gate output is required with w_shared_gate");
    smoe_status st = check_hek(H, E, k);
    if (st != SMOE_OK) return st;
    REQUIRE(I > 0 && I % 128 == 0, SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: I=%d must be a positive multiple of 128", I);
    REQUIRE(group_size == 128, SMOE_ERR_UNSUPPORTED,
            "moe_draft_route_ffn: group_size=%d (only 128 is supported)", group_size);
    REQUIRE(smoe::w4a16_shape_supported(H, I), SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: H=%d, I=%d (each must be <= 16384)", H, I);
    REQUIRE(smoe::draft_route_ffn_supported(E, k), SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: k=%d exceeds 32", k);
    REQUIRE(!counters || (L >= 1 && layer >= 0 && layer < L), SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: layer=%d must be in [0, L=%d)", layer, L);
    REQUIRE(aligned(x, 16) && aligned(w_router, 16) && aligned(w_shared_gate, 16) &&
                aligned(logits, 4),
            SMOE_ERR_SHAPE,
            "moe_draft_route_ffn: x, w_router, w_shared_gate must be 16-byte aligned (logits 4)");
    const size_t need = smoe::w4a16_workspace_bytes(1, k, H, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "moe_draft_route_ffn: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
            workspace_bytes);
    CHECK_DEVICE();
    return hip_result(
        smoe::launch_draft_route_ffn(x, w_router, w_shared_gate, H, E, k, renormalize ? 1 : 0,
                                     counters ? counters + (size_t)layer * E : nullptr, topk_ids,
                                     topk_w, shared_gate, expert_offsets, sorted_token,
                                     sorted_pair, pair_pos, active, n_active, experts, I,
                                     y_sorted, workspace, shared_w13,
                                     shared_w13 ? shared_w2 : nullptr, shared_w13 ? shared_I : 0,
                                     shared_h, shared_out, logits, err_word,
                                     static_cast<hipStream_t>(stream)),
        "moe_draft_route_ffn launch");
}

int smoe_draft_layer_supported(int H, int I, int E, int k, int shared_I) {
    return smoe::draft_layer_supported(H, I, E, k, shared_I) ? 1 : 0;
}

smoe_status moe_draft_layer(const uint16_t* x, const uint16_t* w_router,
                            const uint16_t* w_shared_gate, const float* logits, int H, int I,
                            int E, int k, int renormalize, int layer, int L, int32_t* counters,
                            const smoe_w4_expert* experts, int group_size, int32_t* topk_ids,
                            float* topk_w, float* shared_gate, int32_t* expert_offsets,
                            int32_t* sorted_token, int32_t* sorted_pair, int32_t* pair_pos,
                            int32_t* active, int32_t* n_active, uint16_t* y_sorted,
                            const uint16_t* shared_w13, const uint16_t* shared_w2, int shared_I,
                            uint16_t* shared_h, uint16_t* shared_out, const uint16_t* residual,
                            uint16_t* out, uint16_t* norm_out, float norm_eps,
                            const uint16_t* next_w_router, const uint16_t* next_w_shared_gate,
                            int next_E, float* next_logits, void* workspace,
                            size_t workspace_bytes, int32_t* err_word, void* stream) {
    REQUIRE(x && w_router && experts && topk_ids && topk_w && expert_offsets && sorted_token &&
                sorted_pair && pair_pos && active && n_active && y_sorted && out,
            SMOE_ERR_NULL, "moe_draft_layer: a required pointer is NULL");
    REQUIRE(!shared_w13 || (shared_w2 && shared_h && shared_out), SMOE_ERR_NULL,
            "moe_draft_layer: shared_w2, shared_h and shared_out are required with shared_w13");
    REQUIRE(!w_shared_gate || shared_gate, SMOE_ERR_NULL,
            "moe_draft_layer: shared_gate output is required with w_shared_gate");
    REQUIRE(!next_w_router || (norm_out && next_logits), SMOE_ERR_NULL,
            "moe_draft_layer: norm_out and next_logits are required with next_w_router");
    smoe_status st = check_hek(H, E, k);
    if (st != SMOE_OK) return st;
    REQUIRE(I > 0 && I % 128 == 0, SMOE_ERR_SHAPE,
            "moe_draft_layer: I=%d must be a positive multiple of 128", I);
    REQUIRE(!shared_w13 || (shared_I > 0 && shared_I % 128 == 0), SMOE_ERR_SHAPE,
            "moe_draft_layer: shared_I=%d must be a positive multiple of 128", shared_I);
    REQUIRE(!next_w_router || (next_E >= 1 && next_E <= 256), SMOE_ERR_SHAPE,
            "moe_draft_layer: next_E=%d must be in [1, 256]", next_E);
    REQUIRE(group_size == 128, SMOE_ERR_UNSUPPORTED,
            "moe_draft_layer: group_size=%d (only 128 is supported)", group_size);
    REQUIRE(!counters || (L >= 1 && layer >= 0 && layer < L), SMOE_ERR_SHAPE,
            "moe_draft_layer: layer=%d must be in [0, L=%d)", layer, L);
    REQUIRE(norm_eps >= 0.0f && (!norm_out || norm_out != out), SMOE_ERR_SHAPE,
            "moe_draft_layer: norm_eps must be >= 0 and norm_out must not alias out");
    REQUIRE(aligned(x, 16) && aligned(w_router, 16) && aligned(w_shared_gate, 16) &&
                aligned(logits, 4) && aligned(y_sorted, 16) && aligned(shared_w13, 16) &&
                aligned(shared_w2, 16) && aligned(shared_h, 16) && aligned(shared_out, 16) &&
                aligned(residual, 16) && aligned(out, 16) && aligned(norm_out, 16) &&
                aligned(next_w_router, 16) && aligned(next_w_shared_gate, 16) &&
                aligned(next_logits, 4),
            SMOE_ERR_SHAPE, "moe_draft_layer: fp16 tensors must be 16-byte aligned (fp32 4)");
    const size_t need = smoe::draft_layer_workspace_bytes(k, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "moe_draft_layer: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
            workspace_bytes);
    CHECK_DEVICE();
    REQUIRE(smoe::draft_layer_supported(H, I, E, k, shared_w13 ? shared_I : 0),
            SMOE_ERR_UNSUPPORTED,
            "moe_draft_layer: no one-launch geometry for H=%d I=%d E=%d k=%d shared_I=%d", H, I,
            E, k, shared_w13 ? shared_I : 0);
    smoe::DraftLayerCall c{};
    c.x = x;
    c.wr = w_router;
    c.wsg = w_shared_gate;
    c.logits = logits;
    c.H = H;
    c.I = I;
    c.E = E;
    c.k = k;
    c.renorm = renormalize ? 1 : 0;
    c.counters_row = counters ? counters + (size_t)layer * E : nullptr;
    c.ids = topk_ids;
    c.w = topk_w;
    c.gate = shared_gate;
    c.off = expert_offsets;
    c.st = sorted_token;
    c.sp = sorted_pair;
    c.pp = pair_pos;
    c.active = active;
    c.n_active = n_active;
    c.experts = experts;
    c.y = y_sorted;
    c.sw13 = shared_w13;
    c.sw2 = shared_w2;
    c.Is = shared_w13 ? shared_I : 0;
    c.sh_h = shared_h;
    c.sh_out = shared_out;
    c.resid = residual;
    c.out = out;
    c.norm_out = norm_out;
    c.eps = norm_eps;
    c.wr_next = next_w_router;
    c.wsg_next = next_w_shared_gate;
    c.E_next = next_E;
    c.lg_next = next_logits;
    c.ws = workspace;
    c.err = err_word;
    return hip_result(smoe::launch_draft_layer(c, static_cast<hipStream_t>(stream)),
                      "moe_draft_layer launch");
}

smoe_status moe_combine_route_logits(const uint16_t* y_sorted, const int32_t* pair_pos,
                                     const float* topk_w, const uint16_t* shared_out,
                                     const float* shared_scale, const uint16_t* residual, int k,
                                     int H, uint16_t* out, uint16_t* norm_out, float norm_eps,
                                     const uint16_t* w_router, const uint16_t* w_shared_gate,
                                     int E, float* logits, void* stream) {
    REQUIRE(y_sorted && pair_pos && topk_w && out && norm_out && w_router && logits,
            SMOE_ERR_NULL,
            "moe_combine_route_logits: y_sorted, pair_pos, topk_w, out, norm_out, w_router and "
            "logits are required");
    REQUIRE(k >= 1 && k <= 256, SMOE_ERR_SHAPE, "moe_combine_route_logits: k=%d must be in [1, 256]",
            k);
    REQUIRE(E >= 1 && E <= 256, SMOE_ERR_SHAPE, "moe_combine_route_logits: E=%d must be in [1, 256]",
            E);
    REQUIRE(H > 0 && H % 128 == 0 && smoe::combine_logits_supported(H), SMOE_ERR_SHAPE,
            "moe_combine_route_logits: H=%d must be a multiple of 128 and at most 8192", H);
    REQUIRE(aligned(y_sorted, 16) && aligned(shared_out, 16) && aligned(residual, 16) &&
                aligned(out, 16) && aligned(norm_out, 16) && aligned(w_router, 16) &&
                aligned(w_shared_gate, 16),
            SMOE_ERR_SHAPE, "moe_combine_route_logits: fp16 tensors must be 16-byte aligned");
    REQUIRE(norm_eps >= 0.0f && norm_out != out, SMOE_ERR_SHAPE,
            "moe_combine_route_logits: norm_eps must be >= 0 and norm_out must not alias out");
    CHECK_DEVICE();
    return hip_result(smoe::launch_combine_logits(y_sorted, pair_pos, topk_w, shared_out,
                                                  shared_scale, residual, k, H, out, norm_out,
                                                  norm_eps, w_router, w_shared_gate, E, logits,
                                                  static_cast<hipStream_t>(stream)),
                      "moe_combine_route_logits launch");
}

smoe_status verify_grouped_gemm(const uint16_t* x, const int32_t* sorted_token,
                                const int32_t* expert_offsets, const int32_t* active,
                                const int32_t* n_active, const smoe_f16_expert* experts,
                                const uint8_t* expert_mask, int T, int rows, int H, int I, int E,
                                uint16_t* y_sorted, void* workspace, size_t workspace_bytes,
                                int32_t* err_word, void* stream) {
    REQUIRE(x && sorted_token && expert_offsets && experts && y_sorted, SMOE_ERR_NULL,
            "verify_grouped_gemm: a required pointer is NULL");
    REQUIRE((active == nullptr) == (n_active == nullptr), SMOE_ERR_NULL,
            "verify_grouped_gemm: pass both active and n_active, or neither");
    REQUIRE(T >= 0 && rows >= 0, SMOE_ERR_SHAPE, "verify_grouped_gemm: T=%d, rows=%d", T, rows);
    REQUIRE(H > 0 && H % 128 == 0 && I > 0 && I % 128 == 0, SMOE_ERR_SHAPE,
            "verify_grouped_gemm: H=%d and I=%d must be positive multiples of 128", H, I);
    REQUIRE(E >= 1 && E <= 256, SMOE_ERR_SHAPE, "verify_grouped_gemm: E=%d must be in [1, 256]",
            E);
    REQUIRE(rows <= kMaxPairs, SMOE_ERR_SHAPE, "verify_grouped_gemm: rows exceeds 2^20");
    REQUIRE(aligned(x, 16), SMOE_ERR_SHAPE, "verify_grouped_gemm: x must be 16-byte aligned");
    if (rows == 0 || T == 0) return ok();
    const size_t need = smoe::verify_workspace_bytes(T, rows, H, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "verify_grouped_gemm: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
            workspace_bytes);
    CHECK_DEVICE();
    return hip_result(smoe::launch_verify_ffn(x, sorted_token, expert_offsets, active, n_active,
                                              experts, expert_mask, T, rows, H, I, E, y_sorted,
                                              workspace, err_word,
                                              static_cast<hipStream_t>(stream)),
                      "verify_grouped_gemm launch");
}

smoe_status verify_grouped_gemm_shared(const uint16_t* x, const int32_t* sorted_token,
                                       const int32_t* expert_offsets, const int32_t* active,
                                       const int32_t* n_active, const smoe_f16_expert* experts,
                                       const uint8_t* expert_mask, int T, int rows, int H, int I,
                                       int E, uint16_t* y_sorted, const uint16_t* shared_w13,
                                       const uint16_t* shared_w2, int shared_I,
                                       uint16_t* shared_h, uint16_t* shared_out, void* workspace,
                                       size_t workspace_bytes, int32_t* err_word, void* stream) {
    REQUIRE(x && sorted_token && expert_offsets && experts && y_sorted, SMOE_ERR_NULL,
            "verify_grouped_gemm_shared: a required pointer is NULL");
    REQUIRE(shared_w13 && shared_w2 && shared_h && shared_out, SMOE_ERR_NULL,
            "verify_grouped_gemm_shared: shared_w13, shared_w2, shared_h and shared_out are "
            "required");
    REQUIRE((active == nullptr) == (n_active == nullptr), SMOE_ERR_NULL,
            "verify_grouped_gemm_shared: pass both active and n_active, or neither");
    REQUIRE(T >= 0 && rows >= 0, SMOE_ERR_SHAPE, "verify_grouped_gemm_shared: T=%d, rows=%d", T,
            rows);
    REQUIRE(H > 0 && H % 128 == 0 && I > 0 && I % 128 == 0, SMOE_ERR_SHAPE,
            "verify_grouped_gemm_shared: H=%d and I=%d must be positive multiples of 128", H, I);
    REQUIRE(shared_I > 0 && shared_I % 128 == 0, SMOE_ERR_SHAPE,
            "verify_grouped_gemm_shared: shared_I=%d must be a positive multiple of 128",
            shared_I);
    REQUIRE(E >= 1 && E <= 256, SMOE_ERR_SHAPE,
            "verify_grouped_gemm_shared: E=%d must be in [1, 256]", E);
    REQUIRE(rows <= kMaxPairs, SMOE_ERR_SHAPE, "verify_grouped_gemm_shared: rows exceeds 2^20");
    REQUIRE(aligned(x, 16) && aligned(shared_w13, 16) && aligned(shared_w2, 16) &&
                aligned(shared_h, 16) && aligned(shared_out, 16),
            SMOE_ERR_SHAPE, "verify_grouped_gemm_shared: fp16 tensors must be 16-byte aligned");
    if (T == 0) return ok();
    const size_t need = smoe::verify_workspace_bytes(T, rows, H, I, E);
    REQUIRE(workspace && workspace_bytes >= need && aligned(workspace, 256), SMOE_ERR_WORKSPACE,
            "verify_grouped_gemm_shared: workspace needs %zu bytes, 256-byte aligned (got %zu)",
            need, workspace_bytes);
    CHECK_DEVICE();
    return hip_result(smoe::launch_verify_ffn_shared(
                          x, sorted_token, expert_offsets, active, n_active, experts, expert_mask,
                          T, rows, H, I, E, y_sorted, workspace, shared_w13, shared_w2, shared_I,
                          shared_h, shared_out, err_word, static_cast<hipStream_t>(stream)),
                      "verify_grouped_gemm_shared launch");
}

smoe_status moe_combine(const uint16_t* y_sorted, const int32_t* pair_pos, const float* topk_w,
                        const uint16_t* shared_out, const float* shared_scale,
                        const uint16_t* residual, int T, int k, int H, uint16_t* out,
                        uint16_t* norm_out, float norm_eps, void* stream) {
    REQUIRE(y_sorted && pair_pos && topk_w && out, SMOE_ERR_NULL,
            "moe_combine: y_sorted, pair_pos, topk_w and out are required");
    REQUIRE(T >= 0 && T <= 65535, SMOE_ERR_SHAPE, "moe_combine: T=%d must be in [0, 65535]", T);
    REQUIRE(k >= 1 && k <= 256, SMOE_ERR_SHAPE, "moe_combine: k=%d must be in [1, 256]", k);
    REQUIRE(H > 0 && H % 128 == 0, SMOE_ERR_SHAPE, "moe_combine: H=%d must be a multiple of 128",
            H);
    REQUIRE(aligned(y_sorted, 16) && aligned(shared_out, 16) && aligned(residual, 16) &&
                aligned(out, 16) && aligned(norm_out, 16),
            SMOE_ERR_SHAPE, "moe_combine: fp16 tensors must be 16-byte aligned");
    REQUIRE(!norm_out || (norm_eps >= 0.0f && norm_out != out), SMOE_ERR_SHAPE,
            "moe_combine: norm_out needs norm_eps >= 0 and must not alias out");
    if (T == 0) return ok();
    CHECK_DEVICE();
    return hip_result(smoe::launch_combine(y_sorted, pair_pos, topk_w, shared_out, shared_scale,
                                           residual, T, k, H, out, norm_out, norm_eps,
                                           static_cast<hipStream_t>(stream)),
                      "moe_combine launch");
}

smoe_status expert_stage_async(void* dst_device, const void* src_pinned_host, size_t bytes,
                               void* side_stream, void* done_event) {
    REQUIRE(dst_device && src_pinned_host, SMOE_ERR_NULL,
            "expert_stage_async: dst_device and src_pinned_host are required");
    if (bytes == 0) return ok();
    CHECK_DEVICE();
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, src_pinned_host);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();  // clear the query's error state
        return fail(SMOE_ERR_NOT_PINNED,
                    "expert_stage_async: source %p is not page-locked host memory",
                    src_pinned_host);
    }
    hipStream_t s = static_cast<hipStream_t>(side_stream);
    e = hipMemcpyAsync(dst_device, src_pinned_host, bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_result(e, "expert_stage_async: hipMemcpyAsync");
    if (done_event) {
        e = hipEventRecord(static_cast<hipEvent_t>(done_event), s);
        if (e != hipSuccess) return hip_result(e, "expert_stage_async: hipEventRecord");
    }
    return ok();
}

}  // extern "C"
