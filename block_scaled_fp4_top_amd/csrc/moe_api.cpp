// C ABI of the MoE layer: argument validation, workspace planning and the
// launch sequence. Every check runs before the first launch; no call
// allocates memory or synchronises (except moe_check_prepared and
// moe_stage_times, which say so).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"
#include "moe_kernels.h"

using namespace moe;

namespace moe {
hipError_t launch_write_header(const BlobHeader& h, void* dst, hipStream_t s);
}

static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

namespace moe {
// The same error reporting for the other translation units of the library.
int report_error(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace moe

static int hip_fail(hipError_t e, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define HIP_TRY(expr, where)                          \
    do {                                              \
        hipError_t _e = (expr);                       \
        if (_e != hipSuccess) return hip_fail(_e, where); \
    } while (0)

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_dims(const moe_dims* d) {
    if (!d) return fail(MOE_ERR_INVALID, "dims is NULL");
    if (d->E < 1 || d->E > kMaxE) return fail(MOE_ERR_INVALID, "E=%d outside [1, %d]", d->E, kMaxE);
    if (d->H <= 0 || d->I <= 0) return fail(MOE_ERR_INVALID, "H=%d, I=%d must be positive", d->H, d->I);
    if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_RELU2)
        return fail(MOE_ERR_INVALID, "act=%d is not a moe_act", d->act);
    if (d->wfmt != MOE_FMT_NVFP4 && d->wfmt != MOE_FMT_MXFP8 && d->wfmt != MOE_FMT_MXFP4)
        return fail(MOE_ERR_INVALID, "wfmt=%d is not a moe_wfmt", d->wfmt);
    if (d->H % kTileK || d->I % kTileK)
        return fail(MOE_ERR_UNSUPPORTED, "H=%d and I=%d must be multiples of %d", d->H, d->I, kTileK);
    if (d->H > 32768 || d->I > 32768)
        return fail(MOE_ERR_UNSUPPORTED, "H=%d, I=%d above 32768", d->H, d->I);
    return MOE_OK;
}

extern "C" const char* moe_last_error(void) { return g_err.c_str(); }

extern "C" size_t moe_prepared_bytes(const moe_dims* d) {
    if (check_dims(d) != MOE_OK) return 0;
    BlobLayout L;
    make_blob_layout(*d, &L);
    return L.h.total;
}

extern "C" int moe_prepare_weights(const moe_dims* d, const float* w1, const float* w2,
                                   void* prepared, size_t prepared_bytes, hipStream_t stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (!w1 || !w2 || !prepared) return fail(MOE_ERR_INVALID, "NULL weight or prepared pointer");
    if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MOE_ERR_INVALID, "w1/w2 must be 16-byte aligned");
    if (!aligned(prepared, 256)) return fail(MOE_ERR_INVALID, "prepared must be 256-byte aligned");
    BlobLayout L;
    make_blob_layout(*d, &L);
    if (prepared_bytes < L.h.total)
        return fail(MOE_ERR_WORKSPACE, "prepared buffer %zu bytes < %llu needed", prepared_bytes,
                    (unsigned long long)L.h.total);
    uint8_t* b = static_cast<uint8_t*>(prepared);
    const int E = d->E, H = d->H, I = d->I, N1 = L.h.N1;
    uint32_t* amax = reinterpret_cast<uint32_t*>(b + L.h.off_amax);
    float* g1 = reinterpret_cast<float*>(b + L.h.off_g1);
    float* g2 = reinterpret_cast<float*>(b + L.h.off_g2);
    const int swI = d->act == MOE_ACT_SWIGLU ? I : 0;
    HIP_TRY(launch_write_header(L.h, b, stream), "write header");
    if (d->wfmt == MOE_FMT_NVFP4 || d->wfmt == MOE_FMT_MXFP4) {
        const bool mx4 = d->wfmt == MOE_FMT_MXFP4;
        HIP_TRY(launch_fill_u32(amax, 2 * (size_t)E, 0u, stream), "prepare zero");
        HIP_TRY(launch_prep_amax(w1, E, (size_t)N1 * H, amax, stream), "prepare amax W1");
        HIP_TRY(launch_prep_amax(w2, E, (size_t)H * I, amax + E, stream), "prepare amax W2");
        HIP_TRY((mx4 ? launch_prep_mxfp4 : launch_prep_nvfp4)(w1, E, N1, H, swI, amax, g1, b + L.h.off_w1,
                                                             b + L.h.off_s1, stream),
                "prepare W1");
        HIP_TRY((mx4 ? launch_prep_mxfp4 : launch_prep_nvfp4)(w2, E, H, I, 0, amax + E, g2, b + L.h.off_w2,
                                                             b + L.h.off_s2, stream),
                "prepare W2");
    } else {
        HIP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(g1), (size_t)E, 0x3F800000u, stream), "g1");
        HIP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(g2), (size_t)E, 0x3F800000u, stream), "g2");
        HIP_TRY(launch_prep_mxfp8(w1, E, N1, H, swI, b + L.h.off_w1, b + L.h.off_s1, stream), "prepare W1");
        HIP_TRY(launch_prep_mxfp8(w2, E, H, I, 0, b + L.h.off_w2, b + L.h.off_s2, stream), "prepare W2");
    }
    return MOE_OK;
}

extern "C" int moe_check_prepared(const moe_dims* d, const void* prepared, hipStream_t stream) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (!prepared) return fail(MOE_ERR_INVALID, "prepared is NULL");
    BlobHeader h;
    HIP_TRY(hipMemcpyAsync(&h, prepared, sizeof h, hipMemcpyDeviceToHost, stream), "read header");
    HIP_TRY(hipStreamSynchronize(stream), "sync");
    BlobLayout L;
    make_blob_layout(*d, &L);
    if (h.magic0 != kBlobMagic0 || h.magic1 != kBlobMagic1) return fail(MOE_ERR_INVALID, "bad blob magic");
    if (h.version != kBlobVersion) return fail(MOE_ERR_INVALID, "blob version %u != %u", h.version, kBlobVersion);
    if (memcmp(&h, &L.h, sizeof h) != 0) return fail(MOE_ERR_INVALID, "blob header does not match dims");
    return MOE_OK;
}

static int check_mode(const moe_dims* d, int32_t T, int32_t K, int32_t mode) {
    if (mode < MOE_W4A4_TENSOR || mode > MOE_W4A4_TOKEN_MXFP4)
        return fail(MOE_ERR_INVALID, "mode=%d is not a moe_mode", mode);
    if (T < 1) return fail(MOE_ERR_INVALID, "T=%d must be >= 1", T);
    if (K < 1 || K > d->E || K > kMaxK) return fail(MOE_ERR_INVALID, "K=%d outside [1, min(E=%d, %d)]", K, d->E, kMaxK);
    if ((long long)T * K > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "T*K=%lld too large", (long long)T * K);
    // the GEMMs address their activation rows with 32-bit byte offsets
    const long long widest = d->H > d->I ? d->H : d->I;
    if ((long long)T * K * widest * 2 >= (1LL << 32))
        return fail(MOE_ERR_UNSUPPORTED, "T*K*max(H, I)*2 = %lld bytes of activations: 4 GiB or more",
                    (long long)T * K * widest * 2);
    const int want = mode == MOE_MXFP8 ? MOE_FMT_MXFP8
                     : (mode == MOE_W4A4_TOKEN_MXFP4 ? MOE_FMT_MXFP4 : MOE_FMT_NVFP4);
    if (d->wfmt != want)
        return fail(MOE_ERR_INVALID, "mode %d needs a %s weight blob", mode,
                    want == MOE_FMT_MXFP8 ? "MXFP8" : (want == MOE_FMT_MXFP4 ? "MXFP4" : "NVFP4"));
    return MOE_OK;
}

extern "C" size_t moe_workspace_bytes(const moe_dims* d, int32_t T_max, int32_t K, int32_t mode) {
    if (check_dims(d) != MOE_OK || check_mode(d, T_max, K, mode) != MOE_OK) return 0;
    WsPlan p;
    plan_workspace(*d, T_max, K, mode, &p);
    return p.total;
}

extern "C" int moe_workspace_view(const moe_dims* d, int32_t T, int32_t K, int32_t mode,
                                  int32_t view_id, size_t* offset, size_t* bytes) {
    int rc = check_dims(d);
    if (rc) return rc;
    rc = check_mode(d, T, K, mode);
    if (rc) return rc;
    if (!offset || !bytes) return fail(MOE_ERR_INVALID, "NULL output pointer");
    if (view_id < 0 || view_id >= V_NUM_PUBLIC) return fail(MOE_ERR_INVALID, "view %d unknown", view_id);
    WsPlan p;
    plan_workspace(*d, T, K, mode, &p);
    if (p.bytes[view_id] == 0) return fail(MOE_ERR_INVALID, "view %d not produced in mode %d", view_id, mode);
    *offset = p.off[view_id];
    *bytes = p.bytes[view_id];
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// optional stage timing
// ---------------------------------------------------------------------------
namespace {
constexpr int kStages = 7;
constexpr int kRing = 128;
// All timer state is touched only with `mu` held: a forward holds it from its
// first to its last event while timing is on (so forwards on several host
// threads serialise then), moe_stage_times while it drains.
struct StageTimer {
    std::mutex mu;
    std::atomic<bool> enabled{false};
    bool init = false;
    hipEvent_t ev[kRing][kStages + 1];
    bool used[kRing][kStages + 1];
    int head = 0, pending = 0;
    double sum_ms[kStages] = {0};
    int forwards = 0;
};
StageTimer g_timer;

void timer_drain_one(int slot) {
    StageTimer& T = g_timer;
    int last = kStages;
    while (last > 0 && !T.used[slot][last]) --last;
    (void)hipEventSynchronize(T.ev[slot][last]);
    int prev = -1;
    for (int s = 0; s <= kStages; ++s) {
        if (!T.used[slot][s]) continue;
        if (prev >= 0) {
            float ms = 0;
            if (hipEventElapsedTime(&ms, T.ev[slot][prev], T.ev[slot][s]) == hipSuccess)
                T.sum_ms[prev] += ms;
        }
        prev = s;
    }
    T.forwards++;
}

// Takes a ring slot for one forward (the caller holds mu and timing is on).
int timer_begin() {
    StageTimer& T = g_timer;
    if (!T.init) {
        for (int i = 0; i < kRing; ++i)
            for (int j = 0; j <= kStages; ++j) (void)hipEventCreate(&T.ev[i][j]);
        T.init = true;
    }
    if (T.pending == kRing) {  // ring full: account the oldest forward (waits for its events)
        timer_drain_one((T.head - T.pending + kRing) % kRing);
        T.pending--;
    }
    const int slot = T.head;
    T.head = (T.head + 1) % kRing;
    T.pending++;
    for (int j = 0; j <= kStages; ++j) T.used[slot][j] = false;
    return slot;
}

// Events recorded by a kernel launch itself (its start and end) for the
// boundaries `stage` and `stage + 1`; null when the forward is not timed
// (slot < 0).
void timer_kernel_events(int slot, int stage, hipEvent_t* t0, hipEvent_t* t1) {
    StageTimer& T = g_timer;
    *t0 = *t1 = nullptr;
    if (slot < 0) return;
    *t0 = T.ev[slot][stage];
    *t1 = T.ev[slot][stage + 1];
    T.used[slot][stage] = T.used[slot][stage + 1] = true;
}

void timer_mark(int slot, int stage, hipStream_t s) {
    StageTimer& T = g_timer;
    if (slot < 0) return;
    (void)hipEventRecord(T.ev[slot][stage], s);
    T.used[slot][stage] = true;
}
}  // namespace

extern "C" int moe_stage_timing(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    g_timer.enabled.store(enable != 0);
    return MOE_OK;
}

extern "C" int moe_stage_times(float* ms, int32_t n, int32_t* forwards) {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    StageTimer& T = g_timer;
    while (T.pending > 0) {
        timer_drain_one((T.head - T.pending + kRing) % kRing);
        T.pending--;
    }
    for (int i = 0; i < n && i < kStages; ++i) ms[i] = (float)T.sum_ms[i];
    if (forwards) *forwards = T.forwards;
    for (int i = 0; i < kStages; ++i) T.sum_ms[i] = 0;
    T.forwards = 0;
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
static int pick_bm_index(long long R, int E) {
    const long long avg = (R + E - 1) / E;
    if (avg <= 16) return 0;
    if (avg <= 32) return 1;
    if (avg <= 64) return 2;
    return 3;
}

// Every check of a forward's arguments except the workspace's (all before any
// launch).
static int check_forward_args(const moe_dims* d, const void* prepared, size_t prepared_bytes,
                              const uint16_t* x, const float* logits, int32_t T, int32_t K,
                              int32_t mode, int32_t act, int32_t router_weight_on_input,
                              int32_t deterministic_finalize, const uint16_t* y) {
    int rc = check_dims(d);
    if (rc) return rc;
    rc = check_mode(d, T, K, mode);
    if (rc) return rc;
    if (act != d->act) return fail(MOE_ERR_INVALID, "act=%d differs from the prepared act=%d", act, d->act);
    if (!prepared || !x || !logits || !y) return fail(MOE_ERR_INVALID, "NULL pointer argument");
    BlobLayout L0;
    make_blob_layout(*d, &L0);
    if (prepared_bytes < L0.h.total)
        return fail(MOE_ERR_WORKSPACE, "prepared blob %zu bytes < %llu for these dimensions",
                    prepared_bytes, (unsigned long long)L0.h.total);
    if (!aligned(prepared, 256)) return fail(MOE_ERR_INVALID, "prepared must be 256-byte aligned");
    if (!aligned(x, 16) || !aligned(logits, 16) || !aligned(y, 16))
        return fail(MOE_ERR_INVALID, "x, logits and y must be 16-byte aligned");
    if (router_weight_on_input != 0 && router_weight_on_input != 1)
        return fail(MOE_ERR_INVALID, "router_weight_on_input must be 0 or 1");
    if (deterministic_finalize != 0 && deterministic_finalize != 1)
        return fail(MOE_ERR_INVALID, "deterministic_finalize must be 0 or 1");
    return MOE_OK;
}

namespace moe {
// Bytes of workspace a forward of this shape uses (arguments already checked).
size_t forward_workspace_bytes(const moe_dims* d, int32_t T, int32_t K, int32_t mode) {
    WsPlan P;
    plan_workspace(*d, T, K, mode, &P);
    return P.total;
}

int forward_checked(const moe_dims* d, const void* prepared, size_t prepared_bytes,
                    const uint16_t* x, const float* logits, int32_t T, int32_t K, int32_t mode,
                    int32_t act, int32_t router_weight_on_input, int32_t deterministic_finalize,
                    const uint16_t* y) {
    return check_forward_args(d, prepared, prepared_bytes, x, logits, T, K, mode, act,
                              router_weight_on_input, deterministic_finalize, y);
}
int enqueue_forward(const moe_dims* d, const void* prepared, const uint16_t* x,
                    const float* logits, int32_t T, int32_t K, int32_t mode, int32_t act,
                    int32_t router_weight_on_input, int32_t deterministic_finalize,
                    void* workspace, uint16_t* y, hipStream_t stream);
}  // namespace moe

extern "C" int moe_forward(const moe_dims* d, const void* prepared, size_t prepared_bytes,
                           const uint16_t* x, const float* logits, int32_t T, int32_t K,
                           int32_t mode, int32_t act, int32_t router_weight_on_input,
                           int32_t deterministic_finalize, void* workspace,
                           size_t workspace_bytes, uint16_t* y, hipStream_t stream) {
    int rc = check_forward_args(d, prepared, prepared_bytes, x, logits, T, K, mode, act,
                                router_weight_on_input, deterministic_finalize, y);
    if (rc) return rc;
    if (!workspace) return fail(MOE_ERR_INVALID, "NULL workspace");
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID, "workspace must be 256-byte aligned");
    const size_t need = forward_workspace_bytes(d, T, K, mode);
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    return enqueue_forward(d, prepared, x, logits, T, K, mode, act, router_weight_on_input,
                           deterministic_finalize, workspace, y, stream);
}

// The launch sequence of one forward; every argument has been checked and
// `workspace` holds at least forward_workspace_bytes(d, T, K, mode) bytes.
int moe::enqueue_forward(const moe_dims* d, const void* prepared, const uint16_t* x,
                         const float* logits, int32_t T, int32_t K, int32_t mode, int32_t act,
                         int32_t router_weight_on_input, int32_t deterministic_finalize,
                         void* workspace, uint16_t* y, hipStream_t stream) {
    WsPlan P;
    plan_workspace(*d, T, K, mode, &P);

    BlobLayout L;
    make_blob_layout(*d, &L);
    const uint8_t* blob = static_cast<const uint8_t*>(prepared);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
#define WS(T_, v) reinterpret_cast<T_*>(ws + P.off[v])
    const int E = d->E, H = d->H, I = d->I, N1 = L.h.N1, R = T * K;
    int32_t* ids = WS(int32_t, V_IDS);
    float* topw = WS(float, V_TOPW);
    int32_t* counts = WS(int32_t, V_COUNTS);
    int32_t* offsets = WS(int32_t, V_OFFSETS);
    int32_t* r2r = WS(int32_t, V_R2R);
    int32_t* rt2row = WS(int32_t, V_RT2ROW);
    int32_t* tiles = WS(int32_t, V_TILES);
    int32_t* bhist = WS(int32_t, V_BHIST);
    int32_t* bbase = bhist + (size_t)P.nblk * E;
    uint32_t* misc = WS(uint32_t, V_MISC);
    const bool mx4 = mode == MOE_W4A4_TOKEN_MXFP4;  // NVFP4 re-blocked to MXFP4 for the GEMMs
    const bool nv4 = mode == MOE_W4A4_TENSOR || mode == MOE_W4A4_TOKEN || mode == MOE_W4A4_TOKEN_4O6 || mx4;
    const bool f8 = mode == MOE_MXFP8;
    const bool per_row = mode == MOE_W4A4_TOKEN || mode == MOE_W4A4_TOKEN_4O6 || mx4;
    const int qkind = mode == MOE_W4A4_TOKEN_4O6 ? QK_NV_ROW_4O6 : (per_row ? QK_NV_ROW : QK_NV_TENSOR);
    const bool fused = deterministic_finalize == 0;
    uint32_t* status = reinterpret_cast<uint32_t*>(ws);

    const int bmi = pick_bm_index(R, E);
    const int BM = bm_of(bmi);
    const int mt_max = (R + BM - 1) / BM + E;
    const int32_t* tl = tiles + (size_t)bmi * (E + 1);
    const int ab = mx4 ? AB_FP4 : (nv4 ? AB_F16_NV : (f8 ? AB_FP8 : AB_BF16_NV));

    GemmArgs g1;
    memset(&g1, 0, sizeof g1);
    g1.a = mx4 ? (const void*)WS(uint8_t, V_XMXCODES)
               : (nv4 ? (const void*)WS(uint16_t, V_XDEQ) : (f8 ? (const void*)WS(uint8_t, V_XCODES) : (const void*)x));
    g1.a_scales = mx4 ? WS(uint8_t, V_XMXSCALES) : (f8 ? WS(uint8_t, V_XSCALES) : nullptr);
    g1.a_g = nv4 ? WS(float, V_XG) : nullptr;
    g1.a_g_per_row = per_row;
    g1.gather = 1;
    g1.row_to_route = r2r;
    g1.topk = K;
    g1.b_codes = blob + L.h.off_w1;
    g1.b_scales = blob + L.h.off_s1;
    g1.b_g = f8 ? nullptr : reinterpret_cast<const float*>(blob + L.h.off_g1);
    g1.N = N1;
    g1.Kdim = H;
    g1.offsets = offsets;
    g1.tiles = tl;
    g1.E = E;
    g1.mt_max = mt_max;
    g1.act = act;
    g1.on_input = router_weight_on_input;
    g1.I = I;
    g1.topw = topw;
    if (nv4) {
        g1.out_f32 = WS(float, V_A2F);
    } else if (f8) {
        g1.a2_codes = WS(uint8_t, V_A2CODES);
        g1.a2_scales = WS(uint8_t, V_A2SCALES);
    } else {
        g1.out_bf16 = WS(uint16_t, V_A2F);
    }
    g1.amax_slot = mode == MOE_W4A4_TENSOR ? misc + kMiscA2Amax : nullptr;
    g1.status = status;

    GemmArgs g2;
    memset(&g2, 0, sizeof g2);
    g2.a = mx4 ? (const void*)WS(uint8_t, V_A2MXCODES)
               : (nv4 ? (const void*)WS(uint16_t, V_A2DEQ)
                      : (f8 ? (const void*)WS(uint8_t, V_A2CODES) : (const void*)WS(uint16_t, V_A2F)));
    g2.a_scales = mx4 ? WS(uint8_t, V_A2MXSCALES) : (f8 ? WS(uint8_t, V_A2SCALES) : nullptr);
    g2.a_g = nv4 ? WS(float, V_A2G) : nullptr;
    g2.a_g_per_row = per_row;
    g2.gather = 0;
    g2.row_to_route = r2r;
    g2.topk = K;
    g2.b_codes = blob + L.h.off_w2;
    g2.b_scales = blob + L.h.off_s2;
    g2.b_g = f8 ? nullptr : reinterpret_cast<const float*>(blob + L.h.off_g2);
    g2.N = H;
    g2.Kdim = I;
    g2.offsets = offsets;
    g2.tiles = tl;
    g2.E = E;
    g2.mt_max = mt_max;
    g2.act = act;
    g2.on_input = router_weight_on_input;
    g2.I = I;
    g2.topw = topw;
    g2.out_f32 = WS(float, V_O);
    g2.fused = fused ? FUSE_ARRIVE : FUSE_NONE;
    g2.arrive = WS(uint32_t, V_ARRIVE);
    g2.rt2row = rt2row;
    g2.y = y;
    g2.status = status;

    // while stage timing is on, the timer state belongs to this forward
    std::unique_lock<std::mutex> timing_lock(g_timer.mu, std::defer_lock);
    if (g_timer.enabled.load()) timing_lock.lock();
    const int tslot = timing_lock.owns_lock() && g_timer.enabled.load() ? timer_begin() : -1;
    hipEvent_t t0, t1;
    timer_mark(tslot, 0, stream);

    HIP_TRY(launch_route(logits, T, E, K, ids, topw, misc, blob, L.h, status, stream), "route");
    timer_mark(tslot, 1, stream);
    if (small_route_permute(R, E)) {
        HIP_TRY(launch_permute_small(ids, R, E, counts, offsets, tiles, r2r, rt2row, stream), "permute");
    } else {
        HIP_TRY(launch_permute(ids, R, E, P.nblk, bhist, bbase, counts, offsets, tiles, r2r, rt2row,
                               stream),
                "permute");
    }
    timer_mark(tslot, 2, stream);
    if (nv4) {
        if (!per_row)
            HIP_TRY(launch_amax(x, 1, (size_t)T * H, misc + kMiscXAmax, kAmaxSlots, kAmaxStride, stream),
                    "x amax");
        HIP_TRY(launch_quant_rows(x, 1, T, H, qkind, misc + kMiscXAmax, kAmaxSlots, kAmaxStride,
                                  WS(uint8_t, V_XCODES), WS(uint8_t, V_XSCALES), WS(float, V_XG),
                                  mx4 ? nullptr : WS(uint16_t, V_XDEQ), stream),
                "quantize x");
        if (mx4)
            HIP_TRY(launch_reblock_mxfp4(WS(uint8_t, V_XCODES), WS(uint8_t, V_XSCALES), (size_t)T * H,
                                         WS(uint8_t, V_XMXCODES), WS(uint8_t, V_XMXSCALES), nullptr, stream),
                    "re-block x");
    } else if (f8) {
        HIP_TRY(launch_quant_rows(x, 1, T, H, QK_MX, nullptr, 0, 0, WS(uint8_t, V_XCODES),
                                  WS(uint8_t, V_XSCALES), nullptr, nullptr, stream),
                "quantize x");
    }

    timer_kernel_events(tslot, 3, &t0, &t1);
    HIP_TRY(launch_gemm(ab, EPI_FC1, bmi, g1, stream, t0, t1), "FC1");

    if (nv4) {
        HIP_TRY(launch_quant_rows(WS(float, V_A2F), 0, R, I, qkind,
                                  misc + kMiscA2Amax, kAmaxSlots, kAmaxStride, WS(uint8_t, V_A2CODES), WS(uint8_t, V_A2SCALES),
                                  WS(float, V_A2G), mx4 ? nullptr : WS(uint16_t, V_A2DEQ), stream),
                "quantize FC2 input");
        if (mx4)
            HIP_TRY(launch_reblock_mxfp4(WS(uint8_t, V_A2CODES), WS(uint8_t, V_A2SCALES), (size_t)R * I,
                                         WS(uint8_t, V_A2MXCODES), WS(uint8_t, V_A2MXSCALES), status, stream),
                    "re-block FC2 input");
    }

    if (fused)
        HIP_TRY(launch_fill_u32(WS(uint32_t, V_ARRIVE), (size_t)T * (H / 128), 0u, stream), "zero arrival counters");
    timer_kernel_events(tslot, 5, &t0, &t1);
    HIP_TRY(launch_gemm(ab, EPI_FC2, bmi, g2, stream, t0, t1), "FC2");

    if (!fused) {
        HIP_TRY(launch_finalize(WS(float, V_O), 0, rt2row, router_weight_on_input ? nullptr : topw, T, K, H,
                                y, status, stream),
                "finalize");
    }
    timer_mark(tslot, 7, stream);
#undef WS
    return MOE_OK;
}

extern "C" int moe_forward_status(const void* workspace, int32_t* status, hipStream_t stream) {
    if (!workspace || !status) return fail(MOE_ERR_INVALID, "NULL pointer argument");
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID, "workspace must be 256-byte aligned");
    uint32_t w = 0;
    HIP_TRY(hipMemcpyAsync(&w, workspace, sizeof w, hipMemcpyDeviceToHost, stream), "read status");
    HIP_TRY(hipStreamSynchronize(stream), "sync");
    *status = (int32_t)w;
    return MOE_OK;
}

extern "C" int moe_finalize(const void* permuted_out, int32_t out_is_bf16, const int32_t* route_to_row,
                            const float* weights, int32_t T, int32_t K, int32_t H, uint16_t* y,
                            hipStream_t stream) {
    if (!permuted_out || !route_to_row || !y) return fail(MOE_ERR_INVALID, "NULL pointer argument");
    if (T < 1 || K < 1 || K > kMaxK) return fail(MOE_ERR_INVALID, "T=%d, K=%d invalid", T, K);
    if (H <= 0 || H % 4) return fail(MOE_ERR_UNSUPPORTED, "H=%d must be a positive multiple of 4", H);
    if (out_is_bf16 != 0 && out_is_bf16 != 1) return fail(MOE_ERR_INVALID, "out_is_bf16 must be 0 or 1");
    if (!aligned(permuted_out, 16) || !aligned(y, 16) || !aligned(route_to_row, 4) ||
        (weights && !aligned(weights, 4)))
        return fail(MOE_ERR_INVALID, "misaligned pointer");
    HIP_TRY(launch_finalize(permuted_out, out_is_bf16, route_to_row, weights, T, K, H, y, nullptr, stream),
            "finalize");
    return MOE_OK;
}

extern "C" int moe_quantize(const float* v, int32_t rows, int32_t cols, int32_t kind, uint8_t* codes,
                            uint8_t* scales, float* g, void* scratch, hipStream_t stream) {
    if (!v || !codes || !scales || !scratch) return fail(MOE_ERR_INVALID, "NULL pointer argument");
    if (kind < 0 || kind > 3) return fail(MOE_ERR_INVALID, "kind=%d invalid", kind);
    if (kind != 2 && !g) return fail(MOE_ERR_INVALID, "g is NULL for NVFP4");
    if (rows < 1 || cols < 32 || cols % 32) return fail(MOE_ERR_UNSUPPORTED, "rows=%d cols=%d unsupported", rows, cols);
    if (!aligned(v, 16) || !aligned(codes, 16) || !aligned(scratch, 4))
        return fail(MOE_ERR_INVALID, "misaligned pointer");
    uint32_t* slot = static_cast<uint32_t*>(scratch);
    const int qk = kind == 0 ? QK_NV_TENSOR : (kind == 1 ? QK_NV_ROW : (kind == 2 ? QK_MX : QK_NV_ROW_4O6));
    if (qk == QK_NV_TENSOR) {
        HIP_TRY(launch_fill_u32(slot, 1, 0u, stream), "clear scratch");
        HIP_TRY(launch_amax(v, 0, (size_t)rows * cols, slot, 1, 1, stream), "amax");
    }
    HIP_TRY(launch_quant_rows(v, 0, rows, cols, qk, slot, 1, 1, codes, scales, g, nullptr, stream), "quantize");
    return MOE_OK;
}
