// Host side of the C ABI: argument validation (before any HIP call), dtype /
// head-dim dispatch, the per-stream scratch for rotated copies, tables and
// live-tile lists, the ring-share plan and its executor.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.h"

using namespace bosa;

namespace {

thread_local std::string g_err;

// Launch timing (attn_profile_start / attn_profile_stop).
struct Profile {
    bool on = false;
    int cap = 0, n = 0;
    std::vector<hipEvent_t> ev;   // 2 per launch
};
thread_local Profile g_prof;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kTile = 64;   // key tile of the bf16 kernel (live-tile list granularity)
constexpr int kChainRows = 256;   // query rows per workgroup of the chained bf16 kernel

// Device scratch of one call.  Outside stream capture it is the calling
// stream's buffer, which the library keeps (one per device and stream) and
// reuses from call to call, growing it when a call needs more.  Freeing device memory at the
// end of every call (hipFreeAsync) waits here for the stream's pending work,
// which made each call synchronous with the one before it.  A call holds the
// buffer's lock while it enqueues, so calls from several host threads on one
// stream take turns: each call's kernels follow the previous call's in the
// stream and never share the buffer with another call's.  Under stream
// capture the scratch is allocated and freed in stream order instead (graph
// allocation nodes), since a captured graph must not keep pointing at a
// buffer that a later, larger call replaces; so it is on the per-thread
// default stream, whose one handle names another stream in every host thread
// and whose thread may end with work still queued on it, so that a buffer
// kept for it could not be handed safely to the next thread.
// attn_release_scratch frees the kept buffers of the current device.
struct ScratchSlot {
    std::mutex m;
    void* ptr = nullptr;
    size_t bytes = 0;
};
using SlotKey = std::pair<int, uintptr_t>;
std::mutex g_slots_m;
// never destroyed: no buffer is freed from a static destructor after the
// HIP runtime has gone
std::map<SlotKey, std::unique_ptr<ScratchSlot>>& scratch_slots() {
    static auto* m = new std::map<SlotKey, std::unique_ptr<ScratchSlot>>();
    return *m;
}
ScratchSlot* scratch_slot(int dev, hipStream_t s) {
    std::lock_guard<std::mutex> g(g_slots_m);
    auto& p = scratch_slots()[SlotKey(dev, reinterpret_cast<uintptr_t>(s))];
    if (!p) p = std::make_unique<ScratchSlot>();
    return p.get();
}
constexpr size_t kScratchGrain = size_t(2) << 20;   // kept buffers grow in 2 MiB steps

struct Scratch {
    void* ptr = nullptr;
    hipStream_t s = nullptr;
    bool owned = false;   // allocated for this call in stream order (capture, per-thread stream)
    std::unique_lock<std::mutex> lk;  // the stream's kept buffer, held while the call enqueues
    ~Scratch() {
        if (owned && ptr) (void)hipFreeAsync(ptr, s);
    }
    hipError_t alloc(size_t bytes, hipStream_t stream) {
        s = stream;
        if (bytes == 0) return hipSuccess;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone || stream == hipStreamPerThread) {
            owned = true;
            return hipMallocAsync(&ptr, bytes, stream);
        }
        int dev = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        ScratchSlot* slot = scratch_slot(dev, stream);
        lk = std::unique_lock<std::mutex>(slot->m);
        if (slot->bytes < bytes) {
            if (slot->ptr) {
                // after the stream's earlier work, which may still use it
                if ((e = hipFreeAsync(slot->ptr, stream)) != hipSuccess) return e;
                slot->ptr = nullptr;
                slot->bytes = 0;
            }
            const size_t want = (bytes + kScratchGrain - 1) / kScratchGrain * kScratchGrain;
            if ((e = hipMallocAsync(&slot->ptr, want, stream)) != hipSuccess) {
                slot->ptr = nullptr;
                return e;
            }
            slot->bytes = want;
        }
        ptr = slot->ptr;
        return hipSuccess;
    }
};

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Positions are limited to |pos| <= 2^52 and lengths to 2^31, so a window
// wider than 2^54 excludes nothing: it is passed on as "no limit" (-1),
// which keeps the kernels' position + window sums far from overflow.
long long window_arg(long long w) { return w > (1LL << 54) ? -1 : w; }

// Whether a (query block, key block) sub-call of a ring share holds any pair
// that causal order and the window allow: the key - query position
// differences of the pair of blocks span [lo, hi]; the allowed ones
// [-window_left, min(0 if causal, window_right)].
bool subcall_live(const attn_ring_call& c, int causal, long long wl, long long wr) {
    const long long lo = c.kv_pos0 - (c.q_pos0 + c.q_rows - 1);
    const long long hi = c.kv_pos0 + c.kv_rows - 1 - c.q_pos0;
    long long amax = hi, amin = lo;
    if (causal) amax = std::min(amax, 0LL);
    if (wr >= 0) amax = std::min(amax, wr);
    if (wl >= 0) amin = std::max(amin, -wl);
    return amin <= amax;
}

// Remove the sub-calls no pair of which the window allows, and renumber the
// write / accumulate order: the first remaining sub-call of a query block
// writes its partial, the later ones merge into it.
void drop_dead_subcalls(std::vector<attn_ring_call>& plan, int causal, long long wl, long long wr) {
    if (wl < 0 && wr < 0) return;
    std::vector<attn_ring_call> live;
    bool touched[2] = {false, false};
    for (const attn_ring_call& c : plan) {
        if (!subcall_live(c, causal, wl, wr)) continue;
        attn_ring_call e = c;
        const int ph = c.q_row0 == 0 ? 0 : 1;
        e.accumulate = touched[ph] ? 1 : 0;
        touched[ph] = true;
        live.push_back(e);
    }
    plan.swap(live);
}

// [0, T) minus the given row ranges, as sorted disjoint ranges.
std::vector<std::pair<int, int>> complement_rows(std::vector<std::pair<int, int>> used, int T) {
    std::sort(used.begin(), used.end());
    std::vector<std::pair<int, int>> out;
    int at = 0;
    for (const auto& r : used) {
        if (r.first > at) out.push_back({at, r.first});
        at = std::max(at, r.first + r.second);
    }
    if (at < T) out.push_back({at, T});
    return out;
}

struct Call {
    const void* q; const void* k; const void* v; void* out; float* lse;
    int B, H, Tq, Tkv, d;
    long long q_off, kv_off;
    int causal;
    const uint8_t* kpm; const uint8_t* amask;
    int dtype; unsigned flags;
    // strides (elements)
    long long q_bstride, kv_bstride, o_bstride, kpm_bstride, lse_bstride;
    int lse_hstride, amask_stride;
    const double2* rope_q; const double2* rope_k;
    long long win_left = -1, win_right = -1;
    const float* alibi = nullptr;
    int paired = 0;            // bf16 kernel: pair light and heavy query units (FwdParams.paired)
};

Call plain_call(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Tq, int Tkv,
                int d, long long q_off, long long kv_off, int causal, const uint8_t* kpm, const uint8_t* amask,
                int dtype, unsigned flags) {
    Call c{};
    c.q = q; c.k = k; c.v = v; c.out = out; c.lse = lse;
    c.B = B; c.H = H; c.Tq = Tq; c.Tkv = Tkv; c.d = d;
    c.q_off = q_off; c.kv_off = kv_off; c.causal = causal;
    c.kpm = kpm; c.amask = amask; c.dtype = dtype; c.flags = flags;
    c.q_bstride = (long long)Tq * H * d;
    c.kv_bstride = (long long)Tkv * H * d;
    c.o_bstride = (long long)Tq * H * d;
    c.kpm_bstride = Tkv;
    c.lse_bstride = (long long)H * Tq;
    c.lse_hstride = Tq;
    c.amask_stride = Tkv;
    return c;
}

size_t kpm_list_bytes(const uint8_t* kpm, int dtype, unsigned flags, int B, int Tkv) {
    if (!kpm || dtype != ATTN_BF16 || (flags & ATTN_NO_TILE_SKIP)) return 0;
    const long long ntk = (Tkv + kTile - 1) / kTile;
    return align_up((size_t)B * (size_t)(ntk + 2) * sizeof(int));
}

size_t kpm_list_bytes(const Call& c) {
    if (!c.kpm || c.dtype != ATTN_BF16 || (c.flags & ATTN_NO_TILE_SKIP)) return 0;
    const long long ntk = (c.Tkv + kTile - 1) / kTile;
    return align_up((size_t)c.B * (size_t)(ntk + 2) * sizeof(int));
}

// Kernel parameters of one validated call (without its live-tile list).
FwdParams fwd_params(const Call& c) {
    FwdParams p{};
    p.q = c.q; p.k = c.k; p.v = c.v; p.out = c.out; p.lse = c.lse;
    p.kpm = c.kpm; p.amask = c.amask;
    p.rope_q = c.rope_q; p.rope_k = c.rope_k;
    p.kpm_list = nullptr;
    p.q_bstride = c.q_bstride; p.kv_bstride = c.kv_bstride; p.o_bstride = c.o_bstride;
    p.kpm_bstride = c.kpm_bstride; p.lse_bstride = c.lse_bstride;
    p.row_stride = c.H * c.d; p.lse_hstride = c.lse_hstride; p.amask_stride = c.amask_stride;
    p.B = c.B; p.H = c.H; p.Tq = c.Tq; p.Tkv = c.Tkv;
    p.q_off = c.q_off; p.kv_off = c.kv_off; p.causal = c.causal ? 1 : 0;
    p.flags = c.flags;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.d));
    p.win_left = c.win_left;
    p.win_right = c.win_right;
    p.alibi = c.alibi;
    p.sqrt_d = (float)std::sqrt((double)c.d);
    return p;
}

// Build the live-tile list of a call's key-padding mask into `list` (scratch
// of kpm_list_bytes(c) bytes).
int build_tile_list(const Call& c, int* list, hipStream_t s) {
    const int ntk = (c.Tkv + kTile - 1) / kTile;
    const hipError_t e = launch_kpm_tiles(c.kpm, c.kpm_bstride, c.B, c.Tkv, kTile, list, ntk + 2, s);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "key-padding tile list launch");
}

// Enqueue one validated call.  `list` is scratch of kpm_list_bytes(c) bytes.
int enqueue(const Call& c, int* list, hipStream_t s) {
    hipError_t e;
    if (c.Tkv == 0) {
        if (c.flags & ATTN_ACCUMULATE) return ATTN_OK;  // merging an empty partial changes nothing
        const bool f32out = c.dtype == ATTN_F32 || (c.flags & ATTN_OUT_F32);
        e = launch_fill_empty(c.out, f32out ? 0 : 1, c.lse, c.B, c.H, c.Tq, c.d, c.o_bstride, c.H * c.d,
                              c.lse_bstride, c.lse_hstride, s);
        return e == hipSuccess ? ATTN_OK : hip_fail(e, "empty-key fill");
    }
    FwdParams p = fwd_params(c);
    p.paired = c.paired;
    if (c.dtype == ATTN_BF16 && list) {
        if (int rc = build_tile_list(c, list, s)) return rc;
        p.kpm_list = list;
        p.kpm_list_stride = (c.Tkv + kTile - 1) / kTile + 2;
    }
    const bool timed = g_prof.on && g_prof.n < g_prof.cap;
    if (timed && (e = hipEventRecord(g_prof.ev[2 * g_prof.n], s)) != hipSuccess) return hip_fail(e, "event record");
    e = c.dtype == ATTN_BF16 ? launch_fwd_bf16(p, c.d, s) : launch_fwd_f32(p, c.d, s);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    if (timed) {
        if ((e = hipEventRecord(g_prof.ev[2 * g_prof.n + 1], s)) != hipSuccess) return hip_fail(e, "event record");
        ++g_prof.n;
    }
    return ATTN_OK;
}

// Run one kernel launch, bracketed by profiling events when profiling is on.
template <typename F>
int timed_launch(F&& launch, const char* what, hipStream_t s) {
    hipError_t e;
    const bool timed = g_prof.on && g_prof.n < g_prof.cap;
    if (timed && (e = hipEventRecord(g_prof.ev[2 * g_prof.n], s)) != hipSuccess) return hip_fail(e, "event record");
    e = launch();
    if (e != hipSuccess) return hip_fail(e, what);
    if (timed) {
        if ((e = hipEventRecord(g_prof.ev[2 * g_prof.n + 1], s)) != hipSuccess) return hip_fail(e, "event record");
        ++g_prof.n;
    }
    return ATTN_OK;
}

// One backward sub-call: q, k (rotated when RoPE is on), v, dout, ld2 and the
// float32 gradients in place, with element strides.
struct BwdCall {
    const void* q; const void* k; const void* v; const void* dout; const float2* ld2;
    float* dq; float* dk; float* dv;
    int B, H, Tq, Tkv, d;
    long long q_off, kv_off;
    int causal;
    const uint8_t* kpm; const uint8_t* amask;
    unsigned flags;            // ATTN_ACCUMULATE here: every gradient adds to what it holds
    long long q_bstride, kv_bstride, kpm_bstride, lse_bstride;
    int lse_hstride, amask_stride;
    long long win_left = -1, win_right = -1;
    const float* alibi = nullptr;
    // ring sub-calls: the first to touch a gradient's rows writes them (the
    // flags without ATTN_ACCUMULATE), later ones add
    int write_dq = 0, write_dkdv = 0;
    // the final bf16 dk, dv of this call's key rows (no other call adds to
    // them), written by the dK/dV kernel instead of dk / dv; dk_rope: the
    // (cos, sin) rows of those keys when dk is to be rotated back
    uint16_t* dk_out = nullptr;
    uint16_t* dv_out = nullptr;
    const double2* dk_rope = nullptr;
};

// Enqueue the dQ and dK/dV kernels of one sub-call; `list` is scratch of
// kpm_list_bytes bytes for the live key tiles of the dQ kernel (or null).
int enqueue_bwd(const BwdCall& c, int* list, hipStream_t s) {
    BwdParams p{};
    p.q = c.q; p.k = c.k; p.v = c.v; p.dout = c.dout; p.ld2 = c.ld2;
    p.dq = c.dq; p.dk = c.dk; p.dv = c.dv;
    p.kpm = c.kpm; p.amask = c.amask; p.kpm_list = nullptr;
    p.q_bstride = c.q_bstride; p.kv_bstride = c.kv_bstride; p.kpm_bstride = c.kpm_bstride;
    p.lse_bstride = c.lse_bstride; p.lse_hstride = c.lse_hstride; p.amask_stride = c.amask_stride;
    p.row_stride = c.H * c.d;
    p.B = c.B; p.H = c.H; p.Tq = c.Tq; p.Tkv = c.Tkv;
    p.q_off = c.q_off; p.kv_off = c.kv_off; p.causal = c.causal ? 1 : 0;
    p.flags = c.flags;
    p.scale = (float)(1.0 / std::sqrt((double)c.d));
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.d));
    p.win_left = c.win_left;
    p.win_right = c.win_right;
    p.alibi = c.alibi;
    p.sqrt_d = (float)std::sqrt((double)c.d);
    p.dk_out = c.dk_out;
    p.dv_out = c.dv_out;
    p.dk_rope = c.dk_rope;
    hipError_t e;
    if (list) {
        const int ntk = (c.Tkv + kTile - 1) / kTile;
        e = launch_kpm_tiles(c.kpm, c.kpm_bstride, c.B, c.Tkv, kTile, list, ntk + 2, s);
        if (e != hipSuccess) return hip_fail(e, "key-padding tile list launch");
        p.kpm_list = list;
        p.kpm_list_stride = ntk + 2;
    }
    p.flags = c.write_dq ? (c.flags & ~(unsigned)ATTN_ACCUMULATE) : c.flags;
    if (int rc = timed_launch([&] { return launch_bwd_dq(p, c.d, s); }, "backward dQ kernel launch", s)) return rc;
    p.flags = c.write_dkdv ? (c.flags & ~(unsigned)ATTN_ACCUMULATE) : c.flags;
    return timed_launch([&] { return launch_bwd_dkdv(p, c.d, s); }, "backward dK/dV kernel launch", s);
}

int check_sizes(int B, int H, int Tq, int Tkv, int d) {
    if (B < 0 || H < 0 || Tq < 0 || Tkv < 0) return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 0 (B=%d H=%d Tq=%d Tkv=%d)", B, H, Tq, Tkv);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d is not supported (64 or 128)", d);
    const long long rs = (long long)H * d;
    if (rs > (1LL << 30)) return fail(ATTN_ERR_UNSUPPORTED, "H*d=%lld too large", rs);
    if ((long long)B * H * (long long)((Tq + 31) / 32) >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
    return ATTN_OK;
}

}  // namespace

// Slots per decoding chunk: enough chunks to fill the chip for any batch
// (about 8192 (row, head, chunk) workgroups), each chunk at least four
// workgroup iterations long.
long long bosa::decode_chunk_size(long long Tcap, long long bh, int d, int is_bf16) {
    const int epl = is_bf16 ? 8 : 4;   // elements per 16-byte load
    const long long gran = (64 / (d / epl)) * kDecodeWaves * kDecodeUnroll;   // keys one iteration covers
    const long long nch = (8192 + bh - 1) / bh;
    long long CH = Tcap > 0 ? (Tcap + nch - 1) / nch : gran;
    CH = (CH + gran - 1) / gran * gran;
    return CH < 4 * gran ? 4 * gran : CH;
}

namespace {

// The bf16 kernel addresses one 64-key tile of a head with 32-bit byte
// offsets: 64 rows of H * d bf16 values must stay below 4 GiB.
int check_bf16_rows(int dtype, int H, int d) {
    if (dtype == ATTN_BF16 && (long long)H * d > (1LL << 25))
        return fail(ATTN_ERR_UNSUPPORTED, "H*d=%lld too large for bf16 (max 2^25)", (long long)H * d);
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err.c_str(); }

int attn_version(void) { return 100; }

int attn_profile_start(int max_launches) {
    g_err.clear();
    if (g_prof.on) return fail(ATTN_ERR_INVALID_ARG, "profiling already started");
    if (max_launches <= 0 || max_launches > (1 << 20)) return fail(ATTN_ERR_INVALID_ARG, "max_launches out of range");
    g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
    for (auto& ev : g_prof.ev) {
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) {
            for (auto& x : g_prof.ev)
                if (x) (void)hipEventDestroy(x);
            g_prof.ev.clear();
            return hip_fail(e, "event create");
        }
    }
    g_prof.cap = max_launches;
    g_prof.n = 0;
    g_prof.on = true;
    return ATTN_OK;
}

int attn_release_scratch(void) {
    g_err.clear();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "device query");
    std::lock_guard<std::mutex> g(g_slots_m);
    bool synced = false;
    for (auto& kv : scratch_slots()) {
        if (kv.first.first != dev) continue;
        ScratchSlot& slot = *kv.second;
        std::lock_guard<std::mutex> l(slot.m);   // no call is enqueuing with it
        if (!slot.ptr) continue;
        if (!synced) {   // the kept buffers' streams may be gone: wait for all work instead
            if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "device synchronisation");
            synced = true;
        }
        if ((e = hipFreeAsync(slot.ptr, nullptr)) != hipSuccess) return hip_fail(e, "scratch release");
        slot.ptr = nullptr;
        slot.bytes = 0;
    }
    return ATTN_OK;
}

int attn_profile_stop(float* ms, int cap) {
    g_err.clear();
    if (!g_prof.on) return -fail(ATTN_ERR_INVALID_ARG, "profiling not started");
    int rc = g_prof.n;
    for (int i = 0; i < g_prof.n && rc >= 0; ++i) {
        hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (e != hipSuccess) rc = -hip_fail(e, "event timing");
        else if (ms && i < cap) ms[i] = t;
    }
    for (auto& x : g_prof.ev) (void)hipEventDestroy(x);
    g_prof = Profile{};
    return rc;
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Tq, int Tkv, int d,
             long long q_off, long long kv_off, int causal, const uint8_t* kpm, const uint8_t* attn_mask,
             double rope_base, int dtype, unsigned flags, attn_stream_t stream) {
    return attn_fwd_ex(q, k, v, out, lse, B, H, Tq, Tkv, d, q_off, kv_off, causal, kpm, attn_mask, rope_base, dtype,
                       flags, nullptr, stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Tq, int Tkv,
                int d, long long q_off, long long kv_off, int causal, const uint8_t* kpm, const uint8_t* attn_mask,
                double rope_base, int dtype, unsigned flags, const attn_variant* var, attn_stream_t stream) {
    g_err.clear();
    if (var && (var->window_left < -1 || var->window_right < -1))
        return fail(ATTN_ERR_INVALID_ARG, "window sizes must be >= -1 (got %lld, %lld)", var->window_left,
                    var->window_right);
    if (int rc = check_sizes(B, H, Tq, Tkv, d)) return rc;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (flags & ~(unsigned)(ATTN_ACCUMULATE | ATTN_OUT_F32 | ATTN_NO_TILE_SKIP))
        return fail(ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
    if ((flags & ATTN_ACCUMULATE) && dtype == ATTN_BF16 && !(flags & ATTN_OUT_F32))
        return fail(ATTN_ERR_INVALID_ARG, "ATTN_ACCUMULATE needs a float32 out (ATTN_OUT_F32)");
    if ((flags & ATTN_ACCUMULATE) && !lse) return fail(ATTN_ERR_INVALID_ARG, "ATTN_ACCUMULATE needs lse");
    if (!(rope_base >= 0.0) || std::isinf(rope_base)) return fail(ATTN_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
    if (B == 0 || H == 0 || Tq == 0) return ATTN_OK;
    if (!q || !out) return fail(ATTN_ERR_INVALID_ARG, "q and out must not be NULL");
    if (Tkv > 0 && (!k || !v)) return fail(ATTN_ERR_INVALID_ARG, "k and v must not be NULL");
    if (!aligned16(q) || !aligned16(out) || (Tkv > 0 && (!aligned16(k) || !aligned16(v))))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (std::llabs(q_off) > (1LL << 52) || std::llabs(kv_off) > (1LL << 52))
        return fail(ATTN_ERR_INVALID_ARG, "positions out of range");

    if (int rc = check_bf16_rows(dtype, H, d)) return rc;

    Call c = plain_call(q, k, v, out, lse, B, H, Tq, Tkv, d, q_off, kv_off, causal, kpm, attn_mask, dtype, flags);
    if (var) {
        c.win_left = window_arg(var->window_left);
        c.win_right = window_arg(var->window_right);
        c.alibi = var->alibi_slopes;
    }
    hipStream_t s = (hipStream_t)stream;
    // bf16 under causal order without a window, all workgroups at once (at
    // most one per CU): pair light and heavy query units, since the heaviest
    // workgroup sets the time.  The CU count is read before anything is enqueued.
    if (dtype == ATTN_BF16 && causal && Tkv > 0 && c.win_left < 0 && c.win_right < 0) {
        int dev = 0, n_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "device query");
        c.paired = (long long)B * H * ((Tq + kChainRows - 1) / kChainRows) <= n_cu ? 1 : 0;
    }
    const bool rope = rope_base > 0.0 && Tkv > 0;
    // bf16: the queries and the keys are rotated once, in one launch that
    // computes its own (cos, sin) values, into scratch copies that the
    // attention kernel reads; float32: the kernel rotates them on the fly from
    // float64 (cos, sin) tables.
    const bool krot = rope && dtype == ATTN_BF16;
    const size_t tab_q = rope && !krot ? align_up((size_t)Tq * (d / 2) * sizeof(double2)) : 0;
    const size_t tab_k = rope && !krot ? align_up((size_t)Tkv * (d / 2) * sizeof(double2)) : 0;
    const size_t kbuf = krot ? align_up((size_t)B * Tkv * H * d * 2) : 0;
    const size_t qbuf = krot ? align_up((size_t)B * Tq * H * d * 2) : 0;
    const size_t lst = kpm_list_bytes(c);
    Scratch ws;
    hipError_t e = ws.alloc(tab_q + tab_k + kbuf + qbuf + lst, s);
    if (e != hipSuccess) return hip_fail(e, "scratch allocation");
    char* wp = (char*)ws.ptr;
    if (krot) {
        void* kr = wp;
        void* qr = wp + kbuf;
        e = launch_rope_rotate_bf16(rope_job(k, kr, B, Tkv, H, d, Tkv, kv_off, 0),
                                    rope_job(q, qr, B, Tq, H, d, Tq, q_off, 0), H, d, std::log(rope_base), s);
        if (e != hipSuccess) return hip_fail(e, "key / query rotation launch");
        c.k = kr;
        c.q = qr;
    } else if (rope) {
        const double lb = std::log(rope_base);
        c.rope_q = (const double2*)wp;
        c.rope_k = (const double2*)(wp + tab_q);
        e = launch_rope_table((double2*)wp, q_off, Tq, d, lb, s);
        if (e == hipSuccess) e = launch_rope_table((double2*)(wp + tab_q), kv_off, Tkv, d, lb, s);
        if (e != hipSuccess) return hip_fail(e, "rotary table launch");
    }
    return enqueue(c, lst ? (int*)(wp + tab_q + tab_k + kbuf + qbuf) : nullptr, s);
}

int attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, int* cache_len, int B, int H,
                   int Tcap, int d, double rope_base, int dtype, attn_stream_t stream) {
    g_err.clear();
    if (B < 0 || H < 0 || Tcap < 0) return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 0");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d is not supported (64 or 128)", d);
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (!(rope_base >= 0.0) || std::isinf(rope_base)) return fail(ATTN_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
    if (B == 0 || H == 0 || Tcap == 0) return ATTN_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !cache_len) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    const uintptr_t al = dtype == ATTN_BF16 ? 3u : 7u;
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_cache | (uintptr_t)v_cache) & al)
        return fail(ATTN_ERR_INVALID_ARG, "tensors must be %d-byte aligned", (int)al + 1);
    if ((long long)B * Tcap * H * d >= (1LL << 47)) return fail(ATTN_ERR_UNSUPPORTED, "cache too large");
    hipError_t e = launch_kv_append(k_new, v_new, k_cache, v_cache, cache_len, B, H, Tcap, d,
                                    rope_base > 0.0 ? std::log(rope_base) : 0.0, dtype == ATTN_BF16,
                                    (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "cache append launch");
}

// attn_decode and attn_decode_noalloc: the same validation and kernels; the
// chunk partials go to stream-ordered scratch, or (static_ws) to the
// library's per-device static workspace.
static int decode_call(const void* q, const void* k_cache, const void* v_cache, const int* cache_len, void* out,
                       float* lse, int B, int H, int Tcap, int d, double rope_base, int dtype, unsigned flags,
                       const attn_variant* var, attn_stream_t stream, bool static_ws) {
    g_err.clear();
    if (B < 0 || H < 0 || Tcap < 0) return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 0");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d is not supported (64 or 128)", d);
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (flags & ~(unsigned)ATTN_OUT_F32) return fail(ATTN_ERR_INVALID_ARG, "only ATTN_OUT_F32 may be passed");
    if (!(rope_base >= 0.0) || std::isinf(rope_base)) return fail(ATTN_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
    if (var && (var->window_left < -1 || var->window_right < -1))
        return fail(ATTN_ERR_INVALID_ARG, "window sizes must be >= -1");
    if (B == 0 || H == 0) return ATTN_OK;
    if (!q || !out || !cache_len || (Tcap > 0 && (!k_cache || !v_cache))) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(q) || (Tcap > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) || ((uintptr_t)out & 3))
        return fail(ATTN_ERR_INVALID_ARG, "q and the caches must be 16-byte aligned, out 4-byte");
    if ((long long)B * Tcap * H * d >= (1LL << 47)) return fail(ATTN_ERR_UNSUPPORTED, "cache too large");
    const bool bf16 = dtype == ATTN_BF16;
    // chunks of CH slots
    const long long bh = (long long)B * H;
    const long long CH = decode_chunk_size(Tcap, bh, d, bf16);
    const long long nch = Tcap > 0 ? (Tcap + CH - 1) / CH : 1;
    if (bh * nch >= (1LL << 31) || CH >= (1LL << 30)) return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
    const size_t po = align_up((size_t)bh * nch * d * sizeof(float));
    const size_t pl = align_up((size_t)bh * nch * sizeof(float));
    if (static_ws && po + pl > kDecodeStaticBytes)
        return fail(ATTN_ERR_UNSUPPORTED,
                    "attn_decode_noalloc: the chunk partials of B*H=%lld rows need %zu bytes, more than the "
                    "%zu-byte static workspace (about B*H <= %lld at d=%d)", bh, po + pl, kDecodeStaticBytes,
                    (long long)(kDecodeStaticBytes / (4 * (size_t)(d + 1))) - 8192, d);
    DecodeParams p{};
    p.q = q; p.k = k_cache; p.v = v_cache; p.cache_len = cache_len; p.out = out; p.lse = lse;
    p.alibi = var ? var->alibi_slopes : nullptr;
    p.B = B; p.H = H; p.Tcap = Tcap; p.CH = (int)CH; p.n_chunks = (int)nch;
    p.win_left = var ? window_arg(var->window_left) : -1;
    p.log_base = rope_base > 0.0 ? std::log(rope_base) : 0.0;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    p.sqrt_d = (float)std::sqrt((double)d);
    hipStream_t s = (hipStream_t)stream;
    Scratch ws;
    void* wsp = nullptr;
    hipError_t e;
    if (static_ws) {
        if ((e = decode_static_workspace(&wsp)) != hipSuccess) return hip_fail(e, "static workspace lookup");
    } else {
        if ((e = ws.alloc(po + pl, s)) != hipSuccess) return hip_fail(e, "scratch allocation");
        wsp = ws.ptr;
    }
    p.part_o = (float*)wsp;
    p.part_lse = (float*)((char*)wsp + po);
    if (Tcap > 0)
        if (int rc = timed_launch([&] { return launch_decode_chunks(p, d, bf16, s); }, "decode kernel launch", s))
            return rc;
    e = launch_decode_merge(p, d, bf16 && !(flags & ATTN_OUT_F32), s);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "decode merge launch");
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cache_len, void* out, float* lse,
                int B, int H, int Tcap, int d, double rope_base, int dtype, unsigned flags, const attn_variant* var,
                attn_stream_t stream) {
    return decode_call(q, k_cache, v_cache, cache_len, out, lse, B, H, Tcap, d, rope_base, dtype, flags, var, stream,
                       false);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* cache_len, void* out,
                        float* lse, int B, int H, int Tcap, int d, double rope_base, int dtype, unsigned flags,
                        const attn_variant* var, attn_stream_t stream) {
    return decode_call(q, k_cache, v_cache, cache_len, out, lse, B, H, Tcap, d, rope_base, dtype, flags, var, stream,
                       true);
}

int attn_merge(float* out_a, float* lse_a, const void* out_b, const float* lse_b, int B, int H, int Tq, int d,
               int b_dtype, attn_stream_t stream) {
    g_err.clear();
    if (B < 0 || H < 0 || Tq < 0) return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 0");
    if (d <= 0 || d % 4) return fail(ATTN_ERR_UNSUPPORTED, "d=%d must be a positive multiple of 4", d);
    if (b_dtype != ATTN_F32 && b_dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", b_dtype);
    if ((long long)B * Tq * H == 0) return ATTN_OK;
    if (!out_a || !lse_a || !out_b || !lse_b) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(out_a) || (b_dtype == ATTN_F32 ? !aligned16(out_b) : ((uintptr_t)out_b & 7)))
        return fail(ATTN_ERR_INVALID_ARG, "out_a must be 16-byte aligned (out_b 16 for float32, 8 for bf16)");
    hipError_t e = launch_merge(out_a, lse_a, out_b, lse_b, B, H, Tq, d, (long long)Tq * H * d, H * d,
                                (long long)H * Tq, Tq, b_dtype == ATTN_BF16, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "merge launch");
}

int rope_apply(void* x, const long long* pos, double base, int B, int T, int H, int d, int dtype, attn_stream_t stream) {
    g_err.clear();
    if (B < 0 || T < 0 || H < 0) return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 0");
    if (d <= 0 || d % 2 || d > 256) return fail(ATTN_ERR_UNSUPPORTED, "d=%d must be even and <= 256", d);
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (!(base > 0.0) || std::isinf(base)) return fail(ATTN_ERR_INVALID_ARG, "base must be finite and > 0");
    if ((long long)B * T * H == 0) return ATTN_OK;
    if (T > 65535 * 1024LL || B > 65535) return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
    if (!x || !pos) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    if ((uintptr_t)x & (dtype == ATTN_BF16 ? 3u : 7u)) return fail(ATTN_ERR_INVALID_ARG, "x misaligned");
    hipError_t e = launch_rope_apply(x, pos, std::log(base), B, T, H, d, dtype == ATTN_BF16, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "rope launch");
}

int attn_cast(const float* src, void* dst, long long n, int dst_dtype, attn_stream_t stream) {
    g_err.clear();
    if (n < 0) return fail(ATTN_ERR_INVALID_ARG, "n must be >= 0");
    if (dst_dtype != ATTN_F32 && dst_dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dst_dtype);
    if (n == 0) return ATTN_OK;
    if (!src || !dst) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(src) || ((uintptr_t)dst & 7)) return fail(ATTN_ERR_INVALID_ARG, "src must be 16-byte and dst 8-byte aligned");
    hipError_t e = launch_cast(src, dst, n, dst_dtype == ATTN_BF16, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "cast launch");
}

int attn_ring_plan(int T, int P, int rank, int zigzag, int causal, attn_ring_call* plan, int cap) {
    g_err.clear();
    if (P <= 0 || rank < 0 || rank >= P || T <= 0) return -fail(ATTN_ERR_INVALID_ARG, "need T > 0, P > 0, 0 <= rank < P");
    const int parts = zigzag ? 2 * P : P;
    if (T % parts) return -fail(ATTN_ERR_INVALID_ARG, "T=%d is not divisible by %d", T, parts);
    if (cap < 0 || (cap > 0 && !plan)) return -fail(ATTN_ERR_INVALID_ARG, "bad plan buffer");
    const int c = T / parts;
    // local query chunks: (chunk index, first local row)
    int qchunk[2] = {rank, 2 * P - 1 - rank};
    const int nq = zigzag ? 2 : 1;
    bool touched[2] = {false, false};
    int n = 0;
    for (int step = 0; step < P; ++step) {
        const int blk = ((rank - step) % P + P) % P;
        int kchunk[2] = {blk, 2 * P - 1 - blk};
        const int nk = zigzag ? 2 : 1;
        for (int qh = 0; qh < nq; ++qh) {
            for (int kh = 0; kh < nk; ++kh) {
                const int qc = qchunk[qh], kc = kchunk[kh];
                if (causal && kc > qc) continue;   // every key after every query
                if (n < cap) {
                    attn_ring_call& e = plan[n];
                    e.step = step;
                    e.block = blk;
                    e.q_row0 = qh * c;
                    e.q_rows = c;
                    e.q_pos0 = (long long)qc * c;
                    e.kv_pos0 = (long long)kc * c;
                    e.kv_rows = c;
                    e.accumulate = touched[qh] ? 1 : 0;
                }
                touched[qh] = true;
                ++n;
            }
        }
    }
    return n;
}

int attn_ring_fwd(const void* q, const void* k, const void* v, void* out, float* lse, float* acc, int B, int H, int T,
                  int d, int P, int rank, int zigzag, int causal, const uint8_t* kpm, double rope_base, int dtype,
                  unsigned flags, attn_stream_t stream) {
    return attn_ring_fwd_ex(q, k, v, out, lse, acc, B, H, T, d, P, rank, zigzag, causal, kpm, rope_base, dtype, flags,
                            nullptr, stream);
}

int attn_ring_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, float* acc, int B, int H,
                     int T, int d, int P, int rank, int zigzag, int causal, const uint8_t* kpm, double rope_base,
                     int dtype, unsigned flags, const attn_variant* var, attn_stream_t stream) {
    g_err.clear();
    if (var && (var->window_left < -1 || var->window_right < -1))
        return fail(ATTN_ERR_INVALID_ARG, "window sizes must be >= -1");
    const long long wl = var ? window_arg(var->window_left) : -1, wr = var ? window_arg(var->window_right) : -1;
    const int n = attn_ring_plan(T, P, rank, zigzag, causal, nullptr, 0);
    if (n < 0) return -n;
    const int Tl = T / P;
    if (int rc = check_sizes(B, H, Tl, T, d)) return rc;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (flags & ~(unsigned)ATTN_NO_TILE_SKIP) return fail(ATTN_ERR_INVALID_ARG, "only ATTN_NO_TILE_SKIP may be passed");
    if (!(rope_base >= 0.0) || std::isinf(rope_base)) return fail(ATTN_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
    if (B == 0 || H == 0) return ATTN_OK;
    if (!q || !k || !v || !out || !lse || !acc) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(acc) || ((uintptr_t)out & 7))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v, acc must be 16-byte aligned, out 8-byte");
    if (int rc = check_bf16_rows(dtype, H, d)) return rc;
    std::vector<attn_ring_call> plan(n);
    attn_ring_plan(T, P, rank, zigzag, causal, plan.data(), n);
    drop_dead_subcalls(plan, causal, wl, wr);
    const int n_live = (int)plan.size();

    hipStream_t s = (hipStream_t)stream;
    const bool rope = rope_base > 0.0;
    // bf16: every key block is rotated once (at its absolute positions) into
    // a scratch copy, as the block's owner would before passing it on, and so
    // are the local queries, which every sub-call reads again (rotating them
    // in each sub-call's kernel would re-read cos/sin values several times the
    // bytes of the queries, once per sub-call); one launch rotates both and
    // computes its own (cos, sin) values.  float32: the kernel rotates on the
    // fly from one table over [0, T) (the local queries' positions are
    // positions of the keys).
    const bool krot = rope && dtype == ATTN_BF16;
    const size_t tab_k = rope && !krot ? align_up((size_t)T * (d / 2) * sizeof(double2)) : 0;
    const size_t kbuf = krot ? align_up((size_t)B * T * H * d * 2) : 0;
    const size_t qbuf = krot ? align_up((size_t)B * Tl * H * d * 2) : 0;
    std::vector<size_t> lst_off(n_live, 0);
    size_t total = tab_k + kbuf + qbuf;
    std::vector<Call> calls(n_live);
    const int rs = H * d;
    const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
    for (int i = 0; i < n_live; ++i) {
        const attn_ring_call& e = plan[i];
        Call c{};
        c.q = (const char*)q + (size_t)e.q_row0 * rs * esz;
        c.k = (const char*)k + (size_t)e.kv_pos0 * rs * esz;
        c.v = (const char*)v + (size_t)e.kv_pos0 * rs * esz;
        c.out = acc + (size_t)e.q_row0 * rs;
        c.lse = lse + e.q_row0;
        c.B = B; c.H = H; c.Tq = e.q_rows; c.Tkv = e.kv_rows; c.d = d;
        c.q_off = e.q_pos0; c.kv_off = e.kv_pos0; c.causal = causal;
        c.kpm = kpm ? kpm + e.kv_pos0 : nullptr;
        c.amask = nullptr;
        c.win_left = wl;
        c.win_right = wr;
        c.alibi = var ? var->alibi_slopes : nullptr;
        c.dtype = dtype;
        c.flags = (flags & ATTN_NO_TILE_SKIP) | ATTN_OUT_F32 | (e.accumulate ? ATTN_ACCUMULATE : 0u);
        c.q_bstride = (long long)Tl * rs;
        c.kv_bstride = (long long)T * rs;
        c.o_bstride = (long long)Tl * rs;
        c.kpm_bstride = T;
        c.lse_bstride = (long long)H * Tl;
        c.lse_hstride = Tl;
        c.amask_stride = 0;
        calls[i] = c;
        lst_off[i] = total;
        total += kpm_list_bytes(c);
    }
    const bool chain = dtype == ATTN_BF16 && wl < 0 && wr < 0 && !(var && var->alibi_slopes);
    // the chained executor's cut rule needs the CU count: queried before anything is enqueued
    int n_cu = 0;
    hipError_t err = hipSuccess;
    if (chain) {
        int dev = 0;
        if ((err = hipGetDevice(&dev)) != hipSuccess ||
            (err = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return hip_fail(err, "device query");
    }
    Scratch ws;
    err = ws.alloc(total, s);
    if (err != hipSuccess) return hip_fail(err, "scratch allocation");
    char* wp = (char*)ws.ptr;
    const double2* tab = (const double2*)wp;
    char* krb = wp + tab_k;
    char* qrb = krb + kbuf;
    if (krot) {
        // keys at their absolute positions; local rows [0, c) sit at rank * c,
        // zigzag rows [c, 2c) at (2P - 1 - rank) * c
        const int parts = zigzag ? 2 : 1;
        const int c = Tl / parts;
        err = launch_rope_rotate_bf16(rope_job(k, krb, B, T, H, d, T, 0, 0),
                                      rope_job(q, qrb, B, Tl, H, d, c, (long long)rank * c,
                                               (long long)(2 * P - 1 - rank) * c),
                                      H, d, std::log(rope_base), s);
        if (err != hipSuccess) return hip_fail(err, "key / query rotation launch");
    } else if (rope) {
        err = launch_rope_table((double2*)wp, 0, T, d, std::log(rope_base), s);
        if (err != hipSuccess) return hip_fail(err, "rotary table launch");
    }
    for (int i = 0; i < n_live; ++i) {
        Call& c = calls[i];
        if (krot) {
            c.k = (const uint16_t*)krb + (size_t)plan[i].kv_pos0 * rs;
            c.q = (const uint16_t*)qrb + (size_t)plan[i].q_row0 * rs;
        } else if (rope) {
            c.rope_q = tab + (size_t)plan[i].q_pos0 * (d / 2);
            c.rope_k = tab + (size_t)plan[i].kv_pos0 * (d / 2);
        }
    }
    bool covered[2] = {false, false};
    // bf16 without a window or ALiBi: a query block's sub-calls run in plan
    // order, several to a launch of the chained kernel, which carries each
    // row's softmax state across the sub-calls of the launch and writes or
    // merges one partial per launch; the query block's last launch writes the
    // final bf16 output itself (no cast pass).  A chain ends after kMaxChain
    // blocks, and after a block that causal order cuts through the query
    // block when the launch runs its workgroups in more than one round per
    // CU: those workgroups finish that block at different times, and a new
    // launch lines them up again, so the workgroups of one head keep reading
    // the same key tiles at about the same time.  With a single round (the 8K
    // share) there is no later round to fall out of step, and going on in the
    // same launch was 4.7% faster there.
    if (chain) {
        for (int i = 0; i < n_live; ++i)
            if (kpm_list_bytes(calls[i]))
                if (int rc = build_tile_list(calls[i], (int*)(wp + lst_off[i]), s)) return rc;
        auto cut = [&](int i) {
            const long long wgs = (long long)B * H * ((plan[i].q_rows + kChainRows - 1) / kChainRows);
            return causal && wgs > n_cu && plan[i].kv_pos0 + plan[i].kv_rows - 1 > plan[i].q_pos0;
        };
        for (int ph = 0; ph < 2; ++ph) {
            std::vector<int> idx;
            for (int i = 0; i < n_live; ++i)
                if ((plan[i].q_row0 == 0 ? 0 : 1) == ph) idx.push_back(i);
            for (size_t j0 = 0, n1 = 0; j0 < idx.size(); j0 += n1) {
                n1 = 0;
                while (j0 + n1 < idx.size() && (int)n1 < kMaxChain) {
                    ++n1;
                    if (cut(idx[j0 + n1 - 1])) break;
                }
                ChainParams cpm{};
                cpm.p = fwd_params(calls[idx[j0]]);
                // all workgroups at once (one per CU): pair light and heavy
                // query units, since the heaviest workgroup sets the time
                const long long wgs = (long long)B * H * ((plan[idx[j0]].q_rows + kChainRows - 1) / kChainRows);
                cpm.p.paired = causal && wgs <= n_cu ? 1 : 0;
                if (j0 + n1 == idx.size())   // the query block's last launch
                    cpm.out_bf16 = (uint16_t*)out + (size_t)plan[idx[j0]].q_row0 * rs;
                cpm.nblk = (int)n1;
                for (int j = 0; j < cpm.nblk; ++j) {
                    const Call& c = calls[idx[j0 + j]];
                    ChainBlock& cb = cpm.blk[j];
                    cb.k = c.k;
                    cb.v = c.v;
                    cb.kpm = c.kpm;
                    cb.kpm_list = kpm_list_bytes(c) ? (const int*)(wp + lst_off[idx[j0 + j]]) : nullptr;
                    cb.kv_off = c.kv_off;
                    cb.Tkv = c.Tkv;
                    cb.accumulate = plan[idx[j0 + j]].accumulate;
                }
                if (int rc = timed_launch([&] { return launch_fwd_bf16_chain(cpm, d, s); },
                                          "attention kernel launch", s))
                    return rc;
            }
            if (!idx.empty()) covered[ph] = true;
        }
    } else {
        for (int i = 0; i < n_live; ++i) {
            const Call& c = calls[i];
            const size_t lb = kpm_list_bytes(c);
            if (int rc = enqueue(c, lb ? (int*)(wp + lst_off[i]) : nullptr, s)) return rc;
            covered[plan[i].q_row0 == 0 ? 0 : 1] = true;
        }
    }
    // rows no sub-call reached (not possible with a causal diagonal, kept for
    // safety): the empty result, in out directly on the chained path (whose
    // launches wrote the rest of out), else in acc before the cast
    const int parts = zigzag ? 2 : 1;
    for (int ph = 0; ph < parts; ++ph) {
        if (covered[ph]) continue;
        const int c = Tl / parts;
        if (chain)
            err = launch_fill_empty((uint16_t*)out + (size_t)ph * c * rs, 1, lse + (size_t)ph * c, B, H, c, d,
                                    (long long)Tl * rs, rs, (long long)H * Tl, Tl, s);
        else
            err = launch_fill_empty(acc + (size_t)ph * c * rs, 0, lse + (size_t)ph * c, B, H, c, d, (long long)Tl * rs,
                                    rs, (long long)H * Tl, Tl, s);
        if (err != hipSuccess) return hip_fail(err, "fill launch");
    }
    if (chain) return ATTN_OK;
    const long long nel = (long long)B * Tl * rs;
    if (dtype == ATTN_F32 && (void*)acc == out) return ATTN_OK;
    err = launch_cast(acc, out, nel, dtype == ATTN_BF16, s);
    return err == hipSuccess ? ATTN_OK : hip_fail(err, "cast launch");
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int Tq, int Tkv, int d, long long q_off, long long kv_off,
             int causal, const uint8_t* kpm, const uint8_t* attn_mask, double rope_base, int dtype, unsigned flags,
             attn_stream_t stream) {
    return attn_bwd_ex(q, k, v, out, dout, lse, dq, dk, dv, B, H, Tq, Tkv, d, q_off, kv_off, causal, kpm, attn_mask,
                       rope_base, dtype, flags, nullptr, stream);
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, int B, int H, int Tq, int Tkv, int d, long long q_off,
                long long kv_off, int causal, const uint8_t* kpm, const uint8_t* attn_mask, double rope_base,
                int dtype, unsigned flags, const attn_variant* var, attn_stream_t stream) {
    g_err.clear();
    if (var && (var->window_left < -1 || var->window_right < -1))
        return fail(ATTN_ERR_INVALID_ARG, "window sizes must be >= -1");
    if (int rc = check_sizes(B, H, Tq, Tkv, d)) return rc;
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the backward pass supports bf16 inputs only");
    if (int rc = check_bf16_rows(dtype, H, d)) return rc;
    if (flags & ~(unsigned)(ATTN_ACCUMULATE | ATTN_OUT_F32 | ATTN_NO_TILE_SKIP))
        return fail(ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
    if ((flags & ATTN_ACCUMULATE) && !(flags & ATTN_OUT_F32))
        return fail(ATTN_ERR_INVALID_ARG, "ATTN_ACCUMULATE needs float32 gradients (ATTN_OUT_F32)");
    if (!(rope_base >= 0.0) || std::isinf(rope_base)) return fail(ATTN_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
    if (B == 0 || H == 0 || (Tq == 0 && Tkv == 0)) return ATTN_OK;
    if (Tq > 0 && (!q || !out || !dout || !lse || !dq)) return fail(ATTN_ERR_INVALID_ARG, "q, out, dout, lse and dq must not be NULL");
    if (Tkv > 0 && (!k || !v || !dk || !dv)) return fail(ATTN_ERR_INVALID_ARG, "k, v, dk and dv must not be NULL");
    for (const void* ptr : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
        if (ptr && !aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (std::llabs(q_off) > (1LL << 52) || std::llabs(kv_off) > (1LL << 52))
        return fail(ATTN_ERR_INVALID_ARG, "positions out of range");

    hipStream_t s = (hipStream_t)stream;
    const bool f32 = (flags & ATTN_OUT_F32) != 0;
    const bool accum = (flags & ATTN_ACCUMULATE) != 0;
    const long long rs = (long long)H * d;
    const size_t nq = (size_t)B * Tq * rs, nk = (size_t)B * Tkv * rs;
    if (Tq == 0 || Tkv == 0) {
        // nothing reaches the empty side; the other side's gradients are zero
        if (accum) return ATTN_OK;
        hipError_t e = hipSuccess;
        void* z = Tq == 0 ? dk : dq;
        const size_t n = Tq == 0 ? nk : nq;
        if (f32) {
            e = launch_zero_f32((float*)z, (long long)n, s);
            if (e == hipSuccess && Tq == 0) e = launch_zero_f32((float*)dv, (long long)n, s);
        } else {
            e = launch_fill_empty(z, 1, nullptr, B, H, Tq == 0 ? Tkv : Tq, d, (long long)(Tq == 0 ? Tkv : Tq) * rs,
                                  (int)rs, 0, 0, s);
            if (e == hipSuccess && Tq == 0)
                e = launch_fill_empty(dv, 1, nullptr, B, H, Tkv, d, (long long)Tkv * rs, (int)rs, 0, 0, s);
        }
        return e == hipSuccess ? ATTN_OK : hip_fail(e, "zero fill");
    }
    const bool rope = rope_base > 0.0;
    // float32 results go straight to the caller's buffers unless they must
    // still be rotated back (dq, dk with RoPE) or cast (bf16 outputs); bf16
    // dk and dv are written by the dK/dV kernel itself (rounded once, dk
    // rotated back first), so only dq goes through a finalize pass
    const bool dq_direct = f32 && !rope, kv_final = !f32;
    const bool dk_direct = dq_direct || kv_final, dv_direct = dk_direct;
    const size_t ld_b = align_up((size_t)B * H * Tq * sizeof(float2));
    const size_t tab_q = rope ? align_up((size_t)Tq * (d / 2) * sizeof(double2)) : 0;
    const size_t tab_k = rope ? align_up((size_t)Tkv * (d / 2) * sizeof(double2)) : 0;
    const size_t qr_b = rope ? align_up(nq * 2) : 0, kr_b = rope ? align_up(nk * 2) : 0;
    const size_t dq_b = dq_direct ? 0 : align_up(nq * 4), dk_b = dk_direct ? 0 : align_up(nk * 4);
    const size_t dv_b = dv_direct ? 0 : align_up(nk * 4);
    const size_t lst = kpm_list_bytes(kpm, dtype, flags, B, Tkv);
    Scratch ws;
    hipError_t e = ws.alloc(ld_b + tab_q + tab_k + qr_b + kr_b + dq_b + dk_b + dv_b + lst, s);
    if (e != hipSuccess) return hip_fail(e, "scratch allocation");
    char* wp = (char*)ws.ptr;
    float2* ld2 = (float2*)wp;
    wp += ld_b;
    double2* tq = (double2*)wp;
    wp += tab_q;
    double2* tk = (double2*)wp;
    wp += tab_k;
    void* qr = wp;
    wp += qr_b;
    void* kr = wp;
    wp += kr_b;
    float* gq = dq_direct ? (float*)dq : (float*)wp;
    wp += dq_b;
    float* gk = dk_direct ? (float*)dk : (float*)wp;
    wp += dk_b;
    float* gv = dv_direct ? (float*)dv : (float*)wp;
    wp += dv_b;
    int* list = lst ? (int*)wp : nullptr;

    e = launch_bwd_delta(dout, out, lse, ld2, B, H, Tq, d, (long long)Tq * rs, (int)rs, (long long)H * Tq, Tq, s);
    if (e != hipSuccess) return hip_fail(e, "delta launch");
    if (rope) {
        const double lb = std::log(rope_base);
        e = launch_rope_table(tq, q_off, Tq, d, lb, s);
        if (e == hipSuccess) e = launch_rope_table(tk, kv_off, Tkv, d, lb, s);
        if (e == hipSuccess) e = launch_rope_copy_bf16(q, qr, tq, B, Tq, H, d, s);
        if (e == hipSuccess) e = launch_rope_copy_bf16(k, kr, tk, B, Tkv, H, d, s);
        if (e != hipSuccess) return hip_fail(e, "rotary launch");
    }
    BwdCall c{};
    if (var) {
        c.win_left = window_arg(var->window_left);
        c.win_right = window_arg(var->window_right);
        c.alibi = var->alibi_slopes;
    }
    c.q = rope ? qr : q; c.k = rope ? kr : k; c.v = v; c.dout = dout; c.ld2 = ld2;
    c.dq = gq; c.dk = gk; c.dv = gv;
    c.B = B; c.H = H; c.Tq = Tq; c.Tkv = Tkv; c.d = d; c.q_off = q_off; c.kv_off = kv_off; c.causal = causal;
    c.kpm = kpm; c.amask = attn_mask;
    // accumulate in the kernels only where they write the caller's buffers
    c.flags = (flags & ATTN_NO_TILE_SKIP) | (accum && dq_direct ? ATTN_ACCUMULATE : 0u);
    c.q_bstride = (long long)Tq * rs; c.kv_bstride = (long long)Tkv * rs; c.kpm_bstride = Tkv;
    c.lse_bstride = (long long)H * Tq; c.lse_hstride = Tq; c.amask_stride = Tkv;
    if (kv_final) {
        c.dk = c.dv = nullptr;
        c.dk_out = (uint16_t*)dk;
        c.dv_out = (uint16_t*)dv;
        c.dk_rope = rope ? tk : nullptr;
    }
    if (int rc = enqueue_bwd(c, list, s)) return rc;
    // finalize: rotate back, cast, accumulate
    const int tobf = f32 ? 0 : 1;
    const int acc = accum ? 1 : 0;
    if (!dq_direct) {
        e = launch_bwd_finalize(gq, dq, rope ? tq : nullptr, B, Tq, H, d, (long long)Tq * rs, (long long)Tq * rs, tobf, acc, s);
        if (e != hipSuccess) return hip_fail(e, "finalize launch");
    }
    if (!dk_direct) {
        e = launch_bwd_finalize(gk, dk, rope ? tk : nullptr, B, Tkv, H, d, (long long)Tkv * rs, (long long)Tkv * rs, tobf, acc, s);
        if (e != hipSuccess) return hip_fail(e, "finalize launch");
    }
    if (!dv_direct) {
        e = launch_bwd_finalize(gv, dv, nullptr, B, Tkv, H, d, (long long)Tkv * rs, (long long)Tkv * rs, tobf, acc, s);
        if (e != hipSuccess) return hip_fail(e, "finalize launch");
    }
    return ATTN_OK;
}

int attn_ring_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int T, int d, int P, int rank, int zigzag, int causal,
                  const uint8_t* kpm, double rope_base, int dtype, unsigned flags, attn_stream_t stream) {
    return attn_ring_bwd_ex(q, k, v, out, dout, lse, dq, dk, dv, B, H, T, d, P, rank, zigzag, causal, kpm, rope_base,
                            dtype, flags, nullptr, stream);
}

int attn_ring_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int d, int P, int rank,
                     int zigzag, int causal, const uint8_t* kpm, double rope_base, int dtype, unsigned flags,
                     const attn_variant* var, attn_stream_t stream) {
    g_err.clear();
    if (var && (var->window_left < -1 || var->window_right < -1))
        return fail(ATTN_ERR_INVALID_ARG, "window sizes must be >= -1");
    const long long wl = var ? window_arg(var->window_left) : -1, wr = var ? window_arg(var->window_right) : -1;
    const int n = attn_ring_plan(T, P, rank, zigzag, causal, nullptr, 0);
    if (n < 0) return -n;
    const int Tl = T / P;
    if (int rc = check_sizes(B, H, Tl, T, d)) return rc;
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the backward pass supports bf16 inputs only");
    if (int rc = check_bf16_rows(dtype, H, d)) return rc;
    if (flags & ~(unsigned)(ATTN_NO_TILE_SKIP | ATTN_OUT_F32))
        return fail(ATTN_ERR_INVALID_ARG, "only ATTN_NO_TILE_SKIP and ATTN_OUT_F32 may be passed");
    if (!(rope_base >= 0.0) || std::isinf(rope_base)) return fail(ATTN_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
    if (B == 0 || H == 0) return ATTN_OK;
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return fail(ATTN_ERR_INVALID_ARG, "NULL pointer");
    for (const void* ptr : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
        if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    std::vector<attn_ring_call> plan(n);
    attn_ring_plan(T, P, rank, zigzag, causal, plan.data(), n);
    drop_dead_subcalls(plan, causal, wl, wr);
    const int n_live = (int)plan.size();

    hipStream_t s = (hipStream_t)stream;
    const bool rope = rope_base > 0.0;
    const long long rs = (long long)H * d;
    const size_t nq = (size_t)B * Tl * rs, nk = (size_t)B * T * rs;
    const size_t ld_b = align_up((size_t)B * H * Tl * sizeof(float2));
    const size_t tab_q = rope ? align_up((size_t)Tl * (d / 2) * sizeof(double2)) : 0;
    const size_t tab_k = rope ? align_up((size_t)T * (d / 2) * sizeof(double2)) : 0;
    const size_t qr_b = rope ? align_up(nq * 2) : 0, kr_b = rope ? align_up(nk * 2) : 0;
    const size_t g_b = align_up(nq * 4) + 2 * align_up(nk * 4);
    std::vector<size_t> lst_off(n_live, 0);
    size_t total = ld_b + tab_q + tab_k + qr_b + kr_b + g_b;
    for (int i = 0; i < n_live; ++i) {
        lst_off[i] = total;
        total += kpm_list_bytes(kpm ? kpm + plan[i].kv_pos0 : nullptr, dtype, flags, B, plan[i].kv_rows);
    }
    Scratch ws;
    hipError_t e = ws.alloc(total, s);
    if (e != hipSuccess) return hip_fail(e, "scratch allocation");
    char* base = (char*)ws.ptr;
    char* wp = base;
    float2* ld2 = (float2*)wp; wp += ld_b;
    double2* tq = (double2*)wp; wp += tab_q;
    double2* tk = (double2*)wp; wp += tab_k;
    char* qr = wp; wp += qr_b;
    char* kr = wp; wp += kr_b;
    float* gq = (float*)wp; wp += align_up(nq * 4);
    float* gk = (float*)wp; wp += align_up(nk * 4);
    float* gv = (float*)wp;

    // The first sub-call that touches a query block's dq, or a key block's
    // dk and dv, writes them; later ones add.  Key blocks of the plan are
    // equal or disjoint row ranges; rows no sub-call touches are zeroed.
    std::vector<int> write_dq(n_live, 0), write_kv(n_live, 0);
    std::vector<std::pair<int, int>> kv_seen;   // (first row, rows)
    bool q_seen[2] = {false, false}, disjoint = true;
    for (int i = 0; i < n_live; ++i) {
        const int ph = plan[i].q_row0 == 0 ? 0 : 1;
        write_dq[i] = !q_seen[ph];
        q_seen[ph] = true;
        const int r0 = (int)plan[i].kv_pos0, nr = plan[i].kv_rows;
        bool same = false;
        for (const auto& r : kv_seen) {
            if (r.first == r0 && r.second == nr) same = true;
            else if (r0 < r.first + r.second && r.first < r0 + nr) disjoint = false;
        }
        write_kv[i] = !same;
        if (!same) kv_seen.push_back({r0, nr});
    }
    e = launch_bwd_delta(dout, out, lse, ld2, B, H, Tl, d, (long long)Tl * rs, (int)rs, (long long)H * Tl, Tl, s);
    if (!disjoint) {   // not the plan's layout: zero everything, every sub-call adds
        std::fill(write_dq.begin(), write_dq.end(), 0);
        std::fill(write_kv.begin(), write_kv.end(), 0);
        if (e == hipSuccess) e = launch_zero_f32(gq, (long long)nq, s);
        if (e == hipSuccess) e = launch_zero_f32(gk, (long long)nk, s);
        if (e == hipSuccess) e = launch_zero_f32(gv, (long long)nk, s);
    } else {
        const int parts = zigzag ? 2 : 1, c = Tl / parts;
        for (int ph = 0; ph < parts && e == hipSuccess; ++ph)
            if (!q_seen[ph])
                for (int b = 0; b < B && e == hipSuccess; ++b)
                    e = launch_zero_f32(gq + ((size_t)b * Tl + (size_t)ph * c) * rs, (long long)c * rs, s);
        for (const auto& r : complement_rows(kv_seen, T))
            for (int b = 0; b < B && e == hipSuccess; ++b) {
                const size_t off = ((size_t)b * T + r.first) * rs;
                e = launch_zero_f32(gk + off, (long long)(r.second - r.first) * rs, s);
                if (e == hipSuccess) e = launch_zero_f32(gv + off, (long long)(r.second - r.first) * rs, s);
            }
    }
    if (e != hipSuccess) return hip_fail(e, "setup launch");
    if (rope) {
        const double lb = std::log(rope_base);
        const int parts = zigzag ? 2 : 1;
        const int c = Tl / parts;
        for (int ph = 0; ph < parts && e == hipSuccess; ++ph) {
            const long long pos0 = (long long)(ph == 0 ? rank : 2 * P - 1 - rank) * c;
            e = launch_rope_table(tq + (size_t)ph * c * (d / 2), pos0, c, d, lb, s);
        }
        if (e == hipSuccess) e = launch_rope_table(tk, 0, T, d, lb, s);
        if (e == hipSuccess) e = launch_rope_copy_bf16(q, qr, tq, B, Tl, H, d, s);
        if (e == hipSuccess) e = launch_rope_copy_bf16(k, kr, tk, B, T, H, d, s);
        if (e != hipSuccess) return hip_fail(e, "rotary launch");
    }
    // A key block only one sub-call touches gets its final bf16 dk, dv from
    // that sub-call's dK/dV kernel (rounded once, dk rotated back first, as
    // the finalize pass would); the finalize covers the other rows.
    const int tobf = (flags & ATTN_OUT_F32) ? 0 : 1;
    std::vector<int> kv_final(n_live, 0);
    std::vector<std::pair<int, int>> final_rows;   // (first row, rows)
    if (disjoint && tobf)
        for (int i = 0; i < n_live; ++i) {
            int touched = 0;
            for (int j = 0; j < n_live; ++j)
                touched += plan[j].kv_pos0 == plan[i].kv_pos0 && plan[j].kv_rows == plan[i].kv_rows;
            if (touched == 1) {
                kv_final[i] = 1;
                final_rows.push_back({(int)plan[i].kv_pos0, plan[i].kv_rows});
            }
        }
    const size_t esz = 2;
    for (int i = 0; i < n_live; ++i) {
        const attn_ring_call& pc = plan[i];
        BwdCall c{};
        c.q = (rope ? (const char*)qr : (const char*)q) + (size_t)pc.q_row0 * rs * esz;
        c.k = (rope ? (const char*)kr : (const char*)k) + (size_t)pc.kv_pos0 * rs * esz;
        c.v = (const char*)v + (size_t)pc.kv_pos0 * rs * esz;
        c.dout = (const char*)dout + (size_t)pc.q_row0 * rs * esz;
        c.ld2 = ld2 + pc.q_row0;
        c.dq = gq + (size_t)pc.q_row0 * rs;
        c.dk = gk + (size_t)pc.kv_pos0 * rs;
        c.dv = gv + (size_t)pc.kv_pos0 * rs;
        c.B = B; c.H = H; c.Tq = pc.q_rows; c.Tkv = pc.kv_rows; c.d = d;
        c.q_off = pc.q_pos0; c.kv_off = pc.kv_pos0; c.causal = causal;
        c.kpm = kpm ? kpm + pc.kv_pos0 : nullptr;
        c.amask = nullptr;
        c.win_left = wl;
        c.win_right = wr;
        c.alibi = var ? var->alibi_slopes : nullptr;
        c.flags = (flags & ATTN_NO_TILE_SKIP) | ATTN_ACCUMULATE;
        c.write_dq = write_dq[i];
        c.write_dkdv = write_kv[i];
        if (kv_final[i]) {
            c.dk = c.dv = nullptr;
            c.dk_out = (uint16_t*)dk + (size_t)pc.kv_pos0 * rs;
            c.dv_out = (uint16_t*)dv + (size_t)pc.kv_pos0 * rs;
            c.dk_rope = rope ? tk + (size_t)pc.kv_pos0 * (d / 2) : nullptr;
        }
        c.q_bstride = (long long)Tl * rs; c.kv_bstride = (long long)T * rs; c.kpm_bstride = T;
        c.lse_bstride = (long long)H * Tl; c.lse_hstride = Tl; c.amask_stride = 0;
        const size_t lb = kpm_list_bytes(c.kpm, dtype, flags, B, c.Tkv);
        if (int rc = enqueue_bwd(c, lb ? (int*)(base + lst_off[i]) : nullptr, s)) return rc;
    }
    e = launch_bwd_finalize(gq, dq, rope ? tq : nullptr, B, Tl, H, d, (long long)Tl * rs, (long long)Tl * rs, tobf, 0, s);
    const size_t osz = tobf ? 2 : 4;
    for (const auto& r : complement_rows(final_rows, T)) {
        const int r0 = r.first, nr = r.second - r.first;
        if (e == hipSuccess)
            e = launch_bwd_finalize(gk + (size_t)r0 * rs, (char*)dk + (size_t)r0 * rs * osz,
                                    rope ? tk + (size_t)r0 * (d / 2) : nullptr, B, nr, H, d, (long long)T * rs,
                                    (long long)T * rs, tobf, 0, s);
        if (e == hipSuccess)
            e = launch_bwd_finalize(gv + (size_t)r0 * rs, (char*)dv + (size_t)r0 * rs * osz, nullptr, B, nr, H, d,
                                    (long long)T * rs, (long long)T * rs, tobf, 0, s);
    }
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "finalize launch");
}

}  // extern "C"
