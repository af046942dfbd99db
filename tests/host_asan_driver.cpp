// Host-side harness for the C ABI's host logic (validation, ring plan, dead
// sub-call pruning, scratch layout, launch parameters), run under
// AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.
//
// It links the library's host translation unit (api.hip, compiled host-only)
// against stand-ins for the HIP runtime calls it makes and for every kernel
// launcher.  "Device" buffers are ordinary host allocations of exactly the
// size an entry point documents; each stand-in launcher touches (reads or
// writes the first and last byte of) every row its kernel would read or
// write, so a wrong stride, offset, scratch size or row count shows up as a
// heap-buffer-overflow report.  The stand-in allocator records the scratch of
// each call, which is checked against the formulas of include/attn.h, and can
// be told to fail, to check that the failure returns ATTN_ERR_HIP before any
// launch.  No GPU is involved.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../blockwise_online_softmax_attn_amd/csrc/common.h"

// ------------------------------------------------------------ bookkeeping
static int g_launches = 0;            // launcher calls since the last reset
static size_t g_alloc_bytes = 0;      // scratch bytes requested since the last reset
static int g_allocs = 0;
static bool g_fail_alloc = false;
static bool g_fail_launch = false;
// the stand-in reports stream capture by default: each call then allocates
// exactly its scratch in stream order, which the size checks compare with
// the formulas; kept_scratch_cases() turns it off
static bool g_capturing = true;
static int g_frees = 0;
static int g_syncs = 0;
static int g_kv_final = 0;     // dK/dV launches that wrote final bf16 rows
static int g_failures = 0;

#define CHECK(cond, ...)                                          \
    do {                                                          \
        if (!(cond)) {                                            \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                    \
            std::fprintf(stderr, "\n");                           \
            ++g_failures;                                         \
        }                                                         \
    } while (0)

static void reset() {
    g_launches = 0;
    g_alloc_bytes = 0;
    g_allocs = 0;
}

// Read the first and last byte of [p, p + n), or write them.
static void touch(const void* p, size_t n, bool write) {
    if (n == 0) return;
    if (!p) {
        std::fprintf(stderr, "FAIL: a launcher was handed a null buffer for %zu bytes\n", n);
        ++g_failures;
        return;
    }
    volatile unsigned char* c = (volatile unsigned char*)p;
    unsigned char a = c[0], b = c[n - 1];
    if (write) {
        c[0] = a;
        c[n - 1] = b;
    }
}
static hipError_t launched() {
    ++g_launches;
    return g_fail_launch ? hipErrorLaunchFailure : hipSuccess;
}

// ------------------------------------------------------------ HIP runtime stand-ins
extern "C" {
hipError_t hipMallocAsync(void** p, size_t n, hipStream_t) {
    if (g_fail_alloc) return hipErrorOutOfMemory;
    *p = std::malloc(n ? n : 1);
    g_alloc_bytes += n;
    ++g_allocs;
    return hipSuccess;
}
hipError_t hipFreeAsync(void* p, hipStream_t) {
    std::free(p);
    ++g_frees;
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* st) {
    *st = g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipDeviceSynchronize() {
    ++g_syncs;
    return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t a, int) {
    *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
    *e = (hipEvent_t)std::malloc(8);
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    std::free((void*)e);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
    *ms = 1.f;
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stand-in HIP error"; }
}

// ------------------------------------------------------------ launcher stand-ins
namespace bosa {

static size_t bytes_of(bool f32) { return f32 ? 4 : 2; }

// rows (b, t, h) of a (B, T, H, d) tensor with batch stride bs and row stride rs (elements)
static void rows(const void* base, int B, int T, int H, int d, long long bs, long long rs, size_t esz, bool w) {
    if (!base) return;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h)
                touch((const char*)base + ((size_t)b * bs + (size_t)t * rs + (size_t)h * d) * esz, (size_t)d * esz, w);
}
static void lse_rows(const float* lse, int B, int H, int T, long long bs, long long hs, bool w) {
    if (!lse) return;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) touch(lse + (size_t)b * bs + (size_t)h * hs, (size_t)T * 4, w);
}
static void mask_rows(const uint8_t* m, int B, long long bs, int n) {
    if (!m) return;
    for (int b = 0; b < B; ++b) touch(m + (size_t)b * bs, (size_t)n, false);
}
static void tile_list(const int* l, int B, int stride, int Tkv) {
    if (!l) return;
    for (int b = 0; b < B; ++b) touch(l + (size_t)b * stride, (size_t)(2 + (Tkv + 63) / 64) * 4, false);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t) {
    const bool of32 = (p.flags & ATTN_OUT_F32) != 0;
    rows(p.q, p.B, p.Tq, p.H, d, p.q_bstride, p.row_stride, 2, false);
    rows(p.k, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, false);
    rows(p.v, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, false);
    rows(p.out, p.B, p.Tq, p.H, d, p.o_bstride, p.row_stride, bytes_of(of32), true);
    lse_rows(p.lse, p.B, p.H, p.Tq, p.lse_bstride, p.lse_hstride, true);
    mask_rows(p.kpm, p.B, p.kpm_bstride, p.Tkv);
    if (p.amask) for (int t = 0; t < p.Tq; ++t) touch(p.amask + (size_t)t * p.amask_stride, (size_t)p.Tkv, false);
    tile_list(p.kpm_list, p.B, p.kpm_list_stride, p.Tkv);
    if (p.alibi) touch(p.alibi, (size_t)p.H * 4, false);
    CHECK(!p.rope_q && !p.rope_k, "the bf16 kernel takes rotated operands");
    return launched();
}
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t) {
    rows(p.q, p.B, p.Tq, p.H, d, p.q_bstride, p.row_stride, 4, false);
    rows(p.k, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 4, false);
    rows(p.v, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 4, false);
    rows(p.out, p.B, p.Tq, p.H, d, p.o_bstride, p.row_stride, 4, true);
    lse_rows(p.lse, p.B, p.H, p.Tq, p.lse_bstride, p.lse_hstride, true);
    mask_rows(p.kpm, p.B, p.kpm_bstride, p.Tkv);
    if (p.amask) for (int t = 0; t < p.Tq; ++t) touch(p.amask + (size_t)t * p.amask_stride, (size_t)p.Tkv, false);
    if (p.rope_q) touch(p.rope_q, (size_t)p.Tq * (d / 2) * sizeof(double2), false);
    if (p.rope_k) touch(p.rope_k, (size_t)p.Tkv * (d / 2) * sizeof(double2), false);
    if (p.alibi) touch(p.alibi, (size_t)p.H * 4, false);
    return launched();
}
hipError_t launch_fwd_bf16_chain(const ChainParams& c, int d, hipStream_t) {
    const FwdParams& p = c.p;
    CHECK(c.nblk >= 1 && c.nblk <= kMaxChain, "chain of %d blocks", c.nblk);
    rows(p.q, p.B, p.Tq, p.H, d, p.q_bstride, p.row_stride, 2, false);
    rows(p.out, p.B, p.Tq, p.H, d, p.o_bstride, p.row_stride, 4, true);
    if (c.out_bf16) rows(c.out_bf16, p.B, p.Tq, p.H, d, p.o_bstride, p.row_stride, 2, true);
    lse_rows(p.lse, p.B, p.H, p.Tq, p.lse_bstride, p.lse_hstride, true);
    for (int s = 0; s < c.nblk; ++s) {
        const ChainBlock& k = c.blk[s];
        rows(k.k, p.B, k.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, false);
        rows(k.v, p.B, k.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, false);
        mask_rows(k.kpm, p.B, p.kpm_bstride, k.Tkv);
        tile_list(k.kpm_list, p.B, (k.Tkv + 63) / 64 + 2, k.Tkv);
    }
    return launched();
}
hipError_t launch_rope_table(double2* tab, long long, int n, int d, double, hipStream_t) {
    touch(tab, (size_t)n * (d / 2) * sizeof(double2), true);
    return launched();
}
hipError_t launch_kpm_tiles(const uint8_t* kpm, long long bs, int B, int Tkv, int tile, int* list, int stride,
                            hipStream_t) {
    mask_rows(kpm, B, bs, Tkv);
    for (int b = 0; b < B; ++b) touch(list + (size_t)b * stride, (size_t)(2 + (Tkv + tile - 1) / tile) * 4, true);
    return launched();
}
hipError_t launch_merge(float* oa, float* la, const void* ob, const float* lb, int B, int H, int Tq, int d,
                        long long o_bstride, int row_stride, long long lse_bstride, int lse_hstride, int b_is_bf16,
                        hipStream_t) {
    rows(oa, B, Tq, H, d, o_bstride, row_stride, 4, true);
    rows(ob, B, Tq, H, d, o_bstride, row_stride, b_is_bf16 ? 2 : 4, false);
    lse_rows(la, B, H, Tq, lse_bstride, lse_hstride, true);
    lse_rows(lb, B, H, Tq, lse_bstride, lse_hstride, false);
    return launched();
}
hipError_t launch_cast(const float* src, void* dst, long long n, int to_bf16, hipStream_t) {
    touch(src, (size_t)n * 4, false);
    touch(dst, (size_t)n * (to_bf16 ? 2 : 4), true);
    return launched();
}
hipError_t launch_rope_apply(void* x, const long long* pos, double, int B, int T, int H, int d, int is_bf16,
                             hipStream_t) {
    touch(pos, (size_t)T * 8, false);
    touch(x, (size_t)B * T * H * d * (is_bf16 ? 2 : 4), true);
    return launched();
}
hipError_t launch_rope_rotate_bf16(const RopeJob& a, const RopeJob& b, int H, int d, double, hipStream_t) {
    const int hpt = (H % 4 == 0) ? 4 : 1;
    for (const RopeJob* j : {&a, &b}) {
        const long long tokens = j->n_threads / ((H / hpt) * (d / 8));
        touch(j->src, (size_t)tokens * H * d * 2, false);
        touch(j->dst, (size_t)tokens * H * d * 2, true);
    }
    return launched();
}
hipError_t launch_rope_copy_bf16(const void* src, void* dst, const double2* tab, int B, int T, int H, int d, int split,
                                 long long off0, long long off1, hipStream_t) {
    touch(src, (size_t)B * T * H * d * 2, false);
    touch(dst, (size_t)B * T * H * d * 2, true);
    for (int t = 0; t < T; ++t) {
        const long long r = t < split ? off0 + t : off1 + (t - split);
        touch(tab + (size_t)r * (d / 2), (size_t)(d / 2) * sizeof(double2), false);
    }
    return launched();
}
hipError_t launch_rope_copy_bf16(const void* src, void* dst, const double2* tab, int B, int T, int H, int d,
                                 hipStream_t s) {
    return launch_rope_copy_bf16(src, dst, tab, B, T, H, d, T, 0, 0, s);
}
static void bwd_common(const BwdParams& p, int d) {
    rows(p.q, p.B, p.Tq, p.H, d, p.q_bstride, p.row_stride, 2, false);
    rows(p.dout, p.B, p.Tq, p.H, d, p.q_bstride, p.row_stride, 2, false);
    rows(p.k, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, false);
    rows(p.v, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, false);
    for (int b = 0; b < p.B; ++b)
        for (int h = 0; h < p.H; ++h)
            touch(p.ld2 + (size_t)b * p.lse_bstride + (size_t)h * p.lse_hstride, (size_t)p.Tq * sizeof(float2), false);
    mask_rows(p.kpm, p.B, p.kpm_bstride, p.Tkv);
    if (p.amask) for (int t = 0; t < p.Tq; ++t) touch(p.amask + (size_t)t * p.amask_stride, (size_t)p.Tkv, false);
    if (p.alibi) touch(p.alibi, (size_t)p.H * 4, false);
}
hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t) {
    bwd_common(p, d);
    tile_list(p.kpm_list, p.B, p.kpm_list_stride, p.Tkv);
    rows(p.dq, p.B, p.Tq, p.H, d, p.q_bstride, p.row_stride, 4, true);
    return launched();
}
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t) {
    bwd_common(p, d);
    if (p.dk_out || p.dv_out) {
        CHECK(p.dk_out && p.dv_out && !p.dk && !p.dv, "dK/dV launch with a mix of final and float32 outputs");
        rows(p.dk_out, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, true);
        rows(p.dv_out, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 2, true);
        if (p.dk_rope) touch(p.dk_rope, (size_t)p.Tkv * (d / 2) * sizeof(double2), false);
        ++g_kv_final;
    } else {
        rows(p.dk, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 4, true);
        rows(p.dv, p.B, p.Tkv, p.H, d, p.kv_bstride, p.row_stride, 4, true);
    }
    return launched();
}
hipError_t launch_bwd_delta(const void* dout, const void* out, const float* lse, float2* ld2, int B, int H, int Tq,
                            int d, long long bstride, int row_stride, long long lse_bstride, int lse_hstride,
                            hipStream_t) {
    rows(dout, B, Tq, H, d, bstride, row_stride, 2, false);
    rows(out, B, Tq, H, d, bstride, row_stride, 2, false);
    lse_rows(lse, B, H, Tq, lse_bstride, lse_hstride, false);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            touch(ld2 + (size_t)b * lse_bstride + (size_t)h * lse_hstride, (size_t)Tq * sizeof(float2), true);
    return launched();
}
hipError_t launch_bwd_finalize(const float* src, void* dst, const double2* tab, int B, int T, int H, int d,
                               long long src_bstride, long long dst_bstride, int dst_bf16, int, hipStream_t) {
    rows(src, B, T, H, d, src_bstride, (long long)H * d, 4, false);
    rows(dst, B, T, H, d, dst_bstride, (long long)H * d, dst_bf16 ? 2 : 4, true);
    if (tab) touch(tab, (size_t)T * (d / 2) * sizeof(double2), false);
    return launched();
}
hipError_t launch_zero_f32(float* x, long long n, hipStream_t) {
    touch(x, (size_t)n * 4, true);
    return launched();
}
hipError_t launch_fill_empty(void* out, int out_bf16, float* lse, int B, int H, int rows_, int d, long long o_bstride,
                             int row_stride, long long lse_bstride, int lse_hstride, hipStream_t) {
    rows(out, B, rows_, H, d, o_bstride, row_stride, out_bf16 ? 2 : 4, true);
    lse_rows(lse, B, H, rows_, lse_bstride, lse_hstride, true);
    return launched();
}
hipError_t launch_decode_chunks(const DecodeParams& p, int d, int is_bf16, hipStream_t) {
    const size_t e = is_bf16 ? 2 : 4;
    touch(p.q, (size_t)p.B * p.H * d * e, false);
    touch(p.k, (size_t)p.B * p.Tcap * p.H * d * e, false);
    touch(p.v, (size_t)p.B * p.Tcap * p.H * d * e, false);
    touch(p.cache_len, (size_t)p.B * 4, false);
    touch(p.part_o, (size_t)p.B * p.H * p.n_chunks * d * 4, true);
    touch(p.part_lse, (size_t)p.B * p.H * p.n_chunks * 4, true);
    CHECK((long long)p.CH * p.n_chunks >= p.Tcap, "chunks cover %d of %d slots", p.CH * p.n_chunks, p.Tcap);
    return launched();
}
hipError_t launch_decode_merge(const DecodeParams& p, int d, int out_bf16, hipStream_t) {
    touch(p.part_o, (size_t)p.B * p.H * p.n_chunks * d * 4, false);
    touch(p.part_lse, (size_t)p.B * p.H * p.n_chunks * 4, false);
    touch(p.out, (size_t)p.B * p.H * d * (out_bf16 ? 2 : 4), true);
    if (p.lse) touch(p.lse, (size_t)p.B * p.H * 4, true);
    return launched();
}
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* kc, void* vc, int* cache_len, int B, int H,
                            int Tcap, int d, double, int is_bf16, hipStream_t) {
    const size_t e = is_bf16 ? 2 : 4;
    touch(k_new, (size_t)B * H * d * e, false);
    touch(v_new, (size_t)B * H * d * e, false);
    touch(cache_len, (size_t)B * 4, true);
    for (int b = 0; b < B; ++b) {
        const int L = cache_len[b];
        if (L < 0 || L >= Tcap) continue;
        touch((char*)kc + ((size_t)b * Tcap + L) * H * d * e, (size_t)H * d * e, true);
        touch((char*)vc + ((size_t)b * Tcap + L) * H * d * e, (size_t)H * d * e, true);
    }
    return launched();
}
static unsigned char g_static_ws[kDecodeStaticBytes];
hipError_t decode_static_workspace(void** ptr) {
    *ptr = g_static_ws;
    return hipSuccess;
}

}  // namespace bosa

// ------------------------------------------------------------ buffers
struct Buf {
    std::vector<void*> owned;
    void* get(size_t bytes) {
        void* p = std::malloc(bytes ? bytes : 1);
        std::memset(p, 0, bytes);
        owned.push_back(p);
        return p;
    }
    ~Buf() {
        for (void* p : owned) std::free(p);
    }
};
static size_t au(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------ cases
static void forward_cases() {
    for (int dtype : {ATTN_BF16, ATTN_F32})
        for (int d : {64, 128})
            for (int rope : {0, 1})
                for (int kp : {0, 1}) {
                    Buf m;
                    const int B = 2, H = 3, Tq = 77, Tkv = 130;
                    const size_t e = dtype == ATTN_BF16 ? 2 : 4;
                    void* q = m.get((size_t)B * Tq * H * d * e);
                    void* k = m.get((size_t)B * Tkv * H * d * e);
                    void* v = m.get((size_t)B * Tkv * H * d * e);
                    void* out = m.get((size_t)B * Tq * H * d * 4);
                    float* lse = (float*)m.get((size_t)B * H * Tq * 4);
                    uint8_t* kpm = kp ? (uint8_t*)m.get((size_t)B * Tkv) : nullptr;
                    uint8_t* am = (uint8_t*)m.get((size_t)Tq * Tkv);
                    reset();
                    int rc = attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 5, 0, 1, kpm, am, rope ? 1e4 : 0.0, dtype,
                                      ATTN_OUT_F32, nullptr);
                    CHECK(rc == ATTN_OK, "attn_fwd rc %d (%s)", rc, attn_last_error());
                    size_t want = 0;
                    if (rope && dtype == ATTN_F32) want += au((size_t)Tq * (d / 2) * 16) + au((size_t)Tkv * (d / 2) * 16);
                    if (rope && dtype == ATTN_BF16) want += au((size_t)B * Tkv * H * d * 2) + au((size_t)B * Tq * H * d * 2);
                    if (kp && dtype == ATTN_BF16) want += au((size_t)B * ((Tkv + 63) / 64 + 2) * 4);
                    CHECK(g_alloc_bytes == want, "attn_fwd dtype %d d %d rope %d kpm %d: scratch %zu, formula %zu",
                          dtype, d, rope, kp, g_alloc_bytes, want);
                    rc = attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 5, 0, 1, kpm, am, rope ? 1e4 : 0.0, dtype,
                                  ATTN_OUT_F32 | ATTN_ACCUMULATE, nullptr);
                    CHECK(rc == ATTN_OK, "accumulate rc %d", rc);
                    attn_variant var{100, 3, (const float*)m.get((size_t)H * 4)};
                    rc = attn_fwd_ex(q, k, v, out, lse, B, H, Tq, Tkv, d, 5, 0, 1, kpm, nullptr, rope ? 1e4 : 0.0,
                                     dtype, 0, &var, nullptr);
                    CHECK(rc == ATTN_OK, "attn_fwd_ex rc %d (%s)", rc, attn_last_error());
                    // Tkv = 0: every row empty
                    rc = attn_fwd(q, nullptr, nullptr, out, lse, B, H, Tq, 0, d, 0, 0, 0, nullptr, nullptr, 0.0,
                                  dtype, 0, nullptr);
                    CHECK(rc == ATTN_OK, "empty keys rc %d", rc);
                }
}

static void invalid_cases() {
    Buf m;
    void* p = m.get(1 << 20);
    reset();
    CHECK(attn_fwd(p, p, p, p, (float*)p, 1, 1, 4, 4, 96, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0, nullptr) ==
              ATTN_ERR_UNSUPPORTED, "d=96");
    CHECK(attn_fwd(p, p, p, p, (float*)p, -1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0, nullptr) ==
              ATTN_ERR_INVALID_ARG, "B<0");
    CHECK(attn_fwd(nullptr, p, p, p, (float*)p, 1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0,
                   nullptr) == ATTN_ERR_INVALID_ARG, "q null");
    CHECK(attn_fwd((char*)p + 2, p, p, p, (float*)p, 1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0,
                   nullptr) == ATTN_ERR_INVALID_ARG, "misaligned q");
    CHECK(attn_fwd(p, p, p, p, (float*)p, 1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, ATTN_ACCUMULATE,
                   nullptr) == ATTN_ERR_INVALID_ARG, "accumulate without f32 out");
    CHECK(attn_fwd(p, p, p, p, (float*)p, 1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, NAN, ATTN_BF16, 0, nullptr) ==
              ATTN_ERR_INVALID_ARG, "nan base");
    CHECK(attn_fwd(p, p, p, p, (float*)p, 1, 1, 4, 4, 64, 1LL << 53, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0,
                   nullptr) == ATTN_ERR_INVALID_ARG, "position range");
    CHECK(attn_fwd(p, p, p, p, (float*)p, 1, 1 << 20, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0,
                   nullptr) == ATTN_ERR_UNSUPPORTED, "H*d too large for bf16");
    attn_variant bad{-2, -1, nullptr};
    CHECK(attn_fwd_ex(p, p, p, p, (float*)p, 1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_BF16, 0, &bad,
                      nullptr) == ATTN_ERR_INVALID_ARG, "window -2");
    CHECK(attn_merge(nullptr, nullptr, nullptr, nullptr, 1, 1, 1, 64, ATTN_F32, nullptr) == ATTN_ERR_INVALID_ARG, "merge");
    CHECK(rope_apply(p, (const long long*)p, 0.0, 1, 4, 1, 64, ATTN_BF16, nullptr) == ATTN_ERR_INVALID_ARG, "rope base");
    CHECK(attn_cast((const float*)p, p, -1, ATTN_BF16, nullptr) == ATTN_ERR_INVALID_ARG, "cast n<0");
    CHECK(attn_ring_fwd(p, p, p, p, (float*)p, (float*)p, 1, 1, 100, 64, 3, 0, 0, 1, nullptr, 0.0, ATTN_BF16, 0,
                        nullptr) == ATTN_ERR_INVALID_ARG, "ring T %% P");
    CHECK(attn_ring_plan(8, 2, 2, 0, 1, nullptr, 0) < 0, "ring rank");
    CHECK(attn_bwd(p, p, p, p, p, (const float*)p, p, p, p, 1, 1, 4, 4, 64, 0, 0, 0, nullptr, nullptr, 0.0, ATTN_F32, 0,
                   nullptr) == ATTN_ERR_UNSUPPORTED, "bwd f32");
    CHECK(attn_decode(p, p, p, (const int*)p, p, (float*)p, 1, 4, 16, 128, 0.0, ATTN_BF16, 8, nullptr, nullptr) ==
              ATTN_ERR_INVALID_ARG, "decode flags");
    CHECK(attn_decode_noalloc(p, p, p, (const int*)p, p, (float*)p, 1, 40000, 1, 128, 0.0, ATTN_BF16, 0, nullptr,
                              nullptr) == ATTN_ERR_UNSUPPORTED, "noalloc over its workspace");
    CHECK(g_launches == 0 && g_allocs == 0, "invalid calls launched %d kernels, made %d allocations", g_launches,
          g_allocs);
}

// Every causal (query position, key position) pair of a rank exactly once.
static void ring_plan_cases() {
    for (int P : {1, 2, 3, 4, 8})
        for (int zz : {0, 1})
            for (int causal : {0, 1})
                for (int rank = 0; rank < P; ++rank) {
                    const int c = 3, T = (zz ? 2 * P : P) * c;
                    const int n = attn_ring_plan(T, P, rank, zz, causal, nullptr, 0);
                    CHECK(n > 0, "plan count %d", n);
                    std::vector<attn_ring_call> plan(n);
                    CHECK(attn_ring_plan(T, P, rank, zz, causal, plan.data(), n) == n, "plan fill");
                    std::vector<int> seen((size_t)T * T, 0);
                    bool started[2] = {false, false};
                    for (const auto& e : plan) {
                        const int ph = e.q_row0 == 0 ? 0 : 1;
                        CHECK(e.accumulate == (started[ph] ? 1 : 0), "accumulate flag");
                        started[ph] = true;
                        for (int i = 0; i < e.q_rows; ++i)
                            for (int j = 0; j < e.kv_rows; ++j) {
                                const long long qp = e.q_pos0 + i, kp = e.kv_pos0 + j;
                                CHECK(qp >= 0 && qp < T && kp >= 0 && kp < T, "position out of range");
                                if (!causal || kp <= qp) ++seen[(size_t)qp * T + kp];
                            }
                    }
                    // the rank's query positions
                    std::vector<int> qpos;
                    if (zz) {
                        for (int t = 0; t < c; ++t) qpos.push_back(rank * c + t);
                        for (int t = 0; t < c; ++t) qpos.push_back((2 * P - 1 - rank) * c + t);
                    } else {
                        const int cc = T / P;
                        for (int t = 0; t < cc; ++t) qpos.push_back(rank * cc + t);
                    }
                    for (int qp : qpos)
                        for (int kp = 0; kp < T; ++kp) {
                            const int want = (!causal || kp <= qp) ? 1 : 0;
                            CHECK(seen[(size_t)qp * T + kp] == want, "P %d rank %d zz %d causal %d: pair (%d,%d) seen %d",
                                  P, rank, zz, causal, qp, kp, seen[(size_t)qp * T + kp]);
                        }
                }
}

static void ring_fwd_cases() {
    for (int dtype : {ATTN_BF16, ATTN_F32})
        for (int P : {1, 2, 4, 8})
            for (int zz : {0, 1})
                for (int rope : {0, 1})
                    for (int kp : {0, 1})
                        for (int win : {0, 1, 2}) {
                            Buf m;
                            const int B = 2, H = 3, d = 64, c = 37, T = (zz ? 2 * P : P) * c, Tl = T / P;
                            const size_t e = dtype == ATTN_BF16 ? 2 : 4;
                            void* q = m.get((size_t)B * Tl * H * d * e);
                            void* k = m.get((size_t)B * T * H * d * e);
                            void* v = m.get((size_t)B * T * H * d * e);
                            void* out = m.get((size_t)B * Tl * H * d * e);
                            float* lse = (float*)m.get((size_t)B * H * Tl * 4);
                            float* acc = (float*)m.get((size_t)B * Tl * H * d * 4);
                            uint8_t* kpm = kp ? (uint8_t*)m.get((size_t)B * T) : nullptr;
                            attn_variant var{win == 1 ? 20 : -1, win == 2 ? 0 : -1,
                                             win == 2 ? (const float*)m.get((size_t)H * 4) : nullptr};
                            for (int rank = 0; rank < P; ++rank) {
                                reset();
                                const int rc = attn_ring_fwd_ex(q, k, v, out, lse, acc, B, H, T, d, P, rank, zz, 1, kpm,
                                                                rope ? 1e4 : 0.0, dtype, 0, win ? &var : nullptr,
                                                                nullptr);
                                CHECK(rc == ATTN_OK, "ring fwd rc %d (%s)", rc, attn_last_error());
                                if (!win) {
                                    size_t want = 0;
                                    if (rope && dtype == ATTN_F32) want += au((size_t)T * (d / 2) * 16);
                                    if (rope && dtype == ATTN_BF16)
                                        want += au((size_t)B * T * H * d * 2) + au((size_t)B * Tl * H * d * 2);
                                    const int n = attn_ring_plan(T, P, rank, zz, 1, nullptr, 0);
                                    const int rows_per = zz ? c : Tl;
                                    if (kp && dtype == ATTN_BF16) want += (size_t)n * au((size_t)B * ((rows_per + 63) / 64 + 2) * 4);
                                    CHECK(g_alloc_bytes == want, "ring fwd P %d rank %d: scratch %zu, formula %zu", P,
                                          rank, g_alloc_bytes, want);
                                }
                            }
                        }
}

static void backward_cases() {
    for (int f32 : {0, 1})
        for (int rope : {0, 1})
            for (int kp : {0, 1}) {
                Buf m;
                const int B = 2, H = 3, Tq = 71, Tkv = 133, d = 128;
                const size_t ge = f32 ? 4 : 2;
                void* q = m.get((size_t)B * Tq * H * d * 2);
                void* k = m.get((size_t)B * Tkv * H * d * 2);
                void* v = m.get((size_t)B * Tkv * H * d * 2);
                void* out = m.get((size_t)B * Tq * H * d * 2);
                void* dout = m.get((size_t)B * Tq * H * d * 2);
                float* lse = (float*)m.get((size_t)B * H * Tq * 4);
                void* dq = m.get((size_t)B * Tq * H * d * ge);
                void* dk = m.get((size_t)B * Tkv * H * d * ge);
                void* dv = m.get((size_t)B * Tkv * H * d * ge);
                uint8_t* kpm = kp ? (uint8_t*)m.get((size_t)B * Tkv) : nullptr;
                reset();
                int rc = attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, H, Tq, Tkv, d, 60, 0, 1, kpm, nullptr,
                                  rope ? 1e4 : 0.0, ATTN_BF16, f32 ? ATTN_OUT_F32 : 0u, nullptr);
                CHECK(rc == ATTN_OK, "bwd rc %d (%s)", rc, attn_last_error());
                size_t want = au((size_t)B * H * Tq * 8);
                if (rope) want += au((size_t)Tq * (d / 2) * 16) + au((size_t)Tkv * (d / 2) * 16) +
                                  au((size_t)B * Tq * H * d * 2) + au((size_t)B * Tkv * H * d * 2);
                if (!(f32 && !rope)) want += au((size_t)B * Tq * H * d * 4);
                if (f32 && rope) want += 2 * au((size_t)B * Tkv * H * d * 4);
                if (kp) want += au((size_t)B * ((Tkv + 63) / 64 + 2) * 4);
                CHECK(g_alloc_bytes == want, "bwd f32 %d rope %d kpm %d: scratch %zu, formula %zu", f32, rope, kp,
                      g_alloc_bytes, want);
            }
    // ring backward, every rank; key blocks a single sub-call touches get
    // their final bf16 rows from that sub-call (none with float32 outputs)
    for (int P : {2, 3, 4})
        for (int zz : {0, 1})
            for (int win : {0, 1})
              for (int B : {1, 2}) {
                Buf m;
                const int H = 2, d = 64, c = 29, T = (zz ? 2 * P : P) * c, Tl = T / P;
                void* q = m.get((size_t)B * Tl * H * d * 2);
                void* k = m.get((size_t)B * T * H * d * 2);
                void* v = m.get((size_t)B * T * H * d * 2);
                void* out = m.get((size_t)B * Tl * H * d * 2);
                void* dout = m.get((size_t)B * Tl * H * d * 2);
                float* lse = (float*)m.get((size_t)B * H * Tl * 4);
                void* dq = m.get((size_t)B * Tl * H * d * 2);
                void* dk = m.get((size_t)B * T * H * d * 2);
                void* dv = m.get((size_t)B * T * H * d * 2);
                uint8_t* kpm = (uint8_t*)m.get((size_t)B * T);
                attn_variant var{15, -1, nullptr};
                void* dk32 = m.get((size_t)B * T * H * d * 4);
                void* dv32 = m.get((size_t)B * T * H * d * 4);
                void* dq32 = m.get((size_t)B * Tl * H * d * 4);
                for (int rank = 0; rank < P; ++rank) {
                    g_kv_final = 0;
                    int rc = attn_ring_bwd_ex(q, k, v, out, dout, lse, dq, dk, dv, B, H, T, d, P, rank, zz, 1,
                                              kpm, 1e4, ATTN_BF16, 0, win ? &var : nullptr, nullptr);
                    CHECK(rc == ATTN_OK, "ring bwd rc %d (%s)", rc, attn_last_error());
                    CHECK(win || g_kv_final > 0, "ring bwd P %d zz %d rank %d: no key block written final", P, zz,
                          rank);
                    g_kv_final = 0;
                    rc = attn_ring_bwd_ex(q, k, v, out, dout, lse, dq32, dk32, dv32, B, H, T, d, P, rank, zz, 1, kpm,
                                          1e4, ATTN_BF16, ATTN_OUT_F32, win ? &var : nullptr, nullptr);
                    CHECK(rc == ATTN_OK && g_kv_final == 0, "ring bwd float32 rc %d, %d final launches", rc,
                          g_kv_final);
                }
              }
}

static void decode_cases() {
    for (int dtype : {ATTN_BF16, ATTN_F32})
        for (int noalloc : {0, 1}) {
            Buf m;
            const int B = 3, H = 5, Tcap = 700, d = 128;
            const size_t e = dtype == ATTN_BF16 ? 2 : 4;
            void* kc = m.get((size_t)B * Tcap * H * d * e);
            void* vc = m.get((size_t)B * Tcap * H * d * e);
            void* kn = m.get((size_t)B * H * d * e);
            void* vn = m.get((size_t)B * H * d * e);
            void* q = m.get((size_t)B * H * d * e);
            int* len = (int*)m.get((size_t)B * 4);
            len[0] = 0;
            len[1] = 400;
            len[2] = Tcap;
            void* out = m.get((size_t)B * H * d * e);
            float* lse = (float*)m.get((size_t)B * H * 4);
            CHECK(attn_kv_append(kn, vn, kc, vc, len, B, H, Tcap, d, 1e4, dtype, nullptr) == ATTN_OK, "append");
            attn_variant var{100, -1, nullptr};
            reset();
            const int rc = noalloc ? attn_decode_noalloc(q, kc, vc, len, out, lse, B, H, Tcap, d, 1e4, dtype, 0, &var,
                                                         nullptr)
                                   : attn_decode(q, kc, vc, len, out, lse, B, H, Tcap, d, 1e4, dtype, 0, &var, nullptr);
            CHECK(rc == ATTN_OK, "decode rc %d (%s)", rc, attn_last_error());
            CHECK(noalloc ? g_allocs == 0 : g_allocs == 1, "decode noalloc %d made %d allocations", noalloc, g_allocs);
        }
}

static void failure_cases() {
    Buf m;
    const int B = 1, H = 2, Tq = 40, Tkv = 40, d = 64;
    void* q = m.get((size_t)B * Tq * H * d * 2);
    void* k = m.get((size_t)B * Tkv * H * d * 2);
    void* v = m.get((size_t)B * Tkv * H * d * 2);
    void* out = m.get((size_t)B * Tq * H * d * 2);
    float* lse = (float*)m.get((size_t)B * H * Tq * 4);
    // an allocation failure returns ATTN_ERR_HIP before any launch
    g_fail_alloc = true;
    reset();
    int rc = attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0, nullptr);
    CHECK(rc == ATTN_ERR_HIP && g_launches == 0, "alloc failure: rc %d, %d launches", rc, g_launches);
    g_fail_alloc = false;
    // a launch failure returns ATTN_ERR_HIP (and frees the scratch: no leak at exit)
    g_fail_launch = true;
    rc = attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0, nullptr);
    CHECK(rc == ATTN_ERR_HIP, "launch failure: rc %d", rc);
    CHECK(std::strlen(attn_last_error()) > 0, "error text");
    g_fail_launch = false;
    // profiling hooks
    CHECK(attn_profile_start(8) == ATTN_OK, "profile start");
    rc = attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 0.0, ATTN_BF16, 0, nullptr);
    float ms[8];
    CHECK(rc == ATTN_OK && attn_profile_stop(ms, 8) == 1, "profiled launch count");
}

// Outside capture a call's scratch is the stream's kept buffer: allocated
// once, replaced only when a call needs more, freed by attn_release_scratch.
static void kept_scratch_cases() {
    Buf m;
    const int B = 1, H = 2, d = 64;
    const int Tq = 300, Tkv = 300, Tbig = 4800;   // rotated copies of 0.15 MB and 2.5 MB
    void* q = m.get((size_t)B * Tbig * H * d * 2);
    void* k = m.get((size_t)B * Tbig * H * d * 2);
    void* v = m.get((size_t)B * Tbig * H * d * 2);
    void* out = m.get((size_t)B * Tbig * H * d * 2);
    float* lse = (float*)m.get((size_t)B * H * Tbig * 4);
    g_capturing = false;
    CHECK(attn_release_scratch() == ATTN_OK, "release with nothing kept");
    reset();
    g_frees = 0;
    for (int i = 0; i < 3; ++i)
        CHECK(attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0, nullptr) ==
                  ATTN_OK, "kept scratch call %d (%s)", i, attn_last_error());
    CHECK(g_allocs == 1 && g_frees == 0, "three equal calls: %d allocations, %d frees", g_allocs, g_frees);
    // a smaller call reuses the buffer, a larger one replaces it
    CHECK(attn_fwd(q, k, v, out, lse, B, H, Tq / 2, Tkv / 2, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0,
                   nullptr) == ATTN_OK, "smaller call");
    CHECK(g_allocs == 1 && g_frees == 0, "smaller call: %d allocations, %d frees", g_allocs, g_frees);
    CHECK(attn_fwd(q, k, v, out, lse, B, H, Tbig, Tbig, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0,
                   nullptr) == ATTN_OK, "larger call");
    CHECK(g_allocs == 2 && g_frees == 1, "larger call: %d allocations, %d frees", g_allocs, g_frees);
    CHECK(g_alloc_bytes % (size_t(2) << 20) == 0, "kept buffers grow in 2 MiB steps (%zu bytes)", g_alloc_bytes);
    // the per-thread default stream keeps nothing: each call allocates its
    // scratch and frees it after its last launch
    for (int i = 0; i < 2; ++i)
        CHECK(attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0,
                       (attn_stream_t)hipStreamPerThread) == ATTN_OK, "per-thread stream call %d", i);
    CHECK(g_allocs == 4 && g_frees == 3, "per-thread stream: %d allocations, %d frees", g_allocs, g_frees);
    // another stream keeps a buffer of its own; an allocation failure while
    // growing it leaves nothing kept there and returns ATTN_ERR_HIP
    const attn_stream_t s2 = (attn_stream_t)(uintptr_t)0x7000;
    CHECK(attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0, s2) ==
              ATTN_OK, "second stream call");
    CHECK(g_allocs == 5 && g_frees == 3, "second stream: %d allocations, %d frees", g_allocs, g_frees);
    g_fail_alloc = true;
    const int rc = attn_fwd(q, k, v, out, lse, B, H, Tbig, Tbig, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16,
                            0, s2);
    CHECK(rc == ATTN_ERR_HIP, "growth failure: rc %d", rc);
    CHECK(g_frees == 4, "growth failure frees the old buffer: %d frees", g_frees);
    g_fail_alloc = false;
    g_syncs = 0;
    const int fr = g_frees;
    CHECK(attn_release_scratch() == ATTN_OK, "release (%s)", attn_last_error());
    CHECK(g_syncs == 1 && g_frees == fr + 1, "release: %d synchronisations, %d frees", g_syncs, g_frees - fr);
    CHECK(attn_fwd(q, k, v, out, lse, B, H, Tq, Tkv, d, 0, 0, 1, nullptr, nullptr, 1e4, ATTN_BF16, 0, nullptr) ==
              ATTN_OK, "call after release");
    CHECK(g_allocs == 6, "call after release: %d allocations", g_allocs);
    CHECK(attn_release_scratch() == ATTN_OK, "final release");
    g_capturing = true;
}

int main() {
    invalid_cases();
    forward_cases();
    ring_plan_cases();
    ring_fwd_cases();
    backward_cases();
    decode_cases();
    failure_cases();
    kept_scratch_cases();
    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host harness: all checks passed\n");
    return 0;
}
