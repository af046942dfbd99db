// Internal declarations shared by the HIP translation units of libattn.
// Device helpers here are the only definitions of the element arithmetic
// that more than one kernel needs (bf16 rounding, the rotary pair rotation,
// the partial-result merge weights), so that fused and standalone paths give
// bit-identical results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/attn.h"

namespace bosa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two float32 -> packed bf16 pair, round-to-nearest-even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- RoPE
// cos and sin of the angle of pair t at position pos, pos * base^(-2t/d),
// all in float64: at positions up to 2^20 the angle keeps ~1e-10 rad.
__device__ __forceinline__ double2 rope_cs64(long long pos, int t, int d, double log_base) {
    const double theta = exp(-(2.0 * (double)t / (double)d) * log_base);
    double s, c;
    sincos((double)pos * theta, &s, &c);
    return make_double2(c, s);
}

// The rotated pair (x0 c - x1 s, x0 s + x1 c) in float64.  With x0, x1 from
// bf16 or float32 inputs this is within two float64 units of the exact
// rotation by (c, s), so one rounding to the input dtype afterwards gives the
// correctly rounded rotated value except within ~1e-16 of a rounding midpoint.
__device__ __forceinline__ double2 rot64(double x0, double x1, double c, double s) {
    return make_double2(fma(x0, c, -(x1 * s)), fma(x0, s, x1 * c));
}

// float64 -> bf16 bit pattern, rounded once to nearest even.  The value is
// first rounded to the nearest float32 f; a second rounding of f to bf16 can
// only differ from rounding the value itself when f lands exactly on a bf16
// midpoint (low 16 bits 0x8000) without being equal to the value, and then
// the value lies on the side f moved away from: f is stepped one float32
// unit toward the value, off the midpoint, before the round to nearest even.
__host__ __device__ __forceinline__ uint32_t bf16_bits_rn(double y) {
    const float f = (float)y;                       // nearest
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0xFFFFu) == 0x8000u) {
        const double back = (double)f;
        if (back != y) u = __builtin_fabs(back) > __builtin_fabs(y) ? u - 1u : u + 1u;
    }
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A packed bf16 pair rotated by (c, s): float64 arithmetic, one rounding each.
__device__ __forceinline__ uint32_t rot_pair_bf16(uint32_t u, double c, double s) {
    const double2 y = rot64((double)bf16_lo(u), (double)bf16_hi(u), c, s);
    return bf16_bits_rn(y.x) | (bf16_bits_rn(y.y) << 16);
}
// A float32 pair rotated by (c, s): float64 arithmetic, one rounding each.
__device__ __forceinline__ float2 rot_pair_f32(float x0, float x1, double c, double s) {
    const double2 y = rot64((double)x0, (double)x1, c, s);
    return make_float2((float)y.x, (float)y.y);
}

// ---------------------------------------------------------------- merge
// Weights of two partial results with log-sum-exp la, lb over disjoint key
// sets: lse = logaddexp(la, lb), wa = e^(la-lse), wb = e^(lb-lse).  Symmetric
// in (a, b); (.., -inf) is the identity; two empty partials give (-inf, 0, 0).
__device__ __forceinline__ void merge_weights(float la, float lb, float& lse, float& wa, float& wb) {
    float mx = fmaxf(la, lb);
    if (mx == -INFINITY) { lse = -INFINITY; wa = 0.f; wb = 0.f; return; }
    float ea = expf(la - mx), eb = expf(lb - mx);
    lse = mx + logf(ea + eb);
    wa = expf(la - lse);
    wb = expf(lb - lse);
}
// wa*oa + wb*ob with two roundings of the products and one of the sum; the
// pragma forbids fusing a product into the sum (an FMA would make the result
// depend on operand order), so swapping (a, b) gives the same bits.
__device__ __forceinline__ float merge_value(float wa, float oa, float wb, float ob) {
#pragma clang fp contract(off)
    const float x = wa * oa;
    const float y = wb * ob;
    return x + y;
}

// ---------------------------------------------------------------- params
// One attention forward launch.  Strides are in elements.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    const uint8_t* kpm;        // row b at kpm + b * kpm_bstride, indexed by local key
    const uint8_t* amask;      // [Tq][amask_stride]
    const double2* rope_q;     // [Tq][d/2] (cos, sin) or null
    const double2* rope_k;     // [Tkv][d/2] or null (float32 kernel; the bf16 kernel takes rotated keys)
    const int* kpm_list;       // per batch: [count, leading clean tiles, entries...] of live key tiles, or null
    long long q_bstride, kv_bstride, o_bstride, kpm_bstride, lse_bstride;
    int row_stride;            // H * d
    int lse_hstride;
    int amask_stride;
    int kpm_list_stride;
    int B, H, Tq, Tkv;
    long long q_off, kv_off;
    int causal;
    unsigned flags;
    float scale_log2;          // log2(e) / sqrt(d)
    int n_qtiles;
    // sliding window: a key at most win_left positions before and at most
    // win_right positions after the query (absolute positions); -1 = no limit
    long long win_left, win_right;
    const float* alibi;        // [H] slopes: score -= slope_h |pos_q - pos_k| (after 1/sqrt(d)), or null
    float sqrt_d;              // sqrt(d): the bias in units of the unscaled dot product
    // chained kernel only: workgroup t holds the 128-row query units t (waves
    // 0-3) and n - 1 - t (waves 4-7) of the n = ceil(Tq / 128) instead of 256
    // consecutive rows, so that under causal order every workgroup has about
    // the same number of allowed pairs (for a launch whose workgroups all run
    // at once, where the heaviest one sets the launch time)
    int paired;
};

// One query block of a ring share against a sequence of key/value blocks in
// one launch (bf16, no window or ALiBi): the blocks are visited in the given
// order and each block's partial (out, lse) is written to or merged into the
// float32 out / lse of FwdParams exactly as by one attn_fwd launch per block.
// At most kMaxChain blocks per launch: measured on the 128K share, chains of
// 4 were 0.7% faster than one launch per block and chains of 16 6% slower.
constexpr int kMaxChain = 16;
struct ChainBlock {
    const void* k;             // (rotated) keys and values of the block: row 0 = the block's first key,
    const void* v;             // batch stride and row stride those of FwdParams
    const uint8_t* kpm;        // key-padding row of batch 0 at the block's first key, or null
    const int* kpm_list;       // live-tile list of the block (as FwdParams.kpm_list, rows of
                               // ceil(Tkv / 64) + 2 entries per batch row), or null
    long long kv_off;          // absolute position of the block's first key
    int Tkv;                   // keys in the block
    int accumulate;            // the first block: 0 = the launch writes its partial, 1 = merges it into
                               // out / lse (later blocks of a launch continue the same softmax state)
};
struct ChainParams {
    FwdParams p;               // q (rotated), out (float32 accumulator), lse, strides, B, H, Tq, q_off, causal, flags
    uint16_t* out_bf16;        // null, or the final bf16 output (the layout of out): the launch merges and
                               // writes there instead of into out
    int nblk;
    ChainBlock blk[kMaxChain];
};

// One attention backward launch (bf16 inputs, float32 outputs).  q and k are
// the operands as the forward multiplied them (rotated when RoPE is on); the
// gradients dq and dk come out in that rotated frame.  Strides in elements.
struct BwdParams {
    const void* q;             // (B, Tq, H, d)
    const void* k;             // (B, Tkv, H, d)
    const void* v;
    const void* dout;          // (B, Tq, H, d)
    const float2* ld2;         // (B, H, Tq): (lse * log2 e, or +inf for a row with no allowed key; delta)
    float* dq;                 // (B, Tq, H, d) float32
    float* dk;                 // (B, Tkv, H, d) float32
    float* dv;
    const uint8_t* kpm;
    const uint8_t* amask;
    const int* kpm_list;       // live key tiles (dq kernel), as for the forward, or null
    long long q_bstride, kv_bstride, kpm_bstride, lse_bstride;
    int row_stride;            // H * d
    int lse_hstride;
    int amask_stride;
    int kpm_list_stride;
    int B, H, Tq, Tkv;
    long long q_off, kv_off;
    int causal;
    unsigned flags;            // ATTN_ACCUMULATE: add into dq / dk / dv; ATTN_NO_TILE_SKIP
    float scale_log2;          // log2(e) / sqrt(d)
    float scale;               // 1 / sqrt(d)
    int n_tiles;               // query tiles (dq kernel) or key tiles (dk/dv kernel) per (b, h)
    long long win_left, win_right;   // sliding window as in FwdParams; -1 = no limit
    const float* alibi;        // [H] slopes or null
    float sqrt_d;
    // dK/dV kernel: when set, the final bf16 gradients of a key block no other
    // call adds to ((B, Tkv, H, d), strides of k), written instead of dk / dv:
    // dv rounded once, dk rotated back by R(-pos) with the float64 (cos, sin)
    // rows of dk_rope (row j at key j, or null without RoPE) and rounded once
    uint16_t* dk_out;
    uint16_t* dv_out;
    const double2* dk_rope;
};

// Entry of a live-tile list: tile index, top bit set when no key of the tile is masked.
constexpr uint32_t kTileClean = 0x80000000u;

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (`done` holds one bit per device id below 64; higher ids set it
// on every call).  Concurrent first calls may both set it, which is harmless.
inline hipError_t set_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// Kernel launchers (each returns hipSuccess or the launch error).
// One decoding call: the newest query of each (batch, head) against the
// filled slots of a static cache, split into chunks of CH slots.
struct DecodeParams {
    const void* q;             // (B, H, d)
    const void* k;             // (B, Tcap, H, d), keys stored rotated
    const void* v;
    const int* cache_len;      // [B] filled slots; the query sits at position cache_len[b] - 1
    void* out;                 // (B, H, d)
    float* lse;                // (B, H) or null
    float* part_o;             // (B, H, n_chunks, d) partial outputs (normalised)
    float* part_lse;           // (B, H, n_chunks)
    const float* alibi;        // [H] slopes or null
    int B, H, Tcap, CH, n_chunks;
    long long win_left;        // -1: every filled slot
    double log_base;           // ln(rope base), or 0: no rotation of the query
    float scale_log2;          // log2(e) / sqrt(d)
    float sqrt_d;
};

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_fwd_bf16_chain(const ChainParams& c, int d, hipStream_t s);
// Decoding splits each row's slots into chunks of a multiple of the keys one
// workgroup iteration covers: (64 lanes / lanes per key row) key groups per
// wave x kDecodeWaves waves x kDecodeUnroll keys per group.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeUnroll = 4;
long long decode_chunk_size(long long Tcap, long long bh, int d, int is_bf16);   // host code (api.hip)
hipError_t launch_decode_chunks(const DecodeParams& p, int d, int is_bf16, hipStream_t s);
// The per-device static workspace of attn_decode_noalloc (kDecodeStaticBytes
// bytes): its device address on the current device (looked up on the first
// call per device, no allocation).
constexpr size_t kDecodeStaticBytes = size_t(16) << 20;
hipError_t decode_static_workspace(void** ptr);
hipError_t launch_decode_merge(const DecodeParams& p, int d, int out_bf16, hipStream_t s);
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, int* cache_len, int B,
                            int H, int Tcap, int d, double log_base, int is_bf16, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_rope_table(double2* tab, long long pos0, int n, int d, double log_base, hipStream_t s);
hipError_t launch_kpm_tiles(const uint8_t* kpm, long long kpm_bstride, int B, int Tkv, int tile,
                            int* list, int list_stride, hipStream_t s);
hipError_t launch_merge(float* oa, float* la, const void* ob, const float* lb, int B, int H, int Tq, int d,
                        long long o_bstride, int row_stride, long long lse_bstride, int lse_hstride,
                        int b_is_bf16, hipStream_t s);
hipError_t launch_cast(const float* src, void* dst, long long n, int to_bf16, hipStream_t s);
hipError_t launch_rope_apply(void* x, const long long* pos, double log_base, int B, int T, int H, int d,
                             int is_bf16, hipStream_t s);
// One tensor of a rope_rotate launch: B x T tokens of H x d bf16 values;
// token t of a batch row sits at position t < split ? off0 + t : off1 + (t - split).
struct RopeJob {
    const void* src;
    void* dst;
    long long n_threads;       // B * T * (H / heads per thread) * (d / 8); 0 = no work
    int T;
    int split;
    long long off0, off1;
};
inline RopeJob rope_job(const void* src, void* dst, int B, int T, int H, int d, int split, long long off0,
                        long long off1) {
    const int hpt = (H % 4 == 0) ? 4 : 1;   // heads per thread, as the launch picks them
    return RopeJob{src, dst, (long long)B * T * (H / hpt) * (d / 8), T, split, off0, off1};
}
// Rotary copies of jobs a and b (same H and d) in one launch, with the (cos, sin)
// values computed in the kernel: no table needed.
hipError_t launch_rope_rotate_bf16(const RopeJob& a, const RopeJob& b, int H, int d, double log_base, hipStream_t s);
hipError_t launch_rope_copy_bf16(const void* src, void* dst, const double2* tab, int B, int T, int H, int d,
                                 hipStream_t s);
// The same with row t taking table row t + off0 for t < split, else
// t - split + off1.
hipError_t launch_rope_copy_bf16(const void* src, void* dst, const double2* tab, int B, int T, int H, int d,
                                 int split, long long off0, long long off1, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t s);
// ld2[b][h][i] = (lse * log2 e or +inf when lse = -inf, sum_c dout * out) for bf16 dout, out.
hipError_t launch_bwd_delta(const void* dout, const void* out, const float* lse, float2* ld2, int B, int H, int Tq,
                            int d, long long bstride, int row_stride, long long lse_bstride, int lse_hstride,
                            hipStream_t s);
// dst (float32 or bf16, optionally += ) = src rotated back by -pos (tab: cos/sin of +pos, or null for no
// rotation); src, dst (B, T, H, d) with batch strides in elements.
hipError_t launch_bwd_finalize(const float* src, void* dst, const double2* tab, int B, int T, int H, int d,
                               long long src_bstride, long long dst_bstride, int dst_bf16, int accumulate,
                               hipStream_t s);
hipError_t launch_zero_f32(float* x, long long n, hipStream_t s);
hipError_t launch_fill_empty(void* out, int out_bf16, float* lse, int B, int H, int rows, int d, long long o_bstride,
                             int row_stride, long long lse_bstride, int lse_hstride, hipStream_t s);

}  // namespace bosa
