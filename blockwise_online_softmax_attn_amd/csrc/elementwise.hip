// Bandwidth-bound helpers of the attention path: the rotary cos/sin table,
// the live key-tile list of a key-padding mask, the partial-result merge, the
// float32 -> output dtype cast, the standalone rotary embedding and the
// empty-row fill.  All are coalesced along the contiguous (H, d) axes.
#include "common.h"

namespace bosa {
namespace {

inline unsigned grid_for(long long n, int block) { return (unsigned)((n + block - 1) / block); }

// tab[i][t] = (cos, sin) of (pos0 + i) * base^(-2t/d) in float64, i < n, t < d/2.
__global__ void rope_table_kernel(double2* __restrict__ tab, long long pos0, int n, int d, double log_base) {
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int half = d / 2;
    if (idx >= (long long)n * half) return;
    const int i = (int)(idx / half), t = (int)(idx % half);
    tab[idx] = rope_cs64(pos0 + i, t, d, log_base);
}

// Classification of keys [k0, k1) under the key-padding mask (nonzero =
// masked): any_ok = some key allowed, all_ok = every key allowed.  Whole
// 16-byte granules are tested four bytes at a time when the row is aligned.
__device__ __forceinline__ bool word_has_zero_byte(uint32_t v) { return ((v - 0x01010101u) & ~v & 0x80808080u) != 0; }
__device__ __forceinline__ void classify(const uint8_t* row, int k0, int k1, bool& any_ok, bool& all_ok) {
    any_ok = false;
    all_ok = true;
    int k = k0;
    if ((((uintptr_t)(row + k)) & 15) == 0) {
        for (; k + 16 <= k1; k += 16) {
            const uint4 u = *(const uint4*)(row + k);
            any_ok |= word_has_zero_byte(u.x) || word_has_zero_byte(u.y) || word_has_zero_byte(u.z) ||
                      word_has_zero_byte(u.w);
            all_ok &= (u.x | u.y | u.z | u.w) == 0;
        }
    }
    for (; k < k1; ++k) {
        const bool ok = row[k] == 0;
        any_ok |= ok;
        all_ok &= ok;
    }
}

// One workgroup (4 waves) per batch row: list[0] = number of tiles with at
// least one allowed key, list[1] = number of leading tiles with no masked
// key, followed by the live tile indices in increasing order (top bit set
// when every key of the tile is allowed).  Fully masked tiles are skipped by
// the attention kernel without being read.  Thread i classifies a run of
// consecutive tiles; the runs' live counts are turned into write offsets by a
// scan over the workgroup (lane shuffles within a wave, LDS across waves).
__global__ __launch_bounds__(256) void kpm_tiles_kernel(const uint8_t* __restrict__ kpm, long long bstride, int Tkv,
                                                        int tile, int* __restrict__ list, int list_stride) {
    __shared__ int wave_sum[4];
    __shared__ int first_unclean;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint8_t* row = kpm + b * bstride;
    int* out = list + (long long)b * list_stride;
    const int ntk = (Tkv + tile - 1) / tile;
    const int per = (ntk + 255) / 256;
    const int t0 = min(tid * per, ntk), t1 = min(t0 + per, ntk);
    if (tid == 0) first_unclean = ntk;
    __syncthreads();
    int cnt = 0, unclean = ntk;
    for (int t = t0; t < t1; ++t) {
        bool any_ok, all_ok;
        classify(row, t * tile, min((t + 1) * tile, Tkv), any_ok, all_ok);
        cnt += any_ok ? 1 : 0;
        if (!all_ok && unclean == ntk) unclean = t;
    }
    if (unclean < ntk) atomicMin(&first_unclean, unclean);
    // inclusive scan of cnt within the wave, then across the four waves
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wave_sum[wv] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        before += i < wv ? wave_sum[i] : 0;
        total += wave_sum[i];
    }
    if (tid == 0) {
        out[0] = total;
        out[1] = first_unclean;
    }
    int pos = before + inc - cnt;
    for (int t = t0; t < t1; ++t) {
        bool any_ok, all_ok;
        classify(row, t * tile, min((t + 1) * tile, Tkv), any_ok, all_ok);
        if (any_ok) out[2 + pos++] = (int)((uint32_t)t | (all_ok ? kTileClean : 0u));
    }
}

// (out_a, lse_a) <- merge((out_a, lse_a), (out_b, lse_b)).  Each 32-lane half of
// a wave owns one (b, t, h) row, so the row's lse is read by every lane before
// lane 0 of the half writes the merged value.
template <bool B_BF16>
__global__ __launch_bounds__(256) void merge_kernel(float* __restrict__ oa, float* __restrict__ la,
                                                    const void* __restrict__ ob_, const float* __restrict__ lb,
                                                    int B, int H, int Tq, int d, long long o_bstride, int row_stride,
                                                    long long lse_bstride, int lse_hstride) {
    const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long rowid = gtid >> 5;
    const int sub = (int)(gtid & 31);
    if (rowid >= (long long)B * Tq * H) return;
    const int h = (int)(rowid % H);
    const long long bt = rowid / H;
    const int t = (int)(bt % Tq);
    const int b = (int)(bt / Tq);
    const long long lidx = b * lse_bstride + (long long)h * lse_hstride + t;
    const long long oidx = b * o_bstride + (long long)t * row_stride + (long long)h * d;
    float lse, wa, wb;
    merge_weights(la[lidx], lb[lidx], lse, wa, wb);
    for (int c = 4 * sub; c < d; c += 128) {
        float4* pa = (float4*)(oa + oidx + c);
        const float4 a = *pa;
        float4 bv;
        if (B_BF16) {
            const uint2 u = *(const uint2*)((const uint16_t*)ob_ + oidx + c);
            bv = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
        } else {
            bv = *(const float4*)((const float*)ob_ + oidx + c);
        }
        float4 r;
        r.x = merge_value(wa, a.x, wb, bv.x);
        r.y = merge_value(wa, a.y, wb, bv.y);
        r.z = merge_value(wa, a.z, wb, bv.z);
        r.w = merge_value(wa, a.w, wb, bv.w);
        *pa = r;
    }
    if (sub == 0) la[lidx] = lse;
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                        long long n) {
    const long long i4 = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 + 4 <= n) {
        const float4 x = *(const float4*)(src + i4);
        uint2 r;
        r.x = pack_bf16x2(x.x, x.y);
        r.y = pack_bf16x2(x.z, x.w);
        *(uint2*)(dst + i4) = r;
    } else {
        for (long long i = i4; i < n; ++i) dst[i] = (uint16_t)pack_bf16x2(src[i], 0.f);
    }
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                       long long n) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// Rotary embedding of one token (all heads of one batch item) per workgroup:
// the token's d/2 float64 (cos, sin) pairs are computed once in LDS; each pair
// is rotated in float64 and rounded once to the tensor's dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_apply_kernel(void* __restrict__ x, const long long* __restrict__ pos,
                                                         int T, int H, int d, double log_base) {
    __shared__ double2 cs[128];
    const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int half = d / 2;
    const long long ps = pos[i];
    for (int t = tid; t < half; t += blockDim.x) cs[t] = rope_cs64(ps, t, d, log_base);
    __syncthreads();
    const long long base = ((long long)b * T + i) * (long long)H * d;
    const int npairs = H * half;
    for (int pi = tid; pi < npairs; pi += blockDim.x) {
        const double2 c = cs[pi % half];
        if (BF16) {
            uint32_t* pp = (uint32_t*)((uint16_t*)x + base) + pi;
            *pp = rot_pair_bf16(*pp, c.x, c.y);
        } else {
            float2* pp = (float2*)((float*)x + base) + pi;
            const float2 v = *pp;
            *pp = rot_pair_f32(v.x, v.y, c.x, c.y);
        }
    }
}

// dst = src with the rotary embedding of its position applied to every head
// (bf16, [B][T][H][d] rows).  Row t takes table row t + off0 for t < split,
// else t - split + off1: a ring share's local queries are two runs of
// positions, all of them positions of the keys, so one table of (cos, sin)
// pairs over the keys' positions serves both.  The attention kernel then
// streams already-rotated operands; the arithmetic is rope_apply's (float64,
// one rounding), bit for bit.  A thread owns one 16-byte granule column
// (4 coordinate pairs) of one token in HPT heads, so each table entry it
// reads serves HPT granules.
template <int HPT>
__global__ __launch_bounds__(256) void rope_copy_bf16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                             const double2* __restrict__ tab, long long n_threads,
                                                             int T, int H, int gpr, int split, long long off0,
                                                             long long off1) {
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_threads) return;
    const int hs = H / HPT;                  // heads apart of this thread's granules
    const int tpt = hs * gpr;                // threads per token
    const long long tok = g / tpt;           // b * T + t
    const int r = (int)(g - tok * tpt);
    const int c = r % gpr, j = r / gpr;
    const int t = (int)(tok % T);
    const long long tr = t < split ? off0 + t : off1 + (t - split);
    const double2* tp = tab + tr * (4 * gpr) + 4 * c;
    const double2 c0 = tp[0], c1 = tp[1], c2 = tp[2], c3 = tp[3];
    const long long row0 = tok * H * gpr + c;
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
        const long long at = row0 + (long long)(j + k * hs) * gpr;
        const uint4 x = src[at];
        dst[at] = make_uint4(rot_pair_bf16(x.x, c0.x, c0.y), rot_pair_bf16(x.y, c1.x, c1.y),
                             rot_pair_bf16(x.z, c2.x, c2.y), rot_pair_bf16(x.w, c3.x, c3.y));
    }
}

// Rotary copies of up to two bf16 tensors in one launch (the keys and the
// queries of a call), each pair rotated in float64 and rounded once, with the
// float64 cos and sin of every (token, pair) a workgroup touches computed by
// that workgroup (rope_cs64, one evaluation each, shared through LDS) instead
// of read from a table: the values are the table's, bit for bit, and the
// table pass and its launch go away.  Workgroups [0, nblk0) serve job 0, the
// rest job 1.  Thread layout as rope_copy_bf16_kernel: a thread owns one
// 16-byte granule column (4 pairs) of one token in HPT heads.
template <int HPT>
__global__ __launch_bounds__(256) void rope_rotate_bf16_kernel(const RopeJob j0, const RopeJob j1, long long nblk0,
                                                               int H, int gpr, double log_base) {
    extern __shared__ double2 cs[];   // [token of the workgroup][pair]
    const bool second = (long long)blockIdx.x >= nblk0;
    const RopeJob& J = second ? j1 : j0;
    const long long g0 = ((long long)blockIdx.x - (second ? nblk0 : 0)) * 256;
    const int hs = H / HPT;
    const int tpt = hs * gpr;                // threads per token
    const int np = 4 * gpr;                  // pairs per token (d / 2)
    const long long tok0 = g0 / tpt;
    const long long ntok = J.n_threads / tpt;
    const long long tok1 = min((g0 + 255) / tpt, ntok - 1);
    const int nent = (int)(tok1 - tok0 + 1) * np;
    for (int e = threadIdx.x; e < nent; e += 256) {
        const long long tok = tok0 + e / np;
        const int t = (int)(tok % J.T);
        const long long pos = t < J.split ? J.off0 + t : J.off1 + (t - J.split);
        cs[e] = rope_cs64(pos, e % np, 2 * np, log_base);
    }
    __syncthreads();
    const long long g = g0 + threadIdx.x;
    if (g >= J.n_threads) return;
    const long long tok = g / tpt;
    const int r = (int)(g - tok * tpt);
    const int c = r % gpr, j = r / gpr;
    const double2* tp = cs + (tok - tok0) * np + 4 * c;
    const double2 c0 = tp[0], c1 = tp[1], c2 = tp[2], c3 = tp[3];
    const uint4* src = (const uint4*)J.src;
    uint4* dst = (uint4*)J.dst;
    const long long row0 = tok * H * gpr + c;
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
        const long long at = row0 + (long long)(j + k * hs) * gpr;
        const uint4 x = src[at];
        dst[at] = make_uint4(rot_pair_bf16(x.x, c0.x, c0.y), rot_pair_bf16(x.y, c1.x, c1.y),
                             rot_pair_bf16(x.z, c2.x, c2.y), rot_pair_bf16(x.w, c3.x, c3.y));
    }
}

// Rows [0, rows) become the merge identity: out = 0 (float32 or bf16), lse = -inf.
template <bool BF16>
__global__ __launch_bounds__(256) void fill_empty_kernel(void* __restrict__ out, float* __restrict__ lse, int B, int H,
                                                         int rows, int d, long long o_bstride, int row_stride,
                                                         long long lse_bstride, int lse_hstride) {
    const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)B * rows * H * d;
    if (gtid >= total) return;
    const int c = (int)(gtid % d);
    long long r = gtid / d;
    const int h = (int)(r % H);
    r /= H;
    const int t = (int)(r % rows);
    const int b = (int)(r / rows);
    if (out) {
        const long long oi = b * o_bstride + (long long)t * row_stride + (long long)h * d + c;
        if (BF16) ((uint16_t*)out)[oi] = 0;
        else ((float*)out)[oi] = 0.f;
    }
    if (lse && c == 0) lse[b * lse_bstride + (long long)h * lse_hstride + t] = -INFINITY;
}

}  // namespace

hipError_t launch_rope_table(double2* tab, long long pos0, int n, int d, double log_base, hipStream_t s) {
    const long long total = (long long)n * (d / 2);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, tab, pos0, n, d, log_base);
    return hipGetLastError();
}

hipError_t launch_kpm_tiles(const uint8_t* kpm, long long kpm_bstride, int B, int Tkv, int tile, int* list,
                            int list_stride, hipStream_t s) {
    hipLaunchKernelGGL(kpm_tiles_kernel, dim3(B), dim3(256), 0, s, kpm, kpm_bstride, Tkv, tile, list, list_stride);
    return hipGetLastError();
}

hipError_t launch_merge(float* oa, float* la, const void* ob, const float* lb, int B, int H, int Tq, int d,
                        long long o_bstride, int row_stride, long long lse_bstride, int lse_hstride, int b_is_bf16,
                        hipStream_t s) {
    const long long threads = (long long)B * Tq * H * 32;
    if (threads == 0) return hipSuccess;
    if (b_is_bf16)
        hipLaunchKernelGGL(merge_kernel<true>, dim3(grid_for(threads, 256)), dim3(256), 0, s, oa, la, ob, lb, B, H,
                           Tq, d, o_bstride, row_stride, lse_bstride, lse_hstride);
    else
        hipLaunchKernelGGL(merge_kernel<false>, dim3(grid_for(threads, 256)), dim3(256), 0, s, oa, la, ob, lb, B, H,
                           Tq, d, o_bstride, row_stride, lse_bstride, lse_hstride);
    return hipGetLastError();
}

hipError_t launch_cast(const float* src, void* dst, long long n, int to_bf16, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (to_bf16)
        hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for((n + 3) / 4, 256)), dim3(256), 0, s, src,
                           (uint16_t*)dst, n);
    else
        hipLaunchKernelGGL(copy_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, src, (float*)dst, n);
    return hipGetLastError();
}

hipError_t launch_rope_apply(void* x, const long long* pos, double log_base, int B, int T, int H, int d, int is_bf16,
                             hipStream_t s) {
    if ((long long)B * T == 0) return hipSuccess;
    if (is_bf16)
        hipLaunchKernelGGL(rope_apply_kernel<true>, dim3(T, B), dim3(256), 0, s, x, pos, T, H, d, log_base);
    else
        hipLaunchKernelGGL(rope_apply_kernel<false>, dim3(T, B), dim3(256), 0, s, x, pos, T, H, d, log_base);
    return hipGetLastError();
}

hipError_t launch_rope_copy_bf16(const void* src, void* dst, const double2* tab, int B, int T, int H, int d,
                                 int split, long long off0, long long off1, hipStream_t s) {
    const int gpr = d / 8;
    const int hpt = (H % 4 == 0) ? 4 : 1;
    const long long n = (long long)B * T * (H / hpt) * gpr;
    if (n == 0) return hipSuccess;
    if (hpt == 4)
        hipLaunchKernelGGL(rope_copy_bf16_kernel<4>, dim3(grid_for(n, 256)), dim3(256), 0, s, (const uint4*)src,
                           (uint4*)dst, tab, n, T, H, gpr, split, off0, off1);
    else
        hipLaunchKernelGGL(rope_copy_bf16_kernel<1>, dim3(grid_for(n, 256)), dim3(256), 0, s, (const uint4*)src,
                           (uint4*)dst, tab, n, T, H, gpr, split, off0, off1);
    return hipGetLastError();
}

hipError_t launch_rope_copy_bf16(const void* src, void* dst, const double2* tab, int B, int T, int H, int d,
                                 hipStream_t s) {
    return launch_rope_copy_bf16(src, dst, tab, B, T, H, d, T, 0, 0, s);
}

hipError_t launch_rope_rotate_bf16(const RopeJob& a, const RopeJob& b, int H, int d, double log_base, hipStream_t s) {
    const int gpr = d / 8;
    const int hpt = (H % 4 == 0) ? 4 : 1;
    const int tpt = (H / hpt) * gpr;
    const long long nb0 = (a.n_threads + 255) / 256, nb1 = (b.n_threads + 255) / 256;
    if (nb0 + nb1 == 0) return hipSuccess;
    // tokens a workgroup touches: at most 256 / tpt + 2, each d / 2 (cos, sin) pairs
    const size_t lds = (size_t)(256 / tpt + 2) * (d / 2) * sizeof(double2);
    if (hpt == 4)
        hipLaunchKernelGGL(rope_rotate_bf16_kernel<4>, dim3((unsigned)(nb0 + nb1)), dim3(256), lds, s, a, b, nb0, H, gpr,
                           log_base);
    else
        hipLaunchKernelGGL(rope_rotate_bf16_kernel<1>, dim3((unsigned)(nb0 + nb1)), dim3(256), lds, s, a, b, nb0, H, gpr,
                           log_base);
    return hipGetLastError();
}

hipError_t launch_fill_empty(void* out, int out_bf16, float* lse, int B, int H, int rows, int d, long long o_bstride,
                             int row_stride, long long lse_bstride, int lse_hstride, hipStream_t s) {
    const long long total = (long long)B * rows * H * d;
    if (total == 0) return hipSuccess;
    if (out_bf16)
        hipLaunchKernelGGL(fill_empty_kernel<true>, dim3(grid_for(total, 256)), dim3(256), 0, s, out, lse, B, H, rows,
                           d, o_bstride, row_stride, lse_bstride, lse_hstride);
    else
        hipLaunchKernelGGL(fill_empty_kernel<false>, dim3(grid_for(total, 256)), dim3(256), 0, s, out, lse, B, H, rows,
                           d, o_bstride, row_stride, lse_bstride, lse_hstride);
    return hipGetLastError();
}

}  // namespace bosa
