// Decoding over a static key/value cache: append the new token's key and
// value, then attend with its query over every retained slot.
//
// Method ("Transformers and Attention" #53, causal key/value caching): at
// step t the new token's key and value are appended to the layer's cache and
// its query attends over the retained and current keys and values; #57: a
// static cache preallocates its slots and masks the unused ones.  The
// attention itself is the same blockwise online softmax as the forward
// kernels, split over the keys: one workgroup per (batch, head, chunk of
// slots) folds its chunk into a partial (out, lse), and a second kernel
// merges the partials of a row (the LogSumExp combination of the
// brunomaga.github.io post, "Improving numerical stability").
//
// Mapping.  With one query per (batch, head) the work is a matrix-vector
// product bound by HBM traffic (each cached key and value row is read once),
// not by the matrix cores.  A key row of d elements is read by a group of
// d * size / 16 lanes with one 16-byte load each; the group's partial dot
// products are summed with lane exchanges; each group keeps its own running
// max, denominator and output slice, and the groups of a workgroup are
// combined through LDS at the end.  Four keys per group are in flight per
// iteration, loaded non-temporally (each row is read once).
#include "common.h"

namespace bosa {
namespace {

constexpr int DW = kDecodeWaves;    // waves per decode workgroup
constexpr int DT = 64 * DW;         // threads
constexpr int DU = kDecodeUnroll;   // keys per group per iteration
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

template <typename T>
struct Elt;
template <>
struct Elt<uint16_t> {       // bf16
    static constexpr int EPL = 8;
    static __device__ __forceinline__ void load(const uint4& u, float (&x)[8]) {
        x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
        x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
    }
};
template <>
struct Elt<float> {
    static constexpr int EPL = 4;
    static __device__ __forceinline__ void load(const uint4& u, float (&x)[4]) {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    }
};

// Slots [c0, c1) of chunk `chunk` that the row's query sees: the filled slots
// [0, L) cut by the window to [L - 1 - window_left, L).
__device__ __forceinline__ void chunk_range(int L, long long win_left, int chunk, int CH, int& c0, int& c1) {
    int lo = 0;
    if (win_left >= 0) {
        const long long x = (long long)(L - 1) - win_left;
        lo = x > 0 ? (int)x : 0;
    }
    c0 = max(lo, chunk * CH);
    c1 = min(L, (chunk + 1) * CH);
}

template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(DT) void decode_chunk_kernel(const DecodeParams p) {
    using E = Elt<T>;
    constexpr int EPL = E::EPL;
    constexpr int LPK = D / EPL;         // lanes per key row
    constexpr int GPW = 64 / LPK;        // key groups per wave
    constexpr int NG = GPW * DW;         // key groups per workgroup
    __shared__ float red[NG][D + 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = (tid >> 6) * GPW + lane / LPK;   // key group
    const int sl = lane % LPK;                     // slice of the row: elements sl*EPL ..
    const int chunk = blockIdx.x % p.n_chunks;
    const int bh = blockIdx.x / p.n_chunks;
    const int h = bh % p.H, b = bh / p.H;
    int L = p.cache_len[b];
    L = L < 0 ? 0 : (L > p.Tcap ? p.Tcap : L);
    int c0, c1;
    chunk_range(L, p.win_left, chunk, p.CH, c0, c1);
    if (c0 >= c1) return;   // the merge skips chunks with no visible slot
    const long long pos = L - 1;

    // query slice, rotated to its position and rounded to the input dtype
    float q[EPL];
    {
        const T* qp = (const T*)p.q + ((long long)b * p.H + h) * D + sl * EPL;
        E::load(*(const uint4*)qp, q);
        if (p.log_base > 0.0) {
#pragma unroll
            for (int e = 0; e < EPL; e += 2) {
                const double2 cs = rope_cs64(pos, (sl * EPL + e) / 2, D, p.log_base);
                const double2 y = rot64((double)q[e], (double)q[e + 1], cs.x, cs.y);
                if (sizeof(T) == 2) {
                    const uint32_t r = bf16_bits_rn(y.x) | (bf16_bits_rn(y.y) << 16);
                    q[e] = bf16_lo(r);
                    q[e + 1] = bf16_hi(r);
                } else {
                    q[e] = (float)y.x;
                    q[e + 1] = (float)y.y;
                }
            }
        }
    }
    const float sl2 = p.scale_log2;
    const float ab = ALIBI ? -p.alibi[h] * p.sqrt_d : 0.f;
    const long long rs = (long long)p.H * D;                 // elements between slots
    const T* kb = (const T*)p.k + (long long)b * p.Tcap * rs + (long long)h * D + sl * EPL;
    const T* vb = (const T*)p.v + (long long)b * p.Tcap * rs + (long long)h * D + sl * EPL;

    float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    for (int j0 = c0 + g; j0 < c1; j0 += NG * DU) {
        uint4 ku[DU], vu[DU];
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            const int j = j0 + u * NG;
            ku[u] = vu[u] = make_uint4(0, 0, 0, 0);
            if (j < c1) {
                // each cached row is read once per step: non-temporal loads
                // keep it from displacing reused data in the caches
                const u32x4v a = __builtin_nontemporal_load((const u32x4v*)(kb + (long long)j * rs));
                const u32x4v c = __builtin_nontemporal_load((const u32x4v*)(vb + (long long)j * rs));
                ku[u] = make_uint4(a.x, a.y, a.z, a.w);
                vu[u] = make_uint4(c.x, c.y, c.z, c.w);
            }
        }
        float s[DU];
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            float kx[EPL];
            E::load(ku[u], kx);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc = fmaf(q[e], kx[e], acc);
#pragma unroll
            for (int off = LPK / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
            const int j = j0 + u * NG;
            if (ALIBI) acc = fmaf((float)(pos - j), ab, acc);   // the query is never before a filled slot
            s[u] = j < c1 ? acc * sl2 : -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int u = 1; u < DU; ++u) mx = fmaxf(mx, s[u]);
        const float mn = fmaxf(m, mx);   // finite: slot j0 < c1 is visible
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float ps = 0.f, pu[DU];
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            pu[u] = __builtin_amdgcn_exp2f(s[u] - mn);
            ps += pu[u];
        }
        l = fmaf(l, alpha, ps);
        m = mn;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            float vx[EPL];
            E::load(vu[u], vx);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = fmaf(pu[u], vx[e], o[e]);
        }
    }

    // combine the groups: red[g] = (o slice ..., m, l); a group that saw no
    // slot has m = -inf and contributes nothing
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[g][sl * EPL + e] = o[e];
    if (sl == 0) {
        red[g][D] = m;
        red[g][D + 1] = l;
    }
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
        for (int x = 0; x < NG; ++x) M = fmaxf(M, red[x][D]);
        float Ls = 0.f, O = 0.f;
        for (int x = 0; x < NG; ++x) {
            const float mx = red[x][D];
            if (mx == -INFINITY) continue;
            const float w = __builtin_amdgcn_exp2f(mx - M);
            Ls = fmaf(red[x][D + 1], w, Ls);
            O = fmaf(red[x][tid], w, O);
        }
        const long long slot = (long long)bh * p.n_chunks + chunk;
        p.part_o[slot * D + tid] = O / Ls;
        if (tid == 0) p.part_lse[slot] = (M + log2f(Ls)) * kLn2;
    }
}

// One workgroup of 128 threads per (batch, head): merge the partials of the
// visible chunks (lse = log-sum-exp of theirs, out = their weighted sum).
template <bool OUT_BF16>
__global__ __launch_bounds__(128) void decode_merge_kernel(const DecodeParams p, int D) {
    const int bh = blockIdx.x;
    const int b = bh / p.H;
    const int t = threadIdx.x;
    int L = p.cache_len[b];
    L = L < 0 ? 0 : (L > p.Tcap ? p.Tcap : L);
    int lo = 0;
    if (p.win_left >= 0) {
        const long long x = (long long)(L - 1) - p.win_left;
        lo = x > 0 ? (int)x : 0;
    }
    const int k0 = lo / p.CH, k1 = lo < L ? (L + p.CH - 1) / p.CH : k0;
    const long long base = (long long)bh * p.n_chunks;
    float M = -INFINITY;
    for (int c = k0; c < k1; ++c) M = fmaxf(M, p.part_lse[base + c]);
    float S = 0.f, O = 0.f;
    for (int c = k0; c < k1; ++c) {
        const float w = expf(p.part_lse[base + c] - M);
        S += w;
        if (t < D) O = fmaf(w, p.part_o[(base + c) * D + t], O);
    }
    const bool empty = k1 <= k0;
    if (t < D) {
        const float r = empty ? 0.f : O / S;
        const long long i = (long long)bh * D + t;
        if (OUT_BF16) ((uint16_t*)p.out)[i] = (uint16_t)(pack_bf16x2(r, 0.f) & 0xffffu);
        else ((float*)p.out)[i] = r;
    }
    if (t == 0 && p.lse) p.lse[bh] = empty ? -INFINITY : M + logf(S);
}

// Append: one workgroup per batch row writes the token into slot L =
// cache_len[b] (the key rotated to position L) and then advances cache_len[b].
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(const void* __restrict__ k_new, const void* __restrict__ v_new,
                                                        void* __restrict__ k_cache, void* __restrict__ v_cache,
                                                        int* __restrict__ cache_len, int H, int Tcap, int d,
                                                        double log_base) {
    const int b = blockIdx.x;
    const int L = cache_len[b];
    __syncthreads();   // every thread has read the length before it moves
    if (L < 0 || L >= Tcap) return;
    const long long row = (long long)H * d;
    const long long src = (long long)b * row;
    const long long dst = ((long long)b * Tcap + L) * row;
    for (long long i = 2 * threadIdx.x; i < row; i += 2 * blockDim.x) {
        const int t = (int)(i % d) / 2;   // coordinate pair within the head
        if (sizeof(T) == 2) {
            uint32_t u = *(const uint32_t*)((const uint16_t*)k_new + src + i);
            if (log_base > 0.0) {
                const double2 cs = rope_cs64(L, t, d, log_base);
                u = rot_pair_bf16(u, cs.x, cs.y);
            }
            *(uint32_t*)((uint16_t*)k_cache + dst + i) = u;
            *(uint32_t*)((uint16_t*)v_cache + dst + i) = *(const uint32_t*)((const uint16_t*)v_new + src + i);
        } else {
            float x0 = ((const float*)k_new)[src + i];
            float x1 = ((const float*)k_new)[src + i + 1];
            if (log_base > 0.0) {
                const double2 cs = rope_cs64(L, t, d, log_base);
                const float2 y = rot_pair_f32(x0, x1, cs.x, cs.y);
                x0 = y.x;
                x1 = y.y;
            }
            ((float*)k_cache)[dst + i] = x0;
            ((float*)k_cache)[dst + i + 1] = x1;
            ((float*)v_cache)[dst + i] = ((const float*)v_new)[src + i];
            ((float*)v_cache)[dst + i + 1] = ((const float*)v_new)[src + i + 1];
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) cache_len[b] = L + 1;
}

template <typename T, int D, bool ALIBI>
hipError_t launch_chunks(const DecodeParams& p, hipStream_t s) {
    const long long grid = (long long)p.B * p.H * p.n_chunks;
    hipLaunchKernelGGL((decode_chunk_kernel<T, D, ALIBI>), dim3((unsigned)grid), dim3(DT), 0, s, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_chunks_a(const DecodeParams& p, hipStream_t s) {
    return p.alibi ? launch_chunks<T, D, true>(p, s) : launch_chunks<T, D, false>(p, s);
}

}  // namespace

// Workspace of attn_decode_noalloc: the chunk partials of a call live here
// instead of in stream-ordered scratch.  One copy per device, kept for the
// life of the process; every call on a device uses (and overwrites) it.
static __device__ __align__(256) unsigned char scratch[kDecodeStaticBytes];

hipError_t decode_static_workspace(void** ptr) {
    // Device address of `scratch` on the current device, looked up once per
    // device.  In host code `scratch` names a host-side stand-in, so only the
    // address returned here may be handed to kernels.
    constexpr int kMaxDev = 64;
    static std::atomic<void*> addr[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    void* a = addr[dev].load(std::memory_order_acquire);
    if (!a) {
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev].store(a, std::memory_order_release);
    }
    *ptr = a;
    return hipSuccess;
}

hipError_t launch_decode_chunks(const DecodeParams& p, int d, int is_bf16, hipStream_t s) {
    if (is_bf16) return d == 128 ? launch_chunks_a<uint16_t, 128>(p, s) : launch_chunks_a<uint16_t, 64>(p, s);
    return d == 128 ? launch_chunks_a<float, 128>(p, s) : launch_chunks_a<float, 64>(p, s);
}

hipError_t launch_decode_merge(const DecodeParams& p, int d, int out_bf16, hipStream_t s) {
    const long long grid = (long long)p.B * p.H;
    if (out_bf16) hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((unsigned)grid), dim3(128), 0, s, p, d);
    else hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((unsigned)grid), dim3(128), 0, s, p, d);
    return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, int* cache_len, int B,
                            int H, int Tcap, int d, double log_base, int is_bf16, hipStream_t s) {
    if (is_bf16)
        hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(B), dim3(256), 0, s, k_new, v_new, k_cache, v_cache,
                           cache_len, H, Tcap, d, log_base);
    else
        hipLaunchKernelGGL(kv_append_kernel<float>, dim3(B), dim3(256), 0, s, k_new, v_new, k_cache, v_cache,
                           cache_len, H, Tcap, d, log_base);
    return hipGetLastError();
}

}  // namespace bosa
