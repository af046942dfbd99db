// Blockwise online-softmax attention forward, float32 inputs.
//
// True float32 products and accumulation (no bf16 or reduced-precision
// operand rounding).  A workgroup of four waves owns 32 query rows; in each
// wave the two lanes of a pair (2i, 2i+1) share row i, each holding half of
// the (rotated) query and of the output accumulator in registers, and add
// their partial dot products with one lane exchange.  Key/value tiles of 32
// rows are staged in LDS by the whole workgroup; wave w folds keys
// 8w .. 8w + 7 of every tile into its own running max / denominator /
// weighted sum, the safe-softmax accumulator rescale of the
// brunomaga.github.io sequence-context-parallelism post ("Improving
// numerical stability"), and the four states are combined at the end in wave
// order.  The key -> wave assignment depends only on the key's position in its
// tile, so skipping tiles changes no bit.
#include "common.h"

namespace bosa {
namespace {

constexpr int BMF = 32;  // query rows per workgroup (two lanes per row in each wave)
constexpr int BNF = 32;  // keys per LDS tile
constexpr int SUB = 8;   // keys per online-softmax update: one group per wave and tile
constexpr int NWF = BNF / SUB;   // waves per workgroup

template <int D>
__global__ __launch_bounds__(64 * NWF, 2) void attn_fwd_f32_kernel(const FwdParams p) {
    constexpr int HD = D / 2;
    __shared__ float4 sKV[2 * BNF * D / 4];   // the K tile, then the V tile
    float4* sK = sKV;
    float4* sV = sKV + BNF * D / 4;
    static_assert((HD + 2) * 64 <= 2 * BNF * D, "one wave's state must fit in the tile buffers");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane & 1;

    int bid = blockIdx.x;
    const int qt = p.n_qtiles - 1 - bid % p.n_qtiles;
    bid /= p.n_qtiles;
    const int h = bid % p.H;
    const int b = bid / p.H;

    const int rs = p.row_stride;
    const float* qg = (const float*)p.q + b * p.q_bstride + (long long)h * D;
    const float* kg = (const float*)p.k + b * p.kv_bstride + (long long)h * D;
    const float* vg = (const float*)p.v + b * p.kv_bstride + (long long)h * D;
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const long long delta = p.q_off - p.kv_off;

    const int q0 = qt * BMF;
    const int qi = q0 + (lane >> 1);
    const bool qvalid = qi < p.Tq;
    const int c0 = half * HD;   // first dim this lane holds

    float q[HD];
    float o[HD];
#pragma unroll
    for (int c = 0; c < HD; c += 4) {
        float4 x = qvalid ? *(const float4*)(qg + (long long)qi * rs + c0 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (qvalid && p.rope_q) {
            const double2* cs = p.rope_q + (long long)qi * (D / 2) + (c0 + c) / 2;
            const float2 y0 = rot_pair_f32(x.x, x.y, cs[0].x, cs[0].y);
            const float2 y1 = rot_pair_f32(x.z, x.w, cs[1].x, cs[1].y);
            x = make_float4(y0.x, y0.y, y1.x, y1.y);
        }
        q[c] = x.x; q[c + 1] = x.y; q[c + 2] = x.z; q[c + 3] = x.w;
        o[c] = o[c + 1] = o[c + 2] = o[c + 3] = 0.f;
    }

    // keys some row of the workgroup may see: [klo, nk)
    const bool wl_on = p.win_left >= 0, wr_on = p.win_right >= 0;
    const int qlast = min(q0 + BMF, p.Tq) - 1;
    long long nk = p.Tkv, klo = 0;
    if (!noskip) {
        if (p.causal) nk = min(nk, delta + qlast + 1);
        if (wr_on) nk = min(nk, delta + qlast + p.win_right + 1);
        if (wl_on) klo = max(klo, delta + q0 - p.win_left);
    }
    const uint8_t* kpm_row = p.kpm ? p.kpm + b * p.kpm_bstride : nullptr;
    const float ab = p.alibi ? -p.alibi[h] * p.sqrt_d : 0.f;

    float m_i = -INFINITY, l_i = 0.f;
    for (long long key0 = klo / BNF * BNF; key0 < nk; key0 += BNF) {
        for (int idx = tid; idx < BNF * D / 4; idx += 64 * NWF) {
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const long long key = key0 + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < p.Tkv) {
                kx = *(const float4*)(kg + (long long)key * rs + 4 * c4);
                vx = *(const float4*)(vg + (long long)key * rs + 4 * c4);
                if (p.rope_k) {
                    const double2* cs = p.rope_k + (long long)key * (D / 2) + 2 * c4;
                    const float2 y0 = rot_pair_f32(kx.x, kx.y, cs[0].x, cs[0].y);
                    const float2 y1 = rot_pair_f32(kx.z, kx.w, cs[1].x, cs[1].y);
                    kx = make_float4(y0.x, y0.y, y1.x, y1.y);
                }
            }
            sK[idx] = kx;
            sV[idx] = vx;
        }
        __syncthreads();

        {
            const int j0 = w * SUB;   // this wave's keys of the tile
            float s[SUB];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                const float4* kr = sK + (j0 + j) * (D / 4) + c0 / 4;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < HD; c += 4) {
                    const float4 kx = kr[c / 4];
                    acc = fmaf(q[c], kx.x, acc);
                    acc = fmaf(q[c + 1], kx.y, acc);
                    acc = fmaf(q[c + 2], kx.z, acc);
                    acc = fmaf(q[c + 3], kx.w, acc);
                }
                // lane pair: the lower half's partial is added first on both lanes
                const float other = __shfl_xor(acc, 1);
                acc = half ? (other + acc) : (acc + other);
                const long long key = key0 + j0 + j;
                const long long rel = key - qi;   // key allowed by causal order iff rel <= delta
                bool ok = key < p.Tkv;
                if (ok && kpm_row) ok = kpm_row[key] == 0;
                if (ok && p.causal) ok = rel <= delta;
                if (ok && wr_on) ok = rel <= delta + p.win_right;
                if (ok && wl_on) ok = rel >= delta - p.win_left;
                if (ok && p.amask && qvalid) ok = p.amask[(long long)qi * p.amask_stride + key] == 0;
                if (ok && p.alibi) acc = fmaf(fabsf((float)(delta - rel)), ab, acc);
                s[j] = ok ? acc : -INFINITY;
                mx = fmaxf(mx, s[j]);
            }
            const float mnew = fmaxf(m_i, mx * p.scale_log2);
            const float muse = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m_i - muse);
            float rsum = 0.f;
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -muse));
                rsum += s[j];
            }
            l_i = fmaf(l_i, alpha, rsum);
            m_i = mnew;
#pragma unroll
            for (int c = 0; c < HD; ++c) o[c] *= alpha;
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                const float4* vr = sV + (j0 + j) * (D / 4) + c0 / 4;
#pragma unroll
                for (int c = 0; c < HD; c += 4) {
                    const float4 vx = vr[c / 4];
                    o[c] = fmaf(s[j], vx.x, o[c]);
                    o[c + 1] = fmaf(s[j], vx.y, o[c + 1]);
                    o[c + 2] = fmaf(s[j], vx.z, o[c + 2]);
                    o[c + 3] = fmaf(s[j], vx.w, o[c + 3]);
                }
            }
        }
        __syncthreads();
    }

    // combine the waves' states in wave order: wave u leaves its state in
    // the tile buffers (free after the loop's last barrier) and wave 0 folds
    // it in; every wave passes the same barriers
    float* xs = (float*)sKV;   // [HD + 2][64 lanes]
    for (int u = 1; u < NWF; ++u) {
        if (w == u) {
            xs[lane] = m_i;
            xs[64 + lane] = l_i;
#pragma unroll
            for (int c = 0; c < HD; ++c) xs[(2 + c) * 64 + lane] = o[c];
        }
        __syncthreads();
        if (w == 0) {
            const float mu = xs[lane], lu = xs[64 + lane];
            const float mn = fmaxf(m_i, mu);
            if (mn != -INFINITY) {   // else neither state has an allowed key yet
                const float a = __builtin_amdgcn_exp2f(m_i - mn), bu = __builtin_amdgcn_exp2f(mu - mn);
                l_i = fmaf(l_i, a, lu * bu);
#pragma unroll
                for (int c = 0; c < HD; ++c) o[c] = fmaf(o[c], a, xs[(2 + c) * 64 + lane] * bu);
                m_i = mn;
            }
        }
        __syncthreads();
    }
    if (w > 0) return;

    if (!qvalid) return;
    const float inv = l_i > 0.f ? 1.f / l_i : 0.f;
    const float lse_b = l_i > 0.f ? (m_i + log2f(l_i)) * kLn2 : -INFINITY;
    float* lse_ptr = p.lse ? p.lse + b * p.lse_bstride + (long long)h * p.lse_hstride + qi : nullptr;
    float* og = (float*)p.out + b * p.o_bstride + (long long)qi * rs + (long long)h * D + c0;
    if (p.flags & ATTN_ACCUMULATE) {
        const float la = *lse_ptr;   // both lanes of the pair read before the lower lane writes
        float lse_n, wa, wb;
        merge_weights(la, lse_b, lse_n, wa, wb);
#pragma unroll
        for (int c = 0; c < HD; c += 4) {
            float4 oa = *(float4*)(og + c);
            oa.x = merge_value(wa, oa.x, wb, o[c] * inv);
            oa.y = merge_value(wa, oa.y, wb, o[c + 1] * inv);
            oa.z = merge_value(wa, oa.z, wb, o[c + 2] * inv);
            oa.w = merge_value(wa, oa.w, wb, o[c + 3] * inv);
            *(float4*)(og + c) = oa;
        }
        if (!half) *lse_ptr = lse_n;
        return;
    }
#pragma unroll
    for (int c = 0; c < HD; c += 4)
        *(float4*)(og + c) = make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
    if (lse_ptr && !half) *lse_ptr = lse_b;
}

template <int D>
hipError_t launch(const FwdParams& p, hipStream_t s) {
    FwdParams q = p;
    q.n_qtiles = (p.Tq + BMF - 1) / BMF;
    const long long grid = (long long)q.n_qtiles * p.H * p.B;
    hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(64 * NWF), 0, s, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t s) {
    if (d == 128) return launch<128>(p, s);
    return launch<64>(p, s);
}

}  // namespace bosa
