// Blockwise online-softmax attention forward, bf16 inputs, gfx950 MFMA.
//
// Method: scores of one key tile at a time, a running row max, a running
// denominator and a rescaled weighted sum per query row (the safe-softmax
// accumulator update of the brunomaga.github.io sequence-context-parallelism
// post, section "Improving numerical stability"), then out = sum / denominator
// and lse = max + ln(denominator).
//
// Mapping to CDNA4.  A workgroup of 4 waves owns 128 query rows of one
// (batch, head); each wave owns 32 rows and keeps its Q operand in registers.
// The scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: in the accumulator a lane then holds one query
// (lane % 32) and 16 of the tile's 32 keys, so the row max and row sum are
// lane-local plus one exchange with lane ^ 32 (v_permlane32_swap).  The
// probabilities are rounded to bf16 in place and are directly the B operand
// of O^T += V^T P^T, whose A operand (V^T) is read from the row-major V tile
// with ds_read_b64_tr_b16; O^T stays in registers with the same lane = query
// layout, so the rescale by exp(m_old - m_new) is a per-lane scalar multiply.
// K and V tiles (64 keys) are double-buffered in LDS with XOR-swizzled 16-byte
// chunks (conflict-free MFMA operand reads), staged through registers so the
// rotary embedding of K is applied on the way in.
#include "common.h"

namespace bosa {
namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup (4 waves)

template <int D>
struct Geo {
    static constexpr int NC = D / 16;           // 16-wide d chunks of Q K^T
    static constexpr int NDB = D / 32;          // 32-row d blocks of O^T
    static constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    static constexpr int CH = BN * CPR / NT;    // chunks per thread per tile
    static constexpr int TILE = BN * D;         // elements of one K or V tile
    static constexpr int LDS_BYTES = 4 * TILE * 2;
};

// Swizzled 16-byte chunk position of chunk c in row r.
template <int D>
__device__ __forceinline__ int ksw(int r, int c) {
    if constexpr (D == 128) return c ^ (r & 15);
    else return c ^ ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vsw(int r, int c) {
    if constexpr (D == 128) return c ^ ((r & 3) << 2);
    else return c ^ (((r >> 1) & 1) << 2);
}

// Partner exchange between lane l and lane l ^ 32: both outputs of the swap
// hold {own value, partner value}.
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct Staging {
    uint4 k[Geo<D>::CH];
    uint4 v[Geo<D>::CH];
    float4 t[Geo<D>::CH][2];
};

// Global -> registers for key tile starting at key0 (rows beyond Tkv are zero).
template <int D>
__device__ __forceinline__ void stage_load(Staging<D>& st, const uint16_t* __restrict__ kg,
                                           const uint16_t* __restrict__ vg, const float2* __restrict__ tab,
                                           int key0, int Tkv, int rs, int tid) {
    using G = Geo<D>;
#pragma unroll
    for (int i = 0; i < G::CH; ++i) {
        const int id = i * NT + tid;
        const int row = id / G::CPR, c = id % G::CPR;
        const int key = key0 + row;
        if (key < Tkv) {
            st.k[i] = *(const uint4*)(kg + (long long)key * rs + c * 8);
            st.v[i] = *(const uint4*)(vg + (long long)key * rs + c * 8);
            if (tab) {
                const float4* tp = (const float4*)(tab + (long long)key * (D / 2) + c * 4);
                st.t[i][0] = tp[0];
                st.t[i][1] = tp[1];
            }
        } else {
            st.k[i] = make_uint4(0, 0, 0, 0);
            st.v[i] = make_uint4(0, 0, 0, 0);
            if (tab) {
                st.t[i][0] = make_float4(1.f, 0.f, 1.f, 0.f);
                st.t[i][1] = make_float4(1.f, 0.f, 1.f, 0.f);
            }
        }
    }
}

// Registers -> LDS buffer (rotary embedding of K applied here).
template <int D>
__device__ __forceinline__ void stage_store(const Staging<D>& st, uint16_t* sK, uint16_t* sV, bool rope, int tid) {
    using G = Geo<D>;
#pragma unroll
    for (int i = 0; i < G::CH; ++i) {
        const int id = i * NT + tid;
        const int row = id / G::CPR, c = id % G::CPR;
        uint4 x = st.k[i];
        if (rope) x = rope8_bf16(x, st.t[i][0], st.t[i][1]);
        *(uint4*)(sK + row * D + ksw<D>(row, c) * 8) = x;
        *(uint4*)(sV + row * D + vsw<D>(row, c) * 8) = st.v[i];
    }
}

// A operand of O^T += V^T P^T for d block db and key chunk (kb, cc): lane holds
// d = 32 db + lane % 32 and the 8 keys the S^T accumulator assigned to its
// half of the wave (see the P^T packing below).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const uint16_t* sVb, int kb, int cc, int db, int lane) {
    const int jj = lane & 15, grp = lane >> 4;
    const int row = kb * 32 + cc * 16 + 4 * (grp >> 1) + (jj >> 2);
    const int col = db * 32 + 16 * (grp & 1) + 4 * (jj & 3);
    const int c = col >> 3, e = col & 7;
    const uint16_t* p0 = sVb + row * D + vsw<D>(row, c) * 8 + e;
    const uint16_t* p1 = sVb + (row + 8) * D + vsw<D>(row + 8, c) * 8 + e;
    s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
    s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 a = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, a);
}

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(const FwdParams p) {
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* sK = (uint16_t*)smem;          // [2][TILE]
    uint16_t* sV = sK + 2 * G::TILE;         // [2][TILE]

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    // Heaviest query tiles (most keys under causal order) are dispatched first.
    int bid = blockIdx.x;
    const int qt = p.n_qtiles - 1 - bid % p.n_qtiles;
    bid /= p.n_qtiles;
    const int h = bid % p.H;
    const int b = bid / p.H;

    const int rs = p.row_stride;
    const uint16_t* qg = (const uint16_t*)p.q + b * p.q_bstride + (long long)h * D;
    const uint16_t* kg = (const uint16_t*)p.k + b * p.kv_bstride + (long long)h * D;
    const uint16_t* vg = (const uint16_t*)p.v + b * p.kv_bstride + (long long)h * D;
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const bool rope = p.rope_q != nullptr;

    const int q0 = qt * BM;
    const int qw0 = q0 + w * 32;
    const int qi = qw0 + l32;
    const bool qvalid = qi < p.Tq;
    const bool wvalid = qw0 < p.Tq;
    const int qwlast = min(qw0 + 31, p.Tq - 1);
    const long long delta = p.q_off - p.kv_off;   // key j allowed for query i iff j - i <= delta

    // ---- Q operand: lane holds query qi, d = 16c + 8hh + 0..7 for each chunk c.
    bf16x8 qreg[G::NC];
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qvalid) {
            x = *(const uint4*)(qg + (long long)qi * rs + 16 * c + 8 * hh);
            if (rope) {
                const float4* tp = (const float4*)(p.rope_q + (long long)qi * (D / 2) + 8 * c + 4 * hh);
                x = rope8_bf16(x, tp[0], tp[1]);
            }
        }
        qreg[c] = __builtin_bit_cast(bf16x8, x);
    }

    // ---- key range of this workgroup
    const int qlast = min(q0 + BM, p.Tq) - 1;
    long long nk = p.Tkv;
    if (p.causal && !noskip) {
        long long lim = delta + qlast + 1;
        nk = lim < 0 ? 0 : (lim < nk ? lim : nk);
    }
    const int nt = (int)((nk + BN - 1) / BN);

    const int* klist = p.kpm_list ? p.kpm_list + (long long)b * p.kpm_list_stride : nullptr;
    const int nlist = klist ? klist[0] : nt;
    const uint8_t* kpm_row = p.kpm ? p.kpm + b * p.kpm_bstride : nullptr;

    // Tile cursor: i-th visited tile and whether no key in it is padding-masked.
    auto fetch = [&](int i, int& t, bool& clean) -> bool {
        if (noskip || !klist) {
            t = i;
            clean = (p.kpm == nullptr);
            return i < nt;
        }
        if (i >= nlist) return false;
        const uint32_t e = (uint32_t)klist[1 + i];
        t = (int)(e & ~kTileClean);
        clean = (e & kTileClean) != 0;
        return t < nt;
    };

    float m_i = -INFINITY;   // running max of scaled scores (log2 units)
    float l_i = 0.f;         // running denominator (this half-wave's keys)
    f32x16 o[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) o[db] = f32x16{};

    Staging<D> st;
    int t;
    bool tclean;
    bool have = fetch(0, t, tclean);
    if (have) {
        stage_load<D>(st, kg, vg, p.rope_k, t * BN, p.Tkv, rs, tid);
        stage_store<D>(st, sK, sV, rope, tid);
    }
    __syncthreads();

    int buf = 0;
    for (int it = 0; have; ++it) {
        int tn;
        bool tnclean;
        const bool hn = fetch(it + 1, tn, tnclean);
        if (hn) stage_load<D>(st, kg, vg, p.rope_k, tn * BN, p.Tkv, rs, tid);

        const int key0 = t * BN;
        const bool wave_dead = !wvalid || (p.causal && !noskip && (long long)key0 - qwlast > delta);
        if (!wave_dead) {
            const uint16_t* Kb = sK + buf * G::TILE;
            const uint16_t* Vb = sV + buf * G::TILE;
            // ---- S^T = K Q^T for keys [key0, key0+32) and [key0+32, key0+64)
            f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
            for (int c = 0; c < G::NC; ++c) {
                const int ch = 2 * c + hh;
                const bf16x8 a0 = *(const bf16x8*)(Kb + l32 * D + ksw<D>(l32, ch) * 8);
                const bf16x8 a1 = *(const bf16x8*)(Kb + (32 + l32) * D + ksw<D>(32 + l32, ch) * 8);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[c], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[c], s1, 0, 0, 0);
            }
            // ---- exclusions: causal order, key padding, attention mask, tile tail
            const bool partial = noskip || !tclean || p.amask != nullptr || key0 + BN > p.Tkv ||
                                 (p.causal && (long long)(key0 + BN - 1) - qw0 > delta);
            if (partial) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        bool ok = key < p.Tkv;
                        if (ok && kpm_row) ok = kpm_row[key] == 0;
                        if (ok && p.causal) ok = (long long)key - qi <= delta;
                        if (ok && p.amask && qvalid) ok = p.amask[(long long)qi * p.amask_stride + key] == 0;
                        if (!ok) {
                            if (kb == 0) s0[r] = -INFINITY;
                            else s1[r] = -INFINITY;
                        }
                    }
                }
            }
            // ---- online softmax update
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
            mx = xhalf_max(mx);
            const float mnew = fmaxf(m_i, mx * p.scale_log2);
            const float muse = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = hw_exp2(m_i - muse);
            const float nm = -muse;
            float rsum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s0[r] = hw_exp2(fmaf(s0[r], p.scale_log2, nm));
                s1[r] = hw_exp2(fmaf(s1[r], p.scale_log2, nm));
                rsum += s0[r] + s1[r];
            }
            l_i = fmaf(l_i, alpha, rsum);
            m_i = mnew;
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < G::NDB; ++db) o[db] *= alpha;
            }
            // ---- P^T operands: chunk (kb, cc) = accumulator registers 8cc .. 8cc+7
            bf16x8 pb[4];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                uint4 u0, u1;
                u0.x = pack_bf16x2(s0[8 * cc + 0], s0[8 * cc + 1]);
                u0.y = pack_bf16x2(s0[8 * cc + 2], s0[8 * cc + 3]);
                u0.z = pack_bf16x2(s0[8 * cc + 4], s0[8 * cc + 5]);
                u0.w = pack_bf16x2(s0[8 * cc + 6], s0[8 * cc + 7]);
                u1.x = pack_bf16x2(s1[8 * cc + 0], s1[8 * cc + 1]);
                u1.y = pack_bf16x2(s1[8 * cc + 2], s1[8 * cc + 3]);
                u1.z = pack_bf16x2(s1[8 * cc + 4], s1[8 * cc + 5]);
                u1.w = pack_bf16x2(s1[8 * cc + 6], s1[8 * cc + 7]);
                pb[cc] = __builtin_bit_cast(bf16x8, u0);
                pb[2 + cc] = __builtin_bit_cast(bf16x8, u1);
            }
            // ---- O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    const bf16x8 a = v_operand<D>(Vb, kc >> 1, kc & 1, db, lane);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], o[db], 0, 0, 0);
                }
            }
        }

        if (hn) stage_store<D>(st, sK + (buf ^ 1) * G::TILE, sV + (buf ^ 1) * G::TILE, rope, tid);
        __syncthreads();
        buf ^= 1;
        t = tn;
        tclean = tnclean;
        have = hn;
    }

    // ---- epilogue: out = O / l, lse = ln(sum exp(scores)); optional merge into a partial
    const float lsum = xhalf_sum(l_i);
    if (!qvalid) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse_b = lsum > 0.f ? (m_i + log2f(lsum)) * kLn2 : -INFINITY;
    float* lse_ptr = p.lse ? p.lse + b * p.lse_bstride + (long long)h * p.lse_hstride + qi : nullptr;
    const long long orow = b * p.o_bstride + (long long)qi * rs + (long long)h * D;

    if (p.flags & ATTN_ACCUMULATE) {
        float* og = (float*)p.out + orow;
        const float la = *lse_ptr;
        float lse_n, wa, wb;
        merge_weights(la, lse_b, lse_n, wa, wb);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4* dst = (float4*)(og + db * 32 + 8 * g + 4 * hh);
                const float4 oa = *dst;
                float4 r;
                r.x = merge_value(wa, oa.x, wb, o[db][4 * g + 0] * inv);
                r.y = merge_value(wa, oa.y, wb, o[db][4 * g + 1] * inv);
                r.z = merge_value(wa, oa.z, wb, o[db][4 * g + 2] * inv);
                r.w = merge_value(wa, oa.w, wb, o[db][4 * g + 3] * inv);
                *dst = r;
            }
        }
        if (hh == 0) *lse_ptr = lse_n;
        return;
    }
    if (p.flags & ATTN_OUT_F32) {
        float* og = (float*)p.out + orow;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 r = make_float4(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                       o[db][4 * g + 3] * inv);
                *(float4*)(og + db * 32 + 8 * g + 4 * hh) = r;
            }
        }
    } else {
        uint16_t* og = (uint16_t*)p.out + orow;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 r;
                r.x = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
                r.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                *(uint2*)(og + db * 32 + 8 * g + 4 * hh) = r;
            }
        }
    }
    if (lse_ptr && hh == 0) *lse_ptr = lse_b;
}

template <int D>
hipError_t launch(const FwdParams& p, hipStream_t s) {
    using G = Geo<D>;
    static bool attr_set = false;  // the attribute is per function; setting it twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)attn_fwd_bf16_kernel<D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    FwdParams q = p;
    q.n_qtiles = (p.Tq + BM - 1) / BM;
    const long long grid = (long long)q.n_qtiles * p.H * p.B;
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<D>, dim3((unsigned)grid), dim3(NT), G::LDS_BYTES, s, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s) {
    if (d == 128) return launch<128>(p, s);
    return launch<64>(p, s);
}

}  // namespace bosa
