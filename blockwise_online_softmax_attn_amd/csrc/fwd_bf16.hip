// Blockwise online-softmax attention forward, bf16 inputs, gfx950 MFMA.
//
// Method: scores of one key tile at a time, a running row max, a running
// denominator and a rescaled weighted sum per query row (the safe-softmax
// accumulator update of the brunomaga.github.io sequence-context-parallelism
// post, section "Improving numerical stability"), then out = sum / denominator
// and lse = max + ln(denominator).
//
// Mapping to CDNA4.  A workgroup of 8 waves owns 256 query rows of one
// (batch, head); each wave owns 32 rows and keeps its Q operand in registers.
// The scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: in the accumulator a lane then holds one query
// (lane % 32) and 16 of the tile's 32 keys, so the row max and row sum are
// lane-local plus one exchange with lane ^ 32 (v_permlane32_swap).  The
// probabilities are rounded to bf16 in place and are directly the B operand
// of O^T += V^T P^T, whose A operand (V^T) is read from the row-major V tile
// with ds_read_b64_tr_b16; O^T stays in registers with the same lane = query
// layout, so the rescale by exp(m_old - m_new) is a per-lane scalar multiply.
// K and V tiles (64 keys) are double-buffered in LDS with padded rows
// (conflict-free MFMA operand reads at base + immediate offsets), staged
// through registers so the rotary embedding of K is applied on the way in.
// Tiles every row of the workgroup may see in full run without any masking
// code; the causal band, padded tails and masks go through a masked copy.
#include "common.h"

namespace bosa {
namespace {

constexpr int BN = 64;    // keys per tile
constexpr int NW = 8;     // waves per workgroup, 32 query rows each
constexpr int BM = 32 * NW;
constexpr int NT = 64 * NW;
// Lazy rescale: the reference max of a row moves only when a tile's row max
// exceeds it by more than this (log2 units), so probabilities stay <= 2^8
// and the O/l rescale is almost never executed.  The result is the same up to
// rounding for any reference.
constexpr float kTau = 8.f;

template <int D>
struct Geo {
    static constexpr int NC = D / 16;           // 16-wide d chunks of Q K^T
    static constexpr int NDB = D / 32;          // 32-row d blocks of O^T
    static constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    static constexpr int CH = BN * CPR / NT;    // chunks per thread per tile
    // Padded LDS rows: K rows step 16 bytes and V rows 64 bytes around the
    // 256-byte bank window, so the 16-lane ds_read_b128 groups of the K
    // operand and the 4-row groups of the transposed V reads hit distinct banks.
    static constexpr int KS = D + 8;            // K row stride (elements)
    static constexpr int VS = D + 32;           // V row stride (elements)
    static constexpr int KTILE = BN * KS;
    static constexpr int VTILE = BN * VS;
    static constexpr int LDS_BYTES = 2 * (KTILE + VTILE) * 2;
    static_assert(CH >= 1 && BN * CPR % NT == 0, "staging must divide evenly");
};

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
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

template <int D>
struct Staging {
    uint4 k[Geo<D>::CH];
    uint4 v[Geo<D>::CH];
    float4 t[Geo<D>::CH][2];
    int key0;   // first key of the staged tile
};

// Global -> registers for the key tile starting at key0.  The loads are
// unconditional (rows beyond Tkv read the last row instead), so that no wait
// for them is needed before the registers are consumed by stage_store; rows
// beyond Tkv are zeroed there.
template <int D>
__device__ __forceinline__ void stage_load(Staging<D>& st, const uint16_t* __restrict__ kg,
                                           const uint16_t* __restrict__ vg, const float2* __restrict__ tab,
                                           int key0, int Tkv, int rs, int tid) {
    using G = Geo<D>;
    st.key0 = key0;
#pragma unroll
    for (int i = 0; i < G::CH; ++i) {
        const int id = i * NT + tid;
        const int row = id / G::CPR, c = id % G::CPR;
        const int key = min(key0 + row, Tkv - 1);
        st.k[i] = *(const uint4*)(kg + (long long)key * rs + c * 8);
        st.v[i] = *(const uint4*)(vg + (long long)key * rs + c * 8);
        if (tab) {
            const float4* tp = (const float4*)(tab + (long long)key * (D / 2) + c * 4);
            st.t[i][0] = tp[0];
            st.t[i][1] = tp[1];
        }
    }
}

// Registers -> LDS buffer (rotary embedding of K applied here, rows beyond
// Tkv written as zeros).
template <int D>
__device__ __forceinline__ void stage_store(const Staging<D>& st, uint16_t* sK, uint16_t* sV, bool rope, int Tkv,
                                            int tid) {
    using G = Geo<D>;
#pragma unroll
    for (int i = 0; i < G::CH; ++i) {
        const int id = i * NT + tid;
        const int row = id / G::CPR, c = id % G::CPR;
        uint4 x = st.k[i];
        uint4 y = st.v[i];
        if (rope) x = rope8_bf16(x, st.t[i][0], st.t[i][1]);
        if (st.key0 + row >= Tkv) {
            x = make_uint4(0, 0, 0, 0);
            y = make_uint4(0, 0, 0, 0);
        }
        *(uint4*)(sK + row * G::KS + c * 8) = x;
        *(uint4*)(sV + row * G::VS + c * 8) = y;
    }
}

__device__ __forceinline__ s16x4 tr_read(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Exclusions of a tile that is not entirely allowed.  The key behind
// accumulator register r of the first (second) 32-key block has local index
// 8 (r / 4) + 4 hh + r % 4 (+ 32).  thr4 = largest allowed local index minus
// 4 hh (causal order and the key tail); kml = the tile's 64 key-padding
// allowed bits shifted right by 4 hh; am = attention-mask row of this lane's
// query at the tile's first key (shifted by 4 hh), or null.
struct TileMask {
    int thr4;
    uint64_t kml;
    const uint8_t* am;
};

// One key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void attend_tile(const uint16_t* __restrict__ Kl, const uint16_t* __restrict__ Vl,
                                            const bf16x8 (&qreg)[Geo<D>::NC], f32x16 (&o)[Geo<D>::NDB],
                                            float& m_i, float& l_i, float sl2, bool masked, const TileMask& mk) {
    using G = Geo<D>;
    // ---- S^T for keys [0, 32) and [32, 64) of the tile; K operand reads run
    // two chunks ahead of the MFMAs that consume them
    bf16x8 ka0[G::NC], ka1[G::NC];
    ka0[0] = *(const bf16x8*)(Kl);
    ka1[0] = *(const bf16x8*)(Kl + 32 * G::KS);
    ka0[1] = *(const bf16x8*)(Kl + 16);
    ka1[1] = *(const bf16x8*)(Kl + 32 * G::KS + 16);
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        if (c + 2 < G::NC) {
            ka0[c + 2] = *(const bf16x8*)(Kl + 16 * (c + 2));
            ka1[c + 2] = *(const bf16x8*)(Kl + 32 * G::KS + 16 * (c + 2));
        }
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0[c], qreg[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1[c], qreg[c], s1, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- exclusions (only tiles that are not entirely allowed)
    if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int b0 = 8 * (r >> 2) + (r & 3);
            bool ok0 = b0 <= mk.thr4 && ((mk.kml >> b0) & 1);
            bool ok1 = b0 + 32 <= mk.thr4 && ((mk.kml >> (b0 + 32)) & 1);
            if (mk.am) {
                ok0 = ok0 && mk.am[b0] == 0;
                ok1 = ok1 && mk.am[b0 + 32] == 0;
            }
            s0[r] = ok0 ? s0[r] : -INFINITY;
            s1[r] = ok1 ? s1[r] : -INFINITY;
        }
    }
    // ---- online softmax with a lazily moved reference max
    float mx = max3(s0[0], s1[0], s0[1]);
    mx = max3(mx, s1[1], s0[2]);
    mx = max3(mx, s1[2], s0[3]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = max3(mx, fmaxf(s1[r], s0[r + 1]), fmaxf(s0[r], s1[r + 1]));
    mx = max3(mx, s1[15], s0[15]);
    mx = xhalf_max(mx) * sl2;
    if (__ballot(mx > m_i + kTau)) {
        const float mnew = fmaxf(m_i, mx);
        const float a = (mnew == -INFINITY) ? 1.f : hw_exp2(m_i - mnew);
        l_i *= a;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) o[db] *= a;
        m_i = mnew;
    }
    const float nm = (m_i == -INFINITY) ? 0.f : -m_i;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        s0[r] = hw_exp2(fmaf(s0[r], sl2, nm));
        s1[r] = hw_exp2(fmaf(s1[r], sl2, nm));
        rs0 += s0[r];
        rs1 += s1[r];
    }
    l_i += rs0 + rs1;
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
    // ---- O^T += V^T P^T; transposed V reads run one d block ahead
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    auto v_load = [&](int db, int kc) -> bf16x8 {
        const uint16_t* p0 = Vl + (kc * 16) * G::VS + db * 32;
        const s16x4 r0 = tr_read(p0);
        const s16x4 r1 = tr_read(p0 + 8 * G::VS);
        const s16x8 a = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        return __builtin_bit_cast(bf16x8, a);
    };
    bf16x8 va[2][4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) va[0][kc] = v_load(0, kc);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        if (db + 1 < G::NDB) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) va[(db + 1) & 1][kc] = v_load(db + 1, kc);
        }
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db & 1][kc], pb[kc], o[db], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
}

template <int D>
__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_kernel(const FwdParams p) {
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* sK = (uint16_t*)smem;          // [2][KTILE]
    uint16_t* sV = sK + 2 * G::KTILE;        // [2][VTILE]

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
    const int Tq = p.Tq, Tkv = p.Tkv;
    const uint16_t* qg = (const uint16_t*)p.q + b * p.q_bstride + (long long)h * D;
    const uint16_t* kg = (const uint16_t*)p.k + b * p.kv_bstride + (long long)h * D;
    const uint16_t* vg = (const uint16_t*)p.v + b * p.kv_bstride + (long long)h * D;
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const bool rope = p.rope_q != nullptr;
    const bool causal = p.causal != 0;
    const float sl2 = p.scale_log2;

    const int q0 = qt * BM;
    const int qw0 = q0 + w * 32;
    const int qi = qw0 + l32;
    const bool qvalid = qi < Tq;
    const bool wvalid = qw0 < Tq;
    const int qwlast = min(qw0 + 31, Tq - 1);
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
    // Finish the Q loads here, so no wait for them is left inside the tile loop.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // ---- key tiles of this workgroup
    const int qlast = min(q0 + BM, Tq) - 1;
    long long nk = Tkv;
    if (causal && !noskip) {
        const long long lim = delta + qlast + 1;
        nk = lim < 0 ? 0 : (lim < nk ? lim : nk);
    }
    const int nt = (int)((nk + BN - 1) / BN);
    const int* klist = (p.kpm_list && !noskip) ? p.kpm_list + (long long)b * p.kpm_list_stride : nullptr;
    const int nlist = klist ? klist[0] : nt;
    // Leading tiles with every key allowed for every row of the workgroup.
    long long nfull = Tkv / BN;
    if (causal) {
        const long long lim = q0 + delta + 1;
        const long long f = lim < 0 ? 0 : lim / BN;
        nfull = f < nfull ? f : nfull;
    }
    if (klist) nfull = klist[1] < nfull ? klist[1] : nfull;
    if (noskip || p.amask || (p.kpm && !klist)) nfull = 0;
    const int n_full = (int)(nfull < nt ? nfull : nt);

    auto tile_at = [&](int i) -> int { return klist ? (int)((uint32_t)klist[2 + i] & ~kTileClean) : i; };
    auto clean_at = [&](int i) -> bool { return klist ? ((uint32_t)klist[2 + i] & kTileClean) != 0 : p.kpm == nullptr; };

    // per-lane LDS operand offsets (elements)
    const int k_off = l32 * G::KS + 8 * hh;
    const int jj = lane & 15, grp = lane >> 4;
    const int v_off = (4 * (grp >> 1) + (jj >> 2)) * G::VS + 16 * (grp & 1) + 4 * (jj & 3);
    const uint8_t* kpm_row = p.kpm ? p.kpm + b * p.kpm_bstride : nullptr;
    const uint8_t* am_row = (p.amask && qvalid) ? p.amask + (long long)qi * p.amask_stride : nullptr;

    float m_i = -INFINITY;   // reference max of scaled scores (log2 units)
    float l_i = 0.f;         // running denominator (this half-wave's keys)
    f32x16 o[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) o[db] = f32x16{};

    Staging<D> st;
    int ntiles = 0;
    if (nt > 0 && nlist > 0 && tile_at(0) < nt) {
        ntiles = 1;
        stage_load<D>(st, kg, vg, p.rope_k, tile_at(0) * BN, Tkv, rs, tid);
        stage_store<D>(st, sK, sV, rope, Tkv, tid);
    }
    __syncthreads();

    int buf = 0;
    for (int i = 0; i < ntiles; ++i) {
        const int t = tile_at(i);
        const bool more = (i + 1 < nlist) && tile_at(i + 1) < nt;
        if (more) {
            ntiles = i + 2;
            stage_load<D>(st, kg, vg, p.rope_k, tile_at(i + 1) * BN, Tkv, rs, tid);
        }
        const uint16_t* Kl = sK + buf * G::KTILE + k_off;
        const uint16_t* Vl = sV + buf * G::VTILE + v_off;
        const int key0 = t * BN;
        const bool full = i < n_full;
        if (full || (wvalid && !(causal && !noskip && (long long)key0 - qwlast > delta))) {
            TileMask mk{63, ~0ull, nullptr};
            if (!full) {
                long long thr = (long long)Tkv - key0 - 1;
                if (causal) {
                    const long long c = (long long)qi + delta - key0;
                    thr = c < thr ? c : thr;
                }
                mk.thr4 = (int)(thr < -1 ? -1 : (thr > 63 ? 63 : thr)) - 4 * hh;
                uint64_t km = ~0ull;
                if (kpm_row && !clean_at(i)) {
                    const bool okk = key0 + lane < Tkv && kpm_row[key0 + lane] == 0;
                    km = __ballot(okk);
                }
                mk.kml = km >> (4 * hh);
                mk.am = am_row ? am_row + key0 + 4 * hh : nullptr;
            }
            attend_tile<D>(Kl, Vl, qreg, o, m_i, l_i, sl2, !full, mk);
        }
        if (more) stage_store<D>(st, sK + (buf ^ 1) * G::KTILE, sV + (buf ^ 1) * G::VTILE, rope, Tkv, tid);
        __syncthreads();
        buf ^= 1;
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
