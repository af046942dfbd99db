// Blockwise attention backward, bf16 inputs, gfx950 MFMA.
//
// Method (brunomaga.github.io sequence-context-parallelism post, section
// "Ring Attention", item 3, and the backward pass of its "Implementation"):
// gradients are computed block by block from dout, the operands, the final
// out and the saved log-sum-exp, without the attention matrix.  With
// P = exp(s - lse) on allowed pairs and delta_i = sum_c dout_ic out_ic:
//   dv_j  = sum_i P_ij dout_i
//   dS_ij = P_ij (dout_i . v_j - delta_i)
//   dq_i  = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i
// (q, k rotated when RoPE is on; the caller rotates dq, dk back).
//
// Two kernels, so that every output element has one writer and the result is
// deterministic:
// * dQ: 8 waves x 32 query rows per workgroup, as in the forward kernel.
//   K tiles are read row-wise for S^T = K Q^T and transposed for
//   dQ^T += K^T dS^T, so each K tile is loaded twice, once per LDS swizzle;
//   the V tile serves dP^T = V dO^T.  Q and dO stay in registers.
// * dK/dV: 128 keys per workgroup, each 32-key block shared by two waves (one
//   computes P and dV, the other dP, dS and dK, with P passed through LDS);
//   K and V stay in registers as the B operands of S = Q K^T and dP = dO V^T;
//   32-query tiles of Q and dO (each twice, row-read and transposed
//   swizzles) and their (lse, delta) stream through LDS.  The accumulators
//   dK^T and dV^T keep lane = key.
// Tiles move HBM -> LDS with buffer loads in LDS mode (out-of-range rows
// arrive as zeros), as in the forward kernel.
#include "tile_io.h"

namespace bosa {
namespace {

template <int D>
struct BG {
    static constexpr int NC = D / 16;     // 16-wide d chunks (contraction over d)
    static constexpr int NDB = D / 32;    // 32-row d blocks of a transposed accumulator
    static constexpr int GPR = D / 8;     // 16-byte granules per row
    static constexpr int ROW = 2 * D;     // bytes per bf16 row in LDS
    static constexpr int RP = 256 / ROW;  // rows per 256-byte bank window
    static constexpr int RPB = 1024 / ROW;
    // Stored granule position = granule ^ h(row), one permutation for both
    // read patterns: it is a bijection on 16 consecutive bank windows (the
    // 16 rows of a 16-lane ds_read_b128 hit distinct banks) and gives the 4
    // rows of a transposed-read pass distinct groups of 4 granules.
    static __device__ __forceinline__ int h(int r) {
        const int w = r / RP;
        return 4 * (w % (GPR / 4)) + (w / (GPR / 4)) % 4;
    }
};

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Wait until at most n tiles of PT loads each are still in flight
// (0 <= n <= N; n is wave-uniform), then synchronise the workgroup.
template <int PT, int N>
__device__ __forceinline__ void wait_tiles(int n) {
    if constexpr (N == 0) {
        wait_barrier<0>();
    } else {
        if (n >= N) wait_barrier<N * PT>();
        else wait_tiles<PT, N - 1>(n);
    }
}

// A operand of a 32x32x16 MFMA holding the transpose of 16 rows x 32 columns
// of a row-major LDS tile (rows 16 kc .. 16 kc + 15, columns 32 db ..).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, uint2 voff_db, int kc) {
    const char* p0 = tile + (16 * kc) * BG<D>::ROW;
    const s16x4 r0 = tr_read(p0 + voff_db.x);
    const s16x4 r1 = tr_read(p0 + voff_db.y);
    const s16x8 a = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, a);
}

// Per-lane byte offsets of the transposed reads for each 32-column block
// (rows r0 and r0 + 8 of a 16-row chunk; the swizzle repeats every 16 rows),
// and of the row reads of granule 2c + hh of row lane % 32.
template <int D>
__device__ __forceinline__ void lane_offsets(int lane, uint32_t (&roff)[BG<D>::NC], uint2 (&toff)[BG<D>::NDB]) {
    using G = BG<D>;
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int c = 0; c < G::NC; ++c) roff[c] = l32 * G::ROW + 16 * ((2 * c + hh) ^ G::h(l32));
    const int jj = lane & 15, grp = lane >> 4;
    const int r0 = 4 * (grp >> 1) + (jj >> 2);
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        const int g = 4 * db + 2 * (grp & 1) + ((jj & 3) >> 1);
        toff[db].x = r0 * G::ROW + 16 * (g ^ G::h(r0)) + 8 * (jj & 1);
        toff[db].y = (r0 + 8) * G::ROW + 16 * (g ^ G::h(r0 + 8)) + 8 * (jj & 1);
    }
}

// Source offset (bytes, relative to the tile's first row) of the granule a
// lane moves into 1 KB block m of a tile.
template <int D>
__device__ __forceinline__ uint32_t dma_offset(int m, int lane, uint32_t rs2) {
    using G = BG<D>;
    const int row = m * G::RPB + lane / G::GPR;
    const int pos = lane % G::GPR;
    return (uint32_t)row * rs2 + 16u * (uint32_t)(pos ^ G::h(row));
}

// Packed bf16 operand from accumulator registers 8 cc .. 8 cc + 7.
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int cc) {
    uint4 u;
    u.x = pack_bf16x2(x[8 * cc + 0], x[8 * cc + 1]);
    u.y = pack_bf16x2(x[8 * cc + 2], x[8 * cc + 3]);
    u.z = pack_bf16x2(x[8 * cc + 4], x[8 * cc + 5]);
    u.w = pack_bf16x2(x[8 * cc + 6], x[8 * cc + 7]);
    return __builtin_bit_cast(bf16x8, u);
}

// Workgroup renumbering for the eight XCDs: workgroup b runs on XCD b % 8,
// and the result l gives the (batch row, head) pair l / nt and its tile
// l % nt (tiles heaviest first).  With a multiple of 8 pairs each XCD
// receives whole pairs (their tiles share its L2): a contiguous range of
// them, or, with `spread` (the pairs' work differs, as with a key-padding
// length per batch row), the pairs round-robin, so that one batch row's pairs
// are spread over all XCDs.  With any other pair count contiguous ranges
// would cut pairs into a heavy piece on one XCD and a light one on another;
// there workgroup b takes tile rank b / n of pair b % n (n pairs), every 8th
// tile of the list ordered heaviest first over all pairs.
__device__ __forceinline__ int xcd_order(int bid, int nt, bool spread) {
    const int npairs = (int)gridDim.x / nt;
    if (npairs & 7) return (bid % npairs) * nt + bid / npairs;
    if (spread) {
        const int k = bid >> 3;
        return ((k / nt) * 8 + (bid & 7)) * nt + k % nt;
    }
    return (bid & 7) * ((int)gridDim.x >> 3) + (bid >> 3);
}

// ============================================================== dQ
// VAR: a sliding window and/or ALiBi slopes (compile-time switch; without
// them every window term folds away).
template <int D, bool VAR>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const BwdParams p) {
    using G = BG<D>;
    constexpr int BN = 64, NW = 8, BM = 32 * NW, NSL = 4;
    constexpr int TILE = BN * G::ROW;        // bytes of one 64-row tile
    constexpr int SLOT = 2 * TILE;           // K | V (one swizzle serves row and transposed reads)
    constexpr int NI = TILE / 1024 / NW;     // 1 KB blocks per wave per tile copy
    constexpr int PT = 2 * NI;               // loads per wave per tile
    static_assert(NI >= 1 && (TILE / 1024) % NW == 0, "blocks must divide over the waves");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    int bid = xcd_order(blockIdx.x, p.n_tiles, p.kpm != nullptr && p.B > 1);
    const int qt = p.n_tiles - 1 - bid % p.n_tiles;   // heaviest causal query tiles first
    bid /= p.n_tiles;
    const int h = bid % p.H, b = bid / p.H;

    const int rs = p.row_stride;
    const uint32_t rs2 = 2u * (uint32_t)rs;
    const int Tq = p.Tq, Tkv = p.Tkv;
    const long long qrow0 = b * p.q_bstride + (long long)h * D;
    const char* kg = (const char*)((const uint16_t*)p.k + b * p.kv_bstride + (long long)h * D);
    const char* vg = (const char*)((const uint16_t*)p.v + b * p.kv_bstride + (long long)h * D);
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const bool causal = p.causal != 0;
    const float sl2 = p.scale_log2;
    const int q0 = qt * BM, qw0 = q0 + w * 32, qi = qw0 + l32;
    const bool qvalid = qi < Tq, wvalid = qw0 < Tq;
    const int qwlast = min(qw0 + 31, Tq - 1);
    const long long delta = p.q_off - p.kv_off;

    // Q and dO operands (B of S^T = K Q^T and dP^T = V dO^T): lane = query.
    bf16x8 qreg[G::NC], oreg[G::NC];
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
        if (qvalid) {
            const long long o = qrow0 + (long long)qi * rs + 16 * c + 8 * hh;
            x = *(const uint4*)((const uint16_t*)p.q + o);
            y = *(const uint4*)((const uint16_t*)p.dout + o);
        }
        qreg[c] = __builtin_bit_cast(bf16x8, x);
        oreg[c] = __builtin_bit_cast(bf16x8, y);
    }
    float2 ld = make_float2(INFINITY, 0.f);
    if (qvalid) ld = p.ld2[b * p.lse_bstride + (long long)h * p.lse_hstride + qi];
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): only tile loads are counted below

    // key tiles (as in the forward kernel): the keys some row of the
    // workgroup may see are [klo, khi)
    const bool wl_on = VAR && p.win_left >= 0, wr_on = VAR && p.win_right >= 0;
    const int qlast = min(q0 + BM, Tq) - 1;
    long long khi = Tkv, klo = 0;
    if (!noskip) {
        if (causal) khi = min(khi, delta + qlast + 1);
        if (wr_on) khi = min(khi, delta + qlast + p.win_right + 1);
        if (wl_on) klo = max(klo, delta + q0 - p.win_left);
    }
    khi = max(khi, 0LL);
    const int nt = (int)((khi + BN - 1) / BN);
    const int t_lo = klo >= khi ? nt : (int)(klo / BN);
    // tiles whose every key is allowed for every row: [tf_lo, tf_hi)
    long long kf_hi = Tkv, kf_lo = 0;
    if (causal) kf_hi = min(kf_hi, q0 + delta + 1);
    if (wr_on) kf_hi = min(kf_hi, q0 + delta + p.win_right + 1);
    if (wl_on) kf_lo = max(kf_lo, qlast + delta - p.win_left);
    const long long tf_lo = (kf_lo + BN - 1) / BN;
    const long long tf_hi = kf_hi < 0 ? 0 : kf_hi / BN;
    const bool force_mask = noskip || p.amask != nullptr || (p.kpm && !p.kpm_list);
    typedef const __attribute__((address_space(4))) int* cint_ptr;
    cint_ptr klist = (p.kpm_list && !noskip) ? (cint_ptr)(p.kpm_list + (long long)b * p.kpm_list_stride) : nullptr;
    int ntiles = nt - t_lo;
    if (klist) {
        auto first_at_least = [&](int t) {
            int lo = 0, hi = klist[0];
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((int)((uint32_t)klist[2 + mid] & ~kTileClean) < t) lo = mid + 1;
                else hi = mid;
            }
            return lo;
        };
        const int i0 = first_at_least(t_lo);
        ntiles = first_at_least(nt) - i0;
        klist += i0;
    }
    auto tile_at = [&](int i) -> int { return klist ? (int)((uint32_t)klist[2 + i] & ~kTileClean) : t_lo + i; };
    auto clean_at = [&](int i) -> bool { return klist ? ((uint32_t)klist[2 + i] & kTileClean) != 0 : p.kpm == nullptr; };
    int n_full = 0;   // without a window the entirely allowed tiles are the leading ones
    if constexpr (!VAR) {
        long long nf = tf_hi;
        if (klist) nf = min(nf, (long long)klist[1]);
        n_full = force_mask ? 0 : (int)min(nf, (long long)ntiles);
    }
    auto full_at = [&](int i) -> bool {
        if constexpr (!VAR) {
            return i < n_full;
        } else {
            const int t = tile_at(i);
            return !force_mask && t >= tf_lo && t < tf_hi && clean_at(i);
        }
    };
    auto first_tile_after = [&](long long key) {   // first list position whose tile starts after key
        int lo = 0, hi = ntiles;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((long long)tile_at(mid) * BN <= key) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    // tiles [w_first, n_act) hold allowed keys for some row of this wave
    int n_act = ntiles, w_first = 0;
    if (!wvalid) {
        n_act = 0;
    } else if (!noskip) {
        if (causal || wr_on) {
            long long lim = causal ? (long long)qwlast + delta : (long long)Tkv;
            if (wr_on) lim = min(lim, (long long)qwlast + delta + p.win_right);
            n_act = first_tile_after(lim);
        }
        if constexpr (VAR) {
            if (wl_on) w_first = first_tile_after(qw0 + delta - p.win_left - BN);
        }
    }
    const float ab = (VAR && p.alibi) ? -p.alibi[h] * p.sqrt_d : 0.f;

    uint32_t roff[G::NC];
    uint2 toff[G::NDB];
    lane_offsets<D>(lane, roff, toff);
    uint32_t dr[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) dr[n] = dma_offset<D>(w * NI + n, lane, rs2);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
    auto slot_of = [&](int i) -> int { return __builtin_amdgcn_readfirstlane(i % NSL); };
    auto issue = [&](int i) {
        const int key0 = tile_at(i) * BN;
        const uint32_t nb = (uint32_t)min(Tkv - 1 - key0, BN - 1) * rs2 + 2u * D;
        const u32x4 rk = buffer_rsrc(kg + (long long)key0 * rs2, nb);
        const u32x4 rv = buffer_rsrc(vg + (long long)key0 * rs2, nb);
        const uint32_t base = lds0 + (uint32_t)slot_of(i) * SLOT + (uint32_t)(w * NI) * 1024u;
#pragma unroll
        for (int n = 0; n < NI; ++n) load_lds16(dr[n], rk, base + 1024u * n);
#pragma unroll
        for (int n = 0; n < NI; ++n) load_lds16(dr[n], rv, base + TILE + 1024u * n);
    };
    const uint8_t* kpm_row = p.kpm ? p.kpm + b * p.kpm_bstride : nullptr;
    const uint8_t* am_row = (p.amask && qvalid) ? p.amask + (long long)qi * p.amask_stride : nullptr;
    auto tile_mask = [&](int i) -> TileMask {
        TileMask mk{63, ~0ull, nullptr};
        const int key0 = tile_at(i) * BN;
        long long thr = (long long)Tkv - key0 - 1;
        if (causal) thr = min(thr, (long long)qi + delta - key0);
        if (wr_on) thr = min(thr, (long long)qi + delta + p.win_right - key0);
        mk.thr4 = (int)(thr < -1 ? -1 : (thr > 63 ? 63 : thr)) - 4 * hh;
        if (wl_on) {
            const long long lo = (long long)qi + delta - p.win_left - key0;
            mk.lo4 = (int)(lo < -1 ? -1 : (lo > 64 ? 64 : lo)) - 4 * hh;
        }
        uint64_t km = ~0ull;
        if (kpm_row && !clean_at(i)) {
            const bool okk = key0 + lane < Tkv && kpm_row[key0 + lane] == 0;
            km = __ballot(okk);
        }
        mk.kml = km >> (4 * hh);
        mk.am = am_row ? am_row + key0 + 4 * hh : nullptr;
        return mk;
    };

    f32x16 acc[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) acc[db] = f32x16{};

    // tiles i + 1 .. i + NSL - 1 are loaded while tile i is processed
    for (int i = 0; i < NSL - 1 && i < ntiles; ++i) issue(i);
    wait_tiles<PT, NSL - 2>(min(NSL - 2, ntiles - 1));
    for (int i = 0; i < ntiles; ++i) {
        if (i + NSL - 1 < ntiles) issue(i + NSL - 1);
        if (i >= w_first && i < n_act) {
            const char* St = smem + slot_of(i) * SLOT;
            f32x16 s0 = f32x16{}, s1 = f32x16{}, d0 = f32x16{}, d1 = f32x16{};
#pragma unroll
            for (int c = 0; c < G::NC; ++c) {
                const bf16x8 k0 = *(const bf16x8*)(St + roff[c]);
                const bf16x8 k1 = *(const bf16x8*)(St + roff[c] + 32 * G::ROW);
                const bf16x8 v0 = *(const bf16x8*)(St + TILE + roff[c]);
                const bf16x8 v1 = *(const bf16x8*)(St + TILE + roff[c] + 32 * G::ROW);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qreg[c], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qreg[c], s1, 0, 0, 0);
                d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, oreg[c], d0, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, oreg[c], d1, 0, 0, 0);
            }
            if (!full_at(i)) apply_mask(s0, s1, tile_mask(i));
            if (VAR && p.alibi) add_alibi(s0, s1, (float)((long long)qi + delta - (long long)tile_at(i) * BN - 4 * hh), ab);
            // dS^T = P^T (dP^T - delta), P^T = exp2(s sl2 - lse2); lane = query
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p0 = hw_exp2(fmaf(s0[r], sl2, -ld.x));
                const float p1 = hw_exp2(fmaf(s1[r], sl2, -ld.x));
                s0[r] = p0 * (d0[r] - ld.y);
                s1[r] = p1 * (d1[r] - ld.y);
            }
            bf16x8 ds[4];
            ds[0] = pack8(s0, 0);
            ds[1] = pack8(s0, 1);
            ds[2] = pack8(s1, 0);
            ds[3] = pack8(s1, 1);
            // dQ^T += K^T dS^T: A = K^T from the transposed-swizzle copy
#pragma unroll
            for (int db = 0; db < G::NDB; ++db)
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(St, toff[db], kc), ds[kc],
                                                                      acc[db], 0, 0, 0);
        }
        // tile i + 1 resident for the next step
        wait_tiles<PT, NSL - 2>(min(i + NSL - 1, ntiles - 1) - (i + 1));
    }

    if (!qvalid) return;
    float* og = p.dq + b * p.q_bstride + (long long)qi * rs + (long long)h * D;
    const bool accum = (p.flags & ATTN_ACCUMULATE) != 0;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float4* dst = (float4*)(og + db * 32 + 8 * g + 4 * hh);
            float4 r = make_float4(acc[db][4 * g + 0] * p.scale, acc[db][4 * g + 1] * p.scale,
                                   acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
            if (accum) {
                const float4 a = *dst;
                r.x += a.x;
                r.y += a.y;
                r.z += a.z;
                r.w += a.w;
            }
            *dst = r;
        }
    }
}

// ============================================================== dK, dV
// 8 waves, 128 keys per workgroup.  The 32-key block kb = w % 4 is shared by
// two waves: wave A (w < 4) computes S = Q K^T, P and dV^T += dO^T P; wave B
// (w >= 4) computes dP = dO V^T, dS = P (dP - delta) and dK^T += Q^T dS,
// taking P (float32) from wave A through LDS.  Each wave holds one operand
// (K or V) and one accumulator (dV^T or dK^T), so two waves fit per SIMD;
// waves w and w + 4 share a SIMD, one of each role.  Wave B runs one query
// tile behind wave A: in loop step t, A works on tile t and B on tile t - 1,
// whose P A wrote in step t - 1 (two exchange buffers, by tile parity), so the
// one workgroup barrier that ends a step both publishes P and frees the tile
// slot B has finished with.
template <int D, bool VAR>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(const BwdParams p) {
    using G = BG<D>;
    constexpr int NW = 8, BK = 128, BQ = 32, NSL = 6;
    constexpr int QTILE = BQ * G::ROW;           // bytes of one 32-row tile
    constexpr int LDO = 2 * QTILE;               // lse2[32] then delta[32] of the tile after the two copies
    constexpr int SLOT = 2 * QTILE + 256;        // Q | dO | 32 x float2
    constexpr int XCH = NSL * SLOT;              // P exchange after the slots: 2 buffers x 4 blocks x 4 KB
    constexpr int NBLK = QTILE / 1024;           // 1 KB blocks per copy
    constexpr int PW = 2 * NBLK / NW;            // blocks per wave per tile (all in one copy)
    constexpr int PT = PW + 1;                   // loads per wave per tile
    static_assert(PW >= 1 && NBLK % PW == 0, "a wave's blocks must lie in one copy");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const bool roleA = w < 4;
    const int kb = w & 3;
    int bid = xcd_order(blockIdx.x, p.n_tiles, p.kpm != nullptr && p.B > 1);
    const int kt = bid % p.n_tiles;   // low key tiles see the most queries under causal order
    bid /= p.n_tiles;
    const int h = bid % p.H, b = bid / p.H;

    const int rs = p.row_stride;
    const uint32_t rs2 = 2u * (uint32_t)rs;
    const int Tq = p.Tq, Tkv = p.Tkv;
    const bool causal = p.causal != 0;
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const float sl2 = p.scale_log2;
    const long long delta = p.q_off - p.kv_off;   // key j allowed for query i iff j - i <= delta
    const int k0 = kt * BK, kw0 = k0 + 32 * kb, kj = kw0 + l32;
    const bool kvalid = kj < Tkv;
    const bool kmasked = p.kpm && kvalid && p.kpm[b * p.kpm_bstride + kj] != 0;

    // K (wave A) or V (wave B) operand, B of S = Q K^T or dP = dO V^T: lane = key.
    bf16x8 kv[G::NC];
    {
        const uint16_t* src = roleA ? (const uint16_t*)p.k : (const uint16_t*)p.v;
        const long long krow = b * p.kv_bstride + (long long)kj * rs + (long long)h * D;
#pragma unroll
        for (int c = 0; c < G::NC; ++c) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (kvalid) x = *(const uint4*)(src + krow + 16 * c + 8 * hh);
            kv[c] = __builtin_bit_cast(bf16x8, x);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Query tiles: [t0, t_end) for the workgroup, [tw0, tw_end) for this wave.
    // Key j pairs with queries lb(j) .. ub(j) (local indices): causal order
    // or the right edge of a window bound them below, the left edge above.
    const int nqt = (Tq + BQ - 1) / BQ;
    const bool wl_on = VAR && p.win_left >= 0, wr_on = VAR && p.win_right >= 0;
    auto lb = [&](long long j) -> long long {
        return causal ? j - delta : (wr_on ? j - delta - p.win_right : 0);
    };
    auto ub = [&](long long j) -> long long { return wl_on ? j - delta + p.win_left : (long long)Tq - 1; };
    auto tile_of = [&](long long i) -> int { return i <= 0 ? 0 : (i >= Tq ? nqt : (int)(i / BQ)); };
    auto tile_end = [&](long long i) -> int { return i < 0 ? 0 : (i >= Tq ? nqt : (int)(i / BQ) + 1); };
    const int t0 = noskip ? 0 : tile_of(lb(k0));
    const int t_end = (noskip || !wl_on) ? nqt : tile_end(ub((long long)k0 + BK - 1));
    const int tw0 = noskip ? 0 : tile_of(lb(kw0));
    const int tw_end = (noskip || !wl_on) ? nqt : tile_end(ub((long long)kw0 + 31));
    // tiles with every pair of this wave allowed: [tf, tf_hi), before the ragged tail
    int tf = 0, tf_hi = nqt;
    {
        const long long full = lb((long long)kw0 + 31);
        tf = full <= 0 ? 0 : (int)((full + BQ - 1) / BQ);
        if (wl_on) {
            const long long u = ub(kw0) + 1;
            tf_hi = u <= 0 ? 0 : (int)min((long long)nqt, u / BQ);
        }
        if (p.amask || noskip) tf = nqt;
    }
    const bool wactive = kw0 < Tkv;
    const int tail = Tq % BQ ? nqt - 1 : nqt;
    const float ab = (VAR && p.alibi) ? -p.alibi[h] * p.sqrt_d : 0.f;

    uint32_t roff[G::NC];
    uint2 toff[G::NDB];
    lane_offsets<D>(lane, roff, toff);
    // tile loads: this wave moves blocks PW*w .. PW*w+PW-1 of the 2 NBLK blocks
    // (copies: Q, dO)
    const int copy = (PW * w) / NBLK;
    const bool from_q = copy == 0;
    uint32_t dofs[PW];
#pragma unroll
    for (int n = 0; n < PW; ++n) dofs[n] = dma_offset<D>((PW * w + n) % NBLK, lane, rs2);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
    const char* srcg = (const char*)((const uint16_t*)(from_q ? p.q : p.dout) + b * p.q_bstride + (long long)h * D);
    const float2* ldg = p.ld2 + b * p.lse_bstride + (long long)h * p.lse_hstride;
    auto slot_of = [&](int t) -> int { return __builtin_amdgcn_readfirstlane(t % NSL); };
    auto issue = [&](int t) {
        const int qa = t * BQ;
        const uint32_t nb = (uint32_t)min(Tq - 1 - qa, BQ - 1) * rs2 + 2u * D;
        const u32x4 r = buffer_rsrc(srcg + (long long)qa * rs2, nb);
        const uint32_t slot = lds0 + (uint32_t)slot_of(t) * SLOT;
        const uint32_t base = slot + (uint32_t)copy * QTILE + (uint32_t)((PW * w) % NBLK) * 1024u;
#pragma unroll
        for (int n = 0; n < PW; ++n) load_lds16(dofs[n], r, base + 1024u * n);
        // (lse2, delta) of the 32 rows: 64 floats, 8 per wave
        const u32x4 rl = buffer_rsrc(ldg + qa, (uint32_t)min(Tq - qa, BQ) * 8u);
        // (rows of ld2 are float2 (lse2, delta); waves 0-3 move the lse2 of
        // rows 8w .. 8w + 7, waves 4-7 the delta of rows 8(w - 4) ..)
        if (lane < 8) load_lds4((uint32_t)(8 * (8 * (w & 3) + lane) + 4 * (w >> 2)), rl, slot + LDO + 32u * w);
    };
    // P exchange block of this key block in buffer par: [register group j][lane][4 floats]
    auto xch_of = [&](int par) -> float4* { return (float4*)(smem + XCH + 16384 * par + 4096 * kb) + lane; };

    f32x16 acc[G::NDB];   // dV^T (wave A) or dK^T (wave B); lane = key
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) acc[db] = f32x16{};

    const int ntl = t_end - t0;
    // Tile t is read by wave A in step t and by wave B in step t + 1; tiles
    // t + 1 .. t + NSL - 2 are loaded during step t, into the slot of tile
    // t - 2, which B finished with in step t - 1.
    for (int i = 0; i < NSL - 2 && i < ntl; ++i) issue(t0 + i);
    wait_tiles<PT, NSL - 3>(min(NSL - 3, ntl - 1));
    for (int t = t0; ntl > 0 && t <= t_end; ++t) {
        if (t + NSL - 2 < t_end) issue(t + NSL - 2);
        const int tt = roleA ? t : t - 1;   // this wave's tile
        const bool act = wactive && tt >= tw0 && tt < tw_end;   // for tile tt, the same for both waves of a key block
        const char* St = smem + slot_of(max(tt, 0)) * SLOT;
        float4* xch = xch_of(tt & 1);
        // lse2 (wave A) or delta (wave B) of this lane's query rows 8 j + 4 hh .. + 3
        const float4* lp = (const float4*)(St + LDO + (roleA ? 0 : 128));
        f32x16 x = f32x16{};   // S (wave A) or dP (wave B): lane = key, register r = query 8 (r/4) + 4 hh + r%4
        constexpr int NJ = 2 * G::NDB;
        bf16x8 ta[NJ];         // transposed operand of the second product (dO^T or Q^T)
        float4 lr[4];          // lse2 (wave A) or delta (wave B) of rows 8 j + 4 hh + (0 .. 3)
        if (act) {
            // every LDS operand of this tile is requested before the first
            // matrix instruction, so the reads overlap the products
            const char* rows = St + (roleA ? 0 : QTILE);   // Q or dO, row reads
            const char* trt = St + (roleA ? QTILE : 0);    // dO or Q, transposed reads
            bf16x8 ra[G::NC];
#pragma unroll
            for (int c = 0; c < G::NC; ++c) ra[c] = *(const bf16x8*)(rows + roff[c]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lr[j] = lp[2 * j + hh];
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) ta[j] = tr_operand<D>(trt, toff[j % G::NDB], j / G::NDB);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < G::NC; ++c) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[c], kv[c], x, 0, 0, 0);
            if (roleA) {
                if (VAR && p.alibi) {
                    // penalty ab |pos_q - pos_k| on every score of the tile
                    const float base = (float)((long long)tt * BQ + 4 * hh + delta - kj);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        x[r] = fmaf(fabsf(base + (float)(8 * (r >> 2) + (r & 3))), ab, x[r]);
                }
                if (tt < tf || tt >= tf_hi || tt >= tail) {
                    const int qa = tt * BQ;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qi = qa + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const long long rel = (long long)kj - qi;   // allowed by causal order iff rel <= delta
                        bool ok = qi < Tq && (!causal || rel <= delta);
                        if (wr_on) ok = ok && rel <= delta + p.win_right;
                        if (wl_on) ok = ok && rel >= delta - p.win_left;
                        if (p.amask && ok && kvalid) ok = p.amask[(long long)qi * p.amask_stride + kj] == 0;
                        x[r] = ok ? x[r] : -INFINITY;
                    }
                }
                // P = exp2(s sl2 - lse2) with the row's lse2
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[4 * j + 0] = hw_exp2(fmaf(x[4 * j + 0], sl2, -lr[j].x));
                    x[4 * j + 1] = hw_exp2(fmaf(x[4 * j + 1], sl2, -lr[j].y));
                    x[4 * j + 2] = hw_exp2(fmaf(x[4 * j + 2], sl2, -lr[j].z));
                    x[4 * j + 3] = hw_exp2(fmaf(x[4 * j + 3], sl2, -lr[j].w));
                    xch[64 * j] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
                }
            }
        }
        if (act) {
            if (!roleA) {
                // dS = P (dP - delta)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 pr = xch[64 * j];
                    x[4 * j + 0] = pr.x * (x[4 * j + 0] - lr[j].x);
                    x[4 * j + 1] = pr.y * (x[4 * j + 1] - lr[j].y);
                    x[4 * j + 2] = pr.z * (x[4 * j + 2] - lr[j].z);
                    x[4 * j + 3] = pr.w * (x[4 * j + 3] - lr[j].w);
                }
            }
            // dV^T += dO^T P (wave A) or dK^T += Q^T dS (wave B)
            const bf16x8 xb[2] = {pack8(x, 0), pack8(x, 1)};
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[j % G::NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[j], xb[j / G::NDB], acc[j % G::NDB], 0, 0, 0);
        }
        // tile t + 1 resident for A's next step (B's, tile t, already is); the
        // barrier also publishes this step's P
        wait_tiles<PT, NSL - 3>(min(t + NSL - 2, t_end - 1) - (t + 1));
    }

    if (!kvalid) return;
    // A key excluded by the key-padding mask gets exactly zero (its lane may
    // hold anything: its scores were not masked, since they reach no other key).
    const float sc = roleA ? 1.f : p.scale;
    uint16_t* fb = roleA ? p.dv_out : p.dk_out;
    if (fb) {
        // the final bf16 gradient: the float32 value as the float32 path
        // stores it, then (dk with RoPE) rotated back in float64, rounded once
        fb += b * p.kv_bstride + (long long)kj * rs + (long long)h * D;
        const double2* tr = (!roleA && p.dk_rope) ? p.dk_rope + (long long)kj * (D / 2) : nullptr;
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = db * 32 + 8 * g + 4 * hh;
                float4 r = make_float4(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc, acc[db][4 * g + 2] * sc,
                                       acc[db][4 * g + 3] * sc);
                if (kmasked) r = make_float4(0.f, 0.f, 0.f, 0.f);
                uint2 u;
                if (tr) {
                    const double2 ca = tr[c / 2], cb = tr[c / 2 + 1];
                    const double2 y0 = rot64(r.x, r.y, ca.x, -ca.y);
                    const double2 y1 = rot64(r.z, r.w, cb.x, -cb.y);
                    u = make_uint2(bf16_bits_rn(y0.x) | (bf16_bits_rn(y0.y) << 16),
                                   bf16_bits_rn(y1.x) | (bf16_bits_rn(y1.y) << 16));
                } else {
                    u = make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
                }
                *(uint2*)(fb + c) = u;
            }
        }
        return;
    }
    float* og = (roleA ? p.dv : p.dk) + b * p.kv_bstride + (long long)kj * rs + (long long)h * D;
    const bool accum = (p.flags & ATTN_ACCUMULATE) != 0;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float4* dst = (float4*)(og + db * 32 + 8 * g + 4 * hh);
            float4 r = make_float4(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc, acc[db][4 * g + 2] * sc,
                                   acc[db][4 * g + 3] * sc);
            if (kmasked) r = make_float4(0.f, 0.f, 0.f, 0.f);
            if (accum) {
                const float4 a = *dst;
                r.x += a.x;
                r.y += a.y;
                r.z += a.z;
                r.w += a.w;
            }
            *dst = r;
        }
    }
}

// ============================================================== helpers
// ld2 = (lse log2 e, or +inf for an empty row; delta = sum_c dout out): one
// 16-lane group per (row, head).
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ out,
                                                        const float* __restrict__ lse, float2* __restrict__ ld2, int B,
                                                        int H, int Tq, int d, long long bstride, int row_stride,
                                                        long long lse_bstride, int lse_hstride) {
    const long long gid = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 4;   // (b, t, h)
    const int sub = threadIdx.x & 15;
    const long long rows = (long long)B * Tq * H;
    if (gid >= rows) return;
    const int h = (int)(gid % H);
    const long long bt = gid / H;
    const int t = (int)(bt % Tq), b = (int)(bt / Tq);
    const long long base = b * bstride + (long long)t * row_stride + (long long)h * d;
    float acc = 0.f;
    for (int c = sub * 8; c < d; c += 128) {
        const uint4 x = *(const uint4*)(dout + base + c);
        const uint4 y = *(const uint4*)(out + base + c);
        acc = fmaf(bf16_lo(x.x), bf16_lo(y.x), acc);
        acc = fmaf(bf16_hi(x.x), bf16_hi(y.x), acc);
        acc = fmaf(bf16_lo(x.y), bf16_lo(y.y), acc);
        acc = fmaf(bf16_hi(x.y), bf16_hi(y.y), acc);
        acc = fmaf(bf16_lo(x.z), bf16_lo(y.z), acc);
        acc = fmaf(bf16_hi(x.z), bf16_hi(y.z), acc);
        acc = fmaf(bf16_lo(x.w), bf16_lo(y.w), acc);
        acc = fmaf(bf16_hi(x.w), bf16_hi(y.w), acc);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 16);
    if (sub == 0) {
        const long long li = b * lse_bstride + (long long)h * lse_hstride + t;
        const float l = lse[li];
        ld2[li] = make_float2(l == -INFINITY ? INFINITY : l * kLog2e, acc);
    }
}

// dst = (accumulate ? dst : 0) + R(-pos) src per coordinate pair, pos from
// the table row of the token (tab[t][pair] = float64 cos, sin of +pos); the
// rotation is formed in float64 and rounded once to the output dtype;
// tab == null: no rotation.  Workgroups walk the token rows (b, t) in a grid
// stride; each row's H * d values go four at a time (two pairs per thread
// step); d is 64 or 128.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const float* __restrict__ src, void* __restrict__ dst,
                                                           const double2* __restrict__ tab, long long rows, int T,
                                                           int H, int d, long long src_bstride, long long dst_bstride,
                                                           int accumulate) {
    const int n4 = H * d / 4;
    for (long long row = blockIdx.x; row < rows; row += gridDim.x) {
        const long long b = row / T;
        const int t = (int)(row - b * T);
        const float* sp = src + b * src_bstride + (long long)t * H * d;
        const long long doff = b * dst_bstride + (long long)t * H * d;
        const double2* tr = tab ? tab + (long long)t * (d / 2) : nullptr;
        for (int i = threadIdx.x; i < n4; i += blockDim.x) {
            const float4 x = ((const float4*)sp)[i];
            if (!tr) {
                // no rotation: the float32 value rounded once (the float64
                // path below gives the same bits, at several times the cost)
                if (BF16) {
                    ((uint2*)((uint16_t*)dst + doff))[i] = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
                } else {
                    float4* o = (float4*)((float*)dst + doff) + i;
                    float4 r = x;
                    if (accumulate) {
                        const float4 a = *o;
                        r.x += a.x;
                        r.y += a.y;
                        r.z += a.z;
                        r.w += a.w;
                    }
                    *o = r;
                }
                continue;
            }
            const double2 ca = tr[2 * (i & (d / 4 - 1))], cb = tr[2 * (i & (d / 4 - 1)) + 1];
            const double2 y0 = rot64(x.x, x.y, ca.x, -ca.y);
            const double2 y1 = rot64(x.z, x.w, cb.x, -cb.y);
            if (BF16) {
                ((uint2*)((uint16_t*)dst + doff))[i] =
                    make_uint2(bf16_bits_rn(y0.x) | (bf16_bits_rn(y0.y) << 16),
                               bf16_bits_rn(y1.x) | (bf16_bits_rn(y1.y) << 16));
            } else {
                float4* o = (float4*)((float*)dst + doff) + i;
                float4 r = make_float4((float)y0.x, (float)y0.y, (float)y1.x, (float)y1.y);
                if (accumulate) {
                    const float4 a = *o;
                    r.x += a.x;
                    r.y += a.y;
                    r.z += a.z;
                    r.w += a.w;
                }
                *o = r;
            }
        }
    }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ x, long long n4) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n4) x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

inline unsigned grid_for(long long n, int block) { return (unsigned)((n + block - 1) / block); }

template <int D, bool VAR>
hipError_t launch_dq(const BwdParams& p, hipStream_t s) {
    constexpr int BM = 256, LDS = 4 * 2 * 64 * 2 * D;
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = set_lds_limit((const void*)bwd_dq_kernel<D, VAR>, LDS, lds_set); e != hipSuccess) return e;
    BwdParams q = p;
    q.n_tiles = (p.Tq + BM - 1) / BM;
    const long long grid = (long long)q.n_tiles * p.H * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<D, VAR>), dim3((unsigned)grid), dim3(512), LDS, s, q);
    return hipGetLastError();
}

template <int D, bool VAR>
hipError_t launch_dkdv(const BwdParams& p, hipStream_t s) {
    constexpr int BK = 128, LDS = 6 * (2 * 32 * 2 * D + 256) + 2 * 4 * 4096;
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = set_lds_limit((const void*)bwd_dkdv_kernel<D, VAR>, LDS, lds_set); e != hipSuccess) return e;
    BwdParams q = p;
    q.n_tiles = (p.Tkv + BK - 1) / BK;
    const long long grid = (long long)q.n_tiles * p.H * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, VAR>), dim3((unsigned)grid), dim3(512), LDS, s, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t s) {
    const bool var = p.win_left >= 0 || p.win_right >= 0 || p.alibi;
    if (d == 128) return var ? launch_dq<128, true>(p, s) : launch_dq<128, false>(p, s);
    return var ? launch_dq<64, true>(p, s) : launch_dq<64, false>(p, s);
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t s) {
    const bool var = p.win_left >= 0 || p.win_right >= 0 || p.alibi;
    if (d == 128) return var ? launch_dkdv<128, true>(p, s) : launch_dkdv<128, false>(p, s);
    return var ? launch_dkdv<64, true>(p, s) : launch_dkdv<64, false>(p, s);
}

hipError_t launch_bwd_delta(const void* dout, const void* out, const float* lse, float2* ld2, int B, int H, int Tq,
                            int d, long long bstride, int row_stride, long long lse_bstride, int lse_hstride,
                            hipStream_t s) {
    const long long threads = (long long)B * Tq * H * 16;
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3(grid_for(threads, 256)), dim3(256), 0, s, (const uint16_t*)dout,
                       (const uint16_t*)out, lse, ld2, B, H, Tq, d, bstride, row_stride, lse_bstride, lse_hstride);
    return hipGetLastError();
}

hipError_t launch_bwd_finalize(const float* src, void* dst, const double2* tab, int B, int T, int H, int d,
                               long long src_bstride, long long dst_bstride, int dst_bf16, int accumulate,
                               hipStream_t s) {
    const long long rows = (long long)B * T;
    if (rows == 0 || H == 0) return hipSuccess;
    // 2048 workgroups of 256 threads fill the 256 CUs once at 8 per CU, with
    // far more loads in flight per CU than HBM latency needs; more rows go
    // round the grid stride.
    const unsigned grid = (unsigned)(rows < 2048 ? rows : 2048);
    if (dst_bf16)
        hipLaunchKernelGGL(bwd_finalize_kernel<true>, dim3(grid), dim3(256), 0, s, src, dst, tab, rows, T, H, d,
                           src_bstride, dst_bstride, 0);
    else
        hipLaunchKernelGGL(bwd_finalize_kernel<false>, dim3(grid), dim3(256), 0, s, src, dst, tab, rows, T, H, d,
                           src_bstride, dst_bstride, accumulate);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* x, long long n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const long long n4 = n / 4;   // callers pass multiples of 4 (d is 64 or 128)
    hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, s, (float4*)x, n4);
    return hipGetLastError();
}

}  // namespace bosa
