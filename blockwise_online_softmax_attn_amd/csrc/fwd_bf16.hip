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
//
// Data movement.  K (already rotated when the rotary embedding is on) and V
// tiles of 64 keys go from HBM straight into LDS with buffer loads in LDS mode
// (no registers, no LDS store instructions); keys past the end of the sequence
// fall outside the buffer range and arrive as zeros.  Four LDS slots hold the
// tiles in flight: while a wave works on tile i it already computes the scores
// of tile i + 1, and the loads of tiles i + 2 and i + 3 are outstanding.  The
// loads are issued from inline assembly with explicit vmcnt waits, so the
// compiler does not serialise them against the LDS reads of the other slots.
// Rows are stored in 16-byte granules permuted by an XOR of the row index, so
// the MFMA operand reads are free of LDS bank conflicts without padding.
//
// Schedule per tile i: issue the loads of tile i + 3; mask (only tiles that
// are not entirely allowed); S_{i+1} = K_{i+1} Q^T on the matrix cores
// interleaved with the exponentials of S_i against the row's reference max
// on the vector ALU, and a check of the probabilities' sums (rarely out of
// range: then the tile's scores are formed again and its row max moves the
// reference); then O += V_i P_i; wait for tile i + 2 and synchronise the
// workgroup.
#include <type_traits>

#include "tile_io.h"

namespace bosa {
namespace {

constexpr int BN = 64;     // keys per tile
constexpr int NW = 8;      // waves per workgroup, 32 query rows each
constexpr int BM = 32 * NW;
constexpr int NT = 64 * NW;
constexpr int NSLOT = 4;   // LDS tile slots (tiles i .. i + 3)
// Reference max of a row (log2 units): the row max of the tile with the
// row's first allowed keys, then moved only when the probabilities leave the
// range below (those tiles are processed again), so the other tiles take no
// row max.  (0 until then.)
// Bounds on a lane's probabilities against its row's reference max (log2
// units).  A lane's tile sum (32 probabilities) above kSumMax means some
// probability exceeded 2^16: the row's scores rose by more than 16 over the
// reference, which must then move up.  A running sum below kSumMin means
// every probability so far is below 2^-100, where float32 would soon lose
// them to underflow: the reference moves down to the row max.  Between the
// two, any reference gives the same result up to rounding.
constexpr float kSumMax = 0x1p21f;
constexpr float kSumMin = 0x1p-100f;


template <int N>
using IC = std::integral_constant<int, N>;

template <int D>
struct Geo {
    static constexpr int NC = D / 16;                // 16-wide d chunks of Q K^T
    static constexpr int NDB = D / 32;               // 32-row d blocks of O^T
    static constexpr int GPR = D / 8;                // 16-byte granules per K/V row
    static constexpr int ROW = 2 * D;                // bytes per K/V row in LDS
    static constexpr int RP = 256 / ROW;             // rows per 256-byte bank window
    static constexpr int TILE = BN * ROW;            // bytes per K or V tile
    static constexpr int SLOT = 2 * TILE;            // one K and one V tile
    static constexpr int LDS_BYTES = NSLOT * SLOT;
    // The K tiles of the NSLOT slots come first, then the V tiles: with the
    // slot a compile-time constant (the tile loop is unrolled NSLOT times) a
    // K operand read is (lane offset) + immediate, and V reads use lane
    // offsets that already include VBASE, so no per-tile address add is
    // needed (ds_read immediates reach 65535 bytes).
    static constexpr int VBASE = NSLOT * TILE;
    static constexpr int kt(int s) { return s * TILE; }          // K tile of slot s
    static constexpr int vt(int s) { return s * TILE; }          // V tile of slot s, relative to VBASE
    static constexpr int NBLK = TILE / 1024;         // 1 KB load blocks per tile and tensor
    static constexpr int NI = NBLK / NW;             // load blocks per wave per tile and tensor
    static constexpr int RPB = 1024 / ROW;           // rows per load block
    static_assert(NI >= 1 && NBLK % NW == 0, "load blocks must divide evenly over the waves");
    static_assert(2 * NI <= 15, "vmcnt immediates");
    // Granule permutations (involutions): stored position = granule ^ h(row).
    // K: the 16 rows read by one 16-lane group land in 16 distinct bank
    // windows.  V: the 4 rows x 32 bytes of a transposed-read group and the two
    // column halves of a 32-lane pass land in distinct banks.
    static __device__ __forceinline__ int hk(int r) { return (r / RP) % GPR; }
    static __device__ __forceinline__ int hv(int r) { return 4 * ((r / RP) % (GPR / 4)); }
};

// Pass 1 of a tile whose probabilities left their range on some lane, or
// that holds a row's first allowed keys: set or move the reference max m_i
// (log2 units) of each row that needs it, from row totals (the two
// half-waves of a row keep one reference):
//  - to the tile's row max mx for a row with nothing accumulated yet, so its
//    largest probability is exactly 1 before its bf16 rounding;
//  - up to mx when a probability exceeds 2^16 (mx > m_i + 16; every earlier
//    probability was <= 2^16, so mx is the running max);
//  - down when the row's running sum plus the tile's largest probability is
//    still below kSumMin: to the larger of mx and the largest probability
//    already accumulated (at most l above the reference).
// Rows with no allowed key in the tile, and all other rows, keep their
// reference, so a tile that changes no reference gives the same bits in
// either pass, and fully masked tiles never change the state.
template <int D>
__device__ __forceinline__ void remax(const f32x16& s0, const f32x16& s1, f32x16 (&o)[Geo<D>::NDB], float& m_i,
                                      float& l_i, float sl2) {
    float ma = max3(s0[0], s0[1], s0[2]), mb = max3(s1[0], s1[1], s1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
        ma = max3(ma, s0[r], s0[r + 1]);
        mb = max3(mb, s1[r], s1[r + 1]);
    }
    const float mx = xhalf_max(max3(ma, mb, vmax(s0[15], s1[15]))) * sl2;
    const float lrow = xhalf_sum(l_i);
    float mnew = m_i;
    if (mx > m_i + 16.f || (lrow == 0.f && mx > -INFINITY)) {
        mnew = mx;
    } else if (mx > -INFINITY && lrow + hw_exp2(mx - m_i) < kSumMin) {
        mnew = fmaxf(mx, lrow > 0.f ? m_i + log2f(lrow) : -INFINITY);
    }
    if (mnew != m_i) {
        const float a = l_i > 0.f ? hw_exp2(m_i - mnew) : 1.f;
        l_i *= a;
#pragma unroll
        for (int db = 0; db < Geo<D>::NDB; ++db) o[db] *= a;
        m_i = mnew;
    }
}

// S^T of one tile: keys [0, 32) into s0 and [32, 64) into s1.  Kt = offset
// of the K tile in LDS (a constant after inlining); koff = per-lane LDS
// addresses of the operands (granule c of this lane's key row in slot 0).
template <int D>
__device__ __forceinline__ void scores(uint32_t Kt, const uint32_t (&koff)[Geo<D>::NC],
                                       const bf16x8 (&qreg)[Geo<D>::NC], f32x16& s0, f32x16& s1) {
    using G = Geo<D>;
    bf16x8 ka0[G::NC], ka1[G::NC];
    ka0[0] = lds_b128(koff[0] + Kt);
    ka1[0] = lds_b128(koff[0] + Kt + 32 * G::ROW);
    ka0[1] = lds_b128(koff[1] + Kt);
    ka1[1] = lds_b128(koff[1] + Kt + 32 * G::ROW);
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        if (c + 2 < G::NC) {
            ka0[c + 2] = lds_b128(koff[c + 2] + Kt);
            ka1[c + 2] = lds_b128(koff[c + 2] + Kt + 32 * G::ROW);
        }
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0[c], qreg[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1[c], qreg[c], s1, 0, 0, 0);
    }
}

// Probabilities of the current tile, p = exp2(s sl2 + nm), in place of the
// scores in s0, s1, with this lane's sum of them in rs, interleaved with the
// scores of the next tile (K tile at LDS offset Kn into n0, n1).
template <int D>
__device__ __forceinline__ void exp_and_next(f32x16& s0, f32x16& s1, float nm, float sl2, float& rs, uint32_t Kn,
                                             const uint32_t (&koff)[Geo<D>::NC], const bf16x8 (&qreg)[Geo<D>::NC],
                                             f32x16& n0, f32x16& n1) {
    using G = Geo<D>;
    constexpr int PER = 16 / G::NC;   // registers of s0 (and of s1) per chunk of the next tile
    bf16x8 ka0[G::NC], ka1[G::NC];
    ka0[0] = lds_b128(koff[0] + Kn);
    ka1[0] = lds_b128(koff[0] + Kn + 32 * G::ROW);
    ka0[1] = lds_b128(koff[1] + Kn);
    ka1[1] = lds_b128(koff[1] + Kn + 32 * G::ROW);
    n0 = f32x16{};
    n1 = f32x16{};
    float rs0, rs1;   // start from the first probability (no add of 0)
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        if (c + 2 < G::NC) {
            ka0[c + 2] = lds_b128(koff[c + 2] + Kn);
            ka1[c + 2] = lds_b128(koff[c + 2] + Kn + 32 * G::ROW);
        }
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0[c], qreg[c], n0, 0, 0, 0);
#pragma unroll
        for (int r = c * PER; r < c * PER + PER; ++r) {
            s0[r] = hw_exp2(fmaf(s0[r], sl2, nm));
            rs0 = r == 0 ? s0[r] : rs0 + s0[r];
        }
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1[c], qreg[c], n1, 0, 0, 0);
#pragma unroll
        for (int r = c * PER; r < c * PER + PER; ++r) {
            s1[r] = hw_exp2(fmaf(s1[r], sl2, nm));
            rs1 = r == 0 ? s1[r] : rs1 + s1[r];
        }
        // keep the chunks in program order: the exponentials stay interleaved
        // with the matrix instructions instead of being hoisted ahead of them
        __builtin_amdgcn_sched_barrier(0);
    }
    rs = rs0 + rs1;
}

// The probabilities in s0, s1 as the bf16 P^T operands: chunk (kb, cc) =
// accumulator registers 8cc .. 8cc+7.
__device__ __forceinline__ void pack_p(const f32x16& s0, const f32x16& s1, bf16x8 (&pb)[4]) {
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
}

// One tile's softmax update after its (masked) scores are in c0, c1.  Pass 0
// takes no row max: the probabilities are formed against the reference max
// and checked (tile sum <= kSumMax, running sum >= kSumMin, something
// accumulated before).  Returns true when some lane fails (or a sum is not
// finite): the caller then runs pass 1
// on the same tile with its scores recomputed, where remax moves the
// reference before the probabilities are formed again; pass 1 always ends
// the tile.  On return the probabilities are in c0, c1 (their sum added to
// l_i) and the next tile's scores (K at LDS offset Kn) in x0, x1.
template <int D>
__device__ __forceinline__ bool softmax_tile(int pass, f32x16& c0, f32x16& c1, f32x16 (&o)[Geo<D>::NDB], float& m_i,
                                             float& l_i, float sl2, uint32_t Kn, const uint32_t (&koff)[Geo<D>::NC],
                                             const bf16x8 (&qreg)[Geo<D>::NC], f32x16& x0, f32x16& x1) {
    if (pass) remax<D>(c0, c1, o, m_i, l_i, sl2);
    float rs;
    exp_and_next<D>(c0, c1, -m_i, sl2, rs, Kn, koff, qreg, x0, x1);
    const float l_new = l_i + rs;
    // out of range, or nothing accumulated yet (a row's first allowed keys,
    // or scores so far below the reference that they all vanished): pass 1
    if (pass == 0 && __ballot(!(rs <= kSumMax && l_i > 0.f && l_new >= kSumMin))) return true;
    l_i = l_new;
    return false;
}

// O^T += V^T P^T for one tile; Vt = offset of the V tile in LDS (a constant
// after inlining), voff = per-lane LDS addresses of the transposed reads for
// each 32-row d block (slot 0).
template <int D>
__device__ __forceinline__ void accumulate_pv(uint32_t Vt, const uint32_t (&voff)[Geo<D>::NDB], const bf16x8 (&pb)[4],
                                              f32x16 (&o)[Geo<D>::NDB]) {
    using G = Geo<D>;
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    auto v_load = [&](int db, int kc) -> bf16x8 {
        const uint32_t p0 = voff[db] + Vt + (16 * kc) * G::ROW;
        const s16x4 r0 = lds_tr16(p0);
        const s16x4 r1 = lds_tr16(p0 + 8 * G::ROW);
        const s16x8 a = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        return __builtin_bit_cast(bf16x8, a);
    };
    // 4 NDB MFMAs in (db, kc) order; operand reads run PF MFMAs ahead
    constexpr int NM = 4 * G::NDB, PF = 3;
    bf16x8 va[PF + 1];
#pragma unroll
    for (int j = 0; j < PF; ++j) va[j] = v_load(j / 4, j % 4);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
        if (j + PF < NM) va[(j + PF) % (PF + 1)] = v_load((j + PF) / 4, (j + PF) % 4);
        o[j / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j % (PF + 1)], pb[j % 4], o[j / 4], 0, 0, 0);
    }
}

// Query tile, batch row and head of this workgroup.  Workgroup b is
// dispatched to XCD b % 8 (each XCD has its own L2), so the k-th workgroup of
// XCD x is b = 8k + x.  With a multiple of 8 (batch row, head) pairs each XCD
// takes whole pairs, so the query tiles of one head share that XCD's L2 for K
// and V: a contiguous range of pairs, or, when the pairs' work differs
// (`spread`: the batch rows have their own key-padding lengths), pairs
// round-robin (pair 8j + x is its j-th), so that the pairs of one batch row
// are spread over all XCDs instead of filling some of them.  Within a pair
// the heaviest query tiles (most keys under causal order) come first.  With
// any other pair count a pair's tiles would be cut into contiguous pieces on
// different XCDs, the heavy piece on one and the light on another; there
// workgroup b takes tile rank b / n of pair b % n (n pairs), so every XCD gets
// every 8th tile of the list ordered heaviest first over all pairs (with 4
// pairs, XCDs x and x + 4 share pair x % 4).
__device__ __forceinline__ void wg_tile(const FwdParams& p, bool spread, int& qt, int& b, int& h) {
    const int nq = p.n_qtiles;
    const int bid = blockIdx.x;
    const int npairs = (int)gridDim.x / nq;
    int bh, t;
    if (npairs & 7) {
        bh = bid % npairs;
        t = bid / npairs;
    } else if (spread) {
        const int k = bid >> 3;
        bh = (k / nq) * 8 + (bid & 7);
        t = k % nq;
    } else {
        const int l = (bid & 7) * ((int)gridDim.x >> 3) + (bid >> 3);
        bh = l / nq;
        t = l % nq;
    }
    qt = nq - 1 - t;
    h = bh % p.H;
    b = bh / p.H;
}

template <int D, bool ALIBI, bool WIN>
__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_kernel(const FwdParams p) {
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int l32 = lane & 31, hh = lane >> 5;

    int qt, b, h;
    wg_tile(p, p.kpm != nullptr && p.B > 1, qt, b, h);

    const int rs = p.row_stride;
    const uint32_t rs2 = 2u * (uint32_t)rs;   // bytes between consecutive keys
    const int Tq = p.Tq, Tkv = p.Tkv;
    const uint16_t* qg = (const uint16_t*)p.q + b * p.q_bstride + (long long)h * D;
    const char* kg = (const char*)((const uint16_t*)p.k + b * p.kv_bstride + (long long)h * D);
    const char* vg = (const char*)((const uint16_t*)p.v + b * p.kv_bstride + (long long)h * D);
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const bool causal = p.causal != 0;
    const float sl2 = p.scale_log2;

    // this wave's 32 rows: of the workgroup's 256 consecutive rows, or, when
    // paired (no window), of unit qt (waves 0-3) or unit nu - 1 - qt (waves
    // 4-7; idle when that is unit qt itself) of the nu 128-row units
    const int q0 = qt * BM;
    int qw0 = q0 + w * 32;
    int qlast = min(q0 + BM, Tq) - 1;
    if constexpr (!WIN) {
        if (p.paired) {
            const int hi = ((Tq + 127) >> 7) - 1 - qt;   // >= qt
            qw0 = w < 4 ? qt * 128 + 32 * w : (hi > qt ? hi * 128 + 32 * (w - 4) : Tq);
            qlast = min(hi * 128 + 128, Tq) - 1;
        }
    }
    const int qi = qw0 + l32;
    const bool qvalid = qi < Tq;
    const bool wvalid = qw0 < Tq;
    const int qwlast = min(qw0 + 31, Tq - 1);
    const long long delta = p.q_off - p.kv_off;   // key j allowed for query i iff j - i <= delta

    // ---- Q operand (already rotated when the rotary embedding is on): lane
    // holds query qi, d = 16c + 8hh + 0..7 for each chunk c.
    bf16x8 qreg[G::NC];
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qvalid) x = *(const uint4*)(qg + (long long)qi * rs + 16 * c + 8 * hh);
        qreg[c] = __builtin_bit_cast(bf16x8, x);
    }
    // Finish the Q loads here: the vmcnt bookkeeping of the loop below counts
    // only tile loads.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // ---- key tiles of this workgroup
    // Keys some row of the workgroup may see: [klo, khi) (causal order and the
    // window bound them unless every tile is to be visited).  Without a window
    // (WIN false) every window term folds away at compile time.
    const bool wl_on = WIN && p.win_left >= 0, wr_on = WIN && p.win_right >= 0;
    long long khi = Tkv, klo = 0;
    if (!noskip) {
        if (causal) khi = min(khi, delta + qlast + 1);
        if (wr_on) khi = min(khi, delta + qlast + p.win_right + 1);
        if (wl_on) klo = max(klo, delta + q0 - p.win_left);
    }
    khi = max(khi, 0LL);
    const int t_hi = (int)((khi + BN - 1) / BN);
    const int t_lo = klo >= khi ? t_hi : (int)(klo / BN);
    // Tiles whose every key is allowed for every row: [tf_lo, tf_hi) (of the
    // wave without a window, of the workgroup with one).
    long long kf_hi = Tkv, kf_lo = 0;
    if (causal) kf_hi = min(kf_hi, (WIN ? q0 : qw0) + delta + 1);
    if (wr_on) kf_hi = min(kf_hi, q0 + delta + p.win_right + 1);
    if (wl_on) kf_lo = max(kf_lo, qlast + delta - p.win_left);
    const long long tf_lo = (kf_lo + BN - 1) / BN;
    const long long tf_hi = kf_hi < 0 ? 0 : kf_hi / BN;
    const bool force_mask = noskip || p.amask != nullptr || (p.kpm && !p.kpm_list);
    // The live-tile list is read-only for this kernel: constant address space,
    // so its entries come in through scalar loads (a vector load would need a
    // vmcnt wait, which would also wait for the tile loads in flight).
    typedef const __attribute__((address_space(4))) int* cint_ptr;
    cint_ptr klist =
        (p.kpm_list && !noskip) ? (cint_ptr)(p.kpm_list + (long long)b * p.kpm_list_stride) : nullptr;
    int ntiles = t_hi - t_lo;
    if (klist) {
        // list positions of the first live tile >= t_lo and >= t_hi
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
        ntiles = first_at_least(t_hi) - i0;
        klist += i0;
    }
    auto tile_at = [&](int i) -> int { return klist ? (int)((uint32_t)klist[2 + i] & ~kTileClean) : t_lo + i; };
    auto clean_at = [&](int i) -> bool { return klist ? ((uint32_t)klist[2 + i] & kTileClean) != 0 : p.kpm == nullptr; };
    // Without a window the entirely allowed tiles are the leading ones: the
    // first list entries are the clean tiles 0, 1, ... before the first
    // tile with a padded key.
    int n_full = 0;
    if constexpr (!WIN) {
        long long nf = tf_hi;
        if (klist) nf = min(nf, (long long)klist[1]);
        n_full = force_mask ? 0 : (int)min(nf, (long long)ntiles);
    }
    auto full_at = [&](int i) -> bool {
        if constexpr (!WIN) {
            return i < n_full;
        } else {
            const int t = tile_at(i);
            return !force_mask && t >= tf_lo && t < tf_hi && clean_at(i);
        }
    };
    // Tiles [w_first, n_act) hold allowed keys for some row of this wave
    // (causal order and the window cut both ends); the others are skipped by
    // this wave.
    auto first_tile_after = [&](long long key) {   // first list position whose tile starts after key
        int lo = 0, hi = ntiles;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((long long)tile_at(mid) * BN <= key) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    int n_act = ntiles, w_first = 0;
    if (!wvalid) {
        n_act = 0;
    } else if (!noskip) {
        if (causal || wr_on) {
            long long lim = causal ? (long long)qwlast + delta : (long long)Tkv;
            if (wr_on) lim = min(lim, (long long)qwlast + delta + p.win_right);
            n_act = first_tile_after(lim);
        }
        if constexpr (WIN) {
            if (wl_on) w_first = first_tile_after(qw0 + delta - p.win_left - BN);
        }
    }
    const float ab = ALIBI ? -p.alibi[h] * p.sqrt_d : 0.f;

    // ---- per-lane constants
    // LDS operand offsets (bytes within a tile)
    // LDS byte address of the dynamic shared memory, folded into the per-lane
    // operand addresses once
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
    uint32_t koff[G::NC];
#pragma unroll
    for (int c = 0; c < G::NC; ++c) koff[c] = lds0 + l32 * G::ROW + 16 * ((2 * c + hh) ^ G::hk(l32));
    uint32_t voff[G::NDB];
    {
        const int jj = lane & 15, grp = lane >> 4;
        const int r0 = 4 * (grp >> 1) + (jj >> 2);
        const int hv = G::hv(r0);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
            const int g = 4 * db + 2 * (grp & 1) + ((jj & 3) >> 1);
            voff[db] = lds0 + G::VBASE + r0 * G::ROW + 16 * (g ^ hv) + 8 * (jj & 1);
        }
    }
    // Tile loads: this wave moves load blocks w*NI .. w*NI+NI-1 of the K and V
    // tiles; lane -> (row, stored position) -> source granule.
    uint32_t dk[G::NI], dv[G::NI];
#pragma unroll
    for (int n = 0; n < G::NI; ++n) {
        const int m = w * G::NI + n;
        const int row = m * G::RPB + lane / G::GPR;
        const int pos = lane % G::GPR;
        dk[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(pos ^ G::hk(row));
        dv[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(pos ^ G::hv(row));
    }
    auto issue = [&](int i) {
        const int key0 = tile_at(i) * BN;
        // bytes up to the end of the tile's last key row; keys >= Tkv read as zeros
        const uint32_t nb = (uint32_t)min(Tkv - 1 - key0, BN - 1) * rs2 + 2u * D;
        const u32x4 rk = buffer_rsrc(kg + (long long)key0 * rs2, nb);
        const u32x4 rv = buffer_rsrc(vg + (long long)key0 * rs2, nb);
        // opaque per call: the per-slot bases are then formed here with scalar
        // adds instead of being kept live (in spilled scalar registers) across the loop
        uint32_t lw = lds0 + (uint32_t)(w * G::NI) * 1024u;
        asm volatile("" : "+s"(lw));
        const uint32_t base = lw + (uint32_t)(i % NSLOT) * G::TILE;
#pragma unroll
        for (int n = 0; n < G::NI; ++n) load_lds16(dk[n], rk, base + 1024u * n);
#pragma unroll
        for (int n = 0; n < G::NI; ++n) load_lds16(dv[n], rv, base + G::VBASE + 1024u * n);
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

    float m_i = 0.f;         // reference max of scaled scores (log2 units)
    float l_i = 0.f;         // running denominator (this half-wave's keys)
    f32x16 o[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) o[db] = f32x16{};
    f32x16 s0 = f32x16{}, s1 = f32x16{};

    // ---- prologue: tiles 0..2 in flight, tiles 0 and 1 resident, S_0
    constexpr int PT = 2 * G::NI;   // tile loads per wave per tile
    if (ntiles > 0) issue(0);
    if (ntiles > 1) issue(1);
    if (ntiles > 2) {
        issue(2);
        wait_barrier<PT>();
    } else {
        wait_barrier<0>();
    }
    if (n_act > 0 && w_first == 0) scores<D>(G::kt(0), koff, qreg, s0, s1);

    // One tile: softmax of the scores in (c0, c1), scores of the next tile
    // into (x0, x1), O += V P.  Called with the two register sets swapped on
    // alternate tiles, so no copy of the scores is needed; S = i % NSLOT is
    // the tile's slot, a compile-time constant.
    auto step = [&](auto S, int i, f32x16& c0, f32x16& c1, f32x16& x0, f32x16& x1) {
        constexpr int sl = decltype(S)::value, sn = (sl + 1) % NSLOT;
        const bool more = i + 3 < ntiles;
        if (more) issue(i + 3);
        if (i >= w_first && i < n_act) {
            auto mask_tile = [&]() __attribute__((always_inline)) {
                if (!full_at(i)) apply_mask(c0, c1, tile_mask(i));
                if (ALIBI) add_alibi(c0, c1, (float)((long long)qi + delta - (long long)tile_at(i) * BN - 4 * hh), ab);
            };
            mask_tile();
            __builtin_amdgcn_s_setprio(1);
            // The scores of tile i + 1 are computed even when this wave will
            // not use them (last tile, or no allowed key for its rows): the
            // slot is always readable, and one code path keeps the registers
            // in budget.
            if (softmax_tile<D>(0, c0, c1, o, m_i, l_i, sl2, G::kt(sn), koff, qreg, x0, x1)) {
                // pass 1 (rare): the scores again, from the K tile still in LDS
                scores<D>(G::kt(sl), koff, qreg, c0, c1);
                mask_tile();
                softmax_tile<D>(1, c0, c1, o, m_i, l_i, sl2, G::kt(sn), koff, qreg, x0, x1);
            }
            bf16x8 pb[4];
            pack_p(c0, c1, pb);
            accumulate_pv<D>(G::vt(sl), voff, pb, o);
            __builtin_amdgcn_s_setprio(0);
        } else if constexpr (WIN) {
            if (i + 1 == w_first && w_first < n_act) {
                // first tile of a wave whose window starts later: its scores only
                scores<D>(G::kt(sn), koff, qreg, x0, x1);
            }
        }
        // tile i + 2 resident for every wave; tile i + 3 may stay in flight
        if (more) wait_barrier<PT>();
        else wait_barrier<0>();
    };
    f32x16 n0, n1;
    for (int i = 0; i < ntiles; i += NSLOT) {
        static_assert(NSLOT == 4, "the loop below is unrolled once per slot");
        step(IC<0>{}, i, s0, s1, n0, n1);
        if (i + 1 < ntiles) step(IC<1>{}, i + 1, n0, n1, s0, s1);
        if (i + 2 < ntiles) step(IC<2>{}, i + 2, s0, s1, n0, n1);
        if (i + 3 < ntiles) step(IC<3>{}, i + 3, n0, n1, s0, s1);
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

// ---------------------------------------------------------------------------
// A ring share's query block against its key/value blocks in ring order, in
// one launch.  Each workgroup keeps its 256 query rows (Q in registers) and
// runs the tile pipeline of attn_fwd_bf16_kernel over the concatenation of
// every block's live tiles, so the loads of a block's first tiles overlap the
// last tiles of the block before.  The rows' softmax state runs on across the
// blocks (each block keeps its own positions, causal bound and key padding),
// so the launch's blocks act as one key sequence: after the last tile each
// wave writes that partial (out, lse) to the float32 accumulator, or merges
// it into the partial a previous launch left there, or, for the last launch
// of the query block, merges and writes the final output in bf16.  No window,
// ALiBi or attention mask.
template <int D>
__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_chain_kernel(const ChainParams cp) {
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const FwdParams& p = cp.p;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;

    int qt, b, h;
    wg_tile(p, cp.blk[0].kpm != nullptr && p.B > 1, qt, b, h);

    const int rs = p.row_stride;
    const uint32_t rs2 = 2u * (uint32_t)rs;
    const int Tq = p.Tq;
    const uint16_t* qg = (const uint16_t*)p.q + b * p.q_bstride + (long long)h * D;
    const bool noskip = (p.flags & ATTN_NO_TILE_SKIP) != 0;
    const bool causal = p.causal != 0;
    const float sl2 = p.scale_log2;
    const int nb = cp.nblk;

    // this wave's 32 rows: of the workgroup's 256 consecutive rows, or, when
    // paired, of unit qt (waves 0-3) or unit nu - 1 - qt (waves 4-7; idle when
    // that is unit qt itself, the middle of an odd count).  Waves w and w + 4
    // share a SIMD, so each SIMD then runs one wave of each unit.
    int qw0, qlast;
    if (p.paired) {
        const int hi = ((Tq + 127) >> 7) - 1 - qt;   // >= qt
        qw0 = w < 4 ? qt * 128 + 32 * w : (hi > qt ? hi * 128 + 32 * (w - 4) : Tq);
        qlast = min(hi * 128 + 128, Tq) - 1;
    } else {
        qw0 = qt * BM + w * 32;
        qlast = min(qt * BM + BM, Tq) - 1;
    }
    const int qi = qw0 + l32;
    const bool qvalid = qi < Tq;
    const bool wvalid = qw0 < Tq;
    const int qwlast = min(qw0 + 31, Tq - 1);

    // ---- Q operand (rotated when the rotary embedding is on)
    bf16x8 qreg[G::NC];
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qvalid) x = *(const uint4*)(qg + (long long)qi * rs + 16 * c + 8 * hh);
        qreg[c] = __builtin_bit_cast(bf16x8, x);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // ---- per block: live tiles of the workgroup, leading tiles every row of
    // the wave allows, tiles that hold allowed keys for this wave's rows; kept in this
    // wave's LDS table (ntiles | nfull | nact, kMaxChain entries each).
    typedef const __attribute__((address_space(4))) int* cint_ptr;
    auto block_list = [&](int s) __attribute__((always_inline)) -> cint_ptr {
        const int* l = cp.blk[s].kpm_list;
        const int stride = (cp.blk[s].Tkv + BN - 1) / BN + 2;   // a list per batch row: count, clean, entries
        return (l && !noskip) ? (cint_ptr)(l + (long long)b * stride) : nullptr;
    };
    auto list_tile = [&](cint_ptr kl, int i) __attribute__((always_inline)) -> int { return (int)((uint32_t)kl[2 + i] & ~kTileClean); };
    int* tab = (int*)(smem + NSLOT * G::SLOT) + w * 3 * kMaxChain;
    int ntot = 0;
    for (int s = 0; s < nb; ++s) {
        const long long delta = p.q_off - cp.blk[s].kv_off;
        const int Tkv = cp.blk[s].Tkv;
        cint_ptr kl = block_list(s);
        long long khi = Tkv;
        if (!noskip && causal) khi = min(khi, delta + qlast + 1);
        khi = max(khi, 0LL);
        const int t_hi = (int)((khi + BN - 1) / BN);
        int ntl = t_hi;
        if (kl) {
            int lo = 0, hi = kl[0];
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (list_tile(kl, mid) < t_hi) lo = mid + 1;
                else hi = mid;
            }
            ntl = lo;
        }
        long long kf_hi = Tkv;
        if (causal) kf_hi = min(kf_hi, qw0 + delta + 1);   // tiles every row of the wave allows
        long long nf = kf_hi < 0 ? 0 : kf_hi / BN;
        if (kl) nf = min(nf, (long long)kl[1]);
        const bool fm = noskip || (cp.blk[s].kpm && !cp.blk[s].kpm_list);
        const int nfull = fm ? 0 : (int)min(nf, (long long)ntl);
        int nact = ntl;
        if (!wvalid) {
            nact = 0;
        } else if (!noskip && causal) {
            const long long lim = (long long)qwlast + delta;
            int lo = 0, hi = ntl;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((long long)(kl ? list_tile(kl, mid) : mid) * BN <= lim) lo = mid + 1;
                else hi = mid;
            }
            nact = lo;
        }
        if (lane == 0) {
            tab[s] = ntl;
            tab[kMaxChain + s] = nfull;
            tab[2 * kMaxChain + s] = nact;
        }
        ntot += ntl;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the table is written before it is read

    // ---- per-lane constants (as in attn_fwd_bf16_kernel)
    // LDS byte address of the dynamic shared memory, folded into the per-lane
    // operand addresses once
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
    uint32_t koff[G::NC];
#pragma unroll
    for (int c = 0; c < G::NC; ++c) koff[c] = lds0 + l32 * G::ROW + 16 * ((2 * c + hh) ^ G::hk(l32));
    uint32_t voff[G::NDB];
    {
        const int jj = lane & 15, grp = lane >> 4;
        const int r0 = 4 * (grp >> 1) + (jj >> 2);
        const int hv = G::hv(r0);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
            const int g = 4 * db + 2 * (grp & 1) + ((jj & 3) >> 1);
            voff[db] = lds0 + G::VBASE + r0 * G::ROW + 16 * (g ^ hv) + 8 * (jj & 1);
        }
    }
    uint32_t dk[G::NI], dv[G::NI];
#pragma unroll
    for (int n = 0; n < G::NI; ++n) {
        const int m = w * G::NI + n;
        const int row = m * G::RPB + lane / G::GPR;
        const int pos = lane % G::GPR;
        dk[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(pos ^ G::hk(row));
        dv[n] = (uint32_t)row * rs2 + 16u * (uint32_t)(pos ^ G::hv(row));
    }

    // ---- load cursor: block ls, list position li of the next tile to load,
    // and that block's addressing (read from the kernel arguments and the
    // table only when the cursor enters a block: a scalar or LDS read in
    // every tile would make the tile's operand reads wait with it)
    int ls = 0, li = 0, l_ntl = 0, l_Tkv = 0;
    const char* l_kg = nullptr;
    const char* l_vg = nullptr;
    cint_ptr l_list = nullptr;
    auto load_enter = [&](int s) __attribute__((always_inline)) {
        l_ntl = tab[s];
        l_Tkv = cp.blk[s].Tkv;
        l_kg = (const char*)((const uint16_t*)cp.blk[s].k + b * p.kv_bstride + (long long)h * D);
        l_vg = (const char*)((const uint16_t*)cp.blk[s].v + b * p.kv_bstride + (long long)h * D);
        l_list = block_list(s);
    };
    auto load_skip = [&]() __attribute__((always_inline)) {   // past exhausted (or empty) blocks
        while (ls < nb && li >= l_ntl) {
            ++ls;
            li = 0;
            if (ls < nb) load_enter(ls);
        }
    };
    if (nb > 0) load_enter(0);
    load_skip();
    auto issue_next = [&](int g) __attribute__((always_inline)) {   // the cursor's tile is global tile g
        const int key0 = (l_list ? list_tile(l_list, li) : li) * BN;
        const uint32_t nbytes = (uint32_t)min(l_Tkv - 1 - key0, BN - 1) * rs2 + 2u * D;
        const u32x4 rk = buffer_rsrc(l_kg + (long long)key0 * rs2, nbytes);
        const u32x4 rv = buffer_rsrc(l_vg + (long long)key0 * rs2, nbytes);
        // opaque per call: the per-slot bases are then formed here with scalar
        // adds instead of being kept live (in spilled scalar registers) across the loop
        uint32_t lw = lds0 + (uint32_t)(w * G::NI) * 1024u;
        asm volatile("" : "+s"(lw));
        const uint32_t base = lw + (uint32_t)(g % NSLOT) * G::TILE;
#pragma unroll
        for (int n = 0; n < G::NI; ++n) load_lds16(dk[n], rk, base + 1024u * n);
#pragma unroll
        for (int n = 0; n < G::NI; ++n) load_lds16(dv[n], rv, base + G::VBASE + 1024u * n);
        if (++li >= l_ntl) load_skip();
    };

    // ---- compute cursor: block cs, list position ci, and that block's state
    int cs = 0, ci = 0;
    long long c_delta = 0;
    int c_Tkv = 0, c_ntl = 0, c_nfull = 0, c_nact = 0;
    cint_ptr c_list = nullptr;
    const uint8_t* c_kpm = nullptr;
    bool c_clean_all = true;
    auto enter = [&](int s) __attribute__((always_inline)) {
        c_delta = p.q_off - cp.blk[s].kv_off;
        c_Tkv = cp.blk[s].Tkv;
        c_list = block_list(s);
        c_kpm = cp.blk[s].kpm ? cp.blk[s].kpm + b * p.kpm_bstride : nullptr;
        c_clean_all = cp.blk[s].kpm == nullptr;
        c_ntl = tab[s];
        c_nfull = tab[kMaxChain + s];
        c_nact = tab[2 * kMaxChain + s];
    };
    auto tile_mask = [&](int i) __attribute__((always_inline)) -> TileMask {
        TileMask mk{63, ~0ull, nullptr};
        const int key0 = (c_list ? list_tile(c_list, i) : i) * BN;
        long long thr = (long long)c_Tkv - key0 - 1;
        if (causal) thr = min(thr, (long long)qi + c_delta - key0);
        mk.thr4 = (int)(thr < -1 ? -1 : (thr > 63 ? 63 : thr)) - 4 * hh;
        const bool clean = c_list ? ((uint32_t)c_list[2 + i] & kTileClean) != 0 : c_clean_all;
        uint64_t km = ~0ull;
        if (c_kpm && !clean) {
            const bool okk = key0 + lane < c_Tkv && c_kpm[key0 + lane] == 0;
            km = __ballot(okk);
        }
        mk.kml = km >> (4 * hh);
        return mk;
    };

    float m_i = 0.f;   // reference max (log2 units)
    float l_i = 0.f;
    f32x16 o[G::NDB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) o[db] = f32x16{};

    // the launch's partial from (m_i, l_i, o): written to the float32
    // accumulator (the query block's first launch), merged into it, or merged
    // and written as the final bf16 output (cp.out_bf16, same layout)
    float* lse_ptr = p.lse + b * p.lse_bstride + (long long)h * p.lse_hstride + qi;
    const long long orow = b * p.o_bstride + (long long)qi * rs + (long long)h * D;
    auto finish_chain = [&]() __attribute__((always_inline)) {
        const float lsum = xhalf_sum(l_i);
        if (!qvalid) return;
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const float lse_b = lsum > 0.f ? (m_i + log2f(lsum)) * kLn2 : -INFINITY;
        const bool acc_in = cp.blk[0].accumulate != 0;
        float* og = (float*)p.out + orow;
        uint16_t* ob = cp.out_bf16 ? cp.out_bf16 + orow : nullptr;
        float lse_n = lse_b, wa = 0.f, wb = 1.f;
        if (acc_in) merge_weights(*lse_ptr, lse_b, lse_n, wa, wb);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = db * 32 + 8 * g + 4 * hh;
                float4 r = make_float4(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                       o[db][4 * g + 3] * inv);
                if (acc_in) {
                    const float4 oa = *(const float4*)(og + c);
                    r.x = merge_value(wa, oa.x, wb, r.x);
                    r.y = merge_value(wa, oa.y, wb, r.y);
                    r.z = merge_value(wa, oa.z, wb, r.z);
                    r.w = merge_value(wa, oa.w, wb, r.w);
                }
                if (ob) {
                    *(uint2*)(ob + c) = make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
                } else {
                    *(float4*)(og + c) = r;
                }
            }
        }
        if (hh == 0) *lse_ptr = lse_n;
    };
    // past blocks without a live tile for this workgroup
    auto skip_empty_blocks = [&]() __attribute__((always_inline)) {
        while (cs < nb && tab[cs] == 0) ++cs;
        if (cs < nb) enter(cs);
    };
    skip_empty_blocks();

    // ---- prologue: tiles 0..2 in flight, tiles 0 and 1 resident
    constexpr int PT = 2 * G::NI;
    if (ntot > 0) issue_next(0);
    if (ntot > 1) issue_next(1);
    if (ntot > 2) {
        issue_next(2);
        wait_barrier<PT>();
    } else {
        wait_barrier<0>();
    }

    // One tile (global index g): as in attn_fwd_bf16_kernel, plus the scores
    // of the tile when the wave skipped the tile before it, and the move to
    // the next block after a block's last tile.
    f32x16 s0 = f32x16{}, s1 = f32x16{}, n0, n1;
    bool have = false;   // the scores of tile g are in the current register set
    auto step = [&](auto S, int g, f32x16& c0, f32x16& c1, f32x16& x0, f32x16& x1) __attribute__((always_inline)) {
        constexpr int sl = decltype(S)::value, sn = (sl + 1) % NSLOT;   // slots of tiles g and g + 1
        const bool more = g + 3 < ntot;
        if (more) issue_next(g + 3);
        const bool act = ci < c_nact;
        if (act) {
            if (!have) scores<D>(G::kt(sl), koff, qreg, c0, c1);
            if (ci >= c_nfull) apply_mask(c0, c1, tile_mask(ci));
            __builtin_amdgcn_s_setprio(1);
            if (softmax_tile<D>(0, c0, c1, o, m_i, l_i, sl2, G::kt(sn), koff, qreg, x0, x1)) {
                // pass 1 (rare): the scores again, from the K tile still in LDS
                scores<D>(G::kt(sl), koff, qreg, c0, c1);
                if (ci >= c_nfull) apply_mask(c0, c1, tile_mask(ci));
                softmax_tile<D>(1, c0, c1, o, m_i, l_i, sl2, G::kt(sn), koff, qreg, x0, x1);
            }
            bf16x8 pb[4];
            pack_p(c0, c1, pb);
            accumulate_pv<D>(G::vt(sl), voff, pb, o);
            __builtin_amdgcn_s_setprio(0);
        }
        have = act;
        if (++ci == c_ntl) {
            ++cs;
            ci = 0;
            skip_empty_blocks();
        }
        if (!more) wait_barrier<0>();
        else wait_barrier<PT>();
    };
    for (int g = 0; g < ntot; g += NSLOT) {
        static_assert(NSLOT == 4, "the loop below is unrolled once per slot");
        step(IC<0>{}, g, s0, s1, n0, n1);
        if (g + 1 < ntot) step(IC<1>{}, g + 1, n0, n1, s0, s1);
        if (g + 2 < ntot) step(IC<2>{}, g + 2, s0, s1, n0, n1);
        if (g + 3 < ntot) step(IC<3>{}, g + 3, n0, n1, s0, s1);
    }
    finish_chain();
}

template <int D, bool ALIBI, bool WIN>
hipError_t launch(const FwdParams& p, hipStream_t s) {
    using G = Geo<D>;
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = set_lds_limit((const void*)attn_fwd_bf16_kernel<D, ALIBI, WIN>, G::LDS_BYTES, lds_set);
        e != hipSuccess)
        return e;
    FwdParams q = p;
    q.n_qtiles = (p.Tq + BM - 1) / BM;
    const long long grid = (long long)q.n_qtiles * p.H * p.B;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, ALIBI, WIN>), dim3((unsigned)grid), dim3(NT), G::LDS_BYTES, s, q);
    return hipGetLastError();
}

template <int D>
hipError_t launch_chain(const ChainParams& c, hipStream_t s) {
    using G = Geo<D>;
    constexpr int LDS = G::LDS_BYTES + NW * 3 * kMaxChain * 4;
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = set_lds_limit((const void*)attn_fwd_bf16_chain_kernel<D>, LDS, lds_set); e != hipSuccess)
        return e;
    ChainParams q = c;
    q.p.n_qtiles = (c.p.Tq + BM - 1) / BM;
    const long long grid = (long long)q.p.n_qtiles * c.p.H * c.p.B;
    hipLaunchKernelGGL(attn_fwd_bf16_chain_kernel<D>, dim3((unsigned)grid), dim3(NT), LDS, s, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_chain(const ChainParams& c, int d, hipStream_t s) {
    if (c.nblk < 1 || c.nblk > kMaxChain || c.p.rope_q || c.p.rope_k || c.p.amask || c.p.alibi ||
        c.p.win_left >= 0 || c.p.win_right >= 0)
        return hipErrorInvalidValue;
    return d == 128 ? launch_chain<128>(c, s) : launch_chain<64>(c, s);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s) {
    if (p.rope_q || p.rope_k) return hipErrorInvalidValue;   // queries and keys arrive rotated
    const bool win = p.win_left >= 0 || p.win_right >= 0;
    if (d == 128) {
        if (p.alibi) return win ? launch<128, true, true>(p, s) : launch<128, true, false>(p, s);
        return win ? launch<128, false, true>(p, s) : launch<128, false, false>(p, s);
    }
    if (p.alibi) return win ? launch<64, true, true>(p, s) : launch<64, true, false>(p, s);
    return win ? launch<64, false, true>(p, s) : launch<64, false, false>(p, s);
}

}  // namespace bosa
