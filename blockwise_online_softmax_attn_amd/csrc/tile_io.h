// Device helpers shared by the bf16 attention kernels (forward and
// backward): lane-pair exchanges, the NaN-propagating maximum, the
// direct-to-LDS tile loads and their waits, and the transposed LDS read.
#pragma once

#include "common.h"

namespace bosa {

// Partner exchange between lane l and lane l ^ 32: both outputs of the swap
// hold {own value, partner value}.
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// NaN-propagating maximum (v_maximum3_f32): unlike fmaxf it needs no operand
// canonicalisation.  Scores are finite or -inf (excluded keys), where the two agree.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return vmax(vmax(a, b), c); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for raw byte addressing of `bytes` bytes from `base`;
// loads at or beyond `bytes` return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16 bytes per lane from rsrc + voff into LDS at m0 + 16 * lane.  Issued from
// inline assembly: the compiler neither waits for it before unrelated LDS
// reads nor counts it; the kernel waits with explicit vmcnt values.
__device__ __forceinline__ void load_lds16(uint32_t voff, const u32x4& rsrc, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc)
                 : "memory");
}

// 4 bytes per lane from rsrc + voff into LDS at m0 + 4 * lane (active lanes).
__device__ __forceinline__ void load_lds4(uint32_t voff, const u32x4& rsrc, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc)
                 : "memory");
}

// Workgroup synchronisation without any memory-counter wait beyond the LDS
// reads of this wave.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding and every LDS read it issued has returned, then synchronise the
// workgroup.
template <int N>
__device__ __forceinline__ void wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

__device__ __forceinline__ s16x4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// LDS reads at an absolute LDS byte address.  A loop-invariant per-lane
// address plus a compile-time constant becomes one ds_read with the constant
// in its immediate offset (no address arithmetic per read).
__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
    return *(const __attribute__((address_space(3))) bf16x8*)(size_t)addr;
}
__device__ __forceinline__ s16x4 lds_tr16(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(size_t)addr);
}


// Exclusions of a tile that is not entirely allowed.  The key behind
// accumulator register r of the first (second) 32-key block has local index
// 8 (r / 4) + 4 hh + r % 4 (+ 32).  thr4 = largest allowed local index minus
// 4 hh (causal order, the right edge of a window and the key tail); lo4 =
// smallest allowed local index minus 4 hh (the left edge of a window);
// kml = the tile's 64 key-padding allowed bits shifted right by 4 hh; am =
// attention-mask row of this lane's query at the tile's first key (shifted
// by 4 hh), or null.
struct TileMask {
    int thr4;
    uint64_t kml;
    const uint8_t* am;
    int lo4 = -128;
};

__device__ __forceinline__ void apply_mask(f32x16& s0, f32x16& s1, const TileMask& mk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int b0 = 8 * (r >> 2) + (r & 3);
        bool ok0 = b0 <= mk.thr4 && b0 >= mk.lo4 && ((mk.kml >> b0) & 1);
        bool ok1 = b0 + 32 <= mk.thr4 && b0 + 32 >= mk.lo4 && ((mk.kml >> (b0 + 32)) & 1);
        if (mk.am) {
            ok0 = ok0 && mk.am[b0] == 0;
            ok1 = ok1 && mk.am[b0 + 32] == 0;
        }
        s0[r] = ok0 ? s0[r] : -INFINITY;
        s1[r] = ok1 ? s1[r] : -INFINITY;
    }
}

// ALiBi: add ab |base - key| to every score of the tile, where base =
// (query position - position of the lane's first key) and ab = -slope sqrt(d)
// (the penalty in units of the unscaled dot product).  Excluded scores stay -inf.
__device__ __forceinline__ void add_alibi(f32x16& s0, f32x16& s1, float base, float ab) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float k0 = (float)(8 * (r >> 2) + (r & 3));
        s0[r] = fmaf(fabsf(base - k0), ab, s0[r]);
        s1[r] = fmaf(fabsf(base - (k0 + 32.f)), ab, s1[r]);
    }
}

}  // namespace bosa
