// rad_device.h -- device helpers shared by the librad kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rad {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Global -> LDS dword copy without a register round trip: every active lane
// copies the 4 bytes at its own `src` to `lds_base + 4 * lane`; `lds_base`
// must be the same for the whole wave.  Completion is tracked by the vector
// memory counter, like any load: wait on it before reading the LDS words.
typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;
__device__ __forceinline__ void g2lds_dword(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds((gptr_t *)src, (lptr_t *)lds_base, 4, 0, 0);
}

// bf16 bit pattern -> f32 (a bf16 is the high half of an f32; exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// ---- DPP lane exchanges inside one 16-lane row --------------------------
// Each returns the value held by lane (lane ^ X) of the same row.  xor 1 and
// xor 2 are single quad permutations, xor 8 is the row rotation by 8 (i ->
// (i + 8) mod 16 = i ^ 8); xor 4 composes the half-row mirror (i -> i ^ 7)
// with quad permutation [3,2,1,0].
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kQuadXor3 = 0x1B;        // quad_perm [3,2,1,0]
constexpr int kRowRor8 = 0x128;        // lane i <- (i + 8) mod 16 = i ^ 8
constexpr int kRowHalfMirror = 0x141;  // lane i <- i ^ 7

__device__ __forceinline__ int lane_xor1(int v) { return dpp<kQuadXor1>(v); }
__device__ __forceinline__ int lane_xor2(int v) { return dpp<kQuadXor2>(v); }
__device__ __forceinline__ int lane_xor4(int v) { return dpp<kQuadXor3>(dpp<kRowHalfMirror>(v)); }
__device__ __forceinline__ int lane_xor8(int v) { return dpp<kRowRor8>(v); }

template <int X>
__device__ __forceinline__ int lane_xor(int v) {
    static_assert(X == 1 || X == 2 || X == 4 || X == 8, "xor inside a 16-lane row");
    if constexpr (X == 1) return lane_xor1(v);
    else if constexpr (X == 2) return lane_xor2(v);
    else if constexpr (X == 4) return lane_xor4(v);
    else return lane_xor8(v);
}
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
    return __int_as_float(lane_xor<X>(__float_as_int(v)));
}

// Exact integer sum over the 16 lanes of each DPP row (every lane gets it).
__device__ __forceinline__ int row16_sum(int v) {
    v += lane_xor<1>(v);
    v += lane_xor<2>(v);
    v += lane_xor<4>(v);
    v += lane_xor<8>(v);
    return v;
}
// Exact integer sum over the 8 lanes of each half row.
__device__ __forceinline__ int row8_sum(int v) {
    v += lane_xor<1>(v);
    v += lane_xor<2>(v);
    v += lane_xor<4>(v);
    return v;
}

// Exact integer sum over each aligned group of 4 lanes.
__device__ __forceinline__ int row4_sum(int v) {
    v += lane_xor<1>(v);
    v += lane_xor<2>(v);
    return v;
}

// Wave-uniform f32 sum (order fixed: 16-lane butterflies, then rows 0+1+2+3).
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += lane_xor<1>(v);
    v += lane_xor<2>(v);
    v += lane_xor<4>(v);
    v += lane_xor<8>(v);
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, lane_xor<1>(v));
    v = fmaxf(v, lane_xor<2>(v));
    v = fmaxf(v, lane_xor<4>(v));
    v = fmaxf(v, lane_xor<8>(v));
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// 4 x int8 dot products of a 16-byte chunk pair, exact int32.
__device__ __forceinline__ int dot16_i8(v4i a, v4i b, int acc) {
    acc = __builtin_amdgcn_sdot4(a.x, b.x, acc, false);
    acc = __builtin_amdgcn_sdot4(a.y, b.y, acc, false);
    acc = __builtin_amdgcn_sdot4(a.z, b.z, acc, false);
    acc = __builtin_amdgcn_sdot4(a.w, b.w, acc, false);
    return acc;
}

// Direct global -> LDS loads issued from inline asm.  Same data movement as
// g2lds_dword (and its 16-byte form), but invisible to the compiler's
// wait-count pass: it therefore neither drains these loads before every later
// LDS read (as it must for the builtin, not knowing which LDS bytes the load
// writes) nor tracks them at all.  Callers order them with explicit vmcnt waits and
// barriers.  Source = sbase (wave-uniform) + voff (per lane, unsigned 32-bit);
// destination = LDS byte address lds (wave-uniform, passed in M0) + size *
// lane.  The compiler's hazard checks do not look inside asm, so the block
// starts with the 5 wait states the ISA requires between a VALU write of an
// SGPR (v_readlane / v_readfirstlane, e.g. reloading a spilled base address)
// and a vector memory instruction reading that SGPR; they also cover the one
// an M0 write needs before an LDS DMA.  No register outputs, so nothing is
// live while the load is in flight.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "{m0}"(lds)
        : "memory");
}
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(sbase), "{m0}"(lds)
        : "memory");
}
// ---- the drafter's 16-level codebook (4-bit indices) ----------------------
// Values as printed in the recipe rules of section "How this file was made" on
// the model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance container" (rules
// dflash.*: rtn table=-127;-97;-75;-58;-43;-30;-18;-6;6;18;30;43;58;75;97;127).
constexpr uint32_t tbl4_dword(int a, int b, int c, int d) {
    return (static_cast<uint32_t>(a) & 0xFFu) | ((static_cast<uint32_t>(b) & 0xFFu) << 8) |
           ((static_cast<uint32_t>(c) & 0xFFu) << 16) | ((static_cast<uint32_t>(d) & 0xFFu) << 24);
}
constexpr uint32_t kTbl4_0 = tbl4_dword(-127, -97, -75, -58);
constexpr uint32_t kTbl4_1 = tbl4_dword(-43, -30, -18, -6);
constexpr uint32_t kTbl4_2 = tbl4_dword(6, 18, 30, 43);
constexpr uint32_t kTbl4_3 = tbl4_dword(58, 75, 97, 127);

// The three byte masks of the lookups below, held in VGPRs for a whole
// kernel (create them once, outside its loops): with them in registers each
// pick selector is one v_and_or_b32, a three-operand instruction that takes no
// literal on this chip, instead of an and, an or and their literals.
struct Tbl4Masks {
    uint32_t m7, m4, base;
};
__device__ __forceinline__ Tbl4Masks tbl4_masks() {
    Tbl4Masks k{0x07070707u, 0x04040404u, 0x03020100u};
    asm volatile("" : "+v"(k.m7), "+v"(k.m4), "+v"(k.base));
    return k;
}

// One 16-byte run of packed indices (32 elements: byte b holds element b in
// its low nibble and element 16 + b in its high nibble) -> the int8 values of
// elements 0..15 (lo) and 16..31 (hi).  Per dword of indices: v_perm looks up
// (index mod 8) in the lower and in the upper half of the table, then a third
// v_perm picks, byte by byte, the upper result where index bit 3 is set
// (selector byte i + 4 * bit3); all full-rate bit operations, no multiply.
__device__ __forceinline__ uint32_t tbl4_lookup4(uint32_t sel7, uint32_t pick) {
    const uint32_t lo = __builtin_amdgcn_perm(kTbl4_1, kTbl4_0, sel7);   // entries 0..7
    const uint32_t hi = __builtin_amdgcn_perm(kTbl4_3, kTbl4_2, sel7);   // entries 8..15
    return __builtin_amdgcn_perm(hi, lo, pick);
}
__device__ __forceinline__ void tbl4_decode16(v4i packed, v4i &lo, v4i &hi, const Tbl4Masks &k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = static_cast<uint32_t>(packed[i]);
        lo[i] = static_cast<int>(tbl4_lookup4(w & k.m7, ((w >> 1) & k.m4) | k.base));
        hi[i] = static_cast<int>(tbl4_lookup4((w >> 4) & k.m7, ((w >> 5) & k.m4) | k.base));
    }
}

// LDS byte offset of a __shared__ object (the low half of its flat address).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Loads that bypass nothing: plain 16-byte global loads.
__device__ __forceinline__ v4i ld16(const void *p) { return *reinterpret_cast<const v4i *>(p); }
// 16-byte nontemporal loads (global_load_dwordx4 ... nt): for data a call
// reads exactly once.
__device__ __forceinline__ v4i ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

}  // namespace rad
