// rotate_quant.h -- device building blocks of the 128-point rotation and of
// the per-token int8 quantiser, shared by the standalone kernels and the
// fused decode kernel so that every path produces the same bits.
//
// Rotation (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance container",
// table row "Weights": every 128 of K is rotated by the unnormalised Hadamard
// transform; table row "Activations": activations use the same rotation).
//
// Lane layout of one 128-block: 16 lanes (one DPP row), 8 floats per lane.
// Lane l of the row holds elements 4l..4l+3 ("lo") and 64+4l..64+4l+3 ("hi"),
// loaded as two 16-byte chunks; the 16 lanes of a row read 256 contiguous
// bytes per load instruction.  Butterfly stages in the required order:
//   h = 1, 2      inside each chunk
//   h = 4 .. 32   across lanes l ^ 1, ^2, ^4, ^8 (DPP, no LDS traffic)
//   h = 64        between the lo and hi chunk of the same lane
// Each butterfly writes a+b to the lower index and a-b to the upper, where a
// is the lower element: the lower lane adds its partner, the upper lane
// subtracts itself from its partner, so every element sees exactly the IEEE
// operations of the sequential network.
#pragma once

#include "rad_device.h"

namespace rad {

struct Blk8 {
    float4 lo, hi;
};

__device__ __forceinline__ void bfly_in(float &a, float &b) {
    float s = a + b;
    float d = a - b;
    a = s;
    b = d;
}

template <int X>
__device__ __forceinline__ float bfly_x(float v, bool upper) {
    float p = lane_xor<X>(v);
    return upper ? (p - v) : (v + p);
}

template <int X>
__device__ __forceinline__ void bfly_x4(float4 &v, bool upper) {
    v.x = bfly_x<X>(v.x, upper);
    v.y = bfly_x<X>(v.y, upper);
    v.z = bfly_x<X>(v.z, upper);
    v.w = bfly_x<X>(v.w, upper);
}

// Rotate the block held by this lane's 16-lane row; l16 = lane index in the row.
__device__ __forceinline__ void fwht128_regs(Blk8 &b, int l16) {
    // h = 1
    bfly_in(b.lo.x, b.lo.y); bfly_in(b.lo.z, b.lo.w);
    bfly_in(b.hi.x, b.hi.y); bfly_in(b.hi.z, b.hi.w);
    // h = 2
    bfly_in(b.lo.x, b.lo.z); bfly_in(b.lo.y, b.lo.w);
    bfly_in(b.hi.x, b.hi.z); bfly_in(b.hi.y, b.hi.w);
    // h = 4, 8, 16, 32: partner lane l16 ^ 1, 2, 4, 8
    bfly_x4<1>(b.lo, l16 & 1); bfly_x4<1>(b.hi, l16 & 1);
    bfly_x4<2>(b.lo, l16 & 2); bfly_x4<2>(b.hi, l16 & 2);
    bfly_x4<4>(b.lo, l16 & 4); bfly_x4<4>(b.hi, l16 & 4);
    bfly_x4<8>(b.lo, l16 & 8); bfly_x4<8>(b.hi, l16 & 8);
    // h = 64
    bfly_in(b.lo.x, b.hi.x); bfly_in(b.lo.y, b.hi.y);
    bfly_in(b.lo.z, b.hi.z); bfly_in(b.lo.w, b.hi.w);
}

// Quantiser: per token, s = amax / 127 (IEEE f32 division), then each code
// is rne(v / s) clamped to +-127 (IEEE division, ties to even).
__device__ __forceinline__ int quant1(float v, float s) {
    // s > 0 here.  IEEE division, round half to even, clamp to +-127.
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
}

__device__ __forceinline__ uint32_t pack4(float4 v, float s) {
    uint32_t b0 = static_cast<uint32_t>(quant1(v.x, s)) & 0xFFu;
    uint32_t b1 = static_cast<uint32_t>(quant1(v.y, s)) & 0xFFu;
    uint32_t b2 = static_cast<uint32_t>(quant1(v.z, s)) & 0xFFu;
    uint32_t b3 = static_cast<uint32_t>(quant1(v.w, s)) & 0xFFu;
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// The same codes through the reciprocal: t = v * fl(1/s) lies within
// 1.5 * 2^-23 |v / s| (< 2^-15 here, |v / s| <= 127.06) of the rounded
// quotient fl(v / s), so both round to the same integer unless t is within
// 2^-13 of a half-integer (about 1 element in 4000).  pack4_rcp codes four
// elements that way and, if any lane of the wave holds such an element among
// its four, redoes the four with the IEEE division in a wave-uniform branch
// (taken for about 6% of the four-element groups of a wave).  Needs s in
// [2^-120, 2^120] (1/s finite and normal).
__device__ __forceinline__ float quant1_rcp(float v, float rs, bool &near) {
    const float t = v * rs;
    const float r = __builtin_rintf(t);
    // t lies within 2^-13 of a half-integer exactly when its distance to the
    // nearest integer exceeds 1/2 - 2^-13; t - r is exact (Sterbenz: r is 0,
    // or within a factor 2 of t)
    near = near || fabsf(t - r) > 0.5f - 0x1p-13f;
    return r;
}

__device__ __forceinline__ uint32_t pack4_rcp(float4 v, float s, float rs) {
    bool near = false;
    float r0 = quant1_rcp(v.x, rs, near), r1 = quant1_rcp(v.y, rs, near);
    float r2 = quant1_rcp(v.z, rs, near), r3 = quant1_rcp(v.w, rs, near);
    if (__any(near)) {
        r0 = __builtin_rintf(v.x / s);
        r1 = __builtin_rintf(v.y / s);
        r2 = __builtin_rintf(v.z / s);
        r3 = __builtin_rintf(v.w / s);
    }
    auto byte = [](float r) {
        return static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(r, -127.0f), 127.0f))) & 0xFFu;
    };
    return byte(r0) | (byte(r1) << 8) | (byte(r2) << 16) | (byte(r3) << 24);
}

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

}  // namespace rad
