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

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

}  // namespace rad
