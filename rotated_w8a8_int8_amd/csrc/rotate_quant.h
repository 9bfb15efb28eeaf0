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
// is the lower element.
//
// Two implementations of the cross-lane stages:
//   fwht128_regs      each butterfly forms a + b and a - b exactly as the
//                     sequential network does (a DPP move of the partner, the
//                     sum or difference, a select): every output bit matches,
//                     the sign of a zero included.
//   fwht128_regs_signed  a lane holds c * x for a sign c it need not store,
//                     and every cross-lane butterfly is one fused multiply-add
//                     v' = fma(partner, m, v), m = +1 on the lower lane and -1
//                     on the upper: the lower lane gets a + b, the upper
//                     b - a = -(a - b), so its sign flips.  Partners always
//                     carry equal signs (they differ only in the lane bit being
//                     processed), so afterwards c = (-1)^popcount(l) for every
//                     value of lane l; the stage inside the lane keeps it.  A
//                     product by +-1 is exact, the fused add rounds once, and
//                     round-to-nearest-even is symmetric in sign, so c * x
//                     equals the network's value times c, except that an exact
//                     cancellation may give a zero of the other sign.  The
//                     quantisers use it: |c x| = |x|, and symmetric codes of
//                     c * x are c times the codes of x.
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

// The four cross-lane stages on a lane's eight values, as one block of DPP
// fused multiply-adds (v_fmac_f32 with its first source read from the partner
// lane): partner l ^ 1 and l ^ 2 are single quad permutations, l ^ 8 the row
// rotation by 8; l ^ 4 is the half-row mirror (l -> l ^ 7), staged in a
// temporary with a DPP move, followed by quad permutation [3,2,1,0].  Written as one asm block
// because the compiler does not fold its DPP moves into v_fmac_f32.  Hazards:
// a DPP read of a VGPR needs two wait states after the VALU write of it; the
// leading s_nop 1 covers the writes before the block, and inside it every
// DPP source was written at least eight instructions earlier.
__device__ __forceinline__ void fwht_cross_lane(Blk8 &b, float m1, float m2, float m4, float m8) {
    float t0, t1, t2, t3, t4, t5, t6, t7;
#define RAD_FMAC8(CTRL, M)                                                         \
    "v_fmac_f32_dpp %0, %0, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %1, %1, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %2, %2, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %3, %3, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %4, %4, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %5, %5, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %6, %6, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %7, %7, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define RAD_MOV8(CTRL)                                                             \
    "v_mov_b32_dpp %8, %0 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"  \
    "v_mov_b32_dpp %9, %1 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"  \
    "v_mov_b32_dpp %10, %2 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_mov_b32_dpp %11, %3 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_mov_b32_dpp %12, %4 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_mov_b32_dpp %13, %5 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_mov_b32_dpp %14, %6 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_mov_b32_dpp %15, %7 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define RAD_FMACT8(CTRL, M)                                                        \
    "v_fmac_f32_dpp %0, %8, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"  \
    "v_fmac_f32_dpp %1, %9, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"  \
    "v_fmac_f32_dpp %2, %10, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %3, %11, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %4, %12, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %5, %13, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %6, %14, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
    "v_fmac_f32_dpp %7, %15, " M " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
    asm volatile(
        "s_nop 1\n\t"
        RAD_FMAC8("quad_perm:[1,0,3,2]", "%16")
        RAD_FMAC8("quad_perm:[2,3,0,1]", "%17")
        RAD_MOV8("row_half_mirror")
        RAD_FMACT8("quad_perm:[3,2,1,0]", "%18")
        RAD_FMAC8("row_ror:8", "%19")
        : "+v"(b.lo.x), "+v"(b.lo.y), "+v"(b.lo.z), "+v"(b.lo.w),
          "+v"(b.hi.x), "+v"(b.hi.y), "+v"(b.hi.z), "+v"(b.hi.w),
          "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
        : "v"(m1), "v"(m2), "v"(m4), "v"(m8));
#undef RAD_FMAC8
#undef RAD_MOV8
#undef RAD_FMACT8
}

// The sign c = (-1)^popcount(l16) a lane's values carry after
// fwht128_regs_signed, as +-1.0f.
__device__ __forceinline__ float fwht_lane_sign(int l16) {
    return (__builtin_popcount(l16) & 1) ? -1.0f : 1.0f;
}

// Rotate the block held by this lane's 16-lane row, leaving every value
// multiplied by fwht_lane_sign(l16); l16 = lane index in the row.
__device__ __forceinline__ void fwht128_regs_signed(Blk8 &b, int l16) {
    // h = 1
    bfly_in(b.lo.x, b.lo.y); bfly_in(b.lo.z, b.lo.w);
    bfly_in(b.hi.x, b.hi.y); bfly_in(b.hi.z, b.hi.w);
    // h = 2
    bfly_in(b.lo.x, b.lo.z); bfly_in(b.lo.y, b.lo.w);
    bfly_in(b.hi.x, b.hi.z); bfly_in(b.hi.y, b.hi.w);
    // h = 4, 8, 16, 32: partner lane l16 ^ 1, 2, 4, 8
    fwht_cross_lane(b, (l16 & 1) ? -1.0f : 1.0f, (l16 & 2) ? -1.0f : 1.0f, (l16 & 4) ? -1.0f : 1.0f,
                    (l16 & 8) ? -1.0f : 1.0f);
    // h = 64
    bfly_in(b.lo.x, b.hi.x); bfly_in(b.lo.y, b.hi.y);
    bfly_in(b.lo.z, b.hi.z); bfly_in(b.lo.w, b.hi.w);
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
// 2^-13 of a half-integer (about 1 element in 4000).  pack4_rcp_signed codes
// four elements that way and, if any lane of the wave holds such an element
// among its four, redoes the four with the IEEE division in a wave-uniform
// branch (taken for about 6% of the four-element groups of a wave).  Needs s
// in [2^-120, 2^120] (1/s finite and normal).
__device__ __forceinline__ float quant1_rcp(float v, float rs, bool &near) {
    const float t = v * rs;
    const float r = __builtin_rintf(t);
    // t lies within 2^-13 of a half-integer exactly when its distance to the
    // nearest integer exceeds 1/2 - 2^-13; t - r is exact (Sterbenz: r is 0,
    // or within a factor 2 of t)
    near = near || fabsf(t - r) > 0.5f - 0x1p-13f;
    return r;
}

// Codes of c * v (c = +-1, the lane sign of fwht128_regs_signed) for a
// lane holding v: the reciprocal scheme above with rs_c = c * fl(1/s) (so
// v * rs_c equals (c v) * fl(1/s) bit for bit, the sign aside rounding
// alike), and the division fallback on c * v, formed exactly.  No clamp: with
// s = fl(amax / 127) normal and |v| <= amax, |v / s| and |v * fl(1/s)| stay
// below 127 (1 + 2^-21), so both round to at most 127 in magnitude.
__device__ __forceinline__ uint32_t pack4_rcp_signed(float4 v, float s, float rs_c, float c) {
    bool near = false;
    float r0 = quant1_rcp(v.x, rs_c, near), r1 = quant1_rcp(v.y, rs_c, near);
    float r2 = quant1_rcp(v.z, rs_c, near), r3 = quant1_rcp(v.w, rs_c, near);
    if (__any(near)) {
        r0 = __builtin_rintf((c * v.x) / s);
        r1 = __builtin_rintf((c * v.y) / s);
        r2 = __builtin_rintf((c * v.z) / s);
        r3 = __builtin_rintf((c * v.w) / s);
    }
    auto byte = [](float r) { return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu; };
    return byte(r0) | (byte(r1) << 8) | (byte(r2) << 16) | (byte(r3) << 24);
}
__device__ __forceinline__ uint32_t pack4_signed(float4 v, float s, float c) {
    return pack4(make_float4(c * v.x, c * v.y, c * v.z, c * v.w), s);
}

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

}  // namespace rad
