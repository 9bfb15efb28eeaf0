// fwht_quant.hip -- rotation by the 128-point Hadamard transform, and the
// fused rotate + per-token int8 quantisation of activations (gfx950).
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
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

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

// ------------------------------------------------------------------ fwht --
// Each wave rotates 4 consecutive blocks per step; grid-stride over blocks of
// the flattened [rows][K] array (blocks never straddle rows since K % 128 == 0).
// x and y may be the same buffer: a lane writes only what its row read.
__global__ __launch_bounds__(256) void fwht128_kernel(const float *x, float *y, int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    for (int64_t b0 = wave * 4; b0 < nblocks; b0 += nwaves * 4) {
        const int64_t blk = b0 + (lane >> 4);
        const bool valid = blk < nblocks;
        Blk8 v;
        if (valid) {
            const float *p = x + blk * 128 + 4 * l16;
            v.lo = *reinterpret_cast<const float4 *>(p);
            v.hi = *reinterpret_cast<const float4 *>(p + 64);
        } else {
            v.lo = make_float4(0.f, 0.f, 0.f, 0.f);
            v.hi = v.lo;
        }
        fwht128_regs(v, l16);
        if (valid) {
            float *p = y + blk * 128 + 4 * l16;
            *reinterpret_cast<float4 *>(p) = v.lo;
            *reinterpret_cast<float4 *>(p + 64) = v.hi;
        }
    }
}

// ----------------------------------------------------- rotate + quantise --
// One workgroup per token.  WAVES waves, each holding 4 blocks per step, NITER
// steps: the whole rotated row stays in registers between the amax reduction
// and the division.
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

template <int WAVES, int NITER>
__global__ __launch_bounds__(WAVES * 64) void quant_act_kernel(const float *__restrict__ x,
                                                               int8_t *__restrict__ q,
                                                               float *__restrict__ scale,
                                                               int K, int rotate) {
    __shared__ float red[WAVES];
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int nblk = K >> 7;
    const int64_t m = blockIdx.x;
    const float *xr = x + m * K;

    Blk8 v[NITER];
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < NITER; ++it) {
        const int blk = (it * WAVES + wid) * 4 + (lane >> 4);
        if (blk < nblk) {
            const float *p = xr + blk * 128 + 4 * l16;
            v[it].lo = *reinterpret_cast<const float4 *>(p);
            v[it].hi = *reinterpret_cast<const float4 *>(p + 64);
        } else {
            v[it].lo = make_float4(0.f, 0.f, 0.f, 0.f);
            v[it].hi = v[it].lo;
        }
    }
#pragma unroll
    for (int it = 0; it < NITER; ++it) {
        if (rotate) fwht128_regs(v[it], l16);
        amax = fmaxf(amax, fmaxf(amax4(v[it].lo), amax4(v[it].hi)));
    }
    amax = wave_max_f32(amax);
    if (lane == 0) red[wid] = amax;
    __syncthreads();
    float a = red[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) a = fmaxf(a, red[w]);
    const float s = a / 127.0f;
    if (threadIdx.x == 0) scale[m] = s;

    int8_t *qr = q + m * K;
#pragma unroll
    for (int it = 0; it < NITER; ++it) {
        const int blk = (it * WAVES + wid) * 4 + (lane >> 4);
        if (blk < nblk) {
            uint32_t lo = 0, hi = 0;
            if (s != 0.0f) {
                lo = pack4(v[it].lo, s);
                hi = pack4(v[it].hi, s);
            }
            int8_t *p = qr + blk * 128 + 4 * l16;
            *reinterpret_cast<uint32_t *>(p) = lo;
            *reinterpret_cast<uint32_t *>(p + 64) = hi;
        }
    }
}

template <int WAVES, int NITER>
hipError_t launch_quant_t(const float *x, int8_t *q, float *s, int64_t M, int K, int rotate,
                          hipStream_t st) {
    hipLaunchKernelGGL((quant_act_kernel<WAVES, NITER>), dim3(static_cast<uint32_t>(M)),
                       dim3(WAVES * 64), 0, st, x, q, s, K, rotate);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwht128(const float *x, float *y, int64_t rows, int64_t K, hipStream_t st) {
    const int64_t nblocks = rows * (K / 128);
    const int64_t wave_steps = (nblocks + 3) / 4;          // 4 blocks per wave step
    int64_t grid = (wave_steps + 3) / 4;                   // 4 waves per workgroup
    const int64_t cap = 256 * 32;                          // enough to fill every CU many times
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(fwht128_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, x, y,
                       nblocks);
    return hipGetLastError();
}

hipError_t launch_quant_act(const float *x, int8_t *q, float *s, int64_t M, int64_t K, int rotate,
                            hipStream_t st) {
    const int nblk = static_cast<int>(K / 128);
    const int Ki = static_cast<int>(K);
    // Few tokens, or long rows: 16 waves per token (4 blocks per wave per
    // step) so each token finishes in few steps.  Many tokens: 4 waves each.
    const int niter4 = (nblk + 15) / 16;
    if (M < 256 || niter4 > 12) {
        const int niter = (nblk + 63) / 64;
        if (niter <= 1) return launch_quant_t<16, 1>(x, q, s, M, Ki, rotate, st);
        if (niter <= 2) return launch_quant_t<16, 2>(x, q, s, M, Ki, rotate, st);
        if (niter <= 4) return launch_quant_t<16, 4>(x, q, s, M, Ki, rotate, st);
        return launch_quant_t<16, 8>(x, q, s, M, Ki, rotate, st);   // K <= 65536
    }
    switch (niter4) {
        case 1: return launch_quant_t<4, 1>(x, q, s, M, Ki, rotate, st);
        case 2: return launch_quant_t<4, 2>(x, q, s, M, Ki, rotate, st);
        case 3: return launch_quant_t<4, 3>(x, q, s, M, Ki, rotate, st);
        case 4: return launch_quant_t<4, 4>(x, q, s, M, Ki, rotate, st);
        case 5: return launch_quant_t<4, 5>(x, q, s, M, Ki, rotate, st);
        case 6: return launch_quant_t<4, 6>(x, q, s, M, Ki, rotate, st);
        case 7: return launch_quant_t<4, 7>(x, q, s, M, Ki, rotate, st);
        case 8: return launch_quant_t<4, 8>(x, q, s, M, Ki, rotate, st);
        case 9: return launch_quant_t<4, 9>(x, q, s, M, Ki, rotate, st);
        case 10: return launch_quant_t<4, 10>(x, q, s, M, Ki, rotate, st);
        default: return launch_quant_t<4, 12>(x, q, s, M, Ki, rotate, st);
    }
}

}  // namespace rad
