// fwht_quant.hip -- rotation by the 128-point Hadamard transform, and the
// fused rotate + per-token int8 quantisation of activations (gfx950).  The
// lane layout and butterfly order are described in rotate_quant.h.
#include "rad_launch.h"
#include "rotate_quant.h"

namespace rad {
namespace {

// Both kernels stream their input and output once: nontemporal loads and
// stores (global_load/store ... nt).  On 8192 x 17408 activations they
// measured 6.6% faster than plain ones for the rotation, and 12% faster for
// rotate + quantise (130.0 -> 114.0 us; nontemporal stores alone 123.8 us).
// Rotate + quantise uses them from 256 tokens on: for a few tokens the codes
// are read again at once by the contraction (16 tokens: 28.2 against 28.5 us
// for the drafter's step with them).
typedef float nt_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float *p) {
    const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float4 v, float *p) {
    __builtin_nontemporal_store(nt_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f4 *>(p));
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
            v.lo = ld_nt(p);
            v.hi = ld_nt(p + 64);
        } else {
            v.lo = make_float4(0.f, 0.f, 0.f, 0.f);
            v.hi = v.lo;
        }
        fwht128_regs(v, l16);
        if (valid) {
            float *p = y + blk * 128 + 4 * l16;
            st_nt(v.lo, p);
            st_nt(v.hi, p + 64);
        }
    }
}

// ----------------------------------------------------- rotate + quantise --
// One workgroup per token.  WAVES waves, each holding 4 blocks per step, NITER
// steps: the whole rotated row stays in registers between the amax reduction
// and the division.
template <int WAVES, int NITER, bool NT>
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
            if constexpr (NT) {
                v[it].lo = ld_nt(p);
                v[it].hi = ld_nt(p + 64);
            } else {
                v[it].lo = *reinterpret_cast<const float4 *>(p);
                v[it].hi = *reinterpret_cast<const float4 *>(p + 64);
            }
        } else {
            v[it].lo = make_float4(0.f, 0.f, 0.f, 0.f);
            v[it].hi = v[it].lo;
        }
    }
    if (rotate) {
#pragma unroll
        for (int it = 0; it < NITER; ++it) fwht128_regs_signed(v[it], l16);   // values times the lane sign c
    }
#pragma unroll
    for (int it = 0; it < NITER; ++it) amax = fmaxf(amax, fmaxf(amax4(v[it].lo), amax4(v[it].hi)));
    amax = wave_max_f32(amax);
    if (lane == 0) red[wid] = amax;
    __syncthreads();
    float a = red[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) a = fmaxf(a, red[w]);
    const float s = a / 127.0f;
    if (threadIdx.x == 0) scale[m] = s;

    // codes through the reciprocal (each element provably equal to the
    // division's, rare near-half elements redone with it); scales too small
    // for a finite reciprocal use the division throughout (s is per token,
    // so the branch is uniform)
    const bool fast = s >= 0x1p-120f;
    const float c = rotate ? fwht_lane_sign(l16) : 1.0f;
    const float rs_c = c * (1.0f / s);
    int8_t *qr = q + m * K;
#pragma unroll
    for (int it = 0; it < NITER; ++it) {
        const int blk = (it * WAVES + wid) * 4 + (lane >> 4);
        if (blk < nblk) {
            uint32_t lo = 0, hi = 0;
            if (fast) {
                lo = pack4_rcp_signed(v[it].lo, s, rs_c, c);
                hi = pack4_rcp_signed(v[it].hi, s, rs_c, c);
            } else if (s != 0.0f) {
                lo = pack4_signed(v[it].lo, s, c);
                hi = pack4_signed(v[it].hi, s, c);
            }
            int8_t *p = qr + blk * 128 + 4 * l16;
            if constexpr (NT) {
                __builtin_nontemporal_store(lo, reinterpret_cast<uint32_t *>(p));
                __builtin_nontemporal_store(hi, reinterpret_cast<uint32_t *>(p + 64));
            } else {
                *reinterpret_cast<uint32_t *>(p) = lo;
                *reinterpret_cast<uint32_t *>(p + 64) = hi;
            }
        }
    }
}

template <int WAVES, int NITER>
hipError_t launch_quant_t(const float *x, int8_t *q, float *s, int64_t M, int K, int rotate,
                          hipStream_t st) {
    auto kern = M >= 256 ? quant_act_kernel<WAVES, NITER, true> : quant_act_kernel<WAVES, NITER, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(M)), dim3(WAVES * 64), 0, st, x, q, s, K,
                       rotate);
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
    // step) so each token finishes in few steps, 8 waves when the row holds
    // at most 64 blocks (K = 5120: 40 blocks, where 16 waves leave 6 of them
    // without work).  Many tokens: 4 waves each.
    const int niter4 = (nblk + 15) / 16;
    if (M < 256 && nblk <= 32) return launch_quant_t<8, 1>(x, q, s, M, Ki, rotate, st);
    if (M < 256 && nblk <= 64) return launch_quant_t<8, 2>(x, q, s, M, Ki, rotate, st);
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
