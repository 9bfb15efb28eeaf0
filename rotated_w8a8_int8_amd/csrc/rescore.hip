// rescore.hip -- the rotated W8A8 layer evaluated only at candidate rows: for
// token m and candidate j, y[m][j] = the layer's output at row ids[m][j]
// (gfx950).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table row "Speculator": the drafter's top 32 candidates are
// rescored against the model's own head; table row "Weights": that head is
// int8 with a bf16 scale per (row, 128 of K)): exact int32 partials of the
// token's activation codes with the candidate row's codes, then the layer's
// epilogue.  Either weight format is accepted.
//
// One wave per (token, candidate); the four waves of a workgroup take four
// candidates of the same token, so the token's codes are read from HBM once
// and from cache after.  Lane l takes the 16-byte chunks l, l + 64, ... of K
// (all loads of a pass issued before use); every chunk lies in one group.
//   u8 format: sum_g u8 * P is accumulated exactly in int64, reduced across
//     the wave, and y = s * r * 2^-7 * S is evaluated in f64 in that order and
//     rounded once -- the same bits as the full layer's one-token epilogue.
//   head format: f32 sum of float(chunk partial) * scale, then s * 2^-7.
// An id outside 0..N-1 reads nothing and yields NaN.
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

// The gathered weight rows are read once, in short scattered runs, with
// nontemporal loads (ld16_nt): measured faster here than plain loads.

constexpr int kFmtU8 = 0;
constexpr int kRsPass = 8;     // chunks per lane per pass (K = 8192 in one pass)

__device__ __forceinline__ int64_t shfl_xor_i64(int64_t v, int x) {
    const int lo = static_cast<int>(v & 0xFFFFFFFF), hi = static_cast<int>(v >> 32);
    const uint32_t l2 = static_cast<uint32_t>(__shfl_xor(lo, x));
    const int h2 = __shfl_xor(hi, x);
    return (static_cast<int64_t>(h2) << 32) | l2;
}

template <int FMT>
__global__ __launch_bounds__(256) void rescore_kernel(const int8_t *__restrict__ q,
                                                      const float *__restrict__ scale,
                                                      const int8_t *__restrict__ codes,
                                                      const void *__restrict__ gscale,
                                                      const uint16_t *__restrict__ rscale,
                                                      const int32_t *__restrict__ ids,
                                                      float *__restrict__ y, int64_t pairs, int C,
                                                      int N, int K) {
    constexpr int GW16 = (FMT == kFmtU8) ? 16 : 8;      // 16-byte chunks per group
    const int lane = threadIdx.x & 63;
    const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (pair >= pairs) return;                            // whole waves only
    const int64_t m = pair / C;
    const int id = __builtin_amdgcn_readfirstlane(ids[pair]);
    if (id < 0 || id >= N) {
        if (lane == 0) y[pair] = __builtin_nanf("");
        return;
    }
    const int G = K / (16 * GW16);
    const int nchunk = K >> 4;
    const int8_t *wrow = codes + static_cast<int64_t>(id) * K;
    const int8_t *qrow = q + m * K;
    int64_t acc = 0;
    float accf = 0.0f;
    for (int c0 = 0; c0 < nchunk; c0 += 64 * kRsPass) {
        v4i w[kRsPass], a[kRsPass];
#pragma unroll
        for (int u = 0; u < kRsPass; ++u) {
            const int c = c0 + 64 * u + lane;
            if (c < nchunk) {
                w[u] = ld16_nt(wrow + 16 * c);
                a[u] = ld16(qrow + 16 * c);
            }
        }
#pragma unroll
        for (int u = 0; u < kRsPass; ++u) {
            const int c = c0 + 64 * u + lane;
            if (c < nchunk) {
                const int p = dot16_i8(w[u], a[u], 0);
                const int g = c / GW16;
                if constexpr (FMT == kFmtU8) {
                    const int u8 = static_cast<const uint8_t *>(gscale)[static_cast<int64_t>(id) * G + g];
                    acc += static_cast<int64_t>(p) * u8;
                } else {
                    const uint16_t b = static_cast<const uint16_t *>(gscale)[static_cast<int64_t>(id) * G + g];
                    accf += static_cast<float>(p) * bf16_to_f32(b);
                }
            }
        }
    }
    if constexpr (FMT == kFmtU8) {
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) acc += shfl_xor_i64(acc, x);
        if (lane == 0) {
            const double r = static_cast<double>(bf16_to_f32(rscale[id]));
            y[pair] = static_cast<float>(static_cast<double>(scale[m]) * r * 0x1p-7 * static_cast<double>(acc));
        }
    } else {
        const float t = wave_sum_f32(accf);
        if (lane == 0) y[pair] = (scale[m] * 0x1p-7f) * t;
    }
}

}  // namespace

hipError_t launch_rescore(const int8_t *q, const float *s, const WeightArgs &w, const int32_t *ids,
                          int64_t C, float *y, int64_t M, hipStream_t st) {
    const int64_t pairs = M * C;
    const dim3 grid(static_cast<uint32_t>((pairs + 3) / 4)), block(256);
    if (w.fmt == kFmtU8)
        hipLaunchKernelGGL(rescore_kernel<0>, grid, block, 0, st, q, s, w.codes, w.gscale, w.rscale, ids, y,
                           pairs, static_cast<int>(C), static_cast<int>(w.N), static_cast<int>(w.K));
    else
        hipLaunchKernelGGL(rescore_kernel<1>, grid, block, 0, st, q, s, w.codes, w.gscale, w.rscale, ids, y,
                           pairs, static_cast<int>(C), static_cast<int>(w.N), static_cast<int>(w.K));
    return hipGetLastError();
}

}  // namespace rad
