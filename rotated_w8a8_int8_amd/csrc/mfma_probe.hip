// mfma_probe.hip -- a measurement aid, not a step of the layer: back-to-back
// v_mfma_i32_32x32x32_i8 on operand bytes the caller supplies, to measure
// what the int8 matrix cores sustain on given data within the part's power
// budget (on random codes they do not hold the 2.4 GHz clock).
//
// One 8-wave workgroup per CU (its 96 KiB LDS allocation keeps a second one
// off the CU), each wave a 64 x 64 tile: two activation and two weight
// fragments per k-step and four matrix ops on them in serpentine order, as in
// the prefill GEMM.  Register-fed: the wave alternates between two fragment
// sets loaded once.  LDS-fed: every k-step's fragments are read from LDS
// first (one 16-byte read per fragment and lane, double-buffered across
// k-steps), the reads an LDS-staged GEMM of this wave tile has to make; the
// LDS holds the block's 96 KiB of operand bytes, loaded once.  Each lane
// writes the 32-bit wrapping sum of its 64 accumulator elements.
#include "../../include/rad.h"
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kPrWaves = 8;
constexpr int kPrChunks = kProbeBlockBytes / 1024;     // 1 KiB chunks of a block's operands
typedef __attribute__((address_space(3))) const v4i lds_cv4i;

template <bool LDS_FED>
__global__ __launch_bounds__(64 * kPrWaves) void mfma_probe_kernel(const v4i *__restrict__ src,
                                                                   uint32_t *__restrict__ out, int ksteps) {
    __shared__ __attribute__((aligned(1024))) v4i lds[kProbeBlockBytes / 16];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const v4i *blk = src + static_cast<int64_t>(blockIdx.x) * (kProbeBlockBytes / 16);
    for (int i = threadIdx.x; i < kProbeBlockBytes / 16; i += 64 * kPrWaves) lds[i] = blk[i];
    __syncthreads();
    const uint32_t base = lds_offset(&lds[0]) + 16u * lane;
    auto chunk = [&](uint32_t c) -> v4i { return *reinterpret_cast<lds_cv4i *>(base + 1024u * c); };
    // fragment set h of k-step parity h: chunks c0 .. c0 + 3 (two activation, two weight)
    uint32_t c0 = static_cast<uint32_t>((w * 12) % kPrChunks);
    v4i a[2][2], b[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            a[h][t] = chunk(c0 + 4 * h + t);
            b[h][t] = chunk(c0 + 4 * h + 2 + t);
        }
    }
    c0 = (c0 + 8) % kPrChunks;
    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16i{};
    for (int ks = 0; ks < ksteps; ks += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (LDS_FED) {
                // the next k-step's fragments into the other set
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    a[h ^ 1][t] = chunk(c0 + t);
                    b[h ^ 1][t] = chunk(c0 + 2 + t);
                }
                c0 = (c0 + 4) % kPrChunks;
            }
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn_ = 0; tn_ < 2; ++tn_) {
                    const int tn = tm ? 1 - tn_ : tn_;
                    acc[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[h][tm], b[h][tn], acc[tm][tn], 0, 0, 0);
                }
        }
    }
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) r += static_cast<uint32_t>(acc[i][j][e]);
    out[(static_cast<int64_t>(blockIdx.x) * kPrWaves + w) * 64 + lane] = r;
}

}  // namespace

hipError_t launch_mfma_probe(const int8_t *src, int32_t *out, int64_t blocks, int64_t ksteps, bool lds_fed,
                             hipStream_t st) {
    auto kern = lds_fed ? mfma_probe_kernel<true> : mfma_probe_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kPrWaves), 0, st,
                       reinterpret_cast<const v4i *>(src), reinterpret_cast<uint32_t *>(out),
                       static_cast<int>(ksteps));
    return hipGetLastError();
}

}  // namespace rad
