// gemm.hip -- rotated W8A8 contraction + epilogue for prefill sized batches on
// the int8 matrix cores (v_mfma_i32_16x16x64_i8, gfx950).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table rows "Weights" and "Activations"): exact int32 partials
// of int8 activation codes times int8 weight codes per K group, scaled per
// group into f32 accumulators, then y = s_m * (r_n) * 2^-7 * acc.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 tile of y; its 4 waves own
// 64 x 64 quarters (4 x 4 MFMA tiles).  K is walked in 128-byte stages,
// double-buffered in LDS with a 16-byte row pad; each K group (256 or 128)
// ends with the scale epilogue `F += float(P) * scale[n][g]; P = 0`.
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;

template <int FMT, bool WRITE_P>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const int8_t *__restrict__ q,
                                                      const float *__restrict__ scale,
                                                      const int8_t *__restrict__ codes,
                                                      const void *__restrict__ gscale,
                                                      const uint16_t *__restrict__ rscale,
                                                      float *__restrict__ y,
                                                      int32_t *__restrict__ partials, int M, int N,
                                                      int K, int tiles_n) {
    constexpr int BM = 128, BN = 128, KC = 128, LD = KC + 16;
    constexpr int GW = (FMT == kFmtU8) ? 256 : 128;
    constexpr int CPG = GW / KC;                      // stages per group
    constexpr int CPT = BM * KC / 16 / 256;           // 16-byte chunks per thread per operand
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LD];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int j = lane & 15, qd = lane >> 4;
    const int bm = (blockIdx.x / tiles_n) * BM;
    const int bn = (blockIdx.x % tiles_n) * BN;
    const int G = K / GW;
    const int nk = K / KC;

    v4i ra[CPT], rb[CPT];
    auto load_stage = [&](int kc) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx / (KC / 16);
            const int kb = (idx % (KC / 16)) * 16;
            const int64_t koff = static_cast<int64_t>(kc) * KC + kb;
            ra[i] = (bm + row < M) ? ld16(q + static_cast<int64_t>(bm + row) * K + koff) : v4i{0, 0, 0, 0};
            rb[i] = (bn + row < N) ? ld16(codes + static_cast<int64_t>(bn + row) * K + koff) : v4i{0, 0, 0, 0};
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx / (KC / 16);
            const int kb = (idx % (KC / 16)) * 16;
            *reinterpret_cast<v4i *>(&As[buf][row * LD + kb]) = ra[i];
            *reinterpret_cast<v4i *>(&Bs[buf][row * LD + kb]) = rb[i];
        }
    };

    int ncol[4];
    bool nval[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        ncol[tn] = bn + wn * 64 + tn * 16 + j;
        nval[tn] = ncol[tn] < N;
    }
    auto load_scales = [&](float (&sc)[4], int g) {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            if (!nval[tn]) { sc[tn] = 0.0f; continue; }
            const int64_t off = static_cast<int64_t>(ncol[tn]) * G + g;
            if constexpr (FMT == kFmtU8)
                sc[tn] = static_cast<float>(static_cast<const uint8_t *>(gscale)[off]);
            else
                sc[tn] = bf16_to_f32(static_cast<const uint16_t *>(gscale)[off]);
        }
    };

    v4i P[4][4];
    float F[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            P[a][b] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) F[a][b][e] = 0.0f;
        }

    float sc[4];
    load_scales(sc, 0);
    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        const bool more = kc + 1 < nk;
        if (more) load_stage(kc + 1);
#pragma unroll
        for (int st = 0; st < KC / 64; ++st) {
            v4i af[4], bf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[t] = *reinterpret_cast<const v4i *>(&As[buf][(wm * 64 + t * 16 + j) * LD + st * 64 + qd * 16]);
                bf[t] = *reinterpret_cast<const v4i *>(&Bs[buf][(wn * 64 + t * 16 + j) * LD + st * 64 + qd * 16]);
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
                    P[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn], P[tm][tn], 0, 0, 0);
        }
        if ((kc + 1) % CPG == 0) {
            const int g = kc / CPG;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    F[tm][tn][0] += static_cast<float>(P[tm][tn].x) * sc[tn];
                    F[tm][tn][1] += static_cast<float>(P[tm][tn].y) * sc[tn];
                    F[tm][tn][2] += static_cast<float>(P[tm][tn].z) * sc[tn];
                    F[tm][tn][3] += static_cast<float>(P[tm][tn].w) * sc[tn];
                }
            if constexpr (WRITE_P) {
#pragma unroll
                for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn) {
                        if (!nval[tn]) continue;
                        const int pv[4] = {P[tm][tn].x, P[tm][tn].y, P[tm][tn].z, P[tm][tn].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = bm + wm * 64 + tm * 16 + 4 * qd + e;
                            if (m < M) partials[(static_cast<int64_t>(m) * N + ncol[tn]) * G + g] = pv[e];
                        }
                    }
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) P[tm][tn] = v4i{0, 0, 0, 0};
            if (g + 1 < G) load_scales(sc, g + 1);
        }
        if (more) store_stage(buf ^ 1);
        __syncthreads();
    }

    float rn[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        rn[tn] = 0x1p-7f;
        if constexpr (FMT == kFmtU8)
            if (nval[tn]) rn[tn] = bf16_to_f32(rscale[ncol[tn]]) * 0x1p-7f;
    }
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = bm + wm * 64 + tm * 16 + 4 * qd + e;
            if (m >= M) continue;
            const float sm = scale[m];
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                if (nval[tn]) y[static_cast<int64_t>(m) * N + ncol[tn]] = F[tm][tn][e] * (sm * rn[tn]);
        }
}

template <int FMT>
hipError_t launch_gemm_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                         int32_t *P, hipStream_t st) {
    const int tiles_m = static_cast<int>((M + 127) / 128);
    const int tiles_n = static_cast<int>((w.N + 127) / 128);
    const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n;
    auto kern = P ? gemm_kernel<FMT, true> : gemm_kernel<FMT, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, q, s, w.codes,
                       w.gscale, w.rscale, y, P, static_cast<int>(M), static_cast<int>(w.N),
                       static_cast<int>(w.K), tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st) {
    return w.fmt == kFmtU8 ? launch_gemm_t<0>(q, s, w, y, M, partials, st)
                           : launch_gemm_t<1>(q, s, w, y, M, partials, st);
}

}  // namespace rad
