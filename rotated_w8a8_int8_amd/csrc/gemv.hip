// gemv.hip -- rotated W8A8 contraction + epilogue for decode/verify sized
// batches (M <= 128), weight-bandwidth bound (gfx950).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table rows "Weights" and "Activations"): int8 activation codes
// times int8 weight codes of the same rotated domain, exact int32 sums per
// group of K (256 with a u8 scale, or 128 with a bf16 scale for the head),
// then y = s_m * (r_n) * 2^-7 * sum_g scale[n][g] * P[m][n][g].
//
// Two kernels:
//   gemv_m1_kernel   M == 1.  Each wave streams whole weight rows with fully
//                    coalesced 16-byte loads (a wave reads 1 KiB contiguous per
//                    load instruction) and v_dot4 against activation codes held
//                    in registers.  For the u8 format the epilogue is exact
//                    integer arithmetic up to one f64 product, rounded once.
//   skinny_kernel    2 <= M <= 128.  Each wave owns 16 weight rows and streams
//                    them straight from HBM into the B operand of
//                    v_mfma_i32_16x16x64_i8; the activation codes of all M
//                    tokens are staged per K group in LDS and shared by the
//                    workgroup's 4 waves.
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kFmtHead = 1;

// ------------------------------------------------------------- M == 1 ----
// Lane l of a wave handles 16-byte chunks c = l + 64 t (t < CPL) of every row;
// chunk c lies in group c / (GW/16).  U rows are in flight per buffer and two
// buffers alternate, so 2*U*CPL 16-byte loads per lane can be outstanding.
template <int FMT, int CPL, int U, bool WRITE_P>
__global__ __launch_bounds__(256) void gemv_m1_kernel(const int8_t *__restrict__ q,
                                                      const float *__restrict__ scale,
                                                      const int8_t *__restrict__ codes,
                                                      const void *__restrict__ gscale,
                                                      const uint16_t *__restrict__ rscale,
                                                      float *__restrict__ y,
                                                      int32_t *__restrict__ partials, int N, int K,
                                                      int rpw) {
    constexpr int GW16 = (FMT == kFmtU8) ? 16 : 8;   // chunks per group
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int n_begin = wave * rpw;
    if (n_begin >= N) return;
    const int n_end = min(n_begin + rpw, N);
    const int nchunk = K >> 4;
    const int G = nchunk / GW16;

    v4i a[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int c = lane + 64 * t;
        a[t] = (c < nchunk) ? ld16(q + 16 * c) : v4i{0, 0, 0, 0};
    }
    const float s = scale[0];

    auto load_rows = [&](v4i (&w)[U][CPL], int n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int nn = n + u;
            const int8_t *row = codes + static_cast<int64_t>(nn) * K;
#pragma unroll
            for (int t = 0; t < CPL; ++t) {
                const int c = lane + 64 * t;
                w[u][t] = (nn < n_end && c < nchunk) ? ld16(row + 16 * c) : v4i{0, 0, 0, 0};
            }
        }
    };

    auto finish_rows = [&](const v4i (&w)[U][CPL], int n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int nn = n + u;
            if (nn >= n_end) break;                       // wave-uniform
            if constexpr (FMT == kFmtU8) {
                const uint8_t *g8 = static_cast<const uint8_t *>(gscale) + static_cast<int64_t>(nn) * G;
                int acc = 0;                              // |acc| <= CPL * 258064 * 255 < 2^31
#pragma unroll
                for (int t = 0; t < CPL; ++t) {
                    const int c = lane + 64 * t;
                    if (c < nchunk) {
                        const int p = dot16_i8(w[u][t], a[t], 0);
                        const int g = c / GW16;
                        acc += p * static_cast<int>(g8[g]);
                        if constexpr (WRITE_P) {
                            const int pg = row16_sum(p);
                            if ((lane & 15) == 0) partials[static_cast<int64_t>(nn) * G + g] = pg;
                        }
                    }
                }
                // exact 64-lane sum: split into 16-bit halves that cannot overflow
                const int hi = wave_sum_i32(acc >> 16);
                const int lo = wave_sum_i32(acc & 0xFFFF);
                if (lane == 0) {
                    const int64_t S = static_cast<int64_t>(hi) * 65536 + lo;
                    const double r = static_cast<double>(bf16_to_f32(rscale[nn]));
                    y[nn] = static_cast<float>(static_cast<double>(s) * r * 0x1p-7 * static_cast<double>(S));
                }
            } else {
                const uint16_t *gb = static_cast<const uint16_t *>(gscale) + static_cast<int64_t>(nn) * G;
                float acc = 0.0f;
#pragma unroll
                for (int t = 0; t < CPL; ++t) {
                    const int c = lane + 64 * t;
                    if (c < nchunk) {
                        const int p = dot16_i8(w[u][t], a[t], 0);
                        const int g = c / GW16;
                        acc += static_cast<float>(p) * bf16_to_f32(gb[g]);
                        if constexpr (WRITE_P) {
                            const int pg = row8_sum(p);
                            if ((lane & 7) == 0) partials[static_cast<int64_t>(nn) * G + g] = pg;
                        }
                    }
                }
                const float tot = wave_sum_f32(acc);
                if (lane == 0) y[nn] = (s * 0x1p-7f) * tot;
            }
        }
    };

    v4i w0[U][CPL], w1[U][CPL];
    load_rows(w0, n_begin);
    for (int n = n_begin; n < n_end; n += 2 * U) {
        if (n + U < n_end) load_rows(w1, n + U);
        finish_rows(w0, n);
        if (n + U >= n_end) break;
        if (n + 2 * U < n_end) load_rows(w0, n + 2 * U);
        finish_rows(w1, n + U);
    }
}

template <int FMT, int CPL>
hipError_t launch_m1_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int32_t *P,
                       hipStream_t st) {
    constexpr int U = (CPL <= 4) ? 4 : (CPL <= 8 ? 2 : 1);
    const int N = static_cast<int>(w.N);
    // Aim for 8 waves per CU on 256 CUs, equal rows per wave.
    const int target_waves = 256 * 8;
    int rpw = (N + target_waves - 1) / target_waves;
    if (rpw < 1) rpw = 1;
    const int waves = (N + rpw - 1) / rpw;
    const int grid = (waves + 3) / 4;
    auto kern = P ? gemv_m1_kernel<FMT, CPL, U, true> : gemv_m1_kernel<FMT, CPL, U, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, q, s, w.codes, w.gscale, w.rscale, y, P,
                       N, static_cast<int>(w.K), rpw);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_m1(const int8_t *q, const float *s, const WeightArgs &w, float *y, int32_t *P,
                     hipStream_t st) {
    const int cpl = static_cast<int>((w.K / 16 + 63) / 64);
    switch (cpl) {
        case 1: return launch_m1_t<FMT, 1>(q, s, w, y, P, st);
        case 2: return launch_m1_t<FMT, 2>(q, s, w, y, P, st);
        case 3: return launch_m1_t<FMT, 3>(q, s, w, y, P, st);
        case 4: return launch_m1_t<FMT, 4>(q, s, w, y, P, st);
        case 5: return launch_m1_t<FMT, 5>(q, s, w, y, P, st);
        case 6: return launch_m1_t<FMT, 6>(q, s, w, y, P, st);
        case 7: case 8: return launch_m1_t<FMT, 8>(q, s, w, y, P, st);
        case 9: case 10: case 11: case 12: return launch_m1_t<FMT, 12>(q, s, w, y, P, st);
        case 13: case 14: case 15: case 16: return launch_m1_t<FMT, 16>(q, s, w, y, P, st);
        case 17: return launch_m1_t<FMT, 17>(q, s, w, y, P, st);
        case 18: case 19: case 20: case 21: case 22: case 23: case 24:
            return launch_m1_t<FMT, 24>(q, s, w, y, P, st);
        default: return launch_m1_t<FMT, 32>(q, s, w, y, P, st);
    }
}

// ------------------------------------------------------- 2 <= M <= 128 ----
// Workgroup = 4 waves = 64 weight rows.  Lane L = j + 16 qd of a wave holds,
// for MFMA step st of a K group, bytes [64 st + 16 qd, +16) of weight row
// n0 + j (B operand) and of token mb*16 + j (A operand, from LDS).  Both
// operands use the same byte-to-k assignment, so each MFMA sums exactly the
// 64 products of its step.  The int32 result D[i][j] sits in lane
// j + 16 (i / 4), element i % 4: token mb*16 + 4 qd + e, weight row n0 + j.
template <int FMT, int MB, bool WRITE_P>
__global__ __launch_bounds__(256) void skinny_kernel(const int8_t *__restrict__ q,
                                                     const float *__restrict__ scale,
                                                     const int8_t *__restrict__ codes,
                                                     const void *__restrict__ gscale,
                                                     const uint16_t *__restrict__ rscale,
                                                     float *__restrict__ y,
                                                     int32_t *__restrict__ partials, int M, int N,
                                                     int K) {
    constexpr int GW = (FMT == kFmtU8) ? 256 : 128;   // K bytes per group = per LDS stage
    constexpr int SPG = GW / 64;                      // MFMA steps per group
    constexpr int LDA = GW + 16;                      // padded LDS pitch (bytes)
    constexpr int ROWS = MB * 16;
    constexpr int CH = ROWS * GW / 16;                // 16-byte chunks per stage
    constexpr int CPT = (CH + 255) / 256;             // chunks per thread
    __shared__ __attribute__((aligned(16))) int8_t As[2][ROWS * LDA];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = lane & 15;
    const int qd = lane >> 4;
    const int n0 = blockIdx.x * 64 + (tid >> 6) * 16;
    const int nrow = n0 + j;
    const bool nvalid = nrow < N;
    const int8_t *wrow = codes + static_cast<int64_t>(nvalid ? nrow : 0) * K + 16 * qd;
    const int G = K / GW;

    auto load_b = [&](v4i (&b)[SPG], int g) {
#pragma unroll
        for (int st = 0; st < SPG; ++st)
            b[st] = nvalid ? ld16(wrow + static_cast<int64_t>(g) * GW + 64 * st) : v4i{0, 0, 0, 0};
    };
    auto load_a = [&](v4i (&ar)[CPT], int g) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx / (GW / 16);
            const int kb = (idx % (GW / 16)) * 16;
            ar[i] = (idx < CH && row < M)
                        ? ld16(q + static_cast<int64_t>(row) * K + static_cast<int64_t>(g) * GW + kb)
                        : v4i{0, 0, 0, 0};
        }
    };
    auto store_a = [&](const v4i (&ar)[CPT], int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + 256 * i;
            if (idx < CH) {
                const int row = idx / (GW / 16);
                const int kb = (idx % (GW / 16)) * 16;
                *reinterpret_cast<v4i *>(&As[buf][row * LDA + kb]) = ar[i];
            }
        }
    };
    auto load_scale = [&](int g) -> float {
        if (!nvalid) return 0.0f;
        if constexpr (FMT == kFmtU8)
            return static_cast<float>(static_cast<const uint8_t *>(gscale)[static_cast<int64_t>(nrow) * G + g]);
        else
            return bf16_to_f32(static_cast<const uint16_t *>(gscale)[static_cast<int64_t>(nrow) * G + g]);
    };

    float F[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) F[mb][e] = 0.0f;

    v4i bcur[SPG], bnext[SPG], ar[CPT];
    load_b(bcur, 0);
    load_a(ar, 0);
    float sc = load_scale(0);
    store_a(ar, 0);
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        const bool more = g + 1 < G;
        float sc_next = 0.0f;
        if (more) {
            load_b(bnext, g + 1);
            load_a(ar, g + 1);
            sc_next = load_scale(g + 1);
        }
        v4i P[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) P[mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < SPG; ++st) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const v4i af = *reinterpret_cast<const v4i *>(&As[buf][(mb * 16 + j) * LDA + 64 * st + 16 * qd]);
                P[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bcur[st], P[mb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            F[mb][0] += static_cast<float>(P[mb].x) * sc;
            F[mb][1] += static_cast<float>(P[mb].y) * sc;
            F[mb][2] += static_cast<float>(P[mb].z) * sc;
            F[mb][3] += static_cast<float>(P[mb].w) * sc;
        }
        if (WRITE_P && nvalid) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int pv[4] = {P[mb].x, P[mb].y, P[mb].z, P[mb].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = mb * 16 + 4 * qd + e;
                    if (m < M) partials[(static_cast<int64_t>(m) * N + nrow) * G + g] = pv[e];
                }
            }
        }
        if (more) {
            store_a(ar, buf ^ 1);
#pragma unroll
            for (int st = 0; st < SPG; ++st) bcur[st] = bnext[st];
            sc = sc_next;
        }
        __syncthreads();
    }

    if (!nvalid) return;
    float rn = 0x1p-7f;
    if constexpr (FMT == kFmtU8) rn = bf16_to_f32(rscale[nrow]) * 0x1p-7f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = mb * 16 + 4 * qd + e;
            if (m < M) y[static_cast<int64_t>(m) * N + nrow] = F[mb][e] * (scale[m] * rn);
        }
}

template <int FMT, int MB>
hipError_t launch_skinny_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                           int32_t *P, hipStream_t st) {
    const int grid = static_cast<int>((w.N + 63) / 64);
    auto kern = P ? skinny_kernel<FMT, MB, true> : skinny_kernel<FMT, MB, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, q, s, w.codes, w.gscale, w.rscale, y, P,
                       static_cast<int>(M), static_cast<int>(w.N), static_cast<int>(w.K));
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_skinny(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                         int32_t *P, hipStream_t st) {
    switch ((M + 15) / 16) {
        case 1: return launch_skinny_t<FMT, 1>(q, s, w, y, M, P, st);
        case 2: return launch_skinny_t<FMT, 2>(q, s, w, y, M, P, st);
        case 3: return launch_skinny_t<FMT, 3>(q, s, w, y, M, P, st);
        case 4: return launch_skinny_t<FMT, 4>(q, s, w, y, M, P, st);
        case 5: return launch_skinny_t<FMT, 5>(q, s, w, y, M, P, st);
        case 6: return launch_skinny_t<FMT, 6>(q, s, w, y, M, P, st);
        case 7: return launch_skinny_t<FMT, 7>(q, s, w, y, M, P, st);
        default: return launch_skinny_t<FMT, 8>(q, s, w, y, M, P, st);
    }
}

}  // namespace

hipError_t launch_gemv(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st) {
    if (M == 1 && w.K <= 32768) {
        return w.fmt == kFmtU8 ? launch_m1<kFmtU8>(q, s, w, y, partials, st)
                               : launch_m1<kFmtHead>(q, s, w, y, partials, st);
    }
    return w.fmt == kFmtU8 ? launch_skinny<kFmtU8>(q, s, w, y, M, partials, st)
                           : launch_skinny<kFmtHead>(q, s, w, y, M, partials, st);
}

}  // namespace rad
