// skinny_lds.hip -- rotated W8A8 contraction + epilogue for 33..64 tokens
// with both operands staged through LDS (gfx950).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table rows "Weights" and "Activations"): exact int32 partials
// of int8 activation codes times int8 weight codes per K group (256 with a u8
// scale and a bf16 row scale, or 128 with a bf16 scale for the head), folded
// per group into f32, then y = s_m * (r_n) * 2^-7 * sum_g scale[n][g] * P.
//
// A 512-thread workgroup owns 128 weight rows and all (up to 64) tokens.  K
// is walked in 256-byte stages through a 3-deep LDS ring filled by direct
// global -> LDS 16-byte loads: one load instruction covers four rows x 256
// contiguous bytes (the weight stream is the cost, and it streams fastest in
// long runs per row), activation rows likewise.  Wave w computes its 16
// weight rows against the 64 token rows with v_mfma_i32_16x16x64_i8 (A =
// tokens, B = weights; lane j + 16 q holds chunk 4 kk + q of row j for k-step
// kk, on both operands, so each matrix op sums the 64 products of its
// k-step).  Each group's partials are folded into f32 when the group ends.
// Each wave also loads its rows' group-scale dword per stage into LDS with a
// direct load, so the only vector-memory operations of the loop are these
// direct loads and the explicit waits below count them exactly.
//
// LDS: row r of a stage occupies 256 bytes; its logical 16-byte chunk c sits
// in slot c ^ (r & 7), so the eight rows an operand read covers at a time hit
// eight different 16-byte slots of a 128-byte bank line.
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kSlWaves = 8;                        // 8 waves x 16 weight rows
constexpr int kSlBN = 16 * kSlWaves;               // weight rows per workgroup
constexpr int kSlMP = 64;                          // token rows (padded)
constexpr int kSlKC = 256;                         // K bytes per stage
constexpr int kSlStages = 3;
constexpr int kSlA = kSlMP * kSlKC;                // 16 KiB
constexpr int kSlB = kSlBN * kSlKC;                // 32 KiB
constexpr int kSlDmaA = kSlA / 1024 / kSlWaves;    // 1 KiB loads per wave per stage
constexpr int kSlDmaB = kSlB / 1024 / kSlWaves;
constexpr int kSlDma = kSlDmaA + kSlDmaB + 1;      // + the scale dword load
static_assert(kSlDmaA * kSlWaves * 1024 == kSlA && kSlDmaB * kSlWaves * 1024 == kSlB, "stage split");

__device__ __forceinline__ int sl_addr(int row, int c) { return 256 * row + 16 * (c ^ (row & 7)); }

template <int FMT, bool WRITE_P>
__global__ __launch_bounds__(64 * kSlWaves) void skinny_lds_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ scale, const int8_t *__restrict__ codes,
    const void *__restrict__ gscale, const uint16_t *__restrict__ rscale, float *__restrict__ y,
    int32_t *__restrict__ partials, int M, int N, int K) {
    constexpr int GPS = (FMT == kFmtU8) ? 1 : 2;      // groups per stage
    constexpr int KPG = 4 / GPS;                       // k-steps per group
    constexpr int ESZ = (FMT == kFmtU8) ? 1 : 2;       // bytes per group scale
    __shared__ __attribute__((aligned(1024))) int8_t As[kSlStages][kSlA];
    __shared__ __attribute__((aligned(1024))) int8_t Bs[kSlStages][kSlB];
    __shared__ __attribute__((aligned(256))) uint32_t Ss[kSlStages][kSlWaves][64];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wid);
    const int j = lane & 15, qd = lane >> 4;
    const int n0 = static_cast<int>(blockIdx.x) * kSlBN;
    const int NS = K / kSlKC;
    const int G = K / (kSlKC / GPS);

    // ---- direct loads of one stage.  Load i of wave w fills 1 KiB block b:
    // four rows 4 b .. 4 b + 3 (lane l: row 4 b + l / 16, slot l % 16, i.e.
    // logical chunk (l % 16) ^ (row & 7)).  Rows past M or N repeat the last
    // row (never stored).
    const int dr = lane >> 4, dslot = lane & 15;
    uint32_t aoffs[kSlDmaA], boffs[kSlDmaB];
#pragma unroll
    for (int i = 0; i < kSlDmaA; ++i) {
        const int row = 4 * (wid * kSlDmaA + i) + dr;
        aoffs[i] = static_cast<uint32_t>(min(row, M - 1)) * static_cast<uint32_t>(K) +
                   16u * static_cast<uint32_t>(dslot ^ (row & 7));
    }
#pragma unroll
    for (int i = 0; i < kSlDmaB; ++i) {
        const int row = 4 * (wid * kSlDmaB + i) + dr;
        boffs[i] = static_cast<uint32_t>(min(n0 + row, N - 1) - n0) * static_cast<uint32_t>(K) +
                   16u * static_cast<uint32_t>(dslot ^ (row & 7));
    }
    const int8_t *bbase = codes + static_cast<int64_t>(n0) * K;
    // the scale dword of this lane's row for stage s: u8, byte n G + s; head,
    // bytes of groups 2 s and 2 s + 1 (4-byte aligned: G is even).  A dword
    // that would run past the array is moved back to end at its end (the
    // launcher guarantees the array holds at least 4 bytes).
    const int nrow = n0 + 16 * wid + j;
    const bool nvalid = nrow < N;
    const int64_t sc_row = static_cast<int64_t>(min(nrow, N - 1)) * G;
    const int64_t sc_last = static_cast<int64_t>(N) * G * ESZ - 4;
    auto sc_byte = [&](int s) -> int64_t { return (sc_row + static_cast<int64_t>(GPS) * s) * ESZ; };
    auto sc_dword = [&](int s) -> int64_t { return min(sc_byte(s) & ~static_cast<int64_t>(3), sc_last); };

    // stages past the end re-load the last one into a buffer nobody reads
    // again, so every wait count below is uniform
    auto issue_stage = [&](int s) {
        const int sc = min(s, NS - 1);
        const int buf = s % kSlStages;
#pragma unroll
        for (int i = 0; i < kSlDmaA; ++i)
            dma16(q + static_cast<int64_t>(sc) * kSlKC, aoffs[i],
                  lds_offset(&As[buf][(wu * kSlDmaA + i) * 1024]));
#pragma unroll
        for (int i = 0; i < kSlDmaB; ++i)
            dma16(bbase + static_cast<int64_t>(sc) * kSlKC, boffs[i],
                  lds_offset(&Bs[buf][(wu * kSlDmaB + i) * 1024]));
        dma4(gscale, static_cast<uint32_t>(sc_dword(sc)), lds_offset(&Ss[buf][wu][0]));
    };

    v4i P[4];
    float F[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        P[mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) F[mb][e] = 0.0f;
    }

    // LDS offsets of this lane's fragments at k-step 0 (row j of each 16-row
    // block, chunk qd); k-step kk reads chunk 4 kk + qd, i.e. offset XOR 64 kk
    int aoff[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) aoff[mb] = sl_addr(16 * mb + j, qd);
    const int boff = sl_addr(16 * wid + j, qd);

    issue_stage(0);
    issue_stage(1);
    for (int s = 0; s < NS; ++s) {
        // stage s has landed once at most the next stage's loads remain
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSlDma) : "memory");
        // every wave's loads of stage s are in LDS, and every wave is done
        // with stage s - 1, whose buffer the next issue overwrites
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_stage(s + 2);
        const int buf = s % kSlStages;
        const int8_t *Ab = As[buf];
        const int8_t *Bb = Bs[buf];
        const uint32_t sw = Ss[buf][wid][j];
        const int shift = static_cast<int>(sc_byte(s) - sc_dword(s)) * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const v4i b = *reinterpret_cast<const v4i *>(Bb + (boff ^ (64 * kk)));
            v4i a[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) a[mb] = *reinterpret_cast<const v4i *>(Ab + (aoff[mb] ^ (64 * kk)));
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                P[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb], b, (kk % KPG == 0) ? v4i{0, 0, 0, 0} : P[mb],
                                                               0, 0, 0);
            if (kk % KPG == KPG - 1) {
                const int gi = kk / KPG;                 // group inside the stage
                float sc;
                if constexpr (FMT == kFmtU8)
                    sc = static_cast<float>((sw >> shift) & 0xFFu);
                else
                    sc = bf16_to_f32(static_cast<uint16_t>((sw >> (shift + 16 * gi)) & 0xFFFFu));
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) F[mb][e] += static_cast<float>(P[mb][e]) * sc;
                    if constexpr (WRITE_P) {
                        const int g = GPS * s + gi;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = 16 * mb + 4 * qd + e;
                            if (m < M && nvalid)
                                partials[(static_cast<int64_t>(m) * N + nrow) * G + g] = P[mb][e];
                        }
                    }
                }
            }
        }
    }
    // every load has landed (the re-loads past the end included: nothing may
    // still write this workgroup's LDS once its waves end)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!nvalid) return;
    float rn = 0x1p-7f;
    if constexpr (FMT == kFmtU8) rn = bf16_to_f32(rscale[nrow]) * 0x1p-7f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mb + 4 * qd + e;
            if (m < M) y[static_cast<int64_t>(m) * N + nrow] = F[mb][e] * (scale[m] * rn);
        }
}

template <int FMT>
hipError_t launch_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                    int32_t *P, hipStream_t st) {
    const int64_t grid = (w.N + kSlBN - 1) / kSlBN;
    auto kern = P ? skinny_lds_kernel<FMT, true> : skinny_lds_kernel<FMT, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(64 * kSlWaves), 0, st, q, s, w.codes,
                       w.gscale, w.rscale, y, P, static_cast<int>(M), static_cast<int>(w.N),
                       static_cast<int>(w.K));
    return hipGetLastError();
}

}  // namespace

bool skinny_lds_supported(const WeightArgs &w, int64_t M) {
    if (M < 33 || M > kSlMP || w.K % kSlKC != 0) return false;
    if (w.fmt == kFmtU8) return w.N * (w.K / 256) >= 4;
    if (w.fmt == 1) return (w.K / 128) % 2 == 0;   // head: the stage's two scales share a dword
    return false;
}

hipError_t launch_skinny_lds(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                             int32_t *partials, hipStream_t st) {
    return w.fmt == kFmtU8 ? launch_t<0>(q, s, w, y, M, partials, st)
                           : launch_t<1>(q, s, w, y, M, partials, st);
}

}  // namespace rad
