// gemm.hip -- rotated W8A8 contraction + epilogue for prefill sized batches on
// the int8 matrix cores (v_mfma_i32_32x32x32_i8, gfx950).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table rows "Weights" and "Activations"): exact int32 partials
// P of int8 activation codes times int8 weight codes per K group (256 with a
// u8 scale, 128 with a bf16 scale for the head), folded per group into f32
// accumulators F += float(P) * scale[n][g], then y = s_m * (r_n) * 2^-7 * F.
//
// Tiling: a 512-thread workgroup owns a 256 x 128 tile of y; its 8 waves
// (two per SIMD) own 64 x 64 sub-tiles, each a 2 x 2 grid of 32 x 32 MFMA
// tiles (64 int32 partials + 64 f32 accumulators per lane).  K is walked in
// 128-byte stages through a ring of 3 LDS buffers (144 KiB) filled by direct
// global -> LDS 16-byte loads, so two stages are always in flight while a
// third is consumed and no register holds staged data.  Each 128-byte row's
// eight 16-byte chunks are XOR-permuted by (row / 2) mod 8, so the 16 rows
// read by one ds_read_b128 phase cover all 64 banks.  A group's fold into F
// is issued tile by tile right before that tile's first MFMA of the next
// group, so the VALU work overlaps the matrix cores.
//
// Launch order is XCD-aware: workgroup b runs on XCD b % 8, and each XCD is
// handed a slab of 4 M-tiles x all N-tiles, walked M-fastest, so the ~32
// workgroups an XCD runs at once share their activation rows and weight
// columns in that XCD's L2.
#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kBM = 256, kBN = 128, kKC = 128;
constexpr int kThreads = 512;
constexpr int kGroupM = 4;   // M-tiles per XCD slab

__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int nt = tiles_m * tiles_n;
    int t = b;
    if (nt % 8 == 0) t = (b % 8) * (nt / 8) + b / 8;          // contiguous slab per XCD
    const int per_group = kGroupM * tiles_n;
    const int grp = t / per_group;
    const int first_m = grp * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int r = t - grp * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

constexpr int kStages = 3;
constexpr int kABytes = kBM * kKC, kBBytes = kBN * kKC;   // one stage of each operand
constexpr int kDmaA = kABytes / 1024 / 8;                 // 1 KiB loads per wave per stage
constexpr int kDmaB = kBBytes / 1024 / 8;
constexpr int kDmaPerStage = kDmaA + kDmaB;

// LDS layout of a 128-byte-deep operand stage: row r lives in 1 KiB block
// r / 8, chunk-major inside the block; logical 16-byte chunk c of row r sits
// at slot 8 * (c ^ ((r / 8) & 1)) + r % 8.  A ds_read_b128 phase (16 rows,
// one chunk) then covers all 64 banks, k-step kk of a fragment is a constant
// 256 * kk away from k-step 0, and one direct-load instruction fills one
// block: 8 rows x 128 contiguous bytes.
__device__ __forceinline__ int lds_row_base(int row, int c_lo) {
    return (row >> 3) * 1024 + 16 * (row & 7) + 128 * (c_lo ^ ((row >> 3) & 1));
}

template <int FMT, bool WRITE_P>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const int8_t *__restrict__ q,
                                                        const float *__restrict__ scale,
                                                        const int8_t *__restrict__ codes,
                                                        const void *__restrict__ gscale,
                                                        const uint16_t *__restrict__ rscale,
                                                        float *__restrict__ y,
                                                        int32_t *__restrict__ partials, int M, int N,
                                                        int K, int tiles_m, int tiles_n) {
    constexpr int GW = (FMT == kFmtU8) ? 256 : 128;
    constexpr int SPG = GW / kKC;                      // stages per group
    __shared__ __attribute__((aligned(1024))) int8_t As[kStages][kABytes];
    __shared__ __attribute__((aligned(1024))) int8_t Bs[kStages][kBBytes];
    // per group: each wave's 64 columns, one dword each (the dword that holds
    // the column's scale), filled by direct loads like the operands
    __shared__ __attribute__((aligned(256))) uint32_t Ss[kStages][8][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;            // 4 x 2 waves
    const int li = lane & 31, lq = lane >> 5;          // MFMA lane: row/col, k half
    int tmi, tni;
    tile_of(blockIdx.x, tiles_m, tiles_n, tmi, tni);
    const int bm = tmi * kBM, bn = tni * kBN;
    const int G = K / GW;
    const int NK = K / kKC;

    // ---- direct global -> LDS loads of one stage.  Wave w fills 1 KiB blocks
    // (8 rows x 128 B); lane l of a block is row l / 8, physical chunk l % 8,
    // and fetches the logical chunk that the swizzle puts there.  Rows past
    // M or N are clamped to the last row (never stored).
    // lane l of a block's load: row l % 8, physical chunk l / 8.  Sources are
    // a wave-uniform base (tile origin + k offset) plus a 32-bit lane offset.
    const int drow = lane & 7, dphys = lane >> 3;
    uint32_t aoffs[kDmaA], boffs[kDmaB];
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
        const int blk = wid * kDmaA + i, row = blk * 8 + drow;
        const int r_ = min(bm + row, M - 1) - bm;
        aoffs[i] = static_cast<uint32_t>(r_) * static_cast<uint32_t>(K) + 16u * (dphys ^ (blk & 1));
    }
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
        const int blk = wid * kDmaB + i, row = blk * 8 + drow;
        const int r_ = min(bn + row, N - 1) - bn;
        boffs[i] = static_cast<uint32_t>(r_) * static_cast<uint32_t>(K) + 16u * (dphys ^ (blk & 1));
    }
    const int8_t *abase = q + static_cast<int64_t>(bm) * K;
    const int8_t *bbase = codes + static_cast<int64_t>(bn) * K;
    // load j (0..5) of stage ks: 4 activation blocks, then 2 weight blocks
    auto issue_load = [&](int ks, int j) {
        const int buf = ks % kStages;
        if (j < kDmaA)
            g2lds_16(abase + static_cast<int64_t>(ks) * kKC + aoffs[j], &As[buf][(wid * kDmaA + j) * 1024]);
        else
            g2lds_16(bbase + static_cast<int64_t>(ks) * kKC + boffs[j - kDmaA],
                     &Bs[buf][(wid * kDmaB + j - kDmaA) * 1024]);
    };
    auto issue_stage = [&](int ks) {
#pragma unroll
        for (int j = 0; j < kDmaPerStage; ++j) issue_load(ks, j);
    };

    // ---- per-lane output columns and their group scales
    int ncol[2];
    bool nval[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        ncol[t] = bn + wn * 64 + t * 32 + li;
        nval[t] = ncol[t] < N;
    }
    constexpr int ESZ = (FMT == kFmtU8) ? 1 : 2;
    // scale of column c, group g: byte offset (c G + g) ESZ of gscale; the
    // wave's lane l fetches the aligned dword holding column wn*64 + l's
    // (the dword is moved back to end at the array's end if it would run past
    // it; the launcher guarantees the array holds at least 4 bytes)
    const int64_t sc_col = static_cast<int64_t>(min(bn + wn * 64 + lane, N - 1)) * G;
    const int64_t sc_last = static_cast<int64_t>(N) * G * ESZ - 4;
    auto dword_of = [&](int64_t byte) { return min(byte & ~static_cast<int64_t>(3), sc_last); };
    auto issue_scales = [&](int g) {
        g2lds_dword(static_cast<const uint8_t *>(gscale) + dword_of((sc_col + g) * ESZ),
                    &Ss[g % kStages][wid][0]);
    };
    // the two scales this lane folds for group g, read after that group's
    // scale loads are known to have landed
    auto read_scales = [&](int g, float (&sc)[2]) {
        uint32_t w0, w1;
        const uint32_t base = lds_offset(&Ss[g % kStages][wid][0]);
        asm volatile(
            "ds_read_b32 %0, %2\n\t"
            "ds_read_b32 %1, %3\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(w0), "=&v"(w1)
            : "v"(base + 4 * li), "v"(base + 4 * (32 + li))
            : "memory");
        const uint32_t w[2] = {w0, w1};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t c = static_cast<int64_t>(nval[t] ? ncol[t] : N - 1);
            const int64_t byte = (c * G + g) * ESZ;
            const int shift = static_cast<int>(byte - dword_of(byte)) * 8;
            if constexpr (FMT == kFmtU8)
                sc[t] = static_cast<float>((w[t] >> shift) & 0xFFu);
            else
                sc[t] = bf16_to_f32(static_cast<uint16_t>((w[t] >> shift) & 0xFFFFu));
        }
    };

    v16i P[2][2];
    float F[2][2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) F[a][b][e] = 0.0f;

    // element e of a 32x32 result sits at row 8 (e / 4) + 4 lq + e % 4, column li
    auto write_partials = [&](int tm, int tn, int g) {
        if (!nval[tn]) return;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = bm + wm * 64 + tm * 32 + 8 * (e >> 2) + 4 * lq + (e & 3);
            if (m < M) partials[(static_cast<int64_t>(m) * N + ncol[tn]) * G + g] = P[tm][tn][e];
        }
    };
    auto fold = [&](int tm, int tn, float s) {
#pragma unroll
        for (int e = 0; e < 16; ++e) F[tm][tn][e] += static_cast<float>(P[tm][tn][e]) * s;
    };

    // LDS byte offsets of this lane's fragments at k-step 0 of a stage
    // (k-step kk adds 256 * kk): rows of the wave's 32 x 32 tiles, chunk lq
    int aoff[2], boff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        aoff[t] = lds_row_base(wm * 64 + t * 32 + li, lq);
        boff[t] = lds_row_base(wn * 64 + t * 32 + li, lq);
    }

#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) P[a][b] = v16i{};

    // Issue order (all vector-memory operations are direct LDS loads, so the
    // only waits are the explicit ones below):
    //   head format (one stage per group): group g's scales are issued in
    //     stage g - 1 (group 0's before stage 0), ahead of that stage's load;
    //   u8 format (two stages per group): group g's scales are issued in the
    //     group's first stage, ahead of that stage's load.
    // Either way they land before the stage whose wait precedes their fold.
    if constexpr (SPG == 1) issue_scales(0);
    issue_stage(0);
    if (NK > 1) issue_stage(1);

    for (int ks = 0; ks < NK; ++ks) {
        const int st = (SPG == 1) ? 0 : (ks & 1);      // stage within its group
        const int g = (SPG == 1) ? ks : (ks >> 1);
        // stage ks has landed once no more than the loads issued after it
        // are pending: the next stage's 6, plus one scale load if the
        // previous stage issued one
        if (ks + 1 >= NK) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (ks == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerStage) : "memory");
        else if (SPG == 1 || st == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerStage + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerStage) : "memory");
        // all waves' loads of stage ks are in LDS, and all waves are done
        // reading stage ks - 1, whose buffer the next issue overwrites
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (SPG == 1) {
            if (g + 1 < G) issue_scales(g + 1);
        } else {
            if (st == 0) issue_scales(g);
        }
        const bool more = ks + 2 < NK;
        const bool fold_now = st == 0 && g > 0;
        float scf[2] = {0.0f, 0.0f};
        if (fold_now) read_scales(g - 1, scf);
        const uint32_t Ab = lds_offset(As[ks % kStages]);
        const uint32_t Bb = lds_offset(Bs[ks % kStages]);
#pragma unroll
        for (int kk = 0; kk < kKC / 32; ++kk) {
            v4i a[2], b[2];
            lds_read4_b128(a[0], a[1], b[0], b[1], Ab + aoff[0] + 256 * kk,
                           Ab + aoff[1] + 256 * kk, Bb + boff[0] + 256 * kk,
                           Bb + boff[1] + 256 * kk);
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    if (kk == 0 && st == 0) {
                        // fold group g - 1 (all zero when g == 0), restart P
                        if constexpr (WRITE_P) {
                            if (g > 0) write_partials(tm, tn, g - 1);
                        }
                        fold(tm, tn, scf[tn]);
                        P[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[tm], b[tn], v16i{}, 0, 0, 0);
                    } else {
                        P[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[tm], b[tn], P[tm][tn], 0, 0, 0);
                    }
                }
            // the next-but-one stage's loads, spread over the k-steps so a
            // full memory queue delays a few matrix ops, not the whole stage
            if (more && kk < 3) {
                issue_load(ks + 2, 2 * kk);
                issue_load(ks + 2, 2 * kk + 1);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last group's scales
    {
        float scf[2];
        read_scales(G - 1, scf);
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                if constexpr (WRITE_P) write_partials(tm, tn, G - 1);
                fold(tm, tn, scf[tn]);
            }
    }

    float rn[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        rn[t] = 0x1p-7f;
        if constexpr (FMT == kFmtU8)
            if (nval[t]) rn[t] = bf16_to_f32(rscale[ncol[t]]) * 0x1p-7f;
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = bm + wm * 64 + tm * 32 + 8 * (e >> 2) + 4 * lq + (e & 3);
            if (m >= M) continue;
            const float sm = scale[m];
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
                if (nval[tn]) y[static_cast<int64_t>(m) * N + ncol[tn]] = F[tm][tn][e] * (sm * rn[tn]);
        }
}

template <int FMT>
hipError_t launch_gemm_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                         int32_t *P, hipStream_t st) {
    const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
    const int tiles_n = static_cast<int>((w.N + kBN - 1) / kBN);
    const int64_t grid = static_cast<int64_t>(tiles_m) * tiles_n;
    auto kern = P ? gemm_kernel<FMT, true> : gemm_kernel<FMT, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, st, q, s, w.codes,
                       w.gscale, w.rscale, y, P, static_cast<int>(M), static_cast<int>(w.N),
                       static_cast<int>(w.K), tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st) {
    const int64_t scale_bytes = w.N * (w.K / (w.fmt == kFmtU8 ? 256 : 128)) * (w.fmt == kFmtU8 ? 1 : 2);
    if (scale_bytes < 4) {
        // too few group scales for the kernel's dword scale loads: run the
        // batch through the M <= 128 path, 128 tokens at a time
        const int64_t G = w.K / (w.fmt == kFmtU8 ? 256 : 128);
        for (int64_t m0 = 0; m0 < M; m0 += 128) {
            const int64_t mc = M - m0 < 128 ? M - m0 : 128;
            hipError_t e = launch_gemv(q + m0 * w.K, s + m0, w, y + m0 * w.N, mc,
                                       partials ? partials + m0 * w.N * G : nullptr, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    return w.fmt == kFmtU8 ? launch_gemm_t<0>(q, s, w, y, M, partials, st)
                           : launch_gemm_t<1>(q, s, w, y, M, partials, st);
}

}  // namespace rad
