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
// tiles (per lane: 2 x 64 int32 partials, 64 f32 accumulators).  K is walked
// in 128-byte stages through a ring of 3 LDS buffers (144 KiB) filled by
// direct global -> LDS 16-byte loads, so two stages are in flight while a
// third is consumed and no register holds staged data.  Each 128-byte row's
// eight 16-byte chunks are XOR-permuted (row-dependent), so the rows one
// ds_read_b128 phase reads cover all banks, while each direct load still
// reads whole 128-byte row segments with consecutive lanes.  The per-group
// fold (convert + multiply-add per partial) is VALU work of about half the
// matrix time: partials are double-buffered by group parity so that a
// group's fold runs one tile at a time under the next group's matrix ops.
//
// Launch order is XCD-aware: workgroup b runs on XCD b % 8, and each XCD is
// handed a slab of 4 M-tiles x all N-tiles, walked M-fastest, so the ~32
// workgroups an XCD runs at once share their activation rows and weight
// columns in that XCD's L2.
//
// On random codes the chip runs this kernel at its power limit (1400 W, the
// core clock well below its 2.4 GHz maximum), so the time per call follows
// the energy spent per operation rather than the issue schedule alone.
#include <type_traits>

#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kFmtTbl4 = 2;
constexpr int kBM = 256, kBN = 128, kKC = 128;
constexpr int kWavesM = 4, kWavesN = 2;        // 8 waves, two per SIMD
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWTM = kBM / kWavesM, kWTN = kBN / kWavesN;   // wave tile 64 x 64
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;             // of 32 x 32 MFMA tiles
static_assert(kWTN == 64, "one scale dword per lane covers a wave tile's columns");
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
constexpr int kStageBytes = kABytes + kBBytes;            // a stage: A rows, then B rows
constexpr int kDmaA = kABytes / 1024 / kWaves;            // 1 KiB loads per wave per stage
constexpr int kDmaB = kBBytes / 1024 / kWaves;
constexpr int kDmaPerStage = kDmaA + kDmaB;

// LDS layout of a 128-byte-deep operand stage: row r occupies bytes
// 128 r .. 128 r + 127 (one direct-load instruction fills 8 whole rows, 8
// lanes per row, so each lane quad reads 64 contiguous bytes of one row and
// the loads coalesce), with its logical 16-byte chunk c stored in slot
// c ^ swz(r), swz(r) = (r mod 8) ^ ((r / 8) mod 2).  Fragment reads fetch
// one chunk of consecutive rows: any 8 aligned consecutive rows then hit 8
// different 16-byte slots of a 128-byte bank line, and any 16 hit all 16
// slots of a 256-byte line (rows of equal parity differ in the swizzle).
__device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// 16-byte LDS read at a byte address.
typedef __attribute__((address_space(3))) const v4i lds_v4i;
__device__ __forceinline__ v4i lds_ld16(uint32_t addr) {
    return *reinterpret_cast<lds_v4i *>(addr);
}
__device__ __forceinline__ int lds_chunk_addr(int row, int c) {
    return 128 * row + 16 * (c ^ lds_swz(row));
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
    // one allocation, so every fragment address is a uniform stage base plus
    // one per-lane offset (one VALU op per read)
    __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStageBytes];
    // per group: each wave's 64 columns, one dword each (the dword that holds
    // the column's scale), filled by direct loads like the operands
    __shared__ __attribute__((aligned(256))) uint32_t Ss[kStages][kWaves][kWTN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wid);  // the same, known uniform
    const int wm = wid / kWavesN, wn = wid % kWavesN;
    const int li = lane & 31, lq = lane >> 5;          // MFMA lane: row/col, k half
    int tmi, tni;
    tile_of(blockIdx.x, tiles_m, tiles_n, tmi, tni);
    const int bm = tmi * kBM, bn = tni * kBN;
    const int G = K / GW;
    const int NK = K / kKC;

    // ---- direct global -> LDS loads of one stage.  Wave w fills 1 KiB blocks
    // (8 rows x 128 B); lane l of a block's load is row l / 8, physical slot
    // l % 8, and fetches the logical chunk the swizzle puts in that slot.
    // Sources are a wave-uniform base (tile origin + k offset) plus a 32-bit
    // lane offset; rows past M or N are clamped to the last row (never
    // stored).
    const int drow = lane >> 3, dphys = lane & 7;
    uint32_t aoffs[kDmaA], boffs[kDmaB];
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
        const int blk = wid * kDmaA + i, row = blk * 8 + drow;
        const int r_ = min(bm + row, M - 1) - bm;
        aoffs[i] = static_cast<uint32_t>(r_) * static_cast<uint32_t>(K) + 16u * (dphys ^ lds_swz(row));
    }
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
        const int blk = wid * kDmaB + i, row = blk * 8 + drow;
        const int r_ = min(bn + row, N - 1) - bn;
        boffs[i] = static_cast<uint32_t>(r_) * static_cast<uint32_t>(K) + 16u * (dphys ^ lds_swz(row));
    }
    const int8_t *abase = q + static_cast<int64_t>(bm) * K;
    const int8_t *bbase = codes + static_cast<int64_t>(bn) * K;
    // load j of stage ks: kDmaA activation blocks, then kDmaB weight blocks.
    // Stages past the end re-load the last stage (in bounds) into a buffer
    // nobody reads again, which keeps every wait count below uniform.
    auto issue_load = [&](int ks, int j) {
        const int kc = min(ks, NK - 1);
        const int buf = ks % kStages;
        if (j < kDmaA)
            dma16(abase + static_cast<int64_t>(kc) * kKC, aoffs[j],
                  lds_offset(&smem[buf * kStageBytes + (wu * kDmaA + j) * 1024]));
        else
            dma16(bbase + static_cast<int64_t>(kc) * kKC, boffs[j - kDmaA],
                  lds_offset(&smem[buf * kStageBytes + kABytes + (wu * kDmaB + j - kDmaA) * 1024]));
    };
    auto issue_stage = [&](int ks) {
#pragma unroll
        for (int j = 0; j < kDmaPerStage; ++j) issue_load(ks, j);
    };

    // ---- per-lane output columns and their group scales
    int ncol[kTN];
    bool nval[kTN];
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
        ncol[t] = bn + wn * kWTN + t * 32 + li;
        nval[t] = ncol[t] < N;
    }
    constexpr int ESZ = (FMT == kFmtU8) ? 1 : 2;
    // scale of column c, group g: byte offset (c G + g) ESZ of gscale; the
    // wave's lane l fetches the aligned dword holding column wn*kWTN + l's
    // (the dword is moved back to end at the array's end if it would run past
    // it; the launcher guarantees the array holds at least 4 bytes)
    const int64_t sc_col = static_cast<int64_t>(min(bn + wn * kWTN + lane, N - 1)) * G;
    const int64_t sc_last = static_cast<int64_t>(N) * G * ESZ - 4;
    auto dword_of = [&](int64_t byte) { return min(byte & ~static_cast<int64_t>(3), sc_last); };
    auto issue_scales = [&](int g) {
        dma4(gscale, static_cast<uint32_t>(dword_of((sc_col + g) * ESZ)),
             lds_offset(&Ss[g % kStages][wu][0]));
    };
    // the scales this lane folds for group g, read after that group's scale
    // loads are known to have landed
    auto read_scales = [&](int g, float (&sc)[kTN]) {
#pragma unroll
        for (int t = 0; t < kTN; ++t) {
            const uint32_t w = Ss[g % kStages][wid][32 * t + li];
            const int64_t c = static_cast<int64_t>(nval[t] ? ncol[t] : N - 1);
            const int64_t byte = (c * G + g) * ESZ;
            const int shift = static_cast<int>(byte - dword_of(byte)) * 8;
            if constexpr (FMT == kFmtU8)
                sc[t] = static_cast<float>((w >> shift) & 0xFFu);
            else
                sc[t] = bf16_to_f32(static_cast<uint16_t>((w >> shift) & 0xFFFFu));
        }
    };

    // Partials are double-buffered by group parity: group g accumulates into
    // P[g & 1] while the previous group's P[(g & 1) ^ 1] is folded into F one
    // tile at a time, spread over group g's k-steps.  Folding a whole group
    // at its boundary would stall the matrix cores behind a burst of VALU
    // work (both waves of a SIMD reach the boundary together).
    v16i P[2][kTM][kTN];
    float F[kTM][kTN][16];
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int b = 0; b < kTN; ++b) {
            P[0][a][b] = v16i{};
            P[1][a][b] = v16i{};
#pragma unroll
            for (int e = 0; e < 16; ++e) F[a][b][e] = 0.0f;
        }

    // element e of a 32x32 result sits at row 8 (e / 4) + 4 lq + e % 4, column li
    auto write_partials = [&](const v16i &p, int tm, int tn, int g) {
        if (!nval[tn]) return;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = bm + wm * kWTM + tm * 32 + 8 * (e >> 2) + 4 * lq + (e & 3);
            if (m < M) partials[(static_cast<int64_t>(m) * N + ncol[tn]) * G + g] = p[e];
        }
    };
    auto fold = [&](const v16i &p, int tm, int tn, float s) {
#pragma unroll
        for (int e = 0; e < 16; ++e) F[tm][tn][e] += static_cast<float>(p[e]) * s;
    };

    // LDS byte offsets of this lane's fragments at k-step 0 of a stage: rows
    // of the wave's 32 x 32 tiles, chunk 4 lq.  K-step kk reads chunk
    // kk + 4 lq, i.e. the k-step 0 offset XOR 16 kk (the swizzle is an XOR
    // on the chunk index and kk, 4 lq occupy disjoint bits); A and B use the
    // same assignment, so each matrix op sums 32 K positions of its stage.
    // 16 kk is an inline constant, so each read's address is one
    // xor-and-add of the lane offset with the uniform stage base.
    int aoff[kTM], boff[kTN];
#pragma unroll
    for (int t = 0; t < kTM; ++t) aoff[t] = lds_chunk_addr(wm * kWTM + t * 32 + li, 4 * lq);
#pragma unroll
    for (int t = 0; t < kTN; ++t) boff[t] = lds_chunk_addr(wn * kWTN + t * 32 + li, 4 * lq);

    // Issue order (every vector-memory operation of the loop is a direct LDS
    // load issued from asm, so the only waits are the explicit ones below):
    //   one stage per group (head format): group g's scales are issued in
    //     stage g - 1 after that stage's barrier (group 0's between the two
    //     prologue stages);
    //   two stages per group (u8 format): group g's scales are issued in the
    //     group's first stage after its barrier.
    // Either way they are issued before the loads of the stage whose wait
    // precedes their fold, and in-order completion does the rest.
    issue_stage(0);
    if constexpr (SPG == 1) issue_scales(0);
    issue_stage(1);

    constexpr int kSteps = kKC / 32;                   // k-steps per stage
    constexpr int kTiles = kTM * kTN;
    constexpr int kFoldEvery = SPG * kSteps / kTiles;  // k-steps between tile folds
    static_assert(kFoldEvery >= 1 && kFoldEvery * kTiles == SPG * kSteps, "fold schedule");

    // one group; H = g & 1 picks the partial buffer it accumulates into
    auto run_group = [&](int g, auto h_const) {
        constexpr int H = decltype(h_const)::value;
        float scf[kTN] = {};            // previous group's scales (zero before group 0)
#pragma unroll
        for (int st = 0; st < SPG; ++st) {
            const int ks = g * SPG + st;
            // stage ks has landed once no more than the loads issued after
            // it are pending: the next stage's kDmaPerStage, plus one scale
            // load if one was issued between them
            if (SPG == 1 || st == 1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerStage + 1) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerStage) : "memory");
            // all waves' loads of stage ks are in LDS, and all waves are done
            // reading stage ks - 1, whose buffer the next issue overwrites
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if constexpr (SPG == 1) issue_scales(min(g + 1, G - 1));
            else if (st == 0) issue_scales(g);
            if (st == 0 && g > 0) read_scales(g - 1, scf);
            // uniform stage bases, opaque to the compiler so that it keeps
            // them in scalar registers instead of moving constants into the
            // per-lane address arithmetic
            uint32_t sa = lds_offset(&smem[(ks % kStages) * kStageBytes]);
            uint32_t sb = sa + kABytes;
            asm volatile("" : "+s"(sa), "+s"(sb));
            // opaque per stage: keeps the per-k-step XORs below in the loop
            // instead of 16 hoisted, always-live address registers
#pragma unroll
            for (int t = 0; t < kTM; ++t) asm volatile("" : "+v"(aoff[t]));
#pragma unroll
            for (int t = 0; t < kTN; ++t) asm volatile("" : "+v"(boff[t]));
            // fragments double-buffered across k-steps: k-step kk + 1's LDS
            // reads are in flight while k-step kk's matrix ops run
            v4i fa[2][kTM], fb[2][kTN];
            auto read_frags = [&](int kk, v4i(&a)[kTM], v4i(&b)[kTN]) {
#pragma unroll
                for (int t = 0; t < kTM; ++t) a[t] = lds_ld16(sa + (aoff[t] ^ (16 * kk)));
#pragma unroll
                for (int t = 0; t < kTN; ++t) b[t] = lds_ld16(sb + (boff[t] ^ (16 * kk)));
            };
            read_frags(0, fa[0], fb[0]);
#pragma unroll
            for (int kk = 0; kk < kSteps; ++kk) {
                const int pos = st * kSteps + kk;      // k-step within the group
                if (kk + 1 < kSteps) read_frags(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
                // serpentine tile order, (0,0) (0,1) (1,1) (1,0): consecutive
                // matrix ops share one operand, so fewer operand bits toggle;
                // at the power limit the energy per op sets the time
#pragma unroll
                for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
                    for (int tn_ = 0; tn_ < kTN; ++tn_) {
                        const int tn = (tm & 1) ? kTN - 1 - tn_ : tn_;
                        const v4i a = fa[kk & 1][tm], b = fb[kk & 1][tn];
                        P[H][tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            a, b, pos == 0 ? v16i{} : P[H][tm][tn], 0, 0, 0);
                    }
                // fold one tile of the previous group (zeros before group 1)
                if (pos % kFoldEvery == 0) {
                    const int t = pos / kFoldEvery, tm = t / kTN, tn = t % kTN;
                    if constexpr (WRITE_P) {
                        if (g > 0) write_partials(P[H ^ 1][tm][tn], tm, tn, g - 1);
                    }
                    fold(P[H ^ 1][tm][tn], tm, tn, scf[tn]);
                }
                // the next-but-one stage's loads, spread over the k-steps so
                // a full memory queue delays a few matrix ops, not a stage
                if (kk < 3) {
#pragma unroll
                    for (int j = 0; j < kDmaPerStage / 3; ++j) issue_load(ks + 2, (kDmaPerStage / 3) * kk + j);
                }
            }
        }
    };
    for (int g = 0; g < G; g += 2) {
        run_group(g, std::integral_constant<int, 0>{});
        if (g + 1 < G) run_group(g + 1, std::integral_constant<int, 1>{});
    }
    // every load has landed (the re-loads past the end included: nothing may
    // still write this workgroup's LDS once its waves end)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    {
        float scf[kTN];
        read_scales(G - 1, scf);
        auto fold_last = [&](auto h_const) {
            constexpr int H = decltype(h_const)::value;
#pragma unroll
            for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
                for (int tn = 0; tn < kTN; ++tn) {
                    if constexpr (WRITE_P) write_partials(P[H][tm][tn], tm, tn, G - 1);
                    fold(P[H][tm][tn], tm, tn, scf[tn]);
                }
        };
        if ((G - 1) & 1) fold_last(std::integral_constant<int, 1>{});
        else fold_last(std::integral_constant<int, 0>{});
    }

    float rn[kTN];
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
        rn[t] = 0x1p-7f;
        if constexpr (FMT == kFmtU8)
            if (nval[t]) rn[t] = bf16_to_f32(rscale[ncol[t]]) * 0x1p-7f;
    }
#pragma unroll
    for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = bm + wm * kWTM + tm * 32 + 8 * (e >> 2) + 4 * lq + (e & 3);
            if (m >= M) continue;
            const float sm = scale[m];
#pragma unroll
            for (int tn = 0; tn < kTN; ++tn)
                if (nval[tn])     // written once, never re-read here: nontemporal (0.8% faster)
                    __builtin_nontemporal_store(F[tm][tn][e] * (sm * rn[tn]), &y[static_cast<int64_t>(m) * N + ncol[tn]]);
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

bool gemm_grid_fits(int64_t M, int64_t N) {
    return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN) < (int64_t(1) << 31);
}

hipError_t launch_gemm(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st) {
    const int64_t scale_bytes = w.N * (w.K / (w.fmt == kFmtU8 ? 256 : 128)) * (w.fmt == kFmtU8 ? 1 : 2);
    if (scale_bytes < 4 || w.fmt == kFmtTbl4) {
        // too few group scales for the kernel's dword scale loads, or the
        // drafter's 4-bit codebook (expanded in registers by the M <= 128
        // kernels only): run the batch through the M <= 128 path, 128
        // tokens at a time
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
