// skinny_lds.hip -- rotated W8A8 contraction + epilogue with both operands
// staged through LDS (gfx950): 33..64 and 112..128 tokens in the int8
// formats, 9..16 tokens in the drafter's 4-bit codebook format, where the
// workgroups fill their rounds (skinny_lds_supported).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table rows "Weights" and "Activations"): exact int32 partials
// of int8 activation codes times int8 weight codes per K group (256 with a u8
// scale and a bf16 row scale, or 128 with a bf16 scale for the head), folded
// per group into f32, then y = s_m * (r_n) * 2^-7 * sum_g scale[n][g] * P.
// The drafter's format (table row "Speculator") stores 4-bit indices into a
// 16-level integer table with a bf16 scale per 128; they are expanded to the
// table's int8 values in registers and contracted the same way.
//
// A workgroup owns 16 weight rows per wave and all tokens (see SlShape).  K
// is walked in 256-byte stages through an LDS ring filled by direct
// global -> LDS 16-byte loads: one load instruction covers four rows x 256
// contiguous bytes (the weight stream is the cost, and it streams fastest in
// long runs per row), activation rows likewise.  Wave w computes its 16
// weight rows against all (padded) token rows with v_mfma_i32_16x16x64_i8 (A =
// tokens, B = weights; lane j + 16 q holds chunk 4 kk + q of row j for k-step
// kk, on both operands, so each matrix op sums the 64 products of its
// k-step).  Each group's partials are folded into f32 when the group ends.
// Each wave also loads its rows' group-scale dword per stage into LDS with a
// direct load, so the only vector-memory operations of the loop are these
// direct loads and the explicit waits below count them exactly.
//
// LDS: row r of a stage occupies 256 bytes (all 64 banks); its logical
// 16-byte chunk c sits in slot c ^ (r & 15), so the 16 rows x 4 chunks of one
// k-step's operand read spread over all 16 slots, four lanes a slot, the
// fewest passes a 64-lane 16-byte read can take.  (The codebook kernel keeps
// slot c ^ (r & 7).)  With r & 7, half the LDS cycles of these reads were bank
// conflicts (rocprofv3 SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = 0.50 on
// both the 128-token trunk and the 64-token head); r & 15 took the 128-token
// trunk shape from 50.3 to 47.9 us and left the head unchanged.

#include "rad_device.h"
#include "rad_launch.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kSlKC = 256;                         // K bytes per stage

// A workgroup shape: MB blocks of 16 tokens, NW waves of 16 weight rows, NST
// stages in the LDS ring, NT: weight loads nontemporal (each weight byte is
// read once per call), NTY: output stores nontemporal; both measured per
// shape, see the shapes below.  In rings of three or more stages each wave
// issues the same number of 1 KiB direct loads per stage (the explicit waits
// count them): where a stage's blocks do not split evenly over the waves, the
// remainder loads a valid block again into a spare LDS area nobody reads.
// Two-stage rings skip those re-loads (their waits count weight loads only).
template <int MB_, int NW_, int NST_, bool NT_, bool NTY_> struct SlShape {
    static constexpr int MB = MB_, NW = NW_, NST = NST_;
    static constexpr bool NT = NT_;                                // weight loads nontemporal
    static constexpr bool NTY = NTY_;                              // output stores nontemporal
    static constexpr int MP = 16 * MB, BN = 16 * NW;
    static constexpr int A = MP * kSlKC, B = BN * kSlKC;           // bytes per stage
    static constexpr int NA = A / 1024, NB = B / 1024;             // 1 KiB blocks per stage
    static constexpr int DA = (NA + NW - 1) / NW, DB = (NB + NW - 1) / NW;
    static constexpr int SPARE = DA * NW - NA + DB * NW - NB;      // spare blocks
    static constexpr int DMA = DA + DB + 1;                        // + the scale dword load
};

__device__ __forceinline__ int sl_addr(int row, int c) { return 256 * row + 16 * (c ^ (row & 15)); }

// dma16 with the nontemporal cache policy (global_load_lds_dwordx4 ... nt)
__device__ __forceinline__ void dma16nt(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(sbase), "{m0}"(lds)
        : "memory");
}
template <bool NT>
__device__ __forceinline__ void dma16_w(const void *sbase, uint32_t voff, uint32_t lds) {
    if constexpr (NT) dma16nt(sbase, voff, lds);
    else dma16(sbase, voff, lds);
}

template <int FMT, class S, bool WRITE_P>
__global__ __launch_bounds__(64 * S::NW) void skinny_lds_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ scale, const int8_t *__restrict__ codes,
    const void *__restrict__ gscale, const uint16_t *__restrict__ rscale, float *__restrict__ y,
    int32_t *__restrict__ partials, int M, int N, int K) {
    constexpr int MB = S::MB, NST = S::NST, DA = S::DA, DB = S::DB;
    // each wave loads exactly its own 16 weight rows (4 blocks of 4 rows), the
    // rows it alone reads: the schedule below refills them without a barrier
    static_assert(DB == 4 && S::NB == 4 * S::NW, "a wave's weight blocks must be its own rows");
    constexpr int GPS = (FMT == kFmtU8) ? 1 : 2;      // groups per stage
    constexpr int KPG = 4 / GPS;                       // k-steps per group
    constexpr int ESZ = (FMT == kFmtU8) ? 1 : 2;       // bytes per group scale
    __shared__ __attribute__((aligned(1024))) int8_t As[NST][S::A];
    __shared__ __attribute__((aligned(1024))) int8_t Bs[NST][S::B];
    __shared__ __attribute__((aligned(1024))) int8_t Xs[S::SPARE > 0 && NST > 2 ? S::SPARE * 1024 : 16];
    __shared__ __attribute__((aligned(256))) uint32_t Ss[NST][S::NW][64];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wid);
    const int j = lane & 15, qd = lane >> 4;
    const int n0 = static_cast<int>(blockIdx.x) * S::BN;
    const int NS = K / kSlKC;
    const int G = K / (kSlKC / GPS);

    // ---- direct loads of one stage.  Block b of an operand holds its rows
    // 4 b .. 4 b + 3 (lane l: row 4 b + l / 16, slot l % 16, i.e. logical
    // chunk (l % 16) ^ (row & 15)).  Rows past M or N repeat the last row
    // (never stored); block numbers past the operand's re-load block 0.
    const int dr = lane >> 4, dslot = lane & 15;
    uint32_t aoffs[DA], boffs[DB];
#pragma unroll
    for (int i = 0; i < DA; ++i) {
        const int blk = wid * DA + i;
        const int row = blk < S::NA ? 4 * blk + dr : dr;
        aoffs[i] = static_cast<uint32_t>(min(row, M - 1)) * static_cast<uint32_t>(K) +
                   16u * static_cast<uint32_t>(dslot ^ (row & 15));
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) {
        const int blk = wid * DB + i;
        const int row = blk < S::NB ? 4 * blk + dr : dr;
        boffs[i] = static_cast<uint32_t>(min(n0 + row, N - 1) - n0) * static_cast<uint32_t>(K) +
                   16u * static_cast<uint32_t>(dslot ^ (row & 15));
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
    // again, so every wait count below is uniform.  With two stages the wait
    // counts only the weight loads issued after a stage's token blocks, so
    // the spare token re-loads that even out the waves' counts are skipped
    // (1.2% on both the 128-token trunk and the 64-token head shapes once the
    // LDS reads were conflict-free).
    // block numbers are wave-major, so the padding blocks of each operand
    // form one range: A's first, then B's, in the spare area
    auto issue_a = [&](int s) {
        const int sc = min(s, NS - 1);
        const int buf = s % NST;
#pragma unroll
        for (int i = 0; i < DA; ++i) {
            const int blk = wu * DA + i;
            if (NST == 2 && blk >= S::NA) continue;
            const uint32_t dst = blk < S::NA ? lds_offset(&As[buf][0]) + 1024u * blk
                                             : lds_offset(&Xs[0]) + 1024u * (blk - S::NA);
            dma16(q + static_cast<int64_t>(sc) * kSlKC, aoffs[i], dst);
        }
    };
    // a wave's weight blocks are its own 16 rows, and its scale dword theirs
    auto issue_b = [&](int s) {
        const int sc = min(s, NS - 1);
        const int buf = s % NST;
#pragma unroll
        for (int i = 0; i < DB; ++i) {
            const int blk = wu * DB + i;
            if (NST == 2 && blk >= S::NB) continue;
            const uint32_t dst = blk < S::NB ? lds_offset(&Bs[buf][0]) + 1024u * blk
                                             : lds_offset(&Xs[0]) + 1024u * (DA * S::NW - S::NA + blk - S::NB);
            dma16_w<S::NT>(bbase + static_cast<int64_t>(sc) * kSlKC, boffs[i], dst);
        }
        dma4(gscale, static_cast<uint32_t>(sc_dword(sc)), lds_offset(&Ss[buf][wu][0]));
    };

    v4i P[MB];
    float F[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        P[mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) F[mb][e] = 0.0f;
    }

    // LDS offsets of this lane's fragments at k-step 0 (row j of each 16-row
    // block, chunk qd); k-step kk reads chunk 4 kk + qd, i.e. offset XOR 64 kk
    int aoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) aoff[mb] = sl_addr(16 * mb + j, qd);
    const int boff = sl_addr(16 * wid + j, qd);

#pragma unroll
    for (int p = 0; p < NST - 1; ++p) {
        issue_b(p);
        issue_a(p);
    }
    for (int s = 0; s < NS; ++s) {
        // this wave is done with its weight rows of stage s - 1 (no other
        // wave reads them), so their buffer takes stage s + NST - 1 at once,
        // ahead of the wait and the barrier.  Stage s has landed once at most
        // the loads issued after its token blocks remain: NST - 2 whole stages
        // and these weight rows.  The barrier publishes every wave's token
        // blocks of stage s and retires stage s - 1's, whose buffer the token
        // blocks of stage s + NST - 1 then take.
        issue_b(s + NST - 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * S::DMA + DB + 1) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_a(s + NST - 1);
        const int buf = s % NST;
        const int8_t *Ab = As[buf];
        const int8_t *Bb = Bs[buf];
        const uint32_t sw = Ss[buf][wid][j];
        const int shift = static_cast<int>(sc_byte(s) - sc_dword(s)) * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const v4i b = *reinterpret_cast<const v4i *>(Bb + (boff ^ (64 * kk)));
            v4i a[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const v4i *>(Ab + (aoff[mb] ^ (64 * kk)));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
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
                for (int mb = 0; mb < MB; ++mb) {
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
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mb + 4 * qd + e;
            if (m < M) {
                const float v = F[mb][e] * (scale[m] * rn);
                if constexpr (S::NTY) __builtin_nontemporal_store(v, &y[static_cast<int64_t>(m) * N + nrow]);
                else y[static_cast<int64_t>(m) * N + nrow] = v;
            }
        }
}

// 4-bit codebook format: a stage is 256 bytes of each weight row's packed
// indices (512 elements, four 128-element groups with a bf16 scale each) and
// 512 bytes of each token row.  Weight blocks are four rows x 256 bytes as
// above; token blocks are two rows x 512 bytes (lane l: row 2 b + l / 32,
// slot l % 32).  Lane j + 16 q expands run 4 p + q of its weight row (32
// elements: low nibbles 0..15, high nibbles 16..31) for k-steps 2 p and
// 2 p + 1, and reads the matching token chunks 8 p + 2 q and 8 p + 2 q + 1, so
// k-steps 2 p, 2 p + 1 cover exactly group p of the stage.  Each wave fetches
// its rows' two scale dwords per stage (groups 4 s .. 4 s + 3).
template <class S, bool WRITE_P>
__global__ __launch_bounds__(64 * S::NW) void skinny_lds_tbl4_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ scale, const int8_t *__restrict__ codes,
    const void *__restrict__ gscale, float *__restrict__ y, int32_t *__restrict__ partials, int M, int N,
    int K) {
    constexpr int MB = S::MB, NST = S::NST, NW = S::NW;
    constexpr int RA = 2 * kSlKC;                      // token-row bytes per stage
    constexpr int ABYTES = S::MP * RA, BBYTES = S::BN * kSlKC;
    constexpr int NA = ABYTES / 1024, NB = BBYTES / 1024;
    constexpr int DA = (NA + NW - 1) / NW, DB = (NB + NW - 1) / NW;
    constexpr int SPARE = DA * NW - NA + DB * NW - NB;
    constexpr int DMA = DA + DB + 2;                   // + two scale dwords
    static_assert(DB == 4 && NB == 4 * NW, "a wave's weight blocks must be its own rows");
    __shared__ __attribute__((aligned(1024))) int8_t As[NST][ABYTES];
    __shared__ __attribute__((aligned(1024))) int8_t Bs[NST][BBYTES];
    __shared__ __attribute__((aligned(1024))) int8_t Xs[SPARE > 0 ? SPARE * 1024 : 16];
    __shared__ __attribute__((aligned(256))) uint32_t Ss[NST][NW][2][64];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wid);
    const int j = lane & 15, qd = lane >> 4;
    const int n0 = static_cast<int>(blockIdx.x) * S::BN;
    const int NS = K / RA;
    const int G = K / 128;
    const int RB = K / 2;                              // packed bytes of a weight row

    uint32_t aoffs[DA], boffs[DB];
#pragma unroll
    for (int i = 0; i < DA; ++i) {
        const int blk = wid * DA + i;
        const int row = blk < NA ? 2 * blk + (lane >> 5) : (lane >> 5);
        aoffs[i] = static_cast<uint32_t>(min(row, M - 1)) * static_cast<uint32_t>(K) +
                   16u * static_cast<uint32_t>((lane & 31) ^ (row & 7));
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) {
        const int blk = wid * DB + i;
        const int row = blk < NB ? 4 * blk + (lane >> 4) : (lane >> 4);
        boffs[i] = static_cast<uint32_t>(min(n0 + row, N - 1) - n0) * static_cast<uint32_t>(RB) +
                   16u * static_cast<uint32_t>((lane & 15) ^ (row & 7));
    }
    const int8_t *bbase = codes + static_cast<int64_t>(n0) * RB;
    const int nrow = n0 + 16 * wid + j;
    const bool nvalid = nrow < N;
    // bytes of groups 4 s .. 4 s + 3 of this lane's row: two aligned dwords
    // (a row's scales are 2 G bytes, G a multiple of 4)
    const uint32_t sc_row = static_cast<uint32_t>(min(nrow, N - 1)) * static_cast<uint32_t>(2 * G);

    auto issue_a = [&](int s) {
        const int sc = min(s, NS - 1);
        const int buf = s % NST;
#pragma unroll
        for (int i = 0; i < DA; ++i) {
            const int blk = wu * DA + i;
            const uint32_t dst = blk < NA ? lds_offset(&As[buf][0]) + 1024u * blk
                                          : lds_offset(&Xs[0]) + 1024u * (blk - NA);
            dma16(q + static_cast<int64_t>(sc) * RA, aoffs[i], dst);
        }
    };
    // a wave's weight blocks are its own 16 rows, and its scale dwords theirs
    auto issue_b = [&](int s) {
        const int sc = min(s, NS - 1);
        const int buf = s % NST;
#pragma unroll
        for (int i = 0; i < DB; ++i) {
            const int blk = wu * DB + i;
            const uint32_t dst = blk < NB ? lds_offset(&Bs[buf][0]) + 1024u * blk
                                          : lds_offset(&Xs[0]) + 1024u * (DA * NW - NA + blk - NB);
            dma16_w<S::NT>(bbase + static_cast<int64_t>(sc) * kSlKC, boffs[i], dst);
        }
        dma4(gscale, sc_row + 8u * sc, lds_offset(&Ss[buf][wu][0][0]));
        dma4(gscale, sc_row + 8u * sc + 4u, lds_offset(&Ss[buf][wu][1][0]));
    };

    v4i P[MB];
    float F[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        P[mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) F[mb][e] = 0.0f;
    }
    // token chunk 8 p + 2 q + h of row r sits at 512 r + 128 p + 16 ((2 q + h) ^ (r & 7))
    int aoff[2][MB];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) aoff[h][mb] = RA * (16 * mb + j) + 16 * ((2 * qd + h) ^ (j & 7));
    // weight run 4 p + q of row r sits at (256 r + 16 (q ^ (r & 7))) ^ 64 p
    const int boff = kSlKC * (16 * wid + j) + 16 * (qd ^ (j & 7));

    const Tbl4Masks tk = tbl4_masks();
#pragma unroll
    for (int p = 0; p < NST - 1; ++p) {
        issue_b(p);
        issue_a(p);
    }
    for (int s = 0; s < NS; ++s) {
        // as in the kernel above: this wave's own weight rows first, then the
        // wait, the barrier and the token blocks
        issue_b(s + NST - 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * DMA + DB + 2) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_a(s + NST - 1);
        const int buf = s % NST;
        const int8_t *Ab = As[buf];
        const int8_t *Bb = Bs[buf];
        const uint32_t sw0 = Ss[buf][wid][0][j], sw1 = Ss[buf][wid][1][j];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v4i lo, hi;
            tbl4_decode16(*reinterpret_cast<const v4i *>(Bb + (boff ^ (64 * p))), lo, hi, tk);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v4i a[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const v4i *>(Ab + aoff[h][mb] + 128 * p);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    P[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb], h ? hi : lo, h ? P[mb] : v4i{0, 0, 0, 0},
                                                                   0, 0, 0);
            }
            const uint32_t sw = (p < 2) ? sw0 : sw1;
            const float sc = bf16_to_f32(static_cast<uint16_t>((sw >> (16 * (p & 1))) & 0xFFFFu));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) F[mb][e] += static_cast<float>(P[mb][e]) * sc;
                if constexpr (WRITE_P) {
                    const int g = 4 * s + p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = 16 * mb + 4 * qd + e;
                        if (m < M && nvalid) partials[(static_cast<int64_t>(m) * N + nrow) * G + g] = P[mb][e];
                    }
                }
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!nvalid) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mb + 4 * qd + e;
            if (m < M) y[static_cast<int64_t>(m) * N + nrow] = F[mb][e] * (scale[m] * 0x1p-7f);
        }
}

// Nontemporal weight loads: 128 tokens 53.6 -> 49.4 us (34816 rows), codebook
// 16 tokens 26.8 -> 25.0 us; 64 tokens on the 152064-row head with the 128-row
// shape 188.9 -> 190.3 us, so that shape keeps plain loads.  Nontemporal output
// stores: the head at 64 tokens 189.0 -> 170.7 us (its 39 MB of outputs no
// longer displace the token rows every workgroup re-reads); 128 tokens 49.5 ->
// 50.0 us, codebook 16 tokens unchanged, so those keep plain stores.  The head
// format at 33..64 tokens takes 208-row workgroups: 731 on the 152064-row head,
// 2.86 rounds, against 1188 (4.64 rounds) of 128 rows, whose last round leaves
// a third of the CUs idle; 169.9 -> 165.8 us with plain loads, 159.5 us with
// nontemporal ones (160-row workgroups 175.8 us, 112-row 183.1 us).
using Shape64 = SlShape<4, 8, 3, false, true>;    // trunk format, 33..64 tokens: 128 rows, 3 stages of 48 KiB
using Shape128 = SlShape<8, 9, 2, true, false>;   // 112..128 tokens: 144 rows, 2 stages of 68 KiB
using ShapeH64 = SlShape<4, 13, 2, true, true>;   // head format, 33..64 tokens: 208 rows, 2 stages of 68 KiB
using ShapeT16 = SlShape<1, 9, 3, true, false>;   // codebook format, 9..16 tokens: 144 rows, 3 stages of 44 KiB

template <class S>
hipError_t launch_tbl4_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                         int32_t *P, hipStream_t st) {
    const int64_t grid = (w.N + S::BN - 1) / S::BN;
    auto kern = P ? skinny_lds_tbl4_kernel<S, true> : skinny_lds_tbl4_kernel<S, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(64 * S::NW), 0, st, q, s, w.codes,
                       w.gscale, y, P, static_cast<int>(M), static_cast<int>(w.N), static_cast<int>(w.K));
    return hipGetLastError();
}

template <int FMT, class S>
hipError_t launch_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                    int32_t *P, hipStream_t st) {
    const int64_t grid = (w.N + S::BN - 1) / S::BN;
    auto kern = P ? skinny_lds_kernel<FMT, S, true> : skinny_lds_kernel<FMT, S, false>;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(64 * S::NW), 0, st, q, s, w.codes,
                       w.gscale, w.rscale, y, P, static_cast<int>(M), static_cast<int>(w.N),
                       static_cast<int>(w.K));
    return hipGetLastError();
}

}  // namespace

// A CU holds one of these workgroups at a time (LDS), so the kernel takes
// whole rounds of workgroups; it is used only where its workgroups fill at
// least 85% of their rounds.  Measured on MI355X (256 CUs, K = 5120): the
// 152064-row head at 64 tokens (128-row workgroups: 1188, 93%) 189 us against
// 208 us for the register-streaming kernel; the 34816-row trunk at 33..64 tokens
// (272 workgroups, 53%) 55-59 us against 40-43 us, so that shape keeps the
// other kernel; at 112..128 tokens the 144-row workgroups (242, one round)
// beat it by 1-4%, at 65..96 tokens (padded to 128) they lose.  Codebook
// format, 16 tokens on the 34816-row drafter linear (242 workgroups): 26.7 us
// against 31.1 us.
bool skinny_lds_supported(const WeightArgs &w, int64_t M) {
    if (w.fmt == 2) {
        if (M < 9 || M > 16 || w.K % (2 * kSlKC) != 0) return false;
        const int cus = cu_count();
        if (cus <= 0) return false;
        const int64_t wgs = (w.N + ShapeT16::BN - 1) / ShapeT16::BN;
        const int64_t rounds = (wgs + cus - 1) / cus;
        return wgs * 100 >= 85 * rounds * cus;
    }
    if (w.K % kSlKC != 0) return false;
    if (w.fmt == kFmtU8) {
        if (w.N * (w.K / 256) < 4) return false;
    } else if (w.fmt != 1 || (w.K / 128) % 2 != 0) {   // head: the stage's two scales share a dword
        return false;
    }
    int64_t bn;
    if (M >= 33 && M <= 64) bn = w.fmt == kFmtU8 ? Shape64::BN : ShapeH64::BN;
    else if (M >= 112 && M <= 128) bn = Shape128::BN;
    else return false;
    const int cus = cu_count();
    if (cus <= 0) return false;
    const int64_t wgs = (w.N + bn - 1) / bn;
    const int64_t rounds = (wgs + cus - 1) / cus;
    return wgs * 100 >= 85 * rounds * cus;
}

hipError_t launch_skinny_lds(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                             int32_t *partials, hipStream_t st) {
    if (w.fmt == 2) return launch_tbl4_t<ShapeT16>(q, s, w, y, M, partials, st);
    if (M <= 64)
        return w.fmt == kFmtU8 ? launch_t<0, Shape64>(q, s, w, y, M, partials, st)
                               : launch_t<1, ShapeH64>(q, s, w, y, M, partials, st);
    return w.fmt == kFmtU8 ? launch_t<0, Shape128>(q, s, w, y, M, partials, st)
                           : launch_t<1, Shape128>(q, s, w, y, M, partials, st);
}

}  // namespace rad
