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
//   decode_kernel    M == 1.  Waves stream weight rows four at a time with
//                    coalesced 16-byte loads and v_dot4 against activation
//                    codes held in registers; optionally fused with the
//                    rotation and quantisation of the token.  For the u8 format
//                    the epilogue is exact integer arithmetic up to one f64
//                    product, rounded once.
//   skinny_kernel    2 <= M <= 128.  Each compute wave owns 16 weight rows and
//                    streams them straight from HBM into the B operand of
//                    v_mfma_i32_16x16x64_i8 with several stages in flight; a
//                    producer wave stages the activation codes of all M
//                    tokens in LDS for the workgroup.
#include <algorithm>
#include <atomic>

#include "rad_device.h"
#include "rad_launch.h"
#include "rotate_quant.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kFmtHead = 1;
constexpr int kFmtTbl4 = 2;    // 4-bit codebook indices, packed two per byte

// K elements held by one byte of a weight row
template <int FMT> constexpr int kElemsPerByte = (FMT == kFmtTbl4) ? 2 : 1;

// ------------------------------------------------------------- M == 1 ----
// Layout: a wave streams 4 weight rows at a time (a "quad"), one 16-lane DPP
// row per weight row.  In step t, lane l16 of a DPP row reads the 16 bytes
// c = l16 + 16 t of its weight row, so one load instruction of the wave reads
// 4 x 256 contiguous bytes and, for the u8 format, step t is exactly group t.
// A quad's cross-lane reduction is 4 DPP butterflies inside each 16-lane row,
// shared by the 4 rows.  Quads are dealt to waves round-robin (wave w takes
// quads w, w + W, ...), so at any moment the whole GPU streams one contiguous
// window of the weight matrix.  A ring of D 16-byte loads per lane is kept in
// flight across quad boundaries; the quad's steps are padded to SP, a multiple
// of D, with empty steps.  The wave's group and row scales are staged in LDS
// once, so no scale load sits in the in-order vector-memory queue.
//
// u8 format: every partial and every u8-scaled sum is exact integer
// arithmetic; S = sum_g u8[n][g] P[n][g] is formed exactly and
// y = s * r * 2^-7 * S is evaluated in f64 in that order and rounded once, so
// this path reproduces the oracle's output bit for bit.
//
// FUSED: the workgroup first rotates and quantises the f32 token itself (the
// same device code and bits as rad_quant_act_i8) while its first weight loads
// are in flight; block 0 also writes the codes and the scale out.
//
// Codebook format: a row is K / 2 bytes of packed indices, so a 16-byte load
// holds 32 elements (a "run": low nibbles elements 0..15, high nibbles 16..31)
// and step t covers 512 elements of the row; each lane expands its run to
// int8 table values in registers (v_perm lookups) and dots them with 32
// activation codes.  Four lanes make one 128-element group.
constexpr int kScBytes = 2048;   // per-wave LDS staging of group scales
constexpr int kRsBytes = 128;    // per-wave LDS staging of row scales (16 quads)
constexpr int kM1MaxK = 20480;   // K handled by the one-token path

template <int FMT, int STEPS, int D, bool WRITE_P, bool FUSED>
__global__ __launch_bounds__(256) void decode_kernel(const float *__restrict__ x,
                                                     int8_t *__restrict__ qio,
                                                     float *__restrict__ sio,
                                                     const int8_t *__restrict__ codes,
                                                     const void *__restrict__ gscale,
                                                     const uint16_t *__restrict__ rscale,
                                                     float *__restrict__ y,
                                                     int32_t *__restrict__ partials, int N, int K) {
    constexpr int EPB = kElemsPerByte<FMT>;
    constexpr int GW16 = (FMT == kFmtU8) ? 16 : (FMT == kFmtHead ? 8 : 4);   // 16-byte chunks per group
    constexpr int ESZ = (FMT == kFmtU8) ? 1 : 2;      // bytes per group scale
    constexpr int SP = ((STEPS + D - 1) / D) * D;     // steps per quad incl. padding
    constexpr int KSTEP = 256 * EPB;                  // K elements per step
    constexpr int NQ = (STEPS * KSTEP / 128 + 15) / 16;   // 16-block rotation steps
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[4][kScBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rs_lds[4][kRsBytes];
    __shared__ __attribute__((aligned(16))) int8_t q_lds[STEPS * KSTEP];
    __shared__ float red[4];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wid);  // the same, known uniform
    const int l16 = lane & 15;
    const int r4 = lane >> 4;                          // weight row inside the quad
    const int wave = blockIdx.x * 4 + wid;
    const int W = gridDim.x * 4;
    const int nq = (N + 3) >> 2;
    const int cnt = wave < nq ? (nq - wave + W - 1) / W : 0;   // quads of this wave
    const int RB = K / EPB;                            // bytes of a weight row
    const int nchunk = RB >> 4;
    const int G = nchunk / GW16;
    const int qsb = 4 * G * ESZ;                       // scale bytes of one quad (multiple of 4)
    const int64_t allsb = static_cast<int64_t>(N) * G * ESZ;

    // 1. this wave's group and row scales, straight into LDS, dword by dword.
    //    A dword that would run past the end of an array is loaded bytewise.
    //    The direct loads are issued from asm (dma4): the compiler's wait
    //    counting does not see them, so it does not drain them (nor the weight
    //    loads behind them) before the rotation; they are older than every
    //    load the compiler waits for, and the explicit full wait before the
    //    weight stream covers them.
    {
        const uint8_t *gs = static_cast<const uint8_t *>(gscale);
        const int nd = cnt * qsb / 4;
        for (int j0 = 0; j0 < nd; j0 += 64) {
            const int j = j0 + lane;
            const int qi = (4 * j) / qsb;
            const int64_t src = static_cast<int64_t>(4 * (wave + qi * W)) * G * ESZ + (4 * j - qi * qsb);
            const bool ok = j < nd;
            if (ok && src + 4 <= allsb) {
                dma4(gs, static_cast<uint32_t>(src), lds_offset(&sc_lds[wu][4 * j0]));
            } else if (ok && src < allsb) {
                for (int b = 0; b < 4 && src + b < allsb; ++b) sc_lds[wid][4 * j + b] = gs[src + b];
            }
        }
        if constexpr (FMT == kFmtU8) {
            const uint8_t *rs = reinterpret_cast<const uint8_t *>(rscale);
            const int j = lane;                        // 2 dwords per quad, <= 16 quads
            const int qi = j >> 1;
            const int64_t src = static_cast<int64_t>(8) * (wave + qi * W) + 4 * (j & 1);
            const bool ok = j < 2 * cnt;
            if (ok && src + 4 <= 2 * static_cast<int64_t>(N)) {
                dma4(rs, static_cast<uint32_t>(src), lds_offset(&rs_lds[wu][0]));
            } else if (ok && src < 2 * static_cast<int64_t>(N)) {
                for (int b = 0; b < 4 && src + b < 2 * static_cast<int64_t>(N); ++b) rs_lds[wid][4 * j + b] = rs[src + b];
            }
        }
    }

    // 2. the token: f32 into registers (fused) or its codes straight into LDS.
    //    The fused loads are branch-free (blocks past the row re-read the last
    //    block and are zeroed after the load): with no branch around them the
    //    compiler's wait before the rotation counts only the weight loads
    //    issued after them, so the rotation runs while those are in flight.
    Blk8 xv[FUSED ? NQ : 1];
    float s = 0.0f;
    const int nblk = K >> 7;
    if constexpr (FUSED) {
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int blk = (it * 4 + wid) * 4 + r4;
            const float *p = x + min(blk, nblk - 1) * 128 + 4 * l16;
            xv[it].lo = *reinterpret_cast<const float4 *>(p);
            xv[it].hi = *reinterpret_cast<const float4 *>(p + 64);
        }
    } else {
        for (int d0 = wid * 64; d0 < K / 4; d0 += 256) {
            if (d0 + lane < K / 4)
                g2lds_dword(qio + 4 * (d0 + lane), &q_lds[4 * d0]);
        }
        s = sio[0];
    }

    // 3. the first D weight loads of the ring.  Loads are branch-free: a quad
    //    past the wave's last one, or a row past N, is clamped to an in-bounds
    //    row (a re-read of cached data) whose result is never stored; STEPS is
    //    exactly ceil(K / 256), so only the last step can hold lanes past the
    //    end of a row (head format), and those are clamped and not accumulated.
    auto row_ptr = [&](int i) -> const int8_t * {
        const int ii = max(min(i, cnt - 1), 0);
        const int row = min(4 * (wave + ii * W) + r4, N - 1);
        return codes + static_cast<int64_t>(row) * RB + 16 * l16;
    };
    auto wload = [&](const int8_t *rp, int t) -> v4i {
        if (t >= STEPS) return v4i{0, 0, 0, 0};       // padding step: no load
        if (t == STEPS - 1) {
            const int c = min(l16 + 16 * t, nchunk - 1);
            return ld16(rp - 16 * l16 + 16 * c);
        }
        return ld16(rp + 256 * t);
    };
    // (a wave without quads loads a clamped row, never used).  The
    // scheduling fences keep all D loads after the token's and ahead of the
    // rotation, which then waits for the token only.
    v4i ring[D];
    const int8_t *rp_next = row_ptr(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < D; ++t) ring[t] = wload(rp_next, t);
    __builtin_amdgcn_sched_barrier(0);

    // 4. fused: rotate and quantise the token into LDS (and, block 0, to q / s)
    if constexpr (FUSED) {
        float amax = 0.0f;
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            if ((it * 4 + wid) * 4 + r4 >= nblk) {
                xv[it].lo = make_float4(0.f, 0.f, 0.f, 0.f);
                xv[it].hi = xv[it].lo;
            }
            fwht128_regs_signed(xv[it], l16);   // values times the lane sign c
            amax = fmaxf(amax, fmaxf(amax4(xv[it].lo), amax4(xv[it].hi)));
        }
        amax = wave_max_f32(amax);
        if (lane == 0) red[wid] = amax;
        __syncthreads();
        s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / 127.0f;
        // codes through the reciprocal where that provably rounds like the
        // division (the same scheme and bits as rad_quant_act_i8), else
        // through the division
        const bool fast = s >= 0x1p-120f;
        const float c = fwht_lane_sign(l16);
        const float rs_c = c * (1.0f / s);
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int blk = (it * 4 + wid) * 4 + r4;
            if (blk < nblk) {
                uint32_t lo = 0, hi = 0;
                if (fast) {
                    lo = pack4_rcp_signed(xv[it].lo, s, rs_c, c);
                    hi = pack4_rcp_signed(xv[it].hi, s, rs_c, c);
                } else if (s != 0.0f) {
                    lo = pack4_signed(xv[it].lo, s, c);
                    hi = pack4_signed(xv[it].hi, s, c);
                }
                const int off = blk * 128 + 4 * l16;
                *reinterpret_cast<uint32_t *>(&q_lds[off]) = lo;
                *reinterpret_cast<uint32_t *>(&q_lds[off + 64]) = hi;
                if (blockIdx.x == 0) {
                    *reinterpret_cast<uint32_t *>(qio + off) = lo;
                    *reinterpret_cast<uint32_t *>(qio + off + 64) = hi;
                }
            }
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) sio[0] = s;
    }
    // every LDS transfer above has landed (this also waits for the ring,
    // whose first entry the loop needs at once), then make it workgroup-visible
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // 5. the weight stream
    [[maybe_unused]] const Tbl4Masks tk = tbl4_masks();
    for (int i = 0; i < cnt; ++i) {
        const int row = 4 * (wave + i * W) + r4;
        const int8_t *rp_cur = rp_next;
        rp_next = row_ptr(i + 1);
        const uint8_t *scq = &sc_lds[wid][i * qsb + r4 * G * ESZ];
        // an offset the compiler cannot see through keeps the activation reads
        // inside the loop (re-read from LDS each quad) instead of holding all
        // STEPS chunks in registers
        int qoff = 0;
        asm volatile("" : "+v"(qoff));
        int acc = 0, acc_hi = 0;                       // u8: exact integer sums
        float accf = 0.0f;                             // head: f32
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            if (t < STEPS) {
                const int c = l16 + 16 * t;
                int p;
                if constexpr (FMT == kFmtTbl4) {
                    v4i lo, hi;
                    tbl4_decode16(ring[t % D], lo, hi, tk);
                    const v4i a0 = *reinterpret_cast<const v4i *>(&q_lds[32 * c + qoff]);
                    const v4i a1 = *reinterpret_cast<const v4i *>(&q_lds[32 * c + 16 + qoff]);
                    p = dot16_i8(hi, a1, dot16_i8(lo, a0, 0));
                } else {
                    const v4i av = *reinterpret_cast<const v4i *>(&q_lds[16 * c + qoff]);
                    p = dot16_i8(ring[t % D], av, 0);
                }
                if constexpr (FMT == kFmtU8) {
                    // |p| <= 16 * 127^2 < 2^23: a full-rate 24-bit multiply
                    const int prod = __mul24(p, static_cast<int>(scq[t]));     // |prod| < 2^26
                    if constexpr (STEPS <= 32) {
                        acc += prod;                                   // < 32 * 2^26
                    } else {
                        acc += prod & 0xFFFF;
                        acc_hi += prod >> 16;
                    }
                    if constexpr (WRITE_P) {
                        const int pg = row16_sum(p);
                        if (l16 == 0 && row < N) partials[static_cast<int64_t>(row) * G + t] = pg;
                    }
                } else if (c < nchunk) {
                    const int g = c / GW16;                    // GW16 lanes make a group
                    const uint16_t b = *reinterpret_cast<const uint16_t *>(&scq[2 * g]);
                    accf += static_cast<float>(p) * bf16_to_f32(b);
                    if constexpr (WRITE_P) {
                        const int pg = (GW16 == 8) ? row8_sum(p) : row4_sum(p);
                        if ((l16 % GW16) == 0 && row < N) partials[static_cast<int64_t>(row) * G + g] = pg;
                    }
                }
            }
            ring[t % D] = (t + D < SP) ? wload(rp_cur, t + D) : wload(rp_next, t + D - SP);
            // keep the steps in order: without this the scheduler hoists every
            // step's LDS read to the top of the quad and holds them all
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FMT == kFmtU8) {
            // exact 16-lane sums of the 16-bit halves; S = hi * 2^16 + lo
            int hi, lo;
            if constexpr (STEPS <= 32) {
                hi = row16_sum(acc >> 16);
                lo = row16_sum(acc & 0xFFFF);
            } else {
                hi = row16_sum(acc_hi + (acc >> 16));
                lo = row16_sum(acc & 0xFFFF);
            }
            if (l16 == 0 && row < N) {
                const int64_t S = static_cast<int64_t>(hi) * 65536 + lo;
                const uint16_t rb = *reinterpret_cast<const uint16_t *>(&rs_lds[wid][8 * i + 2 * r4]);
                const double rn = static_cast<double>(bf16_to_f32(rb));
                y[row] = static_cast<float>(static_cast<double>(s) * rn * 0x1p-7 * static_cast<double>(S));
            }
        } else {
            accf += lane_xor<1>(accf);
            accf += lane_xor<2>(accf);
            accf += lane_xor<4>(accf);
            accf += lane_xor<8>(accf);
            if (l16 == 0 && row < N) y[row] = (s * 0x1p-7f) * accf;
        }
    }
}

// Quads per wave: about TARGET waves in all, bounded by the LDS staging.
inline int decode_quads_per_wave(int64_t N, int64_t K, int fmt, int target_waves) {
    const int G = static_cast<int>(K / (fmt == kFmtU8 ? 256 : 128));   // head and codebook: 128
    const int esz = fmt == kFmtU8 ? 1 : 2;
    const int nq = static_cast<int>((N + 3) / 4);
    int qpw = (nq + target_waves - 1) / target_waves;
    qpw = std::min(qpw, kScBytes / (4 * G * esz));
    qpw = std::min(qpw, kRsBytes / 8);
    return std::max(qpw, 1);
}


template <int FMT, int STEPS, bool FUSED>
hipError_t launch_m1_t(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y,
                       int32_t *P, hipStream_t st) {
    // ring depth: a divisor of STEPS near 10 when there is one, else pad to 8s
    constexpr int D = (STEPS <= 12) ? STEPS
                    : (STEPS % 10 == 0) ? 10 : (STEPS % 12 == 0) ? 12 : (STEPS % 9 == 0) ? 9
                    : (STEPS % 11 == 0) ? 11 : (STEPS % 8 == 0) ? 8 : 8;
    const int N = static_cast<int>(w.N);
    const int nq = (N + 3) / 4;
    const int qpw = decode_quads_per_wave(w.N, w.K, FMT, 3072);   // ~12 waves per CU
    const int waves = (nq + qpw - 1) / qpw;
    const int grid = (waves + 3) / 4;
    auto kern = P ? decode_kernel<FMT, STEPS, D, true, FUSED> : decode_kernel<FMT, STEPS, D, false, FUSED>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, x, q, s, w.codes, w.gscale, w.rscale, y, P,
                       N, static_cast<int>(w.K));
    return hipGetLastError();
}

// Step counts (ceil(K / 256)) with a one-token kernel; other K use the MFMA path.
#define RAD_M1_STEPS(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(14) \
    X(16) X(20) X(24) X(28) X(32) X(40) X(48) X(56) X(64) X(68) X(72) X(80)

// steps of the one-token kernel: 256 bytes of a weight row each
inline int m1_steps(int64_t K, int fmt) {
    return static_cast<int>((K + 256 * (fmt == kFmtTbl4 ? 2 : 1) - 1) / (256 * (fmt == kFmtTbl4 ? 2 : 1)));
}

inline bool m1_steps_supported(int steps) {
    switch (steps) {
#define RAD_M1_YES(S) case S: return true;
        RAD_M1_STEPS(RAD_M1_YES)
#undef RAD_M1_YES
        default: return false;
    }
}

template <int FMT, bool FUSED>
hipError_t launch_m1(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y, int32_t *P,
                     hipStream_t st) {
    switch (m1_steps(w.K, FMT)) {
#define RAD_M1_CASE(S) case S: return launch_m1_t<FMT, S, FUSED>(x, q, s, w, y, P, st);
        RAD_M1_STEPS(RAD_M1_CASE)
#undef RAD_M1_CASE
        default: return hipErrorInvalidValue;           // excluded by m1_supported
    }
}

// ------------------------------------------------------- 2 <= M <= 128 ----
// The weight stream is the cost (M <= 128 int8 MACs per weight byte is far
// below the matrix units' ridge), so the kernel is built to keep HBM busy:
//
//   * A workgroup is nw compute waves plus one producer wave (nw chosen at
//     launch, see sk_compute_waves).  Compute wave w owns 16 weight rows and
//     streams them from HBM straight into the B operand of
//     v_mfma_i32_16x16x64_i8, keeping SkShape::D stages (128 bytes of K each)
//     of its rows in flight in registers.
//   * The producer wave copies the activation codes of all M tokens, one
//     128-byte stage of K at a time, into a 3-deep LDS ring with direct
//     global -> LDS loads, and the compute waves read their A operands from
//     there.  A separate wave keeps these short, L2-resident loads out of the
//     compute waves' in-order memory queue, where they would wait behind
//     weight loads issued stages ahead.
//   * One s_barrier per stage: the producer arrives once stage s has landed,
//     the compute waves once they are done with stage s - 1, whose buffer the
//     producer refills next.
//
// Lane L = j + 16 q of a compute wave holds, for k-step kk (64 bytes) of a
// stage, bytes [64 kk + 16 q, +16) of weight row n0 + j (B) and of token
// 16 mb + j (A).  Both operands use the same byte-to-k assignment, so each
// MFMA sums exactly the 64 products of its k-step; P[mb] element e is token
// 16 mb + 4 q + e, row n0 + j.  Each K group's partials are folded into f32
// with the group scale once the group's stages are done.
//
// Codebook format: a stage of a weight row is 64 bytes of packed indices;
// lane j + 16 q loads the 16-byte run q (elements 32 q .. 32 q + 31 of the
// stage), expands it in registers, and uses its first 16 values in k-step 0
// and the other 16 in k-step 1.  The A operand follows the same assignment
// (token bytes 32 q + 16 kk of the stage), which keeps every product inside
// the stage, i.e. inside its 128-element group.
//
// LDS: token row m of a stage occupies 128 bytes, its 16-byte chunk c stored
// in slot c ^ (m mod 8).  With the 16x16x64 operand layout (lane j + 16 q
// reads token j, chunk q of the k-step) this measures free of bank conflicts
// (SQ_LDS_BANK_CONFLICT = 0); the variant that also flips by (m / 8) mod 2
// measured 2-way conflicts.  Each producer load still reads whole 128-byte
// segments.
constexpr int kSkStageK = 128;                  // K bytes per stage
constexpr int kSkRing = 3;                      // activation stages in LDS

__device__ __forceinline__ int sk_swz(int row) { return row & 7; }

// Weight stages in flight per compute wave, per token-block count (measured
// on MI355X, random int8 weights, the 34816 x 5120 trunk and the 152064 x 5120
// head): deep for up to 64 tokens, shallow above, where the accumulators and
// a whole k-step of A fragments take the registers.
template <int MB> struct SkShape {
    static constexpr int D = MB == 1 ? 4 : MB <= 4 ? 6 : 2;
};
constexpr int kSkMaxW = 15;                     // compute waves in the largest workgroup

template <int FMT, int MB, bool WRITE_P>
__global__ __launch_bounds__(64 * (kSkMaxW + 1)) void skinny_kernel(const int8_t *__restrict__ q, const float *__restrict__ scale,
                   const int8_t *__restrict__ codes, const void *__restrict__ gscale,
                   const uint16_t *__restrict__ rscale, float *__restrict__ y,
                   int32_t *__restrict__ partials, int M, int N, int K) {
    constexpr int MP = 16 * MB;                       // token rows, padded
    constexpr int ABYTES = MP * kSkStageK;            // one activation stage
    constexpr int GW = (FMT == kFmtU8) ? 256 : 128;   // K bytes per group
    constexpr int SPG = GW / kSkStageK;               // stages per group
    constexpr int NDMA = ABYTES / 1024;               // producer loads per stage
    constexpr int kSkD = SkShape<MB>::D;
    static_assert(kSkD % SPG == 0, "a ring turn holds whole groups");
    __shared__ __attribute__((aligned(1024))) int8_t As[kSkRing][ABYTES];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int nw = static_cast<int>(blockDim.x >> 6) - 1;   // compute waves; the last wave produces
    const int NS = K / kSkStageK;
    const int G = K / GW;
    // Workgroups start their K walk at different groups (and wrap around),
    // so the activation slice every producer reads at a given moment is not
    // the same few cache lines on the same L2 channels across the GPU.
    const int soff = SPG * (static_cast<int>(blockIdx.x) % G);
    auto phys = [&](int s) { return (min(s, NS - 1) + soff) % NS; };   // past the end: re-read

    if (wid == nw) {
        // ---- producer.  Load i of a stage fills token rows 8 i .. 8 i + 7:
        // lane l takes row 8 i + l / 8, slot l % 8, i.e. logical chunk
        // (l % 8) ^ swz(row).  Token rows past M repeat row M - 1.
        uint32_t offs[NDMA];
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int row = 8 * i + (lane >> 3);
            const int r = min(row, M - 1);
            offs[i] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) +
                      16u * static_cast<uint32_t>((lane & 7) ^ sk_swz(row));
        }
        auto issue = [&](int s) {
            const int buf = s % kSkRing;
#pragma unroll
            for (int i = 0; i < NDMA; ++i)
                dma16(q + static_cast<int64_t>(phys(s)) * kSkStageK, offs[i], lds_offset(&As[buf][i * 1024]));
        };
        issue(0);
        if (NS > 1) issue(1);
        for (int s = 0; s < NS; ++s) {
            // stage s has landed once at most the next stage's loads remain
            if (s + 1 < NS)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (s + 2 < NS) issue(s + 2);       // into the buffer of stage s - 1
        }
        return;
    }

    // ---- compute waves
    const int j = lane & 15, qd = lane >> 4;
    const int n0 = (blockIdx.x * nw + wid) * 16;
    const int nrow = n0 + j;
    const bool nvalid = nrow < N;
    const int nr = min(nrow, N - 1);
    constexpr int EPB = kElemsPerByte<FMT>;
    constexpr int WL = 2 / EPB;                       // 16-byte weight loads per stage
    const int8_t *wrow = codes + static_cast<int64_t>(nr) * (K / EPB) + 16 * qd;

    auto load_w = [&](int s, v4i(&dst)[WL]) {
        const int64_t off = static_cast<int64_t>(phys(s)) * (kSkStageK / EPB);
#pragma unroll
        for (int kk = 0; kk < WL; ++kk) dst[kk] = ld16(wrow + off + 64 * kk);
    };
    // Group scales ride in the ring as raw bits and are converted only when
    // folded: converting at load time would make the wave wait for the load
    // right away, and with in-order completion that drains the whole ring.
    auto load_scale = [&](int g) -> uint32_t {
        const int64_t idx = static_cast<int64_t>(nr) * G + phys(SPG * g) / SPG;
        if constexpr (FMT == kFmtU8)
            return static_cast<const uint8_t *>(gscale)[idx];
        else
            return static_cast<const uint16_t *>(gscale)[idx];
    };
    auto scale_value = [&](uint32_t raw) -> float {
        if constexpr (FMT == kFmtU8)
            return static_cast<float>(raw);
        else
            return bf16_to_f32(static_cast<uint16_t>(raw));
    };

    v4i wr[kSkD][WL];
    uint32_t scr[kSkD / SPG];                         // scale bits of each group in the ring
#pragma unroll
    for (int i = 0; i < kSkD; ++i) {
        load_w(i, wr[i]);
        if (i % SPG == 0) scr[i / SPG] = load_scale(i / SPG);
    }

    v4i P[MB];
    float F[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        P[mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) F[mb][e] = 0.0f;
    }

    // the LDS byte offset of this lane's A chunk c of token row 16 mb + j
    auto a_off = [&](int mb, int c) {
        const int row = 16 * mb + j;
        return 128 * row + 16 * (c ^ sk_swz(row));
    };

    [[maybe_unused]] const Tbl4Masks tk = tbl4_masks();
    // one stage: s the stage, i = s mod kSkD its ring slot (a constant after
    // unrolling)
    auto stage = [&](int s, int i) {
        __builtin_amdgcn_s_barrier();                 // stage s is in LDS
        asm volatile("" ::: "memory");
        const int8_t *Ab = As[s % kSkRing];
        v4i bw[2];                                    // the stage's B operands
        if constexpr (FMT == kFmtTbl4) {
            tbl4_decode16(wr[i][0], bw[0], bw[1], tk);
        } else {
            bw[0] = wr[i][0];
            bw[1] = wr[i][1];
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v4i a[MB];                                // the k-step's A fragments, read together
            const int ac = (FMT == kFmtTbl4) ? 2 * qd + kk : 4 * kk + qd;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const v4i *>(Ab + a_off(mb, ac));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                P[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb], bw[kk], P[mb], 0, 0, 0);
        }
        load_w(s + kSkD, wr[i]);                      // refill the slot just used
        if (i % SPG == SPG - 1) {
            // the group ends here: fold it, then refill its scale slot
            const int g = phys(s) / SPG;              // the K group just completed
            // opaque here, after this stage's barrier: keeps the scheduler
            // from converting (and so waiting for) the scale any earlier
            uint32_t raw = scr[i / SPG];
            asm volatile("" : "+v"(raw));
            const float sc = scale_value(raw);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if constexpr (WRITE_P) {
                    if (nvalid) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = 16 * mb + 4 * qd + e;
                            if (m < M) partials[(static_cast<int64_t>(m) * N + nrow) * G + g] = P[mb][e];
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) F[mb][e] += static_cast<float>(P[mb][e]) * sc;
                P[mb] = v4i{0, 0, 0, 0};
            }
            scr[i / SPG] = load_scale(s / SPG + kSkD / SPG);
        }
    };
    // Whole ring turns in a branch-free loop (so the compiler's wait counts
    // keep kSkD stages in flight across the back edge), then the remainder.
    const int NSm = NS - NS % kSkD;
    for (int s0 = 0; s0 < NSm; s0 += kSkD) {
#pragma unroll
        for (int i = 0; i < kSkD; ++i) stage(s0 + i, i);
    }
#pragma unroll
    for (int i = 0; i < kSkD; ++i)
        if (NSm + i < NS) stage(NSm + i, i);

    if (!nvalid) return;
    float rn = 0x1p-7f;
    if constexpr (FMT == kFmtU8) rn = bf16_to_f32(rscale[nrow]) * 0x1p-7f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mb + 4 * qd + e;
            if (m < M) y[static_cast<int64_t>(m) * N + nrow] = F[mb][e] * (scale[m] * rn);
        }
}

// Compute waves per workgroup.  A workgroup costs its rows plus a fixed part
// that does not shrink with them (its own pass of the M x K activation codes
// through LDS, the pipeline fill and drain), and a CU runs one wide
// workgroup at a time, so the kernel takes (rounds of workgroups per CU) x
// (16 nw + fixed).  Measured on MI355X (256 CUs, M = 16 ... 128, the 34816-,
// 152064- and 5120-row layers): if one round covers the rows, the narrowest
// workgroup that does so is fastest (nw = 9 for 34816 rows, 2 for 5120);
// otherwise the width from 8 to 15 minimising rounds x (16 nw + fixed), with
// the fixed part worth about 300 rows (nw = 13 for 152064 rows).
constexpr int kSkFixedRows = 300;

int sk_compute_waves(int64_t N, int cus) {
    const int64_t tiles = (N + 15) / 16;
    if (tiles <= static_cast<int64_t>(kSkMaxW) * cus)
        return static_cast<int>(std::max<int64_t>(1, (tiles + cus - 1) / cus));
    int best = kSkMaxW;
    int64_t best_cost = INT64_MAX;
    for (int w = 8; w <= kSkMaxW; ++w) {
        const int64_t per_round = static_cast<int64_t>(w) * cus;
        const int64_t cost = (tiles + per_round - 1) / per_round * (16 * w + kSkFixedRows);
        if (cost < best_cost) {
            best_cost = cost;
            best = w;
        }
    }
    return best;
}

template <int FMT, int MB>
hipError_t launch_skinny_t(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                           int32_t *P, hipStream_t st) {
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int nw = sk_compute_waves(w.N, cus);
    const int64_t rows_per_wg = 16 * static_cast<int64_t>(nw);
    const int grid = static_cast<int>((w.N + rows_per_wg - 1) / rows_per_wg);
    auto kern = P ? skinny_kernel<FMT, MB, true> : skinny_kernel<FMT, MB, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * (nw + 1)), 0, st, q, s, w.codes, w.gscale, w.rscale, y,
                       P, static_cast<int>(M), static_cast<int>(w.N), static_cast<int>(w.K));
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

inline bool m1_supported(int64_t K, int fmt) {
    const int G = static_cast<int>(K / (fmt == kFmtU8 ? 256 : 128));
    const int esz = fmt == kFmtU8 ? 1 : 2;
    return K <= kM1MaxK && 4 * G * esz <= kScBytes && m1_steps_supported(m1_steps(K, fmt));
}

}  // namespace

int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t launch_gemv(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st) {
    if (M == 1 && decode_row_supported(w)) {
        return launch_decode_row(nullptr, const_cast<int8_t *>(q), const_cast<float *>(s), w, y, partials,
                                 false, st);                     // read only: not fused
    }
    if (M == 1 && m1_supported(w.K, w.fmt)) {
        int8_t *qi = const_cast<int8_t *>(q);            // read only: FUSED == false
        float *si = const_cast<float *>(s);
        if (w.fmt == kFmtU8) return launch_m1<kFmtU8, false>(nullptr, qi, si, w, y, partials, st);
        if (w.fmt == kFmtHead) return launch_m1<kFmtHead, false>(nullptr, qi, si, w, y, partials, st);
        return launch_m1<kFmtTbl4, false>(nullptr, qi, si, w, y, partials, st);
    }
    if (w.fmt == kFmtU8) return launch_skinny<kFmtU8>(q, s, w, y, M, partials, st);
    if (w.fmt == kFmtHead) return launch_skinny<kFmtHead>(q, s, w, y, M, partials, st);
    return launch_skinny<kFmtTbl4>(q, s, w, y, M, partials, st);
}

bool fused_decode_supported(const WeightArgs &w, int64_t M) {
    return M == 1 && (decode_row_supported(w) || m1_supported(w.K, w.fmt));
}

hipError_t launch_fused_decode(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y,
                               hipStream_t st) {
    if (decode_row_supported(w)) return launch_decode_row(x, q, s, w, y, nullptr, true, st);
    if (w.fmt == kFmtU8) return launch_m1<kFmtU8, true>(x, q, s, w, y, nullptr, st);
    if (w.fmt == kFmtHead) return launch_m1<kFmtHead, true>(x, q, s, w, y, nullptr, st);
    return launch_m1<kFmtTbl4, true>(x, q, s, w, y, nullptr, st);
}

}  // namespace rad
