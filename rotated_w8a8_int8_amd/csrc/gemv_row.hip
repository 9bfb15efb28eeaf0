// gemv_row.hip -- the layer for one token (M == 1) with weight rows streamed
// whole, 1 KiB per load instruction: the trunk's int8 format, and below it
// the drafter's 4-bit codebook format (gfx950).
//
// What is computed (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container", table rows "Weights" and "Activations"): int8 activation codes
// times int8 weight codes of the same rotated domain, exact int32 sums per
// 256 of K under a u8 scale, then y = s * r_n * 2^-7 * sum_g u8[n][g] P[n][g].
//
// Layout.  Wave w owns weight rows w, w + W, w + 2W, ... (W waves in all, so
// at any moment the GPU streams one contiguous band of rows).  One load
// instruction of a wave reads 1 KiB of one row (lane l: bytes 16 l .. 16 l +
// 15 of the KiB), so lane l always meets the same activation bytes: its K / 1024
// activation chunks stay in registers for the whole stream and the loop reads
// no LDS.  The loads are nontemporal (each weight byte is read once) and kept
// D deep in a ring that spans R rows.  A row's u8 group scales are K / 1024
// dwords, loaded (one per lane) with the row's weights; at step t every lane
// reads dword t across lanes and takes its byte l / 16 (the 16 lanes with
// l / 16 == j cover group 4 t + j).
//
// Exactness: a lane's partial of one step is a 16-element dot product (|p| <
// 2^18), times u8 (< 2^26); summed over at most 20 steps it stays below 2^31.
// The 64 lanes' sums are added exactly in two 16-bit halves, and
// s * r * 2^-7 * S is evaluated in f64 and rounded once, as the oracle does,
// so y is the oracle's bit for bit.
//
// FUSED: the workgroup first rotates and quantises the f32 token (the same
// device code, bits and reciprocal scheme as rad_quant_act_i8) while its first
// weight loads are in flight; block 0 also writes the codes and the scale.
// (Workgroups with extra waves that only share the rotation measured slower.)
//
// The head format (bf16 scale per 128 of K) uses the same layout with an f32
// fold of the group scales.
//
// The drafter's codebook format (model card, table row "Speculator": 4-bit
// indices into a 16-level table, bf16 scale per 128) has a variant below:
// a row is K / 2 bytes, so one load instruction reads 512 bytes of each of
// two rows (lanes 0..31 and 32..63), 32 elements a lane, expanded with the
// table lookups in registers; group scales are folded in f32.
#include "rad_device.h"
#include "rad_launch.h"
#include "rotate_quant.h"

namespace rad {
namespace {

// Ring of R whole rows, D = NS * R loads of 1 KiB per lane, about ten deep.
template <int NS> struct RowShape {
    static constexpr int R = NS >= 10 ? 1 : (10 + NS - 1) / NS;
    static constexpr int D = NS * R;
};

// Exact sum of an int32 over the 64 lanes of the wave, as int64.
__device__ __forceinline__ int64_t wave_sum_exact(int v) {
    int hi = row16_sum(v >> 16);                 // |hi| < 2^15 per lane
    int lo = row16_sum(v & 0xFFFF);              // < 2^16 per lane
    const int64_t h = static_cast<int64_t>(__builtin_amdgcn_readlane(hi, 0)) +
                      __builtin_amdgcn_readlane(hi, 16) + __builtin_amdgcn_readlane(hi, 32) +
                      __builtin_amdgcn_readlane(hi, 48);
    const int64_t l = static_cast<int64_t>(__builtin_amdgcn_readlane(lo, 0)) +
                      __builtin_amdgcn_readlane(lo, 16) + __builtin_amdgcn_readlane(lo, 32) +
                      __builtin_amdgcn_readlane(lo, 48);
    return h * 65536 + l;
}

constexpr int kRowWgWaves = 4;                   // waves of a workgroup

// The fused prologue, in two parts so the caller can issue its first weight
// loads between them.  Each wave holds blocks (it * WGW + wid) * 4 + r4 of
// the token, 16 lanes a block (blocks past the row re-read the last one).
template <int NQ, int NBLK, int WGW>
__device__ __forceinline__ void token_load(const float *__restrict__ x, Blk8 (&xv)[NQ], int wid, int r4,
                                           int l16) {
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int blk = (it * WGW + wid) * 4 + r4;
        const float *p = x + min(blk, NBLK - 1) * 128 + 4 * l16;
        xv[it].lo = *reinterpret_cast<const float4 *>(p);
        xv[it].hi = *reinterpret_cast<const float4 *>(p + 64);
    }
}

// Rotate, find the token's amax over the workgroup, and write its codes to
// q_lds (block 0 also to qio, and the scale to sio); returns the scale.  Ends
// with a barrier, so q_lds is complete when it returns.
template <int NQ, int NBLK, int WGW>
__device__ __forceinline__ float token_quantise(Blk8 (&xv)[NQ], int8_t *q_lds, float *red,
                                                int8_t *__restrict__ qio, float *__restrict__ sio, int wid,
                                                int r4, int l16, int lane) {
    // A block past the row holds a re-read of the last one: it is rotated
    // with the others and left out of the amax (its codes are never stored).
    // Zeroing it before the rotation instead let the compiler make its load
    // conditional and move it behind the first weight loads, so the rotation
    // waited for all of them.
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        fwht128_regs_signed(xv[it], l16);   // values times the lane sign c
        const float m = fmaxf(amax4(xv[it].lo), amax4(xv[it].hi));
        amax = fmaxf(amax, (it * WGW + wid) * 4 + r4 < NBLK ? m : 0.0f);
    }
    amax = wave_max_f32(amax);
    if (lane == 0) red[wid] = amax;
    __syncthreads();
    float am = red[0];
#pragma unroll
    for (int v = 1; v < WGW; ++v) am = fmaxf(am, red[v]);
    const float s = am / 127.0f;
    const bool fast = s >= 0x1p-120f;
    const float c = fwht_lane_sign(l16);
    const float rs_c = c * (1.0f / s);
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int blk = (it * WGW + wid) * 4 + r4;
        if (blk < NBLK) {
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
    __syncthreads();
    return s;
}

template <int NS, bool FUSED, bool WRITE_P>
__global__ __launch_bounds__(64 * kRowWgWaves) void decode_row_kernel(const float *__restrict__ x,
                                                         int8_t *__restrict__ qio,
                                                         float *__restrict__ sio,
                                                         const int8_t *__restrict__ codes,
                                                         const uint32_t *__restrict__ gscale,
                                                         const uint16_t *__restrict__ rscale,
                                                         float *__restrict__ y,
                                                         int32_t *__restrict__ partials, int N) {
    constexpr int K = NS * 1024;
    constexpr int R = RowShape<NS>::R, D = RowShape<NS>::D;
    constexpr int G = K / 256;                     // groups of a row; its scales are NS dwords
    constexpr int NBLK = K / 128;
    constexpr int WGW = kRowWgWaves;
    constexpr int NQ = (NBLK + 4 * WGW - 1) / (4 * WGW);   // rotation steps: 4 blocks a wave
    __shared__ __attribute__((aligned(16))) int8_t q_lds[FUSED ? K : 16];
    __shared__ float red[WGW];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int l16 = lane & 15, r4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * WGW + wid);
    const int W = gridDim.x * WGW;
    const int cnt = wave < N ? (N - wave + W - 1) / W : 0;   // rows of this wave
    const int groups = (cnt + R - 1) / R;
    // row j of this wave, clamped in bounds (loads past the wave's last row
    // re-read it and are never used)
    auto row_of = [&](int j) { return min(wave + min(j, max(cnt - 1, 0)) * W, N - 1); };
    auto wload = [&](int j, int t) -> v4i {
        return ld16_nt(codes + static_cast<int64_t>(row_of(j)) * K + 1024 * t + 16 * lane);
    };

    // 1. the token: f32 into registers (fused; blocks past the row re-read
    //    the last one and are zeroed after the load), or its codes
    Blk8 xv[NQ];
    v4i a[NS];
    float s = 0.0f;
    if constexpr (FUSED) {
        token_load<NQ, NBLK, WGW>(x, xv, wid, r4, l16);
    } else {
#pragma unroll
        for (int t = 0; t < NS; ++t) a[t] = ld16(qio + 1024 * t + 16 * lane);
        s = sio[0];
    }

    // 2. the scales of rows 0 .. R-1 (each row's NS scale dwords, lane l
    //    holding dword l % NS, and its row scale), then the first D weight
    //    loads (rows 0 .. R-1), all behind the token's loads and ahead of the
    //    rotation, which then waits for the token only.  Issued after the
    //    rotation, the scales cost the first row a whole memory latency.
    auto sload = [&](int j) -> uint32_t { return gscale[static_cast<int64_t>(row_of(j)) * NS + lane % NS]; };
    auto rload = [&](int j) -> uint32_t { return rscale[row_of(j)]; };
    uint32_t scr[R], rsr[R];
    v4i ring[D];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        scr[rr] = sload(rr);
        rsr[rr] = rload(rr);
    }
#pragma unroll
    for (int i = 0; i < D; ++i) ring[i] = wload(i / NS, i % NS);
    __builtin_amdgcn_sched_barrier(0);

    // 3. fused: rotate and quantise the token into LDS (block 0: to q and s)
    if constexpr (FUSED) {
        s = token_quantise<NQ, NBLK, WGW>(xv, q_lds, red, qio, sio, wid, r4, l16, lane);
#pragma unroll
        for (int t = 0; t < NS; ++t) a[t] = *reinterpret_cast<const v4i *>(&q_lds[1024 * t + 16 * lane]);
    }

    // 4. the weight stream, R rows per turn of the ring.  A row's scales ride
    //    in the ring with its weight loads, issued R rows ahead and
    //    unconditionally, so the compiler's in-order wait counts cover them.
    const int shift = 8 * r4;                      // byte of a scale dword this lane takes
    for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int j = gi * R + rr;
            const int row = row_of(j);
            int acc = 0;
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int i = rr * NS + t;
                const int p = dot16_i8(ring[i], a[t], 0);
                const uint32_t sd = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(scr[rr]), t));
                // |p| <= 16 * 127^2 < 2^23: a full-rate 24-bit multiply
                acc += __mul24(p, static_cast<int>((sd >> shift) & 0xFFu));
                if constexpr (WRITE_P) {
                    const int pg = row16_sum(p);
                    if (l16 == 0 && j < cnt) partials[static_cast<int64_t>(row) * G + 4 * t + r4] = pg;
                }
                ring[i] = wload(j + R, t);
            }
            const uint16_t rb = static_cast<uint16_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(rsr[rr])));
            scr[rr] = sload(j + R);
            rsr[rr] = rload(j + R);
            const int64_t S = wave_sum_exact(acc);
            if (lane == 0 && j < cnt) {
                const double rn = static_cast<double>(bf16_to_f32(rb));
                y[row] = static_cast<float>(static_cast<double>(s) * rn * 0x1p-7 * static_cast<double>(S));
            }
        }
    }
}

// The head format (int8 codes, a bf16 scale per 128 of K), K a multiple of
// 1024 up to 16384: the layout, ring and prologue of the kernel above.  Lane l
// meets group 8 t + l / 8 at step t; a row's K / 128 bf16 scales are K / 256
// dwords, loaded one per lane with the row (lanes past them re-load the
// last), and at step t a lane fetches dword 4 t + l / 16 with a lane permute
// and takes its half (l / 8) % 2.  Each lane folds its 16-element dot product
// times the group scale into an f32 sum; the wave adds the 64 sums in a fixed
// order, and y = s * 2^-7 * sum.
template <int NS, bool FUSED, bool WRITE_P>
__global__ __launch_bounds__(64 * kRowWgWaves) void decode_row_head_kernel(const float *__restrict__ x,
                                                              int8_t *__restrict__ qio,
                                                              float *__restrict__ sio,
                                                              const int8_t *__restrict__ codes,
                                                              const uint32_t *__restrict__ gscale,
                                                              float *__restrict__ y,
                                                              int32_t *__restrict__ partials, int N) {
    constexpr int K = NS * 1024;
    constexpr int R = RowShape<NS>::R, D = RowShape<NS>::D;
    constexpr int G = K / 128;                     // groups of a row: G / 2 scale dwords
    constexpr int SD = G / 2;
    static_assert(SD <= 64, "one scale dword of the row per lane");
    constexpr int NBLK = K / 128;
    constexpr int WGW = kRowWgWaves;
    constexpr int NQ = (NBLK + 4 * WGW - 1) / (4 * WGW);
    __shared__ __attribute__((aligned(16))) int8_t q_lds[FUSED ? K : 16];
    __shared__ float red[WGW];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int l16 = lane & 15, r4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * WGW + wid);
    const int W = gridDim.x * WGW;
    const int cnt = wave < N ? (N - wave + W - 1) / W : 0;   // rows of this wave
    const int groups = (cnt + R - 1) / R;
    auto row_of = [&](int j) { return min(wave + min(j, max(cnt - 1, 0)) * W, N - 1); };
    auto wload = [&](int j, int t) -> v4i {
        return ld16_nt(codes + static_cast<int64_t>(row_of(j)) * K + 1024 * t + 16 * lane);
    };

    Blk8 xv[NQ];
    v4i a[NS];
    float s = 0.0f;
    if constexpr (FUSED) {
        token_load<NQ, NBLK, WGW>(x, xv, wid, r4, l16);
    } else {
#pragma unroll
        for (int t = 0; t < NS; ++t) a[t] = ld16(qio + 1024 * t + 16 * lane);
        s = sio[0];
    }

    // the first rows' scales, then the first ring, ahead of the rotation
    auto sload = [&](int j) -> uint32_t {
        return gscale[static_cast<int64_t>(row_of(j)) * SD + min(lane, SD - 1)];
    };
    uint32_t scr[R];
    v4i ring[D];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) scr[rr] = sload(rr);
#pragma unroll
    for (int i = 0; i < D; ++i) ring[i] = wload(i / NS, i % NS);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (FUSED) {
        s = token_quantise<NQ, NBLK, WGW>(xv, q_lds, red, qio, sio, wid, r4, l16, lane);
#pragma unroll
        for (int t = 0; t < NS; ++t) a[t] = *reinterpret_cast<const v4i *>(&q_lds[1024 * t + 16 * lane]);
    }

    const int sperm = 4 * (lane / 16);             // byte address of this lane's scale lane at t = 0
    const int shift = 16 * ((lane >> 3) & 1);
    const float sy = s * 0x1p-7f;
    for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int j = gi * R + rr;
            const int row = row_of(j);
            float accf = 0.0f;
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int i = rr * NS + t;
                const int p = dot16_i8(ring[i], a[t], 0);
                const uint32_t sd = static_cast<uint32_t>(
                    __builtin_amdgcn_ds_bpermute(sperm + 16 * t, static_cast<int>(scr[rr])));
                accf += static_cast<float>(p) * bf16_to_f32(static_cast<uint16_t>((sd >> shift) & 0xFFFFu));
                if constexpr (WRITE_P) {
                    const int pg = row8_sum(p);
                    if ((lane & 7) == 0 && j < cnt) partials[static_cast<int64_t>(row) * G + 8 * t + lane / 8] = pg;
                }
                ring[i] = wload(j + R, t);
            }
            scr[rr] = sload(j + R);
            const float tot = wave_sum_f32(accf);
            if (lane == 0 && j < cnt) y[row] = sy * tot;
        }
    }
}

// The codebook format, K a multiple of 1024 up to 8192.  Wave w owns row
// pairs w, w + W, ...; lanes 0..31 stream the pair's first row and lanes
// 32..63 its second, 512 bytes of packed indices a row per load instruction,
// so lane l32 = l % 32 always holds run 32 t + l32 of step t (elements
// 1024 t + 32 l32 .. + 31, group 8 t + l32 / 4) and keeps the matching 32
// activation codes of every step in registers.  A row's K / 128 bf16 group
// scales are K / 256 dwords, loaded one per lane with the row (lanes past
// them re-load the last); at step t a lane fetches dword 4 t + l32 / 8 of its
// half with a lane permute and takes its half (l32 / 4) % 2.  Each lane folds
// its 32-element dot product times the group scale into an f32 sum; the 32
// lanes of a row add theirs in a fixed order, and y = s * 2^-7 * sum.
template <int NS, bool FUSED, bool WRITE_P>
__global__ __launch_bounds__(64 * kRowWgWaves) void decode_row_tbl4_kernel(const float *__restrict__ x,
                                                              int8_t *__restrict__ qio,
                                                              float *__restrict__ sio,
                                                              const int8_t *__restrict__ codes,
                                                              const uint32_t *__restrict__ gscale,
                                                              float *__restrict__ y,
                                                              int32_t *__restrict__ partials, int N) {
    constexpr int K = NS * 1024;
    constexpr int KB = K / 2;                      // packed bytes of a row
    constexpr int R = RowShape<NS>::R, D = RowShape<NS>::D;   // R row pairs per ring turn
    constexpr int G = K / 128;                     // groups of a row: G / 2 scale dwords
    constexpr int SD = G / 2;
    static_assert(SD <= 32, "a half-wave holds one scale dword of its row per lane");
    constexpr int NBLK = K / 128;
    constexpr int WGW = kRowWgWaves;
    constexpr int NQ = (NBLK + 4 * WGW - 1) / (4 * WGW);
    __shared__ __attribute__((aligned(16))) int8_t q_lds[FUSED ? K : 16];
    __shared__ float red[WGW];

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int l16 = lane & 15, r4 = lane >> 4;
    const int h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * WGW + wid);
    const int W = gridDim.x * WGW;
    const int NP = (N + 1) / 2;                              // row pairs
    const int cnt = wave < NP ? (NP - wave + W - 1) / W : 0;  // pairs of this wave
    const int groups = (cnt + R - 1) / R;
    // pair j of this wave, or pair 0 past the wave's last one (the last ring
    // turn's refills are never used: aimed at one pair, they are served by
    // the caches, 19.7 against 20.3 us when they re-read each wave's last pair,
    // one box; the int8 kernel measured the opposite, 31.1 against 29.8 us);
    // this lane's row of it (the second row of a last pair with N odd
    // re-reads row N - 1, never stored)
    auto pair_of = [&](int j) { return j < cnt ? wave + j * W : 0; };
    auto row_of = [&](int j) { return min(2 * pair_of(j) + h, N - 1); };
    auto wload = [&](int j, int t) -> v4i {
        return ld16_nt(codes + static_cast<int64_t>(row_of(j)) * KB + 512 * t + 16 * l32);
    };

    Blk8 xv[NQ];
    v4i a0[NS], a1[NS];
    float s = 0.0f;
    if constexpr (FUSED) {
        token_load<NQ, NBLK, WGW>(x, xv, wid, r4, l16);
    } else {
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            a0[t] = ld16(qio + 1024 * t + 32 * l32);
            a1[t] = ld16(qio + 1024 * t + 32 * l32 + 16);
        }
        s = sio[0];
    }

    // the first pairs' scales, then the first ring, ahead of the rotation
    auto sload = [&](int j) -> uint32_t {
        return gscale[static_cast<int64_t>(row_of(j)) * SD + min(l32, SD - 1)];
    };
    uint32_t scr[R];
    v4i ring[D];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) scr[rr] = sload(rr);
#pragma unroll
    for (int i = 0; i < D; ++i) ring[i] = wload(i / NS, i % NS);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (FUSED) {
        s = token_quantise<NQ, NBLK, WGW>(xv, q_lds, red, qio, sio, wid, r4, l16, lane);
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            a0[t] = *reinterpret_cast<const v4i *>(&q_lds[1024 * t + 32 * l32]);
            a1[t] = *reinterpret_cast<const v4i *>(&q_lds[1024 * t + 32 * l32 + 16]);
        }
    }

    const Tbl4Masks tk = tbl4_masks();
    const int sperm = 4 * (32 * h + l32 / 8);      // byte address of this lane's scale lane at t = 0
    const int shift = 16 * ((l32 >> 2) & 1);
    const float sy = s * 0x1p-7f;
    for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int j = gi * R + rr;
            const int row = 2 * pair_of(j) + h;
            float accf = 0.0f;
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int i = rr * NS + t;
                v4i lo, hi;
                tbl4_decode16(ring[i], lo, hi, tk);
                const int p = dot16_i8(hi, a1[t], dot16_i8(lo, a0[t], 0));
                const uint32_t sd = static_cast<uint32_t>(
                    __builtin_amdgcn_ds_bpermute(sperm + 16 * t, static_cast<int>(scr[rr])));
                accf += static_cast<float>(p) * bf16_to_f32(static_cast<uint16_t>((sd >> shift) & 0xFFFFu));
                if constexpr (WRITE_P) {
                    const int pg = row4_sum(p);
                    if ((l32 & 3) == 0 && j < cnt && row < N)
                        partials[static_cast<int64_t>(row) * G + 8 * t + l32 / 4] = pg;
                }
                ring[i] = wload(j + R, t);
            }
            scr[rr] = sload(j + R);
            accf += lane_xor<1>(accf);
            accf += lane_xor<2>(accf);
            accf += lane_xor<4>(accf);
            accf += lane_xor<8>(accf);
            const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(accf), 0)) +
                             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(accf), 16));
            const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(accf), 32)) +
                             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(accf), 48));
            if (lane == 0 && j < cnt) {
                const int r = 2 * pair_of(j);
                y[r] = sy * r0;
                if (r + 1 < N) y[r + 1] = sy * r1;
            }
        }
    }
}

// One workgroup of four waves per CU: measured on MI355X (decode_gate_up,
// 256 CUs), 1024 waves in all streamed fastest; more waves (two workgroups on
// some or all CUs), fewer (idle CUs), deeper rings and a deeper first ring
// were all slower.  The codebook kernel issues about twice the vector
// instructions per byte (the table lookups) and runs three such workgroups
// per CU: drafter_decode 20.8 us against 23.5 (one), 21.8 (two) and 20.9
// (four); a ring of one pair instead of two, 21.4 us.  Units per wave (rows,
// or row pairs) are rounded to whole rings where possible.
template <int NS, bool FUSED>
hipError_t launch_row_t(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y, int32_t *P,
                        hipStream_t st) {
    constexpr int R = RowShape<NS>::R;
    const int N = static_cast<int>(w.N);
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const bool tbl = w.fmt == 2;
    const int units = tbl ? (N + 1) / 2 : N;                // rows, or row pairs
    const int target = kRowWgWaves * cus * (tbl ? 3 : 1);
    int per = (units + target - 1) / target;                // units per wave
    per = ((per + R - 1) / R) * R;
    const int waves = (units + per - 1) / per;
    const int grid = (waves + kRowWgWaves - 1) / kRowWgWaves;
    const uint32_t *gs = static_cast<const uint32_t *>(w.gscale);
    if (w.fmt == 1) {
        if constexpr (NS <= 16) {
            auto kern = P ? decode_row_head_kernel<NS, FUSED, true> : decode_row_head_kernel<NS, FUSED, false>;
            hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kRowWgWaves), 0, st, x, q, s, w.codes, gs, y, P, N);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;                      // excluded by decode_row_supported
        }
    }
    if (tbl) {
        if constexpr (NS <= 8) {
            auto kern = P ? decode_row_tbl4_kernel<NS, FUSED, true> : decode_row_tbl4_kernel<NS, FUSED, false>;
            hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kRowWgWaves), 0, st, x, q, s, w.codes, gs, y, P, N);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;                      // excluded by decode_row_supported
        }
    }
    auto kern = P ? decode_row_kernel<NS, FUSED, true> : decode_row_kernel<NS, FUSED, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kRowWgWaves), 0, st, x, q, s, w.codes, gs, w.rscale, y,
                       P, N);
    return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_row(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y, int32_t *P,
                      hipStream_t st) {
    switch (w.K / 1024) {
#define RAD_ROW_CASE(S) case S: return launch_row_t<S, FUSED>(x, q, s, w, y, P, st);
        RAD_ROW_CASE(1) RAD_ROW_CASE(2) RAD_ROW_CASE(3) RAD_ROW_CASE(4) RAD_ROW_CASE(5)
        RAD_ROW_CASE(6) RAD_ROW_CASE(8) RAD_ROW_CASE(10) RAD_ROW_CASE(12) RAD_ROW_CASE(16)
        RAD_ROW_CASE(17) RAD_ROW_CASE(20)
#undef RAD_ROW_CASE
        default: return hipErrorInvalidValue;              // excluded by decode_row_supported
    }
}

}  // namespace

bool decode_row_supported(const WeightArgs &w) {
    if (w.K % 1024 != 0) return false;
    const int64_t ns = w.K / 1024;
    if (w.fmt == 2) return ns <= 6 || ns == 8;               // codebook: K <= 8192
    if (w.fmt == 1 && ns > 16) return false;                  // head: K <= 16384
    if (w.fmt != 0 && w.fmt != 1) return false;
    switch (ns) {
        case 1: case 2: case 3: case 4: case 5: case 6: case 8: case 10: case 12: case 16: case 17: case 20:
            return true;
        default:
            return false;
    }
}

hipError_t launch_decode_row(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y,
                             int32_t *partials, bool fused, hipStream_t st) {
    return fused ? launch_row<true>(x, q, s, w, y, partials, st)
                 : launch_row<false>(x, q, s, w, y, partials, st);
}

}  // namespace rad
