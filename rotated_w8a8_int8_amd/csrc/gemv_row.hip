// gemv_row.hip -- the trunk layer for one token (M == 1) with weight rows
// streamed whole, 1 KiB per load instruction (gfx950).
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
#include "rad_device.h"
#include "rad_launch.h"
#include "rotate_quant.h"

namespace rad {
namespace {

constexpr int kRowMaxSteps = 20;                 // K <= 20480

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
    Blk8 xv[FUSED ? NQ : 1];
    v4i a[NS];
    float s = 0.0f;
    if constexpr (FUSED) {
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int blk = (it * WGW + wid) * 4 + r4;
            const float *p = x + min(blk, NBLK - 1) * 128 + 4 * l16;
            xv[it].lo = *reinterpret_cast<const float4 *>(p);
            xv[it].hi = *reinterpret_cast<const float4 *>(p + 64);
        }
    } else {
#pragma unroll
        for (int t = 0; t < NS; ++t) a[t] = ld16(qio + 1024 * t + 16 * lane);
        s = sio[0];
    }

    // 2. the first D weight loads (rows 0 .. R-1), kept behind the token's
    //    loads and ahead of the rotation, which then waits for the token only
    v4i ring[D];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < D; ++i) ring[i] = wload(i / NS, i % NS);
    __builtin_amdgcn_sched_barrier(0);

    // 3. fused: rotate and quantise the token into LDS (block 0: to q and s)
    if constexpr (FUSED) {
        float amax = 0.0f;
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            if ((it * WGW + wid) * 4 + r4 >= NBLK) {
                xv[it].lo = make_float4(0.f, 0.f, 0.f, 0.f);
                xv[it].hi = xv[it].lo;
            }
            fwht128_regs_signed(xv[it], l16);   // values times the lane sign c
            amax = fmaxf(amax, fmaxf(amax4(xv[it].lo), amax4(xv[it].hi)));
        }
        amax = wave_max_f32(amax);
        if (lane == 0) red[wid] = amax;
        __syncthreads();
        float am = red[0];
#pragma unroll
        for (int v = 1; v < WGW; ++v) am = fmaxf(am, red[v]);
        s = am / 127.0f;
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
#pragma unroll
        for (int t = 0; t < NS; ++t) a[t] = *reinterpret_cast<const v4i *>(&q_lds[1024 * t + 16 * lane]);
    }

    // 4. the weight stream, R rows per turn of the ring.  Each row's NS scale
    //    dwords (lane l holds dword l % NS) and its row scale ride in the ring
    //    with the row's weight loads, issued R rows ahead and unconditionally,
    //    so the compiler's in-order wait counts cover them.
    const int shift = 8 * r4;                      // byte of a scale dword this lane takes
    auto sload = [&](int j) -> uint32_t { return gscale[static_cast<int64_t>(row_of(j)) * NS + lane % NS]; };
    auto rload = [&](int j) -> uint32_t { return rscale[row_of(j)]; };
    uint32_t scr[R], rsr[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        scr[rr] = sload(rr);
        rsr[rr] = rload(rr);
    }
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

// One workgroup of four waves per CU: measured on MI355X (decode_gate_up,
// 256 CUs), 1024 waves in all streamed fastest; more waves (two workgroups on
// some or all CUs), fewer (idle CUs), deeper rings and a deeper first ring
// were all slower.  Rows per wave are rounded to whole rings where possible.
template <int NS, bool FUSED>
hipError_t launch_row_t(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y, int32_t *P,
                        hipStream_t st) {
    constexpr int R = RowShape<NS>::R;
    const int N = static_cast<int>(w.N);
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int target = kRowWgWaves * cus;
    int per = (N + target - 1) / target;                    // rows per wave
    per = ((per + R - 1) / R) * R;
    const int waves = (N + per - 1) / per;
    const int grid = (waves + kRowWgWaves - 1) / kRowWgWaves;
    auto kern = P ? decode_row_kernel<NS, FUSED, true> : decode_row_kernel<NS, FUSED, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kRowWgWaves), 0, st, x, q, s, w.codes,
                       static_cast<const uint32_t *>(w.gscale), w.rscale, y, P, N);
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
    if (w.fmt != 0 || w.K % 1024 != 0) return false;
    switch (w.K / 1024) {
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
