// quant_weight.hip -- weight-side int8 quantiser: rotate each 128-block of a
// float weight row, then choose, per K group, the scale with the least
// squared error among a fixed set of clipping candidates (gfx950).
//
// What is computed (recipe rules of section "How this file was made" on the
// model cards "Qwen3.8-Flash-Next, IQR-V4 -- radiance container": int8
// codes, group 128, bf16 scale, fwht128 transform, symmetric clamp, scale
// searched for least error; and "Qwen3.8-27B IQ8R + DFlash2 -- radiance
// container": int8 codes, group 256, u8 scale under a bf16 scale per row):
//
//   w~ = the row rotated per 128-block (same butterfly network and bits as
//        the activation rotation);
//   candidates c = 0..15 of a group: target_c = (amax_g * (64 - c) / 64) / 127
//        (f32 product, then f32 division);
//   head format: stored scale bf16_rne(target_c), d = its value;
//   u8 format:   row scale r = bf16_rne((amax_row / 127) / 255), stored
//        u8 = clamp(rne(target_c / r), 1, 255), d = r * u8 (exact);
//   codes clamp(rne(w~ / d), -127, 127) (f32 division; d = 0 gives 0);
//   error: sum over the group of (w~ - d q)^2 in f64, the sum taken as the
//        balanced pairwise tree over the group in index order;
//   the least error wins, ties to the smaller c.
// The drafter's codebook format (group 128, bf16 scale, model card "Qwen3.8-27B
// IQ8R + DFlash2 -- radiance container", section "How this file was made",
// rules dflash.*: rtn table=... rule=search) uses the head format's candidates;
// a code is the index of the table entry nearest to w~ / d (f32 division), a
// tie going to the smaller magnitude and 0 to +6, and the error uses d times
// that entry.  Its codes are always taken through the division.
//
// Layout: one 256-thread workgroup per weight row.  Phase 1 rotates the row
// block by block (16 lanes per block, butterflies in registers and DPP) into
// LDS and records each block's largest magnitude.  Phase 2 gives every wave
// whole groups: lane i of a wave holds the 4 consecutive elements 4i..4i+3 of
// a 256-element span (one u8 group, or two head groups on the two half-waves),
// so the pairwise error tree is the lane's own 2 levels followed by
// xor-butterflies across lanes: each level adds a lane's partial and its
// partner's, which is the tree's left + right on the lower lane and the same
// sum (IEEE addition commutes) on the upper one.  All f64 arithmetic uses
// explicitly rounded operations, so no multiply-add is contracted.
#include "rad_device.h"
#include "rad_launch.h"
#include "rotate_quant.h"

namespace rad {
namespace {

constexpr int kFmtU8 = 0;
constexpr int kFmtTbl4 = 2;
constexpr int kWqCandidates = 16;

// Nearest codebook entry to w / d: index (0..15) and value.  |t| is compared
// with the midpoints between the positive entries 6, 18, 30, 43, 58, 75, 97,
// 127 (all exact in f32); equality keeps the inner entry.
__device__ __forceinline__ int tbl4_nearest(float w, float d, float &value) {
    if (d == 0.0f) {
        value = 6.0f;
        return 8;
    }
    const float t = w / d;
    const float a = fabsf(t);
    const int cnt = (a > 12.0f) + (a > 24.0f) + (a > 36.5f) + (a > 50.5f) + (a > 66.5f) + (a > 86.0f) +
                    (a > 112.0f);
    const uint32_t mag = __builtin_amdgcn_perm(tbl4_dword(58, 75, 97, 127), tbl4_dword(6, 18, 30, 43),
                                               static_cast<uint32_t>(cnt)) & 0xFFu;
    const bool pos = t >= 0.0f;
    value = pos ? static_cast<float>(mag) : -static_cast<float>(mag);
    return pos ? 8 + cnt : 7 - cnt;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float wq_code(float w, float d) {
    if (d == 0.0f) return 0.0f;
    const float r = __builtin_rintf(w / d);
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

// The same code through the reciprocal: t = w * fl(1/d) is within
// 1.5 * 2^-23 |w / d| of the rounded quotient fl(w / d), so both round to the
// same integer (and clamp alike) unless t lies within 2^-13 of a half-integer
// (|t| < 256 there; larger |t| clamps either way).  `near` flags that case;
// the caller then redoes the element with the division.  Valid for d in the
// normal range [2^-120, 2^120], where 1/d is finite and normal.
__device__ __forceinline__ float wq_code_rcp(float w, float rd, bool &near) {
    const float t = w * rd;
    const float r = __builtin_rintf(t);
    // within 2^-13 of a half-integer <=> farther than 1/2 - 2^-13 from the
    // nearest integer; t - r is exact (Sterbenz: r is 0, or within a factor 2 of t)
    near = near || fabsf(t - r) > 0.5f - 0x1p-13f;
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

// (w - d q)^2 in f64; d q is exact in f32 (at most 16 + 7 significant bits)
// and the difference is exact in f64.
__device__ __forceinline__ double wq_sq(float w, float d, float q) {
    const double e = __dsub_rn(static_cast<double>(w), static_cast<double>(d * q));
    return __dmul_rn(e, e);
}

// The f64 held by lane (lane ^ X): DPP inside a 16-lane row, else a permute.
template <int X>
__device__ __forceinline__ double xor_f64(double v) {
    const int lo = __double2loint(v), hi = __double2hiint(v);
    if constexpr (X < 16) return __hiloint2double(lane_xor<X>(hi), lane_xor<X>(lo));
    else return __hiloint2double(__shfl_xor(hi, X), __shfl_xor(lo, X));
}

// Pairwise tree over the lanes of a span of 2^LEVELS lanes (6: a whole wave,
// 5: a half wave).
template <int LEVELS>
__device__ __forceinline__ double tree_sum(double v) {
    v = __dadd_rn(v, xor_f64<1>(v));
    v = __dadd_rn(v, xor_f64<2>(v));
    v = __dadd_rn(v, xor_f64<4>(v));
    v = __dadd_rn(v, xor_f64<8>(v));
    v = __dadd_rn(v, xor_f64<16>(v));
    if constexpr (LEVELS == 6) v = __dadd_rn(v, xor_f64<32>(v));
    return v;
}

// LDS: the rotated row (K floats, plus 128 so that the last span of an odd
// head-group count stays inside), then one amax per 128-block.
inline size_t quant_weight_lds_bytes(int64_t K) { return static_cast<size_t>(K + 128 + K / 128) * 4; }

template <int FMT>
__global__ __launch_bounds__(256) void quant_weight_kernel(const float *__restrict__ W,
                                                           int8_t *__restrict__ codes,
                                                           void *__restrict__ gscale,
                                                           uint16_t *__restrict__ rscale, int K) {
    constexpr int GW = (FMT == kFmtU8) ? 256 : 128;
    constexpr int LEVELS = (FMT == kFmtU8) ? 6 : 5;       // lanes per group = 2^LEVELS
    constexpr int CB = (FMT == kFmtTbl4) ? 2 : 1;         // K elements per code byte
    extern __shared__ __attribute__((aligned(16))) float qw_lds[];
    float *wt = qw_lds;
    float *bamax = qw_lds + K + 128;

    const int n = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int l16 = lane & 15, r4 = lane >> 4;
    const int nblk = K / 128;
    const float *wrow = W + static_cast<int64_t>(n) * K;

    // ---- phase 1: rotate every 128-block into LDS, block amax
    for (int b0 = 0; b0 < nblk; b0 += 16) {
        const int blk = b0 + wid * 4 + r4;
        if (blk < nblk) {
            Blk8 v;
            v.lo = *reinterpret_cast<const float4 *>(wrow + blk * 128 + 4 * l16);
            v.hi = *reinterpret_cast<const float4 *>(wrow + blk * 128 + 64 + 4 * l16);
            fwht128_regs(v, l16);
            *reinterpret_cast<float4 *>(&wt[blk * 128 + 4 * l16]) = v.lo;
            *reinterpret_cast<float4 *>(&wt[blk * 128 + 64 + 4 * l16]) = v.hi;
            float a = fmaxf(amax4(v.lo), amax4(v.hi));
            a = fmaxf(a, lane_xor<1>(a));
            a = fmaxf(a, lane_xor<2>(a));
            a = fmaxf(a, lane_xor<4>(a));
            a = fmaxf(a, lane_xor<8>(a));
            if (l16 == 0) bamax[blk] = a;
        }
    }
    __syncthreads();

    // ---- row scale (u8 format), computed by every wave alike
    float rv = 0.0f;
    if constexpr (FMT == kFmtU8) {
        float a = 0.0f;
        for (int j = lane; j < nblk; j += 64) a = fmaxf(a, bamax[j]);
        const float amax_row = wave_max_f32(a);
        const uint16_t rb = bf16_rne((amax_row / 127.0f) / 255.0f);
        rv = bf16_to_f32(rb);
        if (threadIdx.x == 0) rscale[n] = rb;
    }

    // ---- phase 2: one 256-element span per wave at a time
    const int G = K / GW;
    // head format with an odd group count: the last span holds one group; its
    // upper half-wave reads the 128 spare LDS words past K and stores nothing
    const int nspan = (K + 255) / 256;
    const int half = lane >> 5;                        // head format: which group of the span
    for (int sp = wid; sp < nspan; sp += 4) {
        const float4 w = *reinterpret_cast<const float4 *>(&wt[sp * 256 + 4 * lane]);
        float amax;
        int g;
        if constexpr (FMT == kFmtU8) {
            g = sp;
            amax = fmaxf(bamax[2 * sp], bamax[2 * sp + 1]);
        } else {
            g = 2 * sp + half;
            amax = g < G ? bamax[g] : 0.0f;
        }
        // candidate c's scale (and its reciprocal) is computed once per span
        // by lane c of the group (lanes 0..15; a head span's second group:
        // lanes 32..47, whose amax is that group's) and fetched by every lane
        // of the group in the loop below: the same IEEE operations as
        // evaluating it in every lane, without the per-candidate divisions
        const int cl = lane & 15;
        float d_l;
        uint32_t st_l;
        {
            const float target = (amax * (static_cast<float>(64 - cl) / 64.0f)) / 127.0f;
            if constexpr (FMT == kFmtU8) {
                float u = 1.0f;
                if (rv != 0.0f) u = fminf(fmaxf(__builtin_rintf(target / rv), 1.0f), 255.0f);
                st_l = static_cast<uint32_t>(u);
                d_l = rv * u;
            } else {
                st_l = bf16_rne(target);
                d_l = bf16_to_f32(static_cast<uint16_t>(st_l));
            }
        }
        [[maybe_unused]] const float rd_l = 1.0f / d_l;
        auto fetch = [&](uint32_t v, int c) -> uint32_t {
            if constexpr (FMT == kFmtU8)
                return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), c));
            else
                return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * (32 * half + c), static_cast<int>(v)));
        };
        float best_d = 0.0f;
        uint32_t best_stored = 0;
        double best_err = 0.0;
#pragma unroll 1
        for (int c = 0; c < kWqCandidates; ++c) {
            const float d = __uint_as_float(fetch(__float_as_uint(d_l), c));
            const uint32_t stored = fetch(st_l, c);
            if constexpr (FMT == kFmtTbl4) {
                float v0, v1, v2, v3;
                tbl4_nearest(w.x, d, v0);
                tbl4_nearest(w.y, d, v1);
                tbl4_nearest(w.z, d, v2);
                tbl4_nearest(w.w, d, v3);
                const double s01 = __dadd_rn(wq_sq(w.x, d, v0), wq_sq(w.y, d, v1));
                const double s23 = __dadd_rn(wq_sq(w.z, d, v2), wq_sq(w.w, d, v3));
                const double err = tree_sum<LEVELS>(__dadd_rn(s01, s23));
                if (c == 0 || err < best_err) {
                    best_err = err;
                    best_d = d;
                    best_stored = stored;
                }
                continue;
            }
            // codes: through the reciprocal where that provably rounds alike,
            // else (any lane of the wave near a half-integer, or d outside
            // the normal range) through the division for the whole wave
            bool near = !(d >= 0x1p-120f && d <= 0x1p120f);
            const float rd = __uint_as_float(fetch(__float_as_uint(rd_l), c));
            float q0 = wq_code_rcp(w.x, rd, near);
            float q1 = wq_code_rcp(w.y, rd, near);
            float q2 = wq_code_rcp(w.z, rd, near);
            float q3 = wq_code_rcp(w.w, rd, near);
            if (__any(near)) {
                q0 = wq_code(w.x, d);
                q1 = wq_code(w.y, d);
                q2 = wq_code(w.z, d);
                q3 = wq_code(w.w, d);
            }
            const double s01 = __dadd_rn(wq_sq(w.x, d, q0), wq_sq(w.y, d, q1));
            const double s23 = __dadd_rn(wq_sq(w.z, d, q2), wq_sq(w.w, d, q3));
            const double err = tree_sum<LEVELS>(__dadd_rn(s01, s23));
            if (c == 0 || err < best_err) {
                best_err = err;
                best_d = d;
                best_stored = stored;
            }
        }
        if constexpr (FMT == kFmtTbl4) {
            // lane i holds elements 4i..4i+3 of the span: run i / 8, low
            // nibbles if i % 8 < 4, else high nibbles of the same 4 bytes as
            // lane i - 4; the low lane gathers both and stores the dword
            float v;
            const uint32_t ix = static_cast<uint32_t>(tbl4_nearest(w.x, best_d, v)) |
                                (static_cast<uint32_t>(tbl4_nearest(w.y, best_d, v)) << 8) |
                                (static_cast<uint32_t>(tbl4_nearest(w.z, best_d, v)) << 16) |
                                (static_cast<uint32_t>(tbl4_nearest(w.w, best_d, v)) << 24);
            const uint32_t other = static_cast<uint32_t>(lane_xor<4>(static_cast<int>(ix)));
            if (g < G && (lane & 4) == 0) {
                *reinterpret_cast<uint32_t *>(codes + static_cast<int64_t>(n) * (K / CB) + sp * 128 +
                                              16 * (lane >> 3) + 4 * (lane & 3)) = ix | (other << 4);
                if ((lane & 31) == 0)
                    static_cast<uint16_t *>(gscale)[static_cast<int64_t>(n) * G + g] = static_cast<uint16_t>(best_stored);
            }
            continue;
        }
        const uint32_t b0 = static_cast<uint32_t>(static_cast<int>(wq_code(w.x, best_d))) & 0xFFu;
        const uint32_t b1 = static_cast<uint32_t>(static_cast<int>(wq_code(w.y, best_d))) & 0xFFu;
        const uint32_t b2 = static_cast<uint32_t>(static_cast<int>(wq_code(w.z, best_d))) & 0xFFu;
        const uint32_t b3 = static_cast<uint32_t>(static_cast<int>(wq_code(w.w, best_d))) & 0xFFu;
        if (g < G) {
            *reinterpret_cast<uint32_t *>(codes + static_cast<int64_t>(n) * K + sp * 256 + 4 * lane) =
                b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
            if constexpr (FMT == kFmtU8) {
                if (lane == 0) static_cast<uint8_t *>(gscale)[static_cast<int64_t>(n) * G + g] = static_cast<uint8_t>(best_stored);
            } else {
                if ((lane & 31) == 0)
                    static_cast<uint16_t *>(gscale)[static_cast<int64_t>(n) * G + g] = static_cast<uint16_t>(best_stored);
            }
        }
    }
}

template <int FMT>
hipError_t launch_qw(const float *W, int8_t *codes, void *gscale, uint16_t *rscale, int64_t N,
                     int64_t K, hipStream_t st) {
    const size_t lds = quant_weight_lds_bytes(K);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&quant_weight_kernel<FMT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(quant_weight_kernel<FMT>, dim3(static_cast<uint32_t>(N)), dim3(256), lds, st, W,
                       codes, gscale, rscale, static_cast<int>(K));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_weight(const float *W, int8_t *codes, void *gscale, uint16_t *rscale,
                               int64_t N, int64_t K, int fmt, hipStream_t st) {
    if (fmt == kFmtU8) return launch_qw<0>(W, codes, gscale, rscale, N, K, st);
    if (fmt == kFmtTbl4) return launch_qw<2>(W, codes, gscale, rscale, N, K, st);
    return launch_qw<1>(W, codes, gscale, rscale, N, K, st);
}

}  // namespace rad
