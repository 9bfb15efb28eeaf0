// rad_launch.h -- host-side launchers of the librad kernels.  Arguments are
// already validated by rad_api.cpp; each launcher enqueues on `st` and returns
// the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rad {

struct WeightArgs {
    const int8_t *codes;     // int8 [N][K], or packed 4-bit indices [N][K/2] (fmt 2)
    const void *gscale;      // u8 [N][K/256] or bf16 bits [N][K/128]
    const uint16_t *rscale;  // bf16 bits [N] (u8 format) or nullptr
    int64_t N, K;
    int fmt;                 // 0: u8 per 256 + bf16 row; 1: bf16 per 128; 2: codebook, bf16 per 128
};

// Compute units of the current device (looked up once per device), or 0.
int cu_count();

hipError_t launch_fwht128(const float *x, float *y, int64_t rows, int64_t K, hipStream_t st);
hipError_t launch_quant_act(const float *x, int8_t *q, float *s, int64_t M, int64_t K, int rotate,
                            hipStream_t st);
hipError_t launch_gemv(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st);
// 33..64 or 112..128 tokens in the int8 formats (head: an even number of
// groups), 9..16 tokens in the codebook format, enough weight rows to fill
// the rounds of workgroups: both operands staged through LDS.
bool skinny_lds_supported(const WeightArgs &w, int64_t M);
hipError_t launch_skinny_lds(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                             int32_t *partials, hipStream_t st);
// One token, K a multiple of 1024: the u8 format up to K = 20480 and the head
// format up to K = 16384 (weight rows streamed whole, 1 KiB per load), the
// codebook format up to K = 8192 (two rows per load, 512 bytes each);
// optionally fused with the rotation and quantisation of the token.
bool decode_row_supported(const WeightArgs &w);
hipError_t launch_decode_row(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y,
                             int32_t *partials, bool fused, hipStream_t st);
// Whole layer for one token in one kernel (rotate + quantise + contract).
bool fused_decode_supported(const WeightArgs &w, int64_t M);
hipError_t launch_fused_decode(const float *x, int8_t *q, float *s, const WeightArgs &w, float *y,
                               hipStream_t st);
// Weight-side quantiser; K <= kQuantWeightMaxK.
constexpr int kQuantWeightMaxK = 32768;
hipError_t launch_quant_weight(const float *W, int8_t *codes, void *gscale, uint16_t *rscale,
                               int64_t N, int64_t K, int fmt, hipStream_t st);
// The layer at candidate rows ids [M][C] only.
hipError_t launch_rescore(const int8_t *q, const float *s, const WeightArgs &w, const int32_t *ids,
                          int64_t C, float *y, int64_t M, hipStream_t st);
// int8 KV-cache codec; D is 64, 128 or 256.
hipError_t launch_kv_quant(const uint16_t *x, int8_t *codes, uint16_t *scale, int64_t rows, int64_t D,
                           hipStream_t st);
hipError_t launch_kv_dequant(const int8_t *codes, const uint16_t *scale, uint16_t *y, int64_t rows,
                             int64_t D, hipStream_t st);
hipError_t launch_gemm(const int8_t *q, const float *s, const WeightArgs &w, float *y, int64_t M,
                       int32_t *partials, hipStream_t st);
// Whether launch_gemm's grid (one workgroup per output tile) fits a launch.
bool gemm_grid_fits(int64_t M, int64_t N);
// Measurement aid: back-to-back int8 matrix ops, one 8-wave workgroup per
// block, each block reading its own kProbeBlockBytes of operand bytes; every
// lane writes one 32-bit word (blocks * 512 words in all).
constexpr int kProbeBlockBytes = 96 * 1024;
hipError_t launch_mfma_probe(const int8_t *src, int32_t *out, int64_t blocks, int64_t ksteps, bool lds_fed,
                             hipStream_t st);

}  // namespace rad
