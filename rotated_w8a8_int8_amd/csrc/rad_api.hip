// rad_api.hip -- the C ABI of librad.so (declared in include/rad.h).
//
// Every call validates all of its arguments on the host before touching the
// HIP runtime, then enqueues its kernels on the caller's stream.  Check order:
// descriptor present -> format -> shapes -> ranges -> (empty: done) ->
// pointers -> alignment -> aliasing.
#include <stdint.h>

#include <initializer_list>

#include "../../include/rad.h"
#include "rad_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};
// [p, p + bytes), the end clamped to the top of the address space (no real
// buffer wraps; the clamp only keeps the comparison below meaningful).
Span span(const void *p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    const uintptr_t n = static_cast<uintptr_t>(bytes);
    return Span{lo, n > UINTPTR_MAX - lo ? UINTPTR_MAX : lo + n};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

constexpr int64_t kI32Max = 2147483647;
// Group-scale arrays are addressed with 32-bit byte offsets in the kernels.
constexpr int64_t kMaxScaleBytes = int64_t(1) << 31;
static_assert(int64_t(255) * RAD_LINEAR_MAX_K + 128 < (int64_t(1) << 32),
              "a 256-row tile's lane offsets (row * K + chunk) fit 32 bits");

// Product of non-negative sizes, or -1 when it does not fit int64 (no buffer
// is that large, so such sizes are out of range).
int64_t checked_mul(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs)
        if (__builtin_mul_overflow(r, x, &r)) return -1;
    return r;
}
static_assert(RAD_QUANT_WEIGHT_MAX_K == rad::kQuantWeightMaxK, "header and kernel agree on the largest K");
static_assert(RAD_PROBE_BLOCK_BYTES == rad::kProbeBlockBytes, "header and kernel agree on a probe block");

int group_width(int32_t fmt) {
    if (fmt == RAD_FMT_U8G256_BF16ROW) return 256;
    if (fmt == RAD_FMT_BF16G128 || fmt == RAD_FMT_TBL4_BF16G128) return 128;
    return 0;
}
// bytes of weight codes per row
int64_t code_bytes(int32_t fmt, int64_t K) { return fmt == RAD_FMT_TBL4_BF16G128 ? K / 2 : K; }

int hip_status(hipError_t e) { return e == hipSuccess ? RAD_OK : RAD_E_HIP; }

// Shared validation of the two contraction entry points.
int check_linear(const int8_t *q, const float *scale, const rad_w8a8_weight *w, const float *y,
                 int64_t M, const int32_t *partials, int64_t max_m) {
    if (!w) return RAD_E_NULL;
    const int gw = group_width(w->fmt);
    if (gw == 0) return RAD_E_FMT;
    if (w->fmt == RAD_FMT_U8G256_BF16ROW && !w->rscale) return RAD_E_FMT;
    if (w->fmt != RAD_FMT_U8G256_BF16ROW && w->rscale) return RAD_E_FMT;
    if (M < 0 || w->N < 0 || w->K <= 0 || w->K % 128 != 0 || w->K % gw != 0) return RAD_E_SHAPE;
    if (M > max_m || w->N > kI32Max || w->K > RAD_LINEAR_MAX_K) return RAD_E_RANGE;
    const int64_t N = w->N, K = w->K, G = K / gw;
    const int esz = (w->fmt == RAD_FMT_U8G256_BF16ROW) ? 1 : 2;
    const int64_t qb = checked_mul({M, K}), yb = checked_mul({M, N, 4}), gb = checked_mul({N, G, esz}),
                  pb = partials ? checked_mul({M, N, G, 4}) : 0;
    if (qb < 0 || yb < 0 || gb < 0 || pb < 0 || gb >= kMaxScaleBytes) return RAD_E_RANGE;
    if (M > RAD_GEMV_MAX_M && !rad::gemm_grid_fits(M, N)) return RAD_E_RANGE;
    if (M == 0 || w->N == 0) return 1;  // nothing to do
    if (!q || !scale || !y || !w->codes || !w->gscale) return RAD_E_NULL;
    if (!aligned(q, 16) || !aligned(w->codes, 16) || !aligned(w->gscale, 4) ||
        (w->rscale && !aligned(w->rscale, 4)) || !aligned(scale, 4) || !aligned(y, 4) ||
        (partials && !aligned(partials, 4)))
        return RAD_E_ALIGN;
    const Span in[] = {span(q, qb), span(scale, M * 4), span(w->codes, N * code_bytes(w->fmt, K)),
                       span(w->gscale, gb),
                       w->rscale ? span(w->rscale, N * 2) : Span{0, 0}};
    const Span ys = span(y, yb);
    const Span ps = partials ? span(partials, pb) : Span{0, 0};
    for (const Span &s : in) {
        if (overlap(ys, s)) return RAD_E_ALIAS;
        if (partials && overlap(ps, s)) return RAD_E_ALIAS;
    }
    if (partials && overlap(ys, ps)) return RAD_E_ALIAS;
    return RAD_OK;
}

rad::WeightArgs weight_args(const rad_w8a8_weight *w) {
    return rad::WeightArgs{w->codes, w->gscale, w->rscale, w->N, w->K, static_cast<int>(w->fmt)};
}

}  // namespace

// 2..128 tokens: the LDS-staged kernel where it applies, else the
// register-streaming one.
static hipError_t launch_small(const int8_t *q, const float *s, const rad::WeightArgs &w, float *y,
                               int64_t M, int32_t *P, hipStream_t st) {
    if (rad::skinny_lds_supported(w, M)) return rad::launch_skinny_lds(q, s, w, y, M, P, st);
    return rad::launch_gemv(q, s, w, y, M, P, st);
}

extern "C" {

int rad_fwht128(const float *x, float *y, int64_t rows, int64_t K, rad_stream_t stream) {
    if (rows < 0 || K <= 0 || K % 128 != 0) return RAD_E_SHAPE;
    if (rows > 0 && K > INT64_MAX / 4 / rows) return RAD_E_RANGE;
    if (rows == 0) return RAD_OK;
    if (!x || !y) return RAD_E_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return RAD_E_ALIGN;
    if (x != y && overlap(span(x, rows * K * 4), span(y, rows * K * 4))) return RAD_E_ALIAS;
    return hip_status(rad::launch_fwht128(x, y, rows, K, static_cast<hipStream_t>(stream)));
}

int rad_quant_act_i8(const float *x, int8_t *q, float *scale, int64_t M, int64_t K, int rotate,
                     rad_stream_t stream) {
    if (M < 0 || K <= 0 || K % 128 != 0) return RAD_E_SHAPE;
    if (K > RAD_QUANT_MAX_K || M > kI32Max || (rotate != 0 && rotate != 1)) return RAD_E_RANGE;
    if (M == 0) return RAD_OK;
    if (!x || !q || !scale) return RAD_E_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return RAD_E_ALIGN;
    const Span xs = span(x, M * K * 4), qs = span(q, M * K), ss = span(scale, M * 4);
    if (overlap(xs, qs) || overlap(xs, ss) || overlap(qs, ss)) return RAD_E_ALIAS;
    return hip_status(rad::launch_quant_act(x, q, scale, M, K, rotate, static_cast<hipStream_t>(stream)));
}

int rad_w8a8_gemv(const int8_t *q, const float *scale, const rad_w8a8_weight *w, float *y,
                  int64_t M, int32_t *partials, rad_stream_t stream) {
    const int rc = check_linear(q, scale, w, y, M, partials, RAD_GEMV_MAX_M);
    if (rc != RAD_OK) return rc > 0 ? RAD_OK : rc;
    return hip_status(launch_small(q, scale, weight_args(w), y, M, partials,
                                   static_cast<hipStream_t>(stream)));
}

int rad_w8a8_gemm(const int8_t *q, const float *scale, const rad_w8a8_weight *w, float *y,
                  int64_t M, int32_t *partials, rad_stream_t stream) {
    const int rc = check_linear(q, scale, w, y, M, partials, kI32Max);
    if (rc != RAD_OK) return rc > 0 ? RAD_OK : rc;
    return hip_status(rad::launch_gemm(q, scale, weight_args(w), y, M, partials,
                                       static_cast<hipStream_t>(stream)));
}

int rad_w8a8_linear(const float *x, int8_t *q, float *scale, const rad_w8a8_weight *w, float *y,
                    int64_t M, rad_stream_t stream) {
    int rc = check_linear(q, scale, w, y, M, nullptr, kI32Max);
    if (rc < 0) return rc;
    if (w->K > RAD_QUANT_MAX_K) return RAD_E_RANGE;
    if (rc > 0) return RAD_OK;                       // empty
    if (!x) return RAD_E_NULL;
    if (!aligned(x, 16)) return RAD_E_ALIGN;
    const int64_t N = w->N, K = w->K;
    const int gw = group_width(w->fmt);
    const int esz = (w->fmt == RAD_FMT_U8G256_BF16ROW) ? 1 : 2;
    const Span xs = span(x, M * K * 4), qs = span(q, M * K), ss = span(scale, M * 4),
               ys = span(y, M * N * 4);
    const Span ws[] = {span(w->codes, N * code_bytes(w->fmt, K)), span(w->gscale, N * (K / gw) * esz),
                       w->rscale ? span(w->rscale, N * 2) : Span{0, 0}};
    if (overlap(xs, qs) || overlap(xs, ss) || overlap(qs, ss) || overlap(xs, ys)) return RAD_E_ALIAS;
    for (const Span &o : ws)
        if (overlap(qs, o) || overlap(ss, o)) return RAD_E_ALIAS;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const rad::WeightArgs wa = weight_args(w);
    if (rad::fused_decode_supported(wa, M)) return hip_status(rad::launch_fused_decode(x, q, scale, wa, y, st));
    hipError_t e = rad::launch_quant_act(x, q, scale, M, K, 1, st);
    if (e != hipSuccess) return RAD_E_HIP;
    e = (M <= RAD_GEMV_MAX_M) ? launch_small(q, scale, wa, y, M, nullptr, st)
                              : rad::launch_gemm(q, scale, wa, y, M, nullptr, st);
    return hip_status(e);
}

int rad_quant_weight_i8(const float *W, int8_t *codes, void *gscale, uint16_t *rscale, int64_t N,
                        int64_t K, int32_t fmt, rad_stream_t stream) {
    const int gw = group_width(fmt);
    if (gw == 0) return RAD_E_FMT;
    if (fmt == RAD_FMT_U8G256_BF16ROW && !rscale) return RAD_E_FMT;
    if (fmt != RAD_FMT_U8G256_BF16ROW && rscale) return RAD_E_FMT;
    if (N < 0 || K <= 0 || K % 128 != 0 || K % gw != 0) return RAD_E_SHAPE;
    if (K > RAD_QUANT_WEIGHT_MAX_K || N > kI32Max) return RAD_E_RANGE;
    if (N == 0) return RAD_OK;
    if (!W || !codes || !gscale) return RAD_E_NULL;
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(gscale, 4) || (rscale && !aligned(rscale, 4)))
        return RAD_E_ALIGN;
    const int esz = (fmt == RAD_FMT_U8G256_BF16ROW) ? 1 : 2;
    const Span ws = span(W, N * K * 4), cs = span(codes, N * code_bytes(fmt, K)),
               gs = span(gscale, N * (K / gw) * esz),
               rs = rscale ? span(rscale, N * 2) : Span{0, 0};
    if (overlap(ws, cs) || overlap(ws, gs) || overlap(ws, rs) || overlap(cs, gs) || overlap(cs, rs) ||
        overlap(gs, rs))
        return RAD_E_ALIAS;
    return hip_status(rad::launch_quant_weight(W, codes, gscale, rscale, N, K, fmt,
                                               static_cast<hipStream_t>(stream)));
}

int rad_w8a8_rescore(const int8_t *q, const float *scale, const rad_w8a8_weight *w, const int32_t *ids,
                     int64_t C, float *y, int64_t M, rad_stream_t stream) {
    if (!w) return RAD_E_NULL;
    const int gw = group_width(w->fmt);
    if (gw == 0) return RAD_E_FMT;
    if (w->fmt == RAD_FMT_U8G256_BF16ROW && !w->rscale) return RAD_E_FMT;
    if (w->fmt != RAD_FMT_U8G256_BF16ROW && w->rscale) return RAD_E_FMT;
    if (w->fmt == RAD_FMT_TBL4_BF16G128) return RAD_E_FMT;       // int8 weights only
    if (M < 0 || C < 0 || w->N < 0 || w->K <= 0 || w->K % 128 != 0 || w->K % gw != 0) return RAD_E_SHAPE;
    if (w->N > kI32Max || w->K > RAD_LINEAR_MAX_K || C > kI32Max || M > kI32Max ||
        M * C >= (int64_t(1) << 33))
        return RAD_E_RANGE;
    if (checked_mul({w->N, w->K / gw, 2}) >= kMaxScaleBytes) return RAD_E_RANGE;
    if (M == 0 || C == 0) return RAD_OK;
    if (!q || !scale || !ids || !y || !w->codes || !w->gscale) return RAD_E_NULL;
    if (!aligned(q, 16) || !aligned(w->codes, 16) || !aligned(w->gscale, 4) ||
        (w->rscale && !aligned(w->rscale, 4)) || !aligned(scale, 4) || !aligned(ids, 4) || !aligned(y, 4))
        return RAD_E_ALIGN;
    const int64_t N = w->N, K = w->K, G = K / gw;
    const int esz = (w->fmt == RAD_FMT_U8G256_BF16ROW) ? 1 : 2;
    const Span in[] = {span(q, M * K), span(scale, M * 4), span(w->codes, N * K),
                       span(w->gscale, N * G * esz), w->rscale ? span(w->rscale, N * 2) : Span{0, 0},
                       span(ids, M * C * 4)};
    const Span ys = span(y, M * C * 4);
    for (const Span &sp : in)
        if (overlap(ys, sp)) return RAD_E_ALIAS;
    return hip_status(rad::launch_rescore(q, scale, weight_args(w), ids, C, y, M,
                                          static_cast<hipStream_t>(stream)));
}

namespace {
int check_kv(const void *x, const void *codes, const void *scale, int64_t rows, int64_t D) {
    if (rows < 0 || (D != 64 && D != 128 && D != 256)) return RAD_E_SHAPE;
    if (rows > INT64_MAX / 2 / D) return RAD_E_RANGE;
    if (rows == 0) return 1;
    if (!x || !codes || !scale) return RAD_E_NULL;
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scale, 2)) return RAD_E_ALIGN;
    const Span xs = span(x, rows * D * 2), cs = span(codes, rows * D), ss = span(scale, rows * 2);
    if (overlap(xs, cs) || overlap(xs, ss) || overlap(cs, ss)) return RAD_E_ALIAS;
    return RAD_OK;
}
}  // namespace

int rad_kv_quant_i8(const uint16_t *x, int8_t *codes, uint16_t *scale, int64_t rows, int64_t D,
                    rad_stream_t stream) {
    const int rc = check_kv(x, codes, scale, rows, D);
    if (rc != RAD_OK) return rc > 0 ? RAD_OK : rc;
    return hip_status(rad::launch_kv_quant(x, codes, scale, rows, D, static_cast<hipStream_t>(stream)));
}

int rad_kv_dequant_i8(const int8_t *codes, const uint16_t *scale, uint16_t *y, int64_t rows, int64_t D,
                      rad_stream_t stream) {
    const int rc = check_kv(y, codes, scale, rows, D);
    if (rc != RAD_OK) return rc > 0 ? RAD_OK : rc;
    return hip_status(rad::launch_kv_dequant(codes, scale, y, rows, D, static_cast<hipStream_t>(stream)));
}

int rad_probe_mfma_i8(const int8_t *src, int32_t *out, int64_t blocks, int64_t ksteps, int lds_fed,
                      rad_stream_t stream) {
    if (blocks < 0 || ksteps < 0 || ksteps % 2 != 0) return RAD_E_SHAPE;
    if (blocks > RAD_PROBE_MAX_BLOCKS || ksteps > RAD_PROBE_MAX_KSTEPS || (lds_fed != 0 && lds_fed != 1))
        return RAD_E_RANGE;
    if (blocks == 0 || ksteps == 0) return RAD_OK;
    if (!src || !out) return RAD_E_NULL;
    if (!aligned(src, 16) || !aligned(out, 4)) return RAD_E_ALIGN;
    if (overlap(span(src, blocks * rad::kProbeBlockBytes), span(out, blocks * 512 * 4))) return RAD_E_ALIAS;
    return hip_status(rad::launch_mfma_probe(src, out, blocks, ksteps, lds_fed == 1,
                                             static_cast<hipStream_t>(stream)));
}

const char *rad_strerror(int status) {
    switch (status) {
        case RAD_OK: return "success";
        case RAD_E_NULL: return "a required pointer is NULL";
        case RAD_E_SHAPE: return "invalid shape (negative size, or K not a multiple of 128 / the group width)";
        case RAD_E_ALIGN: return "a pointer is not aligned as required";
        case RAD_E_FMT: return "unknown weight format or wrong scale pointers for the format";
        case RAD_E_RANGE: return "a size or flag is beyond what the call supports";
        case RAD_E_ALIAS: return "an output overlaps another argument";
        case RAD_E_HIP: return "the HIP runtime reported an error";
        default: return "unknown status";
    }
}

}  // extern "C"
