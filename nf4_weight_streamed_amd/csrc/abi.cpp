// C ABI of the NF4-LoRA library: argument validation, error reporting, the NF4
// level table and the enqueue order of each linear's kernels.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/nf4lora.h"
#include "common.h"

namespace nf4 {

namespace {

thread_local std::string g_error;

// Standard normal CDF and its inverse in x87 extended precision (64-bit
// significand): the inverse by bisection on erfcl, which converges to the last
// bit of the format. The levels only need about 1e-9 relative accuracy to round
// to the same float32 values; this is far beyond that.
long double normal_cdf(long double z) { return 0.5L * erfcl(-z / sqrtl(2.0L)); }

long double normal_quantile(long double p) {
    long double lo = -40.0L, hi = 40.0L;
    for (int i = 0; i < 400 && lo < hi; ++i) {
        const long double mid = 0.5L * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (normal_cdf(mid) < p)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5L * (lo + hi);
}

// NF4 = QLoRA's 4-bit NormalFloat (Poros API reference, "PorosTrainer.from_pretrained",
// quantization "nf4"): eight positive quantiles on a probability grid from
// delta down to 1/2 (8 steps), seven negative ones on the same span in 7 steps,
// each divided by the quantile at delta so the extremes are exactly -1 and +1,
// plus an exact 0; delta = ((1 - 1/30) + (1 - 1/32)) / 2.
Tables build_tables() {
    Tables t{};
    const long double delta = 0.5L * ((1.0L - 1.0L / 30.0L) + (1.0L - 1.0L / 32.0L));
    const long double top = normal_quantile(delta);
    long double lv[16];
    int n = 0;
    for (int i = 0; i <= 6; ++i) lv[n++] = -normal_quantile(delta - (delta - 0.5L) * i / 7.0L) / top;
    lv[n++] = 0.0L;
    for (int i = 7; i >= 0; --i) lv[n++] = normal_quantile(delta - (delta - 0.5L) * i / 8.0L) / top;
    for (int j = 0; j < 16; ++j) t.level[j] = static_cast<float>(lv[j]);
    t.level[0] = -1.0f;  // the extremes are exact by construction (q(delta)/q(delta))
    t.level[15] = 1.0f;
    for (int j = 0; j < 15; ++j) {
        // midpoint of two float32 values is exact in double
        const double mid = (double(t.level[j]) + double(t.level[j + 1])) * 0.5;
        float c = static_cast<float>(mid);
        if (double(c) <= mid) c = std::nextafter(c, 2.0f);
        t.thresh[j] = c;
    }
    return t;
}

}  // namespace

const Tables& tables() {
    static const Tables t = build_tables();
    return t;
}

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

namespace {
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;
}  // namespace

void prof_gemm_begin(hipStream_t stream) {
    if (g_prof_start) (void)hipEventRecord(g_prof_start, stream);
}

void prof_gemm_end(hipStream_t stream) {
    if (g_prof_stop) (void)hipEventRecord(g_prof_stop, stream);
    g_prof_start = g_prof_stop = nullptr;
}

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NF4_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return NF4_OK;
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NF4_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return NF4_OK;
}

int check_linear_common(const char* fn, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, int64_t T,
                        int r, float alpha) {
    if (N <= 0 || K <= 0 || T < 0)
        return fail(NF4_E_SHAPE, "%s: need N > 0, K > 0, T >= 0 (got N=%lld K=%lld T=%lld)", fn, (long long)N,
                    (long long)K, (long long)T);
    if (K % NF4_BLOCK != 0)
        return fail(NF4_E_SHAPE, "%s: K=%lld is not a multiple of %d", fn, (long long)K, NF4_BLOCK);
    if (N % 16 != 0) return fail(NF4_E_SHAPE, "%s: N=%lld is not a multiple of 16", fn, (long long)N);
    // The kernels address one weight matrix with 32-bit byte offsets (within 2^30
    // bytes) and every activation or partial through descriptors over at most one
    // 128-row tile; T <= 2^23 keeps the tile counts of the 1-D grids below 2^31.
    if (N > (int64_t(1) << 21) || K > (int64_t(1) << 21) || N * K > (int64_t(1) << 31) || T > (int64_t(1) << 23))
        return fail(NF4_E_SHAPE, "%s: sizes beyond the limits N, K <= 2^21, N*K <= 2^31, T <= 2^23 (N=%lld K=%lld T=%lld)",
                    fn, (long long)N, (long long)K, (long long)T);
    if (r < 0 || r > NF4_MAX_RANK) return fail(NF4_E_ARG, "%s: rank r=%d outside 0..%d", fn, r, NF4_MAX_RANK);
    if (!std::isfinite(alpha)) return fail(NF4_E_ARG, "%s: alpha is not finite", fn);
    if (!codes || !absmax) return fail(NF4_E_ARG, "%s: codes/absmax must not be NULL", fn);
    if (!aligned(codes, 16) || !aligned(absmax, 4))
        return fail(NF4_E_ARG, "%s: codes must be 16-byte and absmax 4-byte aligned", fn);
    return NF4_OK;
}

// The dense-bf16 base [N][K]: the NF4 limits, and N*K <= 2^30 (2 bytes a weight within
// 32-bit offsets).
int check_linear_dense(const char* fn, const uint16_t* w, int64_t N, int64_t K, int64_t T, int r, float alpha) {
    // the shape / rank / alpha checks of the NF4 entry points, with stand-ins for codes and absmax
    static const uint8_t kStandIn[16] __attribute__((aligned(16))) = {};
    int st = check_linear_common(fn, kStandIn, reinterpret_cast<const float*>(kStandIn), N, K, T, r, alpha);
    if (st != NF4_OK) return st;
    if (!w) return fail(NF4_E_ARG, "%s: the bf16 base must not be NULL", fn);
    // 2 bytes a weight in one descriptor, below the out-of-range offset the kernels use
    if (N * K >= (int64_t(1) << 30))
        return fail(NF4_E_SHAPE, "%s: dense base beyond N*K < 2^30 (N=%lld K=%lld)", fn, (long long)N, (long long)K);
    if (!aligned(w, 16)) return fail(NF4_E_ARG, "%s: the bf16 base must be 16-byte aligned", fn);
    return NF4_OK;
}

float lora_scale(float alpha, int r) { return r > 0 ? alpha / float(r) : 0.0f; }

}  // namespace

int check_linear_args(const char* fn, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, int64_t T, int r,
                      float alpha) {
    return check_linear_common(fn, codes, absmax, N, K, T, r, alpha);
}

}  // namespace nf4

using namespace nf4;

extern "C" {

const char* nf4_last_error(void) { return g_error.c_str(); }

int nf4_abi_version(void) { return 1; }

int nf4_probe_mfma(float* out, int workgroups, int iters, nf4_stream stream) {
    if (!out || workgroups < 1 || iters < 1)
        return fail(NF4_E_ARG, "nf4_probe_mfma: need out != NULL, workgroups >= 1, iters >= 1");
    return hip_status(launch_probe_mfma(out, workgroups, iters, static_cast<hipStream_t>(stream)), "nf4_probe_mfma");
}

int nf4_probe_read(const void* src, size_t bytes, uint32_t* out, int workgroups, nf4_stream stream) {
    if (!src || !out || workgroups < 1 || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return fail(NF4_E_ARG, "nf4_probe_read: need src != NULL (16-byte aligned), bytes a positive multiple of 16 "
                               "(got %zu), out != NULL, workgroups >= 1 (got %d)", bytes, workgroups);
    return hip_status(nf4::launch_probe_read(src, uint64_t(bytes), out, workgroups, static_cast<hipStream_t>(stream)),
                      "nf4_probe_read");
}

int nf4_probe_read_depth(const void* src, size_t bytes, uint32_t* out, int workgroups, int depth, int nontemporal,
                         nf4_stream stream) {
    if (!src || !out || workgroups < 1 || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        (depth != 4 && depth != 8 && depth != 16 && depth != 32))
        return fail(NF4_E_ARG, "nf4_probe_read_depth: need src != NULL (16-byte aligned), bytes a positive multiple "
                               "of 16 (got %zu), out != NULL, workgroups >= 1 (got %d), depth 4, 8, 16 or 32 (got %d)",
                    bytes, workgroups, depth);
    return hip_status(nf4::launch_probe_read_depth(src, uint64_t(bytes), out, workgroups, depth, nontemporal != 0,
                                                   static_cast<hipStream_t>(stream)),
                      "nf4_probe_read_depth");
}

int nf4_profile_next_gemm(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(NF4_E_ARG, "nf4_profile_next_gemm: pass both events or neither");
    g_prof_start = static_cast<hipEvent_t>(start_event);
    g_prof_stop = static_cast<hipEvent_t>(stop_event);
    return NF4_OK;
}

int nf4_codebook(float levels_out[16]) {
    if (!levels_out) return fail(NF4_E_ARG, "nf4_codebook: NULL output");
    for (int i = 0; i < 16; ++i) levels_out[i] = tables().level[i];
    return NF4_OK;
}

int nf4_quantize(const void* w, int in_dtype, int64_t rows, int64_t cols, uint8_t* codes, float* absmax,
                 nf4_stream stream) {
    if (in_dtype != NF4_DTYPE_BF16 && in_dtype != NF4_DTYPE_F32)
        return fail(NF4_E_ARG, "nf4_quantize: unknown in_dtype %d", in_dtype);
    if (rows < 0 || cols <= 0 || cols % NF4_BLOCK != 0)
        return fail(NF4_E_SHAPE, "nf4_quantize: need rows >= 0 and cols a positive multiple of %d (got %lld x %lld)",
                    NF4_BLOCK, (long long)rows, (long long)cols);
    if (rows == 0) return NF4_OK;
    if (!w || !codes || !absmax) return fail(NF4_E_ARG, "nf4_quantize: NULL pointer");
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4))
        return fail(NF4_E_ARG, "nf4_quantize: w and codes must be 16-byte aligned, absmax 4-byte");
    return hip_status(launch_quantize(w, in_dtype, rows, cols, codes, absmax, static_cast<hipStream_t>(stream)),
                      "nf4_quantize");
}

int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols, uint16_t* w_bf16,
                   nf4_stream stream) {
    if (rows < 0 || cols <= 0 || cols % NF4_BLOCK != 0)
        return fail(NF4_E_SHAPE, "nf4_dequantize: need rows >= 0 and cols a positive multiple of %d (got %lld x %lld)",
                    NF4_BLOCK, (long long)rows, (long long)cols);
    if (rows == 0) return NF4_OK;
    if (!codes || !absmax || !w_bf16) return fail(NF4_E_ARG, "nf4_dequantize: NULL pointer");
    if (!aligned(codes, 4) || !aligned(w_bf16, 16) || !aligned(absmax, 4))
        return fail(NF4_E_ARG, "nf4_dequantize: codes 4-byte, w 16-byte, absmax 4-byte alignment needed");
    return hip_status(launch_dequantize(codes, absmax, rows, cols, w_bf16, static_cast<hipStream_t>(stream)),
                      "nf4_dequantize");
}

int nf4_merge_lora(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, const uint16_t* A,
                   const uint16_t* B, int r, float alpha, uint16_t* w_out, nf4_stream stream) {
    const char* fn = "nf4_merge_lora";
    if (N <= 0 || K <= 0 || K % NF4_BLOCK != 0)
        return fail(NF4_E_SHAPE, "%s: need N > 0 and K a positive multiple of %d (got N=%lld K=%lld)", fn, NF4_BLOCK,
                    (long long)N, (long long)K);
    if (N > (int64_t(1) << 21) || K > (int64_t(1) << 21) || N * K > (int64_t(1) << 31))
        return fail(NF4_E_SHAPE, "%s: sizes beyond the limits N, K <= 2^21, N*K <= 2^31 (N=%lld K=%lld)", fn,
                    (long long)N, (long long)K);
    if (r < 0 || r > NF4_MAX_RANK) return fail(NF4_E_ARG, "%s: rank r=%d outside 0..%d", fn, r, NF4_MAX_RANK);
    if (!std::isfinite(alpha)) return fail(NF4_E_ARG, "%s: alpha is not finite", fn);
    if (!codes || !absmax || !w_out || (r > 0 && (!A || !B)))
        return fail(NF4_E_ARG, "%s: NULL pointer (codes, absmax, w_out; A and B when r > 0)", fn);
    if (!aligned(codes, 4) || !aligned(absmax, 4) || !aligned(w_out, 16) || (r > 0 && (!aligned(A, 16) || !aligned(B, 2))))
        return fail(NF4_E_ARG, "%s: misaligned pointer (w_out and A need 16 bytes, codes and absmax 4)", fn);
    return hip_status(launch_merge_lora(codes, absmax, N, K, A, B, r, lora_scale(alpha, r), w_out,
                                        static_cast<hipStream_t>(stream)),
                      fn);
}

size_t nf4_lora_linear_fwd_workspace(int64_t T, int64_t N, int64_t K, int r) {
    if (T <= 0 || N <= 0 || K <= 0 || K % NF4_BLOCK != 0 || r < 0 || r > NF4_MAX_RANK) return 0;
    return plan_fwd(T, N, K, r).ws_bytes;
}

size_t nf4_lora_linear_fwd_bf16_workspace(int64_t T, int64_t N, int64_t K, int r) {
    if (T <= 0 || N <= 0 || K <= 0 || K % NF4_BLOCK != 0 || r < 0 || r > NF4_MAX_RANK) return 0;
    return plan_fwd(T, N, K, r, true).ws_bytes;
}

size_t nf4_lora_linear_bwd_workspace(int64_t T, int64_t N, int64_t K, int r) {
    if (T <= 0 || N <= 0 || K <= 0 || K % NF4_BLOCK != 0 || r < 0 || r > NF4_MAX_RANK) return 0;
    return plan_bwd(T, N, K, r).ws_bytes;
}

size_t nf4_lora_linear_bwd_bf16_workspace(int64_t T, int64_t N, int64_t K, int r) {
    if (T <= 0 || N <= 0 || K <= 0 || K % NF4_BLOCK != 0 || r < 0 || r > NF4_MAX_RANK) return 0;
    return plan_bwd(T, N, K, r, true).ws_bytes;
}

}  // extern "C"

namespace nf4 {

// The forward after the base-specific checks; the base is NF4 (codes, absmax) or dense
// bf16 (wdense not NULL).
int linear_fwd(const char* fn, const uint8_t* codes, const float* absmax, const uint16_t* wdense, int64_t N, int64_t K,
               const uint16_t* x, int64_t T, const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* y,
               float* u_save, void* ws, size_t ws_bytes, nf4_stream stream) {
    if (T == 0) return NF4_OK;
    if (!x || !y) return fail(NF4_E_ARG, "%s: x/y must not be NULL", fn);
    if (r > 0 && (!A || !B || !u_save)) return fail(NF4_E_ARG, "%s: r=%d needs A, B and u_save", fn, r);
    if (!aligned(x, 16) || !aligned(y, 16) || (r > 0 && (!aligned(A, 16) || !aligned(B, 2) || !aligned(u_save, 4))))
        return fail(NF4_E_ARG, "%s: misaligned pointer (x, y and A need 16 bytes)", fn);
    const FwdPlan p = plan_fwd(T, N, K, r, wdense != nullptr);
    if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !aligned(ws, 256)))
        return fail(NF4_E_ARG, "%s: workspace of %zu bytes (256-byte aligned) needed for T=%lld N=%lld K=%lld r=%d, got %zu",
                    fn, p.ws_bytes, (long long)T, (long long)N, (long long)K, r, ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = lora_scale(alpha, r);
    if (p.skinny)
        return hip_status(launch_skinny_fwd(p.sk, codes, absmax, x, A, B, T, N, K, r, scale, y, u_save, ws, s),
                          "nf4_lora_linear_fwd (few-token path)");
    if (r > 0) {
        float* upart = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_upart);
        int st = hip_status(launch_lora_down(p, x, A, T, K, r, upart, s), "nf4_lora_linear_fwd (x.A^T)");
        if (st != NF4_OK) return st;
    }
    return hip_status(launch_gemm_fwd(p, codes, absmax, wdense, x, B, T, N, K, r, scale, y, u_save, ws, s),
                      "nf4_lora_linear_fwd (gemm)");
}

namespace {

int linear_bwd(const char* fn, const uint8_t* codes, const float* absmax, const uint16_t* wdense, int64_t N, int64_t K,
               const uint16_t* x, const float* u_save, const uint16_t* dy, int64_t T, const uint16_t* A,
               const uint16_t* B, int r, float alpha, uint16_t* dx, float* dA, float* dB, void* ws, size_t ws_bytes,
               nf4_stream stream) {
    if (T == 0) return NF4_OK;
    if (!dy) return fail(NF4_E_ARG, "%s: dy must not be NULL", fn);
    if (r > 0 && (!x || !u_save || !A || !B || !dA || !dB))
        return fail(NF4_E_ARG, "%s: r=%d needs x, u_save, A, B, dA and dB", fn, r);
    if (!aligned(dy, 16) || (dx && !aligned(dx, 16)) ||
        (r > 0 && (!aligned(x, 16) || !aligned(A, 16) || !aligned(B, 2) || !aligned(u_save, 4) || !aligned(dA, 16) ||
                   !aligned(dB, 4))))
        return fail(NF4_E_ARG, "%s: misaligned pointer (dy, dx, x, A and dA need 16 bytes)", fn);
    const BwdPlan p = plan_bwd(T, N, K, r, wdense != nullptr);
    if (!ws || ws_bytes < p.ws_bytes || !aligned(ws, 256))
        return fail(NF4_E_ARG, "%s: workspace of %zu bytes (256-byte aligned) needed for T=%lld N=%lld K=%lld r=%d, got %zu",
                    fn, p.ws_bytes, (long long)T, (long long)N, (long long)K, r, ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = lora_scale(alpha, r);
    if (r == 0 && !dx) return NF4_OK;
    char* w = static_cast<char*>(ws);
    // few-token path: the g / dB pre-pass runs inside the dX launch
    if (p.skinny)
        return hip_status(launch_skinny_bwd(p.sk, p, codes, absmax, dy, x, A, B, u_save, T, N, K, r, scale, dx, dA, dB,
                                            ws, s),
                          "nf4_lora_linear_bwd (few-token path)");
    if (r > 0) {
        int st = hip_status(launch_lora_bwd_pre(p, dy, B, u_save, T, N, r, scale,
                                                reinterpret_cast<float*>(w + p.off_gpart), dB,
                                                reinterpret_cast<float*>(w + p.off_dbpart), s),
                            "nf4_lora_linear_bwd (g, dB)");
        if (st != NF4_OK) return st;
    }
    // dX (when requested) with its LoRA term, and dA
    return hip_status(launch_gemm_bwd(p, codes, absmax, wdense, dy, x, A, T, N, K, r, scale, dx, dA, dB, ws, s),
                      "nf4_lora_linear_bwd (dX, dA)");
}

}  // namespace
}  // namespace nf4

extern "C" {

int nf4_lora_linear_fwd(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, const uint16_t* x,
                        int64_t T, const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* y,
                        float* u_save, void* ws, size_t ws_bytes, nf4_stream stream) {
    const char* fn = "nf4_lora_linear_fwd";
    const int st = nf4::check_linear_common(fn, codes, absmax, N, K, T, r, alpha);
    if (st != NF4_OK) return st;
    return nf4::linear_fwd(fn, codes, absmax, nullptr, N, K, x, T, A, B, r, alpha, y, u_save, ws, ws_bytes, stream);
}

int nf4_lora_linear_fwd_bf16(const uint16_t* w, int64_t N, int64_t K, const uint16_t* x, int64_t T,
                             const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* y, float* u_save,
                             void* ws, size_t ws_bytes, nf4_stream stream) {
    const char* fn = "nf4_lora_linear_fwd_bf16";
    const int st = nf4::check_linear_dense(fn, w, N, K, T, r, alpha);
    if (st != NF4_OK) return st;
    return nf4::linear_fwd(fn, nullptr, nullptr, w, N, K, x, T, A, B, r, alpha, y, u_save, ws, ws_bytes, stream);
}

int nf4_lora_linear_bwd(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, const uint16_t* x,
                        const float* u_save, const uint16_t* dy, int64_t T, const uint16_t* A, const uint16_t* B,
                        int r, float alpha, uint16_t* dx, float* dA, float* dB, void* ws, size_t ws_bytes,
                        nf4_stream stream) {
    const char* fn = "nf4_lora_linear_bwd";
    const int st = nf4::check_linear_common(fn, codes, absmax, N, K, T, r, alpha);
    if (st != NF4_OK) return st;
    return nf4::linear_bwd(fn, codes, absmax, nullptr, N, K, x, u_save, dy, T, A, B, r, alpha, dx, dA, dB, ws,
                           ws_bytes, stream);
}

int nf4_lora_linear_bwd_bf16(const uint16_t* w, int64_t N, int64_t K, const uint16_t* x, const float* u_save,
                             const uint16_t* dy, int64_t T, const uint16_t* A, const uint16_t* B, int r, float alpha,
                             uint16_t* dx, float* dA, float* dB, void* ws, size_t ws_bytes, nf4_stream stream) {
    const char* fn = "nf4_lora_linear_bwd_bf16";
    const int st = nf4::check_linear_dense(fn, w, N, K, T, r, alpha);
    if (st != NF4_OK) return st;
    return nf4::linear_bwd(fn, nullptr, nullptr, w, N, K, x, u_save, dy, T, A, B, r, alpha, dx, dA, dB, ws, ws_bytes,
                           stream);
}

}  // extern "C"
