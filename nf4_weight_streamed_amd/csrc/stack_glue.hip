// Glue kernels of the identity-mixing decoder stack that the streamed NF4 base
// feeds: unit-gain RMSNorm, repeat_kv, SiLU-gated product and residual adds,
// forward and backward. Activations are stored in bf16 (the model dtype of the
// Poros API reference, "PorosModel.from_pretrained", torch_dtype bfloat16); all
// arithmetic is fp32; reductions have a fixed order.
#include "../../include/nf4lora.h"
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;

// Sum over the 256 threads of a workgroup in a fixed order: wave-internal xor
// butterflies (same pattern on every call) then the four wave sums in order.
__device__ __forceinline__ float block_sum(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    const float s = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return s;
}

// One row per workgroup: out = RNbf(h * rstd), rstd = 1 / sqrt(mean(h^2) + eps).
__global__ __launch_bounds__(kThreads) void k_rmsnorm_fwd(const uint16_t* __restrict__ h, int H, float eps,
                                                          uint16_t* __restrict__ out, float* __restrict__ rstd) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    const uint16_t* hr = h + row * H;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < H; i += kThreads) {
        const float v = bf16_to_f32(hr[i]);
        ss += v * v;
    }
    ss = block_sum(ss, red);
    const float rs = 1.0f / sqrtf(ss / float(H) + eps);
    for (int i = threadIdx.x; i < H; i += kThreads) out[row * H + i] = bf16_bits(bf16_to_f32(hr[i]) * rs);
    if (threadIdx.x == 0 && rstd) rstd[row] = rs;
}

// dh = RNbf( dres + rstd*dy - rstd^3 * h * mean(dy*h) ), dres optional.
__global__ __launch_bounds__(kThreads) void k_rmsnorm_bwd(const uint16_t* __restrict__ h,
                                                          const float* __restrict__ rstd,
                                                          const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ dres, int H,
                                                          uint16_t* __restrict__ dh) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    const size_t base = row * H;
    float dot = 0.0f;
    for (int i = threadIdx.x; i < H; i += kThreads) dot += bf16_to_f32(dy[base + i]) * bf16_to_f32(h[base + i]);
    dot = block_sum(dot, red);
    const float rs = rstd[row];
    const float c = rs * rs * rs * (dot / float(H));
    for (int i = threadIdx.x; i < H; i += kThreads) {
        float v = rs * bf16_to_f32(dy[base + i]) - c * bf16_to_f32(h[base + i]);
        if (dres) v = bf16_to_f32(dres[base + i]) + v;
        dh[base + i] = bf16_bits(v);
    }
}

// out = RNbf(a + b (+ c)), elementwise.
__global__ __launch_bounds__(kThreads) void k_add(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                  const uint16_t* __restrict__ c, int64_t n,
                                                  uint16_t* __restrict__ out) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= n) return;
    float v = bf16_to_f32(a[i]) + bf16_to_f32(b[i]);
    if (c) v += bf16_to_f32(c[i]);
    out[i] = bf16_bits(v);
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

// m = RNbf(SiLU(gate) * up)
__global__ __launch_bounds__(kThreads) void k_silu_mul_fwd(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up, int64_t n,
                                                           uint16_t* __restrict__ m) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= n) return;
    const float z = bf16_to_f32(gate[i]);
    m[i] = bf16_bits(z * sigmoid(z) * bf16_to_f32(up[i]));
}

// dgate = RNbf(dm * up * SiLU'(gate)), dup = RNbf(dm * SiLU(gate))
__global__ __launch_bounds__(kThreads) void k_silu_mul_bwd(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up,
                                                           const uint16_t* __restrict__ dm, int64_t n,
                                                           uint16_t* __restrict__ dgate, uint16_t* __restrict__ dup) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= n) return;
    const float z = bf16_to_f32(gate[i]);
    const float sg = sigmoid(z);
    const float d = bf16_to_f32(dm[i]);
    dgate[i] = bf16_bits(d * bf16_to_f32(up[i]) * (sg * (1.0f + z * (1.0f - sg))));
    dup[i] = bf16_bits(d * (z * sg));
}

// a[t][qh*hd + e] = v[t][(qh / rep)*hd + e], rep = q / kv
__global__ __launch_bounds__(kThreads) void k_repeat_kv_fwd(const uint16_t* __restrict__ v, int64_t T, int q, int kv,
                                                            int hd, uint16_t* __restrict__ a) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= T * q) return;
    const int64_t t = i / q;
    const int c = int(i % q);
    const int rep = q / kv;
    a[i] = v[t * kv + (c / hd / rep) * hd + c % hd];
}

// dv[t][kh*hd + e] = RNbf(sum over the rep query heads of kv head kh, in head order)
__global__ __launch_bounds__(kThreads) void k_repeat_kv_bwd(const uint16_t* __restrict__ da, int64_t T, int q, int kv,
                                                            int hd, uint16_t* __restrict__ dv) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= T * kv) return;
    const int64_t t = i / kv;
    const int c = int(i % kv);
    const int rep = q / kv;
    const int kh = c / hd, e = c % hd;
    float s = 0.0f;
    for (int j = 0; j < rep; ++j) s += bf16_to_f32(da[t * q + (kh * rep + j) * hd + e]);
    dv[i] = bf16_bits(s);
}

inline unsigned grid_of(int64_t n) { return unsigned(cdiv(n, kThreads)); }

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NF4_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return NF4_OK;
}

bool bad_ptr(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 1) != 0; }

}  // namespace

}  // namespace nf4

using namespace nf4;

extern "C" {

int nf4_rmsnorm_fwd(const uint16_t* h, int64_t T, int64_t H, float eps, uint16_t* out, float* rstd,
                    nf4_stream stream) {
    if (T < 0 || H <= 0 || H > (int64_t(1) << 30)) return fail(NF4_E_SHAPE, "nf4_rmsnorm_fwd: bad T=%lld H=%lld", (long long)T, (long long)H);
    if (T == 0) return NF4_OK;
    if (bad_ptr(h) || bad_ptr(out)) return fail(NF4_E_ARG, "nf4_rmsnorm_fwd: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_rmsnorm_fwd, dim3(unsigned(T)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), h, int(H),
                       eps, out, rstd);
    return hip_status(hipGetLastError(), "nf4_rmsnorm_fwd");
}

int nf4_rmsnorm_bwd(const uint16_t* h, const float* rstd, const uint16_t* dy, const uint16_t* dres, int64_t T,
                    int64_t H, uint16_t* dh, nf4_stream stream) {
    if (T < 0 || H <= 0 || H > (int64_t(1) << 30)) return fail(NF4_E_SHAPE, "nf4_rmsnorm_bwd: bad T=%lld H=%lld", (long long)T, (long long)H);
    if (T == 0) return NF4_OK;
    if (bad_ptr(h) || !rstd || bad_ptr(dy) || bad_ptr(dh)) return fail(NF4_E_ARG, "nf4_rmsnorm_bwd: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(unsigned(T)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), h, rstd,
                       dy, dres, int(H), dh);
    return hip_status(hipGetLastError(), "nf4_rmsnorm_bwd");
}

int nf4_add_bf16(const uint16_t* a, const uint16_t* b, const uint16_t* c, int64_t n, uint16_t* out, nf4_stream stream) {
    if (n < 0) return fail(NF4_E_SHAPE, "nf4_add_bf16: n=%lld", (long long)n);
    if (n == 0) return NF4_OK;
    if (bad_ptr(a) || bad_ptr(b) || bad_ptr(out)) return fail(NF4_E_ARG, "nf4_add_bf16: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_add, dim3(grid_of(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a, b, c, n, out);
    return hip_status(hipGetLastError(), "nf4_add_bf16");
}

int nf4_silu_mul_fwd(const uint16_t* gate, const uint16_t* up, int64_t n, uint16_t* m, nf4_stream stream) {
    if (n < 0) return fail(NF4_E_SHAPE, "nf4_silu_mul_fwd: n=%lld", (long long)n);
    if (n == 0) return NF4_OK;
    if (bad_ptr(gate) || bad_ptr(up) || bad_ptr(m)) return fail(NF4_E_ARG, "nf4_silu_mul_fwd: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_silu_mul_fwd, dim3(grid_of(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), gate, up,
                       n, m);
    return hip_status(hipGetLastError(), "nf4_silu_mul_fwd");
}

int nf4_silu_mul_bwd(const uint16_t* gate, const uint16_t* up, const uint16_t* dm, int64_t n, uint16_t* dgate,
                     uint16_t* dup, nf4_stream stream) {
    if (n < 0) return fail(NF4_E_SHAPE, "nf4_silu_mul_bwd: n=%lld", (long long)n);
    if (n == 0) return NF4_OK;
    if (bad_ptr(gate) || bad_ptr(up) || bad_ptr(dm) || bad_ptr(dgate) || bad_ptr(dup))
        return fail(NF4_E_ARG, "nf4_silu_mul_bwd: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_silu_mul_bwd, dim3(grid_of(n)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), gate, up,
                       dm, n, dgate, dup);
    return hip_status(hipGetLastError(), "nf4_silu_mul_bwd");
}

int nf4_repeat_kv_fwd(const uint16_t* v, int64_t T, int64_t q, int64_t kv, int64_t head_dim, uint16_t* a,
                      nf4_stream stream) {
    if (T < 0 || head_dim <= 0 || kv <= 0 || q <= 0 || kv % head_dim || q % kv || q > (int64_t(1) << 24))
        return fail(NF4_E_SHAPE, "nf4_repeat_kv_fwd: need head_dim | kv | q (got q=%lld kv=%lld head_dim=%lld)",
                    (long long)q, (long long)kv, (long long)head_dim);
    if (T == 0) return NF4_OK;
    if (bad_ptr(v) || bad_ptr(a)) return fail(NF4_E_ARG, "nf4_repeat_kv_fwd: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_repeat_kv_fwd, dim3(grid_of(T * q)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), v, T,
                       int(q), int(kv), int(head_dim), a);
    return hip_status(hipGetLastError(), "nf4_repeat_kv_fwd");
}

int nf4_repeat_kv_bwd(const uint16_t* da, int64_t T, int64_t q, int64_t kv, int64_t head_dim, uint16_t* dv,
                      nf4_stream stream) {
    if (T < 0 || head_dim <= 0 || kv <= 0 || q <= 0 || kv % head_dim || q % kv || q > (int64_t(1) << 24))
        return fail(NF4_E_SHAPE, "nf4_repeat_kv_bwd: need head_dim | kv | q (got q=%lld kv=%lld head_dim=%lld)",
                    (long long)q, (long long)kv, (long long)head_dim);
    if (T == 0) return NF4_OK;
    if (bad_ptr(da) || bad_ptr(dv)) return fail(NF4_E_ARG, "nf4_repeat_kv_bwd: NULL or misaligned pointer");
    hipLaunchKernelGGL(k_repeat_kv_bwd, dim3(grid_of(T * kv)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), da,
                       T, int(q), int(kv), int(head_dim), dv);
    return hip_status(hipGetLastError(), "nf4_repeat_kv_bwd");
}

}  // extern "C"
