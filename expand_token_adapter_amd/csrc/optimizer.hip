// optimizer.hip -- AdamW step on adapter weights (gfx950).
//
// After the gradients of a backward batch have been accumulated into dA / dB,
// the fine-tuning updates the shared adapter weights in place (DeltaServe,
// section 3.2, "Backward subprocess") with AdamW, learning rate 1e-3 and
// weight decay 0.01 (DeltaServe, section 4.1): Adam with decoupled weight
// decay, element by element, with fp32 moments.
//
// One launch updates a list of tensors (typically dA and dB of every trained
// adapter of a layer): the list travels in the kernel arguments, workgroup b
// takes 2048 consecutive elements of the tensor whose range of workgroups
// holds b.  Each lane updates 8 consecutive elements with 16-byte accesses:
// the step is a stream over w (+ master), grad, m, v, bound by HBM.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cmath>

#include "device_common.h"
#include "host_checks.h"
#include "lora_batch.h"

namespace lora {
namespace {

constexpr int kAdamThreads = 256;
constexpr int kAdamElems = kAdamThreads * 8;  // elements per workgroup

struct AdamTensor {
    void* w;
    float* master;
    float* grad;
    float* m;
    float* v;
    int64_t n;
};

struct AdamArgs {
    AdamTensor t[LORA_ADAMW_MAX_TENSORS];
    int64_t first_wg[LORA_ADAMW_MAX_TENSORS + 1];  // workgroup ranges, prefix sums
    int32_t n_tensors;
    float beta1, beta2, one_m_beta1, one_m_beta2;
    float decay;         // 1 - lr * weight_decay
    float step_size;     // lr / (1 - beta1^t)
    float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
    float eps;
    float grad_scale;
    int32_t zero_grad;
};

// Single-element store of the weight (bf16: one round-to-nearest-even).
template <int DT>
struct WElem;
template <>
struct WElem<LORA_BF16> {
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static void put(void* p, int64_t i, float f) {
        static_cast<uint16_t*>(p)[i] = (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
    }
};
template <>
struct WElem<LORA_F32> {
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static void put(void* p, int64_t i, float f) { static_cast<float*>(p)[i] = f; }
};

// One element: moments, bias-corrected step, decoupled decay (fp32).
__device__ __forceinline__ float adam_elem(const AdamArgs& a, float w, float g, float& m, float& v) {
    g *= a.grad_scale;
    m = a.beta1 * m + a.one_m_beta1 * g;
    v = a.beta2 * v + a.one_m_beta2 * (g * g);
    const float denom = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
    return w * a.decay - a.step_size * (m / denom);
}

template <int DT>
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(AdamArgs a) {
    using E = Elem<DT>;
    const int64_t b = blockIdx.x;
    int ti = 0;
    while (ti + 1 < a.n_tensors && b >= a.first_wg[ti + 1]) ++ti;  // uniform
    const AdamTensor t = a.t[ti];
    const int64_t i0 = (b - a.first_wg[ti]) * kAdamElems + 8 * (int64_t)threadIdx.x;
    if (i0 >= t.n) return;
    if (i0 + 8 <= t.n) {
        float w[8], g[8], m[8], v[8];
        if (t.master)
            Elem<LORA_F32>::load8(t.master + i0, w);
        else
            E::load8(static_cast<char*>(t.w) + i0 * WElem<DT>::kBytes, w);
        Elem<LORA_F32>::load8(t.grad + i0, g);
        Elem<LORA_F32>::load8(t.m + i0, m);
        Elem<LORA_F32>::load8(t.v + i0, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = adam_elem(a, w[e], g[e], m[e], v[e]);
        Elem<LORA_F32>::store8(t.m + i0, m);
        Elem<LORA_F32>::store8(t.v + i0, v);
        if (t.master) Elem<LORA_F32>::store8(t.master + i0, w);
        E::store8(static_cast<char*>(t.w) + i0 * WElem<DT>::kBytes, w);
        if (a.zero_grad) {
            const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            Elem<LORA_F32>::store8(t.grad + i0, z);
        }
        return;
    }
    // the tensor's last, partial group of 8
    for (int64_t i = i0; i < t.n; ++i) {
        float m = t.m[i], v = t.v[i];
        const float w0 = t.master ? t.master[i] : E::get(t.w, i);
        const float w = adam_elem(a, w0, t.grad[i], m, v);
        t.m[i] = m;
        t.v[i] = v;
        if (t.master) t.master[i] = w;
        WElem<DT>::put(t.w, i, w);
        if (a.zero_grad) t.grad[i] = 0.f;
    }
}

}  // namespace
}  // namespace lora

using namespace lora;

extern "C" int lora_adamw_step(int dtype, const lora_adamw_tensor* tensors, int32_t n_tensors,
                               lora_adamw_params hp, void* stream) {
    if (!valid_dtype(dtype) || n_tensors < 0 || n_tensors > LORA_ADAMW_MAX_TENSORS) return LORA_ERR_INVALID_ARG;
    if (n_tensors > 0 && !tensors) return LORA_ERR_INVALID_ARG;
    if (!(hp.lr >= 0.f) || !std::isfinite(hp.lr) || !(hp.beta1 >= 0.f && hp.beta1 < 1.f) ||
        !(hp.beta2 >= 0.f && hp.beta2 < 1.f) || !(hp.eps > 0.f) || !std::isfinite(hp.eps) ||
        !(hp.weight_decay >= 0.f) || !std::isfinite(hp.weight_decay) || !std::isfinite(hp.grad_scale) ||
        hp.step < 1)
        return LORA_ERR_INVALID_ARG;
    AdamArgs a{};
    int64_t wg = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        const lora_adamw_tensor& t = tensors[i];
        if (t.n < 0) return LORA_ERR_INVALID_ARG;
        if (t.n > 0 && (!t.w || !t.grad || !t.m || !t.v)) return LORA_ERR_INVALID_ARG;
        if (t.n > 0 && (!aligned16(t.w) || !aligned16(t.grad) || !aligned16(t.m) || !aligned16(t.v) ||
                        (t.master && !aligned16(t.master))))
            return LORA_ERR_INVALID_ARG;
        a.t[i] = AdamTensor{t.w, t.master, t.grad, t.m, t.v, t.n};
        a.first_wg[i] = wg;
        wg += (t.n + kAdamElems - 1) / kAdamElems;
    }
    a.first_wg[n_tensors] = wg;
    if (wg == 0) return LORA_OK;
    if (wg > 0x7fffffff) return LORA_ERR_UNSUPPORTED;
    a.n_tensors = n_tensors;
    // bias corrections in double on the host, once per call
    const double bc1 = 1.0 - std::pow((double)hp.beta1, (double)hp.step);
    const double bc2 = 1.0 - std::pow((double)hp.beta2, (double)hp.step);
    if (!(bc1 > 0.0) || !(bc2 > 0.0)) return LORA_ERR_INVALID_ARG;
    a.beta1 = hp.beta1;
    a.beta2 = hp.beta2;
    a.one_m_beta1 = (float)(1.0 - (double)hp.beta1);
    a.one_m_beta2 = (float)(1.0 - (double)hp.beta2);
    a.decay = (float)(1.0 - (double)hp.lr * (double)hp.weight_decay);
    a.step_size = (float)((double)hp.lr / bc1);
    a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    a.eps = hp.eps;
    a.grad_scale = hp.grad_scale;
    a.zero_grad = hp.zero_grad ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == LORA_BF16)
        hipLaunchKernelGGL((adamw_kernel<LORA_BF16>), dim3((unsigned)wg), dim3(kAdamThreads), 0, st, a);
    else
        hipLaunchKernelGGL((adamw_kernel<LORA_F32>), dim3((unsigned)wg), dim3(kAdamThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}
