// C <- beta * C for the calls where the product term vanishes (K == 0 or
// alpha == 0). beta == 0 stores zeros without reading C, so NaN or garbage in
// C does not survive (the BLAS convention for beta == 0). With a bias or an
// activation the same calls store act(bias[col]) + beta * C.

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

// One workgroup per row block; threads stride along the row.
template <typename T, bool EPI>
__global__ __launch_bounds__(256) void scale_kernel(int64_t M, int64_t N, float beta, T* C,
                                                    int64_t ldc, const T* bias, int act) {
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        T* r = C + row * ldc;
        for (int64_t j = threadIdx.x; j < N; j += blockDim.x) {
            float v = beta == 0.f ? 0.f : beta * to_f32<T>(r[j]);
            if constexpr (EPI) {
                const float e = activate(bias != nullptr ? to_f32<T>(bias[j]) : 0.f, act);
                v = beta == 0.f ? e : e + v;
            }
            r[j] = from_f32<T>(v);
        }
    }
}

template <typename T>
hipError_t launch(int64_t M, int64_t N, float beta, T* C, int64_t ldc, const T* bias, int act,
                  hipStream_t s) {
    const unsigned blocks = (unsigned)(M < 65536 ? M : 65536);
    void* kargs[] = {&M, &N, &beta, &C, &ldc, &bias, &act};
    const bool epi = bias != nullptr || act != kActNone;
    const void* fn = epi ? (const void*)&scale_kernel<T, true> : (const void*)&scale_kernel<T, false>;
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), kargs, 0, s);
}

}  // namespace

hipError_t launch_scale_f32(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                            const float* bias, int act, hipStream_t s) {
    return launch<float>(M, N, beta, C, ldc, bias, act, s);
}

hipError_t launch_scale_bf16(int64_t M, int64_t N, float beta, uint16_t* C, int64_t ldc,
                             const uint16_t* bias, int act, hipStream_t s) {
    return launch<uint16_t>(M, N, beta, C, ldc, bias, act, s);
}

}  // namespace dg
