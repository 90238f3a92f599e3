// C <- beta * C for the calls where the product term vanishes (K == 0 or
// alpha == 0). beta == 0 stores zeros without reading C, so NaN or garbage in
// C does not survive (the BLAS convention for beta == 0).

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
template <typename T>
__global__ __launch_bounds__(256) void scale_kernel(int64_t M, int64_t N, float beta, T* C,
                                                    int64_t ldc) {
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        T* r = C + row * ldc;
        for (int64_t j = threadIdx.x; j < N; j += blockDim.x)
            r[j] = beta == 0.f ? from_f32<T>(0.f) : from_f32<T>(beta * to_f32<T>(r[j]));
    }
}

template <typename T>
hipError_t launch(int64_t M, int64_t N, float beta, T* C, int64_t ldc, hipStream_t s) {
    const unsigned blocks = (unsigned)(M < 65536 ? M : 65536);
    void* kargs[] = {&M, &N, &beta, &C, &ldc};
    return hipLaunchKernel((const void*)&scale_kernel<T>, dim3(blocks), dim3(256), kargs, 0, s);
}

}  // namespace

hipError_t launch_scale_f32(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                            hipStream_t s) {
    return launch<float>(M, N, beta, C, ldc, s);
}

hipError_t launch_scale_bf16(int64_t M, int64_t N, float beta, uint16_t* C, int64_t ldc,
                             hipStream_t s) {
    return launch<uint16_t>(M, N, beta, C, ldc, s);
}

}  // namespace dg
