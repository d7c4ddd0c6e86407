// tsp_bwd_aux.hip -- memory-bound helpers of the layer backward: transposes (bf16, and fp32
// to bf16), an fp32 to bf16 conversion, and the elementwise backward of the SwiGLU gate.
//
// The weight gradients are sums over tokens (dW = dY^T X); the GEMM kernels take both
// operands contiguous along the reduction, so the token-major activations are transposed
// once, through 32 x 32 LDS tiles (one read and one write of each element).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tsp_device.h"
#include "tsp_internal.h"

namespace tsp {
namespace {

constexpr int kT = 32;  // transpose tile
constexpr int kTy = 8;  // threads per tile column

template <class Src>
__device__ __forceinline__ float load_f(const Src* p) {
  if constexpr (sizeof(Src) == 2) {
    return __uint_as_float((uint32_t)(*p) << 16);
  } else {
    return *p;
  }
}

// dst[c][r] = src[r][c] for r < R, c < C (bf16 result, rounded to nearest even from fp32).
template <class Src>
__global__ __launch_bounds__(kT* kTy) void transpose_kernel(const Src* src, int64_t lds, bf16_t* dst, int64_t ldd,
                                                            int R, int C) {
  __shared__ bf16_t tile[kT][kT + 1];
  const int c0 = blockIdx.x * kT, r0 = blockIdx.y * kT;
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
#pragma unroll
  for (int i = ty; i < kT; i += kTy) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) {
      if constexpr (sizeof(Src) == 2) {
        tile[i][tx] = src[(int64_t)r * lds + c];
      } else {
        tile[i][tx] = to_bf16(src[(int64_t)r * lds + c]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = ty; i < kT; i += kTy) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < C) dst[(int64_t)c * ldd + r] = tile[tx][i];
  }
}

__global__ __launch_bounds__(256) void convert_kernel(const float* src, int64_t lds, bf16_t* dst, int64_t ldd, int R,
                                                      int C) {
  const int64_t n = (int64_t)R * C;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / C, c = e - (e / C) * C;
    dst[r * ldd + c] = to_bf16(src[r * lds + c]);
  }
}

// From the recomputed gate pair gu = [g | u] (bf16 [M, 2 Fs]) and dh = dL/dh (fp32 [M, Fs]),
// with h = silu(g) u and silu'(g) = s (1 + g (1 - s)), s = sigmoid(g):
//   h (bf16), dgu = [dh u silu'(g) | dh silu(g)] (bf16).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16_t* gu, int64_t ldgu, const float* dh,
                                                         int64_t lddh, bf16_t* h, int64_t ldh, bf16_t* dgu,
                                                         int64_t lddgu, int M, int Fs) {
  const int64_t n = (int64_t)M * Fs;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / Fs, f = e - (e / Fs) * Fs;
    const float g = load_f(gu + m * ldgu + f);
    const float u = load_f(gu + m * ldgu + Fs + f);
    const float d = dh[m * lddh + f];
    const float s = 1.0f / (1.0f + __expf(-g));
    const float sl = g * s;
    h[m * ldh + f] = to_bf16(sl * u);
    dgu[m * lddgu + f] = to_bf16(d * u * s * (1.0f + g * (1.0f - s)));
    dgu[m * lddgu + Fs + f] = to_bf16(d * sl);
  }
}

unsigned grid_1d(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 256 * 32); }

}  // namespace

hipError_t launch_transpose_bf16(const void* src, int64_t lds, void* dst, int64_t ldd, int R, int C,
                                 hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel<bf16_t>, dim3((C + kT - 1) / kT, (R + kT - 1) / kT), dim3(kT * kTy), 0, stream,
                     static_cast<const bf16_t*>(src), lds, static_cast<bf16_t*>(dst), ldd, R, C);
  return hipGetLastError();
}

hipError_t launch_transpose_f32_bf16(const float* src, int64_t lds, void* dst, int64_t ldd, int R, int C,
                                     hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel<float>, dim3((C + kT - 1) / kT, (R + kT - 1) / kT), dim3(kT * kTy), 0, stream,
                     src, lds, static_cast<bf16_t*>(dst), ldd, R, C);
  return hipGetLastError();
}

hipError_t launch_convert_f32_bf16(const float* src, int64_t lds, void* dst, int64_t ldd, int R, int C,
                                   hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(convert_kernel, dim3(grid_1d((int64_t)R * C)), dim3(256), 0, stream, src, lds,
                     static_cast<bf16_t*>(dst), ldd, R, C);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* gu, int64_t ldgu, const float* dh, int64_t lddh, void* h, int64_t ldh,
                             void* dgu, int64_t lddgu, int M, int Fs, hipStream_t stream) {
  if (M <= 0 || Fs <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid_1d((int64_t)M * Fs)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(gu), ldgu, dh, lddh, static_cast<bf16_t*>(h), ldh,
                     static_cast<bf16_t*>(dgu), lddgu, M, Fs);
  return hipGetLastError();
}

}  // namespace tsp
