// Per-head output error against a reference output, for the offline
// kernel-aware pattern search (PaperTrace 2.1.2 "MInference", sections 3.1
// and 6.3; blog-zz7 "LLM模型之MInference", section 2.3.1, Eq. 2): every
// candidate pattern's attention output on a calibration input is compared
// with the dense output.
//
// One work-group of 256 threads per (batch, head): thread t sums elements
// t, t + 256, ... of the head's [n, dh] block in fp64 (a fixed order), then
// the threads are combined by a fixed tree in LDS, so two runs give
// identical bits.  Both the squared difference and the reference's squared
// norm are written, so the caller can form absolute or relative errors.
//
// Captured attention mass, the other measure of the same search: a row whose
// kept keys carry the fraction m of the dense softmax has m = exp(lse_kept -
// lse_dense) (both log-sum-exps of the same scores), and Eq. 2's distance
// between the renormalised and the dense attention row is 2 (1 - m) in L1.
// Per (batch, head) the kernel sums exp(lse - lse_ref) over the rows, in the
// same fixed order.
#include "kernels.h"

namespace minf {
namespace {

template <bool BF16>
__device__ __forceinline__ double load_elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    const uint32_t bits = (uint32_t)(reinterpret_cast<const uint16_t*>(p)[i]) << 16;
    return (double)__builtin_bit_cast(float, bits);
  } else {
    return (double)reinterpret_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void output_error_kernel(const void* O, const void* R, int64_t per_head, double* err) {
  const int64_t base = (int64_t)blockIdx.x * per_head;
  double d2 = 0.0, r2 = 0.0;
  for (int64_t i = threadIdx.x; i < per_head; i += 256) {
    const double x = load_elem<BF16>(O, base + i), y = load_elem<BF16>(R, base + i);
    d2 += (x - y) * (x - y);
    r2 += y * y;
  }
  __shared__ double sd[256], sr[256];
  sd[threadIdx.x] = d2;
  sr[threadIdx.x] = r2;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      sd[threadIdx.x] += sd[threadIdx.x + off];
      sr[threadIdx.x] += sr[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    err[2 * blockIdx.x] = sd[0];
    err[2 * blockIdx.x + 1] = sr[0];
  }
}

__global__ __launch_bounds__(256) void captured_mass_kernel(const float* lse, const float* lse_ref, int64_t n,
                                                            double* mass) {
  const int64_t base = (int64_t)blockIdx.x * n;
  double m = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    const float a = lse[base + i], r = lse_ref[base + i];
    // a row without kept keys (lse = -inf) contributes 0; the reference
    // (dense) always has a key
    if (a != -__builtin_huge_valf() && r != -__builtin_huge_valf()) m += exp((double)a - (double)r);
  }
  __shared__ double sm[256];
  sm[threadIdx.x] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) sm[threadIdx.x] += sm[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) mass[blockIdx.x] = sm[0];
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_captured_mass(const float* lse, const float* lse_ref, int64_t heads, int64_t n, double* mass,
                                hipStream_t st) {
  hipLaunchKernelGGL(captured_mass_kernel, dim3((unsigned)heads), dim3(256), 0, st, lse, lse_ref, n, mass);
  return hipGetLastError();
}

hipError_t launch_output_error(const void* O, const void* R, int64_t heads, int64_t per_head, bool bf16, double* err,
                               hipStream_t st) {
  if (bf16) hipLaunchKernelGGL(output_error_kernel<true>, dim3((unsigned)heads), dim3(256), 0, st, O, R, per_head, err);
  else hipLaunchKernelGGL(output_error_kernel<false>, dim3((unsigned)heads), dim3(256), 0, st, O, R, per_head, err);
  return hipGetLastError();
}

}  // namespace minf
