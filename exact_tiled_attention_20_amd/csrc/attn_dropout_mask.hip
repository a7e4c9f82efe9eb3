// Export of the dropout keep-mask (a test aid): keep[b][h][i][j] = 1 iff the
// Philox4x32-10 draw for (seed; b, h, i, j) is at or above the drop threshold.
// The forward and backward kernels draw the same bits in registers and never
// store them; this kernel lets tests compare those bits with the CPU oracle.
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {

// One thread per (b, h, i, t): one Philox call yields keys 4t .. 4t+3 of
// the Nk keys of query row i.
__global__ __launch_bounds__(256) void dropout_mask_kernel(const MaskArgs a) {
  const int groups = (a.Nk + 3) >> 2;
  const long long total = (long long)a.B * a.H * a.N * groups;
  const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int t = (int)(id % groups);
  long long rest = id / groups;
  const int i = (int)(rest % a.N);
  rest /= a.N;
  const int h = (int)(rest % a.H);
  const int b = (int)(rest / a.H);
  const u32x4 u = dropout_draws((uint32_t)t, (uint32_t)i, (uint32_t)h, (uint32_t)b,
                                a.seed_lo, a.seed_hi);
  uint8_t* row = a.keep + (((size_t)b * a.H + h) * a.N + i) * (size_t)a.Nk;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * t + e;
    if (j < a.Nk) row[j] = (u[e] >= a.drop_threshold) ? 1 : 0;
  }
}

hipError_t launch_dropout_mask(const MaskArgs& a, hipStream_t stream) {
  const long long total = (long long)a.B * a.H * a.N * ((a.Nk + 3) / 4);
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
