// Achievable matrix-core rate of this GPU, the measured denominator the
// benchmark reports beside the vendor's dense fp16 figure: every wave runs
// `iters` rounds of eight independent v_mfma_f32_16x16x32_f16 on register
// operands (eight accumulator chains keep the matrix pipe full; the loop
// touches no memory).  Not part of the quantisation or attention path.
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

typedef _Float16 ph8 __attribute__((ext_vector_type(8)));
typedef float pf4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  ph8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (float)(lane + j));
    b[j] = (_Float16)(0.002f * (float)(j - lane));
  }
  pf4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {   // distinct chains (the compiler may not merge them)
    const float v = (float)(j + 1) * (float)(lane + 1);
    acc[j] = pf4{v, -v, 0.5f * v, 2.0f * v};
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;   // keeps every chain live
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_mfma_peak_probe(float* out_dev, int32_t blocks, int32_t iters, void* stream) {
  if (!out_dev || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24)) return KVQ_EINVAL;
  kvq::mfma_peak_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(out_dev, iters);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}
