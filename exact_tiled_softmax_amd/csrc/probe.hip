// Measurement aid: the dense bf16 MFMA rate this device actually sustains,
// reported beside the datasheet peak.  Every compute unit runs one workgroup
// of 4 * waves_per_simd waves; each wave issues `iters` x 8 independent
// v_mfma_f32_32x32x16_bf16 (two accumulator chains), with no memory traffic.
#include "device.hpp"

namespace ets {

__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, float* sink) {
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  BF16::vec8 x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(0.001f * (float)(threadIdx.x & 63) + 0.25f * (float)i);
    y[i] = (__bf16)(0.5f * (float)i);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m & 1] = BF16::mfma32(x, y, acc[m & 1]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;  // keeps the work alive
}

int launch_mfma_probe(int waves_per_simd, int iters, float* sink, int sink_len, long long* mfmas, void* stream) {
  int dev = 0, cus = 0;
  ETS_TRY(hipGetDevice(&dev));
  ETS_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (cus > sink_len) return -1;  // sink shorter than the CU count
  const int threads = 256 * waves_per_simd;
  *mfmas = (long long)cus * (threads / 64) * iters * 8;
  ETS_TRY(launch(mfma_probe_kernel, dim3(cus), dim3(threads), 0, (hipStream_t)stream, iters, sink));
  return 0;
}

}  // namespace ets
