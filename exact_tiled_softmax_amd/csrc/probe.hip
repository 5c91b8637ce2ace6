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

namespace ets {

// Measurement aid: how many independent VALU instructions this device hides
// under MFMAs.  Each wave issues iters x 8 v_mfma_f32_32x32x16_bf16 (four
// accumulators), each followed by K independent v_fma_f32 (TRANS = false) or
// K independent v_exp_f32 (TRANS = true) on registers of their own, the order
// pinned by scheduling groups.  (The exponentials run to infinity after a few
// steps; the rate does not depend on the values.)
constexpr int kSchedTrans = 0x400;  // scheduling-group mask of transcendental instructions

template <int K, bool TRANS>
__global__ __launch_bounds__(512) void issue_probe_kernel(int iters, float* sink) {
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  BF16::vec8 x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(0.001f * (float)(threadIdx.x & 63) + 0.25f * (float)i);
    y[i] = (__bf16)(0.5f * (float)i);
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = 0.01f * (float)(threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      acc[m & 3] = BF16::mfma32(x, y, acc[m & 3]);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float& t = v[(m * K + k) & 15];
        if constexpr (TRANS) t = fast_exp2(t);
        else t = fmaf(t, 0.999f, 0.001f);
      }
      ETS_SCHED(kSchedMFMA, 1);
      if constexpr (K > 0) ETS_SCHED(TRANS ? kSchedTrans : kSchedVALU, K);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += v[i];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;  // keeps the work alive
}

template <bool TRANS>
static int launch_issue_k(int k, int cus, int threads, int iters, float* sink, hipStream_t st) {
  switch (k) {
    case 0: ETS_TRY(launch(issue_probe_kernel<0, TRANS>, dim3(cus), dim3(threads), 0, st, iters, sink)); break;
    case 2: ETS_TRY(launch(issue_probe_kernel<2, TRANS>, dim3(cus), dim3(threads), 0, st, iters, sink)); break;
    case 4: ETS_TRY(launch(issue_probe_kernel<4, TRANS>, dim3(cus), dim3(threads), 0, st, iters, sink)); break;
    case 6: ETS_TRY(launch(issue_probe_kernel<6, TRANS>, dim3(cus), dim3(threads), 0, st, iters, sink)); break;
    case 8: ETS_TRY(launch(issue_probe_kernel<8, TRANS>, dim3(cus), dim3(threads), 0, st, iters, sink)); break;
    case 12: ETS_TRY(launch(issue_probe_kernel<12, TRANS>, dim3(cus), dim3(threads), 0, st, iters, sink)); break;
    default: return -2;
  }
  return 0;
}

int launch_issue_probe(int waves_per_simd, int valu_per_mfma, int trans, int iters, float* sink, int sink_len,
                       long long* mfmas, void* stream) {
  int dev = 0, cus = 0;
  ETS_TRY(hipGetDevice(&dev));
  ETS_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (cus > sink_len) return -1;
  const int threads = 256 * waves_per_simd;
  *mfmas = (long long)cus * (threads / 64) * iters * 8;
  hipStream_t st = (hipStream_t)stream;
  return trans ? launch_issue_k<true>(valu_per_mfma, cus, threads, iters, sink, st)
               : launch_issue_k<false>(valu_per_mfma, cus, threads, iters, sink, st);
}
// Measurement aid: the rate of fp32 atomic adds into random 576-float rows of
// a table, in the access pattern of the sparse dKV scatter: each instruction
// covers 4 rows x 16 consecutive floats (16 lanes per row), 36 instructions
// per group of 4 rows.  Row indices come from idx[0 .. n_idx) cyclically.
__global__ __launch_bounds__(256) void atomic_probe_kernel(float* table, const int32_t* idx, int n_idx, int rows,
                                                          int groups_per_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  for (int it = 0; it < groups_per_wave; ++it) {
    const long long k = (((long long)blockIdx.x * groups_per_wave + it) * 4 + wave) * 4 + g;
    const int r = idx[k % n_idx];
    if ((unsigned)r >= (unsigned)rows) continue;
    float* p = table + (size_t)r * 576 + l16;
#pragma unroll 4
    for (int m = 0; m < 36; ++m) atomicAdd(p + 16 * m, 1.0f);
  }
}

int launch_atomic_probe(float* table, int rows, const int32_t* idx, int n_idx, int blocks, int groups_per_wave,
                        long long* adds, void* stream) {
  *adds = (long long)blocks * 4 * groups_per_wave * 4 * 576;
  ETS_TRY(launch(atomic_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, table, idx, n_idx, rows,
                 groups_per_wave));
  return 0;
}

// Measurement aid: LDS read bandwidth.  One workgroup of `waves` waves per
// compute unit fills 64 KiB of LDS, then every wave issues iters x 16
// conflict-free ds_read_b128 (lane l reads 16 bytes at 16 l + 1 KiB k, all
// addresses inside the 64 KiB array) and XOR-folds them into sink.
__global__ __launch_bounds__(1024) void lds_probe_kernel(int iters, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char buf[65536];
  for (int i = threadIdx.x; i < 65536 / 4; i += blockDim.x) ((uint32_t*)buf)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)(lane * 16 + wave * 8192) & 0xFFFFu;
  u32x4 acc = u32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t addr = (base + (uint32_t)k * 1024u + (uint32_t)it * 64u) & 0xFFF0u;
      acc ^= *(const u32x4*)(buf + addr);
    }
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (threadIdx.x == 0) sink[blockIdx.x] = x;  // keeps the loads alive
}

int launch_lds_probe(int waves, int iters, uint32_t* sink, int sink_len, long long* bytes, void* stream) {
  int dev = 0, cus = 0;
  ETS_TRY(hipGetDevice(&dev));
  ETS_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (cus > sink_len) return -1;
  *bytes = (long long)cus * waves * 64 * 16 * 16 * iters;
  ETS_TRY(launch(lds_probe_kernel, dim3(cus), dim3(64 * waves), 0, (hipStream_t)stream, iters, sink));
  return 0;
}

}  // namespace ets
