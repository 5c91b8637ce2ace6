// Debug checks of the C ABI, enabled per call by the environment variable
// ATTN_DEBUG (a nonzero integer): device-side validation of index and length
// arrays before the attention kernels are launched, and a scan of the outputs
// for non-finite values after them.  The checks raise a per-device flag word
// and never trap; the host reads the flag back (synchronising the stream) and
// turns it into a status.
#include "device.hpp"

namespace ets {

// One flag word per device (each GPU holds its own copy); host code uses the
// address hipGetSymbolAddress returns for the current device, never the name.
static __device__ __align__(256) unsigned debug_flag_word[64];

static hipError_t debug_flag_ptr(unsigned** out) {
  static std::mutex mu;
  static unsigned* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_flag_word));
    if (e != hipSuccess) return e;
    ptrs[dev] = (unsigned*)p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

__global__ void debug_flag_clear_kernel(unsigned* flag) { flag[0] = 0u; }

// lengths[b] must lie in [0, n]
__global__ __launch_bounds__(256) void debug_lengths_kernel(const int32_t* lengths, int B, int n, unsigned* flag) {
  for (int b = blockIdx.x * 256 + threadIdx.x; b < B; b += gridDim.x * 256) {
    const int v = lengths[b];
    if (v < 0 || v > n) atomicOr(flag, 1u);
  }
}

// topk_length[t] must lie in [0, topk]; topk_idx[t][u] in [0, Tkv) for u < topk_length[t]
__global__ __launch_bounds__(256) void debug_topk_kernel(const int32_t* idx, const int32_t* length, int Tq, int topk,
                                                        int Tkv, unsigned* flag) {
  const long long total = (long long)Tq * topk;
  for (long long k = (long long)blockIdx.x * 256 + threadIdx.x; k < total; k += (long long)gridDim.x * 256) {
    const int t = (int)(k / topk), u = (int)(k % topk);
    int L = topk;
    if (length) {
      L = length[t];
      if (u == 0 && (L < 0 || L > topk)) atomicOr(flag, 1u);
    }
    if (u < L) {
      const int j = idx[k];
      if (j < 0 || j >= Tkv) atomicOr(flag, 1u);
    }
  }
}

// Non-finite scan of n elements: kind 0 fp32, 1 fp16, 2 bf16, 3 fp32 where
// -inf is allowed (the LSE of a row with an empty allowed set).
__global__ __launch_bounds__(256) void debug_nonfinite_kernel(const void* p, long long n, int kind, unsigned* flag) {
  bool bad = false;
  for (long long k = (long long)blockIdx.x * 256 + threadIdx.x; k < n; k += (long long)gridDim.x * 256) {
    if (kind == 1) {
      bad |= (((const uint16_t*)p)[k] & 0x7c00u) == 0x7c00u;
    } else if (kind == 2) {
      bad |= (((const uint16_t*)p)[k] & 0x7f80u) == 0x7f80u;
    } else {
      const uint32_t w = ((const uint32_t*)p)[k];
      bad |= (w & 0x7f800000u) == 0x7f800000u && !(kind == 3 && w == 0xff800000u);
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(flag, 2u);
}

static unsigned grid_for(long long n) {
  const long long b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

static int flag_read(unsigned* flag, hipStream_t st, int* bad) {
  unsigned host = 0;
  ETS_TRY(hipMemcpyAsync(&host, flag, sizeof(unsigned), hipMemcpyDeviceToHost, st));
  ETS_TRY(hipStreamSynchronize(st));
  *bad = host != 0;
  return 0;
}

int debug_check_lengths(const int32_t* lengths, int B, int n, void* stream, int* bad) {
  hipStream_t st = (hipStream_t)stream;
  unsigned* flag = nullptr;
  ETS_TRY(debug_flag_ptr(&flag));
  ETS_TRY(launch(debug_flag_clear_kernel, dim3(1), dim3(1), 0, st, flag));
  ETS_TRY(launch(debug_lengths_kernel, dim3(grid_for(B)), dim3(256), 0, st, lengths, B, n, flag));
  return flag_read(flag, st, bad);
}

int debug_check_topk(const int32_t* idx, const int32_t* length, int Tq, int topk, int Tkv, void* stream, int* bad) {
  hipStream_t st = (hipStream_t)stream;
  unsigned* flag = nullptr;
  ETS_TRY(debug_flag_ptr(&flag));
  ETS_TRY(launch(debug_flag_clear_kernel, dim3(1), dim3(1), 0, st, flag));
  ETS_TRY(launch(debug_topk_kernel, dim3(grid_for((long long)Tq * topk)), dim3(256), 0, st, idx, length, Tq, topk,
                 Tkv, flag));
  return flag_read(flag, st, bad);
}

int debug_scan_nonfinite(const DebugBuf* bufs, int nbufs, void* stream, int* bad) {
  hipStream_t st = (hipStream_t)stream;
  unsigned* flag = nullptr;
  ETS_TRY(debug_flag_ptr(&flag));
  ETS_TRY(launch(debug_flag_clear_kernel, dim3(1), dim3(1), 0, st, flag));
  for (int i = 0; i < nbufs; ++i)
    if (bufs[i].ptr && bufs[i].count > 0)
      ETS_TRY(launch(debug_nonfinite_kernel, dim3(grid_for(bufs[i].count)), dim3(256), 0, st, bufs[i].ptr,
                     bufs[i].count, bufs[i].kind, flag));
  return flag_read(flag, st, bad);
}

}  // namespace ets
