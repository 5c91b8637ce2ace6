// Export of the dropout realisation xi (uint8 [B][H][n_q][n_k], 1 = kept) so
// that tests can compare it bit for bit with an independent Philox.  Uses the
// same keep8() the attention kernels call.
#include "device.hpp"

namespace ets {

__global__ __launch_bounds__(256) void dropout_mask_kernel(const DropArgs d, int H, int nq, int nk,
                                                           long long groups, uint8_t* xi) {
  const int ng = (nk + 7) / 8;  // 8-key groups per row
  for (long long t = blockIdx.x * 256LL + threadIdx.x; t < groups; t += (long long)gridDim.x * 256) {
    const int jg = (int)(t % ng);
    const long long row = t / ng;  // (b*H + h)*nq + i
    const int i = (int)(row % nq);
    const int lane_bh = (int)(row / nq);
    const unsigned keep = keep8(d, lane_bh, i, 8 * jg);
    uint8_t* out = xi + row * nk + 8 * jg;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (8 * jg + r < nk) out[r] = (keep >> r) & 1u;
  }
}

int launch_dropout_mask(const DropArgs& d, int B, int H, int nq, int nk, uint8_t* xi, void* stream) {
  const long long groups = (long long)B * H * nq * ((nk + 7) / 8);
  const long long blocks = (groups + 255) / 256;
  ETS_TRY(launch(dropout_mask_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0,
                     (hipStream_t)stream, d, H, nq, nk, groups, xi));
  return 0;
}

}  // namespace ets
