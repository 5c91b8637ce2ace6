// Dense masked attention backward (block-recomputed VJP), bf16/fp16 MFMA
// path for gfx950.
//
// What it computes (alphabetamath.cc, "Tiled attention and its recomputed
// reverse pass are exact", paragraphs 4-6; intale.github.io ch. 19,
// "Reconstruct probabilities when a gradient needs them"):
//   D_i      = sum_a G_ia Y_ia
//   p_ij     = exp(s_ij - LSE_i)                       (zero outside A_i)
//   gamma_ij = p_ij (kappa_ij (G_i . V_j) - D_i)       (kappa = xi / (1 - rho), 1 without dropout)
//   dQ_i = c sum_j gamma_ij K_j,  dK_j = c sum_i gamma_ij Q_i,  dV_j = sum_i p_ij kappa_ij G_i
// with the dropout realisation regenerated from the same Philox counters as
// the forward pass.  Key and value gradients of every query head of a group
// are summed into the shared head.
//
// Three kernels, all on the caller's stream:
//   prep  -D_i from G and Y (fp32, into the workspace);
//   dkdv  key-major: a workgroup owns 128 keys of one K/V head, keeps its K
//         and V rows in registers as MFMA B operands, and walks every query
//         tile (and every query head of the group) that can see them; S = Q K^T
//         and dP = G V^T put keys along lanes, so P and gamma feed
//         dV^T += G^T P and dK^T += Q^T gamma directly, with G^T and Q^T read
//         by LDS transpose reads.  No atomics.
//   dq    query-major: the forward layout (queries along lanes); recomputes
//         S^T and dP^T and accumulates dQ^T += K^T gamma^T, with K^T read by
//         LDS transpose reads.  No atomics.  With dropout and a causal /
//         window mask, and a workspace large enough for them, dkdv also
//         stores its gamma tiles and dq reads them instead of recomputing
//         (dense_bwd_dq_stored_kernel in dense_dq.hip).
#include "device.hpp"

namespace ets {

// --------------------------------------------------------------------- prep
// -D_i = -(G_i . Y_i) and the base-2 LSE, LSE_i log2(e) (+inf for a row with
// an empty allowed set, so every recomputed weight of it is 0).  The 64 rows
// after the last are filled with D = 0, LSE2 = +inf: tiles of 64 rows may read
// them.  -D is stored so that it can start a dP accumulator (dP - D).
template <class E, int D>
__global__ __launch_bounds__(256) void dense_bwd_prep_kernel(const DenseArgs a, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long long nthreads = (rows + 64) * LPR;
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t - threadIdx.x < nthreads;
       t += (long long)gridDim.x * 256) {
    // whole wave-groups of LPR lanes stay together, so the reduction below
    // sees one row per group even on the grid-stride tail
    const long long row = t / LPR;
    const int part = (int)(t % LPR);
    float acc = 0.f;
    if (row < rows) {
      const u32x4 g = *(const u32x4*)((const uint16_t*)a.G + (size_t)row * D + 8 * part);
      const u32x4 y = *(const u32x4*)((const uint16_t*)a.Y + (size_t)row * D + 8 * part);
      const uint32_t gw[4] = {g[0], g[1], g[2], g[3]}, yw[4] = {y[0], y[1], y[2], y[3]};
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += E::lo(gw[k]) * E::lo(yw[k]) + E::hi(gw[k]) * E::hi(yw[k]);
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (part == 0 && row < rows + 64) {
      float l2 = __builtin_huge_valf();
      if (row < rows) {
        const float l = a.LSE[row];
        l2 = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
      } else {
        acc = 0.f;
      }
      a.Dws[row] = -acc;
      a.Lws[row] = l2;
    }
  }
}

template <class E, int D>
static int launch_prep(const DenseArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.H * a.nq;
  const long long blocks = ((rows + 64) * (D / 8) + 255) / 256;
  ETS_TRY(launch((dense_bwd_prep_kernel<E, D>), dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                 a, rows));
  return 0;
}

template <int DT, int D>
static int launch_bwd_ed(const DenseArgs& a, void* stream, int phases) {
  using E = std::conditional_t<DT == (int)Dt::BF16, BF16, F16>;
  hipStream_t st = (hipStream_t)stream;
  if (phases & 1) {
    const int rc = launch_prep<E, D>(a, st);
    if (rc) return rc;
  }
  if (phases & 2) {
    const int rc = launch_dense_dkdv_ed<DT, D>(a, stream);
    if (rc) return rc;
  }
  if (phases & 4) {
    const int rc = launch_dense_dq_ed<DT, D>(a, stream);
    if (rc) return rc;
  }
  return 0;
}

int launch_dense_bwd(const DenseArgs& a, Dt dt, void* stream, int phases) {
  if (dt == Dt::BF16)
    return a.d == 128 ? launch_bwd_ed<2, 128>(a, stream, phases) : launch_bwd_ed<2, 64>(a, stream, phases);
  return a.d == 128 ? launch_bwd_ed<1, 128>(a, stream, phases) : launch_bwd_ed<1, 64>(a, stream, phases);
}

int launch_dense_fwd(const DenseArgs& a, Dt dt, void* stream) {
  if (dt == Dt::BF16)
    return a.d == 128 ? launch_dense_fwd_ed<2, 128>(a, stream) : launch_dense_fwd_ed<2, 64>(a, stream);
  return a.d == 128 ? launch_dense_fwd_ed<1, 128>(a, stream) : launch_dense_fwd_ed<1, 64>(a, stream);
}

bool dense_mfma_supported(int d, int dv) { return d == dv && (d == 64 || d == 128); }

}  // namespace ets
