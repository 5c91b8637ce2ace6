// Dense masked attention in fp32 on the vector ALUs (no MFMA): the
// correctness path for fp32 inputs and any head width up to 128.  The forward
// pass follows the block recurrence literally with the caller's key-block
// size b (alphabetamath.cc, "Tiled attention and its recomputed reverse pass
// are exact", proof paragraph 1; intale.github.io ch. 19, "Rescale earlier
// mass before adding a new tile"):
//   * the row starts in the empty state; a key block whose allowed part is
//     empty leaves the state untouched;
//   * the first contributing block is copied (alpha = 0), later ones merge
//     with alpha = e^{m - m'};
//   * Y = z / l after the last block, LSE = m + ln l.
// The reverse pass recomputes p_ij = e^{s_ij - LSE_i} and accumulates
// gamma_ij = p_ij (kappa_ij G_i.V_j - D_i) into dQ (one thread per query row)
// and into dK, dV (one thread per key row, looping over every query head of
// its group), so no atomics are needed.
#include "device.hpp"

namespace ets {

__device__ __forceinline__ float kappa1(const DropArgs& d, int lane_bh, int i, int j) {
  if (!d.enabled) return 1.f;
  return ((keep8(d, lane_bh, i, j & ~7) >> (j & 7)) & 1u) ? d.inv_keep : 0.f;
}

template <int DM>
__global__ __launch_bounds__(64) void f32_fwd_kernel(const DenseArgs a) {
  const int i = blockIdx.x * 64 + threadIdx.x, bh = blockIdx.y;
  if (i >= a.nq) return;
  const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
  const int d = a.d, dv = a.dv, nk = a.nk;
  const Layout lay = layout_of<kDenseM>(a.mask, b, a.nq, nk);
  const float* Q = (const float*)a.Q + ((size_t)bh * a.nq + i) * d;
  const float* K = (const float*)a.K + (size_t)(b * a.Hkv + g) * nk * d;
  const float* V = (const float*)a.V + (size_t)(b * a.Hkv + g) * nk * dv;
  float q[DM], z[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) { q[r] = (r < d) ? Q[r] : 0.f; z[r] = 0.f; }
  float m = kNegInf, l = 0.f;
  bool empty = true;  // the empty state
  for (int j0 = 0; j0 < nk; j0 += a.block_b) {
    const int j1 = min(nk, j0 + a.block_b);
    float amax = kNegInf;
    bool any = false;
    for (int j = j0; j < j1; ++j) {
      if (!allowed1<kDenseM>(a.mask, i, j, lay.len, lay.nka, true, lay.st)) continue;
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < DM; ++r)
        if (r < d) s = fmaf(q[r], K[(size_t)j * d + r], s);
      s *= a.scale;
      amax = any ? fmaxf(amax, s) : s;
      any = true;
    }
    if (!any) continue;  // empty allowed block: state unchanged
    const float mn = empty ? amax : fmaxf(m, amax);
    const float alpha = empty ? 0.f : expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int r = 0; r < DM; ++r) z[r] *= alpha;
    for (int j = j0; j < j1; ++j) {
      if (!allowed1<kDenseM>(a.mask, i, j, lay.len, lay.nka, true, lay.st)) continue;
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < DM; ++r)
        if (r < d) s = fmaf(q[r], K[(size_t)j * d + r], s);
      const float p = expf(s * a.scale - mn);
      l += p;
      const float w = p * kappa1(a.drop, bh, i, j);
#pragma unroll
      for (int r = 0; r < DM; ++r)
        if (r < dv) z[r] = fmaf(w, V[(size_t)j * dv + r], z[r]);
    }
    m = mn;
    empty = false;
  }
  float* Y = (float*)a.out_Y + ((size_t)bh * a.nq + i) * dv;
  const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
  for (int r = 0; r < DM; ++r)
    if (r < dv) Y[r] = z[r] * inv;
  a.LSE[(size_t)bh * a.nq + i] = empty ? kNegInf : m + logf(l);
}

// D_i = G_i . Y_i
__global__ __launch_bounds__(64) void f32_prep_kernel(const DenseArgs a, int rows) {
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  const float* G = (const float*)a.G + (size_t)r * a.dv;
  const float* Y = (const float*)a.Y + (size_t)r * a.dv;
  float acc = 0.f;
  for (int c = 0; c < a.dv; ++c) acc = fmaf(G[c], Y[c], acc);
  a.Dws[r] = acc;
}

template <int DM>
__global__ __launch_bounds__(64) void f32_dq_kernel(const DenseArgs a) {
  const int i = blockIdx.x * 64 + threadIdx.x, bh = blockIdx.y;
  if (i >= a.nq) return;
  const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
  const int d = a.d, dv = a.dv, nk = a.nk;
  const Layout lay = layout_of<kDenseM>(a.mask, b, a.nq, nk);
  const size_t row = (size_t)bh * a.nq + i;
  const float* Q = (const float*)a.Q + row * d;
  const float* Gr = (const float*)a.G + row * dv;
  const float* K = (const float*)a.K + (size_t)(b * a.Hkv + g) * nk * d;
  const float* V = (const float*)a.V + (size_t)(b * a.Hkv + g) * nk * dv;
  const float lse = a.LSE[row], Di = a.Dws[row];
  float q[DM], gr[DM], dq[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) {
    q[r] = (r < d) ? Q[r] : 0.f;
    gr[r] = (r < dv) ? Gr[r] : 0.f;
    dq[r] = 0.f;
  }
  for (int j = 0; j < nk; ++j) {
    if (!allowed1<kDenseM>(a.mask, i, j, lay.len, lay.nka, true, lay.st)) continue;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int r = 0; r < DM; ++r) {
      if (r < d) s = fmaf(q[r], K[(size_t)j * d + r], s);
      if (r < dv) dp = fmaf(gr[r], V[(size_t)j * dv + r], dp);
    }
    const float p = expf(s * a.scale - lse);
    const float gm = p * (kappa1(a.drop, bh, i, j) * dp - Di);
#pragma unroll
    for (int r = 0; r < DM; ++r)
      if (r < d) dq[r] = fmaf(gm, K[(size_t)j * d + r], dq[r]);
  }
  float* dQ = (float*)a.dQ + row * d;
#pragma unroll
  for (int r = 0; r < DM; ++r)
    if (r < d) dQ[r] = dq[r] * a.scale;
}

template <int DM>
__global__ __launch_bounds__(64) void f32_dkdv_kernel(const DenseArgs a) {
  const int j = blockIdx.x * 64 + threadIdx.x, bg = blockIdx.y;
  if (j >= a.nk) return;
  const int b = bg / a.Hkv, g = bg % a.Hkv, grp = a.H / a.Hkv;
  const int d = a.d, dv = a.dv, nq = a.nq;
  const Layout lay = layout_of<kDenseM>(a.mask, b, nq, a.nk);
  const float* Kr = (const float*)a.K + ((size_t)bg * a.nk + j) * d;
  const float* Vr = (const float*)a.V + ((size_t)bg * a.nk + j) * dv;
  float k[DM], v[DM], dk[DM], dvv[DM];
#pragma unroll
  for (int r = 0; r < DM; ++r) {
    k[r] = (r < d) ? Kr[r] : 0.f;
    v[r] = (r < dv) ? Vr[r] : 0.f;
    dk[r] = 0.f;
    dvv[r] = 0.f;
  }
  for (int hh = 0; hh < grp; ++hh) {
    const int h = g * grp + hh, bh = b * a.H + h;
    const float* Q = (const float*)a.Q + (size_t)bh * nq * d;
    const float* G = (const float*)a.G + (size_t)bh * nq * dv;
    for (int i = 0; i < nq; ++i) {
      if (!allowed1<kDenseM>(a.mask, i, j, lay.len, lay.nka, true, lay.st)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int r = 0; r < DM; ++r) {
        if (r < d) s = fmaf(Q[(size_t)i * d + r], k[r], s);
        if (r < dv) dp = fmaf(G[(size_t)i * dv + r], v[r], dp);
      }
      const size_t row = (size_t)bh * nq + i;
      const float p = expf(s * a.scale - a.LSE[row]);
      const float kap = kappa1(a.drop, bh, i, j);
      const float gm = p * (kap * dp - a.Dws[row]);
      const float w = p * kap;
#pragma unroll
      for (int r = 0; r < DM; ++r) {
        if (r < d) dk[r] = fmaf(gm, Q[(size_t)i * d + r], dk[r]);
        if (r < dv) dvv[r] = fmaf(w, G[(size_t)i * dv + r], dvv[r]);
      }
    }
  }
  float* dK = (float*)a.dK + ((size_t)bg * a.nk + j) * d;
  float* dV = (float*)a.dV + ((size_t)bg * a.nk + j) * dv;
#pragma unroll
  for (int r = 0; r < DM; ++r) {
    if (r < d) dK[r] = dk[r] * a.scale;
    if (r < dv) dV[r] = dvv[r];
  }
}

int launch_dense_fwd_f32(const DenseArgs& a, void* stream) {
  dim3 grid((a.nq + 63) / 64, a.B * a.H), block(64);
  hipStream_t st = (hipStream_t)stream;
  if (a.d <= 32 && a.dv <= 32)
    ETS_TRY(launch(f32_fwd_kernel<32>, grid, block, 0, st, a));
  else
    ETS_TRY(launch(f32_fwd_kernel<128>, grid, block, 0, st, a));
  return 0;
}

int launch_dense_bwd_f32(const DenseArgs& a, void* stream, int phases) {
  hipStream_t st = (hipStream_t)stream;
  const int rows = a.B * a.H * a.nq;
  if (phases & 1) ETS_TRY(launch(f32_prep_kernel, dim3((rows + 63) / 64), dim3(64), 0, st, a, rows));
  dim3 gq((a.nq + 63) / 64, a.B * a.H), gk((a.nk + 63) / 64, a.B * a.Hkv);
  if (a.d <= 32 && a.dv <= 32) {
    if (phases & 2) ETS_TRY(launch(f32_dkdv_kernel<32>, gk, dim3(64), 0, st, a));
    if (phases & 4) ETS_TRY(launch(f32_dq_kernel<32>, gq, dim3(64), 0, st, a));
  } else {
    if (phases & 2) ETS_TRY(launch(f32_dkdv_kernel<128>, gk, dim3(64), 0, st, a));
    if (phases & 4) ETS_TRY(launch(f32_dq_kernel<128>, gq, dim3(64), 0, st, a));
  }
  return 0;
}

}  // namespace ets
