// Shared-KV top-k sparse attention with an attention sink (bf16/fp16 MFMA,
// gfx950).
//
// What it computes (icavan.github.io, "DeepSeek Sparse Attention Forward and
// Backward", sections 1-3, 7.1 and 8): for token t and head h, over the
// selected KV rows I = topk_idx[t][0:L_t],
//   s_u = alpha KV[I_u][0:576] . Q[t][h],   Z = e^{z_h} + sum_u e^{s_u},
//   O = sum_u (e^{s_u}/Z) KV[I_u][0:512],   LSE = ln Z (sink-inclusive),
// and for the gradients, with D = dO . O and dS_u = p_u (dO . v_u - D),
//   dQ = alpha sum_u dS_u k_u,  dKV[I_u] += alpha dS_u q (all 576 columns)
//   + p_u dO (first 512 columns),  dSink_h = -sum_t p_sink D.
//
// Mapping onto CDNA4: one workgroup per token; its four waves own 16 heads
// each and use v_mfma_f32_16x16x32 with heads along lanes.  The token's
// selected rows are gathered 32 at a time into LDS (double buffered, 1152-byte
// swizzled rows, 16-byte loads) and serve both as K (all 576 columns, MFMA A
// operand of S^T = K Q^T) and, through LDS transpose reads, as V^T (first 512
// columns) for O^T += V^T P^T.  The online summary runs per head exactly as in
// the dense kernels; the sink enters once, after the last tile, as one more
// term of the normaliser.
//
// Backward: a prepass (D, zeroing the fp32 dKV accumulator), a dQ kernel
// (token-major, private dQ rows, no atomics), a dKV kernel (recomputes P and
// dS, exchanges them through LDS so that each wave contracts over all 64
// heads for a quarter of the 576 columns; the key and value contributions of
// the tied row are summed in one accumulator and added with fp32 atomics into
// the workspace), and a finalize kernel (fp32 -> storage dtype; dSink summed
// over tokens in a fixed order).
#include "device.hpp"

namespace ets {

namespace sp {
constexpr int H = 64;          // heads per token (4 waves x 16)
constexpr int DQK = 576;       // key width (the whole tied row)
constexpr int DV = 512;        // value width (its first 512 columns)
constexpr int BK = 32;         // selected rows per tile
constexpr int ROWB = DQK * 2;  // bytes per LDS row
constexpr int TILEB = BK * ROWB;
constexpr int CPR = DQK / 8;   // 16-byte chunks per row (72)
constexpr int NCH = BK * CPR / 256;  // chunks per thread per tile (9)
constexpr int KSQ = DQK / 32;  // 32-wide k-steps over the key width (18)
constexpr int KSV = DV / 32;   // 32-wide k-steps over the value width (16)
constexpr int MQ = DQK / 16;   // 16-row blocks over the key width (36)
constexpr int MV = DV / 16;    // 16-row blocks over the value width (32)
constexpr int SMEM = 2 * TILEB;
constexpr float kRescaleSlack = 8.0f;
}  // namespace sp

// Deterministic dKV: each contribution is rounded to a multiple of 2^-32 and
// added as a 64-bit integer, so the sum does not depend on the order of the
// atomics (|dKV| must stay below 2^31).
constexpr float kFix = 4294967296.0f;
constexpr double kFixInv = 1.0 / 4294967296.0;

bool sparse_supported(int H, int dqk, int dv) { return H == sp::H && dqk == sp::DQK && dv == sp::DV; }

// Valid selection count of token t: topk_length[t] clamped to [0, topk]
// (topk without lengths).
__device__ __forceinline__ int sel_count(const SparseArgs& a, int t) {
  return a.length ? min(max(a.length[t], 0), a.topk) : a.topk;
}

// Gather of one tile of selected rows (global -> registers -> LDS).  The row
// indices of a tile are read one tile before its rows (load_idx, then fetch a
// tile later), so a fetch never waits on an index load.  A slot past L or an
// index outside [0, Tkv) reads as a zero row: no access leaves the KV tensor.
struct Gather {
  u32x4 pre[sp::NCH];
  int jrow[sp::NCH];  // KV row of each chunk of the next tile to fetch (-1: zero row)
  __device__ __forceinline__ void load_idx(const int32_t* idx_t, int L, int Tkv, int u0, int tid) {
#pragma unroll
    for (int v = 0; v < sp::NCH; ++v) {
      const int slot = u0 + (tid + 256 * v) / sp::CPR;
      const int j = slot < L ? idx_t[slot] : -1;
      jrow[v] = (unsigned)j < (unsigned)Tkv ? j : -1;
    }
  }
  __device__ __forceinline__ void fetch(const uint16_t* KV, int tid) {
#pragma unroll
    for (int v = 0; v < sp::NCH; ++v) {
      const int cc = (tid + 256 * v) % sp::CPR;
      pre[v] = u32x4{0, 0, 0, 0};
      if (jrow[v] >= 0) pre[v] = *(const u32x4*)(KV + (size_t)jrow[v] * sp::DQK + 8 * cc);
    }
  }
  __device__ __forceinline__ void stash(char ETS_LDS* buf, int tid) {
#pragma unroll
    for (int v = 0; v < sp::NCH; ++v) {
      const int c = tid + 256 * v, row = c / sp::CPR, cc = c % sp::CPR;
      lds_st128(buf, toff<sp::ROWB>(row, 8 * cc), pre[v]);
    }
  }
  // prologue: tile 0 into buf, the indices of tile 1 loaded
  __device__ __forceinline__ void start(const uint16_t* KV, const int32_t* idx_t, int L, int Tkv, int ntiles,
                                        char ETS_LDS* buf, int tid) {
    load_idx(idx_t, L, Tkv, 0, tid);
    fetch(KV, tid);
    stash(buf, tid);
    if (ntiles > 1) load_idx(idx_t, L, Tkv, sp::BK, tid);
  }
  // at the start of tile it: rows of tile it + 1 requested, indices of tile it + 2 loaded
  __device__ __forceinline__ void next(const uint16_t* KV, const int32_t* idx_t, int L, int Tkv, int it,
                                       int ntiles, int tid) {
    if (it + 1 < ntiles) {
      fetch(KV, tid);
      if (it + 2 < ntiles) load_idx(idx_t, L, Tkv, (it + 2) * sp::BK, tid);
    }
  }
};

// max / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float grp4_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return xhalf_max(x);
}
__device__ __forceinline__ float grp4_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return xhalf_sum(x);
}

// S^T = K_tile Q_h^T for this wave's 16 heads: s[mb][i] is key 16mb + 4(lane/16) + i
template <class E>
__device__ __forceinline__ void scores(const char ETS_LDS* kt, const typename E::vec8* qreg,
                                       const RowOps16<sp::ROWB>& rops, f32x4 s[2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[mb][r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < sp::KSQ; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const typename E::vec8 ka = as_vec8<E>(lds_b128(kt, rops.off(16 * mb, kk)));
      s[mb] = E::mfma16(ka, qreg[kk], s[mb]);
    }
  }
}

// Operands whose k-slots are the tile's keys 4G..4G+3, 16+4G..16+4G+3 (the
// order the S^T accumulators hold them in) come from TrOps16::read(tile, m):
// column block 16m .. 16m+15 of the tile by transpose reads.

// ------------------------------------------------------------------ forward
template <class E>
__global__ __launch_bounds__(256, 1) void sparse_fwd_kernel(const SparseArgs a) {
  using namespace sp;
  typedef typename E::vec8 vec8;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  char ETS_LDS* smem = (char ETS_LDS*)smem_dyn;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int G = lane >> 4, l16 = lane & 15;
  const int t = blockIdx.x;
  const int head = 16 * wave + l16;
  const uint16_t* KV = (const uint16_t*)a.KV;
  const int32_t* idx_t = a.idx + (size_t)t * a.topk;
  const int L = sel_count(a, t);

  vec8 qreg[KSQ];
  const uint16_t* Qh = (const uint16_t*)a.Q + ((size_t)t * H + head) * DQK;
#pragma unroll
  for (int kk = 0; kk < KSQ; ++kk) qreg[kk] = as_vec8<E>(*(const u32x4*)(Qh + 32 * kk + 8 * G));

  f32x4 oacc[MV];
#pragma unroll
  for (int m = 0; m < MV; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[m][r] = 0.f;
  float mref = kNegInf, lsum = 0.f;
  const float sl2 = a.scale_log2;

  Gather gat;
  const RowOps16<ROWB> rops(lane);
  const TrOps16<ROWB> tops(lane);
  const int ntiles = (L + BK - 1) / BK;
  if (ntiles > 0) {
    gat.start(KV, idx_t, L, a.Tkv, ntiles, smem, tid);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int u0 = it * BK;
    gat.next(KV, idx_t, L, a.Tkv, it, ntiles, tid);
    const char ETS_LDS* kt = smem + (it & 1) * TILEB;

    f32x4 s[2];
    scores<E>(kt, qreg, rops, s);
    const bool ragged = u0 + BK > L;
    if (ragged) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (u0 + 16 * mb + 4 * G + r >= L) s[mb][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = grp4_max(mx);
    const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
    const bool need = mt > mref + kRescaleSlack;
    if (wave_any(need)) {
      const float alpha = need ? fast_exp2(mref - mt) : 1.f;
      if (need) mref = mt;
      lsum *= alpha;
#pragma unroll
      for (int m = 0; m < MV; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[m][r] *= alpha;
    }
    float p[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = fast_exp2(fmaf(s[mb][r], sl2, -mref));
        if (ragged && u0 + 16 * mb + 4 * G + r >= L) v = 0.f;
        p[mb][r] = v;
        lsum += v;
      }
    const vec8 pb = as_vec8<E>(u32x4{E::pack2(p[0][0], p[0][1]), E::pack2(p[0][2], p[0][3]),
                                     E::pack2(p[1][0], p[1][1]), E::pack2(p[1][2], p[1][3])});
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const vec8 va = as_vec8<E>(tops.read(kt, m));
      oacc[m] = E::mfma16(va, pb, oacc[m]);
    }
    if (it + 1 < ntiles) gat.stash(smem + ((it + 1) & 1) * TILEB, tid);
    __syncthreads();
  }

  // fold in the sink: Z = 2^mref * l + 2^{z log2 e}
  const float l = grp4_sum(lsum);
  const float z2 = a.sink ? a.sink[head] * kLog2e : kNegInf;
  const float M = fmaxf(mref, z2);
  float lt = 0.f, scale_o = 0.f, lse = kNegInf;
  if (M != kNegInf) {
    const float fo = fast_exp2(mref - M);  // 0 when no selected row contributed
    lt = l * fo + fast_exp2(z2 - M);
    scale_o = (lt > 0.f) ? fo / lt : 0.f;
    lse = (M + __log2f(lt)) * kLn2;
  }
  // KV-only convention: ln sum_u e^{s_u}, the sink left out (-inf without rows)
  if (a.lse_kv) lse = (mref == kNegInf || !(l > 0.f)) ? kNegInf : (mref + __log2f(l)) * kLn2;
  uint16_t* Oh = (uint16_t*)a.O + ((size_t)t * H + head) * DV;
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    u32x2 w;
    w[0] = E::pack2(oacc[m][0] * scale_o, oacc[m][1] * scale_o);
    w[1] = E::pack2(oacc[m][2] * scale_o, oacc[m][3] * scale_o);
    *(u32x2*)(Oh + 16 * m + 4 * G) = w;
  }
  if (G == 0) a.LSE[(size_t)t * H + head] = lse;
}

// ------------------------------------------------------------------ backward
// The sink-inclusive LSE of (token, head) from the saved one: a KV-only LSE is
// first combined with the sink logit, LSE_total = logaddexp(LSE_kv, z)
// ([P5] section 7.2); every reconstructed probability uses LSE_total.
__device__ __forceinline__ float lse_total(const SparseArgs& a, size_t th, int head) {
  const float lse = a.LSE[th];
  if (!a.lse_kv || !a.sink) return lse;
  const float z = a.sink[head];
  const float hi = fmaxf(lse, z), lo = fminf(lse, z);
  return (lo == kNegInf) ? hi : hi + log1pf(expf(lo - hi));
}

// D[t][h] = dO . O ; zero the fp32 dKV accumulator
template <class E>
__global__ __launch_bounds__(256) void sparse_bwd_prep_kernel(const SparseArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const long long row = (long long)blockIdx.x * 4 + (tid >> 6);  // (t, h) pair
  if (row < (long long)a.Tq * sp::H) {
    const uint16_t* g = (const uint16_t*)a.dO + row * sp::DV + 8 * lane;
    const uint16_t* o = (const uint16_t*)a.O + row * sp::DV + 8 * lane;
    const u32x4 gw = *(const u32x4*)g, ow = *(const u32x4*)o;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += E::lo(gw[k]) * E::lo(ow[k]) + E::hi(gw[k]) * E::hi(ow[k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) a.Dws[row] = acc;
  }
  // the accumulator: fp32, or int64 fixed point in the deterministic mode
  const long long n4 = (long long)a.Tkv * sp::DQK / 4 * (a.det ? 2 : 1);
  for (long long k = (long long)blockIdx.x * 256 + tid; k < n4; k += (long long)gridDim.x * 256)
    ((f32x4*)a.dKVws)[k] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Shared recompute for both backward kernels: P^T and dS^T of one tile for this
// wave's 16 heads (k-slot order of tile_cols_tr), as packed MFMA operands.
template <class E>
__device__ __forceinline__ void recompute_p_ds(const char ETS_LDS* kt, const typename E::vec8* qreg,
                                               const typename E::vec8* greg, const RowOps16<sp::ROWB>& rops,
                                               int lane, int u0, int L,
                                               float sl2, float lse2, float Dv, typename E::vec8& pb,
                                               typename E::vec8& db) {
  using namespace sp;
  const int G = lane >> 4;
  f32x4 s[2];
  scores<E>(kt, qreg, rops, s);
  f32x4 dp[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) dp[mb][r] = 0.f;
  // dP^T = V_tile dO_h^T : A = V rows (keys) of the tile
#pragma unroll
  for (int kk = 0; kk < KSV; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const typename E::vec8 va = as_vec8<E>(lds_b128(kt, rops.off(16 * mb, kk)));
      dp[mb] = E::mfma16(va, greg[kk], dp[mb]);
    }
  }
  float p[2][4], ds[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = fast_exp2(fmaf(s[mb][r], sl2, -lse2));
      if (u0 + 16 * mb + 4 * G + r >= L) v = 0.f;
      p[mb][r] = v;
      ds[mb][r] = v * (dp[mb][r] - Dv);
    }
  pb = as_vec8<E>(u32x4{E::pack2(p[0][0], p[0][1]), E::pack2(p[0][2], p[0][3]), E::pack2(p[1][0], p[1][1]),
                        E::pack2(p[1][2], p[1][3])});
  db = as_vec8<E>(u32x4{E::pack2(ds[0][0], ds[0][1]), E::pack2(ds[0][2], ds[0][3]),
                        E::pack2(ds[1][0], ds[1][1]), E::pack2(ds[1][2], ds[1][3])});
}

// dQ (private per token) and the per-token sink-gradient terms
template <class E>
__global__ __launch_bounds__(256, 1) void sparse_bwd_dq_kernel(const SparseArgs a, float* dsink_part) {
  using namespace sp;
  typedef typename E::vec8 vec8;
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  char ETS_LDS* smem = (char ETS_LDS*)smem_dyn;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int G = lane >> 4, l16 = lane & 15;
  const int t = blockIdx.x;
  const int head = 16 * wave + l16;
  const uint16_t* KV = (const uint16_t*)a.KV;
  const int32_t* idx_t = a.idx + (size_t)t * a.topk;
  const int L = sel_count(a, t);
  const size_t th = (size_t)t * H + head;

  vec8 qreg[KSQ], greg[KSV];
  const uint16_t* Qh = (const uint16_t*)a.Q + th * DQK;
  const uint16_t* Gh = (const uint16_t*)a.dO + th * DV;
#pragma unroll
  for (int kk = 0; kk < KSQ; ++kk) qreg[kk] = as_vec8<E>(*(const u32x4*)(Qh + 32 * kk + 8 * G));
#pragma unroll
  for (int kk = 0; kk < KSV; ++kk) greg[kk] = as_vec8<E>(*(const u32x4*)(Gh + 32 * kk + 8 * G));
  const float lse = lse_total(a, th, head);
  const float lse2 = (lse == kNegInf) ? 0.f : lse * kLog2e;
  const float Dv = a.Dws[th];

  f32x4 dq[MQ];
#pragma unroll
  for (int m = 0; m < MQ; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) dq[m][r] = 0.f;

  Gather gat;
  const RowOps16<ROWB> rops(lane);
  const TrOps16<ROWB> tops(lane);
  const int ntiles = (L + BK - 1) / BK;
  if (ntiles > 0) {
    gat.start(KV, idx_t, L, a.Tkv, ntiles, smem, tid);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int u0 = it * BK;
    gat.next(KV, idx_t, L, a.Tkv, it, ntiles, tid);
    const char ETS_LDS* kt = smem + (it & 1) * TILEB;
    vec8 pb, db;
    recompute_p_ds<E>(kt, qreg, greg, rops, lane, u0, L, a.scale_log2, lse2, Dv, pb, db);
    // dQ^T += K^T dS^T
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const vec8 ka = as_vec8<E>(tops.read(kt, m));
      dq[m] = E::mfma16(ka, db, dq[m]);
    }
    if (it + 1 < ntiles) gat.stash(smem + ((it + 1) & 1) * TILEB, tid);
    __syncthreads();
  }
  uint16_t* dQh = (uint16_t*)a.dQ + th * DQK;
  const float al = a.scale;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    u32x2 w;
    w[0] = E::pack2(dq[m][0] * al, dq[m][1] * al);
    w[1] = E::pack2(dq[m][2] * al, dq[m][3] * al);
    *(u32x2*)(dQh + 16 * m + 4 * G) = w;
  }
  if (a.sink && G == 0) {
    const float psink = (lse == kNegInf) ? 0.f : fast_exp2(a.sink[head] * kLog2e - lse2);
    dsink_part[th] = -psink * Dv;
  }
}

// dKV: contributions of one token, all 64 heads, into the fp32 accumulator
template <class E, bool DET>
__global__ __launch_bounds__(256, 1) void sparse_bwd_dkv_kernel(const SparseArgs a) {
  using namespace sp;
  typedef typename E::vec8 vec8;
  constexpr int PB = BK * H * 2;          // one [32 keys][64 heads] 16-bit matrix
  constexpr int MW = (DQK / 4) / 16;      // 16-column blocks per wave (9)
  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];
  char ETS_LDS* smem = (char ETS_LDS*)smem_dyn;
  char ETS_LDS* pbuf = smem + 2 * TILEB;  // P  [key][head]
  char ETS_LDS* dbuf = pbuf + PB;         // dS [key][head]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int G = lane >> 4, l16 = lane & 15;
  const int t = blockIdx.x;
  const int head = 16 * wave + l16;
  const uint16_t* KV = (const uint16_t*)a.KV;
  const int32_t* idx_t = a.idx + (size_t)t * a.topk;
  const int L = sel_count(a, t);
  const size_t th = (size_t)t * H + head;
  const int c0w = wave * (DQK / 4);       // first output column of this wave

  vec8 qreg[KSQ], greg[KSV];
  {
    const uint16_t* Qh = (const uint16_t*)a.Q + th * DQK;
    const uint16_t* Gh = (const uint16_t*)a.dO + th * DV;
#pragma unroll
    for (int kk = 0; kk < KSQ; ++kk) qreg[kk] = as_vec8<E>(*(const u32x4*)(Qh + 32 * kk + 8 * G));
#pragma unroll
    for (int kk = 0; kk < KSV; ++kk) greg[kk] = as_vec8<E>(*(const u32x4*)(Gh + 32 * kk + 8 * G));
  }
  const float lse = lse_total(a, th, head);
  const float lse2 = (lse == kNegInf) ? 0.f : lse * kLog2e;
  const float Dv = a.Dws[th];

  // Q^T and dO^T column slices of this wave for all 64 heads, as A operands
  // (row = output column, k-slots = heads 32ks + 8G .. +7), staged through LDS
  vec8 qt[MW][2], gt[MW][2];
  {
    const uint16_t* Qt = (const uint16_t*)a.Q + (size_t)t * H * DQK;
    for (int c = tid; c < H * CPR; c += 256) {
      const int r = c / CPR, cc = c % CPR;
      lds_st128(smem, toff<ROWB>(r, 8 * cc), *(const u32x4*)(Qt + (size_t)r * DQK + 8 * cc));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        qt[m][ks] = as_vec8<E>(lds_tr8<ROWB>(smem, 32 * ks + 8 * G, 32 * ks + 8 * G + 4, c0w + 16 * m, lane));
    __syncthreads();
    const uint16_t* Gt = (const uint16_t*)a.dO + (size_t)t * H * DV;
    for (int c = tid; c < H * (DV / 8); c += 256) {
      const int r = c / (DV / 8), cc = c % (DV / 8);
      lds_st128(smem, toff<ROWB>(r, 8 * cc), *(const u32x4*)(Gt + (size_t)r * DV + 8 * cc));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int col = c0w + 16 * m;
        gt[m][ks] = (col < DV) ? as_vec8<E>(lds_tr8<ROWB>(smem, 32 * ks + 8 * G, 32 * ks + 8 * G + 4, col, lane))
                               : as_vec8<E>(u32x4{0, 0, 0, 0});
      }
    __syncthreads();
  }

  Gather gat;
  const RowOps16<ROWB> rops(lane);
  const TrOps16<ROWB> tops(lane);
  const int ntiles = (L + BK - 1) / BK;
  if (ntiles > 0) {
    gat.start(KV, idx_t, L, a.Tkv, ntiles, smem, tid);
  }
  __syncthreads();
  float* ws = a.dKVws;
  const float al = a.scale;
  for (int it = 0; it < ntiles; ++it) {
    const int u0 = it * BK;
    gat.next(KV, idx_t, L, a.Tkv, it, ntiles, tid);
    const char ETS_LDS* kt = smem + (it & 1) * TILEB;
    vec8 pb, db;
    recompute_p_ds<E>(kt, qreg, greg, rops, lane, u0, L, a.scale_log2, lse2, Dv, pb, db);
    // P and dS of this wave's heads -> LDS [key][head]
    {
      const u32x4 pw = __builtin_bit_cast(u32x4, pb), dw = __builtin_bit_cast(u32x4, db);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * (e >> 2) + 4 * G + (e & 3);
        const int off = key * (H * 2) + head * 2;
        const uint16_t pv = (uint16_t)((e & 1) ? (pw[e >> 1] >> 16) : (pw[e >> 1] & 0xffffu));
        const uint16_t dv = (uint16_t)((e & 1) ? (dw[e >> 1] >> 16) : (dw[e >> 1] & 0xffffu));
        *(uint16_t ETS_LDS*)(pbuf + off) = pv;
        *(uint16_t ETS_LDS*)(dbuf + off) = dv;
      }
    }
    __syncthreads();
    // dKV[keys][cols of this wave] = alpha dS^T Q + P^T dO  (contraction over the 64 heads);
    // the accumulator holds 16 consecutive columns of one key per 16 lanes,
    // so each atomic instruction updates 4 rows x 64 contiguous bytes
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {       // 16-key blocks of the tile
      vec8 ap[2], ad[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int off = (16 * nb + l16) * (H * 2) + (32 * ks + 8 * G) * 2;
        ap[ks] = as_vec8<E>(*(const u32x4 ETS_LDS*)(pbuf + off));
        ad[ks] = as_vec8<E>(*(const u32x4 ETS_LDS*)(dbuf + off));
      }
      int jrow[4];
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // rows outside [0, Tkv) get no update
        const int slot = u0 + 16 * nb + 4 * G + r;
        jrow[r] = slot < L ? idx_t[slot] : -1;
        valid[r] = (unsigned)jrow[r] < (unsigned)a.Tkv;
      }
#pragma unroll
      for (int m = 0; m < MW; ++m) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          acc = E::mfma16(ad[ks], qt[m][ks], acc);
          if (c0w + 16 * m < DV) accv = E::mfma16(ap[ks], gt[m][ks], accv);
        }
        const int col = c0w + 16 * m + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (valid[r]) {
            const float v = fmaf(acc[r], al, accv[r]);
            if constexpr (DET) {
              // integer adds commute exactly: the sum is the same in any order
              const long long q = __float2ll_rn(v * kFix);
              atomicAdd((unsigned long long*)ws + (size_t)jrow[r] * DQK + col, (unsigned long long)q);
            } else {
              atomicAdd(ws + (size_t)jrow[r] * DQK + col, v);
            }
          }
      }
    }
    if (it + 1 < ntiles) gat.stash(smem + ((it + 1) & 1) * TILEB, tid);
    __syncthreads();
  }
}

// dKV fp32 -> storage dtype; dSink[h] = sum over tokens (fixed order)
template <class E, bool DET>
__global__ __launch_bounds__(256) void sparse_bwd_finalize_kernel(const SparseArgs a, const float* dsink_part) {
  const long long n2 = (long long)a.Tkv * sp::DQK / 2;
  for (long long k = (long long)blockIdx.x * 256 + threadIdx.x; k < n2; k += (long long)gridDim.x * 256) {
    if constexpr (DET) {
      const long long* q = (const long long*)a.dKVws + 2 * k;
      ((uint32_t*)a.dKV)[k] = E::pack2((float)((double)q[0] * kFixInv), (float)((double)q[1] * kFixInv));
    } else {
      const f32x2 v = ((const f32x2*)a.dKVws)[k];
      ((uint32_t*)a.dKV)[k] = E::pack2(v[0], v[1]);
    }
  }
  if (a.sink && blockIdx.x < sp::H) {
    __shared__ float red[256];
    float acc = 0.f;
    for (int t = threadIdx.x; t < a.Tq; t += 256) acc += dsink_part[(size_t)t * sp::H + blockIdx.x];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
      __syncthreads();
    }
    if (threadIdx.x == 0) a.dSink[blockIdx.x] = red[0];
  }
}

// ------------------------------------------------------------------ launch
// Dynamic LDS above 64 KB (up to the 160 KB of a CDNA4 CU) needs no opt-in.
template <class E>
static int launch_fwd_e(const SparseArgs& a, hipStream_t st) {
  ETS_TRY(launch(sparse_fwd_kernel<E>, dim3(a.Tq), dim3(256), sp::SMEM, st, a));
  return 0;
}

template <class E>
static int launch_bwd_e(const SparseArgs& a, hipStream_t st) {
  constexpr int SMEM_DKV = 2 * sp::TILEB + 2 * sp::BK * sp::H * 2;
  float* dsink_part = a.dsink_part;
  const int prep_blocks = (a.Tq * sp::H + 3) / 4;
  ETS_TRY(launch(sparse_bwd_prep_kernel<E>, dim3(prep_blocks), dim3(256), 0, st, a));
  ETS_TRY(launch(sparse_bwd_dq_kernel<E>, dim3(a.Tq), dim3(256), sp::SMEM, st, a, dsink_part));
  if (a.det) ETS_TRY(launch(sparse_bwd_dkv_kernel<E, true>, dim3(a.Tq), dim3(256), SMEM_DKV, st, a));
  else ETS_TRY(launch(sparse_bwd_dkv_kernel<E, false>, dim3(a.Tq), dim3(256), SMEM_DKV, st, a));
  const long long n2 = (long long)a.Tkv * sp::DQK / 2;
  long long blocks = (n2 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < sp::H) blocks = sp::H;
  if (a.det) ETS_TRY(launch(sparse_bwd_finalize_kernel<E, true>, dim3((unsigned)blocks), dim3(256), 0, st, a, dsink_part));
  else ETS_TRY(launch(sparse_bwd_finalize_kernel<E, false>, dim3((unsigned)blocks), dim3(256), 0, st, a, dsink_part));
  return 0;
}

int launch_sparse_fwd(const SparseArgs& a, Dt dt, void* stream) {
  return dt == Dt::BF16 ? launch_fwd_e<BF16>(a, (hipStream_t)stream) : launch_fwd_e<F16>(a, (hipStream_t)stream);
}

int launch_sparse_bwd(const SparseArgs& a, Dt dt, void* stream) {
  return dt == Dt::BF16 ? launch_bwd_e<BF16>(a, (hipStream_t)stream) : launch_bwd_e<F16>(a, (hipStream_t)stream);
}

}  // namespace ets
