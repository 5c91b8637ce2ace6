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
//   prep  D_i from G and Y (fp32, into the workspace);
//   dkdv  key-major: a workgroup owns 128 keys of one K/V head, keeps its K
//         and V rows in registers as MFMA B operands, and walks every query
//         tile (and every query head of the group) that can see them; S = Q K^T
//         and dP = G V^T put keys along lanes, so P and gamma feed
//         dV^T += G^T P and dK^T += Q^T gamma directly, with G^T and Q^T read
//         by LDS transpose reads.  No atomics.
//   dq    query-major: the forward layout (queries along lanes); recomputes
//         S^T and dP^T and accumulates dQ^T += K^T gamma^T.  No atomics.
#include "device.hpp"

namespace ets {

// --------------------------------------------------------------------- prep
// D_i = G_i . Y_i and the base-2 LSE, LSE_i log2(e) (+inf for a row with an
// empty allowed set, so every recomputed weight of it is 0).  The 64 rows after
// the last are filled with D = 0, LSE2 = +inf: tiles of 64 rows may read them.
template <class E, int D>
__global__ __launch_bounds__(256) void dense_bwd_prep_kernel(const DenseArgs a, int rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int row = t / LPR, part = t % LPR;
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
    a.Dws[row] = acc;
    a.Lws[row] = l2;
  }
}

// Keep bits (4 query rows i0..i0+3, this lane's key j) for the key-major
// layout.  The four lanes of a quad hold keys 4k..4k+3; lane u of the quad
// draws the Philox block of query row i0 + u (which decides all four keys) and
// the quad exchanges the decisions, so each block is drawn exactly once.
__device__ __forceinline__ unsigned keep4_rows(const DropArgs& d, int lane_bh, int i0, int j) {
  const int u = j & 3;
  const unsigned nib = keep4(d, lane_bh, i0 + u, j & ~3);
  int v = (int)(nib << (4 * u));
  v |= __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  v |= __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  unsigned out = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) out |= (((unsigned)v >> (4 * r + u)) & 1u) << r;
  return out;
}

// --------------------------------------------------------------------- dK, dV
template <class E, int D, int MK, bool DROP>
__global__ __launch_bounds__(256, 1) void dense_bwd_dkdv_kernel(const DenseArgs a) {
  constexpr int BQ = 64;             // query rows per tile
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BQ * ROWB;
  constexpr int STAGEB = 2 * TILEB + 2 * BQ * 4;  // Q, G tiles + LSE2, D
  typedef typename E::vec8 vec8;

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * STAGEB];
  char ETS_LDS* smem = (char ETS_LDS*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h32 = lane >> 5, l32 = lane & 31;
  const int nq = a.nq, nk = a.nk;
  const int BG = a.B * a.Hkv;
  const int kb = (int)(blockIdx.x / BG), bg = (int)(blockIdx.x % BG);  // key block (heavy first), (batch, kv head)
  const int b = bg / a.Hkv, g = bg % a.Hkv, grp = a.H / a.Hkv;
  const int k0 = kb * 128, kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;

  const uint16_t* Kp = (const uint16_t*)a.K + (size_t)bg * nk * D;
  const uint16_t* Vp = (const uint16_t*)a.V + (size_t)bg * nk * D;

  // this wave's 32 keys as B operands of S = Q K^T and dP = G V^T
  vec8 kreg[KS], vreg[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
    if (key < nk) {
      kv = *(const u32x4*)(Kp + (size_t)key * D + 16 * kk + 8 * h32);
      vv = *(const u32x4*)(Vp + (size_t)key * D + 16 * kk + 8 * h32);
    }
    kreg[kk] = as_vec8<E>(kv);
    vreg[kk] = as_vec8<E>(vv);
  }

  f32x16 dk[MD], dv[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[md][r] = 0.f; dv[md][r] = 0.f; }

  // query-tile range that can see keys [k0, k0 + 127]
  const int klast = min(k0 + 127, nk - 1);
  int qt_lo = 0, qt_hi = (nq - 1) / BQ;
  if (a.mask.causal) qt_lo = k0 / BQ;
  if (a.mask.window > 0) qt_hi = min(qt_hi, (klast + a.mask.window - 1) / BQ);
  const int n_qt = qt_hi - qt_lo + 1;
  const int total = (n_qt > 0) ? n_qt * grp : 0;  // (head, q-tile) steps

  auto wg_nonempty = [&](int step) {
    const int qt = qt_lo + step % n_qt;
    return classify<MK>(a.mask, qt * BQ, qt * BQ + BQ - 1, k0, k0 + 127, nq, nk) != kEmpty;
  };
  auto next_step = [&](int s) {
    for (++s; s < total; ++s)
      if (wg_nonempty(s)) return s;
    return -1;
  };
  // Q and G tiles straight to LDS; LSE2 and D (64 floats each) by one
  // half-wave instruction (the workspace holds 64 padding rows after the last)
  auto load = [&](int s, int st) {
    const int h = g * grp + s / n_qt, qt = qt_lo + s % n_qt;
    const size_t lane_off = (size_t)(b * a.H + h) * nq;
    char ETS_LDS* qt_ = smem + st * STAGEB;
    tile_to_lds<BQ, D, 4>(qt_, (const uint16_t*)a.Q + lane_off * D, qt * BQ, nq - 1, wave, lane);
    tile_to_lds<BQ, D, 4>(qt_ + TILEB, (const uint16_t*)a.G + lane_off * D, qt * BQ, nq - 1, wave, lane);
    if (wave == 0 && lane < 32) {
      const float* src = (lane < 16 ? a.Lws : a.Dws) + lane_off + qt * BQ + 4 * (lane & 15);
      __builtin_amdgcn_global_load_lds(src, (void ETS_LDS*)(qt_ + 2 * TILEB), 16, 0, 0);
    }
  };

  int s = (total > 0) ? (wg_nonempty(0) ? 0 : next_step(0)) : -1;
  int st = 0;
  if (s >= 0) load(s, 0);
  wait_vm();
  __syncthreads();
  const float sl2 = a.scale_log2;
  const RowOps32<ROWB> rops(lane);
  const TrOps32<ROWB> tops(lane);

  while (s >= 0) {
    const int nxt = next_step(s);
    if (nxt >= 0) load(nxt, st ^ 1);
    const int h = g * grp + s / n_qt, qt = qt_lo + s % n_qt, qb0 = qt * BQ;
    const int lane_bh = b * a.H + h;
    const char ETS_LDS* qt_ = smem + st * STAGEB;
    const char ETS_LDS* gt_ = qt_ + TILEB;
    const float ETS_LDS* ls = (const float ETS_LDS*)(gt_ + TILEB);
    const float ETS_LDS* ds = ls + BQ;
    const int cinfo = classify<MK>(a.mask, qb0, qb0 + BQ - 1, kw0, kw0 + 31, nq, nk);
    const int cls = cinfo & kClassMask;
    const bool cbm = (cinfo & kCheckBlockMask) != 0;

    if (cls != kEmpty) {
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {  // 32 query rows at a time
        f32x16 sc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
        // Q and G operands read one k-step ahead of their MFMAs
        vec8 qa[2], ga[2];
        qa[0] = as_vec8<E>(lds_b128(qt_, rops.off(32 * mq, 0)));
        ga[0] = as_vec8<E>(lds_b128(gt_, rops.off(32 * mq, 0)));
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          if (kk + 1 < KS) {
            qa[(kk + 1) & 1] = as_vec8<E>(lds_b128(qt_, rops.off(32 * mq, kk + 1)));
            ga[(kk + 1) & 1] = as_vec8<E>(lds_b128(gt_, rops.off(32 * mq, kk + 1)));
          }
          sc = E::mfma32(qa[kk & 1], kreg[kk], sc);
          dp = E::mfma32(ga[kk & 1], vreg[kk], dp);
        }
        // S and dP: lane = key, entries r = query rows 32mq + 8(r/4) + 4h32 + r%4
        uint32_t pw[8], gw[8];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qr = 32 * mq + 8 * g4 + 4 * h32;  // first of 4 query rows in the tile
          const f32x4 l4 = *(const f32x4 ETS_LDS*)(ls + qr);
          const f32x4 d4 = *(const f32x4 ETS_LDS*)(ds + qr);
          unsigned allow = 0xFu, keep = 0xFu;
          if (cls == kPartial) allow = allowed4_rows<MK>(a.mask, qb0 + qr, key, nq, nk, cbm);
          if constexpr (DROP) keep = keep4_rows(a.drop, lane_bh, qb0 + qr, key);
          float pk[4], gm[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = fast_exp2(fmaf(sc[4 * g4 + r], sl2, -l4[r]));
            float dpv = dp[4 * g4 + r];
            bool kp = true;
            if constexpr (DROP) {
              kp = (keep >> r) & 1u;
              dpv = kp ? dpv * a.drop.inv_keep : 0.f;
            }
            const bool al = (allow >> r) & 1u;
            pk[r] = (al && kp) ? pv : 0.f;
            gm[r] = al ? pv * (dpv - d4[r]) : 0.f;
          }
          pw[2 * g4] = E::pack2(pk[0], pk[1]);
          pw[2 * g4 + 1] = E::pack2(pk[2], pk[3]);
          gw[2 * g4] = E::pack2(gm[0], gm[1]);
          gw[2 * g4 + 1] = E::pack2(gm[2], gm[3]);
        }
        // dV^T += G^T P~, dK^T += Q^T gamma over these 32 queries (2 k-steps);
        // transpose operands read one step ahead
        vec8 pb[2], gb[2];
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const int o = 4 * kk2;
          pb[kk2] = as_vec8<E>(u32x4{pw[o], pw[o + 1], pw[o + 2], pw[o + 3]});
          gb[kk2] = as_vec8<E>(u32x4{gw[o], gw[o + 1], gw[o + 2], gw[o + 3]});
        }
        constexpr int NT = 2 * MD;
        vec8 gta[2], qta[2];
        gta[0] = as_vec8<E>(tops.read(gt_, 32 * mq, 0));
        qta[0] = as_vec8<E>(tops.read(qt_, 32 * mq, 0));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int kk2 = t / MD, md = t % MD;
          if (t + 1 < NT) {
            const int R1 = 32 * mq + 16 * ((t + 1) / MD), md1 = (t + 1) % MD;
            gta[(t + 1) & 1] = as_vec8<E>(tops.read(gt_, R1, md1));
            qta[(t + 1) & 1] = as_vec8<E>(tops.read(qt_, R1, md1));
          }
          dv[md] = E::mfma32(gta[t & 1], pb[kk2], dv[md]);
          dk[md] = E::mfma32(qta[t & 1], gb[kk2], dk[md]);
        }
      }
    }

    wait_vm();
    __syncthreads();
    st ^= 1;
    s = nxt;
  }

  // ---- epilogue: dK = c dK^T, dV = (1/(1-rho)) dV^T; lane holds one key
  if (key < nk) {
    uint16_t* dKp = (uint16_t*)a.dK + (size_t)bg * nk * D + (size_t)key * D;
    uint16_t* dVp = (uint16_t*)a.dV + (size_t)bg * nk * D + (size_t)key * D;
    const float ck = a.scale;
    const float cv = DROP ? a.drop.inv_keep : 1.f;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * md + 8 * g4 + 4 * h32;
        u32x2 wk, wv;
        wk[0] = E::pack2(dk[md][4 * g4] * ck, dk[md][4 * g4 + 1] * ck);
        wk[1] = E::pack2(dk[md][4 * g4 + 2] * ck, dk[md][4 * g4 + 3] * ck);
        wv[0] = E::pack2(dv[md][4 * g4] * cv, dv[md][4 * g4 + 1] * cv);
        wv[1] = E::pack2(dv[md][4 * g4 + 2] * cv, dv[md][4 * g4 + 3] * cv);
        *(u32x2*)(dKp + col) = wk;
        *(u32x2*)(dVp + col) = wv;
      }
  }
}

// --------------------------------------------------------------------- dQ
template <class E, int D, int MK, bool DROP>
__global__ __launch_bounds__(256, 1) void dense_bwd_dq_kernel(const DenseArgs a, int n_qtiles) {
  constexpr int BK = 64;
  constexpr int NQW = 32;
  constexpr int BQ = 4 * NQW;
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BK * ROWB;
  typedef typename E::vec8 vec8;

  __shared__ __attribute__((aligned(16))) char smem_raw[4 * TILEB];
  char ETS_LDS* smem = (char ETS_LDS*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h32 = lane >> 5, l32 = lane & 31;
  const int BH = a.B * a.H;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
  const int nq = a.nq, nk = a.nk;
  const int q0 = qt * BQ, qw0 = q0 + wave * NQW;
  const int q = qw0 + l32;

  const uint16_t* Qp = (const uint16_t*)a.Q + (size_t)bh * nq * D;
  const uint16_t* Gp = (const uint16_t*)a.G + (size_t)bh * nq * D;
  const uint16_t* Kp = (const uint16_t*)a.K + (size_t)(b * a.Hkv + g) * nk * D;
  const uint16_t* Vp = (const uint16_t*)a.V + (size_t)(b * a.Hkv + g) * nk * D;

  vec8 qreg[KS], greg[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4 qv = u32x4{0, 0, 0, 0}, gv = u32x4{0, 0, 0, 0};
    if (q < nq) {
      qv = *(const u32x4*)(Qp + (size_t)q * D + 16 * kk + 8 * h32);
      gv = *(const u32x4*)(Gp + (size_t)q * D + 16 * kk + 8 * h32);
    }
    qreg[kk] = as_vec8<E>(qv);
    greg[kk] = as_vec8<E>(gv);
  }
  const float lse2 = (q < nq) ? a.Lws[(size_t)bh * nq + q] : __builtin_huge_valf();
  const float dval = (q < nq) ? a.Dws[(size_t)bh * nq + q] : 0.f;

  f32x16 dq[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[md][r] = 0.f;

  const int qlast = min(q0 + BQ, nq) - 1;
  int jt_lo = 0, jt_hi = (nk - 1) / BK;
  if (a.mask.causal) jt_hi = min(jt_hi, qlast / BK);
  if (a.mask.window > 0) jt_lo = max(0, (q0 - a.mask.window + 1) / BK);
  auto wg_nonempty = [&](int jt) {
    return classify<MK>(a.mask, q0, q0 + BQ - 1, jt * BK, jt * BK + BK - 1, nq, nk) != kEmpty;
  };
  auto next_tile = [&](int jt) {
    for (++jt; jt <= jt_hi; ++jt)
      if (wg_nonempty(jt)) return jt;
    return -1;
  };

  auto load = [&](int jt, int stage) {
    char ETS_LDS* kt = smem + stage * 2 * TILEB;
    tile_to_lds<BK, D, 4>(kt, Kp, jt * BK, nk - 1, wave, lane);
    tile_to_lds<BK, D, 4>(kt + TILEB, Vp, jt * BK, nk - 1, wave, lane);
  };

  int jt = (jt_lo <= jt_hi && wg_nonempty(jt_lo)) ? jt_lo : next_tile(jt_lo);
  int stage = 0;
  if (jt >= 0) load(jt, 0);
  wait_vm();
  __syncthreads();
  const float sl2 = a.scale_log2;
  const RowOps32<ROWB> rops(lane);
  const TrOps32<ROWB> tops(lane);

  while (jt >= 0) {
    const int nxt = next_tile(jt);
    if (nxt >= 0) load(nxt, stage ^ 1);
    const char ETS_LDS* kt = smem + stage * 2 * TILEB;
    const char ETS_LDS* vt = kt + TILEB;
    const int j0 = jt * BK;
    const int cinfo = classify<MK>(a.mask, qw0, qw0 + NQW - 1, j0, j0 + BK - 1, nq, nk);
    const int cls = cinfo & kClassMask;
    const bool cbm = (cinfo & kCheckBlockMask) != 0;

    if (cls != kEmpty) {
      f32x16 sc[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) { sc[mb][r] = 0.f; dp[mb][r] = 0.f; }
      // K and V operands read one k-step ahead of their MFMAs
      vec8 ka[2][2], va[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        ka[0][mb] = as_vec8<E>(lds_b128(kt, rops.off(32 * mb, 0)));
        va[0][mb] = as_vec8<E>(lds_b128(vt, rops.off(32 * mb, 0)));
      }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            ka[(kk + 1) & 1][mb] = as_vec8<E>(lds_b128(kt, rops.off(32 * mb, kk + 1)));
            va[(kk + 1) & 1][mb] = as_vec8<E>(lds_b128(vt, rops.off(32 * mb, kk + 1)));
          }
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          sc[mb] = E::mfma32(ka[kk & 1][mb], qreg[kk], sc[mb]);
          dp[mb] = E::mfma32(va[kk & 1][mb], greg[kk], dp[mb]);
        }
      }
      uint32_t gw[2][8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int jj = j0 + 32 * mb + 8 * g4 + 4 * h32;
          unsigned allow = 0xFu, keep = 0xFu;
          if (cls == kPartial) allow = allowed4<MK>(a.mask, q, jj, nq, nk, cbm);
          if constexpr (DROP) keep = keep4(a.drop, bh, q, jj);
          float gm[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = fast_exp2(fmaf(sc[mb][4 * g4 + r], sl2, -lse2));
            float dpv = dp[mb][4 * g4 + r];
            if constexpr (DROP) dpv = ((keep >> r) & 1u) ? dpv * a.drop.inv_keep : 0.f;
            gm[r] = ((allow >> r) & 1u) ? pv * (dpv - dval) : 0.f;
          }
          gw[mb][2 * g4] = E::pack2(gm[0], gm[1]);
          gw[mb][2 * g4 + 1] = E::pack2(gm[2], gm[3]);
        }
      // dQ^T += K^T gamma^T (K^T operands read one step ahead)
      vec8 gbs[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int mb = ks >> 1, o = (ks & 1) * 4;
        gbs[ks] = as_vec8<E>(u32x4{gw[mb][o], gw[mb][o + 1], gw[mb][o + 2], gw[mb][o + 3]});
      }
      constexpr int NT = 4 * MD;
      vec8 kta[2];
      kta[0] = as_vec8<E>(tops.read(kt, 0, 0));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int ks = t / MD, md = t % MD;
        if (t + 1 < NT) kta[(t + 1) & 1] = as_vec8<E>(tops.read(kt, 16 * ((t + 1) / MD), (t + 1) % MD));
        dq[md] = E::mfma32(kta[t & 1], gbs[ks], dq[md]);
      }
    }

    wait_vm();
    __syncthreads();
    stage ^= 1;
    jt = nxt;
  }

  if (q < nq) {
    uint16_t* dQp = (uint16_t*)a.dQ + (size_t)bh * nq * D + (size_t)q * D;
    const float c = a.scale;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * md + 8 * g4 + 4 * h32;
        u32x2 w;
        w[0] = E::pack2(dq[md][4 * g4] * c, dq[md][4 * g4 + 1] * c);
        w[1] = E::pack2(dq[md][4 * g4 + 2] * c, dq[md][4 * g4 + 3] * c);
        *(u32x2*)(dQp + col) = w;
      }
  }
}

template <class E, int D>
static hipError_t launch_dkdv(const DenseArgs& a, dim3 g, hipStream_t st) {
  const int mk = mask_kind(a.mask);
  if (a.drop.enabled) {
    if (mk == kArith) return launch((dense_bwd_dkdv_kernel<E, D, kArith, true>), g, dim3(256), 0, st, a);
    if (mk == kBlock) return launch((dense_bwd_dkdv_kernel<E, D, kBlock, true>), g, dim3(256), 0, st, a);
    return launch((dense_bwd_dkdv_kernel<E, D, kDenseM, true>), g, dim3(256), 0, st, a);
  }
  if (mk == kArith) return launch((dense_bwd_dkdv_kernel<E, D, kArith, false>), g, dim3(256), 0, st, a);
  if (mk == kBlock) return launch((dense_bwd_dkdv_kernel<E, D, kBlock, false>), g, dim3(256), 0, st, a);
  return launch((dense_bwd_dkdv_kernel<E, D, kDenseM, false>), g, dim3(256), 0, st, a);
}

template <class E, int D>
static hipError_t launch_dq(const DenseArgs& a, dim3 g, hipStream_t st, int n_qtiles) {
  const int mk = mask_kind(a.mask);
  if (a.drop.enabled) {
    if (mk == kArith) return launch((dense_bwd_dq_kernel<E, D, kArith, true>), g, dim3(256), 0, st, a, n_qtiles);
    if (mk == kBlock) return launch((dense_bwd_dq_kernel<E, D, kBlock, true>), g, dim3(256), 0, st, a, n_qtiles);
    return launch((dense_bwd_dq_kernel<E, D, kDenseM, true>), g, dim3(256), 0, st, a, n_qtiles);
  }
  if (mk == kArith) return launch((dense_bwd_dq_kernel<E, D, kArith, false>), g, dim3(256), 0, st, a, n_qtiles);
  if (mk == kBlock) return launch((dense_bwd_dq_kernel<E, D, kBlock, false>), g, dim3(256), 0, st, a, n_qtiles);
  return launch((dense_bwd_dq_kernel<E, D, kDenseM, false>), g, dim3(256), 0, st, a, n_qtiles);
}

template <class E, int D>
static int launch_bwd_t(const DenseArgs& a, void* stream, int phases) {
  hipStream_t st = (hipStream_t)stream;
  if (phases & 1) {
    const int rows = a.B * a.H * a.nq;
    const int prep_threads = (rows + 64) * (D / 8);
    ETS_TRY(launch((dense_bwd_prep_kernel<E, D>), dim3((prep_threads + 255) / 256), dim3(256), 0, st, a, rows));
  }
  const int n_kblocks = (a.nk + 127) / 128;
  dim3 gk(n_kblocks * a.B * a.Hkv);
  const int n_qtiles = (a.nq + 127) / 128;
  dim3 gq(n_qtiles * a.B * a.H);
  if (phases & 2) ETS_TRY((launch_dkdv<E, D>(a, gk, st)));
  if (phases & 4) ETS_TRY((launch_dq<E, D>(a, gq, st, n_qtiles)));
  return 0;
}

int launch_dense_bwd(const DenseArgs& a, Dt dt, void* stream, int phases) {
  if (dt == Dt::BF16)
    return a.d == 128 ? launch_bwd_t<BF16, 128>(a, stream, phases) : launch_bwd_t<BF16, 64>(a, stream, phases);
  return a.d == 128 ? launch_bwd_t<F16, 128>(a, stream, phases) : launch_bwd_t<F16, 64>(a, stream, phases);
}

}  // namespace ets
