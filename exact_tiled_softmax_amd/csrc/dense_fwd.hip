// Dense masked attention forward, bf16/fp16 MFMA path for gfx950.
//
// What it computes (alphabetamath.cc, "Tiled attention and its recomputed
// reverse pass are exact", proof paragraph 1; intale.github.io ch. 19,
// "Rescale earlier mass before adding a new tile"): for every query row the
// key/value tiles are streamed in order and a running summary (m, l, z) is
// carried from the empty state; a tile with no allowed key for a row leaves
// that row's summary unchanged; at the end Y = z / l and LSE = m + ln l.
//
// Mapping onto CDNA4:
//   * a workgroup owns BQ = NW waves x 32*NB query rows of one (batch, head);
//     each wave keeps its Q rows in registers as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16, queries along lanes, keys along the
//     accumulator rows), so a query's running max and sum live in one lane
//     plus its partner lane l ^ 32;
//   * K and V tiles of 64 keys go straight from HBM into an LDS ring of 2-3
//     stages (swizzled rows), so the next tiles load while one is used; the PV product is accumulated transposed, O^T += V^T P^T, with V^T
//     read by ds_read_b64_tr_b16 and P^T fed straight from the S^T
//     accumulators (no shuffles);
//   * scores are kept in base 2 (c*log2 e folded into one FMA before
//     v_exp_f32); the reference maximum of a row is only raised when a tile's
//     maximum exceeds it by more than kRescaleSlack (log2 units), which keeps
//     every weight <= 2^kRescaleSlack and skips most rescales of the O
//     accumulators.  Any reference value gives the same z / l exactly, so the
//     result is unchanged up to rounding; the LSE uses the final reference.
#include "device.hpp"

namespace ets {

constexpr float kRescaleSlack = 8.0f;

template <class E, int D, int NB, int NW, int STAGES, bool DROP>
__global__ __launch_bounds__(64 * NW, NB == 1 ? 2 : 1) void dense_fwd_kernel(const DenseArgs a, int n_qtiles) {
  constexpr int BK = 64;
  constexpr int NQW = 32 * NB;
  constexpr int BQ = NW * NQW;
  static_assert(STAGES == 2 || STAGES == 3, "LDS ring depth");  // launch passes STAGES * 2 * TILEB bytes
  constexpr int KS = D / 16;        // k-steps of the score contraction
  constexpr int MD = D / 32;        // 32-row blocks of O^T
  constexpr int ROWB = D * 2;       // bytes per LDS tile row
  constexpr int TILEB = BK * ROWB;  // bytes per K or V tile
  typedef typename E::vec8 vec8;

  extern __shared__ __attribute__((aligned(16))) char smem_dyn[];  // STAGES x (K, V) tiles
  char ETS_LDS* smem = (char ETS_LDS*)smem_dyn;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;

  // heaviest query tiles first; consecutive blocks walk (batch, head) so a
  // lane's tiles stay on one XCD when B*H is a multiple of 8
  const int BH = a.B * a.H;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
  const int nq = a.nq, nk = a.nk;
  const int q0 = qt * BQ, qw0 = q0 + wave * NQW;

  const uint16_t* Qp = (const uint16_t*)a.Q + (size_t)bh * nq * D;
  const uint16_t* Kp = (const uint16_t*)a.K + (size_t)(b * a.Hkv + g) * nk * D;
  const uint16_t* Vp = (const uint16_t*)a.V + (size_t)(b * a.Hkv + g) * nk * D;

  // Q rows of this wave as B operands: lane holds query qw0 + 32nb + l32,
  // features 16kk + 8h32 .. +7
  vec8 qreg[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int q = qw0 + 32 * nb + l32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = u32x4{0, 0, 0, 0};
      if (q < nq) v = *(const u32x4*)(Qp + (size_t)q * D + 16 * kk + 8 * h32);
      qreg[nb][kk] = as_vec8<E>(v);
    }
  }

  f32x16 oacc[MD][NB];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][nb][r] = 0.f;
  float mref[NB], lsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { mref[nb] = kNegInf; lsum[nb] = 0.f; }

  // key-tile range of the workgroup
  const int qlast = min(q0 + BQ, nq) - 1;
  int jt_lo = 0, jt_hi = (nk - 1) / BK;
  if (a.mask.causal) jt_hi = min(jt_hi, qlast / BK);
  if (a.mask.window > 0) jt_lo = max(0, (q0 - a.mask.window + 1) / BK);

  auto wg_nonempty = [&](int jt) {
    return classify(a.mask, q0, q0 + BQ - 1, jt * BK, jt * BK + BK - 1, nq, nk) != kEmpty;
  };
  auto next_tile = [&](int jt) {
    for (++jt; jt <= jt_hi; ++jt)
      if (wg_nonempty(jt)) return jt;
    return -1;
  };

  // K and V tiles go straight from HBM to LDS (rows past nk read row nk-1;
  // those keys are masked as a ragged tile), STAGES tiles in flight
  constexpr int LOADS = 2 * (BK * D / 8 / 64) / NW;  // load instructions per wave per tile
  auto load = [&](int jt, int stage) {
    char ETS_LDS* kt = smem + stage * 2 * TILEB;
    tile_to_lds<BK, D, NW>(kt, Kp, jt * BK, nk - 1, wave, lane);
    tile_to_lds<BK, D, NW>(kt + TILEB, Vp, jt * BK, nk - 1, wave, lane);
  };

  // tiles[0] is the tile in use, tiles[1 .. STAGES-2] are already in flight
  int tiles[STAGES - 1];
  tiles[0] = (jt_lo <= jt_hi && wg_nonempty(jt_lo)) ? jt_lo : next_tile(jt_lo);
#pragma unroll
  for (int k = 1; k < STAGES - 1; ++k) tiles[k] = (tiles[k - 1] >= 0) ? next_tile(tiles[k - 1]) : -1;
#pragma unroll
  for (int k = 0; k < STAGES - 1; ++k)
    if (tiles[k] >= 0) load(tiles[k], k);
  wait_vm();
  __syncthreads();
  int stage = 0;

  const float sl2 = a.scale_log2;
  const int lane_bh = bh;
  const RowOps32<ROWB> kops(lane);
  const TrOps32<ROWB> vops(lane);

  while (tiles[0] >= 0) {
    const int jt = tiles[0];
    const int tn = (tiles[STAGES - 2] >= 0) ? next_tile(tiles[STAGES - 2]) : -1;
    if (tn >= 0) load(tn, stage == 0 ? STAGES - 1 : stage - 1);  // the stage read last iteration
    const char ETS_LDS* kt = smem + stage * 2 * TILEB;
    const char ETS_LDS* vt = kt + TILEB;
    const int j0 = jt * BK;
    const int cinfo = classify(a.mask, qw0, qw0 + NQW - 1, j0, j0 + BK - 1, nq, nk);
    const int cls = cinfo & kClassMask;
    const bool cbm = (cinfo & kCheckBlockMask) != 0;

    if (cls != kEmpty) {
      // ---- S^T = K Q^T: rows are keys j0 + 32mb + (8(r/4) + 4h32 + r%4)
      f32x16 s[2][NB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[mb][nb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const vec8 ka = as_vec8<E>(lds_b128(kt, kops.off(32 * mb, kk)));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[mb][nb] = E::mfma32(ka, qreg[nb][kk], s[mb][nb]);
        }
      }

      // ---- online summary update per query (one per lane and nb)
      vec8 pb[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int qi = qw0 + 32 * nb + l32;
        unsigned allow[2][4];
        if (cls == kPartial) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              allow[mb][g4] = allowed4(a.mask, qi, j0 + 32 * mb + 8 * g4 + 4 * h32, nq, nk, cbm);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (!((allow[mb][g4] >> r) & 1u)) s[mb][nb][4 * g4 + r] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][nb][r]);
        mx = xhalf_max(mx);
        const float mt = (mx == kNegInf) ? kNegInf : mx * sl2;
        const bool need = mt > mref[nb] + kRescaleSlack;
        if (wave_any(need)) {
          const float alpha = need ? fast_exp2(mref[nb] - mt) : 1.f;
          if (need) mref[nb] = mt;
          lsum[nb] *= alpha;
#pragma unroll
          for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[md][nb][r] *= alpha;
        }
        const float mneg = -mref[nb];
        float ps = 0.f;
        uint32_t packed[2][8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = fast_exp2(fmaf(s[mb][nb][4 * g4 + r], sl2, mneg));
            if (cls == kPartial) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (!((allow[mb][g4] >> r) & 1u)) p[r] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) ps += p[r];
            if constexpr (DROP) {
              const unsigned keep = keep4(a.drop, lane_bh, qi, j0 + 32 * mb + 8 * g4 + 4 * h32);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (!((keep >> r) & 1u)) p[r] = 0.f;
            }
            packed[mb][2 * g4] = E::pack2(p[0], p[1]);
            packed[mb][2 * g4 + 1] = E::pack2(p[2], p[3]);
          }
        }
        lsum[nb] += ps;
        // k-step ks covers accumulator entries 8(ks%2) .. +7 of block ks/2
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int mb = ks >> 1, o = (ks & 1) * 4;
          u32x4 u = u32x4{packed[mb][o], packed[mb][o + 1], packed[mb][o + 2], packed[mb][o + 3]};
          pb[nb][ks] = as_vec8<E>(u);
        }
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const vec8 va = as_vec8<E>(vops.read(vt, 16 * ks, md));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) oacc[md][nb] = E::mfma32(va, pb[nb][ks], oacc[md][nb]);
        }
      }
    }

    // the next tile must be complete; later ones may stay in flight
    if (tn >= 0) wait_vm_n<(STAGES - 2) * LOADS>(); else wait_vm();
    __syncthreads();
#pragma unroll
    for (int k = 0; k < STAGES - 2; ++k) tiles[k] = tiles[k + 1];
    tiles[STAGES - 2] = tn;
    stage = (stage == STAGES - 1) ? 0 : stage + 1;
  }

  // ---- epilogue: Y = z / l, LSE = (m + log2 l) ln 2
  uint16_t* Yp = (uint16_t*)a.out_Y + (size_t)bh * nq * D;
  float* Lp = a.LSE + (size_t)bh * nq;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int q = qw0 + 32 * nb + l32;
    const float l = xhalf_sum(lsum[nb]);
    float inv = (l > 0.f) ? 1.f / l : 0.f;
    if constexpr (DROP) inv *= a.drop.inv_keep;
    if (q < nq) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = 32 * md + 8 * g4 + 4 * h32;
          u32x2 w;
          w[0] = E::pack2(oacc[md][nb][4 * g4] * inv, oacc[md][nb][4 * g4 + 1] * inv);
          w[1] = E::pack2(oacc[md][nb][4 * g4 + 2] * inv, oacc[md][nb][4 * g4 + 3] * inv);
          *(u32x2*)(Yp + (size_t)q * D + col) = w;
        }
      if (h32 == 0) Lp[q] = (l > 0.f) ? (mref[nb] + __log2f(l)) * kLn2 : kNegInf;
    }
  }
}

template <class E, int D, int NB, int NW, int STAGES>
static int launch_fwd_t(const DenseArgs& a, void* stream) {
  constexpr int BQ = NW * 32 * NB;
  constexpr int LDS = STAGES * 2 * 64 * D * 2;
  const int n_qtiles = (a.nq + BQ - 1) / BQ;
  dim3 grid(n_qtiles * a.B * a.H), block(64 * NW);
  if (a.drop.enabled)
    ETS_TRY(launch((dense_fwd_kernel<E, D, NB, NW, STAGES, true>), grid, block, LDS, (hipStream_t)stream, a, n_qtiles));
  else
    ETS_TRY(launch((dense_fwd_kernel<E, D, NB, NW, STAGES, false>), grid, block, LDS, (hipStream_t)stream, a, n_qtiles));
  return 0;
}

bool dense_mfma_supported(int d, int dv) { return d == dv && (d == 64 || d == 128); }

int launch_dense_fwd(const DenseArgs& a, Dt dt, void* stream) {
  if (dt == Dt::BF16) {
    if (a.d == 128) return launch_fwd_t<BF16, 128, 1, 4, 2>(a, stream);
    return launch_fwd_t<BF16, 64, 1, 4, 3>(a, stream);
  }
  if (a.d == 128) return launch_fwd_t<F16, 128, 1, 4, 2>(a, stream);
  return launch_fwd_t<F16, 64, 1, 4, 3>(a, stream);
}

}  // namespace ets
