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
//         LDS transpose reads.  No atomics.
#include "device.hpp"

namespace ets {

// --------------------------------------------------------------------- prep
// -D_i = -(G_i . Y_i) and the base-2 LSE, LSE_i log2(e) (+inf for a row with
// an empty allowed set, so every recomputed weight of it is 0).  The 64 rows
// after the last are filled with D = 0, LSE2 = +inf: tiles of 64 rows may read
// them.  -D is stored so that it can start a dP accumulator (dP - D).
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
    a.Dws[row] = -acc;
    a.Lws[row] = l2;
  }
}

// Keep bits for the key-major layout, where the eight lanes of an octet hold
// the keys 8k .. 8k+7 of one 8-key Philox block (lane u holds key 8k + u) and
// share their query rows: rows i0 .. i0+3 (out0) and i0+8 .. i0+11 (out1).
// Lane u draws the block of row i0 + u (u < 4) or i0 + 4 + u (u >= 4), the
// octet ORs the eight draws together, and each lane keeps its key's bit of
// every row: bit 8 r of out0 (out1) keeps row i0 + r (i0 + 8 + r).  Each
// block is drawn exactly once.
__device__ __forceinline__ void keep8_rows(const DropArgs& d, int lane_bh, int i0, int j, unsigned& out0,
                                           unsigned& out1) {
  const int u = j & 7;
  const unsigned blk = keep8(d, lane_bh, i0 + (u < 4 ? u : 4 + u), j & ~7);
  int lo = u < 4 ? (int)(blk << (8 * u)) : 0;
  int hi = u < 4 ? 0 : (int)(blk << (8 * (u - 4)));
  lo |= __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  hi |= __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false);
  lo |= __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  hi |= __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false);
  lo |= __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, false);  // row_half_mirror: the other quad
  hi |= __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, false);
  out0 = ((unsigned)lo >> u) & 0x01010101u;
  out1 = ((unsigned)hi >> u) & 0x01010101u;
}

// --------------------------------------------------------------------- dK, dV
// Order of the 2 KS products of an A group (S = K Q^T and dP = V G^T of one
// 32-row block, KS k-steps each): S(0), S(1), then dP(k) and S(k + 2)
// alternating, dP(KS - 1) last, so the first dP product comes two slots after
// the group starts (its accumulator starts from -D, read from LDS there).
template <int KS>
constexpr bool a_is_dp(int u) { return u >= 2 && ((u & 1) == 0 || u == 2 * KS - 1); }
template <int KS>
constexpr int a_kstep(int u) {
  return a_is_dp<KS>(u) ? (u == 2 * KS - 1 ? KS - 1 : (u - 2) / 2) : (u < 2 ? u : (u + 1) / 2);
}
// Group plans of a step with NMQ query blocks: group gi is A (S, dP) or B
// (dV, dK) of block mq[gi]; W(wq[gi]) runs under group gi, the LSE / D rows
// of W(nwq[gi]) are read at its end, and the copies of the next step are
// spread over the groups marked in `copies`.
template <int NMQ>
struct DkPlan;
template <>
struct DkPlan<2> {  // A0 | A1+W0 | B0+W1 | B1
  static constexpr int NG = 4;
  static constexpr bool isA[4] = {true, true, false, false};
  static constexpr int mq[4] = {0, 1, 0, 1};
  static constexpr int wq[4] = {-1, 0, 1, -1};
  static constexpr int nwq[4] = {0, 1, -1, -1};
  static constexpr bool copies[4] = {true, false, false, false};
};
template <>
struct DkPlan<4> {  // A0 | A1+W0 | B0 | A2+W1 | B1 | A3+W2 | B2+W3 | B3
  static constexpr int NG = 8;
  static constexpr bool isA[8] = {true, true, false, true, false, true, false, false};
  static constexpr int mq[8] = {0, 1, 0, 2, 1, 3, 2, 3};
  static constexpr int wq[8] = {-1, 0, -1, 1, -1, 2, 3, -1};
  static constexpr int nwq[8] = {0, -1, 1, -1, 2, 3, -1, -1};
  static constexpr bool copies[8] = {true, false, true, false, false, false, false, false};
};
template <class P>
constexpr int plan_start(int gi, int na, int nb) {
  int s0 = 0;
  for (int k = 0; k < gi; ++k) s0 += P::isA[k] ? na : nb;
  return s0;
}
template <class P>
constexpr int plan_group(int t, int na, int nb) {
  int gi = 0;
  while (gi + 1 < P::NG && t >= plan_start<P>(gi + 1, na, nb)) ++gi;
  return gi;
}
template <class P>
constexpr int plan_copy_groups() {
  int n = 0;
  for (int k = 0; k < P::NG; ++k) n += P::copies[k] ? 1 : 0;
  return n;
}
template <class P>
constexpr int plan_copy_rank(int gi) {  // index of group gi among the copy groups
  int n = 0;
  for (int k = 0; k < gi; ++k) n += P::copies[k] ? 1 : 0;
  return n;
}

// A workgroup owns 128 keys (32 per wave) of one K/V head; a step is one
// query head of the group and a tile of BQ = 64 query rows, blocks mq of 32
// rows.  Per block a wave runs
//   A(mq): S = Q K^T and dP = G V^T            (2 D/16 MFMAs)
//   W(mq): P and gamma from S, dP, LSE, D       (VALU)
//   B(mq): dV^T += G^T P~, dK^T += Q^T gamma   (4 D/32 MFMAs)
// in a fixed order (DkPlan), one MFMA per slot with operands read three slots
// ahead, so the VALU work of a block runs under the MFMAs of another; the
// copy of the next step's rows into the other LDS stage is spread over the
// first group.
template <class E, int D, int MK, bool DROP>
__global__ __launch_bounds__(256, 1) void dense_bwd_dkdv_kernel(const DenseArgs a, int n_kblocks) {
  constexpr int BQ = 64;  // query rows per step
  typedef DkPlan<BQ / 32> Plan;
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BQ * ROWB;
  constexpr int NA = 2 * KS, NB = 4 * MD;  // slots of A(mq), B(mq)
  typedef typename E::vec8 vec8;
  typedef std::integral_constant<int, 0> Stage0;
  typedef std::integral_constant<int, 1> Stage1;

  // one array per (stage, tensor): reads of one stage never wait for the
  // copies into the other.  L: LSE2 (128 floats) then D (128 floats).
  __shared__ __attribute__((aligned(16))) char ldsQ0[TILEB], ldsG0[TILEB], ldsQ1[TILEB], ldsG1[TILEB];
  __shared__ __attribute__((aligned(16))) char ldsL0[1024], ldsL1[1024];
  auto qbuf = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return (char ETS_LDS*)ldsQ0;
    else return (char ETS_LDS*)ldsQ1;
  };
  auto gbuf = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return (char ETS_LDS*)ldsG0;
    else return (char ETS_LDS*)ldsG1;
  };
  auto lbuf = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return (char ETS_LDS*)ldsL0;
    else return (char ETS_LDS*)ldsL1;
  };
  // LSE2 and D rows through one buffer resource: the workspace holds D
  // first and the base-2 LSE after it, each with 64 padding rows
  const uint32_t lse_off = (uint32_t)((const char*)a.Lws - (const char*)a.Dws);
  const __amdgpu_buffer_rsrc_t Wrs = make_rsrc(a.Dws, lse_off + (uint32_t)((a.B * a.H * a.nq + 64) * 4));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h32 = lane >> 5, l32 = lane & 31;
  const int nq = a.nq, nk = a.nk;
  const int BG = a.B * a.Hkv, grp = a.H / a.Hkv;
  const float sl2 = a.scale_log2;
  const RowOps32<ROWB> rops(lane);
  const TrOps32<ROWB> tops(lane);
  const TileCopy<BQ, D, 4> tcopy(wave, lane);
  constexpr int PW = TileCopy<BQ, D, 4>::PER_WAVE;
  constexpr int NCOPY = 2 * PW;  // Q and G copy instructions per wave per step

  // Persistent workgroups: workgroup w of G takes items w, 2G-1-w, 2G+w, ...
  // of the list (key block, (batch, kv head)), key blocks with the most
  // query tiles first.
  const int G = (int)gridDim.x, n_items = n_kblocks * BG;
  for (int r = 0; r * G < n_items; ++r) {
    const int item = r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    if (item >= n_items) continue;
    const int kb = item / BG, bg = item % BG;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int k0 = kb * 128, kw0 = k0 + 32 * wave;
    const int key = kw0 + l32;  // this lane's key

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
      for (int r2 = 0; r2 < 16; ++r2) { dk[md][r2] = 0.f; dv[md][r2] = 0.f; }

    // steps s = (head in group) * n_qt + (query tile - qt_lo)
    const int klast = min(k0 + 127, nk - 1);
    int qt_lo = 0, qt_hi = (nq - 1) / BQ;
    if (a.mask.causal) qt_lo = k0 / BQ;
    if (a.mask.window > 0) qt_hi = min(qt_hi, (klast + a.mask.window - 1) / BQ);
    const int n_qt = qt_hi - qt_lo + 1;
    const int total = (n_qt > 0) ? n_qt * grp : 0;
    auto wg_nonempty = [&](int st) {
      const int qt = qt_lo + st % n_qt;
      return classify<MK>(a.mask, qt * BQ, qt * BQ + BQ - 1, k0, k0 + 127, nq, nk) != kEmpty;
    };
    auto next_of = [&](int st) {
      for (++st; st < total; ++st)
        if (MK == kArith || wg_nonempty(st)) return st;
      return -1;
    };
    auto step_rows = [&](int st, size_t& lane_off, int& qb0) __attribute__((always_inline)) {
      const int h = g * grp + st / n_qt;
      lane_off = (size_t)(b * a.H + h) * nq;
      qb0 = (qt_lo + st % n_qt) * BQ;
    };
    // copy instruction u of step st into stage `stg`: Q rows, then G rows
    auto copy_one = [&](int st, auto stg, int u) __attribute__((always_inline)) {
      size_t lo;
      int qb0;
      step_rows(st, lo, qb0);
      const uint32_t lane_bytes = (uint32_t)nq * D * 2;
      if (u < PW) tcopy.issue_one(qbuf(stg), make_rsrc((const uint16_t*)a.Q + lo * D, lane_bytes), qb0, nq - 1, u);
      else tcopy.issue_one(gbuf(stg), make_rsrc((const uint16_t*)a.G + lo * D, lane_bytes), qb0, nq - 1, u - PW);
    };
    // LSE2 and D rows qb0 .. qb0+127 of step st (wave 0): lanes 0-31 LSE2 to
    // bytes 0-511, lanes 32-63 D to bytes 512-1023 (rows past the workspace
    // read as zero through the resource bound)
    auto copy_lse = [&](int st, auto stg) __attribute__((always_inline)) {
      if (wave == 0) {
        size_t lo;
        int qb0;
        step_rows(st, lo, qb0);
        const uint32_t off = (uint32_t)((lo + qb0 + 4 * l32) * 4) + (h32 ? 0u : lse_off);
        copy16_to_lds(Wrs, off, (void ETS_LDS*)lbuf(stg));
      }
    };

    // MFMA operands in slot order (groups as in the plan); A slots alternate
    // Q and G rows per k-step, B slots alternate G^T (dV) and Q^T (dK) per
    // (kh, md).
    constexpr int NSLOT = (BQ / 32) * (NA + NB);
    auto operand = [&](auto stg, int t) __attribute__((always_inline)) {
      const int gi = plan_group<Plan>(t, NA, NB);
      const int u = t - plan_start<Plan>(gi, NA, NB), mq = Plan::mq[gi];
      if (Plan::isA[gi])
        return as_vec8<E>(lds_b128(a_is_dp<KS>(u) ? gbuf(stg) : qbuf(stg), rops.off(32 * mq, a_kstep<KS>(u))));
      const int kh = u / (2 * MD), md = (u % (2 * MD)) / 2;
      return as_vec8<E>(tops.read((u & 1) ? qbuf(stg) : gbuf(stg), 32 * mq + 16 * kh, md));
    };

    // rows interval of this lane's key for arithmetic masks: query row
    // base + c is allowed iff (unsigned)(c - lo) <= rng
    auto arith_interval = [&](int base, int& lo, unsigned& rng) __attribute__((always_inline)) {
      int ilo = 0, ihi = nq - 1;
      if (a.mask.causal) ilo = max(ilo, key);
      if (a.mask.window > 0) ihi = min(ihi, key + a.mask.window - 1);
      const bool any = key < nk && ilo <= ihi;
      lo = any ? ilo - base : (1 << 24);
      rng = any ? (unsigned)(ihi - ilo) : 0u;
    };
    // P and gamma of one block: rows 32mq + 8g4 + 4h32 + r2 (this lane's key)
    struct Weights {
      uint32_t pw[8], gw[8];
      f32x4 l4[4], d4[4];
      unsigned allow[4], keep[4];
    };
    auto read_ld = [&](Weights& w, auto stg, int mq) __attribute__((always_inline)) {
      const float ETS_LDS* ls = (const float ETS_LDS*)lbuf(stg);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qr = 32 * mq + 8 * g4 + 4 * h32;
        w.l4[g4] = *(const f32x4 ETS_LDS*)(ls + qr);
        if constexpr (DROP) w.d4[g4] = *(const f32x4 ETS_LDS*)(ls + 128 + qr);  // -D after 128 LSE2 floats
      }
    };
    // sub-part k = 2 g4 + half: rows r2 = 2 half, 2 half + 1 of group g4
    auto weights = [&](Weights& w, const f32x16& sc, const f32x16& dp, int k, int mq, int qb0, int lane_bh,
                       auto part_tag, bool cbm) __attribute__((always_inline)) {
      constexpr bool PART = decltype(part_tag)::value;
      const int g4 = k / 2, half = k % 2;
      const int qr = 32 * mq + 8 * g4 + 4 * h32;
      if (half == 0) {
        w.allow[g4] = 0xFu;
        if constexpr (PART) {
          if constexpr (MK == kArith) {
            int lo;
            unsigned rng;
            arith_interval(qb0 + qr, lo, rng);
            unsigned al = 0;
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) al |= ((unsigned)(r2 - lo) <= rng ? 1u : 0u) << r2;
            w.allow[g4] = al;
          } else {
            w.allow[g4] = allowed4_rows<MK>(a.mask, qb0 + qr, key, nq, nk, cbm);
          }
        }
        if constexpr (DROP)
          if (g4 % 2 == 0) keep8_rows(a.drop, lane_bh, qb0 + qr, key, w.keep[g4], w.keep[g4 + 1]);
      }
      float pk[2], gm[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r2 = 2 * half + e;
        const float pv = fast_exp2(fmaf(sc[4 * g4 + r2], sl2, -w.l4[g4][r2]));
        float dpv = dp[4 * g4 + r2];
        bool kp = true;
        if constexpr (DROP) {
          kp = (w.keep[g4] >> (8 * r2)) & 1u;
          dpv = kp ? dpv * a.drop.inv_keep : 0.f;
        }
        const bool al = !PART || ((w.allow[g4] >> r2) & 1u);
        pk[e] = (al && kp) ? pv : 0.f;
        // without dropout the dP accumulator started from -D
        if constexpr (DROP) dpv += w.d4[g4][r2];
        gm[e] = al ? pv * dpv : 0.f;
      }
      w.pw[2 * g4 + half] = E::pack2(pk[0], pk[1]);
      w.gw[2 * g4 + half] = E::pack2(gm[0], gm[1]);
      materialize(w.pw[2 * g4 + half]);
      materialize(w.gw[2 * g4 + half]);
    };
    auto pack_op = [&](const uint32_t (&x)[8], int kh) __attribute__((always_inline)) {
      return as_vec8<E>(u32x4{x[4 * kh], x[4 * kh + 1], x[4 * kh + 2], x[4 * kh + 3]});
    };

    // one step on stage stg; its successor's rows go into the other stage
    auto step = [&](auto stg, int st, int sn, auto part_tag, bool cbm) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(stg)::value> Next;
      size_t lo;
      int qb0;
      step_rows(st, lo, qb0);
      const int lane_bh = (int)(lo / nq);
      copy_lse(sn, Next{});
      f32x16 sc[BQ / 32], dp[BQ / 32];
      Weights w[BQ / 32];
      vec8 opb[4];
#pragma unroll
      for (int k = 0; k < 3; ++k) opb[k] = operand(stg, k);
      static_for<NSLOT>([&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        constexpr int gi = plan_group<Plan>(t, NA, NB);
        constexpr int u = t - plan_start<Plan>(gi, NA, NB);
        constexpr bool isA = Plan::isA[gi];
        constexpr int mq = Plan::mq[gi];
        constexpr int gsz = isA ? NA : NB;
        if constexpr (t + 3 < NSLOT) opb[(t + 3) % 4] = operand(stg, t + 3);
        const vec8 op = opb[t % 4];
        if constexpr (isA) {
          constexpr int kk = a_kstep<KS>(u);
          if constexpr (u == 0) {
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) sc[mq][r2] = 0.f;
            if constexpr (DROP) {
#pragma unroll
              for (int r2 = 0; r2 < 16; ++r2) dp[mq][r2] = 0.f;
            } else {  // dP starts from -D of its rows (the first dP product is two slots on)
              const float ETS_LDS* ls = (const float ETS_LDS*)lbuf(stg);
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = *(const f32x4 ETS_LDS*)(ls + 128 + 32 * mq + 8 * g4 + 4 * h32);
#pragma unroll
                for (int r = 0; r < 4; ++r) dp[mq][4 * g4 + r] = x[r];
              }
            }
          }
          if constexpr (a_is_dp<KS>(u)) dp[mq] = E::mfma32(op, vreg[kk], dp[mq]);
          else sc[mq] = E::mfma32(op, kreg[kk], sc[mq]);
        } else {
          constexpr int kh = u / (2 * MD), md = (u % (2 * MD)) / 2;
          if constexpr (u & 1) dk[md] = E::mfma32(op, pack_op(w[mq].gw, kh), dk[md]);
          else dv[md] = E::mfma32(op, pack_op(w[mq].pw, kh), dv[md]);
        }
        // copies of the next step in the plan's copy groups
        if constexpr (Plan::copies[gi]) {
          constexpr int NCG = plan_copy_groups<Plan>(), per = NCOPY / NCG;
          constexpr int base = plan_copy_rank<Plan>(gi) * per;
          static_for<per>([&](auto uc) __attribute__((always_inline)) {
            constexpr int cu = decltype(uc)::value;
            if constexpr ((cu * gsz) / per == u) copy_one(sn, Next{}, base + cu);
          });
        }
        // W(wq) runs under group gi; the LSE / D rows of W(nwq) are read at
        // the end of group gi
        constexpr int wq = Plan::wq[gi];
        constexpr int nwq = Plan::nwq[gi];
        if constexpr (nwq >= 0 && u == gsz - 2) read_ld(w[nwq], stg, nwq);
        if constexpr (wq >= 0) {
          static_for<8>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            if constexpr ((k * gsz) / 8 == u) weights(w[wq], sc[wq], dp[wq], k, wq, qb0, lane_bh, part_tag, cbm);
          });
        }
        ETS_FENCE();
      });
    };
    auto empty_step = [&](auto stg, int sn) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(stg)::value> Next;
      copy_lse(sn, Next{});
#pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(sn, Next{}, u);
    };
    auto finish = [&]() __attribute__((always_inline)) {
      wait_vm();
      __syncthreads();
    };
    auto general_step = [&](auto stg, int st, int sn) __attribute__((always_inline)) {
      size_t lo;
      int qb0;
      step_rows(st, lo, qb0);
      const int cinfo = classify<MK>(a.mask, qb0, qb0 + BQ - 1, kw0, kw0 + 31, nq, nk);
      const int cls = cinfo & kClassMask;
      if (cls == kFull) step(stg, st, sn, std::false_type{}, false);
      else if (cls == kPartial) step(stg, st, sn, std::true_type{}, (cinfo & kCheckBlockMask) != 0);
      else empty_step(stg, sn);
      finish();
    };

    int st = -1;
    if (total > 0) st = (MK == kArith || wg_nonempty(0)) ? 0 : next_of(0);
    if (st >= 0) {
      copy_lse(st, Stage0{});
#pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(st, Stage0{}, u);
    }
    finish();
    // Step number p runs on stage p % 2.  For arithmetic masks the query
    // tiles that the whole key block sees whole form one range per head;
    // pairs of them starting on stage 0 run without classification in a loop
    // of their own (one code path, so the accumulators stay in place).
    int p = 0;
    auto general_until = [&](int st_end) __attribute__((always_inline)) {
      while (st >= 0 && st < st_end) {
        const int sn = next_of(st);
        if (p & 1) general_step(Stage1{}, st, sn >= 0 ? sn : st);
        else general_step(Stage0{}, st, sn >= 0 ? sn : st);
        st = sn;
        ++p;
      }
    };
    if constexpr (MK == kArith) {
      // local q-tile indices i (qb0 = (qt_lo + i) BQ) whose rows see all 128 keys
      int i_lo = 0, i_hi = n_qt - 1;
      if (k0 + 127 >= nk) i_hi = -1;
      i_hi = min(i_hi, (nq - BQ) / BQ - qt_lo);
      if (a.mask.causal) i_lo = max(i_lo, (k0 + 127 + BQ - 1) / BQ - qt_lo);
      if (a.mask.window > 0) {
        const int lim = k0 + a.mask.window - BQ;  // full iff qb0 <= lim
        i_hi = (lim < 0) ? -1 : min(i_hi, lim / BQ - qt_lo);
      }
      for (int hi = 0; hi < grp && i_lo <= i_hi; ++hi) {
        int a0 = hi * n_qt + i_lo, a1 = hi * n_qt + i_hi + 1;
        general_until(a0);
        if (st != a0) break;  // (not reached: arithmetic masks skip no step)
        if (p & 1) {
          general_until(a0 + 1);
          ++a0;
        }
        if ((a1 - a0) & 1) --a1;
        for (; st < a1; st += 2, p += 2) {
          step(Stage0{}, st, st + 1, std::false_type{}, false);
          finish();
          const int sn = next_of(st + 1);
          step(Stage1{}, st + 1, sn >= 0 ? sn : st + 1, std::false_type{}, false);
          finish();
        }
        if (st >= total) st = -1;
      }
    }
    general_until(1 << 30);

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
}

// --------------------------------------------------------------------- dQ
// Query-major, the forward's layout: a workgroup owns 128 query rows (32 per
// wave, queries along lanes) of one (batch, head) and streams the K/V tiles
// of 64 keys through a two-stage LDS ring.  Per 32-key block mb a wave runs
//   A(mb): S^T = K Q^T and dP^T = V G^T     (2 D/16 MFMAs)
//   W(mb): gamma^T from S^T, dP^T, LSE, D    (VALU)
//   B(mb): dQ^T += K^T gamma^T              (2 D/32 MFMAs)
// in the fixed order A0 | A1+W0 | B0+W1 | B1, one MFMA per slot with
// operands read two slots ahead; the next tile's copy is spread over A0.
template <class E, int D, int MK, bool DROP>
__global__ __launch_bounds__(256, 2) void dense_bwd_dq_kernel(const DenseArgs a, int n_qtiles) {
  constexpr int BK = 64;
  constexpr int BQ = 128;
  constexpr int KS = D / 16;
  constexpr int MD = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BK * ROWB;
  constexpr int NA = 2 * KS, NB = 2 * MD;  // slots of A(mb), B(mb)
  constexpr int NSLOT = 2 * NA + 2 * NB;
  typedef typename E::vec8 vec8;
  typedef std::integral_constant<int, 0> Stage0;
  typedef std::integral_constant<int, 1> Stage1;

  __shared__ __attribute__((aligned(16))) char ldsK0[TILEB], ldsV0[TILEB], ldsK1[TILEB], ldsV1[TILEB];
  auto kbuf = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return (char ETS_LDS*)ldsK0;
    else return (char ETS_LDS*)ldsK1;
  };
  auto vbuf = [&](auto st) __attribute__((always_inline)) {
    if constexpr (decltype(st)::value == 0) return (char ETS_LDS*)ldsV0;
    else return (char ETS_LDS*)ldsV1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h32 = lane >> 5, l32 = lane & 31;
  const int nq = a.nq, nk = a.nk;
  const int BH = a.B * a.H;
  const float sl2 = a.scale_log2;
  const RowOps32<ROWB> rops(lane);
  const TrOps32<ROWB> tops(lane);
  const TileCopy<BK, D, 4> tcopy(wave, lane);
  constexpr int PW = TileCopy<BK, D, 4>::PER_WAVE;
  constexpr int NCOPY = 2 * PW;

  // Persistent workgroups over (query tile, (batch, head)), heaviest query
  // tiles first, in boustrophedon order.
  const int G = (int)gridDim.x, n_items = n_qtiles * BH;
  auto item_of = [&](int r) { return r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x); };
  // key-tile range of query tile qt
  auto tile_range = [&](int qt, int& lo, int& hi) __attribute__((always_inline)) {
    const int q0 = qt * BQ, qlast = min(q0 + BQ, nq) - 1;
    lo = 0;
    hi = (nk - 1) / BK;
    if (a.mask.causal) hi = min(hi, qlast / BK);
    if (a.mask.window > 0) lo = max(0, (q0 - a.mask.window + 1) / BK);
  };
  // The wave priority follows the key tiles the workgroup has left, so of two
  // workgroups sharing a compute unit the one further behind issues first
  // (with equal priorities the older one wins every tie).  rem is a scalar.
  int rem = 0;
  for (int r = 0; r * G < n_items; ++r) {
    const int item = item_of(r);
    if (item >= n_items) continue;
    int lo, hi;
    tile_range(n_qtiles - 1 - item / BH, lo, hi);
    rem += max(hi - lo + 1, 0);
  }
  auto set_prio = [&]() __attribute__((always_inline)) {
    if (rem > 16) __builtin_amdgcn_s_setprio(3);
    else if (rem > 8) __builtin_amdgcn_s_setprio(2);
    else if (rem > 3) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };
  for (int r = 0; r * G < n_items; ++r) {
    const int item = item_of(r);
    if (item >= n_items) continue;
    const int qt = n_qtiles - 1 - item / BH;
    const int bh = item % BH;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
    const int q0 = qt * BQ, qw0 = q0 + wave * 32;
    const int qi = qw0 + l32;  // this lane's query row

    const uint16_t* Qp = (const uint16_t*)a.Q + (size_t)bh * nq * D;
    const uint16_t* Gp = (const uint16_t*)a.G + (size_t)bh * nq * D;
    const uint16_t* Kp = (const uint16_t*)a.K + (size_t)(b * a.Hkv + g) * nk * D;
    const uint16_t* Vp = (const uint16_t*)a.V + (size_t)(b * a.Hkv + g) * nk * D;
    const __amdgpu_buffer_rsrc_t Krs = make_rsrc(Kp, (uint32_t)nk * D * 2);
    const __amdgpu_buffer_rsrc_t Vrs = make_rsrc(Vp, (uint32_t)nk * D * 2);

    vec8 qreg[KS], greg[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 qv = u32x4{0, 0, 0, 0}, gv = u32x4{0, 0, 0, 0};
      if (qi < nq) {
        qv = *(const u32x4*)(Qp + (size_t)qi * D + 16 * kk + 8 * h32);
        gv = *(const u32x4*)(Gp + (size_t)qi * D + 16 * kk + 8 * h32);
      }
      qreg[kk] = as_vec8<E>(qv);
      greg[kk] = as_vec8<E>(gv);
    }
    const float lse2 = (qi < nq) ? a.Lws[(size_t)bh * nq + qi] : __builtin_huge_valf();
    const float ndval = (qi < nq) ? a.Dws[(size_t)bh * nq + qi] : 0.f;  // -D
    f32x16 dq[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) dq[md][r2] = 0.f;

    int jt_lo, jt_hi;
    tile_range(qt, jt_lo, jt_hi);
    auto wg_nonempty = [&](int jt) {
      return classify<MK>(a.mask, q0, q0 + BQ - 1, jt * BK, jt * BK + BK - 1, nq, nk) != kEmpty;
    };
    auto next_of = [&](int jt) {
      for (++jt; jt <= jt_hi; ++jt)
        if (MK == kArith || wg_nonempty(jt)) return jt;
      return -1;
    };
    auto copy_one = [&](int jt, auto st, int u) __attribute__((always_inline)) {
      if (u < PW) tcopy.issue_one(kbuf(st), Krs, jt * BK, nk - 1, u);
      else tcopy.issue_one(vbuf(st), Vrs, jt * BK, nk - 1, u - PW);
    };
    // operand t: A(mb) slots alternate K rows (S^T) and V rows (dP^T) per
    // k-step; B(mb) slots read K^T for (16-key step kh, md)
    auto operand = [&](auto st, int t) __attribute__((always_inline)) {
      if (t < 2 * NA) {
        const int mb = t / NA, u = t % NA, kk = u / 2;
        return as_vec8<E>(lds_b128((u & 1) ? vbuf(st) : kbuf(st), rops.off(32 * mb, kk)));
      }
      const int u = t - 2 * NA, mb = u / NB, kh = (u % NB) / MD, md = u % MD;
      return as_vec8<E>(tops.read(kbuf(st), 32 * mb + 16 * kh, md));
    };
    // key interval of this lane's row for arithmetic masks: key base + c is
    // allowed iff (unsigned)(c - lo) <= rng
    auto arith_interval = [&](int base, int& lo, unsigned& rng) __attribute__((always_inline)) {
      int jlo = 0, jhi = nk - 1;
      if (a.mask.causal) jhi = min(jhi, qi);
      if (a.mask.window > 0) jlo = max(jlo, qi - a.mask.window + 1);
      const bool any = qi < nq && jlo <= jhi;
      lo = any ? jlo - base : (1 << 24);
      rng = any ? (unsigned)(jhi - jlo) : 0u;
    };
    struct Gam {
      uint32_t gw[8];
      unsigned allow[4];
      unsigned keep;  // dropout: bit 8 g4 + r keeps key key0 + 8 g4 + 4 h32 + r
    };
    // sub-part k = 2 g4 + half of W(mb): keys key0 + 8 g4 + 4 h32 + 2 half + e
    auto weights = [&](Gam& w, const f32x16& sc, const f32x16& dp, int k, int key0, auto part_tag, bool cbm)
                       __attribute__((always_inline)) {
      constexpr bool PART = decltype(part_tag)::value;
      const int g4 = k / 2, half = k % 2;
      const int jj = key0 + 8 * g4 + 4 * h32;
      if (half == 0) {
        w.allow[g4] = 0xFu;
        if constexpr (PART) {
          if constexpr (MK == kArith) {
            int lo;
            unsigned rng;
            arith_interval(jj, lo, rng);
            unsigned al = 0;
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) al |= ((unsigned)(r2 - lo) <= rng ? 1u : 0u) << r2;
            w.allow[g4] = al;
          } else {
            w.allow[g4] = allowed4<MK>(a.mask, qi, jj, nq, nk, cbm);
          }
        }
      }
      float gm[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r2 = 2 * half + e;
        const float pv = fast_exp2(fmaf(sc[4 * g4 + r2], sl2, -lse2));
        float dpv = dp[4 * g4 + r2];
        if constexpr (DROP) dpv = ((w.keep >> (8 * g4 + r2)) & 1u) ? dpv * a.drop.inv_keep : 0.f;
        const bool al = !PART || ((w.allow[g4] >> r2) & 1u);
        gm[e] = al ? pv * (dpv + ndval) : 0.f;
      }
      w.gw[2 * g4 + half] = E::pack2(gm[0], gm[1]);
      materialize(w.gw[2 * g4 + half]);
    };
    auto pack_op = [&](const uint32_t (&x)[8], int kh) __attribute__((always_inline)) {
      return as_vec8<E>(u32x4{x[4 * kh], x[4 * kh + 1], x[4 * kh + 2], x[4 * kh + 3]});
    };

    auto tile = [&](auto st, int jt, int jn, auto part_tag, bool cbm) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(st)::value> Next;
      const int j0 = jt * BK;
      f32x16 sc[2], dp[2];
      Gam w[2];
      unsigned kd[4];  // dropout draws of the tile's four blocks of 8 keys per lane pair
      vec8 opb[3];
#pragma unroll
      for (int k = 0; k < 2; ++k) opb[k] = operand(st, k);
      static_for<NSLOT>([&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t + 2 < NSLOT) opb[(t + 2) % 3] = operand(st, t + 2);
        const vec8 op = opb[t % 3];
        if constexpr (t < 2 * NA) {
          constexpr int mb = t / NA, u = t % NA, kk = u / 2;
          if constexpr (u == 0) {
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) { sc[mb][r2] = 0.f; dp[mb][r2] = 0.f; }
          }
          if constexpr (u & 1) dp[mb] = E::mfma32(op, greg[kk], dp[mb]);
          else sc[mb] = E::mfma32(op, qreg[kk], sc[mb]);
          if constexpr (mb == 0) {  // the copy of the next tile and the dropout keep bits
            static_for<NCOPY>([&](auto uc) __attribute__((always_inline)) {
              constexpr int cu = decltype(uc)::value;
              if constexpr ((cu * NA) / NCOPY == u) copy_one(jn, Next{}, cu);
            });
            if constexpr (DROP) {
              static_for<4>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                if constexpr ((q * NA) / 4 == u) {
                  kd[q] = keep_qm_draw(a.drop, bh, qi, j0 + 32 * (q / 2), h32, q % 2);
                  if constexpr (q % 2 == 1) w[q / 2].keep = keep_qm_merge(kd[q - 1], kd[q], h32);
                }
              });
            }
          } else {  // W(0) under A(1)
            static_for<8>([&](auto kc) __attribute__((always_inline)) {
              constexpr int k = decltype(kc)::value;
              if constexpr ((k * NA) / 8 == u) weights(w[0], sc[0], dp[0], k, j0, part_tag, cbm);
            });
          }
        } else {
          constexpr int u = t - 2 * NA, mb = u / NB, kh = (u % NB) / MD, md = u % MD;
          dq[md] = E::mfma32(op, pack_op(w[mb].gw, kh), dq[md]);
          if constexpr (mb == 0) {  // W(1) under B(0)
            static_for<8>([&](auto kc) __attribute__((always_inline)) {
              constexpr int k = decltype(kc)::value;
              if constexpr ((k * NB) / 8 == u) weights(w[1], sc[1], dp[1], k, j0 + 32, part_tag, cbm);
            });
          }
        }
        ETS_FENCE();
      });
    };
    auto empty_tile = [&](auto st, int jn) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(st)::value> Next;
#pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(jn, Next{}, u);
    };
    auto finish = [&]() __attribute__((always_inline)) {
      wait_vm();
      __syncthreads();
    };
    auto general_step = [&](auto st, int jt, int jn) __attribute__((always_inline)) {
      set_prio();
      --rem;
      const int j0 = jt * BK;
      const int cinfo = classify<MK>(a.mask, qw0, qw0 + 31, j0, j0 + BK - 1, nq, nk);
      const int cls = cinfo & kClassMask;
      if (cls == kFull) tile(st, jt, jn, std::false_type{}, false);
      else if (cls == kPartial) tile(st, jt, jn, std::true_type{}, (cinfo & kCheckBlockMask) != 0);
      else empty_tile(st, jn);
      finish();
    };

    int jt = -1;
    if (jt_lo <= jt_hi) jt = (MK == kArith || wg_nonempty(jt_lo)) ? jt_lo : next_of(jt_lo);
    if (jt >= 0) {
#pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(jt, Stage0{}, u);
    }
    finish();
    // Tile number p runs on stage p % 2.  For arithmetic masks the tiles
    // every row of the workgroup sees whole form one range; pairs of them
    // starting on stage 0 run in a loop of their own (one code path, so the
    // accumulators stay in place).
    int fp0 = 1 << 30, fp1 = 1 << 30;  // fixed-order pairs cover tile numbers [fp0, fp1) when fp0 < fp1
    if constexpr (MK == kArith) {
      if (q0 + BQ <= nq) {
        int f_lo = jt_lo, f_hi = min(jt_hi, nk / BK - 1);
        if (a.mask.causal) f_hi = min(f_hi, q0 >= BK - 1 ? (q0 - (BK - 1)) / BK : -1);
        if (a.mask.window > 0) {
          const int t = q0 + BQ - 1 - a.mask.window;  // full iff j0 > t
          if (t >= 0) f_lo = max(f_lo, t / BK + 1);
        }
        if (f_lo <= f_hi) {
          const int lo = f_lo - jt_lo, hi = f_hi - jt_lo + 1;
          const int p0 = lo + (lo & 1), p1 = hi - ((hi - p0) & 1);
          if (p0 < p1) { fp0 = p0; fp1 = p1; }
        }
      }
    }
    int p = 0;
    auto general_run = [&](int p_end) __attribute__((always_inline)) {
      for (; jt >= 0 && p < p_end; ++p) {
        const int jn = next_of(jt);
        if (p & 1) general_step(Stage1{}, jt, jn >= 0 ? jn : jt);
        else general_step(Stage0{}, jt, jn >= 0 ? jn : jt);
        jt = jn;
      }
    };
    general_run(fp0);
    if (fp0 < fp1) {
      // general_run stopped at tile number fp0 < N: jt = jt_lo + p, and
      // tile p + 1 is whole too
      for (; p < fp1; p += 2) {
        set_prio();
        rem -= 2;
        tile(Stage0{}, jt, jt + 1, std::false_type{}, false);
        finish();
        const int jn = next_of(jt + 1);
        tile(Stage1{}, jt + 1, jn >= 0 ? jn : jt + 1, std::false_type{}, false);
        finish();
        jt = jn;
      }
    }
    general_run(1 << 30);

    if (qi < nq) {
      uint16_t* dQp = (uint16_t*)a.dQ + (size_t)bh * nq * D + (size_t)qi * D;
      const float c = a.scale;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = 32 * md + 8 * g4 + 4 * h32;
          u32x2 wv;
          wv[0] = E::pack2(dq[md][4 * g4] * c, dq[md][4 * g4 + 1] * c);
          wv[1] = E::pack2(dq[md][4 * g4 + 2] * c, dq[md][4 * g4 + 3] * c);
          *(u32x2*)(dQp + col) = wv;
        }
    }
  }
}

template <class E, int D, int MK, bool DROP>
static int launch_dkdv_k(const DenseArgs& a, hipStream_t st) {
  const int n_kblocks = (a.nk + 127) / 128;
  const int n_items = n_kblocks * a.B * a.Hkv;
  int slots = 0;
  ETS_TRY(resident_slots(dense_bwd_dkdv_kernel<E, D, MK, DROP>, 256, &slots));
  ETS_TRY(launch((dense_bwd_dkdv_kernel<E, D, MK, DROP>), dim3(min(n_items, slots)), dim3(256), 0, st, a,
                 n_kblocks));
  return 0;
}

template <class E, int D>
static int launch_dkdv(const DenseArgs& a, hipStream_t st) {
  const int mk = mask_kind(a.mask);
  if (a.drop.enabled) {
    if (mk == kArith) return launch_dkdv_k<E, D, kArith, true>(a, st);
    if (mk == kBlock) return launch_dkdv_k<E, D, kBlock, true>(a, st);
    return launch_dkdv_k<E, D, kDenseM, true>(a, st);
  }
  if (mk == kArith) return launch_dkdv_k<E, D, kArith, false>(a, st);
  if (mk == kBlock) return launch_dkdv_k<E, D, kBlock, false>(a, st);
  return launch_dkdv_k<E, D, kDenseM, false>(a, st);
}

template <class E, int D, int MK, bool DROP>
static int launch_dq_k(const DenseArgs& a, hipStream_t st) {
  const int n_qtiles = (a.nq + 127) / 128;
  const int n_items = n_qtiles * a.B * a.H;
  int slots = 0;
  ETS_TRY(resident_slots(dense_bwd_dq_kernel<E, D, MK, DROP>, 256, &slots));
  ETS_TRY(launch((dense_bwd_dq_kernel<E, D, MK, DROP>), dim3(min(n_items, slots)), dim3(256), 0, st, a, n_qtiles));
  return 0;
}

template <class E, int D>
static int launch_dq(const DenseArgs& a, hipStream_t st) {
  const int mk = mask_kind(a.mask);
  if (a.drop.enabled) {
    if (mk == kArith) return launch_dq_k<E, D, kArith, true>(a, st);
    if (mk == kBlock) return launch_dq_k<E, D, kBlock, true>(a, st);
    return launch_dq_k<E, D, kDenseM, true>(a, st);
  }
  if (mk == kArith) return launch_dq_k<E, D, kArith, false>(a, st);
  if (mk == kBlock) return launch_dq_k<E, D, kBlock, false>(a, st);
  return launch_dq_k<E, D, kDenseM, false>(a, st);
}

template <class E, int D>
static int launch_bwd_t(const DenseArgs& a, void* stream, int phases) {
  hipStream_t st = (hipStream_t)stream;
  if (phases & 1) {
    const int rows = a.B * a.H * a.nq;
    const int prep_threads = (rows + 64) * (D / 8);
    ETS_TRY(launch((dense_bwd_prep_kernel<E, D>), dim3((prep_threads + 255) / 256), dim3(256), 0, st, a, rows));
  }
  if (phases & 2) {
    const int rc = launch_dkdv<E, D>(a, st);
    if (rc) return rc;
  }
  if (phases & 4) {
    const int rc = launch_dq<E, D>(a, st);
    if (rc) return rc;
  }
  return 0;
}

int launch_dense_bwd(const DenseArgs& a, Dt dt, void* stream, int phases) {
  if (dt == Dt::BF16)
    return a.d == 128 ? launch_bwd_t<BF16, 128>(a, stream, phases) : launch_bwd_t<BF16, 64>(a, stream, phases);
  return a.d == 128 ? launch_bwd_t<F16, 128>(a, stream, phases) : launch_bwd_t<F16, 64>(a, stream, phases);
}

}  // namespace ets
