// Dense masked attention backward, query-major dQ kernel (bf16/fp16 MFMA,
// gfx950).  The operation and the split into three kernels are described in
// dense_bwd.hip.
#include "device.hpp"

namespace ets {

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
  // (active extents nqa x nka, row lower bounds >= smin; empty when hi < lo)
  auto tile_range = [&](int qt, int nqa, int nka, int smin, int& lo, int& hi) __attribute__((always_inline)) {
    const int q0 = qt * BQ, qlast = min(q0 + BQ, nqa) - 1;
    lo = 0;
    hi = (nka - 1) / BK;
    if (nka < 1 || q0 >= nqa) hi = -1;
    if (a.mask.causal) hi = min(hi, qlast / BK);
    if (a.mask.window > 0) lo = max(0, (q0 - a.mask.window + 1) / BK);
    if (smin > 0) lo = max(lo, smin / BK);
  };
  // The wave priority follows the key tiles the workgroup has left, so of two
  // workgroups sharing a compute unit the one further behind issues first
  // (with equal priorities the older one wins every tie).  rem is a scalar.
  int rem = 0;
  for (int r = 0; r * G < n_items; ++r) {
    const int item = item_of(r);
    if (item >= n_items) continue;
    int lo, hi;
    const int nqa = (MK != kArith && a.mask.lengths) ? min(max(a.mask.lengths[(item % BH) / a.H], 0), nq) : nq;
    tile_range(n_qtiles - 1 - item / BH, nqa, (MK != kArith && a.mask.lengths) ? min(nqa, nk) : nk, 0, lo, hi);
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

    // active extents and row lower bounds of this batch (w: the wave's rows,
    // g: the workgroup's)
    const Layout lay = layout_of<MK>(a.mask, b, nq, nk);
    const int nqa = lay.len, nka = lay.nka;
    int sminw = (int)0x80000000, smaxw = (int)0x80000000, sming = sminw, smaxg = smaxw;
    int st_i = (int)0x80000000;
    if (lay.st) {
      start_range(lay.st, qw0, qw0 + 31, nqa, lane, sminw, smaxw);
      start_range(lay.st, q0, q0 + BQ - 1, nqa, lane, sming, smaxg);
      if (qi < nqa) st_i = lay.st[qi];
    }

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
    tile_range(qt, nqa, nka, sming, jt_lo, jt_hi);
    // tile classes of the per-element mask kinds, 64 tiles at a time
    TileClasses tc;
    tc.base = -1;
    auto classes_for = [&](int t0) __attribute__((always_inline)) {
      if (tc.covers(t0)) return;
      const int t = t0 + lane;
      int cg = kEmpty, cw = kEmpty;
      if (t <= jt_hi) {
        cg = classify<MK>(a.mask, q0, q0 + BQ - 1, t * BK, t * BK + BK - 1, nqa, nka, sming, smaxg);
        cw = classify<MK>(a.mask, qw0, qw0 + 31, t * BK, t * BK + BK - 1, nqa, nka, sminw, smaxw);
      }
      tc.set(t0, cg, cw);
    };
    auto first_from = [&](int t) {  // first tile >= t the workgroup sees, or -1
      if constexpr (is_interval(MK)) {
        return t <= jt_hi ? t : -1;
      } else {
        while (t <= jt_hi) {
          classes_for(t);
          const int f = tc.next_nonempty(t);
          if (f >= 0) return f <= jt_hi ? f : -1;
          t = tc.base + 64;
        }
        return -1;
      }
    };
    auto next_of = [&](int jt) { return first_from(jt + 1); };
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
    // allowed keys of this lane's row under the interval parts of the mask
    // (causal, window, lengths, starts), fixed for the item: key j passes them
    // iff (unsigned)(j - iv_lo) <= iv_rng.  Tiles on the interval body (every
    // mask kind, a tile mask only where it is uniform over the wave's tile)
    // apply just this test.
    int iv_lo = 1 << 30;
    unsigned iv_rng = 0u;
    {
      int jlo = max(0, st_i), jhi = nka - 1;
      if (a.mask.causal) jhi = min(jhi, qi);
      if (a.mask.window > 0) jlo = max(jlo, qi - a.mask.window + 1);
      if (qi < nqa && jlo <= jhi) {
        iv_lo = jlo;
        iv_rng = (unsigned)(jhi - jlo);
      }
    }
    struct Gam {
      uint32_t gw[8];
      unsigned allow[4];
      unsigned keep;  // dropout: bit 8 g4 + r keeps key key0 + 8 g4 + 4 h32 + r
    };
    // sub-part k = 2 g4 + half of W(mb): keys key0 + 8 g4 + 4 h32 + 2 half + e
    auto weights = [&](Gam& w, const f32x16& sc, const f32x16& dp, int k, int key0, auto part_tag, bool cbm)
                       __attribute__((always_inline)) {
      constexpr bool PART = decltype(part_tag)::value != kWhole;
      const int g4 = k / 2, half = k % 2;
      const int jj = key0 + 8 * g4 + 4 * h32;
      constexpr bool IV = decltype(part_tag)::value == kPartIv;
      if constexpr (PART && !IV) {
        if (half == 0) w.allow[g4] = allowed4<MK>(a.mask, qi, jj, nqa, nka, cbm, lay.st);
      }
      float gm[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r2 = 2 * half + e;
        const float pv = fast_exp2(fmaf(sc[4 * g4 + r2], sl2, -lse2));
        float dpv = dp[4 * g4 + r2];
        if constexpr (DROP) dpv = ((w.keep >> (8 * g4 + r2)) & 1u) ? dpv * a.drop.inv_keep : 0.f;
        bool al = true;
        if constexpr (IV) al = (unsigned)(jj + r2 - iv_lo) <= iv_rng;
        else if constexpr (PART) al = (w.allow[g4] >> r2) & 1u;
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
      int cinfo;
      if constexpr (is_interval(MK)) {
        cinfo = classify<MK>(a.mask, qw0, qw0 + 31, j0, j0 + BK - 1, nqa, nka, sminw, smaxw);
      } else {
        classes_for(jt);
        cinfo = tc.wave_class(jt);
      }
      const int cls = cinfo & kClassMask;
      if (cls == kFull) {
        tile(st, jt, jn, BodyTag<kWhole>{}, false);
      } else if (cls == kPartial) {
        // a tile mask that is uniform over the wave's tile leaves only the interval parts
        if constexpr (MK == kDenseM) tile(st, jt, jn, BodyTag<kPartEl>{}, (cinfo & kCheckBlockMask) != 0);
        else if constexpr (MK == kBlock) {
          if (cinfo & kCheckBlockMask) tile(st, jt, jn, BodyTag<kPartEl>{}, true);
          else tile(st, jt, jn, BodyTag<kPartIv>{}, false);
        } else {
          tile(st, jt, jn, BodyTag<kPartIv>{}, false);
        }
      }
      else empty_tile(st, jn);
      finish();
    };

    int jt = -1;
    if (jt_lo <= jt_hi) jt = first_from(jt_lo);
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
    if constexpr (is_interval(MK)) {
      if (q0 + BQ <= nqa) {
        int f_lo = jt_lo, f_hi = min(jt_hi, nka / BK - 1);
        if (smaxg > 0) f_lo = max(f_lo, (smaxg + BK - 1) / BK);  // tiles at or past every row's lower bound
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
        tile(Stage0{}, jt, jt + 1, BodyTag<kWhole>{}, false);
        finish();
        const int jn = next_of(jt + 1);
        tile(Stage1{}, jt + 1, jn >= 0 ? jn : jt + 1, BodyTag<kWhole>{}, false);
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

// --------------------------------------------------------------- dQ, stored
// dQ from the gamma^T tiles the dK/dV kernel stored (dropout with causal /
// window masks): dQ_i = c sum_j gamma_ij K_j with no recomputation.  A
// workgroup owns 128 query rows (32 per wave) of one (batch, head) and streams
// half tiles of 32 keys -- their K rows and their half of the gamma^T block --
// through a four-stage LDS ring, three half tiles ahead (the kernel is bound
// by how many bytes it keeps in flight); both operands of
// dQ^T += K^T gamma^T are LDS transpose reads of row-major [key][column]
// tiles, so their key orders agree.  Lane l of wave w accumulates block
// column 32 w + l, i.e. query 32 w + (8 g + 4 h + r) for l = 16 h + 4 g + r
// (the column order of the stored blocks).
template <class E, int D>
__global__ __launch_bounds__(256, 2) void dense_bwd_dq_stored_kernel(const DenseArgs a, int n_qtiles) {
  constexpr int BK = 32;  // keys per half tile
  constexpr int MD = D / 32;
  constexpr int KROWB = D * 2, GROWB = 256, GSUBB = 128;
  typedef typename E::vec8 vec8;
  constexpr int KPW = TileCopy<BK, D, 4>::PER_WAVE;
  constexpr int NV = KPW + 2;  // copy instructions per wave per half tile

  // one array per (stage, tensor), so that every LDS access names its stage
  __shared__ __attribute__((aligned(16))) char ldsK0[BK * KROWB], ldsK1[BK * KROWB], ldsK2[BK * KROWB],
      ldsK3[BK * KROWB], ldsG0[BK * GROWB], ldsG1[BK * GROWB], ldsG2[BK * GROWB], ldsG3[BK * GROWB];
  auto kbuf = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return (char ETS_LDS*)ldsK0;
    else if constexpr (S == 1) return (char ETS_LDS*)ldsK1;
    else if constexpr (S == 2) return (char ETS_LDS*)ldsK2;
    else return (char ETS_LDS*)ldsK3;
  };
  auto gbuf = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return (char ETS_LDS*)ldsG0;
    else if constexpr (S == 1) return (char ETS_LDS*)ldsG1;
    else if constexpr (S == 2) return (char ETS_LDS*)ldsG2;
    else return (char ETS_LDS*)ldsG3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5, l32 = lane & 31;
  const int nq = a.nq, nk = a.nk;
  const int BH = a.B * a.H;
  const TrOps32<KROWB> ktops(lane);
  // The gamma^T half tile sits in LDS as two sub-tiles of 64 columns
  // (32 rows of 128 bytes each, sub-tile s = columns 64 s .. 64 s + 63), so
  // that each copy instruction fetches whole 128-byte runs of the stored
  // images (below).  Transpose-read offsets of this wave's 32 columns (in
  // sub-tile wave / 2): lane i of a 16-lane group addresses rows 4 h + i / 4
  // (and 8 + 4 h + i / 4) of a 16-row group at column 32 (wave % 2) + 16 g +
  // 4 (i % 4) (as TrOps32 does for a fixed column block; the swizzle depends on
  // the row modulo 16 only).
  int gt[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
    gt[sec] = (wave >> 1) * (BK * GSUBB) +
              toff<GSUBB>(4 * h32 + 8 * sec + ((lane & 15) >> 2), 32 * (wave & 1) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  auto gread = [&](const char ETS_LDS* base, int R) __attribute__((always_inline)) {
    const s16x4 x = lds_tr4(base, gt[0] + R * GSUBB), y = lds_tr4(base, gt[1] + R * GSUBB);
    const s16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(u32x4, v);
  };
  const TileCopy<BK, D, 4> kcopy(wave, lane);
  // gamma^T half-tile copy: instruction k = 2 wave + u (u = 0, 1) fills the
  // 64 chunk positions 64 (k % 4) .. of sub-tile s = k / 4, i.e. lane l fills
  // row r = 8 (k % 4) + l / 8, logical chunk c = phys_chunk(r, l % 8) of the
  // sub-tile; row 32 half + r, chunk 8 s + c of the block sits in image
  // 8 s + 4 half + ((c / 4) % 2) 2 + c % 2, lane 32 ((c / 2) % 2) + r, so the
  // instruction reads 8 runs of 8 consecutive 16-byte lanes (offsets below for
  // half 0; half 1 is four images on)
  int goff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = 2 * wave + u, r = 8 * (k & 3) + (lane >> 3), c = phys_chunk<GSUBB>(r, lane & 7);
    goff[u] = ((k >> 2) * 8 + ((c >> 2) & 1) * 2 + (c & 1)) * 1024 + (32 * ((c >> 1) & 1) + r) * 16;
  }
  // this lane's query within the workgroup's 128 rows
  const int qlane = 32 * wave + 8 * ((l32 & 15) >> 2) + 4 * (l32 >> 4) + (l32 & 3);
  const size_t per = (size_t)a.gam_per_bh * kGamBlockBytes;

  const int G = (int)gridDim.x, n_items = n_qtiles * BH;
  for (int r = 0; r * G < n_items; ++r) {
    const int item = r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    if (item >= n_items) continue;
    const int qt = n_qtiles - 1 - item / BH;  // most key tiles first
    const int bh = item % BH;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
    int lo, hi;
    gam_range(a.mask, qt, nq, nk, lo, hi);
    const __amdgpu_buffer_rsrc_t Krs =
        make_rsrc((const uint16_t*)a.K + (size_t)(b * a.Hkv + g) * nk * D, (uint32_t)nk * D * 2);
    const __amdgpu_buffer_rsrc_t Grs = make_rsrc((const char*)a.Gam + (size_t)bh * per, (uint32_t)per);
    const int blk0 = (int)gam_block(a.gam_stride, qt, 0, lo);  // block of key tile 0
    const int t0 = 2 * lo, t1 = 2 * hi + 1;                    // half tiles t0 .. t1 (none when hi < lo)

    f32x16 dq[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) dq[md][r2] = 0.f;

    // half tile t (keys 32 t .. 32 t + 31) into stage st: NV instructions per wave
    auto copy = [&](int t, auto st) __attribute__((always_inline)) {
      kcopy.issue(kbuf(st), Krs, t * BK, nk - 1);
      const int boff = (blk0 + (t >> 1)) * kGamBlockBytes + (t & 1) * 4096;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Grs, (void ETS_LDS*)(gbuf(st) + (wave >> 1) * (BK * GSUBB) + ((2 * wave + u) & 3) * 1024), 16, goff[u],
            boff, 0, 0);
    };
    // half tile t on stage st: wait for its copies (the loads complete in
    // order; the copies of up to two later half tiles may stay in flight),
    // publish them, refill the stage read one step before with half tile
    // t + 3, then the products
    auto step = [&](auto st, int t) __attribute__((always_inline)) {
      constexpr int S = decltype(st)::value;
      if (t + 2 <= t1) wait_vm_n<2 * NV>();
      else if (t + 1 <= t1) wait_vm_n<NV>();
      else wait_vm();
      __syncthreads();
      if (t + 3 <= t1) copy(t + 3, std::integral_constant<int, (S + 3) % 4>{});
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const vec8 gop = as_vec8<E>(gread(gbuf(st), 16 * kh));
#pragma unroll
        for (int md = 0; md < MD; ++md)
          dq[md] = E::mfma32(as_vec8<E>(ktops.read(kbuf(st), 16 * kh, md)), gop, dq[md]);
      }
    };
    wait_vm();  // the previous item's dQ stores: only this item's copies are counted below
    if (t0 <= t1) {
      copy(t0, std::integral_constant<int, 0>{});
      if (t0 + 1 <= t1) copy(t0 + 1, std::integral_constant<int, 1>{});
      if (t0 + 2 <= t1) copy(t0 + 2, std::integral_constant<int, 2>{});
    }
    // the count of half tiles is even: groups of four, then at most one pair
    int t = t0;
    for (; t + 3 <= t1; t += 4) {
      step(std::integral_constant<int, 0>{}, t);
      step(std::integral_constant<int, 1>{}, t + 1);
      step(std::integral_constant<int, 2>{}, t + 2);
      step(std::integral_constant<int, 3>{}, t + 3);
    }
    if (t <= t1) {
      step(std::integral_constant<int, 0>{}, t);
      step(std::integral_constant<int, 1>{}, t + 1);
    }
    __syncthreads();  // every wave is done with the ring before the next item refills it

    const int qi = qt * 128 + qlane;
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
  if (a.Gam && mk == kArith) {
    const int n_qtiles = (a.nq + 127) / 128;
    const int n_items = n_qtiles * a.B * a.H;
    int slots = 0;
    ETS_TRY(resident_slots(dense_bwd_dq_stored_kernel<E, D>, 256, &slots));
    ETS_TRY(launch((dense_bwd_dq_stored_kernel<E, D>), dim3(min(n_items, slots)), dim3(256), 0, st, a, n_qtiles));
    return 0;
  }
  if (a.drop.enabled) {
    if (mk == kArith) return launch_dq_k<E, D, kArith, true>(a, st);
    if (mk == kLayout) return launch_dq_k<E, D, kLayout, true>(a, st);
    if (mk == kBlock) return launch_dq_k<E, D, kBlock, true>(a, st);
    return launch_dq_k<E, D, kDenseM, true>(a, st);
  }
  if (mk == kArith) return launch_dq_k<E, D, kArith, false>(a, st);
  if (mk == kLayout) return launch_dq_k<E, D, kLayout, false>(a, st);
  if (mk == kBlock) return launch_dq_k<E, D, kBlock, false>(a, st);
  return launch_dq_k<E, D, kDenseM, false>(a, st);
}

#if !defined(ETS_DT) || !defined(ETS_D)
#error "compiled once per (dtype, head width): -DETS_DT=<1|2> -DETS_D=<64|128>"
#endif
template <>
int launch_dense_dq_ed<ETS_DT, ETS_D>(const DenseArgs& a, void* stream) {
  using E = std::conditional_t<ETS_DT == (int)Dt::BF16, BF16, F16>;
  return launch_dq<E, ETS_D>(a, (hipStream_t)stream);
}

}  // namespace ets
