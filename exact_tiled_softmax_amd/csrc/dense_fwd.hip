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
//   * a workgroup owns BQ = NW x 32 query rows of one (batch, head); each
//     wave keeps its 32 Q rows in registers as the B operand of S^T = K Q^T
//     (v_mfma_f32_32x32x16, queries along lanes, keys along the accumulator
//     rows), so a query's running max and sum live in one lane plus its
//     partner lane l ^ 32;
//   * K and V tiles of 64 keys go straight from HBM into a two-stage LDS ring
//     (buffer_load ... lds, swizzled rows); the copy of the next tile is issued
//     while the current one is used.  The PV product is accumulated
//     transposed, O^T += V^T P^T, with V^T read by ds_read_b64_tr_b16 and P^T
//     fed straight from the S^T accumulators (no shuffles);
//   * a 64-key tile is consumed as two 32-key blocks, each a full
//     online-summary step, in the order
//       S(0) | S(1) + summary(0) | PV(0) + summary(1) | PV(1)
//     so that the VALU work of one block (max, exponentials, packing) is
//     issued between the MFMAs of the other.  The order is fixed by hand,
//     one MFMA per slot with its operand reads two slots ahead; tiles that a
//     wave's rows see only in part apply the mask in the same slots (for
//     causal and window masks as one key interval per row);
//   * scores are kept in base 2 (c*log2 e folded into one FMA before
//     v_exp_f32); the reference maximum of a row is only raised when a block's
//     maximum exceeds it by more than kRescaleSlack (log2 units), which keeps
//     every weight <= 2^kRescaleSlack and skips most rescales of the O
//     accumulators.  Any reference value gives the same z / l exactly, so the
//     result is unchanged up to rounding; the LSE uses the final reference.
#include "device.hpp"

namespace ets {

constexpr float kRescaleSlack = 8.0f;

template <class E, int D, int NW, int MK, bool DROP>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : (D == 64 ? 3 : 2)) void dense_fwd_kernel(const DenseArgs a, int n_qtiles) {
  constexpr int BK = 64;
  constexpr int BQ = NW * 32;
  constexpr int KS = D / 16;        // k-steps of the score contraction
  constexpr int MD = D / 32;        // 32-row blocks of O^T
  constexpr int ROWB = D * 2;       // bytes per LDS tile row
  constexpr int TILEB = BK * ROWB;  // bytes per K or V tile
  typedef typename E::vec8 vec8;
  typedef std::integral_constant<int, 0> Stage0;
  typedef std::integral_constant<int, 1> Stage1;

  // LDS ring, one array per (stage, K or V): the compiler can then tell the
  // tile being read from the tile still arriving, so a read of one stage
  // does not wait for the copies into the other
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

  // Persistent workgroups: workgroup w of G takes items w, 2G-1-w, 2G+w, ...
  // (boustrophedon over the heaviest-first list), which balances the causal
  // triangle without atomics and keeps every slot busy until the end.
  const int G = (int)gridDim.x, n_items = n_qtiles * a.B * a.H;
  auto item_of = [&](int r) { return r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x); };
  // key-tile range of query tile qt for active extents nqa x nka and row
  // lower bounds >= smin (an empty range when hi < lo)
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
  // (with equal priorities the older one wins every tie, and the younger one
  // ends alone on the unit).  rem is uniform: a scalar.
  int rem = 0;
  for (int r = 0; r * G < n_items; ++r) {
    const int item = item_of(r);
    if (item >= n_items) continue;
    int lo, hi;
    const int nqa = (MK != kArith && a.mask.lengths) ? min(max(a.mask.lengths[(item % (a.B * a.H)) / a.H], 0), a.nq) : a.nq;
    tile_range(n_qtiles - 1 - item / (a.B * a.H), nqa, (MK != kArith && a.mask.lengths) ? min(nqa, a.nk) : a.nk, 0, lo, hi);
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
    // work item = one query tile of one (batch, head); items are numbered
    // heaviest first and consecutive items walk (batch, head)
    const int BH = a.B * a.H;
    const int qt = n_qtiles - 1 - item / BH;
    const int bh = item % BH;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.Hkv);
    const int nq = a.nq, nk = a.nk;
    const int q0 = qt * BQ, qw0 = q0 + wave * 32;
    const int qi = qw0 + l32;  // this lane's query row
    // active extents and row lower bounds of this batch; smin/smax bound the
    // lower bounds of the wave's (w) and the workgroup's (g) active rows
    const Layout lay = layout_of<MK>(a.mask, b, nq, nk);
    const int nqa = lay.len, nka = lay.nka;
    int sminw = (int)0x80000000, smaxw = (int)0x80000000, sming = sminw, smaxg = smaxw;
    int st_i = (int)0x80000000;  // lower bound of this lane's row
    if (lay.st) {
      start_range(lay.st, qw0, qw0 + 31, nqa, lane, sminw, smaxw);
      start_range(lay.st, q0, q0 + BQ - 1, nqa, lane, sming, smaxg);
      if (qi < nqa) st_i = lay.st[qi];
    }

    const uint16_t* Qp = (const uint16_t*)a.Q + (size_t)bh * nq * D;
    const uint16_t* Kp = (const uint16_t*)a.K + (size_t)(b * a.Hkv + g) * nk * D;
    const uint16_t* Vp = (const uint16_t*)a.V + (size_t)(b * a.Hkv + g) * nk * D;
    const __amdgpu_buffer_rsrc_t Krs = make_rsrc(Kp, (uint32_t)nk * D * 2);
    const __amdgpu_buffer_rsrc_t Vrs = make_rsrc(Vp, (uint32_t)nk * D * 2);

    // Q rows of this wave as B operands: lane holds query qi, features
    // 16kk + 8h32 .. +7
    vec8 qreg[KS];
  #pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = u32x4{0, 0, 0, 0};
      if (qi < nq) v = *(const u32x4*)(Qp + (size_t)qi * D + 16 * kk + 8 * h32);
      qreg[kk] = as_vec8<E>(v);
    }

    f32x16 oacc[MD];
  #pragma unroll
    for (int md = 0; md < MD; ++md)
  #pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] = 0.f;
    float mref = kNegInf, lsum = 0.f;

    // key-tile range of the workgroup
    int jt_lo, jt_hi;
    tile_range(qt, nqa, nka, sming, jt_lo, jt_hi);

    const TileCopy<BK, D, NW> tcopy(wave, lane);
    constexpr int NCOPY = 2 * TileCopy<BK, D, NW>::PER_WAVE;  // copy instructions per wave per tile
    // copy instruction u of tile jt into stage st: K rows first, then V rows
    // (rows past nk read row nk-1; those keys are masked as a ragged tile)
    auto copy_one = [&](int jt, auto st, int u) __attribute__((always_inline)) {
      constexpr int PW = TileCopy<BK, D, NW>::PER_WAVE;
      if (u < PW) tcopy.issue_one(kbuf(st), Krs, jt * BK, nk - 1, u);
      else tcopy.issue_one(vbuf(st), Vrs, jt * BK, nk - 1, u - PW);
    };

    const float sl2 = a.scale_log2;
    const RowOps32<ROWB> kops(lane);
    const TrOps32<ROWB> vops(lane);

    // ---------------------------------------------------------------- pieces
    // MFMA operand t of a tile, in slot order: K rows for S(0) (t < KS) and
    // S(1) (t < 2KS), then V^T for PV(0) and PV(1), each in (kh, md) order
    constexpr int NOPS = 2 * KS + 4 * MD;
    auto operand = [&](const char ETS_LDS* kt, const char ETS_LDS* vt, int t) __attribute__((always_inline)) {
      if (t < 2 * KS) return as_vec8<E>(lds_b128(kt, kops.off(32 * (t / KS), t % KS)));
      const int u = t - 2 * KS, mb = u / (2 * MD), kh = (u / MD) % 2, md = u % MD;
      return as_vec8<E>(vops.read(vt, 32 * mb + 16 * kh, md));
    };

    // Online summary step for one 32-key block, split into 7 parts that are
    // spread over MFMA slots.  Block keys of accumulator entry r: key0 + 8(r/4)
    // + 4h32 + r%4 with key0 = j0 + 32mb.  In a masked block (PART) the scores
    // are scaled to base 2 first and disallowed ones set to -inf, so a row with
    // no allowed key in the block raises nothing and gets zero weights.
    struct Summary {
      float mx, alpha, mneg;
      bool need;
      uint32_t packed[8];
      unsigned keep;  // dropout: bit 8 g4 + r keeps key key0 + 8 g4 + 4 h32 + r
    };
    // allowed keys of this lane's row form one interval for arithmetic masks:
    // key0 + c allowed iff lo <= c <= lo + rng (unsigned compare of c - lo)
    auto arith_interval = [&](int key0, int& lo, unsigned& rng) __attribute__((always_inline)) {
      int jlo = max(0, st_i), jhi = nka - 1;
      if (a.mask.causal) jhi = min(jhi, qi);
      if (a.mask.window > 0) jlo = max(jlo, qi - a.mask.window + 1);
      const int base = key0 + 4 * h32;
      const bool any = qi < nqa && jlo <= jhi;
      lo = any ? jlo - base : (1 << 24);
      rng = any ? (unsigned)(jhi - jlo) : 0u;
    };
    auto mask_scale = [&](f32x16& s, int r0, int key0, bool cbm, auto body) __attribute__((always_inline)) {
      if constexpr (decltype(body)::value == kPartIv) {
        int lo;
        unsigned rng;
        arith_interval(key0, lo, rng);
  #pragma unroll
        for (int r = r0; r < r0 + 8; ++r) {
          const int c = 8 * (r / 4) + r % 4;
          s[r] = ((unsigned)(c - lo) <= rng) ? s[r] * sl2 : kNegInf;
        }
      } else {
  #pragma unroll
        for (int g4 = r0 / 4; g4 < r0 / 4 + 2; ++g4) {
          const unsigned allow = allowed4<MK>(a.mask, qi, key0 + 8 * g4 + 4 * h32, nqa, nka, cbm, lay.st);
  #pragma unroll
          for (int r = 0; r < 4; ++r) s[4 * g4 + r] = ((allow >> r) & 1u) ? s[4 * g4 + r] * sl2 : kNegInf;
        }
      }
    };
    auto summary_part = [&](Summary& st, f32x16& s, auto part_c, auto part_tag, int key0, bool cbm)
                            __attribute__((always_inline)) {
      constexpr int part = decltype(part_c)::value;
      constexpr bool PART = decltype(part_tag)::value != kWhole;
      if constexpr (part == 0) {
        if constexpr (PART) mask_scale(s, 0, key0, cbm, part_tag);
        st.mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  #pragma unroll
        for (int r = 4; r < 8; ++r) st.mx = fmaxf(st.mx, s[r]);
      } else if constexpr (part == 1) {
        if constexpr (PART) mask_scale(s, 8, key0, cbm, part_tag);
  #pragma unroll
        for (int r = 8; r < 16; ++r) st.mx = fmaxf(st.mx, s[r]);
      } else if constexpr (part == 2) {
        const float mx = xhalf_max(st.mx);
        const float mt = PART ? mx : mx * sl2;
        st.need = mt > mref + kRescaleSlack;
        st.alpha = st.need ? fast_exp2(mref - mt) : 1.f;
        mref = st.need ? mt : mref;
        lsum *= st.alpha;
        st.mneg = (PART && mref == kNegInf) ? 0.f : -mref;
      } else {
        constexpr int g4 = part - 3;  // 0..3: accumulator entries 4g4 .. 4g4+3
        float p[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r)
          p[r] = PART ? fast_exp2(s[4 * g4 + r] + st.mneg) : fast_exp2(fmaf(s[4 * g4 + r], sl2, st.mneg));
  #pragma unroll
        for (int r = 0; r < 4; ++r) lsum += p[r];  // the normaliser counts dropped weights too
        if constexpr (DROP) {
  #pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!((st.keep >> (8 * g4 + r)) & 1u)) p[r] = 0.f;
        }
        st.packed[2 * g4] = E::pack2(p[0], p[1]);
        st.packed[2 * g4 + 1] = E::pack2(p[2], p[3]);
        // computed here, not sunk to the PV product behind the rescale branch
        // or to the end of the loop
        materialize(st.packed[2 * g4]);
        materialize(st.packed[2 * g4 + 1]);
        materialize(lsum);
      }
    };
    // P^T operand for k-step kh (16 keys) of a block: accumulator entries 8kh .. 8kh+7
    auto pt_operand = [&](const Summary& st, int kh) __attribute__((always_inline)) {
      return as_vec8<E>(u32x4{st.packed[4 * kh], st.packed[4 * kh + 1], st.packed[4 * kh + 2], st.packed[4 * kh + 3]});
    };
    auto rescale = [&](const Summary& st) __attribute__((always_inline)) {
      if (wave_any(st.need)) {
  #pragma unroll
        for (int md = 0; md < MD; ++md)
  #pragma unroll
          for (int r = 0; r < 16; ++r) oacc[md][r] *= st.alpha;
      }
    };

    // ------------------------------------------------------------- one tile
    // One MFMA per slot, operands read two slots ahead, the copy of the next
    // tile in the S(0) slots, summary(0) in the S(1) slots and summary(1) in
    // the PV(0) slots.  Fences keep the compiler from regrouping the slots.
    // part_tag: masked tile (the wave's rows see only part of it) or whole.
    constexpr int NSLOT = NOPS;  // one MFMA per operand
    auto tile = [&](auto st, int jt, int jnext, auto part_tag, bool cbm) __attribute__((always_inline)) {
      const char ETS_LDS* kt = kbuf(st);
      const char ETS_LDS* vt = vbuf(st);
      typedef std::integral_constant<int, 1 - decltype(st)::value> Next;
      const int j0 = jt * BK;
      f32x16 s0, s1;
  #pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
      Summary sm0, sm1;
      unsigned kd[4];  // dropout draws of the tile's four blocks of 8 keys per lane pair
      vec8 opb[3];
      opb[0] = operand(kt, vt, 0);
      opb[1] = operand(kt, vt, 1);
      static_for<NSLOT>([&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t + 2 < NOPS) opb[(t + 2) % 3] = operand(kt, vt, t + 2);
        const vec8 op = opb[t % 3];
        if constexpr (t < KS) {
          s0 = E::mfma32(op, qreg[t], s0);
          static_for<NCOPY>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            if constexpr ((u * KS) / NCOPY == t) copy_one(jnext, Next{}, u);
          });
          if constexpr (DROP) {  // the keep bits of both halves, before their summaries
            static_for<4>([&](auto qc) __attribute__((always_inline)) {
              constexpr int q = decltype(qc)::value;
              if constexpr ((q * KS) / 4 == t) {
                kd[q] = keep_qm_draw(a.drop, bh, qi, j0 + 32 * (q / 2), h32, q % 2);
                if constexpr (q == 1) sm0.keep = keep_qm_merge(kd[0], kd[1], h32);
                if constexpr (q == 3) sm1.keep = keep_qm_merge(kd[2], kd[3], h32);
              }
            });
          }
        } else if constexpr (t < 2 * KS) {
          s1 = E::mfma32(op, qreg[t - KS], s1);
          static_for<7>([&](auto pc) __attribute__((always_inline)) {
            if constexpr ((decltype(pc)::value * KS) / 7 == t - KS) summary_part(sm0, s0, pc, part_tag, j0, cbm);
          });
          if constexpr (t == 2 * KS - 1) {
            ETS_FENCE();
            rescale(sm0);
          }
        } else if constexpr (t < 2 * KS + 2 * MD) {
          constexpr int u = t - 2 * KS;
          oacc[u % MD] = E::mfma32(op, pt_operand(sm0, u / MD), oacc[u % MD]);
          static_for<7>([&](auto pc) __attribute__((always_inline)) {
            if constexpr ((decltype(pc)::value * 2 * MD) / 7 == u) summary_part(sm1, s1, pc, part_tag, j0 + 32, cbm);
          });
          if constexpr (t == 2 * KS + 2 * MD - 1) {
            ETS_FENCE();
            rescale(sm1);
          }
        } else {
          constexpr int u = t - 2 * KS - 2 * MD;
          oacc[u % MD] = E::mfma32(op, pt_operand(sm1, u / MD), oacc[u % MD]);
        }
        ETS_FENCE();
      });
    };

    // a tile none of the wave's rows sees: only the copy of the next tile
    auto empty_tile = [&](auto st, int jnext) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(st)::value> Next;
  #pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(jnext, Next{}, u);
    };

    // ------------------------------------------------------------- the loop
    // The workgroup's non-empty tiles in key order, tile number p on ring stage
    // p % 2; the copy of the next tile is issued during the current one (in the
    // last one the current tile is copied again into the idle stage, which
    // keeps the issue free of branches).  For arithmetic masks the tiles are
    // jt_lo .. jt_hi, and those every row of the workgroup sees whole form one
    // range; pairs of them starting on stage 0 take the fixed-order path.
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
    int jt = -1;
    if (jt_lo <= jt_hi) jt = first_from(jt_lo);

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

    // prologue: the first tile into stage 0
    if (jt >= 0) {
  #pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(jt, Stage0{}, u);
    }
    wait_vm();
    __syncthreads();

    auto finish = [&]() __attribute__((always_inline)) {
      wait_vm();  // this wave's part of the next tile has landed
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
      // a fixed-order range exists (arithmetic masks only): general_run stopped
      // at tile number fp0 < N, so jt = jt_lo + p here and tile p + 1 is full too
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

    // ---- epilogue: Y = z / l, LSE = (m + log2 l) ln 2
    uint16_t* Yp = (uint16_t*)a.out_Y + (size_t)bh * nq * D;
    float* Lp = a.LSE + (size_t)bh * nq;
    const float l = xhalf_sum(lsum);
    float inv = (l > 0.f) ? 1.f / l : 0.f;
    if constexpr (DROP) inv *= a.drop.inv_keep;
    if (qi < nq) {
  #pragma unroll
      for (int md = 0; md < MD; ++md)
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = 32 * md + 8 * g4 + 4 * h32;
          u32x2 w;
          w[0] = E::pack2(oacc[md][4 * g4] * inv, oacc[md][4 * g4 + 1] * inv);
          w[1] = E::pack2(oacc[md][4 * g4 + 2] * inv, oacc[md][4 * g4 + 3] * inv);
          *(u32x2*)(Yp + (size_t)qi * D + col) = w;
        }
      if (h32 == 0) Lp[qi] = (l > 0.f) ? (mref + __log2f(l)) * kLn2 : kNegInf;
    }
  }
}

template <class E, int D, int NW, int MK, bool DROP>
static int launch_fwd_k(const DenseArgs& a, void* stream) {
  constexpr int BQ = NW * 32;
  const int n_qtiles = (a.nq + BQ - 1) / BQ;
  const int n_items = n_qtiles * a.B * a.H;
  int slots = 0;
  ETS_TRY(resident_slots(dense_fwd_kernel<E, D, NW, MK, DROP>, 64 * NW, &slots));
  dim3 grid(min(n_items, slots)), block(64 * NW);
  ETS_TRY(launch((dense_fwd_kernel<E, D, NW, MK, DROP>), grid, block, 0, (hipStream_t)stream, a, n_qtiles));
  return 0;
}

template <class E, int D, int NW, int MK>
static int launch_fwd_mk(const DenseArgs& a, void* stream) {
  if (a.drop.enabled) return launch_fwd_k<E, D, NW, MK, true>(a, stream);
  return launch_fwd_k<E, D, NW, MK, false>(a, stream);
}

template <class E, int D, int NW>
static int launch_fwd_t(const DenseArgs& a, void* stream) {
  switch (mask_kind(a.mask)) {
    case kArith: return launch_fwd_mk<E, D, NW, kArith>(a, stream);
    case kLayout: return launch_fwd_mk<E, D, NW, kLayout>(a, stream);
    case kBlock: return launch_fwd_mk<E, D, NW, kBlock>(a, stream);
    default: return launch_fwd_mk<E, D, NW, kDenseM>(a, stream);
  }
}

#if !defined(ETS_DT) || !defined(ETS_D)
#error "dense_fwd.hip is compiled once per (dtype, head width): -DETS_DT=<1|2> -DETS_D=<64|128>"
#endif
template <>
int launch_dense_fwd_ed<ETS_DT, ETS_D>(const DenseArgs& a, void* stream) {
  using E = std::conditional_t<ETS_DT == (int)Dt::BF16, BF16, F16>;
  return launch_fwd_t<E, ETS_D, 4>(a, stream);
}

}  // namespace ets
