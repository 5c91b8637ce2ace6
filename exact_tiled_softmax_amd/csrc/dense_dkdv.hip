// Dense masked attention backward, key-major dK/dV kernel (bf16/fp16 MFMA,
// gfx950).  The operation and the split into three kernels are described in
// dense_bwd.hip.
//
// A workgroup owns 128 keys of one K/V head, keeps its K and V rows in
// registers as MFMA B operands, and walks every query tile (and every query
// head of the group) that can see them; S = Q K^T and dP = G V^T put keys
// along lanes, so P and gamma feed dV^T += G^T P and dK^T += Q^T gamma
// directly, with G^T and Q^T read by LDS transpose reads.  No atomics.
#include "device.hpp"

namespace ets {

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
// first group.  d = 128 runs one wave per SIMD (the accumulators and the
// wave's K, V rows need more than half the register file); d = 64 runs two
// workgroups per compute unit, whose steps are short enough that a second
// workgroup hiding the other's memory waits pays for the few registers it
// spills (measured on the masked workload: 127 -> 108 us).
template <class E, int D, int MK, bool DROP>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void dense_bwd_dkdv_kernel(const DenseArgs a, int n_kblocks) {
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
  // copies into the other.  L: LSE2 (128 floats), D (128 floats), then the
  // row lower bounds (starts, 128 ints used) when the layout has them.
  __shared__ __attribute__((aligned(16))) char ldsQ0[TILEB], ldsG0[TILEB], ldsQ1[TILEB], ldsG1[TILEB];
  __shared__ __attribute__((aligned(16))) char ldsL0[2048], ldsL1[2048];
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
  // stored gamma (see DenseArgs::Gam): with dropout, causal / window masks only
  constexpr bool kGam = MK == kArith && DROP;
  const bool gam_on = kGam && a.Gam != nullptr;
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
    // active extents and row lower bounds of this batch
    const Layout lay = layout_of<MK>(a.mask, b, nq, nk);
    const int nqa = lay.len, nka = lay.nka;
    // Stored gamma^T (causal / window masks only): this wave's 32 keys are
    // rows 32 (wave & 1) .. + 31 of key tile k0 / 64 + wave / 2, and a step's
    // 64 queries fill columns (qb0 & 64) .. + 63 of query tile qb0 / 128.  A
    // block is stored as 16 register images of 1 KiB (one store instruction
    // each, lane l at byte 16 l): image (qb0 & 64) / 8 + 4 (wave & 1) + 2 mq + u
    // holds, in lane 32 h + r, the 16-byte chunk 4 mq + 2 h + u of the step's
    // columns of row 32 (wave & 1) + r, i.e. columns 32 mq + 16 h + 8 u .. + 7
    // (the dQ kernel's tile copy gathers the chunks back into rows).
    const int gam_jt = (k0 >> 6) + (wave >> 1);
    const uint32_t gam_voff = (uint32_t)(16 * lane);
    // the wave's block of step (qb0, bh) in the dQ kernel's tile set: resource
    // over the (batch, head)'s blocks and the byte offset of its columns
    auto gam_target = [&](int qb0, int bh, __amdgpu_buffer_rsrc_t& rs, uint32_t& soff) __attribute__((always_inline)) {
      int lo, hi;
      const int qt = qb0 >> 7;
      gam_range(a.mask, qt, nq, nk, lo, hi);
      if (gam_jt < lo || gam_jt > hi) return false;
      const size_t per = (size_t)a.gam_per_bh * kGamBlockBytes;
      rs = make_rsrc((const char*)a.Gam + (size_t)bh * per, (uint32_t)per);
      soff = (uint32_t)(gam_block(a.gam_stride, qt, gam_jt, lo) * kGamBlockBytes) +
             (uint32_t)(((qb0 & 64) / 8 + 4 * (wave & 1)) * 1024);
      return true;
    };

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
    int qt_lo = 0, qt_hi = nqa > 0 ? (nqa - 1) / BQ : -1;
    if (a.mask.causal) qt_lo = k0 / BQ;
    if (a.mask.window > 0) qt_hi = min(qt_hi, (klast + a.mask.window - 1) / BQ);
    // with stored gamma, whole 128-query tiles: the dQ kernel reads both halves
    if (gam_on) qt_hi = min(nqa > 0 ? (nqa - 1) / BQ : -1, qt_hi | 1);
    const int n_qt = qt_hi - qt_lo + 1;
    const int total = (n_qt > 0) ? n_qt * grp : 0;
    // step classes of the per-element mask kinds, 64 steps at a time (row
    // lower bounds vary per step: with them a step is never taken as full
    // here, and the per-element test applies them)
    TileClasses tc;
    tc.base = -1;
    auto classes_for = [&](int s0) __attribute__((always_inline)) {
      if (tc.covers(s0)) return;
      const int s = s0 + lane;
      int cg = kEmpty, cw = kEmpty;
      if (s < total) {
        const int qb = (qt_lo + s % n_qt) * BQ;
        cg = classify<MK>(a.mask, qb, qb + BQ - 1, k0, k0 + 127, nqa, nka);
        cw = classify<MK>(a.mask, qb, qb + BQ - 1, kw0, kw0 + 31, nqa, nka);
        if (lay.st && (cw & kClassMask) == kFull) cw = kPartial;
      }
      tc.set(s0, cg, cw);
    };
    auto first_from = [&](int s) {  // first step >= s the workgroup's keys see, or -1
      if constexpr (is_interval(MK)) {
        return s < total ? s : -1;
      } else {
        while (s < total) {
          classes_for(s);
          const int f = tc.next_nonempty(s);
          if (f >= 0) return f < total ? f : -1;
          s = tc.base + 64;
        }
        return -1;
      }
    };
    auto next_of = [&](int st) { return first_from(st + 1); };
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
    const __amdgpu_buffer_rsrc_t Srs = make_rsrc(lay.st, lay.st ? (uint32_t)nq * 4u : 0u);
    auto copy_lse = [&](int st, auto stg) __attribute__((always_inline)) {
      if (wave == 0) {
        size_t lo;
        int qb0;
        step_rows(st, lo, qb0);
        const uint32_t off = (uint32_t)((lo + qb0 + 4 * l32) * 4) + (h32 ? 0u : lse_off);
        copy16_to_lds(Wrs, off, (void ETS_LDS*)lbuf(stg));
      } else if (wave == 1 && lay.st) {  // starts of rows qb0 .. qb0+255 to bytes 1024-2047
        size_t lo;
        int qb0;
        step_rows(st, lo, qb0);
        copy16_to_lds(Srs, (uint32_t)(qb0 + 4 * lane) * 4u, (void ETS_LDS*)(lbuf(stg) + 1024));
      }
    };
    // lowest and highest lower bound of the active rows of the step on stage
    // stg (its starts are in LDS once the step begins)
    auto step_start_range = [&](auto stg, int qb0, int& smin, int& smax) __attribute__((always_inline)) {
      const int ETS_LDS* sl = (const int ETS_LDS*)(lbuf(stg) + 1024);
      int lo = 0x7fffffff, hi = (int)0x80000000;
      if (qb0 + lane < nqa) lo = hi = sl[lane];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        lo = min(lo, __shfl_xor(lo, off, 64));
        hi = max(hi, __shfl_xor(hi, off, 64));
      }
      smin = lo;
      smax = hi;
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
      int ilo = 0, ihi = nqa - 1;
      if (a.mask.causal) ilo = max(ilo, key);
      if (a.mask.window > 0) ihi = min(ihi, key + a.mask.window - 1);
      const bool any = key < nka && ilo <= ihi;
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
                       auto part_tag, bool cbm, const char ETS_LDS* lb) __attribute__((always_inline)) {
      constexpr bool PART = decltype(part_tag)::value != kWhole;
      const int g4 = k / 2, half = k % 2;
      const int qr = 32 * mq + 8 * g4 + 4 * h32;
      if (half == 0) {
        w.allow[g4] = 0xFu;
        if constexpr (PART) {
          if constexpr (decltype(part_tag)::value == kPartIv) {
            int lo;
            unsigned rng;
            arith_interval(qb0 + qr, lo, rng);
            unsigned al = 0;
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) al |= ((unsigned)(r2 - lo) <= rng ? 1u : 0u) << r2;
            if (lay.st) {  // row lower bounds (starts), staged in LDS with the LSE rows
              const i32x4 s4 = *(const i32x4 ETS_LDS*)(lb + 1024 + 4 * qr);
              al &= (s4[0] <= key ? 1u : 0u) | (s4[1] <= key ? 2u : 0u) | (s4[2] <= key ? 4u : 0u) |
                    (s4[3] <= key ? 8u : 0u);
            }
            w.allow[g4] = al;
          } else {
            w.allow[g4] = allowed4_rows<MK>(a.mask, qb0 + qr, key, nqa, nka, cbm, lay.st);
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

    // Stored gamma: block 0 of a step is written during B(0); block 1, whose
    // gamma is complete only at the end of B(0), is kept (g1) and written
    // during the first group of the next step (or by g1_flush), so that the
    // vmcnt wait at the end of a step does not wait for stores issued just
    // before it.
    uint32_t g1[8];
    bool g1_pend = false;
    __amdgpu_buffer_rsrc_t g1_rs = make_rsrc(a.Gam, 0u);
    uint32_t g1_soff = 0;
    auto g1_store = [&](int u) __attribute__((always_inline)) {
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{g1[4 * u], g1[4 * u + 1], g1[4 * u + 2], g1[4 * u + 3]}, g1_rs,
                                             gam_voff, g1_soff + (2 + u) * 1024, 0);
    };
    auto g1_flush = [&]() __attribute__((always_inline)) {
      if constexpr (kGam) {
        if (g1_pend) {
          g1_store(0);
          g1_store(1);
        }
        g1_pend = false;
      }
    };
    // one step on stage stg; its successor's rows go into the other stage
    auto step = [&](auto stg, int st, int sn, auto part_tag, bool cbm) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(stg)::value> Next;
      size_t lo;
      int qb0;
      step_rows(st, lo, qb0);
      const int lane_bh = (int)(lo / nq);
      __amdgpu_buffer_rsrc_t grs = make_rsrc(a.Gam, 0u);
      uint32_t gsoff = 0;
      const bool gst = gam_on && gam_target(qb0, lane_bh, grs, gsoff);
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
          // the previous step's block 1
          if constexpr (kGam && gi == 0 && (u == 2 || u == 5)) {
            if (g1_pend) g1_store(u == 2 ? 0 : 1);
          }
        } else {
          constexpr int kh = u / (2 * MD), md = (u % (2 * MD)) / 2;
          if constexpr (u & 1) dk[md] = E::mfma32(op, pack_op(w[mq].gw, kh), dk[md]);
          else dv[md] = E::mfma32(op, pack_op(w[mq].pw, kh), dv[md]);
          // stored gamma: the block's gamma (complete before B(mq)) to its image
          if constexpr (kGam && mq == 0 && u < 2) {
            if (gst)
              __builtin_amdgcn_raw_buffer_store_b128(
                  u32x4{w[mq].gw[4 * u], w[mq].gw[4 * u + 1], w[mq].gw[4 * u + 2], w[mq].gw[4 * u + 3]}, grs,
                  gam_voff, gsoff + (2 * mq + u) * 1024, 0);
          }
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
            if constexpr ((k * gsz) / 8 == u) weights(w[wq], sc[wq], dp[wq], k, wq, qb0, lane_bh, part_tag, cbm, lbuf(stg));
          });
        }
        ETS_FENCE();
      });
      if constexpr (kGam) {
#pragma unroll
        for (int k = 0; k < 8; ++k) g1[k] = w[1].gw[k];
        g1_pend = gst;
        g1_rs = grs;
        g1_soff = gsoff;
      }
    };
    auto empty_step = [&](auto stg, int st, int sn) __attribute__((always_inline)) {
      typedef std::integral_constant<int, 1 - decltype(stg)::value> Next;
      copy_lse(sn, Next{});
#pragma unroll
      for (int u = 0; u < NCOPY; ++u) copy_one(sn, Next{}, u);
      g1_flush();
      if (gam_on) {  // no allowed pair: a zero block part where the dQ kernel reads one
        size_t lo;
        int qb0;
        step_rows(st, lo, qb0);
        __amdgpu_buffer_rsrc_t grs = make_rsrc(a.Gam, 0u);
        uint32_t gsoff = 0;
        if (gam_target(qb0, (int)(lo / nq), grs, gsoff)) {
          const u32x4 z = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int mq = 0; mq < BQ / 32; ++mq)  // the wave's four images
#pragma unroll
            for (int u = 0; u < 2; ++u) __builtin_amdgcn_raw_buffer_store_b128(z, grs, gam_voff, gsoff + (2 * mq + u) * 1024, 0);
        }
      }
    };
    auto finish = [&]() __attribute__((always_inline)) {
      wait_vm();
      __syncthreads();
    };
    auto general_step = [&](auto stg, int st, int sn) __attribute__((always_inline)) {
      size_t lo;
      int qb0;
      step_rows(st, lo, qb0);
      int cinfo;
      if constexpr (is_interval(MK)) {
        int smin = (int)0x80000000, smax = (int)0x80000000;
        if (lay.st) step_start_range(stg, qb0, smin, smax);
        cinfo = classify<MK>(a.mask, qb0, qb0 + BQ - 1, kw0, kw0 + 31, nqa, nka, smin, smax);
      } else {
        classes_for(st);
        cinfo = tc.wave_class(st);
      }
      const int cls = cinfo & kClassMask;
      if (cls == kFull) {
        step(stg, st, sn, BodyTag<kWhole>{}, false);
      } else if (cls == kPartial) {
        // a tile mask that is uniform over the wave's rectangle leaves only the interval parts
        if constexpr (MK == kDenseM) step(stg, st, sn, BodyTag<kPartEl>{}, (cinfo & kCheckBlockMask) != 0);
        else if constexpr (MK == kBlock) {
          if (cinfo & kCheckBlockMask) step(stg, st, sn, BodyTag<kPartEl>{}, true);
          else step(stg, st, sn, BodyTag<kPartIv>{}, false);
        } else {
          step(stg, st, sn, BodyTag<kPartIv>{}, false);
        }
      }
      else empty_step(stg, st, sn);
      finish();
    };

    int st = -1;
    if (total > 0) st = first_from(0);
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
    if constexpr (is_interval(MK)) {
      // local q-tile indices i (qb0 = (qt_lo + i) BQ) whose rows see all 128 keys
      // (row lower bounds are not known per step here: none with starts)
      int i_lo = 0, i_hi = n_qt - 1;
      if (k0 + 127 >= nka || lay.st) i_hi = -1;
      i_hi = min(i_hi, nqa / BQ - 1 - qt_lo);
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
          step(Stage0{}, st, st + 1, BodyTag<kWhole>{}, false);
          finish();
          const int sn = next_of(st + 1);
          step(Stage1{}, st + 1, sn >= 0 ? sn : st + 1, BodyTag<kWhole>{}, false);
          finish();
        }
        if (st >= total) st = -1;
      }
    }
    general_until(1 << 30);
    g1_flush();

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
    if (mk == kLayout) return launch_dkdv_k<E, D, kLayout, true>(a, st);
    if (mk == kBlock) return launch_dkdv_k<E, D, kBlock, true>(a, st);
    return launch_dkdv_k<E, D, kDenseM, true>(a, st);
  }
  if (mk == kArith) return launch_dkdv_k<E, D, kArith, false>(a, st);
  if (mk == kLayout) return launch_dkdv_k<E, D, kLayout, false>(a, st);
  if (mk == kBlock) return launch_dkdv_k<E, D, kBlock, false>(a, st);
  return launch_dkdv_k<E, D, kDenseM, false>(a, st);
}

#if !defined(ETS_DT) || !defined(ETS_D)
#error "compiled once per (dtype, head width): -DETS_DT=<1|2> -DETS_D=<64|128>"
#endif
template <>
int launch_dense_dkdv_ed<ETS_DT, ETS_D>(const DenseArgs& a, void* stream) {
  using E = std::conditional_t<ETS_DT == (int)Dt::BF16, BF16, F16>;
  return launch_dkdv<E, ETS_D>(a, (hipStream_t)stream);
}

}  // namespace ets
