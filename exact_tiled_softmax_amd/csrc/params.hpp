// Launch parameters shared by the C-ABI layer (abi.cpp) and the HIP kernels.
// Internal to the library: nothing here is part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ets {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

// The allowed-key sets A_i: the AND of every enabled part.
struct MaskArgs {
  int causal;                 // j <= i
  int window;                 // > 0: i - j < window
  const uint8_t* block_mask;  // [ceil(nq/bq)][ceil(nk/bk)] or null
  int bq, bk;                 // block_mask granularity
  int nbk;                    // ceil(nk / bk): row length of block_mask
  const uint8_t* dense_mask;  // [nq][nk] or null
  int dm_stride;              // nk: row length of dense_mask
  const int32_t* lengths;     // [B] active rows (and keys) per batch, or null
  const int32_t* starts;      // [B][nq] lowest allowed key per row, or null
};

// Inverted dropout: keep iff the key's 16-bit Philox draw >= threshold.
struct DropArgs {
  int enabled;
  uint32_t threshold;   // floor(rate * 2^16)
  uint32_t seed_lo, seed_hi;
  float inv_keep;       // 1 / (1 - rate), fp32
};

struct DenseArgs {
  const void* Q; const void* K; const void* V;
  const void* Y; const void* G;       // backward inputs (Y, G)
  void* out_Y;                        // forward output
  float* LSE;                         // forward output / backward input
  void* dQ; void* dK; void* dV;       // backward outputs
  float* Dws;                         // backward workspace: D_i = G_i . Y_i  [B*H*nq + 64]
  float* Lws;                         // backward workspace: LSE_i log2(e)    [B*H*nq + 64]
  int B, H, Hkv, nq, nk, d, dv;
  float scale;                        // c
  float scale_log2;                   // c * log2(e)
  int block_b;                        // key-block size (fp32 path)
  MaskArgs mask;
  DropArgs drop;
  // Stored-gamma form of the backward (bf16/fp16, causal and window masks
  // only): the dK/dV kernel also writes every gamma^T tile it forms into Gam,
  // and the dQ kernel reads them back instead of recomputing S and dP.  Null:
  // the dQ kernel recomputes (the layout is in gam_range / gam_block below).
  void* Gam;
  int gam_stride;                     // blocks per 128-query tile; 0 = causal triangle
  long long gam_per_bh;               // blocks per (batch, query head)
};

// Stored gamma^T blocks.  One block holds gamma^T of 64 keys x 128 queries
// (rows of 128 16-bit values, 16 KiB), for 64-key tile jt and 128-query tile
// qt of one (batch, query head).  Within a 32-query group the columns are
// permuted: column 16h + 4g + r holds query 8g + 4h + r, the order in which a
// dK/dV lane holds its 16 rows of a 32-row block.  gam_range gives the key
// tiles [lo, hi] a query tile sees under a causal / window mask (the tiles
// the dQ kernel visits; hi < lo when none), and gam_block the block index of
// (qt, jt) within its (batch, head): tiles of one query tile are consecutive,
// query tiles follow at a fixed stride, or, for causal masks without a
// window, at the triangle offsets qt (qt + 1) (query tile qt sees at most
// 2 qt + 2 key tiles).
constexpr int kGamBlockBytes = 64 * 128 * 2;
__host__ __device__ inline void gam_range(const MaskArgs& m, int qt, int nq, int nk, int& lo, int& hi) {
  const int q0 = qt * 128, qlast = (q0 + 128 < nq ? q0 + 128 : nq) - 1;
  lo = 0;
  hi = (nk - 1) / 64;
  if (nk < 1 || q0 >= nq) hi = -1;
  if (m.causal && qlast / 64 < hi) hi = qlast / 64;
  if (m.window > 0) {
    const int l = (q0 - m.window + 1) / 64;
    lo = l > 0 ? l : 0;
  }
}
__host__ __device__ inline long long gam_block(int stride, int qt, int jt, int lo) {
  return (stride ? (long long)qt * stride : (long long)qt * (qt + 1)) + (jt - lo);
}
// Blocks per (batch, head) and the stride for a causal / window mask
__host__ __device__ inline long long gam_blocks_per_bh(const MaskArgs& m, int nq, int nk, int& stride) {
  const int nqt = (nq + 127) / 128, nkt = (nk + 63) / 64;
  if (m.causal && m.window <= 0) {
    stride = 0;
    return (long long)nqt * (nqt + 1);
  }
  stride = nkt;
  if (m.causal && m.window > 0 && (m.window + 126) / 64 + 2 < nkt) stride = (m.window + 126) / 64 + 2;
  return (long long)nqt * stride;
}

struct SparseArgs {
  const void* Q; const void* KV;
  const int32_t* idx; const int32_t* length;  // [Tq][topk], [Tq] or null
  const float* sink;                          // [H] or null
  void* O; float* LSE;
  const void* dO;
  void* dQ; void* dKV; float* dSink;
  float* Dws;        // [Tq*H]  D = dO . O
  float* dsink_part; // [Tq*H]  -p_sink D per (token, head)
  float* dKVws;      // [Tkv*dqk] fp32 accumulation
  int Tq, H, Tkv, dqk, dv, topk;
  float scale, scale_log2;
  int lse_kv;        // 1: the LSE written / read covers the selected KV logits only (no sink)
  int det;           // 1: dKVws holds int64 fixed point (units of 2^-32), summed with integer atomics
};

// Kernel launchers (defined in the .hip files).  Each returns 0 on success or
// a hipError_t value.  They assume validated arguments.
int launch_dense_fwd(const DenseArgs& a, Dt dt, void* stream);

// The MFMA kernels of one (dtype, head width): dense_fwd.hip, dense_dkdv.hip
// and dense_dq.hip are each compiled once per combination (-DETS_DT, -DETS_D),
// so that the instantiations build in parallel; each object defines its
// specialisations.  DT is (int)Dt.
template <int DT, int D> int launch_dense_fwd_ed(const DenseArgs& a, void* stream);
template <int DT, int D> int launch_dense_dkdv_ed(const DenseArgs& a, void* stream);
template <int DT, int D> int launch_dense_dq_ed(const DenseArgs& a, void* stream);
#define ETS_DECLARE_ED(DT, D)                                                 \
  template <> int launch_dense_fwd_ed<DT, D>(const DenseArgs& a, void* stream);  \
  template <> int launch_dense_dkdv_ed<DT, D>(const DenseArgs& a, void* stream); \
  template <> int launch_dense_dq_ed<DT, D>(const DenseArgs& a, void* stream);
ETS_DECLARE_ED(1, 64)
ETS_DECLARE_ED(1, 128)
ETS_DECLARE_ED(2, 64)
ETS_DECLARE_ED(2, 128)
#undef ETS_DECLARE_ED
// phases: bit 0 = D prepass, bit 1 = dK/dV, bit 2 = dQ
int launch_dense_bwd(const DenseArgs& a, Dt dt, void* stream, int phases);
int launch_dense_fwd_f32(const DenseArgs& a, void* stream);
int launch_dense_bwd_f32(const DenseArgs& a, void* stream, int phases);
int launch_sparse_fwd(const SparseArgs& a, Dt dt, void* stream);
int launch_sparse_bwd(const SparseArgs& a, Dt dt, void* stream);
int launch_dropout_mask(const DropArgs& d, int B, int H, int nq, int nk, uint8_t* xi, void* stream);
int launch_mfma_probe(int waves_per_simd, int iters, float* sink, int sink_len, long long* mfmas, void* stream);
int launch_issue_probe(int waves_per_simd, int valu_per_mfma, int trans, int iters, float* sink, int sink_len,
                       long long* mfmas, void* stream);
int launch_atomic_probe(float* table, int rows, const int32_t* idx, int n_idx, int blocks, int groups_per_wave,
                        long long* adds, void* stream);
int launch_lds_probe(int waves, int iters, uint32_t* sink, int sink_len, long long* bytes, void* stream);

// Debug checks (debug.hip).  Each returns 0 or a hipError_t value and sets
// *bad (host) when the check fails; each synchronises the stream.
struct DebugBuf {
  const void* ptr;
  long long count;  // elements
  int kind;         // 0 fp32, 1 fp16, 2 bf16, 3 fp32 with -inf allowed
};
int debug_check_lengths(const int32_t* lengths, int B, int n, void* stream, int* bad);
int debug_check_topk(const int32_t* idx, const int32_t* length, int Tq, int topk, int Tkv, void* stream, int* bad);
int debug_scan_nonfinite(const DebugBuf* bufs, int nbufs, void* stream, int* bad);

// Shapes the MFMA kernels are built for.
bool dense_mfma_supported(int d, int dv);
bool sparse_supported(int H, int dqk, int dv);

}  // namespace ets
