// C-ABI entry points of libattn.so: host-side validation and dispatch.
// Every check happens before any launch; on failure nothing is launched and
// no output is written.  The declarations and their contracts are in
// include/attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/attn.h"
#include "params.hpp"

using namespace ets;

namespace {

constexpr int kMaxF32Width = 128;
// Index arithmetic limits of the kernels: 32-bit buffer-resource extents per
// (batch, head) tensor, 32-bit offsets into the backward workspace, and the
// 65535 (batch, head) lanes of the fp32 path's second grid dimension.
constexpr long long kMaxHeadBytes = (1LL << 32) - 1;
constexpr long long kMaxRows = (1LL << 28) - 64;
constexpr long long kMaxF32Lanes = 65535;

// Debug checks for this call: the environment variable ATTN_DEBUG holds a
// nonzero integer.
bool debug_enabled() {
  const char* v = std::getenv("ATTN_DEBUG");
  return v && std::strtol(v, nullptr, 10) != 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool bad_dims(std::initializer_list<long long> v) {
  for (long long x : v)
    if (x < 1 || x > (1LL << 30)) return true;
  return false;
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Shared validation of the dense forward/backward arguments.
attn_status check_dense(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                        const attn_mask_t* mask, float scale, int block_b,
                        const attn_dropout_t* drop) {
  if (dt != ATTN_F32 && dt != ATTN_F16 && dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (bad_dims({B, H, H_kv, n_q, n_k, d, dv})) return ATTN_ERR_INVALID_ARG;
  if (H % H_kv != 0) return ATTN_ERR_INVALID_ARG;
  if ((long long)B * H * n_q > (1LL << 31) - 1 || (long long)B * H_kv * n_k > (1LL << 31) - 1)
    return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
  if (block_b < 0) return ATTN_ERR_INVALID_ARG;
  if (mask) {
    if (mask->causal && n_q != n_k) return ATTN_ERR_INVALID_ARG;
    if (mask->window < 0) return ATTN_ERR_INVALID_ARG;
    if (mask->block_mask && (mask->block_q < 1 || mask->block_k < 1)) return ATTN_ERR_INVALID_ARG;
    if (mask->lengths && n_q != n_k) return ATTN_ERR_INVALID_ARG;
    if ((mask->lengths && !aligned(mask->lengths, 4)) || (mask->starts && !aligned(mask->starts, 4)))
      return ATTN_ERR_INVALID_ARG;
  }
  if (drop) {
    if (!std::isfinite(drop->rate) || drop->rate < 0.f || drop->rate >= 1.f) return ATTN_ERR_INVALID_ARG;
  }
  if (dt == ATTN_F32) {
    if (d > kMaxF32Width || dv > kMaxF32Width) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * H > kMaxF32Lanes) return ATTN_ERR_UNSUPPORTED;
  } else {
    if (!dense_mfma_supported(d, dv)) return ATTN_ERR_UNSUPPORTED;
    if (block_b != 0 && block_b != 64) return ATTN_ERR_UNSUPPORTED;
  }
  const long long esz = dt == ATTN_F32 ? 4 : 2;
  if ((long long)n_q * d * esz > kMaxHeadBytes || (long long)n_k * d * esz > kMaxHeadBytes ||
      (long long)n_q * dv * esz > kMaxHeadBytes || (long long)n_k * dv * esz > kMaxHeadBytes)
    return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * H * n_q > kMaxRows || (long long)B * H_kv * n_k > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

void fill_dense(DenseArgs& a, attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                const attn_mask_t* mask, float scale, int block_b, const attn_dropout_t* drop) {
  std::memset(&a, 0, sizeof(a));
  a.B = B; a.H = H; a.Hkv = H_kv; a.nq = n_q; a.nk = n_k; a.d = d; a.dv = dv;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.block_b = (dt == ATTN_F32) ? (block_b > 0 ? block_b : 64) : 64;
  if (mask) {
    a.mask.causal = mask->causal != 0;
    a.mask.window = mask->window;
    a.mask.block_mask = mask->block_mask;
    a.mask.bq = mask->block_mask ? mask->block_q : 1;
    a.mask.bk = mask->block_mask ? mask->block_k : 1;
    a.mask.nbk = mask->block_mask ? (n_k + mask->block_k - 1) / mask->block_k : 0;
    a.mask.dense_mask = mask->dense_mask;
    a.mask.dm_stride = n_k;
    a.mask.lengths = mask->lengths;
    a.mask.starts = mask->starts;
  }
  if (drop && drop->rate > 0.f) {
    const double r = (double)drop->rate;
    a.drop.enabled = 1;
    a.drop.threshold = (uint32_t)std::floor(r * 65536.0);
    a.drop.seed_lo = (uint32_t)(drop->seed & 0xffffffffu);
    a.drop.seed_hi = (uint32_t)(drop->seed >> 32);
    a.drop.inv_keep = (float)(1.0 / (1.0 - r));
  }
}

// Debug scan kind of a tensor of dtype dt (see DebugBuf)
int kind_of(attn_dtype dt) { return dt == ATTN_F32 ? 0 : (dt == ATTN_F16 ? 1 : 2); }

// Debug checks: lengths within [0, n] before a dense launch; non-finite
// outputs after one.
attn_status debug_check_mask(const attn_mask_t* mask, int B, int n, void* stream) {
  if (!mask || !mask->lengths) return ATTN_OK;
  int bad = 0;
  if (debug_check_lengths(mask->lengths, B, n, stream, &bad) != 0) return ATTN_ERR_HIP;
  return bad ? ATTN_ERR_INVALID_ARG : ATTN_OK;
}

attn_status debug_scan(const DebugBuf* bufs, int n, void* stream) {
  int bad = 0;
  if (debug_scan_nonfinite(bufs, n, stream, &bad) != 0) return ATTN_ERR_HIP;
  return bad ? ATTN_ERR_NONFINITE : ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch failed";
    case ATTN_ERR_NONFINITE: return "non-finite value in an output (debug check)";
  }
  return "unknown status";
}

attn_status attn_fwd(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                     const void* Q, const void* K, const void* V, const attn_mask_t* mask,
                     float scale, int block_b, const attn_dropout_t* dropout, void* Y, float* LSE,
                     void* stream) {
  attn_status st = check_dense(dt, B, H, H_kv, n_q, n_k, d, dv, mask, scale, block_b, dropout);
  if (st != ATTN_OK) return st;
  if (!Q || !K || !V || !Y || !LSE) return ATTN_ERR_INVALID_ARG;
  const size_t al = dt == ATTN_F32 ? 4 : 16;
  if (!aligned(Q, al) || !aligned(K, al) || !aligned(V, al) || !aligned(Y, al) || !aligned(LSE, 4))
    return ATTN_ERR_INVALID_ARG;
  const bool dbg = debug_enabled();
  if (dbg) {
    const attn_status cs = debug_check_mask(mask, B, n_q, stream);
    if (cs != ATTN_OK) return cs;
  }
  DenseArgs a;
  fill_dense(a, dt, B, H, H_kv, n_q, n_k, d, dv, mask, scale, block_b, dropout);
  a.Q = Q; a.K = K; a.V = V; a.out_Y = Y; a.LSE = LSE;
  const int rc = dt == ATTN_F32 ? launch_dense_fwd_f32(a, stream)
                                : launch_dense_fwd(a, dt == ATTN_BF16 ? Dt::BF16 : Dt::F16, stream);
  if (rc != 0) return ATTN_ERR_HIP;
  if (dbg) {
    const long long rows = (long long)B * H * n_q;
    const DebugBuf bufs[2] = {{Y, rows * dv, kind_of(dt)}, {LSE, rows, 3}};
    return debug_scan(bufs, 2, stream);
  }
  return ATTN_OK;
}

size_t attn_bwd_workspace_size(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d,
                               int dv) {
  (void)dt; (void)H_kv; (void)n_k; (void)d; (void)dv;
  if (bad_dims({B, H, n_q})) return 0;
  // D_i and LSE_i log2(e), each with 64 padding rows
  return 2 * round_up(((size_t)B * H * n_q + 64) * sizeof(float));
}

// Stored-gamma form (see DenseArgs::Gam): bf16/fp16 MFMA shapes with dropout
// whose mask is causal and / or a window only, with each (batch, head)'s
// blocks addressable by 32-bit offsets.  (Measured on MI355X: with dropout the
// recomputing dQ kernel also replays the Philox draws and the stored form
// wins; without dropout the extra HBM traffic of writing and reading gamma
// costs more than the recomputation it saves.)  Returns the blocks per
// (batch, head), 0 if not eligible.
static long long gam_eligible(attn_dtype dt, int n_q, int n_k, int d, int dv, const attn_mask_t* mask,
                              const attn_dropout_t* drop, int* stride) {
  if (dt == ATTN_F32 || !dense_mfma_supported(d, dv)) return 0;
  if (!drop || !(drop->rate > 0.f)) return 0;
  MaskArgs m;
  std::memset(&m, 0, sizeof(m));
  if (mask) {
    if (mask->block_mask || mask->dense_mask || mask->lengths || mask->starts) return 0;
    m.causal = mask->causal != 0;
    m.window = mask->window;
  }
  const long long per = gam_blocks_per_bh(m, n_q, n_k, *stride);
  if (per <= 0 || per * kGamBlockBytes >= (1ll << 31)) return 0;
  return per;
}

size_t attn_bwd_workspace_size_fast(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                                    const attn_mask_t* mask, const attn_dropout_t* dropout) {
  const size_t base = attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv);
  if (base == 0 || bad_dims({H_kv, n_k, d, dv})) return base;
  int stride = 0;
  const long long per = gam_eligible(dt, n_q, n_k, d, dv, mask, dropout, &stride);
  if (per == 0) return base;
  return round_up(base) + (size_t)B * H * (size_t)per * kGamBlockBytes;
}

static attn_status bwd_common(int phases, attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d,
                              int dv, const void* Q, const void* K, const void* V, const void* Y,
                              const float* LSE, const void* G, const attn_mask_t* mask, float scale,
                              int block_b, const attn_dropout_t* dropout, void* dQ, void* dK, void* dV,
                              void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_dense(dt, B, H, H_kv, n_q, n_k, d, dv, mask, scale, block_b, dropout);
  if (st != ATTN_OK) return st;
  if (phases < 1 || phases > 7) return ATTN_ERR_INVALID_ARG;
  const size_t al = dt == ATTN_F32 ? 4 : 16;
  // pointers each phase reads or writes
  const bool p0 = phases & 1, p1 = phases & 2, p2 = phases & 4;
  if ((p0 && (!Y || !G)) || ((p1 || p2) && (!Q || !K || !V || !LSE || !G)) || (p1 && (!dK || !dV)) ||
      (p2 && !dQ))
    return ATTN_ERR_INVALID_ARG;
  for (const void* p : {Q, K, V, Y, G, (const void*)dQ, (const void*)dK, (const void*)dV})
    if (p && !aligned(p, al)) return ATTN_ERR_INVALID_ARG;
  if (LSE && !aligned(LSE, 4)) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;
  const bool dbg = debug_enabled();
  if (dbg) {
    const attn_status cs = debug_check_mask(mask, B, n_q, stream);
    if (cs != ATTN_OK) return cs;
  }
  DenseArgs a;
  fill_dense(a, dt, B, H, H_kv, n_q, n_k, d, dv, mask, scale, block_b, dropout);
  a.Q = Q; a.K = K; a.V = V; a.Y = Y; a.LSE = (float*)LSE; a.G = G;
  a.dQ = dQ; a.dK = dK; a.dV = dV; a.Dws = (float*)workspace;
  a.Lws = (float*)((char*)workspace + round_up(((size_t)B * H * n_q + 64) * sizeof(float)));
  // the stored-gamma form when the workspace holds its blocks
  if (workspace_bytes >= attn_bwd_workspace_size_fast(dt, B, H, H_kv, n_q, n_k, d, dv, mask, dropout) &&
      gam_eligible(dt, n_q, n_k, d, dv, mask, dropout, &a.gam_stride) > 0) {
    a.gam_per_bh = gam_eligible(dt, n_q, n_k, d, dv, mask, dropout, &a.gam_stride);
    a.Gam = (char*)workspace + round_up(need);
  }
  const int rc = dt == ATTN_F32 ? launch_dense_bwd_f32(a, stream, phases)
                                : launch_dense_bwd(a, dt == ATTN_BF16 ? Dt::BF16 : Dt::F16, stream, phases);
  if (rc != 0) return ATTN_ERR_HIP;
  if (dbg && (phases & 6)) {
    const int k = kind_of(dt);
    const DebugBuf bufs[3] = {{(phases & 4) ? dQ : nullptr, (long long)B * H * n_q * d, k},
                              {(phases & 2) ? dK : nullptr, (long long)B * H_kv * n_k * d, k},
                              {(phases & 2) ? dV : nullptr, (long long)B * H_kv * n_k * dv, k}};
    return debug_scan(bufs, 3, stream);
  }
  return ATTN_OK;
}

attn_status attn_bwd(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                     const void* Q, const void* K, const void* V, const void* Y, const float* LSE,
                     const void* G, const attn_mask_t* mask, float scale, int block_b,
                     const attn_dropout_t* dropout, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(7, dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, Y, LSE, G, mask, scale, block_b, dropout,
                    dQ, dK, dV, workspace, workspace_bytes, stream);
}

// Fixed device scratch of attn_bwd_noalloc: the backward workspace (D_i and
// the base-2 LSE of every query row) for callers that cannot allocate.  Each
// GPU holds its own copy until the process ends.  Host code never passes this
// name to a kernel or a copy: it uses the address hipGetSymbolAddress returns
// for the current device (noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
static attn_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[256] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return ATTN_OK;
}

attn_status attn_bwd_noalloc(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                             const void* Q, const void* K, const void* V, const void* Y, const float* LSE,
                             const void* G, const attn_mask_t* mask, float scale, int block_b,
                             const attn_dropout_t* dropout, void* dQ, void* dK, void* dV, void* stream) {
  // the argument checks first, so that a bad call touches no device state
  attn_status st = check_dense(dt, B, H, H_kv, n_q, n_k, d, dv, mask, scale, block_b, dropout);
  if (st != ATTN_OK) return st;
  if (attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv) > kNoAllocScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != ATTN_OK) return st;
  // exactly the minimal workspace: the recomputing form, whatever the mask
  return bwd_common(7, dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, Y, LSE, G, mask, scale, block_b, dropout, dQ, dK,
                    dV, ws, attn_bwd_workspace_size(dt, B, H, H_kv, n_q, n_k, d, dv), stream);
}

attn_status attn_bwd_phase(int phases, attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d,
                           int dv, const void* Q, const void* K, const void* V, const void* Y,
                           const float* LSE, const void* G, const attn_mask_t* mask, float scale,
                           int block_b, const attn_dropout_t* dropout, void* dQ, void* dK, void* dV,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(phases, dt, B, H, H_kv, n_q, n_k, d, dv, Q, K, V, Y, LSE, G, mask, scale, block_b,
                    dropout, dQ, dK, dV, workspace, workspace_bytes, stream);
}

static attn_status debug_topk(const int32_t* idx, const int32_t* length, int Tq, int topk, int Tkv, void* stream) {
  int bad = 0;
  if (debug_check_topk(idx, length, Tq, topk, Tkv, stream, &bad) != 0) return ATTN_ERR_HIP;
  return bad ? ATTN_ERR_INVALID_ARG : ATTN_OK;
}

static attn_status check_sparse(attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v, int topk,
                                float scale) {
  if (dt != ATTN_F16 && dt != ATTN_BF16) return dt == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID_ARG;
  if (bad_dims({Tq, H, Tkv, d_qk, d_v, topk})) return ATTN_ERR_INVALID_ARG;
  if (d_v > d_qk) return ATTN_ERR_INVALID_ARG;
  if ((long long)Tq * topk > (1LL << 31) - 1 || (long long)Tq * H > (1LL << 31) - 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
  if (!sparse_supported(H, d_qk, d_v)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

static void fill_sparse(SparseArgs& a, int Tq, int H, int Tkv, int d_qk, int d_v, int topk, float scale) {
  std::memset(&a, 0, sizeof(a));
  a.Tq = Tq; a.H = H; a.Tkv = Tkv; a.dqk = d_qk; a.dv = d_v; a.topk = topk;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
}

attn_status attn_sparse_fwd_lse(attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v,
                                int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale, void* O,
                                float* LSE, void* stream) {
  if (kind != ATTN_LSE_TOTAL && kind != ATTN_LSE_KV) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_sparse(dt, Tq, H, Tkv, d_qk, d_v, topk, scale);
  if (st != ATTN_OK) return st;
  if (!Q || !KV || !topk_idx || !O || !LSE) return ATTN_ERR_INVALID_ARG;
  for (const void* p : {Q, KV, (const void*)O})
    if (!aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(topk_idx, 4) || !aligned(LSE, 4) || (topk_length && !aligned(topk_length, 4)) ||
      (attn_sink && !aligned(attn_sink, 4)))
    return ATTN_ERR_INVALID_ARG;
  SparseArgs a;
  fill_sparse(a, Tq, H, Tkv, d_qk, d_v, topk, scale);
  a.Q = Q; a.KV = KV; a.idx = topk_idx; a.length = topk_length; a.sink = attn_sink;
  a.O = O; a.LSE = LSE;
  a.lse_kv = kind == ATTN_LSE_KV;
  const bool dbg = debug_enabled();
  if (dbg) {
    const attn_status cs = debug_topk(topk_idx, topk_length, Tq, topk, Tkv, stream);
    if (cs != ATTN_OK) return cs;
  }
  const int rc = launch_sparse_fwd(a, dt == ATTN_BF16 ? Dt::BF16 : Dt::F16, stream);
  if (rc != 0) return ATTN_ERR_HIP;
  if (dbg) {
    const DebugBuf bufs[2] = {{O, (long long)Tq * H * d_v, kind_of(dt)}, {LSE, (long long)Tq * H, 3}};
    return debug_scan(bufs, 2, stream);
  }
  return ATTN_OK;
}

attn_status attn_sparse_fwd(attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v, int topk,
                            const void* Q, const void* KV, const int32_t* topk_idx,
                            const int32_t* topk_length, const float* attn_sink, float scale,
                            void* O, float* LSE, void* stream) {
  return attn_sparse_fwd_lse(ATTN_LSE_TOTAL, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length,
                             attn_sink, scale, O, LSE, stream);
}

size_t attn_sparse_bwd_workspace_size(int Tq, int H, int Tkv, int d_qk, int d_v, int topk) {
  (void)d_v; (void)topk;
  if (bad_dims({Tq, H, Tkv, d_qk})) return 0;
  return 2 * round_up((size_t)Tq * H * sizeof(float)) + round_up((size_t)Tkv * d_qk * sizeof(float));
}

size_t attn_sparse_bwd_det_workspace_size(int Tq, int H, int Tkv, int d_qk, int d_v, int topk) {
  (void)d_v; (void)topk;
  if (bad_dims({Tq, H, Tkv, d_qk})) return 0;
  return 2 * round_up((size_t)Tq * H * sizeof(float)) + round_up((size_t)Tkv * d_qk * sizeof(int64_t));
}

static attn_status sparse_bwd_common(int det, attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk,
                                     int d_v, int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale,
                                const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                                float* dSink, void* workspace, size_t workspace_bytes, void* stream) {
  if (kind != ATTN_LSE_TOTAL && kind != ATTN_LSE_KV) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_sparse(dt, Tq, H, Tkv, d_qk, d_v, topk, scale);
  if (st != ATTN_OK) return st;
  if (!Q || !KV || !topk_idx || !O || !LSE || !dO || !dQ || !dKV) return ATTN_ERR_INVALID_ARG;
  if (attn_sink && !dSink) return ATTN_ERR_INVALID_ARG;
  for (const void* p : {Q, KV, O, dO, (const void*)dQ, (const void*)dKV})
    if (!aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(topk_idx, 4) || !aligned(LSE, 4) || (topk_length && !aligned(topk_length, 4)) ||
      (attn_sink && !aligned(attn_sink, 4)) || (dSink && !aligned(dSink, 4)))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = det ? attn_sparse_bwd_det_workspace_size(Tq, H, Tkv, d_qk, d_v, topk)
                          : attn_sparse_bwd_workspace_size(Tq, H, Tkv, d_qk, d_v, topk);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return ATTN_ERR_WORKSPACE;
  SparseArgs a;
  fill_sparse(a, Tq, H, Tkv, d_qk, d_v, topk, scale);
  a.Q = Q; a.KV = KV; a.idx = topk_idx; a.length = topk_length; a.sink = attn_sink;
  a.O = (void*)O; a.LSE = (float*)LSE; a.dO = dO; a.dQ = dQ; a.dKV = dKV; a.dSink = dSink;
  a.lse_kv = kind == ATTN_LSE_KV;
  a.det = det;
  a.Dws = (float*)workspace;
  a.dsink_part = (float*)((char*)workspace + round_up((size_t)Tq * H * sizeof(float)));
  a.dKVws = (float*)((char*)workspace + 2 * round_up((size_t)Tq * H * sizeof(float)));
  const bool dbg = debug_enabled();
  if (dbg) {
    const attn_status cs = debug_topk(topk_idx, topk_length, Tq, topk, Tkv, stream);
    if (cs != ATTN_OK) return cs;
  }
  const int rc = launch_sparse_bwd(a, dt == ATTN_BF16 ? Dt::BF16 : Dt::F16, stream);
  if (rc != 0) return ATTN_ERR_HIP;
  if (dbg) {
    const DebugBuf bufs[3] = {{dQ, (long long)Tq * H * d_qk, kind_of(dt)}, {dKV, (long long)Tkv * d_qk, kind_of(dt)},
                              {dSink, dSink ? H : 0, 0}};
    return debug_scan(bufs, 3, stream);
  }
  return ATTN_OK;
}

attn_status attn_sparse_bwd_lse(attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v,
                                int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale,
                                const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                                float* dSink, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_bwd_common(0, kind, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                           O, LSE, dO, dQ, dKV, dSink, workspace, workspace_bytes, stream);
}

attn_status attn_sparse_bwd_det(attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v,
                                int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale,
                                const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                                float* dSink, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_bwd_common(1, kind, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length, attn_sink, scale,
                           O, LSE, dO, dQ, dKV, dSink, workspace, workspace_bytes, stream);
}

attn_status attn_sparse_bwd(attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v, int topk,
                            const void* Q, const void* KV, const int32_t* topk_idx,
                            const int32_t* topk_length, const float* attn_sink, float scale,
                            const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                            float* dSink, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_sparse_bwd_lse(ATTN_LSE_TOTAL, dt, Tq, H, Tkv, d_qk, d_v, topk, Q, KV, topk_idx, topk_length,
                             attn_sink, scale, O, LSE, dO, dQ, dKV, dSink, workspace, workspace_bytes, stream);
}

attn_status attn_dropout_mask(float rate, uint64_t seed, int B, int H, int n_q, int n_k,
                              uint8_t* xi, void* stream) {
  if (bad_dims({B, H, n_q, n_k}) || !xi) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(rate) || rate < 0.f || rate >= 1.f) return ATTN_ERR_INVALID_ARG;
  if ((long long)B * H * n_q * (long long)n_k > (1LL << 40)) return ATTN_ERR_INVALID_ARG;
  attn_dropout_t d{rate, seed};
  DenseArgs a;
  fill_dense(a, ATTN_F32, B, H, H, n_q, n_k, 1, 1, nullptr, 1.f, 0, &d);
  const int rc = launch_dropout_mask(a.drop, B, H, n_q, n_k, xi, stream);
  return rc == 0 ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_mfma_probe(int waves_per_simd, int iters, float* sink, int sink_len, long long* mfmas,
                            void* stream) {
  if ((waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 || !sink || !mfmas || sink_len < 1)
    return ATTN_ERR_INVALID_ARG;
  const int rc = launch_mfma_probe(waves_per_simd, iters, sink, sink_len, mfmas, stream);
  if (rc == -1) return ATTN_ERR_INVALID_ARG;  // sink shorter than the CU count
  return rc == 0 ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_issue_probe(int waves_per_simd, int valu_per_mfma, int trans, int iters, float* sink, int sink_len,
                             long long* mfmas, void* stream) {
  if ((waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 || !sink || !mfmas || sink_len < 1)
    return ATTN_ERR_INVALID_ARG;
  if (trans != 0 && trans != 1) return ATTN_ERR_INVALID_ARG;
  if (valu_per_mfma != 0 && valu_per_mfma != 2 && valu_per_mfma != 4 && valu_per_mfma != 6 && valu_per_mfma != 8 &&
      valu_per_mfma != 12)
    return ATTN_ERR_INVALID_ARG;
  const int rc = launch_issue_probe(waves_per_simd, valu_per_mfma, trans, iters, sink, sink_len, mfmas, stream);
  if (rc == -1) return ATTN_ERR_INVALID_ARG;  // sink shorter than the CU count
  return rc == 0 ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_atomic_probe(float* table, int rows, const int32_t* idx, int n_idx, int blocks, int groups_per_wave,
                              long long* adds, void* stream) {
  if (!table || !idx || !adds || rows < 1 || n_idx < 1 || blocks < 1 || groups_per_wave < 1)
    return ATTN_ERR_INVALID_ARG;
  if ((long long)rows * 576 > (1LL << 40) || blocks > (1 << 24)) return ATTN_ERR_INVALID_ARG;
  const int rc = launch_atomic_probe(table, rows, idx, n_idx, blocks, groups_per_wave, adds, stream);
  return rc == 0 ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_lds_probe(int waves_per_cu, int iters, uint32_t* sink, int sink_len, long long* bytes, void* stream) {
  if ((waves_per_cu != 4 && waves_per_cu != 8 && waves_per_cu != 16) || iters < 1 || !sink || !bytes || sink_len < 1)
    return ATTN_ERR_INVALID_ARG;
  const int rc = launch_lds_probe(waves_per_cu, iters, sink, sink_len, bytes, stream);
  if (rc == -1) return ATTN_ERR_INVALID_ARG;  // sink shorter than the CU count
  return rc == 0 ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
