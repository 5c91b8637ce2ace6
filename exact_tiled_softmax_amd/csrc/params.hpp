// Launch parameters shared by the C-ABI layer (abi.cpp) and the HIP kernels.
// Internal to the library: nothing here is part of the public ABI.
#pragma once
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
};

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
// phases: bit 0 = D prepass, bit 1 = dK/dV, bit 2 = dQ
int launch_dense_bwd(const DenseArgs& a, Dt dt, void* stream, int phases);
int launch_dense_fwd_f32(const DenseArgs& a, void* stream);
int launch_dense_bwd_f32(const DenseArgs& a, void* stream, int phases);
int launch_sparse_fwd(const SparseArgs& a, Dt dt, void* stream);
int launch_sparse_bwd(const SparseArgs& a, Dt dt, void* stream);
int launch_dropout_mask(const DropArgs& d, int B, int H, int nq, int nk, uint8_t* xi, void* stream);
int launch_mfma_probe(int waves_per_simd, int iters, float* sink, int sink_len, long long* mfmas, void* stream);

// Shapes the MFMA kernels are built for.
bool dense_mfma_supported(int d, int dv);
bool sparse_supported(int H, int dqk, int dv);

}  // namespace ets
