// Device helpers for the gfx950 (CDNA4) attention kernels: element types and
// MFMA wrappers, the swizzled LDS tile format, cross-half lane exchange,
// Philox4x32-10 and the allowed-set tests.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <tuple>
#include <type_traits>
#include <utility>
#include <mutex>

#include "params.hpp"

namespace ets {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define ETS_LDS __attribute__((address_space(3)))

// Launch with the status of this launch only (hipGetLastError would also
// report errors left behind by unrelated earlier runtime calls).
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> vals(args...);
  void* ptrs[sizeof...(P)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = (void*)&v), ...);
  }, vals);
  return hipLaunchKernel((const void*)kernel, grid, block, ptrs, lds, st);
}

// Workgroups of `kernel` that the device keeps resident at once (compute
// units x workgroups per unit), cached per (kernel, device).  Persistent
// kernels launch at most this many workgroups.
inline hipError_t resident_slots_fn(const void* fn, int block_threads, int* slots) {
  struct Entry {
    const void* fn;
    int dev, slots;
  };
  static std::mutex mu;
  static Entry cache[256];
  static int n = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; ++i)
      if (cache[i].fn == fn && cache[i].dev == dev) {
        *slots = cache[i].slots;
        return hipSuccess;
      }
  }
  int per_cu = 0, cus = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block_threads, 0);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *slots = per_cu > 0 && cus > 0 ? per_cu * cus : 1;
  std::lock_guard<std::mutex> lock(mu);
  if (n < 256) cache[n++] = Entry{fn, dev, *slots};
  return hipSuccess;
}
template <class... P>
inline hipError_t resident_slots(void (*kernel)(P...), int block_threads, int* slots) {
  return resident_slots_fn((const void*)kernel, block_threads, slots);
}

#define ETS_TRY(expr)                      \
  do {                                     \
    const hipError_t ets_e_ = (expr);      \
    if (ets_e_ != hipSuccess) return (int)ets_e_; \
  } while (0)

// ------------------------------------------------------------ element types
// Storage is 16-bit in memory; MFMA operands are 8 elements (16 bytes) per lane.

struct BF16 {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // two floats -> packed pair, round to nearest even
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
};

struct F16 {
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    f16x2 r = __builtin_convertvector(v, f16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

template <class E>
__device__ __forceinline__ typename E::vec8 as_vec8(u32x4 u) {
  return __builtin_bit_cast(typename E::vec8, u);
}

// ------------------------------------------------------------ LDS tile format
// A tile is row-major with a fixed byte stride per row; its 16-byte chunks are
// XOR-swizzled by a function of the row within groups of MASK+1 chunks.  The
// swizzle depends on the row width (CDNA4's LDS serves 256 bytes per clock
// from 64 banks): it makes both access patterns of the kernels conflict-free
// or nearly so (measured on MI355X):
//   * 16-byte reads of one chunk column by 16 consecutive rows (MFMA operand
//     rows), and
//   * transpose reads, where 16 lanes read 4 consecutive rows (starting at a
//     multiple of 4) x 32 contiguous bytes.
// Every swizzle below depends on the row modulo 16 only.
template <int ROWB> struct Swizzle;
template <> struct Swizzle<256> {  // 128 16-bit columns
  static constexpr int MASK = 15;
  static constexpr __host__ __device__ int f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};
template <> struct Swizzle<128> {  // 64 16-bit columns: two rows share a bank line
  static constexpr int MASK = 7;
  static constexpr __host__ __device__ int f(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
};
template <> struct Swizzle<1152> {  // 576 16-bit columns: alternate rows start half a bank line apart
  static constexpr int MASK = 7;
  static constexpr __host__ __device__ int f(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
};

template <int ROWB>
constexpr __host__ __device__ int phys_chunk(int row, int chunk) {
  constexpr int M = Swizzle<ROWB>::MASK;
  return (chunk & ~M) | ((chunk & M) ^ Swizzle<ROWB>::f(row));
}

// byte offset of element (row, col) of a 16-bit tile with ROWB bytes per row
template <int ROWB>
__device__ __forceinline__ int toff(int row, int col) {
  return row * ROWB + (phys_chunk<ROWB>(row, col >> 3) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ u32x4 lds_b128(const char ETS_LDS* base, int off) {
  return *(const u32x4 ETS_LDS*)(base + off);
}

__device__ __forceinline__ void lds_st128(char ETS_LDS* base, int off, u32x4 v) {
  *(u32x4 ETS_LDS*)(base + off) = v;
}

// Transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// supplies the address of 4 consecutive elements (row r0 + i/4, cols
// c0 + 4*(i%4) .. +3); it receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ s16x4 lds_tr4(const char ETS_LDS* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 ETS_LDS*)(base + off));
}

// An MFMA operand holding 8 elements of one column (the "m" or "n" index
// col0 + lane%32 for 32x32 shapes) along 8 rows: the lane's k-slots 0..3 are
// rows r0 .. r0+3 and slots 4..7 are rows r1 .. r1+3.
template <int ROWB>
__device__ __forceinline__ u32x4 lds_tr8(const char ETS_LDS* base, int r0, int r1, int col0, int lane) {
  const int i = lane & 15;
  const int col = col0 + 4 * (i & 3);
  s16x4 a = lds_tr4(base, toff<ROWB>(r0 + (i >> 2), col));
  s16x4 b = lds_tr4(base, toff<ROWB>(r1 + (i >> 2), col));
  s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(u32x4, v);
}

// Buffer resource for the raw buffer instructions: `bytes` bytes from `base`
// (reads past them return zero).  Dword 3 selects 32-bit data format, as the
// raw (untyped) loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Copy 16 bytes per lane from global memory straight into LDS: lane l writes
// at ldsdst + 16 l.  The MUBUF form (buffer_load_dwordx4 ... lds) is used
// rather than global_load_lds: with a FLAT-encoded copy in flight the compiler
// makes every later LDS read wait for all outstanding LDS traffic
// (lgkmcnt(0)), while with the buffer form it keeps exact counts.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, void ETS_LDS* ldsdst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ldsdst, 16, byte_off, 0, 0, 0);
}

// Direct global -> LDS copy of a tile of ROWS rows x W 16-bit elements into
// the swizzled tile format.  Each of the NWAVES waves issues
// ROWS*W/8/64/NWAVES instructions; lane l of instruction k fills chunk
// position 64k + l, so it fetches the logical chunk that the swizzle maps
// there.  Rows past last_row are read from last_row instead (finite data; the
// caller masks them), so no access leaves the tensor.  Completion is awaited
// with a vmcnt wait before the barrier that publishes the tile.  The per-lane
// parts of the offsets are computed once; an issue costs three VALU
// operations per instruction (row clamp and byte offset), plus one XOR where
// the swizzle of the instruction's rows differs from that of the first
// instruction's by the same XOR in every lane of every wave (checked at
// compile time): then one register per lane holds the column offsets instead
// of one per instruction.
template <int ROWS, int W, int NWAVES>
struct TileCopy {
  static constexpr int CPR = W / 8;  // 16-byte chunks per row
  static constexpr int INSTS = ROWS * CPR / 64;
  static_assert(INSTS % NWAVES == 0 && 64 % CPR == 0, "tile does not split evenly over the waves");
  static constexpr int PER_WAVE = INSTS / NWAVES;
  static constexpr int RPI = 64 / CPR;  // rows per instruction
  static constexpr int row_of(int wave, int lane) { return wave * PER_WAVE * RPI + lane / CPR; }
  static constexpr int xor_of(int u) { return Swizzle<2 * W>::f(u * RPI) ^ Swizzle<2 * W>::f(0); }
  static constexpr bool xor_uniform() {
    for (int w = 0; w < NWAVES; ++w)
      for (int l = 0; l < 64; ++l)
        for (int u = 0; u < PER_WAVE; ++u) {
          const int r = row_of(w, l);
          if ((Swizzle<2 * W>::f(r + u * RPI) ^ Swizzle<2 * W>::f(r)) != xor_of(u)) return false;
        }
    return true;
  }
  static constexpr bool XOR = xor_uniform();
  static constexpr int NCOL = XOR ? 1 : PER_WAVE;
  int row;                // tile row of this lane in the wave's first instruction
  int col[NCOL];          // byte offset, within its row, of the chunk this lane fetches
  int inst0;              // first instruction index of the wave (uniform)
  __device__ __forceinline__ TileCopy(int wave, int lane) {
    inst0 = wave * PER_WAVE;
    row = row_of(wave, lane);
#pragma unroll
    for (int u = 0; u < NCOL; ++u) col[u] = phys_chunk<2 * W>(row + u * RPI, lane % CPR) * 16;  // involution
  }
  __device__ __forceinline__ int col_of(int u) const {
    if constexpr (XOR) return col[0] ^ (xor_of(u) * 16);
    else return col[u];
  }
  // instruction u (0 .. PER_WAVE-1) of the wave's share; rs covers the tensor
  // whose row 0 is at offset 0
  __device__ __forceinline__ void issue_one(char ETS_LDS* dst, __amdgpu_buffer_rsrc_t rs, int row0, int last_row,
                                            int u) const {
    const unsigned off = (unsigned)min(row0 + row + u * RPI, last_row) * (unsigned)(2 * W) + (unsigned)col_of(u);
    copy16_to_lds(rs, off, (void ETS_LDS*)(dst + (inst0 + u) * 1024));
  }
  __device__ __forceinline__ void issue(char ETS_LDS* dst, __amdgpu_buffer_rsrc_t rs, int row0, int last_row) const {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) issue_one(dst, rs, row0, last_row, u);
  }
};

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (the loads of later tiles stay in flight).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Per-lane byte offsets of the MFMA operand reads.  toff() mixes lane terms
// and loop indices through the swizzle XOR; these split it into a few
// per-lane bases (computed once with toff itself) plus terms that are
// compile-time constants once the loops are unrolled, so every read is
// base + immediate offset.  The split is exact because the swizzles depend on
// the row modulo 16 and the base rows R passed in are multiples of 16, and
// because each XOR group of MASK+1 chunks is visited whole.

// 32x32x16 operand rows: lane reads row R + lane%32, elements 16kk + 8(lane/32) .. +7
template <int ROWB>
struct RowOps32 {
  static constexpr int NB = (Swizzle<ROWB>::MASK + 1) / 2;  // k-steps per XOR group
  int b[NB];
  __device__ __forceinline__ explicit RowOps32(int lane) {
#pragma unroll
    for (int k = 0; k < NB; ++k) b[k] = toff<ROWB>(lane & 31, 16 * k + 8 * (lane >> 5));
  }
  __device__ __forceinline__ int off(int R, int kk) const {
    return b[kk % NB] + (kk / NB) * (Swizzle<ROWB>::MASK + 1) * 16 + R * ROWB;
  }
};

// 32x32x16 transpose operand: column 32md + lane%32, rows R + 4(lane/32) + 0..3
// (k-slots 0..3) and R + 8 + 4(lane/32) + 0..3 (k-slots 4..7)
template <int ROWB>
struct TrOps32 {
  static constexpr int NP = (Swizzle<ROWB>::MASK + 1) / 4;  // md blocks per XOR group
  int t[NP][2];
  __device__ __forceinline__ explicit TrOps32(int lane) {
    const int i = lane & 15, g1 = (lane >> 4) & 1, h = lane >> 5;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec)
        t[p][sec] = toff<ROWB>(4 * h + 8 * sec + (i >> 2), 32 * p + 16 * g1 + 4 * (i & 3));
  }
  __device__ __forceinline__ u32x4 read(const char ETS_LDS* base, int R, int md) const {
    const int o = (md / NP) * (Swizzle<ROWB>::MASK + 1) * 16 + R * ROWB;
    const s16x4 a = lds_tr4(base, t[md % NP][0] + o), c = lds_tr4(base, t[md % NP][1] + o);
    const s16x8 v = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    return __builtin_bit_cast(u32x4, v);
  }
};

// 16x16x32 operand rows: lane reads row R + lane%16, elements 32kk + 8(lane/16) .. +7
template <int ROWB>
struct RowOps16 {
  static constexpr int NB = (Swizzle<ROWB>::MASK + 1) / 4;
  int b[NB];
  __device__ __forceinline__ explicit RowOps16(int lane) {
#pragma unroll
    for (int k = 0; k < NB; ++k) b[k] = toff<ROWB>(lane & 15, 32 * k + 8 * (lane >> 4));
  }
  __device__ __forceinline__ int off(int R, int kk) const {
    return b[kk % NB] + (kk / NB) * (Swizzle<ROWB>::MASK + 1) * 16 + R * ROWB;
  }
};

// 16x16x32 transpose operand: column 16m + lane%16, rows 4(lane/16) + 0..3
// (k-slots 0..3) and 16 + 4(lane/16) + 0..3 (k-slots 4..7)
template <int ROWB>
struct TrOps16 {
  static constexpr int NP = (Swizzle<ROWB>::MASK + 1) / 2;
  int t[NP];
  __device__ __forceinline__ explicit TrOps16(int lane) {
    const int i = lane & 15, G = lane >> 4;
#pragma unroll
    for (int p = 0; p < NP; ++p) t[p] = toff<ROWB>(4 * G + (i >> 2), 16 * p + 4 * (i & 3));
  }
  __device__ __forceinline__ u32x4 read(const char ETS_LDS* base, int m) const {
    const int o = t[m % NP] + (m / NP) * (Swizzle<ROWB>::MASK + 1) * 16;
    const s16x4 a = lds_tr4(base, o), c = lds_tr4(base, o + 16 * ROWB);
    const s16x8 v = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    return __builtin_bit_cast(u32x4, v);
  }
};

// ------------------------------------------------------------ lane exchange
// permlane32_swap(x, x) hands every lane the value of lane (l ^ 32) in one of
// its two results; combining both gives a full cross-half reduction.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled in the source
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction-scheduler groups (LLVM AMDGPU sched_group_barrier masks): the
// compiler fills groups in the order they are declared within a basic block.
enum SchedMask : int { kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedVMEMRead = 0x020, kSchedDSRead = 0x100 };
#define ETS_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
// No instruction may be scheduled across this point.
#define ETS_FENCE() __builtin_amdgcn_sched_barrier(0)

// Pins the computation of x before this point (an empty asm that reads x), so
// that the compiler cannot sink it past a following branch.
template <class T>
__device__ __forceinline__ void materialize(const T& x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3"
// (SC'11): ten rounds of the Philox S-box on a 4x32-bit counter, with the
// 2x32-bit key bumped by the Weyl increments between rounds.
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32 -> 64-bit product gives both halves (v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// Keep bits of dropout for keys j0 .. j0+7 (j0 % 8 == 0) of query row i in
// lane (b*H + h): counter (j0/8, i, lane, 0); key j0 + e is decided by the
// 16-bit half (e mod 2) of word e/2 (low half for even e), kept iff that half
// is >= threshold.  Bit e of the result is key j0 + e.
__device__ __forceinline__ unsigned keep8(const DropArgs& d, int lane_bh, int i, int j0) {
  const U4 w = philox4x32_10((uint32_t)(j0 >> 3), (uint32_t)i, (uint32_t)lane_bh, 0u, d.seed_lo, d.seed_hi);
  const uint32_t t = d.threshold;
  auto two = [t](uint32_t x) __attribute__((always_inline)) {
    return (unsigned)((x & 0xFFFFu) >= t) | ((unsigned)((x >> 16) >= t) << 1);
  };
  return two(w.x) | (two(w.y) << 2) | (two(w.z) << 4) | (two(w.w) << 6);
}

// Query-major layout (a lane of half h32 = lane / 32 holds keys
// key0 + 8 g4 + 4 h32 + r, g4, r < 4, of one query row; lanes l and l ^ 32
// hold the same row).  Each lane of the pair draws two of the four 8-key
// blocks of the 32 keys, block 2 h32 + p on call p ...
__device__ __forceinline__ unsigned keep_qm_draw(const DropArgs& d, int lane_bh, int i, int key0, int h32, int p) {
  return keep8(d, lane_bh, i, key0 + 8 * (2 * h32 + p));
}
// ... and the pair swaps them: bit 8 g4 + r of the result keeps key
// key0 + 8 g4 + 4 h32 + r.
__device__ __forceinline__ unsigned keep_qm_merge(unsigned b0, unsigned b1, int h32) {
  const uint32_t own = b0 | (b1 << 8);
  const auto r = __builtin_amdgcn_permlane32_swap(own, own, false, false);
  // r[0]: lanes 0-31 their own blocks 0, 1, lanes 32-63 their partner's;
  // r[1]: lanes 0-31 the partner's blocks 2, 3, lanes 32-63 their own
  const uint32_t all = (uint32_t)r[0] | ((uint32_t)r[1] << 16);  // byte b = block b
  return (all >> (4 * h32)) & 0x0F0F0F0Fu;
}

// ------------------------------------------------------------ allowed sets
// Kernels are compiled per mask kind so that the common causal / window case
// carries no per-element memory lookups and no layout bookkeeping:
//   kArith   causal and look-back window only (plus ragged tails),
//   kLayout  + variable lengths and row lower bounds (starts): still one key
//            interval per row,
//   kBlock   + the tile mask, read per element only in tiles where it is mixed
//            (lengths and starts handled at run time),
//   kDenseM  + the dense mask.
enum MaskKind { kArith = 0, kLayout = 1, kBlock = 2, kDenseM = 3 };

// one allowed-key interval per row (no per-element memory lookups)
constexpr bool is_interval(int mk) { return mk <= kLayout; }

inline int mask_kind(const MaskArgs& m) {
  if (m.dense_mask) return kDenseM;
  if (m.block_mask) return kBlock;
  return (m.lengths || m.starts) ? kLayout : kArith;
}

// Per-batch view of the layout parts of the allowed set (variable lengths and
// packed segments): rows and keys at or past `len` are inactive, and key j is
// allowed for row i only if j >= st[i] (st null: no lower bound).  `nka` is the
// key extent the allowed set can reach (len when lengths are given, else nk).
struct Layout {
  int len, nka;
  const int32_t* st;
};
// (kArith kernels are built for masks without a layout: nothing to read.)
template <int MK>
__device__ __forceinline__ Layout layout_of(const MaskArgs& m, int b, int nq, int nk) {
  Layout l;
  l.len = nq;
  l.nka = nk;
  l.st = nullptr;
  if constexpr (MK == kArith) return l;
  if (m.lengths) {
    l.len = min(max(m.lengths[b], 0), nq);
    l.nka = min(l.len, nk);
  }
  if (m.starts) l.st = m.starts + (size_t)b * nq;
  return l;
}

// Single (row i, key j) test; nq / nk are the active extents and st the row
// lower bounds of the batch (or null).  check_bm = false skips the block-mask
// lookup (the caller has established that the block mask allows the whole
// tile).
template <int MK>
__device__ __forceinline__ bool allowed1(const MaskArgs& m, int i, int j, int nq, int nk, bool check_bm,
                                         const int32_t* st = nullptr) {
  if (i >= nq || j >= nk) return false;
  if (m.causal && j > i) return false;
  if (m.window > 0 && i - j >= m.window) return false;
  if (st && j < st[i]) return false;
  if constexpr (MK >= kBlock)
    if (check_bm && m.block_mask && m.block_mask[(size_t)(i / m.bq) * m.nbk + j / m.bk] == 0) return false;
  if constexpr (MK == kDenseM)
    if (m.dense_mask && m.dense_mask[(size_t)i * m.dm_stride + j] == 0) return false;
  return true;
}

// Allowed bits of keys j0 .. j0+3 for query row i (bit r <-> key j0 + r).
template <int MK>
__device__ __forceinline__ unsigned allowed4(const MaskArgs& m, int i, int j0, int nq, int nk, bool check_bm,
                                             const int32_t* st = nullptr) {
  unsigned bits = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) bits |= (allowed1<MK>(m, i, j0 + r, nq, nk, check_bm, st) ? 1u : 0u) << r;
  return bits;
}

// Allowed bits of query rows i0 .. i0+3 for key j (bit r <-> row i0 + r).
template <int MK>
__device__ __forceinline__ unsigned allowed4_rows(const MaskArgs& m, int i0, int j, int nq, int nk, bool check_bm,
                                                  const int32_t* st = nullptr) {
  unsigned bits = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) bits |= (allowed1<MK>(m, i0 + r, j, nq, nk, check_bm, st) ? 1u : 0u) << r;
  return bits;
}

// Lowest and highest row lower bound (starts) over rows [r0, r1] (inclusive)
// that are active (< len): every lane of the wave computes the same pair.
// Rows past len do not count; with none active, smin = INT_MAX (every key is
// below it) and smax = INT_MIN.  Covers up to 128 rows.
__device__ __forceinline__ void start_range(const int32_t* st, int r0, int r1, int len, int lane, int& smin,
                                            int& smax) {
  r1 = min(r1, len - 1);
  int lo = 0x7fffffff, hi = (int)0x80000000;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = r0 + lane + 64 * k;
    if (r <= r1) {
      const int v = st[r];
      lo = min(lo, v);
      hi = max(hi, v);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off, 64));
    hi = max(hi, __shfl_xor(hi, off, 64));
  }
  smin = __builtin_amdgcn_readfirstlane(lo);  // uniform: keep it in a scalar register
  smax = __builtin_amdgcn_readfirstlane(hi);
}

enum TileClass { kEmpty = 0, kFull = 1, kPartial = 2, kClassMask = 3, kCheckBlockMask = 4 };

// How a tile's body applies the mask: not at all (every row sees the whole
// tile), as one allowed-key interval per row (causal, window, lengths, starts;
// also a tile mask that is uniform over the tile), or element by element.
enum TileBody { kWhole = 0, kPartIv = 1, kPartEl = 2 };
template <int T>
using BodyTag = std::integral_constant<int, T>;

// Classify the rectangle of query rows [ia, ib] x keys [ja, jb] (inclusive;
// jb may run past nk for a ragged last tile).  Uniform across the wave.
// nq / nk are the active extents; smin / smax bound the row lower bounds
// (starts) of the rectangle's active rows (INT_MIN, INT_MIN without starts).
// Returns kEmpty, kFull or kPartial, plus kCheckBlockMask when the block mask
// is mixed inside the rectangle and must be read per element.
template <int MK>
__device__ __forceinline__ int classify(const MaskArgs& m, int ia, int ib, int ja, int jb, int nq, int nk,
                                        int smin = (int)0x80000000, int smax = (int)0x80000000) {
  if (ia >= nq || ja >= nk) return kEmpty;
  if (jb < smin) return kEmpty;
  // rows or keys past the end are present in the tile: mask them per element
  int cls = (jb >= nk || ib >= nq || ja < smax) ? kPartial : kFull;
  if (ib >= nq) ib = nq - 1;
  if (jb >= nk) jb = nk - 1;
  if (m.causal) {
    if (ja > ib) return kEmpty;
    if (jb > ia) cls = kPartial;
  }
  if (m.window > 0) {
    if (ia - jb >= m.window) return kEmpty;
    if (ib - ja >= m.window) cls = kPartial;
  }
  if (MK >= kBlock && m.block_mask) {
    const int r0 = ia / m.bq, r1 = ib / m.bq, c0 = ja / m.bk, c1 = jb / m.bk;
    if ((r1 - r0 + 1) * (c1 - c0 + 1) > 64) {
      cls = kPartial | kCheckBlockMask;
    } else {
      int ones = 0, tot = 0;
      for (int r = r0; r <= r1; ++r)
        for (int c = c0; c <= c1; ++c) {
          ones += m.block_mask[(size_t)r * m.nbk + c] != 0;
          ++tot;
        }
      if (ones == 0) return kEmpty;
      if (ones != tot) cls = kPartial | kCheckBlockMask;
    }
  }
  if (MK == kDenseM && m.dense_mask) cls = (cls & kCheckBlockMask) | kPartial;
  return cls;
}

// Classes of 64 consecutive tiles (or dK/dV steps) starting at `base`, one
// tile per lane, for the mask kinds that read memory to classify (tile and
// dense masks): the lookups of a whole chunk are issued together instead of a
// dependent load per tile on the way from one tile to the next.  `nonempty`
// is the workgroup's rectangle, the other three the calling wave's.  All bits
// are wave-uniform.
struct TileClasses {
  int base;
  uint64_t nonempty, full, part, cbm;
  __device__ __forceinline__ void set(int b, int cls_wg, int cls_wave) {
    base = b;
    nonempty = __builtin_amdgcn_ballot_w64(cls_wg != kEmpty);
    full = __builtin_amdgcn_ballot_w64((cls_wave & kClassMask) == kFull);
    part = __builtin_amdgcn_ballot_w64((cls_wave & kClassMask) == kPartial);
    cbm = __builtin_amdgcn_ballot_w64((cls_wave & kCheckBlockMask) != 0);
  }
  __device__ __forceinline__ bool covers(int t) const { return base >= 0 && t >= base && t < base + 64; }
  // the wave's class of tile t (covers(t) must hold), in classify()'s encoding
  __device__ __forceinline__ int wave_class(int t) const {
    const uint64_t bit = 1ull << (t - base);
    if (full & bit) return kFull;
    if (part & bit) return kPartial | ((cbm & bit) ? kCheckBlockMask : 0);
    return kEmpty;
  }
  // first tile >= t of the chunk whose workgroup rectangle is not empty, or -1
  __device__ __forceinline__ int next_nonempty(int t) const {
    const uint64_t m = nonempty >> (t - base);
    return m ? t + (int)__builtin_ctzll(m) : -1;
  }
};

}  // namespace ets
