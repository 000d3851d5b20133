// Pieces shared by the forward and backward attention kernels on gfx950:
// vector types, the swizzled LDS layout of 64-row x 64-feature bf16 tiles
// and their two read patterns, lane-half exchanges, the XCD-aware block
// remap, the wait-and-barrier used with LDS DMA, and host-side checks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "attn.h"

namespace attn_detail {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 64;     // head size
constexpr int kRow = 128;  // bytes per tile row (64 bf16)

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// max(x[lane], x[lane ^ 32]) in every lane, via v_permlane32_swap (which
// exchanges the upper half of one register with the lower half of another).
__device__ __forceinline__ float half_swap_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// XCD-aware block remap.  Workgroups are dealt round-robin to the 8 XCDs; this
// makes the workgroups that land on one XCD take consecutive logical tiles, so
// the query tiles of one head share that XCD's L2 while they stream its K/V.
__host__ __device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = w & 7, i = w >> 3;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// Causal order of the logical tiles: n_bh heads of `blocks` row blocks each,
// rank 0 the longest block of a head.  One XCD takes consecutive logical
// tiles, i.e. a block of about n_bh/8 heads; within each block of
// ceil(n_bh/8) heads the tiles run rank by rank (the longest of every head
// first), so the XCD's CUs start on long tiles and finish on short ones.
// (Head by head, a long tile of the block's last heads would start last.)
__device__ __forceinline__ void causal_order(int logical, int n_bh, int blocks, int& bh, int& rank) {
  const int hb = (n_bh + 7) / 8;
  const int blk = logical / (hb * blocks);
  const int within = logical - blk * hb * blocks;
  const int nh = min(hb, n_bh - blk * hb);  // heads in this block
  rank = within / nh;
  bh = blk * hb + (within - rank * nh);
}

// 16-byte chunk c of tile row r lives at chunk position c ^ swz(r) of that
// row: the row-operand reads (16 rows, one chunk) and the transpose reads (4
// rows, 4 chunks per half wave) then hit 64 distinct banks.
__device__ __forceinline__ int swz(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * kRow + ((chunk ^ swz(row)) << 4); }

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, int off) {
  return *(const bf16x8*)(base + off);
}

// Two ds_read_b64_tr_b16: the transposed operand (8 rows of one column per
// lane) of an MFMA from a row-major tile.
__device__ __forceinline__ bf16x8 lds_read_vt(const char* p0, const char* p1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Fourth word of a gfx950 buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

// s_waitcnt vmcnt(N) followed by s_barrier.  A plain s_barrier: the
// compiler's __syncthreads() would also wait for every newer DMA.  The memory
// clobber keeps the compiler from moving memory operations across it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Calls vm_wait_barrier<kPer * c>() for a wave-uniform c in [0, kMax]: c
// tiles of kPer DMAs each may stay in flight.
template <int kPer, int kMax>
__device__ __forceinline__ void vm_wait_barrier_tiles(int c) {
  if constexpr (kMax > 0) {
    if (c >= kMax) {
      vm_wait_barrier<kPer * kMax>();
      return;
    }
    vm_wait_barrier_tiles<kPer, kMax - 1>(c);
  } else {
    vm_wait_barrier<0>();
  }
}

// Calls f(std::integral_constant<int, I>()) for I = kFirst .. kEnd-1.
template <int kFirst, int kEnd>
struct Unroll {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    if constexpr (kFirst < kEnd) {
      f(std::integral_constant<int, kFirst>());
      Unroll<kFirst + 1, kEnd>::run(f);
    }
  }
};

// Host side: ATTN_OK when the current device is a gfx950 (cached per device);
// *cus (if given) receives its compute-unit count.
__attribute__((visibility("hidden"))) attn_status check_device(int* cus = nullptr);

inline bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// The status of a kernel launch.  A rejected launch's error is also taken
// out of the runtime's last-error state: the caller has it as the return
// value, and the next unrelated launch check must not report it again.
inline attn_status launch_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  (void)hipGetLastError();
  return ATTN_E_LAUNCH;
}

// Sizes every kernel handles: tile, row-block and workgroup counts are ints
// (B*H*ceil(N/32) bounds them all), and one head's rows are addressed with
// 32-bit byte offsets (N rows of 128 bytes).  Offsets between heads and
// batch entries are 64-bit, so a tensor may exceed 2^31 elements.
inline bool sizes_fit(int B, int H, int N) {
  return (long long)B * H * ((N + 31LL) / 32) < (1LL << 31) && N < (1 << 24);
}

}  // namespace attn_detail
