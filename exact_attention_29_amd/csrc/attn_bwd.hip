// Backward pass of exact attention for AMD Instinct MI355X (gfx950).
//
// What is computed: for an upstream gradient dO of O = softmax(S) V with
// S = scale * Q K^T (+ causal mask), the gradients
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_f dO_if O_if,
//     dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
// by recomputation as on the page "FlashAttention: Fast and Memory-Efficient
// Exact Attention with IO-Awareness" (reading notes at notes.yuuk.io),
// section "recomputation": the forward pass kept only O and the softmax
// statistics (here LSE), and P = exp(S - LSE) is rebuilt tile by tile from Q
// and K, never stored.
//
// Two kernels on the caller's stream:
//   1. bwd_dq (query-parallel): each wave keeps Q and dO of its 32 queries
//      in registers, first forms each query's L2 = LSE * log2(e) and
//      -D = -sum_f dO_if O_if (from its dO and the matching O features; a
//      lane exchange completes the row) and leaves them in the caller's
//      workspace (rows padded to a multiple of 256; rows past N get
//      L2 = +inf and -D = 0, so a padding query has probability exactly 0),
//      then streams 64-key tiles of K and V: S^T = K Q^T and dP^T = V dO^T
//      (a lane per query), dS^T, then dQ^T += K^T dS^T;
//   2. bwd_dkdv (key-parallel): each wave keeps K and V of its 32 keys in
//      registers as MFMA operands; 64-query tiles of Q, dO, L2 and -D stream
//      through an LDS ring filled by DMA.  S = Q K^T is computed in the layout
//      where each lane holds one key and 16 queries: P and dS then feed
//      dV^T += dO^T P and dK^T += Q^T dS directly as MFMA operands, and the
//      transposed Q / dO operands come from the row-major tiles with
//      ds_read_b64_tr_b16.
// Both kernels run a software pipeline over 32-row steps: step j
// issues the MFMAs of S and dP for step j+1 and of the accumulating products
// of step j-1, one by one, each beside a slice of the vector work of step j
// (exp2, dS, bf16 packing), and reads its MFMA operands from LDS four MFMAs
// ahead.  -D enters dP as the initial value of its accumulator.  Causal
// calls run each XCD's block of heads longest row block first (causal_order).
// Instances for key masks (lengths, bits), block masks and strided tensors
// (each tensor's rows addressed through its own batch, head and row
// strides) share this structure.
// No atomics: every output element is written by exactly one lane, so the
// result is deterministic.  All products on v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation; P and dS are rounded to bf16 for the products, as in
// the forward pass.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

constexpr int kBwdTile = 64;                 // rows of a streamed tile
constexpr int kTileBytes = kBwdTile * kRow;  // 8 KiB
constexpr int kPadRows = 256;                // workspace rows per head: N rounded up to this

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* ws;  // per head bh, at bh * 2 * n_pad: L2[n_pad] = LSE*log2(e), then -D[n_pad]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int n;
  int n_pad;     // n rounded up to kPadRows
  int bh_count;  // B * H
  int blocks;    // ceil(n / rows per workgroup)
  int total;     // B * H * blocks
  float c;       // scale * log2(e)
  float scale;
  const int* key_len;  // [B] or null: keys j >= key_len[b] are hidden (the forward's key mask)
  int heads;           // H: batch entry of head bh is bh / H
  const uint32_t* key_bits;  // [B][words] or null: bit j%32 of word j/32 clear hides key j
  int words;                 // ceil(n / 32)
  const uint8_t* block_mask;  // block-sparse: [ceil(n/128)][mask_cols], 0 hides that block
  int mask_cols;              // ceil(n / 64)
  // strided instances: element strides (batch, head, row) of q, k, v, o,
  // dout, dq, dk, dv (index kTq .. kTdv); the others use [B][H][n][64]
  long long sb[8];
  long long sh[8];
  int sn[8];
};

constexpr int kTq = 0, kTk = 1, kTv = 2, kTo = 3, kTdo = 4, kTdq = 5, kTdk = 6, kTdv = 7;

// Element offset of head bh's [n][64] matrix in tensor t, and its row stride.
template <bool kStrided>
__device__ __forceinline__ size_t head_offset(const BwdArgs& a, int t, int bh) {
  if constexpr (kStrided) {
    const int b = bh / a.heads;
    return (size_t)(b * a.sb[t] + (long long)(bh - b * a.heads) * a.sh[t]);
  } else {
    (void)t;
    return (size_t)bh * a.n * kD;
  }
}
template <bool kStrided>
__device__ __forceinline__ int row_stride(const BwdArgs& a, int t) {
  if constexpr (kStrided) return a.sn[t];
  else {
    (void)a;
    (void)t;
    return kD;
  }
}

// Which (query, key) pairs take part, as a kernel template argument: all of
// them, keys below each entry's valid length, (kKeysBits) keys whose bit is
// set and, when lengths are given too, below the length, or (kKeysBlocks)
// pairs whose 128-query x 64-key block of the block mask is set.
constexpr int kKeysAll = 0, kKeysLen = 1, kKeysBits = 2, kKeysBlocks = 3;
// The block mask's granularity (the forward's block-sparse tiles) and the
// longest list of 64-row tiles a workgroup keeps in LDS (N <= 262,144).
constexpr int kBlockQ = 128, kBlockK = 64, kMaxBlockTiles = 4096;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Keys of head bh that take part: key_len[b] clamped to [0, n] (n when a
// bit-mask call has no lengths), uniform in the workgroup (loaded where
// needed rather than kept live across a loop).
template <int kKeys>
__device__ __forceinline__ int valid_keys(const BwdArgs& a, int bh) {
  if constexpr (kKeys == kKeysLen || kKeys == kKeysBits) {
    if (kKeys == kKeysBits && !a.key_len) return a.n;
    return __builtin_amdgcn_readfirstlane(min(max(a.key_len[bh / a.heads], 0), a.n));
  } else {
    return a.n;
  }
}

// Bit word w (keys 32w .. 32w+31) of head bh's batch entry.
__device__ __forceinline__ uint32_t key_word(const BwdArgs& a, int bh, int w) {
  return a.key_bits[(size_t)(bh / a.heads) * a.words + w];
}

// 16-byte chunk `ch` of row `row` of a [n][64] bf16 matrix whose rows are
// `rs` elements apart, zero past row n.
__device__ __forceinline__ u32x4 load_chunk(const uint16_t* base, int row, int ch, int n, int rs = kD) {
  u32x4 w = {0u, 0u, 0u, 0u};
  if (row < n) w = *(const u32x4*)(base + (size_t)row * rs + 8 * ch);
  return w;
}

// The 8 bf16 of features 16*ks + 8*hi .. +7 of one row, as an MFMA operand.
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* base, int row, int ks, int hi, int n, int rs = kD) {
  return __builtin_bit_cast(bf16x8, load_chunk(base, row, 2 * ks + hi, n, rs));
}

// Per-lane offsets of the transposed-operand reads (two ds_read_b64_tr_b16):
// 8 rows of one column per lane, rows 16*tt + 8*(i/4) + 4*hi + i%4 of a
// 16-row slice, column 32*db + lane%32.
struct TrOffsets {
  int off[2][2];  // [sec][db]
  __device__ TrOffsets(int lane) {
    const int hi = lane >> 5, g = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int row = 4 * hi + (j16 >> 2) + 8 * sec;
        const int byte = 2 * (32 * db + 16 * (g & 1) + 4 * (j16 & 3));
        off[sec][db] = row * kRow + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
      }
  }
};

// Pins a value to the current pipeline slot (left alone, the compiler sinks
// products and packs to the end of a step).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(unsigned& x) { asm volatile("" : "+v"(x)); }

// Word w (0..3) of an 8 x bf16 operand set to the packed pair x.
__device__ __forceinline__ void set_word(bf16x8& op, int w, unsigned x) {
  u32x4 words = __builtin_bit_cast(u32x4, op);
  words[w] = x;
  op = __builtin_bit_cast(bf16x8, words);
}

__device__ __forceinline__ unsigned pack_bf16(float x, float y) {
  const bf16x2 p = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(unsigned, p);
}

// x where bit kb (lanes 0-31) or bit kb + 4 (lanes 32-63) of the uniform
// word w is set, else 0: the two bits as a lane mask in an SGPR pair (scalar
// work; kb is a constant once unrolled, 0 <= kb <= 27) and one v_cndmask_b32
// (the compiler would test the bit per lane).
__device__ __forceinline__ float keep_bit(float x, uint32_t w, int kb) {
  const uint32_t lo = (uint32_t)((int)(w << (31 - kb)) >> 31);
  const uint32_t hi = (uint32_t)((int)(w << (27 - kb)) >> 31);
  const uint64_t m = (uint64_t)lo | ((uint64_t)hi << 32);
  float r;
  asm("v_cndmask_b32 %0, 0, %1, %2" : "=v"(r) : "v"(x), "s"(m));
  return r;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Streaming 64-row tiles of two [n][64] bf16 matrices (and, for dK/dV, the
// 64 values of each workspace array) into one LDS stage by DMA
// (buffer/global loads with the LDS bit, 16 bytes per lane).  In pass p,
// lane l of wave w fills chunk slot l%8 of row 8*w + l/8 + 8*kWaves*p, so it
// fetches global chunk (l%8) ^ swz(row) of that row (swz depends on row bits
// 1-3 only: the same chunk in every pass).  Rows past N of the ragged last
// tile re-read row N-1: finite data whose probability is 0 or masked.
template <int kWaves, bool kStats, bool kStr = false>
struct TileDma {
  static constexpr int kPassRows = 8 * kWaves;
  static constexpr int kPasses = kBwdTile / kPassRows;
  static constexpr int kStatLanes = 32 / kWaves;  // 16-byte stat chunks per wave
  static constexpr int kPerTile = 2 * kPasses + (kStats ? 1 : 0);
  static_assert(kPassRows % 16 == 0, "a pass must not change the row swizzle");

  __amdgpu_buffer_rsrc_t r0, r1, rs;
  const uint16_t* g0;
  const uint16_t* g1;
  int n, lane, row_in, chunk, lane_off, wave_s, stat_voff;
  int e0, e1, lane_off1;  // kStr: row strides of the two matrices (elements), matrix 1's lane offset

  // stats: this head's L2[n_pad], then -D[n_pad] (dK/dV only).  kStr: the
  // matrices' rows are rs0, rs1 elements apart (multiples of 8; the byte
  // offsets up to row n-1 below 2^31, checked on the host), else 64.
  __device__ TileDma(const uint16_t* m0, const uint16_t* m1, int n_, int wave, int lane_, const float* stats,
                     int n_pad, int rs0 = kD, int rs1 = kD)
      : g0(m0), g1(m1), n(n_), lane(lane_) {
    row_in = 8 * wave + (lane >> 3);
    chunk = (lane & 7) ^ swz(row_in);
    wave_s = __builtin_amdgcn_readfirstlane(wave);
    if constexpr (kStr) {
      e0 = rs0;
      e1 = rs1;
      lane_off = row_in * 2 * e0 + chunk * 16;
      lane_off1 = row_in * 2 * e1 + chunk * 16;
      r0 = __builtin_amdgcn_make_buffer_rsrc((void*)m0, (short)0, (n - 1) * 2 * e0 + kRow, kBufferWord3);
      r1 = __builtin_amdgcn_make_buffer_rsrc((void*)m1, (short)0, (n - 1) * 2 * e1 + kRow, kBufferWord3);
    } else {
      (void)rs0;
      (void)rs1;
      e0 = e1 = kD;
      lane_off = row_in * kRow + chunk * 16;
      lane_off1 = lane_off;
      r0 = __builtin_amdgcn_make_buffer_rsrc((void*)m0, (short)0, n * kRow, kBufferWord3);
      r1 = __builtin_amdgcn_make_buffer_rsrc((void*)m1, (short)0, n * kRow, kBufferWord3);
    }
    stat_voff = 0;
    if constexpr (kStats) {
      // chunk ci of a tile's stats: L2 in chunks 0-15, -D in chunks 16-31
      const int ci = kStatLanes * wave + lane;
      stat_voff = ci < 16 ? 16 * ci : n_pad * 4 + 16 * (ci - 16);
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)stats, (short)0, n_pad * 8, kBufferWord3);
    }
  }

  // tile t into stage sb: matrix 0 at sb, matrix 1 at sb + 8 KiB, stats at
  // sb + 16 KiB (L2[64], then -D[64])
  __device__ __forceinline__ void issue(int t, char* sb) const {
    char* d = sb + wave_s * 1024;
    if ((t + 1) * kBwdTile <= n) {
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const int row0 = t * kBwdTile + ps * kPassRows;
        const int soff = kStr ? row0 * 2 * e0 : row0 * kRow;
        const int soff1 = kStr ? row0 * 2 * e1 : soff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, (lds_void*)(d + ps * kPassRows * kRow), 16, lane_off, soff,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_void*)(d + kTileBytes + ps * kPassRows * kRow), 16,
                                                 lane_off1, soff1, 0, 0);
      }
    } else {
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const int row = min(t * kBwdTile + row_in + ps * kPassRows, n - 1);
        __builtin_amdgcn_global_load_lds((global_void*)(g0 + (size_t)row * (kStr ? e0 : kD) + chunk * 8),
                                         (lds_void*)(d + ps * kPassRows * kRow), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((global_void*)(g1 + (size_t)row * (kStr ? e1 : kD) + chunk * 8),
                                         (lds_void*)(d + kTileBytes + ps * kPassRows * kRow), 16, 0, 0);
      }
    }
    if constexpr (kStats) {
      if (lane < kStatLanes)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sb + 2 * kTileBytes + wave_s * kStatLanes * 16),
                                                 16, stat_voff, t * kBwdTile * 4, 0, 0);
    }
  }
};

// The LDS stages of a ring, each its own object: the compiler then tells a
// read of one stage from the DMA in flight into another, and waits only for
// the DMA that wrote the stage it reads.  `ring(s)` with a constant s is the
// stage itself; the objects past kStages are never referenced (and dropped),
// so a ring of exactly 80 KiB still lets two workgroups share a CU.
#define ATTN_BWD_RING(kBytes, kStages, ring)                                                    \
  static_assert((kStages) >= 4 && (kStages) <= 6, "ring of 4 to 6 stages");                    \
  __shared__ __attribute__((aligned(1024))) char ring##0[kBytes];                               \
  __shared__ __attribute__((aligned(1024))) char ring##1[kBytes];                               \
  __shared__ __attribute__((aligned(1024))) char ring##2[kBytes];                               \
  __shared__ __attribute__((aligned(1024))) char ring##3[kBytes];                               \
  __shared__ __attribute__((aligned((kStages) > 4 ? 1024 : 1))) char ring##4[(kStages) > 4 ? (kBytes) : 1]; \
  __shared__ __attribute__((aligned((kStages) > 5 ? 1024 : 1))) char ring##5[(kStages) > 5 ? (kBytes) : 1]; \
  auto ring = [&](int s) -> char* {                                                             \
    if constexpr ((kStages) == 4) return s == 0 ? ring##0 : s == 1 ? ring##1 : s == 2 ? ring##2 : ring##3; \
    else if constexpr ((kStages) == 5)                                                          \
      return s == 0 ? ring##0 : s == 1 ? ring##1 : s == 2 ? ring##2 : s == 3 ? ring##3 : ring##4; \
    else                                                                                        \
      return s == 0 ? ring##0 : s == 1 ? ring##1 : s == 2 ? ring##2 : s == 3 ? ring##3 : s == 4 ? ring##4 \
                                                                                         : ring##5; \
  }

// Tile schedule of both kernels.  During the two steps of tile t the ring
// holds tiles t-1 (accumulating products of step 2t-1), t and t+1 (S and dP
// of step 2t+2); the barrier that ends tile t publishes tile t+2, and then
// the stage of tile t-1 is refilled with tile t+kStages-1.  So: the prologue
// issues tiles t0 .. t0+kStages-2 and waits for t0 and t0+1; the barrier of
// tile t lets tiles t+3 .. min(t_end-1, t+kStages-2) fly on.

// ------------------------------------------------------------------ dK, dV

// kKeys (kKeysAll, kKeysLen, kKeysBits): hidden keys (past the batch
// entry's valid length, or with a clear bit) are hidden from every query;
// they get dK = dV = 0 (each output column is one key, so zeroing it at the
// end is exact whatever its accumulators hold).  A workgroup whose keys all
// lie past the valid length only writes those zeros.  kKeysBlocks: the
// workgroup visits only the query tiles whose block is set in one of its two
// key columns of the block mask, pipelined like the others, and a wave drops
// (P = dS = 0) the tiles its own column, or the causal mask, hides: on the
// general path by a select, on the pipelined one by reading +inf for the
// tile's L2 values.
template <bool kCausal, int kWaves, int kKeys, bool kStrided = false>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kStages = kWaves == 8 ? 5 : 4;
  constexpr int kRows = 32 * kWaves;        // keys per workgroup
  constexpr int kStatOff = 2 * kTileBytes;  // L2[64], then -D[64]
  constexpr int kStageBytes = kStatOff + 2 * kBwdTile * 4;
  using Dma = TileDma<kWaves, true, kStrided>;
  ATTN_BWD_RING(kStageBytes, kStages, stage);

  const int n = a.n;
  const int logical = xcd_remap(blockIdx.x, a.total);
  int bh, kb;
  if constexpr (kCausal) {
    causal_order(logical, a.bh_count, a.blocks, bh, kb);  // key block 0 sees every query
  } else {
    bh = logical / a.blocks;
    kb = logical - bh * a.blocks;
  }
  const uint16_t* qg = a.q + head_offset<kStrided>(a, kTq, bh);
  const uint16_t* kg = a.k + head_offset<kStrided>(a, kTk, bh);
  const uint16_t* vg = a.v + head_offset<kStrided>(a, kTv, bh);
  const uint16_t* dog = a.dout + head_offset<kStrided>(a, kTdo, bh);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int key0 = kb * kRows + wave_s * 32;  // this wave's first key
  const int key = key0 + l32;                 // this lane's key
  if constexpr (kKeys == kKeysLen || kKeys == kKeysBits) {
    if (kb * kRows >= valid_keys<kKeys>(a, bh)) {  // uniform: before any barrier
      if (key < n) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int f = 32 * hi; f < 32 * hi + 32; f += 8) {
          *(u32x4*)(a.dk + head_offset<kStrided>(a, kTdk, bh) + (size_t)key * row_stride<kStrided>(a, kTdk) + f) = z;
          *(u32x4*)(a.dv + head_offset<kStrided>(a, kTdv, bh) + (size_t)key * row_stride<kStrided>(a, kTdv) + f) = z;
        }
      }
      return;
    }
  }

  // kKeysBlocks: the 64-query tiles whose query block has either of this
  // workgroup's two key columns set (causal: none before its first key),
  // compacted into blk_list (wave 0 writes, every wave counts), each entry
  // the tile with bit 14 + c set when column c of the two is set; from here
  // on a tile index is a position in that list.  inf_l2 holds +inf in place
  // of a tile's L2 values: a pipelined step of a wave whose column the tile
  // does not set reads its L2 there, so its probabilities are exactly 0.
  __shared__ uint16_t blk_list[kKeys == kKeysBlocks ? kMaxBlockTiles : 1];
  __shared__ __attribute__((aligned(16))) float inf_l2[kKeys == kKeysBlocks ? 64 : 1];
  int n_listed = 0;
  if constexpr (kKeys == kKeysBlocks) {
    static_assert(kRows == 2 * kBlockK, "a workgroup spans two key columns of the block mask");
    const int tq_end = (n + kBwdTile - 1) / kBwdTile;
    const int c0 = 2 * kb;
    const bool c1_in = c0 + 1 < a.mask_cols;
    for (int base = kCausal ? (kb * kRows) / kBwdTile : 0; base < tq_end; base += 64) {
      const int t = base + lane;
      bool set0 = false, set1 = false;
      if (t < tq_end) {
        const uint8_t* mrow = a.block_mask + (size_t)(t * kBwdTile / kBlockQ) * a.mask_cols;
        set0 = mrow[c0] != 0;
        set1 = c1_in && mrow[c0 + 1] != 0;
      }
      const bool act = set0 || set1;
      const uint64_t bal = __ballot(act);
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
      if (wave == 0 && act) blk_list[n_listed + below] = (uint16_t)(t | (set0 ? 1 << 14 : 0) | (set1 ? 1 << 15 : 0));
      n_listed += __popcll(bal);
    }
    if (tid < 64) inf_l2[tid] = INFINITY;
    __syncthreads();
  }
  // the query tile at list position t (kKeysBlocks), else tile t itself
  auto tile_of = [&](int t) -> int {
    if constexpr (kKeys == kKeysBlocks) return __builtin_amdgcn_readfirstlane((int)blk_list[t]) & 0x3fff;
    else return t;
  };

  // K^T and V^T operands (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kop[4], vop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kop[ks] = row_operand(kg, key, ks, hi, n, row_stride<kStrided>(a, kTk));
    vop[ks] = row_operand(vg, key, ks, hi, n, row_stride<kStrided>(a, kTv));
  }
  const TrOffsets tr(lane);
  int row_off[4];  // row-operand read of step ks: row l32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) row_off[ks] = tile_off(l32, 2 * ks + hi);

  // 64-query tiles of the workgroup (kKeysBlocks: list positions)
  const int t0 = kKeys == kKeysBlocks ? 0 : kCausal ? (kb * kRows) / kBwdTile : 0;
  const int t_end = kKeys == kKeysBlocks ? n_listed : (n + kBwdTile - 1) / kBwdTile;
  // 32-query halves this wave works on: [jf, jl], every half of the tiles.
  // Causal: from the half that starts at the wave's first key (the
  // diagonal, masked per element).  Queries past N have L2 = +inf, so their
  // probabilities are exactly 0.  (A wave whose keys all lie past N runs
  // like the others; nothing of it is written.)
  const int jl = 2 * t_end - 1;
  const int jf = kCausal && kKeys != kKeysBlocks ? key0 / 32 : 0;
  // Tiles t0 .. t0+kHead-1 run on the general path; then tiles whose two
  // steps are fast in every wave (2t > the last wave's first half, 2t+1 <
  // jl) run pipelined, in whole turns of the ring and a last partial one;
  // the rest on the general path again.
  constexpr int kHead = kCausal ? (kWaves + 1) / 2 : 1;
  const int t_fast_end = jl >= 2 ? (jl - 2) / 2 + 1 : 0;
  const Dma dma(qg, dog, n, wave, lane, a.ws + (size_t)bh * 2 * a.n_pad, a.n_pad, row_stride<kStrided>(a, kTq),
                row_stride<kStrided>(a, kTdo));
  auto dma_issue = [&](int t, char* sb) { dma.issue(tile_of(t), sb); };

  // a step is fast (pipelined, unmasked) when it has a step on each side
  auto fast = [&](int j) { return j >= jf + 1 && j <= jl - 1; };
  // stage of half j (tile j/2; the half's rows start at 32*(j&1))
  auto half_stage = [&](int j) { return stage((j / 2 - t0) % kStages); };
  (void)half_stage;

  // operand readers; sb = stage, h = half within the tile (0, 1)
  auto q_row = [&](const char* sb, int h, int ks) { return lds_read_b128(sb, h * 32 * kRow + row_off[ks]); };
  auto do_row = [&](const char* sb, int h, int ks) {
    return lds_read_b128(sb + kTileBytes, h * 32 * kRow + row_off[ks]);
  };
  auto tr_read = [&](const char* m, int h, int i) {  // i = 2*tt + db
    const char* b = m + (32 * h + 16 * (i >> 1)) * kRow;
    return lds_read_vt(b + tr.off[0][i & 1], b + tr.off[1][i & 1]);
  };
  // L2 of registers 4*g4 .. 4*g4+3 (queries 8*g4 + 4*hi + 0..3 of the half);
  // lb = the stage's L2 values (stage + kStatOff) or inf_l2
  auto l2_group = [&](const char* lb, int h, int g4) -> f32x4 {
    return *(const f32x4*)(lb + 16 * (8 * h + 2 * g4 + hi));
  };
  // where a pipelined step of this wave reads the L2 values of list position
  // t held in stage sb: inf_l2 when its column of the block mask is clear
  // (t = n_listed, past the list, is asked for by the last tile and unused:
  // it reads the last entry instead)
  auto l2_base = [&](const char* sb, int t) -> const char* {
    if constexpr (kKeys == kKeysBlocks) {
      const int e = __builtin_amdgcn_readfirstlane((int)blk_list[max(0, min(t, n_listed - 1))]);
      return (e >> (14 + wave_s / 2)) & 1 ? sb + kStatOff : reinterpret_cast<const char*>(inf_l2);
    } else {
      (void)t;
      return sb + kStatOff;
    }
  };
  auto nd_block = [&](const char* sb, int h) -> f32x16 {
    f32x16 r;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 x = *(const f32x4*)(sb + kStatOff + 4 * kBwdTile + 16 * (8 * h + 2 * g4 + hi));
#pragma unroll
      for (int e = 0; e < 4; ++e) r[4 * g4 + e] = x[e];
    }
    return r;
  };
  // A operand of MFMA slot s (0..15) of a fast step; nb/hn = half j+1 (S,
  // dP), pb/hp = half j-1 (dV, dK)
  auto slot_operand = [&](int s, const char* nb, int hn, const char* pb, int hp) {
    const int g = s >> 2;
    switch (s & 3) {
      case 0: return q_row(nb, hn, g);
      case 1: return tr_read(pb + kTileBytes, hp, g);  // dO^T
      case 2: return tr_read(pb, hp, g);               // Q^T
      default: return do_row(nb, hn, g);
    }
  };

  f32x16 acc_dk[2], acc_dv[2];  // dK^T, dV^T: rows = features, columns = keys
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_dk[db][r] = acc_dv[db][r] = 0.f;
  const f32x16 zero16 = {};
  const float c = a.c;

  // pipeline state: S and dP - D of a half (lane = key, register r = query
  // 8*(r/4) + 4*hi + r%4 of the half), its bf16 P and dS as MFMA B operands
  // (even steps fill the A set, odd steps the B set), the A operands of the
  // next four MFMA slots, and L2 of the next half's first four registers
  f32x16 sA = zero16, sB = zero16, dpA = zero16, dpB = zero16;
  bf16x8 pA[2], pB[2], dsA[2], dsB[2];
  bf16x8 ring[4];
  f32x4 l2n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) pA[i] = pB[i] = dsA[i] = dsB[i] = bf16x8{};
#pragma unroll
  for (int i = 0; i < 4; ++i) ring[i] = bf16x8{};

  // Step j on the general path: whichever of S, dP(j+1), P, dS(j) (with the
  // causal diagonal mask) and dV, dK(j-1) exist, in plain order; then, when
  // step j+1 is fast, its first four operands and L2 group.  Stages and half
  // indices as for step_fast.
  auto step_general = [&](int j, const char* nb, int hn, const char* cb, int hc, const char* pb, int hp,
                          const char* nnb, const char* ln, f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt,
                          f32x16& dp_nxt, const bf16x8 (&p_prv)[2], const bf16x8 (&ds_prv)[2], bf16x8 (&p_cur)[2],
                          bf16x8 (&ds_cur)[2]) __attribute__((always_inline)) {
    if (j + 1 >= jf && j + 1 <= jl) {
      dp_nxt = nd_block(nb, hn);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s_nxt = mfma(q_row(nb, hn, ks), kop[ks], ks == 0 ? zero16 : s_nxt);
        dp_nxt = mfma(do_row(nb, hn, ks), vop[ks], dp_nxt);
        __builtin_amdgcn_sched_barrier(0);  // one operand pair in flight at a time
      }
    }
    if (j - 1 >= jf && j - 1 <= jl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc_dv[i & 1] = mfma(tr_read(pb + kTileBytes, hp, i), p_prv[i >> 1], acc_dv[i & 1]);
        acc_dk[i & 1] = mfma(tr_read(pb, hp, i), ds_prv[i >> 1], acc_dk[i & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (j >= jf && j <= jl) {
      bool diag = kCausal && j == jf;  // key > query hidden
      bool none = false;               // kKeysBlocks: the whole half is hidden from this wave
      if constexpr (kKeys == kKeysBlocks) {
        const int tq = tile_of(j >> 1);
        const int rh = 2 * tq + (j & 1);  // the half's query rows start at 32 * rh
        const int col = key0 / kBlockK;
        diag = kCausal && rh == key0 / 32;
        none = (kCausal && rh < key0 / 32) || col >= a.mask_cols ||
               a.block_mask[(size_t)(tq * kBwdTile / kBlockQ) * a.mask_cols + col] == 0;
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 l4 = l2_group(cb + kStatOff, hc, g4);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const int r = 4 * g4 + e;
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], c, -l4[e]));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r + 1], c, -l4[e + 1]));
          if (diag && l32 > 8 * g4 + 4 * hi + e) p0 = 0.f;
          if (diag && l32 > 8 * g4 + 4 * hi + e + 1) p1 = 0.f;
          if constexpr (kKeys == kKeysBlocks) {
            if (none) p0 = p1 = 0.f;
          }
          set_word(p_cur[r >> 3], (r & 7) >> 1, pack_bf16(p0, p1));
          set_word(ds_cur[r >> 3], (r & 7) >> 1, pack_bf16(p0 * dp_cur[r], p1 * dp_cur[r + 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (fast(j + 1)) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ring[s] = slot_operand(s, nnb, hc, cb, hc);
      l2n = l2_group(ln, hn, 0);
    }
  };

  // Step j on the fast path.  nb/hn: half j+1; cb/hc: half j; pb/hp: half
  // j-1; nnb: half j+2 (half index hc); lc, ln: where half j's and half
  // j+1's L2 values are read (l2_base).  16 MFMA slots; in group g: S(j+1)
  // step g, dV(j-1) step g, dK(j-1) step g, dP(j+1) step g (its accumulator
  // starts at -D).  Vector work on score pair k: FMA in slot 2k, exp2 in slot
  // 2k+1, products and packs in slot 2k+2.
  auto step_fast = [&](const char* nb, int hn, const char* cb, int hc, const char* pb, int hp, const char* nnb,
                       const char* lc, const char* ln, f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt,
                       f32x16& dp_nxt, const bf16x8 (&p_prv)[2], const bf16x8 (&ds_prv)[2], bf16x8 (&p_cur)[2],
                       bf16x8 (&ds_cur)[2]) __attribute__((always_inline)) {
    f32x4 l2g[4];
    l2g[0] = l2n;
    dp_nxt = nd_block(nb, hn);
    float t[16], e[16];
    auto finish_pair = [&](int k) {
      const int r = 2 * k;
      unsigned pw = pack_bf16(e[r], e[r + 1]);
      unsigned dw = pack_bf16(e[r] * dp_cur[r], e[r + 1] * dp_cur[r + 1]);
      pin(pw);
      pin(dw);
      set_word(p_cur[r >> 3], (r & 7) >> 1, pw);
      set_word(ds_cur[r >> 3], (r & 7) >> 1, dw);
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int g = s >> 2;
      switch (s & 3) {
        case 0: s_nxt = mfma(ring[s & 3], kop[g], g == 0 ? zero16 : s_nxt); break;
        case 1: acc_dv[g & 1] = mfma(ring[s & 3], p_prv[g >> 1], acc_dv[g & 1]); break;
        case 2: acc_dk[g & 1] = mfma(ring[s & 3], ds_prv[g >> 1], acc_dk[g & 1]); break;
        default: dp_nxt = mfma(ring[s & 3], vop[g], dp_nxt); break;
      }
      // operand of slot s+4 (of the next step, for the last four slots)
      if (s + 4 < 16) ring[s & 3] = slot_operand(s + 4, nb, hn, pb, hp);
      else ring[s & 3] = slot_operand(s - 12, nnb, hc, cb, hc);
      if (s == 1 || s == 5 || s == 9) l2g[(s + 3) >> 2] = l2_group(lc, hc, (s + 3) >> 2);
      if (s == 13) l2n = l2_group(ln, hn, 0);
      const int k = s >> 1;
      if ((s & 1) == 0) {
        t[2 * k] = __builtin_fmaf(s_cur[2 * k], c, -l2g[k >> 1][2 * (k & 1)]);
        t[2 * k + 1] = __builtin_fmaf(s_cur[2 * k + 1], c, -l2g[k >> 1][2 * (k & 1) + 1]);
        pin(t[2 * k]);
        pin(t[2 * k + 1]);
        if (k >= 1) finish_pair(k - 1);
      } else {
        e[2 * k] = __builtin_amdgcn_exp2f(t[2 * k]);
        e[2 * k + 1] = __builtin_amdgcn_exp2f(t[2 * k + 1]);
        pin(e[2 * k]);
        pin(e[2 * k + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    finish_pair(7);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One tile, its two steps on the fast or the general path, then the
  // barrier that publishes tile t+2 and the DMA of tile t+kStages-1 into the
  // stage of tile t-1.  Stage st holds tile t.
  auto tile = [&](int t, auto st_tag, auto fast_tag) __attribute__((always_inline)) {
    constexpr int st = decltype(st_tag)::value;
    constexpr int sp = (st + kStages - 1) % kStages, sn = (st + 1) % kStages;
    const char* lt = l2_base(stage(st), t);       // L2 of tile t
    const char* lt1 = l2_base(stage(sn), t + 1);  // L2 of tile t+1
    if constexpr (decltype(fast_tag)::value) {
      // step 2t: j+1 = (t, 1), j = (t, 0), j-1 = (t-1, 1), j+2 = (t+1, 0)
      step_fast(stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), lt, lt, sA, dpA, sB, dpB, pB, dsB, pA, dsA);
      // step 2t+1: j+1 = (t+1, 0), j = (t, 1), j-1 = (t, 0), j+2 = (t+1, 1)
      step_fast(stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), lt, lt1, sB, dpB, sA, dpA, pA, dsA, pB, dsB);
    } else {
      step_general(2 * t, stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), lt, sA, dpA, sB, dpB, pB, dsB,
                   pA, dsA);
      step_general(2 * t + 1, stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), lt1, sB, dpB, sA, dpA, pA,
                   dsA, pB, dsB);
    }
    vm_wait_barrier_tiles<Dma::kPerTile, kStages - 4>(
        max(0, min(min(t_end - 1, t + kStages - 2) - (t + 2), kStages - 4)));
    if (t + kStages - 1 < t_end) dma_issue(t + kStages - 1, stage(sp));
  };
  using kGeneral = std::false_type;
  using kFast = std::true_type;

  // ---- prologue: tiles t0 .. t0+kStages-2 in flight, t0 and t0+1 landed;
  // S and dP of the first half
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (t0 + i < t_end) dma_issue(t0 + i, stage(i));
  vm_wait_barrier_tiles<Dma::kPerTile, kStages - 3>(max(0, min(t_end - t0, kStages - 1) - 2));
  step_general(2 * t0 - 1, stage(0), 0, stage(kStages - 1), 1, stage(kStages - 1), 0, stage(0),
               l2_base(stage(0), t0), sB, dpB, sA, dpA, pA, dsA, pB, dsB);
  // ---- head, body (whole turns of the ring), tail
  Unroll<0, kHead>::run([&](auto i) {
    if (t0 + decltype(i)::value < t_end) tile(t0 + decltype(i)::value, i, kGeneral());
  });
  int t = t0 + kHead;
  for (; t + kStages - 1 < t_fast_end; t += kStages)
    Unroll<0, kStages>::run([&](auto i) {
      tile(t + decltype(i)::value, std::integral_constant<int, (kHead + decltype(i)::value) % kStages>(), kFast());
    });
  // the last, partial turn of fast tiles (short sequences), then the rest on
  // the general path from the same turn on (skipping what ran fast)
  if (t < t_fast_end)
    Unroll<0, kStages - 1>::run([&](auto i) {
      if (t + decltype(i)::value < t_fast_end)
        tile(t + decltype(i)::value, std::integral_constant<int, (kHead + decltype(i)::value) % kStages>(), kFast());
    });
  for (; t < t_end; t += kStages)
    Unroll<0, kStages>::run([&](auto i) {
      if (t + decltype(i)::value >= t_fast_end && t + decltype(i)::value < t_end)
        tile(t + decltype(i)::value, std::integral_constant<int, (kHead + decltype(i)::value) % kStages>(),
             kGeneral());
    });
  // dV, dK of the last half (every DMA has landed)
  if (jl >= jf) {
    const char* pb = half_stage(2 * t_end - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc_dv[i & 1] = mfma(tr_read(pb + kTileBytes, 1, i), pB[i >> 1], acc_dv[i & 1]);
      acc_dk[i & 1] = mfma(tr_read(pb, 1, i), dsB[i >> 1], acc_dk[i & 1]);
    }
  }

  // epilogue: lane = key, register 4*r4 + e = feature 32*db + 8*r4 + 4*hi + e.
  // The lane's key and its row addresses are formed again here from the lane
  // id (v_mbcnt) and uniform values, so nothing per-lane stays live across
  // the loop for them (the causal instance would spill it to scratch).
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int key_e = key0 + (lane_e & 31);
  const int hi_e = lane_e >> 5;
  if (key_e < n) {
    uint16_t* dkrow = a.dk + head_offset<kStrided>(a, kTdk, bh) + (size_t)key_e * row_stride<kStrided>(a, kTdk);
    uint16_t* dvrow = a.dv + head_offset<kStrided>(a, kTdv, bh) + (size_t)key_e * row_stride<kStrided>(a, kTdv);
    const float scale = a.scale;
    bool hidden = false;  // a key past the valid length or with a clear bit
    if constexpr (kKeys == kKeysLen || kKeys == kKeysBits) hidden = key_e >= valid_keys<kKeys>(a, bh);
    if constexpr (kKeys == kKeysBits) hidden = hidden || !((key_word(a, bh, key_e >> 5) >> (key_e & 31)) & 1u);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f0 = 32 * db + 8 * r4 + 4 * hi_e;
        unsigned k01 = pack_bf16(acc_dk[db][4 * r4] * scale, acc_dk[db][4 * r4 + 1] * scale);
        unsigned k23 = pack_bf16(acc_dk[db][4 * r4 + 2] * scale, acc_dk[db][4 * r4 + 3] * scale);
        unsigned v01 = pack_bf16(acc_dv[db][4 * r4], acc_dv[db][4 * r4 + 1]);
        unsigned v23 = pack_bf16(acc_dv[db][4 * r4 + 2], acc_dv[db][4 * r4 + 3]);
        if constexpr (kKeys == kKeysLen || kKeys == kKeysBits) {
          if (hidden) k01 = k23 = v01 = v23 = 0u;
        }
        *(u32x2*)(dkrow + f0) = u32x2{k01, k23};
        *(u32x2*)(dvrow + f0) = u32x2{v01, v23};
      }
  }
}

// ---------------------------------------------------------------------- dQ

// kKeys: with kKeysLen / kKeysBits only the keys below the batch entry's
// valid length are visited (the half holding the last one masked per
// element), and an entry with no valid key gets dQ = 0; with kKeysBits the
// keys whose bit is clear are dropped too (one mask word per 32-key half, a
// select per probability: on the pipelined path with the lane mask formed by
// scalar instructions from the word that came with the tile).  kKeysBlocks:
// the workgroup (one 128-query block) visits only the key tiles its row of
// the block mask sets, pipelined like the others (no mask is needed away
// from the causal diagonal and a ragged last tile, which are the last
// listed); the ring is one stage shorter so that two workgroups with their
// tile lists share a CU.
template <bool kCausal, int kWaves, int kKeys, bool kStrided = false>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdArgs a) {
  constexpr int kStages = kKeys == kKeysBlocks ? 4 : kWaves == 8 ? 6 : 5;
  constexpr int kRows = 32 * kWaves;  // queries per workgroup
  constexpr int kStageBytes = 2 * kTileBytes;
  using Dma = TileDma<kWaves, false, kStrided>;
  ATTN_BWD_RING(kStageBytes, kStages, stage);

  const int n = a.n;
  const int logical = xcd_remap(blockIdx.x, a.total);
  int bh, qb;
  if constexpr (kCausal) {
    int rank;  // the last query block of a head has the longest rows
    causal_order(logical, a.bh_count, a.blocks, bh, rank);
    qb = a.blocks - 1 - rank;
  } else {
    bh = logical / a.blocks;
    qb = logical - bh * a.blocks;
  }
  const uint16_t* qg = a.q + head_offset<kStrided>(a, kTq, bh);
  const uint16_t* kg = a.k + head_offset<kStrided>(a, kTk, bh);
  const uint16_t* vg = a.v + head_offset<kStrided>(a, kTv, bh);
  const uint16_t* dog = a.dout + head_offset<kStrided>(a, kTdo, bh);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int q0w = qb * kRows + wave_s * 32;  // this wave's first query
  const int qi = q0w + l32;                  // this lane's query (< n_pad)
  // keys that take part: all n, or the entry's valid length
  int n_k = n;
  if constexpr (kKeys == kKeysLen || kKeys == kKeysBits) {
    n_k = valid_keys<kKeys>(a, bh);
    if (n_k == 0) {  // uniform: before any barrier
      if (qi < n) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int f = 32 * hi; f < 32 * hi + 32; f += 8)
          *(u32x4*)(a.dq + head_offset<kStrided>(a, kTdq, bh) + (size_t)qi * row_stride<kStrided>(a, kTdq) + f) = z;
      }
      return;
    }
  }

  // Q^T and dO^T operands (B operands of S^T = K Q^T and dP^T = V dO^T)
  bf16x8 qop[4], dop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qop[ks] = row_operand(qg, qi, ks, hi, n, row_stride<kStrided>(a, kTq));
    dop[ks] = row_operand(dog, qi, ks, hi, n, row_stride<kStrided>(a, kTdo));
  }
  // L2 = LSE * log2(e) and -D = -sum_f dO_f O_f of this lane's query, formed
  // here from the 32 features of dO already in dop and the matching 32 of O
  // (lane l ^ 32 holds the other half of the row), and left in the
  // workspace for the dK/dV kernel, which runs after this one.  Queries past
  // N get L2 = +inf and -D = 0: their probabilities there are exactly 0.
  float* const hs = a.ws + (size_t)bh * 2 * a.n_pad;  // this head's L2, then -D
  float lse2 = INFINITY, ndl = 0.f;
  {
    const uint16_t* og = a.o + head_offset<kStrided>(a, kTo, bh);
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 ow = load_chunk(og, qi, 2 * ks + hi, n, row_stride<kStrided>(a, kTo));
      const u32x4 dw = __builtin_bit_cast(u32x4, dop[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = __builtin_fmaf(bf16_lo(ow[e]), bf16_lo(dw[e]), dsum);
        dsum = __builtin_fmaf(bf16_hi(ow[e]), bf16_hi(dw[e]), dsum);
      }
    }
    dsum = half_swap_sum(dsum);
    if (qi < n) {
      lse2 = a.lse[(size_t)bh * n + qi] * kLog2e;
      ndl = -dsum;
    }
    if (hi == 0) {
      hs[qi] = lse2;
      hs[a.n_pad + qi] = ndl;
    }
  }
  f32x16 nd16;  // -D of this lane's query in every register: dP^T starts there
#pragma unroll
  for (int r = 0; r < 16; ++r) nd16[r] = ndl;
  const TrOffsets tr(lane);
  int row_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) row_off[ks] = tile_off(l32, 2 * ks + hi);

  // 32-key halves this wave works on: [0, jl].  Causal: up to the half that
  // starts at the wave's first query (the diagonal).  The last half is
  // masked per element when it is the diagonal or holds keys past N (past
  // the valid length), and every half that holds a hidden key (kKeysBits).
  // (A wave whose queries all lie past N runs like the others: its L2 is
  // +inf, so its probabilities are 0, and no dQ row of it is written.)
  const int q_last = min(n - 1, qb * kRows + kRows - 1);
  const int kv_end = kCausal ? (kKeys != kKeysAll ? min(q_last + 1, n_k) : q_last + 1) : n_k;
  // kKeysBlocks: the key tiles below kv_end that this query block's row of
  // the block mask sets, compacted into blk_list (wave 0 writes, every wave
  // counts); from here on a tile index is a position in that list, and each
  // wave masks its general-path halves by their real key offsets.  Causal:
  // n_before counts the listed tiles that end before the workgroup's first
  // query (a prefix of the list), which no wave needs to mask.
  __shared__ uint16_t blk_list[kKeys == kKeysBlocks ? kMaxBlockTiles : 1];
  int n_listed = 0, n_before = 0;
  if constexpr (kKeys == kKeysBlocks) {
    static_assert(kRows == kBlockQ, "a workgroup is one query block of the block mask");
    const int kt_end = (kv_end + kBwdTile - 1) / kBwdTile;
    const uint8_t* mrow = a.block_mask + (size_t)qb * a.mask_cols;
    for (int base = 0; base < kt_end; base += 64) {
      const int kt = base + lane;
      const bool act = kt < kt_end && mrow[kt] != 0;
      const uint64_t bal = __ballot(act);
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
      if (wave == 0 && act) blk_list[n_listed + below] = (uint16_t)kt;
      n_listed += __popcll(bal);
      n_before += __popcll(__ballot(act && (kt + 1) * kBwdTile <= qb * kRows));
    }
    if constexpr (!kCausal) n_before = n_listed;
    __syncthreads();
  }
  auto tile_of = [&](int t) -> int {
    if constexpr (kKeys == kKeysBlocks) return __builtin_amdgcn_readfirstlane((int)blk_list[t]);
    else return t;
  };
  const int t_end = kKeys == kKeysBlocks ? n_listed : (kv_end + kBwdTile - 1) / kBwdTile;
  const int jl = kCausal && kKeys != kKeysBlocks ? min(q0w / 32, 2 * t_end - 1) : 2 * t_end - 1;
  // Tile 0 runs on the general path; then tiles whose two steps are fast in
  // every wave (2t+1 < the first wave's jl; kKeysBlocks: listed tiles that
  // need no mask, all but the last), in whole turns of the ring; the rest on
  // the general path again.
  constexpr int kHead = 1;
  const int jl_min = kCausal ? min(qb * kWaves, 2 * t_end - 1) : 2 * t_end - 1;
  const int t_fast_end = kKeys == kKeysBlocks ? max(0, min(n_before, t_end - 1))
                         : jl_min >= 2 ? (jl_min - 2) / 2 + 1 : 0;
  const Dma dma(kg, vg, n, wave, lane, nullptr, 0, row_stride<kStrided>(a, kTk), row_stride<kStrided>(a, kTv));
  auto dma_issue = [&](int t, char* sb) { dma.issue(tile_of(t), sb); };
  // kKeysBits: the two mask words of the tile in each stage (keys 64t ..
  // 64t+63), loaded beside its DMA by every wave in one 8-byte load (one
  // more load per tile in the waits' count, which must match exactly; words
  // past the entry's row read 0)
  uint32_t kw0[kStages], kw1[kStages];
  constexpr int kPerTile = Dma::kPerTile + (kKeys == kKeysBits ? 1 : 0);
  auto words_issue = [&](int t, auto st_tag) {
    if constexpr (kKeys == kKeysBits) {
      constexpr int st = decltype(st_tag)::value;
      const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.key_bits + (size_t)(bh / a.heads) * a.words), (short)0, a.words * 4, kBufferWord3);
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rw, 8 * t, 0, 0);
      kw0[st] = w[0];
      kw1[st] = w[1];
    } else {
      (void)t;
    }
  };

  auto fast = [&](int j) {
    if constexpr (kKeys == kKeysBlocks) return j >= 1 && j < 2 * t_fast_end;
    else return j >= 1 && j <= jl - 1;
  };
  auto half_stage = [&](int j) { return stage((j / 2) % kStages); };
  auto k_row = [&](const char* sb, int h, int ks) { return lds_read_b128(sb, h * 32 * kRow + row_off[ks]); };
  auto v_row = [&](const char* sb, int h, int ks) {
    return lds_read_b128(sb + kTileBytes, h * 32 * kRow + row_off[ks]);
  };
  auto k_tr = [&](const char* sb, int h, int i) {  // i = 2*tt + db
    const char* b = sb + (32 * h + 16 * (i >> 1)) * kRow;
    return lds_read_vt(b + tr.off[0][i & 1], b + tr.off[1][i & 1]);
  };
  // A operand of MFMA slot s (0..11) of a fast step: in group g = s/3,
  // S(j+1) step g, dQ(j-1) step g, dP(j+1) step g
  auto slot_operand = [&](int s, const char* nb, int hn, const char* pb, int hp) {
    const int g = s / 3;
    switch (s % 3) {
      case 0: return k_row(nb, hn, g);
      case 1: return k_tr(pb, hp, g);
      default: return v_row(nb, hn, g);
    }
  };

  f32x16 acc[2];  // dQ^T: rows = features, columns = queries
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const f32x16 zero16 = {};
  const float c = a.c;

  // S^T and dP^T - D of a half (lane = query, register r = key
  // 8*(r/4) + 4*hi + r%4 of the half), its bf16 dS^T as MFMA B operand, and
  // the A operands of the next four MFMA slots
  f32x16 sA = zero16, sB = zero16, dpA = zero16, dpB = zero16;
  bf16x8 dsA[2], dsB[2];
  bf16x8 ring[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) dsA[i] = dsB[i] = bf16x8{};
#pragma unroll
  for (int i = 0; i < 4; ++i) ring[i] = bf16x8{};

  // Step j on the general path (see the dK/dV kernel), with the diagonal
  // and ragged-key masks.
  auto step_general = [&](int j, const char* nb, int hn, const char* cb, int hc, const char* pb, int hp,
                          const char* nnb, f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt,
                          const bf16x8 (&ds_prv)[2], bf16x8 (&ds_cur)[2]) __attribute__((always_inline)) {
    if (j + 1 >= 0 && j + 1 <= jl) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s_nxt = mfma(k_row(nb, hn, ks), qop[ks], ks == 0 ? zero16 : s_nxt);
        dp_nxt = mfma(v_row(nb, hn, ks), dop[ks], ks == 0 ? nd16 : dp_nxt);
        __builtin_amdgcn_sched_barrier(0);  // one operand pair in flight at a time
      }
    }
    if (j - 1 >= 0 && j - 1 <= jl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i & 1] = mfma(k_tr(pb, hp, i), ds_prv[i >> 1], acc[i & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (j >= 0 && j <= jl) {
      const int k0 = 32 * (kKeys == kKeysBlocks ? 2 * tile_of(j >> 1) + (j & 1) : j);  // the half's first key
      const bool diag = kCausal && k0 == q0w;
      const bool ragged = k0 + 32 > n_k;
      const bool none = kKeys == kKeysBlocks && kCausal && k0 > q0w;  // every key after the wave's queries
      uint32_t kept = ~0u;  // kKeysBits: bit kr set = key k0 + kr takes part
      if constexpr (kKeys == kKeysBits) kept = k0 < n ? key_word(a, bh, j) >> (4 * hi) : 0u;  // words: keys < n
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], c, -lse2));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r + 1], c, -lse2));
        if (diag || ragged) {
          const int kr = 8 * (r >> 2) + 4 * hi + (r & 3);  // key - k0
          if ((diag && kr > l32) || k0 + kr >= n_k) p0 = 0.f;
          if ((diag && kr + 1 > l32) || k0 + kr + 1 >= n_k) p1 = 0.f;
        }
        if constexpr (kKeys == kKeysBits) {
          const int kb0 = 8 * (r >> 2) + (r & 3);  // key - k0 - 4 * hi
          if (!((kept >> kb0) & 1u)) p0 = 0.f;
          if (!((kept >> (kb0 + 1)) & 1u)) p1 = 0.f;
        }
        if constexpr (kKeys == kKeysBlocks) {
          if (none) p0 = p1 = 0.f;
        }
        set_word(ds_cur[r >> 3], (r & 7) >> 1, pack_bf16(p0 * dp_cur[r], p1 * dp_cur[r + 1]));
      }
    }
    if (fast(j + 1)) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ring[s] = slot_operand(s, nnb, hc, cb, hc);
    }
  };

  // Step j on the fast path (arguments as in the dK/dV kernel; kw: half j's
  // mask word, kKeysBits).  12 MFMA slots; in group g: S(j+1) step g, dQ(j-1)
  // step g, dP(j+1) step g.  Vector work on score pair k: FMA in slot a_k,
  // exp2 in a_k + 1, (mask,) product and pack in a_k + 2, with a_k = 0, 1,
  // 3, 4, 6, 7, 9, 10.
  auto step_fast = [&](const char* nb, int hn, const char* cb, int hc, const char* pb, int hp, const char* nnb,
                       f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt, const bf16x8 (&ds_prv)[2],
                       bf16x8 (&ds_cur)[2], uint32_t kw) __attribute__((always_inline)) {
    (void)kw;
    float t[16], e[16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s <= 12; ++s) {
      if (s < 12) {
        const int g = s / 3;
        switch (s % 3) {
          case 0: s_nxt = mfma(ring[s & 3], qop[g], g == 0 ? zero16 : s_nxt); break;
          case 1: acc[g & 1] = mfma(ring[s & 3], ds_prv[g >> 1], acc[g & 1]); break;
          default: dp_nxt = mfma(ring[s & 3], dop[g], g == 0 ? nd16 : dp_nxt); break;
        }
        if (s + 4 < 12) ring[s & 3] = slot_operand(s + 4, nb, hn, pb, hp);
        else ring[s & 3] = slot_operand(s - 8, nnb, hc, cb, hc);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 2 * k, a_k = k + (k >> 1);
        if (a_k + 2 == s) {
          if constexpr (kKeys == kKeysBits) {  // keys k0 + 8*(r/4) + 4*hi + r%4 (+1)
            e[r] = keep_bit(e[r], kw, 8 * (r >> 2) + (r & 3));
            e[r + 1] = keep_bit(e[r + 1], kw, 8 * (r >> 2) + (r & 3) + 1);
          }
          unsigned dw = pack_bf16(e[r] * dp_cur[r], e[r + 1] * dp_cur[r + 1]);
          pin(dw);
          set_word(ds_cur[r >> 3], (r & 7) >> 1, dw);
        }
        if (a_k + 1 == s) {
          e[r] = __builtin_amdgcn_exp2f(t[r]);
          e[r + 1] = __builtin_amdgcn_exp2f(t[r + 1]);
          pin(e[r]);
          pin(e[r + 1]);
        }
        if (a_k == s) {
          t[r] = __builtin_fmaf(s_cur[r], c, -lse2);
          t[r + 1] = __builtin_fmaf(s_cur[r + 1], c, -lse2);
          pin(t[r]);
          pin(t[r + 1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto tile = [&](int t, auto st_tag, auto fast_tag) __attribute__((always_inline)) {
    constexpr int st = decltype(st_tag)::value;
    constexpr int sp = (st + kStages - 1) % kStages, sn = (st + 1) % kStages;
    if constexpr (decltype(fast_tag)::value) {
      uint32_t w0 = 0, w1 = 0;  // the mask words of halves 2t, 2t+1
      if constexpr (kKeys == kKeysBits) {
        w0 = __builtin_amdgcn_readfirstlane(kw0[st]);
        w1 = __builtin_amdgcn_readfirstlane(kw1[st]);
      }
      step_fast(stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), sA, dpA, sB, dpB, dsB, dsA, w0);
      step_fast(stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), sB, dpB, sA, dpA, dsA, dsB, w1);
    } else {
      step_general(2 * t, stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), sA, dpA, sB, dpB, dsB, dsA);
      step_general(2 * t + 1, stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), sB, dpB, sA, dpA, dsA, dsB);
    }
    vm_wait_barrier_tiles<kPerTile, kStages - 4>(
        max(0, min(min(t_end - 1, t + kStages - 2) - (t + 2), kStages - 4)));
    if (t + kStages - 1 < t_end) {
      dma_issue(t + kStages - 1, stage(sp));
      words_issue(t + kStages - 1, std::integral_constant<int, sp>());
    }
  };
  using kGeneral = std::false_type;
  using kFast = std::true_type;

  // ---- prologue
  if constexpr (kKeys == kKeysBits) {
    Unroll<0, kStages - 1>::run([&](auto i) {
      if (decltype(i)::value < t_end) {
        dma_issue(decltype(i)::value, stage(decltype(i)::value));
        words_issue(decltype(i)::value, i);
      }
    });
  } else {
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
      if (i < t_end) dma_issue(i, stage(i));
  }
  vm_wait_barrier_tiles<kPerTile, kStages - 3>(max(0, min(t_end, kStages - 1) - 2));
  step_general(-1, stage(0), 0, stage(kStages - 1), 1, stage(kStages - 1), 0, stage(0), sB, dpB, sA, dpA, dsA,
               dsB);
  // ---- head, body (whole turns of the ring), tail
  Unroll<0, kHead>::run([&](auto i) {
    if (decltype(i)::value < t_end) tile(decltype(i)::value, i, kGeneral());
  });
  int t = kHead;
  for (; t + kStages - 1 < t_fast_end; t += kStages)
    Unroll<0, kStages>::run([&](auto i) {
      tile(t + decltype(i)::value, std::integral_constant<int, (kHead + decltype(i)::value) % kStages>(), kFast());
    });
  if (t < t_fast_end)
    Unroll<0, kStages - 1>::run([&](auto i) {
      if (t + decltype(i)::value < t_fast_end)
        tile(t + decltype(i)::value, std::integral_constant<int, (kHead + decltype(i)::value) % kStages>(), kFast());
    });
  for (; t < t_end; t += kStages)
    Unroll<0, kStages>::run([&](auto i) {
      if (t + decltype(i)::value >= t_fast_end && t + decltype(i)::value < t_end)
        tile(t + decltype(i)::value, std::integral_constant<int, (kHead + decltype(i)::value) % kStages>(),
             kGeneral());
    });
  // dQ of the last half (every DMA has landed)
  if ((kKeys != kKeysBlocks || t_end > 0) && 2 * t_end - 1 <= jl) {  // (an empty block list has no last half)
    const char* pb = half_stage(2 * t_end - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i & 1] = mfma(k_tr(pb, 1, i), dsB[i >> 1], acc[i & 1]);
  }

  if (qi < n) {
    uint16_t* row = a.dq + head_offset<kStrided>(a, kTdq, bh) + (size_t)qi * row_stride<kStrided>(a, kTdq);
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f0 = 32 * db + 8 * r4 + 4 * hi;
        const unsigned p01 = pack_bf16(acc[db][4 * r4] * scale, acc[db][4 * r4 + 1] * scale);
        const unsigned p23 = pack_bf16(acc[db][4 * r4 + 2] * scale, acc[db][4 * r4 + 3] * scale);
        *(u32x2*)(row + f0) = u32x2{p01, p23};
      }
  }
}

// Waves per workgroup (32 rows each; build parameters ATTN_BWD_DKDV_WAVES,
// ATTN_BWD_DQ_WAVES and, with the causal mask, ATTN_BWD_CAUSAL_WAVES; 4 or
// 8).  Measured on one MI355X: 4 everywhere is as fast as 8 at N = 11,616
// (within 1%), 3-5% faster at N = 512 and 38,400, and 25% faster causal at
// N = 1,024 (a shorter row block balances the triangle).
#ifndef ATTN_BWD_DKDV_WAVES
#define ATTN_BWD_DKDV_WAVES 4
#endif
#ifndef ATTN_BWD_DQ_WAVES
#define ATTN_BWD_DQ_WAVES 4
#endif
#ifndef ATTN_BWD_CAUSAL_WAVES
#define ATTN_BWD_CAUSAL_WAVES 4
#endif
constexpr int kWavesDkdv = ATTN_BWD_DKDV_WAVES;
constexpr int kWavesDq = ATTN_BWD_DQ_WAVES;
constexpr int kWavesCausal = ATTN_BWD_CAUSAL_WAVES;
static_assert((kWavesDkdv == 4 || kWavesDkdv == 8) && (kWavesDq == 4 || kWavesDq == 8) &&
                  (kWavesCausal == 4 || kWavesCausal == 8),
              "4 or 8 waves per workgroup");

// One launch of a main kernel with kWaves waves per workgroup.
template <int kWaves>
hipError_t launch_main(const void* kernel, const BwdArgs& base, int B, int H, int N, hipStream_t s) {
  BwdArgs a = base;
  a.blocks = (N + 32 * kWaves - 1) / (32 * kWaves);
  a.total = B * H * a.blocks;
  void* args[] = {&a};
  return hipLaunchKernel(kernel, dim3(a.total), dim3(kWaves * 64), args, 0, s);
}

}  // namespace

extern "C" size_t attn_bwd_workspace_size(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  const long long n_pad = ((long long)N + kPadRows - 1) / kPadRows * kPadRows;
  return (size_t)(2LL * B * H * n_pad * (long long)sizeof(float));
}

namespace {

// Checks and launches shared by attn_bwd and attn_bwd_noalloc; ws is the
// workspace of attn_bwd_workspace_size(B, H, N) bytes (already checked).
attn_status bwd_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                         float scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_E_INVALID;
  if (B < 1 || H < 1 || N < 1 || d != kD || !std::isfinite(scale)) return ATTN_E_INVALID;
  if (!sizes_fit(B, H, N)) return ATTN_E_INVALID;
  const void* vec[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : vec)
    if (misaligned(p, 16)) return ATTN_E_ALIGN;
  if (misaligned(lse, 4)) return ATTN_E_ALIGN;
  return ATTN_OK;
}

// Element strides (batch, head, row) of the eight tensors q, k, v, o, dout,
// dq, dk, dv (NULL layout: the contiguous [B][H][N][64] one), checked: every
// stride a multiple of 8 elements (16 bytes: the kernels move 16-byte
// chunks), none negative, a row stride of at most 2^24, the outputs' rows
// at least 64 apart, and every byte offset the buffer loads of a tile form
// (q and dout in the dK/dV kernel, k and v in the dQ kernel) below 2^31.
// Sets *strided when some layout is given.
attn_status bwd_layouts(const attn_layout* const lay[8], int H, int N, BwdArgs& a, bool* strided) {
  *strided = false;
  for (int t = 0; t < 8; ++t) {
    if (!lay[t]) {
      a.sn[t] = kD;
      a.sh[t] = (long long)N * kD;
      a.sb[t] = (long long)H * N * kD;
      continue;
    }
    *strided = true;
    const attn_layout& l = *lay[t];
    if (l.batch < 0 || l.head < 0 || l.row < 0) return ATTN_E_INVALID;
    if ((l.batch | l.head | l.row) & 7) return ATTN_E_ALIGN;
    if (l.row > (1LL << 24)) return ATTN_E_INVALID;
    a.sb[t] = l.batch;
    a.sh[t] = l.head;
    a.sn[t] = (int)l.row;
  }
  for (int t = kTdq; t <= kTdv; ++t)
    if (a.sn[t] < kD) return ATTN_E_INVALID;  // an output's rows must not overlap
  const int dma[4] = {kTq, kTdo, kTk, kTv};
  for (int t : dma)
    if ((long long)(N - 1) * 2 * a.sn[t] + kRow >= (1LL << 31)) return ATTN_E_INVALID;
  return ATTN_OK;
}

attn_status bwd_launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int H, int N,
                       float scale, int causal, const int* key_len, const uint32_t* key_bits,
                       const uint8_t* block_mask, void* stream, const BwdArgs* strides = nullptr) {
  BwdArgs a;
  if (strides) {
    for (int t = 0; t < 8; ++t) {
      a.sb[t] = strides->sb[t];
      a.sh[t] = strides->sh[t];
      a.sn[t] = strides->sn[t];
    }
  } else {
    for (int t = 0; t < 8; ++t) a.sb[t] = a.sh[t] = a.sn[t] = 0;
  }
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.ws = ws;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.n = N;
  a.n_pad = (N + kPadRows - 1) / kPadRows * kPadRows;
  a.bh_count = B * H;
  a.heads = H;
  a.key_len = key_len;
  a.key_bits = key_bits;
  a.words = (N + 31) / 32;
  a.block_mask = block_mask;
  a.mask_cols = (N + kBlockK - 1) / kBlockK;
  a.blocks = a.total = 0;
  a.c = scale * kLog2e;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // The dQ kernel runs first: it writes every workspace entry the dK/dV
  // kernel reads (L2 and -D of each query row up to its row blocks' end,
  // padding rows +inf and 0), so nothing has to start at zero.
  hipError_t e;
  if (block_mask) {  // 4-wave workgroups: one 128-query block (dQ), two 64-key columns (dK/dV)
    const void* k_dq = causal ? reinterpret_cast<const void*>(&bwd_dq_kernel<true, 4, kKeysBlocks>)
                              : reinterpret_cast<const void*>(&bwd_dq_kernel<false, 4, kKeysBlocks>);
    const void* k_dkdv = causal ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, 4, kKeysBlocks>)
                                : reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, 4, kKeysBlocks>);
    e = launch_main<4>(k_dq, a, B, H, N, s);
    if (e == hipSuccess) e = launch_main<4>(k_dkdv, a, B, H, N, s);
    return launch_status(e);
  }
  const int keys = key_bits ? kKeysBits : key_len ? kKeysLen : kKeysAll;
  if (strides) {  // strided tensors: 4-wave workgroups
    const void* k_dq;
    const void* k_dkdv;
    if (causal) {
      const void* const t_dq[3] = {reinterpret_cast<const void*>(&bwd_dq_kernel<true, 4, kKeysAll, true>),
                                   reinterpret_cast<const void*>(&bwd_dq_kernel<true, 4, kKeysLen, true>),
                                   reinterpret_cast<const void*>(&bwd_dq_kernel<true, 4, kKeysBits, true>)};
      const void* const t_dkdv[3] = {reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, 4, kKeysAll, true>),
                                     reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, 4, kKeysLen, true>),
                                     reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, 4, kKeysBits, true>)};
      k_dq = t_dq[keys];
      k_dkdv = t_dkdv[keys];
    } else {
      const void* const t_dq[3] = {reinterpret_cast<const void*>(&bwd_dq_kernel<false, 4, kKeysAll, true>),
                                   reinterpret_cast<const void*>(&bwd_dq_kernel<false, 4, kKeysLen, true>),
                                   reinterpret_cast<const void*>(&bwd_dq_kernel<false, 4, kKeysBits, true>)};
      const void* const t_dkdv[3] = {reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, 4, kKeysAll, true>),
                                     reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, 4, kKeysLen, true>),
                                     reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, 4, kKeysBits, true>)};
      k_dq = t_dq[keys];
      k_dkdv = t_dkdv[keys];
    }
    e = launch_main<4>(k_dq, a, B, H, N, s);
    if (e == hipSuccess) e = launch_main<4>(k_dkdv, a, B, H, N, s);
    return launch_status(e);
  }
  if (causal) {
    const void* const k_dq[3] = {reinterpret_cast<const void*>(&bwd_dq_kernel<true, kWavesCausal, kKeysAll>),
                                 reinterpret_cast<const void*>(&bwd_dq_kernel<true, kWavesCausal, kKeysLen>),
                                 reinterpret_cast<const void*>(&bwd_dq_kernel<true, kWavesCausal, kKeysBits>)};
    const void* const k_dkdv[3] = {reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, kWavesCausal, kKeysAll>),
                                   reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, kWavesCausal, kKeysLen>),
                                   reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, kWavesCausal, kKeysBits>)};
    e = launch_main<kWavesCausal>(k_dq[keys], a, B, H, N, s);
    if (e == hipSuccess) e = launch_main<kWavesCausal>(k_dkdv[keys], a, B, H, N, s);
  } else {
    const void* const k_dq[3] = {reinterpret_cast<const void*>(&bwd_dq_kernel<false, kWavesDq, kKeysAll>),
                                 reinterpret_cast<const void*>(&bwd_dq_kernel<false, kWavesDq, kKeysLen>),
                                 reinterpret_cast<const void*>(&bwd_dq_kernel<false, kWavesDq, kKeysBits>)};
    const void* const k_dkdv[3] = {reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, kWavesDkdv, kKeysAll>),
                                   reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, kWavesDkdv, kKeysLen>),
                                   reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, kWavesDkdv, kKeysBits>)};
    e = launch_main<kWavesDq>(k_dq[keys], a, B, H, N, s);
    if (e == hipSuccess) e = launch_main<kWavesDkdv>(k_dkdv[keys], a, B, H, N, s);
  }
  return launch_status(e);
}

// The workspace of attn_bwd_noalloc: a static device array, one copy per
// device, alive until the process ends.  Host code never uses its name as an
// address (that is a host-side stand-in); it asks the runtime once per device
// for the array's device address and passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_BWD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device; null = not looked up

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current).
attn_status scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return ATTN_E_DEVICE;
  }
  void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return ATTN_E_DEVICE;
    }
    __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
  }
  *out = static_cast<float*>(p);
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H,
                                int N, int d, float scale, int causal, void* stream) {
  if (!workspace) return ATTN_E_INVALID;
  attn_status st = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if (misaligned(workspace, 16)) return ATTN_E_ALIGN;
  st = check_device();
  if (st != ATTN_OK) return st;
  return bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H, N, scale, causal,
                    nullptr, nullptr, nullptr, stream);
}

extern "C" attn_status attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                       const void* dout, void* dq, void* dk, void* dv, void* workspace, int B,
                                       int H, int N, int d, float scale, int causal, const int* key_len,
                                       const unsigned* key_bits, void* stream) {
  if (!workspace) return ATTN_E_INVALID;
  attn_status st = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if (misaligned(workspace, 16) || misaligned(key_len, 4) || misaligned(key_bits, 4)) return ATTN_E_ALIGN;
  st = check_device();
  if (st != ATTN_OK) return st;
  return bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H, N, scale, causal,
                    key_len, key_bits, nullptr, stream);
}

extern "C" attn_status attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                        const void* dout, void* dq, void* dk, void* dv, void* workspace, int B,
                                        int H, int N, int d, float scale, int causal, const attn_layout* q_layout,
                                        const attn_layout* k_layout, const attn_layout* v_layout,
                                        const attn_layout* o_layout, const attn_layout* dout_layout,
                                        const attn_layout* dq_layout, const attn_layout* dk_layout,
                                        const attn_layout* dv_layout, const int* key_len, const unsigned* key_bits,
                                        void* stream) {
  if (!workspace) return ATTN_E_INVALID;
  attn_status st = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  BwdArgs lay;
  bool strided = false;
  const attn_layout* const layouts[8] = {q_layout, k_layout, v_layout, o_layout,
                                         dout_layout, dq_layout, dk_layout, dv_layout};
  st = bwd_layouts(layouts, H, N, lay, &strided);
  if (st != ATTN_OK) return st;
  if (misaligned(workspace, 16) || misaligned(key_len, 4) || misaligned(key_bits, 4)) return ATTN_E_ALIGN;
  st = check_device();
  if (st != ATTN_OK) return st;
  return bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H, N, scale, causal,
                    key_len, key_bits, nullptr, stream, strided ? &lay : nullptr);
}

extern "C" attn_status attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                             void* workspace, int B, int H, int N, int d, float scale, int causal,
                                             const unsigned char* block_mask, void* stream) {
  if (!workspace || !block_mask) return ATTN_E_INVALID;
  attn_status st = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if (N > kBlockK * kMaxBlockTiles) return ATTN_E_INVALID;
  if (misaligned(workspace, 16)) return ATTN_E_ALIGN;
  st = check_device();
  if (st != ATTN_OK) return st;
  return bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H, N, scale, causal,
                    nullptr, nullptr, block_mask, stream);
}

extern "C" attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                                        int H, int N, int d, float scale, int causal, void* stream) {
  attn_status st = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if (attn_bwd_workspace_size(B, H, N) > (size_t)ATTN_BWD_NOALLOC_SCRATCH_BYTES) return ATTN_E_SCRATCH;
  st = check_device();
  if (st != ATTN_OK) return st;
  float* ws = nullptr;
  st = scratch_address(&ws);
  if (st != ATTN_OK) return st;
  return bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, scale, causal, nullptr, nullptr, nullptr,
                    stream);
}
