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
// Three kernels on the caller's stream:
//   1. bwd_prep: per row, L2 = LSE * log2(e) and -D = -sum_f dO_if O_if into
//      the caller's workspace (rows padded to a multiple of 256 with
//      L2 = +inf and -D = 0, so a padding row has probability exactly 0);
//   2. bwd_dkdv (key-parallel): each wave keeps K and V of its 32 keys in
//      registers as MFMA operands; 64-query tiles of Q, dO, L2 and -D stream
//      through an LDS ring filled by DMA.  S = Q K^T is computed in the layout
//      where each lane holds one key and 16 queries: P and dS then feed
//      dV^T += dO^T P and dK^T += Q^T dS directly as MFMA operands, and the
//      transposed Q / dO operands come from the row-major tiles with
//      ds_read_b64_tr_b16;
//   3. bwd_dq (query-parallel): each wave keeps Q and dO of its 32 queries
//      in registers and streams 64-key tiles of K and V: S^T = K Q^T and
//      dP^T = V dO^T (a lane per query), dS^T, then dQ^T += K^T dS^T.
// Both main kernels run a software pipeline over 32-row steps: step j
// issues the MFMAs of S and dP for step j+1 and of the accumulating products
// of step j-1, one by one, each beside a slice of the vector work of step j
// (exp2, dS, bf16 packing), and reads its MFMA operands from LDS four MFMAs
// ahead.  -D enters dP as the initial value of its accumulator.  Causal
// calls run each XCD's block of heads longest row block first (causal_order).
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
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Per row of every head: L2 = LSE * log2(e) and -D = -sum_f dO_f O_f; rows
// of the padding get L2 = +inf and -D = 0.
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdArgs a, long long rows) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int bh = (int)(r / a.n_pad);
  const int row = (int)(r - (long long)bh * a.n_pad);
  float l2 = INFINITY, nd = 0.f;
  if (row < a.n) {
    const size_t g = (size_t)bh * a.n + row;
    const u32x4* po = (const u32x4*)(a.o + g * kD);
    const u32x4* pd = (const u32x4*)(a.dout + g * kD);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 wo = po[i], wd = pd[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(bf16_lo(wo[e]), bf16_lo(wd[e]), acc);
        acc = __builtin_fmaf(bf16_hi(wo[e]), bf16_hi(wd[e]), acc);
      }
    }
    l2 = a.lse[g] * kLog2e;
    nd = -acc;
  }
  float* const hs = a.ws + (size_t)bh * 2 * a.n_pad;  // this head's L2, then -D
  hs[row] = l2;
  hs[a.n_pad + row] = nd;
}

// 16-byte chunk `ch` of row `row` of a [n][64] bf16 matrix, zero past row n.
__device__ __forceinline__ u32x4 load_chunk(const uint16_t* base, int row, int ch, int n) {
  u32x4 w = {0u, 0u, 0u, 0u};
  if (row < n) w = *(const u32x4*)(base + (size_t)row * kD + 8 * ch);
  return w;
}

// The 8 bf16 of features 16*ks + 8*hi .. +7 of one row, as an MFMA operand.
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* base, int row, int ks, int hi, int n) {
  return __builtin_bit_cast(bf16x8, load_chunk(base, row, 2 * ks + hi, n));
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
template <int kWaves, bool kStats>
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

  // stats: this head's L2[n_pad], then -D[n_pad] (dK/dV only)
  __device__ TileDma(const uint16_t* m0, const uint16_t* m1, int n_, int wave, int lane_, const float* stats,
                     int n_pad)
      : g0(m0), g1(m1), n(n_), lane(lane_) {
    row_in = 8 * wave + (lane >> 3);
    chunk = (lane & 7) ^ swz(row_in);
    lane_off = row_in * kRow + chunk * 16;
    wave_s = __builtin_amdgcn_readfirstlane(wave);
    r0 = __builtin_amdgcn_make_buffer_rsrc((void*)m0, (short)0, n * kRow, kBufferWord3);
    r1 = __builtin_amdgcn_make_buffer_rsrc((void*)m1, (short)0, n * kRow, kBufferWord3);
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
        const int soff = (t * kBwdTile + ps * kPassRows) * kRow;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, (lds_void*)(d + ps * kPassRows * kRow), 16, lane_off, soff,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_void*)(d + kTileBytes + ps * kPassRows * kRow), 16,
                                                 lane_off, soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const int row = min(t * kBwdTile + row_in + ps * kPassRows, n - 1);
        __builtin_amdgcn_global_load_lds((global_void*)(g0 + (size_t)row * kD + chunk * 8),
                                         (lds_void*)(d + ps * kPassRows * kRow), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((global_void*)(g1 + (size_t)row * kD + chunk * 8),
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

template <bool kCausal, int kWaves>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kStages = kWaves == 8 ? 5 : 4;
  constexpr int kRows = 32 * kWaves;        // keys per workgroup
  constexpr int kStatOff = 2 * kTileBytes;  // L2[64], then -D[64]
  constexpr int kStageBytes = kStatOff + 2 * kBwdTile * 4;
  using Dma = TileDma<kWaves, true>;
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
  const size_t head = (size_t)bh * n * kD;
  const uint16_t* qg = a.q + head;
  const uint16_t* kg = a.k + head;
  const uint16_t* vg = a.v + head;
  const uint16_t* dog = a.dout + head;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int key0 = kb * kRows + wave_s * 32;  // this wave's first key
  const int key = key0 + l32;                 // this lane's key

  // K^T and V^T operands (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kop[4], vop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kop[ks] = row_operand(kg, key, ks, hi, n);
    vop[ks] = row_operand(vg, key, ks, hi, n);
  }
  const TrOffsets tr(lane);
  int row_off[4];  // row-operand read of step ks: row l32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) row_off[ks] = tile_off(l32, 2 * ks + hi);

  // 64-query tiles of the workgroup
  const int t0 = kCausal ? (kb * kRows) / kBwdTile : 0;
  const int t_end = (n + kBwdTile - 1) / kBwdTile;
  // 32-query halves this wave works on: [jf, jl], every half of the tiles.
  // Causal: from the half that starts at the wave's first key (the
  // diagonal, masked per element).  Queries past N have L2 = +inf, so their
  // probabilities are exactly 0.  (A wave whose keys all lie past N runs
  // like the others; nothing of it is written.)
  const int jl = 2 * t_end - 1;
  const int jf = kCausal ? key0 / 32 : 0;
  // Tiles t0 .. t0+kHead-1 run on the general path; then tiles whose two
  // steps are fast in every wave (2t > the last wave's first half, 2t+1 <
  // jl) run pipelined, in whole turns of the ring and a last partial one;
  // the rest on the general path again.
  constexpr int kHead = kCausal ? (kWaves + 1) / 2 : 1;
  const int t_fast_end = jl >= 2 ? (jl - 2) / 2 + 1 : 0;
  const Dma dma(qg, dog, n, wave, lane, a.ws + (size_t)bh * 2 * a.n_pad, a.n_pad);

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
  // L2 of registers 4*g4 .. 4*g4+3 (queries 8*g4 + 4*hi + 0..3 of the half)
  auto l2_group = [&](const char* sb, int h, int g4) -> f32x4 {
    return *(const f32x4*)(sb + kStatOff + 16 * (8 * h + 2 * g4 + hi));
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
                          const char* nnb, f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt,
                          const bf16x8 (&p_prv)[2], const bf16x8 (&ds_prv)[2], bf16x8 (&p_cur)[2],
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
      const bool diag = kCausal && j == jf;  // key > query hidden
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 l4 = l2_group(cb, hc, g4);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const int r = 4 * g4 + e;
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], c, -l4[e]));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r + 1], c, -l4[e + 1]));
          if (diag && l32 > 8 * g4 + 4 * hi + e) p0 = 0.f;
          if (diag && l32 > 8 * g4 + 4 * hi + e + 1) p1 = 0.f;
          set_word(p_cur[r >> 3], (r & 7) >> 1, pack_bf16(p0, p1));
          set_word(ds_cur[r >> 3], (r & 7) >> 1, pack_bf16(p0 * dp_cur[r], p1 * dp_cur[r + 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (fast(j + 1)) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ring[s] = slot_operand(s, nnb, hc, cb, hc);
      l2n = l2_group(nb, hn, 0);
    }
  };

  // Step j on the fast path.  nb/hn: half j+1; cb/hc: half j; pb/hp: half
  // j-1; nnb: half j+2 (half index hc).  16 MFMA slots; in group g: S(j+1)
  // step g, dV(j-1) step g, dK(j-1) step g, dP(j+1) step g (its accumulator
  // starts at -D).  Vector work on score pair k: FMA in slot 2k, exp2 in slot
  // 2k+1, products and packs in slot 2k+2.
  auto step_fast = [&](const char* nb, int hn, const char* cb, int hc, const char* pb, int hp, const char* nnb,
                       f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt, const bf16x8 (&p_prv)[2],
                       const bf16x8 (&ds_prv)[2], bf16x8 (&p_cur)[2], bf16x8 (&ds_cur)[2]) __attribute__((always_inline)) {
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
      if (s == 1 || s == 5 || s == 9) l2g[(s + 3) >> 2] = l2_group(cb, hc, (s + 3) >> 2);
      if (s == 13) l2n = l2_group(nb, hn, 0);
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
    if constexpr (decltype(fast_tag)::value) {
      // step 2t: j+1 = (t, 1), j = (t, 0), j-1 = (t-1, 1), j+2 = (t+1, 0)
      step_fast(stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), sA, dpA, sB, dpB, pB, dsB, pA, dsA);
      // step 2t+1: j+1 = (t+1, 0), j = (t, 1), j-1 = (t, 0), j+2 = (t+1, 1)
      step_fast(stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), sB, dpB, sA, dpA, pA, dsA, pB, dsB);
    } else {
      step_general(2 * t, stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), sA, dpA, sB, dpB, pB, dsB, pA,
                   dsA);
      step_general(2 * t + 1, stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), sB, dpB, sA, dpA, pA, dsA,
                   pB, dsB);
    }
    vm_wait_barrier_tiles<Dma::kPerTile, kStages - 4>(
        max(0, min(min(t_end - 1, t + kStages - 2) - (t + 2), kStages - 4)));
    if (t + kStages - 1 < t_end) dma.issue(t + kStages - 1, stage(sp));
  };
  using kGeneral = std::false_type;
  using kFast = std::true_type;

  // ---- prologue: tiles t0 .. t0+kStages-2 in flight, t0 and t0+1 landed;
  // S and dP of the first half
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (t0 + i < t_end) dma.issue(t0 + i, stage(i));
  vm_wait_barrier_tiles<Dma::kPerTile, kStages - 3>(max(0, min(t_end - t0, kStages - 1) - 2));
  step_general(2 * t0 - 1, stage(0), 0, stage(kStages - 1), 1, stage(kStages - 1), 0, stage(0), sB, dpB, sA, dpA,
               pA, dsA, pB, dsB);
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

  // epilogue: lane = key, register 4*r4 + e = feature 32*db + 8*r4 + 4*hi + e
  if (key < n) {
    uint16_t* dkrow = a.dk + head + (size_t)key * kD;
    uint16_t* dvrow = a.dv + head + (size_t)key * kD;
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f0 = 32 * db + 8 * r4 + 4 * hi;
        const unsigned k01 = pack_bf16(acc_dk[db][4 * r4] * scale, acc_dk[db][4 * r4 + 1] * scale);
        const unsigned k23 = pack_bf16(acc_dk[db][4 * r4 + 2] * scale, acc_dk[db][4 * r4 + 3] * scale);
        const unsigned v01 = pack_bf16(acc_dv[db][4 * r4], acc_dv[db][4 * r4 + 1]);
        const unsigned v23 = pack_bf16(acc_dv[db][4 * r4 + 2], acc_dv[db][4 * r4 + 3]);
        *(u32x2*)(dkrow + f0) = u32x2{k01, k23};
        *(u32x2*)(dvrow + f0) = u32x2{v01, v23};
      }
  }
}

// ---------------------------------------------------------------------- dQ

template <bool kCausal, int kWaves>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdArgs a) {
  constexpr int kStages = kWaves == 8 ? 6 : 5;
  constexpr int kRows = 32 * kWaves;  // queries per workgroup
  constexpr int kStageBytes = 2 * kTileBytes;
  using Dma = TileDma<kWaves, false>;
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
  const size_t head = (size_t)bh * n * kD;
  const uint16_t* qg = a.q + head;
  const uint16_t* kg = a.k + head;
  const uint16_t* vg = a.v + head;
  const uint16_t* dog = a.dout + head;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int q0w = qb * kRows + wave_s * 32;  // this wave's first query
  const int qi = q0w + l32;                  // this lane's query (< n_pad)

  // Q^T and dO^T operands (B operands of S^T = K Q^T and dP^T = V dO^T)
  bf16x8 qop[4], dop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qop[ks] = row_operand(qg, qi, ks, hi, n);
    dop[ks] = row_operand(dog, qi, ks, hi, n);
  }
  const float* const hs = a.ws + (size_t)bh * 2 * a.n_pad;  // this head's L2, then -D
  const float lse2 = hs[qi];
  const float ndl = hs[a.n_pad + qi];
  f32x16 nd16;  // -D of this lane's query in every register: dP^T starts there
#pragma unroll
  for (int r = 0; r < 16; ++r) nd16[r] = ndl;
  const TrOffsets tr(lane);
  int row_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) row_off[ks] = tile_off(l32, 2 * ks + hi);

  // 32-key halves this wave works on: [0, jl].  Causal: up to the half that
  // starts at the wave's first query (the diagonal).  The last half is
  // masked per element when it is the diagonal or holds keys past N.
  // (A wave whose queries all lie past N runs like the others: its L2 is
  // +inf, so its probabilities are 0, and nothing of it is written.)
  const int q_last = min(n - 1, qb * kRows + kRows - 1);
  const int kv_end = kCausal ? q_last + 1 : n;
  const int t_end = (kv_end + kBwdTile - 1) / kBwdTile;
  const int jl = kCausal ? min(q0w / 32, 2 * t_end - 1) : 2 * t_end - 1;
  // Tile 0 runs on the general path; then tiles whose two steps are fast in
  // every wave (2t+1 < the first wave's jl), in whole turns of the ring; the
  // rest on the general path again.
  constexpr int kHead = 1;
  const int jl_min = kCausal ? min(qb * kWaves, 2 * t_end - 1) : 2 * t_end - 1;
  const int t_fast_end = jl_min >= 2 ? (jl_min - 2) / 2 + 1 : 0;
  const Dma dma(kg, vg, n, wave, lane, nullptr, 0);

  auto fast = [&](int j) { return j >= 1 && j <= jl - 1; };
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
      const int k0 = 32 * j;
      const bool diag = kCausal && k0 == q0w;
      const bool ragged = k0 + 32 > n;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], c, -lse2));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r + 1], c, -lse2));
        if (diag || ragged) {
          const int kr = 8 * (r >> 2) + 4 * hi + (r & 3);  // key - k0
          if ((diag && kr > l32) || k0 + kr >= n) p0 = 0.f;
          if ((diag && kr + 1 > l32) || k0 + kr + 1 >= n) p1 = 0.f;
        }
        set_word(ds_cur[r >> 3], (r & 7) >> 1, pack_bf16(p0 * dp_cur[r], p1 * dp_cur[r + 1]));
      }
    }
    if (fast(j + 1)) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ring[s] = slot_operand(s, nnb, hc, cb, hc);
    }
  };

  // Step j on the fast path (arguments as in the dK/dV kernel).  12 MFMA
  // slots; in group g: S(j+1) step g, dQ(j-1) step g, dP(j+1) step g.
  // Vector work on score pair k: FMA in slot a_k, exp2 in a_k + 1, product
  // and pack in a_k + 2, with a_k = 0, 1, 3, 4, 6, 7, 9, 10.
  auto step_fast = [&](const char* nb, int hn, const char* cb, int hc, const char* pb, int hp, const char* nnb,
                       f32x16& s_cur, f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt, const bf16x8 (&ds_prv)[2],
                       bf16x8 (&ds_cur)[2]) __attribute__((always_inline)) {
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
      step_fast(stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), sA, dpA, sB, dpB, dsB, dsA);
      step_fast(stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), sB, dpB, sA, dpA, dsA, dsB);
    } else {
      step_general(2 * t, stage(st), 1, stage(st), 0, stage(sp), 1, stage(sn), sA, dpA, sB, dpB, dsB, dsA);
      step_general(2 * t + 1, stage(sn), 0, stage(st), 1, stage(st), 0, stage(sn), sB, dpB, sA, dpA, dsA, dsB);
    }
    vm_wait_barrier_tiles<Dma::kPerTile, kStages - 4>(
        max(0, min(min(t_end - 1, t + kStages - 2) - (t + 2), kStages - 4)));
    if (t + kStages - 1 < t_end) dma.issue(t + kStages - 1, stage(sp));
  };
  using kGeneral = std::false_type;
  using kFast = std::true_type;

  // ---- prologue
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < t_end) dma.issue(i, stage(i));
  vm_wait_barrier_tiles<Dma::kPerTile, kStages - 3>(max(0, min(t_end, kStages - 1) - 2));
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
  if (2 * t_end - 1 <= jl) {
    const char* pb = half_stage(2 * t_end - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i & 1] = mfma(k_tr(pb, 1, i), dsB[i >> 1], acc[i & 1]);
  }

  if (qi < n) {
    uint16_t* row = a.dq + head + (size_t)qi * kD;
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

extern "C" attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int H,
                                int N, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_E_INVALID;
  if (B < 1 || H < 1 || N < 1 || d != kD || !std::isfinite(scale)) return ATTN_E_INVALID;
  if (!sizes_fit(B, H, N)) return ATTN_E_INVALID;
  const void* vec[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  for (const void* p : vec)
    if (misaligned(p, 16)) return ATTN_E_ALIGN;
  if (misaligned(lse, 4)) return ATTN_E_ALIGN;
  const attn_status st = check_device();
  if (st != ATTN_OK) return st;

  BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.ws = static_cast<float*>(workspace);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.n = N;
  a.n_pad = (N + kPadRows - 1) / kPadRows * kPadRows;
  a.bh_count = B * H;
  a.blocks = a.total = 0;
  a.c = scale * kLog2e;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);

  long long rows = (long long)B * H * a.n_pad;
  void* pargs[] = {&a, &rows};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_prep_kernel),
                                 dim3((unsigned)((rows + 255) / 256)), dim3(256), pargs, 0, s);
  if (e != hipSuccess) return ATTN_E_LAUNCH;

  if (causal) {
    e = launch_main<kWavesCausal>(reinterpret_cast<const void*>(&bwd_dkdv_kernel<true, kWavesCausal>), a, B, H, N, s);
    if (e == hipSuccess)
      e = launch_main<kWavesCausal>(reinterpret_cast<const void*>(&bwd_dq_kernel<true, kWavesCausal>), a, B, H, N, s);
  } else {
    e = launch_main<kWavesDkdv>(reinterpret_cast<const void*>(&bwd_dkdv_kernel<false, kWavesDkdv>), a, B, H, N, s);
    if (e == hipSuccess)
      e = launch_main<kWavesDq>(reinterpret_cast<const void*>(&bwd_dq_kernel<false, kWavesDq>), a, B, H, N, s);
  }
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
