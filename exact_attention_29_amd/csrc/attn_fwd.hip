// Exact attention forward for AMD Instinct MI355X (gfx950).
//
// What is computed: for each (batch, head), O = softmax(scale * Q K^T
// [+ causal mask]) V and LSE_i = m_i + ln(l_i) -- exact attention as defined
// on the page "FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness" (reading notes at notes.yuuk.io), section "problem setting".
// How: the page's section "proposed method" -- tiling (Q, K, V in blocks, a
// running row max m and row sum l updated block by block), kernel fusion
// (scores, mask, softmax and both products in one kernel, nothing N x N ever
// reaches device memory) and recomputation (only O and the statistics, here
// LSE, are written).  The block sizes on that page were chosen for another
// GPU's shared memory; the tiles below are sized for gfx950 instead.
//
// bf16 kernel.  One workgroup = 8 waves = 256 query rows of one head, one
// workgroup per CU, two waves per SIMD (causal, and non-causal calls too
// small to give every CU a 256-row tile: 4 waves = 128 rows, two workgroups
// per CU):
//   * each wave owns 32 query rows; their Q^T operands stay in VGPRs;
//   * K and V tiles of 64 keys go through an LDS ring filled by buffer-load
//     DMA (no staging registers): 6 stages with a barrier every second tile
//     for 8 waves, 5 stages filled three tiles ahead for 4 waves;
//     16-byte chunks are XOR-swizzled per row so both read patterns below
//     are bank-conflict free, and every LDS address is a per-lane constant
//     plus an immediate (the steady state is unrolled over the stages);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: lane l then holds 16 keys of
//     ONE query (l % 32), so row reductions stay in the lane plus one
//     exchange with lane l ^ 32;
//   * the S^T accumulator layout is exactly the B-operand layout of the next
//     MFMA, so P^T feeds O^T += V^T P^T without any lane shuffle; the V^T
//     operand is read from the row-major V tile with ds_read_b64_tr_b16;
//   * software pipeline over half tiles (32 keys): step j issues the MFMAs of
//     PV(j-1) and S(j+1) interleaved one by one with the vector-ALU softmax of
//     S(j), while the LDS operands of step j+1 are read.  On gfx950 a wave's
//     transcendental ops overlap its own MFMAs only when interleaved this
//     way; another wave's do not;
//   * online softmax in fp32: exp2 with scale*log2(e) folded into one FMA,
//     l sums the fp32 probabilities, P is rounded to bf16 for the PV product.
//     The first half tile sets the reference max from its own scores (on the
//     pipelined path when it needs no mask); masked edge tiles take the
//     exact tile max; the steady state reuses the running reference max and
//     computes none.  A partial row sum above 2^32 (a score
//     far above the reference, or an overflow) flags the wave, which then
//     recomputes its rows with the exact max on every tile (a rare path that
//     reads K and V straight from global memory);
//   * causal: key tiles past a wave's last query are skipped, only the
//     diagonal and ragged half tiles pay for masking;
//   * key masks (a valid length per batch entry, or a bit per key) hide keys
//     by select, like the causal mask; block-sparse calls walk a list of the
//     key tiles set for their 128-row query block instead of every tile;
//   * split calls (attn_fwd_split): when the last round of workgroups would
//     leave most CUs idle, its tiles' key ranges are cut into pieces spread
//     over every CU; each workgroup runs its one or two pieces in a loop,
//     hands each partial (unnormalised O^T, m, l) to a workspace slot, and
//     the last piece of a tile to arrive merges them in piece order.
// fp32 kernel: two lanes per query row on the vector ALU (each holds half of
// the features; scores, row sums and O's accumulators in fp64, exp2 in fp32),
// 8-key K/V tiles broadcast from LDS, hidden keys skipped; same online
// softmax.  Used for fp32 I/O.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "attn.h"
#include "attn_common.h"
#include "attn_split.h"

namespace {

using namespace attn_detail;

constexpr int kBc = 64;                      // keys per K/V tile (two half tiles)
// Waves per workgroup (each owns 32 query rows): 8 (256 rows, one workgroup
// per CU) without a mask, 4 (128 rows, two workgroups per CU) when causal,
// where shorter rows per workgroup balance the triangle better.
#ifndef ATTN_FULL_WAVES
#define ATTN_FULL_WAVES 8
#endif
constexpr int kWavesFull = ATTN_FULL_WAVES;
#ifndef ATTN_CAUSAL_WAVES
#define ATTN_CAUSAL_WAVES 4
#endif
constexpr int kWavesCausal = ATTN_CAUSAL_WAVES;
// Block-sparse calls: one workgroup per 128-row query block (4 waves), a
// 4-stage ring (prefetch distance 2) and the list of the block's key tiles
// in LDS (at most this many: N <= 64 * 4096).
constexpr int kSparseBlockQ = 128;
constexpr int kSparseBlockK = 64;
constexpr int kMaxSparseTiles = 4096;
constexpr int kTileBytes = kBc * kRow;       // 8192
constexpr int kStageBytes = 2 * kTileBytes;  // K tile, then V tile: 16384
// Prefetch distance: after the barrier that ends tile t, tile t+kLead+1 is
// requested.  The ring then needs kLead+2 stages: tile t-1 is still read
// during tile t (its PV), and tile t+1 is being published.
#ifndef ATTN_LEAD
#define ATTN_LEAD 3
#endif
// Grouped barriers for 8-wave workgroups (one per CU, so the LDS has room
// for a deeper ring): only every ATTN_GROUP-th tile ends in a wait and a
// barrier, which publish the next ATTN_GROUP tiles at once and request the
// ATTN_GROUP after them.  Every tile still gets ATTN_GROUP tiles' time to
// arrive; the workgroup meets ATTN_GROUP times less often.  The ring then
// holds 2*ATTN_GROUP+2 tiles, rounded up to a multiple of ATTN_GROUP.
#ifndef ATTN_GROUP
#define ATTN_GROUP 2
#endif
#define ATTN_GROUP_STAGES (((2 * ATTN_GROUP + 2 + ATTN_GROUP - 1) / ATTN_GROUP) * ATTN_GROUP)
#if ATTN_GROUP > 1 && ATTN_LEAD + 2 < ATTN_GROUP_STAGES
#define ATTN_STAGES ATTN_GROUP_STAGES
#else
#define ATTN_STAGES (ATTN_LEAD + 2)
#endif
constexpr int kLead = ATTN_LEAD;
constexpr int kStages = ATTN_STAGES;         // LDS ring of K/V tiles
constexpr int kLdsBytes = kStages * kStageBytes;  // the largest ring (96 KiB grouped by 2);
                                                  // 4-wave workgroups use 80 KiB, two per CU
static_assert(kLead >= 2 && kStages <= 9 && ATTN_GROUP >= 1 && ATTN_GROUP <= 3,
              "prefetch distance or barrier group out of range");
static_assert(kLdsBytes <= 160 * 1024, "LDS ring exceeds the 160 KiB of a gfx950 CU");

constexpr float kTau = 8.0f;                 // slack when the reference max is set
constexpr unsigned kRedoBits = 0x4f800000u;  // bit pattern of 2^32: a partial
                                             // row sum above it means the
                                             // reference max is stale
constexpr unsigned kInfBits = 0x7f800000u;   // bit pattern of +inf

// kinds of pipelined step: steady state; drain (no next S, no read-ahead);
// drain with a per-row last visible key (a causal diagonal or ragged half);
// first (half tile 0: no PV of a previous half)
constexpr int kStepNormal = 0, kStepDrain = 1, kStepLimit = 2, kStepFirst = 3;
using StepNormal = std::integral_constant<int, kStepNormal>;
using StepDrain = std::integral_constant<int, kStepDrain>;
using StepLimit = std::integral_constant<int, kStepLimit>;
using StepFirst = std::integral_constant<int, kStepFirst>;

struct Bf16Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int n;            // sequence length
  int q_tiles;      // ceil(n / rows per workgroup)
  int total_tiles;  // B * H * q_tiles
  float c;          // |scale| * log2(e), at least FLT_MIN
  uint32_t q_sign;  // 0x80008000 when scale < 0 (Q negated), else 0
  int heads;        // H: batch entry of head bh is bh / H
  // element strides of q, k, v, o (index 0..3) between batch entries, heads
  // and rows; the 64 features of a row are contiguous
  long long sb[4], sh[4];
  int sn[4];
  const uint8_t* block_mask;  // block-sparse kernel: [ceil(N/128)][mask_cols]
  int mask_cols;              // ceil(N/64)
  const int* key_len;         // [B] or null: keys j >= key_len[b] are hidden
  const uint32_t* key_bits;   // [B][ceil(N/32)] or null: bit j%32 of word j/32
                              // clear hides key j of entry b
  // Split launch only (see SplitRange): workgroups below dp_blocks take
  // whole query tiles; each of the 8 * sk_cus after them takes one range of
  // the key tiles of the query tiles left over past sk_rounds whole rounds,
  // and pieces merge through the workspace (ws_count: arrival counters, zero
  // between calls; ws_part: partial O, m, l slots).
  int dp_blocks;
  int sk_rounds;
  int sk_cus;     // workgroups one XCD runs at once
  int n_kt;       // key tiles of 64 per query tile: ceil(n / 64)
  int* ws_count;
  float* ws_part;
};

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// The kernel's arguments: the parameter itself, or (kSplit) the same bytes
// read through the kernel-argument segment pointer made opaque, so that
// each piece of a split workgroup reloads what it needs.
template <bool kSplit>
__device__ __forceinline__ decltype(auto) piece_args(const Bf16Args& args) {
  if constexpr (kSplit) {
    const __attribute__((address_space(4))) Bf16Args* ap =
        (const __attribute__((address_space(4))) Bf16Args*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    return (*ap);
  } else {
    return (args);
  }
}

template <bool kCausal, int kWaves, bool kKeyMask, bool kSparse, bool kSplit>
__global__ void __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_kernel(Bf16Args args) {
  constexpr int kBr = kWaves * 32;        // query rows per workgroup
  constexpr int kDmaPasses = 8 / kWaves;  // a DMA instruction covers 8 rows per wave
  constexpr int kDmaPerTile = 2 * kDmaPasses;
  static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves per workgroup");
  static_assert(!kSparse || (kWaves * 32 == kSparseBlockQ && !kKeyMask),
                "a block-sparse workgroup owns one query block; no key mask on that path");
  static_assert(!kSplit || (kWaves == 8 && !kCausal && !kSparse),
                "split launches: 8-wave non-causal dense workgroups");
  constexpr int kLeadK = kSparse ? 2 : kLead;  // prefetch distance (unpaired ring)
  constexpr int kGroup = kWaves == 8 && !kSparse ? ATTN_GROUP : 1;  // tiles per barrier
  constexpr int kStagesK = kGroup > 1 ? ATTN_GROUP_STAGES : kLeadK + 2;  // tile t in stage t % kStagesK
  static_assert(kLeadK >= 2 && kStagesK <= ATTN_STAGES, "ring deeper than the declared stages");
  // One LDS object per ring stage: with the stage known at compile time (the
  // steady state), the compiler can tell a stage being filled by DMA from the
  // stages being read and does not wait for the DMA before those reads.
  __shared__ __attribute__((aligned(1024))) char lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds3[kStageBytes];
  // stages past this kernel's ring take 16 bytes (never selected)
  __shared__ __attribute__((aligned(1024))) char lds4[kStagesK > 4 ? kStageBytes : 16];
#if ATTN_STAGES > 5
  __shared__ __attribute__((aligned(1024))) char lds5[kStagesK > 5 ? kStageBytes : 16];
#endif
#if ATTN_STAGES > 6
  __shared__ __attribute__((aligned(1024))) char lds6[kStagesK > 6 ? kStageBytes : 16];
#endif
#if ATTN_STAGES > 7
  __shared__ __attribute__((aligned(1024))) char lds7[kStagesK > 7 ? kStageBytes : 16];
#endif
#if ATTN_STAGES > 8
  __shared__ __attribute__((aligned(1024))) char lds8[kStagesK > 8 ? kStageBytes : 16];
#endif
  // block-sparse: the key tiles this workgroup's query block visits, ascending
  __shared__ uint16_t tile_list[kSparse ? kMaxSparseTiles : 1];
  auto stage_ptr = [&](int st) -> char* {
    char* p = st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : st == 3 ? lds3 : lds4;
#if ATTN_STAGES > 5
    p = st == 5 ? lds5 : p;
#endif
#if ATTN_STAGES > 6
    p = st == 6 ? lds6 : p;
#endif
#if ATTN_STAGES > 7
    p = st == 7 ? lds7 : p;
#endif
#if ATTN_STAGES > 8
    p = st == 8 ? lds8 : p;
#endif
    return p;
  };

  // ---- this workgroup's work: one whole query tile, or (a split launch,
  // past dp_blocks) the one or two pieces of its range, one after the other
  // through the same LDS ring.
  __shared__ int sk_arrived;  // split: pieces of the tile done before this one
  __shared__ int sk_range;    // split: this workgroup's range id, -1 for a whole tile
  __shared__ int sk_redo;     // split: some wave's reference went stale
  int n_pieces = 1;
  if constexpr (kSplit) {
    int id = -1;
    if ((int)blockIdx.x >= args.dp_blocks) {
      id = (int)blockIdx.x - args.dp_blocks;
      n_pieces = split_range(args, id).count;
      if (n_pieces == 0) return;  // an empty range (before any barrier)
    }
    if (threadIdx.x == 0) {
      sk_range = id;
      sk_redo = 0;
    }
    __syncthreads();
  } else {
    (void)args;
  }
  // pc: the piece of the range; exact: a second pass over the same piece
  // with an exact max on every half tile (the split kernels' fallback)
  int pc = 0;
  bool exact = false;
  for (;;) {
    // In split kernels the kernel arguments and the thread index are taken
    // afresh for every piece, through a pointer and a register the compiler
    // cannot see through: nothing derived from them stays live from one
    // piece to the next (the registers are all but full).
    int tid_raw = threadIdx.x;
    if constexpr (kSplit) asm volatile("" : "+v"(tid_raw));
    const auto& a = piece_args<kSplit>(args);
    const int n = a.n;
    Piece pz = {xcd_remap(blockIdx.x, a.total_tiles), 0, kSplit ? a.n_kt : 0, 1, 0, 0, 0, 0};
    if constexpr (kSplit) {
      if (pc > 0 || exact) __syncthreads();  // the previous pass's DMA and LDS reads are done
      const int id = __builtin_amdgcn_readfirstlane(*(volatile int*)&sk_range);  // uniform
      if (id >= 0) pz = split_piece(split_range(a, id), pc);
    }
    // first key tile of this piece (0 unless split)
    const int kt_base = kSplit ? pz.kt_a : 0;
    const int logical = pz.logical;
    int bh, qt;
    if constexpr (kCausal) {
      int rank;  // the last query tile of a head has the longest rows
      causal_order(logical, a.total_tiles / a.q_tiles, a.q_tiles, bh, rank);
      qt = a.q_tiles - 1 - rank;
    } else {
      bh = logical / a.q_tiles;
      qt = logical - bh * a.q_tiles;
    }
    const int b_entry = bh / a.heads;
    const int h_idx = bh - b_entry * a.heads;
    auto head_off = [&](int t) { return (size_t)(b_entry * a.sb[t] + h_idx * a.sh[t]); };
    const uint16_t* __restrict__ qg = a.q + head_off(0);
    const uint16_t* __restrict__ kg = a.k + head_off(1);
    const uint16_t* __restrict__ vg = a.v + head_off(2);
    const int q_sn = a.sn[0], k_sn = a.sn[1], v_sn = a.sn[2];

    const int tid = tid_raw;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave
    const int l32 = lane & 31;
    const int hi = lane >> 5;  // which half of the wave
    const int q_wave = qt * kBr + wave * 32;
    const int qi = q_wave + l32;  // this lane's query row

    // ---- Q^T operands (B operand of S^T = K Q^T): lane holds 8 consecutive
    // features (16*ks + 8*hi ..) of query qi.
    bf16x8 qop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qi < n) w = *(const u32x4*)(qg + (size_t)qi * q_sn + 16 * ks + 8 * hi);
      w ^= a.q_sign;
      qop[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // ---- key range.  n_k: keys of this batch entry that may be visible (a
    // per-entry valid length hides the rest, like keys past the end).
    // (readfirstlane: one value for the workgroup, which keeps the tile
    // counts below scalar; in a split kernel's piece loop, after stores, the
    // load itself is a vector load)
    const int n_k = a.key_len ? __builtin_amdgcn_readfirstlane(min(max(a.key_len[b_entry], 0), n)) : n;
    int kv_end = n_k;
    if (kCausal) kv_end = min(n_k, qt * kBr + kBr);
    if (kSplit) kv_end = min(kv_end, kBc * pz.kt_b);  // a piece ends at key tile kt_b
    // half tiles of 32 keys from key tile kt_base on (a position j is half
    // tile 2*kt_base + j of the sequence)
    int n_half = max(0, (kv_end + 31) / 32 - 2 * kt_base);
    int n_tiles = (n_half + 1) / 2;
    // last key / half tile (position) with any visible key for this wave
    int wave_last_key = (q_wave >= n || n_k == 0) ? -1 : (kCausal ? min(n_k - 1, q_wave + 31) : n_k - 1);
    if (kSplit && wave_last_key >= 0) {
      wave_last_key = min(wave_last_key, kBc * pz.kt_b - 1);
      if (wave_last_key < kBc * kt_base) wave_last_key = -1;
    }
    int last_h = wave_last_key < 0 ? -1 : wave_last_key / 32 - 2 * kt_base;

    // ---- block-sparse: compact the key tiles whose block of M is set for
    // this query block into tile_list (wave 0 writes, every wave counts); from
    // here on a tile or half-tile index is a position in that list, and
    // kt_of / real_half map it back to key indices.  Tiles past the causal
    // diagonal or the valid length are not listed (n_tiles bounds them).
    int n_act = n_tiles;
    if constexpr (kSparse) {
      const uint8_t* mrow = a.block_mask + (size_t)qt * a.mask_cols;
      n_act = 0;
      for (int base = 0; base < n_tiles; base += 64) {
        const int kt = base + lane;
        const bool act = kt < n_tiles && mrow[kt] != 0;
        const uint64_t bal = __ballot(act);
        const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
        if (wave == 0 && act) tile_list[n_act + below] = (uint16_t)kt;
        n_act += __popcll(bal);
      }
      __syncthreads();
      n_tiles = n_act;
      n_half = 2 * n_act;  // a listed ragged tile's hidden half is masked
      last_h = (wave_last_key < 0 || n_act == 0) ? -1 : n_half - 1;
    }
    auto kt_of = [&](int pos) -> int {
      if constexpr (kSparse) return __builtin_amdgcn_readfirstlane((int)tile_list[pos]);
      else return kt_base + pos;
    };
    auto real_half = [&](int j) -> int {
      if constexpr (kSparse) return 2 * kt_of(j >> 1) + (j & 1);
      else return 2 * kt_base + j;
    };

    // ---- global -> LDS staging by DMA (buffer/global loads with the LDS
    // bit, 16 bytes per lane): in pass p, lane l of wave w fills LDS chunk slot
    // (row 8*w + l/8 + 8*kWaves*p, position l%8) of the K tile and of the V
    // tile, so it fetches global chunk (l%8) ^ swz(row) of that row (the same
    // chunk in every pass: swz depends on row bits 1-3 only).  In the ragged
    // last tile, rows past N read row N-1 instead (finite data; those keys are
    // masked and their probabilities are exactly 0).
    constexpr int kPassRows = 8 * kWaves;
    constexpr int kPassBytes = kPassRows * kRow;
    static_assert(kPassRows % 16 == 0, "a pass must not change the row swizzle");
    const int dma_row = 8 * wave + (lane >> 3);
    const int dma_chunk = (lane & 7) ^ swz(dma_row);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    // byte offsets of this lane's chunk within a K and a V tile (row strides
    // in bytes: 2 * k_sn, 2 * v_sn; the host keeps every offset below 2^31)
    const int k_lane_off = dma_row * 2 * k_sn + dma_chunk * 16;
    const int v_lane_off = dma_row * 2 * v_sn + dma_chunk * 16;
    // Buffer resources over this head's K and V: a whole tile is fetched with
    // the tile's byte offset in a scalar register and this lane's constant
    // offset, so the steady state spends no vector instruction on addresses.
    const int k_bytes = (n - 1) * 2 * k_sn + kRow;
    const int v_bytes = (n - 1) * 2 * v_sn + kRow;
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, k_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t v_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, v_bytes, kBufferWord3);
    auto dma_tile = [&](int pos, char* stage_base) __attribute__((always_inline)) {
      const int kt = kt_of(pos);
      char* kd = stage_base + wave_s * 1024;
      if ((kt + 1) * kBc <= n) {
#pragma unroll
        for (int ps = 0; ps < kDmaPasses; ++ps) {
          const int row0 = kt * kBc + ps * kPassRows;  // first row of this pass
          __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (__attribute__((address_space(3))) void*)(kd + ps * kPassBytes),
                                                   16, k_lane_off, row0 * 2 * k_sn, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc,
                                                   (__attribute__((address_space(3))) void*)(kd + kTileBytes + ps * kPassBytes),
                                                   16, v_lane_off, row0 * 2 * v_sn, 0, 0);
        }
      } else {
        // ragged last tile: rows past N re-read row N-1.  The address is
        // the head's base plus a 32-bit lane offset (below 2^31, like every
        // offset), so the load takes the scalar-base form and no 64-bit
        // address is kept per lane.
#pragma unroll
        for (int ps = 0; ps < kDmaPasses; ++ps) {
          const int key = min(kt * kBc + dma_row + ps * kPassRows, n - 1);
          const char* ks = reinterpret_cast<const char*>(kg) + (unsigned)(key * 2 * k_sn + dma_chunk * 16);
          const char* vs = reinterpret_cast<const char*>(vg) + (unsigned)(key * 2 * v_sn + dma_chunk * 16);
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)ks,
                                           (__attribute__((address_space(3))) void*)(kd + ps * kPassBytes), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)vs,
                                           (__attribute__((address_space(3))) void*)(kd + kTileBytes + ps * kPassBytes),
                                           16, 0, 0);
        }
      }
    };



    // End of tile t: the barrier publishes tile t+2, whose DMAs must be done;
    // those of tiles t+3 .. t+kLeadK (the ones that exist) may still fly.  Every
    // LDS read of the stage the next DMA overwrites has already fed an MFMA, so
    // the barrier needs no LDS wait.
    auto dma_barrier = [&](int t) __attribute__((always_inline)) {
      vm_wait_barrier_tiles<kDmaPerTile, kLeadK - 2>(min(kLeadK - 2, max(0, n_tiles - 3 - t)));
    };
    // End of tile t (in stage st).  Per-tile ring: the barrier above, then
    // tile t+1+kLeadK is requested into the stage of tile t-1.  Grouped ring
    // (g = kGroup): only tiles with t % g == 0 end in a barrier.  There every
    // request is waited for (tiles t+2 .. t+g+1, requested one group ago), the
    // barrier publishes them (they are read up to the next barrier, t+g), and
    // tiles t+g+2 .. t+2g+1 are requested into the stages of tiles
    // t-g .. t-1, whose last reads fed MFMAs of tile t at the latest.  The
    // ring's stage count is a multiple of g, so t % g == st % g.
    auto end_tile = [&](int t, int st) __attribute__((always_inline)) {
      if constexpr (kGroup > 1) {
        if ((unsigned)st % kGroup == 0u) {  // st >= 0
          vm_wait_barrier<0>();
#pragma unroll
          for (int i = kGroup + 2; i <= 2 * kGroup + 1; ++i)
            if (t + i < n_tiles) dma_tile(t + i, stage_ptr((st + i) % kStagesK));
        }
      } else {
        dma_barrier(t);
        if (t + 1 + kLeadK < n_tiles) dma_tile(t + 1 + kLeadK, stage_ptr((st + 1 + kLeadK) % kStagesK));
      }
    };


    // ---- per-lane LDS read offsets within a stage (swizzle constant per lane;
    // half tile h adds 32 rows, PV step tt 16 rows: neither changes swz)
    // K operand (A of S^T), step ks: row l32 (+32h), chunk 2*ks + hi.
    int k_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) k_off[ks] = tile_off(l32, 2 * ks + hi);
    // V^T operand via ds_read_b64_tr_b16: in each 16-lane group g, lane j
    // points at row 16*tt + 4*hi + (j>>2) (+8 for the second half of the
    // operand) and feature 32*db + 16*(g&1) + 4*(j&3).
    const int g = lane >> 4, j16 = lane & 15;
    int v_off[2][2];  // [sec][db]
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int row = 4 * hi + (j16 >> 2) + 8 * sec;
        const int byte = 2 * (32 * db + 16 * (g & 1) + 4 * (j16 & 3));
        v_off[sec][db] = kTileBytes + row * kRow + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
      }
    // The same offsets plus kHiShift, opaque to the compiler.  A ds_read takes
    // a VGPR address plus a 16-bit immediate: reads from the stages at LDS
    // address 64 KiB and above would need an add per read to form the address.
    // Reads of the stages a steady-state step knows at compile time to lie at
    // 32 KiB or above use these registers with (stage address - kHiShift) as
    // the immediate instead.
    constexpr int kHiShift = 32768;
    int k_off_hi[4], v_off_hi[2][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      k_off_hi[ks] = k_off[ks] + kHiShift;
      asm volatile("" : "+v"(k_off_hi[ks]));
    }
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        v_off_hi[sec][db] = v_off[sec][db] + kHiShift;
        asm volatile("" : "+v"(v_off_hi[sec][db]));
      }

    const float c = a.c;
    f32x16 acc[2];  // O^T, feature blocks db = 0, 1
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    float l_part_max = 0.f;  // largest partial row sum of a steady-state step
    const f32x16 zero16 = {};

    // ---- the three pieces of work on one half tile (32 keys).  Half tile j
    // covers keys 32*j .. 32*j+31: tile j/2 (LDS stage (j/2) % kStagesK), rows 32*(j%2)..
    //
    // S^T = K Q^T: s holds keys 32*j + 8*(r/4) + 4*hi + r%4 of query qi.
    auto compute_s = [&](const char* stage_base, int h, f32x16& s) __attribute__((always_inline)) {
      const char* kb = stage_base + 32 * h * kRow;
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(kb, k_off[0]), qop[0], zero16, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(kb, k_off[ks]), qop[ks], s, 0, 0, 0);
    };
    // O^T += V^T P^T over one half tile; pop[tt] covers its keys 16*tt .. +15.
    auto compute_pv = [&](const char* stage_base, int h, const bf16x8 (&pop)[2]) __attribute__((always_inline)) {
      const char* vb = stage_base + 32 * h * kRow;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const char* p = vb + 16 * tt * kRow;
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_vt(p + v_off[0][db], p + v_off[1][db]), pop[tt], acc[db], 0, 0, 0);
        }
    };
    auto stage_base = [&](int j) { return stage_ptr((j >> 1) % kStagesK); };

    // Hidden keys of half tile j become -inf (ragged end or valid length,
    // causal diagonal, and with a key mask every key it hides).
    const uint32_t* const mask_row = kKeyMask ? a.key_bits + (size_t)b_entry * ((n + 31) / 32) : nullptr;
    // Mask words are the same in every lane and read-only while the kernel
    // runs: read through the constant address space they become scalar loads.
    // (A vector load would share its completion counter with the K/V DMA, and
    // waiting for it would wait for every tile in flight.)  The index is
    // clamped to the row's last word, so reading ahead stays in the buffer.
    const int n_words = (n + 31) / 32;
    auto mask_word = [&](int j) -> uint32_t {
      typedef const __attribute__((address_space(4))) uint32_t cword;
      return ((cword*)mask_row)[min(real_half(j), n_words - 1)];
    };
    auto needs_lim = [&](int j) {
      const int jr = real_half(j);
      return 32 * jr + 32 > n_k || (kCausal && 32 * jr + 31 > q_wave);
    };
    auto needs_mask = [&](int j) { return kKeyMask || needs_lim(j); };
    // One mask word covers a half tile's 32 keys, the same for every lane (a
    // scalar load).  Register r holds key 8*(r/4) + 4*hi + r%4: its 64-lane
    // condition is built on the scalar unit and selects with one v_cndmask.
    auto apply_bits = [&](uint32_t vis, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k0 = 8 * (r >> 2) + (r & 3);
        const uint64_t lanes = (((vis >> k0) & 1u) ? 0x00000000ffffffffull : 0ull) |
                               (((vis >> (k0 + 4)) & 1u) ? 0xffffffff00000000ull : 0ull);
        s[r] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? s[r] : -INFINITY;
      }
    };
    auto apply_mask = [&](int j, f32x16& s) __attribute__((always_inline)) {
      if (kKeyMask) apply_bits(mask_word(j), s);  // j < n_half <= ceil(N/32)
      if (!kKeyMask || needs_lim(j)) {
        const int lim = kCausal ? min(qi, n_k - 1) : n_k - 1;  // last visible key
        const int jr = real_half(j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * jr + 8 * (r >> 2) + 4 * hi + (r & 3);
          s[r] = key <= lim ? s[r] : -INFINITY;
        }
      }
    };

    // exp2(c*s - m) for the 16 scores, packed into the two bf16 P operands;
    // returns this lane's fp32 partial row sum.
    auto exp_pack = [&](const f32x16& s, float m, bf16x8 (&pop)[2]) __attribute__((always_inline)) -> float {
      float lsum = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 p8;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * tt + i], c, -m));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * tt + i + 1], c, -m));
          lsum += e0;
          lsum += e1;
          const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
          p8[i] = pr[0];
          p8[i + 1] = pr[1];
        }
        pop[tt] = p8;
      }
      return lsum;
    };

    // Softmax of one half tile with an exact tile max (general path and the
    // rare redo).  m_run (log2 units, scale folded in) is the reference the
    // probabilities are taken against; it is raised only when some row's max
    // exceeds it by more than kTau.  Any reference gives the same O and LSE.
    // Returns the factor acc must be scaled by (1 when unchanged).
    auto softmax_exact = [&](const f32x16& s, bf16x8 (&pop)[2], bool& raised) __attribute__((always_inline)) -> float {
      float mx = fmaxf(s[0], s[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[r], s[r + 1]));
      mx = half_swap_max(mx) * c;
      raised = __any(mx > m_run + kTau);
      const float m_new = raised ? fmaxf(m_run, mx) : m_run;
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      const float msub = (m_new == -INFINITY) ? 0.f : m_new;
      l_run = l_run * alpha + exp_pack(s, msub, pop);
      return alpha;
    };
    auto rescale = [&](float alpha) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    };

    // General step (any j): j is the half tile being softmaxed; s_cur/p_cur its
    // buffers, s_nxt receives S(j+1), p_prv holds P(j-1).
    auto step_general = [&](int j, f32x16& s_cur, bf16x8 (&p_cur)[2], f32x16& s_nxt,
                            const bf16x8 (&p_prv)[2]) __attribute__((always_inline)) {
      if (j >= 1 && j - 1 <= last_h) compute_pv(stage_base(j - 1), (j - 1) & 1, p_prv);
      if (j + 1 < n_half && j + 1 <= last_h) compute_s(stage_base(j + 1), (j + 1) & 1, s_nxt);
      if (j <= last_h) {
        if (needs_mask(j)) apply_mask(j, s_cur);
        bool raised;
        const float alpha = softmax_exact(s_cur, p_cur, raised);
        if (raised) rescale(alpha);
      }
    };

    // a key-mask kernel's words of the next fast tile, loaded one tile ahead
    uint32_t vis_next0 = 0xffffffffu, vis_next1 = 0xffffffffu;

    // Operands of one steady-state step: V^T for PV(j-1) and K for S(j+1).
    struct Ops {
      bf16x8 v[2][2];
      bf16x8 k[4];
    };
    // The K operands of S(j+1) and the V^T operands of one 16-key block tt of
    // PV(j).  s_hi / pv_hi (compile-time in the steady state): the stage lies
    // at LDS address 32 KiB or above, read through the shifted offsets.
    auto load_k = [&](const char* s_base, int s_h, Ops& o, bool s_hi = false, int ks0 = 0,
                      int ks1 = 4) __attribute__((always_inline)) {
      const char* kb = s_base + 32 * s_h * kRow;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        if (ks >= ks0 && ks < ks1)
          o.k[ks] = s_hi ? lds_read_b128(kb, k_off_hi[ks] - kHiShift) : lds_read_b128(kb, k_off[ks]);
    };
    auto load_vt = [&](const char* pv_base, int pv_h, int tt, Ops& o, bool pv_hi = false) __attribute__((always_inline)) {
      const char* p = pv_base + 32 * pv_h * kRow + 16 * tt * kRow;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        if (pv_hi)
          o.v[tt][db] = lds_read_vt(p + (v_off_hi[0][db] - kHiShift), p + (v_off_hi[1][db] - kHiShift));
        else
          o.v[tt][db] = lds_read_vt(p + v_off[0][db], p + v_off[1][db]);
      }
    };
    auto load_ops = [&](const char* pv_base, int pv_h, const char* s_base, int s_h, Ops& o) __attribute__((always_inline)) {
      load_vt(pv_base, pv_h, 0, o);
      load_vt(pv_base, pv_h, 1, o);
      load_k(s_base, s_h, o);
    };

    // Steady-state step: the operands `cur` (read during the previous step)
    // feed PV(j-1) and S(j+1); the reads for the next step go out during the
    // step (K after slot 0, or 0 and 2, V^T after slots 4 and 6); the softmax of S(j) uses
    // the current reference.  One
    // basic block: 8 slots of one MFMA (PV and S alternating, so dependent
    // MFMAs are two slots apart) and one vector-ALU chunk (two exponentials
    // with their FMA, sum and bf16 packing).
    int drain_lim = 31;  // a limited drain step's last visible key offset in its half, per row
    auto step_fast = [&](const Ops& cur, Ops& nxt, const char* npv_base, int npv_h,
                         const char* ns_base, int ns_h, f32x16& s_cur, bf16x8 (&p_cur)[2],
                         f32x16& s_nxt, const bf16x8 (&p_prv)[2], uint32_t vis, bool fetch_words,
                         int word_j, auto mode_tag, bool npv_hi = false,
                         bool ns_hi = false) __attribute__((always_inline)) {
      // a drain step (the wave's last visible half tile): no S of a next half,
      // no operands to read ahead; kStepLimit also hides the keys of the half
      // past offset drain_lim of this lane's row (causal diagonal, sequence end)
      constexpr int kMode = decltype(mode_tag)::value;
      constexpr bool kDrain = kMode == kStepDrain || kMode == kStepLimit;
      if constexpr (kMode == kStepLimit) {
        const int lim = drain_lim - 4 * hi;  // register r holds key offset 8*(r/4) + 4*hi + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) s_cur[r] = 8 * (r >> 2) + (r & 3) <= lim ? s_cur[r] : -INFINITY;
      }
      // with a key mask, hide the masked keys of this half tile first (nothing
      // to do, and no instruction spent, when all 32 keys take part)
      if (kKeyMask && vis != 0xffffffffu) apply_bits(vis, s_cur);
      __builtin_amdgcn_sched_barrier(0);
      const float m = m_run;
      float lsum = 0.f;
      // The vector-ALU work on score pair k (FMA, exp2, sum, bf16 pack) is
      // spread over three slots: slot k-1 does its FMA, slot k its exp2, slot
      // k+1 its sum and pack.  No instruction then waits on the one just before
      // it (exp2 results in particular arrive late), so the wave keeps issuing
      // under its MFMAs.  The empty asm statements pin each piece to its slot
      // (left alone, the compiler sinks sums and packs to the end of the step).
      float t0 = __builtin_fmaf(s_cur[0], c, -m), t1 = __builtin_fmaf(s_cur[1], c, -m);
      float e0 = 0.f, e1 = 0.f;
#pragma unroll
      for (int slot = 0; slot <= 8; ++slot) {
        if (slot < 8) {
          if ((slot & 1) == 1) {
            if constexpr (kMode != kStepFirst) {
              const int i = slot >> 1, tt = i >> 1, db = i & 1;
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.v[tt][db], p_prv[tt], acc[db], 0, 0, 0);
            }
          } else if constexpr (!kDrain) {
            const int ks = slot >> 1;
            s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.k[ks], qop[ks], ks == 0 ? zero16 : s_nxt, 0, 0, 0);
          }
          // the next step's operands: K right after the first MFMA (causal
          // kernels: its second half after slot 2), the two V^T blocks after
          // slots 4 and 6 (spreading the reads over the step evens out the LDS
          // load of the CU's waves: 3 MP +1.6%, 8 MP +2.9%, 3 MP causal +4%
          // against reading them all at slot 0)
          if ((slot == 4 || slot == 6) && !kDrain) {
            __builtin_amdgcn_sched_barrier(0);
            load_vt(npv_base, npv_h, (slot - 4) >> 1, nxt, npv_hi);
          }
          if (kCausal && slot == 2 && !kDrain) {
            __builtin_amdgcn_sched_barrier(0);
            load_k(ns_base, ns_h, nxt, ns_hi, 2, 4);
          }
          if (slot == 0 && !kDrain) {
            __builtin_amdgcn_sched_barrier(0);
            load_k(ns_base, ns_h, nxt, ns_hi, 0, kCausal ? 2 : 4);
            // the next tile's mask words: issued here, a whole step before the
            // next wait on LDS operands (which then also covers them)
            if (kKeyMask && fetch_words) {
              asm volatile("" ::: "memory");  // keeps the loads below the MFMA above
              vis_next0 = mask_word(word_j);
              vis_next1 = mask_word(word_j + 1);
            }
          }
        }
        if (slot >= 1) {
          // sum and pack pair slot-1 into its 32-bit word of the P operand
          const int r = 2 * (slot - 1);
          lsum += e0;
          lsum += e1;
          const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
          unsigned pw = __builtin_bit_cast(unsigned, pr);
          asm volatile("" : "+v"(pw));
          u32x4 words = __builtin_bit_cast(u32x4, p_cur[r >> 3]);
          words[(r & 7) >> 1] = pw;
          p_cur[r >> 3] = __builtin_bit_cast(bf16x8, words);
          asm volatile("" : "+v"(lsum));
        }
        if (slot < 8) {
          e0 = __builtin_amdgcn_exp2f(t0);
          e1 = __builtin_amdgcn_exp2f(t1);
          if (slot < 7) {
            t0 = __builtin_fmaf(s_cur[2 * slot + 2], c, -m);
            t1 = __builtin_fmaf(s_cur[2 * slot + 3], c, -m);
          }
          asm volatile("" : "+v"(e0), "+v"(e1), "+v"(t0), "+v"(t1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Track the largest partial sum (checked once, after the loop): a plain
      // max keeps the step free of compares into scalar registers.  A partial
      // sum is never NaN (a sum of exp2 results, +inf at worst).
      l_part_max = fmaxf(l_part_max, lsum);
      l_run += lsum;
      __builtin_amdgcn_sched_barrier(0);
    };


    f32x16 sA, sB;
    bf16x8 pA[2], pB[2];

    // one tile t (half tiles 2t, 2t+1) on the general path
    auto tile_general = [&](int t) __attribute__((always_inline)) {
      step_general(2 * t, sA, pA, sB, pB);
      if (2 * t + 1 < n_half) step_general(2 * t + 1, sB, pB, sA, pA);
      end_tile(t, t % kStagesK);
    };
    // one tile t whose stage is known at compile time, both steps fast.  Step
    // 2t uses operands A and reads B for step 2t+1 (PV(2t) from this tile's
    // first half, S(2t+2) from the next tile's first half); step 2t+1 reads A
    // for step 2t+2 (PV(2t+1), S(2t+3): second halves).
    Ops opA, opB;
    auto tile_fast = [&](int t, auto stage_tag) __attribute__((always_inline)) {
      constexpr int st = decltype(stage_tag)::value;
      constexpr int st_next = (st + 1) % kStagesK;
      char* const b_cur = stage_ptr(st);
      char* const b_next = stage_ptr(st_next);
      const uint32_t vis0 = vis_next0, vis1 = vis_next1;
      // stages 2 and up sit at LDS addresses of 32 KiB and more (16 KiB each,
      // in declaration order): read through the shifted offsets
      constexpr bool cur_hi = st >= 2, next_hi = st_next >= 2;
      step_fast(opA, opB, b_cur, 0, b_next, 0, sA, pA, sB, pB, vis0, true, 2 * t + 2, StepNormal(), cur_hi,
                next_hi);  // j = 2t
      step_fast(opB, opA, b_cur, 1, b_next, 1, sB, pB, sA, pA, vis1, false, 0, StepNormal(), cur_hi,
                next_hi);  // j = 2t + 1
      end_tile(t, st);
    };
    // Tile t holding this wave's last visible half tile last_h (2t or 2t+1),
    // after a pipelined tile (so opA holds its operands and, with a key mask,
    // vis_next its words), when the halves before last_h need no mask: last_h
    // is a drain step, limited (per row, drain_lim) when it needs a mask.  Its
    // PV follows in the next step of the general path, or after the loop when
    // last_h is the sequence's last half.  K operands read ahead for a half
    // with no S are never used (stage memory, in bounds, whatever it holds).
    auto tile_drain = [&](int t, bool limited) __attribute__((always_inline)) {
      const int st = t % kStagesK;
      char* const b_cur = stage_ptr(st);
      char* const b_next = stage_ptr((st + 1) % kStagesK);
      if (last_h == 2 * t + 1) {
        step_fast(opA, opB, b_cur, 0, b_next, 0, sA, pA, sB, pB, vis_next0, false, 0, StepNormal());
        if (limited) step_fast(opB, opA, b_cur, 1, b_next, 1, sB, pB, sA, pA, vis_next1, false, 0, StepLimit());
        else step_fast(opB, opA, b_cur, 1, b_next, 1, sB, pB, sA, pA, vis_next1, false, 0, StepDrain());
      } else {
        if (limited) step_fast(opA, opB, b_cur, 0, b_next, 0, sA, pA, sB, pB, vis_next0, false, 0, StepLimit());
        else step_fast(opA, opB, b_cur, 0, b_next, 0, sA, pA, sB, pB, vis_next0, false, 0, StepDrain());
        // half 2t+1 exists but is hidden from this wave: PV(2t) now
        if (2 * t + 1 < n_half) compute_pv(b_cur, 0, pA);
      }
      end_tile(t, st);
    };

    // ---- prologue: tiles 0 .. kFirst requested; tiles 0 and 1 (read during
    // tile 0) must land before the first barrier.  Per-tile ring: tile
    // t+kLeadK is requested right after the barrier ending tile t-1.  Grouped
    // ring: the barrier ending tile 0 publishes tiles 2 .. g+1.
    constexpr int kFirst = kGroup > 1 ? kGroup + 1 : kLeadK;
    constexpr int kReady = 2;
#pragma unroll
    for (int tl = 0; tl <= kFirst; ++tl)
      if (tl < n_tiles) dma_tile(tl, stage_ptr(tl));
    // the rest of the min(n_tiles, kFirst+1) requested may still fly
    vm_wait_barrier_tiles<kDmaPerTile, kFirst + 1 - kReady>(max(0, min(n_tiles, kFirst + 1) - kReady));
    if (last_h >= 0) compute_s(lds0, 0, sA);

    // ---- tiles: 0 (its first half on the exact path, which sets the
    // reference; its second half pipelined when tile 1 is), then the steady
    // state (both half steps fast) unrolled over the ring's stages, then the
    // rest on the general path.
    // Tile t is steady when 2t+2 < n_half, 2t+2 <= last_h and neither 2t nor
    // 2t+1 needs a mask; all three conditions only get stricter with t
    int t_fast_end = 1;
    {
      int lim = min((n_half - 3) / 2, (last_h - 2) / 2);  // 2t+2 < n_half, 2t+2 <= last_h
      if (last_h < 2) lim = 0;
      int full = n_k / 32;                                 // halves with no ragged key
      if (kCausal) full = min(full, q_wave / 32);          // halves before the diagonal
      full -= 2 * kt_base;                                 // as positions
      if constexpr (kSparse) {
        // positions whose listed tile kt has 2kt+1 < full: a prefix of the
        // ascending list; binary search for its length
        const int kt_lim = (full - 2) / 2;
        int lo = 0, up = n_act;
        while (lo < up) {
          const int mid = (lo + up) >> 1;
          if (kt_of(mid) <= kt_lim) lo = mid + 1;
          else up = mid;
        }
        lim = min(lim, lo - 1);
      } else {
        lim = min(lim, (full - 2) / 2);                    // 2t+1 < full
      }
      if (full < 2) lim = 0;
      t_fast_end = max(1, lim + 1);
    }
    if (kSplit && exact) t_fast_end = 1;  // the redo pass: the general path throughout
    const int t_fast_steady = t_fast_end;
    // The steady state needs a finite reference in every row: with a key mask
    // or a block list, a row whose first half was all hidden has none yet, so
    // such a wave stays on the exact-max path (no -inf - -inf, no NaN) until
    // it has one.  Without them, key 0 is visible to every row.
    auto no_reference = [&]() { return (kKeyMask || kSparse) && __any(m_run == -INFINITY); };
    if (!kKeyMask && !kSparse && t_fast_end > 1) {
      // Half 0 needs no mask: it runs on the pipelined path too (S(1) beside
      // its softmax), with its own row max as the reference (any finite
      // reference gives the same O and LSE; this is the one the exact path
      // would set).  Its K operands for S(1) are read here; the step reads
      // those of half 1 (PV(0), S(2)).  Then half 1 as below.
      float mx = fmaxf(sA[0], sA[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sA[r], sA[r + 1]));
      m_run = half_swap_max(mx) * c;
      load_ops(lds0, 0, lds0, 1, opA);  // K of S(1); its V^T part is not used
      step_fast(opA, opB, lds0, 0, lds1, 0, sA, pA, sB, pB, 0xffffffffu, false, 0, StepFirst());
      step_fast(opB, opA, lds0, 1, lds1, 1, sB, pB, sA, pA, 0xffffffffu, false, 0, StepNormal());
    } else {
      step_general(0, sA, pA, sB, pB);  // S(1) -> sB, P(0) -> pA
      if (no_reference()) t_fast_end = 1;
      if (t_fast_end > 1) {
        // half 1 on the pipelined path: its operands (PV(0) from tile 0's first
        // half, S(2) from tile 1's) are read here; it reads those of step 2
        // (PV(1), S(3)) and, with a key mask, tile 1's words
        load_ops(lds0, 0, lds1, 0, opB);
        step_fast(opB, opA, lds0, 1, lds1, 1, sB, pB, sA, pA, kKeyMask ? mask_word(1) : 0xffffffffu, true, 2,
                  StepNormal());
      } else if (1 < n_half) {
        step_general(1, sB, pB, sA, pA);
        if (!no_reference()) t_fast_end = t_fast_steady;
        if (t_fast_end > 1) {
          // operands of step 2: PV(1) from tile 0's second half, S(3) from tile 1's
          load_ops(lds0, 1, lds1, 1, opA);
          if constexpr (kKeyMask) {
            vis_next0 = mask_word(2);
            vis_next1 = mask_word(3);
          }
        }
      }
    }
    end_tile(0, 0);
    int t = 1;
    for (; t + kStagesK - 1 < t_fast_end; t += kStagesK) {
      // tiles t .. t+kStagesK-1 sit in stages 1, 2, .., kStagesK-1, 0
      Unroll<0, kStagesK>::run([&](auto i) {
        constexpr int I = decltype(i)::value;
        tile_fast(t + I, std::integral_constant<int, (I + 1) % kStagesK>());
      });
    }
    // A last, partial turn of the ring (short rows: most of a causal or short
    // sequence's tiles are here), in a copy of its own so that the loop above
    // stays branch-free.  Each wave handles every tile exactly once, fast
    // below its t_fast_end and general from there on, so all waves meet the
    // same barriers.
    if (t < t_fast_end) {
      Unroll<0, kStagesK - 1>::run([&](auto i) {
        constexpr int I = decltype(i)::value;
        if (t + I < t_fast_end) tile_fast(t + I, std::integral_constant<int, (I + 1) % kStagesK>());
      });
    }
    t = t_fast_end;
    // (not for causal block lists: there every wave's last listed half is the
    // diagonal tile's, which measured slower drained)
    if (!(kSparse && kCausal) && t >= 2 && (last_h >> 1) == t && (last_h == 2 * t || !needs_lim(2 * t))) {
      // the last visible key of this lane's row, as an offset in half last_h
      // (the general path's limit; only keys below n_k, whose LDS rows hold
      // loaded data, stay visible)
      drain_lim = (kCausal ? min(qi, n_k - 1) : n_k - 1) - 32 * real_half(last_h);
      tile_drain(t, needs_lim(last_h));
      ++t;
    }
    for (; t < n_tiles; ++t) tile_general(t);
    // the last half tile's PV
    if (n_half >= 1 && n_half - 1 <= last_h) {
      if ((n_half - 1) & 1) compute_pv(stage_base(n_half - 1), 1, pB);
      else compute_pv(stage_base(n_half - 1), 0, pA);
    }

    // ---- rare fallback: some steady-state step of this wave had a partial
    // row sum above 2^32, i.e. a score far above the reference max, or an
    // overflow to +inf.  The steady state runs only with a finite reference,
    // so no NaN arises from finite inputs and the largest partial sum is a
    // plain non-negative number (compared as bits), +inf at worst.  Such a
    // wave recomputes its rows with an exact max on every half tile, reading
    // K and V from global memory (other waves may still be using the LDS
    // ring; this path takes no barrier).
    const bool stale = __builtin_bit_cast(unsigned, l_part_max) > kRedoBits ||
                       __builtin_bit_cast(unsigned, l_run) >= kInfBits;
    if constexpr (kSplit) {
      // Split kernels redo the piece instead: the whole workgroup, through
      // the same ring, with an exact max on every half tile (the general
      // path, whose partial sums stay small).  This keeps a second copy of
      // the pipeline's registers out of the piece loop.
      if (!exact && __any(stale) && lane == 0) sk_redo = 1;
      __syncthreads();
      const bool redo = __builtin_amdgcn_readfirstlane(*(volatile int*)&sk_redo) != 0;  // uniform
      __syncthreads();
      if (redo) {
        if (tid == 0) sk_redo = 0;
        exact = true;
        continue;
      }
    } else if (__any(stale)) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
      m_run = -INFINITY;
      l_run = 0.f;
      for (int j = 0; j <= last_h; ++j) {
        f32x16 s;
        {
          const int key = 32 * real_half(j) + l32;
          bf16x8 kop[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key < n) w = *(const u32x4*)(kg + (size_t)key * k_sn + 16 * ks + 8 * hi);
            kop[ks] = __builtin_bit_cast(bf16x8, w);
          }
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qop[0], zero16, 0, 0, 0);
#pragma unroll
          for (int ks = 1; ks < 4; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], s, 0, 0, 0);
        }
        if (needs_mask(j)) apply_mask(j, s);
        bf16x8 pop[2];
        bool raised;
        const float alpha = softmax_exact(s, pop, raised);
        if (raised) {
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            // V^T operand: element i is V[key(i)][32*db + l32], key(i) as in P^T
            bf16x8 vop;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int key = 32 * real_half(j) + 16 * tt + 8 * (i >> 2) + 4 * hi + (i & 3);
              const uint16_t bits = key < n ? vg[(size_t)key * v_sn + 32 * db + l32] : (uint16_t)0;
              vop[i] = __builtin_bit_cast(__bf16, bits);
            }
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[tt], acc[db], 0, 0, 0);
          }
      }
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.  A row that saw no
    // key (all hidden by the valid length or the mask) has l = +0 exactly: O = 0
    // and LSE = -inf, the empty sum.  The test is on the bits (l is a sum of
    // exp2 results: +0, positive or NaN), so a NaN row sum -- a NaN in a key or
    // query the row sees -- stays NaN in O and LSE (and no NaN-aware compare is
    // needed under -fno-honor-nans).
    //
    // A piece of a split tile first hands its partial (the unnormalised O^T
    // accumulators and each lane's m and l) to its slot; the last piece of
    // the tile to arrive merges all of them in piece order (the same sums
    // whichever piece merges) and writes O and LSE, the others are done.
    // The merge refers every piece to the largest m: O = sum_p 2^(m_p - m)
    // O_p and l likewise (the tiling identity of the online softmax); an
    // empty piece has m_p = -inf, weight 0, and if every piece is empty the
    // row is empty (m = -inf, l = +0).
    bool write_out = true;
    if constexpr (kSplit) {
      const int id = __builtin_amdgcn_readfirstlane(*(volatile int*)&sk_range);  // uniform
      if (id >= 0) pz = split_piece(split_range(a, id), pc);
      if (pz.parts > 1) {
        // Visibility across workgroups (possibly on other XCDs) without any
        // cache-wide maintenance: partials are written and read with the sc1
        // policy (agent-coherent: written through the XCD's L2, read from the
        // coherent level), and a writer's stores have completed before the
        // barrier that precedes its counter increment; the merger reads only
        // after seeing the count.  (Agent-scope fences would write back and
        // invalidate the XCD's whole L2 instead, evicting the K/V tiles its
        // other workgroups are streaming.)
        constexpr int kSc1 = 16;
        const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            a.ws_part, (short)0, 16 * a.sk_cus * kSplitSlotFloats * 4, kBufferWord3);
        auto slot_bytes = [&](int k) -> int {
          return (pz.slot_first + 2 * k + (k == 0 ? pz.ord0 : 0)) * kSplitSlotFloats * 4;
        };
        const int acc_lane = (wave * 8 * 64 + lane) * 16;  // chunk ch at + ch * 1024
        const int ml_lane = kSplitAccFloats * 4 + (wave * 64 + lane) * 8;
        const int own = slot_bytes(pz.part);
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          const int db = ch >> 2, r = 4 * (ch & 3);
          const f32x4 v4 = {acc[db][r], acc[db][r + 1], acc[db][r + 2], acc[db][r + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), ws_rsrc, own + acc_lane + ch * 1024, 0,
                                                 kSc1);
        }
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{m_run, l_run}), ws_rsrc, own + ml_lane, 0,
                                              kSc1);
        vm_wait_barrier<0>();  // this workgroup's partial has landed
        if (tid == 0)
          sk_arrived = __hip_atomic_fetch_add(a.ws_count + pz.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        write_out = __builtin_amdgcn_readfirstlane(sk_arrived) == pz.parts - 1;  // uniform
        if (write_out) {
          float mm = -INFINITY;
          for (int k = 0; k < pz.parts; ++k) {
            const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(ws_rsrc, slot_bytes(k) + ml_lane, 0, kSc1);
            mm = fmaxf(mm, __builtin_bit_cast(float, ml[0]));
          }
          const float msub = mm == -INFINITY ? 0.f : mm;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
          float ls = 0.f;
          for (int k = 0; k < pz.parts; ++k) {
            const int sb = slot_bytes(k);
            const f32x2 ml = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(ws_rsrc, sb + ml_lane, 0, kSc1));
            const float w = __builtin_amdgcn_exp2f(ml[0] - msub);
            ls = __builtin_fmaf(w, ml[1], ls);
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
              const f32x4 v4 = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(ws_rsrc, sb + acc_lane + ch * 1024, 0, kSc1));
              const int db = ch >> 2, r = 4 * (ch & 3);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[db][r + i] = __builtin_fmaf(w, v4[i], acc[db][r + i]);
            }
          }
          m_run = mm;
          l_run = ls;
          // leave the counter at zero for the next call
          if (tid == 0) __hip_atomic_store(a.ws_count + pz.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    const float l_tot = half_swap_sum(l_run);
    const bool empty_row = __builtin_bit_cast(unsigned, l_tot) == 0u;
    if (write_out && qi < n) {
      const float inv = empty_row ? 0.f : 1.f / l_tot;
      uint16_t* orow = a.o + head_off(3) + (size_t)qi * a.sn[3];
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int f0 = 32 * db + 8 * r4 + 4 * hi;
          const bf16x2 p01 = {(__bf16)(acc[db][4 * r4 + 0] * inv), (__bf16)(acc[db][4 * r4 + 1] * inv)};
          const bf16x2 p23 = {(__bf16)(acc[db][4 * r4 + 2] * inv), (__bf16)(acc[db][4 * r4 + 3] * inv)};
          u32x2 w = {__builtin_bit_cast(unsigned, p01), __builtin_bit_cast(unsigned, p23)};
          *(u32x2*)(orow + f0) = w;
        }
      }
      if (hi == 0) a.lse[(size_t)bh * n + qi] = empty_row ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
    }
    if constexpr (!kSplit) break;
    exact = false;
    if (++pc >= n_pieces) break;
  }
}

// ---------------------------------------------------------------- fp32 path

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int n;
  int q_tiles;  // ceil(n / kF32Rows)
  float scale;
  int causal;
  int heads;
  const int* key_len;         // [B] or null
  const uint32_t* key_bits;   // [B][ceil(N/32)] or null
};

constexpr int kF32Keys = 8;   // keys per LDS tile in the fp32 kernel
constexpr int kF32Rows = 64;  // query rows per workgroup (two waves)
constexpr int kF32Half = kD / 2;

// x[lane] + x[lane ^ 32] in both lanes of the pair, summed in the same order
// (the lower half's value first), so the two lanes get the same bits.
__device__ __forceinline__ double pair_sum_f64(double x) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = (unsigned)u, hi = (unsigned)(u >> 32);
  const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  // after the swap each element holds one lane's word, the same lane's in both lanes of the pair
  const double a = __builtin_bit_cast(double, ((unsigned long long)(unsigned)rh[0] << 32) | (unsigned)rl[0]);
  const double b = __builtin_bit_cast(double, ((unsigned long long)(unsigned)rh[1] << 32) | (unsigned)rl[1]);
  return a + b;
}

// Two lanes per query row: lane l of a wave owns row l % 32 of the wave's 32
// and features [32 * (l / 32), +32) of its Q row and of its O accumulators,
// so the partial dot products meet in one exchange with lane l ^ 32.
__global__ void __launch_bounds__(2 * 64) attn_fwd_f32_kernel(F32Args a) {
  __shared__ float4 ks[kF32Keys][kD / 4];
  __shared__ float4 vs[kF32Keys][kD / 4];
  const int n = a.n;
  const int bh = blockIdx.x / a.q_tiles;
  const int qt = blockIdx.x - bh * a.q_tiles;
  const size_t head = (size_t)bh * n * kD;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;  // which 32 features this lane holds
  const int qi = qt * kF32Rows + (threadIdx.x >> 6) * 32 + (lane & 31);
  const bool live = qi < n;

  // Scores, the running max and t - m are kept in fp64: a 64-term fp32 dot
  // product and the rounding of s * c would each cost about 2^-24 * |s| in
  // the exponent, i.e. ~1e-5 in O and LSE once |s| reaches ~30 (a large
  // scale); in fp64 the products of fp32 values are exact and only the
  // small difference t - m is rounded to fp32 for exp2.  O's accumulators
  // and the row sum l are fp64 too: with up to N terms of mixed sign in
  // fp32, their rounding reaches ~4e-6 of |O| on sharp rows (l alone
  // ~3e-6), i.e. 1e-5 once |O| is a few units.
  float qv[kF32Half];
  double acc[kF32Half];
  // loads past N read row N - 1 and are replaced by zeros (a select, so no
  // load is predicated)
  const float* const qrow = a.q + head + (size_t)min(qi, n - 1) * kD + half * kF32Half;
#pragma unroll
  for (int f = 0; f < kF32Half; f += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qrow + f);
    qv[f] = live ? x.x : 0.f;
    qv[f + 1] = live ? x.y : 0.f;
    qv[f + 2] = live ? x.z : 0.f;
    qv[f + 3] = live ? x.w : 0.f;
  }
#pragma unroll
  for (int f = 0; f < kF32Half; ++f) acc[f] = 0.0;
  const double c = (double)a.scale * 1.4426950408889634;  // log2(e)
  double m_run = -INFINITY;
  double l_run = 0.0;
  const int b_entry = bh / a.heads;
  const int n_k = a.key_len ? min(max(a.key_len[b_entry], 0), n) : n;
  const uint32_t* const mask_row = a.key_bits ? a.key_bits + (size_t)b_entry * ((n + 31) / 32) : nullptr;
  const int kv_end = a.causal ? min(n_k, qt * kF32Rows + kF32Rows) : n_k;
  const int row_last = a.causal ? min(qi, n_k - 1) : n_k - 1;
  // the tile load: thread t moves 16 bytes of K and of V, row t / 16, chunk
  // t % 16; the next tile's chunks travel while this tile is computed
  static_assert(kF32Keys * kD / 4 == 2 * 64, "one 16-byte chunk of K and of V per thread");
  const int ld_r = threadIdx.x >> 4, ld_c = threadIdx.x & 15;
  float4 kx, vx;
  auto load_chunks = [&](int k0) __attribute__((always_inline)) {
    const size_t off = head + (size_t)min(k0 + ld_r, n - 1) * kD + ld_c * 4;
    kx = *reinterpret_cast<const float4*>(a.k + off);
    vx = *reinterpret_cast<const float4*>(a.v + off);
  };
  if (kv_end > 0) load_chunks(0);

  for (int k0 = 0; k0 < kv_end; k0 += kF32Keys) {
    __syncthreads();
    {
      const bool in = k0 + ld_r < n;
      ks[ld_r][ld_c] = make_float4(in ? kx.x : 0.f, in ? kx.y : 0.f, in ? kx.z : 0.f, in ? kx.w : 0.f);
      vs[ld_r][ld_c] = make_float4(in ? vx.x : 0.f, in ? vx.y : 0.f, in ? vx.z : 0.f, in ? vx.w : 0.f);
    }
    __syncthreads();
    if (k0 + kF32Keys < kv_end) load_chunks(k0 + kF32Keys);
    double t[kF32Keys];
    double mx = -INFINITY;
    uint32_t seen = 0;  // bit r: key k0 + r takes part in this row
    // the tile's keys are a quarter of one mask word (k0 is a multiple of 8, k0 < N)
    static_assert(32 % kF32Keys == 0, "a key tile within one mask word");
    const uint32_t word = mask_row ? mask_row[k0 >> 5] >> (k0 & 31) : 0xffffffffu;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      double part = 0.0;
#pragma unroll
      for (int f4 = 0; f4 < kF32Half / 4; ++f4) {
        const float4 kk = ks[r][half * (kF32Half / 4) + f4];
        part = __builtin_fma((double)qv[4 * f4], (double)kk.x, part);
        part = __builtin_fma((double)qv[4 * f4 + 1], (double)kk.y, part);
        part = __builtin_fma((double)qv[4 * f4 + 2], (double)kk.z, part);
        part = __builtin_fma((double)qv[4 * f4 + 3], (double)kk.w, part);
      }
      const double s = pair_sum_f64(part);
      const bool vis = k0 + r <= row_last && ((word >> r) & 1u);
      seen |= (vis ? 1u : 0u) << r;
      t[r] = vis ? s * c : -INFINITY;
      mx = fmax(mx, t[r]);
    }
    const double m_new = fmax(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((float)(m_run - m_new));
    const double msub = (m_new == -INFINITY) ? 0.0 : m_new;
    m_run = m_new;
    l_run *= (double)alpha;
#pragma unroll
    for (int f = 0; f < kF32Half; ++f) acc[f] *= (double)alpha;
    // a hidden key takes no part: its V row is skipped, not multiplied by
    // p = 0 (so a non-finite value there cannot reach this row)
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      if (!((seen >> r) & 1u)) continue;
      const double p = __builtin_amdgcn_exp2f((float)(t[r] - msub));
      l_run += p;
#pragma unroll
      for (int f4 = 0; f4 < kF32Half / 4; ++f4) {
        const float4 vv = vs[r][half * (kF32Half / 4) + f4];
        acc[4 * f4] = __builtin_fma(p, (double)vv.x, acc[4 * f4]);
        acc[4 * f4 + 1] = __builtin_fma(p, (double)vv.y, acc[4 * f4 + 1]);
        acc[4 * f4 + 2] = __builtin_fma(p, (double)vv.z, acc[4 * f4 + 2]);
        acc[4 * f4 + 3] = __builtin_fma(p, (double)vv.w, acc[4 * f4 + 3]);
      }
    }
  }
  if (live) {
    // a row that saw no key: O = 0, LSE = -inf (the empty sum); l is +0,
    // positive or NaN, and a NaN stays NaN (the test is on the bits)
    const bool empty_row = __builtin_bit_cast(unsigned long long, l_run) == 0ull;
    const double inv = empty_row ? 0.0 : 1.0 / l_run;
    float* const orow = a.o + head + (size_t)qi * kD + half * kF32Half;
#pragma unroll
    for (int f = 0; f < kF32Half; f += 4)
      *reinterpret_cast<float4*>(orow + f) = make_float4((float)(acc[f] * inv), (float)(acc[f + 1] * inv),
                                                         (float)(acc[f + 2] * inv), (float)(acc[f + 3] * inv));
    if (half == 0)
      a.lse[(size_t)bh * n + qi] = empty_row ? -INFINITY
                                             : (float)((m_run + (double)__log2f((float)l_run)) * 0.6931471805599453);
  }
}

// ------------------------------------------------------- key mask packing

// Bit j%32 of word j/32 of row b = (key_valid[b][j] != 0); bits past N are 0.
// One thread per output word.
__global__ void __launch_bounds__(256) attn_pack_key_mask_kernel(const uint8_t* key_valid,
                                                                 uint32_t* key_bits, int n,
                                                                 int words, long long total) {
  const long long w = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= total) return;
  const int b = (int)(w / words);
  const int j0 = (int)(w - (long long)b * words) * 32;
  const uint8_t* row = key_valid + (size_t)b * n;
  uint32_t bits = 0;
  const int cnt = min(32, n - j0);
  for (int i = 0; i < cnt; ++i) bits |= (row[j0 + i] != 0 ? 1u : 0u) << i;
  key_bits[w] = bits;
}

// ---------------------------------------------------------------- host side

}  // namespace

namespace attn_detail {

constexpr int kMaxDevices = 64;
// 0 = not checked, 1 = gfx950, 2 = other architecture
int g_arch_state[kMaxDevices];
int g_cu_count[kMaxDevices];  // compute units of the device (of its partition)

attn_status check_device(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return ATTN_E_DEVICE;
  }
  int state = __atomic_load_n(&g_arch_state[dev], __ATOMIC_ACQUIRE);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return ATTN_E_DEVICE;
    }
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    __atomic_store_n(&g_cu_count[dev], prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                     __ATOMIC_RELAXED);
    __atomic_store_n(&g_arch_state[dev], state, __ATOMIC_RELEASE);
  }
  if (cus) *cus = __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED);
  return state == 1 ? ATTN_OK : ATTN_E_DEVICE;
}

}  // namespace attn_detail

namespace {

attn_status validate(const void* q, const void* k, const void* v, const void* o, const void* lse,
                     int B, int H, int N, int d, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_INVALID;
  if (B < 1 || H < 1 || N < 1 || d != kD || !std::isfinite(scale)) return ATTN_E_INVALID;
  if (!sizes_fit(B, H, N)) return ATTN_E_INVALID;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
      misaligned(lse, 4))
    return ATTN_E_ALIGN;
  return ATTN_OK;
}

// Element strides (batch, head, row) of the four tensors, checked: every
// stride a multiple of 8 elements (16 bytes; the kernel moves 16-byte
// chunks), none negative, o's rows at least 64 apart, and every byte offset
// the K/V buffer loads form below 2^31.  NULL layouts are the contiguous
// [B][H][N][64] one.
attn_status check_layouts(const attn_layout* const lay[4], int H, int N, long long sb[4],
                          long long sh[4], int sn[4]) {
  for (int t = 0; t < 4; ++t) {
    if (!lay[t]) {
      sn[t] = kD;
      sh[t] = (long long)N * kD;
      sb[t] = (long long)H * N * kD;
      continue;
    }
    const attn_layout& l = *lay[t];
    if (l.batch < 0 || l.head < 0 || l.row < 0) return ATTN_E_INVALID;
    if ((l.batch | l.head | l.row) & 7) return ATTN_E_ALIGN;
    if (l.row > (1LL << 24)) return ATTN_E_INVALID;
    sb[t] = l.batch;
    sh[t] = l.head;
    sn[t] = (int)l.row;
  }
  if (sn[3] < kD) return ATTN_E_INVALID;  // o's rows must not overlap
  for (int t = 1; t <= 2; ++t)
    if ((long long)(N - 1) * 2 * sn[t] + kRow >= (1LL << 31)) return ATTN_E_INVALID;
  return ATTN_OK;
}

attn_status launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, float scale, int causal, const int* key_len,
                        const uint32_t* key_bits, void* stream,
                        const attn_layout* const layouts[4] = nullptr,
                        const uint8_t* block_mask = nullptr, bool allow_split = false,
                        void* workspace = nullptr, size_t workspace_bytes = 0) {
  attn_status st = validate(q, k, v, o, lse, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if (misaligned(key_len, 4) || misaligned(key_bits, 4) || misaligned(workspace, 256)) return ATTN_E_ALIGN;
  long long sb[4], sh[4];
  int sn[4];
  const attn_layout* const none[4] = {nullptr, nullptr, nullptr, nullptr};
  st = check_layouts(layouts ? layouts : none, H, N, sb, sh, sn);
  if (st != ATTN_OK) return st;
  if (block_mask && (key_bits || N > kSparseBlockK * kMaxSparseTiles)) return ATTN_E_INVALID;
  int cus = 0;
  st = check_device(&cus);
  if (st != ATTN_OK) return st;

  Bf16Args a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.n = N;
  // Non-causal: 8-wave workgroups (256 rows, one per CU) when they give
  // every CU at least one; otherwise 4-wave ones, twice as many (a short
  // sequence over few heads would leave CUs idle).
  // Through attn_fwd_split, a non-causal dense call may instead split the
  // key tiles of its last, partial round of 8-wave workgroups (plan_split).
  const long long tiles8 = (long long)B * H * ((N + kWavesFull * 32 - 1) / (kWavesFull * 32));
  const int n_kt = (N + kBc - 1) / kBc;
  const SplitPlan sp = allow_split && !causal && !block_mask && kWavesFull == 8 ? plan_split(tiles8, n_kt, cus)
                                                                                : SplitPlan{false, false, 0, 1};
  if (sp.on && (!workspace || workspace_bytes < split_workspace_bytes(cus))) return ATTN_E_INVALID;
  const bool few = !sp.on && tiles8 < cus;
  const int waves = block_mask ? kSparseBlockQ / 32 : causal ? kWavesCausal : few ? 4 : kWavesFull;
  const int rows = waves * 32;
  a.q_tiles = (N + rows - 1) / rows;
  a.block_mask = block_mask;
  a.mask_cols = (N + kSparseBlockK - 1) / kSparseBlockK;
  a.total_tiles = B * H * a.q_tiles;
  // c must be > 0: masked scores are -inf and fma(-inf, c, -m) must stay
  // -inf.  A zero (or denormal) scale becomes FLT_MIN, whose scores differ by
  // far less than one fp32 ulp of exp2's result, i.e. the same uniform rows.
  a.c = std::fmax(std::fabs(scale) * kLog2e, 1.17549435e-38f);
  a.q_sign = scale < 0.f ? 0x80008000u : 0u;
  a.heads = H;
  for (int t = 0; t < 4; ++t) {
    a.sb[t] = sb[t];
    a.sh[t] = sh[t];
    a.sn[t] = sn[t];
  }
  a.key_len = key_len;
  a.key_bits = key_bits;
  int grid = a.total_tiles;
  a.dp_blocks = grid;
  a.sk_rounds = 0;
  a.sk_cus = 1;
  a.n_kt = n_kt;
  a.ws_count = nullptr;
  a.ws_part = nullptr;
  if (sp.on) {
    // whole rounds first (xcd_remap sends workgroup w < dp_blocks to local
    // tile w / 8 < R*C of XCD w % 8), then per XCD C workgroups, one per
    // range of the leftover
    a.sk_rounds = sp.rounds;
    a.sk_cus = sp.cus_per_xcd;
    a.dp_blocks = 8 * sp.rounds * sp.cus_per_xcd;
    grid = a.dp_blocks + 8 * sp.cus_per_xcd;
    a.ws_count = static_cast<int*>(workspace);
    a.ws_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_count_bytes(cus));
  }

  void* args[] = {&a};
  const void* fn;
  if (block_mask)
    fn = causal ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<true, 4, false, true, false>)
                : reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, 4, false, true, false>);
  else if (key_bits)
    fn = causal  ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<true, kWavesCausal, true, false, false>)
         : sp.on ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, 8, true, false, true>)
         : few   ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, 4, true, false, false>)
                 : reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, kWavesFull, true, false, false>);
  else
    fn = causal  ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<true, kWavesCausal, false, false, false>)
         : sp.on ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, 8, false, false, true>)
         : few   ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, 4, false, false, false>)
                 : reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false, kWavesFull, false, false, false>);
  const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(waves * 64), args, 0,
                                       static_cast<hipStream_t>(stream));
  return launch_status(e);
}

attn_status launch_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal, const int* key_len,
                        const uint32_t* key_bits, void* stream) {
  attn_status st = validate(q, k, v, o, lse, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if (misaligned(key_len, 4) || misaligned(key_bits, 4)) return ATTN_E_ALIGN;
  st = check_device();
  if (st != ATTN_OK) return st;

  F32Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.n = N;
  a.q_tiles = (N + kF32Rows - 1) / kF32Rows;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.heads = H;
  a.key_len = key_len;
  a.key_bits = key_bits;
  void* args[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_f32_kernel),
                                       dim3(B * H * a.q_tiles), dim3(2 * 64), args, 0,
                                       static_cast<hipStream_t>(stream));
  return launch_status(e);
}

}  // namespace

extern "C" attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, int d, float scale, int causal,
                                void* stream) {
  return launch_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, nullptr, nullptr, stream);
}

extern "C" attn_status attn_fwd_fp32(const float* q, const float* k, const float* v, float* o,
                                     float* lse, int B, int H, int N, int d, float scale,
                                     int causal, void* stream) {
  return launch_fp32(q, k, v, o, lse, B, H, N, d, scale, causal, nullptr, nullptr, stream);
}

extern "C" attn_status attn_fwd_masked(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int H, int N, int d, float scale,
                                       int causal, const int* key_len, const unsigned* key_bits,
                                       void* stream) {
  return launch_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, key_bits, stream);
}

extern "C" attn_status attn_fwd_fp32_masked(const float* q, const float* k, const float* v,
                                            float* o, float* lse, int B, int H, int N, int d,
                                            float scale, int causal, const int* key_len,
                                            const unsigned* key_bits, void* stream) {
  return launch_fp32(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, key_bits, stream);
}

extern "C" attn_status attn_fwd_strided(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int B, int H, int N, int d, float scale,
                                        int causal, const attn_layout* q_layout,
                                        const attn_layout* k_layout, const attn_layout* v_layout,
                                        const attn_layout* o_layout, const int* key_len,
                                        const unsigned* key_bits, void* stream) {
  const attn_layout* const layouts[4] = {q_layout, k_layout, v_layout, o_layout};
  return launch_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, key_bits, stream, layouts);
}

extern "C" attn_status attn_fwd_split(const void* q, const void* k, const void* v, void* o,
                                      float* lse, int B, int H, int N, int d, float scale,
                                      int causal, const attn_layout* q_layout,
                                      const attn_layout* k_layout, const attn_layout* v_layout,
                                      const attn_layout* o_layout, const int* key_len,
                                      const unsigned* key_bits, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const attn_layout* const layouts[4] = {q_layout, k_layout, v_layout, o_layout};
  return launch_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, key_bits, stream, layouts,
                     nullptr, true, workspace, workspace_bytes);
}

extern "C" attn_status attn_fwd_split_workspace_size(int B, int H, int N, int causal, size_t* bytes) {
  if (!bytes || B < 1 || H < 1 || N < 1 || !sizes_fit(B, H, N)) return ATTN_E_INVALID;
  int cus = 0;
  const attn_status st = check_device(&cus);
  if (st != ATTN_OK) return st;
  const long long tiles8 = (long long)B * H * ((N + kWavesFull * 32 - 1) / (kWavesFull * 32));
  const bool on = !causal && kWavesFull == 8 && plan_split(tiles8, (N + kBc - 1) / kBc, cus).on;
  *bytes = on ? split_workspace_bytes(cus) : 0;
  return ATTN_OK;
}

extern "C" attn_status attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o,
                                             float* lse, int B, int H, int N, int d, float scale,
                                             int causal, const unsigned char* block_mask,
                                             void* stream) {
  if (!block_mask) return ATTN_E_INVALID;
  return launch_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, nullptr, nullptr, stream, nullptr,
                     block_mask);
}

extern "C" attn_status attn_pack_key_mask(const unsigned char* key_valid, unsigned* key_bits,
                                          int B, int N, void* stream) {
  if (!key_valid || !key_bits || B < 1 || N < 1) return ATTN_E_INVALID;
  if (!sizes_fit(B, 1, N)) return ATTN_E_INVALID;
  if (misaligned(key_bits, 4)) return ATTN_E_ALIGN;
  const attn_status st = check_device();
  if (st != ATTN_OK) return st;
  const int words = (N + 31) / 32;
  const long long total = (long long)B * words;
  const int blocks = (int)((total + 255) / 256);
  const uint8_t* kv = key_valid;
  uint32_t* kb = key_bits;
  int n = N;
  void* args[] = {&kv, &kb, &n, (void*)&words, (void*)&total};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_pack_key_mask_kernel),
                                       dim3(blocks), dim3(256), args, 0,
                                       static_cast<hipStream_t>(stream));
  return launch_status(e);
}

extern "C" const char* attn_strerror(attn_status s) {
  switch (s) {
    case ATTN_OK: return "success";
    case ATTN_E_INVALID: return "invalid argument (null pointer, size out of range, d != 64 or non-finite scale)";
    case ATTN_E_ALIGN: return "misaligned pointer (q, k, v, o need 16 bytes, lse 4 bytes)";
    case ATTN_E_DEVICE: return "no usable device (no HIP device current, or it is not gfx950)";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_SCRATCH:
      return "the call needs more than the static scratch of attn_bwd_noalloc (16 MiB: 8*B*H*ceil(N/256)*256 bytes)";
  }
  return "unknown status";
}
