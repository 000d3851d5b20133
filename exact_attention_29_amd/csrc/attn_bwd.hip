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
//   1. bwd_delta: D_i = sum_f dO_if O_if (fp32, one thread per row) into the
//      caller's [B][H][N] scratch;
//   2. bwd_dkdv (key-parallel): a workgroup owns 128 keys (4 waves x 32);
//      each wave keeps K and V of its keys in registers as MFMA operands and
//      streams 64-query tiles of Q, dO, LSE and D through double-buffered
//      LDS.  It computes S = Q K^T in the layout where each lane holds one
//      key and 16 queries: P and dS then feed dV^T += dO^T P and
//      dK^T += Q^T dS directly as MFMA operands, and the transposed Q / dO
//      operands come from the row-major tiles with ds_read_b64_tr_b16;
//   3. bwd_dq (query-parallel): a workgroup owns 128 queries; each wave keeps
//      Q and dO of its rows in registers and streams 64-key tiles of K and V:
//      S^T = K Q^T and dP^T = V dO^T (a lane per query), dS^T, then
//      dQ^T += K^T dS^T.
// No atomics: every output element is written by exactly one lane, so the
// result is deterministic.  All products on v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation; P and dS are rounded to bf16 for the products, as in
// the forward pass.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

constexpr int kBwdWaves = 4;              // waves per workgroup
constexpr int kBwdRows = kBwdWaves * 32;  // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kBwdTile = 64;              // rows of a streamed tile
constexpr int kBwdTileBytes = kBwdTile * kRow;

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int n;
  int blocks;  // ceil(n / kBwdRows)
  int total;   // B * H * blocks
  float c;     // scale * log2(e)
  float scale;
  int causal;
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D_i = sum_f dO_if O_if for every row i of every head.
__global__ void __launch_bounds__(256) bwd_delta_kernel(BwdArgs a, long long rows) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const u32x4* po = (const u32x4*)(a.o + r * kD);
  const u32x4* pd = (const u32x4*)(a.dout + r * kD);
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
  a.delta[r] = acc;
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

// ------------------------------------------------------------------ dK, dV

template <bool kCausal>
__global__ void __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkdv_kernel(BwdArgs a) {
  // double-buffered tiles: Q, dO (64 rows each, swizzled), LSE*log2(e), D
  __shared__ __attribute__((aligned(1024))) char qs[2][kBwdTileBytes];
  __shared__ __attribute__((aligned(1024))) char dos[2][kBwdTileBytes];
  __shared__ __attribute__((aligned(16))) float ls[2][kBwdTile];
  __shared__ __attribute__((aligned(16))) float ds_[2][kBwdTile];

  const int n = a.n;
  const int logical = xcd_remap(blockIdx.x, a.total);
  const int bh = logical / a.blocks;
  const int kb = logical - bh * a.blocks;
  const size_t head = (size_t)bh * n * kD;
  const uint16_t* qg = a.q + head;
  const uint16_t* kg = a.k + head;
  const uint16_t* vg = a.v + head;
  const uint16_t* dog = a.dout + head;
  const float* lseg = a.lse + (size_t)bh * n;
  const float* dg = a.delta + (size_t)bh * n;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int key0 = kb * kBwdRows + wave * 32;  // this wave's first key
  const int key = key0 + l32;                  // this lane's key

  // K^T and V^T operands (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kop[4], vop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kop[ks] = row_operand(kg, key, ks, hi, n);
    vop[ks] = row_operand(vg, key, ks, hi, n);
  }
  const TrOffsets tr(lane);

  // query tiles: all of them, or (causal) from the one holding this
  // workgroup's first key
  const int t_begin = kCausal ? (kb * kBwdRows) / kBwdTile : 0;
  const int t_end = (n + kBwdTile - 1) / kBwdTile;

  // staging: thread tid moves chunks tid and tid + 256 of the Q and dO tiles
  // (row = chunk / 8, chunk position chunk % 8) and one LSE or D value
  u32x4 stq[2], std_[2];
  float stl = 0.f;
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cidx = tid + 256 * i, row = t * kBwdTile + (cidx >> 3), ch = cidx & 7;
      stq[i] = load_chunk(qg, row, ch, n);
      std_[i] = load_chunk(dog, row, ch, n);
    }
    if (tid < 128) {
      const int row = t * kBwdTile + (tid & 63);
      // rows past N: LSE = +inf makes their probabilities exactly 0
      if (tid < 64) stl = row < n ? lseg[row] * kLog2e : INFINITY;
      else stl = row < n ? dg[row] : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 3, ch = cidx & 7;
      *(u32x4*)(qs[buf] + tile_off(row, ch)) = stq[i];
      *(u32x4*)(dos[buf] + tile_off(row, ch)) = std_[i];
    }
    if (tid < 64) ls[buf][tid] = stl;
    else if (tid < 128) ds_[buf][tid - 64] = stl;
  };

  f32x16 acc_dk[2], acc_dv[2];  // dK^T, dV^T: rows = features, columns = keys
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_dk[db][r] = acc_dv[db][r] = 0.f;
  const f32x16 zero16 = {};
  const float c = a.c;

  if (t_begin < t_end) {
    fetch(t_begin);
    store(0);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    if (t + 1 < t_end) fetch(t + 1);
    const char* qt = qs[buf];
    const char* dt = dos[buf];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 32-query halves of the tile
      const int q0 = t * kBwdTile + 32 * j;
      // causal: a half tile of queries before this wave's keys adds nothing
      // (every key is hidden from every query); the one that starts at the
      // wave's first key is the diagonal, the only one masked per element
      if (kCausal && q0 < key0) continue;
      const bool diag = kCausal && q0 == key0;
      // S = Q K^T and dP = dO V^T: lane = key, register r = query
      // q0 + 8*(r/4) + 4*hi + r%4
      f32x16 s = zero16, dp = zero16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = tile_off(32 * j + l32, 2 * ks + hi);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(qt, off), kop[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(dt, off), vop[ks], dp, 0, 0, 0);
      }
      // P = exp2(c s - LSE log2 e), dS = P (dP - D)
      float p[16], dd[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qr = 32 * j + 8 * g4 + 4 * hi;  // tile row of register 4*g4
        const float4 l4 = *(const float4*)&ls[buf][qr];
        const float4 d4 = *(const float4*)&ds_[buf][qr];
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        dd[4 * g4] = d4.x, dd[4 * g4 + 1] = d4.y, dd[4 * g4 + 2] = d4.z, dd[4 * g4 + 3] = d4.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * g4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g4 + e], c, -lv[e]));
      }
      if (diag) {  // wave-uniform: key > query hidden
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (l32 > 8 * (r >> 2) + 4 * hi + (r & 3)) p[r] = 0.f;
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const bf16x2 pp = {(__bf16)p[r], (__bf16)p[r + 1]};
        const bf16x2 dq2 = {(__bf16)(p[r] * (dp[r] - dd[r])), (__bf16)(p[r + 1] * (dp[r + 1] - dd[r + 1]))};
        pb[r >> 3][r & 7] = pp[0];
        pb[r >> 3][(r & 7) + 1] = pp[1];
        dsb[r >> 3][r & 7] = dq2[0];
        dsb[r >> 3][(r & 7) + 1] = dq2[1];
      }
      // dV^T += dO^T P, dK^T += Q^T dS (k index i of half tt <-> query
      // q0 + 16*tt + 8*(i/4) + 4*hi + i%4, matched by the transposed reads)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int rb = (32 * j + 16 * tt) * kRow;
          const bf16x8 dot = lds_read_vt(dt + rb + tr.off[0][db], dt + rb + tr.off[1][db]);
          const bf16x8 qtr = lds_read_vt(qt + rb + tr.off[0][db], qt + rb + tr.off[1][db]);
          acc_dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot, pb[tt], acc_dv[db], 0, 0, 0);
          acc_dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtr, dsb[tt], acc_dk[db], 0, 0, 0);
        }
    }
    if (t + 1 < t_end) store(buf ^ 1);
    __syncthreads();
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
        const bf16x2 k01 = {(__bf16)(acc_dk[db][4 * r4] * scale), (__bf16)(acc_dk[db][4 * r4 + 1] * scale)};
        const bf16x2 k23 = {(__bf16)(acc_dk[db][4 * r4 + 2] * scale), (__bf16)(acc_dk[db][4 * r4 + 3] * scale)};
        const bf16x2 v01 = {(__bf16)acc_dv[db][4 * r4], (__bf16)acc_dv[db][4 * r4 + 1]};
        const bf16x2 v23 = {(__bf16)acc_dv[db][4 * r4 + 2], (__bf16)acc_dv[db][4 * r4 + 3]};
        *(u32x2*)(dkrow + f0) = u32x2{__builtin_bit_cast(unsigned, k01), __builtin_bit_cast(unsigned, k23)};
        *(u32x2*)(dvrow + f0) = u32x2{__builtin_bit_cast(unsigned, v01), __builtin_bit_cast(unsigned, v23)};
      }
  }
}

// ---------------------------------------------------------------------- dQ

template <bool kCausal>
__global__ void __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char ks_[2][kBwdTileBytes];
  __shared__ __attribute__((aligned(1024))) char vs_[2][kBwdTileBytes];

  const int n = a.n;
  const int logical = xcd_remap(blockIdx.x, a.total);
  const int bh = logical / a.blocks;
  int qb = logical - bh * a.blocks;
  if (kCausal) qb = a.blocks - 1 - qb;  // longest rows first
  const size_t head = (size_t)bh * n * kD;
  const uint16_t* qg = a.q + head;
  const uint16_t* kg = a.k + head;
  const uint16_t* vg = a.v + head;
  const uint16_t* dog = a.dout + head;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0w = qb * kBwdRows + wave * 32;  // this wave's first query
  const int qi = q0w + l32;                    // this lane's query

  // Q^T and dO^T operands (B operands of S^T = K Q^T and dP^T = V dO^T)
  bf16x8 qop[4], dop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qop[ks] = row_operand(qg, qi, ks, hi, n);
    dop[ks] = row_operand(dog, qi, ks, hi, n);
  }
  const float lse2 = qi < n ? a.lse[(size_t)bh * n + qi] * kLog2e : INFINITY;
  const float dlt = qi < n ? a.delta[(size_t)bh * n + qi] : 0.f;
  const TrOffsets tr(lane);

  const int q_last = min(n - 1, qb * kBwdRows + kBwdRows - 1);
  const int kv_end = kCausal ? q_last + 1 : n;
  const int t_end = (kv_end + kBwdTile - 1) / kBwdTile;

  u32x4 stk[2], stv[2];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cidx = tid + 256 * i, row = t * kBwdTile + (cidx >> 3), ch = cidx & 7;
      stk[i] = load_chunk(kg, row, ch, n);
      stv[i] = load_chunk(vg, row, ch, n);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 3, ch = cidx & 7;
      *(u32x4*)(ks_[buf] + tile_off(row, ch)) = stk[i];
      *(u32x4*)(vs_[buf] + tile_off(row, ch)) = stv[i];
    }
  };

  f32x16 acc[2];  // dQ^T: rows = features, columns = queries
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const f32x16 zero16 = {};
  const float c = a.c;

  if (t_end > 0) {
    fetch(0);
    store(0);
  }
  __syncthreads();
  for (int t = 0; t < t_end; ++t) {
    const int buf = t & 1;
    if (t + 1 < t_end) fetch(t + 1);
    const char* kt = ks_[buf];
    const char* vt = vs_[buf];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 32-key halves of the tile
      const int k0 = t * kBwdTile + 32 * j;
      // causal: keys past this wave's last query add nothing; the half tile
      // that starts at the wave's first query is the diagonal.  Only the
      // diagonal and the ragged last half tile are masked per element.
      if (kCausal && k0 > q0w) continue;
      const bool diag = kCausal && k0 == q0w;
      const bool ragged = k0 + 32 > n;
      // S^T = K Q^T, dP^T = V dO^T: lane = query, register r = key
      // k0 + 8*(r/4) + 4*hi + r%4
      f32x16 s = zero16, dp = zero16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = tile_off(32 * j + l32, 2 * ks + hi);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(kt, off), qop[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(vt, off), dop[ks], dp, 0, 0, 0);
      }
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
      if (diag || ragged) {  // wave-uniform: only these half tiles pay for masks
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 8 * (r >> 2) + 4 * hi + (r & 3);  // key - k0
          if ((diag && kr > l32) || k0 + kr >= n) p[r] = 0.f;
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const bf16x2 pr = {(__bf16)(p[r] * (dp[r] - dlt)), (__bf16)(p[r + 1] * (dp[r + 1] - dlt))};
        dsb[r >> 3][r & 7] = pr[0];
        dsb[r >> 3][(r & 7) + 1] = pr[1];
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int rb = (32 * j + 16 * tt) * kRow;
          const bf16x8 ktr = lds_read_vt(kt + rb + tr.off[0][db], kt + rb + tr.off[1][db]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktr, dsb[tt], acc[db], 0, 0, 0);
        }
    }
    if (t + 1 < t_end) store(buf ^ 1);
    __syncthreads();
  }

  if (qi < n) {
    uint16_t* row = a.dq + head + (size_t)qi * kD;
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f0 = 32 * db + 8 * r4 + 4 * hi;
        const bf16x2 p01 = {(__bf16)(acc[db][4 * r4] * scale), (__bf16)(acc[db][4 * r4 + 1] * scale)};
        const bf16x2 p23 = {(__bf16)(acc[db][4 * r4 + 2] * scale), (__bf16)(acc[db][4 * r4 + 3] * scale)};
        *(u32x2*)(row + f0) = u32x2{__builtin_bit_cast(unsigned, p01), __builtin_bit_cast(unsigned, p23)};
      }
  }
}

}  // namespace

extern "C" attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                float* delta, int B, int H, int N, int d, float scale, int causal,
                                void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return ATTN_E_INVALID;
  if (B < 1 || H < 1 || N < 1 || d != kD || !std::isfinite(scale)) return ATTN_E_INVALID;
  if ((long long)B * H * N * d >= (1LL << 31)) return ATTN_E_INVALID;
  const void* vec[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : vec)
    if (misaligned(p, 16)) return ATTN_E_ALIGN;
  if (misaligned(lse, 4) || misaligned(delta, 4)) return ATTN_E_ALIGN;
  const attn_status st = check_device();
  if (st != ATTN_OK) return st;

  BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.delta = delta;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.n = N;
  a.blocks = (N + kBwdRows - 1) / kBwdRows;
  a.total = B * H * a.blocks;
  a.c = scale * kLog2e;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);

  long long rows = (long long)B * H * N;
  void* dargs[] = {&a, &rows};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_delta_kernel),
                                 dim3((unsigned)((rows + 255) / 256)), dim3(256), dargs, 0, s);
  if (e != hipSuccess) return ATTN_E_LAUNCH;
  void* args[] = {&a};
  const void* dkdv = causal ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<true>)
                            : reinterpret_cast<const void*>(&bwd_dkdv_kernel<false>);
  const void* dqk = causal ? reinterpret_cast<const void*>(&bwd_dq_kernel<true>)
                           : reinterpret_cast<const void*>(&bwd_dq_kernel<false>);
  e = hipLaunchKernel(dkdv, dim3(a.total), dim3(kBwdWaves * 64), args, 0, s);
  if (e != hipSuccess) return ATTN_E_LAUNCH;
  e = hipLaunchKernel(dqk, dim3(a.total), dim3(kBwdWaves * 64), args, 0, s);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
