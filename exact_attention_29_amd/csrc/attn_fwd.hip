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
// bf16 kernel, one workgroup = 4 waves = 256 query rows of one head:
//   * each wave owns 64 queries as two 32-query blocks; its Q^T operands stay
//     in VGPRs for the whole kernel;
//   * K and V tiles of 64 keys are staged through double-buffered LDS with
//     16-byte global loads, in a row-major layout whose 16-byte chunks are
//     XOR-swizzled per row so both read patterns below are bank-conflict free;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: lane l then holds 16 keys of
//     ONE query (l % 32), so the row max / row sum is a per-lane reduction
//     plus one exchange with lane l ^ 32;
//   * the S^T accumulator layout is exactly the B-operand layout of the next
//     MFMA, so P^T feeds O^T += V^T P^T without any lane shuffle; the V^T
//     operand is read from the row-major V tile with ds_read_b64_tr_b16;
//   * online softmax in fp32 with exp2 and scale*log2(e) folded into one FMA;
//     l sums the fp32 probabilities (so LSE carries fp32 error only), and
//     P is rounded to bf16 just before the PV product;
//   * causal: key tiles past a wave's last query are skipped, only the
//     diagonal and ragged tiles pay for masking.
// fp32 kernel: one thread per query row, fp32 FMA on the vector ALU, K/V
// tiles broadcast from LDS; same online softmax.  Used for fp32 I/O.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 64;                       // head size
constexpr int kBc = 64;                      // keys per K/V tile
constexpr int kWaves = 4;                    // waves per workgroup
constexpr int kQBlocks = 2;                  // 32-query blocks per wave
constexpr int kBr = kWaves * kQBlocks * 32;  // 256 queries per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kTileBytes = kBc * kD * 2;     // 8 KiB per K or V tile
constexpr int kStageBytes = 2 * kTileBytes;  // K tile then V tile
constexpr int kLdsBytes = 2 * kStageBytes;   // double buffered: 32 KiB

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kTau = 8.0f;  // reference-max slack, log2 units: p <= 256

struct Bf16Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int n;            // sequence length
  int q_tiles;      // ceil(n / kBr)
  int total_tiles;  // B * H * q_tiles
  float c;          // |scale| * log2(e)
  uint32_t q_sign;  // 0x80008000 when scale < 0 (Q negated), else 0
};

// 3-bit reversal: the per-row chunk swizzle is bitrev3((row >> 1) & 7).
__device__ __forceinline__ int bitrev3(int x) {
  return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}

__device__ __forceinline__ int swz(int row) { return bitrev3((row >> 1) & 7); }

// Byte offset of 16-byte chunk `chunk` of tile row `row` (8 chunks per row).
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * 128 + ((chunk ^ swz(row)) << 4);
}

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
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = w & 7, i = w >> 3;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

template <bool kCausal>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_kernel(Bf16Args a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int n = a.n;
  const int logical = xcd_remap(blockIdx.x, a.total_tiles);
  const int bh = logical / a.q_tiles;
  int qt = logical - bh * a.q_tiles;
  if (kCausal) qt = a.q_tiles - 1 - qt;  // longest rows first
  const size_t head = (size_t)bh * n * kD;
  const uint16_t* __restrict__ qg = a.q + head;
  const uint16_t* __restrict__ kg = a.k + head;
  const uint16_t* __restrict__ vg = a.v + head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave
  const int q_wave = qt * kBr + wave * (kQBlocks * 32);

  // ---- Q^T operands (B operand of S^T = K Q^T): lane holds 8 consecutive
  // features (16*ks + 8*hi ..) of query q_wave + 32*qb + l32.
  bf16x8 qop[kQBlocks][4];
#pragma unroll
  for (int qb = 0; qb < kQBlocks; ++qb) {
    const int qi = q_wave + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qi < n) w = *(const u32x4*)(qg + (size_t)qi * kD + 16 * ks + 8 * hi);
      w ^= a.q_sign;
      qop[qb][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- number of key tiles this workgroup visits
  int kv_end = n;
  if (kCausal) kv_end = min(n, qt * kBr + kBr);
  const int n_tiles = (kv_end + kBc - 1) / kBc;
  // last key tile with any visible key for this wave (causal skip)
  // (a wave whose rows all lie past N has nothing to compute)
  const int wave_last_key =
      q_wave >= n ? -1 : (kCausal ? min(n - 1, q_wave + kQBlocks * 32 - 1) : n - 1);

  // ---- global -> register staging: thread handles chunks tid and tid+256 of
  // the 512 16-byte chunks of a tile: row = idx / 8, chunk = idx % 8.
  u32x4 kreg[2], vreg[2];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + j * kThreads;
      const int row = idx >> 3, ch = idx & 7;
      const int key = kt * kBc + row;
      u32x4 z = {0u, 0u, 0u, 0u};
      kreg[j] = z;
      vreg[j] = z;
      if (key < n) {
        kreg[j] = *(const u32x4*)(kg + (size_t)key * kD + ch * 8);
        vreg[j] = *(const u32x4*)(vg + (size_t)key * kD + ch * 8);
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* base = lds + stage * kStageBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + j * kThreads;
      const int row = idx >> 3, ch = idx & 7;
      const int off = tile_off(row, ch);
      *(u32x4*)(base + off) = kreg[j];
      *(u32x4*)(base + kTileBytes + off) = vreg[j];
    }
  };

  // ---- per-lane constant LDS offsets
  // K operand (A of S^T): row kb*32 + l32, chunk 2*ks + hi.
  int k_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) k_off[ks] = tile_off(l32, 2 * ks + hi);
  // V^T operand via ds_read_b64_tr_b16: in each 16-lane group g, lane j
  // points at row 16*t + 4*hi + (j >> 2) (+8 for the second half of the
  // operand) and feature 32*db + 16*(g & 1) + 4*(j & 3).
  const int g = lane >> 4, j16 = lane & 15;
  int v_off[2][2];  // [sec][db] for kb = t = 0
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int row = 4 * hi + (j16 >> 2) + 8 * sec;
      const int feat = 32 * db + 16 * (g & 1) + 4 * (j16 & 3);
      const int byte = feat * 2;
      v_off[sec][db] = row * 128 + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
    }
  }
  // rows 16*t + 32*kb keep the swizzle of row (since swz uses bits 1..3 and
  // 16*t + 32*kb only adds multiples of 16): offset += (16*t + 32*kb) * 128.

  const float c = a.c;
  f32x16 acc[kQBlocks][2];
  float m_run[kQBlocks], l_run[kQBlocks];
#pragma unroll
  for (int qb = 0; qb < kQBlocks; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < n_tiles) load_tile(kt + 1);

    const int key0 = kt * kBc;
    if (key0 <= wave_last_key) {
      const char* kbase = lds + stage * kStageBytes;
      const char* vbase = kbase + kTileBytes;

      // ---- S^T = K Q^T : s[qb][kb] holds keys key0 + 32*kb + (8*(r/4) + 4*hi + r%4)
      f32x16 s[kQBlocks][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < kQBlocks; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kop = *(const bf16x8*)(kbase + kb * 32 * 128 + k_off[ks]);
#pragma unroll
          for (int qb = 0; qb < kQBlocks; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb][ks], s[qb][kb], 0, 0, 0);
        }
      }

      // ---- masking (wave-uniform branch: only the ragged last tile and the
      // causal diagonal tile pay for it).  Hidden scores become -inf; c > 0,
      // so fma(-inf, c, -m) stays -inf and exp2 gives exactly 0.
      const bool ragged = key0 + kBc > n;
      const bool diag = kCausal && key0 + kBc - 1 > q_wave;
      if (ragged || diag) {
#pragma unroll
        for (int qb = 0; qb < kQBlocks; ++qb) {
          const int qi = q_wave + qb * 32 + l32;
          const int lim = kCausal ? min(qi, n - 1) : n - 1;  // last visible key
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              s[qb][kb][r] = key <= lim ? s[qb][kb][r] : -INFINITY;
            }
        }
      }

      // ---- online softmax, per query block.  m_run is the reference the
      // probabilities are taken against (log2 units, scale folded in).  It is
      // raised only when some row's tile max exceeds it by more than kTau; any
      // reference gives the same O and LSE, and this one keeps p <= 2^kTau
      // while skipping the O rescale on almost every tile.
      bf16x8 pop[kQBlocks][2][2];  // [qb][kb][t]: B operand of O^T += V^T P^T
#pragma unroll
      for (int qb = 0; qb < kQBlocks; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[qb][kb][r], s[qb][kb][r + 1]));
        mx = half_swap_max(mx) * c;
        if (__any(mx > m_run[qb] + kTau)) {
          const float m_new = fmaxf(m_run[qb], mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
        }
        const float msub = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];

        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            bf16x8 p8;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
              const int r = 8 * tt + i;
              const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][r], c, -msub));
              const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][r + 1], c, -msub));
              lsum += e0;
              lsum += e1;
              const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
              p8[i] = pr[0];
              p8[i + 1] = pr[1];
            }
            pop[qb][kb][tt] = p8;
          }
        }
        l_run[qb] += lsum;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const int base = (32 * kb + 16 * tt) * 128;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vbase + base + v_off[0][db]));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vbase + base + v_off[1][db]));
            const i16x8 both = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 vop = __builtin_bit_cast(bf16x8, both);
#pragma unroll
            for (int qb = 0; qb < kQBlocks; ++qb)
              acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[qb][kb][tt], acc[qb][db], 0, 0, 0);
          }
        }
      }
    }

    if (kt + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < kQBlocks; ++qb) {
    const int qi = q_wave + qb * 32 + l32;
    const float l_tot = half_swap_sum(l_run[qb]);
    if (qi < n) {
      const float inv = 1.f / l_tot;
      uint16_t* orow = a.o + head + (size_t)qi * kD;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int f0 = 32 * db + 8 * r4 + 4 * hi;
          const bf16x2 p01 = {(__bf16)(acc[qb][db][4 * r4 + 0] * inv), (__bf16)(acc[qb][db][4 * r4 + 1] * inv)};
          const bf16x2 p23 = {(__bf16)(acc[qb][db][4 * r4 + 2] * inv), (__bf16)(acc[qb][db][4 * r4 + 3] * inv)};
          u32x2 w = {__builtin_bit_cast(unsigned, p01), __builtin_bit_cast(unsigned, p23)};
          *(u32x2*)(orow + f0) = w;
        }
      }
      if (hi == 0) a.lse[(size_t)bh * n + qi] = (m_run[qb] + __log2f(l_tot)) * kLn2;
    }
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
  int q_tiles;  // ceil(n / 64)
  float scale;
  int causal;
};

constexpr int kF32Keys = 32;  // keys per LDS tile in the fp32 kernel

__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(F32Args a) {
  __shared__ float ks[kF32Keys][kD];
  __shared__ float vs[kF32Keys][kD];
  const int n = a.n;
  const int bh = blockIdx.x / a.q_tiles;
  const int qt = blockIdx.x - bh * a.q_tiles;
  const size_t head = (size_t)bh * n * kD;
  const int qi = qt * 64 + threadIdx.x;
  const bool live = qi < n;

  float qv[kD], acc[kD];
#pragma unroll
  for (int f = 0; f < kD; ++f) {
    qv[f] = live ? a.q[head + (size_t)qi * kD + f] : 0.f;
    acc[f] = 0.f;
  }
  const float c = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = a.causal ? min(n, qt * 64 + 64) : n;
  const int row_last = a.causal ? min(qi, n - 1) : n - 1;

  for (int k0 = 0; k0 < kv_end; k0 += kF32Keys) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kF32Keys * kD; idx += 64) {
      const int r = idx / kD, f = idx % kD;
      const int key = k0 + r;
      ks[r][f] = key < n ? a.k[head + (size_t)key * kD + f] : 0.f;
      vs[r][f] = key < n ? a.v[head + (size_t)key * kD + f] : 0.f;
    }
    __syncthreads();
    float t[kF32Keys];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      float s = 0.f;
#pragma unroll
      for (int f = 0; f < kD; ++f) s = __builtin_fmaf(qv[f], ks[r][f], s);
      const bool vis = k0 + r <= row_last;
      t[r] = vis ? s * c : -INFINITY;
      mx = fmaxf(mx, t[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float msub = (m_new == -INFINITY) ? 0.f : m_new;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int f = 0; f < kD; ++f) acc[f] *= alpha;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      const float p = __builtin_amdgcn_exp2f(t[r] - msub);
      l_run += p;
#pragma unroll
      for (int f = 0; f < kD; ++f) acc[f] = __builtin_fmaf(p, vs[r][f], acc[f]);
    }
  }
  if (live) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int f = 0; f < kD; ++f) a.o[head + (size_t)qi * kD + f] = acc[f] * inv;
    a.lse[(size_t)bh * n + qi] = (m_run + __log2f(l_run)) * kLn2;
  }
}

// ---------------------------------------------------------------- host side

constexpr int kMaxDevices = 64;
// 0 = not checked, 1 = gfx950, 2 = other architecture
int g_arch_state[kMaxDevices];

attn_status check_device() {
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
    __atomic_store_n(&g_arch_state[dev], state, __ATOMIC_RELEASE);
  }
  return state == 1 ? ATTN_OK : ATTN_E_DEVICE;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

attn_status validate(const void* q, const void* k, const void* v, const void* o, const void* lse,
                     int B, int H, int N, int d, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_INVALID;
  if (B < 1 || H < 1 || N < 1 || d != kD || !std::isfinite(scale)) return ATTN_E_INVALID;
  if ((long long)B * H * N * d >= (1LL << 31)) return ATTN_E_INVALID;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
      misaligned(lse, 4))
    return ATTN_E_ALIGN;
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, int d, float scale, int causal,
                                void* stream) {
  attn_status st = validate(q, k, v, o, lse, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;

  Bf16Args a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.n = N;
  a.q_tiles = (N + kBr - 1) / kBr;
  a.total_tiles = B * H * a.q_tiles;
  // c must be > 0: masked scores are -inf and fma(-inf, c, -m) must stay
  // -inf.  A zero (or denormal) scale becomes FLT_MIN, whose scores differ by
  // far less than one fp32 ulp of exp2's result, i.e. the same uniform rows.
  a.c = std::fmax(std::fabs(scale) * kLog2e, 1.17549435e-38f);
  a.q_sign = scale < 0.f ? 0x80008000u : 0u;

  void* args[] = {&a};
  const void* fn = causal ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<true>)
                          : reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false>);
  const hipError_t e = hipLaunchKernel(fn, dim3(a.total_tiles), dim3(kThreads), args, kLdsBytes,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

extern "C" attn_status attn_fwd_fp32(const float* q, const float* k, const float* v, float* o,
                                     float* lse, int B, int H, int N, int d, float scale,
                                     int causal, void* stream) {
  attn_status st = validate(q, k, v, o, lse, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  st = check_device();
  if (st != ATTN_OK) return st;

  F32Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.n = N;
  a.q_tiles = (N + 63) / 64;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  void* args[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_f32_kernel),
                                       dim3(B * H * a.q_tiles), dim3(64), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

extern "C" const char* attn_strerror(attn_status s) {
  switch (s) {
    case ATTN_OK: return "success";
    case ATTN_E_INVALID: return "invalid argument (null pointer, size out of range, d != 64 or non-finite scale)";
    case ATTN_E_ALIGN: return "misaligned pointer (q, k, v, o need 16 bytes, lse 4 bytes)";
    case ATTN_E_DEVICE: return "no usable device (no HIP device current, or it is not gfx950)";
    case ATTN_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}
