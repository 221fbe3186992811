// fa_kernels.h - gfx950 kernels for the exact-attention forward pass.
//
// What is computed (per batch b, head h, query row i):
//   S_ij = scale * q_i . k_j, masked to -inf for j > i when causal,
//   O_i  = sum_j softmax(S_i)_j v_j,  LSE_i = ln sum_j exp(S_ij),
// the standard three-step attention of section 1.1 of "2.3 FlashAttention
// and IO-aware attention" (aiknowledge.cn), evaluated blockwise with the
// online-softmax recurrence of ``flash_attention_forward`` on the
// flash_attention.py teaching page (forceinjection.github.io): per key block,
// new running max, exp of the shifted scores, a correction factor
// exp(m_old - m_new) applied to the running sum and to the output
// accumulator, and one division by the running sum at the end. The page's
// dataflow (load Q, K, V blocks on chip, local QK^T, blockwise softmax, local
// PV, accumulate) is section 9.3 of the flash-attn 2.8.3 build guide
// (intelliparadigm.com); all of it is fused into one kernel (its section 9.2).
//
// gfx950 design (not the pages' design, which targets other hardware):
//  * one workgroup of 4 waves per (batch*head, 128-row query tile); each
//    wave owns 32 query rows, held as MFMA B operands in VGPRs for the
//    whole key loop;
//  * the kernel computes S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}
//    (v_mfma_f32_32x32x2_f32 for fp32), so each lane holds one query column
//    and 16 keys: the row max needs one exchange with lane l^32 and the row
//    sum stays a per-lane partial until the epilogue;
//  * the exponentials use exp2 with log2(e) folded into the scale;
//  * O^T = V^T P^T keeps P in registers: the accumulator layout of S^T is
//    already the B-operand layout of the second MFMA, provided the K tile's
//    rows are stored in LDS with bits 2 and 3 of the key index swapped
//    (sigma below), which makes each lane's eight keys contiguous in V^T;
//  * K/V tiles of 64 keys are staged global -> VGPR -> LDS, the next tile's
//    global loads in flight while the current tile is consumed; K keeps its
//    [key][d] rows, V is transposed to [d][key] on the LDS write; both use a
//    16-byte-chunk XOR swizzle so 8-lane read phases hit distinct banks;
//  * causal: key tiles past the workgroup's last row are never loaded, a
//    wave skips tiles past its own last row, and only diagonal or ragged
//    tiles pay for the element mask.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kBr = 128;       // query rows per workgroup
constexpr int kBc = 64;        // keys per K/V tile
constexpr float kLn2 = 0.69314718055994530942f;

// 16-bit element types: the MFMA and the round-to-nearest-even pack of two
// fp32 values.
struct Bf16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

// Swap bits 2 and 3 of a key index inside its 16-key group (an involution).
__device__ __forceinline__ int sigma(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Key offset (0..31, inside one 32-row MFMA tile) of accumulator register r
// of lane half hh in the 32x32 MFMA output layout.
__device__ __forceinline__ int acc_row(int r, int hh) {
  return 8 * (r >> 2) + 4 * hh + (r & 3);
}

__device__ __forceinline__ float wave_pair_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

__device__ __forceinline__ float wave_pair_sum(float x) {
  return x + __shfl_xor(x, 32, 64);
}

// Maps a hardware workgroup index to (batch*head, query tile). Workgroups are
// dealt round-robin to the 8 XCDs; when the grid is a multiple of 8 the
// remap gives each XCD a contiguous run of heads, so the workgroups that
// stream the same K/V share one L2. Within a head, causal tiles go longest
// (last query tile) first.
__device__ __forceinline__ void decode_block(int nblocks, int nqt, bool causal, int& bh, int& qt) {
  int b = blockIdx.x;
  int L = b;
  if ((nblocks & 7) == 0) L = (b & 7) * (nblocks >> 3) + (b >> 3);
  bh = L / nqt;
  qt = L - bh * nqt;
  if (causal) qt = nqt - 1 - qt;
}

// One online-softmax update for the 32 scores a lane holds (two 16-value
// MFMA tiles s0, s1 covering keys kbase + [0, 64) of query row qrow).
// On return s0/s1 hold P = exp2(S*c - m_new), unrounded fp32; returns alpha.
template <bool CAUSAL>
__device__ __forceinline__ float online_softmax(f32x16& s0, f32x16& s1, float c, int kbase, int qrow,
                                                int q0, int N, int hh, int kperm_mask,
                                                float& m_run, float& l_run) {
  const bool need_mask = (CAUSAL && kbase + kBc - 1 > q0) || (kbase + kBc > N);
  float mx = -INFINITY;
  if (need_mask || c < 0.f) {
    // Scaled path: t = S * c for visible keys, -inf for masked ones.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int kr = acc_row(r, hh);
      int key0 = kbase + (kperm_mask ? sigma(kr) : kr);
      int key1 = key0 + 32;
      bool ok0 = key0 < N && (!CAUSAL || key0 <= qrow);
      bool ok1 = key1 < N && (!CAUSAL || key1 <= qrow);
      s0[r] = ok0 ? s0[r] * c : -INFINITY;
      s1[r] = ok1 ? s1[r] * c : -INFINITY;
      mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    }
    mx = wave_pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(s0[r] - m_new);
      s1[r] = __builtin_amdgcn_exp2f(s1[r] - m_new);
      ls += s0[r] + s1[r];
    }
    l_run = alpha * l_run + ls;
    m_run = m_new;
    return alpha;
  }
  // Fast path (no masked key, c >= 0): max(S) * c == max(S * c).
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = wave_pair_max(mx) * c;
  const float m_new = fmaxf(m_run, mx);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  float ls = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, -m_new));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, -m_new));
    ls += s0[r] + s1[r];
  }
  l_run = alpha * l_run + ls;
  m_run = m_new;
  return alpha;
}

// ---------------------------------------------------------------------------
// fp16 / bf16 kernel.
// LDS: ks = K tile [64 rows][D], row m holds key sigma(m), 16-byte chunk ch of
// a row stored at chunk position ch ^ (m & 7); vt = V^T tile [D rows][64 keys]
// (128 bytes per row), chunk ch (keys 8ch..8ch+7) at position ch ^ (d & 7).
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void fwd16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                  float* __restrict__ LSE, int N, int nqt, int nblocks, float c) {
  constexpr int DCH = D / 8;                        // 16-byte chunks per K/V row
  constexpr int KS_BYTES = kBc * D * 2;
  constexpr int VT_BYTES = D * kBc * 2;
  constexpr int KCH = kBc * DCH / kThreads;         // K chunks staged per thread
  constexpr int KPU = D >= 128 ? 4 : 2;             // keys per V transpose unit
  constexpr int VGROUPS = kBc / KPU;                // key groups per tile
  constexpr int VUNITS = VGROUPS * DCH / kThreads;  // V units per thread
  static_assert(KCH * kThreads == kBc * DCH, "K tile split");
  static_assert(VUNITS * kThreads == VGROUPS * DCH, "V tile split");

  __shared__ __attribute__((aligned(16))) unsigned char smem[KS_BYTES + VT_BYTES];
  unsigned char* const ks = smem;
  unsigned char* const vt = smem + KS_BYTES;

  int bh, qt;
  decode_block(nblocks, nqt, CAUSAL, bh, qt);
  const size_t base = (size_t)bh * (size_t)N * D;
  Q += base;
  K += base;
  V += base;
  O += base;
  LSE += (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBr + wave * 32;
  const int qrow = q0 + n;

  // Q^T as B operands: lane (n, hh), k-step s holds Q[qrow][16s + 8hh .. +7].
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = qrow < N ? *(const u32x4*)(Q + (size_t)qrow * D + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};

  const int nkt_all = (N + kBc - 1) / kBc;
  const int nkt = CAUSAL ? min(nkt_all, (qt * kBr + kBr - 1) / kBc + 1) : nkt_all;

  u32x4 kreg[KCH];
  u32x4 vreg[VUNITS][KPU];

  auto gload = [&](int kt) {
    const int k0 = kt * kBc;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int g = tid + i * kThreads;
      const int key = g / DCH, ch = g % DCH;
      kreg[i] = (k0 + key < N) ? *(const u32x4*)(K + (size_t)(k0 + key) * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VUNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int kg = unit % VGROUPS, dg = unit / VGROUPS;
#pragma unroll
      for (int j = 0; j < KPU; ++j) {
        const int key = k0 + kg * KPU + j;
        vreg[u][j] = key < N ? *(const u32x4*)(V + (size_t)key * D + dg * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int g = tid + i * kThreads;
      const int key = g / DCH, ch = g % DCH;
      const int m = sigma(key);
      *(u32x4*)(ks + m * (D * 2) + ((ch ^ (m & 7)) << 4)) = kreg[i];
    }
#pragma unroll
    for (int u = 0; u < VUNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int kg = unit % VGROUPS, dg = unit / VGROUPS;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dg * 8 + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int w = e >> 1;
        if constexpr (KPU == 4) {
          u32x2 out;
          out.x = __builtin_amdgcn_perm(vreg[u][1][w], vreg[u][0][w], sel);
          out.y = __builtin_amdgcn_perm(vreg[u][3][w], vreg[u][2][w], sel);
          *(u32x2*)(vt + d * (kBc * 2) + (((kg >> 1) ^ (d & 7)) << 4) + ((kg & 1) << 3)) = out;
        } else {
          const uint32_t out = __builtin_amdgcn_perm(vreg[u][1][w], vreg[u][0][w], sel);
          *(uint32_t*)(vt + d * (kBc * 2) + (((kg >> 2) ^ (d & 7)) << 4) + ((kg & 3) << 2)) = out;
        }
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    swrite();
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);
    const int kbase = kt * kBc;
    if (!CAUSAL || kbase <= q0 + 31) {
      f32x16 s0 = {}, s1 = {};
      const unsigned char* kr0 = ks + n * (D * 2);
      const unsigned char* kr1 = ks + (32 + n) * (D * 2);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const int off = ((2 * s + hh) ^ (n & 7)) << 4;
        s0 = T::mfma(*(const u32x4*)(kr0 + off), qf[s], s0);
        s1 = T::mfma(*(const u32x4*)(kr1 + off), qf[s], s1);
      }
      const float alpha = online_softmax<CAUSAL>(s0, s1, c, kbase, qrow, q0, N, hh, 1, m_run, l_run);
      // P^T as B operands: chunk cc covers keys 16cc..16cc+15 of the tile.
      u32x4 pf[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pf[0][w] = T::pack(s0[2 * w], s0[2 * w + 1]);
        pf[1][w] = T::pack(s0[8 + 2 * w], s0[8 + 2 * w + 1]);
        pf[2][w] = T::pack(s1[2 * w], s1[2 * w + 1]);
        pf[3][w] = T::pack(s1[8 + 2 * w], s1[8 + 2 * w + 1]);
      }
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        acc[t] *= alpha;
        const unsigned char* vr = vt + (32 * t + n) * (kBc * 2);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          acc[t] = T::mfma(*(const u32x4*)(vr + (((2 * cc + hh) ^ (n & 7)) << 4)), pf[cc], acc[t]);
      }
    }
    __syncthreads();
  }

  const float l_tot = wave_pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
    uint16_t* orow = O + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 out;
        out.x = T::pack(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
        out.y = T::pack(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
        *(u32x2*)(orow + 32 * t + 8 * g + 4 * hh) = out;
      }
    }
    if (hh == 0) LSE[qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32; P stays fp32).
// LDS: ks = K tile [64][D] floats with the 16-byte chunk swizzle ch ^ (m & 7)
// (no key permutation); vs = V tile [64][D + 8] floats, rows padded by 32
// bytes so the two lane halves (keys 4 apart) land on different banks.
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void fwd32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                  const float* __restrict__ V, float* __restrict__ O,
                  float* __restrict__ LSE, int N, int nqt, int nblocks, float c) {
  constexpr int DCH = D / 4;                  // 16-byte chunks per row
  constexpr int VSTRIDE = D + 8;              // floats per padded V row
  constexpr int KS_BYTES = kBc * D * 4;
  constexpr int VS_BYTES = kBc * VSTRIDE * 4;
  constexpr int CH = kBc * DCH / kThreads;    // chunks per thread, per tensor
  constexpr bool PF = D <= 128;               // keep the next tile in VGPRs

  __shared__ __attribute__((aligned(16))) unsigned char smem[KS_BYTES + VS_BYTES];
  unsigned char* const ks = smem;
  float* const vs = (float*)(smem + KS_BYTES);

  int bh, qt;
  decode_block(nblocks, nqt, CAUSAL, bh, qt);
  const size_t base = (size_t)bh * (size_t)N * D;
  Q += base;
  K += base;
  V += base;
  O += base;
  LSE += (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBr + wave * 32;
  const int qrow = q0 + n;

  // Q^T operands: k-steps 4u + j use d = 8u + 4hh + j.
  f32x4 qf[D / 8];
#pragma unroll
  for (int u = 0; u < D / 8; ++u)
    qf[u] = qrow < N ? *(const f32x4*)(Q + (size_t)qrow * D + 8 * u + 4 * hh) : f32x4{0, 0, 0, 0};

  const int nkt_all = (N + kBc - 1) / kBc;
  const int nkt = CAUSAL ? min(nkt_all, (qt * kBr + kBr - 1) / kBc + 1) : nkt_all;

  f32x4 kreg[PF ? CH : 1], vreg[PF ? CH : 1];

  auto gload = [&](int kt) {
    const int k0 = kt * kBc;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int g = tid + i * kThreads;
      const int key = g / DCH, ch = g % DCH;
      const bool ok = k0 + key < N;
      kreg[i] = ok ? *(const f32x4*)(K + (size_t)(k0 + key) * D + ch * 4) : f32x4{0, 0, 0, 0};
      vreg[i] = ok ? *(const f32x4*)(V + (size_t)(k0 + key) * D + ch * 4) : f32x4{0, 0, 0, 0};
    }
  };
  auto swrite_regs = [&]() {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int g = tid + i * kThreads;
      const int key = g / DCH, ch = g % DCH;
      *(f32x4*)(ks + key * (D * 4) + ((ch ^ (key & 7)) << 4)) = kreg[i];
      *(f32x4*)(vs + key * VSTRIDE + ch * 4) = vreg[i];
    }
  };
  auto copy_direct = [&](int kt) {
    const int k0 = kt * kBc;
#pragma unroll 4
    for (int i = 0; i < CH; ++i) {
      const int g = tid + i * kThreads;
      const int key = g / DCH, ch = g % DCH;
      const bool ok = k0 + key < N;
      const f32x4 kv = ok ? *(const f32x4*)(K + (size_t)(k0 + key) * D + ch * 4) : f32x4{0, 0, 0, 0};
      const f32x4 vv = ok ? *(const f32x4*)(V + (size_t)(k0 + key) * D + ch * 4) : f32x4{0, 0, 0, 0};
      *(f32x4*)(ks + key * (D * 4) + ((ch ^ (key & 7)) << 4)) = kv;
      *(f32x4*)(vs + key * VSTRIDE + ch * 4) = vv;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

  if constexpr (PF) gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    if constexpr (PF) swrite_regs();
    else copy_direct(kt);
    __syncthreads();
    if constexpr (PF) {
      if (kt + 1 < nkt) gload(kt + 1);
    }
    const int kbase = kt * kBc;
    if (!CAUSAL || kbase <= q0 + 31) {
      f32x16 s0 = {}, s1 = {};
      const unsigned char* kr0 = ks + n * (D * 4);
      const unsigned char* kr1 = ks + (32 + n) * (D * 4);
#pragma unroll
      for (int u = 0; u < D / 8; ++u) {
        const int off = ((2 * u + hh) ^ (n & 7)) << 4;
        const f32x4 a0 = *(const f32x4*)(kr0 + off);
        const f32x4 a1 = *(const f32x4*)(kr1 + off);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[j], qf[u][j], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[j], qf[u][j], s1, 0, 0, 0);
        }
      }
      const float alpha = online_softmax<CAUSAL>(s0, s1, c, kbase, qrow, q0, N, hh, 0, m_run, l_run);
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = acc_row(r, hh);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * VSTRIDE + 32 * t + n], s0[r], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[(key + 32) * VSTRIDE + 32 * t + n], s1[r], acc[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  const float l_tot = wave_pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
    float* orow = O + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 out = {acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv, acc[t][4 * g + 2] * inv,
                     acc[t][4 * g + 3] * inv};
        *(f32x4*)(orow + 32 * t + 8 * g + 4 * hh) = out;
      }
    }
    if (hh == 0) LSE[qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace fa
