// fa_kernels.h - gfx950 kernels for the exact-attention forward pass (and
// the split-KV merge), plus the helpers the backward kernels share.
//
// What is computed (per batch b, head h, query row i):
//   S_ij = scale * q_i . k_j, masked to -inf for j > i when causal (and
//          outside a local window),
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
//  * one workgroup of 4 waves per (batch*head, 128-row query tile) for
//    16-bit inputs (64 rows for fp32); each wave owns 32 query rows, held as
//    MFMA B operands in registers for the whole key loop;
//  * the kernel computes S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}
//    (v_mfma_f32_32x32x2_f32 for fp32), so each lane holds one query column
//    and 16 keys: the row max needs one exchange with lane l^32 and the row
//    sum stays a per-lane partial until the epilogue;
//  * the exponentials use exp2 with log2(e) folded into the scale;
//  * O^T = V^T P^T keeps P in registers: the accumulator layout of S^T is
//    already the B-operand layout of the second MFMA, provided the K tile's
//    rows are stored in LDS with bits 2 and 3 of the key index swapped
//    (sigma below), which makes each lane's eight keys contiguous in V^T;
//  * 16-bit K/V tiles of 64 keys go global -> LDS by buffer loads that write
//    LDS directly, two stages each (unpadded rows with a chunk swizzle at
//    d <= 128, padded rows at d = 256); V is read transposed
//    from its natural layout by ds_read_b64_tr_b16 (fp32 tiles go through
//    registers);
//  * causal: key tiles past the workgroup's last row are never loaded, and
//    only diagonal or ragged tiles pay for the element mask; a window
//    narrows the tile range the same way from both sides;
//  * operands are strided views (View), so packed tensors are read in place;
//    with fewer queries than keys the queries take the last positions;
//  * split-KV runs the same kernels on a 2-D grid (query tile x key part)
//    and merge_kernel combines the parts' results by log-sum-exp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Element strides of one [B, H, N, d] operand whose d elements are
// contiguous: batch, head and row (sequence position). A contiguous tensor
// has (H N d, N d, d); a head-interleaved one such as the q slice of a packed
// [B, N, 3, H, d] tensor has (3 N H d, d, 3 H d). The host guarantees that
// every row start is 16-byte aligned and that 64 row strides fit in 32 bits.
struct View {
  long long b, h;
  int r;
};

// Element offset of head bh = b * H + h.
__device__ __forceinline__ long long view_base(const View& v, int bh, int H) {
  const int b = bh / H;
  return (long long)b * v.b + (long long)(bh - b * H) * v.h;
}

// Split-KV partial results. With nsplit > 1 the launch grid has nsplit
// rows (blockIdx.y = s), and workgroup (x, s) covers the s-th of nsplit
// contiguous, near-equal parts of its query tile's key tiles: tiles
// floor(n s / nsplit) .. floor(n (s + 1) / nsplit) - 1 of its n tiles. It
// writes, for each of its query rows, the attention over those keys alone,
// normalised (O_s), and its LSE_s, both fp32, into the workspace `part`:
// O_s at part[((s * BH + bh) * N + i) * d + c], then LSE_s at
// part[nsplit * BH * N * d + (s * BH + bh) * N + i] (BH = B * H). A row with
// no visible key in the part gets O_s = 0 and LSE_s = -inf.
struct SplitOut {
  float* part;  // NULL: no split, write O and LSE directly
  int nsplit;
  int nbh;      // B * H
};

// The part [t_lo, t_lo + nkt) of a tile range that split s of n covers.
__device__ __forceinline__ void split_range(int s, int n, int& t_lo, int& nkt) {
  const int a = (int)((long long)nkt * s / n);
  const int e = (int)((long long)nkt * (s + 1) / n);
  t_lo += a;
  nkt = e - a;
}

// Floor of a / b for b > 0 and any sign of a.
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }

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
// stream the same K/V share one L2. Causal tiles go longest (last query
// tile) first: when the heads split evenly over the XCDs, an XCD takes its
// heads in chunks of C and, within a chunk, all heads' longest tiles before
// any head's next one, C chosen so that a chunk's workgroups about fill the
// XCD's resident slots (xcd_slots; at least one head). Short tiles then end
// each chunk, and the long ones of the next chunk start as slots free up
// (measured 10% faster on a 128-head causal grid than head after head).
__device__ __forceinline__ void decode_block(int nblocks, int nqt, bool causal, int& bh, int& qt,
                                             int xcd_slots = 32) {
  const int b = blockIdx.x;
  const int nbh = nblocks / nqt;
  if (causal && (nbh & 7) == 0) {
    const int hpx = nbh >> 3;  // heads per XCD
    int C = xcd_slots / nqt;
    C = C < 1 ? 1 : (C > hpx ? hpx : C);
    while (hpx % C != 0) --C;
    const int x = b & 7, Lx = b >> 3;
    const int chunk = Lx / (C * nqt), r = Lx - chunk * (C * nqt);
    const int t_rank = r / C;
    bh = x * hpx + chunk * C + (r - t_rank * C);
    qt = nqt - 1 - t_rank;
    return;
  }
  int L = b;
  if ((nblocks & 7) == 0) L = (b & 7) * (nblocks >> 3) + (b >> 3);
  bh = L / nqt;
  qt = L - bh * nqt;
  if (causal) qt = nqt - 1 - qt;
}

// One online-softmax update for the 16 scores a lane holds: the 32x32 MFMA
// tile s of keys kb + [0, 32) (register r: key kb + acc_row(r, hh)) for the
// query at position qrow, which sees keys qrow - wl .. qrow + wr below N
// (q0: position of the wave's first row; N: number of keys). On return s
// holds P = exp2(S*c - m_new), unrounded fp32; returns alpha =
// exp2(m_old - m_new).
__device__ __forceinline__ float online_softmax(f32x16& s, float c, int kb, int qrow, int q0, int N,
                                                int wl, int wr, int hh, float& m_run, float& l_run) {
  const bool need_mask = kb + 31 > q0 + wr || kb + 32 > N || kb < q0 + 31 - wl;
  float mx = -INFINITY;
  if (need_mask || c < 0.f) {
    // Scaled path: t = S * c for visible keys, -inf for masked ones. A row
    // with no visible key so far keeps m = -inf (stand-in reference 0).
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + acc_row(r, hh);
      const bool ok = key < N && key <= qrow + wr && key >= qrow - wl;
      s[r] = ok ? s[r] * c : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = wave_pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
      ls += s[r];
    }
    l_run = alpha * l_run + ls;
    m_run = m_new;
    return alpha;
  }
  // Fast path (no masked key, c >= 0): max(S) * c == max(S * c).
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = wave_pair_max(mx) * c;
  const float m_new = fmaxf(m_run, mx);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  float ls = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_new));
    ls += s[r];
  }
  l_run = alpha * l_run + ls;
  m_run = m_new;
  return alpha;
}

// ---------------------------------------------------------------------------
// fp16 / bf16 kernel.
//
// LDS holds two stages of K and two of V (separate arrays, so the compiler
// can tell a copy into one stage from reads of the other). Tile rows are keys
// in order. The layout keeps the 16 rows read by one 16-lane ds_read_b128
// phase (K) and the 4 rows x 64 bytes read by one 32-lane
// ds_read_b64_tr_b16 phase (V) on distinct banks:
// - d <= 128: rows 2d bytes apart with no padding; 16-byte chunk c of row r
//   sits at chunk c ^ chunk_swz(r) of that row. A tile is a whole number of
//   4 KiB, so each of the 4 waves issues d/32 copies per tile, all of them
//   moving data.
// - d = 256: K rows 2d + 16 bytes apart, V rows 2d + 64, in order, so that
//   every read is one base register plus immediate offsets. (The swizzle
//   needs 8 offsets per lane for K and 8 for V; with 128 KiB of stages,
//   beyond the reach of the 16-bit immediate, that cost the d = 256
//   kernel 15%.) Tiles are rounded up to whole 4 KiB; pad slots and the
//   filler past the 64 rows fetch nothing (tile_src).
// Tiles are copied by buffer_load_dwordx4 ... lds: each wave instruction
// fills 1 KiB of LDS, 16 bytes per lane in lane order, and each lane fetches
// the global chunk that belongs at its slot. Global rows are any 16-byte
// multiple apart (the row stride of the operand's view), so a head of a
// packed tensor is read in place.

template <int D>
struct Geo16 {
  static constexpr bool kSwz = D <= 128;                 // unpadded, swizzled rows
  static constexpr int kRowB = 2 * D;                    // bytes of one K/V row's values
  static constexpr int kSK = kSwz ? kRowB : kRowB + 16;  // LDS K row stride
  static constexpr int kSV = kSwz ? kRowB : kRowB + 64;  // LDS V row stride
  // LDS bytes of a K (V) tile, rounded up to whole 4 KiB so that each of the
  // 4 waves issues the same number of 1 KiB copies.
  static constexpr int kKT = (kBc * kSK + 4095) / 4096 * 4096;
  static constexpr int kVT = (kBc * kSV + 4095) / 4096 * 4096;
  static constexpr int kKPW = kKT / 4096;  // 1 KiB copies per wave per K tile
  static constexpr int kVPW = kVT / 4096;
};

// Chunk swizzle of LDS row r (a function of r mod 16). Rows of 256 bytes:
// ((r & 3) << 2) | ((r >> 2) & 3), a bijection of the 16 rows onto 0..15.
// Rows of 128 bytes (d = 64, two rows per 256-byte bank period):
// (((r >> 1) & 1) << 2) | ((r >> 2) & 3), a bijection of the 8 even (and of
// the 8 odd) rows onto 0..7. tests/test_lds_layout.py checks coverage and
// bank conflicts of every copy and read pattern on the host.
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (D == 64)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else
    return ((r & 3) << 2) | ((r >> 2) & 3);
}

// Source byte offset (relative to the tile's first row, global rows rs
// bytes apart) of LDS slot t (16 bytes) of a tile whose LDS rows are STRIDE
// bytes apart. Padded layout: pad slots and the filler past the 64 rows get
// an offset beyond any tile's buffer range (at most 63 rows of 2^25 bytes
// plus one row), so the range check makes them load zeros without touching
// memory; their LDS bytes are never read. (Measured: bitwise the same
// output, 0.5% faster at d = 256 than fetching a real chunk again.)
template <int D, int STRIDE>
__device__ __forceinline__ uint32_t tile_src(int t, int rs) {
  constexpr int R = STRIDE / 16;  // 16-byte slots per LDS row
  const int m = t / R;
  const int q = t - m * R;
  if constexpr (STRIDE == 2 * D) {
    return (uint32_t)m * (uint32_t)rs + (uint32_t)(16 * (q ^ chunk_swz<D>(m)));
  } else {
    if (q >= D / 8 || m >= kBc) return 0x7FFFFFF0u;  // pad slot or filler
    return (uint32_t)m * (uint32_t)rs + (uint32_t)(16 * q);
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Marks a value as used here (emits no instruction). Keeps the compiler from
// sinking the code that produces it past this point, e.g. into the next loop
// iteration, which would undo the interleaving of the matrix-core and vector
// work.
// (The host pass of hipcc parses device code too; it has no "v" registers.)
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ void pin(u32x4& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
#else
__device__ __forceinline__ void pin(u32x4&) {}
__device__ __forceinline__ void pin(float&) {}
#endif

__device__ __forceinline__ lds_ptr_t as_lds(const void* p) { return (lds_ptr_t)p; }

// max / sum over the lane pair (l, l ^ 32): v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second.
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Stores one row of a 16-bit output from the 32x32 accumulator tiles a[t]
// (t < NT), each value times f: lane (n, hh) holds columns 32t + 8g + 4hh
// .. +3 of the row in registers 4g .. 4g + 3. The lane pair (n, 0), (n, 1)
// first swaps halves, so that each lane writes 16 contiguous bytes (columns
// 32t + 8(2gp + hh) .. +7) rather than each writing 8: half the store
// instructions, and each row segment one 32-byte piece (measured 1-3%
// faster over the forward shapes, bitwise the same output). Every lane
// takes part in the swaps; ok guards the stores (the two lanes of a pair
// share the row, hence ok).
template <class T, int NT>
__device__ __forceinline__ void store_row16(uint16_t* row, const f32x16 (&a)[NT], float f, int hh, bool ok) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      uint32_t lo[2], hi[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        lo[h] = T::pack(a[t][8 * gp + 2 * h] * f, a[t][8 * gp + 2 * h + 1] * f);
        hi[h] = T::pack(a[t][8 * gp + 4 + 2 * h] * f, a[t][8 * gp + 4 + 2 * h + 1] * f);
      }
      // Lanes 0-31 keep their own columns 8(2gp) + 0..3 and take their
      // partner's 8(2gp) + 4..7; lanes 32-63 take their partner's
      // 8(2gp + 1) + 0..3 and keep their own 8(2gp + 1) + 4..7.
      const auto s0 = __builtin_amdgcn_permlane32_swap(lo[0], hi[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(lo[1], hi[1], false, false);
      if (ok) *(u32x4*)(row + 32 * t + 16 * gp + 8 * hh) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
  }
}

// The exponent reference m (log2 units) need not be the exact running max:
// the result is the same in exact arithmetic for any reference (the final
// division by the running sum cancels it), and fp32/bf16 only need the P
// values bounded. A row's m therefore stays put while the row's P sum over
// a 64-key tile is at most 2^kTau (so every P is), which spares both the
// row max and the rescale of the output accumulator on most tiles; it moves
// to the row's true running max otherwise. The first reference is the
// row's max over the first key tile of its query block.
constexpr float kTau = 8.0f;
constexpr float kTauPow = 256.0f;  // 2^kTau

constexpr uint32_t kBufWord3 = 0x00020000u;  // raw buffer, 32-bit data format

// Copies one tile (its first row at `src`, `nvalid` rows of the sequence
// left from there, rows rs >= 2D bytes apart) into LDS at `dst`: wave w
// issues copy blocks w, w + 4, ... of the 1 KiB blocks; off[i] is the lane's
// source offset for its i-th block. The buffer's range ends with the last
// valid row's values, so in a ragged last tile the lanes past the end load
// zeros. No branches: the copies can be interleaved with matrix-core work.
template <int D, int NPW>
__device__ __forceinline__ void copy_tile(const unsigned char* src, int nvalid, int rs, unsigned char* dst,
                                          const uint32_t (&off)[NPW], int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only on the device side
  const int rows = nvalid < kBc ? nvalid : kBc;
  const int range = rows > 0 ? (rows - 1) * rs + 2 * D : 0;
  const __amdgpu_buffer_rsrc_t rs_ =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, range, kBufWord3);
#pragma unroll
  for (int i = 0; i < NPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_, as_lds(dst + 1024 * (wave + 4 * i)), 16, off[i], 0, 0, 0);
#endif
}

// s_waitcnt vmcnt(X) for a compile-time X (lgkmcnt and expcnt not waited on).
// The race-check build (FA_SYNC_CHECK, libfa_sync.so) waits for every copy
// instead, and its tile_barrier below is a full __syncthreads(): with no
// copy in flight across any barrier, a missing wait in the normal build
// would show as a difference between the two builds' results.
template <int X>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(X >= 0 && X < 64, "vmcnt is 6 bits");
#if defined(FA_SYNC_CHECK)
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
#else
  __builtin_amdgcn_s_waitcnt((X & 15) | ((X >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}

// Workgroup barrier for the key loop. __syncthreads() is a release/acquire
// fence plus s_barrier, and the fence waits for every outstanding vector
// memory operation, LDS-bound tile copies included, so it would drain the
// copies that are meant to stay in flight across the barrier. This barrier
// waits only for the wave's own LDS reads (so the stage they read may be
// overwritten once every wave has arrived); the caller waits explicitly
// (wait_vmcnt) for the copies whose data the next phase reads. The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void tile_barrier() {
#if defined(FA_SYNC_CHECK)
  __builtin_amdgcn_s_waitcnt(0);  // every counter
  __syncthreads();
#else
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x0002 | 0x0400;  // VALU and transcendental
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;
constexpr int kSchedVmem = 0x0020;  // vector memory reads

// One 128-row query tile qt of head bh: the body of fwd16_kernel, which
// runs it once per workgroup, or twice (a long and a short causal tile) in
// the balanced causal grid.
template <class T, int D, bool CAUSAL>
__device__ __forceinline__ void fwd16_tile(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                           float* __restrict__ LSE, View vq, View vk, View vv, View vo, int H,
                                           int N, int Nk, float c, int wl, int wr, SplitOut sp, int bh, int qt) {
  using G = Geo16<D>;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;
  __shared__ __attribute__((aligned(1024))) unsigned char k0s[G::kKT];
  __shared__ __attribute__((aligned(1024))) unsigned char k1s[G::kKT];
  __shared__ __attribute__((aligned(1024))) unsigned char v0s[G::kVT];
  __shared__ __attribute__((aligned(1024))) unsigned char v1s[G::kVT];

  Q += view_base(vq, bh, H);
  O += view_base(vo, bh, H);
  LSE += (size_t)bh * N;
  const unsigned char* const kg = (const unsigned char*)(K + view_base(vk, bh, H));
  const unsigned char* const vg = (const unsigned char*)(V + view_base(vv, bh, H));
  const int ksb = 2 * vk.r, vsb = 2 * vv.r;  // K and V row strides, bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBr + wave * 32;
  const int qrow = q0 + n;
  // Query row i sits at position i + Nk - N of the key sequence (the last
  // N positions; 0 when the lengths are equal): masks use positions.
  const int pos_off = Nk - N;
  const int qpos = qrow + pos_off;

  // Q^T as B operands: lane (n, hh), k-step s holds Q[qrow][16s + 8hh .. +7].
  // A negative scale is folded into Q (an exact sign flip) so that c >= 0.
  // c == 0 becomes the smallest normal float: visible scores then still give
  // exp2(S c - m) == exp2(-m) to within rounding for any |S| < 2^100, and a
  // masked score (-inf) still gives 0.
  const uint32_t qflip = c < 0.f ? 0x80008000u : 0u;
  c = fmaxf(fabsf(c), 1.17549435e-38f);
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = qrow < N ? *(const u32x4*)(Q + (long long)qrow * vq.r + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};
    qf[s] ^= qflip;
  }

  // Key tiles the block needs: t_lo .. t_lo + nkt - 1 (a query at position
  // p sees keys p - wl .. p + wr; wr is 0 when causal, and an unbounded side
  // is 2^30). Tiles full_lo .. full_hi are visible to every row of the block.
  const int p_lo = qt * kBr + pos_off;  // position of the block's first row
  int t_lo = max(p_lo - wl, 0) / kBc;
  int nkt = min(min(qt * kBr + kBr - 1, N - 1) + pos_off + wr, Nk - 1) / kBc + 1 - t_lo;
  const int full_lo = (max(p_lo + kBr - 1 - wl, 0) + kBc - 1) / kBc;
  const int full_hi = floor_div(min(Nk, p_lo + wr + 1) - kBc, kBc);
  if (sp.part) {
    split_range(blockIdx.y, sp.nsplit, t_lo, nkt);
    if (nkt == 0) {  // an empty part: O_s = 0, LSE_s = -inf
      if (qrow < N) {
        float* op = sp.part + (((size_t)blockIdx.y * sp.nbh + bh) * N + qrow) * D;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) *(f32x4*)(op + 32 * t + 8 * g + 4 * hh) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (hh == 0)
          sp.part[(size_t)sp.nsplit * sp.nbh * N * D + ((size_t)blockIdx.y * sp.nbh + bh) * N + qrow] = -INFINITY;
      }
      return;
    }
  }

  // Tile-invariant source offsets of this lane's copy slots.
  uint32_t koff[G::kKPW], voff[G::kVPW];
#pragma unroll
  for (int i = 0; i < G::kKPW; ++i) koff[i] = tile_src<D, G::kSK>(64 * (wave + 4 * i) + lane, ksb);
#pragma unroll
  for (int i = 0; i < G::kVPW; ++i) voff[i] = tile_src<D, G::kSV>(64 * (wave + 4 * i) + lane, vsb);

  // With a ragged last tile, the copy of its rows past the end may leave old
  // LDS contents in place; starting from zeros keeps every value read finite
  // (those keys are masked, so their values only ever meet P = 0).
  if (Nk % kBc != 0) {
    const u32x4 z = {0, 0, 0, 0};
    for (int i = tid; i < G::kKT / 16; i += kThreads) {
      ((u32x4*)k0s)[i] = z;
      ((u32x4*)k1s)[i] = z;
    }
    for (int i = tid; i < G::kVT / 16; i += kThreads) {
      ((u32x4*)v0s)[i] = z;
      ((u32x4*)v1s)[i] = z;
    }
    __syncthreads();
  }

  auto issue_k = [&](int kt, unsigned char* dst) {
    copy_tile<D, G::kKPW>(kg + (long long)(kt * kBc) * ksb, Nk - kt * kBc, ksb, dst, koff, wave);
  };
  auto issue_v = [&](int kt, unsigned char* dst) {
    copy_tile<D, G::kVPW>(vg + (long long)(kt * kBc) * vsb, Nk - kt * kBc, vsb, dst, voff, wave);
  };

  // Per-lane LDS read offsets. K: MFMA row n holds key sigma(n) (keys
  // 32..63: 32 rows further), k-step s reads its chunk 2s + hh. V
  // (transposed read): 16-lane block b reads keys 8*(b>>1) + (lane&15)/4
  // (+4 for the second read) of each 16-key step and, in the 32-column
  // group t, columns 32t + 16*(b&1) + 4*(lane&3) .. +3, i.e. chunk
  // 4t + 2*(b&1) + (lane&3)/2. Padded layout: one base each plus
  // immediates. Swizzled layout: one offset per k-step (K) and per column
  // group and read (V).
  constexpr bool kSwz = G::kSwz;
  constexpr int kNKO = kSwz ? D / 16 : 1;
  constexpr int kNVO = kSwz ? D / 32 : 1;
  int kofs[kNKO], vofs[2][kNVO];
  {
    const int vb = lane >> 4, vj = lane & 15;
    const int vr = 8 * (vb >> 1) + (vj >> 2);
    if constexpr (kSwz) {
      const int ksw = chunk_swz<D>(sigma(n));
#pragma unroll
      for (int s = 0; s < kNKO; ++s) kofs[s] = sigma(n) * G::kSK + 16 * ((2 * s + hh) ^ ksw);
      const int vx = 2 * (vb & 1) + ((vj & 3) >> 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int vsw = chunk_swz<D>(vr + 4 * h);
#pragma unroll
        for (int t = 0; t < kNVO; ++t)
          vofs[h][t] = (vr + 4 * h) * G::kSV + 16 * ((4 * t + vx) ^ vsw) + 8 * (vj & 1);
      }
    } else {
      kofs[0] = sigma(n) * G::kSK + 16 * hh;
      vofs[0][0] = vr * G::kSV + 32 * (vb & 1) + 8 * (vj & 3);
      vofs[1][0] = vofs[0][0] + 4 * G::kSV;
    }
  }
  // LDS address of k-step s of key half kh (keys 32 kh .. 32 kh + 31) in K
  // stage ks, and of the V operand read h of 16-key step cc, column group t.
  auto k_addr = [&](const unsigned char* ks, int s, int kh) {
    return kSwz ? ks + kofs[s] + 32 * kh * G::kSK : ks + kofs[0] + 32 * s + 32 * kh * G::kSK;
  };
  auto v_addr = [&](const unsigned char* vt, int cc, int t, int h) {
    return kSwz ? vt + 16 * cc * G::kSV + vofs[h][t] : vt + vofs[h][0] + 16 * cc * G::kSV + 64 * t;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
  f32x16 sc0, sc1;  // raw scores of the tile being turned into P

  // S_t = K_t Q^T into sc0 (keys 0..31 of the tile) and sc1 (keys 32..63):
  // 4 K reads ahead, then one MFMA and one read in turn.
  auto s_tile = [&](const unsigned char* ks, auto nvmem) {
    constexpr int NVMEM = decltype(nvmem)::value;
    sc0 = f32x16{};
    sc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      sc0 = T::mfma(*(const u32x4*)k_addr(ks, s, 0), qf[s], sc0);
      sc1 = T::mfma(*(const u32x4*)k_addr(ks, s, 1), qf[s], sc1);
    }
    constexpr int kDiv = NVMEM > 0 ? NVMEM : 1;
    constexpr int kEvery = (D / 8) / kDiv > 0 ? (D / 8) / kDiv : 1;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (NVMEM > 0 && i % kEvery == 0) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    }
  };

  // O^T += V^T P^T for one tile; the A operand comes from two transposed
  // 8-byte reads of the V tile.
  auto pv_tile = [&](const unsigned char* vt, const u32x4 (&pf)[4]) {
    // Consecutive MFMAs go to different accumulators (t inner), so none
    // waits for the previous one's result.
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)as_lds(v_addr(vt, cc, t, 0)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)as_lds(v_addr(vt, cc, t, 1)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 a = {l2.x, l2.y, h2.x, h2.y};
        acc[t] = T::mfma(a, pf[cc], acc[t]);
      }
    }
  };

  // Sets the scores of keys a row may not see (outside qpos - wl ..
  // qpos + wr, or past the end of the keys) to -inf. Register r of sc0
  // holds key kbase + 8*hh + kc(r) with kc(r) = sigma(acc_row(r, 0)); sc1
  // adds 32; a key is visible iff lo <= its kc <= lim.
  auto mask_tile = [&](int kbase) {
    const int lim = min(qpos + wr, Nk - 1) - kbase - 8 * hh;
    const int lo = qpos - wl - kbase - 8 * hh;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kc = 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
      sc0[r] = kc <= lim && kc >= lo ? sc0[r] : -INFINITY;
      sc1[r] = kc + 32 <= lim && kc + 32 >= lo ? sc1[r] : -INFINITY;
    }
  };
  auto is_full = [&](int t) { return t >= full_lo && t <= full_hi; };

  // P = exp2(S c - m) for the tile held in sc0/sc1, packed to the input
  // type (chunk cc of pf holds registers 8*(cc&1) .. +7 of sc0 for cc < 2,
  // of sc1 otherwise), and the lane's sum of the unrounded P. Masked scores
  // (-inf) give 0.
  auto exp_tile = [&](float m, u32x4 (&pf)[4]) {
    const float negm = -m;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = 8 * (cc & 1) + 2 * w;
        const float s_lo = cc < 2 ? sc0[r] : sc1[r];
        const float s_hi = cc < 2 ? sc0[r + 1] : sc1[r + 1];
        const float p_lo = __builtin_amdgcn_exp2f(__builtin_fmaf(s_lo, c, negm));
        const float p_hi = __builtin_amdgcn_exp2f(__builtin_fmaf(s_hi, c, negm));
        ls[w] += p_lo + p_hi;
        pf[cc][w] = T::pack(p_lo, p_hi);
      }
    }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // Row max of the tile held in sc0/sc1, scaled (c > 0, so max(S) c ==
  // max(S c)); -inf if every key of the row is masked.
  auto tile_max = [&]() {
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      m0 = fmaxf(m0, sc0[r]);
      m1 = fmaxf(m1, sc1[r]);
    }
    const float mx = pair_max(fmaxf(m0, m1));
    return mx == -INFINITY ? -INFINITY : mx * c;
  };

  // Prologue: K0, K1 and V0 copied, then S_0 (tile indices below are
  // relative to t_lo).
  issue_k(t_lo, k0s);
  if (nkt > 1) issue_k(t_lo + 1, k1s);
  issue_v(t_lo, v0s);
  wait_vmcnt<0>();
  __syncthreads();
  s_tile(k0s, std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  if (!is_full(t_lo)) mask_tile(t_lo * kBc);
  // The first tile's own max is the first exponent reference, so its P need
  // not be computed twice (a row with no visible key in it keeps -inf and
  // takes the move in the first iteration, as every row did before).
  m_run = tile_max();

  constexpr int kNK = G::kKPW, kNV = G::kVPW;  // copies per wave per tile

  // Iteration j: block 1 runs O += P_{j-1} V_{j-1} on the matrix cores while
  // the vector ALUs turn S_j into P_j; block 2 computes S_{j+1} (and masks
  // it if tile j+1 is diagonal or ragged). K_t lives in stage t & 1 of K,
  // V_t in stage t & 1 of V. The copies of K_{j+2} are spread through block
  // 1 and those of V_{j+1} through block 2 (issuing them in one burst stalls
  // the wave while the vector-memory queue drains), so each copy has about
  // an iteration and a half to land. Past the last tile the K copy re-reads
  // the last tile into the free stage, which keeps the wait counts uniform.
  auto iter = [&](auto par, auto haspv, int j, u32x4 (&pf_prev)[4], u32x4 (&pf_cur)[4]) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool PV = decltype(haspv)::value;
    unsigned char* const k_cur = PAR == 0 ? k0s : k1s;   // K_j: done, receives K_{j+2}
    unsigned char* const k_next = PAR == 0 ? k1s : k0s;  // holds K_{j+1}
    unsigned char* const v_next = PAR == 0 ? v1s : v0s;  // V_{j-1}: done mid-iteration, receives V_{j+1}
    unsigned char* const v_prev = PAR == 0 ? v1s : v0s;  // holds V_{j-1}

    tile_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // ---- block 1 (at raised wave priority: where two waves share a SIMD,
    // the one in this mixed matrix-core / exponential phase issues first,
    // and the other's S products fill the matrix-core gaps; measured
    // 2-4% faster at d <= 128, neutral at d = 256)
    __builtin_amdgcn_s_setprio(1);
    issue_k(t_lo + min(j + 2, nkt - 1), k_cur);
    if constexpr (PV) pv_tile(v_prev, pf_prev);
    float ls = exp_tile(m_run, pf_cur);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pin(pf_cur[cc]);
    pin(ls);
    if constexpr (PV) {
      constexpr int kValu = 110 / (D / 8) + 1;
      constexpr int kEvery = (D / 8) / kNK > 0 ? (D / 8) / kNK : 1;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, kValu, 0);
        if (i % kEvery == 0) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // A row whose P sum over the tile's 64 keys exceeds 2^kTau (or whose m
    // was still -inf: then the sum is NaN or inf) moves its reference to
    // its running max and redoes P (rare). The move is per row: the other
    // rows of the wave keep m, recompute the same P and scale by
    // exp2(0) = 1, so a row's result depends on its own keys only. A row
    // that has seen no visible key yet (possible with a window) keeps
    // m = -inf and gets P = 0 and l = 0 from a finite stand-in reference.
    const bool need = !(pair_sum(ls) <= kTauPow);
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float tmax = tile_max();
      const float m_new = need ? fmaxf(m_run, tmax) : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      ls = exp_tile(m_use, pf_cur);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
    }
    l_run += ls;
    __builtin_amdgcn_sched_barrier(0);

    // ---- block 2
    if (j + 1 < nkt) {
      // K_{j+1} landed (issued before V_j and K_{j+2}), and every wave is
      // done reading V_{j-1}.
      wait_vmcnt<kNK + kNV>();
      tile_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_v(t_lo + j + 1, v_next);
      s_tile(k_next, std::integral_constant<int, kNV>{});
      __builtin_amdgcn_sched_barrier(0);
      if (!is_full(t_lo + j + 1)) mask_tile((t_lo + j + 1) * kBc);
      // V_j landed before the next iteration reads it.
      wait_vmcnt<kNK + kNV>();
    } else {
      wait_vmcnt<0>();
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  u32x4 pfa[4], pfb[4];
  iter(P0{}, std::false_type{}, 0, pfb, pfa);  // P_0 -> pfa
  int j = 1;
  for (; j + 1 < nkt; j += 2) {
    iter(P1{}, std::true_type{}, j, pfa, pfb);      // P_j -> pfb
    iter(P0{}, std::true_type{}, j + 1, pfb, pfa);  // P_{j+1} -> pfa
  }
  if (j < nkt) {
    iter(P1{}, std::true_type{}, j, pfa, pfb);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pfa[cc] = pfb[cc];
  }
  // Last PV: V_{nkt-1} was copied during the last iteration.
  __syncthreads();
  pv_tile((nkt - 1) & 1 ? v1s : v0s, pfa);

  const float l_tot = pair_sum(l_run);
  if (sp.part) {
    // A part may hold no visible key of a row (l = 0): O_s = 0, LSE_s = -inf.
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < N) {
      float* op = sp.part + (((size_t)blockIdx.y * sp.nbh + bh) * N + qrow) * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(op + 32 * t + 8 * g + 4 * hh) = f32x4{acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv,
                                                          acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv};
      if (hh == 0)
        sp.part[(size_t)sp.nsplit * sp.nbh * N * D + ((size_t)blockIdx.y * sp.nbh + bh) * N + qrow] =
            l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  const float inv = 1.0f / l_tot;
  store_row16<T>(O + (long long)qrow * vo.r, acc, inv, hh, qrow < N);
  if (qrow < N && hh == 0) LSE[qrow] = (m_run + __log2f(l_tot)) * kLn2;
}

// The forward kernel for 16-bit inputs. Plain grid: one workgroup per (b h,
// 128-row query tile), mapped by decode_block. Balanced causal grid (BAL):
// one workgroup per (b h, pair p) of query tiles nqt - 1 - p and p, run one
// after the other, so that every workgroup sees nqt + 1 key tiles (with
// fewer queries than keys, the same plus a constant); the middle tile of an
// odd nqt pairs with itself and runs once. A workgroup index maps to its
// (b h, p) with each XCD taking a contiguous run, as decode_block does for
// equal-work grids.
template <class T, int D, bool CAUSAL, bool BAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(D >= 256 ? 1 : 2, D >= 256 ? 1 : 2)))
void fwd16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                  float* __restrict__ LSE, View vq, View vk, View vv, View vo, int H, int N, int Nk,
                  int nqt, int nblocks, float c, int wl, int wr, SplitOut sp) {
  if constexpr (BAL) {
    const int npair = (nqt + 1) / 2;
    int L = blockIdx.x;
    if ((nblocks & 7) == 0) L = (L & 7) * (nblocks >> 3) + (L >> 3);
    const int bh = L / npair;
    const int p = L - bh * npair;
    fwd16_tile<T, D, CAUSAL>(Q, K, V, O, LSE, vq, vk, vv, vo, H, N, Nk, c, wl, wr, sp, bh, nqt - 1 - p);
    if (p != nqt - 1 - p) {
      __syncthreads();  // every wave is done with the first tile's LDS stages
      fwd16_tile<T, D, CAUSAL>(Q, K, V, O, LSE, vq, vk, vv, vo, H, N, Nk, c, wl, wr, sp, bh, p);
    }
  } else {
    int bh, qt;
    decode_block(nblocks, nqt, CAUSAL, bh, qt, D >= 256 ? 32 : 64);
    fwd16_tile<T, D, CAUSAL>(Q, K, V, O, LSE, vq, vk, vv, vo, H, N, Nk, c, wl, wr, sp, bh, qt);
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32; P stays fp32).
//
// 64 query rows per workgroup, so that a small batch of long sequences
// still gives every compute unit a workgroup. Wave w owns rows 32*(w & 1) ..
// +31 and the 32-key block kq = w >> 1 of every iteration's keys: at d <= 128
// an iteration stages two 64-key tiles (128 keys, 8 waves, two per SIMD),
// at d = 256 one (64 keys, 4 waves). The waves of a row block run the
// online softmax over disjoint key sets, and at the end the waves kq > 0
// hand their (m, l, O) to wave 0 through LDS, which merges them with the
// same rescaling rule. The window (query i sees keys i - wl .. i + wr) only
// narrows the tile range and the masks; a split-KV part keeps whole 64-key
// tiles (a block past the part's last tile is skipped).
// LDS: ks = K keys [KT][D] floats with a 16-byte chunk swizzle ch ^ kswz(m)
// (no key permutation); vs = V keys [KT][D + 8] floats, rows padded by 32
// bytes so the two lane halves (keys 4 apart) land on different banks. At
// d <= 128 the online softmax keeps the 16-bit kernel's lazy exponent
// reference; at d = 256 it tracks the exact running max (online_softmax).
constexpr int kBr32 = 64;  // query rows per fp32 workgroup

// Threads of the fp32 workgroup: 8 waves (two per SIMD) at d <= 128, where
// each 64-row block splits every 128 keys among four waves; 4 waves at
// d = 256 (key halves of every 64 keys), whose tiles take all the LDS.
template <int D>
constexpr int fwd32_threads() {
  return D <= 128 ? 512 : 256;
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(fwd32_threads<D>(), fwd32_threads<D>()),
                          amdgpu_waves_per_eu(D <= 128 ? 2 : 1, D <= 128 ? 2 : 1)))
void fwd32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                  const float* __restrict__ V, float* __restrict__ O,
                  float* __restrict__ LSE, View vq, View vk, View vv, View vo, int H, int N, int Nk,
                  int nqt, int nblocks, float c, int wl, int wr, SplitOut sp) {
  constexpr int NT = fwd32_threads<D>();
  constexpr int KQ = NT / 128;                // 32-key blocks per iteration (waves per row block)
  constexpr int TPI = KQ / 2;                 // 64-key tiles per iteration
  constexpr int KT = 32 * KQ;                 // keys staged per iteration
  constexpr int DCH = D / 4;                  // 16-byte chunks per row
  constexpr int VSTRIDE = D + 8;              // floats per padded V row
  constexpr int KS_BYTES = KT * D * 4;
  constexpr int VS_BYTES = KT * VSTRIDE * 4;
  constexpr int CH = KT * DCH / NT;           // chunks per thread, per tensor
  constexpr bool PF = D <= 64;                // keep the next keys in VGPRs (at d = 128 they would spill)
  // The merge area (after the loop), per row block and wave kq > 0: its
  // accumulator (D/32 x 16 floats per lane), then all the m and l.
  constexpr int XO = 32 * D;                  // floats per partial accumulator
  static_assert((2 * (KQ - 1) * (XO + 128)) * 4 <= KS_BYTES + VS_BYTES, "merge area");

  __shared__ __attribute__((aligned(16))) unsigned char smem[KS_BYTES + VS_BYTES];
  unsigned char* const ks = smem;
  float* const vs = (float*)(smem + KS_BYTES);

  int bh, qt;
  decode_block(nblocks, nqt, CAUSAL, bh, qt);
  Q += view_base(vq, bh, H);
  K += view_base(vk, bh, H);
  V += view_base(vv, bh, H);
  O += view_base(vo, bh, H);
  LSE += (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave & 1;   // row block
  const int kq = wave >> 1;  // 32-key block of each iteration
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBr32 + rb * 32;
  const int qrow = q0 + n;
  // Positions: query row i sits at i + Nk - N (the last N positions).
  const int pos_off = Nk - N;

  // Q^T operands: k-steps 4u + j use d = 8u + 4hh + j.
  f32x4 qf[D / 8];
#pragma unroll
  for (int u = 0; u < D / 8; ++u)
    qf[u] = qrow < N ? *(const f32x4*)(Q + (long long)qrow * vq.r + 8 * u + 4 * hh) : f32x4{0, 0, 0, 0};
  if constexpr (D <= 128) {
    // The lazy exponent reference below needs c > 0: a negative scale is
    // folded into Q (an exact sign flip).
    if (c < 0.f) {
#pragma unroll
      for (int u = 0; u < D / 8; ++u) qf[u] = -qf[u];
    }
    c = fmaxf(fabsf(c), 1.17549435e-38f);
  }

  // Key tiles the block needs (a query at position p sees keys p - wl ..
  // p + wr; wr is 0 when causal, an unbounded side is 2^30).
  const int q_lo = qt * kBr32;
  int t_lo = max(q_lo + pos_off - wl, 0) / kBc;
  int t_end = min(min(q_lo + kBr32 - 1, N - 1) + pos_off + wr, Nk - 1) / kBc + 1;
  if (sp.part) {  // an empty part runs no iteration and stores O_s = 0, LSE_s = -inf
    int nkt = t_end - t_lo;
    split_range(blockIdx.y, sp.nsplit, t_lo, nkt);
    t_end = t_lo + nkt;
  }

  // 16-byte chunk swizzle of K rows. At d <= 128 the 32 lanes of a
  // ds_read_b128 phase (keys krow .. krow + 31, one chunk column) land on 32
  // distinct 16-byte groups of the 512 bytes the LDS serves per clock (rows
  // are 4D bytes apart, so at d = 64 consecutive keys alternate halves):
  // measured free of bank conflicts, where a 3-bit swizzle left 2.1e6
  // conflict cycles per launch on B4 H1 N4096 d64. At d = 256 the 3-bit
  // swizzle stays: the wider one needs per-read address arithmetic that
  // made the one-wave-per-SIMD kernel 5% slower.
  auto kswz = [](int key) { return D == 64 ? ((key >> 1) & 15) : (D == 128 ? (key & 31) : (key & 7)); };
  f32x4 kreg[PF ? CH : 1], vreg[PF ? CH : 1];

  auto gload = [&](int kt) {
    const int k0 = kt * kBc;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int g = tid + i * NT;
      const int key = g / DCH, ch = g % DCH;
      const bool ok = k0 + key < Nk;
      kreg[i] = ok ? *(const f32x4*)(K + (long long)(k0 + key) * vk.r + ch * 4) : f32x4{0, 0, 0, 0};
      vreg[i] = ok ? *(const f32x4*)(V + (long long)(k0 + key) * vv.r + ch * 4) : f32x4{0, 0, 0, 0};
    }
  };
  auto swrite_regs = [&]() {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int g = tid + i * NT;
      const int key = g / DCH, ch = g % DCH;
      *(f32x4*)(ks + key * (D * 4) + ((ch ^ kswz(key)) << 4)) = kreg[i];
      *(f32x4*)(vs + key * VSTRIDE + ch * 4) = vreg[i];
    }
  };
  auto copy_direct = [&](int kt) {
    const int k0 = kt * kBc;
#pragma unroll 4
    for (int i = 0; i < CH; ++i) {
      const int g = tid + i * NT;
      const int key = g / DCH, ch = g % DCH;
      const bool ok = k0 + key < Nk;
      const f32x4 kx = ok ? *(const f32x4*)(K + (long long)(k0 + key) * vk.r + ch * 4) : f32x4{0, 0, 0, 0};
      const f32x4 vx = ok ? *(const f32x4*)(V + (long long)(k0 + key) * vv.r + ch * 4) : f32x4{0, 0, 0, 0};
      *(f32x4*)(ks + key * (D * 4) + ((ch ^ kswz(key)) << 4)) = kx;
      *(f32x4*)(vs + key * VSTRIDE + ch * 4) = vx;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

  // An iteration stages the keys of TPI 64-key tiles from kt on (the last
  // iteration may hold keys past t_end: they are staged but not used).
  if constexpr (PF) gload(t_lo);
  for (int kt = t_lo; kt < t_end; kt += TPI) {
    if constexpr (PF) swrite_regs();
    else copy_direct(kt);
    __syncthreads();
    if constexpr (PF) {
      if (kt + TPI < t_end) gload(kt + TPI);
    }
    // This wave's keys: kb .. kb + 31. A block outside the part's tiles, or
    // one no row of the wave can see, is skipped.
    const int kb = kt * kBc + 32 * kq;
    if (kt + kq / 2 < t_end && kb < Nk && kb <= q0 + pos_off + 31 + wr && kb + 31 >= q0 + pos_off - wl) {
      f32x16 s = {};
      const int krow = 32 * kq + n;
      const unsigned char* kr = ks + krow * (D * 4);
#pragma unroll
      for (int u = 0; u < D / 8; ++u) {
        const f32x4 a = *(const f32x4*)(kr + (((2 * u + hh) ^ kswz(krow)) << 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], qf[u][j], s, 0, 0, 0);
      }
      // O^T += V^T P^T, the V operand one float per lane per product. At
      // d <= 128 the V floats go through a ring of registers, read RING
      // products ahead (bitwise the same result; 1-2% faster at d = 128).
      auto pv = [&](const f32x16& p) {
        if constexpr (D >= 256) {  // no register left for reads ahead
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kq + acc_row(r, hh);
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * VSTRIDE + 32 * t + n], p[r], acc[t], 0, 0, 0);
          }
          return;
        }
        constexpr int RING = 4;
        float va[RING][D / 32];
        auto vload = [&](int r) {
          const int key = 32 * kq + acc_row(r, hh);
#pragma unroll
          for (int t = 0; t < D / 32; ++t) va[r % RING][t] = vs[key * VSTRIDE + 32 * t + n];
        };
#pragma unroll
        for (int r = 0; r < RING; ++r) vload(r);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
          for (int t = 0; t < D / 32; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[r % RING][t], p[r], acc[t], 0, 0, 0);
          if (r + RING < 16) vload(r + RING);
        }
        // Keep the reads RING steps ahead: the scheduler would otherwise put
        // each read next to its products and wait for it there.
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RING * (D / 64), 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, D / 32, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, D / 64, 0);
        }
      };
      if constexpr (D >= 256) {
        // One wave per SIMD with every register taken: the exact running
        // max (online_softmax) measured 4-5% faster here than the lazy
        // reference below.
        const float alpha = online_softmax(s, c, kb, qrow + pos_off, q0 + pos_off, Nk, wl, wr, hh, m_run, l_run);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
        pv(s);
      } else {
        // A 32x32x2 fp32 product writes its result over 16 passes, and a
        // vector instruction may read it only 18 wait states after the
        // product issues (what the compiler leaves on straight-line code).
        // On the taken-branch paths into the mask test and past it the
        // compiler left only 12, and a variant with such a path gave wrong
        // results. 14 are stated here, on every path; the mask test's own
        // scalar instructions after them bring every path to 20 or more.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 5" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // Keys the row may not see (outside qpos - wl .. qpos + wr, or past
        // the end) get -inf, only in blocks that hold such keys.
        const int qp = qrow + pos_off, q0p = q0 + pos_off;
        if (kb + 31 > q0p + wr || kb + 32 > Nk || kb < q0p + 31 - wl) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + acc_row(r, hh);
            s[r] = key < Nk && key <= qp + wr && key >= qp - wl ? s[r] : -INFINITY;
          }
        }
        // P against the current exponent reference m; the reference moves
        // (and the accumulator is rescaled) only for a row whose P sum over
        // the block exceeds 2^kTau, or whose m is still -inf (the sum is then
        // NaN or inf): the 16-bit kernel's rule. Measured 2-4.5% faster than
        // the exact running max at d = 64 and 128.
        f32x16 p;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_run));
          ls += p[r];
        }
        const bool need = !(pair_sum(ls) <= kTauPow);
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
          mx = pair_max(mx);
          const float tmax = mx == -INFINITY ? -INFINITY : mx * c;
          const float m_new = need ? fmaxf(m_run, tmax) : m_run;
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
          m_run = m_new;
          ls = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_use));
            ls += p[r];
          }
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
        }
        l_run += ls;
        pv(p);
      }
    }
    __syncthreads();
  }

  // Merge the key blocks of each row block: lane l of every wave of a row
  // block holds the same rows and output columns; waves kq > 0 hand their
  // (m, l, O) to wave 0 through LDS, which rescales all to the largest m.
  float* const xbase = (float*)smem;
  auto xo = [&](int j) { return xbase + (rb * (KQ - 1) + j - 1) * XO; };  // D/32 x 16 values x 64 lanes
  auto xm = [&](int j) { return xbase + 2 * (KQ - 1) * XO + (rb * (KQ - 1) + j - 1) * 128; };  // m, then l
  if (kq != 0) {
    float* const o = xo(kq);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[(t * 16 + r) * 64 + lane] = acc[t][r];
    xm(kq)[lane] = m_run;
    xm(kq)[64 + lane] = l_run;
  }
  __syncthreads();
  if (kq != 0) return;
  {
    // Any block may have seen no key of a row (then its m is -inf, l 0).
    float mj[KQ], lj[KQ];
    mj[0] = m_run;
    lj[0] = l_run;
#pragma unroll
    for (int j = 1; j < KQ; ++j) {
      mj[j] = xm(j)[lane];
      lj[j] = xm(j)[64 + lane];
    }
    float m = mj[0];
#pragma unroll
    for (int j = 1; j < KQ; ++j) m = fmaxf(m, mj[j]);
    const float m_use = m == -INFINITY ? 0.f : m;
    float a[KQ];
#pragma unroll
    for (int j = 0; j < KQ; ++j) a[j] = __builtin_amdgcn_exp2f(mj[j] - m_use);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = a[0] * acc[t][r];
#pragma unroll
        for (int j = 1; j < KQ; ++j) x += a[j] * xo(j)[(t * 16 + r) * 64 + lane];
        acc[t][r] = x;
      }
    float l = a[0] * lj[0];
#pragma unroll
    for (int j = 1; j < KQ; ++j) l += a[j] * lj[j];
    l_run = l;
    m_run = m;
  }

  const float l_tot = wave_pair_sum(l_run);
  if (sp.part) {
    // A part may hold no visible key of a row (l = 0): O_s = 0, LSE_s = -inf.
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < N) {
      float* op = sp.part + (((size_t)blockIdx.y * sp.nbh + bh) * N + qrow) * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(op + 32 * t + 8 * g + 4 * hh) = f32x4{acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv,
                                                          acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv};
      if (hh == 0)
        sp.part[(size_t)sp.nsplit * sp.nbh * N * D + ((size_t)blockIdx.y * sp.nbh + bh) * N + qrow] =
            l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
    float* orow = O + (long long)qrow * vo.r;
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

// ---------------------------------------------------------------------------
// Split-KV merge: the LSE-weighted combination of the nsplit partial results
// in `part` (layout of SplitOut):
//   LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s,
// with the largest LSE_s as the exponent reference (parts with LSE_s = -inf
// weigh 0). One row per D/4 consecutive lanes, 16 bytes of each part per
// lane; O is rounded once to the output type T (Bf16, F16 or float) and
// stored through its view. Bound by the reads of the parts.
template <class T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ part, int nsplit,
                                                         void* __restrict__ O, View vo,
                                                         float* __restrict__ LSE, int H, int N,
                                                         long long rows) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  constexpr float kLog2e = 1.44269504088896340736f;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  const float* const lp = part + (size_t)nsplit * rows * D + row;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, lp[(size_t)s * rows]);
  const float m_use = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float w = __builtin_amdgcn_exp2f((lp[(size_t)s * rows] - m_use) * kLog2e);
    l += w;
    acc += w * *(const f32x4*)(part + ((size_t)s * rows + row) * D + 4 * c);
  }
  acc *= l > 0.f ? 1.0f / l : 0.f;
  const int bh = (int)(row / N);
  const int i = (int)(row - (long long)bh * N);
  const long long off = view_base(vo, bh, H) + (long long)i * vo.r + 4 * c;
  if constexpr (std::is_same<T, float>::value) {
    *(f32x4*)((float*)O + off) = acc;
  } else {
    *(u32x2*)((uint16_t*)O + off) = u32x2{T::pack(acc[0], acc[1]), T::pack(acc[2], acc[3])};
  }
  if (c == 0) LSE[row] = l > 0.f ? m_use + __logf(l) : -INFINITY;
}

}  // namespace fa
