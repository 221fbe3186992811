// fa_bwd.hip - backward pass of exact attention (fp16 / bf16 inputs, head
// dimension 64, 128 or 256): argument checks, kernels and launches of fa_bwd.
//
// The forward keeps only O and the row statistic LSE; the backward
// recomputes the attention weights from Q, K and LSE instead of storing the
// N x N matrix (the recomputation of section 9.2 of the flash-attn 2.8.3
// build guide, intelliparadigm.com, and of section 7 of the RTX 4070
// FlashAttention-2 page, jsqmd.com). The gradients are the chain rule of the
// forward definition:
//   P = exp(S - LSE) with S = scale Q K^T (masked keys excluded),
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic (= sum_j P_ij dP_ij),
//   dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels on the caller's stream, no atomics (the result does not
// depend on scheduling):
//  * dq_kernel: one workgroup per (batch*head, 128-row query tile), built
//    like the forward: S^T = K Q^T and dP^T = V dO^T on the matrix cores
//    with Q^T and dO^T held as B operands, P^T and dS^T per lane (each lane
//    owns one query), then dQ^T += K^T dS^T with K^T read transposed from
//    LDS and dS^T as the B operand; it first computes its rows'
//    D = rowsum(dO * O) and writes them to the caller's delta buffer;
//  * dkdv8_kernel (d <= 128) and dkdv_kernel (d = 256): one workgroup per
//    (batch*head, 128-key block); a wave owns 32 keys and takes K^T and V^T
//    as B operands; per 32 queries, S = Q K^T and dP = dO V^T with Q and dO
//    from LDS, P and dS per lane (each lane owns one key), then
//    dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read transposed
//    from LDS. At d <= 128 eight waves, two per SIMD, split each 64-query
//    step by halves and add their sums at the end, with K^T and V^T read
//    from LDS copies of the block's rows; at d = 256 four waves hold K^T in
//    registers and read V^T from an LDS copy.
// The index tricks are the forward's: rows of an A operand are read through
// the permutation sigma, which makes the accumulator of one product the B
// operand layout of the next.
//
// LDS tiles hold rows of D 16-bit values with a row stride of max(2D, 256)
// bytes; the 16-byte chunk c of row r is stored at chunk c ^ swz(r). With
// swz(r) = ((r & 3) << 2) | ((r >> 2) & 3) both kinds of read are free of
// bank conflicts: a 16-lane phase of 16-byte reads touches 16 rows whose
// swz values are all different, and a 32-lane phase of transposed 8-byte
// reads touches 4 consecutive rows x 64 bytes, which land in 4 different
// 64-byte groups.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_host.h"
#include "fa_kernels.h"

namespace fa {
namespace bwd {

constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct Tile {
  static constexpr int kRS = 2 * D > 256 ? 2 * D : 256;  // LDS row stride, bytes
  static constexpr int kCh = D / 8;                       // 16-byte chunks per row
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Byte offset of 16-byte chunk c of row r in an LDS tile.
template <int D>
__device__ __forceinline__ int at(int r, int c) {
  return r * Tile<D>::kRS + 16 * (c ^ swz(r));
}

template <class T>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (std::is_same<T, Bf16>::value) {
    return __uint_as_float(bits16 << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

// A lane's LDS byte offsets for its operand reads, with the chunk swizzle
// resolved once (swz depends on r & 15 only, so moving by 16 rows adds a
// plain row offset that the reads take as an immediate). The swizzle flips
// only the low 4 bits of a chunk index, so chunks 16 and up sit exactly 256
// bytes after chunks 0 .. 15 of the same row: only the offsets of the first
// 16 chunks are kept, and the rest is an immediate.
template <int D>
struct Operands {
  static constexpr int kRo = D / 16 < 8 ? D / 16 : 8;
  static constexpr int kTr = D / 32 < 4 ? D / 32 : 4;
  int ro[kRo];  // A operand of X B, k-step s: row sigma(n), chunk 2s + hh
  int tl[kTr];  // A operand of X^T B, 32-column block tb: low 8 bytes
  int th[kTr];  //   and high 8 bytes (rows 4 further), for 16-row step 0

  __device__ __forceinline__ explicit Operands(int lane) {
    const int n = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int s = 0; s < kRo; ++s) ro[s] = at<D>(sigma(n), 2 * s + hh);
    // Transposed reads (the lane pattern of the forward kernel's V^T
    // operand): 16-lane block vb, lane vj reads rows r0 and r0 + 4, chunk
    // 4tb + c0, half vj & 1.
    const int vb = lane >> 4, vj = lane & 15;
    const int r0 = 8 * (vb >> 1) + (vj >> 2);
    const int c0 = 2 * (vb & 1) + ((vj & 3) >> 1);
    const int h8 = 8 * (vj & 1);
#pragma unroll
    for (int tb = 0; tb < kTr; ++tb) {
      tl[tb] = at<D>(r0, 4 * tb + c0) + h8;
      th[tb] = at<D>(r0 + 4, 4 * tb + c0) + h8;
    }
  }

  // X B operand: rows rbase + sigma(m) (rbase a multiple of 16).
  __device__ __forceinline__ u32x4 row(const unsigned char* tile, int rbase, int s) const {
    return *(const u32x4*)(tile + rbase * Tile<D>::kRS + 256 * (s / kRo) + ro[s % kRo]);
  }
  // X^T B operand: 16-row k-step ks (rows 16ks ..), 32-column block tb.
  __device__ __forceinline__ u32x4 tr(const unsigned char* tile, int ks, int tb) const {
    const unsigned char* t = tile + 16 * ks * Tile<D>::kRS + 256 * (tb / kTr);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)as_lds(t + tl[tb % kTr]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)as_lds(t + th[tb % kTr]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  }
};

// Copies of an R-row tile into an LDS tile of the swizzled layout by
// buffer loads that write LDS directly (no registers): each wave
// instruction fills 1 KiB, i.e. 1024 / kRS LDS rows, 16 bytes per lane in
// lane order; lane l of copy block b writes row (1024 / kRS) b + l / L at
// physical chunk l % L (L = kRS / 16 lanes per row) and so fetches the
// logical chunk (l % L) ^ swz(row) of that row (for d = 64 the second half
// of each 256-byte row is padding, filled with a duplicate chunk). With NW
// waves, wave w issues blocks w, w + NW, ...: for 4 waves 16 rows apart
// with 256-byte rows, which all share the lane's row modulo 16 and so one
// source offset plus 16 rows per block, and 8 rows apart with 512-byte rows
// (d = 256), whose blocks alternate between two swizzles and so two source
// offsets; for 8 waves and 256-byte rows, 32 rows apart (one offset).
// Global rows are rs >= 2D bytes apart (the row stride of the operand's
// view); rows past the end of the sequence are outside the buffer's range.
template <int D, int R, int NW = 4>
struct TileDma {
  static constexpr int kRS = Tile<D>::kRS;
  static constexpr int kLPR = kRS / 16;    // lanes per LDS row
  static constexpr int kRPB = 1024 / kRS;  // LDS rows per copy block
  static constexpr int kStep = NW * kRPB;  // rows between a wave's consecutive blocks
  static constexpr int kNOff = kStep >= 16 ? 1 : 16 / kStep;  // distinct swizzles among them
  static constexpr int kPeriod = kStep * kNOff;  // rows after which a wave's offsets repeat
  static constexpr int kBlocks = R * kRS / 1024;
  static constexpr int kPW = kBlocks / NW;  // copy instructions per wave
  static_assert(kBlocks % NW == 0 && kPW % kNOff == 0 && kPeriod % 16 == 0, "blocks per wave");

  struct Off {
    uint32_t v[kNOff];
  };

  __device__ static Off lane_offset(int wave, int lane, int rs) {
    Off o;
#pragma unroll
    for (int j = 0; j < kNOff; ++j) {
      const int row = kRPB * wave + lane / kLPR + kStep * j;
      int c = (lane % kLPR) ^ swz(row);
      if (c >= D / 8) c &= D / 8 - 1;  // padding slot
      o.v[j] = (uint32_t)row * (uint32_t)rs + (uint32_t)(16 * c);
    }
    return o;
  }

  __device__ static void issue(const uint16_t* src, int nvalid, int rs, unsigned char* lds, const Off& off,
                               int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows = nvalid < R ? (nvalid > 0 ? nvalid : 0) : R;
    const int range = rows > 0 ? (rows - 1) * rs + 2 * D : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, range, kBufWord3);
#pragma unroll
    for (int i = 0; i < kPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, as_lds(lds + 1024 * (wave + NW * i)), 16,
                                               off.v[i % kNOff] + (uint32_t)((i / kNOff) * kPeriod) * (uint32_t)rs,
                                               0, 0, 0);
#endif
  }
};

// Row statistics (LSE or delta) of the 64 queries from src into LDS by a
// 4-byte copy per lane (256 bytes per wave instruction). Where a step waits
// for every copy of a wave, one wave copies them; where the wait counts
// leave the next step's copies in flight, every wave copies the same 256
// bytes, so that all waves issue the same number of copies. (With 32-query
// steps the upper half is the next step's and is not read.)
__device__ __forceinline__ void dma_row_stat(const float* src, int nvalid, float* lds, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  // The range is the same for every lane; readfirstlane lets the compiler
  // see that, which spares a loop over lanes around the copy.
  const int rows = __builtin_amdgcn_readfirstlane(nvalid < 64 ? (nvalid > 0 ? nvalid : 0) : 64);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, rows * 4, kBufWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, as_lds(lds), 4, (uint32_t)(4 * lane), 0, 0, 0);
#endif
}

// Offset (0..31) of the row that register r of a 32x32 accumulator holds in
// lane half hh, when the A operand's rows were read through sigma:
// 8*hh + kc(r), the same map as the forward kernel's mask.
__device__ __forceinline__ int perm_row(int r, int hh) {
  return 8 * hh + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
}

// dQ for one 128-row query tile. Query i sees keys i - wl .. i + wr (wr = 0
// when causal; an unbounded side is 2^30).
// Two waves per SIMD (two workgroups per compute unit), within 256 registers.
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(D >= 256 ? 1 : 2, D >= 256 ? 1 : 2)))
void dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
               const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
               const uint16_t* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ Dl,
               uint16_t* __restrict__ dQ, View vq, View vk, View vv, View vdo, View vo, View vdq, int H, int N,
               int nqt, int nblocks, float c, float scale, int wl, int wr) {
  // Two LDS stages, each a K tile then a V tile, filled by direct copies
  // one tile ahead.
  constexpr int TB = kBc * Tile<D>::kRS;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[2 * TB];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[2 * TB];

  int bh, qt;
  decode_block(nblocks, nqt, CAUSAL, bh, qt, D >= 256 ? 32 : 64);
  Q += view_base(vq, bh, H);
  K += view_base(vk, bh, H);
  V += view_base(vv, bh, H);
  dO += view_base(vdo, bh, H);
  dQ += view_base(vdq, bh, H);
  LSE += (size_t)bh * N;
  Dl += (size_t)bh * N;
  const int ksb = 2 * vk.r, vsb = 2 * vv.r;  // K and V row strides, bytes

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBr + 32 * wave;
  const int qrow = q0 + n;
  const Operands<D> op(lane);

  // Q^T and dO^T as B operands: lane (n, hh), k-step s holds row qrow,
  // columns 16s + 8hh .. +7.
  u32x4 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = qrow < N ? *(const u32x4*)(Q + (long long)qrow * vq.r + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};
    gf[s] = qrow < N ? *(const u32x4*)(dO + (long long)qrow * vdo.r + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};
  }
  // Rows past N get P = 0 (exp2(-inf)) and so contribute nothing.
  const float lse2 = qrow < N ? LSE[qrow] * kLog2e : INFINITY;
  // D_i = sum_c dO_ic O_ic of the lane's row: the lane holds half of the
  // row's dO (columns 16s + 8hh .. +7), multiplies it with the same columns
  // of O, and the lane pair (l, l ^ 32) adds the halves. Written to Dl for
  // the dK/dV kernel, which runs after this one on the same stream.
  float dl = 0.f;
  if (qrow < N) {
    const uint16_t* orow = O + view_base(vo, bh, H) + (long long)qrow * vo.r;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 a = *(const u32x4*)(orow + 16 * s + 8 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dl += to_f32<T>(a[e] & 0xffffu) * to_f32<T>(gf[s][e] & 0xffffu);
        dl += to_f32<T>(a[e] >> 16) * to_f32<T>(gf[s][e] >> 16);
      }
    }
  }
  dl = pair_sum(dl);
  if (hh == 0 && qrow < N) Dl[qrow] = dl;

  const int q_lo = qt * kBr;
  const int t_lo = max(q_lo - wl, 0) / kBc;
  const int t_end = min(min(q_lo + kBr - 1, N - 1) + wr, N - 1) / kBc + 1;

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

  using Dma = TileDma<D, kBc>;
  const typename Dma::Off koff = Dma::lane_offset(wave, lane, ksb);
  const typename Dma::Off voff = Dma::lane_offset(wave, lane, vsb);
  // Rows past N of a ragged last tile keep what the stage held; they are
  // masked, and starting from zeros keeps them finite.
  if (N % kBc != 0) {
    for (int i = threadIdx.x; i < 2 * TB / 16; i += kThreads) {
      ((u32x4*)st0)[i] = u32x4{0, 0, 0, 0};
      ((u32x4*)st1)[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
  }
  auto issue = [&](int t, unsigned char* st) {
    Dma::issue(K + (long long)(t * kBc) * vk.r, N - t * kBc, ksb, st, koff, wave);
    Dma::issue(V + (long long)(t * kBc) * vv.r, N - t * kBc, vsb, st + TB, voff, wave);
  };

  auto step = [&](int t, const unsigned char* st, unsigned char* st_next) {
    const unsigned char* const ks = st;
    const unsigned char* const vs = st + TB;
    // Tile t landed (it is the only copy in flight), every wave's copies are
    // visible and every wave is done with tile t - 1: refill its stage.
    wait_vmcnt<0>();
    tile_barrier();
    if (t + 1 < t_end) issue(t + 1, st_next);
    const int kbase = t * kBc;
    if (kbase > q0 + 31 + wr || kbase + kBc - 1 < q0 - wl) return;  // no key visible to the wave

    const bool full = kbase + kBc - 1 <= q0 + wr && kbase >= q0 + 31 - wl && kbase + kBc <= N;
    // The tile in two halves of 32 keys, software-pipelined so that each
    // half's exponentials run beside matrix-core work: S/dP of half 1 beside
    // P/dS of half 0, then dQ of half 0 beside P/dS of half 1 (3.6% off the
    // d = 256 backward, where one wave per SIMD has no other wave to
    // overlap with; neutral at d <= 128). The products accumulate in the
    // same order as half after half.
    f32x16 sa0 = {}, pa0 = {}, sa1 = {}, pa1 = {};
    // S^T (keys x queries) and dP^T for keys 32kh .. 32kh+31.
    auto sdp = [&](int kh, f32x16& sa, f32x16& pa) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sa = T::mfma(op.row(ks, 32 * kh, s), qf[s], sa);
        pa = T::mfma(op.row(vs, 32 * kh, s), gf[s], pa);
      }
    };
    // P^T = exp2(S c - lse2) on visible keys (0 elsewhere), dS^T =
    // P^T (dP^T - D), packed as the B operand of the next product: chunk cc
    // holds keys 32kh + 16cc + 8hh .. +7 of the tile.
    auto make_ds = [&](int kh, const f32x16& sa, const f32x16& pa, u32x4 (&dsp)[2]) {
      auto body = [&](auto masked) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float dsv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 8 * cc + 2 * w + e;
              float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -lse2));
              if constexpr (decltype(masked)::value) {
                const int key = kbase + 32 * kh + perm_row(r, hh);
                p = key < N && key <= qrow + wr && key >= qrow - wl ? p : 0.f;
              }
              dsv[e] = p * (pa[r] - dl);
            }
            dsp[cc][w] = T::pack(dsv[0], dsv[1]);
          }
      };
      if (full) body(std::false_type{});
      else body(std::true_type{});
    };
    // dQ^T += K^T dS^T over the half's two 16-key k-steps.
    auto dqm = [&](int kh, const u32x4 (&dsp)[2]) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int tb = 0; tb < D / 32; ++tb)
          acc[tb] = T::mfma(op.tr(ks, 2 * kh + cc, tb), dsp[cc], acc[tb]);
    };
    u32x4 ds0[2], ds1[2];
    sdp(0, sa0, pa0);
    __builtin_amdgcn_sched_barrier(0);
    make_ds(0, sa0, pa0, ds0);
    sdp(1, sa1, pa1);
    __builtin_amdgcn_sched_barrier(0);
    dqm(0, ds0);
    make_ds(1, sa1, pa1, ds1);
    __builtin_amdgcn_sched_barrier(0);
    dqm(1, ds1);
  };

  issue(t_lo, st0);
  int t = t_lo;
  for (; t + 1 < t_end; t += 2) {
    step(t, st0, st1);
    step(t + 1, st1, st0);
  }
  if (t < t_end) step(t, st0, st1);

  store_row16<T>(dQ + (long long)qrow * vdq.r, acc, scale, hh, qrow < N);
}

constexpr int kStatSlots = 64;  // LDS floats reserved for LSE (and for delta) per stage

// dK and dV for one 128-key block at d = 256; wave w owns keys 32w .. 32w+31
// of it. One wave per SIMD: the dK^T and dV^T accumulators alone take 256
// registers per lane. K^T is held as B operands in registers; V^T is read
// from an LDS copy of the block's V rows (with both in registers the kernel
// spilled). Query tiles of 32 rows (Q, dO, LSE, delta) stream through two
// LDS stages beside the V copy (64 KiB plus padding), filled one step ahead
// by direct copies.
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                 const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                 const float* __restrict__ LSE, const float* __restrict__ Dl, uint16_t* __restrict__ dK,
                 uint16_t* __restrict__ dV, View vq, View vk, View vv, View vdo, View vdk, View vdv, int H,
                 int N, int nkb, int nblocks, float c, float scale, int wl, int wr) {
  static_assert(D == 256, "d <= 128 runs dkdv8_kernel");
  // One array per stage: Q tile, dO tile, LSE (natural log), delta. (Few
  // distinct arrays, so that the compiler can still tell the copies into
  // one stage from the reads of another and does not wait on them.)
  constexpr int kQT = 32;  // query rows per step: the stages of 512-byte rows fit beside the V copy
  constexpr int TB = kQT * Tile<D>::kRS;
  constexpr int SB = 2 * TB + 2 * kStatSlots * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[SB];
  // The block's 128 V rows, rows 2d + 16 bytes apart (the 16 rows read by a
  // 16-lane phase then hit distinct banks).
  constexpr int kVS = 2 * D + 16;
  __shared__ __attribute__((aligned(1024))) unsigned char vblk[kBr * kVS];

  // With a causal mask the first key blocks have the most query tiles, so
  // they start first: decode_block's longest-first order (which counts
  // query tiles from the last) read backwards.
  int bh, kb;
  decode_block(nblocks, nkb, CAUSAL, bh, kb);
  if (CAUSAL) kb = nkb - 1 - kb;
  Q += view_base(vq, bh, H);
  K += view_base(vk, bh, H);
  V += view_base(vv, bh, H);
  dO += view_base(vdo, bh, H);
  dK += view_base(vdk, bh, H);
  dV += view_base(vdv, bh, H);
  LSE += (size_t)bh * N;
  Dl += (size_t)bh * N;
  const int qsb = 2 * vq.r, gsb = 2 * vdo.r;  // Q and dO row strides, bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int key0 = kb * kBr + 32 * wave;
  const int krow = key0 + n;
  const Operands<D> op(lane);
  using Dma = TileDma<D, kQT>;
  const typename Dma::Off qoff = Dma::lane_offset(wave, lane, qsb);
  const typename Dma::Off goff = Dma::lane_offset(wave, lane, gsb);

  // K^T as B operands: lane (n, hh), k-step s holds row krow, columns
  // 16s + 8hh .. +7.
  u32x4 kf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    kf[s] = krow < N ? *(const u32x4*)(K + (long long)krow * vk.r + 16 * s + 8 * hh) : u32x4{0, 0, 0, 0};
  // V rows of the block into LDS (zeros past N); the first step's barrier
  // makes them visible.
  for (int i = tid; i < kBr * (D / 8); i += kThreads) {
    const int r = i / (D / 8), ch = i - r * (D / 8);
    const int key = kb * kBr + r;
    const u32x4 x = key < N ? *(const u32x4*)(V + (long long)key * vv.r + 8 * ch) : u32x4{0, 0, 0, 0};
    *(u32x4*)(vblk + r * kVS + 16 * ch) = x;
  }
  // V^T B operand of k-step s (row krow, columns 16s + 8hh .. +7).
  auto vop = [&](int s) { return *(const u32x4*)(vblk + (32 * wave + n) * kVS + 32 * s + 16 * hh); };

  // Queries that see a key of the block: i - wl <= j <= i + wr.
  const int k_lo = kb * kBr;
  const int q_first = max(k_lo - wr, 0);
  const int q_last = min(min(k_lo + kBr - 1, N - 1) + wl, N - 1);
  const int qt_lo = q_first / kQT, qt_hi = q_last / kQT;

  // Rows past N of a ragged last tile keep whatever the stage held; they
  // are masked, and starting from zeros keeps them finite.
  if (N % kQT != 0) {
    for (int i = tid; i < SB / 16; i += kThreads) {
      ((u32x4*)st0)[i] = u32x4{0, 0, 0, 0};
      ((u32x4*)st1)[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) dk[t] = dv[t] = f32x16{};

  auto issue = [&](int qt, unsigned char* st) {
    const int qbase = qt * kQT;
    Dma::issue(Q + (long long)qbase * vq.r, N - qbase, qsb, st, qoff, wave);
    Dma::issue(dO + (long long)qbase * vdo.r, N - qbase, gsb, st + TB, goff, wave);
    // Each step waits for all of a wave's copies, so one wave copies the
    // statistics for all.
    if (wave == 0) {
      dma_row_stat(LSE + qbase, N - qbase, (float*)(st + 2 * TB), lane);
      dma_row_stat(Dl + qbase, N - qbase, (float*)(st + 2 * TB) + kStatSlots, lane);
    }
  };

  auto step = [&](int qt, const unsigned char* st, unsigned char* st_next) {
    const unsigned char* const qs = st;
    const unsigned char* const gs = st + TB;
    const float* const ls = (const float*)(st + 2 * TB);
    const float* const dls = ls + kStatSlots;
    // This step's copies are the only ones in flight; after the barrier
    // the other stage (step qt - 1) takes step qt + 1 (past the last step
    // the copy repeats the last tile, so every step issues the same copies).
    wait_vmcnt<0>();
    tile_barrier();
    issue(min(qt + 1, qt_hi), st_next);
    const int qbase = qt * kQT;
    // Skip the step if no query of it sees a key of the wave; take the
    // unmasked path if every query of it sees every key of the wave.
    if (key0 > qbase + kQT - 1 + wr || key0 + 31 < qbase - wl) return;
    const bool full = key0 + 31 < N && qbase + kQT <= N && key0 + 31 <= qbase + wr &&
                      key0 >= qbase + kQT - 1 - wl;
#pragma unroll
    for (int qh = 0; qh < kQT / 32; ++qh) {
      const int qb = qbase + 32 * qh;
      // S = Q K^T and dP = dO V^T (queries x keys): lane (n, hh), register r
      // holds query qb + perm_row(r, hh) and key krow. Reads run 8 ahead of
      // the MFMAs.
      f32x16 sa = {}, ga = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sa = T::mfma(op.row(qs, 32 * qh, s), kf[s], sa);
        ga = T::mfma(op.row(gs, 32 * qh, s), vop(s), ga);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Row statistics of the lane's 16 queries: 4 runs of 4 consecutive.
      float l2[16], dl[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int o = 32 * qh + perm_row(4 * g, hh);
        const f32x4 a = *(const f32x4*)(ls + o);
        const f32x4 b = *(const f32x4*)(dls + o);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          l2[4 * g + i] = a[i] * kLog2e;
          dl[4 * g + i] = b[i];
        }
      }
      // P = exp2(S c - lse2) on visible pairs, dS = P (dP - D); both packed
      // as B operands: chunk cc holds queries qb + 16cc + 8hh .. +7. An
      // invisible pair (or a query past N) gets lse2 = +inf, hence P = 0.
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb + perm_row(r, hh);
          const bool vis = (krow < N) & (q < N) & (krow <= q + wr) & (krow >= q - wl);
          l2[r] = vis ? l2[r] : INFINITY;
        }
      }
      u32x4 pp[2], dsp[2];
      auto make_chunk = [&](int cc) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float pv[2], dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 8 * cc + 2 * w + e;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -l2[r]));
            pv[e] = p;
            dsv[e] = p * (ga[r] - dl[r]);
          }
          pp[cc][w] = T::pack(pv[0], pv[1]);
          dsp[cc][w] = T::pack(dsv[0], dsv[1]);
        }
      };
      make_chunk(0);
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS over the step's two 16-query
      // k-steps; the second chunk's exponentials run beside the first
      // k-step's MFMAs.
#pragma unroll
      for (int tb = 0; tb < D / 32; ++tb) {
        dv[tb] = T::mfma(op.tr(gs, 2 * qh, tb), pp[0], dv[tb]);
        dk[tb] = T::mfma(op.tr(qs, 2 * qh, tb), dsp[0], dk[tb]);
      }
      make_chunk(1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < D / 32; ++tb) {
        dv[tb] = T::mfma(op.tr(gs, 2 * qh + 1, tb), pp[1], dv[tb]);
        dk[tb] = T::mfma(op.tr(qs, 2 * qh + 1, tb), dsp[1], dk[tb]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The first step in flight, then two steps per turn of the ring.
  int qt = qt_lo;
  issue(qt_lo, st0);
  for (; qt + 1 <= qt_hi; qt += 2) {
    step(qt, st0, st1);
    step(qt + 1, st1, st0);
  }
  if (qt <= qt_hi) step(qt, st0, st1);
  // The repeated copies of the last steps land before the wave ends.
  wait_vmcnt<0>();

  store_row16<T>(dK + (long long)krow * vdk.r, dk, scale, hh, krow < N);
  store_row16<T>(dV + (long long)krow * vdv.r, dv, 1.f, hh, krow < N);
}


// dK and dV for one 128-key block with eight waves, two per SIMD (d <= 128).
// Wave w owns keys 32 (w & 3) .. +31 of the block and the 32-query half
// w >> 2 of every 64-query step, so the two waves of a key range (w and
// w + 4) sum different queries into their dK^T, dV^T accumulators, and add
// them through LDS at the end. With one wave per SIMD (dkdv_kernel) a wave
// issues its LDS reads, exponentials, copies and products in order and
// they add up; a second wave per SIMD fills those gaps. To fit two waves
// (256 registers each) the K^T and V^T operands are read from LDS copies
// of the block's K and V rows instead of registers, and the query tiles
// stream through a ring of stages beside them: three at d = 64, two at
// d = 128 (refilled one step ahead), for which there is room.
constexpr int kThreads8 = 512;  // 8 waves of 64

template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads8, kThreads8), amdgpu_waves_per_eu(2, 2)))
void dkdv8_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                  const float* __restrict__ LSE, const float* __restrict__ Dl, uint16_t* __restrict__ dK,
                  uint16_t* __restrict__ dV, View vq, View vk, View vv, View vdo, View vdk, View vdv, int H,
                  int N, int nkb, int nblocks, float c, float scale, int wl, int wr) {
  static_assert(D <= 128, "two waves per SIMD hold the accumulators of d <= 128 only");
  constexpr int kStages = D <= 64 ? 3 : 2;
  constexpr int kQT = 64;  // query rows per step
  constexpr int TB = kQT * Tile<D>::kRS;
  constexpr int SB = 2 * TB + 2 * kStatSlots * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[kStages == 3 ? SB : 16];
  // The block's 128 K and V rows, rows 2d + 16 bytes apart (the 16 rows
  // read by a 16-lane phase then hit distinct banks).
  constexpr int kVS = 2 * D + 16;
  __shared__ __attribute__((aligned(1024))) unsigned char kblk[kBr * kVS];
  __shared__ __attribute__((aligned(1024))) unsigned char vblk[kBr * kVS];

  int bh, kb;
  decode_block(nblocks, nkb, CAUSAL, bh, kb);
  if (CAUSAL) kb = nkb - 1 - kb;
  Q += view_base(vq, bh, H);
  K += view_base(vk, bh, H);
  V += view_base(vv, bh, H);
  dO += view_base(vdo, bh, H);
  dK += view_base(vdk, bh, H);
  dV += view_base(vdv, bh, H);
  LSE += (size_t)bh * N;
  Dl += (size_t)bh * N;
  const int qsb = 2 * vq.r, gsb = 2 * vdo.r;  // Q and dO row strides, bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3;   // key range of the wave
  const int qh = wave >> 2;  // query half of every step
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int key0 = kb * kBr + 32 * kw;
  const int krow = key0 + n;
  const Operands<D> op(lane);
  using Dma = TileDma<D, kQT, 8>;
  const typename Dma::Off qoff = Dma::lane_offset(wave, lane, qsb);
  const typename Dma::Off goff = Dma::lane_offset(wave, lane, gsb);

  // K and V rows of the block into LDS (zeros past N); the first step's
  // barrier makes them visible.
  for (int i = tid; i < kBr * (D / 8); i += kThreads8) {
    const int r = i / (D / 8), ch = i - r * (D / 8);
    const int key = kb * kBr + r;
    const u32x4 kx = key < N ? *(const u32x4*)(K + (long long)key * vk.r + 8 * ch) : u32x4{0, 0, 0, 0};
    const u32x4 vx = key < N ? *(const u32x4*)(V + (long long)key * vv.r + 8 * ch) : u32x4{0, 0, 0, 0};
    *(u32x4*)(kblk + r * kVS + 16 * ch) = kx;
    *(u32x4*)(vblk + r * kVS + 16 * ch) = vx;
  }
  // K^T and V^T B operands of k-step s: row krow, columns 16s + 8hh .. +7.
  const int kvo = (32 * kw + n) * kVS + 16 * hh;
  auto kop = [&](int s) { return *(const u32x4*)(kblk + kvo + 32 * s); };
  auto vop = [&](int s) { return *(const u32x4*)(vblk + kvo + 32 * s); };

  // Queries that see a key of the block: i - wl <= j <= i + wr.
  const int k_lo = kb * kBr;
  const int q_first = max(k_lo - wr, 0);
  const int q_last = min(min(k_lo + kBr - 1, N - 1) + wl, N - 1);
  const int qt_lo = q_first / kQT, qt_hi = q_last / kQT;

  // Rows past N of a ragged last tile keep whatever the stage held; they
  // are masked, and starting from zeros keeps them finite.
  if (N % kQT != 0) {
    for (int i = tid; i < SB / 16; i += kThreads8) {
      ((u32x4*)st0)[i] = u32x4{0, 0, 0, 0};
      ((u32x4*)st1)[i] = u32x4{0, 0, 0, 0};
      if constexpr (kStages == 3) ((u32x4*)st2)[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) dk[t] = dv[t] = f32x16{};

  constexpr int kCopies = 2 * Dma::kPW + 2;  // per wave per step (three stages)
  auto issue = [&](int qt, unsigned char* st) {
    const int qbase = qt * kQT;
    Dma::issue(Q + (long long)qbase * vq.r, N - qbase, qsb, st, qoff, wave);
    Dma::issue(dO + (long long)qbase * vdo.r, N - qbase, gsb, st + TB, goff, wave);
    // With three stages every wave copies the (same) statistics, so that
    // all waves issue the same number of copies for the wait counts; with
    // two, each step waits for all of a wave's copies, and wave 0 alone
    // copies them.
    if (kStages == 3 || wave == 0) {
      dma_row_stat(LSE + qbase, N - qbase, (float*)(st + 2 * TB), lane);
      dma_row_stat(Dl + qbase, N - qbase, (float*)(st + 2 * TB) + kStatSlots, lane);
    }
  };

  auto step = [&](int qt, const unsigned char* st, unsigned char* st_next) {
    const unsigned char* const qs = st;
    const unsigned char* const gs = st + TB;
    const float* const ls = (const float*)(st + 2 * TB);
    const float* const dls = ls + kStatSlots;
    if constexpr (kStages == 3) {
      // This step's copies landed (those issued one step later may still
      // fly), then every wave's copies are visible; the stage of step
      // qt - 1 is free and takes step qt + 2 (past the last step the copy
      // repeats the last tile, so every step waits for the same count).
      wait_vmcnt<kCopies>();
      tile_barrier();
      issue(min(qt + 2, qt_hi), st_next);
    } else {
      // Two stages: this step's copies are the only ones in flight; after
      // the barrier the other stage (step qt - 1) takes step qt + 1.
      wait_vmcnt<0>();
      tile_barrier();
      issue(min(qt + 1, qt_hi), st_next);
    }
    const int qb = qt * kQT + 32 * qh;
    // Skip the half if none of its queries sees a key of the wave; take the
    // unmasked path if every one of them sees every key of the wave.
    if (key0 > qb + 31 + wr || key0 + 31 < qb - wl) return;
    const bool full = key0 + 31 < N && qb + 32 <= N && key0 + 31 <= qb + wr && key0 >= qb + 31 - wl;
    // S = Q K^T, then dP = dO V^T (queries x keys): lane (n, hh), register
    // r holds query qb + perm_row(r, hh) and key krow. The S chain's operand
    // reads all go out before its products: asked to interleave them one or
    // two products ahead, the compiler kept each read next to its product
    // and waited for it there (1-8% slower over d = 64..256). P =
    // exp2(S c - lse2) only needs S, so its exponentials are scheduled with
    // the dP products; pairs a row may not see are set to 0 after that
    // block, whose mask branch would otherwise split it.
    f32x16 sa = {}, ga = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sa = T::mfma(op.row(qs, 32 * qh, s), kop(s), sa);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (D / 16), 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, D / 16, 0);
    __builtin_amdgcn_sched_barrier(0);
    // Row statistics of the lane's 16 queries (4 runs of 4 consecutive).
    float pr[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 la = *(const f32x4*)(ls + 32 * qh + perm_row(4 * g, hh));
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[4 * g + i] = la[i] * kLog2e;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) ga = T::mfma(op.row(gs, 32 * qh, s), vop(s), ga);
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -pr[r]));
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (D / 16), 0);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qb + perm_row(r, hh);
        const bool vis = (krow < N) & (q < N) & (krow <= q + wr) & (krow >= q - wl);
        pr[r] = vis ? pr[r] : 0.f;
      }
    }
    u32x4 pp[2], dsp[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int w = 0; w < 4; ++w) pp[cc][w] = T::pack(pr[8 * cc + 2 * w], pr[8 * cc + 2 * w + 1]);
    // dS = P (dP - D), packed as the B operand of dK.
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x4 da = *(const f32x4*)(dls + 32 * qh + perm_row(8 * cc + 4 * g, hh));
        const int r = 8 * cc + 4 * g;
        dsp[cc][2 * g] = T::pack(pr[r] * (ga[r] - da[0]), pr[r + 1] * (ga[r + 1] - da[1]));
        dsp[cc][2 * g + 1] = T::pack(pr[r + 2] * (ga[r + 2] - da[2]), pr[r + 3] * (ga[r + 3] - da[3]));
      }
    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO^T P and dK^T += Q^T dS over the half's two 16-query
    // k-steps.
#pragma unroll
    for (int tb = 0; tb < D / 32; ++tb) {
      dv[tb] = T::mfma(op.tr(gs, 2 * qh, tb), pp[0], dv[tb]);
      dk[tb] = T::mfma(op.tr(qs, 2 * qh, tb), dsp[0], dk[tb]);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < D / 32; ++tb) {
      dv[tb] = T::mfma(op.tr(gs, 2 * qh + 1, tb), pp[1], dv[tb]);
      dk[tb] = T::mfma(op.tr(qs, 2 * qh + 1, tb), dsp[1], dk[tb]);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  int qt = qt_lo;
  if constexpr (kStages == 3) {
    issue(qt_lo, st0);
    issue(min(qt_lo + 1, qt_hi), st1);
    for (; qt + 2 <= qt_hi; qt += 3) {
      step(qt, st0, st2);
      step(qt + 1, st1, st0);
      step(qt + 2, st2, st1);
    }
    if (qt <= qt_hi) step(qt, st0, st2);
    if (qt + 1 <= qt_hi) step(qt + 1, st1, st0);
  } else {
    issue(qt_lo, st0);
    for (; qt + 1 <= qt_hi; qt += 2) {
      step(qt, st0, st1);
      step(qt + 1, st1, st0);
    }
    if (qt <= qt_hi) step(qt, st0, st1);
  }
  // The repeated copies of the last steps land, and every wave is done
  // reading the stages and the K and V copies, before they take the
  // partial sums.
  wait_vmcnt<0>();
  __syncthreads();

  // Wave w + 4 hands its dK^T partial to wave w, which hands back its dV^T
  // partial: PB bytes each, 16 bytes per lane per 4 accumulator registers.
  constexpr int PB = (D / 32) * 4 * 64 * 16;
  static_assert(2 * PB <= SB && 2 * PB <= kBr * kVS, "partial sums fit the stage and block arrays");
  // The upper wave's partial goes to the K or V copy, the lower wave's to a
  // stage; each reads its partner's.
  const bool upper = qh != 0;
  unsigned char* const part_up = (kw < 2 ? kblk : vblk) + (kw & 1) * PB;
  unsigned char* const part_lo = (kw < 2 ? st0 : st1) + (kw & 1) * PB;
  auto put = [&](const f32x16(&a)[D / 32], unsigned char* dst) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(dst + ((4 * t + g) * 64 + lane) * 16) =
            f32x4{a[t][4 * g], a[t][4 * g + 1], a[t][4 * g + 2], a[t][4 * g + 3]};
  };
  auto add = [&](f32x16(&a)[D / 32], const unsigned char* src) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = *(const f32x4*)(src + ((4 * t + g) * 64 + lane) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[t][4 * g + i] += x[i];
      }
  };
  if (upper)
    put(dk, part_up);
  else
    put(dv, part_lo);
  __syncthreads();
  // Rows krow of dK (lower wave, times scale) or dV (upper wave).
  if (upper) {
    add(dv, part_lo);
    store_row16<T>(dV + (long long)krow * vdv.r, dv, 1.f, hh, krow < N);
  } else {
    add(dk, part_up);
    store_row16<T>(dK + (long long)krow * vdk.r, dk, scale, hh, krow < N);
  }
}

}  // namespace bwd
}  // namespace fa

namespace {

template <class T>
struct BwdKernels {
  const void* dq;
  const void* dkdv;
  int dkdv_threads;
};

template <class T, int D>
BwdKernels<T> pick_d(bool causal) {
  const void* dq = causal ? (const void*)fa::bwd::dq_kernel<T, D, true> : (const void*)fa::bwd::dq_kernel<T, D, false>;
  if constexpr (D >= 256) {
    // One wave per SIMD, V^T read from LDS.
    return {dq, causal ? (const void*)fa::bwd::dkdv_kernel<T, D, true> : (const void*)fa::bwd::dkdv_kernel<T, D, false>,
            fa::kThreads};
  } else {
    return {dq, causal ? (const void*)fa::bwd::dkdv8_kernel<T, D, true> : (const void*)fa::bwd::dkdv8_kernel<T, D, false>,
            fa::bwd::kThreads8};
  }
}

template <class T>
BwdKernels<T> pick(int d, bool causal) {
  return d == 64 ? pick_d<T, 64>(causal) : d == 128 ? pick_d<T, 128>(causal) : pick_d<T, 256>(causal);
}

}  // namespace

namespace {

// Everything fa_bwd_strided checks, without a HIP call. On FA_OK, blocks is
// the launch size (0: nothing to do) and view the kernels' operands.
struct BwdPlan {
  long long tiles = 0, blocks = 0;
  fa::View view[8];
};

int plan_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* delta, const long long* strides, int B, int H, int N, int d,
             float scale, int causal, int window_left, int window_right, int dtype, BwdPlan* plan) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (window_left < -1 || window_right < -1) return FA_ERR_ARG;
  if (N > (1 << 30) - fa::kBr) return FA_ERR_SHAPE;
  const long long tiles = (N + fa::kBr - 1) / fa::kBr;
  const long long blocks = (long long)B * (long long)H * tiles;
  if (blocks > INT_MAX) return FA_ERR_SHAPE;
  plan->tiles = tiles;
  plan->blocks = blocks;
  if (blocks == 0) return FA_OK;
  // The eight [B, H, N, d] operands in the order of the strides array: five
  // inputs, then the three gradients.
  const void* ptrs[8] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!p) return FA_ERR_NULL;
  if (!lse || !delta) return FA_ERR_NULL;
  if (((uintptr_t)lse | (uintptr_t)delta) & 3) return FA_ERR_ALIGN;
  const fa::host::Dims g{B, H, N, d, 2};
  fa::host::Operand op[8];
  for (int i = 0; i < 8; ++i) {
    const int st = fa::host::make_operand(ptrs[i], strides ? strides + 3 * i : nullptr, g, &op[i], &plan->view[i]);
    if (st != FA_OK) return st;
  }
  // Outputs: each gradient is free of self-overlap and shares no byte with
  // another operand; delta shares none with anything.
  const long long rb = (long long)B * H * N * (long long)sizeof(float);
  for (int i = 5; i < 8; ++i) {
    if (!fa::host::self_disjoint(op[i], g)) return FA_ERR_ARG;
    for (int j = 0; j < 8; ++j)
      if (j != i && !fa::host::disjoint(op[i], op[j], g)) return FA_ERR_ARG;
    if (fa::host::ranges_overlap((uintptr_t)lse, rb, op[i].p, op[i].span)) return FA_ERR_ARG;
  }
  for (int j = 0; j < 8; ++j)
    if (fa::host::ranges_overlap((uintptr_t)delta, rb, op[j].p, op[j].span)) return FA_ERR_ARG;
  if (fa::host::ranges_overlap((uintptr_t)delta, rb, (uintptr_t)lse, rb)) return FA_ERR_ARG;
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_strided_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                    const void* dout, void* dq, void* dk, void* dv, float* delta,
                                    const long long* strides, int B, int H, int N, int d, float scale,
                                    int causal, int window_left, int window_right, int dtype) {
  BwdPlan plan;
  return plan_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, strides, B, H, N, d, scale, causal, window_left,
                  window_right, dtype, &plan);
}

extern "C" int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, float* delta,
                              const long long* strides, int B, int H, int N, int d, float scale, int causal,
                              int window_left, int window_right, int dtype, void* stream) {
  BwdPlan plan;
  const int status = plan_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, strides, B, H, N, d, scale, causal,
                              window_left, window_right, dtype, &plan);
  if (status != FA_OK || plan.blocks == 0) return status;
  const long long tiles = plan.tiles, blocks = plan.blocks;
  fa::View* const view = plan.view;

  const void* kq;
  const void* kkv;
  int kv_threads;
  if (dtype == FA_BF16) {
    const auto kk = pick<fa::Bf16>(d, causal != 0);
    kq = kk.dq, kkv = kk.dkdv, kv_threads = kk.dkdv_threads;
  } else {
    const auto kk = pick<fa::F16>(d, causal != 0);
    kq = kk.dq, kkv = kk.dkdv, kv_threads = kk.dkdv_threads;
  }
  hipStream_t st = (hipStream_t)stream;
  int h_arg = H, n_arg = N;

  constexpr int kUnbounded = 1 << 30;
  int wl = window_left < 0 ? kUnbounded : window_left;
  int wr = window_right < 0 ? kUnbounded : window_right;
  if (causal) wr = 0;
  float c = (float)((double)scale * 1.4426950408889634074);
  float sc = scale;
  int nt = (int)tiles, nb = (int)blocks;
  // dq_kernel writes the row sums D into delta; dkdv_kernel reads them.
  void* qargs[] = {(void*)&q,       (void*)&k,       (void*)&v,       (void*)&dout,    (void*)&o,
                   (void*)&lse,     (void*)&delta,   (void*)&dq,      (void*)&view[0], (void*)&view[1],
                   (void*)&view[2], (void*)&view[4], (void*)&view[3], (void*)&view[5], (void*)&h_arg,
                   (void*)&n_arg,   (void*)&nt,      (void*)&nb,      (void*)&c,       (void*)&sc,
                   (void*)&wl,      (void*)&wr};
  if (hipLaunchKernel(kq, dim3((unsigned)blocks), dim3(fa::kThreads), qargs, 0, st) != hipSuccess)
    return FA_ERR_LAUNCH;
  const float* delta_c = delta;
  void* kargs[] = {(void*)&q,       (void*)&k,       (void*)&v,       (void*)&dout,    (void*)&lse,
                   (void*)&delta_c, (void*)&dk,      (void*)&dv,      (void*)&view[0], (void*)&view[1],
                   (void*)&view[2], (void*)&view[4], (void*)&view[6], (void*)&view[7], (void*)&h_arg,
                   (void*)&n_arg,   (void*)&nt,      (void*)&nb,      (void*)&c,       (void*)&sc,
                   (void*)&wl,      (void*)&wr};
  if (hipLaunchKernel(kkv, dim3((unsigned)blocks), dim3((unsigned)kv_threads), kargs, 0, st) != hipSuccess)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                      int d, float scale, int causal, int window_left, int window_right, int dtype,
                      void* stream) {
  return fa_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, delta, nullptr, B, H, N, d, scale, causal,
                        window_left, window_right, dtype, stream);
}
