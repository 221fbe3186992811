// fa_fwd.hip - C ABI of the attention forward library: argument checks,
// kernel selection and launch. Declarations and the contract are in
// include/fa.h; the kernels are in fa_kernels.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_host.h"
#include "fa_kernels.h"

// tile_src's out-of-range offset for pad and filler copy slots must lie past
// every tile buffer: at most 63 rows of the largest accepted row stride plus
// one row of values.
static_assert((fa::kBc - 1) * fa::host::kMaxRowBytes + 2 * 256 <= 0x7FFFFFF0LL,
              "pad-slot offset inside a tile's buffer range");

namespace {

typedef void (*fwd16_fn)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*, fa::View,
                         fa::View, fa::View, fa::View, int, int, int, int, int, float, int, int, fa::SplitOut);
typedef void (*fwd32_fn)(const float*, const float*, const float*, float*, float*, fa::View, fa::View,
                         fa::View, fa::View, int, int, int, int, int, float, int, int, fa::SplitOut);

// bal: the balanced causal grid (two query tiles per workgroup; d = 64).
template <class T>
fwd16_fn pick16(int d, bool causal, bool bal) {
  switch (d) {
    case 64:
      return bal ? fa::fwd16_kernel<T, 64, true, true>
                 : (causal ? fa::fwd16_kernel<T, 64, true, false> : fa::fwd16_kernel<T, 64, false, false>);
    case 128:
      return causal ? fa::fwd16_kernel<T, 128, true, false> : fa::fwd16_kernel<T, 128, false, false>;
    case 256: return causal ? fa::fwd16_kernel<T, 256, true, false> : fa::fwd16_kernel<T, 256, false, false>;
  }
  return nullptr;
}

fwd32_fn pick32(int d, bool causal) {
  switch (d) {
    case 64: return causal ? fa::fwd32_kernel<64, true> : fa::fwd32_kernel<64, false>;
    case 128: return causal ? fa::fwd32_kernel<128, true> : fa::fwd32_kernel<128, false>;
    case 256: return causal ? fa::fwd32_kernel<256, true> : fa::fwd32_kernel<256, false>;
  }
  return nullptr;
}

template <class T>
const void* pick_merge(int d) {
  switch (d) {
    case 64: return (const void*)fa::merge_kernel<T, 64>;
    case 128: return (const void*)fa::merge_kernel<T, 128>;
    case 256: return (const void*)fa::merge_kernel<T, 256>;
  }
  return nullptr;
}

constexpr int kMaxSplits = 64;

// Query rows per workgroup of the kernel that serves dtype.
int rows_per_block(int dtype) { return dtype == FA_F32 ? fa::kBr32 : fa::kBr; }

// The balanced causal grid (fwd16_kernel with BAL: query tiles nqt - 1 - p
// and p in one workgroup, every workgroup the same work) serves 16-bit
// causal calls with d = 64, at least two query tiles, no left window bound
// and no split: measured 3% faster than the plain grid's longest-first
// order on B1 H64 N4096, bitwise the same. At d = 128 the two were within
// 1.3% either way (the plain grid faster on the GPT-3 shape), and at d = 256
// (one workgroup per compute unit) the plain order already hides the
// imbalance, so those keep the plain grid.
bool balanced_grid(int d, int dtype, int causal, int nqt, int window_left, int nsplit) {
  return dtype != FA_F32 && d == 64 && causal && nqt >= 2 && window_left < 0 && nsplit <= 1;
}

// Checks that do not involve pointers. Fills the launch shape on success.
int check_shape(int B, int H, int N, int d, int causal, int dtype, long long* nblocks, int* nqt) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  // Row offsets inside one head are computed in 32-bit arithmetic before
  // widening, so keep N comfortably below 2^30.
  const int rows = rows_per_block(dtype);
  if (N > (1 << 30) - fa::kBr) return FA_ERR_SHAPE;
  const long long q_tiles = (N + rows - 1) / rows;
  const long long blocks = (long long)B * (long long)H * q_tiles;
  if (blocks > INT_MAX) return FA_ERR_SHAPE;
  *nblocks = blocks;
  *nqt = (int)q_tiles;
  return FA_OK;
}

}  // namespace

extern "C" const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "a size is negative or too large";
    case FA_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA_ERR_DTYPE: return "dtype must be FA_F16, FA_BF16 or FA_F32";
    case FA_ERR_ALIGN:
      return "q, k, v, o (and every row of their views) must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ARG:
      return "causal must be 0 or 1, scale finite, window sides >= -1, every query row must see a key, "
             "and outputs must not overlap inputs, each other or themselves";
    case FA_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_SCRATCH:
      return "the split-KV partial results exceed the static scratch buffer of fa_fwd_kv_noalloc "
             "(FA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown fa_status";
}

extern "C" int fa_fwd_grid(int B, int H, int N, int d, int causal, int dtype, long long* workgroups,
                           int* rows_per_workgroup) {
  long long nblocks = 0;
  int nqt = 0;
  const int st = check_shape(B, H, N, d, causal, dtype, &nblocks, &nqt);
  if (st != FA_OK) return st;
  const bool bal = balanced_grid(d, dtype, causal, nqt, -1, 1);
  if (workgroups) *workgroups = bal ? nblocks / nqt * ((nqt + 1) / 2) : nblocks;
  if (rows_per_workgroup) *rows_per_workgroup = rows_per_block(dtype);
  return FA_OK;
}

namespace {

// Everything fa_fwd_strided checks, without a HIP call. On FA_OK, nblocks
// is the launch size (0: nothing to do) and view the kernels' operands.
struct FwdPlan {
  long long nblocks = 0;
  int nqt = 0;
  fa::View view[4];
};

// N query rows against Nk key rows (the queries are the last N positions).
int plan_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const long long* strides, int B,
             int H, int N, int Nk, int d, float scale, int causal, int window_left, int window_right, int dtype,
             FwdPlan* plan) {
  int st = check_shape(B, H, N, d, causal, dtype, &plan->nblocks, &plan->nqt);
  if (st != FA_OK) return st;
  if (Nk < 0 || Nk > (1 << 30) - fa::kBr) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (window_left < -1 || window_right < -1) return FA_ERR_ARG;
  if (plan->nblocks == 0) return FA_OK;  // B*H*N == 0: nothing to do
  // Every query row must see a key: some key at all, and with a causal
  // mask or a window no query before the first key position.
  if (Nk == 0) return FA_ERR_ARG;
  if (N > Nk && (causal || window_left >= 0 || window_right >= 0)) return FA_ERR_ARG;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;

  const fa::host::Dims g{B, H, N, d, dtype == FA_F32 ? 4 : 2};
  const fa::host::Dims gk{B, H, Nk, d, g.esz};
  const void* ptrs[4] = {q, k, v, o};
  fa::host::Operand op[4];
  for (int i = 0; i < 4; ++i) {
    st = fa::host::make_operand(ptrs[i], strides ? strides + 3 * i : nullptr, (i == 1 || i == 2) ? gk : g, &op[i],
                                &plan->view[i]);
    if (st != FA_OK) return st;
  }
  const long long lbytes = (long long)B * H * N * (long long)sizeof(float);
  if (!fa::host::self_disjoint(op[3], g)) return FA_ERR_ARG;
  for (int i = 0; i < 3; ++i)
    if (!fa::host::disjoint(op[3], op[i], g)) return FA_ERR_ARG;
  for (int i = 0; i < 4; ++i)
    if (fa::host::ranges_overlap((uintptr_t)lse, lbytes, op[i].p, op[i].span)) return FA_ERR_ARG;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_strided_check(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const long long* strides, int B, int H, int N, int d, float scale,
                                    int causal, int window_left, int window_right, int dtype) {
  FwdPlan plan;
  return plan_fwd(q, k, v, o, lse, strides, B, H, N, N, d, scale, causal, window_left, window_right, dtype, &plan);
}

namespace {

// Workgroups of the forward kernel that fit on the chip at once (256
// compute units; two per unit where the kernel runs two waves per SIMD).
int resident_blocks(int d, int dtype) { return (dtype == FA_F32 || d == 256) ? 256 : 512; }

// Key tiles per part (of the widest query tile) below which a part does
// not pay for its partial result and the merge: measured on one GPU over
// low-occupancy shapes (d = 64 .. 256, N = 256 .. 16384). Causal grids
// split at shorter ranges, because their longest query tile sets the time.
constexpr int kMinTilesCausal = 16;
constexpr int kMinTiles = 32;

// Parts for a grid of nblocks workgroups of N query rows against Nk keys:
// none while the grid fills half the chip; otherwise, as long as each part
// of the widest query tile keeps the minimum number of key tiles:
//  * N of at least half a query tile (the work is matrix-core bound):
//    enough parts to fill every resident slot, at most 16;
//  * fewer rows (a decode step: streaming K and V from HBM sets the time):
//    about one workgroup per compute unit, at most 64.
// Both targets come from sweeps on one GPU (d = 64 .. 256).
int choose_splits(long long nblocks, int N, int Nk, int d, int causal, int wl, int wr, int dtype) {
  const int slots = resident_blocks(d, dtype);
  if (nblocks * 2 > slots) return 1;
  long long span = (long long)rows_per_block(dtype) + (wl < 0 ? Nk : wl) + (causal || wr == 0 ? 0 : (wr < 0 ? Nk : wr));
  span = std::min<long long>(span, Nk);
  const int tiles = (int)((span + fa::kBc - 1) / fa::kBc);
  const bool decode = N <= rows_per_block(dtype) / 2;
  int s = (int)((decode ? 256 : slots) / std::max<long long>(nblocks, 1));
  s = std::min(s, tiles / (causal ? kMinTilesCausal : kMinTiles));
  s = std::min(s, decode ? kMaxSplits : 16);
  return std::max(s, 1);
}

long long workspace_bytes_for(int B, int H, int N, int d, int nsplit) {
  if (nsplit <= 1) return 0;
  return (long long)nsplit * B * H * N * (long long)(d + 1) * (long long)sizeof(float);
}

// Enqueues the forward kernel (and, with a split, the merge) for a plan
// that passed plan_fwd.
int launch_fwd(const FwdPlan& plan, const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int H, int N, int Nk, int d, float scale, int causal, int window_left, int window_right, int dtype,
               float* part, int nsplit, hipStream_t stream) {
  // log2(e) is folded into the scale: exp(x * scale) == exp2(x * c).
  const float c = (float)((double)scale * 1.4426950408889634074);
  const bool bal = balanced_grid(d, dtype, causal, plan.nqt, window_left, nsplit);
  const long long grid = bal ? plan.nblocks / plan.nqt * ((plan.nqt + 1) / 2) : plan.nblocks;
  int h_arg = H, n_arg = N, nk_arg = Nk, nqt_arg = plan.nqt, nb_arg = (int)grid;
  float c_arg = c;
  // Visible keys of the query at position p: p - wl .. p + wr, an unbounded
  // side as 2^30 (positions are below 2^30, so no sum with a side overflows).
  constexpr int kUnbounded = 1 << 30;
  int wl = window_left < 0 ? kUnbounded : window_left;
  int wr = window_right < 0 ? kUnbounded : window_right;
  if (causal) wr = 0;
  fa::View view[4] = {plan.view[0], plan.view[1], plan.view[2], plan.view[3]};
  fa::SplitOut sp{nsplit > 1 ? part : nullptr, nsplit > 1 ? nsplit : 1, B * H};
  void* args[] = {(void*)&q,       (void*)&k,       (void*)&v,       (void*)&o,     (void*)&lse,
                  (void*)&view[0], (void*)&view[1], (void*)&view[2], (void*)&view[3], (void*)&h_arg,
                  (void*)&n_arg,   (void*)&nk_arg,  (void*)&nqt_arg, (void*)&nb_arg,  (void*)&c_arg,
                  (void*)&wl,      (void*)&wr,      (void*)&sp};

  const void* fn = nullptr;
  const void* merge = nullptr;
  if (dtype == FA_F32) {
    fn = (const void*)pick32(d, causal != 0);
    merge = pick_merge<float>(d);
  } else if (dtype == FA_BF16) {
    fn = (const void*)pick16<fa::Bf16>(d, causal != 0, bal);
    merge = pick_merge<fa::Bf16>(d);
  } else {
    fn = (const void*)pick16<fa::F16>(d, causal != 0, bal);
    merge = pick_merge<fa::F16>(d);
  }
  if (!fn || !merge) return FA_ERR_HEADDIM;
  long long rows = (long long)B * H * N;
  const int rpb = fa::kThreads / (d / 4);  // rows per merge workgroup
  const long long mblocks = (rows + rpb - 1) / rpb;
  if (sp.part && mblocks > INT_MAX) return FA_ERR_SHAPE;
  const int threads = dtype == FA_F32 ? (d <= 128 ? fa::fwd32_threads<64>() : fa::fwd32_threads<256>()) : fa::kThreads;
  if (hipLaunchKernel(fn, dim3((unsigned)grid, (unsigned)sp.nsplit), dim3((unsigned)threads), args, 0, stream) !=
      hipSuccess)
    return FA_ERR_LAUNCH;
  if (sp.part) {
    const float* part_c = part;
    int ns = nsplit;
    fa::View vo = view[3];
    void* margs[] = {(void*)&part_c, (void*)&ns, (void*)&o, (void*)&vo, (void*)&lse, (void*)&h_arg, (void*)&n_arg,
                     (void*)&rows};
    if (hipLaunchKernel(merge, dim3((unsigned)mblocks), dim3(fa::kThreads), margs, 0, stream) != hipSuccess)
      return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace

namespace {

int fwd_general(const void* q, const void* k, const void* v, void* o, float* lse, const long long* strides,
                void* workspace, long long workspace_bytes, int num_splits, int B, int H, int N, int Nk, int d,
                float scale, int causal, int window_left, int window_right, int dtype, void* stream) {
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  FwdPlan plan;
  int st =
      plan_fwd(q, k, v, o, lse, strides, B, H, N, Nk, d, scale, causal, window_left, window_right, dtype, &plan);
  if (st != FA_OK || plan.nblocks == 0) return st;
  int ns = num_splits == 0 ? choose_splits(plan.nblocks, N, Nk, d, causal, window_left, window_right, dtype)
                           : num_splits;
  float* part = nullptr;
  if (ns > 1) {
    const long long need = workspace_bytes_for(B, H, N, d, ns);
    if (!workspace) return FA_ERR_NULL;
    if ((uintptr_t)workspace & 15) return FA_ERR_ALIGN;
    if (workspace_bytes < need) return FA_ERR_ARG;
    // The workspace is written: it may not overlap any operand.
    const fa::host::Dims g{B, H, N, d, dtype == FA_F32 ? 4 : 2};
    const fa::host::Dims gk{B, H, Nk, d, g.esz};
    const void* ptrs[4] = {q, k, v, o};
    for (int i = 0; i < 4; ++i) {
      fa::host::Operand op;
      fa::View unused;
      st = fa::host::make_operand(ptrs[i], strides ? strides + 3 * i : nullptr, (i == 1 || i == 2) ? gk : g, &op,
                                  &unused);
      if (st != FA_OK) return st;
      if (fa::host::ranges_overlap((uintptr_t)workspace, need, op.p, op.span)) return FA_ERR_ARG;
    }
    if (fa::host::ranges_overlap((uintptr_t)workspace, need, (uintptr_t)lse,
                                 (long long)B * H * N * (long long)sizeof(float)))
      return FA_ERR_ARG;
    part = (float*)workspace;
  }
  return launch_fwd(plan, q, k, v, o, lse, B, H, N, Nk, d, scale, causal, window_left, window_right, dtype, part,
                    ns, (hipStream_t)stream);
}

}  // namespace

extern "C" int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                              const long long* strides, int B, int H, int N, int d, float scale, int causal,
                              int window_left, int window_right, int dtype, void* stream) {
  return fwd_general(q, k, v, o, lse, strides, nullptr, 0, 1, B, H, N, N, d, scale, causal, window_left,
                     window_right, dtype, stream);
}

extern "C" int fa_fwd_num_splits(int B, int H, int N, int d, int causal, int window_left, int window_right,
                                 int dtype, int* num_splits) {
  return fa_fwd_kv_num_splits(B, H, N, N, d, causal, window_left, window_right, dtype, num_splits);
}

extern "C" int fa_fwd_kv_num_splits(int B, int H, int N, int Nk, int d, int causal, int window_left,
                                    int window_right, int dtype, int* num_splits) {
  long long nblocks = 0;
  int nqt = 0;
  const int st = check_shape(B, H, N, d, causal, dtype, &nblocks, &nqt);
  if (st != FA_OK) return st;
  if (Nk < 0 || Nk > (1 << 30) - fa::kBr) return FA_ERR_SHAPE;
  if (window_left < -1 || window_right < -1) return FA_ERR_ARG;
  if (!num_splits) return FA_ERR_NULL;
  *num_splits =
      nblocks == 0 || Nk == 0 ? 1 : choose_splits(nblocks, N, Nk, d, causal, window_left, window_right, dtype);
  return FA_OK;
}

extern "C" int fa_fwd_splitkv_workspace(int B, int H, int N, int d, int num_splits, long long* bytes) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  if (!bytes) return FA_ERR_NULL;
  *bytes = workspace_bytes_for(B, H, N, d, num_splits);
  return FA_OK;
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              const long long* strides, void* workspace, long long workspace_bytes, int num_splits,
                              int B, int H, int N, int d, float scale, int causal, int window_left,
                              int window_right, int dtype, void* stream) {
  return fwd_general(q, k, v, o, lse, strides, workspace, workspace_bytes, num_splits, B, H, N, N, d, scale, causal,
                     window_left, window_right, dtype, stream);
}

extern "C" int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, const long long* strides,
                         void* workspace, long long workspace_bytes, int num_splits, int B, int H, int N, int Nk,
                         int d, float scale, int causal, int window_left, int window_right, int dtype,
                         void* stream) {
  return fwd_general(q, k, v, o, lse, strides, workspace, workspace_bytes, num_splits, B, H, N, Nk, d, scale, causal,
                     window_left, window_right, dtype, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free split-KV forward (fa_fwd_kv_noalloc): the parts' partial
// results go to a static device array instead of a caller workspace. Each
// GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on the entry point's first call there.

static __device__ __attribute__((aligned(256))) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const long long* strides, int num_splits, int B, int H, int N, int Nk, int d,
                                 float scale, int causal, int window_left, int window_right, int dtype,
                                 void* stream) {
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  FwdPlan plan;
  int st =
      plan_fwd(q, k, v, o, lse, strides, B, H, N, Nk, d, scale, causal, window_left, window_right, dtype, &plan);
  if (st != FA_OK || plan.nblocks == 0) return st;
  const int ns = num_splits == 0
                     ? choose_splits(plan.nblocks, N, Nk, d, causal, window_left, window_right, dtype)
                     : num_splits;
  float* part = nullptr;
  if (ns > 1) {
    // Every element of the parts' region that the merge reads is written
    // by the forward kernel first (a part with no visible key of a row
    // writes O_s = 0, LSE_s = -inf), so nothing needs clearing.
    if (workspace_bytes_for(B, H, N, d, ns) > (long long)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void* p = nullptr;
    st = scratch_address(&p);
    if (st != FA_OK) return st;
    part = (float*)p;
  }
  return launch_fwd(plan, q, k, v, o, lse, B, H, N, Nk, d, scale, causal, window_left, window_right, dtype, part,
                    ns, (hipStream_t)stream);
}

extern "C" int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                             int H, int N, int d, float scale, int causal, int window_left,
                             int window_right, int dtype, void* stream) {
  return fa_fwd_strided(q, k, v, o, lse, nullptr, B, H, N, d, scale, causal, window_left, window_right, dtype,
                        stream);
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, float scale, int causal, int dtype, void* stream) {
  return fa_fwd_window(q, k, v, o, lse, B, H, N, d, scale, causal, -1, -1, dtype, stream);
}
