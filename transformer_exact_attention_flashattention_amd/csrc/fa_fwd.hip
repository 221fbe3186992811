// fa_fwd.hip - C ABI of the attention forward library: argument checks,
// kernel selection and launch. Declarations and the contract are in
// include/fa.h; the kernels are in fa_kernels.h.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_host.h"
#include "fa_kernels.h"

namespace {

typedef void (*fwd16_fn)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*, fa::View,
                         fa::View, fa::View, fa::View, int, int, int, int, float, int, int);
typedef void (*fwd32_fn)(const float*, const float*, const float*, float*, float*, fa::View, fa::View,
                         fa::View, fa::View, int, int, int, int, float, int, int);

template <class T>
fwd16_fn pick16(int d, bool causal) {
  switch (d) {
    case 64: return causal ? fa::fwd16_kernel<T, 64, true> : fa::fwd16_kernel<T, 64, false>;
    case 128: return causal ? fa::fwd16_kernel<T, 128, true> : fa::fwd16_kernel<T, 128, false>;
    case 256: return causal ? fa::fwd16_kernel<T, 256, true> : fa::fwd16_kernel<T, 256, false>;
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

// Query rows per workgroup of the kernel that serves dtype.
int rows_per_block(int dtype) { return dtype == FA_F32 ? fa::kBr32 : fa::kBr; }

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
      return "causal must be 0 or 1, scale finite, window sides >= -1, and outputs must not overlap "
             "inputs, each other or themselves";
    case FA_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
  }
  return "unknown fa_status";
}

extern "C" int fa_fwd_grid(int B, int H, int N, int d, int causal, int dtype, long long* workgroups,
                           int* rows_per_workgroup) {
  long long nblocks = 0;
  int nqt = 0;
  const int st = check_shape(B, H, N, d, causal, dtype, &nblocks, &nqt);
  if (st != FA_OK) return st;
  if (workgroups) *workgroups = nblocks;
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

int plan_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const long long* strides, int B,
             int H, int N, int d, float scale, int causal, int window_left, int window_right, int dtype,
             FwdPlan* plan) {
  int st = check_shape(B, H, N, d, causal, dtype, &plan->nblocks, &plan->nqt);
  if (st != FA_OK) return st;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (window_left < -1 || window_right < -1) return FA_ERR_ARG;
  if (plan->nblocks == 0) return FA_OK;  // B*H*N == 0: nothing to do
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;

  const fa::host::Dims g{B, H, N, d, dtype == FA_F32 ? 4 : 2};
  const void* ptrs[4] = {q, k, v, o};
  fa::host::Operand op[4];
  for (int i = 0; i < 4; ++i) {
    st = fa::host::make_operand(ptrs[i], strides ? strides + 3 * i : nullptr, g, &op[i], &plan->view[i]);
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
  return plan_fwd(q, k, v, o, lse, strides, B, H, N, d, scale, causal, window_left, window_right, dtype, &plan);
}

extern "C" int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                              const long long* strides, int B, int H, int N, int d, float scale, int causal,
                              int window_left, int window_right, int dtype, void* stream) {
  FwdPlan plan;
  const int st =
      plan_fwd(q, k, v, o, lse, strides, B, H, N, d, scale, causal, window_left, window_right, dtype, &plan);
  if (st != FA_OK || plan.nblocks == 0) return st;

  // log2(e) is folded into the scale: exp(x * scale) == exp2(x * c).
  const float c = (float)((double)scale * 1.4426950408889634074);
  int h_arg = H, n_arg = N, nqt_arg = plan.nqt, nb_arg = (int)plan.nblocks;
  float c_arg = c;
  // Visible keys of query i: i - wl .. i + wr, an unbounded side as 2^30
  // (N is below 2^30, so no sum of a row index and a side overflows).
  constexpr int kUnbounded = 1 << 30;
  int wl = window_left < 0 ? kUnbounded : window_left;
  int wr = window_right < 0 ? kUnbounded : window_right;
  if (causal) wr = 0;
  fa::View* const view = plan.view;
  void* args[] = {(void*)&q,       (void*)&k,       (void*)&v,       (void*)&o,     (void*)&lse,
                  (void*)&view[0], (void*)&view[1], (void*)&view[2], (void*)&view[3], (void*)&h_arg,
                  (void*)&n_arg,   (void*)&nqt_arg, (void*)&nb_arg,  (void*)&c_arg, (void*)&wl,
                  (void*)&wr};

  const void* fn = nullptr;
  if (dtype == FA_F32) {
    fn = (const void*)pick32(d, causal != 0);
  } else if (dtype == FA_BF16) {
    fn = (const void*)pick16<fa::Bf16>(d, causal != 0);
  } else {
    fn = (const void*)pick16<fa::F16>(d, causal != 0);
  }
  if (!fn) return FA_ERR_HEADDIM;
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)plan.nblocks), dim3(fa::kThreads), args, 0,
                                       (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
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
