// fa_host.h - host-side argument checks shared by the entry points: the
// strided [B, H, N, d] views of the operands, their alignment and extent,
// and whether two of them can share memory. No HIP calls.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "fa.h"
#include "fa_kernels.h"

namespace fa {
namespace host {

// Largest row stride in bytes: the kernels form tile offsets of up to 64
// rows in 32-bit arithmetic.
constexpr long long kMaxRowBytes = 1LL << 25;

// One [B, H, N, d] operand in bytes: base address, strides, the bytes of a
// row's values (d elements) and the extent [p, p + span) of every byte the
// view can touch.
struct Operand {
  uintptr_t p = 0;
  long long sb = 0, sh = 0, sr = 0;
  long long len = 0;
  long long span = 0;
};

struct Dims {
  int B, H, N, d;
  long long esz;
};

// Builds the operand at ptr from three element strides (batch, head, row),
// or the contiguous ones if s is NULL, and the kernels' View of it. The
// stride of a dimension of extent 1 is never used, so it is replaced by the
// contiguous one (any value is accepted there). Returns FA_ERR_SHAPE for a
// negative stride, a row stride below d or above the 32-bit tile limit, or
// an extent that overflows; FA_ERR_ALIGN unless every row start is 16-byte
// aligned.
inline int make_operand(const void* ptr, const long long* s, const Dims& g, Operand* op, View* view) {
  const long long d = g.d, N = g.N, H = g.H;
  long long sb = s ? s[0] : H * N * d;
  long long sh = s ? s[1] : N * d;
  long long sr = s ? s[2] : d;
  if (g.B == 1) sb = H * N * d;
  if (g.H == 1) sh = N * d;
  if (g.N == 1) sr = d;
  if (sb < 0 || sh < 0 || sr < d) return FA_ERR_SHAPE;
  if (sr * g.esz > kMaxRowBytes) return FA_ERR_SHAPE;
  Operand o;
  o.p = (uintptr_t)ptr;
  o.len = d * g.esz;
  long long span = o.len;
  const long long st[3] = {sb, sh, sr};
  const long long ext[3] = {g.B, g.H, g.N};
  long long* const dst[3] = {&o.sb, &o.sh, &o.sr};
  for (int i = 0; i < 3; ++i) {
    long long bytes, part;
    if (__builtin_mul_overflow(st[i], g.esz, &bytes)) return FA_ERR_SHAPE;
    if (__builtin_mul_overflow(bytes, ext[i] - 1, &part)) return FA_ERR_SHAPE;
    if (__builtin_add_overflow(span, part, &span)) return FA_ERR_SHAPE;
    *dst[i] = bytes;
  }
  if (span > (1LL << 56)) return FA_ERR_SHAPE;
  o.span = span;
  if ((o.p | (uintptr_t)o.sb | (uintptr_t)o.sh | (uintptr_t)o.sr) & 15) return FA_ERR_ALIGN;
  *op = o;
  view->b = sb;
  view->h = sh;
  view->r = (int)sr;
  return FA_OK;
}

// True if no two elements of the view share a byte (so concurrent stores of
// different elements cannot race). Sufficient test: with the dimensions of
// extent > 1 taken in increasing stride order, each stride is at least the
// extent of everything below it.
inline bool self_disjoint(const Operand& o, const Dims& g) {
  std::pair<long long, long long> dims[3] = {{o.sh, g.H}, {o.sr, g.N}, {o.sb, g.B}};
  std::sort(dims, dims + 3);
  long long span = o.len;
  for (const auto& dm : dims) {
    if (dm.second <= 1) continue;
    if (dm.first < span) return false;
    span += dm.first * (dm.second - 1);  // within o.span, no overflow
  }
  return true;
}

inline bool ranges_overlap(uintptr_t a, long long na, uintptr_t b, long long nb) {
  return a < b + (uintptr_t)nb && b < a + (uintptr_t)na;
}

// Residues modulo the common row stride P of the bytes an operand touches,
// as [start, end) intervals, when every batch (and possibly head) offset is
// a multiple of P; false if the operand does not have that form.
inline bool residues(const Operand& o, const Dims& g, long long P,
                     std::vector<std::pair<long long, long long>>* out) {
  if (g.B > 1 && o.sb % P != 0) return false;
  if (o.len > P) return false;
  const int nh = (g.H > 1 && o.sh % P != 0) ? g.H : 1;
  if (nh > 4096) return false;
  const long long p0 = (long long)(o.p % (uintptr_t)P);
  for (int h = 0; h < nh; ++h) {
    const long long s = (p0 + ((long long)h * o.sh) % P) % P;
    const long long e = s + o.len;
    if (e <= P) {
      out->push_back({s, e});
    } else {
      out->push_back({s, P});
      out->push_back({0, e - P});
    }
  }
  std::sort(out->begin(), out->end());
  return true;
}

// True if the two operands cannot share a byte. Either their extents are
// apart, or they are interleaved slices of one tensor, such as the q, k and
// v slices of a packed [B, N, 3, H, d] tensor: with a common row stride P
// and batch offsets that are multiples of P, every byte of an operand lies
// at one of its residues modulo P, so disjoint residue sets mean disjoint
// bytes.
inline bool disjoint(const Operand& a, const Operand& b, const Dims& g) {
  if (!ranges_overlap(a.p, a.span, b.p, b.span)) return true;
  const long long P = a.sr;
  if (P <= 0 || b.sr != P) return false;
  std::vector<std::pair<long long, long long>> ra, rb;
  if (!residues(a, g, P, &ra) || !residues(b, g, P, &rb)) return false;
  size_t i = 0, j = 0;
  while (i < ra.size() && j < rb.size()) {
    if (ra[i].second <= rb[j].first) {
      ++i;
    } else if (rb[j].second <= ra[i].first) {
      ++j;
    } else {
      return false;
    }
  }
  return true;
}

}  // namespace host
}  // namespace fa
