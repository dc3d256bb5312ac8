// axial_api.cpp -- the axial-attention block entries of include/mi355_attn.h:
// argument validation (pure host logic, no HIP call) and the launches.

#include <cmath>
#include <cstdint>

#include "../../include/mi355_attn.h"
#include "attn_launch.h"

namespace {

constexpr int64_t kIntMax = 2147483647;
constexpr int64_t kMaxLen = 64;

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool overlap(const void* p, int64_t n, const void* r, int64_t m) {
  if (n <= 0 || m <= 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)r;
  return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

struct Weights {
  const float* ln_w;
  const float* ln_b;
  const float* w_qkv;
  const float* w_out;
  const float* b_out;
};

// Checks one weight set: present, aligned, and clear of the output (the
// weights may overlap x, which is only read).
int check_weights(const Weights& w, const void* out, int64_t bytes, int64_t C) {
  if (!w.ln_w || !w.ln_b || !w.w_qkv || !w.w_out || !w.b_out) return MI355_ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)w.ln_w | (uintptr_t)w.ln_b | (uintptr_t)w.w_qkv | (uintptr_t)w.w_out) & 15u)
    return MI355_ATTN_ERR_MISALIGNED;
  if ((uintptr_t)w.b_out & 3u) return MI355_ATTN_ERR_MISALIGNED;
  const void* p[5] = {w.ln_w, w.ln_b, w.w_qkv, w.w_out, w.b_out};
  const int64_t n[5] = {4 * C, 4 * C, 12 * C * C, 4 * C * C, 4 * C};
  for (int i = 0; i < 5; ++i)
    if (overlap(out, bytes, p[i], n[i])) return MI355_ATTN_ERR_INVALID_ARG;
  return MI355_ATTN_OK;
}

// Shape, pointer and overlap checks shared by the pass and the block. *bytes
// receives the image size in bytes; MI355_ATTN_OK with *bytes == 0 is a no-op.
int check_image(const void* x, const void* out, int64_t B, int64_t Hh, int64_t W, int64_t C,
                int64_t heads, float eps, int64_t* bytes) {
  *bytes = 0;
  if (B < 0 || Hh < 0 || W < 0 || C < 1 || heads < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.0f) return MI355_ATTN_ERR_INVALID_ARG;
  if (C % heads != 0) return MI355_ATTN_ERR_INVALID_ARG;
  int64_t bh, tokens, elems, nbytes;
  if (!mul_ok(B, Hh, &bh) || !mul_ok(bh, W, &tokens) || !mul_ok(tokens, C, &elems) ||
      !mul_ok(elems, 4, &nbytes))
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (tokens == 0) return MI355_ATTN_OK;
  if (!x || !out) return MI355_ATTN_ERR_INVALID_ARG;
  if (C != 64 || heads != 4) return MI355_ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)x | (uintptr_t)out) & 15u) return MI355_ATTN_ERR_MISALIGNED;
  if (x != out && overlap(x, nbytes, out, nbytes)) return MI355_ATTN_ERR_INVALID_ARG;
  *bytes = nbytes;
  return MI355_ATTN_OK;
}

int check_axis(int64_t B, int64_t Hh, int64_t W, int axis) {
  if (axis != MI355_AXIAL_ROW && axis != MI355_AXIAL_COL) return MI355_ATTN_ERR_INVALID_ARG;
  const int64_t L = axis == MI355_AXIAL_ROW ? W : Hh;
  const int64_t nseq = B * (axis == MI355_AXIAL_ROW ? Hh : W);  // no overflow: checked image
  if (L > kMaxLen || nseq > kIntMax) return MI355_ATTN_ERR_UNSUPPORTED;
  return MI355_ATTN_OK;
}

int validate_pass(const float* x, const float* out, const Weights& w, int64_t B, int64_t Hh,
                  int64_t W, int64_t C, int64_t heads, int axis, float eps, int64_t* bytes) {
  if (axis != MI355_AXIAL_ROW && axis != MI355_AXIAL_COL) return MI355_ATTN_ERR_INVALID_ARG;
  int st = check_image(x, out, B, Hh, W, C, heads, eps, bytes);
  if (st != MI355_ATTN_OK || *bytes == 0) return st;
  if ((st = check_axis(B, Hh, W, axis)) != MI355_ATTN_OK) return st;
  return check_weights(w, out, *bytes, C);
}

mi355::AxialLaunchArgs pass_args(const float* x, float* out, const Weights& w, int64_t B,
                                 int64_t Hh, int64_t W, int64_t C, int axis, float eps,
                                 void* stream) {
  mi355::AxialLaunchArgs a;
  a.x = x;
  a.out = out;
  a.ln_w = w.ln_w;
  a.ln_b = w.ln_b;
  a.w_qkv = w.w_qkv;
  a.w_out = w.w_out;
  a.b_out = w.b_out;
  if (axis == MI355_AXIAL_ROW) {  // sequence (b, y): W tokens C apart
    a.nseq = B * Hh;
    a.L = W;
    a.inner = 1;
    a.outer_stride = W * C;
    a.inner_stride = 0;
    a.tstride = C;
  } else {  // sequence (b, x): Hh tokens W*C apart
    a.nseq = B * W;
    a.L = Hh;
    a.inner = W;
    a.outer_stride = Hh * W * C;
    a.inner_stride = C;
    a.tstride = W * C;
  }
  a.eps = eps;
  a.stream = (hipStream_t)stream;
  return a;
}

}  // namespace

extern "C" {

int axial_pass_validate(const float* x, const float* out, const float* ln_w, const float* ln_b,
                        const float* w_qkv, const float* w_out, const float* b_out, int64_t B,
                        int64_t Hh, int64_t W, int64_t C, int64_t heads, int axis, float eps) {
  int64_t bytes;
  return validate_pass(x, out, {ln_w, ln_b, w_qkv, w_out, b_out}, B, Hh, W, C, heads, axis, eps,
                       &bytes);
}

int axial_pass(const float* x, float* out, const float* ln_w, const float* ln_b,
               const float* w_qkv, const float* w_out, const float* b_out, int64_t B, int64_t Hh,
               int64_t W, int64_t C, int64_t heads, int axis, float eps, void* stream) {
  const Weights w{ln_w, ln_b, w_qkv, w_out, b_out};
  int64_t bytes;
  const int st = validate_pass(x, out, w, B, Hh, W, C, heads, axis, eps, &bytes);
  if (st != MI355_ATTN_OK || bytes == 0) return st;
  const hipError_t err = mi355::launch_axial_pass(pass_args(x, out, w, B, Hh, W, C, axis, eps,
                                                            stream));
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

int axial_pass_split(const float* x, const float* out, int64_t B, int64_t Hh, int64_t W,
                     int axis) {
  if (B < 0 || Hh < 0 || W < 0) return -1;
  int64_t bh, tokens;
  if (!mul_ok(B, Hh, &bh) || !mul_ok(bh, W, &tokens) || tokens == 0) return -1;
  if (check_axis(B, Hh, W, axis) != MI355_ATTN_OK) return -1;
  const int64_t nseq = B * (axis == MI355_AXIAL_ROW ? Hh : W);
  return mi355::axial_split(nseq, x, out);
}

int axial_block(const float* x, float* out, const float* row_ln_w, const float* row_ln_b,
                const float* row_w_qkv, const float* row_w_out, const float* row_b_out,
                const float* col_ln_w, const float* col_ln_b, const float* col_w_qkv,
                const float* col_w_out, const float* col_b_out, int64_t B, int64_t Hh,
                int64_t W, int64_t C, int64_t heads, float eps, void* stream) {
  const Weights rw{row_ln_w, row_ln_b, row_w_qkv, row_w_out, row_b_out};
  const Weights cw{col_ln_w, col_ln_b, col_w_qkv, col_w_out, col_b_out};
  int64_t bytes;
  int st = validate_pass(x, out, rw, B, Hh, W, C, heads, MI355_AXIAL_ROW, eps, &bytes);
  if (st != MI355_ATTN_OK || bytes == 0) return st;
  if ((st = validate_pass(out, out, cw, B, Hh, W, C, heads, MI355_AXIAL_COL, eps, &bytes)) !=
      MI355_ATTN_OK)
    return st;
  hipError_t err = mi355::launch_axial_pass(pass_args(x, out, rw, B, Hh, W, C, MI355_AXIAL_ROW,
                                                      eps, stream));
  if (err == hipSuccess)
    err = mi355::launch_axial_pass(pass_args(out, out, cw, B, Hh, W, C, MI355_AXIAL_COL, eps,
                                             stream));
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

}  // extern "C"
