// attn_api.cpp -- the C ABI declared in include/mi355_attn.h: argument
// validation (pure host logic, no HIP call), kernel-path choice, and the
// launch on the caller's stream.

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/mi355_attn.h"
#include "attn_launch.h"

namespace {

constexpr int64_t kIntMax = 2147483647;

bool supported_d(int64_t D) { return D == 16 || D == 32 || D == 64 || D == 128; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out);
}

// Byte ranges [p, p+n) and [r, r+m) intersect (empty ranges never do).
bool overlap(const void* p, int64_t n, const void* r, int64_t m) {
  if (n <= 0 || m <= 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)r;
  return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

bool small_fits(int64_t M, int64_t N, int64_t D) { return M <= 64 && N <= 64 && D <= 32; }

bool known_dtype(int dtype) {
  return dtype == MI355_ATTN_FP32 || dtype == MI355_ATTN_BF16 || dtype == MI355_ATTN_FP16;
}

int validate(const void* q, const void* k, const void* v, const void* o,
             const float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
             int64_t D, float scale, int is_causal, int dtype) {
  if (B < 0 || H < 0 || M < 0 || D < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return MI355_ATTN_ERR_INVALID_ARG;
  if (is_causal != 0 && is_causal != 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MI355_ATTN_ERR_INVALID_ARG;
  int64_t BH, rows;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, M, &rows)) return MI355_ATTN_ERR_UNSUPPORTED;
  if (rows == 0) return MI355_ATTN_OK;  // nothing to compute
  if (N < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse) return MI355_ATTN_ERR_INVALID_ARG;
  if (!supported_d(D)) return MI355_ATTN_ERR_UNSUPPORTED;

  // Index types: per-head element offsets are 32-bit inside the kernels,
  // head bases and the grid size are checked here.
  const int64_t es = dtype == MI355_ATTN_FP32 ? 4 : 2;
  int64_t md, nd, q_elems, kv_elems, q_bytes, kv_bytes, lse_bytes;
  if (!mul_ok(M, D, &md) || !mul_ok(N, D, &nd) || md > kIntMax || nd > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (!mul_ok(rows, D, &q_elems) || !mul_ok(BH, nd, &kv_elems) ||
      !mul_ok(q_elems, es, &q_bytes) || !mul_ok(kv_elems, es, &kv_bytes) ||
      !mul_ok(rows, 4, &lse_bytes))
    return MI355_ATTN_ERR_UNSUPPORTED;
  const int64_t tile = dtype == MI355_ATTN_FP32 ? mi355::main_f32_tile_rows()
                                                : mi355::main_bf16_tile_rows();
  int64_t grid;
  if (!mul_ok((M + tile - 1) / tile, BH, &grid) || grid > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;

  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
    return MI355_ATTN_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3u) return MI355_ATTN_ERR_MISALIGNED;

  // Outputs must not overlap the inputs or each other (inputs may alias).
  if (overlap(o, q_bytes, q, q_bytes) || overlap(o, q_bytes, k, kv_bytes) ||
      overlap(o, q_bytes, v, kv_bytes) || overlap(lse, lse_bytes, q, q_bytes) ||
      overlap(lse, lse_bytes, k, kv_bytes) || overlap(lse, lse_bytes, v, kv_bytes) ||
      overlap(lse, lse_bytes, o, q_bytes))
    return MI355_ATTN_ERR_INVALID_ARG;
  return MI355_ATTN_OK;
}

bool bwd_supported_d(int64_t D) { return D == 32 || D == 64 || D == 128; }

// own_delta: the library supplies delta (the no-alloc entry), so the delta
// pointer is not the caller's and is not checked.
int validate_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, const void* dq, const void* dk,
                 const void* dv, const float* delta, int64_t B, int64_t H, int64_t M,
                 int64_t N, int64_t D, float scale, int is_causal, int dtype,
                 bool own_delta = false) {
  if (B < 0 || H < 0 || M < 0 || N < 0 || D < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return MI355_ATTN_ERR_INVALID_ARG;
  if (is_causal != 0 && is_causal != 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MI355_ATTN_ERR_INVALID_ARG;
  int64_t BH, q_rows, k_rows;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, M, &q_rows) || !mul_ok(BH, N, &k_rows))
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (q_rows == 0 && k_rows == 0) return MI355_ATTN_OK;  // nothing to compute
  if (M > 0 && N < 1) return MI355_ATTN_ERR_INVALID_ARG;
  // Key-side buffers are always used here; with no query rows the query-side
  // ones are never touched (dK = dV = 0) and may be null.
  if (!k || !v || !dk || !dv) return MI355_ATTN_ERR_INVALID_ARG;
  if (q_rows > 0 && (!q || !o || !lse || !dout || !dq || (!delta && !own_delta)))
    return MI355_ATTN_ERR_INVALID_ARG;
  if (dtype == MI355_ATTN_FP32 || !bwd_supported_d(D)) return MI355_ATTN_ERR_UNSUPPORTED;

  const int64_t es = 2;
  int64_t md, nd, q_elems, kv_elems, q_bytes, kv_bytes, row_bytes;
  if (!mul_ok(M, D, &md) || !mul_ok(N, D, &nd) || md > kIntMax || nd > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (!mul_ok(q_rows, D, &q_elems) || !mul_ok(k_rows, D, &kv_elems) ||
      !mul_ok(q_elems, es, &q_bytes) || !mul_ok(kv_elems, es, &kv_bytes) ||
      !mul_ok(q_rows, 4, &row_bytes))
    return MI355_ATTN_ERR_UNSUPPORTED;
  const int64_t tq = mi355::bwd_dq_tile_rows(), tk = mi355::bwd_dkdv_tile_rows();
  int64_t grid_q, grid_k;
  if (!mul_ok((M + tq - 1) / tq, BH, &grid_q) || grid_q > kIntMax ||
      !mul_ok((N + tk - 1) / tk, BH, &grid_k) || grid_k > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;

  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return MI355_ATTN_ERR_MISALIGNED;
  if (((uintptr_t)lse | (own_delta ? 0 : (uintptr_t)delta)) & 3u)
    return MI355_ATTN_ERR_MISALIGNED;

  // Outputs (dq, dk, dv, delta) must not overlap the inputs or each other
  // (inputs may alias one another).
  const void* in_p[6] = {q, k, v, o, lse, dout};
  const int64_t in_n[6] = {q_bytes, kv_bytes, kv_bytes, q_bytes, row_bytes, q_bytes};
  const void* out_p[4] = {dq, dk, dv, own_delta ? nullptr : delta};
  const int64_t out_n[4] = {q_bytes, kv_bytes, kv_bytes, own_delta ? 0 : row_bytes};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlap(out_p[a], out_n[a], in_p[b], in_n[b])) return MI355_ATTN_ERR_INVALID_ARG;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(out_p[a], out_n[a], out_p[b], out_n[b])) return MI355_ATTN_ERR_INVALID_ARG;
  }
  return MI355_ATTN_OK;
}

// attn_fwd_fp8: e4m3 q, k and transposed v; bf16 o; fp32 lse.
int validate_fp8(const void* q, const void* k, const void* vt, const void* o, const float* lse,
                 int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                 int is_causal) {
  if (B < 0 || H < 0 || M < 0 || D < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (is_causal != 0 && is_causal != 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MI355_ATTN_ERR_INVALID_ARG;
  int64_t BH, rows;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, M, &rows)) return MI355_ATTN_ERR_UNSUPPORTED;
  if (rows == 0) return MI355_ATTN_OK;
  if (N < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!q || !k || !vt || !o || !lse) return MI355_ATTN_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || N % 16 != 0) return MI355_ATTN_ERR_UNSUPPORTED;
  int64_t md, nd, q_bytes, kv_bytes, o_bytes, lse_bytes;
  if (!mul_ok(M, D, &md) || !mul_ok(N, D, &nd) || md > kIntMax || nd > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (!mul_ok(rows, D, &q_bytes) || !mul_ok(BH, nd, &kv_bytes) || !mul_ok(q_bytes, 2, &o_bytes) ||
      !mul_ok(rows, 4, &lse_bytes))
    return MI355_ATTN_ERR_UNSUPPORTED;
  const int64_t tile = mi355::fp8_tile_rows();
  int64_t grid;
  if (!mul_ok((M + tile - 1) / tile, BH, &grid) || grid > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)vt | (uintptr_t)o) & 15u)
    return MI355_ATTN_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3u) return MI355_ATTN_ERR_MISALIGNED;
  if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, k, kv_bytes) ||
      overlap(o, o_bytes, vt, kv_bytes) || overlap(lse, lse_bytes, q, q_bytes) ||
      overlap(lse, lse_bytes, k, kv_bytes) || overlap(lse, lse_bytes, vt, kv_bytes) ||
      overlap(lse, lse_bytes, o, o_bytes))
    return MI355_ATTN_ERR_INVALID_ARG;
  return MI355_ATTN_OK;
}

int select_path(int64_t M, int64_t N, int64_t D) {
  return small_fits(M, N, D) ? MI355_ATTN_PATH_SMALL : MI355_ATTN_PATH_MAIN;
}

}  // namespace

extern "C" {

int attn_fwd_validate(const void* q, const void* k, const void* v, void* o,
                      const float* lse, int64_t B, int64_t H, int64_t M,
                      int64_t N, int64_t D, float scale, int is_causal,
                      int dtype) {
  return validate(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, dtype);
}

int attn_fwd_select_path(int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                         int is_causal, int dtype) {
  if (B < 0 || H < 0 || M < 0 || N < 1 || !supported_d(D)) return -1;
  if (!known_dtype(dtype)) return -1;
  if (is_causal != 0 && is_causal != 1) return -1;
  int64_t BH, rows;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, M, &rows)) return -1;
  return select_path(M, N, D);
}

int attn_fwd_path(const void* q, const void* k, const void* v, void* o,
                  float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                  int64_t D, float scale, int is_causal, int dtype, int path,
                  void* stream) {
  if (path != MI355_ATTN_PATH_AUTO && path != MI355_ATTN_PATH_MAIN &&
      path != MI355_ATTN_PATH_SMALL)
    return MI355_ATTN_ERR_INVALID_ARG;
  const int st = validate(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, dtype);
  if (st != MI355_ATTN_OK) return st;
  if (B * H * M == 0) return MI355_ATTN_OK;
  if (path == MI355_ATTN_PATH_AUTO) path = select_path(M, N, D);
  if (path == MI355_ATTN_PATH_SMALL && !small_fits(M, N, D)) return MI355_ATTN_ERR_UNSUPPORTED;

  mi355::LaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.Dv = D;
  a.scale = scale;
  a.causal = is_causal != 0;
  a.stream = (hipStream_t)stream;
  hipError_t err;
  if (path == MI355_ATTN_PATH_SMALL)
    err = mi355::launch_small(a, dtype);
  else if (dtype == MI355_ATTN_BF16)
    err = mi355::launch_main_bf16(a);
  else if (dtype == MI355_ATTN_FP16)
    err = mi355::launch_main_f16(a);
  else
    err = mi355::launch_main_f32(a);
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
             int is_causal, int dtype, void* stream) {
  return attn_fwd_path(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, dtype,
                       MI355_ATTN_PATH_AUTO, stream);
}

// Checks of attn_fwd_dv when the value head dim differs from D: v is
// [B,H,N,Dv] and o [B,H,M,Dv]; D and Dv each in {16, 32, 64, 128}, any dtype.
static bool dv_pair_supported(int64_t D, int64_t Dv, int dtype) {
  (void)dtype;
  return supported_d(D) && supported_d(Dv);
}

static int validate_dv(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                       int64_t Dv, float scale, int is_causal, int dtype) {
  if (B < 0 || H < 0 || M < 0 || D < 1 || Dv < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return MI355_ATTN_ERR_INVALID_ARG;
  if (is_causal != 0 && is_causal != 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MI355_ATTN_ERR_INVALID_ARG;
  int64_t BH, rows;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, M, &rows)) return MI355_ATTN_ERR_UNSUPPORTED;
  if (rows == 0) return MI355_ATTN_OK;
  if (N < 1) return MI355_ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse) return MI355_ATTN_ERR_INVALID_ARG;
  if (!dv_pair_supported(D, Dv, dtype)) return MI355_ATTN_ERR_UNSUPPORTED;
  int64_t md, nd, nv, mv, q_el, k_el, v_el, o_el;
  if (!mul_ok(M, D, &md) || !mul_ok(N, D, &nd) || !mul_ok(N, Dv, &nv) || !mul_ok(M, Dv, &mv) ||
      md > kIntMax || nd > kIntMax || nv > kIntMax || mv > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (!mul_ok(rows, D, &q_el) || !mul_ok(BH, nd, &k_el) || !mul_ok(BH, nv, &v_el) ||
      !mul_ok(rows, Dv, &o_el) || q_el > INT64_MAX / 4 || k_el > INT64_MAX / 4 ||
      v_el > INT64_MAX / 4 || o_el > INT64_MAX / 4)
    return MI355_ATTN_ERR_UNSUPPORTED;
  const int64_t es = dtype == MI355_ATTN_FP32 ? 4 : 2;
  const int64_t tile = mi355::main_f32_tile_rows();
  int64_t grid;
  if (!mul_ok((M + tile - 1) / tile, BH, &grid) || grid > kIntMax)
    return MI355_ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
    return MI355_ATTN_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3u) return MI355_ATTN_ERR_MISALIGNED;
  const int64_t qb = es * q_el, kb = es * k_el, vb = es * v_el, ob = es * o_el, lb = 4 * rows;
  if (overlap(o, ob, q, qb) || overlap(o, ob, k, kb) || overlap(o, ob, v, vb) ||
      overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, vb) ||
      overlap(lse, lb, o, ob))
    return MI355_ATTN_ERR_INVALID_ARG;
  return MI355_ATTN_OK;
}

int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t H, int64_t M, int64_t N, int64_t D, int64_t Dv, float scale,
                int is_causal, int dtype, void* stream) {
  if (Dv == D)
    return attn_fwd_path(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, dtype,
                         MI355_ATTN_PATH_AUTO, stream);
  const int st = validate_dv(q, k, v, o, lse, B, H, M, N, D, Dv, scale, is_causal, dtype);
  if (st != MI355_ATTN_OK) return st;
  if (B * H * M == 0) return MI355_ATTN_OK;
  mi355::LaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.Dv = Dv;
  a.scale = scale;
  a.causal = is_causal != 0;
  a.stream = (hipStream_t)stream;
  const hipError_t err = dtype == MI355_ATTN_BF16   ? mi355::launch_main_bf16(a)
                         : dtype == MI355_ATTN_FP16 ? mi355::launch_main_f16(a)
                                                    : mi355::launch_main_f32(a);
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

int attn_fwd_dv_validate(const void* q, const void* k, const void* v, void* o, const float* lse,
                         int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, int64_t Dv,
                         float scale, int is_causal, int dtype) {
  if (Dv == D) return validate(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, dtype);
  return validate_dv(q, k, v, o, lse, B, H, M, N, D, Dv, scale, is_causal, dtype);
}

int attn_bwd_validate(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, const void* dq, const void* dk,
                      const void* dv, const float* delta, int64_t B, int64_t H, int64_t M,
                      int64_t N, int64_t D, float scale, int is_causal, int dtype) {
  return validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, scale,
                      is_causal, dtype);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t B,
             int64_t H, int64_t M, int64_t N, int64_t D, float scale, int is_causal,
             int dtype, void* stream) {
  const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D,
                              scale, is_causal, dtype);
  if (st != MI355_ATTN_OK) return st;
  if (B * H * (M + N) == 0) return MI355_ATTN_OK;
  mi355::BwdLaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.BH = B * H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.causal = is_causal != 0;
  a.stream = (hipStream_t)stream;
  const hipError_t err =
      dtype == MI355_ATTN_FP16 ? mi355::launch_bwd_f16(a) : mi355::launch_bwd_bf16(a);
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

int64_t attn_bwd_work_bytes(int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                            int is_causal, int dtype) {
  if (B < 0 || H < 0 || M < 0 || N < 0) return 0;
  if (dtype != MI355_ATTN_BF16 && dtype != MI355_ATTN_FP16) return 0;
  int64_t BH, rows, elems;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, M, &rows) || !mul_ok(rows, D, &elems)) return 0;
  return mi355::bwd_fused_work_bytes(BH, M, N, D, is_causal != 0);
}

int attn_bwd_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t B,
                int64_t H, int64_t M, int64_t N, int64_t D, float scale, int is_causal,
                int dtype, void* work, int64_t work_bytes, void* stream) {
  const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D,
                              scale, is_causal, dtype);
  if (st != MI355_ATTN_OK) return st;
  if (work_bytes < 0) return MI355_ATTN_ERR_INVALID_ARG;
  const int64_t need = attn_bwd_work_bytes(B, H, M, N, D, is_causal, dtype);
  if (need == 0 || work == nullptr || work_bytes < need)
    return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, scale, is_causal,
                    dtype, stream);
  if ((uintptr_t)work & 255u) return MI355_ATTN_ERR_MISALIGNED;
  // the work area is written: it must not overlap any argument buffer
  const int64_t q_bytes = B * H * M * D * 2, kv_bytes = B * H * N * D * 2, rows = B * H * M * 4;
  const void* p[10] = {q, k, v, o, lse, dout, dq, dk, dv, delta};
  const int64_t n[10] = {q_bytes, kv_bytes, kv_bytes, q_bytes, rows, q_bytes,
                         q_bytes, kv_bytes, kv_bytes, rows};
  for (int i = 0; i < 10; ++i)
    if (overlap(work, need, p[i], n[i])) return MI355_ATTN_ERR_INVALID_ARG;
  mi355::BwdLaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.BH = B * H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.causal = is_causal != 0;
  a.stream = (hipStream_t)stream;
  const hipError_t err = mi355::launch_bwd_fused(a, work, dtype == MI355_ATTN_FP16);
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

int attn_bwd_work_error_offset(void) { return mi355::bwd_fused_error_offset(); }

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, float scale,
                     int is_causal, int dtype, void* stream) {
  const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, H, M, N, D,
                              scale, is_causal, dtype, /*own_delta=*/true);
  if (st != MI355_ATTN_OK) return st;
  if (B * H * (M + N) == 0) return MI355_ATTN_OK;
  if (B * H * M > mi355::kNoallocMaxRows) return MI355_ATTN_ERR_SCRATCH;
  float* delta = nullptr;
  if (mi355::noalloc_delta_scratch(&delta) != hipSuccess) return MI355_ATTN_ERR_HIP;
  mi355::BwdLaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.BH = B * H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.causal = is_causal != 0;
  a.stream = (hipStream_t)stream;
  const hipError_t err =
      dtype == MI355_ATTN_FP16 ? mi355::launch_bwd_f16(a) : mi355::launch_bwd_bf16(a);
  return err == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

int attn_fwd_fp8_validate(const void* q, const void* k, const void* vt, const void* o,
                          const float* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                          int64_t D, float scale, int is_causal) {
  return validate_fp8(q, k, vt, o, lse, B, H, M, N, D, scale, is_causal);
}

int attn_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int64_t B,
                 int64_t H, int64_t M, int64_t N, int64_t D, float scale, int is_causal,
                 void* stream) {
  const int st = validate_fp8(q, k, vt, o, lse, B, H, M, N, D, scale, is_causal);
  if (st != MI355_ATTN_OK) return st;
  if (B * H * M == 0) return MI355_ATTN_OK;
  mi355::Fp8LaunchArgs a;
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.M = M;
  a.N = N;
  a.D = D;
  a.scale = scale;
  a.causal = is_causal != 0;
  a.stream = (hipStream_t)stream;
  return mi355::launch_fp8(a) == hipSuccess ? MI355_ATTN_OK : MI355_ATTN_ERR_HIP;
}

const char* attn_status_string(int status) {
  switch (status) {
    case MI355_ATTN_OK: return "ok";
    case MI355_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case MI355_ATTN_ERR_UNSUPPORTED: return "unsupported problem";
    case MI355_ATTN_ERR_MISALIGNED: return "misaligned pointer";
    case MI355_ATTN_ERR_HIP: return "HIP launch error";
    case MI355_ATTN_ERR_SCRATCH: return "problem exceeds the no-alloc scratch buffer";
    default: return "unknown status";
  }
}

}  // extern "C"
