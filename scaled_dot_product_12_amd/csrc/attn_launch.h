// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and
// the kernel launchers. Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mi355_attn.h"

namespace mi355 {

struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t BH;  // B * H
  int64_t M, N, D;
  int64_t Dv;  // value and output head dim (equals D unless v has a head dim of its own)
  float scale;
  bool causal;
  hipStream_t stream;
};

// Tiled MFMA kernels with the online softmax (any M, N >= 1).
hipError_t launch_main_bf16(const LaunchArgs& a);
hipError_t launch_main_f16(const LaunchArgs& a);
hipError_t launch_main_f32(const LaunchArgs& a);
// One-tile register-resident kernel (M <= 64, N <= 64, D <= 32); et is the
// element type: 0 fp32, 1 bf16, 2 fp16 (the ABI's dtype codes).
hipError_t launch_small(const LaunchArgs& a, int et);

// Query rows per workgroup of the main kernels (grid sizing checks).
int main_bf16_tile_rows();
int main_f32_tile_rows();

// fp8 (e4m3) forward: q [BH, M, D], k [BH, N, D], vt [BH, D, N] (V
// transposed), o bf16 [BH, M, D], lse fp32; D in {64, 128}, N % 16 == 0.
struct Fp8LaunchArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  float* lse;
  int64_t BH;
  int64_t M, N, D;
  float scale;
  bool causal;
  hipStream_t stream;
};
hipError_t launch_fp8(const Fp8LaunchArgs& a);
int fp8_tile_rows();

struct BwdLaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B*H*M] workspace, written by the dQ kernel
  int64_t BH;
  int64_t M, N, D;
  float scale;
  bool causal;
  hipStream_t stream;
};

// Backward (bf16 or fp16, D in {32, 64, 128}): dQ kernel (also writes
// delta), then the dK/dV kernel, both on a.stream.
hipError_t launch_bwd_bf16(const BwdLaunchArgs& a);
hipError_t launch_bwd_f16(const BwdLaunchArgs& a);
// Rows per workgroup of the two backward kernels (grid sizing checks).
int bwd_dq_tile_rows();
int bwd_dkdv_tile_rows();
// Single-pass backward (bf16 or fp16, D = 128, no mask): the bytes of device
// work area it needs (0 where it does not apply),
// and its launch (delta kernel, then the fused kernel, on a.stream) with a
// 256-byte aligned work area of at least that size. The int at byte offset
// bwd_fused_error_offset() of the work area is 0 after a run in which every
// wait ended normally.
int64_t bwd_fused_work_bytes(int64_t BH, int64_t M, int64_t N, int64_t D, bool causal);
hipError_t launch_bwd_fused(const BwdLaunchArgs& a, void* work, bool f16);
int bwd_fused_error_offset();

// Capacity (query rows, B*H*M) of the static delta array of the no-alloc
// backward, and the device address of that array on the current device
// (looked up once per device; no allocation).
constexpr int64_t kNoallocMaxRows = MI355_ATTN_NOALLOC_MAX_ROWS;
hipError_t noalloc_delta_scratch(float** out);

struct AxialLaunchArgs {
  const float* x;
  float* out;  // may equal x
  const float* ln_w;
  const float* ln_b;
  const float* w_qkv;
  const float* w_out;
  const float* b_out;
  int64_t nseq;  // sequences (one workgroup each)
  int64_t L;     // tokens per sequence, 1..64
  // sequence s starts at (s / inner) * outer_stride + (s % inner) * inner_stride
  // floats, and its tokens are tstride floats apart
  int64_t inner, outer_stride, inner_stride, tstride;
  float eps;
  hipStream_t stream;
};

// One residual axial-attention pass (C = 64 features, 4 heads of 16).
hipError_t launch_axial_pass(const AxialLaunchArgs& a);
// Workgroups per sequence that launch_axial_pass uses: 2 for at most 128
// sequences read from one buffer and written to another, else 1 (in place).
int axial_split(int64_t nseq, const float* x, const float* out);

}  // namespace mi355
