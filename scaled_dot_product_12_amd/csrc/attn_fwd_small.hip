// attn_fwd_small.hip -- attention forward for short sequences with small
// heads (M <= 64, N <= 64, D <= 32), e.g. the axial-attention passes of the
// PopcornBench trajectory (32 tokens per row or column, head dim 16).
//
// Such a problem is one tile: the whole of Q, K and V for one (batch, head)
// fits in LDS, so there is no online rescaling -- the softmax is taken once
// over the full row, which is the Python reference's loop ("Extend Thunder
// with CUDA-Python") with a single key tile. The work per head is tiny, so
// the bound is HBM latency and bandwidth, not arithmetic: every thread issues
// its global loads at once, the arithmetic runs in fp32 on the vector units
// out of LDS, and the results leave with one store per thread.
//
// One workgroup of 256 threads per (batch, head). Phases, separated by
// barriers:
//   1. Q, K, V -> LDS as fp32 (bf16 inputs widened exactly).
//   2. S = Q K^T * scale*log2(e) for all (row, key) pairs.
//   3. per row: max, p = exp2(s - max), sum -- 4 threads per row with
//      in-wave butterfly reductions; L = ln2 * (max + log2 sum).
//   4. O = P V / sum for all (row, d) pairs, then stored.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

namespace {
constexpr int kSmallMaxM = 64;
constexpr int kSmallMaxN = 64;
constexpr int kSmallMaxD = 32;
constexpr int kSmallThreads = 256;
}  // namespace

template <bool BF16>
__global__ __launch_bounds__(kSmallThreads) void attn_fwd_small_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv,
    const void* __restrict__ vv, void* __restrict__ ov, float* __restrict__ lse,
    int M, int N, int D, int causal, float c) {
  constexpr int SP = kSmallMaxN + 1;  // S row stride (odd: no bank repeats)
  constexpr int XP = kSmallMaxD + 1;  // Q/K/V row stride
  __shared__ float Qs[kSmallMaxM * XP];
  __shared__ float Ks[kSmallMaxN * XP];
  __shared__ float Vs[kSmallMaxN * XP];
  __shared__ float Ss[kSmallMaxM * SP];
  __shared__ float Rinv[kSmallMaxM];

  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x;
  const size_t q_off = bh * (size_t)M * D;
  const size_t kv_off = bh * (size_t)N * D;

  // 1. Stage Q, K, V. Each element is a (row, d) pair; four per step.
  const int qn = M * D, kn = N * D;
  for (int e4 = tid * 4; e4 < qn + 2 * kn; e4 += kSmallThreads * 4) {
    // D is a multiple of 16 and the three tensors are consecutive ranges of
    // e4, so a group of four never straddles a row or a tensor boundary.
    const int which = e4 < qn ? 0 : (e4 < qn + kn ? 1 : 2);
    const int e = which == 0 ? e4 : (which == 1 ? e4 - qn : e4 - qn - kn);
    const size_t base = (which == 0 ? q_off : kv_off) + e;
    const void* src = which == 0 ? qv : (which == 1 ? kv : vv);
    float x[4];
    if (BF16) {
      const u32x2_t w = *(const u32x2_t*)((const uint16_t*)src + base);
      x[0] = __uint_as_float(w[0] << 16);
      x[1] = __uint_as_float(w[0] & 0xffff0000u);
      x[2] = __uint_as_float(w[1] << 16);
      x[3] = __uint_as_float(w[1] & 0xffff0000u);
    } else {
      const f32x4_t w = *(const f32x4_t*)((const float*)src + base);
      x[0] = w[0]; x[1] = w[1]; x[2] = w[2]; x[3] = w[3];
    }
    const int row = e / D, col = e - (e / D) * D;
    float* dst = (which == 0 ? Qs : (which == 1 ? Ks : Vs)) + row * XP + col;
    dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
  }
  __syncthreads();

  // 2. Scores in the log2 domain; masked entries -inf.
  for (int idx = tid; idx < M * N; idx += kSmallThreads) {
    const int i = idx / N, j = idx - (idx / N) * N;
    const float* qr = Qs + i * XP;
    const float* kr = Ks + j * XP;
    float dot = 0.0f;
    for (int d = 0; d < D; ++d) dot = fmaf(qr[d], kr[d], dot);
    Ss[i * SP + j] = (causal && j > i) ? -INFINITY : dot * c;
  }
  __syncthreads();

  // 3. Row statistics: 4 consecutive lanes per row (M <= 64 rows).
  {
    const int i = tid >> 2, part = tid & 3;
    float mx = -INFINITY;
    if (i < M)
      for (int j = part; j < N; j += 4) mx = fmaxf(mx, Ss[i * SP + j]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float m_sub = (mx == -INFINITY) ? 0.0f : mx;
    float sum = 0.0f;
    if (i < M)
      for (int j = part; j < N; j += 4) {
        const float p = __builtin_amdgcn_exp2f(Ss[i * SP + j] - m_sub);
        Ss[i * SP + j] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    if (i < M && part == 0) {
      Rinv[i] = 1.0f / sum;
      lse[bh * (size_t)M + i] = (mx + log2f(sum)) * kLn2;
    }
  }
  __syncthreads();

  // 4. O = P V / sum; each thread makes 4 consecutive d of one row.
  const int dq = D / 4;
  for (int idx = tid; idx < M * dq; idx += kSmallThreads) {
    const int i = idx / dq, d0 = (idx - (idx / dq) * dq) * 4;
    const float* pr = Ss + i * SP;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    const int jn = causal ? min(i + 1, N) : N;
    for (int j = 0; j < jn; ++j) {
      const float p = pr[j];
      const float* vr = Vs + j * XP + d0;
      a0 = fmaf(p, vr[0], a0);
      a1 = fmaf(p, vr[1], a1);
      a2 = fmaf(p, vr[2], a2);
      a3 = fmaf(p, vr[3], a3);
    }
    const float r = Rinv[i];
    const size_t at = q_off + (size_t)i * D + d0;
    if (BF16) {
      u32x2_t st;
      st[0] = pack_bf16x2(a0 * r, a1 * r);
      st[1] = pack_bf16x2(a2 * r, a3 * r);
      *(u32x2_t*)((uint16_t*)ov + at) = st;
    } else {
      const f32x4_t st = {a0 * r, a1 * r, a2 * r, a3 * r};
      *(f32x4_t*)((float*)ov + at) = st;
    }
  }
}

hipError_t launch_small(const LaunchArgs& a, bool bf16) {
  if (a.M > kSmallMaxM || a.N > kSmallMaxN || a.D > kSmallMaxD || a.D % 16)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.BH);
  const float c = a.scale * kLog2e;
  if (bf16)
    hipLaunchKernelGGL(attn_fwd_small_kernel<true>, grid, dim3(kSmallThreads), 0,
                       a.stream, a.q, a.k, a.v, a.o, a.lse, (int)a.M, (int)a.N,
                       (int)a.D, (int)a.causal, c);
  else
    hipLaunchKernelGGL(attn_fwd_small_kernel<false>, grid, dim3(kSmallThreads), 0,
                       a.stream, a.q, a.k, a.v, a.o, a.lse, (int)a.M, (int)a.N,
                       (int)a.D, (int)a.causal, c);
  return hipGetLastError();
}

}  // namespace mi355
