// axial_block.hip -- one residual pass of the fused axial-attention block on
// gfx950 (the PopcornBench axial-attention trajectory: LayerNorm, bias-free
// QKV projection, per-head softmax attention, output projection with bias,
// residual add; the row pass attends along image rows, the column pass along
// image columns of the row pass's output).
//
// One workgroup (4 waves) per sequence of L <= 64 tokens with C = 64 features
// and 4 heads of 16, or, when there are fewer sequences than CUs and the
// pass writes a buffer other than the one it reads, two workgroups per
// sequence that each take half of its query tokens (both project K and V for
// every token; Q, the attention rows, the output projection and the store are
// split). Everything between the token load and
// the final store stays in LDS and registers:
//  * the tokens are gathered straight from the image tensor with the pass's
//    strides (the column pass needs no transposed copy);
//  * LayerNorm runs as the tokens arrive: 16 lanes per token, 4 features
//    each, mean and variance by 16-lane DPP sums;
//  * the three products (QKV = LN(x) W_qkv^T, S = Q K^T per head, P V, and
//    the output projection) run on v_mfma_f32_16x16x4f32 in fp32. Wave w
//    computes QKV column blocks w, w+4, w+8 (head w's Q, K and V), attention
//    head w and output column block w, so every SIMD gets the same share and
//    the attention reads only what its own wave wrote;
//  * the projection weights are loaded into registers right after the
//    tokens, so their latency overlaps the LayerNorm.
//
// v_mfma_f32_16x16x4f32 operand layout (lane l, l16 = l % 16, g = l / 16):
// A[i][k] at lane i + 16k, B[k][j] at lane j + 16k, D[i][j] in register i % 4
// of lane j + 16 (i / 4). Contractions over 64 features take feature 16g + st
// at MFMA step st, so each lane's operands are 16 consecutive floats.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

namespace {

constexpr int kC = 64;       // features per token
constexpr int kHeads = 4;
constexpr int kHd = 16;      // features per head
constexpr int kWaves = 4;
constexpr int kXStr = kC + 4;        // floats per token row in LDS: 16 rows of a
                                     // 16-byte column read hit distinct banks
constexpr int kQStr = 3 * kC + 4;    // floats per token row of the QKV buffer

__device__ __forceinline__ f32x4_t mfma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum over the 16 lanes of a row (DPP: swap neighbours, swap pairs, mirror
// within 8, mirror within 16); every lane of the row gets the sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Combine of lanes l and l ^ 16 (the same exchange as half_pair_*, one row
// apart): after a swap of x with itself each lane holds {x[l], x[l ^ 16]}.
__device__ __forceinline__ float row_pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int LP, int QS>
__global__ __launch_bounds__(kWaves * 64) void axial_pass_kernel(
    const float* __restrict__ x, float* out, const float* __restrict__ ln_w,
    const float* __restrict__ ln_b, const float* __restrict__ w_qkv,
    const float* __restrict__ w_out, const float* __restrict__ b_out, int L, int same_xcd,
    int inner,
    int64_t outer_stride, int64_t inner_stride, int64_t tstride, float eps, float c) {
  constexpr int RB = LP / 16;  // 16-token blocks
  constexpr int QRB = RB / QS;  // query blocks per workgroup
  __shared__ __attribute__((aligned(16))) float xs[LP * kXStr];  // tokens (residual)
  __shared__ __attribute__((aligned(16))) float xn[LP * kXStr];  // LN(x)
  // Head outputs: a buffer of their own, since with no barrier after the
  // projection other waves may still be reading xn.
  __shared__ __attribute__((aligned(16))) float ao[LP * kXStr];
  __shared__ __attribute__((aligned(16))) float qkv[LP * kQStr];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  // Workgroups go to the 8 XCDs round-robin. With two workgroups per
  // sequence and a sequence count divisible by 8 (same_xcd), the two halves
  // of a sequence are ids 16a + 8h + x, both on XCD x, so the second reads
  // the tokens through the L2 the first filled; otherwise ids 2s + h.
  const int wg = workgroup_id();
  int s, h;
  if (QS == 2 && same_xcd) {
    s = ((wg >> 4) << 3) | (wg & 7);
    h = (wg >> 3) & 1;
  } else {
    s = wg / QS;
    h = wg % QS;
  }
  const int q0 = h * QRB;  // first query block
  // x and out may be the same buffer only in the unsplit launch (QS = 1): a
  // workgroup reads all of its tokens before it writes any, and sequences are
  // disjoint. The two halves of a split sequence both read every token of it
  // while each writes half of them, so the host never splits a pass whose
  // output is its input.
  const int64_t base = (int64_t)(s / inner) * outer_stride + (int64_t)(s % inner) * inner_stride;

  // Tokens first (16 threads per token, one 16-byte chunk of 4 features
  // each), then the weights: loads complete in order, so the LayerNorm can
  // start while the weights are still arriving. Padding tokens load token
  // L - 1 (L >= 1) and are replaced by 0: no branch, whose join would wait
  // for the loads before the weights are even issued.
  const int ch = (tid & 15) * 4;
  f32x4_t xv[LP / 16];
#pragma unroll
  for (int i = 0; i < LP / 16; ++i) {
    const int t = (tid >> 4) + 16 * i;
    xv[i] = *(const f32x4_t*)(x + base + (t < L ? t : L - 1) * tstride + ch);
  }
  const f32x4_t gam = *(const f32x4_t*)(ln_w + ch);
  const f32x4_t bet = *(const f32x4_t*)(ln_b + ch);
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weights

  // Weights: QKV output features 16 (wave + 4 cb) + l16, output-projection
  // feature 16 wave + l16; input features 16g .. 16g + 15.
  f32x4_t wq[3][4], wo[4];
#pragma unroll
  for (int cb = 0; cb < 3; ++cb) {
    const float* wp = w_qkv + (16 * (wave + 4 * cb) + l16) * kC + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) wq[cb][e] = *(const f32x4_t*)(wp + 4 * e);
  }
  {
    const float* wp = w_out + (16 * wave + l16) * kC + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) wo[e] = *(const f32x4_t*)(wp + 4 * e);
  }
  const float bias = b_out[16 * wave + l16];

  // LayerNorm: the mean and the biased variance of a token are 16-lane sums.
  // Padding tokens normalise to the LayerNorm bias and are never stored.
#pragma unroll
  for (int i = 0; i < LP / 16; ++i) {
    const int t = (tid >> 4) + 16 * i;
    const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t val = t < L ? xv[i] : z;
    *(f32x4_t*)(xs + t * kXStr + ch) = val;
    const float mean = row16_sum((val[0] + val[1]) + (val[2] + val[3])) * (1.0f / kC);
    const f32x4_t dv = val - mean;
    const float var =
        row16_sum((dv[0] * dv[0] + dv[1] * dv[1]) + (dv[2] * dv[2] + dv[3] * dv[3])) *
        (1.0f / kC);
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);
    *(f32x4_t*)(xn + t * kXStr + ch) = dv * rstd * gam + bet;
  }
  __syncthreads();

  // QKV = LN(x) W_qkv^T, feature blocks wave + 4 cb. This workgroup's query
  // blocks (i < QRB) take Q, K and V, the other token blocks K and V only;
  // the loop has a fixed shape (only the block index depends on q0), so the
  // product chains of a block interleave.
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const bool own = i < QRB;
    const int rb = own ? q0 + i : (q0 == 0 ? i : i - QRB);
    f32x4_t a[4];
    const float* ap = xn + (16 * rb + l16) * kXStr + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = *(const f32x4_t*)(ap + 4 * e);
    f32x4_t acc[3];
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) acc[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < 16; ++st)
#pragma unroll
      for (int cb = 0; cb < 3; ++cb)
        if (own || cb > 0) acc[cb] = mfma16(a[st >> 2][st & 3], wq[cb][st >> 2][st & 3], acc[cb]);
#pragma unroll
    for (int cb = 0; cb < 3; ++cb) {
      if (!own && cb == 0) continue;
      float* dp = qkv + (16 * rb + 4 * g) * kQStr + 16 * (wave + 4 * cb) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) dp[r * kQStr] = acc[cb][r];
    }
  }
  // Attention reads only this wave's own QKV columns: LDS operations of a
  // wave complete in order, so a wave-scope fence (no workgroup barrier) is
  // enough to keep the compiler from moving the reads above the writes.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // Attention, head = wave. S^T = K Q^T per (key block, query block): rows
  // are keys 16 kb + 4g + r, columns queries; the step-st contraction takes
  // head feature 4g + st. Then O^T = V^T P^T: step r contracts keys
  // 16 kb + 4g + r, whose probabilities are this lane's own register r.
  {
    const int qo = wave * kHd, ko = kC + wave * kHd, vo = 2 * kC + wave * kHd;
#pragma unroll
    for (int qb = q0; qb < q0 + QRB; ++qb) {
      const f32x4_t qf = *(const f32x4_t*)(qkv + (16 * qb + l16) * kQStr + qo + 4 * g);
      f32x4_t sc[RB];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < RB; ++kb) {
        const f32x4_t kf = *(const f32x4_t*)(qkv + (16 * kb + l16) * kQStr + ko + 4 * g);
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma16(kf[st], qf[st], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (16 * kb + 4 * g + r >= L) acc[r] = -INFINITY;
          mx = fmaxf(mx, acc[r]);
        }
        sc[kb] = acc;
      }
      mx = half_pair_max(row_pair_max(mx));
      const float mc = mx * c;  // key 0 is always present: mx is finite
      float sum = 0.0f;
      f32x4_t o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < RB; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c, -mc));
          sum += p;
          o = mfma16(qkv[(16 * kb + 4 * g + r) * kQStr + vo + l16], p, o);
        }
      }
      sum = half_pair_sum(row_pair_sum(sum));
      const float inv = 1.0f / sum;
      // o[r] is head feature 4g + r of query 16 qb + l16.
      const f32x4_t ov = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      *(f32x4_t*)(ao + (16 * qb + l16) * kXStr + qo + 4 * g) = ov;
    }
  }
  __syncthreads();

  // Output projection, bias and residual: token block rb, features 16 wave + l16.
#pragma unroll
  for (int rb = q0; rb < q0 + QRB; ++rb) {
    f32x4_t a[4];
    const float* ap = ao + (16 * rb + l16) * kXStr + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = *(const f32x4_t*)(ap + 4 * e);
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < 16; ++st) acc = mfma16(a[st >> 2][st & 3], wo[st >> 2][st & 3], acc);
    const int f = 16 * wave + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * rb + 4 * g + r;
      if (t < L) out[base + t * tstride + f] = acc[r] + bias + xs[t * kXStr + f];
    }
  }
}

}  // namespace

template <int LP, int QS>
void launch_lp(const AxialLaunchArgs& a, float c) {
  hipLaunchKernelGGL((axial_pass_kernel<LP, QS>), dim3((unsigned)(a.nseq * QS)), dim3(kWaves * 64),
                     0, a.stream, a.x, a.out, a.ln_w, a.ln_b, a.w_qkv, a.w_out, a.b_out, (int)a.L,
                     (int)(a.nseq % 8 == 0), (int)a.inner, a.outer_stride, a.inner_stride, a.tstride, a.eps, c);
}

// Query split: two workgroups per sequence while that still leaves at most
// one per CU (256 CUs); the K and V projections they both do cost less than
// the idle CUs would. Never in place: each half reads all tokens of the
// sequence, which the other half's stores would otherwise overwrite.
constexpr int64_t kSplitBelow = 256 / 2;

int axial_split(int64_t nseq, const float* x, const float* out) {
  return (nseq <= kSplitBelow && x != out) ? 2 : 1;
}

hipError_t launch_axial_pass(const AxialLaunchArgs& a) {
  // softmax in base 2: scores scaled by log2(e) / sqrt(head dim)
  const float c = (float)(1.4426950408889634 / 4.0);
  const bool split = axial_split(a.nseq, a.x, a.out) == 2;
  if (a.L <= 32) {
    if (split) launch_lp<32, 2>(a, c);
    else launch_lp<32, 1>(a, c);
  } else {
    if (split) launch_lp<64, 2>(a, c);
    else launch_lp<64, 1>(a, c);
  }
  return hipGetLastError();
}

}  // namespace mi355
