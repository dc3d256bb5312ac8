// attn_fwd_small.hip -- attention forward for short sequences with small
// heads (M <= 64, N <= 64, D in {16, 32}), e.g. the axial-attention passes of
// the PopcornBench trajectory (32 tokens per row or column, head dim 16).
//
// Such a problem is one tile: all of K and V for one (batch, head) fit in the
// registers of one wave, so there is no online rescaling -- the softmax is
// taken once over the full row, which is the Python reference's loop
// ("Extend Thunder with CUDA-Python") with a single key tile. The work per
// head is tiny, so the bound is latency (launch, one round trip to HBM), not
// arithmetic or bandwidth. The kernel therefore has a single phase with no
// barrier and no LDS: every lane issues all its global loads at once, in the
// exact operand layout of the fp32 MFMA, and both products run on the matrix
// cores (fp32 in, fp32 accumulate -- no precision is given up on fp32 inputs).
//
// One wave per block of 16 query rows; a workgroup holds up to four waves:
// one head of up to 64 rows, or two (four) heads of up to 32 (16) rows.
// With v_mfma_f32_16x16x4_f32, lane l = 16 g + n (n = l % 16, g = l / 16):
//   S^T block kb (keys 16 kb .. 16 kb + 15 by queries q0 .. q0 + 15)
//     A = K rows,   lane supplies K[16 kb + n][d],  d = g * D/4 + t
//     B = Q^T,      lane supplies Q[q0 + n][d]      (same d: the contraction
//                                                    order over d is free)
//     result: lane holds S for query q0 + n and keys 16 kb + 4 g + r, r < 4.
//   Row max / sum over the four lanes n, n+16, n+32, n+48 (permlane swaps).
//   O^T block db (d = 16 db .. 16 db + 15 by the 16 queries)
//     A = V^T,      lane supplies V[16 kb + 4 g + r][16 db + n]
//     B = P^T,      lane supplies its own P for key 16 kb + 4 g + r
//     result: lane holds O[q0 + n][16 db + 4 g + r], r < 4 -- one 16-byte
//     (fp32) or 8-byte (bf16, fp16) store per block.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

namespace {
constexpr int kSmallMaxM = 64;
constexpr int kSmallMaxN = 64;
constexpr int kSmallMaxD = 32;
constexpr int kSmallMaxKB = kSmallMaxN / 16;
constexpr int kSmallQRows = 16;  // query rows per wave
// Waves per workgroup. Four (one CU each for the axial passes' 512 heads of
// two waves) measured fastest: 2.6 us per axial pass in a graph, against 3.0
// with eight and 4.1 with sixteen (fewer workgroups leave CUs idle).
constexpr int kSmallWaves = 4;

__device__ __forceinline__ f32x4_t mfma_16x16x4_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Symmetric combines over the lane pairs l, l ^ 16 (permlane16_swap) and
// l, l ^ 32 (permlane32_swap): after a swap of x with itself each lane holds
// {x[l], x[partner]} in some order.
__device__ __forceinline__ float pair16_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Element types of q, k, v and o.
constexpr int kEtF32 = 0, kEtBf16 = 1, kEtF16 = 2;

// Two packed 16-bit elements widened to fp32 (exact for both types; bf16 bits
// are the top half of the fp32 bits).
template <int ET>
__device__ __forceinline__ void widen2(uint32_t w, float* x) {
  if (ET == kEtBf16) {
    x[0] = __uint_as_float(w << 16);
    x[1] = __uint_as_float(w & 0xffff0000u);
  } else {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
    x[0] = (float)h[0];
    x[1] = (float)h[1];
  }
}

// Loads of n consecutive elements (n = 4 or 8) starting at element e,
// widened to fp32.
template <int ET, int NE>
__device__ __forceinline__ void load_row_part(const void* base, size_t e, float* x) {
  if (ET != kEtF32) {
    const uint16_t* p = (const uint16_t*)base + e;
    if (NE == 4) {
      const u32x2_t w = *(const u32x2_t*)p;
#pragma unroll
      for (int i = 0; i < 2; ++i) widen2<ET>(w[i], x + 2 * i);
    } else {
      const u32x4_t w = *(const u32x4_t*)p;
#pragma unroll
      for (int i = 0; i < 4; ++i) widen2<ET>(w[i], x + 2 * i);
    }
  } else {
    const float* p = (const float*)base + e;
#pragma unroll
    for (int i = 0; i < NE; i += 4) {
      const f32x4_t w = *(const f32x4_t*)(p + i);
      x[i] = w[0]; x[i + 1] = w[1]; x[i + 2] = w[2]; x[i + 3] = w[3];
    }
  }
}

template <int ET>
__device__ __forceinline__ float load_one(const void* base, size_t e) {
  if (ET == kEtBf16) return __uint_as_float((uint32_t)((const uint16_t*)base)[e] << 16);
  if (ET == kEtF16) return (float)((const _Float16*)base)[e];
  return ((const float*)base)[e];
}
}  // namespace

template <int ET, int D>
__global__ __launch_bounds__(64 * kSmallWaves) void attn_fwd_small_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv,
    const void* __restrict__ vv, void* __restrict__ ov, float* __restrict__ lse,
    int M, int N, int causal, float c, int BH, int waves_per_head) {
  constexpr int DQ = D / 4;    // contraction elements per lane group in QK^T
  constexpr int DB = D / 16;   // 16-wide d blocks of O
  const int tid = workitem_id();
  const int lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int wave = tid >> 6;
  const int q0 = (wave % waves_per_head) * kSmallQRows;
  const int qi = q0 + n;
  const size_t bh = (size_t)workgroup_id() * (kSmallWaves / waves_per_head) + wave / waves_per_head;
  if (bh >= (size_t)BH) return;  // (no barrier in this kernel)
  const size_t q_off = bh * (size_t)M * D;
  const size_t kv_off = bh * (size_t)N * D;
  // Key blocks this wave needs: all of them, or under the causal mask only
  // those with a key <= the wave's last query.
  const int n_vis = causal ? min(N, q0 + kSmallQRows) : N;
  const int nkb = (n_vis + 15) >> 4;

  // ---- all loads up front (rows past the end are clamped; their scores are
  // masked, so the clamped values never reach the result).
  float qf[DQ];
  load_row_part<ET, DQ>(qv, q_off + (size_t)min(qi, M - 1) * D + g * DQ, qf);
  float kf[kSmallMaxKB][DQ];
  float vf[kSmallMaxKB][DB][4];
#pragma unroll
  for (int kb = 0; kb < kSmallMaxKB; ++kb) {
    if (kb < nkb) {
      const int kr = min(16 * kb + n, N - 1);
      load_row_part<ET, DQ>(kv, kv_off + (size_t)kr * D + g * DQ, kf[kb]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vr = min(16 * kb + 4 * g + r, N - 1);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vf[kb][db][r] = load_one<ET>(vv, kv_off + (size_t)vr * D + 16 * db + n);
      }
    }
  }

  // ---- S^T = K Q^T, log2-domain scores, masks.
  float s[kSmallMaxKB][4];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kSmallMaxKB; ++kb) {
    if (kb < nkb) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < DQ; ++t) acc = mfma_16x16x4_f32(kf[kb][t], qf[t], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kb + 4 * g + r;
        const bool masked = key >= N || (causal && key > qi);
        s[kb][r] = masked ? -INFINITY : acc[r] * c;
        mx = fmaxf(mx, s[kb][r]);
      }
    }
  }
  mx = half_pair_max(pair16_max(mx));
  // Key 0 is visible to every row, so mx is finite for real rows; the guard
  // keeps clamped tail rows free of inf - inf.
  const float m_sub = mx == -INFINITY ? 0.0f : mx;

  // ---- P = exp2(S - max), row sums, O^T = V^T P^T.
  float l = 0.0f;
  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kb = 0; kb < kSmallMaxKB; ++kb) {
    if (kb < nkb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_sub);
        l += p;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma_16x16x4_f32(vf[kb][db][r], p, o[db]);
      }
    }
  }
  l = half_pair_sum(pair16_sum(l));

  // ---- epilogue: O / l in the input dtype, L = ln 2 * (max + log2 l).
  if (qi < M) {
    const float rinv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const size_t at = q_off + (size_t)qi * D + 16 * db + 4 * g;
      if (ET == kEtBf16) {
        u32x2_t st;
        st[0] = pack_bf16x2(o[db][0] * rinv, o[db][1] * rinv);
        st[1] = pack_bf16x2(o[db][2] * rinv, o[db][3] * rinv);
        *(u32x2_t*)((uint16_t*)ov + at) = st;
      } else if (ET == kEtF16) {
        u32x2_t st;
        st[0] = pack_f16x2(o[db][0] * rinv, o[db][1] * rinv);
        st[1] = pack_f16x2(o[db][2] * rinv, o[db][3] * rinv);
        *(u32x2_t*)((uint16_t*)ov + at) = st;
      } else {
        const f32x4_t st = o[db] * rinv;
        *(f32x4_t*)((float*)ov + at) = st;
      }
    }
    if (g == 0) lse[bh * (size_t)M + qi] = (mx + log2f(l)) * kLn2;
  }
}

hipError_t launch_small(const LaunchArgs& a, int et) {
  if (a.M < 1 || a.M > kSmallMaxM || a.N < 1 || a.N > kSmallMaxN ||
      (a.D != 16 && a.D != 32))
    return hipErrorInvalidValue;
  // Short heads share a workgroup of up to four waves: fewer, larger
  // workgroups launch faster.
  const int wph = (int)((a.M + kSmallQRows - 1) / kSmallQRows);  // waves per head, 1..4
  const int hpw = kSmallWaves / wph;                               // heads per workgroup
  const dim3 grid((unsigned)((a.BH + hpw - 1) / hpw));
  const dim3 block((unsigned)(64 * wph * hpw));
  const float c = a.scale * kLog2e;
  const int M = (int)a.M, N = (int)a.N, causal = (int)a.causal;
#define MI355_SMALL_LAUNCH(ET, DD)                                                   \
  hipLaunchKernelGGL((attn_fwd_small_kernel<ET, DD>), grid, block, 0, a.stream, a.q, \
                     a.k, a.v, a.o, a.lse, M, N, causal, c, (int)a.BH, wph)
  if (et == kEtBf16) {
    if (a.D == 16) MI355_SMALL_LAUNCH(kEtBf16, 16);
    else MI355_SMALL_LAUNCH(kEtBf16, 32);
  } else if (et == kEtF16) {
    if (a.D == 16) MI355_SMALL_LAUNCH(kEtF16, 16);
    else MI355_SMALL_LAUNCH(kEtF16, 32);
  } else {
    if (a.D == 16) MI355_SMALL_LAUNCH(kEtF32, 16);
    else MI355_SMALL_LAUNCH(kEtF32, 32);
  }
#undef MI355_SMALL_LAUNCH
  return hipGetLastError();
}

}  // namespace mi355
