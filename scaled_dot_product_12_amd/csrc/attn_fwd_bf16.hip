// attn_fwd_bf16.hip -- FlashAttention-2 forward for bf16 inputs on gfx950.
//
// The algorithm is the tiled online softmax of "Extend Thunder with
// CUDA-Python" (Python reference section): for a tile of query rows, loop
// over key/value tiles; S = scale * Q K^T; keep a running row max m and row
// sum l; rescale the output accumulator when m moves; finish with O / l and
// L = m + ln l. As in the "Blackwell Attention Example" attention kernel the
// softmax runs in base 2 with scale * log2(e) folded in, P is rounded to the
// value dtype (bf16) before the second product, and both products accumulate
// in fp32. Causal tiles past the diagonal are skipped, diagonal tiles masked
// (key > query -> -inf), as in the Python reference.
//
// gfx950 mapping (not the pages' design):
//  * One workgroup = WAVES waves = WAVES*32 query rows of one (batch, head);
//    the K/V tiles (64 keys) are staged through LDS and shared by all waves.
//  * Both products run on v_mfma_f32_32x32x16_bf16 in transposed form,
//    S^T = K Q^T and O^T += V^T P^T, so the accumulator column -- one query
//    row -- belongs to lanes l and l^32. Row max and row sum are then
//    in-register reductions plus one permlane32 swap, and the per-row rescale
//    is a per-lane scalar. The K rows feeding the A operand are permuted so
//    that the 16 score registers of a lane are 16 consecutive keys; those
//    same registers, rounded to bf16, are directly the B operand (P^T) of
//    the second product with no data movement.
//  * V is written to LDS transposed (V^T[d][key]) by an in-register 4x8
//    transpose, so the A operand (V^T) of the second product is one 16-byte
//    LDS read per MFMA, like K for the first.
//  * The running max is moved lazily (only when a row max grows by more than
//    2^8), so most tiles skip the O rescale.
//  * Workgroup ids are renumbered so that the query tiles of one head land on
//    one XCD and share its L2 for K/V; causal grids run heavy tiles first.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

template <int D, int WAVES, bool CAUSAL, bool POS_SCALE>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int M, int N, int tiles_m, float c) {
  constexpr int NT = WAVES * 64;
  constexpr int BM = WAVES * 32;
  constexpr int BN = 64;
  constexpr int KSTR = D + 8;          // bf16 per K row in LDS (16-byte pad)
  constexpr int DP = D < 32 ? 32 : D;  // V^T rows; O^T works in 32-row blocks
  constexpr int VSTR = BN + 8;         // bf16 per V^T row (16-byte pad)
  constexpr int QSTEPS = D / 16;       // k-steps of the first product
  constexpr int DBLK = DP / 32;        // 32-row blocks of O^T
  constexpr int DCH = D / 8;           // 16-byte chunks per row
  constexpr int KCH = BN * DCH;        // 16-byte chunks per K tile
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VIT = (BN / 4) * DCH;  // (4 keys x 8 d) blocks per V tile
  constexpr int VPT = (VIT + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DP * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int wl = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int bh = wl / tiles_m;
  int tm = wl - bh * tiles_m;
  if (CAUSAL) tm = tiles_m - 1 - tm;  // longest rows first

  const size_t q_off = (size_t)bh * M * D;
  const size_t kv_off = (size_t)bh * N * D;
  const uint16_t* qh = q + q_off;
  const uint16_t* kh = k + kv_off;
  const uint16_t* vh = v + kv_off;

  const int q_wg0 = tm * BM;
  const int qw0 = q_wg0 + wave * 32;
  const int qi = qw0 + r32;  // this lane's query row
  const bool wave_live = qw0 < M;
  const int wave_last = min(qw0 + 31, M - 1);

  // Q^T as the B operand: lane holds Q[qi][t*16 + g*8 .. +7].
  bf16x8_t qf[QSTEPS];
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qi < M) x = *(const u32x4_t*)(qh + (size_t)qi * D + t * 16 + g * 8);
    qf[t] = __builtin_bit_cast(bf16x8_t, x);
  }

  int nt = (N + BN - 1) / BN;
  if (CAUSAL) {
    const int q_last = min(q_wg0 + BM, M) - 1;
    nt = min(nt, q_last / BN + 1);
  }

  if (D < 32) {  // V^T rows D..31 stay zero for the whole kernel
    for (int idx = tid; idx < (DP - D) * VSTR; idx += NT) Vt[D * VSTR + idx] = 0;
  }

  u32x4_t kreg[KPT];
  u32x4_t vreg[VPT][4];

  auto load_tile = [&](int j) {
    const int key0 = j * BN;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ch = tid + u * NT;
      if (ch < KCH) {
        const int row = ch / DCH;
        const int col = (ch - row * DCH) * 8;
        const int key = key0 + row;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (key < N) x = *(const u32x4_t*)(kh + (size_t)key * D + col);
        kreg[u] = x;
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int it = tid + u * NT;
      if (it < VIT) {
        const int kg = it / DCH;
        const int dc = it - kg * DCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + kg * 4 + r;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (key < N) x = *(const u32x4_t*)(vh + (size_t)key * D + dc * 8);
          vreg[u][r] = x;
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ch = tid + u * NT;
      if (ch < KCH) {
        const int row = ch / DCH;
        const int col = (ch - row * DCH) * 8;
        *(u32x4_t*)(Ks + row * KSTR + col) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int it = tid + u * NT;
      if (it < VIT) {
        const int kg = it / DCH;
        const int dc = it - kg * DCH;
        // 4 keys x 8 d in registers -> 8 rows of V^T, 4 keys each.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t a0 = vreg[u][0][w], a1 = vreg[u][1][w];
          const uint32_t a2 = vreg[u][2][w], a3 = vreg[u][3][w];
          u32x2_t pk;
          if (e & 1) {
            pk[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            pk[1] = (a2 >> 16) | (a3 & 0xffff0000u);
          } else {
            pk[0] = (a0 & 0xffffu) | (a1 << 16);
            pk[1] = (a2 & 0xffffu) | (a3 << 16);
          }
          *(u32x2_t*)(Vt + (dc * 8 + e) * VSTR + kg * 4) = pk;
        }
      }
    }
  };

  // A-operand row r of each 32-key block reads key perm(r) so that lane
  // group g ends up owning keys g*16 .. g*16+15 in register order.
  const int krow = ((r32 >> 2) & 1) * 16 + (r32 >> 3) * 4 + (r32 & 3);
  const float cc = POS_SCALE ? c : 1.0f;

  float m_run = -INFINITY;  // reference max, log2 domain
  float l_run = 0.0f;       // this lane's part of the row sum
  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;

  if (nt > 0) load_tile(0);
  for (int j = 0; j < nt; ++j) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < nt) load_tile(j + 1);
    const int key0 = j * BN;
    if (!wave_live) continue;
    if (CAUSAL && key0 > wave_last) continue;  // every key after every row

    // S^T = K Q^T for two 32-key blocks.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
      const uint16_t* kp = Ks + (kb * 32 + krow) * KSTR + g * 8;
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kp + t * 16));
        s[kb] = mfma_32x32x16_bf16(a, qf[t], s[kb]);
      }
    }
    if (!POS_SCALE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] *= c;
    }
    const bool need_mask = (key0 + BN > N) || (CAUSAL && key0 + BN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + g * 16 + i;
          if (key >= N || (CAUSAL && key > qi)) s[kb][i] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = half_pair_max(mx);
    const float m_new = fmaxf(m_run, mx * cc);
    if (wave_any(m_new > m_run + kRescaleThreshold)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;
      m_run = m_new;
    }
    const float m_sub = (m_run == -INFINITY) ? 0.0f : m_run;

    // P = exp2(S*c - m), its row sum, and P^T (bf16) as the B operand.
    bf16x8_t pb[2][2];
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(s[kb][t * 8 + e], cc, -m_sub));
          rs += p[e];
        }
        u32x4_t w;
        w[0] = pack_bf16x2(p[0], p[1]);
        w[1] = pack_bf16x2(p[2], p[3]);
        w[2] = pack_bf16x2(p[4], p[5]);
        w[3] = pack_bf16x2(p[6], p[7]);
        pb[kb][t] = __builtin_bit_cast(bf16x8_t, w);
      }
    l_run += rs;

    // O^T += V^T P^T.
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const uint16_t* vp = Vt + (b * 32 + r32) * VSTR + g * 16;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(vp + kb * 32 + t * 8));
          acc[b] = mfma_32x32x16_bf16(a, pb[kb][t], acc[b]);
        }
    }
  }

  if (!wave_live) return;
  const float l_tot = half_pair_sum(l_run);
  if (qi >= M) return;
  const float inv = 1.0f / l_tot;
  uint16_t* orow = o + q_off + (size_t)qi * D;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = b * 32 + i4 * 8 + g * 4;
      if (d0 < D) {
        u32x2_t st;
        st[0] = pack_bf16x2(acc[b][i4 * 4 + 0] * inv, acc[b][i4 * 4 + 1] * inv);
        st[1] = pack_bf16x2(acc[b][i4 * 4 + 2] * inv, acc[b][i4 * 4 + 3] * inv);
        *(u32x2_t*)(orow + d0) = st;
      }
    }
  if (g == 0) lse[(size_t)bh * M + qi] = (m_run + log2f(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool POS>
static hipError_t launch_bf16_d(const LaunchArgs& a) {
  constexpr int WAVES = 8;
  constexpr int BM = WAVES * 32;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(tiles_m * a.BH));
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, WAVES, CAUSAL, POS>), grid,
                     dim3(WAVES * 64), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, (int)a.M, (int)a.N, tiles_m, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_dispatch(const LaunchArgs& a) {
  const bool pos = a.scale > 0.0f;
  if (a.causal) return pos ? launch_bf16_d<D, true, true>(a) : launch_bf16_d<D, true, false>(a);
  return pos ? launch_bf16_d<D, false, true>(a) : launch_bf16_d<D, false, false>(a);
}

hipError_t launch_main_bf16(const LaunchArgs& a) {
  switch (a.D) {
    case 16: return launch_bf16_dispatch<16>(a);
    case 32: return launch_bf16_dispatch<32>(a);
    case 64: return launch_bf16_dispatch<64>(a);
    case 128: return launch_bf16_dispatch<128>(a);
    default: return hipErrorInvalidValue;
  }
}

int main_bf16_tile_rows() { return 8 * 32; }

}  // namespace mi355
