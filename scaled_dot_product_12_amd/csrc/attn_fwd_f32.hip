// attn_fwd_f32.hip -- FlashAttention-2 forward for fp32 inputs on gfx950.
//
// Same algorithm as the bf16 kernel (the tiled online softmax of "Extend
// Thunder with CUDA-Python", Python reference section, run in base 2 as in
// the "Blackwell Attention Example"), with every operand in fp32: both
// products run on v_mfma_f32_32x32x2f32 (the fp32 matrix rate equals the fp32
// vector rate on MI355X, and the MFMA needs no per-lane FMA chains), and P
// stays fp32 for the second product.
//
// Differences from the bf16 kernel:
//  * Q is multiplied by scale*log2(e) once, in fp32, when it is loaded into
//    registers; scores come out of the MFMA already in the log2 domain, for
//    any sign of the scale.
//  * Key tiles are 32 wide. The second product contracts over two keys per
//    MFMA (one per lane half), so its A operand (V^T) is one fp32 from a
//    row-major V tile and V needs no transpose.
//  * Small problems split each row block's keys over 2 or 4 waves of the
//    workgroup and merge the partial (O, m, l) through LDS, so that all
//    SIMDs get an even share (the merge is the one-step combination used to
//    join key-split partial softmaxes: rescale each part to the common max
//    and add).

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

// Waves per workgroup. Wave w takes query rows 32*(w % R) .. +31 of the
// workgroup's tile and key part w / R (KS parts, R = 4 / KS row blocks):
// part p works on key tiles j with j % KS == p, and the KS partial
// results of a row block are merged through LDS at the end. KS > 1 is for
// problems with few 32-row blocks, where one block per wave would leave
// SIMDs idle or unevenly loaded.
constexpr int kF32Waves = 4;

// D is the query/key head dim, DV the value (and output) head dim; the
// Blackwell example's kernel lets them differ.
template <int D, int DV, int KS, bool CAUSAL>
__global__ __launch_bounds__(kF32Waves * 64) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
    int M, int N, int tiles_m, int heads, float c) {
  constexpr int WAVES = kF32Waves;
  constexpr int NT = WAVES * 64;
  constexpr int R = WAVES / KS;        // 32-row blocks per workgroup
  constexpr int BM = R * 32;
  constexpr int BN = 32;
  constexpr int HALF = D / 2;          // d values per lane half
  constexpr int KSTR = D + 4;          // floats per K row in LDS
  constexpr int DP = DV < 32 ? 32 : DV;  // V columns the O^T blocks read
  constexpr int VSTR = DP + 2;           // floats per V row (rows 8-byte aligned)
  constexpr int DBLK = DP / 32;
  constexpr int DCH = D / 4;             // 16-byte chunks per K row
  constexpr int DCHV = DV / 4;           // 16-byte chunks per V row
  constexpr int CH = BN * DCH;           // chunks per K tile
  constexpr int CHV = BN * DCHV;         // chunks per V tile
  constexpr int CPT = (KS * CH + NT - 1) / NT;    // K chunks per thread per step (KS tiles)
  constexpr int CPTV = (KS * CHV + NT - 1) / NT;  // V chunks per thread per step
  constexpr int TILE_F = BN * KSTR + BN * VSTR;  // floats per staged K+V tile
  // partial results of parts 1.. : per lane DBLK*16 accumulators, m, l
  constexpr int PART_F = 64 * (DBLK * 16 + 2);
  constexpr int MERGE_F = (KS - 1) * R * PART_F;
  constexpr int SMEM_F = KS * TILE_F > MERGE_F ? KS * TILE_F : MERGE_F;

  __shared__ __attribute__((aligned(16))) float smem[SMEM_F];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rb = wave % R, part = wave / R;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  float* Ks = smem + part * TILE_F;
  float* Vs = Ks + BN * KSTR;

  const TileId tile = tile_order(workgroup_id(), tiles_m, heads, CAUSAL);
  const int bh = tile.bh, tm = tile.tm;

  const size_t q_off = (size_t)bh * M * D;
  const size_t o_off = (size_t)bh * M * DV;
  const float* qh = q + q_off;
  const float* kh = k + (size_t)bh * N * D;
  const float* vh = v + (size_t)bh * N * DV;

  const int q_wg0 = tm * BM;
  const int qw0 = q_wg0 + rb * 32;
  const int qi = qw0 + r32;
  const bool wave_live = qw0 < M;
  const int wave_last = min(qw0 + 31, M - 1);

  // Q^T as the B operand, pre-scaled: lane holds c*Q[qi][g*HALF + t].
  float qf[HALF];
#pragma unroll
  for (int t4 = 0; t4 < HALF / 4; ++t4) {
    f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
    if (qi < M) x = *(const f32x4_t*)(qh + (size_t)qi * D + g * HALF + t4 * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[t4 * 4 + e] = x[e] * c;
  }

  int nt = (N + BN - 1) / BN;
  if (CAUSAL) {
    const int q_last = min(q_wg0 + BM, M) - 1;
    nt = min(nt, q_last / BN + 1);
  }
  const int steps = (nt + KS - 1) / KS;

  if (DV < 32) {  // V columns DV..31 stay zero
    for (int idx = tid; idx < KS * BN * (DP - DV); idx += NT) {
      const int pp = idx / (BN * (DP - DV)), rem = idx - pp * (BN * (DP - DV));
      const int row = rem / (DP - DV);
      smem[pp * TILE_F + BN * KSTR + row * VSTR + DV + (rem - row * (DP - DV))] = 0.0f;
    }
  }

  // Step s stages tile s*KS + pp into buffer pp, for every part pp.
  // With equal head dims a K chunk and the V chunk at the same position are
  // loaded and stored together (one index computation for both); otherwise
  // the two tiles have their own chunk loops.
  f32x4_t kreg[CPT], vreg[CPTV];
  auto load_step = [&](int st) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ch = tid + u * NT;
      if (ch < KS * CH) {
        const int pp = ch / CH, cl = ch - pp * CH;
        const int row = cl / DCH;
        const int col = (cl - row * DCH) * 4;
        const int key = (st * KS + pp) * BN + row;
        f32x4_t xk = {0.0f, 0.0f, 0.0f, 0.0f}, xv = xk;
        if (key < min(N, nt * BN)) {
          xk = *(const f32x4_t*)(kh + (size_t)key * D + col);
          if constexpr (D == DV) xv = *(const f32x4_t*)(vh + (size_t)key * DV + col);
        }
        kreg[u] = xk;
        if constexpr (D == DV) vreg[u] = xv;
      }
    }
    if constexpr (D != DV) {
#pragma unroll
      for (int u = 0; u < CPTV; ++u) {
        const int ch = tid + u * NT;
        if (ch < KS * CHV) {
          const int pp = ch / CHV, cl = ch - pp * CHV;
          const int row = cl / DCHV;
          const int col = (cl - row * DCHV) * 4;
          const int key = (st * KS + pp) * BN + row;
          f32x4_t xv = {0.0f, 0.0f, 0.0f, 0.0f};
          if (key < min(N, nt * BN)) xv = *(const f32x4_t*)(vh + (size_t)key * DV + col);
          vreg[u] = xv;
        }
      }
    }
  };
  auto store_v = [&](float* vb, int row, int col, const f32x4_t& x) {
    f32x2_t lo = {x[0], x[1]}, hi = {x[2], x[3]};
    *(f32x2_t*)(vb + row * VSTR + col) = lo;
    *(f32x2_t*)(vb + row * VSTR + col + 2) = hi;
  };
  auto store_step = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ch = tid + u * NT;
      if (ch < KS * CH) {
        const int pp = ch / CH, cl = ch - pp * CH;
        const int row = cl / DCH;
        const int col = (cl - row * DCH) * 4;
        float* kb = smem + pp * TILE_F;
        *(f32x4_t*)(kb + row * KSTR + col) = kreg[u];
        if constexpr (D == DV) store_v(kb + BN * KSTR, row, col, vreg[u]);
      }
    }
    if constexpr (D != DV) {
#pragma unroll
      for (int u = 0; u < CPTV; ++u) {
        const int ch = tid + u * NT;
        if (ch < KS * CHV) {
          const int pp = ch / CHV, cl = ch - pp * CHV;
          const int row = cl / DCHV;
          const int col = (cl - row * DCHV) * 4;
          store_v(smem + pp * TILE_F + BN * KSTR, row, col, vreg[u]);
        }
      }
    }
  };

  const int krow = ((r32 >> 2) & 1) * 16 + (r32 >> 3) * 4 + (r32 & 3);

  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;

  if (steps > 0) load_step(0);
  for (int st = 0; st < steps; ++st) {
    __syncthreads();
    store_step();
    __syncthreads();
    if (st + 1 < steps) load_step(st + 1);
    const int j = st * KS + part;
    const int key0 = j * BN;
    if (!wave_live || j >= nt) continue;
    if (CAUSAL && key0 > wave_last) continue;

    // S^T = K (cQ)^T, one 32-key block: lane owns keys g*16 + i.
    f32x16_t s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
    const float* kp = Ks + krow * KSTR + g * HALF;
#pragma unroll
    for (int t4 = 0; t4 < HALF / 4; ++t4) {
      const f32x4_t a = *(const f32x4_t*)(kp + t4 * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma_32x32x2_f32(a[e], qf[t4 * 4 + e], s);
    }
    const bool need_mask = (key0 + BN > N) || (CAUSAL && key0 + BN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + g * 16 + i;
        if (key >= N || (CAUSAL && key > qi)) s[i] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = half_pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
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
    float p[16];
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(s[i] - m_sub);
      rs += p[i];
    }
    l_run += rs;

    // O^T += V^T P^T: MFMA t contracts keys t (lanes 0-31) and 16+t (32-63).
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const float* vp = Vs + (g * 16) * VSTR + b * 32 + r32;
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[b] = mfma_32x32x2_f32(vp[t * VSTR], p[t], acc[b]);
    }
  }

  // Merge the key parts of each row block (same lane layout in every part):
  // m = max_p m_p, O = sum_p 2^(m_p - m) O_p, l = sum_p 2^(m_p - m) l_p.
  if (KS > 1) {
    __syncthreads();  // every wave is done with the staged tiles
    if (part > 0) {
      float* dstp = smem + ((part - 1) * R + rb) * PART_F + lane;
#pragma unroll
      for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) dstp[(b * 16 + i) * 64] = acc[b][i];
      dstp[(DBLK * 16) * 64] = m_run;
      dstp[(DBLK * 16 + 1) * 64] = l_run;
    }
    __syncthreads();
    if (part > 0) return;
#pragma unroll
    for (int pp = 1; pp < KS; ++pp) {
      const float* srcp = smem + ((pp - 1) * R + rb) * PART_F + lane;
      const float m_p = srcp[(DBLK * 16) * 64];
      const float l_p = srcp[(DBLK * 16 + 1) * 64];
      const float m_new = fmaxf(m_run, m_p);
      const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
      const float a_self = __builtin_amdgcn_exp2f(m_run - m_ref);
      const float a_p = __builtin_amdgcn_exp2f(m_p - m_ref);
#pragma unroll
      for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = acc[b][i] * a_self + srcp[(b * 16 + i) * 64] * a_p;
      l_run = l_run * a_self + l_p * a_p;
      m_run = m_new;
    }
  }

  if (!wave_live) return;
  const float l_tot = half_pair_sum(l_run);
  if (qi >= M) return;
  const float inv = 1.0f / l_tot;
  float* orow = o + o_off + (size_t)qi * DV;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = b * 32 + i4 * 8 + g * 4;
      if (d0 < DV) {
        f32x4_t st = {acc[b][i4 * 4 + 0] * inv, acc[b][i4 * 4 + 1] * inv,
                      acc[b][i4 * 4 + 2] * inv, acc[b][i4 * 4 + 3] * inv};
        *(f32x4_t*)(orow + d0) = st;
      }
    }
  if (g == 0) lse[(size_t)bh * M + qi] = (m_run + log2f(l_tot)) * kLn2;
}

// Key parts per row block: 1 when the problem has at least two 32-row blocks
// per SIMD (1024 SIMDs), else split the keys so that every SIMD gets work.
static int f32_key_split(int64_t BH, int64_t M) {
  const int64_t blocks = BH * ((M + 31) / 32);
  return blocks >= 2048 ? 1 : (blocks >= 512 ? 2 : 4);
}

template <int D, int DV, int KS, bool CAUSAL>
static hipError_t launch_f32_dk(const LaunchArgs& a) {
  constexpr int BM = (kF32Waves / KS) * 32;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(tiles_m * a.BH));
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, DV, KS, CAUSAL>), grid, dim3(kF32Waves * 64), 0,
                     a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                     (float*)a.o, a.lse, (int)a.M, (int)a.N, tiles_m, (int)a.BH,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, int DV, bool CAUSAL>
static hipError_t launch_f32_d(const LaunchArgs& a) {
  switch (f32_key_split(a.BH, a.M)) {
    case 1: return launch_f32_dk<D, DV, 1, CAUSAL>(a);
    case 2: return launch_f32_dk<D, DV, 2, CAUSAL>(a);
    default: return launch_f32_dk<D, DV, 4, CAUSAL>(a);
  }
}

template <int D, int DV>
static hipError_t launch_f32_dispatch(const LaunchArgs& a) {
  return a.causal ? launch_f32_d<D, DV, true>(a) : launch_f32_d<D, DV, false>(a);
}

template <int D>
static hipError_t launch_f32_dv(const LaunchArgs& a) {
  switch (a.Dv) {
    case 16: return launch_f32_dispatch<D, 16>(a);
    case 32: return launch_f32_dispatch<D, 32>(a);
    case 64: return launch_f32_dispatch<D, 64>(a);
    case 128: return launch_f32_dispatch<D, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_main_f32(const LaunchArgs& a) {
  switch (a.D) {
    case 16: return launch_f32_dv<16>(a);
    case 32: return launch_f32_dv<32>(a);
    case 64: return launch_f32_dv<64>(a);
    case 128: return launch_f32_dv<128>(a);
    default: return hipErrorInvalidValue;
  }
}

// Smallest query tile of any launch (KS = 4): the grid-size check uses it.
int main_f32_tile_rows() { return 32; }

}  // namespace mi355
