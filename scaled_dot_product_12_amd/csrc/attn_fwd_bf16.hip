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
//  * One workgroup = 8 waves = 256 query rows of one (batch, head), two waves
//    per SIMD. Key/value tiles of 64 rows stream HBM -> VGPRs -> LDS: the
//    global loads of the next tile are issued at the start of an iteration
//    and written to LDS at its end, one s_barrier per iteration.
//  * Ping-pong between the two waves of a SIMD: waves 0-3 (group A) run
//    S(j) = K(j) Q^T, softmax(j), O += V(j)^T P(j)^T in iteration j; waves
//    4-7 (group B) run softmax(j-1), O += V(j-1)^T P(j-1)^T, S(j) = K(j) Q^T,
//    carrying S(j) into the next iteration. While one wave of a SIMD is in
//    its vector-ALU softmax the other keeps the matrix pipe busy.
//  * Both products run on v_mfma_f32_32x32x16_bf16 in transposed form,
//    S^T = K Q^T and O^T += V^T P^T, so the accumulator column -- one query
//    row -- belongs to lanes l and l^32: row max and row sum are in-register
//    reductions plus one permlane32 swap, and the per-row rescale is a
//    per-lane scalar. K rows are stored in LDS in a permuted order so that
//    the 16 score registers of a lane are 16 consecutive keys; rounded to
//    bf16 those registers are directly the B operand (P^T) of the second
//    product.
//  * V stays row-major in LDS. The A operand V^T of the second product is
//    read with ds_read_b64_tr_b16, which transposes 4x16 blocks of 16-bit
//    elements across each 16-lane group on the way out of LDS.
//  * K and V tiles are XOR-swizzled at 16-byte granularity so that the MFMA
//    operand reads of a half-wave hit distinct LDS banks.
//  * Row sums are taken from the bf16-rounded P with v_dot2_f32_bf16, so l
//    and the second product see the same probabilities.
//  * The running max is moved lazily (only when a row max grows by more than
//    2^8), so most tiles skip the O rescale.
//  * Workgroup ids are renumbered so that the query tiles of one head land on
//    one XCD and share its L2 for K/V; causal grids run heavy tiles first.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ s16x4_t lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)(lds_u8*)p);
}

// An empty volatile asm statement: a branch body containing it cannot be
// if-converted into unconditional selects, so the rarely taken wave-uniform
// paths (masking, O rescale) stay off the per-tile instruction stream.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

}  // namespace

// Waves per workgroup: two per SIMD, one of each ping-pong group.
constexpr int kBf16Waves = 8;

template <int D, int WAVES>
struct Bf16Cfg {
  static constexpr int NT = WAVES * 64;
  static constexpr int BM = WAVES * 32;
  static constexpr int BN = 64;                     // keys per tile
  static constexpr int KBUF = 2;                    // K ring depth
  static constexpr int VBUF = 3;                    // V ring depth (group B lags by one tile)
  static constexpr int ROWB = D * 2;                // bytes per key row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;           // bytes per K or V tile
  static constexpr int CHUNKS = TILEB / 16;         // 16-byte chunks per tile
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;  // chunks per thread
  static constexpr int QSTEPS = D / 16;
  static constexpr int DBLK = D < 32 ? 1 : D / 32;  // 32-row blocks of O^T
  static constexpr int V_OFF = KBUF * TILEB;        // V ring after the K ring
  static constexpr int ZERO_OFF = (KBUF + VBUF) * TILEB;  // 64 zero bytes after the rings
  static constexpr int LDS_BYTES = ZERO_OFF + 64;
  // K row r of a tile holds key kperm(r); swizzles act on 16-byte chunks.
  __device__ static constexpr int kperm(int r) {
    const int b = r & 31;
    return (r & ~31) + ((b >> 2) & 1) * 16 + (b >> 3) * 4 + (b & 3);
  }
  __device__ static constexpr int swz_k(int r) { return (r & 15) & (CPR - 1); }
  __device__ static constexpr int swz_v(int r) { return (4 * (r & 3)) & (CPR - 1); }
};

template <int D, int WAVES, bool CAUSAL, bool POS_SCALE>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int M, int N, int tiles_m, int n_wg, float c) {
  using C = Bf16Cfg<D, WAVES>;
  constexpr int NT = C::NT, BM = C::BM, BN = C::BN, ROWB = C::ROWB,
                TILEB = C::TILEB, CPT = C::CPT, QSTEPS = C::QSTEPS, DBLK = C::DBLK;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int wl = xcd_contiguous_id(workgroup_id(), n_wg);
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

  int nt = (N + BN - 1) / BN;
  if (CAUSAL) nt = min(nt, (min(q_wg0 + BM, M) - 1) / BN + 1);
  // tiles this wave computes: [0, wave_nt)
  int wave_nt = 0;
  if (wave_live) wave_nt = CAUSAL ? min(nt, wave_last / BN + 1) : nt;

  if (tid < 16) ((uint32_t*)(smem + C::ZERO_OFF))[tid] = 0u;

  // ---- staging geometry: thread chunk u is LDS chunk ch = tid + u*NT of a
  // tile, i.e. row ch / CPR at swizzled position ch % CPR.
  int k_src[CPT], v_src[CPT], dst[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    int ch = tid + u * NT;
    if (ch >= C::CHUNKS) ch = C::CHUNKS - 1;  // surplus threads repeat the last chunk
    const int R = ch / C::CPR, chp = ch % C::CPR;
    dst[u] = R * ROWB + chp * 16;
    k_src[u] = C::kperm(R) * D + (chp ^ C::swz_k(R)) * 8;  // elements from the tile's first key
    v_src[u] = R * D + (chp ^ C::swz_v(R)) * 8;
  }
  u32x4_t kst[CPT], vst[CPT];
  const int tail_rows = N - (nt - 1) * BN;  // valid rows of the last tile
  auto load_k = [&](int j) {
    const int jc = min(j, nt - 1);
    const uint16_t* base = kh + (size_t)jc * BN * D;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int off = k_src[u];
      if (jc == nt - 1 && off >= tail_rows * D) off = (tail_rows - 1) * D + (off & (D - 1));
      kst[u] = *(const u32x4_t*)(base + off);
    }
  };
  auto load_v = [&](int j) {
    const int jc = min(j, nt - 1);
    const uint16_t* base = vh + (size_t)jc * BN * D;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int off = v_src[u];
      if (jc == nt - 1 && off >= tail_rows * D) off = (tail_rows - 1) * D + (off & (D - 1));
      vst[u] = *(const u32x4_t*)(base + off);
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) *(u32x4_t*)(smem + buf * TILEB + dst[u]) = kst[u];
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) *(u32x4_t*)(smem + C::V_OFF + buf * TILEB + dst[u]) = vst[u];
  };

  // ---- per-lane operand read offsets (bytes within a tile)
  // K (A operand of S^T): LDS row kb*32 + r32, chunk (2t+g) ^ swz.
  const int k_rd = r32 * ROWB;
  const int k_sw = C::swz_k(r32);
  // V^T (A operand of O^T) through ds_read_b64_tr_b16: in 16-lane group G,
  // lane 4*jj + cc supplies row (.. + jj) and d-columns 4*cc .. 4*cc+3 of
  // the group's 16-column slice.
  const int G = lane >> 4, L16 = lane & 15, jj = L16 >> 2, cc = L16 & 3;
  const int gg = G >> 1, nh = G & 1;
  int v_rd[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    const int d0 = b * 32 + nh * 16 + cc * 4;
    if (d0 < D) {
      const int chunk = d0 >> 3;
      v_rd[b] = (gg * 16 + jj) * ROWB + ((chunk ^ C::swz_v(jj)) << 4) + (cc & 1) * 8;
    } else {
      v_rd[b] = -1;  // d beyond the head: read the zero block
    }
  }

  // Q^T as the B operand: lane holds Q[qi][t*16 + g*8 .. +7].
  bf16x8_t qf[QSTEPS];
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qi < M) x = *(const u32x4_t*)(qh + (size_t)qi * D + t * 16 + g * 8);
    qf[t] = __builtin_bit_cast(bf16x8_t, x);
  }

  const float cc_scale = POS_SCALE ? c : 1.0f;
  float m_run = -INFINITY;  // reference max, log2 domain
  float l_run = 0.0f;       // this lane's part of the row sum (of bf16 P)
  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
  f32x16_t s_cur[2];  // scores of the tile in flight

  // Operand fragments are read from LDS PF MFMAs ahead of their use (a ring
  // of PF+1 register fragments), and consecutive MFMAs go to independent
  // accumulators, so LDS latency overlaps matrix work.
  constexpr int PF = 3;

  // S^T = K Q^T for the 64-key tile in buffer buf: fragment i is key block
  // kb = i & 1 at d-step t = i >> 1.
  auto qk = [&](int buf, f32x16_t* s) {
    const unsigned char* kb_base = smem + buf * TILEB + k_rd;
    constexpr int NF = 2 * QSTEPS;
    auto frag = [&](int i) -> u32x4_t {
      const int t = i >> 1, kb = i & 1;
      return *(const u32x4_t*)(kb_base + kb * 32 * ROWB + (((2 * t + g) ^ k_sw) << 4));
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
    u32x4_t fr[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NF; ++i) fr[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      if (i + PF < NF) fr[(i + PF) % (PF + 1)] = frag(i + PF);
      s[i & 1] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[i % (PF + 1)]), qf[i >> 1],
                                    s[i & 1]);
    }
  };

  // O^T += V^T P^T for the tile in V buffer buf: fragment i is O block
  // b = i % DBLK of key step (kb, t) = ((i / DBLK) >> 1, (i / DBLK) & 1).
  auto pv = [&](int buf, const u32x4_t (*p)[2]) {
    const unsigned char* vb_base = smem + C::V_OFF + buf * TILEB;
    const unsigned char* zero = smem + C::ZERO_OFF;
    constexpr int NF = 4 * DBLK;
    typedef __attribute__((ext_vector_type(8))) short s16x8_t;
    auto frag = [&](int i) -> s16x8_t {
      const int b = i % DBLK, kt = i / DBLK, kb = kt >> 1, t = kt & 1;
      const int row_off = (kb * 32 + t * 8) * ROWB;
      const unsigned char* a0 = v_rd[b] < 0 ? zero : vb_base + v_rd[b] + row_off;
      const unsigned char* a1 = v_rd[b] < 0 ? zero : vb_base + v_rd[b] + row_off + 4 * ROWB;
      const s16x4_t lo = lds_read_tr16(a0);
      const s16x4_t hi = lds_read_tr16(a1);
      return (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    s16x8_t fr[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NF; ++i) fr[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      if (i + PF < NF) fr[(i + PF) % (PF + 1)] = frag(i + PF);
      const int b = i % DBLK, kt = i / DBLK;
      acc[b] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[i % (PF + 1)]),
                                  __builtin_bit_cast(bf16x8_t, p[kt >> 1][kt & 1]), acc[b]);
    }
  };

  // Row statistics of a fresh score tile: scale (negative / zero scale),
  // mask (causal diagonal, key tail), tile max, and the lazy reference
  // update. Produces the exponent offset for this tile and whether O and l
  // must be rescaled (by alpha) before its probabilities are added.
  struct TileStats {
    float m_sub;
    float alpha;
    bool resc;
  };
  auto tile_stats = [&](f32x16_t* s, int key0, bool mask) -> TileStats {
    if (!POS_SCALE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] *= c;
    }
    if (mask) {
      keep_branch();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + g * 16 + i;
          if (key >= N || (CAUSAL && key > qi)) s[kb][i] = -INFINITY;
        }
    }
    float mx = __builtin_fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2)
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[kb][i], s[kb][i + 1]));
    mx = half_pair_max(mx);
    const float m_cand = __builtin_fmaxf(m_run, mx * cc_scale);
    TileStats st;
    st.resc = wave_any(m_cand > m_run + kRescaleThreshold);
    const float m_new = st.resc ? m_cand : m_run;
    st.m_sub = (m_new == -INFINITY) ? 0.0f : m_new;
    st.alpha = __builtin_amdgcn_exp2f(m_run - st.m_sub);
    m_run = m_new;
    return st;
  };

  // Probabilities of one 32-key half of a tile: bf16 P (B-operand layout)
  // and their row sum (of the rounded values, via v_dot2_f32_bf16 with 1s).
  auto tile_exp = [&](const f32x16_t& s, float m_sub, u32x4_t* p) -> float {
    // The row sum is accumulated from each freshly rounded bf16 pair (not
    // from elements extracted back out of the packed vector).
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    float rs = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t * 8 + 2 * e], cc_scale, -m_sub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t * 8 + 2 * e + 1], cc_scale, -m_sub));
        const f32x2_t f = {p0, p1};
        const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
        w[e] = __builtin_bit_cast(uint32_t, b);
        rs = __builtin_amdgcn_fdot2_f32_bf16(b, one, rs, false);
      }
      p[t] = w;
    }
    return rs;
  };

  auto rescale = [&](float a) {
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= a;
  };

  auto needs_mask = [&](int j) {
    const int key0 = j * BN;
    return (key0 + BN > N) || (CAUSAL && key0 + BN - 1 > qw0);
  };

  // P(j) from S(j) with its stats, the l update and the O rescale (O holds
  // tiles < j at the previous reference); then O += V(j)^T P(j)^T.
  auto softmax_pv = [&](f32x16_t* s, int j) {
    const TileStats st = tile_stats(s, j * BN, needs_mask(j));
    u32x4_t p[2][2];
    float rs = tile_exp(s[0], st.m_sub, p[0]);
    rs += tile_exp(s[1], st.m_sub, p[1]);
    l_run = (st.resc ? l_run * st.alpha : l_run) + rs;
    if (st.resc) {
      keep_branch();
      rescale(st.alpha);
    }
    pv(j % C::VBUF, p);
  };

  const bool group_b = wave >= WAVES / 2;

  // ---- prologue: K(0), V(0) -> LDS.
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  __syncthreads();  // K(0), V(0) and the zero block visible

  // The two groups run separate copies of the loop (same barrier count) so
  // that each copy is register-allocated for its own live ranges.
  if (!group_b) {
    for (int j = 0; j < nt; ++j) {
      load_k(j + 1);
      load_v(j + 1);
      if (j < wave_nt) {
        qk(j & 1, s_cur);
        softmax_pv(s_cur, j);
      }
      // every wave is past its reads of K(j-1) [buffer (j+1)&1] and of
      // V(j-2) [buffer (j+1)%3]: overwrite them with K(j+1) and V(j+1).
      store_k((j + 1) & 1);
      store_v((j + 1) % C::VBUF);
      __syncthreads();
    }
  } else {
    for (int j = 0; j < nt; ++j) {
      load_k(j + 1);
      load_v(j + 1);
      if (j >= 1 && j - 1 < wave_nt) softmax_pv(s_cur, j - 1);
      if (j < wave_nt) qk(j & 1, s_cur);
      store_k((j + 1) & 1);
      store_v((j + 1) % C::VBUF);
      __syncthreads();
    }
    if (nt - 1 < wave_nt) softmax_pv(s_cur, nt - 1);
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
  constexpr int WAVES = kBf16Waves;
  constexpr int BM = WAVES * 32;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(tiles_m * a.BH));
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, WAVES, CAUSAL, POS>), grid,
                     dim3(WAVES * 64), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, (int)a.M, (int)a.N, tiles_m, tiles_m * (int)a.BH, a.scale * kLog2e);
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

int main_bf16_tile_rows() { return kBf16Waves * 32; }

}  // namespace mi355
