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
//  * One workgroup = 4 waves = 128 query rows of one (batch, head), one wave
//    per SIMD; two workgroups share a CU. Key/value tiles of 64 rows stream
//    HBM -> VGPRs -> LDS: the global loads of a tile are issued one
//    iteration ahead and written to LDS at the end of the iteration, one
//    s_barrier per iteration, double-buffered K and V rings.
//  * Software pipeline inside each wave: iteration j computes
//    S(j+1) = K(j+1) Q^T on the matrix cores while the vector ALU turns S(j)
//    into probabilities P(j), then O += V(j)^T P(j)^T on the matrix cores
//    while the vector ALU takes the row statistics of S(j+1). The two
//    halves of each iteration are independent instruction streams, and
//    sched_group_barrier interleaves them (one MFMA, then a few VALU and LDS
//    instructions), so the softmax runs in the shadow of the MFMAs.
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

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x002;
constexpr int kSgMfma = 0x008;
constexpr int kSgVmemRead = 0x020;
constexpr int kSgDsRead = 0x100;
constexpr int kSgDsWrite = 0x200;
// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle): loads past num_records return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

#define MI355_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

}  // namespace

// Waves per workgroup: one per SIMD.
constexpr int kBf16Waves = 4;

template <int D, int WAVES>
struct Bf16Cfg {
  static constexpr int NT = WAVES * 64;
  static constexpr int BM = WAVES * 32;
  static constexpr int BN = 64;                     // keys per tile
  static constexpr int ROWB = D * 2;                // bytes per key row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;           // bytes per K or V tile
  static constexpr int CHUNKS = TILEB / 16;         // 16-byte chunks per tile
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;  // chunks per thread
  static constexpr int QSTEPS = D / 16;
  static constexpr int DBLK = D < 32 ? 1 : D / 32;  // 32-row blocks of O^T
  static constexpr int NF_QK = 2 * QSTEPS;          // MFMAs of one S tile
  static constexpr int NF_PV = 4 * DBLK;            // MFMAs of one O update
  static constexpr int V_OFF = 2 * TILEB;           // K ring (2), then V ring (2)
  static constexpr int ZERO_OFF = 4 * TILEB;        // 64 zero bytes after the rings
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
                TILEB = C::TILEB, CPT = C::CPT, QSTEPS = C::QSTEPS, DBLK = C::DBLK,
                NF_QK = C::NF_QK, NF_PV = C::NF_PV;

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

  // Key tiles the workgroup visits. Under the causal mask a wave may visit
  // up to two tiles that are fully masked for its rows; they contribute
  // exact zeros.
  int nt = (N + BN - 1) / BN;
  if (CAUSAL) nt = min(nt, (min(q_wg0 + BM, M) - 1) / BN + 1);

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
  // Tile loads go through buffer descriptors bounded by the head's last key
  // row: chunks past it read as zeros (finite, and masked or multiplied by
  // p = 0), so the tail needs no per-lane clamp and tiles past the end need
  // no guard. Offsets are per-lane constants; the tile base is scalar.
  auto tile_rsrc = [&](const uint16_t* head, int j) {
    const int jc = min(j, nt - 1);
    const uint32_t bytes = (uint32_t)(N - jc * BN) * (uint32_t)ROWB;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (size_t)jc * BN * D), (short)0,
                                             (int)bytes, kBufferRsrcWord3);
  };
  auto load_k = [&](int j) {
    const auto r = tile_rsrc(kh, j);
#pragma unroll
    for (int u = 0; u < CPT; ++u) kst[u] = __builtin_amdgcn_raw_buffer_load_b128(r, 2 * k_src[u], 0, 0);
  };
  auto load_v = [&](int j) {
    const auto r = tile_rsrc(vh, j);
#pragma unroll
    for (int u = 0; u < CPT; ++u) vst[u] = __builtin_amdgcn_raw_buffer_load_b128(r, 2 * v_src[u], 0, 0);
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
  float m_sub = 0.0f;       // exponent offset of the tile being exponentiated
  float l_run = 0.0f;       // this lane's part of the row sum (of bf16 P)
  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
  f32x16_t s_a[2], s_b[2];  // scores of two consecutive tiles

  // S^T = K Q^T for the 64-key tile in K buffer buf: fragment i is key
  // block kb = i & 1 at d-step t = i >> 1.
  auto qk = [&](int buf, f32x16_t* s) {
    const unsigned char* kb_base = smem + buf * TILEB + k_rd;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < NF_QK; ++i) {
      const int t = i >> 1, kb = i & 1;
      const u32x4_t fr =
          *(const u32x4_t*)(kb_base + kb * 32 * ROWB + (((2 * t + g) ^ k_sw) << 4));
      s[kb] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr), qf[t], s[kb]);
    }
  };

  // O^T += V^T P^T for the tile in V buffer buf: fragment i is O block
  // b = i % DBLK of key step (kb, t) = ((i / DBLK) >> 1, (i / DBLK) & 1).
  auto pv = [&](int buf, const u32x4_t (*p)[2]) {
    const unsigned char* vb_base = smem + C::V_OFF + buf * TILEB;
    const unsigned char* zero = smem + C::ZERO_OFF;
    typedef __attribute__((ext_vector_type(8))) short s16x8_t;
#pragma unroll
    for (int i = 0; i < NF_PV; ++i) {
      const int b = i % DBLK, kt = i / DBLK, kb = kt >> 1, t = kt & 1;
      const int row_off = (kb * 32 + t * 8) * ROWB;
      const unsigned char* a0 = v_rd[b] < 0 ? zero : vb_base + v_rd[b] + row_off;
      const unsigned char* a1 = v_rd[b] < 0 ? zero : vb_base + v_rd[b] + row_off + 4 * ROWB;
      const s16x4_t lo = lds_read_tr16(a0);
      const s16x4_t hi = lds_read_tr16(a1);
      const s16x8_t fr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[b] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr),
                                  __builtin_bit_cast(bf16x8_t, p[kb][t]), acc[b]);
    }
  };

  // Scale (negative / zero scale only) and mask (causal diagonal, key tail)
  // a fresh score tile. Only tiles that need it go through the mask.
  auto needs_mask = [&](int j) {
    const int key0 = j * BN;
    return (key0 + BN > N) || (CAUSAL && key0 + BN - 1 > qw0);
  };
  auto scale_tile = [&](f32x16_t* s) {
    if (!POS_SCALE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] *= c;
    }
  };
  auto mask_tile = [&](f32x16_t* s, int j) {
    const int key0 = j * BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + kb * 32 + g * 16 + i;
        if (key >= N || (CAUSAL && key > qi)) s[kb][i] = -INFINITY;
      }
  };

  // Row statistics of a prepared score tile: tile max and the lazy
  // reference update. Sets m_sub for the tile's exponentials; returns
  // whether O and l must be rescaled by alpha before its probabilities are
  // added.
  auto stats = [&](const f32x16_t* s, float& alpha) -> bool {
    float mx = __builtin_fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2)
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[kb][i], s[kb][i + 1]));
    mx = half_pair_max(mx);
    const float m_cand = __builtin_fmaxf(m_run, mx * cc_scale);
    const bool resc = wave_any(m_cand > m_run + kRescaleThreshold);
    const float m_new = resc ? m_cand : m_run;
    m_sub = (m_new == -INFINITY) ? 0.0f : m_new;
    alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
    m_run = m_new;
    return resc;
  };

  // Probabilities of one 32-key half of a tile: bf16 P (B-operand layout)
  // and their row sum (of the rounded values, via v_dot2_f32_bf16 with 1s).
  auto tile_exp = [&](const f32x16_t& s, u32x4_t* p) -> float {
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

  // Instruction interleave of the first half of an iteration: the S(j+1)
  // MFMAs with their K reads, the exponentials of S(j), and the global
  // loads of the tiles after next.
  auto sched_a = [&]() {
    constexpr int VALU = (96 + NF_QK - 1) / NF_QK;
    constexpr int VMEM = 2 * CPT;
    MI355_SCHED(kSgDsRead, 2);
#pragma unroll
    for (int i = 0; i < NF_QK; ++i) {
      MI355_SCHED(kSgMfma, 1);
      if (i + 2 < NF_QK) MI355_SCHED(kSgDsRead, 1);
      if (i < VMEM) MI355_SCHED(kSgVmemRead, 1);
      MI355_SCHED(kSgValu, VALU);
    }
  };
  // Second half: the O MFMAs with their V^T reads, the statistics of
  // S(j+1), and the LDS writes of the staged tiles at the end.
  auto sched_b = [&]() {
    MI355_SCHED(kSgDsRead, 4);
#pragma unroll
    for (int i = 0; i < NF_PV; ++i) {
      MI355_SCHED(kSgMfma, 1);
      if (2 * i + 4 < 2 * NF_PV) MI355_SCHED(kSgDsRead, 2);
      MI355_SCHED(kSgValu, 3);
    }
    MI355_SCHED(kSgDsWrite, 2 * CPT);
  };

  // One iteration: tile j is exponentiated and added to O; with a next
  // tile, S(j+1) is computed alongside and its statistics taken, and the
  // tiles K(j+2), V(j+1) are staged into the buffers freed one iteration
  // ago. MASKED: tile j+1 may need the causal / tail mask (a few tiles per
  // workgroup); the common unmasked step has no branch between its halves,
  // so the interleave spans the whole iteration.
  auto step = [&](int j, f32x16_t* sc, f32x16_t* sn, bool has_next, bool masked) {
    if (has_next) {
      load_k(j + 2);
      load_v(j + 1);
      qk((j + 1) & 1, sn);
    }
    u32x4_t p[2][2];
    float rs = tile_exp(sc[0], p[0]);
    rs += tile_exp(sc[1], p[1]);
    if (has_next && !masked) sched_a();
    l_run += rs;
    if (has_next) {
      scale_tile(sn);
      if (masked && needs_mask(j + 1)) {
        keep_branch();
        mask_tile(sn, j + 1);
      }
    }
    pv(j & 1, p);
    if (has_next) {
      float alpha;
      const bool resc = stats(sn, alpha);
      store_k(j & 1);
      store_v((j + 1) & 1);
      if (!masked) sched_b();
      if (resc) {
        keep_branch();
        rescale(alpha);
        l_run *= alpha;
      }
      __syncthreads();
    }
  };

  // ---- prologue: K(0), K(1), V(0) -> LDS; S(0) and its statistics.
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  __syncthreads();  // K(0), K(1), V(0) and the zero block visible
  qk(0, s_a);
  scale_tile(s_a);
  if (needs_mask(0)) {
    keep_branch();
    mask_tile(s_a, 0);
  }
  {
    float alpha;
    stats(s_a, alpha);  // O and l are still zero: nothing to rescale
  }
  __syncthreads();  // every wave is done with K(0) before step 0 restages its buffer

  // Steps j < jf have an unmasked tile j+1 (for every wave of the group);
  // the rest run the masked variant. The current tile is in s_a at the
  // start of each loop.
  int j_free = N / BN;  // tiles without a key tail
  if (CAUSAL) j_free = min(j_free, (q_wg0 + 1) / BN);  // below the diagonal for all rows
  const int jf = max(0, min(nt - 1, j_free - 1));
  int j = 0;
  for (; j + 1 < jf; j += 2) {
    step(j, s_a, s_b, true, false);
    step(j + 1, s_b, s_a, true, false);
  }
  if (j < jf) {
    step(j, s_a, s_b, true, false);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_a[kb] = s_b[kb];
    ++j;
  }
  for (; j + 1 < nt; ++j) {
    step(j, s_a, s_b, true, true);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_a[kb] = s_b[kb];
  }
  step(nt - 1, s_a, s_b, false, false);

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
