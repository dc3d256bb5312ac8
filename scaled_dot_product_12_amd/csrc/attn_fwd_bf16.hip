// attn_fwd_bf16.hip -- FlashAttention-2 forward for 16-bit (bf16, fp16)
// inputs on gfx950.
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
//  * One workgroup = 8 waves = 256 query rows of one (batch, head), two
//    waves per SIMD; each staged K/V tile serves 256 rows. Key/value tiles of 64 rows stream
//    HBM -> VGPRs -> LDS through bounded buffer loads, written to LDS half an
//    iteration after they are issued (K in the first half, V in the second);
//    rings of 3 K and 2 V tiles, one s_barrier per iteration.
//  * Software pipeline inside each wave: iteration j runs S(j+1) =
//    K(j+1) Q^T on the matrix cores while the vector ALU turns S(j) into
//    P(j), then O += V(j)^T P(j)^T, whose MFMAs need almost no vector work,
//    so the two waves of a SIMD overlap one's exponentials with the other's
//    products. Each half is written as sched_barrier-fenced chunks of one
//    MFMA plus a share of the vector work and of the operand reads, so the
//    compiler can neither cluster the MFMAs nor the exponentials.
//  * The common tile needs no row max. After the first tile sets the
//    reference m to its exact row max, a tile is exponentiated against the
//    current m; every p is >= 0, so a lane's partial row sum bounds each of
//    its p. Only when that sum exceeds 2^16 (some score rose more than ~11
//    above m, in log2 units) does the tile take the exact path: S recomputed
//    from the K tile still in LDS, row max, new m, O and l rescaled, P
//    recomputed. The reference therefore moves rarely and never lets p or
//    the fp32 sums approach overflow.
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
//  * V tiles are XOR-swizzled at 16-byte granularity and K rows padded by
//    16 bytes, so that the MFMA operand reads of a half-wave hit distinct
//    LDS banks; the padding makes every K fragment an immediate offset from
//    one base address per tile.
//  * Row sums are taken from the bf16-rounded P with v_dot2_f32_bf16, so l
//    and the second product see the same probabilities.
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

// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle): loads past num_records return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;


}  // namespace

// Waves per workgroup: 8 (256 query rows, two waves per SIMD) for D = 128;
// 4 (128 rows) for smaller heads, whose lighter register use lets three
// workgroups share a CU, i.e. three waves per SIMD to overlap the softmax of
// one with the products of another.
constexpr int kBf16Waves = 8;
__host__ __device__ constexpr int bf16_waves(int D) { return D <= 64 ? 4 : kBf16Waves; }
__host__ __device__ constexpr int bf16_blocks_per_cu(int D) { return D <= 64 ? 3 : 1; }

// D: query/key head dim; DV: value/output head dim (equal unless the caller
// gives v a head dim of its own).
template <int D, int DV, int WAVES>
struct Bf16Cfg {
  static constexpr int NT = WAVES * 64;
  static constexpr int BM = WAVES * 32;
  static constexpr int BN = 64;                     // keys per tile
  static constexpr int ROWB = D * 2;                // bytes per key row
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILEB = BN * ROWB;           // bytes of a K tile's data
  static constexpr int VROWB = DV * 2;              // bytes per value row
  static constexpr int VCPR = DV / 8;               // 16-byte chunks per value row
  static constexpr int VTILEB = BN * VROWB;         // bytes per V tile
  // K rows sit 16 bytes apart beyond their length in LDS: consecutive rows
  // then start 4 banks apart, so the 16 rows a half-wave reads at one column
  // hit 16 distinct 4-bank groups, and a lane's fragment for d-step t is its
  // row base plus 32 t -- an immediate offset, no per-step address register.
  static constexpr int KROWB = ROWB + 16;           // LDS bytes per K row
  static constexpr int KTILEB = BN * KROWB;         // LDS bytes per K tile
  static constexpr int CHUNKS = TILEB / 16;         // 16-byte chunks per tile
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;  // K chunks per thread
  static constexpr int VCHUNKS = VTILEB / 16;
  static constexpr int VCPT = (VCHUNKS + NT - 1) / NT;  // V chunks per thread
  static constexpr int QSTEPS = D / 16;
  static constexpr int DBLK = DV < 32 ? 1 : DV / 32;  // 32-row blocks of O^T
  static constexpr int NF_QK = 2 * QSTEPS;          // MFMAs of one S tile
  static constexpr int NF_PV = 4 * DBLK;            // MFMAs of one O update
  static constexpr int KBUF = 3;                    // K ring depth
  static constexpr int VBUF = 2;                    // V ring depth
  static constexpr int V_OFF = KBUF * KTILEB;       // K ring, then V ring
  // 64 zero bytes after the rings, read in place of V^T columns past the
  // head (only D = 16 has any); without them two workgroups fit a CU's LDS.
  static constexpr int ZERO_OFF = V_OFF + VBUF * VTILEB;
  static constexpr int LDS_BYTES = ZERO_OFF + (DV < 32 ? 64 : 0);
  // K row r of a tile holds key kperm(r); the V swizzle acts on 16-byte chunks.
  __device__ static constexpr int kperm(int r) {
    const int b = r & 31;
    return (r & ~31) + ((b >> 2) & 1) * 16 + (b >> 3) * 4 + (b & 3);
  }
  __device__ static constexpr int swz_v(int r) { return (4 * (r & 3)) & (VCPR - 1); }
};

template <int D, int DV, int WAVES, bool CAUSAL, bool POS_SCALE, bool F16>
__global__ __launch_bounds__(WAVES * 64, bf16_blocks_per_cu(D > DV ? D : DV)) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int M, int N, int tiles_m, int heads, float c) {
  using C = Bf16Cfg<D, DV, WAVES>;
  constexpr int NT = C::NT, BM = C::BM, BN = C::BN, ROWB = C::ROWB, VROWB = C::VROWB,
                VTILEB = C::VTILEB, CPT = C::CPT, VCPT = C::VCPT, QSTEPS = C::QSTEPS,
                DBLK = C::DBLK,
                NF_QK = C::NF_QK, NF_PV = C::NF_PV;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const TileId tile = tile_order(workgroup_id(), tiles_m, heads, CAUSAL);
  const int bh = tile.bh, tm = tile.tm;

  const size_t q_off = (size_t)bh * M * D;
  const size_t o_off = (size_t)bh * M * DV;
  const uint16_t* qh = q + q_off;
  const uint16_t* kh = k + (size_t)bh * N * D;
  const uint16_t* vh = v + (size_t)bh * N * DV;

  const int q_wg0 = tm * BM;
  const int qw0 = q_wg0 + wave * 32;
  const int qi = qw0 + r32;  // this lane's query row

  // Key tiles the workgroup visits. Under the causal mask a wave may visit
  // up to three tiles that are fully masked for its rows (wave 0 of a
  // 256-row tile: keys 64 .. 255 past the tile's first row); they
  // contribute exact zeros.
  int nt = (N + BN - 1) / BN;
  if (CAUSAL) nt = min(nt, (min(q_wg0 + BM, M) - 1) / BN + 1);

  if (DV < 32 && tid < 16) ((uint32_t*)(smem + C::ZERO_OFF))[tid] = 0u;

  // ---- staging geometry: thread chunk u is chunk ch = tid + u*NT of a
  // tile, i.e. row ch / CPR at (for V swizzled) position ch % CPR. Chunk u
  // sits RPU = NT / CPR rows below chunk 0 with the same column, and kperm
  // and the V swizzle act on the low row bits only (a bit permutation of
  // bits 0-4, and bits 0-3), so every per-chunk offset is chunk 0's plus a
  // compile-time constant: one base register per tensor.
  constexpr int RPU = NT / C::CPR;
  int ch0 = tid;
  if (ch0 >= C::CHUNKS) ch0 = C::CHUNKS - 1;  // surplus threads repeat the last chunk
  const int R0 = ch0 / C::CPR, chp0 = ch0 % C::CPR;
  const int kdst0 = R0 * C::KROWB + chp0 * 16;
  const int k_src0 = 2 * (C::kperm(R0) * D + chp0 * 8);  // bytes from the tile's first key
  auto kdst_off = [&](int u) { return u * RPU * C::KROWB; };
  auto k_src_off = [&](int u) { return 2 * C::kperm(u * RPU) * D; };
  static_assert(CPT == 1 || RPU >= 16, "per-chunk offsets need the row bits of chunk 0 below RPU");
  // The same geometry for the V tile, whose rows have DV elements.
  constexpr int VRPU = NT / C::VCPR;
  int vch0 = tid;
  if (vch0 >= C::VCHUNKS) vch0 = C::VCHUNKS - 1;
  const int VR0 = vch0 / C::VCPR, vchp0 = vch0 % C::VCPR;
  const int dst0 = VR0 * VROWB + vchp0 * 16;
  const int v_src0 = 2 * (VR0 * DV + (vchp0 ^ C::swz_v(VR0)) * 8);
  auto dst_off = [&](int u) { return u * NT * 16; };
  auto v_src_off = [&](int u) { return 2 * u * VRPU * DV; };
  static_assert(VCPT == 1 || VRPU >= 16, "per-chunk offsets need the row bits of chunk 0 below VRPU");
  u32x4_t kst[CPT], vst[VCPT];
  // Tile loads go through buffer descriptors bounded by the head's last key
  // row: chunks past it read as zeros (finite, and masked or multiplied by
  // p = 0), so the tail needs no per-lane clamp and tiles past the end need
  // no guard. Offsets are per-lane constants; the tile base is scalar.
  auto tile_rsrc_w = [&](const uint16_t* head, int j, int width) {
    const int jc = min(j, nt - 1);
    const uint32_t bytes = (uint32_t)(N - jc * BN) * (uint32_t)(2 * width);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (size_t)jc * BN * width), (short)0,
                                             (int)bytes, kBufferRsrcWord3);
  };
  auto tile_rsrc = [&](const uint16_t* head, int j) { return tile_rsrc_w(head, j, D); };
  auto tile_rsrc_v = [&](int j) { return tile_rsrc_w(vh, j, DV); };
  auto load_k = [&](int j) {
    const auto r = tile_rsrc(kh, j);
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      kst[u] = __builtin_amdgcn_raw_buffer_load_b128(r, k_src0 + k_src_off(u), 0, 0);
  };
  auto load_v = [&](int j) {
    const auto r = tile_rsrc_v(j);
#pragma unroll
    for (int u = 0; u < VCPT; ++u)
      vst[u] = __builtin_amdgcn_raw_buffer_load_b128(r, v_src0 + v_src_off(u), 0, 0);
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      *(u32x4_t*)(smem + buf * C::KTILEB + kdst0 + kdst_off(u)) = kst[u];
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int u = 0; u < VCPT; ++u)
      *(u32x4_t*)(smem + C::V_OFF + buf * VTILEB + dst0 + dst_off(u)) = vst[u];
  };

  // ---- per-lane operand read offsets (bytes within a tile)
  // K (A operand of S^T): LDS row kb*32 + r32, chunk (2t+g) ^ swz.
  const int k_rd = r32 * C::KROWB;
  // V^T (A operand of O^T) through ds_read_b64_tr_b16: in 16-lane group G,
  // lane 4*jj + cc supplies row (.. + jj) and d-columns 4*cc .. 4*cc+3 of
  // the group's 16-column slice.
  const int G = lane >> 4, L16 = lane & 15, jj = L16 >> 2, cc = L16 & 3;
  const int gg = G >> 1, nh = G & 1;
  int v_rd[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    const int d0 = b * 32 + nh * 16 + cc * 4;
    if (d0 < DV) {
      const int chunk = d0 >> 3;
      v_rd[b] = (gg * 16 + jj) * VROWB + ((chunk ^ C::swz_v(jj)) << 4) + (cc & 1) * 8;
    } else {
      v_rd[b] = -1;  // d beyond the head: read the zero block
    }
  }

  // Q^T as the B operand: lane holds Q[qi][t*16 + g*8 .. +7].
  using H = Half16<F16>;
  u32x4_t qf[QSTEPS];
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (qi < M) x = *(const u32x4_t*)(qh + (size_t)qi * D + t * 16 + g * 8);
    qf[t] = x;
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
    const unsigned char* kb_base = smem + buf * C::KTILEB + k_rd;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < NF_QK; ++i) {
      const int t = i >> 1, kb = i & 1;
      const u32x4_t fr =
          *(const u32x4_t*)(kb_base + kb * 32 * C::KROWB + (2 * t + g) * 16);
      s[kb] = H::mma(fr, qf[t], s[kb]);
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

  // Exact reference update for a prepared score tile (prologue and the
  // rare overflow path): m becomes max(m, row max); returns the factor for
  // O and l.
  auto exact_ref = [&](const f32x16_t* s) -> float {
    float mx = __builtin_fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2)
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[kb][i], s[kb][i + 1]));
    mx = half_pair_max(mx);
    const float m_new = __builtin_fmaxf(m_run, mx * cc_scale);
    const float m_new_sub = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_sub - m_new_sub);
    m_run = m_new;
    m_sub = m_new_sub;
    return alpha;
  };

  // Probabilities of one 32-key half of a tile: bf16 P (B-operand layout)
  // and their row sum (of the rounded values, via a dot2 with 1s).
  auto tile_exp = [&](const f32x16_t& s, u32x4_t* p) -> float {
    // The row sum is accumulated from each freshly rounded pair (not from
    // elements extracted back out of the packed vector).
    float rs = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t * 8 + 2 * e], cc_scale, -m_sub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t * 8 + 2 * e + 1], cc_scale, -m_sub));
        w[e] = H::round_sum(p0, p1, rs);
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

  // K fragment i of the S^T product (key block i & 1, d-step i >> 1) and V^T
  // fragment i of the O^T product (O block i % DBLK, key step i / DBLK).
  typedef __attribute__((ext_vector_type(8))) short s16x8_t;
  auto k_frag = [&](const unsigned char* kb_base, int i) -> u32x4_t {
    const int t = i >> 1, kb = i & 1;
    return *(const u32x4_t*)(kb_base + kb * 32 * C::KROWB + (2 * t + g) * 16);
  };
  auto v_frag = [&](const unsigned char* vb_base, int i) -> s16x8_t {
    const unsigned char* zero = smem + C::ZERO_OFF;
    const int b = i % DBLK, kt = i / DBLK, kb = kt >> 1, t = kt & 1;
    const int row_off = (kb * 32 + t * 8) * VROWB;
    const unsigned char* a0 = v_rd[b] < 0 ? zero : vb_base + v_rd[b] + row_off;
    const unsigned char* a1 = v_rd[b] < 0 ? zero : vb_base + v_rd[b] + row_off + 4 * VROWB;
    const s16x4_t lo = lds_read_tr16(a0);
    const s16x4_t hi = lds_read_tr16(a1);
    return (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // Operand fragments are read KPF / VPF chunks ahead of their MFMA.
  constexpr int KPF = 3, VPF = 3;

  // First half of an iteration, as NF_QK fenced chunks: each issues the K
  // fragment read KPF chunks ahead, one S(j+1) MFMA, a share of the
  // exponentials of S(j) (two at a time: fma, exp2, round to bf16, row sum)
  // and, in the first chunks, the global loads of K(j+2). The fences
  // (sched_barrier) fix the chunk order; inside a chunk the scheduler is
  // free. Returns the lane's partial row sum of P(j).
  auto region_a = [&](int j, const f32x16_t* sc, f32x16_t* sn, u32x4_t (*p)[2])
                      __attribute__((always_inline)) -> float {
    constexpr int PPC = 16 / NF_QK;  // exponential pairs per chunk
    const unsigned char* kb_base = smem + ((j + 1) % C::KBUF) * C::KTILEB + k_rd;
    const auto rk = tile_rsrc(kh, j + 2);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kb][i] = 0.0f;
    u32x4_t fr[KPF + 1];
#pragma unroll
    for (int i = 0; i < KPF && i < NF_QK; ++i) fr[i] = k_frag(kb_base, i);
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < NF_QK; ++i) {
      if (i + KPF < NF_QK) fr[(i + KPF) % (KPF + 1)] = k_frag(kb_base, i + KPF);
      if (i < CPT) kst[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_src0 + k_src_off(i), 0, 0);
#pragma unroll
      for (int q = 0; q < PPC; ++q) {
        const int pr = i * PPC + q, kb = pr >> 3, t = (pr >> 2) & 1, e = pr & 3;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][t * 8 + 2 * e], cc_scale, -m_sub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][t * 8 + 2 * e + 1], cc_scale, -m_sub));
        p[kb][t][e] = H::round_sum(p0, p1, rs);
      }
      // the vector work of the chunk is issued before the MFMA's operand
      // wait, so an LDS stall does not hold it back
      __builtin_amdgcn_sched_barrier(0);
      sn[i & 1] = H::mma(fr[i % (KPF + 1)], qf[i >> 1], sn[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    return rs;
  };

  // Second half, as NF_PV fenced chunks: the V^T fragment reads VPF chunks
  // ahead, one O MFMA each and, with a next tile, the loads of V(j+1) (first
  // chunks). With 8 waves the LDS writes of K(j+2) (from the middle) and
  // V(j+1) (last quarter) go between these products too, rather than all at
  // the end of a half, where they hold up the barrier (about 1% at D = 128;
  // the 4-wave kernels keep them at the ends: their register budget is
  // smaller). Both slots are free: their last reads ended before the
  // previous barrier.
  constexpr bool STG_IN_B = WAVES == 8;
  constexpr int KST0 = NF_PV / 2, KSTEP = NF_PV / (2 * CPT) > 0 ? NF_PV / (2 * CPT) : 1;
  constexpr int VST0 = 3 * NF_PV / 4, VSTEP = NF_PV / (4 * VCPT) > 0 ? NF_PV / (4 * VCPT) : 1;
  static_assert(KST0 + (CPT - 1) * KSTEP < NF_PV && VST0 + (VCPT - 1) * VSTEP < NF_PV &&
                    VST0 >= VCPT,
                "staging writes fit the chunks, after the V loads");
  auto region_b = [&](int j, const u32x4_t (*p)[2], bool has_next) __attribute__((always_inline)) {
    const unsigned char* vb_base = smem + C::V_OFF + (j & 1) * VTILEB;
    const auto rv = tile_rsrc_v(j + 1);
    s16x8_t fr[VPF + 1];
#pragma unroll
    for (int i = 0; i < VPF && i < NF_PV; ++i) fr[i] = v_frag(vb_base, i);
#pragma unroll
    for (int i = 0; i < NF_PV; ++i) {
      if (i + VPF < NF_PV) fr[(i + VPF) % (VPF + 1)] = v_frag(vb_base, i + VPF);
      if (has_next && i < VCPT)
        vst[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_src0 + v_src_off(i), 0, 0);
      if (STG_IN_B && has_next && i >= KST0 && (i - KST0) % KSTEP == 0 && (i - KST0) / KSTEP < CPT) {
        const int u = (i - KST0) / KSTEP;
        *(u32x4_t*)(smem + ((j + 2) % C::KBUF) * C::KTILEB + kdst0 + kdst_off(u)) = kst[u];
      }
      if (STG_IN_B && has_next && i >= VST0 && (i - VST0) % VSTEP == 0 && (i - VST0) / VSTEP < VCPT) {
        const int u = (i - VST0) / VSTEP;
        *(u32x4_t*)(smem + C::V_OFF + ((j + 1) & 1) * VTILEB + dst0 + dst_off(u)) = vst[u];
      }
      const int b = i % DBLK, kt = i / DBLK;
      acc[b] = H::mma(__builtin_bit_cast(u32x4_t, fr[i % (VPF + 1)]), p[kt >> 1][kt & 1], acc[b]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (has_next && NF_PV < VCPT) load_v(j + 1);  // (never: NF_PV >= VCPT for every DV)
  };

  // Row-sum bound that sends a tile to the exact path: a lane's partial sum
  // of p over its 32 keys; any single p above 2^16 / 32 trips it.
  constexpr float kRowSumLimit = 65536.0f;

  // Iteration j: P(j) from S(j) (against the current reference) and
  // O += V(j)^T P(j)^T; with a next tile, S(j+1) = K(j+1) Q^T alongside, its
  // scale and mask, and the staging of K(j+2), V(j+1) into the ring slots
  // freed one iteration ago.
  auto iter = [&](int j, f32x16_t* sc, f32x16_t* sn, bool has_next) __attribute__((always_inline)) {
    u32x4_t p[2][2];
    float rs;
    if (has_next) {
      rs = region_a(j, sc, sn, p);
      if constexpr (!STG_IN_B) store_k((j + 2) % C::KBUF);
    } else {
      rs = tile_exp(sc[0], p[0]) + tile_exp(sc[1], p[1]);
    }
    if (wave_any(rs > kRowSumLimit)) {
      // Some score rose far above the reference: redo this tile exactly
      // (O holds tiles < j; K(j) is still in its ring slot).
      keep_branch();
      qk(j % C::KBUF, sc);
      scale_tile(sc);
      if (needs_mask(j)) mask_tile(sc, j);
      const float alpha = exact_ref(sc);
      rescale(alpha);
      l_run *= alpha;
      rs = tile_exp(sc[0], p[0]) + tile_exp(sc[1], p[1]);
    }
    l_run += rs;
    region_b(j, p, has_next);
    if (has_next) {
      if constexpr (!STG_IN_B) store_v((j + 1) & 1);
      scale_tile(sn);
      if (needs_mask(j + 1)) {
        keep_branch();
        mask_tile(sn, j + 1);
      }
      __syncthreads();
    }
  };

  // ---- prologue: K(0), K(1), V(0) -> LDS; S(0) and its exact reference.
  load_k(0);
  store_k(0);
  load_k(1);
  store_k(1);
  load_v(0);
  store_v(0);
  __syncthreads();  // K(0), K(1), V(0) and the zero block visible
  qk(0, s_a);
  scale_tile(s_a);
  if (needs_mask(0)) {
    keep_branch();
    mask_tile(s_a, 0);
  }
  exact_ref(s_a);  // O and l are still zero: nothing to rescale

  // Iteration j keeps S(j) in s_a (j even) or s_b (j odd).
  int j = 0;
  for (; j + 2 < nt; j += 2) {
    // lgkmcnt(0), free here (LDS is drained: the previous iteration ended in
    // a barrier, the prologue consumed its reads): it tells the
    // wait-count pass that no scalar load from before the loop is still in
    // flight, so the first K fragment wait of the iteration counts only its
    // own LDS read instead of all of them.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    iter(j, s_a, s_b, true);
    iter(j + 1, s_b, s_a, true);
  }
  if (j + 1 < nt) {
    iter(j, s_a, s_b, true);
    iter(j + 1, s_b, s_a, false);
  } else {
    iter(j, s_a, s_b, false);
  }

  const float l_tot = half_pair_sum(l_run);
  if (qi >= M) return;
  const float inv = 1.0f / l_tot;
  uint16_t* orow = o + o_off + (size_t)qi * DV;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = b * 32 + i4 * 8 + g * 4;
      if (d0 < DV) {
        u32x2_t st;
        st[0] = H::pack(acc[b][i4 * 4 + 0] * inv, acc[b][i4 * 4 + 1] * inv);
        st[1] = H::pack(acc[b][i4 * 4 + 2] * inv, acc[b][i4 * 4 + 3] * inv);
        *(u32x2_t*)(orow + d0) = st;
      }
    }
  if (g == 0) lse[(size_t)bh * M + qi] = (m_run + log2f(l_tot)) * kLn2;
}

template <int D, int DV, bool CAUSAL, bool POS, bool F16>
static hipError_t launch_16_d(const LaunchArgs& a) {
  constexpr int WAVES = bf16_waves(D > DV ? D : DV);
  constexpr int BM = WAVES * 32;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const dim3 grid((unsigned)(tiles_m * a.BH));
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, DV, WAVES, CAUSAL, POS, F16>), grid,
                     dim3(WAVES * 64), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, (int)a.M, (int)a.N, tiles_m, (int)a.BH, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, int DV, bool F16>
static hipError_t launch_16_dispatch(const LaunchArgs& a) {
  const bool pos = a.scale > 0.0f;
  if (a.causal)
    return pos ? launch_16_d<D, DV, true, true, F16>(a) : launch_16_d<D, DV, true, false, F16>(a);
  return pos ? launch_16_d<D, DV, false, true, F16>(a) : launch_16_d<D, DV, false, false, F16>(a);
}

template <int D, bool F16>
static hipError_t launch_16_dv(const LaunchArgs& a) {
  switch (a.Dv) {
    case 16: return launch_16_dispatch<D, 16, F16>(a);
    case 32: return launch_16_dispatch<D, 32, F16>(a);
    case 64: return launch_16_dispatch<D, 64, F16>(a);
    case 128: return launch_16_dispatch<D, 128, F16>(a);
    default: return hipErrorInvalidValue;
  }
}

// Head dims D and Dv each in {16, 32, 64, 128} (Dv = D unless v has a head
// dim of its own).
template <bool F16>
static hipError_t launch_main_16(const LaunchArgs& a) {
  switch (a.D) {
    case 16: return launch_16_dv<16, F16>(a);
    case 32: return launch_16_dv<32, F16>(a);
    case 64: return launch_16_dv<64, F16>(a);
    case 128: return launch_16_dv<128, F16>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_main_bf16(const LaunchArgs& a) { return launch_main_16<false>(a); }
hipError_t launch_main_f16(const LaunchArgs& a) { return launch_main_16<true>(a); }

// (the smallest tile of any head dim: grid-size checks stay conservative)
int main_bf16_tile_rows() { return bf16_waves(16) * 32; }

}  // namespace mi355
