// attn_bwd_bf16.hip -- FlashAttention-2 backward for 16-bit (bf16, fp16)
// inputs on gfx950.
//
// The gradient of O = softmax(scale Q K^T [+ causal mask]) V for an upstream
// dO, in the tiled form of "Blackwell Attention Example" (backward kernel
// implementation section): the probabilities are recomputed tile by tile from
// the saved logsumexp (P = exp2(scale log2(e) q.k - log2(e) L)), the row term
// is delta_i = rowsum(O_i * dO_i) (its preprocess kernel), and
//     dV += P^T dO,   dP = dO V^T,   dS = P (dP - delta),
//     dK += dS^T Q (times scale),    dQ += dS K (times scale).
// P and dS are rounded to the input type before their products, which
// accumulate in fp32, as on that page.
//
// gfx950 mapping (not the page's design, which accumulates dQ with atomics
// from the key-tile loop): two kernels, so that every output element has one
// writer and the result is run-to-run deterministic.
//  * attn_bwd_dq_kernel: one workgroup = 8 waves = 256 query rows of one
//    (batch, head); loops over key/value tiles of 64 rows. It first forms
//    delta for its rows (O and dO rows in registers) and writes it out for the
//    second kernel. Per tile: S^T = K Q^T and dP^T = V dO^T (K, V rows from
//    LDS, Q^T, dO^T in registers), P^T and dS^T in registers, then
//    dQ^T += K^T dS^T with K^T read from LDS through ds_read_b64_tr_b16.
//  * attn_bwd_dkdv_kernel: one workgroup = 8 waves = 256 key rows (two
//    waves per SIMD); loops over query tiles of 64 rows. Per 32-query half:
//    S = Q K^T and dP = dO V^T (Q, dO rows from LDS, K^T in registers, V^T
//    from the workgroup's V rows kept in LDS for the whole kernel), P and dS,
//    then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read transposed
//    from LDS.
//  * For D <= 64 both kernels use 4-wave workgroups (128 rows), three per CU,
//    so that three waves share each SIMD.
//  * All products are v_mfma_f32_32x32x16_bf16. Every staged tile is stored
//    with its rows permuted so that the 16 accumulator registers of a lane
//    are 16 consecutive rows of the tile: rounded to bf16 those registers are
//    directly the B operand of the next product. Tiles are XOR-swizzled at
//    16-byte granularity.
//  * Tiles go from HBM straight into LDS (buffer loads with the lds flag,
//    bounded: rows past the head read as zeros), double-buffered, one barrier
//    per tile. Nothing in the loops waits for the next tile's loads before
//    the tile's last product: the loads are issued from inline asm (see
//    lds_dma16), masks are branches, and no spill reload comes before the
//    tile's last product.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(8))) short s16x8_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ s16x4_t lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4_t __attribute__((address_space(3)))*)(lds_u8*)p);
}

// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle): loads past num_records return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Waves per workgroup (32 rows each): 8 for D = 128 (two per SIMD); 4 for
// smaller heads, three workgroups per CU (three waves per SIMD).
__host__ __device__ constexpr int bwd_waves(int D) { return D <= 64 ? 4 : 8; }
__host__ __device__ constexpr int bwd_blocks_per_cu(int D) { return D <= 64 ? 3 : 1; }
constexpr int kTileRows = 64;  // rows of a staged K/V (or Q/dO) tile

// A staged 64-row tile of a [rows, D] bf16 tensor in LDS.
// LDS row R holds source row perm(R); within a row, 16-byte chunk position p
// holds source chunk p ^ swz(R). perm is a bit permutation of the low five
// row bits: after a 32x32 MFMA whose A operand reads rows blk*32 + (lane%32),
// accumulator register r of lane l belongs to source row
// blk*32 + 16*(l/32) + r.
template <int D, int ROWS = kTileRows>
struct Tile {
  static constexpr int ROWB = 2 * D;                 // bytes per row
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int CHUNKS = BYTES / 16;
  static constexpr int QSTEPS = D / 16;              // 16-wide d steps
  static constexpr int DBLK = D / 32;                // 32-wide d blocks
  __device__ static constexpr int perm(int r) {
    const int b = r & 31;
    return (r & ~31) + ((b >> 2) & 1) * 16 + (b >> 3) * 4 + (b & 3);
  }
  // Row reads touch 16 consecutive rows at one logical chunk, transposed
  // reads 4 consecutive rows (from a multiple of 4) at 4 consecutive chunks;
  // with 16 chunks per row, rotating the low row bits (4 (r & 3) + (r >> 2) & 3)
  // gives both patterns 16 distinct bank positions. Narrower rows keep the
  // plain r & (CPR - 1).
  __device__ static constexpr int swz(int r) {
    return CPR == 16 ? ((4 * (r & 3)) | ((r >> 2) & 3)) : (r & 15) & (CPR - 1);
  }
};

// Staging of one tile by NT threads: thread chunk u is LDS chunk
// ch = tid + u*NT (row ch / CPR, position ch % CPR).
template <int D, int NT, int ROWS = kTileRows>
struct Stager {
  using T = Tile<D, ROWS>;
  static constexpr int CPT = (T::CHUNKS + NT - 1) / NT;
  int src[CPT];  // byte offset of the source chunk from the tile's first row
  int dst[CPT];  // byte offset in the LDS tile (-1: no chunk for this thread)
  // Chunk u lies NT / CPR rows (a multiple of 32) below chunk 0 with the same
  // position: perm and swz act on the low five row bits only, so its source
  // is chunk 0's plus u * SRC_STEP bytes.
  static constexpr int SRC_STEP = (NT / T::CPR) * T::ROWB;
  static_assert(CPT == 1 || (NT / T::CPR) % 32 == 0, "chunk offsets are chunk 0's plus a constant");
  __device__ void init(int tid) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ch = tid + u * NT;
      if (ch < T::CHUNKS) {
        const int R = ch / T::CPR, p = ch % T::CPR;
        src[u] = T::perm(R) * T::ROWB + ((p ^ T::swz(R)) << 4);
        dst[u] = ch * 16;
      } else {
        src[u] = 0;
        dst[u] = -1;
      }
    }
  }
};

// Buffer descriptor for rows [row0, rows) of a [rows, D] bf16 head: reads
// past the last row return zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* head, int row0,
                                                            int rows) {
  const int left = rows - row0;
  const uint32_t bytes = left > 0 ? (uint32_t)left * (uint32_t)(2 * D) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (size_t)row0 * D), (short)0,
                                           (int)bytes, kBufferRsrcWord3);
}
// The same descriptor as four words, for the loads into LDS (lds_dma16).
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
template <int D>
__device__ __forceinline__ i32x4_t rows_desc(const uint16_t* head, int row0, int rows) {
  const int left = rows - row0;
  const uint32_t bytes = left > 0 ? (uint32_t)left * (uint32_t)(2 * D) : 0u;
  const uint64_t base = (uint64_t)(head + (size_t)row0 * D);
  return (i32x4_t){(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), (int)bytes,
                   kBufferRsrcWord3};
}

// Per-lane LDS offsets of the two fragment kinds read from a Tile.
template <int D>
struct FragAddr {
  using T = Tile<D>;
  int row;               // row fragment: row (lane%32), chunk base
  int sw;                // swz of that row
  int tr_lo[T::DBLK];    // transposed fragment, rows +0..3 of each 8
  int tr_hi[T::DBLK];    // transposed fragment, rows +4..7
  __device__ void init(int lane) {
    const int r32 = lane & 31;
    row = r32 * T::ROWB;
    sw = T::swz(r32);
    // ds_read_b64_tr_b16: in 16-lane group G, lane 4*jj + cc addresses row
    // jj of a 4-row block and columns 4*cc .. 4*cc+3 of the group's 16-column
    // slice; output lane i then holds column i of the four rows. Lanes
    // l < 32 supply contraction rows 0..7 of a 16-row step, lanes >= 32 rows
    // 8..15; in the permuted tile the source rows 16*gg + 8*t + c (c < 4) of
    // a 32-row block sit at LDS rows 16*t + 4*gg + c, and rows
    // 16*gg + 8*t + 4 + c at 16*t + 8 + 4*gg + c.
    const int G = lane >> 4, L16 = lane & 15, jj = L16 >> 2, cc = L16 & 3;
    const int gg = G >> 1, nh = G & 1;
#pragma unroll
    for (int b = 0; b < T::DBLK; ++b) {
      const int chunk = 4 * b + 2 * nh + (cc >> 1);
      const int r_lo = 4 * gg + jj, r_hi = 8 + 4 * gg + jj;
      tr_lo[b] = r_lo * T::ROWB + ((chunk ^ T::swz(r_lo)) << 4) + (cc & 1) * 8;
      tr_hi[b] = r_hi * T::ROWB + ((chunk ^ T::swz(r_hi)) << 4) + (cc & 1) * 8;
    }
  }
  // A operand: rows blk*32 + (lane%32), d = 16*t + 8*(lane/32) .. +7.
  __device__ bf16x8_t row_frag(const unsigned char* tile, int blk, int t, int g) const {
    const u32x4_t x = *(const u32x4_t*)(tile + blk * 32 * T::ROWB + row +
                                        (((2 * t + g) ^ sw) << 4));
    return __builtin_bit_cast(bf16x8_t, x);
  }
  // A operand of a transposed product: d = 32*b + (lane%32) by the 16
  // source rows blk*32 + 16*(lane/32) + 8*t .. +7 (matching accumulator
  // registers 8t .. 8t+7 of the permuted rows).
  __device__ bf16x8_t tr_frag(const unsigned char* tile, int b, int blk, int t) const {
    const unsigned char* base = tile + (blk * 32 + 16 * t) * T::ROWB;
    const s16x4_t lo = lds_read_tr16(base + tr_lo[b]);
    const s16x4_t hi = lds_read_tr16(base + tr_hi[b]);
    const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// Row x of a [rows, D] bf16 head as the B operand of QSTEPS products:
// step t holds d = 16*t + 8*g .. +7 (zeros past the last row).
template <int D>
__device__ __forceinline__ void load_b_rows(const uint16_t* head, int x, int rows, int g,
                                            bf16x8_t* f) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (x < rows) w = *(const u32x4_t*)(head + (size_t)x * D + t * 16 + g * 8);
    f[t] = __builtin_bit_cast(bf16x8_t, w);
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// An empty volatile asm statement: a branch body containing it is not
// if-converted into selects executed on every tile.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// 16 bytes per lane from a buffer straight into LDS: lane l writes
// lds_wave_base + 16*l (lds_wave_base must be wave-uniform). Written as
// inline asm: the compiler, which cannot tell the two ring slots apart, would
// otherwise make every later LDS read wait for these loads, i.e. wait in the
// middle of each tile for the next tile's data. The kernels order them
// themselves: a slot is loaded only after the barrier that ends its last
// reads, and every load is waited for (wait_vmem) before the barrier that
// publishes its slot. The instruction has no result register; its address
// operands are read when it issues. soffset (wave-uniform) is added to the
// per-lane voffset.
__device__ __forceinline__ void lds_dma16(i32x4_t desc, unsigned char* lds_wave_base, int voffset,
                                          int soffset) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(desc), "s"(soffset)
               : "m0");
}

// Wait for this wave's outstanding vector-memory operations (including
// buffer loads into LDS) to complete.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Store 16 accumulator registers of a transposed (d by row) product: lane
// holds d = 32*b + 8*i4 + 4*g + (0..3) of its row, times `mul`, rounded to
// the 16-bit input type.
template <int D, bool F16>
__device__ __forceinline__ void store_rowT(uint16_t* row, const f32x16_t* acc, int g,
                                           float mul) {
  using H = Half16<F16>;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = b * 32 + i4 * 8 + g * 4;
      u32x2_t st;
      st[0] = H::pack(acc[b][i4 * 4 + 0] * mul, acc[b][i4 * 4 + 1] * mul);
      st[1] = H::pack(acc[b][i4 * 4 + 2] * mul, acc[b][i4 * 4 + 3] * mul);
      *(u32x2_t*)(row + d0) = st;
    }
}

}  // namespace

// ---------------------------------------------------------------- dQ kernel
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(bwd_waves(D) * 64, bwd_blocks_per_cu(D)) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ dq, float* __restrict__ delta, int M, int N, int tiles_m,
    int heads, float c, float scale) {
  using T = Tile<D>;
  using H = Half16<F16>;
  constexpr int NT = bwd_waves(D) * 64, BM = bwd_waves(D) * 32, BN = kTileRows;
  constexpr int QSTEPS = T::QSTEPS, DBLK = T::DBLK;
  // K ring (2), then V ring (2).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * T::BYTES];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, g = lane >> 5;

  const TileId tile = tile_order(workgroup_id(), tiles_m, heads, CAUSAL);
  const int bh = tile.bh;
  const int q_wg0 = tile.tm * BM;
  const int qw0 = q_wg0 + wave * 32;
  const int qi = qw0 + r32;

  const size_t q_off = (size_t)bh * M * D, kv_off = (size_t)bh * N * D;
  const uint16_t* kh = k + kv_off;
  const uint16_t* vh = v + kv_off;

  int nt = (N + BN - 1) / BN;
  if (CAUSAL) nt = min(nt, (min(q_wg0 + BM, M) - 1) / BN + 1);

  Stager<D, NT> st;
  st.init(tid);
  FragAddr<D> fa;
  fa.init(lane);
  // K and V tiles go from HBM straight into LDS (buffer loads with the lds
  // flag; lane l of a wave writes the wave's base + 16 l).
  auto load = [&](int j, int buf) {
    const i32x4_t rk = rows_desc<D>(kh, j * BN, N);
    const i32x4_t rv = rows_desc<D>(vh, j * BN, N);
#pragma unroll
    for (int u = 0; u < Stager<D, NT>::CPT; ++u) {
      const int wbase = (wave * 64 + u * NT) * 16;  // wave-uniform
      if (wbase < T::BYTES) {
        lds_dma16(rk, smem + buf * T::BYTES + wbase, st.src[0], u * Stager<D, NT>::SRC_STEP);
        lds_dma16(rv, smem + (2 + buf) * T::BYTES + wbase, st.src[0], u * Stager<D, NT>::SRC_STEP);
      }
    }
  };

  // Q^T and dO^T as B operands; delta_i = O_i . dO_i from the same layout.
  bf16x8_t qf[QSTEPS], gf[QSTEPS];
  load_b_rows<D>(q + q_off, qi, M, g, qf);
  load_b_rows<D>(dout + q_off, qi, M, g, gf);
  float dl;
  {
    bf16x8_t of[QSTEPS];
    load_b_rows<D>(o + q_off, qi, M, g, of);
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      const u32x4_t ow = __builtin_bit_cast(u32x4_t, of[t]);
      const u32x4_t gw = __builtin_bit_cast(u32x4_t, gf[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(H::lo(ow[e]), H::lo(gw[e]), part);
        part = fmaf(H::hi(ow[e]), H::hi(gw[e]), part);
      }
    }
    dl = half_pair_sum(part);
  }
  float l2 = 0.0f;
  if (qi < M) {
    l2 = lse[(size_t)bh * M + qi] * kLog2e;
    if (g == 0) delta[(size_t)bh * M + qi] = dl;
  }

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;

  if (nt > 0) load(0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < nt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nt) load(j + 1, buf ^ 1);
    const unsigned char* kt = smem + buf * T::BYTES;
    const unsigned char* vt = smem + (2 + buf) * T::BYTES;

    // S^T = K Q^T, dP^T = V dO^T: key block kb, lane's keys 16g + r. Fenced
    // chunks of one MFMA, operands read PF chunks ahead; chunk i is key
    // block (i >> 1) & 1 of d-step i >> 2, S (i even) or dP (i odd).
    constexpr int PF = 2, NA = 4 * QSTEPS, NC = 4 * DBLK;
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = 0.0f;
        dp[kb][i] = 0.0f;
      }
    {
      bf16x8_t fr[PF + 1];
      auto rd = [&](int i) { return fa.row_frag((i & 1) ? vt : kt, (i >> 1) & 1, i >> 2, g); };
#pragma unroll
      for (int i = 0; i < PF; ++i) fr[i] = rd(i);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + PF < NA) fr[(i + PF) % (PF + 1)] = rd(i + PF);
        const int kb = (i >> 1) & 1, t = i >> 2;
        __builtin_amdgcn_sched_barrier(0);
        if (i & 1) dp[kb] = H::mma(fr[i % (PF + 1)], gf[t], dp[kb]);
        else s[kb] = H::mma(fr[i % (PF + 1)], qf[t], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // P^T = exp2(c s - log2e L), dS^T = P^T (dP^T - delta); masked keys give
    // P = 0. Rounded to bf16: the B operand of dQ^T += K^T dS^T.
    const int key0 = j * BN;
    const bool masked = (key0 + BN > N) || (CAUSAL && key0 + BN - 1 > qw0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -l2));
    if (masked) {
      // only tiles that cross the diagonal or the last key: a real branch
      // (not per-element selects on every tile)
      keep_branch();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + g * 16 + i;
          if (key >= N || (CAUSAL && key > qi)) s[kb][i] = 0.0f;
        }
    }
    u32x4_t ds[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = t * 8 + 2 * e;
          ds[kb][t][e] = H::pack(s[kb][i0] * (dp[kb][i0] - dl), s[kb][i0 + 1] * (dp[kb][i0 + 1] - dl));
        }

    // dQ^T += K^T dS^T over the tile's four 16-key steps (chunk i: d block
    // i % DBLK of key step i / DBLK).
    {
      bf16x8_t fr[PF + 1];
      auto rd = [&](int i) {
        const int kt_ = i / DBLK;
        return fa.tr_frag(kt, i % DBLK, kt_ >> 1, kt_ & 1);
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) fr[i] = rd(i);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        if (i + PF < NC) fr[(i + PF) % (PF + 1)] = rd(i + PF);
        const int b = i % DBLK, kt_ = i / DBLK;
        __builtin_amdgcn_sched_barrier(0);
        acc[b] = H::mma(fr[i % (PF + 1)],
                                    __builtin_bit_cast(bf16x8_t, ds[kt_ >> 1][kt_ & 1]), acc[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    wait_vmem();
    __syncthreads();
  }

  if (qi < M) store_rowT<D, F16>(dq + q_off + (size_t)qi * D, acc, g, scale);
}

// ------------------------------------------------------------ dK/dV kernel
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(bwd_waves(D) * 64, bwd_blocks_per_cu(D)) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const float* __restrict__ delta, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int M, int N, int tiles_n,
    int heads, float c, float scale) {
  using T = Tile<D>;
  using H = Half16<F16>;
  constexpr int NT = bwd_waves(D) * 64, BNK = bwd_waves(D) * 32, BQ = kTileRows;
  static_assert(BQ == 64, "one wave loads the 64 per-row statistics of a tile");
  constexpr int QSTEPS = T::QSTEPS, DBLK = T::DBLK;
  // Q ring (2), dO ring (2), then per-row log2e*L and delta (2 x 2 x 64).
  // Then the workgroup's V rows (row-major, swizzled, unpermuted), kept for
  // the whole kernel: V^T is read from there as the B operand of dP.
  constexpr int STAT_OFF = 4 * T::BYTES;
  constexpr int V_OFF = STAT_OFF + 4 * BQ * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[V_OFF + BNK * T::ROWB];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, g = lane >> 5;

  // Under the causal mask the first key tiles see the most query rows: run
  // them first (tile_order runs the last tile index first).
  const TileId tile = tile_order(workgroup_id(), tiles_n, heads, CAUSAL);
  const int bh = tile.bh;
  const int tn = CAUSAL ? tiles_n - 1 - tile.tm : tile.tm;
  const int k_wg0 = tn * BNK;
  const int kw0 = k_wg0 + wave * 32;
  const int kj = kw0 + r32;  // this lane's key row

  const size_t q_off = (size_t)bh * M * D, kv_off = (size_t)bh * N * D;
  const uint16_t* qh = q + q_off;
  const uint16_t* gh = dout + q_off;
  const float* lh = lse + (size_t)bh * M;
  const float* dh = delta + (size_t)bh * M;

  // Query tiles that can see a key of this workgroup.
  const int t_end = (M + BQ - 1) / BQ;
  const int t_beg = CAUSAL ? min(k_wg0 / BQ, t_end) : 0;

  Stager<D, NT> st;
  st.init(tid);
  FragAddr<D> fa;
  fa.init(lane);
  constexpr int CPT = Stager<D, NT>::CPT;
  float stat = 0.0f;  // threads 0..63: L of a row; 64..127: delta (as loaded)
  // Q and dO tiles go from HBM straight into LDS (buffer loads with the lds
  // flag: lane l of a wave writes 16 bytes at the wave's base + 16 l, which
  // is the staging order ch = tid + u*NT), so they need no registers; the
  // per-row statistics pass through one register.
  auto load = [&](int j, int buf) {
    const i32x4_t rq = rows_desc<D>(qh, j * BQ, M);
    const i32x4_t rg = rows_desc<D>(gh, j * BQ, M);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int wbase = (wave * 64 + u * NT) * 16;  // wave-uniform
      if (wbase < T::BYTES) {
        lds_dma16(rq, smem + buf * T::BYTES + wbase, st.src[0], u * Stager<D, NT>::SRC_STEP);
        lds_dma16(rg, smem + (2 + buf) * T::BYTES + wbase, st.src[0], u * Stager<D, NT>::SRC_STEP);
      }
    }
    if (wave < 2) {  // wave 0: log2e*L, wave 1: delta of the tile's rows
      const int r = j * BQ + lane;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(wave == 0 ? lh : dh), (short)0,
                                                        M * 4, kBufferRsrcWord3);
      // used only in store(), after the tile's products, so that the wait
      // for it (which also waits for the tile loads) stays there
      stat = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, r * 4, 0, 0));
    }
  };
  // Make this wave's tile loads and its statistic visible to the workgroup
  // (the caller's barrier follows).
  auto store = [&](int buf, int j) {
    wait_vmem();
    if (wave < 2) {
      // Rows past the end: P = exp2(-inf) = 0 and delta = 0.
      const float x = wave == 0 ? (j * BQ + lane < M ? stat * kLog2e : INFINITY) : stat;
      ((float*)(smem + STAT_OFF))[buf * 2 * BQ + tid] = x;
    }
  };

  // K^T as the B operand (lane's key row) in registers; V rows
  // k_wg0 .. k_wg0 + BNK - 1 (zeros past the head) into LDS.
  bf16x8_t kf[QSTEPS];
  load_b_rows<D>(k + kv_off, kj, N, g, kf);
  {
    constexpr int VCH = BNK * T::CPR;
    static_assert(VCH % NT == 0, "V rows split evenly over the threads");
    const auto rv = rows_rsrc<D>(v + kv_off, k_wg0, N);
#pragma unroll
    for (int u = 0; u < VCH / NT; ++u) {
      const int ch = tid + u * NT;
      const int R = ch / T::CPR, pp = ch % T::CPR;
      *(u32x4_t*)(smem + V_OFF + ch * 16) = __builtin_amdgcn_raw_buffer_load_b128(
          rv, R * T::ROWB + ((pp ^ T::swz(R)) << 4), 0, 0);
    }
  }
  const unsigned char* v_row = smem + V_OFF + (wave * 32 + r32) * T::ROWB;

  f32x16_t dka[DBLK], dva[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[b][i] = 0.0f;
      dva[b][i] = 0.0f;
    }

  // One 64-query tile, block by block (32 queries): S = Q K^T and
  // dP = dO V^T, then P and dS, then dV^T += dO^T P and dK^T += Q^T dS. The
  // second wave of the SIMD runs beside it. `mask` (tile-uniform) applies the
  // causal diagonal.
  auto tile_body = [&](const unsigned char* qt, const unsigned char* gt, const float* lt,
                       int q0, bool mask) __attribute__((always_inline)) {
    const float* dt = lt + BQ;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.0f;
        dp[i] = 0.0f;
      }
      // fenced chunks, one MFMA each, operands read PF chunks ahead:
      // chunk i is S step i/2 (even: Q rows, K^T) or dP step i/2 (odd: dO
      // rows, V^T)
      {
        // (one chunk ahead at D = 128: two would exceed the register budget,
        // and the spill reloads inside the loop would each wait for the next
        // tile's loads)
        constexpr int PF = D == 128 ? 1 : 2, NA = 2 * QSTEPS;
        bf16x8_t fa_[PF + 1], fb_[PF + 1];
        auto rd = [&](int i, bf16x8_t& x, bf16x8_t& y) {
          x = fa.row_frag((i & 1) ? gt : qt, qb, i >> 1, g);
          if (i & 1) {
            const u32x4_t vw = *(const u32x4_t*)(v_row + (((2 * (i >> 1) + g) ^ fa.sw) << 4));
            y = __builtin_bit_cast(bf16x8_t, vw);
          } else {
            y = kf[i >> 1];
          }
        };
#pragma unroll
        for (int i = 0; i < PF; ++i) rd(i, fa_[i], fb_[i]);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          if (i + PF < NA) rd(i + PF, fa_[(i + PF) % (PF + 1)], fb_[(i + PF) % (PF + 1)]);
          __builtin_amdgcn_sched_barrier(0);
          if (i & 1) dp = H::mma(fa_[i % (PF + 1)], fb_[i % (PF + 1)], dp);
          else s = H::mma(fa_[i % (PF + 1)], fb_[i % (PF + 1)], s);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int qr0 = qb * 32 + 16 * g;  // lane's queries q0 + qr0 + r, r < 16
      // first masked register index of this lane on a diagonal tile: query
      // q0 + qr0 + i sees key kj iff i >= kj - q0 - qr0
      const int vis0 = kj - q0 - qr0;
      u32x4_t pb[2], dsb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t la = *(const f32x4_t*)(lt + qr0 + 8 * t + 4 * h);
          const f32x4_t da = *(const f32x4_t*)(dt + qr0 + 8 * t + 4 * h);
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int e = 2 * h + e2, i0 = t * 8 + 2 * e;
            float p0 = __builtin_amdgcn_exp2f(fmaf(s[i0], c, -la[2 * e2]));
            float p1 = __builtin_amdgcn_exp2f(fmaf(s[i0 + 1], c, -la[2 * e2 + 1]));
            if (mask) {
              // diagonal tiles only: a real branch, not selects on every tile
              keep_branch();
              p0 = i0 < vis0 ? 0.0f : p0;
              p1 = i0 + 1 < vis0 ? 0.0f : p1;
            }
            pb[t][e] = H::pack(p0, p1);
            dsb[t][e] = H::pack(p0 * (dp[i0] - da[2 * e2]), p1 * (dp[i0 + 1] - da[2 * e2 + 1]));
          }
        }
      }
      {
        // chunk i: step t = i / (2 DBLK), d block b, dV (even) or dK (odd)
        constexpr int PF = 2, NC = 4 * DBLK;
        bf16x8_t fr[PF + 1];
        auto rd = [&](int i) {
          const int t = i / (2 * DBLK), b = (i % (2 * DBLK)) >> 1;
          return fa.tr_frag((i & 1) ? qt : gt, b, qb, t);
        };
#pragma unroll
        for (int i = 0; i < PF; ++i) fr[i] = rd(i);
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          if (i + PF < NC) fr[(i + PF) % (PF + 1)] = rd(i + PF);
          const int t = i / (2 * DBLK), b = (i % (2 * DBLK)) >> 1;
          __builtin_amdgcn_sched_barrier(0);
          if (i & 1)
            dka[b] = H::mma(fr[i % (PF + 1)], __builtin_bit_cast(bf16x8_t, dsb[t]), dka[b]);
          else
            dva[b] = H::mma(fr[i % (PF + 1)], __builtin_bit_cast(bf16x8_t, pb[t]), dva[b]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  if (t_beg < t_end) {
    load(t_beg, 0);
    store(0, t_beg);
  }
  __syncthreads();
  for (int j = t_beg; j < t_end; ++j) {
    const int buf = (j - t_beg) & 1;
    if (j + 1 < t_end) load(j + 1, buf ^ 1);
    const unsigned char* qt = smem + buf * T::BYTES;
    const unsigned char* gt = smem + (2 + buf) * T::BYTES;
    const float* lt = (const float*)(smem + STAT_OFF) + buf * 2 * BQ;
    const int q0 = j * BQ;
    // Causal: one body with a tile-uniform mask flag (a second inlined copy
    // of the body would not fit the register budget).
    tile_body(qt, gt, lt, q0, CAUSAL && q0 < kw0 + 31);
    if (j + 1 < t_end) store(buf ^ 1, j + 1);
    __syncthreads();
  }

  if (kj < N) {
    store_rowT<D, F16>(dv + kv_off + (size_t)kj * D, dva, g, 1.0f);
    store_rowT<D, F16>(dk + kv_off + (size_t)kj * D, dka, g, scale);
  }
}

// ------------------------------------------------------- single-pass backward
// attn_bwd_fused_kernel (D = 128, no mask): the dK/dV workgroup of 256 keys
// also forms its share of dQ, dQ_i += dS_ij K_j, from the dS it already has
// (the page's backward kernel adds these shares with atomics), so that S and
// dP are formed once instead of twice. The shares of the key workgroups of a
// head are added into an fp32 dQ in one fixed order (the order in which the
// tile schedule below reaches the tile): every (32-query tile, 32-wide d
// block) has a counter of the shares added so far; the wave whose share is
// k-th waits until it reads k, adds its share and sets k + 1, and the last
// share's wave writes dQ in the input type. The sum, and so dQ, is the same
// on every run.
//  * A workgroup takes its (head, key tile) from a ticket counter when it
//    starts, so the key workgroups of a head start together; with the
//    rotation below a head has at most one per CU of an XCD: every wait is
//    for a workgroup that is running (or, without the rotation, for an
//    earlier ticket), and every wait is bounded, setting an error word if it
//    gives up (it never does when the placement holds).
//  * The tickets are counted per XCD and heads are dealt to XCDs, so the
//    workgroups of a head share one L2, where the shares meet: counters and
//    shares are read with device-scope loads that skip the CU's own cache,
//    and a counter is set only after the share's stores have completed.
//  * Query tiles are 32 rows (LDS: the 256 K rows, Q and dO rings, two dS
//    buffers and a staging area for the sums read back; V^T in registers).
//    Per tile: S and dP, P and dS (written to LDS), dV and dK, then -- in
//    four waves, one per d block, alternating between waves 0-3 and 4-7 (the
//    two waves of a SIMD) from tile to tile -- the dQ share of the previous
//    tile from its dS buffer: K^T dS^T over the 256 keys. The counter and
//    the sum so far are loaded straight into LDS while the tile's products
//    run, and no wait for the new sum's stores lies within a step.
//  * The key workgroups of a head walk the query tiles from different
//    starting tiles, two steps apart, so a share rarely waits for its turn.
constexpr int kFusedBQ = 32;   // query rows per tile
constexpr int kFusedBN = 256;  // keys per workgroup
constexpr int kFusedHeader = 256;    // work area: 8 ticket counters, error word
constexpr int kFusedSpinLimit = 1 << 20;

// 4 bytes per lane straight into LDS (lane l writes lds_wave_base + 4 l);
// ordering as for lds_dma16.
__device__ __forceinline__ void lds_dma4(i32x4_t desc, unsigned char* lds_wave_base, int voffset) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(desc)
               : "m0");
}
// 4-byte loads of one word for all lanes straight into LDS (lane l writes
// lds_wave_base + 4 l), device scope; see lds_dma16 for the ordering rules.
// The memory clobber keeps every compiler-issued memory access on its side,
// so that the number of vector-memory operations issued after it is known.
__device__ __forceinline__ void lds_dma4_dev(i32x4_t desc, unsigned char* lds_wave_base,
                                             int voffset) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen sc1 lds"
               :
               : "s"(lds), "v"(voffset), "s"(desc)
               : "m0", "memory");
}
// 16 bytes per lane straight into LDS, device scope (lane l writes
// lds_wave_base + 16 l).
__device__ __forceinline__ void lds_dma16_dev(i32x4_t desc, unsigned char* lds_wave_base,
                                              int voffset) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc1 lds"
               :
               : "s"(lds), "v"(voffset), "s"(desc)
               : "m0", "memory");
}
// The lane index, recomputed where it is used (two VALU instructions)
// rather than kept live or reloaded from scratch: a reload waits for every
// memory operation in flight, including loads of the next tile.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ i32x4_t bytes_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return (i32x4_t){(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), (int)bytes,
                   kBufferRsrcWord3};
}

// delta_i = O_i . dO_i for all B*H*M rows (the same lanes and order of
// operations as the dQ kernel's) and L_i log2(e), and zeroes the counters of
// the fused kernel that follows.
template <int D, bool F16>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ delta, float* __restrict__ l2, int rows,
    int* __restrict__ clear, int nclear) {
  using H = Half16<F16>;
  constexpr int QSTEPS = D / 16;
  const int tid = workitem_id();
  const int lane = tid & 63, wave = tid >> 6;
  // (unsigned: the stride, up to 2^31, does not fit an int; i < nclear <= 2^28
  // never wraps)
  const unsigned stride = gridDim.x * 256u;
  for (unsigned i = workgroup_id() * 256u + tid; i < (unsigned)nclear; i += stride) clear[i] = 0;
  const int r = (workgroup_id() * 4 + wave) * 32 + (lane & 31);
  const int g = lane >> 5;
  bf16x8_t of[QSTEPS], gf[QSTEPS];
  load_b_rows<D>(o, r, rows, g, of);
  load_b_rows<D>(dout, r, rows, g, gf);
  float part = 0.0f;
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    const u32x4_t ow = __builtin_bit_cast(u32x4_t, of[t]);
    const u32x4_t gw = __builtin_bit_cast(u32x4_t, gf[t]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      part = fmaf(H::lo(ow[e]), H::lo(gw[e]), part);
      part = fmaf(H::hi(ow[e]), H::hi(gw[e]), part);
    }
  }
  const float dl = half_pair_sum(part);
  if (g == 0 && r < rows) delta[r] = dl;
  if (g == 1 && r < rows) l2[r] = lse[r] * kLog2e;
}

template <bool F16>
__global__ __launch_bounds__(512, 1) void attn_bwd_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ lse,
    const float* __restrict__ delta, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    unsigned char* __restrict__ work, long long l2_off, long long acc_off, int M, int N,
    int tiles_n, int heads, int heads_padded, int n_xcc, int cus_per_xcc, float c, float scale) {
  constexpr int D = 128, NT = 512, BNK = kFusedBN, BQ = kFusedBQ;
  using T = Tile<D, BQ>;  // Q and dO ring tiles (rows permuted, as in the dK/dV kernel)
  using H = Half16<F16>;
  constexpr int QSTEPS = T::QSTEPS, DBLK = T::DBLK;
  constexpr int DS_ROWB = 2 * BQ;  // a dS row: one key, 32 queries
  constexpr int DS_BYTES = BNK * DS_ROWB;
  constexpr int K_OFF = 0;
  constexpr int Q_OFF = K_OFF + BNK * T::ROWB;
  constexpr int G_OFF = Q_OFF + 2 * T::BYTES;
  constexpr int DS_OFF = G_OFF + 2 * T::BYTES;
  constexpr int STAT_OFF = DS_OFF + 2 * DS_BYTES;
  constexpr int ACC_OFF = STAT_OFF + 2 * 128 * 4;     // 4 x 32x32 fp32 shares read back
  constexpr int POLL_OFF = ACC_OFF + 4 * 4096;        // 4 x 64 counter copies
  constexpr int LDS_BYTES = POLL_OFF + 4 * 256;
  static_assert(LDS_BYTES <= 160 * 1024, "one workgroup per CU");
  static_assert(Stager<D, NT, BQ>::CPT == 1, "one chunk of each tile per thread");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];
  __shared__ int ticket_s;

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, g = lane >> 5;
  int* const hdr = (int*)work;
  int* const flags = (int*)(work + kFusedHeader);
  float* const accw = (float*)(work + acc_off);

  // (head, key tile) in start order from this XCD's ticket counter: heads
  // xcc, xcc + n_xcc, ... run on XCD xcc, key tiles in ticket order.
  if (tid == 0) {
    const int xcc = (__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15) % n_xcc;  // HW_REG_XCC_ID
    ticket_s = (atomicAdd(hdr + xcc, 1) << 3) | xcc;
  }
  __syncthreads();
  const int tk = __builtin_amdgcn_readfirstlane(ticket_s);
  const int ticket = tk >> 3;
  const int bh = (tk & 7) + n_xcc * (ticket / tiles_n);
  const int jk = ticket % tiles_n;  // key tile
  if (bh >= heads) {
    // heads past B*H pad the grid to a multiple of the XCD count; beyond
    // those, this XCD got more workgroups than it has work for: the placement
    // the launch relies on does not hold, so flag it
    if (tid == 0 && bh >= heads_padded) atomicOr(hdr + 8, 2);
    return;
  }

  const size_t q_off = (size_t)bh * M * D, kv_off = (size_t)bh * N * D;
  const uint16_t* qh = q + q_off;
  const uint16_t* gh = dout + q_off;
  // L log2(e) of the head's rows, from the delta kernel
  const float* lh = (const float*)(work + l2_off) + (size_t)bh * M;
  const float* dh = delta + (size_t)bh * M;
  const int k_wg0 = jk * BNK;
  const int kj = k_wg0 + wave * 32 + r32;  // this lane's key row
  const int t_end = (M + BQ - 1) / BQ;
  int* const fl = flags + (size_t)bh * t_end * 4;
  float* const acc_h = accw + (size_t)bh * M * D;

  // V^T as the B operand of dP (lane's key row) in registers; the
  // workgroup's K rows (row-major, swizzled, unpermuted) in LDS: row reads
  // give K^T for S, transposed reads K^T for dQ.
  bf16x8_t vf[QSTEPS];
  load_b_rows<D>(v + kv_off, kj, N, g, vf);
  {
    constexpr int KCH = BNK * T::CPR;
    static_assert(KCH % NT == 0, "K rows split evenly over the threads");
    const auto rk = rows_rsrc<D>(k + kv_off, k_wg0, N);
#pragma unroll
    for (int u = 0; u < KCH / NT; ++u) {
      const int ch = tid + u * NT;
      const int R = ch / T::CPR, pp = ch % T::CPR;
      *(u32x4_t*)(smem + K_OFF + ch * 16) = __builtin_amdgcn_raw_buffer_load_b128(
          rk, R * T::ROWB + ((pp ^ T::swz(R)) << 4), 0, 0);
    }
  }
  const unsigned char* k_row = smem + K_OFF + (wave * 32 + r32) * T::ROWB;

  Stager<D, NT, BQ> st;
  st.init(tid);
  FragAddr<D> fa;
  fa.init(lane);
  // Q and dO tiles, and L log2(e) (wave 0) and delta (wave 1) of the
  // tile's rows, go straight into LDS: no register and no wait of the
  // compiler's own depend on them. Stats buffer: 64 values of L log2(e),
  // then 64 of delta (the tile uses the first 32 of each). Rows past the end
  // read Q = dO = 0, L = delta = 0: P = 1 there but dP = dS = 0, so they add
  // nothing to dV, dK or dQ (and their dQ rows are not stored).
  auto load = [&](int j, int buf) {
    const i32x4_t rq = rows_desc<D>(qh, j * BQ, M);
    const i32x4_t rg = rows_desc<D>(gh, j * BQ, M);
    const int wbase = wave * 64 * 16;  // the wave's 64 chunks of each tile
    lds_dma16(rq, smem + Q_OFF + buf * T::BYTES + wbase, st.src[0], 0);
    lds_dma16(rg, smem + G_OFF + buf * T::BYTES + wbase, st.src[0], 0);
    if (wave < 2)
      lds_dma4(bytes_desc(wave == 0 ? lh : dh, (uint32_t)M * 4),
               smem + STAT_OFF + (buf * 128 + wave * 64) * 4, (j * BQ + lane_id_here()) * 4);
  };

  // dS^T as the B operand of the dQ product, from a dS buffer (key rows of
  // 32 queries, 16-byte chunk position p ^ ((row >> 2) & 3)): the same key
  // rows, in the same order, as FragAddr::tr_frag reads from the K rows.
  int ds_lo, ds_hi;
  {
    const int G = lane >> 4, L16 = lane & 15, jj = L16 >> 2, cc = L16 & 3;
    const int gg = G >> 1, nh = G & 1;
    const int chunk = 2 * nh + (cc >> 1);
    const int rl = 4 * gg + jj, rh = 8 + 4 * gg + jj;
    ds_lo = rl * DS_ROWB + ((chunk ^ ((rl >> 2) & 3)) << 4) + (cc & 1) * 8;
    ds_hi = rh * DS_ROWB + ((chunk ^ ((rh >> 2) & 3)) << 4) + (cc & 1) * 8;
  }
  auto ds_frag = [&](const unsigned char* ds_t, int blk, int t) {
    const unsigned char* base = ds_t + (blk * 32 + 16 * t) * DS_ROWB;
    const s16x4_t lo = lds_read_tr16(base + ds_lo);
    const s16x4_t hi = lds_read_tr16(base + ds_hi);
    const s16x8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, x);
  };

  f32x16_t dka[DBLK], dva[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[b][i] = 0.0f;
      dva[b][i] = 0.0f;
    }

  // The dQ shares. Key workgroup jk walks the query tiles starting at tile
  // -jk*rot (mod t_end), so the workgroups of a head reach any tile rot steps
  // apart and the shares of a tile arrive in a fixed order: by arrival, which
  // is key order rotated to start at the first arriver. (rot = 0: all start
  // at tile 0 and the order is key order.) With rot > 0 a share may wait for
  // a workgroup with a later ticket, so all key workgroups of a head must be
  // resident together: at most one per CU of an XCD. A wait in the
  // middle of step n is for a counter passed in the middle of step
  // n + 1 - rot of another workgroup, and a pass needs nothing but the
  // passing workgroup's barrier at the end of the step before, so every
  // chain of waits runs back through earlier steps and none closes into a
  // cycle (rot = 1 as well, which measured no faster than 2; rot = 0 only
  // waits for lower key tiles).
  const int rot = tiles_n <= cus_per_xcc && t_end >= 2 * tiles_n ? 2 : 0;
  auto tile_at = [&](int n) {  // query tile of step n
    const int t = n - jk * rot;
    return t < 0 ? t + t_end : t;
  };
  auto share_pos = [&](int p) {  // this workgroup's place among the shares of tile p
    const int jw = rot == 0 ? tiles_n : min(tiles_n, (t_end - p + rot - 1) / rot);
    const int r = jk - jw;
    return r < 0 ? r + tiles_n : r;
  };
  // This wave's dQ duty: d block db of the share formed in steps n with
  // (n - 1) % 2 == par (the share of the tile of step n - 1). Waves db and
  // db + 4 share a SIMD and take turns.
  const int db = wave & 3, par = wave >> 2;
  // FragAddr::tr_frag's lane offsets for d block db (db is only known at
  // run time, so they are formed here rather than indexed from fa).
  int ktr_lo, ktr_hi;
  {
    const int G = lane >> 4, L16 = lane & 15, jj = L16 >> 2, cc = L16 & 3;
    const int gg = G >> 1, nh = G & 1;
    const int chunk = 4 * db + 2 * nh + (cc >> 1);
    const int rl = 4 * gg + jj, rh = 8 + 4 * gg + jj;
    ktr_lo = rl * T::ROWB + ((chunk ^ T::swz(rl)) << 4) + (cc & 1) * 8;
    ktr_hi = rh * T::ROWB + ((chunk ^ T::swz(rh)) << 4) + (cc & 1) * 8;
  }
  auto k_tr_frag = [&](int blk, int t) {
    const unsigned char* base = smem + K_OFF + (blk * 32 + 16 * t) * T::ROWB;
    const s16x4_t lo = lds_read_tr16(base + ktr_lo);
    const s16x4_t hi = lds_read_tr16(base + ktr_hi);
    const s16x8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, x);
  };
  unsigned char* const stage = smem + ACC_OFF + db * 4096;
  unsigned char* const poll = smem + POLL_OFF + db * 256;
  // the lane's 16 sums: query row r32 of the tile, d = 32 db + 8 i4 + 4 g + 0..3
  const int acc_voff = r32 * D * 4 + 128 * db + 16 * g;
  bool broken = false;
  auto share_desc = [&](int p) {
    const int rows = min(BQ, M - p * BQ);
    return bytes_desc(acc_h + (size_t)p * BQ * D, (uint32_t)rows * D * 4);
  };
  auto counter_desc = [&]() { return bytes_desc(fl, (uint32_t)t_end * 16); };
  // Wait until the counter of (p, db) reads pos; its first read was issued
  // earlier and is complete once at most `after` later operations are in
  // flight.
  auto wait_turn = [&](int p, int pos, int after) {
    if (after == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (after == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // (a plain LDS read: the asm statements' memory clobbers order it)
    int seen = __builtin_amdgcn_readfirstlane(*(const int*)poll);
    int spins = 0;
    while (seen != pos && !broken) {
      __builtin_amdgcn_s_sleep(2);
      lds_dma4_dev(counter_desc(), poll, (p * 4 + db) * 4);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      seen = __builtin_amdgcn_readfirstlane(*(const int*)poll);
      if (++spins > kFusedSpinLimit) {
        broken = true;
        if (lane == 0) atomicOr(hdr + 8, 1);
      }
    }
  };
  // Issue the loads of the sum so far into the staging area (after wait_turn).
  auto load_sum = [&](int p) {
    const i32x4_t sd = share_desc(p);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) lds_dma16_dev(sd, stage + i4 * 1024, acc_voff + 32 * i4);
  };
  // The dQ share of a tile (dS in ds_t): K^T dS^T over the 256 keys. (Two
  // accumulators for alternate key steps measured slower: the extra
  // registers spill.)
  auto dq_share = [&](const unsigned char* ds_t) {
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    constexpr int PF = 2, NS = BNK / 16;
    bf16x8_t fk[PF + 1], fs[PF + 1];
    auto rd = [&](int i, bf16x8_t& a, bf16x8_t& b) {
      a = k_tr_frag(i >> 1, i & 1);
      b = ds_frag(ds_t, i >> 1, i & 1);
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) rd(i, fk[i], fs[i]);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PF < NS) rd(i + PF, fk[(i + PF) % (PF + 1)], fs[(i + PF) % (PF + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      acc = H::mma(fk[i % (PF + 1)], fs[i % (PF + 1)], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };
  // new sum = sum so far (in the staging area) + share
  auto add_sum = [&](f32x16_t acc) {
    const f32x4_t* const st4 = (const f32x4_t*)(stage + 16 * lane);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4_t x = st4[i4 * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * i4 + e] = x[e] + acc[4 * i4 + e];
    }
    return acc;
  };
  auto wait_vmem_but_4 = [&]() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); };
  // Store a share's sum: back to the fp32 sums, or (the last share) as dQ.
  // Either way exactly four stores, bounded by the tile's rows (rows past M
  // are dropped), and nothing else: the waits that follow count them.
  auto store_share = [&](const f32x16_t& acc, int p, bool last) {
    const int rows = min(BQ, M - p * BQ);
    if (!last) {
      const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(acc_h + (size_t)p * BQ * D),
                                                        (short)0, rows * D * 4, kBufferRsrcWord3);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4_t x = {acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rs,
                                               acc_voff + 32 * i4, 0, 0);
      }
    } else {
      const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(dq + q_off + (size_t)p * BQ * D),
                                                        (short)0, rows * D * 2, kBufferRsrcWord3);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2_t w;
        w[0] = H::pack(acc[4 * i4] * scale, acc[4 * i4 + 1] * scale);
        w[1] = H::pack(acc[4 * i4 + 2] * scale, acc[4 * i4 + 3] * scale);
        __builtin_amdgcn_raw_buffer_store_b64(w, rs, acc_voff / 2 + 16 * i4, 0, 0);
      }
    }
    // nothing the compiler issues later may move above these stores
    asm volatile("" ::: "memory");
  };
  // The share's stores have completed: the next share of tile p may go.
  auto pass_turn = [&](int p, int pos) {
    if (lane == 0)
      __hip_atomic_store(fl + p * 4 + db, pos + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // One 32-query tile: S = Q K^T and dP = dO V^T, P and dS (dS also to LDS
  // for the dQ product), then dV^T += dO^T P and dK^T += Q^T dS. `mid` runs
  // between the dS stores and the dV/dK products.
  auto tile_body = [&](const unsigned char* qt, const unsigned char* gt, const float* lt,
                       unsigned char* ds_out, auto&& mid) __attribute__((always_inline)) {
    const float* dt = lt + 64;
    f32x16_t s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = 0.0f;
      dp[i] = 0.0f;
    }
    {
      // chunk i: S step i/2 (even: Q rows, K^T from the K rows) or dP step
      // i/2 (odd: dO rows, V^T from registers), operands one chunk ahead
      constexpr int PF = 1, NA = 2 * QSTEPS;
      bf16x8_t fa_[PF + 1], fb_[PF + 1];
      auto rd = [&](int i, bf16x8_t& x, bf16x8_t& y) {
        x = fa.row_frag((i & 1) ? gt : qt, 0, i >> 1, g);
        if (i & 1) {
          y = vf[i >> 1];
        } else {
          const u32x4_t kw = *(const u32x4_t*)(k_row + (((2 * (i >> 1) + g) ^ fa.sw) << 4));
          y = __builtin_bit_cast(bf16x8_t, kw);
        }
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) rd(i, fa_[i], fb_[i]);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + PF < NA) rd(i + PF, fa_[(i + PF) % (PF + 1)], fb_[(i + PF) % (PF + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        if (i & 1) dp = H::mma(fa_[i % (PF + 1)], fb_[i % (PF + 1)], dp);
        else s = H::mma(fa_[i % (PF + 1)], fb_[i % (PF + 1)], s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int qr0 = 16 * g;  // lane's queries: tile row qr0 + r, r < 16
    u32x4_t pb[2], dsb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t la = *(const f32x4_t*)(lt + qr0 + 8 * t + 4 * h);
        const f32x4_t da = *(const f32x4_t*)(dt + qr0 + 8 * t + 4 * h);
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int e = 2 * h + e2, i0 = t * 8 + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i0], c, -la[2 * e2]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i0 + 1], c, -la[2 * e2 + 1]));
          pb[t][e] = H::pack(p0, p1);
          dsb[t][e] = H::pack(p0 * (dp[i0] - da[2 * e2]), p1 * (dp[i0 + 1] - da[2 * e2 + 1]));
        }
      }
    }
    {
      // key row wave*32 + r32; queries 16 g + 8 t .. +7 are logical chunk 2 g + t
      const int kk = wave * 32 + r32;
      const int sw = (kk >> 2) & 3;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *(u32x4_t*)(ds_out + kk * DS_ROWB + (((2 * g + t) ^ sw) << 4)) = dsb[t];
    }
    mid();
    {
      // chunk i: step t = i / (2 DBLK), d block b, dV (even) or dK (odd)
      constexpr int PF = 2, NC = 4 * DBLK;
      bf16x8_t fr[PF + 1];
      auto rd = [&](int i) {
        const int t = i / (2 * DBLK), b = (i % (2 * DBLK)) >> 1;
        return fa.tr_frag((i & 1) ? qt : gt, b, 0, t);
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) fr[i] = rd(i);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        if (i + PF < NC) fr[(i + PF) % (PF + 1)] = rd(i + PF);
        const int t = i / (2 * DBLK), b = (i % (2 * DBLK)) >> 1;
        __builtin_amdgcn_sched_barrier(0);
        if (i & 1)
          dka[b] = H::mma(fr[i % (PF + 1)], __builtin_bit_cast(bf16x8_t, dsb[t]), dka[b]);
        else
          dva[b] = H::mma(fr[i % (PF + 1)], __builtin_bit_cast(bf16x8_t, pb[t]), dva[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Step n: the tile of step n (S, dP, dS, dV, dK), then in the duty waves
  // the dQ share of the tile of step n - 1: the wait for its turn and the
  // loads of the sum so far in the middle of the step, the product and the
  // new sum's four stores at its end. The stores are the wave's last memory
  // operations of the step: the wait before the barrier leaves them in
  // flight, and the counter is passed on in the middle of step n + 1, once
  // they have completed (so no wait for them lies on a step's critical path).
  load(tile_at(0), 0);
  wait_vmem();
  __syncthreads();
  int pass_p = -1, pass_pos = 0;  // a share whose counter is still to be passed on
  for (int n = 0; n < t_end; ++n) {
    const int buf = n & 1;
    const bool more = n + 1 < t_end;
    const bool duty = n >= 1 && ((n - 1) & 1) == par;
    const int p = duty ? tile_at(n - 1) : 0;
    const int pos = duty ? share_pos(p) : 0;
    if (duty && pos > 0) lds_dma4_dev(counter_desc(), poll, (p * 4 + db) * 4);
    if (more) load(tile_at(n + 1), buf ^ 1);
    const int after = more ? (wave < 2 ? 3 : 2) : 0;  // this step's loads
    tile_body(smem + Q_OFF + buf * T::BYTES, smem + G_OFF + buf * T::BYTES,
              (const float*)(smem + STAT_OFF) + buf * 128, smem + DS_OFF + buf * DS_BYTES,
              [&]() {
                if (pass_p >= 0) {
                  // the previous step's stores came before this step's loads
                  // (and this wave has no counter read in flight)
                  if (after == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
                  else if (after == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                  pass_turn(pass_p, pass_pos);
                  pass_p = -1;
                }
                if (duty && pos > 0) {
                  wait_turn(p, pos, after);
                  load_sum(p);
                }
              });
    if (duty) {
      f32x16_t acc = dq_share(smem + DS_OFF + (buf ^ 1) * DS_BYTES);
      if (pos > 0) {
        wait_vmem();  // the sum so far is in the staging area
        acc = add_sum(acc);
      }
      store_share(acc, p, pos == tiles_n - 1);
      if (pos != tiles_n - 1) {
        pass_p = p;
        pass_pos = pos;
      }
    }
    if (more) {
      // this step's loads have landed (a share's stores may still be in flight)
      if (duty) wait_vmem_but_4();
      else wait_vmem();
    }
    __syncthreads();
  }
  wait_vmem();
  if (pass_p >= 0) pass_turn(pass_p, pass_pos);
  if (((t_end - 1) & 1) == par) {
    // the share of the last step's tile
    const int p = tile_at(t_end - 1);
    const int pos = share_pos(p);
    if (pos > 0) {
      lds_dma4_dev(counter_desc(), poll, (p * 4 + db) * 4);
      wait_turn(p, pos, 0);
      load_sum(p);
    }
    f32x16_t acc = dq_share(smem + DS_OFF + ((t_end - 1) & 1) * DS_BYTES);
    if (pos > 0) {
      wait_vmem();
      acc = add_sum(acc);
    }
    store_share(acc, p, pos == tiles_n - 1);
    wait_vmem();
    if (pos != tiles_n - 1) pass_turn(p, pos);
  }

  if (kj < N) {
    store_rowT<D, F16>(dv + kv_off + (size_t)kj * D, dva, g, 1.0f);
    store_rowT<D, F16>(dk + kv_off + (size_t)kj * D, dka, g, scale);
  }
}

// ----------------------------------------------------------------- launch
template <int D, bool CAUSAL, bool F16>
static hipError_t launch_bwd_d(const BwdLaunchArgs& a) {
  const float c = a.scale * kLog2e;
  const int heads = (int)a.BH;
  if (a.M > 0) {
    constexpr int BM = bwd_waves(D) * 32;
    const int tiles_m = (int)((a.M + BM - 1) / BM);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, F16>), dim3((unsigned)(tiles_m * heads)),
                       dim3(bwd_waves(D) * 64), 0, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.o,
                       a.lse, (const uint16_t*)a.dout, (uint16_t*)a.dq, a.delta, (int)a.M,
                       (int)a.N, tiles_m, heads, c, a.scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int BNK = bwd_waves(D) * 32;
  const int tiles_n = (int)((a.N + BNK - 1) / BNK);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, F16>), dim3((unsigned)(tiles_n * heads)),
                     dim3(bwd_waves(D) * 64), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.lse, a.delta,
                     (const uint16_t*)a.dout, (uint16_t*)a.dk, (uint16_t*)a.dv, (int)a.M,
                     (int)a.N, tiles_n, heads, c, a.scale);
  return hipGetLastError();
}

template <bool F16>
static hipError_t launch_bwd_16(const BwdLaunchArgs& a) {
  switch (a.D) {
    case 32: return a.causal ? launch_bwd_d<32, true, F16>(a) : launch_bwd_d<32, false, F16>(a);
    case 64: return a.causal ? launch_bwd_d<64, true, F16>(a) : launch_bwd_d<64, false, F16>(a);
    case 128:
      return a.causal ? launch_bwd_d<128, true, F16>(a) : launch_bwd_d<128, false, F16>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_bf16(const BwdLaunchArgs& a) { return launch_bwd_16<false>(a); }
hipError_t launch_bwd_f16(const BwdLaunchArgs& a) { return launch_bwd_16<true>(a); }

// Work area of the single-pass backward: header (ticket counters, error
// word), one counter per (head, 32-query tile, d block), L log2(e) per row,
// fp32 dQ sums.
static int64_t fused_counter_bytes(int64_t BH, int64_t M) {
  return (BH * ((M + kFusedBQ - 1) / kFusedBQ) * 16 + 255) / 256 * 256;
}

static int64_t fused_l2_bytes(int64_t BH, int64_t M) { return (BH * M * 4 + 255) / 256 * 256; }

int64_t bwd_fused_work_bytes(int64_t BH, int64_t M, int64_t N, int64_t D, bool causal) {
  // D = 128 without the mask; row counts that the kernels index with 32-bit
  // integers.
  if (D != 128 || causal || BH < 1 || M < 1 || N < 1) return 0;
  if (BH * M > (int64_t{1} << 30) || M > (int64_t{1} << 24) || N > (int64_t{1} << 24)) return 0;
  // counters cleared by the delta kernel: at most 2^26 tiles (its word count fits an int)
  if (BH * ((M + kFusedBQ - 1) / kFusedBQ) > (int64_t{1} << 26)) return 0;
  return kFusedHeader + fused_counter_bytes(BH, M) + fused_l2_bytes(BH, M) + BH * M * D * 4;
}

// XCDs of the current device and compute units per XCD (host queries, no
// GPU work). The fused kernel deals heads to XCDs (B*H padded to a multiple
// of the XCD count).
static bool fused_placement(int* n_xcc, int* cus_per_xcc) {
  int dev = 0, x = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
      hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  *n_xcc = x;
  *cus_per_xcc = x > 0 ? cu / x : 0;
  return (x == 1 || x == 2 || x == 4 || x == 8) && *cus_per_xcc > 0;
}

template <bool F16>
static hipError_t launch_bwd_fused_16(const BwdLaunchArgs& a, void* work) {
  int n_xcc = 0, cus_per_xcc = 0;
  if (!fused_placement(&n_xcc, &cus_per_xcc))
    return F16 ? launch_bwd_16<true>(a) : launch_bwd_16<false>(a);  // the two-kernel backward
  const int64_t rows = a.BH * a.M;
  const int64_t counters = fused_counter_bytes(a.BH, a.M);
  const int nclear = (int)((kFusedHeader + counters) / 4);
  const int64_t l2_off = kFusedHeader + counters, acc_off = l2_off + fused_l2_bytes(a.BH, a.M);
  hipLaunchKernelGGL((attn_bwd_delta_kernel<128, F16>), dim3((unsigned)((rows + 127) / 128)),
                     dim3(256), 0, a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout,
                     a.lse, a.delta, (float*)((unsigned char*)work + l2_off), (int)rows,
                     (int*)work, nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles_n = (int)((a.N + kFusedBN - 1) / kFusedBN);
  const int64_t heads_padded = (a.BH + n_xcc - 1) / n_xcc * n_xcc;
  hipLaunchKernelGGL((attn_bwd_fused_kernel<F16>), dim3((unsigned)(heads_padded * tiles_n)),
                     dim3(512),
                     0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.lse, a.delta, (const uint16_t*)a.dout,
                     (uint16_t*)a.dq, (uint16_t*)a.dk, (uint16_t*)a.dv, (unsigned char*)work,
                     (long long)l2_off, (long long)acc_off, (int)a.M, (int)a.N, tiles_n,
                     (int)a.BH, (int)heads_padded, n_xcc, cus_per_xcc, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_fused(const BwdLaunchArgs& a, void* work, bool f16) {
  return f16 ? launch_bwd_fused_16<true>(a, work) : launch_bwd_fused_16<false>(a, work);
}
int bwd_fused_error_offset() { return 8 * 4; }

// (the smallest tiles of any head dim: grid-size checks stay conservative)
int bwd_dq_tile_rows() { return bwd_waves(32) * 32; }
int bwd_dkdv_tile_rows() { return bwd_waves(32) * 32; }

}  // namespace mi355
