// attn_fwd_fp8.hip -- FlashAttention-2 forward with fp8 (OCP e4m3) inputs and
// P rounded to fp8 before the second product, on gfx950.
//
// "Blackwell Attention Example", attention kernel: P is cast to the value
// dtype before the second product, so with fp8 values the second product
// runs on fp8 operands too; its note on that product says that fp8 values in
// their natural (non-transposed) layout are a Blackwell-only case, i.e. fp8 V
// is otherwise supplied transposed. Here q and k are [B, H, M, D] /
// [B, H, N, D] e4m3, v comes transposed as vt [B, H, D, N] e4m3, and both
// products run on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit
// scales, fp32 accumulation). O is written in bf16 (not in the input type:
// an fp8 output would throw away most of what the fp32 accumulation keeps)
// and L, as everywhere, in fp32, natural log. The softmax is the tiled online
// one of "Extend Thunder with CUDA-Python" (Python reference section), in
// base 2 with scale * log2(e) folded into the exponent as in the Blackwell
// example.
//
// gfx950 mapping (the bf16 kernel's design, with the fp8 operand shapes):
//  * One workgroup = 8 waves = 256 query rows of one (batch, head); 64-key
//    tiles staged HBM -> VGPRs -> LDS (rings of 3 K and 2 V^T tiles), one
//    barrier per tile; S(j+1) = K(j+1) Q^T on the matrix cores while the
//    vector ALU turns S(j) into P(j), then O += V(j)^T P(j)^T.
//  * The fp8 MFMA takes 64 contraction elements: lane l supplies row (A) or
//    column (B) l % 32 and elements 32 (l / 32) .. + 31, as 32 bytes. The
//    score accumulator of lane l holds query l % 32 and 16 keys per 32-key
//    block; K rows are stored in LDS in an order that makes those 16 keys,
//    over the two blocks of a 64-key tile, exactly keys 32 (l / 32) .. + 31
//    -- the 32 contraction elements lane l must supply as P^T in the second
//    product. The matching V^T operand is then 32 consecutive bytes of one
//    row of the transposed V tile.
//  * The row sum l is one more MFMA per tile: an A operand whose first row is
//    all ones and whose other rows are zero, times P^T, accumulates the sum of
//    the fp8-rounded P of every query row in fp32 -- the same P the second
//    product sees, so a constant V comes back exactly.
//  * e4m3 has no infinity: a value at or above 464 converts to NaN. The
//    reference max therefore moves whenever an exponent argument of a tile
//    exceeds 8 (p <= 256); the tile then takes the exact path (S recomputed
//    from the K tile still in LDS, new m, O and l rescaled, P recomputed).
//  * K rows and V^T rows are padded by 16 bytes in LDS: the 16 rows a
//    half-wave reads at one column start in distinct 4-bank groups.

#include "attn_device.h"
#include "attn_launch.h"

namespace mi355 {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// e4m3 x e4m3 -> fp32, 32 x 32 x 64, unit block scales (e8m0 exponent 127).
__device__ __forceinline__ f32x16_t mma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ void keep_branch8() { asm volatile(""); }

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor word 3 (see attn_fwd_bf16.hip)

// Exponent arguments above this send a tile to the exact path (p <= 2^8,
// below e4m3's largest finite value 448).
constexpr float kFp8ExpLimit = 8.0f;

}  // namespace

template <int D>
struct Fp8Cfg {
  static constexpr int WAVES = 8, NT = 512, BM = 256, BN = 64;
  static constexpr int KROWB = D + 16;          // LDS bytes per K row (padded)
  static constexpr int KTILEB = BN * KROWB;
  static constexpr int VROWB = BN + 16;         // LDS bytes per V^T row (padded)
  static constexpr int VTILEB = D * VROWB;
  static constexpr int KCPR = D / 16;           // 16-byte chunks per K row
  static constexpr int KCHUNKS = BN * KCPR;     // per K tile
  static constexpr int VCHUNKS = D * (BN / 16); // per V^T tile
  static constexpr int QSTEPS = D / 64;         // contraction steps of S
  static constexpr int DBLK = D / 32;           // 32-row blocks of O^T
  static constexpr int KBUF = 3, VBUF = 2;
  static constexpr int V_OFF = KBUF * KTILEB;
  static constexpr int LDS_BYTES = V_OFF + VBUF * VTILEB;
  static_assert(KCHUNKS <= NT && VCHUNKS <= NT, "one staging chunk per thread");
  // LDS row R of a K tile holds key kperm(R): row 8q + 4g + s of 32-row
  // block kb holds key 32 g + 16 kb + 4 q + s, so accumulator register r of
  // lane group g in block kb is key 32 g + 16 kb + r.
  __device__ static constexpr int kperm(int R) {
    const int kb = R >> 5, b = R & 31;
    return 32 * ((b >> 2) & 1) + 16 * kb + 4 * (b >> 3) + (b & 3);
  }
};

template <int D, bool CAUSAL, bool POS_SCALE>
__global__ __launch_bounds__(512, 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ vt, uint16_t* __restrict__ o, float* __restrict__ lse,
    int M, int N, int tiles_m, int heads, float c) {
  using C = Fp8Cfg<D>;
  constexpr int BM = C::BM, BN = C::BN, QSTEPS = C::QSTEPS, DBLK = C::DBLK;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];

  const int tid = workitem_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const TileId tile = tile_order(workgroup_id(), tiles_m, heads, CAUSAL);
  const int bh = tile.bh, tm = tile.tm;
  const uint8_t* qh = q + (size_t)bh * M * D;
  const uint8_t* kh = k + (size_t)bh * N * D;
  const uint8_t* vth = vt + (size_t)bh * D * N;

  const int q_wg0 = tm * BM;
  const int qw0 = q_wg0 + wave * 32;
  const int qi = qw0 + r32;

  int nt = (N + BN - 1) / BN;
  if (CAUSAL) nt = min(nt, (min(q_wg0 + BM, M) - 1) / BN + 1);

  // ---- staging: thread tid moves 16-byte chunk tid of each tile (threads
  // past the chunk count repeat the last chunk: same bytes, same place).
  const int kch = min(tid, C::KCHUNKS - 1);
  const int kR = kch / C::KCPR, kcp = kch % C::KCPR;
  const int k_src = C::kperm(kR) * D + 16 * kcp;   // bytes from the tile's first key
  const int k_dst = kR * C::KROWB + 16 * kcp;
  const int vch = min(tid, C::VCHUNKS - 1);
  const int vd = vch / (BN / 16), vcp = vch % (BN / 16);
  const int v_dst = vd * C::VROWB + 16 * vcp;
  u32x4_t kst, vst;
  auto load_k = [&](int j) {
    const int jc = min(j, nt - 1);
    const uint32_t bytes = (uint32_t)(N - jc * BN) * (uint32_t)D;
    const auto r = __builtin_amdgcn_make_buffer_rsrc((void*)(kh + (size_t)jc * BN * D), (short)0,
                                                     (int)bytes, kRsrcWord3);
    kst = __builtin_amdgcn_raw_buffer_load_b128(r, k_src, 0, 0);
  };
  // V^T tile j: bytes [64 j, 64 j + 64) of each of the D rows (row stride N).
  // The descriptor is bounded by the head's slab; N is a multiple of 16, so a
  // chunk is wholly inside or wholly past the keys and those past are zeroed.
  auto load_v = [&](int j) {
    const int jc = min(j, nt - 1);
    const auto r = __builtin_amdgcn_make_buffer_rsrc((void*)vth, (short)0, (int)(D * N), kRsrcWord3);
    const int col = jc * BN + 16 * vcp;
    u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, vd * N + col, 0, 0);
    if (col >= N) x = u32x4_t{0u, 0u, 0u, 0u};
    vst = x;
  };
  auto store_k = [&](int buf) { *(u32x4_t*)(smem + buf * C::KTILEB + k_dst) = kst; };
  auto store_v = [&](int buf) { *(u32x4_t*)(smem + C::V_OFF + buf * C::VTILEB + v_dst) = vst; };

  // ---- operands
  // Q^T (B of S^T = K Q^T): query qi, d = 64 t + 32 g .. + 31.
  i32x8_t qf[QSTEPS];
#pragma unroll
  for (int t = 0; t < QSTEPS; ++t) {
    u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qi < M) {
      const uint8_t* p = qh + (size_t)qi * D + 64 * t + 32 * g;
      lo = *(const u32x4_t*)p;
      hi = *(const u32x4_t*)(p + 16);
    }
    qf[t] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  // Ones row (A of the row-sum product): lanes of row 0 hold 1.0 (0x38).
  const int one4 = (r32 == 0) ? 0x38383838 : 0;
  const i32x8_t ones = {one4, one4, one4, one4, one4, one4, one4, one4};

  auto frag32 = [](const unsigned char* p) -> i32x8_t {
    const u32x4_t lo = *(const u32x4_t*)p, hi = *(const u32x4_t*)(p + 16);
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // K fragment i of S^T: key block kb = i & 1, d-step t = i >> 1.
  auto k_frag = [&](int buf, int i) {
    const int t = i >> 1, kb = i & 1;
    return frag32(smem + buf * C::KTILEB + (32 * kb + r32) * C::KROWB + 64 * t + 32 * g);
  };
  // V^T fragment of O^T block b: row 32 b + r32, keys 32 g .. + 31.
  auto v_frag = [&](int buf, int b) {
    return frag32(smem + C::V_OFF + buf * C::VTILEB + (32 * b + r32) * C::VROWB + 32 * g);
  };

  const float cc_scale = POS_SCALE ? c : 1.0f;
  float m_run = -INFINITY, m_sub = 0.0f;
  f32x16_t acc[DBLK], accl;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) accl[i] = 0.0f;
  f32x16_t s_a[2], s_b[2];

  auto qk = [&](int buf, f32x16_t* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 2 * QSTEPS; ++i) s[i & 1] = mma_fp8(k_frag(buf, i), qf[i >> 1], s[i & 1]);
  };
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
  // register r of block kb is key 32 g + 16 kb + r; masked when >= lim
  auto mask_tile = [&](f32x16_t* s, int j) {
    const int base = j * BN + 32 * g;
    int lim = N - base;
    if (CAUSAL) lim = min(lim, qi - base + 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * kb + i >= lim) s[kb][i] = -INFINITY;
  };
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
  // Four e4m3 values of P (exp2 of four scores against the reference) packed
  // into one dword in contraction order; xm tracks the largest argument.
  auto exp4 = [&](float x0, float x1, float x2, float x3, float& xm) -> int {
    const float a0 = fmaf(x0, cc_scale, -m_sub), a1 = fmaf(x1, cc_scale, -m_sub);
    const float a2 = fmaf(x2, cc_scale, -m_sub), a3 = fmaf(x3, cc_scale, -m_sub);
    xm = __builtin_fmaxf(xm, __builtin_fmaxf(__builtin_fmaxf(a0, a1), __builtin_fmaxf(a2, a3)));
    // the first conversion fills bytes 0-1 and keeps bytes 2-3 of its third
    // operand, which the second conversion then overwrites: any register will
    // do there (a dead one costs no move, where a zero costs one per dword)
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(a0), __builtin_amdgcn_exp2f(a1),
                                           __float_as_int(a0), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(a2), __builtin_amdgcn_exp2f(a3), w,
                                       true);
    return w;
  };
  // P^T of a whole prepared tile: dwords 0-3 from block 0, 4-7 from block 1.
  auto tile_exp = [&](const f32x16_t* s, i32x8_t& p) -> float {
    float xm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x16_t& sb = s[w >> 2];
      const int r = 4 * (w & 3);
      p[w] = exp4(sb[r], sb[r + 1], sb[r + 2], sb[r + 3], xm);
    }
    return xm;
  };
  auto rescale = [&](float a) {
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= a;
#pragma unroll
    for (int i = 0; i < 16; ++i) accl[i] *= a;
  };

  // First half of iteration j: S(j+1) = K(j+1) Q^T in fenced chunks, each
  // with a share of the exponentials of S(j); the loads of K(j+2) go out at
  // the start. Returns the largest exponent argument of the lane.
  auto region_a = [&](int j, const f32x16_t* sc, f32x16_t* sn, i32x8_t& p)
                      __attribute__((always_inline)) -> float {
    constexpr int NF = 2 * QSTEPS;  // MFMAs of one S tile
    constexpr int WPC = 8 / NF;     // P dwords per chunk
    const int buf = (j + 1) % C::KBUF;
    load_k(j + 2);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kb][i] = 0.0f;
    i32x8_t fr = k_frag(buf, 0);
    float xm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const i32x8_t cur = fr;
      if (i + 1 < NF) fr = k_frag(buf, i + 1);
#pragma unroll
      for (int u = 0; u < WPC; ++u) {
        const int w = i * WPC + u;
        const f32x16_t& sb = sc[w >> 2];
        const int r = 4 * (w & 3);
        p[w] = exp4(sb[r], sb[r + 1], sb[r + 2], sb[r + 3], xm);
      }
      __builtin_amdgcn_sched_barrier(0);
      sn[i & 1] = mma_fp8(cur, qf[i >> 1], sn[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    return xm;
  };
  // Second half: O^T += V^T P^T (DBLK MFMAs) and the row-sum MFMA; the
  // loads of V(j+1) go out at the start, and K(j+2) is written to its ring
  // slot beside the first product (not at the end of the first half, where
  // the write waits for its loads in front of the exact-path check).
  auto region_b = [&](int j, const i32x8_t& p, bool has_next) __attribute__((always_inline)) {
    const int buf = j & 1;
    if (has_next) load_v(j + 1);
    i32x8_t fr = v_frag(buf, 0);
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const i32x8_t cur = fr;
      if (b + 1 < DBLK) fr = v_frag(buf, b + 1);
      if (has_next && b == 0) store_k((j + 2) % C::KBUF);
      acc[b] = mma_fp8(cur, p, acc[b]);
      __builtin_amdgcn_sched_barrier(0);
    }
    accl = mma_fp8(ones, p, accl);
  };

  auto iter = [&](int j, f32x16_t* sc, f32x16_t* sn, bool has_next) __attribute__((always_inline)) {
    i32x8_t p;
    float xm;
    if (has_next) {
      xm = region_a(j, sc, sn, p);
    } else {
      xm = tile_exp(sc, p);
    }
    if (wave_any(xm > kFp8ExpLimit)) {
      // A score rose more than 8 (log2 units) above the reference: redo
      // this tile exactly (O holds tiles < j; K(j) is still in its slot).
      keep_branch8();
      qk(j % C::KBUF, sc);
      scale_tile(sc);
      if (needs_mask(j)) mask_tile(sc, j);
      const float alpha = exact_ref(sc);
      rescale(alpha);
      tile_exp(sc, p);
    }
    region_b(j, p, has_next);
    if (has_next) {
      store_v((j + 1) & 1);
      scale_tile(sn);
      if (needs_mask(j + 1)) {
        keep_branch8();
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
  __syncthreads();
  qk(0, s_a);
  scale_tile(s_a);
  if (needs_mask(0)) {
    keep_branch8();
    mask_tile(s_a, 0);
  }
  exact_ref(s_a);

  int j = 0;
  for (; j + 2 < nt; j += 2) {
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

  // row 0 of the row-sum block sits in register 0 of lanes 0-31 (row 4,
  // all zeros, in lanes 32-63)
  const float l_tot = half_pair_sum(accl[0]);
  if (qi >= M) return;
  const float inv = 1.0f / l_tot;
  uint16_t* orow = o + (size_t)bh * M * D + (size_t)qi * D;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = b * 32 + i4 * 8 + g * 4;
      u32x2_t st;
      st[0] = pack_bf16x2(acc[b][i4 * 4 + 0] * inv, acc[b][i4 * 4 + 1] * inv);
      st[1] = pack_bf16x2(acc[b][i4 * 4 + 2] * inv, acc[b][i4 * 4 + 3] * inv);
      *(u32x2_t*)(orow + d0) = st;
    }
  if (g == 0) lse[(size_t)bh * M + qi] = (m_run + log2f(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool POS>
static hipError_t launch_fp8_d(const Fp8LaunchArgs& a) {
  constexpr int BM = Fp8Cfg<D>::BM;
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL, POS>), dim3((unsigned)(tiles_m * a.BH)),
                     dim3(512), 0, a.stream, (const uint8_t*)a.q, (const uint8_t*)a.k,
                     (const uint8_t*)a.vt, (uint16_t*)a.o, a.lse, (int)a.M, (int)a.N, tiles_m,
                     (int)a.BH, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fp8_dispatch(const Fp8LaunchArgs& a) {
  const bool pos = a.scale > 0.0f;
  if (a.causal) return pos ? launch_fp8_d<D, true, true>(a) : launch_fp8_d<D, true, false>(a);
  return pos ? launch_fp8_d<D, false, true>(a) : launch_fp8_d<D, false, false>(a);
}

hipError_t launch_fp8(const Fp8LaunchArgs& a) {
  switch (a.D) {
    case 64: return launch_fp8_dispatch<64>(a);
    case 128: return launch_fp8_dispatch<128>(a);
    default: return hipErrorInvalidValue;
  }
}

int fp8_tile_rows() { return Fp8Cfg<64>::BM; }

}  // namespace mi355
