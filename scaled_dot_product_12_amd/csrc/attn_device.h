// attn_device.h -- device-side building blocks shared by the gfx950
// attention kernels: vector types, MFMA wrappers, wave64 half exchanges,
// bf16 packing and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// log2(e) and ln(2) in fp32. The kernels run the softmax in base 2
// (exp2 of log2(e)-scaled scores), the form used by the Blackwell attention
// example, and convert the row logsumexp back to the natural log at the end.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// Lazy-rescale threshold in the log2 domain: the running reference max is
// only moved (and O, l rescaled) once a row max exceeds it by more than this,
// so the unnormalised probabilities stay below 2^8.
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b,
                                                        f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_32x32x16_f16(f16x8_t a, f16x8_t b,
                                                       f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_32x32x2_f32(float a, float b,
                                                      f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Lanes l and l^32 of a wave64 hold the two halves of one query row in the
// kernels' layouts. permlane32_swap exchanges the halves; after a swap of x
// with itself the two results at every lane are {x[l], x[l^32]} in some
// order, so a symmetric combine of the pair is the half-pair combine.
__device__ __forceinline__ float half_pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round two fp32 values to bf16 (nearest-even) and pack them, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// Round two fp32 values to fp16 (nearest-even) and pack them, lo first.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  const f16x2_t h = __builtin_convertvector(f, f16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// The two 16-bit input types (bf16, fp16) differ only in the matrix
// instruction, the rounding of P, dS and outputs, the row-sum dot product and
// the widening of stored elements. Operands are carried as raw 16-bit lanes.
template <bool F16>
struct Half16 {
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (F16)
      return mfma_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c);
    else
      return mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                c);
  }
  __device__ static f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return mma(__builtin_bit_cast(u32x4_t, a), __builtin_bit_cast(u32x4_t, b), c);
  }
  // Round (p0, p1) to the input type, add the rounded pair to rs, return it packed.
  __device__ static uint32_t round_sum(float p0, float p1, float& rs) {
    const f32x2_t f = {p0, p1};
    if constexpr (F16) {
      const f16x2_t h = __builtin_convertvector(f, f16x2_t);
      const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
      rs = __builtin_amdgcn_fdot2(h, one, rs, false);
      return __builtin_bit_cast(uint32_t, h);
    } else {
      const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
      const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
      rs = __builtin_amdgcn_fdot2_f32_bf16(b, one, rs, false);
      return __builtin_bit_cast(uint32_t, b);
    }
  }
  __device__ static uint32_t pack(float lo, float hi) {
    return F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
  }
  // The low / high element of a packed pair, widened to fp32 (exact).
  __device__ static float lo(uint32_t w) {
    if constexpr (F16) return (float)__builtin_bit_cast(f16x2_t, w)[0];
    else return __uint_as_float(w << 16);
  }
  __device__ static float hi(uint32_t w) {
    if constexpr (F16) return (float)__builtin_bit_cast(f16x2_t, w)[1];
    else return __uint_as_float(w & 0xffff0000u);
  }
};

// Work-item and workgroup index from the hardware registers. The kernels are
// built with -mno-amdgpu-ieee, which the device library's threadIdx/blockIdx
// accessors are not, so those accessors stay out-of-line calls; the builtins
// below are single register reads.
__device__ __forceinline__ int workitem_id() {
  return (int)__builtin_amdgcn_workitem_id_x();
}
__device__ __forceinline__ int workgroup_id() {
  return (int)__builtin_amdgcn_workgroup_id_x();
}

// Wave-uniform "does any lane want this".
__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Workgroups are handed to the 8 XCDs round-robin by workgroup id, and each
// XCD has its own L2. Renumber them so that the ids one XCD receives form one
// contiguous logical range: neighbouring logical tiles (the query tiles of one
// head, which read the same K/V) then share an L2. Bijective for any count.
__device__ __forceinline__ int xcd_contiguous_id(int wg, int count) {
  const int xcd = wg & 7;
  const int idx = wg >> 3;
  const int per = count >> 3;
  const int rem = count & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// (head, query tile) of a workgroup. Each XCD gets whole heads (their query
// tiles share K/V in its L2). Non-causal: the tiles of one head are
// consecutive. Causal, when the heads split evenly over the XCDs: each XCD
// runs the longest query tiles of all its heads first, then the next
// longest, so the short tiles fill the tail; otherwise heads in order, each
// longest tile first. Bijective onto heads x tiles for any count.
struct TileId {
  int bh, tm;
};
__device__ __forceinline__ TileId tile_order(int wg, int tiles_m, int heads, bool causal) {
  const int count = tiles_m * heads;
  if (causal && (heads & 7) == 0) {
    const int hpx = heads >> 3;  // heads per XCD
    const int xcd = wg & 7, idx = wg >> 3;
    return {xcd * hpx + idx % hpx, tiles_m - 1 - idx / hpx};
  }
  const int wl = xcd_contiguous_id(wg, count);
  const int bh = wl / tiles_m;
  const int tm = wl - bh * tiles_m;
  return {bh, causal ? tiles_m - 1 - tm : tm};
}

}  // namespace mi355
