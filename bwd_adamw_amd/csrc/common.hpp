// Device-side building blocks shared by the liblora kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LORA_DEV __device__ __forceinline__
#define LORA_HD __host__ __device__

namespace lora {

// ---------------------------------------------------------------------------
// Dropout hash ("4.3. Training Guide", "Dropout"): SplitMix64's output
// function (Steele, Lea & Flood 2014) applied to state z.  The host chains it
// over (seed, step, ordinal, layer, proj) into `base`; a row key is
// mix(base ^ t) and the element decision uses mix(row ^ k).
// ---------------------------------------------------------------------------
LORA_DEV uint64_t sm_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct DropParams {
  uint64_t base;   // chained key of (seed, step, ordinal, layer, proj)
  uint32_t thr;    // keep iff top-24 hash bits >= thr; thr == 0: keep all
  float keep;      // float(1/(1-p)), multiplier of kept elements
  int on;          // 0: dropout disabled
};

LORA_DEV uint64_t drop_row(const DropParams& d, int64_t t) {
  return sm_mix(d.base ^ (uint64_t)t);
}
LORA_DEV bool drop_keep(const DropParams& d, uint64_t row, int64_t k) {
  return (uint32_t)(sm_mix(row ^ (uint64_t)k) >> 40) >= d.thr;
}
// Multiplier of element (row key, k): keep ? keep-scale : 0.
LORA_DEV float drop_mul(const DropParams& d, uint64_t row, int64_t k) {
  return drop_keep(d, row, k) ? d.keep : 0.0f;
}

// ---------------------------------------------------------------------------
// bf16 <-> f32 (round to nearest even; NaN stays NaN)
// ---------------------------------------------------------------------------
// Written as a select: an early return for NaN became a divergent branch
// around every conversion.
LORA_DEV uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rn = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : rn;
}
LORA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
LORA_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------------------------
// MFMA wrappers.  Operand/result lane layouts (wave64):
//  32x32x2 f32 : a = A[l%32][l/32], b = B[l/32][l%32],
//                d[v] = D[8*(v/4) + 4*(l/32) + v%4][l%32]
//  16x16x4 f32 : a = A[l%16][l/16], b = B[l/16][l%16],
//                d[v] = D[4*(l/16) + v][l%16]
//  32x32x16 bf16: a = A[l%32][k-group l/32 (8 values)], b likewise,
//                d as for 32x32x2.
// The contraction index carried by a lane group only has to agree between
// the two operands, so kernels permute it freely to get wide LDS reads.
// ---------------------------------------------------------------------------
LORA_DEV f32x16 mfma32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
LORA_DEV f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
LORA_DEV f32x16 mfma32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

LORA_DEV int row32(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// Fragment-tiled bf16 operand (the A operand of the direct-operand bf16
// products, gemm_bf16.hpp): element offset of (row t, contraction index k)
// for a contraction of nkq * 64.  Each 1 KB is one MFMA operand in lane
// order: 32 rows x 16 indices of K-step k / 64, sub-step s = (k % 32) / 8,
// lane t % 32 + 32 ((k % 64) / 32) holding the 8 indices k - k % 8 .. +7.
// Rows stay contiguous in groups of 32, so stacked row ranges that start at
// multiples of 32 start at multiples of 32 * nkq * 64 elements.
LORA_HD inline int64_t atile_off(int64_t t, int64_t k, int64_t nkq) {
  return ((((t >> 5) * nkq + (k >> 6)) * 4 + ((k >> 3) & 3)) * 64 + (t & 31) + 32 * ((k >> 5) & 1)) * 8 +
         (k & 7);
}
LORA_DEV int row16(int v, int lane) { return 4 * (lane >> 4) + v; }

// Wave-wide sum of a double (butterfly over 64 lanes; every lane gets it).
LORA_DEV double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
LORA_DEV float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---------------------------------------------------------------------------
// Split reductions run in a fixed order; no floating-point atomics anywhere.
// ---------------------------------------------------------------------------
// Fixed-order sum of nparts partials of one element: (sum_p part[p*stride+i])
// * alpha (/ div), added to or stored into out[i].
LORA_DEV void sum_partials(const float* part, int64_t stride, int nparts, int64_t i, float alpha,
                           const float* div, int64_t divi, float* out, int accumulate) {
  float s = part[i];
  for (int q = 1; q < nparts; ++q) s += part[(int64_t)q * stride + i];
  s *= alpha;
  if (div) s /= div[divi];
  out[i] = accumulate ? out[i] + s : s;
}

// Fixed-order sum of nparts float4 partials at part[q*stride + i]: loads are
// issued sixteen at a time so their latencies overlap (one round trip for up
// to 17 partials); the additions still run in index order.  Every load is
// unconditional (past the last partial it repeats the last one's address and
// its value is not added): a guarded load becomes a branch, at whose join the
// compiler waits for every load in flight.
LORA_DEV f32x4 sum_parts4(const float* part, int64_t stride, int nparts, int64_t i) {
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
  for (int q = 1; q < nparts; q += 16) {
    f32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(part + (int64_t)min(q + u, nparts - 1) * stride + i);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const f32x4 t = s + v[u];
      s = q + u < nparts ? t : s;
    }
  }
  return s;
}

// The same for one float or double.
template <typename T>
LORA_DEV T sum_parts1(const T* part, int64_t stride, int nparts, int64_t i) {
  T s = part[i];
  for (int q = 1; q < nparts; q += 16) {
    T v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[(int64_t)min(q + u, nparts - 1) * stride + i];
#pragma unroll
    for (int u = 0; u < 16; ++u) s = q + u < nparts ? s + v[u] : s;
  }
  return s;
}

// ---------------------------------------------------------------------------
// Block -> tile order.  Workgroups of a launch are dealt to the 8 XCDs round
// robin (block b runs on XCD b % 8), so tiles that share operands are given
// to blocks of one XCD, where they share its L2.
// ---------------------------------------------------------------------------
// Tile index of linear block b: contiguous per XCD (a bijection on [0, T)).
LORA_DEV int64_t xcd_tile(int64_t b, int64_t T) {
  const int64_t q = T / 8, rem = T % 8;
  const int64_t x = b % 8, idx = b / 8;
  const int64_t start = x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q;
  return start + idx;
}

// Tile index g -> (tile row, tile col), walking groups of GROUP_M tile rows
// column by column (a bijection onto the ntm x ntn tiles).
constexpr int GROUP_M = 4;
LORA_DEV void grouped_tile(int64_t g, int64_t ntm, int64_t ntn, int64_t& tm, int64_t& tn) {
  const int64_t first = (g / (GROUP_M * ntn)) * GROUP_M;
  const int64_t gsize = min((int64_t)GROUP_M, ntm - first);
  const int64_t gin = g - first * ntn;
  tm = first + gin % gsize;
  tn = gin / gsize;
}

}  // namespace lora
