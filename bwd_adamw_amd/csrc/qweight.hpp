// Block-quantized frozen W, decoded to bf16 while the GEMMs stage it.
//
// W [N, K] is stored as planes (one array per field) in one buffer, each
// plane starting at a 256-byte boundary, in this order:
//   Q8_0  qs int8 [N,K]          d fp16 [N,K/32]                  w = d q
//   Q4_0  qs u4   [N,K]          d fp16 [N,K/32]                  w = d (q - 8)
//   Q4_K  qs u4   [N,K]          sm u8 [N,K/32][2] (sc, mn < 64)  w = d sc q - dmin mn
//         dm fp16 [N,K/256][2] (d, dmin)
//   Q6_K  ql u4   [N,K]          qh u2 [N,K]   sc int8 [N,K/16]   w = d sc (q - 32),
//         d fp16 [N,K/256]                                        q = ql | qh << 4
// u4 planes hold element 2j in the low nibble of byte j and 2j+1 in the
// high nibble; the u2 plane holds element 4j+i in bits 2i..2i+1 of byte j.
// (The block arithmetic is that of the GGUF formats of the same names;
// frozen-weight training over such a base: "8. LoRA Fundamentals" (Juno
// docs), opening paragraph and "Training decisions"; the pages' own
// quantized backward paths: "Backward Bug Hunts and Vulkan Tiled GEMM",
// "The fix".)
//
// Both GEMM directions stage W as runs of 8 consecutive elements of one W
// row (the forward's contraction chunks; a dX tile's rows), so one load and
// one decode serve both.  Every element is a * q + b with a, b fixed per
// sub-block: computed in float32 (exact except the one rounding of Q4_K's
// sum), then rounded to bf16 (nearest even).
#pragma once
#include "common.hpp"

namespace lora {

// Values of lora_dtype.
constexpr int WQ_BF16 = 1, WQ_Q8_0 = 2, WQ_Q4_0 = 3, WQ_Q4_K = 4, WQ_Q6_K = 5;

LORA_HD constexpr bool wq_quantized(int f) { return f >= WQ_Q8_0 && f <= WQ_Q6_K; }
// Elements sharing the fp16 scale(s): K must be a multiple of it.
LORA_HD constexpr int wq_super(int f) { return f == WQ_Q4_K || f == WQ_Q6_K ? 256 : 32; }
// 32-bit words of one staged 8-element run.
LORA_HD constexpr int wq_words(int f) {
  return f == WQ_Q8_0 ? 3 : f == WQ_Q4_0 ? 2 : f == WQ_Q4_K ? 3 : 4;
}
// Bytes per row of plane i (0 when the format has no plane i).
LORA_HD inline int64_t wq_plane_row_bytes(int f, int i, int64_t K) {
  switch (f) {
    case WQ_Q8_0: return i == 0 ? K : i == 1 ? K / 16 : 0;
    case WQ_Q4_0: return i == 0 ? K / 2 : i == 1 ? K / 16 : 0;
    case WQ_Q4_K: return i == 0 ? K / 2 : i == 1 ? K / 16 : i == 2 ? K / 64 : 0;
    case WQ_Q6_K: return i == 0 ? K / 2 : i == 1 ? K / 4 : i == 2 ? K / 16 : K / 128;
    default: return 0;
  }
}

// The planes of one quantized W as buffer resources (hardware bounds: a
// read past a plane's end returns zero, which decodes to a zero weight).
struct QPlanes {
  const uint8_t* p[4];
  uint32_t bytes[4];
};

template <int F>
struct QRes {
  __amdgpu_buffer_rsrc_t r[4];
  LORA_DEV explicit QRes(const QPlanes& q) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_amdgcn_make_buffer_rsrc((void*)q.p[i], (short)0, (int)q.bytes[i],
                                               0x00020000);
  }
};

// Raw words of elements [col, col + 8) of W row `row` (col a multiple of 8,
// K the row length).  Offsets are 32-bit: every plane is below 2^30 bytes.
// ok = false reads from past every plane: the run decodes to zeros.
template <int F>
LORA_DEV void wq_load(const QRes<F>& R, uint32_t K, uint32_t row, uint32_t col, uint32_t* w,
                      bool ok = true) {
  auto o = [&](uint32_t x) { return ok ? x : 0xfffffff0u; };
  if constexpr (F == WQ_Q8_0) {
    const u32x2 c = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(R.r[0], o(row * K + col), 0, 0));
    w[0] = c.x;
    w[1] = c.y;
    w[2] = __builtin_amdgcn_raw_buffer_load_b16(R.r[1], o(row * (K / 16) + (col / 32) * 2), 0, 0);
  } else if constexpr (F == WQ_Q4_0) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(R.r[0], o(row * (K / 2) + col / 2), 0, 0);
    w[1] = __builtin_amdgcn_raw_buffer_load_b16(R.r[1], o(row * (K / 16) + (col / 32) * 2), 0, 0);
  } else if constexpr (F == WQ_Q4_K) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(R.r[0], o(row * (K / 2) + col / 2), 0, 0);
    w[1] = __builtin_amdgcn_raw_buffer_load_b16(R.r[1], o(row * (K / 16) + (col / 32) * 2), 0, 0);
    w[2] = __builtin_amdgcn_raw_buffer_load_b32(R.r[2], o(row * (K / 64) + (col / 256) * 4), 0, 0);
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(R.r[0], o(row * (K / 2) + col / 2), 0, 0);
    w[1] = __builtin_amdgcn_raw_buffer_load_b16(R.r[1], o(row * (K / 4) + col / 4), 0, 0);
    w[2] = __builtin_amdgcn_raw_buffer_load_b8(R.r[2], o(row * (K / 16) + col / 16), 0, 0);
    w[3] = __builtin_amdgcn_raw_buffer_load_b16(R.r[3], o(row * (K / 128) + (col / 256) * 2), 0, 0);
  }
}

LORA_DEV float wq_h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// The 8 weights of a staged run, as float32.
template <int F>
LORA_DEV void wq_decode(const uint32_t* w, float* v) {
  if constexpr (F == WQ_Q8_0) {
    const float d = wq_h2f(w[2]);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = d * (float)(int8_t)(w[e / 4] >> (8 * (e % 4)));
  } else if constexpr (F == WQ_Q6_K) {
    const float a = wq_h2f(w[3]) * (float)(int8_t)w[2];
    const float b = -32.0f * a;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t q = ((w[0] >> (4 * e)) & 15u) | (((w[1] >> (2 * e)) & 3u) << 4);
      v[e] = __builtin_fmaf(a, (float)q, b);
    }
  } else {
    float a, b;
    if constexpr (F == WQ_Q4_0) {
      a = wq_h2f(w[1]);
      b = -8.0f * a;
    } else {
      a = wq_h2f(w[2] & 0xffffu) * (float)(w[1] & 0xffu);
      b = -(wq_h2f(w[2] >> 16) * (float)((w[1] >> 8) & 0xffu));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(a, (float)((w[0] >> (4 * e)) & 15u), b);
  }
}

// Two floats as packed bf16 (nearest even), low element first.
LORA_DEV uint32_t wq_pack(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace lora
