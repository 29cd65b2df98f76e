// Frozen-weight GEMMs with bf16 W on bf16 MFMA (v_mfma_f32_32x32x16_bf16),
// float32 accumulation.  Same contractions as gemm_f32.hpp:
//   forward: Z = Xb W^T + s U B^T                 (Xb = bf16(X), written by down)
//   dX     : dX = gb W + (s V A) * mask * keep    (gb = bf16(g), written by k3)
// The LoRA operands (U, B, V, A: float32) are rounded to bf16 while staging;
// U and V may arrive as split partials, summed in split order while staging.
//
// Block: 512 threads = 2 x 4 waves over a BM x BN tile (256x256, 256x128 or
// 128x128), K-step 64, LDS double buffered.  LDS holds both operands as
// [row][contraction] bf16 with a 16-byte pad, so every MFMA operand is one
// 128-bit LDS read: lane half h takes contraction indices 32h..32h+31 of the
// K-step.  For dX the W tile arrives with the contraction index as its row
// (W's native [N,K] layout); each thread loads an 8-row x 4-column block and
// transposes it in registers before the LDS write.
//
// The grid is one-dimensional.  Workgroups are dealt to the 8 XCDs round
// robin, so block b runs on XCD b % 8, and each XCD starts its blocks in
// order.  Block b is mapped to a contiguous run of tile indices per XCD, and
// tile indices walk the output in groups of GROUP_M tile rows, column by
// column, so the tiles an XCD has resident at once form a compact rectangle
// whose A and B K-slices are shared in that XCD's L2.
#pragma once
#include "common.hpp"
#include "gemm_f32.hpp"   // LoraOperand

namespace lora {

struct GemmBf16Args {
  const uint16_t* A;       // [M, Kc] bf16, contraction contiguous
  int64_t lda;
  const uint16_t* B;       // fwd: W [Nc, Kc];  dx: W [Kc, Nc]   (bf16)
  int64_t ldb;
  int64_t M, Nc, Kc;
  LoraOperand xa;          // U (fwd) or V (dx), float32 [M, r], possibly as partials
  const float* XB;         // fwd: B_lora [Nc, r];  dx: A_lora [r, Nc]  (float32)
  int64_t r;
  float xs;
  DropParams drop;
  float* C;
  float* C2;
  const float* cn;
  const float* cd;
};

LORA_DEV uint32_t lo16(uint32_t x) { return x & 0xffffu; }
LORA_DEV uint32_t hi16(uint32_t x) { return x >> 16; }

// EXACT: M, Nc and Kc are multiples of BM, BN and 64, so the main loop runs
// without bounds checks (no divergent branches around its loads).
template <int BM, int BN, bool FWD, bool EXACT>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(GemmBf16Args p) {
  constexpr int NT = 512;
  constexpr int BK = 64;
  constexpr int LDS_ROW = BK + 8;                   // bf16 elements per LDS row (144 B)
  constexpr int WGM = 2, WGN = 4;
  constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
  constexpr int ACH = BM * (BK / 8) / NT;           // 16-byte A chunks per thread
  constexpr int BCH = BN * (BK / 8) / NT;           // 16-byte B chunks per thread (fwd)
  constexpr int BITEMS = (BK / 8) * (BN / 4);       // transposed 8x4 blocks (dx)
  constexpr int BIT = (BITEMS + NT - 1) / NT;
  static_assert(ACH >= 1 && BCH >= 1 && MI >= 1 && NI >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDS_ROW];
  auto As = [&](int b) -> uint16_t* { return smem + b * (BM * LDS_ROW); };
  auto Bs = [&](int b) -> uint16_t* { return smem + 2 * BM * LDS_ROW + b * (BN * LDS_ROW); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int64_t ntn = (p.Nc + BN - 1) / BN, ntm = (p.M + BM - 1) / BM;
  int64_t tm, tn;
  grouped_tile(xcd_tile(blockIdx.x, ntm * ntn), ntm, ntn, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t kend = p.Kc;
  const int hl = lane >> 5, l32 = lane & 31;
  const bool store_xa = p.xa.out != nullptr && n0 == 0;

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  u32x4 ra[ACH];
  u32x4 rbf[FWD ? BCH : 1];
  u32x2 rbt[FWD ? 1 : BIT][8];

  // 8 contiguous bf16 at src[row*ld + k .. +8), zero beyond klim (klim % 8 == 0).
  auto ld8 = [&](const uint16_t* src, int64_t row, int64_t rows, int64_t ld, int64_t k,
                 int64_t klim) -> u32x4 {
    if (EXACT) return *reinterpret_cast<const u32x4*>(src + row * ld + k);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows && k < klim) v = *reinterpret_cast<const u32x4*>(src + row * ld + k);
    return v;
  };
  auto load_a = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int f = tid + NT * q;
      ra[q] = ld8(p.A, m0 + (f >> 3), p.M, p.lda, k0 + 8 * (f & 7), kend);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int f = tid + NT * q;
      *reinterpret_cast<u32x4*>(&As(buf)[(f >> 3) * LDS_ROW + 8 * (f & 7)]) = ra[q];
    }
  };
  auto load_b = [&](int64_t k0) {
    if constexpr (FWD) {
#pragma unroll
      for (int q = 0; q < BCH; ++q) {
        const int f = tid + NT * q;
        rbf[q] = ld8(p.B, n0 + (f >> 3), p.Nc, p.ldb, k0 + 8 * (f & 7), kend);
      }
    } else {
#pragma unroll
      for (int q = 0; q < BIT; ++q) {
        const int f = tid + NT * q;
        const int cq = f % (BN / 4), kg = f / (BN / 4);
        const int64_t gn = n0 + 4 * cq;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t gk = k0 + 8 * kg + i;
          u32x2 v = {0u, 0u};
          if (EXACT ? (f < BITEMS) : (f < BITEMS && gk < kend && gn < p.Nc))
            v = *reinterpret_cast<const u32x2*>(p.B + gk * p.ldb + gn);
          rbt[q][i] = v;
        }
      }
    }
  };
  // Transposed write: column e of the 8x4 block becomes 8 contraction values.
  auto store_bt = [&](int buf, int q, const u32x2 (&w)[8]) {
    const int f = tid + NT * q;
    if (f >= BITEMS) return;
    const int cq = f % (BN / 4), kg = f / (BN / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t x0 = (e < 2) ? w[2 * d].x : w[2 * d].y;
        const uint32_t x1 = (e < 2) ? w[2 * d + 1].x : w[2 * d + 1].y;
        o[d] = (e & 1) ? (hi16(x0) | (hi16(x1) << 16)) : (lo16(x0) | (lo16(x1) << 16));
      }
      *reinterpret_cast<u32x4*>(&Bs(buf)[(4 * cq + e) * LDS_ROW + 8 * kg]) = o;
    }
  };
  auto store_b = [&](int buf) {
    if constexpr (FWD) {
#pragma unroll
      for (int q = 0; q < BCH; ++q) {
        const int f = tid + NT * q;
        *reinterpret_cast<u32x4*>(&Bs(buf)[(f >> 3) * LDS_ROW + 8 * (f & 7)]) = rbf[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < BIT; ++q) store_bt(buf, q, rbt[q]);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 av[MI], bv[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        av[i] = *reinterpret_cast<const u32x4*>(
            &As(buf)[(wm0 + i * 32 + l32) * LDS_ROW + 32 * hl + 8 * s]);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        bv[j] = *reinterpret_cast<const u32x4*>(
            &Bs(buf)[(wn0 + j * 32 + l32) * LDS_ROW + 32 * hl + 8 * s]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = mfma32x32x16_bf16(av[i], bv[j], acc[i][j]);
    }
  };
  // LoRA contraction over the rank: float32 operands rounded to bf16 in LDS.
  auto lora_contraction = [&]() {
    for (int64_t k0 = 0; k0 < p.r; k0 += BK) {
      __syncthreads();
      // A side: XA [M, r] rows m (split partials summed), scaled by s.
      for (int f = tid; f < BM * (BK / 4); f += NT) {
        const int row = f / (BK / 4), c4 = f % (BK / 4);
        const int64_t gm = m0 + row, gk = k0 + 4 * c4;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gm < p.M && gk < p.r) {
          const int64_t i = gm * p.r + gk;
          v = sum_parts4(p.xa.p, p.xa.stride, p.xa.nparts, i);
          if (store_xa && p.xa.nparts > 1) *reinterpret_cast<f32x4*>(p.xa.out + i) = v;
          v *= p.xs;
        }
        u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(&As(0)[row * LDS_ROW + 4 * c4]) = b;
      }
      if constexpr (FWD) {
        // B_lora [Nc, r]: rows n, rank contiguous.
        for (int f = tid; f < BN * (BK / 4); f += NT) {
          const int row = f / (BK / 4), c4 = f % (BK / 4);
          const int64_t gn = n0 + row, gk = k0 + 4 * c4;
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
          if (gn < p.Nc && gk < p.r) v = *reinterpret_cast<const f32x4*>(p.XB + gn * p.r + gk);
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(&Bs(0)[row * LDS_ROW + 4 * c4]) = b;
        }
      } else {
        // A_lora [r, Nc]: rows are the contraction index; transpose on store.
        for (int f = tid; f < BN * BK; f += NT) {
          const int n = f % BN, kk = f / BN;
          const int64_t gn = n0 + n, gk = k0 + kk;
          float v = 0.f;
          if (gn < p.Nc && gk < p.r) v = p.XB[gk * p.Nc + gn];
          Bs(0)[n * LDS_ROW + kk] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
      __syncthreads();
      compute(0);
    }
    __syncthreads();
  };

  if (!FWD && p.r > 0) {
    lora_contraction();
    if (p.drop.on) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t gm = m0 + wm0 + i * 32 + row32(v, lane);
          const uint64_t rk = drop_row(p.drop, gm);
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int64_t gn = n0 + wn0 + j * 32 + l32;
            acc[i][j][v] *= drop_mul(p.drop, rk, gn);
          }
        }
    }
  }

  const int64_t nk = (kend + BK - 1) / BK;
  load_a(0);
  load_b(0);
  store_a(0);
  store_b(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) {
      load_a((kt + 1) * BK);
      load_b((kt + 1) * BK);
    }
    compute(cur);
    if (kt + 1 < nk) {
      store_a(cur ^ 1);
      store_b(cur ^ 1);
    }
    __syncthreads();
  }

  if (FWD && p.r > 0) lora_contraction();

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t gn = n0 + wn0 + j * 32 + l32;
      if (gn >= p.Nc) continue;
      const float c = p.cn ? p.cn[gn] / p.cd[gn] : 1.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gm = m0 + wm0 + i * 32 + row32(v, lane);
        if (gm >= p.M) continue;
        const float x = acc[i][j][v];
        p.C[gm * p.Nc + gn] = x * c;
        if (p.C2) p.C2[gm * p.Nc + gn] = x;
      }
    }
}

}  // namespace lora
