// Frozen-weight GEMMs with float32 W on fp32 MFMA (v_mfma_f32_32x32x2f32).
//
// Forward ("8. LoRA Fundamentals", "How it works"):
//   Z[t,n] = sum_k X[t,k] W[n,k]  +  s * sum_j U[t,j] B[n,j]
// The rank-r up-projection is a second, short contraction into the same
// accumulators, staged through LDS after the main loop.
//
// dX ("Training decisions"; "Backward Bug Hunts ...", "Bug #1"):
//   dX[t,k] = sum_n g[t,n] W[n,k]  +  (s * sum_j V[t,j] A[j,k]) * mask * keep
// W is read in its native [N,K] layout (rows of W are the contraction
// index); nothing is transposed in memory.  The LoRA term is contracted
// first, masked in registers, then the frozen contraction accumulates on top.
//
// The LoRA operand U (forward) or V (dX) may arrive as split partials from
// the rank-side kernels; they are summed in split order while staging, and
// the forward stores the summed U once (blocks of column tile 0).
//
// Block: 256 threads = 2x2 waves, tile BM x BN, K-step 32, LDS double
// buffered.  Within a K-step lane half h takes contraction indices
// 16h..16h+15 so A (and, forward, B) operands are 128-bit LDS reads.
// Short-M shapes split the contraction across blocks (grid z): each split
// writes a partial tile and splitk_reduce_kernel sums them in split order and
// applies the epilogue.  The LoRA contraction belongs to split 0.
#pragma once
#include "common.hpp"

namespace lora {

// LoRA operand of the A side: nparts partials [nparts][M][r] summed in order
// (nparts == 1: the operand itself).  `out`, when set, receives the sum.
struct LoraOperand {
  const float* p;
  int64_t stride;
  int nparts;
  float* out;
};

struct GemmF32Args {
  const float* A;          // [M, Kc] contraction contiguous (X or dY)
  int64_t lda;
  const float* acn;        // per-contraction multiplier num/den on A (DoRA g), or NULL
  const float* acd;
  const float* B;          // fwd: W [Nc, Kc];  dx: W [Kc, Nc]
  int64_t ldb;
  int64_t M, Nc, Kc;
  LoraOperand xa;          // U (fwd) or V (dx), [M, r]
  const float* XB;         // fwd: B_lora [Nc, r];  dx: A_lora [r, Nc]
  int64_t r;
  float xs;                // LoRA scale s
  DropParams drop;         // dx only: mask of the LoRA term at (t = m, k = n)
  int64_t ksplit;          // contraction length per split (multiple of 32)
  int nsplit;
  float* C;                // Y or dX, [M, Nc] (nsplit == 1)
  float* C2;               // fwd DoRA: Z, or NULL
  const float* cn;         // fwd DoRA epilogue column scale cn/cd, or NULL
  const float* cd;
  float* part;             // [nsplit, M, Nc] partials when nsplit > 1
};

// LDS floats of one block (double-buffered A and B stages).
template <int BM, int BN, bool FWD>
constexpr int gemm_f32_lds_floats() {
  return 2 * BM * (32 + 4) + 2 * (FWD ? BN * (32 + 4) : 32 * (BN + 4));
}

// One output tile (tm, tn) of split `split`, in LDS `smem`
// (gemm_f32_lds_floats<BM, BN, FWD>() floats).
//
// The main loop keeps DEPTH K-steps of global loads in flight in registers:
// a K-step's operands take longer to arrive than one K-step of MFMA work, so
// the load for step k + DEPTH is issued while step k is computed.  At step k
// LDS buffer k%2 holds step k, register stage (k+1)%DEPTH holds step k+1 and
// is stored to the other buffer after the MFMAs, and stage k%DEPTH (stored
// one step earlier) is refilled.  The loop is unrolled by DEPTH so every
// stage index is a compile-time constant.
//
// EXACT: M and Nc are multiples of BM and BN and every split range a multiple
// of 32, so the main loop runs without bounds checks.
template <int BM, int BN, bool FWD, bool EXACT, int DEPTH>
LORA_DEV void gemm_f32_block(const GemmF32Args& p, float* smem, int64_t tn, int64_t tm,
                             int split) {
  constexpr int BK = 32;
  constexpr int KW = BK;                // contraction indices per wave per K-step
  constexpr int KH = KW / 2;            // per lane half
  constexpr int LDA = BK + 4;
  constexpr int LDB = FWD ? (BK + 4) : (BN + 4);
  constexpr int BSZ = FWD ? BN * LDB : BK * LDB;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int AF4 = BM * BK / 4 / 256;
  constexpr int BF4 = BN * BK / 4 / 256;
  constexpr int AC4 = BK / 4;           // float4 per A row of a K-step
  static_assert(AF4 >= 1 && BF4 >= 1 && MI >= 1 && NI >= 1, "tile shape");
  static_assert(KH % 4 == 0, "lane-half slice must be whole float4s");
  static_assert(DEPTH >= 2, "at least one K-step of loads in flight");

  auto As = [&](int b) -> float* { return smem + b * (BM * LDA); };
  auto Bs = [&](int b) -> float* { return smem + 2 * BM * LDA + b * BSZ; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t kbeg = (int64_t)split * p.ksplit;
  const int64_t kend = min(p.Kc, kbeg + p.ksplit);
  const int hl = lane >> 5, l32 = lane & 31;
  const bool store_xa = p.xa.out != nullptr && tn == 0 && split == 0;

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  struct Stage {
    f32x4 a[AF4], b[BF4];
  };

  // A side (main operand): rows m, contraction contiguous.
  auto load_a = [&](Stage& S, int64_t k0) {
#pragma unroll
    for (int q = 0; q < AF4; ++q) {
      const int f = tid + 256 * q;
      const int row = f / AC4, c4 = f % AC4;
      const int64_t gm = m0 + row, gk = k0 + 4 * c4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (EXACT || (gm < p.M && gk < kend)) {
        v = *reinterpret_cast<const f32x4*>(p.A + gm * p.lda + gk);
        if (p.acn) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= p.acn[gk + e] / p.acd[gk + e];
        }
      }
      S.a[q] = v;
    }
  };
  // A side (LoRA operand): rows m, rank contiguous, partials summed, times s.
  auto load_xa = [&](Stage& S, int64_t k0) {
#pragma unroll
    for (int q = 0; q < AF4; ++q) {
      const int f = tid + 256 * q;
      const int row = f / AC4, c4 = f % AC4;
      const int64_t gm = m0 + row, gk = k0 + 4 * c4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (gm < p.M && gk < p.r) {
        const int64_t i = gm * p.r + gk;
        v = sum_parts4(p.xa.p, p.xa.stride, p.xa.nparts, i);
        if (store_xa && p.xa.nparts > 1) *reinterpret_cast<f32x4*>(p.xa.out + i) = v;
        v *= p.xs;
      }
      S.a[q] = v;
    }
  };
  auto store_a = [&](const Stage& S, int buf) {
#pragma unroll
    for (int q = 0; q < AF4; ++q) {
      const int f = tid + 256 * q;
      const int row = f / AC4, c4 = f % AC4;
      *reinterpret_cast<f32x4*>(&As(buf)[row * LDA + 4 * c4]) = S.a[q];
    }
  };
  // B side.  fwd: rows n, contraction contiguous.  dx: rows = contraction.
  auto load_b = [&](Stage& S, const float* src, int64_t ld, int64_t k0, int64_t klim, bool exact) {
#pragma unroll
    for (int q = 0; q < BF4; ++q) {
      const int f = tid + 256 * q;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (FWD) {
        const int row = f / AC4, c4 = f % AC4;
        const int64_t gn = n0 + row, gk = k0 + 4 * c4;
        if (exact || (gn < p.Nc && gk < klim)) v = *reinterpret_cast<const f32x4*>(src + gn * ld + gk);
      } else {
        const int row = f / (BN / 4), c4 = f % (BN / 4);
        const int64_t gk = k0 + row, gn = n0 + 4 * c4;
        if (exact || (gk < klim && gn < p.Nc)) v = *reinterpret_cast<const f32x4*>(src + gk * ld + gn);
      }
      S.b[q] = v;
    }
  };
  auto store_b = [&](const Stage& S, int buf) {
#pragma unroll
    for (int q = 0; q < BF4; ++q) {
      const int f = tid + 256 * q;
      if (FWD) {
        const int row = f / AC4, c4 = f % AC4;
        *reinterpret_cast<f32x4*>(&Bs(buf)[row * LDB + 4 * c4]) = S.b[q];
      } else {
        const int row = f / (BN / 4), c4 = f % (BN / 4);
        *reinterpret_cast<f32x4*>(&Bs(buf)[row * LDB + 4 * c4]) = S.b[q];
      }
    }
  };
  auto compute = [&](int buf) {
    const int kb = KH * hl;
    f32x4 av[MI][KH / 4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < KH / 4; ++q)
        av[i][q] = *reinterpret_cast<const f32x4*>(&As(buf)[(wm0 + i * 32 + l32) * LDA + kb + 4 * q]);
    if (FWD) {
      f32x4 bv[NI][KH / 4];
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int q = 0; q < KH / 4; ++q)
          bv[j][q] = *reinterpret_cast<const f32x4*>(&Bs(buf)[(wn0 + j * 32 + l32) * LDB + kb + 4 * q]);
#pragma unroll
      for (int s = 0; s < KH; ++s)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = mfma32x32x2(av[i][s >> 2][s & 3], bv[j][s >> 2][s & 3], acc[i][j]);
    } else {
#pragma unroll
      for (int s = 0; s < KH; ++s) {
        float bv[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) bv[j] = Bs(buf)[(kb + s) * LDB + wn0 + j * 32 + l32];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = mfma32x32x2(av[i][s >> 2][s & 3], bv[j], acc[i][j]);
      }
    }
  };
  // Unpipelined contraction over the LoRA rank (r <= 128).
  auto lora_contraction = [&]() {
    Stage S;
    for (int64_t k0 = 0; k0 < p.r; k0 += BK) {
      load_xa(S, k0);
      load_b(S, p.XB, FWD ? p.r : p.Nc, k0, p.r, false);
      __syncthreads();
      store_a(S, 0);
      store_b(S, 0);
      __syncthreads();
      compute(0);
    }
    __syncthreads();
  };

  const bool lora = split == 0 && p.r > 0 && p.XB != nullptr;
  if (!FWD && lora) {
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

  // Main contraction over [kbeg, kend).
  const int64_t nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    Stage R[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
      if (u < nk) {
        load_a(R[u], kbeg + u * BK);
        load_b(R[u], p.B, p.ldb, kbeg + u * BK, kend, EXACT);
      }
    store_a(R[0], 0);
    store_b(R[0], 0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; kt += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int64_t k = kt + u;
        if (k < nk) {
          if (k + DEPTH < nk) {
            load_a(R[u], kbeg + (k + DEPTH) * BK);
            load_b(R[u], p.B, p.ldb, kbeg + (k + DEPTH) * BK, kend, EXACT);
          }
          const int buf = (int)(k & 1);
          compute(buf);
          if (k + 1 < nk) {
            store_a(R[(u + 1) % DEPTH], buf ^ 1);
            store_b(R[(u + 1) % DEPTH], buf ^ 1);
          }
          __syncthreads();
        }
      }
    }
  }

  if (FWD && lora) lora_contraction();

  // Epilogue.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t gn = n0 + wn0 + j * 32 + l32;
      if (gn >= p.Nc) continue;
      const float c = (p.nsplit == 1 && p.cn) ? p.cn[gn] / p.cd[gn] : 1.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t gm = m0 + wm0 + i * 32 + row32(v, lane);
        if (gm >= p.M) continue;
        const float x = acc[i][j][v];
        if (p.nsplit == 1) {
          p.C[gm * p.Nc + gn] = x * c;
          if (p.C2) p.C2[gm * p.Nc + gn] = x;
        } else {
          p.part[((int64_t)split * p.M + gm) * p.Nc + gn] = x;
        }
      }
    }
}

// K-steps of loads in flight per tile size (register budget of a stage).
template <int BM, int BN>
constexpr int gemm_f32_depth() {
  return BM * BN <= 64 * 64 ? 4 : 2;
}

// Grid (Nc/BN, M/BM, nsplit).
template <int BM, int BN, bool FWD, bool EXACT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args p) {
  __shared__ __attribute__((aligned(16))) float smem[gemm_f32_lds_floats<BM, BN, FWD>()];
  gemm_f32_block<BM, BN, FWD, EXACT, gemm_f32_depth<BM, BN>()>(p, smem, blockIdx.x, blockIdx.y,
                                                                 blockIdx.z);
}

// Sum of the split partials in split order, then the epilogue of the unsplit
// kernel (Z = sum; Y = sum * cn/cd per column).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int nsplit,
                                                            int64_t M, int64_t Nc, float* C,
                                                            float* C2, const float* cn,
                                                            const float* cd) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = M * Nc;
  if (i4 >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i4);
  for (int q = 1; q < nsplit; ++q) s += *reinterpret_cast<const f32x4*>(part + q * total + i4);
  if (C2) *reinterpret_cast<f32x4*>(C2 + i4) = s;
  if (cn) {
    const int64_t n = i4 % Nc;
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] *= cn[n + e] / cd[n + e];
  }
  *reinterpret_cast<f32x4*>(C + i4) = s;
}

}  // namespace lora
