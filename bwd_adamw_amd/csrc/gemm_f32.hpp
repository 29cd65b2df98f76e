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
// stage index is a compile-time constant, and its body has no branches:
// every step issues its loads (past the last step they repeat the last
// step's addresses and are never stored), out-of-range elements are read
// from a valid address and zeroed when stored to LDS.  Straight-line code
// lets the compiler wait for exactly the stage it stores, with the newer
// stages still in flight.
//
// EXACT: M and Nc are multiples of BM and BN and every split range a multiple
// of 32, so nothing is out of range.  SCALEA: the A operand is multiplied per
// contraction index by acn/acd (DoRA g = dY * mag/norm in dX).
template <int BM, int BN, bool FWD, bool EXACT, int DEPTH, bool SCALEA>
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
  constexpr int NS = SCALEA ? AF4 : 1;
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
    f32x4 an[NS], ad[NS];
  };

  // Element coordinates of this thread's q-th float4 of a K-step at k0.
  auto a_at = [&](int q, int64_t k0, int64_t& gm, int64_t& gk) -> bool {
    const int f = tid + 256 * q;
    gm = m0 + f / AC4;
    gk = k0 + 4 * (f % AC4);
    return EXACT || (gm < p.M && gk < kend);
  };
  auto b_at = [&](int q, int64_t k0, int64_t& gr, int64_t& gc) -> bool {
    const int f = tid + 256 * q;
    if (FWD) {   // rows n, contraction contiguous
      gr = n0 + f / AC4;
      gc = k0 + 4 * (f % AC4);
      return EXACT || (gr < p.Nc && gc < kend);
    } else {     // rows = contraction, columns n
      gr = k0 + f / (BN / 4);
      gc = n0 + 4 * (f % (BN / 4));
      return EXACT || (gr < kend && gc < p.Nc);
    }
  };
  auto load = [&](Stage& S, int64_t k0) {
#pragma unroll
    for (int q = 0; q < AF4; ++q) {
      int64_t gm, gk;
      const bool ok = a_at(q, k0, gm, gk);
      S.a[q] = *reinterpret_cast<const f32x4*>(ok ? p.A + gm * p.lda + gk : p.A);
      if constexpr (SCALEA) {
        const int64_t kk = ok ? gk : 0;
        S.an[q] = *reinterpret_cast<const f32x4*>(p.acn + kk);
        S.ad[q] = *reinterpret_cast<const f32x4*>(p.acd + kk);
      }
    }
#pragma unroll
    for (int q = 0; q < BF4; ++q) {
      int64_t gr, gc;
      const bool ok = b_at(q, k0, gr, gc);
      S.b[q] = *reinterpret_cast<const f32x4*>(ok ? p.B + gr * p.ldb + gc : p.B);
    }
  };
  auto store = [&](const Stage& S, int64_t k0, int buf) {
#pragma unroll
    for (int q = 0; q < AF4; ++q) {
      int64_t gm, gk;
      const bool ok = a_at(q, k0, gm, gk);
      f32x4 v = S.a[q];
      if constexpr (SCALEA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= S.an[q][e] / S.ad[q][e];
      }
      if (!ok) v = f32x4{0.f, 0.f, 0.f, 0.f};
      const int f = tid + 256 * q;
      *reinterpret_cast<f32x4*>(&As(buf)[(f / AC4) * LDA + 4 * (f % AC4)]) = v;
    }
#pragma unroll
    for (int q = 0; q < BF4; ++q) {
      int64_t gr, gc;
      const bool ok = b_at(q, k0, gr, gc);
      const f32x4 v = ok ? S.b[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      const int f = tid + 256 * q;
      if (FWD)
        *reinterpret_cast<f32x4*>(&Bs(buf)[(f / AC4) * LDB + 4 * (f % AC4)]) = v;
      else
        *reinterpret_cast<f32x4*>(&Bs(buf)[(f / (BN / 4)) * LDB + 4 * (f % (BN / 4))]) = v;
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
  // Unpipelined contraction over the LoRA rank (r <= 128): the A side is
  // U or V (split partials summed, times s), the B side B_lora (forward,
  // [Nc, r]) or A_lora (dX, [r, Nc]); both masked while loading.
  auto lora_contraction = [&]() {
    for (int64_t k0 = 0; k0 < p.r; k0 += BK) {
      f32x4 ra[AF4], rb[BF4];
#pragma unroll
      for (int q = 0; q < AF4; ++q) {
        const int f = tid + 256 * q;
        const int64_t gm = m0 + f / AC4, gk = k0 + 4 * (f % AC4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gm < p.M && gk < p.r) {
          const int64_t i = gm * p.r + gk;
          v = sum_parts4(p.xa.p, p.xa.stride, p.xa.nparts, i);
          if (store_xa && p.xa.nparts > 1) *reinterpret_cast<f32x4*>(p.xa.out + i) = v;
          v *= p.xs;
        }
        ra[q] = v;
      }
#pragma unroll
      for (int q = 0; q < BF4; ++q) {
        const int f = tid + 256 * q;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (FWD) {
          const int64_t gn = n0 + f / AC4, gk = k0 + 4 * (f % AC4);
          if (gn < p.Nc && gk < p.r) v = *reinterpret_cast<const f32x4*>(p.XB + gn * p.r + gk);
        } else {
          const int64_t gk = k0 + f / (BN / 4), gn = n0 + 4 * (f % (BN / 4));
          if (gk < p.r && gn < p.Nc) v = *reinterpret_cast<const f32x4*>(p.XB + gk * p.Nc + gn);
        }
        rb[q] = v;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < AF4; ++q) {
        const int f = tid + 256 * q;
        *reinterpret_cast<f32x4*>(&As(0)[(f / AC4) * LDA + 4 * (f % AC4)]) = ra[q];
      }
#pragma unroll
      for (int q = 0; q < BF4; ++q) {
        const int f = tid + 256 * q;
        if (FWD)
          *reinterpret_cast<f32x4*>(&Bs(0)[(f / AC4) * LDB + 4 * (f % AC4)]) = rb[q];
        else
          *reinterpret_cast<f32x4*>(&Bs(0)[(f / (BN / 4)) * LDB + 4 * (f % (BN / 4))]) = rb[q];
      }
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
    auto kstep = [&](int64_t k) { return kbeg + min(k, nk - 1) * BK; };
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) load(R[u], kstep(u));
    store(R[0], kbeg, 0);
    __syncthreads();
    int64_t k = 0;
    for (; k + DEPTH <= nk; k += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int64_t kk = k + u;
        load(R[u], kstep(kk + DEPTH));
        // Keep the loads ahead of this step's MFMAs: left to itself the
        // scheduler sinks them next to their LDS stores to shorten register
        // lifetimes, which exposes their whole latency.
        __builtin_amdgcn_sched_barrier(0);
        const int buf = (int)(kk & 1);
        compute(buf);
        store(R[(u + 1) % DEPTH], kstep(kk + 1), buf ^ 1);
        __syncthreads();
      }
    }
    // Fewer than DEPTH steps left; their loads are already in flight.
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u) {
      const int64_t kk = k + u;
      if (kk < nk) {
        const int buf = (int)(kk & 1);
        compute(buf);
        if (kk + 1 < nk) store(R[(u + 1) % DEPTH], kstep(kk + 1), buf ^ 1);
        __syncthreads();
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

// K-steps of loads in flight: two for every tile.  The 64x64 split tiles
// measured 2-3 % slower per step at four (and slower still at six and
// eight); their loads are not what bounds a K-step.
template <int BM, int BN>
constexpr int gemm_f32_depth() {
  return 2;
}

// Grid (Nc/BN, M/BM, nsplit).
template <int BM, int BN, bool FWD, bool EXACT, bool SCALEA>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args p) {
  __shared__ __attribute__((aligned(16))) float smem[gemm_f32_lds_floats<BM, BN, FWD>()];
  gemm_f32_block<BM, BN, FWD, EXACT, gemm_f32_depth<BM, BN>(), SCALEA>(p, smem, blockIdx.x,
                                                                         blockIdx.y, blockIdx.z);
}

// Sum of the split partials in split order, then the epilogue of the unsplit
// kernel (Z = sum; Y = sum * cn/cd per column).
static __global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int nsplit,
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
