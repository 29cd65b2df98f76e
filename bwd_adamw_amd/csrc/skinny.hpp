// Rank-r ("skinny") contractions of the LoRA branch on fp32 MFMA
// (v_mfma_f32_16x16x4f32).  All are HBM-bound streams over one activation:
//
//   down : U[t,j]  = sum_k X~[t,k] A[j,k]            (forward; reads X)
//   k3   : V[t,j]  = sum_n g[t,n] B[n,j]             (backward; reads dY once
//          dB[n,j] = s sum_t g[t,n] U[t,j]            for V, dB and DoRA dm)
//          dm[n]   = sum_t dY[t,n] Z[t,n] / norm[n]
//   k4   : dA[j,k] = s sum_t V[t,j] X~[t,k]          (backward; reads X)
//
// with g = dY (or dY * mag/norm for DoRA) and X~ = X * mask * keep
// ("8. LoRA Fundamentals", "How it works" and "The training loop";
// "Backward Bug Hunts ...", "Bug #1" for the dA = s (B^T g) x^T factor;
// "4.3. Training Guide", "Dropout" for the mask, recomputed inline).
//
// Each block streams 64 x 64 tiles of the activation through LDS and
// contracts them against the small rank-side operand with MFMA.  The long
// axis of each contraction may be split across blocks; each block then writes
// its own partial, and the partials are summed in split order by whoever
// reads them next (the frozen GEMM while staging U or V, k4 while staging V)
// or by reduce_kernel into the gradient arena.  No floating-point atomics and
// no cross-block synchronisation inside a kernel.
#pragma once
#include "common.hpp"

namespace lora {

constexpr int SK_T = 64;      // rows (tokens) per stage
constexpr int SK_C = 64;      // columns per stage
constexpr int SK_LD = SK_C + 4;

// ---------------------------------------------------------------------------
// down: Upart[split][t][j] = sum_{k in split} X~[t,k] A[j,k]; also writes the
// unmasked bf16 copy of X (used by the bf16 frozen GEMM) when Xbf != NULL.
// Grid: (ceil(T/64), nsplit).  RP = rank padded to a multiple of 16.
// With one split the block writes U itself.
// ---------------------------------------------------------------------------
template <int RP>
__global__ __launch_bounds__(256) void down_kernel(const float* __restrict__ X, int64_t T,
                                                   int64_t K, const float* __restrict__ A,
                                                   int64_t r, DropParams drop, int64_t ksplit,
                                                   float* __restrict__ Upart, float* __restrict__ U,
                                                   uint16_t* __restrict__ Xbf) {
  __shared__ __attribute__((aligned(16))) float Xs[SK_T * SK_LD];
  __shared__ __attribute__((aligned(16))) float As_[RP * SK_LD];
  constexpr int JG = RP / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * SK_T;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int64_t kb = (int64_t)split * ksplit, ke = min(K, kb + ksplit);
  const int l16 = lane & 15, h = lane >> 4;

  f32x4 acc[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kb; k0 < ke; k0 += SK_C) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = tid + 256 * q;
      const int row = f >> 4, c4 = f & 15;
      const int64_t t = t0 + row, k = k0 + 4 * c4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (t < T && k < ke) {
        v = *reinterpret_cast<const f32x4*>(X + t * K + k);
        if (Xbf) {
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(Xbf + t * K + k) = b;
        }
        if (drop.on) {
          const uint64_t rk = drop_row(drop, t);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= drop_mul(drop, rk, k + e);
        }
      }
      *reinterpret_cast<f32x4*>(&Xs[row * SK_LD + 4 * c4]) = v;
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      const int f = tid + 256 * q;
      const int row = f >> 4, c4 = f & 15;
      const int64_t k = k0 + 4 * c4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (row < r && k < ke) v = *reinterpret_cast<const f32x4*>(A + row * K + k);
      *reinterpret_cast<f32x4*>(&As_[row * SK_LD + 4 * c4]) = v;
    }
    __syncthreads();
    // wave w: rows 16w..16w+15; lane group h takes columns 16h..16h+15.
    f32x4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xv[q] = *reinterpret_cast<const f32x4*>(&Xs[(16 * wave + l16) * SK_LD + 16 * h + 4 * q]);
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      f32x4 av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        av[q] = *reinterpret_cast<const f32x4*>(&As_[(16 * j + l16) * SK_LD + 16 * h + 4 * q]);
#pragma unroll
      for (int s = 0; s < 16; ++s) acc[j] = mfma16x16x4(xv[s >> 2][s & 3], av[s >> 2][s & 3], acc[j]);
    }
    __syncthreads();
  }
  float* dst = nsplit == 1 ? U : Upart + (int64_t)split * T * r;
#pragma unroll
  for (int j = 0; j < JG; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 16 * wave + row16(v, lane);
      const int64_t jj = 16 * j + l16;
      if (t < T && jj < r) dst[t * r + jj] = acc[j][v];
    }
}

// ---------------------------------------------------------------------------
// k3: one pass over dY.  Grid: (ceil(N/64), nts); block (x, y) owns columns
// [64x, 64x+64) and rows [y*tsplit, (y+1)*tsplit).
//   Vpart[x][t][j]   = sum_{n in strip} g[t,n] B[n,j]
//   dBpart[y][n][j]  = sum_{t in range} g[t,n] U[t,j]
//   dmpart[y][n]     = sum_{t in range} dY[t,n] Z[t,n]          (DoRA)
//   gbf[t][n]        = bf16(g)                                   (optional)
// With one strip V is written directly; with one row range dB (and dm) are
// scaled and written (or added) directly.
// ---------------------------------------------------------------------------
struct K3Out {
  float* Vpart;
  float* V;
  float* dBpart;
  float* dB;
  float* dmpart;
  float* dm;
  uint16_t* gbf;
  float scale;
  int accumulate;
};

template <int RP>
__global__ __launch_bounds__(256) void k3_kernel(
    const float* __restrict__ dY, int64_t T, int64_t N, const float* __restrict__ B,
    const float* __restrict__ U, int64_t r, const float* __restrict__ mag,
    const float* __restrict__ nrm, const float* __restrict__ Z, int64_t tsplit, K3Out o) {
  __shared__ __attribute__((aligned(16))) float Gs[SK_T * SK_LD];
  __shared__ __attribute__((aligned(16))) float Bt[RP * SK_LD];        // B^T tile [j][n]
  __shared__ __attribute__((aligned(16))) float Us[SK_T * (RP + 4)];   // U tile [t][j]
  __shared__ float red[16][64];
  constexpr int JG = RP / 16;
  constexpr int LDU = RP + 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, h = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * SK_C;
  const int64_t tb = (int64_t)blockIdx.y * tsplit, te = min(T, tb + tsplit);
  const int c4 = tid & 15;               // this thread's column quad (fixed)
  const int64_t ncol = n0 + 4 * c4;
  const int nstrip = gridDim.x, nts = gridDim.y;

  float cmul[4] = {1.f, 1.f, 1.f, 1.f};
  if (mag) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ncol + e < N) cmul[e] = mag[ncol + e] / nrm[ncol + e];
  }
  for (int i = tid; i < RP * SK_C; i += 256) {
    const int j = i / SK_C, n = i % SK_C;
    float v = 0.f;
    if (j < r && n0 + n < N) v = B[(n0 + n) * r + j];
    Bt[j * SK_LD + n] = v;
  }

  f32x4 accB[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) accB[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dm[4] = {0.f, 0.f, 0.f, 0.f};
  float* vdst = nstrip == 1 ? o.V : o.Vpart + (int64_t)blockIdx.x * T * r;

  for (int64_t t0 = tb; t0 < te; t0 += SK_T) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (tid >> 4) + 16 * q;
      const int64_t t = t0 + row;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (t < te && ncol < N) {
        v = *reinterpret_cast<const f32x4*>(dY + t * N + ncol);
        if (Z) {
          const f32x4 z = *reinterpret_cast<const f32x4*>(Z + t * N + ncol);
#pragma unroll
          for (int e = 0; e < 4; ++e) dm[e] += v[e] * z[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= cmul[e];
        if (o.gbf) {
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(o.gbf + t * N + ncol) = b;
        }
      }
      *reinterpret_cast<f32x4*>(&Gs[row * SK_LD + 4 * c4]) = v;
    }
    for (int i = tid; i < SK_T * (RP / 4); i += 256) {
      const int row = i / (RP / 4), q = i % (RP / 4);
      const int64_t t = t0 + row;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (t < te && 4 * q < r) v = *reinterpret_cast<const f32x4*>(U + t * r + 4 * q);
      *reinterpret_cast<f32x4*>(&Us[row * LDU + 4 * q]) = v;
    }
    __syncthreads();

    {   // V contribution of this strip for rows 16*wave.. of the stage
      f32x4 gv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        gv[q] = *reinterpret_cast<const f32x4*>(&Gs[(16 * wave + l16) * SK_LD + 16 * h + 4 * q]);
      f32x4 accV[JG];
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        accV[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bv[q] = *reinterpret_cast<const f32x4*>(&Bt[(16 * j + l16) * SK_LD + 16 * h + 4 * q]);
#pragma unroll
        for (int s = 0; s < 16; ++s) accV[j] = mfma16x16x4(gv[s >> 2][s & 3], bv[s >> 2][s & 3], accV[j]);
      }
#pragma unroll
      for (int j = 0; j < JG; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t t = t0 + 16 * wave + row16(v, lane);
          const int64_t jj = 16 * j + l16;
          if (t < te && jj < r) vdst[t * r + jj] = accV[j][v];
        }
    }
    // dB partial: rows n = 16*wave + l16 (A operand g^T), contraction over t.
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int tt = 4 * s + h;
      const float a = Gs[tt * SK_LD + 16 * wave + l16];
#pragma unroll
      for (int j = 0; j < JG; ++j) accB[j] = mfma16x16x4(a, Us[tt * LDU + 16 * j + l16], accB[j]);
    }
  }

  // dB (and dm) of this strip: direct when there is one row range.
  const bool bdirect = nts == 1;
#pragma unroll
  for (int j = 0; j < JG; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t n = n0 + 16 * wave + row16(v, lane);
      const int64_t jj = 16 * j + l16;
      if (n < N && jj < r) {
        if (bdirect) {
          const float x = accB[j][v] * o.scale;
          o.dB[n * r + jj] = o.accumulate ? o.dB[n * r + jj] + x : x;
        } else {
          o.dBpart[((int64_t)blockIdx.y * N + n) * r + jj] = accB[j][v];
        }
      }
    }
  if (o.dm) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[tid >> 4][4 * c4 + e] = dm[e];
    __syncthreads();
    if (tid < 64 && n0 + tid < N) {
      float s = 0.f;
      for (int g = 0; g < 16; ++g) s += red[g][tid];
      if (bdirect) {
        s /= nrm[n0 + tid];
        o.dm[n0 + tid] = o.accumulate ? o.dm[n0 + tid] + s : s;
      } else {
        o.dmpart[(int64_t)blockIdx.y * N + n0 + tid] = s;
      }
    }
  }

}

// ---------------------------------------------------------------------------
// k4: dApart[y][j][k] = sum_{t in range y} V[t,j] X~[t,k], V given as vparts
// partials [vparts][T][r] summed in order while staging.
// Grid: (ceil(K/64), nts).  Wave w owns columns 16w..16w+15 of the strip.
// With one row range the block scales and writes (or adds) dA itself.
// ---------------------------------------------------------------------------
template <int RP>
__global__ __launch_bounds__(256) void k4_kernel(const float* __restrict__ X, int64_t T,
                                                 int64_t K, const float* __restrict__ V,
                                                 int vparts, int64_t r, DropParams drop,
                                                 int64_t tsplit, float* __restrict__ dApart,
                                                 float* __restrict__ dA, float scale,
                                                 int accumulate) {
  __shared__ __attribute__((aligned(16))) float Xs[SK_T * SK_LD];
  __shared__ __attribute__((aligned(16))) float Vs[SK_T * (RP + 4)];
  constexpr int JG = RP / 16;
  constexpr int LDV = RP + 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, h = lane >> 4;
  const int64_t k0 = (int64_t)blockIdx.x * SK_C;
  const int64_t tb = (int64_t)blockIdx.y * tsplit, te = min(T, tb + tsplit);
  const int c4 = tid & 15;
  const int64_t kcol = k0 + 4 * c4;
  const int nts = gridDim.y;

  f32x4 acc[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = tb; t0 < te; t0 += SK_T) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (tid >> 4) + 16 * q;
      const int64_t t = t0 + row;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (t < te && kcol < K) {
        v = *reinterpret_cast<const f32x4*>(X + t * K + kcol);
        if (drop.on) {
          const uint64_t rk = drop_row(drop, t);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= drop_mul(drop, rk, kcol + e);
        }
      }
      *reinterpret_cast<f32x4*>(&Xs[row * SK_LD + 4 * c4]) = v;
    }
    for (int i = tid; i < SK_T * (RP / 4); i += 256) {
      const int row = i / (RP / 4), q = i % (RP / 4);
      const int64_t t = t0 + row;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (t < te && 4 * q < r) {
        const int64_t i = t * r + 4 * q;
        v = sum_parts4(V, T * r, vparts, i);
      }
      *reinterpret_cast<f32x4*>(&Vs[row * LDV + 4 * q]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int tt = 4 * s + h;
      const float b = Xs[tt * SK_LD + 16 * wave + l16];
#pragma unroll
      for (int j = 0; j < JG; ++j) acc[j] = mfma16x16x4(Vs[tt * LDV + 16 * j + l16], b, acc[j]);
    }
  }
  // acc[j][v] = dA[j' = 16j + 4*(l/16) + v][k = 16*wave + l16]
#pragma unroll
  for (int j = 0; j < JG; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t jj = 16 * j + row16(v, lane);
      const int64_t k = k0 + 16 * wave + l16;
      if (jj < r && k < K) {
        if (nts == 1) {
          const float x = acc[j][v] * scale;
          dA[jj * K + k] = accumulate ? dA[jj * K + k] + x : x;
        } else {
          dApart[((int64_t)blockIdx.y * r + jj) * K + k] = acc[j][v];
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Fixed-order reduction of partials: out[i] (+)= alpha * sum_p part[p][i]
// (/ div[i % divn]).  Up to 4 independent jobs per launch.
// ---------------------------------------------------------------------------
struct RedJob {
  const float* part;
  float* out;
  const float* div;
  int64_t n;
  int64_t divn;
  int nparts;
  int accumulate;
  float alpha;
};
struct RedJobs {
  RedJob job[4];
  int64_t blk[5];   // prefix of block counts
  int njobs;
};

__global__ __launch_bounds__(256) void reduce_kernel(RedJobs jobs) {
  int j = 0;
  while (j + 1 < jobs.njobs && (int64_t)blockIdx.x >= jobs.blk[j + 1]) ++j;
  const RedJob& J = jobs.job[j];
  const int64_t i = ((int64_t)blockIdx.x - jobs.blk[j]) * 256 + threadIdx.x;
  if (i >= J.n) return;
  sum_partials(J.part, J.n, J.nparts, i, J.alpha, J.div, J.div ? i % J.divn : 0, J.out,
               J.accumulate);
}

// ---------------------------------------------------------------------------
// Dropout keep mask [T, K] as bytes (1 = keep).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dropout_mask_kernel(DropParams drop, int64_t T, int64_t K,
                                                           uint8_t* __restrict__ mask) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * K) return;
  const int64_t t = i / K, k = i % K;
  mask[i] = drop.on ? (uint8_t)drop_keep(drop, drop_row(drop, t), k) : (uint8_t)1;
}

}  // namespace lora
