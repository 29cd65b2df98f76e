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
// Each block streams a 64 x 64 tile of the activation per stage through LDS
// and contracts it against the small rank-side operand with MFMA.  The long
// axis of each contraction is split across blocks; every block writes its own
// partial and fixed-order reducers sum them (deterministic, no atomics).
#pragma once
#include "common.hpp"

namespace lora {

constexpr int SK_T = 64;      // rows (tokens) per stage
constexpr int SK_C = 64;      // columns per stage
constexpr int SK_LD = SK_C + 4;

// ---------------------------------------------------------------------------
// down: Upart[split][t][j] = sum_{k in split} X~[t,k] A[j,k].  Optionally also
// writes the unmasked bf16 copy of X (used by the bf16 frozen GEMM).
// Grid: (ceil(T/64), nsplit).  RP = rank padded to a multiple of 16.
// ---------------------------------------------------------------------------
template <int RP>
__global__ __launch_bounds__(256) void down_kernel(const float* __restrict__ X, int64_t T,
                                                   int64_t K, const float* __restrict__ A,
                                                   int64_t r, DropParams drop, int64_t ksplit,
                                                   float* __restrict__ Upart,
                                                   uint16_t* __restrict__ Xbf) {
  __shared__ __attribute__((aligned(16))) float Xs[SK_T * SK_LD];
  __shared__ __attribute__((aligned(16))) float As_[RP * SK_LD];
  constexpr int JG = RP / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * SK_T;
  const int split = blockIdx.y;
  const int64_t kb = (int64_t)split * ksplit, ke = min(K, kb + ksplit);
  const int l16 = lane & 15, h = lane >> 4;

  f32x4 acc[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kb; k0 < ke; k0 += SK_C) {
    // X tile: 64 rows x 64 cols = 1024 float4, 4 per thread.
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
    // A tile: RP rows x 64 cols.
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
#pragma unroll
  for (int j = 0; j < JG; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 16 * wave + row16(v, lane);
      const int64_t jj = 16 * j + l16;
      if (t < T && jj < r) Upart[((int64_t)split * T + t) * r + jj] = acc[j][v];
    }
}

// ---------------------------------------------------------------------------
// k3: one pass over dY.  Grid: (ceil(N/64), nts); block (x, y) owns columns
// [64x, 64x+64) and rows [y*tsplit, (y+1)*tsplit).
//   Vpart[x][t][j]   = sum_{n in strip} g[t,n] B[n,j]
//   dBpart[y][n][j]  = sum_{t in range} g[t,n] U[t,j]
//   dmpart[y][n]     = sum_{t in range} dY[t,n] Z[t,n]          (DoRA)
//   gbf[t][n]        = bf16(g)                                   (optional)
// ---------------------------------------------------------------------------
template <int RP>
__global__ __launch_bounds__(256) void k3_kernel(
    const float* __restrict__ dY, int64_t T, int64_t N, const float* __restrict__ B,
    const float* __restrict__ U, int64_t r, const float* __restrict__ mag,
    const float* __restrict__ nrm, const float* __restrict__ Z, int64_t tsplit,
    float* __restrict__ Vpart, float* __restrict__ dBpart, float* __restrict__ dmpart,
    uint16_t* __restrict__ gbf) {
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

  // Column multipliers (DoRA c = mag/norm) of this thread's 4 columns.
  float cmul[4] = {1.f, 1.f, 1.f, 1.f};
  if (mag) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ncol + e < N) cmul[e] = mag[ncol + e] / nrm[ncol + e];
  }
  // B^T tile: Bt[j][n] = B[n0 + n][j]; loaded once.
  for (int i = tid; i < RP * SK_C; i += 256) {
    const int j = i / SK_C, n = i % SK_C;
    float v = 0.f;
    if (j < r && n0 + n < N) v = B[(n0 + n) * r + j];
    Bt[j * SK_LD + n] = v;
  }

  f32x4 accB[JG];   // dB partial: rows n = 16*wave + ..., cols j
#pragma unroll
  for (int j = 0; j < JG; ++j) accB[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dm[4] = {0.f, 0.f, 0.f, 0.f};

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
        if (gbf) {
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(gbf + t * N + ncol) = b;
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

    // V partial for rows 16*wave.. of this stage: contraction over the strip.
    {
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
          if (t < te && jj < r) Vpart[((int64_t)blockIdx.x * T + t) * r + jj] = accV[j][v];
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
  // dB partial out: accB[j][v] = dB[n = 16*wave + 4*(l/16) + v][j = 16j + l16]
#pragma unroll
  for (int j = 0; j < JG; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t n = n0 + 16 * wave + row16(v, lane);
      const int64_t jj = 16 * j + l16;
      if (n < N && jj < r) dBpart[((int64_t)blockIdx.y * N + n) * r + jj] = accB[j][v];
    }
  if (dmpart) {
    // Reduce the per-thread column sums over the 16 row groups in fixed order.
#pragma unroll
    for (int e = 0; e < 4; ++e) red[tid >> 4][4 * c4 + e] = dm[e];
    __syncthreads();
    if (tid < 64) {
      float s = 0.f;
      for (int g = 0; g < 16; ++g) s += red[g][tid];
      if (n0 + tid < N) dmpart[(int64_t)blockIdx.y * N + n0 + tid] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// k4: dApart[y][j][k] = sum_{t in range y} V[t,j] X~[t,k].
// Grid: (ceil(K/64), nts).  Wave w owns columns 16w..16w+15 of the strip.
// ---------------------------------------------------------------------------
template <int RP>
__global__ __launch_bounds__(256) void k4_kernel(const float* __restrict__ X, int64_t T,
                                                 int64_t K, const float* __restrict__ V,
                                                 int64_t r, DropParams drop, int64_t tsplit,
                                                 float* __restrict__ dApart) {
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
      if (t < te && 4 * q < r) v = *reinterpret_cast<const f32x4*>(V + t * r + 4 * q);
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
      if (jj < r && k < K) dApart[((int64_t)blockIdx.y * r + jj) * K + k] = acc[j][v];
    }
}

// ---------------------------------------------------------------------------
// Fixed-order reduction of partials: out[i] (+)= alpha * sum_p part[p][i]
// (optionally divided by div[i % divn]).  Up to 4 independent jobs per launch.
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
  float s = J.part[i];
  for (int q = 1; q < J.nparts; ++q) s += J.part[(int64_t)q * J.n + i];
  s *= J.alpha;
  if (J.div) s /= J.div[i % J.divn];
  J.out[i] = J.accumulate ? J.out[i] + s : s;
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
