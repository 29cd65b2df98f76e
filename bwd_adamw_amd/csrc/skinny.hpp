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
struct DownArgs {
  const float* X;
  int64_t T, K;
  const float* A;
  int64_t r;
  DropParams drop;
  int64_t ksplit;
  int nsplit;
  float* Upart;
  float* U;
  uint16_t* Xbf;
};

template <int RP>
constexpr int down_lds_floats() { return SK_T * SK_LD + RP * SK_LD; }

// Row block bx, split `split`, in LDS `smem` (down_lds_floats<RP>() floats).
template <int RP>
LORA_DEV void down_block(const DownArgs& p, float* smem, int64_t bx, int split) {
  const float* __restrict__ X = p.X;
  const float* __restrict__ A = p.A;
  const int64_t T = p.T, K = p.K, r = p.r, ksplit = p.ksplit;
  const DropParams drop = p.drop;
  const int nsplit = p.nsplit;
  float* __restrict__ Upart = p.Upart;
  float* __restrict__ U = p.U;
  uint16_t* __restrict__ Xbf = p.Xbf;
  float* Xs = smem;
  float* As_ = smem + SK_T * SK_LD;
  constexpr int JG = RP / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = bx * SK_T;
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

template <int RP>
__global__ __launch_bounds__(256) void down_kernel(DownArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[down_lds_floats<RP>()];
  down_block<RP>(p, smem, blockIdx.x, blockIdx.y);
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

struct K3Args {
  const float* dY;
  int64_t T, N;
  const float* B;
  const float* U;
  int64_t r;
  const float* mag;
  const float* nrm;
  const float* Z;
  int64_t tsplit;
  int64_t nstrip;   // 64-column strips of N
  int64_t spb;      // strips per block: V partials = ceil(nstrip / spb)
  int nts;          // row ranges
  K3Out o;
};

template <int RP>
constexpr int k3_lds_floats() { return SK_T * SK_LD + RP * SK_LD + SK_T * (RP + 4) + 16 * 64; }

// Strips [bx*spb, bx*spb + spb) of row range by, in LDS `smem`
// (k3_lds_floats<RP>() floats).  The block's V partial (index bx) sums its
// strips in strip order.
template <int RP>
LORA_DEV void k3_block(const K3Args& p, float* smem, int64_t bx, int by) {
  const float* __restrict__ dY = p.dY;
  const float* __restrict__ B = p.B;
  const float* __restrict__ U = p.U;
  const float* __restrict__ mag = p.mag;
  const float* __restrict__ nrm = p.nrm;
  const float* __restrict__ Z = p.Z;
  const int64_t T = p.T, N = p.N, r = p.r, tsplit = p.tsplit;
  const K3Out& o = p.o;
  constexpr int JG = RP / 16;
  constexpr int LDU = RP + 4;
  float* Gs = smem;                                  // g tile [t][n]
  float* Bt = Gs + SK_T * SK_LD;                     // B^T tile [j][n]
  float* Us = Bt + RP * SK_LD;                       // U tile [t][j]
  float (*red)[64] = reinterpret_cast<float (*)[64]>(Us + SK_T * LDU);   // [16][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, h = lane >> 4;
  const int64_t tb = (int64_t)by * tsplit, te = min(T, tb + tsplit);
  const int c4 = tid & 15;               // this thread's column quad (fixed)
  const int nvp = (int)((p.nstrip + p.spb - 1) / p.spb), nts = p.nts;
  const bool want_v = o.V != nullptr || o.Vpart != nullptr;
  float* vdst = !want_v ? nullptr : nvp == 1 ? o.V : o.Vpart + bx * T * r;
  const int64_t sx0 = bx * p.spb, sx1 = min(p.nstrip, sx0 + p.spb);

  for (int64_t sx = sx0; sx < sx1; ++sx) {
    const int64_t n0 = sx * SK_C;
    const int64_t ncol = n0 + 4 * c4;
    const bool vfirst = sx == sx0;
    __syncthreads();   // the previous strip is done with Bt and red

    float cmul[4] = {1.f, 1.f, 1.f, 1.f};
    if (mag) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ncol + e < N) cmul[e] = mag[ncol + e] / nrm[ncol + e];
    }
    if (want_v) {
      for (int i = tid; i < RP * SK_C; i += 256) {
        const int j = i / SK_C, n = i % SK_C;
        float v = 0.f;
        if (j < r && n0 + n < N) v = B[(n0 + n) * r + j];
        Bt[j * SK_LD + n] = v;
      }
    }

    f32x4 accB[JG];
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

      if (want_v) {   // V contribution of this strip for rows 16*wave.. of the stage
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
        // Each element of the block's partial is written by one thread, so
        // later strips add to it in place.
#pragma unroll
        for (int j = 0; j < JG; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t t = t0 + 16 * wave + row16(v, lane);
            const int64_t jj = 16 * j + l16;
            if (t < te && jj < r) {
              float* d = vdst + t * r + jj;
              *d = vfirst ? accV[j][v] : *d + accV[j][v];
            }
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
            o.dBpart[((int64_t)by * N + n) * r + jj] = accB[j][v];
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
          o.dmpart[(int64_t)by * N + n0 + tid] = s;
        }
      }
    }
  }
}

template <int RP>
__global__ __launch_bounds__(256) void k3_kernel(K3Args p) {
  __shared__ __attribute__((aligned(16))) float smem[k3_lds_floats<RP>()];
  k3_block<RP>(p, smem, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// k4: dApart[y][j][k] = sum_{t in range y} V[t,j] X~[t,k], V given as vparts
// partials [vparts][T][r] summed in order while staging.
// Grid: (ceil(K/64), nts).  Wave w owns columns 16w..16w+15 of the strip.
// With one row range the block scales and writes (or adds) dA itself.
// ---------------------------------------------------------------------------
struct K4Args {
  const float* X;
  int64_t T, K;
  const float* V;
  int vparts;
  int64_t r;
  DropParams drop;
  int64_t tsplit;
  int nts;
  float* dApart;
  float* dA;
  float scale;
  int accumulate;
};

template <int RP>
constexpr int k4_lds_floats() { return SK_T * SK_LD + SK_T * (RP + 4); }

// Column strip bx, row range by, in LDS `smem` (k4_lds_floats<RP>() floats).
template <int RP>
LORA_DEV void k4_block(const K4Args& p, float* smem, int64_t bx, int by) {
  const float* __restrict__ X = p.X;
  const float* __restrict__ V = p.V;
  const int64_t T = p.T, K = p.K, r = p.r, tsplit = p.tsplit;
  const int vparts = p.vparts;
  const DropParams drop = p.drop;
  float* __restrict__ dApart = p.dApart;
  float* __restrict__ dA = p.dA;
  const float scale = p.scale;
  const int accumulate = p.accumulate;
  constexpr int JG = RP / 16;
  constexpr int LDV = RP + 4;
  float* Xs = smem;
  float* Vs = smem + SK_T * SK_LD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, h = lane >> 4;
  const int64_t k0 = bx * SK_C;
  const int64_t tb = (int64_t)by * tsplit, te = min(T, tb + tsplit);
  const int c4 = tid & 15;
  const int64_t kcol = k0 + 4 * c4;
  const int nts = p.nts;

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
          dApart[((int64_t)by * r + jj) * K + k] = acc[j][v];
        }
      }
    }
}

template <int RP>
__global__ __launch_bounds__(256) void k4_kernel(K4Args p) {
  __shared__ __attribute__((aligned(16))) float smem[k4_lds_floats<RP>()];
  k4_block<RP>(p, smem, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// k4 for short chunks (T <= K4N_MAX_T, one row range): block bx owns 16
// columns [16bx, 16bx + 16) over all T rows, so the grid has K/16 blocks.
// V (partials summed in order) is staged in LDS once; wave w takes the token
// groups {4g .. 4g+3 : g = w mod 4} with all its X loads in flight together;
// the four waves' dA tiles are added in LDS in wave order.
//   dA[j,k] (+)= s * sum_t V[t,j] X~[t,k]
// ---------------------------------------------------------------------------
constexpr int K4N_MAX_T = 256;

template <int RP>
constexpr int k4n_lds_floats() { return K4N_MAX_T * RP + 4 * (RP / 16) * 256; }

template <int RP>
LORA_DEV void k4n_block(const K4Args& p, float* smem, int64_t bx) {
  constexpr int JG = RP / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kq = lane >> 4;
  const int64_t T = p.T, K = p.K, r = p.r;
  const int64_t col = bx * 16 + l16;
  const DropParams drop = p.drop;
  float* Vs = smem;                        // [T][RP], zero beyond r
  float* red = smem + K4N_MAX_T * RP;      // [4 waves][JG][256]
  for (int64_t i = tid; i < T * (RP / 4); i += 256) {
    const int64_t t = i / (RP / 4);
    const int q = (int)(i % (RP / 4));
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (4 * q < r) v = sum_parts4(p.V, T * r, p.vparts, t * r + 4 * q);
    *reinterpret_cast<f32x4*>(&Vs[t * RP + 4 * q]) = v;
  }
  __syncthreads();

  f32x4 acc[JG];
#pragma unroll
  for (int j = 0; j < JG; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // token group g covers rows 4g..4g+3; lane group kq takes row 4g + kq
  const int64_t ngroups = (T + 3) / 4;
  for (int64_t g0 = wave; g0 < ngroups; g0 += 16) {
    float xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = 4 * (g0 + 4 * u) + kq;
      float x = 0.f;
      if (t < T && col < K) {
        x = p.X[t * K + col];
        if (drop.on) x *= drop_mul(drop, drop_row(drop, t), col);
      }
      xv[u] = x;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t t = 4 * (g0 + 4 * u) + kq;
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        const float a = t < T ? Vs[t * RP + 16 * j + l16] : 0.f;
        acc[j] = mfma16x16x4(a, xv[u], acc[j]);
      }
    }
  }
  // acc[j][v] = partial dA[16j + 4*kq + v][col] of this wave
#pragma unroll
  for (int j = 0; j < JG; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wave * JG + j) * 256 + v * 64 + lane] = acc[j][v];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    const float* q = red + j * 256 + tid;
    const float sum = ((q[0] + q[JG * 256]) + q[2 * JG * 256]) + q[3 * JG * 256];
    const int v = tid >> 6, ln = tid & 63;
    const int64_t jj = 16 * j + 4 * (ln >> 4) + v;
    const int64_t k = bx * 16 + (ln & 15);
    if (jj < r && k < K) {
      const float x = sum * p.scale;
      p.dA[jj * K + k] = p.accumulate ? p.dA[jj * K + k] + x : x;
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

LORA_DEV void reduce_block(const RedJobs& jobs, int64_t b) {
  int j = 0;
  while (j + 1 < jobs.njobs && b >= jobs.blk[j + 1]) ++j;
  const RedJob& J = jobs.job[j];
  const int64_t i = (b - jobs.blk[j]) * 256 + threadIdx.x;
  if (i >= J.n) return;
  sum_partials(J.part, J.n, J.nparts, i, J.alpha, J.div, J.div ? i % J.divn : 0, J.out,
               J.accumulate);
}

__global__ __launch_bounds__(256) void reduce_kernel(RedJobs jobs) { reduce_block(jobs, blockIdx.x); }

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
