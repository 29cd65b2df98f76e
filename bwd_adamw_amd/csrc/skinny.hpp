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
// unmasked bf16 copy of X (used by the bf16 frozen GEMM) when Xbf != NULL,
// row-major or, when xbf_nkq > 0, in fragment tiles (atile_off).
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
  int64_t xbf_nkq;   // > 0: Xbf in fragment tiles of a contraction of xbf_nkq * 64
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

  // Stages of 64 columns; the next stage's loads are issued before this
  // stage is stored and contracted (branch-free: past the end they repeat
  // the last stage's addresses), so their latency overlaps the work.
  struct Tile {
    f32x4 x[4], a[RP / 16];
  };
  auto x_at = [&](int q, int64_t k0, int64_t& t, int64_t& k) -> bool {
    const int f = tid + 256 * q;
    t = t0 + (f >> 4);
    k = k0 + 4 * (f & 15);
    return t < T && k < ke;
  };
  auto a_at = [&](int q, int64_t k0, int& row, int64_t& k) -> bool {
    const int f = tid + 256 * q;
    row = f >> 4;
    k = k0 + 4 * (f & 15);
    return row < r && k < ke;
  };
  auto load = [&](Tile& S, int64_t k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t t, k;
      const bool ok = x_at(q, k0, t, k);
      S.x[q] = *reinterpret_cast<const f32x4*>(ok ? X + t * K + k : X);
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      int row;
      int64_t k;
      const bool ok = a_at(q, k0, row, k);
      S.a[q] = *reinterpret_cast<const f32x4*>(ok ? A + row * K + k : A);
    }
  };
  auto store = [&](const Tile& S, int64_t k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t t, k;
      const bool ok = x_at(q, k0, t, k);
      f32x4 v = ok ? S.x[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      if (ok) {
        if (Xbf) {
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(Xbf + (p.xbf_nkq ? atile_off(t, k, p.xbf_nkq) : t * K + k)) = b;
        }
        if (drop.on) {
          const uint64_t rk = drop_row(drop, t);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= drop_mul(drop, rk, k + e);
        }
      }
      const int f = tid + 256 * q;
      *reinterpret_cast<f32x4*>(&Xs[(f >> 4) * SK_LD + 4 * (f & 15)]) = v;
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      int row;
      int64_t k;
      const bool ok = a_at(q, k0, row, k);
      const int f = tid + 256 * q;
      *reinterpret_cast<f32x4*>(&As_[row * SK_LD + 4 * (f & 15)]) =
          ok ? S.a[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto contract = [&]() {
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
  };
  const int64_t nst = (ke - kb + SK_C - 1) / SK_C;
  auto kst = [&](int64_t i) { return kb + min(i, nst - 1) * SK_C; };
  Tile R[2];
  if (nst > 0) load(R[0], kst(0));
  auto step = [&](int64_t i, Tile& cur, Tile& nxt) {
    load(nxt, kst(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    store(cur, kst(i));
    __syncthreads();
    contract();
    __syncthreads();
  };
  int64_t i = 0;
  for (; i + 2 <= nst; i += 2) {
    step(i, R[0], R[1]);
    step(i + 1, R[1], R[0]);
  }
  if (i < nst) step(i, R[0], R[1]);
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
//   gbf[t][n]        = bf16(g)            (optional; tiled when gbf_nkq > 0)
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
  int64_t gbf_nkq;   // > 0: gbf in fragment tiles (atile_off) of a contraction of gbf_nkq * 64
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
  const float* dmdiv;   // dm's divisor: nrm, or mag when Z holds the forward's Y
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
// strips in strip order.  ZT: the tiles carry Z (DoRA's dm); without it a
// tile holds only g and U, which leaves room for a third wave per SIMD.
template <int RP, bool ZT = true>
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

  // The block's (strip, row stage) tiles run as one sequence, the next
  // tile's loads in flight while this one is stored and contracted
  // (branch-free loads; see down_block).  Per-strip set-up (column scale,
  // B^T tile) opens a strip and its dB / dm stores close it.
  const int64_t nst = (te - tb + SK_T - 1) / SK_T;
  const int64_t ntot = (sx1 - sx0) * nst;
  struct Tile {
    f32x4 g[4], z[ZT ? 4 : 1], u[RP / 16];
  };
  auto g_ok = [&](int q, int64_t idx, int64_t& t, int64_t& ncol) -> bool {
    const int64_t sx = sx0 + idx / nst, t0 = tb + (idx % nst) * SK_T;
    t = t0 + (tid >> 4) + 16 * q;
    ncol = sx * SK_C + 4 * c4;
    return t < te && ncol < N;
  };
  auto u_ok = [&](int q, int64_t idx, int& row, int& q4, int64_t& t) -> bool {
    const int64_t t0 = tb + (idx % nst) * SK_T;
    const int i = tid + 256 * q;
    row = i / (RP / 4);
    q4 = i % (RP / 4);
    t = t0 + row;
    return t < te && 4 * q4 < r;
  };
  auto load = [&](Tile& S, int64_t idx) {
    idx = min(idx, ntot - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t t, ncol;
      const bool ok = g_ok(q, idx, t, ncol);
      S.g[q] = *reinterpret_cast<const f32x4*>(ok ? dY + t * N + ncol : dY);
      if constexpr (ZT) {
        if (Z) S.z[q] = *reinterpret_cast<const f32x4*>(ok ? Z + t * N + ncol : Z);
      }
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      int row, q4;
      int64_t t;
      const bool ok = u_ok(q, idx, row, q4, t);
      S.u[q] = *reinterpret_cast<const f32x4*>(ok ? U + t * r + 4 * q4 : U);
    }
  };

  float cmul[4] = {1.f, 1.f, 1.f, 1.f};
  f32x4 accB[JG];
  float dm[4] = {0.f, 0.f, 0.f, 0.f};

  auto store = [&](const Tile& S, int64_t idx) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t t, ncol;
      const bool ok = g_ok(q, idx, t, ncol);
      f32x4 v = ok ? S.g[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      if (ok) {
        if constexpr (ZT) {
          if (Z) {
#pragma unroll
            for (int e = 0; e < 4; ++e) dm[e] += v[e] * S.z[q][e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= cmul[e];
        if (o.gbf) {
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(o.gbf + (o.gbf_nkq ? atile_off(t, ncol, o.gbf_nkq) : t * N + ncol)) = b;
        }
      }
      *reinterpret_cast<f32x4*>(&Gs[((tid >> 4) + 16 * q) * SK_LD + 4 * c4]) = v;
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      int row, q4;
      int64_t t;
      const bool ok = u_ok(q, idx, row, q4, t);
      *reinterpret_cast<f32x4*>(&Us[row * LDU + 4 * q4]) =
          ok ? S.u[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto strip_begin = [&](int64_t sx) {
    const int64_t n0 = sx * SK_C, ncol = n0 + 4 * c4;
#pragma unroll
    for (int e = 0; e < 4; ++e) cmul[e] = (mag && ncol + e < N) ? mag[ncol + e] / nrm[ncol + e] : 1.f;
    if (want_v) {
      for (int i = tid; i < RP * SK_C; i += 256) {
        const int j = i / SK_C, n = i % SK_C;
        float v = 0.f;
        if (j < r && n0 + n < N) v = B[(n0 + n) * r + j];
        Bt[j * SK_LD + n] = v;
      }
    }
#pragma unroll
    for (int j = 0; j < JG; ++j) accB[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) dm[e] = 0.f;
  };
  auto contract = [&](int64_t sx, int64_t t0) {
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
      const bool vfirst = sx == sx0;
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
  };
  auto strip_end = [&](int64_t sx) {
    const int64_t n0 = sx * SK_C;
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
          s /= p.dmdiv[n0 + tid];
          o.dm[n0 + tid] = o.accumulate ? o.dm[n0 + tid] + s : s;
        } else {
          o.dmpart[(int64_t)by * N + n0 + tid] = s;
        }
      }
    }
  };
  auto step = [&](int64_t idx, Tile& cur, Tile& nxt) {
    const int64_t i = idx % nst, sx = sx0 + idx / nst, t0 = tb + i * SK_T;
    if (i == 0) strip_begin(sx);
    load(nxt, idx + 1);
    __builtin_amdgcn_sched_barrier(0);
    store(cur, idx);
    __syncthreads();
    contract(sx, t0);
    __syncthreads();
    if (i == nst - 1) strip_end(sx);
  };
  Tile R[2];
  if (ntot > 0) load(R[0], 0);
  int64_t idx = 0;
  for (; idx + 2 <= ntot; idx += 2) {
    step(idx, R[0], R[1]);
    step(idx + 1, R[1], R[0]);
  }
  if (idx < ntot) step(idx, R[0], R[1]);
}

// Waves per SIMD k3 is built for: without Z, ranks up to 32 fit three.
LORA_HD constexpr int k3_waves_per_simd(int rp, bool zt) { return (!zt && rp <= 32) ? 3 : 2; }

// ZT must be true whenever p.Z is set.
template <int RP, bool ZT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(k3_waves_per_simd(RP, ZT))))
void k3_kernel(K3Args p) {
  __shared__ __attribute__((aligned(16))) float smem[k3_lds_floats<RP>()];
  k3_block<RP, ZT>(p, smem, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// k3r: the same pass as k3 for whole tiles (T and N multiples of 64, tsplit
// a multiple of 64, rank padded to RP = 32 or 64, SPB = 1, 2 or 4 strips per
// block), in row-major tile order: for each 64-row stage the block visits
// its strips one after another, so the stage's V rows are summed over the
// block's strips in registers and written once (no read-modify-write of the
// V partial), while each strip keeps its dB tile and dm in registers over
// all stages.  Both contractions run on v_mfma_f32_32x32x2f32:
//   V  [t][j] (+)= sum_n g[t][n] B[n][j]: MFMA e of group c takes n = 8c + 4h + e
//                  (h = lane / 32), so a lane reads four of its n as one
//                  128-bit LDS read from g and from the strip's B^T;
//   dB [n][j] (+)= sum_t g[t][n] U[t][j]: MFMA e of group c takes
//                  t = 16c + 8h + e, the lane halves' rows eight apart, which
//                  puts their 32-bit reads on different LDS banks.
// RP = 64: every wave owns one 32 x 32 tile of V and one of each strip's dB;
// RP = 32: waves 0-1 own V's tiles, waves 2-3 dB's.
// ---------------------------------------------------------------------------
constexpr int K3R_LD = 68;   // row stride (floats) of the g and B^T tiles

template <int RP, int SPB>
constexpr int k3r_lds_floats() { return 64 * K3R_LD + 64 * (RP + 4) + SPB * RP * K3R_LD; }

// Two waves per SIMD (256 registers each), except the DoRA instances with two
// strips per block: their Z tiles in flight need more, and at two waves they
// spilled about 90 registers; at one wave they fit (with AGPRs) and run about
// a fifth faster on [2048, 9728, 64] despite the lower occupancy.  Four
// strips per block (the host groups four only when every block gets four)
// hold four dB tiles and always run at one wave per SIMD.
template <int RP, bool ZT, int SPB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((ZT && SPB == 2) || SPB == 4 ? 1 : 2)))
void k3r_kernel(K3Args p) {
  static_assert(RP == 32 || RP == 64, "rank 32 or 64");
  static_assert(SPB == 1 || SPB == 2 || SPB == 4, "one, two or four strips per block");
  constexpr int LDU = RP + 4;
  constexpr bool BOTH = RP == 64;
  __shared__ __attribute__((aligned(16))) float smem[k3r_lds_floats<RP, SPB>()];
  float* Gs = smem;                      // g tile [t][n]
  float* Us = Gs + 64 * K3R_LD;          // U tile [t][j]
  float* Bt = Us + 64 * LDU;             // strip q's B^T at Bt + q * RP * K3R_LD, [j][n]
  const float* __restrict__ dY = p.dY;
  const float* __restrict__ Z = p.Z;
  const float* __restrict__ U = p.U;
  const int64_t T = p.T, N = p.N, r = p.r;
  const K3Out& o = p.o;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int tr = tid >> 4, tc = tid & 15;          // VALU: rows 4tr..4tr+3, columns 4tc..4tc+3
  const int64_t bx = blockIdx.x;
  const int by = blockIdx.y;
  const int64_t tb = (int64_t)by * p.tsplit, te = min(T, tb + p.tsplit);
  const int64_t sx0 = bx * p.spb;
  const int ns = (int)min<int64_t>(p.spb, p.nstrip - sx0);
  const int nvp = (int)((p.nstrip + p.spb - 1) / p.spb), nts = p.nts;
  const bool want_v = o.V != nullptr || o.Vpart != nullptr;
  float* vdst = !want_v ? nullptr : nvp == 1 ? o.V : o.Vpart + bx * T * r;
  const int nst = (int)((te - tb) / 64);
  const int ntot = nst * ns;
  const bool do_v = BOTH || wave < 2, do_b = BOTH || wave >= 2;
  const int tv = BOTH ? (wave & 1) : wave, jv = BOTH ? (wave >> 1) : 0;
  const int tn = BOTH ? (wave & 1) : wave - 2, jb = BOTH ? (wave >> 1) : 0;

  // Per strip: the column scale of this thread's four columns and B^T.  All
  // of these loads go out before any is used (unconditional, clamped
  // addresses; a strip past the block's last repeats its first), so the
  // prologue costs one round trip instead of one per load.
  constexpr int BQ = RP / 16;   // B float4s per thread and strip
  float cmul[SPB][4];
  {
    const bool hasmag = p.mag != nullptr;
    const float* mg = hasmag ? p.mag : p.B;   // any valid address when there is no scale
    const float* nr = hasmag ? p.nrm : p.B;
    f32x4 mv[SPB], nv[SPB], bv[SPB][BQ];
#pragma unroll
    for (int q = 0; q < SPB; ++q) {
      const int64_t n0 = (sx0 + (q < ns ? q : 0)) * 64;
      mv[q] = *reinterpret_cast<const f32x4*>(mg + (hasmag ? n0 + 4 * tc : 0));
      nv[q] = *reinterpret_cast<const f32x4*>(nr + (hasmag ? n0 + 4 * tc : 0));
#pragma unroll
      for (int u = 0; u < BQ; ++u) {
        const int i = tid + 256 * u, n = i / (RP / 4), jq = i % (RP / 4);
        bv[q][u] = *reinterpret_cast<const f32x4*>(p.B + (n0 + n) * r + min(4 * jq, (int)r - 4));
      }
    }
#pragma unroll
    for (int q = 0; q < SPB; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cmul[q][e] = hasmag ? mv[q][e] / nv[q][e] : 1.f;
      if (want_v && q < ns) {
        float* bt = Bt + q * RP * K3R_LD;
#pragma unroll
        for (int u = 0; u < BQ; ++u) {
          const int i = tid + 256 * u, n = i / (RP / 4), jq = i % (RP / 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) bt[(4 * jq + e) * K3R_LD + n] = 4 * jq < r ? bv[q][u][e] : 0.f;
        }
      }
    }
  }
  f32x16 vacc, dbacc[SPB];
  float dm[SPB][4];
#pragma unroll
  for (int v = 0; v < 16; ++v) vacc[v] = 0.f;
#pragma unroll
  for (int q = 0; q < SPB; ++q) {
#pragma unroll
    for (int v = 0; v < 16; ++v) dbacc[q][v] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dm[q][e] = 0.f;
  }

  // Tile idx: row stage idx / ns, strip idx % ns.  The next tile's loads go
  // out before this tile is scaled, stored and contracted; the U rows of a
  // stage (one register set) are loaded one tile before the stage opens.
  constexpr int UQ = RP / 16;   // U float4s per thread (stage rows x RP / 256)
  struct Tile {
    f32x4 g[4], z[ZT ? 4 : 1];
  };
  auto load = [&](Tile& S, int idx) {
    idx = idx < ntot ? idx : ntot - 1;
    const int64_t t0 = tb + (int64_t)(idx / ns) * 64, n0 = (sx0 + idx % ns) * 64;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int64_t off = (t0 + 4 * tr + qq) * N + n0 + 4 * tc;
      S.g[qq] = *reinterpret_cast<const f32x4*>(dY + off);
      if constexpr (ZT) S.z[qq] = *reinterpret_cast<const f32x4*>(Z + off);
    }
  };
  f32x4 un[UQ];
  auto load_u = [&](int stage) {
    stage = stage < nst ? stage : nst - 1;
    const int64_t t0 = tb + (int64_t)stage * 64;
#pragma unroll
    for (int u = 0; u < UQ; ++u) {   // unconditional load (clamped), value selected
      const int i = tid + 256 * u, row = i / (RP / 4), jq = i % (RP / 4);
      const f32x4 v = *reinterpret_cast<const f32x4*>(U + (t0 + row) * r + min(4 * jq, (int)r - 4));
      un[u] = 4 * jq < r ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  Tile R[2];
  if (ntot > 0) {
    load(R[0], 0);
    load_u(0);
  }
  // Q: the tile's strip, a compile-time index (the loop below visits strips
  // in order, so that each strip's accumulators stay in fixed registers);
  // LAST: the tile closes its row stage.
  auto step = [&](auto QC, auto LASTC, int idx, const Tile& S, Tile& nxt) {
    constexpr int Q = decltype(QC)::value;
    constexpr bool LAST = decltype(LASTC)::value;
    const int64_t t0 = tb + (int64_t)(idx / ns) * 64, n0 = (sx0 + Q) * 64;
    if constexpr (Q == 0) {   // the stage's U rows, loaded one tile ago
#pragma unroll
      for (int u = 0; u < UQ; ++u) {
        const int i = tid + 256 * u, row = i / (RP / 4), jq = i % (RP / 4);
        *reinterpret_cast<f32x4*>(&Us[row * LDU + 4 * jq]) = un[u];
      }
    }
    load(nxt, idx + 1);
    if constexpr (LAST) load_u(idx / ns + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      f32x4 g = S.g[qq];
      if constexpr (ZT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dm[Q][e] += g[e] * S.z[qq][e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] *= cmul[Q][e];
      if (o.gbf) {
        const u32x2 b = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
        const int64_t t = t0 + 4 * tr + qq, n = n0 + 4 * tc;
        *reinterpret_cast<u32x2*>(o.gbf + (o.gbf_nkq ? atile_off(t, n, o.gbf_nkq) : t * N + n)) = b;
      }
      *reinterpret_cast<f32x4*>(&Gs[(4 * tr + qq) * K3R_LD + 4 * tc]) = g;
    }
    __syncthreads();
    if (want_v && do_v) {
      const float* bt = Bt + Q * RP * K3R_LD;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&Gs[(32 * tv + l32) * K3R_LD + 8 * c + 4 * h]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&bt[(32 * jv + l32) * K3R_LD + 8 * c + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vacc = mfma32x32x2(a[e], b[e], vacc);
      }
    }
    if (do_b) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float av[8], bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 16 * c + 8 * h + e;
          av[e] = Gs[t * K3R_LD + 32 * tn + l32];
          bv[e] = Us[t * LDU + 32 * jb + l32];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) dbacc[Q] = mfma32x32x2(av[e], bv[e], dbacc[Q]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    if constexpr (LAST) {   // the stage's V rows, summed over the block's strips
      if (want_v && do_v) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t t = t0 + 32 * tv + row32(v, lane);
          const int64_t j = 32 * jv + l32;
          if (j < r) vdst[t * r + j] = vacc[v];
          vacc[v] = 0.f;
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (SPB == 4 && ns == 4) {
    for (int idx = 0; idx < ntot; idx += 4) {
      step(I0{}, std::false_type{}, idx, R[0], R[1]);
      step(I1{}, std::false_type{}, idx + 1, R[1], R[0]);
      step(std::integral_constant<int, SPB / 2>{}, std::false_type{}, idx + 2, R[0], R[1]);
      step(std::integral_constant<int, SPB - 1>{}, std::true_type{}, idx + 3, R[1], R[0]);
    }
  } else if (SPB == 2 && ns == 2) {
    for (int idx = 0; idx < ntot; idx += 2) {
      step(I0{}, std::false_type{}, idx, R[0], R[1]);
      step(std::integral_constant<int, SPB - 1>{}, std::true_type{}, idx + 1, R[1], R[0]);
    }
  } else {   // one strip: every tile closes its stage
    for (int idx = 0; idx < ntot; idx += 2) {
      step(I0{}, std::true_type{}, idx, R[0], R[1]);
      if (idx + 1 < ntot) step(I0{}, std::true_type{}, idx + 1, R[1], R[0]);
    }
  }

  // dB and dm of each strip: direct when there is one row range.
  const bool bdirect = nts == 1;
  float(*red)[64] = reinterpret_cast<float(*)[64]>(Gs);   // [16][64], g tile no longer read
#pragma unroll
  for (int q = 0; q < SPB; ++q) {
    if (q >= ns) break;
    const int64_t n0 = (sx0 + q) * 64;
    if (do_b) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t n = n0 + 32 * tn + row32(v, lane);
        const int64_t j = 32 * jb + l32;
        if (j < r) {
          if (bdirect) {
            const float x = dbacc[q][v] * o.scale;
            o.dB[n * r + j] = o.accumulate ? o.dB[n * r + j] + x : x;
          } else {
            o.dBpart[((int64_t)by * N + n) * r + j] = dbacc[q][v];
          }
        }
      }
    }
    if (o.dm) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 4; ++e) red[tr][4 * tc + e] = dm[q][e];
      __syncthreads();
      if (tid < 64) {
        float sum = 0.f;
        for (int g = 0; g < 16; ++g) sum += red[g][tid];
        if (bdirect) {
          sum /= p.dmdiv[n0 + tid];
          o.dm[n0 + tid] = o.accumulate ? o.dm[n0 + tid] + sum : sum;
        } else {
          o.dmpart[(int64_t)by * N + n0 + tid] = sum;
        }
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
  // With dropout on: the keep bits of the mask for the dX product after
  // this one, or NULL: 32-bit words, word w of token t at keep[w * T + t]
  // (bit b is column 32 w + b), so a block's rows of one word are contiguous.
  uint32_t* keep;
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

  // Row stages of 64 tokens, the next stage's loads in flight while this one
  // is stored and contracted (branch-free; see down_block).  V items: the
  // 64 x RP/4 float4s of a stage, RP/16 per thread; the first partial is
  // prefetched, further partials (if any) are added when stored.
  struct Tile {
    f32x4 x[4], v[RP / 16];
  };
  auto x_ok = [&](int q, int64_t t0, int64_t& t) -> bool {
    t = t0 + (tid >> 4) + 16 * q;
    return t < te && kcol < K;
  };
  auto v_ok = [&](int q, int64_t t0, int& row, int& q4, int64_t& t) -> bool {
    const int i = tid + 256 * q;
    row = i / (RP / 4);
    q4 = i % (RP / 4);
    t = t0 + row;
    return t < te && 4 * q4 < r;
  };
  auto load = [&](Tile& S, int64_t t0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t t;
      const bool ok = x_ok(q, t0, t);
      S.x[q] = *reinterpret_cast<const f32x4*>(ok ? X + t * K + kcol : X);
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      int row, q4;
      int64_t t;
      const bool ok = v_ok(q, t0, row, q4, t);
      S.v[q] = *reinterpret_cast<const f32x4*>(ok ? V + t * r + 4 * q4 : V);
    }
  };
  auto store = [&](const Tile& S, int64_t t0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t t;
      const bool ok = x_ok(q, t0, t);
      f32x4 v = ok ? S.x[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      uint32_t nib = 0;
      if (ok && drop.on) {
        const uint64_t rk = drop_row(drop, t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool kp = drop_keep(drop, rk, kcol + e);
          v[e] *= kp ? drop.keep : 0.0f;
          nib |= (uint32_t)kp << e;
        }
      }
      if (p.keep != nullptr && drop.on) {
        // the eight lanes of a 32-column word (same row) OR their nibbles:
        // DPP quad permutes (lane ^ 1, lane ^ 2), then the half-row mirror
        // (lane i and 7 - i of each eight, one in each quad)
        int w = (int)(nib << (4 * (c4 & 7)));
        w |= __builtin_amdgcn_mov_dpp(w, 0xB1, 0xf, 0xf, true);
        w |= __builtin_amdgcn_mov_dpp(w, 0x4E, 0xf, 0xf, true);
        w |= __builtin_amdgcn_mov_dpp(w, 0x141, 0xf, 0xf, true);
        if ((c4 & 7) == 0 && t < te && kcol < K) p.keep[(kcol >> 5) * T + t] = (uint32_t)w;
      }
      *reinterpret_cast<f32x4*>(&Xs[((tid >> 4) + 16 * q) * SK_LD + 4 * c4]) = v;
    }
#pragma unroll
    for (int q = 0; q < RP / 16; ++q) {
      int row, q4;
      int64_t t;
      const bool ok = v_ok(q, t0, row, q4, t);
      f32x4 v = ok ? S.v[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      if (ok)
        for (int pp = 1; pp < vparts; ++pp)
          v += *reinterpret_cast<const f32x4*>(V + (int64_t)pp * T * r + t * r + 4 * q4);
      *reinterpret_cast<f32x4*>(&Vs[row * LDV + 4 * q4]) = v;
    }
  };
  auto contract = [&]() {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int tt = 4 * s + h;
      const float b = Xs[tt * SK_LD + 16 * wave + l16];
#pragma unroll
      for (int j = 0; j < JG; ++j) acc[j] = mfma16x16x4(Vs[tt * LDV + 16 * j + l16], b, acc[j]);
    }
  };
  const int64_t nst = (te - tb + SK_T - 1) / SK_T;
  auto tst = [&](int64_t i) { return tb + min(i, nst - 1) * SK_T; };
  Tile R[2];
  if (nst > 0) load(R[0], tst(0));
  auto step = [&](int64_t i, Tile& cur, Tile& nxt) {
    load(nxt, tst(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    store(cur, tst(i));
    __syncthreads();
    contract();
    __syncthreads();
  };
  int64_t i = 0;
  for (; i + 2 <= nst; i += 2) {
    step(i, R[0], R[1]);
    step(i + 1, R[1], R[0]);
  }
  if (i < nst) step(i, R[0], R[1]);
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
  int vec;   // 4: four elements per thread as 16-byte vectors (set by red_vec)
};

// Whether a job can take 16-byte vectors: n a multiple of four, partials and
// output 16-byte aligned.
LORA_HD inline int red_vec(const RedJob& j) {
  return (j.n % 4 == 0 && ((uintptr_t)j.part & 15) == 0 && ((uintptr_t)j.out & 15) == 0) ? 4 : 1;
}
// Blocks of 256 threads a job takes.
LORA_HD inline int64_t red_blocks(const RedJob& j) { return (j.n + 256 * j.vec - 1) / (256 * j.vec); }
struct RedJobs {
  RedJob job[4];
  int64_t blk[5];   // prefix of block counts
  int njobs;
};

LORA_DEV void reduce_block(const RedJobs& jobs, int64_t b) {
  int j = 0;
  while (j + 1 < jobs.njobs && b >= jobs.blk[j + 1]) ++j;
  const RedJob& J = jobs.job[j];
  if (J.vec == 4) {   // the same sums in the same order, sixteen loads in flight
    const int64_t i = ((b - jobs.blk[j]) * 256 + threadIdx.x) * 4;
    if (i >= J.n) return;
    f32x4 s = sum_parts4(J.part, J.n, J.nparts, i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] *= J.alpha;
      if (J.div) s[e] /= J.div[(i + e) % J.divn];
    }
    f32x4* o = reinterpret_cast<f32x4*>(J.out + i);
    *o = J.accumulate ? *o + s : s;
    return;
  }
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
