// Short-chunk path (fp32 W, contraction split across blocks): each linear's
// forward and backward in two launches apiece.
//
// When the token count T is small the frozen GEMM only fills the chip with
// its contraction split across blocks, and every launch costs a few
// microseconds of latency however little it does.  So the rank-side work
// runs beside the GEMM instead of before it:
//
//   forward  1: split GEMM partials of X W^T    |  down: U = X~ A^T (partials)
//            2: Y = sum of partials + s U B^T   (U summed once per row and
//               stored; DoRA: Z = that, Y = Z * mag/norm)
//   backward 1: split GEMM partials of g W  |  k3: V (few partials), dB (, dm)
//            2: dX = sum + (s V A) * mask * keep  |  k4: dA  |  dB/dm reduce
//
// ("8. LoRA Fundamentals", "How it works" for the forward; "Backward Bug
// Hunts ...", "Bug #1" for dX, dA and dB; "4.3. Training Guide", "Dropout"
// for the mask on the LoRA branch only.)  The LoRA terms are rank-r outer
// products that need the finished U or V, so they move out of the GEMM into
// the launch that sums its partials.  All sums run in a fixed order.
//
// Roles of one launch share a single LDS array (the largest role's size), so
// a role's blocks co-reside with the GEMM's on a CU.
//
// A launch may carry NG linears that read the same X (the projections of one
// layer that share their input): each linear keeps its own arguments, blocks
// and workspace, and the launch count per direction stays two for the whole
// group.  Per-linear arguments live in fixed-size arrays indexed inside
// unrolled loops, so every access is a compile-time kernel-argument offset.
#pragma once
#include "common.hpp"
#include "gemm_f32.hpp"
#include "skinny.hpp"

namespace lora {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Output tile of the split GEMM.
constexpr int SPLIT_BM = 64, SPLIT_BN = 64;

// Split GEMM blocks first, then `side_blocks` blocks of the side role on a
// (side_x, *) grid.
struct SplitGrid {
  int64_t ntn, ntm;       // SPLIT_BM x SPLIT_BN output tiles
  int nsplit;
  int64_t gemm_blocks;    // ntn * ntm * nsplit
  int64_t side_x;
  int64_t side_blocks;
};

// GEMM block b -> (tile col, tile row, split).  Consecutive tile indices on
// one XCD walk the M tiles of one W slice first: the blocks that read the
// same W slice share an L2.
LORA_DEV void split_tile(const SplitGrid& f, int64_t b, int64_t& tn, int64_t& tm, int& split) {
  const int64_t g = xcd_tile(b, f.gemm_blocks);
  tm = g % f.ntm;
  const int64_t rest = g / f.ntm;
  tn = rest % f.ntn;
  split = (int)(rest / f.ntn);
}

// Launch 1 of the forward: the split GEMM blocks of every linear (linear i
// owns blocks [gstart[i], gstart[i+1])), then their down blocks (linear i:
// [sstart[i], sstart[i+1]) on its side grid).
template <int NG>
struct FwdMain {
  GemmF32Args g[NG];
  DownArgs d[NG];
  SplitGrid f[NG];
  int64_t gstart[NG + 1];
  int64_t sstart[NG + 1];
};

template <int NG, bool EXACT, int RP>
__global__ __launch_bounds__(256) void fwd_main_kernel(FwdMain<NG> p) {
  constexpr int L = cmax(gemm_f32_lds_floats<SPLIT_BM, SPLIT_BN, true>(), down_lds_floats<RP>());
  __shared__ __attribute__((aligned(16))) float smem[L];
  const int64_t b = blockIdx.x;
  if (b < p.gstart[NG]) {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.gstart[i + 1]) {
        int64_t tn, tm;
        int split;
        split_tile(p.f[i], b - p.gstart[i], tn, tm, split);
        gemm_f32_block<SPLIT_BM, SPLIT_BN, true, EXACT, gemm_f32_depth<SPLIT_BM, SPLIT_BN>(), false>(
            p.g[i], smem, tn, tm, split);
        return;
      }
  } else {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.sstart[i + 1]) {
        const int64_t sb = b - p.sstart[i];
        down_block<RP>(p.d[i], smem, sb % p.f[i].side_x, (int)(sb / p.f[i].side_x));
        return;
      }
  }
}

// Launch 1 of the backward: split GEMM blocks of g W, then k3 blocks.
template <int NG>
struct BwdMain {
  GemmF32Args g[NG];
  K3Args k[NG];
  SplitGrid f[NG];
  int64_t gstart[NG + 1];
  int64_t sstart[NG + 1];
};

template <int NG, bool EXACT, bool SCALEA, int RP>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdMain<NG> p) {
  constexpr int L = cmax(gemm_f32_lds_floats<SPLIT_BM, SPLIT_BN, false>(), k3_lds_floats<RP>());
  __shared__ __attribute__((aligned(16))) float smem[L];
  const int64_t b = blockIdx.x;
  if (b < p.gstart[NG]) {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.gstart[i + 1]) {
        int64_t tn, tm;
        int split;
        split_tile(p.f[i], b - p.gstart[i], tn, tm, split);
        gemm_f32_block<SPLIT_BM, SPLIT_BN, false, EXACT, gemm_f32_depth<SPLIT_BM, SPLIT_BN>(),
                       SCALEA>(p.g[i], smem, tn, tm, split);
        return;
      }
  } else {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.sstart[i + 1]) {
        const int64_t sb = b - p.sstart[i];
        // Z reaches k3 only with a DoRA gradient, which also sets the dX
        // operand's column scale (SCALEA); without it the tile needs no Z slot.
        k3_block<RP, SCALEA>(p.k[i], smem, sb % p.f[i].side_x, (int)(sb / p.f[i].side_x));
        return;
      }
  }
}

// ---------------------------------------------------------------------------
// Epilogue of a split GEMM: C[m, n] = sum_q part[q][m][n] + LoRA term.
//   forward: + sum_j (s U[m,j]) B[n,j]                     XB = B_lora [Nc, r]
//   dx     : + (sum_j (s V[m,j]) A[j,n]) * mask(m,n)*keep  XB = A_lora [r, Nc]
// A block covers `rows` rows x `cols` columns (rows * cols <= 1024, each
// thread 4 consecutive columns); the U or V rows it needs are summed from
// their partials once, into LDS.
// ---------------------------------------------------------------------------
constexpr int EPI_MAX_ROWS = 16;
constexpr int EPI_MAX_RANK = 32;

struct EpiArgs {
  const float* part;      // [nsplit, M, Nc]
  int nsplit;
  int64_t M, Nc;
  LoraOperand xa;         // U or V [M, r] (partials); out: store the summed U
  const float* XB;
  int64_t r;
  float s;
  DropParams drop;        // dx only
  float* C;
  float* C2;              // forward DoRA: Z
  const float* cn;        // forward DoRA: column scale cn / cd
  const float* cd;
  int cols, rows;
  int64_t ncb;            // column blocks per row block
  int64_t blocks;
};

template <bool FWD>
LORA_DEV void epi_block(const EpiArgs& e, float* smem, int64_t b) {
  const int64_t rb = b / e.ncb, cb = b % e.ncb;
  const int64_t m0 = rb * e.rows, c0 = cb * e.cols;
  const int tid = threadIdx.x;
  const int r = (int)e.r;
  const int t4 = 4 * tid;
  const int lr = t4 / e.cols, lc = t4 % e.cols;
  const int64_t m = m0 + lr, n = c0 + lc;
  const bool act = lr < e.rows && m < e.M && n < e.Nc;
  const int64_t i4 = m * e.Nc + n;
  // No barrier: each wave stages, in LDS, the rank-side rows its own lanes
  // read (a row shared by two waves is written by both with equal values),
  // and a wave's LDS write precedes its own reads.  Loads are issued in the
  // order they are consumed, without loops, so their round trips overlap:
  // first the staged rows' partials (up to UP each), then this thread's
  // output split partials (up to PV), added in split order last.
  constexpr int UI = 3;          // staged values per lane (5 rows x 32 ranks at 64+ columns)
  constexpr int UP = 16, PV = 16;
  const int wave = tid >> 6, lane = tid & 63;
  const int wr0 = 256 * wave / e.cols;
  const int wr1 = min((256 * wave + 252) / e.cols, e.rows - 1);
  const int nu = wr0 <= wr1 ? (wr1 - wr0 + 1) * r : 0;
  float uv[UI][UP];
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int i = lane + 64 * it;
    const int64_t mu = m0 + wr0 + (i < nu ? i / r : 0);
    const int64_t idx = mu * e.r + (i < nu ? i % r : 0);
    if (i < nu && mu < e.M) {
#pragma unroll
      for (int u = 0; u < UP; ++u)
        if (u < e.xa.nparts) uv[it][u] = e.xa.p[(int64_t)u * e.xa.stride + idx];
    }
  }
  f32x4 pv[PV];
  if (act) {
#pragma unroll
    for (int u = 0; u < PV; ++u)
      if (u < e.nsplit) pv[u] = *reinterpret_cast<const f32x4*>(e.part + (int64_t)u * e.M * e.Nc + i4);
  }
  // An empty asm with a memory clobber emits nothing but keeps the compiler
  // from sinking the loads above next to their first use.
  asm volatile("" ::: "memory");
  float* xs = smem;   // [rows][r], already times s
#pragma unroll
  for (int it = 0; it < UI; ++it) {
    const int i = lane + 64 * it;
    if (i >= nu) continue;
    const int row = wr0 + i / r;
    const int64_t mu = m0 + row;
    const int64_t idx = mu * e.r + i % r;
    float v = 0.f;
    if (mu < e.M) {
      v = uv[it][0];
#pragma unroll
      for (int u = 1; u < UP; ++u)
        if (u < e.xa.nparts) v += uv[it][u];
      for (int u = UP; u < e.xa.nparts; ++u) v += e.xa.p[(int64_t)u * e.xa.stride + idx];
      if (FWD && e.xa.out && cb == 0) e.xa.out[idx] = v;
    }
    xs[row * r + i % r] = v * e.s;
  }
  // Narrow tiles (fewer than 64 columns) give a wave more rows than UI lanes'
  // worth; the rest are staged plainly.
  for (int i = lane + 64 * UI; i < nu; i += 64) {
    const int row = wr0 + i / r;
    const int64_t mu = m0 + row;
    const int64_t idx = mu * e.r + i % r;
    float v = 0.f;
    if (mu < e.M) {
      v = sum_parts1(e.xa.p, e.xa.stride, e.xa.nparts, idx);
      if (FWD && e.xa.out && cb == 0) e.xa.out[idx] = v;
    }
    xs[row * r + i % r] = v * e.s;
  }
  if (!act) return;
  f32x4 acc = pv[0];
#pragma unroll
  for (int u = 1; u < PV; ++u)
    if (u < e.nsplit) acc += pv[u];
  for (int u = PV; u < e.nsplit; ++u)
    acc += *reinterpret_cast<const f32x4*>(e.part + (int64_t)u * e.M * e.Nc + i4);
  const float* xr = xs + lr * r;
  f32x4 lo = {0.f, 0.f, 0.f, 0.f};
  if (FWD) {
    for (int j4 = 0; j4 < r; j4 += 4) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(xr + j4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 bq = *reinterpret_cast<const f32x4*>(e.XB + (n + q) * e.r + j4);
        lo[q] += u[0] * bq[0] + u[1] * bq[1] + u[2] * bq[2] + u[3] * bq[3];
      }
    }
  } else {
    for (int j = 0; j < r; ++j) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(e.XB + j * e.Nc + n);
      lo += xr[j] * a;
    }
    if (e.drop.on) {
      const uint64_t rk = drop_row(e.drop, m);
#pragma unroll
      for (int q = 0; q < 4; ++q) lo[q] *= drop_mul(e.drop, rk, n + q);
    }
  }
  f32x4 z = acc + lo;
  if (FWD) {
    if (e.C2) *reinterpret_cast<f32x4*>(e.C2 + i4) = z;
    if (e.cn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) z[q] *= e.cn[n + q] / e.cd[n + q];
    }
  }
  *reinterpret_cast<f32x4*>(e.C + i4) = z;
}

// Launch 2 of the forward: linear i's epilogue blocks are [start[i], start[i+1]).
template <int NG>
struct FwdEpi {
  EpiArgs e[NG];
  int64_t start[NG + 1];
};

template <int NG>
__global__ __launch_bounds__(256) void fwd_epi_kernel(FwdEpi<NG> p) {
  __shared__ __attribute__((aligned(16))) float smem[EPI_MAX_ROWS * EPI_MAX_RANK];
  const int64_t b = blockIdx.x;
#pragma unroll
  for (int i = 0; i < NG; ++i)
    if (b < p.start[i + 1]) {
      epi_block<true>(p.e[i], smem, b - p.start[i]);
      return;
    }
}

// Launch 2 of the backward.  Per linear: k4 blocks (the longest) first, then
// the dX epilogue, then reduction jobs (dB and dm when k3 split its token
// range).  All linears' k4 blocks come first, then all epilogues, then all
// reductions.
struct BwdEpiGrid {
  int64_t k4_x, k4_blocks, epi_blocks, red_blocks;
  int narrow;   // k4 as k4n_block (16 columns per block over all T)
};

template <int NG>
struct BwdEpi {
  EpiArgs e[NG];
  K4Args k[NG];
  RedJobs jobs[NG];
  BwdEpiGrid f[NG];
  int64_t kstart[NG + 1];   // k4 blocks of linear i
  int64_t estart[NG + 1];   // epilogue blocks of linear i
  int64_t rstart[NG + 1];   // reduction blocks of linear i
};

template <int NG, int RP>
__global__ __launch_bounds__(256) void bwd_epi_kernel(BwdEpi<NG> p) {
  constexpr int L = cmax(cmax(k4_lds_floats<RP>(), k4n_lds_floats<RP>()),
                         EPI_MAX_ROWS * EPI_MAX_RANK);
  __shared__ __attribute__((aligned(16))) float smem[L];
  const int64_t b = blockIdx.x;
  if (b < p.kstart[NG]) {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.kstart[i + 1]) {
        const int64_t kb = b - p.kstart[i];
        if (p.f[i].narrow) k4n_block<RP>(p.k[i], smem, kb);
        else k4_block<RP>(p.k[i], smem, kb % p.f[i].k4_x, (int)(kb / p.f[i].k4_x));
        return;
      }
  } else if (b < p.estart[NG]) {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.estart[i + 1]) {
        epi_block<false>(p.e[i], smem, b - p.estart[i]);
        return;
      }
  } else {
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (b < p.rstart[i + 1]) {
        reduce_block(p.jobs[i], b - p.rstart[i]);
        return;
      }
  }
}

}  // namespace lora
