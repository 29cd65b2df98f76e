// DoRA row norms of bf16 W for several linears at once, by expanding the
// square of the adapted row ("8. LoRA Fundamentals", "How it works": the
// detached norm ||W_i + s (B A)_i|| that scales each output column):
//
//   ||W_i + s (B A)_i||^2 = ||W_i||^2 + 2 s sum_j B_ij P_ij + s^2 sum_jl B_ij G_jl B_il,
//   P = W A^T [N, r],   G = A A^T [r, r].
//
// W is bf16, so once A is split exactly into three bf16 parts
// (A = hi + mid + lo, nb_split_kernel) every term of P is a sum of exact
// bf16 x bf16 products accumulated in float32 by v_mfma_f32_32x32x16_bf16:
// the accuracy of a float32 product for three bf16 passes, where the direct
// form (forming W + s B A and summing its squares) costs one float32 MFMA
// pass at a sixteenth of the bf16 rate.  G is the same product with the
// parts of A as the row operand (nine part pairs).  The adapters of one W
// (slots) are stacked as columns, so one pass over W serves all of them.
// nb_finish_kernel combines the terms per row in double.
#pragma once
#include "common.hpp"

namespace lora {

constexpr int NB_TM = 128;       // tile rows: four row groups of 32
constexpr int NB_TN = 128;       // tile columns: one 32-column group per wave
constexpr int NB_KS = 32;        // contraction per step: two MFMA k-groups of 16
constexpr int NB_MAX_JOBS = 8;   // W matrices per launch
constexpr int NB_MAX_SLOTS = 4;  // adapters stacked over one W
constexpr int NB_MAX_RP = 64;    // rank padded to a multiple of 32

// ---------------------------------------------------------------------------
// Split: A [r][K] float32 -> parts [S][3][RP][Kp] bf16 with A = hi + mid + lo
// exactly (hi = bf16(a), mid = bf16(a - hi), lo = a - hi - mid; each
// difference is exact in float32 and the last has at most 8 significant
// bits).  Rows r..RP-1 and columns K..Kp-1 are zero.  One thread per eight
// consecutive elements of a row.
// ---------------------------------------------------------------------------
struct NbSplitJob {
  const float* A[NB_MAX_SLOTS];
  uint16_t* parts;
  int64_t K, Kp;
  int r, RP, S;
  int64_t g0;   // first group of this job in the grid
};
struct NbSplitArgs {
  NbSplitJob job[NB_MAX_JOBS];
  int njobs;
  int64_t ngroups;
};

__global__ __launch_bounds__(256) void nb_split_kernel(NbSplitArgs p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= p.ngroups) return;
  int j = 0;
  while (j + 1 < p.njobs && g >= p.job[j + 1].g0) ++j;
  const NbSplitJob& J = p.job[j];
  const int64_t l = g - J.g0, per_row = J.Kp / 8, per_slot = (int64_t)J.RP * per_row;
  const int q = (int)(l / per_slot);
  const int64_t rem = l % per_slot;
  const int row = (int)(rem / per_row);
  const int64_t k0 = 8 * (rem % per_row);
  const float* A = J.A[q];
  u32x4 hv, mv, lv;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t h2[2], m2[2], l2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t k = k0 + e + u;
      const float a = (row < J.r && k < J.K) ? A[(int64_t)row * J.K + k] : 0.f;
      const uint32_t hb = f32_to_bf16_bits(a);
      const float r1 = a - bf16_bits_to_f32(hb);
      const uint32_t mb = f32_to_bf16_bits(r1);
      const float r2 = r1 - bf16_bits_to_f32(mb);
      h2[u] = hb;
      m2[u] = mb;
      l2[u] = f32_to_bf16_bits(r2);
    }
    hv[e / 2] = h2[0] | (h2[1] << 16);
    mv[e / 2] = m2[0] | (m2[1] << 16);
    lv[e / 2] = l2[0] | (l2[1] << 16);
  }
  const int64_t plane = (int64_t)J.RP * J.Kp;
  uint16_t* dst = J.parts + (int64_t)q * 3 * plane + (int64_t)row * J.Kp + k0;
  *reinterpret_cast<u32x4*>(dst) = hv;
  *reinterpret_cast<u32x4*>(dst + plane) = mv;
  *reinterpret_cast<u32x4*>(dst + 2 * plane) = lv;
}

// ---------------------------------------------------------------------------
// Products: out[split][row][c] = sum_{k in split} M[row][k] (hi + mid + lo)[c][k]
// for 128 x 128 tiles, where column c is row c % RP of slot c / RP's parts.
// Items: P (M = W, with each row's sum of squares written beside, from the
// first column tile) and G (M = the parts themselves, 3 S RP rows).
// Block: 4 waves; wave w owns columns 32w..32w+31 of the tile and all 128
// rows (four 32 x 32 accumulators).  The row tile of a step (128 x 32 bf16)
// is staged through LDS, double-buffered, one barrier per step, stored so
// that every MFMA operand read is one conflict-free 16-byte read per lane;
// each wave loads its own columns' parts straight into registers.  Loads run
// two steps ahead (a ring of three register stages).  Rows past `rows` read as zero (buffer bounds) and elements at k >=
// K are masked per 8-element group (K is a multiple of 8).
// ---------------------------------------------------------------------------
struct NbItem {
  const uint16_t* M;      // row operand, bf16 [rows][ldm]
  const uint16_t* parts;  // column operand: [C / RP][3][RP][Kp]
  float* out;             // [nsplit][rows][C]
  double* wsq;            // [nsplit][rows] sums of squares of M's rows, or nullptr
  int64_t rows, ldm, K, Kp, klen;
  int C, RP, nsplit, ncolt;
  int64_t tile0;          // first block of this item
};
struct NbProdArgs {
  NbItem it[2 * NB_MAX_JOBS];
  int nitems;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void nb_prod_kernel(NbProdArgs p) {
  constexpr uint32_t OUT = 0xfffffff0u;   // an offset past every resource
  __shared__ __attribute__((aligned(16))) u32x4 Ms[2][NB_TM * NB_KS / 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Tiles are numbered item by item (a job's P tiles, then its G tiles);
  // each XCD takes a contiguous run of them, so that the parts a job's
  // tiles share stay in one XCD's L2 instead of every L2 holding all jobs'.
  const int64_t b = xcd_tile(blockIdx.x, gridDim.x);
  int i = 0;
  while (i + 1 < p.nitems && b >= p.it[i + 1].tile0) ++i;
  const NbItem& I = p.it[i];
  int64_t t = b - I.tile0;
  const int colt = (int)(t % I.ncolt);
  t /= I.ncolt;
  const int sp = (int)(t % I.nsplit);
  const int64_t R0 = (t / I.nsplit) * NB_TM;
  const int64_t K = I.K, kb = sp * I.klen, ke = min(I.Kp, kb + I.klen);
  const int nsteps = (int)((ke - kb) / NB_KS);
  const int64_t nrows = min<int64_t>(NB_TM, I.rows - R0);
  const bool want_sq = I.wsq != nullptr && colt == 0;

  // Row operand: thread t stages row t/2, elements 16 (t%2) .. +15 of a step.
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(I.M + R0 * I.ldm), (short)0, (int)(uint32_t)(nrows * I.ldm * 2), 0x00020000);
  const int srow = tid >> 1, skh = tid & 1;
  const int64_t sbase = (int64_t)srow * I.ldm + 16 * skh;   // elements
  // LDS slot of piece h: row group srow/32, k-group skh, half h, row srow%32.
  const int sdst = ((srow >> 5) * 2 + skh) * 64 + (srow & 31);

  // Column operand: the wave's 32 columns lie in one slot (RP % 32 == 0).
  const int cw = (int)(colt * NB_TN) + 32 * wave;
  const bool has_cols = cw < I.C;
  const int cslot = has_cols ? cw / I.RP : 0;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(I.parts + (int64_t)cslot * 3 * I.RP * I.Kp), (short)0,
      (int)(uint32_t)(3 * (int64_t)I.RP * I.Kp * 2), 0x00020000);
  const uint32_t coff = (uint32_t)((((cw % I.RP) + (lane & 31)) * I.Kp + 8 * (lane >> 5)) * 2);
  const uint32_t pstride = (uint32_t)((int64_t)I.RP * I.Kp * 2);

  struct Stage {
    u32x4 m[2];
    u32x4 c[2][3];
  };
  auto load = [&](Stage& S, int s) {
    s = s < nsteps ? s : nsteps - 1;
    const int64_t k = kb + (int64_t)NB_KS * s;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool in = k + 16 * skh + 8 * h + 8 <= K;
      S.m[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rm, in ? (uint32_t)((sbase + k + 8 * h) * 2) : OUT, 0, 0));
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        S.c[kk][q] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rc, coff + q * pstride + (uint32_t)(2 * (k + 16 * kk)), 0, 0));
  };
  double dsq = 0.0;
  // `count`: the stage is a real step (not a repeat past the last one).
  auto put = [&](const Stage& S, int buf, bool count) {
#pragma unroll
    for (int h = 0; h < 2; ++h) Ms[buf][sdst + 32 * h] = S.m[h];
    float sq = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_bits_to_f32(S.m[h][e] & 0xffffu);
        const float hi = bf16_bits_to_f32(S.m[h][e] >> 16);
        sq += lo * lo + hi * hi;
      }
    dsq += (count && want_sq) ? (double)sq : 0.0;
  };
  f32x16 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[rt][v] = 0.f;
  auto compute = [&](const Stage& S, int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[rt] = Ms[buf][(rt * 2 + kk) * 64 + lane];
#pragma unroll
      for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma32x32x16_bf16(a[rt], S.c[kk][q], acc[rt]);
    }
  };
  // Step s: the loads of step s + 2 go out (a ring of three register
  // stages), this step's MFMAs run, step s + 1's row tile is stored to the
  // other buffer, one barrier.  The body is straight-line: past the last
  // step the loads repeat its addresses and the stores go to a buffer no
  // step reads (a branch there made the compiler wait for every load in
  // flight at the loop head); a wave without columns multiplies zeros.
  auto step = [&](int s, const Stage& cur, const Stage& nxt, Stage& nxt2) {
    load(nxt2, s + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, s & 1);
    put(nxt, (s + 1) & 1, s + 1 < nsteps);
    __syncthreads();
  };
  Stage R[3];
  load(R[0], 0);
  load(R[1], 1);
  put(R[0], 0, true);
  __syncthreads();
  int s = 0;
  for (; s + 3 <= nsteps; s += 3) {
    step(s, R[0], R[1], R[2]);
    step(s + 1, R[1], R[2], R[0]);
    step(s + 2, R[2], R[0], R[1]);
  }
  if (s < nsteps) step(s, R[0], R[1], R[2]);
  if (s + 1 < nsteps) step(s + 1, R[1], R[2], R[0]);

  if (has_cols) {
    float* out = I.out + (int64_t)sp * I.rows * I.C;
    const int64_t c = cw + (lane & 31);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = R0 + 32 * rt + row32(v, lane);
        if (row < I.rows) out[row * I.C + c] = acc[rt][v];
      }
  }
  if (want_sq) {
    dsq += __shfl_xor(dsq, 1, 64);
    if (skh == 0 && R0 + srow < I.rows) I.wsq[(int64_t)sp * I.rows + R0 + srow] = dsq;
  }
}

// ---------------------------------------------------------------------------
// Combine, four threads per row i of one slot q of a job:
//   n_i^2 = sum_splits wsq + 2 s sum_j B_ij P_ij + s^2 sum_j B_ij (G B_i^T)_j.
// G of the slot is summed over splits and parts in a fixed order (double)
// and held in LDS (zero past RP) with a row stride of 68 floats.  Every
// thread of a row holds the row of B in registers (16-byte loads when B's
// rows are 16-byte aligned); thread part c takes rank rows j = 4k + c of G
// and the P columns 16c..16c+15, so that a wave's G reads are four 16-byte
// pieces on distinct banks, each a broadcast.  The four partial sums meet by
// lane shuffles (double), in a fixed order.
// ---------------------------------------------------------------------------
constexpr int NB_FIN_ROWS = 64;    // one block: 64 rows of one slot, 4 threads each
constexpr int NB_GLD = 68;         // LDS row stride of G (floats)

struct NbFinJob {
  const float* P;      // [nsplit][N][C]
  const double* wsq;   // [nsplit][N]
  const float* G;      // [nsplit][3 S RP][C]
  const float* B[NB_MAX_SLOTS];
  float* out[NB_MAX_SLOTS];
  float s[NB_MAX_SLOTS];
  int64_t N;
  int C, RP, S, r, nsplit;
  int64_t blk0;        // first block; S * ceil(N / NB_FIN_ROWS) blocks
};
struct NbFinArgs {
  NbFinJob job[NB_MAX_JOBS];
  int njobs;
};

__global__ __launch_bounds__(256) void nb_finish_kernel(NbFinArgs p) {
  constexpr int R = NB_MAX_RP;
  __shared__ __attribute__((aligned(16))) float Gs[R * NB_GLD];
  __shared__ __attribute__((aligned(16))) float Ys[NB_FIN_ROWS * NB_GLD];   // B rows
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  int j = 0;
  while (j + 1 < p.njobs && b >= p.job[j + 1].blk0) ++j;
  const NbFinJob& J = p.job[j];
  const int64_t nch = (J.N + NB_FIN_ROWS - 1) / NB_FIN_ROWS, l = b - J.blk0;
  const int q = (int)(l / nch);
  const int c = tid & 3;
  const int64_t i = (l % nch) * NB_FIN_ROWS + (tid >> 2);
  const int64_t grows = 3ll * J.S * J.RP;
  {
    // Element e = tid + 256 u of the slot's G: every partial's loads of all
    // sixteen elements go out together (fixed order of the sums).
    constexpr int U = R * R / 256;
    double g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) g[u] = 0.0;
    for (int s = 0; s < J.nsplit; ++s) {
      float v[3][U];
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) {
        const float* Gp = J.G + ((int64_t)s * grows + (int64_t)(q * 3 + pp) * J.RP) * J.C + q * J.RP;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = tid + 256 * u, jj = e / R, ll = e % R;
          v[pp][u] = Gp[(int64_t)min(jj, J.RP - 1) * J.C + min(ll, J.RP - 1)];
        }
      }
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = tid + 256 * u, jj = e / R, ll = e % R;
          g[u] += (jj < J.RP && ll < J.RP) ? (double)v[pp][u] : 0.0;
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = tid + 256 * u;
      Gs[(e / R) * NB_GLD + e % R] = (float)g[u];
    }
  }
  __syncthreads();
  if (i >= J.N) return;   // the four threads of a row leave together
  const float* Bq = J.B[q];
  const int r = J.r;
  // Every load below is unconditional (clamped address, value selected):
  // guarded loads became branches, and the compiler then waited for each
  // load before the next.
  float y[R];
  if ((r & 3) == 0 && ((uintptr_t)Bq & 15) == 0) {
#pragma unroll
    for (int j4 = 0; j4 < R / 4; ++j4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(Bq + i * r + min(4 * j4, r - 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) y[4 * j4 + e] = 4 * j4 < r ? v[e] : 0.f;
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
      const float v = Bq[i * r + min(jj, r - 1)];
      y[jj] = jj < r ? v : 0.f;
    }
  }
  // Cross term over P columns 16c .. 16c + 15.
  double cross = 0.0;
  f32x4 pv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < J.nsplit; ++s) {
    const float* Pr = J.P + ((int64_t)s * J.N + i) * J.C + q * J.RP;
#pragma unroll
    for (int u = 0; u < 4; ++u)   // columns past RP: the slot's last four, not used
      pv[u] += *reinterpret_cast<const f32x4*>(Pr + min(4 * (4 * c + u), J.RP - 4));
  }
  // The thread's own sixteen B values (columns 16c ..), read from the row's
  // copy in LDS below: selecting them from y by c would index registers by a
  // lane-dependent value.
  float* Yrow = Ys + (tid >> 2) * NB_GLD;
  if (c == 0) {
#pragma unroll
    for (int j4 = 0; j4 < R / 4; ++j4)
      *reinterpret_cast<f32x4*>(&Yrow[4 * j4]) =
          f32x4{y[4 * j4], y[4 * j4 + 1], y[4 * j4 + 2], y[4 * j4 + 3]};
  }
  __builtin_amdgcn_wave_barrier();   // the row's four threads are in one wave
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool in = 4 * (4 * c + u) < J.RP;
    const f32x4 yc = *reinterpret_cast<const f32x4*>(&Yrow[16 * c + 4 * u]);
#pragma unroll
    for (int e = 0; e < 4; ++e) cross += in ? (double)yc[e] * (double)pv[u][e] : 0.0;
  }
  // Quadratic term over rank rows jj = 4k + c (zero rows past RP): a loop
  // kept rolled (unrolled, the compiler hoisted every G read of the 16 rows
  // and spilled), with B_i,jj read back from the row's copy in LDS.
  double quad = 0.0;
#pragma unroll 1
  for (int k = 0; k < R / 4; ++k) {
    const int jj = 4 * k + c;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int l4 = 0; l4 < R / 4; ++l4) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(&Gs[jj * NB_GLD + 4 * l4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] += g[e] * y[4 * l4 + e];
    }
    quad += (double)Yrow[jj] * (double)((d[0] + d[1]) + (d[2] + d[3]));
  }
  cross += __shfl_xor(cross, 1, 64);
  cross += __shfl_xor(cross, 2, 64);
  quad += __shfl_xor(quad, 1, 64);
  quad += __shfl_xor(quad, 2, 64);
  if (c == 0) {
    double w2 = 0.0;
    for (int s = 0; s < J.nsplit; ++s) w2 += J.wsq[(int64_t)s * J.N + i];
    const double sc = J.s[q];
    const double n2 = w2 + 2.0 * sc * cross + sc * sc * quad;
    J.out[q][i] = (float)sqrt(n2 > 0.0 ? n2 : 0.0);
  }
}

}  // namespace lora
