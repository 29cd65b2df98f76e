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
// each wave loads its own columns' parts straight into registers one step
// ahead.  Rows past `rows` read as zero (buffer bounds) and elements at k >=
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
  const int64_t b = blockIdx.x;
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
    if (has_cols) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int q = 0; q < 3; ++q)
          S.c[kk][q] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         rc, coff + q * pstride + (uint32_t)(2 * (k + 16 * kk)), 0, 0));
    }
  };
  double dsq = 0.0;
  auto put = [&](const Stage& S, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) Ms[buf][sdst + 32 * h] = S.m[h];
    if (want_sq) {
      float sq = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_bits_to_f32(S.m[h][e] & 0xffffu);
          const float hi = bf16_bits_to_f32(S.m[h][e] >> 16);
          sq += lo * lo + hi * hi;
        }
      dsq += (double)sq;
    }
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
  // Step s: the next step's loads go out, this step's MFMAs run, the next
  // row tile is stored to the other buffer, one barrier.
  auto step = [&](int s, const Stage& cur, Stage& nxt) {
    load(nxt, s + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (has_cols) compute(cur, s & 1);
    if (s + 1 < nsteps) put(nxt, (s + 1) & 1);
    __syncthreads();
  };
  Stage R[2];
  if (nsteps > 0) {
    load(R[0], 0);
    put(R[0], 0);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, R[0], R[1]);
    if (s + 1 < nsteps) step(s + 1, R[1], R[0]);
  }

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
// Combine, one thread per row i of one slot q of a job:
//   n_i^2 = sum_splits wsq + 2 s sum_j B_ij P_ij + s^2 sum_j B_ij (G B_i^T)_j,
// G of the slot summed over splits and parts in a fixed order (double) and
// held in LDS with a row stride of NB_MAX_RP (zero past RP).
// ---------------------------------------------------------------------------
struct NbFinJob {
  const float* P;      // [nsplit][N][C]
  const double* wsq;   // [nsplit][N]
  const float* G;      // [nsplit][3 S RP][C]
  const float* B[NB_MAX_SLOTS];
  float* out[NB_MAX_SLOTS];
  float s[NB_MAX_SLOTS];
  int64_t N;
  int C, RP, S, r, nsplit;
  int64_t blk0;        // first block; S * ceil(N / 256) blocks
};
struct NbFinArgs {
  NbFinJob job[NB_MAX_JOBS];
  int njobs;
};

__global__ __launch_bounds__(256) void nb_finish_kernel(NbFinArgs p) {
  constexpr int R = NB_MAX_RP;
  __shared__ __attribute__((aligned(16))) float Gs[R * R];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  int j = 0;
  while (j + 1 < p.njobs && b >= p.job[j + 1].blk0) ++j;
  const NbFinJob& J = p.job[j];
  const int64_t nch = (J.N + 255) / 256, l = b - J.blk0;
  const int q = (int)(l / nch);
  const int64_t i = (l % nch) * 256 + tid;
  const int64_t grows = 3ll * J.S * J.RP;
  for (int e = tid; e < R * R; e += 256) {
    const int jj = e / R, ll = e % R;
    double g = 0.0;
    if (jj < J.RP && ll < J.RP)
      for (int s = 0; s < J.nsplit; ++s)
        for (int pp = 0; pp < 3; ++pp)
          g += J.G[((int64_t)s * grows + (int64_t)(q * 3 + pp) * J.RP + jj) * J.C + q * J.RP + ll];
    Gs[e] = (float)g;
  }
  __syncthreads();
  if (i >= J.N) return;
  const float* Bq = J.B[q];
  float y[R];
#pragma unroll
  for (int jj = 0; jj < R; ++jj) y[jj] = jj < J.r ? Bq[i * J.r + jj] : 0.f;
  double cross = 0.0;
#pragma unroll
  for (int j4 = 0; j4 < R / 4; ++j4) {
    if (4 * j4 < J.RP) {
      f32x4 pv = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < J.nsplit; ++s)
        pv += *reinterpret_cast<const f32x4*>(J.P + ((int64_t)s * J.N + i) * J.C + q * J.RP + 4 * j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) cross += (double)y[4 * j4 + e] * (double)pv[e];
    }
  }
  // z = G^T y over the slot's rank rows (y_j re-read from B, an L1 hit, so
  // that y and z are indexed by constants only), then y . z.
  float z[R];
#pragma unroll
  for (int l = 0; l < R; ++l) z[l] = 0.f;
  for (int jj = 0; jj < J.r; ++jj) {
    const float yj = Bq[i * J.r + jj];
#pragma unroll
    for (int l4 = 0; l4 < R / 4; ++l4) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(&Gs[jj * R + 4 * l4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) z[4 * l4 + e] += g[e] * yj;
    }
  }
  double quad = 0.0;
#pragma unroll
  for (int l = 0; l < R; ++l) quad += (double)y[l] * (double)z[l];
  double w2 = 0.0;
  for (int s = 0; s < J.nsplit; ++s) w2 += J.wsq[(int64_t)s * J.N + i];
  const double sc = J.s[q];
  const double n2 = w2 + 2.0 * sc * cross + sc * sc * quad;
  J.out[q][i] = (float)sqrt(n2 > 0.0 ? n2 : 0.0);
}

}  // namespace lora
