// liblora: C-ABI entry points (include/lora.h) over the gfx950 kernels.
//
// Every entry point validates all arguments before enqueueing anything,
// plans its launches from the shapes alone (so equal shapes always give the
// same split structure and bitwise-equal results), carves split partials out
// of the caller's workspace and enqueues on the caller's stream.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/lora.h"
#include "common.hpp"
#include "fused.hpp"
#include "gemm_bf16.hpp"
#include "gemm_f32.hpp"
#include "gemm_wq.hpp"
#include "launch.hpp"
#include "normbatch.hpp"
#include "optim.hpp"
#include "profile.hpp"
#include "skinny.hpp"

using namespace lora;

namespace {

// --------------------------------------------------------------- helpers ---
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline int64_t clampi(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }
inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// bf16 or block-quantized W: the frozen products run on bf16 MFMA.
inline bool bf16_ops(int32_t w_dtype) { return w_dtype != LORA_F32; }

// Planes of a block-quantized W [N, K] in one buffer: offset and size of
// each (a missing plane sits at the end with size 0); returns the total, 0
// for an invalid format or shape.
size_t qweight_layout(int f, int64_t N, int64_t K, size_t off[4], size_t bytes[4]) {
  if (!wq_quantized(f) || N <= 0 || K <= 0 || K % wq_super(f)) return 0;
  size_t o = 0;
  for (int i = 0; i < 4; ++i) {
    const int64_t rb = wq_plane_row_bytes(f, i, K);
    off[i] = o;
    bytes[i] = (size_t)(rb * N);
    o = rup((int64_t)(o + bytes[i]), 256);
  }
  for (int i = 0; i < 4; ++i)
    if (bytes[i] == 0) off[i] = o;
  return o;
}

QPlanes qplanes(const lora_linear* L) {
  QPlanes q;
  size_t off[4], bytes[4];
  qweight_layout(L->w_dtype, L->out_dim, L->in_dim, off, bytes);
  for (int i = 0; i < 4; ++i) {
    q.p[i] = (const uint8_t*)L->W + off[i];
    q.bytes[i] = (uint32_t)bytes[i];
  }
  return q;
}

uint64_t host_mix(uint64_t z) {   // SplitMix64 output function (see common.hpp)
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

bool drop_valid(const lora_dropout* d) {
  if (!d) return true;
  return d->p >= 0.0f && d->p < 1.0f;   // rejects NaN as well
}

DropParams make_drop(const lora_dropout* d) {
  DropParams dp;
  dp.base = 0;
  dp.thr = 0;
  dp.keep = 1.0f;
  dp.on = 0;
  if (!d || d->p == 0.0f) return dp;
  uint64_t h = host_mix(d->seed);
  h = host_mix(h ^ (uint64_t)d->step);
  h = host_mix(h ^ (uint64_t)(int64_t)d->ordinal);
  h = host_mix(h ^ (uint64_t)(int64_t)d->layer);
  h = host_mix(h ^ (uint64_t)(int64_t)d->proj);
  dp.base = h;
  dp.thr = (uint32_t)nearbyint((double)d->p * 16777216.0);   // ties to even
  dp.keep = (float)(1.0 / (1.0 - (double)d->p));
  dp.on = 1;
  return dp;
}

int rank_pad(int64_t r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

// ------------------------------------------------------------- planning ---
struct Split {
  int64_t len;   // contraction (or row) length per split
  int n;         // number of splits
};

// Split a length L into n pieces of a multiple of `q`, aiming for `want`
// blocks in total given `other` blocks along the other axis.
Split plan_split(int64_t L, int64_t other, int64_t want, int64_t q, int64_t min_len) {
  int64_t n = clampi(cdiv(want, other), 1, std::max<int64_t>(1, L / min_len));
  int64_t len = rup(cdiv(L, n), q);
  return {len, (int)cdiv(L, len)};
}

// Blocks of 256 threads of `kern` resident per CU, from the runtime (what
// its registers and LDS allow); 2 where the runtime cannot say (no GPU).
template <typename F>
int64_t resident_per_cu(F kern) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, 0) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 2;
  }
  return n;
}
constexpr int64_t kCUs = 256;

// Resident blocks of k4 on the whole chip, per padded rank; looked up once
// per instance.  (k3 keeps its target of 512 blocks: measured on the
// 9728-wide products, shorter blocks beyond one round of them beat one round
// of longer blocks.)
int64_t k4_slots(int rp) {
  static const int64_t s[4] = {kCUs * resident_per_cu(k4_kernel<16>), kCUs * resident_per_cu(k4_kernel<32>),
                               kCUs * resident_per_cu(k4_kernel<64>), kCUs * resident_per_cu(k4_kernel<128>)};
  return s[rp <= 16 ? 0 : rp <= 32 ? 1 : rp <= 64 ? 2 : 3];
}

// Row range of the rank-side backward kernels: whole T (results written
// directly, no reduction launch) when T is short or the column strips alone
// fill the chip; otherwise split into as many ranges as keep the grid within
// the `slots` blocks the chip holds at once (rounded down: a grid just past
// it would run a second, nearly empty round).
// k3's rows: the same, but rounded up to about `slots` blocks (k3 gains
// more from shorter blocks than it loses to a partly filled second round).
Split plan_rows_k3(int64_t T, int64_t strips, int64_t slots) {
  if (T <= 256 || strips >= 256) return {rup(T, SK_T), 1};
  return plan_split(T, strips, slots, SK_T, SK_T);
}
Split plan_rows(int64_t T, int64_t strips, int64_t slots = 512) {
  if (T <= 256 || strips >= 256) return {rup(T, SK_T), 1};
  const int64_t n = clampi(slots / strips, 1, cdiv(T, SK_T));
  const int64_t len = rup(cdiv(T, n), SK_T);
  return {len, (int)cdiv(T, len)};
}

// k3's grid on the plain path: column strips grouped spb per block (the
// block's V partial sums its strips in strip order) by token ranges (one dB
// partial per range).  V partials and re-reads of U grow with the number of
// block columns, dB partials and re-reads of B with the ranges; among the
// groupings with about 512 blocks (or as many as the shape has) the plan
// takes the one with the least of that traffic.  Each strip a block visits
// costs a B-tile load and the dB stores, so strips are grouped only over
// token ranges of at least four 64-row stages.
struct K3Plan {
  Split rows;
  int64_t spb, nvp;
};
K3Plan plan_k3(int64_t T, int64_t N, int64_t r, int64_t strips, int64_t slots) {
  auto cost = [&](int64_t nvp, int64_t nts) {
    return 4.0 * r * ((double)nvp * T * (nvp > 1 ? 3 : 2) + (double)nts * N * (nts > 1 ? 3 : 2));
  };
  // One strip per block, its rows split until about `slots` blocks run.
  K3Plan best = {plan_rows_k3(T, strips, slots), 1, strips};
  double cbest = cost(strips, best.rows.n);
  const int64_t maxr = cdiv(T, SK_T);
  const int64_t want = std::min<int64_t>(slots, strips * maxr);
  int64_t prev = strips;
  for (int64_t spb = 2; spb <= strips; ++spb) {
    const int64_t nvp = cdiv(strips, spb);
    if (nvp == prev) continue;   // the same partial count with fewer strips per block
    prev = nvp;
    const int64_t len = rup(cdiv(T, clampi(cdiv(want, nvp), 1, maxr)), SK_T);
    const int64_t nts = cdiv(T, len);
    if (nvp * nts * 8 < want * 7 || len < 4 * SK_T) continue;
    const double c = cost(nvp, nts);
    if (c < cbest) {
      cbest = c;
      best = {{len, (int)nts}, spb, nvp};
    }
  }
  return best;
}

struct GemmPlan {
  int bm, bn;
  Split k;           // contraction split across blocks (fp32 only)
  int cfg;           // bf16 kernel configuration (kBf16Cfg)
};

// bf16 kernel configurations: tile, threads, wave rows, K-step, stages in
// flight, the directions (1 forward, 2 dX) that use it, and the cost of one
// round of 256 tiles (one block per CU: LDS and registers admit no second)
// per direction: a microseconds per million (contraction length x tile area)
// plus b microseconds.  a and b were fitted to a sweep of every configuration
// and split on the Qwen3-4B-shaped projections at 2048 and 4096 tokens with
// operands read from HBM (mean error 3.4 %; the plans it picks are within
// 0.4 % of the sweep's best in total).  The wide tile runs its K-steps of 64
// with one stage in flight in both directions: fewer barriers per MFMA beat
// deeper staging.  The rows are LORA_BF16_CFGS
// (gemm_bf16.hpp).
struct Bf16Cfg {
  int bm, bn, nt, wgm, bk, depth, dirs;
  double a_fwd, b_fwd, a_dx, b_dx;
};
constexpr Bf16Cfg kBf16Cfg[] = {
#define LORA_CFG_ROW(i, bm, bn, nt, wgm, bk, d, dirs, af, bf, ad, bd) \
  {bm, bn, nt, wgm, bk, d, dirs, af, bf, ad, bd},
    LORA_BF16_CFGS(LORA_CFG_ROW)
#undef LORA_CFG_ROW
};
constexpr int kBf16NCfg = sizeof(kBf16Cfg) / sizeof(kBf16Cfg[0]);
constexpr int kBf16Slots = 256;  // resident tiles per round
// Cost of a split's fp32 partials (written once, read once by the reduction
// that also writes the result): microseconds per MB.  The single-launch fit
// gave 0.102; launches of other layers running beside the product compete
// for the same bandwidth, and 4x that measured best with four streams
// (DoRA two-slot Qwen3-4B step 279 -> 264 ms; on one stream 0.7-2.5 %
// slower).
constexpr double kSplitUsPerMB = 0.408;

// bf16: the configuration and contraction split (whole K-steps per split,
// at least 8 of them) with the least estimated time.  The direct-operand
// configuration (stages 0) is a candidate only where `tiled` says its A
// operand can be written in fragment tiles.
std::atomic<int> g_bf16_cfg{-1};   // lora_set_bf16_config

GemmPlan plan_gemm_bf16(int64_t M, int64_t Nc, int64_t Kc, bool dx, bool tiled) {
  GemmPlan best = {0, 0, {Kc, 1}, -1};
  double tbest = 1e30;
  auto runs = [&](const Bf16Cfg& c) { return (c.dirs & (dx ? 2 : 1)) && (c.depth != 0 || tiled); };
  const int forced = g_bf16_cfg.load(std::memory_order_relaxed);
  const bool force = forced >= 0 && runs(kBf16Cfg[forced]);
  for (int i = 0; i < kBf16NCfg; ++i) {
    const Bf16Cfg& c = kBf16Cfg[i];
    if (!runs(c) || (force && i != forced)) continue;
    const double a = dx ? c.a_dx : c.a_fwd, b = dx ? c.b_dx : c.b_fwd;
    const int64_t tiles = cdiv(M, c.bm) * cdiv(Nc, c.bn);
    for (int s = 1; s <= 8; ++s) {
      const int64_t len = rup(cdiv(Kc, s), c.bk);
      if (s > 1 && len < 8 * c.bk) break;
      const int64_t n = cdiv(Kc, len);
      if (n != s) continue;
      const double rounds = (double)cdiv(tiles * n, kBf16Slots);
      double t = rounds * (a * len * c.bm * c.bn / 1e6 + b);
      if (n > 1) t += kSplitUsPerMB * (2.0 * n + 1.0) * 4.0 * M * Nc / 1e6;
      if (t < tbest) {
        tbest = t;
        best = {c.bm, c.bn, {len, (int)n}, i};
      }
    }
  }
  return best;
}

// fp32: 128x128 when that fills the chip, else the split tile with the
// contraction split across blocks until about 256 blocks run.
GemmPlan plan_gemm(int64_t M, int64_t Nc, int64_t Kc, bool bf16, bool dx, bool tiled = false) {
  if (bf16) return plan_gemm_bf16(M, Nc, Kc, dx, tiled);
  if (cdiv(M, 128) * cdiv(Nc, 128) >= 256) return {128, 128, {rup(Kc, 32), 1}, 0};
  const int64_t tiles = cdiv(M, SPLIT_BM) * cdiv(Nc, SPLIT_BN);
  return {SPLIT_BM, SPLIT_BN, plan_split(Kc, tiles, 256, 32, 128), 0};
}

// The bf16 product of plan g reads its A operand in fragment tiles.
bool plan_tiled(const GemmPlan& g) { return g.cfg >= 0 && kBf16Cfg[g.cfg].depth == 0; }

// Products over T-row chunks of a linear whose A operand (bf16 X or g, a
// contraction of Kc) may be fragment-tiled: plain bf16 W (the quantized
// loop decodes W while staging it), whole 32-row fragment rows per chunk,
// whole 64-wide K-steps.
bool tiled_ok(const lora_linear* L, int64_t Kc) {
  return L->w_dtype == LORA_BF16 && L->tokens % 32 == 0 && Kc % 64 == 0;
}

// Short chunks: the contraction is split across blocks, and each linear runs
// as two launches per direction with the rank-side kernels beside the GEMM
// (fused.hpp).  The epilogue keeps U or V rows in LDS, hence the rank limit.
bool use_split_path(const GemmPlan& g, int64_t r, bool bf16) {
  return !bf16 && g.k.n > 1 && g.bm == SPLIT_BM && g.bn == SPLIT_BN && r <= EPI_MAX_RANK;
}

EpiArgs epi_shape(int64_t M, int64_t Nc) {
  EpiArgs e;
  memset(&e, 0, sizeof(e));
  e.M = M;
  e.Nc = Nc;
  e.cols = (int)std::min<int64_t>(1024, rup(Nc, 4));
  e.rows = (int)std::min<int64_t>(EPI_MAX_ROWS, 1024 / e.cols);
  e.ncb = cdiv(Nc, e.cols);
  e.blocks = cdiv(M, e.rows) * e.ncb;
  return e;
}

SplitGrid split_grid(int64_t M, int64_t Nc, int nsplit, int64_t side_x, int64_t side_y) {
  SplitGrid f;
  f.ntn = cdiv(Nc, SPLIT_BN);
  f.ntm = cdiv(M, SPLIT_BM);
  f.nsplit = nsplit;
  f.gemm_blocks = f.ntn * f.ntm * nsplit;
  f.side_x = side_x;
  f.side_blocks = side_x * side_y;
  return f;
}

// The consumers of the V partials (dX GEMM head, k4) sum them while staging
// when the repeated reads stay small; otherwise a separate launch sums them.
constexpr double kPartialRereadBytes = 64.0 * 1024 * 1024;

// Workspace layout of one linear.  Forward and backward share the buffer.
struct Layout {
  Split down, k3, k4;
  GemmPlan gf, gd;
  int64_t strips;      // 64-column strips of dY
  int64_t k3spb, k3nvp;   // k3 strips per block; V partials (= k3 grid x)
  bool vreduce;        // V partials summed by a separate launch
  size_t upart, xbf, gfpart;                          // forward
  size_t vpart, v, dbpart, dmpart, gbf, gdpart, dapart;   // backward
  size_t keep;         // the dropout mask's keep bits, ceil(K/32) x T words (k4 -> dX)
  size_t fwd_bytes, bwd_bytes;
};

size_t carve(size_t& off, size_t bytes) {
  const size_t at = off;
  off += (bytes + 255) & ~size_t(255);
  return at;
}

// stack > 1: the linear is one of `stack` slots whose frozen products run
// stacked; its bf16 operand copies and product partials then live in the
// stacked region (StackLayout) instead.
Layout make_layout(const lora_linear* L, int stack = 1) {
  Layout y;
  const int64_t T = L->tokens, K = L->in_dim, N = L->out_dim, r = L->rank;
  const bool bf = bf16_ops(L->w_dtype);
  const bool own = stack <= 1;
  y.down = plan_split(K, cdiv(T, SK_T), 512, SK_C, SK_C);
  y.strips = cdiv(N, SK_C);
  const int rpad = rank_pad(r);
  y.k4 = plan_rows(T, cdiv(K, SK_C), k4_slots(rpad));
  y.gf = plan_gemm(stack * T, N, K, bf, false, tiled_ok(L, K));
  y.gd = plan_gemm(stack * T, K, N, bf, true, tiled_ok(L, N));
  // k3 beside the split dX GEMM keeps its own grid (one strip per block
  // there); the plain path groups strips.
  if (use_split_path(y.gd, r, bf)) {
    y.k3 = plan_rows_k3(T, y.strips, 512);
    y.k3spb = 1;
    y.k3nvp = y.strips;
  } else {
    K3Plan kp = plan_k3(T, N, r, y.strips, 512);
    // DoRA's two-strip k3r blocks carry Z tiles and run one per CU (one wave
    // per SIMD). Their rows are split so that the blocks fill one round of
    // the CUs: the plan's two blocks per CU would leave a few blocks for a
    // third round, and fewer row ranges also mean fewer dB partials. Where
    // the plan keeps one strip per block, two strips per block on such a
    // grid halve the V partials (written here, summed by the reduction)
    // whenever each block still gets at least three 64-row stages.
    // Four strips per block (strip counts that are a multiple of four) halve
    // the V partials again where the blocks still get three stages.
    const int64_t nvp2 = cdiv(y.strips, 2);
    if (L->dora_mag != nullptr && (rpad == 32 || rpad == 64) && T % SK_T == 0 && N % SK_C == 0 &&
        kp.spb <= 2 && y.strips >= 2 && nvp2 <= kCUs) {
      auto one_round = [&](int64_t nvp) { return rup(cdiv(T, clampi(kCUs / nvp, 1, T / SK_T)), SK_T); };
      const int64_t len = one_round(nvp2);
      if (kp.spb == 2 || len >= 3 * SK_T) kp = {{len, (int)cdiv(T, len)}, 2, nvp2};
      const int64_t nvp4 = y.strips / 4, len4 = y.strips % 4 == 0 ? one_round(nvp4) : 0;
      if (kp.spb == 2 && len4 >= 3 * SK_T) kp = {{len4, (int)cdiv(T, len4)}, 4, nvp4};
    }
    y.k3 = kp.rows;
    y.k3spb = kp.spb;
    y.k3nvp = kp.nvp;
  }
  // Beside the split GEMM the down projection needs no parallelism of its
  // own: 256 columns per block keeps its partials few for the epilogue.
  if (use_split_path(y.gf, r, bf)) {
    const int64_t len = rup(cdiv(K, cdiv(K, 256)), SK_C);
    y.down = {len, (int)cdiv(K, len)};
  }
  const double vbytes = 4.0 * y.k3nvp * T * r;
  y.vreduce = y.k3nvp > 1 && vbytes * (cdiv(K, y.gd.bn) + cdiv(K, SK_C)) > kPartialRereadBytes;
  size_t off = 0;
  y.upart = carve(off, y.down.n > 1 ? sizeof(float) * y.down.n * T * r : 0);
  y.xbf = carve(off, (bf && own) ? sizeof(uint16_t) * T * K : 0);
  y.gfpart = carve(off, (own && y.gf.k.n > 1) ? sizeof(float) * y.gf.k.n * T * N : 0);
  y.fwd_bytes = off;
  off = 0;
  y.vpart = carve(off, y.k3nvp > 1 ? sizeof(float) * y.k3nvp * T * r : 0);
  y.v = carve(off, sizeof(float) * T * r);
  y.dbpart = carve(off, y.k3.n > 1 ? sizeof(float) * y.k3.n * N * r : 0);
  y.dmpart = carve(off, (L->dora_mag && y.k3.n > 1) ? sizeof(float) * y.k3.n * N : 0);
  y.gbf = carve(off, (bf && own) ? sizeof(uint16_t) * T * N : 0);
  y.gdpart = carve(off, (own && y.gd.k.n > 1) ? sizeof(float) * y.gd.k.n * T * K : 0);
  y.dapart = carve(off, y.k4.n > 1 ? sizeof(float) * y.k4.n * r * K : 0);
  // dX on the direct-operand loop takes the LoRA term's mask as bits that
  // k4 (which hashes every element of X anyway) leaves behind.
  y.keep = carve(off, (bf && plan_tiled(y.gd)) ? sizeof(uint32_t) * T * cdiv(K, 32) : 0);
  y.bwd_bytes = off;
  return y;
}

// The stacked region of n bf16 slots: the slots' bf16 copies of X (forward)
// and of g (backward), one above another, and the stacked products' split
// partials.
struct StackLayout {
  GemmPlan gf, gd;
  size_t xbf, gfpart, fwd_bytes;
  size_t gbf, gdpart, bwd_bytes;
};
StackLayout make_stack_layout(const lora_linear* L, int n) {
  StackLayout z;
  const int64_t M = n * L->tokens, K = L->in_dim, N = L->out_dim;
  z.gf = plan_gemm(M, N, K, true, false, tiled_ok(L, K));
  z.gd = plan_gemm(M, K, N, true, true, tiled_ok(L, N));
  size_t off = 0;
  z.xbf = carve(off, sizeof(uint16_t) * M * K);
  z.gfpart = carve(off, z.gf.k.n > 1 ? sizeof(float) * z.gf.k.n * M * N : 0);
  z.fwd_bytes = off;
  off = 0;
  z.gbf = carve(off, sizeof(uint16_t) * M * N);
  z.gdpart = carve(off, z.gd.k.n > 1 ? sizeof(float) * z.gd.k.n * M * K : 0);
  z.bwd_bytes = off;
  return z;
}

int check_linear(const lora_linear* L) {
  if (!L) return LORA_E_INVALID;
  if (L->tokens <= 0 || L->in_dim <= 0 || L->out_dim <= 0 || L->rank <= 0) return LORA_E_SHAPE;
  if (L->rank > 128 || L->rank > L->in_dim || L->rank > L->out_dim) return LORA_E_SHAPE;
  const int32_t f = L->w_dtype;
  if (f != LORA_F32 && f != LORA_BF16 && !wq_quantized(f)) return LORA_E_DTYPE;
  // bf16 operands and W's planes are read with 32-bit byte offsets (for
  // quantized W also from rows a tile past the end: in_dim <= 2^22).
  if (bf16_ops(f) &&
      (L->in_dim * L->out_dim >= (1ll << 30) || L->tokens * L->in_dim >= (1ll << 30) ||
       L->tokens * L->out_dim >= (1ll << 30)))
    return LORA_E_SHAPE;
  if (wq_quantized(f) && (L->in_dim % wq_super(f) || L->in_dim > (1 << 22))) return LORA_E_SHAPE;
  const int64_t q = bf16_ops(f) ? 8 : 4;
  if (L->in_dim % q || L->out_dim % q || L->rank % 4) return LORA_E_ALIGN;
  if (!L->W || !L->A || !L->B) return LORA_E_INVALID;
  if (!al16(L->W) || !al16(L->A) || !al16(L->B)) return LORA_E_ALIGN;
  if ((L->dora_mag == nullptr) != (L->dora_norm == nullptr)) return LORA_E_INVALID;
  if (L->dora_from_y && !L->dora_mag) return LORA_E_INVALID;
  if ((L->dora_mag && !al16(L->dora_mag)) || (L->dora_norm && !al16(L->dora_norm)))
    return LORA_E_ALIGN;
  if (!std::isfinite(L->scale)) return LORA_E_INVALID;
  return LORA_OK;
}

int hip_status() { return hipGetLastError() == hipSuccess ? LORA_OK : LORA_E_HIP; }

// ----------------------------------------------------------- launchers ---
#define LORA_RP_DISPATCH_32(rp, call)                 \
  if (rp <= 16) {                                     \
    constexpr int RP = 16;                            \
    call;                                             \
  } else {                                            \
    constexpr int RP = 32;                            \
    call;                                             \
  }

#define LORA_RP_DISPATCH(rp, call)                    \
  switch (rp) {                                       \
    case 16: { constexpr int RP = 16; call; } break;  \
    case 32: { constexpr int RP = 32; call; } break;  \
    case 64: { constexpr int RP = 64; call; } break;  \
    default: { constexpr int RP = 128; call; } break; \
  }

void launch_reduce(const RedJob* jobs, int n, hipStream_t st) {
  RedJobs J;
  memset(&J, 0, sizeof(J));
  int64_t blocks = 0;
  double bytes = 0.0;
  for (int i = 0; i < n; ++i) {
    J.job[i] = jobs[i];
    J.job[i].vec = red_vec(jobs[i]);
    J.blk[i] = blocks;
    blocks += red_blocks(J.job[i]);
    bytes += 4.0 * (double)jobs[i].n * (jobs[i].nparts + 1 + jobs[i].accumulate);
  }
  J.blk[n] = blocks;
  J.njobs = n;
  if (blocks == 0) return;
  prof::Scope ps("reduce", jobs[0].n, n, jobs[0].nparts, 0.0, bytes);
  launch(reduce_kernel, dim3((unsigned)blocks), st, ps, J);
}

void launch_gemm_f32(const GemmPlan& g, bool fwd, const GemmF32Args& a, hipStream_t st) {
  dim3 grid((unsigned)cdiv(a.Nc, g.bn), (unsigned)cdiv(a.M, g.bm), (unsigned)g.k.n);
  const bool exact = a.M % g.bm == 0 && a.Nc % g.bn == 0 && a.Kc % g.k.len == 0 && g.k.len % 32 == 0;
  {
    prof::Scope ps(fwd ? "gemm_f32_fwd" : "gemm_f32_dx", a.M, a.Nc, a.Kc,
                   2.0 * a.M * a.Nc * a.Kc + 2.0 * a.M * a.r * a.Nc,
                   4.0 * (a.M * a.Kc + a.Nc * a.Kc + a.M * a.Nc * (a.C2 ? 2 : 1)));
#define LORA_F32_TILE(BM_, BN_)                                                             \
  if (g.bm == BM_ && g.bn == BN_) {                                                          \
    if (fwd) {                                                                               \
      if (exact) launch(gemm_f32_kernel<BM_, BN_, true, true, false>, grid, st, ps, a);      \
      else launch(gemm_f32_kernel<BM_, BN_, true, false, false>, grid, st, ps, a);           \
    } else if (a.acn) {                                                                      \
      if (exact) launch(gemm_f32_kernel<BM_, BN_, false, true, true>, grid, st, ps, a);      \
      else launch(gemm_f32_kernel<BM_, BN_, false, false, true>, grid, st, ps, a);           \
    } else {                                                                                 \
      if (exact) launch(gemm_f32_kernel<BM_, BN_, false, true, false>, grid, st, ps, a);     \
      else launch(gemm_f32_kernel<BM_, BN_, false, false, false>, grid, st, ps, a);          \
    }                                                                                        \
  }
    LORA_F32_TILE(128, 128) else LORA_F32_TILE(SPLIT_BM, SPLIT_BN)
#undef LORA_F32_TILE
  }
  if (g.k.n > 1) {
    const int64_t n4 = cdiv(a.M * a.Nc, 4);
    prof::Scope ps("splitk_reduce", a.M, a.Nc, g.k.n, 0.0,
                   4.0 * a.M * a.Nc * (g.k.n + (a.C2 ? 2 : 1)));
    launch(splitk_reduce_kernel, dim3((unsigned)cdiv(n4, 256)), st, ps, (const float*)a.part,
           g.k.n, a.M, a.Nc, a.C, a.C2, a.cn, a.cd);
  }
}

void launch_gemm_bf16_tiles(const GemmPlan& g, bool fwd, const GemmBf16Args& a, hipStream_t st);

// W operand of a bf16 product: the bf16 matrix, or a quantized W's planes.
void set_w(GemmBf16Args& a, const lora_linear* L) {
  a.wq = L->w_dtype;
  if (wq_quantized(L->w_dtype)) a.q = qplanes(L);
  else a.B = (const uint16_t*)L->W;
}

// The bf16 GEMM, then (split contraction) the fixed-order sum of its partials
// with the unsplit kernel's epilogue.
void launch_gemm_bf16(const GemmPlan& g, bool fwd, const GemmBf16Args& a, hipStream_t st) {
  launch_gemm_bf16_tiles(g, fwd, a, st);
  if (g.k.n > 1) {
    const int64_t n4 = cdiv(a.M * a.Nc, 4);
    prof::Scope ps("splitk_reduce", a.M, a.Nc, g.k.n, 0.0,
                   4.0 * a.M * a.Nc * (g.k.n + (a.sl[0].C2 ? 2 : 1)));
    launch(splitk_reduce_bf16_kernel, dim3((unsigned)cdiv(n4, 256)), st, ps, a);
  }
}

void launch_gemm_bf16_tiles(const GemmPlan& g, bool fwd, const GemmBf16Args& a, hipStream_t st) {
  const dim3 grid((unsigned)(cdiv(a.Nc, g.bn) * cdiv(a.M, g.bm) * g.k.n));
  const bool quant = wq_quantized(a.wq);
  double wbytes = 2.0 * a.Nc * a.Kc;
  if (quant) wbytes = (double)a.q.bytes[0] + a.q.bytes[1] + a.q.bytes[2] + a.q.bytes[3];
  prof::Scope ps(quant ? (fwd ? "gemm_wq_fwd" : "gemm_wq_dx") : (fwd ? "gemm_bf16_fwd" : "gemm_bf16_dx"),
                 a.M, a.Nc, a.Kc, 2.0 * a.M * a.Nc * a.Kc + 2.0 * a.M * a.r * a.Nc,
                 2.0 * a.M * a.Kc + wbytes +
                     4.0 * a.M * a.Nc * (g.k.n > 1 ? g.k.n : (a.sl[0].C2 ? 2 : 1)));
  const Bf16Cfg& c = kBf16Cfg[g.cfg];
  const bool exact = a.M % c.bm == 0 && a.Nc % c.bn == 0 && a.Kc % c.bk == 0;
  switch (a.wq) {
    case LORA_Q8_0: launch_gemm_wq_tiles<WQ_Q8_0>(g.cfg, fwd, exact, grid, st, ps, a); return;
    case LORA_Q4_0: launch_gemm_wq_tiles<WQ_Q4_0>(g.cfg, fwd, exact, grid, st, ps, a); return;
    case LORA_Q4_K: launch_gemm_wq_tiles<WQ_Q4_K>(g.cfg, fwd, exact, grid, st, ps, a); return;
    case LORA_Q6_K: launch_gemm_wq_tiles<WQ_Q6_K>(g.cfg, fwd, exact, grid, st, ps, a); return;
    default: break;
  }
#define LORA_BF16_TILE(i, BM_, BN_, NT_, WGM_, BK_, D_, DIRS_, AF_, BF_, AD_, BD_)            \
  if (g.cfg == i) {                                                                        \
    if (fwd) {                                                                             \
      if constexpr ((DIRS_)&1) {                                                           \
        if (exact) launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, true, true>, grid, \
                            (unsigned)NT_, st, ps, a);                                     \
        else launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, true, false>, grid,      \
                      (unsigned)NT_, st, ps, a);                                           \
      }                                                                                    \
    } else {                                                                               \
      if constexpr ((DIRS_)&2) {                                                           \
        if (exact) launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, false, true>, grid, \
                            (unsigned)NT_, st, ps, a);                                     \
        else launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, false, false>, grid,     \
                      (unsigned)NT_, st, ps, a);                                           \
      }                                                                                    \
    }                                                                                      \
    return;                                                                                \
  }
  LORA_BF16_CFGS(LORA_BF16_TILE)
#undef LORA_BF16_TILE
}


// ------------------------------------------------------- linear jobs ---
// One linear's forward or backward, validated and planned: either the
// short-chunk split path (fused.hpp; several linears can share its two
// launches per direction) or the plain path.

struct FwdJob {
  bool split;
  const lora_linear* lin;
  int64_t T, K, N, r;
  GemmPlan gf;
  DownArgs da;
  double down_flops, down_bytes;
  LoraOperand xa;
  // split path
  GemmF32Args g;
  SplitGrid f;
  EpiArgs e;
  bool exact;
  int rp;
  // plain path
  uint16_t* Xbf;
  const float* X;
  float *Y, *Z, *gfpart;
  RedJob ured;      // U's split partials summed once before the product, if has_ured
  bool has_ured;
};

// One linear's operands of the bf16 forward product.
Bf16Slot bf16_fwd_slot(const FwdJob& j) {
  Bf16Slot so;
  memset(&so, 0, sizeof(so));
  so.xa = j.xa;
  so.XB = j.lin->B;
  so.xs = j.lin->scale;
  so.C = j.Y;
  so.C2 = j.Z;
  so.cn = j.lin->dora_mag;
  so.cd = j.lin->dora_norm;
  return so;
}

// stack > 1: one of `stack` stacked slots; bf is this slot's rows of the
// stacked bf16 copy of X.
int prepare_fwd(const lora_linear* lin, const float* X, float* Y, float* U, float* Z,
                const lora_dropout* drop, void* ws, size_t ws_bytes, FwdJob& j, int stack = 1,
                uint16_t* bf_rows = nullptr) {
  int rc = check_linear(lin);
  if (rc) return rc;
  if (!X || !Y || !U) return LORA_E_INVALID;
  if (!al16(X) || !al16(Y) || !al16(U) || (Z && !al16(Z))) return LORA_E_ALIGN;
  if (!drop_valid(drop)) return LORA_E_INVALID;
  const Layout y = make_layout(lin, stack);
  if (y.fwd_bytes && (!ws || ws_bytes < y.fwd_bytes || !al16(ws))) return LORA_E_WORKSPACE;
  const int64_t T = lin->tokens, K = lin->in_dim, N = lin->out_dim, r = lin->rank;
  const bool bf = bf16_ops(lin->w_dtype);
  char* w = (char*)ws;
  float* Upart = y.down.n > 1 ? (float*)(w + y.upart) : nullptr;
  j.lin = lin;
  j.T = T; j.K = K; j.N = N; j.r = r;
  j.gf = y.gf;
  j.X = X; j.Y = Y; j.Z = Z;
  j.Xbf = bf ? (stack > 1 ? bf_rows : (uint16_t*)(w + y.xbf)) : nullptr;
  j.gfpart = (stack <= 1 && y.gf.k.n > 1) ? (float*)(w + y.gfpart) : nullptr;
  DownArgs& da = j.da;
  da.X = X; da.T = T; da.K = K; da.A = lin->A; da.r = r; da.drop = make_drop(drop);
  da.ksplit = y.down.len; da.nsplit = y.down.n; da.Upart = Upart; da.U = U; da.Xbf = j.Xbf;
  da.xbf_nkq = (j.Xbf && plan_tiled(y.gf)) ? K / 64 : 0;
  j.down_flops = 2.0 * T * K * r;
  j.down_bytes = 4.0 * (T * K + r * K + T * r) + (j.Xbf ? 2.0 * T * K : 0.0);
  j.xa = y.down.n > 1 ? LoraOperand{Upart, T * r, y.down.n, U} : LoraOperand{U, T * r, 1, nullptr};
  j.split = use_split_path(y.gf, r, bf);
  // The direct-operand product stages U once per column of tiles: it reads
  // U summed by one reduction launch rather than summing the partials in
  // every tile.
  j.has_ured = bf && !j.split && y.down.n > 1 && plan_tiled(y.gf);
  if (j.has_ured) {
    j.ured = RedJob{Upart, U, nullptr, T * r, 1, (int)y.down.n, 0, 1.0f, 1};
    j.xa = LoraOperand{U, T * r, 1, nullptr};
  }
  if (j.split) {
    GemmF32Args& a = j.g;
    memset(&a, 0, sizeof(a));
    a.A = X; a.lda = K; a.B = (const float*)lin->W; a.ldb = K;
    a.M = T; a.Nc = N; a.Kc = K;
    a.ksplit = y.gf.k.len; a.nsplit = y.gf.k.n;
    a.part = j.gfpart;
    j.f = split_grid(T, N, y.gf.k.n, cdiv(T, SK_T), y.down.n);
    j.exact = T % 64 == 0 && N % 64 == 0 && K % y.gf.k.len == 0 && y.gf.k.len % 32 == 0;
    j.rp = rank_pad(r);
    EpiArgs e = epi_shape(T, N);
    e.part = a.part; e.nsplit = y.gf.k.n;
    e.xa = j.xa; e.XB = lin->B; e.r = r; e.s = lin->scale;
    e.C = Y; e.C2 = Z; e.cn = lin->dora_mag; e.cd = lin->dora_norm;
    j.e = e;
  }
  return LORA_OK;
}

// Launch 1: split GEMM partials of X W^T beside the down projection; launch
// 2: Y = sum of partials + s U B^T (DoRA: Z and the row scale).  NG linears
// of one X share both launches.
template <int NG>
void launch_fwd_split(const FwdJob* J, hipStream_t st) {
  FwdMain<NG> m;
  FwdEpi<NG> ep;
  int64_t b = 0, Nsum = 0;
  double fl = 0, by = 0, efl = 0, eby = 0;
  bool exact = true;
  int rp = 16;
  for (int i = 0; i < NG; ++i) {
    m.g[i] = J[i].g;
    m.d[i] = J[i].da;
    m.f[i] = J[i].f;
    m.gstart[i] = b;
    b += J[i].f.gemm_blocks;
    exact = exact && J[i].exact;
    rp = std::max(rp, J[i].rp);
    const int64_t T = J[i].T, N = J[i].N, K = J[i].K, r = J[i].r, ns = J[i].gf.k.n;
    Nsum += N;
    fl += 2.0 * T * N * K + J[i].down_flops;
    by += 4.0 * (T * K + N * K + ns * T * N) + J[i].down_bytes;
    efl += 2.0 * T * N * r;
    eby += 4.0 * T * N * (ns + (J[i].Z ? 2 : 1)) + 4.0 * (J[i].da.nsplit * T * r + N * r);
  }
  m.gstart[NG] = b;
  for (int i = 0; i < NG; ++i) {
    m.sstart[i] = b;
    b += J[i].f.side_blocks;
  }
  m.sstart[NG] = b;
  {
    prof::Scope ps("gemm_f32_fwd+down", J[0].T, Nsum, J[0].K, fl, by);
    LORA_RP_DISPATCH_32(rp, {
      if (exact) launch(fwd_main_kernel<NG, true, RP>, dim3((unsigned)b), st, ps, m);
      else launch(fwd_main_kernel<NG, false, RP>, dim3((unsigned)b), st, ps, m);
    });
  }
  b = 0;
  for (int i = 0; i < NG; ++i) {
    ep.e[i] = J[i].e;
    ep.start[i] = b;
    b += J[i].e.blocks;
  }
  ep.start[NG] = b;
  prof::Scope ps("fwd_epilogue", J[0].T, Nsum, J[0].gf.k.n, efl, eby);
  launch(fwd_epi_kernel<NG>, dim3((unsigned)b), st, ps, ep);
}

// U = X~ A^T, split over K (and the bf16 copy of X); the GEMM sums the
// splits while staging U and stores the summed U.
void launch_fwd_down(const FwdJob& j, hipStream_t st) {
  prof::Scope ps("down_u", j.T, j.r, j.K, j.down_flops, j.down_bytes);
  const dim3 grid((unsigned)cdiv(j.T, SK_T), (unsigned)j.da.nsplit);
  LORA_RP_DISPATCH(rank_pad(j.r), launch(down_kernel<RP>, grid, st, ps, j.da));
}

void launch_fwd_plain(const FwdJob& j, hipStream_t st) {
  const lora_linear* lin = j.lin;
  const int64_t T = j.T, K = j.K, N = j.N, r = j.r;
  launch_fwd_down(j, st);
  if (j.has_ured) launch_reduce(&j.ured, 1, st);
  // Z = X W^T + s U B^T; Y = Z or (mag/norm) * Z.
  if (bf16_ops(lin->w_dtype)) {
    GemmBf16Args a;
    memset(&a, 0, sizeof(a));
    a.A = j.Xbf; a.lda = K; a.ldb = K;
    set_w(a, lin);
    a.M = T; a.Nc = N; a.Kc = K; a.r = r;
    a.nslot = 1;
    a.sl[0] = bf16_fwd_slot(j);
    a.ksplit = j.gf.k.len; a.nsplit = j.gf.k.n; a.part = j.gfpart;
    launch_gemm_bf16(j.gf, true, a, st);
  } else {
    GemmF32Args a;
    memset(&a, 0, sizeof(a));
    a.A = j.X; a.lda = K; a.B = (const float*)lin->W; a.ldb = K;
    a.M = T; a.Nc = N; a.Kc = K;
    a.xa = j.xa; a.XB = lin->B; a.r = r; a.xs = lin->scale;
    a.ksplit = j.gf.k.len; a.nsplit = j.gf.k.n;
    a.C = j.Y; a.C2 = j.Z; a.cn = lin->dora_mag; a.cd = lin->dora_norm;
    a.part = j.gfpart;
    launch_gemm_f32(j.gf, true, a, st);
  }
}

struct BwdJob {
  bool split;
  const lora_linear* lin;
  int64_t T, K, N, r;
  Layout y;
  K3Out o;
  K3Args ka;
  K4Args k4a;
  double k3_flops, k3_bytes, k4_flops, k4_bytes;
  LoraOperand xv;
  DropParams d;
  RedJob jobs[3];
  int nj;
  RedJob ja;        // dA partials (k4 split over token ranges), if any
  bool has_ja;
  const float* dY;
  float* dX;
  char* w;
  // split path
  GemmF32Args g;
  K3Args kb;
  SplitGrid f;
  EpiArgs e;
  RedJobs J;
  BwdEpiGrid eg;
  int64_t nvp;
  bool exact;
  int rp;
};

// One linear's operands of the bf16 dX product.
Bf16Slot bf16_dx_slot(const BwdJob& j) {
  Bf16Slot so;
  memset(&so, 0, sizeof(so));
  so.xa = j.xv;
  so.XB = j.lin->A;
  so.xs = j.lin->scale;
  so.drop = j.d;
  so.C = j.dX;
  so.keep = j.k4a.keep;
  return so;
}

// stack > 1: one of `stack` stacked slots; bf is this slot's rows of the
// stacked bf16 copy of g.
int prepare_bwd(const lora_linear* lin, const float* X, const float* dY, const float* U,
                const float* Z, float* dX, float* dA, float* dB, float* dMag, int accumulate,
                const lora_dropout* drop, void* ws, size_t ws_bytes, BwdJob& j, int stack = 1,
                uint16_t* bf_rows = nullptr) {
  int rc = check_linear(lin);
  if (rc) return rc;
  if (!X || !dY || !U || !dA || !dB) return LORA_E_INVALID;
  if (!al16(X) || !al16(dY) || !al16(U) || !al16(dA) || !al16(dB)) return LORA_E_ALIGN;
  if ((dX && !al16(dX)) || (Z && !al16(Z)) || (dMag && !al16(dMag))) return LORA_E_ALIGN;
  const bool dora = lin->dora_mag != nullptr;
  if (dMag && (!dora || !Z)) return LORA_E_INVALID;
  if (!drop_valid(drop)) return LORA_E_INVALID;
  const Layout y = make_layout(lin, stack);
  if (y.bwd_bytes && (!ws || ws_bytes < y.bwd_bytes || !al16(ws))) return LORA_E_WORKSPACE;
  const int64_t T = lin->tokens, K = lin->in_dim, N = lin->out_dim, r = lin->rank;
  const bool bf = bf16_ops(lin->w_dtype);
  char* w = (char*)ws;
  const int acc = accumulate ? 1 : 0;
  j.lin = lin;
  j.T = T; j.K = K; j.N = N; j.r = r;
  j.y = y;
  j.w = w;
  j.dY = dY;
  j.dX = dX;
  j.d = make_drop(drop);
  j.rp = rank_pad(r);

  // One pass over dY: V (as partials per block column), dB, DoRA dm and
  // bf16 g.
  K3Out& o = j.o;
  o.Vpart = y.k3nvp > 1 ? (float*)(w + y.vpart) : nullptr;
  o.V = (float*)(w + y.v);
  o.dBpart = y.k3.n > 1 ? (float*)(w + y.dbpart) : nullptr;
  o.dB = dB;
  o.dmpart = (dMag && y.k3.n > 1) ? (float*)(w + y.dmpart) : nullptr;
  o.dm = dMag;
  o.gbf = (bf && dX) ? (stack > 1 ? bf_rows : (uint16_t*)(w + y.gbf)) : nullptr;
  o.gbf_nkq = (o.gbf && plan_tiled(y.gd)) ? N / 64 : 0;
  o.scale = lin->scale;
  o.accumulate = acc;
  const float* Zin = dMag ? Z : nullptr;
  K3Args& ka = j.ka;
  ka.dY = dY; ka.T = T; ka.N = N; ka.B = lin->B; ka.U = U; ka.r = r;
  ka.mag = lin->dora_mag; ka.nrm = lin->dora_norm; ka.Z = Zin;
  // Z may hold the forward's Y (dora_from_y): sum_t dY Y / mag is the same dm.
  ka.dmdiv = lin->dora_from_y ? lin->dora_mag : lin->dora_norm;
  ka.tsplit = y.k3.len; ka.nstrip = y.strips; ka.spb = y.k3spb; ka.nts = y.k3.n; ka.o = o;
  j.k3_flops = 4.0 * T * N * r;
  j.k3_bytes = 4.0 * (T * N + T * r + 2 * N * r) + (Zin ? 4.0 * T * N : 0.0) +
               (o.gbf ? 2.0 * T * N : 0.0);
  j.xv = (y.k3nvp == 1 || y.vreduce) ? LoraOperand{o.V, T * r, 1, nullptr}
                                      : LoraOperand{o.Vpart, T * r, (int)y.k3nvp, nullptr};
  float* dApart = y.k4.n > 1 ? (float*)(w + y.dapart) : nullptr;
  K4Args& k4a = j.k4a;
  k4a.X = X; k4a.T = T; k4a.K = K; k4a.V = j.xv.p; k4a.vparts = j.xv.nparts; k4a.r = r;
  k4a.drop = j.d; k4a.tsplit = y.k4.len; k4a.nts = y.k4.n; k4a.dApart = dApart; k4a.dA = dA;
  k4a.scale = lin->scale; k4a.accumulate = acc;
  k4a.keep = (bf && dX && plan_tiled(y.gd)) ? (uint32_t*)(w + y.keep) : nullptr;
  j.k4_flops = 2.0 * T * K * r;
  j.k4_bytes = 4.0 * (T * K + T * r + 2 * r * K);
  // Gradient splits over token ranges: fixed-order reduction jobs.
  j.nj = 0;
  if (y.k3.n > 1) {
    j.jobs[j.nj++] = {o.dBpart, dB, nullptr, N * r, 1, y.k3.n, acc, lin->scale};
    if (dMag) j.jobs[j.nj++] = {o.dmpart, dMag, ka.dmdiv, N, N, y.k3.n, acc, 1.0f};
  }
  j.has_ja = y.k4.n > 1;
  if (j.has_ja) j.ja = {dApart, dA, nullptr, r * K, 1, y.k4.n, acc, lin->scale};

  j.split = dX != nullptr && use_split_path(y.gd, r, bf);
  if (!j.split) return LORA_OK;
  GemmF32Args& a = j.g;
  memset(&a, 0, sizeof(a));
  a.A = dY; a.lda = N; a.acn = lin->dora_mag; a.acd = lin->dora_norm;
  a.B = (const float*)lin->W; a.ldb = K;
  a.M = T; a.Nc = K; a.Kc = N;
  a.ksplit = y.gd.k.len; a.nsplit = y.gd.k.n;
  a.part = (float*)(w + y.gdpart);
  // k3 beside the GEMM: one strip per block (each strip is a chain of
  // dependent loads), several only past 32 strips, so V arrives as at most
  // 32 partials for the two consumers of launch 2.
  K3Args& kb = j.kb;
  kb = ka;
  kb.spb = cdiv(y.strips, 32);
  j.nvp = cdiv(y.strips, kb.spb);
  kb.o.V = (float*)(w + y.v);
  kb.o.Vpart = j.nvp > 1 ? (float*)(w + y.vpart) : nullptr;
  const LoraOperand vd = j.nvp > 1 ? LoraOperand{kb.o.Vpart, T * r, (int)j.nvp, nullptr}
                                   : LoraOperand{kb.o.V, T * r, 1, nullptr};
  j.f = split_grid(T, K, y.gd.k.n, j.nvp, y.k3.n);
  j.exact = T % 64 == 0 && K % 64 == 0 && N % y.gd.k.len == 0 && y.gd.k.len % 32 == 0;
  k4a.V = vd.p;
  k4a.vparts = vd.nparts;
  EpiArgs e = epi_shape(T, K);
  e.part = a.part; e.nsplit = y.gd.k.n;
  e.xa = vd; e.XB = lin->A; e.r = r; e.s = lin->scale; e.drop = j.d;
  e.C = dX;
  j.e = e;
  memset(&j.J, 0, sizeof(j.J));
  int64_t rblocks = 0;
  for (int i = 0; i < j.nj; ++i) {
    j.J.job[i] = j.jobs[i];
    j.J.job[i].vec = red_vec(j.jobs[i]);
    j.J.blk[i] = rblocks;
    rblocks += red_blocks(j.J.job[i]);
  }
  j.J.blk[j.nj] = rblocks;
  j.J.njobs = j.nj;
  BwdEpiGrid& g = j.eg;
  g.narrow = T <= K4N_MAX_T && y.k4.n == 1;
  g.k4_x = g.narrow ? cdiv(K, 16) : cdiv(K, SK_C);
  g.k4_blocks = g.k4_x * y.k4.n;
  g.epi_blocks = e.blocks;
  g.red_blocks = rblocks;
  return LORA_OK;
}

// Launch 1: split GEMM partials of g W beside k3 (V partials, dB, dm);
// launch 2: dX = sum of partials + (s V A) * mask * keep beside k4 and the
// dB / dm reductions; then the dA reduction when k4 split its token range.
template <int NG>
void launch_bwd_split(const BwdJob* J, hipStream_t st) {
  BwdMain<NG> m;
  int64_t b = 0, Ksum = 0;
  double fl = 0, by = 0, efl = 0, eby = 0;
  bool exact = true, scalea = false;
  int rp = 16;
  for (int i = 0; i < NG; ++i) {
    m.g[i] = J[i].g;
    m.k[i] = J[i].kb;
    m.f[i] = J[i].f;
    m.gstart[i] = b;
    b += J[i].f.gemm_blocks;
    exact = exact && J[i].exact;
    scalea = scalea || J[i].g.acn != nullptr;
    rp = std::max(rp, J[i].rp);
    const int64_t T = J[i].T, N = J[i].N, K = J[i].K, r = J[i].r, ns = J[i].y.gd.k.n;
    Ksum += K;
    fl += 2.0 * T * N * K + J[i].k3_flops;
    by += 4.0 * (T * N + N * K + ns * T * K) + J[i].k3_bytes;
    efl += 2.0 * T * K * r + J[i].k4_flops;
    eby += 4.0 * T * K * (ns + 1) + 4.0 * (J[i].nvp * T * r + r * K) + J[i].k4_bytes;
  }
  m.gstart[NG] = b;
  for (int i = 0; i < NG; ++i) {
    m.sstart[i] = b;
    b += J[i].f.side_blocks;
  }
  m.sstart[NG] = b;
  {
    prof::Scope ps("gemm_f32_dx+k3", J[0].T, Ksum, J[0].N, fl, by);
    const dim3 grid((unsigned)b);
    LORA_RP_DISPATCH_32(rp, {
      if (scalea) {
        if (exact) launch(bwd_main_kernel<NG, true, true, RP>, grid, st, ps, m);
        else launch(bwd_main_kernel<NG, false, true, RP>, grid, st, ps, m);
      } else {
        if (exact) launch(bwd_main_kernel<NG, true, false, RP>, grid, st, ps, m);
        else launch(bwd_main_kernel<NG, false, false, RP>, grid, st, ps, m);
      }
    });
  }
  BwdEpi<NG> ep;
  b = 0;
  for (int i = 0; i < NG; ++i) {
    ep.e[i] = J[i].e;
    ep.k[i] = J[i].k4a;
    ep.jobs[i] = J[i].J;
    ep.f[i] = J[i].eg;
    ep.kstart[i] = b;
    b += J[i].eg.k4_blocks;
  }
  ep.kstart[NG] = b;
  for (int i = 0; i < NG; ++i) {
    ep.estart[i] = b;
    b += J[i].eg.epi_blocks;
  }
  ep.estart[NG] = b;
  for (int i = 0; i < NG; ++i) {
    ep.rstart[i] = b;
    b += J[i].eg.red_blocks;
  }
  ep.rstart[NG] = b;
  {
    prof::Scope ps("dx_epilogue+k4", J[0].T, Ksum, J[0].y.gd.k.n, efl, eby);
    LORA_RP_DISPATCH_32(rp, launch(bwd_epi_kernel<NG, RP>, dim3((unsigned)b), st, ps, ep));
  }
  RedJob ja[NG];
  int na = 0;
  for (int i = 0; i < NG; ++i)
    if (J[i].has_ja) ja[na++] = J[i].ja;
  if (na) launch_reduce(ja, na, st);
}

// One pass over dY: V, dB, dm and the bf16 copy of g (then V's partials
// summed when the plan says so).
void launch_bwd_k3(const BwdJob& jb, hipStream_t st) {
  const Layout& y = jb.y;
  const int64_t T = jb.T, N = jb.N, r = jb.r;
  {
    prof::Scope ps("k3_v_db", T, N, r, jb.k3_flops, jb.k3_bytes);
    const dim3 grid((unsigned)y.k3nvp, (unsigned)y.k3.n);
    // Whole 64 x 64 tiles at rank 32 or 64 with one or two strips per
    // block, or four when every block gets four: the row-major variant (same
    // outputs, V partials written once).
    const bool whole = (jb.rp == 32 || jb.rp == 64) && T % SK_T == 0 && N % SK_C == 0 &&
                       y.k3.len % SK_T == 0 && (y.k3spb <= 2 || (y.k3spb == 4 && y.strips % 4 == 0));
    const bool z = jb.ka.Z != nullptr;
    if (whole) {
#define LORA_K3R(RP_, ZT_, SPB_) \
  if (jb.rp == RP_ && z == ZT_ && y.k3spb == SPB_) launch(k3r_kernel<RP_, ZT_, SPB_>, grid, st, ps, jb.ka);
      LORA_K3R(32, false, 1) LORA_K3R(32, false, 2) LORA_K3R(32, true, 1) LORA_K3R(32, true, 2)
      LORA_K3R(64, false, 1) LORA_K3R(64, false, 2) LORA_K3R(64, true, 1) LORA_K3R(64, true, 2)
      LORA_K3R(32, false, 4) LORA_K3R(32, true, 4) LORA_K3R(64, false, 4) LORA_K3R(64, true, 4)
#undef LORA_K3R
    } else if (z) {
      LORA_RP_DISPATCH(jb.rp, launch(k3_kernel<RP, true>, grid, st, ps, jb.ka));
    } else {
      LORA_RP_DISPATCH(jb.rp, launch(k3_kernel<RP, false>, grid, st, ps, jb.ka));
    }
  }
  if (y.vreduce) {
    RedJob jv = {jb.o.Vpart, jb.o.V, nullptr, T * r, 1, (int)y.k3nvp, 0, 1.0f};
    launch_reduce(&jv, 1, st);
  }
}

// dA = s V^T X~, then the fixed-order reductions of the token-range splits.
void launch_bwd_k4(const BwdJob& jb, hipStream_t st) {
  const Layout& y = jb.y;
  {
    prof::Scope ps("k4_da", jb.T, jb.r, jb.K, jb.k4_flops, jb.k4_bytes);
    const dim3 grid((unsigned)cdiv(jb.K, SK_C), (unsigned)y.k4.n);
    LORA_RP_DISPATCH(jb.rp, launch(k4_kernel<RP>, grid, st, ps, jb.k4a));
  }
  RedJob jobs[4];
  int nj = 0;
  for (int i = 0; i < jb.nj; ++i) jobs[nj++] = jb.jobs[i];
  if (jb.has_ja) jobs[nj++] = jb.ja;
  if (nj) launch_reduce(jobs, nj, st);
}

void launch_bwd_plain(const BwdJob& jb, hipStream_t st) {
  const lora_linear* lin = jb.lin;
  const Layout& y = jb.y;
  const int64_t T = jb.T, K = jb.K, N = jb.N, r = jb.r;
  const bool bf = bf16_ops(lin->w_dtype);
  launch_bwd_k3(jb, st);
  // k4 first: it leaves the dropout keep bits that the bf16 dX product reads.
  launch_bwd_k4(jb, st);
  if (jb.dX) {
    if (bf) {
      GemmBf16Args a;
      memset(&a, 0, sizeof(a));
      a.A = jb.o.gbf; a.lda = N; a.ldb = K;
      set_w(a, lin);
      a.M = T; a.Nc = K; a.Kc = N; a.r = r;
      a.nslot = 1;
      a.sl[0] = bf16_dx_slot(jb);
      a.ksplit = y.gd.k.len; a.nsplit = y.gd.k.n;
      a.part = y.gd.k.n > 1 ? (float*)(jb.w + y.gdpart) : nullptr;
      launch_gemm_bf16(y.gd, false, a, st);
    } else {
      GemmF32Args a;
      memset(&a, 0, sizeof(a));
      a.A = jb.dY; a.lda = N; a.acn = lin->dora_mag; a.acd = lin->dora_norm;
      a.B = (const float*)lin->W; a.ldb = K;
      a.M = T; a.Nc = K; a.Kc = N;
      a.xa = jb.xv; a.XB = lin->A; a.r = r; a.xs = lin->scale; a.drop = jb.d;
      a.ksplit = y.gd.k.len; a.nsplit = y.gd.k.n;
      a.C = jb.dX;
      a.part = y.gd.k.n > 1 ? (float*)(jb.w + y.gdpart) : nullptr;
      launch_gemm_f32(y.gd, false, a, st);
    }
  }
}

// Linears of a group read one X: equal token count and input width.  Each
// is planned on its own, so their W types may differ.
int check_group(int n, const lora_linear* lins) {
  for (int i = 0; i < n; ++i) {
    const int rc = check_linear(&lins[i]);
    if (rc) return rc;
    if (lins[i].tokens != lins[0].tokens || lins[i].in_dim != lins[0].in_dim) return LORA_E_SHAPE;
  }
  return LORA_OK;
}

// Slots: adapters over one W with equal shapes (each has its own data,
// factors, dropout keys and DoRA magnitude).
int check_slots(int n, const lora_linear* lins) {
  const lora_linear& a = lins[0];
  for (int i = 0; i < n; ++i) {
    const lora_linear& b = lins[i];
    const int rc = check_linear(&b);
    if (rc) return rc;
    if (b.W != a.W || b.tokens != a.tokens || b.in_dim != a.in_dim || b.out_dim != a.out_dim ||
        b.rank != a.rank)
      return LORA_E_SHAPE;
    if (b.w_dtype != a.w_dtype) return LORA_E_DTYPE;
    if ((b.dora_mag == nullptr) != (a.dora_mag == nullptr)) return LORA_E_INVALID;
  }
  return LORA_OK;
}

// The slots' frozen products run as one product over their stacked rows when
// W is bf16, there is more than one slot, every slot covers whole 256-row
// tiles and the stacked operands stay within 32-bit offsets; otherwise the
// slots run one after another.
bool slots_stacked(int n, const lora_linear* lins) {
  const lora_linear& a = lins[0];
  if (n < 2 || !bf16_ops(a.w_dtype) || a.tokens % 256) return false;
  const int64_t M = n * a.tokens;
  return M * a.in_dim < (1ll << 30) && M * a.out_dim < (1ll << 30);
}

size_t slot_share_bytes(const lora_linear* L, int stack) {
  const Layout y = make_layout(L, stack);
  return rup((int64_t)std::max(y.fwd_bytes, y.bwd_bytes), 256);
}

}  // namespace

// =========================================================================
extern "C" {

size_t lora_qweight_layout(int32_t w_dtype, int64_t out_dim, int64_t in_dim, size_t* offsets) {
  size_t off[4], bytes[4];
  const size_t total = qweight_layout(w_dtype, out_dim, in_dim, off, bytes);
  if (total && offsets)
    for (int i = 0; i < 4; ++i) offsets[i] = off[i];
  return total;
}

int lora_set_bf16_config(int cfg) {
  if (cfg < -1 || cfg >= kBf16NCfg) return LORA_E_INVALID;
  g_bf16_cfg.store(cfg, std::memory_order_relaxed);
  return LORA_OK;
}

const char* lora_status_string(int s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_E_INVALID: return "invalid argument";
    case LORA_E_SHAPE: return "invalid shape";
    case LORA_E_DTYPE: return "unsupported dtype";
    case LORA_E_ALIGN: return "misaligned pointer or dimension";
    case LORA_E_WORKSPACE: return "workspace missing or too small";
    case LORA_E_NONFINITE: return "non-finite gradient: update vetoed";
    case LORA_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

double lora_scaling(double alpha, int64_t rank, int rslora) {
  if (rank <= 0) return NAN;
  return rslora ? alpha / sqrt((double)rank) : alpha / (double)rank;
}

double lora_lr_at(int64_t k, double lr, int schedule, int64_t warmup, int64_t total,
                  double lr_min) {
  if (schedule == 0) return lr;
  if (schedule != 1 || k < 0) return NAN;
  if (k < warmup) return lr * (double)(k + 1) / (double)warmup;
  const int64_t span = total - warmup > 1 ? total - warmup : 1;
  double prog = (double)(k - warmup) / (double)span;
  if (prog > 1.0) prog = 1.0;
  return lr_min + 0.5 * (lr - lr_min) * (1.0 + cos(M_PI * prog));
}

size_t lora_workspace_bytes(const lora_linear* lin) {
  if (check_linear(lin) != LORA_OK) return 0;
  const Layout y = make_layout(lin);
  return y.fwd_bytes > y.bwd_bytes ? y.fwd_bytes : y.bwd_bytes;
}

int lora_forward(const lora_linear* lin, const float* X, float* Y, float* U, float* Z,
                 const lora_dropout* drop, void* ws, size_t ws_bytes, void* stream) {
  FwdJob j;
  const int rc = prepare_fwd(lin, X, Y, U, Z, drop, ws, ws_bytes, j);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (j.split) launch_fwd_split<1>(&j, st);
  else launch_fwd_plain(j, st);
  return hip_status();
}

int lora_backward(const lora_linear* lin, const float* X, const float* dY, const float* U,
                  const float* Z, float* dX, float* dA, float* dB, float* dMag,
                  int accumulate, const lora_dropout* drop, void* ws, size_t ws_bytes,
                  void* stream) {
  BwdJob j;
  const int rc = prepare_bwd(lin, X, dY, U, Z, dX, dA, dB, dMag, accumulate, drop, ws, ws_bytes, j);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (j.split) launch_bwd_split<1>(&j, st);
  else launch_bwd_plain(j, st);
  return hip_status();
}

size_t lora_group_workspace_bytes(int n, const lora_linear* lins) {
  if (n < 1 || n > LORA_MAX_GROUP || !lins) return 0;
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (check_linear(&lins[i]) != LORA_OK) return 0;
    total += rup((int64_t)lora_workspace_bytes(&lins[i]), 256);
  }
  return total;
}

int lora_forward_group(int n, const lora_linear* lins, const float* X, float* const* Y,
                       float* const* U, float* const* Z, const lora_dropout* drops, void* ws,
                       size_t ws_bytes, void* stream) {
  if (n < 1 || n > LORA_MAX_GROUP || !lins || !Y || !U) return LORA_E_INVALID;
  int rc = check_group(n, lins);
  if (rc) return rc;
  const size_t need = lora_group_workspace_bytes(n, lins);
  if (need && (!ws || ws_bytes < need || !al16(ws))) return LORA_E_WORKSPACE;
  FwdJob jobs[LORA_MAX_GROUP];
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const size_t wi = rup((int64_t)lora_workspace_bytes(&lins[i]), 256);
    rc = prepare_fwd(&lins[i], X, Y[i], U[i], Z ? Z[i] : nullptr, drops ? &drops[i] : nullptr,
                     (char*)ws + off, wi, jobs[i]);
    if (rc) return rc;
    off += wi;
  }
  hipStream_t st = (hipStream_t)stream;
  if (n == 2 && jobs[0].split && jobs[1].split) {
    launch_fwd_split<2>(jobs, st);
  } else {
    for (int i = 0; i < n; ++i) {
      if (jobs[i].split) launch_fwd_split<1>(&jobs[i], st);
      else launch_fwd_plain(jobs[i], st);
    }
  }
  return hip_status();
}

int lora_backward_group(int n, const lora_linear* lins, const float* X, const float* const* dY,
                        const float* const* U, const float* const* Z, float* const* dX,
                        float* const* dA, float* const* dB, float* const* dMag, int accumulate,
                        const lora_dropout* drops, void* ws, size_t ws_bytes, void* stream) {
  if (n < 1 || n > LORA_MAX_GROUP || !lins || !dY || !U || !dA || !dB) return LORA_E_INVALID;
  int rc = check_group(n, lins);
  if (rc) return rc;
  const size_t need = lora_group_workspace_bytes(n, lins);
  if (need && (!ws || ws_bytes < need || !al16(ws))) return LORA_E_WORKSPACE;
  BwdJob jobs[LORA_MAX_GROUP];
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const size_t wi = rup((int64_t)lora_workspace_bytes(&lins[i]), 256);
    rc = prepare_bwd(&lins[i], X, dY[i], U[i], Z ? Z[i] : nullptr, dX ? dX[i] : nullptr, dA[i],
                     dB[i], dMag ? dMag[i] : nullptr, accumulate, drops ? &drops[i] : nullptr,
                     (char*)ws + off, wi, jobs[i]);
    if (rc) return rc;
    off += wi;
  }
  hipStream_t st = (hipStream_t)stream;
  if (n == 2 && jobs[0].split && jobs[1].split) {
    launch_bwd_split<2>(jobs, st);
  } else {
    for (int i = 0; i < n; ++i) {
      if (jobs[i].split) launch_bwd_split<1>(&jobs[i], st);
      else launch_bwd_plain(jobs[i], st);
    }
  }
  return hip_status();
}

static_assert(LORA_MAX_SLOTS <= BF16_MAX_SLOTS, "slot operands of the bf16 products");

size_t lora_slots_workspace_bytes(int n, const lora_linear* lins) {
  if (n < 1 || n > LORA_MAX_SLOTS || !lins || check_slots(n, lins) != LORA_OK) return 0;
  size_t total = 0;
  if (!slots_stacked(n, lins)) {
    for (int i = 0; i < n; ++i) total += rup((int64_t)lora_workspace_bytes(&lins[i]), 256);
    return total;
  }
  for (int i = 0; i < n; ++i) total += slot_share_bytes(&lins[i], n);
  const StackLayout z = make_stack_layout(&lins[0], n);
  return total + std::max(z.fwd_bytes, z.bwd_bytes);
}

int lora_forward_slots(int n, const lora_linear* lins, const float* const* X, float* const* Y,
                       float* const* U, float* const* Z, const lora_dropout* drops, void* ws,
                       size_t ws_bytes, void* stream) {
  if (n < 1 || n > LORA_MAX_SLOTS || !lins || !X || !Y || !U) return LORA_E_INVALID;
  int rc = check_slots(n, lins);
  if (rc) return rc;
  const size_t need = lora_slots_workspace_bytes(n, lins);
  if (need && (!ws || ws_bytes < need || !al16(ws))) return LORA_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  FwdJob jobs[LORA_MAX_SLOTS];
  const bool stacked = slots_stacked(n, lins);
  const int64_t T = lins[0].tokens, K = lins[0].in_dim, N = lins[0].out_dim;
  size_t off = 0;
  uint16_t* xbf = nullptr;
  StackLayout z;
  if (stacked) {
    for (int i = 0; i < n; ++i) off += slot_share_bytes(&lins[i], n);
    z = make_stack_layout(&lins[0], n);
    xbf = (uint16_t*)((char*)ws + off + z.xbf);
    off = 0;
  }
  for (int i = 0; i < n; ++i) {
    const size_t wi = stacked ? slot_share_bytes(&lins[i], n)
                              : (size_t)rup((int64_t)lora_workspace_bytes(&lins[i]), 256);
    rc = prepare_fwd(&lins[i], X[i], Y[i], U[i], Z ? Z[i] : nullptr, drops ? &drops[i] : nullptr,
                     (char*)ws + off, wi, jobs[i], stacked ? n : 1,
                     stacked ? xbf + (int64_t)i * T * K : nullptr);
    if (rc) return rc;
    off += wi;
  }
  if (!stacked) {
    for (int i = 0; i < n; ++i) {
      if (jobs[i].split) launch_fwd_split<1>(&jobs[i], st);
      else launch_fwd_plain(jobs[i], st);
    }
    return hip_status();
  }
  for (int i = 0; i < n; ++i) launch_fwd_down(jobs[i], st);
  {
    RedJob red[LORA_MAX_SLOTS];
    int nr = 0;
    for (int i = 0; i < n; ++i)
      if (jobs[i].has_ured) red[nr++] = jobs[i].ured;
    if (nr) launch_reduce(red, nr, st);
  }
  GemmBf16Args a;
  memset(&a, 0, sizeof(a));
  a.A = xbf; a.lda = K; a.ldb = K;
  set_w(a, &lins[0]);
  a.M = n * T; a.Nc = N; a.Kc = K; a.r = lins[0].rank;
  a.nslot = n; a.slot_rows = T;
  for (int i = 0; i < n; ++i) a.sl[i] = bf16_fwd_slot(jobs[i]);
  a.ksplit = z.gf.k.len; a.nsplit = z.gf.k.n;
  a.part = z.gf.k.n > 1 ? (float*)((char*)ws + off + z.gfpart) : nullptr;
  launch_gemm_bf16(z.gf, true, a, st);
  return hip_status();
}

int lora_backward_slots(int n, const lora_linear* lins, const float* const* X,
                        const float* const* dY, const float* const* U, const float* const* Z,
                        float* const* dX, float* const* dA, float* const* dB, float* const* dMag,
                        int accumulate, const lora_dropout* drops, void* ws, size_t ws_bytes,
                        void* stream) {
  if (n < 1 || n > LORA_MAX_SLOTS || !lins || !X || !dY || !U || !dA || !dB)
    return LORA_E_INVALID;
  int rc = check_slots(n, lins);
  if (rc) return rc;
  if (dX)
    for (int i = 0; i < n; ++i)
      if ((dX[i] == nullptr) != (dX[0] == nullptr)) return LORA_E_INVALID;
  const size_t need = lora_slots_workspace_bytes(n, lins);
  if (need && (!ws || ws_bytes < need || !al16(ws))) return LORA_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  BwdJob jobs[LORA_MAX_SLOTS];
  const bool stacked = slots_stacked(n, lins);
  const int64_t T = lins[0].tokens, K = lins[0].in_dim, N = lins[0].out_dim;
  const bool want_dx = dX && dX[0];
  size_t off = 0;
  uint16_t* gbf = nullptr;
  StackLayout z;
  if (stacked) {
    for (int i = 0; i < n; ++i) off += slot_share_bytes(&lins[i], n);
    z = make_stack_layout(&lins[0], n);
    gbf = (uint16_t*)((char*)ws + off + z.gbf);
    off = 0;
  }
  for (int i = 0; i < n; ++i) {
    const size_t wi = stacked ? slot_share_bytes(&lins[i], n)
                              : (size_t)rup((int64_t)lora_workspace_bytes(&lins[i]), 256);
    rc = prepare_bwd(&lins[i], X[i], dY[i], U[i], Z ? Z[i] : nullptr, dX ? dX[i] : nullptr,
                     dA[i], dB[i], dMag ? dMag[i] : nullptr, accumulate,
                     drops ? &drops[i] : nullptr, (char*)ws + off, wi, jobs[i], stacked ? n : 1,
                     stacked ? gbf + (int64_t)i * T * N : nullptr);
    if (rc) return rc;
    off += wi;
  }
  if (!stacked) {
    for (int i = 0; i < n; ++i) {
      if (jobs[i].split) launch_bwd_split<1>(&jobs[i], st);
      else launch_bwd_plain(jobs[i], st);
    }
    return hip_status();
  }
  for (int i = 0; i < n; ++i) launch_bwd_k3(jobs[i], st);
  for (int i = 0; i < n; ++i) launch_bwd_k4(jobs[i], st);   // keep bits before dX
  if (want_dx) {
    GemmBf16Args a;
    memset(&a, 0, sizeof(a));
    a.A = gbf; a.lda = N; a.ldb = K;
    set_w(a, &lins[0]);
    a.M = n * T; a.Nc = K; a.Kc = N; a.r = lins[0].rank;
    a.nslot = n; a.slot_rows = T;
    for (int i = 0; i < n; ++i) a.sl[i] = bf16_dx_slot(jobs[i]);
    a.ksplit = z.gd.k.len; a.nsplit = z.gd.k.n;
    a.part = z.gd.k.n > 1 ? (float*)((char*)ws + off + z.gdpart) : nullptr;
    launch_gemm_bf16(z.gd, false, a, st);
  }
  return hip_status();
}

size_t lora_grad_prepare_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return 4096 + 1024 * (sizeof(double) + sizeof(int)) + 256;
}

}  // extern "C"

// Scratch of lora_grad_prepare_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host the name is only a stand-in for
// the symbol); it takes the device address from hipGetSymbolAddress, once
// per device with that device current, and keeps it per device.
constexpr size_t kNoallocScratchBytes = 16640;   // lora_grad_prepare's workspace, any n
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

// The two gradient-norm passes over `ws` (per-block partials, flags and the
// {norm, clip} pair; every word read is written earlier in the same call).
int grad_prepare_on(const float* grads, int64_t n, int64_t n_pred_tokens, float max_norm,
                    float* d_scale, double* d_stats, double* h_norm, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t nb0 = clampi(cdiv(n, 8192), 1, 1024);
  const int64_t per = rup(cdiv(n, nb0), 1024);
  const int nb = (int)cdiv(n, per);
  char* w = (char*)ws;
  double* norm_out = (double*)w;                // {norm, clip}
  double* part = (double*)(w + 256);
  int* flags = (int*)(w + 256 + 1024 * sizeof(double));
  {
    prof::Scope ps("gradnorm_pass1", n, nb, 0, 2.0 * n, 4.0 * n);
    launch(gradnorm_pass1, dim3(nb), st, ps, grads, n, per, part, flags);
  }
  {
    prof::Scope ps("gradnorm_pass2", nb, 1, 0, 0.0, 12.0 * nb);
    launch(gradnorm_pass2, dim3(1), st, ps, (const double*)part, (const int*)flags, nb,
           n_pred_tokens, max_norm, d_scale, d_stats, norm_out);
  }
  if (hip_status()) return LORA_E_HIP;
  if (h_norm) {
    double host[2];
    if (hipMemcpyAsync(host, norm_out, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess)
      return LORA_E_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_E_HIP;
    *h_norm = host[0];
    if (std::isnan(host[0])) return LORA_E_NONFINITE;
  }
  return LORA_OK;
}

int check_grad_prepare(const float* grads, int64_t n, int64_t n_pred_tokens, float max_norm,
                       const float* d_scale) {
  if (!grads || !d_scale || n <= 0 || n_pred_tokens <= 0) return LORA_E_INVALID;
  if (!(max_norm >= 0.0f) || !std::isfinite(max_norm)) return LORA_E_INVALID;
  if (!al16(grads)) return LORA_E_ALIGN;
  return LORA_OK;
}

constexpr int kNoallocMaxDevices = 64;
std::once_flag scratch_once[kNoallocMaxDevices];
void* scratch_ptr[kNoallocMaxDevices];
hipError_t scratch_err[kNoallocMaxDevices];

// Device address of this device's scratch, or NULL when the device index or
// the symbol lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoallocMaxDevices) return nullptr;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int lora_grad_prepare(const float* grads, int64_t n, int64_t n_pred_tokens, float max_norm,
                      float* d_scale, double* d_stats, double* h_norm, void* ws,
                      size_t ws_bytes, void* stream) {
  if (int e = check_grad_prepare(grads, n, n_pred_tokens, max_norm, d_scale)) return e;
  if (!ws || !al16(ws) || ws_bytes < lora_grad_prepare_workspace_bytes(n)) return LORA_E_WORKSPACE;
  return grad_prepare_on(grads, n, n_pred_tokens, max_norm, d_scale, d_stats, h_norm, ws, stream);
}

int lora_grad_prepare_noalloc(const float* grads, int64_t n, int64_t n_pred_tokens,
                              float max_norm, float* d_scale, double* d_stats, double* h_norm,
                              void* stream) {
  if (int e = check_grad_prepare(grads, n, n_pred_tokens, max_norm, d_scale)) return e;
  if (lora_grad_prepare_workspace_bytes(n) > kNoallocScratchBytes) return LORA_E_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return LORA_E_HIP;
  return grad_prepare_on(grads, n, n_pred_tokens, max_norm, d_scale, d_stats, h_norm, ws, stream);
}

int lora_adamw_step(float* params, const float* grads, float* m, float* v,
                    const lora_segment* segs, int n_seg, const lora_adamw_hparams* hp,
                    const float* d_scale, void* stream) {
  if (!params || !grads || !m || !v || !segs || !hp || !d_scale) return LORA_E_INVALID;
  if (n_seg < 1 || n_seg > ADAM_MAX_SEG) return LORA_E_INVALID;
  if (!al16(params) || !al16(grads) || !al16(m) || !al16(v)) return LORA_E_ALIGN;
  if (!(hp->lr >= 0.0) || !std::isfinite(hp->lr) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
      !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->eps > 0.0) ||
      !std::isfinite(hp->weight_decay) || !std::isfinite(hp->plus_ratio) || hp->t < 1)
    return LORA_E_INVALID;
  AdamSegs S;
  memset(&S, 0, sizeof(S));
  int64_t blocks = 0;
  for (int i = 0; i < n_seg; ++i) {
    const lora_segment& g = segs[i];
    if (g.offset < 0 || g.count < 0 || g.kind < 0 || g.kind > 2) return LORA_E_INVALID;
    if (g.offset % 4 || g.count % 4) return LORA_E_ALIGN;
    S.off[i] = g.offset;
    S.cnt[i] = g.count;
    S.kind[i] = g.kind;
    S.blk[i] = blocks;
    blocks += cdiv(g.count, 1024);
  }
  S.blk[n_seg] = blocks;
  S.n = n_seg;
  AdamHp H;
  H.b1 = (float)hp->beta1;
  H.b2 = (float)hp->beta2;
  H.one_m_b1 = (float)(1.0 - hp->beta1);
  H.one_m_b2 = (float)(1.0 - hp->beta2);
  H.eps = (float)hp->eps;
  H.bc1 = (float)(1.0 - pow(hp->beta1, (double)hp->t));
  H.bc2 = (float)(1.0 - pow(hp->beta2, (double)hp->t));
  H.rate[0] = (float)hp->lr;
  H.rate[1] = (float)(hp->lr * hp->plus_ratio);
  H.rate[2] = (float)hp->lr;
  H.decay[0] = (float)(hp->lr * hp->weight_decay);
  H.decay[1] = 0.0f;
  H.decay[2] = 0.0f;
  if (blocks == 0) return LORA_OK;
  int64_t total = 0;
  for (int i = 0; i < n_seg; ++i) total += segs[i].count;
  prof::Scope ps("adamw", total, n_seg, 0, 0.0, 28.0 * total);
  launch(adamw_kernel, dim3((unsigned)blocks), (hipStream_t)stream, ps, params, grads, m, v, S, H,
         d_scale);
  return hip_status();
}

int lora_dropout_mask(const lora_dropout* drop, int64_t tokens, int64_t in_dim, uint8_t* mask,
                      void* stream) {
  if (!mask || tokens <= 0 || in_dim <= 0) return LORA_E_INVALID;
  if (!drop_valid(drop)) return LORA_E_INVALID;
  const DropParams d = make_drop(drop);
  const int64_t n = tokens * in_dim;
  prof::Scope ps("dropout_mask", tokens, in_dim, 0, 0.0, (double)n);
  launch(dropout_mask_kernel, dim3((unsigned)cdiv(n, 256)), (hipStream_t)stream, ps, d, tokens,
         in_dim, mask);
  return hip_status();
}

// Row-norm grid: DN_ROWS rows per block in x (32 per wave), column splits of
// cpw 64-column chunks in y.  The kernel holds dn_waves_per_simd(rp) waves per
// SIMD, so a launch of W waves takes about ceil(W / slots) rounds of cpw
// chunks each plus a start-up of about one chunk per round; cpw is the one
// that minimises that estimate.
struct DoraNormPlan {
  int64_t nb, nsplit, cpw;
};
DoraNormPlan dora_norm_plan(int64_t N, int64_t K, int rp, bool split, int mode = 0) {
  DoraNormPlan q;
  q.nb = cdiv(N, (int64_t)DN_ROWS);
  const int64_t nch = cdiv(K, (int64_t)DN_CHUNK);
  const int64_t waves = 4 * q.nb;
  const int64_t slots = 1024 * (int64_t)dn_waves_per_simd(rp, mode);
  q.cpw = nch;
  q.nsplit = 1;
  if (!split) return q;
  int64_t best = cdiv(waves, slots) * (q.cpw + 1);
  for (int64_t cpw = nch - 1; cpw >= 1; --cpw) {
    const int64_t s = cdiv(nch, cpw);
    if (s > 65535) break;
    const int64_t cost = cdiv(waves * s, slots) * (cpw + 1);
    if (cost < best) {
      best = cost;
      q.cpw = cpw;
      q.nsplit = s;
    }
  }
  return q;
}

int check_row_norm_linear(const lora_linear* lin) {
  if (!lin) return LORA_E_INVALID;
  // in_dim <= 2^22 keeps the kernel's buffer offsets within 32 bits (for
  // quantized W also every plane: in_dim * out_dim < 2^30).
  if (lin->in_dim <= 0 || lin->out_dim <= 0 || lin->in_dim > (1 << 22)) return LORA_E_SHAPE;
  const int32_t f = lin->w_dtype;
  if (f != LORA_F32 && f != LORA_BF16 && !wq_quantized(f)) return LORA_E_DTYPE;
  if (wq_quantized(f) &&
      (lin->in_dim % wq_super(f) || lin->in_dim * lin->out_dim >= (1ll << 30)))
    return LORA_E_SHAPE;
  if (!lin->W) return LORA_E_INVALID;
  if ((lin->A == nullptr) != (lin->B == nullptr)) return LORA_E_INVALID;
  if (lin->A && (lin->rank <= 0 || lin->rank > 128)) return LORA_E_SHAPE;
  if (!std::isfinite(lin->scale)) return LORA_E_INVALID;
  return LORA_OK;
}

// Bytes of W per element for the launch records, and whether W and A rows
// allow the row pass's 16-byte loads (quantized W is read in runs).
double row_pass_w_bytes(const lora_linear* lin) {
  if (!wq_quantized(lin->w_dtype)) return lin->w_dtype == LORA_BF16 ? 2.0 : 4.0;
  size_t off[4], bytes[4];
  qweight_layout(lin->w_dtype, lin->out_dim, lin->in_dim, off, bytes);
  return (double)(bytes[0] + bytes[1] + bytes[2] + bytes[3]) /
         ((double)lin->out_dim * (double)lin->in_dim);
}
int row_pass_vec(const lora_linear* lin) {
  const bool a_ok = !lin->A || (al16(lin->A) && lin->in_dim % 4 == 0);
  if (wq_quantized(lin->w_dtype)) return a_ok;
  const int64_t wsz = lin->w_dtype == LORA_BF16 ? 2 : 4;
  return al16(lin->W) && (lin->in_dim * wsz) % 16 == 0 && a_ok;
}
void launch_row_pass_quant(const lora_linear* lin, int mode, bool lora_on, int rp, bool out_bf16,
                           dim3 grid, hipStream_t st, const prof::Scope& ps, RowPassArgs& a) {
  a.q = qplanes(lin);
  switch (lin->w_dtype) {
    case LORA_Q8_0: launch_row_pass_wq<WQ_Q8_0>(mode, lora_on, rp, out_bf16, grid, st, ps, a); break;
    case LORA_Q4_0: launch_row_pass_wq<WQ_Q4_0>(mode, lora_on, rp, out_bf16, grid, st, ps, a); break;
    case LORA_Q4_K: launch_row_pass_wq<WQ_Q4_K>(mode, lora_on, rp, out_bf16, grid, st, ps, a); break;
    default: launch_row_pass_wq<WQ_Q6_K>(mode, lora_on, rp, out_bf16, grid, st, ps, a); break;
  }
}

size_t lora_dora_row_norms_workspace_bytes(const lora_linear* lin) {
  if (check_row_norm_linear(lin) != LORA_OK) return 0;
  const DoraNormPlan q =
      dora_norm_plan(lin->out_dim, lin->in_dim, lin->A ? rank_pad(lin->rank) : 16, true);
  return q.nsplit > 1 ? sizeof(double) * q.nsplit * lin->out_dim : 0;
}

int lora_dora_row_norms(const lora_linear* lin, float* out_norm, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const int rc = check_row_norm_linear(lin);
  if (rc != LORA_OK) return rc;
  if (!out_norm) return LORA_E_INVALID;
  const bool lora_on = lin->A != nullptr;
  const int64_t N = lin->out_dim, K = lin->in_dim, r = lora_on ? lin->rank : 0;
  const int rp = rank_pad(r);
  const DoraNormPlan q = dora_norm_plan(N, K, lora_on ? rp : 16, workspace != nullptr);
  if (q.nsplit > 1 && workspace_bytes < sizeof(double) * q.nsplit * N) return LORA_E_WORKSPACE;
  const double wsz = row_pass_w_bytes(lin);
  RowPassArgs a;
  memset(&a, 0, sizeof(a));
  a.W = lin->W;
  a.N = N;
  a.K = K;
  a.A = lin->A;
  a.B = lin->B;
  a.r = (int)r;
  a.s = lin->scale;
  a.cpw = (int)q.cpw;
  a.vec = row_pass_vec(lin);
  a.part = static_cast<double*>(workspace);
  a.out = out_norm;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)q.nb, (unsigned)q.nsplit);
  {
    prof::Scope ps("dora_rownorm", N, K, r, 2.0 * N * K * r + 3.0 * N * K,
                   wsz * N * K + 4.0 * r * (N + K) + (q.nsplit > 1 ? 8.0 : 4.0) * N);
    if (wq_quantized(lin->w_dtype)) {
      launch_row_pass_quant(lin, 0, lora_on, rp, false, grid, st, ps, a);
    } else if (!lora_on) {
      if (lin->w_dtype == LORA_BF16) launch(row_pass_kernel<uint16_t, 16, false, 0, float>, grid, st, ps, a);
      else launch(row_pass_kernel<float, 16, false, 0, float>, grid, st, ps, a);
    } else if (lin->w_dtype == LORA_BF16) {
      LORA_RP_DISPATCH(rp, launch(row_pass_kernel<uint16_t, RP, true, 0, float>, grid, st, ps, a));
    } else {
      LORA_RP_DISPATCH(rp, launch(row_pass_kernel<float, RP, true, 0, float>, grid, st, ps, a));
    }
  }
  if (q.nsplit > 1) {
    prof::Scope ps("dora_norm_finish", N, q.nsplit, 0, (double)N * q.nsplit,
                   8.0 * N * q.nsplit + 4.0 * N);
    launch(dora_norm_finish_kernel, dim3((unsigned)cdiv(N, 256)), st, ps, a.part,
           (int)q.nsplit, N, out_norm);
  }
  return hip_status();
}

namespace {

// Batched DoRA norms: bf16-W linears with LoRA factors (rank <= 64) go
// through the expansion kernels (normbatch.hpp), adjacent linears over one W
// stacked as slots of one job; the rest take lora_dora_row_norms one by one.
struct NbJob {
  int first, S;             // lins[first .. first + S - 1]
  int64_t N, K, Kp, klen;
  int nsplit, RP, C, r;
  size_t parts, P, G, wsq;  // workspace offsets within the job's chunk
};

bool nb_eligible(const lora_linear* l) {
  return l->w_dtype == LORA_BF16 && l->A != nullptr && l->rank <= NB_MAX_RP &&
         l->in_dim % 8 == 0 && al16(l->W);
}
bool nb_same_w(const lora_linear* a, const lora_linear* b) {
  return a->W == b->W && a->out_dim == b->out_dim && a->in_dim == b->in_dim &&
         a->rank == b->rank;
}
size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Contraction splits: about 3072 per tile, whole steps of 32, none empty
// (splits of 1280, twice the tiles per launch, measured no faster and leave
// the combine more partials to sum).
constexpr int64_t kNbSplitLen = 3072;

// Jobs of the eligible linears in order, with their workspace offsets
// inside their chunk of NB_MAX_JOBS jobs; returns the largest chunk's bytes.
size_t nb_plan(int n, const lora_linear* lins, std::vector<NbJob>& jobs) {
  jobs.clear();
  for (int i = 0; i < n;) {
    if (!nb_eligible(&lins[i])) {
      ++i;
      continue;
    }
    NbJob j;
    memset(&j, 0, sizeof(j));
    j.first = i;
    j.S = 1;
    while (j.S < NB_MAX_SLOTS && i + j.S < n && nb_eligible(&lins[i + j.S]) &&
           nb_same_w(&lins[i], &lins[i + j.S]))
      ++j.S;
    const lora_linear* l = &lins[i];
    j.N = l->out_dim;
    j.K = l->in_dim;
    j.r = (int)l->rank;
    j.RP = (int)rup(l->rank, 32);
    j.C = j.S * j.RP;
    j.Kp = rup(j.K, NB_KS);
    const int64_t ns = cdiv(j.Kp, kNbSplitLen);
    j.klen = rup(cdiv(j.Kp, ns), NB_KS);
    j.nsplit = (int)cdiv(j.Kp, j.klen);
    jobs.push_back(j);
    i += j.S;
  }
  size_t best = 0, cur = 0;
  for (size_t k = 0; k < jobs.size(); ++k) {
    if (k % NB_MAX_JOBS == 0) cur = 0;
    NbJob& j = jobs[k];
    j.parts = cur;
    cur += a256((size_t)j.S * 3 * j.RP * j.Kp * 2);
    j.P = cur;
    cur += a256((size_t)j.nsplit * j.N * j.C * 4);
    j.G = cur;
    cur += a256((size_t)j.nsplit * 3 * j.S * j.RP * j.C * 4);
    j.wsq = cur;
    cur += a256((size_t)j.nsplit * j.N * 8);
    best = std::max(best, cur);
  }
  return best;
}

// Split, products and combine of jobs[c0, c1) on one stream.
void nb_launch(const lora_linear* lins, float* const* out, const std::vector<NbJob>& jobs,
               size_t c0, size_t c1, char* w, hipStream_t st) {
  {
    NbSplitArgs a;
    memset(&a, 0, sizeof(a));
    int64_t g = 0;
    double by = 0.0;
    for (size_t k = c0; k < c1; ++k) {
      const NbJob& j = jobs[k];
      NbSplitJob& s = a.job[k - c0];
      for (int q = 0; q < j.S; ++q) s.A[q] = lins[j.first + q].A;
      s.parts = reinterpret_cast<uint16_t*>(w + j.parts);
      s.K = j.K;
      s.Kp = j.Kp;
      s.r = j.r;
      s.RP = j.RP;
      s.S = j.S;
      s.g0 = g;
      g += (int64_t)j.S * j.RP * j.Kp / 8;
      by += 4.0 * j.S * j.r * j.K + 6.0 * j.S * j.RP * j.Kp;
    }
    a.njobs = (int)(c1 - c0);
    a.ngroups = g;
    prof::Scope ps("dora_norm_split", g, a.njobs, 0, 0.0, by);
    launch(nb_split_kernel, dim3((unsigned)cdiv(g, 256)), st, ps, a);
  }
  {
    NbProdArgs a;
    memset(&a, 0, sizeof(a));
    int64_t tiles = 0, nsum = 0;
    double fl = 0.0, by = 0.0;
    int ni = 0;
    for (size_t k = c0; k < c1; ++k)   // each job's P tiles, then its G tiles
      for (int pass = 0; pass < 2; ++pass) {
        const NbJob& j = jobs[k];
        NbItem& it = a.it[ni++];
        const bool P = pass == 0;
        it.M = P ? static_cast<const uint16_t*>(lins[j.first].W)
                 : reinterpret_cast<const uint16_t*>(w + j.parts);
        it.parts = reinterpret_cast<const uint16_t*>(w + j.parts);
        it.out = reinterpret_cast<float*>(w + (P ? j.P : j.G));
        it.wsq = P ? reinterpret_cast<double*>(w + j.wsq) : nullptr;
        it.rows = P ? j.N : 3ll * j.S * j.RP;
        it.ldm = P ? j.K : j.Kp;
        it.K = j.K;
        it.Kp = j.Kp;
        it.klen = j.klen;
        it.C = j.C;
        it.RP = j.RP;
        it.nsplit = j.nsplit;
        it.ncolt = (int)cdiv(j.C, NB_TN);
        it.tile0 = tiles;
        tiles += cdiv(it.rows, NB_TM) * it.nsplit * it.ncolt;
        fl += 6.0 * it.rows * j.C * j.K;
        by += (P ? 2.0 * j.N * j.K + 8.0 * j.nsplit * j.N : 0.0) + 6.0 * j.C * j.Kp +
              4.0 * j.nsplit * it.rows * j.C;
        if (P) nsum += j.N;
      }
    a.nitems = ni;
    prof::Scope ps("dora_norm_prod", nsum, jobs[c0].C, jobs[c0].K, fl, by);
    launch(nb_prod_kernel, dim3((unsigned)tiles), st, ps, a);
  }
  {
    NbFinArgs a;
    memset(&a, 0, sizeof(a));
    int64_t blocks = 0;
    double by = 0.0;
    for (size_t k = c0; k < c1; ++k) {
      const NbJob& j = jobs[k];
      NbFinJob& f = a.job[k - c0];
      f.P = reinterpret_cast<const float*>(w + j.P);
      f.wsq = reinterpret_cast<const double*>(w + j.wsq);
      f.G = reinterpret_cast<const float*>(w + j.G);
      for (int q = 0; q < j.S; ++q) {
        f.B[q] = lins[j.first + q].B;
        f.out[q] = out[j.first + q];
        f.s[q] = lins[j.first + q].scale;
      }
      f.N = j.N;
      f.C = j.C;
      f.RP = j.RP;
      f.S = j.S;
      f.r = j.r;
      f.nsplit = j.nsplit;
      f.blk0 = blocks;
      blocks += j.S * cdiv(j.N, NB_FIN_ROWS);
      by += (double)j.S * j.N * (4.0 * j.nsplit * j.RP + 8.0 * j.nsplit + 4.0 * j.r + 4.0);
    }
    a.njobs = (int)(c1 - c0);
    prof::Scope ps("dora_norm_combine", blocks, a.njobs, 0, 0.0, by);
    launch(nb_finish_kernel, dim3((unsigned)blocks), st, ps, a);
  }
}

}  // namespace

size_t lora_dora_row_norms_batch_workspace_bytes(int n, const lora_linear* lins) {
  if (n < 1 || !lins) return 0;
  for (int i = 0; i < n; ++i)
    if (check_row_norm_linear(&lins[i]) != LORA_OK) return 0;
  std::vector<NbJob> jobs;
  size_t need = nb_plan(n, lins, jobs);
  for (int i = 0; i < n; ++i)
    if (!nb_eligible(&lins[i])) need = std::max(need, lora_dora_row_norms_workspace_bytes(&lins[i]));
  return need;
}

int lora_dora_row_norms_batch(int n, const lora_linear* lins, float* const* out_norms,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 1 || !lins || !out_norms) return LORA_E_INVALID;
  for (int i = 0; i < n; ++i) {
    const int rc = check_row_norm_linear(&lins[i]);
    if (rc != LORA_OK) return rc;
    if (!out_norms[i]) return LORA_E_INVALID;
  }
  const size_t need = lora_dora_row_norms_batch_workspace_bytes(n, lins);
  if (need && (!workspace || workspace_bytes < need)) return LORA_E_WORKSPACE;
  if (need && !al16(workspace)) return LORA_E_ALIGN;
  std::vector<NbJob> jobs;
  nb_plan(n, lins, jobs);
  hipStream_t st = (hipStream_t)stream;
  for (size_t c0 = 0; c0 < jobs.size(); c0 += NB_MAX_JOBS)
    nb_launch(lins, out_norms, jobs, c0, std::min(jobs.size(), c0 + NB_MAX_JOBS),
              static_cast<char*>(workspace), st);
  for (int i = 0; i < n; ++i)
    if (!nb_eligible(&lins[i])) {
      const int rc = lora_dora_row_norms(&lins[i], out_norms[i], workspace, workspace_bytes, stream);
      if (rc != LORA_OK) return rc;
    }
  return hip_status();
}

// Merge for export: the same row pass, writing c (W + s B A) instead of
// summing its squares; the bf16 rounding error goes to per-wave partials
// (the workspace) and one fixed-order finish.
size_t lora_merge_workspace_bytes(const lora_linear* lin) {
  if (check_row_norm_linear(lin) != LORA_OK) return 0;
  const DoraNormPlan q =
      dora_norm_plan(lin->out_dim, lin->in_dim, lin->A ? rank_pad(lin->rank) : 16, true, 1);
  return sizeof(double) * q.nb * q.nsplit * 4;
}

int lora_merge(const lora_linear* lin, void* W_out, int out_dtype, double* rmse, void* workspace,
               size_t workspace_bytes, void* stream) {
  const int rc = check_row_norm_linear(lin);
  if (rc != LORA_OK) return rc;
  if (!W_out) return LORA_E_INVALID;
  if (out_dtype != LORA_F32 && out_dtype != LORA_BF16) return LORA_E_DTYPE;
  if ((lin->dora_mag == nullptr) != (lin->dora_norm == nullptr)) return LORA_E_INVALID;
  const bool lora_on = lin->A != nullptr;
  const int64_t N = lin->out_dim, K = lin->in_dim, r = lora_on ? lin->rank : 0;
  const int rp = rank_pad(r);
  const DoraNormPlan q = dora_norm_plan(N, K, lora_on ? rp : 16, true, 1);
  const bool want_err = rmse != nullptr && out_dtype == LORA_BF16;
  const size_t need = sizeof(double) * q.nb * q.nsplit * 4;
  if (want_err && (!workspace || workspace_bytes < need)) return LORA_E_WORKSPACE;
  const double wsz = row_pass_w_bytes(lin);
  const size_t osz = out_dtype == LORA_BF16 ? 2 : 4;
  RowPassArgs a;
  memset(&a, 0, sizeof(a));
  a.W = lin->W;
  a.N = N;
  a.K = K;
  a.A = lin->A;
  a.B = lin->B;
  a.r = (int)r;
  a.s = lin->scale;
  a.cpw = (int)q.cpw;
  a.vec = row_pass_vec(lin);
  a.wout = W_out;
  a.vec_out = al16(W_out) && (K * osz) % 16 == 0;
  a.mag = lin->dora_mag;
  a.nrm = lin->dora_norm;
  a.epart = want_err ? static_cast<double*>(workspace) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)q.nb, (unsigned)q.nsplit);
  {
    prof::Scope ps("merge", N, K, r, 2.0 * N * K * r + 3.0 * N * K,
                   (wsz + osz) * N * K + 4.0 * r * (N + K));
#define LORA_MERGE_LAUNCH(WT_, OT_)                                                            \
  if (!lora_on) launch(row_pass_kernel<WT_, 16, false, 1, OT_>, grid, st, ps, a);             \
  else LORA_RP_DISPATCH(rp, launch(row_pass_kernel<WT_, RP, true, 1, OT_>, grid, st, ps, a));
    if (wq_quantized(lin->w_dtype)) {
      launch_row_pass_quant(lin, 1, lora_on, rp, out_dtype == LORA_BF16, grid, st, ps, a);
    } else if (lin->w_dtype == LORA_BF16) {
      if (out_dtype == LORA_BF16) { LORA_MERGE_LAUNCH(uint16_t, uint16_t) }
      else { LORA_MERGE_LAUNCH(uint16_t, float) }
    } else {
      if (out_dtype == LORA_BF16) { LORA_MERGE_LAUNCH(float, uint16_t) }
      else { LORA_MERGE_LAUNCH(float, float) }
    }
#undef LORA_MERGE_LAUNCH
  }
  if (rmse) {   // float32 output: no partials, the finish writes 0
    prof::Scope ps("merge_rmse", N, K, 0, 0.0, want_err ? (double)need : 8.0);
    launch(rmse_finish_kernel, dim3(1), st, ps, (const double*)a.epart,
           want_err ? (int64_t)(q.nb * q.nsplit * 4) : (int64_t)0, (double)N * (double)K, rmse);
  }
  return hip_status();
}

// ------------------------------------------------------------ profiling ---
int lora_profile_begin(int max_launches) {
  if (max_launches <= 0) return LORA_E_INVALID;
  prof::State& s = prof::state();
  const size_t need = 2 * (size_t)max_launches;
  while (s.events.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return LORA_E_HIP;
    s.events.push_back(e);
  }
  s.recs.clear();
  s.used = 0;
  s.on = true;
  return LORA_OK;
}

int lora_profile_end(lora_profile_entry* out, int max_entries) {
  prof::State& s = prof::state();
  if (!s.on) return LORA_E_INVALID;
  s.on = false;
  if (hipDeviceSynchronize() != hipSuccess) return LORA_E_HIP;
  int n = 0;
  for (const prof::Rec& r : s.recs) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, s.events[r.ev], s.events[r.ev + 1]) != hipSuccess) return LORA_E_HIP;
    int j = 0;
    while (j < n && !(out[j].kernel == r.name && out[j].M == r.M && out[j].N == r.N &&
                      out[j].K == r.K))
      ++j;
    if (j == n) {
      if (n == max_entries || !out) continue;
      out[n] = {r.name, r.M, r.N, r.K, 0, 0.0, r.flops, r.bytes};
      ++n;
    }
    out[j].launches += 1;
    out[j].total_ms += (double)ms;
  }
  s.recs.clear();
  s.used = 0;
  return n;
}

}  // extern "C"
