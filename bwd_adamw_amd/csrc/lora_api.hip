// liblora: C-ABI entry points (include/lora.h) over the gfx950 kernels.
//
// Every entry point validates all arguments before enqueueing anything,
// plans its launches from the shapes alone (so equal shapes always give the
// same split structure and bitwise-equal results), carves split partials out
// of the caller's workspace and enqueues on the caller's stream.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "../../include/lora.h"
#include "common.hpp"
#include "fused.hpp"
#include "gemm_bf16.hpp"
#include "gemm_f32.hpp"
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

// Row range of the rank-side backward kernels: whole T (results written
// directly, no reduction launch) when T is short or the column strips alone
// fill the chip; otherwise split to about 512 blocks.
Split plan_rows(int64_t T, int64_t strips) {
  if (T <= 256 || strips >= 256) return {rup(T, SK_T), 1};
  return plan_split(T, strips, 512, SK_T, SK_T);
}

struct GemmPlan {
  int bm, bn;
  Split k;           // contraction split across blocks (fp32 only)
  int cfg;           // bf16 kernel configuration (kBf16Cfg)
};

// bf16 kernel configurations, in order of preference per direction: tile,
// threads, wave rows, K-step, stages in flight, and the directions (1
// forward, 2 dX) that use it.  dX's transposing loads take more registers
// per stage, so its wide tiles keep a single stage (chosen by measurement on
// the Qwen3-4B-shaped projections).
struct Bf16Cfg {
  int bm, bn, nt, wgm, bk, depth, dirs;
};
#define LORA_BF16_CFGS(X)             \
  X(0, 256, 256, 512, 2, 32, 3, 1)    \
  X(1, 256, 256, 512, 2, 64, 1, 2)    \
  X(2, 256, 128, 512, 2, 64, 2, 1)    \
  X(3, 256, 128, 512, 2, 64, 1, 2)    \
  X(4, 128, 128, 512, 2, 64, 2, 3)
constexpr Bf16Cfg kBf16Cfg[] = {
#define LORA_CFG_ROW(i, bm, bn, nt, wgm, bk, d, dirs) {bm, bn, nt, wgm, bk, d, dirs},
    LORA_BF16_CFGS(LORA_CFG_ROW)
#undef LORA_CFG_ROW
};
constexpr int kBf16NCfg = sizeof(kBf16Cfg) / sizeof(kBf16Cfg[0]);

// bf16: the first configuration whose grid still covers most of the 256
// CUs.  fp32: 128x128 when that fills the chip, else 64x64 with the
// contraction split across blocks until about 256 blocks run.
GemmPlan plan_gemm(int64_t M, int64_t Nc, int64_t Kc, bool bf16, bool dx) {
  if (bf16) {
    for (int i = 0; i < kBf16NCfg; ++i) {
      const Bf16Cfg& c = kBf16Cfg[i];
      if (!(c.dirs & (dx ? 2 : 1))) continue;
      if (cdiv(M, c.bm) * cdiv(Nc, c.bn) >= 200 || i == kBf16NCfg - 1)
        return {c.bm, c.bn, {Kc, 1}, i};
    }
  }
  if (cdiv(M, 128) * cdiv(Nc, 128) >= 256) return {128, 128, {rup(Kc, 32), 1}, 0};
  const int64_t tiles = cdiv(M, 64) * cdiv(Nc, 64);
  return {64, 64, plan_split(Kc, tiles, 256, 32, 128), 0};
}

// Short chunks: the contraction is split across blocks, and each linear runs
// as two launches per direction with the rank-side kernels beside the GEMM
// (fused.hpp).  The epilogue keeps U or V rows in LDS, hence the rank limit.
bool use_split_path(const GemmPlan& g, int64_t r, bool bf16) {
  return !bf16 && g.k.n > 1 && g.bm == 64 && r <= EPI_MAX_RANK;
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
  f.ntn = cdiv(Nc, 64);
  f.ntm = cdiv(M, 64);
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
  int64_t strips;      // 64-column strips of dY (k3 grid x): V partial count
  bool vreduce;        // V partials summed by a separate launch
  size_t upart, xbf, gfpart;                          // forward
  size_t vpart, v, dbpart, dmpart, gbf, gdpart, dapart;   // backward
  size_t fwd_bytes, bwd_bytes;
};

size_t carve(size_t& off, size_t bytes) {
  const size_t at = off;
  off += (bytes + 255) & ~size_t(255);
  return at;
}

Layout make_layout(const lora_linear* L) {
  Layout y;
  const int64_t T = L->tokens, K = L->in_dim, N = L->out_dim, r = L->rank;
  const bool bf = L->w_dtype == LORA_BF16;
  y.down = plan_split(K, cdiv(T, SK_T), 512, SK_C, SK_C);
  y.strips = cdiv(N, SK_C);
  y.k3 = plan_rows(T, y.strips);
  y.k4 = plan_rows(T, cdiv(K, SK_C));
  y.gf = plan_gemm(T, N, K, bf, false);
  y.gd = plan_gemm(T, K, N, bf, true);
  // Beside the split GEMM the down projection needs no parallelism of its
  // own: 256 columns per block keeps its partials few for the epilogue.
  if (use_split_path(y.gf, r, bf)) {
    const int64_t len = rup(cdiv(K, cdiv(K, 256)), SK_C);
    y.down = {len, (int)cdiv(K, len)};
  }
  const double vbytes = 4.0 * y.strips * T * r;
  y.vreduce = y.strips > 1 && vbytes * (cdiv(K, y.gd.bn) + cdiv(K, SK_C)) > kPartialRereadBytes;
  size_t off = 0;
  y.upart = carve(off, y.down.n > 1 ? sizeof(float) * y.down.n * T * r : 0);
  y.xbf = carve(off, bf ? sizeof(uint16_t) * T * K : 0);
  y.gfpart = carve(off, y.gf.k.n > 1 ? sizeof(float) * y.gf.k.n * T * N : 0);
  y.fwd_bytes = off;
  off = 0;
  y.vpart = carve(off, y.strips > 1 ? sizeof(float) * y.strips * T * r : 0);
  y.v = carve(off, sizeof(float) * T * r);
  y.dbpart = carve(off, y.k3.n > 1 ? sizeof(float) * y.k3.n * N * r : 0);
  y.dmpart = carve(off, (L->dora_mag && y.k3.n > 1) ? sizeof(float) * y.k3.n * N : 0);
  y.gbf = carve(off, bf ? sizeof(uint16_t) * T * N : 0);
  y.gdpart = carve(off, y.gd.k.n > 1 ? sizeof(float) * y.gd.k.n * T * K : 0);
  y.dapart = carve(off, y.k4.n > 1 ? sizeof(float) * y.k4.n * r * K : 0);
  y.bwd_bytes = off;
  return y;
}

int check_linear(const lora_linear* L) {
  if (!L) return LORA_E_INVALID;
  if (L->tokens <= 0 || L->in_dim <= 0 || L->out_dim <= 0 || L->rank <= 0) return LORA_E_SHAPE;
  if (L->rank > 128 || L->rank > L->in_dim || L->rank > L->out_dim) return LORA_E_SHAPE;
  if (L->w_dtype != LORA_F32 && L->w_dtype != LORA_BF16) return LORA_E_DTYPE;
  // bf16 operands are read with 32-bit byte offsets.
  if (L->w_dtype == LORA_BF16 &&
      (L->in_dim * L->out_dim >= (1ll << 30) || L->tokens * L->in_dim >= (1ll << 30) ||
       L->tokens * L->out_dim >= (1ll << 30)))
    return LORA_E_SHAPE;
  const int64_t q = L->w_dtype == LORA_BF16 ? 8 : 4;
  if (L->in_dim % q || L->out_dim % q || L->rank % 4) return LORA_E_ALIGN;
  if (!L->W || !L->A || !L->B) return LORA_E_INVALID;
  if (!al16(L->W) || !al16(L->A) || !al16(L->B)) return LORA_E_ALIGN;
  if ((L->dora_mag == nullptr) != (L->dora_norm == nullptr)) return LORA_E_INVALID;
  if ((L->dora_mag && !al16(L->dora_mag)) || (L->dora_norm && !al16(L->dora_norm)))
    return LORA_E_ALIGN;
  if (!std::isfinite(L->scale)) return LORA_E_INVALID;
  return LORA_OK;
}

int hip_status() { return hipGetLastError() == hipSuccess ? LORA_OK : LORA_E_HIP; }

// ----------------------------------------------------------- launchers ---
// Every kernel goes through here: 256 threads per block, on the caller's
// stream, with the profile's packet-timestamp events when one is open.
template <typename F, typename... Args>
void launch_n(F kern, dim3 grid, unsigned threads, hipStream_t st, const prof::Scope& ps,
              Args... args) {
  hipExtLaunchKernelGGL(kern, grid, dim3(threads), 0, st, ps.start(), ps.stop(), 0, args...);
}
template <typename F, typename... Args>
void launch(F kern, dim3 grid, hipStream_t st, const prof::Scope& ps, Args... args) {
  launch_n(kern, grid, 256u, st, ps, args...);
}

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
    J.blk[i] = blocks;
    blocks += cdiv(jobs[i].n, 256);
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
#define LORA_F32_TILE(BM_)                                                                   \
  if (g.bm == BM_) {                                                                         \
    if (fwd) {                                                                               \
      if (exact) launch(gemm_f32_kernel<BM_, BM_, true, true, false>, grid, st, ps, a);      \
      else launch(gemm_f32_kernel<BM_, BM_, true, false, false>, grid, st, ps, a);           \
    } else if (a.acn) {                                                                      \
      if (exact) launch(gemm_f32_kernel<BM_, BM_, false, true, true>, grid, st, ps, a);      \
      else launch(gemm_f32_kernel<BM_, BM_, false, false, true>, grid, st, ps, a);           \
    } else {                                                                                 \
      if (exact) launch(gemm_f32_kernel<BM_, BM_, false, true, false>, grid, st, ps, a);     \
      else launch(gemm_f32_kernel<BM_, BM_, false, false, false>, grid, st, ps, a);          \
    }                                                                                        \
  }
    LORA_F32_TILE(128) else LORA_F32_TILE(64)
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

void launch_gemm_bf16(const GemmPlan& g, bool fwd, const GemmBf16Args& a, hipStream_t st) {
  const dim3 grid((unsigned)(cdiv(a.Nc, g.bn) * cdiv(a.M, g.bm)));
  prof::Scope ps(fwd ? "gemm_bf16_fwd" : "gemm_bf16_dx", a.M, a.Nc, a.Kc,
                 2.0 * a.M * a.Nc * a.Kc + 2.0 * a.M * a.r * a.Nc,
                 2.0 * (a.M * a.Kc + a.Nc * a.Kc) + 4.0 * a.M * a.Nc * (a.C2 ? 2 : 1));
  const Bf16Cfg& c = kBf16Cfg[g.cfg];
  const bool exact = a.M % c.bm == 0 && a.Nc % c.bn == 0 && a.Kc % c.bk == 0;
#define LORA_BF16_TILE(i, BM_, BN_, NT_, WGM_, BK_, D_, DIRS_)                              \
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

}  // namespace

// =========================================================================
extern "C" {

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
  int rc = check_linear(lin);
  if (rc) return rc;
  if (!X || !Y || !U) return LORA_E_INVALID;
  if (!al16(X) || !al16(Y) || !al16(U) || (Z && !al16(Z))) return LORA_E_ALIGN;
  if (!drop_valid(drop)) return LORA_E_INVALID;
  const Layout y = make_layout(lin);
  if (y.fwd_bytes && (!ws || ws_bytes < y.fwd_bytes || !al16(ws))) return LORA_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int64_t T = lin->tokens, K = lin->in_dim, N = lin->out_dim, r = lin->rank;
  const bool bf = lin->w_dtype == LORA_BF16;
  char* w = (char*)ws;
  float* Upart = y.down.n > 1 ? (float*)(w + y.upart) : nullptr;
  uint16_t* Xbf = bf ? (uint16_t*)(w + y.xbf) : nullptr;
  const DropParams d = make_drop(drop);

  DownArgs da;
  da.X = X; da.T = T; da.K = K; da.A = lin->A; da.r = r; da.drop = d;
  da.ksplit = y.down.len; da.nsplit = y.down.n; da.Upart = Upart; da.U = U; da.Xbf = Xbf;
  const double down_flops = 2.0 * T * K * r;
  const double down_bytes = 4.0 * (T * K + r * K + T * r) + (Xbf ? 2.0 * T * K : 0.0);
  const LoraOperand xa = y.down.n > 1 ? LoraOperand{Upart, T * r, y.down.n, U}
                                      : LoraOperand{U, T * r, 1, nullptr};

  if (use_split_path(y.gf, r, bf)) {
    // Launch 1: split GEMM partials of X W^T beside the down projection.
    GemmF32Args a;
    memset(&a, 0, sizeof(a));
    a.A = X; a.lda = K; a.B = (const float*)lin->W; a.ldb = K;
    a.M = T; a.Nc = N; a.Kc = K;
    a.ksplit = y.gf.k.len; a.nsplit = y.gf.k.n;
    a.part = (float*)(w + y.gfpart);
    const SplitGrid f = split_grid(T, N, y.gf.k.n, cdiv(T, SK_T), y.down.n);
    const bool exact = T % 64 == 0 && N % 64 == 0 && K % y.gf.k.len == 0 && y.gf.k.len % 32 == 0;
    {
      prof::Scope ps("gemm_f32_fwd+down", T, N, K, 2.0 * T * N * K + down_flops,
                     4.0 * (T * K + N * K + y.gf.k.n * T * N) + down_bytes);
      const dim3 grid((unsigned)(f.gemm_blocks + f.side_blocks));
      LORA_RP_DISPATCH_32(rank_pad(r), {
        if (exact) launch(fwd_main_kernel<true, RP>, grid, st, ps, a, da, f);
        else launch(fwd_main_kernel<false, RP>, grid, st, ps, a, da, f);
      });
    }
    // Launch 2: Y = sum of partials + s U B^T (DoRA: Z and the row scale).
    EpiArgs e = epi_shape(T, N);
    e.part = a.part; e.nsplit = y.gf.k.n;
    e.xa = xa; e.XB = lin->B; e.r = r; e.s = lin->scale;
    e.C = Y; e.C2 = Z; e.cn = lin->dora_mag; e.cd = lin->dora_norm;
    prof::Scope ps("fwd_epilogue", T, N, y.gf.k.n, 2.0 * T * N * r,
                   4.0 * T * N * (y.gf.k.n + (Z ? 2 : 1)) + 4.0 * (y.down.n * T * r + N * r));
    launch(fwd_epi_kernel, dim3((unsigned)e.blocks), st, ps, e);
    return hip_status();
  }

  // U = X~ A^T, split over K; the GEMM sums the splits while staging U and
  // stores the summed U.
  {
    prof::Scope ps("down_u", T, r, K, down_flops, down_bytes);
    const dim3 grid((unsigned)cdiv(T, SK_T), (unsigned)y.down.n);
    LORA_RP_DISPATCH(rank_pad(r), launch(down_kernel<RP>, grid, st, ps, da));
  }

  // Z = X W^T + s U B^T; Y = Z or (mag/norm) * Z.
  if (bf) {
    GemmBf16Args a;
    memset(&a, 0, sizeof(a));
    a.A = Xbf; a.lda = K; a.B = (const uint16_t*)lin->W; a.ldb = K;
    a.M = T; a.Nc = N; a.Kc = K;
    a.xa = xa; a.XB = lin->B; a.r = r; a.xs = lin->scale;
    a.C = Y; a.C2 = Z; a.cn = lin->dora_mag; a.cd = lin->dora_norm;
    launch_gemm_bf16(y.gf, true, a, st);
  } else {
    GemmF32Args a;
    memset(&a, 0, sizeof(a));
    a.A = X; a.lda = K; a.B = (const float*)lin->W; a.ldb = K;
    a.M = T; a.Nc = N; a.Kc = K;
    a.xa = xa; a.XB = lin->B; a.r = r; a.xs = lin->scale;
    a.ksplit = y.gf.k.len; a.nsplit = y.gf.k.n;
    a.C = Y; a.C2 = Z; a.cn = lin->dora_mag; a.cd = lin->dora_norm;
    a.part = y.gf.k.n > 1 ? (float*)(w + y.gfpart) : nullptr;
    launch_gemm_f32(y.gf, true, a, st);
  }
  return hip_status();
}

int lora_backward(const lora_linear* lin, const float* X, const float* dY, const float* U,
                  const float* Z, float* dX, float* dA, float* dB, float* dMag,
                  int accumulate, const lora_dropout* drop, void* ws, size_t ws_bytes,
                  void* stream) {
  int rc = check_linear(lin);
  if (rc) return rc;
  if (!X || !dY || !U || !dA || !dB) return LORA_E_INVALID;
  if (!al16(X) || !al16(dY) || !al16(U) || !al16(dA) || !al16(dB)) return LORA_E_ALIGN;
  if ((dX && !al16(dX)) || (Z && !al16(Z)) || (dMag && !al16(dMag))) return LORA_E_ALIGN;
  const bool dora = lin->dora_mag != nullptr;
  if (dMag && (!dora || !Z)) return LORA_E_INVALID;
  if (!drop_valid(drop)) return LORA_E_INVALID;
  const Layout y = make_layout(lin);
  if (y.bwd_bytes && (!ws || ws_bytes < y.bwd_bytes || !al16(ws))) return LORA_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int64_t T = lin->tokens, K = lin->in_dim, N = lin->out_dim, r = lin->rank;
  const bool bf = lin->w_dtype == LORA_BF16;
  char* w = (char*)ws;
  const DropParams d = make_drop(drop);
  const int rp = rank_pad(r);
  const int acc = accumulate ? 1 : 0;

  // One pass over dY: V (as per-strip partials), dB, DoRA dm and bf16 g.
  K3Out o;
  o.Vpart = y.strips > 1 ? (float*)(w + y.vpart) : nullptr;
  o.V = (float*)(w + y.v);
  o.dBpart = y.k3.n > 1 ? (float*)(w + y.dbpart) : nullptr;
  o.dB = dB;
  o.dmpart = (dMag && y.k3.n > 1) ? (float*)(w + y.dmpart) : nullptr;
  o.dm = dMag;
  o.gbf = (bf && dX) ? (uint16_t*)(w + y.gbf) : nullptr;
  o.scale = lin->scale;
  o.accumulate = acc;
  const float* Zin = dMag ? Z : nullptr;
  K3Args ka;
  ka.dY = dY; ka.T = T; ka.N = N; ka.B = lin->B; ka.U = U; ka.r = r;
  ka.mag = lin->dora_mag; ka.nrm = lin->dora_norm; ka.Z = Zin;
  ka.tsplit = y.k3.len; ka.nstrip = y.strips; ka.spb = 1; ka.nts = y.k3.n; ka.o = o;
  const double k3_flops = 4.0 * T * N * r;
  const double k3_bytes = 4.0 * (T * N + T * r + 2 * N * r) + (Zin ? 4.0 * T * N : 0.0) +
                          (o.gbf ? 2.0 * T * N : 0.0);
  const LoraOperand xv = (y.strips == 1 || y.vreduce) ? LoraOperand{o.V, T * r, 1, nullptr}
                                                      : LoraOperand{o.Vpart, T * r, (int)y.strips, nullptr};
  float* dApart = y.k4.n > 1 ? (float*)(w + y.dapart) : nullptr;
  K4Args k4a;
  k4a.X = X; k4a.T = T; k4a.K = K; k4a.V = xv.p; k4a.vparts = xv.nparts; k4a.r = r; k4a.drop = d;
  k4a.tsplit = y.k4.len; k4a.nts = y.k4.n; k4a.dApart = dApart; k4a.dA = dA;
  k4a.scale = lin->scale; k4a.accumulate = acc;
  const double k4_flops = 2.0 * T * K * r;
  const double k4_bytes = 4.0 * (T * K + T * r + 2 * r * K);

  // Gradient splits over token ranges: fixed-order reduction jobs.
  RedJob jobs[3];
  int nj = 0;
  if (y.k3.n > 1) {
    jobs[nj++] = {o.dBpart, dB, nullptr, N * r, 1, y.k3.n, acc, lin->scale};
    if (dMag) jobs[nj++] = {o.dmpart, dMag, lin->dora_norm, N, N, y.k3.n, acc, 1.0f};
  }

  if (dX && use_split_path(y.gd, r, bf)) {
    // Launch 1: split GEMM partials of g W beside k3 (V partials, dB, dm).
    GemmF32Args a;
    memset(&a, 0, sizeof(a));
    a.A = dY; a.lda = N; a.acn = lin->dora_mag; a.acd = lin->dora_norm;
    a.B = (const float*)lin->W; a.ldb = K;
    a.M = T; a.Nc = K; a.Kc = N;
    a.ksplit = y.gd.k.len; a.nsplit = y.gd.k.n;
    a.part = (float*)(w + y.gdpart);
    // k3 beside the GEMM: one strip per block (each strip is a chain of
    // dependent loads), several only past 32 strips, so V arrives as at most
    // 32 partials for the two consumers of launch 2.
    K3Args kb = ka;
    kb.spb = cdiv(y.strips, 32);
    const int64_t nvp = cdiv(y.strips, kb.spb);
    kb.o.V = (float*)(w + y.v);
    kb.o.Vpart = nvp > 1 ? (float*)(w + y.vpart) : nullptr;
    const LoraOperand vd = nvp > 1 ? LoraOperand{kb.o.Vpart, T * r, (int)nvp, nullptr}
                                   : LoraOperand{kb.o.V, T * r, 1, nullptr};
    const SplitGrid f = split_grid(T, K, y.gd.k.n, nvp, y.k3.n);
    const bool exact = T % 64 == 0 && K % 64 == 0 && N % y.gd.k.len == 0 && y.gd.k.len % 32 == 0;
    {
      prof::Scope ps("gemm_f32_dx+k3", T, K, N, 2.0 * T * N * K + k3_flops,
                     4.0 * (T * N + N * K + y.gd.k.n * T * K) + k3_bytes);
      const dim3 grid((unsigned)(f.gemm_blocks + f.side_blocks));
      LORA_RP_DISPATCH_32(rp, {
        if (a.acn) {
          if (exact) launch(bwd_main_kernel<true, true, RP>, grid, st, ps, a, kb, f);
          else launch(bwd_main_kernel<false, true, RP>, grid, st, ps, a, kb, f);
        } else {
          if (exact) launch(bwd_main_kernel<true, false, RP>, grid, st, ps, a, kb, f);
          else launch(bwd_main_kernel<false, false, RP>, grid, st, ps, a, kb, f);
        }
      });
    }
    // Launch 2: dX = sum of partials + (s V A) * mask * keep, beside k4 and
    // the dB / dm reductions.
    k4a.V = vd.p;
    k4a.vparts = vd.nparts;
    EpiArgs e = epi_shape(T, K);
    e.part = a.part; e.nsplit = y.gd.k.n;
    e.xa = vd; e.XB = lin->A; e.r = r; e.s = lin->scale; e.drop = d;
    e.C = dX;
    RedJobs J;
    memset(&J, 0, sizeof(J));
    int64_t rblocks = 0;
    for (int i = 0; i < nj; ++i) {
      J.job[i] = jobs[i];
      J.blk[i] = rblocks;
      rblocks += cdiv(jobs[i].n, 256);
    }
    J.blk[nj] = rblocks;
    J.njobs = nj;
    BwdEpiGrid g;
    g.narrow = T <= K4N_MAX_T && y.k4.n == 1;
    g.k4_x = g.narrow ? cdiv(K, 16) : cdiv(K, SK_C);
    g.k4_blocks = g.k4_x * y.k4.n;
    g.epi_blocks = e.blocks;
    {
      prof::Scope ps("dx_epilogue+k4", T, K, y.gd.k.n, 2.0 * T * K * r + k4_flops,
                     4.0 * T * K * (y.gd.k.n + 1) + 4.0 * (nvp * T * r + r * K) + k4_bytes);
      LORA_RP_DISPATCH_32(rp, launch(bwd_epi_kernel<RP>,
                                     dim3((unsigned)(g.k4_blocks + g.epi_blocks + rblocks)), st,
                                     ps, e, k4a, J, g));
    }
    if (y.k4.n > 1) {
      RedJob ja = {dApart, dA, nullptr, r * K, 1, y.k4.n, acc, lin->scale};
      launch_reduce(&ja, 1, st);
    }
    return hip_status();
  }

  // One pass over dY: V (as per-strip partials), dB, DoRA dm and bf16 g.
  {
    prof::Scope ps("k3_v_db", T, N, r, k3_flops, k3_bytes);
    const dim3 grid((unsigned)y.strips, (unsigned)y.k3.n);
    LORA_RP_DISPATCH(rp, launch(k3_kernel<RP>, grid, st, ps, ka));
  }
  if (y.vreduce) {
    RedJob jv = {o.Vpart, o.V, nullptr, T * r, 1, (int)y.strips, 0, 1.0f};
    launch_reduce(&jv, 1, st);
  }

  if (dX) {
    if (bf) {
      GemmBf16Args a;
      memset(&a, 0, sizeof(a));
      a.A = o.gbf; a.lda = N; a.B = (const uint16_t*)lin->W; a.ldb = K;
      a.M = T; a.Nc = K; a.Kc = N;
      a.xa = xv; a.XB = lin->A; a.r = r; a.xs = lin->scale; a.drop = d;
      a.C = dX;
      launch_gemm_bf16(y.gd, false, a, st);
    } else {
      GemmF32Args a;
      memset(&a, 0, sizeof(a));
      a.A = dY; a.lda = N; a.acn = lin->dora_mag; a.acd = lin->dora_norm;
      a.B = (const float*)lin->W; a.ldb = K;
      a.M = T; a.Nc = K; a.Kc = N;
      a.xa = xv; a.XB = lin->A; a.r = r; a.xs = lin->scale; a.drop = d;
      a.ksplit = y.gd.k.len; a.nsplit = y.gd.k.n;
      a.C = dX;
      a.part = y.gd.k.n > 1 ? (float*)(w + y.gdpart) : nullptr;
      launch_gemm_f32(y.gd, false, a, st);
    }
  }

  {
    prof::Scope ps("k4_da", T, r, K, k4_flops, k4_bytes);
    const dim3 grid((unsigned)cdiv(K, SK_C), (unsigned)y.k4.n);
    LORA_RP_DISPATCH(rp, launch(k4_kernel<RP>, grid, st, ps, k4a));
  }

  if (y.k4.n > 1) jobs[nj++] = {dApart, dA, nullptr, r * K, 1, y.k4.n, acc, lin->scale};
  if (nj) launch_reduce(jobs, nj, st);
  return hip_status();
}

size_t lora_grad_prepare_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return 4096 + 1024 * (sizeof(double) + sizeof(int)) + 256;
}

int lora_grad_prepare(const float* grads, int64_t n, int64_t n_pred_tokens, float max_norm,
                      float* d_scale, double* d_stats, double* h_norm, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!grads || !d_scale || n <= 0 || n_pred_tokens <= 0) return LORA_E_INVALID;
  if (!(max_norm >= 0.0f) || !std::isfinite(max_norm)) return LORA_E_INVALID;
  if (!al16(grads)) return LORA_E_ALIGN;
  if (!ws || !al16(ws) || ws_bytes < lora_grad_prepare_workspace_bytes(n)) return LORA_E_WORKSPACE;
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

int lora_dora_row_norms(const lora_linear* lin, float* out_norm, void* stream) {
  if (!lin || !out_norm) return LORA_E_INVALID;
  if (lin->in_dim <= 0 || lin->out_dim <= 0) return LORA_E_SHAPE;
  if (lin->w_dtype != LORA_F32 && lin->w_dtype != LORA_BF16) return LORA_E_DTYPE;
  if (!lin->W) return LORA_E_INVALID;
  if ((lin->A == nullptr) != (lin->B == nullptr)) return LORA_E_INVALID;
  const bool lora_on = lin->A != nullptr;
  if (lora_on && (lin->rank <= 0 || lin->rank > 128)) return LORA_E_SHAPE;
  if (!std::isfinite(lin->scale)) return LORA_E_INVALID;
  const int64_t N = lin->out_dim, K = lin->in_dim, r = lora_on ? lin->rank : 0;
  const float* A = lin->A;
  const float* B = lin->B;
  const float s = lin->scale;
  constexpr int ROWS = 8;
  const unsigned grid = (unsigned)cdiv(N, ROWS);
  hipStream_t st = (hipStream_t)stream;
  const int rp = lora_on ? rank_pad(r) : 16;
  prof::Scope ps("dora_rownorm", N, K, r, 2.0 * N * K * (r + 1),
                 (lin->w_dtype == LORA_BF16 ? 2.0 : 4.0) * N * K + 4.0 * r * (N + K) + 4.0 * N);
  if (lin->w_dtype == LORA_BF16) {
    const uint16_t* W = (const uint16_t*)lin->W;
    LORA_RP_DISPATCH(rp, launch(dora_rownorm_kernel<uint16_t, RP, ROWS>, dim3(grid), st, ps, W, N,
                                K, A, B, r, s, out_norm));
  } else {
    const float* W = (const float*)lin->W;
    LORA_RP_DISPATCH(rp, launch(dora_rownorm_kernel<float, RP, ROWS>, dim3(grid), st, ps, W, N, K,
                                A, B, r, s, out_norm));
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
