// Gradient preparation, AdamW and DoRA row norms.
//
// gradnorm_pass1/2 ("4.3. Training Guide", "Gradient clipping"): the sum of
// squares of the slot's summed gradient in double with a non-finite flag,
// then one block combines the per-block partials in fixed order and emits
// the single combined normalisation-and-clip scale.
//
// adamw ("4.3. Training Guide", "Optimizer"): decoupled AdamW, weight decay on
// A only from the pre-update value at the uncorrected rate, B at lr*ratio.
//
// The DoRA row norms and the merge (one pass over W's rows): rowpass.hpp.
#pragma once
#include "common.hpp"
#include "rowpass.hpp"

namespace lora {

LORA_DEV bool finite_bits(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

// Pass 1: block b sums squares of g[b*per .. min(n, (b+1)*per)) in double.
__global__ __launch_bounds__(256) void gradnorm_pass1(const float* __restrict__ g, int64_t n,
                                                      int64_t per, double* __restrict__ part,
                                                      int* __restrict__ flags) {
  __shared__ double ws[4];
  __shared__ int wf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = min(n, b0 + per);
  double s = 0.0;
  int bad = 0;
  // per is a multiple of 1024, so b0 is 16-byte aligned.
  const int64_t full = b0 + ((b1 - b0) / 4) * 4;
  for (int64_t i = b0 + 4 * tid; i < full; i += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(g + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bad |= !finite_bits(v[e]);
      s += (double)v[e] * (double)v[e];
    }
  }
  for (int64_t i = full + tid; i < b1; i += 256) {
    const float x = g[i];
    bad |= !finite_bits(x);
    s += (double)x * (double)x;
  }
  s = wave_sum(s);
  bad = __any(bad) ? 1 : 0;
  if (lane == 0) {
    ws[wave] = s;
    wf[wave] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    part[blockIdx.x] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
    flags[blockIdx.x] = wf[0] | wf[1] | wf[2] | wf[3];
  }
}

// Pass 2: one block.  norm = sqrt(ss)/npred; clip; scale = float(clip/npred).
__global__ __launch_bounds__(256) void gradnorm_pass2(const double* __restrict__ part,
                                                      const int* __restrict__ flags, int nb,
                                                      int64_t npred, float max_norm,
                                                      float* __restrict__ d_scale,
                                                      double* __restrict__ d_stats,
                                                      double* __restrict__ ws_norm) {
  __shared__ double ws[4];
  __shared__ int wf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double s = 0.0;
  int bad = 0;
  for (int i = tid; i < nb; i += 256) {
    s += part[i];
    bad |= flags[i];
  }
  s = wave_sum(s);
  bad = __any(bad) ? 1 : 0;
  if (lane == 0) {
    ws[wave] = s;
    wf[wave] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    const double ss = ((ws[0] + ws[1]) + ws[2]) + ws[3];
    const int nonfinite = wf[0] | wf[1] | wf[2] | wf[3];
    double norm = sqrt(ss) / (double)npred;
    double clip = 1.0;
    const double mn = (double)max_norm;
    if (mn > 0.0 && norm > mn) clip = mn / norm;
    float scale = (float)(clip / (double)npred);
    if (nonfinite) {
      norm = __builtin_nan("");
      clip = __builtin_nan("");
      scale = __builtin_nanf("");
    }
    *d_scale = scale;
    ws_norm[0] = norm;
    ws_norm[1] = clip;
    if (d_stats) {
      d_stats[0] = norm;
      d_stats[1] = clip;
    }
  }
}

// AdamW over up to 64 segments; block b belongs to the segment whose block
// range holds b; each thread updates one float4.
constexpr int ADAM_MAX_SEG = 64;
struct AdamSegs {
  int64_t off[ADAM_MAX_SEG];
  int64_t cnt[ADAM_MAX_SEG];
  int64_t blk[ADAM_MAX_SEG + 1];
  int32_t kind[ADAM_MAX_SEG];
  int n;
};
struct AdamHp {
  float b1, one_m_b1, b2, one_m_b2, eps, bc1, bc2;
  float rate[3];    // per kind: lr (A), lr*plus_ratio (B), lr (magnitude)
  float decay[3];   // per kind: lr*weight_decay (A), 0, 0
};

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ P,
                                                    const float* __restrict__ G,
                                                    float* __restrict__ Mo, float* __restrict__ Vo,
                                                    AdamSegs segs, AdamHp hp,
                                                    const float* __restrict__ d_scale) {
  const float sc = *d_scale;
  if (!finite_bits(sc)) return;   // vetoed update: touch nothing
  const int64_t b = blockIdx.x;
  int lo = 0, hi = segs.n - 1;
  while (lo < hi) {   // last segment with blk[s] <= b
    const int mid = (lo + hi + 1) >> 1;
    if (segs.blk[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int64_t e = ((b - segs.blk[s]) * 256 + threadIdx.x) * 4;
  if (e >= segs.cnt[s]) return;
  const int64_t i = segs.off[s] + e;
  const int kind = segs.kind[s];
  const float rate = hp.rate[kind];
  const float decay = hp.decay[kind];
  f32x4 p = *reinterpret_cast<const f32x4*>(P + i);
  const f32x4 g = *reinterpret_cast<const f32x4*>(G + i);
  f32x4 m = *reinterpret_cast<const f32x4*>(Mo + i);
  f32x4 v = *reinterpret_cast<const f32x4*>(Vo + i);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float gp = g[q] * sc;
    m[q] = hp.b1 * m[q] + hp.one_m_b1 * gp;
    v[q] = hp.b2 * v[q] + hp.one_m_b2 * (gp * gp);
    const float mh = m[q] / hp.bc1;
    const float vh = v[q] / hp.bc2;
    const float upd = mh / (sqrtf(vh) + hp.eps);
    p[q] = (p[q] - rate * upd) - decay * p[q];
  }
  *reinterpret_cast<f32x4*>(P + i) = p;
  *reinterpret_cast<f32x4*>(Mo + i) = m;
  *reinterpret_cast<f32x4*>(Vo + i) = v;
}

// rmse = sqrt(sum of the n partials / count): each thread adds a strided
// subset in index order, then the 256 sums combine in a fixed tree.
__global__ __launch_bounds__(256) void rmse_finish_kernel(const double* __restrict__ part,
                                                          int64_t n, double count,
                                                          double* __restrict__ out) {
  __shared__ double red[256];
  double t = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) t += part[i];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = sqrt(red[0] / count);
}

// out[i] = sqrt of the column-split partials of row i, summed in split order.
__global__ __launch_bounds__(256) void dora_norm_finish_kernel(const double* __restrict__ part,
                                                               int nsplit, int64_t N,
                                                               float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  out[i] = (float)sqrt(sum_parts1(part, N, nsplit, i));
}

}  // namespace lora
