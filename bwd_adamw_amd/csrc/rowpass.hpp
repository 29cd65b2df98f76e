// One pass over the rows of W + s B A: DoRA row norms ("8. LoRA
// Fundamentals", "How it works": ||W_i + s (B A)_i||) and the merge for
// export (the same section's effective weight).  W is float32, bf16 or a
// block-quantized format (qweight.hpp), decoded to float32 where it is used.
#pragma once
#include "common.hpp"
#include "qweight.hpp"

namespace lora {

// DoRA row norms, out[i] = || W_i + s (B A)_i ||.  The rank contraction is
// a dense product and runs on v_mfma_f32_32x32x2f32 in transposed form,
// D[m][i] = sum_j A[j][col(m)] B[i][j], so that a lane's 16 accumulator rows
// are 16 columns of one output row i.  Inside a 64-column chunk, tile q's
// row m is column 32*((m>>2)&1) + 8*(m>>3) + 2*(m&3) + q: a lane's two A
// operands (q = 0, 1) are then one float2, and lane l's 32 results are the
// 32 consecutive columns 32*(l/32) .. +31 of row l%32, read from W as whole
// 16-byte vectors.  A block covers DN_ROWS = 128 rows, 32 per wave, and walks
// cpw chunks of one column split: per chunk the block stages A's 64 columns
// once in LDS, in MFMA operand order (double-buffered, one barrier per
// chunk), and each wave contracts them against its rows while the next
// chunk's A and this chunk's W are in flight.  With gridDim.y > 1 the splits
// leave double partials that dora_norm_finish_kernel sums in split order.
constexpr int DN_ROWS = 128;  // 32 per wave
constexpr int DN_CHUNK = 64;
constexpr int DN_LDS_AHEAD = 4;

struct RowPassArgs {
  const void* W;
  int64_t N, K;
  const float* A;  // [r,K] or nullptr (norms of W alone)
  const float* B;  // [N,r]
  int r;
  float s;
  int cpw;         // chunks per block (each wave walks all of them)
  int vec;         // W and A rows are 16-byte aligned: full chunks use vector loads
  double* part;    // norms: [gridDim.y][N] when gridDim.y > 1
  float* out;      // norms: [N]
  // merge: W_out = c_i (W + s B A), c_i = mag[i] / nrm[i] when both are set
  void* wout;      // [N, K] float or bf16
  int vec_out;     // wout rows are 16-byte aligned
  const float* mag;
  const float* nrm;
  double* epart;   // [gridDim.y][gridDim.x][4] squared bf16 rounding error, or nullptr
  QPlanes q;       // W block-quantized (kernels with WQ set)
};

// Waves per SIMD the kernel is built for (registers; the host plans with it).
LORA_HD constexpr int dn_waves_per_simd(int rp, int mode = 0) {
  return mode == 1 ? (rp <= 16 ? 4 : 2) : (rp <= 64 ? 4 : 2);   // the merge holds 32 outputs
}

template <typename WT>
LORA_DEV float dn_w(const u32x4* w, int e) {
  if constexpr (sizeof(WT) == 2) {
    const uint32_t x = w[e / 8][(e % 8) / 2];
    return bf16_bits_to_f32((e & 1) ? x >> 16 : x & 0xffffu);
  } else {
    return __uint_as_float(w[e / 4][e % 4]);
  }
}

// One pass over W's rows with (W + s B A) tiles formed on the fly.
// MODE 0: DoRA row norms.  MODE 1: merge for export, W_out = c (W + s B A)
// stored as OT (float, or bf16 rounded to nearest even), with the squared
// rounding error of bf16 output summed per wave.  WQ: W is block-quantized
// in that format (WT unused); a lane's 32 columns are four 8-element runs,
// decoded to float32 where they are used.
template <typename WT, int RP, bool LORA, int MODE, typename OT, int WQ = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dn_waves_per_simd(RP, MODE))))
void row_pass_kernel(RowPassArgs p) {
  constexpr int NS = RP / 2;                        // MFMA steps (two rank rows each)
  constexpr int WV = WQ ? 1 : (sizeof(WT) == 2 ? 4 : 8);   // u32x4 of W per lane and chunk
  constexpr int QWD = WQ ? wq_words(WQ) : 1;
  constexpr int AQ = LORA ? RP / 16 : 1;            // A float4 per thread and chunk
  constexpr uint32_t OUT = 0xfffffff0u;             // an offset past every resource
  __shared__ f32x2 As[2][LORA ? NS * 64 : 1];       // [buffer][step][lane]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = p.N, K = p.K;
  const int64_t i0 = (int64_t)blockIdx.x * DN_ROWS + 32 * wave;  // this wave's rows
  const int64_t brows = N - i0 < 32 ? (N - i0 > 0 ? N - i0 : 0) : 32;

  // Every load below is an unconditional raw buffer load: rows past N and
  // rank rows past r lie outside their resources and read as zero, and a
  // masked element gets the offset OUT.  Host guarantees 32 * K *
  // sizeof(WT) and (RP + 1) * K * 4 fit in 32 bits.
  float bop[NS];  // B operand of step s: B[i0 + lane%32][2s + lane/32]
  if constexpr (LORA) {
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.B + (brows ? i0 : 0) * p.r), (short)0, (int)(uint32_t)(brows * p.r * 4),
        0x00020000);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int j = 2 * st + (lane >> 5);
      const uint32_t off = j < p.r ? (uint32_t)(((lane & 31) * p.r + j) * 4) : OUT;
      bop[st] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0));
    }
  }
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const WT*>(p.W) + (brows ? i0 : 0) * K), (short)0,
      (int)(uint32_t)(brows * K * (int64_t)sizeof(WT)), 0x00020000);
  const uint32_t woff = (uint32_t)(((lane & 31) * K + 32 * (lane >> 5)) * (int64_t)sizeof(WT));
  const QRes<WQ ? WQ : WQ_Q8_0> QR(p.q);   // quantized W: rows past N read as zero
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.A, (short)0, (int)(uint32_t)(LORA ? (int64_t)p.r * K * 4 : 0), 0x00020000);

  // A staging: thread t moves rows t/16 + 16u, columns 4*(t%16) .. +3 of the
  // chunk; in operand order those four values are lanes m, m+1 of step j/2.
  const int scol = 4 * (tid & 15);
  int sdst[AQ];
#pragma unroll
  for (int u = 0; u < AQ; ++u) {
    const int j = (tid >> 4) + 16 * u;
    const int pr = scol >> 1;
    const int m = ((pr >> 2) & 3) * 8 + (pr >> 4) * 4 + (pr & 3);
    sdst[u] = (j >> 1) * 64 + (j & 1) * 32 + m;
  }
  auto load_a = [&](f32x4 (&a)[AQ], int64_t k0) {
    if constexpr (LORA) {
      const bool full = p.vec && k0 + DN_CHUNK <= K;
#pragma unroll
      for (int u = 0; u < AQ; ++u) {
        const int64_t j = (tid >> 4) + 16 * u;
        const int64_t col = k0 + scol;
        if (full) {
          a[u] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (uint32_t)((j * K + col) * 4), 0, 0));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a[u][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                ra, col + e < K ? (uint32_t)((j * K + col + e) * 4) : OUT, 0, 0));
        }
      }
    }
  };
  auto store_a = [&](const f32x4 (&a)[AQ], int buf) {
    if constexpr (LORA) {
#pragma unroll
      for (int u = 0; u < AQ; ++u) *reinterpret_cast<f32x4*>(&As[buf][sdst[u]]) = a[u];
    }
  };
  auto load_q = [&](uint32_t (&qw)[4][QWD], int64_t k0) {
    if constexpr (WQ != 0) {
      const int64_t kb = k0 + 32 * (lane >> 5);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        wq_load<WQ>(QR, (uint32_t)K, (uint32_t)(i0 + (lane & 31)), (uint32_t)(kb + 8 * h), qw[h],
                    kb < K);
    }
  };
  auto load_w = [&](u32x4 (&w)[WV], int64_t k0) {
    if constexpr (WQ != 0) return;
    if (p.vec && k0 + DN_CHUNK <= K) {
      const uint32_t kw = (uint32_t)k0 * (uint32_t)sizeof(WT);
#pragma unroll
      for (int h = 0; h < WV; ++h)
        w[h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff + kw + 16u * h, 0, 0));
    } else {
      const int64_t kb = k0 + 32 * (lane >> 5);
      const uint32_t rowoff = (uint32_t)((lane & 31) * K);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t off = kb + e < K ? (rowoff + (uint32_t)(kb + e)) * (uint32_t)sizeof(WT) : OUT;
        if constexpr (sizeof(WT) == 2) {
          const uint32_t x = __builtin_amdgcn_raw_buffer_load_b16(rw, off, 0, 0);
          if (e & 1) w[e / 8][(e % 8) / 2] |= x << 16;
          else w[e / 8][(e % 8) / 2] = x;
        } else {
          w[e / 4][e % 4] = __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0);
        }
      }
    }
  };

  const int64_t nch = (K + DN_CHUNK - 1) / DN_CHUNK;
  const int64_t c0 = (int64_t)blockIdx.y * p.cpw;
  const int64_t c1 = c0 + p.cpw < nch ? c0 + p.cpw : nch;
  double sq = 0.0;  // norms: this lane's squares; merge: its rounding error
  float crow = 1.f;
  if constexpr (MODE == 1) {
    if (p.mag && (lane & 31) < brows)
      crow = p.mag[i0 + (lane & 31)] / p.nrm[i0 + (lane & 31)];
  }
  f32x4 a[AQ];
  load_a(a, c0 * DN_CHUNK);
  store_a(a, 0);
  __syncthreads();
  for (int64_t c = c0; c < c1; ++c) {
    const int buf = (int)((c - c0) & 1);
    // Next chunk's A (clamped to the last one) and this chunk's W go out
    // first; the contraction below reads only LDS, and four waves per SIMD
    // cover the W latency.
    load_a(a, (c + 1 < c1 ? c + 1 : c) * DN_CHUNK);
    u32x4 w[WV];
    uint32_t qw[4][QWD];
    load_w(w, c * DN_CHUNK);
    load_q(qw, c * DN_CHUNK);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[q][v] = 0.f;
    if constexpr (LORA) {
      // Operands are read from LDS DN_LDS_AHEAD steps ahead of their MFMAs.
      constexpr int AH = NS < DN_LDS_AHEAD ? NS : DN_LDS_AHEAD;
      f32x2 av[AH];
#pragma unroll
      for (int u = 0; u < AH; ++u) av[u] = As[buf][u * 64 + lane];
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const f32x2 cur = av[st % AH];
        if (st + AH < NS) av[st % AH] = As[buf][(st + AH) * 64 + lane];
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[q] = mfma32x32x2(cur[q], bop[st], acc[q]);
        __builtin_amdgcn_sched_barrier(0);  // keep each read ahead of its step
      }
    }
    // acc[q][v] is column k0 + 32 (lane/32) + 2v + q of row i0 + lane%32;
    // masked columns hold W = 0 and A = 0 and add nothing.
    float wd[WQ ? 32 : 1];
    if constexpr (WQ != 0) {
#pragma unroll
      for (int h = 0; h < 4; ++h) wq_decode<WQ>(qw[h], wd + 8 * h);
    }
    auto wval = [&](int e) -> float {
      if constexpr (WQ != 0) return wd[e];
      else return dn_w<WT>(w, e);
    };
    if constexpr (MODE == 0) {
      float cs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float x = wval(2 * v + q) + p.s * acc[q][v];
          cs += x * x;
        }
      sq += (double)cs;
    } else {
      // Merged values of this lane's 32 consecutive columns.
      float x[32];
#pragma unroll
      for (int v = 0; v < 16; ++v)
#pragma unroll
        for (int q = 0; q < 2; ++q) x[2 * v + q] = (wval(2 * v + q) + p.s * acc[q][v]) * crow;
      const int64_t row = i0 + (lane & 31);
      const int64_t kb = c * DN_CHUNK + 32 * (lane >> 5);
      OT* dst = static_cast<OT*>(p.wout) + (row < N ? row : 0) * K + kb;
      const bool full = p.vec_out && c * DN_CHUNK + DN_CHUNK <= K;
      if constexpr (sizeof(OT) == 2) {
        uint32_t pk[16];
        float es = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t lo = f32_to_bf16_bits(x[2 * e]), hi = f32_to_bf16_bits(x[2 * e + 1]);
          pk[e] = lo | (hi << 16);
          const float d0 = bf16_bits_to_f32(lo) - x[2 * e], d1 = bf16_bits_to_f32(hi) - x[2 * e + 1];
          es += d0 * d0 + d1 * d1;
        }
        if (row < N) {
          if (full) {
#pragma unroll
            for (int h = 0; h < 4; ++h)
              reinterpret_cast<u32x4*>(dst)[h] = u32x4{pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 32; ++e)
              if (kb + e < K) dst[e] = (OT)((pk[e / 2] >> (16 * (e & 1))) & 0xffffu);
          }
          sq += (double)es;   // masked columns are 0 on both sides
        }
      } else {
        if (row < N) {
          if (full) {
#pragma unroll
            for (int h = 0; h < 8; ++h)
              reinterpret_cast<f32x4*>(dst)[h] = f32x4{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 32; ++e)
              if (kb + e < K) dst[e] = x[e];
          }
        }
      }
    }
    store_a(a, buf ^ 1);
    __syncthreads();
  }
  if constexpr (MODE == 0) {
    // The two lanes of a row (lane/32 = 0, 1) combine.
    sq += __shfl_xor(sq, 32, 64);
    if (lane < brows) {
      if (gridDim.y == 1) p.out[i0 + lane] = (float)sqrt(sq);
      else p.part[(int64_t)blockIdx.y * N + i0 + lane] = sq;
    }
  } else if (p.epart) {
    const double t = wave_sum(sq);
    if (lane == 0) p.epart[((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave] = t;
  }
}

}  // namespace lora
