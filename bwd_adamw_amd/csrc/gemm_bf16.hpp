// Frozen-weight GEMMs with bf16 W on bf16 MFMA (v_mfma_f32_32x32x16_bf16),
// float32 accumulation.  Same contractions as gemm_f32.hpp:
//   forward: Z = Xb W^T + s U B^T                 (Xb = bf16(X), written by down)
//   dX     : dX = gb W + (s V A) * mask * keep    (gb = bf16(g), written by k3)
// The LoRA operands (U, B, V, A: float32) are rounded to bf16 while staging;
// U and V may arrive as split partials, summed in split order while staging.
//
// Block: NT threads = WGM x WGN waves over a BM x BN tile, K-step BK.  LDS is
// double buffered and holds both operands as [row][contraction] bf16 with a
// 16-byte pad, so every MFMA operand is one 128-bit LDS read: lane half h
// takes contraction indices h*BK/2 .. (h+1)*BK/2 - 1 of the K-step.  For dX
// the W tile arrives with the contraction index as its row (W's native [N,K]
// layout); it goes to LDS as loaded (16-byte pieces of W rows, XOR-swizzled)
// and each lane reads its operand with the LDS transpose load
// (ds_read_b64_tr_b16).
//
// The main loop keeps DEPTH K-steps of global loads in flight in registers
// (the load for step k + DEPTH is issued while step k is computed; DEPTH 1
// is the plain double buffer) with a straight-line body: every step issues its loads (clamped to the last step
// past the end), out-of-range elements are zeroed when stored to LDS, so the
// compiler waits for exactly the stage it stores.
//
// DEPTH 0 selects the direct-operand loop (bf16 W only, 256 x 256 tiles of
// four waves, K-step 64): LDS is the limit of the loop above (a K-step moves
// 192 KB of fragment reads and 64 KB of staging writes through it, and
// interleaved reads and writes share about 110 bytes per clock per CU).
// Here the activation operand bypasses LDS: it is stored in fragment tiles
// (atile_off: each 1 KB is one MFMA operand of 32 rows x 16 contraction
// indices in lane order, written so by down and k3), and each wave loads its
// own fragments into registers one K-step ahead.  Only W goes through LDS,
// by direct-to-LDS loads three K-steps ahead into a ring of four stages, read
// back as in the loop above (forward: rows of 128 bytes with their 16-byte
// chunks XOR-swizzled by row; dX: the tile as loaded, transpose reads).  A
// K-step is four phases of sixteen MFMAs, each overlapping the next phase's
// W fragment reads and a quarter of the loads, with one barrier per K-step.
// dX's LoRA term, which carries the dropout mask, is added after the loop.
//
// Block-quantized W (qweight.hpp) takes the same kernel with WQ set: W is
// staged as runs of 8 elements of a W row, decoded to bf16 on the way into
// LDS, so the LDS layout and the MFMA loop are unchanged.  For dX a thread's
// item is QR contraction rows x 8 columns, transposed while packing.
//
// The grid is one-dimensional.  Workgroups are dealt to the 8 XCDs round
// robin, so block b runs on XCD b % 8, and each XCD starts its blocks in
// order.  Block b is mapped to a contiguous run of tile indices per XCD, and
// tile indices walk the output in groups of GROUP_M tile rows, column by
// column, so the tiles an XCD has resident at once form a compact rectangle
// whose A and B K-slices are shared in that XCD's L2.
#pragma once
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "gemm_f32.hpp"   // LoraOperand
#include "qweight.hpp"

namespace lora {

// Per-slot operands of one product.  Adapter slots that share W run as one
// product over their stacked rows: rows [i*slot_rows, (i+1)*slot_rows) of the
// bf16 operand and of C belong to slot i, with its own LoRA factors, dropout
// keys and outputs.  A single linear is one slot.
constexpr int BF16_MAX_SLOTS = 4;
struct Bf16Slot {
  LoraOperand xa;          // U (fwd) or V (dx), float32 [rows, r], possibly as partials
  const float* XB;         // fwd: B_lora [Nc, r];  dx: A_lora [r, Nc]  (float32)
  float xs;                // LoRA scale s
  DropParams drop;         // dx: mask of the LoRA term at (slot row, n)
  float* C;                // [rows, Nc]
  float* C2;               // fwd DoRA: Z, or NULL
  const float* cn;         // fwd DoRA column scale cn/cd, or NULL
  const float* cd;
  const uint32_t* keep;    // dx: the mask's keep bits (k4 writes them; word w of
                           // slot row t at keep[w * rows + t]), or NULL: the
                           // mask is hashed here
};

struct GemmBf16Args {
  const uint16_t* A;       // [M, Kc] bf16, contraction contiguous (all slots stacked)
  int64_t lda;
  const uint16_t* B;       // fwd: W [Nc, Kc];  dx: W [Kc, Nc]   (bf16)
  int64_t ldb;
  QPlanes q;               // the same W block-quantized (kernels with WQ != WQ_BF16)
  int wq;                  // lora_dtype of W (host dispatch)
  int64_t M, Nc, Kc;
  int64_t r;
  Bf16Slot sl[BF16_MAX_SLOTS];
  int nslot;               // >= 1
  int64_t slot_rows;       // rows per slot when nslot > 1 (a multiple of the tile rows)
  int64_t ksplit;          // contraction length per split (multiple of BK)
  int nsplit;              // splits of the contraction across blocks
  float* part;             // [nsplit, M, Nc] partials when nsplit > 1
};

// The fields of slot `slot`, chosen scalar by scalar among constant-offset
// reads of the argument block: indexing it by a runtime value, or copying
// one of its structs whole, makes the compiler copy the block to scratch.
LORA_DEV Bf16Slot bf16_slot(const GemmBf16Args& p, int slot) {
  Bf16Slot so;
#define LORA_SEL(f)                          \
  so.f = p.sl[0].f;                          \
  _Pragma("unroll") for (int i = 1; i < BF16_MAX_SLOTS; ++i) \
    if (i == slot) so.f = p.sl[i].f;
  LORA_SEL(xa.p) LORA_SEL(xa.stride) LORA_SEL(xa.nparts) LORA_SEL(xa.out)
  LORA_SEL(XB) LORA_SEL(xs)
  LORA_SEL(drop.base) LORA_SEL(drop.thr) LORA_SEL(drop.keep) LORA_SEL(drop.on)
  LORA_SEL(C) LORA_SEL(C2) LORA_SEL(cn) LORA_SEL(cd) LORA_SEL(keep)
#undef LORA_SEL
  return so;
}

// Tile configurations: index, BM, BN, threads, wave rows, K-step, stages in
// flight (0: the direct-operand loop, whose A operand is fragment-tiled),
// directions (1 forward, 2 dX), then the host planner's fitted cost
// coefficients (forward a, b; dX a, b).
#define LORA_BF16_CFGS(X)                                        \
  X(0, 256, 256, 512, 2, 32, 3, 1, 0.417, 16.4, 0, 0)            \
  X(1, 256, 256, 512, 2, 64, 1, 3, 0.393, 14.7, 0.475, 14.1)     \
  X(2, 256, 128, 512, 2, 64, 2, 1, 0.483, 9.5, 0, 0)             \
  X(3, 256, 128, 512, 2, 64, 1, 2, 0, 0, 0.705, 7.8)             \
  X(4, 128, 128, 512, 2, 64, 2, 3, 0.581, 5.4, 0.967, 5.1)      \
  X(5, 256, 256, 256, 2, 64, 0, 3, 0.326, 12.2, 0.300, 20.0)

LORA_DEV uint32_t lo16(uint32_t x) { return x & 0xffffu; }
LORA_DEV uint32_t hi16(uint32_t x) { return x >> 16; }

// Instruction order of one phase of the direct-operand loop: MFMA i is
// followed by the phase's i-th LDS read (NRD of them) and, from the fifth
// MFMA on, by one of its NV global loads.
template <int NRD, int NV, int I>
LORA_DEV void phase_slot() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (I < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  if constexpr (I >= 4 && I < 4 + NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
}
template <int NRD, int NV, int... I>
LORA_DEV void phase_order(std::integer_sequence<int, I...>) {
  (phase_slot<NRD, NV, I>(), ...);
}

// Two floats to bf16 (round to nearest even, NaN stays NaN) in one
// v_cvt_pk_bf16_f32; a first in the low half.
LORA_DEV uint32_t cvt_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Two LDS transpose reads APART bytes apart, as one MFMA operand.  The
// restrict-qualified LDS pointer tells the compiler that these reads do not
// alias the direct-to-LDS loads in flight, which it would otherwise wait for.
LORA_DEV u32x4 tr_pair(const __attribute__((address_space(3))) char* __restrict__ b, int apart) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)b);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(b + apart));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// EXACT: M, Nc and Kc are multiples of BM, BN and BK: nothing is out of range.
// WQ: the lora_dtype of W (WQ_BF16, or a block-quantized format).
template <int BM, int BN, int NT, int WGM, int BK, int DEPTH, bool FWD, bool EXACT,
          int WQ = WQ_BF16>
__global__ __launch_bounds__(NT) void gemm_bf16_kernel(GemmBf16Args p) {
  constexpr int WGN = NT / 64 / WGM;
  constexpr int LDS_ROW = BK + 8;                   // bf16 elements per LDS row
  constexpr int CPR = BK / 8;                       // 16-byte chunks per row per K-step
  constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
  constexpr int ACH = BM * CPR / NT;                // 16-byte A chunks per thread
  constexpr int BCH = BN * CPR / NT;                // 16-byte B chunks per thread (fwd)
  // dX with bf16 W: the W tile is stored as loaded, [BK][BN] with its rows'
  // 32-byte segments XOR-swizzled by row, and the MFMA operand is read with
  // LDS transpose reads (TRB).  Quantized W decodes and transposes while
  // staging instead.
  constexpr bool TRB = !FWD && !wq_quantized(WQ);
  constexpr int BDC = BK * BN / 8;                  // TRB: 16-byte chunks of the W tile
  constexpr int BDCH = (BDC + NT - 1) / NT;
  constexpr int RPQB = NT / (BN / 8);               // TRB: W rows per thread pass
  static_assert(!TRB || (BDC % NT == 0 && NT % (BN / 8) == 0), "whole W chunks per thread");
  static_assert(!TRB || BK * BN <= BN * LDS_ROW, "TRB tile fits the B buffer");
  constexpr int KS = BK / 16;                       // MFMAs per K-step per output tile
  constexpr int LBK = 64;                           // K-step of the LoRA contraction
  constexpr int LROW = LBK + 8;
  static_assert(WGM * WGN * 64 == NT, "wave grid");
  static_assert(ACH >= 1 && BCH >= 1 && MI >= 1 && NI >= 1, "tile too small");
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "whole chunks per thread");
  static_assert((BM + BN) * LROW <= 2 * (BM + BN) * LDS_ROW, "LoRA staging fits the LDS");
  static_assert(DEPTH >= 0, "stages in flight");
  constexpr bool QW = wq_quantized(WQ);
  constexpr bool AD = DEPTH == 0;                     // direct-operand loop
  static_assert(!AD || (BM == 256 && BN == 256 && NT == 256 && WGM == 2 && BK == 64 && !QW),
                "direct-operand loop shape");
  constexpr int AD_NB = 4;                            // W stages in LDS (direct-operand loop)
  constexpr int QWD = QW ? wq_words(WQ) : 1;          // words per staged 8-element run
  constexpr int QR0 = BK * BN / (8 * NT);
  constexpr int QR = QR0 < 2 ? 2 : (QR0 > 8 ? 8 : QR0);  // dX: contraction rows per item
  constexpr int QCQ = BN / 8;                         // dX: 8-column groups per tile row
  constexpr int QITEMS = (BK / QR) * QCQ;
  constexpr int QIT = (QITEMS + NT - 1) / NT;
  static_assert(!QW || FWD || (BK % QR == 0 && QR % 2 == 0), "whole row pairs per item");

  constexpr int SMEM = AD ? (AD_NB * BN * BK > (BM + BN) * LROW ? AD_NB * BN * BK : (BM + BN) * LROW)
                          : 2 * (BM + BN) * LDS_ROW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  auto As = [&](int b) -> uint16_t* { return smem + b * (BM * LDS_ROW); };
  auto Bs = [&](int b) -> uint16_t* { return smem + 2 * BM * LDS_ROW + b * (BN * LDS_ROW); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int64_t ntn = (p.Nc + BN - 1) / BN, ntm = (p.M + BM - 1) / BM;
  // Blocks are (split, tile) pairs; an XCD's contiguous run of them covers
  // neighbouring tiles of one split, which share that split's K-slices.
  const int64_t tiles = ntm * ntn;
  const int64_t ts = xcd_tile(blockIdx.x, tiles * p.nsplit);
  int split = (int)(ts / tiles);
  int64_t tm, tn;
  grouped_tile(ts % tiles, ntm, ntn, tm, tn);
  if constexpr (AD) {
    // Scalar tile coordinates: W's direct-to-LDS loads take their resource
    // and offsets from them, and where the compiler cannot prove those
    // uniform it wraps every such load in a readfirstlane loop.
    split = __builtin_amdgcn_readfirstlane(split);
    tm = __builtin_amdgcn_readfirstlane((int)tm);
    tn = __builtin_amdgcn_readfirstlane((int)tn);
  }
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t kbeg = (int64_t)split * p.ksplit;
  const int64_t kend = min(p.Kc, kbeg + p.ksplit);
  const int hl = lane >> 5, l32 = lane & 31;
  // The slot's fields are selected only where they are used (LoRA term,
  // epilogue), so that none of them is live across the main loop.
  const int slot = p.nslot > 1 ? (int)(m0 / p.slot_rows) : 0;
  const int64_t moff = (int64_t)slot * p.slot_rows * (p.nslot > 1);   // slot's first row
  const bool lora = split == 0 && p.r > 0;

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  struct Stage {
    u32x4 a[ACH];
    u32x4 bf[(FWD && !QW) ? BCH : 1];
    u32x4 bd[TRB ? BDCH : 1];
    uint32_t qf[(FWD && QW) ? BCH : 1][QWD];          // quantized fwd: one run per chunk
    uint32_t qt[(!FWD && QW) ? QIT : 1][QR][QWD];     // quantized dX: QR runs per item
  };

  // Operand loads are raw buffer loads with a 32-bit byte offset (the
  // thread's base plus a uniform step), so a stage holds no 64-bit
  // addresses.  Each resource starts at this block's tiles and ends at its
  // operand's end, and the hardware returns zero for offsets past that end:
  // rows past the operand read as zero, and only the contraction edge
  // (forward) or column edge (dX) is masked, when the stage is stored.
  constexpr int RPQ = NT / CPR;                     // chunk rows per thread pass
  const int64_t arows = p.M - m0;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + m0 * p.lda), (short)0, (int)(uint32_t)min<int64_t>(0xffffffffll, arows * p.lda * 2),
      0x00020000);
  const uint32_t voffA = (uint32_t)(((tid / CPR) * p.lda + 8 * (tid % CPR)) * 2);
  const __amdgpu_buffer_rsrc_t rB =
      FWD ? __builtin_amdgcn_make_buffer_rsrc(
                (void*)(p.B + n0 * p.ldb), (short)0,
                (int)(uint32_t)min<int64_t>(0xffffffffll, (p.Nc - n0) * p.ldb * 2), 0x00020000)
          : __builtin_amdgcn_make_buffer_rsrc(
                (void*)(p.B + n0), (short)0,
                (int)(uint32_t)min<int64_t>(0xffffffffll, (p.Kc * p.ldb - n0) * 2), 0x00020000);
  static_assert(NT % CPR == 0, "uniform chunk rows");
  const uint32_t voffB = FWD ? (uint32_t)(((tid / CPR) * p.ldb + 8 * (tid % CPR)) * 2)
                             : (uint32_t)(((tid / (BN / 8)) * p.ldb + 8 * (tid % (BN / 8))) * 2);
  // Quantized W: W row length, and the planes' resources.
  const uint32_t qK = (uint32_t)(FWD ? p.Kc : p.Nc);
  const QRes<QW ? WQ : WQ_Q8_0> QRs(p.q);
  auto qt_ok = [&](int q) -> bool {
    const int f = tid + NT * q;
    return (EXACT || n0 + 8 * (f % QCQ) < p.Nc) && f < QITEMS;
  };

  auto a_ok = [&](int64_t k0) -> bool { return EXACT || k0 + 8 * (tid % CPR) < kend; };
  auto bd_ok = [&]() -> bool { return EXACT || n0 + 8 * (tid % (BN / 8)) < p.Nc; };
  // TRB: byte offset of 16-byte chunk c of W-tile row kk in the B buffer.
  auto bd_off = [&](int kk, int c) -> int {
    return kk * (BN * 2) + (((c >> 1) ^ (2 * (kk & 3))) << 5) + ((c & 1) << 4);
  };
  auto load = [&](Stage& S, int64_t k0) {
#pragma unroll
    for (int q = 0; q < ACH; ++q)
      S.a[q] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rA, voffA + (uint32_t)((q * RPQ * p.lda + k0) * 2), 0, 0));
    if constexpr (QW && FWD) {
#pragma unroll
      for (int q = 0; q < BCH; ++q) {
        const int f = tid + NT * q;
        wq_load<WQ>(QRs, qK, (uint32_t)(n0 + f / CPR), (uint32_t)(k0 + 8 * (f % CPR)), S.qf[q]);
      }
    } else if constexpr (QW) {
#pragma unroll
      for (int q = 0; q < QIT; ++q) {
        const int f = tid + NT * q;
        const uint32_t col = (uint32_t)(n0 + 8 * (f % QCQ));
        const uint32_t row = (uint32_t)(k0 + QR * (f / QCQ));
#pragma unroll
        for (int i = 0; i < QR; ++i) wq_load<WQ>(QRs, qK, row + i, col, S.qt[q][i]);
      }
    } else if constexpr (FWD) {
#pragma unroll
      for (int q = 0; q < BCH; ++q)
        S.bf[q] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rB, voffB + (uint32_t)((q * RPQ * p.ldb + k0) * 2), 0, 0));
    } else {
#pragma unroll
      for (int q = 0; q < BDCH; ++q)
        S.bd[q] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rB, voffB + (uint32_t)(((int64_t)q * RPQB + k0) * p.ldb * 2), 0, 0));
    }
  };
  auto store = [&](const Stage& S, int64_t k0, int buf) {
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const bool aok = a_ok(k0);
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int f = tid + NT * q;
      *reinterpret_cast<u32x4*>(&As(buf)[(f / CPR) * LDS_ROW + 8 * (f % CPR)]) = aok ? S.a[q] : z4;
    }
    if constexpr (QW && FWD) {
#pragma unroll
      for (int q = 0; q < BCH; ++q) {
        const int f = tid + NT * q;
        float v[8];
        wq_decode<WQ>(S.qf[q], v);
        const u32x4 o = {wq_pack(v[0], v[1]), wq_pack(v[2], v[3]), wq_pack(v[4], v[5]),
                         wq_pack(v[6], v[7])};
        *reinterpret_cast<u32x4*>(&Bs(buf)[(f / CPR) * LDS_ROW + 8 * (f % CPR)]) = aok ? o : z4;
      }
    } else if constexpr (QW) {
#pragma unroll
      for (int q = 0; q < QIT; ++q) {
        const int f = tid + NT * q;
        if (f >= QITEMS) continue;
        const bool ok = qt_ok(q);
        float v[QR][8];
#pragma unroll
        for (int i = 0; i < QR; ++i) wq_decode<WQ>(S.qt[q][i], v[i]);
        // column e of the QR x 8 run block becomes QR contraction values
        uint16_t* dst = &Bs(buf)[(8 * (f % QCQ)) * LDS_ROW + QR * (f / QCQ)];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t o[QR / 2];
#pragma unroll
          for (int d = 0; d < QR / 2; ++d) o[d] = ok ? wq_pack(v[2 * d][e], v[2 * d + 1][e]) : 0u;
          if constexpr (QR == 8) {
            *reinterpret_cast<u32x4*>(dst + e * LDS_ROW) = u32x4{o[0], o[1], o[2], o[3]};
          } else if constexpr (QR == 4) {
            *reinterpret_cast<u32x2*>(dst + e * LDS_ROW) = u32x2{o[0], o[1]};
          } else {
            *reinterpret_cast<uint32_t*>(dst + e * LDS_ROW) = o[0];
          }
        }
      }
    } else if constexpr (FWD) {
#pragma unroll
      for (int q = 0; q < BCH; ++q) {
        const int f = tid + NT * q;
        *reinterpret_cast<u32x4*>(&Bs(buf)[(f / CPR) * LDS_ROW + 8 * (f % CPR)]) = aok ? S.bf[q] : z4;
      }
    } else {
      const bool ok = bd_ok();
      char* bb = reinterpret_cast<char*>(Bs(buf));
#pragma unroll
      for (int q = 0; q < BDCH; ++q) {
        const int f = tid + NT * q;
        *reinterpret_cast<u32x4*>(bb + bd_off(f / (BN / 8), f % (BN / 8))) = ok ? S.bd[q] : z4;
      }
    }
  };
  // MFMA over one staged K-step: STEPS MFMAs of 16 contraction indices per
  // output tile, lane half hl holding indices hl*HALF .. of each LD-wide row.
  // TRB: lane l = 16 g + i reads W-tile rows kb + i/4 and kb + 4 + i/4 at
  // columns nb + 4 (i%4) .. +3, kb = 32 (g/2) + 8 s, nb = the n-tile's
  // 16 (g%2); the transpose read hands lane l column nb + i with 4 rows each,
  // so the pair is the 8 contraction values 32 (l/32) + 8 s .. +7 of column
  // l%32, the order the A operand uses.
  const int trg = lane >> 4, tri = lane & 15;
  auto tr_frag = [&](const uint16_t* Bb, int n, int s) -> u32x4 {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int kk = 32 * (trg >> 1) + 8 * s + (tri >> 2);
    const int col = n + 16 * (trg & 1) + 4 * (tri & 3);
    const int off = kk * (BN * 2) + (((col >> 4) ^ (2 * (kk & 3))) << 5) + ((col & 15) << 1);
    auto* b = (__attribute__((address_space(3))) char*)(Bb);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(b + off));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(b + off + 4 * (BN * 2)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  auto compute = [&](const uint16_t* Ab, const uint16_t* Bb, auto LD, auto HALF, auto STEPS,
                     auto TR) {
    constexpr int ld = decltype(LD)::value, half = decltype(HALF)::value;
#pragma unroll
    for (int s = 0; s < decltype(STEPS)::value; ++s) {
      u32x4 av[MI], bv[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        av[i] = *reinterpret_cast<const u32x4*>(&Ab[(wm0 + i * 32 + l32) * ld + half * hl + 8 * s]);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if constexpr (decltype(TR)::value)
          bv[j] = tr_frag(Bb, wn0 + j * 32, s);
        else
          bv[j] = *reinterpret_cast<const u32x4*>(&Bb[(wn0 + j * 32 + l32) * ld + half * hl + 8 * s]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          // Both directions compute the tile transposed (W-side operand
          // first): each lane then holds four consecutive output columns of
          // one row per accumulator group (epilogue below).
          acc[i][j] = mfma32x32x16_bf16(bv[j], av[i], acc[i][j]);
        }
    }
  };
  using MainLd = std::integral_constant<int, LDS_ROW>;
  using MainHalf = std::integral_constant<int, BK / 2>;
  using MainSteps = std::integral_constant<int, KS>;
  using MainTr = std::integral_constant<bool, TRB>;
  // dX's LoRA term on the direct-operand loop, added after the main loop (the
  // dropout mask applies to this term only).  Per 32 x 32 fragment: the term
  // t into a 16-register temporary, d = mask * t, then d into the
  // accumulators by MFMA, never by vector ALU work on them (which makes the
  // compiler move all 256 accumulators out of the AGPRs and spill).  The
  // injection uses that lane (m, h) holds d at n = 16u + 8(e/4) + 4h + e%4
  // for its element v = 8u + e: read as contraction slot 8h + e of MFMA u,
  // its own eight values are the m-side operand, and the W-side operand is
  // the constant 0/1 matrix P_u that maps slot 8h + e to that n.  d goes in
  // as bf16 hi and lo parts (hi + lo equals d to about 2^-18 relative).
  auto compute_masked = [&](const uint16_t* Ab, const uint16_t* Bb, DropParams dp, const uint32_t* keep) {
    constexpr int half = LBK / 2, NS = LBK / 16;
    // Opaque per call: the multipliers and the lane's indices do not depend
    // on the rank chunk, and hoisted out of the chunk loop (or above the main
    // loop) they would hold registers across it.
    int ln = lane;
    asm volatile("" : "+s"(dp.base), "+s"(dp.thr), "+v"(ln));
    const int h = ln >> 5, r32 = ln & 31;
    u32x4 P[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int n_lo = 16 * u + 8 * (e >> 2) + 4 * h + (e & 3);
        P[u][e / 2] = (r32 == n_lo ? 0x3f80u : 0u) | (r32 == n_lo + 1 ? 0x3f800000u : 0u);
      }
    // Stored keep bits: row m's word for each 32 columns j of the wave (a
    // wave's load is 32 consecutive rows of one word), all issued first.
    // Words past Nc are not read; their columns are not stored.
    uint32_t kwd[MI][NI];
    if (dp.on && keep != nullptr) {
      const int64_t rows = p.nslot > 1 ? p.slot_rows : p.M;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int64_t m = m0 + wm0 + i * 32 + r32;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int64_t c = n0 + wn0 + 32 * j;
          const bool ok = c < p.Nc && m < p.M;
          kwd[i][j] = keep[ok ? (c >> 5) * rows + (m - moff) : 0];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      u32x4 av[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        av[s] = *reinterpret_cast<const u32x4*>(&Ab[(wm0 + i * 32 + r32) * LROW + half * h + 8 * s]);
      const uint64_t rk = keep != nullptr ? 0 : drop_row(dp, m0 + wm0 + i * 32 + r32 - moff);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        f32x16 t;
#pragma unroll
        for (int v = 0; v < 16; ++v) t[v] = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          t = mfma32x32x16_bf16(
              *reinterpret_cast<const u32x4*>(&Bb[(wn0 + j * 32 + r32) * LROW + half * h + 8 * s]), av[s], t);
        // the fragment's keep bits first, one word (short hash lifetimes)
        uint32_t kb = 0xffffu;
        if (dp.on && keep != nullptr) {
          // bit v: column 8 (v/4) + 4h + v%4 of the fragment's 32
          const uint32_t w = kwd[i][j] >> (4 * h);
          kb = (w & 0xfu) | (w >> 4 & 0xf0u) | (w >> 8 & 0xf00u) | (w >> 12 & 0xf000u);
        } else if (dp.on) {
          kb = 0;
#pragma unroll
          for (int v = 0; v < 16; ++v) kb |= (uint32_t)drop_keep(dp, rk, n0 + wn0 + j * 32 + row32(v, ln)) << v;
        }
        __builtin_amdgcn_sched_barrier(0);
        uint32_t hi[8], lo[8];   // packed pairs (v, v + 1)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float m0_ = (kb >> v & 1u) ? (dp.on ? dp.keep : 1.0f) : 0.0f;
          const float m1_ = (kb >> (v + 1) & 1u) ? (dp.on ? dp.keep : 1.0f) : 0.0f;
          const float d0 = m0_ * t[v], d1 = m1_ * t[v + 1];
          hi[v / 2] = cvt_bf16x2(d0, d1);
          const float r0 = d0 - __uint_as_float(hi[v / 2] << 16);
          const float r1 = d1 - __uint_as_float(hi[v / 2] & 0xffff0000u);
          lo[v / 2] = cvt_bf16x2(r0 == r0 ? r0 : 0.0f, r1 == r1 ? r1 : 0.0f);   // d infinite: hi alone
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 h = {hi[4 * u], hi[4 * u + 1], hi[4 * u + 2], hi[4 * u + 3]};
          const u32x4 l = {lo[4 * u], lo[4 * u + 1], lo[4 * u + 2], lo[4 * u + 3]};
          acc[i][j] = mfma32x32x16_bf16(P[u], h, acc[i][j]);
          acc[i][j] = mfma32x32x16_bf16(P[u], l, acc[i][j]);
        }
      }
    }
  };
  // LoRA contraction over the rank: float32 operands rounded to bf16 in LDS,
  // in 64-wide K-steps over the same LDS (MASKED: dX after the direct-operand
  // loop, through compute_masked).
  auto lora_contraction = [&](auto MASKED) {
    const Bf16Slot so = bf16_slot(p, slot);
    const bool store_xa = so.xa.out != nullptr && n0 == 0 && split == 0;
    uint16_t* La = smem;
    uint16_t* Lb = smem + BM * LROW;
    for (int64_t k0 = 0; k0 < p.r; k0 += LBK) {
      __syncthreads();
      if constexpr (AD) {
      // The direct-operand kernel (accumulators apart from its vector
      // registers) issues all its staging loads before any is used (clamped
      // addresses, values selected): one round trip rather than one per item.
      // A side: XA [M, r] rows m, scaled by s; as split partials, summed in
      // split order (and stored once, by the first column of tiles).
      // Forward B side: B_lora [Nc, r], rows n, rank contiguous.  dX B side:
      // A_lora [r, Nc]: a thread reads four columns of sixteen consecutive
      // rows as 16-byte pieces (each load a contiguous 1 KB per wave) and
      // stores each column's sixteen values transposed, as two 16-byte writes.
      constexpr int AIT = BM * (LBK / 4) / NT;        // A items (four floats) per thread
      constexpr int BIT = FWD ? BN * (LBK / 4) / NT : 0;   // forward B items
      constexpr int NIT = AIT > BIT ? AIT : BIT;
      constexpr int QD = LBK / (NT / 64);             // dX: A_lora rows per thread
      constexpr int SB = NIT;
      static_assert(BM * (LBK / 4) % NT == 0 && BN * (LBK / 4) % NT == 0, "whole staging batches");
      static_assert(FWD || (BN == 4 * 64 && QD == 16), "dX: four columns per lane, 16 rows per wave");
      auto item = [&](int it, int64_t o0, int64_t lim, int& row, int& c4, bool& ok) -> int64_t {
        const int f = tid + NT * it;
        row = f / (LBK / 4);
        c4 = f % (LBK / 4);
        const int64_t g = o0 + row, gk = k0 + 4 * c4;
        ok = g < lim && gk < p.r;
        return ok ? g * p.r + gk : 0;
      };
      auto put = [&](uint16_t* dst, int row, int c4, bool ok, f32x4 v) {
        v = ok ? v : f32x4{0.f, 0.f, 0.f, 0.f};
        const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(&dst[row * LROW + 4 * c4]) = w;
      };
#pragma unroll
      for (int b0 = 0; b0 < NIT; b0 += SB) {
        f32x4 va[SB], vb[SB];
        if (so.xa.nparts == 1) {
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            if (b0 + u >= AIT) continue;
            int row, c4;
            bool ok;
            va[u] = *reinterpret_cast<const f32x4*>(so.xa.p + item(b0 + u, m0 - moff, p.M - moff, row, c4, ok));
          }
        } else {
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            if (b0 + u >= AIT) continue;
            int row, c4;
            bool ok;
            const int64_t i = item(b0 + u, m0 - moff, p.M - moff, row, c4, ok);
            va[u] = sum_parts4(so.xa.p, so.xa.stride, so.xa.nparts, i);
            if (store_xa && ok) *reinterpret_cast<f32x4*>(so.xa.out + i) = va[u];
          }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          if (b0 + u >= BIT) continue;
          int row, c4;
          bool ok;
          vb[u] = *reinterpret_cast<const f32x4*>(so.XB + item(b0 + u, n0, p.Nc, row, c4, ok));
        }
        f32x4 vd[FWD ? 1 : QD];
        const int dc = 4 * (tid & 63), dr = QD * (tid >> 6);   // dX: first column, first row
        if constexpr (!FWD) {
          const bool cok = n0 + dc < p.Nc;                     // Nc is a multiple of 8
#pragma unroll
          for (int q = 0; q < QD; ++q) {
            const int64_t gk = k0 + dr + q;
            vd[q] = *reinterpret_cast<const f32x4*>(so.XB + ((cok && gk < p.r) ? gk * p.Nc + n0 + dc : 0));
          }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          int row, c4;
          bool ok;
          if (b0 + u < AIT) {
            item(b0 + u, m0 - moff, p.M - moff, row, c4, ok);
            put(La, row, c4, ok, va[u] * so.xs);
          }
          if (b0 + u < BIT) {
            item(b0 + u, n0, p.Nc, row, c4, ok);
            put(Lb, row, c4, ok, vb[u]);
          }
        }
        if constexpr (!FWD) {
          const bool cok = n0 + dc < p.Nc;
#pragma unroll
          for (int q = 0; q < QD; ++q)
            if (!(cok && k0 + dr + q < p.r)) vd[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int h8 = 0; h8 < QD; h8 += 8) {
              const u32x4 w = {pack_bf16x2(vd[h8][e], vd[h8 + 1][e]), pack_bf16x2(vd[h8 + 2][e], vd[h8 + 3][e]),
                               pack_bf16x2(vd[h8 + 4][e], vd[h8 + 5][e]), pack_bf16x2(vd[h8 + 6][e], vd[h8 + 7][e])};
              *reinterpret_cast<u32x4*>(&Lb[(dc + e) * LROW + dr + h8]) = w;
            }
        }
      }
      } else {
      // A side: XA [M, r] rows m (split partials summed), scaled by s.
      for (int f = tid; f < BM * (LBK / 4); f += NT) {
        const int row = f / (LBK / 4), c4 = f % (LBK / 4);
        const int64_t gm = m0 + row, gk = k0 + 4 * c4;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gm < p.M && gk < p.r) {
          const int64_t i = (gm - moff) * p.r + gk;
          v = sum_parts4(so.xa.p, so.xa.stride, so.xa.nparts, i);
          if (store_xa && so.xa.nparts > 1) *reinterpret_cast<f32x4*>(so.xa.out + i) = v;
          v *= so.xs;
        }
        u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(&La[row * LROW + 4 * c4]) = b;
      }
      if constexpr (FWD) {
        // B_lora [Nc, r]: rows n, rank contiguous.
        for (int f = tid; f < BN * (LBK / 4); f += NT) {
          const int row = f / (LBK / 4), c4 = f % (LBK / 4);
          const int64_t gn = n0 + row, gk = k0 + 4 * c4;
          f32x4 v = {0.f, 0.f, 0.f, 0.f};
          if (gn < p.Nc && gk < p.r) v = *reinterpret_cast<const f32x4*>(so.XB + gn * p.r + gk);
          u32x2 b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(&Lb[row * LROW + 4 * c4]) = b;
        }
      } else {
        // A_lora [r, Nc]: rows are the contraction index; transpose on store.
        for (int f = tid; f < BN * LBK; f += NT) {
          const int n = f % BN, kk = f / BN;
          const int64_t gn = n0 + n, gk = k0 + kk;
          float v = 0.f;
          if (gn < p.Nc && gk < p.r) v = so.XB[gk * p.Nc + gn];
          Lb[n * LROW + kk] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
      }
      __syncthreads();
      if constexpr (decltype(MASKED)::value)
        compute_masked(La, Lb, so.drop, so.keep);
      else
        compute(La, Lb, std::integral_constant<int, LROW>{}, std::integral_constant<int, LBK / 2>{},
                std::integral_constant<int, LBK / 16>{}, std::false_type{});
    }
    __syncthreads();
  };

  if (!FWD && !AD && lora) {
    lora_contraction(std::false_type{});
    const Bf16Slot so = bf16_slot(p, slot);
    if (so.drop.on) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int64_t gm = m0 + wm0 + i * 32 + l32;
        const uint64_t rk = drop_row(so.drop, gm - moff);
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t gn = n0 + wn0 + j * 32 + row32(v, lane);
            acc[i][j][v] *= drop_mul(so.drop, rk, gn);
          }
      }
    }
  }

  // Main contraction over [kbeg, kend); every split but the last is a whole
  // number of K-steps, so a K-step never reaches into the next split.
  const int64_t nk = (kend - kbeg + BK - 1) / BK;
  if constexpr (AD) {
    constexpr int STG = BN * BK;                      // bf16 elements per W stage
    const int64_t nkq = p.Kc / BK;                    // K-steps of the tiled operand's rows
    // The wave index as a scalar: resources and LDS destinations built from
    // it stay in scalar registers.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // This wave's four 32-row fragment rows of the tiled operand, from its
    // first; the resource ends at the operand's end (rows past M read zero).
    const int64_t rb0 = (m0 + (wv / WGN) * WM) / 32, rbn = (p.M + 31) / 32;
    // (integer selects: a max() here resolves to a floating-point overload,
    // which would put the resource in vector registers)
    const int64_t abytes = (rbn > rb0 ? rbn - rb0 : 0) * nkq * 4096;
    const __amdgpu_buffer_rsrc_t rAt = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.A + rb0 * nkq * 2048), (short)0, (int)(abytes > 0xffffffffll ? 0xffffffffu : (uint32_t)abytes),
        0x00020000);
    auto kq = [&](int64_t k) { return kbeg / BK + min(k, nk - 1); };
    // Fragment (row block i, K-step q, sub-step s) is at byte
    // ((i * nkq + q) * 4 + s) * 1024 + 16 lane: the lane and row-block part
    // is a per-lane constant, the step part a scalar offset.
    uint32_t voffA[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) voffA[i] = (uint32_t)(lane * 16 + (int64_t)i * nkq * 4096);
    auto lda_sub = [&](u32x4 (&R)[MI][KS], int s, int64_t k) {
      const int so = (int)(kq(k) * 4096 + s * 1024);
#pragma unroll
      for (int i = 0; i < MI; ++i)
        R[i][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rAt, voffA[i], so, 0));
    };
    // W: each wave's eight direct-to-LDS loads per stage write 1 KB each.
    // Forward: load q covers W rows 8 (8 wave + q) .. +7, lane l the row's
    // 16-byte slot l%8, which holds chunk (l%8) ^ swz(row).  dX: load q
    // covers contraction rows 2 (8 wave + q) and the next, lane l the row's
    // slot l%32 of the transposed layout (bd_off).
    auto swz = [](int row) { return (row ^ (row >> 3)) & 7; };
    uint32_t voffW[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if constexpr (FWD) {
        const int row = 8 * (8 * wave + q) + (lane >> 3);
        voffW[q] = (uint32_t)(((int64_t)row * p.ldb + 8 * ((lane & 7) ^ swz(row))) * 2);
      } else {
        const int kk = 2 * (8 * wave + q) + (lane >> 5), sl = lane & 31;
        const int c = ((((sl >> 1) ^ (2 * (kk & 3)))) << 1) | (sl & 1);
        voffW[q] = (uint32_t)(((int64_t)kk * p.ldb + 8 * c) * 2);
      }
    }
    auto dma = [&](int q, int64_t k, int buf) {
      const int64_t k0 = kbeg + min(k, nk - 1) * BK;
      uint16_t* dst = smem + buf * STG + (FWD ? 8 * (8 * wv + q) * BK : 2 * (8 * wv + q) * BN);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (__attribute__((address_space(3))) void*)dst, 16, voffW[q],
                                               (int)(uint32_t)(FWD ? k0 * 2 : k0 * p.ldb * 2), 0, 0);
    };
    // W fragment of column block j, sub-step s: forward, row n = wn0 + 32 j
    // + l%32 at chunk (4 (l/32) + s) ^ swz(n), i.e. byte wb[j] + 16 (s ^
    // wm[j]); dX, the transposed read at byte wb[j] + 4096 s (its swizzle
    // depends on the row only modulo 4, which s does not change).
    uint32_t wb[NI], wm[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      if constexpr (FWD) {
        const int row = wn0 + j * 32 + l32, sw = swz(row);
        wb[j] = (uint32_t)(row * BK * 2 + 64 * (hl ^ (sw >> 2)));
        wm[j] = (uint32_t)(sw & 3);
      } else {
        const int kk = 32 * (trg >> 1) + (tri >> 2);
        const int col = wn0 + j * 32 + 16 * (trg & 1) + 4 * (tri & 3);
        wb[j] = (uint32_t)(kk * (BN * 2) + (((col >> 4) ^ (2 * (kk & 3))) << 5) + ((col & 15) << 1));
        wm[j] = 0;
      }
    }
    u32x4 Bf[2][NI];
    auto rdb = [&](u32x4 (&F)[NI], int buf, int s) {
      const char* Bb = reinterpret_cast<const char*>(smem + buf * STG);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if constexpr (FWD) {
          F[j] = *reinterpret_cast<const u32x4*>(Bb + wb[j] + 16 * (s ^ wm[j]));
        } else {
          F[j] = tr_pair((__attribute__((address_space(3))) const char*)(Bb + wb[j] + 4096 * s), 4 * (BN * 2));
        }
      }
    };
    auto mma = [&](const u32x4 (&R)[MI][KS], int s, const u32x4 (&F)[NI]) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          acc[i][j] = mfma32x32x16_bf16(F[j], R[i][s], acc[i][j]);
        }
    };
    // Phase s of K-step k: W fragments of sub-step s + 1 (the last phase:
    // sub-step 0 of the next stage, after the barrier), the tiled operand's
    // sub-step s of step k + 1 (used a whole K-step later), W loads 2s and
    // 2s + 1 for step k + 3, and the sixteen MFMAs of sub-step s.  The
    // barrier waits for this wave's loads of stage k + 1 (issued in step
    // k - 2): at most 7 (MI + 2) loads were issued after them (MI + 2 per
    // phase, step k - 1's four phases and step k's first three).
    using Seq = std::make_integer_sequence<int, MI * NI>;
    u32x4 Ar[2][MI][KS];
    auto step = [&](int64_t k, u32x4 (&Rc)[MI][KS], u32x4 (&Rn)[MI][KS]) {
      const int cur = (int)(k % AD_NB), nx1 = (int)((k + 1) % AD_NB), nx3 = (int)((k + 3) % AD_NB);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        if (s == KS - 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(7 * (MI + 2)) : "memory");
        rdb(Bf[(s + 1) & 1], s == KS - 1 ? nx1 : cur, (s + 1) % KS);
        lda_sub(Rn, s, k + 1);
        dma(2 * s, k + 3, nx3);
        dma(2 * s + 1, k + 3, nx3);
        mma(Rc, s, Bf[s & 1]);
        phase_order<FWD ? NI : 2 * NI, MI + 2>(Seq{});
      }
    };
    // Issue order (fixed by the scheduling barriers): W stages 0, 1 and 2,
    // the operand's step 0; stage 0 is in once 16 + MI KS later loads may
    // remain.
#pragma unroll
    for (int q = 0; q < 8; ++q) dma(q, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) dma(q, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) dma(q, 2, 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ss = 0; ss < KS; ++ss) lda_sub(Ar[0], ss, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(16 + MI * KS) : "memory");
    rdb(Bf[0], 0, 0);
    int64_t k = 0;
    for (; k + 2 <= nk; k += 2) {
      step(k, Ar[0], Ar[1]);
      step(k + 1, Ar[1], Ar[0]);
    }
    if (k < nk) step(k, Ar[0], Ar[1]);
    __builtin_amdgcn_sched_barrier(0);
    // No W load may still be writing LDS when it is reused or released.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    Stage R[DEPTH];
    auto kstep = [&](int64_t k) { return kbeg + min(k, nk - 1) * BK; };
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) load(R[u], kstep(u));
    store(R[0], kbeg, 0);
    __syncthreads();
    int64_t k = 0;
    for (; k + DEPTH <= nk; k += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int64_t kk = k + u;
        load(R[u], kstep(kk + DEPTH));
        // Keep the loads ahead of this step's MFMAs: left to itself the
        // scheduler sinks them next to their LDS stores to shorten register
        // lifetimes, which exposes their whole latency.
        __builtin_amdgcn_sched_barrier(0);
        const int buf = (int)(kk & 1);
        compute(As(buf), Bs(buf), MainLd{}, MainHalf{}, MainSteps{}, MainTr{});
        store(R[(u + 1) % DEPTH], kstep(kk + 1), buf ^ 1);
        __syncthreads();
      }
    }
    // Fewer than DEPTH steps left; their loads are already in flight.
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u) {
      const int64_t kk = k + u;
      if (kk < nk) {
        const int buf = (int)(kk & 1);
        compute(As(buf), Bs(buf), MainLd{}, MainHalf{}, MainSteps{}, MainTr{});
        if (kk + 1 < nk) store(R[(u + 1) % DEPTH], kstep(kk + 1), buf ^ 1);
        __syncthreads();
      }
    }
  }

  if (FWD && lora) lora_contraction(std::false_type{});
  if (!FWD && AD && lora) lora_contraction(std::true_type{});

  const Bf16Slot so = bf16_slot(p, slot);
  // The MFMA computes the tile transposed (W-side operand first), so lane l
  // holds output row m = .. + l%32 and, per group of four accumulators, four
  // consecutive columns: every store is a 16-byte vector (the forward's Y, Z
  // and split partials as much as dX), and dX's dropout mask of the LoRA term
  // needs one row key per row.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t gm = m0 + wm0 + i * 32 + l32;
    if (gm >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int64_t gn = n0 + wn0 + j * 32 + row32(4 * v4, lane);   // Nc is a multiple of 4
        if (gn >= p.Nc) continue;
        f32x4 x = {acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                   acc[i][j][4 * v4 + 3]};
        if (p.nsplit == 1) {
          const int64_t o = (gm - moff) * p.Nc + gn;
          if (so.C2) *reinterpret_cast<f32x4*>(so.C2 + o) = x;
          if (so.cn) {
            const f32x4 cn = *reinterpret_cast<const f32x4*>(so.cn + gn);
            const f32x4 cd = *reinterpret_cast<const f32x4*>(so.cd + gn);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] *= cn[e] / cd[e];
          }
          *reinterpret_cast<f32x4*>(so.C + o) = x;
        } else {
          *reinterpret_cast<f32x4*>(p.part + ((int64_t)split * p.M + gm) * p.Nc + gn) = x;
        }
      }
  }
}

// Sum of the split partials in split order, then the unsplit kernel's
// epilogue, row by row into the row's slot (Z = sum; Y = sum * cn/cd).
static __global__ __launch_bounds__(256) void splitk_reduce_bf16_kernel(GemmBf16Args p) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = p.M * p.Nc;
  if (i4 >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(p.part + i4);
  for (int q = 1; q < p.nsplit; ++q) s += *reinterpret_cast<const f32x4*>(p.part + q * total + i4);
  const int64_t m = i4 / p.Nc, n = i4 % p.Nc;   // Nc is a multiple of 4
  const int slot = p.nslot > 1 ? (int)(m / p.slot_rows) : 0;
  const Bf16Slot so = bf16_slot(p, slot);
  const int64_t o = (m - (int64_t)slot * p.slot_rows * (p.nslot > 1)) * p.Nc + n;
  if (so.C2) *reinterpret_cast<f32x4*>(so.C2 + o) = s;
  if (so.cn) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] *= so.cn[n + e] / so.cd[n + e];
  }
  *reinterpret_cast<f32x4*>(so.C + o) = s;
}

}  // namespace lora
