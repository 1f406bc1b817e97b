// Tiled MFMA GEMM for 16-bit (FP16, BF16) and 8-bit (OCP E4M3) operands on
// gfx950, FP32 accumulation.
//
// One workgroup computes a BP x BQ block of D[p][q] = sum_k P(p,k) Q(q,k)
// (see GemmArgs for how A, B and C map onto P, Q and D).  The structure
// follows the software pipeline the pages build up ("FP16 GEMM Optimization
// on AMD RDNA 3 and RDNA 4", Steps 2-6; "An Educational GEMM Ladder for
// Helios GPUs", Levels 1-5), re-derived for CDNA4:
//
//  * Global -> registers: 16-byte buffer loads through a descriptor whose
//    num_records bounds the block's valid region; rows past the matrix edge
//    and chunks past K are pushed out of range and read as zero (Step 4).
//    A chunk that straddles K is masked element by element in registers.
//  * Registers -> LDS: every LDS row holds one stage of K for one p (or q)
//    index, 128 bytes, K-contiguous for both operands ("What We Are
//    Computing": K last in every LDS tile).  16-byte chunks are XOR-swizzled
//    with key (row / 2) mod 8 (Step 3's permutation, re-keyed for gfx950:
//    64 banks x 4 bytes = 256 bytes per bank row hold two 128-byte tile rows,
//    so rows 2r and 2r+1 share a key and differ in the bank half instead).
//    The NN B operand arrives p-contiguous and is transposed element by
//    element on its way into LDS.
//  * Double buffering with a staged commit: the next stage's global loads are
//    issued before the current stage's MFMAs and written to the other LDS
//    buffer after them, one barrier per stage (Step 2).
//  * MFMA: v_mfma_f32_32x32x16_{f16,bf16} (k = 16, 16 bytes per lane per
//    operand) or the unscaled v_mfma_f32_32x32x64_f8f6f4 (k = 64, 32 bytes
//    per lane), FP32 accumulators in registers.
//  * Epilogue: each lane holds four consecutive p of one q, contiguous in C;
//    convert with round-to-nearest-even and store 8 or 16 bytes at a time.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace dg {

// ---- per-format operations ---------------------------------------------------

struct OpF16 {
  static constexpr int ELEM = 2;   // bytes per input element
  static constexpr int KI = 16;    // k per MFMA
  static constexpr int FC = 1;     // 16-byte chunks per lane per operand per MFMA
  static constexpr int OE = 2;     // bytes per output element
  static constexpr bool SCALED = false;  // scale factors applied in the epilogue
  static constexpr bool MX = false;      // E8M0 block scales fed to the MFMA
  typedef f16x8 Frag;
  __device__ static Frag frag(const char* base, const uint32_t* off) { return *(const Frag*)(base + off[0]); }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float x, float y) {
    const _Float16 hx = (_Float16)x, hy = (_Float16)y;
    return (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
  }
  __device__ static uint16_t one(float x) { const _Float16 h = (_Float16)x; return __builtin_bit_cast(uint16_t, h); }
  __device__ static f32x16 mma_parts(const u32x4 (&a)[1], const u32x4 (&b)[1], f32x16 c) {
    return mma(__builtin_bit_cast(Frag, a[0]), __builtin_bit_cast(Frag, b[0]), c);
  }
  // The 16 x 16 x 32 MFMA (the four-wave kernel): lane l holds row l % 16
  // of A and column l % 16 of B, each with 8 k (lanes 16g .. 16g + 15 the
  // same k); D holds rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.
  __device__ static f32x4 mma16(const u32x4 (&a)[1], const u32x4 (&b)[1], f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(Frag, a[0]), __builtin_bit_cast(Frag, b[0]), c, 0,
                                                   0, 0);
  }
};

struct OpBF16 {
  static constexpr int ELEM = 2, KI = 16, FC = 1, OE = 2;
  static constexpr bool SCALED = false, MX = false;
  typedef bf16x8 Frag;
  __device__ static Frag frag(const char* base, const uint32_t* off) { return *(const Frag*)(base + off[0]); }
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float x, float y) {
    const __bf16 hx = (__bf16)x, hy = (__bf16)y;
    return (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
  }
  __device__ static uint16_t one(float x) { const __bf16 h = (__bf16)x; return __builtin_bit_cast(uint16_t, h); }
  __device__ static f32x16 mma_parts(const u32x4 (&a)[1], const u32x4 (&b)[1], f32x16 c) {
    return mma(__builtin_bit_cast(Frag, a[0]), __builtin_bit_cast(Frag, b[0]), c);
  }
  __device__ static f32x4 mma16(const u32x4 (&a)[1], const u32x4 (&b)[1], f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(Frag, a[0]), __builtin_bit_cast(Frag, b[0]), c,
                                                    0, 0, 0);
  }
};

struct OpFP8 {
  static constexpr int ELEM = 1, KI = 64, FC = 2, OE = 4;
  static constexpr bool SCALED = false, MX = false;
  typedef i32x8 Frag;
  // 32 bytes of k per lane, read as two 16-byte (swizzled) chunks.
  __device__ static Frag frag(const char* base, const uint32_t* off) {
    const i32x4 lo = *(const i32x4*)(base + off[0]);
    const i32x4 hi = *(const i32x4*)(base + off[1]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // Formats 0/0 = E4M3 for both operands.  Scale operands 0: the compiler
  // then emits the unscaled v_mfma_f32_32x32x64_f8f6f4 (the plain product;
  // measured bit-identical to unit E8M0 scales, 127, on random E4M3 data)
  // instead of the scaled form with its extra scale dword.
  __device__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
  __device__ static f32x16 mma_parts(const u32x4 (&a)[2], const u32x4 (&b)[2], f32x16 c) {
    const i32x8 av = __builtin_shufflevector(__builtin_bit_cast(i32x4, a[0]), __builtin_bit_cast(i32x4, a[1]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
    const i32x8 bv = __builtin_shufflevector(__builtin_bit_cast(i32x4, b[0]), __builtin_bit_cast(i32x4, b[1]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
    return mma(av, bv, c);
  }
  // The 16 x 16 x 128 MFMA (the four-wave kernel): lane l holds row l % 16
  // of A and column l % 16 of B, each with 32 bytes of k (lanes 16g .. 16g +
  // 15 the same k); D holds rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.
  __device__ static f32x4 mma16(const u32x4 (&a)[2], const u32x4 (&b)[2], f32x4 c) {
    const i32x8 av = __builtin_shufflevector(__builtin_bit_cast(i32x4, a[0]), __builtin_bit_cast(i32x4, a[1]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
    const i32x8 bv = __builtin_shufflevector(__builtin_bit_cast(i32x4, b[0]), __builtin_bit_cast(i32x4, b[1]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
    // Unscaled form, as mma above (v_mfma_f32_16x16x128_f8f6f4).
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  }
};

// FP8 with per-tensor or per-row scale factors: the same MFMAs, with the
// FP32 accumulators scaled before the store ("FP8 GEMM Optimization on AMD
// RDNA 4", section "What Changes at FP8": the factors a quantized kernel
// carries are applied after the accumulation).
struct OpFP8S : OpFP8 {
  static constexpr bool SCALED = true;
};

// MXFP8: E4M3 operands with one E8M0 scale (2^(e - 127)) per 32 consecutive
// k of each row of A and each column of B, as the block scales of the
// scaled MFMA take them.
struct OpMX8 : OpFP8 {
  static constexpr bool MX = true;
  // 16 x 16 x 128 with block scales.  Lane group L = l / 16 holds bytes 0-15
  // and 16-31 of its row; the instruction's four blocks of 32 k are {groups
  // 0, 1} x bytes 0-15, {2, 3} x bytes 0-15, {0, 1} x bytes 16-31 and {2, 3} x
  // bytes 16-31, and the scale of block L comes from lane group L (byte 0 of
  // its scale register here).  Loading chunk L into bytes 0-15 and chunk L + 4
  // into bytes 16-31 (16 k each) makes block L the L-th 32 k of the stage.
  // (Determined on gfx950 with one-hot operands and one scaled lane at a
  // time, for A and for B.)
  __device__ static f32x4 mma16_mx(const u32x4 (&a)[2], const u32x4 (&b)[2], f32x4 c, uint32_t sa, uint32_t sb) {
    const i32x8 av = __builtin_shufflevector(__builtin_bit_cast(i32x4, a[0]), __builtin_bit_cast(i32x4, a[1]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
    const i32x8 bv = __builtin_shufflevector(__builtin_bit_cast(i32x4, b[0]), __builtin_bit_cast(i32x4, b[1]), 0, 1,
                                             2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, (int)sa, 0, (int)sb);
  }
};

// Zero the bytes of a 16-byte chunk at and beyond `valid_bytes` (0..16).
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int valid_bytes) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int vb = valid_bytes - 4 * d;
    const uint32_t m = vb >= 4 ? 0xffffffffu : (vb <= 0 ? 0u : ((1u << (8 * vb)) - 1u));
    v[d] &= m;
  }
  return v;
}

// Store D[p..p+3][q] (four consecutive p of one accumulator column) at
// C[q*ldc + p], converted to the output format with round-to-nearest-even.
// One 8- or 16-byte store when C allows it, element stores at the p edge.
template <class Op>
__device__ __forceinline__ void store4(const GemmArgs& a, int64_t q, int64_t p, float v0, float v1, float v2,
                                       float v3) {
  if constexpr (Op::OE == 4) {
    float* c = (float*)a.C + q * a.ldc + p;
    if (a.vec_store && p + 3 < a.Pn) {
      *(f32x4*)c = f32x4{v0, v1, v2, v3};
    } else {
      if (p + 0 < a.Pn) c[0] = v0;
      if (p + 1 < a.Pn) c[1] = v1;
      if (p + 2 < a.Pn) c[2] = v2;
      if (p + 3 < a.Pn) c[3] = v3;
    }
  } else {
    uint16_t* c = (uint16_t*)a.C + q * a.ldc + p;
    if (a.vec_store && p + 3 < a.Pn) {
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      *(u32x2*)c = u32x2{Op::pack2(v0, v1), Op::pack2(v2, v3)};
    } else {
      if (p + 0 < a.Pn) c[0] = Op::one(v0);
      if (p + 1 < a.Pn) c[1] = Op::one(v1);
      if (p + 2 < a.Pn) c[2] = Op::one(v2);
      if (p + 3 < a.Pn) c[3] = Op::one(v3);
    }
  }
}

// Scale factors of one wave's tile (FP8 scaled entry point), applied as the
// accumulators are converted: D[p][q] = acc * (sp(p) * sq(q)), each product
// rounded to FP32, where sp(p) = a.sp[p] (a.sp_row) or a.sp[0], and likewise
// sq.  Lane l stores q = qbase + MT j + l % MT (MT the MFMA tile), whose
// factors it holds for the whole epilogue, and groups of four consecutive p,
// whose factors it fetches per group.  Per-row factors are read through
// buffer descriptors sized to the vectors, so a p or q past the edge reads 0
// (never stored).
template <int TQ, int MT = 32>
struct EpiScale {
  float fq[TQ];
  __device__ void init(const GemmArgs& a, int lane, int64_t qbase) {
    if (a.sq_row) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.sq, (uint32_t)(a.Qn * 4));
#pragma unroll
      for (int j = 0; j < TQ; ++j)
        fq[j] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rq, (int)((qbase + MT * j + lane % MT) * 4), 0, 0));
    } else {
      const float f = a.sq[0];
#pragma unroll
      for (int j = 0; j < TQ; ++j) fq[j] = f;
    }
  }
  __device__ static f32x4 p4(const GemmArgs& a, int64_t p) {
    if (!a.sp_row) {
      const float f = a.sp[0];
      return f32x4{f, f, f, f};
    }
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.sp, (uint32_t)(a.Pn * 4));
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (int)((p + e) * 4), 0, 0));
    return r;
  }
  __device__ void apply(const f32x4& fp, int j, float& v0, float& v1, float& v2, float& v3) const {
    v0 *= fp[0] * fq[j];
    v1 *= fp[1] * fq[j];
    v2 *= fp[2] * fq[j];
    v3 *= fp[3] * fq[j];
  }
};

// Epilogue D[p][q] -> C[q*ldc + p] for one wave's WTP x WTQ tile, staged
// through LDS.  Each lane holds four consecutive p of one q per accumulator
// group, so a direct store writes 8 or 16 bytes into each of 32 (16)
// different columns of C.  Instead the wave converts its tile into its own
// LDS region `reg` (WTQ rows of 256 bytes, [q][p]) and reads it back as
// 16-byte chunks: one store instruction then covers four columns with 256
// contiguous bytes each ("An Educational GEMM Ladder for Helios GPUs", the
// LDS-staged epilogue).  Slots of four p are XOR-swizzled by the row so that
// both the scattered writes and the row-wise reads are free of bank
// conflicts.  FP32 output needs twice the space and goes in two passes over
// p.  The caller makes sure no other wave still uses `reg`.
//
// MT is the MFMA tile: 32 x 32 accumulators (lane l: q = 32 j + l % 32,
// p = 32 i + 8 g + 4 (l / 32) + 0..3 for register group g) or 16 x 16
// (lane l: q = 16 j + l % 16, p = 16 i + 4 (l / 16) + 0..3).  With 16 x 16
// one write instruction covers 16 rows and four slots of each, keyed by
// row mod 16 (measured: SQ_LDS_BANK_CONFLICT 0; the even key 2 (row mod 16),
// which keeps 8-byte slot pairs in place, left 4 conflict cycles per write).
template <class Op, int WTP, int WTQ, int TP, int TQ, int MT = 32, class AccT = f32x16>
__device__ __forceinline__ void staged_epilogue(const GemmArgs& a, char* reg, const AccT (&acc)[TP][TQ], int lane,
                                                int64_t pbase, int64_t qbase) {
  constexpr int OE = Op::OE;
  constexpr int PASSES = OE == 4 ? 2 : 1;
  constexpr int TPP = TP / PASSES;            // accumulator tiles along p per pass
  constexpr int RB = TPP * MT * OE;           // bytes of one staged row (one q)
  constexpr int SS = 4 * OE;                  // bytes of one slot (four p)
  constexpr int NSL = RB / SS;                // slots per row
  constexpr int EPC = 16 / OE;                // elements per 16-byte chunk
  constexpr int NG = MT * MT / 256;           // register groups of four per accumulator tile
  static_assert(RB == 256, "staged rows are 256 bytes");
  static_assert(WTQ % 4 == 0, "four rows per read-back instruction");
  auto key = [](int row) { return MT == 32 ? row % NSL : row % 16; };
  const int lr = lane % MT, lg = lane / MT;
  [[maybe_unused]] EpiScale<TQ, MT> sc;
  if constexpr (Op::SCALED) sc.init(a, lane, qbase);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
    for (int i = 0; i < TPP; ++i)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        [[maybe_unused]] f32x4 fp;
        if constexpr (Op::SCALED) fp = EpiScale<TQ, MT>::p4(a, pbase + MT * (pass * TPP + i) + 8 * g + 4 * lg);
#pragma unroll
        for (int j = 0; j < TQ; ++j) {
          const AccT& v = acc[pass * TPP + i][j];
          float v0 = v[4 * g], v1 = v[4 * g + 1], v2 = v[4 * g + 2], v3 = v[4 * g + 3];
          // 16 x 16: through vector registers (see the direct epilogue of
          // the four-wave kernel).
          if constexpr (MT == 16) asm("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
          if constexpr (Op::SCALED) sc.apply(fp, j, v0, v1, v2, v3);
          const int row = MT * j + lr;
          // slot of p = MT i + 8 g + 4 lg (32 x 32) or MT i + 4 lg (16 x 16)
          const int slot = ((MT / 4) * i + 2 * g + lg) ^ key(row);
          char* dst = reg + row * RB + slot * SS;
          if constexpr (OE == 4) {
            *(f32x4*)dst = f32x4{v0, v1, v2, v3};
          } else {
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            *(u32x2*)dst = u32x2{Op::pack2(v0, v1), Op::pack2(v2, v3)};
          }
        }
      }
    const int m = lane & 15;                  // 16-byte chunk within a row
#pragma unroll
    for (int it = 0; it < WTQ / 4; ++it) {
      const int row = 4 * it + (lane >> 4);
      const int kr = key(row);
      u32x4 d;
      if constexpr (OE == 4) {
        d = *(const u32x4*)(reg + row * RB + ((m ^ kr) * 16));
      } else {
        // Chunk m holds slots 2m and 2m+1, which the swizzle keeps in one
        // aligned pair but swaps when the key is odd.
        const u32x4 raw = *(const u32x4*)(reg + row * RB + ((((2 * m) ^ kr) & ~1) * SS));
        d = (kr & 1) ? u32x4{raw[2], raw[3], raw[0], raw[1]} : raw;
      }
      const int64_t q = qbase + row;
      const int64_t p0 = pbase + pass * TPP * MT;   // first p of the staged row
      const int64_t p = p0 + m * EPC;
      if (q >= a.Qn) continue;
      char* c = (char*)a.C + (q * a.ldc + p) * OE;
      if (a.vec16 && p + EPC <= a.Pn) {
        *(u32x4*)c = d;
        continue;
      }
      if constexpr (OE == 2) {
        // The row's 256 bytes of C start off the 16-byte grid (odd ldc or
        // C not 16-byte aligned), delta bytes past a boundary.  Whole rows
        // are stored as the aligned 16-byte blocks that cover them: lane m
        // (m < 15) stores block m + 1, which starts at row byte
        // 16 (m + 1) - delta and is gathered from the staged row as five
        // dwords shifted by (16 (m + 1) - delta) mod 4 bytes; lane 15 stores
        // the partial blocks at both ends element by element.  Rows that
        // end at the p edge keep the element-wise stores below.
        const char* rowc = (const char*)a.C + (q * a.ldc + p0) * 2;
        const int delta = (int)((uintptr_t)rowc & 15);
        if (p0 + RB / 2 <= a.Pn && delta != 0) {
          auto dword_at = [&](int b) {   // dword at logical byte b (4-aligned) of the staged row
            return *(const uint32_t*)(reg + row * RB + ((((b >> 3) ^ kr) << 3) | (b & 7)));
          };
          if (m < 15) {
            const int b0 = 16 * (m + 1) - delta;
            const int bw = b0 & ~3, sh = b0 & 3;
            uint32_t w[5];
#pragma unroll
            for (int k = 0; k < 5; ++k) w[k] = dword_at(bw + 4 * k);
            u32x4 blk;
#pragma unroll
            for (int k = 0; k < 4; ++k) blk[k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], (unsigned)sh);
            *(u32x4*)(rowc + b0) = blk;
          } else {
            auto elem_at = [&](int e) {
              return (uint16_t)(dword_at((2 * e) & ~3) >> ((e & 1) * 16));
            };
            const int head = (16 - delta) / 2, tail = delta / 2;   // elements
            for (int e = 0; e < head; ++e) ((uint16_t*)rowc)[e] = elem_at(e);
            for (int e = RB / 2 - tail; e < RB / 2; ++e) ((uint16_t*)rowc)[e] = elem_at(e);
          }
          continue;
        }
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (p + e < a.Pn) {
          if constexpr (OE == 4) ((uint32_t*)c)[e] = d[e];
          else ((uint16_t*)c)[e] = (uint16_t)(d[e >> 1] >> ((e & 1) * 16));
        }
      }
    }
  }
}

// ---- the kernel ---------------------------------------------------------------

template <class Op, int BP, int BQ, int WP, int WQ, bool P_TRANS>
struct MfmaCfg {
  static constexpr int NT = WP * WQ * 64;
  static constexpr int E = Op::ELEM;
  static constexpr int ROWB = 128;            // bytes of k per LDS row per stage
  static constexpr int BK = ROWB / E;         // k per stage
  static constexpr int CPE = 16 / E;          // elements per 16-byte chunk
  static constexpr int P_LDS = BP * ROWB;
  static constexpr int Q_LDS = BQ * ROWB;
  static constexpr int STAGE = P_LDS + Q_LDS;
  static constexpr int PCH = BP * (ROWB / 16) / NT;  // P chunks per thread per stage (staged path)
  static constexpr int WTP = BP / WP, WTQ = BQ / WQ;
  static constexpr int TP = WTP / 32, TQ = WTQ / 32;
  static constexpr int KSTEPS = BK / Op::KI;
  static constexpr int PT_CPR = BP * E / 16;  // chunks per k-row of a p-contiguous P tile
  static_assert(NT % 8 == 0, "thread count");
  static_assert(BP * 8 % NT == 0 && BQ * 8 % NT == 0, "chunks divide over threads");
  static_assert(WTP % 32 == 0 && WTQ % 32 == 0, "wave tile is whole 32x32 MFMA tiles");
  static_assert(lds_bytes(BP, BQ, BK, E, 0, 2) <= kLdsLimit, "LDS budget");
  static_assert(!P_TRANS || (BP * E) % 16 == 0, "p-contiguous chunks");
};

// Waves per SIMD the kernel is compiled for: 8-wave blocks run two waves on
// each SIMD (256 registers each); 4-wave blocks run one and may use all 512.
template <int WAVES>
constexpr int waves_per_simd() { return WAVES >= 8 ? 2 : 1; }

template <class Op, int BP, int BQ, int WP, int WQ, bool P_TRANS>
__global__ void __launch_bounds__(WP * WQ * 64)
__attribute__((amdgpu_waves_per_eu(waves_per_simd<WP * WQ>(), waves_per_simd<WP * WQ>())))
gemm_mfma_kernel(const GemmArgs a) {
  using Cfg = MfmaCfg<Op, BP, BQ, WP, WQ, P_TRANS>;
  constexpr int NT = Cfg::NT, E = Cfg::E, ROWB = Cfg::ROWB, BK = Cfg::BK, CPE = Cfg::CPE;
  constexpr int PCH = Cfg::PCH, TP = Cfg::TP, TQ = Cfg::TQ, FC = Op::FC;

  __shared__ __attribute__((aligned(1024))) char smem[2 * Cfg::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wp = wave / WQ, wq = wave % WQ;

  int64_t tp, tq;
  tile_map(a.tiles_p, a.tiles_q, a.group, blockIdx.x, &tp, &tq);
  const int64_t p0 = tp * BP, q0 = tq * BQ;
  const int64_t K = a.K;
  const int nst = (int)((K + BK - 1) / BK);
  const uint32_t kbytes16 = (uint32_t)(((K * E) + 15) & ~(int64_t)15);

  // ---- loaders ----
  // K-contiguous tiles are copied global -> LDS directly (buffer_load ... lds,
  // 16 bytes per lane on gfx950), so no registers stage them and no LDS store
  // instructions are issued.  One wave instruction fills one 1 KiB LDS
  // segment = 8 tile rows: lane l lands at byte 16*l, i.e. row 8*seg + l/8,
  // physical chunk l%8.  That slot holds logical k-chunk (l%8) ^ key(row), so
  // the swizzle is applied to the global address each lane fetches.  With
  // row = 8*seg + l/8 and seg = i*NW + wave, key(row) = (row/2) mod 8 =
  // (4*(wave%2) + l/16) mod 8 for every i (NW even).
  constexpr int NW = NT / 64;
  static_assert(NW % 2 == 0, "segment parity must follow the wave index");
  constexpr int QSEG = BQ / 8 / NW;              // LDS segments per wave per stage
  constexpr int PSEG = BP / 8 / NW;
  static_assert(BQ % (8 * NW) == 0 && BP % (8 * NW) == 0, "segments divide over waves");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int seg_row = lane >> 3;
  const int dkc = (lane & 7) ^ ((4 * (wave_u & 1) + (lane >> 4)) & 7);
  const int64_t dkst0 = (int64_t)dkc * CPE;      // first k of this lane's chunk within a stage
  const int dkst0_32 = dkc * CPE;

  const char* qblk = a.Q + q0 * a.ldq;
  const int64_t qrows = (a.Qn - q0) < BQ ? (a.Qn - q0) : BQ;
  const uint32_t qnrec = (uint32_t)((qrows - 1) * a.ldq) + kbytes16;
  uint32_t qvo[QSEG];
#pragma unroll
  for (int i = 0; i < QSEG; ++i) {
    const int row = 8 * (i * NW + wave_u) + seg_row;
    qvo[i] = (row < qrows) ? (uint32_t)(row * a.ldq + dkc * 16) : kOobOffset;
  }

  // P: direct like Q, or (NN's B) p-contiguous rows staged through registers
  // and transposed element by element into the K-contiguous LDS layout.
  const char* pblk;
  uint32_t pnrec;
  uint32_t pvo[P_TRANS ? PCH : PSEG];
  if constexpr (!P_TRANS) {
    pblk = a.P + p0 * a.ldp;
    const int64_t prows = (a.Pn - p0) < BP ? (a.Pn - p0) : BP;
    pnrec = (uint32_t)((prows - 1) * a.ldp) + kbytes16;
#pragma unroll
    for (int i = 0; i < PSEG; ++i) {
      const int row = 8 * (i * NW + wave_u) + seg_row;
      pvo[i] = (row < prows) ? (uint32_t)(row * a.ldp + dkc * 16) : kOobOffset;
    }
  } else {
    // chunk c = i*NT + tid -> k-row c / PT_CPR, p-chunk c % PT_CPR.
    pblk = a.P + p0 * E;
    const int64_t pcols = (a.Pn - p0) < BP ? (a.Pn - p0) : BP;
    pnrec = (uint32_t)((K - 1) * a.ldp) + (uint32_t)(((pcols * E) + 15) & ~(int64_t)15);
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int c = i * NT + tid;
      const int krow = c / Cfg::PT_CPR, pc = c % Cfg::PT_CPR;
      pvo[i] = (pc * CPE < pcols) ? (uint32_t)(krow * a.ldp + pc * 16) : kOobOffset;
    }
  }
  u32x4 pst[P_TRANS ? PCH : 1];

  // Issue the direct copies of one K-contiguous tile for stage s.  In the last
  // stage, chunks that start at or past K are forced out of range (zeros).
  auto direct_tile = [&](const char* blk, uint32_t nrec, const uint32_t* vo, int nseg, char* lds_tile, int s,
                         bool tail) {
    const uint32_t adv = (uint32_t)s * ROWB;
    // (readfirstlane keeps the clamped count in a scalar register: a vector
    // select here would force a per-lane loop around every copy.)
    const uint32_t left = (uint32_t)__builtin_amdgcn_readfirstlane((int)(adv < nrec ? nrec - adv : 0u));
    const __amdgpu_buffer_rsrc_t r = make_rsrc(blk + adv, left);
    // Chunks starting at or past K read zero: setting bit 31 puts the offset
    // beyond num_records (< 2^31) without a branch.  Stages past the last one
    // (issued by the pipeline below to keep its loop branch-free) read zero
    // throughout.
    const int64_t rem64 = K - (int64_t)s * BK;
    const int rem = (int)(rem64 < BK ? rem64 : BK);   // k left from this stage's start, at most BK
    const uint32_t kill = (tail && dkst0_32 >= rem) ? kOobOffset : 0u;
#pragma unroll
    for (int i = 0; i < nseg; ++i) {
      const uint32_t off = vo[i] | kill;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds_tile + (i * NW + wave_u) * 1024), 16, off, 0, 0, 0);
    }
  };
  // After the copies have landed: zero the k >= K part of a chunk that
  // straddles K (only when K is not a multiple of the chunk width).
  auto fix_tail = [&](char* lds_tile, int nseg, int s) {
    const int64_t kst = (int64_t)s * BK + dkst0;
    if (kst < K && kst + CPE > K) {
#pragma unroll
      for (int i = 0; i < nseg; ++i) {
        u32x4* c = (u32x4*)(lds_tile + (i * NW + wave_u) * 1024 + lane * 16);
        *c = mask_tail(*c, (int)((K - kst) * E));
      }
    }
  };

  auto load_stage = [&](int s, auto tail_tag) {
    constexpr bool tail = decltype(tail_tag)::value;
    char* sb = smem + (s & 1) * Cfg::STAGE;
    direct_tile(qblk, qnrec, qvo, QSEG, sb + Cfg::P_LDS, s, tail);
    if constexpr (!P_TRANS) {
      direct_tile(pblk, pnrec, pvo, PSEG, sb, s, tail);
    } else {
      const uint32_t adv = (uint32_t)((int64_t)s * BK * a.ldp);
      const __amdgpu_buffer_rsrc_t r = make_rsrc(pblk + (int64_t)s * BK * a.ldp, pnrec - adv);
#pragma unroll
      for (int i = 0; i < PCH; ++i) {
        uint32_t off = pvo[i];
        const int krow = (i * NT + tid) / Cfg::PT_CPR;
        if (tail && (int64_t)s * BK + krow >= K) off = kOobOffset;
        pst[i] = load16(r, off);
      }
    }
  };

  // Completes stage s's copies: register-staged data is written (transposed),
  // the direct copies are waited for, and the K tail is trimmed.  The caller
  // follows with a barrier.
  auto finish_stage = [&](int s, auto tail_tag) {
    constexpr bool tail = decltype(tail_tag)::value;
    char* sb = smem + (s & 1) * Cfg::STAGE;
    if constexpr (P_TRANS) {
#pragma unroll
      for (int i = 0; i < PCH; ++i) {
        const int c = i * NT + tid;
        const int krow = c / Cfg::PT_CPR, pc = c % Cfg::PT_CPR;
        const int kchunk = krow / CPE, kin = (krow % CPE) * E;
#pragma unroll
        for (int e = 0; e < CPE; ++e) {
          const int p = pc * CPE + e;
          char* dst = sb + p * ROWB + ((kchunk ^ ((p >> 1) & 7)) << 4) + kin;
          const uint32_t w = pst[i][(e * E) >> 2];
          if constexpr (E == 2) *(uint16_t*)dst = (uint16_t)(w >> (((e * E) & 3) * 8));
          else *(uint8_t*)dst = (uint8_t)(w >> (((e * E) & 3) * 8));
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if constexpr (tail) {
      if (K % CPE != 0) {
        fix_tail(sb + Cfg::P_LDS, QSEG, s);
        if constexpr (!P_TRANS) fix_tail(sb, PSEG, s);
      }
    }
  };

  // ---- fragment addressing ----
  const int l32 = lane & 31, h = lane >> 5;
  const int sw_r = (l32 >> 1) & 7;                 // swizzle key of every fragment row of this lane
  const uint32_t pf_base = (uint32_t)((wp * Cfg::WTP + l32) * ROWB);
  const uint32_t qf_base = (uint32_t)(Cfg::P_LDS + (wq * Cfg::WTQ + l32) * ROWB);

  f32x16 acc[TP][TQ];
#pragma unroll
  for (int i = 0; i < TP; ++i)
#pragma unroll
    for (int j = 0; j < TQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One stage of MFMAs.  Fragments for k-step kk+1 are read from LDS while
  // the MFMAs of k-step kk run (two register sets), and the scheduling
  // groups interleave one LDS read after each MFMA so the reads' latency
  // hides under matrix work instead of stalling the wave.
  typedef typename Op::Frag Frag;
  auto read_frags = [&](const char* sb, int kk, Frag (&af)[TP], Frag (&bf)[TQ]) {
    uint32_t off[FC];
#pragma unroll
    for (int f = 0; f < FC; ++f) off[f] = (uint32_t)((((kk * 2 + h) * FC + f) ^ sw_r) << 4);
#pragma unroll
    for (int j = 0; j < TQ; ++j) bf[j] = Op::frag(sb + qf_base + j * 32 * ROWB, off);
#pragma unroll
    for (int i = 0; i < TP; ++i) af[i] = Op::frag(sb + pf_base + i * 32 * ROWB, off);
  };
  constexpr int NREAD = (TP + TQ) * FC;      // ds_read_b128 per k-step
  constexpr int NMFMA = TP * TQ;             // MFMAs per k-step
  auto compute_stage = [&](int buf) {
    const char* sb = smem + buf * Cfg::STAGE;
    Frag af[2][TP], bf[2][TQ];
    read_frags(sb, 0, af[0], bf[0]);
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < Cfg::KSTEPS) read_frags(sb, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < TP; ++i)
#pragma unroll
        for (int j = 0; j < TQ; ++j) acc[i][j] = Op::mma(af[cur][i], bf[cur][j], acc[i][j]);
    }
    // Order: the first k-step's reads, then per k-step its MFMAs with the
    // next k-step's reads threaded between them.
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
      if (kk + 1 < Cfg::KSTEPS) {
#pragma unroll
        for (int t = 0; t < NMFMA; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (t < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
      }
    }
  };

  // ---- pipeline (K-contiguous P: both tiles copied directly) ----
  // Stage s is computed from LDS buffer s % 2.  The one barrier per stage sits
  // before the stage's last k-step: by then every wave holds that k-step's
  // fragments in registers (so buffer s % 2 is free) and has waited for its
  // own copies of stage s + 1.  After the barrier the wave reads stage s + 1's
  // first fragments and starts copying stage s + 2 into buffer s % 2 while the
  // last k-step's MFMAs run, so no MFMA waits on an LDS read at a stage
  // boundary.
  //
  // The instruction order is spelled out slot by slot (one MFMA, then the LDS
  // reads and copies assigned to that slot) and pinned with scheduling
  // fences: copies issued in a burst fill the texture unit's queue and stall
  // the issuing wave, MFMAs included, so they are spread one per MFMA slot.
  if constexpr (!P_TRANS) {
    constexpr int NDMA = QSEG + PSEG;          // copy instructions per wave per stage
    static_assert(NDMA <= 31, "vmcnt range");
    const bool ragged = (K % CPE) != 0;
    // Copies of one tile for stage t: a descriptor advanced to the stage, and
    // a kill bit for chunks at or past K (bit 31 puts the offset beyond
    // num_records < 2^31, so the lane reads zero without a branch).  Stages
    // past the last one read zero throughout.
    auto copy_rsrc = [&](const char* blk, uint32_t nrec, int t) {
      const uint32_t adv = (uint32_t)t * ROWB;
      // (readfirstlane keeps the clamped count in a scalar register: a
      // vector select here would force a per-lane loop around every copy.)
      const uint32_t left = (uint32_t)__builtin_amdgcn_readfirstlane((int)(adv < nrec ? nrec - adv : 0u));
      return make_rsrc(blk + adv, left);
    };
    auto copy_kill = [&](int t) {
      const int64_t rem64 = K - (int64_t)t * BK;
      const int rem = (int)(rem64 < BK ? rem64 : BK);
      return dkst0_32 >= rem ? kOobOffset : 0u;
    };
    auto copy_one = [&](__amdgpu_buffer_rsrc_t r, uint32_t kill, const uint32_t* vo, char* lds_tile, int i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds_tile + (i * NW + wave_u) * 1024), 16, vo[i] | kill, 0, 0,
          0);
    };
    // Copy instruction d of a stage: Q segments first, then P segments.
    auto copy_d = [&](__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rp, uint32_t kill, char* stage_lds, int d) {
      if (d < QSEG) copy_one(rq, kill, qvo, stage_lds + Cfg::P_LDS, d);
      else copy_one(rp, kill, pvo, stage_lds, d - QSEG);
    };
    auto trim = [&](int t, int b) {
      char* sb = smem + b * Cfg::STAGE;
      fix_tail(sb + Cfg::P_LDS, QSEG, t);
      fix_tail(sb, PSEG, t);
    };
    // Fragments as 16-byte parts: [set][tile][part].
    u32x4 fa[2][TP][FC], fb[2][TQ][FC];
    // LDS read r of a k-step: B tiles first, then A tiles, FC parts each.
    auto read_one = [&](const char* sb, int kk, int set, int r) {
      const bool isb = r < TQ * FC;
      const int rr = isb ? r : r - TQ * FC;
      const int tile = rr / FC, f = rr % FC;
      const uint32_t off = (uint32_t)((((kk * 2 + h) * FC + f) ^ sw_r) << 4);
      const char* base = sb + (isb ? qf_base + tile * 32 * ROWB : pf_base + tile * 32 * ROWB);
      const u32x4 v = *(const u32x4*)(base + off);
      if (isb) fb[set][tile][f] = v; else fa[set][tile][f] = v;
    };
    auto mfma_one = [&](int set, int t) {
      const int i = t / TQ, j = t % TQ;
      acc[i][j] = Op::mma_parts(fa[set][i], fb[set][j], acc[i][j]);
    };
    // Slot of read r when NREAD reads are spread over `span` MFMA slots.
    auto read_slot = [](int r, int span) { return r * span / NREAD; };
    constexpr int LAST = (Cfg::KSTEPS - 1) & 1;        // fragment set of the last k-step
    // Two stages per loop trip (fixed buffer offsets) where the registers
    // allow it; FP8's 32-byte fragments leave no room for the extra
    // loop-invariant addresses, so it selects the buffer at run time.
    constexpr bool UNROLL2 = Op::FC == 1;
    // B is the buffer index when it is known at compile time (-1: s % 2).
    auto stage = [&](int s, auto buf) {
      constexpr int B = decltype(buf)::value;
      const int b = B >= 0 ? B : (s & 1);
      const char* sb = smem + b * Cfg::STAGE;
      // A ragged last stage is trimmed in LDS by each wave once its own
      // copies have landed (once per tile, and only when K is not a multiple
      // of the chunk width; the barrier below publishes it).  The branch sits
      // ahead of the MFMAs so they stay in one block with the barrier.
      if (ragged && s + 2 == nst) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        trim(s + 1, b ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // k-steps before the barrier; the reads feeding the last of them are
      // packed into the first half of their slots so they complete before it.
#pragma unroll
      for (int kk = 0; kk + 1 < Cfg::KSTEPS; ++kk) {
        const int span = kk + 2 == Cfg::KSTEPS ? NMFMA / 2 : NMFMA;
#pragma unroll
        for (int t = 0; t < NMFMA; ++t) {
          mfma_one(kk & 1, t);
#pragma unroll
          for (int r = 0; r < NREAD; ++r)
            if (read_slot(r, span) == t) read_one(sb, kk + 1, (kk + 1) & 1, r);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      // Last k-step: next stage's first fragments, copies of stage s + 2.
      const char* nb = smem + (b ^ 1) * Cfg::STAGE;
      char* db = smem + b * Cfg::STAGE;
      const __amdgpu_buffer_rsrc_t rq = copy_rsrc(qblk, qnrec, s + 2), rp = copy_rsrc(pblk, pnrec, s + 2);
      const uint32_t kill = copy_kill(s + 2);
#pragma unroll
      for (int t = 0; t < NMFMA; ++t) {
        mfma_one(LAST, t);
#pragma unroll
        for (int r = 0; r < NREAD; ++r)
          if (read_slot(r, NMFMA) == t) read_one(nb, 0, 0, r);
#pragma unroll
        for (int d = 0; d < NDMA; ++d)
          if (d * NMFMA / NDMA == t) copy_d(rq, rp, kill, db, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (nst > 0) {
      {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const __amdgpu_buffer_rsrc_t rq = copy_rsrc(qblk, qnrec, t), rp = copy_rsrc(pblk, pnrec, t);
          const uint32_t kill = copy_kill(t);
#pragma unroll
          for (int d = 0; d < NDMA; ++d) copy_d(rq, rp, kill, smem + t * Cfg::STAGE, d);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcntBase | vmcnt_bits(NDMA));
      if (ragged && nst == 1) trim(0, 0);
      __syncthreads();
#pragma unroll
      for (int r = 0; r < NREAD; ++r) read_one(smem, 0, 0, r);
      if constexpr (UNROLL2) {
        int s = 0;
        for (; s + 1 < nst; s += 2) {
          stage(s, std::integral_constant<int, 0>{});
          stage(s + 1, std::integral_constant<int, 1>{});
        }
        if (s < nst) stage(s, std::integral_constant<int, 0>{});
      } else {
        for (int s = 0; s < nst; ++s) stage(s, std::integral_constant<int, -1>{});
      }
      // Copies of the two stages past the end are still in flight.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
  } else if (nst > 0) {
    if (nst == 1) { load_stage(0, std::true_type{}); finish_stage(0, std::true_type{}); }
    else { load_stage(0, std::false_type{}); finish_stage(0, std::false_type{}); }
    __syncthreads();
    int s = 0;
    for (; s < nst - 2; ++s) {
      load_stage(s + 1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(s & 1);
      __builtin_amdgcn_sched_barrier(0);
      finish_stage(s + 1, std::false_type{});
      __syncthreads();
    }
    if (s < nst - 1) {
      load_stage(s + 1, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(s & 1);
      __builtin_amdgcn_sched_barrier(0);
      finish_stage(s + 1, std::true_type{});
      __syncthreads();
      ++s;
    }
    compute_stage(s & 1);
  }

  // ---- epilogue ----
  {
    static_assert(Cfg::WTQ * 256 * NW <= 2 * Cfg::STAGE, "staging fits in the stage buffers");
    // Every copy has landed and every wave is done with the stage buffers.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    staged_epilogue<Op, Cfg::WTP, Cfg::WTQ, TP, TQ>(a, smem + wave_u * (Cfg::WTQ * 256), acc, lane,
                                                     p0 + wp * Cfg::WTP, q0 + wq * Cfg::WTQ);
  }
}

}  // namespace dg
