// The dequant-fused small-row GEMM of one column group, as a device
// function shared by the GEMM kernel (one workgroup per column group) and the
// fused layer kernel, with the helpers both use.  See sv_gemm.hip for the
// design.
#pragma once
#include "sv_device.h"
#include "sv_epi.h"
#include "sv_internal.h"
#include "sv_timeline.h"

namespace {

typedef sv_rsrc rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return sv_make_rsrc(p, bytes);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same load marked non-temporal (streaming: its lines are the first the
// caches give up).
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// A 32-bit constant held in a vector register, so that (x & literal) | c can
// be one v_and_or_b32 (an instruction may read only one literal).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// Eight 4-bit codes (slot s at bit 4*(s/2) + 16*(s%2)) to fp16 operands.
// Codes at bits 0..3 of a half are read under the exponent of 1024 (value
// 1024 + q), codes at bits 4..7 under that of 64 (value 64 + q: one unit of
// mantissa bit 4 is 1 there), so both take the same multiplier m and only
// the offsets differ: pair p is (1024 + q) * m + a0 (p even) or
// (64 + q) * m + a1 (p odd).
__device__ __forceinline__ half8 deq4(uint32_t w, uint32_t mg, uint32_t mg64, half2v m,
                                      half2v a0, half2v a1) {
  const uint32_t w8 = w >> 8;
  const half2v h0 = fma_h2(as_h2((w & 0x000F000Fu) | mg), m, a0);
  const half2v h1 = fma_h2(as_h2((w & 0x00F000F0u) | mg64), m, a1);
  const half2v h2 = fma_h2(as_h2((w8 & 0x000F000Fu) | mg), m, a0);
  const half2v h3 = fma_h2(as_h2((w8 & 0x00F000F0u) | mg64), m, a1);
  return make_half8(u32x4{as_u32(h0), as_u32(h1), as_u32(h2), as_u32(h3)});
}

// p * c on both halves, opaque to the compiler: the product is formed once
// per pair of sub-block scales and each k-step picks its half by operand
// selection, instead of one broadcast product per k-step.
__device__ __forceinline__ half2v pk_mul_once(half2v p, uint32_t c) {
  uint32_t r;
  asm("v_pk_mul_f16 %0, %1, %2" : "=v"(r) : "v"(as_u32(p)), "s"(c));
  return as_h2(r);
}

// Six-bit codes minus 32 for one k-step: low nibbles in slot layout, high
// bits (already shifted to the k-step) at 2*(s/2) + 16*(s%2).
__device__ __forceinline__ half8 deq6_t(uint32_t wl, uint32_t wh, uint32_t mg) {
  const half2v c = {(f16)-1056.0f, (f16)-1056.0f};
  const uint32_t wl8 = wl >> 8;
  const uint32_t q0 = ((wl & 0x000F000Fu) | mg) | ((wh & 0x00030003u) << 4);
  const uint32_t q1 = (((wl >> 4) & 0x000F000Fu) | mg) | (((wh >> 2) & 0x00030003u) << 4);
  const uint32_t q2 = ((wl8 & 0x000F000Fu) | mg) | (((wh >> 4) & 0x00030003u) << 4);
  const uint32_t q3 = (((wl8 >> 4) & 0x000F000Fu) | mg) | (((wh >> 6) & 0x00030003u) << 4);
  return make_half8(u32x4{as_u32(as_h2(q0) + c), as_u32(as_h2(q1) + c), as_u32(as_h2(q2) + c),
                          as_u32(as_h2(q3) + c)});
}

__device__ __forceinline__ half2v bcast(half2v p, int hi) {
  return hi ? half2v{p[1], p[1]} : half2v{p[0], p[0]};
}

__device__ __forceinline__ float f16_at(uint32_t w, int half) {
  return (float)__builtin_bit_cast(f16, (uint16_t)((w >> (16 * half)) & 0xFFFFu));
}

// ---- weight operands of one k-step for the column held by this lane --------
// 4-bit super-block format: sc_j * q with the sub-block's 6-bit scale folded
// in (r: the column's 16-byte record, w: the code word of the k-step).  The
// scales come in pairs (k-steps 2i and 2i + 1 share one word of the record);
// (1024 + q) sc - 1024 sc and (64 + q) sc - 64 sc are exact (sc q <= 945).
__device__ __forceinline__ half8 b4s_op(const u32x4 r, uint32_t w, int ks, uint32_t mg,
                                        uint32_t mg64) {
  const half2v k1024 = {(f16)-1024.0f, (f16)-1024.0f};
  const int pi = ks >> 1, hi = ks & 1;
  const uint32_t sw = ((pi < 2) ? r[1] : r[2]) >> ((pi & 1) ? 6 : 0);
  const half2v scp = as_h2((sw & 0x003F003Fu) | mg) + k1024;   // (1024 + sc) - 1024
  const half2v a0p = pk_mul_once(scp, 0xE400E400u);            // -1024 sc
  const half2v a1p = pk_mul_once(scp, 0xD400D400u);            // -64 sc
  return deq4(w, mg, mg64, bcast(scp, hi), bcast(a0p, hi), bcast(a1p, hi));
}

// 4-bit super-block format: the exact 6-bit mins m_j in k slots 0..7 (lane
// group 0), multiplied against the packed sub-block sums of the activation.
__device__ __forceinline__ half8 b4s_min_op(const u32x4 r, uint32_t mg) {
  const half2v k1024 = {(f16)-1024.0f, (f16)-1024.0f};
  const uint32_t mlo = r[3];
  const uint32_t p0 = ((mlo & 0x000F000Fu) | mg) | (((r[1] >> 12) & 0x00030003u) << 4);
  const uint32_t p1 = (((mlo >> 4) & 0x000F000Fu) | mg) | (((r[1] >> 14) & 0x00030003u) << 4);
  const uint32_t p2 = (((mlo >> 8) & 0x000F000Fu) | mg) | (((r[2] >> 12) & 0x00030003u) << 4);
  const uint32_t p3 = (((mlo >> 12) & 0x000F000Fu) | mg) | (((r[2] >> 14) & 0x00030003u) << 4);
  return make_half8(u32x4{as_u32(as_h2(p0) + k1024), as_u32(as_h2(p1) + k1024),
                          as_u32(as_h2(p2) + k1024), as_u32(as_h2(p3) + k1024)});
}

// 4-bit/32 format: q - 8.
__device__ __forceinline__ half8 b432_op(uint32_t w, uint32_t mg, uint32_t mg64) {
  const half2v m = {(f16)1.0f, (f16)1.0f};
  const half2v a0 = {(f16)-1032.0f, (f16)-1032.0f}, a1 = {(f16)-72.0f, (f16)-72.0f};
  return deq4(w, mg, mg64, m, a0, a1);
}

// 6-bit format: sc * (q - 32) as an fp16 high part and its exact remainder.
__device__ __forceinline__ void b6_op(const u32x4 cod[3], const u32x4 r, int ks, int g,
                                      uint32_t mg, half8 &bhi, half8 &blo) {
  const uint32_t wh = cod[2][ks >> 1] >> (8 * (ks & 1));
  const half8 tq = deq6_t(cod[ks >> 2][ks & 3], wh, mg);
  const int j = 2 * ks + (g >> 1);
  const int8_t scs = (int8_t)((r[j >> 2] >> (8 * (j & 3))) & 0xFF);
  const f16 sc = (f16)(float)scs;
  const half8 sv = {sc, sc, sc, sc, sc, sc, sc, sc};
  bhi = tq * sv;
  blo = __builtin_elementwise_fma(tq, sv, -bhi);
}

// x holds in lane group (row of 16 lanes) g the value for tile g % TPW;
// out[t] holds tile t's value in every lane group, with each lane keeping
// its position in the row (the column).  Cross-row swaps: the 32-lane swap
// exchanges rows {2, 3} of one copy with rows {0, 1} of another, the
// 16-lane swap odd rows of one copy with even rows of another.
template <int TPW>
__device__ __forceinline__ void spread_rows(uint32_t x, uint32_t (&out)[TPW]) {
  if constexpr (TPW == 4) {
    const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);   // {0 1 0 1}, {2 3 2 3}
    const auto a = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
    out[0] = a[0];
    out[1] = a[1];
    out[2] = b[0];
    out[3] = b[1];
  } else {
    static_assert(TPW == 2, "tiles per wave");
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);   // rows {0 1 0 1}
    out[0] = a[0];
    out[1] = a[1];
  }
}

// Each lane takes the value of the lane 4 places up in its row of 16 (the
// last 4 lanes of a row take zero): MFMA rows 4..7 move to rows 0..3 and
// 12..15 to 8..11.
__device__ __forceinline__ half8 row_down4(half8 v) {
  u32x4 u = __builtin_bit_cast(u32x4, v), r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u[i], 0x104 /* row_shl:4 */, 0xF, 0xF, true);
  return make_half8(r);
}

// Lanes 0..31 receive the value of lanes 32..63 (and lanes 32..63 that of
// lanes 0..31), through the LDS crossbar.
__device__ __forceinline__ float upper_half_down(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((lane + 32) & 63) << 2,
                                                                __builtin_bit_cast(int, x)));
}

// ---- accumulation steps, written out so that both GEMM kernels round the
// same operations in the same order.  The activation's low part is
// fp16((x - hi) * 2^11), so its products are added as 2^-11 * Tl. --------
__device__ __forceinline__ floatx4 join_hl(floatx4 Th, floatx4 Tl) {
  floatx4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf(SV_LO_INV, Tl[i], Th[i]);
  return r;
}

// acc + d * (Th + 2^-11 Tl)
__device__ __forceinline__ floatx4 upd_d(floatx4 acc, floatx4 Th, floatx4 Tl, float d) {
  const floatx4 h = join_hl(Th, Tl);
  floatx4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf(d, h[i], acc[i]);
  return r;
}

// acc + (d * (Th + 2^-11 Tl) - dmin * (Uh + 2^-11 Ul)): the super-block's
// products scaled by d, less its min term, rounded before the add to the
// running sum.
__device__ __forceinline__ floatx4 upd_b4s(floatx4 acc, floatx4 Th, floatx4 Tl, floatx4 Uh,
                                           floatx4 Ul, float d, float dmin) {
  const floatx4 h = join_hl(Th, Tl), u = join_hl(Uh, Ul);
  floatx4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = d * h[i];
    r[i] = acc[i] + __builtin_fmaf(-dmin, u[i], p);
  }
  return r;
}

}  // namespace

// Up to this many K splits (waves) per column group: a group is one
// workgroup that must fit a CU at two waves per SIMD.
#define SV_MAX_KSPLIT 8

// MTP = number of 16-row M-tiles per launch (1 or 2), or SV_MT_PACK8 /
// SV_MT_PACK4: one M-tile of at most 8 / 4 rows whose activation high parts
// fill MFMA rows 0..7 and low parts rows 8..15 of one operand (super-block
// formats).  Each MFMA row is its own dot product, so one product per k-step
// yields both parts with the same bits as two products over separate
// operands; the two halves of the result meet once per super-block by a lane
// swap.  This halves the activation loads and the products of the small-row
// rounds.
//
// Vector load instructions, more than bytes, bound these kernels: each load
// of a wave passes the CU's in-order address and data path whatever its
// useful bytes.  So a single load brings the records of all the wave's tiles
// (lane group g reads tile g % TPW's), passed to every lane group by
// cross-row swaps, and with SV_MT_PACK4 one load brings two k-steps of the
// activation operand (MFMA rows 4..7 and 12..15, padding for at most 4 rows,
// carry the odd k-step, moved down by a row shift when it is used).  Both are
// for the 4-bit formats; the 6-bit lm_head kernels are bound by vector ALU
// issue, which the swaps would add to.
//
// The body of one column group: grp, the K split `split` of this wave (a
// wave with split >= ksplit, or of a group that is not live, takes part in
// the workgroup's barriers only; a group that is not live stores nothing),
// epilogue threads tid of nthr, LDS at s_dyn (partials, staged rows) and
// s_inv (row norm factors).  FUSED: the first two super-blocks' weights are
// requested, then wait() (a workgroup-wide call) returns once the
// activations this group reads are complete, and only then are they loaded;
// otherwise wait is not called.  COH: the epilogue's outputs are read by other
// workgroups of the same launch (agent-scope stores).
template <int FMT, int TPW, int MTP, int EPI, bool FUSED, bool COH, class Wait>
__device__ __forceinline__ void qgemm_body(const uint8_t *__restrict__ W, int nsb, int ksplit,
                                           int sbps, const uint8_t *__restrict__ ap,
                                           const uint8_t *__restrict__ sx, int M, int mt0,
                                           int MTall, const sv_epi_args &ea, int grp, int split,
                                           bool live, int tid, int nthr, float *s_dyn,
                                           float *s_inv, Wait wait) {
  constexpr bool A2 = (MTP == SV_MT_PACK4);   // two k-steps per activation load
  constexpr bool PK = (MTP == SV_MT_PACK8) || A2;
  constexpr int MT = PK ? 1 : MTP;
  static_assert(!PK || FMT == SV_B4_256 || FMT == SV_B6_256, "packed rows: super-block formats");
  // column group grp, wave = K split (kept in a scalar register by the
  // caller, so the buffer resources derived from it are scalar)
  const int lane = threadIdx.x & 63;
  const int sb0 = split * sbps;
  const int sb1 = min(nsb, sb0 + sbps);
  constexpr int C = 16 * TPW, MLOC = 16 * MT;
  // LDS: the K-split partials [ksplit][MLOC][C], then the staged sums of
  // squares [rows][nssq] (dynamic size, set by the launcher)
  float *const s_part = s_dyn;
  float *const s_ssq = s_dyn + ksplit * MLOC * C;
  // residual epilogues: the rows' x and the next gain over this group's 32
  // columns, copied at kernel start (the epilogue then reads no global memory)
  float *const s_x = s_ssq + (ea.ssq ? MLOC * ea.nssq : 0);
  float *const s_g = s_x + MLOC * 32;
  const bool stage_x = ((EPI == SV_EPI_ANY) ? ea.type : EPI) == SV_EPI_RESID;
  // SWIGLU and RESID: the per-wave epilogue's outputs [MLOC][64]
  float *const s_y = stage_x ? s_g + 32 : s_x;
  const int m0 = 16 * mt0, m1 = min(M, 16 * (mt0 + MT));
  const int n16 = lane & 15, g = lane >> 4;
  const int KS = nsb * 8;
  constexpr int TB = (FMT == SV_B6_256) ? SV_TB_B6 : SV_TB_B4;
  constexpr int NC = (FMT == SV_B6_256) ? 3 : 2;
  const uint32_t mg = vconst(0x64006400u), mg64 = vconst(0x54005400u);

  const rsrc_t wr = make_rsrc(W + (size_t)grp * TPW * nsb * TB, (uint32_t)(TPW * nsb * TB));
  const rsrc_t ar = make_rsrc(ap, (uint32_t)(MTall * KS * 2048));
  const rsrc_t sr = make_rsrc(sx, (uint32_t)(MTall * nsb * 512));
  // padding rows (past M) read row 0 of their group: same cache line, and
  // their outputs are never stored
  uint32_t alane[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    alane[mt] = 16u * (uint32_t)apack_piece((16 * (mt0 + mt) + n16 < M) ? n16 : 0, g, M);
  constexpr uint32_t kOOB = 0x80000000u;   // an offset past every buffer
  // Rounds of at most SV_APACK4_ROWS rows use the compact arrangement (two
  // k-steps per 1024-byte block, real rows only); a lane whose row is past M
  // reads from beyond the buffer (zeros, no traffic).  clane[parity][part]:
  // this lane's offset inside a block.
  // (the 4-bit/256 format reads it only through SV_MT_PACK4)
  const bool c4 = A2 || (FMT != SV_B4_256 && MT == 1 && M <= SV_APACK4_ROWS);
  uint32_t clane[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      // A2: lane l holds piece l (row n16 % 4, parity (n16 / 4) % 2, part
      // n16 / 8); packed: part n16 / 8, row n16 % 8; 16 rows: row n16
      const int r = A2 ? (n16 & 3) : PK ? (n16 & 7) : n16;
      const int p = A2 ? (n16 >> 2) & 1 : e, h = PK ? (n16 >> 3) : hl;
      clane[e][hl] = (uint32_t)(16 * (16 * g + 8 * h + 4 * p + r)) |
                     ((r < SV_APACK4_ROWS && r < M) ? 0u : kOOB);
    }
  if (A2) {
    alane[0] = 0;   // (compact arrangement only: clane)
  } else if (PK) {
    // lanes n16 < 8: high part of row n16; n16 >= 8: low part of row n16 - 8
    const int r = n16 & 7;
    alane[0] = (n16 < 8 ? 0u : 1024u) + 16u * (uint32_t)apack_piece((m0 + r < M) ? r : 0, g, M);
  }

  floatx4 acc[TPW][MT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Two weight buffers (super-blocks sb and sb + 1 in use or in flight) and
  // one activation register set that is refilled a k-step at a time: as
  // soon as k-step ks of super-block sb has been multiplied against every
  // tile, k-step ks of super-block sb + 1 is loaded into the same registers.
  // Every load is thus issued about one super-block of work before its use,
  // and the loop carries no register copies (the two weight buffers
  // alternate within an unrolled pair of steps).
  // 4-bit formats: rraw holds the record of tile g % TPW in lane group g,
  // spread to all lane groups at the step.  The 6-bit format (the lm_head,
  // whose kernels are bound by vector ALU issue, not by loads) loads each
  // tile's record and super-scale.
  constexpr bool RS = (FMT != SV_B6_256);
  u32x4 rraw[2], rtile[2][RS ? 1 : TPW], cod[2][TPW][NC];
  uint32_t dtile[2][RS ? 1 : TPW];
  // A super-block past this wave's K range loads from beyond the buffer
  // resource: the hardware returns zeros without touching memory, and every
  // step issues the same loads (static wait counts).  The gate|up weights
  // (four tiles per wave) stream as non-temporal loads: measured 2% faster
  // for that GEMM, no gain for the others.
  auto wld = [&](uint32_t off) {
    if constexpr (TPW == 4) return bload16_nt(wr, off);
    else return bload16(wr, off);
  };
  auto load_w = [&](int sb, int buf) {
    const uint32_t oob = sb < sb1 ? 0u : kOOB;
    if constexpr (RS) {
      const uint32_t tr = (uint32_t)(((g & (TPW - 1)) * nsb + (sb < sb1 ? sb : sb0)) * TB) | oob;
      rraw[buf] = wld(tr + 16 * n16);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t tb = (uint32_t)((t * nsb + (sb < sb1 ? sb : sb0)) * TB) | oob;
      if constexpr (!RS) {
        rtile[buf][t] = wld(tb + 16 * n16);
        dtile[buf][t] = bload2(wr, tb + 256 + 2 * n16);
      }
      if constexpr (FMT == SV_B6_256) {
        cod[buf][t][0] = wld(tb + 288 + 16 * lane);
        cod[buf][t][1] = wld(tb + 288 + 1024 + 16 * lane);
        cod[buf][t][2] = wld(tb + 2336 + 16 * lane);
      } else {
        cod[buf][t][0] = wld(tb + 256 + 16 * lane);
        cod[buf][t][1] = wld(tb + 256 + 1024 + 16 * lane);
      }
    }
  };

  // activation operand: fp16 high/low parts per k-step and (4-bit
  // super-block format) the packed sub-block sums
  half8 Ah[8][MT], Al[8][MT], shi[MT], slo[MT];
  auto load_a_ks = [&](int sb, int ks) {
    if (A2 && (ks & 1)) return;   // the even k-step's load brought it
    const uint32_t oob = sb < sb1 ? 0u : kOOB;
    const int sbc = sb < sb1 ? sb : sb0;
    // compact arrangement (a single M-tile): block ks / 2 of the super-block
    const uint32_t cbase = (uint32_t)((sbc * 4 + (ks >> 1)) * 1024) | oob;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t base = (uint32_t)(((mt0 + mt) * KS + sbc * 8 + ks) * 2048) | oob;
      const uint32_t oh = c4 ? (cbase | clane[ks & 1][0]) : base + alane[mt];
      Ah[ks][mt] = make_half8(bload16(ar, oh));
      if (!PK) {
        const uint32_t ol = c4 ? (cbase | clane[ks & 1][1]) : base + 1024 + alane[mt];
        Al[ks][mt] = make_half8(bload16(ar, ol));
      }
    }
  };
  auto load_s = [&](int sb) {
    if (FMT != SV_B4_256) return;
    const uint32_t oob = sb < sb1 ? 0u : kOOB;
    const int sbc = sb < sb1 ? sb : sb0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = (16 * (mt0 + mt) + n16 < M) ? n16 : 0;
      // lane groups 1..3 carry k slots 8..31 of the min product: they load
      // from past the buffer resource, which returns zeros
      const uint32_t gz = g == 0 ? 0u : kOOB;
      if (PK) {
        // rows 0..7: high parts, rows 8..15: low parts, as the activations
        const int r = n16 & 7;
        const uint32_t o = (uint32_t)sxpack_off(mt0, nsb, sbc, n16 < 8 ? 0 : 1,
                                                (m0 + r < M) ? r : 0) | oob | gz;
        shi[0] = make_half8(bload16(sr, o));
        break;
      }
      const uint32_t o0 = (uint32_t)sxpack_off(mt0 + mt, nsb, sbc, 0, row) | oob | gz;
      const uint32_t o1 = (uint32_t)sxpack_off(mt0 + mt, nsb, sbc, 1, row) | oob | gz;
      shi[mt] = make_half8(bload16(sr, o0));
      slo[mt] = make_half8(bload16(sr, o1));
    }
  };

  // One super-block: k-step outer, tiles inner (each tile's products still
  // accumulate in k-step order), refilling the activation registers with
  // super-block sb + 1 as they free up.
  auto step = [&](int sb, int buf) {
    u32x4 rec[TPW];
    uint32_t dd[TPW];
    if constexpr (RS) {
      uint32_t rw[4][TPW];
#pragma unroll
      for (int i = 0; i < 4; ++i) spread_rows<TPW>(rraw[buf][i], rw[i]);
#pragma unroll
      for (int t = 0; t < TPW; ++t) rec[t] = u32x4{rw[0][t], rw[1][t], rw[2][t], rw[3][t]};
    } else {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        rec[t] = rtile[buf][t];
        dd[t] = dtile[buf][t];
      }
    }
    floatx4 Th[TPW][MT], Tl[TPW][MT];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) Th[t][mt] = Tl[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      // this k-step's activation operand (A2, odd k-step: moved down from
      // rows 4..7 and 12..15 of the pair's load)
      half8 Ak[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) Ak[mt] = (A2 && (ks & 1)) ? row_down4(Ah[ks - 1][0]) : Ah[ks][mt];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const u32x4 r = rec[t];
        if (FMT == SV_B4_32) {
          const half8 b = b432_op(cod[buf][t][ks >> 2][ks & 3], mg, mg64);
          const float d = f16_at(r[ks >> 1], ks & 1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
            acc[t][mt] = upd_d(acc[t][mt], mfma16(Ak[mt], b, z0), mfma16(Al[ks][mt], b, z0), d);
          }
        } else if (FMT == SV_B4_256) {
          const half8 b = b4s_op(r, cod[buf][t][ks >> 2][ks & 3], ks, mg, mg64);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Th[t][mt] = mfma16(Ak[mt], b, Th[t][mt]);
            if (!PK) Tl[t][mt] = mfma16(Al[ks][mt], b, Tl[t][mt]);
          }
        } else {
          half8 bhi, blo;
          b6_op(cod[buf][t], r, ks, g, mg, bhi, blo);
          if (PK) {
            // rows 0..7 take hi.bhi then hi.blo; rows 8..15 take lo.bhi and
            // then exact zeros (their operand rows are zero for blo)
            const half8 zh = {0, 0, 0, 0, 0, 0, 0, 0};
            const half8 az = (n16 < 8) ? Ak[0] : zh;
            Th[t][0] = mfma16(Ak[0], bhi, Th[t][0]);
            Th[t][0] = mfma16(az, blo, Th[t][0]);
          } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              Th[t][mt] = mfma16(Ak[mt], bhi, Th[t][mt]);
              Th[t][mt] = mfma16(Ak[mt], blo, Th[t][mt]);
              Tl[t][mt] = mfma16(Al[ks][mt], bhi, Tl[t][mt]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // (A2: the pair's registers are refilled after its odd k-step)
      if (!A2) load_a_ks(sb + 1, ks);
      else if (ks & 1) load_a_ks(sb + 1, ks - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (FMT == SV_B4_256) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const u32x4 r = rec[t];
        const half8 bm = b4s_min_op(r, mg);
        const float d = f16_at(r[0], 0), dmin = f16_at(r[0], 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          // (lane groups 1..3 of shi and slo hold zeros)
          const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
          if (PK) {
            // rows 0..7 (lanes 0..31) hold the high parts' products, rows
            // 8..15 (lanes 32..63) the low parts': bring the latter down
            const floatx4 u = mfma16(shi[0], bm, z0);
            floatx4 tl, ul;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              tl[i] = upper_half_down(Th[t][0][i], lane);
              ul[i] = upper_half_down(u[i], lane);
            }
            acc[t][0] = upd_b4s(acc[t][0], Th[t][0], tl, u, ul, d, dmin);
            continue;
          }
          const floatx4 uh = mfma16(shi[mt], bm, z0);
          const floatx4 ul = mfma16(slo[mt], bm, z0);
          acc[t][mt] = upd_b4s(acc[t][mt], Th[t][mt], Tl[t][mt], uh, ul, d, dmin);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_s(sb + 1);
    } else if (FMT == SV_B6_256) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const float d = f16_at(dd[t], 0);
        if (PK) {
          floatx4 tl;
#pragma unroll
          for (int i = 0; i < 4; ++i) tl[i] = upper_half_down(Th[t][0][i], lane);
          acc[t][0] = upd_d(acc[t][0], Th[t][0], tl, d);
          continue;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = upd_d(acc[t][mt], Th[t][mt], Tl[t][mt], d);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Issue order: the first super-block's weights, its activations, the
  // second super-block's weights; then each step refills its weight buffer
  // with the super-block two ahead.  Loads complete in issue order, so each
  // wait covers only loads issued about a step earlier.
  load_w(sb0, 0);
  if constexpr (FUSED) {
    // the weights do not depend on the activations: both buffers are in
    // flight while the producers of the activations finish
    load_w(sb0 + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait();
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) load_a_ks(sb0, ks);
  load_s(sb0);
  if constexpr (!FUSED) load_w(sb0 + 1, 1);
  __builtin_amdgcn_sched_barrier(0);
  int sb = sb0;
  for (; sb + 1 < sb1; sb += 2) {
    step(sb, 0);
    load_w(sb + 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    step(sb + 1, 1);
    load_w(sb + 3, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (sb < sb1) step(sb, 0);

  // The rows' sums of squares for the epilogue's norm factors (and, for the
  // residual epilogue, the rows' x and the next gain) are copied into LDS
  // by wave 0 with direct global -> LDS loads once its products are done.
  // (Issued any earlier, such loads make the compiler wait for every
  // outstanding load at each step of the loop above, which would undo the
  // prefetching.)
#ifdef SV_TIMELINE
  if constexpr (!FUSED) {
    if (lane == 0) sv_tl_max(ea.layer, ea.tl_kind, grp, SV_TLF_LOOP, sv_tl_now());
  }
#endif
  if (!live) split = ksplit;   // no products to keep, no rows to stage
  if (split == 0 && ea.ssq) {
    const uint32_t nbytes = (uint32_t)((m1 - m0) * ea.nssq * sizeof(float));
    const uint8_t *src = (const uint8_t *)(ea.ssq + (size_t)m0 * ea.nssq);
    for (uint32_t o = 0; o < nbytes; o += 1024)
      if (o + 16u * lane < nbytes)
        __builtin_amdgcn_global_load_lds((const void *)(src + o + 16u * lane),
                                         (__attribute__((address_space(3))) void *)((uint8_t *)s_ssq + o),
                                         16, 0, 0);
  }
  if (split == 0 && stage_x) {
    // lane l copies 16 B: local row l / 8, floats 4 (l % 8) .. +3 of the group
    for (int rb = 0; rb < m1 - m0; rb += 8) {
      const int row = rb + (lane >> 3);
      if (row < m1 - m0)
        __builtin_amdgcn_global_load_lds(
            (const void *)(ea.x + (size_t)(m0 + row) * ea.H + 32 * grp + 4 * (lane & 7)),
            (__attribute__((address_space(3))) void *)(s_x + rb * 32), 16, 0, 0);
    }
    if (ea.gnext && lane < 8)
      __builtin_amdgcn_global_load_lds((const void *)(ea.gnext + 32 * grp + 4 * lane),
                                       (__attribute__((address_space(3))) void *)s_g, 16, 0, 0);
  }
  if (split == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the staged rows have landed
    sv_epi::row_scales_lds(ea, m0, m1, lane, s_ssq, s_inv);
#ifdef SV_TIMELINE
    if (!FUSED && lane == 0) sv_tl_put(ea.layer, ea.tl_kind, grp, SV_TLF_STAGED, sv_tl_now());
#endif
  }
  // the splits meet in LDS; the workgroup then applies the group's epilogue
  if (split < ksplit) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_part[(split * MLOC + 16 * mt + 4 * g + i) * C + 16 * t + n16] = acc[t][mt][i];
  }
  __syncthreads();
#ifdef SV_TIMELINE
  if (!FUSED && tid == 0) sv_tl_put(ea.layer, ea.tl_kind, grp, SV_TLF_BARRIER, sv_tl_now());
#endif
  if (!live) return;
  if constexpr (EPI == SV_EPI_SWIGLU || EPI == SV_EPI_RESID)
    sv_epi::epi_rows_wave<EPI, COH>(ea, grp, m0, m1, tid >> 6, nthr >> 6, tid & 63, s_inv, s_part,
                                    MLOC, ksplit, s_x, s_g, s_y);
  else if constexpr (EPI == SV_EPI_QKV)
    sv_epi::epi_qkv_wave<COH>(ea, grp, m0, m1, tid >> 6, nthr >> 6, tid & 63, s_inv, s_part, MLOC,
                              ksplit);
  else
    sv_epi::epi_rows<EPI, COH>(ea, grp, m0, m1, tid, nthr, s_inv, s_part, MLOC, ksplit,
                               stage_x ? s_x : nullptr, stage_x ? s_g : nullptr);
}

