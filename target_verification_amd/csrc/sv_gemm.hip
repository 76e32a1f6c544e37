// Dequant-fused small-M GEMM on the matrix cores: for each group of 16*TPW
// output columns, y[m][c] = sum over k of x[m][k] * w[c][k], computed as
// K-split partials that are summed in a fixed order and then passed through
// the fused epilogue.
//
// One workgroup per tile group, one wave per K split.  A wave streams the
// tile-blocks of its TPW tiles (16 B per lane per load, fully coalesced),
// turns the integer codes into exact fp16 operands in registers, and issues
// v_mfma_f32_16x16x32_f16 with the activation's fp16 high and scaled low
// parts as the A operand (two accumulators, combined per super-block).
//
// Scales: the 6-bit sub-block scale of the 4-bit super-block format is an
// exact integer factor folded into the fp16 operand (sc * q <= 945); the
// 6-bit format's sc * (q - 32) is split into an exact fp16 high part and a
// remainder in {-1, 0, 1}; the super scale d is applied in fp32 once per
// super-block.  The 4-bit super-block's min term sum_j m_j Sx_j is a small
// product of the packed sub-block sums Sx with the exact integers m_j, scaled
// by dmin in fp32.  The 4-bit/32 format applies its block scale per k-step.
//
// Load order: after a super-block's products, the activation operand of the
// next super-block and the weights NB super-blocks ahead are issued into the
// registers just freed; memory counters complete in issue order, so a step
// waits only for loads issued one or more steps earlier.
//
// The K splits of a group meet in LDS and the workgroup applies the group's
// epilogue (summing the splits in increasing order).  The result of a row
// depends only on that row's activations and on the fixed K split of the
// tensor, never on how many rows the call carries.
#include "sv_device.h"
#include "sv_epi.h"
#include "sv_internal.h"

namespace {

typedef sv_rsrc rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return sv_make_rsrc(p, bytes);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
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

// Eight 4-bit codes (slot s at bit 4*(s/2) + 16*(s%2)) to fp16 operands:
// pair p is (1024 + q) * m + a, with q at bits 0..3 (p even: m = m0, a = a0)
// or 16q at bits 4..7 (p odd: m = m1 = m0 / 16, a = a1).
__device__ __forceinline__ half8 deq4(uint32_t w, uint32_t mg, half2v m0, half2v a0, half2v m1,
                                      half2v a1) {
  const uint32_t w8 = w >> 8;
  const half2v h0 = fma_h2(as_h2((w & 0x000F000Fu) | mg), m0, a0);
  const half2v h1 = fma_h2(as_h2((w & 0x00F000F0u) | mg), m1, a1);
  const half2v h2 = fma_h2(as_h2((w8 & 0x000F000Fu) | mg), m0, a0);
  const half2v h3 = fma_h2(as_h2((w8 & 0x00F000F0u) | mg), m1, a1);
  return make_half8(u32x4{as_u32(h0), as_u32(h1), as_u32(h2), as_u32(h3)});
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

}  // namespace

// Up to this many K splits (waves) per column group: a group is one
// workgroup that must fit a CU at two waves per SIMD.
#define SV_MAX_KSPLIT 8

template <int FMT, int TPW, int MT>
__global__ __launch_bounds__(64 * SV_MAX_KSPLIT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_qgemm(const uint8_t *__restrict__ W, int nsb, int ksplit, int sbps,
             const uint8_t *__restrict__ ap, const uint8_t *__restrict__ sx, int M, int mt0,
             int MTall, sv_epi_args ea) {
  // workgroup = column group, wave = K split; the wave index is kept in a
  // scalar register so the buffer resources derived from it are scalar
  const int split = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = blockIdx.x;
  const int sb0 = split * sbps;
  const int sb1 = min(nsb, sb0 + sbps);
  constexpr int C = 16 * TPW, MLOC = 16 * MT;
  // LDS: the K-split partials [ksplit][MLOC][C], then the staged sums of
  // squares [rows][nssq] (dynamic size, set by the launcher)
  __shared__ float s_inv[64];
  extern __shared__ __attribute__((aligned(16))) float s_dyn[];
  float *const s_part = s_dyn;
  float *const s_ssq = s_dyn + ksplit * MLOC * C;
  const int m0 = 16 * mt0, m1 = min(M, 16 * (mt0 + MT));
  // The rows' sums of squares for the epilogue's norm factors are copied
  // into LDS by wave 0 before any weight load (direct global -> LDS loads:
  // no registers held, and nothing issued later waits for them).
  if (split == 0 && ea.ssq) {
    const uint32_t nbytes = (uint32_t)((m1 - m0) * ea.nssq * sizeof(float));
    const uint8_t *src = (const uint8_t *)(ea.ssq + (size_t)m0 * ea.nssq);
    for (uint32_t o = 0; o < nbytes; o += 1024)
      if (o + 16u * lane < nbytes)
        __builtin_amdgcn_global_load_lds((const void *)(src + o + 16u * lane),
                                         (__attribute__((address_space(3))) void *)((uint8_t *)s_ssq + o),
                                         16, 0, 0);
  }
  const int n16 = lane & 15, g = lane >> 4;
  const int KS = nsb * 8;
  constexpr int TB = (FMT == SV_B6_256) ? SV_TB_B6 : SV_TB_B4;
  constexpr int NC = (FMT == SV_B6_256) ? 3 : 2;
  const uint32_t mg = vconst(0x64006400u);

  const rsrc_t wr = make_rsrc(W + (size_t)grp * TPW * nsb * TB, (uint32_t)(TPW * nsb * TB));
  const rsrc_t ar = make_rsrc(ap, (uint32_t)(MTall * KS * 2048));
  const rsrc_t sr = make_rsrc(sx, (uint32_t)(MTall * nsb * 512));
  // padding rows (past M) read row 0 of their group: same cache line, and
  // their outputs are never stored
  uint32_t alane[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    alane[mt] = 16u * ((16 * (mt0 + mt) + n16 < M) ? (uint32_t)lane : (uint32_t)(16 * g));

  floatx4 acc[TPW][MT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // NB weight buffers: the weights of NB super-blocks are in flight or in use
  constexpr int NB = 2;
  u32x4 rec[NB][TPW], cod[NB][TPW][NC];
  uint32_t dd[NB][TPW];
  // A super-block past this wave's K range loads from beyond the buffer
  // resource: the hardware returns zeros without touching memory, and the
  // loop issues the same loads every step (exact wait counts).
  constexpr uint32_t kOOB = 0x80000000u;
  auto load_w = [&](int sb, int buf) {
    const uint32_t oob = sb < sb1 ? 0u : kOOB;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t tb = (uint32_t)((t * nsb + (sb < sb1 ? sb : sb0)) * TB) | oob;
      rec[buf][t] = bload16(wr, tb + 16 * n16);
      if (FMT == SV_B6_256) {
        dd[buf][t] = bload2(wr, tb + 256 + 2 * n16);
        cod[buf][t][0] = bload16(wr, tb + 288 + 16 * lane);
        cod[buf][t][1] = bload16(wr, tb + 288 + 1024 + 16 * lane);
        cod[buf][t][2] = bload16(wr, tb + 2336 + 16 * lane);
      } else {
        dd[buf][t] = 0;
        cod[buf][t][0] = bload16(wr, tb + 256 + 16 * lane);
        cod[buf][t][1] = bload16(wr, tb + 256 + 1024 + 16 * lane);
      }
    }
  };

  // activation operand of one super-block: fp16 high/low parts and (4-bit
  // super-block format) the packed sub-block sums; one register set, reused
  half8 Ah[8][MT], Al[8][MT], shi[MT], slo[MT];
  auto load_a = [&](int sb) {
    const uint32_t oob = sb < sb1 ? 0u : kOOB;
    const int sbc = sb < sb1 ? sb : sb0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t base = (uint32_t)(((mt0 + mt) * KS + sbc * 8 + ks) * 2048) | oob;
        Ah[ks][mt] = make_half8(bload16(ar, base + alane[mt]));
        Al[ks][mt] = make_half8(bload16(ar, base + 1024 + alane[mt]));
      }
    if (FMT == SV_B4_256) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = (16 * (mt0 + mt) + n16 < M) ? n16 : 0;
        const uint32_t o0 = (uint32_t)sxpack_off(mt0 + mt, nsb, sbc, 0, row) | oob;
        const uint32_t o1 = (uint32_t)sxpack_off(mt0 + mt, nsb, sbc, 1, row) | oob;
        shi[mt] = make_half8(bload16(sr, o0));   // masked to lane group 0 at use
        slo[mt] = make_half8(bload16(sr, o1));
      }
    }
  };

  auto compute = [&](int sb, int buf) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      floatx4 Th[MT], Tl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) Th[mt] = Tl[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      const u32x4 r = rec[buf][t];
      if (FMT == SV_B4_256) {
        // sub-block scales as fp16 pairs: (1024 + sc) - 1024
        const half2v k1024 = {(f16)-1024.0f, (f16)-1024.0f};
        half2v scp[4], a0p[4], m1p[4], a1p[4];
        scp[0] = as_h2((r[1] & 0x003F003Fu) | mg) + k1024;
        scp[1] = as_h2(((r[1] >> 6) & 0x003F003Fu) | mg) + k1024;
        scp[2] = as_h2((r[2] & 0x003F003Fu) | mg) + k1024;
        scp[3] = as_h2(((r[2] >> 6) & 0x003F003Fu) | mg) + k1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0p[i] = scp[i] * half2v{(f16)-1024.0f, (f16)-1024.0f};
          m1p[i] = scp[i] * half2v{(f16)0.0625f, (f16)0.0625f};
          a1p[i] = scp[i] * half2v{(f16)-64.0f, (f16)-64.0f};
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int pi = ks >> 1, hi = ks & 1;
          const half8 b = deq4(cod[buf][t][ks >> 2][ks & 3], mg, bcast(scp[pi], hi),
                               bcast(a0p[pi], hi), bcast(m1p[pi], hi), bcast(a1p[pi], hi));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Th[mt] = mfma16(Ah[ks][mt], b, Th[mt]);
            Tl[mt] = mfma16(Al[ks][mt], b, Tl[mt]);
          }
        }
        // min term: U = sum_j m_j Sx_j with m_j exact in fp16
        const uint32_t mlo = r[3];
        half8 bm;
        {
          const uint32_t p0 = ((mlo & 0x000F000Fu) | mg) | (((r[1] >> 12) & 0x00030003u) << 4);
          const uint32_t p1 = (((mlo >> 4) & 0x000F000Fu) | mg) | (((r[1] >> 14) & 0x00030003u) << 4);
          const uint32_t p2 = (((mlo >> 8) & 0x000F000Fu) | mg) | (((r[2] >> 12) & 0x00030003u) << 4);
          const uint32_t p3 = (((mlo >> 12) & 0x000F000Fu) | mg) | (((r[2] >> 14) & 0x00030003u) << 4);
          bm = make_half8(u32x4{as_u32(as_h2(p0) + k1024), as_u32(as_h2(p1) + k1024),
                                as_u32(as_h2(p2) + k1024), as_u32(as_h2(p3) + k1024)});
        }
        const float d = (float)__builtin_bit_cast(f16, (uint16_t)(r[0] & 0xFFFF));
        const float dmin = (float)__builtin_bit_cast(f16, (uint16_t)(r[0] >> 16));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
          // lanes of groups 1..3 carry k slots 8..31 of the min product: zero
          const half8 zh = {0, 0, 0, 0, 0, 0, 0, 0};
          const floatx4 uh = mfma16(g == 0 ? shi[mt] : zh, bm, z0);
          const floatx4 ul = mfma16(g == 0 ? slo[mt] : zh, bm, z0);
          acc[t][mt] += d * (Th[mt] + SV_LO_INV * Tl[mt]) - dmin * (uh + SV_LO_INV * ul);
        }
      } else if (FMT == SV_B4_32) {
        const half2v m0 = {(f16)1.0f, (f16)1.0f}, a0 = {(f16)-1032.0f, (f16)-1032.0f};
        const half2v m1 = {(f16)0.0625f, (f16)0.0625f}, a1 = {(f16)-72.0f, (f16)-72.0f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const half8 b = deq4(cod[buf][t][ks >> 2][ks & 3], mg, m0, a0, m1, a1);
          const uint32_t dw = r[ks >> 1] >> (16 * (ks & 1));
          const float d = (float)__builtin_bit_cast(f16, (uint16_t)(dw & 0xFFFF));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 zh = mfma16(Ah[ks][mt], b, z0);
            const floatx4 zl = mfma16(Al[ks][mt], b, z0);
            acc[t][mt] += d * (zh + SV_LO_INV * zl);
          }
        }
      } else {  // SV_B6_256
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const uint32_t wh = cod[buf][t][2][ks >> 1] >> (8 * (ks & 1));
          const half8 tq = deq6_t(cod[buf][t][ks >> 2][ks & 3], wh, mg);
          const int j = 2 * ks + (g >> 1);
          const int8_t scs = (int8_t)((r[j >> 2] >> (8 * (j & 3))) & 0xFF);
          const f16 sc = (f16)(float)scs;
          const half8 sv = {sc, sc, sc, sc, sc, sc, sc, sc};
          const half8 bhi = tq * sv;
          const half8 blo = __builtin_elementwise_fma(tq, sv, -bhi);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Th[mt] = mfma16(Ah[ks][mt], bhi, Th[mt]);
            Th[mt] = mfma16(Ah[ks][mt], blo, Th[mt]);
            Tl[mt] = mfma16(Al[ks][mt], bhi, Tl[mt]);
          }
        }
        const float d = (float)__builtin_bit_cast(f16, (uint16_t)dd[buf][t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] += d * (Th[mt] + SV_LO_INV * Tl[mt]);
      }
    }
  };

  // Issue order: the next step's activation loads and the weights two steps
  // ahead are issued right after a step's products, into the registers that
  // step has just freed.  Loads complete in issue order, so the wait at the
  // start of a step covers only what was issued one and two steps earlier.
  load_a(sb0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NB; ++j) load_w(sb0 + j, j);
  // (the scheduling barriers keep the load groups in this order: the
  // activation loads of the next step ahead of the weights NB steps ahead)
  int sb = sb0;
  for (; sb + NB - 1 < sb1; sb += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      compute(sb + j, j);
      __builtin_amdgcn_sched_barrier(0);
      load_a(sb + j + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_w(sb + j + NB, j);
    }
  }
  // the last (sb1 - sb) < NB steps: their loads are already issued
#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (sb + j < sb1) {
      compute(sb + j, j);
      __builtin_amdgcn_sched_barrier(0);
      if (sb + j + 1 < sb1) load_a(sb + j + 1);
    }

  if (split == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the staged rows have landed
    sv_epi::row_scales_lds(ea, m0, m1, lane, s_ssq, s_inv);
  }
  // the splits meet in LDS; the workgroup then applies the group's epilogue
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_part[(split * MLOC + 16 * mt + 4 * g + i) * C + 16 * t + n16] = acc[t][mt][i];
  __syncthreads();
  sv_epi::epi_rows(ea, grp, m0, m1, threadIdx.x, blockDim.x, s_inv, s_part, MLOC);
}

static size_t gemm_lds_bytes(int ksplit, int MT, int TPW, const sv_epi_args &ea) {
  return sizeof(float) * ((size_t)ksplit * 16 * MT * 16 * TPW + (ea.ssq ? 16 * MT * ea.nssq : 0));
}

template <int FMT, int TPW, int MT>
static hipError_t allow_lds() {
  return hipFuncSetAttribute((const void *)k_qgemm<FMT, TPW, MT>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, 140 * 1024);
}

// Raise the dynamic LDS limit of every GEMM instantiation (host call made at
// model or weight creation, never inside a round).
hipError_t sv_gemm_prepare() {
  static bool done = false;
  if (done) return hipSuccess;
  hipError_t e = hipSuccess;
#define SV_ALLOW(F, T)                                            \
  if (e == hipSuccess) e = allow_lds<F, T, 1>();                  \
  if (e == hipSuccess) e = allow_lds<F, T, 2>();
  SV_ALLOW(SV_B4_256, 4) SV_ALLOW(SV_B4_256, 2) SV_ALLOW(SV_B4_32, 4) SV_ALLOW(SV_B4_32, 2)
  SV_ALLOW(SV_B6_256, 2)
#undef SV_ALLOW
  done = (e == hipSuccess);
  return e;
}

template <int FMT, int TPW>
static hipError_t launch_mt(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                            int mt0, int mtn, const sv_epi_args &ea, hipStream_t st) {
  if (w->ksplit > SV_MAX_KSPLIT || ea.ksplit != w->ksplit || ea.C != 16 * TPW)
    return hipErrorInvalidValue;
  dim3 grid(w->ngroups), block(64 * w->ksplit);
  const int MTall = (M + 15) / 16;
  while (mtn > 0) {
    const int n = mtn >= 2 ? 2 : mtn;   // at most 2 M-tiles per launch (registers)
#define SV_GEMM_CASE(N)                                                                     \
  case N:                                                                                   \
    hipLaunchKernelGGL((k_qgemm<FMT, TPW, N>), grid, block,                                 \
                       gemm_lds_bytes(w->ksplit, N, TPW, ea), st, w->data, w->nsb,          \
                       w->ksplit, w->sbps, ap, sx, M, mt0, MTall, ea);                      \
    break;
    switch (n) {
      SV_GEMM_CASE(2) SV_GEMM_CASE(1)
    }
#undef SV_GEMM_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    mt0 += n;
    mtn -= n;
  }
  return hipSuccess;
}

hipError_t sv_launch_qgemm(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                           int mt0, int mtn, const sv_epi_args &ea, hipStream_t st) {
  if (w->type == SV_B4_256) {
    if (w->tpw == 4) return launch_mt<SV_B4_256, 4>(w, ap, sx, M, mt0, mtn, ea, st);
    return launch_mt<SV_B4_256, 2>(w, ap, sx, M, mt0, mtn, ea, st);
  }
  if (w->type == SV_B4_32) {
    if (w->tpw == 4) return launch_mt<SV_B4_32, 4>(w, ap, sx, M, mt0, mtn, ea, st);
    return launch_mt<SV_B4_32, 2>(w, ap, sx, M, mt0, mtn, ea, st);
  }
  return launch_mt<SV_B6_256, 2>(w, ap, sx, M, mt0, mtn, ea, st);
}
