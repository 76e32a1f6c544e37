// Dequant-fused small-M GEMM on the matrix cores:
//   part[item][m][c] = sum over the item's K range of x[m][k] * w[n][k]
// for the 16*TPW output columns of the item's tile group.
//
// One wave per work item (tile group, K split).  The wave streams the
// tile-blocks of its TPW tiles (16 B per lane per load, fully coalesced),
// turns the integer codes into exact fp16 operands in registers, and issues
// v_mfma_f32_16x16x32_f16 with the activation's fp16 high and low parts as
// the A operand.  The per-block scales are applied in fp32 once per
// super-block (4-bit super-block and 6-bit formats: the sub-block scale is an
// exact integer factor folded into the fp16 operand) or once per 32-block
// (4-bit/32 format).  The 4-bit super-block's min term sum_j m_j * Sx_j is a
// second small product of the packed sub-block sums with dmin * m_j (split
// exactly into fp16 high and low parts after a power-of-two rescale).
//
// The result of a row depends only on that row's activations and on the
// fixed K split of the tensor, never on how many rows the call carries.
#include "sv_device.h"
#include "sv_internal.h"

namespace {

// fp16 pair constants: magic 0x6400 = 1024.0; (1024 + q) * a + b
__device__ __forceinline__ half8 deq4(uint32_t w, half2v m0, half2v a0, half2v m1, half2v a1) {
  const uint32_t MG = 0x64006400u;
  uint32_t w8 = w >> 8;
  half2v h0 = fma_h2(as_h2((w & 0x000F000Fu) | MG), m0, a0);
  half2v h1 = fma_h2(as_h2((w & 0x00F000F0u) | MG), m1, a1);
  half2v h2 = fma_h2(as_h2((w8 & 0x000F000Fu) | MG), m0, a0);
  half2v h3 = fma_h2(as_h2((w8 & 0x00F000F0u) | MG), m1, a1);
  u32x4 u = {as_u32(h0), as_u32(h1), as_u32(h2), as_u32(h3)};
  return make_half8(u);
}

// 6-bit codes q - 32 for one k-step: low nibbles in slot layout, high bits
// (already shifted to the k-step) at 2*(s/2) + 16*(s%2).
__device__ __forceinline__ half8 deq6_t(uint32_t wl, uint32_t wh) {
  const uint32_t MG = 0x64006400u;
  const half2v c = {(f16)-1056.0f, (f16)-1056.0f};
  uint32_t wl8 = wl >> 8;
  uint32_t q0 = (wl & 0x000F000Fu) | ((wh & 0x00030003u) << 4) | MG;
  uint32_t q1 = ((wl >> 4) & 0x000F000Fu) | (((wh >> 2) & 0x00030003u) << 4) | MG;
  uint32_t q2 = (wl8 & 0x000F000Fu) | (((wh >> 4) & 0x00030003u) << 4) | MG;
  uint32_t q3 = ((wl8 >> 4) & 0x000F000Fu) | (((wh >> 6) & 0x00030003u) << 4) | MG;
  u32x4 u = {as_u32(as_h2(q0) + c), as_u32(as_h2(q1) + c), as_u32(as_h2(q2) + c),
             as_u32(as_h2(q3) + c)};
  return make_half8(u);
}

__device__ __forceinline__ half8 hmul8(half8 a, half2v s) {
  half8 sv = {s[0], s[0], s[0], s[0], s[0], s[0], s[0], s[0]};
  return a * sv;
}
__device__ __forceinline__ half8 hfma8(half8 a, half2v s, half8 c) {
  half8 sv = {s[0], s[0], s[0], s[0], s[0], s[0], s[0], s[0]};
  return __builtin_elementwise_fma(a, sv, c);
}

__device__ __forceinline__ half8 load_a(const uint8_t *ap, size_t off, bool valid) {
  if (valid) return *(const half8 *)(ap + off);
  half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return z;
}

}  // namespace

template <int FMT, int TPW, int MT>
__global__ __launch_bounds__(256) void k_qgemm(const uint8_t *__restrict__ W, int nsb,
                                               int ksplit, int sbps, int nitems,
                                               const uint8_t *__restrict__ ap,
                                               const uint8_t *__restrict__ sx, int M, int mt0,
                                               int Mp, float *__restrict__ part) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wave;
  if (item >= nitems) return;
  const int grp = item / ksplit, split = item - grp * ksplit;
  const int sb0 = split * sbps;
  const int sb1 = min(nsb, sb0 + sbps);
  const int n16 = lane & 15, g = lane >> 4;
  const int KS = nsb * 8;
  constexpr int TB = (FMT == SV_B6_256) ? SV_TB_B6 : SV_TB_B4;

  bool rowok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) rowok[mt] = 16 * (mt0 + mt) + n16 < M;

  floatx4 acc[TPW][MT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int sb = sb0; sb < sb1; ++sb) {
    u32x4 rec[TPW];
    u32x4 cod[TPW][FMT == SV_B6_256 ? 3 : 2];
    uint32_t dd[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint8_t *tb = W + ((size_t)(grp * TPW + t) * nsb + sb) * TB;
      rec[t] = *(const u32x4 *)(tb + 16 * n16);
      if (FMT == SV_B6_256) {
        dd[t] = *(const uint16_t *)(tb + 256 + 2 * n16);
        cod[t][0] = *(const u32x4 *)(tb + 288 + 16 * lane);
        cod[t][1] = *(const u32x4 *)(tb + 288 + 1024 + 16 * lane);
        cod[t][2] = *(const u32x4 *)(tb + 2336 + 16 * lane);
      } else {
        cod[t][0] = *(const u32x4 *)(tb + 256 + 16 * lane);
        cod[t][1] = *(const u32x4 *)(tb + 256 + 1024 + 16 * lane);
      }
    }
    // products with the activations' high parts (Th) and scaled low parts (Tl)
    floatx4 Th[TPW][MT], Tl[TPW][MT];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Th[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        Tl[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }

#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      half8 ahi[MT], alo[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ahi[mt] = load_a(ap, apack_off(mt0 + mt, KS, sb * 8 + ks, 0, lane), rowok[mt]);
        alo[mt] = load_a(ap, apack_off(mt0 + mt, KS, sb * 8 + ks, 1, lane), rowok[mt]);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint32_t w = cod[t][ks >> 2][ks & 3];
        if (FMT == SV_B4_256) {
          const uint32_t scb = (ks < 4 ? rec[t][1] : rec[t][2]) >> (8 * (ks & 3));
          const f16 sc = (f16)(float)(scb & 63u);
          const half2v m0 = {sc, sc};
          const half2v a0 = m0 * (half2v){(f16)-1024.0f, (f16)-1024.0f};
          const half2v m1 = m0 * (half2v){(f16)0.0625f, (f16)0.0625f};
          const half2v a1 = m0 * (half2v){(f16)-64.0f, (f16)-64.0f};
          const half8 b = deq4(w, m0, a0, m1, a1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Th[t][mt] = mfma16(ahi[mt], b, Th[t][mt]);
            Tl[t][mt] = mfma16(alo[mt], b, Tl[t][mt]);
          }
        } else if (FMT == SV_B4_32) {
          const half2v m0 = {(f16)1.0f, (f16)1.0f}, a0 = {(f16)-1032.0f, (f16)-1032.0f};
          const half2v m1 = {(f16)0.0625f, (f16)0.0625f}, a1 = {(f16)-72.0f, (f16)-72.0f};
          const half8 b = deq4(w, m0, a0, m1, a1);
          const uint32_t dw = rec[t][ks >> 1] >> (16 * (ks & 1));
          const float d = (float)__builtin_bit_cast(f16, (uint16_t)(dw & 0xFFFF));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 zh = mfma16(ahi[mt], b, z0);
            const floatx4 zl = mfma16(alo[mt], b, z0);
            acc[t][mt] += d * (zh + SV_LO_INV * zl);
          }
        } else {  // SV_B6_256
          const uint32_t wh = cod[t][2][ks >> 1] >> (8 * (ks & 1));
          const half8 tq = deq6_t(w, wh);
          const int j = 2 * ks + (g >> 1);
          const int8_t scs = (int8_t)((rec[t][j >> 2] >> (8 * (j & 3))) & 0xFF);
          const f16 sc = (f16)(float)scs;
          const half2v s2 = {sc, sc};
          const half8 bhi = hmul8(tq, s2);
          const half8 blo = hfma8(tq, s2, -bhi);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Th[t][mt] = mfma16(ahi[mt], bhi, Th[t][mt]);
            Th[t][mt] = mfma16(ahi[mt], blo, Th[t][mt]);
            Tl[t][mt] = mfma16(alo[mt], bhi, Tl[t][mt]);
          }
        }
      }
    }
    if (FMT == SV_B6_256) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const float d = (float)__builtin_bit_cast(f16, (uint16_t)dd[t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] += d * (Th[t][mt] + SV_LO_INV * Tl[t][mt]);
      }
    } else if (FMT == SV_B4_256) {
      // min term: U = sum_j (dmin*m_j) * Sx_j on lanes of group 0 (k slots = sub-blocks)
      half8 shi[MT], slo[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bool ok = rowok[mt] && g == 0;
        shi[mt] = load_a(sx, sxpack_off(mt0 + mt, nsb, sb, 0, n16), ok);
        slo[mt] = load_a(sx, sxpack_off(mt0 + mt, nsb, sb, 1, n16), ok);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const float d = (float)__builtin_bit_cast(f16, (uint16_t)(rec[t][0] & 0xFFFF));
        const float dmin = (float)__builtin_bit_cast(f16, (uint16_t)(rec[t][0] >> 16));
        // rescale dmin to [1, 2) so the split parts stay normal fp16
        uint32_t bits = __builtin_bit_cast(uint32_t, dmin);
        uint32_t ex = (bits >> 23) & 255u;
        float dms = ex ? __builtin_bit_cast(float, (bits & 0x807FFFFFu) | (127u << 23)) : 0.f;
        float unscale = ex ? __builtin_bit_cast(float, ex << 23) : 0.f;
        half8 bh, bl;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          uint32_t scm = (s < 4 ? rec[t][1] : rec[t][2]) >> (8 * (s & 3));
          uint32_t mj = ((rec[t][3] >> (4 * s)) & 15u) | (((scm >> 6) & 3u) << 4);
          const float v = (g == 0) ? dms * (float)mj : 0.f;
          const f16 h = to_f16_rtz(v);    // v has <= 17 significant bits:
          bh[s] = h;                      // h + (v - h) is exact in fp16
          bl[s] = (f16)(v - (float)h);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const floatx4 z0 = {0.f, 0.f, 0.f, 0.f};
          floatx4 uh = mfma16(shi[mt], bh, z0);
          uh = mfma16(shi[mt], bl, uh);
          const floatx4 ul = mfma16(slo[mt], bh, z0);
          acc[t][mt] += d * (Th[t][mt] + SV_LO_INV * Tl[t][mt]) -
                        unscale * (uh + SV_LO_INV * ul);
        }
      }
    }
  }
  const int C = 16 * TPW;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * (mt0 + mt) + 4 * g + i;
        if (m < M) part[((size_t)item * Mp + m) * C + 16 * t + n16] = acc[t][mt][i];
      }
}

template <int FMT, int TPW>
static hipError_t launch_mt(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                            int mt0, int mtn, int Mp, float *part, hipStream_t st) {
  dim3 grid((w->nitems + 3) / 4), block(256);
  while (mtn > 0) {
    int n = mtn >= 4 ? 4 : mtn;
    switch (n) {
      case 4:
        hipLaunchKernelGGL((k_qgemm<FMT, TPW, 4>), grid, block, 0, st, w->data, w->nsb,
                           w->ksplit, w->sbps, w->nitems, ap, sx, M, mt0, Mp, part);
        break;
      case 3:
        hipLaunchKernelGGL((k_qgemm<FMT, TPW, 3>), grid, block, 0, st, w->data, w->nsb,
                           w->ksplit, w->sbps, w->nitems, ap, sx, M, mt0, Mp, part);
        break;
      case 2:
        hipLaunchKernelGGL((k_qgemm<FMT, TPW, 2>), grid, block, 0, st, w->data, w->nsb,
                           w->ksplit, w->sbps, w->nitems, ap, sx, M, mt0, Mp, part);
        break;
      default:
        hipLaunchKernelGGL((k_qgemm<FMT, TPW, 1>), grid, block, 0, st, w->data, w->nsb,
                           w->ksplit, w->sbps, w->nitems, ap, sx, M, mt0, Mp, part);
        break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    mt0 += n;
    mtn -= n;
  }
  return hipSuccess;
}

hipError_t sv_launch_qgemm(const sv_qweight *w, const uint8_t *ap, const uint8_t *sx, int M,
                           int mt0, int mtn, int Mp, float *part, hipStream_t st) {
  if (w->type == SV_B4_256) {
    if (w->tpw == 4) return launch_mt<SV_B4_256, 4>(w, ap, sx, M, mt0, mtn, Mp, part, st);
    return launch_mt<SV_B4_256, 2>(w, ap, sx, M, mt0, mtn, Mp, part, st);
  }
  if (w->type == SV_B4_32) {
    if (w->tpw == 4) return launch_mt<SV_B4_32, 4>(w, ap, sx, M, mt0, mtn, Mp, part, st);
    return launch_mt<SV_B4_32, 2>(w, ap, sx, M, mt0, mtn, Mp, part, st);
  }
  return launch_mt<SV_B6_256, 2>(w, ap, sx, M, mt0, mtn, Mp, part, st);
}
