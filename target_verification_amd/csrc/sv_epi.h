// GEMM epilogues, run by the GEMM kernel itself, per output column group
// (32 output columns, or 32 SwiGLU outputs from 64 interleaved gate/up
// columns), one thread per (row, 8 consecutive columns).  The split-K
// partials are summed in increasing split order (in LDS by the small-M
// kernel, whose splits are the waves of one workgroup; in registers by the
// wide-M kernel, whose waves walk the splits in turn), then:
//   QKV     scale by the row's deferred RMSNorm factor, rotate q and k
//           (pairs are adjacent after the repack's row permutation), round k
//           and v to fp16 into the cache rows len+r, and pack q for attention;
//   RESID   x += result (O and down projections), then produce the next
//           GEMM's operand x * g_next (fp16 high/low parts), its sub-block
//           sums and the 32-column sums of squares of x for the next RMSNorm;
//   SWIGLU  a = silu(g) * u, packed for the down projection;
//   LM      logits (optionally stored) and per-row partials over the group:
//           (max, lowest argmax) for greedy, (max, sum exp) of logits / T in
//           fp64 for rejection sampling (and the same for the draft logits).
// Every reduction here runs in a fixed order that does not depend on M.
#pragma once
#include "sv_device.h"
#include "sv_internal.h"

namespace sv_epi {

// Sum of the K-split partials of (local row ml, columns col..col+7) held in
// LDS as lp[split][Mloc][C], in increasing split order.  The first eight
// splits' partials are all requested before the first addition (one LDS
// round trip instead of one per split; a slot past ksplit re-reads slot 0
// and is not added).
__device__ __forceinline__ void sum_parts(const float *lp, int ksplit, int Mloc, int C, int ml,
                                          int col, float v[8]) {
  constexpr int NP = 8;
  floatx4 p0[NP], p1[NP];
#pragma unroll
  for (int ks = 0; ks < NP; ++ks) {
    const float *p = lp + ((size_t)(ks < ksplit ? ks : 0) * Mloc + ml) * C + col;
    p0[ks] = *(const floatx4 *)p;
    p1[ks] = *(const floatx4 *)(p + 4);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.f;
#pragma unroll
  for (int ks = 0; ks < NP; ++ks) {
    if (ks < ksplit) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] += p0[ks][j];
        v[4 + j] += p1[ks][j];
      }
    }
  }
  for (int ks = NP; ks < ksplit; ++ks) {
    const float *p = lp + ((size_t)ks * Mloc + ml) * C + col;
    const floatx4 q0 = *(const floatx4 *)p, q1 = *(const floatx4 *)(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] += q0[j];
      v[4 + j] += q1[j];
    }
  }
}

template <bool COH>
__device__ __forceinline__ void store_pack8(uint8_t *ap, int KS, int m, int k, const float y[8],
                                            int M) {
  half8 hi, lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f16 h, l;
    split_hl(y[j], h, l);
    hi[j] = h;
    lo[j] = l;
  }
  st_h8<COH>(ap + apack_elem(m, k, KS, 0, M), hi);
  st_h8<COH>(ap + apack_elem(m, k, KS, 1, M), lo);
}

// Producer tail shared by RESID/SWIGLU/embed: y (8 values at column k of the
// next operand, k % 8 == 0), its 32-block sum, and optionally sum of squares,
// for a round of M rows.  COH: the stores are read by other workgroups of the
// same launch.
template <bool COH>
__device__ __forceinline__ void produce8(uint8_t *ap, uint8_t *sx, int K, int m, int k,
                                         const float y[8], float *ssq, const float *xv,
                                         bool lead, int M) {
  store_pack8<COH>(ap, K / 32, m, k, y, M);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += y[j];
  s = sum4_fixed(s);
  float q = 0.f;
  if (xv) {
#pragma unroll
    for (int j = 0; j < 8; ++j) q += xv[j] * xv[j];
  }
  q = sum4_fixed(q);
  if (lead) {
    const int jb = k >> 5;
    f16 h, l;
    split_hl(s, h, l);
    if (sx) {
      const int nsb = K / 256;
      st_f16<COH>(sx + sxpack_off(m >> 4, nsb, jb >> 3, 0, m & 15) + 2 * (jb & 7), h);
      st_f16<COH>(sx + sxpack_off(m >> 4, nsb, jb >> 3, 1, m & 15) + 2 * (jb & 7), l);
    }
    if (ssq) st_f32<COH>(ssq + (size_t)m * (K / 32) + jb, q);
  }
}

__device__ __forceinline__ size_t qpack_elem(int s, int gq, int nkv, int MTQ, int KQ, int rho,
                                             int dim, int hl) {
  size_t base = (size_t)(s * nkv + gq) * MTQ * KQ * 2048;
  int mt = rho >> 4, kq = dim >> 5, gg = (dim >> 3) & 3;
  return base + ((size_t)(mt * KQ + kq) * 2 + hl) * 1024 + ((rho & 15) + 16 * gg) * 16 +
         2 * (dim & 7);
}


// Sum over the wave by a fixed xor butterfly: at each level, in the order
// 32, 16, 8, 4, 2, 1, lane l adds its value and lane l ^ level's, so every
// lane ends with the same bits (the lane helpers of sv_device.h: register
// moves only, no LDS round trips).
__device__ __forceinline__ float wave_sum_xor(float q) {
  q += lane_xor32(q);
  q += lane_xor16(q);
  q += lane_xor8(q);
  q += lane_xor4_sym8(q);   // lanes l and l ^ 8 hold equal values here
  q += lane_xor2(q);
  q += lane_xor1(q);
  return q;
}

// Row factors of the deferred RMSNorm for rows [m0, m1) (at most 64), by one
// whole wave, from the rows' 32-column partial sums of squares staged in LDS
// (lssq[(m - m0) * nssq + j], nssq a multiple of 4, at most 256) into
// inv_s[m - m0].  Lane l adds partials 4l .. 4l + 3 in increasing order; the
// fixed butterfly above then adds the 64 lane sums, so the order depends on
// nothing but the row length.  Lane m - m0 then forms row m's factor.
__device__ __forceinline__ void row_scales_lds(const sv_epi_args &a, int m0, int m1, int lane,
                                               const float *lssq, float *inv_s) {
  if (!a.ssq) {
    if (lane < m1 - m0) inv_s[lane] = a.rowscale ? a.rowscale[m0 + lane] : 1.0f;
    return;
  }
  float qrow = 0.0f;
  for (int m = m0; m < m1; ++m) {
    float q = 0.0f;
    if (4 * lane < a.nssq) {
      const floatx4 v = *(const floatx4 *)(lssq + (size_t)(m - m0) * a.nssq + 4 * lane);
      q = ((v[0] + v[1]) + v[2]) + v[3];
    }
    q = wave_sum_xor(q);
    if (lane == m - m0) qrow = q;
  }
  if (lane < m1 - m0) inv_s[lane] = 1.0f / sqrtf(qrow / (float)a.normH + a.eps);
}

// One column of the K-split partials, in increasing split order (the same
// additions as sum_parts for that column); the first eight splits' partials
// are requested before the first addition.
__device__ __forceinline__ float sum_parts1(const float *lp, int ksplit, int Mloc, int C, int ml,
                                            int col) {
  constexpr int NP = 8;
  float p[NP];
#pragma unroll
  for (int ks = 0; ks < NP; ++ks) p[ks] = lp[((size_t)(ks < ksplit ? ks : 0) * Mloc + ml) * C + col];
  float v = 0.f;
#pragma unroll
  for (int ks = 0; ks < NP; ++ks)
    if (ks < ksplit) v += p[ks];
  for (int ks = NP; ks < ksplit; ++ks) v += lp[((size_t)ks * Mloc + ml) * C + col];
  return v;
}

// The SWIGLU and RESID epilogues of column group grp for rows [m0, m1), one
// wave at a time (no workgroup barrier; the arithmetic of each output is the
// same as in epi_rows).  Wave `wave` of nw takes rows m0 + 2 wave + h,
// m0 + 2 (wave + nw) + h, ... (h = lane / 32).  First each lane forms one
// output column j = lane % 32 of its row, y (and, for RESID, the new x,
// stored to the residual stream), into ly[(m - m0) * 64 + j] (x at + 32);
// then lanes 4 h + u pack columns 8u .. 8u + 7 of row h for the next GEMM.
// lx, lg: the staged x rows and next gains (RESID).  ly: LDS, Mloc x 64
// floats; a row's entries are written and read by one wave only.
template <int EPI, bool COH>
__device__ __forceinline__ void epi_rows_wave(const sv_epi_args &a, int grp, int m0, int m1,
                                              int wave, int nw, int lane, const float *inv_s,
                                              const float *lp, int Mloc, int nparts,
                                              const float *lx, const float *lg, float *ly) {
  static_assert(EPI == SV_EPI_SWIGLU || EPI == SV_EPI_RESID, "per-wave epilogue types");
  const int h = lane >> 5, j = lane & 31;
  for (int mb = m0 + 2 * wave; mb < m1; mb += 2 * nw) {
    const int m = mb + h;
    if (m < m1) {
      const int ml = m - m0;
      const float inv = inv_s[ml];
      if constexpr (EPI == SV_EPI_SWIGLU) {
        const int gc = 32 * (j >> 4) + (j & 15);   // gate column; up is 16 further
        const float g = sum_parts1(lp, nparts, Mloc, a.C, ml, gc);
        const float u = sum_parts1(lp, nparts, Mloc, a.C, ml, gc + 16);
        const float gg = g * inv, uu = u * inv;
        ly[ml * 64 + j] = gg / (1.0f + expf(-gg)) * uu;
      } else {
        const float xin = lx[ml * 32 + j];
        const float gin = a.gnext ? lg[j] : 1.0f;
        const float v = sum_parts1(lp, nparts, Mloc, a.C, ml, j) * inv;
        const float xv = xin + v;
        st_f32<COH>((a.x_out ? a.x_out : a.x) + (size_t)m * a.H + 32 * grp + j, xv);
        ly[ml * 64 + j] = a.gnext ? xv * gin : xv;
        ly[ml * 64 + 32 + j] = xv;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS writes are done
    const int m2 = mb + (lane >> 2), u = lane & 3;
    if (lane < 8 && m2 < m1) {
      const float *r = ly + (m2 - m0) * 64 + 8 * u;
      const floatx4 y0 = *(const floatx4 *)r, y1 = *(const floatx4 *)(r + 4);
      const float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      if constexpr (EPI == SV_EPI_SWIGLU) {
        produce8<COH>(a.ap_next, a.sx_next, a.Knext, m2, 32 * grp + 8 * u, y, nullptr, nullptr,
                      u == 0, a.M);
      } else {
        const floatx4 x0 = *(const floatx4 *)(r + 32), x1 = *(const floatx4 *)(r + 36);
        const float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        produce8<COH>(a.ap_next, a.sx_next, a.H, m2, 32 * grp + 8 * u, y, a.ssq_next, xv, u == 0,
                      a.M);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next rows' writes
  }
}

// RoPE of one dimension pair (x0, x1) by the angle with cosine c and sine
// sn: (x0 c - x1 sn, x1 c + x0 sn), each one fused multiply-add onto the
// rounded other product, written out so that every kernel rounds it alike.
__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float sn, float &ra,
                                          float &rb) {
#pragma clang fp contract(off)
  ra = __builtin_fmaf(x0, c, -(x1 * sn));
  rb = __builtin_fmaf(x1, c, x0 * sn);
}

// The QKV epilogue of column group grp for rows [m0, m1) one wave at a time
// (no workgroup barrier): wave `wave` of nw takes rows m0 + 4 wave + lane / 16,
// then 4 nw further, ...; lane l % 16 takes columns 2 (l % 16) and
// 2 (l % 16) + 1 of the group, one rotation pair of q or k (the repack puts
// pairs side by side) or two v columns.  The same arithmetic per output as
// epi_rows.
template <bool COH>
__device__ __forceinline__ void epi_qkv_wave(const sv_epi_args &a, int grp, int m0, int m1,
                                             int wave, int nw, int lane, const float *inv_s,
                                             const float *lp, int Mloc, int nparts) {
  const int pr = lane & 15;
  const int c0 = 32 * grp + 2 * pr;
  const int qdim = a.nq * a.hd, kdim = a.nkv * a.hd, half = a.hd >> 1;
  const size_t lay = (size_t)a.layer * a.S * a.nkv * a.cap * a.hd;
  for (int mb = m0 + 4 * wave; mb < m1; mb += 4 * nw) {
    const int m = mb + (lane >> 4);
    if (m >= m1) continue;
    const int ml = m - m0;
    const int s = m / a.nt, r = m - s * a.nt;
    // the sequence's status, length and row count are requested together
    const int serr = a.err[s], slen = a.lens[s], snt = a.nts ? a.nts[s] : a.nt;
    const float inv = inv_s[ml];
    const float x0 = sum_parts1(lp, nparts, Mloc, a.C, ml, 2 * pr) * inv;
    const float x1 = sum_parts1(lp, nparts, Mloc, a.C, ml, 2 * pr + 1) * inv;
    if (serr) continue;
    // padding rows of a ragged round write no cache row and rotate with the
    // last real row's position (their values are never used)
    const bool kvw = !a.nts || r < snt;
    const int pos = slen + (kvw ? r : snt - 1);
    if (c0 < qdim + kdim) {
      const bool isq = c0 < qdim;
      const int cc = isq ? c0 : c0 - qdim;
      const int hh = cc / a.hd, pp = (cc - hh * a.hd) >> 1;
      const float2 cs = *(const float2 *)(a.rope + ((size_t)pos * half + pp) * 2);
      float ra, rb;
      rope_pair(x0, x1, cs.x, cs.y, ra, rb);
      if (isq) {
        const int gq = hh / a.G, rho = r * a.G + (hh - gq * a.G);
        const int KQ = a.hd / 32;
        f16 ah, al, bh, bl;
        split_hl(ra, ah, al);
        split_hl(rb, bh, bl);
        st_f16<COH>(a.qpack + qpack_elem(s, gq, a.nkv, a.MTQ, KQ, rho, pp, 0), ah);
        st_f16<COH>(a.qpack + qpack_elem(s, gq, a.nkv, a.MTQ, KQ, rho, pp, 1), al);
        st_f16<COH>(a.qpack + qpack_elem(s, gq, a.nkv, a.MTQ, KQ, rho, pp + half, 0), bh);
        st_f16<COH>(a.qpack + qpack_elem(s, gq, a.nkv, a.MTQ, KQ, rho, pp + half, 1), bl);
      } else if (kvw) {
        uint16_t *kr = a.kc + lay + (((size_t)s * a.nkv + hh) * a.cap + pos) * a.hd;
        st_f16<COH>(kr + pp, (f16)ra);
        st_f16<COH>(kr + pp + half, (f16)rb);
      }
    } else if (kvw) {
      const int cc = c0 - qdim - kdim;
      const int hh = cc / a.hd, w0 = cc - hh * a.hd;
      uint16_t *vr = a.vc + lay + ((size_t)s * a.nkv + hh) * a.hd * a.cap;
      st_f16<COH>(vr + (size_t)w0 * a.cap + pos, (f16)x0);
      st_f16<COH>(vr + (size_t)(w0 + 1) * a.cap + pos, (f16)x1);
    }
  }
}

// The epilogue of column group grp for rows [m0, m1), spread over nthr
// threads (tid = 0..nthr-1, nthr a multiple of 4; the four threads of a row
// are adjacent lanes of one wave).  inv_s[m - m0] is the row's norm factor;
// the nparts K-split partials are in LDS, lp[split][Mloc][C] with local rows
// (a single part when the splits were already summed in order).
// EPI: the epilogue type when known at compile time (the kernel then carries
// only that type's code and arguments), else SV_EPI_ANY (read from a.type).
// COH: the outputs (next operand, residual stream, cache rows, query
// operand) are read by other workgroups of the same launch.
template <int EPI = SV_EPI_ANY, bool COH = false>
__device__ __forceinline__ void epi_rows(const sv_epi_args &a, int grp, int m0, int m1, int tid,
                                         int nthr, const float *inv_s, const float *lp,
                                         int Mloc, int nparts, const float *lx = nullptr,
                                         const float *lg = nullptr) {
  const int type = (EPI == SV_EPI_ANY) ? a.type : EPI;
  for (int idx = tid; idx < (m1 - m0) * 4; idx += nthr) {
    const int m = m0 + (idx >> 2), u = idx & 3;
    const bool lead = (u == 0);
    const float inv = inv_s[m - m0];
    float v[8];
    if (type == SV_EPI_SWIGLU) {
      const int j0 = 8 * u;             // output column within the group (0..31)
      const int tp = j0 >> 4, c = j0 & 15;
      float gv[8], uv[8];
      sum_parts(lp, nparts, Mloc, a.C, m - m0, 32 * tp + c, gv);
      sum_parts(lp, nparts, Mloc, a.C, m - m0, 32 * tp + 16 + c, uv);
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float gg = gv[j] * inv, uu = uv[j] * inv;
        y[j] = gg / (1.0f + expf(-gg)) * uu;
      }
      produce8<COH>(a.ap_next, a.sx_next, a.Knext, m, 32 * grp + j0, y, nullptr, nullptr, lead,
                    a.M);
      continue;
    }
    const int col = 8 * u;
    const int c0 = 32 * grp + col;
    sum_parts(lp, nparts, Mloc, a.C, m - m0, col, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= inv;

    if (type == SV_EPI_RESID) {
      // x and the next gain come from LDS copies made at kernel start when
      // the caller has them (lx: the group's 32 columns per local row, lg:
      // its 32 gains), else from global memory
      const float *xi = a.x + (size_t)m * a.H + c0;
      float *xr = (a.x_out ? a.x_out : a.x) + (size_t)m * a.H + c0;
      const float *xs = lx ? lx + (size_t)(m - m0) * 32 + col : xi;
      const float *gs = lg ? lg + col : (a.gnext ? a.gnext + c0 : nullptr);
      // every input is read before the first store (xr may be xi): one
      // round trip instead of one per column
      float xin[8], gin[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xin[j] = xs[j];
        gin[j] = a.gnext ? gs[j] : 1.0f;
      }
      float xv[8], y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xv[j] = xin[j] + v[j];
        y[j] = a.gnext ? xv[j] * gin[j] : xv[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) st_f32<COH>(xr + j, xv[j]);
      produce8<COH>(a.ap_next, a.sx_next, a.H, m, c0, y, a.ssq_next, xv, lead, a.M);
    } else if (type == SV_EPI_PLAIN) {
      float *y = a.logits + (size_t)m * (32 * a.ngroups) + c0;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = v[j];
    } else if (type == SV_EPI_QKV) {
      const int s = m / a.nt, r = m - s * a.nt;
      // the sequence's status, length and row count are requested together
      const int serr = a.err[s], slen = a.lens[s], snt = a.nts ? a.nts[s] : a.nt;
      if (serr) continue;
      // Padding rows of a ragged round (r >= nts[s]) write no cache row, and
      // their rotation uses the last real row's position: len + r may lie
      // past the capacity and the RoPE table (their values are never used).
      const bool kvw = !a.nts || r < snt;
      const int pos = slen + (kvw ? r : snt - 1);
      const int qdim = a.nq * a.hd, kdim = a.nkv * a.hd;
      const size_t lay = (size_t)a.layer * a.S * a.nkv * a.cap * a.hd;
      if (c0 < qdim + kdim) {
        const bool isq = c0 < qdim;
        const int cc = isq ? c0 : c0 - qdim;
        const int hh = cc / a.hd, w0 = cc - hh * a.hd;
        const int pi = w0 >> 1, half = a.hd >> 1;
        float ra[4], rb[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float *cs = a.rope + ((size_t)pos * half + pi + p) * 2;
          rope_pair(v[2 * p], v[2 * p + 1], cs[0], cs[1], ra[p], rb[p]);
        }
        if (isq) {
          const int gq = hh / a.G, rho = r * a.G + (hh - gq * a.G);
          const int KQ = a.hd / 32;
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            half4 o1, o2;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              f16 h, l;
              split_hl(ra[p], h, l);
              o1[p] = hl ? l : h;
              split_hl(rb[p], h, l);
              o2[p] = hl ? l : h;
            }
            st_h4<COH>(a.qpack + qpack_elem(s, gq, a.nkv, a.MTQ, KQ, rho, pi, hl), o1);
            st_h4<COH>(a.qpack + qpack_elem(s, gq, a.nkv, a.MTQ, KQ, rho, pi + half, hl), o2);
          }
        } else if (kvw) {
          uint16_t *kr = a.kc + lay + (((size_t)s * a.nkv + hh) * a.cap + pos) * a.hd;
          half4 o1, o2;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o1[p] = (f16)ra[p];
            o2[p] = (f16)rb[p];
          }
          st_h4<COH>(kr + pi, o1);
          st_h4<COH>(kr + pi + half, o2);
        }
      } else if (kvw) {
        const int cc = c0 - qdim - kdim;
        const int hh = cc / a.hd, w0 = cc - hh * a.hd;
        uint16_t *vr = a.vc + lay + ((size_t)s * a.nkv + hh) * a.hd * a.cap;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          st_f16<COH>(vr + (size_t)(w0 + j) * a.cap + pos, (f16)v[j]);
      }
    } else {  // SV_EPI_LM
      const int s = m / a.nt, r = m - s * a.nt;
      // a non-finite logit (or draft logit) fails the sequence closed
      bool bad = false;
#pragma unroll
      for (int j = 0; j < 8; ++j) bad |= !__builtin_isfinite(v[j]);
      if (a.draft_logits && r < a.nt - 1) {
        const float *dl = a.draft_logits + ((size_t)s * (a.nt - 1) + r) * a.V + c0;
#pragma unroll
        for (int j = 0; j < 8; ++j) bad |= !__builtin_isfinite(dl[j]);
      }
      if (bad && a.err) atomicOr(a.err + s, SV_ERRB_NUMERIC);
      if (a.logits) {
        float *lr = a.logits + (size_t)m * a.V + c0;
        *(floatx4 *)lr = floatx4{v[0], v[1], v[2], v[3]};
        *(floatx4 *)(lr + 4) = floatx4{v[4], v[5], v[6], v[7]};
      }
      if (!a.reject) {
        float best = v[0];
        int bi = c0;
#pragma unroll
        for (int j = 1; j < 8; ++j)
          if (v[j] > best) { best = v[j]; bi = c0 + j; }
#pragma unroll
        for (int sh = 1; sh <= 2; sh <<= 1) {
          float ob = __shfl_xor(best, sh);
          int oi = __shfl_xor(bi, sh);
          if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        if (lead) {
          float *lp = a.lm_part + ((size_t)m * a.ngroups + grp) * 2;
          lp[0] = best;
          lp[1] = __builtin_bit_cast(float, bi);
        }
      } else {
        const double invT = 1.0 / (double)a.temperature;
        double z[8];
        double mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          z[j] = (double)v[j] * invT;
          mx = z[j] > mx ? z[j] : mx;
        }
        mx = fmax(mx, __shfl_xor(mx, 1));
        mx = fmax(mx, __shfl_xor(mx, 2));
        double se = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) se += exp(z[j] - mx);
        se += __shfl_xor(se, 1);
        se += __shfl_xor(se, 2);
        if (lead) {
          double *st = a.lm_stat + ((size_t)m * a.ngroups + grp) * 2;
          st[0] = mx;
          st[1] = se;
        }
        if (a.draft_logits && r < a.nt - 1) {
          const float *dl = a.draft_logits + ((size_t)s * (a.nt - 1) + r) * a.V + c0;
          double dmx = -INFINITY;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            z[j] = (double)dl[j] * invT;
            dmx = z[j] > dmx ? z[j] : dmx;
          }
          dmx = fmax(dmx, __shfl_xor(dmx, 1));
          dmx = fmax(dmx, __shfl_xor(dmx, 2));
          double dse = 0.0;
#pragma unroll
          for (int j = 0; j < 8; ++j) dse += exp(z[j] - dmx);
          dse += __shfl_xor(dse, 1);
          dse += __shfl_xor(dse, 2);
          if (lead) {
            double *dt = a.dr_stat + (((size_t)s * (a.nt - 1) + r) * a.ngroups + grp) * 2;
            dt[0] = dmx;
            dt[1] = dse;
          }
        }
      }
    }
  }
}

}  // namespace sv_epi
