// Verify attention as device functions shared by the attention kernels and
// the fused layer kernel: the chunk computation of one (sequence, kv head,
// key chunk) by SV_ATT_NWV waves, and one thread of the chunk merge.  See
// sv_attn.hip for the design.
#pragma once
#include "sv_device.h"
#include "sv_internal.h"

#define SV_ATT_NWV (SV_ATT_CHUNK / 32)   // waves per chunk block
// chunks per merge batch and lane: one batch covers 8 * SV_ATT_MB chunks
#define SV_ATT_MB (SV_ATT_CHUNK >= 128 ? 8 : 9)

// Chunk results live in "slots" of one (sequence, kv head): slot c is key
// chunk c and holds, per query row, (m, l) and O (HD floats), with e^(s - m)
// weights.

// (m, l, O) <- (m_a, l_a, O_a) combined with (m_b, l_b, O_b), a first:
//   m = max(m_a, m_b),  l = w_a l_a + w_b l_b,  O = w_a O_a + w_b O_b,
//   w = e^(m_x - m), 0 for m_x = -inf.  Each sum is one fused multiply-add
// of the a term onto the rounded b product, written out so that the
// rounding does not depend on how the compiler contracts the expression.
__device__ __forceinline__ void ml_combine(float ma, float la, const float *oa, float mb, float lb,
                                           const float *ob, float &m, float &l, float *o) {
#pragma clang fp contract(off)
  m = max_f(ma, mb);
  const float wa = (ma == -INFINITY) ? 0.f : __expf(ma - m);
  const float wb = (mb == -INFINITY) ? 0.f : __expf(mb - m);
  l = __builtin_fmaf(wa, la, wb * lb);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(wa, oa[e], wb * ob[e]);
}

// The value of lane l ^ ST, for ST = 1, 2 (quad permutations) and ST = 4 as
// the eight-lane combine uses it: after the first two steps the four lanes of
// a quad hold the same bits, so the mirror lane within the eight (7 - l % 8)
// holds lane l ^ 4's value.  Register moves, no LDS.
template <int ST>
__device__ __forceinline__ float lane_xor_ml(float v) {
  constexpr int ctrl = ST == 1 ? 0xB1 /* quad [1,0,3,2] */
                       : ST == 2 ? 0x4E /* quad [2,3,0,1] */
                                 : 0x141 /* row_half_mirror */;
  static_assert(ST == 1 || ST == 2 || ST == 4, "combine steps");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Pairwise step of the eight-lane combine: lanes ST apart exchange their
// partial results and both compute the combination with the lower quarter
// index first, so the two lanes hold the same bits.
template <int ST>
__device__ __forceinline__ void ml_pair(float &m, float &l, float *o, bool upper) {
  const float mp = lane_xor_ml<ST>(m), lp = lane_xor_ml<ST>(l);
  float op[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) op[e] = lane_xor_ml<ST>(o[e]);
  float mo, lo, oo[8];
  if (upper) ml_combine(mp, lp, op, m, l, o, mo, lo, oo);
  else ml_combine(m, l, o, mp, lp, op, mo, lo, oo);
  m = mo;
  l = lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = oo[e];
}

// Thread t of the merge: eight adjacent threads per (sequence, kv head,
// query row, 8 dims) item.  Lane q takes the chunks c = q, q + 8, q + 16, ...
// below the sequence's chunk count (one batch up to 64 chunks, 8192 keys),
// in batches of eight in increasing order: per batch,
// m' = max(m, max m_c), the running (l, O) are scaled by e^(m - m') and the
// batch's e^(m_c - m') l_c, e^(m_c - m') O_c added in order.  The lanes
// are then combined as ((0 1)(2 3))((4 5)(6 7)).  Chunks past a row's last
// visible key hold (-inf, 0, 0) and change nothing (a batch of them scales
// by e^0 = 1 and adds zeros), and the assignment of chunks to lanes and
// batches depends only on the chunk index, so a row's bits do not depend on
// nt.  The result O / l goes to the O projection's operand (fp16 high and
// low parts) with its 32-column sums.  Items of one (sequence, kv head) are
// NQ * HD / 8 consecutive indices, a multiple of 4, so the 32 lanes of four
// items share every branch (t must run over whole waves of consecutive
// indices).  COH: the operand is read by other workgroups of the launch.
template <int HD, bool COH>
__device__ __forceinline__ void attn_merge_thread(
    int t, const float *__restrict__ att_o, const float *__restrict__ att_ml,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ err,
    const int32_t *__restrict__ nts, int nkv, int nt, int G, int NQ, int NQp, int nch,
    int nitems, uint8_t *__restrict__ ap_o, uint8_t *__restrict__ sx_o, int Ko) {
  constexpr int OCT = HD / 8;
  constexpr int B = SV_ATT_MB;   // chunks per batch and lane
  const int item = t >> 3, q = t & 7;
  if (item >= nitems) return;
  const int per = NQ * OCT;
  const int M = nitems / (nkv * per) * nt;   // rows of the round (sequences x nt)
  const int sg = item / per, r2 = item - sg * per;
  const int rho = r2 / OCT, oc = r2 - rho * OCT;
  const int s = sg / nkv, gk = sg - s * nkv;
  const size_t row0 = (size_t)sg * nch * NQp + rho;   // slot 0's row
  const size_t cstr = (size_t)NQp;                    // rows per slot

  float mc[B], lc[B];
  floatx4 a[B], b[B];
  // batch cb: chunks cb + 8 j below lim are read, the others are (-inf, 0, 0)
  auto load_batch = [&](int cb, int lim) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int c = cb + 8 * j;
      mc[j] = -INFINITY;
      lc[j] = 0.f;
      a[j] = b[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (c < lim) {
        const size_t r = row0 + (size_t)c * cstr;
        const float2 ml = *(const float2 *)(att_ml + 2 * r);
        mc[j] = ml.x;
        lc[j] = ml.y;
        a[j] = *(const floatx4 *)(att_o + r * HD + 8 * oc);
        b[j] = *(const floatx4 *)(att_o + r * HD + 8 * oc + 4);
      }
    }
  };
  float m = -INFINITY, l = 0.f;
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // (rescale by a plain product, then one fused multiply-add per chunk)
  auto combine_batch = [&]() {
#pragma clang fp contract(off)
    float mn = m;
#pragma unroll
    for (int j = 0; j < B; ++j) mn = max_f(mn, mc[j]);
    const float sc = (m == -INFINITY) ? 0.f : __expf(m - mn);
    l *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= sc;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const float w = (mc[j] == -INFINITY) ? 0.f : __expf(mc[j] - mn);
      l = __builtin_fmaf(w, lc[j], l);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = __builtin_fmaf(w, a[j][e], o[e]);
        o[4 + e] = __builtin_fmaf(w, b[j][e], o[4 + e]);
      }
    }
    m = mn;
  };
  // The sequence's words and the first batch over every slot (slots past
  // the sequence's chunk count may hold an earlier round's values and are
  // reset to (-inf, 0, 0) below) are requested together: one memory round
  // trip instead of three dependent ones.
  const int serr = err[s], slen = lens[s], snt = nts ? nts[s] : nt;
  load_batch(q, nch);
  if (serr) return;
  const int L = slen + snt;
  const int nc = (L + SV_ATT_CHUNK - 1) / SV_ATT_CHUNK;
#pragma unroll
  for (int j = 0; j < B; ++j)
    if (q + 8 * j >= nc) {
      mc[j] = -INFINITY;
      lc[j] = 0.f;
      a[j] = b[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  if (q < nc) combine_batch();
  for (int cb = q + 8 * B; cb < nc; cb += 8 * B) {
    load_batch(cb, nc);
    combine_batch();
  }
  ml_pair<1>(m, l, o, (q & 1) != 0);
  ml_pair<2>(m, l, o, (q & 2) != 0);
  ml_pair<4>(m, l, o, (q & 4) != 0);

  const float il = 1.0f / l;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] *= il;
  // O projection operand: row s*nt + r, column (kv head * G + h) * HD + dim
  const int r = rho / G, h = rho - r * G;
  const int mrow = s * nt + r;
  const int k = (gk * G + h) * HD + 8 * oc;
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += o[j];
  // the four items of a 32-column block sit in lanes 8 apart: lane l adds
  // lane l ^ 8's sum, then lane l ^ 16's (the 32 lanes of the four items
  // share every branch)
  {
    const float x = sum + lane_xor8(sum);
    sum = x + lane_xor16(x);
  }
  if (q != 0) return;
  half8 hi, lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f16 x, y;
    split_hl(o[j], x, y);
    hi[j] = x;
    lo[j] = y;
  }
  st_h8<COH>(ap_o + apack_elem(mrow, k, Ko / 32, 0, M), hi);
  st_h8<COH>(ap_o + apack_elem(mrow, k, Ko / 32, 1, M), lo);
  if ((oc & 3) == 0) {
    const int jb = k >> 5;
    f16 x, y;
    split_hl(sum, x, y);
    const int nsb = Ko / 256;
    st_f16<COH>(sx_o + sxpack_off(mrow >> 4, nsb, jb >> 3, 0, mrow & 15) + 2 * (jb & 7), x);
    st_f16<COH>(sx_o + sxpack_off(mrow >> 4, nsb, jb >> 3, 1, mrow & 15) + 2 * (jb & 7), y);
  }
}

// LDS of one chunk computation.
template <int HD, int MTQ>
struct attn_lds {
  static constexpr int KQ = HD / 32;
  float s_max[SV_ATT_NWV][MTQ * 16];
  float s_sum[SV_ATT_NWV][MTQ * 16];
  __attribute__((aligned(16))) uint8_t s_p[SV_ATT_NWV][MTQ][2][1024];
  __attribute__((aligned(16))) uint8_t s_q[MTQ * KQ * 2 * 1024];
};

// The chunk computation of (key chunk c, kv head gk, sequence s) by the
// SV_ATT_NWV waves of threads tid = 0 .. 64 * SV_ATT_NWV - 1 (one wave per 32
// keys), for query rows rho = r * G + h:
//   S^T = K Q^T     on the matrix cores (K rows exact fp16, Q as fp16 hi+lo)
//   m_c = max over the chunk's visible keys, p = exp(s - m_c)
//   l_c = sum p,    O_c = V^T P^T on the matrix cores (P as fp16 hi+lo)
// stored to the chunk's slot.  Every thread reaches every barrier (a chunk
// past the sequence, or of a failed sequence, computes nothing).
// FUSED: wait() (a workgroup-wide call) returns once the round's query
// operand and in-block cache rows are written; the key and value rows of a
// chunk that lies wholly before the committed length are requested before
// it, everything else after it.  Otherwise wait is not called and every load
// is issued before the sequence's length is read, so the two latencies
// overlap.
template <int HD, int MTQ, bool FUSED, class Wait>
__device__ __forceinline__ void attn_chunk_body(
    int c, int gk, int s, int tid, attn_lds<HD, MTQ> &sm, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const uint8_t *__restrict__ qpack,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ err, int nkv, int cap, int nt,
    int G, float scale, float *__restrict__ att_o, float *__restrict__ att_ml, int nch,
    const int32_t *__restrict__ nts, Wait wait) {
  constexpr int KQ = HD / 32;
  constexpr int NDT = HD / 16;            // dim tiles
  constexpr int NWV = SV_ATT_NWV, NTH = 64 * NWV;
  constexpr int DTW = (NDT + NWV - 1) / NWV;   // dim tiles per wave
  const int kbase = c * SV_ATT_CHUNK;
  const int wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, gg = lane >> 4;
  const int NQ = nt * G;
  const uint16_t *K = kc + (size_t)(s * nkv + gk) * cap * HD;
  const uint16_t *Vt = vc + (size_t)(s * nkv + gk) * HD * cap;
  const uint8_t *Q = qpack + (size_t)(s * nkv + gk) * MTQ * KQ * 2048;
  const int nsl = nch;   // slots per (s, kv head)
  // the stores go through a buffer resource based at this (sequence, kv
  // head)'s own slots (64-bit base), so the 32-bit offsets stay below the
  // region's size, which the host keeps under 2^31 bytes
  const size_t region = (size_t)nsl * (MTQ * 16) * HD;   // floats
  const sv_rsrc orr = sv_make_rsrc(att_o + (size_t)(s * nkv + gk) * region,
                                   (uint32_t)(region * sizeof(float)));

  // ---- loads: this wave's 32 key rows, the V^T rows of its dim tiles over
  // the whole chunk, and its share of the query operand.  The chunk lies
  // inside the cache, whose capacity is a multiple of the chunk; keys at or
  // past L are zeroed before use.
  constexpr int QB = MTQ * KQ * 2 * 1024;                 // query operand bytes
  constexpr int QPT = (QB + 16 * NTH - 1) / (16 * NTH);   // 16-byte loads per thread
  u32x4 qv[QPT];
  half8 ka[2][KQ];
  u32x4 vpre[DTW][NWV];
  // Score tile kt, row r holds key 8 (r / 4) + 4 kt + r % 4 of the wave's
  // 32, so that the scores a lane ends up with (rows 4 gg .. 4 gg + 3 of both
  // tiles) are the 8 consecutive keys 8 gg .. 8 gg + 7: its P^T operand and
  // its V^T operand (16 bytes of one V^T row) then cover the same keys.
  auto load_q = [&]() {
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if ((i * NTH + tid) * 16 < QB) qv[i] = *(const u32x4 *)(Q + (size_t)(i * NTH + tid) * 16);
  };
  auto load_kv = [&]() {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kbase + 32 * wave + 8 * (n16 >> 2) + 4 * kt + (n16 & 3);
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
        ka[kt][kq] = *(const half8 *)(K + (size_t)key * HD + 32 * kq + 8 * gg);
    }
#pragma unroll
    for (int dtw = 0; dtw < DTW; ++dtw) {
      const int dt = wave * DTW + dtw;
      const uint16_t *vr = Vt + (size_t)(16 * (dt < NDT ? dt : 0) + n16) * cap;
#pragma unroll
      for (int kw = 0; kw < NWV; ++kw)
        vpre[dtw][kw] = *(const u32x4 *)(vr + kbase + 32 * kw + 8 * gg);
    }
  };
  int len, L;
  bool act;
  if constexpr (FUSED) {
    len = lens[s];
    L = len + (nts ? nts[s] : nt);   // keys written up to this round's last real row
    act = !err[s] && kbase < L;
    const bool old = act && kbase + SV_ATT_CHUNK <= len;   // no in-block key
    if (old) load_kv();
    wait();
    if (act) {
      if (!old) load_kv();
      load_q();
    }
  } else {
    load_q();
    load_kv();
    __builtin_amdgcn_sched_barrier(0);   // keep every load above the score phase
    len = lens[s];
    L = len + (nts ? nts[s] : nt);
    act = !err[s] && kbase < L;
  }
  if (act) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kbase + 32 * wave + 8 * (n16 >> 2) + 4 * kt + (n16 & 3);
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq)
        if (key >= L) ka[kt][kq] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    // the block's query operand, shared by the waves, into LDS
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if ((i * NTH + tid) * 16 < QB) *(u32x4 *)(sm.s_q + (size_t)(i * NTH + tid) * 16) = qv[i];
  }
  __syncthreads();
  // ---- scores S^T for this wave's 32 keys (two tiles of 16)
  floatx4 sc[2][MTQ];
  if (act) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      floatx4 sl[MTQ];
#pragma unroll
      for (int mt = 0; mt < MTQ; ++mt) {
        sc[kt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        sl[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const half8 a = ka[kt][kq];
#pragma unroll
        for (int mt = 0; mt < MTQ; ++mt) {
          const half8 qh = *(const half8 *)(sm.s_q + ((mt * KQ + kq) * 2 + 0) * 1024 + lane * 16);
          const half8 ql = *(const half8 *)(sm.s_q + ((mt * KQ + kq) * 2 + 1) * 1024 + lane * 16);
          sc[kt][mt] = mfma16(a, qh, sc[kt][mt]);
          sl[mt] = mfma16(a, ql, sl[mt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MTQ; ++mt) sc[kt][mt] += SV_LO_INV * sl[mt];
    }
    // result lane (n16 = query row, gg): key 8*gg + 4*kt + i of tile kt
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      const int rho = 16 * mt + n16;
      const int lim = (rho < NQ) ? len + rho / G : -1;  // last visible key
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kbase + 32 * wave + 8 * gg + 4 * kt + i;
          float v = sc[kt][mt][i] * scale;
          if (key > lim) v = -INFINITY;
          sc[kt][mt][i] = v;
          mx = max_f(mx, v);
        }
      mx = max_f(mx, lane_xor16(mx));
      mx = max_f(mx, lane_xor32(mx));
      if (gg == 0) sm.s_max[wave][rho] = mx;
    }
  }
  __syncthreads();
  float cmax[MTQ];
  if (act) {
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      const int rho = 16 * mt + n16;
      float x = sm.s_max[0][rho];
#pragma unroll
      for (int w = 1; w < NWV; ++w) x = max_f(x, sm.s_max[w][rho]);
      cmax[mt] = x;
    }
    // ---- p = exp(s - m_c), wave partial sums, P^T operand into LDS
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      const int rho = 16 * mt + n16;
      float p[8];
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = sc[kt][mt][i];
          const float e = (v == -INFINITY) ? 0.f : __expf(v - cmax[mt]);
          p[4 * kt + i] = e;
          sum += e;
        }
      sum += lane_xor16(sum);
      sum += lane_xor32(sum);
      if (gg == 0) sm.s_sum[wave][rho] = sum;
      half8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f16 h, l;
        split_hl(p[j], h, l);
        ph[j] = h;
        pl[j] = l;
      }
      *(half8 *)&sm.s_p[wave][mt][0][lane * 16] = ph;
      *(half8 *)&sm.s_p[wave][mt][1][lane * 16] = pl;
    }
  }
  __syncthreads();
  if (!act) return;
  // ---- O^T = V^T P^T for this wave's dim tiles over the chunk's keys
#pragma unroll
  for (int dtw = 0; dtw < DTW; ++dtw) {
    const int dt = wave * DTW + dtw;
    if (dt >= NDT) break;
    floatx4 o[MTQ], ol[MTQ];
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      o[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      ol[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kw = 0; kw < NWV; ++kw) {
      // keys of slot j: 32kw + 8gg + j
      const int k0 = kbase + 32 * kw + 8 * gg;
      half8 a = make_half8(vpre[dtw][kw]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j >= L) a[j] = (f16)0.0f;
#pragma unroll
      for (int mt = 0; mt < MTQ; ++mt) {
        const half8 bh = *(const half8 *)&sm.s_p[kw][mt][0][lane * 16];
        const half8 bl = *(const half8 *)&sm.s_p[kw][mt][1][lane * 16];
        o[mt] = mfma16(a, bh, o[mt]);
        ol[mt] = mfma16(a, bl, ol[mt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) o[mt] += SV_LO_INV * ol[mt];
    // lane (n16 = query row, gg): dims 16*dt + 4*gg + i
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      const int rho = 16 * mt + n16;
      if (rho < NQ) {
        const uint32_t e = ((uint32_t)(c * (MTQ * 16) + rho)) * HD + 16 * dt + 4 * gg;
        st_agent4(orr, e * (uint32_t)sizeof(float), o[mt]);
      }
    }
  }
  if (wave == 0 && gg == 0) {
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      const int rho = 16 * mt + n16;
      if (rho < NQ) {
        float *ml = att_ml + (((size_t)(s * nkv + gk) * nsl + c) * (MTQ * 16) + rho) * 2;
        st_agent(ml, cmax[mt]);
        // the waves' sums in a fixed tree
        float t[NWV];
#pragma unroll
        for (int w = 0; w < NWV; ++w) t[w] = sm.s_sum[w][rho];
#pragma unroll
        for (int st = 1; st < NWV; st *= 2)
#pragma unroll
          for (int w = 0; w + st < NWV; w += 2 * st) t[w] += t[w + st];
        st_agent(ml + 1, t[0]);
      }
    }
  }
}
