// Verify attention: the nt query rows of every sequence (times the G query
// heads that share a KV head) against the fp16 cache, keys 0..len+r for row
// r (causal inside the block).
//
// Keys are split into fixed chunks of SV_KV_CHUNK positions at absolute
// positions; a block computes one (sequence, kv head, chunk):
//   S^T = K Q^T     on the matrix cores (K rows exact fp16, Q as fp16 hi+lo)
//   m_c = max over the chunk's visible keys, p = exp(s - m_c)
//   l_c = sum p,    O_c = V^T P^T on the matrix cores (P as fp16 hi+lo)
// and a second kernel combines the chunks in increasing chunk order:
//   m = max m_c,  o = sum_c e^(m_c - m) O_c / sum_c e^(m_c - m) l_c.
// A row never sees a chunk boundary or a reduction tree that depends on nt:
// keys it may not see contribute exact zeros (masked scores are -inf, fully
// masked chunks have l_c = 0 and O_c = 0), so row r has the same bits for
// every nt > r.
#include "sv_device.h"
#include "sv_internal.h"

// Chunk results live in "slots" of one (sequence, kv head): slot c < nch is
// key chunk c, slot nch + g is the merge of chunks 8g..8g+7.  Each slot holds,
// per query row, (m, l) and O (HD floats), with e^(s - m) weights.
#define SV_MERGE_W 8  // chunks per first-level group

// Merge n consecutive slots starting at slot c0 in increasing slot order:
//   m = max m_c,  l = sum_c e^(m_c - m) l_c,  O = sum_c e^(m_c - m) O_c.
// One thread per (query row, 8 dims); tid = 0..nthr-1, nthr a multiple of 4.
// Slots past a row's last visible key hold (-inf, 0, 0) and add exact zeros.
// final = false: (m, l, O) go to slot dst; final = true: O / l is written as
// the O projection's operand (fp16 high/low parts and 32-column sums).
template <int HD>
__device__ __forceinline__ void merge_slots(float *__restrict__ att_o, float *__restrict__ att_ml,
                                            size_t base, int cstr, int c0, int n, int NQ,
                                            int tid, int nthr, bool final, int dst, int s,
                                            int gk, int nt, int G, uint8_t *ap_o, uint8_t *sx_o,
                                            int Ko) {
  constexpr int OCT = HD / 8;
  constexpr int W = SV_MERGE_W;
  const sv_rsrc orr = sv_make_rsrc(att_o, 0xFFFFFFF0u);
  const int total = NQ * OCT;

  // the merged (m, l, O) of item (rho, oc) to slot dst, or O / l into the O
  // projection's operand
  auto emit = [&](int rho, int oc, float m, float l, float *o) {
    if (!final) {
      float *ml = att_ml + (base + (size_t)dst * cstr + rho) * 2;
      if (oc == 0) {
        st_agent(ml, m);
        st_agent(ml + 1, l);
      }
      const uint32_t off = (uint32_t)(((base + (size_t)dst * cstr + rho) * HD + 8 * oc) *
                                      sizeof(float));
      st_agent4(orr, off, floatx4{o[0], o[1], o[2], o[3]});
      st_agent4(orr, off + 16, floatx4{o[4], o[5], o[6], o[7]});
      return;
    }
    const float il = 1.0f / l;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] *= il;
    // O projection operand: row s*nt + r, column (kv head * G + h) * HD + dim
    const int r = rho / G, h = rho - r * G;
    const int mrow = s * nt + r;
    const int k = (gk * G + h) * HD + 8 * oc;
    half8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16 x, y;
      split_hl(o[j], x, y);
      hi[j] = x;
      lo[j] = y;
    }
    *(half8 *)(ap_o + apack_elem(mrow, k, Ko / 32, 0)) = hi;
    *(half8 *)(ap_o + apack_elem(mrow, k, Ko / 32, 1)) = lo;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += o[j];
    sum = sum4_fixed(sum);
    if ((oc & 3) == 0) {
      const int jb = k >> 5;
      f16 x, y;
      split_hl(sum, x, y);
      const int nsb = Ko / 256;
      *(f16 *)(sx_o + sxpack_off(mrow >> 4, nsb, jb >> 3, 0, mrow & 15) + 2 * (jb & 7)) = x;
      *(f16 *)(sx_o + sxpack_off(mrow >> 4, nsb, jb >> 3, 1, mrow & 15) + 2 * (jb & 7)) = y;
    }
  };

  if (n <= W) {
    // At most one group: each thread takes two items at a time and issues
    // all of their loads before combining either (one round trip for both).
    // (sum4_fixed in emit exchanges between the four lanes of a row, which
    // take the same path: total is a multiple of 4 and nthr of 8.)
    for (int i0 = tid; i0 < total; i0 += 2 * nthr) {
      float mc[2][W], lc[2][W];
      floatx4 a[2][W], b[2][W];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = i0 + u * nthr;
        if (idx >= total) break;      // (a thread with one item loads one)
        const int rho = idx / OCT, oc = idx - rho * OCT;
        const float *mlr = att_ml + (base + rho) * 2;
        const uint32_t obase = (uint32_t)(((base + rho) * HD + 8 * oc) * sizeof(float));
#pragma unroll
        for (int j = 0; j < W; ++j) {
          const int c = c0 + (j < n ? j : 0);
          mc[u][j] = ld_agent(mlr + (size_t)c * cstr * 2);
          lc[u][j] = ld_agent(mlr + (size_t)c * cstr * 2 + 1);
          const uint32_t off = obase + (uint32_t)((size_t)c * cstr * HD * sizeof(float));
          a[u][j] = ld_agent4(orr, off);
          b[u][j] = ld_agent4(orr, off + 16);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = i0 + u * nthr;
        if (idx >= total) break;
        const int rho = idx / OCT, oc = idx - rho * OCT;
        float m = -INFINITY, l = 0.f;
        float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < W; ++j)
          if (j < n) m = max_f(m, mc[u][j]);
#pragma unroll
        for (int j = 0; j < W; ++j) {
          if (j >= n) break;
          const float w = (mc[u][j] == -INFINITY) ? 0.f : __expf(mc[u][j] - m);
          l += w * lc[u][j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] += w * a[u][j][e];
            o[4 + e] += w * b[u][j][e];
          }
        }
        emit(rho, oc, m, l, o);
      }
    }
    return;
  }

  for (int idx = tid; idx < total; idx += nthr) {
    const int rho = idx / OCT, oc = idx - rho * OCT;
    const float *mlr = att_ml + (base + rho) * 2;
    const uint32_t obase = (uint32_t)(((base + rho) * HD + 8 * oc) * sizeof(float));
    float m = -INFINITY, l = 0.f;
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // max first, then the weighted sums, in batches
    for (int j0 = 0; j0 < n; j0 += 16) {
      float mc[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        mc[j] = ld_agent(mlr + (size_t)(c0 + (j0 + j < n ? j0 + j : 0)) * cstr * 2);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < n) m = max_f(m, mc[j]);
    }
    for (int j0 = 0; j0 < n; j0 += W) {
      float mc[W], lc[W];
      floatx4 a[W], b[W];
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const int c = c0 + (j0 + j < n ? j0 + j : 0);
        mc[j] = ld_agent(mlr + (size_t)c * cstr * 2);
        lc[j] = ld_agent(mlr + (size_t)c * cstr * 2 + 1);
        const uint32_t off = obase + (uint32_t)((size_t)c * cstr * HD * sizeof(float));
        a[j] = ld_agent4(orr, off);
        b[j] = ld_agent4(orr, off + 16);
      }
#pragma unroll
      for (int j = 0; j < W; ++j) {
        if (j0 + j >= n) break;
        const float w = (mc[j] == -INFINITY) ? 0.f : __expf(mc[j] - m);
        l += w * lc[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] += w * a[j][e];
          o[4 + e] += w * b[j][e];
        }
      }
    }
    emit(rho, oc, m, l, o);
  }
}

template <int HD, int MTQ>
__global__ __launch_bounds__(256) void k_attn_chunk(const uint16_t *__restrict__ kc,
                                                    const uint16_t *__restrict__ vc,
                                                    const uint8_t *__restrict__ qpack,
                                                    const int32_t *__restrict__ lens,
                                                    const int32_t *__restrict__ err, int nkv,
                                                    int cap, int nt, int G, float scale,
                                                    float *__restrict__ att_o,
                                                    float *__restrict__ att_ml, int nch,
                                                    int32_t *__restrict__ acnt,
                                                    uint8_t *__restrict__ ap_o,
                                                    uint8_t *__restrict__ sx_o, int Ko,
                                                    const int32_t *__restrict__ nts) {
  constexpr int KQ = HD / 32;
  constexpr int NDT = HD / 16;            // dim tiles
  constexpr int DTW = (NDT + 3) / 4;      // dim tiles per wave
  const int c = blockIdx.x, gk = blockIdx.y, s = blockIdx.z;
  const int kbase = c * SV_KV_CHUNK;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, gg = lane >> 4;
  const int NQ = nt * G;
  const uint16_t *K = kc + (size_t)(s * nkv + gk) * cap * HD;
  const uint16_t *Vt = vc + (size_t)(s * nkv + gk) * HD * cap;
  const uint8_t *Q = qpack + (size_t)(s * nkv + gk) * MTQ * KQ * 2048;
  const sv_rsrc orr = sv_make_rsrc(att_o, 0xFFFFFFF0u);
  const int nsl = nch + (nch + SV_MERGE_W - 1) / SV_MERGE_W;  // slots per (s, kv head)

  __shared__ float s_max[4][MTQ * 16];
  __shared__ float s_sum[4][MTQ * 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[4][MTQ][2][1024];

  // ---- loads: this wave's 32 key rows, then the V^T rows of its dim tiles
  // over the whole chunk, all issued before the sequence's length is read
  // (so that the two latencies overlap) and before the score phase.  The
  // chunk lies inside the cache, whose capacity is a multiple of the chunk;
  // keys at or past L are zeroed before use.
  constexpr int QPT = MTQ * KQ * 2 * 1024 / (16 * 256);   // Q bytes per thread / 16
  __shared__ __attribute__((aligned(16))) uint8_t s_q[MTQ * KQ * 2 * 1024];
  u32x4 qv[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) qv[i] = *(const u32x4 *)(Q + (size_t)(i * 256 + threadIdx.x) * 16);
  half8 ka[2][KQ];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = kbase + 32 * wave + 16 * kt + n16;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      ka[kt][kq] = *(const half8 *)(K + (size_t)key * HD + 32 * kq + 8 * gg);
  }
  u32x2 vpre[DTW][4][2];
#pragma unroll
  for (int dtw = 0; dtw < DTW; ++dtw) {
    const int dt = wave * DTW + dtw;
    const uint16_t *vr = Vt + (size_t)(16 * (dt < NDT ? dt : 0) + n16) * cap;
#pragma unroll
    for (int kw = 0; kw < 4; ++kw) {
      const int k0 = kbase + 32 * kw + 4 * gg;
      vpre[dtw][kw][0] = *(const u32x2 *)(vr + k0);
      vpre[dtw][kw][1] = *(const u32x2 *)(vr + k0 + 16);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // keep every load above the score phase
  if (err[s]) return;
  const int len = lens[s];
  const int L = len + (nts ? nts[s] : nt);   // keys written up to this round's last real row
  if (kbase >= L) return;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = kbase + 32 * wave + 16 * kt + n16;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      if (key >= L) ka[kt][kq] = half8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  // the block's query operand, shared by the four waves, into LDS
#pragma unroll
  for (int i = 0; i < QPT; ++i) *(u32x4 *)(s_q + (size_t)(i * 256 + threadIdx.x) * 16) = qv[i];
  __syncthreads();
  // ---- scores S^T for this wave's 32 keys (two tiles of 16)
  floatx4 sc[2][MTQ];
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
        const half8 qh = *(const half8 *)(s_q + ((mt * KQ + kq) * 2 + 0) * 1024 + lane * 16);
        const half8 ql = *(const half8 *)(s_q + ((mt * KQ + kq) * 2 + 1) * 1024 + lane * 16);
        sc[kt][mt] = mfma16(a, qh, sc[kt][mt]);
        sl[mt] = mfma16(a, ql, sl[mt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) sc[kt][mt] += SV_LO_INV * sl[mt];
  }
  // result lane (n16 = query row, gg): keys 4*gg + i of each tile
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt) {
    const int rho = 16 * mt + n16;
    const int lim = (rho < NQ) ? len + rho / G : -1;  // last visible key
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kbase + 32 * wave + 16 * kt + 4 * gg + i;
        float v = sc[kt][mt][i] * scale;
        if (key > lim) v = -INFINITY;
        sc[kt][mt][i] = v;
        mx = max_f(mx, v);
      }
    mx = max_f(mx, __shfl_xor(mx, 16));
    mx = max_f(mx, __shfl_xor(mx, 32));
    if (gg == 0) s_max[wave][rho] = mx;
  }
  __syncthreads();
  float cmax[MTQ];
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt) {
    const int rho = 16 * mt + n16;
    cmax[mt] = max_f(max_f(s_max[0][rho], s_max[1][rho]), max_f(s_max[2][rho], s_max[3][rho]));
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
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    if (gg == 0) s_sum[wave][rho] = sum;
    half8 ph, pl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16 h, l;
      split_hl(p[j], h, l);
      ph[j] = h;
      pl[j] = l;
    }
    *(half8 *)&s_p[wave][mt][0][lane * 16] = ph;
    *(half8 *)&s_p[wave][mt][1][lane * 16] = pl;
  }
  __syncthreads();
  // ---- O^T = V^T P^T for this wave's dim tiles over the chunk's 128 keys
#pragma unroll
  for (int dtw = 0; dtw < DTW; ++dtw) {
    const int dt = wave * DTW + dtw;
    if (dt >= NDT) break;
    const int dim = 16 * dt + n16;
    floatx4 o[MTQ], ol[MTQ];
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      o[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      ol[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kw = 0; kw < 4; ++kw) {
      // keys of slot s: 32kw + 4gg + s (s < 4) and 32kw + 16 + 4gg + (s-4)
      const int k0 = kbase + 32 * kw + 4 * gg;
      const u32x2 v0 = vpre[dtw][kw][0], v1 = vpre[dtw][kw][1];
      half8 a = make_half8(u32x4{v0[0], v0[1], v1[0], v1[1]});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (k0 + j >= L) a[j] = (f16)0.0f;
        if (k0 + 16 + j >= L) a[4 + j] = (f16)0.0f;
      }
#pragma unroll
      for (int mt = 0; mt < MTQ; ++mt) {
        const half8 bh = *(const half8 *)&s_p[kw][mt][0][lane * 16];
        const half8 bl = *(const half8 *)&s_p[kw][mt][1][lane * 16];
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
        const size_t e = (((size_t)(s * nkv + gk) * nsl + c) * (MTQ * 16) + rho) * HD +
                         16 * dt + 4 * gg;
        st_agent4(orr, (uint32_t)(e * sizeof(float)), o[mt]);
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
        st_agent(ml + 1, (s_sum[0][rho] + s_sum[1][rho]) + (s_sum[2][rho] + s_sum[3][rho]));
      }
    }
  }

  // Publish this chunk.  The last block of its group of SV_MERGE_W chunks
  // merges the group into slot nch + g; the last group to be merged merges
  // the groups into the O projection's operand.  Groups are fixed by
  // absolute chunk index, so a row's merge order does not depend on nt.
  __shared__ int s_last;
  const int S_ = gridDim.z;
  const int nc = (L + SV_KV_CHUNK - 1) / SV_KV_CHUNK;
  const int ngrp = (nch + SV_MERGE_W - 1) / SV_MERGE_W, ngu = (nc + SV_MERGE_W - 1) / SV_MERGE_W;
  const int grp = c / SV_MERGE_W, c0 = grp * SV_MERGE_W;
  const int ng = min(SV_MERGE_W, nc - c0);
  const int sg = s * nkv + gk;
  const size_t base = (size_t)sg * (nch + ngrp) * (MTQ * 16);
  wait_stores();
  __syncthreads();
  if (wave == 0) {
    const bool last = arrive_last(acnt + S_ * nkv + sg * ngrp + grp, ng, lane);
    if (lane == 0) s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  compiler_barrier();
  if (ngu == 1) {
    // All of this (sequence, kv head)'s chunks are in group 0: merge them
    // straight into the operand.  The bits equal the two-level merge's,
    // whose second level would weight this group's result by exp(0) = 1
    // and add exact zeros for groups a row cannot see, so a row's result
    // still does not depend on nt.
    merge_slots<HD>(att_o, att_ml, base, MTQ * 16, c0, ng, NQ, threadIdx.x, blockDim.x, true, 0,
                    s, gk, nt, G, ap_o, sx_o, Ko);
    return;
  }
  merge_slots<HD>(att_o, att_ml, base, MTQ * 16, c0, ng, NQ, threadIdx.x, blockDim.x, false,
                  nch + grp, s, gk, nt, G, ap_o, sx_o, Ko);
  wait_stores();
  __syncthreads();
  if (wave == 0) {
    const bool last = arrive_last(acnt + sg, ngu, lane);
    if (lane == 0) s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  compiler_barrier();
  merge_slots<HD>(att_o, att_ml, base, MTQ * 16, nch, ngu, NQ, threadIdx.x, blockDim.x, true, 0,
                  s, gk, nt, G, ap_o, sx_o, Ko);
}

template <int HD>
static hipError_t launch_attn_hd(int MTQ, const uint16_t *kc, const uint16_t *vc,
                                 const uint8_t *qpack, const int32_t *lens, const int32_t *err,
                                 int S, int nkv, int cap, int nt, int G, float *att_o,
                                 float *att_ml, int nch, int32_t *acnt, uint8_t *ap_o,
                                 uint8_t *sx_o, int Ko, const int32_t *nts, hipStream_t st) {
  dim3 grid(nch, nkv, S), block(256);
  const float scale = 1.0f / sqrtf((float)HD);
#define SV_ATT_CASE(N)                                                                       \
  case N:                                                                                    \
    hipLaunchKernelGGL((k_attn_chunk<HD, N>), grid, block, 0, st, kc, vc, qpack, lens, err, \
                       nkv, cap, nt, G, scale, att_o, att_ml, nch, acnt, ap_o, sx_o, Ko, \
                       nts);                                                                 \
    break;
  switch (MTQ) {
    SV_ATT_CASE(1) SV_ATT_CASE(2) SV_ATT_CASE(3) SV_ATT_CASE(4) SV_ATT_CASE(5)
    SV_ATT_CASE(6) SV_ATT_CASE(7)
    default: return hipErrorInvalidValue;
  }
#undef SV_ATT_CASE
  return hipGetLastError();
}

hipError_t sv_launch_attn(int hd, int MTQ, const uint16_t *kc, const uint16_t *vc,
                          const uint8_t *qpack, const int32_t *lens, const int32_t *err,
                          int S, int nkv, int cap, int nt, int G, float *att_o,
                          float *att_ml, int nch, int32_t *acnt, uint8_t *ap_o, uint8_t *sx_o,
                          int Ko, const int32_t *nts, hipStream_t st) {
  if (hd == 128)
    return launch_attn_hd<128>(MTQ, kc, vc, qpack, lens, err, S, nkv, cap, nt, G, att_o,
                               att_ml, nch, acnt, ap_o, sx_o, Ko, nts, st);
  if (hd == 64)
    return launch_attn_hd<64>(MTQ, kc, vc, qpack, lens, err, S, nkv, cap, nt, G, att_o,
                              att_ml, nch, acnt, ap_o, sx_o, Ko, nts, st);
  return hipErrorInvalidValue;
}
