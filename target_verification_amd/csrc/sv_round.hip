// Round-level kernels: the capacity guard, the embedding gather (which also
// produces the first GEMM's operand), the greedy and the strict rejection
// decisions with the on-device commit, and an optional NaN poison of the
// rejected cache rows (a debug aid proving those rows are never read before
// the next round overwrites them).
//
// Decision rules (the Power page, "The exactness transaction", steps 4-6; the
// minfer plan, section 3): greedy takes each row's argmax (lowest id among
// equal maxima), a = first r < d with argmax_r != ids[r+1] (else d), and emits
// argmax_a.  Rejection sampling accepts draft row r iff u_r * q_r(x) < p_r(x)
// with p = softmax(logits/T), q = softmax(draft_logits/T) in fp64; at the first
// reject it draws from max(0, p_a - q_a) (p_a if that has no mass), else from
// p_d, by the smallest k with cumsum_k > u_res * total in token-id order.
// Commit: len += a + 1 (rows past it are dead and overwritten next round).
#include "sv_device.h"
#include "sv_internal.h"

// maxlen > 0: the round's attention visits only the key chunks below
// maxlen + nt, so a longer sequence is failed here (it writes no cache row
// and is not committed) rather than attended over part of its keys.
__global__ void k_init(const int32_t *lens, const int32_t *nts, int32_t *err, int32_t *oldlen,
                       int S, int nt, int cap, int maxlen, int32_t *cnt, int ncnt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < S) {
    int l = lens ? lens[i] : 0;
    const int rows = nts ? nts[i] : nt;
    oldlen[i] = l;
    err[i] = (rows < 1 || rows > nt) ? SV_ERRB_INVALID
             : (l < 0 || l + rows > cap) ? SV_ERRB_CAPACITY
             : (maxlen > 0 && l > maxlen) ? SV_ERRB_INVALID
                                          : 0;
  }
  if (i < ncnt) cnt[i] = 0;
}

hipError_t sv_launch_init(const int32_t *lens, const int32_t *nts, int32_t *err,
                          int32_t *oldlen, int S, int nt, int cap, int maxlen, int32_t *cnt,
                          int ncnt, hipStream_t st) {
  const int n = S > ncnt ? S : ncnt;
  hipLaunchKernelGGL(k_init, dim3((n + 255) / 256), dim3(256), 0, st, lens, nts, err, oldlen, S,
                     nt, cap, maxlen, cnt, ncnt);
  return hipGetLastError();
}

__global__ void k_zero(int32_t *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// A fill kernel rather than a memset node, so that captured graphs replay it
// like any other kernel.
hipError_t sv_launch_zero(int32_t *p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// One thread per (row, 8 columns): x = E[id] (fp16 -> fp32) or the given
// hidden row; operand y = x * gamma (gamma NULL: y = x); 32-block sums of y;
// 32-column sums of squares of x (only when gamma is given: a norm follows).
__global__ __launch_bounds__(256) void k_embed(const int32_t *ids, const uint16_t *tok,
                                               const float *hidden, const float *gamma, int M,
                                               int H, float *x, uint8_t *ap, uint8_t *sx,
                                               float *ssq, int nt, int V, int32_t *err,
                                               const int32_t *nts) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int oct = H / 8;
  const int m = idx / oct, o = idx - m * oct;
  const bool ok = m < M;
  float xv[8], y[8];
  if (ok) {
    if (hidden) {
      const float *hr = hidden + (size_t)m * H + 8 * o;
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = hr[j];
    } else {
      int id = ids[m];
      if (nts && m % nt >= nts[m / nt]) id = 0;   // a padding row of a shorter sequence
      if (id < 0 || id >= V) {  // out-of-range id: flag the sequence, read row 0
        if (o == 0 && err) atomicOr(err + m / nt, SV_ERRB_INVALID);
        id = 0;
      }
      const half8 e = *(const half8 *)(tok + (size_t)id * H + 8 * o);
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = (float)e[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[(size_t)m * H + 8 * o + j] = xv[j];
      y[j] = gamma ? xv[j] * gamma[8 * o + j] : xv[j];
    }
    half8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16 a, b;
      split_hl(y[j], a, b);
      hi[j] = a;
      lo[j] = b;
    }
    *(half8 *)(ap + apack_elem(m, 8 * o, H / 32, 0, M)) = hi;
    *(half8 *)(ap + apack_elem(m, 8 * o, H / 32, 1, M)) = lo;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = y[j] = 0.f;
  }
  float s = 0.f, q = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s += y[j];
    q += xv[j] * xv[j];
  }
  s = sum4_fixed(s);
  q = sum4_fixed(q);
  if (ok && (o & 3) == 0) {
    const int jb = o >> 2;
    f16 a, b;
    split_hl(s, a, b);
    const int nsb = H / 256;
    *(f16 *)(sx + sxpack_off(m >> 4, nsb, jb >> 3, 0, m & 15) + 2 * (jb & 7)) = a;
    *(f16 *)(sx + sxpack_off(m >> 4, nsb, jb >> 3, 1, m & 15) + 2 * (jb & 7)) = b;
    if (gamma) ssq[(size_t)m * (H / 32) + jb] = q;
  }
}

hipError_t sv_launch_embed(const int32_t *ids, const uint16_t *tok, const float *hidden,
                           const float *gamma, int M, int H, float *x, uint8_t *ap,
                           uint8_t *sx, float *ssq, int nt, int V, int32_t *err,
                           const int32_t *nts, hipStream_t st) {
  const int n = M * (H / 8);
  hipLaunchKernelGGL(k_embed, dim3((n + 255) / 256), dim3(256), 0, st, ids, tok, hidden, gamma,
                     M, H, x, ap, sx, ssq, nt, V, err, nts);
  return hipGetLastError();
}

// ---- greedy ---------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// (value, id) of lane l ^ ST joined into this lane's, for the butterfly over
// a wave (ST = 32 .. 1); the order is total, so both lanes of a pair keep the
// same result and the rotations of lane_xor4_sym8 apply.
template <int ST>
__device__ __forceinline__ void better_xor(float &bv, int &bi) {
  float ov, oif;
  const float bif = __int_as_float(bi);
  if constexpr (ST == 32) { ov = lane_xor32(bv); oif = lane_xor32(bif); }
  else if constexpr (ST == 16) { ov = lane_xor16(bv); oif = lane_xor16(bif); }
  else if constexpr (ST == 8) { ov = lane_xor8(bv); oif = lane_xor8(bif); }
  else if constexpr (ST == 4) { ov = lane_xor4_sym8(bv); oif = lane_xor4_sym8(bif); }
  else if constexpr (ST == 2) { ov = lane_xor2(bv); oif = lane_xor2(bif); }
  else { ov = lane_xor1(bv); oif = lane_xor1(bif); }
  const int oi = __float_as_int(oif);
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}

__global__ __launch_bounds__(256) void k_greedy(const float *lm_part, int NG, const int32_t *ids,
                                                int nt, int32_t *err, int32_t *lens,
                                                const int32_t *oldlen, int32_t *acc,
                                                int32_t *emitted, int32_t *argmax_out,
                                                int commit, int32_t *amb, int32_t *dcnt,
                                                const int32_t *nts) {
  const int r = blockIdx.x, s = blockIdx.y, m = s * nt + r;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int s_last;
  // (value, lowest id) is a total order, so the reduction order is free
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const float2 *p = (const float2 *)lm_part + (size_t)m * NG;
  // the first PER groups per thread are requested together (in-range
  // addresses for every lane, so the loads need no branch)
  constexpr int PER = 32;
  float2 e[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int g = threadIdx.x + j * 256;
    e[j] = p[g < NG ? g : 0];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int g = threadIdx.x + j * 256;
    const int i = __builtin_bit_cast(int, e[j].y);
    if (g < NG && better(e[j].x, i, bv, bi)) { bv = e[j].x; bi = i; }
  }
  for (int g = threadIdx.x + PER * 256; g < NG; g += 256) {
    const float2 x = p[g];
    const int i = __builtin_bit_cast(int, x.y);
    if (better(x.x, i, bv, bi)) { bv = x.x; bi = i; }
  }
  better_xor<32>(bv, bi);
  better_xor<16>(bv, bi);
  better_xor<8>(bv, bi);
  better_xor<4>(bv, bi);
  better_xor<2>(bv, bi);
  better_xor<1>(bv, bi);
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  if (wave != 0) return;
  if (lane == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    // row argmax for the sequence's last block (agent scope: another block)
    __hip_atomic_store(amb + m, bi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (argmax_out) argmax_out[m] = bi;
  }
  wait_stores();
  const bool last = arrive_last(dcnt + s, nt, lane);
  if (!last || lane != 0) return;
  if (err[s]) {
    acc[s] = sv_err_status(err[s]);
    emitted[s] = -1;
    return;
  }
  const int rows = nts ? nts[s] : nt;   // 1 <= rows <= nt (checked by the init kernel)
  int am[SV_MAX_NT];
  for (int q = 0; q < rows; ++q)
    am[q] = __hip_atomic_load(amb + s * nt + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int a = rows - 1;
  for (int q = 0; q < rows - 1; ++q)
    if (am[q] != ids[s * nt + q + 1]) { a = q; break; }
  acc[s] = a;
  emitted[s] = am[a];
  if (commit) lens[s] = oldlen[s] + a + 1;
}

hipError_t sv_launch_greedy(const float *lm_part, int NG, const int32_t *ids, int S, int nt,
                            int32_t *err, int32_t *lens, int32_t *oldlen, int32_t *acc,
                            int32_t *emitted, int32_t *argmax_out, int commit, int32_t *amb,
                            int32_t *dcnt, const int32_t *nts, hipStream_t st) {
  hipLaunchKernelGGL(k_greedy, dim3(nt, S), dim3(256), 0, st, lm_part, NG, ids, nt, err, lens,
                     oldlen, acc, emitted, argmax_out, commit, amb, dcnt, nts);
  return hipGetLastError();
}

// ---- strict rejection sampling --------------------------------------------
#define SV_RJ_THREADS 1024

// (max, sum e^(z - max)) over NG groups: max first, then sums in a fixed tree.
__device__ void row_stats(const double *st, int NG, double *s_red, double &M_out,
                          double &Z_out) {
  const int t = threadIdx.x;
  double mx = -INFINITY;
  for (int g = t; g < NG; g += SV_RJ_THREADS) mx = fmax(mx, st[2 * (size_t)g]);
  s_red[t] = mx;
  __syncthreads();
  for (int w = SV_RJ_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) s_red[t] = fmax(s_red[t], s_red[t + w]);
    __syncthreads();
  }
  const double M = s_red[0];
  __syncthreads();
  double z = 0.0;
  for (int g = t; g < NG; g += SV_RJ_THREADS)
    z += exp(st[2 * (size_t)g] - M) * st[2 * (size_t)g + 1];
  s_red[t] = z;
  __syncthreads();
  for (int w = SV_RJ_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) s_red[t] += s_red[t + w];
    __syncthreads();
  }
  Z_out = s_red[0];
  M_out = M;
  __syncthreads();
}

// Strict rejection sampling in three launches.
//  1. k_rj_stats: one block per (row, sequence): the softmax statistics
//     (max, sum e^(z - max)) of the target rows and of the draft rows, from
//     the lm_head epilogue's per-32-column partials.
//  2. k_rj_sums: SV_RJ_NB blocks per sequence: each finds the accepted
//     length a (the ratio tests need only the statistics and two logits per
//     draft) and sums over its slice of the vocabulary the residual
//     max(0, p_a - q_a) and p_a.
//  3. k_rj_pick: one block per sequence: the slice that holds u * Z (slices
//     summed in order), then the inverse CDF inside that slice.

// The accepted length: the first draft r < d with u_r q_r(x) >= p_r(x), else d.
__device__ int rj_accepted(const double *rs, const float *logits, const float *draft_logits,
                           const double *uniforms, const int32_t *ids, int s, int nt, int V,
                           int d, double invT) {
  const int dl = nt - 1;
  for (int r = 0; r < d; ++r) {
    const int x = ids[s * nt + r + 1];
    const double p = exp((double)logits[((size_t)s * nt + r) * V + x] * invT - rs[2 * r]) /
                     rs[2 * r + 1];
    const double q = exp((double)draft_logits[((size_t)s * dl + r) * V + x] * invT -
                         rs[2 * (nt + r)]) / rs[2 * (nt + r) + 1];
    if (!(uniforms[s * nt + r] * q < p)) return r;
  }
  return d;
}

__global__ __launch_bounds__(SV_RJ_THREADS) void k_rj_stats(const double *lm_stat,
                                                            const double *dr_stat, int NG,
                                                            const int32_t *ids, int nt, int V,
                                                            int32_t *err, const int32_t *nts,
                                                            double *rst, int check_ids) {
  const int rr = blockIdx.x, s = blockIdx.y;   // rr < nt: target row rr; else draft row rr - nt
  __shared__ double s_red[SV_RJ_THREADS];
  const double *st = (rr < nt) ? lm_stat + (size_t)(s * nt + rr) * NG * 2
                               : dr_stat + ((size_t)s * (nt - 1) + (rr - nt)) * NG * 2;
  double M, Z;
  row_stats(st, NG, s_red, M, Z);
  if (threadIdx.x == 0) {
    rst[((size_t)s * (2 * nt - 1) + rr) * 2] = M;
    rst[((size_t)s * (2 * nt - 1) + rr) * 2 + 1] = Z;
    if (rr == 0 && check_ids) {   // the drafted ids index the logits rows below
      const int rows = nts ? min(max(nts[s], 1), nt) : nt;
      for (int r = 1; r < rows; ++r) {
        const int x = ids[s * nt + r];
        if (x < 0 || x >= V) err[s] |= SV_ERRB_INVALID;
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_rj_sums(const double *rst, const float *logits,
                                                 const float *draft_logits,
                                                 const double *uniforms, const int32_t *ids,
                                                 int nt, int V, float T, const int32_t *err,
                                                 const int32_t *nts, double *rsum) {
  const int b = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  __shared__ double s_r[256], s_p[256];
  __shared__ int s_a;
  if (err[s]) return;
  const double invT = 1.0 / (double)T;
  const int rows = nts ? min(max(nts[s], 1), nt) : nt;
  const int d = rows - 1;
  const double *rs = rst + (size_t)s * (2 * nt - 1) * 2;
  if (t == 0) s_a = rj_accepted(rs, logits, draft_logits, uniforms, ids, s, nt, V, d, invT);
  __syncthreads();
  const int a = s_a;
  const float *lrow = logits + ((size_t)s * nt + a) * V;
  const float *qrow = (a < d) ? draft_logits + ((size_t)s * (nt - 1) + a) * V : nullptr;
  const double Ma = rs[2 * a], Za = rs[2 * a + 1];
  const double Mq = qrow ? rs[2 * (nt + a)] : 0.0, Zq = qrow ? rs[2 * (nt + a) + 1] : 1.0;
  const int k0 = (int)((int64_t)V * b / SV_RJ_NB), k1 = (int)((int64_t)V * (b + 1) / SV_RJ_NB);
  double sr = 0.0, sp = 0.0;
  for (int k = k0 + t; k < k1; k += 256) {
    const double p = exp((double)lrow[k] * invT - Ma) / Za;
    sp += p;
    if (qrow) sr += fmax(0.0, p - exp((double)qrow[k] * invT - Mq) / Zq);
  }
  s_r[t] = sr;
  s_p[t] = sp;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      s_r[t] += s_r[t + w];
      s_p[t] += s_p[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    rsum[((size_t)s * SV_RJ_NB + b) * 2] = s_r[0];
    rsum[((size_t)s * SV_RJ_NB + b) * 2 + 1] = s_p[0];
  }
}

// Inverse CDF inside [k0, k1): the smallest k with E + C_k > target (C the
// running sum from k0), per-thread sums combined by a fixed-order inclusive
// scan.  Thread t owns the interval [E + S_{t-1}, E + S_t) of the scan's own
// partial sums (S_{-1} = 0), so the intervals tile exactly and at most one
// thread claims the target; inside its stretch it walks its tokens (the last
// token with weight if rounding leaves the walk short of the target).  When
// no thread claims it (the target at or past the slice's sum), the slice's
// last token with weight is taken.  Leaves the pick in *s_pick; called by
// every thread.
template <class WF>
__device__ void invcdf_slice(WF w, int k0, int k1, double E, double target, double *s_red,
                             int *s_pick) {
  const int t = threadIdx.x;
  const int chunk = (k1 - k0 + SV_RJ_THREADS - 1) / SV_RJ_THREADS;
  const int c0 = min(k1, k0 + t * chunk), c1 = min(k1, c0 + chunk);
  double loc = 0.0;
  for (int k = c0; k < c1; ++k) loc += w(k);
  if (t == 0) *s_pick = -1;
  s_red[t] = loc;
  __syncthreads();
  for (int off = 1; off < SV_RJ_THREADS; off <<= 1) {
    const double v = (t >= off) ? s_red[t - off] : 0.0;
    __syncthreads();
    s_red[t] += v;
    __syncthreads();
  }
  const double incl = E + s_red[t];
  const double excl = E + (t > 0 ? s_red[t - 1] : 0.0);
  __syncthreads();
  if (loc > 0.0 && excl <= target && target < incl) {
    double run = excl;
    int pick = -1, last = -1;
    for (int k = c0; k < c1; ++k) {
      const double wk = w(k);
      if (wk > 0.0) last = k;
      run += wk;
      if (run > target) { pick = k; break; }
    }
    *s_pick = pick >= 0 ? pick : last;
  }
  __syncthreads();
  if (*s_pick < 0 && t == SV_RJ_THREADS - 1) {
    for (int k = k1 - 1; k >= k0; --k)
      if (w(k) > 0.0) { *s_pick = k; break; }
  }
  __syncthreads();
}

__global__ __launch_bounds__(SV_RJ_THREADS) void k_rj_pick(
    const double *rst, const double *rsum, const float *logits, const float *draft_logits,
    const double *uniforms, const int32_t *ids, int nt, int V, float T, int32_t *err,
    int32_t *lens, const int32_t *oldlen, int32_t *acc, int32_t *emitted, int commit,
    const int32_t *nts) {
  const int s = blockIdx.x, t = threadIdx.x;
  __shared__ double s_red[SV_RJ_THREADS];
  __shared__ double s_E, s_target;
  __shared__ int s_a, s_b, s_res, s_pick;
  if (err[s]) {
    if (t == 0) {
      acc[s] = sv_err_status(err[s]);
      emitted[s] = -1;
    }
    return;
  }
  const double invT = 1.0 / (double)T;
  const int rows = nts ? min(max(nts[s], 1), nt) : nt;
  const int d = rows - 1;
  const double *rs = rst + (size_t)s * (2 * nt - 1) * 2;
  const double *sums = rsum + (size_t)s * SV_RJ_NB * 2;
  if (t == 0) {
    const int a = rj_accepted(rs, logits, draft_logits, uniforms, ids, s, nt, V, d, invT);
    // the normalised residual max(0, p_a - q_a) after a rejection; p_a for
    // the bonus token or when the residual has no mass
    double Zr = 0.0;
    if (a < d)
      for (int b = 0; b < SV_RJ_NB; ++b) Zr += sums[2 * b];
    const int res = (a < d) && (Zr > 0.0);
    double Z = Zr;
    if (!res) {
      Z = 0.0;
      for (int b = 0; b < SV_RJ_NB; ++b) Z += sums[2 * b + 1];
    }
    const double target = uniforms[s * nt + d] * Z;
    // the slice holding the target (the last slice with weight if rounding
    // puts the target past the total)
    double run = 0.0, E = 0.0;
    int bs = -1;
    for (int b = 0; b < SV_RJ_NB; ++b) {
      const double wb = sums[2 * b + (res ? 0 : 1)];
      if (wb > 0.0) {
        if (run + wb > target) { bs = b; E = run; break; }
        bs = b;
        E = run;
      }
      run += wb;
    }
    s_a = a;
    s_b = bs < 0 ? 0 : bs;
    s_res = res;
    s_E = E;
    s_target = target;
  }
  __syncthreads();
  const int a = s_a, b = s_b;
  const float *lrow = logits + ((size_t)s * nt + a) * V;
  const float *qrow = (a < d) ? draft_logits + ((size_t)s * (nt - 1) + a) * V : nullptr;
  const double Ma = rs[2 * a], Za = rs[2 * a + 1];
  const double Mq = qrow ? rs[2 * (nt + a)] : 0.0, Zq = qrow ? rs[2 * (nt + a) + 1] : 1.0;
  const int k0 = (int)((int64_t)V * b / SV_RJ_NB), k1 = (int)((int64_t)V * (b + 1) / SV_RJ_NB);
  auto p_of = [&](int k) { return exp((double)lrow[k] * invT - Ma) / Za; };
  if (s_res)
    invcdf_slice([&](int k) { return fmax(0.0, p_of(k) - exp((double)qrow[k] * invT - Mq) / Zq); },
                 k0, k1, s_E, s_target, s_red, &s_pick);
  else
    invcdf_slice(p_of, k0, k1, s_E, s_target, s_red, &s_pick);
  if (t == 0) {
    acc[s] = a;
    emitted[s] = s_pick;
    if (commit) lens[s] = oldlen[s] + a + 1;
  }
}

// ---- exact-match sampled verify --------------------------------------------
// Block (r, s) draws row r's token from softmax(logits / T) with its own
// uniform; the last row block of the sequence takes the first row whose draw
// differs from the next draft.
// Exact-match sampled verify in four launches: the rows' softmax statistics
// (k_rj_stats, target rows only), the sums of p_r over SV_RJ_NB vocabulary
// slices per row, each row's draw by inverse CDF inside the slice that holds
// u_r * Z_r (slices summed in order), and the per-sequence decision: accept
// through the first row whose draw differs from the next draft.
__global__ __launch_bounds__(256) void k_smp_sums(const double *rst, const float *logits,
                                                  int nt, int V, float T, const int32_t *err,
                                                  double *rsum) {
  const int b = blockIdx.x, r = blockIdx.y, s = blockIdx.z, t = threadIdx.x;
  __shared__ double s_p[256];
  if (err[s]) return;
  const double invT = 1.0 / (double)T;
  const double *rs = rst + ((size_t)s * (2 * nt - 1) + r) * 2;
  const double M = rs[0], Z = rs[1];
  const float *lrow = logits + ((size_t)s * nt + r) * V;
  const int k0 = (int)((int64_t)V * b / SV_RJ_NB), k1 = (int)((int64_t)V * (b + 1) / SV_RJ_NB);
  double sp = 0.0;
  for (int k = k0 + t; k < k1; k += 256) sp += exp((double)lrow[k] * invT - M) / Z;
  s_p[t] = sp;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) s_p[t] += s_p[t + w];
    __syncthreads();
  }
  if (t == 0) rsum[(((size_t)s * nt + r) * SV_RJ_NB + b) * 2] = s_p[0];
}

__global__ __launch_bounds__(SV_RJ_THREADS) void k_smp_pick(const double *rst,
                                                            const double *rsum,
                                                            const float *logits,
                                                            const double *uniforms, int nt,
                                                            int V, float T, const int32_t *err,
                                                            int32_t *amb, int32_t *draws_out) {
  const int r = blockIdx.x, s = blockIdx.y, t = threadIdx.x, m = s * nt + r;
  __shared__ double s_red[SV_RJ_THREADS];
  __shared__ double s_E, s_target;
  __shared__ int s_b, s_pick;
  if (err[s]) return;
  const double invT = 1.0 / (double)T;
  const double *rs = rst + ((size_t)s * (2 * nt - 1) + r) * 2;
  const double M = rs[0], Z = rs[1];
  const double *sums = rsum + ((size_t)s * nt + r) * SV_RJ_NB * 2;
  if (t == 0) {
    double Zs = 0.0;
    for (int b = 0; b < SV_RJ_NB; ++b) Zs += sums[2 * b];
    const double target = uniforms[m] * Zs;
    double run = 0.0, E = 0.0;
    int bs = -1;
    for (int b = 0; b < SV_RJ_NB; ++b) {
      const double wb = sums[2 * b];
      if (wb > 0.0) {
        if (run + wb > target) { bs = b; E = run; break; }
        bs = b;
        E = run;
      }
      run += wb;
    }
    s_b = bs < 0 ? 0 : bs;
    s_E = E;
    s_target = target;
  }
  __syncthreads();
  const int b = s_b;
  const float *lrow = logits + (size_t)m * V;
  const int k0 = (int)((int64_t)V * b / SV_RJ_NB), k1 = (int)((int64_t)V * (b + 1) / SV_RJ_NB);
  invcdf_slice([&](int k) { return exp((double)lrow[k] * invT - M) / Z; }, k0, k1, s_E,
               s_target, s_red, &s_pick);
  if (t == 0) {
    amb[m] = s_pick;
    if (draws_out) draws_out[m] = s_pick;
  }
}

__global__ void k_smp_decide(const int32_t *amb, const int32_t *ids, int nt, int32_t *err,
                             int32_t *lens, const int32_t *oldlen, int32_t *acc,
                             int32_t *emitted, int commit, const int32_t *nts, int S) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  if (err[s]) {
    acc[s] = sv_err_status(err[s]);
    emitted[s] = -1;
    return;
  }
  const int rows = nts ? nts[s] : nt;   // 1 <= rows <= nt (checked by the init kernel)
  int a = rows - 1;
  for (int q = 0; q < rows - 1; ++q)
    if (amb[s * nt + q] != ids[s * nt + q + 1]) { a = q; break; }
  acc[s] = a;
  emitted[s] = amb[s * nt + a];
  if (commit) lens[s] = oldlen[s] + a + 1;
}

hipError_t sv_launch_sample(const double *lm_stat, double *rj_stat, double *rj_sum, int NG,
                            const float *logits, const double *uniforms, const int32_t *ids,
                            int S, int nt, int V, float T, int32_t *err, int32_t *lens,
                            int32_t *oldlen, int32_t *acc, int32_t *emitted, int32_t *draws_out,
                            int commit, int32_t *amb, int32_t *dcnt, const int32_t *nts,
                            hipStream_t st) {
  (void)dcnt;
  hipLaunchKernelGGL(k_rj_stats, dim3(nt, S), dim3(SV_RJ_THREADS), 0, st, lm_stat,
                     (const double *)nullptr, NG, ids, nt, V, err, nts, rj_stat, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_smp_sums, dim3(SV_RJ_NB, nt, S), dim3(256), 0, st, rj_stat, logits, nt,
                     V, T, err, rj_sum);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_smp_pick, dim3(nt, S), dim3(SV_RJ_THREADS), 0, st, rj_stat, rj_sum,
                     logits, uniforms, nt, V, T, err, amb, draws_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_smp_decide, dim3((S + 63) / 64), dim3(64), 0, st, amb, ids, nt, err,
                     lens, oldlen, acc, emitted, commit, nts, S);
  return hipGetLastError();
}

hipError_t sv_launch_reject(const double *lm_stat, const double *dr_stat, double *rj_stat,
                            double *rj_sum, int NG, const float *logits,
                            const float *draft_logits, const double *uniforms,
                            const int32_t *ids, int S, int nt, int V, float T, int32_t *err,
                            int32_t *lens, int32_t *oldlen, int32_t *acc, int32_t *emitted,
                            int commit, const int32_t *nts, hipStream_t st) {
  hipLaunchKernelGGL(k_rj_stats, dim3(2 * nt - 1, S), dim3(SV_RJ_THREADS), 0, st, lm_stat,
                     dr_stat, NG, ids, nt, V, err, nts, rj_stat, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rj_sums, dim3(SV_RJ_NB, S), dim3(256), 0, st, rj_stat, logits,
                     draft_logits, uniforms, ids, nt, V, T, err, nts, rj_sum);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rj_pick, dim3(S), dim3(SV_RJ_THREADS), 0, st, rj_stat, rj_sum, logits,
                     draft_logits, uniforms, ids, nt, V, T, err, lens, oldlen, acc, emitted,
                     commit, nts);
  return hipGetLastError();
}

// NaN-poison the rows this round wrote but did not commit: positions
// [len_new, oldlen + nt) of every layer.
__global__ void k_poison(uint16_t *kc, uint16_t *vc, const int32_t *lens, const int32_t *oldlen,
                         const int32_t *err, int S, int nkv, int cap, int hd, int nt,
                         const int32_t *nts) {
  const int l = blockIdx.x, s = blockIdx.y;
  if (err[s]) return;
  const int p0 = lens[s], p1 = oldlen[s] + (nts ? nts[s] : nt);
  const uint16_t NAN16 = 0x7E00;
  for (int i = threadIdx.x; i < nkv * hd * nt; i += blockDim.x) {
    const int g = i / (hd * nt), rem = i - g * hd * nt;
    const int dd = rem / nt, p = p0 + (rem - dd * nt);
    if (p >= p1) continue;
    const size_t base = ((size_t)l * S + s) * nkv + g;
    kc[(base * cap + p) * hd + dd] = NAN16;
    vc[(base * hd + dd) * cap + p] = NAN16;
  }
}

hipError_t sv_launch_poison(uint16_t *kc, uint16_t *vc, const int32_t *lens,
                            const int32_t *oldlen, const int32_t *err, int L, int S, int nkv,
                            int cap, int hd, int nt, const int32_t *nts, hipStream_t st) {
  hipLaunchKernelGGL(k_poison, dim3(L, S), dim3(256), 0, st, kc, vc, lens, oldlen, err, S, nkv,
                     cap, hd, nt, nts);
  return hipGetLastError();
}

// ---- device-resident multi-round loop: the next round's ids ----------------
__global__ void k_advance(sv_advance_args a) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= a.n_seq) return;
  const int acc = a.accepted_len[s];
  if (acc < 0) return;
  const int nt = a.nt, len = a.len[s], old = len - acc - 1;
  int32_t *ids = a.ids + (size_t)s * nt;
  if (a.tokens) {
    int32_t *tk = a.tokens + (size_t)s * a.tok_cap;
    for (int j = 0; j < acc; ++j)
      if (old + 1 + j >= 0 && old + 1 + j < a.tok_cap) tk[old + 1 + j] = ids[1 + j];
    if (len >= 0 && len < a.tok_cap) tk[len] = a.emitted[s];
  }
  if (a.committed) a.committed[s] += acc + 1;
  ids[0] = a.emitted[s];
  float p = a.p_accept;
  for (int j = 0; j + 1 < nt; ++j) {
    const int P = len + 1 + j;
    int x = 0;
    if (P >= 0 && P < a.ref_cap) {
      const size_t e = (size_t)s * a.ref_cap + P;
      x = a.noise[e];
      if (a.ref && a.draw[e] < p) x = a.ref[e];
    }
    ids[1 + j] = x;
    p *= a.p_decay;
  }
  if (a.utab) {
    for (int r = 0; r < nt; ++r) {
      const int P = len + 1 + r;
      a.uniforms[(size_t)s * nt + r] =
          (P >= 0 && P < a.ref_cap) ? a.utab[(size_t)s * a.ref_cap + P] : 0.0;
    }
  }
}

hipError_t sv_launch_advance(const sv_advance_args &a, hipStream_t st) {
  hipLaunchKernelGGL(k_advance, dim3((a.n_seq + 63) / 64), dim3(64), 0, st, a);
  return hipGetLastError();
}
