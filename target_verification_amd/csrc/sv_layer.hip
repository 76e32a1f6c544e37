// One decoder layer of the verify round in a single launch (rounds of at
// most 16 rows).
//
// The layer's six operations -- the q|k|v projection with RoPE and the cache
// write, the attention chunks, the chunk merge, the O projection with the
// residual, gate|up with SwiGLU, and down with the residual -- run as
// consecutive ranges of workgroups of one launch, each doing exactly what its
// own kernel does (the same device functions, the same work decomposition,
// hence the same bits).  A workgroup takes a ticket from a counter as it
// starts; the ticket, not the hardware's block index, names its operation
// and item, so tickets follow start order.  A workgroup first requests the
// data that does not depend on the earlier operations (its weights; the key
// and value rows of cache chunks that lie wholly before the committed
// length), then waits until every workgroup of the operation it reads from
// has finished, then completes its work and counts itself finished.  A
// workgroup only ever waits for workgroups with smaller tickets, which have
// already started and wait only for smaller tickets still, so the launch
// always completes; the waits are bounded all the same (on expiry the
// sequence error words get SV_ERRB_TIMEOUT and the round fails closed).
//
// The operations overlap: the weights of the next operation are already in
// flight on the compute units the previous one has left, while its last
// workgroups finish.
//
// Data one workgroup writes and another reads within the launch is stored at
// agent scope (written through to the device's point of coherence), and no
// such buffer is read before it is written within the launch, so no
// compute unit or L2 holds an older copy of it (the launch boundary writes
// back and invalidates the caches): the O projection writes the residual
// stream and the gate|up operand to buffers of their own, distinct from the
// layer's inputs.
#include "sv_attn_body.h"
#include "sv_gemm_body.h"
#include "sv_internal.h"

static_assert(SV_ATT_NWV == 4, "two attention chunks per eight-wave workgroup");

// dynamic LDS of one launch (the static part is a few hundred bytes)
#define SV_LAYER_MAX_LDS (156 * 1024)

#ifndef SV_LAYER_SLEEP
#define SV_LAYER_SLEEP 8          // between polls: 64 * SV_LAYER_SLEEP cycles
#endif
#ifndef SV_LAYER_SPIN
#define SV_LAYER_SPIN (1 << 16)   // polls before a wait expires
#endif

#ifdef SV_LAYER_TRACE
// Timeline of the fused launches (a measurement build only): per layer and
// ticket, (operation, start, end of the wait, end) on the real-time counter.
#define SV_TRACE_LAYERS 64
#define SV_TRACE_TICKETS 2048
__device__ long long g_layer_trace[SV_TRACE_LAYERS][SV_TRACE_TICKETS][4];
extern "C" int sv_layer_trace_read(void *host, int layers) {
  if (layers < 1 || layers > SV_TRACE_LAYERS) return -1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_layer_trace),
                             sizeof(long long) * 4 * SV_TRACE_TICKETS * layers) == hipSuccess ? 0 : -1;
}
#endif

namespace {

enum { PH_QKV = 0, PH_ATT, PH_MERGE, PH_O, PH_GU, PH_DOWN, PH_N };

#ifdef SV_LAYER_TRACE
__shared__ long long s_twait;
#endif

// Workgroup-wide: thread 0 polls the finished count of operation `ph` until
// it reaches the operation's workgroup count; every thread then passes the
// barrier.  On expiry the round is failed closed and the caller proceeds.
__device__ __forceinline__ void wait_done(const sv_layer_args &a, int ph) {
  if (threadIdx.x == 0) {
    const int32_t *c = a.cnt + (1 + ph) * SV_LAYER_CSTRIDE;
    const int target = a.n_wg[ph];
    int i = 0;
    for (; i < SV_LAYER_SPIN; ++i) {
      if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      __builtin_amdgcn_s_sleep(SV_LAYER_SLEEP);
    }
    if (i == SV_LAYER_SPIN)
      for (int s = 0; s < a.S; ++s) atomicOr(a.err + s, SV_ERRB_TIMEOUT);
#ifdef SV_LAYER_TRACE
    s_twait = __builtin_amdgcn_s_memrealtime();
#endif
  }
  __syncthreads();
}

}  // namespace

template <int MTP, int MTQ>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_layer(sv_layer_args a) {
  __shared__ int s_ticket;
  __shared__ float s_inv[2][64];
  extern __shared__ __attribute__((aligned(16))) float s_dyn[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#ifdef SV_LAYER_TRACE
  const long long t_start = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) s_twait = t_start;
#endif
  if (tid == 0)
    s_ticket = __hip_atomic_fetch_add(a.cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int vb = __builtin_amdgcn_readfirstlane(s_ticket);
  int ph = 0;
  while (ph < PH_N && vb >= a.n_wg[ph]) vb -= a.n_wg[ph++];
  if (ph == PH_N) return;   // (the grid holds exactly the operations' workgroups)

  if (ph == PH_QKV) {
    qgemm_body<SV_B4_256, 2, MTP, SV_EPI_QKV, true, true>(
        a.w_qkv, a.nsb_h, a.ks[PH_QKV], a.sbps[PH_QKV], a.ap_h, a.sx_h, a.M, 0, 1, a.e_qkv, vb,
        wave, true, tid, 512, s_dyn, s_inv[0], [] {});
  } else if (ph == PH_ATT) {
    // two chunks per workgroup, four waves each
    typedef attn_lds<128, MTQ> LDS;
    const int half = wave >> 2;
    const int nitem = a.S * a.nkv * a.nch;
    int item = 2 * vb + half;
    int c = a.nch;                      // past every sequence: computes nothing
    int gk = 0, s = 0;
    if (item < nitem) {
      c = item % a.nch;
      item /= a.nch;
      gk = item % a.nkv;
      s = item / a.nkv;
    }
    LDS *sm = reinterpret_cast<LDS *>(s_dyn) + half;
    attn_chunk_body<128, MTQ, true>(c, gk, s, tid & 255, *sm, a.kc, a.vc, a.qpack, a.lens, a.err,
                                    a.nkv, a.cap, a.nt, a.G, a.scale, a.att_o, a.att_ml, a.nch,
                                    a.nts, [&] { wait_done(a, PH_QKV); });
  } else if (ph == PH_MERGE) {
    wait_done(a, PH_ATT);
    attn_merge_thread<128, true>(vb * 512 + tid, a.att_o, a.att_ml, a.lens, a.err, a.nts, a.nkv,
                                 a.nt, a.G, a.NQ, a.NQp, a.nch, a.nitems, a.ap_o, a.sx_o, a.Ko);
  } else if (ph == PH_O) {
    qgemm_body<SV_B4_256, 2, MTP, SV_EPI_RESID, true, true>(
        a.w_o, a.nsb_o, a.ks[PH_O], a.sbps[PH_O], a.ap_o, a.sx_o, a.M, 0, 1, a.e_o, vb, wave, true,
        tid, 512, s_dyn, s_inv[0], [&] { wait_done(a, PH_MERGE); });
  } else if (ph == PH_GU) {
    // two column groups per workgroup, four waves (K splits) each
    const int half = wave >> 2;
    const int grp = 2 * vb + half;
    const bool live = grp < a.ng_gu;
    const int ks = a.ks[PH_GU];
    qgemm_body<SV_B4_256, 4, MTP, SV_EPI_SWIGLU, true, true>(
        a.w_gu, a.nsb_h, ks, a.sbps[PH_GU], a.ap_h2, a.sx_h2, a.M, 0, 1, a.e_gu,
        live ? grp : 0, live ? (wave & 3) : ks, live, tid & 255, 256,
        s_dyn + half * a.lds_gu_floats, s_inv[half], [&] { wait_done(a, PH_O); });
  } else {
    qgemm_body<SV_B4_256, 2, MTP, SV_EPI_RESID, true, false>(
        a.w_down, a.nsb_f, a.ks[PH_DOWN], a.sbps[PH_DOWN], a.ap_f, a.sx_f, a.M, 0, 1, a.e_down, vb,
        wave, true, tid, 512, s_dyn, s_inv[0], [&] { wait_done(a, PH_GU); });
  }
  // finished: this workgroup's stores are performed, then it is counted
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_add(a.cnt + (1 + ph) * SV_LAYER_CSTRIDE, 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
#ifdef SV_LAYER_TRACE
  if (tid == 0 && a.layer < SV_TRACE_LAYERS && s_ticket < SV_TRACE_TICKETS) {
    long long *t = g_layer_trace[a.layer][s_ticket];
    t[0] = ph;
    t[1] = t_start;
    t[2] = s_twait;
    t[3] = __builtin_amdgcn_s_memrealtime();
  }
#endif
}

// LDS bytes of one launch: the largest operation (two chunk computations,
// two gate|up groups, or one group of the other projections).
template <int MTQ>
static size_t layer_lds_bytes(const sv_layer_args &a) {
  size_t b = 2 * sizeof(attn_lds<128, MTQ>);
  const size_t gu = 2 * sizeof(float) * (size_t)a.lds_gu_floats;
  for (size_t x : {gu, a.lds_qkv, a.lds_o, a.lds_down}) b = b > x ? b : x;
  return b;
}

template <int MTP, int MTQ>
static hipError_t launch_layer(const sv_layer_args &a, hipStream_t st) {
  int grid = 0;
  for (int p = 0; p < PH_N; ++p) grid += a.n_wg[p];
  hipLaunchKernelGGL((k_layer<MTP, MTQ>), dim3(grid), dim3(512), layer_lds_bytes<MTQ>(a), st, a);
  return hipGetLastError();
}

template <int MTP, int MTQ>
static hipError_t allow_layer_lds() {
  return hipFuncSetAttribute((const void *)k_layer<MTP, MTQ>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, SV_LAYER_MAX_LDS);
}

// One-time host setup (dynamic LDS limit), at model creation.
hipError_t sv_layer_prepare() {
  static bool done = false;
  if (done) return hipSuccess;
  hipError_t e = hipSuccess;
#define SV_LAYER_ALLOW(Q)                                      \
  if (e == hipSuccess) e = allow_layer_lds<SV_MT_PACK4, Q>();  \
  if (e == hipSuccess) e = allow_layer_lds<SV_MT_PACK8, Q>();  \
  if (e == hipSuccess) e = allow_layer_lds<1, Q>();
  SV_LAYER_ALLOW(1) SV_LAYER_ALLOW(2) SV_LAYER_ALLOW(3) SV_LAYER_ALLOW(4)
#undef SV_LAYER_ALLOW
  done = (e == hipSuccess);
  return e;
}

bool sv_layer_supported(int M, int MTQ) { return M >= 1 && M <= 16 && MTQ >= 1 && MTQ <= 4; }

hipError_t sv_launch_layer(const sv_layer_args &a, int MTQ, hipStream_t st) {
  if (!sv_layer_supported(a.M, MTQ)) return hipErrorInvalidValue;
  if (sizeof(float) * (size_t)a.lds_gu_floats * 2 > SV_LAYER_MAX_LDS ||
      a.lds_qkv > SV_LAYER_MAX_LDS || a.lds_o > SV_LAYER_MAX_LDS || a.lds_down > SV_LAYER_MAX_LDS)
    return hipErrorInvalidValue;
#define SV_LAYER_CASE(Q)                                                              \
  case Q:                                                                             \
    return a.M <= SV_APACK4_ROWS ? launch_layer<SV_MT_PACK4, Q>(a, st)                  \
           : a.M <= 8 ? launch_layer<SV_MT_PACK8, Q>(a, st)                             \
                      : launch_layer<1, Q>(a, st);
  switch (MTQ) {
    SV_LAYER_CASE(1) SV_LAYER_CASE(2) SV_LAYER_CASE(3) SV_LAYER_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef SV_LAYER_CASE
}
