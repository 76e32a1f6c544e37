// Verify attention: the nt query rows of every sequence (times the G query
// heads that share a KV head) against the fp16 cache, keys 0..len+r for row
// r (causal inside the block).
//
// Keys are split into fixed chunks of SV_ATT_CHUNK positions at absolute
// positions; a block computes one (sequence, kv head, chunk), one wave per
// 32 keys:
//   S^T = K Q^T     on the matrix cores (K rows exact fp16, Q as fp16 hi+lo)
//   m_c = max over the chunk's visible keys, p = exp(s - m_c)
//   l_c = sum p,    O_c = V^T P^T on the matrix cores (P as fp16 hi+lo)
// and a second kernel combines the chunks, o = sum_c w_c O_c / sum_c w_c l_c
// with w_c = e^(m_c - m) relative to the maximum of the chunks combined, in
// an order fixed by absolute chunk index (see k_attn_merge).
// A row never sees a chunk boundary or a reduction tree that depends on nt:
// keys it may not see contribute exact zeros (masked scores are -inf, fully
// masked chunks have l_c = 0 and O_c = 0), so row r has the same bits for
// every nt > r.
#include "sv_attn_body.h"
#include "sv_timeline.h"

// The merge, one thread per (item, lane) (see attn_merge_thread), one wave
// per block: its loads are a single round trip, and spread over one wave per
// CU instead of four they return sooner (eight items per block; 240 blocks
// for the 14B shapes at nt = 3 instead of 60 blocks of four waves).
#ifndef SV_MERGE_BLOCK
#define SV_MERGE_BLOCK 64
#endif
template <int HD>
__global__ __launch_bounds__(SV_MERGE_BLOCK) void k_attn_merge(const float *__restrict__ att_o,
                                                    const float *__restrict__ att_ml,
                                                    const int32_t *__restrict__ lens,
                                                    const int32_t *__restrict__ err,
                                                    const int32_t *__restrict__ nts, int nkv,
                                                    int nt, int G, int NQ, int NQp, int nch,
                                                    int nitems, uint8_t *__restrict__ ap_o,
                                                    uint8_t *__restrict__ sx_o, int Ko, int layer) {
#ifdef SV_TIMELINE
  const long long t0 = sv_tl_now();
#endif
  attn_merge_thread<HD, false>(blockIdx.x * blockDim.x + threadIdx.x, att_o, att_ml, lens, err,
                               nts, nkv, nt, G, NQ, NQp, nch, nitems, ap_o, sx_o, Ko);
#ifdef SV_TIMELINE
  __syncthreads();
  if (threadIdx.x == 0) {
    sv_tl_put(layer, SV_TL_MERGE, blockIdx.x, SV_TLF_START, t0);
    sv_tl_put(layer, SV_TL_MERGE, blockIdx.x, SV_TLF_END, sv_tl_now());
  }
#else
  (void)layer;
#endif
}

// One block per (kv head, key chunk, sequence), the kv head fastest: the
// workgroups dispatched last are the sequences' last chunks, which hold the
// fewest keys (the block's own rows at most), so the few CUs that take a
// second workgroup take a light one; and a kv head's chunks, which share its
// query operand, go to one XCD (workgroups are dealt to the XCDs in turn).
template <int HD, int MTQ>
__global__ __launch_bounds__(64 * SV_ATT_NWV) void k_attn_chunk(const uint16_t *__restrict__ kc,
                                                    const uint16_t *__restrict__ vc,
                                                    const uint8_t *__restrict__ qpack,
                                                    const int32_t *__restrict__ lens,
                                                    const int32_t *__restrict__ err, int nkv,
                                                    int cap, int nt, int G, float scale,
                                                    float *__restrict__ att_o,
                                                    float *__restrict__ att_ml, int nch,
                                                    const int32_t *__restrict__ nts, int layer) {
  __shared__ attn_lds<HD, MTQ> sm;
#ifdef SV_TIMELINE
  const long long t0 = sv_tl_now();
#endif
  attn_chunk_body<HD, MTQ, false>(blockIdx.y, blockIdx.x, blockIdx.z, threadIdx.x, sm, kc, vc,
                                  qpack, lens, err, nkv, cap, nt, G, scale, att_o, att_ml, nch,
                                  nts, [] {});
#ifdef SV_TIMELINE
  __syncthreads();
  if (threadIdx.x == 0) {
    const int b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    sv_tl_put(layer, SV_TL_CHUNK, b, SV_TLF_START, t0);
    sv_tl_put(layer, SV_TL_CHUNK, b, SV_TLF_END, sv_tl_now());
  }
#else
  (void)layer;
#endif
}

template <int HD>
static hipError_t launch_attn_hd(int MTQ, const uint16_t *kc, const uint16_t *vc,
                                 const uint8_t *qpack, const int32_t *lens, const int32_t *err,
                                 int S, int nkv, int cap, int nt, int G, float *att_o,
                                 float *att_ml, int nch, uint8_t *ap_o, uint8_t *sx_o, int Ko,
                                 const int32_t *nts, hipStream_t st, int layer) {
  dim3 grid(nkv, nch, S), block(64 * SV_ATT_NWV);
  const float scale = 1.0f / sqrtf((float)HD);
#define SV_ATT_CASE(N)                                                                       \
  case N:                                                                                    \
    hipLaunchKernelGGL((k_attn_chunk<HD, N>), grid, block, 0, st, kc, vc, qpack, lens, err, \
                       nkv, cap, nt, G, scale, att_o, att_ml, nch, nts, layer);             \
    break;
  switch (MTQ) {
    SV_ATT_CASE(1) SV_ATT_CASE(2) SV_ATT_CASE(3) SV_ATT_CASE(4) SV_ATT_CASE(5)
    SV_ATT_CASE(6) SV_ATT_CASE(7)
    default: return hipErrorInvalidValue;
  }
#undef SV_ATT_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int NQ = nt * G;
  const int nitems = S * nkv * NQ * (HD / 8);
  const int nthr = 8 * nitems;
  hipLaunchKernelGGL((k_attn_merge<HD>), dim3((nthr + SV_MERGE_BLOCK - 1) / SV_MERGE_BLOCK),
                     dim3(SV_MERGE_BLOCK), 0, st, att_o,
                     att_ml, lens, err, nts, nkv, nt, G, NQ, 16 * MTQ, nch, nitems, ap_o, sx_o,
                     Ko, layer);
  return hipGetLastError();
}

// Bytes of one (sequence, kv head)'s chunk slots: the chunk kernel
// addresses them with 32-bit offsets from the region's own base.
size_t sv_attn_region_bytes(int hd, int MTQ, int nch) {
  return (size_t)nch * MTQ * 16 * hd * sizeof(float);
}

hipError_t sv_launch_attn(int hd, int MTQ, const uint16_t *kc, const uint16_t *vc,
                          const uint8_t *qpack, const int32_t *lens, const int32_t *err,
                          int S, int nkv, int cap, int nt, int G, float *att_o,
                          float *att_ml, int nch, uint8_t *ap_o, uint8_t *sx_o, int Ko,
                          const int32_t *nts, hipStream_t st, int layer) {
  if (hd == 128)
    return launch_attn_hd<128>(MTQ, kc, vc, qpack, lens, err, S, nkv, cap, nt, G, att_o,
                               att_ml, nch, ap_o, sx_o, Ko, nts, st, layer);
  if (hd == 64)
    return launch_attn_hd<64>(MTQ, kc, vc, qpack, lens, err, S, nkv, cap, nt, G, att_o,
                              att_ml, nch, ap_o, sx_o, Ko, nts, st, layer);
  return hipErrorInvalidValue;
}

#ifdef SV_TIMELINE
SV_TL_READER(sv_timeline_read_attn)
#endif
