// Measurement build only (compiled with -DSV_TIMELINE): each GEMM and
// attention workgroup records the GPU's real-time counter (100 MHz) per
// (layer, kernel class, workgroup): at its start and its end, and for the
// small-row GEMMs also at the end of its main loop (the latest of its
// waves), when wave 0 has its staged rows and norm factors, after the
// workgroup barrier that joins the K splits, when thread 0 has issued the
// epilogue's stores and when those are acknowledged.  Every translation
// unit that records holds its own copy of the table and exports a reader;
// nothing here changes what the kernels compute.
#pragma once
#ifdef SV_TIMELINE
#include <hip/hip_runtime.h>
#include "sv_internal.h"

#define SV_TL_LAYERS 64
#define SV_TL_KINDS 7   // q|k|v, attention chunks, merge, o, gate|up, down, lm_head
#define SV_TL_WG 1024

// fields of a record
enum { SV_TLF_START = 0, SV_TLF_LOOP = 1, SV_TLF_END = 2, SV_TLF_STAGED = 3, SV_TLF_EPI = 4,
       SV_TLF_BARRIER = 5, SV_TLF_STORED = 6, SV_TL_FIELDS = 7 };

static __device__ long long g_sv_tl[SV_TL_LAYERS][SV_TL_KINDS][SV_TL_WG][SV_TL_FIELDS];

__device__ __forceinline__ long long sv_tl_now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ bool sv_tl_slot(int layer, int kind, int wg) {
  return layer >= 0 && layer < SV_TL_LAYERS && kind >= 0 && kind < SV_TL_KINDS && wg < SV_TL_WG;
}

__device__ __forceinline__ void sv_tl_put(int layer, int kind, int wg, int field, long long t) {
  if (sv_tl_slot(layer, kind, wg)) g_sv_tl[layer][kind][wg][field] = t;
}
__device__ __forceinline__ void sv_tl_max(int layer, int kind, int wg, int field, long long t) {
  if (sv_tl_slot(layer, kind, wg))
    atomicMax((unsigned long long *)&g_sv_tl[layer][kind][wg][field], (unsigned long long)t);
}

#define SV_TL_READER(NAME)                                                               \
  extern "C" int NAME(void *host, size_t bytes) {                                        \
    if (bytes != sizeof(g_sv_tl)) return -1;                                             \
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_sv_tl), sizeof(g_sv_tl)) == hipSuccess \
               ? 0                                                                       \
               : -1;                                                                     \
  }
#endif
