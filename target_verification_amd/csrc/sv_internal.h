// Host-side internal definitions: repacked weights, the model, the workspace
// carve-up, and the launch wrappers each kernel file provides.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"

// Repacked ("tile-block") weight layout.  Output features are grouped in
// tiles of 16; K in super-blocks of 256.  Tile t, super-block sb occupies
// tb_bytes at data + (t * nsb + sb) * tb_bytes:
//
//  B4_256 (2304 B): [16 columns x 16 B scale records][2 x 1024 B codes]
//     record: d fp16 | dmin fp16 | two dwords of 6-bit sub-block scales and
//     the high 2 bits of the 6-bit mins | the mins' low nibbles (bit layout
//     in the repack).  Codes: chunk h, lane l (column l%16, k-octet g = l/16),
//     dword i = k-step 4h+i holding the 8 codes k = 32*ks + 8g + s, slot s
//     at bit 4*(s/2) + 16*(s%2).
//  B4_32  (2304 B): [16 columns x 8 fp16 block scales][codes as B4_256]
//  B6_256 (3360 B): [16 x 16 B int8 sc][16 x fp16 d][low nibbles: 2 x 1024 B
//     as B4_256][high bits: 1024 B, lane l dword i = k-steps 2i, 2i+1; k-step
//     parity a at bits 8a..8a+7 and 16+8a.., slot s at bit 8a + 2*(s/2) +
//     16*(s%2)].
enum { SV_TB_B4 = 2304, SV_TB_B6 = 3360 };

// M-tile arrangement of the small-row GEMM (its template argument MTP): 1 or
// 2 sixteen-row M-tiles; SV_MT_PACK8: one tile of at most 8 rows whose
// activation high parts fill MFMA rows 0-7 and low parts rows 8-15;
// SV_MT_PACK4: the same for at most 4 rows, two k-steps per activation load.
enum { SV_MT_PACK8 = 0, SV_MT_PACK4 = 3 };

#ifndef SV_KV_CHUNK
#define SV_KV_CHUNK 128   // KV capacity granularity (positions)
#endif
#ifndef SV_ATT_CHUNK
#define SV_ATT_CHUNK 128  // attention key chunk at absolute positions (64 or 128)
#endif
static_assert(SV_ATT_CHUNK == 64 || SV_ATT_CHUNK == 128,
              "attention chunks of 64 or 128 keys (the capacity is a multiple of 128)");

// SV_EPI_ANY: a kernel that reads the epilogue type from its arguments
enum { SV_EPI_ANY = 0, SV_EPI_QKV = 1, SV_EPI_RESID = 2, SV_EPI_SWIGLU = 3, SV_EPI_LM = 4,
       SV_EPI_PLAIN = 5 };

struct sv_qweight {
  int32_t type;       // sv_qtype
  int64_t rows, cols; // N (output features, after any interleave), K
  int32_t nsb, ntile, tb_bytes;
  uint8_t *data;
  // work decomposition, a function of (rows, cols) only: tiles per group
  // (one workgroup), K splits (one wave each) of sbps super-blocks
  int32_t tpw, ngroups, ksplit, sbps;
};

struct sv_model {
  sv_model_desc d;   // copy; host pointer arrays cleared
  int32_t L, H, nq, nkv, hd, F, V, G;
  sv_qweight *qkv, *wo, *gu, *down;  // [L]; qkv rows permuted for RoPE pairs, gu interleaved
  sv_qweight lm;
  float *rope;       // device [max_pos][hd/2][2] (cos, sin), fp32 from fp64
};

// Workspace carve-up of one round.
struct sv_ws {
  int32_t *err;        // [S]  device-side error word per sequence
  int32_t *oldlen;     // [S]
  int32_t *argmax;     // [Mp]
  float *x;            // [Mp][H]
  float *x1;           // [Mp][H]  residual stream after the O projection (fused layer)
  uint8_t *ap_h2, *sx_h2;  // gate|up operand (fused layer)
  float *ssq2;         // [Mp][H/32] its sums of squares (fused layer)
  int32_t *lcnt;       // fused layer: SV_LAYER_NCNT counters per layer
  uint8_t *ap_h, *sx_h;  // activation operand for K = H
  uint8_t *ap_o, *sx_o;  // K = nq*hd
  uint8_t *ap_f, *sx_f;  // K = F
  float *ssq;          // [Mp][H/32]   32-column sums of squares
  float *rinv;         // [Mp]         row scales (wide-M GEMM)
  uint8_t *qpack;      // attention query operand
  float *att_o;        // [S][nkv][nch][NQp][hd]
  float *att_ml;       // [S][nkv][nch][NQp][2]
  float *lm_part;      // greedy: [M][NGlm] (max, argmax as bits)
  double *lm_stat;     // reject: [M][NGlm][2]
  double *dr_stat;     // reject: [S][nt-1][NGlm][2]
  double *rj_stat;     // reject: [S][2 nt - 1][2] row (max, sum) of target then draft rows
  double *rj_sum;      // reject: [S][SV_RJ_NB][2] slice sums of the residual and of p;
                       // sample: [S][nt][SV_RJ_NB][2] slice sums of p per row
  float *logits;       // reject without caller logits: [M][V]
  int32_t *cnt;        // arrival counters: attention, then decision
  int32_t *dcnt;       // decision: one counter per sequence
  int32_t *amb;        // decision: per-row argmax [Mp]
  int ncnt;            // total counters (zeroed at the start of a round)
};

struct sv_dims {       // per-round sizes
  int S, nt, M, MT, Mp;      // rows M = S*nt, MT = ceil(M/16), Mp = 16*MT
  int NQ, MTQ, nch;          // attention query rows per (s, kv head), tiles, key chunks
  int NGlm;                  // lm_head column groups (32 columns each)
};

// ---- launch wrappers (each returns hipError_t of the launch) ---------------
hipError_t sv_launch_repack(int type, const uint8_t *const *srcs_dev, const int32_t *rowmap,
                            int64_t nrows, int nsb, uint8_t *dst, hipStream_t st);

// Kernel classes of the timeline measurement build (sv_timeline.h).
enum { SV_TL_QKV = 0, SV_TL_CHUNK, SV_TL_MERGE, SV_TL_O, SV_TL_GU, SV_TL_DOWN, SV_TL_LM };

struct sv_epi_args {
  int type;            // SV_EPI_*
  int M, Mp, S, nt, H;
  int ksplit, C, ngroups;   // the GEMM's K splits, columns per group, groups
  // deferred norm of the GEMM input (ssq partials) or NULL (scale 1)
  const float *ssq; int nssq; int normH; float eps;
  const float *rowscale;  // explicit per-row scale (overrides ssq) or NULL
  float *rinv;            // [Mp] scratch: row scales for the wide-M GEMM
  // QKV
  int layer, nq, nkv, hd, G, cap, MTQ;
  int tl_kind;   // kernel class (SV_TL_*) in the timeline build (sv_timeline.h)
  const int32_t *lens; int32_t *err; const int32_t *nts;
  const float *rope; uint16_t *kc, *vc; uint8_t *qpack;
  // residual / producer for the next GEMM (the residual epilogue reads x
  // and writes x_out, or x when x_out is NULL)
  float *x; float *x_out; const float *gnext; uint8_t *ap_next, *sx_next; float *ssq_next; int Knext;
  // lm head
  float *logits; float *lm_part; double *lm_stat; double *dr_stat;
  const float *draft_logits; int V; float temperature; int reject;
};

// ---- the fused layer kernel (sv_layer.hip) ----------------------------------
#define SV_LAYER_NCNT 8   // per layer: ticket, six finished counts, spare
#ifndef SV_LAYER_CSTRIDE
#define SV_LAYER_CSTRIDE 64   // ints between counters: each on a cache line of its own
#endif
struct sv_layer_args {
  int32_t *cnt;               // this layer's SV_LAYER_NCNT counters, SV_LAYER_CSTRIDE apart
                              // (zero on entry)
  int32_t *err; int S;        // sequence error words (a wait that expires fails them all)
  int layer;
  int M;                      // rows (at most 16)
  // projections: repacked weights, super-blocks along K, K splits and
  // super-blocks per split, by operation (qkv, -, -, o, gate|up, down)
  const uint8_t *w_qkv, *w_o, *w_gu, *w_down;
  int nsb_h, nsb_o, nsb_f;
  int ks[6], sbps[6];
  int ng_gu;                  // gate|up column groups
  // activation operands: layer input, attention output, gate|up input, down input
  const uint8_t *ap_h, *sx_h, *ap_h2, *sx_h2, *ap_f, *sx_f;
  uint8_t *ap_o, *sx_o;       // written by the merge, read by the O projection
  sv_epi_args e_qkv, e_o, e_gu, e_down;
  // attention
  const uint16_t *kc, *vc;    // this layer's cache
  const uint8_t *qpack;
  const int32_t *lens, *nts;
  int nkv, cap, nt, G, nch, NQ, NQp, nitems, Ko;
  float scale;
  float *att_o, *att_ml;
  int n_wg[6];                // workgroups per operation
  int lds_gu_floats;          // LDS of one gate|up group (floats)
  size_t lds_qkv, lds_o, lds_down;
};
// Whether the fused layer kernel serves M rows with MTQ query tiles.
bool sv_layer_supported(int M, int MTQ);
hipError_t sv_launch_layer(const sv_layer_args &a, int MTQ, hipStream_t st);
hipError_t sv_layer_prepare();
size_t sv_gemm_lds_bytes(int ksplit, int MT, int TPW, const sv_epi_args &ea);

// GEMM over M-tiles [mt0, mt0 + mtn) followed by the epilogue ea for those
// rows: one workgroup per column group, one wave per K split (ksplit <= 8).
hipError_t sv_launch_qgemm(const sv_qweight *w, const uint8_t *apack, const uint8_t *sxpack,
                           int M, int mt0, int mtn, const sv_epi_args &ea, hipStream_t st);
hipError_t sv_launch_zero(int32_t *p, int n, hipStream_t st);
// One-time host setup of the GEMM kernels (dynamic LDS limit).
hipError_t sv_gemm_prepare();


// Per-sequence error word bits: SV_ERRB_CAPACITY (len + rows past the
// capacity), SV_ERRB_INVALID (a bad id or row count), SV_ERRB_NUMERIC (a
// non-finite logit or draft logit).  A sequence with any bit set is not
// decided and not committed; its accepted_len receives sv_err_status().
// SV_ERRB_TIMEOUT: a bounded wait of the fused layer kernel expired.
enum { SV_ERRB_CAPACITY = 1, SV_ERRB_INVALID = 2, SV_ERRB_NUMERIC = 4, SV_ERRB_TIMEOUT = 8 };
__host__ __device__ inline int32_t sv_err_status(int32_t e) {
  if (e & SV_ERRB_TIMEOUT) return SV_E_TIMEOUT;
  return (e & SV_ERRB_CAPACITY) ? SV_E_CAPACITY
                                : ((e & SV_ERRB_INVALID) ? SV_E_INVALID : SV_E_NUMERIC);
}

// Per-sequence error words and saved lengths; also zeroes ncnt counters.
hipError_t sv_launch_init(const int32_t *lens, const int32_t *nts, int32_t *err,
                          int32_t *oldlen, int S, int nt, int cap, int maxlen, int32_t *cnt,
                          int ncnt, hipStream_t st);
hipError_t sv_launch_embed(const int32_t *ids, const uint16_t *tok, const float *hidden,
                           const float *gamma, int M, int H, float *x, uint8_t *ap,
                           uint8_t *sx, float *ssq, int nt, int V, int32_t *err,
                           const int32_t *nts, hipStream_t st);
// Attention: the chunk kernel (one slot per key chunk), then the merge
// kernel into the O projection's operand.  The chunk slots of one
// (sequence, kv head) must stay under 2^31 bytes (sv_attn_region_bytes).
size_t sv_attn_region_bytes(int hd, int MTQ, int nch);
hipError_t sv_launch_attn(int hd, int MTQ, const uint16_t *kc, const uint16_t *vc,
                          const uint8_t *qpack, const int32_t *lens, const int32_t *err,
                          int S, int nkv, int cap, int nt, int G, float *att_o,
                          float *att_ml, int nch, uint8_t *ap_o, uint8_t *sx_o, int Ko,
                          const int32_t *nts, hipStream_t st, int layer = -1);
// One block per row finds the row's argmax; the last row block of a
// sequence decides (amb: [M] row argmaxes, dcnt: S counters, zero on entry).
hipError_t sv_launch_greedy(const float *lm_part, int NG, const int32_t *ids, int S, int nt,
                            int32_t *err, int32_t *lens, int32_t *oldlen, int32_t *acc,
                            int32_t *emitted, int32_t *argmax_out, int commit, int32_t *amb,
                            int32_t *dcnt, const int32_t *nts, hipStream_t st);
// strict rejection sampling: vocabulary slices per sequence
#define SV_RJ_NB 32
hipError_t sv_launch_reject(const double *lm_stat, const double *dr_stat, double *rj_stat,
                            double *rj_sum, int NG,
                            const float *logits, const float *draft_logits,
                            const double *uniforms, const int32_t *ids, int S, int nt,
                            int V, float T, int32_t *err, int32_t *lens, int32_t *oldlen,
                            int32_t *acc, int32_t *emitted, int commit, const int32_t *nts,
                            hipStream_t st);
// Exact-match sampled verify: one block per row draws the row's token by
// inverse CDF (argmax_out, if not NULL, receives the draws); the last row
// block of a sequence decides (amb: [M] draws, dcnt: S counters, zero on
// entry).
hipError_t sv_launch_sample(const double *lm_stat, double *rj_stat, double *rj_sum, int NG,
                            const float *logits,
                            const double *uniforms, const int32_t *ids, int S, int nt, int V,
                            float T, int32_t *err, int32_t *lens, int32_t *oldlen, int32_t *acc,
                            int32_t *emitted, int32_t *draws_out, int commit, int32_t *amb,
                            int32_t *dcnt, const int32_t *nts, hipStream_t st);
hipError_t sv_launch_advance(const sv_advance_args &a, hipStream_t st);
hipError_t sv_launch_poison(uint16_t *kc, uint16_t *vc, const int32_t *lens,
                            const int32_t *oldlen, const int32_t *err, int L, int S, int nkv,
                            int cap, int hd, int nt, const int32_t *nts, hipStream_t st);
