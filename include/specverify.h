/*
 * specverify.h -- C ABI of the batched target-verify round of speculative
 * decoding on AMD MI355X (gfx950).
 *
 * One call evaluates the anchor token plus d drafted tokens (nt = d + 1 rows
 * per sequence) through the target model in one pass that streams the
 * block-quantized weights once, computes the lm_head logits, decides per row
 * (greedy argmax or strict rejection sampling), returns the accepted length
 * and the one correction/bonus token, and commits the KV length on the
 * device.  Sources: the round order of the Power page ("Model-neutral
 * Speculative Decoding", section "The exactness transaction"); the one-round
 * mechanism of the minfer plan ("Speculative Decoding (D5-R) -- Plan",
 * section 3 "Mechanism -- one round"), where rejected KV rows are not copied
 * back but simply overwritten next round; the strict rejection sampler named
 * on the DFlash/DSpark wiki page ("DFlash and DSpark Speculative Decoding",
 * "How DSpark Works", "Notes").
 *
 * Conventions shared by every entry point:
 *  - Pointers documented as "device" point to GPU memory owned by the caller
 *    (for example PyTorch tensors); "host" pointers are read during the call
 *    only.  The library never keeps a caller pointer beyond the documented
 *    lifetime (sv_model borrows the norm gains and the token table for its own
 *    lifetime).
 *  - Errors are integer status codes (sv_status); no exception crosses the
 *    ABI.  Argument and shape checks run before anything is enqueued, and an
 *    unsupported format, mode or size fails closed (SV_E_UNSUPPORTED) rather
 *    than falling back to another path.
 *  - spec_verify_round is asynchronous: it enqueues kernels on `stream` and
 *    returns; outputs are valid once the caller has synchronized the stream.
 *    It never synchronizes, allocates or frees, so it may be captured into a
 *    HIP graph.
 *
 * Canonical block formats (weights row-major over output features; each row
 * is cols/block_size blocks in order of k):
 *  SV_B4_32  (32 weights, 18 B): d fp16 | 16 B codes (code k in byte k/2,
 *            low nibble for even k).  w_k = d * (q_k - 8).
 *  SV_B4_256 (256 weights, 144 B): d fp16 | dmin fp16 | 12 B = sixteen 6-bit
 *            fields, LSB-first bitstream (sc_0..sc_7 then m_0..m_7) | 128 B
 *            codes as above.  Sub-block j = k/32.  w_k = d*sc_j*q_k - dmin*m_j.
 *  SV_B6_256 (256 weights, 210 B): 128 B low nibbles as above | 64 B high
 *            2-bit fields (code k's bits 4..5 at byte k/4, bit 2*(k%4)) |
 *            16 B int8 sc_j | d fp16.  Sub-block j = k/16.
 *            w_k = d*sc_j*(q_k - 32).
 *  Every inner dimension (hidden, n_head*head_dim, ffn) must be a multiple
 *  of 256 and every output dimension a multiple of 256, with hidden at most
 *  8192; other shapes return SV_E_UNSUPPORTED.
 *
 * KV cache layout (fp16, caller-owned, device):
 *  k: [n_layer][n_seq][n_kv_head][capacity][head_dim]
 *  v: [n_layer][n_seq][n_kv_head][head_dim][capacity]   (transposed)
 *  len: int32 [n_seq], the committed length of every sequence.
 *  Rows at positions >= len are dead: a round writes rows len..len+nt-1 and
 *  commits len + a + 1, so rejected rows are overwritten by the next round.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_E_INVALID = -1,      /* bad argument: NULL pointer, size or shape mismatch */
  SV_E_UNSUPPORTED = -2,  /* well-formed but not provided (format, nt, mode) */
  SV_E_CAPACITY = -3,     /* len + nt would exceed the KV capacity */
  SV_E_HIP = -4,          /* a HIP runtime call failed */
  SV_E_FAULT_INJECTED = -5, /* SV_FAULT=after_verify was set (tests only) */
  SV_E_NOMEM = -6,        /* model creation could not allocate */
  SV_E_NUMERIC = -7,      /* a logit or draft logit of the sequence was NaN or infinite:
                             the sequence is not decided and not committed */
  SV_E_TIMEOUT = -8       /* a bounded device-side wait between the operations of a layer
                             expired: the round is not decided and not committed */
} sv_status;

typedef enum { SV_B4_32 = 1, SV_B4_256 = 2, SV_B6_256 = 3 } sv_qtype;
/* SV_GREEDY: accept while each row's argmax equals the next draft (lowest id
 *   among equal maxima); emit the argmax of the first mismatching row.
 * SV_REJECT: strict rejection sampling against draft probabilities.
 * SV_SAMPLE: exact-match sampled verify (the Power page, "The exactness
 *   transaction", step 4 and the sampler-state rule after it): every row r
 *   draws the token at position len + r + 1 from softmax(logits_r / T) by
 *   inverse CDF with its own pre-generated uniform; drafts are accepted
 *   while equal to those draws, and the draw of the first mismatching row
 *   (or of row nt - 1) is emitted.  With uniforms keyed by absolute position
 *   the committed stream equals seeded one-token-at-a-time sampling. */
typedef enum { SV_GREEDY = 0, SV_REJECT = 1, SV_SAMPLE = 2 } sv_mode;

#define SV_MAX_NT 16

/* Model description.  Device pointers are borrowed by sv_model for its
 * lifetime, except the quantized tensors, which sv_model_create repacks into
 * memory it owns (the canonical bytes may be freed after creation). */
typedef struct {
  int32_t n_layer, hidden, n_head, n_kv_head, head_dim, ffn, vocab, max_pos;
  float rms_eps;     /* RMSNorm epsilon */
  float rope_base;   /* RoPE base; pair (i, i + head_dim/2) rotates by pos * base^(-2i/head_dim) */
  int32_t fmt_proj;  /* sv_qtype of every projection */
  int32_t fmt_lm;    /* sv_qtype of the lm_head */
  int32_t lm_only;   /* 1: no layers; rounds pass final hidden states (sv_round.hidden) */
  int32_t reserved;
  const uint16_t *tok_embd;   /* device fp16 [vocab][hidden]; NULL if lm_only */
  const float *attn_norm;     /* device fp32 [n_layer][hidden] */
  const float *ffn_norm;      /* device fp32 [n_layer][hidden] */
  const float *out_norm;      /* device fp32 [hidden]; NULL if lm_only */
  /* host arrays of n_layer device pointers to canonical bytes */
  const void *const *wq, *const *wk, *const *wv, *const *wo;
  const void *const *w_gate, *const *w_up, *const *w_down;
  const void *lm_head;        /* device canonical bytes [vocab][hidden] */
} sv_model_desc;

typedef struct sv_model sv_model;

/* capacity: positions per (layer, sequence, kv head); a multiple of 128, at
 * least 128 and at most the model's max_pos (else SV_E_UNSUPPORTED /
 * SV_E_INVALID).  The attention chunk results of one (sequence, kv head),
 * capacity / 128 * 16 * ceil(nt * G / 16) * head_dim * 4 bytes with
 * G = n_head / n_kv_head, must stay below 2^31 (else SV_E_UNSUPPORTED). */
typedef struct {
  int32_t n_seq, capacity;
  uint16_t *k;   /* device fp16, layout in the file header */
  uint16_t *v;   /* device fp16, layout in the file header */
  int32_t *len;  /* device int32 [n_seq] */
} sv_kv;

typedef struct {
  int32_t n_seq, nt;         /* nt = d + 1, 1 <= nt <= SV_MAX_NT; with layers, nt * G <= 112
                                (G = n_head / n_kv_head), else SV_E_UNSUPPORTED */
  int32_t mode;              /* sv_mode */
  float temperature;         /* > 0 in SV_REJECT and SV_SAMPLE, ignored in SV_GREEDY */
  const int32_t *ids;        /* device [n_seq][nt]: [0] anchor, [1..nt-1] drafts */
  const float *hidden;       /* device fp32 [n_seq][nt][hidden]: lm_only models only */
  const float *draft_logits; /* device fp32 [n_seq][nt-1][vocab]: SV_REJECT only (NULL
                                otherwise) */
  const double *uniforms;    /* device fp64 [n_seq][nt] in [0, 1).  SV_REJECT: [r < nt-1]
                                acceptance draw of draft row r, [nt-1] residual/bonus
                                draw.  SV_SAMPLE: [r] the draw of row r.  NULL in
                                SV_GREEDY */
  int32_t *accepted_len;     /* device out [n_seq]: a (negative sv_status on a device-side error) */
  int32_t *emitted;          /* device out [n_seq]: the correction or bonus token */
  float *logits;             /* device out fp32 [n_seq][nt][vocab], or NULL */
  int32_t *argmax;           /* device out [n_seq][nt] or NULL: the row argmaxes (SV_GREEDY)
                                or the row draws (SV_SAMPLE); unused in SV_REJECT */
  int32_t commit;            /* 1: len += a + 1 on the device; 0: dry run */
  int32_t max_len;           /* 0, or a host-known upper bound on every sequence's len at
                                this round (>= 0, else SV_E_INVALID).  Attention then visits
                                only the key chunks below max_len + nt, instead of the
                                whole capacity: its work and traffic follow the lengths
                                rather than the cache size.  A sequence whose len exceeds
                                it fails on the device with SV_E_INVALID (no KV write, no
                                commit).  For a captured graph replayed over several
                                committing rounds, pass the largest len it can reach. */
  const int32_t *nts;        /* device [n_seq] or NULL: ragged rounds.  Sequence s verifies
                                its first nts[s] rows (1 <= nts[s] <= nt; the anchor and
                                nts[s] - 1 drafts); its rows past that are padding: their ids
                                are not read as tokens, they write no cache row and they do
                                not take part in the decision (SV_REJECT: uniforms[s][r <
                                nts[s] - 1] test draft rows, [nts[s] - 1] is the residual
                                draw).  The capacity check is len + nts[s] <= capacity; an
                                nts[s] out of range is a device-side SV_E_INVALID for that
                                sequence.  NULL: every sequence has nt rows. */
} sv_round;

/* Build a model on the current HIP device: validates the description,
 * allocates device memory for the repacked weights and the RoPE table
 * (built on the host in fp64, stored fp32), repacks, and synchronizes.
 * Returns SV_OK and *out, or an error and *out = NULL. */
int sv_model_create(const sv_model_desc *desc, sv_model **out);
void sv_model_destroy(sv_model *m);

/* Device workspace bytes spec_verify_round needs for (n_seq, nt, mode).  The
 * attention part is sized for a cache of the model's max_pos positions, so
 * one workspace serves every cache capacity the model accepts. */
size_t sv_workspace_bytes(const sv_model *m, int32_t n_seq, int32_t nt, int32_t mode);

/* One verify round (see the file header).  `workspace` is caller-owned
 * device memory of at least sv_workspace_bytes(); it need not be zeroed.
 * The stream is a hipStream_t (NULL for the default stream).
 * On an error returned here nothing was enqueued, with one exception for
 * tests: with the environment variable SV_FAULT=after_verify the call
 * enqueues the forward pass and the lm_head, then returns
 * SV_E_FAULT_INJECTED without enqueueing the decision and the commit (len
 * stays unchanged; accepted_len, emitted and argmax are not written).  Errors found on the device
 * fail only the sequence concerned: its accepted_len receives the negative
 * status, its emitted token is -1 and its len is not committed --
 * SV_E_CAPACITY (len + nt > capacity; every KV write of the sequence is
 * skipped), SV_E_INVALID (an id outside [0, vocab), a bad nts entry, or len above a
 * nonzero max_len),
 * SV_E_NUMERIC (a NaN or infinite logit or draft logit).
 * With the environment variable SV_FUSED_LAYER=1, rounds of at most 16 rows
 * of a 4-bit/256 model with 128-dim heads run each decoder layer as one
 * launch (same results, bit for bit; slower on MI355X, kept for
 * comparisons); a device-side wait of that launch that expires fails every
 * sequence of the round with SV_E_TIMEOUT. */
int spec_verify_round(const sv_model *m, const sv_kv *kv, const sv_round *r,
                      void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * round as spec_verify_round, with the same kernels, arguments and results,
 * but its workspace is the library's own scratch array of
 * SV_STATIC_SCRATCH_BYTES on the current device (one array per device, kept
 * until the process ends; its address is located once per device, at model
 * creation or on the first call).  The call allocates and frees nothing.
 * The workspace is laid out for kv->capacity (not max_pos), or for the key
 * chunks below r->max_len + nt when a length bound is given, and the
 * stochastic modes keep logits in the scratch only when r->logits is NULL.
 * A round whose workspace would exceed SV_STATIC_SCRATCH_BYTES returns
 * SV_E_UNSUPPORTED before anything is enqueued.  Every call on one device
 * shares that device's array and leaves its contents behind (a round clears
 * what it needs zeroed itself): calls that overlap on one device -- on
 * different streams, or from different host threads without ordering --
 * race and give undefined results.  Other errors as spec_verify_round. */
#define SV_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int spec_verify_round_static(const sv_model *m, const sv_kv *kv, const sv_round *r,
                             void *stream);

/* ---- device-resident multi-round loop -----------------------------------
 * After a committed round (commit = 1), sv_advance turns its outcome into the
 * next round's input on the device, so rounds can run back to back (or be
 * replayed from one captured HIP graph) without the host reading anything.
 * Positions are data (the minfer plan, section 3 "Mechanism -- one round"):
 * the round committed the anchor and a drafts at positions len_old ..
 * len_old + a, and the emitted token is the next anchor, at position
 * len = len_old + a + 1.  Per sequence s (a = accepted_len[s] >= 0):
 *   tokens[s][len_old + 1 + j] = ids[s][1 + j] for j < a, tokens[s][len] =
 *     emitted[s]  (the committed stream by absolute position; skipped where
 *     the position is >= tok_cap, or when tokens is NULL);
 *   committed[s] += a + 1 (when committed is not NULL);
 *   ids[s][0] = emitted[s]; ids[s][1 + j] = the stub drafter's proposal for
 *     position P = len + 1 + j: ref[s][P] when draw[s][P] < p_accept *
 *     p_decay^j, else noise[s][P] (the DFlash/DSpark page, "Is it worth it?",
 *     step 4, projects a drafter by synthetic per-depth acceptance rates;
 *     here the rates apply to a reference stream such as the target's own
 *     output).  ref NULL:
 *     noise only.  Positions >= ref_cap propose token 0;
 *   uniforms[s][r] = utab[s][len + r + 1] when utab is not NULL: the next
 *     round's SV_SAMPLE draws, from a table of draws by absolute position
 *     (0.0 past ref_cap), so the sampler advances once per emitted token.
 * A sequence whose accepted_len is negative (a device-side error) is left
 * unchanged.  All pointers are device pointers owned by the caller; ids is
 * updated in place.  Asynchronous on `stream`; returns SV_E_INVALID for bad
 * arguments (nothing enqueued). */
typedef struct {
  int32_t n_seq, nt;
  int32_t *ids;                 /* [n_seq][nt], in: the round's ids; out: the next round's */
  const int32_t *accepted_len;  /* [n_seq] from the round */
  const int32_t *emitted;       /* [n_seq] from the round */
  const int32_t *len;           /* [n_seq] committed lengths after the round */
  int32_t *tokens;              /* [n_seq][tok_cap] or NULL */
  int32_t tok_cap;
  int32_t *committed;           /* [n_seq] running count, or NULL */
  const int32_t *ref;           /* [n_seq][ref_cap] or NULL */
  const float *draw;            /* [n_seq][ref_cap] uniforms in [0, 1); NULL iff ref is NULL */
  const int32_t *noise;         /* [n_seq][ref_cap] token ids */
  int32_t ref_cap;
  float p_accept, p_decay;
  const double *utab;           /* [n_seq][ref_cap] draws by position, or NULL */
  double *uniforms;             /* [n_seq][nt] out (with utab), or NULL */
} sv_advance_args;
int sv_advance(const sv_advance_args *a, void *stream);

/* ---- adaptive draft depth (host only; no GPU call) ----------------------
 * A policy that picks the next round's draft depth d (nt = d + 1) from the
 * acceptance observed per depth and the round times measured per nt (the
 * minfer plan's status notes, doc 95).  Draft j's conditional acceptance is
 * Beta(prior_a, prior_b)-smoothed; a depth not yet observed is taken to be at
 * least as good as the one before it.  The expected committed tokens of a
 * round are E(d) = 1 + sum_{k<=d} prod_{j<=k} c_j; its cost is the minimum
 * of the last four round times measured at nt = d + 1 (an unmeasured nt is
 * priced by the least-squares line through the measured ones, or, with one
 * measured nt_m, at T(nt_m) for deeper rounds and T(nt_m) * nt / nt_m for
 * shallower ones) plus d * draft_ms.  The policy
 * moves to the depth with the highest E(d) / cost only when that beats the
 * current depth by the factor 1 + hysteresis; d never exceeds d_max.
 *   sv_depth_create: 1 <= d_max <= SV_MAX_NT - 1, 0 <= d_start <= d_max,
 *     prior_a, prior_b > 0, hysteresis >= 0, draft_ms >= 0 (host memory the
 *     policy owns; SV_E_INVALID / SV_E_NOMEM, *out = NULL on failure);
 *   sv_depth_observe: one round at depth d; accepted_len is a HOST array of
 *     n_seq values (negative entries, failed sequences, are skipped; a value
 *     above d is SV_E_INVALID); round_ms <= 0 records no time;
 *   sv_depth_next: the depth for the next round (or a negative sv_status);
 *   sv_depth_estimates: HOST outputs, each optional: accept[d_max] (c_j for
 *     j = 1..d_max), cost_ms[d_max + 1] and tok_per_ms[d_max + 1] per depth. */
typedef struct sv_depth sv_depth;
int sv_depth_create(int32_t d_max, int32_t d_start, float prior_a, float prior_b,
                    float hysteresis, float draft_ms, sv_depth **out);
void sv_depth_destroy(sv_depth *p);
int sv_depth_observe(sv_depth *p, int32_t d, int32_t n_seq, const int32_t *accepted_len,
                     double round_ms);
int32_t sv_depth_next(sv_depth *p);
int sv_depth_estimates(const sv_depth *p, double *accept, double *cost_ms, double *tok_per_ms);

/* ---- single-operation entry points (used by the tests) ------------------ */

typedef struct sv_qweight sv_qweight;

/* Repack one canonical tensor (device bytes, rows x cols) for sv_qgemm. */
int sv_qweight_create(int32_t type, int64_t rows, int64_t cols, const void *canonical,
                      sv_qweight **out);
void sv_qweight_destroy(sv_qweight *w);
size_t sv_qgemm_workspace_bytes(const sv_qweight *w, int32_t m_rows);

/* y[m][n] = scale[m] * sum_k x[m][k] w[n][k] for m < m_rows, with the same
 * kernels and precision as the verify round (fp32 activations split into
 * fp16 high and low parts, exact integer weight codes, fp32 accumulation).
 * x: device fp32 [m_rows][cols]; scale: device fp32 [m_rows] or NULL (1);
 * y: device fp32 [m_rows][rows].  Asynchronous on `stream`. */
int sv_qgemm(const sv_qweight *w, const float *x, const float *scale, int32_t m_rows,
             float *y, void *workspace, size_t workspace_bytes, void *stream);

/* ---- per-kernel timing ---------------------------------------------------
 * For measurement tools: while profiling is on, spec_verify_round records a
 * pair of HIP events around every kernel it launches, on the round's stream,
 * tagged by kernel class (below).  Not for graph capture.  sv_profile_begin
 * creates a pool of max_launches event pairs (host call, may allocate);
 * sv_profile_end synchronizes on the recorded events, writes per-class
 * statistics into out[0..SV_PROF_NCLASS) and releases the pool.  Returns the
 * number of launches recorded, or a negative sv_status. */
enum {
  SV_PROF_EMBED = 0, SV_PROF_GEMM_QKV, SV_PROF_EPI_QKV, SV_PROF_ATTN, SV_PROF_COMBINE,
  SV_PROF_GEMM_O, SV_PROF_EPI_O, SV_PROF_GEMM_GU, SV_PROF_EPI_GU, SV_PROF_GEMM_DOWN,
  SV_PROF_EPI_DOWN, SV_PROF_GEMM_LM, SV_PROF_EPI_LM, SV_PROF_DECIDE, SV_PROF_OTHER,
  SV_PROF_LAYER, SV_PROF_NCLASS
};
typedef struct {
  int32_t launches;   /* launches recorded in this class */
  int32_t reserved;
  double total_ms, min_ms, max_ms;
} sv_profile_stat;
int sv_profile_begin(int32_t max_launches);
int sv_profile_end(sv_profile_stat *out);

const char *sv_status_string(int32_t status);
int32_t sv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
