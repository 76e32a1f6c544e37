// C ABI of the verify round: argument validation (fail closed), model
// creation (repack + RoPE table), workspace carve-up, and the round's kernel
// sequence on one stream.  Nothing here synchronizes or allocates during a
// round, so a round can be captured into a HIP graph.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "sv_internal.h"

#define SV_CHECK_HIP(x)                          \
  do {                                           \
    hipError_t e_ = (x);                         \
    if (e_ != hipSuccess) return SV_E_HIP;       \
  } while (0)

// Launch through a wrapper, timing it when profiling is on.
#define SV_LAUNCH(tag, x)                        \
  do {                                           \
    const int pi_ = prof_start((tag), st);       \
    hipError_t e_ = (x);                         \
    prof_stop(pi_, st);                          \
    if (e_ != hipSuccess) return SV_E_HIP;       \
  } while (0)

namespace {

// Work decomposition of a quantized GEMM, a function of the tensor's shape
// only (so a row's result never depends on how many rows a call carries):
// one workgroup per group of tpw 16-column tiles, one wave per K split.
// The split count is at most 8 (a workgroup must fit a CU at two waves per
// SIMD) and at most what keeps groups x splits within the 2048 waves
// resident at once.
const int kMaxWaves = 2048;
const int kMaxKsplit = 8;

void decompose(sv_qweight *w, int tpw) {
  w->tpw = tpw;
  w->ngroups = w->ntile / tpw;
  int ks = kMaxWaves / w->ngroups;
  if (ks > kMaxKsplit) ks = kMaxKsplit;
  if (ks < 1) ks = 1;
  if (ks > w->nsb) ks = w->nsb;
  w->sbps = (w->nsb + ks - 1) / ks;
  w->ksplit = (w->nsb + w->sbps - 1) / w->sbps;
}

int canonical_row_bytes(int type, int64_t cols) {
  if (type == SV_B6_256) return (int)(cols / 256 * 210);
  return (int)(cols / 256 * 144);  // B4_256 and 8 x B4_32 blocks are both 144 B
}

bool valid_type(int t) { return t == SV_B4_32 || t == SV_B4_256 || t == SV_B6_256; }

// Repack `rows` destination rows; rowmap[n] = (source index << 24) | source row.
int make_qweight(int type, int64_t rows, int64_t cols, const std::vector<const void *> &srcs,
                 const std::vector<int32_t> &rowmap, int tpw, sv_qweight *w) {
  std::memset(w, 0, sizeof(*w));
  w->type = type;
  w->rows = rows;
  w->cols = cols;
  w->nsb = (int)(cols / 256);
  w->ntile = (int)(rows / 16);
  w->tb_bytes = (type == SV_B6_256) ? SV_TB_B6 : SV_TB_B4;
  size_t bytes = (size_t)w->ntile * w->nsb * w->tb_bytes;
  if (hipMalloc(&w->data, bytes) != hipSuccess) {
    w->data = nullptr;
    return SV_E_NOMEM;
  }
  const uint8_t **d_srcs = nullptr;
  int32_t *d_map = nullptr;
  int rc = SV_OK;
  if (hipMalloc(&d_srcs, srcs.size() * sizeof(void *)) != hipSuccess ||
      hipMalloc(&d_map, rowmap.size() * sizeof(int32_t)) != hipSuccess) {
    rc = SV_E_NOMEM;
  } else if (hipMemcpy(d_srcs, srcs.data(), srcs.size() * sizeof(void *),
                       hipMemcpyHostToDevice) != hipSuccess ||
             hipMemcpy(d_map, rowmap.data(), rowmap.size() * sizeof(int32_t),
                       hipMemcpyHostToDevice) != hipSuccess ||
             sv_launch_repack(type, d_srcs, d_map, rows, w->nsb, w->data, 0) != hipSuccess ||
             hipDeviceSynchronize() != hipSuccess) {
    rc = SV_E_HIP;
  }
  if (d_srcs) (void)hipFree(d_srcs);
  if (d_map) (void)hipFree(d_map);
  if (rc != SV_OK) {
    (void)hipFree(w->data);
    w->data = nullptr;
    return rc;
  }
  decompose(w, tpw);
  return SV_OK;
}

void free_qweight(sv_qweight *w) {
  if (w && w->data) (void)hipFree(w->data);
  if (w) w->data = nullptr;
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
  uint8_t *base;
  size_t off = 0;
  template <class T>
  T *take(size_t bytes) {
    T *p = base ? (T *)(base + off) : nullptr;
    off += al(bytes);
    return p;
  }
};

sv_dims make_dims(const sv_model *m, int S, int nt, int cap) {
  sv_dims d;
  d.S = S;
  d.nt = nt;
  d.M = S * nt;
  d.MT = (d.M + 15) / 16;
  d.Mp = 16 * d.MT;
  d.NQ = nt * m->G;
  d.MTQ = (d.NQ + 15) / 16;
  d.nch = cap / SV_ATT_CHUNK;   // attention key chunks (the capacity is a multiple of 128)
  d.NGlm = m->V / 32;
  return d;
}

// A length bound narrows attention to the chunks below max_len + nt (the
// slots keep their layout: only the chunk count shrinks).
void narrow_chunks(sv_dims &d, int maxlen, int nt) {
  if (maxlen <= 0) return;
  const int64_t need = ((int64_t)maxlen + nt + SV_ATT_CHUNK - 1) / SV_ATT_CHUNK;
  if (need < d.nch) d.nch = (int)need;
}

// Lay out (or size, when base is NULL) the round workspace.  need_logits:
// the stochastic modes keep their logits in the workspace (the caller passed
// no logits buffer).
size_t carve(const sv_model *m, const sv_dims &d, int mode, uint8_t *base, sv_ws *w,
             bool need_logits = true) {
  Carve c{base};
  sv_ws t;
  const int H = m->H, Ko = m->nq * m->hd, F = m->F;
  t.err = c.take<int32_t>(sizeof(int32_t) * d.S);
  t.oldlen = c.take<int32_t>(sizeof(int32_t) * d.S);
  t.argmax = c.take<int32_t>(sizeof(int32_t) * d.Mp);
  t.x = c.take<float>(sizeof(float) * (size_t)d.Mp * H);
  t.x1 = c.take<float>(sizeof(float) * (size_t)d.Mp * H);
  t.ap_h = c.take<uint8_t>((size_t)d.MT * (H / 32) * 2048);
  t.sx_h = c.take<uint8_t>((size_t)d.MT * (H / 256) * 512);
  t.ssq = c.take<float>(sizeof(float) * (size_t)d.Mp * (H / 32));
  t.ap_h2 = c.take<uint8_t>((size_t)d.MT * (H / 32) * 2048);
  t.sx_h2 = c.take<uint8_t>((size_t)d.MT * (H / 256) * 512);
  t.ssq2 = c.take<float>(sizeof(float) * (size_t)d.Mp * (H / 32));
  t.rinv = c.take<float>(sizeof(float) * (size_t)d.Mp);
  if (m->L > 0) {
    t.ap_o = c.take<uint8_t>((size_t)d.MT * (Ko / 32) * 2048);
    t.sx_o = c.take<uint8_t>((size_t)d.MT * (Ko / 256) * 512);
    t.ap_f = c.take<uint8_t>((size_t)d.MT * (F / 32) * 2048);
    t.sx_f = c.take<uint8_t>((size_t)d.MT * (F / 256) * 512);
    t.qpack = c.take<uint8_t>((size_t)d.S * m->nkv * d.MTQ * (m->hd / 32) * 2048);
    // one slot per key chunk
    const size_t nsl = (size_t)d.nch;
    t.att_o = c.take<float>(sizeof(float) * (size_t)d.S * m->nkv * nsl * d.MTQ * 16 * m->hd);
    t.att_ml = c.take<float>(sizeof(float) * (size_t)d.S * m->nkv * nsl * d.MTQ * 16 * 2);
  } else {
    t.ap_o = t.sx_o = t.ap_f = t.sx_f = t.qpack = nullptr;
    t.att_o = t.att_ml = nullptr;
  }
  if (mode == SV_GREEDY) {
    t.lm_part = c.take<float>(sizeof(float) * (size_t)d.Mp * d.NGlm * 2);
    t.lm_stat = t.dr_stat = nullptr;
    t.rj_stat = t.rj_sum = nullptr;
    t.logits = nullptr;
  } else {
    t.lm_part = nullptr;
    t.lm_stat = c.take<double>(sizeof(double) * (size_t)d.Mp * d.NGlm * 2);
    t.dr_stat = c.take<double>(sizeof(double) * (size_t)d.S * (d.nt > 1 ? d.nt - 1 : 1) *
                               d.NGlm * 2);
    t.logits = need_logits ? c.take<float>(sizeof(float) * (size_t)d.Mp * m->V) : nullptr;
    t.rj_stat = c.take<double>(sizeof(double) * (size_t)d.S * (2 * d.nt - 1) * 2);
    t.rj_sum = c.take<double>(sizeof(double) * (size_t)d.S * d.nt * SV_RJ_NB * 2);
  }
  // one decision counter per sequence, then the fused layers' counters (all
  // zeroed at the start of a round)
  const int nd = (d.S + SV_LAYER_CSTRIDE - 1) / SV_LAYER_CSTRIDE * SV_LAYER_CSTRIDE;
  const int nl = m->L * SV_LAYER_NCNT * SV_LAYER_CSTRIDE;
  t.cnt = c.take<int32_t>(sizeof(int32_t) * ((size_t)nd + nl));
  t.dcnt = t.cnt;
  t.lcnt = t.cnt + nd;
  t.ncnt = nd + nl;
  t.amb = c.take<int32_t>(sizeof(int32_t) * (size_t)d.Mp);
  if (w) *w = t;
  return c.off;
}

// ---- optional per-launch timing (see sv_profile_begin) ----
struct Prof {
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;   // 2 per launch
  std::vector<int> tag;
};
Prof g_prof;

int prof_start(int tag, hipStream_t st) {
  if (!g_prof.on || g_prof.n >= g_prof.cap) return -1;
  const int i = g_prof.n++;
  g_prof.tag[i] = tag;
  (void)hipEventRecord(g_prof.ev[2 * i], st);
  return i;
}
void prof_stop(int i, hipStream_t st) {
  if (i >= 0) (void)hipEventRecord(g_prof.ev[2 * i + 1], st);
}

bool env_is(const char *name, const char *val) {
  const char *e = std::getenv(name);
  return e && std::strcmp(e, val) == 0;
}

// ---- the library's own scratch array (spec_verify_round_static) ----------
// One copy per device.  Host code never uses the array's name as an
// address: each device's copy is located once with hipGetSymbolAddress
// (with that device current) and kept in g_scratch.
__device__ __align__(256) uint8_t scratch[SV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// This device's scratch address (located on first use), or NULL.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}


}  // namespace

extern "C" {

int32_t sv_version(void) { return 1; }

const char *sv_status_string(int32_t s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_E_INVALID: return "invalid argument";
    case SV_E_UNSUPPORTED: return "unsupported";
    case SV_E_CAPACITY: return "KV capacity exceeded";
    case SV_E_HIP: return "HIP runtime error";
    case SV_E_FAULT_INJECTED: return "fault injected";
    case SV_E_NOMEM: return "out of device memory";
    case SV_E_NUMERIC: return "non-finite logits";
    case SV_E_TIMEOUT: return "device-side wait expired";
    default: return "unknown status";
  }
}

void sv_model_destroy(sv_model *m) {
  if (!m) return;
  for (int l = 0; l < m->L; ++l) {
    if (m->qkv) free_qweight(&m->qkv[l]);
    if (m->wo) free_qweight(&m->wo[l]);
    if (m->gu) free_qweight(&m->gu[l]);
    if (m->down) free_qweight(&m->down[l]);
  }
  delete[] m->qkv;
  delete[] m->wo;
  delete[] m->gu;
  delete[] m->down;
  free_qweight(&m->lm);
  if (m->rope) (void)hipFree(m->rope);
  delete m;
}

int sv_model_create(const sv_model_desc *d, sv_model **out) {
  if (!out) return SV_E_INVALID;
  *out = nullptr;
  if (!d) return SV_E_INVALID;
  const int L = d->n_layer, H = d->hidden, nq = d->n_head, nkv = d->n_kv_head;
  const int hd = d->head_dim, F = d->ffn, V = d->vocab;
  if (L < 0 || H <= 0 || V <= 0 || !d->lm_head) return SV_E_INVALID;
  if (!valid_type(d->fmt_lm)) return SV_E_UNSUPPORTED;
  if (H % 256 || V % 32 || H > 8192) return SV_E_UNSUPPORTED;  // norms read <= 256 partials
  if (d->lm_only) {
    if (L != 0) return SV_E_INVALID;
  } else {
    if (L < 1 || !d->tok_embd || !d->attn_norm || !d->ffn_norm || !d->out_norm)
      return SV_E_INVALID;
    if (!d->wq || !d->wk || !d->wv || !d->wo || !d->w_gate || !d->w_up || !d->w_down)
      return SV_E_INVALID;
    if (d->fmt_proj != SV_B4_32 && d->fmt_proj != SV_B4_256) return SV_E_UNSUPPORTED;
    if (nq <= 0 || nkv <= 0 || nq % nkv) return SV_E_INVALID;
    if (hd != 64 && hd != 128) return SV_E_UNSUPPORTED;
    if ((nq * hd) % 256 || F % 256 || (nkv * hd) % 32) return SV_E_UNSUPPORTED;
    if (d->max_pos <= 0 || !(d->rms_eps > 0.f) || !(d->rope_base > 0.f)) return SV_E_INVALID;
  }
  if (sv_gemm_prepare() != hipSuccess || sv_layer_prepare() != hipSuccess) return SV_E_HIP;
  sv_model *m = new (std::nothrow) sv_model();
  if (!m) return SV_E_NOMEM;
  std::memset(m, 0, sizeof(*m));
  m->d = *d;
  m->d.wq = m->d.wk = m->d.wv = m->d.wo = m->d.w_gate = m->d.w_up = m->d.w_down = nullptr;
  m->L = L;
  m->H = H;
  m->nq = nq;
  m->nkv = nkv;
  m->hd = hd;
  m->F = F;
  m->V = V;
  m->G = d->lm_only ? 1 : nq / nkv;
  int rc = SV_OK;
  if (L > 0) {
    m->qkv = new (std::nothrow) sv_qweight[L]();
    m->wo = new (std::nothrow) sv_qweight[L]();
    m->gu = new (std::nothrow) sv_qweight[L]();
    m->down = new (std::nothrow) sv_qweight[L]();
    if (!m->qkv || !m->wo || !m->gu || !m->down) rc = SV_E_NOMEM;
  }
  const int qd = nq * hd, kd = nkv * hd, half = hd / 2;
  for (int l = 0; l < L && rc == SV_OK; ++l) {
    std::vector<int32_t> map;
    map.reserve(qd + 2 * kd);
    for (int region = 0; region < 2; ++region) {
      const int heads = region == 0 ? nq : nkv;
      for (int h = 0; h < heads; ++h)
        for (int j = 0; j < hd; ++j) {
          const int i = j >> 1, srow = h * hd + i + ((j & 1) ? half : 0);
          map.push_back((region << 24) | srow);
        }
    }
    for (int r = 0; r < kd; ++r) map.push_back((2 << 24) | r);
    rc = make_qweight(d->fmt_proj, qd + 2 * kd, H, {d->wq[l], d->wk[l], d->wv[l]}, map, 2,
                      &m->qkv[l]);
    if (rc != SV_OK) break;
    map.clear();
    for (int r = 0; r < H; ++r) map.push_back(r);
    rc = make_qweight(d->fmt_proj, H, qd, {d->wo[l]}, map, 2, &m->wo[l]);
    if (rc != SV_OK) break;
    map.clear();
    for (int t = 0; t < F / 16; ++t)
      for (int src = 0; src < 2; ++src)
        for (int c = 0; c < 16; ++c) map.push_back((src << 24) | (16 * t + c));
    rc = make_qweight(d->fmt_proj, 2 * F, H, {d->w_gate[l], d->w_up[l]}, map, 4, &m->gu[l]);
    if (rc != SV_OK) break;
    map.clear();
    for (int r = 0; r < H; ++r) map.push_back(r);
    rc = make_qweight(d->fmt_proj, H, F, {d->w_down[l]}, map, 2, &m->down[l]);
  }
  if (rc == SV_OK) {
    std::vector<int32_t> map(V);
    for (int r = 0; r < V; ++r) map[r] = r;
    rc = make_qweight(d->fmt_lm, V, H, {d->lm_head}, map, 2, &m->lm);
  }
  // locate this device's scratch array now, with the device current
  if (rc == SV_OK && !device_scratch()) rc = SV_E_HIP;
  if (rc == SV_OK && L > 0) {
    std::vector<float> tab((size_t)d->max_pos * half * 2);
    for (int p = 0; p < d->max_pos; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow((double)d->rope_base, -2.0 * i / (double)hd);
        tab[((size_t)p * half + i) * 2] = (float)std::cos(ang);
        tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    if (hipMalloc(&m->rope, tab.size() * sizeof(float)) != hipSuccess) {
      m->rope = nullptr;
      rc = SV_E_NOMEM;
    } else if (hipMemcpy(m->rope, tab.data(), tab.size() * sizeof(float),
                         hipMemcpyHostToDevice) != hipSuccess) {
      rc = SV_E_HIP;
    }
  }
  if (rc != SV_OK) {
    sv_model_destroy(m);
    return rc;
  }
  *out = m;
  return SV_OK;
}

size_t sv_workspace_bytes(const sv_model *m, int32_t n_seq, int32_t nt, int32_t mode) {
  if (!m || n_seq < 1 || nt < 1 || nt > SV_MAX_NT) return 0;
  // the attention buffers depend on the KV capacity; size for max_pos
  const int cap = (m->d.max_pos / SV_KV_CHUNK) * SV_KV_CHUNK;
  sv_dims dd = make_dims(m, n_seq, nt, cap > 0 ? cap : SV_KV_CHUNK);
  return carve(m, dd, mode, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Argument and shape checks of a round (nothing is enqueued).
int check_round(const sv_model *m, const sv_kv *kv, const sv_round *r) {
  if (!m || !r) return SV_E_INVALID;
  const int S = r->n_seq, nt = r->nt;
  if (S < 1 || nt < 1) return SV_E_INVALID;
  if (nt > SV_MAX_NT) return SV_E_UNSUPPORTED;
  if (r->mode != SV_GREEDY && r->mode != SV_REJECT && r->mode != SV_SAMPLE)
    return SV_E_UNSUPPORTED;
  if (!r->accepted_len || !r->emitted || !r->ids) return SV_E_INVALID;
  if (r->max_len < 0) return SV_E_INVALID;
  if (r->mode == SV_REJECT) {
    if (!(r->temperature > 0.f) || !r->uniforms) return SV_E_INVALID;
    if (nt > 1 && !r->draft_logits) return SV_E_INVALID;
  }
  if (r->mode == SV_SAMPLE) {
    if (!(r->temperature > 0.f) || !r->uniforms || r->draft_logits) return SV_E_INVALID;
  }
  if (m->d.lm_only) {
    if (!r->hidden) return SV_E_INVALID;
  } else {
    if (r->hidden) return SV_E_INVALID;
    if (!kv || !kv->k || !kv->v || !kv->len || kv->n_seq != S) return SV_E_INVALID;
    if (kv->capacity < SV_KV_CHUNK || kv->capacity % SV_KV_CHUNK) return SV_E_UNSUPPORTED;
    if (kv->capacity > m->d.max_pos) return SV_E_INVALID;
    if (nt * m->G > 112) return SV_E_UNSUPPORTED;
    const int mtq = (nt * m->G + 15) / 16;
    if (sv_attn_region_bytes(m->hd, mtq, kv->capacity / SV_ATT_CHUNK) >= (size_t)1 << 31)
      return SV_E_UNSUPPORTED;
  }
  return SV_OK;
}

// With the environment variable SV_FUSED_LAYER=1, rounds of at most 16 rows
// of a 4-bit super-block model with 128-dim heads run each layer as one
// fused launch (sv_layer.hip) with the same bits as the separate kernels.
// It is off by default: each of its five in-launch hand-offs costs about as
// much as a kernel boundary, and the separate kernels are faster.
bool use_fused_layer(const sv_model *m, const sv_dims &d) {
  if (m->d.lm_only || m->L == 0 || m->d.fmt_proj != SV_B4_256 || m->hd != 128) return false;
  if (!sv_layer_supported(d.M, d.MTQ) || !env_is("SV_FUSED_LAYER", "1")) return false;
  const sv_qweight &q = m->qkv[0], &o = m->wo[0], &g = m->gu[0], &dn = m->down[0];
  return q.tpw == 2 && o.tpw == 2 && dn.tpw == 2 && g.tpw == 4 && g.ksplit <= 4 &&
         q.ksplit <= 8 && o.ksplit <= 8 && dn.ksplit <= 8;
}

// The round's kernels on stream st, with the workspace laid out in w.
int enqueue_round(const sv_model *m, const sv_kv *kv, const sv_round *r, const sv_ws &w,
                  hipStream_t st) {
  const int S = r->n_seq, nt = r->nt;
  const int cap = m->d.lm_only ? SV_KV_CHUNK : kv->capacity;
  sv_dims d = make_dims(m, S, nt, cap);
  const int maxlen = m->d.lm_only ? 0 : r->max_len;
  narrow_chunks(d, maxlen, nt);
  const int H = m->H, L = m->L;
  int32_t *lens = m->d.lm_only ? nullptr : kv->len;
  float *logits = r->logits ? r->logits : w.logits;

  const bool fused = use_fused_layer(m, d);
  // lm_head-only rounds have no cache (lens NULL): every sequence is in range;
  // the fused layers' counters are cleared only when they are used
  const int ncnt = fused ? w.ncnt : (int)(w.lcnt - w.cnt);
  SV_LAUNCH(SV_PROF_OTHER, sv_launch_init(lens, r->nts, w.err, w.oldlen, S, nt, cap, maxlen, w.cnt, ncnt, st));
  const float *g0 = m->d.lm_only ? nullptr : (L > 0 ? m->d.attn_norm : m->d.out_norm);
  SV_LAUNCH(SV_PROF_EMBED, sv_launch_embed(r->ids, m->d.tok_embd, r->hidden, g0, d.M, H, w.x, w.ap_h,
                               w.sx_h, w.ssq, nt, m->V, w.err, r->nts, st));
  sv_epi_args base;
  std::memset(&base, 0, sizeof(base));
  base.M = d.M;
  base.Mp = d.Mp;
  base.S = S;
  base.nt = nt;
  base.H = H;
  base.eps = m->d.rms_eps;
  base.normH = H;
  base.nssq = H / 32;
  base.rinv = w.rinv;
  for (int l = 0; l < L; ++l) {
    const size_t Hoff = (size_t)l * H;
    const size_t lay = (size_t)l * S * m->nkv * cap * m->hd;
    const sv_qweight *wq = &m->qkv[l], *wo = &m->wo[l], *wg = &m->gu[l], *wd = &m->down[l];
    // q|k|v with RoPE and the cache append
    sv_epi_args aq = base;
    aq.type = SV_EPI_QKV;
    aq.tl_kind = SV_TL_QKV;
    aq.ksplit = wq->ksplit;
    aq.C = 16 * wq->tpw;
    aq.ngroups = wq->ngroups;
    aq.ssq = w.ssq;
    aq.layer = l;
    aq.nq = m->nq;
    aq.nkv = m->nkv;
    aq.hd = m->hd;
    aq.G = m->G;
    aq.cap = cap;
    aq.MTQ = d.MTQ;
    aq.lens = lens;
    aq.err = w.err;
    aq.nts = r->nts;
    aq.rope = m->rope;
    aq.kc = kv->k;
    aq.vc = kv->v;
    aq.qpack = w.qpack;
    // O projection + residual; operand for the FFN (the fused layer keeps
    // the residual stream after O and the FFN's operand in buffers of their
    // own, written and read within its launch)
    sv_epi_args ao = base;
    ao.type = SV_EPI_RESID;
    ao.layer = l;
    ao.tl_kind = SV_TL_O;
    ao.ksplit = wo->ksplit;
    ao.C = 16 * wo->tpw;
    ao.ngroups = wo->ngroups;
    ao.x = w.x;
    ao.x_out = fused ? w.x1 : nullptr;
    ao.gnext = m->d.ffn_norm + Hoff;
    ao.ap_next = fused ? w.ap_h2 : w.ap_h;
    ao.sx_next = fused ? w.sx_h2 : w.sx_h;
    ao.ssq_next = fused ? w.ssq2 : w.ssq;
    ao.Knext = H;
    // gate|up + SwiGLU
    sv_epi_args ag = base;
    ag.type = SV_EPI_SWIGLU;
    ag.layer = l;
    ag.tl_kind = SV_TL_GU;
    ag.ksplit = wg->ksplit;
    ag.C = 16 * wg->tpw;
    ag.ngroups = wg->ngroups;
    ag.ssq = fused ? w.ssq2 : w.ssq;
    ag.ap_next = w.ap_f;
    ag.sx_next = w.sx_f;
    ag.Knext = m->F;
    // down + residual; operand for the next layer (or the lm_head)
    sv_epi_args ad = base;
    ad.type = SV_EPI_RESID;
    ad.layer = l;
    ad.tl_kind = SV_TL_DOWN;
    ad.ksplit = wd->ksplit;
    ad.C = 16 * wd->tpw;
    ad.ngroups = wd->ngroups;
    ad.x = fused ? w.x1 : w.x;
    ad.x_out = fused ? w.x : nullptr;
    ad.gnext = (l + 1 < L) ? m->d.attn_norm + Hoff + H : m->d.out_norm;
    ad.ap_next = w.ap_h;
    ad.sx_next = w.sx_h;
    ad.ssq_next = w.ssq;
    ad.Knext = H;
    if (fused) {
      sv_layer_args la;
      std::memset(&la, 0, sizeof(la));
      la.cnt = w.lcnt + (size_t)l * SV_LAYER_NCNT * SV_LAYER_CSTRIDE;
      la.layer = l;
      la.err = w.err;
      la.S = S;
      la.M = d.M;
      la.w_qkv = wq->data;
      la.w_o = wo->data;
      la.w_gu = wg->data;
      la.w_down = wd->data;
      la.nsb_h = wq->nsb;
      la.nsb_o = wo->nsb;
      la.nsb_f = wd->nsb;
      la.ks[0] = wq->ksplit; la.sbps[0] = wq->sbps;
      la.ks[3] = wo->ksplit; la.sbps[3] = wo->sbps;
      la.ks[4] = wg->ksplit; la.sbps[4] = wg->sbps;
      la.ks[5] = wd->ksplit; la.sbps[5] = wd->sbps;
      la.ng_gu = wg->ngroups;
      la.ap_h = w.ap_h; la.sx_h = w.sx_h;
      la.ap_o = w.ap_o; la.sx_o = w.sx_o;
      la.ap_h2 = w.ap_h2; la.sx_h2 = w.sx_h2;
      la.ap_f = w.ap_f; la.sx_f = w.sx_f;
      la.e_qkv = aq;
      la.e_o = ao;
      la.e_gu = ag;
      la.e_down = ad;
      la.kc = kv->k + lay;
      la.vc = kv->v + lay;
      la.qpack = w.qpack;
      la.lens = lens;
      la.nts = r->nts;
      la.nkv = m->nkv;
      la.cap = cap;
      la.nt = nt;
      la.G = m->G;
      la.nch = d.nch;
      la.NQ = d.NQ;
      la.NQp = 16 * d.MTQ;
      la.nitems = S * m->nkv * d.NQ * (m->hd / 8);
      la.Ko = m->nq * m->hd;
      la.scale = 1.0f / std::sqrt((float)m->hd);
      la.att_o = w.att_o;
      la.att_ml = w.att_ml;
      la.n_wg[0] = wq->ngroups;
      la.n_wg[1] = (S * m->nkv * d.nch + 1) / 2;
      la.n_wg[2] = (la.nitems * 8 + 511) / 512;
      la.n_wg[3] = wo->ngroups;
      la.n_wg[4] = (wg->ngroups + 1) / 2;
      la.n_wg[5] = wd->ngroups;
      la.lds_gu_floats = (int)(sv_gemm_lds_bytes(wg->ksplit, 1, wg->tpw, ag) / sizeof(float));
      la.lds_qkv = sv_gemm_lds_bytes(wq->ksplit, 1, wq->tpw, aq);
      la.lds_o = sv_gemm_lds_bytes(wo->ksplit, 1, wo->tpw, ao);
      la.lds_down = sv_gemm_lds_bytes(wd->ksplit, 1, wd->tpw, ad);
      SV_LAUNCH(SV_PROF_LAYER, sv_launch_layer(la, d.MTQ, st));
      continue;
    }
    SV_LAUNCH(SV_PROF_GEMM_QKV, sv_launch_qgemm(wq, w.ap_h, w.sx_h, d.M, 0, d.MT, aq, st));
    // attention
    SV_LAUNCH(SV_PROF_ATTN,
              sv_launch_attn(m->hd, d.MTQ, kv->k + lay, kv->v + lay, w.qpack, lens, w.err, S,
                             m->nkv, cap, nt, m->G, w.att_o, w.att_ml, d.nch, w.ap_o,
                             w.sx_o, m->nq * m->hd, r->nts, st, l));
    SV_LAUNCH(SV_PROF_GEMM_O, sv_launch_qgemm(wo, w.ap_o, w.sx_o, d.M, 0, d.MT, ao, st));
    SV_LAUNCH(SV_PROF_GEMM_GU, sv_launch_qgemm(wg, w.ap_h, w.sx_h, d.M, 0, d.MT, ag, st));
    SV_LAUNCH(SV_PROF_GEMM_DOWN, sv_launch_qgemm(wd, w.ap_f, w.sx_f, d.M, 0, d.MT, ad, st));
  }
  // lm_head
  sv_epi_args a = base;
  a.type = SV_EPI_LM;
  a.tl_kind = SV_TL_LM;
  a.ksplit = m->lm.ksplit;
  a.C = 16 * m->lm.tpw;
  a.ngroups = m->lm.ngroups;
  a.ssq = m->d.lm_only ? nullptr : w.ssq;
  a.logits = logits;
  a.lm_part = w.lm_part;
  a.lm_stat = w.lm_stat;
  a.dr_stat = w.dr_stat;
  a.draft_logits = r->mode == SV_REJECT ? r->draft_logits : nullptr;
  a.V = m->V;
  a.err = w.err;
  a.temperature = r->temperature;
  a.reject = r->mode != SV_GREEDY;   // fp64 softmax statistics per group
  SV_LAUNCH(SV_PROF_GEMM_LM,
            sv_launch_qgemm(&m->lm, w.ap_h, w.sx_h, d.M, 0, d.MT, a, st));
  if (env_is("SV_FAULT", "after_verify")) return SV_E_FAULT_INJECTED;
  int32_t *lens_commit = lens;
  if (!lens_commit) {
    // no cache: the decision kernels still need a length array to update
    lens_commit = w.oldlen;
  }
  if (r->mode == SV_GREEDY) {
    SV_LAUNCH(SV_PROF_DECIDE, sv_launch_greedy(w.lm_part, d.NGlm, r->ids, S, nt, w.err, lens_commit, w.oldlen,
                                  r->accepted_len, r->emitted, r->argmax, lens ? r->commit : 0,
                                  w.amb, w.dcnt, r->nts, st));
  } else if (r->mode == SV_SAMPLE) {
    SV_LAUNCH(SV_PROF_DECIDE, sv_launch_sample(w.lm_stat, w.rj_stat, w.rj_sum, d.NGlm, logits,
                                               r->uniforms, r->ids, S,
                                               nt, m->V, r->temperature, w.err, lens_commit,
                                               w.oldlen, r->accepted_len, r->emitted, r->argmax,
                                               lens ? r->commit : 0, w.amb, w.dcnt, r->nts, st));
  } else {
    SV_LAUNCH(SV_PROF_DECIDE, sv_launch_reject(w.lm_stat, w.dr_stat, w.rj_stat, w.rj_sum, d.NGlm,
                                  logits, r->draft_logits,
                                  r->uniforms, r->ids, S, nt, m->V, r->temperature, w.err,
                                  lens_commit, w.oldlen, r->accepted_len, r->emitted,
                                  lens ? r->commit : 0, r->nts, st));
  }
  if (lens && env_is("SV_DEBUG_POISON", "1"))
    SV_LAUNCH(SV_PROF_OTHER, sv_launch_poison(kv->k, kv->v, lens, w.oldlen, w.err, L, S, m->nkv, cap, m->hd,
                                  nt, r->nts, st));
  return SV_OK;
}

}  // namespace

extern "C" {

int spec_verify_round(const sv_model *m, const sv_kv *kv, const sv_round *r, void *workspace,
                      size_t workspace_bytes, void *stream) {
  const int rc = check_round(m, kv, r);
  if (rc != SV_OK) return rc;
  if (!workspace) return SV_E_INVALID;
  // laid out for a cache of max_pos positions, as sv_workspace_bytes sized it
  const int wcap = (m->d.max_pos / SV_KV_CHUNK) * SV_KV_CHUNK;
  const sv_dims dmax = make_dims(m, r->n_seq, r->nt, wcap > 0 ? wcap : SV_KV_CHUNK);
  if (workspace_bytes < carve(m, dmax, r->mode, nullptr, nullptr)) return SV_E_INVALID;
  sv_ws w;
  carve(m, dmax, r->mode, (uint8_t *)workspace, &w);
  return enqueue_round(m, kv, r, w, (hipStream_t)stream);
}

int spec_verify_round_static(const sv_model *m, const sv_kv *kv, const sv_round *r,
                             void *stream) {
  const int rc = check_round(m, kv, r);
  if (rc != SV_OK) return rc;
  // laid out for this round's own cache capacity (or its length bound); the
  // stochastic modes keep logits in the scratch only when the caller passed
  // none
  const int cap = m->d.lm_only ? SV_KV_CHUNK : kv->capacity;
  sv_dims d = make_dims(m, r->n_seq, r->nt, cap);
  if (!m->d.lm_only) narrow_chunks(d, r->max_len, r->nt);   // as the round will use it
  const bool need_logits = r->logits == nullptr;
  if (carve(m, d, r->mode, nullptr, nullptr, need_logits) > SV_STATIC_SCRATCH_BYTES)
    return SV_E_UNSUPPORTED;
  uint8_t *base = (uint8_t *)device_scratch();
  if (!base) return SV_E_HIP;
  sv_ws w;
  carve(m, d, r->mode, base, &w, need_logits);
  return enqueue_round(m, kv, r, w, (hipStream_t)stream);
}

int sv_advance(const sv_advance_args *a, void *stream) {
  if (!a || a->n_seq < 1 || a->nt < 1 || a->nt > SV_MAX_NT) return SV_E_INVALID;
  if (!a->ids || !a->accepted_len || !a->emitted || !a->len) return SV_E_INVALID;
  if (a->tokens && a->tok_cap < 1) return SV_E_INVALID;
  if (a->nt > 1 && (!a->noise || a->ref_cap < 1)) return SV_E_INVALID;
  if ((a->ref == nullptr) != (a->draw == nullptr)) return SV_E_INVALID;
  if ((a->utab == nullptr) != (a->uniforms == nullptr)) return SV_E_INVALID;
  if (a->utab && a->ref_cap < 1) return SV_E_INVALID;
  if (!(a->p_accept >= 0.f && a->p_accept <= 1.f && a->p_decay >= 0.f && a->p_decay <= 1.f))
    return SV_E_INVALID;
  SV_CHECK_HIP(sv_launch_advance(*a, (hipStream_t)stream));
  return SV_OK;
}

// ---- per-kernel timing -------------------------------------------------------
int sv_profile_begin(int32_t max_launches) {
  if (max_launches < 1) return SV_E_INVALID;
  if (g_prof.on) return SV_E_INVALID;
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto &e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return SV_E_HIP;
  g_prof.tag.assign(max_launches, 0);
  g_prof.cap = max_launches;
  g_prof.n = 0;
  g_prof.on = true;
  return SV_OK;
}

int sv_profile_end(sv_profile_stat *out) {
  if (!g_prof.on) return SV_E_INVALID;
  g_prof.on = false;
  int rc = g_prof.n;
  if (out)
    for (int c = 0; c < SV_PROF_NCLASS; ++c) out[c] = sv_profile_stat{0, 0, 0.0, 1e30, 0.0};
  for (int i = 0; i < g_prof.n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) {
      rc = SV_E_HIP;
      break;
    }
    if (out) {
      sv_profile_stat &st = out[g_prof.tag[i]];
      st.launches += 1;
      st.total_ms += ms;
      st.min_ms = ms < st.min_ms ? ms : st.min_ms;
      st.max_ms = ms > st.max_ms ? ms : st.max_ms;
    }
  }
  for (auto &e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.n = g_prof.cap = 0;
  return rc;
}

// ---- single GEMM entry points ---------------------------------------------
int sv_qweight_create(int32_t type, int64_t rows, int64_t cols, const void *canonical,
                      sv_qweight **out) {
  if (!out) return SV_E_INVALID;
  *out = nullptr;
  if (!canonical || rows <= 0 || cols <= 0) return SV_E_INVALID;
  if (!valid_type(type)) return SV_E_UNSUPPORTED;
  if (rows % 32 || cols % 256 || rows >= (1 << 24)) return SV_E_UNSUPPORTED;
  if (sv_gemm_prepare() != hipSuccess) return SV_E_HIP;
  sv_qweight *w = new (std::nothrow) sv_qweight();
  if (!w) return SV_E_NOMEM;
  std::vector<int32_t> map(rows);
  for (int64_t r = 0; r < rows; ++r) map[r] = (int32_t)r;
  int rc = make_qweight(type, rows, cols, {canonical}, map, 2, w);
  if (rc != SV_OK) {
    delete w;
    return rc;
  }
  *out = w;
  return SV_OK;
}

void sv_qweight_destroy(sv_qweight *w) {
  if (!w) return;
  free_qweight(w);
  delete w;
}

static size_t qgemm_carve(const sv_qweight *w, int M, uint8_t *base, float **x, uint8_t **ap,
                          uint8_t **sx) {
  const int MT = (M + 15) / 16, Mp = 16 * MT;
  Carve c{base};
  float *xx = c.take<float>(sizeof(float) * (size_t)Mp * w->cols);
  uint8_t *a = c.take<uint8_t>((size_t)MT * (w->cols / 32) * 2048);
  uint8_t *s = c.take<uint8_t>((size_t)MT * (w->cols / 256) * 512);
  if (x) *x = xx;
  if (ap) *ap = a;
  if (sx) *sx = s;
  return c.off;
}

size_t sv_qgemm_workspace_bytes(const sv_qweight *w, int32_t m_rows) {
  if (!w || m_rows < 1) return 0;
  return qgemm_carve(w, m_rows, nullptr, nullptr, nullptr, nullptr);
}

int sv_qgemm(const sv_qweight *w, const float *x, const float *scale, int32_t m_rows, float *y,
             void *workspace, size_t workspace_bytes, void *stream) {
  if (!w || !x || !y || !workspace || m_rows < 1) return SV_E_INVALID;
  if (workspace_bytes < sv_qgemm_workspace_bytes(w, m_rows)) return SV_E_INVALID;
  float *xx;
  uint8_t *ap, *sx;
  qgemm_carve(w, m_rows, (uint8_t *)workspace, &xx, &ap, &sx);
  hipStream_t st = (hipStream_t)stream;
  const int MT = (m_rows + 15) / 16;
  SV_CHECK_HIP(sv_launch_embed(nullptr, nullptr, x, nullptr, m_rows, (int)w->cols, xx, ap, sx,
                               nullptr, 1, 0, nullptr, nullptr, st));
  sv_epi_args a;
  std::memset(&a, 0, sizeof(a));
  a.type = SV_EPI_PLAIN;
  a.M = m_rows;
  a.Mp = 16 * MT;
  a.ksplit = w->ksplit;
  a.C = 16 * w->tpw;
  a.ngroups = w->ngroups;
  a.rowscale = scale;
  a.logits = y;
  SV_CHECK_HIP(sv_launch_qgemm(w, ap, sx, m_rows, 0, MT, a, st));
  return SV_OK;
}

}  // extern "C"
