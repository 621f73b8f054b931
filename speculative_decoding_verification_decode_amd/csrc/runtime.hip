// Host runtime of libsf: the C ABI declared in include/sf.h.
//
// Ownership and allocation: device memory is allocated only in sf_model_create (packed
// weights) and sf_cache_alloc (KV pool, scratch, counters, staging, graphs).  Every later
// call reuses those fixed addresses, which is what keeps captured graph replays valid
// ("I Got 28 TPS Out of Free Kaggle GPUs", section "Why It Kept Breaking (and How I Fixed
// It)": a graph reads the addresses it was captured with).
#include "sf.h"
#include "sf_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace sf;

static thread_local std::string g_err;

static sf_status fail(sf_status code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(expr)                                                                          \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(SF_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// Fault injection for tests of the error path.  SF_FAULT=alloc makes every device allocation
// fail as an out-of-memory hipMalloc would (the call returns SF_E_NOMEM); SF_FAULT=launch makes
// every graph replay and eager pass fail as a failed launch would (SF_E_HIP), before the call
// changes any sequence state.  Read at every use, so a process can switch it on and off.
static bool injected(const char* what) {
  const char* v = getenv("SF_FAULT");
  return v && strcmp(v, what) == 0;
}

static hipError_t dev_malloc(void** p, size_t bytes) {
  if (injected("alloc")) return hipErrorOutOfMemory;
  return hipMalloc(p, bytes);
}

static hipError_t graph_launch(hipGraphExec_t x, hipStream_t s) {
  if (injected("launch")) return hipErrorLaunchFailure;
  return hipGraphLaunch(x, s);
}

namespace {

struct Layer {
  uint4 *wqkv, *wo, *wgu, *wd;
  float *bqkv, *g1, *g2;
};

struct DevAllocs {
  std::vector<void*> ptrs;
  hipError_t alloc(void** p, size_t bytes) {
    hipError_t e = dev_malloc(p, std::max<size_t>(bytes, 256));
    if (e == hipSuccess) ptrs.push_back(*p);
    return e;
  }
  void release() {
    for (void* p : ptrs) (void)hipFree(p);
    ptrs.clear();
  }
};

}  // namespace

struct sf_model {
  sf_model_desc d;
  int dev = 0;                     // the device current at creation (weights and stream live there)
  hipStream_t stream = nullptr;
  bool own_stream = false;
  int H, Q, KV, F, V, dh, nq, nkv, L;
  int nb_qkv, nb_h, nb_gu, nb_head;
  bool nf4 = false;                // projections packed as NF4 blocks (embedding and head bf16)
  uint16_t* embed = nullptr;
  std::vector<Layer> layers;
  float* gfinal = nullptr;
  float* ones = nullptr;
  uint4* head = nullptr;
  DevAllocs mem;
};

// Per-pass working memory: everything a pass writes besides the KV pool and the sequence state
// (length, pending token).  A cache owns one set (allocated in sf_cache_alloc, captured by its
// graphs); the no-allocation entry point carves another from a static device array.
struct Scratch {
  Stage* stage_d = nullptr;        // staging block: flags, k, drafts
  float* x = nullptr;              // residual [rows][H] fp32
  uint16_t *a_h = nullptr, *a_o = nullptr, *a_f = nullptr;   // GEMM operands (hi/lo, MFMA order)
  uint16_t* hidden = nullptr;      // bf16 hidden-state output [rows][H] (hidden-only stacks)
  float *ssq = nullptr, *q = nullptr, *apart = nullptr;
  float2* amax = nullptr;          // LM head per-block (max, index) [rows][V/32]
  float* part = nullptr;           // k-split partials
  int* cnt = nullptr;              // k-split arrival counters [layer][QKV, O, down][block][row group]
  int cnt_stride = 0;
  int32_t* res_d = nullptr;        // {accepted[B], target[B][T]}
  int32_t* dout_d = nullptr;       // draft-step outputs [B][kMaxDraftSteps]
  uint32_t* sink = nullptr;        // target of the L2 warm-ups' checksums (never read)
};

struct Run {
  int B, T, seq0, kmax;
  float* logits;
  bool draft_mode;
  bool prefill;
  // First row whose LM-head output is needed; -1: none (the pass only writes K/V and commits).
  int head_from = 0;
  // Device flag: the pass's kernels run only while it is nonzero (nullptr: always run).
  const int* gate = nullptr;
  // Working memory of the pass (nullptr: the cache's own).
  const Scratch* sc = nullptr;
};

struct sf_cache {
  sf_model* m;
  int B, cap, kmax, T, nchunk;
  int pchunk = kPrefillChunk;       // prompt positions per prefill pass
  size_t layer_stride, seq_stride;  // elements
  uint16_t *kpool = nullptr, *vpool = nullptr;
  int32_t *len = nullptr, *next = nullptr;
  Scratch sc;
  Stage* stage_h = nullptr;
  float2* rope = nullptr;
  int32_t *res_h = nullptr, *dout_h = nullptr;
  int nw_qkv, nw_o, nw_gu, nw_d, nw_head;
  int sp_qkv, sp_o, sp_gu, sp_d, sp_head;
  int kh = 4;                      // GEMM: weight tiles per pipelined batch (one-tile row counts)
  bool warm_o = true;              // read the O projection's weights into L2 during attention
  hipGraphExec_t gx_verify = nullptr, gx_draft = nullptr;
  uint16_t *snap_k = nullptr, *snap_v = nullptr;   // state snapshot: K/V rows [len, len+T)
  int32_t *snap_len = nullptr, *snap_next = nullptr;
  bool snap_valid = false;
  std::vector<int> len_h, next_h, len_hi;
  bool dirty = false;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  DevAllocs mem;
};

// ------------------------------------------------------------------------------------------
// Waves per GEMM workgroup: four, so that up to five workgroups share a compute unit (the
// kernel keeps about 100 registers per lane with 4-tile batches) and one streams while
// another finishes.  Four is also the batched kernel's k split, which a row's result must
// share at every row count (bitwise batch invariance), so eight (SF_NW_*) is for
// experiments only.
static int choose_nw(int nb, int kb, const char* env) {
  (void)nb;
  (void)kb;
  int nw = 4;
  if (const char* v = getenv(env)) {
    int o = atoi(v);
    if (o == 4 || o == 8) nw = o;
  }
  return nw;
}

// Workgroups per n block.  Narrow projections (O, down: 112 blocks at 7B) have too few
// 32-row blocks to occupy the GPU, so their k range is split over about 256/nb workgroups,
// at most 4, each wave keeping at least eight 16-k tiles; the last to finish adds the
// partial sums.  Measured at the 7B verify shape: down 35.9 us with 2 splits vs 44.9 with 4,
// O 11.6 vs 12.6, QKV (144 blocks) best unsplit; at the 0.5B draft shape (k ranges of 56
// tiles) an unsplit QKV and O and a down split 4 ways (not 8) were each 24-30 us faster per
// step.  SF_SP_* override.
static int choose_sp(int nb, int kb, int nw, const char* env, bool nf4 = false) {
  int sp = std::max(1, 256 / nb);
  sp = std::max(1, std::min({sp, kb / (nw * 8), 4}));
  // NF4 blocks: a split pays only over long k ranges (the 14B down projection, 864 tiles:
  // 23.2 -> 20.3 us with 3 splits; QKV and O, 320 tiles, were slower split 2 ways).
  if (nf4) sp = (nb < 256 && kb >= 512) ? 3 : 1;
  if (const char* v = getenv(env)) {
    int o = atoi(v);
    if (o >= 1) sp = o;
  }
  return std::min(sp, 8);
}

static sf_status check_desc(const sf_model_desc* d) {
  if (!d) return fail(SF_E_ARG, "desc is NULL");
  if (d->n_layers < 1 || d->hidden < 32 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->ffn < 32 || d->vocab < 16)
    return fail(SF_E_ARG, "non-positive dimension");
  if (d->hidden % 32 || d->ffn % 32 || d->vocab % 32)
    return fail(SF_E_ARG, "hidden, ffn and vocab must be multiples of 32");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(SF_E_ARG, "head_dim must be 64 or 128");
  if (d->n_q_heads % d->n_kv_heads) return fail(SF_E_ARG, "n_kv_heads must divide n_q_heads");
  if ((d->n_q_heads * d->head_dim) % 32) return fail(SF_E_ARG, "n_q_heads*head_dim must be a multiple of 32");
  if (d->hidden > 6144) return fail(SF_E_ARG, "hidden must be <= 6144");
  if (!(d->rms_eps >= 0.f) || !(d->rope_base > 1.f)) return fail(SF_E_ARG, "bad rms_eps or rope_base");
  return SF_OK;
}

// Upload a pointer table, run `fn(dev_table)`, wait, free the table.
template <typename Fn>
static sf_status with_table(const std::vector<const uint16_t*>& tab, hipStream_t s, Fn fn) {
  const uint16_t** dt = nullptr;
  HIPCHK(dev_malloc((void**)&dt, tab.size() * sizeof(void*)));
  hipError_t e = hipMemcpyAsync(dt, tab.data(), tab.size() * sizeof(void*), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = fn(dt);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(dt);
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("weight packing: ") + hipGetErrorString(e));
  return SF_OK;
}

// Bytes of one projection of n outputs and k inputs as stored: bf16, or NF4 codes (half a
// byte per weight) plus one bf16 scale per 64 inputs.
static double proj_bytes(const sf_model* m, double n, double k) {
  return m->nf4 ? n * k * 0.5 + n * (k / kNf4Block) * 2 : n * k * 2;
}

static sf_status create_model(const sf_model_desc* desc, const void* const* weights, void* stream,
                              sf_model** out, bool nf4) {
  if (sf_status st = check_desc(desc)) return st;
  if (!weights || !out) return fail(SF_E_ARG, "weights or out is NULL");
  *out = nullptr;
  if (nf4 && (desc->hidden % kNf4Block || desc->ffn % kNf4Block || (desc->n_q_heads * desc->head_dim) % kNf4Block))
    return fail(SF_E_ARG, "NF4 needs hidden, ffn and n_q_heads*head_dim to be multiples of 64");
  sf_model* m = new sf_model();
  m->nf4 = nf4;
  if (hipGetDevice(&m->dev) != hipSuccess) m->dev = 0;
  m->d = *desc;
  const sf_model_desc& d = *desc;
  m->H = d.hidden; m->nq = d.n_q_heads; m->nkv = d.n_kv_heads; m->dh = d.head_dim;
  m->Q = d.n_q_heads * d.head_dim; m->KV = d.n_kv_heads * d.head_dim; m->F = d.ffn; m->V = d.vocab;
  m->L = d.n_layers;
  m->nb_qkv = (m->Q + 2 * m->KV) / kTileN;
  m->nb_h = m->H / kTileN;
  m->nb_gu = 2 * m->F / kTileN;
  m->nb_head = m->V / kTileN;

  // Count and validate the weight table.
  const int per_layer = (d.qkv_bias ? 12 : 9) + (nf4 ? 7 : 0);   // NF4: codes + scales per projection
  const int n_tensors = 1 + d.n_layers * per_layer + (d.has_head ? 1 + (d.tied_head ? 0 : 1) : 0);
  for (int i = 0; i < n_tensors; ++i)
    if (!weights[i]) { delete m; return fail(SF_E_ARG, "weight pointer " + std::to_string(i) + " is NULL"); }

  auto cleanup = [&](sf_status st) {
    m->mem.release();
    if (m->own_stream && m->stream) (void)hipStreamDestroy(m->stream);
    delete m;
    return st;
  };
  if (stream) {
    m->stream = (hipStream_t)stream;
  } else {
    hipError_t e = hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking);
    if (e != hipSuccess) return cleanup(fail(SF_E_HIP, std::string("stream: ") + hipGetErrorString(e)));
    m->own_stream = true;
  }
  hipStream_t s = m->stream;
  const int H = m->H, Q = m->Q, KV = m->KV, F = m->F, V = m->V, dh = m->dh, half = dh / 2;
  auto W = [&](int i) { return (const uint16_t*)weights[i]; };
  // A projection's source: bf16 rows, or NF4 codes (two per byte) and bf16 scales per 64.
  struct Proj {
    const uint16_t* w = nullptr;
    const uint8_t* codes = nullptr;
    const uint16_t* scales = nullptr;
  };
  auto P = [&](int& i) {
    Proj p;
    if (nf4) {
      p.codes = (const uint8_t*)weights[i++];
      p.scales = (const uint16_t*)weights[i++];
    } else {
      p.w = (const uint16_t*)weights[i++];
    }
    return p;
  };

  auto dalloc = [&](void** p, size_t bytes) -> sf_status {
    hipError_t e = m->mem.alloc(p, bytes);
    if (e != hipSuccess) return fail(SF_E_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
    return SF_OK;
  };
#define TRY(x)                           \
  do {                                   \
    sf_status st_ = (x);                 \
    if (st_ != SF_OK) return cleanup(st_); \
  } while (0)
  // Pack projection rows (row n of the packed matrix = source row src_row[n] of proj[n]) with
  // k inputs into library-owned tiles.
  auto pack = [&](uint4** dst, const std::vector<const Proj*>& proj, const std::vector<int>& src_row, int k) -> sf_status {
    const int N = (int)src_row.size();
    if (!nf4) {
      std::vector<const uint16_t*> rows(N);
      for (int n = 0; n < N; ++n) rows[n] = proj[n]->w + (size_t)src_row[n] * k;
      if (sf_status st = dalloc((void**)dst, (size_t)N * k * 2)) return st;
      return with_table(rows, s, [&](const uint16_t* const* t) { return launch_pack(*dst, t, N / kTileN, k / kTileK, s); });
    }
    // NF4: a table of 2N row addresses, codes then scales, handed over as one pointer array.
    std::vector<const uint16_t*> rows(2 * N);
    for (int n = 0; n < N; ++n) {
      rows[n] = (const uint16_t*)(proj[n]->codes + (size_t)src_row[n] * (k / 2));
      rows[N + n] = proj[n]->scales + (size_t)src_row[n] * (k / kNf4Block);
    }
    if (sf_status st = dalloc((void**)dst, (size_t)(N / kTileN) * (k / kNf4Block) * kNf4BlockBytes)) return st;
    return with_table(rows, s, [&](const uint16_t* const* t) {
      return launch_pack_nf4((uint8_t*)*dst, (const uint8_t* const*)t, N, k / kNf4Block, s);
    });
  };

  TRY(dalloc((void**)&m->embed, (size_t)V * H * 2));
  {
    hipError_t e = hipMemcpyAsync(m->embed, W(0), (size_t)V * H * 2, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return cleanup(fail(SF_E_HIP, std::string("embed copy: ") + hipGetErrorString(e)));
  }
  TRY(dalloc((void**)&m->ones, (size_t)H * 4));
  {
    std::vector<float> ones(H, 1.0f);
    hipError_t e = hipMemcpy(m->ones, ones.data(), (size_t)H * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return cleanup(fail(SF_E_HIP, std::string("ones: ") + hipGetErrorString(e)));
  }

  int idx = 1;
  m->layers.resize(d.n_layers);
  for (int l = 0; l < d.n_layers; ++l) {
    Layer& Ly = m->layers[l];
    const uint16_t* ln1 = W(idx++);
    const Proj wq = P(idx);
    const uint16_t* bq = d.qkv_bias ? W(idx++) : nullptr;
    const Proj wk = P(idx);
    const uint16_t* bk = d.qkv_bias ? W(idx++) : nullptr;
    const Proj wv = P(idx);
    const uint16_t* bv = d.qkv_bias ? W(idx++) : nullptr;
    const Proj wo = P(idx);
    const uint16_t* ln2 = W(idx++);
    const Proj wg = P(idx);
    const Proj wu = P(idx);
    const Proj wd = P(idx);

    // QKV rows: 32-row block -> (section, head, dims i0..i0+15 and their RoPE partners
    // i0+dh/2..i0+dh/2+15), so each rotated pair lands in one block.
    const int N = Q + 2 * KV, bph = dh / 32;
    std::vector<const Proj*> pq(N);
    std::vector<int> rq(N);
    std::vector<const uint16_t*> bias(N);
    for (int n = 0; n < N; ++n) {
      const int nb = n / 32, nl = n % 32;
      const int qb = m->nq * bph, kvb = m->nkv * bph;
      int head, blk;
      const Proj* wsrc;
      const uint16_t* bsrc;
      if (nb < qb) { head = nb / bph; blk = nb % bph; wsrc = &wq; bsrc = bq; }
      else if (nb < qb + kvb) { head = (nb - qb) / bph; blk = (nb - qb) % bph; wsrc = &wk; bsrc = bk; }
      else { head = (nb - qb - kvb) / bph; blk = (nb - qb - kvb) % bph; wsrc = &wv; bsrc = bv; }
      const int dim = blk * 16 + (nl % 16) + (nl >= 16 ? half : 0);
      const int r = head * dh + dim;
      pq[n] = wsrc;
      rq[n] = r;
      bias[n] = bsrc ? bsrc + r : nullptr;
    }
    TRY(pack(&Ly.wqkv, pq, rq, H));
    TRY(dalloc((void**)&Ly.bqkv, (size_t)N * 4));
    TRY(with_table(bias, s, [&](const uint16_t* const* t) { return launch_gather_f32(Ly.bqkv, t, N, s); }));

    std::vector<int> ident(H);
    for (int n = 0; n < H; ++n) ident[n] = n;
    TRY(pack(&Ly.wo, std::vector<const Proj*>(H, &wo), ident, Q));

    // gate/up rows: 32-row block nb -> gate rows 16nb..16nb+15 then up rows 16nb..16nb+15.
    std::vector<const Proj*> pgu(2 * F);
    std::vector<int> rgu(2 * F);
    for (int n = 0; n < 2 * F; ++n) {
      const int nb = n / 32, nl = n % 32;
      pgu[n] = nl < 16 ? &wg : &wu;
      rgu[n] = nb * 16 + (nl % 16);
    }
    TRY(pack(&Ly.wgu, pgu, rgu, H));
    TRY(pack(&Ly.wd, std::vector<const Proj*>(H, &wd), ident, F));

    std::vector<const uint16_t*> g1(H), g2(H);
    for (int n = 0; n < H; ++n) { g1[n] = ln1 + n; g2[n] = ln2 + n; }
    TRY(dalloc((void**)&Ly.g1, (size_t)H * 4));
    TRY(dalloc((void**)&Ly.g2, (size_t)H * 4));
    TRY(with_table(g1, s, [&](const uint16_t* const* t) { return launch_gather_f32(Ly.g1, t, H, s); }));
    TRY(with_table(g2, s, [&](const uint16_t* const* t) { return launch_gather_f32(Ly.g2, t, H, s); }));
  }
  if (d.has_head) {
    const uint16_t* gf = W(idx++);
    const uint16_t* hsrc = d.tied_head ? W(0) : W(idx++);
    std::vector<const uint16_t*> gfv(H), rh(V);
    for (int n = 0; n < H; ++n) gfv[n] = gf + n;
    for (int n = 0; n < V; ++n) rh[n] = hsrc + (size_t)n * H;
    TRY(dalloc((void**)&m->gfinal, (size_t)H * 4));
    TRY(with_table(gfv, s, [&](const uint16_t* const* t) { return launch_gather_f32(m->gfinal, t, H, s); }));
    TRY(dalloc((void**)&m->head, (size_t)V * H * 2));
    TRY(with_table(rh, s, [&](const uint16_t* const* t) { return launch_pack(m->head, t, V / kTileN, H / kTileK, s); }));
  }
#undef TRY
  *out = m;
  return SF_OK;
}

extern "C" sf_status sf_model_create(const sf_model_desc* desc, const void* const* weights, void* stream,
                                     sf_model** out) {
  return create_model(desc, weights, stream, out, false);
}

extern "C" sf_status sf_model_create_nf4(const sf_model_desc* desc, const void* const* weights, void* stream,
                                         sf_model** out) {
  return create_model(desc, weights, stream, out, true);
}

extern "C" sf_status sf_nf4_levels(float* out) {
  if (!out) return fail(SF_E_ARG, "out is NULL");
  for (int i = 0; i < 16; ++i) {
    const uint32_t u = (uint32_t)kNf4Bits[i] << 16;
    memcpy(&out[i], &u, 4);
  }
  return SF_OK;
}

extern "C" sf_status sf_model_free(sf_model* m) {
  if (!m) return fail(SF_E_ARG, "model is NULL");
  (void)hipStreamSynchronize(m->stream);
  m->mem.release();
  if (m->own_stream) (void)hipStreamDestroy(m->stream);
  delete m;
  return SF_OK;
}


// One GEMM of kind `kind` in layer `layer`; a k split (g.sp > 1) uses the arrival counters
// of that layer and kind.
enum GemmKind { kGQkv = 0, kGO = 1, kGGateUp = 2, kGDown = 3, kGHead = 4 };

static hipError_t run_gemm(const sf_cache* c, const Scratch& S, int kind, int layer, int epi, GemmArgs g,
                           hipStream_t s) {
  g.kh = c->kh;
  if (g.sp > 1) {
    if (kind == kGGateUp || kind == kGHead) return hipErrorInvalidValue;
    const int slot = layer * 3 + (kind == kGQkv ? 0 : kind == kGO ? 1 : 2);
    g.counters = S.cnt + (size_t)slot * S.cnt_stride;
  }
  if (c->m->nf4 && kind != kGHead) return launch_gemm_nf4(epi, g, s);
  return launch_gemm(epi, g, s);
}

// ------------------------------------------------------------------------------------------
// ------------------------------------------------------------------------------------------
// One forward pass (embed .. accept) enqueued on the model stream.  Used both eagerly and
// under stream capture, so it must not allocate or synchronise.
static hipError_t enqueue_forward(sf_cache* c, const Run& r) {
  if (injected("launch")) return hipErrorLaunchFailure;
  sf_model* m = c->m;
  const sf_model_desc& d = m->d;
  const Scratch& S = r.sc ? *r.sc : c->sc;
  hipStream_t s = m->stream;
  const int rows = r.B * r.T;
  int32_t* len = c->len + r.seq0;
  int32_t* next = c->next + r.seq0;
  const size_t kvoff = (size_t)r.seq0 * c->seq_stride;
  hipError_t e;

  EmbedArgs ea{};
  ea.embed = m->embed; ea.stage = S.stage_d; ea.len = len; ea.next = next; ea.gain = m->layers[0].g1;
  ea.x = S.x; ea.a = S.a_h; ea.ssq = S.ssq; ea.rows = rows; ea.T = r.T; ea.H = m->H; ea.V = m->V;
  ea.kmax = r.kmax; ea.gate = r.gate;
  if ((e = launch_embed(ea, s)) != hipSuccess) return e;

  GemmArgs base{};
  base.rows = rows; base.ssq_in = S.ssq; base.part = S.part; base.sp = 1;
  base.nparts_in = m->H / kTileN; base.eps = d.rms_eps; base.T = r.T; base.len = len; base.cap = c->cap;
  base.seq_stride = (long)c->seq_stride; base.rope = c->rope; base.nq = m->nq; base.nkv = m->nkv; base.dh = m->dh;
  base.gate = r.gate;

  AttnArgs aa{};
  aa.q = S.q; aa.seq_stride = (long)c->seq_stride; aa.cap = c->cap; aa.len = len; aa.T = r.T; aa.nq = m->nq;
  aa.nkv = m->nkv; aa.nchunk = c->nchunk; aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)m->dh));
  aa.part = S.apart; aa.out = S.a_o; aa.rows = rows; aa.dh = m->dh; aa.gate = r.gate;

  for (int l = 0; l < m->L; ++l) {
    const Layer& Ly = m->layers[l];
    uint16_t* kc = c->kpool + (size_t)l * c->layer_stride + kvoff;
    uint16_t* vc = c->vpool + (size_t)l * c->layer_stride + kvoff;

    GemmArgs g = base;
    g.w = Ly.wqkv; g.a = S.a_h; g.k = m->H; g.kb = m->H / kTileK; g.nb = m->nb_qkv; g.nw = c->nw_qkv;
    g.sp = c->sp_qkv; g.n_out = m->Q + 2 * m->KV;
    g.bias = Ly.bqkv; g.q = S.q; g.kc = kc; g.vc = vc;
    if ((e = run_gemm(c, S, kGQkv, l, kEpiQkv, g, s)) != hipSuccess) return e;

    aa.kc = kc; aa.vc = vc;
    // While attention runs (latency-bound, HBM mostly idle) extra workgroups read the O
    // projection's weights into the L2 of the XCD each O workgroup will run on.  Compact
    // (<= 64-row) bf16 passes only: other GEMM layouts map workgroups to blocks differently.
    aa.warm = WarmArgs{};
    if (c->warm_o && rows <= 64 && !m->nf4) {
      aa.warm.w = Ly.wo; aa.warm.kb = m->Q / kTileK; aa.warm.sp = c->sp_o; aa.warm.n = m->nb_h * c->sp_o;
      aa.warm.head = 1 << 30; aa.warm.nwarm = (aa.warm.n + 7) & ~7; aa.warm.sink = S.sink;
    }
    if ((e = launch_attention(aa, m->dh, r.B, s)) != hipSuccess) return e;

    g = base;
    g.w = Ly.wo; g.a = S.a_o; g.k = m->Q; g.kb = m->Q / kTileK; g.nb = m->nb_h; g.nw = c->nw_o;
    g.sp = c->sp_o;
    g.x = S.x; g.a_next = S.a_h; g.gain_next = Ly.g2; g.ssq_out = S.ssq; g.n_out = m->H;
    if ((e = run_gemm(c, S, kGO, l, kEpiResid, g, s)) != hipSuccess) return e;

    g = base;
    g.w = Ly.wgu; g.a = S.a_h; g.k = m->H; g.kb = m->H / kTileK; g.nb = m->nb_gu; g.nw = c->nw_gu;
    g.sp = 1;
    g.h = S.a_f; g.ffn = m->F;
    if ((e = run_gemm(c, S, kGGateUp, l, kEpiSwiglu, g, s)) != hipSuccess) return e;

    const bool last = (l + 1 == m->L);
    g = base;
    g.w = Ly.wd; g.a = S.a_f; g.k = m->F; g.kb = m->F / kTileK; g.nb = m->nb_h; g.nw = c->nw_d;
    g.x = S.x; g.a_next = S.a_h;
    g.gain_next = !last ? m->layers[l + 1].g1 : (d.has_head ? m->gfinal : m->ones);
    g.ssq_out = S.ssq; g.n_out = m->H;
    g.hidden = (last && !d.has_head) ? S.hidden : nullptr;
    g.sp = c->sp_d;
    if ((e = run_gemm(c, S, kGDown, l, kEpiResid, g, s)) != hipSuccess) return e;
  }

  const bool head = d.has_head && r.head_from >= 0;
  if (head) {
    GemmArgs g = base;
    g.w = m->head; g.a = S.a_h; g.k = m->H; g.kb = m->H / kTileK; g.nb = m->nb_head; g.nw = c->nw_head;
    g.sp = 1;
    g.amax = S.amax; g.logits = r.logits; g.vocab = m->V;
    g.row_lo = r.head_from;
    if ((e = run_gemm(c, S, kGHead, 0, kEpiArgmax, g, s)) != hipSuccess) return e;
  }

  AcceptArgs ac{};
  ac.amax = S.amax; ac.nparts = m->nb_head; ac.stage = S.stage_d; ac.len = len; ac.next = next;
  ac.result = S.res_d; ac.draft_out = r.draft_mode ? S.dout_d : nullptr; ac.B = r.B; ac.T = r.T;
  ac.has_head = head; ac.gate = r.gate;
  ac.slot_lo = head ? r.head_from : 0;
  ac.cap = c->cap;
  return launch_accept(ac, s);
}

static sf_status capture(sf_cache* c, const Run& r, hipGraphExec_t* out) {
  hipStream_t s = c->m->stream;
  hipGraph_t graph = nullptr;
  HIPCHK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
  hipError_t e = enqueue_forward(c, r);
  hipError_t e2 = hipStreamEndCapture(s, &graph);
  if (e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return fail(SF_E_HIP, std::string("capture: ") + hipGetErrorString(e));
  }
  if (e2 != hipSuccess) return fail(SF_E_HIP, std::string("end capture: ") + hipGetErrorString(e2));
  e = hipGraphInstantiate(out, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("instantiate: ") + hipGetErrorString(e));
  return SF_OK;
}

// Lay out the working memory of passes of up to R rows on cache c: take(&ptr, bytes) hands out
// each buffer (an allocation for the cache's own set, a piece of the static array for the
// no-allocation entry point).  With `own`, also the result and draft-output buffers, which the
// no-allocation entry point takes from its caller or does not need.
template <typename Take>
static sf_status plan_scratch(const sf_cache* c, size_t R, Scratch& S, bool own, Take take) {
  const sf_model* m = c->m;
  sf_status st;
  if ((st = take((void**)&S.stage_d, sizeof(Stage)))) return st;
  if ((st = take((void**)&S.x, R * m->H * 4))) return st;
  if ((st = take((void**)&S.a_h, act_bytes(2 * (int)R, m->H)))) return st;
  if ((st = take((void**)&S.a_o, act_bytes(2 * (int)R, m->Q)))) return st;
  if ((st = take((void**)&S.a_f, act_bytes(2 * (int)R, m->F)))) return st;
  if ((st = take((void**)&S.hidden, R * m->H * 2))) return st;
  if ((st = take((void**)&S.ssq, R * (m->H / kTileN) * 4))) return st;
  const size_t n_qkv = (size_t)m->Q + 2 * m->KV;
  const size_t pe = std::max({(size_t)c->sp_qkv * n_qkv, (size_t)c->sp_o * m->H, (size_t)c->sp_d * m->H});
  if ((st = take((void**)&S.part, pe * R * 4))) return st;
  S.cnt_stride = std::max(m->nb_qkv, m->nb_h) * (int)((R + 63) / 64);   // [block][64-row group]
  if ((st = take((void**)&S.cnt, (size_t)m->L * 3 * S.cnt_stride * 4))) return st;
  if ((st = take((void**)&S.q, R * m->Q * 4))) return st;
  if ((st = take((void**)&S.apart, R * m->nq * (size_t)c->nchunk * (m->dh + 2) * 4))) return st;
  if ((st = take((void**)&S.amax, R * m->nb_head * 8))) return st;
  if ((st = take((void**)&S.sink, 256))) return st;
  if (own) {
    if ((st = take((void**)&S.res_d, 4 * kMaxRows * 4))) return st;
    if ((st = take((void**)&S.dout_d, (size_t)c->B * kMaxDraftSteps * 4))) return st;
  }
  return SF_OK;
}

static void cache_release(sf_cache* c) {
  if (c->gx_verify) (void)hipGraphExecDestroy(c->gx_verify);
  if (c->gx_draft) (void)hipGraphExecDestroy(c->gx_draft);
  if (c->stage_h) (void)hipHostFree(c->stage_h);
  if (c->res_h) (void)hipHostFree(c->res_h);
  if (c->dout_h) (void)hipHostFree(c->dout_h);
  if (c->ev0) (void)hipEventDestroy(c->ev0);
  if (c->ev1) (void)hipEventDestroy(c->ev1);
  c->mem.release();
  delete c;
}

extern "C" sf_status sf_cache_alloc(sf_model* m, int32_t n_seqs, int32_t capacity, int32_t k_max,
                                    sf_cache** out) {
  if (!m || !out) return fail(SF_E_ARG, "model or out is NULL");
  *out = nullptr;
  if (k_max < 0 || k_max >= kMaxK) return fail(SF_E_ARG, "k_max must be in 0..15");
  if (n_seqs < 1 || n_seqs > kMaxSeqs || n_seqs * (k_max + 1) > kMaxRows)
    return fail(SF_E_ARG, "n_seqs must be in 1..64 and n_seqs*(k_max+1) in 1..512");
  if (capacity < k_max + 1 || capacity > kMaxCapacity) return fail(SF_E_ARG, "capacity must be in k_max+1..16384");
  if (m->nf4 && n_seqs * (k_max + 1) > kNf4MaxRows)
    return fail(SF_E_ARG, "an NF4 model runs passes of at most 64 rows: n_seqs*(k_max+1) <= 64");
  sf_cache* c = new sf_cache();
  c->m = m; c->B = n_seqs; c->cap = capacity; c->kmax = k_max; c->T = k_max + 1;
  c->nchunk = attention_spans(capacity);
  c->seq_stride = (size_t)m->nkv * capacity * m->dh;
  c->layer_stride = c->seq_stride * n_seqs;
  c->len_h.assign(n_seqs, 0); c->next_h.assign(n_seqs, 0); c->len_hi.assign(n_seqs, 0);
  c->nw_qkv = choose_nw(m->nb_qkv, m->H / kTileK, "SF_NW_QKV");
  c->nw_o = choose_nw(m->nb_h, m->Q / kTileK, "SF_NW_O");
  c->nw_gu = choose_nw(m->nb_gu, m->H / kTileK, "SF_NW_GU");
  c->nw_d = choose_nw(m->nb_h, m->F / kTileK, "SF_NW_D");
  c->nw_head = choose_nw(m->nb_head, m->H / kTileK, "SF_NW_HEAD");
  c->sp_qkv = choose_sp(m->nb_qkv, m->H / kTileK, c->nw_qkv, "SF_SP_QKV", m->nf4);
  c->sp_o = choose_sp(m->nb_h, m->Q / kTileK, c->nw_o, "SF_SP_O", m->nf4);
  c->sp_gu = 1;
  c->sp_d = choose_sp(m->nb_h, m->F / kTileK, c->nw_d, "SF_SP_D", m->nf4);
  c->sp_head = 1;
  if (const char* v = getenv("SF_KH")) c->kh = (atoi(v) == 8) ? 8 : 4;
  if (const char* v = getenv("SF_WARM_O")) c->warm_o = atoi(v) != 0;

  hipStream_t s = m->stream;
  auto bail = [&](sf_status st) { cache_release(c); return st; };
  auto dalloc = [&](void** p, size_t bytes) -> sf_status {
    hipError_t e = c->mem.alloc(p, bytes);
    if (e != hipSuccess) return fail(SF_E_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
    e = hipMemsetAsync(*p, 0, std::max<size_t>(bytes, 256), s);
    if (e != hipSuccess) return fail(SF_E_HIP, std::string("hipMemset: ") + hipGetErrorString(e));
    return SF_OK;
  };
#define TRY(x)                        \
  do {                                \
    sf_status st_ = (x);              \
    if (st_ != SF_OK) return bail(st_); \
  } while (0)
  // Rows of the largest pass this cache runs: a verify (n_seqs x (k_max+1)) or a prefill chunk.
  c->pchunk = kPrefillChunk;
  if (const char* v = getenv("SF_PREFILL_CHUNK")) c->pchunk = std::min(std::max(atoi(v), 1), kMaxRows);
  if (m->nf4) c->pchunk = std::min(c->pchunk, kNf4MaxRows);
  const size_t R = std::max(n_seqs * (k_max + 1), c->pchunk);
  const size_t pool = c->layer_stride * m->L * 2;
  TRY(dalloc((void**)&c->kpool, pool));
  TRY(dalloc((void**)&c->vpool, pool));
  TRY(dalloc((void**)&c->len, n_seqs * 4));
  TRY(dalloc((void**)&c->next, n_seqs * 4));
  TRY(plan_scratch(c, R, c->sc, true, dalloc));
  TRY(dalloc((void**)&c->rope, (size_t)capacity * (m->dh / 2) * 8));
  {
    const size_t snap = (size_t)m->L * n_seqs * m->nkv * c->T * m->dh * 2;
    TRY(dalloc((void**)&c->snap_k, snap));
    TRY(dalloc((void**)&c->snap_v, snap));
    TRY(dalloc((void**)&c->snap_len, n_seqs * 4));
    TRY(dalloc((void**)&c->snap_next, n_seqs * 4));
  }
  {
    hipError_t e = hipHostMalloc((void**)&c->stage_h, sizeof(Stage), hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void**)&c->res_h, 4 * kMaxRows * 4, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void**)&c->dout_h, (size_t)n_seqs * kMaxDraftSteps * 4, hipHostMallocDefault);
    if (e != hipSuccess) return bail(fail(SF_E_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e)));
    memset(c->stage_h, 0, sizeof(Stage));
  }
  {
    hipError_t e = launch_rope_table(c->rope, capacity, m->dh / 2, (double)m->d.rope_base, s);
    if (e == hipSuccess) e = hipEventCreate(&c->ev0);
    if (e == hipSuccess) e = hipEventCreate(&c->ev1);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return bail(fail(SF_E_HIP, std::string("cache init: ") + hipGetErrorString(e)));
  }
  TRY(capture(c, Run{n_seqs, c->T, 0, k_max, nullptr, false, false}, &c->gx_verify));
  if (m->d.has_head) TRY(capture(c, Run{n_seqs, 1, 0, 0, nullptr, true, false}, &c->gx_draft));
#undef TRY
  *out = c;
  return SF_OK;
}

extern "C" sf_status sf_cache_free(sf_cache* c) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  (void)hipStreamSynchronize(c->m->stream);
  cache_release(c);
  return SF_OK;
}

// Refresh the host copies of length / pending token from the device.
static sf_status refresh(sf_cache* c) {
  hipStream_t s = c->m->stream;
  HIPCHK(hipStreamSynchronize(s));
  HIPCHK(hipMemcpy(c->res_h, c->len, c->B * 4, hipMemcpyDeviceToHost));
  for (int b = 0; b < c->B; ++b) c->len_h[b] = c->res_h[b];
  HIPCHK(hipMemcpy(c->res_h, c->next, c->B * 4, hipMemcpyDeviceToHost));
  for (int b = 0; b < c->B; ++b) c->next_h[b] = c->res_h[b];
  c->len_hi = c->len_h;
  c->dirty = false;
  return SF_OK;
}

static size_t stage_bytes(int B, int kmax) { return offsetof(Stage, draft) + (size_t)B * std::max(kmax, 1) * 4; }

extern "C" sf_status sf_verify(sf_cache* c, const int32_t* draft, const int32_t* k, uint32_t flags,
                               int32_t* accepted, int32_t* target, void* dev_out) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  sf_model* m = c->m;
  if (flags & ~(SF_NO_COMMIT | SF_FORCE_ACCEPT | SF_DEBUG_LOGITS)) return fail(SF_E_ARG, "unknown flags");
  if (!draft && c->kmax > 0) return fail(SF_E_ARG, "draft is NULL");
  const bool dbg = (flags & SF_DEBUG_LOGITS) != 0;
  if (dbg && (!m->d.has_head || !dev_out)) return fail(SF_E_ARG, "SF_DEBUG_LOGITS needs a head and dev_out");
  if (c->dirty) {
    if (sf_status st = refresh(c)) return st;
  }
  for (int b = 0; b < c->B; ++b) {
    const int kb = k ? k[b] : c->kmax;
    if (kb < 0 || kb > c->kmax) return fail(SF_E_ARG, "k out of range");
    for (int j = 0; j < kb; ++j) {
      const int t = draft[b * c->kmax + j];
      if (t < 0 || t >= m->V) return fail(SF_E_ARG, "draft token outside [0,V)");
    }
    if (c->len_h[b] + c->T > c->cap)
      return fail(SF_E_CAPACITY, "sequence " + std::to_string(b) + ": length + k_max + 1 exceeds capacity");
  }
  hipStream_t s = m->stream;
  Stage* st = c->stage_h;
  st->flags = (int)(flags & (SF_NO_COMMIT | SF_FORCE_ACCEPT));
  st->kmax = c->kmax;
  for (int b = 0; b < c->B; ++b) {
    const int kb = k ? k[b] : c->kmax;
    st->k[b] = kb;
    st->step[b] = 0;
    for (int j = 0; j < c->kmax; ++j) st->draft[b * c->kmax + j] = (j < kb) ? draft[b * c->kmax + j] : 0;
  }
  HIPCHK(hipMemcpyAsync(c->sc.stage_d, st, stage_bytes(c->B, c->kmax), hipMemcpyHostToDevice, s));
  if (dbg) {
    hipError_t e = enqueue_forward(c, Run{c->B, c->T, 0, c->kmax, (float*)dev_out, false, false});
    if (e != hipSuccess) return fail(SF_E_HIP, std::string("forward: ") + hipGetErrorString(e));
  } else {
    HIPCHK(graph_launch(c->gx_verify, s));
  }
  // Results {accepted[B], target[B][T]}, behind the pass.
  HIPCHK(hipMemcpyAsync(c->res_h, c->sc.res_d, (size_t)(c->B + c->B * c->T) * 4, hipMemcpyDeviceToHost, s));
  if (!m->d.has_head && dev_out)
    HIPCHK(hipMemcpyAsync(dev_out, c->sc.hidden, (size_t)c->B * c->T * m->H * 2, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipStreamSynchronize(s));
  for (int b = 0; b < c->B; ++b) {
    const int M = c->res_h[b];
    if (accepted) accepted[b] = M;
    if (target)
      for (int j = 0; j < c->T; ++j) target[b * c->T + j] = c->res_h[c->B + b * c->T + j];
    if (!(flags & SF_NO_COMMIT)) {
      if (m->d.has_head) {
        c->len_h[b] += M + 1;
        c->next_h[b] = c->res_h[c->B + b * c->T + M];
      } else {
        c->len_h[b] += (k ? k[b] : c->kmax) + 1;
      }
    }
  }
  c->len_hi = c->len_h;
  return SF_OK;
}

extern "C" sf_status sf_verify_device(sf_cache* c, const int32_t* dev_draft, const int32_t* dev_k, uint32_t flags) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (flags & ~(SF_NO_COMMIT | SF_FORCE_ACCEPT)) return fail(SF_E_ARG, "unsupported flags");
  if (!dev_draft && c->kmax > 0) return fail(SF_E_ARG, "dev_draft is NULL");
  for (int b = 0; b < c->B; ++b)
    if (c->len_hi[b] + c->T > c->cap)
      return fail(SF_E_CAPACITY, "sequence " + std::to_string(b) + ": length may exceed capacity (sf_sync first)");
  hipStream_t s = c->m->stream;
  const int32_t* dd = dev_draft ? dev_draft : c->sc.res_d;
  hipError_t e = launch_stage_device(c->sc.stage_d, dd, dev_k, c->B, c->kmax, (int)flags, s);
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("stage: ") + hipGetErrorString(e));
  HIPCHK(graph_launch(c->gx_verify, s));
  if (!(flags & SF_NO_COMMIT)) {
    for (int b = 0; b < c->B; ++b) c->len_hi[b] += c->T;
    c->dirty = true;
  }
  return SF_OK;
}

// ------------------------------------------------------------------------------------------
// The no-allocation verify: sf_verify_device's pass, run eagerly with its working memory
// taken from one static device array instead of the cache's own scratch, for callers that
// cannot allocate (graph capture, tight serving loops).
//
// `scratch` is the array as this file's device code object holds it, one copy per GPU, kept
// until the process ends.  In host code its name is a host-side stand-in, not a device
// address; the device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used afterwards.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
static void* g_scratch_ptr[kMaxDevices] = {};
static std::mutex g_scratch_mu;

static sf_status static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(SF_E_ARG, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    HIPCHK(hipGetDevice(&cur));
    if (cur != dev) HIPCHK(hipSetDevice(dev));
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) HIPCHK(hipSetDevice(cur));
    if (e != hipSuccess || !ptr)
      return fail(SF_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SF_OK;
}

extern "C" sf_status sf_verify_device_static(sf_cache* c, const int32_t* dev_draft, const int32_t* dev_k,
                                             uint32_t flags, int32_t* dev_result) {
  if (!c || !dev_result) return fail(SF_E_ARG, "cache or dev_result is NULL");
  if (flags & ~(SF_NO_COMMIT | SF_FORCE_ACCEPT)) return fail(SF_E_ARG, "unsupported flags");
  if (!dev_draft && c->kmax > 0) return fail(SF_E_ARG, "dev_draft is NULL");
  for (int b = 0; b < c->B; ++b)
    if (c->len_hi[b] + c->T > c->cap)
      return fail(SF_E_CAPACITY, "sequence " + std::to_string(b) + ": length may exceed capacity (sf_sync first)");
  // Lay the pass's working memory out in the static array (256-byte aligned pieces).
  Scratch S;
  size_t need = 0;
  auto count = [&](void** p, size_t bytes) -> sf_status {
    *p = nullptr;
    need += (std::max<size_t>(bytes, 256) + 255) & ~(size_t)255;
    return SF_OK;
  };
  plan_scratch(c, (size_t)c->B * c->T, S, false, count);
  if (need > kStaticScratchBytes)
    return fail(SF_E_CAPACITY, "this pass needs " + std::to_string(need) + " bytes of working memory; the static "
                "scratch holds " + std::to_string(kStaticScratchBytes) + " (fewer sequences or a smaller capacity fit)");
  void* base = nullptr;
  if (sf_status st = static_scratch(c->m->dev, &base)) return st;
  size_t off = 0;
  auto carve = [&](void** p, size_t bytes) -> sf_status {
    *p = (uint8_t*)base + off;
    off += (std::max<size_t>(bytes, 256) + 255) & ~(size_t)255;
    return SF_OK;
  };
  plan_scratch(c, (size_t)c->B * c->T, S, false, carve);
  S.res_d = dev_result;
  hipStream_t s = c->m->stream;
  // The array keeps the previous call's contents: the split-K arrival counters must start at
  // zero (cleared by a fill kernel, which a capturing caller may record); everything else is
  // written before it is read.
  hipError_t e = launch_zero(S.cnt, (size_t)c->m->L * 3 * S.cnt_stride, s);
  if (e == hipSuccess) e = launch_stage_device(S.stage_d, dev_draft ? dev_draft : dev_result, dev_k, c->B, c->kmax,
                                               (int)flags, s);
  if (e == hipSuccess) {
    Run r{c->B, c->T, 0, c->kmax, nullptr, false, false};
    r.sc = &S;
    e = enqueue_forward(c, r);
  }
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("static verify: ") + hipGetErrorString(e));
  if (!(flags & SF_NO_COMMIT)) {
    for (int b = 0; b < c->B; ++b) c->len_hi[b] += c->T;
    c->dirty = true;
  }
  return SF_OK;
}

extern "C" sf_status sf_results_device(sf_cache* c, int32_t** dev_accepted, int32_t** dev_target) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (dev_accepted) *dev_accepted = c->sc.res_d;
  if (dev_target) *dev_target = c->sc.res_d + c->B;
  return SF_OK;
}

extern "C" sf_status sf_prefill(sf_cache* c, int32_t seq, const int32_t* tokens, int32_t n, int32_t* next_token) {
  if (!c || !tokens) return fail(SF_E_ARG, "cache or tokens is NULL");
  sf_model* m = c->m;
  if (seq < 0 || seq >= c->B) return fail(SF_E_ARG, "seq out of range");
  if (n < 1) return fail(SF_E_ARG, "n < 1");
  if (n > c->cap) return fail(SF_E_CAPACITY, "prompt longer than capacity");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= m->V) return fail(SF_E_ARG, "token outside [0,V)");
  if (c->dirty) {
    if (sf_status st = refresh(c)) return st;
  }
  hipStream_t s = m->stream;
  if (injected("launch")) return fail(SF_E_HIP, "prefill forward: injected launch failure (SF_FAULT=launch)");
  HIPCHK(launch_set_state(c->len, c->next, seq, 0, 0, 1, s));
  int last_cnt = 1;
  for (int j0 = 0; j0 < n; j0 += c->pchunk) {
    const int cnt = std::min(c->pchunk, n - j0);
    Stage* st = c->stage_h;
    st->flags = kFlagForce | kFlagFirst;
    st->kmax = cnt - 1;
    st->k[0] = cnt - 1;
    st->first[0] = tokens[j0];
    st->step[0] = 0;
    for (int j = 1; j < cnt; ++j) st->draft[j - 1] = tokens[j0 + j];
    HIPCHK(hipMemcpyAsync(c->sc.stage_d, st, stage_bytes(1, cnt - 1), hipMemcpyHostToDevice, s));
    // Every position is forced accepted and the next pass stages its own first token, so only
    // the last pass's last row needs the LM head (a pass without it commits len += cnt).
    Run run{1, cnt, seq, cnt - 1, nullptr, false, true};
    run.head_from = (j0 + cnt == n) ? cnt - 1 : -1;
    hipError_t e = enqueue_forward(c, run);
    if (e != hipSuccess) return fail(SF_E_HIP, std::string("prefill forward: ") + hipGetErrorString(e));
    HIPCHK(hipStreamSynchronize(s));  // the pinned stage block is reused by the next chunk
    last_cnt = cnt;
  }
  HIPCHK(hipMemcpy(c->res_h, c->sc.res_d, (1 + last_cnt) * 4, hipMemcpyDeviceToHost));
  c->len_h[seq] = n;
  c->len_hi[seq] = n;
  int nxt = 0;
  if (m->d.has_head) {
    nxt = c->res_h[1 + last_cnt - 1];
    c->next_h[seq] = nxt;
  }
  if (next_token) *next_token = nxt;
  return SF_OK;
}

static SnapArgs snap_args(sf_cache* c) {
  sf_model* m = c->m;
  SnapArgs a{};
  a.kpool = c->kpool; a.vpool = c->vpool; a.sk = c->snap_k; a.sv = c->snap_v;
  a.len = c->len; a.next = c->next; a.slen = c->snap_len; a.snext = c->snap_next;
  a.layer_stride = (long)c->layer_stride; a.seq_stride = (long)c->seq_stride;
  a.L = m->L; a.B = c->B; a.nkv = m->nkv; a.cap = c->cap; a.dh = m->dh; a.T = c->T;
  return a;
}

extern "C" sf_status sf_snapshot_save(sf_cache* c) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  const hipError_t e = launch_snapshot(snap_args(c), 1, c->m->stream);
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("snapshot save: ") + hipGetErrorString(e));
  c->snap_valid = true;
  return SF_OK;
}

extern "C" sf_status sf_snapshot_restore(sf_cache* c) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (!c->snap_valid) return fail(SF_E_STATE, "no snapshot has been saved on this cache");
  const hipError_t e = launch_snapshot(snap_args(c), 0, c->m->stream);
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("snapshot restore: ") + hipGetErrorString(e));
  c->dirty = true;
  return SF_OK;
}

extern "C" sf_status sf_rollback(sf_cache* c, int32_t seq, int32_t pos) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (seq < 0 || seq >= c->B) return fail(SF_E_ARG, "seq out of range");
  if (c->dirty) {
    if (sf_status st = refresh(c)) return st;
  }
  if (pos < 0 || pos > c->len_h[seq]) return fail(SF_E_STATE, "rollback position outside 0..length");
  HIPCHK(launch_set_state(c->len, c->next, seq, pos, 0, 1, c->m->stream));
  c->len_h[seq] = pos;
  c->len_hi[seq] = pos;
  return SF_OK;
}

extern "C" sf_status sf_set_next(sf_cache* c, int32_t seq, int32_t token) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (seq < 0 || seq >= c->B) return fail(SF_E_ARG, "seq out of range");
  if (token < 0 || token >= c->m->V) return fail(SF_E_ARG, "token outside [0,V)");
  HIPCHK(launch_set_state(c->len, c->next, seq, 0, token, 2, c->m->stream));
  c->next_h[seq] = token;
  return SF_OK;
}

extern "C" sf_status sf_cache_state(sf_cache* c, int32_t seq, int32_t* length, int32_t* next_token) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (seq < 0 || seq >= c->B) return fail(SF_E_ARG, "seq out of range");
  if (sf_status st = refresh(c)) return st;
  if (length) *length = c->len_h[seq];
  if (next_token) *next_token = c->next_h[seq];
  return SF_OK;
}

extern "C" sf_status sf_sync(sf_cache* c) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  return refresh(c);
}

extern "C" sf_status sf_draft_step(sf_cache* c, int32_t n_steps, int32_t* tokens) {
  if (!c) return fail(SF_E_ARG, "cache is NULL");
  if (!c->m->d.has_head || !c->gx_draft) return fail(SF_E_STATE, "draft steps need a stack with a head");
  if (n_steps < 1 || n_steps > kMaxDraftSteps) return fail(SF_E_ARG, "n_steps must be in 1..256");
  if (c->dirty) {
    if (sf_status st = refresh(c)) return st;
  }
  for (int b = 0; b < c->B; ++b)
    if (c->len_h[b] + n_steps > c->cap) return fail(SF_E_CAPACITY, "length + n_steps exceeds capacity");
  hipStream_t s = c->m->stream;
  Stage* st = c->stage_h;
  st->flags = 0;
  st->kmax = 0;
  for (int b = 0; b < c->B; ++b) { st->k[b] = 0; st->step[b] = 0; }
  HIPCHK(hipMemcpyAsync(c->sc.stage_d, st, stage_bytes(c->B, 0), hipMemcpyHostToDevice, s));
  for (int i = 0; i < n_steps; ++i) HIPCHK(graph_launch(c->gx_draft, s));
  HIPCHK(hipMemcpyAsync(c->dout_h, c->sc.dout_d, (size_t)c->B * kMaxDraftSteps * 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  for (int b = 0; b < c->B; ++b) {
    for (int i = 0; i < n_steps; ++i)
      if (tokens) tokens[b * n_steps + i] = c->dout_h[b * kMaxDraftSteps + i];
    c->len_h[b] += n_steps;
    c->next_h[b] = c->dout_h[b * kMaxDraftSteps + n_steps - 1];
  }
  c->len_hi = c->len_h;
  return SF_OK;
}

// ------------------------------------------------------------------------------------------
// Device-resident speculative round: drafter steps, verify, accept and the drafter's rewind,
// captured once into one graph over two caches that share a stream.
struct sf_round {
  sf_cache* d = nullptr;
  sf_cache* v = nullptr;
  int k = 0;
  int32_t* scratch = nullptr;
  hipGraphExec_t gx = nullptr;
};

static void round_release(sf_round* r) {
  if (r->gx) (void)hipGraphExecDestroy(r->gx);
  if (r->scratch) (void)hipFree(r->scratch);
  delete r;
}

extern "C" sf_status sf_round_create(sf_cache* d, sf_cache* v, int32_t k, sf_round** out) {
  if (!d || !v || !out) return fail(SF_E_ARG, "NULL argument");
  *out = nullptr;
  if (d == v) return fail(SF_E_ARG, "drafter and verifier must be different caches");
  if (!d->m->d.has_head || !v->m->d.has_head || !d->gx_draft)
    return fail(SF_E_STATE, "both stacks need an LM head");
  if (d->B != v->B) return fail(SF_E_ARG, "drafter and verifier must hold the same number of sequences");
  if (d->m->stream != v->m->stream) return fail(SF_E_ARG, "drafter and verifier models must share one stream");
  if (d->m->V > v->m->V) return fail(SF_E_ARG, "the drafter's vocabulary must not exceed the verifier's");
  if (k < 1 || k > v->kmax) return fail(SF_E_ARG, "k must be in 1..verifier k_max");
  sf_round* r = new sf_round();
  r->d = d;
  r->v = v;
  r->k = k;
  // [0, B): verifier lengths; [B, 2B): catch-up needed per sequence; [2B]: any of them.
  hipError_t e = dev_malloc((void**)&r->scratch, (size_t)(2 * d->B + 1) * 4);
  if (e != hipSuccess) {
    round_release(r);
    return fail(SF_E_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
  }
  RoundArgs a{};
  a.dstage = d->sc.stage_d; a.vstage = v->sc.stage_d; a.dlen = d->len; a.dnext = d->next; a.vlen = v->len;
  a.vnext = v->next; a.dout = d->sc.dout_d; a.vres = v->sc.res_d; a.scratch = r->scratch;
  a.B = d->B; a.k = k; a.vkmax = v->kmax; a.vT = v->T;
  const Run draft{d->B, 1, 0, 0, nullptr, true, false};
  const Run verify{v->B, v->T, 0, v->kmax, nullptr, false, false};
  hipStream_t s = d->m->stream;
  hipGraph_t graph = nullptr;
  e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t c = launch_round(a, kRoundBegin, s);
    for (int i = 0; i < k && c == hipSuccess; ++i) c = enqueue_forward(d, draft);
    if (c == hipSuccess) c = launch_round(a, kRoundStage, s);
    if (c == hipSuccess) c = enqueue_forward(v, verify);
    if (c == hipSuccess) c = launch_round(a, kRoundReconcile, s);
    // Catch-up step, commit off; its kernels return at once unless a sequence needs it.
    Run catchup = draft;
    catchup.gate = r->scratch + 2 * d->B;
    if (c == hipSuccess) c = enqueue_forward(d, catchup);
    if (c == hipSuccess) c = launch_round(a, kRoundFinish, s);
    const hipError_t ce = hipStreamEndCapture(s, &graph);
    e = (c != hipSuccess) ? c : ce;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&r->gx, graph, nullptr, nullptr, 0);
  if (graph) (void)hipGraphDestroy(graph);
  if (e != hipSuccess) {
    round_release(r);
    return fail(SF_E_HIP, std::string("round capture: ") + hipGetErrorString(e));
  }
  *out = r;
  return SF_OK;
}

extern "C" sf_status sf_round_run(sf_round* r, int32_t n_rounds) {
  if (!r) return fail(SF_E_ARG, "round is NULL");
  if (n_rounds < 1 || n_rounds > 1 << 20) return fail(SF_E_ARG, "n_rounds out of range");
  sf_cache* d = r->d;
  sf_cache* v = r->v;
  if (d->dirty)
    if (sf_status st = refresh(d)) return st;
  if (v->dirty)
    if (sf_status st = refresh(v)) return st;
  const long grow = (long)n_rounds * (r->k + 1);
  for (int b = 0; b < d->B; ++b) {
    if (d->len_h[b] != v->len_h[b] || d->next_h[b] != v->next_h[b])
      return fail(SF_E_STATE, "sequence " + std::to_string(b) + ": drafter and verifier are not at the same point");
    if (v->len_h[b] + grow + v->T > v->cap || d->len_h[b] + grow + v->T > d->cap)
      return fail(SF_E_CAPACITY, "sequence " + std::to_string(b) + ": the rounds may exceed a capacity");
  }
  hipStream_t s = d->m->stream;
  for (int i = 0; i < n_rounds; ++i) HIPCHK(graph_launch(r->gx, s));
  for (int b = 0; b < d->B; ++b) {
    d->len_hi[b] += (int)grow;
    v->len_hi[b] += (int)grow;
  }
  d->dirty = v->dirty = true;
  return SF_OK;
}

extern "C" sf_status sf_round_free(sf_round* r) {
  if (!r) return fail(SF_E_ARG, "round is NULL");
  (void)hipStreamSynchronize(r->d->m->stream);
  round_release(r);
  return SF_OK;
}

extern "C" int32_t sf_ngram_propose(const int32_t* hist, int32_t n_hist, int32_t min_n, int32_t max_n,
                                    int32_t k_max, int32_t* out) {
  if ((!hist && n_hist > 0) || n_hist < 0 || min_n < 1 || max_n < min_n || k_max < 0 || (!out && k_max > 0))
    return fail(SF_E_ARG, "bad n-gram arguments");
  for (int n = max_n; n >= min_n; --n) {
    if (n_hist < n + 1) continue;
    const int32_t* suf = hist + n_hist - n;
    for (int j = n_hist - n - 1; j >= 0; --j) {
      if (memcmp(hist + j, suf, (size_t)n * sizeof(int32_t)) == 0) {
        const int cnt = std::min(k_max, n_hist - (j + n));
        for (int i = 0; i < cnt; ++i) out[i] = hist[j + n + i];
        return cnt;
      }
    }
  }
  return 0;
}

extern "C" sf_status sf_kv_write(sf_cache* c, int32_t seq, const void* dev_k, const void* dev_v, int32_t n_pos,
                                 int32_t src_positions) {
  if (!c || !dev_k || !dev_v) return fail(SF_E_ARG, "NULL argument");
  if (seq < 0 || seq >= c->B) return fail(SF_E_ARG, "seq out of range");
  if (n_pos < 0 || src_positions < n_pos) return fail(SF_E_ARG, "bad n_pos / src_positions");
  if (n_pos > c->cap) return fail(SF_E_CAPACITY, "n_pos exceeds capacity");
  // The caller's buffers may have been written on any stream (a torch fill or copy on its own
  // stream does not order before the model stream): wait for the whole device first.
  HIPCHK(hipDeviceSynchronize());
  if (c->dirty) {
    if (sf_status st = refresh(c)) return st;
  }
  sf_model* m = c->m;
  hipStream_t s = m->stream;
  const size_t off = (size_t)seq * c->seq_stride;
  HIPCHK(launch_copy_kv(c->kpool + off, (uint16_t*)dev_k, (long)c->layer_stride, m->nkv, c->cap, m->dh, m->L, n_pos,
                        src_positions, 1, s));
  HIPCHK(launch_copy_kv(c->vpool + off, (uint16_t*)dev_v, (long)c->layer_stride, m->nkv, c->cap, m->dh, m->L, n_pos,
                        src_positions, 1, s));
  HIPCHK(launch_set_state(c->len, c->next, seq, n_pos, 0, 1, s));
  HIPCHK(hipStreamSynchronize(s));
  c->len_h[seq] = n_pos;
  c->len_hi[seq] = n_pos;
  return SF_OK;
}

extern "C" sf_status sf_kv_read(sf_cache* c, int32_t seq, void* dev_k, void* dev_v, int32_t n_pos,
                                int32_t dst_positions) {
  if (!c || !dev_k || !dev_v) return fail(SF_E_ARG, "NULL argument");
  if (seq < 0 || seq >= c->B) return fail(SF_E_ARG, "seq out of range");
  if (n_pos < 0 || dst_positions < n_pos || n_pos > c->cap) return fail(SF_E_ARG, "bad n_pos / dst_positions");
  // As in sf_kv_write: a fill of the destination still pending on another stream must not
  // land after the copy.
  HIPCHK(hipDeviceSynchronize());
  sf_model* m = c->m;
  hipStream_t s = m->stream;
  const size_t off = (size_t)seq * c->seq_stride;
  HIPCHK(launch_copy_kv(c->kpool + off, (uint16_t*)dev_k, (long)c->layer_stride, m->nkv, c->cap, m->dh, m->L, n_pos,
                        dst_positions, 0, s));
  HIPCHK(launch_copy_kv(c->vpool + off, (uint16_t*)dev_v, (long)c->layer_stride, m->nkv, c->cap, m->dh, m->L, n_pos,
                        dst_positions, 0, s));
  HIPCHK(hipStreamSynchronize(s));
  return SF_OK;
}

extern "C" sf_status sf_time_kernel(sf_cache* c, int32_t kernel, int32_t iters, float* avg_us, double* bytes) {
  if (!c || !avg_us) return fail(SF_E_ARG, "NULL argument");
  if (iters < 1 || iters > 100000) return fail(SF_E_ARG, "iters out of range");
  sf_model* m = c->m;
  if (kernel < SF_KERNEL_QKV || kernel > SF_KERNEL_VERIFY) return fail(SF_E_ARG, "unknown kernel");
  if (kernel == SF_KERNEL_LMHEAD && !m->d.has_head) return fail(SF_E_ARG, "no LM head");
  if (c->dirty) {
    if (sf_status st = refresh(c)) return st;
  }
  for (int b = 0; b < c->B; ++b)
    if (c->len_h[b] + c->T > c->cap) return fail(SF_E_CAPACITY, "length + k_max + 1 exceeds capacity");
  hipStream_t s = m->stream;
  const int rows = c->B * c->T;
  double L_total = 0;
  for (int b = 0; b < c->B; ++b) L_total += c->len_h[b] + c->T;
  if (kernel == SF_KERNEL_VERIFY) {
    Stage* st = c->stage_h;
    st->flags = kFlagNoCommit;
    st->kmax = c->kmax;
    for (int b = 0; b < c->B; ++b) { st->k[b] = 0; st->step[b] = 0; }
    for (int j = 0; j < c->B * c->kmax; ++j) st->draft[j] = 0;
    HIPCHK(hipMemcpyAsync(c->sc.stage_d, st, stage_bytes(c->B, c->kmax), hipMemcpyHostToDevice, s));
    HIPCHK(graph_launch(c->gx_verify, s));  // warm-up
    HIPCHK(hipEventRecord(c->ev0, s));
    for (int i = 0; i < iters; ++i) HIPCHK(graph_launch(c->gx_verify, s));
    HIPCHK(hipEventRecord(c->ev1, s));
    HIPCHK(hipEventSynchronize(c->ev1));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, c->ev0, c->ev1));
    HIPCHK(hipMemcpy(c->res_h, c->sc.res_d, 4 * kMaxRows * 4, hipMemcpyDeviceToHost));
    *avg_us = ms * 1000.f / iters;
    if (bytes) {
      const double kvdim = (double)m->KV;
      double w = (double)m->L * (proj_bytes(m, m->Q + 2 * m->KV, m->H) + proj_bytes(m, m->H, m->Q) +
                                 proj_bytes(m, 2.0 * m->F, m->H) + proj_bytes(m, m->H, m->F));
      w += (double)m->L * ((m->Q + 2 * m->KV) + 2.0 * m->H) * 2;  // q/k/v biases and norm gains (bf16)
      if (m->d.has_head) w += ((double)m->V * m->H + m->H) * 2;
      w += (double)rows * m->H * 2;                                  // embedding rows
      const double kv = (double)m->L * (L_total * 2.0 * kvdim * 2 + (double)rows * 2.0 * kvdim * 2);
      *bytes = w + kv;
    }
    return SF_OK;
  }
  GemmArgs base{};
  base.rows = rows; base.ssq_in = c->sc.ssq; base.part = c->sc.part; base.sp = 1;
  base.nparts_in = m->H / kTileN; base.eps = m->d.rms_eps; base.T = c->T; base.len = c->len; base.cap = c->cap;
  base.seq_stride = (long)c->seq_stride; base.rope = c->rope; base.nq = m->nq; base.nkv = m->nkv; base.dh = m->dh;
  double by = 0;
  auto launch = [&](int it) -> hipError_t {
    const int l = it % m->L;
    const Layer& Ly = m->layers[l];
    uint16_t* kc = c->kpool + (size_t)l * c->layer_stride;
    uint16_t* vc = c->vpool + (size_t)l * c->layer_stride;
    GemmArgs g = base;
    switch (kernel) {
      case SF_KERNEL_QKV:
        g.w = Ly.wqkv; g.a = c->sc.a_h; g.k = m->H; g.kb = m->H / kTileK; g.nb = m->nb_qkv; g.nw = c->nw_qkv;
        g.bias = Ly.bqkv; g.q = c->sc.q; g.kc = kc; g.vc = vc; g.sp = c->sp_qkv; g.n_out = m->Q + 2 * m->KV;
        by = proj_bytes(m, m->Q + 2 * m->KV, m->H) + (double)rows * (m->H * 4 + m->Q * 4 + 2 * m->KV * 2);
        return run_gemm(c, c->sc, kGQkv, l, kEpiQkv, g, s);
      case SF_KERNEL_ATTENTION: {
        AttnArgs aa{};
        aa.q = c->sc.q; aa.kc = kc; aa.vc = vc; aa.seq_stride = (long)c->seq_stride; aa.cap = c->cap; aa.len = c->len;
        aa.T = c->T; aa.nq = m->nq; aa.nkv = m->nkv; aa.nchunk = c->nchunk;
        aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)m->dh));
        aa.part = c->sc.apart; aa.out = c->sc.a_o; aa.rows = rows; aa.dh = m->dh;
        by = L_total * 2.0 * m->KV * 2 + (double)rows * (m->Q * 4 + m->Q * 2);
        return launch_attention(aa, m->dh, c->B, s);
      }
      case SF_KERNEL_OPROJ:
        g.w = Ly.wo; g.a = c->sc.a_o; g.k = m->Q; g.kb = m->Q / kTileK; g.nb = m->nb_h; g.nw = c->nw_o;
        g.x = c->sc.x; g.a_next = c->sc.a_h; g.gain_next = Ly.g2; g.ssq_out = c->sc.ssq; g.n_out = m->H; g.sp = c->sp_o;
        by = proj_bytes(m, m->H, m->Q) + (double)rows * (m->Q * 4 + m->H * (4 + 4 + 4));
        return run_gemm(c, c->sc, kGO, l, kEpiResid, g, s);
      case SF_KERNEL_GATEUP:
        g.w = Ly.wgu; g.a = c->sc.a_h; g.k = m->H; g.kb = m->H / kTileK; g.nb = m->nb_gu; g.nw = c->nw_gu;
        g.h = c->sc.a_f; g.ffn = m->F; g.sp = 1;
        by = proj_bytes(m, 2.0 * m->F, m->H) + (double)rows * (m->H * 4 + m->F * 4);
        return run_gemm(c, c->sc, kGGateUp, l, kEpiSwiglu, g, s);
      case SF_KERNEL_DOWN:
        g.w = Ly.wd; g.a = c->sc.a_f; g.k = m->F; g.kb = m->F / kTileK; g.nb = m->nb_h; g.nw = c->nw_d;
        g.x = c->sc.x; g.a_next = c->sc.a_h; g.gain_next = Ly.g1; g.ssq_out = c->sc.ssq; g.n_out = m->H; g.sp = c->sp_d;
        by = proj_bytes(m, m->H, m->F) + (double)rows * (m->F * 4 + m->H * (4 + 4 + 4));
        return run_gemm(c, c->sc, kGDown, l, kEpiResid, g, s);
      default:
        g.w = m->head; g.a = c->sc.a_h; g.k = m->H; g.kb = m->H / kTileK; g.nb = m->nb_head; g.nw = c->nw_head;
        g.amax = c->sc.amax; g.vocab = m->V; g.sp = 1;
        by = (double)m->V * m->H * 2 + (double)rows * (m->H * 4 + m->nb_head * 8);
        return run_gemm(c, c->sc, kGHead, 0, kEpiArgmax, g, s);
    }
  };
  hipError_t e = launch(0);  // warm-up
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("launch: ") + hipGetErrorString(e));
  HIPCHK(hipEventRecord(c->ev0, s));
  for (int it = 0; it < iters; ++it) {
    e = launch(it + 1);
    if (e != hipSuccess) return fail(SF_E_HIP, std::string("launch: ") + hipGetErrorString(e));
  }
  HIPCHK(hipEventRecord(c->ev1, s));
  HIPCHK(hipEventSynchronize(c->ev1));
  float ms = 0;
  HIPCHK(hipEventElapsedTime(&ms, c->ev0, c->ev1));
  *avg_us = ms * 1000.f / iters;
  if (bytes) *bytes = by;
  return SF_OK;
}

extern "C" sf_status sf_debug_counters(sf_cache* c, int64_t* sum, int32_t* max) {
  if (!c || !sum || !max) return fail(SF_E_ARG, "NULL argument");
  const size_t n = (size_t)c->m->L * 3 * c->sc.cnt_stride;
  std::vector<int32_t> h(n);
  HIPCHK(hipStreamSynchronize(c->m->stream));
  HIPCHK(hipMemcpy(h.data(), c->sc.cnt, n * 4, hipMemcpyDeviceToHost));
  int64_t s = 0;
  int32_t mx = 0;
  for (int32_t v : h) {
    s += v;
    mx = std::max(mx, v);
  }
  *sum = s;
  *max = mx;
  return SF_OK;
}

extern "C" sf_status sf_debug_checks(uint32_t* bits, int32_t clear) {
  if (!bits) return fail(SF_E_ARG, "bits is NULL");
  *bits = 0;
  const hipError_t e = read_checks(bits, clear != 0);
  if (e == hipErrorNotSupported) return fail(SF_E_STATE, "built without device checks");
  if (e != hipSuccess) return fail(SF_E_HIP, std::string("checks: ") + hipGetErrorString(e));
  return SF_OK;
}

extern "C" const char* sf_last_error(void) { return g_err.c_str(); }
