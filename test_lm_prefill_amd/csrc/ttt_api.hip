// Host side of libttt: handle, weight packing, the per-chunk step of
// Algorithm 1 (reading notes, section 7) and its HIP-graph replay.
//
// One chunk step, all on one stream, no host synchronisation:
//   forward  embed -> L x [RMSNorm, QKV GEMM, QK-norm + rotary + ring write,
//            window attention, O GEMM (+residual), RMSNorm, gate|up GEMM with
//            fused SwiGLU, down GEMM (+residual)] -> final RMSNorm ->
//            LM-head GEMM, slab by slab, with the cross-entropy partials and
//            the shifted exponentials fused, and the product of those with the
//            head (dX of the head) -> row reduce (losses recorded here, before
//            any update: Alg. 1 step 3.3)
//   backward (skipped with TTT_NO_UPDATE) the head's dX finished from the
//            losses -> final RMSNorm backward -> for blocks L-1 .. L-n_u: MLP
//            backward with the fast-weight gradient GEMMs carrying the SGD
//            step in their epilogue (Eq. 9), then (above block L-n_u) the
//            attention sub-block backward; keys/values of earlier chunks are
//            constants.
//   counter  the device-side chunk start advances by the chunk size.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ttt.h"
#include "attn.h"
#include "elem.h"
#include "gemm.h"

// ----------------------------------------------------------------------------
// Static scratch for ttt_prefill_noalloc: the partial results of split-K products
// (first SCRATCH_GEMM_FLOATS floats) and of key-range-split attention (the rest)
// live in this array instead of the handle's workspaces.  Each device holds its own
// copy from the library's load until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: its device address is taken
// once per device with hipGetSymbolAddress (scratch_setup) and only that address
// is passed to kernels.
constexpr size_t SCRATCH_BYTES = (size_t)160 << 20;
constexpr size_t SCRATCH_GEMM_FLOATS = (size_t)24 << 20;  // 96 MiB of split-K partials
constexpr size_t SCRATCH_ATTN_FLOATS = SCRATCH_BYTES / 4 - SCRATCH_GEMM_FLOATS;  // 64 MiB
static __device__ __align__(256) float scratch[SCRATCH_BYTES / 4];

namespace {

thread_local std::string g_thread_err;

// device address of `scratch` per device (nullptr until set up), guarded by g_scratch_mu
constexpr int SCRATCH_MAX_DEV = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[SCRATCH_MAX_DEV] = {};

struct LayerBuf {
  void *attn_norm = nullptr, *wqkv = nullptr, *wo = nullptr, *q_norm = nullptr, *k_norm = nullptr,
       *mlp_norm = nullptr;
  // gate/up rows interleaved by 16.  Frozen layers: [2F][d].  Updated layers:
  // per sequence, fast rows [2F][2d] holding the forward working copy as hi | lo
  // (in bf16 mode fp16 of s*W with s = wscale: hi = round(sW), lo = round(sW -
  // hi), so hi + lo carries the fp32 master to ~22 bits and the small inner
  // updates are not lost to rounding); the static rows [2F][d] in wgu_s.
  void *wgu = nullptr, *wgu_s = nullptr;
  // Frozen layers: [d][F].  Updated layers: per sequence [d][3F] = fast hi |
  // static | fast lo (each sequence holds its own copy of the static columns, so
  // that one product covers both MLPs).
  void *wd = nullptr;
  bool fast = false, bwd_attn = false;
  int u = -1;
  float sbound = 0.f;  // bound of the scaled scores (log2 units) for the bounded forward, 0 = none
  int fsplit = 1;      // key-range split of the forward
  int R = 0;           // ring rows: k + b, or k + G for the frozen prefix run in groups of G tokens
  bool fwd16 = false;  // attention forward operands (q, ring K and V^T) are fp16
  // ring planes: K, Vt in the attention forward's type; Kb (bf16 copy of K when the
  // forward is fp16), Kt, V in the working dtype for the backward
  void *K = nullptr, *Vt = nullptr, *Kb = nullptr, *Kt = nullptr, *V = nullptr;
  // transposed working copies used by the backward GEMMs (k-contiguous
  // operands); the first three are fp16 in bf16 mode (the MLP backward and the
  // dO product take fp16 operands), wqkvT is bf16
  void *wdT = nullptr;    // [2F][d]  (fast units first), updated layers
  void *wguT = nullptr;   // [d][4F], updated layers
  void *woT = nullptr;    // [d][d], layers whose attention is back-propagated
  void *wqkvT = nullptr;  // [d][3d], same
};

struct Saved {
  float *h_in = nullptr, *r1 = nullptr, *lse2 = nullptr, *h1 = nullptr, *r2 = nullptr;
  float *qkv = nullptr;  // [b][3d] fp32
  // qh: forward q (attention forward type); qhb / qht: working-dtype copies for the backward
  void *qh = nullptr, *qhb = nullptr, *qht = nullptr, *o = nullptr, *m = nullptr, *gu = nullptr, *hmid = nullptr;
};

}  // namespace

struct ttt_handle {
  ttt_config cfg;
  int dt = 0;
  size_t es = 4;
  // bf16 mode: the forward copies of the updated blocks' MLP weights (fast hi | lo
  // and the static down projection) are stored multiplied by this power of two,
  // which keeps the fp16 lo part of small weights out of the subnormal range;
  // the GEMMs that read them divide their accumulators by it.  1 in fp32 mode.
  float wscale = 1.f;
  // independent sequences per call; each has its own fast weights (and their
  // copies) and ring; the frozen weights and the chunk scratch rows are shared
  int B = 1;
  size_t ring_sbytes = 0;                          // ring bytes of one sequence
  size_t fgu_sb = 0, fd_sb = 0, fdT_sb = 0, fguT_sb = 0;  // per-sequence strides of the fast copies (bytes)
  long ld_tok = 0;                                 // ids per sequence in tok (max_tokens + 1)
  int *ids = nullptr, *labs = nullptr;             // [B*b] the chunk's ids and labels
  int *zero = nullptr;                             // a device 0 (offset for gathered rows)
  float *closs = nullptr;                          // [B*b] the chunk's losses before the scatter
  // bf16 mode: the backward carries the chunk loss times this power of two (so
  // that its fp16 operands sit well inside fp16's normal range); the SGD step
  // divides it out.  1 in fp32 mode.
  float gscale = 1.f;
  int L = 0, d = 0, H = 0, hd = 0, F = 0, V = 0, k = 0, b = 0, nu = 0, R = 0, Vs = 0, P = 0;
  std::vector<void *> allocs;
  std::vector<std::pair<void *, size_t>> zero_list;
  std::string err;
  // weights
  void *tok_emb = nullptr, *lm_head = nullptr, *final_norm = nullptr;
  std::vector<LayerBuf> layers;
  std::vector<float *> m_gu, m_d, i_gu, i_d;  // fp32 master and initial fast weights
  // state and scratch
  int *tok = nullptr, *pos0 = nullptr, *flag = nullptr;
  float *losses = nullptr;
  float2 *rope = nullptr;
  void *ring_base = nullptr;
  size_t ring_bytes = 0;
  float *h = nullptr, *lse2 = nullptr, *hf = nullptr, *rf = nullptr, *zlab = nullptr, *lse = nullptr;
  float *shift = nullptr;  // per-row shift of the single-pass head [B b]
  bool head1 = false;      // the head's loss and gradient in one pass (exact for these weights)
  float *qkv = nullptr;  // [b][3d] fp32
  void *a = nullptr, *qh = nullptr, *o = nullptr, *m = nullptr, *hmid = nullptr, *nf = nullptr;
  float2 *part = nullptr;
  void *dz = nullptr, *dy = nullptr, *dhmid = nullptr, *dgu = nullptr, *dO = nullptr, *dOt = nullptr, *dqkv = nullptr;
  void *lm_headT = nullptr;                                  // [d][V]
  void *dyT = nullptr, *hmidT = nullptr, *dguT = nullptr, *mT = nullptr;  // [rows][b], zero past the chunk
  float *dn = nullptr, *dh = nullptr, *dm = nullptr, *Dq = nullptr, *dq = nullptr, *dk = nullptr, *dv = nullptr,
        *da = nullptr;
  float *ws = nullptr;
  size_t ws_elems = 0;
  int attn_split = 1;
  int dec_split = 1;   // key-range split of the forward for chunks of at most 16 rows (decode steps)
  // Frozen prefix: blocks 0 .. Lf-1 carry no fast weights, so a prefill runs them over groups
  // of G tokens (a multiple of b) ahead of the chunk loop; their output residual rows wait in
  // h_lead [B][G][d].  G = 0: no grouping (every chunk step runs all blocks).
  int G = 0, Lf = 0;
  float *h_lead = nullptr;
  int *lead_n = nullptr;  // device: rows per sequence of the current group (G, or fewer at the end)
  // The frozen-prefix pass writes its own scratch rows and residual rows (ls.h) and
  // keeps its own position counter (ls.pos0, advanced by each pass), so that the next
  // group's pass can run on lead_st beside the current group's chunk steps; ls.h is
  // copied into h_lead when those steps are done.
  struct LeadScratch {
    int *pos0 = nullptr, *ids = nullptr, *labs = nullptr;
    float *h = nullptr, *lse2 = nullptr, *qkv = nullptr;
    void *a = nullptr, *qh = nullptr, *o = nullptr, *m = nullptr, *hmid = nullptr;
  } ls;
  hipStream_t lead_st = nullptr;
  // [0] a frozen-prefix pass is done (lead_st), [1] the prefill's stream has taken its rows
  hipEvent_t ev_lead[2] = {nullptr, nullptr};
  float *attn_ws = nullptr;
  size_t attn_ws_n = 0;      // floats of attn_ws
  int dev = 0;               // device the handle lives on
  float *scratch = nullptr;  // this device's static scratch (device address), or nullptr
  std::string scratch_err;   // why it is unavailable
  std::vector<Saved> saved;
  // graphs: [0] update, [1] no-update
  // captured steps: full-chunk prefill with / without update, decode step greedy /
  // forced, full-chunk recompute-and-update of a decoded chunk
  // [5]: the frozen prefix over a full group of G tokens
  hipGraphExec_t gexec[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  // continuation state for ttt_decode: positions processed, start of the open
  // decode chunk, and whether a prefill has set them
  int64_t len = 0, dstart = 0;
  bool have_state = false;
  float *rlosses = nullptr;  // [max_tokens] losses of recomputed decode chunks
  int *part_arg = nullptr;   // [b][P] argmax columns beside the CE partials
  hipStream_t cap = nullptr;
  int64_t chunks_last = 0;
  int64_t launches = 0;
  // events on the caller's stream at the start and the end of the last prefill
  hipEvent_t ev_pf[2] = {nullptr, nullptr};
  bool ev_pf_set = false;
  // kernel-class timing (diagnostics)
  bool prof = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_cls;
  int ev_used = 0;
  double kt_ms[32] = {0};
  int64_t kt_n[32] = {0};
};

namespace {

struct HipFail {
  hipError_t e;
  const char *what;
};

#define HIPCHK(x)                               \
  do {                                          \
    hipError_t e_ = (x);                        \
    if (e_ != hipSuccess) throw HipFail{e_, #x}; \
  } while (0)

void *dalloc(ttt_handle *h, size_t bytes, bool zero = true) {
  void *p = nullptr;
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) throw HipFail{e, "hipMalloc"};
  h->allocs.push_back(p);
  if (zero) h->zero_list.push_back({p, bytes});
  return p;
}


GemmArgs gargs(const void *A, long lda, const void *B, long ldb, int M, int N, int K) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.alpha = 1.f;
  g.acc_scale = 1.f;
  g.c_scale = 1.f;
  return g;
}

char *off(void *p, size_t bytes) { return reinterpret_cast<char *>(p) + bytes; }

enum KClass {
  K_EMBED, K_RMSNORM, K_GEMM_QKV, K_ROPE, K_ATTN_FWD, K_GEMM_O, K_GEMM_GATE_UP, K_GEMM_DOWN, K_GEMM_HEAD_CE,
  K_CE_REDUCE, K_GEMM_DN, K_RMSNORM_BWD, K_GEMM_DHMID, K_GEMM_DW_SGD, K_SWIGLU_BWD, K_GEMM_DM,
  K_GEMM_DO, K_ATTN_BWD_PRE, K_ATTN_BWD_DQ, K_ATTN_BWD_DKDV, K_ROPE_BWD, K_GEMM_DA, K_TRANSPOSE, K_SPLITK_REDUCE, K_ATTN_MERGE, K_MISC, K_NCLASS
};
const char *const kclass_names[K_NCLASS] = {
    "embed", "rmsnorm", "gemm_qkv", "qknorm_rope_ring", "attn_fwd", "gemm_o_residual", "gemm_gate_up_swiglu",
    "gemm_down_residual", "gemm_lmhead_ce", "ce_reduce", "gemm_dn", "rmsnorm_bwd", "gemm_dhmid",
    "gemm_dw_sgd", "swiglu_bwd", "gemm_dm", "gemm_do", "attn_bwd_pre", "attn_bwd_dq", "attn_bwd_dkdv",
    "qknorm_rope_bwd", "gemm_da", "transpose", "splitk_reduce", "attn_merge", "misc"};

// Brackets one kernel group with events when kernel timing is on.
struct Prof {
  ttt_handle *h;
  hipStream_t st;
  int idx = -1;
  Prof(ttt_handle *h_, int cls, hipStream_t st_) : h(h_), st(st_) {
    if (!h->prof) return;
    if ((size_t)(2 * h->ev_used + 2) > h->ev.size()) {
      hipEvent_t a, b;
      HIPCHK(hipEventCreate(&a));
      HIPCHK(hipEventCreate(&b));
      h->ev.push_back(a);
      h->ev.push_back(b);
      h->ev_cls.push_back(0);
    }
    idx = h->ev_used++;
    h->ev_cls[idx] = cls;
    HIPCHK(hipEventRecord(h->ev[2 * idx], st));
  }
  ~Prof() {
    if (idx >= 0) (void)hipEventRecord(h->ev[2 * idx + 1], st);
  }
};

// Adds the recorded intervals of the last chunk to the per-class totals.
void prof_collect(ttt_handle *h, hipStream_t st) {
  if (!h->prof || h->ev_used == 0) return;
  HIPCHK(hipStreamSynchronize(st));
  for (int i = 0; i < h->ev_used; ++i) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, h->ev[2 * i], h->ev[2 * i + 1]));
    h->kt_ms[h->ev_cls[i]] += ms;
    h->kt_n[h->ev_cls[i]] += 1;
  }
  h->ev_used = 0;
}
#define PROF(cls) Prof prof_(h, cls, st)

// f16op: the operands are fp16 in bf16 mode (forward activations and weights,
// and the MLP part of the backward)
// whole: one tiled product with no K split (each output element then depends only on its
// own row and column, whatever the row count; used for the frozen prefix)
void gemm(ttt_handle *h, int cls, bool akc, bool bkc, int epi, GemmArgs g, hipStream_t st, bool f16op = false,
          bool whole = false) {
  const int odt = (f16op && h->dt == 1) ? 2 : h->dt;
  GemmPlan plan = gemm_plan(odt, akc, bkc, epi, g, h->ws_elems);
  if (whole) plan.split = 1;  // the wide / narrow choice never changes a result bit
  const int split = plan.split;
  {
    Prof prof_(h, cls, st);
    HIPCHK(gemm_main_launch(odt, akc, bkc, epi, g, h->ws, plan, st, !whole));
  }
  if (split > 1) {
    Prof prof_(h, K_SPLITK_REDUCE, st);
    HIPCHK(gemm_reduce_launch(odt, epi, g, h->ws, split, st));
  }
  h->launches += split > 1 ? 2 : 1;
}

// Products with the same epilogue and k-contiguous operands that each fill less of the GPU
// than one round of tiles: one launch over all their 256 x 256 tiles when they have at
// least 200 together, else one launch each (the same results either way).
void gemm_group(ttt_handle *h, int cls, int epi, const GemmArgs *gs, int n, hipStream_t st, bool f16op = false) {
  const int odt = (f16op && h->dt == 1) ? 2 : h->dt;
  long t256 = 0;
  for (int p = 0; p < n; ++p) t256 += (long)((gs[p].M + 255) / 256) * ((gs[p].N + 255) / 256);
  if (n < 2 || t256 < 200) {
    for (int p = 0; p < n; ++p) gemm(h, cls, true, true, epi, gs[p], st, f16op);
    return;
  }
  {
    Prof prof_(h, cls, st);
    HIPCHK(gemm_group_launch(odt, epi, gs, n, h->ws, h->ws_elems, st));
  }
  h->launches += 1;
}

// A residual product h += A B^T (EPI_ADD_F32, 16-bit operands) whose split-K reduction
// is left to the RMSNorm that reads h next: returns the pending fp32 partials, or an
// empty descriptor when the product was not split (then h is already updated).  The
// partials live in h->ws until the next GEMM, so the norm must come first.
ResidualPartials gemm_residual(ttt_handle *h, int cls, GemmArgs g, hipStream_t st) {
  const int odt = h->dt == 1 ? 2 : h->dt;
  const GemmPlan plan = gemm_plan(odt, true, true, EPI_ADD_F32, g, h->ws_elems);
  const int split = plan.split;
  {
    Prof prof_(h, cls, st);
    HIPCHK(gemm_main_launch(odt, true, true, EPI_ADD_F32, g, h->ws, plan, st));
  }
  h->launches += 1;
  ResidualPartials r;
  if (split > 1) {
    r.ws = h->ws;
    r.split = split;
    r.sc = g.acc_scale;
  }
  return r;
}

// --------------------------------------------------------------------------- the chunk step
// What a step does besides the chunk forward (and, with update, its backward and SGD).
enum ChunkMode {
  MODE_PREFILL = 0,   // losses[pos] = loss of the stored label
  MODE_GREEDY = 1,    // decode: also picks the argmax as the next token (tok[pos + n]) with its loss
  MODE_RECOMPUTE = 2, // a decoded chunk run again for its update; losses go to rlosses
  MODE_FORCED = 3     // decode of a given token: losses[pos] as MODE_PREFILL, computed as a greedy step
                      // computes them (so that forced and greedy decodes agree bit for bit)
};

// lb > 0: blocks below lb were run ahead by the frozen-prefix pass (lead); the chunk's
// residual rows are taken from h_lead.  lead: run only the frozen prefix over n rows per
// sequence (a group) with the frozen-prefix scratch, into ls.h, advancing ls.pos0 by n
// (no head, no backward).
void enqueue_chunk(ttt_handle *h, int n, bool update, hipStream_t st, int mode = MODE_PREFILL, int lb = 0,
                   bool lead = false) {
  const int d = h->d, F = h->F, L = h->L, dt = h->dt, B = h->B, H = h->H, hd = h->hd, b = h->b;
  const int Bn = B * n;  // rows of the batched chunk: sequence s owns rows [s*n, (s+1)*n)
  const size_t es = h->es;
  const float eps = h->cfg.rms_eps;
  const bool f16 = dt == 1;  // bf16 mode: forward activations and weights are fp16
  // byte offset of sequence s's rows in a [Bn][cols] buffer of element size esz
  auto rows = [n](int s, long cols, size_t esz) { return (size_t)s * n * cols * esz; };
  h->launches = 0;
  ResidualPartials pend;  // split-K partials of the last residual product, reduced by the next RMSNorm
  float *const hres = lead ? h->ls.h : h->h;  // the residual stream of this pass
  int *const pos0 = lead ? h->ls.pos0 : h->pos0;
  int *const ids = lead ? h->ls.ids : h->ids;
  void *const act = lead ? h->ls.a : h->a;
  const int ldr = lead ? h->G : b;              // rows per sequence of the per-row statistics buffers
  const int le = lead ? h->Lf : L;

  {
    PROF(K_EMBED);
    HIPCHK(gather_chunk_ids_launch(h->tok, h->ld_tok, pos0, n, B, ids, lead ? h->ls.labs : h->labs, st));
    if (lb == 0)
      HIPCHK(embed_launch(dt, h->tok_emb, ids, h->zero, hres, Bn, d, st));
    else
      HIPCHK(lead_rows_launch(h->h_lead, h->lead_n, h->G, h->pos0, h->h, n, d, B, st));
  }
  h->launches += 2;
  for (int l = lb; l < le; ++l) {
    LayerBuf &lw = h->layers[l];
    // blocks below Lf: unsplit products and one key range per head, so that a token's
    // result does not depend on how many rows share the pass (a group or a chunk)
    // (decode steps of one or a few rows keep the few-row products: nothing compares them
    // with a prefill bit for bit; a lead pass always runs whole, so no split-K partials are
    // left pending when it returns)
    const bool frozen_whole = h->G > 0 && l < h->Lf && (lead || n > 16);
    Saved *S = (lw.fast && update) ? &h->saved[lw.u] : nullptr;
    const bool sb = S && lw.bwd_attn;  // attention of this block is back-propagated
    // --- attention sub-block
    {
      PROF(K_RMSNORM);
      HIPCHK(rmsnorm_fwd_launch(dt, hres, lw.attn_norm, act, sb ? S->r1 : nullptr, sb ? S->h_in : nullptr, Bn, d, eps,
                                st, f16, pend));
      pend = ResidualPartials();
    }
    // fp32: q, k, v are normalised / cached without a 16-bit rounding first
    float *qkv = sb ? S->qkv : lead ? h->ls.qkv : h->qkv;
    {
      GemmArgs g = gargs(act, d, lw.wqkv, d, Bn, 3 * d, d);
      g.Cf = qkv;
      g.ldcf = 3 * d;
      gemm(h, K_GEMM_QKV, true, true, EPI_STORE_F32, g, st, true, frozen_whole);
    }
    void *qh = sb ? S->qh : lead ? h->ls.qh : h->qh;
    void *o = sb ? S->o : lead ? h->ls.o : h->o;
    float *lse2 = sb ? S->lse2 : lead ? h->ls.lse2 : h->lse2;
    for (int s = 0; s < B; ++s) {  // per sequence: its ring and its positions
      const size_t rs = s * h->ring_sbytes;
      {
        RopeArgs ra;
        memset(&ra, 0, sizeof(ra));
        ra.qkv = (const float *)off(qkv, rows(s, 3 * d, 4));
        ra.gq = lw.q_norm;
        ra.gk = lw.k_norm;
        ra.cs = h->rope;
        ra.pos0 = pos0;
        ra.n = n;
        ra.d = d;
        ra.H = H;
        ra.hd = hd;
        ra.R = lw.R;
        ra.eps = eps;
        ra.qh = off(qh, rows(s, d, es));
        ra.qhb = (sb && lw.fwd16) ? off(S->qhb, rows(s, d, es)) : nullptr;
        ra.qht = sb ? off(S->qht, (size_t)s * b * d * es) : nullptr;
        ra.K = off(lw.K, rs);
        ra.Vt = off(lw.Vt, rs);
        ra.Kb = lw.bwd_attn && lw.Kb ? off(lw.Kb, rs) : nullptr;
        ra.Kt = lw.bwd_attn ? off(lw.Kt, rs) : nullptr;
        ra.V = lw.bwd_attn ? off(lw.V, rs) : nullptr;
        ra.fwd_f16 = lw.fwd16;
        ra.ldt = b;
        PROF(K_ROPE);
        HIPCHK(qk_rope_fwd_launch(dt, ra, st));
      }
      {
        AttnArgs aa;
        memset(&aa, 0, sizeof(aa));
        aa.q = off(qh, rows(s, d, es));
        aa.K = off(lw.K, rs);
        aa.Vt = off(lw.Vt, rs);
        aa.o = off(o, rows(s, d, es));
        aa.lse2 = lse2 + (size_t)s * H * ldr;
        aa.n = n;
        aa.d = d;
        aa.H = H;
        aa.R = lw.R;
        aa.window = h->k;
        aa.ldl = ldr;
        aa.ldt = b;
        aa.pos0 = pos0;
        aa.scale = 1.f / sqrtf((float)hd);
        aa.nsplit = frozen_whole ? 1 : n <= 16 ? std::max(lw.fsplit, h->dec_split) : lw.fsplit;
        aa.sbound = lw.sbound;
        aa.fwd_f16 = lw.fwd16;
        aa.o_f16 = f16;
        aa.ws = h->attn_ws;
        {
          PROF(K_ATTN_FWD);
          HIPCHK(attn_fwd_launch(dt, hd, aa, st));
        }
        if (aa.nsplit > 1) {
          PROF(K_ATTN_MERGE);
          HIPCHK(attn_merge_launch(dt, hd, false, aa, st));
        }
        h->launches += aa.nsplit > 1 ? 3 : 2;  // QK-norm + RoPE, attention, merge
      }
    }
    {
      GemmArgs g = gargs(o, d, lw.wo, d, Bn, d, d);
      g.Cf = hres;
      g.ldcf = d;
      if (frozen_whole)
        gemm(h, K_GEMM_O, true, true, EPI_ADD_F32, g, st, true, true);
      else
        pend = gemm_residual(h, K_GEMM_O, g, st);
    }
    // --- MLP sub-block (fast + static summed on one norm for updated blocks)
    void *m = S ? S->m : lead ? h->ls.m : h->m;
    {
      PROF(K_RMSNORM);
      HIPCHK(rmsnorm_fwd_launch(dt, hres, lw.mlp_norm, m, S ? S->r2 : nullptr, S ? S->h1 : nullptr, Bn, d, eps, st, f16,
                                pend));
      pend = ResidualPartials();
    }
    void *hm = S ? S->hmid : lead ? h->ls.hmid : h->hmid;  // hidden units: F (frozen) or 2F = fast then static
    if (!lw.fast) {
      GemmArgs g = gargs(m, d, lw.wgu, d, Bn, 2 * F, d);
      g.C = hm;
      g.ldc = F;
      g.c_f16 = f16;
      gemm(h, K_GEMM_GATE_UP, true, true, EPI_SWIGLU, g, st, true, frozen_whole);
      GemmArgs g2 = gargs(hm, F, lw.wd, F, Bn, d, F);
      g2.Cf = hres;
      g2.ldcf = d;
      if (frozen_whole)
        gemm(h, K_GEMM_DOWN, true, true, EPI_ADD_F32, g2, st, true, true);
      else
        pend = gemm_residual(h, K_GEMM_DOWN, g2, st);
      h->launches += 2;  // the block's two RMSNorms (the GEMM helpers count their own launches)
    } else {
      // gate/up: the static units [F, 2F) for all sequences at once and each sequence's
      // fast units [0, F), launched together in groups of up to GEMM_GROUP_MAX products
      GemmArgs gs[GEMM_GROUP_MAX];
      int ng = 0;
      gs[ng] = gargs(m, d, lw.wgu_s, d, Bn, 2 * F, d);
      gs[ng].C = off(hm, (size_t)F * es);
      gs[ng].ldc = 2 * F;
      gs[ng].C2 = S ? off(S->gu, (size_t)2 * F * es) : nullptr;
      gs[ng].ldc2 = 4 * F;
      gs[ng].c_f16 = f16;
      ++ng;
      for (int s = 0; s < B; ++s) {
        // fast units: bf16 runs the reduction over [m | m] x [hi | lo]
        GemmArgs &g = gs[ng++];
        g = gargs(off(m, rows(s, d, es)), d, off(lw.wgu, s * h->fgu_sb), 2 * d, n, 2 * F, dt == 1 ? 2 * d : d);
        g.a_kwrap = dt == 1 ? d : 0;
        g.C = off(hm, rows(s, 2 * F, es));
        g.ldc = 2 * F;
        g.C2 = S ? off(S->gu, rows(s, 4 * F, es)) : nullptr;
        g.ldc2 = 4 * F;
        g.c_f16 = f16;
        g.acc_scale = 1.f / h->wscale;
        if (ng == GEMM_GROUP_MAX || s == B - 1) {
          gemm_group(h, K_GEMM_GATE_UP, EPI_SWIGLU, gs, ng, st, true);
          ng = 0;
        }
      }
      for (int s = 0; s < B; ++s) {
        void *wd = off(lw.wd, s * h->fd_sb);
        // down: [fast | static | fast] units x [hi | static | lo] columns (bf16 mode)
        GemmArgs g2 = gargs(off(hm, rows(s, 2 * F, es)), 2 * F, wd, 3 * F, n, d, dt == 1 ? 3 * F : 2 * F);
        g2.a_kwrap = dt == 1 ? 2 * F : 0;
        g2.Cf = h->h + (size_t)s * n * d;
        g2.ldcf = d;
        g2.acc_scale = 1.f / h->wscale;
        if (B == 1)
          pend = gemm_residual(h, K_GEMM_DOWN, g2, st);
        else
          gemm(h, K_GEMM_DOWN, true, true, EPI_ADD_F32, g2, st, true);
      }
      h->launches += 2;  // the block's two RMSNorms
    }
  }
  if (lead) {  // the frozen prefix of a group: its residual rows stay in ls.h
    HIPCHK(add_int_launch(h->ls.pos0, n, st));
    h->launches++;
    return;
  }
  // --- head: final norm, LM head + cross-entropy (losses written before any update)
  {
    PROF(K_RMSNORM);
    HIPCHK(rmsnorm_fwd_launch(dt, h->h, h->final_norm, h->nf, update ? h->rf : nullptr, update ? h->hf : nullptr, Bn, d,
                              eps, st, f16, pend));
    pend = ResidualPartials();
  }
  h->launches++;
  const bool head_bwd = update && h->nu > 0;
  if (mode == MODE_GREEDY || mode == MODE_FORCED) {
    // a decode step: per-tile (max, sum) partials and each tile's argmax for the pick
    GemmArgs g = gargs(h->nf, d, h->lm_head, d, Bn, h->V, d);
    g.rowi = h->labs;  // label of row r = labs[*zero + r]
    g.pos0 = h->zero;
    g.part = h->part;
    g.part_ld = h->P;
    g.zlab = h->zlab;
    g.part_arg = h->part_arg;
    gemm(h, K_GEMM_HEAD_CE, true, true, EPI_CE, g, st, true);
  } else if (!head_bwd) {
    // losses only, computed as the update path of this handle computes them (so that the
    // losses match a prefill with eta = 0 bit for bit): the partials of the single pass
    // without its exponentials stored, or the cross-entropy pass
    GemmArgs g = gargs(h->nf, d, h->lm_head, d, Bn, h->V, d);
    g.rowi = h->labs;  // label of row r = labs[*zero + r]
    g.pos0 = h->zero;
    g.part = h->part;
    g.part_ld = h->P;
    g.zlab = h->zlab;
    if (h->head1) {
      {
        PROF(K_CE_REDUCE);
        HIPCHK(head_shift_launch(dt, f16, h->nf, h->lm_head, h->labs, h->zero, h->shift, Bn, d, 40.f, st));
      }
      h->launches++;
      g.rowf = h->shift;
      gemm(h, K_GEMM_HEAD_CE, true, true, EPI_PROBS, g, st, true, true);
    } else {
      gemm(h, K_GEMM_HEAD_CE, true, true, EPI_CE, g, st, true, true);
    }
  } else {
    // losses and the head's gradient.  Single pass (head1): with a per-row shift c (the
    // label's logit + 40) the epilogue writes p = exp(z - c) for a vocabulary slab, the loss
    // partials (c, sum p) and the label logit, and dn accumulates p W over the slabs; once
    // the losses are reduced, dn = (dn / sum p - W[label]) 2^s / n.  That is exact while no
    // logit of a row exceeds its label's logit by more than 126 - ln V, which the handle checks
    // once from the weights: |z_v - z_label| <= 2 sqrt(d) max|g_final| max_v |W_v|.
    // Otherwise the cross-entropy pass gives the losses (lse) first and the slabs write the
    // softmax itself, p = exp(z - lse), with sum p = 1.
    {
      PROF(K_CE_REDUCE);
      if (h->head1)
        HIPCHK(head_shift_launch(dt, f16, h->nf, h->lm_head, h->labs, h->zero, h->shift, Bn, d, 40.f, st));
    }
    if (h->head1) {
      h->launches++;
    } else {
      GemmArgs g = gargs(h->nf, d, h->lm_head, d, Bn, h->V, d);
      g.rowi = h->labs;
      g.pos0 = h->zero;
      g.part = h->part;
      g.part_ld = h->P;
      g.zlab = h->zlab;
      gemm(h, K_GEMM_HEAD_CE, true, true, EPI_CE, g, st, true, true);
      {
        PROF(K_CE_REDUCE);
        HIPCHK(ce_reduce_launch(h->part, h->P, h->zlab, h->zero, h->lse, h->closs, Bn, st));
      }
      h->launches++;
    }
    for (int v0 = 0, sl = 0; v0 < h->V; v0 += h->Vs, ++sl) {
      const int vs = std::min(h->Vs, h->V - v0);
      {
        GemmArgs g = gargs(h->nf, d, off(h->lm_head, (size_t)v0 * d * es), d, Bn, vs, d);
        g.C = h->dz;  // p in the working dtype
        g.ldc = h->Vs;
        g.rowf = h->head1 ? h->shift : h->lse;
        g.rowi = h->labs;  // label of row r = labs[*zero + r]
        g.pos0 = h->zero;
        g.part = h->head1 ? h->part : nullptr;
        g.part_ld = h->P;
        g.zlab = h->head1 ? h->zlab : nullptr;
        g.col_off = v0;
        gemm(h, K_GEMM_HEAD_CE, true, true, EPI_PROBS, g, st, true);
      }
      {
        // B[n = model dim][k = vocab] from the transposed head [d][V]
        GemmArgs g = gargs(h->dz, h->Vs, off(h->lm_headT, (size_t)v0 * es), h->V, Bn, d, vs);
        g.Cf = h->dn;
        g.ldcf = d;
        gemm(h, K_GEMM_DN, true, true, sl == 0 ? EPI_STORE_F32 : EPI_ADD_F32, g, st);
      }
    }
  }
  {
    PROF(K_CE_REDUCE);
    if (!head_bwd || h->head1)
      HIPCHK(ce_reduce_launch(h->part, h->P, h->zlab, h->zero, h->lse, h->closs, Bn, st));
    HIPCHK(scatter_chunk_losses_launch(h->closs, mode == MODE_RECOMPUTE ? h->rlosses : h->losses, h->cfg.max_tokens,
                                       h->pos0, n, B, st));
    if (mode == MODE_GREEDY)  // one sequence
      HIPCHK(decode_pick_launch(h->part, h->part_arg, h->P, h->lse, h->pos0, n, h->tok, h->losses, st));
  }
  h->launches += (mode == MODE_GREEDY ? 3 : 2) - (head_bwd && !h->head1 ? 1 : 0);

  if (head_bwd) {
    const int np = (n + 63) / 64 * 64;  // token count padded for the weight-gradient GEMMs
    {
      PROF(K_CE_REDUCE);
      HIPCHK(head_grad_finish_launch(dt, f16, h->dn, h->head1 ? h->shift : h->lse, h->lse, h->lm_head, h->labs, h->zero, Bn, d,
                                     h->gscale / (float)n, st));
    }
    h->launches++;
    {
      PROF(K_RMSNORM_BWD);
      HIPCHK(rmsnorm_bwd_launch(dt, h->dn, h->hf, h->rf, h->final_norm, nullptr, h->dh, h->dy, Bn, d, st, f16));
    }
    h->launches++;
    for (int l = L - 1; l >= L - h->nu; --l) {
      LayerBuf &lw = h->layers[l];
      Saved &S = h->saved[lw.u];
      const bool last = (l == L - h->nu);
      const int Fu = last ? F : 2 * F;  // hidden units whose gradient is needed
      for (int s = 0; s < B; ++s) {
        void *wdT = off(lw.wdT, s * h->fdT_sb);
        void *wd = off(lw.wd, s * h->fd_sb);
        float *md = h->m_d[lw.u] + (size_t)s * d * F;
        // dhmid = dy Wd_cat[:, :Fu]  (B from the transposed [2F][d] copy)
        {
          GemmArgs g = gargs(off(h->dy, rows(s, d, es)), d, wdT, d, n, Fu, d);
          g.C = off(h->dhmid, rows(s, 2 * F, es));
          g.ldc = 2 * F;
          g.c_f16 = f16;
          gemm(h, K_GEMM_DHMID, true, true, EPI_STORE, g, st, true);
        }
        {
          PROF(K_TRANSPOSE);
          HIPCHK(transpose_launch(dt, f16 ? SRC_F16 : SRC_WORK, off(h->dy, rows(s, d, es)), d, h->dyT, b, n, np, d, st,
                                  f16));
          HIPCHK(transpose_launch(dt, f16 ? SRC_F16 : SRC_WORK, off(S.hmid, rows(s, 2 * F, es)), 2 * F, h->hmidT, b,
                                  n, np, F, st, f16));
        }
        // dWd_fast = dy^T hmid_fast over the chunk's tokens, SGD fused into the epilogue
        {
          GemmArgs g = gargs(h->dyT, b, h->hmidT, b, d, F, np);
          g.Cf = md;
          g.ldcf = F;
          g.C = wd;  // hi columns [0, F)
          g.ldc = 3 * F;
          g.C2 = dt == 1 ? off(wd, (size_t)2 * F * es) : nullptr;  // lo columns [2F, 3F)
          g.ldc2 = 3 * F;
          g.c_f16 = f16;
          g.c_scale = h->wscale;
          g.alpha = h->cfg.eta / h->gscale;
          g.CT = wdT;  // the backward's transposed copy [F][d] of the fast rows, refreshed in place
          g.ldct = d;
          gemm(h, K_GEMM_DW_SGD, true, true, EPI_SGD, g, st, true);
        }
        h->launches += 2;  // the transposes
      }
      {
        PROF(K_SWIGLU_BWD);
        HIPCHK(swiglu_bwd_launch(dt, S.gu, h->dhmid, h->dgu, Bn, Fu, 4 * F, 2 * F, st, f16));
      }
      h->launches++;
      for (int s = 0; s < B; ++s) {
        void *wguT = off(lw.wguT, s * h->fguT_sb);
        void *wgu = off(lw.wgu, s * h->fgu_sb);
        float *mgu = h->m_gu[lw.u] + (size_t)s * 2 * F * d;
        if (!last) {
          GemmArgs g = gargs(off(h->dgu, rows(s, 4 * F, es)), 4 * F, wguT, 4 * F, n, d, 4 * F);
          g.Cf = h->dm + (size_t)s * n * d;
          g.ldcf = d;
          gemm(h, K_GEMM_DM, true, true, EPI_STORE_F32, g, st, true);
        }
        {
          PROF(K_TRANSPOSE);
          HIPCHK(transpose_launch(dt, f16 ? SRC_F16 : SRC_WORK, off(h->dgu, rows(s, 4 * F, es)), 4 * F, h->dguT, b, n,
                                  np, 2 * F, st, f16));
          HIPCHK(transpose_launch(dt, f16 ? SRC_F16 : SRC_WORK, off(S.m, rows(s, d, es)), d, h->mT, b, n, np, d, st,
                                  f16));
        }
        // dW(gate|up)_fast = dGU_fast^T m, SGD fused
        {
          GemmArgs g = gargs(h->dguT, b, h->mT, b, 2 * F, d, np);
          g.Cf = mgu;
          g.ldcf = d;
          g.C = wgu;  // hi columns of the fast rows
          g.ldc = 2 * d;
          g.C2 = dt == 1 ? off(wgu, (size_t)d * es) : nullptr;  // lo columns
          g.ldc2 = 2 * d;
          g.c_f16 = f16;
          g.c_scale = h->wscale;
          g.alpha = h->cfg.eta / h->gscale;
          g.CT = wguT;  // transposed copy [d][4F], fast columns [0, 2F)
          g.ldct = 4 * F;
          gemm(h, K_GEMM_DW_SGD, true, true, EPI_SGD, g, st, true);
        }
        h->launches += 2;  // the transposes
      }
      if (last) break;
      {
        PROF(K_RMSNORM_BWD);
        HIPCHK(rmsnorm_bwd_launch(dt, h->dm, S.h1, S.r2, lw.mlp_norm, h->dh, h->dh, h->dy, Bn, d, st, f16));
      }
      // attention sub-block backward
      {
        GemmArgs g = gargs(h->dy, d, lw.woT, d, Bn, d, d);
        g.C = h->dO;
        g.ldc = d;
        gemm(h, K_GEMM_DO, true, true, EPI_STORE, g, st, true);  // dO itself is bf16
      }
      h->launches += 1;
      for (int s = 0; s < B; ++s) {
        const size_t rs = s * h->ring_sbytes;
        void *dO = off(h->dO, rows(s, d, es));
        {
          PROF(K_ATTN_BWD_PRE);
          HIPCHK(attn_bwd_pre_launch(dt, dO, off(S.o, rows(s, d, es)), h->Dq, h->dOt, n, d, H, hd, b, b, st, f16));
        }
        {
          AttnArgs aa;
          memset(&aa, 0, sizeof(aa));
          aa.q = off(lw.fwd16 ? S.qhb : S.qh, rows(s, d, es));  // working-dtype copies for the backward
          aa.qt = off(S.qht, (size_t)s * b * d * es);
          aa.dout = dO;
          aa.doutt = h->dOt;
          aa.K = off(lw.fwd16 ? lw.Kb : lw.K, rs);
          aa.Vt = off(lw.Vt, rs);
          aa.Kt = off(lw.Kt, rs);
          aa.V = off(lw.V, rs);
          aa.lse2 = S.lse2 + (size_t)s * H * b;
          aa.Dq = h->Dq;
          aa.dq = h->dq + (size_t)s * n * d;
          aa.dk = h->dk + (size_t)s * n * d;
          aa.dv = h->dv + (size_t)s * n * d;
          aa.n = n;
          aa.d = d;
          aa.H = H;
          aa.R = lw.R;
          aa.window = h->k;
          aa.ldl = b;
          aa.ldt = b;
          aa.pos0 = h->pos0;
          aa.scale = 1.f / sqrtf((float)hd);
          aa.nsplit = h->attn_split;
          aa.ws = h->attn_ws;
          {
            PROF(K_ATTN_BWD_DQ);
            HIPCHK(attn_bwd_dq_launch(dt, hd, aa, st));
          }
          if (aa.nsplit > 1) {
            PROF(K_ATTN_MERGE);
            HIPCHK(attn_merge_launch(dt, hd, true, aa, st));
          }
          {
            PROF(K_ATTN_BWD_DKDV);
            HIPCHK(attn_bwd_dkdv_launch(dt, hd, aa, st));
          }
        }
        {
          RopeArgs ra;
          memset(&ra, 0, sizeof(ra));
          ra.qkv = S.qkv + (size_t)s * n * 3 * d;
          ra.gq = lw.q_norm;
          ra.gk = lw.k_norm;
          ra.cs = h->rope;
          ra.pos0 = h->pos0;
          ra.n = n;
          ra.d = d;
          ra.H = H;
          ra.hd = hd;
          ra.R = lw.R;
          ra.eps = eps;
          ra.dqh = h->dq + (size_t)s * n * d;
          ra.dkh = h->dk + (size_t)s * n * d;
          ra.dv = h->dv + (size_t)s * n * d;
          ra.dqkv = off(h->dqkv, rows(s, 3 * d, es));
          PROF(K_ROPE_BWD);
          HIPCHK(qk_rope_bwd_launch(dt, ra, st));
        }
        h->launches += h->attn_split > 1 ? 5 : 4;
      }
      {
        GemmArgs g = gargs(h->dqkv, 3 * d, lw.wqkvT, 3 * d, Bn, d, 3 * d);
        g.Cf = h->da;
        g.ldcf = d;
        gemm(h, K_GEMM_DA, true, true, EPI_STORE_F32, g, st);
      }
      {
        PROF(K_RMSNORM_BWD);
        HIPCHK(rmsnorm_bwd_launch(dt, h->da, S.h_in, S.r1, lw.attn_norm, h->dh, h->dh, h->dy, Bn, d, st, f16));
      }
      h->launches += 1;
    }
  }
  {
    PROF(K_MISC);
    HIPCHK(add_int_launch(h->pos0, n, st));
  }
  h->launches++;
}

// Copies W_init into every sequence's fp32 masters, forward copies (hi | lo,
// fp16 and scaled by wscale in bf16 mode) and the fast parts of the transposed
// working-dtype copies of the backward (the static parts are set at creation).
void reset_fast(ttt_handle *h, hipStream_t st) {
  const int d = h->d, F = h->F;
  const int fdt = h->dt == 1 ? 2 : h->dt;  // forward copy type
  for (int l = 0; l < h->L; ++l) {
    LayerBuf &lw = h->layers[l];
    if (!lw.fast) continue;
    for (int s = 0; s < h->B; ++s) {
      float *mgu = h->m_gu[lw.u] + (size_t)s * 2 * F * d, *md = h->m_d[lw.u] + (size_t)s * d * F;
      void *wgu = off(lw.wgu, s * h->fgu_sb), *wd = off(lw.wd, s * h->fd_sb);
      HIPCHK(hipMemcpyAsync(mgu, h->i_gu[lw.u], (size_t)2 * F * d * 4, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(md, h->i_d[lw.u], (size_t)d * F * 4, hipMemcpyDeviceToDevice, st));
      HIPCHK(convert_rows_launch(fdt, h->i_gu[lw.u], d, wgu, 2 * d, 2 * F, d, st,
                                 h->dt == 1 ? off(wgu, (size_t)d * h->es) : nullptr, 2 * d, h->wscale));
      HIPCHK(convert_rows_launch(fdt, h->i_d[lw.u], F, wd, 3 * F, d, F, st,
                                 h->dt == 1 ? off(wd, (size_t)2 * F * h->es) : nullptr, 3 * F, h->wscale));
      // Wd_cat^T [2F][d] rows [0, F) and Wgu_cat^T [d][4F] columns [0, 2F), from the masters
      HIPCHK(transpose_launch(h->dt, SRC_F32, h->i_d[lw.u], F, off(lw.wdT, s * h->fdT_sb), d, d, d, F, st,
                              h->dt == 1));
      HIPCHK(transpose_launch(h->dt, SRC_F32, h->i_gu[lw.u], d, off(lw.wguT, s * h->fguT_sb), 4 * F, 2 * F, 2 * F, d,
                              st, h->dt == 1));
    }
  }
}

// flag |= 1 if any fp32 master fast weight of any sequence is NaN or infinite: the
// masters are W_0 - eta * (sum of every update so far), so a non-finite gradient in
// any chunk leaves a non-finite entry behind.
void check_masters(ttt_handle *h, hipStream_t st) {
  const long gu = (long)h->B * 2 * h->F * h->d, dd = (long)h->B * h->d * h->F;
  for (int u = 0; u < h->nu; ++u) {
    HIPCHK(finite_check_launch(h->m_gu[u], gu, h->flag, st));
    HIPCHK(finite_check_launch(h->m_d[u], dd, h->flag, st));
  }
}

ttt_status fail_hip(ttt_handle *h, const HipFail &f) {
  char buf[512];
  snprintf(buf, sizeof(buf), "HIP error %d (%s) in %s", (int)f.e, hipGetErrorString(f.e), f.what);
  if (h) h->err = buf;
  g_thread_err = buf;
  return TTT_EHIP;
}
ttt_status fail(ttt_handle *h, ttt_status s, const std::string &msg) {
  if (h) h->err = msg;
  g_thread_err = msg;
  return s;
}

// Once per device, with that device current: the device address of the static
// scratch, cleared to zeros (finite start values for partials that masked lanes
// read before a split overwrites them).  Failures are kept in h->scratch_err; only
// ttt_prefill_noalloc needs the scratch.
void scratch_setup(ttt_handle *h, hipStream_t st) {
  if (h->dev < 0 || h->dev >= SCRATCH_MAX_DEV) {
    h->scratch_err = "device index beyond the static scratch table";
    return;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[h->dev]) {
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && !p) e = hipErrorInvalidSymbol;
    if (e == hipSuccess) e = zero_launch(p, SCRATCH_BYTES, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      h->scratch_err = std::string("static scratch set-up failed: ") + hipGetErrorString(e);
      return;
    }
    g_scratch_ptr[h->dev] = reinterpret_cast<float *>(p);
  }
  h->scratch = g_scratch_ptr[h->dev];
}

// Modelled time of one frozen block over a pass of `rows` rows (B sequences of `seq` rows
// each), in units of one k-step of the 256 x 256 GEMM tile.  Each product takes
// ceil(tiles / CUs) rounds, a round costing its K steps plus a fixed part (prologue,
// epilogue, dispatch: about 609 steps, measured as 14.5 us against 24.4 us per 1024 of
// K); the attention takes ceil(work-groups / 2 CUs) rounds of (k + 256) / 32 key tiles of
// 256 queries, about 1.51 (k + 256) steps at head dim 80 (1.15 us per tile), scaled by hd.
static double frozen_pass_cost(long rows, long seq, int d, int F, int H, int k, int cus) {
  if (rows <= 0) return 0.0;
  const int tw = 256;
  const long rt = (rows + tw - 1) / tw;
  const long N[4] = {3L * d, d, 2L * F, d}, K[4] = {d, d, d, F};
  double t = 0.0;
  for (int p = 0; p < 4; ++p) {
    const long tiles = rt * ((N[p] + tw - 1) / tw);
    t += (double)((tiles + cus - 1) / cus) * (609.0 + (double)K[p]);
  }
  const long wg = (seq + 255) / 256 * H * (rows / seq);
  t += (double)((wg + 2L * cus - 1) / (2L * cus)) * 1.51 * (k + 256) * ((double)d / H) / 80.0;
  return t;
}

// Tokens per sequence in a frozen-prefix group.  The group's products run unsplit on the
// 256 x 256 tile (one work-group per CU) and its attention on work-groups of 256 queries of
// one head (two per CU), so how full their rounds are depends on the row count, and a
// ragged last group pays whole rounds for a few rows: at 2.7B 8192 rows leave the d-wide
// O and down products at 1.25 rounds of 256 CUs.  Among row counts from 8192 to 16384
// (multiples of the chunk over the B sequences) this takes the one whose groups over T
// tokens cost least in the model above, the smallest on ties: 12288 at 2.7B and 128K (8192
// and 16384 measured 55 and 35 ms slower per prefill), 16384 at 1.3B, 760M and 125M (125M:
// 1.5 ms faster than 10240, whose last group is 2048 rows) and at 2.7B and 32K (the same
// time as 12288 there).
long frozen_group_tokens(int d, int F, int H, int k, int b, int B, long T, int cus) {
  const long step = (long)b * B;
  long best = std::max(1L, 8192 / step) * b;
  double best_t = -1.0;
  for (long rows = step * std::max(1L, 8192 / step); rows <= 16384; rows += step) {
    const long G = rows / B, full = T / G, last = T % G;
    const double t = (double)full * frozen_pass_cost(rows, G, d, F, H, k, cus) +
                     frozen_pass_cost(last * B, last, d, F, H, k, cus);
    if (best_t < 0.0 || t < best_t - 1e-9) {
      best_t = t;
      best = G;
    }
  }
  return best;
}

void free_all(ttt_handle *h) {
  for (int i = 0; i < 6; ++i)
    if (h->gexec[i]) hipGraphExecDestroy(h->gexec[i]);
  if (h->cap) hipStreamDestroy(h->cap);
  if (h->lead_st) hipStreamDestroy(h->lead_st);
  for (int i = 0; i < 2; ++i) {
    if (h->ev_pf[i]) hipEventDestroy(h->ev_pf[i]);
    if (h->ev_lead[i]) hipEventDestroy(h->ev_lead[i]);
  }
  for (void *p : h->allocs) hipFree(p);
  h->allocs.clear();
}

// Interleaves gate and up rows in blocks of 16: packed row 32j+t = gate 16j+t, 32j+16+t = up 16j+t.
void pack_gu(const void *gate, const void *up, void *dst, int F, int d, size_t es, hipStream_t st) {
  const size_t blk = (size_t)16 * d * es;
  HIPCHK(hipMemcpy2DAsync(dst, 2 * blk, gate, blk, blk, F / 16, hipMemcpyDeviceToDevice, st));
  HIPCHK(hipMemcpy2DAsync(off(dst, blk), 2 * blk, up, blk, blk, F / 16, hipMemcpyDeviceToDevice, st));
}

// Bound of scale * q.k in log2 units for one layer: with QK-norm every row has
// Euclidean norm at most max|gain| * sqrt(hd), so |q.k| / sqrt(hd) is at most
// max|g_q| * max|g_k| * sqrt(hd).  Returns 0 (no bound) for fp32 or when the
// bound is too large for the bounded forward.
float score_bound(ttt_handle *h, const void *gq, const void *gk, hipStream_t st) {
  if (h->dt != 1) return 0.f;
  std::vector<uint16_t> q(h->hd), k(h->hd);
  HIPCHK(hipMemcpyAsync(q.data(), gq, h->hd * 2, hipMemcpyDeviceToHost, st));
  HIPCHK(hipMemcpyAsync(k.data(), gk, h->hd * 2, hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  auto mx = [](const std::vector<uint16_t> &v) {
    float m = 0.f;
    for (uint16_t x : v) {
      uint32_t u = (uint32_t)x << 16;
      float f;
      std::memcpy(&f, &u, 4);
      m = std::max(m, std::fabs(f));
    }
    return m;
  };
  // 1% headroom for the bf16 rounding of the normalised rows
  const double b = 1.01 * mx(q) * mx(k) * std::sqrt((double)h->hd) * 1.4426950408889634;
  return (b > 0.0 && b <= ATTN_MAX_SBOUND) ? (float)b : 0.f;
}

// One step of n positions in the given mode: replayed from a captured graph when
// graph replay is on and the step has its full size (b for chunks, 1 for decode
// steps), else enqueued launch by launch.
// lead: the frozen prefix of a group of n tokens.  grouped: a prefill chunk whose frozen
// prefix the lead pass has run (the graphs of full prefill chunks are only used this way
// when the handle groups).
void run_step(ttt_handle *h, int n, bool update, int mode, bool use_graph, hipStream_t st, bool lead = false,
              bool grouped = false) {
  int gi = -1;
  if (use_graph) {
    if (lead) {
      if (n == h->G) gi = 5;
    } else {
      if (mode == MODE_PREFILL && n == h->b && grouped == (h->G > 0)) gi = update ? 0 : 1;
      if (mode == MODE_GREEDY && n == 1 && !update) gi = 2;
      if (mode == MODE_FORCED && n == 1 && !update) gi = 3;
      if (mode == MODE_RECOMPUTE && n == h->b && update) gi = 4;
    }
  }
  const int lb = grouped ? h->Lf : 0;
  if (gi < 0) {
    enqueue_chunk(h, n, update, st, mode, lb, lead);
    prof_collect(h, st);
    return;
  }
  if (!h->gexec[gi]) {
    hipGraph_t gr = nullptr;
    HIPCHK(hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal));
    try {
      enqueue_chunk(h, n, update, h->cap, mode, lb, lead);
    } catch (...) {
      hipStreamEndCapture(h->cap, &gr);
      if (gr) hipGraphDestroy(gr);
      throw;
    }
    HIPCHK(hipStreamEndCapture(h->cap, &gr));
    hipError_t e = hipGraphInstantiate(&h->gexec[gi], gr, nullptr, nullptr, 0);
    hipGraphDestroy(gr);
    HIPCHK(e);
  }
  HIPCHK(hipGraphLaunch(h->gexec[gi], st));
}

void copy_fast_out(ttt_handle *h, float *const *d_fast_out, hipStream_t st) {
  const int d = h->d, F = h->F;
  const size_t blk = (size_t)16 * d * 4;
  for (int s = 0; s < h->B; ++s)
    for (int u = 0; u < h->nu; ++u) {
      float *const *o = d_fast_out + 3 * (s * h->nu + u);
      const float *mgu = h->m_gu[u] + (size_t)s * 2 * F * d, *md = h->m_d[u] + (size_t)s * d * F;
      HIPCHK(hipMemcpy2DAsync(o[0], blk, mgu, 2 * blk, blk, F / 16, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpy2DAsync(o[1], blk, (const char *)mgu + blk, 2 * blk, blk, F / 16, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(o[2], md, (size_t)d * F * 4, hipMemcpyDeviceToDevice, st));
    }
}

}  // namespace

// =========================================================================== C ABI
extern "C" {

ttt_status ttt_create(const ttt_config *cfg, const ttt_weights *w, void *stream, ttt_handle **out) {
  if (out) *out = nullptr;
  if (!cfg || !w || !out) return fail(nullptr, TTT_EINVAL, "null argument");
  const ttt_config c = *cfg;
  if (c.n_layers < 1 || c.n_update < 0 || c.n_update > c.n_layers)
    return fail(nullptr, TTT_EINVAL, "n_layers >= 1 and 0 <= n_update <= n_layers required");
  if (c.n_seq < 0 || c.n_seq > 256) return fail(nullptr, TTT_EINVAL, "n_seq must be in [0, 256] (0 means 1)");
  if (c.n_heads < 1 || c.d_model != c.n_heads * c.head_dim) return fail(nullptr, TTT_EINVAL, "d_model != n_heads * head_dim");
  if (c.d_model % 16 || c.d_ff % 16 || c.vocab % 16 || c.d_model <= 0 || c.d_ff <= 0 || c.vocab <= 0)
    return fail(nullptr, TTT_EINVAL, "d_model, d_ff and vocab must be positive multiples of 16");
  if (!attn_supported_hd(c.head_dim)) return fail(nullptr, TTT_EUNSUPPORTED, "head_dim not in {16,32,64,80,96,128}");
  if (c.dtype != TTT_FP32 && c.dtype != TTT_BF16) return fail(nullptr, TTT_EINVAL, "dtype");
  if (c.dtype == TTT_FP32 && c.head_dim > 64) return fail(nullptr, TTT_EUNSUPPORTED, "fp32 supports head_dim <= 64");
  if (c.d_model > 8192) return fail(nullptr, TTT_EUNSUPPORTED, "d_model > 8192");
  if (c.dtype == TTT_BF16 && (c.d_model % 64 || c.d_ff % 64))
    return fail(nullptr, TTT_EUNSUPPORTED, "bf16 mode needs d_model and d_ff multiples of 64");
  if (c.chunk <= 0 || c.window <= 0 || c.chunk % 64 || c.window % 64 || c.window < c.chunk)
    return fail(nullptr, TTT_EINVAL, "chunk and window must be positive multiples of 64 with window >= chunk");
  if (c.max_tokens < 1 || c.max_tokens > (1ll << 30)) return fail(nullptr, TTT_EINVAL, "max_tokens out of range");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f) || !std::isfinite(c.eta))
    return fail(nullptr, TTT_EINVAL, "rms_eps, rope_theta must be > 0 and eta finite");
  if (!w->tok_emb || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->q_norm || !w->k_norm || !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
    return fail(nullptr, TTT_EINVAL, "null weight pointer");
  for (int l = 0; l < c.n_layers; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->q_norm[l] || !w->k_norm[l] ||
        !w->mlp_norm[l] || !w->w_gate[l] || !w->w_up[l] || !w->w_down[l])
      return fail(nullptr, TTT_EINVAL, "null per-layer weight pointer");
  if (c.n_update > 0) {
    if (!w->fast_gate || !w->fast_up || !w->fast_down) return fail(nullptr, TTT_EINVAL, "null fast weight array");
    for (int u = 0; u < c.n_update; ++u)
      if (!w->fast_gate[u] || !w->fast_up[u] || !w->fast_down[u]) return fail(nullptr, TTT_EINVAL, "null fast weight");
  }

  ttt_handle *h = new ttt_handle();
  h->cfg = c;
  h->dt = c.dtype == TTT_BF16 ? 1 : 0;
  h->es = h->dt ? 2 : 4;
  h->gscale = h->dt ? 4096.f : 1.f;
  h->L = c.n_layers;
  h->d = c.d_model;
  h->H = c.n_heads;
  h->hd = c.head_dim;
  h->F = c.d_ff;
  h->V = c.vocab;
  h->k = c.window;
  h->b = c.chunk;
  h->nu = c.n_update;
  h->R = c.window + c.chunk;  // positions s-k+1 .. s+b-1 must coexist; multiple of 64
  h->B = c.n_seq > 0 ? c.n_seq : 1;
  // frozen-prefix groups of G tokens per sequence (B G rows per pass), never longer than
  // the longest sequence: frozen_group_tokens picks G.
  h->Lf = c.n_layers - c.n_update;
  {
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const long gmax = (c.max_tokens + c.chunk - 1) / c.chunk * (long)c.chunk;
    h->G = (int)std::min<long>(frozen_group_tokens(c.d_model, c.d_ff, c.n_heads, c.window, c.chunk, h->B, gmax, cus),
                               gmax);
    if (h->Lf == 0 || h->G <= c.chunk) h->G = 0;
  }
  h->ld_tok = c.max_tokens + 1;
  // vocabulary slab of the head: its [B b, Vs] unnormalised softmax is about 64 MiB or less
  // (32768 columns at B b = 1024; measured 13 ms per 128K prefill faster than 16384, and
  // 65536 no better); a multiple of 256 columns, so that every slab starts at a partial slot
  // of the 256-wide tile
  h->Vs = std::min(h->V, std::max(1024, (32768 * 1024 / std::max(1, h->B * c.chunk)) / 256 * 256));
  h->P = 2 * ((h->V + 127) / 128);
  hipStream_t st = (hipStream_t)stream;
  const int d = h->d, F = h->F, b = h->b, L = h->L, V = h->V;
  const size_t es = h->es;
  try {
    // ---- weights
    h->tok_emb = dalloc(h, (size_t)V * d * es, false);
    h->lm_head = dalloc(h, (size_t)V * d * es, false);
    h->final_norm = dalloc(h, d * es, false);
    HIPCHK(hipMemcpyAsync(h->tok_emb, w->tok_emb, (size_t)V * d * es, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipMemcpyAsync(h->lm_head, w->lm_head, (size_t)V * d * es, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipMemcpyAsync(h->final_norm, w->final_norm, d * es, hipMemcpyDeviceToDevice, st));
    h->layers.resize(L);
    h->m_gu.resize(h->nu);
    h->m_d.resize(h->nu);
    h->i_gu.resize(h->nu);
    h->i_d.resize(h->nu);
    h->saved.resize(h->nu);
    size_t ring_sb = 0;  // one sequence's ring planes, all layers
    for (int l = 0; l < L; ++l) {
      LayerBuf &lw = h->layers[l];
      lw.fast = l >= L - h->nu;
      lw.bwd_attn = l > L - h->nu;
      lw.sbound = score_bound(h, w->q_norm[l], w->k_norm[l], st);
      lw.fwd16 = attn_fwd_f16_ok(h->dt, lw.sbound, h->hd);
      lw.R = (h->G > 0 && l < h->Lf) ? c.window + h->G : h->R;
      ring_sb += (size_t)h->H * lw.R * h->hd * es * (2 + (lw.bwd_attn ? (lw.fwd16 ? 3 : 2) : 0));
    }
    {
      // the single-pass head is exact when every row's logits lie within a band of the
      // label's logit: |z_v - z_label| <= |W_v - W_label| |g_final * x / rms(x)| <=
      // 2 max_v |W_v| max|g_final| sqrt(d) = 2 bound (1% headroom for the rounding of the
      // normalised rows); with the shift label + 40, exp(z - shift) summed over V columns
      // stays below fp32's (and bf16's) largest value while 2 bound + ln V <= 126
      unsigned *hm = (unsigned *)dalloc(h, 64, false);
      HIPCHK(hipMemsetAsync(hm, 0, 8, st));
      HIPCHK(rownorm_max_launch(h->dt, w->lm_head, d, V, d, hm, st));
      HIPCHK(absmax_launch(h->dt, w->final_norm, d, 1, d, hm + 1, st));
      unsigned bits[2] = {0, 0};
      HIPCHK(hipMemcpyAsync(bits, hm, 8, hipMemcpyDeviceToHost, st));
      HIPCHK(hipStreamSynchronize(st));
      float wn, gm;
      std::memcpy(&wn, &bits[0], 4);
      std::memcpy(&gm, &bits[1], 4);
      const double bound = 1.01 * (double)wn * (double)gm * std::sqrt((double)d);
      h->head1 = std::isfinite(bound) && 2.0 * bound + std::log((double)V) <= 126.0;
    }
    if (h->dt == 1 && h->nu > 0) {
      // largest |w| over the weights whose forward copies are stored scaled
      unsigned *amax = (unsigned *)dalloc(h, 64, false);
      HIPCHK(hipMemsetAsync(amax, 0, 4, st));
      for (int u = 0; u < h->nu; ++u) {
        HIPCHK(absmax_launch(0, w->fast_gate[u], d, F, d, amax, st));
        HIPCHK(absmax_launch(0, w->fast_up[u], d, F, d, amax, st));
        HIPCHK(absmax_launch(0, w->fast_down[u], F, d, F, amax, st));
        HIPCHK(absmax_launch(1, w->w_down[L - h->nu + u], F, d, F, amax, st));
      }
      unsigned bits = 0;
      HIPCHK(hipMemcpyAsync(&bits, amax, 4, hipMemcpyDeviceToHost, st));
      HIPCHK(hipStreamSynchronize(st));
      float mx;
      std::memcpy(&mx, &bits, 4);
      if (!(mx < 8192.f)) {
        hipStreamSynchronize(st);
        free_all(h);
        delete h;
        return fail(nullptr, TTT_EUNSUPPORTED,
                    "bf16 mode needs finite MLP weights below 8192 in magnitude in the updated blocks");
      }
      // 2^s with max|w| * 2^s <= 4096 (16x headroom below fp16's largest value), s <= 12
      int sh = 12;
      while (sh > 0 && std::ldexp(mx, sh) > 4096.f) --sh;
      h->wscale = std::ldexp(1.f, sh);
    }
    h->ring_sbytes = ring_sb;
    h->ring_bytes = h->ring_sbytes * h->B;  // sequence s's planes at s * ring_sbytes
    h->ring_base = dalloc(h, h->ring_bytes);
    size_t roff = 0;
    for (int l = 0; l < L; ++l) {
      LayerBuf &lw = h->layers[l];
      lw.u = lw.fast ? l - (L - h->nu) : -1;
      lw.attn_norm = dalloc(h, d * es, false);
      lw.mlp_norm = dalloc(h, d * es, false);
      lw.q_norm = dalloc(h, h->hd * es, false);
      lw.k_norm = dalloc(h, h->hd * es, false);
      HIPCHK(hipMemcpyAsync(lw.attn_norm, w->attn_norm[l], d * es, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(lw.mlp_norm, w->mlp_norm[l], d * es, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(lw.q_norm, w->q_norm[l], h->hd * es, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(lw.k_norm, w->k_norm[l], h->hd * es, hipMemcpyDeviceToDevice, st));
      lw.fsplit = attn_fwd_split(h->dt, lw.sbound, h->hd, b, h->H, h->k, b);
      const size_t dd = (size_t)d * d * es;
      lw.wqkv = dalloc(h, 3 * dd, false);
      HIPCHK(hipMemcpyAsync(lw.wqkv, w->wq[l], dd, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(off(lw.wqkv, dd), w->wk[l], dd, hipMemcpyDeviceToDevice, st));
      HIPCHK(hipMemcpyAsync(off(lw.wqkv, 2 * dd), w->wv[l], dd, hipMemcpyDeviceToDevice, st));
      lw.wo = dalloc(h, dd, false);
      HIPCHK(hipMemcpyAsync(lw.wo, w->wo[l], dd, hipMemcpyDeviceToDevice, st));
      const size_t fd = (size_t)F * d * es;
      if (!lw.fast) {
        lw.wgu = dalloc(h, 2 * fd, false);
        pack_gu(w->w_gate[l], w->w_up[l], lw.wgu, F, d, es, st);
        lw.wd = dalloc(h, fd, false);
        HIPCHK(hipMemcpyAsync(lw.wd, w->w_down[l], fd, hipMemcpyDeviceToDevice, st));
      } else {
        const int u = lw.u;
        h->fgu_sb = 4 * fd;
        h->fd_sb = 3 * fd;
        h->fdT_sb = 2 * fd;
        h->fguT_sb = 4 * fd;
        lw.wgu = dalloc(h, h->B * h->fgu_sb, false);  // fast hi | lo rows per sequence (written by reset_fast)
        lw.wgu_s = dalloc(h, 2 * fd, false);
        pack_gu(w->w_gate[l], w->w_up[l], lw.wgu_s, F, d, es, st);
        lw.wd = dalloc(h, h->B * h->fd_sb, false);
        for (int sq = 0; sq < h->B; ++sq)
          HIPCHK(hipMemcpy2DAsync(off(lw.wd, sq * h->fd_sb + (size_t)F * es), 3 * F * es, w->w_down[l], F * es, F * es,
                                  d, hipMemcpyDeviceToDevice, st));
        const size_t f32fd = (size_t)F * d * 4;
        h->m_gu[u] = (float *)dalloc(h, h->B * 2 * f32fd);
        h->m_d[u] = (float *)dalloc(h, h->B * f32fd);
        h->i_gu[u] = (float *)dalloc(h, 2 * f32fd, false);
        h->i_d[u] = (float *)dalloc(h, f32fd, false);
        pack_gu(w->fast_gate[u], w->fast_up[u], h->i_gu[u], F, d, 4, st);
        HIPCHK(hipMemcpyAsync(h->i_d[u], w->fast_down[u], f32fd, hipMemcpyDeviceToDevice, st));
      }
      if (lw.fast && h->nu > 0) {
        lw.wdT = dalloc(h, h->B * h->fdT_sb, false);
        lw.wguT = dalloc(h, h->B * h->fguT_sb, false);
        // static parts of each sequence's Wd_cat^T (rows [F, 2F)) and Wgu_cat^T (columns [2F, 4F))
        for (int sq = 0; sq < h->B; ++sq) {
          HIPCHK(transpose_launch(h->dt, SRC_WORK, off(lw.wd, (size_t)F * es), 3 * F, off(lw.wdT, sq * h->fdT_sb + fd), d,
                                  d, d, F, st, h->dt == 1));
          HIPCHK(transpose_launch(h->dt, SRC_WORK, lw.wgu_s, d, off(lw.wguT, sq * h->fguT_sb + (size_t)2 * F * es),
                                  4 * F, 2 * F, 2 * F, d, st, h->dt == 1));
        }
      }
      if (lw.bwd_attn) {
        lw.woT = dalloc(h, dd, false);
        lw.wqkvT = dalloc(h, 3 * dd, false);
        HIPCHK(transpose_launch(h->dt, SRC_WORK, lw.wo, d, lw.woT, d, d, d, d, st, h->dt == 1));  // fp16 in bf16 mode
        HIPCHK(transpose_launch(h->dt, SRC_WORK, lw.wqkv, d, lw.wqkvT, 3 * d, 3 * d, 3 * d, d, st));
      }
      if (h->dt == 1) {
        // the forward GEMMs take fp16 operands: convert the forward copies in place
        // (the fast hi | lo rows and columns are written by reset_fast)
        HIPCHK(bf16_to_f16_launch(lw.wqkv, 3 * d, lw.wqkv, 3 * d, 1, 3 * d * d, st));
        HIPCHK(bf16_to_f16_launch(lw.wo, d, lw.wo, d, 1, d * d, st));
        void *gus = lw.fast ? lw.wgu_s : lw.wgu;
        HIPCHK(bf16_to_f16_launch(gus, d, gus, d, 2 * F, d, st));
        if (lw.fast)  // static down columns share the fast ones' scale
          for (int sq = 0; sq < h->B; ++sq) {
            void *sc = off(lw.wd, sq * h->fd_sb + (size_t)F * es);
            HIPCHK(bf16_to_f16_launch(sc, 3 * F, sc, 3 * F, d, F, st, h->wscale));
          }
        else
          HIPCHK(bf16_to_f16_launch(lw.wd, F, lw.wd, F, d, F, st));
      }
      const size_t plane = (size_t)h->H * lw.R * h->hd * es;
      lw.K = off(h->ring_base, roff);
      roff += plane;
      lw.Vt = off(h->ring_base, roff);
      roff += plane;
      if (lw.bwd_attn) {
        if (lw.fwd16) {
          lw.Kb = off(h->ring_base, roff);
          roff += plane;
        }
        lw.Kt = off(h->ring_base, roff);
        roff += plane;
        lw.V = off(h->ring_base, roff);
        roff += plane;
      }
    }
    // ---- state and chunk scratch
    const size_t bd = (size_t)b * d;        // one sequence's chunk
    const int Bb = h->B * b;                 // rows of a batched chunk
    const size_t Bbd = (size_t)Bb * d;
    const int Br = h->B * std::max(b, h->G);  // rows of the forward scratch: a chunk or a frozen-prefix group
    const size_t Brd = (size_t)Br * d;
    h->tok = (int *)dalloc(h, h->B * h->ld_tok * sizeof(int));
    h->losses = (float *)dalloc(h, h->B * c.max_tokens * sizeof(float));
    h->ids = (int *)dalloc(h, Br * sizeof(int));
    h->labs = (int *)dalloc(h, Br * sizeof(int));
    h->zero = (int *)dalloc(h, 64);
    h->closs = (float *)dalloc(h, Bb * sizeof(float));
    h->pos0 = (int *)dalloc(h, 64);
    h->flag = (int *)dalloc(h, 64);
    h->rope = (float2 *)dalloc(h, (size_t)c.max_tokens * (h->hd / 2) * sizeof(float2), false);
    HIPCHK(rope_table_launch(h->rope, c.max_tokens, h->hd, (double)c.rope_theta, st));
    h->h = (float *)dalloc(h, Bbd * 4);
    if (h->G > 0) {
      const size_t Gr = (size_t)h->B * h->G;  // rows of a frozen-prefix group
      h->h_lead = (float *)dalloc(h, Gr * d * 4);
      h->lead_n = (int *)dalloc(h, 64);
      h->ls.pos0 = (int *)dalloc(h, 64);
      h->ls.ids = (int *)dalloc(h, Gr * sizeof(int));
      h->ls.labs = (int *)dalloc(h, Gr * sizeof(int));
      h->ls.h = (float *)dalloc(h, Gr * d * 4);
      h->ls.lse2 = (float *)dalloc(h, (size_t)h->H * Gr * 4);
      h->ls.qkv = (float *)dalloc(h, 3 * Gr * d * 4);
      h->ls.a = dalloc(h, Gr * d * es);
      h->ls.qh = dalloc(h, Gr * d * es);
      h->ls.o = dalloc(h, Gr * d * es);
      h->ls.m = dalloc(h, Gr * d * es);
      h->ls.hmid = dalloc(h, Gr * F * es);
    }
    h->lse2 = (float *)dalloc(h, (size_t)h->H * Br * 4);
    h->a = dalloc(h, Brd * es);
    h->qkv = (float *)dalloc(h, 3 * Brd * 4);
    h->qh = dalloc(h, Brd * es);
    h->o = dalloc(h, Brd * es);
    h->m = dalloc(h, Brd * es);
    h->hmid = dalloc(h, (size_t)Br * (h->nu > 0 ? 2 * F : F) * es);
    h->nf = dalloc(h, Bbd * es);
    h->hf = (float *)dalloc(h, Bbd * 4);
    h->rf = (float *)dalloc(h, Bb * 4);
    h->zlab = (float *)dalloc(h, Bb * 4);
    h->lse = (float *)dalloc(h, Bb * 4);
    h->shift = (float *)dalloc(h, Bb * 4);
    h->part = (float2 *)dalloc(h, (size_t)Bb * h->P * sizeof(float2));
    h->part_arg = (int *)dalloc(h, (size_t)Bb * h->P * sizeof(int));
    h->rlosses = (float *)dalloc(h, c.max_tokens * sizeof(float));
    if (h->nu > 0) {
      h->dz = dalloc(h, (size_t)Bb * h->Vs * es);
      h->dn = (float *)dalloc(h, Bbd * 4);
      h->dh = (float *)dalloc(h, Bbd * 4);
      h->dy = dalloc(h, Bbd * es);
      h->dhmid = dalloc(h, (size_t)Bb * 2 * F * es);
      h->dgu = dalloc(h, (size_t)Bb * 4 * F * es);
      h->dm = (float *)dalloc(h, Bbd * 4);
      h->dO = dalloc(h, Bbd * es);
      h->dOt = dalloc(h, bd * es);                       // one sequence at a time
      h->Dq = (float *)dalloc(h, (size_t)h->H * b * 4);  // one sequence at a time
      h->dq = (float *)dalloc(h, Bbd * 4);
      h->dk = (float *)dalloc(h, Bbd * 4);
      h->dv = (float *)dalloc(h, Bbd * 4);
      h->dqkv = dalloc(h, 3 * Bbd * es);
      h->da = (float *)dalloc(h, Bbd * 4);
      for (int u = 0; u < h->nu; ++u) {
        Saved &S = h->saved[u];
        S.h_in = (float *)dalloc(h, Bbd * 4);
        S.r1 = (float *)dalloc(h, Bb * 4);
        S.lse2 = (float *)dalloc(h, (size_t)h->H * Bb * 4);
        S.h1 = (float *)dalloc(h, Bbd * 4);
        S.r2 = (float *)dalloc(h, Bb * 4);
        S.qkv = (float *)dalloc(h, 3 * Bbd * 4);
        S.qh = dalloc(h, Bbd * es);
        if (h->layers[h->L - h->nu + u].fwd16) S.qhb = dalloc(h, Bbd * es);
        S.qht = dalloc(h, Bbd * es);
        S.o = dalloc(h, Bbd * es);
        S.m = dalloc(h, Bbd * es);
        S.gu = dalloc(h, (size_t)Bb * 4 * F * es);
        S.hmid = dalloc(h, (size_t)Bb * 2 * F * es);
      }
    }
    h->attn_split = attn_pick_split(b, h->H, h->k, b);
    {
      int smax = h->attn_split;
      for (const LayerBuf &lw : h->layers) smax = std::max(smax, lw.fsplit);
      h->attn_ws_n = attn_ws_floats(smax, b, d, h->H, b);
      h->attn_ws = (float *)dalloc(h, h->attn_ws_n * 4);
      // a decode step has one query per head: split its window into up to 32 ranges of at
      // least 8 key tiles each (a work-group streams its tiles one after another)
      int ds = 32;
      while (ds > 1 && ((h->k + b) / 32 < 8 * ds ||
                        attn_ws_floats(ds, 16, d, h->H, b) > attn_ws_floats(smax, b, d, h->H, b)))
        ds /= 2;
      h->dec_split = ds;
    }
    if (h->nu > 0) {
      h->lm_headT = dalloc(h, (size_t)V * d * es, false);
      HIPCHK(transpose_launch(h->dt, SRC_WORK, h->lm_head, d, h->lm_headT, V, V, V, d, st));
      h->dyT = dalloc(h, bd * es);
      h->mT = dalloc(h, bd * es);
      h->hmidT = dalloc(h, (size_t)b * F * es);
      h->dguT = dalloc(h, (size_t)b * 2 * F * es);
    }
    // the LM head's forward copy (the logits of the cross-entropy and of the softmax) is fp16 in bf16 mode
    if (h->dt == 1) HIPCHK(bf16_to_f16_launch(h->lm_head, d, h->lm_head, d, 1, V * d, st));
    h->ws_elems = gemm_ws_elems(b, d);
    h->ws = (float *)dalloc(h, h->ws_elems * 4);
    // scratch starts as zeros (finite), so masked tile entries never carry NaN
    HIPCHK(hipStreamSynchronize(st));
    for (auto &z : h->zero_list) HIPCHK(hipMemsetAsync(z.first, 0, z.second, st));
    HIPCHK(hipStreamSynchronize(st));
    HIPCHK(hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking));
    if (h->G > 0) {
      HIPCHK(hipStreamCreateWithFlags(&h->lead_st, hipStreamNonBlocking));
      HIPCHK(hipEventCreateWithFlags(&h->ev_lead[0], hipEventDisableTiming));
      HIPCHK(hipEventCreateWithFlags(&h->ev_lead[1], hipEventDisableTiming));
    }
    HIPCHK(hipEventCreate(&h->ev_pf[0]));
    HIPCHK(hipEventCreate(&h->ev_pf[1]));
    HIPCHK(hipGetDevice(&h->dev));
    scratch_setup(h, st);
  } catch (const HipFail &f) {
    ttt_status s = fail_hip(h, f);
    hipStreamSynchronize(st);
    free_all(h);
    delete h;
    return f.e == hipErrorOutOfMemory ? TTT_ENOMEM : s;
  }
  *out = h;
  return TTT_OK;
}

}  // extern "C"

namespace {

// Algorithm 1 over every sequence of the handle.  noalloc: the split-K and attention
// partials go to this device's static scratch, every kernel is launched one by one
// (no graph is captured or instantiated) and no event is recorded, so the call
// allocates nothing; the results are the same bits as the graph-replayed call.
ttt_status prefill_impl(ttt_handle *h, const int32_t *d_tokens, int64_t T, float *d_losses,
                        float *const *d_fast_out, uint32_t flags, void *stream, bool noalloc) {
  if (!h) return fail(nullptr, TTT_EINVAL, "null handle");
  if (T < 0 || T > h->cfg.max_tokens) return fail(h, TTT_EINVAL, "T out of range [0, max_tokens]");
  if (T > 0 && (!d_tokens || !d_losses)) return fail(h, TTT_EINVAL, "null tokens or losses");
  if (d_fast_out)
    for (int i = 0; i < 3 * h->nu * h->B; ++i)
      if (!d_fast_out[i]) return fail(h, TTT_EINVAL, "null entry in d_fast_out");
  float *ws_keep = h->ws, *attn_keep = h->attn_ws;
  if (noalloc) {
    if (h->prof) return fail(h, TTT_EINVAL, "kernel timing is on (it creates events); disable it first");
    if (!h->scratch) return fail(h, TTT_EHIP, "static scratch unavailable: " + h->scratch_err);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->dev)
      return fail(h, TTT_EINVAL, "the current device is not the handle's device");
    // every split-K plan keeps its partials within ws_elems floats; the attention
    // splits within attn_ws_n
    if (h->ws_elems > SCRATCH_GEMM_FLOATS || h->attn_ws_n > SCRATCH_ATTN_FLOATS) {
      char buf[256];
      snprintf(buf, sizeof(buf),
               "shape needs %zu MiB of split-K and %zu MiB of attention partials; the static scratch holds "
               "%zu and %zu MiB",
               (h->ws_elems * 4) >> 20, (h->attn_ws_n * 4) >> 20, (SCRATCH_GEMM_FLOATS * 4) >> 20,
               (SCRATCH_ATTN_FLOATS * 4) >> 20);
      return fail(h, TTT_EUNSUPPORTED, buf);
    }
    h->ws = h->scratch;
    h->attn_ws = h->scratch + SCRATCH_GEMM_FLOATS;
  }
  flags |= h->cfg.flags;
  const bool update = !(flags & TTT_NO_UPDATE) && h->nu > 0;
  const bool use_graph = !(flags & TTT_NO_GRAPH) && !h->prof && !noalloc;
  hipStream_t st = (hipStream_t)stream;
  const int b = h->b;
  ttt_status ret = TTT_OK;
  try {
    h->ev_pf_set = false;
    if (!noalloc) HIPCHK(hipEventRecord(h->ev_pf[0], st));
    if (d_tokens)
      HIPCHK(hipMemcpy2DAsync(h->tok, h->ld_tok * sizeof(int), d_tokens, (size_t)(T + 1) * sizeof(int),
                              (size_t)(T + 1) * sizeof(int), h->B, hipMemcpyDeviceToDevice, st));
    HIPCHK(set_int_launch(h->pos0, 0, st));
    HIPCHK(set_int_launch(h->flag, 0, st));
    HIPCHK(zero_launch(h->ring_base, h->ring_bytes, st));
    reset_fast(h, st);
    const int64_t nfull = T / b;
    const int tail = (int)(T % b);
    if (h->G > 0) {
      // The frozen prefix of each group of G tokens, then the group's chunks from block Lf.
      // With graph replay the next group's frozen prefix runs on lead_st while this group's
      // chunk steps run on st (it reads only ids, frozen weights and the frozen blocks'
      // rings, and writes only its own scratch); otherwise everything runs on st in the
      // same order.  Results are the same either way.
      const bool ovl = use_graph;
      hipStream_t lst = ovl ? h->lead_st : st;
      HIPCHK(set_int_launch(h->ls.pos0, 0, st));
      if (ovl) {  // after the ids, the ring reset and the counter
        HIPCHK(hipEventRecord(h->ev_lead[1], st));
        HIPCHK(hipStreamWaitEvent(lst, h->ev_lead[1], 0));
      }
      if (T > 0) run_step(h, (int)std::min<int64_t>(h->G, T), false, MODE_PREFILL, use_graph, lst, true);
      if (ovl) HIPCHK(hipEventRecord(h->ev_lead[0], lst));
      for (int64_t g0 = 0; g0 < T; g0 += h->G) {
        const int gn = (int)std::min<int64_t>(h->G, T - g0);
        if (ovl) HIPCHK(hipStreamWaitEvent(st, h->ev_lead[0], 0));
        HIPCHK(hipMemcpyAsync(h->h_lead, h->ls.h, (size_t)h->B * h->G * h->d * 4, hipMemcpyDeviceToDevice, st));
        HIPCHK(set_int_launch(h->lead_n, gn, st));
        if (g0 + h->G < T) {
          if (ovl) {
            HIPCHK(hipEventRecord(h->ev_lead[1], st));
            HIPCHK(hipStreamWaitEvent(lst, h->ev_lead[1], 0));
          }
          run_step(h, (int)std::min<int64_t>(h->G, T - g0 - h->G), false, MODE_PREFILL, use_graph, lst, true);
          if (ovl) HIPCHK(hipEventRecord(h->ev_lead[0], lst));
        }
        for (int c0 = 0; c0 < gn; c0 += b) run_step(h, std::min(b, gn - c0), update, MODE_PREFILL, use_graph, st, false, true);
      }
      if (ovl) HIPCHK(hipStreamWaitEvent(st, h->ev_lead[0], 0));  // lead_st joins st (already, unless T = 0)
    } else {
      for (int64_t c = 0; c < nfull; ++c) run_step(h, b, update, MODE_PREFILL, use_graph, st);
      if (tail > 0) run_step(h, tail, update, MODE_PREFILL, use_graph, st);
    }
    if (T > 0) {
      const size_t ldl = (size_t)h->cfg.max_tokens * sizeof(float);
      HIPCHK(hipMemcpy2DAsync(d_losses, (size_t)T * sizeof(float), h->losses, ldl, (size_t)T * sizeof(float), h->B,
                              hipMemcpyDeviceToDevice, st));
      for (int s = 0; s < h->B; ++s)
        HIPCHK(finite_check_launch(h->losses + (size_t)s * h->cfg.max_tokens, T, h->flag, st));
    }
    if (update && T > 0) check_masters(h, st);
    if (d_fast_out) copy_fast_out(h, d_fast_out, st);
    if (!noalloc) {
      HIPCHK(hipEventRecord(h->ev_pf[1], st));
      h->ev_pf_set = true;
    }
    h->len = T;
    h->dstart = T;
    h->have_state = d_tokens != nullptr;  // the token at position T is known
    h->chunks_last = nfull + (tail > 0 ? 1 : 0);
  } catch (const HipFail &f) {
    h->have_state = false;
    ret = fail_hip(h, f);
  }
  h->ws = ws_keep;
  h->attn_ws = attn_keep;
  return ret;
}

}  // namespace

extern "C" {

ttt_status ttt_prefill(ttt_handle *h, const int32_t *d_tokens, int64_t T, float *d_losses, float *const *d_fast_out,
                       uint32_t flags, void *stream) {
  return prefill_impl(h, d_tokens, T, d_losses, d_fast_out, flags, stream, false);
}

ttt_status ttt_prefill_noalloc(ttt_handle *h, const int32_t *d_tokens, int64_t T, float *d_losses,
                               float *const *d_fast_out, uint32_t flags, void *stream) {
  return prefill_impl(h, d_tokens, T, d_losses, d_fast_out, flags, stream, true);
}

ttt_status ttt_decode(ttt_handle *h, int64_t n_steps, const int32_t *d_forced, int32_t *d_tokens_out,
                      float *d_losses_out, float *const *d_fast_out, uint32_t flags, void *stream) {
  if (!h) return fail(nullptr, TTT_EINVAL, "null handle");
  if (h->B != 1) return fail(h, TTT_EUNSUPPORTED, "ttt_decode continues a single sequence (n_seq = 1)");
  if (!h->have_state) return fail(h, TTT_EINVAL, "no prefill state to continue (run ttt_prefill with tokens first)");
  if (n_steps < 0 || h->len + n_steps > h->cfg.max_tokens)
    return fail(h, TTT_EINVAL, "n_steps out of range: the sequence may not exceed max_tokens positions");
  if (n_steps > 0 && (!d_tokens_out || !d_losses_out)) return fail(h, TTT_EINVAL, "null tokens_out or losses_out");
  if (d_fast_out)
    for (int i = 0; i < 3 * h->nu; ++i)
      if (!d_fast_out[i]) return fail(h, TTT_EINVAL, "null entry in d_fast_out");
  flags |= h->cfg.flags;
  const bool update = !(flags & TTT_NO_UPDATE) && h->nu > 0;
  const bool use_graph = !(flags & TTT_NO_GRAPH) && !h->prof;
  hipStream_t st = (hipStream_t)stream;
  const int64_t len0 = h->len;
  try {
    HIPCHK(set_int_launch(h->pos0, (int)len0, st));
    if (d_forced && n_steps > 0)
      HIPCHK(hipMemcpyAsync(h->tok + len0 + 1, d_forced, (size_t)n_steps * sizeof(int), hipMemcpyDeviceToDevice, st));
    for (int64_t j = 0; j < n_steps; ++j) {
      // position len: predict the token after it (the forced one's loss, or the argmax)
      run_step(h, 1, false, d_forced ? MODE_FORCED : MODE_GREEDY, use_graph, st);
      h->len += 1;
      if (h->len - h->dstart == h->b) {
        // every target of the open chunk is known: its update (Algorithm 3 step 3)
        // before the next position is fed
        if (update) {
          HIPCHK(set_int_launch(h->pos0, (int)h->dstart, st));
          run_step(h, h->b, true, MODE_RECOMPUTE, use_graph, st);
        }
        h->dstart += h->b;
      }
    }
    if (n_steps > 0) {
      HIPCHK(hipMemcpyAsync(d_tokens_out, h->tok + len0 + 1, (size_t)n_steps * sizeof(int), hipMemcpyDeviceToDevice,
                            st));
      HIPCHK(hipMemcpyAsync(d_losses_out, h->losses + len0, (size_t)n_steps * sizeof(float), hipMemcpyDeviceToDevice,
                            st));
      HIPCHK(finite_check_launch(h->losses + len0, n_steps, h->flag, st));
    }
    if (update && h->dstart > len0) check_masters(h, st);
    if (d_fast_out) copy_fast_out(h, d_fast_out, st);
  } catch (const HipFail &f) {
    h->have_state = false;
    return fail_hip(h, f);
  }
  return TTT_OK;
}

ttt_status ttt_check_finite(ttt_handle *h, void *stream) {
  if (!h) return fail(nullptr, TTT_EINVAL, "null handle");
  int flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, h->flag, sizeof(int), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(h, HipFail{e, "ttt_check_finite"});
  return flag ? fail(h, TTT_ENONFINITE, "non-finite loss or fast weight") : TTT_OK;
}

ttt_status ttt_get_stats(ttt_handle *h, double *ms_last, int64_t *chunks_last, int64_t *launches_per_chunk) {
  if (!h) return fail(nullptr, TTT_EINVAL, "null handle");
  if (chunks_last) *chunks_last = h->chunks_last;
  if (launches_per_chunk) *launches_per_chunk = h->launches;
  if (ms_last) {
    *ms_last = 0.0;
    if (h->ev_pf_set) {
      float ms = 0.f;
      hipError_t e = hipEventSynchronize(h->ev_pf[1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, h->ev_pf[0], h->ev_pf[1]);
      if (e != hipSuccess) return fail_hip(h, HipFail{e, "ttt_get_stats"});
      *ms_last = ms;
    }
  }
  return TTT_OK;
}

ttt_status ttt_set_kernel_timing(ttt_handle *h, int enable) {
  if (!h) return fail(nullptr, TTT_EINVAL, "null handle");
  h->prof = enable != 0;
  for (int i = 0; i < K_NCLASS; ++i) {
    h->kt_ms[i] = 0.0;
    h->kt_n[i] = 0;
  }
  h->ev_used = 0;
  return TTT_OK;
}

int ttt_kernel_class_count(void) { return K_NCLASS; }

ttt_status ttt_get_kernel_time(const ttt_handle *h, int cls, const char **name, double *total_ms, int64_t *count) {
  if (!h || cls < 0 || cls >= K_NCLASS) return TTT_EINVAL;
  if (name) *name = kclass_names[cls];
  if (total_ms) *total_ms = h->kt_ms[cls];
  if (count) *count = h->kt_n[cls];
  return TTT_OK;
}

const char *ttt_last_error(const ttt_handle *h) { return h ? h->err.c_str() : g_thread_err.c_str(); }

void ttt_destroy(ttt_handle *h) {
  if (!h) return;
  hipDeviceSynchronize();
  for (hipEvent_t e : h->ev) hipEventDestroy(e);
  free_all(h);
  delete h;
}

}  // extern "C"
