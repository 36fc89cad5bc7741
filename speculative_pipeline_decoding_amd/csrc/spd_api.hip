// Host side of the SPD library: configuration, workspace plan, the pipeline
// state machine (in-flight ring, stage plan, commit / rollback bookkeeping),
// and the per-step launch plan. Step semantics follow arXiv 2605.30852 as
// summarised on the pith.science review page ("What carries the argument"):
// n stages, n tokens in flight, the PDM on the step's input states, streaming
// verification, truncate / flush / reseed on rejection.
//
// Device rings are indexed by position mod (n + 1): the residual and anchor
// states of in-flight positions, their tokens, and the draft distributions.
// A rejection therefore needs no device work: KV lengths are host state, and
// every ring slot of a discarded position is rewritten before it is read.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "spd.h"
#include "spd_internal.h"

using namespace spd;

namespace spd {
int attn_max_split();
bool attn_supported_head_dim(int hd, bool bf16);
}

// Device memory for spd_prefill_static_scratch, the prefill entry point for callers that
// cannot allocate: its chunk buffers live in this array. Each GPU the library runs on holds
// its own copy until the process ends. In host code the name is only a stand-in: the
// device address comes from hipGetSymbolAddress, looked up once per device at spd_init.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kScratchDevices] = {};
std::string g_scratch_err[kScratchDevices];

// The current device's copy of `scratch` (looked up on its first use), or nullptr with a
// message in err.
char* scratch_of_current_device(std::string& err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { err = std::string("hipGetDevice: ") + hipGetErrorString(e); return nullptr; }
  if (dev < 0 || dev >= kScratchDevices) { err = "device index beyond the static scratch table"; return nullptr; }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev] && g_scratch_err[dev].empty()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      g_scratch_err[dev] = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
    else
      g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}
}  // namespace

namespace {

thread_local std::string g_init_error;

constexpr int kPrefillChunk = 512;
constexpr int kVocabBlocks = 256;
constexpr size_t kDescBytes = 512 * 1024;
constexpr int kTensorsPerLayer = 7;
enum { T_ATTN_NORM = 0, T_QKV, T_O, T_FFN_NORM, T_GATE, T_UP, T_DOWN };

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Distance in floats between two float arrays that may live in different allocations.
long long float_gap(const float* to, const float* from) {
  return ((long long)(intptr_t)to - (long long)(intptr_t)from) / (long long)sizeof(float);
}

struct Inflight {
  int pos;
  int stage;
  int w = 1;       // candidates at this position: the token and w - 1 siblings (draft trees)
};

// Launch kinds of a step (and their timing buckets). The PDM's launches run on a
// second stream, concurrently with the target's sub-layers (fork after the embed,
// join before the LM head).
enum OpKind { OP_EMBED = 0, OP_GEMV_PROJ, OP_GEMV_QKV, OP_ATTN, OP_LIN, OP_GEMV_O, OP_GEMV_GU,
              OP_GEMV_DOWN, OP_GEMV_HEAD, OP_VOCAB, OP_FINAL, OP_RESID, OP_PDM_QKV, OP_PDM_ATTN,
              OP_PDM_O, OP_PDM_GU, OP_PDM_DOWN, OP_NUCLEUS, OP_GATHER, OP_NKINDS, OP_FORK = 100,
              OP_JOIN = 101 };

struct Op {
  int kind;
  size_t off;      // descriptor offset in the step's descriptor block
  int count;       // problems
  int ntiles;      // workgroups
  int split;       // attention split length
  double bytes;    // algorithmic HBM bytes (weights + KV) for the timing report
  int stream = 0;  // 0: the caller's stream, 1: the PDM stream
  GemvPlan plan;   // GEMV: kernel kind, workgroups and LDS (gemv_plan)
  int layer = -1;  // the one target layer this launch serves, when only one token is in it
  int adopt = 0;   // OP_EMBED: target layers of a sibling's keys to adopt (extra workgroups);
                   // OP_ATTN: 1 if a problem is a sibling candidate (its own key in a side row)
};

struct Plan {
  int L, d, hq, hkv, hd, F, V, n, k, Ls, max_ctx, ring, qrows, linrows, qo;
  bool bf16;       // weights
  int esz;
  bool kv_bf16;    // KV caches (target and PDM): bf16, key-blocked V; else fp32, row-major
  int kv_esz;
  float theta, eps;
  int fill;
  int spec_output;   // the PDM reads the step's output states, after the target layers
  int W;             // draft candidates per position; ring rows are slot * W + candidate
  int side_rows;     // rows of each layer's sibling side cache per kv head: ring * (W - 1)
  size_t side_layer_bytes;
  std::vector<int> kind, sizes, starts, anchors, ord;   // ord: index among softmax / linear layers
  int nsoft = 0, nlin = 0;
  // workspace offsets
  size_t o_kv, o_pkv, o_side, o_top, o_lin, o_h, o_anch, o_tok, o_qring, o_qlse, o_cut, o_nuc, o_X, o_hp, o_qbuf, o_attn,
      o_act, o_lqkv, o_logits, o_part, o_verdict, o_desc, o_apart, o_rope,
      o_forced, o_ptok, o_pH, o_pA, o_pQKV, o_pO, o_pG, o_pU, o_pZ, o_panch, total;
  size_t kv_layer_bytes;     // K and V of one layer
  size_t lin_state_bytes;    // one state [hq][hd][hd] f32
};

bool plan_config(const spd_model_config* c, Plan& p, std::string& err) {
  auto bad = [&](const char* m) { err = m; return false; };
  if (!c) return bad("null config");
  p.L = c->n_layers; p.d = c->d_model; p.hq = c->n_q_heads; p.hkv = c->n_kv_heads;
  p.hd = c->head_dim; p.F = c->d_ffn; p.V = c->vocab; p.n = c->n_stages; p.k = c->n_anchors;
  p.Ls = c->pdm_layers; p.max_ctx = c->max_ctx; p.theta = c->rope_theta; p.eps = c->rms_eps;
  p.fill = c->anchor_fill;
  if (c->speculate_from != SPD_SPEC_INPUT && c->speculate_from != SPD_SPEC_OUTPUT)
    return bad("speculate_from must be SPD_SPEC_INPUT or SPD_SPEC_OUTPUT");
  p.spec_output = c->speculate_from == SPD_SPEC_OUTPUT;
  if (c->draft_width < 0 || c->draft_width > kMaxWidth)
    return bad("draft_width must be in [1, 4] (0 means 1)");
  p.W = c->draft_width < 1 ? 1 : c->draft_width;
  if (p.W > 1 && p.spec_output) return bad("draft trees (draft_width > 1) need SPD_SPEC_INPUT");
  if (c->dtype != SPD_F32 && c->dtype != SPD_BF16) return bad("dtype must be SPD_F32 or SPD_BF16");
  p.bf16 = c->dtype == SPD_BF16;
  p.esz = p.bf16 ? 2 : 4;
  if (c->kv_dtype != SPD_KV_AUTO && c->kv_dtype != SPD_KV_F32)
    return bad("kv_dtype must be SPD_KV_AUTO or SPD_KV_F32");
  p.kv_bf16 = p.bf16 && c->kv_dtype == SPD_KV_AUTO;
  p.kv_esz = p.kv_bf16 ? 2 : 4;
  if (p.L < 1 || p.d < 8 || p.hq < 1 || p.hkv < 1 || p.hd < 2 || p.F < 8 || p.V < 2)
    return bad("model dimensions out of range");
  if (p.d % 8 || p.F % 8 || (p.hq * p.hd) % 8) return bad("d_model, d_ffn, n_q_heads*head_dim must be multiples of 8");
  if (!attn_supported_head_dim(p.hd, p.kv_bf16))
    return bad("head_dim must be 16, 32, 64, 80 or 128");
  if (p.hq % p.hkv || p.hq / p.hkv > 16) return bad("n_q_heads must be a multiple of n_kv_heads, group <= 16");
  if (p.n < 1 || p.n > kMaxStages || p.n > p.L) return bad("n_stages must be in [1, min(L, 16)]");
  if (p.k < 1 || p.k > kMaxAnchors || !c->anchors) return bad("need 1..8 anchors");
  if (p.Ls < 1 || p.Ls > 16) return bad("pdm_layers must be in [1, 16]");
  if (p.fill != SPD_FILL_CLAMP && p.fill != SPD_FILL_ZERO) return bad("bad anchor_fill");
  if (p.max_ctx < 2) return bad("max_ctx too small");
  if (!(p.eps > 0.f) || !(p.theta > 0.f)) return bad("rms_eps and rope_theta must be positive");
  p.anchors.assign(c->anchors, c->anchors + p.k);
  if (p.anchors[0] != 0) return bad("anchors[0] must be 0 (the embedding)");
  for (int i = 1; i < p.k; ++i)
    if (p.anchors[i] <= p.anchors[i - 1]) return bad("anchors must be strictly ascending");
  if (p.anchors.back() > p.L) return bad("anchor depth beyond n_layers");
  p.kind.assign(p.L, SPD_LAYER_SOFTMAX);
  if (c->layer_kind)
    for (int l = 0; l < p.L; ++l) p.kind[l] = c->layer_kind[l];
  for (int l = 0; l < p.L; ++l) {
    if (p.kind[l] != SPD_LAYER_SOFTMAX && p.kind[l] != SPD_LAYER_LINEAR) return bad("bad layer_kind");
    if (p.W > 1 && p.kind[l] == SPD_LAYER_LINEAR)
      return bad("draft trees (draft_width > 1) need softmax layers only");
  }
  p.sizes.resize(p.n);
  if (c->stage_layers) {
    int s = 0;
    for (int i = 0; i < p.n; ++i) {
      p.sizes[i] = c->stage_layers[i];
      if (p.sizes[i] < 1) return bad("stage sizes must be >= 1");
      s += p.sizes[i];
    }
    if (s != p.L) return bad("stage sizes must sum to n_layers");
  } else {
    for (int i = 0; i < p.n; ++i) p.sizes[i] = p.L / p.n + (i < p.L % p.n ? 1 : 0);
  }
  p.starts.resize(p.n);
  for (int i = 0, s = 0; i < p.n; ++i) { p.starts[i] = s; s += p.sizes[i]; }
  p.ord.assign(p.L, 0);
  for (int l = 0; l < p.L; ++l) p.ord[l] = p.kind[l] == SPD_LAYER_SOFTMAX ? p.nsoft++ : p.nlin++;
  p.ring = p.n + 1;
  p.qrows = (p.hq + 2 * p.hkv) * p.hd;
  p.linrows = 3 * p.hq * p.hd;
  p.qo = p.hq * p.hd;
  // workspace plan
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  const size_t ctx = p.max_ctx;
  p.kv_layer_bytes = 2 * (size_t)p.hkv * kv_ctx(p.max_ctx) * p.hd * p.kv_esz;
  p.lin_state_bytes = (size_t)p.hq * p.hd * p.hd * 4;
  p.o_kv = take(p.nsoft * p.kv_layer_bytes);
  p.o_pkv = take((size_t)p.Ls * p.kv_layer_bytes);
  p.side_rows = p.ring * (p.W - 1);
  p.side_layer_bytes = 2 * (size_t)p.hkv * p.side_rows * p.hd * p.kv_esz;
  p.o_side = take(p.nsoft * p.side_layer_bytes);
  p.o_lin = take((size_t)p.nlin * p.ring * p.lin_state_bytes);
  p.o_h = take((size_t)p.ring * p.W * p.d * 4);
  p.o_anch = take((size_t)p.ring * p.W * p.k * p.d * 4);
  p.o_tok = take((size_t)p.ring * p.W * 4);
  p.o_qring = take((size_t)p.ring * p.V * 4);
  p.o_qlse = take((size_t)p.ring * 4);
  p.o_cut = take((size_t)(1 + p.ring) * sizeof(NucleusCut));   // target row, then draft ring
  p.o_nuc = take(kNucPartBytes + kNucHistBytes + kNucCntBytes + (size_t)2 * p.V * sizeof(int2));
  const int T = p.n * p.W + p.ring;   // decode rows: target candidates + PDM rows
  p.o_X = take((size_t)p.ring * p.k * p.d * 4);
  p.o_hp = take((size_t)p.ring * p.d * 4);
  p.o_qbuf = take((size_t)T * p.qo * 4);
  p.o_attn = take((size_t)T * p.qo * 4);
  p.o_act = take((size_t)T * p.F * 4);
  p.o_lqkv = take((size_t)p.n * p.linrows * 4);
  p.o_logits = take((size_t)p.V * 4);
  p.o_part = take((size_t)3 * kVocabBlocks * sizeof(VocabPartial));
  p.o_top = take((size_t)kVocabBlocks * sizeof(VocabTop));
  p.o_verdict = take(sizeof(Verdict));
  p.o_desc = take(kDescBytes);
  const int G = p.hq / p.hkv;
  p.o_apart = take((size_t)T * p.hkv * attn_max_split() * std::max(G, 16) * (p.hd + 2) * 4);
  p.o_rope = take((size_t)ctx * (p.hd / 2) * sizeof(float2));
  p.o_forced = take(ctx * 4);
  const size_t CH = kPrefillChunk;
  const size_t widest = std::max({(size_t)p.d, (size_t)p.qo, (size_t)p.F, (size_t)p.k * p.d});
  p.o_ptok = take(ctx * 4);
  p.o_pH = take(CH * p.d * 4);
  p.o_pA = take(CH * widest * 4);
  p.o_pQKV = take(CH * std::max(p.qrows, p.linrows) * 4);
  p.o_pO = take(CH * p.qo * 4);
  p.o_pG = take(CH * p.F * 4);
  p.o_pU = take(CH * p.F * 4);
  p.o_pZ = take(CH * p.d * 4);
  p.o_panch = take((size_t)p.k * CH * p.d * 4);
  p.total = o;
  return true;
}

}  // namespace

struct spd_handle {
  Plan p;
  // weights
  const void* embed;
  const void* head;
  const float* final_norm;
  const void* proj;
  const float* pdm_final_norm;
  std::vector<const void*> lw;   // [L][7]
  std::vector<const void*> pw;   // [Ls][7]
  // sampling
  float temp, top_p, forced_p;
  unsigned long long seed;
  int forced_mode;
  std::vector<int> forced_ref;
  // device
  char* ws;
  char* scratch = nullptr;         // this device's copy of the static scratch array
  std::string scratch_err;
  hipStream_t st;                 // the caller's stream: target chain, head, verify
  hipStream_t st2 = nullptr;      // library-owned stream for the PDM chain
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // pinned host staging
  char* h_desc = nullptr;          // pinned staging of the step's descriptor block
  char* d_hdesc = nullptr;         // its device view
  size_t desc_used = 0;            // bytes of the current step's block
  // two staging blocks: while a step runs, the next one (when nothing exits, its state
  // is known at launch) is built into the other block, off the critical path
  char* h_desc_base = nullptr;
  char* d_hdesc_base = nullptr;
  int next_buf = 0;
  bool pre_valid = false;
  std::deque<Inflight> pre_F;      // the state the prebuilt step was built for
  int pre_pdm_len = 0;
  std::vector<Op> pre_ops;
  std::vector<std::pair<int, int>> pre_layers;
  bool pre_exit = false;
  int pre_v = 0, pre_dpos = 0, pre_newest = 0;
  size_t pre_used = 0;
  // pinned verdicts, one per staging block: the verdict kernels of a step write the slot of
  // the block that step was built in (d_hverdict: the current block's device view)
  Verdict* h_verdict_base = nullptr;
  Verdict* d_hverdict_base = nullptr;
  Verdict* d_hverdict = nullptr;
  int cur_buf = 0;                 // the staging block h_desc / d_hdesc / d_hverdict point at
  int pend_buf = 0;                // the block of the pending step
  hipEvent_t ev_step[2] = {nullptr, nullptr};   // end of the last step run from each block
  // lookahead: a step that verifies nothing fixes the next step's state at launch, so that
  // step is launched at once (from the other block) and the GPU never waits for the host
  bool lookahead = false;
  bool ahead = false;              // the prebuilt step has been launched already
  int pre_buf = 0;
  // state machine
  enum { S_INIT, S_READY, S_PENDING } state = S_INIT;
  int P0 = 0;
  std::deque<Inflight> F;
  int pdm_len = 0;
  std::vector<int> kv_len;
  long long N = 0, K = 0, acc = 0, rej = 0;
  // a sibling candidate accepted at adopt_pos: the next step adopts it (its states and
  // keys move to the position's main rows) before anything reads them
  bool adopt = false;
  int adopt_pos = 0, adopt_idx = 0, adopt_layers = 0;
  // the pending step
  bool pend_exit = false;
  int pend_v = 0, pend_dpos = 0, pend_newest = 0;
  std::vector<std::pair<int, int>> pend_layers;   // (layer, pos) processed
  std::vector<Op> ops;
  // timing
  bool timing = false;
  bool serial = false;            // the PDM chain on the caller's stream (timing mode 2)
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_kind;
  std::vector<int> ev_layer;
  std::vector<double> kl_ms;        // per target layer: kernel time of its single-token passes
  std::vector<long long> kl_passes;
  std::vector<double> ev_bytes;
  double kt_ms[OP_NKINDS] = {};
  double kt_bytes[OP_NKINDS] = {};
  long long kt_count[OP_NKINDS] = {};
  std::string err;

  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  int slot(int pos) const { return pos % p.ring; }
  const void* W(int l, int t) const { return lw[(size_t)l * kTensorsPerLayer + t]; }
  const void* PW(int r, int t) const { return pw[(size_t)r * kTensorsPerLayer + t]; }
  void* kvK(int l) const { return ws + p.o_kv + (size_t)p.ord[l] * p.kv_layer_bytes; }
  void* kvV(int l) const { return (char*)kvK(l) + p.kv_layer_bytes / 2; }
  void* pK(int r) const { return ws + p.o_pkv + (size_t)r * p.kv_layer_bytes; }
  // sibling candidates' keys and values of softmax layer l: [hkv][side_rows][hd] each
  void* sideK(int l) const { return ws + p.o_side + (size_t)p.ord[l] * p.side_layer_bytes; }
  void* sideV(int l) const { return (char*)sideK(l) + p.side_layer_bytes / 2; }
  // ring row of the token (candidate 0) at a position
  int row(int pos) const { return slot(pos) * p.W; }
  // state of linear layer l after the position whose ring slot is `slot`
  float* lin(int l, int slot) const {
    return reinterpret_cast<float*>(ws + p.o_lin +
                                    ((size_t)p.ord[l] * p.ring + slot) * p.lin_state_bytes);
  }
  void* pV(int r) const { return (char*)pK(r) + p.kv_layer_bytes / 2; }
  // the top-p selection's scratch regions
  void nucleus_scratch(VocabDesc& vd) const {
    char* b = ws + p.o_nuc;
    vd.nuc_part = reinterpret_cast<unsigned long long*>(b);
    vd.nuc_hist = reinterpret_cast<unsigned long long*>(b + kNucPartBytes);
    vd.nuc_cnt = reinterpret_cast<int*>(b + kNucPartBytes + kNucHistBytes);
    vd.nuc_max = reinterpret_cast<float*>(b + kNucPartBytes + kNucHistBytes + 2 * 64 * 4);
    vd.nuc_cand = reinterpret_cast<int2*>(b + kNucPartBytes + kNucHistBytes + kNucCntBytes);
  }
};

namespace {

// Points the step-building state at staging block b (descriptors and verdict slot).
void use_desc_buf(spd_handle* h, int b) {
  h->cur_buf = b;
  h->h_desc = h->h_desc_base + (size_t)b * kDescBytes;
  h->d_hdesc = h->d_hdesc_base + (size_t)b * kDescBytes;
  h->d_hverdict = h->d_hverdict_base + b;
}

int fail(spd_handle* h, int code, const std::string& m) {
  if (h) h->err = m;
  return code;
}

#define HIPCHK(h, call)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(h, SPD_E_DEVICE, std::string(#call) + ": " + hipGetErrorString(e_));   \
  } while (0)

// ---- descriptor block builder -------------------------------------------------
// Appends descriptors to one pinned staging block. Nothing is written past the block (the
// other block may belong to a step on the GPU): an item that does not fit is dropped,
// `used` still counts it, and the caller rejects the step when used > kDescBytes.
struct DescWriter {
  char* base;
  size_t used = 0;
  template <typename T> size_t put(const T* items, int count) {
    used = align_up(used, 64);
    const size_t at = used;
    const size_t n = sizeof(T) * (size_t)count;
    if (at + n <= kDescBytes) std::memcpy(base + at, items, n);
    used += n;
    return at;
  }
};

GemvPlan finish_tiles(const Plan& p, std::vector<GemvProb>& v) {
  return gemv_plan(v.data(), (int)v.size(), p.bf16);
}

GemvProb gemv(const void* W, int rows, int K, const float* x, long long xs, int nvec, int epi,
              float* y, long long ys, const float* gain, long long gs, float eps) {
  GemvProb g{};
  g.W = W; g.rows = rows; g.K = K; g.x = x; g.x_stride = xs; g.nvec = nvec; g.epi = epi;
  g.y = y; g.y_stride = ys; g.gain = gain; g.gain_stride = gs; g.eps = eps;
  return g;
}

double gemv_bytes(const std::vector<GemvProb>& v, int esz) {
  double b = 0;
  for (auto& g : v) b += (double)g.rows * g.K * esz * (g.epi == EPI_SWIGLU ? 2 : 1);
  return b;
}

int attn_split(const Plan& p, const std::vector<AttnProb>& v) {
  long long keys = 0;
  int maxlen = 1;
  for (auto& a : v) {
    const int last = a.len + a.nrows - 1;   // keys of the problem's last row
    keys += last;
    maxlen = std::max(maxlen, last);
  }
  const long long target = 2 * 256;   // workgroups to fill 256 CUs twice
  long long s = (keys * p.hkv + target - 1) / target;
  s = std::max<long long>(kAttnTile, (s + kAttnTile - 1) / kAttnTile * kAttnTile);
  while ((maxlen + s - 1) / s > attn_max_split()) s += kAttnTile;
  return (int)s;
}

int finish_attn(const Plan& p, std::vector<AttnProb>& v, int split, int slot0) {
  int t = 0;
  for (size_t i = 0; i < v.size(); ++i) {
    v[i].nsplit = (v[i].len + v[i].nrows - 1 + split - 1) / split;
    v[i].tile0 = t;
    v[i].slot = slot0 + (int)i;
    t += p.hkv * v[i].nsplit;
  }
  return t;
}

void fill_rope(const Plan& p, std::vector<float2>& tab) {
  const int half = p.hd / 2;
  tab.resize((size_t)p.max_ctx * half);
  for (int pos = 0; pos < p.max_ctx; ++pos)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)p.theta, -2.0 * i / p.hd);
      const double a = (double)pos * inv;
      tab[(size_t)pos * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
}

hipStream_t op_stream(const spd_handle* h, const Op& op) {
  return op.stream && !h->serial ? h->st2 : h->st;
}

int gemv_role(int kind) {
  switch (kind) {
    case OP_GEMV_PROJ: return GEMV_PROJ;
    case OP_GEMV_QKV: return GEMV_QKV;
    case OP_GEMV_O: return GEMV_O;
    case OP_GEMV_GU: return GEMV_GATE_UP;
    case OP_GEMV_DOWN: return GEMV_DOWN;
    case OP_PDM_QKV: return GEMV_PDM_QKV;
    case OP_PDM_O: return GEMV_PDM_O;
    case OP_PDM_GU: return GEMV_PDM_GATE_UP;
    case OP_PDM_DOWN: return GEMV_PDM_DOWN;
  }
  return GEMV_HEAD;
}

// Launch one op of the plan (with packet-bound timing events when ev is set).
hipError_t run_op(spd_handle* h, const Op& op, LaunchEv ev = {}) {
  const Plan& p = h->p;
  char* d = h->ws + p.o_desc;
  const float2* rope = h->at<float2>(p.o_rope);
  hipStream_t st = op_stream(h, op);
  switch (op.kind) {
    case OP_FORK: {
      hipError_t e = hipEventRecord(h->ev_fork, h->st);
      return e != hipSuccess ? e : hipStreamWaitEvent(h->st2, h->ev_fork, 0);
    }
    case OP_JOIN: {
      hipError_t e = hipEventRecord(h->ev_join, h->st2);
      return e != hipSuccess ? e : hipStreamWaitEvent(h->st, h->ev_join, 0);
    }
    case OP_EMBED:
      // the step's first launch: it reads its own descriptor from the pinned staging and
      // copies the whole block to the device for the launches that follow
      return launch_embed_gather(reinterpret_cast<const EmbedGather*>(h->d_hdesc + op.off),
                                 h->d_hdesc, d, h->desc_used, op.count, p.k, p.d, p.bf16, st, ev,
                                 op.adopt);
    case OP_GATHER:
      // gather-only (output states): the descriptor block is on the device by now
      return launch_embed_gather(reinterpret_cast<const EmbedGather*>(d + op.off), nullptr,
                                 nullptr, 0, op.count, p.k, p.d, p.bf16, st, ev);
    case OP_GEMV_PROJ: case OP_GEMV_QKV: case OP_GEMV_O: case OP_GEMV_GU: case OP_GEMV_DOWN:
    case OP_GEMV_HEAD: case OP_PDM_QKV: case OP_PDM_O: case OP_PDM_GU: case OP_PDM_DOWN:
      return launch_gemv(gemv_role(op.kind), reinterpret_cast<const GemvProb*>(d + op.off),
                         op.count, op.plan, p.bf16, rope, st, ev);
    case OP_LIN:
      return launch_linear_step(reinterpret_cast<const LinProb*>(d + op.off), op.count, p.hq, p.hd,
                                kLinEps, st, ev);
    case OP_ATTN: case OP_PDM_ATTN:
      return launch_attention(reinterpret_cast<const AttnProb*>(d + op.off), op.count, op.ntiles,
                              p.kv_bf16, p.hq, p.hkv, p.hd, p.max_ctx, op.split,
                              op.ntiles > op.count * p.hkv, h->at<float>(p.o_apart), st, ev,
                              op.adopt != 0);
    case OP_VOCAB:
      return launch_vocab_stats(reinterpret_cast<const VocabDesc*>(d + op.off), kVocabBlocks,
                                h->at<VocabPartial>(p.o_part), st, ev);
    case OP_NUCLEUS:
      return launch_nucleus(reinterpret_cast<const VocabDesc*>(d + op.off), kVocabBlocks,
                            h->at<VocabPartial>(p.o_part), st, ev);
    case OP_FINAL:
      return launch_finalize(reinterpret_cast<const FinalizeDesc*>(d + op.off), st, ev);
    case OP_RESID:
      // after a rejection at T > 0: the residual draw, or with draft trees the later rounds
      if (p.W > 1)
        return launch_tree_rounds(reinterpret_cast<const FinalizeDesc*>(d + op.off),
                                  h->at<VocabPartial>(p.o_part), kVocabBlocks, st, ev);
      return launch_residual_impl(reinterpret_cast<const FinalizeDesc*>(d + op.off),
                                  h->at<VocabPartial>(p.o_part), kVocabBlocks, st, ev);
  }
  return hipErrorInvalidValue;
}

// Launches one step's ops from staging block buf (used bytes of it) and records the
// block's end-of-step event on the caller's stream.
int run_ops(spd_handle* h, const std::vector<Op>& ops, int buf, size_t used) {
  use_desc_buf(h, buf);
  h->desc_used = used;
  size_t k = 0;
  for (const Op& op : ops) {
    if (h->timing && op.kind < OP_NKINDS) {
      if (2 * k + 1 >= h->ev.size()) return fail(h, SPD_E_CAPACITY, "internal: timing event pool");
      const LaunchEv ev{h->ev[2 * k], h->ev[2 * k + 1]};
      HIPCHK(h, run_op(h, op, ev));
      h->ev_kind.push_back(op.kind);
      h->ev_layer.push_back(op.layer);
      h->ev_bytes.push_back(op.bytes);
      ++k;
    } else {
      HIPCHK(h, run_op(h, op));
    }
  }
  HIPCHK(h, hipEventRecord(h->ev_step[buf], h->st));
  return SPD_OK;
}

int collect_timing(spd_handle* h) {
  for (size_t i = 0; i < h->ev_kind.size(); ++i) {
    float ms = 0.f;
    HIPCHK(h, hipEventElapsedTime(&ms, h->ev[2 * i], h->ev[2 * i + 1]));
    h->kt_ms[h->ev_kind[i]] += ms;
    h->kt_bytes[h->ev_kind[i]] += h->ev_bytes[i];
    h->kt_count[h->ev_kind[i]] += 1;
    const int l = h->ev_layer[i];
    if (l >= 0 && l < (int)h->kl_ms.size()) {
      h->kl_ms[l] += ms;
      if (h->ev_kind[i] == OP_GEMV_QKV) h->kl_passes[l] += 1;   // one per pass through the layer
    }
  }
  h->ev_kind.clear();
  h->ev_layer.clear();
  h->ev_bytes.clear();
  return SPD_OK;
}

// ---- the per-step plan -----------------------------------------------------------
int build_step(spd_handle* h, DescWriter& dw) {
  const Plan& p = h->p;
  h->ops.clear();
  h->pend_layers.clear();
  const int newest = h->F.back().pos;
  const int first = h->F.front().pos;
  const int dpos = newest + 1;
  const bool exited = h->F.front().stage == p.n - 1;
  const int ex_pos = first;
  const int v = ex_pos + 1;
  const int M = newest - h->pdm_len + 1;
  if (M < 1 || M > p.ring) return fail(h, SPD_E_STATE, "internal: PDM window out of range");
  float* hring = h->at<float>(p.o_h);
  float* anch = h->at<float>(p.o_anch);
  float* hp = h->at<float>(p.o_hp);
  float* X = h->at<float>(p.o_X);
  float* qbuf = h->at<float>(p.o_qbuf);
  float* attn = h->at<float>(p.o_attn);
  float* lqkv = h->at<float>(p.o_lqkv);
  float* act = h->at<float>(p.o_act);
  float* logits = h->at<float>(p.o_logits);
  float* qring = h->at<float>(p.o_qring);
  float* qlse = h->at<float>(p.o_qlse);
  const int kd = p.k * p.d;
  auto push_gemv = [&](int kind, std::vector<GemvProb>& g, int stream) {
    if (g.empty()) return;
    const GemvPlan plan = finish_tiles(p, g);
    Op op{kind, dw.put(g.data(), (int)g.size()), (int)g.size(), plan.ntiles, 0,
          gemv_bytes(g, p.esz)};
    op.stream = stream;
    op.plan = plan;
    h->ops.push_back(op);
  };
  auto push_attn = [&](int kind, std::vector<AttnProb>& a, int stream, int slot0, double kvb) {
    if (a.empty()) return;
    const int split = attn_split(p, a);
    const int nt = finish_attn(p, a, split, slot0);
    Op op{kind, dw.put(a.data(), (int)a.size()), (int)a.size(), nt, split, kvb};
    op.stream = stream;
    for (const AttnProb& x : a)
      if (x.side_k && x.self_row >= 0) op.adopt = 1;
    h->ops.push_back(op);
  };

  // 1. embedding + PDM feature gather, on the caller's stream (it must precede the
  //    target's first writes to the residual and anchor rings)
  // a token enters stage 0 every step, except right after a sibling's adoption (then the
  // newest token is the adopted one, in its last stage)
  const bool fresh = h->F.back().stage == 0;
  EmbedGather eg{};
  eg.embed = h->embed;
  eg.tok_ring = h->at<int>(p.o_tok);
  eg.h_ring = hring;
  eg.anchors = anch;
  eg.X = X;
  eg.newest_slot = h->row(newest);
  eg.embed_new = fresh ? 1 : 0;
  eg.embed_w = h->F.back().w;
  eg.d = p.d; eg.k = p.k; eg.M = M;
  if (h->adopt) {
    // the adopted sibling's rows move in this launch; the gather reads them where they are
    eg.adopt_layers = h->adopt_layers;
    eg.adopt_from = h->row(h->adopt_pos) + h->adopt_idx;
    eg.adopt_to = h->row(h->adopt_pos);
    eg.adopt_pos = h->adopt_pos;
    eg.adopt_side_row = h->slot(h->adopt_pos) * (p.W - 1) + h->adopt_idx - 1;
    eg.kv_base = h->ws + p.o_kv;
    eg.side_base = h->ws + p.o_side;
    eg.kv_layer_bytes = p.kv_layer_bytes;
    eg.side_layer_bytes = p.side_layer_bytes;
    eg.hkv = p.hkv; eg.hd = p.hd; eg.max_ctx = p.max_ctx; eg.side_rows = p.side_rows;
    eg.kv_bf16 = p.kv_bf16 ? 1 : 0;
  }
  const bool out_states = p.spec_output != 0;
  for (int r = 0; r < M; ++r) {
    const int x = h->pdm_len + r;
    eg.row_slot[r] = h->row(x) + (h->adopt && x == h->adopt_pos ? h->adopt_idx : 0);
    // the row's depth when the PDM reads it: at the step's start, or (output states)
    // after its stage's layers
    int depth = p.L;
    if (x >= first) {
      const int st = h->F[x - first].stage;
      depth = p.starts[st] + (out_states ? p.sizes[st] : 0);
    }
    int deepest = 0;
    for (int i = 0; i < p.k; ++i)
      if (p.anchors[i] <= depth) deepest = i;
    for (int i = 0; i < p.k; ++i) {
      int src;
      if (p.anchors[i] <= depth) src = i;
      else src = p.fill == SPD_FILL_CLAMP ? deepest : -1;
      // the newest g0 is embedded in this launch (input states); after the target layers
      // it is read from its anchor slot like any other
      if (!out_states && fresh && x == newest && src == 0) src = -2;
      eg.src[r][i] = (signed char)src;
    }
  }
  // the PDM chain: on its own stream beside the target (input states), or after the
  // target's layers on the caller's stream (output states)
  const int pdm_stream = out_states ? 0 : 1;
  size_t gather_off = 0;
  if (out_states) {
    EmbedGather e0 = eg;
    e0.M = 0;
    h->ops.push_back({OP_EMBED, dw.put(&e0, 1), 0, 0, 0, 0.0});
    eg.embed_new = 0;
    gather_off = dw.put(&eg, 1);
  } else {
    Op op{OP_EMBED, dw.put(&eg, 1), M, 0, 0, 0.0};
    op.adopt = eg.adopt_layers;
    h->ops.push_back(op);
    h->ops.push_back({OP_FORK, 0, 0, 0, 0, 0.0});
  }
  // 3. target sub-layers on the caller's stream: every in-flight token at layer
  //    start(stage) + r, all stages in one launch per sub-layer op (output states: before
  //    the PDM chain, which then reads what they produced)
  const int n_inf = (int)h->F.size();
  auto target_rounds = [&]() {
    const int R = *std::max_element(p.sizes.begin(), p.sizes.end());
    for (int r = 0; r < R; ++r) {
      std::vector<GemvProb> qkv, o, gu, down;
      std::vector<AttnProb> at;
      std::vector<LinProb> lin;
      double kvb = 0, linb = 0;
      const size_t first_op = h->ops.size();
      int round_layer = -1, round_tokens = 0;
      for (int j = 0; j < n_inf; ++j) {
        const Inflight f = h->F[j];
        if (p.sizes[f.stage] <= r) continue;
        const int l = p.starts[f.stage] + r;
        const int s = h->row(f.pos);       // ring row of the position's token
        const int w = f.w;                 // its candidates: rows s .. s + w - 1
        const int jr = j * p.W;            // their decode rows
        float* hv = hring + (size_t)s * p.d;
        round_layer = l;
        ++round_tokens;
        if (p.kind[l] == SPD_LAYER_LINEAR) {
          // q, k, v to the token's scratch row, then the recurrent step from the state
          // after pos - 1 to the state after pos
          float* lrow = lqkv + (size_t)j * p.linrows;
          qkv.push_back(gemv(h->W(l, T_QKV), p.linrows, p.d, hv, 0, 1, EPI_STORE, lrow, 0,
                             (const float*)h->W(l, T_ATTN_NORM), 0, p.eps));
          LinProb lp{};
          lp.qkv = lrow; lp.out = attn + (size_t)jr * p.qo;
          lp.s_prev = h->lin(l, h->slot(f.pos - 1)); lp.s_next = h->lin(l, h->slot(f.pos));
          lin.push_back(lp);
          linb += 2.0 * p.lin_state_bytes;
        } else {
          // the candidates of one position: one problem of w vectors at the same position;
          // the siblings' keys and values go to their side rows
          GemvProb q = gemv(h->W(l, T_QKV), p.qrows, p.d, hv, p.d, w, EPI_QKV, nullptr, 0,
                            (const float*)h->W(l, T_ATTN_NORM), 0, p.eps);
          q.aux = qbuf + (size_t)jr * p.qo; q.aux_stride = p.qo;
          q.kv_k = h->kvK(l); q.kv_v = h->kvV(l); q.kv_f32 = !p.kv_bf16;
          q.pos0 = f.pos; q.hq = p.hq; q.hkv = p.hkv; q.hd = p.hd; q.max_ctx = p.max_ctx;
          q.same_pos = 1;
          if (w > 1) {
            q.side_k = h->sideK(l); q.side_v = h->sideV(l);
            q.side_row0 = h->slot(f.pos) * (p.W - 1); q.side_rows = p.side_rows;
          }
          qkv.push_back(q);
          for (int b = 0; b < w; ++b) {
            AttnProb a{};
            a.q = qbuf + (size_t)(jr + b) * p.qo; a.out = attn + (size_t)(jr + b) * p.qo;
            a.q_stride = p.qo; a.out_stride = p.qo; a.nrows = 1;
            a.K = h->kvK(l); a.V = h->kvV(l); a.len = f.pos + 1;
            a.self_row = -1;
            if (b > 0) {   // a sibling: its own key from its side row
              a.self_row = h->slot(f.pos) * (p.W - 1) + b - 1;
              a.side_k = h->sideK(l); a.side_v = h->sideV(l); a.side_rows = p.side_rows;
            }
            at.push_back(a);
          }
          kvb += 2.0 * (f.pos + 1) * p.hkv * p.hd * p.kv_esz;
        }
        o.push_back(gemv(h->W(l, T_O), p.d, p.qo, attn + (size_t)jr * p.qo, p.qo, w, EPI_ADD, hv,
                         p.d, nullptr, 0, 0.f));
        GemvProb g = gemv(h->W(l, T_GATE), p.F, p.d, hv, p.d, w, EPI_SWIGLU, act + (size_t)jr * p.F,
                          p.F, (const float*)h->W(l, T_FFN_NORM), 0, p.eps);
        g.W2 = h->W(l, T_UP);
        gu.push_back(g);
        GemvProb dn = gemv(h->W(l, T_DOWN), p.d, p.F, act + (size_t)jr * p.F, p.F, w, EPI_ADD, hv,
                           p.d, nullptr, 0, 0.f);
        for (int i = 0; i < p.k; ++i)
          if (p.anchors[i] == l + 1) {
            dn.aux = anch + ((size_t)s * p.k + i) * p.d;
            dn.aux_stride = kd;
          }
        down.push_back(dn);
        h->pend_layers.push_back({l, f.pos});
      }
      push_gemv(OP_GEMV_QKV, qkv, 0);
      push_attn(OP_ATTN, at, 0, 0, kvb);
      if (!lin.empty()) {
        Op op{OP_LIN, dw.put(lin.data(), (int)lin.size()), (int)lin.size(), (int)lin.size() * p.hq,
              0, linb};
        h->ops.push_back(op);
      }
      push_gemv(OP_GEMV_O, o, 0);
      push_gemv(OP_GEMV_GU, gu, 0);
      push_gemv(OP_GEMV_DOWN, down, 0);
      if (round_tokens == 1)   // these launches serve one layer alone: its per-layer time
        for (size_t i = first_op; i < h->ops.size(); ++i)
          if (h->ops[i].stream == 0) h->ops[i].layer = round_layer;
    }
  };
  if (out_states) {
    target_rounds();
    h->ops.push_back({OP_GATHER, gather_off, M, 0, 0, 0.0});
  }

  // 2. the PDM chain: projection of the gathered features, then Ls decoder layers over
  //    the M window rows (decode rows n .. n + M - 1)
  {
    std::vector<GemvProb> g{gemv(h->proj, p.d, kd, X, kd, M, EPI_STORE, hp, p.d, nullptr, 0, 0.f)};
    push_gemv(OP_GEMV_PROJ, g, pdm_stream);
  }
  const int base = p.n * p.W;
  for (int r = 0; r < p.Ls; ++r) {
    const bool last = r == p.Ls - 1;
    std::vector<GemvProb> qkv, o, gu, down;
    std::vector<AttnProb> at;
    GemvProb q = gemv(h->PW(r, T_QKV), p.qrows, p.d, hp, p.d, M, EPI_QKV, nullptr, 0,
                      (const float*)h->PW(r, T_ATTN_NORM), 0, p.eps);
    q.aux = qbuf + (size_t)base * p.qo; q.aux_stride = p.qo;
    q.kv_k = h->pK(r); q.kv_v = h->pV(r); q.kv_f32 = !p.kv_bf16;
    q.pos0 = h->pdm_len; q.hq = p.hq; q.hkv = p.hkv; q.hd = p.hd; q.max_ctx = p.max_ctx;
    qkv.push_back(q);
    // the last PDM layer only feeds the LM head: its attention, O and FFN run on the
    // newest row alone (its QKV still writes every row's keys and values)
    const int r0 = last ? M - 1 : 0, nr = last ? 1 : M;
    const int rpp = attn_rows_per_problem(p.kv_bf16, p.hq, p.hkv);
    for (int m = r0; m < M; m += rpp) {
      AttnProb a{};
      a.q = qbuf + (size_t)(base + m) * p.qo; a.out = attn + (size_t)(base + m) * p.qo;
      a.q_stride = p.qo; a.out_stride = p.qo;
      a.K = h->pK(r); a.V = h->pV(r); a.len = h->pdm_len + m + 1;
      a.nrows = std::min(rpp, M - m);
      at.push_back(a);
    }
    const double kvb = 2.0 * (h->pdm_len + M) * p.hkv * p.hd * p.kv_esz;
    float* hrow = hp + (size_t)r0 * p.d;
    o.push_back(gemv(h->PW(r, T_O), p.d, p.qo, attn + (size_t)(base + r0) * p.qo, p.qo, nr,
                     EPI_ADD, hrow, p.d, nullptr, 0, 0.f));
    GemvProb g = gemv(h->PW(r, T_GATE), p.F, p.d, hrow, p.d, nr, EPI_SWIGLU,
                      act + (size_t)(base + r0) * p.F, p.F, (const float*)h->PW(r, T_FFN_NORM), 0,
                      p.eps);
    g.W2 = h->PW(r, T_UP);
    gu.push_back(g);
    down.push_back(gemv(h->PW(r, T_DOWN), p.d, p.F, act + (size_t)(base + r0) * p.F, p.F, nr,
                        EPI_ADD, hrow, p.d, nullptr, 0, 0.f));
    push_gemv(OP_PDM_QKV, qkv, pdm_stream);
    push_attn(OP_PDM_ATTN, at, pdm_stream, base, kvb);
    push_gemv(OP_PDM_O, o, pdm_stream);
    push_gemv(OP_PDM_GU, gu, pdm_stream);
    push_gemv(OP_PDM_DOWN, down, pdm_stream);
  }

  if (!out_states) {
    target_rounds();
    h->ops.push_back({OP_JOIN, 0, 0, 0, 0, 0.0});
  }

  // 4. one sweep of the tied LM head: the exiting token's row and the PDM's newest row
  float* qnew = qring + (size_t)h->slot(dpos) * p.V;
  float* hnew = hp + (size_t)(M - 1) * p.d;
  {
    GemvProb g;
    if (exited) {
      float* hx = hring + (size_t)h->row(ex_pos) * p.d;
      g = gemv(h->head, p.V, p.d, hx, float_gap(hnew, hx), 2, EPI_STORE, logits,
               float_gap(qnew, logits), h->final_norm, float_gap(h->pdm_final_norm, h->final_norm),
               p.eps);
    } else {
      g = gemv(h->head, p.V, p.d, hnew, 0, 1, EPI_STORE, qnew, 0, h->pdm_final_norm, 0, p.eps);
    }
    std::vector<GemvProb> gv{g};
    push_gemv(OP_GEMV_HEAD, gv, 0);
  }
  const bool sampled = h->temp > 0.f;
  const float inv_t = sampled ? 1.f / h->temp : 1.f;
  VocabDesc vd{};
  vd.logits[0] = logits; vd.logits[1] = qnew;
  vd.active[0] = exited ? 1 : 0; vd.active[1] = 1;
  vd.gumbel_stream[1] = sampled ? RNG_DRAFT : 0;
  vd.gumbel_pos[1] = dpos;
  vd.V = p.V; vd.nblocks = kVocabBlocks; vd.inv_temp = inv_t; vd.sampled = sampled;
  vd.seed = h->seed;
  const bool nucleus = sampled && h->top_p < 1.f;
  NucleusCut* cuts = h->at<NucleusCut>(p.o_cut);
  vd.nucleus = nucleus; vd.top_p = h->top_p;
  vd.cut[0] = cuts; vd.cut[1] = cuts + 1 + h->slot(dpos);
  h->nucleus_scratch(vd);
  vd.topw = p.W;
  vd.top = h->at<VocabTop>(p.o_top);
  const size_t voff = dw.put(&vd, 1);
  h->ops.push_back({OP_VOCAB, voff, 1, kVocabBlocks, 0, 0.0});
  if (nucleus) h->ops.push_back({OP_NUCLEUS, voff, 1, kVocabBlocks, 0, 0.0});
  FinalizeDesc fd{};
  fd.mode = 0; fd.exited = exited; fd.single = n_inf == 1; fd.v = v; fd.dpos = dpos;
  fd.ring = p.ring; fd.V = p.V; fd.nblocks = kVocabBlocks; fd.temp = h->temp; fd.inv_temp = inv_t;
  fd.seed = h->seed; fd.forced_mode = h->forced_mode; fd.forced_p = h->forced_p;
  fd.forced_base = h->P0; fd.forced_len = (int)h->forced_ref.size();
  fd.forced_ref = h->at<int>(p.o_forced);
  fd.zt = logits;
  fd.zq_v = qring + (size_t)h->slot(v) * p.V;
  fd.lse_q_v = qlse + h->slot(v);
  fd.lse_q_new = qlse + h->slot(dpos);
  fd.tok_ring = h->at<int>(p.o_tok);
  fd.verdict = h->at<Verdict>(p.o_verdict);
  fd.host_verdict = h->d_hverdict;
  fd.part = h->at<VocabPartial>(p.o_part);
  fd.nucleus = nucleus;
  fd.cut_t = cuts; fd.cut_q = cuts + 1 + h->slot(dpos); fd.cut_q_v = cuts + 1 + h->slot(v);
  fd.W = p.W;
  fd.top = h->at<VocabTop>(p.o_top);
  // the rejection rounds keep p and q of the verified position in the top-p scratch, which
  // draft trees leave unused (they refuse top_p < 1)
  fd.pq = p.W > 1 ? h->at<float>(p.o_nuc) : nullptr;
  const size_t foff = dw.put(&fd, 1);
  h->ops.push_back({OP_FINAL, foff, 1, 1, 0, 0.0});
  if (sampled && exited) h->ops.push_back({OP_RESID, foff, 1, kVocabBlocks, 0, 0.0});
  h->pend_exit = exited;
  h->pend_v = v;
  h->pend_dpos = dpos;
  h->pend_newest = newest;
  return SPD_OK;
}

}  // namespace

// ======================================================================================
extern "C" {

size_t spd_workspace_bytes(const spd_model_config* cfg) {
  Plan p;
  std::string err;
  if (!plan_config(cfg, p, err)) return 0;
  return p.total;
}

const char* spd_init_error(void) { return g_init_error.c_str(); }

int spd_init(const spd_model_config* cfg, const spd_weights* w, const spd_sampling* s,
             void* d_workspace, size_t ws_bytes, void* hip_stream, spd_handle** out) {
  g_init_error.clear();
  if (!out) { g_init_error = "null out"; return SPD_E_ARG; }
  *out = nullptr;
  Plan p;
  std::string err;
  if (!cfg || !w || !s || !d_workspace) { g_init_error = "null argument"; return SPD_E_ARG; }
  if (!plan_config(cfg, p, err)) { g_init_error = err; return SPD_E_CONFIG; }
  if (ws_bytes < p.total) {
    g_init_error = "workspace too small: need " + std::to_string(p.total) + " bytes";
    return SPD_E_CAPACITY;
  }
  if (!(s->temperature >= 0.f)) { g_init_error = "temperature must be >= 0"; return SPD_E_ARG; }
  if (!(s->top_p > 0.f)) { g_init_error = "top_p must be > 0"; return SPD_E_ARG; }
  if (s->forced_mode && s->temperature != 0.f) {
    g_init_error = "forced mode needs temperature 0";
    return SPD_E_CONFIG;
  }
  if (p.W > 1 && (s->forced_mode || s->top_p < 1.f)) {
    g_init_error = "draft trees (draft_width > 1) need top_p >= 1 and forced_mode 0";
    return SPD_E_CONFIG;
  }
  if (s->forced_mode && (s->forced_ref_len < 0 || (s->forced_ref_len > 0 && !s->forced_ref))) {
    g_init_error = "forced mode needs forced_ref";
    return SPD_E_ARG;
  }
  if (!w->embed || !w->lm_head || !w->final_norm || !w->layers || !w->pdm_proj ||
      !w->pdm_layers || !w->pdm_final_norm) {
    g_init_error = "null weight pointer";
    return SPD_E_ARG;
  }
  spd_handle* h = new spd_handle();
  h->p = p;
  h->embed = w->embed; h->head = w->lm_head; h->final_norm = w->final_norm;
  h->proj = w->pdm_proj; h->pdm_final_norm = w->pdm_final_norm;
  h->lw.assign(w->layers, w->layers + (size_t)p.L * kTensorsPerLayer);
  h->pw.assign(w->pdm_layers, w->pdm_layers + (size_t)p.Ls * kTensorsPerLayer);
  for (auto ptr : h->lw)
    if (!ptr) { g_init_error = "null layer weight"; delete h; return SPD_E_ARG; }
  for (auto ptr : h->pw)
    if (!ptr) { g_init_error = "null PDM layer weight"; delete h; return SPD_E_ARG; }
  h->temp = s->temperature; h->top_p = s->top_p; h->seed = s->seed;
  h->forced_mode = s->forced_mode; h->forced_p = s->forced_p;
  if (s->forced_mode && s->forced_ref_len > 0) {
    for (int i = 0; i < s->forced_ref_len; ++i)
      if (s->forced_ref[i] < 0 || s->forced_ref[i] >= p.V) {
        g_init_error = "forced_ref id out of range [0, vocab)";
        delete h;
        return SPD_E_ARG;
      }
    h->forced_ref.assign(s->forced_ref, s->forced_ref + s->forced_ref_len);
  }
  if ((int)h->forced_ref.size() > p.max_ctx) h->forced_ref.resize(p.max_ctx);
  h->ws = static_cast<char*>(d_workspace);
  h->st = static_cast<hipStream_t>(hip_stream);
  h->kv_len.assign(p.L, 0);
  auto dev_fail = [&](hipError_t e, const char* what) {
    g_init_error = std::string(what) + ": " + hipGetErrorString(e);
    if (h->h_desc_base) (void)hipHostFree(h->h_desc_base);
    if (h->h_verdict_base) (void)hipHostFree(h->h_verdict_base);
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    if (h->ev_join) (void)hipEventDestroy(h->ev_join);
    for (hipEvent_t ev : h->ev_step)
      if (ev) (void)hipEventDestroy(ev);
    if (h->st2) (void)hipStreamDestroy(h->st2);
    delete h;
    return SPD_E_DEVICE;
  };
  hipError_t e;
  if ((e = hipHostMalloc((void**)&h->h_desc_base, 2 * kDescBytes, hipHostMallocDefault)) != hipSuccess)
    return dev_fail(e, "hipHostMalloc");
  if ((e = hipHostGetDevicePointer((void**)&h->d_hdesc_base, h->h_desc_base, 0)) != hipSuccess)
    return dev_fail(e, "hipHostGetDevicePointer");
  if ((e = hipHostMalloc((void**)&h->h_verdict_base, 2 * sizeof(Verdict), hipHostMallocDefault)) != hipSuccess)
    return dev_fail(e, "hipHostMalloc");
  if ((e = hipHostGetDevicePointer((void**)&h->d_hverdict_base, h->h_verdict_base, 0)) != hipSuccess)
    return dev_fail(e, "hipHostGetDevicePointer");
  use_desc_buf(h, 0);
  for (hipEvent_t& ev : h->ev_step)
    if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess)
      return dev_fail(e, "hipEventCreateWithFlags");
  // the PDM stream (default priority) and the events that fork and join it each step
  if ((e = hipStreamCreateWithFlags(&h->st2, hipStreamNonBlocking)) != hipSuccess)
    return dev_fail(e, "hipStreamCreateWithFlags");
  if ((e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming)) != hipSuccess)
    return dev_fail(e, "hipEventCreateWithFlags");
  if ((e = hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming)) != hipSuccess)
    return dev_fail(e, "hipEventCreateWithFlags");
  // the static scratch of this device (spd_prefill_static_scratch); a failed lookup only
  // disables that entry point
  h->scratch = scratch_of_current_device(h->scratch_err);
  std::vector<float2> rope;
  fill_rope(p, rope);
  if ((e = hipMemcpyAsync(h->ws + p.o_rope, rope.data(), rope.size() * sizeof(float2),
                          hipMemcpyHostToDevice, h->st)) != hipSuccess)
    return dev_fail(e, "hipMemcpyAsync(rope)");
  // KV caches start zeroed: attention reads whole 32-key blocks, and the unwritten tail of
  // the last one must hold finite values (its scores are masked, its values weigh 0)
  if ((e = hipMemsetAsync(h->ws + p.o_kv, 0, (size_t)p.nsoft * p.kv_layer_bytes, h->st)) != hipSuccess ||
      (e = hipMemsetAsync(h->ws + p.o_pkv, 0, (size_t)p.Ls * p.kv_layer_bytes, h->st)) != hipSuccess ||
      (e = hipMemsetAsync(h->ws + p.o_cut, 0, (size_t)(1 + p.ring) * sizeof(NucleusCut), h->st)) != hipSuccess)
    return dev_fail(e, "hipMemsetAsync(kv)");
  if ((e = hipStreamSynchronize(h->st)) != hipSuccess) return dev_fail(e, "hipStreamSynchronize");
  *out = h;
  return SPD_OK;
}

}  // extern "C"

namespace {

// Activation buffers of the chunked prefill: CH rows each (the anchor buffer k x CH rows).
struct PrefillBufs {
  float *H, *A, *QKV, *O, *G, *U, *Z, *AN;
  int CH;
};

// Carves the chunk buffers for CH rows out of `base` (nullptr: only sizes them); returns
// the bytes used.
size_t carve_prefill(const Plan& p, char* base, int CH, PrefillBufs& b) {
  const size_t widest = std::max({(size_t)p.d, (size_t)p.qo, (size_t)p.F, (size_t)p.k * p.d});
  size_t o = 0;
  auto take = [&](size_t floats) {
    float* at = reinterpret_cast<float*>(base + o);
    o = align_up(o + floats * sizeof(float));
    return at;
  };
  b.CH = CH;
  b.H = take((size_t)CH * p.d);
  b.A = take((size_t)CH * widest);
  b.QKV = take((size_t)CH * std::max(p.qrows, p.linrows));
  b.O = take((size_t)CH * p.qo);
  b.G = take((size_t)CH * p.F);
  b.U = take((size_t)CH * p.F);
  b.Z = take((size_t)CH * p.d);
  b.AN = take((size_t)p.k * CH * p.d);
  return o;
}

int prefill_impl(spd_handle* h, const int32_t* prompt, int32_t len, int32_t* first_token,
                 const PrefillBufs& bufs);

}  // namespace

extern "C" {

int spd_prefill(spd_handle* h, const int32_t* prompt, int32_t len, int32_t* first_token) {
  if (!h) return SPD_E_ARG;
  PrefillBufs b{};
  b.CH = kPrefillChunk;
  b.H = h->at<float>(h->p.o_pH);
  b.A = h->at<float>(h->p.o_pA);
  b.QKV = h->at<float>(h->p.o_pQKV);
  b.O = h->at<float>(h->p.o_pO);
  b.G = h->at<float>(h->p.o_pG);
  b.U = h->at<float>(h->p.o_pU);
  b.Z = h->at<float>(h->p.o_pZ);
  b.AN = h->at<float>(h->p.o_panch);
  return prefill_impl(h, prompt, len, first_token, b);
}

int spd_prefill_static_scratch(spd_handle* h, const int32_t* prompt, int32_t len,
                               int32_t* first_token) {
  if (!h) return SPD_E_ARG;
  h->err.clear();
  if (!h->scratch) return fail(h, SPD_E_DEVICE, "static scratch unavailable: " + h->scratch_err);
  // as many prompt rows per chunk as the array holds (at most the regular chunk)
  PrefillBufs b{};
  int CH = kPrefillChunk;
  while (CH > 0 && carve_prefill(h->p, nullptr, CH, b) > kStaticScratchBytes) CH -= 16;
  if (CH <= 0) {
    const size_t need = carve_prefill(h->p, nullptr, 16, b);
    return fail(h, SPD_E_CAPACITY,
                "the model is too wide for the static prefill scratch: 16 prompt rows need " +
                    std::to_string(need) + " bytes, the array holds " +
                    std::to_string(kStaticScratchBytes));
  }
  carve_prefill(h->p, h->scratch, CH, b);
  return prefill_impl(h, prompt, len, first_token, b);
}

}  // extern "C"

namespace {

int prefill_impl(spd_handle* h, const int32_t* prompt, int32_t len, int32_t* first_token,
                 const PrefillBufs& bufs) {
  h->err.clear();
  if (h->state != spd_handle::S_INIT) return fail(h, SPD_E_STATE, "already prefilled (spd_reset first)");
  if (!prompt || len < 1) return fail(h, SPD_E_ARG, "empty prompt");
  const Plan& p = h->p;
  if (len >= p.max_ctx) return fail(h, SPD_E_CAPACITY, "prompt does not fit max_ctx");
  for (int i = 0; i < len; ++i)
    if (prompt[i] < 0 || prompt[i] >= p.V) return fail(h, SPD_E_ARG, "token id out of range");
  hipStream_t st = h->st;
  int* toks = h->at<int>(p.o_ptok);
  // The prompt and the forced reference go to the device through the pinned staging block,
  // one block's worth at a time (no step is in flight before a prefill, so the block is free)
  auto upload = [&](void* dst, const int32_t* src, size_t count) -> int {
    const size_t per = kDescBytes / sizeof(int32_t);
    for (size_t i = 0; i < count; i += per) {
      const size_t c = std::min(per, count - i);
      std::memcpy(h->h_desc, src + i, c * sizeof(int32_t));
      HIPCHK(h, hipMemcpyAsync(static_cast<char*>(dst) + i * sizeof(int32_t), h->h_desc,
                               c * sizeof(int32_t), hipMemcpyHostToDevice, st));
      HIPCHK(h, hipStreamSynchronize(st));
    }
    return SPD_OK;
  };
  int urc = upload(toks, prompt, (size_t)len);
  if (urc == SPD_OK && !h->forced_ref.empty())
    urc = upload(h->ws + p.o_forced, h->forced_ref.data(), h->forced_ref.size());
  if (urc != SPD_OK) return urc;
  const bool bf = p.bf16;
  float* H = bufs.H;
  float* A = bufs.A;
  float* QKV = bufs.QKV;
  float* O = bufs.O;
  float* Gb = bufs.G;
  float* Ub = bufs.U;
  float* Z = bufs.Z;
  float* AN = bufs.AN;
  const float2* rope = h->at<float2>(p.o_rope);
  const int CH = bufs.CH;
  const int kd = p.k * p.d;
  // one decoder layer over P rows of the residual Rb (fp32 activations throughout)
  // lin_l >= 0: a linear-attention target layer (its state ring), else a softmax layer
  auto layer = [&](float* Rb, int P, int pos0, const void* const* wt, void* Kc, void* Vc,
                   int lin_l = -1) -> int {
    HIPCHK(h, launch_rmsnorm_rows(Rb, p.d, (const float*)wt[T_ATTN_NORM], A, p.d, P, p.d, p.eps, false, st));
    if (lin_l >= 0) {
      // the state after the previous chunk to the state after this chunk's last row
      HIPCHK(h, launch_gemm(A, p.d, wt[T_QKV], QKV, p.linrows, P, p.linrows, p.d, false, bf, st));
      const float* s_in = pos0 > 0 ? h->lin(lin_l, h->slot(pos0 - 1)) : nullptr;
      HIPCHK(h, launch_linear_scan(QKV, p.linrows, O, p.qo, s_in, h->lin(lin_l, h->slot(pos0 + P - 1)),
                                   P, p.hq, p.hd, kLinEps, st));
    } else {
      HIPCHK(h, launch_gemm(A, p.d, wt[T_QKV], QKV, p.qrows, P, p.qrows, p.d, false, bf, st));
      HIPCHK(h, launch_rope_kv(QKV, p.qrows, Kc, Vc, rope, pos0, P, p.hq, p.hkv, p.hd, p.max_ctx,
                               p.kv_bf16, st));
      HIPCHK(h, launch_attention_prefill(QKV, p.qrows, O, p.qo, Kc, Vc, pos0, P, p.kv_bf16, p.hq, p.hkv,
                                         p.hd, p.max_ctx, st));
    }
    HIPCHK(h, launch_gemm(O, p.qo, wt[T_O], Rb, p.d, P, p.d, p.qo, true, bf, st));
    HIPCHK(h, launch_rmsnorm_rows(Rb, p.d, (const float*)wt[T_FFN_NORM], A, p.d, P, p.d, p.eps, false, st));
    HIPCHK(h, launch_gemm(A, p.d, wt[T_GATE], Gb, p.F, P, p.F, p.d, false, bf, st));
    HIPCHK(h, launch_gemm(A, p.d, wt[T_UP], Ub, p.F, P, p.F, p.d, false, bf, st));
    HIPCHK(h, launch_swiglu_rows(Gb, Ub, p.F, A, p.F, P, p.F, false, st));
    HIPCHK(h, launch_gemm(A, p.F, wt[T_DOWN], Rb, p.d, P, p.d, p.F, true, bf, st));
    return SPD_OK;
  };
  for (int c0 = 0; c0 < len; c0 += CH) {
    const int P = std::min(CH, len - c0);
    HIPCHK(h, launch_embed_rows(h->embed, toks + c0, H, P, p.d, bf, st));
    HIPCHK(h, launch_copy_rows(H, p.d, AN, p.d, P, p.d, st));   // anchor 0: the embedding
    for (int l = 0; l < p.L; ++l) {
      const bool lin = p.kind[l] == SPD_LAYER_LINEAR;
      const int rc = layer(H, P, c0, &h->lw[(size_t)l * kTensorsPerLayer], lin ? nullptr : h->kvK(l),
                           lin ? nullptr : h->kvV(l), lin ? l : -1);
      if (rc != SPD_OK) return rc;
      for (int i = 1; i < p.k; ++i)
        if (p.anchors[i] == l + 1)
          HIPCHK(h, launch_copy_rows(H, p.d, AN + (size_t)i * CH * p.d, p.d, P, p.d, st));
    }
    // the verified prefix's depth-maximised PDM features: every anchor, concatenated
    for (int i = 0; i < p.k; ++i)
      HIPCHK(h, launch_copy_rows(AN + (size_t)i * CH * p.d, p.d, A + (size_t)i * p.d, kd, P, p.d, st));
    HIPCHK(h, launch_gemm(A, kd, h->proj, Z, p.d, P, p.d, kd, false, bf, st));
    for (int r = 0; r < p.Ls; ++r) {
      const int rc = layer(Z, P, c0, &h->pw[(size_t)r * kTensorsPerLayer], h->pK(r), h->pV(r));
      if (rc != SPD_OK) return rc;
    }
    if (c0 + P == len) {
      // first token from the last prompt row (fp32 input to the head, as in decode)
      DescWriter dw{h->h_desc};
      std::vector<GemvProb> g{gemv(h->head, p.V, p.d, H + (size_t)(P - 1) * p.d, 0, 1, EPI_STORE,
                                   h->at<float>(p.o_logits), 0, h->final_norm, 0, p.eps)};
      const GemvPlan plan = finish_tiles(p, g);
      const size_t go = dw.put(g.data(), 1);
      const bool sampled = h->temp > 0.f;
      VocabDesc vd{};
      vd.logits[0] = h->at<float>(p.o_logits); vd.logits[1] = nullptr;
      vd.active[0] = 1; vd.active[1] = 0;
      vd.gumbel_stream[0] = sampled ? RNG_FIRST : 0; vd.gumbel_pos[0] = len;
      vd.V = p.V; vd.nblocks = kVocabBlocks; vd.inv_temp = sampled ? 1.f / h->temp : 1.f;
      vd.sampled = sampled; vd.seed = h->seed;
      const bool nucleus = sampled && h->top_p < 1.f;
      vd.nucleus = nucleus; vd.top_p = h->top_p;
      vd.cut[0] = h->at<NucleusCut>(p.o_cut);
      h->nucleus_scratch(vd);
      const size_t vo = dw.put(&vd, 1);
      FinalizeDesc fd{};
      fd.mode = 1; fd.dpos = len; fd.ring = p.ring; fd.V = p.V; fd.nblocks = kVocabBlocks;
      fd.W = p.W;
      fd.temp = h->temp; fd.inv_temp = vd.inv_temp; fd.seed = h->seed;
      fd.tok_ring = h->at<int>(p.o_tok); fd.verdict = h->at<Verdict>(p.o_verdict);
      fd.host_verdict = h->d_hverdict;
      fd.part = h->at<VocabPartial>(p.o_part);
      fd.nucleus = nucleus; fd.cut_t = vd.cut[0];
      const size_t fo = dw.put(&fd, 1);
      char* d = h->ws + p.o_desc;
      HIPCHK(h, hipMemcpyAsync(d, h->h_desc, dw.used, hipMemcpyHostToDevice, st));
      HIPCHK(h, launch_gemv(GEMV_HEAD, reinterpret_cast<const GemvProb*>(d + go), 1, plan, bf, rope, st));
      HIPCHK(h, launch_vocab_stats(reinterpret_cast<const VocabDesc*>(d + vo), kVocabBlocks,
                                   h->at<VocabPartial>(p.o_part), st));
      if (nucleus)
        HIPCHK(h, launch_nucleus(reinterpret_cast<const VocabDesc*>(d + vo), kVocabBlocks,
                                 h->at<VocabPartial>(p.o_part), st));
      HIPCHK(h, launch_finalize(reinterpret_cast<const FinalizeDesc*>(d + fo), st));
      // the exiting-row residual of the last prompt position (debug view)
      HIPCHK(h, launch_copy_rows(H + (size_t)(P - 1) * p.d, p.d, h->at<float>(p.o_h) +
                                 (size_t)h->row(len - 1) * p.d, p.d, 1, p.d, st));
    }
  }
  HIPCHK(h, hipStreamSynchronize(st));
  const int t0 = h->h_verdict_base[h->cur_buf].first_token;
  if (first_token) *first_token = t0;
  h->P0 = len;
  h->F.clear();
  h->F.push_back({len, 0, 1});
  h->adopt = false;
  h->pdm_len = len;
  std::fill(h->kv_len.begin(), h->kv_len.end(), len);
  h->N = h->K = h->acc = h->rej = 0;
  h->state = spd_handle::S_READY;
  return SPD_OK;
}

}  // namespace

extern "C" {

// The host issues launches one at a time, so the order of the two streams' work in the
// op list is the order in which each stream receives it. build_step lists the whole PDM
// chain before the target's sub-layers; interleave them so neither stream waits behind
// the other's launches (each stream keeps its own order).
void interleave_streams(std::vector<Op>& ops) {
  auto f = std::find_if(ops.begin(), ops.end(), [](const Op& o) { return o.kind == OP_FORK; });
  auto j = std::find_if(ops.begin(), ops.end(), [](const Op& o) { return o.kind == OP_JOIN; });
  if (f == ops.end() || j == ops.end() || j < f) return;
  std::vector<Op> side, main;
  for (auto it = f + 1; it != j; ++it) (it->stream ? side : main).push_back(*it);
  auto out = f + 1;
  size_t a = 0, b = 0;
  while (a < main.size() || b < side.size()) {
    if (a < main.size()) *out++ = main[a++];
    if (b < side.size()) *out++ = side[b++];
  }
}

bool same_inflight(const std::deque<Inflight>& a, const std::deque<Inflight>& b) {
  if (a.size() != b.size()) return false;
  for (size_t i = 0; i < a.size(); ++i)
    if (a[i].pos != b[i].pos || a[i].stage != b[i].stage || a[i].w != b[i].w) return false;
  return true;
}

// Builds the step that will follow the pending one when the pending one verifies nothing
// (a refill step): verify_commit then only advances every stage and appends the draft, so
// the next state is known now. The pending step's bookkeeping is left as it was.
void prebuild_next(spd_handle* h) {
  const Plan& p = h->p;
  h->pre_valid = false;
  if (h->pend_exit) return;
  std::deque<Inflight> F2 = h->F;
  for (auto& f : F2) f.stage += 1;
  F2.push_back({h->pend_dpos, 0, p.W});
  if (F2.back().pos >= p.max_ctx || F2.front().stage >= p.n) return;
  const int pdm2 = std::max(h->pdm_len, h->F.front().pos);
  // save the pending step's state
  std::deque<Inflight> F0 = h->F;
  const int pdm0 = h->pdm_len;
  std::vector<Op> ops0;
  ops0.swap(h->ops);
  std::vector<std::pair<int, int>> layers0;
  layers0.swap(h->pend_layers);
  const bool ex0 = h->pend_exit;
  const int v0 = h->pend_v, d0 = h->pend_dpos, n0 = h->pend_newest;
  const int buf0 = h->cur_buf;
  const std::string err0 = h->err;
  // build for the predicted state into the block the next step uses
  h->F = F2;
  h->pdm_len = pdm2;
  use_desc_buf(h, h->next_buf);
  DescWriter dw{h->h_desc};
  const int rc = build_step(h, dw);
  if (rc == SPD_OK && dw.used <= kDescBytes && !h->ops.empty() && h->ops.front().kind == OP_EMBED) {
    interleave_streams(h->ops);
    h->pre_ops.swap(h->ops);
    h->pre_layers.swap(h->pend_layers);
    h->pre_exit = h->pend_exit;
    h->pre_v = h->pend_v; h->pre_dpos = h->pend_dpos; h->pre_newest = h->pend_newest;
    h->pre_used = dw.used;
    h->pre_F = F2;
    h->pre_pdm_len = pdm2;
    h->pre_valid = true;
  }
  // restore
  h->F = F0;
  h->pdm_len = pdm0;
  h->ops.swap(ops0);
  h->pend_layers.swap(layers0);
  h->pend_exit = ex0;
  h->pend_v = v0; h->pend_dpos = d0; h->pend_newest = n0;
  use_desc_buf(h, buf0);
  h->err = err0;
}

// The prebuilt step becomes the pending one.
void take_prebuilt(spd_handle* h) {
  h->ops.swap(h->pre_ops);
  h->pend_layers.swap(h->pre_layers);
  h->pend_exit = h->pre_exit;
  h->pend_v = h->pre_v; h->pend_dpos = h->pre_dpos; h->pend_newest = h->pre_newest;
  h->desc_used = h->pre_used;
  h->pre_valid = false;
}

int spd_step(spd_handle* h) {
  if (!h) return SPD_E_ARG;
  h->err.clear();
  if (h->state != spd_handle::S_READY)
    return fail(h, SPD_E_STATE, h->state == spd_handle::S_INIT ? "no prefill" : "a step is pending");
  const int newest = h->F.back().pos;
  if (newest >= h->p.max_ctx) return fail(h, SPD_E_CAPACITY, "newest position reached max_ctx");
  const bool pre_ok = h->pre_valid && !h->adopt && h->pre_pdm_len == h->pdm_len &&
                      same_inflight(h->pre_F, h->F);
  if (h->ahead) {
    // launched while the previous step ran (that step verified nothing, so this state was
    // fixed at its launch)
    if (!pre_ok) return fail(h, SPD_E_STATE, "internal: the step launched ahead does not match");
    take_prebuilt(h);
    h->pend_buf = h->pre_buf;
    h->ahead = false;
  } else {
    const int b = h->next_buf;
    if (pre_ok) {
      // built while the previous step ran, for exactly this state
      take_prebuilt(h);
    } else {
      use_desc_buf(h, b);
      DescWriter dw{h->h_desc};
      int rc = build_step(h, dw);
      if (rc != SPD_OK) return rc;
      h->adopt = false;   // the embedding launch of this step moves the adopted sibling
      interleave_streams(h->ops);
      if (dw.used > kDescBytes) return fail(h, SPD_E_CAPACITY, "internal: descriptor block overflow");
      if (h->ops.empty() || h->ops.front().kind != OP_EMBED)
        return fail(h, SPD_E_STATE, "internal: a step must start with the embedding");
      h->desc_used = dw.used;   // uploaded by the embedding kernel
    }
    h->pre_valid = false;
    const int rc = run_ops(h, h->ops, b, h->desc_used);
    if (rc != SPD_OK) return rc;
    h->pend_buf = b;
    h->next_buf = b ^ 1;
  }
  h->state = spd_handle::S_PENDING;
  // the other block is free: the step that used it last has been verified
  prebuild_next(h);
  if (h->lookahead && !h->timing && h->pre_valid) {
    const int rc = run_ops(h, h->pre_ops, h->next_buf, h->pre_used);
    if (rc != SPD_OK) return rc;
    h->pre_buf = h->next_buf;
    h->next_buf ^= 1;
    h->ahead = true;
    use_desc_buf(h, h->pend_buf);
  }
  return SPD_OK;
}

int spd_verify_commit(spd_handle* h, spd_commit* out) {
  if (!h) return SPD_E_ARG;
  h->err.clear();
  if (h->state != spd_handle::S_PENDING) return fail(h, SPD_E_STATE, "no pending step");
  // The verdict kernels wrote their result straight to pinned host memory (this step's
  // block's slot); poll the step's end event rather than block on it, so the host sees the
  // end of the step at once (the PDM stream was joined into the caller's before the head;
  // a step launched ahead may still be running behind it).
  hipError_t qe;
  while ((qe = hipEventQuery(h->ev_step[h->pend_buf])) == hipErrorNotReady) {
  }
  HIPCHK(h, qe);
  if (h->timing) {
    const int rc = collect_timing(h);
    if (rc != SPD_OK) return rc;
  }
  const Verdict vd = h->h_verdict_base[h->pend_buf];
  const Plan& p = h->p;
  h->K += 1;
  for (auto& lp : h->pend_layers) h->kv_len[lp.first] = lp.second + 1;
  // rows whose depth is L are final: those before the oldest in flight, and (output
  // states) the exiting one, whose row the PDM read at depth L in this step
  h->pdm_len = std::max(h->pdm_len, h->F.front().pos + (p.spec_output && h->pend_exit ? 1 : 0));
  for (auto& f : h->F) f.stage += 1;
  spd_commit c{};
  c.newest = h->pend_newest;
  c.new_draft = vd.draft;
  c.flags = vd.flags;
  c.accepted_index = -1;
  if (h->pend_exit) {
    const int v = h->pend_v;
    // the exiting token alone: the candidates at v were this step's drafts, none of which
    // has entered the pipeline
    const bool single = h->F.size() == 1;
    h->N += 1;
    c.verified = 1;
    c.position = v;
    c.token = vd.committed;
    c.accepted = vd.accepted;
    c.accepted_index = vd.accepted ? vd.accepted_index : -1;
    c.draft_token = vd.verified_draft;
    if (vd.accepted && (vd.accepted_index <= 0 || single)) {
      // the first candidate at v is the token there (or v holds this step's drafts): the
      // pipeline shifts, and v's other candidates are dropped
      h->acc += 1;
      h->F.pop_front();
      if (!h->F.empty()) h->F.front().w = 1;
      h->F.push_back({h->pend_dpos, 0, single ? 1 : p.W});
    } else if (vd.accepted) {
      // a sibling at v: it becomes the token there, with the layers it has run; every
      // token after v goes. The next step's embedding launch moves its rows.
      h->acc += 1;
      const int st = h->F[1].stage;
      const int depth = p.starts[st];
      for (int l = 0; l < p.L; ++l) h->kv_len[l] = std::min(h->kv_len[l], l < depth ? v + 1 : v);
      h->F.clear();
      h->F.push_back({v, st, 1});
      h->adopt = true;
      h->adopt_pos = v;
      h->adopt_idx = vd.accepted_index;
      h->adopt_layers = depth;
    } else {
      h->rej += 1;
      for (auto& k : h->kv_len) k = std::min(k, v);
      h->F.clear();
      h->F.push_back({v, 0, 1});
    }
  } else {
    h->F.push_back({h->pend_dpos, 0, p.W});
  }
  c.committed_total = (int)h->N;
  c.inflight = (int)h->F.size();
  if (out) *out = c;
  h->state = spd_handle::S_READY;
  return SPD_OK;
}

int spd_get_stats(const spd_handle* h, spd_stats* out) {
  if (!h || !out) return SPD_E_ARG;
  out->K = h->K; out->N = h->N; out->accepted = h->acc; out->rejected = h->rej;
  out->alpha = h->K ? (double)h->N / (double)h->K : 0.0;
  out->s0 = out->alpha * h->p.n;
  return SPD_OK;
}

int spd_get_kv_lens(const spd_handle* h, int32_t* per_layer, int32_t* pdm_len) {
  if (!h) return SPD_E_ARG;
  if (per_layer)
    for (int l = 0; l < h->p.L; ++l) per_layer[l] = h->kv_len[l];
  if (pdm_len) *pdm_len = h->pdm_len;
  return SPD_OK;
}

size_t spd_debug_size(const spd_handle* h, int32_t what) {
  if (!h) return 0;
  const Plan& p = h->p;
  switch (what) {
    case SPD_DBG_TARGET_LOGITS: case SPD_DBG_DRAFT_LOGITS: return (size_t)p.V * 4;
    case SPD_DBG_H_RING: return (size_t)p.ring * p.W * p.d * 4;
    case SPD_DBG_PDM_ROWS: return (size_t)p.ring * p.d * 4;
    case SPD_DBG_ANCHORS: return (size_t)p.ring * p.W * p.k * p.d * 4;
    case SPD_DBG_TARGET_KV: return (size_t)p.nsoft * 2 * p.hkv * p.max_ctx * p.hd * p.kv_esz;
    case SPD_DBG_PDM_KV: return (size_t)p.Ls * 2 * p.hkv * p.max_ctx * p.hd * p.kv_esz;
    case SPD_DBG_TOKENS: return (size_t)p.ring * p.W * 4;
    case SPD_DBG_TOP_P: return (size_t)(1 + p.ring) * sizeof(NucleusCut);
  }
  return 0;
}

int spd_debug_copy(const spd_handle* hc, int32_t what, void* dst, size_t bytes) {
  spd_handle* h = const_cast<spd_handle*>(hc);
  if (!h || !dst) return SPD_E_ARG;
  const Plan& p = h->p;
  const size_t need = spd_debug_size(h, what);
  if (need == 0 || bytes != need) return fail(h, SPD_E_ARG, "bad debug buffer or size");
  const char* src = nullptr;
  switch (what) {
    case SPD_DBG_TARGET_LOGITS: src = h->ws + p.o_logits; break;
    case SPD_DBG_DRAFT_LOGITS: {
      // the most recent draft: position newest + 1 of the last step
      const int dpos = h->state == spd_handle::S_INIT ? 0 : h->pend_dpos;
      src = h->ws + p.o_qring + (size_t)h->slot(dpos) * p.V * 4;
      break;
    }
    case SPD_DBG_H_RING: src = h->ws + p.o_h; break;
    case SPD_DBG_PDM_ROWS: src = h->ws + p.o_hp; break;
    case SPD_DBG_ANCHORS: src = h->ws + p.o_anch; break;
    case SPD_DBG_TARGET_KV: src = h->ws + p.o_kv; break;
    case SPD_DBG_PDM_KV: src = h->ws + p.o_pkv; break;
    case SPD_DBG_TOKENS: src = h->ws + p.o_tok; break;
    case SPD_DBG_TOP_P: src = h->ws + p.o_cut; break;
  }
  HIPCHK(h, hipStreamSynchronize(h->st));
  if (what == SPD_DBG_TARGET_KV || what == SPD_DBG_PDM_KV) {
    // device layers hold K [hkv][max_ctx][hd] then V (v_index) in kv_layer_bytes; the copy
    // is [layers][2][hkv][max_ctx][hd] row-major
    const int layers = what == SPD_DBG_TARGET_KV ? p.nsoft : p.Ls;
    std::vector<char> raw((size_t)layers * p.kv_layer_bytes);
    HIPCHK(h, hipMemcpy(raw.data(), src, raw.size(), hipMemcpyDeviceToHost));
    const size_t plane = (size_t)p.hkv * p.max_ctx * p.hd;   // elements of K (or V) of a layer
    char* o = static_cast<char*>(dst);
    for (int l = 0; l < layers; ++l) {
      const char* kl = raw.data() + (size_t)l * p.kv_layer_bytes;
      const char* vl = kl + p.kv_layer_bytes / 2;
      const size_t e = p.kv_esz;
      char* ok = o + (size_t)l * 2 * plane * e;
      char* ov = ok + plane * e;
      std::memcpy(ok, kl, plane * e);
      for (int g = 0; g < p.hkv; ++g)
        for (int pos = 0; pos < p.max_ctx; ++pos)
          for (int d = 0; d < p.hd; ++d)
            std::memcpy(ov + (((size_t)g * p.max_ctx + pos) * p.hd + d) * e,
                        vl + v_index(p.kv_bf16, g, pos, d, p.hd, p.max_ctx) * e, e);
    }
    return SPD_OK;
  }
  HIPCHK(h, hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost));
  return SPD_OK;
}

int spd_reset(spd_handle* h) {
  if (!h) return SPD_E_ARG;
  if (h->state == spd_handle::S_PENDING || h->ahead) HIPCHK(h, hipStreamSynchronize(h->st));
  h->ahead = false;
  h->state = spd_handle::S_INIT;
  h->F.clear();
  h->pdm_len = 0;
  std::fill(h->kv_len.begin(), h->kv_len.end(), 0);
  h->N = h->K = h->acc = h->rej = 0;
  h->P0 = 0;
  h->pend_dpos = 0;
  h->pre_valid = false;
  h->adopt = false;
  return SPD_OK;
}

const char* spd_last_error(const spd_handle* h) { return h ? h->err.c_str() : "null handle"; }

void spd_destroy(spd_handle* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->st);
  for (auto e : h->ev) (void)hipEventDestroy(e);
  if (h->st2) (void)hipStreamSynchronize(h->st2);
  if (h->h_desc_base) (void)hipHostFree(h->h_desc_base);
  if (h->h_verdict_base) (void)hipHostFree(h->h_verdict_base);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  for (hipEvent_t ev : h->ev_step)
    if (ev) (void)hipEventDestroy(ev);
  if (h->st2) (void)hipStreamDestroy(h->st2);
  delete h;
}

// ---- measurement -------------------------------------------------------------------
int spd_lookahead(spd_handle* h, int on) {
  if (!h) return SPD_E_ARG;
  h->err.clear();
  h->lookahead = on != 0;
  return SPD_OK;
}

int spd_timing_enable(spd_handle* h, int on) {
  if (!h) return SPD_E_ARG;
  if (h->state == spd_handle::S_PENDING || h->ahead) return fail(h, SPD_E_STATE, "a step is pending");
  h->timing = on != 0;
  h->serial = on == 2;
  for (int i = 0; i < OP_NKINDS; ++i) { h->kt_ms[i] = 0; h->kt_bytes[i] = 0; h->kt_count[i] = 0; }
  h->kl_ms.assign(h->p.L, 0.0);
  h->kl_passes.assign(h->p.L, 0);
  // two events per timed launch of a step, created once and reused every step
  const size_t want = 2 * (size_t)(8 + 5 * (h->p.L + h->p.Ls));
  while (h->timing && h->ev.size() < want) {
    hipEvent_t e;
    HIPCHK(h, hipEventCreate(&e));
    h->ev.push_back(e);
  }
  return SPD_OK;
}

int spd_timing_read(const spd_handle* h, int32_t kind, int64_t* count, double* total_ms,
                    double* bytes) {
  if (!h || kind < 0 || kind >= OP_NKINDS) return SPD_E_ARG;
  if (count) *count = h->kt_count[kind];
  if (total_ms) *total_ms = h->kt_ms[kind];
  if (bytes) *bytes = h->kt_bytes[kind];
  return SPD_OK;
}

int spd_timing_read_layers(const spd_handle* h, double* total_ms, int64_t* passes) {
  if (!h || !total_ms || !passes) return SPD_E_ARG;
  for (int l = 0; l < h->p.L; ++l) {
    total_ms[l] = l < (int)h->kl_ms.size() ? h->kl_ms[l] : 0.0;
    passes[l] = l < (int)h->kl_passes.size() ? h->kl_passes[l] : 0;
  }
  return SPD_OK;
}

// ---- stage planning (host only) -----------------------------------------------------
int spd_balance_stages(int32_t n_layers, const float* layer_cost, int32_t n_stages,
                       int32_t* stage_layers) {
  const int L = n_layers, n = n_stages;
  if (!layer_cost || !stage_layers || L < 1 || L > 4096 || n < 1 || n > L) return SPD_E_ARG;
  for (int l = 0; l < L; ++l)
    if (!(layer_cost[l] >= 0.f) || !std::isfinite(layer_cost[l])) return SPD_E_ARG;
  // cost of layers [i, j), summed in double from i upward
  auto seg = [&](int i, int j) {
    double s = 0.0;
    for (int l = i; l < j; ++l) s += (double)layer_cost[l];
    return s;
  };
  // ok[i * (n + 1) + k]: layers [i, L) split into exactly k stages, each of cost in [A, B]
  std::vector<char> ok((size_t)(L + 1) * (n + 1));
  auto solve = [&](double A, double B) {
    std::fill(ok.begin(), ok.end(), 0);
    ok[(size_t)L * (n + 1)] = 1;
    for (int i = L - 1; i >= 0; --i) {
      double s = 0.0;
      for (int j = i + 1; j <= L; ++j) {
        s += (double)layer_cost[j - 1];
        if (s > B) break;
        if (s < A) continue;
        for (int k = 1; k <= n; ++k)
          if (ok[(size_t)j * (n + 1) + k - 1]) ok[(size_t)i * (n + 1) + k] = 1;
      }
    }
    return ok[n] != 0;
  };
  // both bounds of an optimal split are segment costs
  std::vector<double> cand;
  cand.reserve((size_t)L * (L + 1) / 2);
  for (int i = 0; i < L; ++i) {
    double s = 0.0;
    for (int j = i; j < L; ++j) { s += (double)layer_cost[j]; cand.push_back(s); }
  }
  std::sort(cand.begin(), cand.end());
  // 1. the smallest largest-stage cost B
  size_t lo = 0, hi = cand.size() - 1;          // one stage per layer run is always possible
  while (lo < hi) {
    const size_t mid = (lo + hi) / 2;
    if (solve(0.0, cand[mid])) hi = mid; else lo = mid + 1;
  }
  const double B = cand[lo];
  // 2. with that, the largest smallest-stage cost A
  lo = 0; hi = cand.size() - 1;
  while (lo < hi) {
    const size_t mid = (lo + hi + 1) / 2;
    if (solve(cand[mid], B)) lo = mid; else hi = mid - 1;
  }
  const double A = cand[lo];
  // 3. among splits within [A, B], each stage in turn takes as many layers as it can
  solve(A, B);
  int i = 0;
  for (int st = 0; st < n; ++st) {
    const int rest = n - st - 1;
    int take = 0;
    for (int j = L - rest; j > i; --j) {
      const double c = seg(i, j);
      if (c >= A && c <= B && ok[(size_t)j * (n + 1) + rest]) { take = j - i; break; }
    }
    if (take < 1) return SPD_E_ARG;   // unreachable for valid input
    stage_layers[st] = take;
    i += take;
  }
  return SPD_OK;
}

}  // extern "C"
