// Internal declarations shared by the host scheduler and the CDNA4 kernels.
// Descriptor structs live in device memory (uploaded once per step) and are
// read by every workgroup of a grouped launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spd {

constexpr int kMaxStages = 16;          // n
constexpr int kMaxRows = kMaxStages + 1;  // PDM rows per step: n + 1
constexpr int kMaxAnchors = 8;          // k
constexpr int kMaxWidth = 4;            // W: draft candidates per position
// a launch finds its problem with one load per lane of a wave: at most 64 problems, and a
// target attention launch holds one per candidate of every in-flight position
static_assert(kMaxStages * kMaxWidth <= 64, "attention problems per launch exceed a wave");
constexpr int kWaves = 4;               // waves per GEMV workgroup
constexpr int kMaxVec = kMaxRows;       // input vectors of one GEMV problem
constexpr int kAttnTile = 64;           // keys per attention tile
constexpr int kVocabBlock = 1024;       // threads of the vocabulary reduction blocks
constexpr float kNearTie = 1e-3f;
constexpr float kLinEps = 1e-6f;          // linear attention: q, k / sqrt(|.|^2 + eps)

// GEMV epilogues.
enum Epi : int {
  EPI_STORE = 0,   // y[v][row] = acc
  EPI_ADD = 1,     // y[v][row] += acc; aux (if set): aux[v][row] = new y (anchor capture)
  EPI_SWIGLU = 2,  // y[v][row] = silu(W row) * (W2 row)
  EPI_QKV = 3,     // rotate q,k pairs (RoPE at pos0 + v, or pos0 for every vector when
                   // same_pos); q -> aux, k,v -> KV cache (vectors v >= 1 of a same_pos
                   // problem, sibling candidates, -> their side rows)
};

// One matrix times nvec vectors, y = epilogue(W * (x ⊙ gain) * rms_scale(x)).
struct GemvProb {
  const void* W;       // [rows][K] in the weight dtype
  const void* W2;      // SWIGLU: the up matrix (W is the gate)
  const float* x;      // vector v at x + v * x_stride
  const float* gain;   // RMSNorm gain of vector v at gain + v * gain_stride; null: no norm
  float* y;            // output of vector v at y + v * y_stride
  float* aux;          // EPI_QKV: rotated q; EPI_ADD: optional copy of the new residual
  void* kv_k;          // EPI_QKV: K cache of this layer [hkv][max_ctx][hd]
  void* kv_v;          // EPI_QKV: V cache of this layer
  long long x_stride, gain_stride, y_stride, aux_stride;
  float eps;
  int rows;            // matrix rows (SWIGLU: rows of each of W and W2)
  int K;
  int nvec;
  int epi;
  int pos0;            // EPI_QKV: position of vector 0
  int tile0;           // first workgroup of this problem in the launch
  int ntiles;
  int hq, hkv, hd, max_ctx;
  int ksplit;          // matrix-core kernel: waves sharing one row tile's K
  int pad;             // matrix-core kernel: row tiles per workgroup
  int kv_f32;          // EPI_QKV: the KV cache is fp32 (row-major V) even with bf16 weights
  int same_pos;        // EPI_QKV: every vector is a candidate for position pos0
  int side_row0;       // EPI_QKV, same_pos: side row of vector 1 (vector v: side_row0 + v - 1)
  int side_rows;       // rows of the side caches per kv head
  void* side_k;        // EPI_QKV, same_pos: side K [hkv][side_rows][hd], row-major
  void* side_v;        // side V, same layout
  int kchunk;          // rows kernel, chunked: K columns staged at a time (0: all of K)
  int pad2;
};

// Attention over one layer's KV cache for a group of query rows that share it: row r
// (position pos0 + r) attends keys 0 .. len + r - 1. A row of the staircase is a
// problem of its own; rows of the PDM window (one PDM layer) are grouped, up to
// 16 / group query heads per problem on the bf16 path (one row on the fp32 path).
struct AttnProb {
  const float* q;      // row r: [hq][hd] at q + r * q_stride, rotated
  float* out;          // row r: [hq][hd] at out + r * out_stride
  const void* K;       // [hkv][max_ctx][hd]
  const void* V;       // bf16: key-blocked (v_index); fp32: [hkv][max_ctx][hd]
  int len;             // keys of row 0
  int tile0;           // first workgroup: tile0 + g * nsplit + s
  int nsplit;
  int slot;            // index of this problem's partial area
  int nrows;           // query rows
  int q_stride, out_stride;
  int self_row;        // with side_k set: a sibling candidate (nrows 1), whose own key,
                       // position len - 1, is side row self_row, not the cache's row
  int side_rows;
  const void* side_k;  // [hkv][side_rows][hd] row-major, in the cache's dtype
  const void* side_v;
};

// Rows of a layer's K or V cache, padded to whole 32-key blocks.
__host__ __device__ constexpr int kv_ctx(int max_ctx) { return (max_ctx + 31) / 32 * 32; }

// Element of V[kv head g][key pos][dim d] in a layer's V cache. bf16 caches keep every
// block of 32 keys transposed ([dim][32 keys]), so the 8 consecutive keys of one dim
// that a matrix-core operand lane takes are one contiguous piece; fp32 caches are
// row-major.
__host__ __device__ inline size_t v_index(bool blocked, int g, int pos, int d, int hd,
                                          int max_ctx) {
  if (blocked)
    return (((size_t)g * (kv_ctx(max_ctx) / 32) + pos / 32) * hd + d) * 32 + (pos & 31);
  return ((size_t)g * max_ctx + pos) * hd + d;
}

// Linear-attention (recurrent) step for one token at one layer.
struct LinProb {
  const float* qkv;    // [3][H][hd]: q, k, v of this token
  float* out;          // [H][hd]
  const float* s_prev; // state after the previous position [H][hd][hd]
  float* s_next;       // state after this position
};

// The embedding of the stage-0 token and the PDM feature gather (anchor clamp).
struct EmbedGather {
  const void* embed;          // [V][d]
  const int* tok_ring;        // token of position p at tok_ring[p % ring]
  float* h_ring;              // [ring][d]
  float* anchors;             // [ring][k][d]
  float* X;                   // [M][k * d] gathered PDM features
  int newest_slot;             // ring row of the newest token (rows: slot * W + candidate)
  int embed_new;              // 1: block 0 embeds the newest token (0: a gather-only launch)
  int embed_w;                // candidates of the newest position embedded (rows newest_slot ..)
  int d, k, M;
  int row_slot[kMaxRows];     // ring row of PDM row r
  signed char src[kMaxRows][kMaxAnchors];  // anchor index feeding segment i; -1: zeros; -2: newest g0
  // adoption of a sibling candidate as the token at position adopt_pos: its residual and
  // anchors move from ring row adopt_from to adopt_to, and its keys and values of the
  // first adopt_layers target layers from its side row into the cache at adopt_pos
  int adopt_layers;           // 0: nothing to adopt
  int adopt_from, adopt_to, adopt_pos, adopt_side_row;
  char* kv_base;              // target KV region: softmax layer l at kv_base + l * kv_layer_bytes
  char* side_base;            // side caches: layer l at side_base + l * side_layer_bytes
  size_t kv_layer_bytes, side_layer_bytes;
  int hkv, hd, max_ctx, side_rows, kv_bf16;
};

// The vocabulary pass: statistics of up to two logit rows (target, draft).
// Top-p set of one logit row (T > 0, top_p < 1): the tokens with z > zb, and the
// tokens with z == zb and id <= id_cut. lse: log of the sum over the set of exp(z / T).
struct NucleusCut {
  float zb;
  int id_cut;
  float lse;
  int pad;
};

__device__ __forceinline__ bool in_cut(float z, int i, const NucleusCut& c) {
  return z > c.zb || (z == c.zb && i <= c.id_cut);
}

struct VocabDesc {
  const float* logits[2];     // row 0: target head output, row 1: draft (PDM) head output
  int active[2];
  int gumbel_stream[2];       // 0: none
  int gumbel_pos[2];
  int V;
  int nblocks;
  float inv_temp;             // 1/T (T > 0) else 1
  int sampled;                // T > 0
  unsigned long long seed;
  int nucleus;                // T > 0 and top_p < 1: the Gumbel draw runs over the top-p set
  float top_p;
  NucleusCut* cut[2];         // where each active row's top-p set is written
  int topw;                   // > 1: the draft row's topw + 1 best (score, id) per block
  struct VocabTop* top;       // [nblocks] (scores: the logit at T = 0, z / T + G at T > 0)
  unsigned long long* nuc_part;   // scratch: per-slice histograms [2][64][4096]
  unsigned long long* nuc_hist;   // scratch: merged histograms [2][4096]
  int2* nuc_cand;                 // scratch: listed (logit bits, id) [2][V]
  int* nuc_cnt;                   // scratch: listed per slice [2][64]
  float* nuc_max;                 // scratch: each row's largest logit [2]
};

// top-p scratch sizes (bytes), for the workspace plan
constexpr size_t kNucPartBytes = (size_t)2 * 64 * 4096 * 8;
constexpr size_t kNucHistBytes = (size_t)2 * 4096 * 8;
constexpr size_t kNucCntBytes = (size_t)2 * 64 * 4 + 16;   // counts, then the two maxima

// The best scores of one slice of the draft row, highest first, lower id first on ties.
struct VocabTop {
  float s[kMaxWidth + 1];
  int id[kMaxWidth + 1];
};

struct VocabPartial {
  float max, second;          // raw logit max and runner-up
  int arg;
  float sum;                  // sum exp(z/T - max/T)
  float gmax, gsecond;        // Gumbel-perturbed z/T + G
  int garg;
  int pad;
};

// Device-side verdict of one step, copied to pinned host memory at its end.
struct Verdict {
  int draft;            // this step's draft (position newest + 1)
  int committed;        // y
  int accepted;
  int flags;            // bit 0 verify near-tie, bit 1 draft near-tie
  int verified_draft;
  int exited;
  int need_residual;
  int first_token;      // prefill: first generated token
  float lse_t, lse_q, p_d, q_d;
  int accepted_index;   // which candidate at v was accepted (-1: none)
  int need_rrs;         // T > 0, W > 1, the first candidate rejected: the later rounds run
  int target_arg;       // argmax of the target row (lowest id on ties)
  int pad;
};

struct FinalizeDesc {
  int mode;             // 0: step, 1: prefill (first token)
  int exited;
  int single;           // the exiting token is the only one in flight (v = newest + 1)
  int v;                // verified position
  int dpos;             // position of this step's draft
  int ring;             // n + 1
  int V;
  int nblocks;
  float temp;
  float inv_temp;
  unsigned long long seed;
  int forced_mode;
  float forced_p;
  int forced_base;      // position of forced_ref[0]
  int forced_len;
  const int* forced_ref;
  const float* zt;      // target logits (row 0)
  const float* zq_v;    // stored draft logits of the draft at v
  const float* lse_q_v; // its log-sum-exp (of z/T)
  float* lse_q_new;     // where to store this draft's log-sum-exp
  int* tok_ring;
  Verdict* verdict;
  Verdict* host_verdict;     // device view of pinned host memory: the finished verdict, so the
                             // host reads it once the stream is idle, with no copy
  const VocabPartial* part;  // [2][nblocks]
  int nucleus;               // top_p < 1: probabilities are renormalised over the top-p sets
  const NucleusCut* cut_t;   // the target row's set (this step)
  const NucleusCut* cut_q;   // this step's draft row's set
  const NucleusCut* cut_q_v; // the set of the draft at v
  int W;                     // candidates per draft position (token ring rows: slot * W + b)
  const VocabTop* top;       // [nblocks] the draft row's best scores (W > 1)
  float* pq;                 // W > 1: [2][V] scratch, p(x) then q(x) of the verified position
};

enum RngStream : int { RNG_DRAFT = 1, RNG_ACC = 2, RNG_RES = 3, RNG_FORCE = 4, RNG_FIRST = 5 };

// ---- small device helpers ------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// SplitMix64 output function (Steele, Lea & Flood 2014).
__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Counter-based uniform in (0,1): a pure function of (seed, stream, pos, idx).
__device__ __forceinline__ float rng_uniform(unsigned long long seed, int stream, int pos,
                                             unsigned long long idx) {
  unsigned long long k0 = mix64(seed);
  unsigned long long key = ((unsigned long long)(unsigned)stream << 32) | (unsigned)pos;
  unsigned long long k1 = mix64(k0 ^ key);
  unsigned long long x = mix64(k1 + idx * 0x9E3779B97F4A7C15ull);
  return ((float)(x >> 41) + 0.5f) * (1.0f / 8388608.0f);
}

__device__ __forceinline__ float gumbel_of(float u) { return -logf(-logf(u)); }

// ---- wavefront (64-lane) reductions with DPP moves --------------------------
// Within each row of 16 lanes: xor 1 and xor 2 by quad permutes, then the
// half-row and row mirrors; across the four rows: readlane of lanes 0, 16, 32,
// 48. Every lane gets the same result, in the same order in every wave.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sum over the 16 lanes of a DPP row (every lane of the row gets it); LANES = 8 stops at
// half rows.
template <int LANES>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  if constexpr (LANES == 16) v += dpp_mov<0x140>(v);
  return v;
}

// Operand and accumulator types of the CDNA4 bf16 matrix instruction
// v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16] (e = 0..7) and D[4 (l / 16) + r][l % 16] (r = 0..3).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x = hi + mid + lo with each term a bfloat16 (round to nearest even at every step);
// the residual left out is below 2^-24 |x|, so three bf16 products summed in fp32 give
// an fp32-accurate product with an exact bf16 operand.
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f2bf(x);
  const float r1 = x - __uint_as_float(hi << 16);
  mid = f2bf(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f2bf(r2);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// 16 bytes of weights, streamed once: a nontemporal load keeps them from
// displacing reusable lines (activations, KV rows) in the caches.
// The pointer is taken as a global-memory one: a generic (flat) load would count on the
// LDS counter too, and every wait for it would also drain pending LDS traffic.
#define SPD_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ uint4 load_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const SPD_GLOBAL u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Ordinary 16- and 8-byte loads through a global-memory pointer.
__device__ __forceinline__ uint4 load_g16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const SPD_GLOBAL u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_g8(const void* p) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *(const SPD_GLOBAL u32x2*)p;
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 load_g4(const float* p) {
  const f32x4_t v = *(const SPD_GLOBAL f32x4_t*)p;
  return make_float4(v[0], v[1], v[2], v[3]);
}
#define SPD_LOCAL __attribute__((address_space(3)))
// 8-byte LDS store through a local-memory pointer.
__device__ __forceinline__ void lds_store8(void* p, uint32_t a, uint32_t b) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  *(SPD_LOCAL u32x2*)p = u32x2{a, b};
}
// 16-byte read of LDS through a local-memory pointer (ds_read_b128, LDS counter only).
__device__ __forceinline__ uint4 lds_load16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const SPD_LOCAL u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Index of the problem that owns workgroup b in a grouped launch whose problems
// start at ascending workgroups tile0 (nprob <= 64). Each lane reads one start,
// so the search costs one memory round trip instead of a chain of dependent loads.
template <typename P>
__device__ __forceinline__ int find_problem(const P* __restrict__ probs, int nprob, int b) {
  const int lane = threadIdx.x & 63;
  const bool owns = lane < nprob && probs[lane < nprob ? lane : 0].tile0 <= b;
  const unsigned long long mask = __ballot(owns);
  return __popcll(mask) - 1;
}

}  // namespace spd

// ---- kernel launchers (one per .hip file) -----------------------------------
namespace spd {
// Optional timing events bound to the dispatch packets themselves (start: when the
// first launch of an op begins, stop: when its last one ends), so a measured
// duration is the kernels' own and excludes the command processor's gaps.
struct LaunchEv {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
#define SPD_LAUNCH(ev, kernel, grid, block, shm, st, ...)                                     \
  do {                                                                                       \
    if ((ev).start || (ev).stop)                                                             \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, st, (ev).start, (ev).stop, 0, __VA_ARGS__); \
    else                                                                                     \
      hipLaunchKernelGGL(kernel, grid, block, shm, st, __VA_ARGS__);                         \
  } while (0)

enum GemvRole : int { GEMV_PROJ = 0, GEMV_QKV, GEMV_O, GEMV_GATE_UP, GEMV_DOWN, GEMV_HEAD,
                      GEMV_PDM_QKV, GEMV_PDM_O, GEMV_PDM_GATE_UP, GEMV_PDM_DOWN, GEMV_NROLES };
// How one grouped GEMV launch runs: kernel kind, waves per workgroup, workgroups, and
// the dynamic LDS each workgroup takes (staged inputs). gemv_plan chooses the kind for
// a grouped launch and fills tile0 / ntiles / ksplit of every problem.
struct GemvPlan {
  int kind = 0, waves = 0, ntiles = 0;
  int shm = 0;
  int tpp = 0;   // workgroups of every problem when all problems have the same count, else 0
};
GemvPlan gemv_plan(GemvProb* probs, int nprob, bool bf16);
hipError_t launch_gemv(int role, const GemvProb* d_probs, int nprob, const GemvPlan& plan, bool bf16,
                       const float2* rope, hipStream_t st, LaunchEv ev = {});
hipError_t launch_attention(const AttnProb* d_probs, int nprob, int ntiles, bool bf16,
                            int hq, int hkv, int hd, int max_ctx, int split_len, bool any_split,
                            float* partials, hipStream_t st, LaunchEv ev = {},
                            bool siblings = false);   // siblings: some problem has self_row >= 0
hipError_t launch_attention_prefill(const float* q, int q_stride, float* out, int out_stride,
                                    const void* K, const void* V, int pos0, int P, bool bf16,
                                    int hq, int hkv, int hd, int max_ctx, hipStream_t st);
int attn_max_split();
// Query rows per attention problem when rows share a cache (bf16: 16 / group).
int attn_rows_per_problem(bool bf16, int hq, int hkv);
hipError_t launch_linear_step(const LinProb* d_probs, int nprob, int H, int hd, float eps,
                              hipStream_t st, LaunchEv ev = {});
hipError_t launch_linear_scan(const float* qkv, int qkv_stride, float* out, int out_stride,
                              const float* s_in, float* s_out, int P, int H, int hd, float eps,
                              hipStream_t st);
// desc: the gather descriptor, readable by the device (it may sit in pinned host memory);
// blk_src / blk_dst / blk_bytes: the step's descriptor block, copied to the device first.
hipError_t launch_embed_gather(const EmbedGather* desc, const void* blk_src, void* blk_dst,
                               size_t blk_bytes, int M, int k, int d, bool bf16, hipStream_t st,
                               LaunchEv ev = {}, int adopt_layers = 0);
hipError_t launch_vocab_stats(const VocabDesc* d_desc, int nblocks, VocabPartial* part,
                              hipStream_t st, LaunchEv ev = {});
hipError_t launch_nucleus(const VocabDesc* d_desc, int nblocks, VocabPartial* part,
                          hipStream_t st, LaunchEv ev = {});
hipError_t launch_finalize(const FinalizeDesc* d_desc, hipStream_t st, LaunchEv ev = {});
hipError_t launch_residual_impl(const FinalizeDesc* d_desc, VocabPartial* part, int nblocks,
                                hipStream_t st, LaunchEv ev = {});
// Draft trees at T > 0: the verification rounds after the first candidate's rejection.
hipError_t launch_tree_rounds(const FinalizeDesc* d_desc, VocabPartial* part, int nblocks,
                              hipStream_t st, LaunchEv ev = {});
// prefill helpers
hipError_t launch_embed_rows(const void* embed, const int* toks, float* H, int P, int d,
                             bool bf16, hipStream_t st);
hipError_t launch_rmsnorm_rows(const float* H, int h_stride, const float* gain, void* out,
                               int out_stride, int P, int d, float eps, bool out_bf16,
                               hipStream_t st);
hipError_t launch_round_rows(const float* X, int x_stride, void* out, int out_stride, int P,
                             int n, bool out_bf16, hipStream_t st);
hipError_t launch_rope_kv(float* QKV, int stride, void* Kc, void* Vc, const float2* rope,
                          int pos0, int P, int hq, int hkv, int hd, int max_ctx, bool bf16,
                          hipStream_t st);
hipError_t launch_swiglu_rows(const float* G, const float* U, int stride, void* out,
                              int out_stride, int P, int F, bool out_bf16, hipStream_t st);
hipError_t launch_copy_rows(const float* src, int src_stride, float* dst, int dst_stride,
                            int P, int n, hipStream_t st);
// C[P][N] (=|+=) A[P][K] * W[N][K]^T, A and C float32, W in the weight dtype.
hipError_t launch_gemm(const float* A, int lda, const void* W, float* C, int ldc, int P, int N,
                       int K, bool accumulate, bool bf16, hipStream_t st);
}  // namespace spd
