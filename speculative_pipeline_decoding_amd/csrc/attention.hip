// Staircase decode attention: every query row attends over its own layer's KV
// cache with its own length (the in-flight tokens sit at different layers and
// positions). One workgroup = one (problem, kv head, key split); the hq/hkv
// query heads that share the kv head (GQA) are scored together, so each K/V
// row is read from HBM once per kv head.
//
// Inside a workgroup the four waves walk disjoint 64-key tiles with no block
// barrier in the loop: a lane holds its key's K row in registers and scores
// it against every query head of the group (q broadcast from LDS), the wave
// keeps a running max / sum per head, and V is accumulated with lanes owning
// pairs of head dimensions. The waves merge in LDS at the end; the key splits
// of one (problem, kv head) are merged by a second small kernel (the kernel
// boundary orders the partials; no device-wide fence in the hot loop).
//
// That kernel serves fp32 caches. bf16 caches take the matrix-core kernel below, which
// also groups query rows that share a cache (the PDM window, prompt rows).
//
// Prefill uses the same kernels with the prompt rows as problems and no split.
#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kMaxSplit = 16;     // key splits per (problem, kv head)
constexpr int kAttnWaves = 4;


template <typename T, int HD>
__device__ __forceinline__ void unpack(const uint4& u, float* f) {
  if constexpr (sizeof(T) == 2) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  } else {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
}

// LDS words per V row in a wave's tile: bf16 rows hold HD/2 words, float rows HD;
// one pad word makes the stride odd, so the row-major writes do not collide on banks.
template <typename T, int HD>
constexpr int v_words() { return (sizeof(T) == 2 ? HD / 2 : HD) + 1; }

// fp32 rows wider than 64 dims would make each wave's V tile most of the CU's LDS: there
// the wave reads the tile's V rows straight from memory in the p V sum instead (one whole,
// coalesced row per key, the lanes over the head dims).
template <typename T, int HD>
constexpr bool direct_v() { return sizeof(T) == 4 && HD > 64; }

// LDS: q [GMAX][HD], p [waves][64][GMAX], V tiles [waves][64][v_words] (none when V is
// read directly); after the key loop the same space holds the wave merge
// [waves][GMAX][HD + 2].
template <typename T, int HD, int GMAX>
constexpr size_t attn_lds_floats() {
  constexpr size_t tile = direct_v<T, HD>() ? 0 : (size_t)kAttnWaves * 64 * v_words<T, HD>();
  constexpr size_t merge = (size_t)kAttnWaves * GMAX * (HD + 2);
  return (size_t)GMAX * HD + kAttnWaves * 64 * GMAX + (tile > merge ? tile : merge);
}

template <typename T, int HD, int GMAX>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_kernel(
    const AttnProb* __restrict__ probs, int nprob,
    // prefill mode (probs == nullptr): problem r is prompt row r
    const float* __restrict__ pq, int q_stride, float* __restrict__ pout, int out_stride,
    const void* pK, const void* pV, int pos0,
    int G, int hkv, int max_ctx, int split_len, float* __restrict__ partials) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int NC = HD / E;                 // chunks per K row
  constexpr int HALF = HD / 2;
  constexpr int VW = v_words<T, HD>();
  __shared__ __attribute__((aligned(16))) float lds[attn_lds_floats<T, HD, GMAX>()];
  float* qs = lds;                                        // [GMAX][HD]
  float* pb = lds + GMAX * HD;                            // [waves][64][GMAX]
  float* mg = pb + kAttnWaves * 64 * GMAX;                // [waves][GMAX][HD + 2] (after the loop)
  uint32_t* vt = reinterpret_cast<uint32_t*>(mg) + (size_t)(threadIdx.x >> 6) * 64 * VW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const float* q;
  float* out;
  const T* Kb;
  const T* Vb;
  int len, nsplit, s, g, slot;
  int self_key = -1;             // a sibling candidate's own key: read from its side row
  const T* sk_row = nullptr;
  const T* sv_row = nullptr;
  if (probs) {
    const int pi = find_problem(probs, nprob, b);
    const AttnProb& P = probs[pi];
    const int t = b - P.tile0;
    g = t / P.nsplit;
    s = t % P.nsplit;
    nsplit = P.nsplit;
    q = P.q; out = P.out; len = P.len; slot = P.slot;
    Kb = static_cast<const T*>(P.K);
    Vb = static_cast<const T*>(P.V);
    if (P.side_k && P.self_row >= 0) {
      self_key = P.len - 1;
      sk_row = static_cast<const T*>(P.side_k) + ((size_t)g * P.side_rows + P.self_row) * HD;
      sv_row = static_cast<const T*>(P.side_v) + ((size_t)g * P.side_rows + P.self_row) * HD;
    }
  } else {
    const int r = b / hkv;
    g = b % hkv;
    s = 0; nsplit = 1; slot = 0;
    q = pq + (size_t)r * q_stride;
    out = pout + (size_t)r * out_stride;
    len = pos0 + r + 1;
    Kb = static_cast<const T*>(pK);
    Vb = static_cast<const T*>(pV);
  }
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) qs[i] = q[(size_t)g * G * HD + i];
  __syncthreads();
  const int k_lo = s * split_len;
  const int k_hi = min(len, k_lo + split_len);
  const float scale = rsqrtf((float)HD);
  const T* Kh = Kb + (size_t)g * max_ctx * HD;
  const T* Vh = Vb + (size_t)g * max_ctx * HD;
  float m[GMAX], l[GMAX];
  float2 acc[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) { m[h] = -INFINITY; l[h] = 0.f; acc[h] = make_float2(0.f, 0.f); }
  float* mypb = pb + w * 64 * GMAX;
  for (int t0 = k_lo + w * 64; t0 < k_hi; t0 += kAttnWaves * 64) {
    const int nrows = min(64, k_hi - t0);
    const bool valid = lane < nrows;
    // this lane's key: K and V rows, both requested before either is used
    const int key = t0 + (valid ? lane : 0);
    const size_t rowoff = (size_t)key * HD;
    const bool own = key == self_key;
    const uint4* krow = reinterpret_cast<const uint4*>(own ? sk_row : Kh + rowoff);
    const uint4* vrow = reinterpret_cast<const uint4*>(own ? sv_row : Vh + rowoff);
    constexpr bool DV = direct_v<T, HD>();
    uint4 kr[NC], vr[DV ? 1 : NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = krow[c];
    if constexpr (!DV) {
#pragma unroll
      for (int c = 0; c < NC; ++c) vr[c] = vrow[c];
    }
    float sc[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      sc[h] = -INFINITY;
      if (h < G) {
        const float4* qh = reinterpret_cast<const float4*>(qs + h * HD);
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float kf[E];
          unpack<T, HD>(kr[c], kf);
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            const float4 qv = qh[(c * E + e) / 4];
            a += qv.x * kf[e] + qv.y * kf[e + 1] + qv.z * kf[e + 2] + qv.w * kf[e + 3];
          }
        }
        sc[h] = valid ? a * scale : -INFINITY;
      }
    }
    // the V row goes to the wave's LDS tile, to be summed by columns below
    if constexpr (!DV) {
      uint32_t* vdst = vt + lane * VW;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        vdst[4 * c] = vr[c].x; vdst[4 * c + 1] = vr[c].y;
        vdst[4 * c + 2] = vr[c].z; vdst[4 * c + 3] = vr[c].w;
      }
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        const float mn = fmaxf(m[h], wave_max(sc[h]));
        const float p = valid ? expf(sc[h] - mn) : 0.f;
        const float corr = expf(m[h] - mn);   // 0 on the first tile (m = -inf)
        l[h] = l[h] * corr + wave_sum(p);
        m[h] = mn;
        acc[h].x *= corr;
        acc[h].y *= corr;
        mypb[lane * GMAX + h] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (lane < HALF) {
#pragma unroll 4
      for (int j = 0; j < nrows; ++j) {
        float2 vv;
        if constexpr (DV) {
          const float* vr0 = t0 + j == self_key ? reinterpret_cast<const float*>(sv_row)
                                                : reinterpret_cast<const float*>(Vh) + (size_t)(t0 + j) * HD;
          vv = *reinterpret_cast<const float2*>(vr0 + 2 * lane);
        } else if constexpr (sizeof(T) == 2) {
          const uint32_t wv = vt[j * VW + lane];
          vv = make_float2(bf16_lo(wv), bf16_hi(wv));
        } else {
          vv = make_float2(__uint_as_float(vt[j * VW + 2 * lane]),
                           __uint_as_float(vt[j * VW + 2 * lane + 1]));
        }
        const float* pj = mypb + j * GMAX;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          if (h < G) {
            acc[h].x += pj[h] * vv.x;
            acc[h].y += pj[h] * vv.y;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  __syncthreads();   // every wave is done with its V tile before the merge reuses the space
  // merge the four waves: mg[w][h] = {m, l, acc[HD]}
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      float* row = mg + ((size_t)w * GMAX + h) * (HD + 2);
      if (lane == 0) { row[0] = m[h]; row[1] = l[h]; }
      if (lane < HALF) { row[2 + 2 * lane] = acc[h].x; row[3 + 2 * lane] = acc[h].y; }
    }
  }
  __syncthreads();
  const size_t pstride = HD + 2;
  for (int h = w; h < G; h += kAttnWaves) {
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kAttnWaves; ++u) M = fmaxf(M, mg[((size_t)u * GMAX + h) * (HD + 2)]);
    float L = 0.f;
    float2 a = make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kAttnWaves; ++u) {
      const float* row = mg + ((size_t)u * GMAX + h) * (HD + 2);
      const float f = row[0] == -INFINITY ? 0.f : expf(row[0] - M);
      L += row[1] * f;
      if (lane < HALF) { a.x += row[2 + 2 * lane] * f; a.y += row[3 + 2 * lane] * f; }
    }
    const int head = g * G + h;
    if (nsplit == 1) {
      if (lane < HALF) {
        out[head * HD + 2 * lane] = a.x / L;
        out[head * HD + 2 * lane + 1] = a.y / L;
      }
    } else {
      float* mine = partials + ((((size_t)slot * hkv + g) * kMaxSplit + s) * G + h) * pstride;
      if (lane == 0) { mine[0] = M; mine[1] = L; }
      if (lane < HALF) { mine[2 + 2 * lane] = a.x; mine[3 + 2 * lane] = a.y; }
    }
  }
}

// Merge the key splits of every (problem, kv head) whose keys were split:
// out = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M), in split order. A record holds
// CW query columns (column c = row c / G, head g G + c % G). The split weights are found
// once per column (every record's m and l read in one round), then each output element
// sums its splits with the loads of eight splits in flight at a time.
template <int HD>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_merge_kernel(
    const AttnProb* __restrict__ probs, int G, int hkv, int CW, const float* __restrict__ partials) {
  constexpr int PW = HD + 2;
  constexpr int PER = (16 * HD + kAttnWaves * 64 - 1) / (kAttnWaves * 64);   // workgroups per pair
  __shared__ float wgt[kMaxSplit][16];      // e^(m_s - M) / L per split and column
  __shared__ float ml[kMaxSplit][16][2];
  const int pair = blockIdx.x / PER, part = blockIdx.x % PER;
  const AttnProb& P = probs[pair / hkv];
  const int g = pair % hkv;
  const int nsplit = P.nsplit;
  if (nsplit == 1) return;
  const int ncol = P.nrows * G;
  const int t = part * blockDim.x + threadIdx.x;          // this thread's (column, dim)
  if (part * (int)blockDim.x >= ncol * HD) return;        // nothing for this workgroup
  const float* base = partials + ((size_t)P.slot * hkv + g) * kMaxSplit * CW * PW;
  // the element loads go out first, so both round trips overlap
  const int c = min(t / HD, ncol - 1), d = t % HD;
  float v[kMaxSplit];
#pragma unroll
  for (int u = 0; u < kMaxSplit; ++u)
    v[u] = u < nsplit ? base[((size_t)u * CW + c) * PW + 2 + d] : 0.f;
  for (int i = threadIdx.x; i < nsplit * ncol; i += blockDim.x) {
    const int u = i / ncol, cc = i % ncol;
    const float2 mv = *reinterpret_cast<const float2*>(base + ((size_t)u * CW + cc) * PW);
    ml[u][cc][0] = mv.x;
    ml[u][cc][1] = mv.y;
  }
  __syncthreads();
  if (threadIdx.x < ncol) {
    const int cc = threadIdx.x;
    float M = -INFINITY;
    for (int u = 0; u < nsplit; ++u) M = fmaxf(M, ml[u][cc][0]);
    float L = 0.f;
    for (int u = 0; u < nsplit; ++u) {
      const float f = ml[u][cc][0] == -INFINITY ? 0.f : expf(ml[u][cc][0] - M);
      wgt[u][cc] = f;
      L += ml[u][cc][1] * f;
    }
    const float inv = 1.f / L;
    for (int u = 0; u < nsplit; ++u) wgt[u][cc] *= inv;
  }
  __syncthreads();
  if (t >= ncol * HD) return;
  float a = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxSplit; ++u)
    if (u < nsplit) a += v[u] * wgt[u][c];
  P.out[(size_t)(c / G) * P.out_stride + (size_t)(g * G + c % G) * HD + d] = a;
}

// ---- matrix-core kernel (bf16 caches) ------------------------------------------------
// One workgroup = (problem, kv head, key split); its four waves take contiguous runs of
// 32-key blocks. The up-to-16 query columns of the problem (its rows x the G heads of
// the kv head) are the B operand of v_mfma_f32_16x16x32_bf16 throughout:
//   scores  S[key][col] = K[key][:] . q[col][:]   (A = K rows; q split into three bf16
//                                                   terms, so q.k is fp32-accurate)
//   output  O[dim][col] += V[key][dim] p[col][key] (A = the key-blocked V; p split into
//                                                   two bf16 terms)
// The score tile leaves lane (col = l % 16, q = l / 16) holding keys 4q..4q+3 of each
// 16-key half; the PV step takes exactly those keys as its k slots, so p goes from
// the softmax to the next MFMA without leaving the lane. The softmax is the usual
// running max / sum per column, reduced over the four lane groups with shuffles.
// SIB: the launch holds sibling candidates (draft trees), whose own key and value come
// from side rows; without it the kernel carries none of that code.
template <int HD, bool SIB>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_mfma_kernel(
    const AttnProb* __restrict__ probs, int nprob,
    // prefill mode (probs == nullptr): workgroup b covers prompt rows R (b / hkv) .. of kv
    // head b % hkv, R = 16 / G, row r at position pos0 + r
    const float* __restrict__ pq, int pq_stride, float* __restrict__ pout, int pout_stride,
    const void* pK, const void* pV, int pos0, int prows,
    int G, int hkv, int max_ctx, int split_len, float* __restrict__ partials) {
  constexpr int KST = (HD + 31) / 32;     // 32-dim steps of q.k
  constexpr int DT = HD / 16;             // 16-dim output tiles
  constexpr int PW = HD + 2;              // record: m, l, o[HD]
  __shared__ float mg[kAttnWaves][16][PW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const float* q;
  float* out;
  const uint16_t* Kb;
  const uint16_t* Vb;
  int len, nrows, qs, os, nsplit, s, g, slot;
  int self_key = -1;             // a sibling candidate's own key: read from its side row
  const uint16_t* sk_row = nullptr;
  const uint16_t* sv_row = nullptr;
  if (probs) {
    const int pi = find_problem(probs, nprob, blockIdx.x);
    const AttnProb& P = probs[pi];
    const int t = blockIdx.x - P.tile0;
    g = t / P.nsplit; s = t % P.nsplit; nsplit = P.nsplit; slot = P.slot;
    q = P.q; out = P.out; len = P.len; nrows = P.nrows; qs = P.q_stride; os = P.out_stride;
    Kb = static_cast<const uint16_t*>(P.K);
    Vb = static_cast<const uint16_t*>(P.V);
    if (SIB && P.side_k && P.self_row >= 0) {
      self_key = P.len - 1;
      sk_row = static_cast<const uint16_t*>(P.side_k) + ((size_t)g * P.side_rows + P.self_row) * HD;
      sv_row = static_cast<const uint16_t*>(P.side_v) + ((size_t)g * P.side_rows + P.self_row) * HD;
    }
  } else {
    const int R = 16 / G;
    const int r0 = (blockIdx.x / hkv) * R;
    g = blockIdx.x % hkv; s = 0; nsplit = 1; slot = 0;
    nrows = min(R, prows - r0); len = pos0 + r0 + 1;
    q = pq + (size_t)r0 * pq_stride; out = pout + (size_t)r0 * pout_stride;
    qs = pq_stride; os = pout_stride;
    Kb = static_cast<const uint16_t*>(pK);
    Vb = static_cast<const uint16_t*>(pV);
  }
  const int ncol = nrows * G;
  const bool cvalid = c < ncol;
  const int crow = cvalid ? c / G : 0, chead = g * G + c % G;
  const int clen = cvalid ? len + crow : 0;          // keys visible to this column
  const int k_lo = s * split_len, k_hi = min(len + nrows - 1, k_lo + split_len);
  const float scale = rsqrtf((float)HD);

  const int nb = (k_hi - k_lo + 31) / 32;
  const int j_lo = nb * w / kAttnWaves, j_hi = nb * (w + 1) / kAttnWaves;
  const uint16_t* Kg = Kb + (size_t)g * max_ctx * HD;
  const uint16_t* Vg = Vb + (size_t)g * (kv_ctx(max_ctx) / 32) * HD * 32;

  // a sibling's own value row, the DT dims this lane takes in the PV step, read once
  uint32_t svv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) svv[dt] = SIB && self_key >= 0 ? sv_row[16 * dt + c] : 0u;

  // K and V pieces of block j; rows past the cache end are clamped (their scores are
  // masked, and the cache is zero-filled at set-up, so every value is finite)
  uint4 kf[2][2][KST], vf[2][DT];
  auto load = [&](int buf, int j) {
    const int kb = k_lo + 32 * min(j, j_hi - 1);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = min(kb + 16 * kt + c, max_ctx - 1);
      const uint16_t* krow = SIB && key == self_key ? sk_row : Kg + (size_t)key * HD;
#pragma unroll
      for (int st = 0; st < KST; ++st) {
        const int d0 = 32 * st + 8 * gq;
        kf[buf][kt][st] = load_g16(krow + (d0 < HD ? d0 : 0));
      }
    }
    const uint16_t* vb = Vg + (size_t)(min(kb, max_ctx - 1) / 32) * HD * 32;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vp = vb + (size_t)(16 * dt + c) * 32 + 4 * gq;
      const uint2 a = load_g8(vp);
      const uint2 b = load_g8(vp + 16);
      vf[buf][dt] = make_uint4(a.x, a.y, b.x, b.y);
    }
  };
  // the first block is requested before q, so the two round trips overlap
  if (j_lo < j_hi) load(0, j_lo);

  // q of this lane's column, dims 32 st + 8 gq .. + 7, as three bf16 terms
  uint4 qf[KST][3];
#pragma unroll
  for (int st = 0; st < KST; ++st) {
    const int d0 = 32 * st + 8 * gq;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    if (cvalid && d0 < HD) {
      const float* qp = q + (size_t)crow * qs + (size_t)chead * HD + d0;
      const float4 a = load_g4(qp), b = load_g4(qp + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    uint32_t hi[8], mi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split3(v[e], hi[e], mi[e], lo[e]);
    qf[st][0] = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16, hi[6] | hi[7] << 16);
    qf[st][1] = make_uint4(mi[0] | mi[1] << 16, mi[2] | mi[3] << 16, mi[4] | mi[5] << 16, mi[6] | mi[7] << 16);
    qf[st][2] = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16, lo[6] | lo[7] << 16);
  }

  float m = -INFINITY, l = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto block = [&](int buf, int j) {
    const int kb = k_lo + 32 * j;
    // a sibling's own key sits in this block: the lane holding it (keys 4 gq .. 4 gq + 3,
    // and 16 + 4 gq .. of the block, dim 16 dt + c) swaps in the side row's value. Done
    // here, where the values are consumed anyway, with selects only (a swap at load time
    // would make every load wait at once), and only in a sibling's workgroups.
    if (SIB && self_key >= 0) {
      const int off = self_key - kb;
      const bool own = self_key >= 0 && off >= 0 && off < 32 && ((off & 15) >> 2) == gq;
      const int word = ((off >> 4) & 1) * 2 + ((off >> 1) & 1);
      const uint32_t mask = own ? (0xffffu << (16 * (off & 1))) : 0u;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t ins = (off & 1) ? (svv[dt] << 16) : svv[dt];
        uint4& v = vf[buf][dt];
        v.x = word == 0 ? ((v.x & ~mask) | (ins & mask)) : v.x;
        v.y = word == 1 ? ((v.y & ~mask) | (ins & mask)) : v.y;
        v.z = word == 2 ? ((v.z & ~mask) | (ins & mask)) : v.z;
        v.w = word == 3 ? ((v.w & ~mask) | (ins & mask)) : v.w;
      }
    }
    f32x4_t sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KST; ++st) {
        acc = mfma_bf16(kf[buf][kt][st], qf[st][2], acc);
        acc = mfma_bf16(kf[buf][kt][st], qf[st][1], acc);
        acc = mfma_bf16(kf[buf][kt][st], qf[st][0], acc);
      }
      sc[kt] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 16 * kt + 4 * gq + r;
        const float v = key < clen && key < k_hi ? sc[kt][r] * scale : -INFINITY;
        sc[kt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const bool live = mn != -INFINITY;
    const float corr = live ? expf(m - mn) : 1.f;
    float ps = 0.f;
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = live ? expf(sc[kt][r] - mn) : 0.f;
        ps += pv;
        ph[4 * kt + r] = f2bf(pv);
        pl[4 * kt + r] = f2bf(pv - __uint_as_float(ph[4 * kt + r] << 16));
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * corr + ps;
    m = mn;
    const uint4 bh = make_uint4(ph[0] | ph[1] << 16, ph[2] | ph[3] << 16, ph[4] | ph[5] << 16, ph[6] | ph[7] << 16);
    const uint4 bl = make_uint4(pl[0] | pl[1] << 16, pl[2] | pl[3] << 16, pl[4] | pl[5] << 16, pl[6] | pl[7] << 16);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[dt][r] *= corr;
      o[dt] = mfma_bf16(vf[buf][dt], bl, o[dt]);
      o[dt] = mfma_bf16(vf[buf][dt], bh, o[dt]);
    }
  };
  // two blocks in flight per wave
  if (j_lo < j_hi) {
    for (int j = j_lo; j < j_hi; j += 2) {
      load(1, j + 1);
      block(0, j);
      if (j + 1 < j_hi) {
        load(0, j + 2);
        block(1, j + 1);
      }
    }
  }

  // merge the four waves: mg[w][col] = {m, l, o[HD]}
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mg[w][c][2 + 16 * dt + 4 * gq + r] = o[dt][r];
  if (gq == 0) { mg[w][c][0] = m; mg[w][c][1] = l; }
  __syncthreads();
  for (int t = threadIdx.x; t < ncol * HD; t += blockDim.x) {
    const int cc = t / HD, d = t % HD;
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kAttnWaves; ++u) M = fmaxf(M, mg[u][cc][0]);
    float L = 0.f, a = 0.f;
#pragma unroll
    for (int u = 0; u < kAttnWaves; ++u) {
      const float f = mg[u][cc][0] == -INFINITY ? 0.f : expf(mg[u][cc][0] - M);
      L += mg[u][cc][1] * f;
      a += mg[u][cc][2 + d] * f;
    }
    const int row = cc / G, head = g * G + cc % G;
    if (nsplit == 1) {
      out[(size_t)row * os + (size_t)head * HD + d] = a / L;
    } else {
      float* rec = partials + ((((size_t)slot * hkv + g) * kMaxSplit + s) * 16 + cc) * PW;
      if (d == 0) { rec[0] = M; rec[1] = L; }
      rec[2 + d] = a;
    }
  }
}

// workgroups of the merge per (problem, kv head): one thread per (column, dim)
constexpr int merge_parts(int hd) { return (16 * hd + kAttnWaves * 64 - 1) / (kAttnWaves * 64); }

template <typename T, int HD, int GMAX>
void launch_valu(dim3 grid, hipStream_t st, const AttnProb* probs, int nprob, const float* pq,
                 int q_stride, float* pout, int out_stride, const void* pK, const void* pV,
                 int pos0, int G, int hkv, int max_ctx, int split, float* part, bool merge,
                 LaunchEv ev) {
  LaunchEv e1{ev.start, merge ? nullptr : ev.stop}, e2{nullptr, ev.stop};
  SPD_LAUNCH(e1, (attn_kernel<T, HD, GMAX>), grid, dim3(kAttnWaves * 64), 0, st, probs, nprob,
             pq, q_stride, pout, out_stride, pK, pV, pos0, G, hkv, max_ctx, split, part);
  if (merge)
    SPD_LAUNCH(e2, (attn_merge_kernel<HD>), dim3(nprob * hkv * merge_parts(HD)),
               dim3(kAttnWaves * 64), 0, st, probs, G, hkv, G, part);
}

template <int HD>
void launch_mfma(bool sib, dim3 grid, hipStream_t st, const AttnProb* probs, int nprob, const float* pq,
                 int q_stride, float* pout, int out_stride, const void* pK, const void* pV,
                 int pos0, int prows, int G, int hkv, int max_ctx, int split, float* part,
                 bool merge, LaunchEv ev) {
  LaunchEv e1{ev.start, merge ? nullptr : ev.stop}, e2{nullptr, ev.stop};
  if (sib)
    SPD_LAUNCH(e1, (attn_mfma_kernel<HD, true>), grid, dim3(kAttnWaves * 64), 0, st, probs, nprob,
               pq, q_stride, pout, out_stride, pK, pV, pos0, prows, G, hkv, max_ctx, split, part);
  else
    SPD_LAUNCH(e1, (attn_mfma_kernel<HD, false>), grid, dim3(kAttnWaves * 64), 0, st, probs, nprob,
               pq, q_stride, pout, out_stride, pK, pV, pos0, prows, G, hkv, max_ctx, split, part);
  if (merge)
    SPD_LAUNCH(e2, (attn_merge_kernel<HD>), dim3(nprob * hkv * merge_parts(HD)),
               dim3(kAttnWaves * 64), 0, st, probs, G, hkv, 16, part);
}

// grid: workgroups; prows: prompt rows in prefill mode (probs == nullptr)
hipError_t dispatch(bool bf16, dim3 grid, hipStream_t st, const AttnProb* probs, int nprob,
                    const float* pq, int q_stride, float* pout, int out_stride, const void* pK,
                    const void* pV, int pos0, int prows, int hq, int hkv, int hd, int max_ctx,
                    int split, float* part, bool merge, LaunchEv ev = {}, bool sib = false) {
  const int G = hq / hkv;
  if (bf16) {
#define SPD_ATTN_CASE(HDV)                                                                    \
    if (hd == HDV) {                                                                          \
      launch_mfma<HDV>(sib, grid, st, probs, nprob, pq, q_stride, pout, out_stride, pK, pV,   \
                       pos0, prows, G, hkv, max_ctx, split, part, merge, ev);                 \
      return hipGetLastError();                                                               \
    }
    SPD_ATTN_CASE(16)
    SPD_ATTN_CASE(32)
    SPD_ATTN_CASE(64)
    SPD_ATTN_CASE(80)
    SPD_ATTN_CASE(128)
#undef SPD_ATTN_CASE
    return hipErrorInvalidValue;
  }
#define SPD_ATTN_CASE(HDV)                                                                   \
  if (hd == HDV) {                                                                           \
    if (G <= 4)                                                                              \
      launch_valu<float, HDV, 4>(grid, st, probs, nprob, pq, q_stride, pout, out_stride, pK, \
                                 pV, pos0, G, hkv, max_ctx, split, part, merge, ev);         \
    else                                                                                     \
      launch_valu<float, HDV, 16>(grid, st, probs, nprob, pq, q_stride, pout, out_stride, pK,\
                                  pV, pos0, G, hkv, max_ctx, split, part, merge, ev);        \
    return hipGetLastError();                                                                \
  }
  SPD_ATTN_CASE(16)
  SPD_ATTN_CASE(32)
  SPD_ATTN_CASE(64)
  SPD_ATTN_CASE(80)
  SPD_ATTN_CASE(128)
#undef SPD_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool attn_supported_head_dim(int hd, bool bf16) {
  (void)bf16;
  return hd == 16 || hd == 32 || hd == 64 || hd == 80 || hd == 128;
}

hipError_t launch_attention(const AttnProb* d_probs, int nprob, int ntiles, bool bf16, int hq,
                            int hkv, int hd, int max_ctx, int split_len, bool any_split,
                            float* partials, hipStream_t st, LaunchEv ev, bool siblings) {
  if (ntiles <= 0) return hipSuccess;
  return dispatch(bf16, dim3(ntiles), st, d_probs, nprob, nullptr, 0, nullptr, 0, nullptr, nullptr,
                  0, 0, hq, hkv, hd, max_ctx, split_len, partials, any_split, ev, siblings);
}

hipError_t launch_attention_prefill(const float* q, int q_stride, float* out, int out_stride,
                                    const void* K, const void* V, int pos0, int P, bool bf16,
                                    int hq, int hkv, int hd, int max_ctx, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  const int split = 1 << 30;
  // bf16: one workgroup per (16 / G prompt rows, kv head); fp32: per (row, kv head)
  const int R = bf16 ? 16 / (hq / hkv) : 1;
  const int groups = (P + R - 1) / R;
  return dispatch(bf16, dim3(groups * hkv), st, nullptr, 0, q, q_stride, out, out_stride, K, V,
                  pos0, P, hq, hkv, hd, max_ctx, split, nullptr, false);
}

int attn_rows_per_problem(bool bf16, int hq, int hkv) { return bf16 ? 16 / (hq / hkv) : 1; }

// splits per (problem, kv head): the merge keeps every split's value in registers
int attn_max_split() { return kMaxSplit; }

}  // namespace spd
