// LM-head statistics, draft selection and streaming verification.
//
// vocab_stats: one pass over up to two logit rows (the target's exiting token
//   and the PDM's newest row, both produced by one sweep of the tied head):
//   per block max / argmax / runner-up (the near-tie gap), sum of exp(z/T),
//   and the Gumbel-perturbed argmax z/T + G used to sample.
// finalize (one block): merges the partials in a fixed order, selects the
//   draft, and verifies the position after the exiting token: greedy match at
//   T = 0; at T > 0 rejection sampling (accept iff u q(d) < p(d), Leviathan et
//   al. 2023, the paper's section 3.5 assumption on the pith.science review).
// residual (rejections at T > 0 only): y = argmax over {p > q} of
//   log(p - q) + G, per-block partials merged by a one-block kernel.
// nucleus (T > 0 and top_p < 1): the top-p set of each row, the smallest prefix of
//   the tokens in order of decreasing probability (lower id first on ties) whose
//   mass reaches top_p (Holtzman et al. 2019), found by selection rather than a
//   sort; then the Gumbel draw restricted to the set, one partial per block.
#include <climits>

#include "spd_internal.h"

namespace spd {
namespace {

struct Stat {
  float max, second;
  int arg;
  float sum;
  float gmax, gsecond;
  int garg;
};

__device__ __forceinline__ Stat stat_empty() {
  return Stat{-INFINITY, -INFINITY, INT_MAX, 0.f, -INFINITY, -INFINITY, INT_MAX};
}

// top-2 merge with lowest-id tie-break on the arg
__device__ __forceinline__ void top2_merge(float& m1, float& s1, int& a1, float m2, float s2, int a2) {
  const float lo = fminf(m1, m2);
  float sec = fmaxf(lo, fmaxf(s1, s2));
  if (m2 > m1 || (m2 == m1 && a2 < a1)) { m1 = m2; a1 = a2; }
  s1 = sec;
}

__device__ __forceinline__ Stat merge(Stat a, const Stat& b, float invT) {
  // sum of exp((z - max) / T): rescale both to the larger max
  const float M = fmaxf(a.max, b.max);
  float sum = 0.f;
  if (a.max != -INFINITY) sum += a.sum * expf((a.max - M) * invT);
  if (b.max != -INFINITY) sum += b.sum * expf((b.max - M) * invT);
  top2_merge(a.max, a.second, a.arg, b.max, b.second, b.arg);
  a.sum = sum;
  top2_merge(a.gmax, a.gsecond, a.garg, b.gmax, b.gsecond, b.garg);
  return a;
}

__device__ __forceinline__ VocabPartial to_partial(const Stat& s) {
  VocabPartial p;
  p.max = s.max; p.second = s.second; p.arg = s.arg; p.sum = s.sum;
  p.gmax = s.gmax; p.gsecond = s.gsecond; p.garg = s.garg; p.pad = 0;
  return p;
}
__device__ __forceinline__ Stat from_partial(const VocabPartial& p) {
  return Stat{p.max, p.second, p.arg, p.sum, p.gmax, p.gsecond, p.garg};
}

// Tree reduction of one Stat per thread over a 1024-thread block (fixed order).
__device__ Stat block_reduce(Stat s, float invT, Stat* sh) {
  const int t = threadIdx.x;
  sh[t] = s;
  __syncthreads();
  for (int off = blockDim.x / 2; off > 0; off >>= 1) {
    if (t < off) sh[t] = merge(sh[t], sh[t + off], invT);
    __syncthreads();
  }
  Stat r = sh[0];
  __syncthreads();
  return r;
}

// ---- the best W + 1 scores of a row (draft trees) ---------------------------------
// A list holds kTopL (score, id) pairs, best first: higher score, lower id on ties.
constexpr int kTopL = kMaxWidth + 1;
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}
__device__ __forceinline__ void top_clear(float* s, int* id) {
#pragma unroll
  for (int j = 0; j < kTopL; ++j) { s[j] = -INFINITY; id[j] = INT_MAX; }
}
__device__ __forceinline__ void top_insert(float* s, int* id, float v, int i) {
  if (!better(v, i, s[kTopL - 1], id[kTopL - 1])) return;   // the common case: not in the list
#pragma unroll
  for (int j = 0; j < kTopL; ++j) {
    if (better(v, i, s[j], id[j])) {
      const float tv = s[j]; const int ti = id[j];
      s[j] = v; id[j] = i; v = tv; i = ti;
    }
  }
}
// The block's best kTopL of every thread's list (each thread passes its own, best first):
// each wave pops its best head kTopL times (butterfly reductions, the same order in every
// wave), then wave 0 pops the best of the waves' lists the same way. The result lands in
// os / oid (written by thread 0).
__device__ __forceinline__ void top_block(const float* s, const int* id, float* ws, int* wid,
                                          float* os, int* oid) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int head = 0;
  for (int k = 0; k < kTopL; ++k) {
    float bs = head < kTopL ? s[0] : -INFINITY;
    int bi = head < kTopL ? id[0] : INT_MAX;
#pragma unroll
    for (int j = 1; j < kTopL; ++j)
      if (j == head) { bs = s[j]; bi = id[j]; }
    float ms = bs;
    int mi = bi;
    for (int o = 32; o > 0; o >>= 1) {
      const float s2 = __shfl_xor(ms, o);
      const int i2 = __shfl_xor(mi, o);
      if (better(s2, i2, ms, mi)) { ms = s2; mi = i2; }
    }
    if (bi == mi && bs == ms && mi != INT_MAX) ++head;   // ids are distinct: one lane pops
    if (lane == 0) { ws[w * kTopL + k] = ms; wid[w * kTopL + k] = mi; }
  }
  __syncthreads();
  // wave 0 merges the waves' lists (at most 128 entries, two per lane) by the same pops
  if (w == 0) {
    const int n = (int)(blockDim.x >> 6) * kTopL;
    float h0 = lane < n ? ws[lane] : -INFINITY, h1 = lane + 64 < n ? ws[lane + 64] : -INFINITY;
    int j0 = lane < n ? wid[lane] : INT_MAX, j1 = lane + 64 < n ? wid[lane + 64] : INT_MAX;
    if (better(h1, j1, h0, j0)) {
      const float t = h0; h0 = h1; h1 = t;
      const int ti = j0; j0 = j1; j1 = ti;
    }
    for (int k = 0; k < kTopL; ++k) {
      float ms = h0;
      int mi = j0;
      for (int o = 32; o > 0; o >>= 1) {
        const float s2 = __shfl_xor(ms, o);
        const int i2 = __shfl_xor(mi, o);
        if (better(s2, i2, ms, mi)) { ms = s2; mi = i2; }
      }
      if (mi == j0 && ms == h0 && mi != INT_MAX) { h0 = h1; j0 = j1; h1 = -INFINITY; j1 = INT_MAX; }
      if (lane == 0) { os[k] = ms; oid[k] = mi; }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kVocabBlock) void vocab_stats_kernel(const VocabDesc* __restrict__ dd,
                                                                   VocabPartial* __restrict__ part) {
  __shared__ Stat sh[kVocabBlock];
  const VocabDesc& d = *dd;
  const int chunk = (d.V + d.nblocks - 1) / d.nblocks;
  const int lo = blockIdx.x * chunk, hi = min(d.V, lo + chunk);
  for (int r = 0; r < 2; ++r) {
    if (!d.active[r]) continue;
    const float* z = d.logits[r];
    Stat s = stat_empty();
    const bool gum = d.gumbel_stream[r] != 0 && !d.nucleus;
    // draft trees: the draft row's best scores (logits at T = 0, Gumbel scores at T > 0)
    const bool tops = r == 1 && d.topw > 1;
    float ts[kTopL];
    int ti[kTopL];
    top_clear(ts, ti);
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
      const float v = z[i];
      if (d.sampled) {
        if (v > s.max) { s.sum = s.sum * expf((s.max - v) * d.inv_temp) + 1.f; }
        else { s.sum += expf((v - s.max) * d.inv_temp); }
      }
      if (v > s.max) { s.second = s.max; s.max = v; s.arg = i; }
      else if (v > s.second) { s.second = v; }
      float g = v;
      if (gum) {
        const float u = rng_uniform(d.seed, d.gumbel_stream[r], d.gumbel_pos[r], (unsigned long long)i);
        g = v * d.inv_temp + gumbel_of(u);
        if (g > s.gmax) { s.gsecond = s.gmax; s.gmax = g; s.garg = i; }
        else if (g > s.gsecond) { s.gsecond = g; }
      }
      if (tops) top_insert(ts, ti, g, i);
    }
    const Stat b = block_reduce(s, d.inv_temp, sh);
    if (threadIdx.x == 0) part[r * d.nblocks + blockIdx.x] = to_partial(b);
    if (tops) {
      __shared__ float tws[kVocabBlock / 64 * kTopL], tos[kTopL];
      __shared__ int twi[kVocabBlock / 64 * kTopL], toi[kTopL];
      top_block(ts, ti, tws, twi, tos, toi);
      if (threadIdx.x == 0) {
        VocabTop& o = d.top[blockIdx.x];
#pragma unroll
        for (int j = 0; j < kTopL; ++j) { o.s[j] = tos[j]; o.id[j] = toi[j]; }
      }
    }
  }
}

// ---- top-p set ---------------------------------------------------------------
// Masses are fixed point: w(z) = floor(exp((z - max) / T) 2^40) as a 64-bit integer,
// so every sum is exact and independent of the order of the additions. A token is in
// the set iff the mass ahead of it is < top_p W (W: the row's total), i.e. < ceil(top_p W).
// Four launches, both rows at once:
//   hist   (kNucBlocks blocks per row) the mass of each slice over depth bins of
//          (max - z) / T, 256 per unit up to depth 16 (a bin index is monotone in z;
//          fine bins keep the crossing bin's tokens few enough for LDS);
//   merge  the slices' histograms, bin by bin;
//   cand   every block finds the bin where the running mass crosses the threshold
//          (a block scan of the merged histogram) and lists its slice's tokens in it;
//   select (one block per row) four 8-bit radix passes over the order-preserving
//          integer key of the listed logits, each keeping the digit where the running
//          mass crosses, give zb, the logit of the last token kept; of the tokens tied
//          at zb the first j* = ceil(rest / w(zb)) in id order are kept, and when that
//          splits the ties a bisection over ids names the last one.
constexpr int kNucBins = 4096;       // depth bins
constexpr int kNucBlocks = 64;       // slices per row
constexpr int kNucThreads = 256;
constexpr int kNucMergeThreads = 64;
constexpr int kNucList = 8192;       // listed tokens the select kernel keeps in LDS
constexpr int kNucBatch = 10;        // logits a thread loads at once (a slice is <= 10 per thread
                                     // at V = 151936)
static_assert(kNucBlocks * kNucBins * 8 * 2 == kNucPartBytes, "top-p histogram scratch");
static_assert(kNucBins * 8 * 2 == kNucHistBytes, "top-p merged histogram scratch");
static_assert(kNucBins % kNucMergeThreads == 0, "merge grid");
typedef unsigned long long u64;

__device__ __forceinline__ int nuc_bin(float z, float M, float invT) {
  // explicitly rounded operations: every evaluation of a token's bin gives the same bin
  const float b = __fmul_rn(__fmul_rn(__fsub_rn(M, z), invT), 256.f);
  return b < (float)(kNucBins - 1) ? (int)b : kNucBins - 1;
}
__device__ __forceinline__ u64 nuc_weight(float z, float M, float invT) {
  return (u64)(expf((z - M) * invT) * 1099511627776.f);   // 2^40
}
// order-preserving key of a float (-0 and +0 share the key of +0)
__device__ __forceinline__ uint32_t f_key(float z) {
  uint32_t b = __float_as_uint(z);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ u64 shfl_up64(u64 v, int d) {
  const int lo = __shfl_up((int)(uint32_t)v, d), hi = __shfl_up((int)(uint32_t)(v >> 32), d);
  return ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Exclusive prefix sum over the block in thread order; `total` gets the block's sum.
// wsum holds one entry per wave.
__device__ u64 block_excl_scan(u64 v, u64* wsum, u64& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u64 inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = shfl_up64(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  u64 before = 0, tot = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    const u64 s = wsum[i];
    if (i < w) before += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// The row's largest logit, from the statistics partials (red: one float per wave).
__device__ float row_max(const VocabPartial* part, int r, int nblocks, float* red) {
  float m = -INFINITY;
  for (int i = threadIdx.x; i < nblocks; i += blockDim.x) m = fmaxf(m, part[r * nblocks + i].max);
  m = wave_max(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float M = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) M = fmaxf(M, red[i]);
  return M;
}

struct Crossing {
  int bin;      // the bin holding the last token kept
  u64 above;    // mass of the bins before it
  u64 T;        // ceil(top_p W), at least 1 and at most W
};
// PER consecutive bins per thread, read once into registers.
template <int PER>
__device__ Crossing find_crossing(const u64* hist, float top_p, u64* wsum, Crossing* sh) {
  const int b0 = threadIdx.x * PER;
  if (threadIdx.x == 0) sh->bin = kNucBins - 1;
  u64 h[PER];
  u64 mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    h[j] = b0 + j < kNucBins ? hist[b0 + j] : 0ull;
    mine += h[j];
  }
  u64 W;
  u64 run = block_excl_scan(mine, wsum, W);
  const double thr = ceil((double)top_p * (double)W);
  const u64 T = thr < 1.0 ? 1ull : (thr >= (double)W ? W : (u64)thr);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (run < T && T <= run + h[j]) { sh->bin = b0 + j; sh->above = run; }
    run += h[j];
  }
  __syncthreads();
  Crossing c = *sh;
  c.T = T;
  __syncthreads();
  return c;
}

__global__ __launch_bounds__(kNucThreads) void nuc_hist_kernel(const VocabDesc* __restrict__ dd,
                                                                const VocabPartial* __restrict__ part) {
  __shared__ u64 hist[kNucBins];
  __shared__ float red[kNucThreads / 64];
  const VocabDesc& d = *dd;
  const int r = blockIdx.y, b = blockIdx.x;
  if (!d.active[r]) return;
  for (int i = threadIdx.x; i < kNucBins; i += blockDim.x) hist[i] = 0;
  const float M = row_max(part, r, d.nblocks, red), invT = d.inv_temp;
  if (b == 0 && threadIdx.x == 0) d.nuc_max[r] = M;    // for the kernels that follow
  const int C = (d.V + kNucBlocks - 1) / kNucBlocks;
  const int lo = min(d.V, b * C), hi = min(d.V, lo + C);
  const float* z = d.logits[r];
  // loads in batches of kNucBatch per thread, issued before any of them is used
  for (int base = lo + threadIdx.x; base < hi; base += kNucBatch * kNucThreads) {
    float v[kNucBatch];
#pragma unroll
    for (int k = 0; k < kNucBatch; ++k) {
      const int i = base + k * kNucThreads;
      v[k] = i < hi ? z[i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kNucBatch; ++k)
      if (base + k * kNucThreads < hi) atomicAdd(&hist[nuc_bin(v[k], M, invT)], nuc_weight(v[k], M, invT));
  }
  __syncthreads();
  u64* out = d.nuc_part + ((size_t)r * kNucBlocks + b) * kNucBins;
  for (int i = threadIdx.x; i < kNucBins; i += blockDim.x) out[i] = hist[i];
}

__global__ __launch_bounds__(kNucMergeThreads) void nuc_merge_kernel(const VocabDesc* __restrict__ dd) {
  const VocabDesc& d = *dd;
  const int r = blockIdx.y;
  if (!d.active[r]) return;
  const int bin = blockIdx.x * blockDim.x + threadIdx.x;
  const u64* p = d.nuc_part + (size_t)r * kNucBlocks * kNucBins + bin;
  u64 s = 0;
  for (int b = 0; b < kNucBlocks; ++b) s += p[(size_t)b * kNucBins];
  d.nuc_hist[r * kNucBins + bin] = s;
}

__global__ __launch_bounds__(kNucThreads) void nuc_cand_kernel(const VocabDesc* __restrict__ dd,
                                                                const VocabPartial* __restrict__ part) {
  __shared__ u64 wsum[kNucThreads / 64];
  __shared__ Crossing sh;
  __shared__ int s_n;
  const VocabDesc& d = *dd;
  const int r = blockIdx.y, b = blockIdx.x;
  if (!d.active[r]) return;
  if (threadIdx.x == 0) s_n = 0;
  const float M = d.nuc_max[r], invT = d.inv_temp;
  const Crossing c = find_crossing<kNucBins / kNucThreads>(d.nuc_hist + r * kNucBins, d.top_p,
                                                           wsum, &sh);
  const int C = (d.V + kNucBlocks - 1) / kNucBlocks;
  const int lo = min(d.V, b * C), hi = min(d.V, lo + C);
  const float* z = d.logits[r];
  int2* seg = d.nuc_cand + (size_t)r * d.V + lo;     // room for hi - lo entries
  for (int base = lo + threadIdx.x; base < hi; base += kNucBatch * kNucThreads) {
    float v[kNucBatch];
#pragma unroll
    for (int k = 0; k < kNucBatch; ++k) {
      const int i = base + k * kNucThreads;
      v[k] = i < hi ? z[i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kNucBatch; ++k) {
      const int i = base + k * kNucThreads;
      if (i < hi && nuc_bin(v[k], M, invT) == c.bin) {
        const int n = atomicAdd(&s_n, 1);
        seg[n] = make_int2(__float_as_int(v[k]), i);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) d.nuc_cnt[r * kNucBlocks + b] = s_n;
}

__global__ __launch_bounds__(kVocabBlock) void nuc_select_kernel(const VocabDesc* __restrict__ dd,
                                                                  const VocabPartial* __restrict__ part) {
  __shared__ float lz[kNucList];
  __shared__ int lid[kNucList];
  __shared__ u64 hist[256];
  __shared__ u64 wsum[kVocabBlock / 64];
  __shared__ Crossing sh;
  __shared__ int s_off[kNucBlocks + 1];
  __shared__ int s_digit;
  __shared__ u64 s_above, s_mass;
  const VocabDesc& d = *dd;
  const int r = blockIdx.x;
  if (!d.active[r]) return;
  const int V = d.V, t = threadIdx.x, nthr = blockDim.x;
  const float M = d.nuc_max[r], invT = d.inv_temp;
  const Crossing c = find_crossing<kNucBins / kVocabBlock>(d.nuc_hist + r * kNucBins, d.top_p,
                                                           wsum, &sh);
  const int C = (V + kNucBlocks - 1) / kNucBlocks;
  const int2* cand = d.nuc_cand + (size_t)r * V;
  // where each slice's listed tokens start (the counts load in parallel, then one wave scans)
  if (t < kNucBlocks) s_off[t + 1] = d.nuc_cnt[r * kNucBlocks + t];
  if (t == 0) { s_off[0] = 0; s_digit = 0; s_above = c.above; s_mass = 0; }
  __syncthreads();
  if (t < 64) {
    static_assert(kNucBlocks == 64, "one wave scans the slice counts");
    int v = s_off[t + 1];
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if ((t & 63) >= o) v += u;
    }
    s_off[t + 1] = v;
  }
  __syncthreads();
  const int total = s_off[kNucBlocks];
  const bool in_lds = total <= kNucList;
  if (in_lds) {
    // listed token j lives in slice b with s_off[b] <= j < s_off[b + 1]
    for (int j = t; j < total; j += nthr) {
      int lo = 0, hi = kNucBlocks - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= j) lo = mid; else hi = mid - 1;
      }
      const int2 e = cand[(size_t)lo * C + (j - s_off[lo])];
      lz[j] = __int_as_float(e.x);
      lid[j] = e.y;
    }
  }
  __syncthreads();
  // every listed token once, over the block: f(logit, id)
  auto visit = [&](auto&& f) {
    if (in_lds) {
      for (int j = t; j < total; j += nthr) f(lz[j], lid[j]);
    } else {
      for (int b = 0; b < kNucBlocks; ++b) {
        const int n = s_off[b + 1] - s_off[b];
        const int2* sg = cand + (size_t)b * C;
        for (int j = t; j < n; j += nthr) {
          const int2 e = sg[j];
          f(__int_as_float(e.x), e.y);
        }
      }
    }
  };
  const u64 T = c.T;
  u64 above = c.above;
  uint32_t prefix = 0;
  u64 tie_mass = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (t < 256) hist[t] = 0;
    __syncthreads();
    const uint32_t hmask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
    visit([&](float v, int) {
      const uint32_t k = f_key(v);
      if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], nuc_weight(v, M, invT));
    });
    __syncthreads();
    // thread t holds digit 255 - t: the prefix sum in thread order is the mass of larger digits
    const u64 hv = t < 256 ? hist[255 - t] : 0ull;
    u64 tot;
    const u64 e = block_excl_scan(hv, wsum, tot);
    if (t < 256 && above + e < T && T <= above + e + hv) {
      s_digit = 255 - t; s_above = above + e; s_mass = hv;
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    above = s_above;
    tie_mass = s_mass;
    __syncthreads();
  }
  const float zb = key_f(prefix);
  // ties at zb (all of them are listed: equal logits share a bin): keep the first j*
  const u64 wb = nuc_weight(zb, M, invT);
  const u64 ties = wb ? tie_mass / wb : 0ull;
  const u64 js = wb ? (T - above + wb - 1) / wb : 0ull;
  int id_cut = INT_MAX;
  if (js < ties) {
    // smallest id X with at least j* tied tokens of id <= X
    int lo = 0, hi = V - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      u64 n = 0;
      visit([&](float v, int id) { n += (v == zb && id <= mid) ? 1ull : 0ull; });
      u64 all;
      (void)block_excl_scan(n, wsum, all);
      if (all >= js) hi = mid; else lo = mid + 1;
    }
    id_cut = lo;
  }
  if (t == 0) {
    NucleusCut out;
    out.zb = zb;
    out.id_cut = id_cut;
    out.lse = (float)((double)M * invT + log((double)(above + js * wb)) - 40.0 * 0.69314718055994531);
    out.pad = 0;
    *d.cut[r] = out;
  }
}

// Gumbel-max over each row's top-p set: per block top-2 of z/T + G over the set, into the
// Gumbel fields of the row's statistics partials.
__global__ __launch_bounds__(kVocabBlock) void nucleus_gumbel_kernel(const VocabDesc* __restrict__ dd,
                                                                      VocabPartial* __restrict__ part) {
  __shared__ Stat sh[kVocabBlock];
  const VocabDesc& d = *dd;
  const int chunk = (d.V + d.nblocks - 1) / d.nblocks;
  const int lo = blockIdx.x * chunk, hi = min(d.V, lo + chunk);
  for (int r = 0; r < 2; ++r) {
    if (!d.active[r] || d.gumbel_stream[r] == 0) continue;
    const float* z = d.logits[r];
    const NucleusCut c = *d.cut[r];
    Stat s = stat_empty();
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
      const float v = z[i];
      if (!in_cut(v, i, c)) continue;
      const float u = rng_uniform(d.seed, d.gumbel_stream[r], d.gumbel_pos[r], (unsigned long long)i);
      const float g = v * d.inv_temp + gumbel_of(u);
      if (g > s.gmax) { s.gsecond = s.gmax; s.gmax = g; s.garg = i; }
      else if (g > s.gsecond) { s.gsecond = g; }
    }
    const Stat b = block_reduce(s, 1.f, sh);
    if (threadIdx.x == 0) {
      VocabPartial& p = part[r * d.nblocks + blockIdx.x];
      p.gmax = b.gmax; p.gsecond = b.gsecond; p.garg = b.garg;
    }
  }
}

__device__ Stat merge_row(const VocabPartial* part, int nblocks, float invT, Stat* sh) {
  Stat s = stat_empty();
  for (int i = threadIdx.x; i < nblocks; i += blockDim.x) s = merge(s, from_partial(part[i]), invT);
  return block_reduce(s, invT, sh);
}

__global__ __launch_bounds__(kVocabBlock) void finalize_kernel(const FinalizeDesc* __restrict__ fd) {
  __shared__ Stat sh[kVocabBlock];
  const FinalizeDesc& f = *fd;
  const bool sampled = f.temp > 0.f;
  const int W = f.W > 0 ? f.W : 1;           // token ring rows: slot * W + candidate
  Stat t = stat_empty(), q = stat_empty();
  if (f.mode == 1 || f.exited) t = merge_row(f.part, f.nblocks, f.inv_temp, sh);
  if (f.mode == 0) q = merge_row(f.part + f.nblocks, f.nblocks, f.inv_temp, sh);
  // draft trees: the draft row's best W + 1 scores over every slice's list
  __shared__ float tws[kVocabBlock / 64 * kTopL], tos[kTopL];
  __shared__ int twi[kVocabBlock / 64 * kTopL], toi[kTopL];
  if (f.mode == 0 && W > 1) {
    float ls[kTopL];
    int li[kTopL];
    top_clear(ls, li);
    for (int b = threadIdx.x; b < f.nblocks; b += blockDim.x)
#pragma unroll
      for (int j = 0; j < kTopL; ++j) top_insert(ls, li, f.top[b].s[j], f.top[b].id[j]);
    top_block(ls, li, tws, twi, tos, toi);
  }
  if (threadIdx.x != 0) return;
  Verdict v{};
  v.committed = -1;
  v.verified_draft = -1;
  v.lse_t = t.max * f.inv_temp + logf(t.sum);
  if (f.nucleus && (f.mode == 1 || f.exited)) v.lse_t = f.cut_t->lse;
  if (f.mode == 1) {
    int y;
    bool flag;
    if (sampled) { y = t.garg; flag = (t.gmax - t.gsecond) < kNearTie; }
    else { y = t.arg; flag = (t.max - t.second) < kNearTie; }
    v.first_token = y;
    v.flags = flag ? 1 : 0;
    f.tok_ring[(f.dpos % f.ring) * W] = y;
    *f.verdict = v;
    *f.host_verdict = v;
    return;
  }
  // draft for position dpos: the best candidate (the only one when W = 1)
  int d;
  bool dflag;
  if (W > 1) {
    d = toi[0];
    dflag = false;
    for (int j = 0; j < W; ++j) dflag = dflag || (tos[j] - tos[j + 1]) < kNearTie;
  } else if (sampled) { d = q.garg; dflag = (q.gmax - q.gsecond) < kNearTie; }
  else { d = q.arg; dflag = (q.max - q.second) < kNearTie; }
  v.lse_q = f.nucleus ? f.cut_q->lse : q.max * f.inv_temp + logf(q.sum);
  *f.lse_q_new = v.lse_q;
  if (f.forced_mode) {
    const int j = f.dpos - f.forced_base;
    if (j >= 0 && j < f.forced_len) {
      const int ref = f.forced_ref[j];
      const float u = rng_uniform(f.seed, RNG_FORCE, f.dpos, 0);
      d = (u < f.forced_p) ? ref : (ref + 1) % f.V;
      dflag = false;
    }
  }
  v.draft = d;
  v.flags = dflag ? 2 : 0;
  v.accepted_index = -1;
  const int drow = (f.dpos % f.ring) * W;
  f.tok_ring[drow] = d;
  for (int j = 1; j < W; ++j) f.tok_ring[drow + j] = toi[j];
  if (f.exited) {
    v.exited = 1;
    // the candidates at v: this step's drafts when the exiting token was alone (then v is
    // dpos and their ring rows were just written)
    const int vrow = (f.v % f.ring) * W;
    const int dv = f.tok_ring[vrow];
    v.verified_draft = dv;
    v.target_arg = t.arg;
    if (!sampled) {
      const int y = t.arg;
      int idx = -1;
      for (int j = 0; j < W; ++j)
        if (idx < 0 && f.tok_ring[vrow + j] == y) idx = j;
      v.committed = y;
      v.accepted = idx >= 0;
      v.accepted_index = idx;
      if ((t.max - t.second) < kNearTie) v.flags |= 1;
      f.tok_ring[vrow] = y;
    } else {
      float pd = expf(f.zt[dv] * f.inv_temp - v.lse_t);
      float qd = expf(f.zq_v[dv] * f.inv_temp - *f.lse_q_v);
      if (f.nucleus) {
        if (!in_cut(f.zt[dv], dv, *f.cut_t)) pd = 0.f;
        if (!in_cut(f.zq_v[dv], dv, *f.cut_q_v)) qd = 0.f;
      }
      const float u = rng_uniform(f.seed, RNG_ACC, f.v, 0);
      v.p_d = pd;
      v.q_d = qd;
      v.accepted = (u * qd < pd);
      if (fabsf(u * qd - pd) < kNearTie * qd) v.flags |= 1;
      if (v.accepted) { v.committed = dv; v.accepted_index = 0; }
      else if (W > 1) v.need_rrs = 1;       // the later candidates' rounds (tree_rounds_kernel)
      else v.need_residual = 1;
    }
  }
  *f.verdict = v;
  *f.host_verdict = v;
}

// Residual sample after a rejection at T > 0: every block writes the Gumbel
// top-2 of its slice of log(p - q) + G to part[2 * nblocks + b] ...
__global__ __launch_bounds__(kVocabBlock) void residual_kernel(const FinalizeDesc* __restrict__ fd,
                                                                VocabPartial* __restrict__ part) {
  __shared__ Stat sh[kVocabBlock];
  const FinalizeDesc& f = *fd;
  if (!f.verdict->need_residual) return;
  const float lse_t = f.verdict->lse_t;
  const float lse_q = *f.lse_q_v;
  const int chunk = (f.V + f.nblocks - 1) / f.nblocks;
  const int lo = blockIdx.x * chunk, hi = min(f.V, lo + chunk);
  const bool nuc = f.nucleus != 0;
  NucleusCut ct{}, cq{};
  if (nuc) { ct = *f.cut_t; cq = *f.cut_q_v; }
  Stat s = stat_empty();
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const float zt = f.zt[i], zq = f.zq_v[i];
    const float p = nuc && !in_cut(zt, i, ct) ? 0.f : expf(zt * f.inv_temp - lse_t);
    const float qq = nuc && !in_cut(zq, i, cq) ? 0.f : expf(zq * f.inv_temp - lse_q);
    const float r = p - qq;
    if (r > 0.f) {
      const float u = rng_uniform(f.seed, RNG_RES, f.v, (unsigned long long)i);
      const float g = logf(r) + gumbel_of(u);
      if (g > s.gmax) { s.gsecond = s.gmax; s.gmax = g; s.garg = i; }
      else if (g > s.gsecond) { s.gsecond = g; }
    }
  }
  const Stat b = block_reduce(s, 1.f, sh);
  if (threadIdx.x == 0) part[2 * f.nblocks + blockIdx.x] = to_partial(b);
}

// ... and one block merges them in block order and commits the sample.
__global__ __launch_bounds__(kVocabBlock) void residual_final_kernel(
    const FinalizeDesc* __restrict__ fd, const VocabPartial* __restrict__ part) {
  __shared__ Stat sh[kVocabBlock];
  const FinalizeDesc& f = *fd;
  if (!f.verdict->need_residual) return;
  Stat m = stat_empty();
  for (int i = threadIdx.x; i < f.nblocks; i += blockDim.x)
    m = merge(m, from_partial(part[2 * f.nblocks + i]), 1.f);
  m = block_reduce(m, 1.f, sh);
  int y = m.garg;
  bool flag = (m.gmax - m.gsecond) < kNearTie;
  if (y == INT_MAX) {
    // no token has p > q in floating point (the two distributions agree to rounding), so
    // max(0, p - q) has no mass: commit the target's argmax instead, flagged as a near-tie
    // (every thread sees the same reduced result, so the whole block takes this branch)
    const Stat t = merge_row(f.part, f.nblocks, f.inv_temp, sh);
    y = t.arg;
    flag = true;
  }
  if (threadIdx.x == 0) {
    Verdict* v = f.verdict;
    v->committed = y;
    if (flag) v->flags |= 1;
    f.tok_ring[(f.v % f.ring) * (f.W > 0 ? f.W : 1)] = y;
    *f.host_verdict = *v;
  }
}

// The final draw of the tree rounds when every candidate was rejected, handed from the
// rounds kernel (one block) to a pass over the vocabulary on many blocks: R_W(x) =
// max(0, A_W p(x) - B_W q(x)) off the candidates, Rc at the candidates; p and q are the ones
// the first round stored (pq). It sits in the scratch right after pq ([2][V] floats).
struct TreeRes {
  float AW, BW;
  int cand[kMaxWidth];
  float Rc[kMaxWidth];
  int W;
  int flag;       // a near-tie already met in the rounds
  int pending;    // 1: the draw is still to be made
};
__device__ __forceinline__ TreeRes* tree_res_of(const FinalizeDesc& f) {
  return reinterpret_cast<TreeRes*>(f.pq + 2 * (size_t)f.V);
}

// Draft trees at T > 0, after finalize rejected the first candidate: the remaining rounds of
// recursive rejection sampling, in one block. Round i tests candidate c_i, proposed from q_i
// (q without c_0 .. c_{i-1}, renormalised), against r_i = R_i / Z_i, where R_1 = max(0, p - q)
// and R_{i+1} = max(0, R_i / Z_i - q_i) (R_0 = p, Z_0 = 1): accept iff u_i q_i(c_i) < r_i(c_i).
// If all rounds reject, y = argmax over R_W > 0 of log R_W(x) + G(x) (RES stream), which draws
// from r_W; a residual without mass commits the target's argmax, flagged. That draw, a pass of
// three logarithms per token, runs on many blocks (tree_res_kernel, tree_res_final_kernel).
//
// Off the candidates, q_j(x) = q(x) s_j with s_0 = 1, s_j = 1 / (1 - E_j) (E_j: the mass of
// c_0 .. c_{j-1}), and since max(0, max(0, a) / Z - b) = max(0, a / Z - b) for b >= 0, Z > 0,
// every R_i there is one clamp: R_i(x) = max(0, A_i p(x) - B_i q(x)), A_{i+1} = A_i / Z_i,
// B_{i+1} = B_i / Z_i + s_i (A_0 = 1, B_0 = 0). The W candidates follow the recursion itself.
// So a pass over the vocabulary costs two exponentials and a clamp per token; Z_i is the
// block's sum in a fixed order.
__global__ __launch_bounds__(kVocabBlock) void tree_rounds_kernel(const FinalizeDesc* __restrict__ fd) {
  __shared__ Stat sh[kVocabBlock];
  __shared__ float red[kVocabBlock / 64];
  const FinalizeDesc& f = *fd;
  Verdict* vd = f.verdict;
  if (!vd->need_rrs) return;
  const int W = f.W;
  const int vrow = (f.v % f.ring) * W;
  int cand[kMaxWidth];
  float qcand[kMaxWidth], pcand[kMaxWidth];
  const float lse_t = vd->lse_t, lse_q = *f.lse_q_v, invT = f.inv_temp;
#pragma unroll
  for (int j = 0; j < kMaxWidth; ++j) {
    cand[j] = j < W ? f.tok_ring[vrow + j] : -1;
    pcand[j] = j < W ? expf(f.zt[cand[j]] * invT - lse_t) : 0.f;
    qcand[j] = j < W ? expf(f.zq_v[cand[j]] * invT - lse_q) : 0.f;
  }
  float Z[kMaxWidth + 1], S[kMaxWidth + 1], A[kMaxWidth + 1], B[kMaxWidth + 1];
  float Rc[kMaxWidth];                 // R_i at each candidate for the current round i
  Z[0] = 1.f; S[0] = 1.f; A[0] = 1.f; B[0] = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxWidth; ++k) Rc[k] = pcand[k];   // R_0 = p
  float E = 0.f;                                          // mass of the candidates so far
  int y = -1, idx = -1;
  bool flag = (vd->flags & 1) != 0;
  // R_i at the candidates from R_{i-1}: candidate k is out of q_{i-1} once k < i - 1
  auto step_cands = [&](int i) {
#pragma unroll
    for (int k = 0; k < kMaxWidth; ++k) {
      const float qj = k < i - 1 ? 0.f : qcand[k] * S[i - 1];
      Rc[k] = fmaxf(0.f, Rc[k] / Z[i - 1] - qj);
    }
  };
  auto is_cand = [&](int x, int& k) {
    k = -1;
#pragma unroll
    for (int j = 0; j < kMaxWidth; ++j)
      if (j < W && cand[j] == x) k = j;
    return k >= 0;
  };
  for (int i = 1; i < W && y < 0; ++i) {
    A[i] = A[i - 1] / Z[i - 1];
    B[i] = B[i - 1] / Z[i - 1] + S[i - 1];
    step_cands(i);
    float part = 0.f;
    // the first round evaluates p(x) and q(x) and keeps them; later passes read them back
    // (each thread reads only what it stored itself)
    if (i == 1) {
      for (int x = threadIdx.x; x < f.V; x += blockDim.x) {
        int k;
        if (is_cand(x, k)) continue;     // added below, once
        const float px = expf(f.zt[x] * invT - lse_t), qx = expf(f.zq_v[x] * invT - lse_q);
        f.pq[x] = px;
        f.pq[f.V + x] = qx;
        part += fmaxf(0.f, A[i] * px - B[i] * qx);
      }
    } else {
      for (int x = threadIdx.x; x < f.V; x += blockDim.x) {
        int k;
        if (is_cand(x, k)) continue;
        part += fmaxf(0.f, A[i] * f.pq[x] - B[i] * f.pq[f.V + x]);
      }
    }
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    float Zi = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) Zi += red[w];
#pragma unroll
    for (int k = 0; k < kMaxWidth; ++k)
      if (k < W) Zi += Rc[k];
    __syncthreads();
    if (!(Zi > 0.f)) { y = vd->target_arg; flag = true; break; }
    Z[i] = Zi;
    E += qcand[i - 1];
    S[i] = 1.f / (1.f - E);
    const float qc = qcand[i] * S[i];
    const float rc = Rc[i] / Zi;
    const float u = rng_uniform(f.seed, RNG_ACC, f.v, (unsigned long long)i);
    if (fabsf(u * qc - rc) < kNearTie * qc) flag = true;
    if (u * qc < rc) { y = cand[i]; idx = i; }
  }
  TreeRes* tr = tree_res_of(f);
  if (y < 0) {
    // every round rejected: y ~ r_W (R_W from Z_{W-1}, s_{W-1}), drawn by tree_res_kernel
    // and committed by tree_res_final_kernel
    const float AW = A[W - 1] / Z[W - 1], BW = B[W - 1] / Z[W - 1] + S[W - 1];
    step_cands(W);
    if (threadIdx.x == 0) {
      tr->AW = AW; tr->BW = BW; tr->W = W; tr->flag = flag;
#pragma unroll
      for (int k = 0; k < kMaxWidth; ++k) { tr->cand[k] = cand[k]; tr->Rc[k] = Rc[k]; }
      tr->pending = 1;
    }
    return;
  }
  if (threadIdx.x == 0) {
    tr->pending = 0;
    vd->committed = y;
    vd->accepted = idx >= 0;
    vd->accepted_index = idx;
    if (flag) vd->flags |= 1;
    f.tok_ring[vrow] = y;
    *f.host_verdict = *vd;
  }
}

// The final draw over the vocabulary, one slice per block: the largest log R_W(x) + G(x)
// (RES stream at (v, x)) of each slice, ties to the lower id, with the runner-up score.
__global__ __launch_bounds__(kVocabBlock) void tree_res_kernel(const FinalizeDesc* __restrict__ fd,
                                                               VocabPartial* __restrict__ part) {
  __shared__ Stat sh[kVocabBlock];
  const FinalizeDesc& f = *fd;
  const TreeRes& tr = *tree_res_of(f);
  if (!f.verdict->need_rrs || !tr.pending) return;
  const int chunk = (f.V + f.nblocks - 1) / f.nblocks;
  const int lo = blockIdx.x * chunk, hi = min(f.V, lo + chunk);
  Stat s = stat_empty();
  for (int x = lo + threadIdx.x; x < hi; x += blockDim.x) {
    int k = -1;
#pragma unroll
    for (int j = 0; j < kMaxWidth; ++j)
      if (j < tr.W && tr.cand[j] == x) k = j;
    float r = 0.f;
    if (k >= 0) {
#pragma unroll
      for (int j = 0; j < kMaxWidth; ++j)
        if (j == k) r = tr.Rc[j];
    } else {
      r = fmaxf(0.f, tr.AW * f.pq[x] - tr.BW * f.pq[f.V + x]);   // stored by the first round
    }
    if (r > 0.f) {
      const float g = logf(r) + gumbel_of(rng_uniform(f.seed, RNG_RES, f.v, (unsigned long long)x));
      if (g > s.gmax) { s.gsecond = s.gmax; s.gmax = g; s.garg = x; }
      else if (g > s.gsecond) { s.gsecond = g; }
    }
  }
  const Stat b = block_reduce(s, 1.f, sh);
  if (threadIdx.x == 0) part[2 * f.nblocks + blockIdx.x] = to_partial(b);
}

// ... one block merges the slices in block order and commits the draw (a residual without
// mass commits the target's argmax, flagged).
__global__ __launch_bounds__(kVocabBlock) void tree_res_final_kernel(
    const FinalizeDesc* __restrict__ fd, const VocabPartial* __restrict__ part) {
  __shared__ Stat sh[kVocabBlock];
  const FinalizeDesc& f = *fd;
  TreeRes* tr = tree_res_of(f);
  Verdict* vd = f.verdict;
  if (!vd->need_rrs || !tr->pending) return;
  Stat m = stat_empty();
  for (int i = threadIdx.x; i < f.nblocks; i += blockDim.x)
    m = merge(m, from_partial(part[2 * f.nblocks + i]), 1.f);
  m = block_reduce(m, 1.f, sh);
  int y;
  bool flag = tr->flag != 0;
  if (m.garg == INT_MAX) { y = vd->target_arg; flag = true; }
  else { y = m.garg; if ((m.gmax - m.gsecond) < kNearTie) flag = true; }
  if (threadIdx.x == 0) {
    tr->pending = 0;
    vd->committed = y;
    vd->accepted = 0;
    vd->accepted_index = -1;
    if (flag) vd->flags |= 1;
    f.tok_ring[(f.v % f.ring) * f.W] = y;
    *f.host_verdict = *vd;
  }
}

}  // namespace

hipError_t launch_vocab_stats(const VocabDesc* d_desc, int nblocks, VocabPartial* part,
                              hipStream_t st, LaunchEv ev) {
  SPD_LAUNCH(ev, vocab_stats_kernel, dim3(nblocks), dim3(kVocabBlock), 0, st, d_desc, part);
  return hipGetLastError();
}

hipError_t launch_nucleus(const VocabDesc* d_desc, int nblocks, VocabPartial* part,
                          hipStream_t st, LaunchEv ev) {
  const LaunchEv e1{ev.start, nullptr}, e0{nullptr, nullptr}, e2{nullptr, ev.stop};
  SPD_LAUNCH(e1, nuc_hist_kernel, dim3(kNucBlocks, 2), dim3(kNucThreads), 0, st, d_desc, part);
  SPD_LAUNCH(e0, nuc_merge_kernel, dim3(kNucBins / kNucMergeThreads, 2), dim3(kNucMergeThreads), 0,
             st, d_desc);
  SPD_LAUNCH(e0, nuc_cand_kernel, dim3(kNucBlocks, 2), dim3(kNucThreads), 0, st, d_desc, part);
  SPD_LAUNCH(e0, nuc_select_kernel, dim3(2), dim3(kVocabBlock), 0, st, d_desc, part);
  SPD_LAUNCH(e2, nucleus_gumbel_kernel, dim3(nblocks), dim3(kVocabBlock), 0, st, d_desc, part);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeDesc* d_desc, hipStream_t st, LaunchEv ev) {
  SPD_LAUNCH(ev, finalize_kernel, dim3(1), dim3(kVocabBlock), 0, st, d_desc);
  return hipGetLastError();
}

hipError_t launch_tree_rounds(const FinalizeDesc* d_desc, VocabPartial* part, int nblocks,
                              hipStream_t st, LaunchEv ev) {
  const LaunchEv e1{ev.start, nullptr}, e0{nullptr, nullptr}, e2{nullptr, ev.stop};
  SPD_LAUNCH(e1, tree_rounds_kernel, dim3(1), dim3(kVocabBlock), 0, st, d_desc);
  SPD_LAUNCH(e0, tree_res_kernel, dim3(nblocks), dim3(kVocabBlock), 0, st, d_desc, part);
  SPD_LAUNCH(e2, tree_res_final_kernel, dim3(1), dim3(kVocabBlock), 0, st, d_desc, part);
  return hipGetLastError();
}

hipError_t launch_residual_impl(const FinalizeDesc* d_desc, VocabPartial* part, int nblocks,
                                hipStream_t st, LaunchEv ev) {
  const LaunchEv e1{ev.start, nullptr}, e2{nullptr, ev.stop};
  SPD_LAUNCH(e1, residual_kernel, dim3(nblocks), dim3(kVocabBlock), 0, st, d_desc, part);
  SPD_LAUNCH(e2, residual_final_kernel, dim3(1), dim3(kVocabBlock), 0, st, d_desc, part);
  return hipGetLastError();
}

}  // namespace spd
