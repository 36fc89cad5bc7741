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
    const bool gum = d.gumbel_stream[r] != 0;
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
      const float v = z[i];
      if (d.sampled) {
        if (v > s.max) { s.sum = s.sum * expf((s.max - v) * d.inv_temp) + 1.f; }
        else { s.sum += expf((v - s.max) * d.inv_temp); }
      }
      if (v > s.max) { s.second = s.max; s.max = v; s.arg = i; }
      else if (v > s.second) { s.second = v; }
      if (gum) {
        const float u = rng_uniform(d.seed, d.gumbel_stream[r], d.gumbel_pos[r], (unsigned long long)i);
        const float g = v * d.inv_temp + gumbel_of(u);
        if (g > s.gmax) { s.gsecond = s.gmax; s.gmax = g; s.garg = i; }
        else if (g > s.gsecond) { s.gsecond = g; }
      }
    }
    const Stat b = block_reduce(s, d.inv_temp, sh);
    if (threadIdx.x == 0) part[r * d.nblocks + blockIdx.x] = to_partial(b);
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
  Stat t = stat_empty(), q = stat_empty();
  if (f.mode == 1 || f.exited) t = merge_row(f.part, f.nblocks, f.inv_temp, sh);
  if (f.mode == 0) q = merge_row(f.part + f.nblocks, f.nblocks, f.inv_temp, sh);
  if (threadIdx.x != 0) return;
  Verdict v{};
  v.committed = -1;
  v.verified_draft = -1;
  v.lse_t = t.max * f.inv_temp + logf(t.sum);
  if (f.mode == 1) {
    int y;
    bool flag;
    if (sampled) { y = t.garg; flag = (t.gmax - t.gsecond) < kNearTie; }
    else { y = t.arg; flag = (t.max - t.second) < kNearTie; }
    v.first_token = y;
    v.flags = flag ? 1 : 0;
    f.tok_ring[f.dpos % f.ring] = y;
    *f.verdict = v;
    *f.host_verdict = v;
    return;
  }
  // draft for position dpos
  int d;
  bool dflag;
  if (sampled) { d = q.garg; dflag = (q.gmax - q.gsecond) < kNearTie; }
  else { d = q.arg; dflag = (q.max - q.second) < kNearTie; }
  v.lse_q = q.max * f.inv_temp + logf(q.sum);
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
  f.tok_ring[f.dpos % f.ring] = d;
  if (f.exited) {
    v.exited = 1;
    const int dv = f.tok_ring[f.v % f.ring];
    v.verified_draft = dv;
    if (!sampled) {
      const int y = t.arg;
      v.committed = y;
      v.accepted = (y == dv);
      if ((t.max - t.second) < kNearTie) v.flags |= 1;
      if (!v.accepted) f.tok_ring[f.v % f.ring] = y;
    } else {
      const float pd = expf(f.zt[dv] * f.inv_temp - v.lse_t);
      const float qd = expf(f.zq_v[dv] * f.inv_temp - *f.lse_q_v);
      const float u = rng_uniform(f.seed, RNG_ACC, f.v, 0);
      v.p_d = pd;
      v.q_d = qd;
      v.accepted = (u * qd < pd);
      if (fabsf(u * qd - pd) < kNearTie * qd) v.flags |= 1;
      if (v.accepted) v.committed = dv;
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
  Stat s = stat_empty();
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const float p = expf(f.zt[i] * f.inv_temp - lse_t);
    const float qq = expf(f.zq_v[i] * f.inv_temp - lse_q);
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
  if (threadIdx.x == 0) {
    Verdict* v = f.verdict;
    v->committed = m.garg;
    if ((m.gmax - m.gsecond) < kNearTie) v->flags |= 1;
    f.tok_ring[f.v % f.ring] = m.garg;
    *f.host_verdict = *v;
  }
}

}  // namespace

hipError_t launch_vocab_stats(const VocabDesc* d_desc, int nblocks, VocabPartial* part,
                              hipStream_t st, LaunchEv ev) {
  SPD_LAUNCH(ev, vocab_stats_kernel, dim3(nblocks), dim3(kVocabBlock), 0, st, d_desc, part);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeDesc* d_desc, hipStream_t st, LaunchEv ev) {
  SPD_LAUNCH(ev, finalize_kernel, dim3(1), dim3(kVocabBlock), 0, st, d_desc);
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
