// Prefill GEMMs: C[P][N] (= or +=) A[P][K] * W[N][K]^T with fp32 activations A
// and weights W in bf16 or f32, both operands K-major. bf16 weights go to the bf16
// matrix cores with A split into three bf16 terms (gemm_x3_kernel, below); f32 weights,
// and shapes it does not take, use the fp32 kernel that follows.
//
// Activations stay fp32 (no bf16 rounding of GEMM inputs), so the prefill
// feeds the same values into the caches as one-position decode would, up to
// fp32 rounding order. The contraction runs on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32): a 128x128 block tile of four waves, each wave
// 64x64 = 4x4 MFMA tiles; K is staged through LDS 16 at a time and bf16
// weights are widened to fp32 on the way into LDS.
#include "spd_internal.h"

namespace spd {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16, LDK = BK + 1;

template <typename T>
__device__ __forceinline__ void stage_w(float* dst, const T* W, int n0, int k0, int N, int K,
                                        int tid) {
  // 128 rows x 16 k: bf16 -> one 16-byte load (8 values) per thread per half tile
  if constexpr (sizeof(T) == 2) {
    for (int c = tid; c < BN * (BK / 8); c += 256) {
      const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int gn = n0 + r, gk = k0 + kc;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (gn < N && gk < K) u = *reinterpret_cast<const uint4*>(W + (size_t)gn * K + gk);
      float* d = dst + r * LDK + kc;
      d[0] = bf16_lo(u.x); d[1] = bf16_hi(u.x); d[2] = bf16_lo(u.y); d[3] = bf16_hi(u.y);
      d[4] = bf16_lo(u.z); d[5] = bf16_hi(u.z); d[6] = bf16_lo(u.w); d[7] = bf16_hi(u.w);
    }
  } else {
    for (int c = tid; c < BN * (BK / 4); c += 256) {
      const int r = c / (BK / 4), kc = (c % (BK / 4)) * 4;
      const int gn = n0 + r, gk = k0 + kc;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gn < N && gk < K) u = *reinterpret_cast<const float4*>(W + (size_t)gn * K + gk);
      float* d = dst + r * LDK + kc;
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(const float* __restrict__ A, int lda,
                                                    const T* __restrict__ W, float* __restrict__ C,
                                                    int ldc, int P, int N, int K, int accumulate) {
  __shared__ float As[BM * LDK];
  __shared__ float Bs[BN * LDK];
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int c = tid; c < BM * (BK / 4); c += 256) {
      const int r = c / (BK / 4), kc = (c % (BK / 4)) * 4;
      const int gr = m0 + r, gk = k0 + kc;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gr < P && gk < K) u = *reinterpret_cast<const float4*>(A + (size_t)gr * lda + gk);
      float* d = As + r * LDK + kc;
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
    stage_w<T>(Bs, W, n0, k0, N, K, tid);
    __syncthreads();
    // 16x16x4 operands: lane l supplies A[row l%16][k l/16] and B[k l/16][col l%16]
    const int rr = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 4) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[(wm + i * 16 + rr) * LDK + ks + kq];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[(wn + j * 16 + rr) * LDK + ks + kq];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D layout of a 16x16 MFMA tile: lane l holds rows 4*(l/16)+e of column l%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm + i * 16 + (lane >> 4) * 4 + e;
        if (row >= P) continue;
        float* cp = C + (size_t)row * ldc + col;
        *cp = accumulate ? *cp + acc[i][j][e] : acc[i][j][e];
      }
    }
}

// ---- bf16 weights on the bf16 matrix cores ---------------------------------------------
// C = A W^T with the fp32 A split into three bf16 terms (split3) and W exact in bf16:
// three v_mfma_f32_16x16x32_bf16 per 32 columns of K (smallest term first) give the fp32
// product to fp32 rounding, at the bf16 matrix rate. Block tile 128x128 of four waves, each
// 64x64 (4x4 tiles of 16x16). K goes through LDS in chunks of 32, double-buffered: the next
// chunk's global loads are in flight while the waves run the current chunk's 48 MFMAs.
// Lane l reads 16 bytes at row l % 16, columns 8 (l / 16) .. + 7 of an A plane and of W,
// the operand layout of the instruction; rows are padded by 8 bf16 in LDS.
constexpr int XM = 128, XN = 128, XK = 32, XLD = XK + 8;

__global__ __launch_bounds__(256) void gemm_x3_kernel(const float* __restrict__ A, int lda,
                                                      const uint16_t* __restrict__ W,
                                                      float* __restrict__ C, int ldc, int P,
                                                      int N, int K, int accumulate) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][3][XM * XLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][XN * XLD];
  const int m0 = blockIdx.y * XM, n0 = blockIdx.x * XN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  // staging: A chunk = 128 rows x 8 float4 (4 per thread), W chunk = 128 rows x 4 pieces of
  // 8 bf16 (2 per thread); addresses are clamped into the matrices, values past them zeroed
  float4 ra[4];
  uint4 rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 3, c = (q & 7) * 4;
      const int gr = min(m0 + r, P - 1), gk = min(k0 + c, K - 4);
      ra[i] = load_g4(A + (size_t)gr * lda + gk);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, r = q >> 2, c = (q & 3) * 8;
      const int gn = min(n0 + r, N - 1), gk = min(k0 + c, K - 8);
      rb[i] = load_g16(W + (size_t)gn * K + gk);
    }
  };
  auto stage = [&](int buf, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 3, c = (q & 7) * 4;
      const bool ok = m0 + r < P && k0 + c < K;
      const float4 x = ok ? ra[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      uint32_t h0, d0, l0, h1, d1, l1, h2, d2, l2, h3, d3, l3;
      split3(x.x, h0, d0, l0);
      split3(x.y, h1, d1, l1);
      split3(x.z, h2, d2, l2);
      split3(x.w, h3, d3, l3);
      const int o = r * XLD + c;
      lds_store8(&As[buf][0][o], h0 | h1 << 16, h2 | h3 << 16);
      lds_store8(&As[buf][1][o], d0 | d1 << 16, d2 | d3 << 16);
      lds_store8(&As[buf][2][o], l0 | l1 << 16, l2 | l3 << 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, r = q >> 2, c = (q & 3) * 8;
      const bool ok = n0 + r < N && k0 + c < K;
      const uint4 w = ok ? rb[i] : make_uint4(0u, 0u, 0u, 0u);
      const int o = r * XLD + c;
      lds_store8(&Bs[buf][o], w.x, w.y);
      lds_store8(&Bs[buf][o + 4], w.z, w.w);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  gload(0);
  stage(0, 0);
  __syncthreads();
  const int rr = lane & 15, kq = (lane >> 4) * 8;
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += XK) {
    const bool more = k0 + XK < K;
    if (more) gload(k0 + XK);
    uint4 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = lds_load16(&Bs[buf][(wn + 16 * j + rr) * XLD + kq]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (wm + 16 * i + rr) * XLD + kq;
      const uint4 a0 = lds_load16(&As[buf][0][o]);
      const uint4 a1 = lds_load16(&As[buf][1][o]);
      const uint4 a2 = lds_load16(&As[buf][2][o]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma_bf16(a2, b[j], acc[i][j]);
        acc[i][j] = mfma_bf16(a1, b[j], acc[i][j]);
        acc[i][j] = mfma_bf16(a0, b[j], acc[i][j]);
      }
    }
    if (more) stage(buf ^ 1, k0 + XK);   // the other buffer: every wave left it at the last barrier
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm + i * 16 + (lane >> 4) * 4 + e;
        if (row >= P) continue;
        float* cp = C + (size_t)row * ldc + col;
        *cp = accumulate ? *cp + acc[i][j][e] : acc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_gemm(const float* A, int lda, const void* W, float* C, int ldc, int P, int N,
                       int K, bool accumulate, bool bf16, hipStream_t st) {
  if (P <= 0 || N <= 0) return hipSuccess;
  const bool x3 = bf16 && K >= 8 && K % 8 == 0 && lda % 4 == 0 && ((uintptr_t)A & 15) == 0 &&
                  ((uintptr_t)W & 15) == 0;
  if (x3) {
    hipLaunchKernelGGL(gemm_x3_kernel, dim3((N + XN - 1) / XN, (P + XM - 1) / XM), dim3(256), 0,
                       st, A, lda, static_cast<const uint16_t*>(W), C, ldc, P, N, K,
                       accumulate ? 1 : 0);
    return hipGetLastError();
  }
  dim3 grid((N + BN - 1) / BN, (P + BM - 1) / BM);
  if (bf16)
    hipLaunchKernelGGL(gemm_kernel<uint16_t>, grid, dim3(256), 0, st, A, lda,
                       static_cast<const uint16_t*>(W), C, ldc, P, N, K, accumulate ? 1 : 0);
  else
    hipLaunchKernelGGL(gemm_kernel<float>, grid, dim3(256), 0, st, A, lda,
                       static_cast<const float*>(W), C, ldc, P, N, K, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace spd
