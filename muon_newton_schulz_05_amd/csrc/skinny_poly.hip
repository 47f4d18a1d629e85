// skinny_poly.hip -- the m x m part of the skinny path (m <= 32): per slice,
// the normalisation and the Newton-Schulz rounds in the Gram space.
//
// With X_{t+1} = P_t X_t and P_t = a I + b A_t + c A_t^2, a polynomial in
// A_t = X_t X_t^T, the rounds need only A_{t+1} = P_t^2 A_t and the product
// Q = P_{k-1} ... P_0; the slice's output is then (s Q) M with
// s = 1 / (||M||_F + eps) ("关于分布式Muon的想法整合及讨论" §2 and §6: Gram matrix
// every round, normalisation by the whole matrix's sum of squares).  The
// Gram partials and sums of squares come from k_skinny_gram; s Q goes to
// k_skinny_apply.
#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

// One workgroup per slice; all m x m arithmetic in float64.  Products run on
// the float64 matrix cores: each of the four waves owns one 16 x 16 tile of
// the 32 x 32 result (16x16x4 float64 instruction: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] of each 4-wide k step and receives
// rows l / 16 + 4 r, r = 0..3, of column l % 16).  Everything outside the
// leading m x m block is kept at zero, so the padding never contributes.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_skinny_poly(SkinnyLaunch a) {
  // Double-buffered A and Q so that a product never overwrites its own input.
  __shared__ double A[2][32][33], Q[2][32][33], P[32][33], S[32][33];
  __shared__ double sh_s;
  const int z = blockIdx.x;
  const int m = a.m, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double ca = a.sc->a, cb = a.sc->b, cc = a.sc->c;
  const int ns = a.sc->ns_steps;
  const int mm = m * m;
  const int nch = a.n_chunks;

  // Sum of squares: wave 3 loads the chunk partials together and adds them
  // in chunk order (lane 0 walks the loaded values), alongside the Gram sums.
  if (wave == 3) {
    const float* sq = a.sq_parts + (int64_t)z * nch;
    double tot = 0.0;
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const double v = c0 + lane < nch ? (double)sq[c0 + lane] : 0.0;
      const int cnt = min(64, nch - c0);
      for (int u = 0; u < cnt; ++u) tot += __shfl(v, u);
    }
    if (lane == 0) {
      sh_s = 1.0 / (sqrt(tot) + (double)a.sc->eps);
      if (!isfinite(tot)) atomicOr(a.err, kErrNonFinite);
    }
  }
  // Gram sums: entry v = tid + 256 k of the compact m x m block, k < 4
  // (m <= 32); the loads of all of a thread's entries for kBatch chunks are
  // in flight together, and each entry is summed in chunk order.
  constexpr int kBatch = 10, kPer = 4;
  const double* parts = a.gram_parts + (int64_t)z * nch * mm;
  double sum[kPer] = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = 0; c0 < nch; c0 += kBatch) {
    double part[kPer][kBatch];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int v = tid + kThreads * k;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        part[k][u] = (v < mm && c0 + u < nch) ? parts[(int64_t)(c0 + u) * mm + v] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
#pragma unroll
      for (int u = 0; u < kBatch; ++u) sum[k] += part[k][u];
  }
  for (int e = tid; e < 1024; e += kThreads) {
    A[0][e >> 5][e & 31] = 0.0;
    Q[0][e >> 5][e & 31] = ((e >> 5) == (e & 31) && (e >> 5) < m) ? 1.0 : 0.0;
  }
  __syncthreads();
  const double s = sh_s;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int v = tid + kThreads * k;
    if (v < mm) A[0][v / m][v % m] = sum[k] * s * s;
  }
  __syncthreads();

  // Each wave owns one 16 x 16 tile of a 32 x 32 product; f64 matrix-core
  // layout: X lane l -> X[l mod 16][l / 16], Y lane l -> Y[l / 16][l mod 16],
  // result register r -> row l / 16 + 4 r, column l mod 16.
  const int ti = 16 * (wave >> 1), tj = 16 * (wave & 1);
  const int li = lane & 15, lk = lane >> 4;
  // All 32 columns of the zero-padded buffers: the operands of the eight
  // k-steps are read from LDS first, then the products run.
  auto prod = [&](const double (*X)[33], const double (*Y)[33]) {
    double xv[8], yv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      xv[q] = X[ti + li][4 * q + lk];
      yv[q] = Y[4 * q + lk][tj + li];
    }
    // Two independent chains (even and odd k-steps) keep two products in flight.
    f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < 8; q += 2) {
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[q], yv[q], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[q + 1], yv[q + 1], acc1, 0, 0, 0);
    }
    return acc0 + acc1;
  };
  int cur = 0;
  for (int it = 0; it < ns; ++it) {
    // P = a I + b A + c A^2
    {
      const f64x4_t t = prod(A[cur], A[cur]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti + lk + 4 * r, j = tj + li;
        P[i][j] = cb * A[cur][i][j] + cc * t[r] + ((i == j && i < m) ? ca : 0.0);
      }
    }
    __syncthreads();
    // Q <- P Q and, unless this is the last round, S = P P
    {
      const f64x4_t q = prod(P, Q[cur]);
      f64x4_t sp = {0.0, 0.0, 0.0, 0.0};
      if (it + 1 < ns) sp = prod(P, P);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ti + lk + 4 * r, j = tj + li;
        Q[cur ^ 1][i][j] = q[r];
        S[i][j] = sp[r];
      }
    }
    __syncthreads();
    if (it + 1 < ns) {
      // A <- P^2 A
      const f64x4_t t = prod(S, A[cur]);
#pragma unroll
      for (int r = 0; r < 4; ++r) A[cur ^ 1][ti + lk + 4 * r][tj + li] = t[r];
      __syncthreads();
    }
    cur ^= 1;
  }
  for (int e = tid; e < 1024; e += kThreads) a.qs[(int64_t)z * 1024 + e] = (float)(s * Q[cur][e >> 5][e & 31]);
}

}  // namespace

hipError_t launch_skinny_poly(const SkinnyLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_skinny_poly, dim3(a.count), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
