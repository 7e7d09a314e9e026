// Shared device building blocks of the Brand fold kernels (fold.hip: one
// workgroup per head, every operand in LDS; fold_joint.hip: one basis over
// a layer's KV heads, streamed a head at a time): LDS products on the matrix cores, blocked
// Cholesky, triangular solves, Householder QR of the core and the one-sided
// Jacobi SVD on its rows (internal linkage: each kernel file has its own copy).
#pragma once

#include <cfloat>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int kThreads = 512;
constexpr int kMaxSweeps = 40;
constexpr float kJacobiTol = 1.0e-6f;     // rotate while |y_p . y_q| > tol |y_p||y_q|
// Stop after a sweep whose largest |y_p . y_q| / (|y_p||y_q|) (before its
// rotations) was below this: the cyclic sweep leaves O(that^2) behind, which is
// at the fp32 floor of the inner products, so a further sweep only chases noise.
constexpr float kJacobiQuad = 1.0e-3f;
// First CholeskyQR pass: a pivot of the residual Gram G = Res Res^T is dropped
// when it is at most max(kGuardAbs ||A||_F^2, min(kGuard ||A||_F^2, kGuardRel tr G)).
// kGuard ||A||^2 keeps kept directions below condition number ~1/sqrt(kGuard)
// when the residual is large (it holds signal, as in the first folds); when
// the residual is small against A (steady state, and square when r = d - 64)
// that guard would drop real directions and move the leading subspace by
// ~5e-4, so the bound becomes relative to tr G = ||Res||_F^2 (condition number
// below ~1000, where CholeskyQR2 still ends orthonormal).  kGuardAbs drops
// only the rounding of the projection A - P B^T (~16 fp32 ulps of ||A||).
constexpr float kGuard = 1.0e-7f;
constexpr float kGuardRel = 1.0e-6f;
constexpr float kGuardAbs = 1.0e-12f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4(float *p, const float4 &v) { *reinterpret_cast<float4 *>(p) = v; }

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Sum over aligned groups of GS = 4 or 8 lanes (identical result in every
// lane of the group): DPP quad permutations, then the half-row mirror.
template <int GS>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(GS == 4 || GS == 8, "group size");
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (GS == 8)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

// A zero the compiler cannot see through.  Added to an LDS pointer before a
// fully unrolled loop, it keeps the base in one register with small
// immediate offsets, instead of one materialized absolute address per access
// (LDS offsets above 64 KiB do not fit the instruction's offset field).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// ---------------------------------------------------------------------------
// C(m, n) = sum_k A(m, k) B(k, n) over 16-byte-aligned LDS operands on the
// matrix cores (v_mfma_f32_16x16x4_f32: fp32 inputs, fp32 accumulation),
// each output handed once to out(m, n, value):
//   A(m, k) = A[m * lda + k] (AT = false)  or  A[k * lda + m] (AT = true)
//   B(k, n) = B[k * ldb + n] (BT = false)  or  B[n * ldb + k] (BT = true)
// 16 x 16 output tiles are dealt to waves wave, wave + nw, ... .  In each
// group of four MFMAs covering k0 .. k0 + 15, lane (j = lane % 16,
// g = lane / 16) supplies A(i0 + j, k) and B(k, n0 + j) for k = k0 + 4 g + m
// in MFMA m: every k once (the sum is order-free), with the lane's four A
// values contiguous when A is row-major and its four B values contiguous when
// B is given transposed.  Output rows 4 g .. 4 g + 3, column j of the tile are
// the lane's accumulator.  gemm_mfma_part lets two independent products share
// the workgroup's waves.
// ---------------------------------------------------------------------------
template <int M, int N, int K, bool AT, bool BT, typename Out>
__device__ __forceinline__ void gemm_mfma_part(const float *A, int lda, const float *B, int ldb, Out out,
                                               int wave, int nw) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 16 == 0, "16-wide tiles");
  constexpr int TN = N / 16, TILES = (M / 16) * TN;
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  for (int tile = wave; tile < TILES; tile += nw) {
    const int i0 = (tile / TN) * 16, n0 = (tile % TN) * 16;
    floatx4 acc = zero4();
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 16) {
      const int kb = k0 + 4 * g;
      float a[4], b[4];
      if constexpr (!AT) {
        const float4 v = ld4(A + (i0 + j) * lda + kb);
        a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = A[(kb + m) * lda + i0 + j];
      }
      if constexpr (BT) {
        const float4 v = ld4(B + (n0 + j) * ldb + kb);
        b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) b[m] = B[(kb + m) * ldb + n0 + j];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = mfma4(a[m], b[m], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) out(i0 + 4 * g + r, n0 + j, acc[r]);
  }
}

template <int M, int N, int K, bool AT, bool BT, typename Out>
__device__ __forceinline__ void gemm_mfma(const float *A, int lda, const float *B, int ldb, Out out) {
  gemm_mfma_part<M, N, K, AT, BT>(A, lda, B, ldb, out, (int)(threadIdx.x >> 6), kThreads / 64);
}

// ---------------------------------------------------------------------------
// The 64 x d block leaving the window, from the ring, as float rows in LDS
// (row stride LA).  Keys are stored [slot][d], values [d][slot].  Returns this
// thread's share of ||A||_F^2.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&v)[8]) {
  const float4 a = ld4(p), b = ld4(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t *p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

template <typename T, int LA>
__device__ float load_block(const T *ring, int X, int s0, int slots, float *sA) {
  constexpr int D = kHeadDim, TB = kBlock;
  float asq = 0.f;
  if (X == 0) {
    for (int i = threadIdx.x; i < TB * D / 8; i += kThreads) {
      const int t = i / (D / 8), f0 = (i % (D / 8)) * 8;
      float v[8];
      load8<T>(ring + (size_t)(s0 + t) * D + f0, v);
      st4(sA + t * LA + f0, make_float4(v[0], v[1], v[2], v[3]));
      st4(sA + t * LA + f0 + 4, make_float4(v[4], v[5], v[6], v[7]));
#pragma unroll
      for (int j = 0; j < 8; ++j) asq = fmaf(v[j], v[j], asq);
    }
  } else {
    for (int i = threadIdx.x; i < TB * D / 8; i += kThreads) {
      const int f = i / (TB / 8), t0 = (i % (TB / 8)) * 8;
      float v[8];
      load8<T>(ring + (size_t)f * slots + s0 + t0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sA[(t0 + j) * LA + f] = v[j];
        asq = fmaf(v[j], v[j], asq);
      }
    }
  }
  return asq;
}

// ---------------------------------------------------------------------------
// Lower Cholesky factor of the n x n matrix G (row stride ldg, lower part
// read), in place, by the whole workgroup, in blocks of 8 columns: every
// thread factors the 8 x 8 diagonal block in registers (the same values in
// all threads, no exchange), one thread per row below solves its 8 panel
// entries, then the trailing matrix takes the rank-8 update.  Three barriers
// per block.  A pivot <= tau drops its column (L_:j = 0), exactly as in the
// unblocked right-looking order.  L ends in the lower part of G (upper part
// zeroed), 1/L_jj (0 where dropped) in invd.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_rcp(float x) {
  float r = __builtin_amdgcn_rcpf(x);
  return r * fmaf(-x, r, 2.f);               // one Newton step
}

template <int n>
__device__ __forceinline__ void chol_lds(float *G, int ldg, float tau, float *invd) {
  constexpr int BS = 8, TPR = kThreads / n, KMAX = (n + TPR - 1) / TPR;
  static_assert(n % BS == 0 && kThreads % n == 0, "block shape");
  const int tid = threadIdx.x;
  const int ri = tid / TPR, rc = tid % TPR;     // trailing-update row and lane
  for (int J = 0; J < n; J += BS) {
    // diagonal block (lower part), right-looking in registers
    float l[BS][BS], inv[BS];
#pragma unroll
    for (int a = 0; a < BS; ++a)
#pragma unroll
      for (int c = 0; c <= a; ++c) l[a][c] = G[(J + a) * ldg + J + c];
#pragma unroll
    for (int c = 0; c < BS; ++c) {
      const float piv = l[c][c];
      const float ljj = piv > tau ? __builtin_amdgcn_sqrtf(piv) : 0.f;
      inv[c] = ljj > 0.f ? fast_rcp(ljj) : 0.f;
      l[c][c] = ljj;
#pragma unroll
      for (int a = c + 1; a < BS; ++a) l[a][c] *= inv[c];
#pragma unroll
      for (int a = c + 1; a < BS; ++a)
#pragma unroll
        for (int b = c + 1; b <= a; ++b) l[a][b] = fmaf(-l[a][c], l[b][c], l[a][b]);
    }
    // every wave has read the diagonal block (and, at J = 0, whatever the
    // caller read from G before this call) before it is overwritten
    __syncthreads();
#pragma unroll
    for (int a = 0; a < BS; ++a) {               // static indices keep l in registers
      if (tid == a) {
#pragma unroll
        for (int c = 0; c <= a; ++c) G[(J + a) * ldg + J + c] = l[a][c];
        invd[J + a] = inv[a];
      }
    }
    // panel: rows below the block, L_iJ = G_iJ L_JJ^{-T}
    for (int i = J + BS + tid; i < n; i += kThreads) {
      const float4 g0 = ld4(G + i * ldg + J), g1 = ld4(G + i * ldg + J + 4);
      float x[BS] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int c = 0; c < BS; ++c) {
        float acc = x[c];
#pragma unroll
        for (int k = 0; k < c; ++k) acc = fmaf(-x[k], l[c][k], acc);
        x[c] = acc * inv[c];
      }
      st4(G + i * ldg + J, make_float4(x[0], x[1], x[2], x[3]));
      st4(G + i * ldg + J + 4, make_float4(x[4], x[5], x[6], x[7]));
    }
    __syncthreads();
    // trailing update G_ik -= L_iJ . L_kJ  (J + 8 <= k <= i): reads first
    if (ri >= J + BS) {
      const float4 a0 = ld4(G + ri * ldg + J), a1 = ld4(G + ri * ldg + J + 4);
      constexpr int CH = KMAX < 8 ? KMAX : 8;     // reads batched per chunk
#pragma unroll
      for (int u0 = 0; u0 < KMAX; u0 += CH) {
        float4 k0[CH], k1[CH];
        float gi[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const int k = J + BS + rc + (u0 + u) * TPR;
          const bool ok = k <= ri;
          k0[u] = ok ? ld4(G + k * ldg + J) : make_float4(0.f, 0.f, 0.f, 0.f);
          k1[u] = ok ? ld4(G + k * ldg + J + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
          gi[u] = ok ? G[ri * ldg + k] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const int k = J + BS + rc + (u0 + u) * TPR;
          float v = gi[u];
          v = fmaf(-a0.x, k0[u].x, v); v = fmaf(-a0.y, k0[u].y, v);
          v = fmaf(-a0.z, k0[u].z, v); v = fmaf(-a0.w, k0[u].w, v);
          v = fmaf(-a1.x, k1[u].x, v); v = fmaf(-a1.y, k1[u].y, v);
          v = fmaf(-a1.z, k1[u].z, v); v = fmaf(-a1.w, k1[u].w, v);
          if (k <= ri) G[ri * ldg + k] = v;
        }
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < n * n; e += kThreads) {
    const int r = e / n, k = e % n;
    if (k > r) G[r * ldg + k] = 0.f;
  }
  __syncthreads();
}

// x <- L^{-1} x for a vector held in registers (L lower triangular, row
// stride ldl, invd = 1/diag or 0).  Four partial sums shorten the chains.
template <int n>
__device__ __forceinline__ void fwd_solve(float (&x)[n], const float *L0, int ldl,
                                          const float *invd0) {
  const int z = opaque_zero();
  const float *L = L0 + z, *invd = invd0 + z;
#pragma unroll
  for (int i = 0; i < n; ++i) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 + 4 <= i; k0 += 4) {
      const float4 l = ld4(L + i * ldl + k0);
      s[0] = fmaf(l.x, x[k0], s[0]);
      s[1] = fmaf(l.y, x[k0 + 1], s[1]);
      s[2] = fmaf(l.z, x[k0 + 2], s[2]);
      s[3] = fmaf(l.w, x[k0 + 3], s[3]);
    }
#pragma unroll
    for (int k = i & ~3; k < i; ++k) s[k & 3] = fmaf(L[i * ldl + k], x[k], s[k & 3]);
    x[i] = (x[i] - ((s[0] + s[1]) + (s[2] + s[3]))) * invd[i];
  }
}

// Linv <- L^{-1} (n x n, row strides ldl / ldi) from the factor L and invd
// that chol_lds left: column j is the forward solve of e_j, so Linv X equals
// the column-by-column forward solve of X, dropped pivots included (their rows
// of Linv are 0).  Applied to a head's tile as one product over the whole
// workgroup instead of one sequential solve per column per thread.
template <int n>
__device__ __forceinline__ void tri_inverse(const float *L, int ldl, const float *invd, float *Linv, int ldi) {
  const int tid = threadIdx.x;
  if (tid < n) {
    float x[n];
#pragma unroll
    for (int t = 0; t < n; ++t) x[t] = t == tid ? 1.f : 0.f;
    fwd_solve<n>(x, L, ldl, invd);
#pragma unroll
    for (int t = 0; t < n; ++t) Linv[t * ldi + tid] = x[t];
  }
}

// ---------------------------------------------------------------------------
// Householder QR of the core (N x NC, N >= NC, rows in LDS): the core is
// replaced by R (upper triangular, NC nonzero rows; rows past NC become zero).
// R has the core's singular values and right singular vectors, and the
// row Jacobi on R needs about a third fewer sweeps than on the core itself
// (Jacobi preconditioned by QR; Q is not needed, only right vectors are used).
// Thread (column c, quarter k) keeps rows [k N/4, (k+1) N/4) of column c in
// registers for the whole factorization.  Step j: every column right of j
// takes w = v_j^T x and x -= beta_j w v_j; then the four threads of column
// j+1 form the next reflector from their updated values (v to the other of
// two LDS buffers), so each step has one barrier.
// ---------------------------------------------------------------------------
template <int N, int NC, int LC>
__device__ __forceinline__ void qr_rows(float *core, float *vbuf0, float *vbuf1) {
  static_assert(N % 16 == 0 && N >= NC && 4 * NC <= kThreads, "QR shape");
  constexpr int RPC = N / 4;                              // rows per thread
  constexpr int STEPS = N - 1 < NC ? N - 1 : NC;          // reflectors
  __shared__ float s_beta[2];
  const int tid = threadIdx.x, c = tid >> 2, q = tid & 3, r0 = q * RPC;
  const bool act = tid < 4 * NC;
  float x[RPC];
  if (act) {
#pragma unroll
    for (int i = 0; i < RPC; ++i) x[i] = core[(r0 + i) * LC + c];
  }
  // reflector of column j (the calling quad holds column j): v = x over rows
  // >= j with v_j = x_j - alpha, alpha = -sign(x_j) |x|; beta = 2 / v^T v.
  // Column j becomes (alpha, 0, ...) from row j on.  Row tests are integer
  // arithmetic on the row offset (1.0 / 0.0 masks), not lane-mask compares.
  auto reflector = [&](int j, float *vb, int slot) {
    float ss = 0.f, xj = 0.f;
#pragma unroll
    for (int i = 0; i < RPC; ++i) {
      const int d = r0 + i - j;
      const float gt = (float)((unsigned)(-d) >> 31);                 // row > j
      const float eq = 1.f - gt - (float)((unsigned)d >> 31);         // row == j
      ss = fmaf(gt * x[i], x[i], ss);
      xj = fmaf(eq, x[i], xj);
    }
    ss = group_sum<4>(ss);
    xj = group_sum<4>(xj);
    const float nrm = __builtin_amdgcn_sqrtf(fmaf(xj, xj, ss));
    const float alpha = xj >= 0.f ? -nrm : nrm;
    const float beta = nrm > 0.f ? __builtin_amdgcn_rcpf(fmaf(nrm, fabsf(xj), nrm * nrm)) : 0.f;
    const float keep = nrm > 0.f ? 1.f : 0.f;
    float4 *vb4 = reinterpret_cast<float4 *>(vb + r0);
#pragma unroll
    for (int i4 = 0; i4 < RPC / 4; ++i4) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e, d = r0 + i - j;
        const float gt = (float)((unsigned)(-d) >> 31);
        const float eq = 1.f - gt - (float)((unsigned)d >> 31);
        v[e] = (gt + eq) * x[i] - eq * alpha;
        x[i] = fmaf(keep, eq * alpha - (gt + eq) * x[i], x[i]);
      }
      vb4[i4] = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (q == 0) s_beta[slot] = beta;
  };
  if (act && c == 0) reflector(0, vbuf0, 0);
  __syncthreads();
  for (int j = 0; j < STEPS; ++j) {
    const float4 *vb4 = reinterpret_cast<const float4 *>(((j & 1) ? vbuf1 : vbuf0) + r0);
    const float beta = s_beta[j & 1];
    if (act && c > j) {
      float v[RPC];
#pragma unroll
      for (int i4 = 0; i4 < RPC / 4; ++i4) {
        const float4 t = vb4[i4];
        v[4 * i4] = t.x; v[4 * i4 + 1] = t.y; v[4 * i4 + 2] = t.z; v[4 * i4 + 3] = t.w;
      }
      float w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RPC; ++i) w[i & 3] = fmaf(v[i], x[i], w[i & 3]);
      const float bw = beta * group_sum<4>((w[0] + w[1]) + (w[2] + w[3]));
#pragma unroll
      for (int i = 0; i < RPC; ++i) x[i] = fmaf(-bw, v[i], x[i]);
      if (c == j + 1 && j + 1 < STEPS) reflector(j + 1, (j & 1) ? vbuf0 : vbuf1, (j + 1) & 1);
    }
    __syncthreads();
  }
  if (act) {
#pragma unroll
    for (int i = 0; i < RPC; ++i) core[(r0 + i) * LC + c] = x[i];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// One-sided Jacobi on the N rows (length NC, stride LC) of `core`.  A pair
// (x, y) is rotated while |x.y| > tol |x||y|.  The squared row norms are
// computed at the start of each sweep and carried through its rotations
// (|x'|^2 = |x|^2 - t x.y, |y'|^2 = |y|^2 + t x.y), so a pair only forms x.y;
// carried over more than one sweep they drifted and stalled convergence on
// clusters of near-equal singular values.  Rows whose squared norm is below
// (64 eps)^2 times the largest are at the rounding level of the core and are
// left alone.
//
// Only the `keep` largest singular values and their right vectors are used.
// Each sweep therefore starts by choosing a leading set: the rows of the k
// largest norms, k >= keep the smallest count for which the squared norms of
// all other rows add up to less than kLeadMargin times the k-th largest.
// Pairs of two rows outside the set are skipped.  When the set's rows are
// orthogonal to each other and to every other row, the singular values of the
// other rows form a matrix of spectral norm at most the square root of that
// sum, below every leading norm, so the leading rows are the leading singular
// triplets however the other rows stand among themselves.  (In the cores of
// steady-state folds the non-leading rows are the residual directions, whose
// near-equal small singular values took most of the sweeps.)  The sweeps stop
// when one rotates nothing, or when its largest pair measure was below
// kJacobiQuad, and the final norms certify the split (leading minimum above
// the rest's sum); without the certificate every pair is taken from then on.
// Returns the number of rotating sweeps, or kMaxSweeps + 1 if it did not
// converge within kMaxSweeps.
// ---------------------------------------------------------------------------
constexpr float kLeadMargin = 0.25f;

template <int N, int NC, int LC>
__device__ int jacobi_rows(float *core, float *nrm, int *rank, int *lead, int keep) {
  constexpr int GS = NC % 32 == 0 ? 8 : 4;      // lanes per pair
  constexpr int NP = N / 2, CPT = NC / (4 * GS);
  static_assert(NC % (4 * GS) == 0 && N % 2 == 0 && N <= kThreads, "row shape");
  constexpr float kNegl = (64.f * FLT_EPSILON) * (64.f * FLT_EPSILON);
  __shared__ int s_flag, s_max, s_big, s_lead;
  __shared__ float s_red[2][kThreads / 64];
  const int tid = threadIdx.x, li = tid & (GS - 1);
  bool all_pairs = keep >= N;
  int sweep = 0;
  for (; sweep < kMaxSweeps; ++sweep) {
    if (tid == 0) { s_flag = 0; s_max = 0; s_big = 0; s_lead = N; }
    int big = 0;                         // a pair measure of this thread reached kJacobiQuad
    __syncthreads();
    if (tid < N) {
      const float *row = core + tid * LC;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll 4
      for (int i = 0; i < NC; i += 4) {
        const float4 v = ld4(row + i);
        s0 = fmaf(v.x, v.x, s0); s1 = fmaf(v.y, v.y, s1);
        s0 = fmaf(v.z, v.z, s0); s1 = fmaf(v.w, v.w, s1);
      }
      nrm[tid] = s0 + s1;
      atomicMax(&s_max, __float_as_int(s0 + s1));
    }
    __syncthreads();
    if (!all_pairs) {
      // rank by norm (ties by index), the norms in descending order, the
      // leading set from their tail sums
      float *sorted = reinterpret_cast<float *>(lead);
      if (tid < N) {
        const float nj = nrm[tid];
        int rk = 0;
#pragma unroll 4
        for (int i = 0; i < N; i += 4) {
          const float4 v = ld4(nrm + i);
          rk += (v.x > nj || (v.x == nj && i < tid)) + (v.y > nj || (v.y == nj && i + 1 < tid)) +
                (v.z > nj || (v.z == nj && i + 2 < tid)) + (v.w > nj || (v.w == nj && i + 3 < tid));
        }
        rank[tid] = rk;
        sorted[rk] = nj;
      }
      __syncthreads();
      if (tid < N && tid >= keep - 1) {
        float tail = 0.f;
        for (int i = tid + 1; i < N; ++i) tail += sorted[i];
        if (tail < kLeadMargin * sorted[tid]) atomicMin(&s_lead, tid + 1);
      }
      __syncthreads();
      if (tid < N) lead[tid] = rank[tid] < s_lead;
      // a leading set of more than half the rows saves at most a quarter of
      // the pairs: take every pair from here on
      all_pairs = 2 * s_lead > N;
      __syncthreads();
    }
    const float negl = kNegl * __int_as_float(s_max);
    const float inv_max = __int_as_float(s_max) > 0.f ? 1.f / __int_as_float(s_max) : 0.f;
    for (int k = 0; k < N - 1; ++k) {
      for (int g = tid / GS; g < NP; g += kThreads / GS) {
        int p, q;
        if (g == 0) { p = k; q = N - 1; }
        else { p = (k + g) % (N - 1); q = (k - g + N - 1) % (N - 1); }
        if (!all_pairs && !lead[p] && !lead[q]) continue;
        float *rp = core + p * LC + 4 * li, *rq = core + q * LC + 4 * li;
        float4 x[CPT], y[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          x[i] = ld4(rp + 4 * GS * i);
          y[i] = ld4(rq + 4 * GS * i);
        }
        float c0 = 0.f, c1 = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          c0 = fmaf(x[i].x, y[i].x, c0); c1 = fmaf(x[i].y, y[i].y, c1);
          c0 = fmaf(x[i].z, y[i].z, c0); c1 = fmaf(x[i].w, y[i].w, c1);
        }
        const float a = nrm[p], b = nrm[q], c = group_sum<GS>(c0 + c1);
        // the pair measure |c| / sqrt(a b) compared through squares (a, b > 0),
        // on values scaled by the largest squared row norm (no overflow)
        const float cs_ = c * inv_max, c2 = cs_ * cs_, ab = (a * inv_max) * (b * inv_max);
        const bool live = c != 0.f && a > negl && b > negl;
        if (live && c2 > (kJacobiQuad * kJacobiQuad) * ab) big = 1;
        if (live && c2 > (kJacobiTol * kJacobiTol) * ab) {
          // tan of the angle that zeroes the pair's inner product (the
          // smaller root), then cos by rsqrt refined with one Newton step
          const float zeta = (b - a) * __builtin_amdgcn_rcpf(2.f * c);
          const float az = fabsf(zeta);
          const float t = copysignf(az > 1.0e18f ? 0.5f * __builtin_amdgcn_rcpf(az)
                                                 : __builtin_amdgcn_rcpf(
                                                       az + __builtin_amdgcn_sqrtf(fmaf(az, az, 1.f))),
                                    zeta);
          const float s2 = fmaf(t, t, 1.f);
          float cs = __builtin_amdgcn_rsqf(s2);
          cs = cs * fmaf(-0.5f * s2 * cs, cs, 1.5f);
          const float sn = cs * t;
#pragma unroll
          for (int i = 0; i < CPT; ++i) {
            const float4 u = x[i], v = y[i];
            st4(rp + 4 * GS * i, make_float4(cs * u.x - sn * v.x, cs * u.y - sn * v.y,
                                         cs * u.z - sn * v.z, cs * u.w - sn * v.w));
            st4(rq + 4 * GS * i, make_float4(sn * u.x + cs * v.x, sn * u.y + cs * v.y,
                                         sn * u.z + cs * v.z, sn * u.w + cs * v.w));
          }
          if (li == 0) {
            s_flag = 1;
            nrm[p] = fmaf(-t, c, a);          // |x'|^2 = a - t c, |y'|^2 = b + t c
            nrm[q] = fmaf(t, c, b);
          }
        }
      }
      __syncthreads();
    }
    if (big) s_big = 1;
    __syncthreads();
    const int rotated = s_flag, any_big = s_big, n_lead = s_lead;
    __syncthreads();                           // read before the next sweep resets them
    if (rotated && any_big) continue;          // uniform: shared values
    if (all_pairs || n_lead >= N) return rotated ? sweep + 1 : sweep;
    // certificate: smallest leading norm above the sum of the others
    float mn = INFINITY, rest = 0.f;
    if (tid < N) {
      if (lead[tid]) mn = nrm[tid];
      else rest = nrm[tid];
    }
    for (int o = 32; o > 0; o >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      rest += __shfl_xor(rest, o);
    }
    if ((tid & 63) == 0) { s_red[0][tid >> 6] = mn; s_red[1][tid >> 6] = rest; }
    __syncthreads();
    mn = INFINITY; rest = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) { mn = fminf(mn, s_red[0][w]); rest += s_red[1][w]; }
    if (mn > rest) return rotated ? sweep + 1 : sweep;
    all_pairs = true;                          // uniform
  }
  return kMaxSweeps + 1;
}

}  // namespace

}  // namespace iskv
