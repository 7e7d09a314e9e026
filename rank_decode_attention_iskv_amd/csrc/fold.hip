// Brand block-incremental SVD fold for gfx950 -- one workgroup per (selected
// layer, unit, K|V), every operand resident in LDS.
//
// Page: "iS-KV -- Basis-synchronized online low-rank KV compression -- What does
// it mean?" (learnaivisually.com), Jargon "Block-incremental SVD" and the drift
// paragraph: each 64-token block that ages out of the exact window joins the
// rank-r factorization in one update; the SVD is taken of an (r+64)-square core
// built from S and the block, so its cost is fixed however long the history.
//
// With the old history H = U diag(S) B^T (U orthonormal; the stored
// coefficients are U diag(S)) and a new block A (64 x d):
//   P = A B, Res = A - P B^T (projected twice);
//   Res = L Q with Q (64 x d) orthonormal rows, orthogonal to B (CholeskyQR2,
//     with a pivot guard that drops directions the fp32 Gram cannot resolve);
//   [H; A] = diag(U, I) K [B Q^T]^T,  K = [[diag S, 0], [P, A Q^T]]  ((r+64)^2);
//   K = U' diag(s') V'^T;  B_new = [B Q^T] V'[:, :r];  S_new = s'[:r];
//   old coefficients map by M = B^T B_new; the block's are A B_new.
// The SVD of K is a one-sided (Hestenes) Jacobi on the rows of K: rows are
// rotated pairwise (round-robin ordering, 8 lanes per pair) until mutually
// orthogonal, after which row j = s'_j v'_j^T.
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

// LDS plan in floats.  Row strides are padded by 4 floats: rows stay 16-byte
// aligned and consecutive rows start in different LDS banks.
template <int R>
struct FoldLayout {
  static constexpr int D = kHeadDim, TB = kBlock;
  static constexpr bool kRes = R < D;           // a residual space exists
  static constexpr int N = R + TB;              // core rows
  static constexpr int NC = kRes ? N : R;       // core columns
  static constexpr int LA = D + 4, LB = R + 4, LG = TB + 4, LC = NC + 4;
  static constexpr int oB = 0;                               // B (d x r), r < d only
  static constexpr int oQ = oB + (kRes ? D * LB : 0);        // Res -> Q; later B_new
  static constexpr int oA = oQ + cmax(TB * LA, D * LB);      // A
  static constexpr int oP = oA + TB * LA;                    // P
  static constexpr int oG = oP + TB * LB;                    // Gram / L / A Q^T
  static constexpr int end12 = oG + (kRes ? TB * LG : 0);
  static constexpr int oCore = kRes ? oA : 0;                // core over A, P, G
  static constexpr int endCore = oCore + N * LC;
  static constexpr int oNrm = cmax(end12, endCore);
  static constexpr int oSig = oNrm + N;
  static constexpr int oPerm = oSig + N;
  static constexpr int oAct = oPerm + N;
  static constexpr int oInv = oAct + R;
  static constexpr int oRem = oInv + cmax(TB, R);
  static constexpr int oVec = oRem + D;
  static constexpr int oDot = oVec + D;
  static constexpr int floats = oDot + R;
  static constexpr size_t bytes = (size_t)floats * 4;
  static_assert(oQ % 4 == 0 && oA % 4 == 0 && oP % 4 == 0 && oG % 4 == 0 && oCore % 4 == 0,
                "16-byte aligned regions");
};

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
// C(m, n) = sum_k A(m, k) B(k, n) over 16-byte-aligned operands, 4 x 4
// outputs per thread tile, handed to out(m, n, value).
//   A(m, k) = A[m * lda + k] (AT = false)  or  A[k * lda + m] (AT = true)
//   B(k, n) = B[k * ldb + n] (BT = false)  or  B[n * ldb + k] (BT = true)
// With BT the tile's four n are strided by N/4, so the lanes of a wave read
// rows that start in different banks.
// ---------------------------------------------------------------------------
template <int M, int N, int K, bool AT, bool BT, typename Out>
__device__ __forceinline__ void gemm4(const float *A, int lda, const float *B, int ldb, Out out) {
  static_assert(M % 4 == 0 && N % 4 == 0 && K % 4 == 0, "tile multiples");
  constexpr int TN = N / 4, TILES = (M / 4) * TN;
  for (int tile = threadIdx.x; tile < TILES; tile += kThreads) {
    const int m0 = (tile / TN) * 4, tn = tile % TN;
    int nn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) nn[j] = BT ? tn + j * TN : tn * 4 + j;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 4) {
      float a[4][4], b[4][4];     // a[m][k], b[k][n]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (!AT) {
          const float4 v = ld4(A + (m0 + i) * lda + k0);
          a[i][0] = v.x; a[i][1] = v.y; a[i][2] = v.z; a[i][3] = v.w;
        } else {
          const float4 v = ld4(A + (k0 + i) * lda + m0);
          a[0][i] = v.x; a[1][i] = v.y; a[2][i] = v.z; a[3][i] = v.w;
        }
        if constexpr (!BT) {
          const float4 v = ld4(B + (k0 + i) * ldb + nn[0]);
          b[i][0] = v.x; b[i][1] = v.y; b[i][2] = v.z; b[i][3] = v.w;
        } else {
          const float4 v = ld4(B + nn[i] * ldb + k0);
          b[0][i] = v.x; b[1][i] = v.y; b[2][i] = v.z; b[3][i] = v.w;
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i][kk], b[kk][j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) out(m0 + i, nn[j], acc[i][j]);
  }
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
// entries, then the trailing matrix takes the rank-8 update.  Two barriers
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

// One Brand fold of a unit's factor: the block's 64 rows come from load_A
// (fills sA, row stride LA, and returns this thread's share of ||A||_F^2;
// called twice), B and S are read from basis / sing, the new ones written to
// basis_out / sing_out (which may be the same arrays), M to msync and the
// block's coefficient rows to coef at rows n_c .. n_c + 63.
template <int R, typename T, typename Loader>
__device__ __forceinline__ void fold_one(const Model &M, float *lds, const float *basis, const float *sing,
                                         float *basis_out, float *sing_out, float *msync, T *coef,
                                         int64_t n_c, Loader load_A) {
  using Ly = FoldLayout<R>;
  constexpr int D = kHeadDim, TB = kBlock, N = Ly::N, NC = Ly::NC;
  constexpr int LA = Ly::LA, LB = Ly::LB, LG = Ly::LG, LC = Ly::LC;
  constexpr bool kRes = Ly::kRes;
  __shared__ float red[kThreads / 64];
  __shared__ int s_int[4];
  __shared__ float s_f[4];
  const int tid = threadIdx.x;

  float *sB = lds + Ly::oB, *sQ = lds + Ly::oQ, *sA = lds + Ly::oA, *sP = lds + Ly::oP;
  float *sG = lds + Ly::oG, *core = lds + Ly::oCore;
  float *sig = lds + Ly::oSig, *invd = lds + Ly::oInv;
  int *perm = reinterpret_cast<int *>(lds + Ly::oPerm);
  int *act = reinterpret_cast<int *>(lds + Ly::oAct);
  float *sBn = sQ;                  // B_new (d x LB) once Q is consumed
  const float *Bsrc;
  int ldB;
  if constexpr (kRes) { Bsrc = sB; ldB = LB; } else { Bsrc = basis; ldB = R; }

  // ---------------- phase 1: load, projection (twice) ----------------
  const float asq = load_A(sA);
  if constexpr (kRes) {
    for (int i = tid; i < D * R / 4; i += kThreads) {
      const int f = (4 * i) / R, c = (4 * i) % R;
      st4(sB + f * LB + c, ld4(basis + 4 * i));
    }
  }
  const float normA2 = block_sum(asq, red);     // barriers inside
  gemm4<TB, R, D, false, false>(sA, LA, Bsrc, ldB,
                                [&](int t, int c, float v) { sP[t * LB + c] = v; });
  __syncthreads();
  if constexpr (kRes) {
    // Res = A - P B^T
    gemm4<TB, D, R, false, true>(sP, LB, sB, LB, [&](int t, int f, float v) {
      sQ[t * LA + f] = sA[t * LA + f] - v;
    });
    __syncthreads();
    // second projection: T = Res B (in the G region), Res -= T B^T, P += T
    gemm4<TB, R, D, false, false>(sQ, LA, sB, LB,
                                  [&](int t, int c, float v) { sG[t * LB + c] = v; });
    __syncthreads();
    gemm4<TB, D, R, false, true>(sG, LB, sB, LB,
                                 [&](int t, int f, float v) { sQ[t * LA + f] -= v; });
    for (int i = tid; i < TB * R; i += kThreads) {
      const int t = i / R, c = i % R;
      sP[t * LB + c] += sG[t * LB + c];
    }
    __syncthreads();

    // ---------------- phase 2: Q by CholeskyQR2 ----------------
    // pass 0 drops directions at the guard above (unresolved by the fp32
    // Gram, or float noise of the projection); pass 1 sees ~unit rows and
    // drops those that lost their norm.
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      gemm4<TB, TB, D, false, true>(sQ, LA, sQ, LA,
                                    [&](int a, int b, float v) { sG[a * LG + b] = v; });
      __syncthreads();
      float tau = 0.25f;
      if (pass == 0) {
        float tr = 0.f;                           // ||Res||_F^2 (LDS broadcast reads)
#pragma unroll 8
        for (int t = 0; t < TB; ++t) tr += sG[t * LG + t];
        tau = fmaxf(kGuardAbs * normA2, fminf(kGuard * normA2, kGuardRel * tr));
      }
      chol_lds<TB>(sG, LG, tau, invd);
      if (tid < D) {
        float x[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) x[t] = sQ[t * LA + tid];
        fwd_solve<TB>(x, sG, LG, invd);
#pragma unroll
        for (int t = 0; t < TB; ++t) sQ[t * LA + tid] = x[t];
      }
      __syncthreads();
    }
    // re-orthogonalize Q against B
    gemm4<TB, R, D, false, false>(sQ, LA, sB, LB,
                                  [&](int t, int c, float v) { sG[t * LB + c] = v; });
    __syncthreads();
    gemm4<TB, D, R, false, true>(sG, LB, sB, LB,
                                 [&](int t, int f, float v) { sQ[t * LA + f] -= v; });
    __syncthreads();
    // A Q^T (64 x 64) into the G region
    gemm4<TB, TB, D, false, true>(sA, LA, sQ, LA,
                                  [&](int t, int j, float v) { sG[t * LG + j] = v; });
    __syncthreads();
  }

  // ---------------- phase 3: core ----------------
  {
    constexpr int PER = TB * NC / kThreads;
    static_assert(TB * NC % kThreads == 0, "core rows per thread");
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = tid + j * kThreads, t = e / NC, c = e % NC;
      if constexpr (kRes) v[j] = c < R ? sP[t * LB + c] : sG[t * LG + (c - R)];
      else v[j] = sP[t * LB + c];
    }
    __syncthreads();
    int bad = !isfinite(normA2);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = tid + j * kThreads, t = e / NC, c = e % NC;
      bad |= !isfinite(v[j]);
      core[(R + t) * LC + c] = v[j];
    }
    for (int e = tid; e < R * NC; e += kThreads) {
      const int i = e / NC, c = e % NC;
      const float x = (c == i) ? sing[i] : 0.f;
      bad |= !isfinite(x);
      core[i * LC + c] = x;
    }
    if (bad) set_flag(M.sh, 1);
    __syncthreads();
  }

  // ---------------- phase 4: QR of the core, one-sided Jacobi on R ----------
  {
    qr_rows<N, NC, LC>(core, sig, reinterpret_cast<float *>(perm));
    const int sweeps = jacobi_rows<NC, NC, LC>(core, lds + Ly::oNrm, reinterpret_cast<int *>(sig), perm, R);
    if (sweeps > kMaxSweeps && tid == 0) set_flag(M.sh, 2);
  }

  // ---------------- phase 5: singular values, descending order -------------
  for (int j = tid; j < N; j += kThreads) {
    const float *row = core + j * LC;
    float s0a = 0.f, s1a = 0.f;
    for (int i = 0; i < NC; i += 4) {
      const float4 w = ld4(row + i);
      s0a = fmaf(w.x, w.x, s0a); s1a = fmaf(w.y, w.y, s1a);
      s0a = fmaf(w.z, w.z, s0a); s1a = fmaf(w.w, w.w, s1a);
    }
    sig[j] = sqrtf(s0a + s1a);
  }
  __syncthreads();
  for (int j = tid; j < N; j += kThreads) {
    const float sj = sig[j];
    int rank = 0;
    for (int i = 0; i < N; ++i) rank += (sig[i] > sj) || (sig[i] == sj && i < j);
    perm[rank] = j;
  }
  __syncthreads();

  // ---------------- phase 6: B_new = [B Q^T] V'[:, :r] ----------------
  const float sig0 = sig[perm[0]];
  const float tol_null = 64.f * N * FLT_EPSILON * sig0;
  if (!isfinite(sig0) && tid == 0) set_flag(M.sh, 1);
  {
    constexpr int TK = R / 4, TILES = (D / 4) * TK, TPT = (TILES + kThreads - 1) / kThreads;
    float acc[TPT][4][4];
#pragma unroll
    for (int tt = 0; tt < TPT; ++tt) {
      const int tile = tid + tt * kThreads;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[tt][i][j] = 0.f;
      if (tile < TILES) {
        const int f0 = (tile / TK) * 4, k0 = (tile % TK) * 4;
        const float *zr[4];
        float zs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = perm[k0 + j];
          zr[j] = core + row * LC;
          zs[j] = sig[row] > tol_null ? 1.f / sig[row] : 0.f;
        }
#pragma unroll 2
        for (int c0 = 0; c0 < R; c0 += 4) {
          float xb[4][4], z[4][4];     // xb[f][c], z[k][c]
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 w = ld4(Bsrc + (f0 + i) * ldB + c0);
            xb[i][0] = w.x; xb[i][1] = w.y; xb[i][2] = w.z; xb[i][3] = w.w;
            const float4 y = ld4(zr[i] + c0);
            z[i][0] = y.x; z[i][1] = y.y; z[i][2] = y.z; z[i][3] = y.w;
          }
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[tt][i][j] = fmaf(xb[i][cc], z[j][cc], acc[tt][i][j]);
        }
        if constexpr (kRes) {
#pragma unroll 2
          for (int j0 = 0; j0 < TB; j0 += 4) {
            float xq[4][4], z[4][4];   // xq[j][f] = Q[j0 + j][f0 + f], z[k][j]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 w = ld4(sQ + (j0 + i) * LA + f0);
              xq[i][0] = w.x; xq[i][1] = w.y; xq[i][2] = w.z; xq[i][3] = w.w;
              const float4 y = ld4(zr[i] + R + j0);
              z[i][0] = y.x; z[i][1] = y.y; z[i][2] = y.z; z[i][3] = y.w;
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[tt][i][j] = fmaf(xq[jj][i], z[j][jj], acc[tt][i][j]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[tt][i][j] *= zs[j];
      }
    }
    __syncthreads();              // Q and the core are no longer read
#pragma unroll
    for (int tt = 0; tt < TPT; ++tt) {
      const int tile = tid + tt * kThreads;
      if (tile < TILES) {
        const int f0 = (tile / TK) * 4, k0 = (tile % TK) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st4(sBn + (f0 + i) * LB + k0,
              make_float4(acc[tt][i][0], acc[tt][i][1], acc[tt][i][2], acc[tt][i][3]));
      }
    }
  }
  // null completion: each column whose singular value is ~0 becomes the unit
  // vector with the largest remainder against the columns kept so far, made
  // orthogonal to them by two Gram-Schmidt passes.
  float *rem = lds + Ly::oRem, *vec = lds + Ly::oVec, *dot = lds + Ly::oDot;
  for (int k = tid; k < R; k += kThreads) act[k] = sig[perm[k]] > tol_null;
  __syncthreads();
  for (int k = 0; k < R; ++k) {
    if (act[k]) continue;                      // uniform: act is shared
    for (int e = tid; e < D; e += kThreads) {
      float s = 0.f;
      for (int c = 0; c < R; ++c) s += act[c] ? sBn[e * LB + c] * sBn[e * LB + c] : 0.f;
      rem[e] = 1.f - s;
    }
    __syncthreads();
    if (tid == 0) {
      int best = 0;
      for (int e = 1; e < D; ++e)
        if (rem[e] > rem[best]) best = e;
      s_int[1] = best;
    }
    __syncthreads();
    for (int e = tid; e < D; e += kThreads) vec[e] = (e == s_int[1]) ? 1.f : 0.f;
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
      for (int c = tid; c < R; c += kThreads) {
        float s = 0.f;
        if (act[c])
          for (int f = 0; f < D; ++f) s += sBn[f * LB + c] * vec[f];
        dot[c] = s;
      }
      __syncthreads();
      for (int f = tid; f < D; f += kThreads) {
        float s = vec[f];
        for (int c = 0; c < R; ++c) s -= sBn[f * LB + c] * dot[c];
        vec[f] = s;
      }
      __syncthreads();
    }
    if (tid == 0) {
      float s = 0.f;
      for (int f = 0; f < D; ++f) s += vec[f] * vec[f];
      s_f[1] = sqrtf(s);
    }
    __syncthreads();
    for (int f = tid; f < D; f += kThreads) sBn[f * LB + k] = vec[f] / s_f[1];
    __syncthreads();
    if (tid == 0) act[k] = 1;
    __syncthreads();
  }
  __syncthreads();

  // Re-orthonormalize B_new (one CholeskyQR pass on its columns): the Jacobi
  // stopping tolerance leaves the columns orthogonal only to ~1e-6, which
  // would otherwise accumulate fold after fold.
  {
    float *sGb = lds + Ly::oA;     // R x LB, over the dead A / core region
    gemm4<R, R, D, true, false>(sBn, LB, sBn, LB,
                                [&](int a, int b, float v) { sGb[a * LB + b] = v; });
    __syncthreads();
    chol_lds<R>(sGb, LB, 0.25f, invd);
    if (tid < D) {
      float x[R];
#pragma unroll
      for (int c = 0; c < R; ++c) x[c] = sBn[tid * LB + c];
      fwd_solve<R>(x, sGb, LB, invd);
#pragma unroll
      for (int c = 0; c < R; ++c) sBn[tid * LB + c] = x[c];
    }
    __syncthreads();
  }

  // ---------------- phase 7: M, block coefficients, new basis --------------
  gemm4<R, R, D, true, false>(Bsrc, ldB, sBn, LB,
                              [&](int c, int k, float v) { msync[c * R + k] = v; });
  // the block again (the core region over A is free now)
  (void)load_A(sA);
  __syncthreads();
  gemm4<TB, R, D, false, false>(sA, LA, sBn, LB, [&](int t, int k, float v) {
    Store<T>::store(coef, (size_t)(n_c + t) * R + k, v);
  });
  __syncthreads();                 // M (which reads the old basis) is done
  for (int i = tid; i < D * R / 4; i += kThreads) {
    const int f = (4 * i) / R, c = (4 * i) % R;
    st4(basis_out + 4 * i, ld4(sBn + f * LB + c));
  }
  if (tid < R) sing_out[tid] = sig[perm[tid]];
}

template <int R, typename T>
__global__ __launch_bounds__(kThreads) void block_update_kernel(Model M, LayerSel sel,
                                                                int64_t n_c, int xsel, SeqTab tab) {
  constexpr int D = kHeadDim;
  extern __shared__ float4 lds4[];
  float *lds = reinterpret_cast<float *>(lds4);
  const Dims &Dm = M.D;
  const int layer = sel.idx[blockIdx.y];
  // grid.x: units (one factor, xsel) or units x 2 (both factors, equal ranks)
  const int u = xsel < 0 ? blockIdx.x >> 1 : blockIdx.x, X = xsel < 0 ? blockIdx.x & 1 : xsel;
  if (!seq_in(tab, u / Dm.kv_heads)) return;    // ragged: a sequence whose ring is not full
  if (tab.n) n_c = tab.nc[u / Dm.kv_heads];
  // reads the layer's current generation; writes the new basis, S and block
  // coefficients into the same one, or (copy-on-write) into the other
  LayerPtrs P = layer_ptrs(M, layer), Po = layer_ptrs_out(M, layer);
  const T *ring = reinterpret_cast<const T *>(X == 0 ? P.ringk : P.ringv) + (size_t)u * Dm.slots * D;
  const int s0 = (int)(n_c % Dm.slots), slots = Dm.slots;
  fold_one<R, T>(M, lds, P.basis[X] + (size_t)u * D * R, P.sing[X] + (size_t)u * R,
                 Po.basis[X] + (size_t)u * D * R, Po.sing[X] + (size_t)u * R,
                 P.msync[X] + (size_t)u * R * R,
                 reinterpret_cast<T *>(Po.coef[X]) + (size_t)u * Dm.max_tokens * R, n_c,
                 [&](float *sA) { return load_block<T, FoldLayout<R>::LA>(ring, X, s0, slots, sA); });
}

// ---------------------------------------------------------------------------
// Bulk folding of a prompt (prefill): one workgroup per (unit, factor) folds
// nblk consecutive blocks in order, each read from the caller's input rows
// (rounded to the storage type, as the ring would hold them) instead of the
// ring, and leaves every block's M in mbulk (slot j) for one deferred
// synchronization.  The fold itself is the same as above, block after block;
// B and S pass from one block to the next through global memory, which the
// workgroup's own barrier orders.
// ---------------------------------------------------------------------------
template <typename T, typename IN, int LA>
__device__ float load_input_block(const IN *x, int64_t row0, int n_in, int b, int h, int kv, float *sA,
                                  const Shared &S) {
  constexpr int D = kHeadDim, TB = kBlock;
  float asq = 0.f;
  int bad = 0;
  for (int i = threadIdx.x; i < TB * D / 8; i += kThreads) {
    const int t = i / (D / 8), f0 = (i % (D / 8)) * 8;
    float v[8];
    load8<IN>(x + (((size_t)b * n_in + row0 + t) * kv + h) * D + f0, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (std::is_same<T, bf16_t>::value && std::is_same<IN, float>::value)
        v[j] = bf16_to_f32(f32_to_bf16(v[j]));     // the value a bf16 ring row would hold
      bad |= !isfinite(v[j]);
      asq = fmaf(v[j], v[j], asq);
    }
    st4(sA + t * LA + f0, make_float4(v[0], v[1], v[2], v[3]));
    st4(sA + t * LA + f0 + 4, make_float4(v[4], v[5], v[6], v[7]));
  }
  if (bad) set_flag(S, 4);
  return asq;
}

template <int R, typename T, typename IN>
__global__ __launch_bounds__(kThreads) void bulk_fold_kernel(Model M, BulkIn in, int64_t n_c0, int nblk,
                                                             int xsel, int64_t row0, int n_in, float *mbulk,
                                                             int bulk_blocks) {
  constexpr int D = kHeadDim;
  extern __shared__ float4 lds4[];
  float *lds = reinterpret_cast<float *>(lds4);
  const Dims &Dm = M.D;
  const int li = blockIdx.y, layer = in.layer[li];
  const int u = xsel < 0 ? blockIdx.x >> 1 : blockIdx.x, X = xsel < 0 ? blockIdx.x & 1 : xsel;
  const int b = u / Dm.kv_heads, h = u % Dm.kv_heads;
  const IN *kin = reinterpret_cast<const IN *>(in.k[li]), *vin = reinterpret_cast<const IN *>(in.v[li]);
  mbulk += (size_t)li * bulk_layer_floats(Dm, bulk_blocks);
  LayerPtrs P = layer_ptrs(M, layer);
  float *basis = P.basis[X] + (size_t)u * D * R;
  float *sing = P.sing[X] + (size_t)u * R;
  T *coef = reinterpret_cast<T *>(P.coef[X]) + (size_t)u * Dm.max_tokens * R;
  const IN *x = X == 0 ? kin : vin;
  // [factor][unit][block][R][R]; the V part follows the K part
  float *mb = mbulk + (X ? (size_t)Dm.units * bulk_blocks * Dm.rk * Dm.rk : 0) +
              (size_t)u * bulk_blocks * R * R;
  for (int j = 0; j < nblk; ++j) {
    const int64_t r0 = row0 + (int64_t)j * kBlock;
    fold_one<R, T>(M, lds, basis, sing, basis, sing, mb + (size_t)j * R * R, coef,
                   n_c0 + (int64_t)j * kBlock, [&](float *sA) {
                     return load_input_block<T, IN, FoldLayout<R>::LA>(x, r0, n_in, b, h, Dm.kv_heads,
                                                                       sA, M.sh);
                   });
    __syncthreads();                 // B, S of this block visible to the next one
  }
}

template <int R, typename T>
hipError_t launch_fold_t(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                         const SeqTab &tab) {
  static bool attr = false;
  const size_t bytes = FoldLayout<R>::bytes;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&block_update_kernel<R, T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(x < 0 ? M.D.units * 2 : M.D.units, sel.n);
  hipLaunchKernelGGL((block_update_kernel<R, T>), grid, dim3(kThreads), bytes, s, M, sel, n_c, x, tab);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_fold(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                         const SeqTab &tab) {
  const int r = x == 1 ? M.D.rv : M.D.rk;
  if (x < 0 && M.D.rk != M.D.rv) return hipErrorInvalidValue;
  switch (r) {
    case 16: return launch_fold_t<16, T>(M, sel, n_c, x, s, tab);
    case 32: return launch_fold_t<32, T>(M, sel, n_c, x, s, tab);
    case 64: return launch_fold_t<64, T>(M, sel, n_c, x, s, tab);
    case 128: return launch_fold_t<128, T>(M, sel, n_c, x, s, tab);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Suffix products of a bulk fold's M_0 .. M_{n-1}: slot j becomes
// S_j = M_j M_{j+1} ... M_{n-1} (slot n-1 keeps M_{n-1}).  Rows older than the
// first block are synchronized by S_0, the rows of block j by S_{j+1}, the
// last block's rows need nothing: each row then carries the product of every
// M applied after it was written, as block-by-block synchronization would
// have applied them one at a time.  One workgroup per (unit, factor); both
// matrices of a step in LDS.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void bulk_suffix_kernel(Model M, int nblk, int xsel, float *mbulk,
                                                          int bulk_blocks) {
  extern __shared__ float4 sfx4[];
  float *sA = reinterpret_cast<float *>(sfx4), *sS = sA + R * R;
  const Dims &Dm = M.D;
  mbulk += (size_t)blockIdx.y * bulk_layer_floats(Dm, bulk_blocks);
  const int u = xsel < 0 ? blockIdx.x >> 1 : blockIdx.x, X = xsel < 0 ? blockIdx.x & 1 : xsel;
  float *mb = mbulk + (X ? (size_t)Dm.units * bulk_blocks * Dm.rk * Dm.rk : 0) +
              (size_t)u * bulk_blocks * R * R;
  constexpr int PER = (R * R + 255) / 256;
  for (int e = threadIdx.x; e < R * R; e += 256) sS[e] = mb[(size_t)(nblk - 1) * R * R + e];
  for (int j = nblk - 2; j >= 0; --j) {
    for (int e = threadIdx.x; e < R * R; e += 256) sA[e] = mb[(size_t)j * R * R + e];
    __syncthreads();
    float acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = threadIdx.x + 256 * q;
      float a = 0.f;
      if (e < R * R) {
        const int i = e / R, cc = e % R;
#pragma unroll 8
        for (int k = 0; k < R; ++k) a = fmaf(sA[i * R + k], sS[k * R + cc], a);
      }
      acc[q] = a;
    }
    __syncthreads();                 // every read of S done before it is replaced
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = threadIdx.x + 256 * q;
      if (e < R * R) {
        sS[e] = acc[q];
        mb[(size_t)j * R * R + e] = acc[q];
      }
    }
    __syncthreads();
  }
}

template <int R, typename T, typename IN>
hipError_t launch_bulk_t(const Model &M, const BulkIn &in, int64_t n_c0, int nblk, int x,
                         int64_t row0, int n_in, float *mbulk, int bulk_blocks, hipStream_t s) {
  static bool attr = false;
  const size_t bytes = FoldLayout<R>::bytes;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bulk_fold_kernel<R, T, IN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(x < 0 ? M.D.units * 2 : M.D.units, in.n);
  hipLaunchKernelGGL((bulk_fold_kernel<R, T, IN>), grid, dim3(kThreads), bytes, s, M, in, n_c0, nblk, x,
                     row0, n_in, mbulk, bulk_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nblk < 2) return e;
  static bool sattr = false;
  const size_t sbytes = (size_t)2 * R * R * 4;
  if (!sattr) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bulk_suffix_kernel<R>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sbytes);
    if (e != hipSuccess) return e;
    sattr = true;
  }
  hipLaunchKernelGGL((bulk_suffix_kernel<R>), grid, dim3(256), sbytes, s, M, nblk, x, mbulk, bulk_blocks);  // grid.y: layers
  return hipGetLastError();
}

template <typename T, typename IN>
hipError_t dispatch_bulk(const Model &M, const BulkIn &in, int64_t n_c0, int nblk, int x, int64_t row0,
                         int n_in, float *mbulk, int bulk_blocks, hipStream_t s) {
  const int r = x == 1 ? M.D.rv : M.D.rk;
  if (x < 0 && M.D.rk != M.D.rv) return hipErrorInvalidValue;
  switch (r) {
    case 16: return launch_bulk_t<16, T, IN>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s);
    case 32: return launch_bulk_t<32, T, IN>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s);
    case 64: return launch_bulk_t<64, T, IN>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s);
    case 128: return launch_bulk_t<128, T, IN>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bulk_fold(const Model &M, const BulkIn &in, int64_t n_c0, int nblk, int x, int in_dtype,
                            int64_t row0, int n_in, float *mbulk, int bulk_blocks, hipStream_t s) {
  if (nblk <= 0 || in.n <= 0) return hipSuccess;
  if (M.D.storage == 1)
    return in_dtype == 1 ? dispatch_bulk<bf16_t, bf16_t>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s)
                         : dispatch_bulk<bf16_t, float>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s);
  return in_dtype == 1 ? dispatch_bulk<float, bf16_t>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s)
                       : dispatch_bulk<float, float>(M, in, n_c0, nblk, x, row0, n_in, mbulk, bulk_blocks, s);
}

hipError_t launch_block_update(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                               const SeqTab &tab) {
  return M.D.storage == 1 ? dispatch_fold<bf16_t>(M, sel, n_c, x, s, tab)
                          : dispatch_fold<float>(M, sel, n_c, x, s, tab);
}

}  // namespace iskv
