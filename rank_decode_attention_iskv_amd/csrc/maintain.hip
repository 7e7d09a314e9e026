// Cache maintenance kernels for gfx950: ring append, Brand block-incremental
// SVD fold, and basis synchronization of the stored coefficients.
//
// Page: "iS-KV -- Basis-synchronized online low-rank KV compression -- What does
// it mean?" (learnaivisually.com), cited as [iS-KV explainer]:
//   - append: recent tokens stay exact (window paragraph); keys are stored
//     before RoPE (Jargon "Pre-RoPE keys").
//   - fold: 64 tokens that leave the window are folded as one block by Brand's
//     block-incremental SVD on a small core whose size does not depend on the
//     history (Jargon "Block-incremental SVD"; drift paragraph).
//   - sync: old coefficients are rewritten for the new basis (FAQ "What is
//     basis synchronization?").
#include <cfloat>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int kThreads = 256;

__device__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// Reset: basis = I[:, :r] (the basis before any block has been seen).
// ---------------------------------------------------------------------------
__global__ void reset_basis_kernel(Model M, int layer) {
  const Dims &D = M.D;
  LayerPtrs P = layer_ptrs(M, layer);
  const size_t n = (size_t)D.units * 2 * D.d * D.r;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % D.r);
    const int f = (int)((i / D.r) % D.d);
    P.basis[i] = (f == c) ? 1.f : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Append: grid (n tokens, kv heads, batch), block = head_dim threads.
// ---------------------------------------------------------------------------
template <typename T, typename In>
__global__ void append_kernel(Model M, int layer, const In *k, const In *v, int n, int64_t pos0) {
  const Dims &D = M.D;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, f = threadIdx.x;
  const int u = b * D.kv_heads + h;
  const size_t src = (((size_t)b * n + t) * D.kv_heads + h) * D.d + f;
  const float kx = Store<In>::load(k, src);
  const float vx = Store<In>::load(v, src);
  if (!isfinite(kx) || !isfinite(vx)) set_flag(M.sh, 4);
  LayerPtrs P = layer_ptrs(M, layer);
  const int slot = (int)((pos0 + t) % D.slots);
  T *rk = reinterpret_cast<T *>(P.ringk) + (size_t)u * D.slots * D.d;
  T *rv = reinterpret_cast<T *>(P.ringv) + (size_t)u * D.slots * D.d;
  Store<T>::store(rk, (size_t)slot * D.d + f, kx);
  Store<T>::store(rv, (size_t)f * D.slots + slot, vx);
}

// ---------------------------------------------------------------------------
// Decode operand copy of the basis.
//
// The decode kernel rebuilds keys with MFMA: A operand = basis rows (16 per
// M-block), B operand = coefficient rows of 16 tokens.  Lane l = m + 16*rho
// of a wave holds basis row 16*mb + m and the coefficient range
// [rho*r/4, (rho+1)*r/4).  Layout per (unit, K|V): 8 M-blocks, each with r/16
// chunks of [64 lanes][16 bytes] (512*r bytes in all):
//   bf16, r >= 32: chunk 2*kb + hl = 8 bf16 of coefficients rho*r/4 + 8*kb + j,
//                  hl = 0 high part, 1 low part (x = hi + lo to ~2^-16)
//   bf16, r == 16: chunk 0 = 4 bf16 high parts, then 4 bf16 low parts
//   f32:           chunk j4 = 4 floats, coefficients rho*r/4 + 4*j4 + j
// ---------------------------------------------------------------------------
__global__ void prep_frag_kernel(Model M, LayerSel sel) {
  const Dims &D = M.D;
  const int l = sel.idx[blockIdx.y];
  const int ux = blockIdx.x;
  LayerPtrs P = layer_ptrs(M, l);
  const float *B = P.basis + (size_t)ux * D.d * D.r;
  uint8_t *F = P.frag + (size_t)ux * 4 * D.d * D.r;
  const int r = D.r, per = r / 4;             // coefficients per lane
  const int chunks = r / 16;
  const int total = 8 * chunks * 64;           // (mb, chunk, lane)
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int lane = i & 63, ch = (i >> 6) % chunks, mb = (i >> 6) / chunks;
    const int m = lane & 15, rho = lane >> 4;
    const int row = 16 * mb + m;
    uint8_t *dst = F + ((size_t)(mb * chunks + ch) * 64 + lane) * 16;
    const float *src = B + (size_t)row * r + rho * per;
    if (D.storage == 1) {
      uint16_t *o = reinterpret_cast<uint16_t *>(dst);
      for (int j = 0; j < 8; ++j) {
        // coefficient index and part of slot j of this chunk
        const int c = (r >= 32) ? (ch >> 1) * 8 + j : (j & 3);
        const int hl = (r >= 32) ? (ch & 1) : (j >> 2);
        const float x = src[c];
        const uint16_t hi = f32_to_bf16(x);
        o[j] = hl == 0 ? hi : f32_to_bf16(x - bf16_to_f32(hi));
      }
    } else {
      float *o = reinterpret_cast<float *>(dst);
      for (int j = 0; j < 4; ++j) o[j] = src[ch * 4 + j];
    }
  }
}

// ---------------------------------------------------------------------------
// Sync: C[t] <- C[t] M for rows t < n_old.  grid (row tiles, units*2, layers)
// ---------------------------------------------------------------------------
template <int R, typename T>
__global__ __launch_bounds__(kThreads) void sync_rows_kernel(Model M, LayerSel sel, int64_t n_old) {
  __shared__ float sM[R * R];
  const Dims &D = M.D;
  const int l = sel.idx[blockIdx.z];
  const int ux = blockIdx.y;
  LayerPtrs P = layer_ptrs(M, l);
  const float *Ms = P.msync + (size_t)ux * R * R;
  T *C = reinterpret_cast<T *>(P.coef) + (size_t)ux * D.max_tokens * R;
  for (int i = threadIdx.x; i < R * R; i += blockDim.x) sM[i] = Ms[i];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_old) return;
  float row[R];
#pragma unroll
  for (int c = 0; c < R; ++c) row[c] = Store<T>::load(C, (size_t)t * R + c);
  for (int k = 0; k < R; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < R; ++c) acc = fmaf(row[c], sM[c * R + k], acc);
    Store<T>::store(C, (size_t)t * R + k, acc);
  }
}

// ---------------------------------------------------------------------------
// Block update (Brand's block-incremental SVD) -- one workgroup per
// (selected layer, unit, K|V).
//
// With the old history H = U diag(S) B^T (U orthonormal, the stored
// coefficients being U diag(S)) and a new block A (64 x d):
//   P = A B, R = A - P B^T (twice); R = R_r^T Q^T with Q orthonormal and
//   orthogonal to B (CholeskyQR2 with a pivot guard);
//   [H; A] = diag(U, I) K [B Q]^T,  K = [[diag S, 0], [P, R_r^T]]  ((r+64)^2);
//   K = U' diag(s') V'^T;  B_new = [B Q] V'[:, :r];  S_new = s'[:r];
//   old coefficients map by M = B^T B_new; the block's are A B_new.
// The SVD of K is a one-sided (Hestenes) Jacobi on the rows of K: the rows
// are rotated pairwise until mutually orthogonal; then row j = s'_j v'_j^T.
// ---------------------------------------------------------------------------
constexpr int kMaxSweeps = 40;
constexpr float kJacobiTol = 1.0e-6f;     // rotate while |y_p . y_q| > tol |y_p||y_q|
// A residual direction is dropped when its squared norm is below
// kGuard * ||A||_F^2 (so kept directions have condition number < ~1/sqrt(kGuard)).
constexpr float kGuard = 1.0e-7f;

__device__ void cholesky_lower(float *G, int ld, int n, float tau, float *s_piv) {
  // In-place lower Cholesky of the n x n matrix G (lower part used).  Pivots
  // <= tau zero the column (semidefinite guard).
  const int tid = threadIdx.x;
  for (int j = 0; j < n; ++j) {
    if (tid == 0) {
      const float piv = G[j * ld + j];
      const float Ljj = (piv > tau) ? sqrtf(piv) : 0.f;
      G[j * ld + j] = Ljj;
      *s_piv = Ljj;
    }
    __syncthreads();
    const float Ljj = *s_piv;
    for (int i = j + 1 + tid; i < n; i += blockDim.x)
      G[i * ld + j] = (Ljj > 0.f) ? G[i * ld + j] / Ljj : 0.f;
    __syncthreads();
    const int m = n - 1 - j;                 // trailing size
    for (int e = tid; e < m * m; e += blockDim.x) {
      const int i = j + 1 + e / m, k = j + 1 + e % m;
      if (k <= i) G[i * ld + k] -= G[i * ld + j] * G[k * ld + j];
    }
    __syncthreads();
  }
}

// n rows of length d (stride ld) <- L^{-1} rows (forward substitution); one
// thread per column.
__device__ void forward_solve_rows(float *Qr, int ld, int n, const float *L, int ldl) {
  const int f = threadIdx.x;
  if (f < kHeadDim) {
    for (int i = 0; i < n; ++i) {
      float acc = Qr[i * ld + f];
      for (int k = 0; k < i; ++k) acc -= L[i * ldl + k] * Qr[k * ld + f];
      const float Lii = L[i * ldl + i];
      Qr[i * ld + f] = (Lii > 0.f) ? acc / Lii : 0.f;
    }
  }
  __syncthreads();
}

template <int R>
struct FoldLds {
  static constexpr int N = R + kBlock;
  static constexpr int AP = kHeadDim + 1;
  static constexpr int BP = R + 1;
  static constexpr bool kResidual = R < kHeadDim;
  // phase 1-2 regions (floats)
  static constexpr int oA = 0;
  static constexpr int oB = oA + kBlock * AP;
  static constexpr int oP = oB + kHeadDim * BP;
  static constexpr int oT = oP + kBlock * BP;
  static constexpr int end12 = kResidual ? oT + kBlock * AP : oT;
  // phase 3+ regions
  static constexpr int oCore = 0;
  static constexpr int oSig = N * N;
  static constexpr int oPerm = oSig + N;
  static constexpr int oAct = oPerm + N;
  static constexpr int oRem = oAct + R;
  static constexpr int oVec = oRem + kHeadDim;
  static constexpr int oDot = oVec + kHeadDim;
  static constexpr int oMisc = oDot + R;
  static constexpr int end3 = oMisc + 16;
  // phase 7 (reload A and B_new over the core)
  static constexpr int oA7 = 0;
  static constexpr int oB7 = kBlock * AP;
  static constexpr int end7 = oB7 + kHeadDim * BP;
  static constexpr int floats = (end12 > end3 ? (end12 > end7 ? end12 : end7)
                                              : (end3 > end7 ? end3 : end7));
  static constexpr size_t bytes = (size_t)floats * 4;
};

template <int R, typename T>
__global__ __launch_bounds__(kThreads) void block_update_kernel(Model M, LayerSel sel,
                                                                int64_t n_c) {
  using L = FoldLds<R>;
  constexpr int D = kHeadDim, TB = kBlock, N = L::N, AP = L::AP, BP = L::BP;
  extern __shared__ float lds[];
  __shared__ float red[8];
  __shared__ float s_misc[4];
  __shared__ int s_int[4];
  const Dims &Dm = M.D;
  const int layer = sel.idx[blockIdx.y];
  const int ux = blockIdx.x, u = ux >> 1, X = ux & 1;
  const int tid = threadIdx.x;
  LayerPtrs P = layer_ptrs(M, layer);
  float *basis = P.basis + (size_t)ux * D * R;
  float *sing = P.sing + (size_t)ux * R;
  float *msync = P.msync + (size_t)ux * R * R;
  T *coef = reinterpret_cast<T *>(P.coef) + (size_t)ux * Dm.max_tokens * R;
  const T *ring = reinterpret_cast<const T *>(X == 0 ? P.ringk : P.ringv) +
                  (size_t)u * Dm.slots * D;
  float *scr = M.sh.fold + ((size_t)layer * Dm.units * 2 + ux) * fold_scratch_floats(R);
  float *gQ = scr;              // [64][128] rows of Q^T
  float *gP = gQ + TB * D;      // [64][R]
  float *gRr = gP + TB * R;     // [64][64]
  float *gBn = gRr + TB * TB;   // [128][R]
  const int s0 = (int)(n_c % Dm.slots);
  auto ringA = [&](int t, int f) -> float {
    const size_t idx = (X == 0) ? (size_t)(s0 + t) * D + f : (size_t)f * Dm.slots + (s0 + t);
    return Store<T>::load(ring, idx);
  };

  // ---------------- phase 1: projection, twice ----------------
  float *sA = lds + L::oA, *sB = lds + L::oB, *sP = lds + L::oP, *sT = lds + L::oT;
  float asq = 0.f;
  for (int i = tid; i < TB * D; i += kThreads) {
    const int t = i >> 7, f = i & 127;
    const float a = ringA(t, f);
    sA[t * AP + f] = a;
    asq += a * a;
  }
  for (int i = tid; i < D * R; i += kThreads) sB[(i / R) * BP + (i % R)] = basis[i];
  const float normA2 = block_sum(asq, red);   // includes barriers
  for (int i = tid; i < TB * R; i += kThreads) {
    const int t = i / R, c = i % R;
    float acc = 0.f;
    for (int f = 0; f < D; ++f) acc += sA[t * AP + f] * sB[f * BP + c];
    sP[t * BP + c] = acc;
  }
  __syncthreads();
  if constexpr (L::kResidual) {
    for (int i = tid; i < TB * D; i += kThreads) {
      const int t = i >> 7, f = i & 127;
      float acc = sA[t * AP + f];
      for (int c = 0; c < R; ++c) acc -= sP[t * BP + c] * sB[f * BP + c];
      sA[t * AP + f] = acc;
    }
    __syncthreads();
    for (int i = tid; i < TB * R; i += kThreads) {
      const int t = i / R, c = i % R;
      float acc = 0.f;
      for (int f = 0; f < D; ++f) acc += sA[t * AP + f] * sB[f * BP + c];
      sT[t * BP + c] = acc;
    }
    __syncthreads();
    for (int i = tid; i < TB * D; i += kThreads) {
      const int t = i >> 7, f = i & 127;
      float acc = sA[t * AP + f];
      for (int c = 0; c < R; ++c) acc -= sT[t * BP + c] * sB[f * BP + c];
      sA[t * AP + f] = acc;
    }
    for (int i = tid; i < TB * R; i += kThreads) {
      const int t = i / R, c = i % R;
      sP[t * BP + c] += sT[t * BP + c];
    }
    __syncthreads();
  }
  for (int i = tid; i < TB * R; i += kThreads) gP[i] = sP[(i / R) * BP + (i % R)];

  // ---------------- phase 2: residual basis by CholeskyQR2 ----------------
  if constexpr (L::kResidual) {
    constexpr int GL = 65;
    for (int pass = 0; pass < 2; ++pass) {
      for (int e = tid; e < TB * TB; e += kThreads) {
        const int a = e >> 6, b = e & 63;
        if (b <= a) {
          float g = 0.f;
          for (int f = 0; f < D; ++f) g += sA[a * AP + f] * sA[b * AP + f];
          sT[a * GL + b] = g;
        }
      }
      __syncthreads();
      // pass 0: drop directions with sigma^2 <= kGuard ||A||^2 (they are at the
      // float noise level of the projection); pass 1: rows are ~unit, drop
      // the ones that lost their norm.
      const float tau = (pass == 0) ? kGuard * normA2 : 0.25f;
      cholesky_lower(sT, GL, kBlock, tau, &s_misc[0]);
      forward_solve_rows(sA, AP, kBlock, sT, GL);
    }
    // re-orthogonalize the rows of Q against B
    for (int i = tid; i < TB * R; i += kThreads) {
      const int t = i / R, c = i % R;
      float acc = 0.f;
      for (int f = 0; f < D; ++f) acc += sA[t * AP + f] * sB[f * BP + c];
      sP[t * BP + c] = acc;
    }
    __syncthreads();
    for (int i = tid; i < TB * D; i += kThreads) {
      const int t = i >> 7, f = i & 127;
      float acc = sA[t * AP + f];
      for (int c = 0; c < R; ++c) acc -= sP[t * BP + c] * sB[f * BP + c];
      sA[t * AP + f] = acc;
    }
    __syncthreads();
    for (int i = tid; i < TB * D; i += kThreads) gQ[i] = sA[(i >> 7) * AP + (i & 127)];
    // R_r^T = A Q (A reloaded; A Q = R Q since Q is orthogonal to B)
    for (int i = tid; i < TB * D; i += kThreads) sT[(i >> 7) * AP + (i & 127)] = ringA(i >> 7, i & 127);
    __syncthreads();
    for (int e = tid; e < TB * TB; e += kThreads) {
      const int t = e >> 6, j = e & 63;
      float acc = 0.f;
      for (int f = 0; f < D; ++f) acc += sT[t * AP + f] * sA[j * AP + f];
      gRr[e] = acc;
    }
  } else {
    for (int i = tid; i < TB * D; i += kThreads) gQ[i] = 0.f;
    for (int i = tid; i < TB * TB; i += kThreads) gRr[i] = 0.f;
  }
  __syncthreads();

  // ---------------- phase 3: core ----------------
  float *core = lds + L::oCore;
  int bad = !isfinite(normA2);
  for (int e = tid; e < N * N; e += kThreads) {
    const int i = e / N, j = e % N;
    float x;
    if (i < R) x = (j == i) ? sing[i] : 0.f;
    else if (j < R) x = gP[(i - R) * R + j];
    else x = gRr[(i - R) * TB + (j - R)];
    bad |= !isfinite(x);
    core[e] = x;
  }
  if (bad) set_flag(M.sh, 1);
  __syncthreads();

  // ---------------- phase 4: one-sided Jacobi on the rows of the core -------
  {
    constexpr int GS = (N <= 128) ? 4 : 2;
    constexpr int NP = N / 2;
    const int g = tid / GS, li = tid % GS;
    int sweep = 0;
    for (; sweep < kMaxSweeps; ++sweep) {
      if (tid == 0) s_int[0] = 0;
      __syncthreads();
      for (int k = 0; k < N - 1; ++k) {
        if (g < NP) {
          int p, q;
          if (g == 0) { p = k; q = N - 1; }
          else { p = (k + g) % (N - 1); q = (k - g + N - 1) % (N - 1); }
          float *yp = core + p * N, *yq = core + q * N;
          float a = 0.f, b = 0.f, c = 0.f;
          for (int e = li; e < N; e += GS) {
            const float x = yp[e], y = yq[e];
            a += x * x; b += y * y; c += x * y;
          }
          for (int o = 1; o < GS; o <<= 1) {
            a += __shfl_xor(a, o); b += __shfl_xor(b, o); c += __shfl_xor(c, o);
          }
          if (c != 0.f && fabsf(c) > kJacobiTol * sqrtf(a * b)) {
            const float zeta = (b - a) / (2.f * c);
            const float t = (fabsf(zeta) > 1.0e18f)
                                ? 0.5f / zeta
                                : copysignf(1.f, zeta) / (fabsf(zeta) + sqrtf(1.f + zeta * zeta));
            const float cs = 1.f / sqrtf(1.f + t * t);
            const float sn = cs * t;
            for (int e = li; e < N; e += GS) {
              const float x = yp[e], y = yq[e];
              yp[e] = cs * x - sn * y;
              yq[e] = sn * x + cs * y;
            }
            if (li == 0) s_int[0] = 1;
          }
        }
        __syncthreads();
      }
      const int rotated = s_int[0];
      __syncthreads();
      if (!rotated) break;
    }
    if (sweep == kMaxSweeps && tid == 0) set_flag(M.sh, 2);
  }

  // ---------------- phase 5: singular values, descending order -------------
  float *sig = lds + L::oSig;
  int *perm = reinterpret_cast<int *>(lds + L::oPerm);
  for (int j = tid; j < N; j += kThreads) {
    float s2 = 0.f;
    for (int e = 0; e < N; ++e) s2 += core[j * N + e] * core[j * N + e];
    sig[j] = sqrtf(s2);
  }
  __syncthreads();
  for (int j = tid; j < N; j += kThreads) {
    const float sj = sig[j];
    int rank = 0;
    for (int i = 0; i < N; ++i) rank += (sig[i] > sj) || (sig[i] == sj && i < j);
    perm[rank] = j;
  }
  __syncthreads();

  // ---------------- phase 6: B_new = [B Q] V'[:, :r] ----------------
  const float sig0 = sig[perm[0]];
  const float tol_null = 64.f * N * FLT_EPSILON * sig0;
  if (!isfinite(sig0) && tid == 0) set_flag(M.sh, 1);
  for (int i = tid; i < D * R; i += kThreads) {
    const int f = i / R, k = i % R;
    const int j = perm[k];
    const float s = sig[j];
    float val = 0.f;
    if (s > tol_null) {
      float acc = 0.f;
      for (int c = 0; c < R; ++c) acc += basis[f * R + c] * core[j * N + c];
      if constexpr (L::kResidual)
        for (int c = 0; c < TB; ++c) acc += gQ[c * D + f] * core[j * N + R + c];
      val = acc / s;
    }
    gBn[i] = val;
  }
  // null completion: each column whose singular value is ~0 becomes the unit
  // vector with the largest remainder against the columns kept so far, made
  // orthogonal to them by two Gram-Schmidt passes.
  int *act = reinterpret_cast<int *>(lds + L::oAct);
  float *rem = lds + L::oRem, *vec = lds + L::oVec, *dot = lds + L::oDot;
  for (int k = tid; k < R; k += kThreads) act[k] = sig[perm[k]] > tol_null;
  __syncthreads();
  for (int k = 0; k < R; ++k) {
    if (act[k]) continue;                      // uniform: act is shared
    for (int e = tid; e < D; e += kThreads) {
      float s = 0.f;
      for (int c = 0; c < R; ++c) s += act[c] ? gBn[e * R + c] * gBn[e * R + c] : 0.f;
      rem[e] = 1.f - s;
    }
    __syncthreads();
    if (tid == 0) {
      int best = 0;
      for (int e = 1; e < D; ++e) if (rem[e] > rem[best]) best = e;
      s_int[1] = best;
    }
    __syncthreads();
    for (int e = tid; e < D; e += kThreads) vec[e] = (e == s_int[1]) ? 1.f : 0.f;
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
      for (int c = tid; c < R; c += kThreads) {
        float s = 0.f;
        if (act[c]) for (int f = 0; f < D; ++f) s += gBn[f * R + c] * vec[f];
        dot[c] = s;
      }
      __syncthreads();
      for (int f = tid; f < D; f += kThreads) {
        float s = vec[f];
        for (int c = 0; c < R; ++c) s -= gBn[f * R + c] * dot[c];
        vec[f] = s;
      }
      __syncthreads();
    }
    if (tid == 0) {
      float s = 0.f;
      for (int f = 0; f < D; ++f) s += vec[f] * vec[f];
      s_misc[1] = sqrtf(s);
    }
    __syncthreads();
    for (int f = tid; f < D; f += kThreads) gBn[f * R + k] = vec[f] / s_misc[1];
    __syncthreads();
    if (tid == 0) act[k] = 1;
    __syncthreads();
  }
  __syncthreads();
  // keep the singular values (sig/perm are overwritten below)
  float sv = 0.f;
  if (tid < R) sv = sig[perm[tid]];
  __syncthreads();
  // Re-orthonormalize B_new (one CholeskyQR pass on its columns): the Jacobi
  // stopping tolerance leaves the columns orthogonal only to ~1e-6, which
  // would otherwise accumulate fold after fold.
  {
    constexpr int LDB = kHeadDim + 1, LDG = R + 1;
    float *sBt = lds;                        // [R][LDB] rows = columns of B_new
    float *sG = lds + R * LDB;               // [R][LDG]
    for (int i = tid; i < D * R; i += kThreads) sBt[(i % R) * LDB + (i / R)] = gBn[i];
    __syncthreads();
    for (int e = tid; e < R * R; e += kThreads) {
      const int a = e / R, b = e % R;
      if (b <= a) {
        float g = 0.f;
        for (int f = 0; f < D; ++f) g += sBt[a * LDB + f] * sBt[b * LDB + f];
        sG[a * LDG + b] = g;
      }
    }
    __syncthreads();
    cholesky_lower(sG, LDG, R, 0.25f, &s_misc[0]);
    forward_solve_rows(sBt, LDB, R, sG, LDG);
    for (int i = tid; i < D * R; i += kThreads) gBn[i] = sBt[(i % R) * LDB + (i / R)];
    __syncthreads();
  }

  // ---------------- phase 7: M, block coefficients, new basis --------------
  for (int i = tid; i < R * R; i += kThreads) {
    const int c = i / R, k = i % R;
    float acc = 0.f;
    for (int f = 0; f < D; ++f) acc += basis[f * R + c] * gBn[f * R + k];
    msync[i] = acc;
  }
  __syncthreads();
  float *sA7 = lds + L::oA7, *sB7 = lds + L::oB7;
  for (int i = tid; i < TB * D; i += kThreads) sA7[(i >> 7) * AP + (i & 127)] = ringA(i >> 7, i & 127);
  for (int i = tid; i < D * R; i += kThreads) sB7[(i / R) * BP + (i % R)] = gBn[i];
  __syncthreads();
  for (int i = tid; i < TB * R; i += kThreads) {
    const int t = i / R, k = i % R;
    float acc = 0.f;
    for (int f = 0; f < D; ++f) acc += sA7[t * AP + f] * sB7[f * BP + k];
    Store<T>::store(coef, (size_t)(n_c + t) * R + k, acc);
  }
  for (int i = tid; i < D * R; i += kThreads) basis[i] = sB7[(i / R) * BP + (i % R)];
  if (tid < R) sing[tid] = sv;
}

template <int R, typename T>
hipError_t launch_fold_t(const Model &M, const LayerSel &sel, int64_t n_c, hipStream_t s) {
  static bool attr = false;
  const size_t bytes = FoldLds<R>::bytes;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&block_update_kernel<R, T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(M.D.units * 2, sel.n);
  hipLaunchKernelGGL((block_update_kernel<R, T>), grid, dim3(kThreads), bytes, s, M, sel, n_c);
  return hipGetLastError();
}

template <int R, typename T>
hipError_t launch_sync_t(const Model &M, const LayerSel &sel, int64_t n_old, hipStream_t s) {
  if (n_old <= 0) return hipSuccess;
  dim3 grid((unsigned)((n_old + kThreads - 1) / kThreads), M.D.units * 2, sel.n);
  hipLaunchKernelGGL((sync_rows_kernel<R, T>), grid, dim3(kThreads), 0, s, M, sel, n_old);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_fold(const Model &M, const LayerSel &sel, int64_t n_c, hipStream_t s) {
  switch (M.D.r) {
    case 16: return launch_fold_t<16, T>(M, sel, n_c, s);
    case 32: return launch_fold_t<32, T>(M, sel, n_c, s);
    case 64: return launch_fold_t<64, T>(M, sel, n_c, s);
    case 128: return launch_fold_t<128, T>(M, sel, n_c, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_sync(const Model &M, const LayerSel &sel, int64_t n_old, hipStream_t s) {
  switch (M.D.r) {
    case 16: return launch_sync_t<16, T>(M, sel, n_old, s);
    case 32: return launch_sync_t<32, T>(M, sel, n_old, s);
    case 64: return launch_sync_t<64, T>(M, sel, n_old, s);
    case 128: return launch_sync_t<128, T>(M, sel, n_old, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reset_layer(const Model &M, int layer, hipStream_t s) {
  hipLaunchKernelGGL(reset_basis_kernel, dim3(256), dim3(256), 0, s, M, layer);
  return hipGetLastError();
}

hipError_t launch_append(const Model &M, int layer, const void *k, const void *v, int n,
                         int in_dtype, int64_t pos0, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid(n, M.D.kv_heads, M.D.batch);
  if (M.D.storage == 1) {
    if (in_dtype == 1)
      hipLaunchKernelGGL((append_kernel<bf16_t, bf16_t>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const bf16_t *)k, (const bf16_t *)v, n, pos0);
    else
      hipLaunchKernelGGL((append_kernel<bf16_t, float>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const float *)k, (const float *)v, n, pos0);
  } else {
    if (in_dtype == 1)
      hipLaunchKernelGGL((append_kernel<float, bf16_t>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const bf16_t *)k, (const bf16_t *)v, n, pos0);
    else
      hipLaunchKernelGGL((append_kernel<float, float>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const float *)k, (const float *)v, n, pos0);
  }
  return hipGetLastError();
}

hipError_t launch_block_update(const Model &M, const LayerSel &sel, int64_t n_c, hipStream_t s) {
  return M.D.storage == 1 ? dispatch_fold<bf16_t>(M, sel, n_c, s)
                          : dispatch_fold<float>(M, sel, n_c, s);
}

hipError_t launch_sync(const Model &M, const LayerSel &sel, int64_t n_old, hipStream_t s) {
  return M.D.storage == 1 ? dispatch_sync<bf16_t>(M, sel, n_old, s)
                          : dispatch_sync<float>(M, sel, n_old, s);
}

hipError_t launch_prep_frag(const Model &M, const LayerSel &sel, hipStream_t s) {
  dim3 grid(M.D.units * 2, sel.n);
  hipLaunchKernelGGL(prep_frag_kernel, grid, dim3(256), 0, s, M, sel);
  return hipGetLastError();
}

}  // namespace iskv
