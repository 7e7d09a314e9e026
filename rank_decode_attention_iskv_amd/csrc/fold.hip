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
#include "fold_core.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

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
  gemm_mfma<TB, R, D, false, false>(sA, LA, Bsrc, ldB,
                                [&](int t, int c, float v) { sP[t * LB + c] = v; });
  __syncthreads();
  if constexpr (kRes) {
    // Res = A - P B^T
    gemm_mfma<TB, D, R, false, true>(sP, LB, sB, LB, [&](int t, int f, float v) {
      sQ[t * LA + f] = sA[t * LA + f] - v;
    });
    __syncthreads();
    // second projection: T = Res B (in the G region), Res -= T B^T, P += T
    gemm_mfma<TB, R, D, false, false>(sQ, LA, sB, LB,
                                  [&](int t, int c, float v) { sG[t * LB + c] = v; });
    __syncthreads();
    gemm_mfma<TB, D, R, false, true>(sG, LB, sB, LB,
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
      gemm_mfma<TB, TB, D, false, true>(sQ, LA, sQ, LA,
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
    gemm_mfma<TB, R, D, false, false>(sQ, LA, sB, LB,
                                  [&](int t, int c, float v) { sG[t * LB + c] = v; });
    __syncthreads();
    gemm_mfma<TB, D, R, false, true>(sG, LB, sB, LB,
                                 [&](int t, int f, float v) { sQ[t * LA + f] -= v; });
    __syncthreads();
    // A Q^T (64 x 64) into the G region
    gemm_mfma<TB, TB, D, false, true>(sA, LA, sQ, LA,
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
    gemm_mfma<R, R, D, true, false>(sBn, LB, sBn, LB,
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
  gemm_mfma<R, R, D, true, false>(Bsrc, ldB, sBn, LB,
                              [&](int c, int k, float v) { msync[c * R + k] = v; });
  // the block again (the core region over A is free now)
  (void)load_A(sA);
  __syncthreads();
  gemm_mfma<TB, R, D, false, false>(sA, LA, sBn, LB, [&](int t, int k, float v) {
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
  if (M.D.joint) return launch_joint_fold(M, sel, n_c, x, s, tab);
  return M.D.storage == 1 ? dispatch_fold<bf16_t>(M, sel, n_c, x, s, tab)
                          : dispatch_fold<float>(M, sel, n_c, x, s, tab);
}

}  // namespace iskv
