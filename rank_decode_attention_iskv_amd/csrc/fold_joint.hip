// Brand block-incremental SVD fold over a joint basis: one basis per
// (sequence, layer) and factor that spans all H KV heads, so a token's row is
// its H heads' rows side by side (H*d wide).  Rank 64 over eight 128-dim heads
// keeps one 64-entry coefficient row per token for all of them, the kind of
// ratio the iS-KV explainer reports for ranks 64-128 (its worked example and
// Table 1), which a per-head basis cannot reach.
//
// The arithmetic is the per-head fold's (fold.hip; page: "iS-KV --
// Basis-synchronized online low-rank KV compression -- What does it mean?",
// Jargon "Block-incremental SVD" and the drift paragraph):
//   P = A B, Res = A - P B^T (projected twice);
//   Res = L Q (CholeskyQR2 with the pivot guard), Q orthogonal to B;
//   K = [[diag S, 0], [P, A Q^T]] ((r+64)^2);  K = U' diag(s') V'^T;
//   B_new = [B Q^T] V'[:, :r];  S_new = s'[:r];  M = B^T B_new;  C_blk = A B_new.
// What changes is where the operands live: the block A (64 x H*d), the basis B
// (H*d x r), Res / Q and B_new no longer fit one workgroup's LDS, so every
// product over the long dimension is a sum over the H heads: the workgroup
// streams one head's 128 columns (A_h, B_h, Res_h / Q_h, B_new_h) through LDS
// at a time and accumulates the 64-row and r-row results in LDS.  Res / Q and
// B_new pass between the sweeps through a per-(sequence, factor) scratch in
// global memory (jres, jbn), written and read back by the same workgroup, whose
// barriers order them.  The core (at most 128 x 128 at r = 64), its QR and its
// Jacobi SVD are the per-head fold's, unchanged.
//
// One workgroup per (selected layer, sequence, K|V); r in {16, 32, 64}.
#include <cfloat>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "fold_core.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

// LDS plan in floats (row strides padded by 4 floats).  Region 1 holds the
// head's block columns A_h, P and two 64-row accumulators S1, S2 while the
// block is projected; the core over it from the core's assembly until B_new
// is formed; then B_new's Gram; then A_h, M and C_blk.  Region 2 holds B_h.
// Region 3 holds Res_h / Q_h (64 x d) or B_new_h (d x r), and the two
// H*d-vectors of the null completion.
template <int R>
struct JointLayout {
  static constexpr int D = kHeadDim, TB = kBlock;
  static constexpr int N = R + TB, NC = N;
  static constexpr int LA = D + 4, LB = R + 4, LC = NC + 4, LS = cmax(LB, TB + 4);
  static constexpr int oA = 0;
  static constexpr int oP = oA + TB * LA;
  static constexpr int oS1 = oP + TB * LB;
  static constexpr int oS2 = oS1 + TB * LS;
  static constexpr int oM = oA + TB * LA;              // phase 7, after A_h
  static constexpr int oCb = oM + R * LB;
  static constexpr int end1 = cmax(cmax(oS2 + TB * LS, N * LC), cmax(oCb + TB * LB, R * LB));
  static constexpr int oB = end1;
  static constexpr int oX = oB + D * LB;
  static constexpr int szX = cmax(TB * LA, D * LB);
  static constexpr int oNrm = oX + szX;
  static constexpr int oSig = oNrm + N;
  static constexpr int oPerm = oSig + N;
  static constexpr int oAct = oPerm + N;
  static constexpr int oInv = oAct + R;
  static constexpr int oDot = oInv + cmax(TB, R);
  static constexpr int floats = oDot + R;
  static constexpr size_t bytes = (size_t)floats * 4;
  static constexpr int kMaxHeads = szX / (2 * D);      // rem and vec of the null completion
  static_assert(oP % 4 == 0 && oS1 % 4 == 0 && oS2 % 4 == 0 && oM % 4 == 0 && oCb % 4 == 0 &&
                    oB % 4 == 0 && oX % 4 == 0,
                "16-byte aligned regions");
};

template <int R, typename T>
__global__ __launch_bounds__(kThreads) void joint_fold_kernel(Model M, LayerSel sel, int64_t n_c, int xsel,
                                                              SeqTab tab) {
  using Ly = JointLayout<R>;
  constexpr int D = kHeadDim, TB = kBlock, N = Ly::N, NC = Ly::NC;
  constexpr int LA = Ly::LA, LB = Ly::LB, LC = Ly::LC, LS = Ly::LS;
  extern __shared__ float4 lds4[];
  float *lds = reinterpret_cast<float *>(lds4);
  __shared__ float red[kThreads / 64];
  __shared__ int s_int[2];
  __shared__ float s_f[2];
  const Dims &Dm = M.D;
  const int tid = threadIdx.x;
  const int H = Dm.kv_heads, HD = H * D;
  const int layer = sel.idx[blockIdx.y];
  // grid.x: sequences (one factor, xsel) or sequences x 2 (both, equal ranks)
  const int g = xsel < 0 ? blockIdx.x >> 1 : blockIdx.x, X = xsel < 0 ? blockIdx.x & 1 : xsel;
  if (!seq_in(tab, g)) return;
  if (tab.n) n_c = tab.nc[g];
  LayerPtrs P = layer_ptrs(M, layer), Po = layer_ptrs_out(M, layer);
  const float *basis = P.basis[X] + (size_t)g * HD * R;     // H*d x r (the H slices)
  float *basis_out = Po.basis[X] + (size_t)g * HD * R;
  const float *sing = P.sing[X] + (size_t)g * R;
  float *sing_out = Po.sing[X] + (size_t)g * R;
  float *msync = P.msync[X] + (size_t)g * R * R;
  T *coef = reinterpret_cast<T *>(Po.coef[X]) + (size_t)g * Dm.max_tokens * R;
  float *gres = P.jres[X] + (size_t)g * TB * HD;            // 64 x H*d
  float *gbn = P.jbn[X] + (size_t)g * HD * R;               // H*d x r
  const T *ring0 = reinterpret_cast<const T *>(X == 0 ? P.ringk : P.ringv) + (size_t)g * H * Dm.slots * D;
  const int s0 = (int)(n_c % Dm.slots), slots = Dm.slots;

  float *sA = lds + Ly::oA, *sP = lds + Ly::oP, *sS1 = lds + Ly::oS1, *sS2 = lds + Ly::oS2;
  float *sB = lds + Ly::oB, *sX = lds + Ly::oX, *core = lds + Ly::oA;
  float *sig = lds + Ly::oSig, *invd = lds + Ly::oInv, *dot = lds + Ly::oDot;
  int *perm = reinterpret_cast<int *>(lds + Ly::oPerm);
  int *act = reinterpret_cast<int *>(lds + Ly::oAct);

  // head h's 64 x d block columns from its ring; this thread's share of ||A_h||^2
  auto load_A = [&](int h) { return load_block<T, LA>(ring0 + (size_t)h * slots * D, X, s0, slots, sA); };
  // a d x r slice (rows h*d..) of an H*d x r matrix, into LDS at row stride LB
  auto load_slice = [&](const float *src, float *dst) {
    for (int i = tid; i < D * R / 4; i += kThreads) {
      const int f = (4 * i) / R, c = (4 * i) % R;
      st4(dst + f * LB + c, ld4(src + 4 * i));
    }
  };
  // columns h*d.. of the 64 x H*d scratch, to / from LDS at row stride LA
  auto load_cols = [&](int h, float *dst) {
    for (int i = tid; i < TB * D / 4; i += kThreads) {
      const int t = (4 * i) / D, f = (4 * i) % D;
      st4(dst + t * LA + f, ld4(gres + (size_t)t * HD + h * D + f));
    }
  };
  auto store_cols = [&](int h, const float *src) {
    for (int i = tid; i < TB * D / 4; i += kThreads) {
      const int t = (4 * i) / D, f = (4 * i) % D;
      st4(gres + (size_t)t * HD + h * D + f, ld4(src + t * LA + f));
    }
  };
  auto zero = [&](float *p, int n) {
    for (int i = tid; i < n; i += kThreads) p[i] = 0.f;
  };

  // ---------------- phase 1: projection (twice), residual, its Gram ----------
  zero(sP, TB * LB);
  zero(sS1, TB * LS);
  zero(sS2, TB * LS);
  __syncthreads();
  float asq = 0.f;
  for (int h = 0; h < H; ++h) {                    // P = A B
    asq += load_A(h);
    load_slice(basis + (size_t)h * D * R, sB);
    __syncthreads();
    gemm_mfma<TB, R, D, false, false>(sA, LA, sB, LB, [&](int t, int c, float v) { sP[t * LB + c] += v; });
    __syncthreads();
  }
  const float normA2 = block_sum(asq, red);
  for (int h = 0; h < H; ++h) {                    // T = (A - P B^T) B, into S1
    (void)load_A(h);
    load_slice(basis + (size_t)h * D * R, sB);
    __syncthreads();
    gemm_mfma<TB, D, R, false, true>(sP, LB, sB, LB, [&](int t, int f, float v) {
      sX[t * LA + f] = sA[t * LA + f] - v;
    });
    __syncthreads();
    gemm_mfma<TB, R, D, false, false>(sX, LA, sB, LB, [&](int t, int c, float v) { sS1[t * LS + c] += v; });
    __syncthreads();
  }
  for (int i = tid; i < TB * R; i += kThreads) {
    const int t = i / R, c = i % R;
    sP[t * LB + c] += sS1[t * LS + c];
  }
  __syncthreads();
  for (int h = 0; h < H; ++h) {                    // Res = A - P B^T; G = Res Res^T, into S2
    (void)load_A(h);
    load_slice(basis + (size_t)h * D * R, sB);
    __syncthreads();
    gemm_mfma<TB, D, R, false, true>(sP, LB, sB, LB, [&](int t, int f, float v) {
      sX[t * LA + f] = sA[t * LA + f] - v;
    });
    __syncthreads();
    store_cols(h, sX);
    gemm_mfma<TB, TB, D, false, true>(sX, LA, sX, LA, [&](int a, int b, float v) { sS2[a * LS + b] += v; });
    __syncthreads();
  }

  // ---------------- phase 2: Q by CholeskyQR2, against B once more ----------
  // (A is not needed until the last pass: its region holds each head's new
  // Q rows between the product that makes them and their store.)
  {
    float tr = 0.f;
#pragma unroll 8
    for (int t = 0; t < TB; ++t) tr += sS2[t * LS + t];
    const float tau = fmaxf(kGuardAbs * normA2, fminf(kGuard * normA2, kGuardRel * tr));
    chol_lds<TB>(sS2, LS, tau, invd);              // L0 in S2
  }
  tri_inverse<TB>(sS2, LS, invd, sS1, LS);         // L0^{-1} in S1
  __syncthreads();
  zero(sS2, TB * LS);
  __syncthreads();
  for (int h = 0; h < H; ++h) {                    // Q0 = L0^{-1} Res; G1 = Q0 Q0^T, into S2
    load_cols(h, sX);
    __syncthreads();
    gemm_mfma<TB, D, TB, false, false>(sS1, LS, sX, LA, [&](int t, int f, float v) { sA[t * LA + f] = v; });
    __syncthreads();
    store_cols(h, sA);
    gemm_mfma<TB, TB, D, false, true>(sA, LA, sA, LA, [&](int a, int b, float v) { sS2[a * LS + b] += v; });
    __syncthreads();
  }
  chol_lds<TB>(sS2, LS, 0.25f, invd);              // L1 in S2
  tri_inverse<TB>(sS2, LS, invd, sS1, LS);         // L1^{-1} in S1
  __syncthreads();
  zero(sS2, TB * LS);
  __syncthreads();
  for (int h = 0; h < H; ++h) {                    // Q1 = L1^{-1} Q0; T = Q1 B, into S2
    load_cols(h, sX);
    load_slice(basis + (size_t)h * D * R, sB);
    __syncthreads();
    gemm_mfma<TB, D, TB, false, false>(sS1, LS, sX, LA, [&](int t, int f, float v) { sA[t * LA + f] = v; });
    __syncthreads();
    store_cols(h, sA);
    gemm_mfma<TB, R, D, false, false>(sA, LA, sB, LB, [&](int t, int c, float v) { sS2[t * LS + c] += v; });
    __syncthreads();
  }
  zero(sS1, TB * LS);
  __syncthreads();
  for (int h = 0; h < H; ++h) {                    // Q = Q1 - T B^T; A Q^T, into S1
    load_cols(h, sX);
    load_slice(basis + (size_t)h * D * R, sB);
    (void)load_A(h);
    __syncthreads();
    gemm_mfma<TB, D, R, false, true>(sS2, LS, sB, LB, [&](int t, int f, float v) { sX[t * LA + f] -= v; });
    __syncthreads();
    store_cols(h, sX);
    gemm_mfma<TB, TB, D, false, true>(sA, LA, sX, LA, [&](int t, int j, float v) { sS1[t * LS + j] += v; });
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
      v[j] = c < R ? sP[t * LB + c] : sS1[t * LS + (c - R)];
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

  // ---------------- phase 6: B_new = [B Q^T] V'[:, :r], a head at a time ----
  const float sig0 = sig[perm[0]];
  const float tol_null = 64.f * N * FLT_EPSILON * sig0;
  if (!isfinite(sig0) && tid == 0) set_flag(M.sh, 1);
  {
    // On the matrix cores, as gemm_mfma_part: 16 x 16 tiles (16 basis rows f,
    // 16 new columns k) dealt to the waves; the B operand is row perm[k] of
    // the core, read along its columns (contiguous), then each column is
    // scaled by 1/s'_k (0 for a null direction).
    constexpr int TN = R / 16, TILES = (D / 16) * TN, NW = kThreads / 64;
    const int lane = tid & 63, wave = tid >> 6, j = lane & 15, g = lane >> 4;
    for (int h = 0; h < H; ++h) {
      load_slice(basis + (size_t)h * D * R, sB);
      load_cols(h, sX);                            // Q_h
      __syncthreads();
      for (int tile = wave; tile < TILES; tile += NW) {
        const int f0 = (tile / TN) * 16, k0 = (tile % TN) * 16;
        const int row = perm[k0 + j];
        const float *zr = core + row * LC;         // this lane's new column k0 + j
        floatx4 acc = zero4();
#pragma unroll 2
        for (int c0 = 0; c0 < R; c0 += 16) {       // B_h (f, c) x V'(c, k)
          const int cb = c0 + 4 * g;
          const float4 x = ld4(sB + (f0 + j) * LB + cb);
          const float4 z = ld4(zr + cb);
          acc = mfma4(x.x, z.x, acc);
          acc = mfma4(x.y, z.y, acc);
          acc = mfma4(x.z, z.z, acc);
          acc = mfma4(x.w, z.w, acc);
        }
#pragma unroll 2
        for (int j0 = 0; j0 < TB; j0 += 16) {      // Q_h^T (f, j) x V'(R + j, k)
          const int jb = j0 + 4 * g;
          const float4 z = ld4(zr + R + jb);
          acc = mfma4(sX[(jb + 0) * LA + f0 + j], z.x, acc);
          acc = mfma4(sX[(jb + 1) * LA + f0 + j], z.y, acc);
          acc = mfma4(sX[(jb + 2) * LA + f0 + j], z.z, acc);
          acc = mfma4(sX[(jb + 3) * LA + f0 + j], z.w, acc);
        }
        const float zs = sig[row] > tol_null ? 1.f / sig[row] : 0.f;
        float *dst = gbn + ((size_t)h * D + f0 + 4 * g) * R + k0 + j;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)r * R] = acc[r] * zs;
      }
      __syncthreads();             // sB, sX are reloaded for the next head
    }
  }
  // null completion, as in the per-head fold, over the H*d rows in scratch:
  // each column whose singular value is ~0 becomes the unit vector with the
  // largest remainder against the columns kept so far, made orthogonal to them
  // by two Gram-Schmidt passes.
  float *rem = sX, *vec = sX + HD;
  for (int k = tid; k < R; k += kThreads) act[k] = sig[perm[k]] > tol_null;
  __syncthreads();
  for (int k = 0; k < R; ++k) {
    if (act[k]) continue;                      // uniform: act is shared
    for (int e = tid; e < HD; e += kThreads) {
      float s = 0.f;
      for (int c = 0; c < R; ++c) s += act[c] ? gbn[(size_t)e * R + c] * gbn[(size_t)e * R + c] : 0.f;
      rem[e] = 1.f - s;
    }
    __syncthreads();
    if (tid == 0) {
      int best = 0;
      for (int e = 1; e < HD; ++e)
        if (rem[e] > rem[best]) best = e;
      s_int[1] = best;
    }
    __syncthreads();
    for (int e = tid; e < HD; e += kThreads) vec[e] = (e == s_int[1]) ? 1.f : 0.f;
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
      for (int c = tid; c < R; c += kThreads) {
        float s = 0.f;
        if (act[c])
          for (int f = 0; f < HD; ++f) s += gbn[(size_t)f * R + c] * vec[f];
        dot[c] = s;
      }
      __syncthreads();
      for (int f = tid; f < HD; f += kThreads) {
        float s = vec[f];
        for (int c = 0; c < R; ++c) s -= gbn[(size_t)f * R + c] * dot[c];
        vec[f] = s;
      }
      __syncthreads();
    }
    if (tid == 0) {
      float s = 0.f;
      for (int f = 0; f < HD; ++f) s += vec[f] * vec[f];
      s_f[1] = sqrtf(s);
    }
    __syncthreads();
    for (int f = tid; f < HD; f += kThreads) gbn[(size_t)f * R + k] = vec[f] / s_f[1];
    __syncthreads();
    if (tid == 0) act[k] = 1;
    __syncthreads();
  }

  // Re-orthonormalize B_new (one CholeskyQR pass on its columns, as in the
  // per-head fold): G_b = sum_h B_new_h^T B_new_h over the dead core region.
  {
    float *sGb = lds + Ly::oA;
    zero(sGb, R * LB);
    __syncthreads();
    for (int h = 0; h < H; ++h) {
      load_slice(gbn + (size_t)h * D * R, sX);
      __syncthreads();
      gemm_mfma<R, R, D, true, false>(sX, LB, sX, LB, [&](int a, int b, float v) { sGb[a * LB + b] += v; });
      __syncthreads();
    }
    chol_lds<R>(sGb, LB, 0.25f, invd);
    for (int e = tid; e < HD; e += kThreads) {
      float x[R];
      float *row = gbn + (size_t)e * R;
#pragma unroll
      for (int c = 0; c < R; c += 4) {
        const float4 w = ld4(row + c);
        x[c] = w.x; x[c + 1] = w.y; x[c + 2] = w.z; x[c + 3] = w.w;
      }
      fwd_solve<R>(x, sGb, LB, invd);
#pragma unroll
      for (int c = 0; c < R; c += 4) st4(row + c, make_float4(x[c], x[c + 1], x[c + 2], x[c + 3]));
    }
    __syncthreads();
  }

  // ---------------- phase 7: M, block coefficients, new basis --------------
  {
    float *sM = lds + Ly::oM, *sCb = lds + Ly::oCb;
    zero(sM, R * LB);
    zero(sCb, TB * LB);
    __syncthreads();
    for (int h = 0; h < H; ++h) {
      load_slice(basis + (size_t)h * D * R, sB);
      load_slice(gbn + (size_t)h * D * R, sX);
      (void)load_A(h);
      __syncthreads();
      // two independent products, one per half of the workgroup
      constexpr int NW2 = kThreads / 128;
      const int wave = tid >> 6;
      if (wave < NW2)
        gemm_mfma_part<R, R, D, true, false>(sB, LB, sX, LB, [&](int c, int k, float v) { sM[c * LB + k] += v; },
                                             wave, NW2);
      else
        gemm_mfma_part<TB, R, D, false, false>(sA, LA, sX, LB, [&](int t, int k, float v) { sCb[t * LB + k] += v; },
                                               wave - NW2, NW2);
      __syncthreads();
    }
    for (int i = tid; i < R * R; i += kThreads) msync[i] = sM[(i / R) * LB + i % R];
    for (int i = tid; i < TB * R; i += kThreads)
      Store<T>::store(coef, (size_t)(n_c + i / R) * R + i % R, sCb[(i / R) * LB + i % R]);
    // every read of the old basis is done: it may be overwritten in place
    for (int i = tid; i < HD * R / 4; i += kThreads) st4(basis_out + 4 * i, ld4(gbn + 4 * i));
    if (tid < R) sing_out[tid] = sig[perm[tid]];
  }
}

template <int R, typename T>
hipError_t launch_joint_t(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                          const SeqTab &tab) {
  static bool attr = false;
  const size_t bytes = JointLayout<R>::bytes;
  if (M.D.kv_heads > JointLayout<R>::kMaxHeads) return hipErrorInvalidValue;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&joint_fold_kernel<R, T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(x < 0 ? M.D.cunits * 2 : M.D.cunits, sel.n);
  hipLaunchKernelGGL((joint_fold_kernel<R, T>), grid, dim3(kThreads), bytes, s, M, sel, n_c, x, tab);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_joint(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                          const SeqTab &tab) {
  const int r = x == 1 ? M.D.rv : M.D.rk;
  if (x < 0 && M.D.rk != M.D.rv) return hipErrorInvalidValue;
  switch (r) {
    case 16: return launch_joint_t<16, T>(M, sel, n_c, x, s, tab);
    case 32: return launch_joint_t<32, T>(M, sel, n_c, x, s, tab);
    case 64: return launch_joint_t<64, T>(M, sel, n_c, x, s, tab);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_joint_fold(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                             const SeqTab &tab) {
  return M.D.storage == 1 ? dispatch_joint<bf16_t>(M, sel, n_c, x, s, tab)
                          : dispatch_joint<float>(M, sel, n_c, x, s, tab);
}

}  // namespace iskv
