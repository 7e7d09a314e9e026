// Cache maintenance kernels for gfx950: ring append, basis synchronization of
// the stored coefficients, and the decode operand copy of the basis (the
// block-update fold itself is in fold.hip).
//
// Page: "iS-KV -- Basis-synchronized online low-rank KV compression -- What does
// it mean?" (learnaivisually.com), cited as [iS-KV explainer]:
//   - append: recent tokens stay exact (window paragraph); keys are stored
//     before RoPE (Jargon "Pre-RoPE keys").
//   - sync: old coefficients are rewritten for the new basis (FAQ "What is
//     basis synchronization?").
#include <cfloat>
#include <cstdint>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Reset: basis = I[:, :r] (the basis before any block has been seen).
// ---------------------------------------------------------------------------
__global__ void reset_basis_kernel(Model M, int layer) {
  const Dims &D = M.D;
  LayerPtrs P = layer_ptrs(M, layer);
  for (int x = 0; x < 2; ++x) {
    const int r = x ? D.rv : D.rk;
    const size_t n = (size_t)D.units * D.d * r;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x) {
      const int c = (int)(i % r);
      const int f = (int)((i / r) % D.d);
      P.basis[x][i] = (f == c) ? 1.f : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// Append: grid (n tokens, kv heads, batch), block = head_dim threads.
// ---------------------------------------------------------------------------
template <typename T, typename In>
__global__ void append_kernel(Model M, int layer, const In *k, const In *v, int n, int64_t pos0,
                              SeqTab tab) {
  const Dims &D = M.D;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, f = threadIdx.x;
  if (!seq_in(tab, b) || t >= (tab.n ? tab.aux[b] : n)) return;     // ragged: this sequence's count
  if (tab.n) pos0 = tab.len[b];
  const int u = b * D.kv_heads + h;
  const size_t src = (((size_t)b * n + t) * D.kv_heads + h) * D.d + f;
  const float kx = Store<In>::load(k, src);
  const float vx = Store<In>::load(v, src);
  if (!isfinite(kx) || !isfinite(vx)) set_flag(M.sh, 4);
  LayerPtrs P = layer_ptrs(M, layer);
  const int64_t pos = pos0 + t;
  // protected prefix rows (positions < P) keep their own exact store; later
  // positions go to ring slot pos % slots.  Both keep V transposed.
  const bool pre = pos < D.prefix;
  const int rows = pre ? D.prefix : D.slots;
  const int slot = pre ? (int)pos : (int)(pos % D.slots);
  T *rk = reinterpret_cast<T *>(pre ? P.prek : P.ringk) + (size_t)u * rows * D.d;
  T *rv = reinterpret_cast<T *>(pre ? P.prev : P.ringv) + (size_t)u * rows * D.d;
  Store<T>::store(rk, (size_t)slot * D.d + f, kx);
  Store<T>::store(rv, (size_t)f * rows + slot, vx);
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
  const int u = blockIdx.x;                    // key basis of unit u
  LayerPtrs P = layer_ptrs(M, l);
  const float *B = P.basis[0] + (size_t)u * D.d * D.rk;
  uint8_t *F = P.frag + (size_t)u * 4 * D.d * D.rk;
  const int r = D.rk, per = r / 4;            // coefficients per lane
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
// Sync: C[t] <- C[t] M for rows t < n_old (page: FAQ "What is basis
// synchronization?" -- every stored coefficient row is rewritten for the new
// basis).  An N x r by r x r product, streamed once through HBM.
//
// bf16 storage: MFMA.  Each wave takes 8 (4 at r = 128) tiles of 16 rows
// and computes C_new^T = M^T C^T: A operand = M^T as bf16 high + low parts
// (M = hi + lo to ~2^-16, so C M is exact to float accumulation), B operand =
// 16 coefficient rows as stored (exact bf16), output rounded once to bf16.
// f32 storage: one row per thread on the vector ALUs.
// grid (row tiles, units (one factor) or units*2 (both), layers)
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(kThreads) void sync_mfma_kernel(Model M, LayerSel sel, int64_t n_old, int xsel,
                                                              SeqTab tab) {
  static_assert(R == 16 || R == 32 || R == 64 || R == 128, "MFMA sync ranks");
  constexpr int KB = R >= 32 ? R / 32 : 1;      // K blocks (32 wide; one of 16 at r = 16)
  constexpr int MB = R / 16;                    // output column blocks
  constexpr int TPW = R == 128 ? 4 : 8;         // 16-row tiles per wave
  const Dims &D = M.D;
  const int l = sel.idx[blockIdx.z];
  // grid.y: units (one factor, xsel) or units x 2 (both, equal ranks)
  const int u = xsel < 0 ? blockIdx.y >> 1 : blockIdx.y, x = xsel < 0 ? blockIdx.y & 1 : xsel;
  if (!seq_in(tab, u / D.kv_heads)) return;     // ragged: a sequence that did not fold
  if (tab.n) n_old = tab.nc[u / D.kv_heads];
  LayerPtrs P = layer_ptrs(M, l);
  const float *Ms = P.msync[x] + (size_t)u * R * R;
  uint16_t *C = reinterpret_cast<uint16_t *>(P.coef[x]) + (size_t)u * D.max_tokens * R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, rho = lane >> 4;
  const int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * TPW * 16;
  if (base >= n_old) return;                    // uniform per wave
  // every input row of the wave is in registers before any output is written
  uint4_ b[TPW][KB];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t tok = base + 16 * t + n;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (R >= 32) {
        b[t][kb] = tok < n_old ? *reinterpret_cast<const uint4_ *>(C + tok * R + kb * 32 + 8 * rho)
                               : uint4_{0u, 0u, 0u, 0u};
      } else {
        const uint2_ v = tok < n_old ? *reinterpret_cast<const uint2_ *>(C + tok * R + 4 * rho)
                                     : uint2_{0u, 0u};
        b[t][kb] = uint4_{v.x, v.y, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // A operand: M^T rows mb*16 + n, high and low bf16 parts
    uint4_ ahi[KB], alo[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      constexpr int PAIRS = R >= 32 ? 4 : 2;
      unsigned h[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < PAIRS; ++i) {
        const int c = R >= 32 ? kb * 32 + 8 * rho + 2 * i : 4 * rho + 2 * i;
        split2(Ms[c * R + mb * 16 + n], Ms[(c + 1) * R + mb * 16 + n], h[i], lo[i]);
      }
      ahi[kb] = uint4_{h[0], h[1], h[2], h[3]};
      alo[kb] = uint4_{lo[0], lo[1], lo[2], lo[3]};
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      floatx4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (R >= 32) {
          acc = mfma32(ahi[kb], b[t][kb], acc);
          acc = mfma32(alo[kb], b[t][kb], acc);
        } else {
          const uint2_ bb{b[t][kb].x, b[t][kb].y};
          acc = mfma16(uint2_{ahi[kb].x, ahi[kb].y}, bb, acc);
          acc = mfma16(uint2_{alo[kb].x, alo[kb].y}, bb, acc);
        }
      }
      const int64_t tok = base + 16 * t + n;
      if (tok < n_old) {
        const bf16x2 p0 = __builtin_convertvector((floatx2){acc[0], acc[1]}, bf16x2);
        const bf16x2 p1 = __builtin_convertvector((floatx2){acc[2], acc[3]}, bf16x2);
        *reinterpret_cast<uint2_ *>(C + tok * R + mb * 16 + 4 * rho) =
            uint2_{__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1)};
      }
    }
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void sync_valu_kernel(Model M, LayerSel sel, int64_t n_old, int xsel,
                                                              SeqTab tab) {
  __shared__ float4 sM4[R * R / 4];
  const float *sM = reinterpret_cast<const float *>(sM4);
  const Dims &D = M.D;
  const int l = sel.idx[blockIdx.z];
  const int u = xsel < 0 ? blockIdx.y >> 1 : blockIdx.y, x = xsel < 0 ? blockIdx.y & 1 : xsel;
  if (!seq_in(tab, u / D.kv_heads)) return;     // block-uniform, before the barrier
  if (tab.n) n_old = tab.nc[u / D.kv_heads];
  LayerPtrs P = layer_ptrs(M, l);
  const float4 *Ms = reinterpret_cast<const float4 *>(P.msync[x] + (size_t)u * R * R);
  float *C = reinterpret_cast<float *>(P.coef[x]) + (size_t)u * D.max_tokens * R;
  for (int i = threadIdx.x; i < R * R / 4; i += blockDim.x) sM4[i] = Ms[i];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_old) return;
  float row[R];
#pragma unroll
  for (int c = 0; c < R; c += 4) {
    const float4 v = *reinterpret_cast<const float4 *>(C + t * R + c);
    row[c] = v.x; row[c + 1] = v.y; row[c + 2] = v.z; row[c + 3] = v.w;
  }
#pragma clang loop unroll(disable)
  for (int k0 = 0; k0 < R; k0 += 4) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const float x = row[c];
      const float4 m = *reinterpret_cast<const float4 *>(sM + c * R + k0);
      a0 = fmaf(x, m.x, a0);
      a1 = fmaf(x, m.y, a1);
      a2 = fmaf(x, m.z, a2);
      a3 = fmaf(x, m.w, a3);
      // keep the scheduler from hoisting every LDS read of M at once
      if ((c & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
    *reinterpret_cast<float4 *>(C + t * R + k0) = make_float4(a0, a1, a2, a3);
  }
}

template <int R, typename T>
hipError_t launch_sync_t(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                         const SeqTab &tab) {
  if (n_old <= 0) return hipSuccess;
  const unsigned ny = x < 0 ? M.D.units * 2 : M.D.units;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int64_t rows_per_block = (int64_t)(kThreads / 64) * (R == 128 ? 4 : 8) * 16;
    dim3 grid((unsigned)((n_old + rows_per_block - 1) / rows_per_block), ny, sel.n);
    hipLaunchKernelGGL((sync_mfma_kernel<R>), grid, dim3(kThreads), 0, s, M, sel, n_old, x, tab);
  } else {
    dim3 grid((unsigned)((n_old + kThreads - 1) / kThreads), ny, sel.n);
    hipLaunchKernelGGL((sync_valu_kernel<R>), grid, dim3(kThreads), 0, s, M, sel, n_old, x, tab);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_sync(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                         const SeqTab &tab) {
  const int r = x == 1 ? M.D.rv : M.D.rk;
  if (x < 0 && M.D.rk != M.D.rv) return hipErrorInvalidValue;
  switch (r) {
    case 16: return launch_sync_t<16, T>(M, sel, n_old, x, s, tab);
    case 32: return launch_sync_t<32, T>(M, sel, n_old, x, s, tab);
    case 64: return launch_sync_t<64, T>(M, sel, n_old, x, s, tab);
    case 128: return launch_sync_t<128, T>(M, sel, n_old, x, s, tab);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reset_layer(const Model &M, int layer, hipStream_t s) {
  hipLaunchKernelGGL(reset_basis_kernel, dim3(256), dim3(256), 0, s, M, layer);
  return hipGetLastError();
}

hipError_t launch_append(const Model &M, int layer, const void *k, const void *v, int n,
                         int in_dtype, int64_t pos0, hipStream_t s, const SeqTab &tab) {
  if (n <= 0) return hipSuccess;
  dim3 grid(n, M.D.kv_heads, M.D.batch);
  if (M.D.storage == 1) {
    if (in_dtype == 1)
      hipLaunchKernelGGL((append_kernel<bf16_t, bf16_t>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const bf16_t *)k, (const bf16_t *)v, n, pos0, tab);
    else
      hipLaunchKernelGGL((append_kernel<bf16_t, float>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const float *)k, (const float *)v, n, pos0, tab);
  } else {
    if (in_dtype == 1)
      hipLaunchKernelGGL((append_kernel<float, bf16_t>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const bf16_t *)k, (const bf16_t *)v, n, pos0, tab);
    else
      hipLaunchKernelGGL((append_kernel<float, float>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const float *)k, (const float *)v, n, pos0, tab);
  }
  return hipGetLastError();
}

hipError_t launch_sync(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                       const SeqTab &tab) {
  return M.D.storage == 1 ? dispatch_sync<bf16_t>(M, sel, n_old, x, s, tab)
                          : dispatch_sync<float>(M, sel, n_old, x, s, tab);
}

hipError_t launch_prep_frag(const Model &M, const LayerSel &sel, hipStream_t s) {
  dim3 grid(M.D.units, sel.n);
  hipLaunchKernelGGL(prep_frag_kernel, grid, dim3(256), 0, s, M, sel);
  return hipGetLastError();
}

}  // namespace iskv
