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
// Reset: basis = I[:, :r] (the basis before any block has been seen).  A joint
// basis is the identity over its H*d rows: only head 0's slice holds ones.
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
      const int h = D.joint ? (int)(i / ((size_t)D.d * r)) % D.kv_heads : 0;
      P.basis[x][i] = (h * D.d + f == c) ? 1.f : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// Append: grid (n tokens, kv heads, batch), block = head_dim threads.
// ---------------------------------------------------------------------------
template <typename T, typename In>
__global__ void append_kernel(Model M, int layer, const In *k, const In *v, int n, int n_stride,
                              int64_t pos0, SeqTab tab) {
  const Dims &D = M.D;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, f = threadIdx.x;
  if (!seq_in(tab, b) || t >= (tab.n ? tab.aux[b] : n)) return;     // ragged: this sequence's count
  if (tab.n) pos0 = tab.len[b];
  const int u = b * D.kv_heads + h;
  const size_t src = (((size_t)b * n_stride + t) * D.kv_heads + h) * D.d + f;
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
  LayerPtrs P = layer_ptrs_out(M, l);           // the generation the maintenance wrote
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
      // fp16 (round to nearest) operand of the f16 key product: chunk 2 kb
      // holds coefficients rho * r/4 + 8 kb .. + 7 (r >= 32; r = 16: chunk 0,
      // coefficients 4 rho .. + 3 in slots 0..3); the other slots are zero
      uint16_t *o = reinterpret_cast<uint16_t *>(dst);
      for (int j = 0; j < 8; ++j) {
        const bool used = (r >= 32) ? (ch & 1) == 0 : j < 4;
        const int c = (r >= 32) ? (ch >> 1) * 8 + j : j;
        o[j] = used ? __builtin_bit_cast(uint16_t, (_Float16)src[c]) : 0;
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
// basis).  An N x r by r x r product, streamed once through HBM.  In place,
// or, with copy-on-write maintenance, from the current generation into the
// other one (a row is read in full before its output is written either way).
//
// bf16 storage: MFMA.  Each wave takes 8 (4 at r = 128) tiles of 16 rows
// and computes C_new^T = M^T C^T: A operand = M^T as three bf16 parts
// (M = hi + mid + lo to ~2^-24, i.e. M as an fp32 value; with two parts the
// ~2^-17 representation error of M moved one rounding of C M in a few
// hundred to the neighbouring bf16 value, which accumulates sync after sync),
// B operand = 16 coefficient rows as stored (exact bf16), so every product is
// exact and the output is rounded once to bf16.
// f32 storage: one row per thread on the vector ALUs.
// grid (row tiles, coefficient units (one factor) or twice that (both), layers)
// ---------------------------------------------------------------------------
// Bulk mode (prefill): the matrix depends on the row's 64-row block (see
// bulk_suffix_kernel): rows older than n_c0 take slot 0, rows of bulk block j
// slot j + 1, the last bulk block's rows are skipped; one block per wave.
struct BulkSync {
  const float *mbulk;     // null: plain sync with the layer's M
  int bulk_blocks;
  int nblk;
  int64_t n_c0;
};

__device__ __forceinline__ const float *bulk_matrix(const Model &M, const BulkSync &bk, int li, int x, int u,
                                                    int R, int64_t row) {
  const int64_t blk = row < bk.n_c0 ? 0 : (row - bk.n_c0) / kBlock + 1;
  if (blk >= bk.nblk) return nullptr;
  return bk.mbulk + (size_t)li * bulk_layer_floats(M.D, bk.bulk_blocks) +
         (x ? (size_t)M.D.units * bk.bulk_blocks * M.D.rk * M.D.rk : 0) +
         ((size_t)u * bk.bulk_blocks + blk) * R * R;
}

template <int R, bool BULK>
__global__ __launch_bounds__(kThreads) void sync_mfma_kernel(Model M, LayerSel sel, int64_t n_old, int xsel,
                                                              SeqTab tab, BulkSync bk) {
  static_assert(R == 16 || R == 32 || R == 64 || R == 128, "MFMA sync ranks");
  constexpr int KB = R >= 32 ? R / 32 : 1;      // K blocks (32 wide; one of 16 at r = 16)
  constexpr int MB = R / 16;                    // output column blocks
  constexpr int TPW = BULK ? 4 : (R == 128 ? 4 : 8);   // 16-row tiles per wave
  const Dims &D = M.D;
  const int l = sel.idx[blockIdx.z];
  // grid.y: coefficient units (one factor, xsel) or twice that (both, equal ranks)
  const int u = xsel < 0 ? blockIdx.y >> 1 : blockIdx.y, x = xsel < 0 ? blockIdx.y & 1 : xsel;
  if (!seq_in(tab, cunit_seq(D, u))) return;    // ragged: a sequence that did not fold
  if (tab.n) n_old = tab.nc[cunit_seq(D, u)];
  LayerPtrs P = layer_ptrs(M, l);
  const float *Ms = P.msync[x] + (size_t)u * R * R;
  const uint16_t *C = reinterpret_cast<const uint16_t *>(P.coef[x]) + (size_t)u * D.max_tokens * R;
  uint16_t *Co = reinterpret_cast<uint16_t *>(layer_ptrs_out(M, l).coef[x]) + (size_t)u * D.max_tokens * R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, rho = lane >> 4;
  const int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * TPW * 16;
  // plain sync at r >= 32: every wave of the workgroup uses the same M, so
  // the workgroup splits it into LDS in the A-operand order -- at once up to
  // r = 64, in two halves of the M-blocks at r = 128 (48 KiB of LDS each) --
  // and the waves read their operands from there.  The first (or only) part
  // of M is requested before the rows, so its split waits for M alone (loads
  // complete in order).  At r = 16 each wave splits its own operands (cheap
  // there; the barrier would cost more).
  constexpr bool kShareM = !BULK && R >= 32;
  constexpr int PAIRS = R >= 32 ? 4 : 2;
  constexpr int MBP = R == 128 ? MB / 2 : MB;    // M-blocks per LDS phase
  constexpr int NPH = MB / MBP;
  __shared__ uint4_ s_a[kShareM ? MBP * KB * 3 * 64 : 1];
  if (!kShareM && base >= n_old) return;        // uniform per wave
  if constexpr (BULK) {
    Ms = bulk_matrix(M, bk, blockIdx.z, x, u, R, base);
    if (!Ms) return;
  }
  // slot e of a phase: pair i of lane ln's A operand of (local) M-block mbl,
  // K-block kb; (MBP * KB * 64 * 4) / kThreads slots a thread
  constexpr int NIT = kShareM ? MBP * KB : 1;
  static_assert(!kShareM || kThreads == 256, "slots per thread");
  float mv0[NIT], mv1[NIT];
  auto fetch_m = [&](int ph) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int e = threadIdx.x + j * kThreads;
      const int i = e & 3, ln = (e >> 2) & 63, kb = (e >> 8) % KB, mb = ph * MBP + (e >> 8) / KB;
      const int c = kb * 32 + 8 * (ln >> 4) + 2 * i;
      mv0[j] = Ms[c * R + mb * 16 + (ln & 15)];
      mv1[j] = Ms[(c + 1) * R + mb * 16 + (ln & 15)];
    }
  };
  if constexpr (kShareM) fetch_m(0);
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
  // output column block mb from its A operand: M^T rows mb*16 + n, as high,
  // middle and low bf16 parts
  auto column_block = [&](int mb, const uint4_ (&ahi)[KB], const uint4_ (&amid)[KB], const uint4_ (&alo)[KB]) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      floatx4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // smallest parts first: they are added to the accumulator while it
        // is still small
        if constexpr (R >= 32) {
          acc = mfma32(alo[kb], b[t][kb], acc);
          acc = mfma32(amid[kb], b[t][kb], acc);
          acc = mfma32(ahi[kb], b[t][kb], acc);
        } else {
          const uint2_ bb{b[t][kb].x, b[t][kb].y};
          acc = mfma16(uint2_{alo[kb].x, alo[kb].y}, bb, acc);
          acc = mfma16(uint2_{amid[kb].x, amid[kb].y}, bb, acc);
          acc = mfma16(uint2_{ahi[kb].x, ahi[kb].y}, bb, acc);
        }
      }
      const int64_t tok = base + 16 * t + n;
      if (tok < n_old) {
        const bf16x2 p0 = __builtin_convertvector((floatx2){acc[0], acc[1]}, bf16x2);
        const bf16x2 p1 = __builtin_convertvector((floatx2){acc[2], acc[3]}, bf16x2);
        *reinterpret_cast<uint2_ *>(Co + tok * R + mb * 16 + 4 * rho) =
            uint2_{__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1)};
      }
    }
  };
  if constexpr (kShareM) {
    unsigned *sa = reinterpret_cast<unsigned *>(s_a);
    const bool active = base < n_old;           // uniform per wave; every wave takes the barriers
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      if (ph > 0) {
        __syncthreads();                        // the previous phase's operands are read
        fetch_m(ph);
      }
#pragma unroll
      for (int j = 0; j < NIT; ++j) {
        const int e = threadIdx.x + j * kThreads;
        const int i = e & 3, ln = (e >> 2) & 63;
        unsigned h, md, lo;
        split3(mv0[j], mv1[j], h, md, lo);
        const int q = (e >> 8) * 3 * 64 + ln;   // (mbl * KB + kb) * 3 * 64 + ln
        sa[(q + 0 * 64) * 4 + i] = h;
        sa[(q + 1 * 64) * 4 + i] = md;
        sa[(q + 2 * 64) * 4 + i] = lo;
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int mbl = 0; mbl < MBP; ++mbl) {
          uint4_ ahi[KB], amid[KB], alo[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int q = (mbl * KB + kb) * 3 * 64 + lane;
            ahi[kb] = s_a[q];
            amid[kb] = s_a[q + 64];
            alo[kb] = s_a[q + 128];
          }
          column_block(ph * MBP + mbl, ahi, amid, alo);
        }
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      uint4_ ahi[KB], amid[KB], alo[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        unsigned h[4] = {0u, 0u, 0u, 0u}, md[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < PAIRS; ++i) {
          const int c = R >= 32 ? kb * 32 + 8 * rho + 2 * i : 4 * rho + 2 * i;
          split3(Ms[c * R + mb * 16 + n], Ms[(c + 1) * R + mb * 16 + n], h[i], md[i], lo[i]);
        }
        ahi[kb] = uint4_{h[0], h[1], h[2], h[3]};
        amid[kb] = uint4_{md[0], md[1], md[2], md[3]};
        alo[kb] = uint4_{lo[0], lo[1], lo[2], lo[3]};
      }
      column_block(mb, ahi, amid, alo);
    }
  }
}

template <int R, bool BULK>
__global__ __launch_bounds__(kThreads) void sync_valu_kernel(Model M, LayerSel sel, int64_t n_old, int xsel,
                                                              SeqTab tab, BulkSync bk) {
  __shared__ float4 sM4[R * R / 4];
  const float *sM = reinterpret_cast<const float *>(sM4);
  const Dims &D = M.D;
  const int l = sel.idx[blockIdx.z];
  const int u = xsel < 0 ? blockIdx.y >> 1 : blockIdx.y, x = xsel < 0 ? blockIdx.y & 1 : xsel;
  if (!seq_in(tab, cunit_seq(D, u))) return;    // block-uniform, before the barrier
  if (tab.n) n_old = tab.nc[cunit_seq(D, u)];
  LayerPtrs P = layer_ptrs(M, l);
  const float4 *Ms = reinterpret_cast<const float4 *>(P.msync[x] + (size_t)u * R * R);
  if constexpr (BULK) {                         // one 64-row block per workgroup (block-uniform)
    const float *mb = bulk_matrix(M, bk, blockIdx.z, x, u, R, (int64_t)blockIdx.x * blockDim.x);
    if (!mb) return;
    Ms = reinterpret_cast<const float4 *>(mb);
  }
  const float *C = reinterpret_cast<const float *>(P.coef[x]) + (size_t)u * D.max_tokens * R;
  float *Co = reinterpret_cast<float *>(layer_ptrs_out(M, l).coef[x]) + (size_t)u * D.max_tokens * R;
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
    *reinterpret_cast<float4 *>(Co + t * R + k0) = make_float4(a0, a1, a2, a3);
  }
}

template <int R, typename T>
hipError_t launch_sync_t(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                         const SeqTab &tab, const BulkSync &bk) {
  if (n_old <= 0) return hipSuccess;
  const unsigned ny = x < 0 ? M.D.cunits * 2 : M.D.cunits;
  const bool bulk = bk.mbulk != nullptr;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int64_t rows_per_block = (int64_t)(kThreads / 64) * (bulk ? 4 : (R == 128 ? 4 : 8)) * 16;
    dim3 grid((unsigned)((n_old + rows_per_block - 1) / rows_per_block), ny, sel.n);
    if (bulk)
      hipLaunchKernelGGL((sync_mfma_kernel<R, true>), grid, dim3(kThreads), 0, s, M, sel, n_old, x, tab, bk);
    else
      hipLaunchKernelGGL((sync_mfma_kernel<R, false>), grid, dim3(kThreads), 0, s, M, sel, n_old, x, tab, bk);
  } else {
    const int threads = bulk ? kBlock : kThreads;
    dim3 grid((unsigned)((n_old + threads - 1) / threads), ny, sel.n);
    if (bulk)
      hipLaunchKernelGGL((sync_valu_kernel<R, true>), grid, dim3(threads), 0, s, M, sel, n_old, x, tab, bk);
    else
      hipLaunchKernelGGL((sync_valu_kernel<R, false>), grid, dim3(threads), 0, s, M, sel, n_old, x, tab, bk);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_sync(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                         const SeqTab &tab, const BulkSync &bk) {
  const int r = x == 1 ? M.D.rv : M.D.rk;
  if (x < 0 && M.D.rk != M.D.rv) return hipErrorInvalidValue;
  switch (r) {
    case 16: return launch_sync_t<16, T>(M, sel, n_old, x, s, tab, bk);
    case 32: return launch_sync_t<32, T>(M, sel, n_old, x, s, tab, bk);
    case 64: return launch_sync_t<64, T>(M, sel, n_old, x, s, tab, bk);
    case 128: return launch_sync_t<128, T>(M, sel, n_old, x, s, tab, bk);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reset_layer(const Model &M, int layer, hipStream_t s) {
  hipLaunchKernelGGL(reset_basis_kernel, dim3(256), dim3(256), 0, s, M, layer);
  return hipGetLastError();
}

hipError_t launch_append(const Model &M, int layer, const void *k, const void *v, int n,
                         int in_dtype, int64_t pos0, hipStream_t s, const SeqTab &tab, int n_stride) {
  if (n <= 0) return hipSuccess;
  if (n_stride <= 0) n_stride = n;
  dim3 grid(n, M.D.kv_heads, M.D.batch);
  if (M.D.storage == 1) {
    if (in_dtype == 1)
      hipLaunchKernelGGL((append_kernel<bf16_t, bf16_t>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const bf16_t *)k, (const bf16_t *)v, n, n_stride, pos0, tab);
    else
      hipLaunchKernelGGL((append_kernel<bf16_t, float>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const float *)k, (const float *)v, n, n_stride, pos0, tab);
  } else {
    if (in_dtype == 1)
      hipLaunchKernelGGL((append_kernel<float, bf16_t>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const bf16_t *)k, (const bf16_t *)v, n, n_stride, pos0, tab);
    else
      hipLaunchKernelGGL((append_kernel<float, float>), grid, dim3(kHeadDim), 0, s, M, layer,
                         (const float *)k, (const float *)v, n, n_stride, pos0, tab);
  }
  return hipGetLastError();
}

hipError_t launch_sync(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                       const SeqTab &tab) {
  const BulkSync none{nullptr, 0, 0, 0};
  return M.D.storage == 1 ? dispatch_sync<bf16_t>(M, sel, n_old, x, s, tab, none)
                          : dispatch_sync<float>(M, sel, n_old, x, s, tab, none);
}

hipError_t launch_sync_bulk(const Model &M, const BulkIn &in, int64_t n_c0, int nblk, int x,
                            const float *mbulk, int bulk_blocks, hipStream_t s) {
  if (nblk < 2 && n_c0 <= M.D.prefix) return hipSuccess;     // nothing older than the last block
  LayerSel sel;
  sel.n = in.n;
  for (int i = 0; i < in.n; ++i) sel.idx[i] = in.layer[i];
  const BulkSync bk{mbulk, bulk_blocks, nblk, n_c0};
  const int64_t rows = n_c0 + (int64_t)(nblk - 1) * kBlock;  // up to the last bulk block
  return M.D.storage == 1 ? dispatch_sync<bf16_t>(M, sel, rows, x, s, SeqTab{}, bk)
                          : dispatch_sync<float>(M, sel, rows, x, s, SeqTab{}, bk);
}

hipError_t launch_prep_frag(const Model &M, const LayerSel &sel, hipStream_t s) {
  dim3 grid(M.D.units, sel.n);
  hipLaunchKernelGGL(prep_frag_kernel, grid, dim3(256), 0, s, M, sel);
  return hipGetLastError();
}

}  // namespace iskv
