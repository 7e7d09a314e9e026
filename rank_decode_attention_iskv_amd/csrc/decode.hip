// Decode attention over the mixed cache (exact window + low-rank history).
//
// Page: "iS-KV -- Basis-synchronized online low-rank KV compression -- What does
// it mean?" (learnaivisually.com), cited as [iS-KV explainer]: a new query
// attends over all of its predecessors (re-attention paragraph); old keys are
// rebuilt from their coefficients over the shared basis and RoPE is re-applied
// at the key's position (Jargon "Basis and coefficients", "Pre-RoPE keys").  Values are
// accumulated in coefficient space, sum_t p_t c_t, and mapped back once by the
// value basis: (p^T C) B^T = p^T (C B^T).
//
// Split-K: each workgroup attends over one token range of one (sequence, KV
// head) for all query heads of its group and writes a partial record
// (running max m, sum l, accumulator); a second, small kernel merges the
// records of each (sequence, KV head) by log-sum-exp and writes the output
// (the kernel boundary makes every record visible across the XCDs' L2s, so
// no device-wide fences are needed inside the decode kernel).
//
// Per wave and tile of 16 tokens (all on MFMA except RoPE and the softmax):
//   stream  the coefficient tiles of K and V are copied HBM -> LDS by direct
//           DMA loads (no registers), kept several tiles ahead in a per-wave
//           LDS ring;
//   keys    K^T (128 x 16) = B_K (128 x r) C_K^T (r x 16): bf16 storage, one
//           fp16 product per 32 coefficients, the basis rounded to fp16
//           (2^-11 relative) and the stored bf16 coefficients converted to
//           fp16 exactly; fp32 storage, fp32 MFMA.  Lane l holds features 16*mb + 4*(l/16)
//           + i, mb = 0..7, of token l%16: 16 RoPE pairs (f, f + 64), rotated
//           in registers at the token's position;
//   scores  S (16 tokens x 16 heads) = K~ Q~^T.  bf16 storage: the rotated
//           key rounded once to fp16 (2^-11 relative, below the bf16 rounding
//           of the stored coefficients), the query as fp16 hi + lo (two
//           products; with 4 query heads per KV head the low parts ride in
//           columns 4..7 of one product); fp32 storage: both sides split
//           bf16 hi/lo (hi*hi + hi*lo + lo*hi, ~2^-16).  Lane l gets head l%16 and tokens
//           4*(l/16)..+3, the A-operand layout of the value product; query
//           heads beyond the group are zero;
//   softmax running max per head in log2 units, rescaled lazily (only when
//           the max grows by more than 8, so p <= 2^8);
//   values  acc (16 heads x r) += P (16 x 16 tokens) C_V (16 tokens x r) with P
//           split bf16 hi/lo, C_V read transposed from the LDS ring.  Window
//           tiles read V^T straight from the transposed ring (acc over 128
//           features).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int kThreads = 256;

constexpr float kRescale = 8.f;

struct SplitPlan {
  int n_comp;        // splits over compressed tokens (positions P .. n_c-1)
  int comp_len;      // tokens per compressed split (multiple of 64)
  int n_win;         // splits over window tokens (positions n_c .. length-1)
  int win_len;       // tokens per window split (multiple of 16)
  int n_pre;         // splits over the protected prefix (positions 0 .. P-1)
  int pre_len;       // tokens per prefix split (multiple of 16)
  int win_rides;     // 1: n_win == n_comp and window split i is handled by the
                     // workgroup of compressed split i, after its compressed
                     // range (no workgroups of their own)
  // records: compressed splits first, then prefix splits, then window splits
};

// workgroups of one unit under a plan
__host__ __device__ inline int plan_workgroups(const SplitPlan &p) {
  return p.n_comp + p.n_pre + (p.win_rides ? 0 : p.n_win);
}

// A ragged batch's plans, one per sequence: blockIdx.x runs over the
// sequences' splits in order (sequence b owns off[b] .. off[b+1]-1), so each
// sequence gets workgroups in proportion to its own tokens.  n == 0: one plan
// for every unit (grid.y = units).
struct SeqPlans {
  int n;
  int32_t off[kMaxSeqTab + 1];
  int16_t n_comp[kMaxSeqTab], n_pre[kMaxSeqTab], n_win[kMaxSeqTab];
  int32_t comp_len[kMaxSeqTab], pre_len[kMaxSeqTab], win_len[kMaxSeqTab];
  uint8_t win_rides[kMaxSeqTab];
};

__host__ __device__ inline SplitPlan seq_plan(const SeqPlans &sp, int b) {
  SplitPlan p;
  p.n_comp = sp.n_comp[b];
  p.comp_len = sp.comp_len[b];
  p.n_win = sp.n_win[b];
  p.win_len = sp.win_len[b];
  p.win_rides = sp.win_rides[b];
  p.n_pre = sp.n_pre[b];
  p.pre_len = sp.pre_len[b];
  return p;
}

static_assert(sizeof(Model) + sizeof(SeqTab) + sizeof(SeqPlans) + sizeof(SplitPlan) + 128 <= 4096,
              "decode kernel arguments must fit the 4 KiB argument segment");

// A float store performed at agent scope (coherent across the XCDs' L2s).
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Loads performed at agent scope: they read what other XCDs stored with
// store_agent, whatever this XCD's L2 holds.
__device__ __forceinline__ float load_agent(const float *p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned *>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ floatx4 load4_agent(const float *p) {
  return floatx4{load_agent(p), load_agent(p + 1), load_agent(p + 2), load_agent(p + 3)};
}

// feature held by lane row rho in slot j of K-block kb of the score product
__device__ __forceinline__ int score_feature(int kb, int j, int rho) {
  return 16 * (2 * kb + (j >> 2)) + 4 * rho + (j & 3);
}

// 16-byte direct load global -> LDS for this lane (LDS-DMA; the wave-uniform
// LDS base receives lane l's bytes at offset 16*l).  The builtin exists only
// for the device target, so the host pass sees an empty body.
__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
#endif
}

// 16-byte direct load buffer -> LDS: byte offset voff (per lane) + soff
// (wave-uniform) from the descriptor's base
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, void *lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, voff, soff, 0, 0);
#endif
}

// LDS transpose read (ds_read_b64_tr_b16) of a bf16 tile.  Within each group
// of 16 lanes, slot i of lane j receives element j % 4 of the 8 bytes that
// lane 4 i + j / 4 of the group addresses.  A lane addressing row
// 4 (lane / 16) + (lane % 16) / 4, columns 4 (lane % 4) .. + 3 of a
// row-major [token][coefficient] tile thus receives tokens 4 (lane / 16) ..
// + 3 of column lane % 16: the B operand of a 16x16x16 MFMA whose K index is
// the token.  (Layout checked with a probe kernel on gfx950.)
// N such reads at 32-byte steps from p (the B operands of N consecutive
// 16-column blocks), issued together and completed in the same asm block.
// (Through the builtin, the compiler cannot tell that these reads miss the
// LDS DMA writes still in flight into other ring slots and drains all of
// them first: a full memory latency per tile.)
template <int N, typename T>
__device__ __forceinline__ void lds_read_tr16(const T *p, uint2_ (&v)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "blocks per read group");
  const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void *)(
      reinterpret_cast<const void *>(p));
  if constexpr (N == 1) {
    asm volatile("ds_read_b64_tr_b16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a));
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:32\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&v"(v[0]), "=&v"(v[1]) : "v"(a));
  } else if constexpr (N == 4) {
    asm volatile("ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:32\n\t"
                 "ds_read_b64_tr_b16 %2, %4 offset:64\n\tds_read_b64_tr_b16 %3, %4 offset:96\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a));
  } else {
    asm volatile("ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:32\n\t"
                 "ds_read_b64_tr_b16 %2, %8 offset:64\n\tds_read_b64_tr_b16 %3, %8 offset:96\n\t"
                 "ds_read_b64_tr_b16 %4, %8 offset:128\n\tds_read_b64_tr_b16 %5, %8 offset:160\n\t"
                 "ds_read_b64_tr_b16 %6, %8 offset:192\n\tds_read_b64_tr_b16 %7, %8 offset:224\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7])
                 : "v"(a));
  }
}

// s_waitcnt vmcnt(N) with the other counters left free (gfx9 encoding)
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that publishes LDS writes only: waits for this wave's
// LDS operations, not for its vector-memory loads in flight (the memory
// clobber keeps the compiler from moving memory accesses across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Online softmax over one 16-token tile for the lane's head (l%16) and tokens
// 4*(l/16)..+3.  Rescales the value accumulators (lane layout: heads
// 4*(l/16)+i) when the running max of any head grows by more than kRescale.
// ---------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ void softmax_tile(floatx4 sc, int valid_mask, float &m, float &l,
                                             floatx4 (&acc)[NB], int rho, float (&p)[4]) {
  float s[4] = {sc[0], sc[1], sc[2], sc[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) if (!((valid_mask >> i) & 1)) s[i] = -INFINITY;
  float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  tmax = row_max(tmax);
  const bool need = tmax > m + kRescale;
  if (__any(need)) {
    const float mnew = need ? tmax : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // m = -inf -> 0
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __shfl(alpha, 4 * rho + i);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb][i] *= a;
    }
    m = mnew;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(s[i] - m);
    l += p[i];
  }
}

// ---------------------------------------------------------------------------
// Merge of the split records of one unit (sequence, KV head), run by the last
// split workgroup of the unit to finish:
// log-sum-exp weights w_s = 2^(m_s - max m), L = sum w_s l_s,
// acc_C = sum over compressed splits of w_s acc_s (r wide), acc_W likewise over
// window splits (128 wide); out = (B_V acc_C + acc_W) / L for each query head.
// Latency-bound: every global load (record accumulators, m/l pairs, the value
// basis) is issued before any of them is used.
// ---------------------------------------------------------------------------
// XOR swizzle of the 16-byte chunks of value-basis row f in LDS
template <int R> __device__ __forceinline__ int bv_swz(int f) { return f & ((R / 4 < 8 ? R / 4 : 8) - 1); }

// sum over aligned groups of gp lanes (gp a wave-uniform power of two <= 64):
// DPP swaps of lane pairs 1 and 2 apart, the half-row and row mirrors, then
// the 16- and 32-lane swaps; every lane ends with its group's sum
__device__ __forceinline__ float dpp_mov(float v, int ctrl_sel) {
  const int x = __float_as_int(v);
  int y;
  switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;    // quad_perm 1,0,3,2
    case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;    // quad_perm 2,3,0,1
    case 2: y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;   // row_half_mirror
    default: y = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break;  // row_mirror
  }
  return __int_as_float(y);
}
__device__ __forceinline__ float lane_group_sum(float v, int gp) {
  if (gp >= 2) v += dpp_mov(v, 0);
  if (gp >= 4) v += dpp_mov(v, 1);
  if (gp >= 8) v += dpp_mov(v, 2);
  if (gp >= 16) v += dpp_mov(v, 3);
  if (gp >= 32) v = xor16_sum(v);
  if (gp >= 64) v = xor32_sum(v);
  return v;
}
__device__ __forceinline__ float lane_group_max(float v, int gp) {
  if (gp >= 2) v = max2(v, dpp_mov(v, 0));
  if (gp >= 4) v = max2(v, dpp_mov(v, 1));
  if (gp >= 8) v = max2(v, dpp_mov(v, 2));
  if (gp >= 16) v = max2(v, dpp_mov(v, 3));
  if (gp >= 32) v = xor16_max(v);
  if (gp >= 64) v = xor32_max(v);
  return v;
}

template <int R, int NW> struct MergeLds {
  static constexpr int oBv = 0;                              // value basis [128][R/4] float4, swizzled
  static constexpr int oWt = oBv + kHeadDim * R * 4;         // per wave: weights of 64 records
  static constexpr int oAcc = oWt + NW * 64 * 4;             // per wave: acc_C [R], acc_W [128]
  static constexpr int bytes = oAcc + NW * (R + kHeadDim) * 4;
};

// record loads at agent scope (sc1), 16 bytes, through a buffer descriptor
// whose range covers the unit's records (reads past it return zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t agent_rsrc(const float *p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ floatx4 load4_rec(__amdgpu_buffer_rsrc_t r, int float_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, float_off * 4, 0, 16);
}
__device__ __forceinline__ float2 load2_agent(const float *p) {
  const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32))};
}

// Merge of one unit's split records (log-sum-exp combination; compressed
// records hold p^T C_V, which the value basis maps to head space), by a
// workgroup of NW waves.  Each wave merges whole query heads on its own
// (heads wave, wave + NW, ...): maxima and
// sums are lane reductions, the weights of a batch of records go through a
// per-wave LDS slot, so the only workgroup barrier is the one that publishes
// the value basis.  The wave's first head has its (m, l) pairs and first
// record batches in flight together with the value basis DMA.
template <int R, int NW>
__device__ void merge_unit(const Model &M, int layer, float *out, const SplitPlan &plan, int u,
                           uint8_t *lds) {
  using ML = MergeLds<R, NW>;
  constexpr int CC = R / 4, GC = 64 / CC;              // compressed: float4 columns, lanes per column
  constexpr int NBC = 8 * GC < 64 ? 8 * GC : 64;       // compressed records per batch (8 loads a lane)
  constexpr int NBW = 16;                              // window records per batch (32 columns x 2 lanes)
  const floatx4 *s_bv = reinterpret_cast<const floatx4 *>(lds + ML::oBv);
  const Dims &D = M.D;
  const int G = D.group, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // exact records (prefix and window splits) follow the compressed ones
  const int n_comp = plan.n_comp, n_win = plan.n_pre + plan.n_win, n_rec = n_comp + n_win;
  float *wt = reinterpret_cast<float *>(lds + ML::oWt) + wave * 64;
  float *sacc = reinterpret_cast<float *>(lds + ML::oAcc) + wave * (R + kHeadDim);
  const float *ml = M.sh.recml + (size_t)u * D.max_rec * G * 2;
  const float *acc = M.sh.rec + (size_t)u * D.max_rec * G * kRecStride;
  const __amdgpu_buffer_rsrc_t rr = agent_rsrc(acc, n_rec * G * kRecStride * 4);
  LayerPtrs P = layer_ptrs(M, layer);
  const uint8_t *Bv = reinterpret_cast<const uint8_t *>(P.basis[1] + (size_t)u * kHeadDim * R);

  // ---- value basis [128][R] -> LDS (R/2 KiB, 1 KiB per wave DMA).  16-byte
  // chunk c4 of row f lands at chunk c4 ^ bv_swz(f) of the row, so the output
  // phase (lane = row) reads without bank conflicts.
#pragma unroll
  for (int j = 0; j < (R / 2 + NW - 1) / NW; ++j) {
    const int c = wave + NW * j;
    if (c < R / 2) {
      const int pos = c * 64 + lane, f = pos / (R / 4), c4 = (pos % (R / 4)) ^ bv_swz<R>(f);
      dma16(Bv + (f * (R / 4) + c4) * 16, lds + ML::oBv + c * 1024);
    }
  }

  // lane roles: compressed column cc, record group cg (records s = cg mod GC);
  // window column wc, group wg (records s = wg mod 2)
  const int cc = lane / GC, cg = lane % GC, wc = lane >> 1, wg = lane & 1;
  float2 mlp0, mlp1;                    // (m, l) of records lane and 64 + lane
  floatx4 vc[8], vw[8];                 // first compressed / window batch
  auto fetch = [&](int h) {
    mlp0 = lane < n_rec ? load2_agent(ml + 2 * (lane * G + h)) : float2{-INFINITY, 0.f};
    mlp1 = 64 + lane < n_rec ? load2_agent(ml + 2 * ((64 + lane) * G + h)) : float2{-INFINITY, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = cg + GC * k;
      vc[k] = s < NBC && s < n_comp ? load4_rec(rr, (s * G + h) * kRecStride + 4 * cc) : zero4();
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = wg + 2 * k;
      vw[k] = s < NBW && s < n_win ? load4_rec(rr, ((n_comp + s) * G + h) * kRecStride + 4 * wc) : zero4();
    }
  };
  if (wave < G) fetch(wave);
  wait_vmcnt<0>();
  __syncthreads();                      // the value basis is in LDS

  const int b = u / D.kv_heads, hk = u % D.kv_heads;
  for (int h = wave; h < G; h += NW) {
    if (h != wave) fetch(h);
    // max and sum over all records: registers for the first 128, reads past
    float mx = max2(mlp0.x, mlp1.x);
    for (int s = 128 + lane; s < n_rec; s += 64) mx = max2(mx, load_agent(ml + 2 * (s * G + h)));
    mx = lane_group_max(mx, 64);
    float l = __builtin_amdgcn_exp2f(mlp0.x - mx) * mlp0.y + __builtin_amdgcn_exp2f(mlp1.x - mx) * mlp1.y;
    for (int s = 128 + lane; s < n_rec; s += 64) {
      const float2 p = load2_agent(ml + 2 * (s * G + h));
      l += __builtin_amdgcn_exp2f(p.x - mx) * p.y;
    }
    l = lane_group_sum(l, 64);
    // weights of records b0 .. b0 + 63 -> wt (lane i: record b0 + i)
    auto weights = [&](int b0) {
      const int s = b0 + lane;
      const float m0 = __shfl(mlp0.x, s & 63), m1 = __shfl(mlp1.x, s & 63);
      float m = s < 64 ? m0 : m1;
      if (s >= 128 && s < n_rec) m = load_agent(ml + 2 * (s * G + h));
      wt[lane] = s < n_rec ? __builtin_amdgcn_exp2f(m - mx) : 0.f;
    };
    // compressed records: acc_C = sum w_s acc_s
    {
      floatx4 a = zero4();
      for (int b0 = 0; b0 < n_comp; b0 += NBC) {
        weights(b0);
        if (b0 > 0) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int s = b0 + cg + GC * k;
            vc[k] = cg + GC * k < NBC && s < n_comp ? load4_rec(rr, (s * G + h) * kRecStride + 4 * cc) : zero4();
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) a += wt[(cg + GC * k) & 63] * vc[k];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = lane_group_sum(a[j], GC);
      if (cg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[4 * cc + j] = a[j];
      }
    }
    // window records: acc_W = sum w_s acc_s
    {
      floatx4 a = zero4();
      for (int b0 = n_comp; b0 < n_rec; b0 += NBW) {
        weights(b0);
        if (b0 > n_comp) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int s = b0 + wg + 2 * k;
            vw[k] = s < n_rec ? load4_rec(rr, (s * G + h) * kRecStride + 4 * wc) : zero4();
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) a += wt[wg + 2 * k] * vw[k];
      }
      a[0] = lane_group_sum(a[0], 2); a[1] = lane_group_sum(a[1], 2);
      a[2] = lane_group_sum(a[2], 2); a[3] = lane_group_sum(a[3], 2);
      if (wg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[R + 4 * wc + j] = a[j];
      }
    }
    // out = (B_V acc_C + acc_W) / L; lane -> features lane, lane + 64
    const float inv_l = 1.f / l;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = lane + 64 * i;
      float a = sacc[R + f];
      if (n_comp > 0) {
#pragma unroll
        for (int c4 = 0; c4 < R / 4; ++c4) {
          const floatx4 bv = s_bv[f * (R / 4) + (c4 ^ bv_swz<R>(f))];
          a += bv[0] * sacc[4 * c4] + bv[1] * sacc[4 * c4 + 1] + bv[2] * sacc[4 * c4 + 2] +
               bv[3] * sacc[4 * c4 + 3];
        }
      }
      out[((size_t)b * D.q_heads + hk * G + h) * kHeadDim + f] = a * inv_l;
    }
  }
}

// ---------------------------------------------------------------------------
// Tunables per (rank, storage, waves per workgroup): occupancy, the LDS
// layout and the per-wave ring.
// ---------------------------------------------------------------------------
// RK, RV: ranks of the key and value factors.
template <int RK, int RV, typename T, int NW> struct Cfg {
  static constexpr int R = RK;
  static constexpr bool BF = std::is_same<T, bf16_t>::value;
  static constexpr int kElem = BF ? 2 : 4;
  static constexpr int kMatK = 16 * RK * kElem;              // one 16-token tile of C_K
  static constexpr int kMatV = 16 * RV * kElem;              // ... and of C_V
  static constexpr int kSlot = kMatK + kMatV;                // ring slot [C_K tile | C_V tile]
  static constexpr int kDmaK = kMatK >= 1024 ? kMatK / 1024 : 1;   // dwordx4 DMAs per matrix
  static constexpr int kDmaV = kMatV >= 1024 ? kMatV / 1024 : 1;
  // Eight-wave workgroups (bf16, r <= 64; one per CU, two waves per SIMD)
  // share their prologue: the key-basis fragments and the RoPE rotations of
  // offsets 0..15 reach LDS once per workgroup by DMA, and each wave's base
  // angle takes one coalesced load per lane (lane = frequency).  Four-wave
  // workgroups load both per wave.
  static_assert(NW == 4 || (NW == 8 && BF && RK <= 64 && RV <= 64), "wave count");
  static constexpr bool kShared = NW == 8;
  // key-basis fragment chunks (16 bytes a lane) per M-block held in
  // registers: bf16 storage, one fp16 operand per 32 coefficients (16 at
  // r = 16); fp32 storage, four fp32 values per chunk
  static constexpr int kFch = BF ? (R >= 32 ? R / 32 : 1) : R / 16;
  // shared prologue data sits in static LDS arrays (fragments, step rows,
  // per-wave base angles): reads of them are then known not to alias the
  // ring DMAs in flight, so the compiler adds no wait for those.  Dynamic
  // LDS: the per-wave rings
  static constexpr int kFragBytes = kShared ? 8 * kFch * 1024 : 16;
  static constexpr int kRingOff = 0;
  // per wave; wide tiles (r = 128, or r = 64 in float) get a deeper ring.
  // Eight-wave workgroups keep four r <= 32 tiles per wave (eight waves per
  // CU hold enough bytes in flight, and a shorter ring is issued sooner)
  static constexpr int kRingBytes = kShared ? (RK == 64 || RV == 64 ? 12288 : 8192)
                                    : (BF && R == 64) ? 12288 : (kSlot >= 8192 ? 32768 : 16384);
  static constexpr int kDepth = kRingBytes / kSlot > 16 ? 16 : kRingBytes / kSlot;
  static_assert(kDepth >= 2, "ring depth");
  static constexpr int kWaves = NW;
  static constexpr int kThr = 64 * NW;
  static constexpr int kOcc = (BF && RK <= 64 && RV <= 64 && NW == 4) ? 2 : 1;
  // compressed tiles in pairs (two register sets for the angle state); wider
  // ranks lack the registers for it
  static constexpr bool kPair = RK <= 32 && RV <= 32;
  static constexpr int kAccBytes = kWaves * 16 * kHeadDim * 4;    // per-wave results, after the loop
  static constexpr int kLoopBytes = (kRingOff + NW * kRingBytes > kAccBytes)
                                        ? kRingOff + NW * kRingBytes : kAccBytes;
  static constexpr int kMrgBytes = MergeLds<RV, kWaves>::bytes;
  static constexpr int kDynBytes = kLoopBytes > kMrgBytes ? kLoopBytes : kMrgBytes;
};

// ---------------------------------------------------------------------------
// The MFMA decode kernel.  grid (splits, units), 64 * kWaves threads.
// ---------------------------------------------------------------------------
// PK (bf16 storage, 4 query heads per KV head): the score product's B
// operand carries the fp16 high parts of the 4 query heads in columns 0..3
// and their low parts in columns 4..7, one product per K-block instead of
// two; lanes 0..3 of each row then add lanes 4..7
template <int RK, int RV, typename T, int NW, bool PK>
__global__ __launch_bounds__((Cfg<RK, RV, T, NW>::kThr), (Cfg<RK, RV, T, NW>::kOcc)) void decode_mfma_kernel(
    Model M, int layer, const float *__restrict__ q, int64_t q_pos_arg, float *out, int64_t length_arg,
    int64_t n_c_arg, SplitPlan plan_arg, int fused, FusedAppend app, SeqTab tab, SeqPlans sp) {
  using C = Cfg<RK, RV, T, NW>;
  constexpr int R = RK;                                  // the key path below uses R
  constexpr bool BF = C::BF;
  constexpr int NBV = RV / 16;                           // value N-blocks (compressed)
  constexpr int DEPTH = C::kDepth;
  constexpr int LPT = C::kDmaK + C::kDmaV;               // DMA loads per tile
  constexpr int QK = 16 / NW;
  extern __shared__ __align__(16) uint8_t s_dyn[];       // per-wave rings, then results
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ float2 s_step[64];          // cos, sin of 16 * theta_i (tile advance)
  __shared__ float s_q[16][kHeadDim];    // rotated, scaled query rows of the group
  __shared__ __align__(16) uint8_t s_frag[C::kFragBytes];          // key-basis fragments (shared prologue)
  // cos, sin of o * theta_f for offsets o < 16, as [f][o] with row stride 17
  // (the lanes of one read take 16 offsets and 4 frequencies: no bank conflict)
  __shared__ float2 s_st16[C::kShared ? 64 * 17 : 1];
  __shared__ float2 s_base[C::kShared ? NW * 64 : 1];              // per wave: cos, sin of w_begin * theta_f
  __shared__ float2 s_wbase[C::kShared ? NW * 64 : 1];             // ... of the riding window part's range
  __shared__ int s_prog[NW];                                       // per wave: tile index in the loop
  float (*s_acc)[16][kHeadDim] = reinterpret_cast<float (*)[16][kHeadDim]>(s_dyn);

  const Dims &D = M.D;
  const int G = D.group;
  // bf16: the wave index in a scalar register (ring and slot addresses, the
  // LDS-DMA base, become scalar arithmetic); the fp32 kernels keep the plain
  // form (see the note at the fp32 rotation below)
  const int wave = BF ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n16 = lane & 15, rho = lane >> 4;
  // ragged: blockIdx.x = (sequence, split) flattened, blockIdx.y = KV head
  int split_i = blockIdx.x, b_i = (int)blockIdx.y / D.kv_heads;
  if (sp.n) {
    b_i = 0;
    while (b_i + 1 < sp.n && sp.off[b_i + 1] <= split_i) ++b_i;
    split_i -= sp.off[b_i];
  }
  const int split = split_i, b = b_i;
  const int hk = sp.n ? (int)blockIdx.y : (int)blockIdx.y % D.kv_heads;
  const int u = b * D.kv_heads + hk;
  const SplitPlan plan = sp.n ? seq_plan(sp, b) : plan_arg;
  // a ragged batch gives each sequence its own length, compressed end and
  // query position, and its own plan; a split with no tokens (none in a
  // uniform or per-sequence plan, kept safe all the same) writes a neutral
  // record
  const int64_t length = tab.n ? (int64_t)tab.len[b] : length_arg;
  const int64_t n_c = tab.n ? (int64_t)tab.nc[b] : n_c_arg;
  const int64_t q_pos = tab.n ? (int64_t)tab.aux[b] : q_pos_arg;
  // a compressed workgroup (split < n_comp) may also take window split
  // `split` after its compressed range (plan.win_rides): two parts, each
  // with its own record
  const bool cwg = split < plan.n_comp;
  const int xs = split - plan.n_comp;                    // exact split index
  const int nparts = (cwg && plan.win_rides) ? 2 : 1;

  LayerPtrs P = layer_ptrs(M, layer);

  const SplitK sk = split_consts();

  // ---- query rows rotated at q_pos and scaled by scale*log2(e), via LDS:
  // thread (frequency qi, heads qh0 + NW k) loads (query_issue), then rotates
  // and stores them, after which the rows are split hi/lo (fp16 with bf16
  // storage, bf16 with fp32 storage) into the B-operand layout of the score
  // product (query_finish, one barrier)
  const int qi = threadIdx.x & 63, qh0 = threadIdx.x >> 6;
  float qx0[QK], qx1[QK];
  float2 qA, qB, qstep;
  auto query_issue = [&]() {
#pragma unroll
    for (int k = 0; k < QK; ++k) {
      const int h = qh0 + NW * k < G ? qh0 + NW * k : G - 1;    // rows past the group: not used
      const float *qr = q + ((size_t)b * D.q_heads + hk * G + h) * kHeadDim;
      qx0[k] = qr[qi];
      qx1[k] = qr[qi + 64];
    }
    rope_load(M.sh, q_pos, qi, qA, qB);
    qstep = reinterpret_cast<const float2 *>(M.sh.rope_step)[16 * 64 + qi];
  };
  uint4_ qhi[4], qlo[4];
  // lds_only: the barrier publishes LDS writes only (no wait for the ring
  // tiles in flight, which a full workgroup fence would drain)
  auto query_finish = [&](bool lds_only) {
    float c, s;
    rope_combine(qA, qB, c, s);
#pragma unroll
    for (int k = 0; k < QK; ++k) {
      const int h = qh0 + NW * k;
      const float x0 = h < G ? qx0[k] : 0.f, x1 = h < G ? qx1[k] : 0.f;
      s_q[h][qi] = fmaf(x0, c, -x1 * s) * D.scale_log2;
      s_q[h][qi + 64] = fmaf(x1, c, x0 * s) * D.scale_log2;
    }
    if (threadIdx.x < 64) s_step[threadIdx.x] = qstep;
    if (lds_only) lds_barrier();
    else __syncthreads();
    // packed (PK): lanes of columns 4..7 take the low parts of heads 0..3;
    // columns 8..15 read rows past the group, which are zero
    const int qrow = PK ? (n16 < 4 ? n16 : n16 - 4) : n16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      unsigned h[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = s_q[qrow][score_feature(kb, 2 * j, rho)];
        const float bq = s_q[qrow][score_feature(kb, 2 * j + 1, rho)];
        if constexpr (BF) split2_f16(a, bq, h[j], lo[j]);
        else split2(a, bq, h[j], lo[j]);
        if constexpr (PK) h[j] = n16 < 4 ? h[j] : lo[j];
      }
      qhi[kb] = uint4_{h[0], h[1], h[2], h[3]};
      qlo[kb] = uint4_{lo[0], lo[1], lo[2], lo[3]};
    }
  };


  bool q_ready = false;                                 // query operands built (first part)
  // this wave's tile range within [r_begin, r_end): an even split, the first
  // ntiles % NW waves take one tile more (waves w and w + NW/2 share a SIMD,
  // so every SIMD gets the same count within one)
  auto wave_tiles = [&](int64_t r_begin, int64_t r_end, int &tile_lo, int &tile_hi) {
    const int ntiles = (int)((r_end - r_begin + 15) / 16);
    const int tb = ntiles / NW, tx = ntiles % NW;
    tile_lo = wave * tb + (wave < tx ? wave : tx);
    tile_hi = tile_lo + tb + (wave < tx ? 1 : 0);
  };
  // range of the window split that rides on compressed split `split`
  auto ride_range = [&](int64_t &r_begin, int64_t &r_end) {
    r_begin = n_c + (int64_t)split * plan.win_len;
    r_end = r_begin + plan.win_len < length ? r_begin + plan.win_len : length;
    if (r_end < r_begin) r_end = r_begin;
  };
  auto run_part = [&](const int part) {
  // ---- RoPE angle state of the lane's token for its 16 frequencies; the
  // table loads (anchor_issue) and the products (anchor_finish) are apart so
  // the prologue issues every load before its first wait
  float cs_c[16], cs_s[16];          // separate arrays: no 64-bit register pairs
  float2 an_A[16], an_B[16];
  auto anchor_issue = [&](int64_t t) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rope_load(M.sh, t, 16 * mb + 4 * rho + i, an_A[mb * 4 + i], an_B[mb * 4 + i]);
  };
  auto anchor_finish = [&]() {
#pragma unroll
    for (int j = 0; j < 16; ++j) rope_combine(an_A[j], an_B[j], cs_c[j], cs_s[j]);
  };
  auto anchor = [&](int64_t t) {
    anchor_issue(t);
    anchor_finish();
  };

  // rotate the key tile by the angle state (then advance it 16 positions),
  // then the score product
  auto rope_scores = [&](floatx4 (&ka)[8]) -> floatx4 {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = cs_c[mb * 4 + i], s = cs_s[mb * 4 + i];
        const float x0 = ka[mb][i], x1 = ka[mb + 4][i];
        ka[mb][i] = fmaf(x0, c, -x1 * s);
        ka[mb + 4][i] = fmaf(x1, c, x0 * s);
        if constexpr (!BF) {
          // fp32 storage keeps the advance inline: with the bf16 forms below
          // (scalar wave index, buffer-descriptor DMA, batched step reads) the
          // fp32 r = 64 kernel gave wrong results for the last query head of
          // each group on joint-basis data, with no cause found in the source
          const float2 st = s_step[16 * mb + 4 * rho + i];
          cs_c[mb * 4 + i] = fmaf(c, st.x, -s * st.y);
          cs_s[mb * 4 + i] = fmaf(s, st.x, c * st.y);
        }
      }
    // advance the angle state by 16 positions, after the score products are
    // issued (they run while the step rotations arrive from LDS)
    auto advance = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      // the lane's 16 step rotations in one batch of LDS reads (one wait)
      floatx4 w[8];
      {
        const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void *)(
            reinterpret_cast<const void *>(s_step + 4 * rho));
        asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\t"
                     "ds_read_b128 %2, %8 offset:128\n\tds_read_b128 %3, %8 offset:144\n\t"
                     "ds_read_b128 %4, %8 offset:256\n\tds_read_b128 %5, %8 offset:272\n\t"
                     "ds_read_b128 %6, %8 offset:384\n\tds_read_b128 %7, %8 offset:400\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]),
                       "=&v"(w[6]), "=&v"(w[7])
                     : "v"(a));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float c = cs_c[mb * 4 + i], s = cs_s[mb * 4 + i];
          const floatx4 &wv = w[2 * mb + (i >> 1)];
          const float2 st = (i & 1) ? float2{wv[2], wv[3]} : float2{wv[0], wv[1]};
          float cc = c, ss = s, t0, t1;
          // written in place, so the loop-carried state keeps its registers
          // (the compiler's own form copied all 32 of them every tile)
          asm("v_mul_f32 %2, %1, %5\n\t"
              "v_mul_f32 %3, %0, %5\n\t"
              "v_fma_f32 %0, %0, %4, -%2\n\t"
              "v_fma_f32 %1, %1, %4, %3"
              : "+v"(cc), "+v"(ss), "=&v"(t0), "=&v"(t1) : "v"(st.x), "v"(st.y));
          cs_c[mb * 4 + i] = cc;
          cs_s[mb * 4 + i] = ss;
        }
    };
    floatx4 sc[2] = {zero4(), zero4()};          // two chains of dependent MFMAs
    if constexpr (BF) {
      // bf16 storage: the rotated key enters once, rounded to fp16 (2^-12
      // relative; the query as fp16 hi + lo), two products per K-block
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint4_ kh = {pack_f16(ka[2 * kb][0], ka[2 * kb][1]), pack_f16(ka[2 * kb][2], ka[2 * kb][3]),
                           pack_f16(ka[2 * kb + 1][0], ka[2 * kb + 1][1]),
                           pack_f16(ka[2 * kb + 1][2], ka[2 * kb + 1][3])};
        floatx4 &a = sc[kb & 1];
        if constexpr (!PK) a = mfma32h(kh, qlo[kb], a);
        a = mfma32h(kh, qhi[kb], a);
      }
      advance();
      floatx4 st = sc[0] + sc[1];
      if constexpr (PK) {
        // head h (lanes h of each row) adds its low-part column h + 4
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st[e] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(st[e]), 0x104, 0xF, 0xF, false));
      }
      return st;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      unsigned h[4], lo[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        split2(ka[2 * kb][2 * j], ka[2 * kb][2 * j + 1], h[j], lo[j], sk);
        split2(ka[2 * kb + 1][2 * j], ka[2 * kb + 1][2 * j + 1], h[2 + j], lo[2 + j], sk);
      }
      const uint4_ kh = {h[0], h[1], h[2], h[3]}, kl = {lo[0], lo[1], lo[2], lo[3]};
      floatx4 &a = sc[kb & 1];
      a = mfma32(kh, qhi[kb], a);
      a = mfma32(kh, qlo[kb], a);
      a = mfma32(kl, qhi[kb], a);
    }
    return sc[0] + sc[1];
  };
  const bool comp = cwg && part == 0;                    // compressed range
  const bool pre = !cwg && xs < plan.n_pre;              // a protected-prefix split
  // record of this part: compressed records first, then prefix, then window
  const int rec_idx = comp ? split : (cwg ? plan.n_comp + plan.n_pre + split : split);
  int64_t r_begin, r_end;
  if (comp) {
    r_begin = D.prefix + (int64_t)split * plan.comp_len;
    r_end = r_begin + plan.comp_len < n_c ? r_begin + plan.comp_len : n_c;
  } else if (pre) {
    const int64_t pend = length < D.prefix ? length : D.prefix;
    r_begin = (int64_t)xs * plan.pre_len;
    r_end = r_begin + plan.pre_len < pend ? r_begin + plan.pre_len : pend;
  } else if (cwg) {
    ride_range(r_begin, r_end);
  } else {
    r_begin = n_c + (int64_t)(xs - plan.n_pre) * plan.win_len;
    r_end = r_begin + plan.win_len < length ? r_begin + plan.win_len : length;
  }
  if (r_end < r_begin) r_end = r_begin;
  int tile_lo, tile_hi;
  wave_tiles(r_begin, r_end, tile_lo, tile_hi);
  const int64_t w_begin = r_begin + 16 * (int64_t)tile_lo;
  const int nt = __builtin_amdgcn_readfirstlane(tile_hi - tile_lo);   // wave-uniform

  float m = -INFINITY, l = 0.f;
  const int64_t w_end = r_end;

  if (comp) {
    // ================= compressed tokens =================
    floatx4 vacc[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) vacc[nb] = zero4();
    // per-wave LDS ring of DEPTH slots, each [C_K tile | C_V tile]
    uint8_t *ring = s_dyn + C::kRingOff + wave * C::kRingBytes;
    const size_t cu = (size_t)coef_unit(D, u);     // a joint basis shares one stream per sequence
    const uint8_t *gk = P.coef[0] + (cu * D.max_tokens * RK + (size_t)w_begin * RK) * C::kElem;
    const uint8_t *gv = P.coef[1] + (cu * D.max_tokens * RV + (size_t)w_begin * RV) * C::kElem;
    // one tile: kDmaK / kDmaV dwordx4 DMAs per matrix; lane l moves 16 bytes
    // of chunk d*64 + l of the tile (lanes past the tile size idle)
    // tile `src` into ring slot `it` % DEPTH
    // descriptors over the wave's range: per-lane offsets are constants, the
    // tile offset is a scalar
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(gk), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(gv), 0, 0x7fffffff, 0x00020000);
    auto issue_from = [&](int it, int src) {
      uint8_t *slot = ring + (it % DEPTH) * C::kSlot;
#pragma unroll
      for (int d = 0; d < C::kDmaK; ++d) {
        const int off = (d * 64 + lane) * 16;
        if (off >= C::kMatK) continue;
        if constexpr (BF) dma16_buf(rk, off, src * C::kMatK, slot + d * 1024);
        else dma16(gk + (size_t)src * C::kMatK + off, slot + d * 1024);
      }
#pragma unroll
      for (int d = 0; d < C::kDmaV; ++d) {
        const int off = (d * 64 + lane) * 16;
        if (off >= C::kMatV) continue;
        if constexpr (BF) dma16_buf(rv, off, src * C::kMatV, slot + C::kMatK + d * 1024);
        else dma16(gv + (size_t)src * C::kMatV + off, slot + C::kMatK + d * 1024);
      }
    };
    auto issue = [&](int it) { issue_from(it, it); };
    // prologue: the LDS copies (basis fragments, step rows), the query, the
    // register-resident basis fragments and the first angle state are loaded
    // and consumed before the first DEPTH-1 ring tiles are issued.  (The
    // compiler waits for every outstanding load, LDS DMAs included, before
    // the first use of a value loaded ahead of an LDS DMA, so any use after
    // the ring issue would wait for the whole ring.)  Every wave's LDS copies
    // are older than its query loads, so they have completed before the
    // barrier in query_finish, after which all waves read them.
    const uint8_t *FB = P.frag + (size_t)u * 4 * kHeadDim * R;
    constexpr int FCH = C::kFch;                         // register-resident chunks per M-block
    // HBM chunk of register chunk ch of M-block mb (bf16 storage: the fp16
    // operands sit in the even chunks)
    auto gchunk = [&](int mb, int ch) { return mb * (R / 16) + (BF ? (R >= 32 ? 2 * ch : 0) : ch); };
    if constexpr (C::kShared) {
      // every used fragment chunk and step rows 0..15
      constexpr int NCH = 8 * FCH;
      static_assert(NCH % NW == 0, "fragment chunks per wave");
#pragma unroll
      for (int j = 0; j < NCH / NW; ++j) {
        const int c = wave + NW * j;
        dma16(FB + ((size_t)gchunk(c / FCH, c % FCH) * 64 + lane) * 16, s_frag + c * 1024);
      }
    }
    query_issue();
    uint4_ F[8][FCH];
    float2 bA, bB, stv[2], wA, wB;
    if constexpr (C::kShared) {
      rope_load(M.sh, w_begin, lane, bA, bB);       // base angle of the range, frequency = lane
      if (nparts == 2) {
        // and of this wave's tiles of the riding window split, so that part
        // starts without a memory round trip
        int64_t wb, we;
        int wlo, whi;
        ride_range(wb, we);
        wave_tiles(wb, we, wlo, whi);
        rope_load(M.sh, wb + 16 * (int64_t)wlo, lane, wA, wB);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k)                   // step rows 0..15, entry threadIdx.x + 512 k
        stv[k] = reinterpret_cast<const float2 *>(M.sh.rope_step)[threadIdx.x + 512 * k];
    } else {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int ch = 0; ch < FCH; ++ch)
          F[mb][ch] = *reinterpret_cast<const uint4_ *>(FB + ((size_t)gchunk(mb, ch) * 64 + lane) * 16);
      anchor_issue(w_begin + n16);
    }
    wait_vmcnt<0>();
    if constexpr (C::kShared) {
      float c, sn;
      rope_combine(bA, bB, c, sn);
      s_base[wave * 64 + lane] = float2{c, sn};
      if (nparts == 2) {
        rope_combine(wA, wB, c, sn);
        s_wbase[wave * 64 + lane] = float2{c, sn};
      }
      if (lane == 0) s_prog[wave] = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = threadIdx.x + 512 * k;
        s_st16[(e & 63) * 17 + (e >> 6)] = stv[k];
      }
    } else {
      anchor_finish();
    }
    __builtin_amdgcn_sched_barrier(0);
    // the first ring tile only: each DMA passes the CU's address path at
    // ~1 KiB per 16 clocks, so a deep prologue issue would hold every wave
    // (and the set-up after it) for microseconds; tiles 1 .. DEPTH-2 follow
    // the barrier.  Always all of them, so the waits in the loop have fixed
    // counts (a range shorter than that re-reads its last tile into slots it
    // never uses).
    if (nt > 0) issue_from(0, 0);
    query_finish(true);
    if (nt > 0) {
#pragma unroll
      for (int j = 1; j < DEPTH - 1; ++j) issue_from(j, j < nt ? j : nt - 1);
    }
    if constexpr (C::kShared) {
      if (nt > 0) {
        // register fragments from LDS; the lane's angle state = base angle of
        // its frequency x rotation by its token offset n16
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int ch = 0; ch < FCH; ++ch)
            F[mb][ch] = *reinterpret_cast<const uint4_ *>(s_frag + ((mb * FCH + ch) * 64 + lane) * 16);
        const float2 *base = s_base + wave * 64;
        const float2 *st16 = s_st16 + n16;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = 16 * mb + 4 * rho + i;
            rope_combine(base[f], st16[17 * f], cs_c[mb * 4 + i], cs_s[mb * 4 + i]);
          }
      }
    }
    // one 16-token tile: wait for its ring slot, rebuild the keys, scores,
    // online softmax, values
    // Two waves share each SIMD in eight-wave workgroups (waves w and w ^ 4),
    // and issue goes to the older one first; each wave posts its tile index
    // in LDS and lowers its priority while it is ahead of the other, so both
    // finish together instead of one running alone at the end.  (Reads of
    // the other's index race with its writes; a stale value only delays the
    // switch by a tile.)
    auto comp_tile = [&](int it) {
      if constexpr (NW == 8) {
        const int other = __builtin_amdgcn_readfirstlane(s_prog[wave ^ 4]);
        if (lane == 0) s_prog[wave] = it;
        if (it > other) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(2);
      }
      if (it + DEPTH - 1 < nt) {
        issue(it + DEPTH - 1);
        wait_vmcnt<(DEPTH - 1) * LPT>();
      } else {
        wait_vmcnt<0>();
      }
      const uint8_t *slot = ring + (it % DEPTH) * C::kSlot;
      const T *tk = reinterpret_cast<const T *>(slot);
      const T *tv = reinterpret_cast<const T *>(slot + C::kMatK);
      // keys: rebuild from the basis fragments and this lane's coefficients
      floatx4 ka[8];
      if constexpr (BF) {
        // one fp16 product per 32 coefficients: the stored bf16 coefficients
        // convert exactly, the basis enters rounded to fp16
        const T *row = tk + n16 * R + rho * (R / 4);
        if constexpr (R == 16) {
          const uint2_ bop = *reinterpret_cast<const uint2_ *>(row);
          const uint2_ bh = {bf16x2_to_f16x2(bop.x), bf16x2_to_f16x2(bop.y)};
#pragma unroll
          for (int mb = 0; mb < 8; ++mb) ka[mb] = mfma16h(uint2_{F[mb][0].x, F[mb][0].y}, bh, zero4());
        } else {
          uint4_ bop[R / 32];
#pragma unroll
          for (int kb = 0; kb < R / 32; ++kb) {
            const uint4_ x = reinterpret_cast<const uint4_ *>(row)[kb];
            bop[kb] = uint4_{bf16x2_to_f16x2(x.x), bf16x2_to_f16x2(x.y), bf16x2_to_f16x2(x.z),
                             bf16x2_to_f16x2(x.w)};
          }
#pragma unroll
          for (int mb = 0; mb < 8; ++mb) {
            floatx4 a = zero4();
#pragma unroll
            for (int kb = 0; kb < R / 32; ++kb) a = mfma32h(F[mb][kb], bop[kb], a);
            ka[mb] = a;
          }
        }
      } else {
        const float *row = reinterpret_cast<const float *>(tk) + n16 * R + rho * (R / 4);
        float cf[R / 4];
#pragma unroll
        for (int c = 0; c < R / 4; ++c) cf[c] = row[c];
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          floatx4 a = zero4();
#pragma unroll
          for (int c = 0; c < R / 4; ++c) a = mfma4(__uint_as_float(F[mb][c / 4][c % 4]), cf[c], a);
          ka[mb] = a;
        }
      }
      const floatx4 sc = rope_scores(ka);
      float p[4];
      softmax_tile<NBV>(sc, 0xf, m, l, vacc, rho, p);
      // values: the B operand (C_V tokens 4*rho..+3 of coefficient 16*nb +
      // n16) straight from the row-major tile by the LDS transpose read
      if constexpr (BF) {
        unsigned h0, l0, h1, l1;
        split2(p[0], p[1], h0, l0, sk);
        split2(p[2], p[3], h1, l1, sk);
        uint2_ v[NBV];
        lds_read_tr16<NBV>(tv + (4 * rho + (n16 >> 2)) * RV + 4 * (n16 & 3), v);
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) {
          vacc[nb] = mfma16(uint2_{h0, h1}, v[nb], vacc[nb]);
          vacc[nb] = mfma16(uint2_{l0, l1}, v[nb], vacc[nb]);
        }
      } else {
        const float *tf = reinterpret_cast<const float *>(tv);
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vacc[nb] = mfma4(p[i], tf[(4 * rho + i) * RV + 16 * nb + n16], vacc[nb]);
      }
    };
    // chunks of 32 tiles: the angle state is re-anchored from the table at
    // each chunk start (bounding the recurrence) outside the inner loop.
    // Paired tiles let the angle state alternate between two register sets
    // instead of being copied back after every tile.
    for (int c0 = 0; c0 < nt; c0 += 32) {
      if (c0 > 0) anchor(w_begin + 16 * (int64_t)c0 + n16);
      const int c1 = nt < c0 + 32 ? nt : c0 + 32;
      int it = c0;
      if constexpr (C::kPair)
        for (; it + 1 < c1; it += 2) {
          comp_tile(it);
          comp_tile(it + 1);
        }
      for (; it < c1; ++it) comp_tile(it);
    }
    if constexpr (NW == 8) __builtin_amdgcn_s_setprio(0);
    // per-wave results: acc[head 4*rho+i][coef 16*nb + n16] (over the rings)
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_acc[wave][4 * rho + i][16 * nb + n16] = vacc[nb][i];
  } else {
    // ================= exact window tokens =================
    if (app.k != nullptr && !pre && r_end == length && r_begin < length && threadIdx.x < 2 * kHeadDim) {
      // fused append: this window split ends at the newest position; write
      // its ring rows (rounded to the storage type) before the barrier below,
      // after which this workgroup reads them
      const int e = threadIdx.x & (kHeadDim - 1), x = threadIdx.x >> 7;   // K for x = 0, V for x = 1
      const size_t src = ((size_t)b * D.kv_heads + hk) * kHeadDim + e;
      const float val = app.in_dtype == 1 ? bf16_to_f32(reinterpret_cast<const bf16_t *>(x ? app.v : app.k)[src].bits)
                                          : reinterpret_cast<const float *>(x ? app.v : app.k)[src];
      if (!isfinite(val)) set_flag(M.sh, 4);
      const int slot = (int)((length - 1) % D.slots);
      T *ring = reinterpret_cast<T *>(x ? P.ringv : P.ringk) + (size_t)u * D.slots * kHeadDim;
      Store<T>::store(ring, x ? (size_t)e * D.slots + slot : (size_t)slot * kHeadDim + e, val);
    }
    floatx4 wacc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) wacc[nb] = zero4();
    // exact rows: the protected prefix (row = position) or the ring (row =
    // position % slots); V transposed in both, row stride `rows`
    const int rows = pre ? D.prefix : D.slots;
    const T *EK = reinterpret_cast<const T *>(pre ? P.prek : P.ringk) + (size_t)u * rows * kHeadDim;
    const T *EV = reinterpret_cast<const T *>(pre ? P.prev : P.ringv) + (size_t)u * rows * kHeadDim;
    // raw K rows and V columns of a tile, both issued together (one memory
    // latency per tile instead of a second one for V)
    using Raw = typename std::conditional<BF, uint2_, floatx4>::type;
    auto load_raw = [&](int it, Raw (&k)[8], Raw (&v)[8]) {
      const int64_t t0 = w_begin + 16 * (int64_t)it;
      const int slot = (int)((t0 + n16) % rows);
      const int slot0 = (int)(t0 % rows);             // tiles never wrap (16 | slots, 64 | P)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
        k[mb] = *reinterpret_cast<const Raw *>(EK + (size_t)slot * kHeadDim + 16 * mb + 4 * rho);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        v[nb] = *reinterpret_cast<const Raw *>(EV + (size_t)(16 * nb + n16) * rows + slot0 + 4 * rho);
    };
    // the riding part of an eight-wave workgroup takes its base angles from
    // the prologue (LDS); other exact parts load them here
    const bool lds_angles = C::kShared && part == 1;
    if (!q_ready) query_issue();
    if (nt > 0 && !lds_angles) anchor_issue(w_begin + n16);
    __builtin_amdgcn_sched_barrier(0);
    if (nt > 0 && !lds_angles) anchor_finish();
    if (!q_ready) query_finish(false);
    else __syncthreads();               // the fused append's ring rows are visible
    if (nt > 0 && lds_angles) {
      const float2 *base = s_wbase + wave * 64;
      const float2 *st16 = s_st16 + n16;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = 16 * mb + 4 * rho + i;
          rope_combine(base[f], st16[17 * f], cs_c[mb * 4 + i], cs_s[mb * 4 + i]);
        }
    }
    if (nt > 0) {
      for (int it = 0; it < nt; ++it) {
        const int64_t t0 = w_begin + 16 * (int64_t)it;
        Raw kc[8], vc[8];
        load_raw(it, kc, vc);
        floatx4 ka[8];
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          if constexpr (BF) {
            const uint2_ v = kc[mb];
            ka[mb] = floatx4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                             __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
          } else {
            ka[mb] = kc[mb];
          }
        }
        const floatx4 sc = rope_scores(ka);
        int vm = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) vm |= (t0 + 4 * rho + i < w_end) ? (1 << i) : 0;
        float p[4];
        softmax_tile<8>(sc, vm, m, l, wacc, rho, p);
        if constexpr (BF) {
          unsigned h0, l0, h1, l1;
          split2(p[0], p[1], h0, l0, sk);
          split2(p[2], p[3], h1, l1, sk);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            wacc[nb] = mfma16(uint2_{h0, h1}, vc[nb], wacc[nb]);
            wacc[nb] = mfma16(uint2_{l0, l1}, vc[nb], wacc[nb]);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) wacc[nb] = mfma4(p[i], vc[nb][i], wacc[nb]);
        }
        if ((it & 31) == 31) anchor(t0 + 16 + n16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_acc[wave][4 * rho + i][16 * nb + n16] = wacc[nb][i];
  }
  const float lt = row_sum(l);
  if (rho == 0) {
    s_m[wave][n16] = m;
    s_l[wave][n16] = lt;
  }
  __syncthreads();

  // ---- combine the waves into this part's record
  const int width = comp ? RV : kHeadDim;
  const size_t rec0 = ((size_t)u * D.max_rec + rec_idx) * G;
  for (int e = threadIdx.x; e < G * (2 + width); e += C::kThr) {
    const int h = e / (2 + width), x = e % (2 + width);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w][h]);
    if (x == 0) {
      store_agent(M.sh.recml + (rec0 + h) * 2, mx);
      continue;
    }
    // an empty split (ragged batch) has no finite max: record l = 0, acc = 0
    const float mref = mx == -INFINITY ? 0.f : mx;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = __builtin_amdgcn_exp2f(s_m[w][h] - mref);
      v += wt * (x == 1 ? s_l[w][h] : s_acc[w][h][x - 2]);
    }
    if (x == 1) store_agent(M.sh.recml + (rec0 + h) * 2 + 1, v);
    else store_agent(M.sh.rec + (rec0 + h) * kRecStride + x - 2, v);
  }
  q_ready = true;
  };
  run_part(0);
  if (nparts == 2) run_part(1);

  // ---- fused: the last split workgroup of this unit to finish merges all
  // records (used when the whole grid is resident at once, so no merge holds
  // a CU that later workgroups wait for).  No workgroup waits on another.
  //
  // Why the merging workgroup, possibly on another XCD with its own L2, sees
  // every record:
  //   1. every record word is written and read only by agent-scope atomics,
  //      which are coherent across all XCDs of the device (the hardware keeps
  //      no private L2 copy of them), so there is no data race and no stale
  //      L2 line to write back or invalidate;
  //   2. each thread waits for its record stores to complete (vmcnt(0): a
  //      completed agent-scope store is performed at agent scope, the same
  //      wait the compiler's own release sequence ends with) before the
  //      barrier, and thread 0 increments the unit's count only after it;
  //   3. the workgroup whose increment returns splits - 1 comes after every
  //      other increment, hence after every record store completed; its
  //      threads issue their record loads only after a barrier that follows
  //      that return.
  // The relaxed orders leave steps 2-3 to the hardware's in-order completion.
  // The portable form (agent-scope release fence before the increment,
  // acquire fence in the merging workgroup) adds an L2 write-back and
  // invalidate meant for non-atomic data, which the records are not:
  // measured at +5% per call for batch 16 x 16K and +15% for one 32K
  // sequence, with identical results.
  if (!fused) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned done =
        __hip_atomic_fetch_add(M.sh.cnt + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned splits = sp.n ? (unsigned)plan_workgroups(plan) : gridDim.x;
    s_last = (done + 1 == splits) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  merge_unit<RV, NW>(M, layer, out, plan, u, s_dyn);
  if (threadIdx.x == 0) __hip_atomic_store(M.sh.cnt + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Unfused: one workgroup per unit merges after the split kernel.
template <int R>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(Model M, int layer, float *out,
                                                                SplitPlan plan, SeqPlans sp) {
  extern __shared__ __align__(16) uint8_t s_mrg[];
  const int u = blockIdx.x;
  merge_unit<R, 4>(M, layer, out, sp.n ? seq_plan(sp, u / M.D.kv_heads) : plan, u, s_mrg);
}

// Workgroups (of `waves` waves, `occ` per CU) per decode call: one resident
// round (every workgroup on a CU at once: one set-up per workgroup, the merge
// in the split kernel, no tail of late workgroups) when there are at least
// two tiles per wave, else enough for two tiles per wave.
// ISKV_DECODE_WORKGROUPS overrides it.
int target_workgroups(const Dims &D, int64_t length, int waves, int occ) {
  static int v = -1;
  if (v < 0) {
    const char *e = std::getenv("ISKV_DECODE_WORKGROUPS");
    v = e ? std::atoi(e) : 0;
    if (v < 0) v = 0;
  }
  if (v > 0) return v;
  const int64_t tiles = (int64_t)D.units * ((length + 15) / 16);
  const int64_t slots = (int64_t)D.cus * occ;
  int64_t t = (tiles + 2 * waves - 1) / (2 * waves);
  return (int)(t < slots ? t : slots);
}

// n_k compressed, n_e ring and n_p prefix tokens (for a ragged batch, the
// sequence's own); per_unit workgroups for the unit.  The window either gets
// workgroups of its own (about four tiles per wave each) or rides on the
// compressed workgroups (one window split after each compressed range),
// whichever gives the smaller largest workgroup: an exact tile costs about two
// compressed ones (its rows are 128 wide and loaded without the DMA ring),
// and a ride adds a second record (about two tiles).
SplitPlan make_plan_core(const Dims &D, int64_t n_k, int64_t n_e, int64_t n_p, int64_t per_unit,
                         int waves) {
  SplitPlan plan{};
  if (n_p > 0) {
    // the prefix as exact splits of about 256 tokens
    int64_t np = (n_p + 255) / 256;
    if (np > D.max_rec / 4) np = D.max_rec / 4;
    plan.pre_len = (int)(((n_p + np - 1) / np + 15) / 16 * 16);
    plan.n_pre = (int)((n_p + plan.pre_len - 1) / plan.pre_len);
  }
  // compressed splits: `want` workgroups, at least 2 tiles per wave, records
  // within max_rec (n_comp compressed + up to n_comp window + n_pre prefix)
  auto comp_splits = [&](int64_t want) {
    int64_t nc = (n_k + 32 * waves - 1) / (32 * waves);
    if (nc > want) nc = want;
    if (nc > (D.max_rec - plan.n_pre) / 2) nc = (D.max_rec - plan.n_pre) / 2;
    if (nc < 1) nc = 1;
    plan.comp_len = (int)(((n_k + nc - 1) / nc + 63) / 64 * 64);
    plan.n_comp = (int)((n_k + plan.comp_len - 1) / plan.comp_len);
  };
  const int64_t kt = (n_k + 15) / 16, et = (n_e + 15) / 16;     // tiles
  int64_t nw = (et + 4 * waves - 1) / (4 * waves);               // own window splits
  if (nw > D.max_rec / 2) nw = D.max_rec / 2;
  const int64_t avail = per_unit - plan.n_pre;
  bool rides = false;
  if (n_k > 0 && n_e > 0) {
    const int64_t sep_comp = avail - nw;
    if (sep_comp < 1) {
      rides = true;
    } else {
      const int64_t sep = std::max((kt + sep_comp - 1) / sep_comp, (2 * et + nw - 1) / nw);
      const int64_t ride = (kt + 2 * et + avail - 1) / std::max<int64_t>(avail, 1) + 2 * waves;
      rides = ride < sep;
    }
  }
  if (n_k > 0) {
    comp_splits(rides ? avail : (n_e > 0 ? avail - nw : avail));
    if (rides) {
      plan.win_rides = 1;
      plan.n_win = plan.n_comp;
      plan.win_len = (int)(((n_e + plan.n_comp - 1) / plan.n_comp + 15) / 16 * 16);
      return plan;
    }
  }
  if (n_e > 0) {
    if (nw > avail - (n_k > 0 ? plan.n_comp : 0)) nw = std::max<int64_t>(1, avail - (n_k > 0 ? plan.n_comp : 0));
    if (nw > D.max_rec - plan.n_pre - plan.n_comp) nw = D.max_rec - plan.n_pre - plan.n_comp;
    if (nw < 1) nw = 1;
    plan.win_len = (int)(((n_e + nw - 1) / nw + 15) / 16 * 16);
    plan.n_win = (int)((n_e + plan.win_len - 1) / plan.win_len);
  }
  return plan;
}

SplitPlan make_plan(const Dims &D, int64_t length, int64_t n_c, int waves, int occ) {
  const int64_t n_e = length > n_c ? length - n_c : 0;           // ring tokens
  const int64_t n_p = length < D.prefix ? length : D.prefix;     // prefix tokens
  const int64_t per_unit = target_workgroups(D, length, waves, occ) / D.units;
  return make_plan_core(D, n_c - D.prefix, n_e, n_p, per_unit < 1 ? 1 : per_unit, waves);
}

// Ragged batch: the workgroups a batch of the average length would get, per
// KV head `budget`, shared out so that the largest share of tokens is as
// small as the budget allows: the smallest cap c (tokens per workgroup) with
// sum_b max(1, ceil(L_b / c)) <= budget, sequence b taking ceil(L_b / c).
// With all lengths equal each sequence takes budget / n, the uniform call's
// count; with more sequences than the budget every sequence takes one.
// *largest (if given) = the most tokens any workgroup of the plan takes.
SeqPlans make_seq_plans(const Dims &D, const SeqTab &tab, int waves, int occ,
                        int64_t *largest = nullptr) {
  SeqPlans sp{};
  sp.n = tab.n;
  int64_t total = 0, lmax = 1;
  bool equal = true;
  for (int b = 0; b < tab.n; ++b) {
    total += tab.len[b];
    lmax = std::max<int64_t>(lmax, tab.len[b]);
    equal = equal && tab.len[b] == tab.len[0];
  }
  const int64_t target = target_workgroups(D, (total + tab.n - 1) / tab.n, waves, occ);
  const int64_t budget = target / D.kv_heads;
  auto shares = [&](int64_t cap) {
    int64_t s = 0;
    for (int b = 0; b < tab.n; ++b) s += std::max<int64_t>(1, (tab.len[b] + cap - 1) / cap);
    return s;
  };
  int64_t lo = 1, hi = lmax;                 // shares(lmax) = tab.n, the fewest
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (shares(mid) <= budget) hi = mid;
    else lo = mid + 1;
  }
  const int64_t cap = lo;
  int64_t most = 0;
  sp.off[0] = 0;
  for (int b = 0; b < tab.n; ++b) {
    const int64_t L = tab.len[b], c = tab.nc[b];
    const int64_t n_e = L > c ? L - c : 0;
    const int64_t n_p = L < D.prefix ? L : D.prefix;
    const int64_t per_unit = std::max<int64_t>(1, equal ? budget / tab.n : (L + cap - 1) / cap);
    most = std::max(most, (L + per_unit - 1) / per_unit);
    const SplitPlan p = make_plan_core(D, c - D.prefix, n_e, n_p, per_unit, waves);
    sp.n_comp[b] = (int16_t)p.n_comp;
    sp.n_pre[b] = (int16_t)p.n_pre;
    sp.n_win[b] = (int16_t)p.n_win;
    sp.comp_len[b] = p.comp_len;
    sp.pre_len[b] = p.pre_len;
    sp.win_len[b] = p.win_len;
    sp.win_rides[b] = (uint8_t)p.win_rides;
    sp.off[b + 1] = sp.off[b] + plan_workgroups(p);
  }
  if (largest) *largest = most;
  return sp;
}

template <int RK, int RV, typename T, int NW>
hipError_t launch_mfma(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                       int64_t length, int64_t n_c, const SplitPlan &plan, hipStream_t s,
                       FusedAppend app, const SeqTab &tab, const SeqPlans &sp) {
  using C = Cfg<RK, RV, T, NW>;
  const dim3 grid = sp.n ? dim3(sp.off[sp.n], M.D.kv_heads)
                         : dim3(plan_workgroups(plan), M.D.units);
  constexpr int dyn = C::kDynBytes;
  // the packed score product: bf16 storage with 4 query heads per KV head
  const bool pk = C::BF && M.D.group == 4;
  auto kern = pk ? &decode_mfma_kernel<RK, RV, T, NW, C::BF> : &decode_mfma_kernel<RK, RV, T, NW, false>;
  static bool dattr[2] = {false, false};
  hipError_t e;
  if (!dattr[pk]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
    if (e != hipSuccess) return e;
    dattr[pk] = true;
  }
  // fuse the merge when every workgroup is resident at once
  const int64_t slots = (int64_t)M.D.cus * C::kOcc;
  const int fused = (int64_t)grid.x * grid.y <= slots ? 1 : 0;
  hipLaunchKernelGGL(kern, grid, dim3(C::kThr), dyn, s, M, layer, q, q_pos,
                     out, length, n_c, plan, fused, app, tab, sp);
  e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  constexpr int mbytes = MergeLds<RV, 4>::bytes;
  static bool mattr = false;
  if (!mattr) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_merge_kernel<RV>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, mbytes);
    if (e != hipSuccess) return e;
    mattr = true;
  }
  hipLaunchKernelGGL((decode_merge_kernel<RV>), dim3(M.D.units), dim3(kThreads), mbytes, s, M, layer,
                     out, plan, sp);
  return hipGetLastError();
}

// bf16, r <= 64: eight-wave workgroups when their grid fits one per CU (a
// single launch wave, where two waves per SIMD and an even share per CU set
// the time); four-wave workgroups, two per CU (one for wider ranks and fp32),
// for larger grids.  ISKV_DECODE_WAVES=4 or 8 forces a form where it exists.
int forced_waves() {
  static int v = -1;
  if (v < 0) {
    const char *e = std::getenv("ISKV_DECODE_WAVES");
    v = e ? std::atoi(e) : 0;
  }
  return v;
}

template <int RK, int RV, typename T>
hipError_t launch_rank(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                       int64_t length, int64_t n_c, hipStream_t s, FusedAppend app, const SeqTab &tab) {
  constexpr int occ4 = Cfg<RK, RV, T, 4>::kOcc;
  constexpr bool has8 = std::is_same<T, bf16_t>::value && RK <= 64 && RV <= 64;
  if (tab.n) {
    // ragged: one plan per sequence, (sequence, split) flattened into grid.x;
    // with lengths that differ, eight waves only if the four-wave plan's
    // finer shares (twice the workgroups) do not leave each wave fewer
    // tokens; with equal lengths the uniform call's choice
    const SplitPlan none{};
    int64_t most4 = 0;
    const SeqPlans s4 = make_seq_plans(M.D, tab, 4, occ4, &most4);
    if constexpr (has8) {
      int64_t most8 = 0;
      const SeqPlans s8 = make_seq_plans(M.D, tab, 8, 1, &most8);
      bool same = true;
      for (int b = 1; b < tab.n; ++b) same = same && tab.len[b] == tab.len[0];
      if (forced_waves() == 8 ||
          (forced_waves() != 4 && (int64_t)s8.off[s8.n] * M.D.kv_heads <= M.D.cus &&
           (same || most8 <= 2 * most4)))
        return launch_mfma<RK, RV, T, 8>(M, layer, q, q_pos, out, length, n_c, none, s, app, tab, s8);
    }
    return launch_mfma<RK, RV, T, 4>(M, layer, q, q_pos, out, length, n_c, none, s, app, tab, s4);
  }
  const SeqPlans one{};
  if constexpr (has8) {
    const SplitPlan p8 = make_plan(M.D, length, n_c, 8, 1);
    if (forced_waves() == 8 ||
        (forced_waves() != 4 && (int64_t)plan_workgroups(p8) * M.D.units <= M.D.cus))
      return launch_mfma<RK, RV, T, 8>(M, layer, q, q_pos, out, length, n_c, p8, s, app, tab, one);
  }
  return launch_mfma<RK, RV, T, 4>(M, layer, q, q_pos, out, length, n_c,
                                   make_plan(M.D, length, n_c, 4, occ4), s, app, tab, one);
}

// (r_K, r_V): equal ranks, or a value rank twice the key rank
template <typename T>
hipError_t dispatch_decode(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                           int64_t length, int64_t n_c, hipStream_t s, FusedAppend app,
                           const SeqTab &tab) {
  const int rk = M.D.rk, rv = M.D.rv;
  if (rv == rk) {
    switch (rk) {
      case 16: return launch_rank<16, 16, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
      case 32: return launch_rank<32, 32, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
      case 64: return launch_rank<64, 64, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
      case 128: return launch_rank<128, 128, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
    }
  } else if (rv == 2 * rk) {
    switch (rk) {
      case 16: return launch_rank<16, 32, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
      case 32: return launch_rank<32, 64, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
      case 64: return launch_rank<64, 128, T>(M, layer, q, q_pos, out, length, n_c, s, app, tab);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------------------
// Split records of the allocation-free decode entry point: a file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// uses only the address hipGetSymbolAddress returns for the current device.
// Its merge counters start at zero when the code object loads and every
// completed decode call leaves them at zero again (the merging workgroup
// resets its unit's counter), so no per-call clear is needed; calls that
// overlap on one GPU would share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

void *scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

hipError_t launch_decode(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                         int64_t length, int64_t n_c, hipStream_t s, FusedAppend app) {
  const SeqTab none{};
  return M.D.storage == 1 ? dispatch_decode<bf16_t>(M, layer, q, q_pos, out, length, n_c, s, app, none)
                          : dispatch_decode<float>(M, layer, q, q_pos, out, length, n_c, s, app, none);
}

hipError_t launch_decode_ragged(const Model &M, int layer, const float *q, float *out,
                                const SeqTab &tab, hipStream_t s) {
  const FusedAppend none{};
  return M.D.storage == 1 ? dispatch_decode<bf16_t>(M, layer, q, 0, out, 0, 0, s, none, tab)
                          : dispatch_decode<float>(M, layer, q, 0, out, 0, 0, s, none, tab);
}

}  // namespace iskv
