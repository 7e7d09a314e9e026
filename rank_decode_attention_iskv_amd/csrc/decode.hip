// Decode attention over the mixed cache (exact window + low-rank history).
//
// Page: "iS-KV -- Basis-synchronized online low-rank KV compression -- What does
// it mean?" (learnaivisually.com), cited as [iS-KV explainer]: every new query
// scores every earlier key (re-attention paragraph); old keys are rebuilt from
// their coefficients over the shared basis and RoPE is re-applied at the key's
// position (Jargon "Basis and coefficients", "Pre-RoPE keys").  Values are
// accumulated in coefficient space, sum_t p_t c_t, and mapped back once by the
// value basis: (p^T C) B^T = p^T (C B^T).
//
// Split-K: each workgroup attends over one token range of one (sequence, KV
// head) for all query heads of its group and writes a partial record
// (running max m, sum l, accumulator); the last workgroup to arrive for that
// (sequence, KV head) merges the records by log-sum-exp and writes the output.
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct SplitPlan {
  int n_comp;        // splits over compressed tokens
  int comp_len;      // tokens per compressed split (multiple of 64)
  int n_win;         // splits over window tokens
  int win_len;       // tokens per window split
};

// Merge the split records of unit u and write out[b][h_kv*G + h][:].
// Called by every thread of the last-arriving workgroup.
template <int R>
__device__ void merge_records(const Model &M, int layer, int u, int n_rec, int n_comp,
                              float *out, float *lds) {
  const Dims &D = M.D;
  const int G = D.group, tid = threadIdx.x;
  const float *rec = M.sh.rec + (size_t)u * D.max_rec * G * kRecStride;
  float *sMx = lds;                       // [G]
  float *sL = sMx + 16;                   // [G]
  float *sC = sL + 16;                    // [G][R]
  float *sW = sC + 16 * R;                // [G][128]
  if (tid < G) {
    float mx = -INFINITY;
    for (int s = 0; s < n_rec; ++s) mx = fmaxf(mx, rec[((size_t)s * G + tid) * kRecStride]);
    float l = 0.f;
    for (int s = 0; s < n_rec; ++s) {
      const float *r = rec + ((size_t)s * G + tid) * kRecStride;
      l += r[1] * exp2f(r[0] - mx);
    }
    sMx[tid] = mx;
    sL[tid] = l;
  }
  __syncthreads();
  for (int e = tid; e < G * R; e += blockDim.x) {
    const int h = e / R, c = e % R;
    float a = 0.f;
    for (int s = 0; s < n_comp; ++s) {
      const float *r = rec + ((size_t)s * G + h) * kRecStride;
      a += r[2 + c] * exp2f(r[0] - sMx[h]);
    }
    sC[h * R + c] = a;
  }
  for (int e = tid; e < G * kHeadDim; e += blockDim.x) {
    const int h = e / kHeadDim, f = e % kHeadDim;
    float a = 0.f;
    for (int s = n_comp; s < n_rec; ++s) {
      const float *r = rec + ((size_t)s * G + h) * kRecStride;
      a += r[2 + f] * exp2f(r[0] - sMx[h]);
    }
    sW[h * kHeadDim + f] = a;
  }
  __syncthreads();
  LayerPtrs P = layer_ptrs(M, layer);
  const float *Bv = P.basis + ((size_t)u * 2 + 1) * kHeadDim * R;
  const int b = u / D.kv_heads, hk = u % D.kv_heads;
  for (int e = tid; e < G * kHeadDim; e += blockDim.x) {
    const int h = e / kHeadDim, f = e % kHeadDim;
    float a = sW[h * kHeadDim + f];
    if (n_comp > 0)
      for (int c = 0; c < R; ++c) a += Bv[f * R + c] * sC[h * R + c];
    out[((size_t)b * D.q_heads + hk * G + h) * kHeadDim + f] = a / sL[h];
  }
}

// Arrival counter; returns true in every thread of the last workgroup.
__device__ bool arrive_last(const Model &M, int u, int total, int *s_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = atomicAdd(&M.sh.cnt[u], 1u);
    const bool last = (old == (unsigned)total - 1);
    if (last) M.sh.cnt[u] = 0;       // self-reset for the next call
    *s_flag = last;
  }
  __syncthreads();
  const bool last = *s_flag;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------------------
// Reference-style decode: one token per thread, fp32 VALU throughout.
// grid (splits, units); LDS: q (G x 128), B_K (128 x (R+1)), scores (G x 256).
// ---------------------------------------------------------------------------
template <int R, typename T>
__global__ __launch_bounds__(kThreads) void decode_simple_kernel(Model M, int layer,
                                                                 const float *q, int64_t q_pos,
                                                                 float *out, int64_t length,
                                                                 int64_t n_c, SplitPlan plan) {
  extern __shared__ float lds[];
  __shared__ float sm[16], sl[16], salpha[16];
  __shared__ int s_flag;
  const Dims &D = M.D;
  const int G = D.group, tid = threadIdx.x;
  const int split = blockIdx.x, u = blockIdx.y;
  const int b = u / D.kv_heads, hk = u % D.kv_heads;
  const bool comp = split < plan.n_comp;
  int64_t t_begin, t_end;
  if (comp) {
    t_begin = (int64_t)split * plan.comp_len;
    t_end = t_begin + plan.comp_len < n_c ? t_begin + plan.comp_len : n_c;
  } else {
    t_begin = n_c + (int64_t)(split - plan.n_comp) * plan.win_len;
    t_end = t_begin + plan.win_len < length ? t_begin + plan.win_len : length;
  }
  constexpr int BP = R + 1;
  float *sq = lds;                          // [16][128]
  float *sB = sq + 16 * kHeadDim;           // [128][BP]
  float *ssc = sB + kHeadDim * BP;          // [16][256]
  float *sacc = ssc + 16 * kThreads;        // [16][128]

  LayerPtrs P = layer_ptrs(M, layer);
  // query rows of the group, rotated at q_pos, scaled by scale*log2(e)
  for (int e = tid; e < G * 64; e += kThreads) {
    const int h = e / 64, i = e % 64;
    const float *qr = q + ((size_t)b * D.q_heads + hk * G + h) * kHeadDim;
    float c, s;
    rope_cs(M.sh, q_pos, i, c, s);
    const float x0 = qr[i], x1 = qr[i + 64];
    sq[h * kHeadDim + i] = (x0 * c - x1 * s) * D.scale_log2;
    sq[h * kHeadDim + i + 64] = (x1 * c + x0 * s) * D.scale_log2;
  }
  const float *Bk = P.basis + ((size_t)u * 2 + 0) * kHeadDim * R;
  if (comp)
    for (int e = tid; e < kHeadDim * R; e += kThreads) sB[(e / R) * BP + e % R] = Bk[e];
  const int accw = comp ? R : kHeadDim;
  for (int e = tid; e < G * kHeadDim; e += kThreads) sacc[e] = 0.f;
  if (tid < 16) { sm[tid] = -INFINITY; sl[tid] = 0.f; }
  __syncthreads();

  const T *Ck = reinterpret_cast<const T *>(P.coef) + ((size_t)u * 2 + 0) * D.max_tokens * R;
  const T *Cv = reinterpret_cast<const T *>(P.coef) + ((size_t)u * 2 + 1) * D.max_tokens * R;
  const T *rk = reinterpret_cast<const T *>(P.ringk) + (size_t)u * D.slots * kHeadDim;
  const T *rv = reinterpret_cast<const T *>(P.ringv) + (size_t)u * D.slots * kHeadDim;

  for (int64_t base = t_begin; base < t_end; base += kThreads) {
    const int64_t t = base + tid;
    const bool valid = t < t_end;
    float s[16];
    for (int h = 0; h < 16; ++h) s[h] = 0.f;
    if (valid) {
      float cf[R];
      if (comp) {
#pragma unroll
        for (int c = 0; c < R; ++c) cf[c] = Store<T>::load(Ck, (size_t)t * R + c);
      }
      const int slot = (int)(t % D.slots);
      for (int i = 0; i < 64; ++i) {
        float k0, k1;
        if (comp) {
          k0 = 0.f; k1 = 0.f;
#pragma unroll
          for (int c = 0; c < R; ++c) {
            k0 += sB[i * BP + c] * cf[c];
            k1 += sB[(i + 64) * BP + c] * cf[c];
          }
        } else {
          k0 = Store<T>::load(rk, (size_t)slot * kHeadDim + i);
          k1 = Store<T>::load(rk, (size_t)slot * kHeadDim + i + 64);
        }
        float cs, sn;
        rope_cs(M.sh, t, i, cs, sn);
        const float r0 = k0 * cs - k1 * sn, r1 = k1 * cs + k0 * sn;
        for (int h = 0; h < G; ++h)
          s[h] += sq[h * kHeadDim + i] * r0 + sq[h * kHeadDim + i + 64] * r1;
      }
    }
    for (int h = 0; h < G; ++h) ssc[h * kThreads + tid] = valid ? s[h] : -INFINITY;
    __syncthreads();
    // online softmax update, one wave per head
    const int w = tid >> 6, ln = tid & 63;
    for (int h = w; h < G; h += kThreads / 64) {
      float mx = -INFINITY;
      for (int j = ln; j < kThreads; j += 64) mx = fmaxf(mx, ssc[h * kThreads + j]);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float mnew = fmaxf(sm[h], mx);
      float sum = 0.f;
      for (int j = ln; j < kThreads; j += 64) {
        const float p = exp2f(ssc[h * kThreads + j] - mnew);
        ssc[h * kThreads + j] = p;
        sum += p;
      }
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (ln == 0) {
        const float al = exp2f(sm[h] - mnew);
        salpha[h] = al;
        sl[h] = sl[h] * al + sum;
        sm[h] = mnew;
      }
    }
    __syncthreads();
    const int n = (int)((t_end - base) < kThreads ? (t_end - base) : kThreads);
    for (int e = tid; e < G * accw; e += kThreads) {
      const int h = e / accw, x = e % accw;
      float a = sacc[h * kHeadDim + x] * salpha[h];
      if (comp) {
        for (int j = 0; j < n; ++j) a += ssc[h * kThreads + j] * Store<T>::load(Cv, (size_t)(base + j) * R + x);
      } else {
        for (int j = 0; j < n; ++j)
          a += ssc[h * kThreads + j] *
               Store<T>::load(rv, (size_t)x * D.slots + (size_t)((base + j) % D.slots));
      }
      sacc[h * kHeadDim + x] = a;
    }
    __syncthreads();
  }
  // partial record
  float *rec = M.sh.rec + ((size_t)u * D.max_rec + split) * G * kRecStride;
  for (int e = tid; e < G * (2 + kHeadDim); e += kThreads) {
    const int h = e / (2 + kHeadDim), x = e % (2 + kHeadDim);
    float v;
    if (x == 0) v = sm[h];
    else if (x == 1) v = sl[h];
    else v = sacc[h * kHeadDim + x - 2];
    rec[(size_t)h * kRecStride + x] = v;
  }
  const int total = plan.n_comp + plan.n_win;
  if (!arrive_last(M, u, total, &s_flag)) return;
  merge_records<R>(M, layer, u, total, plan.n_comp, out, lds);
}

template <int R, typename T>
hipError_t launch_simple(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                         int64_t length, int64_t n_c, hipStream_t s) {
  const Dims &D = M.D;
  SplitPlan plan{};
  const int64_t n_e = length - n_c;
  if (n_e > 0) {
    int64_t nw = (n_e + 255) / 256;
    if (nw > D.max_rec / 2) nw = D.max_rec / 2;
    plan.n_win = (int)nw;
    plan.win_len = (int)((n_e + nw - 1) / nw);
  }
  const int target = 1024;
  const int want = (target + D.units - 1) / D.units;
  if (n_c > 0) {
    int64_t nc = (n_c + 255) / 256;
    if (nc > want) nc = want;
    if (nc > D.max_rec - plan.n_win) nc = D.max_rec - plan.n_win;
    if (nc < 1) nc = 1;
    plan.comp_len = (int)(((n_c + nc - 1) / nc + 63) / 64 * 64);
    plan.n_comp = (int)((n_c + plan.comp_len - 1) / plan.comp_len);
  }
  const size_t bytes = (size_t)(16 * kHeadDim + kHeadDim * (R + 1) + 16 * kThreads + 16 * kHeadDim) * 4;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_simple_kernel<R, T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  dim3 grid(plan.n_comp + plan.n_win, D.units);
  hipLaunchKernelGGL((decode_simple_kernel<R, T>), grid, dim3(kThreads), bytes, s, M, layer, q,
                     q_pos, out, length, n_c, plan);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_decode(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                           int64_t length, int64_t n_c, hipStream_t s) {
  switch (M.D.r) {
    case 16: return launch_simple<16, T>(M, layer, q, q_pos, out, length, n_c, s);
    case 32: return launch_simple<32, T>(M, layer, q, q_pos, out, length, n_c, s);
    case 64: return launch_simple<64, T>(M, layer, q, q_pos, out, length, n_c, s);
    case 128: return launch_simple<128, T>(M, layer, q, q_pos, out, length, n_c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                         int64_t length, int64_t n_c, hipStream_t s) {
  return M.D.storage == 1 ? dispatch_decode<bf16_t>(M, layer, q, q_pos, out, length, n_c, s)
                          : dispatch_decode<float>(M, layer, q, q_pos, out, length, n_c, s);
}

}  // namespace iskv
