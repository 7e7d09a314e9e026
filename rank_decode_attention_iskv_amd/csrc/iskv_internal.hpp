// Internal layout and kernel-launch interface of libiskv (not part of the ABI).
//
// Device workspace, per layer (u = sequence * kv_heads + kv_head) and factor
// X = K, V with its rank r_X (r_K = rank, r_V = rank_v):
//   basis[X]  float [U][d][r_X]         row f, column c (orthonormal columns)
//   sing[X]   float [U][r_X]            singular values S
//   msync[X]  float [U][r_X][r_X]       pending synchronization matrix M = B_old^T B_new
//   coef[X]   T     [U][max_tokens][r_X]  coefficient rows (row = position)
//   frag      bytes [U][4*d*r_K]        key basis in the decode kernel's MFMA operand order
//   ringk  T     [U][slots][d]       exact keys, row = ring slot (pre-RoPE)
//   ringv  T     [U][d][slots]       exact values, transposed (column = ring slot)
//   prek   T     [U][P][d]           protected prefix keys, row = position (pre-RoPE)
//   prev   T     [U][d][P]           protected prefix values, transposed
// plus, shared by all layers:
//   rec    float [U][max_rec][G][128]         split-K partial accumulators of decode
//   recml  float [U][max_rec][G][2]           split-K running max m and sum l
//   cnt    uint  [U]                          (reserved)
//   flags  int                                numeric flags (ISKV_FLAG_*)
//   rope   float                              RoPE tables (see rope_tables below)
// with T = float or bf16 (uint16 bit pattern) per the storage dtype.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace iskv {

constexpr int kHeadDim = 128;
constexpr int kBlock = 64;
constexpr int kRecStride = kHeadDim;           // accumulator floats per (record, head)
constexpr int kRopeAnchor = 64;                 // positions per anchor of the RoPE table

struct Dims {
  int batch, layers, kv_heads, q_heads, group, d, window, slots, max_tokens;
  int rk, rv;             // ranks of the key and value factors
  int storage;            // 0 f32, 1 bf16
  int elem;               // bytes per stored element
  float scale_log2;       // softmax scale * log2(e)
  float rope_base;
  int units;              // batch * kv_heads
  int max_rec;            // decode records per unit
  int rope_anchors;       // anchors in the RoPE table
  int cus;                // compute units of the device (decode grid sizing)
  int prefix;             // P: protected exact positions 0..P-1 (multiple of 64)
};

// Pointers of one layer.
struct LayerPtrs {
  float *basis[2], *sing[2], *msync[2];   // [X]: K = 0, V = 1
  uint8_t *coef[2];
  uint8_t *frag;
  uint8_t *ringk, *ringv, *prek, *prev;
};

struct Shared {
  float *rec;
  float *recml;
  unsigned *cnt;
  int *flags;
  const float *rope_anchor;   // [anchors][64 freq][2] cos, sin of (a * 64) * theta_i
  const float *rope_step;     // [64 offsets][64 freq][2] cos, sin of o * theta_i
};

inline __host__ __device__ size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

struct LayerLayout {
  size_t basis[2], sing[2], msync[2], coef[2], frag, ringk, ringv, prek, prev, bytes;
};

inline LayerLayout layer_layout(const Dims &D) {
  LayerLayout L{};
  size_t o = 0;
  const size_t U = (size_t)D.units;
  for (int x = 0; x < 2; ++x) {
    const size_t r = x ? D.rv : D.rk;
    L.basis[x] = o; o = align_up(o + U * D.d * r * 4);
    L.sing[x] = o;  o = align_up(o + U * r * 4);
    L.msync[x] = o; o = align_up(o + U * r * r * 4);
    L.coef[x] = o;  o = align_up(o + U * (size_t)D.max_tokens * r * D.elem);
  }
  L.frag = o;  o = align_up(o + U * 4 * (size_t)D.d * D.rk);
  L.ringk = o; o = align_up(o + (size_t)D.units * D.slots * D.d * D.elem);
  L.ringv = o; o = align_up(o + (size_t)D.units * D.slots * D.d * D.elem);
  L.prek = o;  o = align_up(o + (size_t)D.units * D.prefix * D.d * D.elem);
  L.prev = o;  o = align_up(o + (size_t)D.units * D.prefix * D.d * D.elem);
  L.bytes = o;
  return L;
}

struct GlobalLayout {
  LayerLayout layer;
  size_t layers_base, rec, recml, cnt, flags, rope_anchor, rope_step, total;
};

inline GlobalLayout global_layout(const Dims &D) {
  GlobalLayout G{};
  G.layer = layer_layout(D);
  size_t o = 0;
  G.layers_base = o; o = align_up(o + G.layer.bytes * D.layers);
  G.rec = o;   o = align_up(o + (size_t)D.units * D.max_rec * D.group * kRecStride * 4);
  G.recml = o; o = align_up(o + (size_t)D.units * D.max_rec * D.group * 2 * 4);
  G.cnt = o;   o = align_up(o + (size_t)D.units * 4);
  G.flags = o; o = align_up(o + 4);
  G.rope_anchor = o; o = align_up(o + (size_t)D.rope_anchors * 64 * 2 * 4);
  G.rope_step = o;   o = align_up(o + (size_t)kRopeAnchor * 64 * 2 * 4);
  G.total = o;
  return G;
}

// Whole-workspace view handed to kernels by value.
struct Model {
  uint8_t *base;          // workspace base
  size_t layers_base;     // offset of layer 0
  size_t layer_stride;    // bytes per layer
  LayerLayout lay;        // offsets inside a layer
  Shared sh;
  Dims D;
};

constexpr int kMaxLayerSel = 64;
struct LayerSel {
  int n;
  int idx[kMaxLayerSel];
};

__host__ __device__ inline LayerPtrs layer_ptrs(const Model &M, int l) {
  uint8_t *b = M.base + M.layers_base + (size_t)l * M.layer_stride;
  LayerPtrs P;
  for (int x = 0; x < 2; ++x) {
    P.basis[x] = (float *)(b + M.lay.basis[x]);
    P.sing[x] = (float *)(b + M.lay.sing[x]);
    P.msync[x] = (float *)(b + M.lay.msync[x]);
    P.coef[x] = b + M.lay.coef[x];
  }
  P.frag = b + M.lay.frag;
  P.ringk = b + M.lay.ringk;
  P.ringv = b + M.lay.ringv;
  P.prek = b + M.lay.prek;
  P.prev = b + M.lay.prev;
  return P;
}

// Per-sequence values of a call over a ragged batch (sequences at different
// lengths), passed to the kernels by value.  n == 0: every sequence takes the
// call's scalar arguments and takes part.  Otherwise n == batch (at most
// kMaxSeqTab), bit b of mask says whether sequence b takes part, and
//   decode: len = tokens held, nc = end of the compressed rows, aux = query position
//   append: len = first position written, aux = tokens written (<= the call's n)
//   fold:   nc = end of the compressed rows before the fold
//   sync:   nc = end of the rows the sync maps (n_old)
constexpr int kMaxSeqTab = 64;
struct SeqTab {
  int n;
  uint64_t mask;
  int32_t len[kMaxSeqTab];
  int32_t nc[kMaxSeqTab];
  int32_t aux[kMaxSeqTab];
};

__host__ __device__ inline bool seq_in(const SeqTab &t, int b) {
  return t.n == 0 || ((t.mask >> b) & 1ull) != 0;
}

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files). Each returns hipSuccess or the
// launch error.
// ---------------------------------------------------------------------------

// Reset one layer: basis = I[:, :r], S = 0, M = 0, coefficients and rings 0.
hipError_t launch_reset_layer(const Model &M, int layer, hipStream_t s);

// Write n tokens at positions pos0.. into the protected prefix (positions < P)
// or the rings (in_dtype 0 f32, 1 bf16).
hipError_t launch_append(const Model &M, int layer, const void *k, const void *v, int n,
                         int in_dtype, int64_t pos0, hipStream_t s, const SeqTab &tab = SeqTab{});

// Fold the block at positions n_c..n_c+63 of every unit of the selected
// layers: factor x (0 K, 1 V), or both (x = -1, one launch; equal ranks only).
hipError_t launch_block_update(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                               const SeqTab &tab = SeqTab{});

// C[0:n_old] <- C[0:n_old] * M for every unit of the selected layers, factor
// x (0 K, 1 V) or both (x = -1; equal ranks only).
hipError_t launch_sync(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                       const SeqTab &tab = SeqTab{});

// Rebuild the decode operand copy of the basis from the fp32 basis.
hipError_t launch_prep_frag(const Model &M, const LayerSel &sel, hipStream_t s);

// A token appended by the decode launch itself (k, v: [batch][1][kv_heads][d],
// in_dtype 0 f32, 1 bf16; k == nullptr: none).  The workgroup whose window
// split ends at the newest position writes its ring rows before reading them.
struct FusedAppend {
  const void *k, *v;
  int in_dtype;
};

// Decode attention for one layer.  With a fused append, `length` already
// counts the appended token.
hipError_t launch_decode(const Model &M, int layer, const float *q, int64_t q_pos, float *out,
                         int64_t length, int64_t n_c, hipStream_t s, FusedAppend app = FusedAppend{});

// Decode attention over a ragged batch: tab (n == batch) holds every
// sequence's length, compressed end and query position.
hipError_t launch_decode_ragged(const Model &M, int layer, const float *q, float *out,
                                const SeqTab &tab, hipStream_t s);

}  // namespace iskv
