// Internal layout and kernel-launch interface of libiskv (not part of the ABI).
//
// Device workspace, per layer (u = sequence * kv_heads + kv_head) and factor
// X = K, V with its rank r_X (r_K = rank, r_V = rank_v), in one generation
// (two with copy-on-write maintenance: the layer's current one, read by
// decode, and the one its maintenance writes):
//   basis[X]  float [U][d][r_X]         row f, column c (orthonormal columns)
//   sing[X]   float [CU][r_X]           singular values S
//   coef[X]   T     [CU][max_tokens][r_X]  coefficient rows (row = position)
//   frag      bytes [U][4*d*r_K]        key basis in the decode kernel's MFMA operand order
// and once per layer:
//   msync[X]  float [CU][r_X][r_X]      pending synchronization matrix M = B_old^T B_new
//   jres[X]   float [CU][64][H*d]       joint fold only: residual / Q rows of the block
//   jbn[X]    float [CU][H*d][r_X]      joint fold only: the new basis before it is stored
// CU, the coefficient units, is U (one basis per KV head) or, with a joint
// basis over a layer's H = kv_heads heads, the batch: sequence b's joint basis
// (H*d x r_X) is then the H slices [u = b*H .. b*H+H-1][d][r_X], row h*d + f
// of it being row f of unit b*H + h, and its one coefficient row per token
// serves all H heads.
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
  int cow;                // 1: copy-on-write maintenance (two generations, 64 more slots)
  int bulk_blocks;        // prefill: blocks folded per bulk pass (M slots per unit)
  int joint;              // 1: one basis per (sequence, layer) over all KV heads
  int cunits;             // coefficient units per layer: units, or batch when joint
};

// Coefficient unit of unit u, and the sequence of coefficient unit cu.
__host__ __device__ inline int coef_unit(const Dims &D, int u) { return D.joint ? u / D.kv_heads : u; }
__host__ __device__ inline int cunit_seq(const Dims &D, int cu) { return D.joint ? cu : cu / D.kv_heads; }

// Pointers of one layer.
struct LayerPtrs {
  float *basis[2], *sing[2], *msync[2];   // [X]: K = 0, V = 1
  float *jres[2], *jbn[2];                // joint fold scratch
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

struct GenLayout {
  size_t basis[2], sing[2], coef[2], frag;
};

struct LayerLayout {
  GenLayout gen[2];       // gen[1] == gen[0] without copy-on-write
  size_t msync[2], jres[2], jbn[2], ringk, ringv, prek, prev, bytes;
};

inline LayerLayout layer_layout(const Dims &D) {
  LayerLayout L{};
  size_t o = 0;
  const size_t U = (size_t)D.units, CU = (size_t)D.cunits;
  for (int g = 0; g < (D.cow ? 2 : 1); ++g) {
    GenLayout &G = L.gen[g];
    for (int x = 0; x < 2; ++x) {
      const size_t r = x ? D.rv : D.rk;
      G.basis[x] = o; o = align_up(o + U * D.d * r * 4);
      G.sing[x] = o;  o = align_up(o + CU * r * 4);
      G.coef[x] = o;  o = align_up(o + CU * (size_t)D.max_tokens * r * D.elem);
    }
    G.frag = o;  o = align_up(o + U * 4 * (size_t)D.d * D.rk);
  }
  if (!D.cow) L.gen[1] = L.gen[0];
  const size_t hd = D.joint ? (size_t)D.kv_heads * D.d : 0;
  for (int x = 0; x < 2; ++x) {
    const size_t r = x ? D.rv : D.rk;
    L.msync[x] = o; o = align_up(o + CU * r * r * 4);
    L.jres[x] = o;  o = align_up(o + CU * kBlock * hd * 4);
    L.jbn[x] = o;   o = align_up(o + CU * hd * r * 4);
  }
  L.ringk = o; o = align_up(o + (size_t)D.units * D.slots * D.d * D.elem);
  L.ringv = o; o = align_up(o + (size_t)D.units * D.slots * D.d * D.elem);
  L.prek = o;  o = align_up(o + (size_t)D.units * D.prefix * D.d * D.elem);
  L.prev = o;  o = align_up(o + (size_t)D.units * D.prefix * D.d * D.elem);
  L.bytes = o;
  return L;
}

struct GlobalLayout {
  LayerLayout layer;
  size_t layers_base, rec, recml, cnt, flags, rope_anchor, rope_step, bulk, total;
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
  G.bulk = o;        o = align_up(o + (size_t)D.units * D.bulk_blocks * ((size_t)D.rk * D.rk + (size_t)D.rv * D.rv) * 4);
  G.total = o;
  return G;
}

// Whole-workspace view handed to kernels by value.  Layer l's current
// generation is bit l of gen_mask (copy-on-write, at most 64 layers); a launch
// with out_flip = 1 reads the current generation and writes the other one.
struct Model {
  uint8_t *base;          // workspace base
  size_t layers_base;     // offset of layer 0
  size_t layer_stride;    // bytes per layer
  LayerLayout lay;        // offsets inside a layer
  Shared sh;
  Dims D;
  uint64_t gen_mask;
  int out_flip;
};

constexpr int kMaxLayerSel = 64;
struct LayerSel {
  int n;
  int idx[kMaxLayerSel];
};

__host__ __device__ inline int layer_gen(const Model &M, int l) {
  return l < 64 ? (int)((M.gen_mask >> l) & 1ull) : 0;
}

// Pointers of layer l in generation g (the per-layer parts are shared).
__host__ __device__ inline LayerPtrs layer_ptrs_gen(const Model &M, int l, int g) {
  uint8_t *b = M.base + M.layers_base + (size_t)l * M.layer_stride;
  const GenLayout &G = M.lay.gen[g];
  LayerPtrs P;
  for (int x = 0; x < 2; ++x) {
    P.basis[x] = (float *)(b + G.basis[x]);
    P.sing[x] = (float *)(b + G.sing[x]);
    P.msync[x] = (float *)(b + M.lay.msync[x]);
    P.jres[x] = (float *)(b + M.lay.jres[x]);
    P.jbn[x] = (float *)(b + M.lay.jbn[x]);
    P.coef[x] = b + G.coef[x];
  }
  P.frag = b + G.frag;
  P.ringk = b + M.lay.ringk;
  P.ringv = b + M.lay.ringv;
  P.prek = b + M.lay.prek;
  P.prev = b + M.lay.prev;
  return P;
}

// The generation a launch reads, and the one it writes.
__host__ __device__ inline LayerPtrs layer_ptrs(const Model &M, int l) {
  return layer_ptrs_gen(M, l, layer_gen(M, l));
}
__host__ __device__ inline LayerPtrs layer_ptrs_out(const Model &M, int l) {
  return layer_ptrs_gen(M, l, layer_gen(M, l) ^ M.out_flip);
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
// n_stride: tokens per sequence in the input (0: n), so that a range of a
// longer input can be appended.
hipError_t launch_append(const Model &M, int layer, const void *k, const void *v, int n,
                         int in_dtype, int64_t pos0, hipStream_t s, const SeqTab &tab = SeqTab{},
                         int n_stride = 0);

// Fold the block at positions n_c..n_c+63 of every unit of the selected
// layers: factor x (0 K, 1 V), or both (x = -1, one launch; equal ranks only).
// With a joint basis this is launch_joint_fold.
hipError_t launch_joint_fold(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                             const SeqTab &tab);
hipError_t launch_block_update(const Model &M, const LayerSel &sel, int64_t n_c, int x, hipStream_t s,
                               const SeqTab &tab = SeqTab{});

// C[0:n_old] <- C[0:n_old] * M for every unit of the selected layers, factor
// x (0 K, 1 V) or both (x = -1; equal ranks only).
hipError_t launch_sync(const Model &M, const LayerSel &sel, int64_t n_old, int x, hipStream_t s,
                       const SeqTab &tab = SeqTab{});

// Prefill of up to kMaxBulkLayers layers at once (the same length and
// compressed count): per layer i its input k[i], v[i] ([batch][n_in]
// [kv_heads][d], in_dtype 0 f32 / 1 bf16).
constexpr int kMaxBulkLayers = 16;
struct BulkIn {
  int n;
  int layer[kMaxBulkLayers];
  const void *k[kMaxBulkLayers], *v[kMaxBulkLayers];
};

// M slots of one layer in a bulk pass: [factor][unit][block][r][r].
__host__ __device__ inline size_t bulk_layer_floats(const Dims &D, int bulk_blocks) {
  return (size_t)D.units * bulk_blocks * ((size_t)D.rk * D.rk + (size_t)D.rv * D.rv);
}

// Fold nblk consecutive blocks of the inputs (rows row0..), the first at
// positions n_c0.., leaving each block's M in mbulk (bulk_blocks slots per
// unit, layer i at i * bulk_layer_floats) replaced by its suffix product;
// then launch_sync_bulk maps every older row by the product of the later M's.
hipError_t launch_bulk_fold(const Model &M, const BulkIn &in, int64_t n_c0, int nblk, int x, int in_dtype,
                            int64_t row0, int n_in, float *mbulk, int bulk_blocks, hipStream_t s);
hipError_t launch_sync_bulk(const Model &M, const BulkIn &in, int64_t n_c0, int nblk, int x,
                            const float *mbulk, int bulk_blocks, hipStream_t s);

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

// Allocation-free decode: the split records live in a file-scope device
// array of kScratchBytes (decode.hip).  scratch_setup looks its address up
// once per device (that device current); scratch_address returns it (null
// before setup).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_setup(int device);
void *scratch_address(int device);

// Bytes of the split records (rec, recml, cnt) a decode call of D uses, and
// their offsets when carved from one buffer.
struct RecLayout {
  size_t rec, recml, cnt, bytes;
};
inline RecLayout rec_layout(const Dims &D) {
  RecLayout R{};
  size_t o = 0;
  R.rec = o;   o = align_up(o + (size_t)D.units * D.max_rec * D.group * kRecStride * 4);
  R.recml = o; o = align_up(o + (size_t)D.units * D.max_rec * D.group * 2 * 4);
  R.cnt = o;   o = align_up(o + (size_t)D.units * 4);
  R.bytes = o;
  return R;
}

// Decode attention over a ragged batch: tab (n == batch) holds every
// sequence's length, compressed end and query position.
hipError_t launch_decode_ragged(const Model &M, int layer, const float *q, float *out,
                                const SeqTab &tab, hipStream_t s);

}  // namespace iskv
