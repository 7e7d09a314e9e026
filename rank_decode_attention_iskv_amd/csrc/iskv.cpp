// libiskv host side: configuration checks, workspace carving, the per-layer
// state machine (length, compressed count, pending synchronization), launches,
// status, and state export/import.
//
// Operations follow [iS-KV explainer] ("iS-KV -- Basis-synchronized online
// low-rank KV compression -- What does it mean?", learnaivisually.com):
// exact recent window, 64-token blocks folded by Brand's block-incremental
// SVD, basis synchronization of old coefficients, decode attention over every
// position; persistent-KV bytes as in its Jargon entry.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "iskv.h"
#include "iskv_internal.hpp"

using namespace iskv;

namespace {

struct SeqState {
  int64_t length = 0;
  int64_t n_c = 0;
  bool pending = false;
};

// A layer whose sequences agree is uniform (length, n_c, pending).  The ragged
// verbs split it into one SeqState per sequence (ragged = true); the uniform
// verbs merge it back when every sequence agrees again.
struct LayerState {
  int64_t length = 0;
  int64_t n_c = 0;          // end position of the compressed rows (P + N_c)
  bool pending = false;
  int64_t folds = 0;
  int64_t syncs = 0;
  bool inflight = false;    // copy-on-write: a maintenance of this layer is enqueued
  bool ragged = false;
  std::vector<SeqState> seq;
};

bool valid_config(const iskv_config *c) {
  if (!c) return false;
  if (c->batch < 1 || c->num_layers < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1) return false;
  if (c->num_q_heads % c->num_kv_heads) return false;
  const int g = c->num_q_heads / c->num_kv_heads;
  if (g < 1 || g > 16) return false;           // query heads of a group fill <= 16 MFMA columns
  if (c->head_dim != kHeadDim) return false;
  if (c->rank != 16 && c->rank != 32 && c->rank != 64 && c->rank != 128) return false;
  if (c->rank > c->head_dim) return false;
  // value rank: 0 (= rank), rank, or twice rank (<= head_dim)
  if (c->rank_v != 0 && c->rank_v != c->rank && c->rank_v != 2 * c->rank) return false;
  if (c->rank_v > c->head_dim) return false;
  if (c->block != kBlock) return false;
  if (c->window < kBlock || c->window % kBlock) return false;
  if (c->max_tokens < 1 || c->max_tokens > (1 << 24)) return false;
  if (c->storage != ISKV_F32 && c->storage != ISKV_BF16) return false;
  if (!(c->rope_base > 1.f) || !std::isfinite(c->rope_base)) return false;
  if (!std::isfinite(c->softmax_scale)) return false;
  if (c->protected_prefix < 0 || c->protected_prefix % kBlock || c->protected_prefix > c->max_tokens)
    return false;
  if (c->async_maintenance != 0 && c->async_maintenance != 1) return false;
  if (c->async_maintenance && c->num_layers > 64) return false;   // one generation bit per layer
  if (c->joint_heads != 0 && c->joint_heads != 1) return false;
  if (c->joint_heads) {
    // the joint fold keeps an (r+64)-square core and a head's block columns in
    // LDS: r <= 64, and at most 32 heads for its null-completion vectors
    const int rv = c->rank_v ? c->rank_v : c->rank;
    if (c->rank > 64 || rv > 64 || c->num_kv_heads > 32) return false;
  }
  return true;
}

Dims make_dims(const iskv_config *c) {
  Dims D{};
  D.batch = c->batch;
  D.layers = c->num_layers;
  D.kv_heads = c->num_kv_heads;
  D.q_heads = c->num_q_heads;
  D.group = c->num_q_heads / c->num_kv_heads;
  D.d = c->head_dim;
  D.rk = c->rank;
  D.rv = c->rank_v ? c->rank_v : c->rank;
  D.window = c->window;
  D.cow = c->async_maintenance;
  D.slots = c->window + kBlock * (1 + D.cow);     // copy-on-write: a block of slack
  D.max_tokens = c->max_tokens;
  D.storage = c->storage;
  D.elem = c->storage == ISKV_BF16 ? 2 : 4;
  const double scale = c->softmax_scale > 0.f ? (double)c->softmax_scale
                                              : 1.0 / std::sqrt((double)c->head_dim);
  D.scale_log2 = (float)(scale * 1.4426950408889634);
  D.rope_base = c->rope_base;
  D.units = c->batch * c->num_kv_heads;
  D.joint = c->joint_heads;
  D.cunits = D.joint ? c->batch : D.units;
  // decode split records per unit: enough to spread the history over a few
  // waves of workgroups on 256 compute units, plus the window splits; the
  // merge keeps every (record, head) max and sum of a unit in LDS (<= 4096)
  int per_unit = (4096 + D.units - 1) / D.units;
  if (per_unit < 16) per_unit = 16;
  if (per_unit * D.group > 4096) per_unit = 4096 / D.group;
  D.max_rec = per_unit;
  D.rope_anchors = (c->max_tokens + kBlock) / kRopeAnchor + 2;
  D.prefix = c->protected_prefix;
  // prefill: M slots per unit for one bulk pass, within 64 MiB (ISKV_BULK_BLOCKS
  // lowers the count, e.g. to exercise several passes)
  const size_t per_block = (size_t)D.units * ((size_t)D.rk * D.rk + (size_t)D.rv * D.rv) * 4;
  int64_t nb = (int64_t)((64ull << 20) / per_block);
  nb = std::min<int64_t>(nb, c->max_tokens / kBlock + 1);
  if (const char *e = std::getenv("ISKV_BULK_BLOCKS")) {
    const int64_t v = std::atoll(e);
    if (v > 0) nb = std::min<int64_t>(nb, v);
  }
  D.bulk_blocks = (int)std::max<int64_t>(1, nb);
  return D;
}

uint16_t host_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float host_from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

struct iskv_ctx {
  iskv_config cfg;
  Dims D;
  GlobalLayout G;
  Model M;
  hipStream_t stream;
  int device;
  std::vector<LayerState> layers;
  // optional maintenance stream: block update + sync of a layer run there,
  // after the main stream's earlier work, and the main stream's later work on
  // that layer waits for them (per-layer events)
  hipStream_t mstream = nullptr;
  hipEvent_t ev_main = nullptr;
  // different K and V ranks: the V fold / sync run on `aux`, forked from and
  // joined back into the stream of the call, so both factors' kernels overlap
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  std::vector<hipEvent_t> ev_done;
  std::vector<char> maint_pending;
  // copy-on-write: per-layer event recorded after the layer's maintenance
  std::vector<hipEvent_t> ev_cow;
};

namespace {

int hip_err(hipError_t e) { return e == hipSuccess ? ISKV_OK : ISKV_EDEVICE; }

int check_layer(const iskv_ctx *c, int layer) {
  return (layer >= 0 && layer < c->D.layers) ? ISKV_OK : ISKV_EINVAL;
}

void make_ragged(const iskv_ctx *c, LayerState &L);
bool make_uniform(LayerState &L);

// A block can be folded: the ring holds window + 64 rows past the compressed
// ones (and, with copy-on-write, no maintenance is in flight).
bool block_ready(const iskv_ctx *c, const LayerState &L) {
  const int64_t held = L.length - L.n_c;
  if (c->D.cow) return !L.inflight && held >= c->D.window + kBlock;
  return held == c->D.slots;
}

// Copy-on-write decode boundary: switch `layer` to the generation its
// maintenance wrote once that has finished (wait: make the init stream wait
// for it).  1 switched, 0 not, < 0 error code.
int cow_switch(iskv_ctx *c, int layer, bool wait) {
  LayerState &L = c->layers[layer];
  if (!c->D.cow || !L.inflight) return 0;
  if (!wait) {
    const hipError_t q = hipEventQuery(c->ev_cow[layer]);
    if (q == hipErrorNotReady) return 0;
    if (q != hipSuccess) return ISKV_EDEVICE;
  }
  // finished or not, later init-stream work is ordered after it
  if (hipStreamWaitEvent(c->stream, c->ev_cow[layer], 0) != hipSuccess) return ISKV_EDEVICE;
  c->M.gen_mask ^= 1ull << layer;
  L.n_c += kBlock;
  L.inflight = false;
  return 1;
}

SeqState seq_state(const LayerState &L, int b) {
  return L.ragged ? L.seq[(size_t)b] : SeqState{L.length, L.n_c, L.pending};
}

// Main-stream work on `layer` from here on waits for its pending maintenance.
hipError_t join_layer(iskv_ctx *c, int layer) {
  if (!c->mstream || !c->maint_pending[layer]) return hipSuccess;
  c->maint_pending[layer] = 0;
  return hipStreamWaitEvent(c->stream, c->ev_done[layer], 0);
}

hipError_t join_all(iskv_ctx *c) {
  for (int l = 0; l < c->D.layers; ++l) {
    hipError_t e = join_layer(c, l);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The stream maintenance work goes to, ordered after the main stream's work
// enqueued so far.
hipStream_t maint_stream(iskv_ctx *c, hipError_t *err) {
  *err = hipSuccess;
  if (!c->mstream) return c->stream;
  *err = hipEventRecord(c->ev_main, c->stream);
  if (*err == hipSuccess) *err = hipStreamWaitEvent(c->mstream, c->ev_main, 0);
  return c->mstream;
}

hipError_t maint_done(iskv_ctx *c, int layer) {
  if (!c->mstream) return hipSuccess;
  c->maint_pending[layer] = 1;
  return hipEventRecord(c->ev_done[layer], c->mstream);
}

void fill_sel(LayerSel &sel, const std::vector<int> &idx, size_t from) {
  sel.n = 0;
  for (size_t i = from; i < idx.size() && sel.n < kMaxLayerSel; ++i) sel.idx[sel.n++] = idx[i];
}

// Run launch(x, stream) for both factors: one launch (x = -1) when the ranks
// are equal; otherwise K on s and V on the helper stream, forked from s and
// joined back into it.
template <typename F>
hipError_t for_factors(iskv_ctx *c, hipStream_t s, F launch) {
  if (c->D.rk == c->D.rv) return launch(-1, s);
  hipError_t e = hipEventRecord(c->ev_fork, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->aux, c->ev_fork, 0);
  if (e == hipSuccess) e = launch(0, s);
  if (e == hipSuccess) e = launch(1, c->aux);
  if (e == hipSuccess) e = hipEventRecord(c->ev_join, c->aux);
  if (e == hipSuccess) e = hipStreamWaitEvent(s, c->ev_join, 0);
  return e;
}

uint64_t persistent_bytes(const iskv_ctx *c) {
  const Dims &D = c->D;
  uint64_t tot = 0;
  for (const LayerState &L : c->layers) {
    for (int b = 0; b < D.batch; ++b) {
      const SeqState q = seq_state(L, b);
      // exact rows: the protected prefix written so far and the ring
      const uint64_t n_pre = (uint64_t)(q.length < D.prefix ? q.length : D.prefix);
      const uint64_t n_e = (uint64_t)(q.length > q.n_c ? q.length - q.n_c : 0) + n_pre;
      const uint64_t n_comp = (uint64_t)(q.n_c - D.prefix);
      // per unit: both factors' coefficients, bases and singular values, and
      // the exact rows of K and V; a joint basis keeps one coefficient row and
      // one S per sequence, its basis rows are the heads' slices
      const uint64_t rs = (uint64_t)D.rk + D.rv;
      const uint64_t H = (uint64_t)D.kv_heads;
      const uint64_t shared = n_comp * rs * D.elem + rs * 4;
      tot += (D.joint ? shared : shared * H) +
             H * ((uint64_t)D.d * rs * 4 + 2ull * n_e * D.d * D.elem);
    }
  }
  return tot;
}

void make_ragged(const iskv_ctx *c, LayerState &L) {
  if (L.ragged) return;
  L.seq.assign((size_t)c->D.batch, SeqState{L.length, L.n_c, L.pending});
  L.ragged = true;
}

bool make_uniform(LayerState &L) {
  if (!L.ragged) return true;
  const SeqState &a = L.seq[0];
  for (const SeqState &q : L.seq)
    if (q.length != a.length || q.n_c != a.n_c || q.pending != a.pending) return false;
  L.length = a.length;
  L.n_c = a.n_c;
  L.pending = a.pending;
  L.ragged = false;
  return true;
}

uint64_t seq_bits(int batch) { return batch >= 64 ? ~0ull : (1ull << batch) - 1; }

// Fold every sequence of a ragged layer whose ring is full (one launch per
// factor; the others' workgroups return at once).  need: no sequence ready is
// an error.
int fold_ragged(iskv_ctx *c, int layer, bool need) {
  LayerState &L = c->layers[layer];
  SeqTab tab{};
  tab.n = c->D.batch;
  for (int b = 0; b < c->D.batch; ++b) {
    const SeqState &q = L.seq[(size_t)b];
    tab.nc[b] = (int32_t)q.n_c;
    if (!q.pending && q.length - q.n_c == c->D.slots) tab.mask |= 1ull << b;
  }
  if (!tab.mask) return need ? ISKV_ESTATE : ISKV_OK;
  hipError_t se;
  hipStream_t s = maint_stream(c, &se);
  if (se != hipSuccess) return ISKV_EDEVICE;
  LayerSel sel;
  fill_sel(sel, std::vector<int>{layer}, 0);
  hipError_t e = for_factors(c, s, [&](int x, hipStream_t st) {
    return launch_block_update(c->M, sel, 0, x, st, tab);
  });
  if (e == hipSuccess) e = launch_prep_frag(c->M, sel, s);
  if (e != hipSuccess) return ISKV_EDEVICE;
  for (int b = 0; b < c->D.batch; ++b)
    if ((tab.mask >> b) & 1ull) {
      L.seq[(size_t)b].n_c += kBlock;
      L.seq[(size_t)b].pending = true;
    }
  L.folds += 1;
  return maint_done(c, layer) != hipSuccess ? ISKV_EDEVICE : ISKV_OK;
}

// Synchronize every sequence of a ragged layer with a pending fold.
int sync_ragged(iskv_ctx *c, int layer, bool need) {
  LayerState &L = c->layers[layer];
  SeqTab tab{};
  tab.n = c->D.batch;
  int64_t n_max = 0;
  for (int b = 0; b < c->D.batch; ++b) {
    const SeqState &q = L.seq[(size_t)b];
    if (!q.pending) continue;
    tab.mask |= 1ull << b;
    tab.nc[b] = (int32_t)(q.n_c - kBlock);
    n_max = std::max<int64_t>(n_max, q.n_c - kBlock);
  }
  if (!tab.mask) return need ? ISKV_ESTATE : ISKV_OK;
  hipError_t se;
  hipStream_t s = maint_stream(c, &se);
  if (se != hipSuccess) return ISKV_EDEVICE;
  LayerSel sel;
  fill_sel(sel, std::vector<int>{layer}, 0);
  if (for_factors(c, s, [&](int x, hipStream_t st) {
        return launch_sync(c->M, sel, n_max, x, st, tab);
      }) != hipSuccess)
    return ISKV_EDEVICE;
  for (int b = 0; b < c->D.batch; ++b)
    if ((tab.mask >> b) & 1ull) L.seq[(size_t)b].pending = false;
  L.syncs += 1;
  return maint_done(c, layer) != hipSuccess ? ISKV_EDEVICE : ISKV_OK;
}

}  // namespace

extern "C" {

size_t iskv_workspace_bytes(const iskv_config *cfg) {
  if (!valid_config(cfg)) return 0;
  return global_layout(make_dims(cfg)).total;
}

size_t iskv_state_bytes(const iskv_config *cfg) {
  if (!valid_config(cfg)) return 0;
  const Dims D = make_dims(cfg);
  size_t per_u = 0;
  for (int x = 0; x < 2; ++x) {
    const size_t r = x ? D.rv : D.rk;
    per_u += (size_t)D.d * r + r + (size_t)D.max_tokens * r + (size_t)D.slots * D.d +
             (size_t)D.prefix * D.d;
  }
  return 16 + (size_t)D.units * per_u * 4;
}

int iskv_init(const iskv_config *cfg, void *dev_ws, size_t ws_bytes, void *hip_stream,
              iskv_ctx **out) {
  if (!out) return ISKV_EINVAL;
  *out = nullptr;
  if (!valid_config(cfg) || !dev_ws) return ISKV_EINVAL;
  if (((uintptr_t)dev_ws) % 256) return ISKV_EINVAL;
  iskv_ctx *c = new (std::nothrow) iskv_ctx();
  if (!c) return ISKV_ENOMEM;
  c->cfg = *cfg;
  c->D = make_dims(cfg);
  c->G = global_layout(c->D);
  if (ws_bytes < c->G.total) {
    delete c;
    return ISKV_ENOMEM;
  }
  c->stream = reinterpret_cast<hipStream_t>(hip_stream);
  if (hipGetDevice(&c->device) != hipSuccess ||
      hipDeviceGetAttribute(&c->D.cus, hipDeviceAttributeMultiprocessorCount, c->device) != hipSuccess ||
      c->D.cus < 1) {
    delete c;
    return ISKV_EDEVICE;
  }
  LayerState empty;
  empty.n_c = c->D.prefix;                  // compression starts after the protected prefix
  c->layers.assign(c->D.layers, empty);
  if (c->D.rk != c->D.rv &&
      (hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking) != hipSuccess ||
       hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
       hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess)) {
    if (c->aux) (void)hipStreamDestroy(c->aux);
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    delete c;
    return ISKV_EDEVICE;
  }
  uint8_t *base = reinterpret_cast<uint8_t *>(dev_ws);
  Model &M = c->M;
  M.base = base;
  M.layers_base = c->G.layers_base;
  M.layer_stride = c->G.layer.bytes;
  M.lay = c->G.layer;
  M.D = c->D;
  M.gen_mask = 0;
  M.out_flip = 0;
  M.sh.rec = reinterpret_cast<float *>(base + c->G.rec);
  M.sh.recml = reinterpret_cast<float *>(base + c->G.recml);
  M.sh.cnt = reinterpret_cast<unsigned *>(base + c->G.cnt);
  M.sh.flags = reinterpret_cast<int *>(base + c->G.flags);
  M.sh.rope_anchor = reinterpret_cast<const float *>(base + c->G.rope_anchor);
  M.sh.rope_step = reinterpret_cast<const float *>(base + c->G.rope_step);

  // RoPE tables: theta_i = base^(-2i/d), angles in double, stored as float.
  const int na = c->D.rope_anchors;
  std::vector<float> anchor((size_t)na * 64 * 2), step((size_t)kRopeAnchor * 64 * 2);
  for (int i = 0; i < 64; ++i) {
    const double th = std::pow((double)cfg->rope_base, -2.0 * i / (double)cfg->head_dim);
    for (int a = 0; a < na; ++a) {
      const double ang = (double)a * kRopeAnchor * th;
      anchor[((size_t)a * 64 + i) * 2] = (float)std::cos(ang);
      anchor[((size_t)a * 64 + i) * 2 + 1] = (float)std::sin(ang);
    }
    for (int o = 0; o < kRopeAnchor; ++o) {
      const double ang = (double)o * th;
      step[((size_t)o * 64 + i) * 2] = (float)std::cos(ang);
      step[((size_t)o * 64 + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  // the allocation-free decode's split records (one lookup per device)
  hipError_t e = scratch_setup(c->device);
  if (c->D.cow) {
    c->ev_cow.assign(c->D.layers, nullptr);
    for (hipEvent_t &ev : c->ev_cow)
      if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipMemsetAsync(dev_ws, 0, c->G.total, c->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + c->G.rope_anchor, anchor.data(), anchor.size() * 4,
                       hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + c->G.rope_step, step.data(), step.size() * 4,
                       hipMemcpyHostToDevice, c->stream);
  for (int l = 0; l < c->D.layers && e == hipSuccess; ++l) e = launch_reset_layer(M, l, c->stream);
  std::vector<int> all(c->D.layers);
  for (int l = 0; l < c->D.layers; ++l) all[l] = l;
  for (size_t from = 0; from < all.size() && e == hipSuccess; from += kMaxLayerSel) {
    LayerSel sel;
    fill_sel(sel, all, from);
    e = launch_prep_frag(M, sel, c->stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    if (c->aux) (void)hipStreamDestroy(c->aux);
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    if (c->ev_join) (void)hipEventDestroy(c->ev_join);
    for (hipEvent_t ev : c->ev_cow)
      if (ev) (void)hipEventDestroy(ev);
    delete c;
    return ISKV_EDEVICE;
  }
  *out = c;
  return ISKV_OK;
}

int iskv_append(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int n_tokens,
                int in_dtype, int *blocks_ready) {
  if (!c || check_layer(c, layer) || !dev_k || !dev_v || n_tokens < 0) return ISKV_EINVAL;
  if (in_dtype != ISKV_F32 && in_dtype != ISKV_BF16) return ISKV_EINVAL;
  LayerState &L = c->layers[layer];
  if (!make_uniform(L)) return ISKV_ESTATE;
  if (c->D.cow) {
    // decode boundary; an append that would overflow the ring waits for the switch
    int r = cow_switch(c, layer, false);
    if (r >= 0 && L.length + n_tokens - L.n_c > c->D.slots) r = cow_switch(c, layer, true);
    if (r < 0) return r;
  }
  // ring tokens after the append: the positions from n_c on (>= P)
  if (L.length + n_tokens - L.n_c > c->D.slots) return ISKV_ESTATE;
  if (L.length + n_tokens > c->D.max_tokens) return ISKV_ESTATE;
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  hipError_t e = launch_append(c->M, layer, dev_k, dev_v, n_tokens, in_dtype, L.length, c->stream);
  if (e != hipSuccess) return ISKV_EDEVICE;
  L.length += n_tokens;
  if (blocks_ready) *blocks_ready = block_ready(c, L) ? 1 : 0;
  return ISKV_OK;
}

int iskv_block_update(iskv_ctx *c, int layer) {
  if (!c) return ISKV_EINVAL;
  if (c->D.cow) return ISKV_ESTATE;           // iskv_maintain
  std::vector<int> idx;
  if (layer >= 0) {
    if (check_layer(c, layer)) return ISKV_EINVAL;
    LayerState &L = c->layers[layer];
    if (!make_uniform(L)) return fold_ragged(c, layer, true);
    if (L.pending || L.length - L.n_c != c->D.slots) return ISKV_ESTATE;
    idx.push_back(layer);
  } else if (layer == -1) {
    for (int l = 0; l < c->D.layers; ++l) {
      LayerState &L = c->layers[l];
      if (!make_uniform(L)) {
        const int r = fold_ragged(c, l, false);
        if (r != ISKV_OK) return r;
        continue;
      }
      if (!L.pending && L.length - L.n_c == c->D.slots) idx.push_back(l);
    }
  } else {
    return ISKV_EINVAL;
  }
  if (idx.empty()) return ISKV_OK;
  hipError_t se;
  hipStream_t s = maint_stream(c, &se);
  if (se != hipSuccess) return ISKV_EDEVICE;
  // group layers by their compressed count (one launch per distinct n_c)
  std::vector<bool> done(idx.size(), false);
  for (size_t i = 0; i < idx.size(); ++i) {
    if (done[i]) continue;
    const int64_t n_c = c->layers[idx[i]].n_c;
    std::vector<int> grp;
    for (size_t j = i; j < idx.size(); ++j)
      if (!done[j] && c->layers[idx[j]].n_c == n_c) { grp.push_back(idx[j]); done[j] = true; }
    for (size_t from = 0; from < grp.size(); from += kMaxLayerSel) {
      LayerSel sel;
      fill_sel(sel, grp, from);
      hipError_t e = for_factors(c, s, [&](int x, hipStream_t st) {
        return launch_block_update(c->M, sel, n_c, x, st);
      });
      if (e == hipSuccess) e = launch_prep_frag(c->M, sel, s);
      if (e != hipSuccess) return ISKV_EDEVICE;
    }
    for (int l : grp) {
      c->layers[l].n_c += kBlock;
      c->layers[l].pending = true;
      c->layers[l].folds += 1;
      if (maint_done(c, l) != hipSuccess) return ISKV_EDEVICE;
    }
  }
  return ISKV_OK;
}

int iskv_sync(iskv_ctx *c, int layer) {
  if (!c) return ISKV_EINVAL;
  if (c->D.cow) return ISKV_ESTATE;
  std::vector<int> idx;
  if (layer >= 0) {
    if (check_layer(c, layer)) return ISKV_EINVAL;
    if (!make_uniform(c->layers[layer])) return sync_ragged(c, layer, true);
    if (!c->layers[layer].pending) return ISKV_ESTATE;
    idx.push_back(layer);
  } else if (layer == -1) {
    for (int l = 0; l < c->D.layers; ++l) {
      if (!make_uniform(c->layers[l])) {
        const int r = sync_ragged(c, l, false);
        if (r != ISKV_OK) return r;
        continue;
      }
      if (c->layers[l].pending) idx.push_back(l);
    }
  } else {
    return ISKV_EINVAL;
  }
  if (idx.empty()) return ISKV_OK;
  hipError_t se;
  hipStream_t s = maint_stream(c, &se);
  if (se != hipSuccess) return ISKV_EDEVICE;
  std::vector<bool> done(idx.size(), false);
  for (size_t i = 0; i < idx.size(); ++i) {
    if (done[i]) continue;
    const int64_t n_c = c->layers[idx[i]].n_c;
    std::vector<int> grp;
    for (size_t j = i; j < idx.size(); ++j)
      if (!done[j] && c->layers[idx[j]].n_c == n_c) { grp.push_back(idx[j]); done[j] = true; }
    for (size_t from = 0; from < grp.size(); from += kMaxLayerSel) {
      LayerSel sel;
      fill_sel(sel, grp, from);
      if (for_factors(c, s, [&](int x, hipStream_t st) {
            return launch_sync(c->M, sel, n_c - kBlock, x, st);
          }) != hipSuccess)
        return ISKV_EDEVICE;
    }
    for (int l : grp) {
      c->layers[l].pending = false;
      c->layers[l].syncs += 1;
      if (maint_done(c, l) != hipSuccess) return ISKV_EDEVICE;
    }
  }
  return ISKV_OK;
}

int iskv_discard_sync(iskv_ctx *c, int layer) {
  if (!c) return ISKV_EINVAL;
  if (c->D.cow) return ISKV_ESTATE;
  if (layer >= 0) {
    if (check_layer(c, layer)) return ISKV_EINVAL;
    LayerState &L = c->layers[layer];
    if (L.ragged) {
      bool any = false;
      for (SeqState &q : L.seq) { any |= q.pending; q.pending = false; }
      make_uniform(L);
      return any ? ISKV_OK : ISKV_ESTATE;
    }
    if (!L.pending) return ISKV_ESTATE;
    L.pending = false;
    return ISKV_OK;
  }
  if (layer != -1) return ISKV_EINVAL;
  for (LayerState &L : c->layers) {
    L.pending = false;
    for (SeqState &q : L.seq) q.pending = false;
    make_uniform(L);
  }
  return ISKV_OK;
}

int iskv_decode_attn(iskv_ctx *c, int layer, const float *dev_q, int64_t q_pos, float *dev_out) {
  if (!c || check_layer(c, layer) || !dev_q || !dev_out) return ISKV_EINVAL;
  if (q_pos < 0 || q_pos >= (int64_t)c->D.rope_anchors * kRopeAnchor) return ISKV_EINVAL;
  LayerState &L = c->layers[layer];
  if (!make_uniform(L)) return ISKV_ESTATE;
  if (L.length <= 0) return ISKV_ESTATE;
  const int r = cow_switch(c, layer, false);   // decode boundary
  if (r < 0) return r;
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  return hip_err(launch_decode(c->M, layer, dev_q, q_pos, dev_out, L.length, L.n_c, c->stream));
}

int iskv_decode_attn_noalloc(iskv_ctx *c, int layer, const float *dev_q, int64_t q_pos,
                             float *dev_out) {
  if (!c || check_layer(c, layer) || !dev_q || !dev_out) return ISKV_EINVAL;
  if (q_pos < 0 || q_pos >= (int64_t)c->D.rope_anchors * kRopeAnchor) return ISKV_EINVAL;
  const RecLayout R = rec_layout(c->D);
  if (R.bytes > kScratchBytes) return ISKV_ESCRATCH;
  LayerState &L = c->layers[layer];
  if (!make_uniform(L)) return ISKV_ESTATE;
  if (L.length <= 0) return ISKV_ESTATE;
  uint8_t *base = reinterpret_cast<uint8_t *>(scratch_address(c->device));
  if (!base) return ISKV_EDEVICE;
  const int r = cow_switch(c, layer, false);   // decode boundary
  if (r < 0) return r;
  Model M = c->M;
  M.sh.rec = reinterpret_cast<float *>(base + R.rec);
  M.sh.recml = reinterpret_cast<float *>(base + R.recml);
  M.sh.cnt = reinterpret_cast<unsigned *>(base + R.cnt);
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  return hip_err(launch_decode(M, layer, dev_q, q_pos, dev_out, L.length, L.n_c, c->stream));
}

size_t iskv_noalloc_scratch_bytes(const iskv_config *cfg) {
  if (!valid_config(cfg)) return 0;
  return rec_layout(make_dims(cfg)).bytes;
}

int iskv_append_decode(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int in_dtype,
                       const float *dev_q, int64_t q_pos, float *dev_out, int *blocks_ready) {
  if (!c || check_layer(c, layer) || !dev_k || !dev_v || !dev_q || !dev_out) return ISKV_EINVAL;
  if (in_dtype != ISKV_F32 && in_dtype != ISKV_BF16) return ISKV_EINVAL;
  if (q_pos < 0 || q_pos >= (int64_t)c->D.rope_anchors * kRopeAnchor) return ISKV_EINVAL;
  LayerState &L = c->layers[layer];
  if (!make_uniform(L)) return ISKV_ESTATE;
  if (c->D.cow) {
    int r = cow_switch(c, layer, false);        // decode boundary
    if (r >= 0 && L.length - L.n_c + 1 > c->D.slots) r = cow_switch(c, layer, true);
    if (r < 0) return r;
  }
  if (L.length - L.n_c + 1 > c->D.slots) return ISKV_ESTATE;
  if (L.length + 1 > c->D.max_tokens) return ISKV_ESTATE;
  if (L.length < c->D.prefix) {
    // the token lands in the protected prefix: the two calls, not fused
    const int a = iskv_append(c, layer, dev_k, dev_v, 1, in_dtype, blocks_ready);
    return a != ISKV_OK ? a : iskv_decode_attn(c, layer, dev_q, q_pos, dev_out);
  }
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  const FusedAppend app{dev_k, dev_v, in_dtype};
  hipError_t e = launch_decode(c->M, layer, dev_q, q_pos, dev_out, L.length + 1, L.n_c, c->stream, app);
  if (e != hipSuccess) return ISKV_EDEVICE;
  L.length += 1;
  if (blocks_ready) *blocks_ready = block_ready(c, L) ? 1 : 0;
  return ISKV_OK;
}

namespace {
int fill_status(iskv_ctx *c, int layer, const SeqState &q, iskv_status_t *st) {
  if (join_all(c) != hipSuccess) return ISKV_EDEVICE;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return ISKV_EDEVICE;
  int flags = 0;
  if (hipMemcpy(&flags, c->M.sh.flags, 4, hipMemcpyDeviceToHost) != hipSuccess) return ISKV_EDEVICE;
  const LayerState &L = c->layers[layer];
  std::memset(st, 0, sizeof(*st));
  st->length = q.length;
  st->compressed = q.n_c - c->D.prefix;
  st->blocks_ready = L.ragged ? ((q.length - q.n_c == c->D.slots) ? 1 : 0) : (block_ready(c, L) ? 1 : 0);
  st->pending_sync = (q.pending || L.inflight) ? 1 : 0;
  st->folds = L.folds;
  st->syncs = L.syncs;
  st->persistent_bytes = persistent_bytes(c);
  uint64_t full = 0;
  for (const LayerState &S : c->layers)
    for (int b = 0; b < c->D.batch; ++b)
      full += 2ull * (uint64_t)seq_state(S, b).length * c->D.kv_heads * c->D.d * c->D.elem;
  st->full_bytes = full;
  st->numeric_flags = flags;
  return flags ? ISKV_ENUMERIC : ISKV_OK;
}
}  // namespace

int iskv_status(iskv_ctx *c, int layer, iskv_status_t *st) {
  if (!c || !st || check_layer(c, layer)) return ISKV_EINVAL;
  LayerState &L = c->layers[layer];
  if (!make_uniform(L)) return ISKV_ESTATE;
  return fill_status(c, layer, seq_state(L, 0), st);
}

int iskv_seq_status(iskv_ctx *c, int layer, int seq, iskv_status_t *st) {
  if (!c || !st || check_layer(c, layer) || seq < 0 || seq >= c->D.batch) return ISKV_EINVAL;
  return fill_status(c, layer, seq_state(c->layers[layer], seq), st);
}

int iskv_append_ragged(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int n_tokens,
                       int in_dtype, const int32_t *counts, int *seqs_ready) {
  if (!c || check_layer(c, layer) || !dev_k || !dev_v || !counts || n_tokens < 0) return ISKV_EINVAL;
  if (in_dtype != ISKV_F32 && in_dtype != ISKV_BF16) return ISKV_EINVAL;
  if (c->D.batch > kMaxSeqTab) return ISKV_EINVAL;
  if (c->D.cow) return ISKV_ESTATE;
  LayerState &L = c->layers[layer];
  for (int b = 0; b < c->D.batch; ++b) {
    if (counts[b] < 0 || counts[b] > n_tokens) return ISKV_EINVAL;
    const SeqState q = seq_state(L, b);
    if (q.length + counts[b] - q.n_c > c->D.slots) return ISKV_ESTATE;
    if (q.length + counts[b] > c->D.max_tokens) return ISKV_ESTATE;
  }
  make_ragged(c, L);
  SeqTab tab{};
  tab.n = c->D.batch;
  for (int b = 0; b < c->D.batch; ++b) {
    tab.len[b] = (int32_t)L.seq[(size_t)b].length;
    tab.aux[b] = counts[b];
    if (counts[b] > 0) tab.mask |= 1ull << b;
  }
  if (tab.mask) {
    if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
    if (launch_append(c->M, layer, dev_k, dev_v, n_tokens, in_dtype, 0, c->stream, tab) != hipSuccess)
      return ISKV_EDEVICE;
  }
  int ready = 0;
  for (int b = 0; b < c->D.batch; ++b) {
    SeqState &q = L.seq[(size_t)b];
    q.length += counts[b];
    ready += (q.length - q.n_c == c->D.slots) ? 1 : 0;
  }
  if (seqs_ready) *seqs_ready = ready;
  return ISKV_OK;
}

int iskv_decode_attn_ragged(iskv_ctx *c, int layer, const float *dev_q, const int64_t *q_pos,
                            float *dev_out) {
  if (!c || check_layer(c, layer) || !dev_q || !q_pos || !dev_out) return ISKV_EINVAL;
  if (c->D.batch > kMaxSeqTab) return ISKV_EINVAL;
  if (c->D.cow) return ISKV_ESTATE;
  const LayerState &L = c->layers[layer];
  SeqTab tab{};
  tab.n = c->D.batch;
  tab.mask = seq_bits(c->D.batch);
  for (int b = 0; b < c->D.batch; ++b) {
    if (q_pos[b] < 0 || q_pos[b] >= (int64_t)c->D.rope_anchors * kRopeAnchor) return ISKV_EINVAL;
    const SeqState q = seq_state(L, b);
    if (q.length <= 0) return ISKV_ESTATE;
    tab.len[b] = (int32_t)q.length;
    tab.nc[b] = (int32_t)q.n_c;
    tab.aux[b] = (int32_t)q_pos[b];
  }
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  return hip_err(launch_decode_ragged(c->M, layer, dev_q, dev_out, tab, c->stream));
}

int iskv_export_state(iskv_ctx *c, int layer, void *host_buf, size_t bytes) {
  if (!c || check_layer(c, layer) || !host_buf) return ISKV_EINVAL;
  if (!make_uniform(c->layers[layer])) return ISKV_ESTATE;
  if (bytes < iskv_state_bytes(&c->cfg)) return ISKV_EINVAL;
  const int sw = cow_switch(c, layer, true);   // a maintenance in flight is joined first
  if (sw < 0) return sw;
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return ISKV_EDEVICE;
  const Dims &D = c->D;
  const LayerLayout &Ly = c->G.layer;
  const GenLayout &Gn = Ly.gen[layer_gen(c->M, layer)];
  const size_t lb = Ly.bytes;
  std::vector<uint8_t> raw(lb);
  const uint8_t *src = c->M.base + c->G.layers_base + (size_t)layer * lb;
  if (hipMemcpy(raw.data(), src, lb, hipMemcpyDeviceToHost) != hipSuccess) return ISKV_EDEVICE;
  auto elem = [&](size_t off, size_t i) -> float {
    if (D.storage == ISKV_BF16) {
      uint16_t h;
      std::memcpy(&h, raw.data() + off + i * 2, 2);
      return host_from_bf16(h);
    }
    float f;
    std::memcpy(&f, raw.data() + off + i * 4, 4);
    return f;
  };
  uint8_t *o = reinterpret_cast<uint8_t *>(host_buf);
  const LayerState &L = c->layers[layer];
  const int64_t n_comp = L.n_c - D.prefix;
  std::memcpy(o, &L.length, 8);
  std::memcpy(o + 8, &n_comp, 8);
  float *f = reinterpret_cast<float *>(o + 16);
  for (int u = 0; u < D.units; ++u) {
    const int cu = coef_unit(D, u);          // joint: every head lists its sequence's S and rows
    for (int x = 0; x < 2; ++x) {
      const size_t r = x ? D.rv : D.rk;
      std::memcpy(f, raw.data() + Gn.basis[x] + (size_t)u * D.d * r * 4, (size_t)D.d * r * 4);
      f += (size_t)D.d * r;
      std::memcpy(f, raw.data() + Gn.sing[x] + (size_t)cu * r * 4, r * 4);
      f += r;
      const size_t coff = Gn.coef[x] + (size_t)cu * D.max_tokens * r * D.elem;
      for (size_t i = 0; i < (size_t)D.max_tokens * r; ++i)
        f[i] = (i >= (size_t)D.prefix * r && i < (size_t)L.n_c * r) ? elem(coff, i) : 0.f;
      f += (size_t)D.max_tokens * r;
      for (int s = 0; s < D.slots; ++s)
        for (int d = 0; d < D.d; ++d) {
          const size_t i = (x == 0)
              ? (size_t)u * D.slots * D.d + (size_t)s * D.d + d
              : (size_t)u * D.slots * D.d + (size_t)d * D.slots + s;
          f[(size_t)s * D.d + d] = elem(x == 0 ? Ly.ringk : Ly.ringv, i);
        }
      f += (size_t)D.slots * D.d;
      for (int p = 0; p < D.prefix; ++p)
        for (int d = 0; d < D.d; ++d) {
          const size_t i = (x == 0)
              ? (size_t)u * D.prefix * D.d + (size_t)p * D.d + d
              : (size_t)u * D.prefix * D.d + (size_t)d * D.prefix + p;
          f[(size_t)p * D.d + d] = elem(x == 0 ? Ly.prek : Ly.prev, i);
        }
      f += (size_t)D.prefix * D.d;
    }
  }
  return ISKV_OK;
}

int iskv_import_state(iskv_ctx *c, int layer, const void *host_buf, size_t bytes) {
  if (!c || check_layer(c, layer) || !host_buf) return ISKV_EINVAL;
  if (bytes < iskv_state_bytes(&c->cfg)) return ISKV_EINVAL;
  const Dims &D = c->D;
  const uint8_t *in = reinterpret_cast<const uint8_t *>(host_buf);
  int64_t length, n_comp;
  std::memcpy(&length, in, 8);
  std::memcpy(&n_comp, in + 8, 8);
  const int64_t n_c = D.prefix + n_comp;    // end position of the compressed rows
  if (length < 0 || n_comp < 0 || n_comp % kBlock || length > D.max_tokens ||
      (n_comp > 0 && n_c > length) || length - n_c > D.slots)
    return ISKV_EINVAL;
  const int sw = cow_switch(c, layer, true);   // a maintenance in flight is joined first
  if (sw < 0) return sw;
  if (join_layer(c, layer) != hipSuccess) return ISKV_EDEVICE;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return ISKV_EDEVICE;
  const LayerLayout &Ly = c->G.layer;
  const GenLayout &Gn = Ly.gen[layer_gen(c->M, layer)];
  const size_t lb = Ly.bytes;
  std::vector<uint8_t> raw(lb, 0);
  auto put = [&](size_t off, size_t i, float v) {
    if (D.storage == ISKV_BF16) {
      const uint16_t h = host_bf16(v);
      std::memcpy(raw.data() + off + i * 2, &h, 2);
    } else {
      std::memcpy(raw.data() + off + i * 4, &v, 4);
    }
  };
  const float *f = reinterpret_cast<const float *>(in + 16);
  for (int u = 0; u < D.units; ++u) {
    // joint: S and the coefficient rows of a sequence come from its head 0
    const int cu = coef_unit(D, u);
    const bool owner = !D.joint || u % D.kv_heads == 0;
    for (int x = 0; x < 2; ++x) {
      const size_t r = x ? D.rv : D.rk;
      std::memcpy(raw.data() + Gn.basis[x] + (size_t)u * D.d * r * 4, f, (size_t)D.d * r * 4);
      f += (size_t)D.d * r;
      if (owner) std::memcpy(raw.data() + Gn.sing[x] + (size_t)cu * r * 4, f, r * 4);
      f += r;
      const size_t coff = Gn.coef[x] + (size_t)cu * D.max_tokens * r * D.elem;
      if (owner)
        for (size_t i = (size_t)D.prefix * r; i < (size_t)n_c * r; ++i) put(coff, i, f[i]);
      f += (size_t)D.max_tokens * r;
      for (int s = 0; s < D.slots; ++s)
        for (int d = 0; d < D.d; ++d) {
          const size_t i = (x == 0)
              ? (size_t)u * D.slots * D.d + (size_t)s * D.d + d
              : (size_t)u * D.slots * D.d + (size_t)d * D.slots + s;
          put(x == 0 ? Ly.ringk : Ly.ringv, i, f[(size_t)s * D.d + d]);
        }
      f += (size_t)D.slots * D.d;
      for (int p = 0; p < D.prefix; ++p)
        for (int d = 0; d < D.d; ++d) {
          const size_t i = (x == 0)
              ? (size_t)u * D.prefix * D.d + (size_t)p * D.d + d
              : (size_t)u * D.prefix * D.d + (size_t)d * D.prefix + p;
          put(x == 0 ? Ly.prek : Ly.prev, i, f[(size_t)p * D.d + d]);
        }
      f += (size_t)D.prefix * D.d;
    }
  }
  uint8_t *dst = c->M.base + c->G.layers_base + (size_t)layer * lb;
  if (hipMemcpy(dst, raw.data(), lb, hipMemcpyHostToDevice) != hipSuccess) return ISKV_EDEVICE;
  LayerSel sel;
  sel.n = 1;
  sel.idx[0] = layer;
  if (launch_prep_frag(c->M, sel, c->stream) != hipSuccess) return ISKV_EDEVICE;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return ISKV_EDEVICE;
  LayerState &L = c->layers[layer];
  L.length = length;
  L.n_c = n_c;
  L.pending = false;
  L.ragged = false;
  L.seq.clear();
  return ISKV_OK;
}

int iskv_set_maintenance_stream(iskv_ctx *c, void *hip_stream) {
  if (!c) return ISKV_EINVAL;
  hipStream_t ms = reinterpret_cast<hipStream_t>(hip_stream);
  if (ms == c->stream) ms = nullptr;
  // pending maintenance of the old stream is joined into the main stream first
  if (join_all(c) != hipSuccess) return ISKV_EDEVICE;
  if (ms && !c->ev_main) {
    if (hipEventCreateWithFlags(&c->ev_main, hipEventDisableTiming) != hipSuccess) return ISKV_EDEVICE;
    c->ev_done.assign(c->D.layers, nullptr);
    for (hipEvent_t &e : c->ev_done)
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return ISKV_EDEVICE;
    c->maint_pending.assign(c->D.layers, 0);
  }
  c->mstream = ms;
  return ISKV_OK;
}

int iskv_join_maintenance(iskv_ctx *c, int layer) {
  if (!c) return ISKV_EINVAL;
  if (c->D.cow) {
    if (layer != -1 && check_layer(c, layer)) return ISKV_EINVAL;
    for (int l = (layer == -1 ? 0 : layer); l < (layer == -1 ? c->D.layers : layer + 1); ++l) {
      const int r = cow_switch(c, l, true);
      if (r < 0) return r;
    }
    return ISKV_OK;
  }
  if (layer == -1) return hip_err(join_all(c));
  if (check_layer(c, layer)) return ISKV_EINVAL;
  return hip_err(join_layer(c, layer));
}

int iskv_maintain(iskv_ctx *c, int layer) {
  if (!c) return ISKV_EINVAL;
  if (!c->D.cow) return ISKV_ESTATE;
  std::vector<int> idx;
  if (layer >= 0) {
    if (check_layer(c, layer)) return ISKV_EINVAL;
    if (!block_ready(c, c->layers[layer])) return ISKV_ESTATE;
    idx.push_back(layer);
  } else if (layer == -1) {
    for (int l = 0; l < c->D.layers; ++l)
      if (block_ready(c, c->layers[l])) idx.push_back(l);
  } else {
    return ISKV_EINVAL;
  }
  if (idx.empty()) return ISKV_OK;
  hipError_t se;
  hipStream_t s = maint_stream(c, &se);     // after the init stream's work so far
  if (se != hipSuccess) return ISKV_EDEVICE;
  Model Mo = c->M;
  Mo.out_flip = 1;                           // read the current generation, write the other
  std::vector<bool> done(idx.size(), false);
  for (size_t i = 0; i < idx.size(); ++i) {
    if (done[i]) continue;
    const int64_t n_c = c->layers[idx[i]].n_c;
    std::vector<int> grp;
    for (size_t j = i; j < idx.size(); ++j)
      if (!done[j] && c->layers[idx[j]].n_c == n_c) { grp.push_back(idx[j]); done[j] = true; }
    for (size_t from = 0; from < grp.size(); from += kMaxLayerSel) {
      LayerSel sel;
      fill_sel(sel, grp, from);
      hipError_t e = for_factors(c, s, [&](int x, hipStream_t st) {
        return launch_block_update(Mo, sel, n_c, x, st);
      });
      if (e == hipSuccess)
        e = for_factors(c, s, [&](int x, hipStream_t st) { return launch_sync(Mo, sel, n_c, x, st); });
      if (e == hipSuccess) e = launch_prep_frag(Mo, sel, s);
      if (e != hipSuccess) return ISKV_EDEVICE;
    }
    for (int l : grp) {
      LayerState &L = c->layers[l];
      L.inflight = true;
      L.folds += 1;
      L.syncs += 1;
      if (hipEventRecord(c->ev_cow[l], s) != hipSuccess) return ISKV_EDEVICE;
    }
  }
  return ISKV_OK;
}

int iskv_prefill_layers(iskv_ctx *c, int n_layers, const int *layers, const void *const *dev_k,
                        const void *const *dev_v, int n_tokens, int in_dtype) {
  if (!c || n_layers < 1 || !layers || !dev_k || !dev_v || n_tokens < 0) return ISKV_EINVAL;
  if (in_dtype != ISKV_F32 && in_dtype != ISKV_BF16) return ISKV_EINVAL;
  if (c->D.cow || c->D.joint) return ISKV_ESTATE;
  const Dims &D = c->D;
  for (int i = 0; i < n_layers; ++i) {
    if (check_layer(c, layers[i]) || !dev_k[i] || !dev_v[i]) return ISKV_EINVAL;
    for (int j = 0; j < i; ++j)
      if (layers[j] == layers[i]) return ISKV_EINVAL;
    LayerState &L = c->layers[layers[i]];
    if (!make_uniform(L)) return ISKV_ESTATE;
    if (L.pending || L.length != L.n_c || L.length < D.prefix) return ISKV_ESTATE;
    if (L.length + n_tokens > D.max_tokens) return ISKV_ESTATE;
    const LayerState &L0 = c->layers[layers[0]];
    if (L.length != L0.length || L.n_c != L0.n_c) return ISKV_ESTATE;
  }
  const LayerState &L0 = c->layers[layers[0]];
  const int64_t length0 = L0.length, n_c_start = L0.n_c;
  // blocks that leave the window: the same count block-by-block appends would fold
  const int m = n_tokens >= D.window + kBlock ? (n_tokens - D.window) / kBlock : 0;
  for (int i = 0; i < n_layers; ++i)
    if (join_layer(c, layers[i]) != hipSuccess) return ISKV_EDEVICE;
  hipStream_t s = c->stream;
  float *mbulk = reinterpret_cast<float *>(c->M.base + c->G.bulk);
  const size_t row_bytes = (size_t)D.kv_heads * D.d * (in_dtype == ISKV_BF16 ? 2 : 4);
  const int tail = n_tokens - m * kBlock;
  int passes = 0;
  for (int first = 0; first < n_layers; first += kMaxBulkLayers) {
    BulkIn in{};
    in.n = std::min(kMaxBulkLayers, n_layers - first);
    for (int i = 0; i < in.n; ++i) {
      in.layer[i] = layers[first + i];
      in.k[i] = dev_k[first + i];
      in.v[i] = dev_v[first + i];
    }
    // M slots: one layer's worth of the workspace shared by the launch's layers
    const int per_pass = std::max(1, D.bulk_blocks / in.n);
    passes = 0;
    for (int done = 0; done < m; done += per_pass, ++passes) {
      const int nb = std::min(per_pass, m - done);
      const int64_t n_c0 = n_c_start + (int64_t)done * kBlock;
      hipError_t e = for_factors(c, s, [&](int x, hipStream_t st) {
        hipError_t r = launch_bulk_fold(c->M, in, n_c0, nb, x, in_dtype, (int64_t)done * kBlock, n_tokens,
                                        mbulk, per_pass, st);
        if (r == hipSuccess) r = launch_sync_bulk(c->M, in, n_c0, nb, x, mbulk, per_pass, st);
        return r;
      });
      if (e != hipSuccess) return ISKV_EDEVICE;
    }
    // the rows that stay exact go to the ring
    for (int i = 0; i < in.n; ++i) {
      const uint8_t *kt = reinterpret_cast<const uint8_t *>(in.k[i]) + (size_t)m * kBlock * row_bytes;
      const uint8_t *vt = reinterpret_cast<const uint8_t *>(in.v[i]) + (size_t)m * kBlock * row_bytes;
      if (launch_append(c->M, in.layer[i], kt, vt, tail, in_dtype, length0 + (int64_t)m * kBlock, s,
                        SeqTab{}, n_tokens) != hipSuccess)
        return ISKV_EDEVICE;
    }
    if (m > 0) {
      LayerSel sel;
      sel.n = in.n;
      for (int i = 0; i < in.n; ++i) sel.idx[i] = in.layer[i];
      if (launch_prep_frag(c->M, sel, s) != hipSuccess) return ISKV_EDEVICE;
    }
    for (int i = 0; i < in.n; ++i) {
      LayerState &L = c->layers[in.layer[i]];
      L.length += n_tokens;
      L.n_c += (int64_t)m * kBlock;
      L.folds += m;
      L.syncs += passes;
    }
  }
  return ISKV_OK;
}

int iskv_prefill(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int n_tokens,
                 int in_dtype) {
  return iskv_prefill_layers(c, 1, &layer, &dev_k, &dev_v, n_tokens, in_dtype);
}

int iskv_switch(iskv_ctx *c, int layer, int wait) {
  if (!c || check_layer(c, layer)) return ISKV_EINVAL;
  if (!c->D.cow) return ISKV_ESTATE;
  return cow_switch(c, layer, wait != 0);
}

int iskv_destroy(iskv_ctx *c) {
  if (!c) return ISKV_EINVAL;
  hipError_t e = join_all(c);
  for (int l = 0; l < c->D.layers && e == hipSuccess && c->D.cow; ++l)
    if (cow_switch(c, l, true) < 0) e = hipErrorUnknown;
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  for (hipEvent_t ev : c->ev_cow)
    if (ev) (void)hipEventDestroy(ev);
  if (c->ev_main) (void)hipEventDestroy(c->ev_main);
  if (c->aux) (void)hipStreamDestroy(c->aux);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  for (hipEvent_t ev : c->ev_done)
    if (ev) (void)hipEventDestroy(ev);
  delete c;
  return hip_err(e);
}

const char *iskv_strerror(int code) {
  switch (code) {
    case ISKV_OK: return "ok";
    case ISKV_EINVAL: return "invalid argument or unsupported configuration";
    case ISKV_ESTATE: return "operation not allowed in the current cache state";
    case ISKV_ENOMEM: return "workspace too small";
    case ISKV_EDEVICE: return "HIP runtime error";
    case ISKV_ENUMERIC: return "device numeric flag raised";
    case ISKV_ESCRATCH:
      return "configuration needs more split-record memory than the allocation-free decode's "
             "static array holds (see iskv_noalloc_scratch_bytes)";
  }
  return "unknown error";
}

}  // extern "C"
