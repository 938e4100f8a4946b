// abi.hip -- the extern "C" entry points of libdlrm_mi355x: argument
// validation, kernel selection and the DLRMv1 forward composition.  Every
// argument error is reported before any work is enqueued; nothing here
// allocates device memory or synchronizes the stream.
#include <limits.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "../../include/dlrm_embedding_bag.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace dlrm;

static_assert(DLRM_MAX_TABLES == kMaxTables, "table limit mismatch");
static_assert(DLRM_F32 == kF32 && DLRM_BF16 == kBF16 && DLRM_FP8_E4M3 == kFP8,
              "dtype codes mismatch");

namespace {

bool valid_act(int act) {
  return act == DLRM_ACT_NONE || act == DLRM_ACT_RELU || act == DLRM_ACT_SIGMOID;
}

int64_t round4(int64_t x) { return (x + 3) & ~int64_t(3); }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Elements per 16-byte row chunk of a table type.
int dtype_chunk(int dtype) { return dtype == kFP8 ? 16 : dtype == kBF16 ? 8 : 4; }

// Validates the bag arguments shared by the gather entry points and packs
// them into the by-value kernel argument.  gc.vec says whether the dim and
// the tables allow the 16-byte chunk path (outputs are checked by the caller).
int pack_bags(const dlrm_bags &g, TableSet &ts, GatherConfig &gc) {
  const int32_t K = g.num_tables, B = g.batch, D = g.dim;
  if (K < 1 || K > DLRM_MAX_TABLES || B < 0 || D < 1 || D > DLRM_MAX_DIM) return DLRM_ERR_SHAPE;
  if (g.table_dtype != DLRM_F32 && g.table_dtype != DLRM_BF16 && g.table_dtype != DLRM_FP8_E4M3)
    return DLRM_ERR_SHAPE;
  if (g.pool != DLRM_POOL_SUM && g.pool != DLRM_POOL_MEAN) return DLRM_ERR_SHAPE;
  if (!g.tables || !g.rows || !g.indices || !g.n_idx) return DLRM_ERR_NULL;
  if (g.weights && g.pool != DLRM_POOL_SUM) return DLRM_ERR_UNSUPPORTED;
  memset(&ts, 0, sizeof(ts));
  gc.dtype = g.table_dtype;
  gc.csr = g.offsets != nullptr;
  gc.psw = g.weights != nullptr;
  gc.vec = (D % dtype_chunk(g.table_dtype)) == 0;
  ts.mean = g.pool == DLRM_POOL_MEAN;
  ts.scaled = g.scales != nullptr;
  for (int k = 0; k < K; ++k) {
    if (!g.tables[k]) return DLRM_ERR_NULL;
    if (g.rows[k] < 1 || g.n_idx[k] < 0 || g.n_idx[k] > INT32_MAX) return DLRM_ERR_SHAPE;
    if (g.n_idx[k] > 0 && !g.indices[k]) return DLRM_ERR_NULL;
    if (gc.psw && g.n_idx[k] > 0 && !g.weights[k]) return DLRM_ERR_NULL;
    if (gc.csr) {
      if (!g.offsets[k] && B > 0) return DLRM_ERR_NULL;
    } else if (B > 0 && g.n_idx[k] % B != 0) {
      return DLRM_ERR_SHAPE;
    }
    ts.table[k] = g.tables[k];
    ts.idx[k] = g.indices[k];
    ts.off[k] = gc.csr ? g.offsets[k] : nullptr;
    ts.wt[k] = gc.psw ? g.weights[k] : nullptr;
    ts.bag[k] = (!gc.csr && B > 0) ? (int32_t)(g.n_idx[k] / B) : 0;
    ts.nidx[k] = (int32_t)g.n_idx[k];
    ts.scale[k] = g.scales ? g.scales[k] : 1.0f;
    gc.vec = gc.vec && aligned16(g.tables[k]);
  }
  return DLRM_OK;
}

// The dlrm_bags form of float32 sum lookups.
dlrm_bags f32_sum_bags(int32_t K, int32_t B, int32_t D, const float *const *tables,
                       const int64_t *rows, const int32_t *const *indices,
                       const int32_t *const *offsets, const int64_t *n_idx) {
  dlrm_bags g;
  g.num_tables = K;
  g.batch = B;
  g.dim = D;
  g.table_dtype = DLRM_F32;
  g.pool = DLRM_POOL_SUM;
  g.tables = reinterpret_cast<const void *const *>(tables);
  g.rows = rows;
  g.indices = indices;
  g.offsets = offsets;
  g.n_idx = n_idx;
  g.weights = nullptr;
  g.scales = nullptr;
  return g;
}

int chunk_elems(const GatherConfig &gc) { return gc.vec ? dtype_chunk(gc.dtype) : 1; }

int hip_status(hipError_t e) { return e == hipSuccess ? DLRM_OK : DLRM_ERR_HIP; }

// Packs a validated layer stack into chain parameters; false if the chain
// kernel cannot run it.
bool pack_chain(int32_t m, int32_t n, const dlrm_layer *layers, const float *a, int64_t lda,
                float *c, int64_t ldc, ChainParams &cp) {
  if (n < 1 || n > kMaxChainLayers) return false;
  memset(&cp, 0, sizeof(cp));
  cp.M = m;
  cp.nlayers = n;
  cp.A = a;
  cp.lda = lda;
  cp.C = c;
  cp.ldc = ldc;
  for (int l = 0; l < n; ++l) {
    cp.layer[l].W = layers[l].weight;
    cp.layer[l].bias = layers[l].bias;
    cp.layer[l].K = layers[l].in_features;
    cp.layer[l].N = layers[l].out_features;
    cp.layer[l].act = layers[l].act;
  }
  return chain_supported(cp);
}

// How a forward's MLP layers are launched at one batch size: fused launches,
// and how many k partials each layer stores (1 = its finished output).
struct MlpComposition {
  bool fuse_bottom = false;  // the three-layer bottom MLP as one launch, 32 rows per workgroup
  int bottom_slices = 0;     // > 0: the three-layer bottom MLP as one slice launch storing
                             // this many partials of its last layer, which the interaction adds
  bool fuse_head = false;    // the last top layer folded into the one before
  std::vector<int> split_bottom, split_top;  // partials each layer launched on its own stores
};

struct ForwardLayout {
  int64_t P = 0, ldR = 0, ld_buf = 0;
  size_t off_R = 0, off_buf0 = 0, off_buf1 = 0, total = 0;
  MlpComposition mc;
};

constexpr uint32_t kForwardOptions = DLRM_FORWARD_LAYERED | DLRM_FORWARD_UNFUSED_HEAD |
                                     DLRM_FORWARD_UNFUSED_BOTTOM | DLRM_FORWARD_UNSPLIT_K;

// The bottom-MLP kernel's parameters for a three-layer stack, or false.
bool pack_bottom(int32_t m, const dlrm_layer *L, const float *x, int64_t ldx, float *y,
                 int64_t ldy, BottomParams &bp) {
  bp = BottomParams{};
  bp.M = m;
  bp.K0 = L[0].in_features;
  bp.N0 = L[0].out_features;
  bp.N1 = L[1].out_features;
  bp.N2 = L[2].out_features;
  if (L[1].in_features != bp.N0 || L[2].in_features != bp.N1) return false;
  bp.x = x;
  bp.ldx = ldx;
  bp.W0 = L[0].weight;
  bp.b0 = L[0].bias;
  bp.W1 = L[1].weight;
  bp.b1 = L[1].bias;
  bp.W2 = L[2].weight;
  bp.b2 = L[2].bias;
  bp.act0 = L[0].act;
  bp.act1 = L[1].act;
  bp.act2 = L[2].act;
  bp.y = y;
  bp.ldy = ldy;
  return bottom_mlp_supported(bp);
}

// Partials stored by each layer of a layered MLP: a layer whose tiles leave
// CUs idle splits its k (linear_split_count) when the next layer can read
// that many partials; the last layer stores its output.
std::vector<int> plan_layer_splits(int B, int n, const dlrm_layer *L, bool allow) {
  std::vector<int> sp((size_t)n, 1);
  for (int l = 0; allow && l + 1 < n; ++l) {
    int s = linear_split_count(B, L[l].out_features, L[l].in_features);
    while (s > 1 && !linear_reduce_supported(B, L[l + 1].out_features, L[l + 1].in_features,
                                             L[l + 1].weight, s))
      s /= 2;
    sp[(size_t)l] = s;
  }
  return sp;
}

// The slice launch takes the bottom MLP while its grid (one workgroup per
// 16-row band and slice of layer 1) is small.  With 64-column slices, up to
// 1.5 workgroups per CU: measured in the forward (13-512-256-64) at B = 256
// 15.8 us against 20.6 for the three layer launches, B = 1024 15.1 against
// 20.4; the whole cold forward at B = 1536 (384 workgroups) 78.3-78.6 us
// against 81.7, at B = 2048 (512) 85.8-86.1 against 85.2-85.5, at B = 3072
// 126.1 against 121.0.  16-column
// slices move a quarter of the W1 bytes per workgroup (each workgroup's
// weight loads take memory round trips, which set these launches' time):
// measured (trace) at B = 256 7.8 us against 14.7 for 64-column ones; the
// forward at B = 512 50.4 us with them (512 workgroups) against 52.9 with
// 64-column slices, at B = 1024 66.9 against 60.6.
constexpr int64_t kSliceMaxWorkgroups = 384;
constexpr int64_t kNarrowMaxWorkgroups = 512;

// The slice launch's parameters for a three-layer bottom MLP (shapes only;
// the buffers are set at launch); false if it cannot run them.
bool pack_slice(int B, const dlrm_layer *L, SliceParams &sp) {
  sp = SliceParams{};
  sp.M = B;
  sp.K0 = L[0].in_features;
  sp.N0 = L[0].out_features;
  sp.N1 = L[1].out_features;
  sp.N2 = L[2].out_features;
  if (L[1].in_features != sp.N0 || L[2].in_features != sp.N1) return false;
  sp.W0 = L[0].weight;
  sp.b0 = L[0].bias;
  sp.act0 = L[0].act;
  sp.W1 = L[1].weight;
  sp.b1 = L[1].bias;
  sp.act1 = L[1].act;
  sp.W2 = L[2].weight;
  // placeholders for the shape check
  sp.x = L[0].weight;
  sp.ldx = sp.K0;
  sp.P = reinterpret_cast<float *>(uintptr_t(256));
  sp.ldp = round4(sp.N2);
  sp.pstride = 0;
  // 16-column slices while their grid is at most two workgroups per CU,
  // else 64
  sp.sw = 16;
  if (slice_mlp_supported(sp) && slice_mlp_workgroups(sp) <= kNarrowMaxWorkgroups) return true;
  sp.sw = 64;
  return slice_mlp_supported(sp);
}


// The launch composition of a validated model's MLPs at batch B.
MlpComposition plan_mlps(const dlrm_model *m, int B) {
  MlpComposition mc;
  const uint32_t o = m->options;
  const bool split = !(o & DLRM_FORWARD_UNSPLIT_K);
  const int nb = m->num_bottom, nt = m->num_top;
  BottomParams bp;
  mc.fuse_bottom = !(o & DLRM_FORWARD_UNFUSED_BOTTOM) && nb == 3 && bottom_mlp_preferred(B) &&
                   pack_bottom(B, m->bottom, nullptr, m->bottom[0].in_features, nullptr,
                               m->bottom[2].out_features, bp);
  SliceParams sp;
  if (!mc.fuse_bottom && split && !(o & DLRM_FORWARD_UNFUSED_BOTTOM) && nb == 3 &&
      pack_slice(B, m->bottom, sp) &&
      slice_mlp_workgroups(sp) <= (sp.sw == 16 ? kNarrowMaxWorkgroups : kSliceMaxWorkgroups))
    mc.bottom_slices = slice_mlp_count(sp);
  mc.fuse_head = !(o & DLRM_FORWARD_UNFUSED_HEAD) && nt >= 2 &&
                 m->top[nt - 1].out_features == 1 &&
                 linear_head_supported(m->top[nt - 2].out_features, m->top[nt - 2].in_features) &&
                 linear_head_preferred(B);
  const bool layered_bottom = !mc.fuse_bottom && mc.bottom_slices == 0;
  mc.split_bottom = plan_layer_splits(B, nb, m->bottom, split && layered_bottom);
  mc.split_top = plan_layer_splits(B, nt, m->top, split && !mc.fuse_head);
  return mc;
}

// Checks the model's shapes and computes the workspace layout for batch B.
int plan_forward(const dlrm_model *m, int32_t B, ForwardLayout &lay) {
  if (!m) return DLRM_ERR_NULL;
  if (m->num_bottom < 1 || m->num_top < 1 || m->num_tables < 1 ||
      m->num_tables > DLRM_MAX_TABLES || m->dim < 1 || m->dim > DLRM_MAX_DIM || B < 0)
    return DLRM_ERR_SHAPE;
  if ((m->options & ~kForwardOptions) != 0) return DLRM_ERR_SHAPE;
  if (!m->bottom || !m->top || !m->tables || !m->rows) return DLRM_ERR_NULL;
  const int64_t F = (int64_t)m->num_tables + 1;
  lay.P = F * (F - 1) / 2;
  lay.ldR = round4(m->dim + lay.P);
  int64_t widest = 4;
  for (int l = 0; l < m->num_bottom; ++l) {
    const dlrm_layer &L = m->bottom[l];
    if (!L.weight) return DLRM_ERR_NULL;
    if (L.in_features < 1 || L.out_features < 1 || !valid_act(L.act)) return DLRM_ERR_SHAPE;
    if (l > 0 && L.in_features != m->bottom[l - 1].out_features) return DLRM_ERR_SHAPE;
    if (l + 1 < m->num_bottom) widest = widest > L.out_features ? widest : L.out_features;
  }
  if (m->bottom[m->num_bottom - 1].out_features != m->dim) return DLRM_ERR_SHAPE;
  for (int l = 0; l < m->num_top; ++l) {
    const dlrm_layer &L = m->top[l];
    if (!L.weight) return DLRM_ERR_NULL;
    if (L.in_features < 1 || L.out_features < 1 || !valid_act(L.act)) return DLRM_ERR_SHAPE;
    if (l > 0 && L.in_features != m->top[l - 1].out_features) return DLRM_ERR_SHAPE;
    if (l + 1 < m->num_top) widest = widest > L.out_features ? widest : L.out_features;
  }
  if (m->top[0].in_features != m->dim + lay.P) return DLRM_ERR_SHAPE;
  lay.ld_buf = round4(widest);
  lay.mc = plan_mlps(m, B);
  // What each of the two activation buffers holds, at B rows: the outputs
  // (or k partials) of layers launched on their own, alternating buffers;
  // the bottom slice launch's partials of the dense feature in buffer 0.
  const MlpComposition &mc = lay.mc;
  size_t need[2] = {0, 0};
  auto use = [&](int b, int64_t parts, int64_t ld) {
    need[b] = std::max(need[b], (size_t)parts * (size_t)B * (size_t)ld);
  };
  if (!mc.fuse_bottom && mc.bottom_slices == 0)
    for (int l = 0; l + 1 < m->num_bottom; ++l) use(l & 1, mc.split_bottom[(size_t)l], lay.ld_buf);
  if (mc.bottom_slices > 0) use(0, mc.bottom_slices, round4(m->dim));
  // (with the head folded in, layers 0 .. nt - 3 write buffers; otherwise
  // every layer but the last)
  const int nbuf = mc.fuse_head ? m->num_top - 2 : m->num_top - 1;
  for (int l = 0; l < nbuf; ++l) use(l & 1, mc.split_top[(size_t)l], lay.ld_buf);
  lay.off_R = 0;
  lay.off_buf0 = round256((size_t)B * (size_t)lay.ldR * sizeof(float));
  lay.off_buf1 = lay.off_buf0 + round256(need[0] * sizeof(float));
  lay.total = lay.off_buf1 + round256(need[1] * sizeof(float));
  return DLRM_OK;
}

// Where a forward's launches go: straight onto a stream, or into a list that
// a plan replays later.  Each launch is a callable taking the stream.
using Launch = std::function<hipError_t(hipStream_t)>;
struct Emitter {
  hipStream_t stream = nullptr;
  std::vector<Launch> *record = nullptr;
};

template <typename F>
int emit(const Emitter &em, F &&f) {
  if (em.record) {
    em.record->emplace_back(std::forward<F>(f));
    return DLRM_OK;
  }
  return hip_status(f(em.stream));
}

SmallLayer small_layer_of(const dlrm_layer &L) {
  return SmallLayer{L.weight, L.bias, L.in_features, L.out_features, L.act};
}

// Checks every argument of a forward (nothing is enqueued); the workspace
// only when check_ws.
int validate_forward(const dlrm_model *model, int32_t batch, const float *dense_in,
                     const int32_t *const *indices, const int32_t *const *offsets,
                     const int64_t *n_idx, const float *out, const void *workspace,
                     size_t workspace_bytes, bool check_ws = true) {
  ForwardLayout lay;
  int rc = plan_forward(model, batch, lay);
  if (rc) return rc;
  TableSet ts;
  GatherConfig gc;
  const dlrm_bags g = f32_sum_bags(model->num_tables, batch, model->dim, model->tables,
                                   model->rows, indices, offsets, n_idx);
  rc = pack_bags(g, ts, gc);
  if (rc) return rc;
  if (batch == 0) return DLRM_OK;
  if (!dense_in || !out) return DLRM_ERR_NULL;
  if (!check_ws) return DLRM_OK;
  if (!workspace) return DLRM_ERR_NULL;
  if (workspace_bytes < lay.total || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return DLRM_ERR_WORKSPACE;
  return DLRM_OK;
}

// A layer's input: a plain matrix, or nred partial sums of the layer before
// (stride floats apart) still to be added, biased and activated.
struct MlpInput {
  const float *p;
  int64_t ld;
  int nred = 1;
  int64_t stride = 0;
  const float *bias = nullptr;
  int act = 0;
};

// Emits layers [0, n) of an MLP, each as its own launch: layer l stores
// split[l] partials (or its output) in buf[l & 1], row stride ld_buf,
// partials pstride floats apart; the last one writes `out` (row stride ldo).
// `in` is the first layer's input on entry and the next layer's on return
// (so a caller may run further layers).  With out == nullptr every layer
// writes a buffer.
int emit_layers(const Emitter &em, int B, int n, const dlrm_layer *layers,
                const std::vector<int> &split, MlpInput &in, float *const buf[2],
                int64_t ld_buf, int64_t pstride, float *out, int64_t ldo) {
  for (int l = 0; l < n; ++l) {
    const dlrm_layer &L = layers[l];
    const bool last = out && l + 1 == n;
    const int ns = last ? 1 : split[(size_t)l];
    float *y = last ? out : buf[l & 1];
    const int64_t ldy = last ? ldo : ld_buf;
    const LinearCall c{B, L.out_features, L.in_features, in.p, in.ld, in.nred, in.stride,
                       in.bias, in.act, L.weight, L.bias, L.act, y, ldy, ns,
                       ns > 1 ? pstride : 0};
    const int rc = emit(em, [=](hipStream_t s) { return launch_linear_call(c, s); });
    if (rc) return rc;
    in = ns > 1 ? MlpInput{y, ldy, ns, pstride, L.bias, L.act} : MlpInput{y, ldy};
  }
  return DLRM_OK;
}

int enqueue_forward(const dlrm_model *model, int32_t batch, const float *dense_in,
                    const int32_t *const *indices, const int32_t *const *offsets,
                    const int64_t *n_idx, float *out, void *workspace, size_t workspace_bytes,
                    const Emitter &em) {
  ForwardLayout lay;
  int rc = plan_forward(model, batch, lay);
  if (rc) return rc;
  TableSet ts;
  GatherConfig gc;
  const dlrm_bags g = f32_sum_bags(model->num_tables, batch, model->dim, model->tables,
                                   model->rows, indices, offsets, n_idx);
  rc = pack_bags(g, ts, gc);
  if (rc) return rc;
  if (batch == 0) return DLRM_OK;  // nothing to read or write
  if (!dense_in || !out || !workspace) return DLRM_ERR_NULL;
  if (workspace_bytes < lay.total || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return DLRM_ERR_WORKSPACE;
  const int B = batch, D = model->dim, K = model->num_tables;

  // Models whose MLPs are small run the whole forward as one launch, unless
  // the model asks for the layered composition.
  if (!(model->options & DLRM_FORWARD_LAYERED) && model->num_bottom <= kMaxSmallLayers &&
      model->num_top <= kMaxSmallLayers) {
    SmallLayer bl[kMaxSmallLayers], tl[kMaxSmallLayers];
    for (int l = 0; l < model->num_bottom; ++l) bl[l] = small_layer_of(model->bottom[l]);
    for (int l = 0; l < model->num_top; ++l) tl[l] = small_layer_of(model->top[l]);
    SmallForwardParams sp{};
    int threads = 0;
    if (plan_forward_small(B, K, D, gc.vec, model->bottom[0].in_features, model->num_bottom, bl,
                           model->num_top, tl, sp, threads)) {
      sp.dense_in = dense_in;
      sp.out = out;
      sp.n_out = model->top[model->num_top - 1].out_features;
      const bool csr = gc.csr, vec = gc.vec;
      return emit(em, [=](hipStream_t s) {
        return launch_forward_small(ts, csr, vec, sp, threads, s);
      });
    }
  }

  char *ws = static_cast<char *>(workspace);
  float *R = reinterpret_cast<float *>(ws + lay.off_R);
  float *buf[2] = {reinterpret_cast<float *>(ws + lay.off_buf0),
                   reinterpret_cast<float *>(ws + lay.off_buf1)};

  // Bottom MLP.  A three-layer stack runs as one launch: at about one 32-row
  // band per CU the fused kernel (the last layer writes the dense feature
  // straight into R[:, 0:D]); at other batches the slice kernel, whose
  // partials of the last layer the interaction adds as it loads the dense
  // feature.  Otherwise layer by layer, a layer whose tiles would leave CUs
  // idle storing k partials that the next layer adds.
  const MlpComposition &mc = lay.mc;
  const int64_t pstride = (int64_t)B * lay.ld_buf;  // floats between partials
  MlpInput in{dense_in, model->bottom[0].in_features};
  if (mc.fuse_bottom) {
    BottomParams bp;
    if (!pack_bottom(B, model->bottom, dense_in, in.ld, R, lay.ldR, bp))
      return DLRM_ERR_UNSUPPORTED;
    rc = emit(em, [=](hipStream_t s) { return launch_bottom_mlp(bp, s); });
    if (rc) return rc;
  } else if (mc.bottom_slices > 0) {
    SliceParams sp;
    if (!pack_slice(B, model->bottom, sp)) return DLRM_ERR_UNSUPPORTED;
    sp.x = dense_in;
    sp.ldx = in.ld;
    sp.P = buf[0];
    sp.ldp = round4(D);
    sp.pstride = (int64_t)B * sp.ldp;
    rc = emit(em, [=](hipStream_t s) { return launch_slice_mlp(sp, s); });
    if (rc) return rc;
  } else {
    rc = emit_layers(em, B, model->num_bottom, model->bottom, mc.split_bottom, in, buf,
                     lay.ld_buf, pstride, R, lay.ldR);
    if (rc) return rc;
  }

  // Gather + interaction: the dense feature is read from R[:, 0:D] (or added
  // up from the slice kernel's partials and written there), dots go to
  // R[:, D:].
  gc.vec = gc.vec && lay.ldR % 4 == 0;
  InteractParams ip{};
  int threads = 0;
  if (!plan_interact(B, K, D, gc.vec, chunk_elems(gc), ip, threads)) return DLRM_ERR_UNSUPPORTED;
  ip.copy_dense = 0;
  ip.dot_off = D;
  ip.dense = R;
  ip.ld_dense = lay.ldR;
  if (mc.bottom_slices > 0) {
    const dlrm_layer &L2 = model->bottom[2];
    ip.copy_dense = 1;
    ip.dense = buf[0];
    ip.ld_dense = round4(D);
    ip.dense_nred = mc.bottom_slices;
    ip.dense_stride = (int64_t)B * ip.ld_dense;
    ip.dense_bias = L2.bias;
    ip.dense_act = L2.act;
  }
  ip.out = R;
  ip.ld_out = lay.ldR;
  ip.out_vec = 1;
  ip.emb_out = nullptr;
  ip.emb_in = nullptr;
  rc = emit(em, [=](hipStream_t s) { return launch_interact(&ts, gc, ip, threads, s); });
  if (rc) return rc;

  // Top MLP on cat(dense, dots) = R.  A one-output last layer (the sigmoid
  // head) is folded into the epilogue of the layer before it when that layer
  // is at most 256 wide and the batch is about one 32-row band per CU: its
  // activations are then never stored.
  const int nt = model->num_top;
  in = MlpInput{R, lay.ldR};
  if (mc.fuse_head) {
    rc = emit_layers(em, B, nt - 2, model->top, mc.split_top, in, buf, lay.ld_buf, pstride,
                     nullptr, 0);
    if (rc) return rc;
    const dlrm_layer &L = model->top[nt - 2], &H = model->top[nt - 1];
    const MlpInput x = in;
    return emit(em, [=](hipStream_t s) {
      return launch_linear_head(B, L.out_features, L.in_features, x.p, x.ld, L.weight, L.bias,
                                L.act, H.weight, H.bias, H.act, out, 1, s);
    });
  }
  return emit_layers(em, B, nt, model->top, mc.split_top, in, buf, lay.ld_buf, pstride, out,
                     model->top[nt - 1].out_features);
}

// Long bags whose pooled tensor the caller also asks for: the gather as its
// own launch into emb_out (its table-major grid lets each XCD's L2 specialise
// in a few tables), then the interaction reading emb_out, beats the fused
// kernel, whose workgroups each need rows of all K tables.  Measured on
// MI355X at B = 16384, K = 26, D = 128, 40 Zipf(1.05) indices per bag:
// 746 us against 826 us for the fused kernel writing emb_out; at 20 indices
// and D = 64 the fused kernel wins.
// Taken when the mean bag pools at least kTwoPassElems elements (L x D).
constexpr int64_t kTwoPassElems = 4096;

bool take_two_pass(const dlrm_bags &g, const GatherConfig &gc, const float *dense,
                   const float *emb_out) {
  if (!emb_out || !gc.vec || g.dim % 4 != 0 || !aligned16(dense) || !aligned16(emb_out))
    return false;
  int64_t n = 0;
  for (int k = 0; k < g.num_tables; ++k) n += g.n_idx[k];
  return n * g.dim >= kTwoPassElems * (int64_t)g.batch * g.num_tables;
}

// The two-launch form of the fused call: pooled bags to emb_out, then the
// interaction over them into out (layout as InteractParams describes).
int run_two_pass(const TableSet &ts, const GatherConfig &gc, int32_t B, int32_t K, int32_t D,
                 const float *dense, float *out, int64_t ld_out, int dot_off, int copy_dense,
                 int out_vec, float *emb_out, hipStream_t stream) {
  GatherConfig lg;
  lg.vec = true;
  InteractParams ip{};
  int threads = 0;
  // planned as the fused launch would be (same samples per workgroup, same
  // dot teams), so the dots are computed in the same order
  if (!plan_interact(B, K, D, true, chunk_elems(gc), ip, threads)) return DLRM_ERR_UNSUPPORTED;
  ip.copy_dense = copy_dense;
  ip.dot_off = dot_off;
  ip.dense = dense;
  ip.ld_dense = D;
  ip.out = out;
  ip.ld_out = ld_out;
  ip.out_vec = out_vec;
  ip.emb_out = nullptr;
  ip.emb_in = emb_out;
  const hipError_t e = launch_emb_bag(ts, gc, B, K, D, emb_out, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_interact(nullptr, lg, ip, threads, stream));
}

// Records the forward's launches on `st` (a capturing stream) into a graph.
int capture_forward(const dlrm_model &model, int32_t batch, const float *dense_in,
                    const int32_t *const *indices, const int32_t *const *offsets,
                    const int64_t *n_idx, float *out, void *workspace, size_t workspace_bytes,
                    hipStream_t st, hipGraph_t *graph) {
  *graph = nullptr;
  // kernel timing events are not recorded into a graph: the captured
  // launches are plain ones
  const LaunchTiming timing = launch_timing();
  launch_timing() = LaunchTiming{};
  if (hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed) != hipSuccess) {
    launch_timing() = timing;
    return DLRM_ERR_HIP;
  }
  const int rc = enqueue_forward(&model, batch, dense_in, indices, offsets, n_idx, out, workspace,
                                 workspace_bytes, Emitter{st, nullptr});
  launch_timing() = timing;
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(st, &g);
  if (rc || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return rc ? rc : DLRM_ERR_HIP;
  }
  *graph = g;
  return DLRM_OK;
}

// The workspace of dlrm_forward_noalloc: a fixed device array of the library
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes `scratch` itself to a kernel (on the host it is a
// stand-in, not a device address): it takes the array's device address from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) char scratch[DLRM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address, or nullptr (status in *rc).
void *scratch_address(int *rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *rc = DLRM_ERR_HIP;
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    *rc = DLRM_ERR_UNSUPPORTED;
    return nullptr;
  }
  ScratchSlot &slot = g_scratch[dev];
  std::call_once(slot.once, [&slot]() {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr) {
    *rc = DLRM_ERR_HIP;
    return nullptr;
  }
  *rc = DLRM_OK;
  return slot.ptr;
}

}  // namespace

LaunchTiming &dlrm::launch_timing() {
  static thread_local LaunchTiming timing;
  return timing;
}

extern "C" {

const char *dlrm_status_string(int status) {
  switch (status) {
    case DLRM_OK: return "DLRM_OK";
    case DLRM_ERR_NULL: return "DLRM_ERR_NULL: a required pointer is NULL";
    case DLRM_ERR_SHAPE: return "DLRM_ERR_SHAPE: a size is out of range or sizes disagree";
    case DLRM_ERR_UNSUPPORTED: return "DLRM_ERR_UNSUPPORTED: request beyond a documented limit";
    case DLRM_ERR_WORKSPACE: return "DLRM_ERR_WORKSPACE: workspace too small or misaligned";
    case DLRM_ERR_HIP: return "DLRM_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown dlrm_status";
  }
}

int dlrm_abi_version(void) { return DLRM_ABI_VERSION; }

int dlrm_set_kernel_timing_events(void *start, void *stop) {
  if ((start == nullptr) != (stop == nullptr)) return DLRM_ERR_NULL;
  launch_timing() = LaunchTiming{(hipEvent_t)start, (hipEvent_t)stop};
  return DLRM_OK;
}

int emb_bag_pool(const dlrm_bags *bags, float *out, void *stream) {
  if (!bags) return DLRM_ERR_NULL;
  TableSet ts;
  GatherConfig gc;
  int rc = pack_bags(*bags, ts, gc);
  if (rc) return rc;
  if (bags->batch == 0) return DLRM_OK;  // nothing to write: out may be NULL
  if (!out) return DLRM_ERR_NULL;
  gc.vec = gc.vec && aligned16(out);
  return hip_status(launch_emb_bag(ts, gc, bags->batch, bags->num_tables, bags->dim, out,
                                   (hipStream_t)stream));
}

int emb_bag_sum_multi(int32_t num_tables, int32_t batch, int32_t dim,
                      const float *const *tables, const int64_t *rows,
                      const int32_t *const *indices, const int32_t *const *offsets,
                      const int64_t *n_idx, float *out, void *stream) {
  const dlrm_bags g =
      f32_sum_bags(num_tables, batch, dim, tables, rows, indices, offsets, n_idx);
  return emb_bag_pool(&g, out, stream);
}

int dlrm_interact_lower_tri(int32_t batch, int32_t num_emb, int32_t dim, const float *dense,
                            const float *emb, float *out, void *stream) {
  if (batch < 0 || num_emb < 1 || num_emb > DLRM_MAX_TABLES || dim < 1 || dim > DLRM_MAX_DIM)
    return DLRM_ERR_SHAPE;
  if (batch == 0) return DLRM_OK;  // nothing to read or write
  if (!dense || !emb || !out) return DLRM_ERR_NULL;
  GatherConfig gc;
  gc.vec = dim % 4 == 0 && aligned16(dense) && aligned16(emb);
  InteractParams ip{};
  int threads = 0;
  if (!plan_interact(batch, num_emb, dim, gc.vec, gc.vec ? 4 : 1, ip, threads))
    return DLRM_ERR_UNSUPPORTED;
  ip.copy_dense = 1;
  ip.dot_off = dim;
  ip.dense = dense;
  ip.ld_dense = dim;
  ip.out = out;
  ip.ld_out = dim + ip.P;
  ip.out_vec = aligned16(out) && ip.ld_out % 4 == 0;
  ip.emb_out = nullptr;
  ip.emb_in = emb;
  return hip_status(launch_interact(nullptr, gc, ip, threads, (hipStream_t)stream));
}

int dlrm_emb_interact_pool(const dlrm_bags *bags, const float *dense, float *out,
                           float *emb_out, void *stream) {
  if (!bags) return DLRM_ERR_NULL;
  TableSet ts;
  GatherConfig gc;
  int rc = pack_bags(*bags, ts, gc);
  if (rc) return rc;
  const int32_t batch = bags->batch, K = bags->num_tables, dim = bags->dim;
  if (batch == 0) return DLRM_OK;  // nothing to read or write
  if (!dense || !out) return DLRM_ERR_NULL;
  if (take_two_pass(*bags, gc, dense, emb_out)) {
    const int64_t ld = dim + (int64_t)(K + 1) * K / 2;
    return run_two_pass(ts, gc, batch, K, dim, dense, out, ld, dim, 1,
                        aligned16(out) && ld % 4 == 0, emb_out, (hipStream_t)stream);
  }
  gc.vec = gc.vec && aligned16(dense) && (!emb_out || aligned16(emb_out));
  InteractParams ip{};
  int threads = 0;
  if (!plan_interact(batch, K, dim, gc.vec, chunk_elems(gc), ip, threads))
    return DLRM_ERR_UNSUPPORTED;
  ip.copy_dense = 1;
  ip.dot_off = dim;
  ip.dense = dense;
  ip.ld_dense = dim;
  ip.out = out;
  ip.ld_out = dim + ip.P;
  ip.out_vec = aligned16(out) && ip.ld_out % 4 == 0;
  ip.emb_out = emb_out;
  ip.emb_in = nullptr;
  return hip_status(launch_interact(&ts, gc, ip, threads, (hipStream_t)stream));
}

int dlrm_emb_interact_dots(const dlrm_bags *bags, const float *dense, float *dots,
                           int64_t ld_dots, float *emb_out, void *stream) {
  if (!bags) return DLRM_ERR_NULL;
  TableSet ts;
  GatherConfig gc;
  int rc = pack_bags(*bags, ts, gc);
  if (rc) return rc;
  const int32_t batch = bags->batch, K = bags->num_tables, dim = bags->dim;
  const int64_t F = (int64_t)K + 1;
  if (ld_dots < F * (F - 1) / 2) return DLRM_ERR_SHAPE;
  if (batch == 0) return DLRM_OK;  // nothing to read or write
  if (!dense || !dots) return DLRM_ERR_NULL;
  if (take_two_pass(*bags, gc, dense, emb_out))
    return run_two_pass(ts, gc, batch, K, dim, dense, dots, ld_dots, 0, 0, 0, emb_out,
                        (hipStream_t)stream);
  gc.vec = gc.vec && aligned16(dense) && (!emb_out || aligned16(emb_out));
  InteractParams ip{};
  int threads = 0;
  if (!plan_interact(batch, K, dim, gc.vec, chunk_elems(gc), ip, threads))
    return DLRM_ERR_UNSUPPORTED;
  ip.copy_dense = 0;
  ip.dot_off = 0;
  ip.dense = dense;
  ip.ld_dense = dim;
  ip.out = dots;
  ip.ld_out = ld_dots;
  ip.out_vec = 0;
  ip.emb_out = emb_out;
  ip.emb_in = nullptr;
  return hip_status(launch_interact(&ts, gc, ip, threads, (hipStream_t)stream));
}

int dlrm_emb_interact(int32_t num_tables, int32_t batch, int32_t dim,
                      const float *const *tables, const int64_t *rows,
                      const int32_t *const *indices, const int32_t *const *offsets,
                      const int64_t *n_idx, const float *dense, float *out, float *emb_out,
                      void *stream) {
  const dlrm_bags g =
      f32_sum_bags(num_tables, batch, dim, tables, rows, indices, offsets, n_idx);
  return dlrm_emb_interact_pool(&g, dense, out, emb_out, stream);
}

int linear_bias_act(int32_t m, int32_t n, int32_t k, const float *a, int64_t lda,
                    const float *w, const float *bias, int32_t act, float *c, int64_t ldc,
                    void *stream) {
  if (m < 0 || n < 1 || k < 1 || lda < k || ldc < n || !valid_act(act)) return DLRM_ERR_SHAPE;
  if (m == 0) return DLRM_OK;  // nothing to read or write
  if (!a || !w || !c) return DLRM_ERR_NULL;
  return hip_status(launch_linear(m, n, k, a, lda, w, bias, act, c, ldc, (hipStream_t)stream));
}

int linear_bias_act_split(int32_t m, int32_t n, int32_t k_lo, const float *a_lo, int64_t lda_lo,
                          int32_t k_hi, const float *a_hi, int64_t lda_hi, const float *w,
                          const float *bias, int32_t act, float *c, int64_t ldc, void *stream) {
  if (m < 0 || n < 1 || k_lo < 1 || k_hi < 1 || (int64_t)k_lo + k_hi > INT32_MAX ||
      lda_lo < k_lo || lda_hi < k_hi || ldc < n || !valid_act(act))
    return DLRM_ERR_SHAPE;
  if (m == 0) return DLRM_OK;  // nothing to read or write
  if (!a_lo || !a_hi || !w || !c) return DLRM_ERR_NULL;
  return hip_status(launch_linear_split(m, n, k_lo, a_lo, lda_lo, k_hi, a_hi, lda_hi, w, bias,
                                        act, c, ldc, (hipStream_t)stream));
}

int linear_bias_act_head(int32_t m, int32_t n, int32_t k, const float *a, int64_t lda,
                         const float *w, const float *bias, int32_t act, const float *head_w,
                         const float *head_bias, int32_t head_act, float *out, int64_t ldo,
                         void *stream) {
  if (m < 0 || n < 1 || k < 1 || lda < k || ldo < 1 || !valid_act(act) || !valid_act(head_act))
    return DLRM_ERR_SHAPE;
  if (!linear_head_supported(n, k)) return DLRM_ERR_UNSUPPORTED;
  if (m == 0) return DLRM_OK;  // nothing to read or write
  if (!a || !w || !head_w || !out) return DLRM_ERR_NULL;
  return hip_status(launch_linear_head(m, n, k, a, lda, w, bias, act, head_w, head_bias,
                                       head_act, out, ldo, (hipStream_t)stream));
}

int mlp_forward(int32_t m, int32_t num_layers, const dlrm_layer *layers, const float *a,
                int64_t lda, float *c, int64_t ldc, void *stream) {
  if (m < 0 || num_layers < 1) return DLRM_ERR_SHAPE;
  if (!layers) return DLRM_ERR_NULL;
  for (int l = 0; l < num_layers; ++l) {
    const dlrm_layer &L = layers[l];
    if (L.in_features < 1 || L.out_features < 1 || !valid_act(L.act)) return DLRM_ERR_SHAPE;
    if (l > 0 && L.in_features != layers[l - 1].out_features) return DLRM_ERR_SHAPE;
    if (!L.weight) return DLRM_ERR_NULL;
  }
  if (lda < layers[0].in_features || ldc < layers[num_layers - 1].out_features)
    return DLRM_ERR_SHAPE;
  if (m == 0) return DLRM_OK;  // nothing to read or write
  if (!a || !c) return DLRM_ERR_NULL;
  // A three-layer stack of the bottom-MLP shape takes the fused bottom
  // kernel (faster than the chain kernel at every row count); anything else
  // the MLP chain kernel.
  BottomParams bp;
  if (num_layers == 3 && pack_bottom(m, layers, a, lda, c, ldc, bp))
    return hip_status(launch_bottom_mlp(bp, (hipStream_t)stream));
  ChainParams cp;
  if (!pack_chain(m, num_layers, layers, a, lda, c, ldc, cp)) return DLRM_ERR_UNSUPPORTED;
  return hip_status(launch_mlp_chain(cp, (hipStream_t)stream));
}

size_t dlrm_forward_workspace_bytes(const dlrm_model *model, int32_t batch) {
  ForwardLayout lay;
  if (plan_forward(model, batch, lay) != DLRM_OK) return 0;
  return lay.total;
}

int dlrm_forward(const dlrm_model *model, int32_t batch, const float *dense_in,
                 const int32_t *const *indices, const int32_t *const *offsets,
                 const int64_t *n_idx, float *out, void *workspace, size_t workspace_bytes,
                 void *stream) {
  return enqueue_forward(model, batch, dense_in, indices, offsets, n_idx, out, workspace,
                         workspace_bytes, Emitter{(hipStream_t)stream, nullptr});
}

int dlrm_forward_noalloc(const dlrm_model *model, int32_t batch, const float *dense_in,
                         const int32_t *const *indices, const int32_t *const *offsets,
                         const int64_t *n_idx, float *out, void *stream) {
  // every argument is checked before the scratch array is looked up
  int rc = validate_forward(model, batch, dense_in, indices, offsets, n_idx, out, nullptr, 0,
                            /*check_ws=*/false);
  if (rc) return rc;
  if (batch == 0) return DLRM_OK;  // nothing to read or write
  ForwardLayout lay;
  rc = plan_forward(model, batch, lay);
  if (rc) return rc;
  // A composition whose k partials do not fit runs without k splits.
  dlrm_model unsplit = *model;
  unsplit.options |= DLRM_FORWARD_UNSPLIT_K;
  const dlrm_model *use = model;
  if (lay.total > (size_t)DLRM_NOALLOC_SCRATCH_BYTES) {
    use = &unsplit;
    rc = plan_forward(use, batch, lay);
    if (rc) return rc;
    if (lay.total > (size_t)DLRM_NOALLOC_SCRATCH_BYTES) return DLRM_ERR_WORKSPACE;
  }
  void *ws = scratch_address(&rc);
  if (!ws) return rc;
  return enqueue_forward(use, batch, dense_in, indices, offsets, n_idx, out, ws,
                         (size_t)DLRM_NOALLOC_SCRATCH_BYTES, Emitter{(hipStream_t)stream, nullptr});
}

// ---------------------------------------------------------------------------
// Plans: the forward captured once into a HIP graph, replayed per call.
// ---------------------------------------------------------------------------
struct dlrm_plan {
  // The model, copied so that a plan does not depend on the caller's host
  // arrays after creation (the layers and tables it points to stay the
  // caller's device memory).
  std::vector<dlrm_layer> bottom, top;
  std::vector<const float *> tables;
  std::vector<int64_t> rows;
  dlrm_model model;
  int32_t batch = 0;
  int32_t mode = DLRM_PLAN_DIRECT;
  void *workspace = nullptr;
  size_t workspace_bytes = 0;
  std::vector<Launch> launches;  // direct mode
  hipStream_t capture = nullptr;  // graph mode
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

int dlrm_plan_create(const dlrm_model *model, int32_t batch, const float *dense_in,
                     const int32_t *const *indices, const int32_t *const *offsets,
                     const int64_t *n_idx, float *out, void *workspace, size_t workspace_bytes,
                     int32_t mode, dlrm_plan **plan_out) {
  if (!plan_out) return DLRM_ERR_NULL;
  *plan_out = nullptr;
  if (mode != DLRM_PLAN_DIRECT && mode != DLRM_PLAN_GRAPH) return DLRM_ERR_SHAPE;
  int rc = validate_forward(model, batch, dense_in, indices, offsets, n_idx, out, workspace,
                            workspace_bytes);
  if (rc) return rc;
  if (batch < 1) return DLRM_ERR_SHAPE;  // a plan of nothing is not useful
  dlrm_plan *p = new (std::nothrow) dlrm_plan;
  if (!p) return DLRM_ERR_UNSUPPORTED;
  p->bottom.assign(model->bottom, model->bottom + model->num_bottom);
  p->top.assign(model->top, model->top + model->num_top);
  p->tables.assign(model->tables, model->tables + model->num_tables);
  p->rows.assign(model->rows, model->rows + model->num_tables);
  p->model = *model;
  p->model.bottom = p->bottom.data();
  p->model.top = p->top.data();
  p->model.tables = p->tables.data();
  p->model.rows = p->rows.data();
  p->batch = batch;
  p->mode = mode;
  p->workspace = workspace;
  p->workspace_bytes = workspace_bytes;
  if (mode == DLRM_PLAN_DIRECT) {
    rc = enqueue_forward(&p->model, batch, dense_in, indices, offsets, n_idx, out, workspace,
                         workspace_bytes, Emitter{nullptr, &p->launches});
    if (rc) {
      delete p;
      return rc;
    }
    *plan_out = p;
    return DLRM_OK;
  }
  if (hipStreamCreateWithFlags(&p->capture, hipStreamNonBlocking) != hipSuccess) {
    delete p;
    return DLRM_ERR_HIP;
  }
  rc = capture_forward(p->model, batch, dense_in, indices, offsets, n_idx, out, workspace,
                       workspace_bytes, p->capture, &p->graph);
  if (rc == DLRM_OK &&
      hipGraphInstantiate(&p->exec, p->graph, nullptr, nullptr, 0) != hipSuccess)
    rc = DLRM_ERR_HIP;
  if (rc) {
    dlrm_plan_destroy(p);
    return rc;
  }
  *plan_out = p;
  return DLRM_OK;
}

int dlrm_plan_update(dlrm_plan *plan, const float *dense_in, const int32_t *const *indices,
                     const int32_t *const *offsets, const int64_t *n_idx, float *out) {
  if (!plan) return DLRM_ERR_NULL;
  int rc = validate_forward(&plan->model, plan->batch, dense_in, indices, offsets, n_idx, out,
                            plan->workspace, plan->workspace_bytes);
  if (rc) return rc;
  if (plan->mode == DLRM_PLAN_DIRECT) {
    std::vector<Launch> fresh;
    rc = enqueue_forward(&plan->model, plan->batch, dense_in, indices, offsets, n_idx, out,
                         plan->workspace, plan->workspace_bytes, Emitter{nullptr, &fresh});
    if (rc) return rc;
    plan->launches.swap(fresh);
    return DLRM_OK;
  }
  hipGraph_t g = nullptr;
  rc = capture_forward(plan->model, plan->batch, dense_in, indices, offsets, n_idx, out,
                       plan->workspace, plan->workspace_bytes, plan->capture, &g);
  if (rc) return rc;
  hipGraphNode_t err_node = nullptr;
  hipGraphExecUpdateResult res = hipGraphExecUpdateError;
  if (hipGraphExecUpdate(plan->exec, g, &err_node, &res) != hipSuccess ||
      res != hipGraphExecUpdateSuccess) {
    // The launch shapes changed (e.g. other offsets switch the gather's
    // kernel): instantiate the new graph instead.
    (void)hipGetLastError();
    hipGraphExec_t fresh = nullptr;
    if (hipGraphInstantiate(&fresh, g, nullptr, nullptr, 0) != hipSuccess) {
      (void)hipGraphDestroy(g);
      return DLRM_ERR_HIP;
    }
    (void)hipGraphExecDestroy(plan->exec);
    plan->exec = fresh;
  }
  (void)hipGraphDestroy(plan->graph);
  plan->graph = g;
  return DLRM_OK;
}

int dlrm_plan_run(dlrm_plan *plan, void *stream) {
  if (!plan) return DLRM_ERR_NULL;
  const hipStream_t st = (hipStream_t)stream;
  if (plan->mode == DLRM_PLAN_GRAPH) return hip_status(hipGraphLaunch(plan->exec, st));
  for (const Launch &f : plan->launches)
    if (f(st) != hipSuccess) return DLRM_ERR_HIP;
  return DLRM_OK;
}

int dlrm_plan_destroy(dlrm_plan *plan) {
  if (!plan) return DLRM_OK;
  int rc = DLRM_OK;
  if (plan->exec && hipGraphExecDestroy(plan->exec) != hipSuccess) rc = DLRM_ERR_HIP;
  if (plan->graph && hipGraphDestroy(plan->graph) != hipSuccess) rc = DLRM_ERR_HIP;
  if (plan->capture && hipStreamDestroy(plan->capture) != hipSuccess) rc = DLRM_ERR_HIP;
  delete plan;
  return rc;
}

}  // extern "C"
