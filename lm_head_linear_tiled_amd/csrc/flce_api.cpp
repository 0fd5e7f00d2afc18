// Host layer of the fused linear + cross-entropy library: the C ABI declared in
// include/flce.h.  Every argument is checked here, before any HIP call, so that
// a bad call enqueues nothing; then the launch plan is drawn up, the caller's
// workspace is carved, and the kernels are enqueued on the caller's stream.
#include "flce.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "flce_launch.h"

namespace {

using flce::BwdPlan;
using flce::FwdPlan;
using flce::kTile;

constexpr int64_t kMaxDim = int64_t(1) << 30;     // keeps every int index in range
#ifndef FLCE_FWD_TARGET_WGS
#define FLCE_FWD_TARGET_WGS 256
#endif
constexpr int kFwdTargetWorkgroups = FLCE_FWD_TARGET_WGS;  // forward workgroups to aim for (256 CUs)
// At least 4 vocabulary splits: with many token tiles and only 2 splits, the 32
// workgroups an XCD runs at once hold 16 different token tiles of x (32 MB) and
// the x tiles in use across the chip outgrow the last-level cache; 4 splits keep
// 8 per XCD (32768 tokens, V 128256: forward 1154 -> 1352 TFLOP/s).
#ifndef FLCE_FWD_MIN_SPLITS
#define FLCE_FWD_MIN_SPLITS 4
#endif
constexpr int kFwdMinSplits = FLCE_FWD_MIN_SPLITS;
#ifndef FLCE_PANEL_MB
#define FLCE_PANEL_MB 128
#endif
constexpr size_t kDefaultPanelBytes = size_t(FLCE_PANEL_MB) << 20;  // dlogit panel budget
#ifndef FLCE_PANEL_GROUP
#define FLCE_PANEL_GROUP 2
#endif
constexpr int kPanelGroup = FLCE_PANEL_GROUP;  // panels per grad_x launch when all tokens form one chunk
constexpr int kPlanCUs = 256;  // compute units the panel shape is planned for (MI355X)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t esize(flce_dtype dt) { return dt == FLCE_BF16 ? 2 : 4; }

// Each size in [1, 2^30], and the 256 x 256 tiles of every contraction (N x V,
// N x H, V x H) countable in 32 bits.
bool dims_ok(int64_t N, int64_t H, int64_t V) {
  if (!(N > 0 && H > 0 && V > 0 && N <= kMaxDim && H <= kMaxDim && V <= kMaxDim)) return false;
  constexpr int64_t kMaxTiles = int64_t(1) << 31;
  const int64_t tn = (N + 255) / 256, th = (H + 255) / 256, tv = (V + 255) / 256;
  return tn * tv < kMaxTiles && tn * th < kMaxTiles && tv * th < kMaxTiles;
}
bool dtype_ok(flce_dtype dt) { return dt == FLCE_F32 || dt == FLCE_BF16; }
// A copy of a 256-row operand tile addresses its rows from one buffer resource
// with a 2 GiB range, so a row (H entries of x or W, the padded V entries of a
// dlogit panel) may span at most 8 MiB.
bool rows_ok(int64_t H, int64_t V, flce_dtype dt) {
  constexpr int64_t kMaxRowBytes = int64_t(8) << 20;
  const int64_t es = (int64_t)esize(dt);
  return H * es <= kMaxRowBytes && ceil_div(V, kTile) * kTile * es <= kMaxRowBytes;
}

FwdPlan plan_forward(int64_t N, int64_t V) {
  FwdPlan p{};
  p.tiles_tok = (int)ceil_div(N, kTile);
  p.Np = p.tiles_tok * kTile;
  const int tiles_v = (int)ceil_div(V, kTile);
  int splits = (int)std::min<int64_t>(
      tiles_v, std::max<int64_t>(kFwdMinSplits, ceil_div(kFwdTargetWorkgroups, p.tiles_tok)));
  p.tiles_per_split = (int)ceil_div(tiles_v, splits);
  p.splits = (int)ceil_div(tiles_v, p.tiles_per_split);  // no empty split
  size_t o = 0;
  p.off_m = o;
  o = align_up(o + sizeof(float) * (size_t)p.splits * p.Np, 256);
  p.off_s = o;
  o = align_up(o + sizeof(float) * (size_t)p.splits * p.Np, 256);
  p.off_zt = o;
  o = align_up(o + sizeof(float) * (size_t)p.Np, 256);
  p.nb = (int)ceil_div(N, 64);
  p.off_blk = o;
  o = align_up(o + sizeof(double) * (size_t)p.nb + sizeof(unsigned int), 256);
  p.total = o;
  return p;
}

BwdPlan plan_backward_shape(int64_t N, int64_t H, int64_t V, flce_dtype dt, int64_t Nc, int64_t Vb,
                            int group = 1);

// grad_x K splits for chunks of Nc tokens and panels of Vb entries: when a
// grad_x launch has fewer output tiles than half the compute units, its K
// (vocabulary) range is split over up to 4 workgroups per tile, each keeping at
// least 2048 entries; the float32 partial sums are added by a small kernel.
int64_t gx_splits_for(int64_t Nc, int64_t Vb, int64_t H) {
  const int64_t tiles = ceil_div(Nc, kTile) * ceil_div(H, kTile);
  const int64_t ks = std::min<int64_t>({4, kPlanCUs / tiles, Vb / 2048});
  return ks >= 2 ? ks : 1;
}

// Estimated backward time for chunks of Nc tokens and panels of Vb vocabulary
// entries, in units of one 256 x 256 x 256 tile contraction on one CU (a
// persistent launch of T tiles takes ceil(T / cus) rounds of tiles, each as
// many units as its K extent has 256-slices), plus a fixed cost per launch and
// the float32 accumulator traffic of gradients summed over several launches.
double backward_cost(int64_t N, int64_t H, int64_t V, int64_t Nc, int64_t Vb, int cus) {
  constexpr double kLaunch = 1.0;       // launch, fill and drain
  constexpr double kUnitsPerGB = 32.0;  // accumulator read-modify-write at ~4 TB/s
  const int64_t th = ceil_div(H, kTile);  // hidden tiles of grad_x / grad_W, and 256-slices of H
  auto rounds = [&](int64_t tiles) { return (double)ceil_div(tiles, cus); };
  // dlogits, grad_W (and grad_x without K splits): full rounds of whole tiles,
  // the partial last round cut along K (kunits 256-wide units per tile) into
  // pieces, plus their float32 fixup
  auto gw_cost = [&](int64_t tiles, int64_t kunits, bool bal) {
    const int64_t g = std::min<int64_t>(tiles, cus);
    // balanced: every workgroup the same number of slices, plus the hand-over of
    // one partial tile per workgroup
    if (bal && flce::balanced_launch(tiles, g)) return (double)tiles * kunits / g + kLaunch;
    const flce::TailSplit ts = flce::tail_split(tiles, cus, cus, kunits * kTile);
    if (ts.kts < 2) return rounds(tiles) * kunits;
    return (double)(ts.full / g) * kunits + (double)ceil_div(kunits, ts.kts) + kLaunch +
           (double)ts.tail * (ts.kts + 2) * kTile * kTile * 4 / 1e9 * kUnitsPerGB;
  };
  // chunk and panel sizes: full ones and the ragged last one
  const int64_t nc_full = N / Nc, nc_last = N % Nc, nv_full = V / Vb, nv_last = V % Vb;
  const int64_t n_chunks = nc_full + (nc_last ? 1 : 0), n_panels = nv_full + (nv_last ? 1 : 0);
  double t = 0;
  for (int ci = 0; ci < 2; ++ci) {
    const int64_t cnt_c = ci == 0 ? nc_full : (nc_last ? 1 : 0), Kc = ci == 0 ? Nc : nc_last;
    if (cnt_c == 0) continue;
    for (int vi = 0; vi < 2; ++vi) {
      const int64_t cnt_v = vi == 0 ? nv_full : (nv_last ? 1 : 0), Kv = vi == 0 ? Vb : nv_last;
      if (cnt_v == 0) continue;
      const int64_t tm = ceil_div(Kc, kTile), tv = ceil_div(Kv, kTile);
      const int64_t ks = gx_splits_for(Nc, Vb, H);
      const double gx = ks > 1 ? rounds(tm * th * ks) * ceil_div(tv, ks) : gw_cost(tm * th, tv, flce::kBalance);
      double one = gw_cost(tm * tv, th, flce::kBalanceDlogits) + gw_cost(tv * th, tm, flce::kBalance) + gx +
                   3 * kLaunch;
      if (ks > 1) one += kLaunch + (double)(ks + 1) * Kc * H * 4 / 1e9 * kUnitsPerGB;  // partial-sum pass
      t += (double)(cnt_c * cnt_v) * one;
    }
  }
  // grad_x rows are read and written once per panel after the first, grad_W rows
  // once per chunk after the first (float32), whatever the output type
  const double acc_gb = ((double)(n_panels - 1) * N * H + (double)(n_chunks - 1) * V * H) * 2 * 4 / 1e9;
  return t + acc_gb * kUnitsPerGB;
}

// Dlogit panel of Nc tokens x Vb vocabulary entries holding at most panel_elems
// values: of the chunk sizes Nc (each with the widest panel that fits), the one
// of least estimated time; accumulators only where a gradient is summed over
// several launches.  (Also trying narrower panels that fill whole rounds of the
// compute units was measured no better.)
//
// group = 2 (used when every token fits in one chunk and there are several
// panels): two consecutive panels are kept in the panel buffer, one block each,
// the dlogit and grad_W launches still work one panel at a time, and grad_x runs
// once per pair over both blocks: half the float32 accumulator passes over
// grad_x (each a burst of loads at the start and of stores at the end of a
// launch) for one more panel of workspace.
BwdPlan plan_backward_for(int64_t N, int64_t H, int64_t V, flce_dtype dt, int64_t panel_elems, int group = 1) {
  const int64_t Np = ceil_div(N, kTile) * kTile;
  const int64_t Vp = ceil_div(V, kTile) * kTile;
  int64_t best_nc = kTile, best_vb = kTile;
  double best = -1;
  for (int64_t Nc = kTile; Nc <= Np; Nc += kTile) {
    const int64_t Vb = std::min(Vp, panel_elems / Nc / kTile * kTile);
    if (Vb < kTile) break;
    const double c = backward_cost(N, H, V, Nc, Vb, kPlanCUs);
    if (best < 0 || c <= best) {  // ties: the larger token chunk
      best = c;
      best_nc = Nc;
      best_vb = Vb;
    }
  }
  const bool one_chunk = best_nc >= N, several_panels = best_vb < V;
  return plan_backward_shape(N, H, V, dt, best_nc, best_vb, one_chunk && several_panels ? group : 1);
}

// Plan for chunks of Nc tokens and panels of Vb vocabulary entries (both
// multiples of kTile, at most the padded N and V).
BwdPlan plan_backward_shape(int64_t N, int64_t H, int64_t V, flce_dtype dt, int64_t Nc, int64_t Vb, int group) {
  BwdPlan p{};
  p.Nc = (int)Nc;
  p.Ncp = (int)Nc;  // a multiple of kTile
  p.n_chunks = (int)ceil_div(N, Nc);
  p.Vb = (int)Vb;
  p.Vbp = (int)Vb;  // a multiple of kTile
  p.n_panels = (int)ceil_div(V, Vb);
  p.gx_group = std::max(1, std::min(group, p.n_panels));
  const size_t es = esize(dt);
  // float32 gradients accumulate in place; bfloat16 ones through float32 buffers.
  p.gx_bytes = (dt == FLCE_BF16 && p.n_panels > 1) ? sizeof(float) * (size_t)N * H : 0;
  p.gw_bytes = (dt == FLCE_BF16 && p.n_chunks > 1) ? sizeof(float) * (size_t)Vb * H : 0;
  p.gx_splits = (int)gx_splits_for(Nc, std::min<int64_t>((int64_t)p.gx_group * Vb, V), H);
  p.gxpart_bytes = p.gx_splits > 1 ? sizeof(float) * (size_t)p.gx_splits * p.Ncp * H : 0;
  size_t o = 0;
  p.off_panel = o;
  o = align_up(o + es * (size_t)p.Ncp * p.Vbp * p.gx_group, 256);
  p.off_gx = o;
  o = align_up(o + p.gx_bytes, 256);
  p.off_gw = o;
  o = align_up(o + p.gw_bytes, 256);
  p.off_gxpart = o;
  o = align_up(o + p.gxpart_bytes, 256);
  // partial tiles for the split tail of grad_W launches: the most any launch
  // shape (full or ragged chunk x full or ragged panel) needs on kPlanCUs
  // workgroups (the launcher splits no more than this holds); with balanced
  // launches, one slot per workgroup if any launch shape is balanced (the
  // launcher balances only when its grid has no more workgroups than slots)
  p.tail_cap = 0;
  p.slots = 0;
  const int64_t th = ceil_div(H, kTile);
  auto need = [&](int64_t T, int64_t K, bool bal) {
    if (bal && flce::balanced_launch(T, std::min<int64_t>(T, kPlanCUs))) {
      p.slots = kPlanCUs;
      return;
    }
    const flce::TailSplit ts = flce::tail_split(T, kPlanCUs, kPlanCUs, K);
    p.tail_cap = std::max(p.tail_cap, ts.tail * ts.kts);
  };
  const int64_t Kv_last = V - (p.n_panels - 1) * Vb, Kc_last = N - (p.n_chunks - 1) * Nc;
  for (int64_t Kv : {Vb, Kv_last})
    for (int64_t Kc : {Nc, Kc_last}) {
      need(ceil_div(Kv, kTile) * th, Kc, flce::kBalance);                                  // grad_W
      need(ceil_div(Kc, kTile) * ceil_div(Kv, kTile), H, flce::kBalanceDlogits);           // dlogits
    }
  if (p.gx_splits == 1) {
    // grad_x K: a whole group of panels, or the last group (it holds the last panel)
    const int64_t Kg_last = V - (int64_t)((p.n_panels - 1) / p.gx_group) * p.gx_group * Vb;
    for (int64_t Kc : {Nc, Kc_last})
      for (int64_t Kg : {std::min<int64_t>((int64_t)p.gx_group * Vb, V), Kg_last})
        need(ceil_div(Kc, kTile) * th, Kg, flce::kBalance);
  }
  p.tail_bytes = sizeof(float) * (size_t)std::max(p.tail_cap, p.slots) * kTile * kTile;
  p.off_tail = o;
  o = align_up(o + p.tail_bytes, 256);
  p.off_flags = o;
  o = align_up(o + sizeof(int) * (size_t)p.slots, 256);
  p.total = o;
  return p;
}

// Largest panel (up to the default budget) whose plan fits in ws_bytes; at each
// panel size the grouped plan first.
bool plan_backward(int64_t N, int64_t H, int64_t V, flce_dtype dt, size_t ws_bytes, BwdPlan* out) {
  int64_t elems = (int64_t)(kDefaultPanelBytes / esize(dt));
  const int64_t min_elems = int64_t(kTile) * kTile;
  while (true) {
    for (int group : {kPanelGroup, 2, 1}) {
      if (group > kPanelGroup) continue;
      BwdPlan p = plan_backward_for(N, H, V, dt, elems, group);
      if (p.total <= ws_bytes) {
        *out = p;
        return true;
      }
    }
    if (elems <= min_elems) return false;
    elems = std::max(min_elems, elems / 2);
  }
}

// Token chunks of chunk_tokens (rounded up to kTile, at most the padded N), each
// with the whole vocabulary as one panel.
BwdPlan plan_backward_chunked(int64_t N, int64_t H, int64_t V, flce_dtype dt, int64_t chunk_tokens) {
  const int64_t Np = ceil_div(N, kTile) * kTile;
  const int64_t Nc = std::min(Np, ceil_div(chunk_tokens, kTile) * kTile);
  return plan_backward_shape(N, H, V, dt, Nc, ceil_div(V, kTile) * kTile);
}

struct Range {
  const void* p;
  size_t n;
};
bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
// Does any output overlap an input, another output or the workspace?
bool any_alias(const Range* in, int nin, const Range* out, int nout, Range ws) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(out[i], in[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return true;
    if (overlap(out[i], ws)) return true;
  }
  for (int j = 0; j < nin; ++j)
    if (overlap(ws, in[j])) return true;
  return false;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

flce_status check_common(const void* x, const void* W, const int64_t* target, int64_t N, int64_t H, int64_t V,
                         flce_dtype dt, flce_reduction reduction) {
  if (!x || !W || !target) return FLCE_ERR_NULL;
  if (!dims_ok(N, H, V)) return FLCE_ERR_SHAPE;
  if (!dtype_ok(dt)) return FLCE_ERR_DTYPE;
  if (!rows_ok(H, V, dt)) return FLCE_ERR_SHAPE;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_REDUCTION;
  if (!aligned16(x) || !aligned16(W) || (H * (int64_t)esize(dt)) % 16 != 0) return FLCE_ERR_ALIGN;
  return FLCE_OK;
}

}  // namespace

int flce::device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

extern "C" {

const char* flce_status_string(flce_status s) {
  switch (s) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_NULL: return "FLCE_ERR_NULL: a required pointer is NULL";
    case FLCE_ERR_SHAPE:
      return "FLCE_ERR_SHAPE: N, H and V must lie in [1, 2^30], and H and V (rounded up to 256) times the element "
             "size may not exceed 8 MiB";
    case FLCE_ERR_DTYPE: return "FLCE_ERR_DTYPE: unknown element type";
    case FLCE_ERR_REDUCTION: return "FLCE_ERR_REDUCTION: unknown reduction";
    case FLCE_ERR_ALIAS: return "FLCE_ERR_ALIAS: an output overlaps an input, another output or the workspace";
    case FLCE_ERR_ALIGN: return "FLCE_ERR_ALIGN: x and W must be 16-byte aligned and H * sizeof(dtype) a multiple of 16";
    case FLCE_ERR_WORKSPACE: return "FLCE_ERR_WORKSPACE: workspace missing or too small";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP: a HIP kernel launch failed";
    case FLCE_ERR_SCRATCH:
      return "FLCE_ERR_SCRATCH: these sizes need more forward workspace than the library's static scratch "
             "(FLCE_STATIC_SCRATCH_BYTES, 16 MiB); use flce_forward with a workspace";
  }
  return "FLCE: unknown status";
}

size_t flce_forward_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt) {
  if (!dims_ok(N, H, V) || !dtype_ok(dt) || !rows_ok(H, V, dt)) return 0;
  return plan_forward(N, V).total;
}

size_t flce_backward_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt) {
  if (!dims_ok(N, H, V) || !dtype_ok(dt) || !rows_ok(H, V, dt)) return 0;
  return plan_backward_for(N, H, V, dt, (int64_t)(kDefaultPanelBytes / esize(dt)), kPanelGroup).total;
}

size_t flce_backward_min_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt) {
  if (!dims_ok(N, H, V) || !dtype_ok(dt) || !rows_ok(H, V, dt)) return 0;
  return plan_backward_for(N, H, V, dt, int64_t(kTile) * kTile).total;
}

flce_status flce_forward(const void* x, const void* W, const int64_t* target, int64_t N, int64_t H, int64_t V,
                         flce_dtype dt, flce_reduction reduction, float* loss, float* lse, float* target_logit,
                         void* ws, size_t ws_bytes, void* hip_stream) {
  return flce_forward_timed(x, W, target, N, H, V, dt, reduction, loss, lse, target_logit, ws, ws_bytes, hip_stream,
                            nullptr);
}

flce_status flce_forward_timed(const void* x, const void* W, const int64_t* target, int64_t N, int64_t H, int64_t V,
                               flce_dtype dt, flce_reduction reduction, float* loss, float* lse, float* target_logit,
                               void* ws, size_t ws_bytes, void* hip_stream, flce_timing* timing) {
  flce_status st = check_common(x, W, target, N, H, V, dt, reduction);
  if (st != FLCE_OK) return st;
  if (!loss || !lse) return FLCE_ERR_NULL;
  const FwdPlan p = plan_forward(N, V);
  const size_t es = esize(dt);
  const Range in[3] = {{x, (size_t)N * H * es}, {W, (size_t)V * H * es}, {target, 8 * (size_t)N}};
  const Range out[3] = {{loss, 4}, {lse, 4 * (size_t)N}, {target_logit, 4 * (size_t)N}};
  if (any_alias(in, 3, out, 3, Range{ws, ws_bytes})) return FLCE_ERR_ALIAS;
  if (!ws || ws_bytes < p.total) return FLCE_ERR_WORKSPACE;

  char* base = (char*)ws;
  float* zt = target_logit ? target_logit : (float*)(base + p.off_zt);
  const double scale = reduction == FLCE_MEAN ? 1.0 / (double)N : 1.0;
  flce::Recorder rec{timing, (hipStream_t)hip_stream, hipSuccess};
  rec.start();
  hipError_t e = flce::launch_forward((int)dt, p, x, W, target, (int)N, (int)H, (int)V, (float*)(base + p.off_m),
                                      (float*)(base + p.off_s), zt, lse, (double*)(base + p.off_blk), scale, loss,
                                      (hipStream_t)hip_stream, rec);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int64_t flce_forward_noalloc_max_tokens(int64_t V) {
  if (V < 1 || V > kMaxDim) return 0;
  // the workspace grows with N (splits level off at the minimum): largest N that fits
  int64_t lo = 0, hi = kMaxDim;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (plan_forward(mid, V).total <= (size_t)FLCE_STATIC_SCRATCH_BYTES)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

flce_status flce_forward_noalloc(const void* x, const void* W, const int64_t* target, int64_t N, int64_t H,
                                 int64_t V, flce_dtype dt, flce_reduction reduction, float* loss, float* lse,
                                 float* target_logit, void* hip_stream) {
  flce_status st = check_common(x, W, target, N, H, V, dt, reduction);
  if (st != FLCE_OK) return st;
  if (!loss || !lse) return FLCE_ERR_NULL;
  const FwdPlan p = plan_forward(N, V);
  const size_t es = esize(dt);
  const Range in[3] = {{x, (size_t)N * H * es}, {W, (size_t)V * H * es}, {target, 8 * (size_t)N}};
  const Range out[3] = {{loss, 4}, {lse, 4 * (size_t)N}, {target_logit, 4 * (size_t)N}};
  if (any_alias(in, 3, out, 3, Range{nullptr, 0})) return FLCE_ERR_ALIAS;
  if (p.total > (size_t)FLCE_STATIC_SCRATCH_BYTES) return FLCE_ERR_SCRATCH;
  // The static scratch's device address (never its host-side name).  Nothing the
  // forward keeps there must start at zero: every split partial is written before
  // it is read, and target logits are written by their one owner or set to NaN.
  void* sp = nullptr;
  if (flce::static_scratch(&sp) != hipSuccess) return FLCE_ERR_HIP;
  char* base = (char*)sp;
  float* zt = target_logit ? target_logit : (float*)(base + p.off_zt);
  const double scale = reduction == FLCE_MEAN ? 1.0 / (double)N : 1.0;
  flce::Recorder rec{nullptr, (hipStream_t)hip_stream, hipSuccess};
  hipError_t e = flce::launch_forward((int)dt, p, x, W, target, (int)N, (int)H, (int)V, (float*)(base + p.off_m),
                                      (float*)(base + p.off_s), zt, lse, (double*)(base + p.off_blk), scale, loss,
                                      (hipStream_t)hip_stream, rec);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

flce_status flce_backward(const void* x, const void* W, const int64_t* target, const float* lse,
                          const float* grad_loss, int64_t N, int64_t H, int64_t V, flce_dtype dt,
                          flce_reduction reduction, void* grad_x, void* grad_W, void* ws, size_t ws_bytes,
                          void* hip_stream) {
  return flce_backward_timed(x, W, target, lse, grad_loss, N, H, V, dt, reduction, grad_x, grad_W, ws, ws_bytes,
                             hip_stream, nullptr);
}

flce_status flce_backward_timed(const void* x, const void* W, const int64_t* target, const float* lse,
                                const float* grad_loss, int64_t N, int64_t H, int64_t V, flce_dtype dt,
                                flce_reduction reduction, void* grad_x, void* grad_W, void* ws, size_t ws_bytes,
                                void* hip_stream, flce_timing* timing) {
  flce_status st = check_common(x, W, target, N, H, V, dt, reduction);
  if (st != FLCE_OK) return st;
  if (!lse || !grad_loss || !grad_x || !grad_W) return FLCE_ERR_NULL;
  const size_t es = esize(dt);
  const Range in[5] = {{x, (size_t)N * H * es},
                       {W, (size_t)V * H * es},
                       {target, 8 * (size_t)N},
                       {lse, 4 * (size_t)N},
                       {grad_loss, 4}};
  const Range out[2] = {{grad_x, (size_t)N * H * es}, {grad_W, (size_t)V * H * es}};
  if (any_alias(in, 5, out, 2, Range{ws, ws_bytes})) return FLCE_ERR_ALIAS;
  BwdPlan p;
  if (!ws || !plan_backward(N, H, V, dt, ws_bytes, &p)) return FLCE_ERR_WORKSPACE;
  p.max_workgroups = flce::device_cu_count();

  char* base = (char*)ws;
  const float red_scale = reduction == FLCE_MEAN ? (float)(1.0 / (double)N) : 1.0f;
  flce::Recorder rec{timing, (hipStream_t)hip_stream, hipSuccess};
  rec.start();
  hipError_t e = flce::launch_backward((int)dt, p, x, W, target, lse, grad_loss, red_scale, (int)N, (int)H, (int)V,
                                       grad_x, grad_W, base + p.off_panel, (float*)(base + p.off_gx),
                                       (float*)(base + p.off_gw), (float*)(base + p.off_gxpart),
                                       (float*)(base + p.off_tail), (int*)(base + p.off_flags), (hipStream_t)hip_stream,
                                       rec);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

size_t flce_backward_chunked_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt, int64_t chunk_tokens) {
  if (!dims_ok(N, H, V) || !dtype_ok(dt) || !rows_ok(H, V, dt) || chunk_tokens < 1) return 0;
  return plan_backward_chunked(N, H, V, dt, chunk_tokens).total;
}

flce_status flce_backward_chunked(const void* x, const void* W, const int64_t* target, const float* lse,
                                  const float* grad_loss, int64_t N, int64_t H, int64_t V, flce_dtype dt,
                                  flce_reduction reduction, int64_t chunk_tokens, void* grad_x, void* grad_W,
                                  void* ws, size_t ws_bytes, void* hip_stream, flce_timing* timing) {
  flce_status st = check_common(x, W, target, N, H, V, dt, reduction);
  if (st != FLCE_OK) return st;
  if (chunk_tokens < 1) return FLCE_ERR_SHAPE;
  if (!lse || !grad_loss || !grad_x || !grad_W) return FLCE_ERR_NULL;
  const size_t es = esize(dt);
  const Range in[5] = {{x, (size_t)N * H * es},
                       {W, (size_t)V * H * es},
                       {target, 8 * (size_t)N},
                       {lse, 4 * (size_t)N},
                       {grad_loss, 4}};
  const Range out[2] = {{grad_x, (size_t)N * H * es}, {grad_W, (size_t)V * H * es}};
  if (any_alias(in, 5, out, 2, Range{ws, ws_bytes})) return FLCE_ERR_ALIAS;
  BwdPlan p = plan_backward_chunked(N, H, V, dt, chunk_tokens);
  if (!ws || ws_bytes < p.total) return FLCE_ERR_WORKSPACE;
  p.max_workgroups = flce::device_cu_count();

  char* base = (char*)ws;
  const float red_scale = reduction == FLCE_MEAN ? (float)(1.0 / (double)N) : 1.0f;
  flce::Recorder rec{timing, (hipStream_t)hip_stream, hipSuccess};
  rec.start();
  hipError_t e = flce::launch_backward((int)dt, p, x, W, target, lse, grad_loss, red_scale, (int)N, (int)H, (int)V,
                                       grad_x, grad_W, base + p.off_panel, (float*)(base + p.off_gx),
                                       (float*)(base + p.off_gw), (float*)(base + p.off_gxpart),
                                       (float*)(base + p.off_tail), (int*)(base + p.off_flags), (hipStream_t)hip_stream,
                                       rec);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// Workspace of the float32-atomic backward: kAtomicWGs dlogit tiles (one per
// workgroup of its persistent grid), then for bfloat16 the float32 grad_x [N, H]
// and grad_W [V, H] accumulators.
constexpr int kAtomicWGs = 256;
struct AtomicPlan {
  size_t off_dtile, off_gx, off_gw, total;
};
AtomicPlan plan_backward_atomic(int64_t N, int64_t H, int64_t V, flce_dtype dt) {
  AtomicPlan p{};
  size_t o = 0;
  p.off_dtile = o;
  o = align_up(o + esize(dt) * (size_t)kAtomicWGs * kTile * kTile, 256);
  const bool bf = dt == FLCE_BF16;
  p.off_gx = o;
  o = align_up(o + (bf ? sizeof(float) * (size_t)N * H : 0), 256);
  p.off_gw = o;
  o = align_up(o + (bf ? sizeof(float) * (size_t)V * H : 0), 256);
  p.total = o;
  return p;
}

size_t flce_backward_atomic_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt) {
  if (!dims_ok(N, H, V) || !dtype_ok(dt) || !rows_ok(H, V, dt)) return 0;
  return plan_backward_atomic(N, H, V, dt).total;
}

flce_status flce_backward_atomic(const void* x, const void* W, const int64_t* target, const float* lse,
                                 const float* grad_loss, int64_t N, int64_t H, int64_t V, flce_dtype dt,
                                 flce_reduction reduction, void* grad_x, void* grad_W, void* ws, size_t ws_bytes,
                                 void* hip_stream, flce_timing* timing) {
  flce_status st = check_common(x, W, target, N, H, V, dt, reduction);
  if (st != FLCE_OK) return st;
  if (!lse || !grad_loss || !grad_x || !grad_W) return FLCE_ERR_NULL;
  const size_t es = esize(dt);
  const Range in[5] = {{x, (size_t)N * H * es},
                       {W, (size_t)V * H * es},
                       {target, 8 * (size_t)N},
                       {lse, 4 * (size_t)N},
                       {grad_loss, 4}};
  const Range out[2] = {{grad_x, (size_t)N * H * es}, {grad_W, (size_t)V * H * es}};
  if (any_alias(in, 5, out, 2, Range{ws, ws_bytes})) return FLCE_ERR_ALIAS;
  const AtomicPlan p = plan_backward_atomic(N, H, V, dt);
  if (!ws || ws_bytes < p.total) return FLCE_ERR_WORKSPACE;
  char* base = (char*)ws;
  const float red_scale = reduction == FLCE_MEAN ? (float)(1.0 / (double)N) : 1.0f;
  flce::Recorder rec{timing, (hipStream_t)hip_stream, hipSuccess};
  rec.start();
  hipError_t e = flce::launch_backward_atomic(
      (int)dt, x, W, target, lse, grad_loss, red_scale, (int)N, (int)H, (int)V, grad_x, grad_W, base + p.off_dtile,
      (float*)(base + p.off_gx), (float*)(base + p.off_gw), std::min(kAtomicWGs, flce::device_cu_count()),
      (hipStream_t)hip_stream, rec);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

size_t flce_forward_backward_workspace_bytes(int64_t N, int64_t H, int64_t V, flce_dtype dt) {
  if (!dims_ok(N, H, V) || !dtype_ok(dt) || !rows_ok(H, V, dt)) return 0;
  return 256 + std::max(plan_forward(N, V).total,
                        plan_backward_for(N, H, V, dt, (int64_t)(kDefaultPanelBytes / esize(dt)), kPanelGroup).total);
}

flce_status flce_forward_backward(const void* x, const void* W, const int64_t* target, int64_t N, int64_t H,
                                  int64_t V, flce_dtype dt, flce_reduction reduction, const float* grad_loss,
                                  float* loss, float* lse, void* grad_x, void* grad_W, void* ws, size_t ws_bytes,
                                  void* hip_stream) {
  flce_status st = check_common(x, W, target, N, H, V, dt, reduction);
  if (st != FLCE_OK) return st;
  if (!loss || !lse || !grad_x || !grad_W) return FLCE_ERR_NULL;
  const size_t es = esize(dt);
  const Range in[4] = {{x, (size_t)N * H * es}, {W, (size_t)V * H * es}, {target, 8 * (size_t)N}, {grad_loss, 4}};
  const Range out[4] = {{loss, 4}, {lse, 4 * (size_t)N}, {grad_x, (size_t)N * H * es}, {grad_W, (size_t)V * H * es}};
  if (any_alias(in, 4, out, 4, Range{ws, ws_bytes})) return FLCE_ERR_ALIAS;
  // [0, 256): the implicit grad_loss; then one region the two phases share
  // (the forward's partials are dead once its last kernel has run).
  const FwdPlan fp = plan_forward(N, V);
  BwdPlan bp;
  if (!ws || ws_bytes < 256 + fp.total || !plan_backward(N, H, V, dt, ws_bytes - 256, &bp))
    return FLCE_ERR_WORKSPACE;
  bp.max_workgroups = flce::device_cu_count();
  char* base = (char*)ws + 256;
  hipStream_t s = (hipStream_t)hip_stream;
  flce::Recorder rec{nullptr, s, hipSuccess};
  const float* gl = grad_loss;
  hipError_t e = hipSuccess;
  if (!gl) {
    e = flce::launch_fill((float*)ws, 1.0f, s, rec);
    gl = (const float*)ws;
  }
  if (e == hipSuccess)
    e = flce::launch_forward((int)dt, fp, x, W, target, (int)N, (int)H, (int)V, (float*)(base + fp.off_m),
                             (float*)(base + fp.off_s), (float*)(base + fp.off_zt), lse,
                             (double*)(base + fp.off_blk), reduction == FLCE_MEAN ? 1.0 / (double)N : 1.0, loss, s,
                             rec);
  if (e == hipSuccess)
    e = flce::launch_backward((int)dt, bp, x, W, target, lse, gl,
                              reduction == FLCE_MEAN ? (float)(1.0 / (double)N) : 1.0f, (int)N, (int)H, (int)V,
                              grad_x, grad_W, base + bp.off_panel, (float*)(base + bp.off_gx),
                              (float*)(base + bp.off_gw), (float*)(base + bp.off_gxpart), (float*)(base + bp.off_tail),
                              (int*)(base + bp.off_flags), s, rec);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

}  // extern "C"
