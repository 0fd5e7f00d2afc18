// Internal interface between the host layer (argument checks, planning,
// workspace carving) and the kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

#include "flce.h"

namespace flce {

constexpr int kTile = 256;  // square output tile of every contraction kernel

struct FwdPlan {
  int tiles_tok;        // token tiles of kTile
  int splits;           // vocabulary splits (workgroups per token tile)
  int tiles_per_split;  // vocabulary tiles per split
  int Np;               // tiles_tok * kTile
  int nb;               // combine blocks (64 tokens each)
  size_t off_m, off_s, off_zt, off_blk, total;  // workspace carving (bytes); off_blk: nb doubles, then a ticket
};

struct BwdPlan {
  int Nc, n_chunks;         // tokens per chunk, chunks
  int Vb, Vbp, n_panels;    // vocabulary per panel, padded, panels
  int gx_group;             // panels kept in the panel buffer (one [Ncp, Vbp] block each); grad_x runs once per group
  int Ncp;                  // Nc padded to kTile
  int gx_splits;            // grad_x K splits per launch (1: none), partial sums in gxpart
  int tail_cap;             // float32 256 x 256 partial tiles for split tail tiles of grad_W launches
  int slots;                // balanced launches: float32 256 x 256 partial-sum slots (one per workgroup) and flags
  size_t off_panel, off_gx, off_gw, off_gxpart, off_tail, off_flags, total;  // workspace carving (bytes); 0-sized parts unused
  size_t gx_bytes, gw_bytes, gxpart_bytes, tail_bytes;
  int max_workgroups;                       // persistent grid size: one workgroup per CU
};

// Compute units of the current HIP device (cached per device; 256 if the query fails).
int device_cu_count();

// Records the caller's timing events between kernel launches (no-op without one).
struct Recorder {
  flce_timing* t;
  hipStream_t s;
  hipError_t err;
  bool started = false;
  // Record events[0] once per library call (later phases of a combined call keep
  // counting from where the previous one stopped).
  void start() {
    if (t && !started) {
      started = true;
      t->n_launches = 0;
      if (t->n_events > 0) record(t->events[0]);
    }
  }
  void after(int kind) {
    if (!t) return;
    const int k = t->n_launches++;
    if (k + 1 < t->n_events) {
      if (t->kinds) t->kinds[k] = kind;
      record(t->events[k + 1]);
    }
  }
  void record(void* ev) {
    const hipError_t e = hipEventRecord((hipEvent_t)ev, s);
    if (e != hipSuccess && err == hipSuccess) err = e;
  }
};

hipError_t launch_forward(int dt, const FwdPlan& p, const void* x, const void* W, const int64_t* target, int N,
                          int H, int V, float* part_m, float* part_s, float* zt, float* lse, double* block_loss,
                          double scale, float* loss, hipStream_t st, Recorder& rec);

hipError_t launch_fill(float* p, float v, hipStream_t st, Recorder& rec);

// Float32-atomic backward (comparison): zero the float32 accumulators (grad_x and
// grad_W themselves for float32), one persistent launch over the (token tile,
// vocabulary tile) pairs, then casts to bfloat16.  dtile: max_wgs 256 x 256 tiles.
hipError_t launch_backward_atomic(int dt, const void* x, const void* W, const int64_t* target, const float* lse,
                                  const float* grad_loss, float red_scale, int N, int H, int V, void* gx, void* gw,
                                  void* dtile, float* gx_acc, float* gw_acc, int max_wgs, hipStream_t st,
                                  Recorder& rec);

// Device address, on the current device, of the library's static forward scratch
// (FLCE_STATIC_SCRATCH_BYTES), looked up once per device.
hipError_t static_scratch(void** out);

hipError_t launch_backward(int dt, const BwdPlan& p, const void* x, const void* W, const int64_t* target,
                           const float* lse, const float* grad_loss, float red_scale, int N, int H, int V, void* gx,
                           void* gw, void* panel, float* gx_acc, float* gw_acc, float* gx_part, float* tail,
                           int* flags, hipStream_t st, Recorder& rec);

// Balanced schedules of the gradient launches (a launch of T > G tiles on G
// workgroups, T % G a nonzero multiple of G / 8, cuts its last T - (T / G - 1) G
// tiles evenly along K over all workgroups, keeping each XCD's workgroups at
// one K offset; the partial sums of a tile shared by two workgroups pass
// through one slot per workgroup); the dlogit launches only in builds with
// FLCE_BALANCE_DLOGITS.  Otherwise the partial last round is split into K pieces.
#ifndef FLCE_BALANCE
#define FLCE_BALANCE 1
#endif
#ifndef FLCE_BALANCE_DLOGITS
#define FLCE_BALANCE_DLOGITS 0
#endif
constexpr bool kBalance = FLCE_BALANCE != 0;
constexpr bool kBalanceDlogits = kBalance && FLCE_BALANCE_DLOGITS != 0;
__host__ __device__ inline bool balanced_launch(int64_t T, int64_t G) {
  return G > 0 && G % 8 == 0 && T > G && T % G != 0 && (T % G) % (G / 8) == 0;
}

// Split of the last, partial round of a persistent launch of T tiles of K
// entries along K on `cus` workgroups: the T - T % cus tiles of the full rounds
// are done whole; the tail (T % cus tiles) is cut along K into kts pieces each
// when at least two pieces per tail tile fit in the workgroups and in `cap`
// partial-tile buffers (kts = 0: no split).  A launch of few tiles (T <= cus / 2,
// at least 1024 entries of K) is all tail: each tile cut into kts >= 2 pieces,
// so that the idle CUs share its work.  Shared by the planner (workspace size)
// and the launcher.
struct TailSplit {
  int full, tail, kts;
};
inline TailSplit tail_split(int64_t T, int64_t cus, int cap, int64_t K) {
  TailSplit s{(int)T, 0, 0};
  if (cus <= 0 || T <= 0) return s;
  const int64_t room = std::min<int64_t>(cus, cap);
  if (2 * T <= cus && K >= 1024) {
    const int64_t kts = room / T;
    if (kts >= 2) s = TailSplit{0, (int)T, (int)kts};
    return s;
  }
  const int64_t G = std::min<int64_t>(T, cus);
  const int64_t tail = T % G;
  if (tail == 0) return s;
  const int64_t kts = std::min<int64_t>(G, cap) / tail;
  if (kts < 2) return s;
  s.full = (int)(T - tail);
  s.tail = (int)tail;
  s.kts = (int)kts;
  return s;
}

}  // namespace flce
