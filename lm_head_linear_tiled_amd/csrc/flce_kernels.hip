// HIP kernels of fused linear + cross-entropy for gfx950.
//
// Forward (helion PR #1268, PR description: tiled matmul plus online softmax for
// the log-sum-exp and the target logit; the log-sum-exp is kept):
//   fwd_partial   one workgroup per (token tile, vocabulary split); for each
//                 vocabulary tile of its split it forms the logit tile
//                 S^T = W_tile . x_tile^T with MFMA and folds it into a running
//                 (max, sum of exp) per token held in registers; the target logit
//                 is picked out of the one tile that holds it.  The split exists so
//                 that small token counts still fill all 256 CUs (Liger-Kernel PR
//                 #928 thread: fusing the logits and the softmax leaves too little
//                 parallelism at small shapes).
//   fwd_combine   merges the split partials into lse and the per-token loss,
//                 reduces the losses per block in a fixed order, and its last
//                 block sums the block partials in a fixed order into the loss.
// Backward (helion PR #1268: the backward recomputes the logits; the dlogits
// drive both gradients; Liger-Kernel PR #928: zero the out-of-range dlogits):
//   bwd_dlogits   recomputes a logit tile S^T = W_tile . x_tile^T and writes
//                 D = s (exp(S - lse) - onehot) into a bounded panel [token][vocab],
//                 exactly 0 outside i < N, v < V;
//   bwd_grad_w    grad_W[v, h] (+)= sum_i D[i, v] x[i, h] over the panel's tokens;
//   bwd_grad_x    grad_x[i, h] (+)= sum_v D[i, v] W[v, h] over the panel's vocabulary.
// The three backward kernels compute transposed tiles (the output's contiguous
// dimension on the accumulator rows) and write them through the LDS stage their
// last K slice frees (staged_epilogue), as whole 128-byte lines.
#include <mutex>

#include "gemm_core.h"
#include "flce_launch.h"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#ifndef FLCE_BK_BF16
#define FLCE_BK_BF16 64
#endif
#ifndef FLCE_NSTAGE_BF16
#define FLCE_NSTAGE_BF16 2
#endif
#ifndef FLCE_BK_F32
#define FLCE_BK_F32 32
#endif
#ifndef FLCE_NSTAGE_F32
#define FLCE_NSTAGE_F32 2
#endif
// MFMA output block of the bfloat16 kernels: 16 (v_mfma_f32_16x16x32_bf16) or 32
// (v_mfma_f32_32x32x16_bf16); float32 always uses 32 x 32 blocks
#ifndef FLCE_MI_FWD
#define FLCE_MI_FWD 32
#endif
#ifndef FLCE_WAVES_M
#define FLCE_WAVES_M 4
#endif
#ifndef FLCE_WAVES_N
#define FLCE_WAVES_N 2
#endif

// K slice width and LDS pipeline depth per element type: 128-byte K slices in two
// stages (one slice in flight while one is multiplied; deeper pipelines measured
// no faster), and the wave grid of a 256 x 256 tile.
constexpr int kThreads = 64 * FLCE_WAVES_M * FLCE_WAVES_N;
// The forward's wave grid on its own (measurement builds: 2 x 2 = one wave per
// SIMD with a 128 x 128 sub-tile each)
#ifndef FLCE_FWD_WAVES_M
#define FLCE_FWD_WAVES_M FLCE_WAVES_M
#endif
#ifndef FLCE_FWD_WAVES_N
#define FLCE_FWD_WAVES_N FLCE_WAVES_N
#endif
constexpr int kFwdThreads = 64 * FLCE_FWD_WAVES_M * FLCE_FWD_WAVES_N;

template <typename T>
struct Cfg;
template <>
struct Cfg<bf16_t> {
  static constexpr int BK = FLCE_BK_BF16;
  static constexpr int NS = FLCE_NSTAGE_BF16;
  static constexpr int MI_FWD = FLCE_MI_FWD;  // MFMA block of the forward
};
template <>
struct Cfg<float> {
  static constexpr int BK = FLCE_BK_F32;
  static constexpr int NS = FLCE_NSTAGE_F32;
  static constexpr int MI_FWD = 32;
};

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kFwdThreads) void fwd_partial(const T* __restrict__ x, const T* __restrict__ W,
                                                   const int64_t* __restrict__ target, int N, int H, int V,
                                                   int tiles_tok, int tiles_per_split, int Np,
                                                   float* __restrict__ part_m, float* __restrict__ part_s,
                                                   float* __restrict__ zt_out, unsigned int* __restrict__ ticket) {
  // S^T tile: rows = vocabulary (A = W, K-major), cols = tokens (B = x, K-major).
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_FWD_WAVES_M, FLCE_FWD_WAVES_N,
                   STAGE_DMA, false, Cfg<T>::MI_FWD>
      G;
  constexpr int MI = G::MI;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];

  // the combine kernel's ticket starts from zero (it runs after this kernel)
  if (blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0u;
  const int lid = xcd_grouped_id((int)blockIdx.x, (int)gridDim.x);
  int tt, split;
  grouped_tile(lid, tiles_tok, (int)gridDim.x / tiles_tok, tt, split);
  const int n0 = tt * kTile;
  const int tiles_v = (V + kTile - 1) / kTile;
  const int vt_begin = split * tiles_per_split;
  const int vt_end = min(tiles_v, vt_begin + tiles_per_split);

  const int l = (int)threadIdx.x & 63;
  // wave-uniform: kept in scalar registers
  const int wm = __builtin_amdgcn_readfirstlane(G::wave_m()), wn = __builtin_amdgcn_readfirstlane(G::wave_n());

  const Operand<T> A{W, H, V, H};
  const Operand<T> B{x, H, N, H};

  // per column block j: this lane's token n0 + WN wn + MI j + l % MI
  float mrun[G::FN], srun[G::FN];
  int tgt[G::FN];
#pragma unroll
  for (int j = 0; j < G::FN; ++j) {
    mrun[j] = -INFINITY;
    srun[j] = 0.f;
    const int tok = n0 + wn * G::WN + j * MI + G::acc_n(l);
    tgt[j] = tok < N ? (int)min<int64_t>(max<int64_t>(target[tok], -1), (int64_t)V) : -1;
  }

  typename G::Acc acc;
  auto next = [&](int j, int& m0, int& tn0) {
    m0 = (vt_begin + j) * kTile;
    tn0 = n0;
    return vt_begin + j < vt_end;
  };
  auto fold = [&](typename G::Acc& a, int m0, int, char*) {
    // interior vocabulary tile: no row masks, and the max taken before the log2(e)
    // scaling (a positive factor, so the same value)
    const bool interior = m0 + kTile <= V;
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      float tmax = -INFINITY;
      if (interior) {
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int r = 0; r < G::NR; ++r) tmax = fmaxf(tmax, a[i][j][r]);
        tmax *= kLog2e;
      } else {
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int r = 0; r < G::NR; ++r) {
            const int v = m0 + wm * G::WM + i * MI + G::acc_m(r, l);
            const float val = v < V ? a[i][j][r] * kLog2e : -INFINITY;
            tmax = fmaxf(tmax, val);
          }
      }
      const float mnew = fmaxf(mrun[j], tmax);
      if (mnew != -INFINITY) {
        float ssum = 0.f;
        if (interior) {
#pragma unroll
          for (int i = 0; i < G::FM; ++i)
#pragma unroll
            for (int r = 0; r < G::NR; ++r) ssum += __builtin_amdgcn_exp2f(__builtin_fmaf(a[i][j][r], kLog2e, -mnew));
        } else {
#pragma unroll
          for (int i = 0; i < G::FM; ++i)
#pragma unroll
            for (int r = 0; r < G::NR; ++r) {
              const int v = m0 + wm * G::WM + i * MI + G::acc_m(r, l);
              ssum += v < V ? __builtin_amdgcn_exp2f(a[i][j][r] * kLog2e - mnew) : 0.f;
            }
        }
        srun[j] = srun[j] * __builtin_amdgcn_exp2f(mrun[j] - mnew) + ssum;
        mrun[j] = mnew;
      }
      // Target logit: exactly one lane of one workgroup holds (t, tok); most
      // waves hold none in a given tile and skip the search.
      const int local0 = tgt[j] - (m0 + wm * G::WM);
      if (__any(local0 >= 0 && local0 < G::WM)) {
#pragma unroll
        for (int i = 0; i < G::FM; ++i) {
          const int local = local0 - i * MI;
          // the lane holding block row `local` of this lane's column, and its register
          const bool mine = MI == 32 ? ((local >> 2) & 1) == (l >> 5) : (local >> 2) == (l >> 4);
          if (local >= 0 && local < MI && mine) {
            const int rr = MI == 32 ? (local >> 3) * 4 + (local & 3) : (local & 3);
            // element rr of the lane's NR accumulators, by a select tree on the
            // bits of rr (log2 NR lane masks rather than NR)
            float v[G::NR];
#pragma unroll
            for (int r = 0; r < G::NR; ++r) v[r] = a[i][j][r];
#pragma unroll
            for (int b = 0, w = G::NR / 2; w > 0; ++b, w >>= 1) {
              const bool hi = (rr >> b) & 1;
#pragma unroll
              for (int k = 0; k < w; ++k) v[k] = hi ? v[2 * k + 1] : v[2 * k];
            }
            zt_out[n0 + wn * G::WN + j * MI + G::acc_n(l)] = v[0];
          }
        }
      }
    }
  };
  G::run_tiles(A, B, H, lds, acc, next, fold);

  // Merge the lane groups that hold the same tokens (different vocabulary rows)
  // ...
#pragma unroll
  for (int sh = MI; sh < 64; sh <<= 1) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const float mo = __shfl_xor(mrun[j], sh);
      const float so = __shfl_xor(srun[j], sh);
      const float M = fmaxf(mrun[j], mo);
      if (M != -INFINITY) {
        srun[j] = srun[j] * __builtin_amdgcn_exp2f(mrun[j] - M) + so * __builtin_amdgcn_exp2f(mo - M);
        mrun[j] = M;
      }
    }
  }
  // ... then the WGM waves that share the token columns, in a fixed order.
  float* sm = reinterpret_cast<float*>(lds);  // [WGM - 1][BN] max, then [WGM - 1][BN] sum
  constexpr int SM = (G::WGM - 1) * kTile;
  if (wm > 0 && l < MI) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      sm[(wm - 1) * kTile + wn * G::WN + j * MI + l] = mrun[j];
      sm[SM + (wm - 1) * kTile + wn * G::WN + j * MI + l] = srun[j];
    }
  }
  __syncthreads();
  if (wm == 0 && l < MI) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      float M = mrun[j], S = srun[j];
      for (int q = 0; q < G::WGM - 1; ++q) {
        const float mo = sm[q * kTile + wn * G::WN + j * MI + l];
        const float so = sm[SM + q * kTile + wn * G::WN + j * MI + l];
        const float Mn = fmaxf(M, mo);
        if (Mn != -INFINITY) S = S * __builtin_amdgcn_exp2f(M - Mn) + so * __builtin_amdgcn_exp2f(mo - Mn);
        M = Mn;
      }
      const int tok = n0 + wn * G::WN + j * MI + l;
      if (tok < N) {
        part_m[(int64_t)split * Np + tok] = M;
        part_s[(int64_t)split * Np + tok] = S;
      }
    }
  }
}

// One wavefront per 64 tokens: merge the split partials of each token into lse
// and its loss term (a NaN target logit for a target outside [0, V)), sum the
// block's terms in a fixed order; the last block to finish (a ticket counter,
// zeroed by fwd_partial) sums the block sums in a fixed order into the loss.
constexpr int kCombineThreads = 64;
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__global__ __launch_bounds__(kCombineThreads) void fwd_combine(const float* __restrict__ part_m,
                                                               const float* __restrict__ part_s, int splits, int Np,
                                                               int N, int V, const int64_t* __restrict__ target,
                                                               float* __restrict__ zt, float* __restrict__ lse,
                                                               double* __restrict__ block_loss,
                                                               unsigned int* __restrict__ ticket, double scale,
                                                               float* __restrict__ loss) {
  const int i = (int)blockIdx.x * kCombineThreads + (int)threadIdx.x;
  double li = 0.0;
  if (i < N) {
    float M = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) M = fmaxf(M, part_m[(int64_t)s * Np + i]);
    float S = 0.f;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) S += part_s[(int64_t)s * Np + i] * exp2f(part_m[(int64_t)s * Np + i] - M);
    const float l2 = M + log2f(S);
    const float lsei = l2 * kLn2;
    lse[i] = lsei;
    const int64_t t = target[i];
    float z = zt[i];
    if (t < 0 || t >= V) {
      z = __int_as_float(0x7fc00000);
      zt[i] = z;
    }
    li = (double)lsei - (double)z;
  }
  li = wave_sum(li);
  const int nb = (int)gridDim.x;
  if (threadIdx.x == 0) {
    block_loss[blockIdx.x] = li;
    __threadfence();  // the block sum is visible before the ticket is taken
    const unsigned int k = atomicAdd(ticket, 1u);
    li = k == (unsigned int)nb - 1 ? 1.0 : 0.0;  // reused as the "last block" flag
  }
  const bool last = __shfl(li, 0) == 1.0 && nb > 0;
  if (!last) return;
  __threadfence();  // every other block's sum is visible
  double a = 0.0;
  for (int bb = (int)threadIdx.x; bb < nb; bb += kCombineThreads) a += block_loss[bb];
  a = wave_sum(a);
  if (threadIdx.x == 0) loss[0] = (float)(a * scale);
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
// The backward kernels are persistent: one workgroup per CU walks the tiles
// t = lid, lid + G, ... of its launch (lid: XCD-grouped id, G: grid size), each
// tile (tm, tn) taken in the grouped order, so the copy of a tile's first K slice
// overlaps the previous tile's last slice and epilogue.
template <int GM = FLCE_GROUP_M>
__device__ __forceinline__ bool persistent_tile(int j, int tiles_m, int tiles_n, int& tm, int& tn,
                                                int ntiles = -1) {
  const int G = (int)gridDim.x;
  const int t = xcd_grouped_id((int)blockIdx.x, G) + j * G;
  if (t >= (ntiles < 0 ? tiles_m * tiles_n : ntiles)) return false;
  grouped_tile<GM>(t, tiles_m, tiles_n, tm, tn);
  return true;
}

// Schedule of a persistent backward launch over T tiles (taken in the grouped
// order) of KT K slices each, on the G = gridDim.x workgroups.  Unbalanced:
// workgroup lw (XCD-grouped id) takes the whole tiles lw, lw + G, ...
// Balanced (balanced_launch(T, G): T > G, r = T % G a nonzero multiple of
// g = G / 8): the first R = T / G - 1 rounds go the same way, and the T' = G + r
// tiles left form one run of T' KT slices cut evenly into G ranges of at least
// KT slices, range p = [s0, s1) with s0 = T' KT p / G.  A tile of the run is then
// shared by at most two ranges: the head of its K range (from k = 0) ends range
// p, the rest of it starts range p + 1.  Range p = 8 m + x goes to workgroup m
// of XCD x (lw = x g + m).  As T' = g D with D = 8 + r / g, range 8 m + x starts
// at run tile D m + floor(D x / 8) and K slice (D KT x / 8) mod KT, both the
// same for every m: the run's tile u = D m + d is taken as tile d g + m, so at
// any time the g workgroups of an XCD work on g consecutive tiles of the grouped
// order at the same K slice, as in a round of whole tiles, and share their
// operand slices in the XCD's L2.  (KT D x / 8 not a whole number: ranges of one
// XCD start up to a slice apart.)
struct TileSched {
  int T, KT, G, w, R;  // w: the range of a balanced run, else the XCD-grouped id
  int D, g;            // balanced run: tiles per row, rows (= workgroups per XCD)
  int f, k0f;          // ... this range's first run tile and its first slice
  int e, ke;           // ... its last run tile and the end slice within it (1 .. KT)
  __device__ __forceinline__ TileSched(int T_, int KT_, int balance) : T(T_), KT(KT_) {
    G = (int)gridDim.x;
    const int lw = xcd_grouped_id((int)blockIdx.x, G);
    if (balance && balanced_launch(T, G)) {
      R = T / G - 1;
      g = G / 8;
      const int Tp = T - R * G;
      D = Tp / g;
      w = 8 * (lw % g) + lw / g;
      const int64_t tot = (int64_t)Tp * KT;
      const int64_t s0 = tot * w / G, s1 = tot * (w + 1) / G;
      f = (int)(s0 / KT);
      k0f = (int)(s0 - (int64_t)f * KT);
      e = (int)((s1 - 1) / KT);
      ke = (int)(s1 - (int64_t)e * KT);
    } else {
      w = lw;
      R = (T + G - 1) / G;
      D = 1;
      g = 1;
      f = 0;
      k0f = 0;
      e = -1;
      ke = 0;
    }
  }
  // item j: tile t of the grouped order, K slices [k0, k0 + nk)
  __device__ __forceinline__ bool item(int j, int& t, int& k0, int& nk) const {
    if (j < R) {
      t = w + j * G;
      k0 = 0;
      nk = KT;
      return t < T;
    }
    const int u = f + (j - R);
    if (u > e) return false;
    k0 = j == R ? k0f : 0;
    nk = (u == e ? ke : KT) - k0;
    t = R * G + (u % D) * g + u / D;
    return true;
  }
  // the head of a shared tile (finished with the partner's partial sums), and
  // the rest of one (whose partial sums are published), from an item's K offset
  // and slice count
  __device__ __forceinline__ bool head(int kb, int nk) const { return kb == 0 && nk < KT; }
  static __device__ __forceinline__ bool rest(int kb) { return kb > 0; }
};

// Float32 partial sums of a shared tile, handed from the workgroup that computes
// the rest of its K range (publish_partial, slot and flag of its own id) to the
// one that computes the head (take_partial, the same slot: the partner's id).  A
// slot holds every thread's accumulators as 16-byte groups interleaved over the
// workgroup's threads (whole 1 KiB blocks per wave and group), kTile x kTile
// floats for 512 threads.  The slot and its flag are only written and read with
// device-coherent accesses (written through to, and read from, the point where
// the XCDs' caches agree), so no L2 write-back or invalidation is needed: each
// thread waits for its slot stores to complete, the workgroup barrier orders all
// of them before the flag store, and the reader's loads follow its flag load.
// The head's workgroup waits for the flag before its first K slice: the rest is
// the first item of the partner, which depends on nothing, so every wait ends
// (the wait is also bounded: past kSpinCap polls the partial sums are taken as
// they are).  It clears the flag again, so the flags are all 0 after each
// launch; the launcher zeroes them once per backward.
constexpr int kSpinCap = 1 << 20;
constexpr int kCoherent = 16;  // buffer access cache policy: coherent across the device
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float* slots, int w) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(slots + (int64_t)w * kTile * kTile), (short)0,
                                           kTile * kTile * (int)sizeof(float), 0x00020000);
}
template <class G>
__device__ __forceinline__ void publish_partial(const typename G::Acc& acc, float* __restrict__ slots,
                                                int* __restrict__ flags, int w) {
  static_assert(G::NT * G::FM * G::FN * G::NR <= kTile * kTile, "slot size");
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(slots, w);
  const int vo = (int)threadIdx.x * 16;
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int g = 0; g < G::NR / 4; ++g) {
        const int q = (i * G::FN + j) * (G::NR / 4) + g;
        const float4 v = make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, vo, q * G::NT * 16, kCoherent);
      }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's stores are complete
  __syncthreads();                                   // ... and every other thread's
  if (threadIdx.x == 0) __hip_atomic_store(flags + w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class G>
__device__ __forceinline__ void take_partial(typename G::Acc& acc, const float* __restrict__ slots,
                                             int* __restrict__ flags, int w) {
  if (threadIdx.x == 0) {
    int n = 0;
    while (__hip_atomic_load(flags + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 && ++n < kSpinCap)
      __builtin_amdgcn_s_sleep(2);
    __hip_atomic_store(flags + w, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(slots, w);
  const int vo = (int)threadIdx.x * 16;
  // one accumulator block (NR / 4 groups) in flight at a time
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
#pragma unroll
      for (int g = 0; g < G::NR / 4; ++g) {
        const int q = (i * G::FN + j) * (G::NR / 4) + g;
        const float4 v =
            __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, q * G::NT * 16, kCoherent));
        acc[i][j][4 * g] += v.x;
        acc[i][j][4 * g + 1] += v.y;
        acc[i][j][4 * g + 2] += v.z;
        acc[i][j][4 * g + 3] += v.w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// The dlogit kernel splits its waves into copy waves and store waves (its panel
// stores then drain while the next tile runs).
#ifndef FLCE_SPLIT_DLOGITS
#define FLCE_SPLIT_DLOGITS 1
#endif
constexpr bool kSplitDlogits = FLCE_SPLIT_DLOGITS != 0;

// Tile groups of the dlogit and grad_x launches: 8 rows (vocabulary tiles of W,
// hidden tiles of W) per group, measured better there than 4.
#ifndef FLCE_GROUP_M_WIDE
#define FLCE_GROUP_M_WIDE 8
#endif

// Four consecutive float outputs as 4 elements of T (bfloat16: hardware
// round-to-nearest-even conversion), and the 16-byte LDS accesses of the
// dlogit staging below.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){a, b}, bf16x2v_t));
}

// Tile epilogue through the spare LDS stage.  A wave's 64 x 128 accumulator
// sub-tile (M side: four consecutive rows per lane and accumulator group; N side:
// one column per lane) is written to 8 KiB of LDS per wave, a round of N columns
// at a time, and read back so that each lane holds 16 contiguous bytes of one
// output row n, along which M is contiguous in memory: the global accesses then
// cover whole 128-byte lines.
//   val(i, j, g, d): d[0..3] = values of rows 32 i + 8 g + 4 (l / 32) + 0..3 and
//                    column 32 j + l % 32 of the sub-tile (l: lane)
//   out(n, m, v):    n in [0, 128), m in [0, 64) a multiple of 16 / sizeof(S),
//                    v = 16 bytes: elements m .. of row n, as S
// LDS slots are XOR-swizzled so that the writes (32 lanes of different n) and the
// reads (whole rows) are free of bank conflicts.  Starts with a workgroup barrier.
// PAIRW = 0: every wave stores its own sub-tile, out(n, m, v).  PAIRW = the
// workgroup's wave count: only the second half of the waves store, wave w the
// sub-tiles of waves w - PAIRW / 2 and w, handed over through LDS (a barrier
// after each round's writes and between rounds), out(src, n, m, v) with src the
// wave whose sub-tile it is.
//   fix(j, tb, poke): called for each column block j of a round after its values
//   are in LDS (tb: the block's first row of the round); poke(t, m, x) replaces
//   the element of row t of the round, M index m, of this lane's own region by x.
template <typename S, int FM, int FN, int PAIRW = 0, class Val, class Out, class Fix>
__device__ __forceinline__ void staged_epilogue(char* spare, Val&& val, Out&& out, Fix&& fix) {
  static_assert(FM == 2 && FN == 4, "64 x 128 wave sub-tile");
  constexpr bool BF = sizeof(S) == 2;
  constexpr int RB = 64 * (int)sizeof(S);  // bytes of one output row of the sub-tile
  constexpr int TR = 8192 / RB;            // rows per round: 64 (bf16) or 32 (fp32)
  constexpr int JR = TR / 32;              // accumulator column blocks per round
  // The lane id is hidden from the optimiser here, so the per-lane row offsets
  // below are recomputed in each epilogue instead of being kept live across the
  // tile loop: kept, they are spilled, and every reload from scratch memory waits
  // for all of the wave's outstanding global stores.
  int l = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  char* sc = spare + ((int)threadIdx.x >> 6) * 8192;
  // every wave has read its last fragments from spare (the copies still in flight
  // go to the other stage, so no vmcnt wait here)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int rd = 0; rd < FN / JR; ++rd) {
#pragma unroll
    for (int jj = 0; jj < JR; ++jj) {
      const int tl = jj * 32 + (l & 31);  // row of the round
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ml = i * 32 + 8 * g + 4 * (l >> 5);  // elements ml .. ml + 3 of the row
          float d[4];
          val(i, rd * JR + jj, g, d);
          if constexpr (BF) {
            // 8-byte half of a 16-byte slot: slot ^ (tl/2 % 8), half ^ (tl/16 % 2)
            const int slot = (ml >> 3) ^ ((tl >> 1) & 7);
            const int half = ((ml >> 2) & 1) ^ ((tl >> 4) & 1);
            *reinterpret_cast<uint2*>(sc + tl * RB + slot * 16 + half * 8) =
                make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
          } else {
            const int slot = (ml >> 2) ^ (tl & 15);
            *reinterpret_cast<float4*>(sc + tl * RB + slot * 16) = make_float4(d[0], d[1], d[2], d[3]);
          }
        }
    }
    auto poke = [&](int t, int m, float x) {
      if constexpr (BF) {
        const int slot = (m >> 3) ^ ((t >> 1) & 7);
        const int half = ((m >> 2) & 1) ^ ((t >> 4) & 1);
        *reinterpret_cast<bf16_t*>(sc + t * RB + slot * 16 + half * 8 + 2 * (m & 3)) = f32_to_bf16(x);
      } else {
        const int slot = (m >> 2) ^ (t & 15);
        *reinterpret_cast<float*>(sc + t * RB + slot * 16 + 4 * (m & 3)) = x;
      }
    };
#pragma unroll
    for (int jj = 0; jj < JR; ++jj) fix(rd * JR + jj, jj * 32, poke);
    // read back whole output rows of one wave's region and store them, NB reads
    // issued before their stores (the stores are predicated on the output
    // bounds, and a read behind such a branch waits for the one before it); the
    // paired drain of the dlogit store waves keeps one read in flight (its
    // kernel has no registers to spare)
    auto drain = [&](const char* src_sc, auto&& put) {
      constexpr int NB = PAIRW == 0 ? 8 : 1;
      constexpr int RQ = BF ? 8 : 4;  // rows per read
      const int k = BF ? (l & 7) : (l & 15);
#pragma unroll
      for (int q0 = 0; q0 < 8; q0 += NB) {
        uint4 v[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int row = (q0 + q) * RQ + l / (64 / RQ);
          const int slot = BF ? (k ^ ((row >> 1) & 7)) : (k ^ (row & 15));
          v[q] = *reinterpret_cast<const uint4*>(src_sc + row * RB + slot * 16);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int row = (q0 + q) * RQ + l / (64 / RQ);
          // the halves were swapped in rows with bit 4 set: (q0 + q) / 2 odd, as
          // l / 8 < 8
          if constexpr (BF)
            if (((q0 + q) >> 1) & 1) v[q] = make_uint4(v[q].z, v[q].w, v[q].x, v[q].y);
          put(rd * TR + row, k * (16 / (int)sizeof(S)), v[q]);
        }
      }
    };
    if constexpr (PAIRW == 0) {
      drain(sc, out);
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave's round is in LDS
      const int w = (int)threadIdx.x >> 6;
      if (w >= PAIRW / 2) {
        const int w0 = w - PAIRW / 2;
        drain(spare + w0 * 8192, [&](int n, int m, uint4 v) { out(w0, n, m, v); });
        drain(sc, [&](int n, int m, uint4 v) { out(w, n, m, v); });
      }
      if (rd + 1 < FN / JR) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // read before rewritten
    }
  }
}
template <typename S, int FM, int FN, int PAIRW = 0, class Val, class Out>
__device__ __forceinline__ void staged_epilogue(char* spare, Val&& val, Out&& out) {
  staged_epilogue<S, FM, FN, PAIRW>(spare, val, out, [](int, int, auto&&) {});
}


// Tile epilogue of a recomputed logit tile: acc holds S^T for vocabulary rows
// m0.. and tokens n0.. (the layout of TileGemm G); writes
// D = s (exp(S - lse) - onehot) for those entries into `panel` [token][vocab]
// (row stride Vbp, token i at row i - i0, vocabulary v at column v - v0),
// exactly 0 outside i < N, v < V.  PAIRW: G's waves split into copy and store
// waves (staged_epilogue).
template <typename T, class G, int PAIRW>
__device__ __forceinline__ void dlogit_epilogue(typename G::Acc& acc, int m0, int n0, char* spare,
                                                const int64_t* __restrict__ target, const float* __restrict__ lse,
                                                float s, int N, int V, int i0, int v0, int Vbp,
                                                T* __restrict__ panel) {
  const int l = (int)threadIdx.x & 63;
  const int wm = G::wave_m(), wn = G::wave_n();
  const int vw = m0 + wm * G::WM;  // first vocabulary row of this wave
  const int tw = n0 + wn * G::WN;  // first token of this wave
  // lse (log2 units) and target of this lane's token in each column block; a
  // target outside [0, V) gets no one-hot term
  float lr[G::FN];
  int tt[G::FN];
  bool tv[G::FN];
#pragma unroll
  for (int j = 0; j < G::FN; ++j) {
    // unconditional loads (clamped index), all in flight together
    const int tok = tw + j * 32 + (l & 31);
    const int tc = tok < N ? tok : N - 1;
    const int64_t t64 = target[tc];
    const float lv = lse[tc];
    tv[j] = tok < N;
    lr[j] = tv[j] ? lv * kLog2e : 0.f;
    tt[j] = tv[j] && t64 >= 0 && t64 < V ? (int)t64 : -1;
  }
  // src: the wave whose sub-tile (rows from m0 + WM (src / WGN), tokens from
  // n0 + WN (src % WGN)) the 16 bytes belong to
  auto out = [&](int src, int n, int m, uint4 v) {
    const int vs = m0 + (src / G::WGN) * G::WM, ts = n0 + (src % G::WGN) * G::WN;
    *reinterpret_cast<uint4*>(panel + (int64_t)(ts + n - i0) * Vbp + (vs - v0) + m) = v;
  };
  auto out_own = [&](int n, int m, uint4 v) { out((int)threadIdx.x >> 6, n, m, v); };
  if (m0 + kTile <= V && n0 + kTile <= N) {
    // interior tile, no masks: s exp2(a log2e - l) = +-exp2(a log2e - (l - log2|s|)),
    // so each element costs an fma, an exp2 and a sign flip; the one-hot term of
    // the target element (one per token column, in at most one lane of one wave)
    // is patched into the staged values afterwards, computed as before:
    // fma(s, p, -s).  s = 0 gives exp2(-inf) = 0.
    const float ls = __builtin_amdgcn_logf(__builtin_fabsf(s));
    const uint32_t sbit = __float_as_uint(s) & 0x80000000u;
    float lrs[G::FN];
    int lt[G::FN];
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      lrs[j] = lr[j] - ls;
      // target row offset within this wave's rows of this lane's half
      lt[j] = tt[j] < 0 ? -1024 : tt[j] - (vw + 4 * (l >> 5));
    }
    auto val = [&](int i, int j, int g, float* d) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        d[u] = __uint_as_float(
            __float_as_uint(__builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][4 * g + u], kLog2e, -lrs[j]))) ^ sbit);
    };
    auto fix = [&](int j, int tb, auto&& poke) {
      const int r = lt[j];
      const bool hit = r >= 0 && r < G::WM && (r & 4) == 0;
      if (!__any(hit)) return;
      if (hit) {
        // acc[i][j][4 g + u] with i = r / 32, g = r / 8 % 4, u = r % 4
        const int want = (r >> 5) * 16 + ((r >> 3) & 3) * 4 + (r & 3);
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int q = 0; q < 16; ++q) a = want == i * 16 + q ? acc[i][j][q] : a;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(a, kLog2e, -lr[j]));
        poke(tb + (l & 31), r + 4 * (l >> 5), __builtin_fmaf(s, p, -s));
      }
    };
    if constexpr (PAIRW > 0)
      staged_epilogue<T, G::FM, G::FN, PAIRW>(spare, val, out, fix);
    else
      staged_epilogue<T, G::FM, G::FN>(spare, val, out_own, fix);
  } else {
    auto val = [&](int i, int j, int g, float* d) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = vw + i * 32 + 8 * g + 4 * (l >> 5) + u;
        d[u] = 0.f;
        if (tv[j] && v < V) {
          const float p = __builtin_amdgcn_exp2f(acc[i][j][4 * g + u] * kLog2e - lr[j]);
          d[u] = s * (p - (v == tt[j] ? 1.f : 0.f));
        }
      }
    };
    if constexpr (PAIRW > 0)
      staged_epilogue<T, G::FM, G::FN, PAIRW>(spare, val, out);
    else
      staged_epilogue<T, G::FM, G::FN>(spare, val, out_own);
  }
}

// Sᵀ tile: rows = vocabulary (A = W, K-major), cols = tokens (B = x, K-major), as
// in the forward, so lse and target are read once per token column; the D tile
// reaches the panel [token][vocabulary] through the staged epilogue.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dlogits(const T* __restrict__ x, const T* __restrict__ W,
                                                        const int64_t* __restrict__ target,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ grad_loss, float red_scale, int N,
                                                        int H, int V, int i0, int v0, int tiles_v, int tiles_t,
                                                        int ntiles, int Vbp, T* __restrict__ panel, int balance,
                                                        float* __restrict__ slots, int* __restrict__ flags) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_DMA,
                   kSplitDlogits>
      G;
  static_assert(G::WM == 64 && G::STAGE_BYTES >= G::NWAVES * 8192, "dlogit staging layout");
  constexpr int PAIRW = kSplitDlogits ? G::NWAVES : 0;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const Operand<T> A{W, H, V, H};
  const Operand<T> B{x, H, N, H};
  const float s = grad_loss[0] * red_scale;
  const TileSched sc(ntiles, (H + G::BK - 1) / G::BK, kBalanceDlogits && balance);
  auto next = [&](int j, int& m0, int& n0, int& kb, int& nk) {
    int t, k0, tm, tn;
    if (!sc.item(j, t, k0, nk)) return false;
    grouped_tile<FLCE_GROUP_M_WIDE>(t, tiles_v, tiles_t, tm, tn);
    m0 = v0 + tm * kTile;
    n0 = i0 + tn * kTile;
    kb = k0 * G::BK;
    return true;
  };
  // (balanced schedules only in builds with kBalanceDlogits: the hand-over
  // pushes this kernel's registers into scratch memory)
  auto init = [&](typename G::Acc& acc, int, int, int kb, int nk) {
    G::zero(acc);
    if constexpr (kBalanceDlogits)
      if (sc.head(kb, nk)) take_partial<G>(acc, slots, flags, sc.w + 1);
  };
  auto store = [&](typename G::Acc& acc, int m0, int n0, char* spare, int kb, int) {
    if constexpr (kBalanceDlogits)
      if (TileSched::rest(kb)) {
        publish_partial<G>(acc, slots, flags, sc.w);
        return;
      }
    dlogit_epilogue<T, G, PAIRW>(acc, m0, n0, spare, target, lse, s, N, V, i0, v0, Vbp, panel);
  };
  typename G::Acc acc;
  // items of whole slices inside H take the lean copies
  G::run_tiles(A, B, H, lds, acc, next, store, init, true);
}

// (defined with the gradient kernels below)
template <typename T, class G, class RowOk, class RowOff>
__device__ __forceinline__ void grad_epilogue(typename G::Acc& acc, char* spare, int hw, int nw, int H, int final,
                                              T* __restrict__ dst, float* __restrict__ acc_buf, RowOk&& row_ok,
                                              RowOff&& row_off);

// The split tail of a bwd_dlogits launch (its tiles full .. in the grouped
// order over tiles_v x tiles_t): workgroup p computes the logit tile S^T of tail
// tile full + p / kts over hidden offsets [q Kp, (q + 1) Kp), q = p % kts, and
// writes the float32 partial sums [256 tokens][256 vocabulary] to
// pieces + p 256 256; dlogit_tail_fixup adds them and forms the dlogits.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dlogit_pieces(const T* __restrict__ x, const T* __restrict__ W,
                                                              int N, int H, int V, int i0, int v0, int tiles_v,
                                                              int tiles_t, int full, int kts, int Kp,
                                                              float* __restrict__ pieces) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_DMA>
      G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int wm = G::wave_m(), wn = G::wave_n();
  const int p = (int)blockIdx.x;
  int tm, tn;
  grouped_tile<FLCE_GROUP_M_WIDE>(full + p / kts, tiles_v, tiles_t, tm, tn);
  const int q = p % kts;
  auto next = [&](int j, int& m0, int& n0, int& kb) {
    m0 = v0 + tm * kTile;
    n0 = i0 + tn * kTile;
    kb = q * Kp;
    return j == 0;
  };
  float* const pc = pieces + (int64_t)p * kTile * kTile;
  auto all_rows = [](int) { return true; };
  auto piece_off = [](int n) { return (int64_t)n * kTile; };
  auto store = [&](typename G::Acc& a, int, int, char* spare) {
    grad_epilogue<T, G>(a, spare, wm * G::WM, wn * G::WN, kTile, 0, (T*)nullptr, pc, all_rows, piece_off);
  };
  typename G::Acc acc;
  // pieces of whole slices that end at H exactly take the lean copies
  G::run_tiles(Operand<T>{W, H, V, H}, Operand<T>{x, H, N, H}, Kp, lds, acc, next, store,
               [](typename G::Acc& a, int, int) { G::zero(a); }, (int64_t)kts * Kp <= H);
}

// Dlogits of the split tail tiles of a bwd_dlogits launch: S = the sum of the
// kts pieces (fixed order), then D = s (exp(S - lse) - onehot) for i < N, v < V
// and 0 elsewhere, into the panel (token i at row i - i0, vocabulary v at column
// v - v0, row stride Vbp).  Block b: tail tile b / 64, tokens 4 (b % 64) .. + 3
// of it; each thread 4 vocabulary entries.
template <typename T>
__global__ __launch_bounds__(256) void dlogit_tail_fixup(const float* __restrict__ pieces, int kts, int full,
                                                         int tiles_v, int tiles_t, int N, int V, int i0, int v0,
                                                         const int64_t* __restrict__ target,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ grad_loss, float red_scale,
                                                         int Vbp, T* __restrict__ panel) {
  const int i = (int)blockIdx.x / 64;
  const int r = ((int)blockIdx.x % 64) * 4 + (int)threadIdx.x / 64;
  const int c = ((int)threadIdx.x % 64) * 4;
  int tm, tn;
  grouped_tile<FLCE_GROUP_M_WIDE>(full + i, tiles_v, tiles_t, tm, tn);
  const int tok = i0 + tn * kTile + r, vb = v0 + tm * kTile + c;
  const float* pc = pieces + (int64_t)i * kts * kTile * kTile + r * kTile + c;
  float4 a = *reinterpret_cast<const float4*>(pc);
  for (int q = 1; q < kts; ++q) {
    const float4 b = *reinterpret_cast<const float4*>(pc + (int64_t)q * kTile * kTile);
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  const float s = grad_loss[0] * red_scale;
  float d[4] = {0.f, 0.f, 0.f, 0.f};
  if (tok < N) {
    const float lr = lse[tok] * kLog2e;
    const int64_t t64 = target[tok];
    const int tt = t64 >= 0 && t64 < V ? (int)t64 : -1;
    const float sv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = vb + u;
      if (v < V) {
        const float pr = __builtin_amdgcn_exp2f(sv[u] * kLog2e - lr);
        d[u] = s * (pr - (v == tt ? 1.f : 0.f));
      }
    }
  }
  T* dst = panel + (int64_t)(tok - i0) * Vbp + (vb - v0);
  if constexpr (sizeof(T) == 2)
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
  else
    *reinterpret_cast<float4*>(dst) = make_float4(d[0], d[1], d[2], d[3]);
}

// Output of a backward contraction through the staged epilogue: out rows are
// the N side of the tile (row_ok tells which exist, a prefix of them, and
// row_off gives their element offset, linear in the row), M (hidden) is
// contiguous.  final: write T to dst, else the float32 partial sums to acc_buf
// (the sums of earlier launches are already in acc, see grad_init); a final
// tile stages T directly.  The stores are buffer stores from the wave's first
// output element: rows past the last existing one fall outside the buffer's
// range and hidden entries >= H get an offset outside it, so no store is
// predicated (no branch, 32-bit offsets; a row spans at most 16 MiB, so the 128
// rows of a wave stay below 2^31 bytes).
template <typename T, class G, class RowOk, class RowOff>
__device__ __forceinline__ void grad_epilogue(typename G::Acc& acc, char* spare, int hw, int nw, int H, int final,
                                              T* __restrict__ dst, float* __restrict__ acc_buf, RowOk&& row_ok,
                                              RowOff&& row_off) {
  auto val = [&](int i, int j, int g, float* d) {
#pragma unroll
    for (int u = 0; u < 4; ++u) d[u] = acc[i][j][4 * g + u];
  };
  hw = __builtin_amdgcn_readfirstlane(hw);
  nw = __builtin_amdgcn_readfirstlane(nw);
  int nv = 0, hi = G::FN * 32;  // rows < nv exist, rows >= hi do not
  while (nv < hi) {
    const int mid = (nv + hi) >> 1;
    if (row_ok(nw + mid))
      nv = mid + 1;
    else
      hi = mid;
  }
  const int64_t o0 = row_off(nw);
  const uint32_t ld = (uint32_t)(row_off(nw + 1) - o0);
  auto store = [&](auto* base) {
    constexpr uint32_t ES = sizeof(*base);
    const uint64_t bytes = (uint64_t)nv * ld * ES;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + o0 + hw), (short)0, (uint32_t)(bytes < 0x80000000ull ? bytes : 0x80000000ull), 0x00020000);
    return [=](int n, int m, uint4 v) {
      const uint32_t off = hw + m < H ? ((uint32_t)n * ld + (uint32_t)m) * ES : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 0);
    };
  };
  if (final)
    staged_epilogue<T, G::FM, G::FN>(spare, val, store(dst));
  else
    staged_epilogue<float, G::FM, G::FN>(spare, val, store(acc_buf));
}

// Start of a gradient tile: zero, or, when the output is summed over several
// launches, the float32 partial sums so far, loaded straight into the
// accumulator layout (four consecutive hidden entries of one output row per lane
// and group, 16 bytes) while the tile's first K slice is copied; the epilogue
// then only stores.
template <class G, class RowOk, class RowOff>
__device__ __forceinline__ void grad_init(typename G::Acc& acc, int hw, int nw, int H, int accumulate,
                                          const float* __restrict__ acc_buf, RowOk&& row_ok, RowOff&& row_off) {
  if (!accumulate) {
    G::zero(acc);
    return;
  }
  int l = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(l));  // recomputed offsets, as in staged_epilogue
#pragma unroll
  for (int j = 0; j < G::FN; ++j) {
    const int n = nw + j * 32 + (l & 31);
    const bool ok = row_ok(n);
    const int64_t base = ok ? row_off(n) : 0;
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int h = hw + i * 32 + 8 * g + 4 * (l >> 5);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok && h < H) v = *reinterpret_cast<const float4*>(acc_buf + base + h);
        acc[i][j][4 * g + 0] = v.x;
        acc[i][j][4 * g + 1] = v.y;
        acc[i][j][4 * g + 2] = v.z;
        acc[i][j][4 * g + 3] = v.w;
      }
  }
}

// grad_Wᵀ tile of the panel: rows = hidden (A = x rows i0.. as [k = token][m =
// hidden], MN-major), cols = panel vocabulary (B = the panel as [k = token][n =
// vocabulary], MN-major); written as grad_W rows v0 + n, hidden contiguous.
// gw_out and gw_acc point at row v0 of their buffers.  The launch covers the
// first `ntiles` tiles of the grouped order (the rest: bwd_grad_pieces).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_grad_w(const T* __restrict__ panel, int Vbp, int Kc,
                                                       const T* __restrict__ x, int H, int V, int i0, int v0,
                                                       int Vb, int tiles_h, int tiles_v, int ntiles,
                                                       T* __restrict__ gw_out, float* __restrict__ gw_acc,
                                                       int accumulate, int final, int balance,
                                                       float* __restrict__ slots, int* __restrict__ flags) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, MN_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int wm = G::wave_m(), wn = G::wave_n();
  const Operand<T> A{x + (int64_t)i0 * H, H, H, Kc};
  const Operand<T> B{panel, Vbp, Vbp, Kc};
  const TileSched sc(ntiles, (Kc + G::BK - 1) / G::BK, balance);
  auto next = [&](int j, int& m0, int& n0, int& kb, int& nk) {
    int t, k0, tm, tn;
    if (!sc.item(j, t, k0, nk)) return false;
    grouped_tile(t, tiles_h, tiles_v, tm, tn);
    m0 = tm * kTile;
    n0 = tn * kTile;
    kb = k0 * G::BK;
    return true;
  };
  auto row_ok = [&](int v) { return v < Vb && v0 + v < V; };
  auto row_off = [&](int v) { return (int64_t)v * H; };
  auto init = [&](typename G::Acc& acc, int m0, int n0, int kb, int nk) {
    // the rest of a shared tile starts from zero; the head from the earlier
    // launches' sums plus the rest's partial sums
    grad_init<G>(acc, m0 + wm * G::WM, n0 + wn * G::WN, H, accumulate && !TileSched::rest(kb), gw_acc, row_ok,
                 row_off);
    if (sc.head(kb, nk)) take_partial<G>(acc, slots, flags, sc.w + 1);
  };
  auto store = [&](typename G::Acc& acc, int m0, int n0, char* spare, int kb, int) {
    if (TileSched::rest(kb))
      publish_partial<G>(acc, slots, flags, sc.w);
    else
      grad_epilogue<T, G>(acc, spare, m0 + wm * G::WM, n0 + wn * G::WN, H, final, gw_out, gw_acc, row_ok, row_off);
  };
  typename G::Acc acc;
  // items of whole slices inside the chunk take the lean copies
  G::run_tiles(A, B, Kc, lds, acc, next, store, init, true);
}

// The split tail of a gradient launch (the tiles full .. of its grouped order
// over tiles_m (hidden) x tiles_n, GM its row grouping): workgroup p computes
// piece q = p % kts of tail tile full + p / kts, i.e. the tile over K offsets
// [q Kp, (q + 1) Kp) (past the operands' K extent read as zeros), and writes the
// float32 partial tile [256 n][256 hidden] to pieces + p 256 256;
// grad_tail_fixup adds the pieces up.  Operands as in bwd_grad_w (WGRAD) or
// bwd_grad_x (the panel as a K-major operand in blocks).
template <typename T, bool WGRAD, int GM>
__global__ __launch_bounds__(kThreads) void bwd_grad_pieces(const T* __restrict__ panel, int Vbp, int Kgp, int Kc,
                                                            int Kv, const T* __restrict__ src, int H, int i0, int v0,
                                                            int Ncp, int tiles_m, int tiles_n, int full, int kts,
                                                            int Kp, float* __restrict__ pieces) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, WGRAD ? MN_MAJOR : K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M,
                   FLCE_WAVES_N, STAGE_REG>
      G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int wm = G::wave_m(), wn = G::wave_n();
  const int p = (int)blockIdx.x;
  int tm, tn;
  grouped_tile<GM>(full + p / kts, tiles_m, tiles_n, tm, tn);
  const int q = p % kts;
  // grad_W: A = x rows i0.., B = the panel [k = token][n = vocabulary];
  // grad_x: A = W rows v0.., B = the panel group [n = token][k = vocabulary]
  const Operand<T> A = WGRAD ? Operand<T>{src + (int64_t)i0 * H, H, H, Kc} : Operand<T>{src + (int64_t)v0 * H, H, H, Kv};
  const Operand<T> B = WGRAD ? Operand<T>{panel, Vbp, Vbp, Kc}
                             : Operand<T>{panel, Vbp, Kc, Kgp, Kgp > Vbp ? Vbp : 0x7fffffff, (int64_t)Ncp * Vbp};
  auto next = [&](int j, int& m0, int& n0, int& kb) {
    m0 = tm * kTile;
    n0 = tn * kTile;
    kb = q * Kp;
    return j == 0;
  };
  float* const pc = pieces + (int64_t)p * kTile * kTile;
  auto all_rows = [](int) { return true; };
  auto piece_off = [](int n) { return (int64_t)n * kTile; };
  auto store = [&](typename G::Acc& a, int, int, char* spare) {
    grad_epilogue<T, G>(a, spare, wm * G::WM, wn * G::WN, kTile, 0, (T*)nullptr, pc, all_rows, piece_off);
  };
  typename G::Acc acc;
  // pieces of whole slices that end at the K extent exactly take the lean copies
  G::run_tiles(A, B, Kp, lds, acc, next, store, [](typename G::Acc& a, int, int) { G::zero(a); },
               (int64_t)kts * Kp <= (WGRAD ? Kc : Kv));
}

// Sum of the kts float32 pieces of each split tail tile of a gradient launch
// (bwd_grad_w: GM = FLCE_GROUP_M, rows = vocabulary; bwd_grad_x: GM =
// FLCE_GROUP_M_WIDE, rows = tokens), in a fixed order, plus the earlier launches'
// sums (accumulate), into the output rows (final: as T) or their float32
// accumulator.  Tail tile i is tile full + i of the launch's grouped order over
// tiles_m (hidden) x tiles_n tiles; its row r lands at output row 256 tn + r,
// which exists below `rows`.  Block b: tail tile b / 64, rows 4 (b % 64) .. + 3;
// each thread 4 hidden entries.
template <typename T, int GM>
__global__ __launch_bounds__(256) void grad_tail_fixup(const float* __restrict__ pieces, int kts, int full,
                                                       int tiles_m, int tiles_n, int H, int rows,
                                                       T* __restrict__ out, float* __restrict__ acc_buf,
                                                       int accumulate, int final) {
  const int i = (int)blockIdx.x / 64;
  const int r = ((int)blockIdx.x % 64) * 4 + (int)threadIdx.x / 64;
  const int c = ((int)threadIdx.x % 64) * 4;
  int tm, tn;
  grouped_tile<GM>(full + i, tiles_m, tiles_n, tm, tn);
  const int h = tm * kTile + c, v = tn * kTile + r;
  if (v >= rows || h >= H) return;
  const float* pc = pieces + (int64_t)i * kts * kTile * kTile + r * kTile + c;
  float4 a = *reinterpret_cast<const float4*>(pc);
  for (int q = 1; q < kts; ++q) {
    const float4 b = *reinterpret_cast<const float4*>(pc + (int64_t)q * kTile * kTile);
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  const int64_t o = (int64_t)v * H + h;
  if (accumulate) {
    const float4 b = *reinterpret_cast<const float4*>(acc_buf + o);
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  if (final) {
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<uint2*>(out + o) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
    else
      *reinterpret_cast<float4*>(out + o) = a;
  } else {
    *reinterpret_cast<float4*>(acc_buf + o) = a;
  }
}

// grad_xᵀ tile of the token chunk: rows = hidden (A = W rows v0.. as [k =
// vocabulary][m = hidden], MN-major), cols = chunk tokens (B = the panel as [n =
// token][k = vocabulary], K-major; Kgp padded columns, each Vbp of them in a
// panel block of their own); written as grad_x rows i0 + n.  With ks > 1
// the panel's vocabulary is split into ks ranges of Ks entries: work item
// (split s, tile) covers range s and writes its float32 partial sums to
// part + s * Ncp * H (rows chunk-local); split 0 starts from the sums of earlier
// panels; bwd_gx_reduce adds the splits.  The launch covers the first `nitems`
// work items (without splits, the tiles after them: bwd_grad_pieces).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_grad_x(const T* __restrict__ panel, int Vbp, int Kgp, int Kc, int Kv,
                                                       const T* __restrict__ W, int H, int N, int i0, int v0,
                                                       int tiles_h, int tiles_t, int ks, int Ks, int Ncp,
                                                       T* __restrict__ gx_out, float* __restrict__ gx_acc,
                                                       float* __restrict__ part, int accumulate, int final,
                                                       int nitems, int balance, float* __restrict__ slots,
                                                       int* __restrict__ flags) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int wm = G::wave_m(), wn = G::wave_n();
  const Operand<T> A{W + (int64_t)v0 * H, H, H, Kv};
  // a group of panels: block b starts b Ncp Vbp elements further and holds K
  // offsets b Vbp .. (b + 1) Vbp - 1 (the last one up to Kgp - 1)
  const Operand<T> B{panel, Vbp, Kc, Kgp, Kgp > Vbp ? Vbp : 0x7fffffff, (int64_t)Ncp * Vbp};
  const int tiles = tiles_h * tiles_t;
  // the j-th work item of this workgroup: split s, tile origin (m0, n0)
  auto item = [&](int j, int& s, int& m0, int& n0) {
    const int G_ = (int)gridDim.x;
    const int t = xcd_grouped_id((int)blockIdx.x, G_) + j * G_;
    if (t >= nitems) return false;
    s = t / tiles;
    int tm, tn;
    grouped_tile<FLCE_GROUP_M_WIDE>(t - s * tiles, tiles_h, tiles_t, tm, tn);
    m0 = tm * kTile;
    n0 = tn * kTile;
    return true;
  };
  auto next = [&](int j, int& m0, int& n0, int& kb) {
    int s;
    if (!item(j, s, m0, n0)) return false;
    kb = s * Ks;
    return true;
  };
  auto row_ok = [&](int t) { return t < Kc && i0 + t < N; };
  auto row_off = [&](int t) { return (int64_t)(i0 + t) * H; };
  auto row_local = [&](int t) { return (int64_t)t * H; };
  int ji = 0, je = 0;  // items started / finished by this workgroup
  auto init = [&](typename G::Acc& acc, int m0, int n0) {
    int s, a0, a1;
    item(ji++, s, a0, a1);
    grad_init<G>(acc, m0 + wm * G::WM, n0 + wn * G::WN, H, accumulate && s == 0, gx_acc, row_ok, row_off);
  };
  auto store = [&](typename G::Acc& acc, int m0, int n0, char* spare) {
    int s, a0, a1;
    item(je++, s, a0, a1);
    if (ks == 1)
      grad_epilogue<T, G>(acc, spare, m0 + wm * G::WM, n0 + wn * G::WN, H, final, gx_out, gx_acc, row_ok, row_off);
    else
      grad_epilogue<T, G>(acc, spare, m0 + wm * G::WM, n0 + wn * G::WN, H, 0, gx_out,
                          part + (int64_t)s * Ncp * H, row_ok, row_local);
  };
  typename G::Acc acc;
  if (ks == 1) {
    // one split: the schedule of bwd_grad_w over the launch's tiles
    const TileSched sc(nitems, (Ks + G::BK - 1) / G::BK, balance);
    auto next1 = [&](int j, int& m0, int& n0, int& kb, int& nk) {
      int t, k0, tm, tn;
      if (!sc.item(j, t, k0, nk)) return false;
      grouped_tile<FLCE_GROUP_M_WIDE>(t, tiles_h, tiles_t, tm, tn);
      m0 = tm * kTile;
      n0 = tn * kTile;
      kb = k0 * G::BK;
      return true;
    };
    auto init1 = [&](typename G::Acc& acc, int m0, int n0, int kb, int nk) {
      grad_init<G>(acc, m0 + wm * G::WM, n0 + wn * G::WN, H, accumulate && !TileSched::rest(kb), gx_acc, row_ok,
                   row_off);
      if (sc.head(kb, nk)) take_partial<G>(acc, slots, flags, sc.w + 1);
    };
    auto store1 = [&](typename G::Acc& acc, int m0, int n0, char* spare, int kb, int) {
      if (TileSched::rest(kb))
        publish_partial<G>(acc, slots, flags, sc.w);
      else
        grad_epilogue<T, G>(acc, spare, m0 + wm * G::WM, n0 + wn * G::WN, H, final, gx_out, gx_acc, row_ok, row_off);
    };
    // items of whole slices inside the group's entries take the lean copies
    G::run_tiles(A, B, Ks, lds, acc, next1, store1, init1, true);
  } else {
    // splits of whole slices that end at the group's last entry exactly take
    // the lean copies too
    G::run_tiles(A, B, Ks, lds, acc, next, store, init, (int64_t)ks * Ks <= Kv);
  }
}

// Sum of the ks float32 partial grad_x row blocks [Kc, H] (fixed order) into
// grad_x rows i0.. (final: as T) or into their float32 accumulator.
template <typename T>
__global__ __launch_bounds__(256) void bwd_gx_reduce(const float* __restrict__ part, int ks, int64_t stride, int Kc,
                                                     int H, int i0, int final, T* __restrict__ gx_out,
                                                     float* __restrict__ gx_acc) {
  const int64_t n4 = (int64_t)Kc * H / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += (int64_t)gridDim.x * 256) {
    float4 a = reinterpret_cast<const float4*>(part)[q];
    for (int s = 1; s < ks; ++s) {
      const float4 b = reinterpret_cast<const float4*>(part + s * stride)[q];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    const int64_t o = (int64_t)i0 * H + 4 * q;
    if (final) {
      if constexpr (sizeof(T) == 2)
        *reinterpret_cast<uint2*>(gx_out + o) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
      else
        *reinterpret_cast<float4*>(gx_out + o) = a;
    } else {
      *reinterpret_cast<float4*>(gx_acc + o) = a;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward with float32 atomics (a comparison for the bounded panels; helion PR
// #1268, PR description: the weight gradient is accumulated with an atomic add)
// ---------------------------------------------------------------------------
// Pairs (token tile, vocabulary tile) in launches of up to 256, one pair per
// workgroup (bwd_atomic): recompute the pair's logit tile S^T = W_tile . x_tile^T
// (K = H), write its dlogit tile D [256 tokens][256 vocab] into the workgroup's
// slot of `dtile` (256 slots, one per workgroup of a launch: never the whole
// dlogit matrix), then contract D with the tile's rows of W and x over the hidden
// size and add both gradients' partial sums into float32 buffers with atomics:
//   grad_x[n0 + i, h] += sum_v D[i, v] W[m0 + v, h]   (one tile per 256 of h, K = 256)
//   grad_W[m0 + v, h] += sum_i D[i, v] x[n0 + i, h]   (one tile per 256 of h, K = 256)
// Every partial sum reaches the L2 as an atomic: 4 N H V (1/256 + 1/256) bytes
// over the whole backward.  The result depends on the order in which the
// atomics land (not bitwise reproducible).  One pair per workgroup, not a
// persistent loop over pairs: the loop would keep the per-lane addressing of all
// three contractions live at once and spill.

// One of the two gradient contractions of a pair's D tile (dt), with its
// float32 atomic epilogue.
template <typename T, bool WGRAD>
__device__ __forceinline__ void atomic_grad_phase(const T* __restrict__ x, const T* __restrict__ W, int N, int H,
                                                  int V, int m0, int n0, const T* __restrict__ dt,
                                                  float* __restrict__ gx_acc, float* __restrict__ gw_acc, T* lds) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      GX;  // grad_x^T tile: A = W rows as [k = vocab][m = hidden], B = D as [n = token][k = vocab]
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, MN_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      GW;  // grad_W^T tile: A = x rows as [k = token][m = hidden], B = D as [k = token][n = vocab]
  const int tiles_h = (H + kTile - 1) / kTile;
  const int wm = GX::wave_m(), wn = GX::wave_n();
  auto hnext = [&](int j, int& hm0, int& hn0) {
    hm0 = j * kTile;
    hn0 = 0;
    return j < tiles_h;
  };
  // K of every tile, hidden from the optimiser: a known K of 4 slices gets the
  // slice loop unrolled, and the unrolled copies spill
  int Kt = kTile;
  asm volatile("" : "+s"(Kt));
  // four float32 atomics per 16 staged bytes (whole 256-byte row segments per 16
  // lanes), as buffer atomics on the tile's 256 output rows (byte offsets within
  // them fit 32 bits: a row holds at most 8 MiB)
  auto add4 = [](__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(__uint_as_float(v.x), r, off + 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(__uint_as_float(v.y), r, off + 4, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(__uint_as_float(v.z), r, off + 8, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(__uint_as_float(v.w), r, off + 12, 0, 0);
  };
  if constexpr (!WGRAD) {
    // grad_x rows n0.. : tile (hidden m, token n) added at grad_x[n0 + n][m]
    typename GX::Acc acc;
    const Operand<T> A{W + (int64_t)m0 * H, H, H, V - m0 < kTile ? V - m0 : kTile};
    const Operand<T> B{dt, kTile, kTile, kTile};
    auto add = [&](typename GX::Acc& a, int hm0, int, char* spare) {
      auto val = [&](int i, int j, int g, float* d) {
#pragma unroll
        for (int u = 0; u < 4; ++u) d[u] = a[i][j][4 * g + u];
      };
      const int hw = hm0 + wm * GX::WM, nw = wn * GX::WN;
      const int rows = N - n0 < kTile ? N - n0 : kTile;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(gx_acc + (int64_t)n0 * H), (short)0, (uint32_t)rows * (uint32_t)H * 4u, 0x00020000);
      staged_epilogue<float, GX::FM, GX::FN>(spare, val, [&](int n, int m, uint4 v) {
        const int t = nw + n, h = hw + m;
        if (t < rows && h < H) add4(r, ((uint32_t)t * (uint32_t)H + (uint32_t)h) * 4u, v);
      });
    };
    GX::run_tiles(A, B, Kt, lds, acc, hnext, add);
  } else {
    // grad_W rows m0.. : tile (hidden m, vocabulary n) added at grad_W[m0 + n][m]
    typename GW::Acc acc;
    const Operand<T> A{x + (int64_t)n0 * H, H, H, N - n0 < kTile ? N - n0 : kTile};
    const Operand<T> B{dt, kTile, kTile, kTile};
    auto add = [&](typename GW::Acc& a, int hm0, int, char* spare) {
      auto val = [&](int i, int j, int g, float* d) {
#pragma unroll
        for (int u = 0; u < 4; ++u) d[u] = a[i][j][4 * g + u];
      };
      const int hw = hm0 + wm * GW::WM, nw = wn * GW::WN;
      const int rows = V - m0 < kTile ? V - m0 : kTile;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(gw_acc + (int64_t)m0 * H), (short)0, (uint32_t)rows * (uint32_t)H * 4u, 0x00020000);
      staged_epilogue<float, GW::FM, GW::FN>(spare, val, [&](int n, int m, uint4 v) {
        const int vr = nw + n, h = hw + m;
        if (vr < rows && h < H) add4(r, ((uint32_t)vr * (uint32_t)H + (uint32_t)h) * 4u, v);
      });
    };
    GW::run_tiles(A, B, Kt, lds, acc, hnext, add);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_atomic(const T* __restrict__ x, const T* __restrict__ W,
                                                       const int64_t* __restrict__ target,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ grad_loss, float red_scale, int N,
                                                       int H, int V, int tiles_t, int tiles_v, int pair0,
                                                       T* __restrict__ dtile, float* __restrict__ gx_acc,
                                                       float* __restrict__ gw_acc) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_DMA,
                   kSplitDlogits>
      GS;  // logit tile, as in bwd_dlogits
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      GX;  // grad_x^T tile: A = W rows as [k = vocab][m = hidden], B = D as [n = token][k = vocab]
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, MN_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      GW;  // grad_W^T tile: A = x rows as [k = token][m = hidden], B = D as [k = token][n = vocab]
  static_assert(GS::LDS_ELEMS == GX::LDS_ELEMS && GX::LDS_ELEMS == GW::LDS_ELEMS, "one LDS array");
  constexpr int PAIRW = kSplitDlogits ? GS::NWAVES : 0;
  __shared__ __attribute__((aligned(16))) T lds[GS::LDS_ELEMS];
  const int p = pair0 + xcd_grouped_id((int)blockIdx.x, (int)gridDim.x);
  if (p >= tiles_t * tiles_v) return;
  int tm, tn;  // vocabulary tile, token tile
  grouped_tile<FLCE_GROUP_M_WIDE>(p, tiles_v, tiles_t, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;
  T* const dt = dtile + (int64_t)blockIdx.x * kTile * kTile;
  const float s = grad_loss[0] * red_scale;
  {
    auto one = [&](int j, int& am0, int& an0) {
      am0 = m0;
      an0 = n0;
      return j == 0;
    };
    auto store = [&](typename GS::Acc& a, int am0, int an0, char* spare) {
      dlogit_epilogue<T, GS, PAIRW>(a, am0, an0, spare, target, lse, s, N, V, n0, m0, kTile, dt);
    };
    typename GS::Acc acc;
    GS::run_tiles(Operand<T>{W, H, V, H}, Operand<T>{x, H, N, H}, H, lds, acc, one, store);
  }
  // the D tile's stores are complete and visible to the whole workgroup
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  atomic_grad_phase<T, false>(x, W, N, H, V, m0, n0, dt, gx_acc, gw_acc, lds);
  atomic_grad_phase<T, true>(x, W, N, H, V, m0, n0, dt, gx_acc, gw_acc, lds);
}

// Zero n floats (a fill kernel rather than a memset, so that the call can be
// captured in a HIP graph).
__global__ __launch_bounds__(256) void zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t n4 = n / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += (int64_t)gridDim.x * 256)
    reinterpret_cast<float4*>(p)[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t q = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (int64_t)gridDim.x * 256) p[q] = 0.f;
}

// float32 -> bfloat16 (round to nearest even) of n values, n a multiple of 4.
__global__ __launch_bounds__(256) void cast_f32_bf16(const float* __restrict__ src, bf16_t* __restrict__ dst,
                                                     int64_t n) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n / 4; q += (int64_t)gridDim.x * 256) {
    const float4 a = reinterpret_cast<const float4*>(src)[q];
    reinterpret_cast<uint2*>(dst)[q] = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
  }
}

__global__ void fill_scalar(float* p, float v) { p[0] = v; }

// Forward workspace of flce_forward_noalloc, for callers that cannot allocate: a
// file-scope device array (each GPU holds its own copy, at its own address, until
// the process ends).  In host code its name is only a stand-in, so kernels get
// the device address looked up below, never the name.
static __device__ __align__(256) unsigned char scratch[FLCE_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device
// with that device current (hipGetSymbolAddress) and kept.
hipError_t static_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers (host side)
// ---------------------------------------------------------------------------
hipError_t launch_fill(float* p, float v, hipStream_t st, Recorder& rec) {
  hipLaunchKernelGGL(fill_scalar, dim3(1), dim3(1), 0, st, p, v);
  rec.after(FLCE_K_FILL);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : rec.err;
}

template <typename T>
static hipError_t launch_fwd_t(const FwdPlan& p, const void* x, const void* W, const int64_t* target, int N,
                               int H, int V, float* part_m, float* part_s, float* zt, float* lse, double* block_loss,
                               double scale, float* loss, hipStream_t st, Recorder& rec) {
  const int grid = p.tiles_tok * p.splits;
  rec.start();
  hipLaunchKernelGGL(fwd_partial<T>, dim3(grid), dim3(kFwdThreads), 0, st, (const T*)x, (const T*)W, target, N, H, V,
                     p.tiles_tok, p.tiles_per_split, p.Np, part_m, part_s, zt, (unsigned int*)(block_loss + p.nb));
  rec.after(FLCE_K_FWD_PARTIAL);
  hipLaunchKernelGGL(fwd_combine, dim3(p.nb), dim3(kCombineThreads), 0, st, part_m, part_s, p.splits, p.Np, N, V,
                     target, zt, lse, block_loss, (unsigned int*)(block_loss + p.nb), scale, loss);
  rec.after(FLCE_K_FWD_COMBINE);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : rec.err;
}

hipError_t launch_forward(int dt, const FwdPlan& p, const void* x, const void* W, const int64_t* target, int N,
                          int H, int V, float* part_m, float* part_s, float* zt, float* lse, double* block_loss,
                          double scale, float* loss, hipStream_t st, Recorder& rec) {
  return dt == 1 ? launch_fwd_t<bf16_t>(p, x, W, target, N, H, V, part_m, part_s, zt, lse, block_loss, scale, loss, st,
                                        rec)
                 : launch_fwd_t<float>(p, x, W, target, N, H, V, part_m, part_s, zt, lse, block_loss, scale, loss, st,
                                       rec);
}

// The tail split of one backward launch (T tiles on `cus` workgroups, KT K slices
// of BK per tile): tail tiles, pieces per tail tile, K extent per piece (a whole
// number of slices); tail = 0: no split.  With tail = T (a launch of few tiles)
// the main launch has no tiles and runs as a single idle workgroup.
struct Tail {
  int tail, kts, Kp;
};
static Tail plan_tail(int T, int cus, int cap, int KT, int BK) {
  const TailSplit ts = tail_split(T, cus, cap, (int64_t)KT * BK);
  if (ts.kts < 2) return Tail{0, 0, 0};
  const int per = (KT + ts.kts - 1) / ts.kts;  // K slices per piece
  const int kts = (KT + per - 1) / per;
  if (kts < 2) return Tail{0, 0, 0};
  return Tail{ts.tail, kts, per * BK};
}

template <typename T>
static hipError_t launch_bwd_t(const BwdPlan& p, const void* xv, const void* Wv, const int64_t* target,
                               const float* lse, const float* grad_loss, float red_scale, int N, int H, int V,
                               void* gxv, void* gwv, void* panelv, float* gx_acc, float* gw_acc, float* gx_part,
                               float* tail_buf, int* flags, hipStream_t st, Recorder& rec) {
  const T* x = (const T*)xv;
  const T* W = (const T*)Wv;
  T* gx = (T*)gxv;
  T* gw = (T*)gwv;
  T* panel = (T*)panelv;
  const bool f32 = sizeof(T) == 4;
  // Accumulate float32 outputs in place; bfloat16 outputs go through float32 buffers.
  float* gxa = f32 ? (float*)gxv : gx_acc;  // [N, H]
  float* gwa0 = f32 ? (float*)gwv : gw_acc;  // [V, H] in place, or one panel [Vb, H]
  const int tiles_h = (H + kTile - 1) / kTile;
  rec.start();
  // balanced launches need a partial-sum slot per workgroup; their flags start
  // at 0 (each launch leaves them so)
  const bool can_balance = p.slots > 0 && p.max_workgroups <= p.slots;
  if (can_balance) hipLaunchKernelGGL(zero_f32, dim3(1), dim3(256), 0, st, (float*)flags, (int64_t)p.slots);
  auto balance = [&](bool on, int T_, int G_) { return on && can_balance && balanced_launch(T_, G_) ? 1 : 0; };
  for (int pv = 0; pv < p.n_panels; ++pv) {
    const int v0 = pv * p.Vb;
    const int Kv = min(p.Vb, V - v0);
    const int Vbp = p.Vbp;
    // panel pv goes to block g of the panel buffer (gx_group > 1 only with one
    // token chunk); grad_x runs after the last panel of each group
    const int g = pv % p.gx_group;
    T* sub = panel + (int64_t)g * p.Ncp * Vbp;
    const bool gx_now = g == p.gx_group - 1 || pv == p.n_panels - 1;
    const int gv0 = (pv - g) * p.Vb;                          // first vocabulary entry of the group
    const int Kg = v0 + Kv - gv0;                             // its entries
    const int Kgp = g * Vbp + (Kv + kTile - 1) / kTile * kTile;  // its padded columns
    for (int c = 0; c < p.n_chunks; ++c) {
      const int i0 = c * p.Nc;
      const int Kc = min(p.Nc, N - i0);
      const int tiles_m = (Kc + kTile - 1) / kTile;
      const int tiles_n = (Kv + kTile - 1) / kTile;
      auto grid = [&](int tiles) { return dim3(min(tiles, p.max_workgroups)); };
      {
        // the partial last round of logit tiles is cut along K (hidden) into pieces
        constexpr int BK = Cfg<T>::BK;
        const int T_ = tiles_m * tiles_n;
        const int bal = balance(kBalanceDlogits, T_, (int)grid(T_).x);
        const Tail tl = bal ? Tail{0, 0, 0} : plan_tail(T_, p.max_workgroups, p.tail_cap, (H + BK - 1) / BK, BK);
        const dim3 g = grid(tl.tail < T_ ? T_ : 1);
        hipLaunchKernelGGL(bwd_dlogits<T>, g, dim3(kThreads), 0, st, x, W, target, lse, grad_loss, red_scale, N, H,
                           V, i0, v0, tiles_n, tiles_m, T_ - tl.tail, Vbp, sub, bal, tail_buf, flags);
        rec.after(FLCE_K_BWD_DLOGITS);
        if (tl.tail) {
          hipLaunchKernelGGL(bwd_dlogit_pieces<T>, dim3(tl.tail * tl.kts), dim3(kThreads), 0, st, x, W, N, H, V, i0,
                             v0, tiles_n, tiles_m, T_ - tl.tail, tl.kts, tl.Kp, tail_buf);
          rec.after(FLCE_K_TAIL_PIECES);
          hipLaunchKernelGGL(dlogit_tail_fixup<T>, dim3(tl.tail * 64), dim3(256), 0, st, (const float*)tail_buf,
                             tl.kts, T_ - tl.tail, tiles_n, tiles_m, N, V, i0, v0, target, lse, grad_loss, red_scale,
                             Vbp, sub);
          rec.after(FLCE_K_TAIL_FIXUP);
        }
      }
      // grad_W rows of this panel accumulate over token chunks.
      float* gwa = f32 ? gwa0 + (int64_t)v0 * H : gwa0;
      {
        // the partial last round of tiles is cut along K (tokens) into pieces
        constexpr int BK = Cfg<T>::BK;
        const int T_ = tiles_n * tiles_h;
        const int bal = balance(kBalance, T_, (int)grid(T_).x);
        const Tail tl = bal ? Tail{0, 0, 0} : plan_tail(T_, p.max_workgroups, p.tail_cap, (Kc + BK - 1) / BK, BK);
        const dim3 g = grid(tl.tail < T_ ? T_ : 1);
        const int acc_w = c > 0 ? 1 : 0, fin_w = c == p.n_chunks - 1 ? 1 : 0;
        hipLaunchKernelGGL(bwd_grad_w<T>, g, dim3(kThreads), 0, st, (const T*)sub, Vbp, Kc, x, H, V, i0, v0, Kv,
                           tiles_h, tiles_n, T_ - tl.tail, gw + (int64_t)v0 * H, gwa, acc_w, fin_w, bal, tail_buf,
                           flags);
        rec.after(FLCE_K_BWD_GRAD_W);
        if (tl.tail) {
          hipLaunchKernelGGL((bwd_grad_pieces<T, true, FLCE_GROUP_M>), dim3(tl.tail * tl.kts), dim3(kThreads), 0, st,
                             (const T*)sub, Vbp, 0, Kc, 0, x, H, i0, v0, 0, tiles_h, tiles_n, T_ - tl.tail, tl.kts,
                             tl.Kp, tail_buf);
          rec.after(FLCE_K_TAIL_PIECES);
          hipLaunchKernelGGL((grad_tail_fixup<T, FLCE_GROUP_M>), dim3(tl.tail * 64), dim3(256), 0, st,
                             (const float*)tail_buf, tl.kts, T_ - tl.tail, tiles_h, tiles_n, H, min(Kv, V - v0),
                             gw + (int64_t)v0 * H, gwa, acc_w, fin_w);
          rec.after(FLCE_K_TAIL_FIXUP);
        }
      }
      if (!gx_now) continue;
      // grad_x rows of this chunk accumulate over panel groups; a launch with
      // few output tiles splits the group's vocabulary (partial sums in gx_part).
      constexpr int BK = Cfg<T>::BK;
      const int Ks = (int)((((int64_t)Kg + p.gx_splits - 1) / p.gx_splits + BK - 1) / BK * BK);
      const int ks = (Kg + Ks - 1) / Ks;
      const int acc_x = gv0 > 0 ? 1 : 0, fin_x = pv == p.n_panels - 1 ? 1 : 0;
      // without K splits, the partial last round of tiles is cut along K instead
      const int Tx = tiles_m * tiles_h;
      const int balx = ks == 1 ? balance(kBalance, Tx, (int)grid(Tx).x) : 0;
      const Tail tl = ks == 1 && !balx ? plan_tail(Tx, p.max_workgroups, p.tail_cap, Ks / BK, BK) : Tail{0, 0, 0};
      const dim3 gxg = grid(tl.tail < Tx * ks ? Tx * ks : 1);
      hipLaunchKernelGGL(bwd_grad_x<T>, gxg, dim3(kThreads), 0, st, (const T*)panel, Vbp, Kgp, Kc, Kg, W, H, N, i0,
                         gv0, tiles_h, tiles_m, ks, Ks, p.Ncp, gx, gxa, gx_part, acc_x, fin_x, Tx * ks - tl.tail,
                         balx, tail_buf, flags);
      rec.after(FLCE_K_BWD_GRAD_X);
      if (tl.tail) {
        hipLaunchKernelGGL((bwd_grad_pieces<T, false, FLCE_GROUP_M_WIDE>), dim3(tl.tail * tl.kts), dim3(kThreads), 0,
                           st, (const T*)panel, Vbp, Kgp, Kc, Kg, W, H, i0, gv0, p.Ncp, tiles_h, tiles_m,
                           Tx - tl.tail, tl.kts, tl.Kp, tail_buf);
        rec.after(FLCE_K_TAIL_PIECES);
        hipLaunchKernelGGL((grad_tail_fixup<T, FLCE_GROUP_M_WIDE>), dim3(tl.tail * 64), dim3(256), 0, st,
                           (const float*)tail_buf, tl.kts, Tx - tl.tail, tiles_h, tiles_m, H, min(Kc, N - i0),
                           gx + (int64_t)i0 * H, gxa + (int64_t)i0 * H, acc_x, fin_x);
        rec.after(FLCE_K_TAIL_FIXUP);
      }
      if (ks > 1) {
        const int64_t n4 = (int64_t)Kc * H / 4;
        const int rgrid = (int)std::min<int64_t>((n4 + 255) / 256, 4 * (int64_t)p.max_workgroups);
        hipLaunchKernelGGL(bwd_gx_reduce<T>, dim3(rgrid), dim3(256), 0, st, (const float*)gx_part, ks,
                           (int64_t)p.Ncp * H, Kc, H, i0, fin_x, gx, gxa);
        rec.after(FLCE_K_BWD_GX_REDUCE);
      }
    }
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : rec.err;
}

template <typename T>
static hipError_t launch_bwd_atomic_t(const void* xv, const void* Wv, const int64_t* target, const float* lse,
                                      const float* grad_loss, float red_scale, int N, int H, int V, void* gxv,
                                      void* gwv, void* dtile, float* gx_acc, float* gw_acc, int max_wgs,
                                      hipStream_t st, Recorder& rec) {
  const bool f32 = sizeof(T) == 4;
  float* gxa = f32 ? (float*)gxv : gx_acc;
  float* gwa = f32 ? (float*)gwv : gw_acc;
  const int64_t nx = (int64_t)N * H, nw = (int64_t)V * H;
  auto fill_grid = [&](int64_t n) { return dim3((unsigned)std::min<int64_t>((n / 4 + 255) / 256 + 1, 4096)); };
  rec.start();
  hipLaunchKernelGGL(zero_f32, fill_grid(nx), dim3(256), 0, st, gxa, nx);
  rec.after(FLCE_K_ZERO);
  hipLaunchKernelGGL(zero_f32, fill_grid(nw), dim3(256), 0, st, gwa, nw);
  rec.after(FLCE_K_ZERO);
  const int tiles_t = (N + kTile - 1) / kTile, tiles_v = (V + kTile - 1) / kTile;
  const int pairs = tiles_t * tiles_v;
  // launches of max_wgs pairs, one per workgroup, each with its own D tile slot;
  // stream order keeps a slot from being reused before its last reader is done
  for (int p0 = 0; p0 < pairs; p0 += max_wgs) {
    const int grid = std::min(max_wgs, pairs - p0);
    hipLaunchKernelGGL(bwd_atomic<T>, dim3(grid), dim3(kThreads), 0, st, (const T*)xv, (const T*)Wv, target, lse,
                       grad_loss, red_scale, N, H, V, tiles_t, tiles_v, p0, (T*)dtile, gxa, gwa);
    rec.after(FLCE_K_BWD_ATOMIC);
  }
  if (!f32) {
    hipLaunchKernelGGL(cast_f32_bf16, fill_grid(nx), dim3(256), 0, st, (const float*)gxa, (bf16_t*)gxv, nx);
    rec.after(FLCE_K_CAST);
    hipLaunchKernelGGL(cast_f32_bf16, fill_grid(nw), dim3(256), 0, st, (const float*)gwa, (bf16_t*)gwv, nw);
    rec.after(FLCE_K_CAST);
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : rec.err;
}

hipError_t launch_backward_atomic(int dt, const void* x, const void* W, const int64_t* target, const float* lse,
                                  const float* grad_loss, float red_scale, int N, int H, int V, void* gx, void* gw,
                                  void* dtile, float* gx_acc, float* gw_acc, int max_wgs, hipStream_t st,
                                  Recorder& rec) {
  return dt == 1 ? launch_bwd_atomic_t<bf16_t>(x, W, target, lse, grad_loss, red_scale, N, H, V, gx, gw, dtile,
                                               gx_acc, gw_acc, max_wgs, st, rec)
                 : launch_bwd_atomic_t<float>(x, W, target, lse, grad_loss, red_scale, N, H, V, gx, gw, dtile,
                                              gx_acc, gw_acc, max_wgs, st, rec);
}

hipError_t launch_backward(int dt, const BwdPlan& p, const void* x, const void* W, const int64_t* target,
                           const float* lse, const float* grad_loss, float red_scale, int N, int H, int V, void* gx,
                           void* gw, void* panel, float* gx_acc, float* gw_acc, float* gx_part, float* tail,
                           int* flags, hipStream_t st, Recorder& rec) {
  return dt == 1 ? launch_bwd_t<bf16_t>(p, x, W, target, lse, grad_loss, red_scale, N, H, V, gx, gw, panel, gx_acc,
                                        gw_acc, gx_part, tail, flags, st, rec)
                 : launch_bwd_t<float>(p, x, W, target, lse, grad_loss, red_scale, N, H, V, gx, gw, panel, gx_acc,
                                       gw_acc, gx_part, tail, flags, st, rec);
}

}  // namespace flce

#if FLCE_TILE_CLOCK
// Measurement builds: copy the tile clock records (4 x 256 x 64 x 5 64-bit
// values, see gemm_core.h) to host memory `dst` (at most `bytes`), or clear
// them; synchronous, on the current device.  hipError_t codes.
extern "C" int flce_tile_clock_read(void* dst, size_t bytes) {
  const size_t n = bytes < sizeof(flce::tile_clock) ? bytes : sizeof(flce::tile_clock);
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(flce::tile_clock), n, 0, hipMemcpyDeviceToHost);
}
extern "C" int flce_tile_clock_clear() {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(flce::tile_clock));
  if (e == hipSuccess) e = hipMemset(p, 0, sizeof(flce::tile_clock));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return (int)e;
}
#endif
