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
//   fwd_combine   merges the split partials into lse and the per-token loss, then
//                 reduces the losses per block in a fixed order.
//   fwd_loss      sums the block partials in a fixed order into the scalar loss.
// Backward (helion PR #1268: the backward recomputes the logits; the dlogits
// drive both gradients; Liger-Kernel PR #928: zero the out-of-range dlogits):
//   bwd_dlogits   recomputes a logit tile S = x_tile . W_tile^T and writes
//                 D = s (exp(S - lse) - onehot) into a bounded panel, exactly 0
//                 outside i < N, v < V;
//   bwd_grad_w    grad_W[v, h] (+)= sum_i D[i, v] x[i, h] over the panel's tokens;
//   bwd_grad_x    grad_x[i, h] (+)= sum_v D[i, v] W[v, h] over the panel's vocabulary.
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

template <typename T>
struct Cfg;
template <>
struct Cfg<bf16_t> {
  static constexpr int BK = FLCE_BK_BF16;
  static constexpr int NS = FLCE_NSTAGE_BF16;
};
template <>
struct Cfg<float> {
  static constexpr int BK = FLCE_BK_F32;
  static constexpr int NS = FLCE_NSTAGE_F32;
};

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void fwd_partial(const T* __restrict__ x, const T* __restrict__ W,
                                                   const int64_t* __restrict__ target, int N, int H, int V,
                                                   int tiles_tok, int tiles_per_split, int Np,
                                                   float* __restrict__ part_m, float* __restrict__ part_s,
                                                   float* __restrict__ zt_out) {
  // S^T tile: rows = vocabulary (A = W, K-major), cols = tokens (B = x, K-major).
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N> G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];

  const int lid = xcd_grouped_id((int)blockIdx.x, (int)gridDim.x);
  int tt, split;
  grouped_tile(lid, tiles_tok, (int)gridDim.x / tiles_tok, tt, split);
  const int n0 = tt * kTile;
  const int tiles_v = (V + kTile - 1) / kTile;
  const int vt_begin = split * tiles_per_split;
  const int vt_end = min(tiles_v, vt_begin + tiles_per_split);

  const int l = (int)threadIdx.x & 63;
  const int wm = G::wave_m(), wn = G::wave_n();

  const Operand<T> A{W, H, V, H};
  const Operand<T> B{x, H, N, H};

  float mrun[G::FN], srun[G::FN];
  int tgt[G::FN];
#pragma unroll
  for (int j = 0; j < G::FN; ++j) {
    mrun[j] = -INFINITY;
    srun[j] = 0.f;
    const int tok = n0 + wn * G::WN + j * 32 + (l & 31);
    tgt[j] = tok < N ? (int)min<int64_t>(max<int64_t>(target[tok], -1), (int64_t)V) : -1;
  }

  typename G::Acc acc;
  auto next = [&](int j, int& m0, int& tn0) {
    m0 = (vt_begin + j) * kTile;
    tn0 = n0;
    return vt_begin + j < vt_end;
  };
  auto fold = [&](typename G::Acc& a, int m0, int, char*) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = m0 + wm * G::WM + i * 32 + acc_row(r, l);
          const float val = v < V ? a[i][j][r] * kLog2e : -INFINITY;
          tmax = fmaxf(tmax, val);
        }
      const float mnew = fmaxf(mrun[j], tmax);
      if (mnew != -INFINITY) {
        float ssum = 0.f;
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int v = m0 + wm * G::WM + i * 32 + acc_row(r, l);
            ssum += v < V ? __builtin_amdgcn_exp2f(a[i][j][r] * kLog2e - mnew) : 0.f;
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
          const int local = local0 - i * 32;
          if (local >= 0 && local < 32 && ((local >> 2) & 1) == (l >> 5)) {
            const int rr = (local >> 3) * 4 + (local & 3);
            float z = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) z = r == rr ? a[i][j][r] : z;
            zt_out[n0 + wn * G::WN + j * 32 + (l & 31)] = z;
          }
        }
      }
    }
  };
  G::run_tiles(A, B, H, lds, acc, next, fold);

  // Merge the two lane halves (same token, different vocabulary rows) ...
#pragma unroll
  for (int j = 0; j < G::FN; ++j) {
    const float mo = __shfl_xor(mrun[j], 32);
    const float so = __shfl_xor(srun[j], 32);
    const float M = fmaxf(mrun[j], mo);
    if (M != -INFINITY) {
      srun[j] = srun[j] * __builtin_amdgcn_exp2f(mrun[j] - M) + so * __builtin_amdgcn_exp2f(mo - M);
      mrun[j] = M;
    }
  }
  // ... then the WGM waves that share the token columns, in a fixed order.
  float* sm = reinterpret_cast<float*>(lds);  // [WGM - 1][BN] max, then [WGM - 1][BN] sum
  constexpr int SM = (G::WGM - 1) * kTile;
  if (wm > 0 && l < 32) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      sm[(wm - 1) * kTile + wn * G::WN + j * 32 + l] = mrun[j];
      sm[SM + (wm - 1) * kTile + wn * G::WN + j * 32 + l] = srun[j];
    }
  }
  __syncthreads();
  if (wm == 0 && l < 32) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      float M = mrun[j], S = srun[j];
      for (int q = 0; q < G::WGM - 1; ++q) {
        const float mo = sm[q * kTile + wn * G::WN + j * 32 + l];
        const float so = sm[SM + q * kTile + wn * G::WN + j * 32 + l];
        const float Mn = fmaxf(M, mo);
        if (Mn != -INFINITY) S = S * __builtin_amdgcn_exp2f(M - Mn) + so * __builtin_amdgcn_exp2f(mo - Mn);
        M = Mn;
      }
      const int tok = n0 + wn * G::WN + j * 32 + l;
      if (tok < N) {
        part_m[(int64_t)split * Np + tok] = M;
        part_s[(int64_t)split * Np + tok] = S;
      }
    }
  }
}

__global__ __launch_bounds__(256) void fwd_combine(const float* __restrict__ part_m,
                                                   const float* __restrict__ part_s, int splits, int Np, int N,
                                                   int V, const int64_t* __restrict__ target,
                                                   float* __restrict__ zt, float* __restrict__ lse,
                                                   double* __restrict__ block_loss) {
  __shared__ double red[256];
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  double li = 0.0;
  if (i < N) {
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, part_m[(int64_t)s * Np + i]);
    float S = 0.f;
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
  red[threadIdx.x] = li;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) block_loss[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void fwd_loss(const double* __restrict__ block_loss, int nb, double scale,
                                                float* __restrict__ loss) {
  __shared__ double red[256];
  double a = 0.0;
  for (int b = (int)threadIdx.x; b < nb; b += 256) a += block_loss[b];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(red[0] * scale);
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
// The backward kernels are persistent: one workgroup per CU walks the tiles
// t = lid, lid + G, ... of its launch (lid: XCD-grouped id, G: grid size), each
// tile (tm, tn) taken in the grouped order, so the copy of a tile's first K slice
// overlaps the previous tile's last slice and epilogue.
__device__ __forceinline__ bool persistent_tile(int j, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int G = (int)gridDim.x;
  const int t = xcd_grouped_id((int)blockIdx.x, G) + j * G;
  if (t >= tiles_m * tiles_n) return false;
  grouped_tile(t, tiles_m, tiles_n, tm, tn);
  return true;
}

// Four consecutive float outputs as 4 elements of T (bfloat16: hardware
// round-to-nearest-even conversion), and the 16-byte LDS accesses of the
// dlogit staging below.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){a, b}, bf16x2v_t));
}

// Sᵀ tile: rows = vocabulary (A = W, K-major), cols = tokens (B = x, K-major), as
// in the forward, so lse and target are read once per token column.  The D
// tile goes to the panel [token][vocabulary] through the spare LDS stage: each
// wave owns 8 KiB of it, writes its 64-entry vocabulary span for a round of
// tokens (four consecutive vocabulary entries per lane and accumulator group),
// reads the rows back 16 bytes per lane and stores whole 128-byte lines.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dlogits(const T* __restrict__ x, const T* __restrict__ W,
                                                        const int64_t* __restrict__ target,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ grad_loss, float red_scale, int N,
                                                        int H, int V, int i0, int v0, int tiles_v, int tiles_t,
                                                        int Vbp, T* __restrict__ panel) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, K_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N> G;
  static_assert(G::WM == 64 && G::STAGE_BYTES >= G::NWAVES * 8192, "dlogit staging layout");
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int l = (int)threadIdx.x & 63;
  const int wm = G::wave_m(), wn = G::wave_n();
  const Operand<T> A{W, H, V, H};
  const Operand<T> B{x, H, N, H};
  const float s = grad_loss[0] * red_scale;
  auto next = [&](int j, int& m0, int& n0) {
    int tm, tn;
    if (!persistent_tile(j, tiles_v, tiles_t, tm, tn)) return false;
    m0 = v0 + tm * kTile;
    n0 = i0 + tn * kTile;
    return true;
  };
  constexpr bool BF = sizeof(T) == 2;
  constexpr int RB = 64 * (int)sizeof(T);  // bytes of one token row of a wave's vocabulary span
  constexpr int TR = 8192 / RB;            // tokens per round: 64 (bf16) or 32 (fp32)
  constexpr int JR = TR / 32;              // accumulator column blocks per round
  auto store = [&](typename G::Acc& acc, int m0, int n0, char* spare) {
    char* sc = spare + ((int)threadIdx.x >> 6) * 8192;
    const int vw = m0 + wm * G::WM;  // first vocabulary row of this wave
    // every wave has read its last fragments from spare (the copies still in
    // flight go to the other stage, so no vmcnt wait here)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int rd = 0; rd < G::FN / JR; ++rd) {
#pragma unroll
      for (int jj = 0; jj < JR; ++jj) {
        const int j = rd * JR + jj;
        const int tl = jj * 32 + (l & 31);  // token row within the round
        const int tok = n0 + wn * G::WN + j * 32 + (l & 31);
        const bool tv = tok < N;
        const float lr = tv ? lse[tok] * kLog2e : 0.f;
        const int64_t tt = tv ? target[tok] : -1;
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int vl = i * 32 + 8 * g + 4 * (l >> 5);  // entries vl .. vl + 3 of the span
            float d[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int v = vw + vl + u;
              d[u] = 0.f;
              if (tv && v < V) {
                const float p = __builtin_amdgcn_exp2f(acc[i][j][4 * g + u] * kLog2e - lr);
                d[u] = s * (p - (v == tt ? 1.f : 0.f));
              }
            }
            if constexpr (BF) {
              // 8-byte half of 16-byte slot: slot ^ (tl/2 % 8), half ^ (tl/16 % 2), so the
              // 32 lanes of a write phase (tl = 0..31) hit 32 distinct bank pairs
              const int slot = (vl >> 3) ^ ((tl >> 1) & 7);
              const int half = ((vl >> 2) & 1) ^ ((tl >> 4) & 1);
              *reinterpret_cast<uint2*>(sc + tl * RB + slot * 16 + half * 8) =
                  make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
            } else {
              const int slot = (vl >> 2) ^ (tl & 15);
              *reinterpret_cast<float4*>(sc + tl * RB + slot * 16) = make_float4(d[0], d[1], d[2], d[3]);
            }
          }
      }
      // rows back, 16 bytes per lane, whole rows per group of lanes
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int row, k;
        uint4 v;
        if constexpr (BF) {
          row = q * 8 + (l >> 3);
          k = l & 7;
          v = *reinterpret_cast<const uint4*>(sc + row * RB + ((k ^ ((row >> 1) & 7)) * 16));
          if ((row >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        } else {
          row = q * 4 + (l >> 4);
          k = l & 15;
          v = *reinterpret_cast<const uint4*>(sc + row * RB + ((k ^ (row & 15)) * 16));
        }
        const int tok = n0 + wn * G::WN + rd * TR + row;
        *reinterpret_cast<uint4*>(panel + (int64_t)(tok - i0) * Vbp + (vw - v0) + k * (16 / (int)sizeof(T))) = v;
      }
    }
  };
  typename G::Acc acc;
  G::run_tiles(A, B, H, lds, acc, next, store);
}

// grad_W[v0 + m, h] for m in the panel: A = panel as [k = token][m = vocab]
// (MN-major), B = x rows i0.. as [k = token][n = hidden] (MN-major).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_grad_w(const T* __restrict__ panel, int Vbp, int Kc,
                                                       const T* __restrict__ x, int H, int V, int i0, int v0,
                                                       int Vb, int tiles_m, int tiles_n, T* __restrict__ gw_out,
                                                       float* __restrict__ gw_acc, int accumulate, int final) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, MN_MAJOR, MN_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int l = (int)threadIdx.x & 63;
  const int wm = G::wave_m(), wn = G::wave_n();
  const Operand<T> A{panel, Vbp, Vbp, Kc};
  const Operand<T> B{x + (int64_t)i0 * H, H, H, Kc};
  auto next = [&](int j, int& m0, int& n0) {
    int tm, tn;
    if (!persistent_tile(j, tiles_m, tiles_n, tm, tn)) return false;
    m0 = tm * kTile;
    n0 = tn * kTile;
    return true;
  };
  // gw_out and gw_acc point at row v0 of their buffers; rows are panel-local.
  auto store = [&](typename G::Acc& acc, int m0, int n0, char*) {
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * G::WM + i * 32 + acc_row(r, l);
        if (m >= Vb || v0 + m >= V) continue;
#pragma unroll
        for (int j = 0; j < G::FN; ++j) {
          const int h = n0 + wn * G::WN + j * 32 + (l & 31);
          if (h >= H) continue;
          const int64_t o = (int64_t)m * H + h;
          float val = acc[i][j][r];
          if (accumulate) val += gw_acc[o];
          if (final)
            gw_out[o] = from_f32<T>(val);
          else
            gw_acc[o] = val;
        }
      }
  };
  typename G::Acc acc;
  G::run_tiles(A, B, Kc, lds, acc, next, store);
}

// grad_x[i0 + m, h]: A = panel as [m = token][k = vocab] (K-major), B = W rows
// v0.. as [k = vocab][n = hidden] (MN-major).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_grad_x(const T* __restrict__ panel, int Vbp, int Kc, int Kv,
                                                       const T* __restrict__ W, int H, int N, int i0, int v0,
                                                       int tiles_m, int tiles_n, T* __restrict__ gx_out,
                                                       float* __restrict__ gx_acc, int accumulate, int final) {
  typedef TileGemm<T, kTile, kTile, Cfg<T>::BK, K_MAJOR, MN_MAJOR, Cfg<T>::NS, FLCE_WAVES_M, FLCE_WAVES_N, STAGE_REG>
      G;
  __shared__ __attribute__((aligned(16))) T lds[G::LDS_ELEMS];
  const int l = (int)threadIdx.x & 63;
  const int wm = G::wave_m(), wn = G::wave_n();
  const Operand<T> A{panel, Vbp, Kc, Vbp};
  const Operand<T> B{W + (int64_t)v0 * H, H, H, Kv};
  auto next = [&](int j, int& m0, int& n0) {
    int tm, tn;
    if (!persistent_tile(j, tiles_m, tiles_n, tm, tn)) return false;
    m0 = tm * kTile;
    n0 = tn * kTile;
    return true;
  };
  auto store = [&](typename G::Acc& acc, int m0, int n0, char*) {
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * G::WM + i * 32 + acc_row(r, l);
        if (m >= Kc) continue;
        const int row = i0 + m;
        if (row >= N) continue;
#pragma unroll
        for (int j = 0; j < G::FN; ++j) {
          const int h = n0 + wn * G::WN + j * 32 + (l & 31);
          if (h >= H) continue;
          const int64_t o = (int64_t)row * H + h;
          float val = acc[i][j][r];
          if (accumulate) val += gx_acc[o];
          if (final)
            gx_out[o] = from_f32<T>(val);
          else
            gx_acc[o] = val;
        }
      }
  };
  typename G::Acc acc;
  G::run_tiles(A, B, Kv, lds, acc, next, store);
}

__global__ void fill_scalar(float* p, float v) { p[0] = v; }

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
  hipLaunchKernelGGL(fwd_partial<T>, dim3(grid), dim3(kThreads), 0, st, (const T*)x, (const T*)W, target, N, H, V,
                     p.tiles_tok, p.tiles_per_split, p.Np, part_m, part_s, zt);
  rec.after(FLCE_K_FWD_PARTIAL);
  const int nb = (N + 255) / 256;
  hipLaunchKernelGGL(fwd_combine, dim3(nb), dim3(256), 0, st, part_m, part_s, p.splits, p.Np, N, V, target, zt, lse,
                     block_loss);
  rec.after(FLCE_K_FWD_COMBINE);
  hipLaunchKernelGGL(fwd_loss, dim3(1), dim3(256), 0, st, block_loss, nb, scale, loss);
  rec.after(FLCE_K_FWD_LOSS);
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

template <typename T>
static hipError_t launch_bwd_t(const BwdPlan& p, const void* xv, const void* Wv, const int64_t* target,
                               const float* lse, const float* grad_loss, float red_scale, int N, int H, int V,
                               void* gxv, void* gwv, void* panelv, float* gx_acc, float* gw_acc, hipStream_t st,
                               Recorder& rec) {
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
  for (int pv = 0; pv < p.n_panels; ++pv) {
    const int v0 = pv * p.Vb;
    const int Kv = min(p.Vb, V - v0);
    const int Vbp = p.Vbp;
    for (int c = 0; c < p.n_chunks; ++c) {
      const int i0 = c * p.Nc;
      const int Kc = min(p.Nc, N - i0);
      const int tiles_m = (Kc + kTile - 1) / kTile;
      const int tiles_n = (Kv + kTile - 1) / kTile;
      auto grid = [&](int tiles) { return dim3(min(tiles, p.max_workgroups)); };
      hipLaunchKernelGGL(bwd_dlogits<T>, grid(tiles_m * tiles_n), dim3(kThreads), 0, st, x, W, target, lse, grad_loss,
                         red_scale, N, H, V, i0, v0, tiles_n, tiles_m, Vbp, panel);
      rec.after(FLCE_K_BWD_DLOGITS);
      // grad_W rows of this panel accumulate over token chunks.
      float* gwa = f32 ? gwa0 + (int64_t)v0 * H : gwa0;
      hipLaunchKernelGGL(bwd_grad_w<T>, grid(tiles_n * tiles_h), dim3(kThreads), 0, st, (const T*)panel, Vbp, Kc, x, H,
                         V, i0, v0, Kv, tiles_n, tiles_h, gw + (int64_t)v0 * H, gwa, c > 0 ? 1 : 0,
                         c == p.n_chunks - 1 ? 1 : 0);
      rec.after(FLCE_K_BWD_GRAD_W);
      // grad_x rows of this chunk accumulate over vocabulary panels.
      hipLaunchKernelGGL(bwd_grad_x<T>, grid(tiles_m * tiles_h), dim3(kThreads), 0, st, (const T*)panel, Vbp, Kc, Kv, W,
                         H, N, i0, v0, tiles_m, tiles_h, gx, gxa, pv > 0 ? 1 : 0, pv == p.n_panels - 1 ? 1 : 0);
      rec.after(FLCE_K_BWD_GRAD_X);
    }
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : rec.err;
}

hipError_t launch_backward(int dt, const BwdPlan& p, const void* x, const void* W, const int64_t* target,
                           const float* lse, const float* grad_loss, float red_scale, int N, int H, int V, void* gx,
                           void* gw, void* panel, float* gx_acc, float* gw_acc, hipStream_t st,
                           Recorder& rec) {
  return dt == 1 ? launch_bwd_t<bf16_t>(p, x, W, target, lse, grad_loss, red_scale, N, H, V, gx, gw, panel, gx_acc,
                                        gw_acc, st, rec)
                 : launch_bwd_t<float>(p, x, W, target, lse, grad_loss, red_scale, N, H, V, gx, gw, panel, gx_acc,
                                       gw_acc, st, rec);
}

}  // namespace flce
