// Tiled MFMA contraction core for gfx950 (CDNA4, wave64).
//
// One workgroup of 256 threads (4 waves in a 2 x 2 grid) computes a BM x BN
// float32 tile C[m][n] = sum_k A(m, k) * B(n, k) into registers, streaming K in
// BK-wide slices through double-buffered LDS.  Each operand is stored either
// K-major ([mn][k], k contiguous, e.g. x [N,H] and W [V,H] contracted over H) or
// MN-major ([k][mn], mn contiguous, e.g. W [V,H] contracted over V).
//
// bfloat16 uses v_mfma_f32_32x32x16_bf16; float32 uses v_mfma_f32_32x32x2f32.
// Lane layouts (checked on the device):
//   A operand: lane l holds row m = l % 32, k = KPL * (l / 32) + [0, KPL)
//   B operand: lane l holds col n = l % 32, k = KPL * (l / 32) + [0, KPL)
//   C / acc  : lane l, register r holds row 8 (r / 4) + 4 (l / 32) + r % 4, col l % 32
// with KPL = 8 for bfloat16 and 1 for float32.  MN-major bfloat16 fragments are
// read with ds_read_b64_tr_b16, which, within each 16-lane group, returns to
// lane i element j of the 4-element chunk that lane 4 j + i / 4 addressed,
// position i % 4; pointing lane s at row k0 + s / 4, columns c0 + 4 (s % 4) thus
// gives lane i the column c0 + i for rows k0 .. k0 + 3.
//
// Out-of-range rows (mn >= mn_ext) and K slices (k >= k_ext) are zero-filled in
// LDS, never read from memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef uint16_t bf16_t;  // bfloat16 storage bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

enum Major { K_MAJOR = 0, MN_MAJOR = 1 };

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<bf16_t> {
  static constexpr int VEC = 8;     // elements per 16-byte chunk
  static constexpr int KSTEP = 16;  // k per MFMA
};
template <>
struct ElemTraits<float> {
  static constexpr int VEC = 4;
  static constexpr int KSTEP = 2;
};

// A strided view of one contraction operand.
template <typename T>
struct Operand {
  const T* ptr;  // element (mn = 0, k = 0)
  int64_t ld;    // elements between consecutive storage rows
  int mn_ext;    // rows/cols [0, mn_ext) are valid
  int k_ext;     // k in [0, k_ext) is valid
};

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }

// Row (within the 32 x 32 block) of accumulator register r in lane l.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <typename T, int BM_, int BN_, int BK_, int AMAJ, int BMAJ>
struct TileGemm {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int NT = 256;
  static constexpr int VEC = ElemTraits<T>::VEC;
  static constexpr int KSTEP = ElemTraits<T>::KSTEP;
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  static constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BK % KSTEP == 0 && BK % VEC == 0, "BK");

  static constexpr int A_ROWS = AMAJ == K_MAJOR ? BM : BK;
  static constexpr int A_COLS = AMAJ == K_MAJOR ? BK : BM;
  static constexpr int B_ROWS = BMAJ == K_MAJOR ? BN : BK;
  static constexpr int B_COLS = BMAJ == K_MAJOR ? BK : BN;
  static constexpr int A_PITCH = A_COLS + VEC;  // 16-byte pad against bank conflicts
  static constexpr int B_PITCH = B_COLS + VEC;
  static constexpr int A_STAGE = A_ROWS * A_PITCH;
  static constexpr int B_STAGE = B_ROWS * B_PITCH;
  static constexpr int LDS_ELEMS = 2 * (A_STAGE + B_STAGE);
  static constexpr int LDS_BYTES = LDS_ELEMS * (int)sizeof(T);
  static constexpr int A_CH = A_ROWS * A_COLS / VEC / NT;  // 16-byte chunks per thread
  static constexpr int B_CH = B_ROWS * B_COLS / VEC / NT;
  static_assert(A_ROWS * A_COLS % (VEC * NT) == 0 && B_ROWS * B_COLS % (VEC * NT) == 0, "chunks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  typedef f32x16_t Acc[FM][FN];

  template <int MAJ, int COLS, int NCH>
  static __device__ __forceinline__ void gload(const Operand<T>& op, int mn0, int k0, u32x4_t (&r)[NCH]) {
    constexpr int CPR = COLS / VEC;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = (int)threadIdx.x + c * NT;
      const int row = ch / CPR, col = (ch % CPR) * VEC;
      const int mn = MAJ == K_MAJOR ? mn0 + row : mn0 + col;
      const int k = MAJ == K_MAJOR ? k0 + col : k0 + row;
      r[c] = u32x4_t{0u, 0u, 0u, 0u};
      if (mn < op.mn_ext && k < op.k_ext) {
        const int64_t off = MAJ == K_MAJOR ? (int64_t)mn * op.ld + k : (int64_t)k * op.ld + mn;
        r[c] = *reinterpret_cast<const u32x4_t*>(op.ptr + off);
      }
    }
  }

  template <int COLS, int PITCH, int NCH>
  static __device__ __forceinline__ void lstore(T* s, const u32x4_t (&r)[NCH]) {
    constexpr int CPR = COLS / VEC;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = (int)threadIdx.x + c * NT;
      const int row = ch / CPR, col = (ch % CPR) * VEC;
      *reinterpret_cast<u32x4_t*>(s + row * PITCH + col) = r[c];
    }
  }

  // bfloat16 operand fragment for the 32-wide block starting at mnb, k slice kk.
  template <int MAJ, int PITCH>
  static __device__ __forceinline__ bf16x8_t frag(const bf16_t* s, int mnb, int kk) {
    const int l = (int)threadIdx.x & 63;
    if (MAJ == K_MAJOR) {
      return *reinterpret_cast<const bf16x8_t*>(s + (mnb + (l & 31)) * PITCH + kk + 8 * (l >> 5));
    } else {
      const int g = l >> 4, q = l & 15;
      const int col = mnb + 16 * (g & 1) + 4 * (q & 3);
      const int row = kk + 8 * (g >> 1) + (q >> 2);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(s + row * PITCH + col));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(s + (row + 4) * PITCH + col));
      const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // float32 operand fragment (one k per lane).
  template <int MAJ, int PITCH>
  static __device__ __forceinline__ float frag(const float* s, int mnb, int kk) {
    const int l = (int)threadIdx.x & 63;
    return MAJ == K_MAJOR ? s[(mnb + (l & 31)) * PITCH + kk + (l >> 5)]
                          : s[(kk + (l >> 5)) * PITCH + mnb + (l & 31)];
  }

  static __device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16_t mfma(float a, float b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }

  // acc = A[m0:m0+BM, 0:K] . B[n0:n0+BN, 0:K]^T.  Ends with a barrier, so the caller
  // may reuse the LDS right after.
  static __device__ __forceinline__ void run(const Operand<T>& A, const Operand<T>& B, int m0, int n0,
                                             int K, T* lds, Acc& acc) {
    const int w = (int)threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    T* As[2] = {lds, lds + A_STAGE + B_STAGE};
    T* Bs[2] = {lds + A_STAGE, lds + 2 * A_STAGE + B_STAGE};
    u32x4_t ra[A_CH], rb[B_CH];
    const int KT = (K + BK - 1) / BK;
    gload<AMAJ, A_COLS, A_CH>(A, m0, 0, ra);
    gload<BMAJ, B_COLS, B_CH>(B, n0, 0, rb);
    lstore<A_COLS, A_PITCH, A_CH>(As[0], ra);
    lstore<B_COLS, B_PITCH, B_CH>(Bs[0], rb);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        gload<AMAJ, A_COLS, A_CH>(A, m0, (kt + 1) * BK, ra);
        gload<BMAJ, B_COLS, B_CH>(B, n0, (kt + 1) * BK, rb);
      }
      const T* as = As[cur];
      const T* bs = Bs[cur];
#pragma unroll
      for (int kk = 0; kk < BK; kk += KSTEP) {
        decltype(frag<AMAJ, A_PITCH>(as, 0, 0)) fa[FM];
        decltype(frag<BMAJ, B_PITCH>(bs, 0, 0)) fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = frag<AMAJ, A_PITCH>(as, wm * WM + i * 32, kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = frag<BMAJ, B_PITCH>(bs, wn * WN + j * 32, kk);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
      }
      if (more) {
        lstore<A_COLS, A_PITCH, A_CH>(As[cur ^ 1], ra);
        lstore<B_COLS, B_PITCH, B_CH>(Bs[cur ^ 1], rb);
      }
      __syncthreads();
    }
  }
};

// Logical workgroup id whose consecutive values run on the same XCD: the
// hardware hands workgroup b to XCD b % 8, so XCD x receives b = x, x + 8, ...
__device__ __forceinline__ int xcd_grouped_id(int b, int G) {
  const int q = G >> 3, r = G & 7;
  const int x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

}  // namespace flce
