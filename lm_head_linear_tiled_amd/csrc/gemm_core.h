// Tiled MFMA contraction core for gfx950 (CDNA4, wave64).
//
// One workgroup of WGM x WGN waves computes a BM x BN
// float32 tile C[m][n] = sum_k A(m, k) * B(n, k) into registers, streaming K in
// BK-wide slices through double-buffered LDS.  Each operand is stored either
// K-major ([mn][k], k contiguous, e.g. x [N,H] and W [V,H] contracted over H) or
// MN-major ([k][mn], mn contiguous, e.g. W [V,H] contracted over V).
//
// The MFMA shape is a parameter MI: MI x MI output blocks.  MI = 32: bfloat16
// uses v_mfma_f32_32x32x16_bf16, float32 v_mfma_f32_32x32x2f32; MI = 16
// (bfloat16 only): v_mfma_f32_16x16x32_bf16.  Lane layouts (checked on the device):
//   MI = 32:  A operand: lane l holds row m = l % 32, k = KPL * (l / 32) + [0, KPL)
//             B operand: lane l holds col n = l % 32, k = KPL * (l / 32) + [0, KPL)
//             C / acc  : lane l, register r holds row 8 (r / 4) + 4 (l / 32) + r % 4, col l % 32
//             with KPL = 8 for bfloat16 and 1 for float32;
//   MI = 16:  A operand: lane l holds row m = l % 16, k = 8 (l / 16) + [0, 8)
//             B operand: lane l holds col n = l % 16, k = 8 (l / 16) + [0, 8)
//             C / acc  : lane l, register r (of 4) holds row 4 (l / 16) + r, col l % 16.
// Either way a lane holds runs of four consecutive rows of one column.  At the
// chip's power limit the 16 x 16 form sustains more bfloat16 MFMA throughput (it
// moves half the accumulator registers per multiply-add).  MN-major bfloat16
// fragments are read with ds_read_b64_tr_b16, which, within each 16-lane group,
// returns to lane i element j of the 4-element chunk that lane 4 j + i / 4
// addressed, position i % 4; pointing lane s at row k0 + s / 4, columns
// c0 + 4 (s % 4) thus gives lane i the column c0 + i for rows k0 .. k0 + 3.
//
// Out-of-range rows (mn >= mn_ext) and K slices (k >= k_ext) are zero-filled in
// LDS by the buffer unit's range check, never read from memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace flce {

typedef uint16_t bf16_t;  // bfloat16 storage bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

enum Major { K_MAJOR = 0, MN_MAJOR = 1 };

// Measurement builds only (FLCE_TILE_CLOCK=1): every persistent tile loop
// records, for workgroup b < 256 and its items j < 64, the shader clock
// (s_memtime, a per-CU counter: only differences within a workgroup mean
// anything) at the start of the item's first K slice, after that slice, after
// its last slice and after its epilogue, and its slice count, in
// tile_clock[kind][b][j]; kind 0: register-staged with both operands MN-major
// (grad_W), 1: register-staged with B K-major (grad_x), 2: DMA copies by copy
// waves with separate store waves (dlogits), 3: other DMA kernels (the forward,
// the dlogit tail pieces).  Every launch overwrites the entries of the items it
// runs.
#ifndef FLCE_TILE_CLOCK
#define FLCE_TILE_CLOCK 0
#endif
#if FLCE_TILE_CLOCK
__device__ unsigned long long tile_clock[4][256][64][5];
#endif

#ifndef FLCE_COPY_STEPS
#define FLCE_COPY_STEPS 0
#endif

// Compile-time loop: f(std::integral_constant<int, i>) for i in [0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_<0, N>(f); }

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

// A strided view of one contraction operand, optionally in blocks along K: K
// offsets [b ksplit, (b + 1) ksplit) live at ptr + b jump as the view of
// k - b ksplit (ksplit a multiple of the K slice, so no slice straddles a block).
template <typename T>
struct Operand {
  const T* ptr;  // element (mn = 0, k = 0)
  int64_t ld;    // elements between consecutive storage rows
  int mn_ext;    // rows/cols [0, mn_ext) are valid
  int k_ext;     // k in [0, k_ext) is valid
  int ksplit = 0x7fffffff;
  int64_t jump = 0;
  // origin of the block holding K offset k0 (wave-uniform), k0 made block-relative
  __device__ __forceinline__ const T* block(int& k0) const {
    const T* p = ptr;
    while (k0 >= ksplit) {
      k0 -= ksplit;
      p += jump;
    }
    return p;
  }
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

// LDS layout.  Tiles are stored unpadded in rows of 16-byte slots; the slot index
// is XOR-swizzled with a function of the row so that the fragment reads below hit
// distinct banks (64 banks of 4 bytes: 256 bytes per bank cycle):
//   K-major tile  [mn][k], RB-byte rows (RB = BK * sizeof(T), 64 or 128): the
//       256 / RB rows that share a bank cycle differ in bank half / quarter, and
//       slot ^ ((row / (256 / RB)) % (RB / 16)) spreads the next rows over slots;
//   MN-major tile [k][mn], bfloat16 (512-byte rows):  slot ^ (4 (row & 3)) for
//       MI = 32 (a 32-lane pass reads 4 rows at two column offsets), and
//       slot ^ (2 (row & 3) + 8 ((row / 8) & 1)) for MI = 16 (a pass reads rows
//       k .. k + 3 and k + 8 .. k + 11 at one column offset);
//   MN-major tile [k][mn], float32 (1024-byte rows):  slot ^ (8 (row & 1))
template <typename T, int MAJ, int RB, int MI = 32>
__device__ __forceinline__ int swz(int row) {
  if (MAJ == K_MAJOR) return (row / (256 / RB)) % (RB / 16);
  if (sizeof(T) == 4) return 8 * (row & 1);
  return MI == 16 ? 2 * (row & 3) + 8 * ((row >> 3) & 1) : 4 * (row & 3);
}

// How a K slice travels from global memory to LDS.
enum Staging {
  STAGE_DMA = 0,  // buffer_load ... lds: straight into LDS, no registers
  STAGE_REG = 1   // 16-byte buffer loads into registers, then ds_write_b128
};

// SPLIT (DMA staging only): the first half of the waves issue every K-slice copy
// and are the only ones that wait for copies; the second half issue none, so
// global stores they leave in flight (an epilogue's) are never waited for by the
// tile loop -- the memory counter that copies are awaited with also counts
// stores, in issue order.
template <typename T, int BM_, int BN_, int BK_, int AMAJ, int BMAJ, int NSTAGE_ = 2, int WGM_ = 2, int WGN_ = 2,
          int STAGING = STAGE_DMA, bool SPLIT = false, int MI_ = 32>
struct TileGemm {
  static constexpr int MI = MI_;  // MFMA output block: MI x MI
  static_assert(MI == 32 || (MI == 16 && sizeof(T) == 2), "16 x 16 blocks for bfloat16 only");
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int NSTAGE = NSTAGE_;  // LDS stages: NSTAGE - 1 K slices in flight
  static constexpr int WGM = WGM_, WGN = WGN_;  // wave grid over the tile
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int NT = 64 * NWAVES;
  static constexpr int NCW = SPLIT ? NWAVES / 2 : NWAVES;  // waves that issue copies
  static_assert(!SPLIT || STAGING == STAGE_DMA, "split copy/store waves need DMA staging");
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VEC = ElemTraits<T>::VEC;
  static constexpr int KSTEP = MI == 16 ? 32 : ElemTraits<T>::KSTEP;  // k per MFMA
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int FM = WM / MI, FN = WN / MI;
  static_assert(WM % MI == 0 && WN % MI == 0, "wave tile must be a multiple of the MFMA block");
  // accumulator registers per block, and the runs of four consecutive rows among them
  static constexpr int NR = MI * MI / 64, NG = NR / 4;
  // first row (within its block) of run g of lane l, and the block row / column of
  // accumulator register r of lane l
  static __device__ __forceinline__ int qrow(int g, int l) { return MI == 32 ? 8 * g + 4 * (l >> 5) : 4 * (l >> 4); }
  static __device__ __forceinline__ int acc_m(int r, int l) { return qrow(r >> 2, l) + (r & 3); }
  static __device__ __forceinline__ int acc_n(int l) { return l & (MI - 1); }
  static_assert(BK * ES == 128 || BK * ES == 64, "K-major rows are 64 or 128 bytes");

  static constexpr int A_BYTES = BM * BK * ES;
  static constexpr int B_BYTES = BN * BK * ES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  static constexpr int LDS_ELEMS = LDS_BYTES / ES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(A_BYTES % (NCW * 1024) == 0 && B_BYTES % (NCW * 1024) == 0, "whole 1 KiB wave loads");

  // Does this wave issue K-slice copies?  (wave-uniform)
  static __device__ __forceinline__ bool copy_wave() { return !SPLIT || ((int)threadIdx.x >> 6) < NCW; }

  static __device__ __forceinline__ int wave_m() { return ((int)threadIdx.x >> 6) / WGN; }
  static __device__ __forceinline__ int wave_n() { return ((int)threadIdx.x >> 6) % WGN; }

  typedef std::conditional_t<MI == 32, f32x16_t, f32x4_t> AccT;
  typedef AccT Acc[FM][FN];

  // Row length in bytes of an operand tile stored with major MAJ and mn extent MNT.
  template <int MAJ, int MNT>
  static constexpr int row_bytes() { return MAJ == K_MAJOR ? BK * ES : MNT * ES; }

  // Enqueue the global -> LDS copy of one operand tile (rows mn0.., K slice k0..).
  // Every lane moves one 16-byte chunk per instruction straight into LDS
  // (buffer_load ... lds: lane l of a wave instruction lands at M0 + 16 l); chunks
  // outside the valid range get an offset past the buffer bound, which the
  // hardware reads as zeros.  Completion is awaited by the barrier's vmcnt(0).
  template <int MAJ, int MNT, int J0 = 0, int J1 = MNT * BK * ES / 1024 / NCW, bool LEAN = false>
  static __device__ __forceinline__ void load_tile(const Operand<T>& op, int mn0, int k0, T* lds_op) {
    constexpr int RB = row_bytes<MAJ, MNT>();
    constexpr int SLOTS = RB / 16;
    if constexpr (J0 >= J1) return;
    const int l = (int)threadIdx.x & 63;
    if constexpr (LEAN) {
      // Whole K slice of a K-major operand (k0 + BK <= k_ext <= ld, checked by the
      // caller): the descriptor starts at row mn0 (k = 0) and ends after its last
      // valid row, so rows past mn_ext fail the range check and read zeros, and
      // every other bound holds.  Copy j of a wave reads rows ROWS_J further down
      // than copy j - 1 with the same swizzled slot, so its lane offset is the
      // first one plus a scalar: no per-copy address math.
      static_assert(MAJ == K_MAJOR, "lean copies are K-major");
      constexpr int ROWS_J = NCW * 64 / SLOTS;
      static_assert((NCW * 4) % (RB / 16) == 0, "copy j keeps the swizzled slot of copy 0");
      const uint32_t ldb = (uint32_t)(op.ld * ES);  // at most 8 MiB: offsets stay below 2^31 + 2^23
      const int rows = op.mn_ext - mn0 < MNT ? op.mn_ext - mn0 : MNT;
      const uint32_t num = rows > 0 ? (uint32_t)rows * ldb : 0u;
      const T* const org = op.block(k0);
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)(org + (int64_t)mn0 * op.ld), (short)0, num, 0x00020000);
      const int w = (int)threadIdx.x >> 6;
      const int row0 = (J0 * NCW + w) * (64 / SLOTS) + l / SLOTS;
      const uint32_t off0 = (uint32_t)row0 * ldb + 16u * (uint32_t)((l % SLOTS) ^ swz<T, MAJ, RB, MI>(row0));
      const int ws = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
      for (int j = J0; j < J1; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)((char*)lds_op + (j * NCW + ws) * 1024), 16,
            off0 + (uint32_t)((j - J0) * ROWS_J) * ldb, k0 * ES, 0, 0);
      return;
    }
    const int w = (int)threadIdx.x >> 6;
    const int kg = k0;  // K offset for the bounds check
    const T* const org = op.block(k0);
    const T* base = MAJ == K_MAJOR ? org + (int64_t)mn0 * op.ld + k0 : org + (int64_t)k0 * op.ld + mn0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7ffffff0, 0x00020000);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int blk = j * NCW + w;  // 1 KiB block of the tile
      const int chunk = blk * 64 + l;
      const int row = chunk / SLOTS;
      const int slot = (chunk % SLOTS) ^ swz<T, MAJ, RB, MI>(row);
      const int mn = MAJ == K_MAJOR ? mn0 + row : mn0 + slot * VEC;
      const int k = MAJ == K_MAJOR ? kg + slot * VEC : kg + row;
      const bool ok = mn < op.mn_ext && k < op.k_ext;
      const uint32_t off = (uint32_t)(((int64_t)row * op.ld + slot * VEC) * ES);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)((char*)lds_op + blk * 1024), 16, ok ? off : 0x80000000u, 0,
          0, 0);
    }
  }

  // bfloat16 operand fragment for the 32-wide block starting at mnb, k slice kk.
  template <int MAJ, int MNT>
  static __device__ __forceinline__ bf16x8_t frag(const bf16_t* s, int mnb, int kk) {
    constexpr int RB = row_bytes<MAJ, MNT>();
    const char* sb = (const char*)s;
    const int l = (int)threadIdx.x & 63;
    if (MAJ == K_MAJOR) {
      const int row = mnb + (l & (MI - 1));
      const int slot = (kk >> 3) + (MI == 32 ? (l >> 5) : (l >> 4));
      return *reinterpret_cast<const bf16x8_t*>(sb + row * RB + 16 * (slot ^ swz<bf16_t, MAJ, RB, MI>(row)));
    } else {
      const int g = l >> 4, q = l & 15;
      const int col = MI == 32 ? mnb + 16 * (g & 1) + 4 * (q & 3) : mnb + 4 * (q & 3);
      const int row = MI == 32 ? kk + 8 * (g >> 1) + (q >> 2) : kk + 8 * g + (q >> 2);
      const int cb = 16 * ((col >> 3) ^ swz<bf16_t, MAJ, RB, MI>(row)) + 2 * (col & 7);  // same swizzle for row + 4
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(sb + row * RB + cb));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(sb + (row + 4) * RB + cb));
      const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // float32 operand fragment (one k per lane).
  template <int MAJ, int MNT>
  static __device__ __forceinline__ float frag(const float* s, int mnb, int kk) {
    constexpr int RB = row_bytes<MAJ, MNT>();
    const char* sb = (const char*)s;
    const int l = (int)threadIdx.x & 63;
    if (MAJ == K_MAJOR) {
      const int row = mnb + (l & 31), k = kk + (l >> 5);
      return *reinterpret_cast<const float*>(sb + row * RB + 16 * ((k >> 2) ^ swz<float, MAJ, RB, MI>(row)) + 4 * (k & 3));
    } else {
      const int row = kk + (l >> 5), col = mnb + (l & 31);
      return *reinterpret_cast<const float*>(sb + row * RB + 16 * ((col >> 2) ^ swz<float, MAJ, RB, MI>(row)) + 4 * (col & 3));
    }
  }

  static __device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16_t mfma(float a, float b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }

  // LDS read instructions per fragment step, MFMAs per step, global loads per K slice.
  static constexpr int DS_A = (AMAJ == MN_MAJOR && ES == 2) ? 2 : 1;
  static constexpr int DS_B = (BMAJ == MN_MAJOR && ES == 2) ? 2 : 1;
  static constexpr int N_DS = FM * DS_A + FN * DS_B;
  static constexpr int N_MFMA = FM * FN;
  static constexpr int N_VMEM = (BM + BN) * BK * ES / 1024 / NCW;

  // The copies of one K slice (A's then B's wave instructions, N_VMEM in all) are
  // spread over the first VSTEPS fragment steps, VPER per step, so that the eight
  // waves do not flood the texture-address queue at the start of a slice
  // (FLCE_COPY_STEPS > 0: over that many steps instead, a measurement knob).
  static constexpr int NSTEP_ = BK / KSTEP;
  static constexpr int VSTEPS = FLCE_COPY_STEPS > 0 && FLCE_COPY_STEPS < NSTEP_ ? FLCE_COPY_STEPS
                                : (NSTEP_ > 1 ? NSTEP_ - 1 : 1);
  static constexpr int VPER = (N_VMEM + VSTEPS - 1) / VSTEPS;
  static constexpr int INSTR_A = BM * BK * ES / 1024 / NCW;

  // Register-staged copies: buffer loads (out-of-range lanes read zeros) into
  // registers, written to the same swizzled LDS slots later.
  template <int MAJ, int MNT, int J0, int J1, bool LEAN = false>
  static __device__ __forceinline__ void rload(const Operand<T>& op, int mn0, int k0, u32x4_t* r) {
    constexpr int RB = row_bytes<MAJ, MNT>();
    constexpr int SLOTS = RB / 16;
    if constexpr (J0 >= J1) return;
    if constexpr (LEAN) {
      // As the lean DMA copies (load_tile): one lane offset, copy j ROWS_J storage
      // rows further.  K-major: rows past mn_ext fail the descriptor's range
      // check; MN-major (whole tile inside mn_ext, whole K slice): every chunk is
      // inside the operand.
      constexpr int ROWS_J = NWAVES * 64 / SLOTS;
      static_assert(MAJ == K_MAJOR ? ROWS_J % (256 / RB) == 0 && (ROWS_J / (256 / RB)) % (RB / 16) == 0
                                   : ROWS_J % (ES == 2 ? (MI == 16 ? 16 : 4) : 2) == 0,
                    "copy j keeps the swizzled slot of copy 0");
      const int l = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
      const uint32_t ldb = (uint32_t)(op.ld * ES);  // at most 8 MiB: offsets stay below 2^31 + 2^23
      const T* const org = op.block(k0);
      __amdgpu_buffer_rsrc_t rsrc;
      uint32_t soff;
      if constexpr (MAJ == K_MAJOR) {
        const int rows = op.mn_ext - mn0 < MNT ? op.mn_ext - mn0 : MNT;
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(org + (int64_t)mn0 * op.ld), (short)0,
                                                 rows > 0 ? (uint32_t)rows * ldb : 0u, 0x00020000);
        soff = (uint32_t)(k0 * ES);
      } else {
        // the tile's BK rows of MNT elements; none if it lies past mn_ext (the
        // copy cursor's origin past the last tile)
        const bool in = mn0 + MNT <= op.mn_ext;
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(org + (int64_t)k0 * op.ld + mn0), (short)0,
                                                 in ? (uint32_t)(BK - 1) * ldb + MNT * ES : 0u, 0x00020000);
        soff = 0;
      }
      const int row0 = (J0 * NWAVES + w) * (64 / SLOTS) + l / SLOTS;
      const uint32_t off0 = (uint32_t)row0 * ldb + 16u * (uint32_t)((l % SLOTS) ^ swz<T, MAJ, RB, MI>(row0));
#pragma unroll
      for (int j = J0; j < J1; ++j)
        r[j - J0] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off0 + (uint32_t)((j - J0) * ROWS_J) * ldb, soff, 0));
      return;
    }
    const int l = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
    const int kg = k0;  // K offset for the bounds check
    const T* const org = op.block(k0);
    const T* base = MAJ == K_MAJOR ? org + (int64_t)mn0 * op.ld + k0 : org + (int64_t)k0 * op.ld + mn0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7ffffff0, 0x00020000);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int blk = j * NWAVES + w;
      const int chunk = blk * 64 + l;
      const int row = chunk / SLOTS;
      const int slot = (chunk % SLOTS) ^ swz<T, MAJ, RB, MI>(row);
      const int mn = MAJ == K_MAJOR ? mn0 + row : mn0 + slot * VEC;
      const int k = MAJ == K_MAJOR ? kg + slot * VEC : kg + row;
      const bool ok = mn < op.mn_ext && k < op.k_ext;
      const uint32_t off = (uint32_t)(((int64_t)row * op.ld + slot * VEC) * ES);
      r[j - J0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, ok ? off : 0x80000000u, 0, 0));
    }
  }
  template <int MNT, int J0, int J1>
  static __device__ __forceinline__ void rstore(T* lds_op, const u32x4_t* r) {
    const int l = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
#pragma unroll
    for (int j = J0; j < J1; ++j)
      *reinterpret_cast<u32x4_t*>((char*)lds_op + (j * NWAVES + w) * 1024 + 16 * l) = r[j - J0];
  }

  // Issue copy instructions [C0, C1) of the combined A-then-B sequence.
  template <int C0, int C1, bool LEAN>
  static __device__ __forceinline__ void load_part(const Operand<T>& A, const Operand<T>& B, int m0, int n0, int k0,
                                                   T* stage) {
    constexpr int A0 = C0 < INSTR_A ? C0 : INSTR_A, A1 = C1 < INSTR_A ? C1 : INSTR_A;
    constexpr int B0 = (C0 > INSTR_A ? C0 : INSTR_A) - INSTR_A, B1 = (C1 > INSTR_A ? C1 : INSTR_A) - INSTR_A;
    load_tile<AMAJ, BM, A0, A1, LEAN>(A, m0, k0, stage);
    load_tile<BMAJ, BN, B0, B1, LEAN>(B, n0, k0, stage + A_BYTES / ES);
  }

  template <int S, bool LEAN>
  static __device__ __forceinline__ void load_step(const Operand<T>& A, const Operand<T>& B, int m0, int n0, int k0,
                                                   T* stage) {
    constexpr int C0 = S * VPER < N_VMEM ? S * VPER : N_VMEM;
    constexpr int C1 = (S + 1) * VPER < N_VMEM ? (S + 1) * VPER : N_VMEM;
    if constexpr (S < VSTEPS) load_part<C0, C1, LEAN>(A, B, m0, n0, k0, stage);
  }
  static constexpr int vmem_in_step(int s) {
    return s < VSTEPS ? ((s + 1) * VPER < N_VMEM ? (s + 1) * VPER : N_VMEM) - (s * VPER < N_VMEM ? s * VPER : N_VMEM)
                      : 0;
  }

  // One scheduling pattern per fragment step: after each of the step's N_MFMA
  // MFMAs, first up to RPER of the NR LDS reads (the next step's fragments, so
  // they are in flight as early as possible), then, once those are placed, the NV
  // global loads / DMA copies and the NW LDS writes spread over the remaining
  // MFMAs.  RPER: 3 with DMA copies, 2 with register staging (measured best).
  template <int NR, int NV, int NW>
  static __device__ __forceinline__ void schedule_step() {
    constexpr int RPER = STAGING == STAGE_DMA ? 3 : 2;
    constexpr int QR = (NR + RPER - 1) / RPER;              // MFMA slots taken by the reads
    constexpr int REST = N_MFMA - QR > 0 ? N_MFMA - QR : 1;  // slots left for the rest
    constexpr int VPER_ = (NV + REST - 1) / REST;
    constexpr int WPER_ = (NW + REST - 1) / REST;
    static_for<N_MFMA>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int r = NR - RPER * q < RPER ? (NR - RPER * q > 0 ? NR - RPER * q : 0) : RPER;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      constexpr int k = q - QR;  // index among the remaining slots
      if constexpr (k >= 0) {
        constexpr int v = NV - VPER_ * k < VPER_ ? (NV - VPER_ * k > 0 ? NV - VPER_ * k : 0) : VPER_;
        constexpr int w = NW - WPER_ * k < WPER_ ? (NW - WPER_ * k > 0 ? NW - WPER_ * k : 0) : WPER_;
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
        if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);
      }
    });
    // anything that did not fit (fewer MFMAs than reads) goes last
    constexpr int RLEFT = NR - RPER * N_MFMA > 0 ? NR - RPER * N_MFMA : 0;
    if constexpr (RLEFT > 0) __builtin_amdgcn_sched_group_barrier(0x100, RLEFT, 0);
    constexpr int VLEFT = N_MFMA <= QR ? NV : 0, WLEFT = N_MFMA <= QR ? NW : 0;
    if constexpr (VLEFT > 0) __builtin_amdgcn_sched_group_barrier(0x020, VLEFT, 0);
    if constexpr (WLEFT > 0) __builtin_amdgcn_sched_group_barrier(0x200, WLEFT, 0);
  }

  // Scheduling groups: spread NI instructions of class MASK evenly between the
  // N_MFMA MFMAs of one step.
  template <int NI, int MASK>
  static __device__ __forceinline__ void interleave() {
    constexpr int PER = NI >= N_MFMA ? NI / N_MFMA : 1;
    constexpr int EVERY = NI >= N_MFMA ? 1 : N_MFMA / NI;
#pragma unroll
    for (int q = 0; q < N_MFMA; q += EVERY) {
      __builtin_amdgcn_sched_group_barrier(0x008, EVERY, 0);
      __builtin_amdgcn_sched_group_barrier(MASK, PER, 0);
    }
  }

  typedef decltype(frag<AMAJ, BM>((const T*)nullptr, 0, 0)) FragA;
  typedef decltype(frag<BMAJ, BN>((const T*)nullptr, 0, 0)) FragB;

  static __device__ __forceinline__ void load_frags(const T* as, const T* bs, int wm, int wn, int kk, FragA (&fa)[FM],
                                                    FragB (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = frag<AMAJ, BM>(as, wm * WM + i * MI, kk);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = frag<BMAJ, BN>(bs, wn * WN + j * MI, kk);
  }

  // Wait until at most N of this wave's global -> LDS copies are outstanding, then
  // meet the other waves.  The asm is also a compiler memory barrier.
  template <int N>
  static __device__ __forceinline__ void wait_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    if constexpr (STAGING == STAGE_REG)  // the staged ds_writes must also have landed
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
    else if (copy_wave())
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
    else
      asm volatile("s_barrier" ::: "memory");
  }

  static __device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.f;
  }

  // Multiply one K slice held in LDS stage `cur` into acc while the copy of the
  // next slice (origin pm0/pn0, K offset pk0) goes into the other stage: the
  // copies are spread over the first fragment steps (DMA) or loaded at the first
  // step and written at the last (register staging), and the LDS fragment reads of
  // step s+1 are interleaved with the MFMAs of step s.
  // The slice with 16 x 16 blocks (DMA staging): FM x FN = 4 x 8 MFMAs per
  // fragment step, issued column by column (acc[.][j] for B fragment j), so B
  // fragment j is dead after its column and the next step's B fragment j is read
  // into the same registers right after it; only the 4 A fragments are double
  // buffered (64 fragment registers instead of 96 next to the 128 accumulator
  // registers).  The instruction order is fixed column by column (a scheduling
  // barrier after each): the column's MFMAs, then its next-step reads (B j, and
  // A j for the first FM columns), then its share of the slice's copies (in the
  // first VSTEPS steps).
  template <bool LEAN, bool COPY>
  static __device__ __forceinline__ void slice16(const Operand<T>& A, const Operand<T>& B, T* lds, int cur, int pm0,
                                                 int pn0, int pk0, Acc& acc) {
    static_assert(MI == 16 && STAGING == STAGE_DMA, "16 x 16 slice: DMA staging");
    constexpr int STAGE = STAGE_BYTES / ES;
    constexpr int AOFF = A_BYTES / ES;
    constexpr int NSTEP = BK / KSTEP;
    constexpr int CPC = (VPER + FN - 1) / FN;  // copies per column in a copying step
    const int wm = wave_m(), wn = wave_n();
    T* const nstage = lds + (cur ^ 1) * STAGE;
    const T* as = lds + cur * STAGE;
    const T* bs = lds + cur * STAGE + AOFF;
    FragA fa[2][FM];
    FragB fb[FN];
    load_frags(as, bs, wm, wn, 0, fa[0], fb);
    static_for<NSTEP>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      static_for<FN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[i][j] = mfma(fa[s & 1][i], fb[j], acc[i][j]);
        if constexpr (s + 1 < NSTEP) {
          fb[j] = frag<BMAJ, BN>(bs, wn * WN + j * MI, (s + 1) * KSTEP);
          if constexpr (j < FM) fa[(s + 1) & 1][j] = frag<AMAJ, BM>(as, wm * WM + j * MI, (s + 1) * KSTEP);
        }
        if constexpr (COPY && s < VSTEPS) {
          constexpr int c0 = s * VPER + j * CPC, c1 = s * VPER + (j + 1) * CPC;
          constexpr int e = (s + 1) * VPER < N_VMEM ? (s + 1) * VPER : N_VMEM;
          constexpr int a0 = c0 < e ? c0 : e, a1 = c1 < e ? c1 : e;
          if constexpr (a0 < a1) load_part<a0, a1, LEAN>(A, B, pm0, pn0, pk0, nstage);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }

  template <bool LEAN, bool COPY = true>
  static __device__ __forceinline__ void slice(const Operand<T>& A, const Operand<T>& B, T* lds, int cur, int pm0,
                                               int pn0, int pk0, Acc& acc) {
    if constexpr (MI == 16) {
      slice16<LEAN, COPY>(A, B, lds, cur, pm0, pn0, pk0, acc);
      return;
    }
    constexpr int STAGE = STAGE_BYTES / ES;
    constexpr int AOFF = A_BYTES / ES;
    constexpr int NSTEP = BK / KSTEP;
    const int wm = wave_m(), wn = wave_n();
    T* const nstage = lds + (cur ^ 1) * STAGE;
    const T* as = lds + cur * STAGE;
    const T* bs = lds + cur * STAGE + AOFF;
    FragA fa[2][FM];
    FragB fb[2][FN];
    load_frags(as, bs, wm, wn, 0, fa[0], fb[0]);
    u32x4_t rg[STAGING == STAGE_REG ? N_VMEM : 1];
    static_for<NSTEP>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (STAGING == STAGE_REG) {
        if constexpr (s == 0) {
          rload<AMAJ, BM, 0, INSTR_A, LEAN>(A, pm0, pk0, rg);
          rload<BMAJ, BN, 0, N_VMEM - INSTR_A, LEAN>(B, pn0, pk0, rg + INSTR_A);
        }
        if constexpr (s == NSTEP - 1) {
          rstore<BM, 0, INSTR_A>(nstage, rg);
          rstore<BN, 0, N_VMEM - INSTR_A>(nstage + AOFF, rg + INSTR_A);
        }
      } else if constexpr (COPY) {
        load_step<s, LEAN>(A, B, pm0, pn0, pk0, nstage);
      }
      if constexpr (s + 1 < NSTEP) load_frags(as, bs, wm, wn, (s + 1) * KSTEP, fa[(s + 1) & 1], fb[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
      constexpr int NR = s + 1 < NSTEP ? N_DS : 0;
      if constexpr (STAGING == STAGE_REG)
        schedule_step<NR, s == 0 ? N_VMEM : 0, s == NSTEP - 1 ? N_VMEM : 0>();
      else
        schedule_step<NR, COPY ? vmem_in_step(s) : 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // Persistent main loop over a sequence of output tiles with K = K each:
  // next(j, m0, n0) gives the origin of the j-th tile (false past the last one) and
  // epi(acc, m0, n0, spare) consumes a finished tile; init(acc, m0, n0) (zero by
  // default) sets acc up before a tile's first slice, after that slice's copies
  // are issued, so loads it issues are covered by the barrier's vmcnt wait.  The
  // slices of all tiles form one stream through two LDS stages, so the first
  // slice of tile j + 1 is copied while the last slice of tile j is multiplied
  // and its epilogue runs.  spare is the stage that last slice was
  // read from: an epilogue may use its STAGE_BYTES after a workgroup barrier
  // (other waves may still be reading their last fragments from it) and until
  // it returns (the next slice's copies into it start after the barrier that
  // opens that slice).  Every wave of the workgroup calls epi for the same tiles.
  // Ends with a barrier: the caller may reuse the LDS afterwards.
  // next(j, m0, n0), next(j, m0, n0, kb) or next(j, m0, n0, kb, nk): the second
  // form also gives the K offset at which the tile's K range of length K starts
  // (split-K tiles), the third the K offset and the number of K slices of the
  // item (at least one; segments of a tile's K range, kb + nk BK <= the K
  // given to run_tiles rounded up to BK).
  // (nk is written by the third form only)
  template <class Next>
  static __device__ __forceinline__ bool next_tile(Next& next, int j, int& m0, int& n0, int& kb, int& nk) {
    if constexpr (std::is_invocable_v<Next&, int, int&, int&, int&, int&>) {
      return next(j, m0, n0, kb, nk);
    } else if constexpr (std::is_invocable_v<Next&, int, int&, int&, int&>) {
      return next(j, m0, n0, kb);
    } else {
      kb = 0;
      return next(j, m0, n0);
    }
  }

  // init(acc, m0, n0) and epi(acc, m0, n0, spare) may also take the item's K
  // offset and number of K slices as two more arguments.
  template <class Init>
  static __device__ __forceinline__ void call_init(Init& init, Acc& acc, int m0, int n0, int kb, int nk) {
    if constexpr (std::is_invocable_v<Init&, Acc&, int, int, int, int>)
      init(acc, m0, n0, kb, nk);
    else
      init(acc, m0, n0);
  }
  template <class Epi>
  static __device__ __forceinline__ void call_epi(Epi& epi, Acc& acc, int m0, int n0, char* spare, int kb, int nk) {
    if constexpr (std::is_invocable_v<Epi&, Acc&, int, int, char*, int, int>)
      epi(acc, m0, n0, spare, kb, nk);
    else
      epi(acc, m0, n0, spare);
  }

  // k_whole (split-K sequences, next with a K offset only): the caller guarantees
  // that every item's K range ([kb, kb + K), or [kb, kb + nk BK)) lies inside
  // both operands' K extents with kb a multiple of BK (so no slice straddles an
  // operand's block split, itself a multiple of BK), which lets those sequences
  // take the lean copies too.
  template <class Next, class Epi, class Init>
  static __device__ __forceinline__ void run_tiles(const Operand<T>& A, const Operand<T>& B, int K, T* lds, Acc& acc,
                                                   Next&& next, Epi&& epi, Init&& init, bool k_whole = false) {
    // Lean copies (load_tile, rload) when every slice is a whole K slice -- tiles
    // start at K offset 0 (or k_whole) and K is a multiple of BK inside both K
    // ranges -- and each operand is either K-major with its K range inside its
    // rows, or (register staging only) MN-major with every tile inside its mn range.
    constexpr bool LEAN_OK = STAGING == STAGE_REG || (AMAJ == K_MAJOR && BMAJ == K_MAJOR);
    constexpr bool SPLIT_K = std::is_invocable_v<Next&, int, int&, int&, int&> ||
                             std::is_invocable_v<Next&, int, int&, int&, int&, int&>;
    auto fits = [&](const Operand<T>& op, bool kmajor, int MNT) {
      if (op.k_ext < K) return false;
      const int k1 = op.k_ext < op.ksplit ? op.k_ext : op.ksplit;  // K extent of the widest block
      return kmajor ? k1 <= op.ld : op.mn_ext % MNT == 0 && op.mn_ext <= op.ld;
    };
    if constexpr (LEAN_OK) {
      if ((!SPLIT_K || k_whole) && K % BK == 0 && fits(A, AMAJ == K_MAJOR, BM) && fits(B, BMAJ == K_MAJOR, BN)) {
        run_tiles_impl<true>(A, B, K, lds, acc, next, epi, init);
        return;
      }
    }
    run_tiles_impl<false>(A, B, K, lds, acc, next, epi, init);
  }

  template <bool LEAN, class Next, class Epi, class Init>
  static __device__ __forceinline__ void run_tiles_impl(const Operand<T>& A, const Operand<T>& B, int K, T* lds,
                                                        Acc& acc, Next&& next, Epi&& epi, Init&& init) {
    static_assert(NSTAGE == 2, "the persistent loop double-buffers K slices");
    constexpr int AOFF = A_BYTES / ES;
    // items with their own slice counts (next with five arguments); otherwise
    // every item has KT slices
    constexpr bool SEG = std::is_invocable_v<Next&, int, int&, int&, int&, int&>;
    const int KT = (K + BK - 1) / BK;
    int tm0, tn0, tkb, tkt = KT;
    if (!next_tile(next, 0, tm0, tn0, tkb, tkt)) return;
    // copy cursor: slice pk of tile pj (pkt slices), origin (pm0, pn0), K offset
    // pkb; past the last tile it points at K offset KT * BK, and its copies (into
    // a stage no slice reads) stay inside the operands or read zeros
    int pj = 0, pk = 0, pm0 = tm0, pn0 = tn0, pkb = tkb, pkt = tkt;
    bool pvalid = true;
    const bool cw = copy_wave();
    if (cw) {
      load_tile<AMAJ, BM>(A, pm0, pkb, lds);
      load_tile<BMAJ, BN>(B, pn0, pkb, lds + AOFF);
    }
    auto advance = [&]() {
      if (++pk == (SEG ? pkt : KT)) {
        pk = 0;
        ++pj;
        pvalid = pvalid && next_tile(next, pj, pm0, pn0, pkb, pkt);
      }
    };
    advance();
    if constexpr (SEG)
      call_init(init, acc, tm0, tn0, tkb, tkt);
    else
      init(acc, tm0, tn0);
    // tile clock (measurement builds): item jj, field f
    auto stamp = [&](int jj, int f, unsigned long long v) {
#if FLCE_TILE_CLOCK
      constexpr int KIND = STAGING == STAGE_REG ? (BMAJ == MN_MAJOR ? 0 : 1) : (SPLIT ? 2 : 3);
      if (threadIdx.x == 0 && blockIdx.x < 256 && jj < 64) tile_clock[KIND][blockIdx.x][jj][f] = v;
#endif
    };
    int q = 0;
    for (int j = 0;;) {
      const int nkt = SEG ? tkt : KT;
      if constexpr (FLCE_TILE_CLOCK != 0) {
        stamp(j, 0, __builtin_amdgcn_s_memtime());
        stamp(j, 4, (unsigned long long)nkt);
      }
      for (int kt = 0; kt < nkt; ++kt, ++q) {
        // After an epilogue only LDS work is drained: every wave waited for its
        // copies of this slice before the epilogue, so the global stores the
        // epilogue issued stay in flight.
        if (kt == 0 && j > 0)
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
          wait_and_barrier<0>();
        // past the last tile the copies go to a stage no slice reads: lean ones
        // re-read K offset 0 (inside the operands), the others K offset KT * BK,
        // where every chunk fails its bounds check and reads zeros
        const int pk0 = pvalid ? pkb + pk * BK : (LEAN ? 0 : KT * BK);
        if (!SPLIT || cw)
          slice<LEAN>(A, B, lds, q & 1, pm0, pn0, pk0, acc);
        else
          slice<LEAN, false>(A, B, lds, q & 1, pm0, pn0, pk0, acc);
        advance();
        if constexpr (FLCE_TILE_CLOCK != 0)
          if (kt == 0) stamp(j, 1, __builtin_amdgcn_s_memtime());
      }
      if constexpr (FLCE_TILE_CLOCK != 0) stamp(j, 2, __builtin_amdgcn_s_memtime());
      // this wave's copies of the next tile's first slice have landed (a wave
      // without copies leaves its stores in flight)
      if (cw) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (SEG)
        call_epi(epi, acc, tm0, tn0, (char*)lds + ((q - 1) & 1) * STAGE_BYTES, tkb, tkt);
      else
        epi(acc, tm0, tn0, (char*)lds + ((q - 1) & 1) * STAGE_BYTES);
      if constexpr (FLCE_TILE_CLOCK != 0) stamp(j, 3, __builtin_amdgcn_s_memtime());
      if (!next_tile(next, ++j, tm0, tn0, tkb, tkt)) break;
      if constexpr (SEG)
        call_init(init, acc, tm0, tn0, tkb, tkt);
      else
        init(acc, tm0, tn0);
    }
    wait_and_barrier<0>();
  }

  template <class Next, class Epi>
  static __device__ __forceinline__ void run_tiles(const Operand<T>& A, const Operand<T>& B, int K, T* lds, Acc& acc,
                                                   Next&& next, Epi&& epi) {
    run_tiles(A, B, K, lds, acc, next, epi, [](Acc& a, int, int) { zero(a); });
  }

  // acc = A[m0:m0+BM, 0:K] . B[n0:n0+BN, 0:K]^T for a single tile.
  static __device__ __forceinline__ void run(const Operand<T>& A, const Operand<T>& B, int m0, int n0, int K,
                                             T* lds, Acc& acc) {
    run_tiles(
        A, B, K, lds, acc,
        [&](int j, int& tm, int& tn) {
          tm = m0;
          tn = n0;
          return j == 0;
        },
        [](Acc&, int, int, char*) {});
  }
};

// Logical workgroup id whose consecutive values run on the same XCD: the
// hardware hands workgroup b to XCD b % 8, so XCD x receives b = x, x + 8, ...
__device__ __forceinline__ int xcd_grouped_id(int b, int G) {
  const int q = G >> 3, r = G & 7;
  const int x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

#ifndef FLCE_GROUP_M
#define FLCE_GROUP_M 4
#endif

// Tile (tm, tn) of a tiles_m x tiles_n grid for logical id t, walking groups of
// GM tile rows column by column: any GM * c consecutive ids form a GM x c block,
// so the 32 workgroups an XCD runs at once share GM row tiles and 32 / GM column
// tiles of the operands in its L2 (GM = 1: plain row-fastest order).
template <int GM = FLCE_GROUP_M>
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  if (GM <= 1) {
    tm = t % tiles_m;
    tn = t / tiles_m;
    return;
  }
  const int per_group = GM * tiles_n;
  const int g = t / per_group;
  const int first = g * GM;
  const int rows = min(GM, tiles_m - first);
  const int in = t - g * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

}  // namespace flce
