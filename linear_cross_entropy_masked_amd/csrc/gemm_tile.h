// Block-tiled bf16 GEMM on gfx950 MFMA, shared by the three products of the fused linear CE.
//
//   C[M, N] = Σ_k A(m, k) · B(k, n),   fp32 accumulation, result handed to an epilogue.
//
// Tile: 256 × 256 outputs per workgroup, K advanced 64 at a time; 4 wavefronts in a 2 × 2
// arrangement, each owning a 128 × 128 block of accumulators (8 × 8 fragments of
// v_mfma_f32_16x16x32_bf16, 256 fp32 registers per lane). Both operands are staged in LDS in
// the layout the MFMA wants — 64 contiguous k per row — so every fragment is one 16-byte LDS
// read. 16-byte chunks within a row are XOR-swizzled by a function of the row so that the
// 16 rows a fragment read touches, and the rows a transposing store touches, fall in
// different banks.
//
// Operands come in two layouts:
//   K-major  (row m holds contiguous k): copied straight into LDS;
//   MN-major (row k holds contiguous m): each lane loads a 4 (k) × 8 (m) block with four
//            16-byte loads and writes eight 4-element k-runs, transposing in registers.
// The next K-tile is loaded into registers while the MFMAs work on the current one, and
// LDS is double-buffered, so one barrier per K-tile suffices.
#pragma once

#include <type_traits>

#include "common.h"

namespace lce {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * BK * 2;  // one operand tile in LDS (32 KiB)

// Row-major bf16 matrix whose contiguous dimension is split into 64-wide groups placed `gs`
// elements apart (gs == 64: an ordinary dense matrix).
struct View {
  const uint16_t* p;
  int64_t ld;    // elements between consecutive rows
  int64_t gs;    // elements between consecutive 64-column groups
  int64_t rows;  // valid rows
  int64_t cols;  // valid columns
  // Two-segment operand (pipelined GEMM launched with SEGA): k rows kseg .. of an MN-major
  // operand sit at p2 + (row − kseg) · ld instead of p + row · ld; k columns kseg .. of a
  // K-major panel operand (below) at p2 with column col − kseg. kseg is a multiple of the K
  // slice (and of 64 for panels).
  const uint16_t* p2 = nullptr;
  int64_t kseg = 0;
  // Panels (ext > 0): the 64-column groups lie gs apart as whole [rows][64] blocks (gs >=
  // rows · ld), and ext / ext2 are the elements stored from p / p2 on. The DMA window then
  // runs to the end of that storage instead of masking rows or k past the valid range: the
  // caller zero-fills what a product may read there (padding rows and columns of the last
  // panel); rows past the last panel of a K-major operand only reach output rows past M.
  int64_t ext = 0;
  int64_t ext2 = 0;
};

// Buffer resource over [base, base + bytes): loads at offsets past the end return zero, which
// masks rows beyond the valid range without branches and can never fault.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : uint32_t(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(n), 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 0);
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
// Byte offset of 16-byte chunk c (k = 8c .. 8c+7) of row `row` in a [256][64] bf16 tile.
__device__ __forceinline__ int lds_off(int row, int c) { return row * 128 + ((c ^ swz(row)) << 4); }

// Per-lane byte offset of this lane's first 16-byte load within an operand tile.
template <bool KMAJOR>
__device__ __forceinline__ uint32_t lane_offset(const View& X) {
  const int t = threadIdx.x;
  if constexpr (KMAJOR) {
    return uint32_t((int64_t(t >> 3) * X.ld + (t & 7) * 8) * 2);
  } else {
    const int m = 8 * (t & 31);
    return uint32_t((int64_t(t >> 5) * 4 * X.ld + (m >> 6) * X.gs + (m & 63)) * 2);
  }
}

// Global -> registers for one operand tile: rows r0 .. r0+255 (m or n), k0 .. k0+63 of a
// contraction of length K. Rows past the valid range and k >= K read as zero.
template <bool KMAJOR>
__device__ __forceinline__ void load_tile(const View& X, int64_t r0, int64_t k0, int64_t K,
                                          uint32_t voff, uint4 (&reg)[8]) {
  const int t = threadIdx.x;
  if constexpr (KMAJOR) {
    const int64_t g = (k0 >> 6) * X.gs;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(X.p + r0 * X.ld + g, ((X.rows - r0) * X.ld - g) * 2);
    const bool kin = k0 + (t & 7) * 8 < K;
    const uint32_t step = uint32_t(32 * X.ld * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 v = buf_load16(rs, voff, uint32_t(j) * step);
      reg[j] = kin ? v : uint4{0u, 0u, 0u, 0u};
    }
  } else {
    const int64_t kr = (X.rows < K ? X.rows : K) - k0;  // valid k rows from k0
    const int64_t shift = (r0 >> 6) * X.gs;              // window ends with the matrix too
    const int64_t avail = (X.rows - k0) * X.ld - shift;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(X.p + k0 * X.ld + shift, (kr * X.ld < avail ? kr * X.ld : avail) * 2);
    const uint32_t row = uint32_t(X.ld * 2);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) reg[4 * b + q] = buf_load16(rs, voff, uint32_t(32 * b + q) * row);
  }
}

// Registers -> LDS in the MFMA layout.
template <bool KMAJOR>
__device__ __forceinline__ void store_tile(char* lds, const uint4 (&reg)[8]) {
  const int t = threadIdx.x;
  if constexpr (KMAJOR) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(lds + lds_off((t >> 3) + 32 * j, t & 7)) = reg[j];
  } else {
    const int mc = t & 31;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int kq = (t >> 5) + 8 * b;  // k = 4 kq .. 4 kq + 3
      const uint32_t w[4][4] = {
          {reg[4 * b + 0].x, reg[4 * b + 0].y, reg[4 * b + 0].z, reg[4 * b + 0].w},
          {reg[4 * b + 1].x, reg[4 * b + 1].y, reg[4 * b + 1].z, reg[4 * b + 1].w},
          {reg[4 * b + 2].x, reg[4 * b + 2].y, reg[4 * b + 2].z, reg[4 * b + 2].w},
          {reg[4 * b + 3].x, reg[4 * b + 3].y, reg[4 * b + 3].z, reg[4 * b + 3].w}};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int wd = j >> 1;
        uint32_t lo, hi;
        if (j & 1) {
          lo = (w[0][wd] >> 16) | (w[1][wd] & 0xffff0000u);
          hi = (w[2][wd] >> 16) | (w[3][wd] & 0xffff0000u);
        } else {
          lo = (w[0][wd] & 0xffffu) | (w[1][wd] << 16);
          hi = (w[2][wd] & 0xffffu) | (w[3][wd] << 16);
        }
        const int m = 8 * mc + j;
        *reinterpret_cast<uint2*>(lds + lds_off(m, kq >> 1) + (kq & 1) * 8) = uint2{lo, hi};
      }
    }
  }
}

// Map a linear workgroup id to a tile id so that the tiles one XCD runs (ids congruent mod 8
// are dispatched to the same XCD) are consecutive in tile order and share operands in its L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t w, int64_t total) {
  const int64_t per = total / 8;
  if (w >= per * 8) return w;
  return (w % 8) * per + w / 8;
}

// Tile order: `inner` tiles along the fast dimension share the slow-dimension operand.
struct TileMap {
  int64_t m_tiles, n_tiles, splits;
  bool m_fast;  // true: consecutive tiles walk m (sharing the B tile), else walk n
  int xn = 0;   // > 0 (pipelined kernel, one split): the 8 XCDs own a (8 / xn) × xn grid of
                // m × n tile blocks, so each XCD's L2 sees 1 / xn of the B operand
};

template <bool AK, bool BKM, class Epi>
__global__ void __launch_bounds__(kThreads, 1)
    gemm256_kernel(View A, View B, int64_t M, int64_t N, int64_t K, int64_t ksplit, TileMap tm,
                   Epi epi) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][kTileBytes];

  const int64_t total = tm.m_tiles * tm.n_tiles * tm.splits;
  const int64_t tile = xcd_tile(blockIdx.x, total);
  const int64_t mn = tm.m_tiles * tm.n_tiles;
  const int64_t kz = tile / mn;
  const int64_t rest = tile % mn;
  const int64_t mt = tm.m_fast ? rest % tm.m_tiles : rest / tm.n_tiles;
  const int64_t nt = tm.m_fast ? rest / tm.m_tiles : rest % tm.n_tiles;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t kbeg = kz * ksplit;
  const int64_t kend = kbeg + ksplit < K ? kbeg + ksplit : K;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[8], rb[8];
  const uint32_t va = lane_offset<AK>(A), vb = lane_offset<BKM>(B);
  int buf = 0;
  if (kbeg < kend) {
    load_tile<AK>(A, m0, kbeg, K, va, ra);
    load_tile<BKM>(B, n0, kbeg, K, vb, rb);
    store_tile<AK>(lds[0][0], ra);
    store_tile<BKM>(lds[0][1], rb);
  }
  __syncthreads();

  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) {
      load_tile<AK>(A, m0, k0 + BK, K, va, ra);
      load_tile<BKM>(B, n0, k0 + BK, K, vb, rb);
    }
    const char* la = lds[buf][0];
    const char* lb = lds[buf][1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8_t bfr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(lb + lds_off(wn * 128 + j * 16 + (lane & 15), c));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_t af =
            *reinterpret_cast<const bf16x8_t*>(la + lds_off(wm * 128 + i * 16 + (lane & 15), c));
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) {
      store_tile<AK>(lds[buf ^ 1][0], ra);
      store_tile<BKM>(lds[buf ^ 1][1], rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  epi.begin(kz);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t gm = m0 + wm * 128 + i * 16 + 4 * (lane >> 4) + q;
        const int64_t gn = n0 + wn * 128 + j * 16 + (lane & 15);
        if (gm < M && gn < N) epi(gm, gn, acc[i][j][q]);
      }
}

template <bool AK, bool BKM, class Epi>
hipError_t launch(const View& A, const View& B, int64_t M, int64_t N, int64_t K, int64_t splits,
                  bool m_fast, const Epi& epi, hipStream_t s) {
  TileMap tm{(M + BM - 1) / BM, (N + BN - 1) / BN, splits < 1 ? 1 : splits, m_fast};
  int64_t ksplit = (K + tm.splits - 1) / tm.splits;
  ksplit = (ksplit + BK - 1) / BK * BK;
  const int64_t total = tm.m_tiles * tm.n_tiles * tm.splits;
  hipLaunchKernelGGL((gemm256_kernel<AK, BKM, Epi>), dim3(unsigned(total)), dim3(kThreads), 0, s,
                     A, B, M, N, K, ksplit, tm, epi);
  return hipGetLastError();
}


// ============================================================================ pipelined variant
//
// Operands go global -> LDS directly (buffer_load ... lds, 16 bytes per lane, no registers
// involved) into a ring of STAGES K-slices of depth BK, STAGES - 1 slices ahead of the MFMAs.
// LDS layouts of one slice:
//   K-major operand : [R rows][BK k]   (2·BK-byte rows, 16-byte chunks XOR-swizzled by row)
//   MN-major operand: [BK k][R rows]   (2·R-byte rows, 32-byte pairs XOR-swizzled by k),
//                     read back with ds_read_b64_tr_b16, which hands each lane 4
//                     consecutive k of one row — the MFMA operand order.
// The MFMA is issued with B as its first operand, so each lane ends up owning 4 consecutive
// output columns of one row (16-byte epilogue accesses).
// Requirement: for a K-major operand, K must be a multiple of BK or the columns past K must
// read as zero (true for the probability slice, whose padding is zero-filled).
namespace v2 {

// Tile shape and pipeline of one instantiation.
//   BM × BN outputs per workgroup, WM × WN wavefronts (each owns (BM/WM) × (BN/WN)),
//   K slices of BK (64 makes every DMA row segment of a K-major operand a full 128-byte line;
//   32 leaves 64-byte segments, which measured at half the L2->LDS throughput), STAGES slices
//   in the LDS ring, OCC workgroups meant to share one CU (register and LDS budgets).
template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_, int OCC_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_;
  static constexpr int OCC = OCC_, NW = WM * WN, THREADS = 64 * NW;
  static constexpr int ABytes = BM * BK * 2, BBytes = BN * BK * 2;
  static constexpr int StageBytes = ABytes + BBytes, LdsBytes = STAGES * StageBytes;
  static constexpr int PA = ABytes / 1024 / NW, PB = BBytes / 1024 / NW;  // DMA per wave
  static constexpr int PER = PA + PB;
  static constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(PA * NW * 1024 == ABytes && PB * NW * 1024 == BBytes, "DMA split");
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert(BM == 128 || BM == 256, "MN-major rows are 256 or 512 bytes");
  static_assert(BN == 128 || BN == 256, "MN-major rows are 256 or 512 bytes");
  static_assert(LdsBytes * OCC <= 160 * 1024, "LDS");
  static_assert(PER * (STAGES - 1) <= 63, "vmcnt");
};

// Large-K products: one 256 × 256 workgroup per CU, 8 wavefronts, K = 64 slices, 2 stages.
// Measured on the logits product's access pattern, direct-to-LDS streaming reaches about
// 12 TB/s with one 64-deep slice in flight per CU and about 16 TB/s with two, while 32-deep
// slices (64-byte row segments) stay near 12 TB/s at any depth. Two slices in flight do not
// fit next to the one being multiplied; the variants that approximate it (a 5-slot ring of
// single operands; refilling a slot mid-slice after a second barrier) measured slower.
using CfgWide = Cfg<256, 256, 64, 2, 2, 4, 1>;
// Products whose epilogue streams HBM (fp32 read-modify-write): two 256 × 128 workgroups per
// CU, so one's epilogue overlaps the other's MFMAs; K = 32 slices, 3 stages.
using CfgPair = Cfg<256, 128, 32, 3, 2, 2, 2>;

typedef short v4s __attribute__((ext_vector_type(4)));

// Chunk swizzle of K-major rows. Measured on gfx950 for 16-row fragment reads (lanes 0-15 =
// 16 consecutive rows, one 16-byte chunk each): with 64-byte rows XOR with (row >> 1) & 3 is
// conflict-free (row & 3 or no swizzle cost about 2x in LDS cycles); with 128-byte rows
// XOR with row & 7 is. Neither depends on the fragment's 16-row block.
template <int BK>
__device__ __forceinline__ int swz_k(int r) {
  return BK == 64 ? (r & 7) : ((r >> 1) & 3);
}
// 32-byte-pair swizzle of MN-major k rows: the 8 k rows one half-wavefront of a transposing
// read touches ({0..3, 8..11} + 16j) land on 8 different 32-byte bank groups.
__device__ __forceinline__ int swz_mn(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }

// Per-lane byte offsets (within one slice's global window) of the lane's P DMA loads for an
// operand with R rows (K-major) or R columns (MN-major). One slice of the operand is
// R·BK·2 / 1024 instructions of 1 KiB; wavefront w issues instructions w·P .. w·P + P − 1.
template <bool KMAJOR, int R, int BK, int P>
__device__ __forceinline__ void dma_offsets(const View& X, uint32_t (&off)[P]) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int g = w * P + j;  // instruction index within the slice
    if constexpr (KMAJOR) {
      constexpr int kc = BK / 8;                // 16-byte chunks per row
      const int r = (64 / kc) * g + l / kc;     // 64 / kc rows per instruction
      const int c = (l % kc) ^ swz_k<BK>(r);
      off[j] = uint32_t((int64_t(r) * X.ld + 8 * c) * 2);
    } else {
      constexpr int rc = R / 8;                 // 16-byte chunks per k row
      const int k = (64 / rc) * g + l / rc;     // 64 / rc k rows per instruction
      const int c = (l % rc) ^ swz_mn(k);
      const int m = 8 * c;
      off[j] = uint32_t((int64_t(k) * X.ld + (m >> 6) * X.gs + (m & 63)) * 2);
    }
  }
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global straight into LDS at byte address m0 + 16 * lane. Issued as
// inline asm on purpose: the compiler then leaves these loads to the explicit vmcnt waits
// below instead of draining every in-flight slice before each LDS read. `rs` (buffer
// resource) and `m0` are wave-uniform and live in SGPRs.
__device__ __forceinline__ void dma16(i32x4_t rs, uint32_t voff, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(rs)
      : "memory");
}

// Wave-uniform DMA window of one operand: byte address of the current K slice, bytes
// readable from there (loads past them return zero; <= 0 reads nothing) and the advance per
// slice. Built once per tile, so a slice costs a 64-bit add instead of address arithmetic.
struct Stream {
  uint64_t base;
  int64_t recs;
  int64_t step;   // advance after the next slice
  int64_t step2;  // advance after the one after (differs from step only for 32-deep slices
                  // of a grouped K-major operand: 32 elements, then the gap to the next group)
  // two-segment operands only: slices left before the window moves to (base2, recs2); 0 never
  int64_t left;
  uint64_t base2;
  int64_t recs2;
};

// Window of the K slice starting at k0 (a multiple of BK) for rows / columns r0 .. r0 + R − 1.
// SEG: the operand's k rows (MN-major) or k columns (K-major panels) come in the two segments
// View::p / View::p2.
template <bool KMAJOR, int BK, bool SEG = false>
__device__ __forceinline__ Stream stream_at(const View& X, int64_t r0, int64_t k0, int64_t K) {
  Stream st;
  st.left = 0;
  st.base2 = 0;
  st.recs2 = 0;
  if constexpr (KMAJOR) {
    if (X.ext > 0) {  // panels: the window runs to the end of the segment's storage
      auto at = [&](int64_t kk) { return (kk >> 6) * X.gs + (kk & 63) + r0 * X.ld; };
      if (SEG && k0 >= X.kseg) {
        st.base = reinterpret_cast<uint64_t>(X.p2 + at(k0 - X.kseg));
        st.recs = (X.ext2 - at(k0 - X.kseg)) * 2;
      } else {
        st.base = reinterpret_cast<uint64_t>(X.p + at(k0));
        st.recs = (X.ext - at(k0)) * 2;
        if (SEG) {
          st.left = (X.kseg - k0) / BK;
          st.base2 = reinterpret_cast<uint64_t>(X.p2 + at(0));
          st.recs2 = (X.ext2 - at(0)) * 2;
        }
      }
    } else {
      const int64_t g = (k0 >> 6) * X.gs + (k0 & 63);
      st.base = reinterpret_cast<uint64_t>(X.p + r0 * X.ld + g);
      st.recs = ((X.rows - r0) * X.ld - g) * 2;
    }
    if (BK == 64) {
      st.step = st.step2 = X.gs * 2;
    } else {  // 32 within a group, then on to the next group's start
      const int64_t in = 64, across = (X.gs - 32) * 2;
      st.step = (k0 & 32) ? across : in;
      st.step2 = (k0 & 32) ? in : across;
    }
  } else {
    // k rows past min(rows, K) read as zero; the window also stops at the end of the matrix
    // (the shifted base would otherwise let the last row's columns past `cols` run over it)
    const int64_t kall = X.rows < K ? X.rows : K;
    const int64_t shift = (r0 >> 6) * X.gs;
    if (X.ext > 0) {  // panels (one segment): the window runs to the end of the storage
      st.base = reinterpret_cast<uint64_t>(X.p + k0 * X.ld + shift);
      st.recs = (X.ext - (k0 * X.ld + shift)) * 2;
    } else if (SEG && k0 >= X.kseg) {  // starts in the second segment
      const int64_t kr = kall - k0;
      const int64_t avail = (X.rows - k0) * X.ld - shift;
      st.base = reinterpret_cast<uint64_t>(X.p2 + (k0 - X.kseg) * X.ld + shift);
      st.recs = (kr * X.ld < avail ? kr * X.ld : avail) * 2;
    } else {
      const int64_t e1 = SEG ? X.kseg : X.rows;  // k rows of the first segment
      const int64_t kr = (kall < e1 ? kall : e1) - k0;
      const int64_t avail = (e1 - k0) * X.ld - shift;
      st.base = reinterpret_cast<uint64_t>(X.p + k0 * X.ld + shift);
      st.recs = (kr * X.ld < avail ? kr * X.ld : avail) * 2;
      if (SEG) {
        const int64_t kr2 = kall - X.kseg;
        const int64_t avail2 = (X.rows - X.kseg) * X.ld - shift;
        st.left = (X.kseg - k0) / BK;
        st.base2 = reinterpret_cast<uint64_t>(X.p2 + shift);
        st.recs2 = kr2 <= 0 ? 0 : (kr2 * X.ld < avail2 ? kr2 * X.ld : avail2) * 2;
      }
    }
    st.step = st.step2 = int64_t(BK) * X.ld * 2;
  }
  // every input is wave-uniform; saying so keeps the window in SGPRs for the whole K loop.
  // readfirstlane returns a signed int: each half goes through uint32_t before widening, or
  // a low word with bit 31 set would be sign-extended into the high word.
  auto u64 = [](uint64_t x) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(x)));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(x >> 32)));
    return uint64_t(lo) | (uint64_t(hi) << 32);
  };
  st.base = u64(st.base);
  st.recs = int64_t(u64(uint64_t(st.recs)));
  st.step = int64_t(u64(uint64_t(st.step)));
  st.step2 = int64_t(u64(uint64_t(st.step2)));
  if (SEG) {
    st.left = int64_t(u64(uint64_t(st.left)));
    st.base2 = u64(st.base2);
    st.recs2 = int64_t(u64(uint64_t(st.recs2)));
  }
  return st;
}

// Issue one operand's P loads of the current slice (LDS bytes m0 .. m0 + P KiB), then advance
// (SEG: to the second segment after the first one's last slice).
template <int P, bool SEG = false>
__device__ __forceinline__ void dma_issue(Stream& st, const uint32_t (&off)[P], uint32_t m0) {
  const int64_t r = st.recs;
  const uint32_t n = r <= 0 ? 0u : (r >= 0xffffffffLL ? 0xffffffffu : uint32_t(r));
  const i32x4_t rs = {int(uint32_t(st.base)), int(uint32_t(st.base >> 32) & 0xffffu), int(n),
                      0x00020000};
#pragma unroll
  for (int j = 0; j < P; ++j) dma16(rs, off[j], m0 + uint32_t(j) * 1024u);
  st.base += uint64_t(st.step);
  st.recs -= st.step;
  const int64_t t = st.step;
  st.step = st.step2;
  st.step2 = t;
  if (SEG && --st.left == 0) {
    st.base = st.base2;
    st.recs = st.recs2;
  }
}

// One 16 × 32 MFMA operand fragment for rows rbase .. rbase+15 and k = 32 kk .. 32 kk + 31 of
// the slice tile (R rows / columns, depth BK).
template <bool KMAJOR, int R, int BK>
__device__ __forceinline__ bf16x8_t frag(const char* lds, int rbase, int kk) {
  const int l = threadIdx.x & 63;
  if constexpr (KMAJOR) {
    const int r = rbase + (l & 15);
    const int c = (4 * kk + (l >> 4)) ^ swz_k<BK>(r);
    return *reinterpret_cast<const bf16x8_t*>(lds + r * (2 * BK) + c * 16);
  } else {
    const int g = l >> 4, L = l & 15;
    const int m = rbase + 4 * (L & 3);
    const int k0 = 32 * kk + 8 * g + (L >> 2), k1 = k0 + 4;
    const int c = m >> 3, h = ((m >> 2) & 1) * 8;
    const char* p0 = lds + k0 * (2 * R) + ((c ^ swz_mn(k0)) << 4) + h;
    const char* p1 = lds + k1 * (2 * R) + ((c ^ swz_mn(k1)) << 4) + h;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p1);
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

// s_waitcnt vmcnt(PER · s) for the runtime s in [0, S], other counters untouched.
template <int PER, int S>
__device__ __forceinline__ void wait_slices(int s) {
  if constexpr (S < 0) {
    (void)s;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // never reached: s is always in range
  } else {
    if (s == S) {
      constexpr int n = PER * S;
      __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    } else {
      wait_slices<PER, S - 1>(s);
    }
  }
}

// Epilogues that set kRowTag get each row's row_tag (e.g. its label) loaded once per tile,
// ahead of the epilogue's other loads, and receive it in load4t(m, n, tag) in place of
// load4(m, n): loads that depend on the tag then issue together instead of each waiting for
// its own tag load.
template <class E, class = void>
struct RowTagged {
  static constexpr bool value = false;
};
template <class E>
struct RowTagged<E, std::void_t<decltype(E::kRowTag)>> {
  static constexpr bool value = E::kRowTag;
};

// Tile coordinates (m-tile, n-tile, K split) of workgroup w; false for a workgroup with no
// tile (the XCD-block mapping pads every XCD to the largest block).
struct TileCoord {
  int64_t mt, nt, kz;
};
__device__ __forceinline__ bool tile_coord(const TileMap& tm, int64_t w, TileCoord& t) {
  if (tm.xn > 0) {
    // workgroups are dispatched to XCDs round-robin: XCD x runs w = x, x + 8, x + 16, ...
    const int64_t x = w & 7, li = w >> 3, gm = 8 / tm.xn;
    const int64_t xm = x / tm.xn, xq = x % tm.xn;
    const int64_t m_lo = xm * tm.m_tiles / gm, m_hi = (xm + 1) * tm.m_tiles / gm;
    const int64_t n_lo = xq * tm.n_tiles / tm.xn, n_hi = (xq + 1) * tm.n_tiles / tm.xn;
    const int64_t nn = n_hi - n_lo;
    if (nn <= 0 || li >= (m_hi - m_lo) * nn) return false;
    t = TileCoord{m_lo + li / nn, n_lo + li % nn, 0};
    return true;
  }
  const int64_t mn = tm.m_tiles * tm.n_tiles;
  const int64_t tile = xcd_tile(w, mn * tm.splits);
  const int64_t rest = tile % mn;
  t = TileCoord{tm.m_fast ? rest % tm.m_tiles : rest / tm.n_tiles,
                tm.m_fast ? rest / tm.m_tiles : rest % tm.n_tiles, tile / mn};
  return true;
}

// One BM × BN output tile at tile coordinates `tc`.
template <class C, bool AK, bool BKM, class Epi, bool SEGA = false>
__device__ __forceinline__ void run_tile(const View& A, const View& B, int64_t M, int64_t N,
                                         int64_t K, int64_t ksplit, const TileCoord& tc,
                                         Epi& epi, char* lds) {
  constexpr int TM = C::TM, TN = C::TN, BK = C::BK, STAGES = C::STAGES;
  const int64_t kz = tc.kz;
  const int64_t m0 = tc.mt * C::BM, n0 = tc.nt * C::BN;
  const int64_t kbeg = kz * ksplit;
  const int64_t kend = kbeg + ksplit < K ? kbeg + ksplit : K;
  const int nk = kend > kbeg ? int((kend - kbeg + BK - 1) / BK) : 0;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  uint32_t offa[C::PA], offb[C::PB];
  dma_offsets<AK, C::BM, BK, C::PA>(A, offa);
  dma_offsets<BKM, C::BN, BK, C::PB>(B, offb);
  Stream sa = stream_at<AK, BK, SEGA>(A, m0, kbeg, K);
  Stream sb = stream_at<BKM, BK>(B, n0, kbeg, K);
  // LDS byte addresses of this wavefront's DMA destinations in slot 0
  const uint32_t wv = __builtin_amdgcn_readfirstlane(uint32_t(threadIdx.x >> 6));
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
  const uint32_t ma0 = lds0 + wv * uint32_t(C::PA * 1024);
  const uint32_t mb0 = lds0 + uint32_t(C::ABytes) + wv * uint32_t(C::PB * 1024);

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // MFMAs over one slice whose A and B tiles sit at sA and sB
  auto compute = [&](const char* sA, const char* sB) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8_t bf[TN], af[TM];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = frag<BKM, C::BN, BK>(sB, wn * (C::BN / C::WN) + 16 * j, kk);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = frag<AK, C::BM, BK>(sA, wm * (C::BM / C::WM) + 16 * i, kk);
      // all fragment reads are in flight before the first MFMA; the MFMAs then wait on them
      // one by one instead of the scheduler trading registers for exposed LDS latency
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  int issued = 0;  // slices whose DMA has been issued (the same count in every wavefront)
  int wslot = 0;   // ring slot the next issue fills
  auto issue = [&]() {
    const uint32_t o = uint32_t(wslot * C::StageBytes);
    dma_issue<C::PA, SEGA>(sa, offa, ma0 + o);
    dma_issue<C::PB>(sb, offb, mb0 + o);
    wslot = wslot + 1 == STAGES ? 0 : wslot + 1;
    ++issued;
  };

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue();
  int rslot = 0;  // ring slot of slice kt
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt has landed once at most the later slices' DMA is pending; then sync the
    // block with a bare barrier (a __syncthreads() fence would drain the later slices too)
    wait_slices<C::PER, STAGES - 2>(issued - 1 - kt);
    __builtin_amdgcn_s_barrier();
    // refill the slot of slice kt-1 first (every wavefront's reads of it were consumed by
    // its MFMAs before it reached this barrier), so that nothing separates the fragment
    // reads below from the MFMAs that wait on them one by one
    if (kt + STAGES - 1 < nk) issue();
    const char* st = lds + rslot * C::StageBytes;
    rslot = rslot + 1 == STAGES ? 0 : rslot + 1;
    compute(st, st + C::ABytes);
  }

  // Epilogue in batches of two 16-row blocks: every load a batch needs (old accumulator
  // values, bias, label rows) is issued before any of its stores, so the loads overlap
  // instead of each waiting behind a store the compiler cannot prove disjoint.
  // Epilogues with kRowStats also get, per output row, the (max, sum of exp(x - max)) of the
  // values they store over this tile's valid columns (value4 says what those values are).
  epi.begin(kz);
  // Epilogues with kTileMax store values relative to their row's maximum over this tile's
  // valid columns: that maximum is reduced first (over the four lanes sharing a row, then
  // over the WN wavefronts through LDS) and handed to every store of the row.
  // They also get a per-row tag (row_tag, e.g. the row's label), loaded here ahead of the
  // stores that use it.
  constexpr bool kTagged = RowTagged<Epi>::value;
  float tmax[TM];
  int rtag[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    tmax[i] = -INFINITY;
    rtag[i] = -1;
  }
  if constexpr (Epi::kTileMax || kTagged) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t gm = m0 + wm * (C::BM / C::WM) + 16 * i + (lane & 15);
      if (gm < M) rtag[i] = epi.row_tag(gm);
    }
  }
  // Each row's maximum over this wavefront's valid columns (the four lanes sharing the row
  // reduced with shuffles): the shift of the row statistics and the start of the tile maximum.
  float wmax[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) wmax[i] = -INFINITY;
  if constexpr (Epi::kTileMax || Epi::kRowStats) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t gm = m0 + wm * (C::BM / C::WM) + 16 * i + (lane & 15);
      float mx = -INFINITY;
      if (gm < M) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t gn = n0 + wn * (C::BN / C::WN) + 16 * j + 4 * (lane >> 4);
          if (gn + 4 <= N) {
            const f32x4_t z = epi.value4(acc[i][j], epi.load4(gm, gn));
            mx = fmaxf(mx, fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (gn + q < N) mx = fmaxf(mx, epi.value1(gn + q, acc[i][j][q]));
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      wmax[i] = fmaxf(mx, __shfl_xor(mx, 32, 64));
    }
  }
  if constexpr (Epi::kTileMax) {
    __syncthreads();  // every wavefront is past the main loop: the LDS ring is free
    float* red = reinterpret_cast<float*>(lds);  // [WN][BM]
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) red[wn * C::BM + wm * (C::BM / C::WM) + 16 * i + lane] = wmax[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * (C::BM / C::WM) + 16 * i + (lane & 15);
      float m = red[r];
#pragma unroll
      for (int w = 1; w < C::WN; ++w) m = fmaxf(m, red[w * C::BM + r]);
      tmax[i] = m;
    }
    // the row-stats reduction below writes the same LDS only after its own barrier, which
    // every wavefront reaches after these reads
  }
  float rm[TM], rs[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    rm[i] = -INFINITY;
    rs[i] = 0.f;
  }
  f32x4_t cs[TN];  // kColSums: this lane's column sums (4 columns per fragment column)
#pragma unroll
  for (int j = 0; j < TN; ++j) cs[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i0 = 0; i0 < TM; i0 += 2) {
    typename Epi::Aux aux[2][TN];
#pragma unroll
    for (int di = 0; di < 2; ++di) {
      const int64_t gm = m0 + wm * (C::BM / C::WM) + 16 * (i0 + di) + (lane & 15);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t gn = n0 + wn * (C::BN / C::WN) + 16 * j + 4 * (lane >> 4);
        if (gm < M && gn + 4 <= N) {
          if constexpr (kTagged)
            aux[di][j] = epi.load4t(gm, gn, rtag[i0 + di]);
          else
            aux[di][j] = epi.load4(gm, gn);
        }
      }
    }
#pragma unroll
    for (int di = 0; di < 2; ++di) {
      const int64_t gm = m0 + wm * (C::BM / C::WM) + 16 * (i0 + di) + (lane & 15);
      if (gm >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t gn = n0 + wn * (C::BN / C::WN) + 16 * j + 4 * (lane >> 4);
        if (gn + 4 <= N) {
          if constexpr (Epi::kTileMax)
            epi.store4m(gm, gn, acc[i0 + di][j], aux[di][j], tmax[i0 + di], rtag[i0 + di]);
          else
            epi.store4(gm, gn, acc[i0 + di][j], aux[di][j]);
          if constexpr (Epi::kColSums) cs[j] += epi.colvalue4(acc[i0 + di][j], aux[di][j]);
          if constexpr (Epi::kRowStats) {
            // shift as (z − max) · log2 e: the wavefront's row maximum contributes exactly 1
            const f32x4_t z = epi.value4(acc[i0 + di][j], aux[di][j]);
            const float mw = wmax[i0 + di];
            float t = rs[i0 + di];
#pragma unroll
            for (int q = 0; q < 4; ++q) t += fast_exp2((z[q] - mw) * kLog2e);
            rs[i0 + di] = t;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (gn + q < N) {
              if constexpr (Epi::kTileMax)
                epi.put1m(gm, gn + q, acc[i0 + di][j][q], tmax[i0 + di], rtag[i0 + di]);
              else
                epi(gm, gn + q, acc[i0 + di][j][q]);
              if constexpr (Epi::kRowStats)
                rs[i0 + di] +=
                    fast_exp2((epi.value1(gn + q, acc[i0 + di][j][q]) - wmax[i0 + di]) * kLog2e);
            }
        }
      }
    }
  }
  if constexpr (Epi::kColSums) {
    // (launched with N % 4 == 0: every column went through colvalue4.) Lanes 16 g .. 16 g + 15
    // hold the same columns: reduce over them, then over the WM wavefronts sharing the
    // columns through LDS, in wavefront order.
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int off = 1; off <= 8; off <<= 1) cs[j][q] += __shfl_xor(cs[j][q], off, 64);
    __syncthreads();  // every wavefront is past the main loop: the LDS ring is free
    float* cred = reinterpret_cast<float*>(lds + 16384);  // [WM][BN]
    if ((lane & 15) == 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          cred[wm * C::BN + wn * (C::BN / C::WN) + 16 * j + 4 * (lane >> 4) + q] = cs[j][q];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C::BN; c += C::THREADS) {
      float sum = cred[c];
#pragma unroll
      for (int w = 1; w < C::WM; ++w) sum += cred[w * C::BN + c];
      if (n0 + c < N) epi.col_sums(tc.mt, n0 + c, sum);
    }
  }
  if constexpr (Epi::kRowStats) {
    // lanes l, l ^ 16, l ^ 32 and l ^ 48 hold the same rows under the same shift: add their
    // sums, then merge the WN wavefronts that share each row through LDS, in wavefront order
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      rs[i] += __shfl_xor(rs[i], 16, 64);
      rs[i] += __shfl_xor(rs[i], 32, 64);
      rm[i] = wmax[i];
    }
    __syncthreads();  // every wavefront is past the main loop: the LDS ring is free
    float2* red = reinterpret_cast<float2*>(lds);  // [WN][BM]
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        red[wn * C::BM + wm * (C::BM / C::WM) + 16 * i + lane] = float2{rm[i], rs[i]};
    }
    __syncthreads();
    for (int r = threadIdx.x; r < C::BM; r += C::THREADS) {
      float m = red[r].x, sum = red[r].y;
#pragma unroll
      for (int w = 1; w < C::WN; ++w) lse_merge(m, sum, red[w * C::BM + r].x, red[w * C::BM + r].y);
      if (m0 + r < M) epi.row_stats(m0 + r, tc.nt, m, sum);
    }
  }
}

template <class C, bool AK, bool BKM, class Epi, bool SEGA>
__global__ void __launch_bounds__(C::THREADS, C::OCC)
    gemm_pipe_kernel(View A, View B, int64_t M, int64_t N, int64_t K, int64_t ksplit,
                     TileMap tm, Epi epi) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LdsBytes];
  TileCoord tc;
  if (!tile_coord(tm, blockIdx.x, tc)) return;  // uniform over the workgroup
  run_tile<C, AK, BKM, Epi, SEGA>(A, B, M, N, K, ksplit, tc, epi, lds);
}

// C[M, N] = A · B over K with configuration C; `splits` > 1 cuts K into that many ranges
// (multiples of C::BK), each its own tile set handed to the epilogue with its index.
// xcd_blocks (splits == 1, at least 8 m-tiles) hands each XCD a block of the m × n tile
// grid instead of a run of consecutive tiles: with n split xn ways (xn = 4, 2 or 1, the
// first that divides the n-tile count) an XCD reads 1 / xn of B and xn / 8 of A; worth it
// when B is re-read by every m-tile and too large for one L2.
template <class C, bool AK, bool BKM, class Epi, bool SEGA = false>
hipError_t launch(const View& A, const View& B, int64_t M, int64_t N, int64_t K, int64_t splits,
                  bool m_fast, const Epi& epi, hipStream_t s, bool xcd_blocks = false) {
  // grouped K-major operands keep whole groups of 64 (see stream_at)
  if ((AK && A.gs < 64) || (BKM && B.gs < 64)) return hipErrorInvalidValue;
  // a two-segment A: MN-major rows or K-major panel columns, both segments given, split at a
  // slice boundary (a panel boundary for panels); MN-major panels come in one segment
  if (SEGA && (A.p2 == nullptr || A.kseg <= 0 || A.kseg % C::BK != 0 ||
               (AK ? (A.ext <= 0 || A.ext2 <= 0 || A.kseg % 64 != 0 || A.kseg >= A.cols)
                   : (A.ext > 0 || A.kseg >= A.rows))))
    return hipErrorInvalidValue;
  TileMap tm{(M + C::BM - 1) / C::BM, (N + C::BN - 1) / C::BN, splits < 1 ? 1 : splits, m_fast};
  int64_t ksplit = (K + tm.splits - 1) / tm.splits;
  ksplit = (ksplit + C::BK - 1) / C::BK * C::BK;
  int64_t grid = tm.m_tiles * tm.n_tiles * tm.splits;
  if (xcd_blocks && tm.splits == 1 && tm.m_tiles >= 8) {
    tm.xn = tm.n_tiles % 4 == 0 ? 4 : (tm.n_tiles % 2 == 0 ? 2 : 1);
    const int64_t gm = 8 / tm.xn;
    grid = 8 * ((tm.m_tiles + gm - 1) / gm) * (tm.n_tiles / tm.xn);
  }
  hipLaunchKernelGGL((gemm_pipe_kernel<C, AK, BKM, Epi, SEGA>), dim3(unsigned(grid)),
                     dim3(C::THREADS), 0, s, A, B, M, N, K, ksplit, tm, epi);
  return hipGetLastError();
}

}  // namespace v2
}  // namespace gemm
}  // namespace lce
