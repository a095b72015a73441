// Fused linear cross-entropy for gfx950: loss, grad_hidden, fp32 grad_weight and grad_bias
// from hidden [n, h] and weight [v, h] without keeping the [n, v] logits.
//
// What is computed follows Liger-Kernel issue #533 ("Gradient checkpointing for grad_weight
// in LFCE"), feature pitch: per chunk of rows the logits are input · weightᵀ, the CE
// gradient of those logits is formed, and grad_weight collects (logits gradient)ᵀ · input;
// and Liger-Kernel issue #941 ("No gain in VRAM usage with
// LigerFusedLinearCrossEntropyLoss"): hidden, targets, lm_head weight and optional bias.
// The CE part is the sum-reduced masked CE of NeMo Automodel PR #2996 (first commit
// message).
//
// Schedule, per chunk of C rows (rows are processed chunk after chunk on one stream):
//   1. logits GEMM   Z = H_c · Wᵀ + b  (bf16 MFMA, fp32 accumulate) → fp32 slice [C, ldz]
//   2. row pass      lse_i, loss term lse_i − z_{i,y_i}
//   3. bias pass     grad_bias += g·s·Σ_i (p_iv − [y_i = v])   (only when requested)
//   4. convert       P = bf16(exp(Z − lse)) written in place over the fp32 slice: each
//                    64-column group keeps its probabilities in the first half of the
//                    bytes its fp32 logits occupied, so the slice is the only big buffer
//   5. grad_hidden   dH_c = g·s·(P · W − W[y])     (bf16 MFMA over K = V; the one-hot
//                    term is subtracted exactly in fp32 in the epilogue)
//   6. grad_weight   dW (=|+=) g·s·Pᵀ · H_c         (bf16 MFMA over K = C)
//   7. one-hot fix   dW[y] −= g·s·Σ_{i: y_i = y} h_i, in a fixed order (no atomics)
// The probabilities enter the MFMA as unscaled bf16; the scale g·s and the one-hot are
// applied in fp32, which keeps the fp32 grad_weight within 1e-4 normwise of the exact
// result (scaling or subtracting inside the bf16 operand would not).
//
// Where h is a multiple of 64 and C >= 64 (the compact workspace: the slice and nothing
// else), the stored-logits schedule keeps each chunk's logits as fp16(z − tile max), two
// chunks per slice, and runs step 6 once per two chunks (flce_paired): the fp32 accumulator
// is then read and written half as often. When, in addition, grad_weight is overwritten, C is
// a multiple of 64 and the batch is no longer than about 2h (flce_transposed), steps 4-7 run
// over the whole batch instead: every row's probabilities are kept, transposed, in the slice
// and in grad_weight's own bytes, then grad_hidden is one product over all rows and
// grad_weight one plain product per vocabulary range, with no fp32 read-modify-write. The
// lse and the loss come from the fp32 logits in every form.
#include <algorithm>

#include "common.h"
#include "flce.h"
#include "gemm_tile.h"
#include "lce_masked.h"

namespace lce {

namespace {

constexpr int kGroup = 64;  // column-group width of the logits slice / probability layout

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

using gemm::View;
using Wide = gemm::v2::CfgWide;  // the two large-K products
using Pair = gemm::v2::CfgPair;  // grad_weight: fp32 read-modify-write epilogue

// grad_weight over K = `rows` chunk rows into the fp32 accumulator. Two 256 × 128
// workgroups per CU overlap one's read-modify-write epilogue with the other's MFMAs; from
// K = 4096 on, a 256 × 256 tile's mainloop is long enough that its faster operand stream
// wins back more than its exposed epilogue costs. Measured, ms per step on 256 × 128 against
// 256 × 256: Llama3-8B head, K = 1024, 11.9 against 13.3; K = 2048, 9.00–9.05 against 9.07;
// long-context workload, K = 4096, 65.7 against 64.2–64.4.
constexpr int64_t kGradWeightWideK = 4096;
template <class Epi>
hipError_t launch_grad_weight(const View& A, const View& B, int64_t v, int64_t h, int64_t rows,
                              const Epi& e, hipStream_t s) {
  if (rows >= kGradWeightWideK)
    return gemm::v2::launch<Wide, false, false>(A, B, v, h, rows, 1, false, e, s, true);
  return gemm::v2::launch<Pair, false, false>(A, B, v, h, rows, 1, false, e, s, true);
}

__device__ __forceinline__ float flce_coef(const long long* count_dev, long long count_host,
                                           const float* gout) {
  const long long t = count_host >= 0 ? count_host : *count_dev;
  const float g = gout ? *gout : 1.f;
  return t > 0 ? float(double(g) / double(t)) : 0.f;
}

__device__ __forceinline__ bool has_label(int32_t y, int64_t v, int32_t ignore_index) {
  return y != ignore_index && y >= 0 && int64_t(y) < v;
}

// Z[m, n] = acc + bias[n] into the fp32 slice. With the pipelined GEMM it also leaves, per row
// m and 256-column tile t, part[m · part_ld + t] = (max_n z, Σ_n exp(z − max)) over the tile:
// the logsumexp of each row is then a merge of ⌈V / 256⌉ pairs instead of a pass over Z.
struct EpiLogits {
  static constexpr bool kColSums = false;
  static constexpr bool kTileMax = false;
  float* z;
  int64_t ldz;
  const float* bias;
  float2* part;
  int64_t part_ld;
  static constexpr bool kRowStats = true;
  __device__ void begin(int64_t) {}
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float a) {
    z[m * ldz + n] = bias ? a + bias[n] : a;
  }
  using Aux = gemm::f32x4_t;
  __device__ __forceinline__ Aux load4(int64_t, int64_t n) const {
    return bias ? Aux{bias[n], bias[n + 1], bias[n + 2], bias[n + 3]} : Aux{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, gemm::f32x4_t a, Aux b) {
    *reinterpret_cast<gemm::f32x4_t*>(z + m * ldz + n) = a + b;
  }
  __device__ __forceinline__ gemm::f32x4_t value4(gemm::f32x4_t a, Aux b) const { return a + b; }
  __device__ __forceinline__ float value1(int64_t n, float a) const { return bias ? a + bias[n] : a; }
  __device__ __forceinline__ void row_stats(int64_t m, int64_t t, float mx, float sum) {
    part[m * part_ld + t] = float2{mx, sum};
  }
};

// fp16 encoding of a shifted logit (round to nearest even) and back (exact).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = static_cast<_Float16>(lo), b = static_cast<_Float16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xffffu)));
}

// The stored-logits schedule's logits tile in 16 bits: d = fp16(z − m_t) into a 16-bit
// [rows, ldz] array, m_t = the row's maximum over this 256-column tile (known before the
// stores, see kTileMax). The per-tile (max, Σ exp(z − max)) pairs come from the fp32 values
// as in EpiLogits (so the lse is unchanged), and the label logit is kept in fp32 in zy[m]
// (the loss term is then exact); the row's label is its row_tag. exp(d + m_t − lse) is within 2^-11 · |z − m_t| relative of
// the exact probability, and a chunk's logits take half the bytes of the fp32 slice.
struct EpiLogits16 {
  static constexpr bool kColSums = false;
  static constexpr bool kTileMax = true;
  static constexpr bool kRowStats = true;
  uint16_t* z;
  int64_t ldz;
  const float* bias;
  float2* part;
  int64_t part_ld;
  const int32_t* labels;
  float* zy;
  __device__ void begin(int64_t) {}
  __device__ __forceinline__ void operator()(int64_t, int64_t, float) {}  // put1m instead
  __device__ __forceinline__ int row_tag(int64_t m) const { return labels[m]; }
  __device__ __forceinline__ void put1m(int64_t m, int64_t n, float a, float mx, int y) {
    const float x = bias ? a + bias[n] : a;
    z[m * ldz + n] = uint16_t(pack_f16x2(x - mx, 0.f) & 0xffffu);
    if (int64_t(y) == n) zy[m] = x;
  }
  using Aux = gemm::f32x4_t;
  __device__ __forceinline__ Aux load4(int64_t, int64_t n) const {
    return bias ? Aux{bias[n], bias[n + 1], bias[n + 2], bias[n + 3]} : Aux{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void store4m(int64_t m, int64_t n, gemm::f32x4_t a, Aux b, float mx,
                                          int y) {
    const gemm::f32x4_t x = a + b;
    *reinterpret_cast<uint2*>(z + m * ldz + n) =
        uint2{pack_f16x2(x[0] - mx, x[1] - mx), pack_f16x2(x[2] - mx, x[3] - mx)};
    const int64_t d = int64_t(y) - n;
    if (d >= 0 && d < 4) zy[m] = d == 0 ? x[0] : d == 1 ? x[1] : d == 2 ? x[2] : x[3];
  }
  __device__ __forceinline__ gemm::f32x4_t value4(gemm::f32x4_t a, Aux b) const { return a + b; }
  __device__ __forceinline__ float value1(int64_t n, float a) const { return bias ? a + bias[n] : a; }
  __device__ __forceinline__ void row_stats(int64_t m, int64_t t, float mx, float sum) {
    part[m * part_ld + t] = float2{mx, sum};
  }
};

// Once the slice holds probabilities (first half of every 64-column group), the second half
// of every group is free scratch: flat element e sits at float offset (e / 32) * 64 + 32 +
// e % 32. It takes grad_hidden's split-K partial sums and the recomputing schedule's
// probability column sums.
__host__ __device__ __forceinline__ int64_t gap_index(int64_t e) {
  return (e >> 5) * 64 + 32 + (e & 31);
}

// Where row i's lse sits: lse[i], or (gap >= 0) flat free-half element gap + i of the slice
// that lse points at, for a schedule with no other room beside the probabilities.
__device__ __forceinline__ int64_t lse_off(int64_t gap, int64_t i) {
  return gap < 0 ? i : gap_index(gap + i);
}

// One fp32 value per chunk row kept in memory the call owns anyway: p[i] (layout 0), or the
// slice's free halves from element `base` on (layout 2). p == nullptr: none.
struct RowVec {
  float* p;
  int64_t base;
  int layout;
  __device__ __forceinline__ float& operator[](int64_t i) const {
    if (layout == 2) return p[gap_index(base + i)];
    return p[i];
  }
};

// The label's one-hot coefficient with the rounding residual of the label's bf16
// probability: the products see q = bf16(p_y) where the gradient wants p_y, so the fp32
// one-hot term subtracts (1 − (p_y − q)) instead of 1, which makes the label element's
// total exactly p_y − 1 up to fp32 rounding. p − q is exact (q is p rounded, within a factor
// of two of it). Without it the label element carries q's rounding, up to 2^-9 · p_y, which
// for rows a model predicts well (p_y near 1) is as large as the whole label gradient.
__device__ __forceinline__ float label_coef(float p, float q) { return 1.f - (p - q); }

// Pass 1 of the recomputing schedule: the logits tile is only reduced, never stored. Leaves
// the per-tile (max, Σ exp) pairs like EpiLogits, and zy[m] = z[m, y_m] for the tile holding
// the label column.
struct EpiLseOnly {
  const float* bias;
  float2* part;
  int64_t part_ld;
  const int32_t* labels;
  float* zy;
  static constexpr bool kRowStats = true;
  static constexpr bool kColSums = false;
  static constexpr bool kTileMax = false;
  __device__ void begin(int64_t) {}
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float a) {
    if (int64_t(labels[m]) == n) zy[m] = bias ? a + bias[n] : a;
  }
  using Aux = gemm::f32x4_t;
  __device__ __forceinline__ Aux load4(int64_t, int64_t n) const {
    return bias ? Aux{bias[n], bias[n + 1], bias[n + 2], bias[n + 3]} : Aux{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, gemm::f32x4_t a, Aux b) {
    const int64_t d = int64_t(labels[m]) - n;
    if (d >= 0 && d < 4) {
      const gemm::f32x4_t z = a + b;
      zy[m] = d == 0 ? z[0] : d == 1 ? z[1] : d == 2 ? z[2] : z[3];
    }
  }
  __device__ __forceinline__ gemm::f32x4_t value4(gemm::f32x4_t a, Aux b) const { return a + b; }
  __device__ __forceinline__ float value1(int64_t n, float a) const { return bias ? a + bias[n] : a; }
  __device__ __forceinline__ void row_stats(int64_t m, int64_t t, float mx, float sum) {
    part[m * part_ld + t] = float2{mx, sum};
  }
};

// Pass 2 of the recomputing schedule: the recomputed logits tile becomes bf16 probabilities
// P = exp(z − lse) in the slice's probability layout (first half of every 64-column group,
// p_gs = 128; or a dense [rows, ldz] array, p_gs = 64, when two chunks share the slice),
// 0 for rows without a label and for the padding columns v .. ldz − 1 (the GEMM runs over
// N = ldz; weight rows past v read as zero). With grad_bias it also leaves, per 256-row tile
// mt and column n, Σ_m p (the fp32 values, before rounding) as flat element mt · v + n of the
// slice's free halves.
struct EpiProbs {
  uint16_t* p;
  int64_t p_ld;  // elements between rows (2 · ldz, or ldz when dense)
  int64_t p_gs;  // elements between 64-column groups (128, or 64 when dense)
  const float* bias;
  const float* lse;
  int64_t lse_gap;  // lse layout (lse_off)
  const int32_t* labels;
  int64_t v;
  int32_t ignore_index;
  float* colsum;  // the slice as floats, or NULL: no column sums
  RowVec coef_out, coef_out2;  // each labelled row's label_coef (second copy optional)
  static constexpr bool kRowStats = false;
  static constexpr bool kColSums = true;
  static constexpr bool kTileMax = false;
  __device__ void begin(int64_t) {}
  __device__ __forceinline__ int64_t at(int64_t m, int64_t n) const {
    return m * p_ld + (n >> 6) * p_gs + (n & 63);
  }
  struct Aux {
    gemm::f32x4_t b;
    float c;  // the row's lse, or NaN for a row without a label
    int y;    // the row's label
  };
  __device__ __forceinline__ Aux load4(int64_t m, int64_t n) const {
    Aux x;
    x.b = gemm::f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (bias) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < v) x.b[q] = bias[n + q];
    }
    x.y = labels[m];
    x.c = has_label(x.y, v, ignore_index) ? lse[lse_off(lse_gap, m)] : __builtin_nanf("");
    return x;
  }
  __device__ __forceinline__ gemm::f32x4_t colvalue4(gemm::f32x4_t a, Aux x) const {
    gemm::f32x4_t r{0.f, 0.f, 0.f, 0.f};
    if (x.c == x.c) {  // labelled row
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = fast_exp2(((a[q] + x.b[q]) - x.c) * kLog2e);
    }
    return r;
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, gemm::f32x4_t a, Aux x) {
    gemm::f32x4_t r = colvalue4(a, x);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (n + q >= v) r[q] = 0.f;
    const uint2 o = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    *reinterpret_cast<uint2*>(p + at(m, n)) = o;
    const int64_t d = int64_t(x.y) - n;
    if (coef_out.p && d >= 0 && d < 4 && x.c == x.c) {  // this row's label column
      const float pr = r[int(d)];
      const float q = d < 2 ? (d == 0 ? bf16_lo(o.x) : bf16_hi(o.x)) : (d == 2 ? bf16_lo(o.y) : bf16_hi(o.y));
      coef_out[m] = label_coef(pr, q);
      if (coef_out2.p) coef_out2[m] = label_coef(pr, q);
    }
  }
  __device__ __forceinline__ void operator()(int64_t, int64_t, float) {}  // N % 4 == 0: unused
  __device__ __forceinline__ void col_sums(int64_t mt, int64_t n, float sum) {
    if (colsum && n < v) colsum[gap_index(mt * v + n)] = sum;
  }
};

// dH[m, n] = coef · (acc − W[y_m, n]) for labelled rows, 0 otherwise; bf16 out.
struct EpiGradHidden {
  static constexpr bool kColSums = false;
  static constexpr bool kTileMax = false;
  static constexpr bool kRowStats = false;
  uint16_t* dh;
  int64_t ldh;
  const int32_t* labels;  // chunk rows
  const uint16_t* w;
  int64_t ldw, v;
  int32_t ignore_index;
  const long long* count_dev;
  long long count_host;
  const float* gout;
  float coef;
  RowVec ycoef;  // each labelled row's label_coef
  __device__ void begin(int64_t) { coef = flce_coef(count_dev, count_host, gout); }
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float a) {
    const int32_t y = labels[m];
    float r = 0.f;
    if (has_label(y, v, ignore_index))
      r = coef * (a - ycoef[m] * bf16_to_f32(w[int64_t(y) * ldw + n]));
    dh[m * ldh + n] = f32_to_bf16(r);
  }
  // aux: the 4 weights W[y_m, n .. n+3] as two bf16 pairs and the row's label coefficient;
  // ok = 0 for a row without label. The row's label comes in as its tag (loaded once per
  // tile) and the weight load does not branch on it (row 0 stands in for a row without a
  // label), so the gathers of a batch are in flight together.
  static constexpr bool kRowTag = true;
  __device__ __forceinline__ int row_tag(int64_t m) const { return labels[m]; }
  struct Aux {
    uint32_t a, b, ok;
    float c;
  };
  __device__ __forceinline__ Aux load4t(int64_t m, int64_t n, int y) const {
    const bool ok = has_label(y, v, ignore_index);
    const uint2 wy = *reinterpret_cast<const uint2*>(w + (ok ? int64_t(y) : 0) * ldw + n);
    return Aux{wy.x, wy.y, ok ? 1u : 0u, ycoef[m]};
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, gemm::f32x4_t a, Aux x) {
    uint2 o = {0u, 0u};
    if (x.ok) {
      o.x = pack_bf16x2(coef * (a[0] - x.c * bf16_lo(x.a)), coef * (a[1] - x.c * bf16_hi(x.a)));
      o.y = pack_bf16x2(coef * (a[2] - x.c * bf16_lo(x.b)), coef * (a[3] - x.c * bf16_hi(x.b)));
    }
    *reinterpret_cast<uint2*>(dh + m * ldh + n) = o;
  }
};

// dW[m, n] = (overwrite ? 0 : dW[m, n]) + coef · acc.
struct EpiGradWeight {
  static constexpr bool kColSums = false;
  static constexpr bool kTileMax = false;
  static constexpr bool kRowStats = false;
  float* dw;
  int64_t ldw;
  int overwrite;
  const long long* count_dev;
  long long count_host;
  const float* gout;
  float coef;
  __device__ void begin(int64_t) { coef = flce_coef(count_dev, count_host, gout); }
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float a) {
    float* p = dw + m * ldw + n;
    *p = overwrite ? coef * a : *p + coef * a;
  }
  using Aux = gemm::f32x4_t;
  __device__ __forceinline__ Aux load4(int64_t m, int64_t n) const {
    if (overwrite) return Aux{0.f, 0.f, 0.f, 0.f};
    return *reinterpret_cast<const gemm::f32x4_t*>(dw + m * ldw + n);
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, gemm::f32x4_t a, Aux old) {
    *reinterpret_cast<gemm::f32x4_t*>(dw + m * ldw + n) = old + coef * a;
  }
};

// One chunk's rows sorted by label, stably (rows in increasing order within a label):
// slab[p] is the chunk's p-th smallest label (rows without a label count as 0x7fffffff and
// come last) and srow[p] its row. Each row's sort key is label · kSortMax + row, all keys
// distinct, so a row's position is the number of keys below its own. Workgroup b places
// rows 64 b .. 64 b + 63: its kRankWaves wavefronts count over one slice each of the keys,
// held in LDS (one 64-bit compare per key), and the counts are added.
constexpr int kSortMax = 8192;
constexpr int kRankWaves = 16;
__global__ void __launch_bounds__(64 * kRankWaves) label_rank_kernel(
    const int32_t* __restrict__ labels, int64_t rows, int64_t v, int32_t ignore_index,
    int32_t* __restrict__ slab, int32_t* __restrict__ srow) {
  __shared__ __attribute__((aligned(16))) long long k[kSortMax];
  __shared__ int cnt[kRankWaves][64];
  const int n = int(rows);
  const int n2 = (n + 1) & ~1;  // padded with the largest key: never below any row's
  for (int i = threadIdx.x; i < n2; i += 64 * kRankWaves) {
    long long key = 0x7fffffffffffffffLL;
    if (i < n) {
      const int32_t y = labels[i];
      key = (long long)(has_label(y, v, ignore_index) ? y : 0x7fffffff) * kSortMax + i;
    }
    k[i] = key;
  }
  __syncthreads();
  const int r = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int i = int(blockIdx.x) * 64 + r;
  int rank = 0;
  if (i < n) {
    const long long x = k[i];
    const int per = ((n2 + kRankWaves - 1) / kRankWaves + 1) & ~1;  // even, kRankWaves · per >= n2
    const int lo = q * per, hi = lo + per < n2 ? lo + per : n2;
    for (int j = lo; j < hi; j += 2) {
      const longlong2 c = *reinterpret_cast<const longlong2*>(k + j);
      rank += int(c.x < x) + int(c.y < x);
    }
  }
  cnt[q][r] = rank;
  __syncthreads();
  if (q == 0 && i < n) {
    int p = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) p += cnt[w][r];
    slab[p] = int32_t(k[i] / kSortMax);
    srow[p] = i;
  }
}

// dW[y] −= coef · Σ_{i in chunk, y_i = y} h_i. Workgroup p handles sorted position p if it
// starts a run of equal labels: it adds the run's hidden rows in increasing row order and
// updates dW row y once.
__global__ void __launch_bounds__(256) onehot_segments_kernel(
    const uint16_t* __restrict__ hidden, int64_t h, int64_t rows,
    const int32_t* __restrict__ slab, const int32_t* __restrict__ srow, int64_t v,
    float* grad_weight, const long long* count_dev, long long count_host, const float* gout,
    RowVec ycoef) {
  const int64_t p = blockIdx.x;
  const int32_t y = slab[p];
  if (y >= v || (p > 0 && slab[p - 1] == y)) return;
  int64_t end = p + 1;
  while (end < rows && slab[end] == y) ++end;
  const float coef = flce_coef(count_dev, count_host, gout);
  for (int64_t col = 4 * int64_t(threadIdx.x); col < h; col += 4 * 256) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int64_t e = p; e < end; ++e) {
      const int64_t r = srow[e];
      const float c = ycoef[r];  // the row's label coefficient (1 − its label residual)
      const uint16_t* hr = hidden + r * h + col;
      if (col + 4 <= h) {
        const uint2 x = *reinterpret_cast<const uint2*>(hr);
        a0 += c * bf16_lo(x.x); a1 += c * bf16_hi(x.x); a2 += c * bf16_lo(x.y); a3 += c * bf16_hi(x.y);
      } else {
        a0 += c * bf16_to_f32(hr[0]);
        if (col + 1 < h) a1 += c * bf16_to_f32(hr[1]);
        if (col + 2 < h) a2 += c * bf16_to_f32(hr[2]);
      }
    }
    float* d = grad_weight + int64_t(y) * h + col;
    d[0] -= coef * a0;
    if (col + 1 < h) d[1] -= coef * a1;
    if (col + 2 < h) d[2] -= coef * a2;
    if (col + 3 < h) d[3] -= coef * a3;
  }
}


// grad_hidden's fp32 split-K partial sums: element e of split z at float dense ? z·M·N + e :
// gap_index(z·M·N + e) of `slice` (the free halves of the slice's 64-column groups, or a
// region of its own).
struct EpiPartial {
  static constexpr bool kColSums = false;
  static constexpr bool kTileMax = false;
  static constexpr bool kRowStats = false;
  float* slice;
  int64_t M, N;
  int64_t kz;
  int dense;
  __device__ void begin(int64_t z) { kz = z; }
  __device__ __forceinline__ int64_t at(int64_t e) const { return dense ? e : gap_index(e); }
  __device__ __forceinline__ void operator()(int64_t m, int64_t n, float a) {
    slice[at((kz * M + m) * N + n)] = a;
  }
  struct Aux {};
  __device__ __forceinline__ Aux load4(int64_t, int64_t) const { return Aux{}; }
  // N % 4 == 0 and n % 4 == 0 keep the 4 values inside one 32-float gap
  __device__ __forceinline__ void store4(int64_t m, int64_t n, gemm::f32x4_t a, Aux) {
    *reinterpret_cast<gemm::f32x4_t*>(slice + at((kz * M + m) * N + n)) = a;
  }
};

// dH[m, n] = coef · (Σ_z partial_z[m, n] − W[y_m, n]), summed in split order; bf16 out. Each
// lane takes 4 consecutive elements (N % 4 == 0: a 16-byte read of each split's partials,
// which stay inside one 32-float gap, 8-byte accesses to W and dH).
__global__ void __launch_bounds__(256) grad_hidden_reduce_kernel(
    const float* __restrict__ slice, int dense, int64_t M, int64_t N, int64_t splits,
    uint16_t* __restrict__ dh, const int32_t* __restrict__ labels, const uint16_t* __restrict__ w,
    int64_t v, int32_t ignore_index, const long long* count_dev, long long count_host,
    const float* gout, RowVec ycoef) {
  const int64_t e = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= M * N) return;
  const int64_t m = e / N, n = e % N;
  const int32_t y = labels[m];
  uint2 o = {0u, 0u};
  if (has_label(y, v, ignore_index)) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t z = 0; z < splits; ++z) {
      const int64_t f = z * M * N + e;
      const float4 p = *reinterpret_cast<const float4*>(slice + (dense ? f : gap_index(f)));
      acc.x += p.x;
      acc.y += p.y;
      acc.z += p.z;
      acc.w += p.w;
    }
    const float coef = flce_coef(count_dev, count_host, gout);
    const float c = ycoef[m];
    const uint2 wy = *reinterpret_cast<const uint2*>(w + int64_t(y) * N + n);
    o.x = pack_bf16x2(coef * (acc.x - c * bf16_lo(wy.x)), coef * (acc.y - c * bf16_hi(wy.x)));
    o.y = pack_bf16x2(coef * (acc.z - c * bf16_lo(wy.y)), coef * (acc.w - c * bf16_hi(wy.y)));
  }
  *reinterpret_cast<uint2*>(dh + e) = o;
}

// ------------------------------------------------------------------ row / column passes

constexpr int kRowThreads = 256;

// lse of one fp32 slice row; loss term and lse written for labelled rows. 16-byte loads,
// four in flight per lane; rows are 256-byte aligned (ldz % 64 == 0), so only the last
// vector of a row can be partial.
__global__ void __launch_bounds__(kRowThreads) slice_row_lse_kernel(
    const float* __restrict__ z, int64_t ldz, int64_t v, const int32_t* __restrict__ labels,
    int32_t ignore_index, float* __restrict__ lse_c, float* __restrict__ row_loss,
    float* __restrict__ lse_out) {
  const int64_t i = blockIdx.x;
  const int32_t y = labels[i];
  if (!has_label(y, v, ignore_index)) {
    if (threadIdx.x == 0) {
      lse_c[i] = 0.f;
      row_loss[i] = 0.f;
      if (lse_out) lse_out[i] = 0.f;
    }
    return;
  }
  const float* row = z + i * ldz;
  const float4* r4 = reinterpret_cast<const float4*>(row);
  const int64_t nfull = v >> 2;
  float m = -INFINITY, s = 0.f;
  auto absorb = [&](const float* x, int cnt) {
    float mx = x[0];
    for (int k = 1; k < cnt; ++k) mx = fmaxf(mx, x[k]);
    const float mn = fmaxf(m, mx);
    float acc = (m == mn) ? s : s * fast_exp2((m - mn) * kLog2e);
    for (int k = 0; k < cnt; ++k) acc += fast_exp2((x[k] - mn) * kLog2e);
    s = acc;
    m = mn;
  };
  int64_t j = threadIdx.x;
  for (; j + 3 * kRowThreads < nfull; j += 4 * kRowThreads) {
    float4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = r4[j + u * kRowThreads];
    float x[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[4 * u] = q[u].x; x[4 * u + 1] = q[u].y; x[4 * u + 2] = q[u].z; x[4 * u + 3] = q[u].w;
    }
    absorb(x, 16);
  }
  for (; j < nfull; j += kRowThreads) {
    const float4 q = r4[j];
    const float x[4] = {q.x, q.y, q.z, q.w};
    absorb(x, 4);
  }
  if (threadIdx.x < (v & 3)) {
    const float x = row[nfull * 4 + threadIdx.x];
    absorb(&x, 1);
  }
  __shared__ float sm[kRowThreads / 64], ss[kRowThreads / 64];
  wave_lse_reduce(m, s);
  if ((threadIdx.x & 63) == 0) {
    sm[threadIdx.x >> 6] = m;
    ss[threadIdx.x >> 6] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = sm[0], sss = ss[0];
    for (int w = 1; w < kRowThreads / 64; ++w) lse_merge(mm, sss, sm[w], ss[w]);
    const float lse = mm + fast_log2(sss) * kLn2;
    lse_c[i] = lse;
    row_loss[i] = lse - row[y];
    if (lse_out) lse_out[i] = lse;
  }
}

// lse of each labelled row from the logits GEMM's per-tile (max, Σ exp) pairs, merged in a
// fixed order; loss term lse − z[y] and lse_out. z[y] comes from zy when given, else from the
// fp32 slice; zy and row_loss may be the same array (each row reads its label logit before
// writing its term). The lse goes to lse_c in the layout lse_gap names (lse_off). One
// wavefront per row.
//
// With `yc` (the stored-logits schedule that keeps fp16(z − m_t), whose probability pass is
// shifted_to_probs_kernel): each labelled row's label_coef, from the fp32 label logit and the
// label's probability operand exactly as that pass will form it; also into yc2 when given.
__global__ void __launch_bounds__(256) lse_merge_rows_kernel(
    const float2* __restrict__ part, int64_t tiles, const float* __restrict__ z, int64_t ldz,
    const float* zy, int64_t rows, int64_t v, const int32_t* __restrict__ labels,
    int32_t ignore_index, float* __restrict__ lse_c, int64_t lse_gap,
    float* row_loss, float* __restrict__ lse_out, RowVec yc, RowVec yc2) {
  const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= rows) return;
  const int32_t y = labels[i];
  if (!has_label(y, v, ignore_index)) {
    if (lane == 0) {
      lse_c[lse_off(lse_gap, i)] = 0.f;
      row_loss[i] = 0.f;
      if (lse_out) lse_out[i] = 0.f;
    }
    return;
  }
  float m = -INFINITY, sum = 0.f;
  for (int64_t t = lane; t < tiles; t += 64) {
    const float2 p = part[i * tiles + t];
    lse_merge(m, sum, p.x, p.y);
  }
  wave_lse_reduce(m, sum);
  if (lane == 0) {
    const float lse = m + fast_log2(sum) * kLn2;
    const float zl = zy ? zy[i] : z[i * ldz + y];
    lse_c[lse_off(lse_gap, i)] = lse;
    row_loss[i] = lse - zl;
    if (lse_out) lse_out[i] = lse;
    if (yc.p) {
      const float mt = part[i * tiles + (y >> 8)].x;  // the label column's tile maximum
      const float d = f16_to_f32(pack_f16x2(zl - mt, 0.f));
      const float q = bf16_lo(pack_bf16x2(fast_exp2((d + (mt - lse)) * kLog2e), 0.f));
      const float c = label_coef(fast_exp2((zl - lse) * kLog2e), q);
      yc[i] = c;
      if (yc2.p) yc2[i] = c;
    }
  }
}

// grad_bias[v] (=|+=) coef · (Σ_{labelled i} p_iv − #{i: y_i = v}). One 1024-thread
// workgroup per 128 columns: lane l of wavefront w takes the 8 columns 8 (l % 16) .. + 7 of
// the block (one 16-byte load per row) over the rows i ≡ 4 w + l / 16 (mod 64), in
// increasing order, four rows' loads in flight; the 64 partial sums of a column are then
// added in residue order through LDS, the same order on every run.
// prob.load8(i, c0, p) gives p_iv in fp32 (before any bf16 rounding) for the 8 columns
// c0 .. c0 + 7, c0 < v and c0 + 8 <= ldz.
constexpr int kBiasCols = 64, kBiasWaves = 16;  // bias_from_colsums_kernel
constexpr int kBiasBlockCols = 128, kBiasThreads = 1024, kBiasParts = 64;

template <class Prob>
__device__ __forceinline__ void bias_grad_columns(const Prob& prob, int64_t rows, int64_t v,
                                                  const int32_t* __restrict__ labels,
                                                  int32_t ignore_index, float* grad_bias,
                                                  int overwrite, const long long* count_dev,
                                                  long long count_host, const float* gout) {
  __shared__ float ps[kBiasParts][kBiasBlockCols];
  __shared__ int pc[kBiasParts][kBiasBlockCols];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cg = lane & 15, part = 4 * wv + (lane >> 4);
  const int64_t c0 = int64_t(blockIdx.x) * kBiasBlockCols + 8 * cg;
  float sp[8];
  int cnt[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    sp[q] = 0.f;
    cnt[q] = 0;
  }
  if (c0 < v) {
    for (int64_t i0 = part; i0 < rows; i0 += 4 * kBiasParts) {
      int32_t y[4];
      float p[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kBiasParts;
        y[u] = i < rows ? labels[i] : -1;
        if (i < rows) prob.load8(i, c0, p[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!has_label(y[u], v, ignore_index)) continue;
        const int64_t d = int64_t(y[u]) - c0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (c0 + q < v) sp[q] += p[u][q];
          cnt[q] += d == q;
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    ps[part][8 * cg + q] = sp[q];
    pc[part][8 * cg + q] = cnt[q];
  }
  __syncthreads();
  if (threadIdx.x < kBiasBlockCols) {
    const int64_t col = int64_t(blockIdx.x) * kBiasBlockCols + threadIdx.x;
    if (col < v) {
      float s = 0.f;
      int c = 0;
#pragma unroll 8
      for (int r = 0; r < kBiasParts; ++r) {
        s += ps[r][threadIdx.x];
        c += pc[r][threadIdx.x];
      }
      const float d = flce_coef(count_dev, count_host, gout) * (s - float(c));
      grad_bias[col] = overwrite ? d : grad_bias[col] + d;
    }
  }
}

// p from the fp32 slice: exp(z − lse) (rows of 64-column groups, so c0 is 32-byte aligned).
struct SliceProb {
  const float* z;
  int64_t ldz;
  const float* lse_c;
  __device__ __forceinline__ void load8(int64_t i, int64_t c0, float (&p)[8]) const {
    const float4 a = *reinterpret_cast<const float4*>(z + i * ldz + c0);
    const float4 b = *reinterpret_cast<const float4*>(z + i * ldz + c0 + 4);
    const float c = lse_c[i];
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) p[q] = fast_exp2((x[q] - c) * kLog2e);
  }
};

__global__ void __launch_bounds__(kBiasThreads) slice_bias_grad_kernel(
    const float* __restrict__ z, int64_t ldz, int64_t rows, int64_t v,
    const int32_t* __restrict__ labels, int32_t ignore_index, const float* __restrict__ lse_c,
    float* __restrict__ grad_bias, int overwrite, const long long* count_dev,
    long long count_host, const float* gout) {
  bias_grad_columns(SliceProb{z, ldz, lse_c}, rows, v, labels, ignore_index, grad_bias,
                    overwrite, count_dev, count_host, gout);
}

// grad_bias[v] (=|+=) coef · (Σ_mt colsum[mt, v] − #{labelled i: y_i = v}), the column sums
// (in the slice's free halves) added in row-tile order; the label count split over the
// wavefronts as in bias_grad_columns.
__global__ void __launch_bounds__(64 * kBiasWaves) bias_from_colsums_kernel(
    const float* __restrict__ colsum, int64_t mtiles, int64_t rows, int64_t v,
    const int32_t* __restrict__ labels, int32_t ignore_index, float* __restrict__ grad_bias,
    int overwrite, const long long* count_dev, long long count_host, const float* gout) {
  __shared__ int pc[kBiasWaves][kBiasCols];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t col = int64_t(blockIdx.x) * kBiasCols + lane;
  int cnt = 0;
  if (col < v) {
    for (int64_t i = wv; i < rows; i += kBiasWaves) {
      const int32_t y = labels[i];
      cnt += (has_label(y, v, ignore_index) && int64_t(y) == col);
    }
  }
  pc[wv][lane] = cnt;
  __syncthreads();
  if (wv == 0 && col < v) {
    float sp = 0.f;
    for (int64_t t = 0; t < mtiles; ++t) sp += colsum[gap_index(t * v + col)];
    int c = 0;
#pragma unroll
    for (int w = 0; w < kBiasWaves; ++w) c += pc[w][lane];
    const float d = flce_coef(count_dev, count_host, gout) * (sp - float(c));
    grad_bias[col] = overwrite ? d : grad_bias[col] + d;
  }
}

// In place: the fp32 logits of row i, column group g (bytes [256 g, 256 g + 256) of the row)
// become 64 bf16 probabilities in the group's first 128 bytes. Sixteen lanes of one
// wavefront own a group: each loads 4 floats (16 B) and stores 4 bf16 (8 B) at a lower
// address inside the same group; the wavefront's load completes for every lane before its
// dependent store issues, so no lane overwrites bytes another lane has yet to read.
__global__ void __launch_bounds__(256) slice_to_probs_kernel(float* z, int64_t ldz, int64_t v,
                                                             const int32_t* __restrict__ labels,
                                                             int32_t ignore_index,
                                                             const float* __restrict__ lse_c,
                                                             RowVec yc) {
  const int64_t i = blockIdx.y;
  const int64_t g = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int L = threadIdx.x & 15;
  if (g >= ldz / kGroup) return;
  const int32_t y = labels[i];
  const bool ok = has_label(y, v, ignore_index);
  float* row = z + i * ldz;
  const int64_t col = g * kGroup + 4 * L;
  const float4 x = *reinterpret_cast<const float4*>(row + col);
  const float c = ok ? lse_c[i] : 0.f;
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  if (ok) {  // exp((z − lse)): as the recomputing schedule's probabilities, bit for bit
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (col + k < v) p[k] = fast_exp2((xs[k] - c) * kLog2e);
  }
  uint2 o;
  o.x = pack_bf16x2(p[0], p[1]);
  o.y = pack_bf16x2(p[2], p[3]);
  *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(row) + g * (2 * kGroup) + 4 * L) = o;
  const int64_t d = int64_t(y) - col;
  if (ok && d >= 0 && d < 4) {  // the label column: its label coefficient
    const float q = d < 2 ? (d == 0 ? bf16_lo(o.x) : bf16_hi(o.x)) : (d == 2 ? bf16_lo(o.y) : bf16_hi(o.y));
    yc[i] = label_coef(p[int(d)], q);
  }
}

// In place over a 16-bit [rows, ldz] array of shifted logits d = fp16(z − m_t) (EpiLogits16):
// P = bf16(exp(d + (m_t − lse))), m_t = part[i · tiles + t].x for the column's 256-wide tile
// t; 0 for rows without a label and for the padding columns v .. ldz − 1. Each lane converts
// 8 consecutive elements (one 16-byte load, one 16-byte store at the same address).
__global__ void __launch_bounds__(256) shifted_to_probs_kernel(
    uint16_t* z, int64_t ldz, int64_t v, const int32_t* __restrict__ labels, int32_t ignore_index,
    const float* __restrict__ lse_c, const float2* __restrict__ part, int64_t tiles) {
  const int64_t i = blockIdx.y;
  const int64_t col = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (col >= ldz) return;
  uint16_t* p = z + i * ldz + col;
  uint4 o = {0u, 0u, 0u, 0u};
  if (has_label(labels[i], v, ignore_index) && col < v) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const float sh = part[i * tiles + (col >> 8)].x - lse_c[i];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float d = f16_to_f32(w[k >> 1] >> (16 * (k & 1)));
      r[k] = col + k < v ? fast_exp2((d + sh) * kLog2e) : 0.f;
    }
    o = uint4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
              pack_bf16x2(r[6], r[7])};
  }
  *reinterpret_cast<uint4*>(p) = o;
}

// The same conversion with the result stored in vocabulary panels, for the schedule that keeps
// every row's probabilities (flce_transposed): the probabilities of columns 64 b .. 64 b + 63
// form panel b, a token-major [ldp][64] block (Pᵀ's rows 64 b .. in 64-row blocks, each stored
// transposed); panels b < seg_panels sit at pt1 + b · ldp · 64, the others at
// pt2 + (b − seg_panels) · ldp · 64. Chunk rows c0 .. c0 + rows − 1 are tokens c0 ...; values
// are shifted_to_probs_kernel's bit for bit; tokens past the chunk's rows (the last chunk's, up
// to ldp) and the last panel's columns past v get zeros. A workgroup converts 256 columns (one
// logits tile: one m_t per token, four panels) × 64 tokens: lane i takes columns
// 8 (i % 32) .. + 7 of token 8 it + i / 32 over eight passes, so a wavefront reads 512
// contiguous bytes of each of two token rows per pass and the workgroup writes 8 KB of each
// of its panels.
__global__ void __launch_bounds__(256) shifted_to_probs_p_kernel(
    const uint16_t* __restrict__ z, int64_t ldz, int64_t rows, int64_t v,
    const int32_t* __restrict__ labels, int32_t ignore_index, const float* __restrict__ lse_c,
    const float2* __restrict__ part, int64_t tiles, uint16_t* pt1, uint16_t* pt2,
    int64_t seg_panels, int64_t ldp, int64_t c0) {
  const int64_t vt = blockIdx.x;
  const int q = threadIdx.x & 31;
  const int64_t v0 = vt * 256 + 8 * q;
  if (v0 >= round_up(v, 64)) return;  // past the last panel
  const int64_t b = v0 >> 6;
  uint16_t* panel = (b < seg_panels ? pt1 + b * ldp * 64 : pt2 + (b - seg_panels) * ldp * 64) +
                    (v0 & 63);
  const int64_t tend = round_up(rows, 64);
#pragma unroll 4
  for (int it = 0; it < 8; ++it) {
    const int64_t t = int64_t(blockIdx.y) * 64 + it * 8 + (threadIdx.x >> 5);
    if (t >= tend) break;
    uint4 o = {0u, 0u, 0u, 0u};
    if (t < rows && v0 < v && has_label(labels[t], v, ignore_index)) {
      const uint4 x = *reinterpret_cast<const uint4*>(z + t * ldz + v0);
      const float sh = part[t * tiles + vt].x - lse_c[t];
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      float r[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float d = f16_to_f32(w[k >> 1] >> (16 * (k & 1)));
        r[k] = v0 + k < v ? fast_exp2((d + sh) * kLog2e) : 0.f;
      }
      o = uint4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                pack_bf16x2(r[6], r[7])};
    }
    *reinterpret_cast<uint4*>(panel + (c0 + t) * 64) = o;
  }
}

// p from the shifted 16-bit logits d = fp16(z − m_t): exp(d + m_t − lse) in fp32 (the
// probability before its bf16 rounding); m_t is the row's maximum over the column's 256-wide
// tile t, the same for the 8 columns of one load.
struct ShiftedProb {
  const uint16_t* z;
  int64_t ldz;
  const float* lse_c;
  const float2* part;
  int64_t tiles;
  __device__ __forceinline__ void load8(int64_t i, int64_t c0, float (&p)[8]) const {
    const uint4 x = *reinterpret_cast<const uint4*>(z + i * ldz + c0);
    const float sh = part[i * tiles + (c0 >> 8)].x - lse_c[i];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 8; ++q)
      p[q] = fast_exp2((f16_to_f32(w[q >> 1] >> (16 * (q & 1))) + sh) * kLog2e);
  }
};

__global__ void __launch_bounds__(kBiasThreads) shifted_bias_grad_kernel(
    const uint16_t* __restrict__ z, int64_t ldz, int64_t rows, int64_t v,
    const int32_t* __restrict__ labels, int32_t ignore_index, const float* __restrict__ lse_c,
    const float2* __restrict__ part, int64_t tiles, float* __restrict__ grad_bias, int overwrite,
    const long long* count_dev, long long count_host, const float* gout) {
  bias_grad_columns(ShiftedProb{z, ldz, lse_c, part, tiles}, rows, v, labels, ignore_index,
                    grad_bias, overwrite, count_dev, count_host, gout);
}

// dW[y] −= coef · Σ_{i in chunk, y_i = y} h_i. The first chunk row carrying label y owns that
// dW row and adds the matching hidden rows in increasing row order.
__global__ void __launch_bounds__(256) onehot_weight_fix_kernel(
    const uint16_t* __restrict__ hidden, int64_t h, int64_t rows,
    const int32_t* __restrict__ labels, int32_t ignore_index, int64_t v, float* grad_weight,
    const long long* count_dev, long long count_host, const float* gout, RowVec ycoef) {
  const int64_t i = blockIdx.x;
  const int32_t y = labels[i];
  if (!has_label(y, v, ignore_index)) return;
  __shared__ int earlier;
  __shared__ int nmatch;
  __shared__ int match[1024];
  if (threadIdx.x == 0) earlier = 0;
  __syncthreads();
  for (int64_t j = threadIdx.x; j < i; j += 256)
    if (labels[j] == y) earlier = 1;
  __syncthreads();
  if (earlier) return;
  const float coef = flce_coef(count_dev, count_host, gout);
  // Rows j >= i with the same label, gathered in increasing order, 1024 at a time.
  for (int64_t base = i; base < rows; base += 1024) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int c = 0;
      const int64_t end = base + 1024 < rows ? base + 1024 : rows;
      for (int64_t j = base; j < end; ++j)
        if (labels[j] == y) match[c++] = int(j - base);
      nmatch = c;
    }
    __syncthreads();
    const int cnt = nmatch;
    if (cnt == 0) continue;
    for (int64_t col = threadIdx.x; col < h; col += 256) {
      float acc = 0.f;
      for (int k = 0; k < cnt; ++k)
        acc += ycoef[base + match[k]] * bf16_to_f32(hidden[(base + match[k]) * h + col]);
      grad_weight[int64_t(y) * h + col] -= coef * acc;
    }
  }
}

// The call's label count (when counted on the device) and its running loss sum.
struct FlceState {
  long long count;
  double sum;
};

// Adds one chunk's loss terms to the running fp64 sum one at a time, in row order, so the
// loss is the same sum whatever the chunk size; first = 1 starts the sum. The terms are
// staged in LDS 4096 at a time; one lane then adds them, its LDS reads issued a few vectors
// ahead of the dependent additions.
constexpr int kAccStage = 4096;
__global__ void __launch_bounds__(256) loss_accumulate_kernel(const float* __restrict__ term,
                                                              int64_t rows, FlceState* st,
                                                              int first) {
  __shared__ __attribute__((aligned(16))) float t[kAccStage];
  double acc = (first || threadIdx.x != 0) ? 0.0 : st->sum;
  for (int64_t b = 0; b < rows; b += kAccStage) {
    const int cnt = rows - b < kAccStage ? int(rows - b) : kAccStage;
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += 256) t[i] = term[b + i];
    __syncthreads();
    if (threadIdx.x == 0) {
      const float4* t4 = reinterpret_cast<const float4*>(t);
      const int n16 = cnt >> 4;
      float4 q[4] = {};
      if (n16 > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = t4[u];
      }
      for (int k = 0; k < n16; ++k) {
        float4 nx[4] = {q[0], q[1], q[2], q[3]};
        if (k + 1 < n16) {  // the next 16 terms load while these are added
#pragma unroll
          for (int u = 0; u < 4; ++u) nx[u] = t4[4 * (k + 1) + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc += double(q[u].x);
          acc += double(q[u].y);
          acc += double(q[u].z);
          acc += double(q[u].w);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = nx[u];
      }
      for (int i = n16 * 16; i < cnt; ++i) acc += double(t[i]);
    }
  }
  if (threadIdx.x == 0) st->sum = acc;
}

// loss = Σ terms / T, 0 when T = 0 or there are no rows.
__global__ void loss_finish_kernel(const FlceState* __restrict__ st, long long count_host,
                                   int64_t n, float* __restrict__ loss_out) {
  if (threadIdx.x != 0) return;
  const long long t = count_host >= 0 ? count_host : st->count;
  *loss_out = (n > 0 && t > 0) ? float(st->sum / double(t)) : 0.f;
}

__global__ void state_move_kernel(const FlceState* __restrict__ src, FlceState* __restrict__ dst) {
  if (threadIdx.x == 0) *dst = *src;
}

__global__ void fill_zero_f32(float* p, int64_t count) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

// dst[i] = src[i] for i < n (per-row values moved out of memory that is about to be written)
__global__ void copy_rows_kernel(RowVec src, RowVec dst, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t lse_tiles(int64_t v) { return (v + Wide::BN - 1) / Wide::BN; }
int64_t row_tiles(int64_t c) { return (c + Wide::BM - 1) / Wide::BM; }

// Free-half elements kept at the end of the slice in the compact layout: the chunk's lse
// (recomputing schedule), its label coefficients, then, in the last 32, the call's FlceState.
int64_t reserved_gap(int64_t c) { return 2 * round_up(c, 32) + 32; }

// Compact layout: the workspace is the fp32 slice [C, ldz] and nothing else. What the call
// keeps beside the logits lives in memory it owns anyway:
// - stored-slice schedule: each chunk's tile pairs, lse and loss terms in the chunk's own
//   grad_hidden rows, which only the chunk's grad_hidden product writes, later; the
//   FlceState in the last 16 bytes of grad_hidden, moved into the slice's reserved free
//   halves before the last chunk's rows are written;
// - recomputing schedule: its first pass never stores logits, so the tile pairs, label
//   logits and loss terms sit at the start of the slice, the lse and the FlceState in the
//   reserved free halves, clear of the probabilities and the column sums;
// - per chunk, the labels sorted for the one-hot term at the start of the slice, once the
//   probabilities are consumed.
// It needs the pipelined GEMM's hooks (h a multiple of 64) and a chunk of 64 rows or more.
// The free halves before the reserved ones take the column sums (row_tiles · v of them) and
// the grad_hidden split partials; the first pass's scratch must end before them too.
bool compact_layout(int64_t h, int64_t v, int64_t c) {
  if (h % Wide::BK != 0 || c < 64) return false;
  const int64_t usable = c * round_up(v, kGroup) / 2 - reserved_gap(c);
  return row_tiles(c) * v <= usable && c * (lse_tiles(v) + 1) <= usable;
}

struct FlceWs {
  float* slice;  // [C, ldz] fp32
  int64_t ldz, tiles;
  bool compact;
  // extended layout only: bookkeeping beside the slice
  FlceState* state;
  float* lse_c;   // [C]
  float2* part;   // [C, tiles] per-tile (max, Σ exp) of the logits rows
  float* zy;      // [C] label logits (recomputing schedule)
  float* term;    // [C] loss terms
};

FlceWs flce_carve(void* base, int64_t h, int64_t v, int64_t c) {
  char* b = static_cast<char*>(base);
  FlceWs w{};
  w.ldz = round_up(v, kGroup);
  w.tiles = lse_tiles(v);
  w.compact = compact_layout(h, v, c);
  if (w.compact) {
    w.slice = reinterpret_cast<float*>(b);
    return w;
  }
  w.state = reinterpret_cast<FlceState*>(b);
  size_t off = 256;
  w.lse_c = reinterpret_cast<float*>(b + off);
  off += align256(size_t(c) * 4);
  w.part = reinterpret_cast<float2*>(b + off);
  off += align256(size_t(c) * size_t(w.tiles) * 8);
  w.zy = reinterpret_cast<float*>(b + off);
  off += align256(size_t(c) * 4);
  w.term = reinterpret_cast<float*>(b + off);
  off += align256(size_t(c) * 4);
  w.slice = reinterpret_cast<float*>(b + off);
  return w;
}

// Two chunks per slice in the compact layout. Each half of the slice is a [C, ldz] 16-bit
// array that ends up holding one chunk's bf16 probabilities:
//   stored logits (kPairStored): the logits GEMM writes the chunk's logits as 16-bit shifted
//     values (EpiLogits16), then lse and loss terms, grad_bias, and the conversion in place;
//   recomputing (kPairRecompute): a first GEMM pass reduces the logits to lse and loss terms
//     (EpiLseOnly), a second writes the probabilities (EpiProbs, dense);
//   backward only (kPairBwdOnly): the second pass alone, from the caller's lse.
// Chunk A (half 0) and the chunk after it, B (half 1), then share one grad_weight product
// over K = rows_A + rows_B (their probability rows are contiguous), so the fp32 accumulator
// is read and written once per two chunks. Per pair:
//   A: probabilities into half 0 → grad_hidden, its split partials in half 1
//   B: probabilities into half 1
//   grad_weight over A ∪ B; its one-hot term over A ∪ B (sorted labels at the start of half 0)
//   B: grad_hidden, its split partials in half 0
// A chunk's tile pairs, lse and label logits / loss terms sit in its own grad_hidden rows
// until its grad_hidden product overwrites them. The call state starts in the last 16 bytes
// of grad_hidden (`st`) and moves, just before the last chunk's grad_hidden product, to the
// end of the half that takes that product's partials; the partials stop short of it.
enum PairMode { kPairStored, kPairRecompute, kPairBwdOnly };

hipError_t flce_paired(const FlceArgs& a, const FlceWs& ws, int64_t chunk, FlceState* st,
                       PairMode mode, hipStream_t s) {
  const int64_t n = a.n, h = a.h, v = a.v;
  const long long th = a.num_label_tokens >= 0 ? a.num_label_tokens : -1;
  const bool accumulate = (a.flags & FLCE_ACCUMULATE) != 0;
  uint16_t* const half[2] = {reinterpret_cast<uint16_t*>(ws.slice),
                             reinterpret_cast<uint16_t*>(ws.slice) + chunk * ws.ldz};
  const int64_t half_bytes = chunk * ws.ldz * 2;
  constexpr int64_t kStateReserve = 256;  // end of a half kept for the moved call state
  // before it, the label coefficients of the chunk whose grad_hidden runs from that half
  const int64_t coef_off = half_bytes / 4 - kStateReserve / 4 - round_up(chunk, 64);
  hipError_t e;

  const RowVec none{nullptr, 0, 0};
  // the probabilities of rows [c0, c0 + rows) into half hf (with lse, loss terms and
  // grad_bias on the way, as the mode has them), the rows' label coefficients into yc (and
  // yc2 when given)
  auto front = [&](int64_t c0, int64_t rows, int hf, bool first, RowVec yc,
                   RowVec yc2) -> hipError_t {
    const int32_t* lab = a.labels + c0;
    float* scr = reinterpret_cast<float*>(a.grad_hidden + c0 * h);
    float2* part = reinterpret_cast<float2*>(scr);
    float* lse_c = scr + 2 * rows * ws.tiles;
    float* term = lse_c + rows;  // first the label logits, then the loss terms
    View Ah{a.hidden + c0 * h, h, kGroup, rows, h};
    View Bw{a.weight, h, kGroup, v, h};
    if (mode != kPairStored) {
      if (mode == kPairRecompute) {
        EpiLseOnly e1{a.bias, part, ws.tiles, lab, term};
        {
          TimedLaunch t(s, K_FLCE_GEMM_LOGITS);
          hipError_t r = gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, v, h, 1, true, e1, s);
          if (r != hipSuccess) return r;
        }
        {
          TimedLaunch t(s, K_FLCE_ROW_LSE);
          hipLaunchKernelGGL(lse_merge_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0,
                             s, part, ws.tiles, nullptr, int64_t(0), term, rows, v, lab,
                             a.ignore_index, lse_c, int64_t(-1), term,
                             a.lse_out ? a.lse_out + c0 : nullptr, none, none);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        TimedLaunch t(s, K_FLCE_LOSS_ACC);
        hipLaunchKernelGGL(loss_accumulate_kernel, dim3(1), dim3(256), 0, s, term, rows, st,
                           int(first));
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      const float* lse = mode == kPairBwdOnly ? a.lse_in + c0 : lse_c;
      // the GEMM runs over N = ldz: weight rows past v read as zero, their columns become 0
      EpiProbs e2{half[hf], ws.ldz, kGroup, a.bias, lse, int64_t(-1), lab, v, a.ignore_index,
                  nullptr, yc, yc2};
      TimedLaunch t(s, K_FLCE_GEMM_PROBS);
      return gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, ws.ldz, h, 1, true, e2, s);
    }
    EpiLogits16 el{half[hf], ws.ldz, a.bias, part, ws.tiles, lab, term};
    {
      TimedLaunch t(s, K_FLCE_GEMM_LOGITS);
      hipError_t r = gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, v, h, 1, true, el, s);
      if (r != hipSuccess) return r;
    }
    {
      TimedLaunch t(s, K_FLCE_ROW_LSE);
      hipLaunchKernelGGL(lse_merge_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s,
                         part, ws.tiles, nullptr, int64_t(0), term, rows, v, lab,
                         a.ignore_index, lse_c, int64_t(-1), term,
                         a.lse_out ? a.lse_out + c0 : nullptr, yc, yc2);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
      TimedLaunch t(s, K_FLCE_LOSS_ACC);
      hipLaunchKernelGGL(loss_accumulate_kernel, dim3(1), dim3(256), 0, s, term, rows, st,
                         int(first));
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.grad_bias) {
      TimedLaunch t(s, K_FLCE_BIAS_GRAD);
      hipLaunchKernelGGL(shifted_bias_grad_kernel,
                         dim3(unsigned((v + kBiasBlockCols - 1) / kBiasBlockCols)),
                         dim3(kBiasThreads), 0,
                         s, half[hf], ws.ldz, rows, v, lab, a.ignore_index, lse_c, part,
                         ws.tiles, a.grad_bias, int(first && !accumulate), &st->count, th,
                         a.grad_output);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    TimedLaunch t(s, K_FLCE_TO_PROBS);
    hipLaunchKernelGGL(shifted_to_probs_kernel,
                       dim3(unsigned((ws.ldz / 8 + 255) / 256), unsigned(rows)), dim3(256), 0, s,
                       half[hf], ws.ldz, v, lab, a.ignore_index, lse_c, part, ws.tiles);
    return hipGetLastError();
  };

  // grad_hidden of rows [c0, c0 + rows), probabilities in half hf, split partials in the
  // other half, label coefficients in yc
  auto grad_hidden = [&](int64_t c0, int64_t rows, int hf, bool last, RowVec yc) -> hipError_t {
    float* other = reinterpret_cast<float*>(half[1 - hf]);
    if (last) {
      FlceState* dst = reinterpret_cast<FlceState*>(reinterpret_cast<char*>(other) + half_bytes - 16);
      TimedLaunch t(s, K_FLCE_LOSS_ACC);
      hipLaunchKernelGGL(state_move_kernel, dim3(1), dim3(64), 0, s, st, dst);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      st = dst;
    }
    const int32_t* lab = a.labels + c0;
    View Ap{half[hf], ws.ldz, kGroup, rows, v};  // P: rows = chunk rows, cols = vocab (K-major)
    View Bw2{a.weight, h, kGroup, v, h};         // W: rows = k (vocab), cols = n (hidden)
    const int64_t tiles = row_tiles(rows) * ((h + Wide::BN - 1) / Wide::BN);
    // partial element e of split z sits at float z · rows · h + e of `other`, short of the
    // label coefficients and the state reserve at its end
    const int64_t cap = coef_off / (rows * h);
    int64_t splits = 256 / tiles;
    if (splits > cap) splits = cap;
    if (splits > (v + 1023) / 1024) splits = (v + 1023) / 1024;  // keep >= 1024 of K per split
    if (splits < 1) splits = 1;
    const long long* cnt = &st->count;
    uint16_t* dh = a.grad_hidden + c0 * h;
    {
      TimedLaunch t(s, K_FLCE_GEMM_GRAD_HIDDEN);
      hipError_t r;
      if (splits == 1) {
        EpiGradHidden eh{dh, h, lab, a.weight, h, v, a.ignore_index, cnt, th, a.grad_output, 0.f,
                         yc};
        r = gemm::v2::launch<Wide, true, false>(Ap, Bw2, rows, h, v, 1, true, eh, s);
      } else {
        EpiPartial ep{other, rows, h, 0, 1};
        r = gemm::v2::launch<Wide, true, false>(Ap, Bw2, rows, h, v, splits, true, ep, s);
      }
      if (r != hipSuccess) return r;
    }
    if (splits == 1) return hipSuccess;
    TimedLaunch t(s, K_FLCE_GRAD_HIDDEN_REDUCE);
    hipLaunchKernelGGL(grad_hidden_reduce_kernel, dim3(unsigned((rows * h / 4 + 255) / 256)),
                       dim3(256), 0, s, other, 1, rows, h, splits, dh, lab, a.weight, v,
                       a.ignore_index, cnt, th, a.grad_output, yc);
    return hipGetLastError();
  };

  // grad_weight over K = rows of the pair starting at c0 (probabilities from half 0 on), then
  // its one-hot term (label coefficients of the pair's rows in yc)
  auto grad_weight = [&](int64_t c0, int64_t rows, bool first, RowVec yc) -> hipError_t {
    const int32_t* lab = a.labels + c0;
    const uint16_t* hid = a.hidden + c0 * h;
    const long long* cnt = &st->count;
    View Ap{half[0], ws.ldz, kGroup, rows, v};  // Pᵀ: rows = k (chunk rows), cols = vocab
    View Bh{hid, h, kGroup, rows, h};           // hidden rows: rows = k, cols = n
    EpiGradWeight ew{a.grad_weight, h, int(first && !accumulate), cnt, th, a.grad_output, 0.f};
    {
      TimedLaunch t(s, K_FLCE_GEMM_GRAD_WEIGHT);
      hipError_t r = launch_grad_weight(Ap, Bh, v, h, rows, ew, s);
      if (r != hipSuccess) return r;
    }
    if (rows <= kSortMax) {
      int32_t* slab = reinterpret_cast<int32_t*>(half[0]);
      int32_t* srow = slab + rows;
      {
        TimedLaunch t(s, K_FLCE_LABEL_SORT);
        hipLaunchKernelGGL(label_rank_kernel, dim3(unsigned((rows + 63) / 64)),
                           dim3(64 * kRankWaves), 0, s, lab, rows, v, a.ignore_index, slab, srow);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      TimedLaunch t(s, K_FLCE_ONEHOT_FIX);
      hipLaunchKernelGGL(onehot_segments_kernel, dim3(unsigned(rows)), dim3(256), 0, s, hid, h,
                         rows, slab, srow, v, a.grad_weight, cnt, th, a.grad_output, yc);
    } else {
      TimedLaunch t(s, K_FLCE_ONEHOT_FIX);
      hipLaunchKernelGGL(onehot_weight_fix_kernel, dim3(unsigned(rows)), dim3(256), 0, s, hid, h,
                         rows, lab, a.ignore_index, v, a.grad_weight, cnt, th, a.grad_output, yc);
    }
    return hipGetLastError();
  };

  // Label coefficients (label_coef) of a pair's rows: A's go to the end of half 1 (before its
  // state reserve; A's grad_hidden partials stop short of them) and, when the pair has a B,
  // beside B's bookkeeping in B's grad_hidden rows, where B's follow; the one-hot term of
  // grad_weight reads them there. B's are then copied to the end of half 0 (free once
  // grad_weight is done) for B's grad_hidden, which overwrites B's rows. A B whose rows
  // cannot hold the pair's coefficients beside its bookkeeping (a short last chunk) starts a
  // pair of its own.
  for (int64_t c0 = 0, ra = 0, rb = 0; c0 < n; c0 += ra + rb) {
    ra = n - c0 < chunk ? n - c0 : chunk;
    const int64_t rest = n - c0 - ra;
    rb = rest < chunk ? rest : chunk;
    float* pair_coef = nullptr;
    if (rb > 0) {
      float* scr_b = reinterpret_cast<float*>(a.grad_hidden + (c0 + ra) * h);
      const int64_t used = (2 * ws.tiles + 2) * rb;  // B's tile pairs, lse and loss terms
      if (used + ra + rb + 4 <= rb * h / 2)
        pair_coef = scr_b + used;
      else
        rb = 0;
    }
    const bool first = c0 == 0;
    const RowVec in_half1{reinterpret_cast<float*>(half[1]) + coef_off, 0, 0};
    const RowVec in_half0{reinterpret_cast<float*>(half[0]) + coef_off, 0, 0};
    const RowVec pair_a{pair_coef, 0, 0};
    if ((e = front(c0, ra, 0, first, in_half1, pair_coef ? pair_a : none)) != hipSuccess)
      return e;
    if ((e = grad_hidden(c0, ra, 0, c0 + ra >= n, in_half1)) != hipSuccess) return e;
    if (rb > 0 && (e = front(c0 + ra, rb, 1, false, RowVec{pair_coef + ra, 0, 0}, none)) !=
                      hipSuccess)
      return e;
    if (a.grad_weight &&
        (e = grad_weight(c0, ra + rb, first, rb > 0 ? pair_a : in_half1)) != hipSuccess)
      return e;
    if (rb > 0) {
      {
        TimedLaunch t(s, K_FLCE_LOSS_ACC);
        hipLaunchKernelGGL(copy_rows_kernel, dim3(unsigned((rb + 255) / 256)), dim3(256), 0, s,
                           RowVec{pair_coef + ra, 0, 0}, in_half0, rb);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if ((e = grad_hidden(c0 + ra, rb, 1, c0 + ra + rb >= n, in_half0)) != hipSuccess) return e;
    }
  }
  if (mode == kPairBwdOnly) return hipSuccess;
  TimedLaunch t(s, K_LOSS_REDUCE);
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(64), 0, s, st, th, n, a.loss_out);
  return hipGetLastError();
}

// Every row's probabilities kept at once, transposed (stored-logits schedule, no
// FLCE_ACCUMULATE). Pᵀ [v, ldp] in bf16 takes 2 · ldp bytes per vocabulary row against
// grad_weight's 4 · h, so when the batch is no longer than about 2h it fits the bytes of the
// fp32 grad_weight the call is about to overwrite, plus the slice. Pᵀ is kept in 64-row
// panels, each a token-major [ldp][64] block (shifted_to_probs_p_kernel):
//   - grad_weight's bytes [T0, v · 4h) hold Pᵀ rows 0 .. S − 1 (T0 = v · 4h − S · 2 ldp, S a
//     multiple of 64); the slice's start holds rows S .. round_up(v, 64) − 1, followed by
//     every row's label coefficient and loss term and the call state;
//   - grad_weight's bytes [0, T0) hold one chunk's 16-bit shifted logits while the chunks are
//     formed, then grad_hidden's split partials (if any);
//   - grad_hidden is then one product over all n rows (K = v, the panels read K-major) and
//     grad_weight one product over all n rows (K = n, the panels read MN-major) per
//     vocabulary range of whole panels: a plain store, no fp32 read-modify-write. The launch
//     for rows [r_i, r_{i+1}) writes grad_weight bytes [r_i · 4h, r_{i+1} · 4h), which must
//     hold no Pᵀ row >= r_i: r_{i+1} · 4h <= T0 + r_i · 2 ldp. The rows in the slice form the
//     last range, free of that condition.
// Each chunk's tile pairs, lse and loss terms sit in its own grad_hidden rows (flce_paired's
// layout) until the single grad_hidden product writes them.
constexpr int kMaxRanges = 64;
struct TransposedPlan {
  int64_t ldp;             // Pᵀ row length: n rounded up to 64 tokens
  int64_t seg;             // S: Pᵀ rows [0, S) in grad_weight's bytes, [S, v) in the slice
  int64_t vp;              // v rounded up to whole 64-row panels
  int64_t t0;              // byte offset of Pᵀ row 0 in grad_weight
  int64_t yc_off, lt_off, st_off;  // slice byte offsets: label coefficients, loss terms, state
  int nr;                  // grad_weight launches
  int64_t r[kMaxRanges + 1];
};

bool plan_transposed(int64_t n, int64_t h, int64_t v, int64_t c, int64_t ldz, int64_t slice_bytes,
                     TransposedPlan& p) {
  if (n < 1 || c % 64 != 0 || h % Wide::BK != 0 || (c + 63) / 64 > 65535 ||
      (v + 255) / 256 > (int64_t(1) << 31) - 1)
    return false;
  p.ldp = round_up(n, 64);
  p.vp = round_up(v, 64);
  const int64_t pb = 2 * p.ldp, wb = 4 * h;
  // the slice's tail: label coefficients and loss terms (n floats each) and the state; its
  // head also takes the sorted labels of the one-hot pass (2 · kSortMax ints) once
  // grad_weight is done
  const int64_t tail = 2 * int64_t(align256(size_t(n) * 4)) + 256;
  const int64_t head_min = 2 * kSortMax * 4;
  const int64_t e_max = (slice_bytes - tail - 256) / pb;  // Pᵀ rows the slice can take
  if (e_max < 1) return false;
  const int64_t scratch = c * ldz * 2;                       // one chunk's 16-bit logits
  if (v * wb - scratch < 0) return false;
  const int64_t s_hi = std::min(v, (v * wb - scratch) / pb);  // T0 >= scratch
  const int64_t s_lo = std::max<int64_t>(0, p.vp - e_max);
  // one 256 x 256 workgroup per CU: q m-tiles fill the 256 CUs once
  const int64_t nt = (h + Wide::BN - 1) / Wide::BN;
  const int64_t q = 256 % nt == 0 ? 256 / nt : 1;
  int64_t S = round_up(s_lo, q * 256);
  if (S > s_hi) S = round_up(s_lo, 256);
  if (S > s_hi) S = round_up(s_lo, 64);
  if (S > s_hi) return false;  // (s_hi <= v, so S <= v and S is a multiple of 64)
  p.seg = S;
  p.t0 = v * wb - S * pb;
  p.yc_off = std::max<int64_t>(int64_t(align256(size_t((p.vp - S) * pb))), head_min);
  p.lt_off = p.yc_off + int64_t(align256(size_t(n) * 4));
  p.st_off = p.lt_off + int64_t(align256(size_t(n) * 4));
  if (p.st_off + 256 > slice_bytes) return false;
  // grad_weight ranges over the rows in grad_weight's bytes, then the slice's rows
  p.nr = 0;
  p.r[0] = 0;
  int64_t r = 0;
  while (r < S) {
    const int64_t lim = std::min(S, (p.t0 + r * pb) / wb);  // rows writable from r on
    int64_t nx = lim;
    if (nx < S) {  // keep ranges whole waves of tiles, else whole tiles, else whole panels
      if (nx - r >= q * 256)
        nx = r + (nx - r) / (q * 256) * (q * 256);
      else if (nx - r >= 256)
        nx = r + (nx - r) / 256 * 256;
      else
        nx = r + (nx - r) / 64 * 64;
    }
    if (nx <= r || p.nr >= kMaxRanges) return false;
    p.r[++p.nr] = nx;
    r = nx;
  }
  if (S < v) {
    if (p.nr >= kMaxRanges) return false;
    p.r[++p.nr] = v;
  }
  return true;
}

hipError_t flce_transposed(const FlceArgs& a, const FlceWs& ws, int64_t chunk,
                           const TransposedPlan& pl, hipStream_t s) {
  const int64_t n = a.n, h = a.h, v = a.v, S = pl.seg;
  const long long th = a.num_label_tokens >= 0 ? a.num_label_tokens : -1;
  char* const sl = reinterpret_cast<char*>(ws.slice);
  char* const gwb = reinterpret_cast<char*>(a.grad_weight);
  uint16_t* const z16 = reinterpret_cast<uint16_t*>(gwb);         // one chunk's 16-bit logits
  uint16_t* const pt1 = reinterpret_cast<uint16_t*>(gwb + pl.t0);  // Pᵀ panels of rows [0, S)
  uint16_t* const pt2 = reinterpret_cast<uint16_t*>(sl);           // ... of rows [S, v)
  const int64_t pg = pl.ldp * 64;                                   // elements per panel
  float* const ycall = reinterpret_cast<float*>(sl + pl.yc_off);  // label coefficients [n]
  float* const lterm = reinterpret_cast<float*>(sl + pl.lt_off);  // loss terms [n]
  FlceState* const st = reinterpret_cast<FlceState*>(sl + pl.st_off);
  const long long* cnt = &st->count;
  const RowVec none{nullptr, 0, 0};
  hipError_t e;

  if ((e = launch_label_prep(a.labels, n, v, a.ignore_index, &st->count, a.status_out, s)) !=
      hipSuccess)
    return e;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int64_t rows = n - c0 < chunk ? n - c0 : chunk;
    const bool first = c0 == 0;
    const int32_t* lab = a.labels + c0;
    float* scr = reinterpret_cast<float*>(a.grad_hidden + c0 * h);
    float2* part = reinterpret_cast<float2*>(scr);
    float* lse_c = scr + 2 * rows * ws.tiles;
    float* zy = lse_c + rows;  // the label logits
    View Ah{a.hidden + c0 * h, h, kGroup, rows, h};
    View Bw{a.weight, h, kGroup, v, h};
    EpiLogits16 el{z16, ws.ldz, a.bias, part, ws.tiles, lab, zy};
    {
      TimedLaunch t(s, K_FLCE_GEMM_LOGITS);
      if ((e = gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, v, h, 1, true, el, s)) !=
          hipSuccess)
        return e;
    }
    {
      TimedLaunch t(s, K_FLCE_ROW_LSE);
      hipLaunchKernelGGL(lse_merge_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s,
                         part, ws.tiles, nullptr, int64_t(0), zy, rows, v, lab, a.ignore_index,
                         lse_c, int64_t(-1), lterm + c0, a.lse_out ? a.lse_out + c0 : nullptr,
                         RowVec{ycall + c0, 0, 0}, none);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.grad_bias) {
      TimedLaunch t(s, K_FLCE_BIAS_GRAD);
      hipLaunchKernelGGL(shifted_bias_grad_kernel,
                         dim3(unsigned((v + kBiasBlockCols - 1) / kBiasBlockCols)),
                         dim3(kBiasThreads), 0, s, z16, ws.ldz, rows, v, lab, a.ignore_index,
                         lse_c, part, ws.tiles, a.grad_bias, int(first), cnt, th, a.grad_output);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    TimedLaunch t(s, K_FLCE_PROBS_TRANSPOSED);
    hipLaunchKernelGGL(shifted_to_probs_p_kernel,
                       dim3(unsigned((v + 255) / 256), unsigned((rows + 63) / 64)), dim3(256), 0,
                       s, z16, ws.ldz, rows, v, lab, a.ignore_index, lse_c, part, ws.tiles, pt1,
                       pt2, S / 64, pl.ldp, c0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // the loss terms of all rows added in row order, in one pass
  {
    TimedLaunch t(s, K_FLCE_LOSS_ACC);
    hipLaunchKernelGGL(loss_accumulate_kernel, dim3(1), dim3(256), 0, s, lterm, n, st, 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // grad_hidden = g·s·(P · W − c·W[y]) over all rows, K = v (the panels read K-major: rows
  // = tokens, 64 columns per panel, the panels in two segments); split over K only when the
  // row tiles alone do not fill the chip, the partials then in grad_weight's bytes below Pᵀ.
  // (Leaving fp32 P · W there and applying the one-hot term in the streaming reduce pass
  // measured no faster than the epilogue.)
  {
    const bool two = S > 0 && S < v;
    View Ap{S > 0 ? pt1 : pt2, 64, pg, n, v};
    Ap.ext = (S > 0 ? S : pl.vp) * pl.ldp;
    if (two) {
      Ap.p2 = pt2;
      Ap.kseg = S;
      Ap.ext2 = (pl.vp - S) * pl.ldp;
    }
    View Bw2{a.weight, h, kGroup, v, h};
    const int64_t tiles = row_tiles(n) * ((h + Wide::BN - 1) / Wide::BN);
    const int64_t room = pl.t0 / (8 * n * h);  // partial sets that fit below Pᵀ
    int64_t splits = 256 / tiles;
    if (splits > (v + 2047) / 2048) splits = (v + 2047) / 2048;
    if (splits > room) splits = room;
    if (splits < 1) splits = 1;
    const bool partials = splits > 1;
    float* part = reinterpret_cast<float*>(gwb);
    const RowVec yc{ycall, 0, 0};
    {
      TimedLaunch t(s, K_FLCE_GEMM_GRAD_HIDDEN);
      if (!partials) {
        EpiGradHidden eh{a.grad_hidden, h, a.labels, a.weight, h, v, a.ignore_index, cnt, th,
                         a.grad_output, 0.f, yc};
        e = two ? gemm::v2::launch<Wide, true, false, EpiGradHidden, true>(Ap, Bw2, n, h, v, 1,
                                                                            true, eh, s, true)
                : gemm::v2::launch<Wide, true, false>(Ap, Bw2, n, h, v, 1, true, eh, s, true);
      } else {
        EpiPartial ep{part, n, h, 0, 0};
        e = two ? gemm::v2::launch<Wide, true, false, EpiPartial, true>(Ap, Bw2, n, h, v,
                                                                         splits, true, ep, s)
                : gemm::v2::launch<Wide, true, false>(Ap, Bw2, n, h, v, splits, true, ep, s);
      }
      if (e != hipSuccess) return e;
    }
    if (partials) {
      TimedLaunch t(s, K_FLCE_GRAD_HIDDEN_REDUCE);
      hipLaunchKernelGGL(grad_hidden_reduce_kernel, dim3(unsigned((n * h / 4 + 255) / 256)),
                         dim3(256), 0, s, part, 0, n, h, splits, a.grad_hidden, a.labels, a.weight,
                         v, a.ignore_index, cnt, th, a.grad_output, yc);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }

  // grad_weight = g·s·Pᵀ · hidden over all rows (K = n), one launch per vocabulary range of
  // whole panels (read MN-major: k rows = tokens, 64 vocabulary columns per panel)
  View Bh{a.hidden, h, kGroup, n, h};
  for (int i = 0; i < pl.nr; ++i) {
    const int64_t r0 = pl.r[i], r1 = pl.r[i + 1];
    const uint16_t* base = r0 < S ? pt1 + r0 * pl.ldp : pt2 + (r0 - S) * pl.ldp;
    View Ap{base, 64, pg, n, r1 - r0};
    Ap.ext = ((r0 < S ? S : pl.vp) - r0) * pl.ldp;
    EpiGradWeight ew{a.grad_weight + r0 * h, h, 1, cnt, th, a.grad_output, 0.f};
    TimedLaunch t(s, K_FLCE_GEMM_GRAD_WEIGHT);
    if ((e = gemm::v2::launch<Wide, false, false>(Ap, Bh, r1 - r0, h, n, 1, true, ew, s, true)) !=
        hipSuccess)
      return e;
  }

  // one-hot term of grad_weight, kSortMax rows at a time: labels sorted into runs at the
  // slice's start (free once grad_weight is formed), one pass over the runs
  int32_t* slab = reinterpret_cast<int32_t*>(sl);
  int32_t* srow = slab + kSortMax;
  for (int64_t g0 = 0; g0 < n; g0 += kSortMax) {
    const int64_t rows = n - g0 < kSortMax ? n - g0 : kSortMax;
    {
      TimedLaunch t(s, K_FLCE_LABEL_SORT);
      hipLaunchKernelGGL(label_rank_kernel, dim3(unsigned((rows + 63) / 64)),
                         dim3(64 * kRankWaves), 0, s, a.labels + g0, rows, v, a.ignore_index,
                         slab, srow);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    TimedLaunch t(s, K_FLCE_ONEHOT_FIX);
    hipLaunchKernelGGL(onehot_segments_kernel, dim3(unsigned(rows)), dim3(256), 0, s,
                       a.hidden + g0 * h, h, rows, slab, srow, v, a.grad_weight, cnt, th,
                       a.grad_output, RowVec{ycall + g0, 0, 0});
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  TimedLaunch t(s, K_LOSS_REDUCE);
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(64), 0, s, st, th, n, a.loss_out);
  return hipGetLastError();
}

}  // namespace

int flce_check_shape(int64_t n, int64_t h, int64_t v, int64_t chunk_size, uint32_t flags) {
  if (flags & ~(FLCE_RECOMPUTE | FLCE_ACCUMULATE)) return LCE_ERR_BAD_FLAGS;
  if (n < 0 || h < 1 || v < 1 || (h % 8) != 0) return LCE_ERR_BAD_SHAPE;
  if (n > (int64_t(1) << 31) - 1 || v > (int64_t(1) << 31) - 1) return LCE_ERR_BAD_SHAPE;
  if (h > (int64_t(1) << 20)) return LCE_ERR_BAD_SHAPE;
  if (chunk_size <= 0) return LCE_ERR_BAD_CHUNK;
  return LCE_OK;
}

size_t flce_workspace_bytes(int64_t n, int64_t h, int64_t v, int64_t chunk_size, uint32_t flags) {
  (void)flags;
  const int64_t c = chunk_size < n ? chunk_size : (n > 0 ? n : 1);
  const size_t slice = size_t(c) * size_t(round_up(v, kGroup)) * 4;
  if (compact_layout(h, v, c)) return slice;
  return 256 + 3 * align256(size_t(c) * 4) + align256(size_t(c) * size_t(lse_tiles(v)) * 8) +
         slice;
}

hipError_t flce_run(const FlceArgs& a, hipStream_t s) {
  const int64_t n = a.n, h = a.h, v = a.v;
  const int64_t chunk = a.chunk_size < n ? a.chunk_size : (n > 0 ? n : 1);
  FlceWs ws = flce_carve(a.workspace, h, v, chunk);
  const long long th = a.num_label_tokens >= 0 ? a.num_label_tokens : -1;
  const bool accumulate = (a.flags & FLCE_ACCUMULATE) != 0;
  const bool fwd_only = a.pass == kFwdOnly, bwd_only = a.pass == kBwdOnly;
  // The split exports always take the recomputing passes (the forward keeps no logits; the
  // backward rebuilds them from the saved lse). That schedule needs the pipelined GEMM's
  // epilogue hooks (h % 64 == 0); for other h the stored-slice schedule runs, with the same
  // results. In the compact layout the stored-slice schedule keeps its bookkeeping in
  // grad_hidden rows: without grad_hidden, or with fewer than 4 · ⌈v / 256⌉ + 12 hidden
  // columns to hold it, the recomputing schedule runs instead.
  const bool want_recompute = (a.flags & FLCE_RECOMPUTE) != 0 || fwd_only || bwd_only;
  const bool gh_scratch = a.grad_hidden && 2 * h >= 8 * ws.tiles + 24;
  const bool recompute =
      ws.compact ? (want_recompute || !gh_scratch) : (want_recompute && h % Wide::BK == 0);
  const int64_t usable_gap = chunk * ws.ldz / 2 - reserved_gap(chunk);  // compact layout
  FlceState* st_slice =
      ws.compact ? reinterpret_cast<FlceState*>(ws.slice + gap_index(chunk * ws.ldz / 2 - 32))
                 : ws.state;
  // two chunks per slice (flce_paired): the stored-logits schedule of the compact layout, and
  // its recomputing schedule when grad_hidden rows can take the bookkeeping and no grad_bias
  // is asked for (its column sums need the room the second chunk takes)
  const bool paired = ws.compact && (!recompute || (gh_scratch && !fwd_only && !a.grad_bias));
  // every row's probabilities kept transposed in grad_weight's bytes and the slice
  // (flce_transposed): the stored-logits schedule, when grad_weight is overwritten and the
  // batch fits
  TransposedPlan tp;
  if (paired && !recompute && !accumulate && a.grad_weight &&
      plan_transposed(n, h, v, chunk, ws.ldz, chunk * ws.ldz * 4, tp))
    return flce_transposed(a, ws, chunk, tp, s);
  FlceState* st = st_slice;  // where the state is now
  if (paired)
    st = reinterpret_cast<FlceState*>(reinterpret_cast<char*>(a.grad_hidden + n * h) - 16);
  hipError_t e;

  if ((e = launch_label_prep(a.labels, n, v, a.ignore_index, &st->count, a.status_out, s)) !=
      hipSuccess)
    return e;
  if (n == 0 && !accumulate) {
    if (a.grad_weight) {
      TimedLaunch t(s, K_FILL);
      hipLaunchKernelGGL(fill_zero_f32, dim3(1024), dim3(256), 0, s, a.grad_weight, v * h);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.grad_bias) {
      TimedLaunch t(s, K_FILL);
      hipLaunchKernelGGL(fill_zero_f32, dim3(64), dim3(256), 0, s, a.grad_bias, v);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }

  if (paired)
    return flce_paired(a, ws, chunk, st,
                       !recompute ? kPairStored : (bwd_only ? kPairBwdOnly : kPairRecompute), s);

  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int64_t rows = (n - c0) < chunk ? (n - c0) : chunk;
    const bool first = c0 == 0;
    const int32_t* lab = a.labels + c0;
    const uint16_t* hid = a.hidden + c0 * h;

    View Ah{hid, h, kGroup, rows, h};
    View Bw{a.weight, h, kGroup, v, h};
    const bool fused_lse = h % Wide::BK == 0;
    float* lo = a.lse_out ? a.lse_out + c0 : nullptr;
    // grad_bias column sums of the recomputing schedule sit in the slice's free halves: in the
    // extended layout the highest float offset they reach must stay inside the slice (fails
    // only for chunks of a row or two; those take the stored-slice schedule, same results)
    const bool recompute_chunk =
        recompute && (ws.compact || !a.grad_bias || 2 * row_tiles(rows) * v + 64 <= chunk * ws.ldz);

    // the chunk's bookkeeping (see compact_layout; the compact layout's stored-logits
    // schedule is flce_paired)
    float2* part = ws.part;
    float* lse_c = ws.lse_c;
    int64_t lse_gap = -1;
    float* zy = ws.zy;
    float* term = ws.term;
    if (ws.compact) {
      part = reinterpret_cast<float2*>(ws.slice);
      zy = ws.slice + 2 * rows * ws.tiles;
      term = zy + rows;
      lse_c = ws.slice;
      lse_gap = usable_gap;
    }
    if (bwd_only) {  // the chunk's lse is given
      lse_c = const_cast<float*>(a.lse_in + c0);
      lse_gap = -1;
    }
    // the chunk's label coefficients: beside the slice (the label-logit array, free once the
    // loss terms are formed), or in the compact layout's reserved free halves after the lse
    const RowVec none{nullptr, 0, 0};
    const RowVec yc = ws.compact ? RowVec{ws.slice, usable_gap + round_up(chunk, 32), 2}
                                 : RowVec{ws.zy, 0, 0};

    if (!recompute_chunk) {
      // 1. logits slice (the pipelined GEMM also leaves per-tile logsumexp pairs; the
      //    register-staged one, used when h is not a multiple of 64, does not)
      EpiLogits el{ws.slice, ws.ldz, a.bias, part, ws.tiles};
      {
        TimedLaunch t(s, K_FLCE_GEMM_LOGITS);
        e = fused_lse ? gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, v, h, 1, true, el, s)
                      : gemm::launch<true, true>(Ah, Bw, rows, v, h, 1, true, el, s);
        if (e != hipSuccess) return e;
      }

      // 2. row logsumexp and loss terms (the backward-only pass has the lse already)
      if (!bwd_only) {
        {
          TimedLaunch t(s, K_FLCE_ROW_LSE);
          if (fused_lse)
            hipLaunchKernelGGL(lse_merge_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256),
                               0, s, part, ws.tiles, ws.slice, ws.ldz, nullptr, rows, v, lab,
                               a.ignore_index, lse_c, int64_t(-1), term, lo, none, none);
          else
            hipLaunchKernelGGL(slice_row_lse_kernel, dim3(unsigned(rows)), dim3(kRowThreads), 0,
                               s, ws.slice, ws.ldz, v, lab, a.ignore_index, lse_c, term, lo);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        TimedLaunch t(s, K_FLCE_LOSS_ACC);
        hipLaunchKernelGGL(loss_accumulate_kernel, dim3(1), dim3(256), 0, s, term, rows, st,
                           int(first));
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }

      // 3. bias gradient from the fp32 logits
      if (a.grad_bias) {
        TimedLaunch t(s, K_FLCE_BIAS_GRAD);
        hipLaunchKernelGGL(slice_bias_grad_kernel,
                           dim3(unsigned((v + kBiasBlockCols - 1) / kBiasBlockCols)),
                           dim3(kBiasThreads), 0,
                           s, ws.slice, ws.ldz, rows, v, lab, a.ignore_index, lse_c,
                           a.grad_bias, int(first && !accumulate), &st->count, th, a.grad_output);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if (!a.grad_hidden && !a.grad_weight) continue;

      // 4. probabilities in place
      const int64_t groups = ws.ldz / kGroup;
      {
        TimedLaunch t(s, K_FLCE_TO_PROBS);
        hipLaunchKernelGGL(slice_to_probs_kernel,
                           dim3(unsigned((groups + 15) / 16), unsigned(rows)), dim3(256), 0, s,
                           ws.slice, ws.ldz, v, lab, a.ignore_index, lse_c, yc);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    } else {
      if (!bwd_only) {
        // 1'. pass 1: the logits are reduced to per-tile logsumexp pairs and the label logit,
        //     never stored
        EpiLseOnly e1{a.bias, part, ws.tiles, lab, zy};
        {
          TimedLaunch t(s, K_FLCE_GEMM_LOGITS);
          if ((e = gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, v, h, 1, true, e1, s)) !=
              hipSuccess)
            return e;
        }
        // 2'. row logsumexp and loss terms
        {
          TimedLaunch t(s, K_FLCE_ROW_LSE);
          hipLaunchKernelGGL(lse_merge_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0,
                             s, part, ws.tiles, nullptr, 0, zy, rows, v, lab, a.ignore_index,
                             lse_c, lse_gap, term, lo, none, none);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        TimedLaunch t(s, K_FLCE_LOSS_ACC);
        hipLaunchKernelGGL(loss_accumulate_kernel, dim3(1), dim3(256), 0, s, term, rows, st,
                           int(first));
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if (!a.grad_hidden && !a.grad_weight && !a.grad_bias) continue;
      // 3'. pass 2: the logits are recomputed tile by tile and leave as bf16 probabilities in
      //     the slice (and, for grad_bias, as fp32 column sums)
      EpiProbs e2{reinterpret_cast<uint16_t*>(ws.slice), 2 * ws.ldz, 2 * kGroup, a.bias, lse_c,
                  lse_gap, lab, v, a.ignore_index, a.grad_bias ? ws.slice : nullptr, yc, none};
      {
        TimedLaunch t(s, K_FLCE_GEMM_PROBS);
        if ((e = gemm::v2::launch<Wide, true, true>(Ah, Bw, rows, ws.ldz, h, 1, true, e2, s)) !=
            hipSuccess)
          return e;
      }
      if (a.grad_bias) {
        TimedLaunch t(s, K_FLCE_BIAS_GRAD);
        hipLaunchKernelGGL(bias_from_colsums_kernel,
                           dim3(unsigned((v + kBiasCols - 1) / kBiasCols)), dim3(64 * kBiasWaves), 0,
                           s, ws.slice, row_tiles(rows), rows, v, lab, a.ignore_index,
                           a.grad_bias, int(first && !accumulate), &st->count, th, a.grad_output);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if (!a.grad_hidden && !a.grad_weight) continue;
    }
    const uint16_t* P = reinterpret_cast<const uint16_t*>(ws.slice);
    const int64_t p_ld = 2 * ws.ldz, p_gs = 2 * kGroup;

    // 5.-7. gradients. grad_hidden splits K = V so that its few [rows, h] output tiles still
    // fill the chip; its fp32 partials live in the free half of every slice group (in the
    // compact layout, short of the reserved ones).
    View Ap{P, p_ld, p_gs, rows, v};         // P: rows = chunk rows, cols = vocab (K-major)
    View Bw2{a.weight, h, kGroup, v, h};      // W: rows = k (vocab), cols = n (hidden)
    View Bh{hid, h, kGroup, rows, h};         // hidden chunk: rows = k, cols = n
    const int64_t tiles = ((rows + Wide::BM - 1) / Wide::BM) * ((h + Wide::BN - 1) / Wide::BN);
    const int64_t gap_free = ws.compact ? usable_gap : rows * ws.ldz / 2;
    const int64_t gap_cap = gap_free / (rows * h);  // partial sets that fit the free halves
    int64_t splits = 256 / tiles;
    if (splits > gap_cap) splits = gap_cap;
    if (splits > (v + 2047) / 2048) splits = (v + 2047) / 2048;  // keep >= 2048 of K per split
    if (splits < 1) splits = 1;
    const long long* cnt = &st->count;
    EpiGradHidden eh{a.grad_hidden + c0 * h, h, lab, a.weight, h, v, a.ignore_index,
                     cnt, th, a.grad_output, 0.f, yc};
    EpiPartial ep{ws.slice, rows, h, 0, 0};
    EpiGradWeight ew{a.grad_weight, h, int(first && !accumulate), cnt, th, a.grad_output, 0.f};
    if (a.grad_hidden) {
      TimedLaunch t(s, K_FLCE_GEMM_GRAD_HIDDEN);
      e = splits == 1 ? gemm::v2::launch<Wide, true, false>(Ap, Bw2, rows, h, v, 1, true, eh, s)
                      : gemm::v2::launch<Wide, true, false>(Ap, Bw2, rows, h, v, splits, true, ep, s);
      if (e != hipSuccess) return e;
    }
    if (a.grad_weight) {
      TimedLaunch t(s, K_FLCE_GEMM_GRAD_WEIGHT);
      if ((e = launch_grad_weight(Ap, Bh, v, h, rows, ew, s)) != hipSuccess) return e;
    }
    if (a.grad_hidden && splits > 1) {
      TimedLaunch t(s, K_FLCE_GRAD_HIDDEN_REDUCE);
      hipLaunchKernelGGL(grad_hidden_reduce_kernel, dim3(unsigned((rows * h / 4 + 255) / 256)),
                         dim3(256), 0, s, ws.slice, 0, rows, h, splits, a.grad_hidden + c0 * h, lab,
                         a.weight, v, a.ignore_index, cnt, th, a.grad_output, yc);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.grad_weight) {
      // one-hot term of dW: the chunk's labels sorted into runs at the start of the slice
      // (free once both products have read the probabilities), one pass over the runs; chunks
      // longer than kSortMax take the per-row pass that finds each label's first row
      if (rows <= kSortMax) {
        int32_t* slab = reinterpret_cast<int32_t*>(ws.slice);
        int32_t* srow = slab + rows;
        {
          TimedLaunch t(s, K_FLCE_LABEL_SORT);
          hipLaunchKernelGGL(label_rank_kernel, dim3(unsigned((rows + 63) / 64)),
                             dim3(64 * kRankWaves), 0, s, lab, rows, v, a.ignore_index, slab,
                             srow);
          if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        TimedLaunch t(s, K_FLCE_ONEHOT_FIX);
        hipLaunchKernelGGL(onehot_segments_kernel, dim3(unsigned(rows)), dim3(256), 0, s, hid, h,
                           rows, slab, srow, v, a.grad_weight, cnt, th, a.grad_output, yc);
      } else {
        TimedLaunch t(s, K_FLCE_ONEHOT_FIX);
        hipLaunchKernelGGL(onehot_weight_fix_kernel, dim3(unsigned(rows)), dim3(256), 0, s, hid,
                           h, rows, lab, a.ignore_index, v, a.grad_weight, cnt, th,
                           a.grad_output, yc);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (bwd_only) return hipSuccess;
  TimedLaunch t(s, K_LOSS_REDUCE);
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(64), 0, s, st, th, n, a.loss_out);
  return hipGetLastError();
}

}  // namespace lce
