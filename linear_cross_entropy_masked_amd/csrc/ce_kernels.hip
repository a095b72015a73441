// Chunked masked cross-entropy over materialised bf16 logits, for gfx950.
//
// What is computed follows NeMo Automodel PR #2996 ("feat(loss): chunked masked CE,
// packing-mask preservation, scoped MoE AC"), first and fourth commit messages: an fp32
// logsumexp per row and the label logit gathered, summed into one scalar scaled by
// 1/num_label_tokens; the backward recomputes softmax minus one-hot and may write the
// gradient over the logits storage.
//
// How it is computed here: the PR bounds the fp32 working set by processing one
// [chunk_size, V] slice at a time. These kernels go further and never build an fp32 slice
// at all: one workgroup streams one bf16 row through registers with 16-byte loads, keeps an
// online (max, sum-exp) per lane, and merges lanes with wavefront shuffles. The work is
// HBM-bound (2 bytes per element read in the forward, 2 read + 2 written in the backward),
// so the kernels are written around coalesced 16-byte accesses, several loads in flight per
// lane, and about 7 VALU operations per element (unpack, max, one FMA, exp2, add).
//
// No implicit multiply-add contraction in this file (the helpers included below too): every
// fused multiply-add is an explicit fmaf, so a value is computed by the same operations in
// every kernel that inlines the same helper, and the one-pass kernel reproduces the two
// passes bit for bit.
#pragma clang fp contract(off)
#include "common.h"

namespace lce {

namespace {

// Launch shapes (threads per row, 16-byte loads in flight per lane, cache policy), chosen by
// measurement on the [16384, 128256] logits. Every pass over a row keeps all of its loads in
// flight (the last pass predicated) instead of finishing the row one vector per lane at a time.
// The forward reads with non-temporal loads (about 14% faster than ordinary loads; a plain
// non-temporal read kernel peaks near 6.8 TB/s on this buffer) and the in-place backward uses
// non-temporal loads and stores (each row is touched once). The backward walks the rows last
// to first, so it starts on the rows the forward read last; in that order it runs about 2%
// faster after the forward. 1024 threads per row beat 256 and 512 in both passes.
#ifndef LCE_CE_FWD_THREADS
#define LCE_CE_FWD_THREADS 1024
#endif
#ifndef LCE_CE_BWD_THREADS
#define LCE_CE_BWD_THREADS 1024
#endif
#ifndef LCE_CE_BWD_UNROLL
#define LCE_CE_BWD_UNROLL 4
#endif
constexpr int kFwdThreads = LCE_CE_FWD_THREADS, kFwdUnroll = 4;
constexpr int kBwdThreads = LCE_CE_BWD_THREADS, kBwdUnroll = LCE_CE_BWD_UNROLL;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load / store, optionally non-temporal (streamed data that will not be reused).
template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return uint4{v.x, v.y, v.z, v.w};
  } else {
    return *p;
  }
}
template <bool NT>
__device__ __forceinline__ void st16(uint4* p, uint4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
  else
    *p = v;
}

// Split a row of v bf16 elements starting at p into: `head` scalar elements up to the first
// 16-byte boundary, `nvec` aligned 8-element vectors, and `tail` trailing scalars.
struct RowSplit {
  int head;
  int64_t nvec;
  int tail;
};

__device__ __forceinline__ RowSplit split_row(const void* p, int64_t v) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  int head = int(((16u - (a & 15u)) & 15u) >> 1);
  if (head > v) head = int(v);
  int64_t rest = v - head;
  return RowSplit{head, rest >> 3, int(rest & 7)};
}

__device__ __forceinline__ bool row_has_label(int32_t y, int64_t v, int32_t ignore_index) {
  return y != ignore_index && y >= 0 && int64_t(y) < v;
}

// Block-wide merge of per-lane (m, s); result broadcast to every lane.
template <int kRowThreads>
__device__ __forceinline__ void block_lse_reduce(float& m, float& s) {
  __shared__ float sm[kRowThreads / 64], ss[kRowThreads / 64];
  wave_lse_reduce(m, s);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) lse_merge(m, s, sm[w], ss[w]);
}

// Fold cnt values into a running (m, s) = (max, sum of exp(x - max)) pair; -inf values add
// nothing. The shift is taken as (x - max) · log2(e): the difference of two bf16 values is
// exact in fp32, so the maximum contributes exactly 1 (a one-column row has lse = z exactly
// and loss 0), where exp2(fma(x, log2 e, -max · log2 e)) would leave the rounding residue of
// max · log2 e.
__device__ __forceinline__ void lse_absorb(float& m, float& s, const float* x, int cnt) {
  float mx = x[0];
  for (int k = 1; k < cnt; ++k) mx = fmaxf(mx, x[k]);
  const float mn = fmaxf(m, mx);
  if (mn == -INFINITY) return;
  float acc = (m == mn) ? s : s * fast_exp2((m - mn) * kLog2e);
  for (int k = 0; k < cnt; ++k) acc += fast_exp2((x[k] - mn) * kLog2e);
  s = acc;
  m = mn;
}

// Element k (0..7) of eight packed bf16, widened to fp32.
__device__ __forceinline__ float elem8(uint4 q, int k) {
  const uint32_t w = k < 2 ? q.x : (k < 4 ? q.y : (k < 6 ? q.z : q.w));
  return (k & 1) ? bf16_hi(w) : bf16_lo(w);
}

// lse_absorb over the 8·N bf16 of q[0..N-1] in element order.
template <int N>
__device__ __forceinline__ void lse_absorb_vecs(float& m, float& s, const uint4* q) {
  float mx = elem8(q[0], 0);
#pragma unroll
  for (int v = 0; v < N; ++v)
#pragma unroll
    for (int k = (v == 0 ? 1 : 0); k < 8; ++k) mx = fmaxf(mx, elem8(q[v], k));
  const float mn = fmaxf(m, mx);
  if (mn == -INFINITY) return;
  float acc = (m == mn) ? s : s * fast_exp2((m - mn) * kLog2e);
#pragma unroll
  for (int v = 0; v < N; ++v)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += fast_exp2((elem8(q[v], k) - mn) * kLog2e);
  s = acc;
  m = mn;
}

// Eight bf16 of q unpacked to fp32 into x[0..7].
__device__ __forceinline__ void unpack8(uint4 q, float* x) {
  x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x); x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
  x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z); x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
}

// Gradient of one 8-element vector: coef · (exp(x − lse) − onehot), each rounded to bf16
// (nearest even); `off` is the label's position in the vector (none unless 0 <= off < 8).
// `others` accumulates the probabilities of the non-label elements, in element order: the
// label element is rewritten at the end of the row as −coef · (their row sum), exact where
// p_y − 1 computed in fp32 would cancel (p_y near 1).
__device__ __forceinline__ uint4 grad_vec8(uint4 q, float lse, float coef, int64_t off,
                                           float& others) {
  float x[8];
  unpack8(q, x);
  float p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = fast_exp2((x[k] - lse) * kLog2e);
#pragma unroll
  for (int k = 0; k < 8; ++k) others += (k == off) ? 0.f : p[k];
  if (off >= 0 && off < 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k == off) p[k] -= 1.f;
  }
  uint4 o;
  o.x = pack_bf16x2(coef * p[0], coef * p[1]);
  o.y = pack_bf16x2(coef * p[2], coef * p[3]);
  o.z = pack_bf16x2(coef * p[4], coef * p[5]);
  o.w = pack_bf16x2(coef * p[6], coef * p[7]);
  return o;
}

// Sum over the workgroup in a fixed order (wavefront butterflies, then the wavefronts in
// order); every lane gets the same value.
template <int kRowThreads>
__device__ __forceinline__ float block_sum(float x) {
  __shared__ float part[kRowThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = part[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) t += part[w];
  return t;
}

// The lane that wrote element y of a row split as `sp` and walked by kRowThreads lanes
// (vector j by lane j mod kRowThreads, head and tail scalars by lane = their index there).
template <int kRowThreads>
__device__ __forceinline__ int label_owner(const RowSplit& sp, int64_t y) {
  if (y < sp.head) return int(y);
  const int64_t r = y - sp.head;
  if (r >= sp.nvec * 8) return int(r - sp.nvec * 8);
  return int((r >> 3) % kRowThreads);
}

// Per-lane online logsumexp over one row. Returns the lane's (m, s) pair.
template <int kRowThreads, int kUnroll, bool NT>
__device__ __forceinline__ void row_lse_partial(const uint16_t* row, int64_t v, float& m_out,
                                                float& s_out) {
  const RowSplit sp = split_row(row, v);
  const uint4* vec = reinterpret_cast<const uint4*>(row + sp.head);
  float m = -INFINITY, s = 0.f;
  const int tid = threadIdx.x;

  auto absorb = [&](const float* x, int cnt) { lse_absorb(m, s, x, cnt); };

  // kUnroll vectors per lane per pass; lanes past the row's end read -inf (bf16 0xff80),
  // which adds nothing to the sum
  for (int64_t j = tid; j < sp.nvec; j += int64_t(kRowThreads) * kUnroll) {
    uint4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t jj = j + int64_t(u) * kRowThreads;
      q[u] = jj < sp.nvec ? ld16<NT>(&vec[jj])
                          : uint4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    }
    lse_absorb_vecs<kUnroll>(m, s, q);
  }
  if (tid < sp.head) {
    float x = bf16_to_f32(row[tid]);
    absorb(&x, 1);
  }
  if (tid < sp.tail) {
    float x = bf16_to_f32(row[sp.head + sp.nvec * 8 + tid]);
    absorb(&x, 1);
  }
  m_out = m;
  s_out = s;
}

__global__ void __launch_bounds__(1024) label_prep_kernel(const int32_t* __restrict__ labels,
                                                          int64_t n, int64_t v,
                                                          int32_t ignore_index,
                                                          long long* __restrict__ count_out,
                                                          int32_t* __restrict__ status_out) {
  __shared__ long long part[1024 / 64];
  __shared__ int bad_any[1024 / 64];
  long long cnt = 0;
  int bad = 0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int32_t y = labels[i];
    if (row_has_label(y, v, ignore_index)) ++cnt;
    else if (y != ignore_index) bad = 1;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    cnt += __shfl_xor(cnt, off, 64);
    bad |= __shfl_xor(bad, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    part[threadIdx.x >> 6] = cnt;
    bad_any[threadIdx.x >> 6] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t = 0;
    int b = 0;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) {
      t += part[w];
      b |= bad_any[w];
    }
    if (count_out) *count_out = t;
    if (status_out) *status_out = b ? 1 : 0;
  }
}

template <int kRowThreads, int kUnroll>
__global__ void __launch_bounds__(kRowThreads) ce_fwd_rows_kernel(
    const uint16_t* logits, int64_t v, int64_t ld, const int32_t* __restrict__ labels,
    int32_t ignore_index, float* __restrict__ row_loss, float* __restrict__ lse_out) {
  const int64_t i = blockIdx.x;
  const int32_t y = labels[i];
  if (!row_has_label(y, v, ignore_index)) {  // rows without a label are never read
    if (threadIdx.x == 0) {
      row_loss[i] = 0.f;
      if (lse_out) lse_out[i] = 0.f;
    }
    return;
  }
  const uint16_t* row = logits + i * ld;
  float m, s;
  row_lse_partial<kRowThreads, kUnroll, true>(row, v, m, s);
  block_lse_reduce<kRowThreads>(m, s);
  if (threadIdx.x == 0) {
    const float lse = m + fast_log2(s) * kLn2;
    row_loss[i] = lse - bf16_to_f32(row[y]);
    if (lse_out) lse_out[i] = lse;
  }
}

// Fixed-order fp64 sum of the per-row terms, times 1/T (0 when T == 0).
__global__ void __launch_bounds__(1024) loss_reduce_kernel(const float* __restrict__ row_loss,
                                                           int64_t n,
                                                           const long long* __restrict__ count_dev,
                                                           long long count_host,
                                                           float* __restrict__ loss_out) {
  __shared__ double part[1024 / 64];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) acc += double(row_loss[i]);
  acc = wave_sum_f64(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double total = 0.0;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) total += part[w];
    const long long t = count_host >= 0 ? count_host : *count_dev;
    *loss_out = t > 0 ? float(total / double(t)) : 0.f;
  }
}

template <int kRowThreads, int kUnroll>
__global__ void __launch_bounds__(kRowThreads) ce_bwd_rows_kernel(
    const uint16_t* logits, int64_t ld, uint16_t* grad, int64_t ldg, int64_t v,
    const int32_t* __restrict__ labels, int32_t ignore_index, const float* __restrict__ lse_in,
    const long long* __restrict__ count_dev, long long count_host,
    const float* __restrict__ grad_output, const float* __restrict__ grad_rows) {
  // No __restrict__ on logits/grad: in place they are the same memory, and every element is
  // read before the same lane overwrites it. grad_rows (unreduced loss): row i's upstream
  // gradient, used as its coefficient in place of g / T.
  // rows last to first: the forward's last rows are the likeliest to still be cached
  const int64_t i = int64_t(gridDim.x) - 1 - blockIdx.x;
  const int32_t y = labels[i];
  uint16_t* grow = grad + i * ldg;
  const long long t = count_host >= 0 ? count_host : *count_dev;
  const float g = grad_output ? *grad_output : 1.f;
  const RowSplit gs = split_row(grow, v);
  const int tid = threadIdx.x;

  // zero row (also the T == 0 guard of the reduced loss)
  if (!row_has_label(y, v, ignore_index) || (!grad_rows && t <= 0)) {
    uint4* gv = reinterpret_cast<uint4*>(grow + gs.head);
    const uint4 z = {0u, 0u, 0u, 0u};
    for (int64_t j = tid; j < gs.nvec; j += kRowThreads) st16<true>(&gv[j], z);
    if (tid < gs.head) grow[tid] = 0;
    if (tid < gs.tail) grow[gs.head + gs.nvec * 8 + tid] = 0;
    return;
  }
  const uint16_t* row = logits + i * ld;
  float lse;
  if (lse_in) {
    lse = lse_in[i];
  } else {
    float m, s;
    row_lse_partial<kRowThreads, kUnroll, true>(row, v, m, s);
    block_lse_reduce<kRowThreads>(m, s);
    lse = m + fast_log2(s) * kLn2;
  }
  const float coef = grad_rows ? grad_rows[i] : float(double(g) / double(t));
  float others = 0.f;  // this lane's probabilities of the non-label elements
  int owner;           // the lane that writes the label element
  // The input and output rows share their alignment when ld == ldg (always in place); the
  // vector path needs it, otherwise fall back to scalars.
  const RowSplit sp = split_row(row, v);
  auto scalar_p = [&](int64_t col, float x) {
    const float p = fast_exp2((x - lse) * kLog2e);
    if (col != y) others += p;
    return col == y ? p - 1.f : p;
  };
  if (sp.head == gs.head) {
    const uint4* xv = reinterpret_cast<const uint4*>(row + sp.head);
    uint4* gv = reinterpret_cast<uint4*>(grow + sp.head);
    const int64_t ylocal = int64_t(y) - sp.head;  // label position relative to the vector base
    auto one = [&](uint4 q, int64_t j) -> uint4 {
      return grad_vec8(q, lse, coef, ylocal - j * 8, others);
    };
    for (int64_t j = tid; j < sp.nvec; j += int64_t(kRowThreads) * kUnroll) {
      uint4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t jj = j + int64_t(u) * kRowThreads;
        if (jj < sp.nvec) q[u] = ld16<true>(&xv[jj]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t jj = j + int64_t(u) * kRowThreads;
        if (jj < sp.nvec) st16<true>(&gv[jj], one(q[u], jj));
      }
    }
    auto scalar = [&](int64_t col) {
      grow[col] = f32_to_bf16(coef * scalar_p(col, bf16_to_f32(row[col])));
    };
    if (tid < sp.head) scalar(tid);
    if (tid < sp.tail) scalar(sp.head + sp.nvec * 8 + tid);
    owner = label_owner<kRowThreads>(sp, y);
  } else {
    for (int64_t col = tid; col < v; col += kRowThreads)
      grow[col] = f32_to_bf16(coef * scalar_p(col, bf16_to_f32(row[col])));
    owner = int(int64_t(y) % kRowThreads);
  }
  // the label element again, from the other elements: p_y − 1 = −Σ_{v≠y} p_v. The lane that
  // stored it above stores it again, so this value is the one that stays.
  const float rest = block_sum<kRowThreads>(others);
  if (tid == owner) grow[y] = f32_to_bf16(coef * -rest);
}

// Forward and in-place backward in one pass: the row stays in registers (kVec 16-byte
// vectors per lane) from its logsumexp to its gradient, so a labelled row is read once and
// written once instead of read twice. Each lane folds the same vectors in the same groups of
// four as the forward kernel, so lse, the loss terms and the gradient are bitwise those of
// the two passes. Rows of more than kRowThreads · kVec vectors are not handled here (the
// launcher falls back to the two passes).
template <int kRowThreads, int kVec>
__global__ void __launch_bounds__(kRowThreads) ce_fused_rows_kernel(
    uint16_t* logits, int64_t ld, int64_t v, const int32_t* __restrict__ labels,
    int32_t ignore_index, const long long* __restrict__ count_dev, long long count_host,
    const float* __restrict__ grad_output, float* __restrict__ row_loss,
    float* __restrict__ lse_out) {
  static_assert(kVec % 4 == 0, "vectors are folded four at a time");
  const int64_t i = blockIdx.x;
  const int32_t y = labels[i];
  uint16_t* row = logits + i * ld;
  const long long t = count_host >= 0 ? count_host : *count_dev;
  const RowSplit sp = split_row(row, v);
  const int tid = threadIdx.x;
  uint4* vec = reinterpret_cast<uint4*>(row + sp.head);
  auto zero_row = [&]() {
    const uint4 z = {0u, 0u, 0u, 0u};
    for (int64_t j = tid; j < sp.nvec; j += kRowThreads) st16<true>(&vec[j], z);
    if (tid < sp.head) row[tid] = 0;
    if (tid < sp.tail) row[sp.head + sp.nvec * 8 + tid] = 0;
  };
  if (!row_has_label(y, v, ignore_index)) {  // never read; loss term and lse 0
    zero_row();
    if (tid == 0) {
      row_loss[i] = 0.f;
      if (lse_out) lse_out[i] = 0.f;
    }
    return;
  }
  // every element this workgroup writes is read before the barrier in block_lse_reduce
  uint4 q[kVec];
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int64_t jj = tid + int64_t(u) * kRowThreads;
    q[u] = jj < sp.nvec ? ld16<true>(&vec[jj])
                        : uint4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
  }
  const float xh = tid < sp.head ? bf16_to_f32(row[tid]) : -INFINITY;
  const float xt = tid < sp.tail ? bf16_to_f32(row[sp.head + sp.nvec * 8 + tid]) : -INFINITY;
  const float zy = tid == 0 ? bf16_to_f32(row[y]) : 0.f;
  float m = -INFINITY, s = 0.f;
  // one group at a time: the whole row already takes half of the registers, so the scheduler
  // is not allowed to interleave the groups (or, below, the vectors) and their temporaries
#pragma unroll
  for (int u0 = 0; u0 < kVec; u0 += 4) {
    lse_absorb_vecs<4>(m, s, q + u0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (tid < sp.head) lse_absorb(m, s, &xh, 1);
  if (tid < sp.tail) lse_absorb(m, s, &xt, 1);
  block_lse_reduce<kRowThreads>(m, s);
  const float lse = m + fast_log2(s) * kLn2;
  if (tid == 0) {
    row_loss[i] = lse - zy;
    if (lse_out) lse_out[i] = lse;
  }
  if (t <= 0) {  // T == 0: all-zero gradient
    zero_row();
    return;
  }
  const float g = grad_output ? *grad_output : 1.f;
  const float coef = float(double(g) / double(t));
  float others = 0.f;  // this lane's probabilities of the non-label elements
  const int64_t ylocal = int64_t(y) - sp.head;
  // the packed row is made opaque here so that the gradient unpacks it again instead of the
  // compiler keeping the logsumexp pass's fp32 copy of it (twice the registers) alive
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    u32x4_t w = {q[u].x, q[u].y, q[u].z, q[u].w};
    asm volatile("" : "+v"(w));
    q[u] = uint4{w.x, w.y, w.z, w.w};
  }
  // the loads' 16 addresses are not kept for the stores (32 VGPRs): the store addresses are
  // recomputed from a base the compiler cannot match to the earlier ones
  uint4* vt = vec + tid;
  asm volatile("" : "+v"(vt));
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int64_t jj = tid + int64_t(u) * kRowThreads;
    if (jj < sp.nvec)
      st16<true>(vt + int64_t(u) * kRowThreads,
                 grad_vec8(q[u], lse, coef, ylocal - jj * 8, others));
    __builtin_amdgcn_sched_barrier(0);
  }
  auto scalar = [&](int64_t col, float x) {
    const float p = fast_exp2((x - lse) * kLog2e);
    if (col != y) others += p;
    row[col] = f32_to_bf16(coef * (col == y ? p - 1.f : p));
  };
  if (tid < sp.head) scalar(tid, xh);
  if (tid < sp.tail) scalar(sp.head + sp.nvec * 8 + tid, xt);
  // the label element again, from the other elements (as in the two-pass backward)
  const float rest = block_sum<kRowThreads>(others);
  if (tid == label_owner<kRowThreads>(sp, y)) row[y] = f32_to_bf16(coef * -rest);
}

}  // namespace

size_t ce_workspace_bytes(int64_t n) {
  const size_t rows = (size_t(n) * sizeof(float) + 255) & ~size_t(255);
  return 256 + rows;
}

CeWorkspace ce_workspace_carve(void* base, int64_t n) {
  (void)n;
  char* b = static_cast<char*>(base);
  return CeWorkspace{reinterpret_cast<long long*>(b), reinterpret_cast<float*>(b + 256)};
}

hipError_t launch_label_prep(const int32_t* labels, int64_t n, int64_t v, int32_t ignore_index,
                             long long* count_out, int32_t* status_out, hipStream_t stream) {
  TimedLaunch t(stream, K_LABEL_PREP);
  hipLaunchKernelGGL(label_prep_kernel, dim3(1), dim3(1024), 0, stream, labels, n, v,
                     ignore_index, count_out, status_out);
  return hipGetLastError();
}

hipError_t launch_ce_fwd_rows(const uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                              const int32_t* labels, int32_t ignore_index, float* row_loss,
                              float* lse_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  TimedLaunch t(stream, K_CE_FWD_ROWS);
  hipLaunchKernelGGL((ce_fwd_rows_kernel<kFwdThreads, kFwdUnroll>), dim3(unsigned(n)),
                     dim3(kFwdThreads), 0, stream,
                     logits, v, ld, labels, ignore_index, row_loss, lse_out);
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const float* row_loss, int64_t n, const long long* count_dev,
                              long long count_host, float* loss_out, hipStream_t stream) {
  TimedLaunch t(stream, K_LOSS_REDUCE);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, stream, row_loss, n,
                     count_dev, count_host, loss_out);
  return hipGetLastError();
}

hipError_t launch_ce_bwd_rows(const uint16_t* logits, int64_t ld, uint16_t* grad, int64_t ldg,
                              int64_t n, int64_t v, const int32_t* labels, int32_t ignore_index,
                              const float* lse, const long long* count_dev, long long count_host,
                              const float* grad_output, const float* grad_rows,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  TimedLaunch t(stream, K_CE_BWD_ROWS);
  hipLaunchKernelGGL((ce_bwd_rows_kernel<kBwdThreads, kBwdUnroll>), dim3(unsigned(n)),
                     dim3(kBwdThreads), 0, stream,
                     logits, ld, grad, ldg, v, labels, ignore_index, lse, count_dev, count_host,
                     grad_output, grad_rows);
  return hipGetLastError();
}


bool ce_fused_fits(int64_t v) { return (v >> 3) <= int64_t(kFwdThreads) * 16; }

hipError_t launch_ce_fused_rows(uint16_t* logits, int64_t n, int64_t v, int64_t ld,
                                const int32_t* labels, int32_t ignore_index,
                                const long long* count_dev, long long count_host,
                                const float* grad_output, float* row_loss, float* lse_out,
                                hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (!ce_fused_fits(v)) return hipErrorInvalidValue;
  TimedLaunch t(stream, K_CE_FUSED_ROWS);
  const int64_t nvec_max = v >> 3;  // a row's aligned vectors never exceed v / 8
  if (nvec_max <= int64_t(kFwdThreads) * 4)
    hipLaunchKernelGGL((ce_fused_rows_kernel<kFwdThreads, 4>), dim3(unsigned(n)),
                       dim3(kFwdThreads), 0, stream, logits, ld, v, labels, ignore_index,
                       count_dev, count_host, grad_output, row_loss, lse_out);
  else if (nvec_max <= int64_t(kFwdThreads) * 8)
    hipLaunchKernelGGL((ce_fused_rows_kernel<kFwdThreads, 8>), dim3(unsigned(n)),
                       dim3(kFwdThreads), 0, stream, logits, ld, v, labels, ignore_index,
                       count_dev, count_host, grad_output, row_loss, lse_out);
  else
    hipLaunchKernelGGL((ce_fused_rows_kernel<kFwdThreads, 16>), dim3(unsigned(n)),
                       dim3(kFwdThreads), 0, stream, logits, ld, v, labels, ignore_index,
                       count_dev, count_host, grad_output, row_loss, lse_out);
  return hipGetLastError();
}

}  // namespace lce
