// Label-restricted next-token distribution for single-token classification
// (openjev-sglang tutorial: "how inference works", step 5; the question types;
// "interpret confidence carefully").
//
// One wave per row of logits, lane i holding option i (64 labels at most, one
// per lane).  Each lane gathers its label's logit, and wave-wide butterfly
// reductions give the maximum, the softmax denominator, the expected index and
// the entropy.  The entropy is taken as
//   H = -sum p_i log p_i = log(S) + sum p_i (m - x_i),   S = sum exp(x_i - m),
// two sums of non-negative terms: no logarithm per lane and no cancellation.
// The work is a gather of at most 64 values per row: latency, not bandwidth,
// bounds it, so four rows share a 256-thread workgroup.
#include <cmath>

#include "hip_common.h"

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void label_dist_kernel(const void* __restrict__ logits, int64_t stride,
                                                         int64_t vocab, int32_t n_rows,
                                                         const int32_t* __restrict__ label_ids, int32_t n_labels,
                                                         const int32_t* __restrict__ counts,
                                                         float* __restrict__ probs, int32_t* __restrict__ choice,
                                                         float* __restrict__ expected,
                                                         float* __restrict__ confidence, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // whole waves leave together
  int32_t k = n_labels;
  if (counts) {
    k = counts[row];
    if (k < 1 || k > n_labels) {
      if (err && lane == 0) atomicOr(err, RC_DEVERR_LABEL);
      k = k < 1 ? 1 : n_labels;
    }
  }
  const bool on = lane < k;
  float x = -INFINITY;
  if (on) {
    const int32_t id = label_ids[lane];
    if (id >= 0 && (int64_t)id < vocab) {
      const int64_t at = row * stride + id;
      if (BF16) {
        const uint32_t b = ((const uint16_t*)logits)[at];
        x = __uint_as_float(b << 16);
      } else {
        x = ((const float*)logits)[at];
      }
    } else if (err) {
      atomicOr(err, RC_DEVERR_LABEL);
    }
  }
  const float m = wave_max(x);
  // the most probable option: the lowest lane holding the maximum logit
  const uint64_t top = __ballot(on && x == m);
  const float e = on ? expf(x - m) : 0.f;
  const float s = wave_sum(e);
  const float p = e / s;
  const float ex = wave_sum(on ? (float)lane * p : 0.f);
  const float tail = wave_sum(p > 0.f ? p * (m - x) : 0.f);
  if (lane < n_labels) probs[row * n_labels + lane] = on ? p : 0.f;
  if (lane == 0) {
    if (choice) choice[row] = top ? (int32_t)__builtin_ctzll(top) : 0;
    if (expected) expected[row] = ex;
    if (confidence) confidence[row] = k > 1 ? 1.f - (logf(s) + tail) / logf((float)k) : 1.f;
  }
}

}  // namespace

extern "C" rc_status rc_label_distribution(const void* logits, int32_t dtype, int64_t row_stride, int64_t vocab,
                                           int32_t n_rows, const int32_t* label_ids, int32_t n_labels,
                                           const int32_t* counts, float* probs, int32_t* choice, float* expected,
                                           float* confidence, void* stream) {
  using namespace rc;
  if (dtype != RC_F32 && dtype != RC_BF16) return fail(RC_ERR_DTYPE, "logits dtype %d is neither RC_F32 nor RC_BF16", dtype);
  if (n_rows < 0) return fail(RC_ERR_ARG, "n_rows = %d is negative", n_rows);
  if (n_labels < 1 || n_labels > 64) return fail(RC_ERR_RANGE, "n_labels = %d outside [1, 64]", n_labels);
  if (vocab < 1 || row_stride < vocab)
    return fail(RC_ERR_SHAPE, "vocab %lld and row stride %lld: need 1 <= vocab <= stride", (long long)vocab,
                (long long)row_stride);
  if (n_rows == 0) return RC_OK;
  if (!logits || !label_ids || !probs) return fail(RC_ERR_ARG, "NULL device pointer in rc_label_distribution");
  const unsigned blocks = (unsigned)((n_rows + 3) / 4);
  hipStream_t s = (hipStream_t)stream;
  {
    ProfScope p("label_distribution", s);
    if (dtype == RC_BF16)
      hipLaunchKernelGGL(label_dist_kernel<true>, dim3(blocks), dim3(256), 0, s, logits, row_stride, vocab, n_rows,
                         label_ids, n_labels, counts, probs, choice, expected, confidence, error_word());
    else
      hipLaunchKernelGGL(label_dist_kernel<false>, dim3(blocks), dim3(256), 0, s, logits, row_stride, vocab, n_rows,
                         label_ids, n_labels, counts, probs, choice, expected, confidence, error_word());
  }
  return check_launch("label_distribution");
}
