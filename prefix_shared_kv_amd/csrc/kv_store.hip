// KV-pool scatter.  "Prompt Caching" glossary, section "How prompt caching
// works": the key and value of every token are kept so later tokens (and later
// requests sharing the prefix) read them instead of recomputing.
//
// pool[slots[i], :, :] = new[i, :, :] for K and V: a bit copy of whole rows.
// A row is Hkv*D elements (>= 1 KiB for bf16, D >= 64), moved as 16-byte
// vectors, several rows per 256-thread block so every wave streams whole,
// contiguous rows.  Offsets are 64-bit: pools exceed 2^31 bytes.
#include "hip_common.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_store_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                                                      const u32x4* __restrict__ k_new,
                                                      const u32x4* __restrict__ v_new,
                                                      const int32_t* __restrict__ slots, int64_t n,
                                                      int32_t row_vecs, int32_t rows_per_block,
                                                      int64_t pool_slots, int32_t* err) {
  const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
  const int32_t span = rows_per_block * row_vecs;
  for (int32_t j = threadIdx.x; j < span; j += blockDim.x) {
    const int32_t r = j / row_vecs;
    const int32_t c = j - r * row_vecs;
    const int64_t i = row0 + r;
    if (i >= n) break;
    const int32_t s = slots[i];
    if (s < 0 || (int64_t)s >= pool_slots) {
      if (err && c == 0) atomicOr(err, RC_DEVERR_SLOT);
      continue;
    }
    const int64_t src = i * row_vecs + c;
    const int64_t dst = (int64_t)s * row_vecs + c;
    const u32x4 kv = __builtin_nontemporal_load(&k_new[src]);
    const u32x4 vv = __builtin_nontemporal_load(&v_new[src]);
    k_pool[dst] = kv;
    v_pool[dst] = vv;
  }
}

}  // namespace

extern "C" rc_status rc_kv_store(const rc_shape* shape, void* k_pool, void* v_pool, const void* k_new,
                                 const void* v_new, const int32_t* slots, int64_t n, void* stream) {
  using namespace rc;
  rc_status st = check_shape(shape);
  if (st != RC_OK) return st;
  if (n < 0) return fail(RC_ERR_ARG, "n = %lld is negative", (long long)n);
  if (n == 0) return RC_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slots) return fail(RC_ERR_ARG, "NULL device pointer in rc_kv_store");
  const int64_t row_bytes = (int64_t)shape->num_kv_heads * shape->head_dim * dtype_bytes(shape->dtype);
  if (row_bytes % 16) return fail(RC_ERR_SHAPE, "row of %lld bytes is not a multiple of 16", (long long)row_bytes);
  const int32_t row_vecs = (int32_t)(row_bytes / 16);
  const int32_t rpb = row_vecs >= 256 ? 1 : 256 / row_vecs;
  const int64_t blocks = (n + rpb - 1) / rpb;
  if (blocks > INT32_MAX) return fail(RC_ERR_RANGE, "n = %lld too large for one launch", (long long)n);
  hipStream_t s = (hipStream_t)stream;
  {
    ProfScope p("kv_store", s);
    hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (u32x4*)k_pool, (u32x4*)v_pool,
                       (const u32x4*)k_new, (const u32x4*)v_new, slots, n, row_vecs, rpb, shape->pool_slots,
                       error_word());
  }
  return check_launch("kv_store");
}
