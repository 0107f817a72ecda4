// Extend attention: each request's new tokens attend causally, by absolute
// position, over its cached prefix in the pool and over themselves.
#include "attn_tile.h"

namespace {

// Order of extend tiles.  Workgroup p goes to XCD p % 8 (blocks are dealt to
// the XCDs in turn).  Tiles are grouped into chunks of up to CK consecutive
// tiles of one (request, kv head), which run back to back on one XCD and
// share its L2; chunks are dealt to the XCDs in turn, later tile positions
// first: under a causal mask a later tile sees more keys, so every XCD gets
// the same mix of long and short tiles and the long ones start first.
// Returns the tile's work index (bh * tiles + tile), or -1 for padding.
__device__ __forceinline__ int extend_order(int p, int n_bh, int tiles, int ck) {
  const int n_tc = (tiles + ck - 1) / ck;
  const int x = p & 7, i = p >> 3;
  const int c = (i / ck) * 8 + x;
  if (c >= n_bh * n_tc) return -1;
  const int tc = n_tc - 1 - c / n_bh, bh = c - (c / n_bh) * n_bh;
  const int t = tc * ck + i % ck;
  return t < tiles ? bh * tiles + t : -1;
}

// Extend tiles take 8 waves (256 query columns, two waves per SIMD, one
// workgroup per CU): each K/V stage loaded into LDS feeds twice the columns of
// a 4-wave tile, which halves the loads per FLOP.
constexpr int EXT_WAVES = 8;

template <int D>
__global__ __launch_bounds__(64 * EXT_WAVES, 1) void extend_attn_bf16(Args a, int n_bh, int ck) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * D];
  const int L = extend_order(blockIdx.x, n_bh, a.tiles, ck);
  if (L < 0) return;
  attn_bf16_tile<D, EXT_WAVES, false>(a, EXTEND, L, sK, sV);
}

template <int D>
__global__ __launch_bounds__(NT) void extend_attn_f32(Args a) {
  attn_f32_body<D>(a, EXTEND);
}

template <int D>
void launch_extend(const Args& a, int n_bh, bool bf16, hipStream_t s, const char* name) {
  rc::ProfScope p(name, s);
  if (bf16) {
    const int ck = a.tiles < 4 ? a.tiles : 4;
    const int64_t chunks = (int64_t)n_bh * ((a.tiles + ck - 1) / ck);
    const int64_t grid = (chunks + 7) / 8 * 8 * ck;
    hipLaunchKernelGGL(extend_attn_bf16<D>, dim3((unsigned)grid), dim3(64 * EXT_WAVES), 0, s, a, n_bh, ck);
  } else {
    hipLaunchKernelGGL(extend_attn_f32<D>, dim3(a.n_work), dim3(NT), 0, s, a);
  }
}

}  // namespace

extern "C" rc_status rc_extend_attention(const rc_shape* shape, void* o, const void* q, const void* k_new,
                                         const void* v_new, const void* k_pool, const void* v_pool,
                                         const int32_t* req_to_token, int32_t table_rows, int64_t stride,
                                         const int32_t* rows, const int32_t* prefix_lens, const int32_t* extend_lens,
                                         const int32_t* extend_start, int32_t batch, int64_t total_extend,
                                         int32_t max_extend, float sm_scale, void* stream) {
  using namespace rc;
  rc_status st = check_common(shape, sm_scale);
  if (st != RC_OK) return st;
  if (batch < 0 || total_extend < 0 || max_extend < 0 || stride <= 0 || table_rows < 0)
    return fail(RC_ERR_ARG, "negative size (batch=%d total_extend=%lld max_extend=%d) or stride <= 0", batch,
                (long long)total_extend, max_extend);
  if (batch == 0 || max_extend == 0 || total_extend == 0) return RC_OK;
  if (!o || !q || !k_new || !v_new || !k_pool || !v_pool || !req_to_token || !prefix_lens || !extend_lens ||
      !extend_start)
    return fail(RC_ERR_ARG, "NULL device pointer in rc_extend_attention");
  const int g = shape->num_q_heads / shape->num_kv_heads;
  Args a{};
  a.q = q; a.o = o; a.k_new = k_new; a.v_new = v_new; a.k_pool = k_pool; a.v_pool = v_pool;
  a.table = req_to_token; a.table_rows = table_rows; a.stride = stride; a.pool_slots = shape->pool_slots;
  a.page_shift = shape->page_size > 1 ? __builtin_ctz((unsigned)shape->page_size) : 0;
  a.Hq = shape->num_q_heads; a.Hkv = shape->num_kv_heads; a.g = g;
  a.scale_log2 = sm_scale * LOG2E;
  a.err = error_word();
  a.total_extend = total_extend;
  a.rows = rows; a.prefix_lens = prefix_lens; a.extend_lens = extend_lens; a.extend_start = extend_start;
  a.batch = batch; a.max_extend = max_extend;
  // bf16: 32 columns per wave of the MFMA tile; fp32: one column per wave
  a.tok_per_tile = shape->dtype == RC_BF16 ? 32 * EXT_WAVES / g : (g < NT / 64 ? NT / 64 / g : 1);
  a.tiles = (max_extend + a.tok_per_tile - 1) / a.tok_per_tile;
  const int64_t n_work = (int64_t)batch * a.Hkv * a.tiles;
  if (n_work > INT32_MAX / 8) return fail(RC_ERR_RANGE, "grid of %lld workgroups too large", (long long)n_work);
  a.n_work = (int32_t)n_work;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = shape->dtype == RC_BF16;
  if (shape->head_dim == 128)
    launch_extend<128>(a, batch * a.Hkv, bf16, s, bf16 ? "extend_bf16_d128" : "extend_f32_d128");
  else
    launch_extend<64>(a, batch * a.Hkv, bf16, s, bf16 ? "extend_bf16_d64" : "extend_f32_d64");
  return check_launch("extend attention");
}
