// Error plumbing and shape validation for the C ABI.
#include <cstdio>
#include <string>

#include "rc_internal.h"

namespace rc {

static thread_local std::string t_err;

rc_status fail(rc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_err = buf;
  return st;
}

void clear_error() { t_err.clear(); }

rc_status check_shape(const rc_shape* s) {
  if (!s) return fail(RC_ERR_ARG, "shape is NULL");
  if (s->dtype != RC_F32 && s->dtype != RC_BF16) return fail(RC_ERR_DTYPE, "dtype %d not supported", s->dtype);
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0)
    return fail(RC_ERR_SHAPE, "head counts must be positive (Hq=%d Hkv=%d)", s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads)
    return fail(RC_ERR_SHAPE, "Hq=%d not a multiple of Hkv=%d", s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads / s->num_kv_heads > 128)
    return fail(RC_ERR_SHAPE, "group size %d above 128", s->num_q_heads / s->num_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128) return fail(RC_ERR_SHAPE, "head_dim %d not in {64,128}", s->head_dim);
  if (s->pool_slots < 0 || s->pool_slots > INT32_MAX) return fail(RC_ERR_SHAPE, "pool_slots %lld out of range", (long long)s->pool_slots);
  if (s->page_size < 0 || s->page_size > 1024 || (s->page_size & (s->page_size - 1)))
    return fail(RC_ERR_SHAPE, "page_size %d is not 0, 1 or a power of two up to 1024", s->page_size);
  if (s->page_size > 1 && s->pool_slots % s->page_size)
    return fail(RC_ERR_SHAPE, "pool_slots %lld is not a multiple of page_size %d", (long long)s->pool_slots, s->page_size);
  return RC_OK;
}

}  // namespace rc

extern "C" const char* rc_last_error(void) { return rc::t_err.c_str(); }
extern "C" const char* rc_version(void) { return "rcattn 0.1 gfx950"; }
