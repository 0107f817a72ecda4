// Kernel timing with HIP events and the device error word.
#include <cstring>
#include <string>
#include <vector>

#include "hip_common.h"

namespace rc {

static int32_t* g_err_word = nullptr;
int32_t* error_word() { return g_err_word; }

namespace {
struct Rec {
  std::string name;
  hipEvent_t a, b;
};
bool g_on = false;
std::string g_tag;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t stream, bool timed) : stream_(stream) {
  if (!g_on || !timed) return;
  hipEvent_t a = get_event(), b = get_event();
  if (!a || !b) return;
  if (hipEventRecord(a, stream) != hipSuccess) return;  // not timed
  g_recs.push_back({g_tag.empty() ? std::string(name) : std::string(name) + "@" + g_tag, a, b});
  idx_ = (int)g_recs.size() - 1;
}

ProfScope::~ProfScope() {
  // a failed end record is reported by rc_prof_collect when it times the pair
  if (idx_ >= 0) (void)hipEventRecord(g_recs[idx_].b, stream_);
}

rc_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RC_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return RC_OK;
}

}  // namespace rc

extern "C" rc_status rc_set_error_word(int32_t* device_word) {
  rc::g_err_word = device_word;
  return RC_OK;
}

extern "C" rc_status rc_upload_table_rows(int32_t* dev_table, int64_t dev_stride, const int32_t* host_table,
                                          int64_t host_stride, int64_t row0, int64_t n_rows, int64_t col0,
                                          int64_t col1, void* stream) {
  if (n_rows < 0 || row0 < 0 || col0 < 0 || col1 < col0 || col1 > dev_stride || col1 > host_stride)
    return rc::fail(RC_ERR_ARG, "bad table rectangle: rows %lld+%lld, entries [%lld, %lld), strides %lld/%lld",
                    (long long)row0, (long long)n_rows, (long long)col0, (long long)col1, (long long)dev_stride,
                    (long long)host_stride);
  if (n_rows == 0 || col1 == col0) return RC_OK;
  if (!dev_table || !host_table) return rc::fail(RC_ERR_ARG, "NULL table");
  const size_t e = sizeof(int32_t);
  hipError_t st = hipMemcpy2DAsync(dev_table + row0 * dev_stride + col0, (size_t)dev_stride * e,
                                   host_table + row0 * host_stride + col0, (size_t)host_stride * e,
                                   (size_t)(col1 - col0) * e, (size_t)n_rows, hipMemcpyHostToDevice,
                                   (hipStream_t)stream);
  if (st != hipSuccess) return rc::fail(RC_ERR_HIP, "table upload failed: %s", hipGetErrorString(st));
  return RC_OK;
}

extern "C" rc_status rc_prof_enable(int32_t on) {
  rc::g_on = on != 0;
  // events are created here, not at the launches, so a timed region pays
  // only for the records (creating an event takes far longer)
  constexpr size_t kPool = 16384;
  while (rc::g_on && rc::g_pool.size() + rc::g_recs.size() * 2 < kPool) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return rc::fail(RC_ERR_HIP, "hipEventCreate failed");
    rc::g_pool.push_back(e);
  }
  return RC_OK;
}

extern "C" rc_status rc_prof_tag(const char* tag) {
  rc::g_tag = tag ? tag : "";
  if (rc::g_tag.size() > 15) rc::g_tag.resize(15);
  return RC_OK;
}

extern "C" rc_status rc_prof_collect(rc_prof_entry* out, int32_t capacity, int32_t* n_out) {
  using namespace rc;
  if (!n_out || capacity < 0 || (capacity > 0 && !out)) return fail(RC_ERR_ARG, "bad argument to rc_prof_collect");
  std::vector<rc_prof_entry> agg;
  rc_status st = RC_OK;
  for (auto& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = fail(RC_ERR_HIP, "event timing failed for %s", r.name.c_str());
      ms = 0.f;
    }
    size_t i = 0;
    for (; i < agg.size(); ++i)
      if (!strncmp(agg[i].name, r.name.c_str(), sizeof(agg[i].name) - 1)) break;
    if (i == agg.size()) {
      rc_prof_entry e{};
      strncpy(e.name, r.name.c_str(), sizeof(e.name) - 1);
      agg.push_back(e);
    }
    agg[i].launches++;
    agg[i].total_ms += ms;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  int32_t n = (int32_t)agg.size();
  for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = agg[i];
  *n_out = n;
  return st;
}
