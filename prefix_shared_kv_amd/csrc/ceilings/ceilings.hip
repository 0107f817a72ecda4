// Measured ceilings of the two resources the attention kernels are bound by,
// for the roofline figures beside the datasheet peaks: streaming reads of
// HBM (16-byte loads, plain or nontemporal, grid-strided or one contiguous
// region per wave) and a dense bf16 MFMA loop
// (v_mfma_f32_32x32x16_bf16, the extend tile's instruction).  Built into its
// own library (libceilings.so); the attention library does not contain it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every thread reads 16-byte vectors at a grid-wide stride and folds them into
// one word, written only if it could be zero (never, for the inputs used), so
// the loads are not removed.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, int64_t n_vec, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < n_vec ? (NT ? __builtin_nontemporal_load(src + j) : src[j]) : u32x4{1, 1, 1, 1};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

// Every wave streams its own contiguous region of n_stages x 16 KiB: the
// lanes load a stage as 16 consecutive 1 KiB pieces (16 bytes each, the
// pattern of a decode wave reading a run of keys) and fold the previous stage
// while the next one is in flight, so 16 KiB per wave are outstanding.
__global__ __launch_bounds__(256, 2) void wave_stream(const u32x4* __restrict__ src, int n_stages, uint32_t* out) {
  constexpr int NI = 16;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const u32x4* base = src + wave * (int64_t)n_stages * NI * 64 + lane;
  u32x4 buf[NI];
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) buf[i] = __builtin_nontemporal_load(base + i * 64);
  for (int s = 1; s <= n_stages; ++s) {
#pragma unroll
    for (int i = 0; i < NI; ++i) acc ^= buf[i].x ^ buf[i].y ^ buf[i].z ^ buf[i].w;
    if (s < n_stages) {
#pragma unroll
      for (int i = 0; i < NI; ++i) buf[i] = __builtin_nontemporal_load(base + ((int64_t)s * NI + i) * 64);
    }
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave,
// iters rounds; the results are folded into one word so nothing is removed.
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (threadIdx.x - i));
  }
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 1234.5f) out[0] = s;
}

}  // namespace

// Average milliseconds of `reps` launches (after one warm-up) of a streaming
// read of n_bytes (a multiple of 16) at `src`; nontemporal: 0 or 1.
// Returns a negative value on a HIP error.
extern "C" double ceil_stream_read_ms(const void* src, int64_t n_bytes, int32_t nontemporal, int32_t reps,
                                      uint32_t* scratch_word, void* stream) {
  if (!src || n_bytes <= 0 || n_bytes % 16 || reps < 1 || !scratch_word) return -1.0;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n_vec = n_bytes / 16;
  const int blocks = 256 * 16;  // 16 workgroups of 4 waves per CU on 256 CUs
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -2.0;
  auto launch = [&]() {
    if (nontemporal)
      hipLaunchKernelGGL(stream_read<true>, dim3(blocks), dim3(256), 0, s, (const u32x4*)src, n_vec, scratch_word);
    else
      hipLaunchKernelGGL(stream_read<false>, dim3(blocks), dim3(256), 0, s, (const u32x4*)src, n_vec, scratch_word);
  };
  launch();
  (void)hipEventRecord(e0, s);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(e1, s);
  float ms = -3.f;
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) ms = -3.f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return hipGetLastError() == hipSuccess ? ms / reps : -4.0;
}

// Average milliseconds of `reps` launches (after one warm-up) of `waves`
// waves (a multiple of 4) each streaming its own n_stages x 16 KiB of `src`
// (which holds at least waves x n_stages x 16 KiB).
extern "C" double ceil_wave_stream_ms(const void* src, int32_t waves, int32_t n_stages, int32_t reps,
                                      uint32_t* scratch_word, void* stream) {
  if (!src || waves < 4 || waves % 4 || n_stages < 1 || reps < 1 || !scratch_word) return -1.0;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -2.0;
  hipLaunchKernelGGL(wave_stream, dim3(waves / 4), dim3(256), 0, s, (const u32x4*)src, n_stages, scratch_word);
  (void)hipEventRecord(e0, s);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(wave_stream, dim3(waves / 4), dim3(256), 0, s, (const u32x4*)src, n_stages, scratch_word);
  (void)hipEventRecord(e1, s);
  float ms = -3.f;
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) ms = -3.f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return hipGetLastError() == hipSuccess ? ms / reps : -4.0;
}

// Average milliseconds of `reps` launches of the MFMA loop on `blocks`
// workgroups of 4 waves, each wave issuing 4 * iters MFMAs (32x32x16 bf16:
// 32768 flops each).
extern "C" double ceil_mfma_ms(int32_t blocks, int32_t iters, int32_t reps, float* scratch_word, void* stream) {
  if (blocks < 1 || iters < 1 || reps < 1 || !scratch_word) return -1.0;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -2.0;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, s, iters, scratch_word);
  (void)hipEventRecord(e0, s);
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, s, iters, scratch_word);
  (void)hipEventRecord(e1, s);
  float ms = -3.f;
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) ms = -3.f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return hipGetLastError() == hipSuccess ? ms / reps : -4.0;
}
