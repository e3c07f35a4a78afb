// Measurement kernels for the two ceilings of the cache kernels on gfx950:
// dense FP8 matrix throughput and the HBM bandwidth of an in-place stream,
// with their C ABI (rkv_probe.h).  Built into librkv_probe.so, a library of
// its own beside the cache library: these are measurement aids of the
// benchmark, not steps of the cache method.
#include <hip/hip_runtime.h>

#include <string>

#include "rkv_probe.h"

namespace rkv {

typedef int v8i_p __attribute__((ext_vector_type(8)));
typedef float v16f_p __attribute__((ext_vector_type(16)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// Four independent accumulation chains per wave keep the matrix unit busy
// without depending on the latency of one instruction.  The operands are
// e4m3 1.0 (0x38) in every byte: each instruction adds 64 to every
// accumulator element, exact in fp32 for any iteration count used here.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* sink) {
  const int one = 0x38383838;
  v8i_p a = {one, one, one, one, one, one, one, one};
  v8i_p b = a;
  v16f_p c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = c0[0] + c1[5] + c2[10] + c3[15];
}

// Grid-stride in-place pass: each workgroup takes 4 x 256 consecutive
// 16-byte words per step, issuing all four loads before the stores.
__global__ __launch_bounds__(256) void probe_stream_kernel(u4v* p, long long n16) {
  constexpr int R = 4;
  const long long stride = (long long)gridDim.x * 256 * R;
  for (long long base = (long long)blockIdx.x * 256 * R + threadIdx.x; base < n16; base += stride) {
    u4v x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const long long i = base + r * 256;
      if (i < n16) x[r] = __builtin_nontemporal_load(p + i);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const long long i = base + r * 256;
      if (i < n16) {
        u4v y = x[r];
        y.x = ~y.x;
        __builtin_nontemporal_store(y, p + i);
      }
    }
  }
}

static hipError_t launch_probe_mfma(int workgroups, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

static hipError_t launch_probe_stream(void* buf, size_t bytes, hipStream_t s) {
  const long long n16 = (long long)(bytes / 16);
  // one 16 KiB block per workgroup up to 65,536 workgroups (1 GiB); larger
  // buffers loop.  Many short workgroups measured faster than a persistent
  // grid (6.2 against 6.0 TB/s at 8,192) or contiguous chunks (5.5 TB/s).
  long long wg = (n16 + 1023) / 1024;
  if (wg > 65536) wg = 65536;
  hipLaunchKernelGGL(probe_stream_kernel, dim3((unsigned)wg), dim3(256), 0, s, (u4v*)buf, n16);
  return hipGetLastError();
}

}  // namespace rkv

namespace {
thread_local std::string g_probe_err;
int probe_fail(int code, const std::string& msg) {
  g_probe_err = msg;
  return code;
}
bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }
}  // namespace

extern "C" {

const char* rkv_probe_last_error(void) { return g_probe_err.c_str(); }

int rkv_probe_fp8_mfma(int32_t workgroups, int32_t iters, float* sink, hipStream_t stream) {
  if (!sink) return probe_fail(RKV_PROBE_EINVAL, "sink is null");
  if (!aligned(sink, 4)) return probe_fail(RKV_PROBE_EINVAL, "sink must be 4-byte aligned");
  if (workgroups < 1 || workgroups > 65536) return probe_fail(RKV_PROBE_EINVAL, "workgroups outside [1, 65536]");
  if (iters < 1 || iters > (1 << 20)) return probe_fail(RKV_PROBE_EINVAL, "iters outside [1, 2^20]");
  hipError_t e = rkv::launch_probe_mfma(workgroups, iters, sink, stream);
  if (e != hipSuccess) return probe_fail(RKV_PROBE_EHIP, std::string("mfma probe launch: ") + hipGetErrorString(e));
  return 0;
}

int rkv_probe_stream(void* buf, size_t bytes, hipStream_t stream) {
  if (!buf) return probe_fail(RKV_PROBE_EINVAL, "buf is null");
  if (!aligned(buf, 16)) return probe_fail(RKV_PROBE_EINVAL, "buf must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0) return probe_fail(RKV_PROBE_EINVAL, "bytes must be a positive multiple of 16");
  hipError_t e = rkv::launch_probe_stream(buf, bytes, stream);
  if (e != hipSuccess) return probe_fail(RKV_PROBE_EHIP, std::string("stream probe launch: ") + hipGetErrorString(e));
  return 0;
}

}  // extern "C"
