// Foreign-load helper for tests and measurement: a kernel that holds a chosen number of CUs
// for a bounded time, so the scan can be run while part of the GPU is taken.
//
// The pages' scheduling argument (flashinfer PR #8691, description and ticket-word commit):
// with a fixed per-block schedule a kernel holding SMs pushes the blocks it displaces into a
// second wave; with work drawn from a ticket counter the resident blocks take that work.
// This helper reproduces the condition on the AMD GPU: `cus` workgroups of 1024 threads, each
// reserving 128 KiB of a CU's 160 KiB of LDS and keeping about 100 VGPRs per wave live (four
// waves per SIMD), so that each lands on its own CU and no score workgroup (two waves of up to
// 224 VGPRs per SIMD) fits beside it, spin on the 100 MHz real-time counter until the requested
// time has passed.  Every wave exits on time; an iteration bound backs the time bound.

#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdint>
#include <mutex>

namespace {

constexpr size_t kHoldLds = 128 * 1024;

constexpr int kHoldThreads = 1024;  // 16 waves: 4 per SIMD
constexpr int kHoldLive = 96;       // values kept live across the wait: > 96 VGPRs per wave

__global__ __launch_bounds__(kHoldThreads) void hold_kernel(uint64_t ticks, const float* src, float* sink,
                                                           volatile uint32_t* started) {
  extern __shared__ unsigned char reserve[];
  float live[kHoldLive];
#pragma unroll
  for (int i = 0; i < kHoldLive; ++i) live[i] = src[i * 64 + (threadIdx.x & 63)];  // per lane: VGPRs
  if (threadIdx.x == 0) {  // tell the host this workgroup holds its CU
    started[blockIdx.x] = 1u;
    __threadfence_system();
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint64_t it = 0;
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks && it < (1ull << 28)) {
    __builtin_amdgcn_s_sleep(2);
    ++it;
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kHoldLive; ++i) acc += live[i] * (float)(it & (i + 1));
  reserve[threadIdx.x] = (unsigned char)it;
  if (acc == 12345.f && reserve[threadIdx.x] == 0xff) sink[threadIdx.x] = acc;  // keeps registers and LDS in use
}

struct Held {
  hipStream_t stream = nullptr;
  uint32_t* started = nullptr;  // pinned host flags, one per holding workgroup
  float* src = nullptr;         // device: kHoldLive x 64 zeros
  float* sink = nullptr;        // device: never written in practice
  int cus = 0;
};
std::mutex g_mu;
Held g_held;

}  // namespace

extern "C" {

// Launch the holder on `cus` CUs (1..256) for `microseconds` on a stream of its own; returns 0,
// or 1000/2000/3000/4000/5000 + the HIP error of stream creation / attribute / launch / flags /
// buffers.
int spinner_start(int cus, double microseconds) {
  if (cus < 1 || cus > 256 || microseconds < 0 || microseconds > 1e6) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_held.stream) {
    hipError_t e = hipStreamCreateWithFlags(&g_held.stream, hipStreamNonBlocking);
    if (e != hipSuccess) return 1000 + (int)e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&hold_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHoldLds);
    if (e != hipSuccess) return 2000 + (int)e;
    e = hipHostMalloc(reinterpret_cast<void**>(&g_held.started), 256 * sizeof(uint32_t), hipHostMallocDefault);
    if (e != hipSuccess) return 4000 + (int)e;
    e = hipMalloc(reinterpret_cast<void**>(&g_held.src), kHoldLive * 64 * sizeof(float));
    if (e != hipSuccess) return 5000 + (int)e;
    e = hipMalloc(reinterpret_cast<void**>(&g_held.sink), kHoldThreads * sizeof(float));
    if (e != hipSuccess) return 5000 + (int)e;
    e = hipMemset(g_held.src, 0, kHoldLive * 64 * sizeof(float));
    if (e != hipSuccess) return 5000 + (int)e;
  }
  for (int i = 0; i < 256; ++i) reinterpret_cast<volatile uint32_t*>(g_held.started)[i] = 0u;
  g_held.cus = cus;
  const uint64_t ticks = (uint64_t)(microseconds * 100.0);  // 100 MHz counter
  hipLaunchKernelGGL(hold_kernel, dim3(cus), dim3(kHoldThreads), kHoldLds, g_held.stream, ticks,
                     (const float*)g_held.src, g_held.sink, g_held.started);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : 3000 + (int)e;
}

// LDS limits of the current device: bytes per workgroup and per CU.
int spinner_lds_limits(int* per_block, int* per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return -2;
  if (hipDeviceGetAttribute(per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
    return -3;
  return 0;
}

// Wait (polling host memory, at most timeout_ms) until every holding workgroup of the last
// spinner_start has started; returns 0, or -1 on timeout.
int spinner_wait_resident(double timeout_ms) {
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    int n = 0;
    {
      std::lock_guard<std::mutex> lk(g_mu);
      if (!g_held.started) return -1;
      for (int i = 0; i < g_held.cus; ++i) n += reinterpret_cast<volatile uint32_t*>(g_held.started)[i] ? 1 : 0;
      if (n == g_held.cus) return 0;
    }
    const double el = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (el > timeout_ms) return -1;
  }
}

int spinner_sync() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_held.stream) return 0;
  return (int)hipStreamSynchronize(g_held.stream);
}

}  // extern "C"
