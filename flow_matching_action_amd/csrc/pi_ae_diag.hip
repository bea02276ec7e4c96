// Measurement diagnostics of the machine the loop runs on (test-only exports,
// declared in include/pi_ae.h): the floors under the batch-1 design.
//
// Realtime-VLA technical blog, section 5 (roofline): the loop's lower bound is
// the weights streamed from memory once per step; sections "CUDA Graph" and
// 4 (kernel fusion): the loop is a replayed graph of about 900 decoder
// kernels.  These calls measure what those two facts cost on this GPU:
//   * a plain streaming read of a large buffer (the practical ceiling of the
//     weight stream),
//   * the time per kernel of a replayed graph of dependent empty kernels (the
//     floor that every kernel boundary of the graph adds),
//   * the time per round of a grid-wide barrier inside one persistent kernel
//     (what replacing those boundaries with in-kernel synchronisation costs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>

#include "pi_ae.h"
#include "pi_ae_kernels.h"

#define PI_AE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming read: every 16-byte word once, 4 loads in flight per thread; a
// workgroup writes only if the XOR of what it read hits a magic value, which
// keeps the loads.
__global__ __launch_bounds__(256) void k_diag_read(const u32x4* __restrict__ a, size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = size_t(gridDim.x) * 256;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t j = i + size_t(k) * stride;
      v[k] = j < n16 ? a[j] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ void k_diag_empty(uint32_t* sink) {
  if (threadIdx.x == 0xFFFFu) sink[0] = 1;
}

// Grid barrier rounds in one persistent kernel (one workgroup per CU, all
// resident).  Every wait is bounded: a workgroup that spins past the limit
// raises the abort flag, and every workgroup leaves at its next wait, so the
// kernel always ends.
//   mode 0: each workgroup stores its round number into its own 128-byte line
//           (agent-scope store), then waits until every line holds the round;
//   mode 1: each workgroup adds one to the counter of its XCD residue
//           (blockIdx mod 8); the last arriver of a residue adds one to a
//           global counter, which every workgroup waits on.
constexpr int kSpinLimit = 1 << 22;
constexpr int kFlagStride = 32;  // ints: one 128-byte line per workgroup

__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_diag_grid_sync(int* flags, int* counters, int* abort_flag, int rounds,
                                                        int mode) {
  const int G = int(gridDim.x), wg = int(blockIdx.x), t = int(threadIdx.x);
  __shared__ int stop;
  for (int r = 1; r <= rounds; ++r) {
    if (t == 0) {
      if (mode == 0) {
        st_agent(flags + wg * kFlagStride, r);
      } else {
        const int res = wg & 7, per = (G - res + 7) / 8;
        const int old = __hip_atomic_fetch_add(counters + 32 * (1 + res), 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (old == r * per - 1) __hip_atomic_fetch_add(counters, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (mode == 0) {
      for (int i = t; i < G; i += 256) {
        int it = 0;
        while (ld_agent(flags + i * kFlagStride) < r) {
          if (++it > kSpinLimit || ld_agent(abort_flag)) {
            st_agent(abort_flag, 1);
            break;
          }
        }
      }
    } else if (t == 0) {
      const int target = r * ((G < 8) ? G : 8);
      int it = 0;
      while (ld_agent(counters) < target) {
        if (++it > kSpinLimit || ld_agent(abort_flag)) {
          st_agent(abort_flag, 1);
          break;
        }
      }
    }
    if (t == 0) stop = ld_agent(abort_flag);
    __syncthreads();
    if (stop) return;
    __syncthreads();
  }
}

pi_ae_status diag_fail(pi_ae_status st, const std::string& m) {
  pi_ae::set_last_error(m);
  return st;
}

pi_ae_status diag_hip(hipError_t e, const char* what) {
  return diag_fail(e == hipErrorOutOfMemory ? PI_AE_ENOMEM : PI_AE_EHIP,
                   std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

PI_AE_API pi_ae_status pi_ae_debug_stream_read(size_t bytes, int32_t reps, void* stream, float* gbps) {
  if (!gbps || reps < 1 || reps > 1000 || bytes < (size_t(1) << 20) || bytes > (size_t(16) << 30))
    return diag_fail(PI_AE_EINVAL, "stream_read: bytes in [1 MiB, 16 GiB], reps in [1, 1000], gbps non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* buf = nullptr;
  uint32_t* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&buf, bytes);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&sink), 64);
  if (e == hipSuccess) e = hipMemsetAsync(buf, 1, bytes, s);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  int cus = 0, dev = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  float best = 0.f;
  const size_t n16 = bytes / 16;
  const unsigned grid = unsigned(cus > 0 ? 32 * cus : 8192);
  for (int r = -1; r < reps && e == hipSuccess; ++r) {  // r = -1: warm-up
    e = hipEventRecord(e0, s);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_diag_read, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(buf), n16, sink);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && r >= 0 && ms > 0.f) best = std::max(best, float(double(n16) * 16.0 / (ms * 1e6)));
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (buf) (void)hipFree(buf);
  if (e != hipSuccess) return diag_hip(e, "stream_read");
  *gbps = best;
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_debug_graph_floor(int32_t kernels, int32_t grid, void* stream, float* us_per_kernel) {
  if (!us_per_kernel || kernels < 1 || kernels > 4096 || grid < 1 || grid > 65536)
    return diag_fail(PI_AE_EINVAL, "graph_floor: kernels in [1, 4096], grid in [1, 65536], output non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t cap = nullptr;
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  uint32_t* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&sink), 64);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t e2 = hipSuccess;
    for (int i = 0; i < kernels && e2 == hipSuccess; ++i) {
      hipLaunchKernelGGL(k_diag_empty, dim3(unsigned(grid)), dim3(256), 0, cap, sink);
      e2 = hipGetLastError();
    }
    e = hipStreamEndCapture(cap, &g);
    if (e2 != hipSuccess) e = e2;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  constexpr int kReps = 10;
  for (int w = 0; w < 2 && e == hipSuccess; ++w) e = hipGraphLaunch(ge, s);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  for (int r = 0; r < kReps && e == hipSuccess; ++r) e = hipGraphLaunch(ge, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (ge) (void)hipGraphExecDestroy(ge);
  if (g) (void)hipGraphDestroy(g);
  if (cap) (void)hipStreamDestroy(cap);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (e != hipSuccess) return diag_hip(e, "graph_floor");
  *us_per_kernel = ms * 1000.f / float(kReps * kernels);
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_debug_grid_sync(int32_t rounds, int32_t mode, void* stream, float* us_per_round) {
  if (!us_per_round || rounds < 1 || rounds > 100000 || mode < 0 || mode > 1)
    return diag_fail(PI_AE_EINVAL, "grid_sync: rounds in [1, 100000], mode 0 or 1, output non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 0, occ = 0, dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(k_diag_grid_sync), 256, 0);
  if (e != hipSuccess) return diag_hip(e, "grid_sync");
  // one workgroup per CU: all of them resident at once, so every wait can end
  if (cus < 1 || occ < 1) return diag_fail(PI_AE_EUNSUPPORTED, "grid_sync: no resident workgroup per CU");
  int *flags = nullptr, *counters = nullptr, *abort_flag = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const size_t flag_bytes = size_t(cus) * kFlagStride * 4;
  e = hipMalloc(reinterpret_cast<void**>(&flags), flag_bytes);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&counters), 32 * 9 * 4);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&abort_flag), 64);
  if (e == hipSuccess) e = hipMemsetAsync(flags, 0, flag_bytes, s);
  if (e == hipSuccess) e = hipMemsetAsync(counters, 0, 32 * 9 * 4, s);
  if (e == hipSuccess) e = hipMemsetAsync(abort_flag, 0, 64, s);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_diag_grid_sync, dim3(unsigned(cus)), dim3(256), 0, s, flags, counters, abort_flag, rounds,
                       mode);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  int aborted = 0;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) e = hipMemcpy(&aborted, abort_flag, 4, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (flags) (void)hipFree(flags);
  if (counters) (void)hipFree(counters);
  if (abort_flag) (void)hipFree(abort_flag);
  if (e != hipSuccess) return diag_hip(e, "grid_sync");
  if (aborted) return diag_fail(PI_AE_ESTATE, "grid_sync: a wait passed its spin limit (rounds abandoned)");
  *us_per_round = ms * 1000.f / float(rounds);
  return PI_AE_OK;
}
