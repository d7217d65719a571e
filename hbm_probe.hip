// HBM measurement probe (not part of the layer): the streaming-read ceiling that
// the decode kernels are compared against, and a plain copy kernel of known size
// whose FETCH_SIZE / WRITE_SIZE counter readings calibrate the byte counters.
//
//   hbm_probe read   -> read bandwidth: large grid-stride reads and decode-sized
//                       reads (each wave streams a contiguous chunk)
//   hbm_probe copy N -> copies N MiB (default 1024) five times
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#define CK(x)                                                                      \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);  \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ void k_read_stride(const u32x4 *__restrict__ p, size_t n, unsigned *out) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) out[0] = 1;  // keeps the loads alive
}

// Wave w streams bytes [w*chunk, (w+1)*chunk) in 1 KB wave loads, D in flight.
template <int D>
__global__ void k_read_chunk(const unsigned char *__restrict__ p, size_t chunk, size_t nwaves, unsigned *out) {
  const size_t w = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x & 63;
  if (w >= nwaves) return;
  const unsigned char *base = p + w * chunk + lane * 16;
  const size_t steps = chunk / 1024;
  u32x4 acc = {0, 0, 0, 0};
  size_t s = 0;
  for (; s + D <= steps; s += D) {
    u32x4 v[D];
#pragma unroll
    for (int u = 0; u < D; ++u) v[u] = *(const u32x4 *)(base + (s + u) * 1024);
#pragma unroll
    for (int u = 0; u < D; ++u) acc ^= v[u];
  }
  for (; s < steps; ++s) acc ^= *(const u32x4 *)(base + s * 1024);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) out[0] = 1;
}

__global__ void k_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

int main(int argc, char **argv) {
  const char *mode = argc > 1 ? argv[1] : "read";
  int dev = 0;
  CK(hipGetDevice(&dev));
  hipDeviceProp_t pr;
  CK(hipGetDeviceProperties(&pr, dev));
  unsigned *out = nullptr;
  CK(hipMalloc(&out, 64));
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  if (!std::strcmp(mode, "copy")) {
    const size_t mib = argc > 2 ? (size_t)std::atol(argv[2]) : 1024;
    const size_t bytes = mib << 20;
    unsigned char *s = nullptr, *d = nullptr;
    CK(hipMalloc(&s, bytes));
    CK(hipMalloc(&d, bytes));
    CK(hipMemset(s, 1, bytes));
    CK(hipDeviceSynchronize());
    for (int r = 0; r < 5; ++r) {
      CK(hipEventRecord(a));
      hipLaunchKernelGGL(k_copy, dim3(pr.multiProcessorCount * 8), dim3(256), 0, 0, (const u32x4 *)s, (u32x4 *)d,
                         bytes / 16);
      CK(hipEventRecord(b));
      CK(hipEventSynchronize(b));
      float ms = 0.f;
      CK(hipEventElapsedTime(&ms, a, b));
      std::printf("copy %zu MiB: %.1f us, %.0f GB/s (read + write)\n", mib, ms * 1e3, 2.0 * bytes / (ms * 1e-3) / 1e9);
    }
    return 0;
  }
  const size_t bytes = (size_t)8 << 30;
  unsigned char *buf = nullptr;
  CK(hipMalloc(&buf, bytes));
  CK(hipMemset(buf, 1, bytes));
  CK(hipDeviceSynchronize());
  std::printf("device %s, %d CUs, %d kHz\n", pr.gcnArchName, pr.multiProcessorCount, pr.clockRate);
  auto best_of = [&](auto launch, int reps) -> float {
    launch();
    (void)hipDeviceSynchronize();
    float best = 1e30f;
    for (int r = 0; r < reps; ++r) {
      (void)hipEventRecord(a);
      launch();
      (void)hipEventRecord(b);
      (void)hipEventSynchronize(b);
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, a, b);
      best = ms < best ? ms : best;
    }
    return best;
  };
  for (int per_cu : {2, 4, 8}) {
    const int grid = pr.multiProcessorCount * per_cu;
    const float ms = best_of([&] { hipLaunchKernelGGL(k_read_stride<4>, dim3(grid), dim3(256), 0, 0,
                                                      (const u32x4 *)buf, bytes / 16, out); }, 5);
    std::printf("read 8 GiB grid-stride, %d blocks/CU: %8.1f us  %6.0f GB/s\n", per_cu, ms * 1e3, bytes / (ms * 1e-3) / 1e9);
  }
  // decode-sized reads, a different region each repetition (no reuse from the 256 MB Infinity Cache)
  const size_t totals[3] = {127401984, 63700992, 191102976};
  for (size_t total : totals) {
    for (size_t nw : {(size_t)1024, (size_t)2048, (size_t)4096}) {
      const size_t chunk = total / nw / 1024 * 1024;
      const size_t nbytes = chunk * nw;
      size_t off = 0;
      auto L = [&] {
        off = (off + nbytes + ((size_t)64 << 20)) % (bytes - nbytes - 4096) & ~(size_t)4095;
        hipLaunchKernelGGL(k_read_chunk<4>, dim3((unsigned)((nw * 64 + 255) / 256)), dim3(256), 0, 0, buf + off, chunk,
                           nw, out);
      };
      const float ms = best_of(L, 20);
      std::printf("read %6.1f MB as %5zu waves x %4zu KB: %7.1f us  %6.0f GB/s\n", nbytes / 1e6, nw, chunk >> 10,
                  ms * 1e3, nbytes / (ms * 1e-3) / 1e9);
    }
  }
  const float e_ms = best_of([&] { hipLaunchKernelGGL(k_read_chunk<4>, dim3(1), dim3(64), 0, 0, buf, 0, 0, out); }, 20);
  std::printf("empty launch (event to event): %.1f us\n", e_ms * 1e3);
  return 0;
}
