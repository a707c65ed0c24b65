// Measurement probe (not part of libcpattn): throughput of fp32 atomic adds
// on MI355X for the access pattern a KV-outer backward would use to
// accumulate dQ.  It backs the design choice of a separate dQ kernel that
// recomputes S and dP instead of adding dS K into dQ with atomics.
//
// Grid of 1024 work-groups x 8 waves.  Work-group b runs ITEMS items; item it
// is (query tile t, head h) with t = NT-1 - it/4 (every work-group on the
// same tile at the same time: the kernel's own order) or staggered per
// work-group, h = it % 4.  Wave w adds 1.0 to its 32 rows x 128 floats of
// dq[t*64 + 32(w/4) + r][h][:] in the layout an MFMA accumulator holds them
// (lane = column within a 32-float block, 4 instructions per row pair).
// Modes: 0 one buffer; 1 eight copies, the work-group adding into the copy
// of the XCD it runs on (s_getreg XCC_ID); 2 plain stores (one buffer, for
// comparison); 4 and 5 as 0 and 1 with staggered tiles.  Every atomic mode
// is checked: the sum over the buffer(s) must equal the number of adds.
//
// Build and run (prints one line per mode and repetition):
//   hipcc --offload-arch=gfx950 -O3 -o /tmp/atomic_add sequence_context_parallelism_amd/probes/atomic_add.hip
//   /tmp/atomic_add 256
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

constexpr int D = 128, H = 4;

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

__global__ __launch_bounds__(512, 1) void add_kernel(float* dq, int nt, int items, int mode, int* xcc_out,
                                                     size_t copy_elems) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  if (threadIdx.x == 0) xcc_out[blockIdx.x] = (int)x;
  const int m = mode & 3;
  float* base = dq + (m == 1 ? (size_t)(x & 7) * copy_elems : 0);
  for (int it = 0; it < items; ++it) {
    const int stagger = (mode >> 2) ? (int)blockIdx.x * 7 : 0;
    const int t = (int)((unsigned)(nt - 1 - (it / H) + stagger) % (unsigned)nt);
    const int h = it % H;
    const int row0 = t * 64 + 32 * (w >> 2);          // rows row0 .. row0 + 31 < nt * 64
    for (int i = 0; i < 16; ++i) {
      const int r = row0 + 2 * i + (lane >> 5);
      float* p = base + ((size_t)r * H + h) * D + (lane & 31);
      for (int e = 0; e < 4; ++e) {
        if (m == 2) p[32 * e] = 1.f;
        else __hip_atomic_fetch_add(p + 32 * e, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int nt = 1024, nwg = 1024, items = argc > 1 ? std::atoi(argv[1]) : 256;
  const size_t copy_elems = (size_t)nt * 64 * H * D;
  float* dq;
  int* xo;
  CHECK(hipMalloc(&dq, 8 * copy_elems * sizeof(float)));
  CHECK(hipMalloc(&xo, nwg * sizeof(int)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<float> h(copy_elems);
  const int modes[] = {0, 1, 2, 4, 5};
  for (int mode : modes) {
    for (int rep = 0; rep < 2; ++rep) {
      CHECK(hipMemset(dq, 0, 8 * copy_elems * sizeof(float)));
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(add_kernel, dim3(nwg), dim3(512), 0, 0, dq, nt, items, mode, xo, copy_elems);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double bytes = (double)nwg * items * 8 * 32 * D * 4;
      double tot = 0;
      for (int c = 0; c < ((mode & 3) == 1 ? 8 : 1); ++c) {
        CHECK(hipMemcpy(h.data(), dq + c * copy_elems, copy_elems * sizeof(float), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < copy_elems; ++i) tot += h[i];
      }
      std::printf("mode %d rep %d: %.3f ms, %.2f TB/s of fp32 %s traffic, sum %.0f (atomic modes expect %.0f)\n",
                  mode, rep, ms, bytes / (ms * 1e-3) / 1e12, (mode & 3) == 2 ? "store" : "atomic-add", tot,
                  bytes / 4);
      std::fflush(stdout);
    }
  }
  std::vector<int> xh(nwg);
  CHECK(hipMemcpy(xh.data(), xo, nwg * sizeof(int), hipMemcpyDeviceToHost));
  int cnt[16] = {0};
  for (int i = 0; i < nwg; ++i) cnt[xh[i] & 15]++;
  std::printf("work-groups per XCC:");
  for (int i = 0; i < 8; ++i) std::printf(" %d", cnt[i]);
  std::printf("\n");
  CHECK(hipFree(dq));
  CHECK(hipFree(xo));
  return 0;
}
