// HBM bandwidth probe for the fused pass's access patterns (no arithmetic).
//
// Measures what the memory system delivers for the byte patterns the fused
// verify + distillation kernel produces, on rows of the concurrent workload's
// shape (2048 rows of V = 151936 bfloat16 logits for zp and for zq, a float32
// gradient row per row):
//   read   : stream zp and zq once (16-byte nontemporal loads)
//   write  : store the gradient array once (16-byte stores)
//   copy   : read zp and zq, write the gradient array, element by element
//   rows   : one workgroup per row: read the row's zp and zq, workgroup
//            barrier, write the row's gradient (the fused kernel's phases for
//            a verified row, without its arithmetic)
// Each pattern is timed with HIP events: 3 launches of warm-up, then the
// median of 10.  Output: one line per pattern and launch shape,
//   <pattern> <block> <workgroups per CU> <microseconds> <GB/s>
// where GB/s counts every byte read and written once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                    \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      std::exit(1);                                                                 \
    }                                                                               \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kU = 8;  // loads in flight per thread and loop trip

// XOR of every vector; stored only if it equals a value the inputs never give.
__global__ void read_k(const u32x4* __restrict__ a, size_t n, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kU - 1) * stride < n; i += kU * stride) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(a + i + u * stride);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= a[i];
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}

__global__ void write_k(u32x4* __restrict__ b, size_t n) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) b[i] = z;
}

__global__ void copy_k(const u32x4* __restrict__ a, u32x4* __restrict__ b, size_t n) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(a + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], b + i + u * stride);
  }
  for (; i < n; i += stride) b[i] = a[i];
}

// Workgroup g takes rows g, g + grid, ...: reads rv vectors of zp and of zq,
// barrier, writes 2 rv vectors of the gradient row.
__global__ void rows_k(const u32x4* __restrict__ zp, const u32x4* __restrict__ zq, u32x4* __restrict__ g,
                       int R, int rv, u32x4* sink) {
  constexpr int U = 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const u32x4* p = zp + (size_t)r * rv;
    const u32x4* q = zq + (size_t)r * rv;
    int i = threadIdx.x;
    for (; i + (U - 1) * (int)blockDim.x < rv; i += U * blockDim.x) {
      u32x4 v[2 * U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u] = __builtin_nontemporal_load(p + i + u * blockDim.x);
        v[U + u] = __builtin_nontemporal_load(q + i + u * blockDim.x);
      }
#pragma unroll
      for (int u = 0; u < 2 * U; ++u) acc ^= v[u];
    }
    for (; i < rv; i += blockDim.x) acc ^= p[i] ^ q[i];
    __syncthreads();
    u32x4* o = g + (size_t)r * 2 * rv;
    const u32x4 z = {acc.x & 0u, 0u, 0u, 0u};
    for (int j = threadIdx.x; j < 2 * rv; j += blockDim.x) __builtin_nontemporal_store(z, o + j);
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}

template <class F>
float median_ms(hipEvent_t e0, hipEvent_t e1, F&& launch) {
  for (int i = 0; i < 3; ++i) launch();
  std::vector<float> t;
  for (int i = 0; i < 10; ++i) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    t.push_back(ms);
  }
  CHECK(hipGetLastError());
  std::sort(t.begin(), t.end());
  return t[t.size() / 2];
}

void report(const char* pattern, int block, int per_cu, float ms, double bytes) {
  std::printf("%s %d %d %.1f %.0f\n", pattern, block, per_cu, ms * 1e3, bytes / (ms * 1e-3) / 1e9);
  std::fflush(stdout);
}

}  // namespace

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  const int R = 2048, V = 151936;
  const int rv = V * 2 / 16;           // 16-byte vectors per bfloat16 row
  const size_t n = (size_t)R * rv;     // vectors per logit array
  u32x4 *zp = nullptr, *zq = nullptr, *g = nullptr, *sink = nullptr;
  CHECK(hipMalloc(&zp, n * 16));
  CHECK(hipMalloc(&zq, n * 16));
  CHECK(hipMalloc(&g, 2 * n * 16));
  CHECK(hipMalloc(&sink, 1024 * 16));
  CHECK(hipMemset(zp, 1, n * 16));
  CHECK(hipMemset(zq, 2, n * 16));
  CHECK(hipMemset(g, 0, 2 * n * 16));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const double logit_bytes = 2.0 * n * 16, grad_bytes = 2.0 * n * 16;
  for (int block : {256, 1024})
    for (int per : {1, 2, 4}) {
      const int grid = cus * per * (1024 / block);
      report("read", block, per * (1024 / block),
             median_ms(e0, e1, [&] {
               read_k<<<grid, block>>>(zp, n, sink);
               read_k<<<grid, block>>>(zq, n, sink);
             }),
             logit_bytes);
      report("write", block, per * (1024 / block),
             median_ms(e0, e1, [&] { write_k<<<grid, block>>>(g, 2 * n); }), grad_bytes);
      report("copy", block, per * (1024 / block),
             median_ms(e0, e1, [&] {
               copy_k<<<grid, block>>>(zp, g, n);
               copy_k<<<grid, block>>>(zq, g + n, n);
             }),
             logit_bytes + grad_bytes);
    }
  for (int block : {256, 512, 1024})
    for (int per : {1, 2, 4}) {
      if (block * per > 2048) continue;
      const int grid = cus * per;
      report("rows", block, per, median_ms(e0, e1, [&] { rows_k<<<grid, block>>>(zp, zq, g, R, rv, sink); }),
             logit_bytes + grad_bytes);
    }
  CHECK(hipFree(zp));
  CHECK(hipFree(zq));
  CHECK(hipFree(g));
  CHECK(hipFree(sink));
  return 0;
}
