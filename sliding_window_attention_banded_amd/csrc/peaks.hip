// Achievable-peak probes for MI355X (gfx950), run beside the published peaks
// that the roofline divides by:
//   * dense bf16 MFMA (v_mfma_f32_32x32x16_bf16, 8 independent accumulators
//     per wave): once with constant operands and once with random ones, since
//     the sustained clock depends on how much the operands toggle;
//   * LDS read bandwidth (conflict-free ds_read_b128 streams) per CU;
//   * HBM bandwidth on 1 GiB buffers: a plain copy (16 bytes per lane per
//     step), a copy with four 16-byte loads in flight per lane and
//     non-temporal stores, a read-only stream (summed, so the loads stay) and
//     a write-only stream of non-temporal stores.
// The shader clock is measured from s_memtime against the 100 MHz
// s_memrealtime counter on one wave. Prints one line per probe.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

__device__ unsigned mix(unsigned x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

// clk[0] = shader clocks, clk[1] = 100 MHz ticks of wave 0 of block 0
template <int RANDOM>
__global__ __launch_bounds__(256) void mfma_probe(float* out, int iters, unsigned long long* clk) {
  bf16x8 a[4], b[4];
  const unsigned gid = blockIdx.x * 256 + threadIdx.x;
  for (int s = 0; s < 4; ++s)
    for (int i = 0; i < 8; ++i) {
      const float ra = RANDOM ? (mix(gid * 64 + s * 8 + i) & 0xffff) / 32768.f - 1.f : 0.25f * i;
      const float rb = RANDOM ? (mix(gid * 64 + s * 8 + i + 0x9e3779b9u) & 0xffff) / 32768.f - 1.f : 0.5f;
      a[s][i] = (__bf16)ra;
      b[s][i] = (__bf16)rb;
    }
  f32x16 acc[8];
  for (int j = 0; j < 8; ++j)
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 1) & 3], acc[j], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[gid] = s;
  if (gid == 0) { clk[0] = t1 - t0; clk[1] = r1 - r0; }
}

__global__ __launch_bounds__(512) void lds_probe(unsigned* out, int iters, unsigned long long* clk) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  for (int i = threadIdx.x; i < 65536 / 4; i += 512) reinterpret_cast<unsigned*>(lds)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 acc = {0, 0, 0, 0};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  unsigned off = (unsigned)(wave * 4096 + lane * 16);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= *reinterpret_cast<const u32x4*>(lds + ((off + u * 1024) & 65535));
    off += 8192;
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  out[blockIdx.x * 512 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (blockIdx.x == 0 && threadIdx.x == 0) { clk[0] = t1 - t0; clk[1] = r1 - r0; }
}

__global__ __launch_bounds__(256) void copy_probe(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

// four 16-byte loads in flight per lane, then four non-temporal stores; n is
// a multiple of 4 * 256 * gridDim.x
__global__ __launch_bounds__(256) void copy4_probe(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], dst + i + k * stride);
  }
}

// read-only: four loads in flight per lane, summed; one word per lane out
__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ src, unsigned* out, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  unsigned acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// write-only: non-temporal 16-byte stores
__global__ __launch_bounds__(256) void write_probe(u32x4* __restrict__ dst, size_t n) {
  const u32x4 v{1u, 2u, 3u, 4u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    __builtin_nontemporal_store(v, dst + i);
}

float time_ms(hipEvent_t e0, hipEvent_t e1) {
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  return ms;
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  std::printf("device %s, %d CUs, max clock %d MHz\n", prop.gcnArchName, cus, prop.clockRate / 1000);

  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  unsigned long long* clk;
  CHECK(hipMalloc(&clk, 2 * sizeof(unsigned long long)));
  unsigned long long h[2];

  // MFMA: 4 blocks of 4 waves per CU, 8 accumulators per wave
  {
    const int blocks = 4 * cus, iters = 4000;
    float* out;
    CHECK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));
    for (int rnd = 0; rnd < 2; ++rnd) {
      for (int pass = 0; pass < 2; ++pass) {  // warm-up, then timed
        if (pass) CHECK(hipEventRecord(e0));
        const int it = pass ? iters : 200;
        if (rnd) hipLaunchKernelGGL(mfma_probe<1>, dim3(blocks), dim3(256), 0, 0, out, it, clk);
        else hipLaunchKernelGGL(mfma_probe<0>, dim3(blocks), dim3(256), 0, 0, out, it, clk);
        if (!pass) CHECK(hipDeviceSynchronize());
      }
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipGetLastError());
      const float ms = time_ms(e0, e1);
      CHECK(hipMemcpy(h, clk, sizeof h, hipMemcpyDeviceToHost));
      const double flops = 2.0 * 32 * 32 * 16 * 8.0 * iters * blocks * 4;
      std::printf("mfma_bf16 %-8s %8.1f TFLOP/s  clock %5.0f MHz  %.1f cycles per MFMA per wave\n",
                  rnd ? "random" : "constant", flops / ms / 1e9, h[0] / (h[1] / 100.0), h[0] / (8.0 * iters));
    }
    CHECK(hipFree(out));
  }

  // LDS: 2 blocks of 8 waves per CU, 8 KB read per wave per iteration
  {
    const int blocks = 2 * cus, iters = 4000;
    unsigned* out;
    CHECK(hipMalloc(&out, (size_t)blocks * 512 * sizeof(unsigned)));
    hipLaunchKernelGGL(lds_probe, dim3(blocks), dim3(512), 0, 0, out, 100, clk);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(lds_probe, dim3(blocks), dim3(512), 0, 0, out, iters, clk);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipGetLastError());
    const float ms = time_ms(e0, e1);
    CHECK(hipMemcpy(h, clk, sizeof h, hipMemcpyDeviceToHost));
    const double bytes = 8.0 * 1024 * iters * 8 * blocks;
    const double mhz = h[0] / (h[1] / 100.0);
    std::printf("lds_read  b128     %8.1f TB/s    clock %5.0f MHz  %.0f B/clk per CU; one wave alone %.1f B/clk\n",
                bytes / ms / 1e9, mhz, bytes / (ms * 1e-3) / (mhz * 1e6) / cus, 8.0 * 1024 * iters / h[0]);
    CHECK(hipFree(out));
  }

  // HBM: copy 1 GiB
  {
    const size_t bytes = (size_t)1 << 30, n = bytes / 16;
    u32x4 *src, *dst;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMalloc(&dst, bytes));
    CHECK(hipMemset(src, 1, bytes));
    const int blocks = 8 * cus;
    hipLaunchKernelGGL(copy_probe, dim3(blocks), dim3(256), 0, 0, src, dst, n);
    CHECK(hipDeviceSynchronize());
    float best = 1e30f;
    for (int rep = 0; rep < 5; ++rep) {
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(copy_probe, dim3(blocks), dim3(256), 0, 0, src, dst, n);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipGetLastError());
      const float ms = time_ms(e0, e1);
      if (ms < best) best = ms;
    }
    std::printf("hbm_copy  1 GiB    %8.1f GB/s   (read + write bytes over the best of 5 copies)\n",
                2.0 * bytes / (best * 1e-3) / 1e9);
    // the other streams, best of 5 each; the grid divides n evenly
    unsigned* sink;
    CHECK(hipMalloc(&sink, sizeof(unsigned) * 256 * (size_t)blocks));
    auto best_of = [&](auto launch) {
      launch();
      CHECK(hipDeviceSynchronize());
      float b = 1e30f;
      for (int rep = 0; rep < 5; ++rep) {
        CHECK(hipEventRecord(e0));
        launch();
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipGetLastError());
        const float ms = time_ms(e0, e1);
        if (ms < b) b = ms;
      }
      return b;
    };
    if (n % (4 * 256 * (size_t)blocks) != 0) {
      std::fprintf(stderr, "grid does not divide the buffer\n");
      std::exit(1);
    }
    const float t4 = best_of([&] { hipLaunchKernelGGL(copy4_probe, dim3(blocks), dim3(256), 0, 0, src, dst, n); });
    std::printf("hbm_copy4 1 GiB    %8.1f GB/s   (4 loads in flight per lane, non-temporal stores)\n",
                2.0 * bytes / (t4 * 1e-3) / 1e9);
    const float tr = best_of([&] { hipLaunchKernelGGL(read_probe, dim3(blocks), dim3(256), 0, 0, src, sink, n); });
    std::printf("hbm_read  1 GiB    %8.1f GB/s   (read only, 4 loads in flight per lane)\n",
                1.0 * bytes / (tr * 1e-3) / 1e9);
    const float tw = best_of([&] { hipLaunchKernelGGL(write_probe, dim3(blocks), dim3(256), 0, 0, dst, n); });
    std::printf("hbm_write 1 GiB    %8.1f GB/s   (write only, non-temporal stores)\n",
                1.0 * bytes / (tw * 1e-3) / 1e9);
    CHECK(hipFree(sink));
    CHECK(hipFree(src));
    CHECK(hipFree(dst));
  }
  CHECK(hipFree(clk));
  return 0;
}
