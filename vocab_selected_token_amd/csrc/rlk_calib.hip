// rlk_calib -- stream ceilings of the GPU it runs on, for the benchmark's report.
//
// Three streams over 8 GiB buffers, each lane moving 16 bytes per instruction so
// that a wave instruction covers 1 KB contiguous (the access shape of the
// library's streaming kernels):
//   read   loads with the nontemporal hint (as stage 1 loads the logits)
//   write  stores with the nontemporal hint (as the backward stores dX)
//   copy   the two together, read and written in equal amounts
// and two copies of 32768 rows of 305,152 bytes (152576 bf16 columns), the
// shapes a forward+backward that reads every logit once and writes every dX
// once can take, with no arithmetic:
//   row_copy    one 512-thread block per row reads it and writes it back out
//               (the shape of a schedule in which one block owns a row);
//   slice_copy  a block reads one sixteenth of a row, then re-reads the same
//               sixteenth of the row two rows back (read by a block on its own
//               XCD, so it comes from that XCD's L2) and writes it out: the
//               traffic of a schedule whose blocks share rows, without the
//               synchronisation such a schedule needs.
// Each runs 7 times after one warm-up; the median is printed as one JSON line,
// in GB/s (1e9 bytes; the row shapes count one read and one write of every
// byte).  The program allocates its own buffers and frees them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256, kPer = 4;  // 16 KB per block
constexpr int kNt = 2;                   // cache-policy bits: nontemporal

__global__ __launch_bounds__(kThreads) void stream_read(const char* p, uint32_t* sink) {
  const uint64_t off = (uint64_t)blockIdx.x * kThreads * kPer * 16;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p + off), 0, kThreads * kPer * 16,
                                                     0x00020000);
  u32x4 q[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    q[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * kThreads + threadIdx.x) * 16, 0, kNt);
  u32x4 acc = q[0] ^ q[1] ^ q[2] ^ q[3];
  // the loads must stay: a store that never happens for the buffers used here
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

__global__ __launch_bounds__(kThreads) void stream_write(char* p) {
  const uint64_t off = (uint64_t)blockIdx.x * kThreads * kPer * 16;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(p + off, 0, kThreads * kPer * 16, 0x00020000);
  const u32x4 v = {threadIdx.x, blockIdx.x, 1u, 2u};
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (k * kThreads + threadIdx.x) * 16, 0, kNt);
}

__global__ __launch_bounds__(kThreads) void stream_copy(const char* src, char* dst) {
  const uint64_t off = (uint64_t)blockIdx.x * kThreads * kPer * 16;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + off), 0, kThreads * kPer * 16,
                                                     0x00020000);
  const auto ws = __builtin_amdgcn_make_buffer_rsrc(dst + off, 0, kThreads * kPer * 16, 0x00020000);
  u32x4 q[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    q[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * kThreads + threadIdx.x) * 16, 0, kNt);
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(q[k], ws, (k * kThreads + threadIdx.x) * 16, 0, kNt);
}

constexpr int64_t kRows = 32768;
constexpr int64_t kRowChunks = 19072;  // 16-byte chunks per 152576-column bf16 row

__global__ __launch_bounds__(512) void row_copy(const u32x4* __restrict__ src,
                                                u32x4* __restrict__ dst) {
  const u32x4* r = src + (int64_t)blockIdx.x * kRowChunks;
  u32x4* w = dst + (int64_t)blockIdx.x * kRowChunks;
  for (int c0 = threadIdx.x; c0 < kRowChunks; c0 += 512 * 4) {
    u32x4 q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (c0 + k * 512 < kRowChunks) q[k] = __builtin_nontemporal_load(r + c0 + k * 512);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (c0 + k * 512 < kRowChunks) __builtin_nontemporal_store(q[k], w + c0 + k * 512);
  }
}

constexpr int kSlices = 16, kSliceBack = 2;  // 2 * 16 blocks back: the same XCD
constexpr int kSliceChunks = (kRowChunks + kSlices - 1) / kSlices;

__global__ __launch_bounds__(256) void slice_copy(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, uint32_t* sink) {
  const int64_t t = blockIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (t < kRows * kSlices) {  // this unit's first read
    const u32x4* p = src + (t / kSlices) * kRowChunks;
    const int c1 = min((int)kRowChunks, (int)(t % kSlices + 1) * kSliceChunks);
    for (int c = (int)(t % kSlices) * kSliceChunks + threadIdx.x; c < c1; c += 256 * 4) {
      u32x4 q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = c + k * 256 < c1 ? p[c + k * 256] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= q[k];
    }
  }
  const int64_t u = t - (int64_t)kSliceBack * kSlices;
  if (u >= 0 && u < kRows * kSlices) {  // the unit read two rows back: read again, write out
    const u32x4* p = src + (u / kSlices) * kRowChunks;
    u32x4* w = dst + (u / kSlices) * kRowChunks;
    const int c1 = min((int)kRowChunks, (int)(u % kSlices + 1) * kSliceChunks);
    for (int c = (int)(u % kSlices) * kSliceChunks + threadIdx.x; c < c1; c += 256 * 4) {
      u32x4 q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k * 256 < c1) q[k] = p[c + k * 256];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k * 256 < c1) __builtin_nontemporal_store(q[k], w + c + k * 256);
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[1] = 1u;
}

template <typename F>
float median_ms(F launch, hipEvent_t a, hipEvent_t b) {
  launch();
  if (hipDeviceSynchronize() != hipSuccess) return -1.0f;
  std::vector<float> t;
  for (int i = 0; i < 7; ++i) {
    if (hipEventRecord(a) != hipSuccess) return -1.0f;
    launch();
    if (hipEventRecord(b) != hipSuccess || hipEventSynchronize(b) != hipSuccess) return -1.0f;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return -1.0f;
    t.push_back(ms);
  }
  std::sort(t.begin(), t.end());
  return t[t.size() / 2];
}

}  // namespace

int main() {
  const size_t bytes = size_t{8} << 30;
  const size_t row_bytes = (size_t)kRows * kRowChunks * 16;  // 10.0 GB; the buffers hold it
  const size_t per_block = size_t{kThreads} * kPer * 16;
  const unsigned blocks = (unsigned)(bytes / per_block);  // 524288 blocks of 256 threads
  char *a = nullptr, *b = nullptr;
  uint32_t* sink = nullptr;
  if (hipMalloc(&a, row_bytes) != hipSuccess || hipMalloc(&b, row_bytes) != hipSuccess ||
      hipMalloc(&sink, 64) != hipSuccess) {
    fprintf(stderr, "rlk_calib: could not allocate 2 x 10 GB\n");
    return 1;
  }
  if (hipMemset(a, 1, row_bytes) != hipSuccess || hipMemset(b, 2, row_bytes) != hipSuccess)
    return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  const float t_read = median_ms([&] { stream_read<<<blocks, kThreads>>>(a, sink); }, e0, e1);
  const float t_write = median_ms([&] { stream_write<<<blocks, kThreads>>>(a); }, e0, e1);
  // the copy moves 4 GiB each way, so its rate counts 8 GiB like the others
  const float t_copy = median_ms([&] { stream_copy<<<blocks / 2, kThreads>>>(a, b); }, e0, e1);
  const u32x4* ra = reinterpret_cast<const u32x4*>(a);
  u32x4* rb = reinterpret_cast<u32x4*>(b);
  const float t_row = median_ms([&] { row_copy<<<(unsigned)kRows, 512>>>(ra, rb); }, e0, e1);
  const float t_slice = median_ms(
      [&] {
        slice_copy<<<(unsigned)((kRows + kSliceBack) * kSlices), 256>>>(ra, rb, sink);
      },
      e0, e1);
  const hipError_t err = hipGetLastError();
  (void)hipEventDestroy(e0);  // clean-up; the process ends next
  (void)hipEventDestroy(e1);
  (void)hipFree(a);
  (void)hipFree(b);
  (void)hipFree(sink);
  if (err != hipSuccess || t_read <= 0.0f || t_write <= 0.0f || t_copy <= 0.0f ||
      t_row <= 0.0f || t_slice <= 0.0f) {
    fprintf(stderr, "rlk_calib: %s\n", hipGetErrorString(err));
    return 1;
  }
  const double gb = bytes / 1e9;
  const double rgb = 2.0 * row_bytes / 1e9;
  printf("{\"read_GBps\": %.1f, \"write_GBps\": %.1f, \"copy_GBps\": %.1f, "
         "\"row_copy_GBps\": %.1f, \"slice_copy_GBps\": %.1f}\n",
         gb / t_read * 1e3, gb / t_write * 1e3, gb / t_copy * 1e3, rgb / t_row * 1e3,
         rgb / t_slice * 1e3);
  return 0;
}
