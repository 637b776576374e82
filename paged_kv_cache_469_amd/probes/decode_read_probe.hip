// Read-pattern probe for the decode path: how fast can one GPU read a
// decode-shaped pool of scattered 16-token KV blocks, per way of reading?
//
// The pool holds 37,184 blocks of 64 KiB (K of 16 rows x 8 KV heads x 128
// bf16, then V of the same), the size of the 8B-shaped decode batch's pool,
// handed out in a seeded random order.  A work item is (64 consecutive blocks
// of the order, KV head g), one wave each, taken from an atomic queue, one
// wave per SIMD, as the decode kernel works; every byte of the pool is read
// once per launch.  The three kernels differ only in how a wave reads an
// item's 64 x 2 pieces of 16 rows x 256 bytes (K and V of head g):
//   direct   into registers as the decode kernel loads them: K as 16 rows x
//            64 bytes per load instruction (lane (m, j): row m, bytes 16j +
//            64 sl), V as 4 rows x 256 bytes; the loads of the next 32 keys
//            are issued before the current ones are consumed;
//   staged   whole 256-byte rows (4 rows per instruction) copied straight
//            into a two-stage LDS ring per wave (global -> LDS, no
//            registers), the next 32 keys' copies issued before the current
//            ones are read back from LDS in the K operand layout;
//   blocks   each of 8 whole 64 KiB blocks read contiguously (the pattern a
//            plain stream of the pool would use: an upper bound).
// Consuming the data is an XOR into one register per lane (no arithmetic
// that could limit the rate).  Prints the GB/s of each kernel (median of 9
// launches after one warm-up); run it under rocprofv3 --kernel-trace --stats
// for the per-kernel durations.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                       \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);       \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

namespace {

constexpr int kBlocks = 37184;        // a multiple of 64
constexpr int kHeads = 8;
constexpr int kRowBytes = 2048;       // one token's K (or V) row of all heads
constexpr int kHalf = 16 * kRowBytes; // K half of a block; V half follows
constexpr int kBlockBytes = 2 * kHalf;
constexpr int kPerItem = 64;          // blocks of one item
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ int next_item(int* ctr, int lane) {
  int it = 0;
  if (lane == 0) it = atomicAdd(ctr, 1);
  return __builtin_amdgcn_readfirstlane(__shfl(it, 0));
}

// direct: lane (m, j) loads K row m, 16 bytes at 16j + 64 sl (sl = 0..3), and
// V rows 4j .. 4j+3, 16 bytes at 16m; two blocks (32 keys) per stage
__global__ void __launch_bounds__(256) direct(const char* pool, const int* order, int nitems,
                                              int* ctr, u32x4* sink) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, j = lane >> 4;
  u32x4 acc = {0, 0, 0, 0};
  for (;;) {
    const int it = next_item(ctr, lane);
    if (it >= nitems) break;
    const int g = it % kHeads, part = it / kHeads;
    u32x4 a[16], b[16];
    auto load = [&](u32x4 (&r)[16], int pair) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const char* blk = pool + (size_t)order[part * kPerItem + 2 * pair + x] * kBlockBytes + g * 256;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          r[8 * x + sl] = *(const u32x4*)(blk + m * kRowBytes + 16 * j + 64 * sl);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          r[8 * x + 4 + rr] = *(const u32x4*)(blk + kHalf + (4 * j + rr) * kRowBytes + 16 * m);
      }
    };
    load(a, 0);
    for (int pair = 0; pair < kPerItem / 2; pair += 2) {
      load(b, pair + 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc ^= a[i];
      if (pair + 2 < kPerItem / 2) load(a, pair + 2);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc ^= b[i];
    }
  }
  if (acc.x == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// staged: per wave a ring of two 16 KiB stages; a stage is 32 keys: for each
// of two blocks, its 16 K rows then its 16 V rows of head g (256 bytes each),
// 4 rows per copy instruction (lane i's 16 bytes land at M0 + 16 i)
__device__ __forceinline__ void copy_pair(const char* pool, const int* order, int part, int pair,
                                          int g, int lane, uint32_t lds_stage) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const uint64_t base = (uint64_t)(pool + (size_t)order[part * kPerItem + 2 * pair + x] * kBlockBytes);
    const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xffffu)),
                      (uint32_t)kBlockBytes, (uint32_t)kRsrcWord3};
#pragma unroll
    for (int h = 0; h < 2; ++h) {          // K half, then V half
      const uint32_t off0 = h * kHalf + g * 256 + (lane >> 4) * kRowBytes + 16 * (lane & 15);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_stage + (2 * x + h) * 4096);
      asm volatile(
          "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds"
          :: "s"(dst), "v"(off0), "v"(off0 + 4 * kRowBytes), "v"(off0 + 8 * kRowBytes),
             "v"(off0 + 12 * kRowBytes), "s"(rs)
          : "memory", "scc");
    }
  }
}

__global__ void __launch_bounds__(256) staged(const char* pool, const int* order, int nitems,
                                              int* ctr, u32x4* sink) {
  __shared__ __attribute__((aligned(1024))) char ring[4][2][16384];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: an SGPR
  const int m = lane & 15, j = lane >> 4;
  u32x4 acc = {0, 0, 0, 0};
  for (;;) {
    const int it = next_item(ctr, lane);
    if (it >= nitems) break;
    const int g = it % kHeads, part = it / kHeads;
    copy_pair(pool, order, part, 0, g, lane, (uint32_t)(uintptr_t)ring[wave][0]);
    for (int pair = 0; pair < kPerItem / 2; ++pair) {
      if (pair + 1 < kPerItem / 2) {
        // the reads of the stage about to be overwritten returned when they
        // were consumed (the XOR below used them)
        copy_pair(pool, order, part, pair + 1, g, lane, (uint32_t)(uintptr_t)ring[wave][(pair + 1) & 1]);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // this stage landed, the next in flight
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      const char* st = ring[wave][pair & 1];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        // K in the operand layout of the decode kernel (row m, 16 bytes at
        // 16j + 64 sl), V rows 4j .. 4j+3 at 16m
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) acc ^= *(const u32x4*)(st + 2 * x * 4096 + m * 256 + 16 * j + 64 * sl);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc ^= *(const u32x4*)(st + (2 * x + 1) * 4096 + (4 * j + rr) * 256 + 16 * m);
      }
    }
  }
  if (acc.x == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// blocks: one wave reads 8 whole blocks, 1 KiB per instruction
__global__ void __launch_bounds__(256) blocks(const char* pool, const int* order, int nitems8,
                                              int* ctr, u32x4* sink) {
  const int lane = threadIdx.x & 63;
  u32x4 acc = {0, 0, 0, 0};
  for (;;) {
    const int it = next_item(ctr, lane);
    if (it >= nitems8) break;
    for (int b = 0; b < 8; ++b) {
      const char* blk = pool + (size_t)order[it * 8 + b] * kBlockBytes;
#pragma unroll 8
      for (int c = 0; c < kBlockBytes / 1024; ++c) acc ^= *(const u32x4*)(blk + c * 1024 + 16 * lane);
    }
  }
  if (acc.x == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  char* pool;
  int *order, *ctr;
  u32x4* sink;
  CHECK(hipMalloc(&pool, (size_t)kBlocks * kBlockBytes));
  CHECK(hipMemset(pool, 1, (size_t)kBlocks * kBlockBytes));
  std::vector<int> h(kBlocks);
  for (int i = 0; i < kBlocks; ++i) h[i] = i;
  std::shuffle(h.begin(), h.end(), std::mt19937(469));
  CHECK(hipMalloc(&order, kBlocks * sizeof(int)));
  CHECK(hipMemcpy(order, h.data(), kBlocks * sizeof(int), hipMemcpyHostToDevice));
  CHECK(hipMalloc(&ctr, sizeof(int)));
  CHECK(hipMalloc(&sink, (size_t)cus * 256 * sizeof(u32x4)));
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  const double bytes = (double)kBlocks * kBlockBytes;
  const int nitems = kBlocks / kPerItem * kHeads;
  const char* names[3] = {"direct", "staged", "blocks"};
  std::printf("pool %.3f GB in %d blocks of %d bytes, %d CUs, one 256-thread workgroup per CU\n",
              bytes / 1e9, kBlocks, kBlockBytes, cus);
  for (int k = 0; k < 3; ++k) {
    std::vector<float> ms;
    for (int rep = 0; rep < 10; ++rep) {
      CHECK(hipMemset(ctr, 0, sizeof(int)));
      CHECK(hipEventRecord(a));
      if (k == 0) direct<<<cus, 256>>>(pool, order, nitems, ctr, sink);
      else if (k == 1) staged<<<cus, 256>>>(pool, order, nitems, ctr, sink);
      else blocks<<<cus, 256>>>(pool, order, kBlocks / 8, ctr, sink);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(b));
      CHECK(hipEventSynchronize(b));
      float t = 0.f;
      CHECK(hipEventElapsedTime(&t, a, b));
      if (rep > 0) ms.push_back(t);
    }
    std::sort(ms.begin(), ms.end());
    const float med = ms[ms.size() / 2];
    std::printf("%-7s median %.1f us  %.0f GB/s  (%.1f %% of 8 TB/s), min %.1f us\n", names[k],
                1e3f * med, bytes / (med * 1e-3) / 1e9, bytes / (med * 1e-3) / 8e12 * 100, 1e3f * ms[0]);
  }
  CHECK(hipFree(pool));
  CHECK(hipFree(order));
  CHECK(hipFree(ctr));
  CHECK(hipFree(sink));
  return 0;
}
