// Shared device helpers for the gfx950 (CDNA4) kernels of this library.
//
// bf16 values travel as raw 16-bit patterns.  Widening is a 16-bit shift;
// narrowing uses the bf16 conversion of the compiler, which on gfx950 is the
// hardware convert with round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;  // tokens per KV block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define PKV_LDS __attribute__((address_space(3)))

// Workspace header: one 256-byte line at the start of the workspace, rewritten
// by the plan kernel on every call.
constexpr int kMaxQueues = 8;   // prefill work queues, one per XCD when the KV heads split evenly
struct WsHeader {
  uint32_t status;                  // PAGED_STATUS_* bits
  int32_t n_decode;                 // decode work items (segment, partition)
  int32_t n_prefill;                // prefill work items (segment, query tile)
  int32_t decode_next;              // dynamic scheduling counter of the decode kernel
  int32_t prefill_next[kMaxQueues]; // dynamic scheduling counters of the prefill kernel
  int32_t n_group;                  // shared-prefix group items (first segment, partition, members)
  int32_t part_tokens;              // decode partition size the plan chose for this call
  int32_t pad0[2];
  uint32_t zeros[16];               // 64 zero bytes: the source of K/V rows never loaded
  int32_t group_next[kMaxQueues];   // per-XCD queues of the decode kernel's group items
  int32_t pad1[24];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte line");

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16x16x32 bf16 MFMA: A is 16x32 (lane l holds row l%16, k = 8*(l/16)..+7),
// B is 32x16 (lane l holds column l%16, the same k), C/D is 16x16 (lane l
// holds column l%16, rows 4*(l/16)..+3).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA: A is 32x16 (lane l holds row l%32, k = 8*(l/32)..+7),
// B is 16x32 (column l%32, the same k), C/D is 32x32 (lane l holds column
// l%32; register r holds row 8*(r/4) + 4*(l/32) + r%4).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Pack the low (sel_hi = false) or high 16-bit halves of two words:
// result = { lo16 = half of `first`, hi16 = half of `second` }.
__device__ __forceinline__ uint32_t pick_halves(uint32_t first, uint32_t second, bool sel_hi) {
  return __builtin_amdgcn_perm(second, first, sel_hi ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace pkv
