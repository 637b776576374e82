// KV block write: scatter the new tokens' K/V rows into 16-token blocks
// through the slot mapping ("vLLM 学习笔记 01", section 1.6: each token's K/V
// goes to a given position of a given block; section 1.5: 16-slot blocks).
//
// HBM-bound bit copy.  One thread moves one 16-byte chunk of one token's K
// or V row; a token row (Hkv * D * 2 bytes, 2 KiB for 8 x 128) is read and
// written by consecutive lanes, so both sides are fully coalesced.  Slots out
// of the pool are skipped, never written.
#include "kernels.hpp"

namespace pkv {

__global__ void __launch_bounds__(256)
kv_write_vec_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const int32_t* __restrict__ slots, uint16_t* __restrict__ cache,
                    int32_t num_tokens, int32_t row_chunks, int64_t k_stride,
                    int64_t v_stride, int64_t num_slots) {
  const int64_t per_token = 2 * (int64_t)row_chunks;
  const int64_t total = (int64_t)num_tokens * per_token;
  const int64_t row_elems = (int64_t)row_chunks * 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int32_t rem = (int32_t)(i - t * per_token);
    const int32_t half = rem >= row_chunks;  // 0 = K, 1 = V
    const int32_t c = rem - half * row_chunks;
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const uint16_t* src = half ? v + t * v_stride : k + t * k_stride;
    const int64_t dst = (((s >> 4) * 2 + half) * kBlock + (s & 15)) * row_elems + (int64_t)c * 8;
    const u32x4 val = *reinterpret_cast<const u32x4*>(src + (int64_t)c * 8);
    *reinterpret_cast<u32x4*>(cache + dst) = val;
  }
}

// Element-wise fallback for rows or strides that are not 16-byte aligned.
__global__ void __launch_bounds__(256)
kv_write_elem_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     const int32_t* __restrict__ slots, uint16_t* __restrict__ cache,
                     int32_t num_tokens, int32_t row_elems, int64_t k_stride,
                     int64_t v_stride, int64_t num_slots) {
  const int64_t per_token = 2 * (int64_t)row_elems;
  const int64_t total = (int64_t)num_tokens * per_token;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int32_t rem = (int32_t)(i - t * per_token);
    const int32_t half = rem >= row_elems;
    const int32_t e = rem - half * row_elems;
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const uint16_t* src = half ? v + t * v_stride : k + t * k_stride;
    cache[(((s >> 4) * 2 + half) * kBlock + (s & 15)) * (int64_t)row_elems + e] = src[e];
  }
}

hipError_t launch_kv_write(const void* k, const void* v, const int32_t* slots, void* cache,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int64_t num_blocks, int64_t k_stride, int64_t v_stride,
                           hipStream_t stream) {
  const int32_t row_elems = num_kv_heads * head_dim;
  const int64_t num_slots = num_blocks * kBlock;
  const bool vec = (row_elems % 8 == 0) && (k_stride % 8 == 0) && (v_stride % 8 == 0) &&
                   ((uintptr_t)k % 16 == 0) && ((uintptr_t)v % 16 == 0) &&
                   ((uintptr_t)cache % 16 == 0);
  const int64_t work = (int64_t)num_tokens * 2 * (vec ? row_elems / 8 : row_elems);
  if (work == 0) return hipSuccess;
  const int64_t max_blocks = 256 * 64;
  const int blocks = (int)((work + 255) / 256 < max_blocks ? (work + 255) / 256 : max_blocks);
  if (vec) {
    kv_write_vec_kernel<<<blocks, 256, 0, stream>>>(
        (const uint16_t*)k, (const uint16_t*)v, slots, (uint16_t*)cache, num_tokens,
        row_elems / 8, k_stride, v_stride, num_slots);
  } else {
    kv_write_elem_kernel<<<blocks, 256, 0, stream>>>(
        (const uint16_t*)k, (const uint16_t*)v, slots, (uint16_t*)cache, num_tokens,
        row_elems, k_stride, v_stride, num_slots);
  }
  return hipGetLastError();
}

}  // namespace pkv
