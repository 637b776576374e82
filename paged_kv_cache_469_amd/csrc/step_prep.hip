// Device-side metadata of a steady-state decode step ("vLLM 学习笔记 01",
// section 1.4: a decode catches a request up by one token; section 1.6: the
// new token's K/V goes to a given position of a given block, and attention
// is told the segment bounds and each sequence's length).
//
// Every segment gains one new token at position L (its current length): the
// kernel sets seq_lens[s] = L + 1, cu_seqlens_q[s] = s (and [S] = S) and
// slot_mapping[s] = block_tables[s][L / 16] * 16 + L % 16, or -1 when that
// table entry is past the table or outside the pool (the write then skips
// the token and attention flags the block).  So a decode loop whose tables
// already hold the blocks of the coming positions needs no host metadata
// per step and can be captured in a graph once and replayed.
#include "kernels.hpp"

namespace pkv {

__global__ void __launch_bounds__(256)
decode_advance_kernel(int32_t* __restrict__ seq_lens, int32_t* __restrict__ cu,
                      int32_t* __restrict__ slots, const int32_t* __restrict__ bt,
                      int32_t num_seqs, int32_t width, int64_t num_blocks) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s == 0) cu[num_seqs] = num_seqs;
  if (s >= num_seqs) return;
  const int32_t pos = seq_lens[s];
  int32_t slot = -1;
  if (pos >= 0 && pos / kBlock < width) {
    const int32_t b = bt[(int64_t)s * width + pos / kBlock];
    if (b >= 0 && (int64_t)b < num_blocks) slot = b * kBlock + pos % kBlock;
  }
  slots[s] = slot;
  cu[s] = s;
  seq_lens[s] = pos + 1;
}

hipError_t launch_decode_advance(int32_t* seq_lens, int32_t* cu, int32_t* slots, const int32_t* bt,
                                 int32_t num_seqs, int32_t width, int64_t num_blocks,
                                 hipStream_t stream) {
  const int grid = (num_seqs + 1 + 255) / 256;
  decode_advance_kernel<<<grid, 256, 0, stream>>>(seq_lens, cu, slots, bt, num_seqs, width,
                                                  num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
