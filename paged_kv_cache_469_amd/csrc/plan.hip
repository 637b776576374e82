// Segment classification and work lists ("vLLM 学习笔记 01", section 1.6:
// the attention operator is told where each segment of the packed batch
// starts and ends; section 1.4: each request catches up from its computed
// tokens to its total, one token for a decode, many for a prefill or chunk).
//
// One workgroup of 1024 threads walks the segments on the device, so the
// host never reads metadata and the whole call can be captured in a graph:
//   n == 1 -> decode: ceil(L / P) items (segment, partition)
//   n >  1 -> prefill: ceil(n / QT) items (segment, query tile), the tile
//             with the most keys (the last) first
//   n == 0 -> nothing
// Segments whose bounds are out of range are skipped and flagged.  It also
// resets the status word and the dynamic-scheduling counters the attention
// kernels use, so the workspace needs no clearing between calls.
#include "kernels.hpp"

namespace pkv {

// Exclusive prefix sum over the 1024 threads of the block; returns the
// thread's offset and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[16] = run;
  }
  __syncthreads();
  const int res = scratch[wave] + x - v;
  *total = scratch[16];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(1024) plan_kernel(PlanParams p) {
  __shared__ int scratch[17];
  int dec_base = 0;
  int pre_base = 0;
  uint32_t status = 0;
  for (int base = 0; base < p.num_seqs; base += 1024) {
    const int s = base + (int)threadIdx.x;
    int nd = 0, np = 0, L = 0, n = 0;
    if (s < p.num_seqs) {
      const int c0 = p.cu[s];
      const int c1 = p.cu[s + 1];
      L = p.lens[s];
      n = c1 - c0;
      const bool ok = c0 >= 0 && c1 <= p.num_tokens && n >= 0 && L >= n && L <= p.max_len;
      if (!ok) {
        status |= 1u;
      } else if (n == 1) {
        nd = (L + p.part_tokens - 1) / p.part_tokens;
      } else if (n > 1) {
        np = (n + p.query_tile - 1) / p.query_tile;
      }
    }
    int tot_d, tot_p;
    const int od = dec_base + block_exclusive_scan(nd, scratch, &tot_d);
    const int op = pre_base + block_exclusive_scan(np, scratch, &tot_p);
    // overlapping segments (only possible when some segment is malformed)
    // could overflow the lists: items past the capacity are dropped and flagged
    for (int i = 0; i < nd; ++i)
      if (od + i < p.decode_cap) p.decode_items[od + i] = make_int2(s, i);
    for (int i = 0; i < np; ++i)
      if (op + i < p.prefill_cap) p.prefill_items[op + i] = make_int2(s, np - 1 - i);
    if (od + nd > p.decode_cap || op + np > p.prefill_cap) status |= 1u;
    dec_base += tot_d;
    pre_base += tot_p;
  }
  const int any_bad = __syncthreads_or((int)status);
  if (threadIdx.x == 0) {
    p.hdr->status = any_bad ? 1u : 0u;
    p.hdr->n_decode = min(dec_base, p.decode_cap);
    p.hdr->n_prefill = min(pre_base, p.prefill_cap);
    p.hdr->decode_next = 0;
    p.hdr->prefill_next = 0;
  }
}

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  plan_kernel<<<1, 1024, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pkv
