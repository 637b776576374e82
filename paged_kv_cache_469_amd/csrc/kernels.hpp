// Kernel parameter blocks and launchers shared by the kernel sources and the
// host-side C ABI layer.
#pragma once

#include "common.hpp"

namespace pkv {

// One prefill work entry as the plan kernel leaves it: the segment, its
// query tile, and what the attention kernel needs before its first tile
// (the segment bounds and the block ids of keys 0..127).
struct PrefillItem {
  int32_t seq, qt;
  int32_t L;        // tokens in the sequence
  int32_t tok0;     // first new token in the packed batch
  int32_t n;        // new tokens of the segment
  int32_t pad[3];
  int32_t bid[8];   // block-table entries 0..7, clamped to the entries in use
};
static_assert(sizeof(PrefillItem) == 64, "one scalar load of 16 dwords");

// One shared-prefix group work entry: a partition that its members (single-
// token decode segments, listed in seg[0 .. nmem - 1]) all hold in the same
// blocks.
struct GroupItem {
  int32_t part, nmem;
  int32_t pad[2];
  int32_t seg[8];
};
static_assert(sizeof(GroupItem) == 48, "three 16-byte lines");

struct PlanParams {
  const int32_t* cu;
  const int32_t* lens;
  const int32_t* bt;
  WsHeader* hdr;
  int2* decode_items;
  PrefillItem* prefill_items;
  int32_t* seg_row;      // per segment: first partial row of a decode segment, else -1
  GroupItem* group_items;   // shared-prefix groups
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t width;         // block-table row length
  int32_t max_len;       // max_blocks_per_seq * 16
  int32_t part_tokens;   // P chosen by the host (the workspace is sized for it)
  int32_t part_double;   // 1: use 2P when no two decode segments share a first block
  int32_t query_tile;    // QT
  int32_t decode_cap;    // capacity of decode_items
  int32_t prefill_cap;   // capacity of prefill_items
  int32_t max_decode_n;  // segments with 1 <= n <= this take the decode path
  int32_t rows_cap;      // partial rows (one per new token of a decode segment)
  int32_t group_cap;     // capacity of group_items
  int32_t group_max;     // most members of a group (0 or 1: no grouping)
};

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* cache;
  const int32_t* bt;
  const int32_t* cu;
  const int32_t* lens;
  uint16_t* out;
  uint16_t* part_o;        // [rows, pmax, Hq, D] bf16: each partition's o / l
  float2* part_ml;         // [rows, pmax, Hq]  (running max in log2 units, sum)
  const int32_t* seg_row;  // per segment: its first partial row (token 0), -1 if not decode
  WsHeader* hdr;
  const int2* items;       // (segment, partition)
  const GroupItem* groups; // shared-prefix groups, taken before items
  int64_t q_stride;
  int64_t num_blocks;
  int32_t width;           // block table row length
  int32_t hq, hkv, group;
  int32_t part_tokens;     // P chosen by the host; the kernels use the plan's (header)
  int32_t pmax;
  float scale_log2;        // scale * log2(e)
};

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* cache;
  const int32_t* bt;
  const int32_t* cu;
  const int32_t* lens;
  uint16_t* out;
  WsHeader* hdr;
  const PrefillItem* items;   // most key tiles first
  int64_t q_stride;
  int64_t num_blocks;
  int32_t width;
  int32_t hq, hkv, group;
  int32_t heads_per_item;  // HW: query heads of one work item (1, 2 or 4), one per wave
  int32_t head_chunks;     // group / HW
  int32_t query_tile;      // QT = 64 * 4 / HW queries per work item
  int32_t num_queues;      // 8 (KV head g served by the XCD queue g % 8) or 1
  float c;                 // |scale| * log2(e)
  uint32_t q_sign;         // 0x80008000 when scale < 0 (queries negated), else 0
};

hipError_t launch_kv_write(const void* k, const void* v, const int32_t* slots, void* cache,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int64_t num_blocks, int64_t k_stride, int64_t v_stride,
                           hipStream_t stream);
hipError_t launch_plan(const PlanParams& p, hipStream_t stream);
hipError_t launch_decode_advance(int32_t* seq_lens, int32_t* cu, int32_t* slots, const int32_t* bt,
                                 int32_t num_seqs, int32_t width, int64_t num_blocks,
                                 hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int head_dim, int grid, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int num_seqs, int num_tokens,
                               hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int head_dim, int grid, hipStream_t stream);
const void* decode_kernel_ptr(int head_dim);
const void* prefill_kernel_ptr(int head_dim);

}  // namespace pkv
