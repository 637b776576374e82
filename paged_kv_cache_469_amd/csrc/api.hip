// Host side of the C ABI declared in include/paged_attn.h: argument checks,
// workspace layout, work-split choices and kernel launches.  No entry point
// allocates memory, reads device memory or synchronises, except the two debug
// calls that say so (paged_validate, paged_attention_device_status).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/paged_attn.h"
#include "kernels.hpp"

using namespace pkv;

namespace {

// Message of the last failing call on this thread (a fixed buffer: setting it
// allocates nothing).
thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_stage_events[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
thread_local bool g_stage_on = false;

hipError_t stage(int i, hipStream_t stream) {
  return g_stage_on && g_stage_events[i] ? hipEventRecord(g_stage_events[i], stream) : hipSuccess;
}
// Tuning knobs of the calling thread (set by the paged_attention_set_* calls):
// one thread's measurement setting never changes another caller's work split.
thread_local int32_t g_part_tokens = 0;     // 0: automatic
thread_local int32_t g_group_members = 0;   // 0: automatic, 1: no shared-prefix groups

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(PAGED_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kQueryTileMin = 32;   // smallest prefill query tile (heads_per_item = 4)

// Segments with at most this many new tokens take the split-context decode
// path: their n * G query rows must fit its at most two 16-column tiles, and
// n stays within the few tokens of a speculative-decoding check.
int32_t max_decode_tokens(int32_t group) { return std::min(8, 32 / std::max(1, group)); }

// Most members of a shared-prefix group: the group's query rows (members * G)
// fill at most two 16-row column tiles of the decode kernel.
int32_t group_members(int32_t group) {
  const int32_t cap = std::min(8, 32 / std::max(1, group));
  const int32_t forced = g_group_members;
  return forced > 0 ? std::min(cap, forced) : cap;
}

// Tokens per decode partition.  Automatic choice: the largest of 1024 .. 64
// that still gives at least 8192 wave-sized items for the longest allowed
// context (the items then outnumber the chip's resident waves several times,
// so the dynamic queue balances the tail); long partitions keep the merge's
// extra traffic, about G * (D + 2) * 8 bytes per partition, under 2 %.  2048
// when that still gives 16384 items (long contexts): an item's start (its
// queries, block ids and first K/V latency) and the partials are then paid
// half as often, and twice the items keep the tail of the longer ones short.
int32_t partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks) {
  const int32_t forced = g_part_tokens;
  if (forced > 0) return forced;
  const int64_t max_len = (int64_t)max_blocks * kBlock;
  const auto items = [&](int32_t p) {
    return (int64_t)num_seqs * num_kv_heads * ((max_len + p - 1) / p);
  };
  if (items(2048) >= 16384) return 2048;
  for (int32_t p : {1024, 512, 256, 128}) {
    if (items(p) >= 8192) return p;
  }
  return 64;
}

struct Layout {
  int32_t part_tokens = 0;
  int32_t pmax = 0;
  int64_t decode_cap = 0;
  int64_t prefill_cap = 0;
  int64_t rows_cap = 0;   // partial rows: one per new token of a decode segment
  int64_t group_cap = 0;  // shared-prefix group items: each replaces two or more decode items
  size_t decode_items = 0, prefill_items = 0, seg_row = 0, group_items = 0, part_ml = 0,
         part_o = 0, total = 0;
};

Layout layout(int32_t num_seqs, int32_t num_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
              int32_t max_blocks) {
  Layout l;
  l.part_tokens = partition_tokens(num_seqs, hkv, max_blocks);
  const int64_t max_len = (int64_t)max_blocks * kBlock;
  l.pmax = (int32_t)std::max<int64_t>(1, (max_len + l.part_tokens - 1) / l.part_tokens);
  l.decode_cap = (int64_t)num_seqs * l.pmax;
  l.prefill_cap = (num_tokens + kQueryTileMin - 1) / kQueryTileMin + (int64_t)num_seqs;
  // decode segments hold at most max_decode_tokens new tokens each, and all
  // of them together at most num_tokens
  l.rows_cap = std::min<int64_t>(num_tokens, (int64_t)num_seqs * max_decode_tokens(hq / hkv));
  size_t off = sizeof(WsHeader);
  l.decode_items = off;
  off = align256(off + (size_t)l.decode_cap * sizeof(int2));
  l.prefill_items = off;
  off = align256(off + (size_t)l.prefill_cap * sizeof(pkv::PrefillItem));
  l.seg_row = off;
  off = align256(off + (size_t)num_seqs * sizeof(int32_t));
  l.group_cap = l.decode_cap / 2 + 1;
  l.group_items = off;
  off = align256(off + (size_t)l.group_cap * sizeof(pkv::GroupItem));
  l.part_ml = off;
  off = align256(off + (size_t)l.rows_cap * l.pmax * hq * sizeof(float2));
  l.part_o = off;
  off = align256(off + (size_t)l.rows_cap * l.pmax * hq * head_dim * sizeof(uint16_t));
  l.total = off;
  return l;
}

struct DeviceInfo {
  int cus = 0;
  int decode_wg[2] = {0, 0};    // resident 256-thread workgroups per CU, D = 64 / 128
  int prefill_wg[2] = {0, 0};
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];   // filled on the first call on each device

hipError_t device_info(DeviceInfo& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (d.cus == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    for (int i = 0; i < 2; ++i) {
      const int hd = i ? 128 : 64;
      int nb = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_kernel_ptr(hd), 256, 0);
      if (e != hipSuccess) return e;
      d.decode_wg[i] = std::max(1, nb);
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, prefill_kernel_ptr(hd), 512, 0);
      if (e != hipSuccess) return e;
      d.prefill_wg[i] = std::max(1, nb);
    }
    d.cus = cus;
  }
  out = d;
  return hipSuccess;
}

bool supported_dims(int32_t hq, int32_t hkv, int32_t head_dim, int* code) {
  if (hq <= 0 || hkv <= 0 || head_dim <= 0 || hq % hkv) {
    *code = fail(PAGED_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                 hq, hkv);
    return false;
  }
  if (head_dim != 64 && head_dim != 128) {
    *code = fail(PAGED_EUNSUPPORTED, "head_dim %d is not built (64 or 128)", head_dim);
    return false;
  }
  if (hq / hkv > 16) {
    *code = fail(PAGED_EUNSUPPORTED, "query heads per KV head %d > 16 is not built", hq / hkv);
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

size_t paged_kv_block_bytes(int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype_bytes) {
  if (block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || dtype_bytes <= 0) return 0;
  return (size_t)2 * block_size * num_kv_heads * head_dim * dtype_bytes;
}

int paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping, void* kv_cache,
                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_blocks, int64_t k_token_stride, int64_t v_token_stride,
                   hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0)
    return fail(PAGED_EINVAL, "paged_kv_write: negative or zero size");
  if (num_tokens == 0) return PAGED_OK;
  if (!k || !v || !slot_mapping || !kv_cache)
    return fail(PAGED_EINVAL, "paged_kv_write: null pointer");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(PAGED_EINVAL, "paged_kv_write: token stride below num_kv_heads * head_dim");
  hipError_t e = launch_kv_write(k, v, slot_mapping, kv_cache, num_tokens, num_kv_heads,
                                 head_dim, num_blocks, k_token_stride, v_token_stride, stream);
  if (e != hipSuccess) return fail_hip(e, "paged_kv_write launch");
  return PAGED_OK;
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_blocks_per_seq < 0)
    return 0;
  return layout(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq)
      .total;
}

}  // extern "C"

namespace {

// Both attention entry points: argument checks, plan, decode, merge and
// prefill launches over the given workspace (`who` names the entry point in
// messages).
int attention_impl(const char* who, const void* q, const void* kv_cache,
                   const int32_t* block_tables, const int32_t* cu_seqlens_q,
                   const int32_t* seq_lens, float scale, void* out, int32_t num_seqs,
                   int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                   int64_t q_token_stride, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  int code = 0;
  if (num_seqs < 0 || num_tokens < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(PAGED_EINVAL, "%s: negative size", who);
  if (!supported_dims(num_q_heads, num_kv_heads, head_dim, &code)) return code;
  if (num_seqs == 0 || num_tokens == 0) return PAGED_OK;
  if (!q || !kv_cache || !block_tables || !cu_seqlens_q || !seq_lens || !out || !workspace)
    return fail(PAGED_EINVAL, "%s: null pointer", who);
  if (q_token_stride < (int64_t)num_q_heads * head_dim || q_token_stride % 8)
    return fail(PAGED_EINVAL, "%s: q_token_stride must be >= Hq * D and a multiple of 8", who);
  if ((uintptr_t)q % 16 || (uintptr_t)kv_cache % 16 || (uintptr_t)out % 16 ||
      (uintptr_t)workspace % 256)
    return fail(PAGED_EINVAL, "%s: q/kv_cache/out need 16-byte and workspace "
                              "256-byte alignment", who);
  if ((int64_t)max_blocks_per_seq * kBlock > INT32_MAX / 2)
    return fail(PAGED_EINVAL, "%s: max_blocks_per_seq too large", who);
  if (!(scale == scale) || std::isinf(scale))
    return fail(PAGED_EINVAL, "%s: scale must be finite", who);
  const Layout l = layout(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                          max_blocks_per_seq);
  // the plan kernel sums up to 1024 per-segment item counts of at most
  // prefill_cap + 1 each in 32-bit integers
  if (l.decode_cap > INT32_MAX / 64 || l.prefill_cap >= (1 << 20) || l.rows_cap > INT32_MAX / 64)
    return fail(PAGED_EINVAL, "%s: too many work items", who);
  if (workspace_bytes < l.total)
    return fail(PAGED_EINVAL, "%s: workspace of %zu bytes, %zu needed", who,
                workspace_bytes, l.total);
  DeviceInfo dev;
  hipError_t e = device_info(dev);
  if (e != hipSuccess) return fail_hip(e, "device query");

  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  const int group = num_q_heads / num_kv_heads;
  // prefill: 8 waves of 32 queries; the heads of one item share the KV head
  const int heads_per_item = group % 8 == 0 ? 8 : (group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1));
  const int query_tile = 32 * (8 / heads_per_item);
  const float scale_log2 = scale * 1.4426950408889634f;

  PlanParams pp{};
  pp.cu = cu_seqlens_q;
  pp.lens = seq_lens;
  pp.bt = block_tables;
  pp.hdr = hdr;
  pp.decode_items = reinterpret_cast<int2*>(ws + l.decode_items);
  pp.prefill_items = reinterpret_cast<pkv::PrefillItem*>(ws + l.prefill_items);
  pp.num_seqs = num_seqs;
  pp.num_tokens = num_tokens;
  pp.width = max_blocks_per_seq;
  pp.max_len = max_blocks_per_seq * kBlock;
  pp.part_tokens = l.part_tokens;
  // automatic choice of 1024 keys: the plan doubles it when no shared-prefix
  // group can form (the workspace for 1024 holds the partials of 2048)
  pp.part_double = (g_part_tokens == 0 && l.part_tokens == 1024) ? 1 : 0;
  pp.query_tile = query_tile;
  pp.decode_cap = (int32_t)l.decode_cap;
  pp.prefill_cap = (int32_t)l.prefill_cap;
  pp.seg_row = reinterpret_cast<int32_t*>(ws + l.seg_row);
  pp.max_decode_n = max_decode_tokens(group);
  pp.rows_cap = (int32_t)l.rows_cap;
  pp.group_items = reinterpret_cast<pkv::GroupItem*>(ws + l.group_items);
  pp.group_cap = (int32_t)l.group_cap;
  pp.group_max = group_members(group);
  e = stage(0, stream);
  if (e == hipSuccess) e = launch_plan(pp, stream);
  if (e == hipSuccess) e = stage(1, stream);
  if (e != hipSuccess) return fail_hip(e, "plan launch");

  const int di = head_dim == 128 ? 1 : 0;
  DecodeParams dp{};
  dp.q = static_cast<const uint16_t*>(q);
  dp.cache = static_cast<const uint16_t*>(kv_cache);
  dp.bt = block_tables;
  dp.cu = cu_seqlens_q;
  dp.lens = seq_lens;
  dp.out = static_cast<uint16_t*>(out);
  dp.part_o = reinterpret_cast<uint16_t*>(ws + l.part_o);
  dp.part_ml = reinterpret_cast<float2*>(ws + l.part_ml);
  dp.hdr = hdr;
  dp.items = pp.decode_items;
  dp.groups = pp.group_items;
  dp.seg_row = pp.seg_row;
  dp.q_stride = q_token_stride;
  dp.num_blocks = num_blocks;
  dp.width = max_blocks_per_seq;
  dp.hq = num_q_heads;
  dp.hkv = num_kv_heads;
  dp.group = group;
  dp.part_tokens = l.part_tokens;
  dp.pmax = l.pmax;
  dp.scale_log2 = scale_log2;
  const int64_t decode_waves = l.decode_cap * num_kv_heads;
  const int decode_grid = (int)std::max<int64_t>(
      1, std::min<int64_t>((int64_t)dev.cus * dev.decode_wg[di], (decode_waves + 3) / 4));
  e = launch_decode(dp, head_dim, decode_grid, stream);
  if (e == hipSuccess) e = stage(2, stream);
  if (e == hipSuccess) e = launch_decode_merge(dp, head_dim, num_seqs, num_tokens, stream);
  if (e == hipSuccess) e = stage(3, stream);
  if (e != hipSuccess) return fail_hip(e, "decode launch");

  PrefillParams fp{};
  fp.q = dp.q;
  fp.cache = dp.cache;
  fp.bt = block_tables;
  fp.cu = cu_seqlens_q;
  fp.lens = seq_lens;
  fp.out = dp.out;
  fp.hdr = hdr;
  fp.items = pp.prefill_items;
  fp.q_stride = q_token_stride;
  fp.num_blocks = num_blocks;
  fp.width = max_blocks_per_seq;
  fp.hq = num_q_heads;
  fp.hkv = num_kv_heads;
  fp.group = group;
  fp.heads_per_item = heads_per_item;
  fp.head_chunks = group / heads_per_item;
  fp.query_tile = query_tile;
  // KV head g is served by the queue of XCD g % 8 (workgroup i runs on XCD
  // i % 8), so the workgroups reading one head's K/V share that XCD's L2
  fp.num_queues = num_kv_heads % kMaxQueues == 0 ? kMaxQueues : 1;
  // |scale| * log2(e), at least 1e-30 so masked logits (-inf) still map to 0
  fp.c = std::max(std::fabs(scale_log2), 1e-30f);
  fp.q_sign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const int64_t prefill_wgs = l.prefill_cap * num_kv_heads * fp.head_chunks;
  int64_t prefill_grid = std::min<int64_t>((int64_t)dev.cus * dev.prefill_wg[di], prefill_wgs);
  prefill_grid = std::max<int64_t>(fp.num_queues, prefill_grid / fp.num_queues * fp.num_queues);
  e = launch_prefill(fp, head_dim, (int)prefill_grid, stream);
  if (e == hipSuccess) e = stage(4, stream);
  if (e != hipSuccess) return fail_hip(e, "prefill launch");
  return PAGED_OK;
}


// Scratch of paged_attention_noalloc: one array per GPU (each device that
// loads the library holds its own copy until the process ends).  Host code
// never passes the array's name to a kernel: that is a host-side stand-in,
// not a device address.  The address of each device's copy comes from
// hipGetSymbolAddress with that device current, once, and is kept here.
constexpr size_t kScratchBytes = PAGED_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_ptr(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "paged_attention_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PAGED_EINVAL, "paged_attention_noalloc: device %d beyond the %d supported", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "paged_attention_noalloc: hipGetSymbolAddress");
    if (!p) return fail(PAGED_EHIP, "paged_attention_noalloc: no address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PAGED_OK;
}

}  // namespace

extern "C" {

int paged_attention(const void* q, const void* kv_cache, const int32_t* block_tables,
                    const int32_t* cu_seqlens_q, const int32_t* seq_lens, float scale, void* out,
                    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                    int32_t max_blocks_per_seq, int64_t q_token_stride, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return attention_impl("paged_attention", q, kv_cache, block_tables, cu_seqlens_q, seq_lens,
                        scale, out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                        num_blocks, max_blocks_per_seq, q_token_stride, workspace,
                        workspace_bytes, stream);
}

int paged_attention_noalloc(const void* q, const void* kv_cache, const int32_t* block_tables,
                            const int32_t* cu_seqlens_q, const int32_t* seq_lens, float scale,
                            void* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                            int32_t max_blocks_per_seq, int64_t q_token_stride,
                            hipStream_t stream) {
  if (num_seqs >= 0 && num_tokens >= 0 && num_q_heads > 0 && num_kv_heads > 0 && head_dim > 0 &&
      max_blocks_per_seq >= 0) {
    const size_t need = paged_attention_workspace_size(num_seqs, num_tokens, num_q_heads,
                                                       num_kv_heads, head_dim, max_blocks_per_seq);
    if (need > kScratchBytes)
      return fail(PAGED_EINVAL,
                  "paged_attention_noalloc: these shapes need %zu bytes of scratch, more than "
                  "the %zu the library holds per GPU (use paged_attention with a workspace)",
                  need, kScratchBytes);
  }
  void* ws = nullptr;
  if (num_seqs > 0 && num_tokens > 0) {
    const int code = scratch_ptr(&ws);
    if (code != PAGED_OK) return code;
  }
  return attention_impl("paged_attention_noalloc", q, kv_cache, block_tables, cu_seqlens_q,
                        seq_lens, scale, out, num_seqs, num_tokens, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, max_blocks_per_seq, q_token_stride, ws,
                        kScratchBytes, stream);
}

int paged_decode_advance(int32_t* seq_lens, int32_t* cu_seqlens_q, int32_t* slot_mapping,
                         const int32_t* block_tables, int32_t num_seqs,
                         int32_t max_blocks_per_seq, int64_t num_blocks, hipStream_t stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return fail(PAGED_EINVAL, "paged_decode_advance: negative size");
  if (!cu_seqlens_q) return fail(PAGED_EINVAL, "paged_decode_advance: null pointer");
  if (num_seqs > 0 && (!seq_lens || !slot_mapping || !block_tables))
    return fail(PAGED_EINVAL, "paged_decode_advance: null pointer");
  hipError_t e = launch_decode_advance(seq_lens, cu_seqlens_q, slot_mapping, block_tables,
                                       num_seqs, max_blocks_per_seq, num_blocks, stream);
  if (e != hipSuccess) return fail_hip(e, "paged_decode_advance launch");
  return PAGED_OK;
}

int paged_validate(const int32_t* slot_mapping, int32_t num_new_tokens,
                   const int32_t* block_tables, const int32_t* cu_seqlens_q,
                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_tokens,
                   int64_t num_blocks, int32_t max_blocks_per_seq, hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail_hip(e, "paged_validate sync");
  if (slot_mapping && num_new_tokens > 0) {
    std::vector<int32_t> slots(num_new_tokens);
    e = hipMemcpy(slots.data(), slot_mapping, slots.size() * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "paged_validate copy");
    std::vector<int32_t> live;
    for (int32_t t = 0; t < num_new_tokens; ++t) {
      const int32_t s = slots[t];
      if (s == -1) continue;
      if (s < 0 || (int64_t)s >= num_blocks * kBlock)
        return fail(PAGED_EINVAL, "slot_mapping[%d] = %d is outside the pool", t, s);
      live.push_back(s);
    }
    std::sort(live.begin(), live.end());
    for (size_t i = 1; i < live.size(); ++i)
      if (live[i] == live[i - 1])
        return fail(PAGED_EINVAL, "slot %d is written twice in one call", live[i]);
  }
  if (block_tables && num_seqs > 0) {
    if (!cu_seqlens_q || !seq_lens) return fail(PAGED_EINVAL, "paged_validate: null pointer");
    std::vector<int32_t> cu(num_seqs + 1), lens(num_seqs);
    std::vector<int32_t> bt((size_t)num_seqs * max_blocks_per_seq);
    e = hipMemcpy(cu.data(), cu_seqlens_q, cu.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess && !bt.empty())
      e = hipMemcpy(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "paged_validate copy");
    if (cu[0] != 0) return fail(PAGED_EINVAL, "cu_seqlens_q[0] = %d, not 0", cu[0]);
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t n = cu[s + 1] - cu[s];
      if (n < 0) return fail(PAGED_EINVAL, "cu_seqlens_q decreases at segment %d", s);
      if (cu[s + 1] > num_tokens)
        return fail(PAGED_EINVAL, "segment %d ends at row %d > num_tokens %d", s, cu[s + 1], num_tokens);
      if (lens[s] < n)
        return fail(PAGED_EINVAL, "segment %d: seq_len %d < new tokens %d", s, lens[s], n);
      if ((int64_t)lens[s] > (int64_t)max_blocks_per_seq * kBlock)
        return fail(PAGED_EINVAL, "segment %d: seq_len %d exceeds max_blocks_per_seq * 16", s, lens[s]);
      if (n == 0) continue;
      const int32_t nb = (lens[s] + kBlock - 1) / kBlock;
      for (int32_t b = 0; b < nb; ++b) {
        const int32_t id = bt[(size_t)s * max_blocks_per_seq + b];
        if (id < 0 || id >= num_blocks)
          return fail(PAGED_EINVAL, "block_tables[%d][%d] = %d is outside the pool", s, b, id);
      }
    }
  }
  return PAGED_OK;
}

int paged_attention_device_status(const void* workspace, uint32_t* status, hipStream_t stream) {
  if (!workspace || !status) return fail(PAGED_EINVAL, "paged_attention_device_status: null pointer");
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(status, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail_hip(e, "paged_attention_device_status");
  return PAGED_OK;
}

int paged_attention_set_partition_tokens(int32_t tokens) {
  if (tokens != 0 && (tokens < 32 || tokens > 2048 || tokens % 32))
    return fail(PAGED_EINVAL, "partition tokens must be 0 or a multiple of 32 in [32, 2048]");
  g_part_tokens = tokens;
  return PAGED_OK;
}

int paged_attention_set_group_members(int32_t members) {
  if (members < 0 || members > 8)
    return fail(PAGED_EINVAL, "group members must be in [0, 8] (0: automatic, 1: off)");
  g_group_members = members;
  return PAGED_OK;
}

int paged_attention_set_stage_events(void* const* events, int32_t count) {
  if (events == nullptr || count == 0) {
    g_stage_on = false;
    return PAGED_OK;
  }
  if (count != 5) return fail(PAGED_EINVAL, "stage events: count must be 0 or 5");
  bool any = false;
  for (int i = 0; i < 5; ++i) {
    g_stage_events[i] = static_cast<hipEvent_t>(events[i]);   // NULL: that point is not recorded
    any = any || events[i];
  }
  if (!any) return fail(PAGED_EINVAL, "stage events: all five are NULL");
  g_stage_on = true;
  return PAGED_OK;
}

const char* paged_last_error(void) { return g_last_error; }

}  // extern "C"
