// Segment classification and work lists ("vLLM 学习笔记 01", section 1.6:
// the attention operator is told where each segment of the packed batch
// starts and ends; section 1.4: each request catches up from its computed
// tokens to its total, one token for a decode, many for a prefill or chunk).
//
// One workgroup of 1024 threads walks the segments on the device, so the
// host never reads metadata and the whole call can be captured in a graph:
//   1 <= n <= N_dec -> decode: ceil(L / P) items (segment, partition); the
//             segment's n tokens get n consecutive rows of partial results
//             (seg_row[s] is the first), n * G <= 32 query rows per KV head
//             (one decode step, or a few tokens of a speculative-decoding
//             check, over a long history); leading partitions shared with
//             neighbouring segments go to group items instead (pass 0)
//   n >  N_dec -> prefill: ceil(n / QT) items (segment, query tile), each
//             with the segment bounds and its first eight block ids
//   n == 0 -> nothing
// Both lists are ordered longest work first, so the dynamic queues hand out
// the long items first and the short ones fill the tail.  Prefill items go
// segment by segment, the segments by the number of 64-key tiles of their
// costliest (last) query tile (a counting sort over 1024 cost buckets), a
// segment's query tiles by decreasing cost: the workgroups of one XCD then
// work on one segment at a time and read its K/V through their L2 (with
// more than 1024 segments, items are sorted one by one by their own cost).
// Decode items go by their keys (full partitions first, then the partial
// last partitions of the segments by decreasing length, in 32-key buckets).
// Segments whose bounds are out of range are skipped and flagged.  The kernel also resets
// the status word and the dynamic-scheduling counters and writes the zero
// line of the header, so the workspace needs no clearing between calls.
#include "kernels.hpp"

namespace pkv {

constexpr int kCostBuckets = 1024;
constexpr int kPrefillTileKeys = 64;   // key tile of the prefill kernel

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

// Exclusive prefix sums of N values at once over the 1024 threads of the
// block, with one set of barriers for all of them: v[i] becomes the thread's
// offset of value i, tot[i] the block total.  scratch holds 17 * N ints.
template <int N>
__device__ void block_exclusive_scan_n(int (&v)[N], int (*scratch)[N], int (&tot)[N]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = v[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int y = __shfl_up(x[i], off);
      if (lane >= off) x[i] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) scratch[wave][i] = x[i];
  }
  __syncthreads();
  if ((int)threadIdx.x < N) {
    const int i = threadIdx.x;
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = scratch[w][i];
      scratch[w][i] = run;
      run += t;
    }
    scratch[16][i] = run;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    tot[i] = scratch[16][i];
    v[i] = scratch[wave][i] + x[i] - v[i];
  }
  __syncthreads();
}

// Inclusive maximum over the 1024 threads of the block.
__device__ int block_inclusive_max(int v, int* scratch) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x = max(x, y);
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = INT_MIN;
    for (int w = 0; w < 16; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run = max(run, t);
    }
  }
  __syncthreads();
  const int res = max(scratch[wave], x);
  __syncthreads();
  return res;
}

// Value of lane (lane ^ J) of the wave: a quad permutation (DPP) for J = 1
// and 2, a swizzle within 32 lanes for J = 4 .. 16, a permute for J = 32.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  } else if constexpr (J < 32) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (J << 10));   // and 31, xor J
  } else {
    return __shfl_xor(x, J);
  }
}

// One compare-exchange stage of a bitonic sort with the partner at distance
// J: the lower position of a pair keeps the smaller key in an ascending
// block ((pos & k) == 0), the larger in a descending one.
template <int J>
__device__ __forceinline__ uint32_t bitonic_lane_stage(uint32_t key, int pos, int k) {
  const uint32_t other = lane_xor<J>(key);
  const bool lower = (pos & J) == 0;
  const bool ascending = (pos & k) == 0;
  return (lower == ascending) ? min(key, other) : max(key, other);
}

// The stages of block size k whose partners are in the same wave (J < 64).
__device__ __forceinline__ uint32_t bitonic_wave_stages(uint32_t key, int pos, int k) {
  if (k > 32) key = bitonic_lane_stage<32>(key, pos, k);
  if (k > 16) key = bitonic_lane_stage<16>(key, pos, k);
  if (k > 8) key = bitonic_lane_stage<8>(key, pos, k);
  if (k > 4) key = bitonic_lane_stage<4>(key, pos, k);
  if (k > 2) key = bitonic_lane_stage<2>(key, pos, k);
  return bitonic_lane_stage<1>(key, pos, k);
}

struct SegInfo {
  int n, L, c0;
  bool ok;
};

__device__ __forceinline__ SegInfo seg_info(const PlanParams& p, int s) {
  SegInfo r{0, 0, 0, false};
  if (s >= p.num_seqs) return r;
  const int c0 = p.cu[s];
  const int c1 = p.cu[s + 1];
  r.L = p.lens[s];
  r.n = c1 - c0;
  r.c0 = c0;
  r.ok = c0 >= 0 && c1 <= p.num_tokens && r.n >= 0 && r.L >= r.n && r.L <= p.max_len;
  return r;
}

// Sort key of prefill item (query tile qt of a segment with n new tokens and
// L total): bucket 0 holds the items with the most key tiles.
__device__ __forceinline__ int cost_key(int n, int L, int qt, int qtile) {
  const int kmax = L - n + min(n, (qt + 1) * qtile);
  const int tiles = (kmax + kPrefillTileKeys - 1) / kPrefillTileKeys;
  return kCostBuckets - 1 - min(tiles, kCostBuckets - 1);
}

// Bucket of a segment's partial last partition of `keys` keys (1 .. P - 1):
// one bucket per 32 keys fewer than P, after bucket 0, which holds the full
// partitions (placed by a scan, in segment order).
__device__ __forceinline__ int decode_bucket(int keys, int part_tokens) {
  return 1 + (part_tokens - keys) / 32;
}
constexpr int kDecodeBuckets = 2048 / 32 + 2;   // partitions of up to 2048 keys

__global__ void __launch_bounds__(1024) plan_kernel(PlanParams p) {
  __shared__ int scratch[17];
  __shared__ int scan5[17][5];
  __shared__ int hist[kCostBuckets];
  __shared__ int dhist[kDecodeBuckets];
  __shared__ int dscan_total;
  // prefill segments of a batch of at most 1024 segments, listed so that one
  // wave per segment spreads its query tiles over the lanes
  __shared__ int pl_seg[1024], pl_n[1024], pl_len[1024], pl_c0[1024];
  __shared__ int pl_count;
  // shared-prefix grouping of the first 1024 segments: a 2048-slot
  // hash set of first table entries (its storage then holds the sort keys), per segment its
  // length and covered partitions, per sorted position its segment, length,
  // link and group scratch
  __shared__ int g_hash[2048];
  uint32_t* g_key = (uint32_t*)g_hash;   // the sort keys reuse the hash set's storage
  __shared__ int g_lseg[1024], g_cov[1024];
  __shared__ int g_seg[1024], g_len[1024], g_link[1024], g_cand[1024], g_size[1024], g_cnt[1024];
  const bool one_chunk = p.num_seqs <= 1024;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  hist[threadIdx.x] = 0;   // blockDim.x == kCostBuckets
  if (threadIdx.x < kDecodeBuckets) dhist[threadIdx.x] = 0;
  if (threadIdx.x < 16) p.hdr->zeros[threadIdx.x] = 0u;
  __syncthreads();

  // pass 0: shared-prefix groups.  Single-token decode segments of more
  // than one partition whose leading full partitions start with the same
  // block ids (a cached prefix the block manager shares, "vLLM 学习笔记 01",
  // section 2.2) are grouped whatever their order in the batch: the
  // eligible segments are sorted so that equal first table entries are
  // adjacent, each in index order; neighbours in that order that share
  // leading partitions form runs, each run is cut
  // into groups of at most group_max members, and a group reads each
  // partition that all its members share once, for all of them (one group
  // item per partition).  Those partitions leave the members' own item
  // lists.  A hash set of the first entries finds whether any two are equal
  // at all; only then is the batch sorted.
  SegInfo si0{0, 0, 0, false};
  int cov = 0;       // leading partitions of the thread's segment that group items cover
  int n_group = 0;
  // (the first 1024 segments of a larger batch are grouped among themselves)
  const bool grouping = p.group_max >= 2;
  si0 = seg_info(p, threadIdx.x);
  // The partition size: the host's P, or 2P (when the host allows it) if no
  // two single-token decode segments of more than one partition start with
  // the same block, that is, when no shared-prefix group can form: longer
  // partitions pay an item's start and its partials half as often.  The
  // hash pass below finds whether two such first entries are equal; it runs
  // whether or not grouping is on, so the choice does not depend on it.
  int P = p.part_tokens;
  if (grouping || p.part_double) {
    const int s = threadIdx.x;
    const bool elig0 = si0.ok && si0.n == 1 && si0.L > p.part_tokens;
    // a table entry is read only below ceil(L / 16)
    const int fb = elig0 ? p.bt[(int64_t)s * p.width] : -1;
    const bool elig = elig0 && fb >= 0;
    g_hash[s] = -1;
    g_hash[s + 1024] = -1;
    g_lseg[s] = si0.L;
    g_cov[s] = 0;
    __syncthreads();
    bool dup = false;
    uint32_t h = 2048;   // the slot of the segment's first entry (2048: not eligible)
    if (elig) {   // open addressing over 2048 slots for at most 1024 keys: always ends
      h = ((uint32_t)fb * 2654435761u) >> 21;
      for (;;) {
        const int old = atomicCAS(&g_hash[h], -1, fb);
        if (old == -1) break;
        if (old == fb) {
          dup = true;
          break;
        }
        h = (h + 1) & 2047u;
      }
    }
    // each distinct first entry owns one slot, so equal slots mean equal
    // first entries; sorting by (slot, index) keeps the segments of one
    // first entry together, in index order
    const bool any_dup = __syncthreads_or(dup);
    if (!any_dup && p.part_double) P = 2 * p.part_tokens;
    if (grouping && any_dup) {
      // bitonic sort of (slot, index) over the first nsort positions (a
      // power of two >= the number of segments, at most 1024; ineligible
      // segments sort last).  Thread s holds position s; its partner s ^ j
      // is in the same wave for j < 64 (exchanged by DPP, swizzle or lane
      // permute), else it is read from LDS.
      int nsort = 2;
      while (nsort < min(p.num_seqs, 1024)) nsort <<= 1;
      __syncthreads();   // the hash set's storage becomes the key array
      uint32_t key = (h << 10) | (uint32_t)s;
      for (int k = 2; k <= nsort; k <<= 1) {
        for (int j = k >> 1; j >= 64; j >>= 1) {
          g_key[s] = key;
          __syncthreads();
          const uint32_t other = g_key[s ^ j];
          __syncthreads();
          // the lower position of a pair keeps the smaller key in an
          // ascending block ((s & k) == 0), the larger in a descending one
          const bool lower = (s & j) == 0;
          const bool ascending = (s & k) == 0;
          key = (lower == ascending) ? min(key, other) : max(key, other);
        }
        key = bitonic_wave_stages(key, s, k);
      }
      g_key[s] = key;
      __syncthreads();
      // thread r now works on sorted position r
      const int r = s;   // its key is `key` (g_key[r])
      const bool relig = (key >> 10) < 2048u;
      const int seg = (int)(key & 1023u);
      g_seg[r] = seg;
      g_len[r] = relig ? g_lseg[seg] : 0;   // 0: not eligible
      g_link[r] = 0;
      __syncthreads();
      const bool cand = relig && r > 0 && g_len[r - 1] > 0 && (g_key[r - 1] >> 10) == (key >> 10);
      int ncand;
      const int ci = block_exclusive_scan(cand ? 1 : 0, scratch, &ncand);
      if (cand) g_cand[ci] = r;
      __syncthreads();
      // link of each candidate position: how many leading full partitions
      // its segment has whose first and last block ids equal the previous
      // position's.  Only those two ids of a partition are compared here (two
      // pairs of loads per partition, all in one trip to memory): a prefix
      // shared by block tables covers whole blocks from the first, so a
      // partition that the prefix ends inside has a differing last id and is
      // not linked (the members would then each be computed on their own
      // inside the group item).  The decode kernel compares a grouped
      // partition's ids whole and computes a member that differs on its own.  Rounds of 8 partitions: a unit is (candidate,
      // partition); g_size holds a candidate's first differing partition,
      // g_cnt marks finished candidates.
      constexpr int kRound = 8;
      const int npb = p.part_tokens / kBlock;   // block ids per partition
      if ((int)threadIdx.x < ncand) g_cnt[threadIdx.x] = 0;
      for (int c0 = 0;; c0 += kRound) {
        if ((int)threadIdx.x < ncand) g_size[threadIdx.x] = INT_MAX;
        __syncthreads();
        for (int u = threadIdx.x; u < ncand * kRound; u += 1024) {
          const int k = u / kRound;
          if (g_cnt[k]) continue;
          const int rc = g_cand[k];
          const int c = c0 + u % kRound;
          // a partition counts when it is full in both segments
          bool differ = c >= min(g_len[rc], g_len[rc - 1]) / p.part_tokens;
          if (!differ) {
            const int32_t* a = p.bt + (int64_t)g_seg[rc] * p.width + c * npb;
            const int32_t* b = p.bt + (int64_t)g_seg[rc - 1] * p.width + c * npb;
            differ = a[0] != b[0] || a[npb - 1] != b[npb - 1];
          }
          if (differ) atomicMin(&g_size[k], c);
        }
        __syncthreads();
        int more = 0;
        if ((int)threadIdx.x < ncand && !g_cnt[threadIdx.x]) {
          const int f = g_size[threadIdx.x];
          g_link[g_cand[threadIdx.x]] = min(f, c0 + kRound);
          if (f == INT_MAX)
            more = 1;
          else
            g_cnt[threadIdx.x] = 1;
        }
        if (!__syncthreads_or(more)) break;
      }
      const int link = g_link[r];
      const int start = block_inclusive_max(link > 0 ? -1 : r, scratch);   // the run's first position
      const int mi = (r - start) % p.group_max;
      const int leader = r - mi;
      g_size[r] = 1;
      g_cnt[r] = INT_MAX;
      __syncthreads();
      if (mi > 0) {
        atomicMax(&g_size[leader], mi + 1);
        atomicMin(&g_cnt[leader], link);
      }
      __syncthreads();
      const int size = g_size[leader];
      const int my_cov = size >= 2 ? g_cnt[leader] : 0;
      if (my_cov > 0) g_cov[seg] = my_cov;
      const int ng = (mi == 0 && size >= 2) ? my_cov : 0;
      int tot_g;
      const int og = block_exclusive_scan(ng, scratch, &tot_g);
      if (ng > 0) {
        GroupItem gi{};
        gi.nmem = size;
        for (int i = 0; i < 8; ++i) gi.seg[i] = g_seg[r + min(i, size - 1)];
        for (int i = 0; i < ng; ++i) {
          gi.part = i;
          if (og + i < p.group_cap) p.group_items[og + i] = gi;
        }
      }
      n_group = min(tot_g, p.group_cap);
      __syncthreads();
      cov = g_cov[s];
    }
  }

  // pass 1: decode items and partial rows in segment order; prefill item
  // count (and, for a batch of at most 1024 segments, the list of prefill
  // segments).  Well-formed segments do not overlap, so their prefill items
  // number at most prefill_cap (num_tokens / 32 + num_seqs); each count is
  // capped at prefill_cap + 1 before the scan and the running total
  // saturates there, so overlapping (malformed) segments can neither
  // overflow a sum nor place a segment past the list: such a batch is
  // flagged and its prefill items are dropped.
  int dec_base = 0;
  int row_base = 0;
  int pre_total = 0;
  uint32_t status = 0;
  SegInfo first{0, 0, 0, false};   // the thread's segment of the first 1024, kept for the later passes
  int first_ofull = 0;              // and the place of its first full decode partition
  int first_tot_f = 0;              // and the first chunk's full decode partitions in all
  int full_base = 0;
  if (threadIdx.x == 0) pl_count = 0;
  for (int base = 0; base < p.num_seqs; base += 1024) {
    const int s = base + (int)threadIdx.x;
    const SegInfo si = base == 0 ? si0 : seg_info(p, s);
    if (base == 0) first = si;
    const int cov_s = base == 0 ? cov : 0;
    int nd = 0, np = 0, nr = 0, nfull = 0;
    if (s < p.num_seqs && !si.ok) {
      status |= 1u;
    } else if (si.ok && si.n >= 1 && si.n <= p.max_decode_n) {
      const int parts = (si.L + P - 1) / P;
      nd = parts - cov_s;
      nfull = si.L / P - cov_s;
      nr = si.n;
      if (parts * P > si.L)
        atomicAdd(&dhist[decode_bucket(si.L - (parts - 1) * P, P)], 1);
    } else if (si.ok && si.n > p.max_decode_n) {
      np = min((si.n + p.query_tile - 1) / p.query_tile, p.prefill_cap + 1);
    }
    // offsets and totals of: decode items, full decode partitions, prefill
    // items, partial rows, prefill segments
    int sc[5] = {nd, nfull, np, nr, np > 0 ? 1 : 0};
    int tot[5];
    block_exclusive_scan_n<5>(sc, scan5, tot);
    const int ofull = full_base + sc[1];
    if (base == 0) {
      first_ofull = ofull;
      first_tot_f = tot[1];
    }
    full_base += tot[1];
    if (one_chunk) {
      if (np > 0) {
        const int k = sc[4];   // < 1024: the thread's place among the chunk's segments
        pl_seg[k] = s;
        pl_n[k] = si.n;
        pl_len[k] = si.L;
        pl_c0[k] = si.c0;
      }
      if (threadIdx.x == 0) pl_count = tot[4];
    }
    const int orow = row_base + sc[3];
    if (s < p.num_seqs) {
      // rows past the capacity (only possible with overlapping segments):
      // the segment is skipped by the decode kernels and flagged
      const bool fits = nr > 0 && orow + nr <= p.rows_cap;
      p.seg_row[s] = fits ? orow : -1;
      if (nr > 0 && !fits) status |= 1u;
    }
    row_base += tot[3];
    dec_base += tot[0];
    pre_total = min(pre_total + tot[2], p.prefill_cap + 1);
  }
  // overlapping segments (only possible when some segment is malformed)
  // could overflow the lists: decode items past the capacity are dropped,
  // and so are all prefill items when they do not fit; both are flagged
  if (pre_total > p.prefill_cap) {
    status |= 1u;
    pre_total = 0;
  }
  if (dec_base > p.decode_cap) status |= 1u;
  __syncthreads();
  if (one_chunk && pre_total > 0) {   // pass 1b: the cost histogram, one wave per prefill segment
    // segment-major: a segment's items go together, in the bucket of its
    // costliest (last) query tile
    for (int k = wave; k < pl_count; k += 16) {
      const int n = pl_n[k], L = pl_len[k];
      const int np = (n + p.query_tile - 1) / p.query_tile;
      if (lane == 0) atomicAdd(&hist[cost_key(n, L, np - 1, p.query_tile)], np);
    }
    __syncthreads();
  } else if (pre_total > 0) {   // more than 1024 segments: one thread per segment
    for (int base = 0; base < p.num_seqs; base += 1024) {
      const int s = base + (int)threadIdx.x;
      const SegInfo si = base == 0 ? first : seg_info(p, s);
      if (si.ok && si.n > p.max_decode_n) {
        const int np = (si.n + p.query_tile - 1) / p.query_tile;
        for (int qt = 0; qt < np; ++qt) atomicAdd(&hist[cost_key(si.n, si.L, qt, p.query_tile)], 1);
      }
    }
    __syncthreads();
  }

  // pass 2: bucket offsets (exclusive scans of the histograms): the decode
  // buckets by the first two waves (one bucket per thread; bucket 0 holds
  // the full partitions), the prefill cost buckets by the whole block, only
  // when the step has prefill items (pre_total is the same in every thread)
  int dc = 0, dx = 0;
  if (threadIdx.x < 128) {   // whole waves 0 and 1
    const int b = threadIdx.x;
    dc = b == 0 ? full_base : (b < kDecodeBuckets ? dhist[b] : 0);
    dx = dc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(dx, off);
      if (lane >= off) dx += y;
    }
    if (threadIdx.x == 63) dscan_total = dx;   // buckets 0 .. 63
  }
  __syncthreads();
  if (threadIdx.x < kDecodeBuckets) dhist[threadIdx.x] = (threadIdx.x >= 64 ? dscan_total : 0) + dx - dc;
  if (pre_total > 0) {
    int unused;
    hist[threadIdx.x] = block_exclusive_scan(hist[threadIdx.x], scratch, &unused);
  }
  __syncthreads();

  // pass 3a: decode items: a segment's full partitions at their scanned
  // places, its partial last one at its bucket's next place
  full_base = 0;
  for (int base = 0; base < p.num_seqs; base += 1024) {
    const int s = base + (int)threadIdx.x;
    const SegInfo si = base == 0 ? first : seg_info(p, s);
    const bool dec = si.ok && si.n >= 1 && si.n <= p.max_decode_n;
    const int full = dec ? si.L / P : 0;
    const int cov_s = base == 0 ? cov : 0;   // partitions 0 .. cov_s - 1 are in group items
    int at = first_ofull;
    if (base == 0) {
      full_base = first_tot_f;
    } else {   // more than 1024 segments: place the full partitions again
      int tot_f;
      at = full_base + block_exclusive_scan(full - cov_s, scratch, &tot_f);
      full_base += tot_f;
    }
    if (dec) {
      for (int i = cov_s; i < full; ++i)
        if (at + i - cov_s < p.decode_cap) p.decode_items[at + i - cov_s] = make_int2(s, i);
      if (si.L > full * P) {
        const int at2 = atomicAdd(&dhist[decode_bucket(si.L - full * P, P)], 1);
        if (at2 < p.decode_cap) p.decode_items[at2] = make_int2(s, full);
      }
    }
  }

  // pass 3b: prefill items to their bucket's next place
  if (pre_total > 0 && one_chunk) {
    // one wave per prefill segment: lanes 0-7 read its first eight block ids,
    // every lane writes the descriptors of query tiles lane, lane + 64, ...
    for (int k = wave; k < pl_count; k += 16) {
      const int s = pl_seg[k], n = pl_n[k], L = pl_len[k];
      const int np = (n + p.query_tile - 1) / p.query_tile;
      const int nblk = (L + kBlock - 1) / kBlock;   // >= 1: L >= n > 1
      int bid = 0;
      if (lane < 8) bid = p.bt[(int64_t)s * p.width + min(lane, nblk - 1)];
      PrefillItem it{};
      it.seq = s;
      it.L = L;
      it.tok0 = pl_c0[k];
      it.n = n;
#pragma unroll
      for (int j = 0; j < 8; ++j) it.bid[j] = __shfl(bid, j);
      int at0 = 0;
      if (lane == 0) at0 = atomicAdd(&hist[cost_key(n, L, np - 1, p.query_tile)], np);
      at0 = __shfl(at0, 0);
      for (int qt = lane; qt < np; qt += 64) {
        const int at = at0 + (np - 1 - qt);   // the segment's tiles by decreasing cost
        it.qt = qt;
        if (at < p.prefill_cap) p.prefill_items[at] = it;
      }
    }
  } else if (pre_total > 0) {
    for (int base = 0; base < p.num_seqs; base += 1024) {
      const int s = base + (int)threadIdx.x;
      const SegInfo si = base == 0 ? first : seg_info(p, s);
      if (si.ok && si.n > p.max_decode_n) {
        const int np = (si.n + p.query_tile - 1) / p.query_tile;
        PrefillItem it{};
        it.seq = s;
        it.L = si.L;
        it.tok0 = si.c0;
        it.n = si.n;
        const int32_t* bt_row = p.bt + (int64_t)s * p.width;
        const int nblk = (si.L + kBlock - 1) / kBlock;   // >= 1: L >= n > 1
#pragma unroll
        for (int j = 0; j < 8; ++j) it.bid[j] = bt_row[min(j, nblk - 1)];
        for (int qt = 0; qt < np; ++qt) {
          const int at = atomicAdd(&hist[cost_key(si.n, si.L, qt, p.query_tile)], 1);
          it.qt = qt;
          if (at < p.prefill_cap) p.prefill_items[at] = it;
        }
      }
    }
  }

  const int any_bad = __syncthreads_or((int)status);
  if (threadIdx.x == 0) {
    p.hdr->status = any_bad ? 1u : 0u;
    p.hdr->n_decode = min(dec_base, p.decode_cap);
    p.hdr->n_prefill = min(pre_total, p.prefill_cap);
    p.hdr->n_group = n_group;
    p.hdr->part_tokens = P;
    p.hdr->decode_next = 0;
  }
  if (threadIdx.x < kMaxQueues) {
    p.hdr->prefill_next[threadIdx.x] = 0;
    p.hdr->group_next[threadIdx.x] = 0;
  }
}

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  plan_kernel<<<1, kCostBuckets, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pkv
