// Split-context decode attention and its cross-partition log-sum-exp reduce.
//
// What is computed ("vLLM 学习笔记 01", sections 1.4-1.6): a decode segment
// has one new token at position L-1 of a sequence whose L keys/values sit in
// 16-token blocks listed by the segment's block table; its query heads of
// group g (G = Hq/Hkv of them) attend to all L keys of KV head g.  Decode
// reads every cached K/V byte once per step, so it is bound by HBM bandwidth
// ("从0开始的vLLM学习": decode is memory-bandwidth bound).  A segment of a few
// new tokens (n * G <= 32: a speculative-decoding check of n - 1 drafted
// tokens, for instance) is the same read: its n * G query rows share the
// item in one or two column tiles of 16, and row (token i, head h) sees keys
// 0 .. L - n + i.
//
// Work split: a work item is (segment, partition of P keys, KV head) and is
// run by one wavefront; partitions of long contexts run on different waves
// and are merged by decode_reduce_kernel with the online-softmax identity
// (each partition keeps its running max m, sum l and unnormalised output o;
// the merge rescales by exp(m_p - max_p m_p)).
//
// Per wave, per 32 keys (two blocks):
//   S^T[key, row] = K[key, :] . Q[row, :]       16x16x32 bf16 MFMA, D/32 slabs,
//                                               Q (n * G rows, zero-padded to
//                                               16) in registers for the item
//   online softmax in fp32 (exp2 with scale*log2(e) folded in)
//   O^T[d, head] += V^T[d, key] . P^T[key, head] 16x16x32 bf16 MFMA, D/16 tiles
// The C layout of the first product (lane = head, 4 keys per lane group) is
// exactly the B operand layout the second product needs, so P never leaves
// its registers.  V rows are loaded fully coalesced (16 lanes cover one
// 256-byte row) with a permuted d order (tile t, row m <-> d = (D/16)*m + t)
// and transposed to the A operand with v_perm in registers.  Next 32 keys'
// K/V loads are issued before the current 32 keys are computed.  The loads
// are raw buffer loads ranged to the rows before the partition end (rows
// past it and blocks outside the pool read as zeros, with no per-lane
// branch), marked non-temporal.
#include "kernels.hpp"

namespace pkv {

template <int D>
struct KvRegs {
  static constexpr int NS = D / 32;           // 32-wide d slabs of the QK product
  static constexpr int VW = D / 32;           // dwords of one lane's V piece (D/16 bf16)
  u32x4 k[2][NS];
  uint32_t v[8][VW];
};

// Buffer views of one 16-key block of KV head g: K half and V half, each
// ranged to the block's rows before the partition end (rows past it, and a
// block outside the pool, read as zeros through the range check of the raw
// buffer access, so the loads need no per-lane conditions).
struct BlockRs {
  __amdgpu_buffer_rsrc_t k, v;
};

constexpr int kRsrcWord3 = 0x00020000;   // fourth descriptor word on gfx950
// Cache policy of the K/V loads: non-temporal (each byte is read once per
// step, so it should not displace what the caches hold for reuse).
constexpr int kNonTemporal = 2;

__device__ __forceinline__ BlockRs block_rs(const uint16_t* cache, int bid, bool ok, int nvalid,
                                            int64_t block_bytes, int64_t row_bytes, int g,
                                            int head_bytes) {
  const char* base = reinterpret_cast<const char*>(cache) + (ok ? (int64_t)bid * block_bytes : 0) +
                     (int64_t)g * head_bytes;
  const int nrec = __builtin_amdgcn_readfirstlane(ok ? nvalid * (int)row_bytes : 0);
  BlockRs r;
  r.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nrec, kRsrcWord3);
  r.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + kBlock * row_bytes), (short)0,
                                          nrec, kRsrcWord3);
  return r;
}

// K and V of 32 keys (two blocks): lane (m, j) loads K row m, d 8j + 32sl
// .. +7 of each block, and V rows 4j .. 4j+3 of each block, d (D/16)m ..
// (D/16)m + D/16 - 1.
template <int D>
__device__ __forceinline__ void load_kv(KvRegs<D>& r, const BlockRs& b0, const BlockRs& b1,
                                        int m, int j, uint32_t row_bytes) {
  constexpr int NS = KvRegs<D>::NS;
  constexpr int VW = KvRegs<D>::VW;
  constexpr int NT = D / 16;
  const uint32_t koff = m * row_bytes + 16 * j;
  const uint32_t voff = 4 * j * row_bytes + 2 * NT * m;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const BlockRs& rs = b ? b1 : b0;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      r.k[b][sl] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.k, koff + 64 * sl, 0, kNonTemporal));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if constexpr (VW == 4) {
        const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.v, voff, rr * row_bytes, kNonTemporal));
        r.v[4 * b + rr][0] = x[0]; r.v[4 * b + rr][1] = x[1]; r.v[4 * b + rr][2] = x[2]; r.v[4 * b + rr][3] = x[3];
      } else {
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs.v, voff, rr * row_bytes, kNonTemporal));
        r.v[4 * b + rr][0] = x[0]; r.v[4 * b + rr][1] = x[1];
      }
    }
  }
}

// How far (log2 units) the running maximum may trail a row's true maximum:
// m moves only when a step's maximum exceeds it by more than this, so P stays
// below 2^8 and O is rescaled only in the rare steps where some row's m moved.
constexpr float kLazyMax = 8.f;

// One step of 32 keys for CT column tiles of 16 query rows: the K fragments
// are multiplied against every tile's queries and each V operand against
// every tile's P, so the tiles share one read of K and V.  `edge` (wave-
// uniform) is set for a step some row does not see whole (a partition's
// last keys, a row's causal limit, a block outside the pool); the other
// steps skip the per-key checks.
template <int D, int CT>
__device__ __forceinline__ void attend_step(const KvRegs<D>& r, const u32x4 (&qf)[CT][D / 32],
                                            f32x4 (&o)[CT][D / 16], float (&m_run)[CT],
                                            float (&l_run)[CT], int kb, const int (&kend)[CT],
                                            bool edge, bool ok0, bool ok1, int j, float scale_log2) {
  constexpr int NS = D / 32;
  constexpr int NT = D / 16;
  f32x4 sc[CT][2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int c = 0; c < CT; ++c) sc[c][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
      for (int c = 0; c < CT; ++c) sc[c][b] = mfma16(r.k[b][sl], qf[c][sl], sc[c][b]);
  }
  float alpha[CT];
  bool moved = false;
  u32x4 pb[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = sc[c][i >> 2][i & 3] * scale_log2;
    if (edge) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b = i >> 2;
        const bool okb = b ? ok1 : ok0;
        const bool live = okb && (kb + 16 * b + 4 * j + (i & 3) < kend[c]);
        x[i] = live ? x[i] : -INFINITY;
      }
    }
    float cmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    cmax = wave_max_xor(cmax, 16);
    cmax = wave_max_xor(cmax, 32);
    // m_run = -inf: no key seen yet (then O and l are zero, nothing to rescale)
    const bool first = m_run[c] == -INFINITY;
    const bool upd = first ? cmax != -INFINITY : cmax - m_run[c] > kLazyMax;
    const float m_new = upd ? cmax : m_run[c];
    alpha[c] = upd && !first ? __builtin_amdgcn_exp2f(m_run[c] - m_new) : 1.f;
    moved = moved || (upd && !first);
    // keys left out have x = -inf and P = 0; while no key was seen m stays
    // -inf and every P is 0
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - mu);
      psum += p[i];
    }
    l_run[c] = l_run[c] * alpha[c] + psum;
    m_run[c] = m_new;
    pb[c] = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                  pack_bf16(p[6], p[7])};
  }
  if (__any(moved)) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) o[c][t] *= alpha[c];
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int w = t >> 1;
    const bool hi = t & 1;
    u32x4 a = {pick_halves(r.v[0][w], r.v[1][w], hi), pick_halves(r.v[2][w], r.v[3][w], hi),
               pick_halves(r.v[4][w], r.v[5][w], hi), pick_halves(r.v[6][w], r.v[7][w], hi)};
#pragma unroll
    for (int c = 0; c < CT; ++c) o[c][t] = mfma16(a, pb[c], o[c][t]);
  }
}

// Query rows of one work item: CT column tiles of 16 rows; row 16c + m reads
// token qtok[c] of the packed batch, query head hq[c], sees the partition's
// keys below kend[c], and leaves its result in partial row prow[c] (or, when
// the item is the whole context, in output row qtok[c]).
template <int CT>
struct RowMap {
  int qtok[CT], hq[CT], kend[CT], prow[CT];
  bool live[CT];
};

// One work item: the keys key0 .. key1 - 1 of the block table row `bt_row`
// for KV head g, attended by the query rows of `rm`; every row sees the keys
// before kfull.
template <int D, int CT>
__device__ __forceinline__ void decode_rows(const DecodeParams& p, const int32_t* bt_row, int key0,
                                            int key1, int kfull, int part, bool direct, int g,
                                            int lane, const RowMap<CT>& rm, int64_t row_bytes,
                                            int64_t block_bytes) {
  constexpr int NS = D / 32;
  constexpr int NT = D / 16;
  const int m = lane & 15;
  const int j = lane >> 4;
  int kend[CT];
  u32x4 qf[CT][NS];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    kend[c] = rm.kend[c];
    const uint16_t* qrow = p.q + (int64_t)rm.qtok[c] * p.q_stride + (int64_t)rm.hq[c] * D + 8 * j;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[c][sl] = rm.live[c] ? *reinterpret_cast<const u32x4*>(qrow + 32 * sl) : z;
    }
  }
  // the partition's block ids, lane i holding entries i and 64 + i
  // (P <= 2048 keys = 128 blocks)
  const int nblk = (key1 - key0 + kBlock - 1) / kBlock;
  int my_bid = -1, my_bid2 = -1;
  if (lane < nblk) my_bid = bt_row[key0 / kBlock + lane];
  if (64 + lane < nblk) my_bid2 = bt_row[key0 / kBlock + 64 + lane];
  const bool bad_bid = (lane < nblk && (my_bid < 0 || (int64_t)my_bid >= p.num_blocks)) ||
                       (64 + lane < nblk && (my_bid2 < 0 || (int64_t)my_bid2 >= p.num_blocks));
  if (__any(bad_bid)) {
    if (lane == 0) atomicOr(&p.hdr->status, 2u);
  }

  f32x4 o[CT][NT];
  float m_run[CT], l_run[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
#pragma unroll
    for (int t = 0; t < NT; ++t) o[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
  }

  // block b of the 32 keys starting at kb; its keys count as present
  // (ok) when the block is inside the pool
  auto block_at = [&](int kb, int b, bool& ok) -> BlockRs {
    const int first = kb + kBlock * b;
    const int nvalid = min(max(key1 - first, 0), kBlock);
    const int e = min((first - key0) / kBlock, 127);   // wave-uniform
    const int bid = nvalid <= 0 ? -1
                    : e < 64   ? __builtin_amdgcn_readlane(my_bid, e)
                               : __builtin_amdgcn_readlane(my_bid2, e - 64);
    ok = nvalid > 0 && bid >= 0 && (int64_t)bid < p.num_blocks;
    return block_rs(p.cache, bid, ok, nvalid, block_bytes, row_bytes, g, D * 2);
  };

  KvRegs<D> ra, rb;
  bool ao0, ao1, bo0, bo1;
  {
    const BlockRs x0 = block_at(key0, 0, ao0), x1 = block_at(key0, 1, ao1);
    load_kv<D>(ra, x0, x1, m, j, (uint32_t)row_bytes);
  }
  // Two register sets: the loads of the next 32 keys are issued before the
  // current 32 are computed.  They are issued on every step, also past the
  // partition's end (zero-range buffers: nothing is read), so the code has
  // no branch around them and each step waits only for its own loads, not
  // for the next step's as well.
  for (int kb = key0;; kb += 64) {
    const int kn = kb + 32;
    {
      const BlockRs x0 = block_at(kn, 0, bo0), x1 = block_at(kn, 1, bo1);
      load_kv<D>(rb, x0, x1, m, j, (uint32_t)row_bytes);
    }
    attend_step<D, CT>(ra, qf, o, m_run, l_run, kb, kend, !(ao0 && ao1 && kb + 32 <= kfull), ao0, ao1, j,
                       p.scale_log2);
    if (kn >= key1) break;
    const int kn2 = kb + 64;
    {
      const BlockRs x0 = block_at(kn2, 0, ao0), x1 = block_at(kn2, 1, ao1);
      load_kv<D>(ra, x0, x1, m, j, (uint32_t)row_bytes);
    }
    attend_step<D, CT>(rb, qf, o, m_run, l_run, kn, kend, !(bo0 && bo1 && kn + 32 <= kfull), bo0, bo1, j,
                       p.scale_log2);
    if (kn2 >= key1) break;
  }

  // Each row leaves normalised, o / l, in bf16: into the output when the
  // item is the segment's only partition, else into the partition's partial
  // row (its m and l beside it in fp32), which the merge weighs by l.  Partial
  // rows in bf16 halve the bytes this kernel writes into the middle of its
  // read stream, where a written byte costs several read bytes.
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    float l = l_run[c];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!rm.live[c]) continue;
    const int hq = rm.hq[c];
    const float inv = l > 0.f ? 1.f / l : 0.f;   // l = 0: the row saw no key of the partition
    const int64_t slot = ((int64_t)rm.prow[c] * p.pmax + part) * p.hq + hq;
    uint16_t* orow = direct ? p.out + ((int64_t)rm.qtok[c] * p.hq + hq) * D : p.part_o + slot * D;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      uint32_t wv[NT / 2];
#pragma unroll
      for (int t = 0; t < NT; t += 2) wv[t / 2] = pack_bf16(o[c][t][rr] * inv, o[c][t + 1][rr] * inv);
      uint16_t* dst = orow + NT * (4 * j + rr);
      if constexpr (NT == 8) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
      } else {
        *reinterpret_cast<u32x2*>(dst) = u32x2{wv[0], wv[1]};
      }
    }
    if (!direct && j == 0) p.part_ml[slot] = make_float2(m_run[c], l);
  }
}

// Work item (segment s, partition part, KV head g) of a decode segment of n
// new tokens: row 16c + m is (token ti, head hh) of the segment and sees the
// partition's keys up to its own position (causal in the segment).
template <int D, int CT>
__device__ __forceinline__ void decode_item(const DecodeParams& p, int P, int s, int part, int g,
                                            int lane, int L, int tok, int n, int row0,
                                            int64_t row_bytes, int64_t block_bytes) {
  const int key0 = part * P;
  const int key1 = min(L, key0 + P);
  const int nparts = (L + P - 1) / P;
  RowMap<CT> rm;
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int row = 16 * c + (lane & 15);
    const int ti = row / p.group;
    rm.live[c] = ti < n;
    rm.kend[c] = min(key1, L - n + 1 + ti);
    rm.qtok[c] = tok + ti;
    rm.hq[c] = g * p.group + (row - ti * p.group);
    rm.prow[c] = row0 + ti;
  }
  // every row sees the keys before L - n + 1 (the first new token's)
  decode_rows<D, CT>(p, p.bt + (int64_t)s * p.width, key0, key1, min(key1, L - n + 1), part, nparts == 1,
                     g, lane, rm,
                     row_bytes, block_bytes);
}

// Group item (partition part of the member segments gi.seg[0 .. nmem - 1],
// KV head g): single-token decode segments that the plan found to share
// this full partition (by its first block id): each member's block ids of
// the partition are compared with the first member's, and the keys are read
// once for all members that match.  Row 16c + m is (member mi, head hh) and
// sees all P keys (each member's token comes after them); results go to
// each member's own partial row.  A member whose ids differ is computed on
// its own afterwards, from its own table.
template <int D, int CT>
__device__ __forceinline__ void group_item(const DecodeParams& p, int P, const GroupItem& gi, int g,
                                           int lane, int64_t row_bytes, int64_t block_bytes) {
  const int part = gi.part;
  const int nmem = gi.nmem;
  const int key0 = part * P;
  const int key1 = key0 + P;
  const int npb = P / kBlock;   // <= 128: two ids per lane
  int ids[8], ids2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int32_t* row = p.bt + (int64_t)gi.seg[i] * p.width + key0 / kBlock;
    ids[i] = (i < nmem && lane < npb) ? row[lane] : 0;
    ids2[i] = (i < nmem && 64 + lane < npb) ? row[64 + lane] : 0;
  }
  uint32_t differ = 0;
#pragma unroll
  for (int i = 1; i < 8; ++i)
    if (i < nmem && __any(ids[i] != ids[0] || ids2[i] != ids2[0])) differ |= 1u << i;
  RowMap<CT> rm;
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int row = 16 * c + (lane & 15);
    const int mi = row / p.group;
    int sm = gi.seg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if (mi == i) sm = gi.seg[i];
    const int r0 = p.seg_row[sm];
    rm.live[c] = mi < nmem && r0 >= 0 && !((differ >> mi) & 1u);
    rm.kend[c] = key1;
    rm.qtok[c] = p.cu[sm];
    rm.hq[c] = g * p.group + (row - mi * p.group);
    rm.prow[c] = r0;
  }
  decode_rows<D, CT>(p, p.bt + (int64_t)gi.seg[0] * p.width, key0, key1, key1, part, false, g, lane, rm,
                     row_bytes, block_bytes);
  while (differ) {
    const int mi = __builtin_ctz(differ);
    differ &= differ - 1;
    int sm = gi.seg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if (mi == i) sm = gi.seg[i];
    const int hh = lane & 15;
    RowMap<1> one;
    one.live[0] = hh < p.group && p.seg_row[sm] >= 0;
    one.kend[0] = key1;
    one.qtok[0] = p.cu[sm];
    one.hq[0] = g * p.group + min(hh, p.group - 1);
    one.prow[0] = p.seg_row[sm];
    decode_rows<D, 1>(p, p.bt + (int64_t)sm * p.width, key0, key1, key1, part, false, g, lane, one,
                      row_bytes, block_bytes);
  }
}

// One wave per SIMD: forcing two (256 registers each) measured slower.
template <int D>
__global__ void __launch_bounds__(256)
decode_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int n_group = p.hdr->n_group;
  if (n_group + p.hdr->n_decode == 0) return;   // no decode segment in this step: no queue traffic
  const int64_t row_bytes = (int64_t)p.hkv * D * 2;
  const int64_t block_bytes = 2 * kBlock * row_bytes;
  const int P = wave_uniform(p.hdr->part_tokens);   // the plan's partition size

  // Group items first, every one a full partition.  When the KV heads split
  // evenly over the eight XCDs, the group items of head g go to the queue of
  // XCD g mod 8 (workgroup b runs on XCD b mod 8), which its waves drain
  // before they turn to the shared queue: the groups that share a partition
  // then read its K/V of head g through one L2, so the partition comes from
  // HBM about once instead of once per group.
  const bool xcd_groups = p.hkv % kMaxQueues == 0;
  const int xq = blockIdx.x % kMaxQueues;
  const int hpq = p.hkv / kMaxQueues;                     // heads per XCD queue
  const int n_grp = xcd_groups ? 0 : n_group * p.hkv;     // group items in the shared queue
  const int n_items = n_grp + p.hdr->n_decode * p.hkv;
  bool own = xcd_groups && n_group > 0;   // still taking from this XCD's group queue
  for (;;) {
    int it = 0;
    if (lane == 0) it = atomicAdd(own ? &p.hdr->group_next[xq] : &p.hdr->decode_next, 1);
    it = wave_uniform(__shfl(it, 0));
    int gix = -1, g = 0;   // a group item: its entry and head
    if (own) {
      if (it >= n_group * hpq) {
        own = false;
        continue;
      }
      gix = it / hpq;
      g = xq + kMaxQueues * (it % hpq);
    } else {
      if (it >= n_items) break;
      if (it < n_grp) {
        gix = it / p.hkv;
        g = it % p.hkv;
      }
    }
    if (gix >= 0) {
      const GroupItem gi = p.groups[gix];
      if (gi.nmem * p.group <= 16)
        group_item<D, 1>(p, P, gi, g, lane, row_bytes, block_bytes);
      else
        group_item<D, 2>(p, P, gi, g, lane, row_bytes, block_bytes);
      continue;
    }
    it -= n_grp;
    const int2 item = p.items[it / p.hkv];
    g = it % p.hkv;
    const int s = item.x;
    const int part = item.y;
    const int L = p.lens[s];
    const int tok = p.cu[s];
    const int n = p.cu[s + 1] - tok;
    const int row0 = p.seg_row[s];   // first partial row of the segment
    if (row0 < 0) continue;          // skipped by the plan (and flagged there)
    // 16 or 32 query rows (n * G of them live)
    if (n * p.group <= 16)
      decode_item<D, 1>(p, P, s, part, g, lane, L, tok, n, row0, row_bytes, block_bytes);
    else
      decode_item<D, 2>(p, P, s, part, g, lane, L, tok, n, row0, row_bytes, block_bytes);
  }
}

// Merge of the partitions of every multi-partition decode segment.  One wave
// per (segment, query head), for each of the segment's new tokens; lanes
// split d.  Partition p left o_p / l_p (bf16) with m_p and l_p; the weights
// l_p exp2(m_p - max m) bring every partition to the common maximum (a
// partition none of whose keys a token sees has m_p = -inf and weight 0;
// partition 0 always holds key 0), and the output is their weighted mean.  Lane i
// holds the weight of partitions i, i + 64, ...; the partials' rows are read
// eight partitions at a time, so their loads overlap instead of paying one
// memory round trip per partition.
template <int D>
__global__ void __launch_bounds__(256)
decode_reduce_kernel(DecodeParams p, int32_t num_seqs, int32_t num_tokens) {
  constexpr int PER = D / 64;
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  const int hchunks = (p.hq + 3) / 4;
  const int s = blockIdx.x / hchunks;
  const int hq = (blockIdx.x % hchunks) * 4 + (threadIdx.x >> 6);
  if (s >= num_seqs || hq >= p.hq) return;
  const int row0 = p.seg_row[s];
  if (row0 < 0) return;   // not a decode segment (or skipped by the plan)
  const int c0 = p.cu[s];
  const int c1 = p.cu[s + 1];
  const int L = p.lens[s];
  if (c0 < 0 || c1 > num_tokens || c1 <= c0 || L < c1 - c0 || L > p.width * kBlock) return;
  const int P = p.hdr->part_tokens;   // the plan's partition size
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  for (int ti = 0; ti < c1 - c0; ++ti) {
    const int64_t base = (int64_t)(row0 + ti) * p.pmax * p.hq + hq;   // slot of partition 0
    float mx = -INFINITY;
    for (int i = lane; i < nparts; i += 64) mx = fmaxf(mx, p.part_ml[base + (int64_t)i * p.hq].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float den = 0.f;
    for (int i = lane; i < nparts; i += 64) {
      const float2 ml = p.part_ml[base + (int64_t)i * p.hq];
      den += ml.x == -INFINITY ? 0.f : ml.y * exp2f(ml.x - mx);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int i0 = 0; i0 < nparts; i0 += 64) {
      // weight of partition i0 + lane: its share of the sum, l_p exp2(m_p - M)
      // (its row holds o_p / l_p)
      float wl = 0.f;
      if (i0 + lane < nparts) {
        const float2 ml = p.part_ml[base + (int64_t)(i0 + lane) * p.hq];
        wl = ml.x == -INFINITY ? 0.f : ml.y * exp2f(ml.x - mx);
      }
      const int cnt = min(64, nparts - i0);
      for (int j0 = 0; j0 < cnt; j0 += kBatch) {
        float v[kBatch][PER];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int i = i0 + min(j0 + j, cnt - 1);   // past the end: a repeated row, weight 0 below
          const uint16_t* src = p.part_o + (base + (int64_t)i * p.hq) * D + lane * PER;
          if constexpr (PER == 2) {
            const uint32_t w2 = *reinterpret_cast<const uint32_t*>(src);
            v[j][0] = bf16_lo(w2);
            v[j][1] = bf16_hi(w2);
          } else {
            v[j][0] = bf16_lo(*src);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const float w = __shfl(wl, min(j0 + j, 63));
          const float wj = j0 + j < cnt ? w : 0.f;
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += wj * v[j][e];
        }
      }
    }
    const float inv = 1.f / den;
    uint16_t* dst = p.out + ((int64_t)(c0 + ti) * p.hq + hq) * D + lane * PER;
    if constexpr (PER == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16(acc[0] * inv, acc[1] * inv);
    } else {
      __bf16 b = (__bf16)(acc[0] * inv);
      *dst = __builtin_bit_cast(uint16_t, b);
    }
  }
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 128) {
    decode_kernel<128><<<grid, 256, 0, stream>>>(p);
  } else {
    decode_kernel<64><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int num_seqs, int num_tokens,
                               hipStream_t stream) {
  const int hchunks = (p.hq + 3) / 4;
  const int rgrid = num_seqs * hchunks;
  if (rgrid == 0) return hipSuccess;
  if (head_dim == 128) {
    decode_reduce_kernel<128><<<rgrid, 256, 0, stream>>>(p, num_seqs, num_tokens);
  } else {
    decode_reduce_kernel<64><<<rgrid, 256, 0, stream>>>(p, num_seqs, num_tokens);
  }
  return hipGetLastError();
}

const void* decode_kernel_ptr(int head_dim) {
  return head_dim == 128 ? (const void*)decode_kernel<128> : (const void*)decode_kernel<64>;
}

}  // namespace pkv
