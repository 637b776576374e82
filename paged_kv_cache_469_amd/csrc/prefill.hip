// Prefill and chunked-prefill attention over the paged pool.
//
// What is computed ("vLLM 学习笔记 01", sections 1.4-1.6 and 2.1): a segment
// with n > 1 new tokens at the end of a sequence of L tokens (h = L - n of
// them cached earlier, h = 0 for a fresh prompt, h > 0 for a later chunk of a
// long prompt) attends causally: query i sees keys 0 .. h + i of its own
// sequence, read through its block table.  Prefill is a dense contraction
// ("从0开始的vLLM学习": prefill is compute bound), so both products run on
// the bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Work item: (segment, query tile of QT queries, KV head, head chunk), run by
// one workgroup of 8 waves, two per SIMD, in a persistent grid fed by one
// queue per XCD.  Each wave owns one query head and 32 queries; the waves
// share the KV head, so each 64-key K/V tile is copied from its four
// 16-token blocks once into LDS (straight from global memory, one block per
// wave of group A for each of K and V) and read by all eight.
//
// Per wave and tile:
//   S^T[key, q] = K[key, :] . Q[q, :]         Q held in registers (B operand)
//   P = exp2(S * c - m * c) in fp32 -> bf16   c = |scale| * log2(e)
//   O^T[d, q] += V^T[d, key] . P^T[key, q]    V^T fragments come from the
//                                             transposing LDS read
//                                             (ds_read_b64_tr_b16)
// The C layout of S^T (lane = query) is the B operand layout of the second
// product, so P never leaves registers.  The running maximum m is lazy: it
// moves only when a tile's maximum exceeds it by more than 8 (log2 units),
// so rescaling O is rare and P stays below 2^8; the normaliser l sums P in
// fp32, the numerator uses P rounded to bf16 (the MFMA operand).
//
// Ping-pong: waves 0-3 (group A) and 4-7 (group B) sit on the four SIMDs in
// pairs and alternate phases, separated by workgroup barriers.  While group
// A issues the matrix products (QK^T of tile t, PV of tile t-1), group B runs
// its softmax on the vector ALUs of the same SIMDs, and then the other way
// round; so the matrix cores and the vector ALUs work at the same time.  K
// and V have three LDS slots each; copies run two tiles (K) and one tile (V)
// ahead.  K/V rows past the item's last needed key, and rows of blocks
// outside the pool, arrive as zeros, so poison in unused pool memory never
// reaches the products.
#include "kernels.hpp"
#include "matrix_phase.inc"

namespace pkv {
namespace {

constexpr int kKeys = 64;           // keys per tile
constexpr int kWaves = 8;
constexpr float kLazyMax = 8.f;     // how far (log2 units) m may trail the true maximum
// MFMAs by which the LDS operand reads of the compiled matrix phase (head
// size 64) run ahead
constexpr int kQkLead = 3;
constexpr int kPvLead = 3;

template <int D>
struct Geo {
  static constexpr int ROWB = 2 * D;           // bytes of one key row of a head
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int TILEB = kKeys * ROWB;   // bytes of one K or V tile
  static constexpr int NSL = D / 16;           // d slabs of QK^T
  static constexpr int NDT = D / 32;           // d tiles of PV
  static_assert(kKeys == kBlock * (kWaves / 2), "each wave of a group copies one block per tile");
};

// Chunk c (16 bytes) of K row r sits at chunk c ^ (r % CPR): the rows one
// quarter-wave reads with 16-byte operand loads hit different banks.
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) {
  return c ^ (r & (Geo<D>::CPR - 1));
}

// Chunk c of V row r sits at chunk c ^ s(r % 4), s = 0, 4, 10, 14 (mod CPR):
// the transposing reads take 4 consecutive rows x 32 or 64 bytes at once,
// and these land on disjoint banks.
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) {
  const int s = (r & 3) * 4 + ((r >> 1) & 1) * 2;
  return c ^ (s & (Geo<D>::CPR - 1));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

// Combine a value with the other half of the wave (lane l and l ^ 32).
// v_permlane32_swap on two copies of x leaves x's low half in both halves of
// one copy and its high half in both halves of the other.  Written as inline
// asm: through the builtin, the compiler keeps only one of the two results
// when both operands hold the same value.  The s_nop covers the wait the
// instruction needs after a VALU write of its operands.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float halves_max(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float halves_sum(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

// Workgroup barrier with no memory wait of its own; the empty asm statements
// keep the compiler from moving memory accesses across it and the scheduling
// barriers keep every other instruction on its side.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The item's block table lives in LDS, in windows of 256 entries (64 tiles),
// two of them: window w (blocks 256w .. 256w+255, entries past the table
// clamped to its last one) in slot w % 2.  Group B, which has no copy in
// flight, loads the windows with vector loads (window 0 when the item
// starts, window w+1 during step 64w+1, written a step later); group A reads
// its block ids from them.  So the tile steps issue no scalar loads, which
// would hold up every LDS wait until they return.
constexpr int kWindow = 256;

__device__ __forceinline__ int window_entry(const int32_t* bt_row, int w, int wb, int lane, int nblk) {
  return bt_row[min(kWindow * w + 64 * wb + lane, nblk - 1)];
}

// Fourth word of a raw buffer descriptor on gfx950 (32-bit data, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

// Copy of one 16-key block straight from global memory into LDS: group A's
// wave w copies K of block 4t + w of a tile, group B's wave 4 + w copies V of
// that block, into the swizzled LDS rows 16w .. 16w+15 of the tile's slot.
// Each buffer_load_dwordx4 ... lds writes lane i's 16 bytes at M0 + 16 i, so
// lane i reads the global chunk that belongs at that LDS position.  The
// buffer range ends at the last key the item needs: rows past it, and every
// row of a block outside the pool, arrive as zeros (the range check of a raw
// buffer access returns zeros), without a branch.  The copies are issued as
// inline asm and waited for explicitly (copies_landed) before the barrier
// that hands the slot to its readers; the compiler, not knowing of them,
// adds no waits of its own to the LDS reads in between.
template <int D>
struct CopyOff {
  static constexpr int NCH = kBlock * Geo<D>::CPR / 64;   // copies per block
  uint32_t g[NCH];                                        // per-lane byte offsets into the block half
};

template <int D>
__device__ __forceinline__ CopyOff<D> copy_offsets(bool vhalf, int wq, int lane, uint32_t row_bytes) {
  using G = Geo<D>;
  CopyOff<D> o;
#pragma unroll
  for (int i = 0; i < CopyOff<D>::NCH; ++i) {
    const int j = lane + 64 * i;           // 16-byte position in the wave's rows
    const int row = j / G::CPR;            // row within the block
    const int pc = j % G::CPR;             // chunk position within the LDS row
    const int r = kBlock * wq + row;       // row within the tile
    // both swizzles are involutions: position pc holds chunk swizzle(r, pc)
    const int c = vhalf ? v_chunk<D>(r, pc) : k_chunk<D>(r, pc);
    o.g[i] = row * row_bytes + 16 * c;
  }
  return o;
}

// What a wave's block copies of one item share: the address of its group's
// half (K for group A, V for group B) of KV head g in block 0, the bytes
// from one block to the next and of one key row, and the pool's block count
// (capped at 2^31 - 1: every nonnegative 32-bit id below it is in the pool).
struct CopyGeo {
  uint64_t base;
  uint32_t bstride, rbytes, nb;
};

// Copy this wave's block (id bid, first key key0) of a tile into LDS at
// lds_dst.  Keys at or past kend (one past the item's last needed key) and
// every key of a block outside the pool arrive as zeros; a block outside the
// pool that holds needed keys sets bad.  All of it is scalar arithmetic:
// one unsigned compare checks the id, one 32 x 32 -> 64-bit product places
// the block.
template <int D>
__device__ __forceinline__ void copy_block(const CopyGeo& cg, int bid, int key0, int kend,
                                           const CopyOff<D>& co, uint32_t lds_dst, uint32_t& bad) {
  const uint32_t ub = (uint32_t)bid;
  const int nv = min(kend - key0, kBlock);   // keys of the block the item needs, if positive
  const bool need = nv > 0;
  const bool ok = ub < cg.nb;
  if (need && !ok) bad = 1;
  // a select, not a clamp: a clamp becomes a vector med3
  const uint32_t records = need && ok ? (uint32_t)nv * cg.rbytes : 0u;
  const uint64_t base = cg.base + (uint64_t)(ok ? ub : 0u) * cg.bstride;
  // every field is wave-uniform; readfirstlane keeps the descriptor in SGPRs
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xffffu)),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)records),
                    (uint32_t)kRsrcWord3};
  // one asm block: copy i lands 1 KiB after copy i-1 (M0 steps by 0x400;
  // an M0 write needs one wait state before the copy that uses it)
  if constexpr (CopyOff<D>::NCH == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds"
        :: "s"(lds_dst), "v"(co.g[0]), "v"(co.g[1]), "v"(co.g[2]), "v"(co.g[3]), "s"(rs)
        : "memory", "scc", "m0");
  } else {
    static_assert(CopyOff<D>::NCH == 2, "copies per block");
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
        :: "s"(lds_dst), "v"(co.g[0]), "v"(co.g[1]), "s"(rs) : "memory", "scc", "m0");
  }
}

// Wait until all but the last N of this wave's copies have landed in LDS
// (the wave issues no other vector memory operations meanwhile).
template <int N>
__device__ __forceinline__ void copies_landed() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const PKV_LDS char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// Order of a matrix phase: a few LDS reads ahead, then one MFMA per read
// (two reads per MFMA for the transposed V operand), so only a handful of
// operand fragments are live at a time; VALU independent vector
// instructions go after each MFMA, where they issue while it runs.
template <int MFMAS, int READS, int LEAD, int VALU = 0>
__device__ __forceinline__ void pipe_order() {
#pragma unroll
  for (int i = 0; i < LEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
#pragma unroll
  for (int i = 0; i < MFMAS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + LEAD < MFMAS) __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
    if (VALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
  }
}

// S^T of this wave's 32 queries over the two 32-key halves of the K tile `kt_lds`.
template <int D, int VALU = 0>
__device__ __forceinline__ void qk(f32x16 (&s)[2], const u32x4 (&q)[Geo<D>::NSL],
                                   const uint32_t (&ak)[Geo<D>::NSL], const PKV_LDS char* kt_lds) {
  using G = Geo<D>;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int sl = 0; sl < G::NSL; ++sl) {
      const u32x4 k =
          *reinterpret_cast<const PKV_LDS u32x4*>(kt_lds + ak[sl] + kt * 32 * G::ROWB);
      s[kt] = mfma32(k, q[sl], sl == 0 ? f32x16{} : s[kt]);
    }
  }
  pipe_order<2 * G::NSL, 1, kQkLead, VALU>();
}

// Scale O by alpha in the lanes whose maximum moved (a divergent branch:
// the multiplies run in place under the exec mask and are skipped when no
// lane of the wave needs them).
template <int D>
__device__ __forceinline__ void rescale_o(f32x16 (&o)[Geo<D>::NDT], float alpha) {
  if (alpha != 1.f) {
#pragma unroll
    for (int dt = 0; dt < Geo<D>::NDT; ++dt) o[dt] *= alpha;
  }
}

// O^T += V^T P^T over the V tile `vt_lds`.
template <int D, int VALU = 0>
__device__ __forceinline__ void pv(f32x16 (&o)[Geo<D>::NDT], const u32x4 (&pr)[2][2],
                                   const uint32_t (&av)[Geo<D>::NDT], const PKV_LDS char* vt_lds) {
  using G = Geo<D>;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int dt = 0; dt < G::NDT; ++dt) {
        const PKV_LDS char* at = vt_lds + av[dt] + (32 * kt + 16 * u) * G::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4*)at);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4*)(at + 8 * G::ROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        o[dt] = mfma32(u32x4{l2[0], l2[1], h2[0], h2[1]}, pr[kt][u], o[dt]);
      }
    }
  }
  pipe_order<4 * G::NDT, 2, kPvLead, VALU>();
}

// The matrix phase at head size 128 as one fixed instruction stream (the
// schedule comes from gen_matrix_phase.py): QK(t) and PV(t-1) back to back
// with the operand reads three groups ahead and every wait counting only the
// reads issued after the one it needs.  (The compiler's own schedule of the
// two loops drains the reads at the end of QK and leaves several reads one
// MFMA ahead.)  Two scalar branches inside the stream skip PV at t = 0 (no
// P yet: tt = t is zero) and QK at t = ntiles (no tile left to score: qrem =
// ntiles - t is zero).  The branches are the stream's own, so one asm
// statement serves every step and the accumulators stay in the same
// registers (alternative statements on different paths make the compiler
// copy them and spill).  ak and av hold the lane's offsets plus
// the slot array's base; KB and VB are the K and V slot's offsets in it.
static_assert(PKV_MAT_RING_FIRST == 240, "the clobber list names the schedule's ring registers");

template <int KB, int VB>
__device__ __forceinline__ void matrix_phase_128(f32x16 (&s)[2], f32x16 (&o)[4], const u32x4 (&q)[8],
                                                 const u32x4 (&pr)[2][2], const uint32_t (&ak)[8],
                                                 const uint32_t (&av)[4], int qrem, int tt) {
  asm volatile(PKV_MAT_QKPV
               : [s0] "=&v"(s[0]), [s1] "=&v"(s[1]), [o0] "+v"(o[0]), [o1] "+v"(o[1]), [o2] "+v"(o[2]),
                 [o3] "+v"(o[3])
               : [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]),
                 [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [p0] "v"(pr[0][0]), [p1] "v"(pr[0][1]),
                 [p2] "v"(pr[1][0]), [p3] "v"(pr[1][1]), [k0] "v"(ak[0]), [k1] "v"(ak[1]), [k2] "v"(ak[2]),
                 [k3] "v"(ak[3]), [k4] "v"(ak[4]), [k5] "v"(ak[5]), [k6] "v"(ak[6]), [k7] "v"(ak[7]),
                 [v0] "v"(av[0]), [v1] "v"(av[1]), [v2] "v"(av[2]), [v3] "v"(av[3]), [kb] "n"(KB),
                 [vb] "n"(VB), [qrem] "s"(qrem), [tt] "s"(tt)
               : "memory", "scc", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249",
                 "v250", "v251", "v252", "v253", "v254", "v255");
}

// Online softmax of one tile, in two parts so the matrix phase can take
// the first:
//   tile_max  the row maximum of the tile's scores (after dropping keys past
//             lim in a diagonal tile), both halves of the wave combined;
//   tile_exp  moves the lazy maximum m, sets alpha (the factor O and l are
//             scaled by: 1 unless the lane's maximum moved), turns the
//             scores into P = exp2(S c - m c) (bf16, as the B operands of
//             PV) and adds their fp32 row sum to l.
template <bool MASK>
__device__ __forceinline__ float tile_max(f32x16 (&s)[2], int k0, int lim, int lane) {
  if constexpr (MASK) {
    // key of register r of half kt = k0 + 4h + (32kt + 8(r/4) + r%4); the
    // distance t = lim - key is compared with 0 in float arithmetic: a
    // dropped key gets t * 1e38 <= -1e38 added (-inf for t <= -4), a kept one
    // gets 0.  No lane masks or selects, and the scores are finite, so no NaN.
    const float fb = (float)(lim - k0 - 4 * (lane >> 5));
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float t = fb - (float)(32 * kt + 8 * (r >> 2) + (r & 3));
        s[kt][r] = fmaf(fminf(t, 0.f), 1e38f, s[kt][r]);
      }
  }
  // a tree of three-input maxima (v_max3_f32): 16 instructions for 32 values
  float a[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int j = 3 * i;
    a[i] = fmaxf(fmaxf(s[j / 16][j % 16], s[(j + 1) / 16][(j + 1) % 16]), s[(j + 2) / 16][(j + 2) % 16]);
  }
  a[10] = fmaxf(s[1][14], s[1][15]);
  const float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]);
  const float b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float b2 = fmaxf(fmaxf(a[6], a[7]), a[8]);
  const float b3 = fmaxf(a[9], a[10]);
  const float mx = fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
  return halves_max(mx);
}

__device__ __forceinline__ void tile_exp(const f32x16 (&s)[2], float mx, u32x4 (&pr)[2][2],
                                         float& alpha, float& m, float& l, float c) {
  const bool first = m == -INFINITY;
  const bool upd = first || (mx - m) * c > kLazyMax;
  alpha = upd ? (first ? 0.f : fast_exp2((m - mx) * c)) : 1.f;
  l *= alpha;
  m = upd ? mx : m;
  const float mc = m * c;
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * u + 2 * i;
        const float e0 = fast_exp2(fmaf(s[kt][r], c, -mc));
        const float e1 = fast_exp2(fmaf(s[kt][r + 1], c, -mc));
        w[i] = pack_bf16(e0, e1);
        const bool first = kt == 0 && u == 0 && i == 0;   // no add to a zero start
        sa = first ? e0 : sa + e0;
        sb = first ? e1 : sb + e1;
      }
      pr[kt][u] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  l += sa + sb;
}

// Everything one wave needs for one work item.
template <int D>
struct Item {
  const int32_t* bt_row;
  int nblk;    // ceil(L / 16): entries of the block table in use
  int L, n, h, g, head, qw, kmax, ntiles, kfull, kend, lim, qi, tok0;
  bool active;
  CopyGeo cg;  // this wave's block copies
};

// Item itx (descriptor d, in LDS) as this wave sees it.
template <int D>
__device__ __forceinline__ Item<D> item_of(const PrefillParams& p, const PrefillItem* d,
                                           int itx, int per_entry, int queue, int wave, int lane) {
  const int sub = itx % per_entry;
  const int hc = sub % p.head_chunks;
  const int s = __builtin_amdgcn_readfirstlane(d->seq);
  const int qt = __builtin_amdgcn_readfirstlane(d->qt);
  const int hw = p.heads_per_item;
  Item<D> it;
  it.g = queue + p.num_queues * (sub / p.head_chunks);
  it.L = __builtin_amdgcn_readfirstlane(d->L);
  it.tok0 = __builtin_amdgcn_readfirstlane(d->tok0);
  it.n = __builtin_amdgcn_readfirstlane(d->n);
  it.h = it.L - it.n;
  it.head = it.g * p.group + hc * hw + wave % hw;
  it.qw = qt * p.query_tile + (wave / hw) * 32;                 // first query of this wave
  it.kmax = it.h + min(it.n, (qt + 1) * p.query_tile);          // keys the item needs
  it.ntiles = (it.kmax + kKeys - 1) / kKeys;
  it.active = it.qw < it.n;                                     // wave has real queries
  it.kfull = it.h + it.qw + 1;                                  // keys all its queries see
  it.kend = it.h + min(it.n - 1, it.qw + 31) + 1;               // keys some query sees
  it.bt_row = p.bt + (int64_t)s * p.width;
  it.nblk = (it.L + kBlock - 1) / kBlock;
  it.qi = it.qw + (lane & 31);
  it.lim = it.h + it.qi;
  const uint32_t rbytes = (uint32_t)(p.hkv * D * 2);
  it.cg.rbytes = rbytes;
  it.cg.bstride = 2 * kBlock * rbytes;
  it.cg.nb = (uint32_t)min(p.num_blocks, (int64_t)INT32_MAX);
  it.cg.base = reinterpret_cast<uint64_t>(p.cache) + (wave >= kWaves / 2 ? (uint64_t)kBlock * rbytes : 0) +
               (uint64_t)it.g * D * 2;
  return it;
}

// LDS slots: K of three tiles (tile j in slot j % 3) and V of two (slot
// j % 2).
template <int D>
struct Slots {
  PKV_LDS char* k[3];
  PKV_LDS char* v[2];
};

// The workgroup's queue has run dry: its next item comes from the queue with
// the most items left (that item's K/V are then not in this XCD's L2 but come
// from HBM or the last-level cache), at the cost of one read of the eight
// counters and one atomic.  A race that empties that queue too ends the
// workgroup.
__device__ __forceinline__ int steal_item(const PrefillParams& p, int n_items, int& nq, int lane) {
  int left = -1;
  if (lane < p.num_queues)
    left = n_items - __hip_atomic_load(&p.hdr->prefill_next[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int best = 0, bq = 0;
#pragma unroll
  for (int k = 0; k < kMaxQueues; ++k) {
    const int lk = __builtin_amdgcn_readlane(left, k);
    if (lk > best) {
      best = lk;
      bq = k;
    }
  }
  if (best <= 0) return n_items;
  int v = 0;
  if (lane == 0) v = atomicAdd(&p.hdr->prefill_next[bq], 1);
  nq = bq;
  return __builtin_amdgcn_readfirstlane(__shfl(v, 0));
}

// One tile step t (S = t % 6: the K slots cycle over three, the V slots over
// two, so every slot address is a compile-time constant) of one wave: QK(t) and PV(t-1) on the
// matrix cores, a barrier, the softmax of tile t, a barrier.  Group B runs
// the same sequence one phase later (it passes one extra barrier first), so
// each SIMD pairs one wave's matrix phase with the other's softmax.  With
// barrier 2t opening group A's step t:
//   group A: matrix phase (2t, 2t+1], softmax phase (2t+1, 2t+2];
//   group B: matrix phase (2t+1, 2t+2], softmax phase (2t+2, 2t+3].
// Copies:
//   wave w of group A copies block w of K(t+2) into the slot of K(t-1) at
//     the end of its matrix phase of step t, and waits for it before its
//     closing barrier of step t+1 (barrier 2t+4);
//   wave w of group B copies block w of V(t+1) into the slot of V(t-1) when
//     its softmax phase of step t starts, and waits for it before the end of
//     its matrix phase of step t+1 (2t+4).
// The K slot's last readers (group B's QK(t-1)) finished by barrier 2t; the
// V slot's (group B's PV(t-1)) by barrier 2t+2; the copying wave has passed
// both.  The first readers of the new tiles (group A's QK(t+2) and
// PV(t+1)) start after barrier 2t+4.  The products of both groups between
// those barriers read the other slots.
template <int D, int S>
__device__ __forceinline__ void tile_step(const PrefillParams& p, const Item<D>& it, const Slots<D>& sl,
                                          int t, bool group_b, int wave, int lane,
                                          const u32x4 (&q)[Geo<D>::NSL], f32x16 (&o)[Geo<D>::NDT],
                                          f32x16 (&sc)[2], u32x4 (&pr)[2][2], float& alpha, float& m,
                                          float& l, const uint32_t (&ak)[Geo<D>::NSL],
                                          const uint32_t (&av)[Geo<D>::NDT], const CopyOff<D>& ck,
                                          const CopyOff<D>& cv, int32_t (*bt)[kWindow],
                                          int& bt_next, uint32_t& bad, int& nxt, int& nq, int& nxt_word,
                                          int n_items, int per_entry) {
  constexpr int RK = S % 3;              // K slot of tile t
  constexpr int RP = (RK + 2) % 3;       // K slot of tiles t - 1 and t + 2
  constexpr int RV = (S % 2) ^ 1;        // V slot of tiles t - 1 and t + 1
  constexpr uint32_t kBlockBytes = kBlock * Geo<D>::ROWB;   // LDS bytes of one block's rows
  const int wq = wave & 3;
  // Matrix phase: QK(t) and PV(t-1); the first step skips PV and the last
  // QK (wave-uniform branches, at head size 128 inside the stream).  A tile
  // the wave's queries do not see (past every key they see) has P = 0, and
  // every slot read holds finite values, so its products change nothing.
  PKV_LDS char* const v_prev = sl.v[RV];
  // The partner wave of this SIMD runs its softmax meanwhile: this wave's
  // products go first when both have an instruction ready.
  __builtin_amdgcn_s_setprio(1);
  if constexpr (D == 128) {
    matrix_phase_128<RK * Geo<D>::TILEB, RV * Geo<D>::TILEB>(sc, o, q, pr, ak, av,
                                                             __builtin_amdgcn_readfirstlane(it.ntiles - t),
                                                             __builtin_amdgcn_readfirstlane(t));
  } else {
    if (t < it.ntiles) qk<D>(sc, q, ak, sl.k[RK]);
    if (t > 0) pv<D>(o, pr, av, v_prev);
  }
  __builtin_amdgcn_s_setprio(0);
  if (!group_b) {
    // after the products are issued, while the last of them run
    const uint32_t bk = 4 * (t + 2) + wq;   // block of K(t+2); window (bk / 256) % 2
    const int bid_k = __builtin_amdgcn_readfirstlane((&bt[0][0])[bk & (2 * kWindow - 1)]);
    copy_block<D>(it.cg, bid_k, kKeys * (t + 2) + kBlock * wq, it.kmax, ck,
                  lds_addr(sl.k[RP]) + wq * kBlockBytes, bad);
  }
  if (group_b) copies_landed<0>();   // V(t), copied during the step before
  wg_barrier();
  if (group_b) {
    // Uses of values loaded during earlier steps come before this step's
    // copy: the compiler waits for those loads there (every load of the
    // wave has landed by then, before its matrix phase ended), so nothing
    // waits for the copy.
    const int w = t / 64 + 1;   // the window after the current one
    if ((t & 63) == 2 && kWindow * w < it.nblk) bt[w & 1][64 * (wave - kWaves / 2) + lane] = bt_next;
    if (wave == kWaves / 2 && t == 1) {
      // the next item: its index (asked for when this item started) and its
      // descriptor, one dword per lane, written to LDS when this item ends
      nxt = __builtin_amdgcn_readfirstlane(nxt);
      if (nxt >= n_items && p.num_queues > 1) nxt = steal_item(p, n_items, nq, lane);
      const int32_t* src = reinterpret_cast<const int32_t*>(p.items + min(nxt, n_items - 1) / per_entry);
      nxt_word = src[lane & 15];
    }
    const uint32_t bv = 4 * (t + 1) + wq;   // block of V(t+1)
    const int bid_v = __builtin_amdgcn_readfirstlane((&bt[0][0])[bv & (2 * kWindow - 1)]);
    copy_block<D>(it.cg, bid_v, kKeys * (t + 1) + kBlock * wq, it.kmax, cv,
                  lds_addr(v_prev) + wq * kBlockBytes, bad);
    if ((t & 63) == 1 && kWindow * w < it.nblk) bt_next = window_entry(it.bt_row, w, wave - kWaves / 2, lane, it.nblk);
  }
  // tile t for the softmax; tiles no query of the wave sees are skipped
  const bool do_t = it.active && t < it.ntiles && kKeys * t < it.kend;
  if (do_t) {
    // a diagonal tile (some query of the wave drops keys of it) is masked
    const float mx = kKeys * t + kKeys > it.kfull ? tile_max<true>(sc, kKeys * t, it.lim, lane)
                                                  : tile_max<false>(sc, kKeys * t, it.lim, lane);
    tile_exp(sc, mx, pr, alpha, m, l, p.c);
    rescale_o<D>(o, alpha);   // O is scaled before the next PV adds tile t
  } else {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) pr[kt][u] = u32x4{0u, 0u, 0u, 0u};
  }
  // group A: the copy of the step before has landed (this step's may not)
  if (!group_b) copies_landed<CopyOff<D>::NCH>();
  __syncthreads();
}

// Queries of one wave (32 rows from row qw of the segment, one head) into
// its LDS area with global -> LDS copies: copy k puts rows RPI*k .. of the
// area in place, lane i the 16-byte chunk at position i % CPR of row
// RPI*k + i / CPR, which holds chunk position ^ (row % CPR) of that row (the
// same swizzle as K), so the 16 lanes of a row read one contiguous row.  Rows
// past the segment's end arrive as zeros (range-checked buffer).
template <int D>
__device__ __forceinline__ void copy_queries(const PrefillParams& p, int tok0, int qw, int n, int head,
                                             int lane, uint32_t lds_dst) {
  using G = Geo<D>;
  // the per-lane offsets are recomputed here (a few instructions per item)
  // rather than hoisted out of the item loop, where they would hold
  // registers through every tile step
  asm volatile("" : "+v"(lane));
  constexpr int RPI = 1024 / G::ROWB;          // rows per copy
  constexpr int NQ = 32 / RPI;                 // copies per wave
  const int64_t rstride = p.q_stride * 2;      // bytes between query rows
  const int rows = min(max(n - qw, 0), 32);
  const char* base = reinterpret_cast<const char*>(p.q) + ((int64_t)(tok0 + qw) * p.q_stride + (int64_t)head * D) * 2;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(base), (short)0,
      __builtin_amdgcn_readfirstlane(rows > 0 ? (int)(rows * rstride) : 0), kRsrcWord3);
  uint32_t off[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int r = RPI * k + lane / G::CPR;
    off[k] = (uint32_t)(r * rstride) + 16 * k_chunk<D>(r, lane % G::CPR);
  }
  if constexpr (NQ == 8) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %7, %9, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %8, %9, 0 offen lds"
        :: "s"(lds_dst), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]),
           "v"(off[5]), "v"(off[6]), "v"(off[7]), "s"(rs)
        : "memory", "scc", "m0");
  } else {
    static_assert(NQ == 4, "copies per wave");
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds"
        :: "s"(lds_dst), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(rs)
        : "memory", "scc", "m0");
  }
}

// The wave's queries from its LDS area into the B operands of QK^T (lane:
// row lane % 32, d-chunk 2i + lane / 32 of slab i), sign applied.
template <int D>
__device__ __forceinline__ void read_queries(u32x4 (&q)[Geo<D>::NSL], const PKV_LDS char* io,
                                             int lane, uint32_t q_sign) {
  using G = Geo<D>;
  const int r = lane & 31;
#pragma unroll
  for (int i = 0; i < G::NSL; ++i)
    q[i] = *reinterpret_cast<const PKV_LDS u32x4*>(io + r * G::ROWB + 16 * k_chunk<D>(r, 2 * i + (lane >> 5))) ^ q_sign;
}

// Normalise the wave's output and store it: bf16 pairs into its LDS area
// (lane: row lane % 32, d = 32dt + 8i + 4(lane/32) + 0..3, same swizzle),
// then whole rows out, 16 lanes per 256-byte row, through a range-checked
// buffer that drops rows past the segment's end.
template <int D>
__device__ __forceinline__ void store_output(const PrefillParams& p, const f32x16 (&o)[Geo<D>::NDT],
                                             float lt, int tok0, int qw, int n, int head, int lane,
                                             PKV_LDS char* io) {
  using G = Geo<D>;
  constexpr int RPI = 1024 / G::ROWB;
  constexpr int NQ = 32 / RPI;
  asm volatile("" : "+v"(lane));   // offsets computed here, not hoisted (see copy_queries)
  const float inv = __builtin_amdgcn_rcpf(lt);
  const int r = lane & 31;
#pragma unroll
  for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<PKV_LDS u32x2*>(io + r * G::ROWB + 16 * k_chunk<D>(r, 4 * dt + i) + 8 * (lane >> 5)) =
          u32x2{pack_bf16(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv),
                pack_bf16(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv)};
  const int64_t rstride = (int64_t)p.hq * D * 2;   // bytes between output rows
  const int rows = min(max(n - qw, 0), 32);
  const char* base = reinterpret_cast<const char*>(p.out) + ((int64_t)(tok0 + qw) * p.hq + head) * D * 2;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(base), (short)0,
      __builtin_amdgcn_readfirstlane(rows > 0 ? (int)(rows * rstride) : 0), kRsrcWord3);
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int rr = RPI * k + lane / G::CPR;
    const int pc = lane % G::CPR;
    const u32x4 v = *reinterpret_cast<const PKV_LDS u32x4*>(io + rr * G::ROWB + 16 * pc);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (uint32_t)(rr * rstride) + 16 * k_chunk<D>(rr, pc), 0, 0);
  }
}

template <int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
prefill_kernel(PrefillParams p) {
  using G = Geo<D>;
  // The five tile slots are one array (K slots 0-2, V slots 0-1), aligned
  // to a slot's size: the matrix phase addresses a slot with a lane's offset
  // in a register and the slot's place in the instruction's 16-bit offset
  // field, with no address arithmetic between the operand reads.
  __shared__ __attribute__((aligned(G::TILEB))) char kv_lds[5 * G::TILEB];   // K0 K1 K2 V0 V1
  // per wave: its queries on their way in, its output on its way out
  __shared__ __attribute__((aligned(1024))) char io_lds[kWaves][32 * G::ROWB];
  __shared__ PrefillItem s_desc[2];   // the current and the next item
  __shared__ int s_itx[2];
  __shared__ int s_q[2];              // the queues they came from
  __shared__ int32_t s_bt[2][kWindow];   // block-table windows of the current item
  PKV_LDS char* const kv = (PKV_LDS char*)kv_lds;
  const Slots<D> sl = {{kv, kv + G::TILEB, kv + 2 * G::TILEB}, {kv + 3 * G::TILEB, kv + 4 * G::TILEB}};
  PKV_LDS char* const io = (PKV_LDS char*)io_lds[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_b = wave >= kWaves / 2;
  const int per_entry = (p.hkv / p.num_queues) * p.head_chunks;
  const int queue = blockIdx.x % p.num_queues;
  const int n_items = p.hdr->n_prefill * per_entry;
  if (n_items == 0) return;   // no prefill segment in this step

  // per-lane LDS addresses within a slot
  uint32_t ak[G::NSL], av[G::NDT];
  {
    const int hh = lane >> 5;
    const int r = lane & 31;
#pragma unroll
    for (int i = 0; i < G::NSL; ++i) ak[i] = r * G::ROWB + 16 * k_chunk<D>(r, 2 * i + hh);
    const int rr = 4 * hh + ((lane & 15) >> 2);   // row within a 16-key slab
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) {
      const int d = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      av[dt] = rr * G::ROWB + 16 * v_chunk<D>(rr, d >> 3) + 2 * (d & 7);
    }
    if constexpr (D == 128) {
      // the asm matrix phase addresses a slot by its offset in kv_lds
#pragma unroll
      for (int i = 0; i < G::NSL; ++i) ak[i] += lds_addr(sl.k[0]);
#pragma unroll
      for (int dt = 0; dt < G::NDT; ++dt) av[dt] += lds_addr(sl.v[0]);
    }
  }

  // group A copies only K and group B only V: one set of lane offsets each
  const CopyOff<D> ck = copy_offsets<D>(group_b, wave & 3, lane, (uint32_t)(p.hkv * D * 2));
  const CopyOff<D>& cv = ck;

  // the first item: wave 4 asks for its index and reads its descriptor
  if (wave == kWaves / 2) {
    int itx0 = 0;
    if (lane == 0) itx0 = atomicAdd(&p.hdr->prefill_next[queue], 1);
    itx0 = __builtin_amdgcn_readfirstlane(itx0);
    if (lane < 16) {
      const int32_t* src = reinterpret_cast<const int32_t*>(p.items + min(itx0, n_items - 1) / per_entry);
      reinterpret_cast<int32_t*>(&s_desc[0])[lane] = src[lane];
    }
    if (lane == 0) {
      s_itx[0] = itx0;
      s_q[0] = queue;
    }
  }
  __syncthreads();
  int cur = 0;
  int itx = s_itx[0];
  if (itx >= n_items) return;
  Item<D> it = item_of<D>(p, &s_desc[0], itx, per_entry, queue, wave, lane);

  const int wq = wave & 3;
  u32x4 q[G::NSL];
  int bt_next = 0;   // group B: a lane's entry of the next block-table window
  uint32_t bad = 0;
  // Start of an item: its queries into the wave's LDS area, the copies of
  // K(0), K(1) (group A) and V(0) (group B), one block per wave each, with the
  // block ids from the descriptor, and (group B) the loads of block-table
  // window 0, written when the item runs.  (The first step runs no PV, so the
  // other V slot is not read before V(1) lands in it.)
  auto start_item = [&](const Item<D>& nx, const PrefillItem* d) {
    // the descriptor's block ids are read before any copy is issued: the
    // wait for an LDS read would otherwise also wait for the copies
    const int bid0 = __builtin_amdgcn_readfirstlane(d->bid[wq]);
    const int bid1 = __builtin_amdgcn_readfirstlane(d->bid[4 + wq]);   // block of tile 1
    if (group_b) bt_next = window_entry(nx.bt_row, 0, wave - kWaves / 2, lane, nx.nblk);
    copy_queries<D>(p, nx.tok0, nx.qw, nx.n, nx.head, lane, lds_addr(io));
    if (!group_b) {
      copy_block<D>(nx.cg, bid0, kBlock * wq, nx.kmax, ck, lds_addr(sl.k[0]) + wq * kBlock * G::ROWB, bad);
      copy_block<D>(nx.cg, bid1, kKeys + kBlock * wq, nx.kmax, ck, lds_addr(sl.k[1]) + wq * kBlock * G::ROWB,
                    bad);
    } else {
      copy_block<D>(nx.cg, bid0, kBlock * wq, nx.kmax, cv, lds_addr(sl.v[0]) + wq * kBlock * G::ROWB, bad);
    }
  };
  start_item(it, &s_desc[0]);

  for (;;) {
    int nxt = 0, nxt_word = 0;   // wave 4: the next item's index and descriptor
    const int cq = __builtin_amdgcn_readfirstlane(s_q[cur]);   // the queue of the current item
    int nq = cq;                 // wave 4: the queue of the next item
    f32x16 o[G::NDT];
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) o[dt] = f32x16{};
    float m = -INFINITY, l = 0.f, alpha = 1.f;
    f32x16 sc[2];
    u32x4 pr[2][2];   // P of the tile before the first: zero
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) pr[kt][u] = u32x4{0u, 0u, 0u, 0u};

    if (group_b) s_bt[0][64 * (wave - kWaves / 2) + lane] = bt_next;   // window 0
    copies_landed<0>();   // the copies of K/V and of the queries
    __syncthreads();   // K(0), K(1), V(0), window 0 in LDS
    read_queries<D>(q, io, lane, p.q_sign);
    // asked for only now, so the wait for the copies above does not include it
    if (wave == kWaves / 2 && lane == 0) nxt = atomicAdd(&p.hdr->prefill_next[cq], 1);
    if (group_b) wg_barrier();
#define PKV_STEP(S)                                                                          \
  tile_step<D, S>(p, it, sl, t + S, group_b, wave, lane, q, o, sc, pr, alpha, m, l, ak, av, ck, \
                  cv, s_bt, bt_next, bad, nxt, nq, nxt_word, n_items, per_entry)
    for (int t = 0; t <= it.ntiles; t += 6) {
      PKV_STEP(0);
      if (t + 1 > it.ntiles) break;
      PKV_STEP(1);
      if (t + 2 > it.ntiles) break;
      PKV_STEP(2);
      if (t + 3 > it.ntiles) break;
      PKV_STEP(3);
      if (t + 4 > it.ntiles) break;
      PKV_STEP(4);
      if (t + 5 > it.ntiles) break;
      PKV_STEP(5);
    }
#undef PKV_STEP
    copies_landed<0>();     // nothing in flight into the slots past the item
    if (!group_b) wg_barrier();   // group B's last step ends here
    if (wave == kWaves / 2) {
      if (lane < 16) reinterpret_cast<int32_t*>(&s_desc[cur ^ 1])[lane] = nxt_word;
      if (lane == 0) {
        s_itx[cur ^ 1] = nxt;
        s_q[cur ^ 1] = nq;
      }
    }
    __syncthreads();   // every slot read; the next item's descriptor in LDS

    const int itx_n = s_itx[cur ^ 1];
    const Item<D> prev = it;
    if (itx_n < n_items)
      it = item_of<D>(p, &s_desc[cur ^ 1], itx_n, per_entry, __builtin_amdgcn_readfirstlane(s_q[cur ^ 1]),
                      wave, lane);

    // normalise; out through the wave's LDS area, so the stores are whole rows
    store_output<D>(p, o, halves_sum(l), prev.tok0, prev.qw, prev.n, prev.head, lane, io);
    // the next item's queries (into the same area, once this wave's reads of
    // it have returned: the stores above consumed them) and first copies
    if (itx_n < n_items) start_item(it, &s_desc[cur ^ 1]);
    cur ^= 1;
    if (itx_n >= n_items) break;
  }
  if (bad && lane == 0) atomicOr(&p.hdr->status, 2u);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 128) {
    prefill_kernel<128><<<grid, 512, 0, stream>>>(p);
  } else {
    prefill_kernel<64><<<grid, 512, 0, stream>>>(p);
  }
  return hipGetLastError();
}

const void* prefill_kernel_ptr(int head_dim) {
  return head_dim == 128 ? (const void*)prefill_kernel<128> : (const void*)prefill_kernel<64>;
}

}  // namespace pkv
