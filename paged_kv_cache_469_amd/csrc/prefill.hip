// Prefill and chunked-prefill attention over the paged pool.
//
// What is computed ("vLLM 学习笔记 01", sections 1.4-1.6 and 2.1): a segment
// with n > 1 new tokens at the end of a sequence of L tokens (h = L - n of
// them cached earlier, h = 0 for a fresh prompt, h > 0 for a later chunk of a
// long prompt) attends causally: query i sees keys 0 .. h + i of its own
// sequence, read through its block table.  Prefill is a dense contraction
// ("从0开始的vLLM学习": prefill is compute bound), so both products run on
// the bf16 matrix cores.
//
// Work item: (segment, query tile, KV head, head chunk), run by a workgroup
// of 4 waves.  Each wave owns one query head and 32 queries; the 4 waves of a
// workgroup share the KV head, so each 64-key K/V tile is gathered from its
// four 16-token blocks once into LDS and used by all of them.  Per wave, per
// 32 keys:
//   S^T[key, q] = K[key, :] . Q[q, :]        32x32x16 bf16 MFMA over D/16 slabs
//   causal mask (only on tiles that cross the diagonal), online softmax in
//   fp32 with exp2 (scale*log2(e) folded in)
//   O^T[d, q] += V^T[d, key] . P^T[key, q]   32x32x16 bf16 MFMA, D/32 d tiles
// The C layout of S^T (lane = query, 16 keys per lane) is the B operand layout
// of the second product, so P stays in registers.  LDS rows are XOR-swizzled
// in 16-byte chunks by row so the K operand reads (32 rows, one chunk each)
// and the V reads are free of bank conflicts; V is read with a permuted d
// order (tile t, row m <-> d = (D/32)*m + t) and transposed with v_perm.
// Keys at or past L are written to LDS as zeros, never loaded.
#include "kernels.hpp"

namespace pkv {

constexpr int kTileKeys = 64;

template <int D>
struct PrefillTile {
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int CHUNKS = kTileKeys * CPR;       // per K (or V) tile
  static constexpr int PER_THREAD = CHUNKS / 256;      // 4 for D = 128
  static constexpr int ELEMS = kTileKeys * D;          // bf16 per K (or V) tile
};

template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * D + ((chunk ^ (row & (PrefillTile<D>::CPR - 1))) << 3);
}

template <int D>
__device__ __forceinline__ void gather_tile(u32x4 (&kr)[PrefillTile<D>::PER_THREAD],
                                            u32x4 (&vr)[PrefillTile<D>::PER_THREAD],
                                            const PrefillParams& p, const int32_t* bt_row,
                                            int k0, int L, int g, int64_t row_elems,
                                            int64_t block_elems, uint32_t& bad) {
  constexpr int CPR = PrefillTile<D>::CPR;
#pragma unroll
  for (int i = 0; i < PrefillTile<D>::PER_THREAD; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / CPR;
    const int ch = c % CPR;
    const int key = k0 + row;
    u32x4 z = {0u, 0u, 0u, 0u};
    kr[i] = z;
    vr[i] = z;
    if (key < L) {
      const int bid = bt_row[key / kBlock];
      if (bid >= 0 && (int64_t)bid < p.num_blocks) {
        const uint16_t* src = p.cache + (int64_t)bid * block_elems +
                              (int64_t)(key % kBlock) * row_elems + (int64_t)g * D + ch * 8;
        kr[i] = *reinterpret_cast<const u32x4*>(src);
        vr[i] = *reinterpret_cast<const u32x4*>(src + kBlock * row_elems);
      } else {
        bad = 1;
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(uint16_t* lk, uint16_t* lv,
                                           const u32x4 (&kr)[PrefillTile<D>::PER_THREAD],
                                           const u32x4 (&vr)[PrefillTile<D>::PER_THREAD]) {
  constexpr int CPR = PrefillTile<D>::CPR;
#pragma unroll
  for (int i = 0; i < PrefillTile<D>::PER_THREAD; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int at = swz<D>(c / CPR, c % CPR);
    *reinterpret_cast<u32x4*>(lk + at) = kr[i];
    *reinterpret_cast<u32x4*>(lv + at) = vr[i];
  }
}

template <int D>
__global__ void __launch_bounds__(256)
prefill_kernel(PrefillParams p) {
  constexpr int NSL = D / 16;    // k slabs of the QK product
  constexpr int NDT = D / 32;    // d tiles of the PV product
  constexpr int CPR = PrefillTile<D>::CPR;
  constexpr int PT = PrefillTile<D>::PER_THREAD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][PrefillTile<D>::ELEMS];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;     // query within the wave's 32
  const int j = lane >> 5;       // k group of the MFMA operands
  const int per_tile = p.hkv * p.head_chunks;
  const int n_items = p.hdr->n_prefill * per_tile;
  const int64_t row_elems = (int64_t)p.hkv * D;
  const int64_t block_elems = 2 * kBlock * row_elems;
  const int qblocks = 4 / p.heads_per_item;   // 32-query blocks per item

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&p.hdr->prefill_next, 1);
    __syncthreads();
    const int it = s_item;
    __syncthreads();
    if (it >= n_items) break;
    const int2 item = p.items[it / per_tile];
    const int sub = it % per_tile;
    const int g = sub / p.head_chunks;
    const int hc = sub % p.head_chunks;
    const int s = item.x;
    const int qt = item.y;
    const int L = p.lens[s];
    const int tok0 = p.cu[s];
    const int n = p.cu[s + 1] - tok0;
    const int h = L - n;
    const int head = g * p.group + hc * p.heads_per_item + (wave % p.heads_per_item);
    const int qb0 = (qt * qblocks + wave / p.heads_per_item) * 32;   // first query of the wave
    const int q_item_end = min(n, (qt + 1) * qblocks * 32);
    const int kmax = h + q_item_end;                                  // keys the item needs
    const int qi = qb0 + col;
    const int lim = h + min(qi, n - 1);                               // last key this lane sees
    const int32_t* bt_row = p.bt + (int64_t)s * p.width;

    u32x4 qf[NSL];
    {
      const uint16_t* qrow = p.q + (int64_t)(tok0 + qi) * p.q_stride + (int64_t)head * D + 8 * j;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qf[sl] = qi < n ? *reinterpret_cast<const u32x4*>(qrow + 16 * sl) : z;
      }
    }
    f32x16 o[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;
    uint32_t bad = 0;

    const int ntiles = (kmax + kTileKeys - 1) / kTileKeys;
    u32x4 kr[PT], vr[PT];
    gather_tile<D>(kr, vr, p, bt_row, 0, L, g, row_elems, block_elems, bad);
    store_tile<D>(lds[0][0], lds[0][1], kr, vr);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int k0 = t * kTileKeys;
      if (t + 1 < ntiles)
        gather_tile<D>(kr, vr, p, bt_row, k0 + kTileKeys, L, g, row_elems, block_elems, bad);
      const uint16_t* lk = lds[t & 1][0];
      const uint16_t* lv = lds[t & 1][1];

      // S^T for the two 32-key halves of the tile
      f32x16 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt] = f32x16{};
        const int row = kt * 32 + col;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(lk + swz<D>(row, 2 * sl + j));
          sc[kt] = mfma32(a, qf[sl], sc[kt]);
        }
      }
      // scores, causal mask where the tile crosses this wave's diagonal
      const bool need_mask = k0 + kTileKeys - 1 > h + qb0;
      float cmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[kt][r] * p.scale_log2;
          if (need_mask) {
            const int key = k0 + kt * 32 + 8 * (r >> 2) + 4 * j + (r & 3);
            x = key <= lim ? x : -INFINITY;
          }
          sc[kt][r] = x;
          cmax = fmaxf(cmax, x);
        }
      }
      cmax = wave_max_xor(cmax, 32);
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2f(sc[kt][r] - m_new);
          sc[kt][r] = e;
          psum += e;
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

      // O^T += V^T P^T over four 16-key slabs
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 pb = {pack_bf16(sc[kt][8 * u + 0], sc[kt][8 * u + 1]),
                            pack_bf16(sc[kt][8 * u + 2], sc[kt][8 * u + 3]),
                            pack_bf16(sc[kt][8 * u + 4], sc[kt][8 * u + 5]),
                            pack_bf16(sc[kt][8 * u + 6], sc[kt][8 * u + 7])};
          // lane's V pieces: 8 keys x (D/32) consecutive d starting at (D/32)*col
          uint32_t vv[8][NDT / 2 > 0 ? NDT / 2 : 1];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int row = kt * 32 + 16 * u + 8 * (e >> 2) + 4 * j + (e & 3);
            const int d0 = NDT * col;
            const uint16_t* src = lv + swz<D>(row, d0 >> 3) + (d0 & 7);
            if constexpr (NDT == 4) {
              const u32x2 x = *reinterpret_cast<const u32x2*>(src);
              vv[e][0] = x[0];
              vv[e][1] = x[1];
            } else {
              vv[e][0] = *reinterpret_cast<const uint32_t*>(src);
            }
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int w = dt >> 1;
            const bool hi = dt & 1;
            const u32x4 a = {pick_halves(vv[0][w], vv[1][w], hi), pick_halves(vv[2][w], vv[3][w], hi),
                             pick_halves(vv[4][w], vv[5][w], hi), pick_halves(vv[6][w], vv[7][w], hi)};
            o[dt] = mfma32(a, pb, o[dt]);
          }
        }
      }
      if (t + 1 < ntiles) store_tile<D>(lds[(t + 1) & 1][0], lds[(t + 1) & 1][1], kr, vr);
      __syncthreads();
    }
    if (bad && lane == 0) atomicOr(&p.hdr->status, 2u);

    l_run += __shfl_xor(l_run, 32);
    if (qi < n) {
      const float inv = 1.f / l_run;
      uint16_t* orow = p.out + ((int64_t)(tok0 + qi) * p.hq + head) * D;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int drow = 8 * (r >> 2) + 4 * j + (r & 3);
        uint16_t* dst = orow + NDT * drow;
        if constexpr (NDT == 4) {
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{pack_bf16(o[0][r] * inv, o[1][r] * inv), pack_bf16(o[2][r] * inv, o[3][r] * inv)};
        } else {
          *reinterpret_cast<uint32_t*>(dst) = pack_bf16(o[0][r] * inv, o[1][r] * inv);
        }
      }
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 128) {
    prefill_kernel<128><<<grid, 256, 0, stream>>>(p);
  } else {
    prefill_kernel<64><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

const void* prefill_kernel_ptr(int head_dim) {
  return head_dim == 128 ? (const void*)prefill_kernel<128> : (const void*)prefill_kernel<64>;
}

}  // namespace pkv
