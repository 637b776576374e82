"""Writes phase_probe.hip: the two kinds of work of a prefill tile step, side
by side on one CU, with every instruction stream fixed in inline asm.

  matrix block   the prefill kernel's matrix phase at head size 128: 16
                 MFMAs (32x32x16 bf16) whose A operand comes from
                 ds_read_b128 and 16 whose A operand comes from two
                 ds_read_b64_tr_b16, the reads three groups ahead with
                 counted waits (each wave reads its own 16 KiB of LDS)
  softmax block  the vector work of one tile's online softmax for one wave:
                 a tree of 3-input maxima over 32 scores, the lane-half
                 swap, the running-maximum update, 32 fma + exp, two chains
                 of row-sum adds, 16 bf16 packs (143 vector instructions,
                 33 of them v_exp_f32)

A "unit" is one matrix block plus one softmax block; a prefill step puts two
units on every SIMD (two waves, each with one of each).  Cases (cycles per
iteration from s_memtime around the loop, mean and slowest wave):

  matrix alone / softmax alone     one wave per SIMD running one block
  side by side                     wave w runs matrix blocks, wave w + 4
                                   softmax blocks on the same SIMD, no
                                   barriers (each side's own rate)
  ping-pong                        the kernel's order: group A matrix while
                                   group B softmax, a barrier, swapped, a
                                   barrier (matrix at s_setprio 1)
  ping-pong + copies               as the kernel: group A copies one 4 KiB
                                   block (global -> LDS) after its matrix
                                   block, group B before its softmax, with
                                   the kernel's waits; then with the block id
                                   read from an LDS table first
  softmax without exp / fma / adds / max / cvt
                                   ping-pong with one kind of instruction
                                   taken out of the softmax (timing only)
  + 80 scalar (softmax), + 40 (matrix), + 5 taken branches (softmax)
  one wave per SIMD: blocks in turn / interleaved (the softmax's
                                   instructions placed between the MFMAs)
  two waves per SIMD interleaved

and, separately, whether a global -> LDS copy (buffer_load ... lds) counts
in the LGKM counter: one wave per CU issues one and times s_waitcnt
lgkmcnt(0), then vmcnt(0).

Run from this folder: python gen_phase_probe.py (the generated file is
committed; build() compiles every probes/*.hip into an executable beside it).
"""

import os

HERE = os.path.dirname(os.path.abspath(__file__))
RING = 200   # v200 .. v219: the matrix block's operand ring (clobbered)
SB = 140     # v140 .. v171: softmax scores
PB = 172     # v172 .. v187: packed P
TT = 188     # v188 .. v199: softmax temporaries


def matrix_block():
    """[(kind, text)], kind 'mfma' or 'other'"""
    groups = []
    for g in range(32):
        b = RING + 4 * (g % 5)
        if g < 16:
            off = (g * 1024) % 16384 + (g * 1024 // 16384) * 16
            groups.append(([f"ds_read_b128 v[{b}:{b + 3}], %[addr] offset:{off}"], 1))
        else:
            off = ((g - 16) * 512) % 16384
            groups.append(([f"ds_read_b64_tr_b16 v[{b}:{b + 1}], %[addr2] offset:{off}",
                            f"ds_read_b64_tr_b16 v[{b + 2}:{b + 3}], %[addr2] offset:{off + 8208}"], 2))
    out, issued = [], 0
    for g in range(3):
        out += [("other", r) for r in groups[g][0]]
        issued += 1
    for g in range(32):
        after = sum(groups[j][1] for j in range(g + 1, issued))
        out.append(("other", f"s_waitcnt lgkmcnt({after})"))
        b = RING + 4 * (g % 5)
        acc = f"%[c{g % 4}]"
        out.append(("mfma", f"v_mfma_f32_32x32x16_bf16 {acc}, v[{b}:{b + 3}], %[b0], {acc}"))
        if issued < 32:
            out += [("other", r) for r in groups[issued][0]]
            issued += 1
    return out


def softmax_block():
    S = lambda i: f"v{SB + i}"
    T = lambda i: f"v{TT + i}"
    P = lambda i: f"v{PB + i}"
    head = []
    for i in range(10):
        head.append(f"v_max3_f32 {T(i)}, {S(3 * i)}, {S(3 * i + 1)}, {S(3 * i + 2)}")
    head += [f"v_max_f32_e32 {T(10)}, {S(30)}, {S(31)}",
             f"v_max3_f32 {T(0)}, {T(0)}, {T(1)}, {T(2)}",
             f"v_max3_f32 {T(3)}, {T(3)}, {T(4)}, {T(5)}",
             f"v_max3_f32 {T(6)}, {T(6)}, {T(7)}, {T(8)}",
             f"v_max_f32_e32 {T(9)}, {T(9)}, {T(10)}",
             f"v_max3_f32 {T(0)}, {T(0)}, {T(3)}, {T(6)}",
             f"v_max_f32_e32 {T(0)}, {T(0)}, {T(9)}",
             f"v_mov_b32_e32 {T(1)}, {T(0)}",
             "s_nop 1",
             f"v_permlane32_swap_b32 {T(0)}, {T(1)}",
             f"v_max_f32_e32 {T(0)}, {T(0)}, {T(1)}",
             # the running maximum and the factor of O (T11 holds m)
             f"v_sub_f32_e32 {T(2)}, {T(11)}, {T(0)}",
             f"v_mul_f32_e32 {T(2)}, %[c], {T(2)}",
             f"v_exp_f32_e32 {T(2)}, {T(2)}",
             f"v_sub_f32_e32 {T(3)}, {T(0)}, {T(11)}",
             f"v_mul_f32_e32 {T(3)}, %[c], {T(3)}",
             f"v_cmp_ge_f32_e32 vcc, 0x41000000, {T(3)}",
             f"v_cndmask_b32_e64 {T(2)}, {T(2)}, 1.0, vcc",
             f"v_cndmask_b32_e32 {T(11)}, {T(0)}, {T(11)}, vcc",
             f"v_mul_f32_e64 {T(4)}, {T(11)}, -%[c]"]
    body = []
    for i in range(32):
        body.append(f"v_fma_f32 {T(5 + i % 4)}, %[c], {S(i)}, {T(4)}")
        body.append(f"v_exp_f32_e32 {S(i)}, {T(5 + i % 4)}")
    sums = [f"v_mov_b32_e32 {T(9 + i)}, {S(i)}" for i in range(2)] + \
           [f"v_add_f32_e32 {T(9 + i % 2)}, {T(9 + i % 2)}, {S(i)}" for i in range(2, 32)]
    merged, ai, n_exp = [], 0, 0
    for ln in body:
        merged.append(ln)
        if ln.startswith("v_exp"):
            n_exp += 1
            while ai < 32 and ai <= n_exp - 4:   # each sum trails its exp by four
                merged.append(sums[ai])
                ai += 1
    merged += sums[ai:]
    merged += [f"v_add_f32_e32 {T(9)}, {T(9)}, {T(10)}", f"v_fmac_f32_e32 {T(11)}, {T(9)}, {T(2)}"]
    merged += [f"v_cvt_pk_bf16_f32 {P(i)}, {S(2 * i)}, {S(2 * i + 1)}" for i in range(16)]
    return head + merged


def interleave(mat, smx):
    """the softmax's lines spread evenly after the MFMAs"""
    n_m = sum(1 for k, _ in mat if k == "mfma")
    per = [len(smx) * (i + 1) // n_m - len(smx) * i // n_m for i in range(n_m)]
    out, si, mi = [], 0, 0
    for k, t in mat:
        out.append(t)
        if k == "mfma":
            out += smx[si:si + per[mi]]
            si += per[mi]
            mi += 1
    return out


def scalar_pad(n):
    return [f"s_add_u32 s{80 + i % 4}, s{80 + i % 4}, {i + 1}" for i in range(n)]


def esc(lines):
    return "\\n\\t".join(lines)


def main():
    mat = matrix_block()
    matt = [t for _, t in mat]
    smx = softmax_block()
    nval = sum(1 for ln in smx if ln.startswith("v_"))
    nexp = sum(1 for ln in smx if ln.startswith("v_exp"))
    taken = []
    for i, cut in enumerate((20, 45, 70, 95, 120)):
        prev = (0, 20, 45, 70, 95)[i]
        taken += smx[prev:cut] + [f"s_branch {i + 1}f", "s_nop 0", f"{i + 1}:"]
    taken += smx[120:]
    blocks = {
        "MAT": matt,
        "MATP": ["s_setprio 1"] + matt + ["s_setprio 0"],
        "MATPS": ["s_setprio 1"] + matt + ["s_setprio 0"] + scalar_pad(40),
        "SMX": smx,
        "SMX_NO_EXP": [ln for ln in smx if not ln.startswith("v_exp")],
        "SMX_NO_FMA": [ln for ln in smx if not ln.startswith("v_fma_f32")],
        "SMX_NO_ADD": [ln for ln in smx if not ln.startswith("v_add_f32")],
        "SMX_NO_MAX": [ln for ln in smx if not ln.startswith("v_max")],
        "SMX_NO_CVT": [ln for ln in smx if not ln.startswith("v_cvt_pk")],
        "SMX_SALU": scalar_pad(40) + smx[:40] + scalar_pad(40) + smx[40:],
        "SMX_TAKEN": taken,
        "SEQ": matt + smx,
        "INT": interleave(mat, smx),
    }
    clob = ", ".join(f'"v{i}"' for i in range(SB, 256))
    ops = (': [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3) '
           ': [addr] "v"(addr), [addr2] "v"(addr2), [b0] "v"(b0), [c] "v"(cc) '
           ': "memory", "vcc", "scc", "s80", "s81", "s82", "s83", ' + clob)
    src = [f'''// Generated by gen_phase_probe.py in this folder; edit that, not this.
//
// The two kinds of work of a prefill tile step side by side on one CU (one
// 512-thread workgroup per CU): the matrix phase's instruction stream and a
// softmax-like sequence of {nval} vector instructions ({nexp} v_exp_f32), in the
// arrangements listed in the generator's docstring.  Cycles from s_memtime
// around each wave's loop; a unit is one matrix block plus one softmax block.
// Every LDS access stays inside the workgroup's 97 KiB (96 KiB dynamic plus a
// 1 KiB table), every global access inside a 256 MiB buffer.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDSP __attribute__((address_space(3)))

#define CHECK(x)                                                                 \\
  do {{                                                                           \\
    hipError_t e_ = (x);                                                         \\
    if (e_ != hipSuccess) {{                                                      \\
      std::printf("HIP error %s at line %d\\n", hipGetErrorString(e_), __LINE__); \\
      return 1;                                                                  \\
    }}                                                                            \\
  }} while (0)

namespace {{

constexpr int kLds = 96 * 1024;
constexpr int kNblk = 4096;   // 64 KiB blocks of the copy source: 256 MiB
#define ASM(B) asm volatile(B {ops})
''']
    for k, v in blocks.items():
        src.append(f'#define {k} "{esc(v)}"\n')
    src.append('''
enum Mode {
  MATRIX_ALONE, SOFTMAX_ALONE, SIDE_BY_SIDE, PINGPONG, PINGPONG_COPIES, PINGPONG_COPIES_BT,
  NO_EXP, NO_FMA, NO_ADD, NO_MAX, NO_CVT, SALU_SOFTMAX, SALU_BOTH, TAKEN_BRANCHES,
  ONE_WAVE_IN_TURN, ONE_WAVE_INTERLEAVED, TWO_WAVES_INTERLEAVED
};

// one 4 KiB block (16 rows of 256 bytes, 2 KiB apart) global -> LDS in four copies
__device__ __forceinline__ void copy_block(const char* gbuf, int it, int wave, uint32_t m0, uint32_t vo0,
                                           uint32_t vo1, uint32_t vo2, uint32_t vo3, const LDSP int* bt) {
  int blk;
  if (bt) blk = __builtin_amdgcn_readfirstlane(bt[(it * 4 + (wave & 3)) & 255]);
  else blk = (int)(((uint32_t)it * 2654435761u + blockIdx.x * 40503u + (uint32_t)wave * 977u) % kNblk);
  const uint64_t base = reinterpret_cast<uint64_t>(gbuf) + (uint64_t)blk * 65536 +
                        (uint32_t)__builtin_amdgcn_readfirstlane((wave & 3) * 256);
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xffffu)), 16u * 2048u,
                    0x00020000u};
  asm volatile(
      "s_mov_b32 m0, %0\\n\\ts_nop 0\\n\\tbuffer_load_dwordx4 %1, %5, 0 offen lds\\n\\t"
      "s_add_u32 m0, m0, 0x400\\n\\ts_nop 0\\n\\tbuffer_load_dwordx4 %2, %5, 0 offen lds\\n\\t"
      "s_add_u32 m0, m0, 0x400\\n\\ts_nop 0\\n\\tbuffer_load_dwordx4 %3, %5, 0 offen lds\\n\\t"
      "s_add_u32 m0, m0, 0x400\\n\\ts_nop 0\\n\\tbuffer_load_dwordx4 %4, %5, 0 offen lds"
      :: "s"(m0), "v"(vo0), "v"(vo1), "v"(vo2), "v"(vo3), "s"(rs) : "memory", "scc", "m0");
}

template <int MODE>
__global__ void __launch_bounds__(512) probe(float* out, long long* cyc, int iters, const char* gbuf) {
  extern __shared__ char lds_raw[];
  LDSP char* lds = (LDSP char*)lds_raw;
  __shared__ int bt_s[256];
  for (int i = threadIdx.x; i < kLds / 4; i += 512) ((LDSP uint32_t*)lds)[i] = i * 2654435761u;
  if (threadIdx.x < 256) bt_s[threadIdx.x] = (int)(((uint32_t)threadIdx.x * 2654435761u + blockIdx.x * 40503u) % kNblk);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u32x4 b0 = {(uint32_t)lane, 1u, 2u, 3u};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const float cc = 0.18f;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds + (wave & 3) * 16384 + lane * 16);
  const uint32_t addr2 = (uint32_t)(uintptr_t)(lds + (wave & 3) * 16384 + lane * 8);
  // copies: 4 rows of 256 B per instruction, rows 2 KiB apart, into 80..96 KiB (read by nobody)
  const uint32_t vo0 = (uint32_t)((lane >> 4) * 2048 + (lane & 15) * 16);
  const uint32_t vo1 = vo0 + 4 * 2048, vo2 = vo0 + 8 * 2048, vo3 = vo0 + 12 * 2048;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(uintptr_t)lds + 81920u +
                                                                     (uint32_t)(wave & 3) * 4096u));
  const LDSP int* btp = MODE == PINGPONG_COPIES_BT ? (const LDSP int*)bt_s : nullptr;
  const bool gb = wave >= 4;
  const bool one_group = MODE == MATRIX_ALONE || MODE == SOFTMAX_ALONE || MODE == ONE_WAVE_IN_TURN ||
                         MODE == ONE_WAVE_INTERLEAVED;
  long long t0 = 0, t1 = 0;
  if (!(one_group && gb)) {
    t0 = clock64();
    for (int it = 0; it < iters; ++it) {
      if constexpr (MODE == MATRIX_ALONE) ASM(MAT);
      else if constexpr (MODE == SOFTMAX_ALONE) ASM(SMX);
      else if constexpr (MODE == SIDE_BY_SIDE) { if (gb) ASM(SMX); else ASM(MAT); }
      else if constexpr (MODE == PINGPONG_COPIES || MODE == PINGPONG_COPIES_BT) {
        if (!gb) { ASM(MATP); copy_block(gbuf, it, wave, m0, vo0, vo1, vo2, vo3, btp); }
        else { copy_block(gbuf, it, wave, m0, vo0, vo1, vo2, vo3, btp); ASM(SMX); }
        __builtin_amdgcn_s_barrier();
        if (gb) { ASM(MATP); asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
        else { ASM(SMX); asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
        __builtin_amdgcn_s_barrier();
      } else if constexpr (MODE == ONE_WAVE_IN_TURN) ASM(SEQ);
      else if constexpr (MODE == ONE_WAVE_INTERLEAVED || MODE == TWO_WAVES_INTERLEAVED) ASM(INT);
      else {
        // ping-pong: the matrix block in one group while the other runs its softmax
#define PP_HALF(MAT_BLOCK, SMX_BLOCK)               \\
  {                                                  \\
    if (!gb) ASM(MAT_BLOCK); else ASM(SMX_BLOCK);    \\
    __builtin_amdgcn_s_barrier();                    \\
    if (gb) ASM(MAT_BLOCK); else ASM(SMX_BLOCK);     \\
    __builtin_amdgcn_s_barrier();                    \\
  }
        if constexpr (MODE == PINGPONG) PP_HALF(MATP, SMX)
        else if constexpr (MODE == NO_EXP) PP_HALF(MATP, SMX_NO_EXP)
        else if constexpr (MODE == NO_FMA) PP_HALF(MATP, SMX_NO_FMA)
        else if constexpr (MODE == NO_ADD) PP_HALF(MATP, SMX_NO_ADD)
        else if constexpr (MODE == NO_MAX) PP_HALF(MATP, SMX_NO_MAX)
        else if constexpr (MODE == NO_CVT) PP_HALF(MATP, SMX_NO_CVT)
        else if constexpr (MODE == SALU_SOFTMAX) PP_HALF(MATP, SMX_SALU)
        else if constexpr (MODE == SALU_BOTH) PP_HALF(MATPS, SMX_SALU)
        else if constexpr (MODE == TAKEN_BRANCHES) PP_HALF(MATP, SMX_TAKEN)
#undef PP_HALF
      }
    }
    t1 = clock64();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy in flight when the wave ends
  float res = 0.f;
  for (int r = 0; r < 16; ++r) res += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * 512 + threadIdx.x] = res;
  if (lane == 0) cyc[blockIdx.x * 8 + wave] = t1 - t0;
}

// Does a global -> LDS copy count in LGKM_CNT?  One wave per CU issues one,
// then times s_waitcnt lgkmcnt(0), then (VM = true) also vmcnt(0).
template <bool VM>
__global__ void __launch_bounds__(64) dma_count(const char* g, long long* out) {
  extern __shared__ char dlds[];
  const int lane = threadIdx.x;
  const uint64_t base = reinterpret_cast<uint64_t>(g) + (uint64_t)blockIdx.x * 65536;
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xffffu)), 65536u, 0x00020000u};
  const uint32_t voff = lane * 16;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)dlds);
  long long t0, t1, t2;
  if constexpr (VM) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\\n\\ts_memtime %0\\n\\ts_waitcnt lgkmcnt(0)\\n\\t"
                 "s_mov_b32 m0, %3\\n\\ts_nop 0\\n\\tbuffer_load_dwordx4 %4, %5, 0 offen lds\\n\\t"
                 "s_memtime %1\\n\\ts_waitcnt lgkmcnt(0)\\n\\ts_waitcnt vmcnt(0)\\n\\ts_memtime %2\\n\\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(t0), "=&s"(t1), "=&s"(t2) : "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
  } else {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\\n\\ts_memtime %0\\n\\ts_waitcnt lgkmcnt(0)\\n\\t"
                 "s_mov_b32 m0, %3\\n\\ts_nop 0\\n\\tbuffer_load_dwordx4 %4, %5, 0 offen lds\\n\\t"
                 "s_memtime %1\\n\\ts_waitcnt lgkmcnt(0)\\n\\ts_memtime %2\\n\\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(t0), "=&s"(t1), "=&s"(t2) : "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the copy has landed before the wave ends
  if (lane == 0) out[blockIdx.x] = t2 - t1;
  (void)t0;
}

template <int MODE>
int measure(float* out, long long* cyc, int iters, const char* gbuf, int w0, int w1, double& mean,
            double& slowest, float& ms) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  probe<MODE><<<256, 512, kLds>>>(out, cyc, iters, gbuf);   // warm-up
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(a));
  probe<MODE><<<256, 512, kLds>>>(out, cyc, iters, gbuf);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  CHECK(hipEventElapsedTime(&ms, a, b));
  static long long h[256 * 8];
  CHECK(hipMemcpy(h, cyc, sizeof(h), hipMemcpyDeviceToHost));
  double s = 0, mx = 0;
  int n = 0;
  for (int w = 0; w < 256; ++w)
    for (int v = w0; v < w1; ++v, ++n) {
      s += (double)h[w * 8 + v];
      mx = (double)h[w * 8 + v] > mx ? (double)h[w * 8 + v] : mx;
    }
  mean = s / n / iters;
  slowest = mx / iters;
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return 0;
}

}  // namespace

int main() {
  float* out;
  long long* cyc;
  char* gbuf;
  CHECK(hipMalloc(&out, 256 * 512 * sizeof(float)));
  CHECK(hipMalloc(&cyc, 256 * 8 * sizeof(long long)));
  CHECK(hipMalloc(&gbuf, (size_t)kNblk * 65536));
  CHECK(hipMemset(gbuf, 0, (size_t)kNblk * 65536));
  const int iters = 1000;
  double mean, slowest;
  float ms;
  std::printf("ticks per iteration (s_memtime) of the measured waves: mean, slowest; units per SIMD per "
              "iteration; ticks per unit; kernel time\\n");
#define RUN(MODE, NAME, W0, W1, UNITS)                                                                 \\
  if (measure<MODE>(out, cyc, iters, gbuf, W0, W1, mean, slowest, ms)) return 1;                       \\
  std::printf("  %-44s %8.1f %8.1f   %d  %8.1f   %8.1f us\\n", NAME, mean, slowest, UNITS, mean / UNITS, \\
              ms * 1e3f);
  RUN(MATRIX_ALONE, "matrix alone (1 wave/SIMD)", 0, 4, 1)
  RUN(SOFTMAX_ALONE, "softmax alone (1 wave/SIMD)", 0, 4, 1)
  RUN(SIDE_BY_SIDE, "side by side: the matrix waves", 0, 4, 1)
  RUN(SIDE_BY_SIDE, "side by side: the softmax waves", 4, 8, 1)
  RUN(PINGPONG, "ping-pong", 0, 8, 2)
  RUN(PINGPONG_COPIES, "ping-pong + copies", 0, 8, 2)
  RUN(PINGPONG_COPIES_BT, "ping-pong + copies, block id from LDS", 0, 8, 2)
  RUN(NO_EXP, "ping-pong, softmax without exp", 0, 8, 2)
  RUN(NO_FMA, "ping-pong, softmax without fma", 0, 8, 2)
  RUN(NO_ADD, "ping-pong, softmax without adds", 0, 8, 2)
  RUN(NO_MAX, "ping-pong, softmax without max", 0, 8, 2)
  RUN(NO_CVT, "ping-pong, softmax without cvt", 0, 8, 2)
  RUN(SALU_SOFTMAX, "ping-pong + 80 scalar in the softmax", 0, 8, 2)
  RUN(SALU_BOTH, "ping-pong + 80 scalar softmax, 40 matrix", 0, 8, 2)
  RUN(TAKEN_BRANCHES, "ping-pong + 5 taken branches in the softmax", 0, 8, 2)
  RUN(ONE_WAVE_IN_TURN, "1 wave/SIMD, blocks in turn", 0, 4, 1)
  RUN(ONE_WAVE_INTERLEAVED, "1 wave/SIMD, interleaved", 0, 4, 1)
  RUN(TWO_WAVES_INTERLEAVED, "2 waves/SIMD, interleaved", 0, 8, 2)
#undef RUN
  static long long h[256];
  long long* d;
  CHECK(hipMalloc(&d, 256 * sizeof(long long)));
  for (int vm = 0; vm < 2; ++vm) {
    if (vm) dma_count<true><<<256, 64, 4096>>>(gbuf, d);
    else dma_count<false><<<256, 64, 4096>>>(gbuf, d);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost));
    double s = 0;
    for (int i = 0; i < 256; ++i) s += (double)h[i];
    std::printf("global -> LDS copy, then %s: %.0f ticks (mean over 256 waves)\\n",
                vm ? "lgkmcnt(0) and vmcnt(0)" : "lgkmcnt(0) only    ", s / 256);
  }
  CHECK(hipFree(d));
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  CHECK(hipFree(gbuf));
  return 0;
}
''')
    with open(os.path.join(HERE, "phase_probe.hip"), "w") as f:
        f.write("".join(src))


if __name__ == "__main__":
    main()
