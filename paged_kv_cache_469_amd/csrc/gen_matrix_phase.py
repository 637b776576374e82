"""Writes matrix_phase.inc: the instruction schedule of the prefill kernel's
matrix phase at head size 128, as inline-asm strings.

A matrix phase is QK (S^T of one 64-key tile: two 32-key halves x 8 d slabs,
16 MFMAs, the A operand read from the K slot with ds_read_b128) and PV
(O^T += V^T P^T: 4 d tiles x 2 halves x 2 16-key slabs, 16 MFMAs, the A
operand read from the V slot with two ds_read_b64_tr_b16).  The schedule
keeps the operand reads LEAD groups ahead of their MFMA in a ring of RING
four-register slots (fixed registers RING_BASE..), and every wait counts
only the reads issued after the one it needs, so QK and PV run as one
stream with no drain between them.

Two scalar branches inside the stream skip the half of it that a step does
not need: QK when %[qrem] (tiles left after this one) is zero, the last
step, whose scores would go unused; PV when %[tt] (the step) is zero, the
first step, which has no P yet.  The path without QK issues the first LEAD
PV reads itself, in the order and into the slots the QK path issues them,
so both paths reach the PV body with the same reads in flight; every path
ends by waiting for all reads, so none lands in a ring register after the
block.  The branches are wave-uniform and invisible to the compiler, so
the accumulators stay in one set of registers on every path.

Operands of the asm statement that uses these strings (prefill.hip):
  %[s0] %[s1]      S^T halves (f32x16, written)
  %[o0] .. %[o3]   O^T d tiles (f32x16, read-write)
  %[q0] .. %[q7]   query slabs (B of QK)
  %[p0] .. %[p3]   P of the previous tile, pr[kt][u] at 2 kt + u (B of PV)
  %[k0] .. %[k7]   lane offsets of the K operand of slab i (bytes)
  %[v0] .. %[v3]   lane offsets of the V operand of d tile i (bytes)
  %[kb] %[vb]      LDS byte address of the K and V slot (immediates)
  %[qrem] %[tt]    tiles left after this step, and the step (scalars)

Run from this folder: python gen_matrix_phase.py (the generated file is
committed; the build does not run this).
"""

import os

HERE = os.path.dirname(os.path.abspath(__file__))
D = 128
ROWB = 2 * D          # bytes of one key row
NSL = D // 16         # d slabs of QK
NDT = D // 32         # d tiles of PV
RING = 4
RING_BASE = 240       # v240 .. v255
LEAD = 3
# wait states after the block: the last MFMA's result is read by vector
# instructions only after these (an XDL write followed by a VALU read of
# the same register needs the MFMA's passes plus a few)
TAIL_NOPS = ["s_nop 7", "s_nop 3"]


def slot(g):
    b = RING_BASE + 4 * (g % RING)
    return b


def qk_groups():
    out = []
    for g in range(2 * NSL):
        kt, sl = g & 1, g >> 1            # the two halves' chains alternate
        def reads(r, sl=sl, kt=kt):
            return [f"ds_read_b128 v[{r}:{r + 3}], %[k{sl}] offset:%[kb]+{kt * 32 * ROWB}"]
        def mfma(r, sl=sl, kt=kt):
            c = "0" if sl == 0 else f"%[s{kt}]"
            return f"v_mfma_f32_32x32x16_bf16 %[s{kt}], v[{r}:{r + 3}], %[q{sl}], {c}"
        out.append((1, reads, mfma))
    return out


def pv_groups():
    out = []
    for kt in range(2):
        for u in range(2):
            for dt in range(NDT):
                base = (32 * kt + 16 * u) * ROWB
                def reads(r, dt=dt, base=base):
                    return [f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[v{dt}] offset:%[vb]+{base}",
                            f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[v{dt}] offset:%[vb]+{base + 8 * ROWB}"]
                def mfma(r, dt=dt, kt=kt, u=u):
                    return f"v_mfma_f32_32x32x16_bf16 %[o{dt}], v[{r}:{r + 3}], %[p{2 * kt + u}], %[o{dt}]"
                out.append((2, reads, mfma))
    return out


def run(groups, first, last, issued):
    """MFMAs first .. last - 1, each after the wait for its own reads and
    followed by the reads LEAD groups ahead; issued = groups whose reads are
    already out.  Returns (lines, issued)."""
    lines = []
    for g in range(first, last):
        after = sum(groups[j][0] for j in range(g + 1, issued))
        lines.append(f"s_waitcnt lgkmcnt({after})")
        lines.append(groups[g][2](slot(g)))
        if issued < len(groups):
            lines += groups[issued][1](slot(issued))
            issued += 1
    return lines, issued


def schedule(qk, pv):
    groups = qk + pv
    nq, n = len(qk), len(qk) + len(pv)
    lines = ["s_cmp_eq_u32 %[qrem], 0", "s_cbranch_scc1 2f"]   # no QK: to 2
    for g in range(LEAD):
        lines += groups[g][1](slot(g))
    body, issued = run(groups, 0, nq, LEAD)
    lines += body
    lines += ["s_cmp_eq_u32 %[tt], 0", "s_cbranch_scc1 4f",     # no PV: to the end
              "s_branch 3f",
              "2:",
              "s_cmp_eq_u32 %[tt], 0", "s_cbranch_scc1 4f"]
    # the PV reads the QK path issued during its last MFMAs
    for g in range(nq, issued):
        lines += groups[g][1](slot(g))
    lines.append("3:")
    body, issued = run(groups, nq, n, issued)
    lines += body
    # nothing in flight past the block (a path without PV leaves reads out)
    return lines + ["4:", "s_waitcnt lgkmcnt(0)"] + TAIL_NOPS


def cstr(lines):
    return '"' + "\\n\\t".join(lines) + '"'


def text():
    """The contents of matrix_phase.inc."""
    # an outstanding scalar load would make the counted waits unsound: the
    # block starts by draining the LGKM counter (nothing is in flight there
    # in the kernel, so this costs nothing)
    head = ["s_waitcnt lgkmcnt(0)"]
    return "".join([
        "// Generated by gen_matrix_phase.py in this folder; edit that, not this.\n",
        f"// Matrix phase of the prefill kernel at head size {D}: operand reads {LEAD} groups\n",
        f"// ahead in a ring of {RING} slots (v{RING_BASE}..v{RING_BASE + 4 * RING - 1}).\n",
        f"#define PKV_MAT_RING_FIRST {RING_BASE}\n",
        f"#define PKV_MAT_QKPV {cstr(head + schedule(qk_groups(), pv_groups()))}\n",
    ])


def main():
    with open(os.path.join(HERE, "matrix_phase.inc"), "w") as f:
        f.write(text())


if __name__ == "__main__":
    main()
