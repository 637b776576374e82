"""The prefill kernel's matrix phase at head size 128 is a generated inline-asm
stream (paged_kv_cache_469_amd/csrc/gen_matrix_phase.py ->
matrix_phase.inc).  These CPU tests check that the committed file is what
the generator writes, and replay the stream symbolically: every MFMA reads
an operand slot that the read for its own group filled and that has landed
by the LDS counter's rule (a wait for N lets the newest N reads stay in
flight), no read overwrites a slot before the MFMA that uses its previous
contents has issued, and the products are exactly the QK and PV terms of one
tile (each accumulator chain complete, S chains started from zero)."""

import importlib.util
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_469_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_matrix_phase",
                                                  os.path.join(CSRC, "gen_matrix_phase.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stream():
    text = open(os.path.join(CSRC, "matrix_phase.inc")).read()
    m = re.search(r'#define PKV_MAT_QKPV "(.*)"\n', text)
    assert m
    return m.group(1).split("\\n\\t")


def test_committed_file_is_the_generators_output():
    assert open(os.path.join(CSRC, "matrix_phase.inc")).read() == _gen().text()


def _regs(tok):
    """v[a:b] -> set of register numbers"""
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    assert m, tok
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _replay(lines, g, no_qk, no_pv):
    """Follows the stream with %[qrem] == 0 iff no_qk and %[tt] == 0 iff no_pv;
    returns the QK and PV terms of the MFMAs it issues."""
    labels = {ln[:-1]: i for i, ln in enumerate(lines) if re.fullmatch(r"\d+:", ln)}
    zero = {"%[qrem]": no_qk, "%[tt]": no_pv}
    inflight = []      # reads issued and not known to have landed: (regs, what it loads)
    holds = {}         # register -> what the last landed-or-pending read put there
    pending = set()    # registers with a read in flight
    consumed = set()   # registers whose contents an issued MFMA has read
    qk_terms, pv_terms = [], []
    s_started = {}
    scc = None
    pc, steps = 0, 0
    while pc < len(lines):
        steps += 1
        assert steps < 10 * len(lines), "the branches loop"
        ln = lines[pc]
        pc += 1
        op = ln.split()[0]
        if op == "s_cmp_eq_u32":
            reg, imm = [t.rstrip(",") for t in ln.split()[1:3]]
            assert imm == "0" and reg in zero, ln
            scc = zero[reg]
        elif op in ("s_cbranch_scc1", "s_branch"):
            target = ln.split()[1]
            assert target.endswith("f") and target[:-1] in labels, ln
            assert labels[target[:-1]] > pc - 1, "branches only go forward"
            if op == "s_branch" or scc:
                pc = labels[target[:-1]] + 1
            scc = None if op == "s_cbranch_scc1" else scc
        elif re.fullmatch(r"\d+:", op):
            pass
        elif op == "s_waitcnt":
            n = int(re.search(r"lgkmcnt\((\d+)\)", ln).group(1))
            while len(inflight) > n:
                regs, _ = inflight.pop(0)
                pending -= regs
        elif op.startswith("ds_read"):
            dst = ln.split()[1].rstrip(",")
            regs = _regs(dst)
            # the slot's previous contents were used by an MFMA already issued
            for r in regs:
                if r in holds:
                    assert r in consumed, f"a read overwrites v{r} before its MFMA issued"
            addr = re.search(r"%\[(\w+)\] offset:%\[(\w+)\]\+(\d+)", ln)
            what = (op, addr.group(1), addr.group(2), int(addr.group(3)))
            inflight.append((regs, what))
            for r in regs:
                holds[r] = what
                pending.add(r)
                consumed.discard(r)
        elif op == "v_mfma_f32_32x32x16_bf16":
            dst, a, b, c = [t.rstrip(",") for t in ln.split()[1:5]]
            regs = _regs(a)
            assert not (regs & pending), f"MFMA reads {a} before its read landed: {ln}"
            loads = {holds[r] for r in regs}
            consumed |= regs
            if dst in ("%[s0]", "%[s1]"):
                # one ds_read_b128 of K slab i, half kt, for B = query slab i
                assert len(loads) == 1
                (rop, lane_off, base, off), = loads
                assert rop == "ds_read_b128" and base == "kb"
                kt = int(dst[3])
                assert off == kt * 32 * g.ROWB
                sl = int(lane_off[1:])
                assert lane_off == f"k{sl}" and b == f"%[q{sl}]"
                if dst not in s_started:
                    assert c == "0", "an S chain starts from zero"
                    s_started[dst] = True
                else:
                    assert c == dst
                qk_terms.append((kt, sl))
            else:
                # two transposing reads of one 16-key slab of d tile dt
                assert c == dst and len(loads) == 2
                dt = int(dst[3])
                kinds = sorted(loads, key=lambda w: w[3])
                assert all(w[0] == "ds_read_b64_tr_b16" and w[1] == f"v{dt}" and w[2] == "vb" for w in kinds)
                base = kinds[0][3]
                assert kinds[1][3] == base + 8 * g.ROWB
                kt, rem = divmod(base // g.ROWB, 32)
                u = rem // 16
                assert rem % 16 == 0 and b == f"%[p{2 * kt + u}]"
                pv_terms.append((dt, kt, u))
        else:
            assert op == "s_nop", ln
    assert not inflight, "every read is waited for inside the block"
    return qk_terms, pv_terms


def test_stream_replays_correctly():
    g = _gen()
    lines = _stream()
    assert lines[0] == "s_waitcnt lgkmcnt(0)"
    all_qk = [(kt, sl) for kt in range(2) for sl in range(g.NSL)]
    all_pv = [(dt, kt, u) for dt in range(g.NDT) for kt in range(2) for u in range(2)]
    for no_qk in (False, True):
        for no_pv in (False, True):
            qk_terms, pv_terms = _replay(lines, g, no_qk, no_pv)
            assert sorted(qk_terms) == ([] if no_qk else all_qk), (no_qk, no_pv)
            assert sorted(pv_terms) == ([] if no_pv else all_pv), (no_qk, no_pv)


def test_offsets_fit_the_instruction_field():
    """ds_read offsets are 16 bits: the largest slot place plus term fits."""
    g = _gen()
    tilebytes = 64 * g.ROWB
    most = 0
    for ln in _stream():
        m = re.search(r"offset:%\[(kb|vb)\]\+(\d+)", ln)
        if m:
            base = 2 * tilebytes if m.group(1) == "kb" else 1 * tilebytes   # K slots 0-2, V slots 0-1
            most = max(most, base + int(m.group(2)))
    assert 0 < most < 65536


def test_stream_ends_with_the_wait_states():
    lines = _stream()
    nops = [ln for ln in lines if ln.startswith("s_nop")]
    assert lines[-len(nops):] == nops
    assert sum(int(ln.split()[1]) + 1 for ln in nops) >= 11
