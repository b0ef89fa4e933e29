"""Writes own_asm.inc: the instruction sequences of the 128-row attention
kernel's inner loop (attn_own_kernel in attn.hip), as inline-asm templates.

The loop body is emitted instruction by instruction so that the schedule is
exactly the one intended: LDS operand reads issued several MFMAs ahead of
their use with exact lgkmcnt waits, the softmax VALU work interleaved with the
score MFMAs, and no register traffic between the accumulators and VGPRs.
Register allocation stays with the compiler through named operands; only a
few short-lived temporaries are fixed registers (declared as clobbers).

Templates:
  OWN_ASM_PRO  scores of the first half tile of a segment (36 k-steps)
  OWN_ASM_A    first half of the softmax of half tile e (mask, row max,
               rescale factor) interleaved with the score MFMAs of half
               tile e+1, k-steps 0..17, and the nine
               buffer -> LDS copies of this wave's share of half tile e+3;
               leaves the K fragments of k-steps 18..21 loaded
  OWN_ASM_A_FULL  the same for a half tile whose keys every row sees (no mask)
  OWN_ASM_B    score MFMAs of half tile e+1, k-steps 18..35, carrying the
               second half of the softmax (probabilities, row sum, bf16
               packing), then the 32 PV MFMAs of half tile e (V^T fragments
               read transposed, prefetched under the last score MFMAs)
  OWN_ASM_B_FIRST  the same for the first half tile of a segment: the PV
               accumulators start from zero inside the MFMAs

Operand names and layouts are those of attn_own_kernel; the MFMA is
v_mfma_f32_32x32x16_bf16 throughout. Run: python gen_own_asm.py (the build
runs it before compiling).
"""

import os

KSTEPS = 36          # 576 features / 16
A_STEPS = 18         # score k-steps in template A
PF_K = int(os.environ.get("OWN_PF_K", "4"))   # K fragments in flight
PF_V = int(os.environ.get("OWN_PF_V", "4"))   # V^T fragments in flight (two reads each)
assert PF_K + 2 * PF_V <= 15, "LDS reads in flight must fit lgkmcnt"
NEG_INF = "0xff800000"
HERE = os.path.dirname(os.path.abspath(__file__))

# fixed temporaries (clobbered): A uses TA; B uses the V ring, the packed
# probabilities P (two MFMA operands of 4 registers) and one accumulator
TA = ["v%d" % r for r in range(252, 256)]
VR0 = 256 - 4 * PF_V
VRING = [("v[%d:%d]" % (VR0 + 4 * i, VR0 + 4 * i + 1), "v[%d:%d]" % (VR0 + 4 * i + 2, VR0 + 4 * i + 3),
          "v[%d:%d]" % (VR0 + 4 * i, VR0 + 4 * i + 3)) for i in range(PF_V)]
PR0 = VR0 - 8
P_OP = ["v[%d:%d]" % (PR0, PR0 + 3), "v[%d:%d]" % (PR0 + 4, PR0 + 7)]
TB = "v%d" % (PR0 - 1)
B_CLOB0 = PR0 - 1
GUARD = ["s_nop 7", "s_nop 7", "s_nop 7"]   # MFMA results settle before the compiler's code reads them


class Seq:
    """Instruction list with a model of the in-order LDS counter (lgkmcnt)."""

    def __init__(self):
        self.lines = []
        self.pending = []          # tags of LDS reads not yet waited for, in issue order

    def op(self, s):
        self.lines.append(s)

    def lds(self, s, tag):
        assert len(self.pending) < 15, "too many LDS reads in flight for lgkmcnt"
        self.lines.append(s)
        self.pending.append(tag)

    def need(self, tag):
        if tag not in self.pending:
            return
        i = max(k for k, t in enumerate(self.pending) if t == tag)
        self.lines.append("s_waitcnt lgkmcnt(%d)" % (len(self.pending) - i - 1))
        self.pending = self.pending[i + 1:]

    def drain(self):
        if self.pending:
            self.lines.append("s_waitcnt lgkmcnt(0)")
            self.pending = []

    def text(self):
        return "".join(l + "\\n\\t" for l in self.lines)


def kread(seq, ks):
    """K fragment of k-step ks into ring slot ks % PF_K (16 bytes per lane)."""
    seq.lds("ds_read_b128 %%[kb%d], %%[ka%d] offset:%d" % (ks % PF_K, ks & 3, (ks >> 2) * 1024), "K%d" % ks)


def score_mfma(seq, ks, first):
    seq.need("K%d" % ks)
    seq.op("v_mfma_f32_32x32x16_bf16 %%[sn], %%[kb%d], %%[q%d], %s" % (ks % PF_K, ks, "0" if first else "%[sn]"))


def vread(seq, j):
    """V^T fragment of PV step j (column block j / 2, token block j % 2): two
    transposing reads into the two halves of ring slot j % PF_V."""
    cb, kk = j >> 1, j & 1
    lo, hi, _ = VRING[j % PF_V]
    seq.lds("ds_read_b64_tr_b16 %s, %%[va%d] offset:%d" % (lo, cb & 1, kk * 18432 + (cb >> 1) * 1024), "V%da" % j)
    seq.lds("ds_read_b64_tr_b16 %s, %%[va%d] offset:%d" % (hi, 2 + (cb & 1), kk * 18432 + 9216 + (cb >> 1) * 1024),
            "V%db" % j)


def gen_pro():
    s = Seq()
    s.op("s_nop 1")
    for ks in range(PF_K):
        kread(s, ks)
    for ks in range(KSTEPS):
        score_mfma(s, ks, ks == 0)
        if ks + PF_K < KSTEPS:
            kread(s, ks + PF_K)
    s.lines += GUARD
    return s.text()


def softmax_max(mask=True):
    """First half of the online softmax of one half tile for the lane's row,
    on operands s0..s15 (score value i = token 8 (i / 4) + 4 h + i % 4 of the
    half tile; lr = last visible key minus the token of value 0): key mask,
    row max, the rescale factor alpha of the running state, the new running
    max and the reference mref the probabilities are taken against."""
    t0, t1, t2, ninf = TA
    v = []
    if mask:
        # v_cndmask reads VCC over the constant bus, so -inf comes from a register
        v.append("v_mov_b32 %s, %s" % (ninf, NEG_INF))
        for i in range(16):   # keys past the row's position -> -inf
            off = 8 * (i >> 2) + (i & 3)
            v.append("v_cmp_le_i32 vcc, %d, %%[lr]" % off)
            v.append("v_cndmask_b32 %%[s%d], %s, %%[s%d], vcc" % (i, ninf, i))
    v.append("v_max3_f32 %s, %%[s0], %%[s1], %%[s2]" % t0)
    for i in range(3, 15, 2):
        v.append("v_max3_f32 %s, %s, %%[s%d], %%[s%d]" % (t0, t0, i, i + 1))
    v.append("v_max_f32 %s, %s, %%[s15]" % (t0, t0))
    v.append("v_mov_b32 %s, %s" % (t1, t0))
    v.append("s_nop 1")
    v.append("v_permlane32_swap_b32 %s, %s" % (t0, t1))      # halves of the wave swapped
    v.append("v_max_f32 %s, %s, %s" % (t0, t0, t1))            # row max over both halves
    v.append("v_mul_f32 %s, %s, %%[scale]" % (t0, t0))        # in log2 units
    v.append("v_add_f32 %s, 0x41000000, %%[mrun]" % t1)       # running max + 8
    v.append("v_cmp_gt_f32 vcc, %s, %s" % (t0, t1))
    v.append("v_cndmask_b32 %s, %%[mrun], %s, vcc" % (t2, t0))  # new max
    v.append("v_sub_f32 %s, %%[mrun], %s" % (t1, t2))
    v.append("v_exp_f32 %s, %s" % (t1, t1))
    v.append("v_cmp_neq_f32 vcc, %s, %%[mrun]" % t2)
    v.append("v_cndmask_b32 %%[alpha], 1.0, %s, vcc" % t1)     # 1 unless the max moved
    v.append("v_mov_b32 %%[mrun], %s" % t2)
    v.append("v_cmp_neq_f32 vcc, %s, %s" % (NEG_INF, t2))
    v.append("v_cndmask_b32 %%[mref], 0, %s, vcc" % t2)        # reference: 0 while nothing is visible
    return v


def softmax_exp():
    """Second half: probabilities 2^(s scale - mref), their sum into the
    running l (after alpha), and the bf16 packing into P for the PV MFMAs."""
    v = []
    for i in range(16):
        v.append("v_fma_f32 %%[s%d], %%[s%d], %%[scale], -%%[mref]" % (i, i))
        v.append("v_exp_f32 %%[s%d], %%[s%d]" % (i, i))
    v.append("v_add_f32 %s, %%[s0], %%[s1]" % TB)
    for i in range(2, 16):
        v.append("v_add_f32 %s, %s, %%[s%d]" % (TB, TB, i))
    for j in range(8):
        v.append("v_cvt_pk_bf16_f32 v%d, %%[s%d], %%[s%d]" % (PR0 + j, 2 * j, 2 * j + 1))
    v.append("v_fma_f32 %%[lrun], %%[lrun], %%[alpha], %s" % TB)
    return v


# The nine copies of the wave's share of the next stage, spread over the
# whole iteration (the vector memory unit takes the four waves' copies one
# at a time; bunched together they stall the issuing waves): lines 0..3
# after these score MFMAs of A, lines 4..8 after these PV MFMAs of B.
DMA_A = [1, 5, 9, 13]
DMA_B = [2, 8, 14, 20, 26]


def dma(seq, cg):
    """Line cg of this wave's share of the next stage: buffer -> LDS copy of
    1 KiB (M0 = LDS base of the line; the copy counts in vmcnt, not lgkmcnt)."""
    seq.op("s_add_u32 m0, %%[mb], 0x%x" % (cg * 1024))
    seq.op("s_nop 0")
    seq.op("buffer_load_dwordx4 %%[go], %%[rs], %%[so%d] offen lds" % cg)


def gen_a(mask=True):
    s = Seq()
    s.op("s_nop 1")
    for ks in range(PF_K):
        kread(s, ks)
    valu = softmax_max(mask)
    per = (len(valu) + A_STEPS - 1) // A_STEPS
    for ks in range(A_STEPS):
        score_mfma(s, ks, ks == 0)
        kread(s, ks + PF_K)               # the last PF_K of these are template B's first k-steps
        if ks in DMA_A:
            dma(s, DMA_A.index(ks))
        for ins in valu[ks * per:(ks + 1) * per]:
            s.op(ins)
    s.drain()
    s.lines += GUARD
    return s.text()


B_VALU_STEPS = 13      # score MFMAs of B that carry the exp half of the softmax


def gen_b(first=False):
    s = Seq()
    s.op("s_nop 1")
    valu = softmax_exp()
    per = (len(valu) + B_VALU_STEPS - 1) // B_VALU_STEPS
    vnext = 0
    for j in range(KSTEPS - A_STEPS):
        ks = A_STEPS + j
        score_mfma(s, ks, False)
        if ks + PF_K < KSTEPS:
            kread(s, ks + PF_K)
        elif vnext < PF_V:                 # K reads done: start the V^T ring
            vread(s, vnext)
            vnext += 1
        for ins in valu[j * per:(j + 1) * per]:
            s.op(ins)
    while vnext < PF_V:
        vread(s, vnext)
        vnext += 1
    for j in range(32):
        s.need("V%db" % j)
        acc = "0" if first and j % 2 == 0 else "%%[o%d]" % (j >> 1)   # first half tile: start from 0
        s.op("v_mfma_f32_32x32x16_bf16 %%[o%d], %s, %s, %s" % (j >> 1, VRING[j % PF_V][2], P_OP[j & 1], acc))
        if j + PF_V < 32:
            vread(s, j + PF_V)
        if j in DMA_B:
            dma(s, len(DMA_A) + DMA_B.index(j))
    s.drain()
    s.lines += GUARD
    return s.text()


def main():
    out = os.path.join(HERE, "own_asm.inc")
    body = ["// Generated by gen_own_asm.py; do not edit.", ""]
    for name, text in (("OWN_ASM_PRO", gen_pro()), ("OWN_ASM_A", gen_a()), ("OWN_ASM_A_FULL", gen_a(False)),
                       ("OWN_ASM_B", gen_b()), ("OWN_ASM_B_FIRST", gen_b(True))):
        body.append('#define %s "%s"' % (name, text))
        body.append("")
    # operand lists (names of attn_own_kernel's variables)
    ops = {
        "OWN_OPS_Q0_17": ", ".join('[q%d] "v"(qf[%d])' % (i, i) for i in range(A_STEPS)),
        "OWN_OPS_Q18_35": ", ".join('[q%d] "v"(qf[%d])' % (i, i) for i in range(A_STEPS, KSTEPS)),
        "OWN_OPS_Q0_35": ", ".join('[q%d] "v"(qf[%d])' % (i, i) for i in range(KSTEPS)),
        "OWN_OPS_KA": ", ".join('[ka%d] "v"(ka[%d])' % (i, i) for i in range(4)),
        "OWN_OPS_VA": ", ".join('[va%d] "v"(va[%d])' % (i, i) for i in range(4)),
        "OWN_OPS_KB_OUT": ", ".join('[kb%d] "=&v"(kb[%d])' % (i, i) for i in range(PF_K)),
        "OWN_OPS_KB_INOUT": ", ".join('[kb%d] "+v"(kb[%d])' % (i, i) for i in range(PF_K)),
        "OWN_OPS_S": ", ".join('[s%d] "+v"(s[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_O": ", ".join('[o%d] "+a"(o[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_O_OUT": ", ".join('[o%d] "=&a"(o[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_SO_A": ", ".join('[so%d] "s"(so[%d])' % (i, i) for i in range(len(DMA_A))),
        "OWN_OPS_SO_B": ", ".join('[so%d] "s"(so[%d])' % (i, i) for i in range(len(DMA_A), 9)),
        "OWN_CLOB_A": ", ".join('"%s"' % r for r in TA),
        "OWN_CLOB_B": ", ".join('"v%d"' % r for r in range(B_CLOB0, 256)),
        "OWN_PF_K": str(PF_K),
    }
    for name, text in ops.items():
        body.append("#define %s %s" % (name, text))
    body.append("")
    new = "\n".join(body)
    if not os.path.exists(out) or open(out).read() != new:
        with open(out, "w") as f:
            f.write(new)
    return out


if __name__ == "__main__":
    print(main())
