#!/usr/bin/env python3
"""Writes mfma_steps.inc: the hand-scheduled inline-asm blocks of the bf16
grouped GEMM (ffn_bf16.hip), one set per wave tile of (32*TM tokens) x
(32*TN features).

Each block is an unrolled list of v_mfma_f32_32x32x16_bf16 with the other
instructions of the step spread between the MFMAs (see the kernel's notes on
the matrix-core issue shadow). A stage's LDS-DMA loads go out in two halves,
with the last K16 step of one stage and the first of the next, so that the
load queue is never handed a whole stage at once. The blocks are generated
rather than typed because every operand index depends on the tile shape.

  python3 gen_mfma_steps.py        (rewrites mfma_steps.inc next to this file)
"""
import os

SHAPES = [(4, 4), (3, 4), (2, 4), (1, 4)]  # (TM, TN): 256, 192, 128 and 64 x 256 block tiles


def q(s):
    return '      "' + s + '\\n\\t"'


def acc_list(TM, TN):
    return ", ".join(f'"+a"(acc[{i}][{j}])' for i in range(TN) for j in range(TM))


def cur_list(TM, TN):
    return ", ".join([f'"v"(w[{i}])' for i in range(TN)] + [f'"v"(t[{j}])' for j in range(TM)])


def next_list(TM, TN):
    return ", ".join([f'"=&v"(nt[{j}])' for j in range(TM)] + [f'"=&v"(nw[{i}])' for i in range(TN)])


def next_list_t(TM, TN):
    return ", ".join([f'"=&v"(nt[{j}])' for j in range(TM)] + [f'"=&v"(nlo[{i}])' for i in range(TN)] +
                     [f'"=&v"(nhi[{i}])' for i in range(TN)])


def wa_list(TN):
    return ", ".join(f'"v"(wa[{i}])' for i in range(TN))


def mfmas(TM, TN, w0, t0):
    return [f"v_mfma_f32_32x32x16_bf16 %{TM*i+j}, %{w0+i}, %{t0+j}, %{TM*i+j}"
            for i in range(TN) for j in range(TM)]


def step_body(TM, TN, dma, half=None, wt=False):
    """wt: the weight stage is stored K-major (64 rows of 256 features); each
    weight fragment comes from two transposing reads (k 0..3 and 4..7 of the
    lane's 8, 4 rows = 2048 bytes apart) into a low and a high 64-bit half,
    from one address operand per fragment tile."""
    nacc = TM * TN
    nt0 = nacc
    nw0 = nt0 + TM
    w0 = nw0 + (2 * TN if wt else TN)
    t0 = w0 + TN
    ta = t0 + TM
    wa = ta + 1
    LA, LB = 2 * TM, 2 * TN
    vo0 = wa + (TN if wt else 1)
    la = vo0 + LA + LB
    lb, ga, gw = la + 1, la + 2, la + 3
    reads = [f"ds_read_b128 %{nt0+j}, %{ta} offset:{4096*j}" for j in range(TM)]
    if wt:
        reads += [f"ds_read_b64_tr_b16 %{nw0+i+TN*h}, %{wa+i} offset:{2048*h}"
                  for i in range(TN) for h in range(2)]
    else:
        reads += [f"ds_read_b128 %{nw0+i}, %{wa} offset:{4096*i}" for i in range(TN)]
    mf = mfmas(TM, TN, w0, t0)
    loads = []
    if dma:
        loads = ([(f"s_add_u32 m0, %{la}, 0x{b*0x400:x}", f"global_load_lds_dwordx4 %{vo0+b}, %{ga}")
                  for b in range(LA)] +
                 [(f"s_add_u32 m0, %{lb}, 0x{b*0x400:x}", f"global_load_lds_dwordx4 %{vo0+LA+b}, %{gw}")
                  for b in range(LB)])
    if half is not None:
        n1 = (len(loads) + 1) // 2
        loads = loads[:n1] if half == 0 else loads[n1:]
    # loads evenly over the step's MFMAs
    per = [0] * len(mf)
    for k in range(len(loads)):
        per[(k * len(mf)) // len(loads)] += 1
    out, di, ri = [], 0, 0
    for m in range(len(mf)):
        pend = loads[di:di + per[m]]
        di += per[m]
        if pend:
            out.append(pend[0][0])  # M0 write; the MFMA gives the wait state
        out.append(mf[m])
        for k, (m0, ld) in enumerate(pend):
            if k > 0:
                out += [m0, "s_nop 0"]
            out.append(ld)
        if ri < len(reads):
            out.append(reads[ri])
            ri += 1
    out += reads[ri:]
    return "\n".join(q(s) for s in out) + '\n      "s_waitcnt lgkmcnt(0)"'


def dma_half(TM, TN, half, wt=False):
    LA, LB = 2 * TM, 2 * TN
    n = f"{TM}x{TN}"
    vo = ", ".join(f'"v"(vo[{b}])' for b in range(LA + LB))
    sig_cur = f"const bf16x8_t (&w)[{TN}], const bf16x8_t (&t)[{TM}]"
    if wt:
        name = f"step_dma{half}_t_{n}"
        sig_next = f"bf16x8_t (&nt)[{TM}], v4i16 (&nlo)[{TN}], v4i16 (&nhi)[{TN}]"
        addr_sig = f"uint32_t ta, const uint32_t (&wa)[{TN}]"
        addr = f'"v"(ta), {wa_list(TN)}'
        nxt = next_list_t(TM, TN)
    else:
        name = f"step_dma{half}_{n}"
        sig_next = f"bf16x8_t (&nw)[{TN}], bf16x8_t (&nt)[{TM}]"
        addr_sig = "uint32_t ta, uint32_t wa"
        addr = '"v"(ta), "v"(wa)'
        nxt = next_list(TM, TN)
    which = "first" if half == 0 else "second"
    return f'''// a K16 step that also issues the {which} half of a stage's LDS-DMA loads
__device__ __forceinline__ void {name}(f32x16_t (&acc)[{TN}][{TM}], {sig_cur},
    {sig_next}, {addr_sig}, const uint32_t (&vo)[{LA+LB}], uint32_t la, uint32_t lb,
    const char* ga, const char* gw) {{
  asm volatile(
{step_body(TM, TN, True, half, wt)}
      : {acc_list(TM, TN)},
        {nxt}
      : {cur_list(TM, TN)}, {addr},
        {vo},
        "s"(la), "s"(lb), "s"(ga), "s"(gw)
      : "memory", "m0", "scc");
}}'''


def emit(TM, TN):
    LA, LB = 2 * TM, 2 * TN
    n = f"{TM}x{TN}"
    vo = ", ".join(f'"v"(vo[{b}])' for b in range(LA + LB))
    w0 = TM * TN
    t0 = w0 + TN
    last = "\n".join(q(s) for s in ["s_nop 1"] + mfmas(TM, TN, w0, t0) + ["s_nop 7", "s_nop 7"])
    frag = ([f"ds_read_b128 %{j}, %{TM+TN} offset:{4096*j}" for j in range(TM)] +
            [f"ds_read_b128 %{TM+i}, %{TM+TN+1} offset:{4096*i}" for i in range(TN)])
    frag_t = ([f"ds_read_b128 %{j}, %{TM+2*TN} offset:{4096*j}" for j in range(TM)] +
              [f"ds_read_b64_tr_b16 %{TM+i+TN*h}, %{TM+2*TN+1+i} offset:{2048*h}"
               for i in range(TN) for h in range(2)])
    frag_outs = ", ".join([f'"=&v"(nt[{j}])' for j in range(TM)] + [f'"=&v"(nw[{i}])' for i in range(TN)])
    stg = []
    for b in range(LA):
        stg += [f"s_add_u32 m0, %{LA+LB}, 0x{b*0x400:x}", "s_nop 0", f"global_load_lds_dwordx4 %{b}, %{LA+LB+2}"]
    for b in range(LB):
        stg += [f"s_add_u32 m0, %{LA+LB+1}, 0x{b*0x400:x}", "s_nop 0",
                f"global_load_lds_dwordx4 %{LA+b}, %{LA+LB+3}"]
    stg_ins = ", ".join([f'"v"(ao[{b}])' for b in range(LA)] + [f'"v"(bo[{b}])' for b in range(LB)])
    stg_a = []
    for b in range(LA):
        stg_a += [f"s_add_u32 m0, %{LA}, 0x{b*0x400:x}", "s_nop 0", f"global_load_lds_dwordx4 %{b}, %{LA+1}"]
    ao_ins = ", ".join(f'"v"(ao[{b}])' for b in range(LA))
    sig_cur = f"const bf16x8_t (&w)[{TN}], const bf16x8_t (&t)[{TM}]"
    sig_next = f"bf16x8_t (&nw)[{TN}], bf16x8_t (&nt)[{TM}]"
    return f'''
// ---- wave tile {32*TM} tokens x {32*TN} features ({TM}x{TN} MFMA tiles)
__device__ __forceinline__ void step_{n}(f32x16_t (&acc)[{TN}][{TM}], {sig_cur},
    {sig_next}, uint32_t ta, uint32_t wa) {{
  asm volatile(
{step_body(TM, TN, False)}
      : {acc_list(TM, TN)},
        {next_list(TM, TN)}
      : {cur_list(TM, TN)}, "v"(ta), "v"(wa)
      : "memory");
}}

{dma_half(TM, TN, 0)}
{dma_half(TM, TN, 1)}
// the last K16 step of a tile; its results are read by VALU next (24 wait states)
__device__ __forceinline__ void last_{n}(f32x16_t (&acc)[{TN}][{TM}], {sig_cur}) {{
  asm volatile(
{last}
      "s_nop 7"
      : {acc_list(TM, TN)}
      : {cur_list(TM, TN)}
      : "memory");
}}

// the first fragments of a tile (early-clobber: a read may land before the
// later reads are issued, so no destination may share an address register)
__device__ __forceinline__ void frags_{n}({sig_next}, uint32_t ta, uint32_t wa) {{
  asm volatile(
{chr(10).join(q(s) for s in frag)}
      "s_waitcnt lgkmcnt(0)"
      : {frag_outs}
      : "v"(ta), "v"(wa)
      : "memory");
}}

// Variants for a K-major weight stage: the weight fragments come from
// transposing reads, in 64-bit halves the caller joins.
__device__ __forceinline__ void step_t_{n}(f32x16_t (&acc)[{TN}][{TM}], {sig_cur},
    bf16x8_t (&nt)[{TM}], v4i16 (&nlo)[{TN}], v4i16 (&nhi)[{TN}], uint32_t ta, const uint32_t (&wa)[{TN}]) {{
  asm volatile(
{step_body(TM, TN, False, None, True)}
      : {acc_list(TM, TN)},
        {next_list_t(TM, TN)}
      : {cur_list(TM, TN)}, "v"(ta), {wa_list(TN)}
      : "memory");
}}

{dma_half(TM, TN, 0, True)}
{dma_half(TM, TN, 1, True)}

__device__ __forceinline__ void frags_t_{n}(bf16x8_t (&nt)[{TM}], v4i16 (&nlo)[{TN}], v4i16 (&nhi)[{TN}],
    uint32_t ta, const uint32_t (&wa)[{TN}]) {{
  asm volatile(
{chr(10).join(q(s) for s in frag_t)}
      "s_waitcnt lgkmcnt(0)"
      : {next_list_t(TM, TN)}
      : "v"(ta), {wa_list(TN)}
      : "memory");
}}

// one stage's LDS-DMA loads of the token tile only ({LA} blocks)
__device__ __forceinline__ void stage_a_{n}(const uint32_t (&ao)[{LA}], uint32_t la, const char* ga) {{
  asm volatile(
{chr(10).join(q(x) for x in stg_a[:-1])}
      "{stg_a[-1]}"
      :
      : {ao_ins},
        "s"(la), "s"(ga)
      : "memory", "m0", "scc");
}}

// one stage's LDS-DMA loads: {LA} token blocks, then {LB} weight blocks
__device__ __forceinline__ void stage_{n}(const uint32_t (&ao)[{LA}], const uint32_t (&bo)[{LB}],
    uint32_t la, uint32_t lb, const char* ga, const char* gw) {{
  asm volatile(
{chr(10).join(q(s) for s in stg[:-1])}
      "{stg[-1]}"
      :
      : {stg_ins},
        "s"(la), "s"(lb), "s"(ga), "s"(gw)
      : "memory", "m0", "scc");
}}
'''


def emit_w_stage(TN=4):
    """One stage's weight loads alone (the weight ring runs ahead of the
    token ring, so a tile's first weight stages come without token loads)."""
    LB = 2 * TN
    stg = []
    for b in range(LB):
        stg += [f"s_add_u32 m0, %{LB}, 0x{b*0x400:x}", "s_nop 0", f"global_load_lds_dwordx4 %{b}, %{LB+1}"]
    ins = ", ".join(f'"v"(bo[{b}])' for b in range(LB))
    return f'''
// one stage's LDS-DMA loads of the weight tile only ({LB} blocks)
__device__ __forceinline__ void stage_w_b{LB}(const uint32_t (&bo)[{LB}], uint32_t lb, const char* gw) {{
  asm volatile(
{chr(10).join(q(s) for s in stg[:-1])}
      "{stg[-1]}"
      :
      : {ins},
        "s"(lb), "s"(gw)
      : "memory", "m0", "scc");
}}
'''


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    parts = ["// Generated by gen_mfma_steps.py; do not edit by hand.\n"
             "// Inline-asm K16 steps of the bf16 grouped GEMM (included by ffn_bf16.hip).\n"
             "#pragma clang diagnostic push\n#pragma clang diagnostic ignored \"-Winline-asm\"\n"]
    for TM, TN in SHAPES:
        parts.append(emit(TM, TN))
    parts.append(emit_w_stage())
    parts.append("#pragma clang diagnostic pop\n")
    with open(os.path.join(here, "mfma_steps.inc"), "w") as f:
        f.write("".join(parts))


if __name__ == "__main__":
    main()
