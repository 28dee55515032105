"""Find DPP instructions that may run under a partial exec mask (CFG-aware).

A DPP move reads a neighbouring lane's register; if that lane is inactive the
read returns 0 (bound_ctrl), silently.  The kernels exchange values between
lane pairs with quad_perm DPP and rely on every lane executing those moves, so
this checks the compiler's output: per kernel, split the gfx950 assembly into
basic blocks, track whether exec may be partial (s_and_saveexec and friends
make it partial, s_or_b64 exec, exec, s[..] restores it), propagate through
branches conservatively, and report every DPP instruction reached with a
possibly partial mask.
"""
import re

BR = re.compile(r's_(cbranch_\w+|branch)\s+(\.LBB\w+)')
PART = re.compile(r's_(and|andn2)_saveexec_b64|s_and_b64 exec,|s_andn2_b64 exec,|s_xor_b64 exec,')
FULL = re.compile(r's_or_b64 exec, exec,')


def scan(asm: str):
    """-> {kernel: (number of DPP instructions, number under a possibly partial mask)}"""
    out = {}
    for name in re.findall(r'^(_Z\w+):', asm, re.M):
        i = asm.index(name + ':')
        j = asm.find('.Lfunc_end', i)
        lines = [l.split(';')[0].strip() for l in asm[i:j].split('\n')[1:]]
        blocks, cur = [], []
        for t in lines:
            if not t:
                continue
            if re.match(r'\.LBB\w+:', t):
                if cur:
                    blocks.append(cur)
                cur = [t]
                continue
            cur.append(t)
            if BR.search(t) or t.startswith('s_endpgm') or t.startswith('s_setpc'):
                blocks.append(cur)
                cur = []
        if cur:
            blocks.append(cur)
        lab = {b[0][:-1]: k for k, b in enumerate(blocks) if b[0].startswith('.LBB') and b[0].endswith(':')}
        succ = {k: [] for k in range(len(blocks))}
        for k, b in enumerate(blocks):
            m = BR.search(b[-1])
            if m:
                succ[k].append(lab[m.group(2)])
                if m.group(1) != 'branch' and k + 1 < len(blocks):
                    succ[k].append(k + 1)
            elif not b[-1].startswith('s_endpgm') and k + 1 < len(blocks):
                succ[k].append(k + 1)
        state = {k: None for k in range(len(blocks))}
        if blocks:
            state[0] = False
        changed = True
        while changed:
            changed = False
            for k, b in enumerate(blocks):
                if state[k] is None:
                    continue
                st = state[k]
                for t in b:
                    if PART.search(t):
                        st = True
                    elif FULL.search(t):
                        st = False
                for n in succ[k]:
                    new = st if state[n] is None else (state[n] or st)
                    if new != state[n]:
                        state[n] = new
                        changed = True
        ndpp = bad = 0
        for k, b in enumerate(blocks):
            st = bool(state[k])
            for t in b:
                if PART.search(t):
                    st = True
                elif FULL.search(t):
                    st = False
                if 'quad_perm' in t or re.match(r'v_\w+_dpp', t):
                    ndpp += 1
                    bad += st
        out[name] = (ndpp, bad)
    return out
