"""Plant plausible mistakes in a copy of the oracle and check the pins catch each one.

Every mutant below is a small edit of the oracle's decode (a dropped term, a wrong
index, a wrong sign, a transposed operand, a wrong head mapping ...).  The pins in
``oracle_pins`` must flag each mutant; a mutant that passes every pin would mean
the pins cannot tell that mistake from the real thing.  CPU only.
"""

import numpy as np
import pytest

import oracle
from oracle.attention import widen
from oracle_pins import DECODE_CHECKS


def _decode_factory(gather_off=lambda j, bs: j % bs, gather_blk=lambda j, bs: j // bs,
                    head_map=lambda h, G, Hkv: h // G, drop_last=False, no_max=False,
                    sign=1.0, transpose_v=False, scale_mode="ok", ctx_shift=0):
    def decode(q, kc, vc, tables, ctx, scale, block_size=16):
        qf = widen(q)
        S, Hq, D = qf.shape
        Hkv = kc.shape[2]
        G = Hq // Hkv
        sc = float(np.float32(scale))
        out = np.zeros((S, Hq, D))
        for s in range(S):
            n = int(ctx[s]) + ctx_shift
            if n <= 0:
                continue
            j = np.arange(n)
            blk = np.asarray(tables[s])[gather_blk(j, block_size)].astype(np.int64)
            K = widen(kc[blk, gather_off(j, block_size)])
            V = widen(vc[blk, gather_off(j, block_size)])
            for h in range(Hq):
                g = head_map(h, G, Hkv)
                x = K[:, g, :] @ qf[s, h]
                x = x * (sc if scale_mode == "ok" else (1.0 if scale_mode == "none" else sc * sc))
                x = sign * x
                m = 0.0 if no_max else x.max()
                w = np.exp(x - m)
                if drop_last:
                    w = w[:-1]
                Vg = V[:, g, :]
                if transpose_v:
                    Vg = np.flip(Vg, axis=0)
                out[s, h] = (w @ Vg[: len(w)]) / w.sum() if len(w) else 0.0
        return out
    return decode


MUTANTS = {
    "offset_plus_one": _decode_factory(gather_off=lambda j, bs: (j + 1) % bs),
    "block_index_off_by_one": _decode_factory(gather_blk=lambda j, bs: np.minimum(j // bs + (j % bs == bs - 1), j.max() // bs)),
    "gqa_modulo_mapping": _decode_factory(head_map=lambda h, G, Hkv: h % Hkv),
    "dropped_last_token": _decode_factory(drop_last=True),
    "negated_scores": _decode_factory(sign=-1.0),
    "reversed_values": _decode_factory(transpose_v=True),
    "scale_ignored": _decode_factory(scale_mode="none"),
    "scale_squared": _decode_factory(scale_mode="squared"),
    "context_one_short": _decode_factory(ctx_shift=-1),
}


def test_real_oracle_passes_factory_baseline():
    # the factory with no mutation is the oracle itself (sanity of the harness)
    base = _decode_factory()
    for name, (check, bound) in DECODE_CHECKS.items():
        assert check(base) <= bound, name
    assert oracle.decode_attention is not base


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mutant = MUTANTS[name]
    caught = []
    for check_name, (check, bound) in DECODE_CHECKS.items():
        with np.errstate(all="ignore"):
            try:
                v = check(mutant)
            except (IndexError, ValueError, FloatingPointError):
                v = float("inf")
        if not (v <= bound):
            caught.append(check_name)
    assert caught, f"mutant {name} passed every pin"
