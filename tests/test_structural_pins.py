"""The structural checks can fail: planted mistakes in copies of the oracle.

The GPU tests compare the kernels with the oracle on inputs from
``structural_checks``: peaked queries (every row's softmax puts half its mass
on one target token, and over the rows every block of a context is a target)
and tied-key queries (three equal keys, one in one 512-token partition and
two in another).
Here, on the CPU, each kind of mistake a paged kernel can make -- a block
dropped, a block read twice, a block read from the wrong place, a causal mask
one key short, partition partials merged with wrong weights -- is planted in a
copy of the oracle's computation, and the check must flag it by at least
WIDE times the bf16 bar (2e-2) in the gate it fails.  The real oracle passes.
This is what makes a pass of the GPU tests evidence that every block was read
once, from the right place, and that the merge weighs partitions correctly
("vLLM and PagedAttention", §2 "Reworking the Attention Computation": each
block's attention computed separately, then accumulated).
"""

import numpy as np
import pytest

import oracle
import structural_checks as sc
from gpu_util import BF16_ABS, errors
from oracle.attention import widen

WIDE = 5.0
BS = 16


def attend(q_row, K, V, scale):
    """softmax(scale q.K^T) V over the given rows of K, V (float64)."""
    x = float(np.float32(scale)) * (K @ q_row)
    w = np.exp(x - x.max())
    return (w @ V) / w.sum()


def decode_with_positions(inp, positions_of, table_of=None):
    """Decode where sequence s reads logical positions positions_of(s, n) (a
    planted mistake may drop or repeat some; a pair (key positions, value
    positions) reads keys and values at different positions), through
    table_of(s) (default: its own table row)."""
    q = widen(inp["q"])
    S, Hq, D = q.shape
    Hkv = inp["key_cache"].shape[2]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    for s in range(S):
        n = int(inp["context_lens"][s])
        pos = positions_of(s, n)
        kpos, vpos = (pos if isinstance(pos, tuple) else (pos, pos))
        kpos, vpos = np.asarray(kpos, np.int64), np.asarray(vpos, np.int64)
        t = np.asarray(inp["block_tables"][s] if table_of is None else table_of(s))
        K = widen(inp["key_cache"][t[kpos // BS].astype(np.int64), kpos % BS])
        V = widen(inp["value_cache"][t[vpos // BS].astype(np.int64), vpos % BS])
        for h in range(Hq):
            out[s, h] = attend(q[s, h], K[:, h // G], V[:, h // G], inp["scale"])
    return out


def chunk_with_positions(inp, positions_of):
    """Causal chunk attention where row r of sequence s reads positions_of(s, last)
    for its visible keys 0 .. last (a planted mistake may change that set)."""
    q = widen(inp["q"])
    T, Hq, D = q.shape
    Hkv = inp["key_cache"].shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    qsl = inp["qsl"]
    for s in range(len(inp["context_lens"])):
        n, r0, r1 = int(inp["context_lens"][s]), int(qsl[s]), int(qsl[s + 1])
        t = np.asarray(inp["block_tables"][s])
        for r in range(r1 - r0):
            last = n - (r1 - r0) + r
            if last < 0:
                continue
            pos = np.asarray(positions_of(s, last), np.int64)
            K = widen(inp["key_cache"][t[pos // BS], pos % BS])
            V = widen(inp["value_cache"][t[pos // BS], pos % BS])
            for h in range(Hq):
                out[r0 + r, h] = attend(q[r0 + r, h], K[:, h // G], V[:, h // G], inp["scale"])
    return out


def margin(got, ref):
    """How far past the bf16 bars the worse gate is (1.0 = exactly at the bar)."""
    a, r = errors(got, ref)
    return max(a / BF16_ABS, r / BF16_ABS)


# ------------------------------------------------------------------ decode sweep
@pytest.fixture(scope="module")
def decode_sweep():
    # 64 blocks, 16 sequences x 4 q heads per KV head: every block is a target
    # of every KV head (the GPU sweep uses 8192 tokens and 128 sequences)
    inp = sc.peaked_decode_case(21, 16, 32, 8, 64, 1024)
    ref = oracle.decode_attention(inp["q"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                                  inp["context_lens"], inp["scale"])
    return inp, ref


def test_decode_sweep_inputs_have_power(decode_sweep):
    inp, ref = decode_sweep
    nblk = 1024 // BS
    G = 4
    for g in range(8):
        covered = set((inp["targets"][:, g * G:(g + 1) * G] // BS).reshape(-1).tolist())
        assert covered == set(range(nblk)), f"KV head {g} misses blocks"
    assert np.all(np.abs(inp["mass"] - sc.PEAK_MASS) < 1e-6)
    assert np.min(np.max(np.abs(ref), axis=-1)) > 0.3, "outputs must be unit scale"
    assert margin(decode_with_positions(inp, lambda s, n: np.arange(n)), ref) < 1e-9


@pytest.mark.parametrize("b", list(range(0, 64, 1)))
def test_decode_sweep_flags_dropped_block(decode_sweep, b):
    inp, ref = decode_sweep
    got = decode_with_positions(inp, lambda s, n: np.array([j for j in range(n) if j // BS != b]))
    assert margin(got, ref) > WIDE


@pytest.mark.parametrize("b", [0, 1, 17, 31, 32, 50, 63])
def test_decode_sweep_flags_block_read_twice(decode_sweep, b):
    inp, ref = decode_sweep
    got = decode_with_positions(inp, lambda s, n: np.concatenate([np.arange(n), np.arange(b * BS, min(n, b * BS + BS))]))
    assert margin(got, ref) > WIDE


@pytest.mark.parametrize("b", [0, 9, 40, 63])
def test_decode_sweep_flags_misplaced_block(decode_sweep, b):
    """Block b read through the next sequence's table row, or with its value
    rows one offset away from their key rows."""
    inp, ref = decode_sweep
    S = len(inp["context_lens"])

    def wrong_row(s):
        t = inp["block_tables"][s].copy()
        t[b] = inp["block_tables"][(s + 1) % S][b]
        return t
    assert margin(decode_with_positions(inp, lambda s, n: np.arange(n), table_of=wrong_row), ref) > WIDE

    def mispaired(s, n):
        k = np.arange(n)
        v = k.copy()
        inb = v // BS == b
        cnt = min(BS, n - b * BS)                       # the block's tokens inside the context
        v[inb] = b * BS + (v[inb] - b * BS + 1) % cnt
        return k, v
    assert margin(decode_with_positions(inp, mispaired), ref) > WIDE


# ------------------------------------------------------------------ chunk sweep
@pytest.fixture(scope="module")
def chunk_sweep():
    inp = sc.peaked_chunk_case(22, 32, 8, 64, [64, 1, 100], [600, 700, 1100])
    ref = oracle.causal_chunk_attention(inp["q"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                                        inp["context_lens"], inp["qsl"], inp["scale"])
    return inp, ref


def test_chunk_sweep_inputs_have_power(chunk_sweep):
    inp, ref = chunk_sweep
    live = inp["targets"] >= 0
    assert np.all(np.abs(inp["mass"][live] - sc.PEAK_MASS) < 1e-6)
    assert np.min(np.max(np.abs(ref), axis=-1)) > 0.3
    # the causal edge (the row's own position) is a target of every row
    qsl, ctx = inp["qsl"], inp["context_lens"]
    for s in range(3):
        ql = qsl[s + 1] - qsl[s]
        edge = ctx[s] - ql + np.arange(ql)
        assert np.all(inp["targets"][qsl[s]:qsl[s + 1], 0] == edge)
    # every block of the 1100-token chunk's context is a target of every KV head
    t = inp["targets"][qsl[2]:qsl[3]]
    for g in range(8):
        assert set((t[:, 4 * g:4 * g + 4] // BS).reshape(-1).tolist()) == set(range(-(-1100 // BS)))
    assert margin(chunk_with_positions(inp, lambda s, last: np.arange(last + 1)), ref) < 1e-9


@pytest.mark.parametrize("b", list(range(0, 69, 4)) + [68])
def test_chunk_sweep_flags_dropped_block(chunk_sweep, b):
    inp, ref = chunk_sweep
    got = chunk_with_positions(inp, lambda s, last: np.array([j for j in range(last + 1) if j // BS != b]))
    assert margin(got, ref) > WIDE


@pytest.mark.parametrize("b", [0, 33, 68])
def test_chunk_sweep_flags_block_read_twice(chunk_sweep, b):
    inp, ref = chunk_sweep
    got = chunk_with_positions(inp, lambda s, last: np.concatenate(
        [np.arange(last + 1), np.arange(b * BS, min(last + 1, b * BS + BS))]))
    assert margin(got, ref) > WIDE


def test_chunk_sweep_flags_causal_mask_one_short(chunk_sweep):
    inp, ref = chunk_sweep
    got = chunk_with_positions(inp, lambda s, last: np.arange(max(1, last)))
    assert margin(got, ref) > WIDE


# ------------------------------------------------------------------ tied keys
def split_merge_decode(inp, merge):
    """Decode through 512-token partitions: per-partition (m, l, o) from the
    oracle's split, combined by `merge` (the oracle's or a planted mistake)."""
    q = widen(inp["q"])
    S, Hq, D = q.shape
    G = Hq // inp["key_cache"].shape[2]
    out = np.zeros((S, Hq, D))
    for s in range(S):
        K, V = oracle.gather_kv(inp["key_cache"], inp["value_cache"], inp["block_tables"][s],
                                int(inp["context_lens"][s]))
        for h in range(Hq):
            x = float(np.float32(inp["scale"])) * (K[:, h // G] @ q[s, h])
            m, l, o = oracle.split_decode_partials(x, V[:, h // G], 512)
            out[s, h] = merge(m, l, o)
    return out


def _merge_no_max(m, l, o):
    return (l[:, None] * o).sum(0) / l.sum()


def _merge_no_sum(m, l, o):
    w = np.exp(m - m.max())
    return (w[:, None] * o).sum(0) / w.sum()


def _merge_uniform(m, l, o):
    return o.mean(0)


def _merge_last_wins(m, l, o):
    return o[-1]


@pytest.fixture(scope="module")
def tied():
    inp = sc.tied_keys_decode_case(23, 32, 8, 64, [600, 1100, 1600, 2100, 2600, 3000, 514, 1800, 1025])
    return inp, sc.tied_keys_expected(inp)


def test_tied_keys_closed_form_is_the_oracle(tied):
    inp, cf = tied
    ref = oracle.decode_attention(inp["q"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                                  inp["context_lens"], inp["scale"])
    assert np.abs(ref - cf).max() < 1e-9
    assert np.min(np.max(np.abs(cf), axis=-1)) > 0.3
    assert np.abs(split_merge_decode(inp, oracle.merge_partials) - cf).max() < 1e-9
    parts = inp["tied"] // 512
    assert np.all(parts[:, 0] < parts[:, 1]) and np.all(parts[:, 1] == parts[:, 2])


@pytest.mark.parametrize("merge", [_merge_no_max, _merge_no_sum, _merge_uniform, _merge_last_wins],
                         ids=["no_max", "no_sum", "uniform", "last_wins"])
def test_tied_keys_flag_wrong_merge_weights(tied, merge):
    inp, cf = tied
    with np.errstate(all="ignore"):
        got = split_merge_decode(inp, merge)
    assert margin(got, cf) > WIDE


@pytest.mark.parametrize("which", [0, 1, 2])
def test_tied_keys_flag_dropped_block(tied, which):
    inp, cf = tied
    b = {s: int(inp["tied"][s, which]) // BS for s in range(len(inp["context_lens"]))}
    got = decode_with_positions(inp, lambda s, n: np.array([j for j in range(n) if j // BS != b[s]]))
    assert margin(got, cf) > WIDE


def test_tied_keys_chunk_closed_form_is_the_oracle():
    inp = sc.tied_keys_chunk_case(24, 32, 8, 64, [64, 1, 200], [700, 900, 2300])
    ref = oracle.causal_chunk_attention(inp["q"], inp["key_cache"], inp["value_cache"], inp["block_tables"],
                                        inp["context_lens"], inp["qsl"], inp["scale"])
    assert np.abs(ref - sc.tied_keys_expected(inp)).max() < 1e-9
