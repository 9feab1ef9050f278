"""The decode plan's per-row partial counts on the GPU against the bench's
accounting of them.

The split-context decode ("vLLM and PagedAttention", §2 "Reworking the
Attention Computation": each block's attention is computed separately and the
results are combined) leaves each decode row a number of partial results that
the log-sum-exp merge combines.  The matrix-core partition kernel writes one
per work item:
- items are two 512-token partitions, or four for a sequence of nine
  partitions or more;
- a sequence's last item is split into one-partition pieces when it covers
  more than one partition;
- a row whose sequence has one record is written directly (count 1).

The plan launch writes these counts into the workspace (the merge reads them).
`bench.partial_slots` prices the partial results of the bench line's
algorithmic bytes from the same rule, written independently on the host.
This test checks that the two agree for contexts on every edge of the rule
and for a seeded random mix.  The counts sit after the 256-byte ticket header
and the decode records: one int32 per row.
"""

import math

import numpy as np
import pytest
import torch

import bench
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_360_amd") if torch.cuda.is_available() else None

SCHED_BYTES = 256
DEC_RECORD_BYTES = 16
EDGE_CONTEXTS = [1, 15, 16, 17, 511, 512, 513, 1023, 1024, 1025, 1535, 1536, 1537, 2048, 2049, 2560, 2561,
                 3072, 3073, 3584, 4095, 4096, 4097, 4607, 4608, 4609, 5120, 5121, 5632, 6144, 6145, 6656,
                 7168, 8192, 8193, 9000, 12345, 16384, 16385, 20000, 32768, 32769]


def _align256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("seed", [0, 1])
def test_plan_slot_counts_match_the_bench_accounting(seed):
    rng = np.random.default_rng(seed)
    rand = np.exp(rng.uniform(0.0, math.log(40000.0), 300)).astype(np.int64)
    ctx = np.concatenate([np.array(EDGE_CONTEXTS, np.int64), rand]).astype(np.int32)
    rng.shuffle(ctx)
    S, Hq, Hkv, D, nb = ctx.size, 4, 1, 64, 4096
    bound = int(ctx.max())
    mb = -(-bound // 16)
    tables = ((np.arange(S)[:, None] * 7 + np.arange(mb)[None, :]) % nb).astype(np.int32)
    kc = torch.zeros((nb, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    ws = pkv.decode_workspace(S, Hq, D, bound)
    say(f"plan slots: seed {seed}, {S} sequences, contexts up to {bound}")
    pkv.pkv_attention_decode_plan(out, q, kc, vc, dev(tables), dev(ctx), 1.0 / math.sqrt(D), bound, workspace=ws)
    torch.cuda.synchronize()
    P = max(1, -(-bound // 512))
    off = SCHED_BYTES + _align256(S * P * DEC_RECORD_BYTES)
    got = ws[off:off + 4 * S].cpu().numpy().view(np.int32)
    want = bench.partial_slots(np, ctx.astype(np.int64), True)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(int(ctx[i]), int(got[i]), int(want[i])) for i in bad[:10]]
