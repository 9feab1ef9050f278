"""pkv_attention_decode_noalloc: decode with the library's static workspace.

The entry point is for callers that cannot allocate device memory.  Through the
C ABI, its output must equal pkv_attention_decode's with a caller workspace
byte for byte (same kernels, same work list), on two calls in a row where the
second is smaller (the array keeps the first call's contents; the plan launch
resets what must start at zero).  A batch whose workspace would exceed the
array is refused before any HIP call.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, host, host_f64, say
from workloads import normal_values, random_block_tables

pkv = pytest.importorskip("paged_kv_cache_360_amd")
from paged_kv_cache_360_amd._lib import (PKV_BF16, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_F32,  # noqa: E402
                                         STATIC_WORKSPACE_BYTES, lib)

FAKE = 0x10000


def _case(seed, S, Hq, Hkv, D, ctx_lo, ctx_hi, dtype):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=S).astype(np.int32)
    nb = int(np.sum(-(-ctx // 16))) + 7
    mb = int(-(-ctx.max() // 16)) + 1
    tables = random_block_tables(rng, ctx, nb, mb)
    return {"ctx": ctx, "tables": tables, "nb": nb, "mb": mb, "Hq": Hq, "Hkv": Hkv, "D": D, "dtype": dtype,
            "kc": normal_values(rng, (nb, 16, Hkv, D), dtype), "vc": normal_values(rng, (nb, 16, Hkv, D), dtype),
            "q": normal_values(rng, (S, Hq, D), dtype), "scale": np.float32(1.0 / math.sqrt(D))}


def _noalloc(c, out, q, kc, vc, tables, ctx):
    S = len(c["ctx"])
    return lib().pkv_attention_decode_noalloc(
        out.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(), tables.data_ptr(), ctx.data_ptr(),
        float(c["scale"]), 16, c["Hq"], c["Hkv"], c["D"], S, c["mb"], c["nb"], int(c["ctx"].max()),
        PKV_BF16 if c["dtype"] == "bf16" else PKV_F32, torch.cuda.current_stream().cuda_stream)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_decode_on_two_calls(dtype):
    # first call: the bench's shape class (GQA 32/8, head_dim 128, contexts up
    # to 8192: a workspace of tens of MB); second: a smaller MHA batch
    cases = [_case(91, 128, 32, 8, 128, 512, 8192, dtype), _case(92, 40, 16, 16, 64, 1, 3000, dtype)]
    need = [pkv.pkv_decode_workspace_bytes(len(c["ctx"]), c["Hq"], c["D"], int(c["ctx"].max())) for c in cases]
    say(f"noalloc {dtype}: workspaces {need} bytes, static array {STATIC_WORKSPACE_BYTES}")
    assert need[0] > need[1] and need[0] <= STATIC_WORKSPACE_BYTES
    for i, c in enumerate(cases):
        q, kc, vc = dev(c["q"]), dev(c["kc"]), dev(c["vc"])
        tables, ctx = dev(c["tables"]), dev(c["ctx"])
        ref = torch.full_like(q, float("nan"))
        pkv.pkv_attention_decode(ref, q, kc, vc, tables, ctx, float(c["scale"]), int(c["ctx"].max()),
                                 workspace=pkv.decode_workspace(len(c["ctx"]), c["Hq"], c["D"], int(c["ctx"].max())))
        got = torch.full_like(q, float("nan"))
        assert _noalloc(c, got, q, kc, vc, tables, ctx) == 0, lib().pkv_last_error()
        torch.cuda.synchronize()
        assert host(got).tobytes() == host(ref).tobytes(), f"call {i}: differs from pkv_attention_decode"
        rows = np.unique(np.concatenate([np.argsort(c["ctx"])[[0, -1]], [len(c["ctx"]) // 2]]))
        want = oracle.decode_attention(c["q"][rows], c["kc"], c["vc"], c["tables"][rows], c["ctx"][rows], c["scale"])
        assert_close(host_f64(got)[rows], want, dtype, f"noalloc call {i}")


def test_noalloc_refuses_batches_beyond_the_static_array():
    """Checked on the host before any HIP call (no GPU needed)."""
    L = lib()

    def call(S=4, hq=32, hkv=8, d=128, mb=600, nb=100000, maxctx=9000, bs=16):
        return L.pkv_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, bs, hq, hkv, d, S, mb, nb,
                                              maxctx, PKV_BF16, None)
    assert pkv.pkv_decode_workspace_bytes(1024, 32, 128, 9000) > STATIC_WORKSPACE_BYTES
    assert call(S=1024) == PKV_EWORKSPACE
    assert b"static" in L.pkv_last_error()
    assert call(bs=32) == PKV_EUNSUPPORTED            # the decode checks apply as well
