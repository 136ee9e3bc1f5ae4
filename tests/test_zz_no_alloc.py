"""The allocation-free decode step (bsa_decode_topk_noalloc, static per-GPU
scratch) against bsa_decode_topk with a caller workspace: same kernels, so the
outputs and selections must be identical, on consecutive calls whose second
input is smaller (the static scratch keeps the first call's contents), on the
partitioned path (few rows: the scratch is used) and the fused path."""
import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
import block_sparse_attention_summarize_amd as bsa  # noqa: E402

W = synth.WORKLOADS["bf16_decode_l128k"]
CASES = [
    # rows = batch x kv heads = 4: partitioned path, scratch in use
    W.scaled(batch=2, hq=8, hkv=2, n=64 * 50, k_total=9, kv_lens=(3200, 1537)),
    # a smaller second input: 1 row, fewer blocks, shorter k
    W.scaled(batch=1, hq=4, hkv=1, n=64 * 16 + 9, k_total=5, kv_lens=(1000,)),
    # 128 rows: the fused single-launch path (no scratch)
    W.scaled(batch=16, hq=16, hkv=8, n=64 * 12, k_total=4),
    # B = 128, G = 8, fp32 output, back on the partitioned path
    W.scaled(batch=3, hq=8, hkv=1, n=128 * 20 + 5, B=128, k_total=6, kv_lens=(2565, 700, 129)),
]


def _run(w, out_f32):
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    lens = torch.tensor(w.lens(), dtype=torch.int32, device="cuda")
    odt = torch.float32 if out_f32 else None
    O1, i1, c1 = bsa.decode_step(x["Q"], x["K"], x["V"], S, w.B, w.k_total, w.force,
                                 kv_lens=lens, out_dtype=odt)
    O2, i2, c2 = bsa.decode_step_noalloc(x["Q"], x["K"], x["V"], S, w.B, w.k_total, w.force,
                                         kv_lens=lens, out_dtype=odt)
    torch.cuda.synchronize()
    return (O1, i1, c1), (O2, i2, c2)


@pytest.mark.parametrize("out_f32", [False, True])
def test_noalloc_decode_matches_workspace_decode(out_f32):
    for n, w in enumerate(CASES):
        print(f"[noalloc decode] case {n}: {w} out_f32={out_f32}", flush=True)
        (O1, i1, c1), (O2, i2, c2) = _run(w, out_f32)
        assert torch.equal(c1, c2) and torch.equal(i1, i2), f"case {n}: selections differ"
        assert torch.equal(O1, O2), f"case {n}: outputs differ"
        assert torch.isfinite(O2.float()).all()


def test_noalloc_decode_repeated_calls():
    """Two calls in a row on the same inputs reuse the scratch and agree."""
    w = CASES[0]
    (O1, i1, c1), (O2, i2, c2) = _run(w, False)
    (_, _, _), (O3, i3, c3) = _run(CASES[1], False)
    (_, _, _), (O4, i4, c4) = _run(w, False)
    assert torch.equal(O2, O4) and torch.equal(i2, i4) and torch.equal(c2, c4)
    assert torch.equal(O1, O4)
