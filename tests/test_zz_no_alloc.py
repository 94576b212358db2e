"""dcoco_correct_block_static (no workspace argument, nothing allocated) against
dcoco_correct_block on the same inputs: the same kernels run, so every output
must be bit-identical.  Two calls in a row, the second smaller than the first,
so the second runs on a buffer still holding the first call's data."""
import numpy as np
import pytest

import synth
from helpers import device_inputs, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()


def _outputs(dims, dev):
    import torch
    N, B, K = dims.n_blocks, dims.B, dims.K
    return {"sel_tok": torch.full((N, B), -1, dtype=torch.int32, device=dev),
            "sel_idx": torch.full((N, B), -1, dtype=torch.int32, device=dev),
            "S": torch.full((N, max(B - 1, 1), K, K), float("nan"), dtype=torch.float32, device=dev),
            "cand_ids": torch.full((N, B, K), -1, dtype=torch.int32, device=dev),
            "cand_logits": torch.full((N, B, K), float("nan"), dtype=torch.float32, device=dev)}


def _compare(dims, w, logits, h, E, tag):
    import draft_block_contextual_amd as dc
    import torch
    dev = logits.device
    a = _outputs(dims, dev)
    b = _outputs(dims, dev)
    dc.correct_block(dims, w, logits, h, E, **a)
    dc.correct_block_static(dims, w, logits, h, E, **b)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), (tag, k)
    assert int((b["sel_tok"] < 0).sum()) == 0, tag


def test_static_matches_workspace_path_two_calls():
    import draft_block_contextual_amd as dc
    import torch
    assert dc.static_scratch_bytes() == 96 << 20
    # first call: the 32-stream workload (drawn on the GPU: only the two
    # device paths are compared), then a smaller bf16 shape, then fp32
    print("case static q8b_32", flush=True)
    g = synth.make_inputs_device("q8b_32", sets=1)
    D = g["dims"]
    dims = dc.Dims.from_synth(D)
    w = dc.Weights(P_e=g["P_e"], P_h=g["P_h"], W_f=g["W_f"], W_pair=g["W_pair"], W1=g["W1"], b1=g["b1"],
                   w2=g["w2"], b2=g["b2"])
    lg, h = g["sets"][0]
    need = dc.correct_block_workspace_bytes(dims, w)
    assert need <= dc.static_scratch_bytes()
    _compare(dims, w, lg, h, g["E"], "q8b_32")
    del g, w, lg, h
    for name in ("mid_bf16", "small_bf16", "tiny"):
        print(f"case static {name}", flush=True)
        inp = synth.make_inputs(name)
        dims, w, logits, h, E = device_inputs(inp)
        _compare(dims, w, logits, h, E, name)


def test_static_rejects_problems_beyond_its_buffer():
    import draft_block_contextual_amd as dc
    print("case static too large", flush=True)
    # the d = 8192 workload needs several times the buffer; the call must
    # refuse before launching (no inputs are touched: the pointers are null)
    dims = dc.Dims.from_synth(synth.get_config("large").dims)
    w = dc.Weights(None, None, None, None, None, None, None, 0.0)
    assert dc.correct_block_workspace_bytes(dims, w) > dc.static_scratch_bytes()
    with pytest.raises(dc.DcocoError) as e:
        dc.correct_block_static(dims, w, None, None, None, None)
    assert e.value.status == dc.DCOCO_ERR_UNSUPPORTED
