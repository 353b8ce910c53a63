"""The no-allocation quantize entry point (mx_quantize_noalloc) against
mx_quantize, through the C ABI: two calls in a row on one GPU, the second on a
smaller tensor, each equal to mx_quantize's outputs bit for bit (codes,
scales, side outputs, dequantized values and the statistics record), for
formats whose kernels use scratch memory (fused statistics, the NVFP4 / E3M0
tensor pre-pass, column and 2D blocks) and one that uses none."""
import numpy as np
import pytest
import torch

import microscaling_block_quantization_amd as mx
import synth
from parity import to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("mxfp4 fast kernel + stats", mx.MXFP4, False, True),
    ("mxfp4 + dequant + stats", mx.MXFP4, True, True),
    ("nvfp4 pre-pass + stats", mx.Format(scale=mx.SCALE_NVFP4, block_cols=16), False, True),
    ("e3m0 scale pre-pass, no stats", mx.Format(scale=mx.SCALE_E3M0, rule=mx.RULE_CEIL), True, False),
    ("32x32 tiles + stats", mx.Format(block_rows=32, block_cols=32, round=mx.ROUND_SR, seed=3), True, True),
    ("h128 + oas, codes only", mx.Format(hadamard=128, rule=mx.RULE_OAS, oas_tau=7.5), False, False),
]

SHAPES = [(2048, 4096), (96, 1024)]       # the second call is smaller


def outputs(q, dq, st):
    t = [q.codes, q.scales]
    for extra in (q.offsets, q.macro_scales, q.tensor_scale, q.ref_exp, dq, st):
        if extra is not None:
            t.append(extra)
    return [x.detach().view(torch.uint8).reshape(-1).cpu().numpy() if x.dtype != torch.uint8
            else x.reshape(-1).cpu().numpy() for x in t]


@pytest.mark.parametrize("name,fmt,with_dq,with_stats", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_quantize(name, fmt, with_dq, with_stats):
    for i, (rows, cols) in enumerate(SHAPES):
        x = to_dev(synth.w4(shape=(rows, cols), seed=60 + i))
        res = []
        for noalloc in (False, True):
            q = mx.alloc_qtensor(fmt, rows, cols, x.device)
            dq = torch.empty((rows, cols), dtype=torch.float32, device=x.device) if with_dq else None
            st = torch.empty(48, dtype=torch.uint8, device=x.device) if with_stats else None
            if noalloc:
                mx.mx_quantize_noalloc(fmt, x, out=q, dequant=dq, stats=st)
            else:
                mx.mx_quantize(fmt, x, out=q, dequant=dq, stats=st)
            torch.cuda.synchronize()
            res.append(outputs(q, dq, st))
        for a, b in zip(*res):
            assert np.array_equal(a, b), f"{name}: call {i + 1} ({rows}x{cols}) differs"


def test_noalloc_refuses_more_than_its_scratch():
    x = torch.empty((1 << 15, 1 << 15), dtype=torch.bfloat16, device="cuda")  # 2 GiB, never read
    q = mx.QTensor(x.shape[0], x.shape[1], torch.empty(16, dtype=torch.uint8, device="cuda"),
                   torch.empty(16, dtype=torch.uint8, device="cuda"))
    st = torch.empty(48, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError) as e:
        mx.mx_quantize_noalloc(mx.MXFP4, x, out=q, stats=st)
    assert e.value.status == mx.MX_ERR_TOO_LARGE
