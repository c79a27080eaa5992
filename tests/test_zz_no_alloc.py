"""GPU: eagle_lm_head_argmax_noalloc (scratch in a static device array, nothing
allocated) against eagle_lm_head_argmax (caller workspace), called through the C ABI.

Both run the same kernels on the same plan, so every output (max, argmax, second,
lse and the fp32 logits) must agree bit for bit.  Two calls in a row, the second on a
smaller problem, so the second call reads the array the first one left behind; and a
size past the array's limit, which the host rejects before launching anything."""
import numpy as np
import pytest
import torch

import speculative_decoding_attn_amd as sda
import synth
from inputs import to_dev_bf16

pytestmark = pytest.mark.gpu

UNSUPPORTED = 3


def _outputs(M, V, dev):
    f = dict(device=dev)
    return {"max": torch.full((M,), float("nan"), dtype=torch.float32, **f),
            "argmax": torch.full((M,), -7, dtype=torch.int32, **f),
            "lse": torch.full((M,), float("nan"), dtype=torch.float32, **f),
            "second": torch.full((M,), float("nan"), dtype=torch.float32, **f),
            "logits": torch.full((M, V), float("nan"), dtype=torch.float32, **f)}


def _call(lib, hidden, weight, out, noalloc):
    M, H = hidden.shape
    V = weight.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    args = [hidden.data_ptr(), weight.data_ptr(), M, H, V, sda.EAGLE_BF16, out["max"].data_ptr(),
            out["argmax"].data_ptr(), out["lse"].data_ptr(), out["second"].data_ptr(),
            out["logits"].data_ptr()]
    if noalloc:
        return lib.eagle_lm_head_argmax_noalloc(*args, stream)
    ws = torch.empty(lib.eagle_lm_head_workspace(M, H, V), dtype=torch.uint8, device=hidden.device)
    return lib.eagle_lm_head_argmax(*args, ws.data_ptr(), ws.numel(), stream)


# (M, H, V): the second is smaller in every dimension than the first
SIZES = [(240, 1024, 50000), (37, 512, 3001)]


def test_noalloc_matches_workspace_call_twice(gpu_lib):
    lib = sda.load()
    dev = torch.device("cuda")
    for i, (M, H, V) in enumerate(SIZES):
        print(f"lm head noalloc call {i}: M={M} H={H} V={V}", flush=True)
        hidden = to_dev_bf16(synth.normal_bf16_bits((M, H), 1.0, i, 820, 1))
        weight = to_dev_bf16(synth.normal_bf16_bits((V, H), H ** -0.5, i, 820, 2))
        got, want = _outputs(M, V, dev), _outputs(M, V, dev)
        assert _call(lib, hidden, weight, got, noalloc=True) == 0, lib.eagle_last_error()
        assert _call(lib, hidden, weight, want, noalloc=False) == 0, lib.eagle_last_error()
        torch.cuda.synchronize()
        for key in want:
            g, w = got[key].cpu().numpy(), want[key].cpu().numpy()
            assert np.array_equal(g.view(np.uint32) if g.dtype == np.float32 else g,
                                  w.view(np.uint32) if w.dtype == np.float32 else w), key
        assert not np.isnan(got["lse"].cpu().numpy()).any()


def test_noalloc_rejects_sizes_past_the_static_scratch(gpu_lib):
    lib = sda.load()
    M, H, V = 2048, 64, 128256       # 2048 rows x 501 vocabulary tiles x 16 bytes > 8 MiB
    need = lib.eagle_lm_head_workspace(M, H, V)
    assert need > 8 << 20
    fake = 1 << 20                   # never dereferenced: the call fails on the host
    st = lib.eagle_lm_head_argmax_noalloc(fake, fake, M, H, V, sda.EAGLE_BF16, fake, fake, fake,
                                          None, None, None)
    assert st == UNSUPPORTED and b"static scratch" in lib.eagle_last_error()
