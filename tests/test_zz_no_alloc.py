"""The allocation-free decode entry point (qlayer_decode_noalloc, for callers
that cannot allocate device memory) against qlayer_decode of a handle on the
same inputs: two calls in a row on one GPU, the second with fewer sequences,
output and caches equal bit for bit (the same kernels run on the same data;
only the workspace differs)."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from harness import log, small_cfg, small_moe_cfg, weights_for  # noqa: E402
from transformer_decoder_layer_qwen_amd import binding as B  # noqa: E402
from transformer_decoder_layer_qwen_amd import configs, synth  # noqa: E402

pytestmark = pytest.mark.gpu


def decode_noalloc(layer, x, lens, lens_host, kc, vc):
    Bn = x.shape[0]
    y = torch.full_like(x, float("nan"))
    arr = (ctypes.c_int * Bn)(*[int(v) for v in lens_host])
    B.qlayer_decode_noalloc(layer.c_config, layer.c_weights, x.data_ptr(), Bn, lens.data_ptr(),
                            ctypes.cast(arr, ctypes.c_void_p).value, 0, kc.data_ptr(),
                            vc.data_ptr(), kc.shape[1], y.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    return y


CASES = {
    # (config, weight seed, [(sequences, cache length, T_max), ...]): MFMA
    # tiles then the VALU GEMV path; MoE; the Qwen2.5-7B layer at B = 32 then 1
    "small_dense": (small_cfg(), 1000, [(70, 150, 160), (3, 40, 48)]),
    "small_moe": (small_moe_cfg(), 1000, [(40, 100, 104), (5, 17, 20)]),
    "qwen2.5-7b": (configs.QWEN25_7B, configs.weight_seed(2), [(32, 1024, 1025), (1, 700, 1025)]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_decode_matches_handle_decode(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg, wseed, calls = CASES[case]
    w_np, _ = weights_for(cfg, wseed)
    layer = B.QLayer(cfg, B.device_weights(w_np), max_tokens=1,
                     max_batch=max(c[0] for c in calls))
    for i, (Bn, L, T_max) in enumerate(calls):
        log(f"[gpu] noalloc {case}: call {i}: B={Bn} cache {L} T_max {T_max}")
        x, kc, vc, lens = synth.make_decode_input(cfg, 7000 + 10 * i, Bn, L, T_max=T_max)
        lens = np.array([max(0, L - (b * 7) % (L + 1)) for b in range(Bn)], np.int32)  # ragged
        xd = B.to_device(x)
        ld = torch.from_numpy(lens).cuda()
        k1, v1 = B.to_device(kc), B.to_device(vc)
        k2, v2 = k1.clone(), v1.clone()
        y1 = layer.decode(xd, ld, k1, v1, cache_len_host=lens.tolist())
        y2 = decode_noalloc(layer, xd, ld, lens.tolist(), k2, v2)
        torch.cuda.synchronize()
        assert torch.isfinite(y2.float()).all()
        assert torch.equal(y1, y2), case
        assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
        assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    layer.close()
