"""Host-side checks of the binding that need GPU tensors.  The library
launches its kernels on the current device, so a tensor or a stream of another
device is refused before the library is called.  No kernel runs here."""

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_binding_rejects_tensors_and_streams_of_another_device(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_entropy_amd import kvq
    plan = kvq.Plan(2, 128, 8, 6, 90, 62, 128, 1.4)
    c = kvq.alloc_cache(plan, 1, 128)
    k = torch.zeros(1, 128, 256, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    assert (kvq._stream(stream).value or 0) == stream.cuda_stream     # the null stream is 0
    # pretend another device is current: every GPU tensor here is now foreign
    monkeypatch.setattr(torch.cuda, "current_device", lambda: k.device.index + 1)
    with pytest.raises(ValueError, match="current device"):
        kvq.kvq_encode_streams(plan, k, k, c["k_cont"], c["v_cont"], c["k_so"], c["v_so"],
                               c["k_mean_q"], c["k_mean_scale"])
    with pytest.raises(ValueError, match="current device"):
        kvq._stream(stream)
