"""The calibration kernels run, and the streaming read reads every byte of
its buffer exactly once: the XOR of what its waves store equals the XOR of
all words of the buffer."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 37, 64 << 20])
def test_peak_read_covers_every_byte_once(nbytes):
    import gemm_wq_quantize_amd as wq
    print(f"wq_peak_read nbytes={nbytes}", flush=True)
    gen = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=gen)
    buf = host.cuda()
    sink = torch.zeros(wq.wq_peak_read_sink_words(), dtype=torch.int32, device="cuda")
    wq.wq_peak_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_peak_loops_run():
    import gemm_wq_quantize_amd as wq
    print("wq_peak_mfma_bf16 / wq_peak_valu_fma", flush=True)
    sink = torch.zeros(8 * 256, dtype=torch.float32, device="cuda")
    wq.wq_peak_mfma_bf16(8, 16, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all() and (sink != 0).any()
    sink.zero_()
    wq.wq_peak_valu_fma(8, 64, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all() and (sink != 0).any()
