"""The streaming-read probe (a measurement utility beside the attention path):
it reads every size in bounds, including sizes that leave a remainder after
the unrolled passes, and leaves the flag alone unless the fold hits its key."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words16,workgroups", [(1, 1), (5, 1), (5, 8), (1023, 3), (4096 * 4 + 7, 8),
                                                (1 << 20, 4096)])
def test_probe_stream_read(words16, workgroups):
    import torch
    import paged_kv_cache_fa_amd as fa
    src = torch.zeros(words16 * 4, dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"probe: {words16} x 16 B, {workgroups} workgroups", flush=True)
    fa.probe_stream_read(src, flag, workgroups)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0  # the fold of zeros is 0, not the key
