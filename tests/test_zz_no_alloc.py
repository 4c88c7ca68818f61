"""The allocation-free entry point (jolt_decode_attention_noalloc) against the
workspace entry point it mirrors: with the fixed block schedule both run the
same kernels on the same inputs, so their outputs must be bitwise equal --
for two calls in a row, the second on a smaller input (the library's static
buffer keeps the first call's partials), on the MFMA and the float32 kernel.
A call that needs more partials than the buffer holds is refused before
anything is launched."""
import numpy as np
import pytest

import compressed_cache_decode_jolt_amd as J
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    J.lib()


def both(caches, q, q_pos, inv, kernel, split):
    hs = [J.jolt_load_cache(c) for c in caches]
    qt = torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).cuda()
    o1 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    o2 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(J.jolt_decode_workspace_size(hs, 0, kernel=kernel, split_tokens=split),
                     dtype=torch.uint8, device="cuda")
    J.jolt_decode_attention(hs, 0, qt, q_pos, inv, 0.088, o1, ws, kernel=kernel,
                            split_tokens=split, deterministic=True)
    J.jolt_decode_attention_noalloc(hs, 0, qt, q_pos, inv, 0.088, o2, kernel=kernel,
                                    split_tokens=split, deterministic=True)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), o2.cpu().numpy()


@pytest.mark.parametrize("kernel", [J.KERNEL_MFMA, J.KERNEL_GENERIC])
def test_noalloc_matches_workspace_entry_point(kernel):
    d, H, H_q = 128, 4, 16
    inv = gen.rope_inv_freq_input(5e5, d)
    # first call: three sequences, long
    big = [gen.small_cache(190 + i, T, H, H_q, d, [((64, 32, 4), (96, 64, 8))], [1])
           for i, T in enumerate((3000, 2500, 1800))]
    q = np.stack([gen.queries(191, i, 0, H_q, d, "bf16") for i in range(3)])
    a, b = both(big, q, [3000, 2500, 1800], inv, kernel, 256)
    assert np.isfinite(a).all() and np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # second call: one short sequence (fewer splits than the first left behind)
    small = [gen.small_cache(195, 300, H, H_q, d, [((32, 16, 2), (48, 32, 4))], [1])]
    q = gen.queries(196, 0, 0, H_q, d, "bf16")[None]
    a, b = both(small, q, [300], inv, kernel, 0)
    assert np.isfinite(a).all() and np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_refuses_more_partials_than_its_buffer():
    d, H, H_q, T = 128, 8, 32, 8192
    c = gen.small_cache(197, T, H, H_q, d, [((32, 16, 0), (512, 32, 0))], [1])
    hs = [J.jolt_load_cache(c), J.jolt_load_cache(c)]
    need = J.jolt_decode_workspace_size(hs, 0, kernel=J.KERNEL_GENERIC, split_tokens=32)
    assert need > J.jolt_noalloc_scratch_bytes()
    q = torch.zeros((2, H_q, d), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((2, H_q, d), dtype=torch.float32, device="cuda")
    with pytest.raises(J.JoltError) as e:
        J.jolt_decode_attention_noalloc(hs, 0, q, [T, T], gen.rope_inv_freq_input(5e5, d), 0.088,
                                        out, kernel=J.KERNEL_GENERIC, split_tokens=32)
    assert e.value.status == -5
