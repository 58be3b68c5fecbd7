"""pa_decode_static (the decode entry point that allocates nothing) against
pa_decode with a caller workspace: same kernels, same grid, so the outputs
must agree bit for bit; both against the oracle within the tolerance.  Two
calls in a row, the second with a smaller input, then a shape whose partial
records exceed the static scratch, which is refused before any launch."""
import numpy as np
import pytest
import torch

from paged_kv_cache_157_amd import binding
from pa_testlib import TOL, max_err, oracle_problem, random_problem, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield


def _both(p, partition_tokens=0):
    a = torch.full(p["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full(p["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.decode(a, p["q"], p["k"], p["v"], p["bt"], p["lens"], p["scale"],
                   partition_tokens=partition_tokens, kv_scale=p["kv_scale"])
    binding.decode_static(b, p["q"], p["k"], p["v"], p["bt"], p["lens"], p["scale"],
                          partition_tokens=partition_tokens, kv_scale=p["kv_scale"])
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_static_scratch_matches_the_workspace_entry_point():
    rng = np.random.default_rng(81)
    # a Qwen2.5-7B-shaped batch (one KV head per work-group), then a smaller
    # batch of another shape (four KV heads per work-group, fp8 cache)
    big = random_problem(81, 64, 28, 4, 128, [int(x) for x in rng.integers(512, 4097, 64)],
                         11000, "bf16")
    small = random_problem(82, 9, 32, 8, 128, [1, 17, 300, 0, 2049, 16, 700, 5, 1024], 400, "fp8")
    for name, p, ptok in (("qwen7b-shaped", big, 0), ("small fp8", small, 0),
                          ("small fp8, fixed partitions", small, 64)):
        say(f"no-alloc decode: {name}")
        a, b = _both(p, ptok)
        assert np.array_equal(a, b), f"{name}: static scratch and workspace outputs differ"
        assert max_err(b, oracle_problem(p)) <= TOL[p["storage"]]
        assert np.all(b[3] == 0.0) if name.startswith("small") else True


def test_static_scratch_refuses_a_shape_that_does_not_fit():
    # tables 2048 entries wide (32k tokens) in fixed 16-token partitions: 8
    # sequences x 8 KV heads x 2048 partial records of 4 query heads x 130
    # floats = 272 MB > 31 MiB
    p = random_problem(83, 8, 32, 8, 128, [16] * 8, 64, "bf16", width=2048)
    out = torch.zeros(p["q"].shape, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.PAError) as ei:
        binding.decode_static(out, p["q"], p["k"], p["v"], p["bt"], p["lens"], p["scale"],
                              partition_tokens=16)
    assert ei.value.status == binding.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 0).all().item())  # nothing was launched
