"""GPU test of parallax_attn_fwd_noalloc (MI355X only): the allocation-free
prefill, whose workspace is the library's own device array, against
parallax_attn_fwd with a caller workspace, on two calls in a row (the second
smaller, so it reuses the array that the first filled), and against the
oracle."""
import pytest
import torch

from gpu_util import compare, default_scale, f64, say
from parallax_local_linear_amd import parallax_attn_fwd, parallax_attn_fwd_noalloc, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_noalloc_matches_workspace_call_twice(orc):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    cases = [(2, 4, 3000, 128, 0, 0), (1, 3, 1000, 64, 128, 4)]
    for i, (B, H, L, d, window, n_sink) in enumerate(cases):
        say("[case] noalloc call %d: B=%d H=%d L=%d d=%d window=%d n_sink=%d"
            % (i, B, H, L, d, window, n_sink))
        q, k, v, r = (workloads.random_tensor((B, H, L, d), 4400 + 10 * i + t, device=DEV)
                      for t in range(4))
        o_ref, l_ref = parallax_attn_fwd(q, k, v, r, window=window, n_sink=n_sink)
        o = torch.full((B, H, L, d), float("nan"), device=DEV)
        lse = torch.full((B, H, L), float("nan"), device=DEV)
        parallax_attn_fwd_noalloc(q, k, v, r, window=window, n_sink=n_sink, out=o, lse=lse)
        torch.cuda.synchronize()
        # The same kernels on the same inputs: identical bits.
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        ref_o, ref_l = orc.fwd(f64(q[:1, :1]), f64(k[:1, :1]), f64(v[:1, :1]), f64(r[:1, :1]),
                               scale=default_scale(d), window=window, n_sink=n_sink)
        compare(f64(o[:1, :1]), f64(lse[:1, :1]), ref_o, ref_l, "noalloc call %d vs oracle" % i)


def test_noalloc_rejects_sizes_beyond_its_array():
    from parallax_local_linear_amd.binding import ParallaxError
    q = torch.zeros((2, 16, 8224, 128), dtype=torch.bfloat16, device=DEV)
    o = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    with pytest.raises(ParallaxError) as e:
        parallax_attn_fwd_noalloc(q, q, q, q, out=o, lse=lse)
    assert e.value.name == "PARALLAX_ERR_UNSUPPORTED"
