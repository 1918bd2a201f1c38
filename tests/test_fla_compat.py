"""Host-side checks of the FLA-convention entry: its signature and the argument
errors it raises before touching any device."""
import inspect

import pytest


def test_signature_follows_the_fla_entry():
    from gated_deltanet_chunked_delta_amd.fla_compat import chunk_gated_delta_rule
    params = list(inspect.signature(chunk_gated_delta_rule).parameters.values())
    names = [p.name for p in params]
    assert names == ["q", "k", "v", "g", "beta", "scale", "initial_state", "output_final_state", "cu_seqlens",
                     "head_first", "use_qk_l2norm_in_kernel"]
    defaults = {p.name: p.default for p in params if p.default is not inspect.Parameter.empty}
    assert defaults == dict(scale=None, initial_state=None, output_final_state=False, cu_seqlens=None,
                            head_first=False, use_qk_l2norm_in_kernel=False)


def test_packed_sequences_need_batch_one():
    import torch
    from gated_deltanet_chunked_delta_amd import GDNError
    from gated_deltanet_chunked_delta_amd.fla_compat import chunk_gated_delta_rule
    q = torch.zeros(2, 8, 1, 64)
    g = torch.zeros(2, 8, 1)
    with pytest.raises(GDNError, match="batch size 1"):
        chunk_gated_delta_rule(q, q, q, g, g, cu_seqlens=torch.tensor([0, 4, 8]))


def test_rank_errors():
    import torch
    from gated_deltanet_chunked_delta_amd import GDNError
    from gated_deltanet_chunked_delta_amd.fla_compat import chunk_gated_delta_rule
    q = torch.zeros(1, 8, 1, 64)
    g = torch.zeros(1, 8, 1)
    with pytest.raises(GDNError, match="4-d"):
        chunk_gated_delta_rule(q[0], q, q, g, g)
    with pytest.raises(GDNError, match="3-d"):
        chunk_gated_delta_rule(q, q, q, g[0], g)
