"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes

import numpy as np
import pytest

from gated_deltanet_chunked_delta_amd import binding as B


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_symbol(L):
    names = B.exported_symbols()
    assert {"gdn_chunk_fwd", "gdn_chunk_bwd", "gdn_chunk_fwd_workspace_size",
            "gdn_chunk_bwd_workspace_size", "gdn_last_error", "gdn_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.gdn_abi_version() == 11


FAKE = 1 << 20  # a 16-byte aligned fake device address; never dereferenced


def fwd_args(**kw):
    a = B.CommonArgs()
    a.dtype, a.B, a.T, a.H, a.Dk, a.Dv = B.GDN_BF16, 1, 128, 2, 128, 128
    a.q = a.k = a.v = a.g = a.beta = FAKE
    a.scale = 0.1
    a.num_seqs = 1
    a.workspace = FAKE
    a.workspace_bytes = 1 << 30
    for key, val in kw.items():
        setattr(a, key, val)
    f = B.FwdArgs()
    f.a = a
    f.o = FAKE
    return f


def call_fwd(L, f):
    return L.gdn_chunk_fwd(ctypes.byref(f), None)


@pytest.mark.parametrize("field,value,status", [
    ("q", None, 1), ("g", None, 1), ("beta", None, 1),
    ("B", 0, 1), ("H", 0, 1), ("T", -1, 1),
    ("Dk", 96, 2), ("Dv", 32, 2), ("dtype", 7, 2),
    ("q", FAKE + 8, 1),          # misaligned
    ("cp_mode", -2, 1),
    ("num_seqs", 2, 1),          # != B without cu_seqlens
    ("workspace_bytes", 16, 3), ("workspace", None, 3),
])
def test_forward_rejects_bad_arguments(L, field, value, status):
    f = fwd_args(**{field: value})
    assert call_fwd(L, f) == status
    assert L.gdn_last_error()


def test_f32_only_head_size_64(L):
    assert call_fwd(L, fwd_args(dtype=B.GDN_F32)) == 2


def test_cu_seqlens_validation(L):
    import numpy as np
    for cu, status in [([0, 5, 3, 128], 1), ([1, 64, 128], 1), ([0, 64, 100], 1)]:
        host = np.array(cu, dtype=np.int32)
        f = fwd_args(cu_seqlens=FAKE, cu_seqlens_host=host.ctypes.data, num_seqs=len(cu) - 1)
        assert call_fwd(L, f) == status, cu
    host = np.array([0, 64, 128], dtype=np.int32)
    f = fwd_args(B=2, T=64, cu_seqlens=FAKE, cu_seqlens_host=host.ctypes.data, num_seqs=2)
    assert call_fwd(L, f) == 1           # B != 1 with cu_seqlens
    f = fwd_args(cu_seqlens=FAKE, num_seqs=2)
    assert call_fwd(L, f) == 1           # host copy missing


def test_workspace_size_query(L):
    f = fwd_args()
    n1 = L.gdn_chunk_fwd_workspace_size(ctypes.byref(f))
    assert n1 > 0
    bad = fwd_args(Dk=96)
    assert L.gdn_chunk_fwd_workspace_size(ctypes.byref(bad)) == 0
    b = B.BwdArgs()
    b.a = fwd_args().a
    assert L.gdn_chunk_bwd_workspace_size(ctypes.byref(b)) > n1


def test_backward_rejects_missing_gradients(L):
    b = B.BwdArgs()
    b.a = fwd_args().a
    b.do_ = FAKE
    assert L.gdn_chunk_bwd(ctypes.byref(b), None) == 1


def test_states_bytes(L):
    import numpy as np
    f = fwd_args()                                        # B=1, T=128, H=2, 128 x 128, bf16
    per = (128 * 128 + 2 * 64 * 128) * 2                  # state + U + U's bf16 residual per chunk and head
    assert L.gdn_chunk_states_bytes(ctypes.byref(f.a)) == 2 * 2 * per
    host = np.array([0, 1, 64, 65, 128], dtype=np.int32)  # lengths 1, 63, 1, 63: one chunk each
    f = fwd_args(cu_seqlens=FAKE, cu_seqlens_host=host.ctypes.data, num_seqs=4)
    assert L.gdn_chunk_states_bytes(ctypes.byref(f.a)) == (1 + 1 + 1 + 1) * 2 * per
    f = fwd_args(dtype=B.GDN_F32, Dk=64, Dv=64, T=129)
    assert L.gdn_chunk_states_bytes(ctypes.byref(f.a)) == 3 * 2 * (64 * 64 + 64 * 64) * 4
    assert L.gdn_chunk_states_bytes(ctypes.byref(fwd_args(Dk=96).a)) == 0


def test_saved_states_shrink_backward_workspace(L):
    b = B.BwdArgs()
    b.a = fwd_args().a
    full = L.gdn_chunk_bwd_workspace_size(ctypes.byref(b))
    b.h_saved = FAKE
    saved = L.gdn_chunk_bwd_workspace_size(ctypes.byref(b))
    assert full - saved >= 2 * 2 * 128 * 128 * 2


def test_misaligned_saved_states_rejected(L):
    f = fwd_args()
    f.h_save = FAKE + 8
    assert call_fwd(L, f) == 1
    f = fwd_args()
    f.t_save = FAKE + 8
    assert call_fwd(L, f) == 1


REC = 5 * 64 + 4   # floats of a chunk's scalar record


def test_t_bytes(L):
    f = fwd_args()                                        # B=1, T=128, H=2
    assert L.gdn_chunk_t_bytes(ctypes.byref(f.a)) == 2 * 2 * (64 * 64 + REC) * 4
    f = fwd_args(dtype=B.GDN_F32, Dk=64, Dv=64, T=129)
    assert L.gdn_chunk_t_bytes(ctypes.byref(f.a)) == 3 * 2 * (64 * 64 + REC) * 4
    assert L.gdn_chunk_t_bytes(ctypes.byref(fwd_args(Dk=96).a)) == 0


def test_saved_t_shrinks_workspaces(L):
    """Given chunk matrices T, neither pass keeps its own copy in the workspace."""
    b = B.BwdArgs()
    b.a = fwd_args().a
    full = L.gdn_chunk_bwd_workspace_size(ctypes.byref(b))
    b.t_saved = FAKE
    assert full - L.gdn_chunk_bwd_workspace_size(ctypes.byref(b)) >= 2 * 2 * 64 * 64 * 4
    f = fwd_args(T=4096)
    full = L.gdn_chunk_fwd_workspace_size(ctypes.byref(f))
    f.t_save = FAKE
    assert full - L.gdn_chunk_fwd_workspace_size(ctypes.byref(f)) >= 64 * 2 * (64 * 64 + REC) * 4


def dec_args(**kw):
    a = B.DecodeArgs()
    a.dtype, a.N, a.H, a.Dk, a.Dv = B.GDN_BF16, 4, 2, 128, 128
    a.q = a.k = a.v = a.g = a.beta = a.state = a.o = FAKE
    a.scale = 0.1
    a.num_slots = 4
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q", None, 1), ("state", None, 1), ("o", None, 1), ("H", 0, 1), ("N", -1, 1),
    ("Dk", 96, 2), ("Dv", 32, 2), ("dtype", 5, 2),
    ("state", FAKE + 4, 1), ("q", FAKE + 8, 1),
    ("num_slots", 3, 1),          # fewer slots than sequences without state_idx
])
def test_decode_rejects_bad_arguments(L, field, value, status):
    a = dec_args(**{field: value})
    assert L.gdn_decode_step(ctypes.byref(a), None) == status
    assert L.gdn_last_error()


def test_decode_empty_batch_is_a_no_op(L):
    a = dec_args(N=0, q=None, k=None, v=None, state=None, o=None)
    assert L.gdn_decode_step(ctypes.byref(a), None) == 0


def test_state_block_layout_is_a_permutation():
    """The saved-state block order (include/gdn.h) maps every (i, j) of a Dk x Dv
    state to its own offset below Dk * Dv, and unblock_states inverts it."""
    from tests.helpers import unblock_states
    for Dk, Dv in ((128, 128), (64, 128), (128, 64), (64, 64)):
        i, j = np.meshgrid(np.arange(Dk), np.arange(Dv), indexing="ij")
        off = ((i // 4) * (Dv // 16) + j // 16) * 64 + (i % 4) * 16 + j % 16
        assert np.array_equal(np.sort(off.ravel()), np.arange(Dk * Dv))
        h = np.random.default_rng(Dk + Dv).standard_normal((Dk, Dv))
        flat = np.empty(Dk * Dv)
        flat[off] = h
        assert np.array_equal(unblock_states(flat, 1, 1, Dk, Dv)[0, 0], h)


def test_noalloc_rejects_oversize_before_any_device_call(L):
    """gdn_chunk_fwd_noalloc refuses arguments whose workspace exceeds its
    scratch (GDN_NOALLOC_SCRATCH_BYTES) with GDN_E_WORKSPACE, and invalid ones
    like gdn_chunk_fwd, before touching a device (this runs with none)."""
    big = fwd_args(T=64 * 4096, H=16)                      # 65,536 chunk-heads: T alone needs 1.1 GiB
    big.a.workspace = None
    big.a.workspace_bytes = 0
    assert L.gdn_chunk_fwd_workspace_size(ctypes.byref(big)) > (64 << 20)
    assert L.gdn_chunk_fwd_noalloc(ctypes.byref(big), None) == 3
    assert b"scratch" in L.gdn_last_error()
    bad = fwd_args(Dk=96)
    assert L.gdn_chunk_fwd_noalloc(ctypes.byref(bad), None) == 2
    assert L.gdn_chunk_fwd_noalloc(None, None) == 1
