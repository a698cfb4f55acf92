"""The binding's own checks (device tensors; nothing is launched).

Every call below is rejected on the host, by the binding (dtype, shape,
contiguity, memory kind) or by the library's validation (aliasing, window
position), before any launch; the slab is left untouched.
"""
import pytest
import torch

import recurrent_state_quant_amd as lq
from recurrent_state_quant_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _tok(n, gate="gdn"):
    z = lambda *s: torch.zeros(s, device=DEV)  # noqa: E731
    return dict(q=z(n, 128), k=z(n, 128), v=z(n, 128), beta=z(n), alpha=z(n) if gate == "gdn" else z(n, 128))


def test_rejections_leave_the_slab_untouched():
    n, p, r = 5, 4, 2
    st = lq.LeapQuantState(n, p, r, "gdn", DEV)
    assert st.device.index is not None
    before = {k: getattr(st, k).clone() for k in st.boundary_keys + ("buf_gate", "buf_k", "buf_u")}
    tok = _tok(n)
    o = torch.empty((n, 128), device=DEV)
    args = [tok[x] for x in ("q", "k", "v", "beta", "alpha")]

    def bad(**kw):
        a = dict(zip(("q", "k", "v", "beta", "alpha"), args), o=o)
        a.update(kw)
        return [a[x] for x in ("q", "k", "v", "beta", "alpha", "o")]

    with pytest.raises(ValueError, match="float32"):
        lq.leapquant_decode_step(st, 0, *bad(q=tok["q"].double()))
    with pytest.raises(ValueError, match="shape"):
        lq.leapquant_decode_step(st, 0, *bad(k=torch.zeros((n, 64), device=DEV)))
    with pytest.raises(ValueError, match="contiguous"):
        lq.leapquant_decode_step(st, 0, *bad(v=torch.zeros((128, n), device=DEV).t()))
    with pytest.raises(ValueError, match="device memory"):
        lq.leapquant_decode_step(st, 0, *bad(o=torch.empty((n, 128))))
    with pytest.raises(ValueError, match="int32"):
        lq.leapquant_decode_step_slots(st, torch.zeros(n, dtype=torch.int64, device=DEV), *bad())
    with pytest.raises(TypeError):
        lq.leapquant_quantize_state(st, [[0.0]])
    # the library's checks, reached through the binding
    with pytest.raises(L.LeapQuantError) as e:
        lq.leapquant_decode_step(st, p, *bad())                 # t outside the window
    assert e.value.status == L.LQ_ERR_SHAPE
    with pytest.raises(L.LeapQuantError) as e:
        lq.leapquant_decode_step(st, 0, *bad(o=tok["q"]))       # o over an input
    assert e.value.status == L.LQ_ERR_ALIAS
    with pytest.raises(L.LeapQuantError) as e:
        lq.leapquant_window_close(st, 0)
    assert e.value.status == L.LQ_ERR_SHAPE
    torch.cuda.synchronize()
    for k, v in before.items():
        assert torch.equal(getattr(st, k), v), k
