"""C ABI checks that need no GPU: exported symbols and argument validation.

Every call here is rejected by the library's host-side validation before any
launch, so fake (never dereferenced) device addresses are safe to pass.
"""
import ctypes
import os
import re

import pytest

from recurrent_state_quant_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "leapquant.h")
FAKE = 0x7F0000000000  # 4 KiB aligned, never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(leapquant_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libleapquant.so not built (run __graft_entry__.build())")
    return L.load()


def test_exports_every_declared_symbol(lib):
    decl = _declared_functions()
    assert decl == sorted(L.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.leapquant_abi_version() == L.ABI_VERSION == 6
    for code in (L.LQ_OK, L.LQ_ERR_NULL, L.LQ_ERR_SHAPE, L.LQ_ERR_UNSUPPORTED, L.LQ_ERR_ALIGN,
                 L.LQ_ERR_ALIAS, L.LQ_ERR_HIP, 12345):
        assert lib.leapquant_status_string(code)


def _params(**kw):
    d = dict(n=4, dk=128, dv=128, p=16, r=4, gate=L.LQ_GATE_GDN, flags=0, comp_iters=0)
    d.update(kw)
    return L.LqParams(d["n"], d["dk"], d["dv"], d["p"], d["r"], d["gate"], d["flags"], d["comp_iters"])


def _state(**kw):
    n, p, r = 4, 16, 4
    base = FAKE
    sizes = dict(codes=n * 128 * 128, row_scale=n * 512, col_scale=n * 512, comp_idx=n * r * 4,
                 comp_val=n * r * 512, buf_gate=n * p * 512, buf_k=n * p * 512, buf_u=n * p * 512,
                 comp_key=n * r * 512)
    addrs = {}
    for name, sz in sizes.items():
        addrs[name] = base
        base += (sz + 4095) // 4096 * 4096
    addrs.update(kw)
    return L.LqState(*[addrs[f] for f, _ in L.LqState._fields_]), base


# both token entry points validate the same way
TOKEN_ENTRIES = ("leapquant_decode_step", "leapquant_decode_close")
_ENTRY = {"name": TOKEN_ENTRIES[0]}


@pytest.fixture(params=TOKEN_ENTRIES)
def entry(request):
    _ENTRY["name"] = request.param
    yield request.param
    _ENTRY["name"] = TOKEN_ENTRIES[0]


def _decode(lib, prm, st, t=0, **kw):
    _, base = _state()
    vec = 4 * 512
    a = dict(q=base, k=base + vec, v=base + 2 * vec, beta=base + 3 * vec, alpha=base + 3 * vec + 64,
             o=base + 4 * vec)
    a.update(kw)
    return getattr(lib, _ENTRY["name"])(ctypes.byref(prm) if prm is not None else None,
                                        ctypes.byref(st) if st is not None else None, t,
                                        a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["o"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=64), L.LQ_ERR_UNSUPPORTED), (dict(dv=256), L.LQ_ERR_UNSUPPORTED),
    (dict(n=0), L.LQ_ERR_SHAPE), (dict(p=0), L.LQ_ERR_SHAPE), (dict(p=65), L.LQ_ERR_SHAPE),
    (dict(r=-1), L.LQ_ERR_SHAPE), (dict(r=17), L.LQ_ERR_SHAPE), (dict(gate=2), L.LQ_ERR_SHAPE),
    (dict(flags=8), L.LQ_ERR_SHAPE), (dict(comp_iters=-1), L.LQ_ERR_SHAPE),
    (dict(comp_iters=9), L.LQ_ERR_SHAPE),
])
def test_bad_params(lib, entry, kw, code):
    st, _ = _state()
    prm = _params(**kw)
    assert _decode(lib, prm, st) == code
    assert lib.leapquant_window_close(ctypes.byref(prm), ctypes.byref(st), 16, None) == code
    assert lib.leapquant_quantize_state(ctypes.byref(prm), FAKE + (1 << 36), ctypes.byref(st), None) == code
    assert lib.leapquant_dequantize_state(ctypes.byref(prm), ctypes.byref(st), FAKE + (1 << 36), None) == code


def test_null_pointers(lib, entry):
    st, _ = _state()
    prm = _params()
    assert _decode(lib, None, st) == L.LQ_ERR_NULL
    assert _decode(lib, prm, None) == L.LQ_ERR_NULL
    for f in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_gate", "buf_k", "buf_u"):
        bad, _ = _state(**{f: 0})
        assert _decode(lib, prm, bad) == L.LQ_ERR_NULL, f
    for f in ("q", "k", "v", "beta", "alpha", "o"):
        assert _decode(lib, prm, st, **{f: 0}) == L.LQ_ERR_NULL, f
    assert lib.leapquant_quantize_state(ctypes.byref(prm), None, ctypes.byref(st), None) == L.LQ_ERR_NULL
    assert lib.leapquant_dequantize_state(ctypes.byref(prm), ctypes.byref(st), None, None) == L.LQ_ERR_NULL
    # buffer pointers are not needed by quantize/dequantize, compensators not at r = 0
    nobuf, _ = _state(buf_gate=0, buf_k=0, buf_u=0, comp_idx=0, comp_val=0)
    assert lib.leapquant_window_close(ctypes.byref(_params(r=0)), ctypes.byref(nobuf), 16, None) == L.LQ_ERR_NULL


def test_misaligned(lib, entry):
    prm = _params()
    for f in ("codes", "row_scale", "col_scale", "comp_val", "buf_k", "buf_u"):
        st, _ = _state()
        setattr(st, f, getattr(st, f) + 4)
        assert _decode(lib, prm, st) == L.LQ_ERR_ALIGN, f
    st, _ = _state()
    st.comp_idx = st.comp_idx + 2
    assert _decode(lib, prm, st) == L.LQ_ERR_ALIGN
    for f in ("q", "k", "v", "o"):
        _, base = _state()
        vec = 4 * 512
        addr = dict(q=base, k=base + vec, v=base + 2 * vec, o=base + 4 * vec)[f] + 4
        assert _decode(lib, prm, _state()[0], **{f: addr}) == L.LQ_ERR_ALIGN, f
    # KDA alpha is read as vectors: 16-byte alignment required; GDN alpha is scalar
    kda = _params(gate=L.LQ_GATE_KDA)
    _, base = _state()
    assert _decode(lib, kda, _state()[0], alpha=base + 3 * 2048 + 68) == L.LQ_ERR_ALIGN
    assert lib.leapquant_quantize_state(ctypes.byref(prm), FAKE + (1 << 36) + 8, ctypes.byref(_state()[0]), None) == L.LQ_ERR_ALIGN


def test_window_position_ranges(lib, entry):
    st, _ = _state()
    prm = _params()
    assert _decode(lib, prm, st, t=-1) == L.LQ_ERR_SHAPE
    assert _decode(lib, prm, st, t=16) == L.LQ_ERR_SHAPE
    assert lib.leapquant_window_close(ctypes.byref(prm), ctypes.byref(st), 0, None) == L.LQ_ERR_SHAPE
    assert lib.leapquant_window_close(ctypes.byref(prm), ctypes.byref(st), 17, None) == L.LQ_ERR_SHAPE


def test_aliasing_rejected(lib, entry):
    st, base = _state()
    prm = _params()
    assert _decode(lib, prm, st, o=base) == L.LQ_ERR_ALIAS            # o == q
    assert _decode(lib, prm, st, o=st.buf_u + 512) == L.LQ_ERR_ALIAS  # o inside the buffer
    assert lib.leapquant_quantize_state(ctypes.byref(prm), st.codes, ctypes.byref(st), None) == L.LQ_ERR_ALIAS
    assert lib.leapquant_dequantize_state(ctypes.byref(prm), ctypes.byref(st), st.row_scale, None) == L.LQ_ERR_ALIAS


def test_inputs_overlapping_the_state_rejected(lib, entry):
    """The token calls write records (decode) or the whole boundary (fused
    close) while they read their inputs: an input inside any state array is
    a race and is rejected before a launch."""
    st, _ = _state()
    prm = _params()
    assert _decode(lib, prm, st, k=st.buf_k) == L.LQ_ERR_ALIAS             # k over the records
    assert _decode(lib, prm, st, q=st.codes + 1024) == L.LQ_ERR_ALIAS      # q inside the codes
    assert _decode(lib, prm, st, v=st.buf_u + 2048) == L.LQ_ERR_ALIAS      # v inside the buffer
    assert _decode(lib, prm, st, beta=st.buf_gate + 8) == L.LQ_ERR_ALIAS   # beta inside the gates
    assert _decode(lib, prm, st, alpha=st.row_scale) == L.LQ_ERR_ALIAS     # alpha over the row scales
    assert _decode(lib, prm, st, q=st.comp_val + 16) == L.LQ_ERR_ALIAS     # q inside the compensators
    assert _decode(lib, prm, st, beta=st.comp_idx) == L.LQ_ERR_ALIAS       # beta over the row indices


def test_step_close_list_checks(lib):
    """The one-launch continuous-batching token validates like
    decode_close_list."""
    st, base = _state()
    prm = _params()
    vec = 4 * 512
    a = dict(q=base, k=base + vec, v=base + 2 * vec, beta=base + 3 * vec, alpha=base + 3 * vec + 64,
             o=base + 4 * vec)
    pos, lst = base + 5 * vec, base + 5 * vec + 64
    f = lib.leapquant_decode_step_close_list

    def call(pos_=pos, lst_=lst, count=2, **kw):
        x = dict(a, **kw)
        return f(ctypes.byref(prm), ctypes.byref(st), pos_, lst_, count, x["q"], x["k"], x["v"],
                 x["beta"], x["alpha"], x["o"], None)
    assert call(pos_=None) == L.LQ_ERR_NULL
    assert call(lst_=None) == L.LQ_ERR_NULL
    assert call(count=-1) == L.LQ_ERR_SHAPE and call(count=5) == L.LQ_ERR_SHAPE
    assert call(pos_=pos + 2) == L.LQ_ERR_ALIGN
    assert call(lst_=st.codes + 64) == L.LQ_ERR_ALIAS              # list inside the codes
    assert call(lst_=pos + 4) == L.LQ_ERR_ALIAS                    # list over the positions
    assert call(k=st.buf_k) == L.LQ_ERR_ALIAS                      # input over the records


def test_overlapping_state_arrays_rejected(lib, entry):
    """Every call that writes the state rejects a state whose own arrays
    overlap (the launch would read what it writes); arrays a call does not
    use are not looked at."""
    prm = _params()
    _, base = _state()
    pos = base + 5 * 2048
    lst = base + 6 * 2048
    for f, g in (("buf_k", "codes"), ("buf_u", "buf_k"), ("comp_val", "row_scale"), ("buf_gate", "col_scale"),
                 ("comp_idx", "comp_val")):
        st, _ = _state()
        setattr(st, f, getattr(st, g) + 256)
        what = f"{f} inside {g}"
        assert _decode(lib, prm, st) == L.LQ_ERR_ALIAS, what
        assert lib.leapquant_window_close(ctypes.byref(prm), ctypes.byref(st), 16, None) == L.LQ_ERR_ALIAS, what
        assert lib.leapquant_window_close_slots(ctypes.byref(prm), ctypes.byref(st), pos, None) == L.LQ_ERR_ALIAS, what
        assert lib.leapquant_window_close_list(ctypes.byref(prm), ctypes.byref(st), pos, lst, 1, None) == \
            L.LQ_ERR_ALIAS, what
    # quantize writes the boundary only: boundary arrays overlapping each
    # other are rejected, the (unused) buffer is not looked at
    st, _ = _state()
    st.row_scale = st.codes + 4096
    assert lib.leapquant_quantize_state(ctypes.byref(prm), FAKE + (1 << 36), ctypes.byref(st), None) == L.LQ_ERR_ALIAS
    st, _ = _state()
    st.buf_u = st.buf_k
    st.codes = st.codes + 8   # misaligned: the buffer overlap was not what failed
    assert lib.leapquant_quantize_state(ctypes.byref(prm), FAKE + (1 << 36), ctypes.byref(st), None) == L.LQ_ERR_ALIGN
    # the bf16 + per-window calls use only the buffer of the state
    B = FAKE + (1 << 37)
    st, _ = _state(codes=0, row_scale=0, col_scale=0, comp_idx=0, comp_val=0, comp_key=0)
    st.buf_u = st.buf_k + 512
    assert lib.leapquant_bf16w_window_close(ctypes.byref(prm), B, ctypes.byref(st), 16, None) == L.LQ_ERR_ALIAS
    dense = _params(flags=L.LQ_DENSE_COMP, comp_iters=1)
    st, _ = _state()
    st.comp_key = st.buf_gate
    assert _decode(lib, dense, st) == L.LQ_ERR_ALIAS


def test_dense_step_validation(lib):
    prm = _params()
    _, base = _state()
    vec = 4 * 512
    S = base + (1 << 30)
    a = dict(q=base, k=base + vec, v=base + 2 * vec, beta=base + 3 * vec, alpha=base + 3 * vec + 64,
             o=base + 4 * vec)

    def call(S_=S, dtype=L.LQ_DENSE_FP32, prm_=prm, **kw):
        x = dict(a, **kw)
        return lib.leapquant_dense_step(ctypes.byref(prm_), S_, dtype, x["q"], x["k"], x["v"],
                                        x["beta"], x["alpha"], x["o"], None)

    assert call(S_=None) == L.LQ_ERR_NULL
    assert call(o=0) == L.LQ_ERR_NULL
    assert call(dtype=7) == L.LQ_ERR_SHAPE
    assert call(prm_=_params(dk=64)) == L.LQ_ERR_UNSUPPORTED
    assert call(S_=S + 8) == L.LQ_ERR_ALIGN                       # fp32 state: 16 bytes
    assert call(S_=S + 4, dtype=L.LQ_DENSE_BF16) == L.LQ_ERR_ALIGN  # bf16 state: 8 bytes
    assert call(S_=base) == L.LQ_ERR_ALIAS                         # S over q
    assert call(o=S + 4096) == L.LQ_ERR_ALIAS                      # o inside S


def test_slot_entry_points_validation(lib):
    st, base = _state()
    prm = _params()
    vec = 4 * 512
    a = dict(q=base, k=base + vec, v=base + 2 * vec, beta=base + 3 * vec, alpha=base + 3 * vec + 64,
             o=base + 4 * vec)
    pos = base + 5 * vec
    for name in ("leapquant_decode_step_slots", "leapquant_decode_close_slots"):
        f = getattr(lib, name)

        def call(p_=pos, prm_=prm, **kw):
            x = dict(a, **kw)
            return f(ctypes.byref(prm_), ctypes.byref(st), p_, x["q"], x["k"], x["v"], x["beta"],
                     x["alpha"], x["o"], None)
        assert call(p_=None) == L.LQ_ERR_NULL, name
        assert call(p_=pos + 2) == L.LQ_ERR_ALIGN, name
        assert call(p_=st.buf_u + 64) == L.LQ_ERR_ALIAS, name       # positions inside the buffer
        assert call(p_=a["o"]) == L.LQ_ERR_ALIAS, name              # positions over the output
        assert call(prm_=_params(p=0)) == L.LQ_ERR_SHAPE, name
        assert call(o=0) == L.LQ_ERR_NULL, name
    f = lib.leapquant_window_close_slots
    assert f(ctypes.byref(prm), ctypes.byref(st), None, None) == L.LQ_ERR_NULL
    assert f(ctypes.byref(prm), ctypes.byref(st), pos + 1, None) == L.LQ_ERR_ALIGN
    assert f(ctypes.byref(prm), ctypes.byref(st), st.codes + 128, None) == L.LQ_ERR_ALIAS


def test_list_entry_points_validation(lib):
    """Compacted closes: count in [0, n], the list non-NULL, 4-byte aligned
    and clear of the state, the outputs and the per-slot array; count == 0
    is accepted and launches nothing.  Every other call here fails its
    checks, so nothing is launched on these host addresses."""
    st, base = _state()
    prm = _params()
    vec = 4 * 512
    a = dict(q=base, k=base + vec, v=base + 2 * vec, beta=base + 3 * vec, alpha=base + 3 * vec + 64,
             o=base + 4 * vec)
    pos = base + 5 * vec
    lst = base + 6 * vec
    f = lib.leapquant_decode_close_list

    def call(l_=lst, count=2, p_=pos, **kw):
        x = dict(a, **kw)
        return f(ctypes.byref(prm), ctypes.byref(st), p_, l_, count, x["q"], x["k"], x["v"], x["beta"],
                 x["alpha"], x["o"], None)
    assert call(count=-1) == L.LQ_ERR_SHAPE
    assert call(count=5) == L.LQ_ERR_SHAPE                       # more entries than slots
    assert call(l_=None) == L.LQ_ERR_NULL
    assert call(l_=lst + 2) == L.LQ_ERR_ALIGN
    assert call(l_=st.codes + 64) == L.LQ_ERR_ALIAS              # list inside the codes
    assert call(l_=pos + 4) == L.LQ_ERR_ALIAS                    # list over the positions
    assert call(l_=a["o"]) == L.LQ_ERR_ALIAS                     # list over the output
    assert call(p_=None) == L.LQ_ERR_NULL
    assert call(o=0) == L.LQ_ERR_NULL
    assert call(l_=None, count=0) == L.LQ_OK                     # nothing to do: no launch
    g = lib.leapquant_window_close_list
    assert g(ctypes.byref(prm), ctypes.byref(st), pos, lst, -1, None) == L.LQ_ERR_SHAPE
    assert g(ctypes.byref(prm), ctypes.byref(st), pos, lst, 5, None) == L.LQ_ERR_SHAPE
    assert g(ctypes.byref(prm), ctypes.byref(st), pos, None, 1, None) == L.LQ_ERR_NULL
    assert g(ctypes.byref(prm), ctypes.byref(st), pos, lst + 1, 1, None) == L.LQ_ERR_ALIGN
    assert g(ctypes.byref(prm), ctypes.byref(st), pos, st.buf_k + 8, 1, None) == L.LQ_ERR_ALIAS
    assert g(ctypes.byref(prm), ctypes.byref(st), None, lst, 1, None) == L.LQ_ERR_NULL
    assert g(ctypes.byref(prm), ctypes.byref(st), pos, None, 0, None) == L.LQ_OK


def test_dense_compensator_validation(lib, entry):
    """LQ_DENSE_COMP needs comp_key (16-byte aligned) when r > 0; without the
    flag, or at r = 0, comp_key is not looked at."""
    dense = _params(flags=L.LQ_DENSE_COMP, comp_iters=2)
    st, _ = _state(comp_key=0)
    assert _decode(lib, dense, st) == L.LQ_ERR_NULL
    assert lib.leapquant_window_close(ctypes.byref(dense), ctypes.byref(st), 16, None) == L.LQ_ERR_NULL
    assert lib.leapquant_quantize_state(ctypes.byref(dense), FAKE + (1 << 36), ctypes.byref(st), None) == L.LQ_ERR_NULL
    assert lib.leapquant_dequantize_state(ctypes.byref(dense), ctypes.byref(st), FAKE + (1 << 36), None) == L.LQ_ERR_NULL
    st, _ = _state()
    st.comp_key = st.comp_key + 8
    assert _decode(lib, dense, st) == L.LQ_ERR_ALIGN
    # an output over the keys
    st, _ = _state()
    assert _decode(lib, dense, st, o=st.comp_key) == L.LQ_ERR_ALIAS
    assert lib.leapquant_quantize_state(ctypes.byref(dense), st.comp_key, ctypes.byref(st), None) == L.LQ_ERR_ALIAS
    assert lib.leapquant_dequantize_state(ctypes.byref(dense), ctypes.byref(st), st.comp_key, None) == L.LQ_ERR_ALIAS
    # the same pointers are fine without the flag or at r = 0 (nothing is launched here:
    # only argument errors are checked, so stop at the first call that would launch)
    nokey, _ = _state(comp_key=0)
    r0 = _params(flags=L.LQ_DENSE_COMP, r=0)
    assert lib.leapquant_dequantize_state(ctypes.byref(r0), ctypes.byref(nokey), 0, None) == L.LQ_ERR_NULL


def test_bf16_window_validation(lib):
    """"BF16 + per-window": B must be given, 16-byte aligned and apart from
    the buffer; only LQ_NO_DELTA applies; t and len ranges as for the int8
    entry points."""
    st, base = _state()
    prm = _params()
    vec = 4 * 512
    B = base + (1 << 30)
    a = dict(q=base, k=base + vec, v=base + 2 * vec, beta=base + 3 * vec, alpha=base + 3 * vec + 64,
             o=base + 4 * vec)

    def dec(B_=B, prm_=prm, t=0, **kw):
        x = dict(a, **kw)
        return lib.leapquant_bf16w_decode_step(ctypes.byref(prm_), B_, ctypes.byref(st), t, x["q"], x["k"],
                                               x["v"], x["beta"], x["alpha"], x["o"], None)

    def close(B_=B, prm_=prm, n_=16):
        return lib.leapquant_bf16w_window_close(ctypes.byref(prm_), B_, ctypes.byref(st), n_, None)

    assert dec(B_=None) == L.LQ_ERR_NULL and close(B_=None) == L.LQ_ERR_NULL
    assert dec(B_=B + 8) == L.LQ_ERR_ALIGN and close(B_=B + 8) == L.LQ_ERR_ALIGN
    assert dec(B_=st.buf_k) == L.LQ_ERR_ALIAS and close(B_=st.buf_u) == L.LQ_ERR_ALIAS
    assert dec(o=B + 4096) == L.LQ_ERR_ALIAS
    assert dec(prm_=_params(flags=L.LQ_NO_SMOOTH)) == L.LQ_ERR_SHAPE
    assert dec(prm_=_params(flags=L.LQ_DENSE_COMP)) == L.LQ_ERR_SHAPE
    assert dec(t=-1) == L.LQ_ERR_SHAPE and dec(t=16) == L.LQ_ERR_SHAPE
    assert close(n_=0) == L.LQ_ERR_SHAPE and close(n_=17) == L.LQ_ERR_SHAPE
    assert dec(q=0) == L.LQ_ERR_NULL
    assert close(prm_=_params(dk=64)) == L.LQ_ERR_UNSUPPORTED


def test_stream_reference_validation(lib):
    """The stream reference: read blocks a multiple of 1 KiB, written blocks
    a multiple of 512 bytes, idle sleeps in [0, 4096], at least one wave,
    aligned pointers, outputs outside the bytes read and apart from each
    other."""
    f = lib.leapquant_stream_reference
    src, dst, out = FAKE, FAKE + (1 << 24), FAKE + (1 << 25)

    def call(s_=src, rb=1024, d_=dst, wb=512, idle=0, waves=4, o_=out):
        return f(s_, rb, d_, wb, idle, waves, o_, None)
    assert call(s_=None) == L.LQ_ERR_NULL
    assert call(o_=None) == L.LQ_ERR_NULL
    assert call(d_=None) == L.LQ_ERR_NULL
    for kw in (dict(rb=0), dict(rb=1000), dict(rb=1536), dict(rb=(1 << 30) + 1024, waves=1), dict(waves=0),
               dict(waves=-1), dict(wb=256), dict(wb=-512), dict(wb=(1 << 30) + 512, waves=1), dict(idle=-1),
               dict(idle=4097)):
        assert call(**kw) == L.LQ_ERR_SHAPE, kw
    assert call(s_=src + 8) == L.LQ_ERR_ALIGN
    assert call(d_=dst + 8) == L.LQ_ERR_ALIGN
    assert call(o_=out + 2) == L.LQ_ERR_ALIGN
    assert call(o_=src + 4096 - 4) == L.LQ_ERR_ALIAS        # checksums over the last block
    assert call(o_=src - 4 * 64 * 4 + 4) == L.LQ_ERR_ALIAS  # ... ending inside the first
    assert call(d_=src + 1024) == L.LQ_ERR_ALIAS            # writes over the reads
    assert call(d_=out - 16) == L.LQ_ERR_ALIAS              # writes over the checksums
