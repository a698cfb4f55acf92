"""Python binding of the LeapQuant C ABI (argument marshalling only).

The functions carry the C names and forward to libleapquant.so; every step of
the decode path runs in the HIP kernels.  PyTorch provides device memory and
streams.  See include/leapquant.h for the semantics of each call.
"""
import ctypes

import torch

from . import _lib as L

_F32, _I32, _I8 = torch.float32, torch.int32, torch.int8


def _gate_id(gate):
    if gate in ("gdn", L.LQ_GATE_GDN):
        return L.LQ_GATE_GDN
    if gate in ("kda", L.LQ_GATE_KDA):
        return L.LQ_GATE_KDA
    raise ValueError(f"unknown gate {gate!r}")


def _ptr(x, dtype, shape, name, device=None):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, the state on {device}")
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(x.data_ptr()) if x.numel() else None


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the state on {device}")
    return ctypes.c_void_p(stream.cuda_stream)


def code_offsets(dk=128, dv=128):
    """Byte offset, inside one state's 16 KiB code block, of code (i, j), as
    an int64 array [dk][dv].  Codes are stored column-major in two 64-row
    halves: offset (i >> 6) * 8192 + j * 64 + slot(i & 63), where slot swaps
    the two 2-bit fields above the lowest two bits of i & 63."""
    if (dk, dv) != (128, 128):
        raise ValueError("the code layout is defined for dk = dv = 128")
    i = torch.arange(dk, dtype=torch.int64).view(dk, 1)
    j = torch.arange(dv, dtype=torch.int64).view(1, dv)
    x = i & 63
    slot = ((x & 0x0C) << 2) | ((x & 0x30) >> 2) | (x & 3)
    return (i >> 6) * 8192 + j * 64 + slot


_OFFSETS = {}


def _offsets(device):
    key = str(device)
    if key not in _OFFSETS:
        _OFFSETS[key] = code_offsets().reshape(-1).to(device)
    return _OFFSETS[key]


def codes_to_matrix(raw):
    """Stored codes [n][dk*dv] -> row-major int8 matrices [n][dk][dv]."""
    n = raw.shape[0]
    return raw.reshape(n, -1).index_select(1, _offsets(raw.device)).reshape(n, 128, 128)


def codes_from_matrix(mat):
    """Row-major int8 matrices [n][dk][dv] -> stored codes [n][dk*dv]."""
    n = mat.shape[0]
    out = torch.empty((n, 128 * 128), dtype=mat.dtype, device=mat.device)
    out[:, _offsets(mat.device)] = mat.reshape(n, -1)
    return out


class LeapQuantState:
    """Device arrays of one slab of n states: boundary state + window buffer.

    codes int8 [n][dk*dv] in the stored layout (see code_offsets);
    row_scale [n,dk]; col_scale [n,dv]; comp_idx int32 [n,r]; comp_val
    [n,r,dv]; buf_gate [n,p] (gdn) or [n,p,dk] (kda); buf_k [n,p,dk];
    buf_u [n,p,dv].  With LQ_DENSE_COMP in flags also comp_key [n,r,dk]
    (dense compensator keys, found by comp_iters rounds of subspace
    iteration at every split).
    """

    BOUNDARY = ("codes", "row_scale", "col_scale", "comp_idx", "comp_val")

    def __init__(self, n, p, r, gate="gdn", device="cuda", flags=0, dk=128, dv=128, comp_iters=0):
        self.n, self.p, self.r, self.dk, self.dv = int(n), int(p), int(r), int(dk), int(dv)
        self.gate = _gate_id(gate)
        self.flags = int(flags)
        self.comp_iters = int(comp_iters)
        dev = torch.device(device)
        self.device = dev
        self.codes = torch.zeros((n, dk * dv), dtype=_I8, device=dev)
        self.row_scale = torch.zeros((n, dk), dtype=_F32, device=dev)
        self.col_scale = torch.ones((n, dv), dtype=_F32, device=dev)
        self.comp_idx = torch.zeros((n, r), dtype=_I32, device=dev)
        self.comp_val = torch.zeros((n, r, dv), dtype=_F32, device=dev)
        gshape = (n, p) if self.gate == L.LQ_GATE_GDN else (n, p, dk)
        self.buf_gate = torch.zeros(gshape, dtype=_F32, device=dev)
        self.buf_k = torch.zeros((n, p, dk), dtype=_F32, device=dev)
        self.buf_u = torch.zeros((n, p, dv), dtype=_F32, device=dev)
        self.comp_key = torch.zeros((n, r, dk) if self.dense else (0,), dtype=_F32, device=dev)
        self.device = self.codes.device   # with its index resolved

    @property
    def dense(self):
        """Dense compensator keys (LQ_DENSE_COMP)."""
        return bool(self.flags & L.LQ_DENSE_COMP)

    @property
    def boundary_keys(self):
        """Names of the boundary-state arrays of this slab."""
        return self.BOUNDARY + (("comp_key",) if self.dense else ())

    def params(self):
        return L.LqParams(self.n, self.dk, self.dv, self.p, self.r, self.gate, self.flags,
                          self.comp_iters)

    def view(self, start, count):
        """States start .. start+count-1 of this slab as a slab of their own
        (views of the same memory).  Stacked layers kept in one allocation
        can be decoded layer by layer through views and closed together in
        one window-close call on the whole slab."""
        if not (0 <= start and count >= 1 and start + count <= self.n):
            raise ValueError("view out of range")
        v = object.__new__(LeapQuantState)
        v.n, v.p, v.r, v.dk, v.dv = int(count), self.p, self.r, self.dk, self.dv
        v.gate, v.flags, v.device, v.comp_iters = self.gate, self.flags, self.device, self.comp_iters
        for k in self.BOUNDARY + ("buf_gate", "buf_k", "buf_u"):
            setattr(v, k, getattr(self, k)[start:start + count])
        v.comp_key = self.comp_key[start:start + count] if self.dense else self.comp_key
        return v

    def ptrs(self):
        def vp(x):
            return x.data_ptr() if x.numel() else None
        return L.LqState(vp(self.codes), vp(self.row_scale), vp(self.col_scale),
                         vp(self.comp_idx), vp(self.comp_val), vp(self.buf_gate),
                         vp(self.buf_k), vp(self.buf_u), vp(self.comp_key))

    def _index(self, idx):
        if idx is None:
            return None
        return torch.as_tensor(idx, dtype=torch.long, device=self.device).reshape(-1)

    def boundary(self, idx=None):
        """Copy of the boundary state of all states (or of states idx), with
        the codes as row-major int8 matrices [m][dk][dv]."""
        ix = self._index(idx)
        out = {}
        for k in self.boundary_keys:
            x = getattr(self, k)
            x = x.clone() if ix is None else x.index_select(0, ix)
            out[k] = codes_to_matrix(x) if k == "codes" else x
        return out

    def snapshot(self):
        """The boundary state (the prefix-cache snapshot), as boundary()."""
        return self.boundary()

    def load_boundary(self, b, idx=None):
        """Write a boundary state (dict of tensors or arrays, codes as
        row-major matrices [m][dk][dv]) into all states or into states idx."""
        ix = self._index(idx)
        for k in self.boundary_keys:
            dst = getattr(self, k)
            src = torch.as_tensor(b[k]).to(device=dst.device, dtype=dst.dtype)
            if k == "codes":
                src = codes_from_matrix(src.reshape(-1, self.dk, self.dv))
            if ix is None:
                dst.copy_(src.reshape(dst.shape))
            else:
                dst[ix] = src.reshape((len(ix),) + tuple(dst.shape[1:]))


def leapquant_quantize_state(state, S, stream=None):
    n, dk, dv = state.n, state.dk, state.dv
    s = _ptr(S, _F32, (n, dk, dv), "S", state.device)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_quantize_state(ctypes.byref(prm), s, ctypes.byref(st),
                                                  _stream(stream, state.device)))


def leapquant_decode_step(state, t, q, k, v, beta, alpha, o, stream=None):
    args = _token_args(state, q, k, v, beta, alpha, o)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_decode_step(ctypes.byref(prm), ctypes.byref(st), int(t), *args,
                                               _stream(stream, state.device)))


def _token_args(state, q, k, v, beta, alpha, o):
    n, dk, dv = state.n, state.dk, state.dv
    ashape = (n,) if state.gate == L.LQ_GATE_GDN else (n, dk)
    d = state.device
    return [_ptr(q, _F32, (n, dk), "q", d), _ptr(k, _F32, (n, dk), "k", d), _ptr(v, _F32, (n, dv), "v", d),
            _ptr(beta, _F32, (n,), "beta", d), _ptr(alpha, _F32, ashape, "alpha", d),
            _ptr(o, _F32, (n, dv), "o", d)]


def leapquant_decode_close(state, t, q, k, v, beta, alpha, o, stream=None):
    args = _token_args(state, q, k, v, beta, alpha, o)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_decode_close(ctypes.byref(prm), ctypes.byref(st), int(t), *args,
                                                _stream(stream, state.device)))


def _slots_ptr(x, state, name):
    return _ptr(x, _I32, (state.n,), name, state.device)


def leapquant_decode_step_slots(state, pos, q, k, v, beta, alpha, o, stream=None):
    """Per-slot window positions pos (int32 [n] on the device); slots with
    pos outside [0, p) are idle."""
    args = _token_args(state, q, k, v, beta, alpha, o)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_decode_step_slots(ctypes.byref(prm), ctypes.byref(st),
                                                     _slots_ptr(pos, state, "pos"), *args,
                                                     _stream(stream, state.device)))


def leapquant_decode_close_slots(state, pos, q, k, v, beta, alpha, o, stream=None):
    args = _token_args(state, q, k, v, beta, alpha, o)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_decode_close_slots(ctypes.byref(prm), ctypes.byref(st),
                                                      _slots_ptr(pos, state, "pos"), *args,
                                                      _stream(stream, state.device)))


def leapquant_window_close_slots(state, lengths, stream=None):
    """Close slot s with lengths[s] records (int32 [n] on the device) when
    1 <= lengths[s] <= p; other slots are left as they are."""
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_window_close_slots(ctypes.byref(prm), ctypes.byref(st),
                                                      _slots_ptr(lengths, state, "lengths"),
                                                      _stream(stream, state.device)))


def _list_ptr(slots, state):
    if not isinstance(slots, torch.Tensor) or slots.dim() != 1:
        raise ValueError("slots must be a 1-D int32 tensor of slot ids")
    return _ptr(slots, _I32, (slots.numel(),), "slots", state.device), slots.numel()


def leapquant_decode_close_list(state, pos, slots, q, k, v, beta, alpha, o, stream=None):
    """Fused last-token decode and close of the listed slots only: slots is
    an int32 tensor of distinct slot ids on the device (one workgroup each);
    slot s works as in leapquant_decode_close_slots with pos[s]."""
    args = _token_args(state, q, k, v, beta, alpha, o)
    lp, count = _list_ptr(slots, state)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_decode_close_list(ctypes.byref(prm), ctypes.byref(st),
                                                     _slots_ptr(pos, state, "pos"), lp, int(count), *args,
                                                     _stream(stream, state.device)))


def leapquant_decode_step_close_list(state, pos, slots, q, k, v, beta, alpha, o, stream=None):
    """One continuous-batching token in one launch: slots at positions
    0 .. p-2 decode their token (as leapquant_decode_step_slots), listed
    slots at position p-1 decode their token and close their window (as
    leapquant_decode_close_list); slots is an int32 tensor of distinct slot
    ids on the device."""
    args = _token_args(state, q, k, v, beta, alpha, o)
    lp, count = _list_ptr(slots, state)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_decode_step_close_list(ctypes.byref(prm), ctypes.byref(st),
                                                          _slots_ptr(pos, state, "pos"), lp, int(count), *args,
                                                          _stream(stream, state.device)))


def leapquant_window_close_list(state, lengths, slots, stream=None):
    """Window close of the listed slots only (distinct int32 slot ids on
    the device); slot s is closed with lengths[s] records as in
    leapquant_window_close_slots."""
    lp, count = _list_ptr(slots, state)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_window_close_list(ctypes.byref(prm), ctypes.byref(st),
                                                     _slots_ptr(lengths, state, "lengths"), lp, int(count),
                                                     _stream(stream, state.device)))


def _bf16_ptr(state, B):
    return _ptr(B, torch.bfloat16, (state.n, state.dk, state.dv), "B", state.device)


def leapquant_bf16w_decode_step(state, B, t, q, k, v, beta, alpha, o, stream=None):
    """"BF16 + per-window": decode token t from the bf16 boundary state B
    [n, dk, dv] (torch.bfloat16) and the window buffer of `state` (its
    int8 boundary arrays are not used)."""
    args = _token_args(state, q, k, v, beta, alpha, o)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_bf16w_decode_step(ctypes.byref(prm), _bf16_ptr(state, B), ctypes.byref(st),
                                                     int(t), *args, _stream(stream, state.device)))


def leapquant_bf16w_window_close(state, B, length, stream=None):
    """"BF16 + per-window": B <- bf16(Gamma * B + K_w U) over `length`
    buffered records."""
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_bf16w_window_close(ctypes.byref(prm), _bf16_ptr(state, B), ctypes.byref(st),
                                                      int(length), _stream(stream, state.device)))


def leapquant_dense_step(S, gate, q, k, v, beta, alpha, o, stream=None, flags=0):
    """One token for dense states S [n][dk][dv] (float32, or bfloat16), in
    place; the uncompressed baseline of the quantized path.  flags may hold
    LQ_NO_DELTA."""
    if not isinstance(S, torch.Tensor) or S.dim() != 3:
        raise ValueError("S must be a [n, dk, dv] tensor")
    if S.dtype == torch.float32:
        dtype = L.LQ_DENSE_FP32
    elif S.dtype == torch.bfloat16:
        dtype = L.LQ_DENSE_BF16
    else:
        raise ValueError(f"S must be float32 or bfloat16, got {S.dtype}")
    n, dk, dv = S.shape
    sp = _ptr(S, S.dtype, (n, dk, dv), "S")
    g = _gate_id(gate)
    ashape = (n,) if g == L.LQ_GATE_GDN else (n, dk)
    d = S.device
    args = [_ptr(q, _F32, (n, dk), "q", d), _ptr(k, _F32, (n, dk), "k", d), _ptr(v, _F32, (n, dv), "v", d),
            _ptr(beta, _F32, (n,), "beta", d), _ptr(alpha, _F32, ashape, "alpha", d),
            _ptr(o, _F32, (n, dv), "o", d)]
    prm = L.LqParams(n, dk, dv, 1, 0, g, int(flags))
    with torch.cuda.device(S.device):
        L.check(L.load().leapquant_dense_step(ctypes.byref(prm), sp, dtype, *args, _stream(stream, S.device)))


def leapquant_stream_reference(src, read_bytes_per_wave, dst, write_bytes_per_wave, out, stream=None,
                               idle_sleeps=0):
    """Measurement reference: a plain stream in the decode step's launch
    shape, one wave per read_bytes_per_wave block of src (uint8, 16-byte
    aligned, a whole number of blocks), each wave then idling idle_sleeps x
    512 cycles and writing write_bytes_per_wave bytes of dst (uint8, waves *
    write_bytes_per_wave bytes; None when 0); out (int32 [waves, 64])
    receives a checksum per lane."""
    if not isinstance(src, torch.Tensor) or src.dtype != torch.uint8 or src.dim() != 1:
        raise ValueError("src must be a 1-d uint8 tensor")
    if read_bytes_per_wave <= 0 or src.numel() % read_bytes_per_wave:
        raise ValueError("src must hold a whole number of read_bytes_per_wave blocks")
    waves = src.numel() // read_bytes_per_wave
    d = src.device
    sp = _ptr(src, torch.uint8, (src.numel(),), "src", d)
    dp = None if write_bytes_per_wave == 0 else _ptr(dst, torch.uint8, (waves * write_bytes_per_wave,), "dst", d)
    op = _ptr(out, torch.int32, (waves, 64), "out", d)
    with torch.cuda.device(d):
        L.check(L.load().leapquant_stream_reference(sp, int(read_bytes_per_wave), dp, int(write_bytes_per_wave),
                                                    int(idle_sleeps), int(waves), op, _stream(stream, d)))


def leapquant_window_close(state, length, stream=None):
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_window_close(ctypes.byref(prm), ctypes.byref(st), int(length),
                                                _stream(stream, state.device)))


def leapquant_dequantize_state(state, S_out, stream=None):
    n, dk, dv = state.n, state.dk, state.dv
    s = _ptr(S_out, _F32, (n, dk, dv), "S_out", state.device)
    prm, st = state.params(), state.ptrs()
    with torch.cuda.device(state.device):
        L.check(L.load().leapquant_dequantize_state(ctypes.byref(prm), ctypes.byref(st), s,
                                                    _stream(stream, state.device)))


def leapquant_status_string(status):
    return L.load().leapquant_status_string(int(status)).decode()


def leapquant_abi_version():
    return L.load().leapquant_abi_version()
