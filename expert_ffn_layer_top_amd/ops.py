"""Torch-facing wrappers of the C ABI: argument marshalling only.

Each function checks dtype, contiguity and every size the library's kernels index (across all
of its tensors: a mismatch raises ValueError here, on the host, instead of becoming an
out-of-range device access), then the device, allocates the outputs (and any workspace) with
torch on the input's device, and passes raw pointers plus the current HIP stream to the library.
All arithmetic happens in the library's kernels; nothing here computes.

Tensor conventions: bf16 tensors are torch.bfloat16; E4M3 elements and E8M0 scales are
torch.uint8 bytes; indices are torch.int32; gates and logits are torch.float32.
"""

import torch

from ._lib import call, lib

BF16, MXFP8 = 0, 1


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(t, dtype, name, shape=None, ndim=None):
    """dtype, contiguity and shape (a tuple of ints, None entries free) of one argument."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name}: expected shape {want}, got {list(t.shape)}")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts):
    """Every tensor argument on the same GPU (checked after the shapes)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("expected GPU tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _mx_pad_cap(n, E):
    # moe_mx_pad_cap: n + 128 E rounded up to a multiple of 128 (the library's padded token axis,
    # long enough for any pad up to 128)
    return (n + 128 * E + 127) // 128 * 128


# ---------------------------------------------------------------- router

def router_project(x, w_r):
    """logits [T,E] fp32 = x [T,d] bf16 @ w_r [d,E] fp32."""
    _check(x, torch.bfloat16, "x", ndim=2)
    T, d = x.shape
    _check(w_r, torch.float32, "w_r", (d, None))
    E = w_r.shape[1]
    _on_gpu(x, w_r)
    logits = _empty((T, E), torch.float32, x)
    call("moe_router_project", _ptr(x), _ptr(w_r), T, d, E, _ptr(logits), _stream(x))
    return logits


def router_project_bwd(x, w_r, d_logits, want_dx=True, want_dw=True):
    """(dx_router [T,d] fp32 or None, dw_r [d,E] fp32 or None)."""
    _check(x, torch.bfloat16, "x", ndim=2)
    T, d = x.shape
    _check(w_r, torch.float32, "w_r", (d, None))
    E = w_r.shape[1]
    _check(d_logits, torch.float32, "d_logits", (T, E))
    _on_gpu(x, w_r, d_logits)
    dx = _empty((T, d), torch.float32, x) if want_dx else None
    dw = _empty((d, E), torch.float32, x) if want_dw else None
    nbytes = lib.moe_router_bwd_workspace_bytes(T, d, E) if (want_dx or want_dw) else 0
    ws = _empty((max(nbytes, 1),), torch.uint8, x)
    call("moe_router_project_bwd", _ptr(x), _ptr(w_r), _ptr(d_logits), T, d, E, _ptr(dx), _ptr(dw),
         _ptr(ws), nbytes, _stream(x))
    return dx, dw


def route_topk(logits, k, want_probs=False, pad=None, want_row_token=True):
    """Router top-k + routing metadata.  Returns a dict with topk_idx, topk_gate, probs (or None),
    counts, offsets, offsets_pad (or None), dest, row_token (or None)."""
    _check(logits, torch.float32, "logits", ndim=2)
    T, E = logits.shape
    _need(pad is None or pad >= 1, "pad must be >= 1")
    _on_gpu(logits)
    out = dict(
        topk_idx=_empty((T, k), torch.int32, logits),
        topk_gate=_empty((T, k), torch.float32, logits),
        probs=_empty((T, E), torch.float32, logits) if want_probs else None,
        counts=_empty((E,), torch.int32, logits),
        offsets=_empty((E + 1,), torch.int32, logits),
        offsets_pad=_empty((E + 1,), torch.int32, logits) if pad else None,
        dest=_empty((T, k), torch.int32, logits),
        row_token=_empty((T * k,), torch.int32, logits) if want_row_token else None,
    )
    nbytes = lib.moe_route_workspace_bytes(T, E, k)
    ws = _empty((max(nbytes, 1),), torch.uint8, logits)
    call("moe_route_topk", _ptr(logits), T, E, k, _ptr(out["topk_idx"]), _ptr(out["topk_gate"]),
         _ptr(out["probs"]), _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["offsets_pad"]),
         int(pad or 0), _ptr(out["dest"]), _ptr(out["row_token"]), _ptr(ws), nbytes, _stream(logits))
    return out


def route_topk_bwd(topk_gate, topk_idx, d_gate, E, balance=None):
    """d_logits [T,E] fp32.  balance = (probs [T,E] fp32, counts [E] int32, weight): also the
    gradient of weight * the balance score (route_balance), counts held fixed."""
    _check(topk_idx, torch.int32, "topk_idx", ndim=2)
    T, k = topk_idx.shape
    _check(topk_gate, torch.float32, "topk_gate", (T, k))
    _check(d_gate, torch.float32, "d_gate", (T, k))
    if balance is not None:
        probs, counts, weight = balance
        _check(probs, torch.float32, "probs", (T, E))
        _check(counts, torch.int32, "counts", (E,))
        _on_gpu(topk_gate, topk_idx, d_gate, probs, counts)
    else:
        _on_gpu(topk_gate, topk_idx, d_gate)
    dl = _empty((T, E), torch.float32, topk_gate)
    if balance is None:
        call("moe_route_topk_bwd", _ptr(topk_gate), _ptr(topk_idx), _ptr(d_gate), T, E, k, _ptr(dl),
             _stream(topk_gate))
    else:
        call("moe_route_topk_bwd_balance", _ptr(topk_gate), _ptr(topk_idx), _ptr(d_gate), _ptr(probs),
             _ptr(counts), float(weight), T, E, k, _ptr(dl), _stream(topk_gate))
    return dl


def route_balance(probs, counts, k):
    """(p_mean [E] fp32, stats [4] fp32 = aux, load_max, prob_max, load_cv), on the device."""
    _check(probs, torch.float32, "probs", ndim=2)
    T, E = probs.shape
    _check(counts, torch.int32, "counts", (E,))
    _on_gpu(probs, counts)
    p_mean = _empty((E,), torch.float32, probs)
    stats = _empty((4,), torch.float32, probs)
    nbytes = lib.moe_route_balance_workspace_bytes(T, E)
    ws = _empty((max(nbytes, 1),), torch.uint8, probs)
    call("moe_route_balance", _ptr(probs), _ptr(counts), T, E, k, _ptr(p_mean), _ptr(stats), _ptr(ws), nbytes,
         _stream(probs))
    return p_mean, stats


# ---------------------------------------------------------------- rows

def permute(x, dest, x_scale=None):
    """xp [n,d] (bf16, or E4M3 bytes + xp_scale when x_scale is given)."""
    _check(dest, torch.int32, "dest", ndim=2)
    T, k = dest.shape
    if x_scale is None:
        _check(x, torch.bfloat16, "x", (T, None))
        _on_gpu(x, dest)
        xp = _empty((T * k, x.shape[1]), torch.bfloat16, x)
        call("moe_permute", BF16, _ptr(x), None, _ptr(dest), T, x.shape[1], k, _ptr(xp), None, _stream(x))
        return xp
    _check(x, torch.uint8, "x", (T, None))
    d = x.shape[1]
    _need(d % 32 == 0, f"x: d = {d} must be a multiple of 32 (one scale per 32 elements)")
    _check(x_scale, torch.uint8, "x_scale", (T, d // 32))
    _on_gpu(x, x_scale, dest)
    xp = _empty((T * k, d), torch.uint8, x)
    xps = _empty((T * k, d // 32), torch.uint8, x)
    call("moe_permute", MXFP8, _ptr(x), _ptr(x_scale), _ptr(dest), T, d, k, _ptr(xp), _ptr(xps), _stream(x))
    return xp, xps


def permute_quant_mx(x, dest):
    """(xpq [n,d] E4M3, xps [n,d/32] E8M0): the row blocks of bf16 x permuted into the expert
    buffers, as mxfp8_quantize(x, 0) followed by permute(.., x_scale=..), in one pass, with xps
    in the GEMM scale layout (bytes rearranged) for the gate/up product."""
    _check(dest, torch.int32, "dest", ndim=2)
    T, k = dest.shape
    _check(x, torch.bfloat16, "x", (T, None))
    _on_gpu(x, dest)
    d = x.shape[1]
    xpq = _empty((T * k, d), torch.uint8, x)
    xps = _empty((T * k, d // 32), torch.uint8, x)
    call("moe_permute_quant_mx", _ptr(x), _ptr(dest), T, d, k, _ptr(xpq), _ptr(xps), _stream(x))
    return xpq, xps


def unpermute_combine(yexp, topk_gate, dest):
    _check(dest, torch.int32, "dest", ndim=2)
    T, k = dest.shape
    _check(yexp, torch.bfloat16, "yexp", (T * k, None))
    _check(topk_gate, torch.float32, "topk_gate", (T, k))
    _on_gpu(yexp, topk_gate, dest)
    d = yexp.shape[1]
    y = _empty((T, d), torch.bfloat16, yexp)
    call("moe_unpermute_combine", _ptr(yexp), _ptr(topk_gate), _ptr(dest), T, d, k, _ptr(y), _stream(yexp))
    return y


def _combine_bwd_args(dy, yexp, topk_gate, dest):
    _check(dest, torch.int32, "dest", ndim=2)
    T, k = dest.shape
    _check(dy, torch.bfloat16, "dy", (T, None))
    d = dy.shape[1]
    _check(yexp, torch.bfloat16, "yexp", (T * k, d))
    _check(topk_gate, torch.float32, "topk_gate", (T, k))
    _on_gpu(dy, yexp, topk_gate, dest)
    return T, d, k


def unpermute_combine_bwd(dy, yexp, topk_gate, dest):
    """(dyexp [n,d] bf16, d_gate [T,k] fp32)."""
    T, d, k = _combine_bwd_args(dy, yexp, topk_gate, dest)
    dyexp = _empty((T * k, d), torch.bfloat16, dy)
    dgate = _empty((T, k), torch.float32, dy)
    call("moe_unpermute_combine_bwd", _ptr(dy), _ptr(yexp), _ptr(topk_gate), _ptr(dest), T, d, k,
         _ptr(dyexp), _ptr(dgate), _stream(dy))
    return dyexp, dgate


def unpermute_combine_bwd_mx(dy, yexp, topk_gate, dest):
    """(dyq [n,d] E4M3, dys [n,d/32] E8M0, row_gate [n] fp32, d_gate [T,k] fp32): the combine
    backward with dyexp emitted only as MXFP8 row blocks (the bf16 rows are never written); dys
    in the GEMM scale layout (bytes rearranged) for the down dgrad."""
    T, d, k = _combine_bwd_args(dy, yexp, topk_gate, dest)
    _need(d % 32 == 0, f"dy: d = {d} must be a multiple of 32")
    n = T * k
    dyq = _empty((n, d), torch.uint8, dy)
    dys = _empty((n, d // 32), torch.uint8, dy)
    row_gate = _empty((n,), torch.float32, dy)
    dgate = _empty((T, k), torch.float32, dy)
    call("moe_unpermute_combine_bwd_mx", _ptr(dy), _ptr(yexp), _ptr(topk_gate), _ptr(dest), T, d, k, _ptr(dyq),
         _ptr(dys), _ptr(row_gate), _ptr(dgate), _stream(dy))
    return dyq, dys, row_gate, dgate


def permute_bwd(dxp, dest, addend=None):
    _check(dest, torch.int32, "dest", ndim=2)
    T, k = dest.shape
    _check(dxp, torch.bfloat16, "dxp", (T * k, None))
    d = dxp.shape[1]
    if addend is not None:
        _check(addend, torch.float32, "addend", (T, d))
    _on_gpu(dxp, dest, addend)
    dx = _empty((T, d), torch.bfloat16, dxp)
    call("moe_permute_bwd", _ptr(dxp), _ptr(dest), T, d, k, _ptr(addend), _ptr(dx), _stream(dxp))
    return dx


def permute_bwd_router(dxp, dest, w_r, d_logits):
    """dx [T,d] bf16 = permute_bwd(dxp, dest, addend=router_project_bwd(x, w_r, d_logits)[0]) in
    one kernel, byte for byte."""
    _check(dest, torch.int32, "dest", ndim=2)
    T, k = dest.shape
    _check(dxp, torch.bfloat16, "dxp", (T * k, None))
    d = dxp.shape[1]
    _check(w_r, torch.float32, "w_r", (d, None))
    E = w_r.shape[1]
    _check(d_logits, torch.float32, "d_logits", (T, E))
    _on_gpu(dxp, dest, w_r, d_logits)
    dx = _empty((T, d), torch.bfloat16, dxp)
    nbytes = lib.moe_router_bwd_workspace_bytes(T, d, E)
    ws = _empty((max(nbytes, 1),), torch.uint8, dxp)
    call("moe_permute_bwd_router", _ptr(dxp), _ptr(dest), T, d, k, _ptr(w_r), _ptr(d_logits), E, _ptr(dx),
         _ptr(ws), nbytes, _stream(dxp))
    return dx


# ---------------------------------------------------------------- MXFP8

def _rc(x):
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x.shape
    raise ValueError("x must be 2-D or 3-D")


def mxfp8_quantize(x, axis, scale_mode=0):
    """x [..., R, C] bf16 (2-D or 3-D).  axis 0: blocks along C, outputs in x's layout;
    axis 1: blocks along R, outputs transposed to [..., C, R].  scale_mode 0: the MX floor rule;
    1: the smallest power-of-two scale under which no element saturates."""
    _check(x, torch.bfloat16, "x")
    batch, R, C = _rc(x)
    _need(axis in (0, 1), "axis must be 0 or 1")
    _need(scale_mode in (0, 1), "scale_mode must be 0 or 1")
    _need((C if axis == 0 else R) % 32 == 0, "the blocked dimension must be a multiple of 32")
    _on_gpu(x)
    lead = x.shape[:-2]
    if axis == 0:
        q = _empty((*lead, R, C), torch.uint8, x)
        s = _empty((*lead, R, C // 32), torch.uint8, x)
    else:
        q = _empty((*lead, C, R), torch.uint8, x)
        s = _empty((*lead, C, R // 32), torch.uint8, x)
    call("mxfp8_quantize", _ptr(x), batch, R, C, axis, scale_mode, _ptr(q), _ptr(s), _stream(x))
    return q, s


def mxfp8_quantize_both(x):
    """x [..., R, C] bf16 (2-D or 3-D) -> (q, s) as mxfp8_quantize(x, 0) and (qT, sT) as
    mxfp8_quantize(x, 1), from one read of x; s and sT in the GEMM scale layout of each matrix
    (shapes as the row-major scales, bytes rearranged): the weights' operands of the products."""
    _check(x, torch.bfloat16, "x")
    batch, R, C = _rc(x)
    _need(R % 32 == 0 and C % 64 == 0, "need rows % 32 == 0 and cols % 64 == 0")
    _on_gpu(x)
    lead = x.shape[:-2]
    q = _empty((*lead, R, C), torch.uint8, x)
    s = _empty((*lead, R, C // 32), torch.uint8, x)
    qT = _empty((*lead, C, R), torch.uint8, x)
    sT = _empty((*lead, C, R // 32), torch.uint8, x)
    call("mxfp8_quantize_both", _ptr(x), batch, R, C, _ptr(q), _ptr(s), _ptr(qT), _ptr(sT), _stream(x))
    return q, s, qT, sT


def mx_pad_cap(n, E):
    return lib.moe_mx_pad_cap(n, E)


def mxfp8_quantize_grouped(x, offsets, offsets_pad, n, row_token=None, row_gate=None):
    """Token-axis blocks per expert group: (qT [C, P], sT [P/32, C]), P = mx_pad_cap(n, E); the
    scales are block-major (sT[b, c]: channel c, position block b).  row_token: rows gathered
    from a token-major x; row_gate [n] (with row_token): row r is bf16(row_gate[r] * x[row_token[r]])."""
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    _need(E >= 1, "offsets must hold E + 1 >= 2 entries")
    _check(offsets_pad, torch.int32, "offsets_pad", (E + 1,))
    if row_token is None:
        _check(x, torch.bfloat16, "x", (n, None))
    else:
        _check(x, torch.bfloat16, "x", ndim=2)
        _check(row_token, torch.int32, "row_token", (n,))
    if row_gate is not None:
        _need(row_token is not None, "row_gate needs row_token")
        _check(row_gate, torch.float32, "row_gate", (n,))
    C = x.shape[1]
    _on_gpu(x, offsets, offsets_pad, row_token, row_gate)
    P = mx_pad_cap(n, E)
    q = _empty((C, P), torch.uint8, x)
    s = _empty((P // 32, C), torch.uint8, x)
    if row_gate is None:
        call("mxfp8_quantize_grouped", _ptr(x), _ptr(row_token), _ptr(offsets), _ptr(offsets_pad), E, n, C,
             _ptr(q), _ptr(s), _stream(x))
    else:
        call("mxfp8_quantize_grouped_gated", _ptr(x), _ptr(row_token), _ptr(row_gate), _ptr(offsets),
             _ptr(offsets_pad), E, n, C, _ptr(q), _ptr(s), _stream(x))
    return q, s


def mxfp8_quantize_gemm(x):
    """Row blocks of x [..., R, C] bf16 as mxfp8_quantize(x, 0): (q [..., R, C], s) with s the
    scales in the GEMM scale layout of each [R, C] matrix (shaped [..., R, C/32] like the row-major
    scales, bytes rearranged): an operand of the MXFP8 forward and dgrad grouped GEMMs."""
    _check(x, torch.bfloat16, "x")
    _need(x.dim() >= 2, "x must have at least 2 dims")
    R, C = x.shape[-2], x.shape[-1]
    _need(C % 32 == 0, f"x: C = {C} must be a multiple of 32")
    batch = x.numel() // (R * C)
    _on_gpu(x)
    q = _empty(tuple(x.shape), torch.uint8, x)
    s = _empty(tuple(x.shape[:-1]) + (C // 32,), torch.uint8, x)
    call("mxfp8_quantize_gemm", _ptr(x), batch, R, C, _ptr(q), _ptr(s), _stream(x))
    return q, s


def mxfp8_scales_to_gemm(s, K):
    """Row-major E8M0 scales [..., R, K/32] rearranged into the GEMM scale layout of each [R, K]
    matrix (same shape, bytes rearranged)."""
    _check(s, torch.uint8, "s")
    _need(s.dim() >= 2 and K % 32 == 0 and s.shape[-1] == K // 32, "s must be [..., R, K/32]")
    R = s.shape[-2]
    batch = s.numel() // (R * (K // 32))
    _on_gpu(s)
    out = _empty(tuple(s.shape), torch.uint8, s)
    call("mxfp8_scales_to_gemm", _ptr(s), batch, R, K, _ptr(out), _stream(s))
    return out


def mxfp8_quantize_rows_grouped(x, offsets, offsets_pad):
    """Both MXFP8 layouts of a grouped [n, C] bf16 tensor from one read: (q [n, C], s [n, C/32])
    row blocks as mxfp8_quantize(x, 0) with s in the GEMM scale layout (bytes rearranged), and
    (qT [C, P], sT [P/32, C]) grouped token blocks as mxfp8_quantize_grouped(x, offsets,
    offsets_pad, n)."""
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    _need(E >= 1, "offsets must hold E + 1 >= 2 entries")
    _check(offsets_pad, torch.int32, "offsets_pad", (E + 1,))
    _check(x, torch.bfloat16, "x", ndim=2)
    n, C = x.shape
    _need(C % 64 == 0, "C must be a multiple of 64")
    _on_gpu(x, offsets, offsets_pad)
    P = mx_pad_cap(n, E)
    q = _empty((n, C), torch.uint8, x)
    s = _empty((n, C // 32), torch.uint8, x)
    qT = _empty((C, P), torch.uint8, x)
    sT = _empty((P // 32, C), torch.uint8, x)
    call("mxfp8_quantize_rows_grouped", _ptr(x), _ptr(offsets), _ptr(offsets_pad), E, n, C, _ptr(q), _ptr(s),
         _ptr(qT), _ptr(sT), _stream(x))
    return q, s, qT, sT


# ---------------------------------------------------------------- grouped GEMMs

def gg_workspace(dtype, E, n, d, f, like):
    nbytes = lib.moe_gg_workspace_bytes(dtype, E, n, d, f)
    return _empty((max(nbytes, 1),), torch.uint8, like), nbytes


def _gg_ws(ws, dtype, E, n, d, f, like):
    if ws is None:
        return gg_workspace(dtype, E, n, d, f, like)
    _check(ws, torch.uint8, "ws", ndim=1)
    return ws, ws.numel()


def _forward_weights(w_gate, w_up, w_down, dtype):
    wdt = torch.bfloat16 if dtype == BF16 else torch.uint8
    _check(w_gate, wdt, "w_gate", ndim=3)
    E, f, d = w_gate.shape
    _check(w_up, wdt, "w_up", (E, f, d))
    if w_down is not None:
        _check(w_down, wdt, "w_down", (E, d, f))
    return E, f, d


def _forward_scales(scales, n, E, d, f, with_down):
    xs, wgs, wus = scales[:3]
    _check(xs, torch.uint8, "xp_scale", (n, d // 32))
    _check(wgs, torch.uint8, "w_gate_scale", (E, f, d // 32))
    _check(wus, torch.uint8, "w_up_scale", (E, f, d // 32))
    if with_down:
        _check(scales[3], torch.uint8, "w_down_scale", (E, d, f // 32))


def grouped_gemm_swiglu(xp, offsets, w_gate, w_up, w_down, scales=None, ws=None):
    """(g, u, a [n,f], yexp [n,d]) bf16.  bf16: xp, w_* bf16 and scales None.  MXFP8: xp and w_*
    are E4M3 bytes and scales = (xp_scale, w_gate_scale, w_up_scale, w_down_scale)."""
    dtype = BF16 if scales is None else MXFP8
    E, f, d = _forward_weights(w_gate, w_up, w_down, dtype)
    _check(offsets, torch.int32, "offsets", (E + 1,))
    _check(xp, torch.bfloat16 if dtype == BF16 else torch.uint8, "xp", (None, d))
    n = xp.shape[0]
    if scales is not None:
        _need(len(scales) == 4, "scales = (xp_scale, w_gate_scale, w_up_scale, w_down_scale)")
        _forward_scales(scales, n, E, d, f, True)
    sc = (None,) * 4 if scales is None else scales
    _on_gpu(xp, offsets, w_gate, w_up, w_down, *sc)
    g = _empty((n, f), torch.bfloat16, xp)
    u = _empty((n, f), torch.bfloat16, xp)
    a = _empty((n, f), torch.bfloat16, xp)
    yexp = _empty((n, d), torch.bfloat16, xp)
    ws, nbytes = _gg_ws(ws, dtype, E, n, d, f, xp)
    call("moe_grouped_gemm_swiglu", dtype, E, n, d, f, _ptr(offsets), _ptr(xp), _ptr(sc[0]), _ptr(w_gate),
         _ptr(sc[1]), _ptr(w_up), _ptr(sc[2]), _ptr(w_down), _ptr(sc[3]), _ptr(g), _ptr(u), _ptr(a), _ptr(yexp),
         _ptr(ws), nbytes, _stream(xp))
    return g, u, a, yexp


def grouped_gemm_gate_up(xp, offsets, w_gate, w_up, scales=None):
    """(g, u, a [n,f]) bf16: the first grouped product with the SwiGLU epilogue.  MXFP8: xp and
    w_* are E4M3 bytes and scales = (xp_scale, w_gate_scale, w_up_scale)."""
    dtype = BF16 if scales is None else MXFP8
    E, f, d = _forward_weights(w_gate, w_up, None, dtype)
    _check(offsets, torch.int32, "offsets", (E + 1,))
    _check(xp, torch.bfloat16 if dtype == BF16 else torch.uint8, "xp", (None, d))
    n = xp.shape[0]
    if scales is not None:
        _need(len(scales) == 3, "scales = (xp_scale, w_gate_scale, w_up_scale)")
        _forward_scales(scales, n, E, d, f, False)
    sc = (None,) * 3 if scales is None else scales
    _on_gpu(xp, offsets, w_gate, w_up, *sc)
    g = _empty((n, f), torch.bfloat16, xp)
    u = _empty((n, f), torch.bfloat16, xp)
    a = _empty((n, f), torch.bfloat16, xp)
    call("moe_grouped_gemm_gate_up", dtype, E, n, d, f, _ptr(offsets), _ptr(xp), _ptr(sc[0]), _ptr(w_gate),
         _ptr(sc[1]), _ptr(w_up), _ptr(sc[2]), _ptr(g), _ptr(u), _ptr(a), _stream(xp))
    return g, u, a


def grouped_gemm_down(a, offsets, w_down, w_down_scale=None, ws=None):
    """yexp [n,d] bf16 = a W_down[e]^T per expert (MXFP8 when w_down_scale is given)."""
    dtype = BF16 if w_down_scale is None else MXFP8
    _check(w_down, torch.bfloat16 if dtype == BF16 else torch.uint8, "w_down", ndim=3)
    E, d, f = w_down.shape
    _check(offsets, torch.int32, "offsets", (E + 1,))
    _check(a, torch.bfloat16, "a", (None, f))
    n = a.shape[0]
    if w_down_scale is not None:
        _check(w_down_scale, torch.uint8, "w_down_scale", (E, d, f // 32))
    _on_gpu(a, offsets, w_down, w_down_scale)
    yexp = _empty((n, d), torch.bfloat16, a)
    ws, nbytes = _gg_ws(ws, dtype, E, n, d, f, a)
    call("moe_grouped_gemm_down", dtype, E, n, d, f, _ptr(offsets), _ptr(a), _ptr(w_down), _ptr(w_down_scale),
         _ptr(yexp), _ptr(ws), nbytes, _stream(a))
    return yexp


def grouped_gemm_down_mx(a_q, a_scale, offsets, w_down, w_down_scale):
    """yexp [n,d] bf16 = a W_down[e]^T per expert from an MXFP8 a (a_q [n,f] E4M3, a_scale its row
    blocks in the GEMM scale layout, as mxfp8_quantize_rows_grouped gives them)."""
    _check(w_down, torch.uint8, "w_down", ndim=3)
    E, d, f = w_down.shape
    _check(offsets, torch.int32, "offsets", (E + 1,))
    _check(a_q, torch.uint8, "a_q", (None, f))
    n = a_q.shape[0]
    _check(a_scale, torch.uint8, "a_scale", (n, f // 32))
    _check(w_down_scale, torch.uint8, "w_down_scale", (E, d, f // 32))
    _on_gpu(a_q, a_scale, offsets, w_down, w_down_scale)
    yexp = _empty((n, d), torch.bfloat16, a_q)
    call("moe_grouped_gemm_down_mx", E, n, d, f, _ptr(offsets), _ptr(a_q), _ptr(a_scale), _ptr(w_down),
         _ptr(w_down_scale), _ptr(yexp), _stream(a_q))
    return yexp


def grouped_gemm_swiglu_bwd(x_rows, g, u, a, dyexp, offsets, w_gate, w_up, w_down, scales=None,
                            offsets_pad=None, row_token=None, ws=None):
    """dict(dg, du, dxp, dw_gate, dw_up, dw_down), all bf16.
    bf16: x_rows = xp [n,d]; w_* the forward weights.
    MXFP8: x_rows = x [T,d] (read through row_token); w_gate, w_up [E,d,f] and w_down [E,f,d] are
    the dgrad-direction E4M3 weights with scales = (w_gate_scale, w_up_scale, w_down_scale)."""
    dtype = BF16 if scales is None else MXFP8
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    _check(g, torch.bfloat16, "g", ndim=2)
    n, f = g.shape
    _check(dyexp, torch.bfloat16, "dyexp", (n, None))
    d = dyexp.shape[1]
    _check(u, torch.bfloat16, "u", (n, f))
    _check(a, torch.bfloat16, "a", (n, f))
    if dtype == BF16:
        _check(x_rows, torch.bfloat16, "x_rows", (n, d))
        _need(row_token is None and offsets_pad is None, "bf16 backward takes neither row_token nor offsets_pad")
        _forward_weights(w_gate, w_up, w_down, BF16)
        _check(w_gate, torch.bfloat16, "w_gate", (E, f, d))
        sc = (None,) * 3
    else:
        _need(len(scales) == 3, "scales = (w_gate_scale, w_up_scale, w_down_scale)")
        _check(x_rows, torch.bfloat16, "x_rows", (None, d))
        _check(row_token, torch.int32, "row_token", (n,))
        _check(offsets_pad, torch.int32, "offsets_pad", (E + 1,))
        for t, name in ((w_gate, "w_gate"), (w_up, "w_up")):
            _check(t, torch.uint8, name, (E, d, f))
        _check(w_down, torch.uint8, "w_down", (E, f, d))
        _check(scales[0], torch.uint8, "w_gate_scale", (E, d, f // 32))
        _check(scales[1], torch.uint8, "w_up_scale", (E, d, f // 32))
        _check(scales[2], torch.uint8, "w_down_scale", (E, f, d // 32))
        sc = scales
    _on_gpu(x_rows, g, u, a, dyexp, offsets, w_gate, w_up, w_down, offsets_pad, row_token, *sc)
    out = dict(dg=_empty((n, f), torch.bfloat16, g), du=_empty((n, f), torch.bfloat16, g),
               dxp=_empty((n, d), torch.bfloat16, g), dw_gate=_empty((E, f, d), torch.bfloat16, g),
               dw_up=_empty((E, f, d), torch.bfloat16, g), dw_down=_empty((E, d, f), torch.bfloat16, g))
    ws, nbytes = _gg_ws(ws, dtype, E, n, d, f, g)
    call("moe_grouped_gemm_swiglu_bwd", dtype, E, n, d, f, _ptr(offsets), _ptr(offsets_pad), _ptr(row_token),
         _ptr(x_rows), _ptr(g), _ptr(u), _ptr(a), _ptr(dyexp), _ptr(w_gate), _ptr(sc[0]), _ptr(w_up),
         _ptr(sc[1]), _ptr(w_down), _ptr(sc[2]), _ptr(out["dg"]), _ptr(out["du"]), _ptr(out["dxp"]),
         _ptr(out["dw_gate"]), _ptr(out["dw_up"]), _ptr(out["dw_down"]), _ptr(ws), nbytes, _stream(g))
    return out


# ------------------------------------------------- backward grouped GEMMs, one kernel per call

def _bwd_dtype(scales, n_scales):
    if scales is None:
        return BF16, (None,) * n_scales
    _need(len(scales) == n_scales, f"expected {n_scales} scale tensors")
    return MXFP8, scales


def grouped_gemm_dgrad_down(dyexp, offsets, w_down_t, g, u, scales=None):
    """(dg, du) [n,f] bf16: da = dyexp W_down[e] through the SwiGLU backward of (g, u).
    bf16: dyexp [n,d], w_down_t = W_down [E,d,f].  MXFP8: dyexp [n,d] E4M3, w_down_t [E,f,d] E4M3,
    scales = (dyexp_scale [n,d/32], w_down_t_scale [E,f,d/32])."""
    dtype, sc = _bwd_dtype(scales, 2)
    wdt = torch.bfloat16 if dtype == BF16 else torch.uint8
    _check(g, torch.bfloat16, "g", ndim=2)
    n, f = g.shape
    _check(u, torch.bfloat16, "u", (n, f))
    _check(dyexp, wdt, "dyexp", (n, None))
    d = dyexp.shape[1]
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    _check(w_down_t, wdt, "w_down_t", (E, d, f) if dtype == BF16 else (E, f, d))
    if dtype == MXFP8:
        _check(sc[0], torch.uint8, "dyexp_scale", (n, d // 32))
        _check(sc[1], torch.uint8, "w_down_t_scale", (E, f, d // 32))
    _on_gpu(dyexp, offsets, w_down_t, g, u, *sc)
    dg = _empty((n, f), torch.bfloat16, g)
    du = _empty((n, f), torch.bfloat16, g)
    call("moe_grouped_gemm_dgrad_down", dtype, E, n, d, f, _ptr(offsets), _ptr(dyexp), _ptr(sc[0]),
         _ptr(w_down_t), _ptr(sc[1]), _ptr(g), _ptr(u), _ptr(dg), _ptr(du), _stream(g))
    return dg, du


def grouped_gemm_wgrad_down(dyexp_t, a_t, offsets, n, offsets_pad=None, scales=None):
    """dw_down [E,d,f] bf16 = dyexp_e^T a_e.  bf16: dyexp_t = dyexp [n,d], a_t = a [n,f].
    MXFP8: grouped-token quantised [d,P], [f,P] with scales = (dyexp_t_scale, a_t_scale)."""
    dtype, sc = _bwd_dtype(scales, 2)
    wdt = torch.bfloat16 if dtype == BF16 else torch.uint8
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    if dtype == BF16:
        _check(dyexp_t, wdt, "dyexp_t", (n, None))
        _check(a_t, wdt, "a_t", (n, None))
        _need(offsets_pad is None, "bf16 weight gradients take no offsets_pad")
        d, f = dyexp_t.shape[1], a_t.shape[1]
    else:
        P = _mx_pad_cap(n, E)
        _check(dyexp_t, wdt, "dyexp_t", (None, P))
        _check(a_t, wdt, "a_t", (None, P))
        d, f = dyexp_t.shape[0], a_t.shape[0]
        _check(offsets_pad, torch.int32, "offsets_pad", (E + 1,))
        _check(sc[0], torch.uint8, "dyexp_t_scale", (P // 32, d))
        _check(sc[1], torch.uint8, "a_t_scale", (P // 32, f))
    _on_gpu(dyexp_t, a_t, offsets, offsets_pad, *sc)
    dw = _empty((E, d, f), torch.bfloat16, dyexp_t)
    call("moe_grouped_gemm_wgrad_down", dtype, E, n, d, f, _ptr(offsets), _ptr(offsets_pad), _ptr(dyexp_t),
         _ptr(sc[0]), _ptr(a_t), _ptr(sc[1]), _ptr(dw), _stream(dyexp_t))
    return dw


def grouped_gemm_dgrad_gate_up(dg, du, offsets, w_gate_t, w_up_t, scales=None):
    """dxp [n,d] bf16 = dg W_gate[e] + du W_up[e].  bf16: dg, du [n,f], w_*_t = forward weights
    [E,f,d].  MXFP8: dg, du [n,f] E4M3, w_*_t [E,d,f] E4M3, scales = (dg_scale, du_scale,
    w_gate_t_scale, w_up_t_scale)."""
    dtype, sc = _bwd_dtype(scales, 4)
    wdt = torch.bfloat16 if dtype == BF16 else torch.uint8
    _check(dg, wdt, "dg", ndim=2)
    n, f = dg.shape
    _check(du, wdt, "du", (n, f))
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    _check(w_gate_t, wdt, "w_gate_t", ndim=3)
    d = w_gate_t.shape[2] if dtype == BF16 else w_gate_t.shape[1]
    wshape = (E, f, d) if dtype == BF16 else (E, d, f)
    _check(w_gate_t, wdt, "w_gate_t", wshape)
    _check(w_up_t, wdt, "w_up_t", wshape)
    if dtype == MXFP8:
        _check(sc[0], torch.uint8, "dg_scale", (n, f // 32))
        _check(sc[1], torch.uint8, "du_scale", (n, f // 32))
        _check(sc[2], torch.uint8, "w_gate_t_scale", (E, d, f // 32))
        _check(sc[3], torch.uint8, "w_up_t_scale", (E, d, f // 32))
    _on_gpu(dg, du, offsets, w_gate_t, w_up_t, *sc)
    dxp = _empty((n, d), torch.bfloat16, dg)
    call("moe_grouped_gemm_dgrad_gate_up", dtype, E, n, d, f, _ptr(offsets), _ptr(dg), _ptr(sc[0]), _ptr(du),
         _ptr(sc[1]), _ptr(w_gate_t), _ptr(sc[2]), _ptr(w_up_t), _ptr(sc[3]), _ptr(dxp), _stream(dg))
    return dxp


def grouped_gemm_wgrad_gate_up(dg_t, du_t, xp_t, offsets, n, offsets_pad=None, scales=None):
    """(dw_gate, dw_up) [E,f,d] bf16 = dg_e^T xp_e, du_e^T xp_e.  bf16: the row tensors dg, du
    [n,f], xp [n,d].  MXFP8: grouped-token quantised [f,P], [f,P], [d,P] with scales =
    (dg_t_scale, du_t_scale, xp_t_scale)."""
    dtype, sc = _bwd_dtype(scales, 3)
    wdt = torch.bfloat16 if dtype == BF16 else torch.uint8
    _check(offsets, torch.int32, "offsets", ndim=1)
    E = offsets.shape[0] - 1
    if dtype == BF16:
        _check(dg_t, wdt, "dg_t", (n, None))
        f = dg_t.shape[1]
        _check(du_t, wdt, "du_t", (n, f))
        _check(xp_t, wdt, "xp_t", (n, None))
        d = xp_t.shape[1]
        _need(offsets_pad is None, "bf16 weight gradients take no offsets_pad")
    else:
        P = _mx_pad_cap(n, E)
        _check(dg_t, wdt, "dg_t", (None, P))
        f = dg_t.shape[0]
        _check(du_t, wdt, "du_t", (f, P))
        _check(xp_t, wdt, "xp_t", (None, P))
        d = xp_t.shape[0]
        _check(offsets_pad, torch.int32, "offsets_pad", (E + 1,))
        _check(sc[0], torch.uint8, "dg_t_scale", (P // 32, f))
        _check(sc[1], torch.uint8, "du_t_scale", (P // 32, f))
        _check(sc[2], torch.uint8, "xp_t_scale", (P // 32, d))
    _on_gpu(dg_t, du_t, xp_t, offsets, offsets_pad, *sc)
    dwg = _empty((E, f, d), torch.bfloat16, dg_t)
    dwu = _empty((E, f, d), torch.bfloat16, dg_t)
    call("moe_grouped_gemm_wgrad_gate_up", dtype, E, n, d, f, _ptr(offsets), _ptr(offsets_pad), _ptr(dg_t),
         _ptr(sc[0]), _ptr(du_t), _ptr(sc[1]), _ptr(xp_t), _ptr(sc[2]), _ptr(dwg), _ptr(dwu), _stream(dg_t))
    return dwg, dwu
