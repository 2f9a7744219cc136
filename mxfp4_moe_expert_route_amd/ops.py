"""Torch-tensor wrappers with the C ABI's names (argument marshalling only).

Each wrapper checks device, dtype, shape and contiguity, allocates outputs
that were not passed in, and calls the library on the current HIP stream.
Every step of the computation runs in libmxfp4moe.so."""

import torch

from ._lib import check, lib

F32, BF16 = 0, 1


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t


def _out(t, name, dtype, shape, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, name, dtype, shape, device)


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() else None


# ---------------------------------------------------------------------------

def mxfp4_pack(x, codes=None, scales=None):
    """x [rows, K] float32 or bfloat16 -> (codes uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, "x", x.dtype)
    rows, K = x.shape
    codes = _out(codes, "codes", torch.uint8, (rows, K // 2), x.device)
    scales = _out(scales, "scales", torch.uint8, (rows, K // 32), x.device)
    check(lib().mxfp4_pack(_ptr(x), BF16 if x.dtype == torch.bfloat16 else F32, rows, K,
                           _ptr(codes), _ptr(scales), _stream()), "mxfp4_pack")
    return codes, scales


def mxfp4_unpack(codes, scales, dtype=torch.float32, out=None):
    """(codes [rows, K/2], scales [rows, K/32]) -> [rows, K] float32 or bfloat16."""
    _need(codes, "codes", torch.uint8)
    rows, half = codes.shape
    K = 2 * half
    _need(scales, "scales", torch.uint8, (rows, K // 32), codes.device)
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dtype must be float32 or bfloat16")
    out = _out(out, "out", dtype, (rows, K), codes.device)
    check(lib().mxfp4_unpack(_ptr(codes), _ptr(scales), rows, K, _ptr(out),
                             BF16 if dtype == torch.bfloat16 else F32, _stream()), "mxfp4_unpack")
    return out


def moe_route_topk(logits, k, topk_ids=None, topk_w=None):
    """logits [T, E] float32 -> (ids int32 [T, k], weights float32 [T, k])."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    topk_ids = _out(topk_ids, "topk_ids", torch.int32, (T, k), logits.device)
    topk_w = _out(topk_w, "topk_w", torch.float32, (T, k), logits.device)
    check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _stream()),
          "moe_route_topk")
    return topk_ids, topk_w


def moe_router_topk(x, w_router, k, bias=None, logits=None, topk_ids=None, topk_w=None):
    """x [T, H] bfloat16, w_router [E, H] float32 (bias [E] float32 or None)
    -> (logits float32 [T, E], ids int32 [T, k], weights float32 [T, k])."""
    _need(x, "x", torch.bfloat16)
    _need(w_router, "w_router", torch.float32)
    T, H = x.shape
    E, H2 = w_router.shape
    if H2 != H:
        raise ValueError("w_router must be [E, H] with H = x.shape[1]")
    if bias is not None:
        _need(bias, "bias", torch.float32)
        if tuple(bias.shape) != (E,):
            raise ValueError("bias must be [E]")
    logits = _out(logits, "logits", torch.float32, (T, E), x.device)
    topk_ids = _out(topk_ids, "topk_ids", torch.int32, (T, k), x.device)
    topk_w = _out(topk_w, "topk_w", torch.float32, (T, k), x.device)
    check(lib().moe_router_topk(_ptr(x), _ptr(w_router), _ptr(bias) if bias is not None else None,
                                T, H, E, k, _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                _stream()), "moe_router_topk")
    return logits, topk_ids, topk_w


def dflash_verify_accept(target_logits, draft_probs, draft_tokens, uniforms, accept_len=None,
                         next_token=None, workspace=None):
    """target_logits [B, L+1, V] f32, draft_probs [B, L, V] f32, draft_tokens
    [B, L] int32, uniforms [B, L+1] f32 -> (accept_len int32 [B], next_token
    int32 [B])."""
    _need(target_logits, "target_logits", torch.float32)
    _need(draft_probs, "draft_probs", torch.float32)
    _need(draft_tokens, "draft_tokens", torch.int32)
    _need(uniforms, "uniforms", torch.float32)
    B, L1, V = target_logits.shape
    L = L1 - 1
    if tuple(draft_probs.shape) != (B, L, V) or tuple(draft_tokens.shape) != (B, L) or \
            tuple(uniforms.shape) != (B, L + 1):
        raise ValueError("shapes must be [B, L+1, V], [B, L, V], [B, L], [B, L+1]")
    dev = target_logits.device
    accept_len = _out(accept_len, "accept_len", torch.int32, (B,), dev)
    next_token = _out(next_token, "next_token", torch.int32, (B,), dev)
    nbytes = int(lib().dflash_verify_workspace_bytes(B, L, V))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=dev)
    check(lib().dflash_verify_accept(_ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens),
                                     _ptr(uniforms), B, L, V, _ptr(accept_len), _ptr(next_token),
                                     _ptr(workspace), workspace.numel(), _stream()),
          "dflash_verify_accept")
    return accept_len, next_token


def moe_permute_workspace_bytes(T, E, k):
    return int(lib().moe_permute_workspace_bytes(T, E, k))


def moe_permute(topk_ids, E, counts=None, offsets=None, sorted_pairs=None, pair_to_row=None,
                workspace=None):
    """topk_ids [T, k] int32 -> (counts [E], offsets [E+1], sorted_pairs [T*k], pair_to_row [T*k])."""
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = _out(counts, "counts", torch.int32, (E,), dev)
    offsets = _out(offsets, "offsets", torch.int32, (E + 1,), dev)
    sorted_pairs = _out(sorted_pairs, "sorted_pairs", torch.int32, (T * k,), dev)
    pair_to_row = _out(pair_to_row, "pair_to_row", torch.int32, (T * k,), dev)
    nws = moe_permute_workspace_bytes(T, E, k)
    if workspace is None and nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() if workspace is not None else 0
    check(lib().moe_permute(_ptr(topk_ids), T, E, k, _ptr(counts), _ptr(offsets),
                            _ptr(sorted_pairs), _ptr(pair_to_row), _ptr(workspace), wsb,
                            _stream()), "moe_permute")
    return counts, offsets, sorted_pairs, pair_to_row


def moe_route_permute(logits, k, topk_ids=None, topk_w=None, counts=None, offsets=None,
                      sorted_pairs=None, pair_to_row=None, workspace=None):
    """logits [T, E] f32 -> (topk_ids [T, k], topk_w [T, k], counts [E], offsets [E+1],
    sorted_pairs [T*k], pair_to_row [T*k]); moe_route_topk then moe_permute in one call."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    topk_ids = _out(topk_ids, "topk_ids", torch.int32, (T, k), dev)
    topk_w = _out(topk_w, "topk_w", torch.float32, (T, k), dev)
    counts = _out(counts, "counts", torch.int32, (E,), dev)
    offsets = _out(offsets, "offsets", torch.int32, (E + 1,), dev)
    sorted_pairs = _out(sorted_pairs, "sorted_pairs", torch.int32, (T * k,), dev)
    pair_to_row = _out(pair_to_row, "pair_to_row", torch.int32, (T * k,), dev)
    nws = moe_permute_workspace_bytes(T, E, k)
    if workspace is None and nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() if workspace is not None else 0
    check(lib().moe_route_permute(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(counts), _ptr(offsets), _ptr(sorted_pairs),
                                  _ptr(pair_to_row), _ptr(workspace), wsb, _stream()),
          "moe_route_permute")
    return topk_ids, topk_w, counts, offsets, sorted_pairs, pair_to_row


def moe_mxfp4_gate_up_swiglu(x, sorted_pairs, offsets, k, w13_codes, w13_scales, h=None):
    """x [T, H] bf16 -> h [T*k, I] bf16 (rows in sorted order)."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    E, two_i, half_h = w13_codes.shape
    I = two_i // 2
    dev = x.device
    _need(sorted_pairs, "sorted_pairs", torch.int32, (T * k,), dev)
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H // 2), dev)
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32), dev)
    h = _out(h, "h", torch.bfloat16, (T * k, I), dev)
    check(lib().moe_mxfp4_gate_up_swiglu(_ptr(x), _ptr(sorted_pairs), _ptr(offsets), T, H, I, E,
                                         k, _ptr(w13_codes), _ptr(w13_scales), _ptr(h),
                                         _stream()), "moe_mxfp4_gate_up_swiglu")
    return h


def moe_mxfp4_down(h, offsets, k, w2_codes, w2_scales, y=None):
    """h [T*k, I] bf16 -> y [T*k, H] float32 (rows in sorted order)."""
    _need(h, "h", torch.bfloat16)
    R, I = h.shape
    T = R // k
    E, H, _ = w2_codes.shape
    dev = h.device
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I // 2), dev)
    _need(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32), dev)
    y = _out(y, "y", torch.float32, (R, H), dev)
    check(lib().moe_mxfp4_down(_ptr(h), _ptr(offsets), T, H, I, E, k, _ptr(w2_codes),
                               _ptr(w2_scales), _ptr(y), _stream()), "moe_mxfp4_down")
    return y


def moe_combine(y, topk_w, pair_to_row, out=None):
    """y [T*k, H] float32, topk_w [T, k] -> out [T, H] float32."""
    _need(topk_w, "topk_w", torch.float32)
    T, k = topk_w.shape
    _need(y, "y", torch.float32)
    H = y.shape[1]
    dev = y.device
    _need(y, "y", torch.float32, (T * k, H), dev)
    _need(pair_to_row, "pair_to_row", torch.int32, (T * k,), dev)
    out = _out(out, "out", torch.float32, (T, H), dev)
    check(lib().moe_combine(_ptr(y), _ptr(topk_w), _ptr(pair_to_row), T, H, k, _ptr(out),
                            _stream()), "moe_combine")
    return out


class LayerBuffers:
    """Preallocated intermediates of one layer call (so a timed loop allocates nothing)."""

    def __init__(self, T, H, I, E, k, device):
        R = T * k
        z = dict(device=device)
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, **z)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, **z)
        self.counts = torch.empty((E,), dtype=torch.int32, **z)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, **z)
        self.sorted_pairs = torch.empty((R,), dtype=torch.int32, **z)
        self.pair_to_row = torch.empty((R,), dtype=torch.int32, **z)
        self.h = torch.empty((R, I), dtype=torch.bfloat16, **z)
        self.y = torch.empty((R, H), dtype=torch.float32, **z)
        self.out = torch.empty((T, H), dtype=torch.float32, **z)
        nws = moe_permute_workspace_bytes(T, E, k)
        self.workspace = torch.empty(max(nws, 1), dtype=torch.uint8, **z)


def moe_mxfp4_layer(x, logits, k, w13_codes, w13_scales, w2_codes, w2_scales, buffers=None):
    """Whole layer in one C call (route, permute, gate/up, down, combine).

    Returns the LayerBuffers holding every intermediate; `.out` is the result."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    E, two_i, _ = w13_codes.shape
    I = two_i // 2
    dev = x.device
    _need(logits, "logits", torch.float32, (T, E), dev)
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H // 2), dev)
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32), dev)
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I // 2), dev)
    _need(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32), dev)
    b = buffers if buffers is not None else LayerBuffers(T, H, I, E, k, dev)
    if (b.T, b.H, b.I, b.E, b.k) != (T, H, I, E, k):
        raise ValueError("buffers were made for another shape")
    check(lib().moe_mxfp4_layer(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(b.topk_ids), _ptr(b.topk_w), _ptr(b.counts), _ptr(b.offsets),
        _ptr(b.sorted_pairs), _ptr(b.pair_to_row), _ptr(b.h), _ptr(b.y), _ptr(b.out),
        _ptr(b.workspace), b.workspace.numel(), _stream()), "moe_mxfp4_layer")
    return b


def moe_mxfp4_decode_layer_workspace_bytes(T, H, I, E, k):
    """Bytes of the zero-filled workspace moe_mxfp4_decode_layer needs (0: the
    persistent kernel does not take these sizes)."""
    return int(lib().moe_mxfp4_decode_layer_workspace_bytes(T, H, I, E, k))


def decode_layer_workspace(T, H, I, E, k, device):
    """A zero-filled workspace for moe_mxfp4_decode_layer (None if the sizes
    are not taken).  Each call leaves it zero-filled, so it is reusable."""
    n = moe_mxfp4_decode_layer_workspace_bytes(T, H, I, E, k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def moe_mxfp4_decode_layer(x, logits, k, w13_codes, w13_scales, w2_codes, w2_scales, workspace,
                           buffers=None):
    """The whole layer as one persistent kernel (verify-sized batches, T <= 16).

    `workspace` comes from decode_layer_workspace (zero-filled; the call leaves
    it so).  Returns the LayerBuffers holding every intermediate; `.out` is the
    result, equal bit for bit to moe_mxfp4_layer's."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    E, two_i, _ = w13_codes.shape
    I = two_i // 2
    dev = x.device
    _need(logits, "logits", torch.float32, (T, E), dev)
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H // 2), dev)
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32), dev)
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I // 2), dev)
    _need(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    b = buffers if buffers is not None else LayerBuffers(T, H, I, E, k, dev)
    if (b.T, b.H, b.I, b.E, b.k) != (T, H, I, E, k):
        raise ValueError("buffers were made for another shape")
    check(lib().moe_mxfp4_decode_layer(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(b.topk_ids), _ptr(b.topk_w), _ptr(b.counts), _ptr(b.offsets),
        _ptr(b.sorted_pairs), _ptr(b.pair_to_row), _ptr(b.h), _ptr(b.y), _ptr(b.out),
        _ptr(workspace), workspace.numel(), _stream()), "moe_mxfp4_decode_layer")
    return b


def moe_mxfp4_layer_noalloc(x, logits, k, w13_codes, w13_scales, w2_codes, w2_scales, buffers):
    """moe_mxfp4_layer through the entry point that allocates nothing: its
    grouping workspace is the library's fixed device scratch (the workspace
    tensor of `buffers` is not used).  `buffers` (LayerBuffers of this shape)
    must be passed in, so the call itself allocates nothing either."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    E, two_i, _ = w13_codes.shape
    I = two_i // 2
    dev = x.device
    _need(logits, "logits", torch.float32, (T, E), dev)
    _need(w13_codes, "w13_codes", torch.uint8, (E, 2 * I, H // 2), dev)
    _need(w13_scales, "w13_scales", torch.uint8, (E, 2 * I, H // 32), dev)
    _need(w2_codes, "w2_codes", torch.uint8, (E, H, I // 2), dev)
    _need(w2_scales, "w2_scales", torch.uint8, (E, H, I // 32), dev)
    b = buffers
    if (b.T, b.H, b.I, b.E, b.k) != (T, H, I, E, k):
        raise ValueError("buffers were made for another shape")
    check(lib().moe_mxfp4_layer_noalloc(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
        _ptr(w2_scales), _ptr(b.topk_ids), _ptr(b.topk_w), _ptr(b.counts), _ptr(b.offsets),
        _ptr(b.sorted_pairs), _ptr(b.pair_to_row), _ptr(b.h), _ptr(b.y), _ptr(b.out),
        _stream()), "moe_mxfp4_layer_noalloc")
    return b


def mxm_stream_xor(src, result, nontemporal=False):
    """Streaming-read probe (a measurement aid): XOR every 32-bit word of the
    contiguous tensor `src` (byte size a multiple of 16) into `result`, an
    int32 tensor of one element that the caller initialises."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _need(result, "result", torch.int32, (1,), src.device)
    nbytes = src.numel() * src.element_size()
    check(lib().mxm_stream_xor(_ptr(src), nbytes, 1 if nontemporal else 0, _ptr(result),
                               _stream()), "mxm_stream_xor")
    return result
