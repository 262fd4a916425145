"""torch-facing wrappers of libqv.so: argument marshalling only.

Each function checks dtypes and shapes, hands raw device pointers and the current HIP stream
to the C ABI (include/qv.h) and returns the output tensors.  Every step of the computation
runs in the library's HIP kernels; nothing here computes.  Calls are asynchronous on the
current stream, like any torch op.

The optional `tune` argument of quant_act, prepare_w8 and the linears is a {key: value} dict of
work-split overrides (keys of ``_binding.TUNE_KEYS``) for tests and launch-shape measurements:
it routes the call to its qv_test_* twin (include/qv_test.h).  Without it the qv.h call runs,
whose plan depends on the shape alone.

Workspaces (split-K partial sums and arrival counters) are cached per (device, stream):
allocated zero-filled once, grown on demand, and left with zeroed counters by every call.
A buffer that has been outgrown stays alive (a captured HIP graph may still use it).
"""
from __future__ import annotations

import torch

from . import _binding as B

__all__ = ["prepare_w8", "prepare_w4", "quant_act", "linear_w8a8", "linear_w4a16", "linear_w4a8", "verify_greedy", "verify_tree",
           "verify_sample", "workspace_bytes", "workspace", "read_stream"]

_WORKSPACES: dict = {}
_OUTGROWN: list = []


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev2d(t: torch.Tensor, name: str, dtypes) -> None:
    _need(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.dtype in dtypes, f"{name} must have dtype in {dtypes}, got {t.dtype}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def workspace_bytes(op: int, M: int, N: int, K: int = 0, tune: dict | None = None) -> int:
    if tune:
        return int(B.lib().qv_test_workspace_bytes(op, M, N, K, B.tune_array(tune)))
    return int(B.lib().qv_workspace_bytes(op, M, N, K))


def workspace(nbytes: int, device: torch.device) -> torch.Tensor | None:
    """A zero-initialised uint8 device buffer of at least `nbytes` for the current stream."""
    if nbytes == 0:
        return None
    key = (device.index, _stream(device))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _OUTGROWN.append(ws)
        size = max(nbytes, 2 * ws.numel() if ws is not None else 0)
        ws = torch.zeros(size, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def quant_act(x: torch.Tensor, inv_smooth: torch.Tensor | None = None,
              out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
              tune: dict | None = None):
    """x fp16 [M][K] -> (x_q int8 [M][K], x_scale fp32 [M])."""
    _dev2d(x, "x", (torch.float16,))
    _need(x.dim() == 2, "x must be [M][K]")
    M, K = x.shape
    if inv_smooth is not None:
        _dev2d(inv_smooth, "inv_smooth", (torch.float32,))
        _need(inv_smooth.shape == (K,), "inv_smooth must be [K]")
    xq = out if out is not None else torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = scale_out if scale_out is not None else torch.empty((M,), dtype=torch.float32,
                                                             device=x.device)
    _need(xq.shape == (M, K) and xq.dtype == torch.int8 and xq.is_contiguous(), "bad out")
    _need(sx.shape == (M,) and sx.dtype == torch.float32, "bad scale_out")
    args = (_ptr(x), _ptr(inv_smooth), M, K, _ptr(xq), _ptr(sx), _stream(x.device))
    if tune:
        B.check("qv_test_quant_act", B.lib().qv_test_quant_act(*args, B.tune_array(tune)))
    else:
        B.check("qv_quant_act", B.lib().qv_quant_act(*args))
    return xq, sx


def prepare_w8(w: torch.Tensor, inv_s: torch.Tensor | None = None, tune: dict | None = None):
    """Offline: bf16 [N][K] (int16/uint16 bit patterns also accepted), optional fp32 column
    multipliers [K] -> (w_q int8 [N][K], w_scale fp32 [N]) for linear_w8a8."""
    _dev2d(w, "w", (torch.bfloat16, torch.int16, torch.uint16))
    _need(w.dim() == 2, "w must be [N][K]")
    N, K = w.shape
    if inv_s is not None:
        _dev2d(inv_s, "inv_s", (torch.float32,))
        _need(inv_s.shape == (K,), "inv_s must be [K]")
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    ws = torch.empty((N,), dtype=torch.float32, device=w.device)
    args = (_ptr(w), _ptr(inv_s), N, K, _ptr(wq), _ptr(ws), _stream(w.device))
    if tune:
        B.check("qv_test_prepare_w8", B.lib().qv_test_prepare_w8(*args, B.tune_array(tune)))
    else:
        B.check("qv_prepare_w8", B.lib().qv_prepare_w8(*args))
    return wq, ws


def prepare_w4(w: torch.Tensor, group_size: int = 128):
    """Offline: bf16 [N][K] -> (qweight int32 [N][K/8], scales fp16 [N][K/128], zeros uint8
    [N][K/128]) for linear_w4a16 / linear_w4a8."""
    _dev2d(w, "w", (torch.bfloat16, torch.int16, torch.uint16))
    _need(w.dim() == 2, "w must be [N][K]")
    N, K = w.shape
    _need(group_size > 0 and K % group_size == 0, "K must be a multiple of group_size")
    qw = torch.empty((N, K // 8), dtype=torch.int32, device=w.device)
    sc = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    z = torch.empty((N, K // group_size), dtype=torch.uint8, device=w.device)
    B.check("qv_prepare_w4", B.lib().qv_prepare_w4(_ptr(w), N, K, group_size, _ptr(qw), _ptr(sc),
                                                   _ptr(z), _stream(w.device)))
    return qw, sc, z


def linear_w8a8(x_q: torch.Tensor, x_scale: torch.Tensor, w: torch.Tensor,
                w_scale: torch.Tensor, out: torch.Tensor | None = None,
                acc_out: torch.Tensor | bool | None = None, tune: dict | None = None):
    """x_q int8 [M][K], x_scale fp32 [M], w int8 [N][K], w_scale fp32 [N] -> y fp16 [M][N].

    With acc_out=True (or an int32 [M][N] tensor) also returns the int32 accumulators.
    """
    _dev2d(x_q, "x_q", (torch.int8,))
    _dev2d(w, "w", (torch.int8,))
    _dev2d(x_scale, "x_scale", (torch.float32,))
    _dev2d(w_scale, "w_scale", (torch.float32,))
    M, K = x_q.shape
    N = w.shape[0]
    _need(w.shape == (N, K), "w must be [N][K]")
    _need(x_scale.shape == (M,) and w_scale.shape == (N,), "scale shapes")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=w.device)
    _need(y.shape == (M, N) and y.dtype == torch.float16 and y.is_contiguous(), "bad out")
    acc = None
    if acc_out is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=w.device)
    elif isinstance(acc_out, torch.Tensor):
        acc = acc_out
        _need(acc.shape == (M, N) and acc.dtype == torch.int32 and acc.is_contiguous(), "bad acc")
    nbytes = workspace_bytes(B.QV_OP_W8A8, M, N, K, tune)
    ws = workspace(nbytes, w.device)
    args = (_ptr(x_q), _ptr(x_scale), M, K, _ptr(w), _ptr(w_scale), N, _ptr(y), _ptr(acc),
            _ptr(ws), ws.numel() if ws is not None else 0, _stream(w.device))
    if tune:
        B.check("qv_test_linear_w8a8", B.lib().qv_test_linear_w8a8(*args, B.tune_array(tune)))
    else:
        B.check("qv_linear_w8a8", B.lib().qv_linear_w8a8(*args))
    return (y, acc) if acc is not None else y


def linear_w4a16(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor, group_size: int = 128, out: torch.Tensor | None = None,
                 tune: dict | None = None):
    """x fp16 [M][K], qweight int32/uint32 [N][K/8] (eight 4-bit codes per word, low nibble
    first), scales fp16 [N][K/128], zeros uint8 [N][K/128] -> y fp16 [M][N]."""
    _dev2d(x, "x", (torch.float16,))
    _dev2d(qweight, "qweight", (torch.int32, torch.uint32))
    _dev2d(scales, "scales", (torch.float16,))
    _dev2d(zeros, "zeros", (torch.uint8,))
    M, K = x.shape
    N = qweight.shape[0]
    _need(qweight.shape == (N, K // 8) and K % 8 == 0, "qweight must be [N][K/8]")
    _need(group_size > 0 and K % group_size == 0, "K must be a multiple of group_size")
    _need(scales.shape == (N, K // group_size) and zeros.shape == scales.shape,
          "scales/zeros must be [N][K/group_size]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    _need(y.shape == (M, N) and y.dtype == torch.float16 and y.is_contiguous(), "bad out")
    nbytes = workspace_bytes(B.QV_OP_W4A16, M, N, K, tune)
    ws = workspace(nbytes, x.device)
    args = (_ptr(x), M, K, _ptr(qweight), _ptr(scales), _ptr(zeros), N, group_size, _ptr(y),
            _ptr(ws), ws.numel() if ws is not None else 0, _stream(x.device))
    if tune:
        B.check("qv_test_linear_w4a16", B.lib().qv_test_linear_w4a16(*args, B.tune_array(tune)))
    else:
        B.check("qv_linear_w4a16", B.lib().qv_linear_w4a16(*args))
    return y


def linear_w4a8(x_q: torch.Tensor, x_scale: torch.Tensor, qweight: torch.Tensor,
                scales: torch.Tensor, zeros: torch.Tensor, group_size: int = 128,
                out: torch.Tensor | None = None, tune: dict | None = None):
    """x_q int8 [M][K] and x_scale fp32 [M] (from quant_act), qweight int32/uint32 [N][K/8],
    scales fp16 [N][K/128], zeros uint8 [N][K/128] -> y fp16 [M][N]."""
    _dev2d(x_q, "x_q", (torch.int8,))
    _dev2d(x_scale, "x_scale", (torch.float32,))
    _dev2d(qweight, "qweight", (torch.int32, torch.uint32))
    _dev2d(scales, "scales", (torch.float16,))
    _dev2d(zeros, "zeros", (torch.uint8,))
    M, K = x_q.shape
    N = qweight.shape[0]
    _need(x_scale.shape == (M,), "x_scale must be [M]")
    _need(qweight.shape == (N, K // 8) and K % 8 == 0, "qweight must be [N][K/8]")
    _need(group_size > 0 and K % group_size == 0, "K must be a multiple of group_size")
    _need(scales.shape == (N, K // group_size) and zeros.shape == scales.shape,
          "scales/zeros must be [N][K/group_size]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x_q.device)
    _need(y.shape == (M, N) and y.dtype == torch.float16 and y.is_contiguous(), "bad out")
    nbytes = workspace_bytes(B.QV_OP_W4A8, M, N, K, tune)
    ws = workspace(nbytes, x_q.device)
    args = (_ptr(x_q), _ptr(x_scale), M, K, _ptr(qweight), _ptr(scales), _ptr(zeros), N,
            group_size, _ptr(y), _ptr(ws), ws.numel() if ws is not None else 0,
            _stream(x_q.device))
    if tune:
        B.check("qv_test_linear_w4a8", B.lib().qv_test_linear_w4a8(*args, B.tune_array(tune)))
    else:
        B.check("qv_linear_w4a8", B.lib().qv_linear_w4a8(*args))
    return y


def verify_greedy(logits: torch.Tensor, draft: torch.Tensor | None,
                  argmax_out: torch.Tensor | None = None,
                  n_accept_out: torch.Tensor | None = None):
    """logits fp16 [M][V], draft int32 [M-1] -> (argmax int32 [M], n_accept int32 [1]).

    n_accept stays on the device; reading it (e.g. .item()) is the step's only sync."""
    _dev2d(logits, "logits", (torch.float16,))
    M, V = logits.shape
    if M > 1:
        _dev2d(draft, "draft", (torch.int32,))
        _need(draft.shape == (M - 1,), "draft must be [M-1]")
    am = argmax_out if argmax_out is not None else torch.empty((M,), dtype=torch.int32,
                                                               device=logits.device)
    na = n_accept_out if n_accept_out is not None else torch.empty((1,), dtype=torch.int32,
                                                                   device=logits.device)
    nbytes = workspace_bytes(B.QV_OP_VERIFY, M, V, 0)
    ws = workspace(nbytes, logits.device)
    B.check("qv_verify_greedy", B.lib().qv_verify_greedy(
        _ptr(logits), M, V, _ptr(draft) if M > 1 else None, _ptr(am), _ptr(na),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(logits.device)))
    return am, na


def verify_tree(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                argmax_out: torch.Tensor | None = None, path_out: torch.Tensor | None = None,
                accept_out: torch.Tensor | None = None):
    """logits fp16 [M][V] (one row per tree node), tokens int32 [M], parent int32 [M] ->
    (argmax int32 [M], path int32 [M] (-1 past its end), accept int32 [2] = {L, bonus})."""
    _dev2d(logits, "logits", (torch.float16,))
    M, V = logits.shape
    _dev2d(tokens, "tokens", (torch.int32,))
    _dev2d(parent, "parent", (torch.int32,))
    _need(tokens.shape == (M,) and parent.shape == (M,), "tokens and parent must be [M]")
    dev = logits.device
    am = argmax_out if argmax_out is not None else torch.empty((M,), dtype=torch.int32, device=dev)
    path = path_out if path_out is not None else torch.empty((M,), dtype=torch.int32, device=dev)
    acc = accept_out if accept_out is not None else torch.empty((2,), dtype=torch.int32, device=dev)
    nbytes = workspace_bytes(B.QV_OP_VERIFY, M, V, 0)
    ws = workspace(nbytes, dev)
    B.check("qv_verify_tree", B.lib().qv_verify_tree(
        _ptr(logits), M, V, _ptr(tokens), _ptr(parent), _ptr(am), _ptr(path), _ptr(acc),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(dev)))
    return am, path, acc


def verify_sample(logits: torch.Tensor, draft: torch.Tensor | None, uniforms: torch.Tensor,
                  temperature: float, draft_logits: torch.Tensor | None = None,
                  result_out: torch.Tensor | None = None):
    """Speculative sampling at temperature T > 0.  logits fp16 [M][V] (target), draft int32
    [M-1], uniforms float64 [M] in [0, 1), draft_logits fp16 [M-1][V] or None (a point-mass
    drafter) -> result int32 [2] = {n_accept, token}, left on the device."""
    _dev2d(logits, "logits", (torch.float16,))
    M, V = logits.shape
    dev = logits.device
    if M > 1:
        _dev2d(draft, "draft", (torch.int32,))
        _need(draft.shape == (M - 1,), "draft must be [M-1]")
        if draft_logits is not None:
            _dev2d(draft_logits, "draft_logits", (torch.float16,))
            _need(draft_logits.shape == (M - 1, V), "draft_logits must be [M-1][V]")
    _dev2d(uniforms, "uniforms", (torch.float64,))
    _need(uniforms.shape == (M,), "uniforms must be [M]")
    res = result_out if result_out is not None else torch.empty((2,), dtype=torch.int32, device=dev)
    nbytes = workspace_bytes(B.QV_OP_SAMPLE, M, V, 0)
    ws = workspace(nbytes, dev)
    B.check("qv_verify_sample", B.lib().qv_verify_sample(
        _ptr(logits), M, V, _ptr(draft_logits) if M > 1 else None, _ptr(draft) if M > 1 else None,
        _ptr(uniforms), float(temperature), _ptr(res), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(dev)))
    return res


def read_stream(buf: torch.Tensor, pattern: int = B.QV_READ_LINEAR, row_bytes: int = 0,
                nontemporal: bool = False, blocks: int = 2048,
                sink: torch.Tensor | None = None) -> torch.Tensor:
    """Read-only bandwidth probe (qv_test_read_stream): reads every byte of `buf` once and
    returns the per-workgroup XOR sink, int32 [blocks, 4] (XOR over its rows = XOR of the
    buffer's 16-byte vectors)."""
    _need(isinstance(buf, torch.Tensor) and buf.is_cuda and buf.is_contiguous(),
          "buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(blocks, 4, dtype=torch.int32, device=buf.device)
    _need(sink.is_cuda and sink.dtype == torch.int32 and sink.is_contiguous() and
          sink.numel() >= 4 * blocks, "sink must be a contiguous int32 GPU tensor of blocks x 4")
    B.check("qv_test_read_stream", B.lib().qv_test_read_stream(
        buf.data_ptr(), nbytes, pattern, row_bytes, int(nontemporal), blocks, sink.data_ptr(),
        _stream(buf.device)))
    return sink
