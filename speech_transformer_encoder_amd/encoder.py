"""Device-memory plumbing around the C ABI: packed layer blobs, workspace and output buffers.

PyTorch supplies device memory and the stream; every step of the forward pass runs in the
library's kernels through :mod:`binding`.  Nothing here computes any part of the block.
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import binding as B

_ORDER = ("ln1_g", "ln1_b", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo", "ln2_g", "ln2_b",
          "w1", "b1", "w2", "b2")


def _device_f32(a, device):
    import torch
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.float32).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class EncoderStack:
    """``n_layers`` packed blocks of one shape and path, plus an optional final LayerNorm.

    ``layers``: per-block parameter dicts in PyTorch layout (numpy or torch, fp32 values), keys
    ``ln1_g ln1_b wq bq wk bk wv bv wo bo ln2_g ln2_b w1 b1 w2 b2`` (``bk`` may be None).

    One object holds one workspace: calls that may run at the same time on different streams
    need one object each (or are ordered by the caller), since they would share it.
    """

    def __init__(self, layers: Sequence[Dict], d_model: int, heads: int, ffn_dim: int,
                 path: int = B.WENC_PATH_BF16, ln_post=None, device="cuda"):
        import torch
        self.d_model, self.heads, self.ffn_dim, self.path = d_model, heads, ffn_dim, path
        self.device = torch.device(device)
        self.n_layers = len(layers)
        self.layer_bytes = B.whisper_enc_layer_bytes(d_model, ffn_dim, path)
        if self.layer_bytes == 0:
            raise B.WencError(B.WENC_ERR_ARG, "whisper_enc_layer_bytes")
        self.blob = torch.empty(max(1, self.layer_bytes * self.n_layers), dtype=torch.uint8,
                                device=self.device)
        assert self.blob.data_ptr() % 256 == 0
        for i, p in enumerate(layers):
            src = [_device_f32(p.get(k), self.device) for k in _ORDER]
            B.whisper_enc_pack_layer(*src, d_model, ffn_dim, path,
                                     self.blob.data_ptr() + i * self.layer_bytes)
            torch.cuda.current_stream(self.device).synchronize()  # sources may be freed now
        self.ln_post = None
        if ln_post is not None:
            self.ln_post = (_device_f32(ln_post[0], self.device), _device_f32(ln_post[1], self.device))
        self._ws = None

    def _launch_stream(self, stream):
        """The stream the library enqueues on, as a torch stream object (``None``: torch's
        current stream; an integer: a raw ``hipStream_t`` handle)."""
        import torch
        if stream is None:
            return torch.cuda.current_stream(self.device)
        if isinstance(stream, int):
            return torch.cuda.ExternalStream(stream, device=self.device)
        return stream

    def _keep_for(self, tensor, launch):
        """Tensors the kernels read must outlive the work enqueued on ``launch``: tell the caching
        allocator so when ``launch`` is not the stream they were allocated on."""
        import torch
        if launch != torch.cuda.current_stream(self.device):
            tensor.record_stream(launch)

    def workspace(self, batch: int, t: int):
        import torch
        need = B.whisper_enc_workspace_bytes(batch, t, self.d_model, self.heads, self.ffn_dim,
                                             self.path)
        if need == 0 and batch * t > 0:
            raise B.WencError(B.WENC_ERR_ARG, "whisper_enc_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def forward(self, x, y=None, n_layers: Optional[int] = None, final_norm: bool = True,
                stream=None):
        """Run the stack on ``x [batch, t, d]`` (fp32, on the device); returns ``y``."""
        import torch
        batch, t, d = x.shape
        assert d == self.d_model and x.dtype == torch.float32 and x.is_contiguous()
        n = self.n_layers if n_layers is None else n_layers
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace(batch, t)
        launch = self._launch_stream(stream)
        self._keep_for(ws, launch)
        g, b = (self.ln_post if (final_norm and self.ln_post is not None) else (None, None))
        B.whisper_enc_stack_forward(x, y, self.blob, n, g, b, batch, t, self.d_model, self.heads,
                                    self.ffn_dim, self.path, ws, ws.numel(), launch.cuda_stream)
        return y


    def forward_varlen(self, x, seqlens: Sequence[int], y=None, n_layers: Optional[int] = None,
                       final_norm: bool = True, stream=None):
        """Run the stack on a ragged batch: ``x [sum(seqlens), d]`` (fp32, on the device) holds
        the windows back to back, window ``b`` the next ``seqlens[b]`` rows; returns ``y``."""
        import torch
        total, d = x.shape
        assert d == self.d_model and x.dtype == torch.float32 and x.is_contiguous()
        lens = [int(n) for n in seqlens]
        assert sum(lens) == total and min(lens, default=0) >= 0
        max_t = max(lens, default=0)
        launch = self._launch_stream(stream)
        # The offsets are copied to the device on the launch stream and kept alive for it.
        with torch.cuda.stream(launch):
            cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                              device=self.device)
        n = self.n_layers if n_layers is None else n_layers
        if y is None:
            y = torch.empty_like(x)
        need = B.whisper_enc_varlen_workspace_bytes(len(lens), total, max_t, self.d_model,
                                                    self.heads, self.ffn_dim, self.path)
        if need == 0 and total > 0:
            raise B.WencError(B.WENC_ERR_ARG, "whisper_enc_varlen_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        self._keep_for(self._ws, launch)
        g, b = (self.ln_post if (final_norm and self.ln_post is not None) else (None, None))
        B.whisper_enc_stack_forward_varlen(x, y, self.blob, n, g, b, cu, len(lens), total, max_t,
                                           self.d_model, self.heads, self.ffn_dim, self.path,
                                           self._ws, self._ws.numel(), launch.cuda_stream)
        return y


def build_from_workload(w, path: int, device="cuda") -> EncoderStack:
    """Pack a :class:`synth.Workload`'s layers for ``path``."""
    c = w.cfg
    return EncoderStack(w.layers, c.d_model, c.heads, c.ffn_dim, path, w.ln_post, device)


def to_device_input(x: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
