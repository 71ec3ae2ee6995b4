"""A whole DLRM training step on the library's kernels (page "DLRM For PyTorch", §Model
architecture): bottom MLP -> embedding bags + dot interaction -> top MLP -> one logit ->
logistic loss, then the backward of every stage and SGD on the dense parameters and on
the embedding rows.

Only orchestration lives here: buffers are torch device tensors, every arithmetic step is a
call into ``libembcore`` (``el_linear_fwd`` / ``el_linear_bwd`` on MFMA, ``emb_dot_fwd``,
``dot_interact_bwd``, ``el_relu_bwd``, ``el_bce_logits``, ``el_sgd_dense``,
``emb_grad_prepare`` / ``emb_grad_apply``).

Layout choices:
  * dense parameters of each MLP live in three flat buffers (fp32 master, 16-bit copy read
    by the products, fp32 gradient), so one SGD launch updates them all; weights are
    w[n][k] ([N][K] row-major), biases stay fp32;
  * the 13 dense features are zero-padded to 16 columns (and the first layer's weights get
    zero columns), the interaction output keeps a zero-padded width as the top MLP's input
    width (479 -> 512: a multiple of 128 once it is 256 or wider, so that the top MLP's
    first products have no partial reduction stage and take the GEMM's unmasked instance):
    padded inputs are always zero, so the layers compute what the unpadded ones would.
"""
from typing import Sequence

import torch

from . import embcore as ec
from . import synth


def _pad8(n: int) -> int:
    return (n + 7) // 8 * 8


def inter_stride(wl: synth.Workload) -> int:
    """Row width of the interaction output as the top MLP's input: the workload's padded
    width, rounded up to a multiple of 128 once it is 256 or wider."""
    w = wl.out_stride
    return (w + 127) // 128 * 128 if w >= 256 else w


class DenseMLP:
    """Parameters and gradients of a stack of dense layers (sizes[0] -> ... -> sizes[-1])."""

    def __init__(self, params, dtype: torch.dtype, device):
        self.shapes = [tuple(w.shape) for w, _ in params]  # (N, K) per layer
        offs, o = [], 0
        for (N, K) in self.shapes:
            offs.append((o, o + N * K))
            o += _pad8(N * K) + _pad8(N)
        self.numel = o
        self.master = torch.zeros(o, dtype=torch.float32, device=device)
        self.copy = torch.zeros(o, dtype=dtype, device=device)
        self.grad = torch.zeros(o, dtype=torch.float32, device=device)
        self.w, self.b, self.w_master, self.dw, self.db = [], [], [], [], []
        for (w, b), (N, K), (ow, ob) in zip(params, self.shapes, offs):
            self.master[ow:ow + N * K] = w.reshape(-1)
            self.master[ob:ob + N] = b
            self.w_master.append(self.master[ow:ow + N * K].view(N, K))
            self.b.append(self.master[ob:ob + N])
            self.w.append(self.copy[ow:ow + N * K].view(N, K))
            self.dw.append(self.grad[ow:ow + N * K].view(N, K))
            self.db.append(self.grad[ob:ob + N])
        self.copy.copy_(self.master.to(dtype))

    def sgd(self, lr: float, stream=None):
        ec.sgd_dense(self.master, self.grad, lr, self.copy, stream=stream)


class DLRMStep:
    """Buffers and parameters for one workload; `train_step` runs forward, backward and the
    SGD updates for one batch, `forward` the inference half."""

    def __init__(self, wl: synth.Workload, tables: ec.Tables, device, top: Sequence[int] = synth.TOP_MLP,
                 k_pad: int = 16):
        self.wl = wl
        self.tables = tables
        self.dtype = synth.act_dtype(wl)
        dt, B, D, F = self.dtype, wl.batch, wl.dim, wl.num_tables
        if wl.bottom_mlp[-1] != D:
            raise ValueError("the bottom MLP must end at the embedding dim")
        self.k_pad = k_pad
        self.bottom = DenseMLP(synth.make_mlp_params(wl, "bottom", wl.bottom_mlp, k_pad, device), dt, device)
        self.top_sizes = (wl.out_width,) + tuple(top)
        self.istride = inter_stride(wl)
        self.top = DenseMLP(synth.make_mlp_params(wl, "top", self.top_sizes, self.istride, device), dt, device)
        e = lambda *s: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        # forward activations (kept for the backward)
        self.h_bot = [e(B, n) for n in wl.bottom_mlp[1:]]       # ..., x0 = h_bot[-1]
        self.emb = e(B, F, D)
        self.inter = e(B, self.istride)
        self.h_top = [e(B, n) for n in top]                      # ..., logits = h_top[-1]
        # backward buffers
        widest = max(max(top[:-1]), max(wl.bottom_mlp[1:]), self.istride)
        self.gbuf = [torch.empty(B * widest, dtype=dt, device=device) for _ in range(2)]
        self.dlogit = e(B, 1)
        self.dout = e(B, self.istride)
        self.dx0 = e(B, D)
        self.demb = e(B, F, D)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        sizes = [(B, K, N) for (N, K) in self.bottom.shapes + self.top.shapes]
        self.lin_ws = torch.empty(max(256, max(ec.linear_bwd_workspace_bytes(*s) for s in sizes),
                                      ec.bce_workspace_bytes(B)), dtype=torch.uint8, device=device)

    def _g(self, i: int, n: int) -> torch.Tensor:
        return self.gbuf[i][: self.wl.batch * n].view(self.wl.batch, n)

    # ------------------------------------------------------------------ forward
    def forward(self, dense: torch.Tensor, bags: ec.Bags, keep_emb: bool = True, mark=None):
        """Bottom MLP, emb-bag + interaction, top MLP; returns the logits [B, 1] view."""
        h = dense
        for i, (w, b) in enumerate(zip(self.bottom.w, self.bottom.b)):
            ec.linear_fwd(h, w, b, self.h_bot[i], relu=True)
            h = self.h_bot[i]
        mark and mark("bottom_fwd")
        ec.emb_dot_fwd(self.tables, bags, self.h_bot[-1], self.inter, self.emb if keep_emb else None)
        mark and mark("emb_dot_fwd")
        h = self.inter
        n_top = len(self.top.w)
        for i, (w, b) in enumerate(zip(self.top.w, self.top.b)):
            ec.linear_fwd(h, w, b, self.h_top[i], relu=(i < n_top - 1))
            h = self.h_top[i]
        mark and mark("top_fwd")
        return self.h_top[-1]

    # ------------------------------------------------------------------ backward
    def backward(self, dense: torch.Tensor, labels: torch.Tensor, mark=None, record=None):
        """Loss and gradients of every dense parameter, dx0 and demb (after forward).  With
        `record` (a dict), a copy of every layer's dz is kept under ("top" | "bottom", i)
        for inspection."""
        keep = (lambda key, t: record.__setitem__(key, t.clone())) if record is not None else None
        ec.bce_logits(self.h_top[-1], labels, self.loss, self.dlogit, workspace=self.lin_ws)
        # dz of each layer; the data gradient of the layer goes to the other ping-pong buffer
        dz, cur = self.dlogit, 1
        n_top = len(self.top.w)
        for i in reversed(range(n_top)):
            keep and keep(("top", i), dz)
            x = self.h_top[i - 1] if i > 0 else self.inter
            dx = self._g(1 - cur, x.shape[1]) if i > 0 else self.dout
            ec.linear_bwd(x, self.top.w[i], dz, self.top.dw[i], self.top.db[i], dx=dx,
                          relu_mask=(i > 0), workspace=self.lin_ws)
            dz, cur = dx, 1 - cur
        mark and mark("top_bwd")
        ec.dot_interact_bwd(self.h_bot[-1], self.emb, self.dout, self.dx0, self.demb)
        mark and mark("dot_interact_bwd")
        n_bot = len(self.bottom.w)
        cur = 0
        dz = self._g(cur, self.wl.dim)
        ec.relu_bwd(self.dx0, self.h_bot[-1], dz)
        for i in reversed(range(n_bot)):
            keep and keep(("bottom", i), dz)
            x = self.h_bot[i - 1] if i > 0 else dense
            dx = self._g(1 - cur, x.shape[1]) if i > 0 else None
            ec.linear_bwd(x, self.bottom.w[i], dz, self.bottom.dw[i], self.bottom.db[i], dx=dx,
                          relu_mask=(i > 0), workspace=self.lin_ws)
            dz, cur = dx, 1 - cur
        mark and mark("bottom_bwd")

    def train_step(self, dense, bags, labels, emb_ws, side=None, mark=None):
        """One SGD step of the whole model.  With `side` (a stream), the embedding-gradient
        sort runs there from the start of the step (it needs only the lookups) and the
        row update waits for it with an event."""
        lr = self.wl.lr
        cur = torch.cuda.current_stream()
        if side is not None:
            ev = torch.cuda.Event()
            ev.record(cur)
            side.wait_event(ev)
            ec.emb_grad_prepare(self.tables, bags, emb_ws, stream=side)
            done = torch.cuda.Event()
            done.record(side)
        self.forward(dense, bags, mark=mark)
        self.backward(dense, labels, mark=mark)
        self.bottom.sgd(lr)
        self.top.sgd(lr)
        mark and mark("dense_sgd")
        if side is None:
            ec.emb_grad_prepare(self.tables, bags, emb_ws)
        else:
            cur.wait_event(done)
        ec.emb_grad_apply(self.tables, bags, self.demb, lr, emb_ws)
        mark and mark("emb_update")

    def dense_flops(self) -> dict:
        """Algorithmic flops of the dense layers for one batch (2 per multiply-add; the
        padded input columns are not counted): forward, data gradients, weight gradients."""
        B = self.wl.batch
        fwd = dgrad = wgrad = 0
        real_k = [self.wl.bottom_mlp[0]] + [K for (_, K) in self.bottom.shapes[1:]] + \
                 [self.wl.out_width] + [K for (_, K) in self.top.shapes[1:]]
        shapes = self.bottom.shapes + self.top.shapes
        for li, ((N, _), K) in enumerate(zip(shapes, real_k)):
            fwd += 2 * B * N * K
            wgrad += 2 * B * N * K
            if li != 0:
                dgrad += 2 * B * N * K
        return {"fwd": fwd, "dgrad": dgrad, "wgrad": wgrad}
