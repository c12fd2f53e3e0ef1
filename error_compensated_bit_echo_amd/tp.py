"""Echo inside tensor-parallel layers: autograd operators over one emulated TP group.

A tensor-parallel block needs two collectives (rit.work blog post
"echo-4-bit-gpu-communication", «Почему обычное 4-битное суммирование портит
модель»: the layer's matrices are split over the GPUs, each computes a part of
the result and an all-reduce sums the parts; in training it repeats on the
backward pass):

* ``g`` after a row-parallel product: forward sums the P partial outputs (an
  Echo all-reduce on the forward compensator state); backward hands the
  replicated gradient to every rank unchanged.
* ``f`` before a column-parallel product: forward gives every rank the same
  input; backward sums the P partial input gradients (an Echo all-reduce on
  the backward compensator state).

Forward and backward keep separate compensator state (same page, «Как Echo
возвращает ошибку в следующие вызовы»); one state per residual stream, shared
by all the block's calls of one pass and reset at the start of each step.
The P ranks are P tensors on one GPU; every reduction runs in libecho's
kernels through the C ABI.  A ``mode`` of "exact" replaces both collectives by
a plain sum (the bf16 wire values added in fp32), for comparison.

The row-parallel product and ``g`` can also run as one step in bfloat16
(``product="bf16_fused"``): libecho's MFMA product writes each rank's stage-1
payload straight from its accumulators, then the owner and decode stages
finish the all-reduce; ``"bf16"`` runs the same product written out followed
by a whole Echo call, which gives bit-identical results.  The same holds for
``f`` in the backward pass: the input-gradient products of the column-parallel
layer run on libecho's kernel, on the backward state.
"""
from __future__ import annotations

from typing import List, Optional

from . import binding as B


class EchoGroup:
    """P emulated ranks sharing one Echo state (forward and backward directions)
    for messages of ``numel`` elements in bfloat16 on the wire.  ``variant``
    passes the configuration switches ``sender_feedback``, ``state_bf16``,
    ``own_exact`` and ``group`` through to the state (the output stays fp32)."""

    VARIANT_KEYS = ("sender_feedback", "state_bf16", "own_exact", "group")

    def __init__(self, P: int, numel: int, mode: str = "echo", device=None, record: bool = False,
                 **variant):
        import torch

        if mode not in ("echo", "echo_off", "exact"):
            raise ValueError(f"mode {mode!r}")
        unknown = set(variant) - set(self.VARIANT_KEYS)
        if unknown:
            raise ValueError(f"unknown variant switches {sorted(unknown)}")
        self.P, self.numel, self.mode, self.variant = P, numel, mode, dict(variant)
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.state = None
        if mode != "exact":
            cfg = B.EchoConfig.make(P, numel, "bf16", compensate=(mode == "echo"), **variant)
            self.state = B.echo_init_state(cfg, device=self.device)
        # when recording, every reduction appends (direction, [partials], out)
        self.record = record
        self.log: List[tuple] = []

    def reset(self):
        """Start of a step: fresh compensator for both directions."""
        if self.state is not None:
            B.echo_reset(self.state, 3)
        self.log.clear()

    def product_allreduce(self, A, W, fused: bool, direction: int = B.ECHO_FWD):
        """All-reduce of bf16(A_r @ W_r^T) (A_r [T, K], W_r [H, K] bf16) on the
        state of `direction`: fused, stage 1 runs in the product's epilogue;
        otherwise the product is written out and reduced by a whole call."""
        import torch

        if self.mode == "exact":
            raise ValueError("the bf16 product path needs an Echo state")
        if fused and (self.variant.get("own_exact") or self.variant.get("group", 32) != 32):
            raise ValueError("the fused product takes group 32 without the owners' own shares")
        T, H = A[0].shape[0], W[0].shape[0]
        out = torch.empty(self.numel, dtype=torch.float32, device=self.device)
        if fused:
            B.echo_gemm_stage1(A, W, self.state, direction)
            B.echo_owner(self.state, direction)
            B.echo_decode(out, self.state)
        else:
            parts = [torch.empty(T, H, dtype=torch.bfloat16, device=self.device) for _ in range(self.P)]
            B.echo_gemm_bf16(A, W, parts)
            B.echo_reduce([p.view(-1) for p in parts], out, self.state, direction)
        if self.record:
            self.log.append((direction, ("product", [a.detach().clone() for a in A],
                                         [w.detach().clone() for w in W]), out.detach().clone()))
        return out

    def allreduce(self, partials, direction: int):
        """Sum of the P bf16 partials ([..] contiguous, numel each) as fp32."""
        import torch

        parts = [p.contiguous() for p in partials]
        if self.mode == "exact":
            out = torch.zeros(self.numel, dtype=torch.float32, device=self.device)
            for p in parts:
                out += p.reshape(-1).float()
        else:
            out = torch.empty(self.numel, dtype=torch.float32, device=self.device)
            B.echo_reduce([p.reshape(-1) for p in parts], out, self.state, direction)
        if self.record:
            self.log.append((direction, [p.detach().clone() for p in parts], out.detach().clone()))
        return out


def _fns():
    import torch

    class RowParallelEcho(torch.autograd.Function):
        """g(h_r @ W2_r) with the products in bfloat16 on libecho's matrix-core
        kernel: forward gives sum_r bf16(bf16(h_r) @ bf16(W2_r)) through Echo
        (fused: stage 1 in the product's epilogue); backward is the fp32
        gradient of sum_r h_r @ W2_r (the rounding passed straight through)."""

        @staticmethod
        def forward(ctx, group: "EchoGroup", shape, fused: bool, *hw):
            P = group.P
            hs, ws = hw[:P], hw[P:]
            A = [h.to(torch.bfloat16).contiguous() for h in hs]   # [T, F/P]
            W = [w.t().to(torch.bfloat16).contiguous() for w in ws]  # [H, F/P]: output features by K
            out = group.product_allreduce(A, W, fused)
            ctx.save_for_backward(*hs, *ws)
            ctx.P = P
            return out.view(shape)

        @staticmethod
        def backward(ctx, grad):
            P = ctx.P
            saved = ctx.saved_tensors
            hs, ws = saved[:P], saved[P:]
            g = grad.contiguous()
            dh = [g @ w.t().contiguous() for w in ws]
            dw = [h.t().contiguous() @ g for h in hs]
            return (None, None, None) + tuple(dh) + tuple(dw)

    class ReduceForward(torch.autograd.Function):
        """g: forward all-reduce of the P partial outputs; backward identity per rank."""

        @staticmethod
        def forward(ctx, group: EchoGroup, shape, *partials):
            ctx.dtypes = [p.dtype for p in partials]
            return group.allreduce([p.to(torch.bfloat16) for p in partials], B.ECHO_FWD).view(shape)

        @staticmethod
        def backward(ctx, grad):
            g = grad.contiguous()
            return (None, None) + tuple(g.reshape(-1).to(dt) for dt in ctx.dtypes)

    class ReduceBackward(torch.autograd.Function):
        """f: forward replicates the input to every rank; backward all-reduces the
        P input gradients."""

        @staticmethod
        def forward(ctx, group: EchoGroup, x):
            ctx.group, ctx.shape, ctx.dtype = group, x.shape, x.dtype
            return tuple(x.clone() for _ in range(group.P))

        @staticmethod
        def backward(ctx, *grads):
            parts = [g.to(torch.bfloat16).contiguous() for g in grads]
            out = ctx.group.allreduce(parts, B.ECHO_BWD)
            return None, out.view(ctx.shape).to(ctx.dtype)

    class ColumnParallelEcho(torch.autograd.Function):
        """f(a) @ W1_r with the input-gradient products in bfloat16 on libecho's
        matrix-core kernel: forward gives every rank's pre-activation a @ W1_r
        (fp32, no reduction); backward gives dL/da through Echo on the backward
        state as sum_r bf16(bf16(dpre_r) @ bf16(W1_r)^T) (fused: stage 1 in the
        product's epilogue), and the fp32 weight gradients a^T dpre_r."""

        @staticmethod
        def forward(ctx, group: "EchoGroup", fused: bool, a, *w1s):
            ctx.save_for_backward(a, *w1s)
            ctx.group, ctx.fused = group, fused
            return tuple(a @ w for w in w1s)

        @staticmethod
        def backward(ctx, *gpres):
            a, *w1s = ctx.saved_tensors
            A = [g.to(torch.bfloat16).contiguous() for g in gpres]   # [T, F/P]
            W = [w.to(torch.bfloat16).contiguous() for w in w1s]     # [H, F/P]: output features by K
            da = ctx.group.product_allreduce(A, W, ctx.fused, B.ECHO_BWD).view(a.shape)
            dw = [a.t().contiguous() @ g for g in gpres]
            return (None, None, da) + tuple(dw)

    return ReduceForward, ReduceBackward, RowParallelEcho, ColumnParallelEcho


_FNS = None


def row_parallel_echo(group: "EchoGroup", hs, ws, shape, fused: bool):
    """g(sum_r h_r @ W2_r) with bf16 products on libecho's kernel (see RowParallelEcho)."""
    global _FNS
    if _FNS is None:
        _FNS = _fns()
    return _FNS[2].apply(group, shape, fused, *hs, *ws)


def column_parallel_echo(group: "EchoGroup", a, ws, fused: bool):
    """[a @ W1_r] with the input gradient through bf16 products on libecho's
    kernel and Echo's backward state (see ColumnParallelEcho)."""
    global _FNS
    if _FNS is None:
        _FNS = _fns()
    return _FNS[3].apply(group, fused, a, *ws)


def reduce_forward(group: EchoGroup, partials, shape):
    """g(partials): all-reduce on the forward state; gradient passes through."""
    global _FNS
    if _FNS is None:
        _FNS = _fns()
    return _FNS[0].apply(group, shape, *partials)


def replicate(group: EchoGroup, x):
    """f(x): P copies of x; their gradients are all-reduced on the backward state."""
    global _FNS
    if _FNS is None:
        _FNS = _fns()
    return _FNS[1].apply(group, x)


class TPMLPStack:
    """L pre-norm MLP blocks, each split over P ranks: W1 column-parallel
    ([H, F] in P slices of F/P columns), W2 row-parallel ([F, H] in P slices of
    F/P rows); x <- x + g(sum_r gelu(f(a)_r @ W1_r) @ W2_r), a = rmsnorm(x).
    Weights are fp32 and seeded.  product "f32": the products are taken in fp32
    and each rank's partial output is rounded to bf16 (the wire dtype);
    "bf16" / "bf16_fused": the products whose outputs are reduced run in
    bfloat16 on libecho's kernel, the row-parallel W2 product in the forward
    pass and the column-parallel W1 input-gradient product in the backward
    pass (written out, or with stage 1 in their epilogues; T a multiple of 64,
    H of 128, F/P of 64)."""

    def __init__(self, layers: int, hidden: int, ffn: int, P: int, seed: int = 0, device=None,
                 product: str = "f32"):
        import torch

        if ffn % P:
            raise ValueError("ffn must be divisible by P")
        if product not in ("f32", "bf16", "bf16_fused"):
            raise ValueError(f"product {product!r}")
        self.L, self.H, self.F, self.P, self.product = layers, hidden, ffn, P, product
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        self.w1, self.w2 = [], []
        for _ in range(layers):
            w1 = torch.randn(hidden, ffn, generator=g, device=dev) / hidden ** 0.5
            w2 = torch.randn(ffn, hidden, generator=g, device=dev) / ffn ** 0.5 * 0.5
            self.w1.append([w1[:, r * ffn // P:(r + 1) * ffn // P].contiguous().requires_grad_()
                            for r in range(P)])
            self.w2.append([w2[r * ffn // P:(r + 1) * ffn // P, :].contiguous().requires_grad_()
                            for r in range(P)])

    def parameters(self):
        return [w for layer in self.w1 + self.w2 for w in layer]

    def forward(self, x, group: EchoGroup):
        import torch

        for l in range(self.L):
            a = x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
            if self.product == "f32":
                xs = replicate(group, a)
                hs = [torch.nn.functional.gelu(xs[r] @ self.w1[l][r]) for r in range(self.P)]
            else:
                pres = column_parallel_echo(group, a, self.w1[l], self.product == "bf16_fused")
                hs = [torch.nn.functional.gelu(p) for p in pres]
            if self.product == "f32":
                partials = [(hs[r] @ self.w2[l][r]).to(torch.bfloat16) for r in range(self.P)]
                y = reduce_forward(group, [p.reshape(-1) for p in partials], x.shape)
            else:
                y = row_parallel_echo(group, hs, self.w2[l], x.shape, self.product == "bf16_fused")
            x = x + y
        return x


def train_step(model: TPMLPStack, group: EchoGroup, x0, target):
    """One forward + backward; returns (loss, dL/dx0, [dL/dW...])."""
    import torch

    group.reset()
    x = x0.detach().clone().requires_grad_()
    for p in model.parameters():
        p.grad = None
    y = model.forward(x, group)
    loss = torch.nn.functional.mse_loss(y, target)
    loss.backward()
    return loss.detach(), x.grad.detach(), [p.grad.detach() for p in model.parameters()]
