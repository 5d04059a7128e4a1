"""One speculative-decoding verify step on the GPU (orchestration only).

The organisers' results page (section 3) describes the step: the target runs
one forward pass over the block of K+1 positions per sequence, its 8-bit
lm_head yields the greedy token of every row, and greedy acceptance keeps the
longest matching draft prefix plus the bonus token.  Here the target is a
chain of W4A16 linears (each reads the leading ``k_in`` columns of the
previous output; no attention or activation function is modelled), followed
by the fused lm_head + argmax + verify launch.  Every launch goes to the
current stream through the C ABI; the object owns the activation buffers and
one workspace shared by the stream-ordered calls, so a step allocates
nothing and can be captured in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (Chain, f16_gemm, f16_gemm_workspace_size, f16_lmhead_argmax_verify,
               gemm_workspace_size, lmhead_workspace_size, new_workspace, w4a16_gemm,
               w8a16_lmhead_argmax_verify)


@dataclass
class DeviceLinear:
    qweight: torch.Tensor | None   # int32 [k/8, n]
    scales: torch.Tensor | None    # fp16 [k/g, n]
    qzeros: torch.Tensor | None    # int32 [k/g, n/8]
    k_in: int
    n_out: int
    alpha: float
    group_size: int = 128
    w16: torch.Tensor | None = None   # fp16 [n, k]: a half-precision linear instead


class VerifyStep:
    def __init__(self, linears, lm_w, lm_s, m: int, batch: int, k_draft: int,
                 device="cuda", chain: bool | None = None):
        if m != batch * (k_draft + 1):
            raise ValueError("rows must be batch * (k_draft + 1)")
        self.linears = list(linears)
        self.lm_w, self.lm_s = lm_w, lm_s
        self.m, self.batch, self.k = m, batch, k_draft
        dev = torch.device(device)
        # one output buffer per distinct (position-in-layer) width, reused across layers
        self.out = []
        cache = {}
        for i, lin in enumerate(self.linears):
            key = (i % 4, lin.n_out) if len(self.linears) % 4 == 0 else (i, lin.n_out)
            if key not in cache:
                cache[key] = torch.empty((m, lin.n_out), dtype=torch.float16, device=dev)
            self.out.append(cache[key])
        for i in range(1, len(self.out)):
            if self.out[i].data_ptr() == self.out[i - 1].data_ptr():
                raise ValueError("consecutive linears would share a buffer")
        need = max([f16_gemm_workspace_size(m, l.n_out, l.k_in) if l.w16 is not None
                    else gemm_workspace_size(m, l.n_out, l.k_in, l.group_size)
                    for l in self.linears] + [0])
        if lm_w is not None:
            need = max(need, lmhead_workspace_size(m, lm_w.shape[1], lm_w.shape[0]))
        self.workspace = new_workspace(need, dev)
        # one launch for the whole chain when the block fits the chain kernel
        self.chain = None
        if chain is None:
            chain = False
        if chain:
            self.chain = Chain([(l.qweight, l.scales, l.qzeros, l.alpha) for l in self.linears],
                               m, dev)
        self.target_ids = torch.empty(m, dtype=torch.int32, device=dev)
        self.max_logits = torch.empty(m, dtype=torch.float32, device=dev)
        self.accepted_len = torch.empty(batch, dtype=torch.int32, device=dev)
        self.out_tokens = torch.empty((batch, k_draft + 1), dtype=torch.int32, device=dev)

    def linears_only(self, x: torch.Tensor) -> torch.Tensor:
        """Run the chain of linears on x (fp16 [m, >= k_in of the first]); returns the last output."""
        if self.chain is not None:
            return self.chain(x, out=self.out[-1])
        h = x
        for lin, y in zip(self.linears, self.out):
            if lin.w16 is not None:
                f16_gemm(h[:, :lin.k_in], lin.w16, alpha=lin.alpha, out=y, workspace=self.workspace)
            else:
                w4a16_gemm(h[:, :lin.k_in], lin.qweight, lin.scales, lin.qzeros, alpha=lin.alpha,
                           out=y, workspace=self.workspace, group_size=lin.group_size)
            h = y
        return h

    def head(self, h: torch.Tensor, drafts: torch.Tensor, accepted_len=None, out_tokens=None):
        """Fused lm_head + argmax + greedy verify on the final hidden rows (an fp16 lm_head
        when no scales are given).  accepted_len / out_tokens: caller buffers for the
        verify's outputs (int32 [batch] / [batch, K+1]); the step's own by default."""
        acc = self.accepted_len if accepted_len is None else accepted_len
        out = self.out_tokens if out_tokens is None else out_tokens
        if self.lm_s is None:
            return f16_lmhead_argmax_verify(h, self.lm_w, drafts, target_ids=self.target_ids,
                                            max_logits=self.max_logits, accepted_len=acc,
                                            out_tokens=out, workspace=self.workspace)
        return w8a16_lmhead_argmax_verify(h, self.lm_w, self.lm_s, drafts,
                                          target_ids=self.target_ids, max_logits=self.max_logits,
                                          accepted_len=acc, out_tokens=out,
                                          workspace=self.workspace)

    def __call__(self, x: torch.Tensor, drafts: torch.Tensor, accepted_len=None, out_tokens=None):
        return self.head(self.linears_only(x), drafts, accepted_len, out_tokens)
