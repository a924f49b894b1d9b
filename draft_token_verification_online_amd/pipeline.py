"""MineDraft's two-batch schedule on one GPU (MineDraft page, section 2).

Two batches alternate: while one batch is verified, the other is drafted, and
the roles swap every step.  MineDraft runs the two halves on separate GPUs
(the draft model on a GPU of its own); here both halves share one GPU and are
issued on two HIP streams of default priority, so drafting of one batch
overlaps verification of the other.

Step i verifies batch i % 2 with the tokens drafted for it in step i - 1, and
drafts batch (i + 1) % 2.  Verifying a batch waits (a stream event) for its
drafting; drafting a batch waits for the verification that read its previous
tokens.  Every call is a library call (spec_draft_sample, spec_verify_*); this
module only orders them.
"""
from __future__ import annotations

import torch

from . import Drafter, Verifier


class TwoBatchPipeline:
    """Holds a drafter and a verifier per batch and the two streams.

    batches: two dicts with device tensors target [B][K][L+1][V], draft
    [B][K][L][V], temperature [B] (the synthetic generator's layout).
    uniforms(i, b) must return (u_draft [B][K][L], u_accept [B][K][L],
    u_correct [B]) device tensors for the drafting of batch b in step i - 1 and
    its verification in step i; it is called on the host, once per step and
    batch, with the drafting stream current (tensors it makes are made on it),
    and the pipeline keeps what it returns alive until it is dropped."""

    def __init__(self, method, batches, uniforms, device="cuda"):
        t = batches[0]["target"]
        B, K, L1, V = t.shape
        self.shape = (B, K, L1 - 1, V)
        self.batches = batches
        self.uniforms = uniforms
        self.drafters = [Drafter(B, K, L1 - 1, V, t.dtype, device=device) for _ in range(2)]
        self.verifiers = [Verifier(method, B, K, L1 - 1, V, t.dtype, device=device)
                          for _ in range(2)]
        self.s_verify = torch.cuda.Stream(device=device)   # default priority
        self.s_draft = torch.cuda.Stream(device=device)
        self.ev_drafted = [torch.cuda.Event(), torch.cuda.Event()]
        self.ev_verified = [torch.cuda.Event(), torch.cuda.Event()]
        self._u = [None, None]      # uniforms of the pending (drafted, not yet verified) step
        self._keep = []
        self.step_index = 0

    def _draft(self, b, i, stream):
        bt = self.batches[b]
        # made on the drafting stream, so the verification that reads them later
        # (after the drafted event) sees them written; kept alive while a stream
        # may still read them
        with torch.cuda.stream(stream):
            self._u[b] = self.uniforms(i + 1, b)
        self._keep.append(self._u[b])
        self.drafters[b](bt["draft"], bt["temperature"], self._u[b][0],
                         stream=stream.cuda_stream)

    def _verify(self, b, stream):
        bt = self.batches[b]
        u = self._u[b]
        self.verifiers[b](bt["target"], bt["draft"], self.drafters[b].out["draft_tokens"],
                          bt["temperature"], u[1], u[2], stream=stream.cuda_stream)

    def prime(self):
        """Draft both batches once (the tokens step 0 and step 1 verify)."""
        for b in range(2):
            self._draft(b, b - 1, self.s_draft)
            self.ev_drafted[b].record(self.s_draft)
            self.ev_verified[b].record(self.s_verify)
        self.step_index = 0

    def step(self, on_verified=None, on_drafted=None):
        """One step: verify batch a = i % 2 on one stream, draft batch 1 - a on the
        other.  on_verified(i, a, stream) and on_drafted(i, b, stream) may enqueue
        work (copies of the outputs) on the stream that produced them."""
        i = self.step_index
        a, b = i % 2, (i + 1) % 2
        self.s_verify.wait_event(self.ev_drafted[a])
        self._verify(a, self.s_verify)
        if on_verified is not None:
            with torch.cuda.stream(self.s_verify):
                on_verified(i, a, self.s_verify)
        self.ev_verified[a].record(self.s_verify)
        self.s_draft.wait_event(self.ev_verified[b])
        self._draft(b, i, self.s_draft)
        if on_drafted is not None:
            with torch.cuda.stream(self.s_draft):
                on_drafted(i, b, self.s_draft)
        self.ev_drafted[b].record(self.s_draft)
        self.step_index += 1
