"""Device-side plumbing around the C-ABI library: put a workload's tensors in
HBM (torch is used only to allocate device memory and streams), create a head,
run forwards, read outputs and debug snapshots back.  No arithmetic of the head
happens here; every step runs in libclefhead's HIP kernels."""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import clefhead as C


def to_device_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> a bfloat16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


class HeadRunner:
    """share: another HeadRunner whose device weights and lexical table this
    one reuses (clef_head_create_sharing); it gets its own workspace."""

    def __init__(self, case, table: Optional[torch.Tensor] = None, device="cuda",
                 share: Optional["HeadRunner"] = None):
        if not torch.cuda.is_available():
            raise RuntimeError("HeadRunner needs a HIP device")
        C.load()
        self.case = case
        self.device = device
        if share is not None:
            self.table = share.table
            self.handle = C.clef_head_create_sharing(share.handle)
        else:
            self.table = table if table is not None else to_device_bf16(case.table, device)
            self.handle = C.clef_head_create(case.head, case.weights, self.table.data_ptr())
        self.hidden = None
        self.args = None

    def close(self):
        if self.handle:
            C.clef_head_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_batch(self, batch=None, layout: int = C.CLEF_PADDED):
        batch = batch if batch is not None else self.case.batch
        host = batch.hidden if layout == C.CLEF_PADDED else batch.varlen_hidden()
        self.hidden = to_device_bf16(host, self.device)
        self.batch = batch
        self.args = C.BatchArgs(batch, self.hidden.data_ptr(), layout)
        self.logits = torch.empty(max(batch.NO, 1), dtype=torch.float32, device=self.device)
        self.probs = torch.empty_like(self.logits)
        self.argmax = torch.empty(max(batch.NQ, 1), dtype=torch.int32, device=self.device)

    def forward(self, stream: Optional[torch.cuda.Stream] = None):
        s = stream if stream is not None else torch.cuda.current_stream()
        C.clef_head_forward(self.handle, self.args, self.logits.data_ptr(), self.probs.data_ptr(),
                            self.argmax.data_ptr(), s.cuda_stream)

    def forward_noalloc(self, stream: Optional[torch.cuda.Stream] = None):
        """clef_head_forward_noalloc: the same forward in the library's static scratch."""
        s = stream if stream is not None else torch.cuda.current_stream()
        C.clef_head_forward_noalloc(self.handle, self.args, self.logits.data_ptr(), self.probs.data_ptr(),
                                    self.argmax.data_ptr(), s.cuda_stream)

    def forward_answers(self, stream: Optional[torch.cuda.Stream] = None):
        """Forward plus the answer mapping; answers() reads the answer buffers."""
        s = stream if stream is not None else torch.cuda.current_stream()
        nq, no = max(self.batch.NQ, 1), max(self.batch.NO, 1)
        if getattr(self, "ans", None) is None or self.ans[0].numel() < nq or self.ans[4].numel() < no:
            self.ans = [torch.empty(nq, dtype=torch.float32, device=self.device) for _ in range(4)] + \
                       [torch.empty(no, dtype=torch.float32, device=self.device)]
        C.clef_head_forward_answers(self.handle, self.args, self.logits.data_ptr(), self.probs.data_ptr(),
                                    self.argmax.data_ptr(), *[t.data_ptr() for t in self.ans],
                                    stream_ptr=s.cuda_stream)

    def answers(self):
        """(value, confidence, value_4dp, confidence_4dp) fp32 [NQ] and probs_4dp fp32 [NO], as numpy."""
        torch.cuda.synchronize()
        NO, NQ = self.batch.NO, self.batch.NQ
        return tuple(t[:NQ].cpu().numpy() for t in self.ans[:4]) + (self.ans[4][:NO].cpu().numpy(),)

    def outputs(self):
        torch.cuda.synchronize()
        NO, NQ = self.batch.NO, self.batch.NQ
        return (self.logits[:NO].cpu().numpy().astype(np.float64), self.probs[:NO].cpu().numpy().astype(np.float64),
                self.argmax[:NQ].cpu().numpy().astype(np.int64))

    def set_trace(self, on: bool):
        C.clef_head_set_trace(self.handle, on)

    def trace(self, which: int, shape, dtype=np.float32) -> np.ndarray:
        out = np.empty(shape, dtype)
        return C.clef_head_trace(self.handle, which, out)
