"""Device buffers for one synthetic problem, and the call through the C ABI.

PyTorch is used here for device memory, host<->device copies and the current
stream only; every step of the prefill runs in the HIP library through
``binding.gdn_prefill`` / ``binding.gdn_prefill_stage``.
"""

import numpy as np
import torch

from . import binding as B
from .inputs import CHUNK, HEAD_DIM, pack_contiguous, pack_conv

TP_ELEMS = 2560  # bf16 elements of each part (hi, lo) of a slot's T' (include/gdn_prefill.h)


def _to_bf16_tensor(u16, device):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(device).view(torch.bfloat16)


def _bf16_tensor_to_f32(t):
    return t.float().cpu().numpy()


def current_stream_handle():
    return torch.cuda.current_stream().cuda_stream


class DeviceProblem:
    """Upload a ``inputs.Problem`` in one of the accepted layouts.

    layout : "contiguous" -- separate q, k, v, g, beta buffers
             "conv"       -- one bf16 conv buffer for q|k|v, one f32 buffer for g|beta
    state  : "contiguous" -- h_state [B][nv][128][128]
             "table"      -- one allocation per sequence, passed as a pointer table
    ragged : None picks dense mode when every sequence has the same length,
             True forces cu_seqlens / cu_chunks.
    flags  : GDN_OPT_* options of the calls (default: entry states emitted,
             q and k passed normalised).
    """

    def __init__(self, p, layout="contiguous", state="contiguous", ragged=None, device="cuda",
                 flags=B.GDN_OPT_ENTRY_STATES):
        self.p = p
        self.device = device
        self.flags = int(flags)
        self.nseq, self.nk, self.nv = p.nseq, p.nk, p.nv
        self.N = p.n_tokens
        lens = p.lengths
        self._chunk0 = p.cu_chunks  # chunk offsets, computed once (slot() reads them per slot)
        self.ragged = (len(set(lens)) != 1) if ragged is None else bool(ragged)
        if not self.ragged and lens[0] == 0:
            raise ValueError("dense mode needs T > 0")
        self.layout, self.state_kind = layout, state

        if layout == "contiguous":
            c = pack_contiguous(p)
            self._bufs = dict(q=_to_bf16_tensor(c["q"], device), k=_to_bf16_tensor(c["k"], device),
                              v=_to_bf16_tensor(c["v"], device),
                              g=torch.from_numpy(c["g"]).to(device), beta=torch.from_numpy(c["beta"]).to(device))
            self.q, self.k, self.v = (self._bufs[x].data_ptr() for x in ("q", "k", "v"))
            self.g, self.beta = self._bufs["g"].data_ptr(), self._bufs["beta"].data_ptr()
        elif layout == "conv":
            c = pack_conv(p)
            conv = _to_bf16_tensor(c["conv"], device)
            gb = torch.from_numpy(c["gb"]).to(device)
            self._bufs = dict(conv=conv, gb=gb)
            base = conv.data_ptr()
            self.q, self.k, self.v = base + 2 * c["q_off"], base + 2 * c["k_off"], base + 2 * c["v_off"]
            self.g, self.beta = gb.data_ptr() + 4 * c["g_off"], gb.data_ptr() + 4 * c["beta_off"]
        else:
            raise ValueError(layout)
        self.strides = B.gdn_strides(c["qk_row"], c["v_row"], c["gb_row"])

        if self.ragged:
            self.cu_seqlens_host = p.cu_seqlens
            self.cu_chunks_host = p.cu_chunks
            self._cu_s = torch.from_numpy(self.cu_seqlens_host).to(device)
            self._cu_c = torch.from_numpy(self.cu_chunks_host).to(device)
            nch = np.diff(self.cu_chunks_host)
            max_c, total_c = (int(nch.max()) if len(nch) else 0), int(self.cu_chunks_host[-1])
            # the library trusts device offsets; check the host copies once here
            if B.gdn_varlen_check_host(self.nseq, self.N, self.cu_seqlens_host, self.cu_chunks_host, max_c,
                                       total_c) != B.GDN_OK:
                raise ValueError(B.gdn_last_error())
            self.varlen = B.gdn_varlen(self._cu_s.data_ptr(), self._cu_c.data_ptr(), max_c, total_c)
            self.B, self.T = self.nseq, self.N
        else:
            self.varlen = None
            self.B, self.T = self.nseq, lens[0]

        if state == "contiguous":
            self.h = torch.empty((self.nseq, self.nv, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=device)
            self.h_ptr, self.h_is_table = self.h.data_ptr(), 0
        elif state == "table":
            self.h_list = [torch.empty((self.nv, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=device)
                           for _ in range(self.nseq)]
            self.h_table = torch.tensor([t.data_ptr() for t in self.h_list], dtype=torch.int64, device=device)
            self.h_ptr, self.h_is_table = self.h_table.data_ptr(), 1
        else:
            raise ValueError(state)
        self.reset_state()

        self.out = torch.empty((self.N, self.nv, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.scratch_bytes = B.gdn_prefill_scratch_bytes_ex(self.B, self.T, self.nk, self.nv, HEAD_DIM, HEAD_DIM,
                                                            self.varlen, self.flags)
        if self.scratch_bytes == 0:
            raise ValueError("invalid sizes for the scratch layout")
        self.scratch = torch.empty(self.scratch_bytes, dtype=torch.uint8, device=device)
        self.layout_info = B.gdn_prefill_scratch_layout_ex(self.B, self.T, self.nk, self.nv, HEAD_DIM, HEAD_DIM,
                                                           self.varlen, self.flags)

    # -- state ---------------------------------------------------------------
    def reset_state(self):
        h0 = self.p.h0
        if hasattr(h0, "to_torch"):  # initial states that build themselves on the device
            h0 = h0.to_torch(self.device)
        else:
            h0 = torch.from_numpy(np.ascontiguousarray(h0))
        if self.state_kind == "contiguous":
            self.h.copy_(h0)
        else:
            for i, t in enumerate(self.h_list):
                t.copy_(h0[i])

    def state(self):
        if self.state_kind == "contiguous":
            return self.h.cpu().numpy()
        return np.stack([t.cpu().numpy() for t in self.h_list])

    def state_of(self, i):
        """The state [nv][128][128] of sequence i, copied to the host."""
        return (self.h[i] if self.state_kind == "contiguous" else self.h_list[i]).cpu().numpy()

    # -- calls ---------------------------------------------------------------
    def args(self):
        return (self.q, self.k, self.v, self.g, self.beta, self.h_ptr, self.h_is_table, self.out.data_ptr(),
                self.scratch.data_ptr(), self.scratch_bytes, self.B, self.T, self.nk, self.nv, HEAD_DIM,
                HEAD_DIM, self.strides, self.varlen)

    def run(self, stream=None):
        s = current_stream_handle() if stream is None else stream
        return B.gdn_prefill_ex(*self.args(), self.flags, s)

    def run_stage(self, stage, stream=None):
        s = current_stream_handle() if stream is None else stream
        return B.gdn_prefill_stage_ex(stage, *self.args(), self.flags, s)

    def decode_step(self, t, out=None, stream=None, flags=None):
        """One gdn_decode_ex call on token t of every sequence (dense problems,
        all of length T): the token pointers advance t rows and the row pitch
        becomes T rows, so sequence b's token t is decode row b.  Writes bf16
        [B][nv][128] into ``out`` (default: ``self.dec_out``).  ``flags``
        defaults to the problem's q/k normalisation bit."""
        if self.ragged:
            raise ValueError("decode steps need sequences of one length")
        if not 0 <= t < self.T:
            raise ValueError(f"token {t} outside [0, {self.T})")
        if out is None:
            if getattr(self, "dec_out", None) is None:
                self.dec_out = torch.empty((self.nseq, self.nv, HEAD_DIM), dtype=torch.bfloat16, device=self.device)
            out = self.dec_out
        st, T = self.strides, self.T
        strides = B.gdn_strides(st.qk_row * T, st.v_row * T, st.gb_row * T)
        s = current_stream_handle() if stream is None else stream
        fl = self.flags & B.GDN_OPT_L2NORM_QK if flags is None else int(flags)
        return B.gdn_decode_ex(self.q + 2 * t * st.qk_row, self.k + 2 * t * st.qk_row, self.v + 2 * t * st.v_row,
                               self.g + 4 * t * st.gb_row, self.beta + 4 * t * st.gb_row, self.h_ptr,
                               self.h_is_table, out.data_ptr(), self.nseq, self.nk, self.nv, HEAD_DIM, HEAD_DIM,
                               strides, fl, s)

    # -- results ---------------------------------------------------------------
    def output(self):
        return _bf16_tensor_to_f32(self.out)

    def output_rows(self, a, b, heads):
        """Output rows a..b-1 of the v-heads ``heads`` as float32, copied to
        the host without converting the rest."""
        idx = torch.as_tensor(list(heads), device=self.out.device)
        return _bf16_tensor_to_f32(self.out[a:b].index_select(1, idx))

    def region(self, name):
        """A scratch region as a torch view shaped [slots, ...]."""
        L = self.layout_info
        S = int(L.slots)
        off = getattr(L, name)
        if off == B.GDN_NO_REGION:
            raise KeyError(f"region {name} is not in this layout (flags 0x{self.flags:x})")
        if name == "gc":
            return self.scratch[off:off + S * CHUNK * 4].view(torch.float32).view(S, CHUNK)
        if name == "nrm":
            return self.scratch[off:off + S * 2 * CHUNK * 4].view(torch.float32).view(S, 2, CHUNK)
        if name == "tp":
            return self.scratch[off:off + S * 2 * TP_ELEMS * 2].view(torch.bfloat16).view(S, 2, TP_ELEMS)
        if name == "s_entry":
            return self.scratch[off:off + S * HEAD_DIM * HEAD_DIM * 2].view(torch.bfloat16).view(S, HEAD_DIM, HEAD_DIM)
        raise KeyError(name)

    def slot(self, i, h, c):
        """Slot index of (sequence i, v-head h, chunk c)."""
        chunk0 = int(self._chunk0[i])
        nch = int(self._chunk0[i + 1]) - chunk0
        return chunk0 * self.nv + h * nch + c
