"""Host checks of the packed-batch backward (gdn2_chunk_bwd_varlen, include/gdn2.h) that
need no GPU.  Every pointer, the offsets included, is a fake device address that is never
dereferenced, so a call that passes every check stops at the missing GPU
(GDN2_ERR_DEVICE)."""
import ctypes
import itertools

import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import _binding as bnd

OK, NULL, SHAPE, DTYPE, ALIAS, WS, DEVICE, ALIGN = range(8)
BASE = 0x7f0000000000
NAMES = ("cu", "q", "k", "v", "alpha", "b", "w", "S0", "dO", "dS_T", "dq", "dk", "dv", "dalpha", "db", "dw", "dS0",
         "ws")


class VB:
    def __init__(self, lengths=(70, 0, 129, 5), H=2, dk=64, dv=32, io=torch.bfloat16):
        N, T = len(lengths), sum(lengths)
        self.p = bnd.problem(N, T, H, dk, dv, io)
        es = 2 if io == torch.bfloat16 else 4
        rows = max(T, 1) * H
        tok = dict(cu=4 * (N + 1), q=rows * dk * es, v=rows * dv * es, gk=rows * dk * 4, gv=rows * dv * 4,
                   st=N * H * dk * dv * 4)
        kind = dict(cu="cu", q="q", k="q", v="v", alpha="gk", b="gk", w="gv", S0="st", dO="v", dS_T="st", dq="q",
                    dk="q", dv="v", dalpha="gk", db="gk", dw="gv", dS0="st")
        self.ws_need = g.lib().gdn2_chunk_bwd_varlen_workspace_size(ctypes.byref(self.p))
        self.ptr, at = {}, BASE
        for n in NAMES:
            size = self.ws_need if n == "ws" else tok[kind[n]]
            self.ptr[n] = at
            at += (max(size, 1) + 65535) // 65536 * 65536
        self.lengths = lengths

    def call(self, ws_bytes=None, **over):
        a = dict(self.ptr)
        a.update(over)
        return g.lib().gdn2_chunk_bwd_varlen(ctypes.byref(self.p),
                                             *(None if a[n] is None else ctypes.c_void_p(a[n]) for n in NAMES),
                                             self.ws_need if ws_bytes is None else ws_bytes, None)


def test_valid_call_reaches_the_device_check():
    c = VB()
    assert c.call() == DEVICE
    assert c.call(S0=None, dS_T=None, dS0=None) == DEVICE
    f = VB(io=torch.float32, dk=16, dv=48)                        # the vector-ALU path
    assert f.call() == DEVICE


def test_workspace_depends_on_the_counts_only():
    c = VB()
    need = c.ws_need
    assert need > 0
    # one more sequence of the same tokens needs more chunk slots
    more = bnd.problem(5, 204, 2, 64, 32, torch.bfloat16)
    assert g.lib().gdn2_chunk_bwd_varlen_workspace_size(ctypes.byref(more)) > need
    # at least the equal-length backward over the same tokens as one sequence
    one = g.lib().gdn2_chunk_bwd_workspace_size(ctypes.byref(bnd.problem(1, 204, 2, 64, 32, torch.bfloat16)))
    assert need > one
    assert c.call(ws_bytes=need - 1) == WS and c.call(ws=None) == WS
    assert c.call(ws=c.ptr["ws"] + 16) == WS                      # 256-byte alignment


def test_offsets_are_an_input():
    c = VB()
    assert c.call(cu=None) == NULL
    assert c.call(cu=c.ptr["cu"] + 2) == ALIGN
    assert c.call(cu=c.ptr["dq"]) == ALIAS                         # an output over the offsets
    assert c.call(cu=c.ptr["ws"] + 256) == ALIAS                   # the workspace over the offsets
    assert c.call(cu=c.ptr["q"]) == DEVICE                         # inputs may share memory


def test_alias_null_and_alignment():
    c = VB()
    assert c.call(dq=c.ptr["q"]) == ALIAS
    assert c.call(dS0=c.ptr["S0"]) == ALIAS
    assert c.call(ws=c.ptr["dO"]) == ALIAS
    assert c.call(dv=None) == NULL and c.call(q=None) == NULL
    assert c.call(dw=c.ptr["dw"] + 8) == ALIGN


def test_empty_batches():
    c = VB(lengths=(0, 0))
    assert c.call(dS0=None) == OK                                 # nothing to do
    assert c.call() == DEVICE                                     # dS_T passes through to dS0
    n0 = VB()
    n0.p.B = 0
    assert n0.call(**{n: None for n in NAMES}) == OK


def test_lengths_do_not_change_the_size():
    sizes = set()
    for lengths in itertools.permutations((70, 0, 129, 5)):
        sizes.add(VB(lengths=lengths).ws_need)
    assert len(sizes) == 1
