"""gla_chunk_fwd_varlen_noalloc (the packed forward for callers that cannot
allocate: its scratch is a fixed per-GPU array in the library) against
gla_chunk_fwd_varlen on the same inputs. Both run the same kernels, so the
outputs and final states must be bitwise equal; both are also held to the
oracle's bf16 bar. Three calls in a row share the array: a packed batch of
long sequences (time segments: item table, dispatch order and segment
states in the scratch), then a smaller one (dispatch order only), then a
third with new data, so stale scratch from the call before never leaks."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _case(seed, lengths, H=16, dk=96, dv=192):
    return W.varlen_inputs(seed, len(lengths), 0, H, dk, dv, "bf16", 0.1,
                           W.geometric_decays(H), lengths=lengths)


def _compare(x, name):
    q, k, v, s0, cu = (dev(x[n]) for n in ("q", "k", "v", "s0", "cu_seqlens"))
    N = len(x["lengths"])
    o_ref, sf_ref = gla.gla_chunk_fwd_varlen(q, k, v, cu, x["decay"], initial_state=s0)
    o = torch.full_like(o_ref, float("nan"))
    sf = torch.full_like(sf_ref, float("nan"))
    gla.gla_chunk_fwd_varlen_noalloc(q, k, v, cu, x["decay"], o, initial_state=s0,
                                     final_state=sf)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), name
    assert torch.equal(sf, sf_ref), name
    ro, rs = O.gla_varlen(x["cu_seqlens"], x["q"], x["k"], x["v"], x["decay"], 1.0, x["s0"])
    eo, es = rel_err(host(o), ro), rel_err(host(sf), rs)
    print("%s (N %d): bitwise equal to the workspace call; oracle o %.2e S %.2e"
          % (name, N, eo, es), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = gla.lib()
    big = _case(901, [9000, 3000])
    need = L.gla_chunk_fwd_varlen_workspace_bytes(1, 2, 12000, 16, 96, 192, 0)
    assert 16 * 96 * 192 * 4 < need <= 32 << 20  # segment states live in the scratch
    small = _case(902, [100, 0, 64, 1])
    assert 0 < L.gla_chunk_fwd_varlen_workspace_bytes(1, 4, 165, 16, 96, 192, 0) < 4096
    _compare(big, "long sequences, time segments")
    _compare(small, "short sequences, dispatch order only")
    _compare(_case(903, [7000, 1, 5000]), "long sequences again, new data")
